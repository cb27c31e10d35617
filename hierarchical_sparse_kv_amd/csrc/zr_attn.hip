// Split-K decode attention over a paged KV pool, sparse ("zoomed-in") and dense.
//
// The tokens of one (sequence b, KV head g), a "pair", arrive as a list of
// (physical block, 16-bit slot mask) entries (KV-cache management page, paged
// KV cache, eq. 4: attention as a sum over blocks fetched through the block
// table). Sparse: the pair kernel lists the blocks of the window and the
// selected thoughts' spans (ZoomR Sec. 3.3, eq. I_f restricted to those
// spans); dense: every block of [0, T), read from the block table here. Only
// attended slots enter the softmax; the gather reads the listed blocks, it
// does not mask a full read.
//
// Work split. The grid is sized once for the whole GPU (`nwg` workgroups).
// Every workgroup reads all pairs' list lengths n_p and takes an equal range
// (total / nwg entries, rounded down or up) of the pairs' lists laid end to
// end, so every workgroup streams the same number of blocks however ragged
// the pairs are; a range that crosses pairs is processed as one segment per
// pair. For
// each segment the 4 waves take chunks of NBW blocks in turn: a wave loads
// all its entries at once (one lane per entry), then streams its chunks with
// the next chunk's K/V loads in flight while the current one is computed,
// keeping a running (max, sum, weighted V) per query head (online softmax
// across chunks, two-pass inside one). The waves merge in LDS into one
// partial per segment; a combine kernel merges each pair's partials by
// log-sum-exp.
// (Merging inside the attention kernel would need a device-scope
// release/acquire per workgroup, which on this GPU writes back and
// invalidates the whole L2; the kernel boundary is far cheaper.)
//
// bf16 kernel (matrix cores), on chunks of two blocks (32 slots):
//   S^T[slot][head] = K (16 slots x d) . Q^T (d x 16 heads, zero padded)
// on v_mfma_f32_16x16x32_bf16, twice per chunk, with the key rows taken in an
// order that leaves each lane 8 consecutive slots of one block for one head:
// exactly the A-operand layout of
//   O[head][dim] += P[head][slot] . V[slot][dim]
// on v_mfma_f32_16x16x32_bf16 over the chunk's 32 slots, so P never leaves
// the lane. V blocks are stored dimension-major, so each lane's B operand (8
// slots of one dimension) is one 16-byte load and a wave reads a block's
// values as contiguous 512-byte segments. P is split into bf16 hi + lo parts
// (p - hi rounded again), so the probabilities keep ~16 significant bits;
// products accumulate in fp32.
//
// fp32 inputs run the same kernel on v_mfma_f32_16x16x4_f32, one block per
// chunk (16 slots, the same 16 KB of keys and values as a bf16 chunk):
// S^T and P.V take their operands from one 16-byte load per lane each (keys
// by row, values dimension-major), P needs no splitting, and S^T and O keep
// the bf16 kernel's head layout, so the running states, the rescaling and
// the merges are shared. The query of each segment is read from LDS rather
// than held in registers.
//
// Exponentials are base 2 with the scale folded in (exp(x) = 2^(x log2 e)).
//
// Each key and value tile is read once per call, with one 16-byte load per
// lane, so both kernels load them with the non-temporal hint (measured on
// bf16: 5 to 10 % less time per call on the 16K x 8, 64K x 4 and ragged
// workloads).
#include <math.h>

#include <type_traits>

#include "zr_internal.h"

namespace zr {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr float kNegInf = -INFINITY;
constexpr int kTargetWorkgroups = 512;  // two per CU on MI355X: one resident round
constexpr int kMinBlocksPerWg = 8;
constexpr int kPairsPerThread = (ZR_MAX_PAIRS + kThreads - 1) / kThreads;

typedef short bf16x8 __attribute__((vector_size(16)));
typedef short bf16x4 __attribute__((vector_size(8)));
typedef float f32x4 __attribute__((vector_size(16)));
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Work assignment
// ---------------------------------------------------------------------------

// The pairs' lists, concatenated in pair order (total entries), are cut into
// nr = min(nwg, total) ranges: workgroup w takes entries [R(w), R(w + 1)) of
// the concatenation, R(w) = floor(w total / nr), so the workgroups' block
// counts differ by at most one however ragged the pairs are (and no range is
// empty). A range that crosses
// the end of a pair is split into segments, one per pair met, each merged
// into a partial of its own. Pair p (entries [start_p, start_p + n_p) of the
// concatenation) is met by the workgroups w0_p = W(start_p) ..
// W(start_p + n_p - 1), W(x) = the range holding entry x; its partials take
// slots [base_p, base_p + S_p) (base = exclusive prefix of the S_p), segment
// (p, w) the slot base_p + w - w0_p. Workgroup 0 publishes
// base_p (ws_pref) for the combine kernel. Every workgroup computes the
// whole plan itself from the lists' lengths.
struct Assign {
  int p;       // pair
  int T;       // cached tokens of the pair's sequence
  int tw;      // first window token (dense: 0)
  int ncache;  // leading list entries read from the block lists (dense: 0)
  int lo, hi;  // entries [lo, hi) of the pair's list
  int slot;    // partial slot
};

// A pair's list: its ncache span entries (sparse), then the blocks of the
// window [tw, T) (dense: [0, T)).
struct PairList {
  int T, tw, ncache, n;
};

// The plan covers the window [T0 - window, T0 + horizon) of the planned
// length T0 (plan_lens); the current length T (seq_lens, at most T0 +
// horizon) ends the attended slots. An ordinary call plans on the current
// length (plan_lens = seq_lens) with no horizon.
template <bool DENSE>
__device__ __forceinline__ PairList pair_list(const AttnArgs& a, int p) {
  PairList r;
  const int b = div_small(p, a.Hkv);
  const int cap = a.max_blocks * kBlock;
  const int t_plan = a.plan_lens[b], t_now = a.seq_lens[b];
  const int T0 = t_plan < 0 ? 0 : (t_plan > cap ? cap : t_plan);
  const int Tp = T0 + a.horizon < cap ? T0 + a.horizon : cap;
  r.T = t_now < 0 ? 0 : (t_now > Tp ? Tp : t_now);
  r.tw = DENSE ? 0 : (T0 - a.window > 0 ? T0 - a.window : 0);
  r.ncache = 0;
  if (!DENSE) {
    const int c = a.counts[p];
    r.ncache = c < 0 ? 0 : (c > a.max_blocks ? a.max_blocks : c);
    // the window starts no earlier than where the lists' spans stop, so a
    // token is never attended twice
    const int t0 = a.list_tw[p];
    r.tw = r.tw > t0 ? r.tw : (t0 < Tp ? t0 : Tp);
  }
  const int wb = Tp > r.tw ? ((Tp - 1) >> 4) - (r.tw >> 4) + 1 : 0;
  r.n = r.ncache + wb;
  return r;
}

// First entry of range w, R(w) = floor(w total / nr), and the range W(x)
// holding entry x (the largest w with R(w) <= x), for nr <= total ranges.
// The quotients are taken in float64: numerator and denominator are exact
// integers below 2^52, so the rounded quotient never crosses the integer
// above the exact one (they differ by at least 1 / denominator, more than an
// ulp), and the floor is exact; integer 64-bit division is a long sequence.
__device__ __forceinline__ int floor_div(int64_t n, int d) {
  return static_cast<int>(floor(static_cast<double>(n) / static_cast<double>(d)));
}
__device__ __forceinline__ int range_start(int w, int total, int nr) {
  return floor_div(static_cast<int64_t>(w) * total, nr);
}
__device__ __forceinline__ int range_of(int x, int total, int nr) {
  return floor_div((static_cast<int64_t>(x) + 1) * nr - 1, total);
}

// Partial slots of a pair whose entries are [s, s + n) of the concatenation.
__device__ __forceinline__ int pair_slots(int s, int n, int total, int nr) {
  return n > 0 ? range_of(s + n - 1, total, nr) - range_of(s, total, nr) + 1 : 0;
}

// The segments reach the kernel body as LDS records, up to kMaxSeg at a
// time. A range can meet more than kMaxSeg pairs only when they are short
// and more than 64; every segment between the first and the last of a range
// is then a whole pair with one partial, so the next records follow from
// where the last one ended (next pair, its position in the concatenation,
// its slot).
constexpr int kMaxSeg = 64;
struct PlanLds {
  int tmp[kWaves];
  int nrec;                 // records in rec
  int next_p, next_pos, next_slot, r1;
  int4 rec[kMaxSeg][2];     // {p, T, tw, ncache}, {lo, hi, slot, -}
};

__device__ __forceinline__ void put_record(PlanLds& sm, int i, int p, int T, int tw, int ncache,
                                           int lo, int hi, int slot) {
  sm.rec[i][0] = make_int4(p, T, tw, ncache);
  sm.rec[i][1] = make_int4(lo, hi, slot, 0);
}

// (The values are the same in every lane: readfirstlane keeps them, and all
// that is derived from them, in scalar registers.)
__device__ __forceinline__ void get_record(const PlanLds& sm, int i, Assign* as) {
  const int4 r0 = sm.rec[i][0], r1 = sm.rec[i][1];
  as->p = __builtin_amdgcn_readfirstlane(r0.x);
  as->T = __builtin_amdgcn_readfirstlane(r0.y);
  as->tw = __builtin_amdgcn_readfirstlane(r0.z);
  as->ncache = __builtin_amdgcn_readfirstlane(r0.w);
  as->lo = __builtin_amdgcn_readfirstlane(r1.x);
  as->hi = __builtin_amdgcn_readfirstlane(r1.y);
  as->slot = __builtin_amdgcn_readfirstlane(r1.z);
}

// Up to kWavePairs pairs every wave computes the plan by itself (lane l owns
// pairs [l K, (l + 1) K), K = ceil(P / 64) <= kLanePairs, DPP scans) and
// takes its first two segments into scalar registers, with no LDS and no
// barrier; the records are written to LDS (the same values by every wave)
// only when asked for or when there are more than two segments. Returns the
// number of segments.
//
// Where whole-pair slices are about as even, they are used instead of the
// ranges: pair p gets S_p = max(1, round(n_p / per)) workgroups (per =
// ceil(total / nwg)), each an equal slice of its list, one segment per
// workgroup, slot = workgroup. That is chosen when it needs no more than nwg
// workgroups and no slice is longer than the ranges' largest plus 1/8: one
// segment per workgroup and fewer partials then beat the exact balance.
constexpr int kLanePairs = 4;
constexpr int kWavePairs = 64 * kLanePairs;

__device__ __forceinline__ void lane_segment(int src, int p, int T, int tw, int ncache, int lo,
                                             int hi, int slot, Assign* as) {
  as->p = __builtin_amdgcn_readlane(p, src);
  as->T = __builtin_amdgcn_readlane(T, src);
  as->tw = __builtin_amdgcn_readlane(tw, src);
  as->ncache = __builtin_amdgcn_readlane(ncache, src);
  as->lo = __builtin_amdgcn_readlane(lo, src);
  as->hi = __builtin_amdgcn_readlane(hi, src);
  as->slot = __builtin_amdgcn_readlane(slot, src);
}

template <bool DENSE>
__device__ int plan_wave(const AttnArgs& a, PlanLds& sm, bool records, Assign* sa, Assign* sb) {
  const int P = a.B * a.Hkv;
  const int lane = threadIdx.x & 63, w = blockIdx.x;
  const bool publish = w == 0 && threadIdx.x < 64;
  const int K = (P + 63) / 64;
  const int p0 = lane * K;
  int n[kLanePairs], T[kLanePairs], tws[kLanePairs], nc[kLanePairs];
  int nsum = 0;
#pragma unroll
  for (int j = 0; j < kLanePairs; ++j) {
    PairList L{0, 0, 0, 0};
    if (j < K && p0 + j < P) L = pair_list<DENSE>(a, p0 + j);
    n[j] = L.n;
    T[j] = L.T;
    tws[j] = L.tw;
    nc[j] = L.ncache;
    nsum += L.n;
  }
  const int incl = wave_incl_sum(nsum);
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int run = incl - nsum;  // first entry of this lane's pairs
  const int nr = total < a.nwg ? total : a.nwg;  // ranges: none empty

  // whole-pair slices
  const int per = total > 0 ? floor_div(total - 1, a.nwg) + 1 : 1;
  const int range_max = nr > 0 ? floor_div(total - 1, nr) + 1 : 0;
  const int cap = range_max + range_max / 8;
  int S[kLanePairs];
  int ssum = 0;
  bool uneven = false;
#pragma unroll
  for (int j = 0; j < kLanePairs; ++j) {
    S[j] = 0;
    if (j < K) {  // uniform: pair slots past K hold nothing and cost no division
      // round(n / per), halves up, without forming n + per / 2
      const int q = floor_div(n[j], per), r = n[j] - q * per;
      S[j] = n[j] > 0 ? max(1, q + (r >= per - per / 2 ? 1 : 0)) : 0;
      ssum += S[j];
      uneven = uneven || n[j] > S[j] * cap;
    }
  }
  const int sincl = wave_incl_sum(ssum);
  const int total_s = __builtin_amdgcn_readlane(sincl, 63);
  if (total_s <= a.nwg && __ballot(uneven) == 0ull) {  // uniform
    const int srun = sincl - ssum;
    if (publish) {
      int r = srun;
#pragma unroll
      for (int j = 0; j < kLanePairs; ++j) {
        if (j < K && p0 + j < P) a.ws_pref[p0 + j] = r;
        r += S[j];
      }
      if (lane == 0) a.ws_pref[P] = total_s;
    }
    if (w >= total_s) return 0;
    const bool mine = w >= srun && w < srun + ssum;
    int pj = 0, tj = 0, twj = 0, cj = 0, nj = 0, sj = 1, r = 0;
    if (mine) {
      int r0 = srun;
#pragma unroll
      for (int j = 0; j < kLanePairs; ++j) {
        if (w >= r0 && w < r0 + S[j]) {
          r = w - r0;
          pj = p0 + j;
          tj = T[j];
          twj = tws[j];
          cj = nc[j];
          nj = n[j];
          sj = S[j];
        }
        r0 += S[j];
      }
    }
    // the slice bounds of the owning lane's pair only (one division pair)
    const int lo = floor_div(static_cast<int64_t>(r) * nj, sj);
    const int hi = floor_div(static_cast<int64_t>(r + 1) * nj, sj);
    const int src = __ffsll(static_cast<unsigned long long>(__ballot(mine))) - 1;
    lane_segment(src, pj, tj, twj, cj, lo, hi, w, sa);
    if (records && mine) put_record(sm, 0, pj, tj, twj, cj, lo, hi, w);
    return 1;
  }

  // ranges
  int nssum = 0;
  {
    int st = run;
#pragma unroll
    for (int j = 0; j < kLanePairs; ++j) {
      if (j < K) nssum += pair_slots(st, n[j], total, nr);
      st += n[j];
    }
  }
  const int rincl = wave_incl_sum(nssum);
  const int R0 = w < nr ? range_start(w, total, nr) : total;
  const int R1 = w < nr ? range_start(w + 1, total, nr) : total;
  int cnt = 0;
  {
    int st = run, bs = rincl - nssum;
#pragma unroll
    for (int j = 0; j < kLanePairs; ++j) {
      if (publish && j < K && p0 + j < P) a.ws_pref[p0 + j] = bs;
      cnt += n[j] > 0 && st < R1 && st + n[j] > R0 ? 1 : 0;
      if (j < K) bs += pair_slots(st, n[j], total, nr);
      st += n[j];
    }
  }
  if (publish && lane == 0) a.ws_pref[P] = __builtin_amdgcn_readlane(rincl, 63);
  const int cincl = wave_incl_sum(cnt);
  const int nseg = __builtin_amdgcn_readlane(cincl, 63);
  const bool put = records || nseg > 2;
  // this lane's segments, ordinals from cincl - cnt on; keep ordinals 0 and 1
  int v0[7] = {0, 0, 0, 0, 0, 0, 0}, v1[7] = {0, 0, 0, 0, 0, 0, 0};
  {
    int st = run, bs = rincl - nssum, ord = cincl - cnt;
#pragma unroll
    for (int j = 0; j < kLanePairs; ++j) {
      const int e = st + n[j];
      if (n[j] > 0 && st < R1 && e > R0) {
        const int v[7] = {p0 + j, T[j], tws[j], nc[j], (st > R0 ? st : R0) - st,
                          (e < R1 ? e : R1) - st, bs + w - range_of(st, total, nr)};
        if (put && ord < kMaxSeg) put_record(sm, ord, v[0], v[1], v[2], v[3], v[4], v[5], v[6]);
        if (put && ord == kMaxSeg - 1) {  // more segments follow only if this one ends inside
          sm.next_p = v[0] + 1;
          sm.next_pos = e;
          sm.next_slot = v[6] + 1;
        }
#pragma unroll
        for (int i = 0; i < 7; ++i) {
          v0[i] = ord == 0 ? v[i] : v0[i];
          v1[i] = ord == 1 ? v[i] : v1[i];
        }
        ++ord;
      }
      if (j < K) bs += pair_slots(st, n[j], total, nr);
      st += n[j];
    }
  }
  if (put && lane == 0) sm.r1 = R1;
  const int before = cincl - cnt;
  if (nseg >= 1) {
    const int src = __ffsll(static_cast<unsigned long long>(__ballot(cnt > 0 && before == 0))) - 1;
    lane_segment(src, v0[0], v0[1], v0[2], v0[3], v0[4], v0[5], v0[6], sa);
  }
  if (nseg >= 2) {
    const int src =
        __ffsll(static_cast<unsigned long long>(__ballot(before <= 1 && before + cnt > 1))) - 1;
    lane_segment(src, v1[0], v1[1], v1[2], v1[3], v1[4], v1[5], v1[6], sb);
  }
  return nseg;
}

// More pairs: thread t owns a contiguous run of pairs, and the scans go
// through LDS. Writes the first kMaxSeg records and the continuation state,
// returns the number of segments (uniform). Contains barriers: every thread
// must call it.
template <bool DENSE>
__device__ int plan_block(const AttnArgs& a, PlanLds& sm) {
  const int P = a.B * a.Hkv;
  const int t = threadIdx.x, w = blockIdx.x;
  const int per_t = (P + kThreads - 1) / kThreads;  // <= kPairsPerThread
  const int p0 = t * per_t;
  int nreg[kPairsPerThread], treg[kPairsPerThread], twreg[kPairsPerThread],
      creg[kPairsPerThread];
  int mine = 0;
#pragma unroll
  for (int j = 0; j < kPairsPerThread; ++j) {
    const int p = p0 + j;
    PairList L{0, 0, 0, 0};
    if (j < per_t && p < P) L = pair_list<DENSE>(a, p);
    nreg[j] = L.n;
    treg[j] = L.T;
    twreg[j] = L.tw;
    creg[j] = L.ncache;
    mine += L.n;
  }
  int total;
  const int run = wg_exclusive_scan<kWaves>(mine, sm.tmp, &total);
  const int nr = total < a.nwg ? total : a.nwg;  // ranges: none empty
  int ms = 0;
  {
    int st = run;
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      ms += pair_slots(st, nreg[j], total, nr);
      st += nreg[j];
    }
  }
  int total_slots;
  const int sbase = wg_exclusive_scan<kWaves>(ms, sm.tmp, &total_slots);
  const int R0 = w < nr ? range_start(w, total, nr) : total;
  const int R1 = w < nr ? range_start(w + 1, total, nr) : total;
  int cnt = 0;
  {
    int st = run, bs = sbase;
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int p = p0 + j, n = nreg[j];
      if (w == 0 && j < per_t && p < P) a.ws_pref[p] = bs;
      cnt += n > 0 && st < R1 && st + n > R0 ? 1 : 0;
      bs += pair_slots(st, n, total, nr);
      st += n;
    }
  }
  if (w == 0 && t == 0) a.ws_pref[P] = total_slots;
  int nseg;
  int ord = wg_exclusive_scan<kWaves>(cnt, sm.tmp, &nseg);
  {
    int st = run, bs = sbase;
#pragma unroll
    for (int j = 0; j < kPairsPerThread; ++j) {
      const int n = nreg[j], e = st + n;
      if (n > 0 && st < R1 && e > R0) {
        const int slot = bs + w - range_of(st, total, nr);
        if (ord < kMaxSeg)
          put_record(sm, ord, p0 + j, treg[j],
                     twreg[j], creg[j],
                     (st > R0 ? st : R0) - st, (e < R1 ? e : R1) - st, slot);
        if (ord == kMaxSeg - 1) {  // more segments follow only if this one ends inside
          sm.next_p = p0 + j + 1;
          sm.next_pos = e;
          sm.next_slot = slot + 1;
        }
        ++ord;
      }
      bs += pair_slots(st, n, total, nr);
      st += n;
    }
  }
  if (t == 0) {
    sm.nrec = nseg < kMaxSeg ? nseg : kMaxSeg;
    sm.r1 = R1;
  }
  __syncthreads();
  return nseg;
}

// The next records after a full batch (workgroups of more than kMaxSeg
// segments): wave 0 walks the pairs from next_p, 64 at a time, and every
// non-empty pair whose start is below the range end gives a record (the
// last one clipped at the range end). Contains barriers: every thread must
// call it. Returns the number of records (uniform, > 0 while segments
// remain).
template <bool DENSE>
__device__ int plan_next(const AttnArgs& a, PlanLds& sm) {
  __syncthreads();  // every thread has read the previous records
  if (threadIdx.x < 64) {
    const int P = a.B * a.Hkv, lane = threadIdx.x;
    int p = sm.next_p, pos = sm.next_pos, slot = sm.next_slot;
    const int r1 = sm.r1;
    int cnt = 0;
    while (cnt < kMaxSeg && pos < r1 && p < P) {
      const int q = p + lane;
      PairList L{0, 0, 0, 0};
      if (q < P) L = pair_list<DENSE>(a, q);
      const int incl = wave_incl_sum(L.n);
      const int st = pos + incl - L.n, e = st + L.n;
      const bool take = q < P && L.n > 0 && st < r1;
      const uint64_t bal = __ballot(take);
      const int ord = cnt + __popcll(bal & ((1ull << lane) - 1ull));
      const bool put = take && ord < kMaxSeg;
      if (put)
        put_record(sm, ord, q, L.T, L.tw, L.ncache, 0, (e < r1 ? e : r1) - st,
                   slot + ord - cnt);
      // go on after the last pair put when the record cap cut the batch,
      // else after all 64
      const uint64_t bput = __ballot(put);
      const int nput = __popcll(bput);
      if (nput < static_cast<int>(__popcll(bal))) {
        const int last = 63 - __builtin_clzll(bput);
        p = p + last + 1;
        pos = __builtin_amdgcn_readlane(e, last);
      } else {
        p += 64;
        pos += __builtin_amdgcn_readlane(incl, 63);
      }
      slot += nput;
      cnt += nput;
    }
    if (lane == 0) {
      sm.nrec = cnt;
      sm.next_p = p;
      sm.next_pos = pos;
      sm.next_slot = slot;
    }
  }
  __syncthreads();
  return sm.nrec;
}

// This workgroup's number of segments (uniform) and its first two segments
// (*sa, *sb, scalar). The records [0, kMaxSeg) are in sm.rec, behind a
// barrier, when `records` is set or there are more than two segments.
// Contains barriers: every thread must call it.
template <bool DENSE>
__device__ int plan_work(const AttnArgs& a, PlanLds& sm, bool records, Assign* sa, Assign* sb) {
  if (a.B * a.Hkv > kWavePairs) {
    const int nseg = plan_block<DENSE>(a, sm);
    if (nseg >= 1) get_record(sm, 0, sa);
    if (nseg >= 2) get_record(sm, 1, sb);
    return nseg;
  }
  const int nseg = plan_wave<DENSE>(a, sm, records, sa, sb);
  if (records || nseg > 2) {  // uniform
    if (threadIdx.x == 0) sm.nrec = nseg < kMaxSeg ? nseg : kMaxSeg;
    __syncthreads();
  }
  return nseg;
}

// Slots of [tw, T) in logical block lb (0 when the block holds none of them:
// a block planned ahead of the current length).
__device__ __forceinline__ uint32_t window_mask(int lb, int tw, int T) {
  const int b0 = lb << 4;
  const int from = (tw > b0 ? tw : b0) - b0;
  const int to = (T < b0 + kBlock ? T : b0 + kBlock) - b0;
  return to > from ? ((1u << to) - 1u) & ~((1u << from) - 1u) : 0u;
}

// Entry j of the pair's list -> physical block and slot mask ((0, 0) when j
// is -1 or the block id is out of range).
template <bool DENSE>
__device__ __forceinline__ void resolve_entry(const AttnArgs& a, const Assign& as, int b, int j,
                                              int* pb, uint32_t* mask) {
  *pb = 0;
  *mask = 0;
  if (j < 0) return;
  int blk;
  uint32_t m;
  if (!DENSE && j < as.ncache) {
    const int2 e = a.entries[static_cast<size_t>(as.p) * a.max_blocks + j];
    blk = e.x;
    m = static_cast<uint32_t>(e.y) & 0xffffu;
  } else {
    // window block: slots of [tw, T) in logical block lb
    const int lb = (as.tw >> 4) + (j - as.ncache);
    m = window_mask(lb, as.tw, as.T);
    blk = m ? a.block_table[static_cast<size_t>(b) * a.max_blocks + lb] : -1;
  }
  if (blk < 0 || blk >= a.num_blocks) return;
  *pb = blk;
  *mask = m;
}

// Entry of this wave for lane-indexed position e (chunks of NBW round-robin
// over the waves): the list index j, or -1.
template <int NBW>
__device__ __forceinline__ int wave_entry(const Assign& as, int wave, int e) {
  const int j = as.lo + ((e / NBW) * kWaves + wave) * NBW + e % NBW;
  return j < as.hi ? j : -1;
}

// Number of this wave's chunks that hold at least one entry of the range.
template <int NBW>
__device__ __forceinline__ int wave_chunks(const Assign& as, int wave) {
  const int nck = (as.hi - as.lo + NBW - 1) / NBW;  // chunks in the range
  return nck > wave ? (nck - wave + kWaves - 1) / kWaves : 0;
}

// Merge the waves' (m, l, acc) and write this workgroup's partial.
// red_m / red_l: [kWaves][G]; red_o: [kWaves][G][D].
template <int G, int D>
__device__ void write_partial(const AttnArgs& a, int slot_i, const float (*red_m)[G],
                              const float (*red_l)[G], const float (*red_o)[G][D]) {
  const size_t slot = static_cast<size_t>(slot_i);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, e = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, red_m[w][h]);
    float L = 0.f, A = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        if (red_m[w][h] != kNegInf) {
          const float f = exp2f(red_m[w][h] - M);
          L = fmaf(red_l[w][h], f, L);
          A = fmaf(red_o[w][h][e], f, A);
        }
      }
    }
    const size_t o = slot * G + h;
    a.ws_acc[o * D + e] = A;
    if (e == 0) {
      a.ws_m[o] = M;
      a.ws_l[o] = L;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernel. G query heads per KV head (G <= 16), head dim D,
// NBW blocks per wave per chunk.
// ---------------------------------------------------------------------------
__device__ __forceinline__ bf16x4 pack_bf16x4(float p0, float p1, float p2, float p3) {
  const bf16x2v lo = __builtin_convertvector((f32x2v){p0, p1}, bf16x2v);
  const bf16x2v hi = __builtin_convertvector((f32x2v){p2, p3}, bf16x2v);
  const unsigned u0 = __builtin_bit_cast(unsigned, lo), u1 = __builtin_bit_cast(unsigned, hi);
  bf16x4 r;
  r[0] = static_cast<short>(u0 & 0xffffu);
  r[1] = static_cast<short>(u0 >> 16);
  r[2] = static_cast<short>(u1 & 0xffffu);
  r[3] = static_cast<short>(u1 >> 16);
  return r;
}

__device__ __forceinline__ float bf16_at(const bf16x4& v, int i) {
  return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(v[i])) << 16);
}

// One chunk is two blocks: the K dimension of the P.V product is their 32
// slots. Lane group lg (lanes 16 lg .. 16 lg + 15) owns the 8 consecutive
// slots 8 (lg & 1) .. +7 of block lg >> 1, so that its value operand of
// v_mfma_f32_16x16x32_bf16 (8 slots of one dimension) is one 16-byte load
// from the dimension-major value tile, and its probabilities come from the
// two S^T products below without any exchange between lanes: product hf
// takes as row i the key of block i >> 3, slot 8 ((i >> 2) & 1) + 4 hf +
// (i & 3), and its output rows 4 lg .. 4 lg + 3 are then slots
// 8 (lg & 1) + 4 hf .. +3 of block lg >> 1.
template <int D, int NBW>
struct Chunk {
  static_assert(NBW == 2, "a chunk is two blocks");
  bf16x8 k[2][D / 32];  // K rows of product hf: lane holds row l16, dims 32 kk + 8 lg .. +7
  bf16x8 v[D / 16];     // V: lane holds dim 16 nt + l16, slots 8 (lg & 1) .. +7 of block lg >> 1
  uint32_t msk[2];      // slot masks of the two blocks (uniform)
};

// Issue the loads of this wave's chunk `c` (entries held lane-wise in
// pb_l/msk_l). Branch-free, so the compiler keeps the next chunk's loads in
// flight while the current one is computed: a lane whose key row is outside
// the set re-reads the row of the block's first attended slot (a line that
// is fetched anyway), and its logit is replaced by -inf; value slots outside
// the set are cleared before use (a value tile is read whole: each of its
// 32-byte dimension rows holds all 16 slots).
// The segment a chunk belongs to: its KV head, and for entries taken from a
// segment record its sequence, window start and current length.
struct SegCtx {
  int g, b, tw, T;
};

// Entry `idx` of the wave's lane-held entries (scalar). An entry from a
// segment record may be a window entry: its slots follow the current length
// and a block not yet cached at the boundary is looked up in the block table.
__device__ __forceinline__ void chunk_entry(const AttnArgs& a, const SegCtx& sc, bool from_rec,
                                            int pb_l, uint32_t msk_l, int idx, int* pb,
                                            uint32_t* msk) {
  int p = __builtin_amdgcn_readlane(pb_l, idx);
  uint32_t w = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(msk_l), idx));
  if (from_rec && (w & kWindowEntry)) {  // uniform
    const int lb = static_cast<int>(w & ~kWindowEntry);
    w = window_mask(lb, sc.tw, sc.T);
    if (p == -1 && w) p = a.block_table[static_cast<size_t>(sc.b) * a.max_blocks + lb];
    if (p < 0 || p >= a.num_blocks) {
      p = 0;
      w = 0u;
    }
  }
  *pb = p;
  *msk = w & 0xffffu;
}

template <int D, int NBW>
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const SegCtx& sc, bool from_rec,
                                           int c, int pb_l, uint32_t msk_l, Chunk<D, NBW>& ch) {
  constexpr int KS = D / 32, NT = D / 16;
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int g = sc.g;
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k_pool);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v_pool);
  int pb0, pb1;
  uint32_t m0, m1;
  chunk_entry(a, sc, from_rec, pb_l, msk_l, c * 2, &pb0, &m0);
  chunk_entry(a, sc, from_rec, pb_l, msk_l, c * 2 + 1, &pb1, &m1);
  ch.msk[0] = m0;
  ch.msk[1] = m1;
  // keys: row l16 of product hf is block l16 >> 3
  {
    const bool hi = (l16 >> 3) != 0;
    const int pb = hi ? pb1 : pb0;
    const uint32_t msk = hi ? m1 : m0;
    const int first = msk ? __builtin_ctz(msk) : 0;
    const size_t tile = static_cast<size_t>(pb) * a.Hkv + g;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int s = 8 * ((l16 >> 2) & 1) + 4 * hf + (l16 & 3);
      const int kslot = ((msk >> s) & 1u) ? s : first;
      const uint16_t* krow = kpool + (tile * kBlock + kslot) * D + 8 * lg;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk)
        ch.k[hf][kk] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(krow + 32 * kk));
    }
  }
  // values: lane group lg reads block lg >> 1, slots 8 (lg & 1) .. +7
  {
    const int pb = (lg >> 1) ? pb1 : pb0;
    const size_t tile = static_cast<size_t>(pb) * a.Hkv + g;
    const uint16_t* vcol = vpool + tile * (D * kBlock) + l16 * kBlock + 8 * (lg & 1);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
      ch.v[nt] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(vcol + nt * 16 * kBlock));
  }
}

struct MfmaState {
  float m_run;  // running max of head l16 (log2 units)
  float l_run;  // running sum of this lane's slots of head l16
  bool first;
};

// The larger of x and its copies in lanes l ^ 16 and l ^ 32 (the four lane
// groups that hold one head), with the row-swap permutes of this GPU: a swap
// of a register with itself gives each lane the values of lanes l & ~16 and
// l | 16 (then l & ~32 and l | 32), no LDS round trip.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
  const uint32_t v = __float_as_uint(x);
  const auto s32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
}

template <int G, int D, int NBW>
__device__ __forceinline__ void compute_chunk(const AttnArgs& a, Chunk<D, NBW>& ch,
                                              const bf16x8 (&qop)[D / 32], f32x4 (&o)[D / 16],
                                              MfmaState& stt) {
  constexpr int KS = D / 32, NT = D / 16;
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  // this lane group's 8 slots of its block
  const uint32_t m8 = (((lg >> 1) ? ch.msk[1] : ch.msk[0]) >> (8 * (lg & 1))) & 0xffu;
  // clear value slots outside the set (never trust their bits): one 16-bit
  // lane mask per slot; nothing to clear when both blocks are whole (uniform)
  const bool whole = (ch.msk[0] & ch.msk[1]) == 0xffffu;
  if (!whole) {
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 keep;
#pragma unroll
    for (int w = 0; w < 4; ++w)
      keep[w] = (((m8 >> (2 * w)) & 1u) ? 0x0000ffffu : 0u) |
                (((m8 >> (2 * w + 1)) & 1u) ? 0xffff0000u : 0u);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      u32x4 bits = __builtin_bit_cast(u32x4, ch.v[nt]);
      bits &= keep;
      ch.v[nt] = __builtin_bit_cast(bf16x8, bits);
    }
  }
  // S^T = K . Q^T: product hf gives this lane slots 8 (lg & 1) + 4 hf + r of
  // block lg >> 1, head l16
  float z[2][4];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ch.k[hf][kk], qop[kk], sacc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) z[hf][r] = sacc[r] * a.scale_log2;
  }
  if (!whole) {  // slots outside the set take no weight
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (!((m8 >> i) & 1u)) z[i >> 2][i & 3] = kNegInf;
  }
  float mc = kNegInf;
#pragma unroll
  for (int i = 0; i < 8; ++i) mc = fmaxf(mc, z[i >> 2][i & 3]);
  mc = max_over_lane_groups(mc);
  const float m_new = fmaxf(stt.m_run, mc);
  // rescale what this wave accumulated under the old maximum; where no
  // head's maximum moved every factor is exactly 1 (uniform skip)
  if (!stt.first && __ballot(m_new != stt.m_run) != 0ull) {
    const float alpha = m_new == kNegInf ? 1.f : exp2f(stt.m_run - m_new);
    stt.l_run *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      // O row r of lane group lg is head 4 lg + r; with G <= 4 only lane
      // group 0's rows are heads, and head r's factor is lane r's
      const float ar = G <= 4 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r))
                              : __shfl(alpha, lg * 16 + 4 * lg + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][r] *= ar;
    }
  }
  stt.m_run = m_new;
  stt.first = false;
  // 2^(z - m) with the hardware exponential (a weight below 2^-126 of the
  // largest may flush to 0): a slot outside the set (z = -inf) gives exactly
  // 0; while no slot of the head has been seen (m = -inf) subtract 0 instead,
  // so that every p is 0 and none is NaN
  const float m_sub = m_new == kNegInf ? 0.f : m_new;
  float pr[8];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pr[4 * hf + r] = __builtin_amdgcn_exp2f(z[hf][r] - m_sub);
      stt.l_run += pr[4 * hf + r];
    }
  // P as bf16 hi + lo parts (about 16 significant bits), slots in the order
  // of the value operand
  const bf16x4 h0 = pack_bf16x4(pr[0], pr[1], pr[2], pr[3]);
  const bf16x4 h1 = pack_bf16x4(pr[4], pr[5], pr[6], pr[7]);
  const bf16x4 l0 = pack_bf16x4(pr[0] - bf16_at(h0, 0), pr[1] - bf16_at(h0, 1),
                                pr[2] - bf16_at(h0, 2), pr[3] - bf16_at(h0, 3));
  const bf16x4 l1 = pack_bf16x4(pr[4] - bf16_at(h1, 0), pr[5] - bf16_at(h1, 1),
                                pr[6] - bf16_at(h1, 2), pr[7] - bf16_at(h1, 3));
  const bf16x8 phi = __builtin_shufflevector(h0, h1, 0, 1, 2, 3, 4, 5, 6, 7);
  const bf16x8 plo = __builtin_shufflevector(l0, l1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(phi, ch.v[nt], o[nt], 0, 0, 0);
    o[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(plo, ch.v[nt], o[nt], 0, 0, 0);
  }
}

// A wave's running state -> LDS slot (segment s, wave): m and l of head
// h = l16; O rows are heads 4 lg + r.
template <int G, int D>
__device__ __forceinline__ void flush_state(const MfmaState& stt, const f32x4 (&o)[D / 16],
                                            float (*red_m)[G], float (*red_l)[G],
                                            float (*red_o)[G][D]) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int l16 = lane & 15, lg = lane >> 4;
  float l_run = stt.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
  if (lg == 0 && l16 < G) {
    red_m[wave][l16] = stt.m_run;
    red_l[wave][l16] = l_run;
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int h = 4 * lg + r;
    if (h < G) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) red_o[wave][h][16 * nt + l16] = o[nt][r];
    }
  }
}

// Q^T of pair p as the B operand: lane holds head l16, dims 32 kk + 8 lg .. +7.
template <int G, int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int p, bf16x8 (&qop)[D / 32]) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int b = div_small(p, a.Hkv), g = p - b * a.Hkv;
  const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(b) * a.Hq + g * G + (l16 < G ? l16 : 0)) * D;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) qop[kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
  if (l16 < G) {  // padding heads load nothing (fewer lanes through the address unit)
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      qop[kk] = *reinterpret_cast<const bf16x8*>(qrow + 32 * kk + 8 * lg);
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs on the matrix cores (v_mfma_f32_16x16x4_f32): one block per
// chunk. S^T = K . Q^T takes, at step (t, j), d = 16 t + 4 lg + j: the lane
// (lg, l16) gives K[slot l16][d] (A) and Q[head l16][d] (B), so each lane's
// operands are the components of one 16-byte load per t, and S^T lands with
// slots 4 lg + r of head l16 in the lane (the bf16 layout's head mapping).
// P.V then takes slot 4 lg + s at step s: the lane's own weights are the A
// operand, and its value operand, 4 consecutive slots of one dimension of
// the dimension-major tile, is again one 16-byte load; O rows are heads
// 4 lg + r, as in the bf16 kernel, so states, rescaling and merging are
// shared.
// ---------------------------------------------------------------------------
template <int D>
struct ChunkF32 {
  f32x4 k[D / 16];  // K: lane holds slot l16, dims 16 t + 4 lg .. +3
  f32x4 v[D / 16];  // V: lane holds dim 16 nt + l16, slots 4 lg .. +3
  uint32_t msk;     // slot mask (uniform)
  int pb;           // physical block (uniform)
};

template <int D>
__device__ __forceinline__ void load_chunk(const AttnArgs& a, const SegCtx& sc, bool from_rec,
                                           int c, int pb_l, uint32_t msk_l, ChunkF32<D>& ch) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const float* kpool = static_cast<const float*>(a.k_pool);
  int pb;
  uint32_t m;
  chunk_entry(a, sc, from_rec, pb_l, msk_l, c, &pb, &m);
  ch.msk = m;
  ch.pb = pb;
  // a key row outside the set re-reads the block's first attended row
  const int kslot = ((m >> l16) & 1u) ? l16 : (m ? __builtin_ctz(m) : 0);
  const float* krow =
      kpool + ((static_cast<size_t>(pb) * a.Hkv + sc.g) * kBlock + kslot) * D + 4 * lg;
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
    ch.k[t] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(krow + 16 * t));
  const float* vcol = static_cast<const float*>(a.v_pool) +
                      (static_cast<size_t>(pb) * a.Hkv + sc.g) * (D * kBlock) + l16 * kBlock +
                      4 * lg;
#pragma unroll
  for (int nt = 0; nt < D / 16; ++nt)
    ch.v[nt] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vcol + nt * 16 * kBlock));
}

// The query operand is read from LDS (q[t][lane], written by this lane):
// 32 registers less over the chunk pipeline than holding it.
template <int G, int D>
__device__ __forceinline__ void compute_chunk(const AttnArgs& a, ChunkF32<D>& ch,
                                              const f32x4 (*q)[64], f32x4 (&o)[D / 16],
                                              MfmaState& stt) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63, lg = lane >> 4;
  const uint32_t m4 = (ch.msk >> (4 * lg)) & 0xfu;  // this lane's slots 4 lg .. +3
  const bool whole = ch.msk == 0xffffu;              // uniform
  f32x4 sacc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const f32x4 qv = q[t][lane];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ch.k[t][j], qv[j], sacc, 0, 0, 0);
  }
  float z[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) z[r] = sacc[r] * a.scale_log2;
  if (!whole) {  // slots outside the set take no weight
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (!((m4 >> r) & 1u)) z[r] = kNegInf;
  }
  float mc = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
  mc = max_over_lane_groups(mc);
  const float m_new = fmaxf(stt.m_run, mc);
  if (!stt.first && __ballot(m_new != stt.m_run) != 0ull) {
    const float alpha = m_new == kNegInf ? 1.f : exp2f(stt.m_run - m_new);
    stt.l_run *= alpha;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float ar = G <= 4 ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(alpha), r))
                              : __shfl(alpha, lg * 16 + 4 * lg + r);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) o[nt][r] *= ar;
    }
  }
  stt.m_run = m_new;
  stt.first = false;
  const float m_sub = m_new == kNegInf ? 0.f : m_new;
  float pr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    pr[r] = __builtin_amdgcn_exp2f(z[r] - m_sub);
    stt.l_run += pr[r];
  }
  if (!whole) {  // value slots outside the set are cleared (never trust their bits)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (!((m4 >> r) & 1u)) ch.v[nt][r] = 0.f;
  }
#pragma unroll
  for (int nt = 0; nt < NT; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      o[nt] = __builtin_amdgcn_mfma_f32_16x16x4f32(pr[r], ch.v[nt][r], o[nt], 0, 0, 0);
}

// Q^T of pair p as the B operand: lane holds head l16, dims 16 t + 4 lg .. +3.
template <int G, int D>
__device__ __forceinline__ void load_q(const AttnArgs& a, int p, f32x4 (&qop)[D / 16]) {
  const int lane = threadIdx.x & 63, l16 = lane & 15, lg = lane >> 4;
  const int b = div_small(p, a.Hkv), g = p - b * a.Hkv;
  const float* qrow = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(b) * a.Hq + g * G + (l16 < G ? l16 : 0)) * D;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) qop[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (l16 < G) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qop[t] = *reinterpret_cast<const f32x4*>(qrow + 16 * t + 4 * lg);
  }
}

// The matrix-core kernel's per-element-type pieces: chunk registers, query
// operand, blocks per chunk.
template <typename E, int D>
struct MfmaTypes;
template <int D>
struct MfmaTypes<BF16, D> {
  using CK = Chunk<D, 2>;
  using QV = bf16x8;
  static constexpr int QN = D / 32, NBW = 2;
};
template <int D>
struct MfmaTypes<F32, D> {
  using CK = ChunkF32<D>;
  using QV = f32x4;
  static constexpr int QN = D / 16, NBW = 1;
};

// One or two segments (A, then B) streamed as one sequence of chunks: the
// chunks of A, then those of B, dealt round-robin to the waves, so both
// segments share one pipeline and the waves stay balanced. A wave that
// crosses from A to B stores its A state to LDS slot 0 and starts B with
// B's query (kept in LDS: each lane reads back what it wrote itself). Three
// or more segments (short pairs) are taken one after the other.
template <typename E, int G, int D, int NBW, bool DENSE, bool REUSE>
__global__ void __launch_bounds__(kThreads, 2)
attn_mfma_kernel(AttnArgs a) {
  using CK = typename MfmaTypes<E, D>::CK;
  static_assert(NBW == MfmaTypes<E, D>::NBW, "blocks per chunk of the element type");
  using QV = typename MfmaTypes<E, D>::QV;
  constexpr int KS = MfmaTypes<E, D>::QN, NT = D / 16;
  constexpr int EPB = 64;         // entries resolved per batch (one per lane)
  constexpr int CPB = EPB / NBW;  // chunks per batch
  __shared__ float red_m[2][kWaves][G];
  __shared__ float red_l[2][kWaves][G];
  __shared__ float red_o[2][kWaves][G][D];
  // fp32: the queries stay in LDS (segment A's in q_a, B's in q_b; every
  // wave that writes one writes the same values); bf16 keeps its query in
  // registers and only B's in LDS, for a wave that crosses into B
  constexpr bool kQLds = std::is_same<E, F32>::value;
  __shared__ QV q_a[kQLds ? KS : 1][64];
  __shared__ QV q_b[KS][64];
  __shared__ PlanLds psm;

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int l16 = lane & 15;
  Assign sa, sb;
  int nseg;
  bool from_rec = false;  // segments and entries from this workgroup's record
  int rec_b = 0;          // first record entry of segment B
  if constexpr (REUSE) {
    if (blockIdx.x == 0)  // the slot bases of the records' split, for the combine kernel
      for (int i = threadIdx.x; i <= a.B * a.Hkv; i += kThreads) a.ws_pref[i] = a.reuse_pref[i];
    const ReuseRecord& rec = a.records[blockIdx.x];
    const int nr = __builtin_amdgcn_readfirstlane(rec.nseg);
    if (nr == 0) return;  // uniform
    if (nr > 0) {
      from_rec = true;
      nseg = nr;
      auto seg = [&](int s, Assign* as) {
        const int4 x = rec.seg[s][0], y = rec.seg[s][1];
        as->p = __builtin_amdgcn_readfirstlane(x.x);
        as->tw = __builtin_amdgcn_readfirstlane(x.y);
        as->ncache = __builtin_amdgcn_readfirstlane(x.z);
        as->slot = __builtin_amdgcn_readfirstlane(x.w);
        as->lo = __builtin_amdgcn_readfirstlane(y.x);
        as->hi = __builtin_amdgcn_readfirstlane(y.y);
        const int tp = __builtin_amdgcn_readfirstlane(y.w);
        const int t = a.seq_lens[div_small(as->p, a.Hkv)];
        as->T = t < 0 ? 0 : (t > tp ? tp : t);
      };
      seg(0, &sa);
      if (nr > 1) {
        seg(1, &sb);
        rec_b = __builtin_amdgcn_readfirstlane(rec.seg[1][1].z);
      }
    } else {
      // the record did not fit: the plan of zr_reuse_plan again, on the
      // boundary's lengths and settings
      a.plan_lens = a.reuse_lens;
      a.window = __builtin_amdgcn_readfirstlane(a.reuse_meta[0]);
      a.horizon = __builtin_amdgcn_readfirstlane(a.reuse_meta[1]);
      a.ws_pref = a.reuse_pref;  // (workgroup 0 would publish the same bases again)
      nseg = plan_work<DENSE>(a, psm, false, &sa, &sb);
    }
  } else {
    nseg = plan_work<DENSE>(a, psm, false, &sa, &sb);
  }
  if (nseg == 0) return;  // uniform over the workgroup

  if (nseg <= 2) {
    if (nseg == 1) {
      sb = sa;
      sb.lo = sb.hi;
    }
    const int gA = sa.p - div_small(sa.p, a.Hkv) * a.Hkv;
    const int gB = sb.p - div_small(sb.p, a.Hkv) * a.Hkv;
    const SegCtx xA{gA, div_small(sa.p, a.Hkv), sa.tw, sa.T};
    const SegCtx xB{gB, div_small(sb.p, a.Hkv), sb.tw, sb.T};
    const int nA = (sa.hi - sa.lo + NBW - 1) / NBW, nB = (sb.hi - sb.lo + NBW - 1) / NBW;
    const int ntot = nA + nB;
    const int nck_all = ntot > wave ? (ntot - wave + kWaves - 1) / kWaves : 0;
    const int iB = nA > wave ? (nA - wave + kWaves - 1) / kWaves : 0;  // this wave's A chunks
    // empty states for both segments (a wave may have chunks of one only)
    if ((lane >> 4) == 0 && l16 < G) {
      red_m[0][wave][l16] = kNegInf;
      red_m[1][wave][l16] = kNegInf;
      red_l[0][wave][l16] = 0.f;
      red_l[1][wave][l16] = 0.f;
    }
    // this wave's first query in registers; B's query goes to LDS for a wave
    // that crosses from A to B
    // one lane per entry: resolve a batch of the wave's entries at once
    int pb_l;
    uint32_t msk_l;
    auto resolve_batch = [&](int c0) {
      const int e = c0 * NBW + lane;
      const int k = (e / NBW) * kWaves + wave;  // chunk in the workgroup's sequence
      const bool inB = k >= nA;
      Assign al = inB ? sb : sa;
      const int j = inB ? sb.lo + (k - nA) * NBW + e % NBW : sa.lo + k * NBW + e % NBW;
      if (from_rec) {  // uniform: the record holds A's entries, then B's from rec_b
        pb_l = 0;
        msk_l = 0;
        if (j < al.hi) {
          const int2 r = a.records[blockIdx.x].ent[inB ? rec_b + j - sb.lo : j - sa.lo];
          pb_l = r.x;
          msk_l = static_cast<uint32_t>(r.y);
        }
      } else {
        resolve_entry<DENSE>(a, al, div_small(al.p, a.Hkv), j < al.hi ? j : -1, &pb_l, &msk_l);
      }
    };
    // the entries first: the first K/V loads wait for them, the queries are
    // needed only once those loads have returned
    resolve_batch(0);
    QV qop[KS], qb[KS];
    const bool keep_b = iB > 0 && nck_all > iB;  // this wave crosses from A to B
    const QV(*qsrc)[64] = q_a;
    if constexpr (kQLds) {
      if (iB > 0) load_q<G, D>(a, sa.p, qop);
      if (nck_all > iB) load_q<G, D>(a, sb.p, qb);
      if (iB > 0) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q_a[kk][lane] = qop[kk];
      }
      if (nck_all > iB) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q_b[kk][lane] = qb[kk];
      }
      qsrc = iB > 0 ? q_a : q_b;
    } else {
      load_q<G, D>(a, iB > 0 ? sa.p : sb.p, qop);
      if (keep_b) load_q<G, D>(a, sb.p, qb);
    }
    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    MfmaState stt{kNegInf, 0.f, true};

    for (int c0 = 0; c0 < nck_all; c0 += CPB) {
      if (c0 > 0) resolve_batch(c0);
      const int nck = nck_all - c0 < CPB ? nck_all - c0 : CPB;
      // chunk c of the batch is this wave's chunk c0 + c: in A while < iB.
      // Before computing the first chunk of B the wave stores its A state
      // and starts over with B's query (checked ahead of the next chunk's
      // loads, so that loads and matrix work stay in one block of code).
      auto switch_at = [&](int c) {
        if (c0 + c == iB && iB > 0) {
          flush_state<G, D>(stt, o, red_m[0], red_l[0], red_o[0]);
          if constexpr (kQLds) {
            qsrc = q_b;
          } else {
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) qop[kk] = q_b[kk][lane];
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
          stt = MfmaState{kNegInf, 0.f, true};
        }
      };
      auto compute = [&](CK& ch) {
        if constexpr (kQLds)
          compute_chunk<G, D>(a, ch, qsrc, o, stt);
        else
          compute_chunk<G, D>(a, ch, qop, o, stt);
      };
      CK cA, cB;
      load_chunk(a, c0 < iB ? xA : xB, from_rec, 0, pb_l, msk_l, cA);
      if (!kQLds && c0 == 0 && keep_b) {  // B's query to LDS once the first loads are out
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) q_b[kk][lane] = qb[kk];
      }
      for (int c = 0; c < nck; c += 2) {
        switch_at(c);
        if (c + 1 < nck)
          load_chunk(a, c0 + c + 1 < iB ? xA : xB, from_rec, c + 1, pb_l, msk_l, cB);
        compute(cA);
        if (c + 1 < nck) {
          switch_at(c + 1);
          if (c + 2 < nck)
            load_chunk(a, c0 + c + 2 < iB ? xA : xB, from_rec, c + 2, pb_l, msk_l, cA);
          compute(cB);
        }
      }
    }
    if (nck_all > 0) {
      const int s = nck_all > iB ? 1 : 0;  // the segment of this wave's last chunk
      flush_state<G, D>(stt, o, red_m[s], red_l[s], red_o[s]);
    }
    __syncthreads();
    write_partial<G, D>(a, sa.slot, red_m[0], red_l[0], red_o[0]);
    if (nseg == 2) write_partial<G, D>(a, sb.slot, red_m[1], red_l[1], red_o[1]);
    return;
  }

  // three or more segments: one after the other, one chunk in flight
  int nrec = psm.nrec, ri = 0;
  for (int si = 0; si < nseg; ++si) {
    if (si > 0) __syncthreads();  // the previous segment's LDS results have been read
    if (ri == nrec) {             // uniform
      nrec = plan_next<DENSE>(a, psm);
      ri = 0;
    }
    Assign as;
    get_record(psm, ri++, &as);
    const int b = div_small(as.p, a.Hkv), g = as.p - b * a.Hkv;
    const int nck_all = wave_chunks<NBW>(as, wave);
    int pb_l;
    uint32_t msk_l;
    auto resolve_batch = [&](int c0) {
      resolve_entry<DENSE>(a, as, b, wave_entry<NBW>(as, wave, c0 * NBW + lane), &pb_l, &msk_l);
    };
    resolve_batch(0);  // the entries before the query, as in the streamed path
    QV qop[KS];
    load_q<G, D>(a, as.p, qop);
    if constexpr (kQLds) {  // (every wave writes the segment's query: same values)
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) q_a[kk][lane] = qop[kk];
    }
    f32x4 o[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) o[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    MfmaState stt{kNegInf, 0.f, true};
    for (int c0 = 0; c0 < nck_all; c0 += CPB) {
      if (c0 > 0) resolve_batch(c0);
      const int nck = nck_all - c0 < CPB ? nck_all - c0 : CPB;
      for (int c = 0; c < nck; ++c) {
        CK ch;
        load_chunk(a, SegCtx{g, b, as.tw, as.T}, false, c, pb_l, msk_l, ch);
        if constexpr (kQLds)
          compute_chunk<G, D>(a, ch, q_a, o, stt);
        else
          compute_chunk<G, D, NBW>(a, ch, qop, o, stt);
      }
    }
    flush_state<G, D>(stt, o, red_m[0], red_l[0], red_o[0]);
    __syncthreads();
    write_partial<G, D>(a, as.slot, red_m[0], red_l[0], red_o[0]);
  }
}

// ---------------------------------------------------------------------------
// Combine: merge the partials of pair (b, g) (workgroups [ws_pref[p],
// ws_pref[p+1])) by log-sum-exp,
//   out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s,  M = max_s m_s.
// Each thread owns four consecutive dimensions of one head and reads a tile
// of partials with independent 16-byte loads (slot indices clamped, so the
// loads need no branches), merging tiles online.
// ---------------------------------------------------------------------------
constexpr int kCombineThreads = 512;

// Log-sum-exp merge state of one item (4 dims of one head).
struct MergeState {
  float M, L;
  float4 A;
};

// Merge slots [c0, s1) of one item, tiles of TILE slots taken `stride`
// slots apart, into st.
template <int G, int D, int TILE>
__device__ __forceinline__ void merge_slots(const AttnArgs& a, int h, int e4, int c0, int s1,
                                            int stride, MergeState& st) {
  constexpr int D4 = D / 4;
  const float4* acc4 = reinterpret_cast<const float4*>(a.ws_acc);
  for (; c0 < s1; c0 += stride) {
    float ms[TILE], ls[TILE];
    float4 vs[TILE];
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      const size_t s = static_cast<size_t>(c0 + u < s1 ? c0 + u : s1 - 1);
      ms[u] = a.ws_m[s * G + h];
      ls[u] = a.ws_l[s * G + h];
      vs[u] = acc4[(s * G + h) * D4 + e4];
      if (c0 + u >= s1) ms[u] = kNegInf;
    }
    float mt = st.M;
#pragma unroll
    for (int u = 0; u < TILE; ++u) mt = fmaxf(mt, ms[u]);
    if (mt == kNegInf) continue;
    const float alpha = st.M == kNegInf ? 0.f : exp2f(st.M - mt);
    st.L *= alpha;
    st.A.x *= alpha;
    st.A.y *= alpha;
    st.A.z *= alpha;
    st.A.w *= alpha;
#pragma unroll
    for (int u = 0; u < TILE; ++u) {
      const float w = ms[u] != kNegInf ? exp2f(ms[u] - mt) : 0.f;
      st.L = fmaf(ls[u], w, st.L);
      st.A.x = fmaf(vs[u].x, w, st.A.x);
      st.A.y = fmaf(vs[u].y, w, st.A.y);
      st.A.z = fmaf(vs[u].z, w, st.A.z);
      st.A.w = fmaf(vs[u].w, w, st.A.w);
    }
    st.M = mt;
  }
}

// One workgroup per pair. When a pair's items (G heads x D/4) leave threads
// over, NGRP groups of threads take the tiles of partials in turn (so up to
// NGRP tiles are loaded at once) and merge their states through LDS. TILE
// (slots per tile) is chosen per launch: the smaller tile when one round of
// NGRP tiles still covers a pair's average slot count (fewer loads per
// thread), else the larger one (fewer rounds).
template <int G, int D>
constexpr int combine_groups() {
  return G * (D / 4) < kCombineThreads ? kCombineThreads / (G * (D / 4)) : 1;
}

template <int G, int D, int TILE>
__global__ void __launch_bounds__(kCombineThreads)
attn_combine_kernel(AttnArgs a) {
  constexpr int D4 = D / 4, ITEMS = G * D4;
  constexpr int PER = (ITEMS + kCombineThreads - 1) / kCombineThreads;
  constexpr int NGRP = combine_groups<G, D>();
  __shared__ MergeState sh[NGRP > 1 ? (NGRP - 1) * ITEMS : 1];
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int p = b * a.Hkv + g;
  // slot range of the pair, kept inside this layout's nwg + P slots (a range
  // written under another layout then reads wrong values, but no memory
  // outside the workspace)
  const int cap = a.nwg + a.B * a.Hkv;
  const int r0 = a.ws_pref[p], r1 = a.ws_pref[p + 1];
  const int s0 = r0 < 0 ? 0 : (r0 > cap ? cap : r0);
  const int s1 = r1 < s0 ? s0 : (r1 > cap ? cap : r1);
  float4* out4 = reinterpret_cast<float4*>(a.out + (static_cast<size_t>(b) * a.Hq + g * G) * D);
  auto finish = [&](int idx, const MergeState& st) {
    const float inv = st.L > 0.f ? 1.f / st.L : 0.f;
    out4[idx] = st.L > 0.f ? make_float4(st.A.x * inv, st.A.y * inv, st.A.z * inv, st.A.w * inv)
                           : make_float4(0.f, 0.f, 0.f, 0.f);
  };
  if constexpr (NGRP > 1) {
    const int grp = t / ITEMS, idx = t - grp * ITEMS;
    const int h = idx / D4, e4 = idx % D4;
    MergeState st{kNegInf, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
    merge_slots<G, D, TILE>(a, h, e4, s0 + grp * TILE, s1, NGRP * TILE, st);
    if (s1 - s0 <= TILE) {  // one tile: group 0 holds everything (uniform)
      if (grp == 0) finish(idx, st);
      return;
    }
    if (grp > 0) sh[(grp - 1) * ITEMS + idx] = st;
    __syncthreads();
    if (grp > 0) return;
#pragma unroll
    for (int k = 0; k < NGRP - 1; ++k) {
      const MergeState o = sh[k * ITEMS + idx];
      if (o.M == kNegInf) continue;
      const float mt = fmaxf(st.M, o.M);
      const float fa = st.M == kNegInf ? 0.f : exp2f(st.M - mt), fb = exp2f(o.M - mt);
      st.L = st.L * fa + o.L * fb;
      st.A.x = st.A.x * fa + o.A.x * fb;
      st.A.y = st.A.y * fa + o.A.y * fb;
      st.A.z = st.A.z * fa + o.A.z * fb;
      st.A.w = st.A.w * fa + o.A.w * fb;
      st.M = mt;
    }
    finish(idx, st);
  } else {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int idx = t + j * kCombineThreads;
      if (idx >= ITEMS) continue;
      MergeState st{kNegInf, 0.f, make_float4(0.f, 0.f, 0.f, 0.f)};
      merge_slots<G, D, TILE>(a, idx / D4, idx % D4, s0, s1, TILE, st);
      finish(idx, st);
    }
  }
}

// ---------------------------------------------------------------------------
// Segment records for the attention calls between semantic boundaries (ZoomR
// Sec. 3.4: the attended set is rebuilt only at a boundary, while the window
// keeps growing): the split an attention call would plan on the current
// lengths T0 with the window planned through T0 + horizon, and each
// workgroup's segments with their list entries resolved (window entries keep
// their logical block, their slots follow the length of each later call).
// One workgroup per attention workgroup; a workgroup whose share has more
// than two segments or kRecEntries entries is marked for planning in the
// kernel. Workgroup 0 keeps the lengths and settings that planning needs
// and publishes the slot bases the combine kernel reads.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
reuse_plan_kernel(AttnArgs a) {
  __shared__ PlanLds psm;
  const int w = blockIdx.x, t = threadIdx.x;
  if (w == 0) {
    for (int b = t; b < a.B; b += kThreads) a.reuse_lens[b] = a.seq_lens[b];
    if (t == 0) {
      a.reuse_meta[0] = a.window;
      a.reuse_meta[1] = a.horizon;
    }
  }
  Assign sa, sb;
  const int nseg = plan_work<false>(a, psm, true, &sa, &sb);
  ReuseRecord& rec = a.records[w];
  const int nA = nseg >= 1 ? sa.hi - sa.lo : 0, nB = nseg >= 2 ? sb.hi - sb.lo : 0;
  const bool fits = nseg <= 2 && nA + nB <= kRecEntries;
  const int cap = a.max_blocks * kBlock;
  if (t == 0) {
    rec.nseg = fits ? nseg : -1;
    if (fits) {
      for (int i = 0; i < nseg; ++i) {
        const Assign& as = i ? sb : sa;
        const int tp = as.T + a.horizon < cap ? as.T + a.horizon : cap;
        rec.seg[i][0] = make_int4(as.p, as.tw, as.ncache, as.slot);
        rec.seg[i][1] = make_int4(as.lo, as.hi, i ? nA : 0, tp);
      }
    }
  }
  if (!fits) return;
  for (int e = t; e < nA + nB; e += kThreads) {
    const bool inB = e >= nA;
    const int p = inB ? sb.p : sa.p, tw = inB ? sb.tw : sa.tw, nc = inB ? sb.ncache : sa.ncache;
    const int T0 = inB ? sb.T : sa.T;
    const int j = inB ? sb.lo + (e - nA) : sa.lo + e;
    int2 r;
    if (j < nc) {
      const int2 en = a.entries[static_cast<size_t>(p) * a.max_blocks + j];
      const bool ok = en.x >= 0 && en.x < a.num_blocks;
      r = ok ? make_int2(en.x, en.y & 0xffff) : make_int2(0, 0);
    } else {
      // a window block: cached at the boundary (its id now), or not yet (-1)
      const int lb = (tw >> 4) + (j - nc);
      int blk = -1;
      if ((lb << 4) < T0) {
        blk = a.block_table[static_cast<size_t>(div_small(p, a.Hkv)) * a.max_blocks + lb];
        blk = blk >= 0 && blk < a.num_blocks ? blk : -2;  // -2: never read
      }
      r = make_int2(blk, static_cast<int>(static_cast<uint32_t>(lb) | kWindowEntry));
    }
    rec.ent[e] = r;
  }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

int attn_workgroups(const zr_geom& gm, int32_t max_attended) {
  const int64_t pairs = static_cast<int64_t>(gm.batch) * gm.n_kv_heads;
  const int64_t blocks = pairs * ((static_cast<int64_t>(max_attended) + kBlock - 1) / kBlock + 2);
  int64_t n = (blocks + kMinBlocksPerWg - 1) / kMinBlocksPerWg;
  if (n < 1) n = 1;
  if (n > kTargetWorkgroups) n = kTargetWorkgroups;
  return static_cast<int>(n);
}

size_t attn_workspace(const zr_geom& gm, int nwg, void* ws, AttnArgs* a) {
  const size_t G = static_cast<size_t>(gm.n_q_heads / gm.n_kv_heads);
  const size_t P = static_cast<size_t>(gm.batch) * gm.n_kv_heads;
  const size_t slots = static_cast<size_t>(nwg) + P;
  auto up16 = [](size_t x) { return (x + 15) & ~static_cast<size_t>(15); };
  const size_t pref_b = up16((P + 1) * sizeof(int32_t));
  const size_t cnt_b = up16(P * sizeof(int32_t));
  const size_t ltw_b = cnt_b;
  const size_t ent_b = P * static_cast<size_t>(gm.max_blocks_per_seq) * sizeof(int2);
  const size_t ml_b = up16(slots * G * sizeof(float));
  const size_t acc_b = slots * G * gm.head_dim * sizeof(float);
  static_assert(sizeof(ReuseRecord) % 16 == 0, "records keep the regions 16-byte aligned");
  const size_t rec_b = static_cast<size_t>(nwg) * sizeof(ReuseRecord);
  const size_t rlen_b = up16(static_cast<size_t>(gm.batch) * sizeof(int32_t));
  const size_t rpref_b = pref_b;
  const size_t meta_b = 4 * sizeof(int32_t);
  if (ws && a) {
    char* c = static_cast<char*>(ws);
    a->ws_pref = reinterpret_cast<int32_t*>(c);
    c += pref_b;
    a->counts = reinterpret_cast<int32_t*>(c);
    c += cnt_b;
    a->list_tw = reinterpret_cast<int32_t*>(c);
    c += ltw_b;
    a->entries = reinterpret_cast<int2*>(c);
    c += ent_b;
    a->ws_m = reinterpret_cast<float*>(c);
    c += ml_b;
    a->ws_l = reinterpret_cast<float*>(c);
    c += ml_b;
    a->ws_acc = reinterpret_cast<float*>(c);
    c += acc_b;
    a->records = reinterpret_cast<ReuseRecord*>(c);
    c += rec_b;
    a->reuse_lens = reinterpret_cast<int32_t*>(c);
    c += rlen_b;
    a->reuse_pref = reinterpret_cast<int32_t*>(c);
    c += rpref_b;
    a->reuse_meta = reinterpret_cast<int32_t*>(c);
    a->nwg = nwg;
  }
  return pref_b + cnt_b + ltw_b + ent_b + 2 * ml_b + acc_b + rec_b + rlen_b + rpref_b + meta_b;
}

// What a launch runs: the attention kernel (partials into the workspace), the
// combine kernel (partials -> out), or both in turn.
enum AttnParts { kAttnOnly = 1, kCombineOnly = 2, kAttnAndCombine = 3 };

template <int G, int D>
static hipError_t launch_combine_gd(const zr_geom& gm, const AttnArgs& a, hipStream_t s) {
  // a pair's partial slots: about nwg / P, plus one where ranges meet
  const int pairs = gm.batch * gm.n_kv_heads;
  const int per_pair = (a.nwg + 2 * pairs - 1) / pairs;
  const dim3 grid(gm.n_kv_heads, gm.batch);
  if (per_pair <= combine_groups<G, D>() * 4)
    hipLaunchKernelGGL((attn_combine_kernel<G, D, 4>), grid, dim3(kCombineThreads), 0, s, a);
  else
    hipLaunchKernelGGL((attn_combine_kernel<G, D, 8>), grid, dim3(kCombineThreads), 0, s, a);
  return hipGetLastError();
}

// Which attention kernel: sparse (lists + window), dense (every block), or
// sparse between semantic boundaries (segment records).
enum AttnKind { kSparse = 0, kDense = 1, kReuse = 2 };

template <typename E, int G, int D>
static hipError_t launch_mfma(const zr_geom& gm, const AttnArgs& a, int kind, int parts,
                              hipStream_t s) {
  constexpr int NBW = MfmaTypes<E, D>::NBW;
  if (parts & kAttnOnly) {
    const dim3 grid(a.nwg);
    if (kind == kDense)
      hipLaunchKernelGGL((attn_mfma_kernel<E, G, D, NBW, true, false>), grid, dim3(kThreads), 0,
                         s, a);
    else if (kind == kReuse)
      hipLaunchKernelGGL((attn_mfma_kernel<E, G, D, NBW, false, true>), grid, dim3(kThreads), 0,
                         s, a);
    else
      hipLaunchKernelGGL((attn_mfma_kernel<E, G, D, NBW, false, false>), grid, dim3(kThreads), 0,
                         s, a);
    const hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return (parts & kCombineOnly) ? launch_combine_gd<G, D>(gm, a, s) : hipSuccess;
}

template <int D>
static hipError_t launch_d(const zr_geom& gm, const AttnArgs& a, int kind, int parts,
                           hipStream_t s) {
  const int G = gm.n_q_heads / gm.n_kv_heads;
  if (gm.dtype == ZR_BF16) {
    switch (G) {
      case 1: return launch_mfma<BF16, 1, D>(gm, a, kind, parts, s);
      case 2: return launch_mfma<BF16, 2, D>(gm, a, kind, parts, s);
      case 4: return launch_mfma<BF16, 4, D>(gm, a, kind, parts, s);
      case 8: return launch_mfma<BF16, 8, D>(gm, a, kind, parts, s);
      case 16: return launch_mfma<BF16, 16, D>(gm, a, kind, parts, s);
      default: return hipErrorInvalidValue;
    }
  }
  switch (G) {
    case 1: return launch_mfma<F32, 1, D>(gm, a, kind, parts, s);
    case 2: return launch_mfma<F32, 2, D>(gm, a, kind, parts, s);
    case 4: return launch_mfma<F32, 4, D>(gm, a, kind, parts, s);
    case 8: return launch_mfma<F32, 8, D>(gm, a, kind, parts, s);
    case 16: return launch_mfma<F32, 16, D>(gm, a, kind, parts, s);
    default: return hipErrorInvalidValue;
  }
}

static hipError_t launch_parts(const zr_geom& gm, const AttnArgs& a, int kind, int parts,
                               hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  return gm.head_dim == 128 ? launch_d<128>(gm, a, kind, parts, s)
                            : launch_d<64>(gm, a, kind, parts, s);
}

hipError_t launch_attention(const zr_geom& gm, const AttnArgs& a, bool dense, hipStream_t s) {
  return launch_parts(gm, a, dense ? kDense : kSparse, kAttnAndCombine, s);
}

hipError_t launch_attention_partials(const zr_geom& gm, const AttnArgs& a, hipStream_t s) {
  return launch_parts(gm, a, kSparse, kAttnOnly, s);
}

hipError_t launch_combine(const zr_geom& gm, const AttnArgs& a, hipStream_t s) {
  return launch_parts(gm, a, kSparse, kCombineOnly, s);
}

hipError_t launch_reuse_plan(const zr_geom& gm, const AttnArgs& a, hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(reuse_plan_kernel, dim3(a.nwg), dim3(kThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attention_reuse(const zr_geom& gm, const AttnArgs& a, hipStream_t s) {
  return launch_parts(gm, a, kReuse, a.out ? kAttnAndCombine : kAttnOnly, s);
}

}  // namespace zr

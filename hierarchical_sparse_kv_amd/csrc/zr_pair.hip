// Per-(sequence, KV head) work before attention: coarse scores, top-k
// selection and the attended-block list, in one workgroup per pair.
//
// Scoring follows ZoomR Sec. 3.3 (eq. alpha): the inner product of the decode
// query with each thought's mean summary key. With grouped-query attention
// one score is kept per KV head: the query heads of the group are summed
// first (their sum dotted with the key equals the sum of the per-head
// scores). Products and sums run in float64 so the float32 result does not
// depend on the summation order for bf16 inputs (products and partial sums
// are exact there for inputs of ordinary range); the float32 scores are what
// the selector compares.
//
// Selection follows ZoomR Sec. 3.3 (eq. I_top-k) under the total order
// (score descending, thought index ascending) on order-preserving 32-bit
// keys: up to 256 thoughts each thread ranks its own thought by counting the
// thoughts ahead of it; beyond that a radix select finds the k-th key and
// the ties at it are taken lowest index first. Winners are emitted in
// ascending thought index.
//
// The attended set is the union of the window [T - W, T) and the selected
// thoughts' spans clipped below T - W (ZoomR Sec. 3.3 eq. I_f restricted to
// the window and full-resolution spans). The spans part is built here as a
// bitmap of slot masks, one 16-bit mask per logical block of the paged
// cache, so tokens shared by several spans count once whatever the order of
// `sel`. The non-empty blocks, resolved through the block table (KV-cache
// management page, paged KV cache, eq. 4), form the pair's list of (physical
// block, slot mask) entries; the attention kernel appends the window's
// blocks itself, so a list stays valid while the window grows between
// semantic boundaries (ZoomR Sec. 3.4).
//
// The four modes (template flags) share this code:
//   SCORE            scores only                       (zr_coarse_score)
//   SELECT           top-k from given scores           (zr_select_topk)
//   PLAN             block list from a given sel       (zr_sparse_decode_attn)
//   SCORE+SELECT+PLAN the whole pre-attention step      (zr_sparse_decode_step)
#include "zr_internal.h"

namespace zr {

constexpr int kPairThreads = 256;
constexpr int kPairWaves = kPairThreads / 64;
constexpr int kRankMax = kPairThreads;  // up to this many thoughts: ranking by counting
constexpr int kBtRegs = 16;             // block-table entries prefetched per thread
constexpr int kSelRegs = (ZR_MAX_K + kPairThreads - 1) / kPairThreads;  // given sel per thread
constexpr int kMaxGroup = 16;           // query heads per KV head
constexpr int kScoreR = 4;              // summary-key rows in flight per lane

// Summary-key rows one scoring batch covers (all lanes, kScoreR rows each).
template <typename E, int D>
constexpr int score_batch_rows() {
  return kPairThreads / (D / (16 / E::kBytes)) * kScoreR;
}

// Larger key = better score. NaN maps below every number; -0 maps like +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int blocks_of_span(int s, int e) {
  return e > s ? ((e - 1) >> 4) - (s >> 4) + 1 : 0;
}

// Dynamic LDS (int32 units), each region 4-int aligned:
//   keys[max(max_per_seq, kRankMax)]  SELECT (order keys, zero padded)
//   th_s[max_per_seq] th_l[...]       PLAN with staged thought spans
//   sel_l[k]                          PLAN
//   bmask[ceil(max_blocks / 2)]       PLAN (two 16-bit slot masks per int)
__host__ __device__ inline int up4(int x) { return (x + 3) & ~3; }

// Size of the keys region: ranking reads up to kRankMax padded entries.
__host__ __device__ inline int keys_ints(int max_per_seq) {
  return up4(max_per_seq) > kRankMax ? up4(max_per_seq) : kRankMax;
}

// Block-table entries (and 16-bit bitmap slots) owned by each thread: up to
// kBtRegs per thread they are prefetched into registers, and the count is
// rounded up to a power of two from 2 so that a thread owns whole bitmap
// words (bt_per / 2 of them, read and cleared with one vector access).
__host__ __device__ inline int pair_bt_per(int max_blocks) {
  int bt = (max_blocks + kPairThreads - 1) / kPairThreads;
  if (bt > kBtRegs) return bt;
  int r = 2;
  while (r < bt) r <<= 1;
  return r;
}

// Size of the bitmap region: every thread's whole words when prefetching,
// else one word per two blocks.
__host__ __device__ inline int bmask_ints(int max_blocks) {
  const int bt = pair_bt_per(max_blocks);
  return bt <= kBtRegs ? kPairThreads * bt / 2 : up4((max_blocks + 1) / 2);
}

struct PairLds {
  uint32_t* keys;
  int32_t* th_s;
  int32_t* th_l;
  int32_t* sel_l;
  uint32_t* bmask;
};

__host__ __device__ inline size_t pair_lds_ints(int max_per_seq, int k, int max_blocks,
                                                bool select, bool plan, bool stage_th) {
  size_t n = 0;
  if (select) n += keys_ints(max_per_seq);
  if (plan) {
    if (stage_th) n += 2 * static_cast<size_t>(up4(max_per_seq));
    n += up4(k);
    n += bmask_ints(max_blocks);
  }
  return n;
}

__device__ inline PairLds pair_lds(int32_t* dyn, int max_per_seq, int k, bool select, bool plan,
                                   bool stage_th) {
  PairLds L{};
  int32_t* c = dyn;
  if (select) {
    L.keys = reinterpret_cast<uint32_t*>(c);
    c += keys_ints(max_per_seq);
  }
  if (plan) {
    if (stage_th) {
      L.th_s = c;
      c += up4(max_per_seq);
      L.th_l = c;
      c += up4(max_per_seq);
    }
    L.sel_l = c;
    c += up4(k);
    L.bmask = reinterpret_cast<uint32_t*>(c);
  }
  return L;
}

// ---------------------------------------------------------------------------
// Selection of the k best of n keys (n > k), written in ascending index to
// L.sel_l (when PLAN) and to `out` (k ints).
// ---------------------------------------------------------------------------

// n <= kRankMax: thought i is ranked by counting the thoughts ahead of it
// (a larger key, or the same key and a lower index); the k of rank < k win.
// The keys are padded with zeros to np, a power of two from 32 to kRankMax
// (a zero key at an index past n is never ahead of a real thought), and
// S = kRankMax / np consecutive lanes share thought i, each counting over
// np / S keys with 16-byte LDS reads, so that few reads are in flight per
// lane before the counts are summed across the S lanes with DPP.
__device__ __forceinline__ int rank_pad(int n) {
  int np = 32;
  while (np < n) np <<= 1;
  return np;
}

// Entries of L.keys that must hold a key or a zero before a selection.
__device__ __forceinline__ int keys_fill(int n) { return n <= kRankMax ? rank_pad(n) : up4(n); }

template <bool PLAN>
__device__ void select_by_rank(const PairLds& L, int n, int k, int32_t* out, int* wtmp) {
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int np = rank_pad(n);
  const int lgS = 8 - (31 - __builtin_clz(np));  // kRankMax = 256 = 2^8
  const int S = 1 << lgS;
  const int i = t >> lgS, q = t & (S - 1);
  const int per4 = np >> (2 + lgS);  // 16-byte reads per lane
  const uint32_t ki = L.keys[i];
  const uint32_t ki1 = ki + 1u;      // keys at or after i must beat ki (no wrap: NaN -> 0, +inf < 2^32 - 1)
  const uint4* k4 = reinterpret_cast<const uint4*>(L.keys) + q * per4;
  int j = q * per4 * 4;
  int cnt = 0;
#pragma unroll 4
  for (int r = 0; r < per4; ++r, j += 4) {
    const uint4 v = k4[r];
    cnt += v.x >= (j < i ? ki : ki1) ? 1 : 0;
    cnt += v.y >= (j + 1 < i ? ki : ki1) ? 1 : 0;
    cnt += v.z >= (j + 2 < i ? ki : ki1) ? 1 : 0;
    cnt += v.w >= (j + 3 < i ? ki : ki1) ? 1 : 0;
  }
  if (S >= 2) cnt += dpp_move<0xb1>(cnt);   // quad_perm [1,0,3,2]
  if (S >= 4) cnt += dpp_move<0x4e>(cnt);   // quad_perm [2,3,0,1]
  if (S >= 8) cnt += dpp_move<0x141>(cnt);  // half-row mirror: the other quad
  const bool take = q == 0 && i < n && cnt < k;
  const uint64_t bal = __ballot(take);
  if (lane == 0) wtmp[wave] = __popcll(bal);
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < kPairWaves; ++w) before += w < wave ? wtmp[w] : 0;
  if (take) {
    const int pos = before + __popcll(bal & ((1ull << lane) - 1ull));
    out[pos] = i;
    if (PLAN) L.sel_l[pos] = i;
  }
}

// General n: radix select (most significant byte first) finds the k-th key
// and how many keys equal to it still belong to the top k; two scans then
// compact the winners in index order. Each thread owns a contiguous run of
// indices so that the scans follow index order.
template <bool PLAN>
__device__ void select_by_radix(const PairLds& L, int n, int k, int32_t* out, uint32_t* hist,
                                int* wtmp, uint32_t* sh) {
  const int t = threadIdx.x, lane = t & 63;
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;  // kPairThreads == 256 bins
    __syncthreads();
    for (int i = t; i < n; i += kPairThreads) {
      const uint32_t key = L.keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (t < 64) {
      // lane owns digits 4 lane .. 4 lane + 3; find the digit d where the
      // count of keys with a larger digit is < remaining <= that + hist[d]
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suffix = mine;  // keys in digits >= 4 lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_down(suffix, o);
        if (lane + o < 64) suffix += x;
      }
      const unsigned long long hit = __ballot(suffix >= remaining);
      const int last = 63 - __clzll(hit);  // last lane whose suffix still covers k
      if (lane == last) {
        uint32_t above = suffix - mine;
        const uint32_t c[4] = {c0, c1, c2, c3};
        int digit = 4 * lane;
        for (int dd = 3; dd >= 0; --dd) {
          if (above + c[dd] >= remaining || dd == 0) {
            digit = 4 * lane + dd;
            break;
          }
          above += c[dd];
        }
        sh[0] = prefix | (static_cast<uint32_t>(digit) << shift);
        sh[1] = remaining - above;
      }
    }
    __syncthreads();
    prefix = sh[0];
    remaining = sh[1];
    mask |= 0xffu << shift;
  }
  const uint32_t kth = prefix;
  const int per = (n + kPairThreads - 1) / kPairThreads;
  const int i0 = t * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  int n_eq = 0;
  for (int i = i0; i < i1; ++i) n_eq += L.keys[i] == kth;
  int tot;
  const int eq_before = wg_exclusive_scan<kPairWaves>(n_eq, wtmp, &tot);
  int n_sel = 0;
  {
    int r = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = L.keys[i];
      if (key > kth) {
        ++n_sel;
      } else if (key == kth) {
        n_sel += r < static_cast<int>(remaining);
        ++r;
      }
    }
  }
  int pos = wg_exclusive_scan<kPairWaves>(n_sel, wtmp, &tot);
  {
    int r = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = L.keys[i];
      bool take = false;
      if (key > kth) {
        take = true;
      } else if (key == kth) {
        take = r < static_cast<int>(remaining);
        ++r;
      }
      if (take && pos < k) {
        out[pos] = i;
        if (PLAN) L.sel_l[pos] = i;
        ++pos;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Block lists from a slot bitmap
// ---------------------------------------------------------------------------

// OR the slots of tokens [s, e) into the bitmap, blocks j0, j0 + step, ...
// of the span (so a workgroup can share one span's blocks).
__device__ __forceinline__ void or_span(uint32_t* bmask, int s, int e, int j0, int step) {
  const int nbk = blocks_of_span(s, e);
  for (int j = j0; j < nbk; j += step) {
    const int lb = (s >> 4) + j;
    const int b0 = lb << 4;
    const int from = (s > b0 ? s : b0) - b0;
    const int to = (e < b0 + kBlock ? e : b0 + kBlock) - b0;
    const uint32_t m = ((1u << to) - 1u) & ~((1u << from) - 1u);
    atomicOr(&bmask[lb >> 1], m << (16 * (lb & 1)));
  }
}

// Bitmap words owned by this thread (bt_per <= kBtRegs): W of them from
// word threadIdx.x * W, as 4-, 8- or 16-byte LDS accesses.
template <int W>
__device__ __forceinline__ void own_words_load(const uint32_t* bmask, uint32_t (&w)[W]) {
  const uint32_t* src = bmask + threadIdx.x * W;
  if constexpr (W == 1) {
    w[0] = src[0];
  } else if constexpr (W == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    w[0] = v.x;
    w[1] = v.y;
  } else {
#pragma unroll
    for (int c = 0; c < W; c += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(src + c);
      w[c] = v.x;
      w[c + 1] = v.y;
      w[c + 2] = v.z;
      w[c + 3] = v.w;
    }
  }
}

template <int W>
__device__ __forceinline__ void own_words_clear(uint32_t* bmask) {
  uint32_t* dst = bmask + threadIdx.x * W;
  if constexpr (W == 1) {
    dst[0] = 0u;
  } else if constexpr (W == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(0u, 0u);
  } else {
#pragma unroll
    for (int c = 0; c < W; c += 4) *reinterpret_cast<uint4*>(dst + c) = make_uint4(0u, 0u, 0u, 0u);
  }
}

// Zero the bitmap before the spans are ORed in: each thread its own words
// when bt_per <= kBtRegs (the whole region), else the words of nb blocks.
__device__ __forceinline__ void clear_bitmap(uint32_t* bmask, int bt_per, int nb) {
  switch (bt_per) {
    case 2: own_words_clear<1>(bmask); break;
    case 4: own_words_clear<2>(bmask); break;
    case 8: own_words_clear<4>(bmask); break;
    case 16: own_words_clear<8>(bmask); break;
    default:
      for (int i = threadIdx.x; i < (nb + 1) / 2; i += kPairThreads) bmask[i] = 0u;
  }
}

// The non-empty blocks of the bitmap in logical order -> the pair's list of
// (physical block, slot mask) entries and its length, with the block ids
// prefetched into registers: thread t owns blocks [2Wt, 2W(t + 1)), whose
// masks stay in registers between the count and the writes. Blocks past the
// sequence have empty masks (the region is cleared whole).
template <int W>
__device__ void emit_list_regs(const PairArgs& a, int p, const uint32_t* bmask,
                               const int (&btr)[kBtRegs], int* wtmp) {
  uint32_t w[W];
  own_words_load<W>(bmask, w);
  int nz = 0;
#pragma unroll
  for (int j = 0; j < W; ++j) nz += ((w[j] & 0xffffu) != 0u ? 1 : 0) + ((w[j] >> 16) != 0u ? 1 : 0);
  int n_list;
  int pos = wg_exclusive_scan<kPairWaves, false>(nz, wtmp, &n_list);
  int2* ent = a.entries + static_cast<size_t>(p) * a.max_blocks;
#pragma unroll
  for (int j = 0; j < 2 * W; ++j) {
    const uint32_t m = (w[j >> 1] >> (16 * (j & 1))) & 0xffffu;
    if (m) {
      const int pb = btr[j];
      const bool ok = pb >= 0 && pb < a.num_blocks;
      ent[pos++] = ok ? make_int2(pb, static_cast<int>(m)) : make_int2(0, 0);
    }
  }
  if (threadIdx.x == 0) a.counts[p] = n_list;
}

// The same list for bt_per > kBtRegs: thread t owns blocks [t bt_per,
// (t + 1) bt_per) and reads their ids from the table. Contains barriers:
// every thread must call it (as must every thread call emit_list).
__device__ void emit_list_table(const PairArgs& a, const PairLds& L, int p, int b, int nb,
                                int* wtmp) {
  const int t = threadIdx.x;
  const int bl0 = t * a.bt_per;
  int nz = 0;
  for (int j = 0; j < a.bt_per; ++j) {
    const int lb = bl0 + j;
    if (lb < nb) nz += ((L.bmask[lb >> 1] >> (16 * (lb & 1))) & 0xffffu) != 0u;
  }
  int n_list;
  int pos = wg_exclusive_scan<kPairWaves, false>(nz, wtmp, &n_list);
  int2* ent = a.entries + static_cast<size_t>(p) * a.max_blocks;
  const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
  for (int j = 0; j < a.bt_per; ++j) {
    const int lb = bl0 + j;
    if (lb < nb) {
      const uint32_t m = (L.bmask[lb >> 1] >> (16 * (lb & 1))) & 0xffffu;
      if (m) {
        const int pb = row[lb];
        const bool ok = pb >= 0 && pb < a.num_blocks;
        ent[pos++] = ok ? make_int2(pb, static_cast<int>(m)) : make_int2(0, 0);
      }
    }
  }
  if (t == 0) a.counts[p] = n_list;
}

__device__ void emit_list(const PairArgs& a, const PairLds& L, int p, int b, int nb,
                          const int (&btr)[kBtRegs], int* wtmp) {
  switch (a.bt_per) {
    case 2: emit_list_regs<1>(a, p, L.bmask, btr, wtmp); break;
    case 4: emit_list_regs<2>(a, p, L.bmask, btr, wtmp); break;
    case 8: emit_list_regs<4>(a, p, L.bmask, btr, wtmp); break;
    case 16: emit_list_regs<8>(a, p, L.bmask, btr, wtmp); break;
    default: emit_list_table(a, L, p, b, nb, wtmp);
  }
}

// ---------------------------------------------------------------------------
// The pair kernel: one 256-thread workgroup per pair p = b * Hkv + g.
// ---------------------------------------------------------------------------
// STH: the thought spans are staged in LDS (a template flag, so that the
// span reads stay LDS reads and never wait on outstanding global stores).
// SPEC: the first batch of summary-key rows is loaded before the thought
// range arrives (a template flag, so that kernels without it keep the plain
// load order and registers).
template <typename E, int D, bool SCORE, bool SELECT, bool PLAN, bool STH, bool SPEC>
__global__ void __launch_bounds__(kPairThreads)
pair_kernel(PairArgs a) {
  constexpr int VPL = 16 / E::kBytes;  // elements per 16-byte load
  constexpr int LPT = D / VPL;         // lanes per thought row
  constexpr int TPP = kPairThreads / LPT;
  constexpr int R = kScoreR;           // rows in flight per lane
  constexpr int NSPEC = TPP * R;       // rows of the speculative batch
  extern __shared__ __align__(16) int32_t dyn[];
  __shared__ int wtmp[kPairWaves];
  __shared__ uint32_t hist[kPairThreads];
  __shared__ uint32_t sh[2];

  // grid (Hkv, B): the pair's indices need no division
  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int p = b * a.Hkv + g;
  const PairLds L = pair_lds(dyn, a.max_per_seq, a.k, SELECT, PLAN, STH);

  using St = typename E::storage;
  const int c = t % LPT, r0 = t / LPT;
  const int G = a.G;

  // --- loads that need nothing but the pair index, all issued up front:
  // thought range, sequence length, query rows, block-table row, given sel
  int lo = a.seq_ptr[b], hi = a.seq_ptr[b + 1];
  int T = 0;
  if (PLAN) T = a.seq_lens[b];
  uint4 qv[kMaxGroup];
  if (SCORE) {
    const St* qg = static_cast<const St*>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h)
      if (h < G) qv[h] = *reinterpret_cast<const uint4*>(qg + h * D + c * VPL);
  }
  // Summary-key rows before the thought range arrives (when the launcher
  // enables it): sequences hold about spec_avg thoughts each, so the NSPEC
  // rows from b * spec_avg - spec_margin usually contain [lo, hi); if not,
  // the rows are loaded again once the range is known.
  const St* kb = static_cast<const St*>(a.kbar);
  constexpr bool spec = SCORE && SPEC;
  int g0 = 0;
  uint4 us[R];
  if (spec) {
    g0 = static_cast<int>(static_cast<float>(b) * a.spec_avg) - a.spec_margin;
    g0 = g0 < 0 ? 0 : g0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int j = g0 + r0 + r * TPP;
      j = j < a.n_total ? j : a.n_total - 1;  // a valid row; the result is dropped
      us[r] = *reinterpret_cast<const uint4*>(kb + (static_cast<size_t>(j) * a.Hkv + g) * D +
                                              c * VPL);
    }
  }
  int btr[kBtRegs];
  const bool bt_pref = a.bt_per <= kBtRegs;
  if (PLAN && bt_pref) {
    const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
#pragma unroll
    for (int j = 0; j < kBtRegs; ++j) {
      const int lb = t * a.bt_per + j;
      btr[j] = (j < a.bt_per && lb < a.max_blocks) ? row[lb] : 0;
    }
  }
  int selr[kSelRegs];
  if (PLAN && !SELECT) {
#pragma unroll
    for (int j = 0; j < kSelRegs; ++j) {
      const int i = t + j * kPairThreads;
      selr[j] = i < a.k ? a.sel[static_cast<size_t>(p) * a.k + i] : -1;
    }
  }

  // --- loads that need the thought range: the first thought spans and the
  // first batch of summary-key rows
  lo = lo < 0 ? 0 : (lo > a.n_total ? a.n_total : lo);
  hi = hi < lo ? lo : (hi > a.n_total ? a.n_total : hi);
  const int n = hi - lo < a.max_per_seq ? hi - lo : a.max_per_seq;
  int ths0 = 0, thl0 = 0;
  if (PLAN && STH && t < n) {
    ths0 = a.th_start[lo + t];
    thl0 = a.th_len[lo + t];
  }
  const bool hit = spec && lo >= g0 && lo + n <= g0 + NSPEC;  // uniform (false unless SPEC)
  uint4 u[R];
  auto load_rows = [&](int i0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      int i = i0 + r0 + r * TPP;
      i = i < n ? i : n - 1;  // a valid row; the result is dropped
      u[r] = *reinterpret_cast<const uint4*>(kb + (static_cast<size_t>(lo + i) * a.Hkv + g) * D +
                                             c * VPL);
    }
  };
  if (SCORE && n > 0 && !hit) load_rows(0);

  int tw = 0, nb = 0;
  if (PLAN) {
    const int cap = a.max_blocks * kBlock;
    T = T < 0 ? 0 : (T > cap ? cap : T);
    tw = T - a.window > 0 ? T - a.window : 0;
    nb = (T + kBlock - 1) / kBlock;
    clear_bitmap(L.bmask, a.bt_per, nb);
    if (!SELECT) {
#pragma unroll
      for (int j = 0; j < kSelRegs; ++j) {
        const int i = t + j * kPairThreads;
        if (i < a.k) L.sel_l[i] = selr[j];
      }
    }
    if (STH) {
      if (t < n) {
        L.th_s[t] = ths0;
        L.th_l[t] = thl0;
      }
      for (int i = t + kPairThreads; i < n; i += kPairThreads) {
        L.th_s[i] = a.th_start[lo + i];
        L.th_l[i] = a.th_len[lo + i];
      }
    }
  }

  if (SCORE) {
    // this lane's VPL dimensions of the group's query sum, in float64
    double qs[VPL];
#pragma unroll
    for (int v = 0; v < VPL; ++v) qs[v] = 0.0;
#pragma unroll
    for (int h = 0; h < kMaxGroup; ++h) {
      if (h < G) {
        float x[VPL];
        unpack16<E>(qv[h], x);
#pragma unroll
        for (int v = 0; v < VPL; ++v) qs[v] += static_cast<double>(x[v]);
      }
    }
    // the rows of one batch: lane row r is thought i0 + r0 + r TPP of the
    // sequence (negative or >= n: not the sequence's, dropped)
    auto score_rows = [&](const uint4 (&cur)[R], int i0) {
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float x[VPL];
        unpack16<E>(cur[r], x);
        double acc = 0.0;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc = fma(qs[v], static_cast<double>(x[v]), acc);
        acc = group_sum_f64<LPT>(acc);
        const int i = i0 + r0 + r * TPP;
        if (c == 0 && i >= 0 && i < n) {
          const float f = static_cast<float>(acc);
          a.scores[static_cast<size_t>(lo + i) * a.Hkv + g] = f;
          if (SELECT) L.keys[i] = order_key(f);
        }
      }
    };
    if (hit) {
      score_rows(us, g0 - lo);
    } else {
      for (int i0 = 0; i0 < n; i0 += TPP * R) {
        uint4 cur[R];
#pragma unroll
        for (int r = 0; r < R; ++r) cur[r] = u[r];
        if (i0 + TPP * R < n) load_rows(i0 + TPP * R);  // next batch in flight
        score_rows(cur, i0);
      }
    }
  } else if (SELECT) {
    for (int i = t; i < n; i += kPairThreads)
      L.keys[i] = order_key(a.scores[static_cast<size_t>(lo + i) * a.Hkv + g]);
  }
  if (SELECT)
    for (int i = n + t; i < keys_fill(n); i += kPairThreads) L.keys[i] = 0u;
  __syncthreads();

  if (SELECT && a.k > 0) {
    int32_t* out = a.sel + static_cast<size_t>(p) * a.k;
    if (n <= a.k) {
      for (int j = t; j < a.k; j += kPairThreads) {
        const int v = j < n ? j : -1;
        out[j] = v;
        if (PLAN) L.sel_l[j] = v;
      }
    } else if (n <= kRankMax) {
      select_by_rank<PLAN>(L, n, a.k, out, wtmp);
    } else {
      select_by_radix<PLAN>(L, n, a.k, out, hist, wtmp, sh);
    }
    if (PLAN) __syncthreads();
  }

  if (PLAN) {
    // the selected thoughts' tokens below the window start (the attention
    // kernel adds the window itself) into the slot bitmap: tps threads share
    // one selected thought, each ORing every tps-th block of its span
    int tps = kPairThreads;
    while (tps > 1 && tps * a.k > kPairThreads) tps >>= 1;
    const int lgt = __builtin_ctz(tps);
    for (int i = t >> lgt; i < a.k; i += kPairThreads >> lgt) {
      const int th = L.sel_l[i];
      if (th < 0 || th >= n) continue;
      int ts, tl;
      if (STH) {
        ts = L.th_s[th];
        tl = L.th_l[th];
      } else {
        ts = a.th_start[lo + th];
        tl = a.th_len[lo + th];
      }
      const int s = ts > 0 ? ts : 0;
      int e = tl > 0 ? ts + tl : s;
      e = e < tw ? e : tw;
      if (e > s) or_span(L.bmask, s, e, t & (tps - 1), tps);
    }
    __syncthreads();
    if (t == 0) a.list_tw[p] = tw;
    emit_list(a, L, p, b, nb, btr, wtmp);
  }
}

// ---------------------------------------------------------------------------
// Consensus (ZoomR Sec. 3.3, "Global Aggregation and Consensus"): one
// workgroup per sequence. Votes v_i = the number of (layer, KV head) top-k
// rows holding thought i, a row counting once however often it lists i (v_i
// is a sum of set-membership indicators). One thread per row walks its
// entries: an index above every earlier index of the row is new (rows written
// by the selector ascend, so they never look back); any other index is
// compared with the earlier entries. Votes are LDS atomics. The consensus set
// is the c thoughts with the most votes among those with any, ties to the
// lower index, in ascending index; agreement = votes of the consensus set
// over all votes (ZoomR Sec. 4).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPairThreads)
consensus_kernel(ConsArgs a) {
  extern __shared__ __align__(16) int32_t dyn[];
  __shared__ int wtmp[kPairWaves];
  __shared__ uint32_t hist[kPairThreads];
  __shared__ uint32_t sh[2];
  __shared__ int tot_tmp[kPairWaves];
  const int b = blockIdx.x, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  PairLds L{};
  L.keys = reinterpret_cast<uint32_t*>(dyn);
  L.sel_l = dyn + keys_ints(a.max_per_seq);
  int lo = a.seq_ptr[b], hi = a.seq_ptr[b + 1];
  lo = lo < 0 ? 0 : (lo > a.n_total ? a.n_total : lo);
  hi = hi < lo ? lo : (hi > a.n_total ? a.n_total : hi);
  const int n = hi - lo < a.max_per_seq ? hi - lo : a.max_per_seq;
  for (int i = t; i < keys_fill(n); i += kPairThreads) L.keys[i] = 0u;
  __syncthreads();
  const int rows = a.n_layers * a.Hkv;
  constexpr int kRowBatch = 8;  // row entries loaded at once
  for (int r = t; r < rows; r += kPairThreads) {
    const int l = r / a.Hkv, g = r - l * a.Hkv;
    const int32_t* row = a.sel + ((static_cast<size_t>(l) * a.B + b) * a.Hkv + g) * a.k;
    int top = -1;  // largest valid index met so far in the row
    for (int j0 = 0; j0 < a.k; j0 += kRowBatch) {
      int v[kRowBatch];
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) v[u] = j0 + u < a.k ? row[j0 + u] : -1;
#pragma unroll
      for (int u = 0; u < kRowBatch; ++u) {
        const int i = v[u];
        if (i < 0 || i >= n) continue;
        bool fresh = i > top;
        if (!fresh) {  // not above every earlier index: look for it among them
          fresh = true;
          for (int jj = 0; jj < j0 + u; ++jj)
            if (row[jj] == i) {
              fresh = false;
              break;
            }
        }
        if (fresh) atomicAdd(&L.keys[i], 1u);
        top = i > top ? i : top;
      }
    }
  }
  __syncthreads();
  int mine = 0;
  for (int i = t; i < n; i += kPairThreads) {
    a.votes[lo + i] = static_cast<int32_t>(L.keys[i]);
    mine += static_cast<int>(L.keys[i]);
  }
  const int wsum = wave_sum(mine);
  if (lane == 0) tot_tmp[wave] = wsum;
  int nsel = 0;
  if (a.c > 0) {
    if (n <= a.c) {
      for (int j = t; j < n; j += kPairThreads) L.sel_l[j] = j;
      nsel = n;
    } else if (n <= kRankMax) {
      select_by_rank<false>(L, n, a.c, L.sel_l, wtmp);
      nsel = a.c;
    } else {
      select_by_radix<false>(L, n, a.c, L.sel_l, hist, wtmp, sh);
      nsel = a.c;
    }
  }
  __syncthreads();
  int total = 0;
#pragma unroll
  for (int v = 0; v < kPairWaves; ++v) total += tot_tmp[v];
  // keep the chosen thoughts that have votes (thread t owns a contiguous run)
  const int per = (nsel + kPairThreads - 1) / kPairThreads;
  const int j0 = t * per, j1 = j0 + per < nsel ? j0 + per : nsel;
  int keep = 0, kvotes = 0;
  for (int j = j0; j < j1; ++j) {
    const uint32_t v = L.keys[L.sel_l[j]];
    keep += v > 0u;
    kvotes += static_cast<int>(v);
  }
  int n_keep;
  int pos = wg_exclusive_scan<kPairWaves>(keep, wtmp, &n_keep);
  int32_t* out = a.cons + static_cast<size_t>(b) * a.c;
  for (int j = j0; j < j1; ++j) {
    const int i = L.sel_l[j];
    if (L.keys[i] > 0u) out[pos++] = i;
  }
  for (int j = n_keep + t; j < a.c; j += kPairThreads) out[j] = -1;
  int kv_all;
  wg_exclusive_scan<kPairWaves>(kvotes, wtmp, &kv_all);
  if (t == 0) a.agree[b] = total > 0 ? static_cast<float>(kv_all) / static_cast<float>(total) : 0.f;
}

// ---------------------------------------------------------------------------
// Block lists of the multi-granularity set (ZoomR Sec. 3.3, "Constructing the
// Final Multi-Granularity Context"): the prompt [0, N_p), the regular segment
// R_i of every consensus thought and the summary segment S_i of every other
// thought with a vote, clipped below the window start (the attention kernel
// adds the window). One workgroup per (sequence, KV head); the list is the
// same for every head of a sequence.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kPairThreads)
zoom_plan_kernel(PairArgs a) {
  extern __shared__ __align__(16) int32_t dyn[];
  __shared__ int wtmp[kPairWaves];
  const int b = blockIdx.y, t = threadIdx.x;  // grid (Hkv, B)
  const int p = b * a.Hkv + blockIdx.x;
  int* flag = dyn;  // [up4(max_per_seq)]: 1 = consensus thought
  PairLds L{};
  L.bmask = reinterpret_cast<uint32_t*>(dyn + up4(a.max_per_seq));
  int lo = a.seq_ptr[b], hi = a.seq_ptr[b + 1];
  int T = a.seq_lens[b];
  int btr[kBtRegs];
  const bool bt_pref = a.bt_per <= kBtRegs;
  if (bt_pref) {
    const int32_t* row = a.block_table + static_cast<size_t>(b) * a.max_blocks;
#pragma unroll
    for (int j = 0; j < kBtRegs; ++j) {
      const int lb = t * a.bt_per + j;
      btr[j] = (j < a.bt_per && lb < a.max_blocks) ? row[lb] : 0;
    }
  }
  lo = lo < 0 ? 0 : (lo > a.n_total ? a.n_total : lo);
  hi = hi < lo ? lo : (hi > a.n_total ? a.n_total : hi);
  const int n = hi - lo < a.max_per_seq ? hi - lo : a.max_per_seq;
  const int cap = a.max_blocks * kBlock;
  T = T < 0 ? 0 : (T > cap ? cap : T);
  const int tw = T - a.window > 0 ? T - a.window : 0;
  const int nb = (T + kBlock - 1) / kBlock;
  clear_bitmap(L.bmask, a.bt_per, nb);
  for (int i = t; i < n; i += kPairThreads) flag[i] = 0;
  __syncthreads();
  for (int j = t; j < a.c; j += kPairThreads) {
    const int i = a.cons[static_cast<size_t>(b) * a.c + j];
    if (i >= 0 && i < n) flag[i] = 1;
  }
  __syncthreads();
  // prompt: its blocks shared by the whole workgroup
  const int pe = a.n_prompt < tw ? a.n_prompt : tw;
  if (pe > 0) or_span(L.bmask, 0, pe, t, kPairThreads);
  // thoughts with votes: one thread per thought walks its segment's blocks
  for (int i = t; i < n; i += kPairThreads) {
    if (a.votes[lo + i] <= 0) continue;
    int s, ln;
    if (flag[i]) {
      s = a.th_start[lo + i];
      ln = a.th_len[lo + i];
    } else {
      s = a.sum_start[lo + i];
      ln = a.sum_len[lo + i];
    }
    s = s > 0 ? s : 0;
    int e = ln > 0 ? s + ln : s;
    e = e < tw ? e : tw;
    if (e > s) or_span(L.bmask, s, e, 0, 1);
  }
  __syncthreads();
  if (t == 0) a.list_tw[p] = tw;
  emit_list(a, L, p, b, nb, btr, wtmp);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr size_t kPairLdsLimit = 64 * 1024;
constexpr size_t kPairStaticLds = (kPairWaves + kPairThreads + 2) * sizeof(int32_t);

static size_t pair_dyn_lds(const PairArgs& a, bool select, bool plan) {
  return pair_lds_ints(a.max_per_seq, a.k, a.max_blocks, select, plan, a.stage_th != 0) *
         sizeof(int32_t);
}

bool pair_lds_ok(const zr_geom& gm, int max_per_seq, int k, bool select, bool plan) {
  return kPairStaticLds + pair_lds_ints(max_per_seq, k, gm.max_blocks_per_seq, select, plan,
                                        false) * sizeof(int32_t) <=
         kPairLdsLimit;
}

// Whether the scorer loads its first batch of summary-key rows before the
// thought range arrives, and where: only for even batches (the caller's bound
// on thoughts per sequence within 1.25x of the mean), where the guess lands,
// and when one batch of rows holds a whole sequence; elsewhere the extra rows
// would only delay the loads that follow them. Sequence b's guess starts at
// max(0, (int)(b * per_seq) - margin), float32 product, and covers `rows`
// rows. per_seq = 0 (and rows = margin = 0) when the rule is off.
void summary_prefetch_rule(const zr_geom& gm, int n_total, int max_per_seq, int* rows,
                           float* per_seq, int* margin) {
  *rows = 0;
  *per_seq = 0.f;
  *margin = 0;
  if (n_total <= 0 || gm.batch <= 0) return;
  int r;
  if (gm.dtype == ZR_BF16)
    r = gm.head_dim == 128 ? score_batch_rows<BF16, 128>() : score_batch_rows<BF16, 64>();
  else
    r = gm.head_dim == 128 ? score_batch_rows<F32, 128>() : score_batch_rows<F32, 64>();
  const float avg = static_cast<float>(n_total) / static_cast<float>(gm.batch);
  if (max_per_seq <= r && static_cast<float>(max_per_seq) <= 1.25f * avg) {
    *rows = r;
    *per_seq = avg;
    *margin = static_cast<int>((static_cast<float>(r) - avg) * 0.5f);
  }
}

template <typename E, int D, bool SCORE, bool SELECT, bool PLAN>
static hipError_t launch_pair_t(const zr_geom& gm, PairArgs a, hipStream_t s) {
  a.bt_per = pair_bt_per(gm.max_blocks_per_seq);
  a.stage_th = 0;
  if (PLAN) {
    PairArgs b2 = a;
    b2.stage_th = 1;
    if (kPairStaticLds + pair_dyn_lds(b2, SELECT, PLAN) <= kPairLdsLimit) a.stage_th = 1;
  }
  const size_t lds = pair_dyn_lds(a, SELECT, PLAN);
  if (kPairStaticLds + lds > kPairLdsLimit) return hipErrorInvalidValue;
  a.G = gm.n_q_heads / gm.n_kv_heads;
  a.spec_avg = 0.f;
  a.spec_margin = 0;
  if (SCORE) {
    int rows = 0;
    summary_prefetch_rule(gm, a.n_total, a.max_per_seq, &rows, &a.spec_avg, &a.spec_margin);
  }
  const dim3 grid(gm.n_kv_heads, gm.batch);
  const dim3 block(kPairThreads);
  const bool spec = SCORE && a.spec_avg > 0.f;
  if (a.stage_th && spec)
    hipLaunchKernelGGL((pair_kernel<E, D, SCORE, SELECT, PLAN, true, SCORE>), grid, block, lds, s,
                       a);
  else if (a.stage_th)
    hipLaunchKernelGGL((pair_kernel<E, D, SCORE, SELECT, PLAN, true, false>), grid, block, lds, s,
                       a);
  else if (spec)
    hipLaunchKernelGGL((pair_kernel<E, D, SCORE, SELECT, PLAN, false, SCORE>), grid, block, lds,
                       s, a);
  else
    hipLaunchKernelGGL((pair_kernel<E, D, SCORE, SELECT, PLAN, false, false>), grid, block, lds,
                       s, a);
  return hipGetLastError();
}

template <bool SCORE, bool SELECT, bool PLAN>
static hipError_t launch_pair_mode(const zr_geom& gm, const PairArgs& a, hipStream_t s) {
  if constexpr (!SCORE) {
    return launch_pair_t<BF16, 128, SCORE, SELECT, PLAN>(gm, a, s);
  } else {
    if (gm.dtype == ZR_BF16)
      return gm.head_dim == 128 ? launch_pair_t<BF16, 128, SCORE, SELECT, PLAN>(gm, a, s)
                                : launch_pair_t<BF16, 64, SCORE, SELECT, PLAN>(gm, a, s);
    return gm.head_dim == 128 ? launch_pair_t<F32, 128, SCORE, SELECT, PLAN>(gm, a, s)
                              : launch_pair_t<F32, 64, SCORE, SELECT, PLAN>(gm, a, s);
  }
}

hipError_t launch_pair(const zr_geom& gm, const PairArgs& a, int mode, hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  switch (mode) {
    case kModeScore: return launch_pair_mode<true, false, false>(gm, a, s);
    case kModeSelect: return launch_pair_mode<false, true, false>(gm, a, s);
    case kModePlan: return launch_pair_mode<false, false, true>(gm, a, s);
    case kModeStep: return launch_pair_mode<true, true, true>(gm, a, s);
    case kModeScoreSelect: return launch_pair_mode<true, true, false>(gm, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace zr

namespace zr {

static size_t consensus_lds(int max_per_seq, int c) {
  return (static_cast<size_t>(keys_ints(max_per_seq)) + up4(c)) * sizeof(int32_t);
}

bool consensus_lds_ok(int max_per_seq, int c) {
  return kPairStaticLds + consensus_lds(max_per_seq, c) + 64 <= kPairLdsLimit;
}

hipError_t launch_consensus(const ConsArgs& a, hipStream_t s) {
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(consensus_kernel, dim3(a.B), dim3(kPairThreads),
                     consensus_lds(a.max_per_seq, a.c), s, a);
  return hipGetLastError();
}

static size_t zoom_lds(const zr_geom& gm, int max_per_seq) {
  return (static_cast<size_t>(up4(max_per_seq)) + bmask_ints(gm.max_blocks_per_seq)) *
         sizeof(int32_t);
}

bool zoom_lds_ok(const zr_geom& gm, int max_per_seq) {
  return zoom_lds(gm, max_per_seq) + 1024 <= kPairLdsLimit;
}

hipError_t launch_zoom_plan(const zr_geom& gm, const PairArgs& a0, hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  PairArgs a = a0;
  a.bt_per = pair_bt_per(gm.max_blocks_per_seq);
  hipLaunchKernelGGL(zoom_plan_kernel, dim3(gm.n_kv_heads, gm.batch), dim3(kPairThreads),
                     zoom_lds(gm, a.max_per_seq), s, a);
  return hipGetLastError();
}

}  // namespace zr

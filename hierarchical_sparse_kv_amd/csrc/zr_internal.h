// Internal declarations shared by the libzr translation units (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "zr.h"

namespace zr {

constexpr int kBlock = ZR_BLOCK_SIZE;

// Element types of q, the pools and the summary keys.
struct F32 {
  using storage = float;
  static constexpr int kBytes = 4;
};
struct BF16 {
  using storage = uint16_t;
  static constexpr int kBytes = 2;
};

// Expand one 16-byte chunk into floats (4 for F32, 8 for BF16; bf16 -> f32
// is exact: the bf16 bits are the high half of the f32 bits).
template <typename E>
__device__ __forceinline__ void unpack16(const uint4& u, float* out);

template <>
__device__ __forceinline__ void unpack16<F32>(const uint4& u, float* out) {
  out[0] = __uint_as_float(u.x);
  out[1] = __uint_as_float(u.y);
  out[2] = __uint_as_float(u.z);
  out[3] = __uint_as_float(u.w);
}

template <>
__device__ __forceinline__ void unpack16<BF16>(const uint4& u, float* out) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// ---------------------------------------------------------------------------
// n / d for 0 <= n < 2^16, d >= 1, in a few instructions (the general 32-bit
// integer division is about 30). The float32 estimate n * rcp(d) is within 1
// of n / d whenever rcp(d) is accurate to 2^-16 relative (the hardware
// reciprocal is accurate to about 1 ulp), and one correction step each way
// makes it exact.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int div_small(int n, int d) {
  int q = static_cast<int>(static_cast<float>(n) * __builtin_amdgcn_rcpf(static_cast<float>(d)));
  q += (q + 1) * d <= n ? 1 : 0;
  q -= q * d > n ? 1 : 0;
  return q;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers built on DPP (data-parallel primitives inside the VALU,
// no LDS round trip). DPP controls: quad_perm 0x00-0xff, row_shr:n 0x110+n,
// row_mirror 0x140, row_half_mirror 0x141, row_bcast:15 0x142,
// row_bcast:31 0x143 (a row is 16 lanes).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ int dpp_move(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}

// Inclusive prefix sum of v over the 64 lanes of the wave. Every lane must
// be active.
__device__ __forceinline__ int wave_incl_sum(int v) {
  const int lane = threadIdx.x & 63, r = lane & 15;
  int t;
  t = dpp_move<0x111>(v);
  v += r >= 1 ? t : 0;
  t = dpp_move<0x112>(v);
  v += r >= 2 ? t : 0;
  t = dpp_move<0x114>(v);
  v += r >= 4 ? t : 0;
  t = dpp_move<0x118>(v);
  v += r >= 8 ? t : 0;
  t = dpp_move<0x142>(v);  // lane 15 of the previous row into rows 1 and 3
  v += (lane & 16) ? t : 0;
  t = dpp_move<0x143>(v);  // lane 31 into rows 2 and 3
  v += (lane & 32) ? t : 0;
  return v;
}

// Index of the calling wave in its workgroup, as a wave-uniform (scalar)
// value, so that what is derived from it stays scalar.
__device__ __forceinline__ int wave_id() {
  return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
}

// Sum of v over the wave, in every lane.
__device__ __forceinline__ int wave_sum(int v) {
  return __builtin_amdgcn_readlane(wave_incl_sum(v), 63);
}

// Exclusive prefix sum of one value per thread across a workgroup of NW
// waves; *total gets the sum. `tmp` holds NW ints. Contains barriers: every
// thread must call it. REUSE = false drops the closing barrier that lets
// `tmp` be written again (for a workgroup's last scan).
template <int NW, bool REUSE = true>
__device__ __forceinline__ int wg_exclusive_scan(int v, int* tmp, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = tmp[w];
    before += w < wave ? x : 0;
    all += x;
  }
  if (REUSE) __syncthreads();
  *total = all;
  return before + incl - v;
}

template <int CTRL>
__device__ __forceinline__ double dpp_move_f64(double x) {
  const int2 w = __builtin_bit_cast(int2, x);
  int2 r;
  r.x = __builtin_amdgcn_update_dpp(0, w.x, CTRL, 0xf, 0xf, false);
  r.y = __builtin_amdgcn_update_dpp(0, w.y, CTRL, 0xf, 0xf, false);
  return __builtin_bit_cast(double, r);
}

// Sum of x over aligned groups of N lanes (N = 4, 8, 16 or 32), in every lane
// of the group: pairs in a quad, then quads mirrored inside a half row, then
// half rows mirrored inside a row, then rows 16 apart.
template <int N>
__device__ __forceinline__ double group_sum_f64(double x) {
  x += dpp_move_f64<0xb1>(x);  // quad_perm [1,0,3,2]
  x += dpp_move_f64<0x4e>(x);  // quad_perm [2,3,0,1]
  if (N >= 8) x += dpp_move_f64<0x141>(x);
  if (N >= 16) x += dpp_move_f64<0x140>(x);
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

template <typename E>
__device__ __forceinline__ float load_elem(const typename E::storage* p, size_t i);

template <>
__device__ __forceinline__ float load_elem<F32>(const float* p, size_t i) {
  return p[i];
}

template <>
__device__ __forceinline__ float load_elem<BF16>(const uint16_t* p, size_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}

// Pre-attention work of one (sequence, KV head) pair (zr_pair.hip): scores,
// top-k and the attended-block list, by mode.
enum PairMode { kModeScore = 0, kModeSelect = 1, kModePlan = 2, kModeStep = 3,
                kModeScoreSelect = 4 };

struct PairArgs {
  const void* q;              // [B][Hq][D]                      (score)
  const void* kbar;           // [n_total][Hkv][D]               (score)
  const int32_t* seq_ptr;     // [B + 1] thoughts CSR
  const int32_t* th_start;    // [n_total]                       (plan)
  const int32_t* th_len;      // [n_total]                       (plan)
  float* scores;              // [n_total][Hkv] written (score) or read (select)
  int32_t* sel;               // [B][Hkv][k] written (select) or read (plan)
  const int32_t* seq_lens;    // [B]                             (plan)
  const int32_t* block_table; // [B][max_blocks]                 (plan)
  int32_t* counts;            // [B * Hkv] list length per pair  (plan)
  int2* entries;              // [B * Hkv][max_blocks] (physical block, slot mask) (plan)
  int32_t* list_tw;           // [B * Hkv] window start the spans are clipped at (plan)
  int32_t n_total, max_per_seq, Hq, Hkv, k, window, max_blocks, num_blocks;
  int32_t bt_per;             // block-table entries per thread (set by the launcher)
  int32_t G;                  // query heads per KV head (set by the launcher)
  float spec_avg;             // > 0: summary-key rows loaded ahead of the thought range,
  int32_t spec_margin;        //   from b * spec_avg - spec_margin (set by the launcher)
  int32_t stage_th;           // 1: thought spans staged in LDS
  // multi-granularity plan (zoom): votes, consensus set, summary spans, prompt
  const int32_t* votes;       // [n_total]
  const int32_t* cons;        // [B][c]
  const int32_t* sum_start;   // [n_total]
  const int32_t* sum_len;     // [n_total]
  int32_t c, n_prompt;
};

// Votes, consensus set and agreement of every sequence (zr_pair.hip).
struct ConsArgs {
  const int32_t* seq_ptr;
  const int32_t* sel;         // [n_layers][B][Hkv][k]
  int32_t* votes;             // [n_total]
  int32_t* cons;              // [B][c]
  float* agree;               // [B]
  int32_t B, Hkv, k, n_layers, c, n_total, max_per_seq;
};

// A workgroup's share of the attention between semantic boundaries, taken
// once per boundary (zr_reuse_plan): its one or two segments and their list
// entries. A cached entry is (physical block, slot mask); a window entry is
// (physical block, or -1 for a block not yet cached at the boundary;
// logical block | kWindowEntry), its slots taken from the current length.
constexpr int kRecEntries = 192;
constexpr uint32_t kWindowEntry = 0x80000000u;
struct ReuseRecord {
  int32_t nseg;       // 0: no work; 1 or 2: the segments below; -1: plan in the kernel
  int32_t pad[3];
  int4 seg[2][2];     // {p, tw, ncache, slot}, {lo, hi, first record entry, planned end T0 + horizon}
  int2 ent[kRecEntries];
};

// Attention launch parameters (device pointers + sizes), passed by value.
// Pair p = b * Hkv + g attends its counts[p] list entries entries[p][0..)
// (sparse only) and then the blocks of its window [T - window, T) (dense:
// [0, T)), read from the block table; a sparse window starts no earlier than
// list_tw[p], where the lists' spans were clipped. Partial results are indexed by slot;
// slots [ws_pref[p], ws_pref[p + 1]) hold pair p's.
struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* plan_lens;  // [B] lengths the split is planned on (= seq_lens, or the boundary's)
  int32_t horizon;           // window tokens planned past plan_lens (0 = none)
  ReuseRecord* records;      // [nwg] (reuse calls)
  int32_t* reuse_lens;       // [B] the boundary's lengths, kept by zr_reuse_plan
  int32_t* reuse_pref;       // [P + 1] the slot bases of that split, kept by zr_reuse_plan
  int32_t* reuse_meta;       // {window, horizon, -, -} kept by zr_reuse_plan
  const int32_t* counts;     // [P] (sparse)
  const int2* entries;       // [P][max_blocks] (sparse)
  const int32_t* list_tw;    // [P] window start of the call that wrote the lists (sparse)
  int32_t* ws_pref;          // [P + 1]: first partial slot of each pair
  float* ws_m;               // [nwg + P][G]
  float* ws_l;               // [nwg + P][G]
  float* ws_acc;             // [nwg + P][G][D]
  float* out;                // [B][Hq][D]
  int32_t B, Hq, Hkv;
  int32_t nwg;               // workgroups of the grid (at most nwg + P partial slots)
  int32_t max_blocks, num_blocks;
  int32_t window;            // sparse: window tokens appended after the cached entries
  float scale_log2;          // scale * log2(e)
};

// Append path (zr_append.hip).
struct AppendArgs {
  void* k_pool;
  void* v_pool;
  int32_t* block_table;       // [B][max_blocks]: a popped block is written here
  int32_t* seq_lens;          // [B]: grows by one per appended token
  const void* k_new;          // [B][Hkv][D]
  const void* v_new;          // [B][Hkv][D]
  const int32_t* free_blocks; // free stack; entries [0, *free_count) are free, top last
  int32_t* free_count;        // [1]
  int32_t* status;            // [B] ZR_APPEND_*
  int32_t Hkv, D, max_blocks, num_blocks;
};

struct SummaryArgs {
  const void* k_pool;
  const int32_t* block_table;
  const int32_t* seq_ptr;
  const int32_t* th_start;
  const int32_t* th_len;
  const int32_t* which;       // [n_which] global thought indices
  void* out;                  // summary keys [n_total][Hkv][D]: rows `which` written
  int32_t B, Hkv, max_blocks, num_blocks, n_total;
};

// Staging of a step's attended tiles into device memory (zr_stage.hip).
struct StageArgs {
  const void* k_pool;         // source pools (device memory or device-mapped host memory)
  const void* v_pool;
  const int32_t* block_table; // [B][max_blocks]
  const int32_t* seq_lens;    // [B]
  const int32_t* counts;      // [P] cached list lengths (pair kernel)
  const int2* entries;        // [P][max_blocks] cached lists (pair kernel)
  void* k_stage;              // [B * stage_blocks][Hkv][16][D]
  void* v_stage;              // [B * stage_blocks][Hkv][D][16]
  int32_t* s_counts;          // [P] staged list lengths
  int32_t* s_list_tw;         // [P] their window start (the current length: window included)
  int2* s_entries;            // [P][s_stride] staged lists
  int32_t* dropped;           // [P] entries that did not fit
  int32_t B, Hkv, max_blocks, num_blocks, window, stage_blocks;
  int32_t lg_pieces;          // log2(16-byte pieces per tile): tile = 16 * D * element bytes
  int32_t item_chunks;        // work items per pair (set by the launcher)
  int32_t s_stride;           // staged list row length: max_blocks + 1
};

// Host-side launchers (defined next to their kernels).
hipError_t launch_stage(const zr_geom& g, const StageArgs& a, hipStream_t s);
hipError_t launch_append(const zr_geom& g, const AppendArgs& a, hipStream_t s);
hipError_t launch_summary_keys(const zr_geom& g, const SummaryArgs& a, int n_which,
                               hipStream_t s);
hipError_t launch_pair(const zr_geom& g, const PairArgs& a, int mode, hipStream_t s);
// The scorer's rule for loading summary-key rows ahead of the thought range
// (rows = 0 when off); the launcher and zr_summary_prefetch_rule share it.
void summary_prefetch_rule(const zr_geom& g, int n_total, int max_per_seq, int* rows,
                           float* per_seq, int* margin);
// Whether the pair kernel's LDS fits (with nothing optional staged).
bool pair_lds_ok(const zr_geom& g, int max_per_seq, int k, bool select, bool plan);
hipError_t launch_consensus(const ConsArgs& a, hipStream_t s);
bool consensus_lds_ok(int max_per_seq, int c);
// Block lists of the multi-granularity set (same list for every KV head).
hipError_t launch_zoom_plan(const zr_geom& g, const PairArgs& a, hipStream_t s);
bool zoom_lds_ok(const zr_geom& g, int max_per_seq);
// Workgroups of the attention kernel for a bound of `max_attended` tokens per
// (sequence, KV head); the workspace layout depends on it.
int attn_workgroups(const zr_geom& g, int32_t max_attended);
// Bytes of workspace for `nwg` workgroups; fills the AttnArgs pointers when
// `ws` is not null. Layout (each region 16-byte aligned): ws_pref [P + 1],
// counts [P], entries [P][max_blocks] (int2), m and l [nwg + P][G],
// acc [nwg + P][G][D], records [nwg], reuse_lens [B], reuse_pref [P + 1],
// reuse_meta [4].
size_t attn_workspace(const zr_geom& g, int nwg, void* ws, AttnArgs* a);
hipError_t launch_attention(const zr_geom& g, const AttnArgs& a, bool dense, hipStream_t s);
// The sparse attention kernel alone (partials stay in the workspace), and the
// combine kernel alone (the workspace's partials -> a.out).
hipError_t launch_attention_partials(const zr_geom& g, const AttnArgs& a, hipStream_t s);
hipError_t launch_combine(const zr_geom& g, const AttnArgs& a, hipStream_t s);
// Segment records for the calls between semantic boundaries, and the
// attention (+ combine when a.out is set) that reads them.
hipError_t launch_reuse_plan(const zr_geom& g, const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_reuse(const zr_geom& g, const AttnArgs& a, hipStream_t s);

}  // namespace zr

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

// Attention launch parameters (device pointers + sizes), passed by value.
// Partial results are indexed by workgroup; workgroups [ws_pref[p],
// ws_pref[p + 1]) hold the partials of pair p = b * Hkv + g (see zr_attn.hip).
struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* seq_ptr;    // thoughts CSR (sparse only)
  const int32_t* th_start;
  const int32_t* th_len;
  const int32_t* sel;        // [B][Hkv][k] (sparse only, may be null when k == 0)
  int32_t* ws_pref;          // [P + 1]: first workgroup of each pair
  float* ws_m;               // [nwg + P][G]
  float* ws_l;               // [nwg + P][G]
  float* ws_acc;             // [nwg + P][G][D]
  float* out;                // [B][Hq][D]
  int32_t B, Hq, Hkv, max_blocks, num_blocks, n_total;
  int32_t k, window;
  int32_t nwg;               // target workgroups; the grid has nwg + P
  int32_t stage_sel;         // 1: stage sel in LDS (else read it from global memory)
  int32_t stage_th;          // 1: stage the thought spans in LDS
  int32_t row_lds;           // 1: copy the workgroup's block-table row to LDS
  float scale_log2;          // scale * log2(e)
};

// Host-side launchers (defined next to their kernels).
hipError_t launch_coarse_score(const zr_geom& g, const void* q, const zr_thoughts& th,
                               float* scores, hipStream_t s);
hipError_t launch_select_topk(const zr_geom& g, const zr_thoughts& th, const float* scores,
                              int k, int32_t* sel, hipStream_t s);
// Workgroups of the attention kernel for a bound of `max_attended` tokens per
// (sequence, KV head); the workspace layout depends on it.
int attn_workgroups(const zr_geom& g, int32_t max_attended);
// Bytes of workspace for `nwg` workgroups; fills the AttnArgs pointers when
// `ws` is not null.
size_t attn_workspace(const zr_geom& g, int nwg, void* ws, AttnArgs* a);
// Whether the attention kernel's LDS fits for this shape (with nothing staged).
bool attn_lds_ok(const zr_geom& g, int k, bool dense);
hipError_t launch_attention(const zr_geom& g, const AttnArgs& a, bool dense, hipStream_t s);

}  // namespace zr

// The append path of a decode step: the new token's key and value go into
// the paged cache, and the mean summary key of a thought is computed once
// the thought is complete (ZoomR Algorithm 1: append k_t, v_t, then the mean
// summary key of a completed segment, before the scores).
//
// Append (KV-cache management page, "Paged KV cache (PagedAttention)"): a
// sequence's next token goes to slot T % 16 of logical block T / 16; when
// T % 16 == 0 the last block is full (or there is none) and a physical block
// is taken from the caller's free stack first (allocation on demand, one new
// block only when the last one fills). One workgroup per sequence; the pop
// is one device-scope atomic on the stack's counter, so concurrent
// sequences take distinct blocks.
//
// Summary keys (ZoomR Sec. 3.3, eq. for the mean summary key, over the
// thought's own cached keys): one workgroup per (thought, KV head); 16
// lanes per key row, float64 sums (exact for bf16 keys of ordinary range,
// so the order of the sum does not matter), one rounding to float32 and,
// for bf16 caches, one to bf16 (nearest even).
#include "zr_internal.h"

namespace zr {

constexpr int kAppendThreads = 256;

template <typename E>
__global__ void __launch_bounds__(kAppendThreads)
append_kernel(AppendArgs a) {
  using St = typename E::storage;
  const int b = blockIdx.x, t = threadIdx.x;
  __shared__ int sh_blk, sh_T, sh_status;
  if (t == 0) {
    const int T = a.seq_lens[b];
    const int col = T >> 4;
    int status = ZR_APPEND_OK, blk = -1;
    if (T < 0 || col >= a.max_blocks) {
      status = ZR_APPEND_TABLE_FULL;
    } else if ((T & (kBlock - 1)) == 0) {
      const int old = atomicSub(a.free_count, 1);
      if (old <= 0) {
        atomicAdd(a.free_count, 1);
        status = ZR_APPEND_NO_FREE_BLOCK;
      } else {
        blk = a.free_blocks[old - 1];
        if (blk < 0 || blk >= a.num_blocks) status = ZR_APPEND_BAD_BLOCK;
        else a.block_table[static_cast<size_t>(b) * a.max_blocks + col] = blk;
      }
    } else {
      blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + col];
      if (blk < 0 || blk >= a.num_blocks) status = ZR_APPEND_BAD_BLOCK;
    }
    sh_blk = blk;
    sh_T = T;
    sh_status = status;
  }
  __syncthreads();
  const int status = sh_status;
  if (status == ZR_APPEND_OK) {
    const int blk = sh_blk, slot = sh_T & (kBlock - 1);
    const int n = a.Hkv * a.D;
    const St* kn = static_cast<const St*>(a.k_new) + static_cast<size_t>(b) * n;
    const St* vn = static_cast<const St*>(a.v_new) + static_cast<size_t>(b) * n;
    St* kp = static_cast<St*>(a.k_pool);
    St* vp = static_cast<St*>(a.v_pool);
    for (int i = t; i < n; i += kAppendThreads) {
      const int g = i / a.D, e = i - g * a.D;
      const size_t tile = static_cast<size_t>(blk) * a.Hkv + g;
      kp[(tile * kBlock + slot) * a.D + e] = kn[i];          // key row of the slot
      vp[(tile * a.D + e) * kBlock + slot] = vn[i];          // value, dimension-major
    }
  }
  if (t == 0) {
    if (status == ZR_APPEND_OK) a.seq_lens[b] = sh_T + 1;
    a.status[b] = status;
  }
}

constexpr int kSumThreads = 256;

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

template <typename E, int D>
__global__ void __launch_bounds__(kSumThreads)
summary_keys_kernel(SummaryArgs a) {
  using St = typename E::storage;
  constexpr int VPL = 16 / E::kBytes;  // elements per 16-byte load
  constexpr int LPR = D / VPL;         // lanes per key row
  constexpr int RPP = kSumThreads / LPR;  // rows per pass
  __shared__ double part[RPP][D];
  __shared__ int sh_b;
  const int w = blockIdx.x, g = blockIdx.y, t = threadIdx.x;
  const int i = a.which[w];
  if (t == 0) sh_b = -1;
  __syncthreads();
  // sequence of thought i: the b with seq_ptr[b] <= i < seq_ptr[b + 1]
  for (int bb = t; bb < a.B; bb += kSumThreads)
    if (a.seq_ptr[bb] <= i && i < a.seq_ptr[bb + 1]) sh_b = bb;
  __syncthreads();
  const int b = sh_b;
  const bool ok = b >= 0 && i >= 0 && i < a.n_total;
  int s = 0, n = 0;
  if (ok) {
    s = a.th_start[i];
    n = a.th_len[i];
    const int cap = a.max_blocks * kBlock;
    s = s < 0 ? 0 : (s > cap ? cap : s);
    n = n < 0 ? 0 : (s + n > cap ? cap - s : n);
  }
  const int c = t % LPR, r0 = t / LPR;
  double acc[VPL];
#pragma unroll
  for (int v = 0; v < VPL; ++v) acc[v] = 0.0;
  const St* kp = static_cast<const St*>(a.k_pool);
  const int32_t* row = a.block_table + static_cast<size_t>(b < 0 ? 0 : b) * a.max_blocks;
  // U rows per lane in flight: their block ids, then their key chunks, then
  // the sums in row order (rows past the thought re-read its last row and
  // are dropped; rows in out-of-range blocks are skipped)
  constexpr int U = 8;
  for (int j0 = r0; j0 < n; j0 += RPP * U) {
    int blk[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RPP;
      blk[u] = row[(s + (j < n ? j : n - 1)) >> 4];
    }
    uint4 raw[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RPP;
      const int tok = s + (j < n ? j : n - 1);
      const int bk = blk[u] >= 0 && blk[u] < a.num_blocks ? blk[u] : 0;
      const size_t tile = static_cast<size_t>(bk) * a.Hkv + g;
      raw[u] = *reinterpret_cast<const uint4*>(kp + (tile * kBlock + (tok & 15)) * D + c * VPL);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * RPP;
      if (j < n && blk[u] >= 0 && blk[u] < a.num_blocks) {
        float x[VPL];
        unpack16<E>(raw[u], x);
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[v] += static_cast<double>(x[v]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VPL; ++v) part[r0][c * VPL + v] = acc[v];
  __syncthreads();
  if (!ok) return;
  St* out = static_cast<St*>(a.out) + (static_cast<size_t>(i) * a.Hkv + g) * D;
  for (int e = t; e < D; e += kSumThreads) {
    double sum = 0.0;
#pragma unroll
    for (int r = 0; r < RPP; ++r) sum += part[r][e];
    const float m = n > 0 ? static_cast<float>(sum / n) : 0.f;
    if constexpr (E::kBytes == 2) out[e] = f32_to_bf16_rne(m);
    else out[e] = m;
  }
}

hipError_t launch_append(const zr_geom& gm, const AppendArgs& a, hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  if (gm.dtype == ZR_BF16)
    hipLaunchKernelGGL(append_kernel<BF16>, dim3(gm.batch), dim3(kAppendThreads), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<F32>, dim3(gm.batch), dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_summary_keys(const zr_geom& gm, const SummaryArgs& a, int n_which,
                               hipStream_t s) {
  if (n_which == 0 || gm.batch == 0) return hipSuccess;
  const dim3 grid(n_which, gm.n_kv_heads);
  if (gm.dtype == ZR_BF16) {
    if (gm.head_dim == 128)
      hipLaunchKernelGGL((summary_keys_kernel<BF16, 128>), grid, dim3(kSumThreads), 0, s, a);
    else
      hipLaunchKernelGGL((summary_keys_kernel<BF16, 64>), grid, dim3(kSumThreads), 0, s, a);
  } else {
    if (gm.head_dim == 128)
      hipLaunchKernelGGL((summary_keys_kernel<F32, 128>), grid, dim3(kSumThreads), 0, s, a);
    else
      hipLaunchKernelGGL((summary_keys_kernel<F32, 64>), grid, dim3(kSumThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace zr

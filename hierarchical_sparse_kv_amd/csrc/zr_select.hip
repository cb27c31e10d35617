// Coarse scorer and per-(sequence, KV head) top-k selector.
//
// Scoring follows ZoomR Sec. 3.3 (eq. alpha): the inner product of the decode
// query with each thought's mean summary key. With grouped-query attention
// one score is kept per KV head: the query heads of the group are summed
// first (their sum dotted with the key equals the sum of the per-head
// scores). Products and sums run in float64 so the float32 result does not
// depend on summation order for bf16 inputs (every product and partial sum
// is exact there); the float32 scores are what the selector compares.
//
// Selection follows ZoomR Sec. 3.3 (eq. I_top-k): a radix select over
// order-preserving 32-bit keys finds the k-th best score exactly, ties at
// that score are taken lowest-index first, and two block-wide prefix scans
// compact the winners in ascending thought index.
#include "zr_internal.h"

namespace zr {

// ---------------------------------------------------------------------------
// Coarse scorer: one workgroup (one wave) per (64 thoughts, KV head, sequence).
// The group's query-head sum lives in LDS as float64; each lane scores one
// thought by walking its summary key in 16-byte chunks.
// ---------------------------------------------------------------------------
template <typename E, int D>
__global__ void __launch_bounds__(64)
coarse_score_kernel(const typename E::storage* __restrict__ q,
                    const typename E::storage* __restrict__ kbar,
                    const int32_t* __restrict__ seq_ptr, float* __restrict__ scores,
                    int Hq, int Hkv, int n_total) {
  constexpr int VPL = 16 / E::kBytes;
  const int b = blockIdx.z, g = blockIdx.y;
  const int G = Hq / Hkv;
  __shared__ double qsum[D];
  for (int e = threadIdx.x; e < D; e += 64) {
    double acc = 0.0;
    for (int h = 0; h < G; ++h)
      acc += static_cast<double>(load_elem<E>(q, (static_cast<size_t>(b) * Hq + g * G + h) * D + e));
    qsum[e] = acc;
  }
  __syncthreads();
  int lo = seq_ptr[b], hi = seq_ptr[b + 1];
  hi = hi < n_total ? hi : n_total;
  const int i = lo + blockIdx.x * 64 + threadIdx.x;
  if (i < lo || i >= hi) return;
  const uint4* row = reinterpret_cast<const uint4*>(kbar + (static_cast<size_t>(i) * Hkv + g) * D);
  double acc = 0.0;
#pragma unroll 4
  for (int c = 0; c < D / VPL; ++c) {
    float x[VPL];
    unpack16<E>(row[c], x);
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc = fma(qsum[c * VPL + v], static_cast<double>(x[v]), acc);
  }
  scores[static_cast<size_t>(i) * Hkv + g] = static_cast<float>(acc);
}

hipError_t launch_coarse_score(const zr_geom& gm, const void* q, const zr_thoughts& th,
                               float* scores, hipStream_t s) {
  if (gm.batch == 0 || th.max_per_seq == 0) return hipSuccess;
  dim3 grid((th.max_per_seq + 63) / 64, gm.n_kv_heads, gm.batch);
  if (gm.dtype == ZR_BF16) {
    auto qp = static_cast<const uint16_t*>(q);
    auto kp = static_cast<const uint16_t*>(th.summary_keys);
    if (gm.head_dim == 128)
      hipLaunchKernelGGL((coarse_score_kernel<BF16, 128>), grid, dim3(64), 0, s, qp, kp,
                         th.seq_ptr, scores, gm.n_q_heads, gm.n_kv_heads, th.n_total);
    else
      hipLaunchKernelGGL((coarse_score_kernel<BF16, 64>), grid, dim3(64), 0, s, qp, kp,
                         th.seq_ptr, scores, gm.n_q_heads, gm.n_kv_heads, th.n_total);
  } else {
    auto qp = static_cast<const float*>(q);
    auto kp = static_cast<const float*>(th.summary_keys);
    if (gm.head_dim == 128)
      hipLaunchKernelGGL((coarse_score_kernel<F32, 128>), grid, dim3(64), 0, s, qp, kp,
                         th.seq_ptr, scores, gm.n_q_heads, gm.n_kv_heads, th.n_total);
    else
      hipLaunchKernelGGL((coarse_score_kernel<F32, 64>), grid, dim3(64), 0, s, qp, kp,
                         th.seq_ptr, scores, gm.n_q_heads, gm.n_kv_heads, th.n_total);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Top-k selector: one 256-thread workgroup per (KV head, sequence).
// ---------------------------------------------------------------------------
constexpr int kSelThreads = 256;

// Larger key = better score. NaN maps below every number; -0 maps like +0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0u;  // NaN
  if (u == 0x80000000u) u = 0u;                     // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum of one value per thread across the workgroup: a
// shuffle scan inside each wave, then the wave totals. `tmp` holds
// kSelThreads / 64 entries. *total gets the workgroup sum. Contains
// barriers: every thread must call it.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* tmp, uint32_t* total) {
  constexpr int kW = kSelThreads / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t x = __shfl_up(incl, o);
    if (lane >= o) incl += x;
  }
  if (lane == 63) tmp[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) {
    const uint32_t t = tmp[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__global__ void __launch_bounds__(kSelThreads)
select_topk_kernel(const float* __restrict__ scores, const int32_t* __restrict__ seq_ptr,
                   int Hkv, int k, int n_total, int max_per_seq, int32_t* __restrict__ sel) {
  extern __shared__ uint32_t keys[];  // max_per_seq entries
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_tmp[kSelThreads / 64];
  __shared__ uint32_t sh_prefix, sh_remaining;

  const int g = blockIdx.x, b = blockIdx.y, t = threadIdx.x;
  const int lane = t & 63;
  int lo = seq_ptr[b], hi = seq_ptr[b + 1];
  hi = hi < n_total ? hi : n_total;
  int n = hi - lo;
  n = n < 0 ? 0 : (n > max_per_seq ? max_per_seq : n);
  int32_t* out = sel + (static_cast<size_t>(b) * Hkv + g) * k;

  if (n <= k) {  // every thought is kept
    for (int i = t; i < k; i += kSelThreads) out[i] = i < n ? i : -1;
    return;
  }
  for (int i = t; i < n; i += kSelThreads)
    keys[i] = order_key(scores[static_cast<size_t>(lo + i) * Hkv + g]);

  // Radix select, most significant byte first: after the four passes
  // `prefix` is the k-th largest key and `remaining` the number of elements
  // equal to it that still belong to the top k.
  uint32_t prefix = 0, mask = 0, remaining = static_cast<uint32_t>(k);
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[t] = 0;  // kSelThreads == 256 bins
    __syncthreads();
    for (int i = t; i < n; i += kSelThreads) {
      const uint32_t key = keys[i];
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (t < 64) {
      // lane L owns digits 4L .. 4L+3; find the digit d where the count of
      // keys with a larger digit is < remaining <= that count + hist[d]
      const uint32_t c0 = hist[4 * lane], c1 = hist[4 * lane + 1], c2 = hist[4 * lane + 2],
                     c3 = hist[4 * lane + 3];
      const uint32_t mine = c0 + c1 + c2 + c3;
      uint32_t suffix = mine;  // keys in digits >= 4 * lane
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_down(suffix, o);
        if (lane + o < 64) suffix += x;
      }
      const unsigned long long hit = __ballot(suffix >= remaining);
      const int L = 63 - __clzll(hit);  // last lane whose suffix still covers k
      if (lane == L) {
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
        sh_prefix = prefix | (static_cast<uint32_t>(digit) << shift);
        sh_remaining = remaining - above;
      }
    }
    __syncthreads();
    prefix = sh_prefix;
    remaining = sh_remaining;
    mask |= 0xffu << shift;
  }
  const uint32_t kth = prefix;

  // Each thread owns a contiguous run of indices so scans follow index order.
  const int per = (n + kSelThreads - 1) / kSelThreads;
  const int i0 = t * per;
  const int i1 = i0 + per < n ? i0 + per : n;
  uint32_t n_eq = 0;
  for (int i = i0; i < i1; ++i) n_eq += keys[i] == kth;
  uint32_t tot;
  const uint32_t eq_before = block_exclusive_scan(n_eq, scan_tmp, &tot);
  uint32_t n_sel = 0;
  {
    uint32_t r = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = keys[i];
      if (key > kth) {
        ++n_sel;
      } else if (key == kth) {
        n_sel += r < remaining;
        ++r;
      }
    }
  }
  uint32_t pos = block_exclusive_scan(n_sel, scan_tmp, &tot);
  {
    uint32_t r = eq_before;
    for (int i = i0; i < i1; ++i) {
      const uint32_t key = keys[i];
      bool take = false;
      if (key > kth) {
        take = true;
      } else if (key == kth) {
        take = r < remaining;
        ++r;
      }
      if (take && pos < static_cast<uint32_t>(k)) out[pos++] = i;
    }
  }
}

hipError_t launch_select_topk(const zr_geom& gm, const zr_thoughts& th, const float* scores,
                              int k, int32_t* sel, hipStream_t s) {
  if (gm.batch == 0 || k == 0) return hipSuccess;
  dim3 grid(gm.n_kv_heads, gm.batch);
  size_t lds = static_cast<size_t>(th.max_per_seq > 0 ? th.max_per_seq : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(select_topk_kernel, grid, dim3(kSelThreads), lds, s, scores, th.seq_ptr,
                     gm.n_kv_heads, k, th.n_total, th.max_per_seq, sel);
  return hipGetLastError();
}

}  // namespace zr

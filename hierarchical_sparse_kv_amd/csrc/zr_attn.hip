// Split-K decode attention over a paged KV pool, sparse ("zoomed-in") and dense.
//
// The attended token list of one (sequence b, KV head g) is
//   sparse: the selected thoughts' spans [start, start+len) clipped below
//           T - window, in the order of `sel`, followed by the window
//           [T - window, T)  (ZoomR Sec. 3.3 eq. I_f restricted to I_w and R_i;
//           clipping makes the union count every token once);
//   dense:  [0, T).
// Each token j is read through the block table, row
// pool[block_table[b][j / 16]][g][j % 16][:] (KV-cache management page,
// paged KV cache, eq. 4), so only the attended rows are fetched: the gather
// reads the kept entries instead of masking the full cache.
//
// Work split. The list is cut into chunks of 4 * CW positions; workgroup
// (split, g, b) handles chunks split, split + S, ... and keeps a running
// (max, sum, weighted V) per query head (online softmax across chunks, a
// two-pass softmax inside a chunk). Each of its four waves resolves CW
// positions (one per lane: binary search of the span prefix sums, block
// table lookup), then loads the K and V rows with 16-byte loads, LPR lanes
// per row (LPR = head_dim * elem_bytes / 16), so a row is one contiguous,
// coalesced segment. Logits are reduced across the row's lanes with lane
// shuffles. The waves merge in LDS and write one partial per workgroup; the
// combine kernel merges the S partials of each (b, g) by log-sum-exp.
// Exponentials use base 2 with the scale folded into q (exp(x) = 2^(x log2 e)).
#include <math.h>

#include "zr_internal.h"

namespace zr {

constexpr int kAttnThreads = 256;
constexpr int kWaves = kAttnThreads / 64;

template <typename E, int D>
struct AttnShape {
  static constexpr int VPL = 16 / E::kBytes;     // values per 16-byte lane load
  static constexpr int LPR = D / VPL;            // lanes per K/V row
  static constexpr int RPW = 64 / LPR;           // rows per wave load
  static constexpr int CW = LPR <= 16 ? 64 : 32; // positions per wave per chunk
  static constexpr int NRG = CW / RPW;           // wave loads per chunk (each of K, V)
  static constexpr int CWG = kWaves * CW;        // positions per workgroup chunk
};

// Sum over the LPR consecutive lanes that hold one row.
template <int LPR>
__device__ __forceinline__ float row_sum(float v) {
#pragma unroll
  for (int o = LPR / 2; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Sum / max over the row slots: lanes that hold the same columns of
// different rows (lane, lane + LPR, lane + 2 LPR, ...).
template <int LPR>
__device__ __forceinline__ float slot_sum(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

template <int LPR>
__device__ __forceinline__ float slot_max(float v) {
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

template <typename E, int D, int G, bool DENSE>
__global__ void __launch_bounds__(kAttnThreads)
attn_partial_kernel(AttnArgs a) {
  using Sh = AttnShape<E, D>;
  using St = typename E::storage;
  constexpr int VPL = Sh::VPL, LPR = Sh::LPR, RPW = Sh::RPW, CW = Sh::CW, NRG = Sh::NRG,
                CWG = Sh::CWG;
  constexpr float kNegInf = -INFINITY;

  extern __shared__ int32_t span_mem[];  // starts [k + 2] then prefix sums [k + 2]
  __shared__ float red_m[kWaves][G];
  __shared__ float red_l[kWaves][G];
  __shared__ float red_acc[kWaves][G][D];
  __shared__ int sh_nspans;

  const int b = blockIdx.z, g = blockIdx.y, split = blockIdx.x, nsplit = gridDim.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > a.max_blocks * kBlock ? a.max_blocks * kBlock : T);
  const int tw = T - a.window > 0 ? T - a.window : 0;
  int32_t* sp_start = span_mem;
  int32_t* sp_pref = span_mem + (DENSE ? 2 : a.k + 2);

  // ---- attended spans of (b, g) and their exclusive prefix sums ----
  if (DENSE) {
    if (threadIdx.x == 0) {
      sp_start[0] = 0;
      sp_pref[0] = 0;
      sp_pref[1] = T;
      sh_nspans = 1;
    }
  } else if (wave == 0) {
    const int lo = a.seq_ptr[b];
    int hi = a.seq_ptr[b + 1];
    hi = hi < a.n_total ? hi : a.n_total;
    const int n_b = hi - lo > 0 ? hi - lo : 0;
    const int32_t* srow = a.sel + (static_cast<size_t>(b) * a.Hkv + g) * a.k;
    int run = 0;
    for (int base = 0; base < a.k; base += 64) {
      const int i = base + lane;
      int s = 0, len = 0;
      if (i < a.k) {
        const int t = srow[i];
        if (t >= 0 && t < n_b) {
          s = a.th_start[lo + t];
          int e = s + a.th_len[lo + t];
          s = s > 0 ? s : 0;
          e = e < tw ? e : tw;
          len = e - s > 0 ? e - s : 0;
        }
      }
      int incl = len;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (lane >= o) incl += v;
      }
      if (i < a.k) {
        sp_start[i] = s;
        sp_pref[i] = run + incl - len;
      }
      run += __shfl(incl, 63);
    }
    if (lane == 0) {
      sp_start[a.k] = tw;
      sp_pref[a.k] = run;
      sp_pref[a.k + 1] = run + (T - tw);
      sh_nspans = a.k + 1;
    }
  }
  __syncthreads();
  const int nspans = sh_nspans;
  const int total = sp_pref[nspans];

  const St* kp = static_cast<const St*>(a.k_pool);
  const St* vp = static_cast<const St*>(a.v_pool);
  const int cl = lane % LPR;  // which 16-byte chunk of a row this lane holds
  const int rs = lane / LPR;  // which row of a wave load

  float qf[G][VPL];
  {
    const St* qb = static_cast<const St*>(a.q) + (static_cast<size_t>(b) * a.Hq + g * G) * D;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 u = *reinterpret_cast<const uint4*>(qb + h * D + cl * VPL);
      unpack16<E>(u, qf[h]);
#pragma unroll
      for (int v = 0; v < VPL; ++v) qf[h][v] *= a.scale_log2;
    }
  }

  float m_run[G], l_run[G], acc[G][VPL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = kNegInf;
    l_run[h] = 0.f;
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[h][v] = 0.f;
  }

  for (int chunk = split; chunk * CWG < total; chunk += nsplit) {
    const int wbase = chunk * CWG + wave * CW;
    // One position per lane -> pool row index (or -1).
    int row = -1;
    {
      const int p = wbase + lane;
      if (lane < CW && p < total) {
        int lo = 0, hi = nspans - 1;
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (sp_pref[mid] <= p) lo = mid;
          else hi = mid - 1;
        }
        const int j = sp_start[lo] + (p - sp_pref[lo]);
        if (j >= 0 && j < T) {
          const int blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + (j >> 4)];
          if (blk >= 0 && blk < a.num_blocks) row = (blk * a.Hkv + g) * kBlock + (j & 15);
        }
      }
    }
    int rr[NRG];
#pragma unroll
    for (int r = 0; r < NRG; ++r) rr[r] = __shfl(row, r * RPW + rs);
    uint4 kr[NRG], vr[NRG];
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      kr[r] = make_uint4(0, 0, 0, 0);
      if (rr[r] >= 0)
        kr[r] = *reinterpret_cast<const uint4*>(kp + static_cast<size_t>(rr[r]) * D + cl * VPL);
    }
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      vr[r] = make_uint4(0, 0, 0, 0);
      if (rr[r] >= 0)
        vr[r] = *reinterpret_cast<const uint4*>(vp + static_cast<size_t>(rr[r]) * D + cl * VPL);
    }

    float z[NRG][G];
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      float x[VPL];
      unpack16<E>(kr[r], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float s = 0.f;
#pragma unroll
        for (int v = 0; v < VPL; ++v) s = fmaf(qf[h][v], x[v], s);
        s = row_sum<LPR>(s);
        z[r][h] = rr[r] >= 0 ? s : kNegInf;
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mc = kNegInf;
#pragma unroll
      for (int r = 0; r < NRG; ++r) mc = fmaxf(mc, z[r][h]);
      mc = slot_max<LPR>(mc);
      const float mn = fmaxf(m_run[h], mc);
      if (mn != kNegInf) {
        const float alpha = exp2f(m_run[h] - mn);  // 0 when m_run is -inf
        l_run[h] *= alpha;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[h][v] *= alpha;
        m_run[h] = mn;
      }
    }
#pragma unroll
    for (int r = 0; r < NRG; ++r) {
      float x[VPL];
      unpack16<E>(vr[r], x);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = z[r][h] != kNegInf ? exp2f(z[r][h] - m_run[h]) : 0.f;
        l_run[h] += p;
#pragma unroll
        for (int v = 0; v < VPL; ++v) acc[h][v] = fmaf(p, x[v], acc[h][v]);
      }
    }
  }

  // ---- merge the row slots of the wave, then the waves of the workgroup ----
#pragma unroll
  for (int h = 0; h < G; ++h) {
    l_run[h] = slot_sum<LPR>(l_run[h]);
#pragma unroll
    for (int v = 0; v < VPL; ++v) acc[h][v] = slot_sum<LPR>(acc[h][v]);
  }
  if (lane < LPR) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int v = 0; v < VPL; ++v) red_acc[wave][h][cl * VPL + v] = acc[h][v];
  }
  if (lane == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      red_m[wave][h] = m_run[h];
      red_l[wave][h] = l_run[h];
    }
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kAttnThreads) {
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
          A = fmaf(red_acc[w][h][e], f, A);
        }
      }
    }
    const size_t o = ((static_cast<size_t>(b) * a.Hkv + g) * nsplit + split) * G + h;
    a.ws_acc[o * D + e] = A;
    if (e == 0) {
      a.ws_m[o] = M;
      a.ws_l[o] = L;
    }
  }
}

// Merge the S partials of each (b, g): out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s.
template <int D, int G>
__global__ void __launch_bounds__(kAttnThreads)
attn_combine_kernel(AttnArgs a, int nsplit) {
  const int g = blockIdx.x, b = blockIdx.y;
  const size_t base = (static_cast<size_t>(b) * a.Hkv + g) * nsplit;
  for (int idx = threadIdx.x; idx < G * D; idx += kAttnThreads) {
    const int h = idx / D, e = idx % D;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, a.ws_m[(base + s) * G + h]);
    float L = 0.f, A = 0.f;
    if (M != -INFINITY) {
      for (int s = 0; s < nsplit; ++s) {
        const float ms = a.ws_m[(base + s) * G + h];
        if (ms != -INFINITY) {
          const float f = exp2f(ms - M);
          L = fmaf(a.ws_l[(base + s) * G + h], f, L);
          A = fmaf(a.ws_acc[((base + s) * G + h) * D + e], f, A);
        }
      }
    }
    a.out[(static_cast<size_t>(b) * a.Hq + g * G + h) * D + e] = L > 0.f ? A / L : 0.f;
  }
}

int attn_tokens_per_split(const zr_geom& gm) {
  const int bytes = gm.dtype == ZR_BF16 ? 2 : 4;
  const int lpr = gm.head_dim * bytes / 16;
  return kWaves * (lpr <= 16 ? 64 : 32);
}

template <typename E, int D, int G>
static hipError_t launch_typed(const zr_geom& gm, const AttnArgs& a, int splits, bool dense,
                               hipStream_t s) {
  dim3 grid(splits, gm.n_kv_heads, gm.batch);
  if (dense) {
    hipLaunchKernelGGL((attn_partial_kernel<E, D, G, true>), grid, dim3(kAttnThreads),
                       4 * sizeof(int32_t), s, a);
  } else {
    const size_t lds = 2 * static_cast<size_t>(a.k + 2) * sizeof(int32_t);
    hipLaunchKernelGGL((attn_partial_kernel<E, D, G, false>), grid, dim3(kAttnThreads), lds, s,
                       a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((attn_combine_kernel<D, G>), dim3(gm.n_kv_heads, gm.batch),
                     dim3(kAttnThreads), 0, s, a, splits);
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t launch_g(const zr_geom& gm, const AttnArgs& a, int splits, bool dense,
                           hipStream_t s) {
  switch (gm.n_q_heads / gm.n_kv_heads) {
    case 1: return launch_typed<E, D, 1>(gm, a, splits, dense, s);
    case 2: return launch_typed<E, D, 2>(gm, a, splits, dense, s);
    case 4: return launch_typed<E, D, 4>(gm, a, splits, dense, s);
    case 8: return launch_typed<E, D, 8>(gm, a, splits, dense, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attention(const zr_geom& gm, const AttnArgs& a, int splits, bool dense,
                            hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  if (gm.dtype == ZR_BF16)
    return gm.head_dim == 128 ? launch_g<BF16, 128>(gm, a, splits, dense, s)
                              : launch_g<BF16, 64>(gm, a, splits, dense, s);
  return gm.head_dim == 128 ? launch_g<F32, 128>(gm, a, splits, dense, s)
                            : launch_g<F32, 64>(gm, a, splits, dense, s);
}

}  // namespace zr

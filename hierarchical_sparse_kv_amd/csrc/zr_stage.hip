// Moving a step's attended set into device memory (ZoomR Sec. 3.4, "Decoding
// Stage": the full cache stays in host memory and each step brings only the
// entries of I_f to the GPU, at the cost of the host link's bandwidth).
//
// The pools may live in pinned host memory (their device-mapped addresses):
// for every (sequence b, KV head g) pair, the stage kernel copies exactly the
// tiles its attention reads -- the blocks of the selected spans listed by the
// pair kernel, then the blocks of the window [T - W, T) from the block table
// -- into a compact staging pool in device memory, and writes the pair's list
// again with staging block ids. Attention over the staging pool with that
// list and no window of its own is then the attention over the original
// pools: same entries, same order, same slot masks, hence the same work
// split and the same result bit for bit.
//
// Staging layout: block id b * stage_blocks + j holds, at KV head g, the tile
// of entry j of pair (b, g) (keys [16][d], values [d][16], as in the pools),
// so the Hkv pairs of a sequence share staging blocks, each in its own head
// slice. A pair's entries past stage_blocks are not staged; their number is
// reported in `dropped`.
//
// Work items are (pair, kStageEntries consecutive entries), taken by a grid
// of at most kStageGrid workgroups in turn (pairs interleaved). Tiles are
// copied with 16-byte loads and stores, all of a thread's loads issued before
// its stores, so that many host-link requests are in flight per workgroup.
// 128 workgroups keep about 8 MB of host reads in flight, enough for the host
// link: measured 55 GB/s, against 53 GB/s with one workgroup per item (2,112
// workgroups at 16K x 8) and 52, 53 and 54 GB/s with 8, 16 and 32.
#include "zr_internal.h"

namespace zr {

constexpr int kStageThreads = 256;
constexpr int kStageEntries = 8;
constexpr int kStageRound = 16;  // 16-byte pieces per thread in flight
constexpr int kStageGrid = 128;  // workgroups of one launch at most

// Work item (pair p, entries j0 .. j0 + kStageEntries - 1): uniform over the
// workgroup, barriers inside.
__device__ void stage_item(const StageArgs& a, int p, int j0, int* s_blk) {
  const int t = threadIdx.x;
  const int b = div_small(p, a.Hkv), g = p - b * a.Hkv;

  // the pair's list: cached span entries, then the window's blocks
  const int cap = a.max_blocks * kBlock;
  int T = a.seq_lens[b];
  T = T < 0 ? 0 : (T > cap ? cap : T);
  const int tw = T - a.window > 0 ? T - a.window : 0;
  int nc = a.counts[p];
  nc = nc < 0 ? 0 : (nc > a.max_blocks ? a.max_blocks : nc);
  const int wb = T > tw ? ((T - 1) >> 4) - (tw >> 4) + 1 : 0;
  const int n = nc + wb;
  const int ns = n < a.stage_blocks ? n : a.stage_blocks;
  if (j0 == 0 && t == 0) {
    a.s_counts[p] = ns;
    a.s_list_tw[p] = T;  // the staged lists hold the window: no window of their own
    a.dropped[p] = n - ns;
  }
  if (j0 >= ns) return;  // uniform
  const int jn = ns - j0 < kStageEntries ? ns - j0 : kStageEntries;

  if (t < jn) {
    const int j = j0 + t;
    int blk;
    uint32_t m;
    if (j < nc) {
      const int2 e = a.entries[static_cast<size_t>(p) * a.max_blocks + j];
      blk = e.x;
      m = static_cast<uint32_t>(e.y) & 0xffffu;
    } else {
      const int lb = (tw >> 4) + (j - nc);
      const int b0 = lb << 4;
      const int from = (tw > b0 ? tw : b0) - b0;
      const int to = (T < b0 + kBlock ? T : b0 + kBlock) - b0;
      blk = a.block_table[static_cast<size_t>(b) * a.max_blocks + lb];
      m = ((1u << to) - 1u) & ~((1u << from) - 1u);
    }
    if (blk < 0 || blk >= a.num_blocks) {  // nothing to copy; the entry stays empty
      blk = -1;
      m = 0u;
    }
    s_blk[t] = blk;
    a.s_entries[static_cast<size_t>(p) * a.s_stride + j] =
        make_int2(b * a.stage_blocks + j, static_cast<int>(m));
  }
  __syncthreads();

  // copy: tile u of the workgroup (entry u / 2, keys if u is even, else
  // values) is 2^lg_pieces pieces of 16 bytes; rounds of kStageRound pieces
  // per thread, loads first
  const int lgp = a.lg_pieces;
  const int total = (jn * 2) << lgp;
  const uint4* ksrc = static_cast<const uint4*>(a.k_pool);
  const uint4* vsrc = static_cast<const uint4*>(a.v_pool);
  uint4* kdst = static_cast<uint4*>(a.k_stage);
  uint4* vdst = static_cast<uint4*>(a.v_stage);
  for (int x0 = 0; x0 < total; x0 += kStageRound * kStageThreads) {
    uint4 buf[kStageRound];
    size_t dst_at[kStageRound];
    bool is_v[kStageRound], live[kStageRound];
#pragma unroll
    for (int i = 0; i < kStageRound; ++i) {
      const int x = x0 + t + i * kStageThreads;
      const bool in = x < total;
      const int u = in ? x >> lgp : 0, piece = in ? x & ((1 << lgp) - 1) : 0;
      const int e = u >> 1;
      const int blk = s_blk[e];
      live[i] = in && blk >= 0;
      is_v[i] = (u & 1) != 0;
      const size_t src_tile = static_cast<size_t>(live[i] ? blk : 0) * a.Hkv + g;
      const size_t dst_tile = static_cast<size_t>(b * a.stage_blocks + j0 + e) * a.Hkv + g;
      dst_at[i] = (dst_tile << lgp) + piece;
      buf[i] = make_uint4(0u, 0u, 0u, 0u);
      const size_t src = (src_tile << lgp) + piece;
      if (live[i]) buf[i] = is_v[i] ? vsrc[src] : ksrc[src];
    }
#pragma unroll
    for (int i = 0; i < kStageRound; ++i) {
      if (live[i]) {
        if (is_v[i]) vdst[dst_at[i]] = buf[i];
        else kdst[dst_at[i]] = buf[i];
      }
    }
  }
}

__global__ void __launch_bounds__(kStageThreads)
stage_kernel(StageArgs a) {
  const int P = a.B * a.Hkv;
  const int n_items = a.item_chunks * P;
  __shared__ int s_blk[kStageEntries];
  for (int item = blockIdx.x; item < n_items; item += gridDim.x) {
    if (item != static_cast<int>(blockIdx.x)) __syncthreads();  // s_blk of the last item read
    stage_item(a, item % P, (item / P) * kStageEntries, s_blk);
  }
}

hipError_t launch_stage(const zr_geom& gm, const StageArgs& a_in, hipStream_t s) {
  if (gm.batch == 0) return hipSuccess;
  StageArgs a = a_in;
  a.item_chunks = (a.stage_blocks + kStageEntries - 1) / kStageEntries;
  const int64_t items = static_cast<int64_t>(a.item_chunks) * gm.batch * gm.n_kv_heads;
  const int grid = static_cast<int>(items < kStageGrid ? items : kStageGrid);
  hipLaunchKernelGGL(stage_kernel, dim3(grid), dim3(kStageThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace zr

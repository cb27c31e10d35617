// C ABI of libzr: argument validation, then kernel launches on the caller's
// stream. Nothing here allocates, frees or synchronizes.
#include <math.h>

#include "zr_internal.h"

#define ZR_API extern "C" __attribute__((visibility("default")))

namespace {

constexpr float kLog2e = 1.4426950408889634f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

zr_status check_geom(const zr_geom* g) {
  if (!g) return ZR_E_NULL;
  if (g->batch < 0 || g->n_q_heads <= 0 || g->n_kv_heads <= 0 || g->head_dim <= 0 ||
      g->max_blocks_per_seq <= 0 || g->num_blocks <= 0)
    return ZR_E_SHAPE;
  if (g->n_q_heads % g->n_kv_heads != 0) return ZR_E_SHAPE;
  const int G = g->n_q_heads / g->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return ZR_E_UNSUPPORTED;
  if (G == 16 && g->dtype != ZR_BF16) return ZR_E_UNSUPPORTED;
  if (g->head_dim != 64 && g->head_dim != 128) return ZR_E_UNSUPPORTED;
  if (g->block_size != ZR_BLOCK_SIZE) return ZR_E_UNSUPPORTED;
  if (g->dtype != ZR_F32 && g->dtype != ZR_BF16) return ZR_E_UNSUPPORTED;
  // pool row indices are int32 inside the kernels
  if (static_cast<int64_t>(g->num_blocks) * g->n_kv_heads * ZR_BLOCK_SIZE > INT32_MAX)
    return ZR_E_UNSUPPORTED;
  if (static_cast<int64_t>(g->max_blocks_per_seq) * ZR_BLOCK_SIZE > INT32_MAX / 2)
    return ZR_E_SHAPE;
  return ZR_OK;
}

zr_status check_thoughts(const zr_thoughts* th, bool need_keys) {
  if (!th) return ZR_E_NULL;
  if (!th->seq_ptr || !th->start || !th->len) return ZR_E_NULL;
  if (need_keys && !th->summary_keys) return ZR_E_NULL;
  if (th->n_total < 0 || th->max_per_seq < 0) return ZR_E_SHAPE;
  if (th->max_per_seq > ZR_MAX_THOUGHTS_PER_SEQ) return ZR_E_UNSUPPORTED;
  if (need_keys && !aligned16(th->summary_keys)) return ZR_E_ALIGN;
  return ZR_OK;
}

zr_status attention_common(const zr_geom* geom, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, float scale, float* out, void* workspace,
                           size_t ws_bytes, int32_t max_attended, zr::AttnArgs* a) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !out) return ZR_E_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool)) return ZR_E_ALIGN;
  if (max_attended < 0) return ZR_E_SHAPE;
  if (!isfinite(scale)) return ZR_E_SHAPE;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS)
    return ZR_E_UNSUPPORTED;
  const int nwg = zr::attn_workgroups(*geom, max_attended);
  const size_t need = zr::attn_workspace(*geom, nwg, nullptr, nullptr);
  if (geom->batch > 0 && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return ZR_E_WORKSPACE;
  zr::attn_workspace(*geom, nwg, workspace, a);
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->out = out;
  a->B = geom->batch;
  a->Hq = geom->n_q_heads;
  a->Hkv = geom->n_kv_heads;
  a->max_blocks = geom->max_blocks_per_seq;
  a->num_blocks = geom->num_blocks;
  a->scale_log2 = scale * kLog2e;
  return ZR_OK;
}

}  // namespace

ZR_API const char* zr_status_string(zr_status s) {
  switch (s) {
    case ZR_OK: return "ok";
    case ZR_E_NULL: return "a required pointer is NULL";
    case ZR_E_SHAPE: return "sizes are inconsistent or out of range";
    case ZR_E_UNSUPPORTED: return "this build has no kernel for the requested shape or dtype";
    case ZR_E_WORKSPACE: return "workspace missing, misaligned or smaller than zr_workspace_bytes()";
    case ZR_E_LAUNCH: return "the HIP runtime reported a launch error";
    case ZR_E_ALIGN: return "q, pools or summary keys are not 16-byte aligned";
  }
  return "unknown zr_status";
}

ZR_API size_t zr_workspace_bytes(const zr_geom* geom, int32_t max_attended) {
  if (check_geom(geom) != ZR_OK || max_attended < 0) return 0;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS) return 0;
  return zr::attn_workspace(*geom, zr::attn_workgroups(*geom, max_attended), nullptr, nullptr);
}

ZR_API zr_status zr_coarse_score(const zr_geom* geom, const void* q, const zr_thoughts* th,
                                 float* scores, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, true);
  if (st != ZR_OK) return st;
  if (!q || !scores) return ZR_E_NULL;
  if (!aligned16(q)) return ZR_E_ALIGN;
  if (zr::launch_coarse_score(*geom, q, *th, scores, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_select_topk(const zr_geom* geom, const zr_thoughts* th, const float* scores,
                                int32_t k, int32_t* sel, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (k < 0 || k > ZR_MAX_K) return ZR_E_SHAPE;
  if (k > 0 && (!scores || !sel)) return ZR_E_NULL;
  if (zr::launch_select_topk(*geom, *th, scores, k, sel, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_sparse_decode_attn(const zr_geom* geom, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       const int32_t* seq_lens, const zr_thoughts* th,
                                       const int32_t* sel, int32_t k, int32_t window,
                                       float scale, int32_t max_attended, float* out,
                                       void* workspace, size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (k < 0 || k > ZR_MAX_K || window < 0) return ZR_E_SHAPE;
  if (k > 0 && !sel) return ZR_E_NULL;
  if (!zr::attn_lds_ok(*geom, k, false)) return ZR_E_UNSUPPORTED;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a);
  if (st != ZR_OK) return st;
  a.seq_ptr = th->seq_ptr;
  a.th_start = th->start;
  a.th_len = th->len;
  a.sel = sel;
  a.n_total = th->n_total;
  a.k = k;
  a.window = window;
  if (zr::launch_attention(*geom, a, false, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_dense_paged_decode_attn(const zr_geom* geom, const void* q,
                                            const void* k_pool, const void* v_pool,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            float scale, float* out, void* workspace,
                                            size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (!zr::attn_lds_ok(*geom, 0, true)) return ZR_E_UNSUPPORTED;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, geom->max_blocks_per_seq * ZR_BLOCK_SIZE, &a);
  if (st != ZR_OK) return st;
  if (zr::launch_attention(*geom, a, true, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

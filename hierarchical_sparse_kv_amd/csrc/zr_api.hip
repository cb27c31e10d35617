// C ABI of libzr: argument validation, then kernel launches on the caller's
// stream. Nothing here allocates, frees or synchronizes.
#include <math.h>

#include <mutex>

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

// The workspace of the attention calls for `max_attended` (its layout depends on
// the grid size), checked and laid out into *a.
zr_status attention_workspace(const zr_geom* geom, int32_t max_attended, void* workspace,
                              size_t ws_bytes, zr::AttnArgs* a) {
  if (max_attended < 0) return ZR_E_SHAPE;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS)
    return ZR_E_UNSUPPORTED;
  const int nwg = zr::attn_workgroups(*geom, max_attended);
  const size_t need = zr::attn_workspace(*geom, nwg, nullptr, nullptr);
  if (geom->batch > 0 && (!workspace || ws_bytes < need || !aligned16(workspace)))
    return ZR_E_WORKSPACE;
  zr::attn_workspace(*geom, nwg, workspace, a);
  a->B = geom->batch;
  a->Hq = geom->n_q_heads;
  a->Hkv = geom->n_kv_heads;
  return ZR_OK;
}

// `out` may be null only when need_out is false (the partials-only call).
zr_status attention_common(const zr_geom* geom, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           const int32_t* seq_lens, float scale, float* out, void* workspace,
                           size_t ws_bytes, int32_t max_attended, zr::AttnArgs* a,
                           bool need_out = true) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || (need_out && !out))
    return ZR_E_NULL;
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || (out && !aligned16(out)))
    return ZR_E_ALIGN;
  if (max_attended < 0) return ZR_E_SHAPE;
  if (!isfinite(scale)) return ZR_E_SHAPE;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS)
    return ZR_E_UNSUPPORTED;
  // the work split counts all pairs' list entries (at most 2 max_blocks each) in int32
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads *
          (2 * static_cast<int64_t>(geom->max_blocks_per_seq) + 1) > INT32_MAX)
    return ZR_E_UNSUPPORTED;
  st = attention_workspace(geom, max_attended, workspace, ws_bytes, a);
  if (st != ZR_OK) return st;
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->block_table = block_table;
  a->seq_lens = seq_lens;
  a->plan_lens = seq_lens;
  a->horizon = 0;
  a->out = out;
  a->max_blocks = geom->max_blocks_per_seq;
  a->num_blocks = geom->num_blocks;
  a->scale_log2 = scale * kLog2e;
  return ZR_OK;
}

void fill_pair_sizes(const zr_geom& g, const zr_thoughts& th, int k, int window,
                     zr::PairArgs* pa) {
  pa->n_total = th.n_total;
  pa->max_per_seq = th.max_per_seq;
  pa->Hq = g.n_q_heads;
  pa->Hkv = g.n_kv_heads;
  pa->k = k;
  pa->window = window;
  pa->max_blocks = g.max_blocks_per_seq;
  pa->num_blocks = g.num_blocks;
}

// Plan-mode arguments: the pair kernel writes its block lists into the
// workspace regions the attention kernel reads.
void fill_plan(const zr_geom& g, const zr_thoughts& th, int k, int window,
               const int32_t* block_table, const int32_t* seq_lens, const zr::AttnArgs& a,
               zr::PairArgs* pa) {
  fill_pair_sizes(g, th, k, window, pa);
  pa->seq_lens = seq_lens;
  pa->block_table = block_table;
  pa->counts = const_cast<int32_t*>(a.counts);
  pa->entries = const_cast<int2*>(a.entries);
  pa->list_tw = const_cast<int32_t*>(a.list_tw);
}

}  // namespace

ZR_API const char* zr_status_string(zr_status s) {
  switch (s) {
    case ZR_OK: return "ok";
    case ZR_E_NULL: return "a required pointer is NULL";
    case ZR_E_SHAPE: return "sizes are inconsistent or out of range";
    case ZR_E_UNSUPPORTED: return "the library has no kernel for the requested shape or dtype";
    case ZR_E_WORKSPACE: return "workspace missing, misaligned or smaller than zr_workspace_bytes()";
    case ZR_E_LAUNCH: return "the HIP runtime reported a launch error";
    case ZR_E_ALIGN: return "q, pools, out or summary keys are not 16-byte aligned";
    case ZR_E_SCRATCH:
      return "the call needs more than the built scratch memory (ZR_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown zr_status";
}

ZR_API size_t zr_workspace_bytes(const zr_geom* geom, int32_t max_attended) {
  if (check_geom(geom) != ZR_OK || max_attended < 0) return 0;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS) return 0;
  return zr::attn_workspace(*geom, zr::attn_workgroups(*geom, max_attended), nullptr, nullptr);
}

ZR_API zr_status zr_summary_prefetch_rule(const zr_geom* geom, int32_t n_total,
                                          int32_t max_per_seq, int32_t* rows, float* per_seq,
                                          int32_t* margin) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (!rows || !per_seq || !margin) return ZR_E_NULL;
  if (n_total < 0 || max_per_seq < 0) return ZR_E_SHAPE;
  int r, m;
  float a;
  zr::summary_prefetch_rule(*geom, n_total, max_per_seq, &r, &a, &m);
  *rows = r;
  *per_seq = a;
  *margin = m;
  return ZR_OK;
}

ZR_API zr_status zr_coarse_score(const zr_geom* geom, const void* q, const zr_thoughts* th,
                                 float* scores, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, true);
  if (st != ZR_OK) return st;
  if (!q || !scores) return ZR_E_NULL;
  if (!aligned16(q)) return ZR_E_ALIGN;
  zr::PairArgs a{};
  a.q = q;
  a.kbar = th->summary_keys;
  a.seq_ptr = th->seq_ptr;
  a.scores = scores;
  fill_pair_sizes(*geom, *th, 0, 0, &a);
  if (zr::launch_pair(*geom, a, zr::kModeScore, static_cast<hipStream_t>(stream)) != hipSuccess)
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
  if (k == 0) return ZR_OK;
  if (!scores || !sel) return ZR_E_NULL;
  if (!zr::pair_lds_ok(*geom, th->max_per_seq, k, true, false)) return ZR_E_UNSUPPORTED;
  zr::PairArgs a{};
  a.seq_ptr = th->seq_ptr;
  a.scores = const_cast<float*>(scores);  // read only in this mode
  a.sel = sel;
  fill_pair_sizes(*geom, *th, k, 0, &a);
  if (zr::launch_pair(*geom, a, zr::kModeSelect, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_score_topk(const zr_geom* geom, const void* q, const zr_thoughts* th,
                               int32_t k, float* scores, int32_t* sel, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, true);
  if (st != ZR_OK) return st;
  if (k < 0 || k > ZR_MAX_K) return ZR_E_SHAPE;
  if (!q || !scores) return ZR_E_NULL;
  if (k > 0 && !sel) return ZR_E_NULL;
  if (!aligned16(q)) return ZR_E_ALIGN;
  if (k == 0) return zr_coarse_score(geom, q, th, scores, stream);
  if (!zr::pair_lds_ok(*geom, th->max_per_seq, k, true, false)) return ZR_E_UNSUPPORTED;
  zr::PairArgs a{};
  a.q = q;
  a.kbar = th->summary_keys;
  a.seq_ptr = th->seq_ptr;
  a.scores = scores;
  a.sel = sel;
  fill_pair_sizes(*geom, *th, k, 0, &a);
  if (zr::launch_pair(*geom, a, zr::kModeScoreSelect, static_cast<hipStream_t>(stream)) !=
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
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a);
  if (st != ZR_OK) return st;
  if (!zr::pair_lds_ok(*geom, th->max_per_seq, k, false, true)) return ZR_E_UNSUPPORTED;
  zr::PairArgs pa{};
  pa.seq_ptr = th->seq_ptr;
  pa.th_start = th->start;
  pa.th_len = th->len;
  pa.sel = const_cast<int32_t*>(sel);  // read only in this mode
  fill_plan(*geom, *th, k, window, block_table, seq_lens, a, &pa);
  a.window = window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (zr::launch_pair(*geom, pa, zr::kModePlan, s) != hipSuccess) return ZR_E_LAUNCH;
  if (zr::launch_attention(*geom, a, false, s) != hipSuccess) return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_sparse_decode_step(const zr_geom* geom, const void* q, const void* k_pool,
                                       const void* v_pool, const int32_t* block_table,
                                       const int32_t* seq_lens, const zr_thoughts* th, int32_t k,
                                       int32_t window, float scale, int32_t max_attended,
                                       float* scores, int32_t* sel, float* out,
                                       void* workspace, size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, true);
  if (st != ZR_OK) return st;
  if (k < 0 || k > ZR_MAX_K || window < 0) return ZR_E_SHAPE;
  if (!scores || (k > 0 && !sel)) return ZR_E_NULL;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a);
  if (st != ZR_OK) return st;
  if (!zr::pair_lds_ok(*geom, th->max_per_seq, k, true, true)) return ZR_E_UNSUPPORTED;
  zr::PairArgs pa{};
  pa.q = q;
  pa.kbar = th->summary_keys;
  pa.seq_ptr = th->seq_ptr;
  pa.th_start = th->start;
  pa.th_len = th->len;
  pa.scores = scores;
  pa.sel = sel;
  fill_plan(*geom, *th, k, window, block_table, seq_lens, a, &pa);
  a.window = window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (zr::launch_pair(*geom, pa, zr::kModeStep, s) != hipSuccess) return ZR_E_LAUNCH;
  if (zr::launch_attention(*geom, a, false, s) != hipSuccess) return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_sparse_decode_attn_cached(const zr_geom* geom, const void* q,
                                              const void* k_pool, const void* v_pool,
                                              const int32_t* block_table,
                                              const int32_t* seq_lens, int32_t window,
                                              float scale, int32_t max_attended, float* out,
                                              void* workspace, size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (window < 0) return ZR_E_SHAPE;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a);
  if (st != ZR_OK) return st;
  a.window = window;
  if (zr::launch_attention(*geom, a, false, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_reuse_plan(const zr_geom* geom, const int32_t* block_table,
                               const int32_t* seq_lens, int32_t window, int32_t horizon,
                               int32_t max_attended, void* workspace, size_t ws_bytes,
                               void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (window < 0 || horizon < 0 || max_attended < 0) return ZR_E_SHAPE;
  // a window cannot reach past the table's last slot: a longer horizon plans
  // the same split (and T0 + horizon stays within int32)
  const int32_t cap = geom->max_blocks_per_seq * ZR_BLOCK_SIZE;
  if (horizon > cap) horizon = cap;
  if (!block_table || !seq_lens) return ZR_E_NULL;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads *
          (2 * static_cast<int64_t>(geom->max_blocks_per_seq) + 1) > INT32_MAX)
    return ZR_E_UNSUPPORTED;
  zr::AttnArgs a{};
  st = attention_workspace(geom, max_attended, workspace, ws_bytes, &a);
  if (st != ZR_OK) return st;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.plan_lens = seq_lens;
  a.window = window;
  a.horizon = horizon;
  a.max_blocks = geom->max_blocks_per_seq;
  a.num_blocks = geom->num_blocks;
  a.ws_pref = a.reuse_pref;  // the split's slot bases, kept apart from other calls'
  if (zr::launch_reuse_plan(*geom, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_sparse_decode_attn_reuse(const zr_geom* geom, const void* q,
                                             const void* k_pool, const void* v_pool,
                                             const int32_t* block_table,
                                             const int32_t* seq_lens, float scale,
                                             int32_t max_attended, float* out, void* workspace,
                                             size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a, false);
  if (st != ZR_OK) return st;
  a.window = 0;  // the records (or the settings zr_reuse_plan kept) fix the window
  if (zr::launch_attention_reuse(*geom, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_sparse_decode_attn_partials(const zr_geom* geom, const void* q,
                                                const void* k_pool, const void* v_pool,
                                                const int32_t* block_table,
                                                const int32_t* seq_lens, int32_t window,
                                                float scale, int32_t max_attended,
                                                void* workspace, size_t ws_bytes,
                                                void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (window < 0) return ZR_E_SHAPE;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, nullptr,
                        workspace, ws_bytes, max_attended, &a, false);
  if (st != ZR_OK) return st;
  a.window = window;
  if (zr::launch_attention_partials(*geom, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_attn_combine(const zr_geom* geom, int32_t max_attended, float* out,
                                 void* workspace, size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (!out) return ZR_E_NULL;
  if (!aligned16(out)) return ZR_E_ALIGN;
  zr::AttnArgs a{};
  st = attention_workspace(geom, max_attended, workspace, ws_bytes, &a);
  if (st != ZR_OK) return st;
  a.out = out;
  if (zr::launch_combine(*geom, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_append_kv(const zr_geom* geom, void* k_pool, void* v_pool,
                              int32_t* block_table, int32_t* seq_lens, const void* k_new,
                              const void* v_new, const int32_t* free_blocks,
                              int32_t* free_count, int32_t* status, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (geom->batch == 0) return ZR_OK;
  if (!k_pool || !v_pool || !block_table || !seq_lens || !k_new || !v_new || !free_blocks ||
      !free_count || !status)
    return ZR_E_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return ZR_E_ALIGN;
  zr::AppendArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.k_new = k_new;
  a.v_new = v_new;
  a.free_blocks = free_blocks;
  a.free_count = free_count;
  a.status = status;
  a.Hkv = geom->n_kv_heads;
  a.D = geom->head_dim;
  a.max_blocks = geom->max_blocks_per_seq;
  a.num_blocks = geom->num_blocks;
  if (zr::launch_append(*geom, a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_summary_keys(const zr_geom* geom, const void* k_pool,
                                 const int32_t* block_table, const zr_thoughts* th,
                                 const int32_t* which, int32_t n_which, void* summary_keys,
                                 void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (n_which < 0) return ZR_E_SHAPE;
  if (n_which == 0 || geom->batch == 0) return ZR_OK;
  if (!k_pool || !block_table || !which || !summary_keys) return ZR_E_NULL;
  if (!aligned16(k_pool) || !aligned16(summary_keys)) return ZR_E_ALIGN;
  if (n_which > 65535 * 1024) return ZR_E_UNSUPPORTED;
  zr::SummaryArgs a{};
  a.k_pool = k_pool;
  a.block_table = block_table;
  a.seq_ptr = th->seq_ptr;
  a.th_start = th->start;
  a.th_len = th->len;
  a.which = which;
  a.out = summary_keys;
  a.B = geom->batch;
  a.Hkv = geom->n_kv_heads;
  a.max_blocks = geom->max_blocks_per_seq;
  a.num_blocks = geom->num_blocks;
  a.n_total = th->n_total;
  if (zr::launch_summary_keys(*geom, a, n_which, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_consensus(const zr_geom* geom, const zr_thoughts* th, const int32_t* sel,
                              int32_t n_layers, int32_t k, int32_t c, int32_t* votes,
                              int32_t* cons, float* agree, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (n_layers < 0 || k < 0 || k > ZR_MAX_K || c < 0 || c > ZR_MAX_K) return ZR_E_SHAPE;
  if (geom->batch == 0) return ZR_OK;
  if (!votes || !agree || (c > 0 && !cons) || (n_layers > 0 && k > 0 && !sel))
    return ZR_E_NULL;
  if (!zr::consensus_lds_ok(th->max_per_seq, c)) return ZR_E_UNSUPPORTED;
  zr::ConsArgs a{};
  a.seq_ptr = th->seq_ptr;
  a.sel = sel;
  a.votes = votes;
  a.cons = cons;
  a.agree = agree;
  a.B = geom->batch;
  a.Hkv = geom->n_kv_heads;
  a.k = (n_layers > 0 && sel) ? k : 0;
  a.n_layers = n_layers;
  a.c = c;
  a.n_total = th->n_total;
  a.max_per_seq = th->max_per_seq;
  if (zr::launch_consensus(a, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_zoom_decode_attn(const zr_geom* geom, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, const zr_thoughts* th,
                                     const int32_t* sum_start, const int32_t* sum_len,
                                     const int32_t* votes, const int32_t* cons, int32_t c,
                                     int32_t n_prompt, int32_t window, float scale,
                                     int32_t max_attended, float* out, void* workspace,
                                     size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (c < 0 || c > ZR_MAX_K || n_prompt < 0 || window < 0) return ZR_E_SHAPE;
  if (!sum_start || !sum_len || !votes || (c > 0 && !cons)) return ZR_E_NULL;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, max_attended, &a);
  if (st != ZR_OK) return st;
  if (!zr::zoom_lds_ok(*geom, th->max_per_seq)) return ZR_E_UNSUPPORTED;
  zr::PairArgs pa{};
  pa.seq_ptr = th->seq_ptr;
  pa.th_start = th->start;
  pa.th_len = th->len;
  pa.sum_start = sum_start;
  pa.sum_len = sum_len;
  pa.votes = votes;
  pa.cons = cons;
  pa.c = c;
  pa.n_prompt = n_prompt;
  fill_plan(*geom, *th, 0, window, block_table, seq_lens, a, &pa);
  a.window = window;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (zr::launch_zoom_plan(*geom, pa, s) != hipSuccess) return ZR_E_LAUNCH;
  if (zr::launch_attention(*geom, a, false, s) != hipSuccess) return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_dense_paged_decode_attn(const zr_geom* geom, const void* q,
                                            const void* k_pool, const void* v_pool,
                                            const int32_t* block_table, const int32_t* seq_lens,
                                            float scale, float* out, void* workspace,
                                            size_t ws_bytes, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  zr::AttnArgs a{};
  st = attention_common(geom, q, k_pool, v_pool, block_table, seq_lens, scale, out, workspace,
                        ws_bytes, geom->max_blocks_per_seq * ZR_BLOCK_SIZE, &a);
  if (st != ZR_OK) return st;
  if (zr::launch_attention(*geom, a, true, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ZR_E_LAUNCH;
  return ZR_OK;
}

ZR_API zr_status zr_stage_selected(const zr_geom* geom, const void* k_pool, const void* v_pool,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const zr_thoughts* th, const int32_t* sel, int32_t k,
                                   int32_t window, int32_t max_attended, void* workspace,
                                   size_t ws_bytes, int32_t stage_blocks, void* k_stage,
                                   void* v_stage, void* stage_workspace, size_t stage_ws_bytes,
                                   int32_t* dropped, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  st = check_thoughts(th, false);
  if (st != ZR_OK) return st;
  if (k < 0 || k > ZR_MAX_K || window < 0 || max_attended < 0) return ZR_E_SHAPE;
  // a pair lists at most max_blocks_per_seq + 1 entries (every block, and
  // the block where its spans stop and its window starts twice)
  if (stage_blocks < 1 || stage_blocks > geom->max_blocks_per_seq + 1) return ZR_E_SHAPE;
  if (!k_pool || !v_pool || !block_table || !seq_lens || !k_stage || !v_stage || !dropped ||
      (k > 0 && !sel))
    return ZR_E_NULL;
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_stage) || !aligned16(v_stage))
    return ZR_E_ALIGN;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS)
    return ZR_E_UNSUPPORTED;
  // staging pool row indices are int32 inside the kernels, as the pools'
  if (static_cast<int64_t>(geom->batch) * stage_blocks * geom->n_kv_heads * ZR_BLOCK_SIZE >
      INT32_MAX)
    return ZR_E_UNSUPPORTED;
  if (!zr::pair_lds_ok(*geom, th->max_per_seq, k, false, true)) return ZR_E_UNSUPPORTED;
  zr::AttnArgs a{}, sa{};
  st = attention_workspace(geom, max_attended, workspace, ws_bytes, &a);
  if (st != ZR_OK) return st;
  zr_geom gs = *geom;  // the staged geometry: lists one entry longer
  gs.num_blocks = geom->batch > 0 ? geom->batch * stage_blocks : 1;
  gs.max_blocks_per_seq = geom->max_blocks_per_seq + 1;
  st = attention_workspace(&gs, max_attended, stage_workspace, stage_ws_bytes, &sa);
  if (st != ZR_OK) return st;
  if (geom->batch == 0) return ZR_OK;
  zr::PairArgs pa{};
  pa.seq_ptr = th->seq_ptr;
  pa.th_start = th->start;
  pa.th_len = th->len;
  pa.sel = const_cast<int32_t*>(sel);  // read only in this mode
  fill_plan(*geom, *th, k, window, block_table, seq_lens, a, &pa);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (zr::launch_pair(*geom, pa, zr::kModePlan, s) != hipSuccess) return ZR_E_LAUNCH;
  zr::StageArgs ga{};
  ga.k_pool = k_pool;
  ga.v_pool = v_pool;
  ga.block_table = block_table;
  ga.seq_lens = seq_lens;
  ga.counts = a.counts;
  ga.entries = a.entries;
  ga.k_stage = k_stage;
  ga.v_stage = v_stage;
  ga.s_counts = const_cast<int32_t*>(sa.counts);  // written by the stage kernel
  ga.s_list_tw = const_cast<int32_t*>(sa.list_tw);
  ga.s_stride = gs.max_blocks_per_seq;
  ga.s_entries = const_cast<int2*>(sa.entries);
  ga.dropped = dropped;
  ga.B = geom->batch;
  ga.Hkv = geom->n_kv_heads;
  ga.max_blocks = geom->max_blocks_per_seq;
  ga.num_blocks = geom->num_blocks;
  ga.window = window;
  ga.stage_blocks = stage_blocks;
  const int tile = ZR_BLOCK_SIZE * geom->head_dim * (geom->dtype == ZR_BF16 ? 2 : 4);
  ga.lg_pieces = __builtin_ctz(static_cast<unsigned>(tile / 16));
  if (zr::launch_stage(*geom, ga, s) != hipSuccess) return ZR_E_LAUNCH;
  return ZR_OK;
}

// ---------------------------------------------------------------------------
// The sparse decode step without a caller workspace: its kernels use a
// file-scope device array instead. In host code `scratch` names a host-side
// stand-in, not device memory, so its device address is taken once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is handed to the kernels.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kScratchBytes = ZR_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's `scratch` (nullptr and *err set on failure).
void* scratch_address(hipError_t* err) {
  int dev = -1;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (*err != hipSuccess || !p) {
      if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

ZR_API zr_status zr_sparse_decode_step_noalloc(const zr_geom* geom, const void* q,
                                               const void* k_pool, const void* v_pool,
                                               const int32_t* block_table,
                                               const int32_t* seq_lens, const zr_thoughts* th,
                                               int32_t k, int32_t window, float scale,
                                               int32_t max_attended, float* scores, int32_t* sel,
                                               float* out, void* stream) {
  zr_status st = check_geom(geom);
  if (st != ZR_OK) return st;
  if (max_attended < 0) return ZR_E_SHAPE;
  if (static_cast<int64_t>(geom->batch) * geom->n_kv_heads > ZR_MAX_PAIRS)
    return ZR_E_UNSUPPORTED;
  const size_t need = zr::attn_workspace(*geom, zr::attn_workgroups(*geom, max_attended),
                                         nullptr, nullptr);
  if (need > kScratchBytes) return ZR_E_SCRATCH;
  if (geom->batch == 0) return ZR_OK;
  hipError_t err;
  void* ws = scratch_address(&err);
  if (!ws) return ZR_E_LAUNCH;
  return zr_sparse_decode_step(geom, q, k_pool, v_pool, block_table, seq_lens, th, k, window,
                               scale, max_attended, scores, sel, out, ws, kScratchBytes, stream);
}

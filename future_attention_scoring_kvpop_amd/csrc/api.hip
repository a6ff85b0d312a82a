// api.hip -- the extern "C" entry points of libkvpop: argument checks on the
// host, workspace sizing, then the kernel launches.  Nothing here allocates,
// frees or synchronises.
#include <math.h>
#include <stdint.h>

#include "kvpop.h"
#include "launch.h"

using kvpop::AttnShape;

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool group_ok(int Hq, int Hkv) {
  if (Hq <= 0 || Hkv <= 0 || Hq % Hkv) return false;
  const int G = Hq / Hkv;
  return 128 % G == 0;
}

// common checks for the (B, Hq, Hkv, S, D) attention shape
kvpop_status check_dims(const kvpop_dims* d, AttnShape* out) {
  if (!d) return KVPOP_ERR_INVALID_ARGUMENT;
  if (d->batch <= 0 || d->n_q_heads <= 0 || d->n_kv_heads <= 0 || d->seq_len <= 0 ||
      d->head_dim <= 0)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (d->n_q_heads % d->n_kv_heads) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!group_ok(d->n_q_heads, d->n_kv_heads)) return KVPOP_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
  if (!(d->scale == d->scale) || isinf(d->scale)) return KVPOP_ERR_INVALID_ARGUMENT;
  // flat indices are formed in 32-bit where a row count fits; keep shapes in range
  const double elems = (double)d->batch * d->n_q_heads * d->seq_len * d->head_dim;
  if (elems > 9.0e15) return KVPOP_ERR_INVALID_ARGUMENT;
  if ((double)d->seq_len * 4 > 2.0e9) return KVPOP_ERR_UNSUPPORTED;
  out->B = d->batch;
  out->Hq = d->n_q_heads;
  out->Hkv = d->n_kv_heads;
  out->S = d->seq_len;
  out->D = d->head_dim;
  out->scale = d->scale > 0.f ? d->scale : 1.0f / sqrtf((float)d->head_dim);
  return KVPOP_OK;
}

kvpop_status from_hip(hipError_t e) { return e == hipSuccess ? KVPOP_OK : KVPOP_ERR_DEVICE; }

}  // namespace

extern "C" {

int kvpop_abi_version(void) { return KVPOP_ABI_VERSION; }

const char* kvpop_status_string(kvpop_status s) {
  switch (s) {
    case KVPOP_OK: return "ok";
    case KVPOP_ERR_INVALID_ARGUMENT: return "invalid argument";
    case KVPOP_ERR_UNSUPPORTED: return "unsupported configuration";
    case KVPOP_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KVPOP_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

size_t kvpop_workspace_bytes(int op, const kvpop_dims* dims, int window) {
  AttnShape s;
  if (check_dims(dims, &s) != KVPOP_OK) return 0;
  if (op == KVPOP_OP_FUTURE_TARGET) {
    if (window < 0) return 0;
    return kvpop::plan_target(s, window).workspace_bytes;
  }
  if (op == KVPOP_OP_DECODE) return kvpop::plan_decode(s).workspace_floats * sizeof(float);
  if (op == KVPOP_OP_FWD_LSE) return kvpop::plan_fwd(s).partial_floats * sizeof(float);
  if (op == KVPOP_OP_FWD_LSE_SPARSE) {  // the third argument is the budget
    if (window < 0) return 0;
    if (window == 0) return kvpop::plan_fwd(s).partial_floats * sizeof(float);
    return kvpop::plan_fwd_sparse(s, window).workspace_bytes;
  }
  if (op == KVPOP_OP_FWD_ATTN) return kvpop::fwd_out_workspace_bytes(s);
  return 0;
}

// Keys, keep_until and V^T of one KV head are addressed by 32-bit byte
// offsets (buffer ranges below 2 GiB).
static bool fwd_ranges_ok(const AttnShape& s) {
  const double s_pad = (double)((s.S + 63) / 64 * 64);
  return (double)s.S * s.D * 2 < 2147483648.0 && s_pad * s.D * 2 < 2147483648.0;
}

// Workspace check of the main pass: LSE-only calls need the plan's bytes
// (none for many row blocks), calls with an attention output the V^T buffer.
static kvpop_status check_fwd_workspace(size_t need, size_t align, const void* workspace,
                                        size_t workspace_bytes) {
  if (!need) return KVPOP_OK;
  if (!workspace || !aligned(workspace, align)) return KVPOP_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  return KVPOP_OK;
}

static kvpop_status check_fwd_output(const void* v, const void* o, kvpop_out_dtype o_dtype) {
  if ((v == nullptr) != (o == nullptr)) return KVPOP_ERR_INVALID_ARGUMENT;
  if (v && (!aligned(v, 16) || !aligned(o, 16))) return KVPOP_ERR_INVALID_ARGUMENT;
  if (o_dtype != KVPOP_OUT_F32 && o_dtype != KVPOP_OUT_BF16) return KVPOP_ERR_INVALID_ARGUMENT;
  return KVPOP_OK;
}

kvpop_status kvpop_fwd_lse(const kvpop_dims* dims, const void* q, const void* k, const void* v,
                           float* lse, void* o, kvpop_out_dtype o_dtype, void* workspace,
                           size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !lse) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4)) return KVPOP_ERR_INVALID_ARGUMENT;
  if ((st = check_fwd_output(v, o, o_dtype)) != KVPOP_OK) return st;
  if (!fwd_ranges_ok(s)) return KVPOP_ERR_UNSUPPORTED;
  const size_t need = v ? kvpop::fwd_out_workspace_bytes(s)
                        : kvpop::plan_fwd(s).partial_floats * sizeof(float);
  if ((st = check_fwd_workspace(need, v ? 256 : 16, workspace, workspace_bytes)) != KVPOP_OK)
    return st;
  return from_hip(kvpop::launch_fwd_lse(s, q, k, nullptr, 0, lse, workspace, stream, v, o,
                                        o_dtype == KVPOP_OUT_BF16 ? 1 : 0));
}

kvpop_status kvpop_mlstm_step(int batch, int n_kv_heads, int head_dim, int n_sink, int window,
                              int budget, int pos_q, const void* k_new, const void* v_new,
                              const void* k_cache, const void* v_cache,
                              const kvpop_mlstm_weights* w, float* state, float* slot_score,
                              hipStream_t stream) {
  if (batch <= 0 || n_kv_heads <= 0 || n_sink < 0 || window < 1 || pos_q < 0)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (budget < n_sink + window) return KVPOP_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
  if (!w || !k_new || !v_new || !state) return KVPOP_ERR_INVALID_ARGUMENT;
  if (w->feat != kvpop::kMlstmFeat || w->vdim != kvpop::kMlstmVdim) return KVPOP_ERR_UNSUPPORTED;
  const float* ws[9] = {w->wk, w->wr, w->wv, w->wi, w->bi, w->wf, w->bf, w->wo, w->bo};
  for (int i = 0; i < 9; ++i)  // weight rows are read 16 bytes at a time
    if (!ws[i] || !aligned(ws[i], (i == 4 || i == 6 || i == 7 || i == 8) ? 4 : 16))
      return KVPOP_ERR_INVALID_ARGUMENT;
  if (slot_score && (!k_cache || !v_cache || !aligned(slot_score, 4) || !aligned(k_cache, 2) ||
                     !aligned(v_cache, 2)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(state, 16))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if ((double)batch * n_kv_heads > 2.0e9 || (double)batch * n_kv_heads * budget * head_dim > 9.0e15)
    return KVPOP_ERR_UNSUPPORTED;
  const kvpop::MlstmWeights mw{w->wk, w->wr, w->wv, w->wi, w->bi, w->wf, w->bf, w->wo, w->bo};
  return from_hip(kvpop::launch_mlstm_step(batch, n_kv_heads, head_dim, n_sink, window, budget,
                                           pos_q, k_new, v_new, k_cache, v_cache, mw, state,
                                           slot_score, stream));
}

kvpop_status kvpop_decode_step_mlstm(const kvpop_dims* dims, int n_sink, int window, int pos_q,
                                     const void* k_new, const void* v_new,
                                     const kvpop_mlstm_weights* w, float* state, void* k_cache,
                                     void* v_cache, int32_t* slot_pos, float* slot_score,
                                     const void* q, void* o, kvpop_out_dtype o_dtype, float* lse,
                                     void* workspace, size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  const int budget = s.S;
  if (n_sink < 0 || window < 1 || budget < n_sink + window || pos_q < 0)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (!w || !k_new || !v_new || !state || !k_cache || !v_cache || !slot_pos || !slot_score || !q ||
      !o)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (o_dtype != KVPOP_OUT_F32 && o_dtype != KVPOP_OUT_BF16) return KVPOP_ERR_INVALID_ARGUMENT;
  if (w->feat != kvpop::kMlstmFeat || w->vdim != kvpop::kMlstmVdim) return KVPOP_ERR_UNSUPPORTED;
  const float* ws[9] = {w->wk, w->wr, w->wv, w->wi, w->bi, w->wf, w->bf, w->wo, w->bo};
  for (int i = 0; i < 9; ++i)  // weight rows are read 16 bytes at a time
    if (!ws[i] || !aligned(ws[i], (i == 4 || i == 6 || i == 7 || i == 8) ? 4 : 16))
      return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_pos, 4) || !aligned(slot_score, 4) ||
      !aligned(state, 16) || !aligned(q, 16) || !aligned(o, 4) || (lse && !aligned(lse, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  const kvpop::DecodePlan p = kvpop::plan_decode(s);
  if (p.workspace_floats) {
    if (!workspace || !aligned(workspace, 16)) return KVPOP_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < p.workspace_floats * sizeof(float)) return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  }
  const kvpop::MlstmWeights mw{w->wk, w->wr, w->wv, w->wi, w->bi, w->wf, w->bf, w->wo, w->bo};
  return from_hip(kvpop::launch_decode_step_mlstm(
      s, n_sink, window, pos_q, k_new, v_new, mw, state, k_cache, v_cache, slot_pos, slot_score, q,
      o, o_dtype == KVPOP_OUT_BF16 ? 1 : 0, lse, (float*)workspace, stream));
}

size_t kvpop_running_topk_workspace_bytes(int batch, int n_kv_heads, int seq_len, int n_sink) {
  if (batch <= 0 || n_kv_heads <= 0 || seq_len <= 0 || n_sink < 0) return 0;
  if (seq_len > kvpop::running_topk_max_len()) return 0;
  return kvpop::running_topk_workspace_bytes(batch, n_kv_heads, seq_len, n_sink);
}

kvpop_status kvpop_running_topk(int batch, int n_kv_heads, int seq_len, int n_sink, int window,
                                int budget, const float* scores, const float* log_decay,
                                int32_t* keep_until, int32_t* cutoff, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (batch <= 0 || n_kv_heads <= 0 || seq_len <= 0 || n_sink < 0 || window < 0)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (budget < n_sink + window || budget <= 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!scores || !keep_until) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(scores, 4) || !aligned(keep_until, 4) || (cutoff && !aligned(cutoff, 4)) ||
      (log_decay && !aligned(log_decay, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  // positions, budgets and query indices stay far inside int32
  if ((double)seq_len + window + budget > 2.0e9) return KVPOP_ERR_UNSUPPORTED;
  if (seq_len > kvpop::running_topk_max_len()) return KVPOP_ERR_UNSUPPORTED;
  if ((double)batch * n_kv_heads * ((seq_len + 63) / 64) > 2.0e9) return KVPOP_ERR_UNSUPPORTED;
  const size_t need = kvpop::running_topk_workspace_bytes(batch, n_kv_heads, seq_len, n_sink);
  if (need) {
    if (!workspace || !aligned(workspace, 16)) return KVPOP_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < need) return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  }
  return from_hip(kvpop::launch_running_topk(batch, n_kv_heads, seq_len, n_sink, window, budget,
                                             scores, log_decay, keep_until, cutoff, workspace,
                                             stream));
}

kvpop_status kvpop_fwd_lse_sparse(const kvpop_dims* dims, const void* q, const void* k,
                                  const void* v, const int32_t* keep_until, int budget,
                                  float* lse, void* o, kvpop_out_dtype o_dtype, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !keep_until || !lse || budget < 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(keep_until, 4) || !aligned(lse, 4))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if ((st = check_fwd_output(v, o, o_dtype)) != KVPOP_OK) return st;
  if (!fwd_ranges_ok(s)) return KVPOP_ERR_UNSUPPORTED;
  const size_t need = v ? kvpop::fwd_out_workspace_bytes(s)
                        : budget > 0 ? kvpop::plan_fwd_sparse(s, budget).workspace_bytes
                                     : kvpop::plan_fwd(s).partial_floats * sizeof(float);
  if ((st = check_fwd_workspace(need, (v || budget > 0) ? 256 : 16, workspace, workspace_bytes)) !=
      KVPOP_OK)
    return st;
  return from_hip(kvpop::launch_fwd_lse(s, q, k, (const int*)keep_until, budget, lse, workspace,
                                        stream, v, o, o_dtype == KVPOP_OUT_BF16 ? 1 : 0));
}

kvpop_status kvpop_future_attn_target(const kvpop_dims* dims, const void* q, const void* k,
                                      const float* lse, int window, int lookahead, kvpop_agg agg,
                                      int count_normalize, float* mass, float* mass_per_qhead,
                                      void* workspace, size_t workspace_bytes,
                                      hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  if (!q || !k || !lse || !mass || !workspace) return KVPOP_ERR_INVALID_ARGUMENT;
  if (window < 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (agg != KVPOP_AGG_SUM && agg != KVPOP_AGG_MEAN && agg != KVPOP_AGG_MAX)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(lse, 4) || !aligned(mass, 4) ||
      !aligned(workspace, 256) || (mass_per_qhead && !aligned(mass_per_qhead, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if ((double)s.S + window + 512.0 > 2.0e9) return KVPOP_ERR_UNSUPPORTED;
  // query rows and normalizers are addressed by 32-bit byte offsets within
  // one group's Q and one group's LSE
  if ((double)s.S * s.D * 2 * (s.Hq / s.Hkv) >= 2147483648.0 ||
      (double)s.S * (s.Hq / s.Hkv) * 4 >= 2147483648.0)
    return KVPOP_ERR_UNSUPPORTED;
  if (workspace_bytes < kvpop::plan_target(s, window).workspace_bytes)
    return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  const int la = (lookahead < 0 || lookahead >= s.S) ? -1 : lookahead;  // >= S-1 has no effect
  return from_hip(kvpop::launch_future_target(s, q, k, lse, window, la, (int)agg,
                                              count_normalize ? 1 : 0, mass, mass_per_qhead,
                                              (float*)workspace, stream));
}

kvpop_status kvpop_evict_select(int batch, int n_kv_heads, int seq_len, int head_dim, int n_sink,
                                int window, int budget, const float* scores, const void* k,
                                const void* v, int32_t* slot_pos, float* slot_score, void* k_cache,
                                void* v_cache, hipStream_t stream) {
  if (batch <= 0 || n_kv_heads <= 0 || seq_len <= 0 || n_sink < 0 || window < 0)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (budget < n_sink + window || budget <= 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!scores || !slot_pos) return KVPOP_ERR_INVALID_ARGUMENT;
  if ((k == nullptr) != (v == nullptr)) return KVPOP_ERR_INVALID_ARGUMENT;
  if ((k_cache == nullptr) != (v_cache == nullptr)) return KVPOP_ERR_INVALID_ARGUMENT;
  if (k && !k_cache) return KVPOP_ERR_INVALID_ARGUMENT;
  if (k_cache && !k) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(scores, 4) || !aligned(slot_pos, 4) || (slot_score && !aligned(slot_score, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (k) {
    if (head_dim != 64 && head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16))
      return KVPOP_ERR_INVALID_ARGUMENT;
  }
  if ((double)seq_len + budget > 2.0e9) return KVPOP_ERR_UNSUPPORTED;
  const hipError_t e =
      k ? kvpop::launch_select_gather(batch, n_kv_heads, seq_len, head_dim, n_sink, window, budget,
                                      scores, slot_pos, slot_score, k, v, k_cache, v_cache, stream)
        : kvpop::launch_select(batch, n_kv_heads, seq_len, n_sink, window, budget, scores, slot_pos,
                               slot_score, stream);
  return from_hip(e);
}

kvpop_status kvpop_decode_attend(const kvpop_dims* dims, const void* q, const void* k_cache,
                                 const void* v_cache, const int32_t* slot_pos, void* o,
                                 kvpop_out_dtype o_dtype, float* lse, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  if (!q || !k_cache || !v_cache || !slot_pos || !o) return KVPOP_ERR_INVALID_ARGUMENT;
  if (o_dtype != KVPOP_OUT_F32 && o_dtype != KVPOP_OUT_BF16) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(slot_pos, 4) ||
      !aligned(o, 4) || (lse && !aligned(lse, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  const kvpop::DecodePlan p = kvpop::plan_decode(s);
  if (p.workspace_floats) {
    if (!workspace || !aligned(workspace, 16)) return KVPOP_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < p.workspace_floats * sizeof(float)) return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  }
  return from_hip(kvpop::launch_decode(s, q, k_cache, v_cache, slot_pos, o,
                                       o_dtype == KVPOP_OUT_BF16 ? 1 : 0, lse, (float*)workspace,
                                       stream));
}

kvpop_status kvpop_decode_attend_noalloc(const kvpop_dims* dims, const void* q,
                                         const void* k_cache, const void* v_cache,
                                         const int32_t* slot_pos, void* o,
                                         kvpop_out_dtype o_dtype, float* lse, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  if (!q || !k_cache || !v_cache || !slot_pos || !o) return KVPOP_ERR_INVALID_ARGUMENT;
  if (o_dtype != KVPOP_OUT_F32 && o_dtype != KVPOP_OUT_BF16) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(slot_pos, 4) ||
      !aligned(o, 4) || (lse && !aligned(lse, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (kvpop::plan_decode(s).workspace_floats * sizeof(float) > kvpop::decode_noalloc_capacity())
    return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  return from_hip(kvpop::launch_decode_noalloc(s, q, k_cache, v_cache, slot_pos, o,
                                               o_dtype == KVPOP_OUT_BF16 ? 1 : 0, lse, stream));
}

kvpop_status kvpop_score_mlp(int batch, int n_kv_heads, int n_tok, int head_dim, int hidden,
                             const void* keys, const float* w1, const float* b1, const float* w2,
                             const float* b2, float* scores, hipStream_t stream) {
  if (batch <= 0 || n_kv_heads <= 0 || n_tok < 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
  if (hidden < 1 || hidden > 64) return KVPOP_ERR_UNSUPPORTED;
  if (!keys || !w1 || !b1 || !w2 || !b2 || !scores) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!aligned(keys, 16) || !aligned(w1, 4) || !aligned(scores, 4)) return KVPOP_ERR_INVALID_ARGUMENT;
  return from_hip(kvpop::launch_score_mlp(batch, n_kv_heads, n_tok, head_dim, hidden, keys, w1,
                                          b1, w2, b2, scores, stream));
}

kvpop_status kvpop_cache_step(int batch, int n_kv_heads, int head_dim, int n_sink, int window,
                              int budget, int delay, int pos_q, const void* k_new,
                              const void* v_new, const float* w1, const float* b1,
                              const float* w2, const float* b2, int hidden,
                              const float* scores_r, void* k_cache, void* v_cache,
                              int32_t* slot_pos, float* slot_score, hipStream_t stream) {
  if (batch <= 0 || n_kv_heads <= 0 || n_sink < 0 || window < 1) return KVPOP_ERR_INVALID_ARGUMENT;
  if (budget < n_sink + window) return KVPOP_ERR_INVALID_ARGUMENT;
  if (delay < 0 || delay >= window || pos_q < 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (head_dim != 64 && head_dim != 128) return KVPOP_ERR_UNSUPPORTED;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_pos || !slot_score)
    return KVPOP_ERR_INVALID_ARGUMENT;
  const bool mlp = w1 != nullptr;
  if (mlp && scores_r) return KVPOP_ERR_INVALID_ARGUMENT;
  if (mlp && (!b1 || !w2 || !b2)) return KVPOP_ERR_INVALID_ARGUMENT;
  if (mlp && (hidden < 1 || hidden > 64)) return KVPOP_ERR_UNSUPPORTED;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_pos, 4) || !aligned(slot_score, 4))
    return KVPOP_ERR_INVALID_ARGUMENT;
  return from_hip(kvpop::launch_cache_step(batch, n_kv_heads, head_dim, n_sink, window, budget,
                                           delay, pos_q, k_new, v_new, w1, b1, w2, b2,
                                           mlp ? hidden : 0, scores_r, k_cache, v_cache,
                                           slot_pos, slot_score, stream));
}

kvpop_status kvpop_decode_step(const kvpop_dims* dims, int n_sink, int window, int delay,
                               int pos_q, const void* k_new, const void* v_new, const float* w1,
                               const float* b1, const float* w2, const float* b2, int hidden,
                               const float* scores_r, void* k_cache, void* v_cache,
                               int32_t* slot_pos, float* slot_score, const void* q, void* o,
                               kvpop_out_dtype o_dtype, float* lse, void* workspace,
                               size_t workspace_bytes, hipStream_t stream) {
  AttnShape s;
  kvpop_status st = check_dims(dims, &s);
  if (st != KVPOP_OK) return st;
  const int budget = s.S;
  if (n_sink < 0 || window < 1 || budget < n_sink + window) return KVPOP_ERR_INVALID_ARGUMENT;
  if (delay < 0 || delay >= window || pos_q < 0) return KVPOP_ERR_INVALID_ARGUMENT;
  if (!k_new || !v_new || !k_cache || !v_cache || !slot_pos || !slot_score || !q || !o)
    return KVPOP_ERR_INVALID_ARGUMENT;
  if (o_dtype != KVPOP_OUT_F32 && o_dtype != KVPOP_OUT_BF16) return KVPOP_ERR_INVALID_ARGUMENT;
  const bool mlp = w1 != nullptr;
  if (mlp && scores_r) return KVPOP_ERR_INVALID_ARGUMENT;
  if (mlp && (!b1 || !w2 || !b2)) return KVPOP_ERR_INVALID_ARGUMENT;
  if (mlp && (hidden < 1 || hidden > 64)) return KVPOP_ERR_UNSUPPORTED;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(slot_pos, 4) || !aligned(slot_score, 4) ||
      !aligned(q, 16) || !aligned(o, 4) || (lse && !aligned(lse, 4)))
    return KVPOP_ERR_INVALID_ARGUMENT;
  const kvpop::DecodePlan p = kvpop::plan_decode(s);
  if (p.workspace_floats) {
    if (!workspace || !aligned(workspace, 16)) return KVPOP_ERR_INVALID_ARGUMENT;
    if (workspace_bytes < p.workspace_floats * sizeof(float)) return KVPOP_ERR_WORKSPACE_TOO_SMALL;
  }
  return from_hip(kvpop::launch_decode_step(
      s, n_sink, window, delay, pos_q, k_new, v_new, w1, b1, w2, b2, mlp ? hidden : 0, scores_r,
      k_cache, v_cache, slot_pos, slot_score, q, o, o_dtype == KVPOP_OUT_BF16 ? 1 : 0, lse,
      (float*)workspace, stream));
}

}  // extern "C"

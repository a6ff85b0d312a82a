// launch.h -- host-side launchers of the libkvpop kernels.  Argument
// validation happens in api.hip before any of these is called; the
// launchers assume valid, already-checked arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kvpop {

struct AttnShape {
  int B, Hq, Hkv, S, D;
  float scale;
};

// ---- main causal pass (log-normalizers only) ----
struct FwdPlan {
  int P;          // query positions per row block (128 / G)
  int n_pb;       // row blocks per (b, KV head)
  int kmax;       // keys per piece of a split row (multiple of 64)
  int n_pieces;   // pieces of the longest row; 1 = no split
  size_t partial_floats;  // workspace floats (0 without split)
};
FwdPlan plan_fwd(const AttnShape& s);
// Workspace of the listed sparse pass: a header per row block, then one
// key list of cap entries per row block at list_offset.
struct SparsePlan {
  long n_blocks;
  int cap;
  size_t list_offset;
  size_t workspace_bytes;
};
SparsePlan plan_fwd_sparse(const AttnShape& s, int budget);
// keep_until: nullable [B][Hkv][S]; when given, key t counts for row d only
// while t <= d < keep_until[t] (the sparse normalizer).  budget > 0 selects
// the listed pass (workspace from plan_fwd_sparse), else every causal key
// is tested (workspace from plan_fwd).  With v (and o) the pass also writes
// the attention output; every causal key is then read (tested against
// keep_until when given) and the workspace holds V^T
// (fwd_out_workspace_bytes).
size_t fwd_out_workspace_bytes(const AttnShape& s);
hipError_t launch_fwd_lse(const AttnShape& s, const void* q, const void* k, const int* keep_until,
                          int budget, float* lse, void* workspace, hipStream_t st,
                          const void* v = nullptr, void* o = nullptr, int o_bf16 = 0);

// ---- delayed stateful mLSTM scorer (one decoding step) ----
constexpr int kMlstmFeat = 32;   // projected features per Hedgehog half
constexpr int kMlstmVdim = 64;   // value features
constexpr int kMlstmStateFloats = kMlstmVdim * 2 * kMlstmFeat + 2 * kMlstmFeat + 4;  // C, n, m, pad
struct MlstmWeights {
  const float *wk, *wr, *wv, *wi, *bi, *wf, *bf, *wo, *bo;
};
hipError_t launch_mlstm_step(int B, int Hkv, int D, int n_sink, int window, int budget, int pos_q,
                             const void* k_new, const void* v_new, const void* kc, const void* vc,
                             const MlstmWeights& w, float* state, float* slot_score,
                             hipStream_t st);

// mLSTM scorer step, cache step with no scorer, then decode attention (one
// launch when the decode plan needs no slot split)
struct AttnShape;
hipError_t launch_decode_step_mlstm(const AttnShape& s, int n_sink, int window, int pos_q,
                                    const void* k_new, const void* v_new, const MlstmWeights& w,
                                    float* state, void* kc, void* vc, int32_t* slot_pos,
                                    float* slot_score, const void* q, void* o, int o_bf16,
                                    float* lse, float* workspace, hipStream_t st);

// ---- running top-k mask ----
int running_topk_max_len();  // longest row the kernels take
// workspace of a launch (0 when its rows take the counting kernel)
size_t running_topk_workspace_bytes(int B, int Hkv, int S, int n_sink);
hipError_t launch_running_topk(int B, int Hkv, int S, int n_sink, int window, int budget,
                               const float* scores, const float* log_decay, int* keep_until,
                               int* cutoff, void* workspace, hipStream_t st);

// ---- transposed future-attention pass ----
constexpr int kTgtMaxChunks = 64;

struct TargetPlan {
  int waves;      // waves per workgroup
  int ksub;       // 32-key sub-tiles per wave
  int key_block;  // keys per key block (32 x waves x ksub)
  int n_kb;       // key blocks per (b, KV head)
  int chunk;      // query positions per chunk (multiple of 32)
  int n_chunks;   // ceil(S / chunk) <= kTgtMaxChunks
  int max_wg;     // workgroups at most (any lookahead)
  size_t runs;            // (b, KV head, chunk, key block) runs, empty ones included
  size_t partial_floats;  // pieces x key_block
  size_t workspace_bytes; // partials + run table
};

// The transposed pass's list of 32-query squares, in the order (b, KV head),
// query chunk c, key block kb, query head of the group, query tile.  Run
// (c, kb) holds G * n_qtiles(c, kb) squares: the query tiles of chunk c from
// the first at or after kb's first allowed query up to the chunk end or the
// lookahead bound.  cpre[c] = squares of the chunks before c of one (b, h).
struct TargetGeom {
  int G, S, window, key_block, kbt, n_kb, n_chunks, ct, w_t, s_t, la_t, n_wg, rounds;
  int item_mode;     // 1: one workgroup per run (n_wg = all runs, empty ones exit)
  // (32-bit: an even split is only used while the whole list fits; larger
  // launches take one run per workgroup and use none of these)
  int per_bh;  // squares per (b, KV head)
  int total;   // squares in the launch
  int share;   // squares per workgroup
  int cpre[kTgtMaxChunks + 1];
};

__host__ __device__ inline int n_qtiles(const TargetGeom& g, int c, int kb) {
  if (kb * g.key_block + g.window >= g.S) return 0;  // no key of the block has a query
  const int u = kb * g.kbt;
  const int lo = c * g.ct;
  const int hi = (c + 1) * g.ct < g.s_t ? (c + 1) * g.ct : g.s_t;
  const int right = hi < u + g.la_t ? hi : u + g.la_t;
  const int left = lo > u + g.w_t ? lo : u + g.w_t;
  return right > left ? right - left : 0;
}

TargetPlan plan_target(const AttnShape& s, int window);
TargetGeom target_geometry(const AttnShape& s, const TargetPlan& p, int window, int lookahead);
int device_cu_count();
hipError_t launch_future_target(const AttnShape& s, const void* q, const void* k,
                                const float* lse, int window, int lookahead, int agg,
                                int count_normalize, float* mass, float* mass_per_qhead,
                                float* workspace, hipStream_t st);

// ---- retention: selection and compaction ----
hipError_t launch_select(int B, int Hkv, int S, int n_sink, int window, int budget,
                         const float* scores, int32_t* slot_pos, float* slot_score,
                         hipStream_t st);
hipError_t launch_gather(int B, int Hkv, int S, int D, int budget, const int32_t* slot_pos,
                         const void* k, const void* v, void* kc, void* vc, hipStream_t st);
// selection and compaction (fused into one launch when the rows are few)
hipError_t launch_select_gather(int B, int Hkv, int S, int D, int n_sink, int window, int budget,
                                const float* scores, int32_t* slot_pos, float* slot_score,
                                const void* k, const void* v, void* kc, void* vc, hipStream_t st);

// ---- decode ----
struct DecodePlan {
  int n_split;
  int slots_per_split;
  size_t workspace_floats;
};
DecodePlan plan_decode(const AttnShape& s);
hipError_t launch_decode(const AttnShape& s, const void* q, const void* kc, const void* vc,
                         const int32_t* slot_pos, void* o, int o_bf16, float* lse,
                         float* workspace, hipStream_t st);

// Decode attention with the split partials in the library's own fixed
// device array (the allocation-free entry point); the caller checks first
// that plan_decode's workspace fits decode_noalloc_capacity() bytes.
size_t decode_noalloc_capacity();
hipError_t launch_decode_noalloc(const AttnShape& s, const void* q, const void* kc, const void* vc,
                                 const int32_t* slot_pos, void* o, int o_bf16, float* lse,
                                 hipStream_t st);

hipError_t launch_score_mlp(int B, int Hkv, int n_tok, int D, int hidden, const void* keys,
                            const float* w1, const float* b1, const float* w2, const float* b2,
                            float* scores, hipStream_t st);
hipError_t launch_cache_step(int B, int Hkv, int D, int n_sink, int window, int budget,
                             int delay, int pos_q, const void* k_new, const void* v_new,
                             const float* w1, const float* b1, const float* w2,
                             const float* b2, int hidden, const float* scores_r, void* kc,
                             void* vc, int32_t* slot_pos, float* slot_score, hipStream_t st);

// cache step, then decode attention over the updated cache (one launch
// when the decode plan needs no slot split)
hipError_t launch_decode_step(const AttnShape& s, int n_sink, int window, int delay, int pos_q,
                              const void* k_new, const void* v_new, const float* w1,
                              const float* b1, const float* w2, const float* b2, int hidden,
                              const float* scores_r, void* kc, void* vc, int32_t* slot_pos,
                              float* slot_score, const void* q, void* o, int o_bf16, float* lse,
                              float* workspace, hipStream_t st);

}  // namespace kvpop

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
hipError_t launch_fwd_lse(const AttnShape& s, const void* q, const void* k, float* lse,
                          float* workspace, hipStream_t st);

// ---- transposed future-attention pass ----
struct TargetPlan {
  int waves;      // waves per workgroup: 4 (128-key blocks) or 8 (256-key blocks)
  int key_block;  // keys per work item (32 per wave)
  int chunk;      // query positions per work item (multiple of 32)
  int n_chunks;   // ceil(S / chunk)
  int n_kb;       // key blocks
  size_t partial_floats;  // workspace floats (per-query-head partials)
};
TargetPlan plan_target(const AttnShape& s, int window);
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

hipError_t launch_score_mlp(int B, int Hkv, int n_tok, int D, int hidden, const void* keys,
                            const float* w1, const float* b1, const float* w2, const float* b2,
                            float* scores, hipStream_t st);
hipError_t launch_cache_step(int B, int Hkv, int D, int n_sink, int window, int budget,
                             int delay, int pos_q, const void* k_new, const void* v_new,
                             const float* w1, const float* b1, const float* w2,
                             const float* b2, int hidden, const float* scores_r, void* kc,
                             void* vc, int32_t* slot_pos, float* slot_score, hipStream_t st);

}  // namespace kvpop

// decode_step.hip -- one bounded-cache decode step followed by decode
// attention over the updated cache, in one launch.
//
// KVpop summary (arXiv 2607.05061v2), Sec. 3 and App. C.1, E.4: at every
// decoding step the token leaving the window is kept or dropped, the new
// token enters the window, a delayed score is taken, and attention then
// runs over the retained entries only.
//
// gfx950 mapping: when one workgroup per (b, KV head) covers all slots (the
// decode plan needs no slot split), the same workgroup applies the cache
// step to its row and then streams the row for attention, so the step
// costs no launch of its own; otherwise the two kernels run back to back.
#include "cache_step_dev.h"
#include "decode_dev.h"
#include "launch.h"
#include "mlstm_dev.h"

namespace kvpop {
namespace {

template <int D, int GC>
__global__ __launch_bounds__(decdev::kThreads) void decode_step_kernel(
    int n_sink, int window, int budget, int delay, int pos_q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, const float* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, int hidden,
    const float* __restrict__ scores_r, bf16_t* __restrict__ kc, bf16_t* __restrict__ vc,
    int32_t* __restrict__ slot_pos, float* __restrict__ slot_score, const bf16_t* __restrict__ q,
    void* __restrict__ o_out, int o_bf16, float* __restrict__ lse_out, int Hq, int Hkv, int sps,
    float c) {
  static_assert(csdev::kThreads == decdev::kThreads, "one workgroup shape for both phases");
  const int row = blockIdx.x;  // b * Hkv + h
  csdev::cache_step_row<D>(row, n_sink, window, budget, delay, pos_q, k_new, v_new, w1, b1, w2,
                           b2, hidden, scores_r, kc, vc, slot_pos, slot_score, Hkv);
  // The step's writes (moved row, new row, positions, scores) are
  // performed before the barrier (workgroup-scope release), and every wave
  // of the workgroup reads them through the one L1 of its CU, so the
  // attention sees the updated row.  (A device-scope fence would also write
  // back L2 on this multi-XCD part, which nothing here needs.)
  __syncthreads();
  decdev::decode_row<D, GC>(row, 0, q, kc, vc, slot_pos, nullptr, o_out, o_bf16, lse_out, Hq, Hkv,
                            budget, 1, sps, c);
}

// The same step with the delayed mLSTM scorer in front: the scorer takes the
// new token and scores the exiting one into its ring slot, then the cache
// step (no scorer of its own) keeps or drops it, then the attention.  Each
// phase's global writes are ordered before the next phase's reads by a
// workgroup barrier, as above.
template <int D, int GC>
__global__ __launch_bounds__(decdev::kThreads) void decode_step_mlstm_kernel(
    int n_sink, int window, int budget, int pos_q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, MlstmWeights wt, float* __restrict__ state,
    bf16_t* __restrict__ kc, bf16_t* __restrict__ vc, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, const bf16_t* __restrict__ q, void* __restrict__ o_out,
    int o_bf16, float* __restrict__ lse_out, int Hq, int Hkv, int sps, float c) {
  static_assert(mldev::kMlThreads == decdev::kThreads, "one workgroup shape for all phases");
  const int row = blockIdx.x;  // b * Hkv + h
  mldev::mlstm_row<D>(row, Hkv, n_sink, window, budget, pos_q, k_new, v_new, kc, vc, wt, state,
                      slot_score);
  __syncthreads();
  csdev::cache_step_row<D>(row, n_sink, window, budget, 0, pos_q, k_new, v_new, nullptr, nullptr,
                           nullptr, nullptr, 0, nullptr, kc, vc, slot_pos, slot_score, Hkv);
  __syncthreads();
  decdev::decode_row<D, GC>(row, 0, q, kc, vc, slot_pos, nullptr, o_out, o_bf16, lse_out, Hq, Hkv,
                            budget, 1, sps, c);
}

}  // namespace

hipError_t launch_decode_step_mlstm(const AttnShape& s, int n_sink, int window, int pos_q,
                                    const void* k_new, const void* v_new, const MlstmWeights& w,
                                    float* state, void* kc, void* vc, int32_t* slot_pos,
                                    float* slot_score, const void* q, void* o, int o_bf16,
                                    float* lse, float* workspace, hipStream_t st) {
  const DecodePlan p = plan_decode(s);
  if (p.n_split > 1) {
    hipError_t e = launch_mlstm_step(s.B, s.Hkv, s.D, n_sink, window, s.S, pos_q, k_new, v_new,
                                     kc, vc, w, state, slot_score, st);
    if (e != hipSuccess) return e;
    e = launch_cache_step(s.B, s.Hkv, s.D, n_sink, window, s.S, 0, pos_q, k_new, v_new, nullptr,
                          nullptr, nullptr, nullptr, 0, nullptr, kc, vc, slot_pos, slot_score, st);
    if (e != hipSuccess) return e;
    return launch_decode(s, q, kc, vc, slot_pos, o, o_bf16, lse, workspace, st);
  }
  const int G = s.Hq / s.Hkv;
  const float c = s.scale * kLog2e;
  dim3 grid(s.B * s.Hkv), block(decdev::kThreads);
  auto* kn = (const bf16_t*)k_new;
  auto* vn = (const bf16_t*)v_new;
  auto* kk = (bf16_t*)kc;
  auto* vv = (bf16_t*)vc;
  auto* qq = (const bf16_t*)q;
#define KVPOP_MSTEP(DD, GG)                                                                          \
  hipLaunchKernelGGL((decode_step_mlstm_kernel<DD, GG>), grid, block, 0, st, n_sink, window, s.S,   \
                     pos_q, kn, vn, w, state, kk, vv, slot_pos, slot_score, qq, o, o_bf16, lse,      \
                     s.Hq, s.Hkv, p.slots_per_split, c)
  const int gc = G >= 8 ? 8 : G;
  if (s.D == 128) {
    switch (gc) {
      case 1: KVPOP_MSTEP(128, 1); break;
      case 2: KVPOP_MSTEP(128, 2); break;
      case 4: KVPOP_MSTEP(128, 4); break;
      default: KVPOP_MSTEP(128, 8); break;
    }
  } else {
    switch (gc) {
      case 1: KVPOP_MSTEP(64, 1); break;
      case 2: KVPOP_MSTEP(64, 2); break;
      case 4: KVPOP_MSTEP(64, 4); break;
      default: KVPOP_MSTEP(64, 8); break;
    }
  }
#undef KVPOP_MSTEP
  return hipGetLastError();
}

hipError_t launch_decode_step(const AttnShape& s, int n_sink, int window, int delay, int pos_q,
                              const void* k_new, const void* v_new, const float* w1,
                              const float* b1, const float* w2, const float* b2, int hidden,
                              const float* scores_r, void* kc, void* vc, int32_t* slot_pos,
                              float* slot_score, const void* q, void* o, int o_bf16, float* lse,
                              float* workspace, hipStream_t st) {
  const DecodePlan p = plan_decode(s);
  if (p.n_split > 1) {
    hipError_t e = launch_cache_step(s.B, s.Hkv, s.D, n_sink, window, s.S, delay, pos_q, k_new,
                                     v_new, w1, b1, w2, b2, hidden, scores_r, kc, vc, slot_pos,
                                     slot_score, st);
    if (e != hipSuccess) return e;
    return launch_decode(s, q, kc, vc, slot_pos, o, o_bf16, lse, workspace, st);
  }
  const int G = s.Hq / s.Hkv;
  const float c = s.scale * kLog2e;
  dim3 grid(s.B * s.Hkv), block(decdev::kThreads);
  auto* kn = (const bf16_t*)k_new;
  auto* vn = (const bf16_t*)v_new;
  auto* kk = (bf16_t*)kc;
  auto* vv = (bf16_t*)vc;
  auto* qq = (const bf16_t*)q;
#define KVPOP_STEP(DD, GG)                                                                          \
  hipLaunchKernelGGL((decode_step_kernel<DD, GG>), grid, block, 0, st, n_sink, window, s.S, delay, \
                     pos_q, kn, vn, w1, b1, w2, b2, hidden, scores_r, kk, vv, slot_pos, slot_score,  \
                     qq, o, o_bf16, lse, s.Hq, s.Hkv, p.slots_per_split, c)
  const int gc = G >= 8 ? 8 : G;
  if (s.D == 128) {
    switch (gc) {
      case 1: KVPOP_STEP(128, 1); break;
      case 2: KVPOP_STEP(128, 2); break;
      case 4: KVPOP_STEP(128, 4); break;
      default: KVPOP_STEP(128, 8); break;
    }
  } else {
    switch (gc) {
      case 1: KVPOP_STEP(64, 1); break;
      case 2: KVPOP_STEP(64, 2); break;
      case 4: KVPOP_STEP(64, 4); break;
      default: KVPOP_STEP(64, 8); break;
    }
  }
#undef KVPOP_STEP
  return hipGetLastError();
}

}  // namespace kvpop

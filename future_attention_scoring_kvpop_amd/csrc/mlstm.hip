// mlstm.hip -- kernel and launcher of one decoding step of the delayed
// stateful mLSTM scorer (device code and the method's formulas in
// mlstm_dev.h; App. A, E.1, E.3, E.4 of the KVpop summary, arXiv
// 2607.05061v2).
#include "mlstm_dev.h"

namespace kvpop {
namespace {

template <int D>
__global__ __launch_bounds__(mldev::kMlThreads) void mlstm_step_kernel(
    int Hkv, int n_sink, int window, int budget, int pos_q, const bf16_t* __restrict__ k_new,
    const bf16_t* __restrict__ v_new, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    MlstmWeights wt, float* __restrict__ state, float* __restrict__ slot_score) {
  mldev::mlstm_row<D>(blockIdx.x, Hkv, n_sink, window, budget, pos_q, k_new, v_new, kc, vc, wt,
                      state, slot_score);
}

}  // namespace

hipError_t launch_mlstm_step(int B, int Hkv, int D, int n_sink, int window, int budget, int pos_q,
                             const void* k_new, const void* v_new, const void* kc, const void* vc,
                             const MlstmWeights& w, float* state, float* slot_score,
                             hipStream_t st) {
  dim3 grid(B * Hkv), block(mldev::kMlThreads);
  if (D == 128)
    hipLaunchKernelGGL(mlstm_step_kernel<128>, grid, block, 0, st, Hkv, n_sink, window, budget,
                       pos_q, (const bf16_t*)k_new, (const bf16_t*)v_new, (const bf16_t*)kc,
                       (const bf16_t*)vc, w, state, slot_score);
  else
    hipLaunchKernelGGL(mlstm_step_kernel<64>, grid, block, 0, st, Hkv, n_sink, window, budget,
                       pos_q, (const bf16_t*)k_new, (const bf16_t*)v_new, (const bf16_t*)kc,
                       (const bf16_t*)vc, w, state, slot_score);
  return hipGetLastError();
}

}  // namespace kvpop

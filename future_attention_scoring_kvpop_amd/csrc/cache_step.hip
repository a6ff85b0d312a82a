// cache_step.hip -- headwise MLP scorer over many tokens and the bounded-
// cache decode step as its own launch (the device code is in
// cache_step_dev.h).
#include "cache_step_dev.h"
#include "launch.h"

namespace kvpop {
namespace {

using csdev::kThreads;
using csdev::mlp_wave;
using csdev::stage_w1;
using csdev::wave_lds_sync;

// Prefix scorer: one workgroup per (b, h, block of tokens); each wave walks
// its tokens one at a time.
__global__ __launch_bounds__(kThreads) void score_mlp_kernel(
    const bf16_t* __restrict__ keys, const float* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, float* __restrict__ scores,
    int Hkv, int n_tok, int D, int hidden, int tok_per_block, int blocks_per_row) {
  extern __shared__ float smem[];
  float* w1s = smem;                               // hidden * (D+1)
  float* keyb = smem + hidden * (D + 1);           // 4 waves * D
  const int bh = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x % blocks_per_row;
  const int h = bh % Hkv;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  stage_w1(w1s, w1 + (size_t)h * hidden * D, D, hidden);
  __syncthreads();
  const int t_begin = blk * tok_per_block;
  const int t_end = min(n_tok, t_begin + tok_per_block);
  float* kw = keyb + wave * D;
  for (int t = t_begin + wave; t < t_end; t += 4) {
    const bf16_t* kr = keys + ((size_t)bh * n_tok + t) * D;
    for (int cc = lane; cc < D; cc += 64) kw[cc] = __uint_as_float((uint32_t)kr[cc] << 16);
    wave_lds_sync();
    const float sc = mlp_wave(kw, w1s, D, hidden, b1 + (size_t)h * hidden, w2 + (size_t)h * hidden,
                              b2[h], lane);
    if (lane == 0) scores[(size_t)bh * n_tok + t] = sc;
    wave_lds_sync();  // kw is rewritten by the next token of this wave
  }
}

__global__ __launch_bounds__(kThreads) void cache_step_kernel(
    int D, int n_sink, int window, int budget, int delay, int pos_q,
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, int hidden, const float* __restrict__ scores_r,
    bf16_t* __restrict__ kc, bf16_t* __restrict__ vc, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, int Hkv) {
  extern __shared__ float smem[];
  csdev::cache_step_row(blockIdx.x, smem, D, n_sink, window, budget, delay, pos_q, k_new, v_new,
                        w1, b1, w2, b2, hidden, scores_r, kc, vc, slot_pos, slot_score, Hkv);
}

}  // namespace

hipError_t launch_score_mlp(int B, int Hkv, int n_tok, int D, int hidden, const void* keys,
                            const float* w1, const float* b1, const float* w2, const float* b2,
                            float* scores, hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  const int tok_per_block = 256;
  const int bpr = (n_tok + tok_per_block - 1) / tok_per_block;
  const size_t smem = sizeof(float) * ((size_t)hidden * (D + 1) + 4 * D);
  hipLaunchKernelGGL(score_mlp_kernel, dim3(B * Hkv * bpr), dim3(kThreads), smem, st,
                     (const bf16_t*)keys, w1, b1, w2, b2, scores, Hkv, n_tok, D, hidden,
                     tok_per_block, bpr);
  return hipGetLastError();
}

hipError_t launch_cache_step(int B, int Hkv, int D, int n_sink, int window, int budget,
                             int delay, int pos_q, const void* k_new, const void* v_new,
                             const float* w1, const float* b1, const float* w2,
                             const float* b2, int hidden, const float* scores_r, void* kc,
                             void* vc, int32_t* slot_pos, float* slot_score, hipStream_t st) {
  const size_t smem = w1 ? sizeof(float) * ((size_t)hidden * (D + 1) + D) : 0;
  hipLaunchKernelGGL(cache_step_kernel, dim3(B * Hkv), dim3(kThreads), smem, st, D, n_sink,
                     window, budget, delay, pos_q, (const bf16_t*)k_new, (const bf16_t*)v_new, w1,
                     b1, w2, b2, hidden, scores_r, (bf16_t*)kc, (bf16_t*)vc, slot_pos, slot_score,
                     Hkv);
  return hipGetLastError();
}

}  // namespace kvpop

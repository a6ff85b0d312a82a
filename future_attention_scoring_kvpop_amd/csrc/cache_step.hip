// cache_step.hip -- headwise MLP scorer over many tokens and the bounded-
// cache decode step as its own launch (the device code is in
// cache_step_dev.h).
#include "cache_step_dev.h"
#include "launch.h"

namespace kvpop {
namespace {

using csdev::kThreads;

// Tokens whose keys a wave of the prefix scorer has in flight.
constexpr int kScorePrefetch = 4;

// Prefix scorer.  Each wave holds the scorer of its head (lane j: hidden
// unit j) and walks a run of tokens; lane i loads dword i of a key
// kScorePrefetch tokens ahead, and the scores of kScorePrefetch tokens are
// reduced together.  Per token the arithmetic is scorer_term + wave_sum,
// the same code as the in-step scorer.
template <int D>
__global__ __launch_bounds__(kThreads) void score_mlp_kernel(
    const bf16_t* __restrict__ keys, const float* __restrict__ w1, const float* __restrict__ b1,
    const float* __restrict__ w2, const float* __restrict__ b2, float* __restrict__ scores,
    int n_rows, int Hkv, int n_tok, int hidden, int tok_per_wave, int waves_per_row) {
  constexpr int KPF = kScorePrefetch;
  constexpr int NW = D / 2;  // key dwords per token
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * (kThreads / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int bh = gw / waves_per_row;
  if (bh >= n_rows) return;
  const int h = bh % Hkv;
  const int t_begin = (gw % waves_per_row) * tok_per_wave;
  const int last = min(n_tok, t_begin + tok_per_wave) - 1 - t_begin;
  csdev::ScorerLane<D> sl;
  csdev::load_scorer<D>(sl, w1, b1, w2, h, hidden, lane);
  const float b2h = b2[h];
  const uint32_t* kp =
      reinterpret_cast<const uint32_t*>(keys + ((size_t)bh * n_tok + t_begin) * D) + lane % NW;
  float* out = scores + (size_t)bh * n_tok + t_begin;
  uint32_t kq[KPF];
#pragma unroll
  for (int i = 0; i < KPF; ++i) kq[i] = kp[(size_t)min(i, last) * NW];
  for (int t0 = 0; t0 <= last; t0 += KPF) {
    float part[KPF];
#pragma unroll
    for (int i = 0; i < KPF; ++i) {
      const uint32_t cur = kq[i];
      kq[i] = kp[(size_t)min(t0 + KPF + i, last) * NW];
      part[i] = csdev::scorer_term<D>(sl, cur);
    }
#pragma unroll
    for (int i = 0; i < KPF; ++i) part[i] = csdev::wave_sum(part[i]);
    if (lane == 0)
#pragma unroll
      for (int i = 0; i < KPF; ++i)
        if (t0 + i <= last) out[t0 + i] = part[i] + b2h;
  }
}

template <int D>
__global__ __launch_bounds__(kThreads) void cache_step_kernel(
    int n_sink, int window, int budget, int delay, int pos_q,
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, int hidden, const float* __restrict__ scores_r,
    bf16_t* __restrict__ kc, bf16_t* __restrict__ vc, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, int Hkv) {
  csdev::cache_step_row<D>(blockIdx.x, n_sink, window, budget, delay, pos_q, k_new, v_new, w1,
                           b1, w2, b2, hidden, scores_r, kc, vc, slot_pos, slot_score, Hkv);
}

}  // namespace

hipError_t launch_score_mlp(int B, int Hkv, int n_tok, int D, int hidden, const void* keys,
                            const float* w1, const float* b1, const float* w2, const float* b2,
                            float* scores, hipStream_t st) {
  if (n_tok == 0) return hipSuccess;
  // runs of up to 512 tokens per wave; shorter runs when that leaves fewer
  // than about three resident waves per SIMD
  const long total = (long)B * Hkv * n_tok;
  const long want = (long)device_cu_count() * 4 * 3;
  long tpw = (total + want - 1) / want;
  tpw = (tpw + kScorePrefetch - 1) / kScorePrefetch * kScorePrefetch;
  const int tok_per_wave = (int)std::min<long>(512, std::max<long>(4 * kScorePrefetch, tpw));
  const int wpr = (n_tok + tok_per_wave - 1) / tok_per_wave;
  const long waves = (long)B * Hkv * wpr;
  const int wpb = kThreads / 64;
  const dim3 grid((unsigned)((waves + wpb - 1) / wpb));
  if (D == 128)
    hipLaunchKernelGGL(score_mlp_kernel<128>, grid, dim3(kThreads), 0, st, (const bf16_t*)keys, w1,
                       b1, w2, b2, scores, B * Hkv, Hkv, n_tok, hidden, tok_per_wave, wpr);
  else
    hipLaunchKernelGGL(score_mlp_kernel<64>, grid, dim3(kThreads), 0, st, (const bf16_t*)keys, w1,
                       b1, w2, b2, scores, B * Hkv, Hkv, n_tok, hidden, tok_per_wave, wpr);
  return hipGetLastError();
}

hipError_t launch_cache_step(int B, int Hkv, int D, int n_sink, int window, int budget,
                             int delay, int pos_q, const void* k_new, const void* v_new,
                             const float* w1, const float* b1, const float* w2,
                             const float* b2, int hidden, const float* scores_r, void* kc,
                             void* vc, int32_t* slot_pos, float* slot_score, hipStream_t st) {
#define KVPOP_CS_LAUNCH(DD)                                                                      \
  hipLaunchKernelGGL(cache_step_kernel<DD>, dim3(B * Hkv), dim3(kThreads), 0, st, n_sink, window, \
                     budget, delay, pos_q, (const bf16_t*)k_new, (const bf16_t*)v_new, w1, b1,  \
                     w2, b2, hidden, scores_r, (bf16_t*)kc, (bf16_t*)vc, slot_pos, slot_score, \
                     Hkv)
  if (D == 128)
    KVPOP_CS_LAUNCH(128);
  else
    KVPOP_CS_LAUNCH(64);
#undef KVPOP_CS_LAUNCH
  return hipGetLastError();
}

}  // namespace kvpop

// mlstm_dev.h -- device code of one decoding step of the delayed stateful
// mLSTM scorer, shared by its own kernel and the fused decode step.
//
// KVpop summary (arXiv 2607.05061v2): App. A (recurrent linear attention:
// a running key-value summary and normalizer updated by rank-one outer
// products), App. E.1 (headwise input x = [k; v] of the cached token),
// App. E.3 (mLSTM matrix memory C and normalizer n with scalar input and
// forget gates from headwise projections, in the numerically stabilised
// form, Hedgehog features), App. E.4 (at query q the state has taken tokens
// through q and the newly eligible token u = q - w is read out through a
// normalised SiLU transformation with a bias).
//   hedgehog(z) = [softmax(z); softmax(-z)]
//   phi = hedgehog(Wk x_q), val = Wv x_q, ig = wi.x_q + bi, lf = log sigmoid(wf.x_q + bf)
//   m' = max(lf + m, ig);  C' = e^(lf+m-m') C + e^(ig-m') val phi^T;  n' likewise
//   r = hedgehog(Wr x_u);  h = C' r / max(|n'.r|, e^(-m'));  score_u = wo.silu(h) + bo
//
// gfx950 mapping: one 256-thread workgroup per (b, KV head) row.  The
// projections are dot products of length 2D: thread o computes output o
// whole, reading its weight row 16 bytes at a time (the weights of a layer
// stay L2-resident across the batch) and the input from LDS as broadcast
// reads, so no projection needs a cross-lane reduction.  The Hedgehog
// softmaxes take their max and sums from LDS the same way (wave 0 for the
// entering token and the gates, wave 1 for the read-out token).  Each
// thread then owns 16 consecutive entries of one row of C (64 x 64, 16 KB
// per row, read and written once per step), updates them in registers and
// forms its part of C' r, reduced over the 4 threads of the row with two
// lane swaps.
#pragma once

#include "common.h"
#include "launch.h"

namespace kvpop {
namespace mldev {

constexpr int kMlThreads = 256;
constexpr int kP = kMlstmFeat;      // projected features per half
constexpr int kF = 2 * kMlstmFeat;  // Hedgehog features
constexpr int kE = kMlstmVdim;      // value features
static_assert(kE * kF == 16 * kMlThreads, "16 entries of C per thread");

__device__ __forceinline__ float wave_sum64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
// Hedgehog features of the kP values z[0..kP) in LDS, without lane
// shuffles: lane j receives feature j (softmax(z) for j < kP, softmax(-z)
// after); every lane reads all of z (broadcast reads) for the max and min,
// lane j writes its exponential to tmp, and every lane sums its half back.
__device__ __forceinline__ float hedgehog_lds(const float* z, float* tmp, int lane) {
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int j = 0; j < kP; ++j) {
    mx = fmaxf(mx, z[j]);
    mn = fminf(mn, z[j]);
  }
  const int j = lane & (kP - 1);
  const float ex = lane < kP ? expf(z[j] - mx) : expf(mn - z[j]);
  tmp[lane] = ex;
  __builtin_amdgcn_wave_barrier();
  const float* half = tmp + (lane < kP ? 0 : kP);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < kP; ++i) sum += half[i];
  return ex / sum;
}

__device__ __forceinline__ float log_sigmoid(float a) {
  return a >= 0.f ? -log1pf(expf(-a)) : a - log1pf(expf(a));
}

// One step of the scorer for row `row` = b * Hkv + h by the calling
// 256-thread workgroup (every thread must call it).
template <int D>
__device__ __forceinline__ void mlstm_row(
    int row, int Hkv, int n_sink, int window, int budget, int pos_q,
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc, const MlstmWeights& wt,
    float* __restrict__ state, float* __restrict__ slot_score) {
  constexpr int X = 2 * D;           // input length
  constexpr int NOUT = kP + kE + 2;  // projections of the entering token
  __shared__ float xs[X], xu[X];
  __shared__ float proj[NOUT + kP];  // zk, val, ig, fg, zr
  __shared__ float phi[kF], rr[kF], val[kE];
  __shared__ float gate[4];          // fs, is, m', e^(-m')
  __shared__ float hpart[kE];
  __shared__ __attribute__((aligned(16))) float hh_tmp[2][kF];

  const int h = row % Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = budget - n_sink - window;
  const int u = pos_q - window;
  const bool readout = slot_score != nullptr && u >= n_sink;
  const int uslot = readout ? n_sink + kk + u % window : 0;

  // inputs: the entering token and (for the readout) the exiting token's
  // cached rows, which the cache step of this decoding step has not yet
  // overwritten
  for (int c = tid; c < X; c += kMlThreads) {
    const bf16_t* src = c < D ? k_new + (size_t)row * D + c : v_new + (size_t)row * D + (c - D);
    xs[c] = bf16_lo(*src);
    if (readout) {
      const size_t base = ((size_t)row * budget + uslot) * D;
      xu[c] = bf16_lo(c < D ? kc[base + c] : vc[base + (c - D)]);
    }
  }
  __syncthreads();

  // projections: thread o computes output o over the whole input, reading
  // its weight row 16 bytes at a time and the input from LDS (all lanes of
  // a wave read the same 16 bytes: a broadcast), so no output needs a
  // cross-lane reduction
  const int n_out = NOUT + (readout ? kP : 0);
  if (tid < n_out) {
    const int o = tid;
    const float* w;
    const float* x = xs;
    if (o < kP) w = wt.wk + ((size_t)h * kP + o) * X;
    else if (o < kP + kE) w = wt.wv + ((size_t)h * kE + (o - kP)) * X;
    else if (o == kP + kE) w = wt.wi + (size_t)h * X;
    else if (o == kP + kE + 1) w = wt.wf + (size_t)h * X;
    else {
      w = wt.wr + ((size_t)h * kP + (o - NOUT)) * X;
      x = xu;
    }
    float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll 8
    for (int i = 0; i < X; i += 4) {
      const float4 wv = *reinterpret_cast<const float4*>(w + i);
      const float4 xv = *reinterpret_cast<const float4*>(x + i);
      s0 = fmaf(wv.x, xv.x, s0);
      s1 = fmaf(wv.y, xv.y, s1);
      s2 = fmaf(wv.z, xv.z, s2);
      s3 = fmaf(wv.w, xv.w, s3);
    }
    proj[o] = (s0 + s1) + (s2 + s3);
  }
  __syncthreads();

  float* st = state + (size_t)row * kMlstmStateFloats;

  // Hedgehog features: wave 0 those of the entering token (and the gates),
  // wave 1 those of the read-out token
  if (wave == 0) {
    phi[lane] = hedgehog_lds(proj, hh_tmp[0], lane);
    val[lane] = proj[kP + lane];
    if (lane == 0) {
      const float ig = proj[kP + kE] + wt.bi[h];
      const float lf = log_sigmoid(proj[kP + kE + 1] + wt.bf[h]);
      const float m = st[kE * kF + kF];
      const float mn = fmaxf(lf + m, ig);  // m = -inf before the first token
      gate[0] = expf(lf + m - mn);
      gate[1] = expf(ig - mn);
      gate[2] = mn;
      gate[3] = expf(-mn);
    }
  } else if (wave == 1 && readout) {
    rr[lane] = hedgehog_lds(proj + NOUT, hh_tmp[1], lane);
  }
  __syncthreads();

  // state update: thread tid owns C[e][f0 .. f0+15]
  const float fs = gate[0], is = gate[1];
  const int e = tid >> 2, f0 = (tid & 3) * 16;
  float4* cp = reinterpret_cast<float4*>(st + e * kF + f0);
  float acc = 0.f;
  const float ve = is * val[e];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float4 c4 = cp[i];
    c4.x = fmaf(fs, c4.x, ve * phi[f0 + 4 * i + 0]);
    c4.y = fmaf(fs, c4.y, ve * phi[f0 + 4 * i + 1]);
    c4.z = fmaf(fs, c4.z, ve * phi[f0 + 4 * i + 2]);
    c4.w = fmaf(fs, c4.w, ve * phi[f0 + 4 * i + 3]);
    cp[i] = c4;
    if (readout) {
      acc = fmaf(c4.x, rr[f0 + 4 * i + 0], acc);
      acc = fmaf(c4.y, rr[f0 + 4 * i + 1], acc);
      acc = fmaf(c4.z, rr[f0 + 4 * i + 2], acc);
      acc = fmaf(c4.w, rr[f0 + 4 * i + 3], acc);
    }
  }
  float nr = 0.f;
  if (wave == 0) {  // normalizer n' and n'.r
    const float nn = fmaf(fs, st[kE * kF + lane], is * phi[lane]);
    st[kE * kF + lane] = nn;
    nr = wave_sum64(readout ? nn * rr[lane] : 0.f);
    if (lane == 0) st[kE * kF + kF] = gate[2];
  }
  if (!readout) return;
  acc += __shfl_xor(acc, 1);
  acc += __shfl_xor(acc, 2);
  if ((tid & 3) == 0) hpart[e] = acc;
  __shared__ float den_s;
  if (tid == 0) den_s = fmaxf(fabsf(nr), gate[3]);
  __syncthreads();
  if (wave == 0) {
    const float hv = hpart[lane] / den_s;
    const float sl = hv / (1.f + expf(-hv));
    const float sc = wave_sum64(wt.wo[(size_t)h * kE + lane] * sl);
    if (lane == 0) slot_score[(size_t)row * budget + uslot] = sc + wt.bo[h];
  }
}

}  // namespace mldev
}  // namespace kvpop

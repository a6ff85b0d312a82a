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
// projections are dot products of length 2D: one wave per output, lanes
// striding the input so every weight row is read coalesced (the weights of
// a layer stay L2-resident across the batch).  Gates, the stabiliser and
// the Hedgehog softmaxes run on one wave; then each thread owns 16
// consecutive entries of one row of C (64 x 64, 16 KB per row, read and
// written once per step), updates them in registers and forms its part of
// C' r, reduced over the 4 threads of the row with two lane swaps.
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
__device__ __forceinline__ float wave_max64(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Hedgehog features of the kP values z (lane j < kP holds z[j]); lane j of
// the wave receives feature j (softmax(z) for j < kP, softmax(-z) after).
__device__ __forceinline__ float hedgehog_lane(float z, int lane) {
  const bool own = lane < kP;
  const float mx = wave_max64(own ? z : -INFINITY);
  const float mn = -wave_max64(own ? -z : -INFINITY);
  const float ep = own ? expf(z - mx) : 0.f;
  const float en = own ? expf(mn - z) : 0.f;
  const float sp = wave_sum64(ep), sn = wave_sum64(en);
  const float zj = __shfl(z, lane & (kP - 1));
  return lane < kP ? expf(zj - mx) / sp : expf(mn - zj) / sn;
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
  constexpr int XPL = X / 64;        // inputs per lane
  constexpr int NOUT = kP + kE + 2;  // projections of the entering token
  __shared__ float xs[X], xu[X];
  __shared__ float proj[NOUT + kP];  // zk, val, ig, fg, zr
  __shared__ float phi[kF], rr[kF], val[kE];
  __shared__ float gate[4];          // fs, is, m', e^(-m')
  __shared__ float hpart[kE];

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

  // projections: output o is wave (o % 4)'s; lanes stride the input
  const int n_out = NOUT + (readout ? kP : 0);
  for (int o = wave; o < n_out; o += 4) {
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
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < XPL; ++i) s = fmaf(w[lane + 64 * i], x[lane + 64 * i], s);
    s = wave_sum64(s);
    if (lane == 0) proj[o] = s;
  }
  __syncthreads();

  float* st = state + (size_t)row * kMlstmStateFloats;
  if (wave == 0) {
    const float pk = hedgehog_lane(lane < kP ? proj[lane] : 0.f, lane);
    phi[lane] = pk;
    val[lane] = proj[kP + lane];
    if (readout) rr[lane] = hedgehog_lane(lane < kP ? proj[NOUT + lane] : 0.f, lane);
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

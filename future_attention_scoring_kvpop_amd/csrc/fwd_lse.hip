// fwd_lse.hip -- main causal pass emitting per-query log-normalizers.
//
// KVpop summary (arXiv 2607.05061v2), App. D.1 "dense target identity" and
// App. D.4, first step: the main attention pass yields one log-normalizer
// per query, which the transposed pass then reuses.
//   LSE[b][g][d] = log sum_{t <= d} exp(scale * q_d . k_t)
//
// gfx950 mapping
//   * One workgroup (4 waves) owns P = 128/G consecutive query positions of
//     every query head of one KV-head group, so all 128 of its query rows
//     share the same causal key range and every K tile is read once per
//     workgroup for the whole group.
//   * Each wave keeps 32 query rows resident as MFMA B fragments (bf16) and
//     streams 64-key tiles of K from LDS (double buffered, one barrier per
//     tile) as A fragments: v_mfma_f32_32x32x16_bf16 gives S^T[key][query].
//   * Softmax statistics are kept per lane (a lane owns one query column and
//     16 key rows of each 32-key sub-tile), in base 2 with the scale folded
//     into one FMA: p = exp2(s * scale*log2e - m * scale*log2e).  The two
//     half-waves holding the same column merge once at the end.
//   * Workgroups are issued longest-row first and renumbered so that each
//     XCD works through whole KV heads (their K stays in that XCD's L2).
#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

constexpr int kKT = 64;        // keys per LDS tile
constexpr int kThreads = 256;  // 4 waves

template <int D>
__global__ __launch_bounds__(kThreads, 2) void fwd_lse_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, float* __restrict__ lse, int Hq,
    int Hkv, int S, float c, float scale, int n_pb, int n_items) {
  constexpr int NS = D / 16;      // MFMA k-slices per 32x32 product
  constexpr int STRIDE = D + 8;   // LDS row stride in bf16 (16-byte pad)
  constexpr int CPR = D / 8;      // 16-byte chunks per K row
  constexpr int PER_T = kKT * CPR / kThreads;
  __shared__ __attribute__((aligned(16))) bf16_t ks[2][kKT * STRIDE];

  const int G = Hq / Hkv;
  const int P = 128 / G;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int bh = item / n_pb;
  const int pb = n_pb - 1 - (item % n_pb);
  const int b = bh / Hkv, h = bh % Hkv;
  const int p0 = pb * P;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  const int ci = wave * 32 + col;
  const int gl = ci / P;
  const int dpos = p0 + (ci % P);
  const bool valid = dpos < S;
  const int g = h * G + gl;

  bf16x8 bq[NS];
  {
    const bf16_t* qrow = q + (((size_t)b * Hq + g) * S + (valid ? dpos : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) bq[s] = as_bf16x8(valid ? ldg16(qrow + 16 * s) : make_uint4(0, 0, 0, 0));
  }

  const int n_keys = min(S, p0 + P);
  const int n_kt = (n_keys + kKT - 1) / kKT;
  const bf16_t* kbase = k + ((size_t)b * Hkv + h) * (size_t)S * D;

  uint4 pre[PER_T];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / CPR, cc = ch % CPR;
      const int t = kt * kKT + row;
      pre[i] = t < S ? ldg16(kbase + (size_t)t * D + cc * 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / CPR, cc = ch % CPR;
      *reinterpret_cast<uint4*>(&ks[buf][row * STRIDE + cc * 8]) = pre[i];
    }
  };

  float m = -INFINITY, l = 0.f;
  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_kt) load_tile(kt + 1);
    const int t0 = kt * kKT;
    f32x16 acc[2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[sub][r] = 0.f;
      const bf16_t* arow = &ks[buf][(sub * 32 + col) * STRIDE + 8 * half];
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc[sub] = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(arow + 16 * s)), bq[s], acc[sub]);
    }
    if (t0 + kKT - 1 > p0) {  // tile reaches the diagonal (or past S): causal mask
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int t = t0 + sub * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
          if (t > dpos) acc[sub][r] = -INFINITY;
        }
    }
    float mx = m;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[sub][r]);
    if (mx > -INFINITY) {
      const float mc = mx * c;
      float ts = 0.f;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) ts += fast_exp2(fmaf(acc[sub][r], c, -mc));
      l = l * fast_exp2(fmaf(m, c, -mc)) + ts;
      m = mx;
    }
    if (kt + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // merge the two half-waves that share a query column
  const float mo = __shfl_xor(m, 32);
  const float lo = __shfl_xor(l, 32);
  const float M = fmaxf(m, mo);
  float L = 0.f;
  if (M > -INFINITY) {
    const float Mc = M * c;
    L = (m > -INFINITY ? l * fast_exp2(fmaf(m, c, -Mc)) : 0.f) +
        (mo > -INFINITY ? lo * fast_exp2(fmaf(mo, c, -Mc)) : 0.f);
  }
  if (half == 0 && valid) lse[((size_t)b * Hq + g) * S + dpos] = M * scale + logf(L);
}

}  // namespace

hipError_t launch_fwd_lse(const AttnShape& s, const void* q, const void* k, float* lse,
                          hipStream_t st) {
  const int G = s.Hq / s.Hkv;
  const int P = 128 / G;
  const int n_pb = (s.S + P - 1) / P;
  const int n_items = s.B * s.Hkv * n_pb;
  const float c = s.scale * kLog2e;
  dim3 grid(n_items), block(kThreads);
  if (s.D == 128)
    hipLaunchKernelGGL(fwd_lse_kernel<128>, grid, block, 0, st, (const bf16_t*)q, (const bf16_t*)k,
                       lse, s.Hq, s.Hkv, s.S, c, s.scale, n_pb, n_items);
  else
    hipLaunchKernelGGL(fwd_lse_kernel<64>, grid, block, 0, st, (const bf16_t*)q, (const bf16_t*)k,
                       lse, s.Hq, s.Hkv, s.S, c, s.scale, n_pb, n_items);
  return hipGetLastError();
}

}  // namespace kvpop

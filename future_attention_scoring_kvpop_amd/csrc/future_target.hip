// future_target.hip -- transposed future-attention pass and its epilogue.
//
// KVpop summary (arXiv 2607.05061v2), App. D.1-D.2 and D.4: the future-
// attention target of key t is the softmax mass it receives from queries
// d >= t + w, computed by a transposed attention pass (keys act as queries,
// the query's own log-normalizer is subtracted, positions d < t + w are
// masked) without ever forming the S x S map; App. B.1 aggregates the query
// heads of a GQA group, App. B.2 adds count normalisation and a finite
// lookahead.
//   m_t^(g) = sum_{d=t+w}^{end_t} exp2(s_dt * scale*log2e - LSE_d * log2e)
//
// gfx950 mapping
//   * A work item is (b, KV head h, 256-key block, query chunk).  Its four
//     waves each keep 64 keys resident as MFMA A fragments (two interleaved
//     32-key sub-tiles: keys t0+32w.. and t0+128+32w.., so every wave meets
//     the window diagonal at about the same query) and stream the chunk's
//     queries of all G heads of the group through double-buffered LDS as B
//     fragments: v_mfma_f32_32x32x16_bf16 yields S^T[key][query].
//   * Each lane owns one query column and 16 key rows per sub-tile, so the
//     per-key sums accumulate in registers across every query tile and head
//     and are reduced across lanes once per item (through padded LDS).
//   * Tiles whose 32x32 (key, query) square lies fully inside the allowed
//     region take a mask-free path (one FMA, one exp2, one add per pair);
//     fully masked squares are skipped; only the diagonal squares mask.
//   * Items write partial sums per (chunk, key); a second kernel sums the
//     chunks of each key in a fixed order (deterministic), aggregates the
//     group and applies count normalisation.
#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

constexpr int kThreads = 256;
constexpr int kQT = 32;        // queries per LDS tile
constexpr int kRedStride = 65; // padded LDS row for the final lane reduction

template <int D, bool PER_HEAD>
__global__ __launch_bounds__(kThreads, 2) void future_target_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const float* __restrict__ lse,
    float* __restrict__ partial, int Hq, int Hkv, int S, int window, int lookahead, float c,
    int chunk, int n_chunks, int n_kb, int n_items) {
  constexpr int NS = D / 16;
  constexpr int STRIDE = D + 8;
  constexpr int CPR = D / 8;
  constexpr int PER_T = kQT * CPR / kThreads;  // 2 (D=128) or 1 (D=64)
  __shared__ __attribute__((aligned(16))) bf16_t qs[2][kQT * STRIDE];
  __shared__ float ls[2][kQT];
  __shared__ float red[4][32 * kRedStride];

  const int G = Hq / Hkv;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int kb = item % n_kb;
  const int rest = item / n_kb;
  const int cidx = rest % n_chunks;
  const int bh = rest / n_chunks;
  const int b = bh / Hkv, h = bh % Hkv;
  const int t0 = kb * kKeyBlock;
  if (t0 + window >= S) return;
  const int c_first = (t0 + window) / chunk;
  int c_last = n_chunks - 1;
  if (lookahead >= 0) c_last = min(c_last, (t0 + kKeyBlock - 1 + window + lookahead) / chunk);
  if (cidx < c_first || cidx > c_last) return;
  const int d_lo = max(cidx * chunk, t0 + window);
  int d_hi = min((cidx + 1) * chunk, S);
  if (lookahead >= 0) d_hi = min(d_hi, t0 + kKeyBlock + window + lookahead);
  const int dt0 = d_lo & ~(kQT - 1);
  const int n_qt = (d_hi - dt0 + kQT - 1) / kQT;
  const int n_iter = G * n_qt;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 31, half = lane >> 5;
  int ts[2];
  ts[0] = t0 + 32 * wave;
  ts[1] = t0 + 128 + 32 * wave;

  bf16x8 ka[2][NS];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
    const int t = ts[sub] + col;
    const bf16_t* krow = k + (((size_t)b * Hkv + h) * S + (t < S ? t : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) ka[sub][s] = as_bf16x8(t < S ? ldg16(krow + 16 * s) : make_uint4(0, 0, 0, 0));
  }

  float macc[2][16];
#pragma unroll
  for (int sub = 0; sub < 2; ++sub)
#pragma unroll
    for (int r = 0; r < 16; ++r) macc[sub][r] = 0.f;

  uint4 pre[PER_T];
  float pre_l = 0.f;
  auto load_tile = [&](int it) {
    const int gl = it / n_qt;
    const int d0 = dt0 + (it % n_qt) * kQT;
    const size_t head = (size_t)b * Hq + h * G + gl;
    const bf16_t* qb = q + head * S * D;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / CPR, cc = ch % CPR;
      const int d = d0 + row;
      pre[i] = d < S ? ldg16(qb + (size_t)d * D + cc * 8) : make_uint4(0, 0, 0, 0);
    }
    if (tid < kQT) {
      const int d = d0 + tid;
      pre_l = d < S ? lse[head * S + d] * kLog2e : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / CPR, cc = ch % CPR;
      *reinterpret_cast<uint4*>(&qs[buf][row * STRIDE + cc * 8]) = pre[i];
    }
    if (tid < kQT) ls[buf][tid] = pre_l;
  };

  // Reduce each key's per-lane partial sums across the 32 lanes that share
  // its rows and write one float per key of the block.
  auto flush = [&](int gout) {
    float* rw = red[wave];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int r = 0; r < 16; ++r) rw[(sub * 16 + r) * kRedStride + lane] = macc[sub][r];
    __syncthreads();
    const int sub = lane >> 5, row = lane & 31;
    const int hf = (row >> 2) & 1, r = ((row >> 3) << 2) | (row & 3);
    const float* src = rw + (sub * 16 + r) * kRedStride + hf * 32;
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) sum += src[i];
    const int t = ts[sub] + row;
    if (t < S) {
      const size_t base = PER_HEAD ? ((size_t)bh * G + gout) : (size_t)bh;
      partial[(base * n_chunks + cidx) * S + t] = sum;
    }
    __syncthreads();
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int it = 0; it < n_iter; ++it) {
    const int buf = it & 1;
    if (it + 1 < n_iter) load_tile(it + 1);
    const int d0 = dt0 + (it % n_qt) * kQT;
    const float L2 = ls[buf][col];
    const bf16_t* brow = &qs[buf][col * STRIDE + 8 * half];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int tsub = ts[sub];
      const bool skip = tsub >= S || d0 + kQT - 1 < tsub + window ||
                        (lookahead >= 0 && d0 > tsub + 31 + window + lookahead);
      if (skip) continue;
      const bool full = d0 >= tsub + 31 + window && d0 + kQT - 1 < S &&
                        (lookahead < 0 || d0 + kQT - 1 <= tsub + window + lookahead);
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = mfma32(ka[sub][s], as_bf16x8(*reinterpret_cast<const uint4*>(brow + 16 * s)), acc);
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) macc[sub][r] += fast_exp2(fmaf(acc[r], c, -L2));
      } else {
        // d - t - w for r = 0; row r adds 8*(r/4) + r%4 to t
        const int d = d0 + col;
        const int base = d - tsub - 4 * half - window;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 8 * (r >> 2) + (r & 3);
          const int diff = base - off;  // d - (t + w)
          const bool ok = diff >= 0 && d < S && (lookahead < 0 || diff <= lookahead);
          if (ok) macc[sub][r] += fast_exp2(fmaf(acc[r], c, -L2));
        }
      }
    }
    if (it + 1 < n_iter) store_tile(buf ^ 1);
    __syncthreads();
    if (PER_HEAD && (it % n_qt) == n_qt - 1) {
      flush(it / n_qt);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) macc[sub][r] = 0.f;
    }
  }
  if (!PER_HEAD) flush(0);
}

// Sum each key's chunk partials in chunk order, aggregate the group and
// apply count normalisation; writes every key (zeros where no query counts).
__global__ __launch_bounds__(256) void target_merge_kernel(
    const float* __restrict__ partial, float* __restrict__ mass, float* __restrict__ mass_ph,
    int B, int Hq, int Hkv, int S, int window, int lookahead, int chunk, int n_chunks, int agg,
    int count_normalize, int per_head) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)B * Hkv * S) return;
  const int t = (int)(idx % S);
  const int bh = (int)(idx / S);
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  long nt = (long)S - t - window;
  if (nt < 0) nt = 0;
  if (lookahead >= 0 && nt > (long)lookahead + 1) nt = (long)lookahead + 1;
  const int t0 = (t / kKeyBlock) * kKeyBlock;
  const bool any = t0 + window < S;
  int c_first = 0, c_last = -1;
  if (any) {
    c_first = (t0 + window) / chunk;
    c_last = n_chunks - 1;
    if (lookahead >= 0) c_last = min(c_last, (t0 + kKeyBlock - 1 + window + lookahead) / chunk);
  }
  float sum = 0.f, mx = 0.f;
  if (per_head) {
    for (int gl = 0; gl < G; ++gl) {
      float v = 0.f;
      const float* pp = partial + ((size_t)bh * G + gl) * n_chunks * (size_t)S + t;
      for (int cc = c_first; cc <= c_last; ++cc) v += pp[(size_t)cc * S];
      if (mass_ph)
        mass_ph[((size_t)b * Hq + h * G + gl) * S + t] = count_normalize ? (nt > 0 ? v / (float)nt : 0.f) : v;
      sum += v;
      mx = gl == 0 ? v : fmaxf(mx, v);
    }
  } else {
    const float* pp = partial + (size_t)bh * n_chunks * (size_t)S + t;
    for (int cc = c_first; cc <= c_last; ++cc) sum += pp[(size_t)cc * S];
  }
  float out = agg == 0 ? sum : agg == 1 ? sum / (float)G : mx;
  if (count_normalize) out = nt > 0 ? out / (float)nt : 0.f;
  mass[idx] = out;
}

}  // namespace

TargetPlan plan_target(const AttnShape& s, int window) {
  TargetPlan p;
  p.n_kb = (s.S + kKeyBlock - 1) / kKeyBlock;
  auto count_items = [&](int C) {
    const int nc = (s.S + C - 1) / C;
    long items = 0;
    for (int kb = 0; kb < p.n_kb; ++kb) {
      const long lo = (long)kb * kKeyBlock + window;
      if (lo >= s.S) continue;
      items += nc - lo / C;
    }
    return items * s.B * s.Hkv;
  };
  int C = 2048;
  while (C > 256 && count_items(C) < 4096) C >>= 1;
  p.chunk = C;
  p.n_chunks = (s.S + C - 1) / C;
  const int G = s.Hq / s.Hkv;
  p.partial_floats = (size_t)s.B * s.Hkv * G * p.n_chunks * (size_t)s.S;
  return p;
}

hipError_t launch_future_target(const AttnShape& s, const void* q, const void* k,
                                const float* lse, int window, int lookahead, int agg,
                                int count_normalize, float* mass, float* mass_per_qhead,
                                float* workspace, hipStream_t st) {
  const TargetPlan p = plan_target(s, window);
  const bool per_head = agg == 2 || mass_per_qhead != nullptr;
  const int n_items = s.B * s.Hkv * p.n_chunks * p.n_kb;
  const float c = s.scale * kLog2e;
  dim3 grid(n_items), block(kThreads);
  auto* qq = (const bf16_t*)q;
  auto* kk = (const bf16_t*)k;
#define KVPOP_TARGET_LAUNCH(DD, PH)                                                                 \
  hipLaunchKernelGGL((future_target_kernel<DD, PH>), grid, block, 0, st, qq, kk, lse, workspace, \
                     s.Hq, s.Hkv, s.S, window, lookahead, c, p.chunk, p.n_chunks, p.n_kb, n_items)
  if (s.D == 128) {
    if (per_head) KVPOP_TARGET_LAUNCH(128, true); else KVPOP_TARGET_LAUNCH(128, false);
  } else {
    if (per_head) KVPOP_TARGET_LAUNCH(64, true); else KVPOP_TARGET_LAUNCH(64, false);
  }
#undef KVPOP_TARGET_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n = (long)s.B * s.Hkv * s.S;
  hipLaunchKernelGGL(target_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     workspace, mass, mass_per_qhead, s.B, s.Hq, s.Hkv, s.S, window, lookahead,
                     p.chunk, p.n_chunks, agg, count_normalize, per_head ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kvpop

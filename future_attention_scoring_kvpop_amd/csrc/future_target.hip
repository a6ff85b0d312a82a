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
//   * A work item is (b, KV head h, key block, query chunk).  Each wave of
//     the item's workgroup keeps 32 keys resident as MFMA A fragments and
//     streams the chunk's queries of all G heads of the group as B
//     fragments: v_mfma_f32_32x32x16_bf16 yields S^T[key][query].  About 120
//     registers per wave keep four waves per SIMD resident, so the MFMA phase
//     of one wave overlaps the exp2/accumulate phase of the others.
//   * All waves of a workgroup share each query tile (32 queries).  Tiles
//     reach LDS by direct global->LDS DMA into a ring of stages, requested
//     two tiles ahead; each stage is its own LDS object so the compiler
//     never drains in-flight prefetches before a read.  Rows are stored
//     unpadded with their 16-byte chunks XOR-swizzled by row, which keeps the
//     fragment reads bank-conflict free.  A bare s_barrier plus explicit
//     vmcnt/lgkmcnt waits orders the ring.
//   * Workgroups of 8 waves (256 keys) halve the L2 traffic per key-query
//     pair against 4 waves (128 keys); launches with few keys use 4 waves to
//     get more, shorter items.
//   * Each lane owns one query column and 16 key rows, so per-key sums stay
//     in registers across every query tile and head; they are reduced
//     across lanes once per item by a register transpose-reduce.
//   * Tiles whose 32x32 (key, query) square lies fully inside the allowed
//     region take a mask-free path (one FMA, one exp2, one add per pair);
//     fully masked squares are skipped; only the diagonal squares mask.
//   * Items write partial sums per (chunk, key); a second kernel sums the
//     chunks of each key in a fixed order (deterministic), aggregates the
//     group and applies count normalisation.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

// Work split: query chunks shrink from the maximum (powers of two) until the
// launch holds enough items to fill the chip, but not below the minimum.
#ifndef KVPOP_TGT_MAX_CHUNK
#define KVPOP_TGT_MAX_CHUNK 2048
#endif
#ifndef KVPOP_TGT_MIN_CHUNK
#define KVPOP_TGT_MIN_CHUNK 256
#endif
#ifndef KVPOP_TGT_MIN_ITEMS
#define KVPOP_TGT_MIN_ITEMS 4096
#endif
#ifndef KVPOP_TGT_STAGES
#define KVPOP_TGT_STAGES 3
#endif
// B * Hkv * S at or below which the 4-wave (128-key) workgroups are used
#ifndef KVPOP_TGT_SMALL_KEYS
#define KVPOP_TGT_SMALL_KEYS 65536
#endif

constexpr int kQT = 32;                    // queries per LDS tile
constexpr int kStages = KVPOP_TGT_STAGES;  // query tiles in the LDS ring
static_assert(kStages >= 2 && kStages <= 4, "stage count");

// One step of the register transpose-reduce: every lane holds 2M values;
// lanes with bit M set keep the upper half, the others the lower half, each
// adding its partner's copy of the half it keeps.
template <int M>
__device__ __forceinline__ void xreduce_step(float* v, int lane) {
  const bool up = (lane & M) != 0;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    const float a = v[j], b = v[j + M];
    v[j] = (up ? b : a) + __shfl_xor(up ? a : b, M);
  }
}

// Wait until at most n of this wave's DMA instructions are in flight
// (n is wave-uniform: later tiles x this wave's instructions per tile).
__device__ __forceinline__ void wait_inflight(int n) {
  if (n <= 0) wait_vmcnt<0>();
  else if (n == 1) wait_vmcnt<1>();
  else if (n == 2) wait_vmcnt<2>();
  else if (n == 3) wait_vmcnt<3>();
  else if (n == 4) wait_vmcnt<4>();
  else if (n == 5) wait_vmcnt<5>();
  else wait_vmcnt<6>();
}

template <int D, bool PER_HEAD, int WAVES>
__global__ __launch_bounds__(64 * WAVES, 16 / WAVES) void future_target_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const float* __restrict__ lse,
    float* __restrict__ partial, int Hq, int Hkv, int S, int window, int lookahead, float c,
    int chunk, int n_chunks, int n_kb, int n_items) {
  constexpr int KB = 32 * WAVES;            // keys per work item
  constexpr int NS = D / 16;                // MFMA k-slices
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int ROWB = D * 2;               // bytes per query row
  constexpr int TILE = kQT * ROWB;          // bytes per query tile
  constexpr int NQI = TILE / 1024;          // 1 KB DMA instructions per query tile
  constexpr int QPW = NQI >= WAVES ? NQI / WAVES : 1;  // per loading wave
  constexpr int Q_WAVES = NQI >= WAVES ? WAVES : NQI;  // waves that load query rows
  constexpr int ROWS_PER_LOAD = 1024 / ROWB;
  static_assert(NQI % Q_WAVES == 0, "tile split over waves");
  // One LDS object per ring stage: every access below names its stage at
  // compile time, so a DMA into one stage is never mistaken for a write to
  // the stage being read.
  __shared__ __attribute__((aligned(1024))) uint8_t qs0[TILE], qs1[TILE], qs2[kStages > 2 ? TILE : 16],
      qs3[kStages > 3 ? TILE : 16];
  __shared__ __attribute__((aligned(256))) float ls0[64], ls1[64], ls2[64], ls3[64];
  auto qst = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? qs0 : j == 1 ? qs1 : j == 2 ? qs2 : qs3;
  };
  auto lst = [&](auto J) -> float* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? ls0 : j == 1 ? ls1 : j == 2 ? ls2 : ls3;
  };

  const int G = Hq / Hkv;
  const int item = xcd_remap(blockIdx.x, n_items);
  const int kb = item % n_kb;
  const int rest = item / n_kb;
  const int cidx = rest % n_chunks;
  const int bh = rest / n_chunks;
  const int b = bh / Hkv, h = bh % Hkv;
  const int t0 = kb * KB;
  if (t0 + window >= S) return;
  const int c_first = (t0 + window) / chunk;
  int c_last = n_chunks - 1;
  if (lookahead >= 0) c_last = min(c_last, (t0 + KB - 1 + window + lookahead) / chunk);
  if (cidx < c_first || cidx > c_last) return;
  const int d_lo = max(cidx * chunk, t0 + window);
  int d_hi = min((cidx + 1) * chunk, S);
  if (lookahead >= 0) d_hi = min(d_hi, t0 + KB + window + lookahead);
  const int dt0 = d_lo & ~(kQT - 1);
  const int n_qt = (d_hi - dt0 + kQT - 1) / kQT;
  const int n_iter = G * n_qt;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int col = lane & 31, half = lane >> 5;
  const int ts = t0 + 32 * wave;  // this wave's 32 keys
  // this wave's share of each tile's DMA: query rows and/or the normalizers
  const bool loads_q = wave < Q_WAVES;
  const bool loads_l = wave == WAVES - 1;
  const int per_tile = (loads_q ? QPW : 0) + (loads_l ? 1 : 0);

  // DMA of query tile `it` (head-major, then position) into stage J.
  auto issue = [&](auto J, int it) {
    uint8_t* qd = qst(J);
    float* ld = lst(J);
    const int gl = it / n_qt;
    const int d0 = dt0 + (it - gl * n_qt) * kQT;
    const size_t head = (size_t)b * Hq + h * G + gl;
    const bf16_t* qb = q + head * S * D;
    if (loads_q) {
#pragma unroll
      for (int j = 0; j < QPW; ++j) {
        const int I = wave * QPW + j;
        const int row = I * ROWS_PER_LOAD + lane / CPR;
        const int pc = lane % CPR;              // physical chunk written by this lane
        const int lc = pc ^ (row & (CPR - 1));  // logical chunk it holds
        const int d = min(d0 + row, S - 1);
        dma16(qb + (size_t)d * D + lc * 8, qd + I * 1024);
      }
    }
    if (loads_l && lane < kQT) dma4(lse + head * S + min(d0 + lane, S - 1), ld);
  };

  bf16x8 ka[NS];
  {
    const int t = ts + col;
    const bf16_t* krow = k + (((size_t)b * Hkv + h) * S + (t < S ? t : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s) ka[s] = as_bf16x8(t < S ? ldg16(krow + 16 * s) : make_uint4(0, 0, 0, 0));
  }
  float macc[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) macc[r] = 0.f;

  // Sum each key's per-lane partials over the 32 lanes sharing its row and
  // write one float per key of this wave's tile.
  auto flush = [&](int gout) {
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) v[r] = macc[r];
    xreduce_step<8>(v, lane);
    xreduce_step<4>(v, lane);
    xreduce_step<2>(v, lane);
    xreduce_step<1>(v, lane);
    v[0] += __shfl_xor(v[0], 16);  // lane col now holds row register col & 15
    const int r = col & 15;
    const int t = ts + 8 * (r >> 2) + 4 * half + (r & 3);
    if (col < 16 && t < S) {
      const size_t base = PER_HEAD ? ((size_t)bh * G + gout) : (size_t)bh;
      partial[(base * n_chunks + cidx) * S + t] = v[0];
    }
  };

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // prologue: tiles 0 .. kStages-2 into stages 0 .. kStages-2
  if (0 < n_iter) issue(I0{}, 0);
  if (1 < n_iter && kStages > 2) issue(I1{}, 1);
  if (2 < n_iter && kStages > 3) issue(I2{}, 2);

  // One iteration on tile `it`, which lives in stage J; the stage of tile
  // it-1 (J-1 mod kStages) is refilled with tile it+kStages-1.
  auto step = [&](auto J, int it) {
    constexpr int j = decltype(J)::value;
    constexpr int jn = (j + kStages - 1) % kStages;
    wait_inflight(per_tile * min(kStages - 2, n_iter - 1 - it));
    wait_lgkmcnt0();  // this wave's reads of earlier stages have completed
    bare_barrier();   // tile `it` is in LDS for every wave; tile it-1's stage is free
    if (it + kStages - 1 < n_iter) issue(std::integral_constant<int, jn>{}, it + kStages - 1);
    const int gl = it / n_qt;
    const int d0 = dt0 + (it - gl * n_qt) * kQT;
    const bool skip = ts >= S || d0 + kQT - 1 < ts + window ||
                      (lookahead >= 0 && d0 > ts + 31 + window + lookahead);
    if (!skip) {
      const float L2 = lst(J)[col] * kLog2e;
      const uint8_t* tile = qst(J) + col * ROWB;
      const int sw = col & (CPR - 1);
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s)
        acc = mfma32(ka[s], as_bf16x8(*reinterpret_cast<const uint4*>(tile + (((2 * s + half) ^ sw) << 4))), acc);
      const bool full = d0 >= ts + 31 + window && d0 + kQT - 1 < S &&
                        (lookahead < 0 || d0 + kQT - 1 <= ts + window + lookahead);
      if (full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) macc[r] += fast_exp2(fmaf(acc[r], c, -L2));
      } else {
        // d - t - w for row r = base - (8*(r/4) + r%4)
        const int d = d0 + col;
        const int base = d - ts - 4 * half - window;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int diff = base - (8 * (r >> 2) + (r & 3));
          const bool ok = diff >= 0 && d < S && (lookahead < 0 || diff <= lookahead);
          const float p = fast_exp2(fmaf(acc[r], c, -L2));
          macc[r] += ok ? p : 0.f;
        }
      }
    }
    if (PER_HEAD && it - gl * n_qt == n_qt - 1) {
      flush(gl);
#pragma unroll
      for (int r = 0; r < 16; ++r) macc[r] = 0.f;
    }
  };

  for (int it = 0; it < n_iter; it += kStages) {
    step(I0{}, it);
    if (it + 1 < n_iter) step(I1{}, it + 1);
    if (kStages > 2 && it + 2 < n_iter) step(I2{}, it + 2);
    if (kStages > 3 && it + 3 < n_iter) step(I3{}, it + 3);
  }
  if (!PER_HEAD) flush(0);
}

// Sum each key's chunk partials in chunk order, aggregate the group and
// apply count normalisation; writes every key (zeros where no query counts).
__global__ __launch_bounds__(256) void target_merge_kernel(
    const float* __restrict__ partial, float* __restrict__ mass, float* __restrict__ mass_ph,
    int B, int Hq, int Hkv, int S, int window, int lookahead, int key_block, int chunk,
    int n_chunks, int agg, int count_normalize, int per_head) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)B * Hkv * S) return;
  const int t = (int)(idx % S);
  const int bh = (int)(idx / S);
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  long nt = (long)S - t - window;
  if (nt < 0) nt = 0;
  if (lookahead >= 0 && nt > (long)lookahead + 1) nt = (long)lookahead + 1;
  const int t0 = (t / key_block) * key_block;
  const bool any = t0 + window < S;
  int c_first = 0, c_last = -1;
  if (any) {
    c_first = (t0 + window) / chunk;
    c_last = n_chunks - 1;
    if (lookahead >= 0) c_last = min(c_last, (t0 + key_block - 1 + window + lookahead) / chunk);
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
  p.waves = (long)s.B * s.Hkv * s.S <= KVPOP_TGT_SMALL_KEYS ? 4 : 8;
  p.key_block = 32 * p.waves;
  p.n_kb = (s.S + p.key_block - 1) / p.key_block;
  auto count_items = [&](int C) {
    const int nc = (s.S + C - 1) / C;
    long items = 0;
    for (int kb = 0; kb < p.n_kb; ++kb) {
      const long lo = (long)kb * p.key_block + window;
      if (lo >= s.S) continue;
      items += nc - lo / C;
    }
    return items * s.B * s.Hkv;
  };
  int C = KVPOP_TGT_MAX_CHUNK;
  while (C > KVPOP_TGT_MIN_CHUNK && count_items(C) < KVPOP_TGT_MIN_ITEMS) C >>= 1;
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
  dim3 grid(n_items), block(64 * p.waves);
  auto* qq = (const bf16_t*)q;
  auto* kk = (const bf16_t*)k;
#define KVPOP_TARGET_LAUNCH(DD, PH, WW)                                                            \
  hipLaunchKernelGGL((future_target_kernel<DD, PH, WW>), grid, block, 0, st, qq, kk, lse,          \
                     workspace, s.Hq, s.Hkv, s.S, window, lookahead, c, p.chunk, p.n_chunks,     \
                     p.n_kb, n_items)
#define KVPOP_TARGET_WAVES(DD, PH)                  \
  if (p.waves == 4) KVPOP_TARGET_LAUNCH(DD, PH, 4); \
  else KVPOP_TARGET_LAUNCH(DD, PH, 8)
  if (s.D == 128) {
    if (per_head) { KVPOP_TARGET_WAVES(128, true); } else { KVPOP_TARGET_WAVES(128, false); }
  } else {
    if (per_head) { KVPOP_TARGET_WAVES(64, true); } else { KVPOP_TARGET_WAVES(64, false); }
  }
#undef KVPOP_TARGET_WAVES
#undef KVPOP_TARGET_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long n = (long)s.B * s.Hkv * s.S;
  hipLaunchKernelGGL(target_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     workspace, mass, mass_per_qhead, s.B, s.Hq, s.Hkv, s.S, window, lookahead,
                     p.key_block, p.chunk, p.n_chunks, agg, count_normalize, per_head ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kvpop

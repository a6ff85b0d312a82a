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
//   * The work is a list of 32x32 (key, query) squares in the order
//     (b, KV head h), query chunk (about 2 MiB of Q), key block, query head,
//     query tile; a run is the squares of one (chunk, key block).  Launches
//     with few runs give every resident workgroup an equal contiguous share
//     of the list, so the causal triangle leaves no idle tail; launches with
//     many rounds of runs give each workgroup one run, so the workgroups of
//     an XCD stream a chunk's query tiles in step and keep them in L2.
//   * Within a run each wave keeps its keys resident as MFMA A fragments
//     and streams the query tiles of all G heads of the group as B
//     fragments: v_mfma_f32_32x32x16_bf16 yields S^T[key][query].  A key
//     block is 256 keys for D = 128: eight waves of 32 keys (about 115
//     registers, four waves per SIMD) where the list is split evenly, four
//     waves of 64 keys (two MFMA chains per fragment read, 168 registers,
//     three waves per SIMD) where each workgroup takes one run.  The MFMA
//     phase of one wave overlaps the exp2/accumulate phase of the others.
//   * All waves of a workgroup share each stage of two query tiles.  Stages reach LDS by direct buffer->LDS loads into a
//     ring, each wave issuing a fixed share (and its own copy of the tiles'
//     normalizers); each stage is its own LDS object so the compiler never
//     drains in-flight prefetches before a read.  A load's address is the
//     group's buffer range plus a 32-bit offset (a scalar row base plus a
//     per-lane constant); rows past S are masked by L = +inf.  Issuing a
//     stage costs one vector add per load (5-7% off the pass against 64-bit
//     per-lane addresses with clamped rows).  Rows are stored unpadded
//     with their 16-byte chunks XOR-swizzled by row, which keeps the
//     fragment reads bank-conflict free.  A bare s_barrier plus explicit
//     vmcnt/lgkmcnt waits orders the ring; B fragments are read in groups of
//     four before one wait (one for the 64-key waves, which keeps them in
//     168 registers).
//   * Each lane owns one query column and 16 key rows, so per-key sums stay
//     in registers across every query tile and head of a run; they are
//     reduced across lanes once per run by a register transpose-reduce.
//   * Squares fully inside the allowed region take a mask-free path (one
//     FMA, one exp2, one add per pair); fully masked squares are skipped;
//     diagonal squares compare each register's key row with a per-lane
//     threshold; queries past S are masked by L = +inf.  Which of the three
//     a tile takes depends only on its first query position, so each wave
//     derives two position ranges once per run and a tile costs two scalar
//     range tests; the fetch and compute positions advance by additions.
//   * Each run writes one partial sum per key and workgroup, into piece
//     run + wg (even split; runs and workgroups both advance along the list,
//     so no two pairs share a piece) or run (one run per workgroup); the
//     workgroup holding a run's first square records where the run starts.
//     A second kernel sums each key's pieces over chunks and workgroups in a
//     fixed order (deterministic for a given device), aggregates the group
//     and applies count normalisation.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

// Work split: the largest share (squares per workgroup), the smallest share
// worth a workgroup, and the bytes of Q one query chunk should span.
#ifndef KVPOP_TGT_SHARE_CAP
#define KVPOP_TGT_SHARE_CAP 384
#endif
// launches with at least this many rounds of non-empty runs give each
// workgroup one whole run (all workgroups then stream a chunk's query tiles
// in step, which keeps them in L2); smaller ones split the list evenly
#ifndef KVPOP_TGT_ITEM_ROUNDS
#define KVPOP_TGT_ITEM_ROUNDS 8
#endif
#ifndef KVPOP_TGT_MIN_SHARE
#define KVPOP_TGT_MIN_SHARE 16
#endif
#ifndef KVPOP_TGT_CHUNK_BYTES
#define KVPOP_TGT_CHUNK_BYTES (2 << 20)
#endif
#ifndef KVPOP_TGT_STAGES
#define KVPOP_TGT_STAGES 3
#endif
// 32-query tiles per LDS ring stage: each barrier, DMA issue and wait then
// covers this many tiles
#ifndef KVPOP_TGT_TPS
#define KVPOP_TGT_TPS 2
#endif
// B fragments read from LDS per wait (8: all at once; 4: two groups; 2: four)
#ifndef KVPOP_TGT_FRAG_GROUP
#define KVPOP_TGT_FRAG_GROUP 4
#endif
// the two-sub-tile kernel reads one fragment per wait, which keeps it within
// the 168 registers of three waves per SIMD
#ifndef KVPOP_TGT_FRAG_GROUP_KS2
#define KVPOP_TGT_FRAG_GROUP_KS2 1
#endif
// waves per SIMD the kernel is compiled for (sets its register budget:
// 512 / n registers per lane)
#ifndef KVPOP_TGT_WPE
#define KVPOP_TGT_WPE 4
#endif
// D = 128 keeps 256-key blocks in two shapes: eight waves of one 32-key
// sub-tile (launches that split the list evenly), and, with this set, four
// waves of two sub-tiles for launches with one run per workgroup (each
// query fragment read from LDS then feeds two MFMA chains: 2.2% faster on
// a 32k layer and on the skewed 16k batch, 10% slower on the 4k layer's
// even split)
#ifndef KVPOP_TGT_WIDE_ITEMS
#define KVPOP_TGT_WIDE_ITEMS 1
#endif
// waves per SIMD of the two-sub-tile kernel: three for the summed target
// (its keys take 64 registers; 3.91 -> 3.78 ms on a 32k layer against two,
// with one fragment per wait and one register for the query-row DMA
// offsets), two for the per-head one, whose extra state would spill at three
#ifndef KVPOP_TGT_WPE_KS2
#define KVPOP_TGT_WPE_KS2 3
#endif
#ifndef KVPOP_TGT_WPE_KS2_HEAD
#define KVPOP_TGT_WPE_KS2_HEAD 2
#endif
// wave priority raised around a tile's MFMA burst (1; ~2% faster than 0:
// the arbiter then feeds the matrix core first while other waves of the
// SIMD run their exp2 work) or around the exp2 work instead (2; the same)
#ifndef KVPOP_TGT_SETPRIO
#define KVPOP_TGT_SETPRIO 1
#endif
// the two-sub-tile kernel's ring stages and priority mode (two stages and
// no priority change measured about 1% faster each on the 32k layer and the
// skewed 16k batch than the eight-wave kernel's three stages and priority 1)
#ifndef KVPOP_TGT_STAGES_KS2
#define KVPOP_TGT_STAGES_KS2 2
#endif
#ifndef KVPOP_TGT_SETPRIO_KS2
#define KVPOP_TGT_SETPRIO_KS2 0
#endif

constexpr int kQT = 32;                    // queries per LDS tile

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

template <int D, bool PER_HEAD, int WAVES, int KS>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(
    KS == 1 ? KVPOP_TGT_WPE : PER_HEAD ? KVPOP_TGT_WPE_KS2_HEAD : KVPOP_TGT_WPE_KS2,
    KS == 1 ? KVPOP_TGT_WPE : PER_HEAD ? KVPOP_TGT_WPE_KS2_HEAD : KVPOP_TGT_WPE_KS2))) void
future_target_kernel(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                     const float* __restrict__ lse, float* __restrict__ partial,
                     int* __restrict__ run_start, int Hq, int Hkv, int S, int window,
                     int lookahead, float c, TargetGeom geo) {
  constexpr int KB = 32 * WAVES * KS;       // keys per key block
  constexpr int NS = D / 16;                // MFMA k-slices
  constexpr int CPR = D / 8;                // 16-byte chunks per row
  constexpr int ROWB = D * 2;               // bytes per query row
  constexpr int TILE = kQT * ROWB;          // bytes per query tile
  constexpr int TPS = KVPOP_TGT_TPS;        // tiles per stage
  constexpr int kStages = KS == 2 ? KVPOP_TGT_STAGES_KS2 : KVPOP_TGT_STAGES;  // LDS ring stages
  static_assert(kStages >= 2 && kStages <= 4, "stage count");
  constexpr int kPrio = KS == 2 ? KVPOP_TGT_SETPRIO_KS2 : KVPOP_TGT_SETPRIO;
  static_assert(TPS == 1 || TPS == 2, "tiles per stage");
  constexpr int NQI = TILE / 1024;          // 1 KB DMA instructions per query tile
  static_assert((TPS * NQI) % WAVES == 0, "every wave loads the same share of a stage");
  constexpr int QPW = TPS * NQI / WAVES;    // query-row DMAs per wave per stage
  constexpr int PT = QPW + 1;               // DMA instructions per wave per stage (+ normalizers)
  constexpr int ROWS_PER_LOAD = 1024 / ROWB;
  // One LDS object per ring stage: every access below names its stage at
  // compile time, so a DMA into one stage is never mistaken for a write to
  // the stage being read.  Each wave keeps its own copy of a stage's
  // normalizers (64 floats: tile tt in lanes 32 tt .. 32 tt + 31; with one
  // tile per stage lanes 32-63 duplicate lanes 0-31).
  constexpr int STAGE = TPS * TILE;
  __shared__ __attribute__((aligned(1024))) uint8_t qs0[STAGE], qs1[STAGE],
      qs2[kStages > 2 ? STAGE : 16], qs3[kStages > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(256))) float ls0[64 * WAVES], ls1[64 * WAVES],
      ls2[kStages > 2 ? 64 * WAVES : 1], ls3[kStages > 3 ? 64 * WAVES : 1];
  auto qst = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? qs0 : j == 1 ? qs1 : j == 2 ? qs2 : qs3;
  };
  auto lst = [&](auto J) -> float* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? ls0 : j == 1 ? ls1 : j == 2 ? ls2 : ls3;
  };

  const int G = Hq / Hkv;
  const int wg = xcd_remap(blockIdx.x, gridDim.x);  // position of this share in the list
  int x, x_end;
  int bh, ch, kb = 0, off;
  if (geo.item_mode) {
    // one whole run: wg is the dense run index (b, h), chunk, key block
    kb = wg % geo.n_kb;
    ch = (wg / geo.n_kb) % geo.n_chunks;
    bh = wg / (geo.n_kb * geo.n_chunks);
    const int n = n_qtiles(geo, ch, kb);
    if (n == 0) return;
    x = 0;
    x_end = G * n;
    off = 0;
  } else {
  x = wg * geo.share;
  x_end = min(geo.total, x + geo.share);
  if (x >= x_end) return;
  // locate the share's first square: (b, h), chunk, key block, offset in the run
  bh = x / geo.per_bh;
  {
    const int rem = x - bh * geo.per_bh;
    int lo = 0, hi = geo.n_chunks - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (geo.cpre[mid] <= rem) lo = mid;
      else hi = mid - 1;
    }
    ch = lo;
    int r2 = rem - geo.cpre[ch];
    for (;; ++kb) {
      const int n = G * n_qtiles(geo, ch, kb);
      if (r2 < n) break;
      r2 -= n;
    }
    off = r2;
  }
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int col = lane & 31, half = lane >> 5;
  const int frow = col * ROWB;      // this lane's query row in a tile
  const int sw = col & (CPR - 1);   // its swizzle
  // byte offset of this lane's B fragment of k-slice s within a tile:
  // loop-invariant, so each fragment read is one ds_read with the stage
  // and tile base as its immediate offset
  uint32_t foff[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) foff[s2] = frow + (((2 * s2 + half) ^ sw) << 4);
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // byte offset of this lane's 16-byte chunk within its first query-row
  // DMA's tile: wave w issues DMAs w, w + WAVES, ..., whose rows agree with
  // the first one's modulo the swizzle period, so the others add a
  // wave-uniform row offset to this one register
  static_assert((WAVES * ROWS_PER_LOAD) % CPR == 0 && kQT % CPR == 0, "one swizzle phase per wave");
  const int qrow0 = (wave % NQI) * ROWS_PER_LOAD + lane / CPR;
  const uint32_t qoff = (uint32_t)(qrow0 * ROWB + (((lane % CPR) ^ (qrow0 & (CPR - 1))) << 4));
  const uint32_t col4 = (uint32_t)col * 4u;

  for (bool first = true;; first = false) {
  const int nq = n_qtiles(geo, ch, kb);
  const int n_iter = min(G * nq - off, x_end - x);
  const int b = bh / Hkv, h = bh - (bh / Hkv) * Hkv;
  const int t0 = kb * KB;
  const int dt0 = 32 * max(ch * geo.ct, kb * geo.kbt + geo.w_t);  // the run's first query tile
  const int ts = t0 + 32 * KS * wave;  // this wave's first key (32 KS keys)
  const int run = (bh * geo.n_chunks + ch) * geo.n_kb + kb;
  const int run0 = run * (PER_HEAD ? G : 1);
  const size_t head0 = (size_t)b * Hq + (size_t)h * G;  // first query head of the group
  const i32x4 rl = buffer_rsrc(lse + head0 * S, (uint32_t)(G * S) * 4u);
  // the group's query rows: one range for its G heads, a head's rows at
  // offset (head * S + row) * ROWB
  const i32x4 rqg = buffer_rsrc(q + head0 * S * D, (uint32_t)(G * S) * ROWB);
  if (!geo.item_mode && off == 0 && tid == 0) run_start[run] = x;
  if (!first) {
    wait_lgkmcnt0();  // every wave is done reading the previous block's stages
    bare_barrier();
  }

  // Fetch state: the stage to fetch next (fst), and a table of the group
  // rows (head * S + query position) of the tiles of 64 stages, lane l
  // holding stage tb + l's (rows past the group read as zero and are never
  // computed); refilled every 64 stages, so a stage's rows cost one
  // v_readlane each.
  const int ig = off / nq;
  const int iq = off - ig * nq;
  const int d_end = dt0 + kQT * nq;
  int fst = 0, tb = 0;
  int trow[TPS];
  auto fill_rows = [&]() {
#pragma unroll
    for (int tt = 0; tt < TPS; ++tt) {
      const int x = off + TPS * (tb + lane) + tt;  // tile of the run
      const int hx = x / nq;
      trow[tt] = min(hx * S + dt0 + (x - hx * nq) * kQT, G * S);
    }
  };
  fill_rows();
  // Compute state: first query position d0 of the tile being computed and
  // its head (cg); a head's tiles end at d_end.
  int d0 = dt0 + iq * kQT, cg = ig;
  // This wave's tiles by d0 (wave-uniform): a tile has allowed pairs when
  // d0 - skip_lo lies in [0, span] (none when the wave's keys start past S)
  // and needs no mask when d0 - full_lo lies in [0, fspan].
  constexpr int kFar = 1 << 29;
  const uint32_t la = lookahead < 0 ? 0x7fffffffu : (uint32_t)lookahead;
  int skip_lo = ts + window - (kQT - 1), span = lookahead < 0 ? kFar : 32 * KS + 30 + lookahead;
  if (ts >= S) {
    skip_lo = kFar;
    span = 0;
  }
  int full_lo = ts + 32 * KS - 1 + window;
  int fspan = min(S - kQT, lookahead < 0 ? kFar : ts + window + lookahead - (kQT - 1)) - full_lo;
  if (fspan < 0) {
    full_lo = kFar;
    fspan = 0;
  }

  // DMA of the stage's tiles (the next to fetch and the one after) into
  // stage J, then advance past them.  Query-row DMA I fetches tile I / NQI.
  auto issue = [&](auto J) {
    if (fst - tb == 64) {
      tb = fst;
      fill_rows();
    }
    int rows[2];
    rows[0] = __builtin_amdgcn_readlane(trow[0], fst - tb);
    rows[1] = TPS == 2 ? __builtin_amdgcn_readlane(trow[TPS - 1], fst - tb) : rows[0];
    ++fst;
    // each lane fetches one 16-byte chunk of a query row; chunks are
    // XOR-swizzled by row in LDS, so the lane holds logical chunk pc ^ row
    // Buffer loads: a query row DMA is the group's range plus this lane's
    // byte offset (the tile's first row, a scalar, plus the lane's fixed
    // offset); rows past S read the next head's first rows (zero past the
    // last head), which the non-full path masks with L = +inf.  The
    // normalizers of the stage's tiles (lanes 32 h .. 32 h + 31: tile h)
    // come from the group's range the same way.
#pragma unroll
    for (int j = 0; j < QPW; ++j) {
      const int I = wave + WAVES * j;
      const int tt = I / NQI;
      const int drow = (I % NQI - wave % NQI) * ROWS_PER_LOAD;
      bdma16(rqg, (uint32_t)(rows[tt] + drow) * ROWB + qoff, qst(J) + I * 1024);
    }
    {
      const uint32_t l0 = (uint32_t)rows[0] * 4u;
      const uint32_t l1 = TPS == 2 ? (uint32_t)rows[1] * 4u : l0;
      bdma4(rl, (half ? l1 : l0) + col4, lst(J) + wave * 64);
    }
  };

  // key sub-tile j of the wave: keys ts + 32 j .. ts + 32 j + 31
  bf16x8 ka[KS][NS];
#pragma unroll
  for (int j = 0; j < KS; ++j) {
    const int t = ts + 32 * j + col;
    const bf16_t* krow = k + (((size_t)b * Hkv + h) * S + (t < S ? t : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      ka[j][s] = as_bf16x8(t < S ? ldg16(krow + 16 * s) : make_uint4(0, 0, 0, 0));
  }
  float macc[KS][16];
#pragma unroll
  for (int j = 0; j < KS; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) macc[j][r] = 0.f;

  // Sum each key's per-lane partials over the 32 lanes sharing its row and
  // write one float per key of this wave's sub-tiles.
  auto flush = [&](int gout) {
#pragma unroll
    for (int j = 0; j < KS; ++j) {
      float v[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) v[r] = macc[j][r];
      xreduce_step<8>(v, lane);
      xreduce_step<4>(v, lane);
      xreduce_step<2>(v, lane);
      xreduce_step<1>(v, lane);
      v[0] += __shfl_xor(v[0], 16);  // lane col now holds row register col & 15
      const int r = col & 15;
      const int t = ts + 32 * j + 8 * (r >> 2) + 4 * half + (r & 3);
      if (col < 16 && t < S) {
        const int piece = run0 + (PER_HEAD ? gout : 0) + (geo.item_mode ? 0 : wg);
        partial[(size_t)piece * KB + (t - t0)] = v[0];
      }
    }
  };

  // prologue: stages 0 .. kStages-2
  const int n_st = (n_iter + TPS - 1) / TPS;  // stages of this segment
  if (0 < n_st) issue(I0{});
  if (1 < n_st && kStages > 2) issue(I1{});
  if (2 < n_st && kStages > 3) issue(I2{});

  // One step on local stage `si`, which lives in ring slot J; the slot of
  // stage si-1 (J-1 mod kStages) is refilled with stage si+kStages-1.
  // the last stage holds one tile when the segment's count is odd
  const int odd = TPS == 2 ? (n_iter & 1) : 0;
  auto step = [&](auto J, int left) {
    constexpr int j = decltype(J)::value;
    constexpr int jn = (j + kStages - 1) % kStages;
    // left = stages after this one; min(kStages - 2, left) of them are
    // already issued
    if (left >= kStages - 2) wait_vmcnt<PT * (kStages - 2)>();
    else if (kStages == 4 && left == 1) wait_vmcnt<PT>();
    else wait_vmcnt<0>();
    wait_lgkmcnt0();  // this wave's reads of earlier stages have completed
    bare_barrier();   // this stage is in LDS for every wave; the previous one's slot is free
    if (left >= kStages - 1) issue(std::integral_constant<int, jn>{});
#pragma unroll
    for (int tt = 0; tt < TPS; ++tt) {
      if (tt > 0 && left < odd) break;  // a stage holds at least one tile
      const int it = (n_st - 1 - left) * TPS + tt;
      if ((uint32_t)(d0 - skip_lo) <= (uint32_t)span) {
        const uint8_t* tile = qst(J) + tt * TILE;
        float lraw = lst(J)[wave * 64 + (TPS == 2 ? tt * 32 + col : lane)];
        f32x16 acc[KS];
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
        // fragment reads in groups of FG, each group issued before one wait
        // (the next group's reads overlap this group's MFMAs)
        constexpr int FG = KS == 2 ? KVPOP_TGT_FRAG_GROUP_KS2 : KVPOP_TGT_FRAG_GROUP;
        if constexpr (kPrio == 1) __builtin_amdgcn_s_setprio(1);
        if constexpr (kPrio == 2) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int s0 = 0; s0 < NS; s0 += FG) {
          u32x4 bu[FG];
#pragma unroll
          for (int s = 0; s < FG; ++s)
            bu[s] = *reinterpret_cast<const u32x4*>(tile + foff[s0 + s]);
          if constexpr (FG == 8)
            asm volatile("" ::"v"(bu[0]), "v"(bu[1]), "v"(bu[2]), "v"(bu[3]), "v"(bu[4]), "v"(bu[5]),
                         "v"(bu[6]), "v"(bu[7]), "v"(lraw));
          else if constexpr (FG == 4)
            asm volatile("" ::"v"(bu[0]), "v"(bu[1]), "v"(bu[2]), "v"(bu[3]), "v"(lraw));
          else if constexpr (FG == 2)
            asm volatile("" ::"v"(bu[0]), "v"(bu[1]), "v"(lraw));
          else
            asm volatile("" ::"v"(bu[0]), "v"(lraw));
#pragma unroll
          for (int s = 0; s < FG; ++s) {
            bf16x8 bq;
            __builtin_memcpy(&bq, &bu[s], 16);
#pragma unroll
            for (int j = 0; j < KS; ++j) acc[j] = mfma32(ka[j][s0 + s], bq, acc[j]);
          }
        }
        if constexpr (kPrio == 1) __builtin_amdgcn_s_setprio(0);
        if constexpr (kPrio == 2) __builtin_amdgcn_s_setprio(1);
        // Squares inside the allowed region and the sequence need no test.
        // Others first set their disallowed pairs to -inf and their queries
        // past S to L = +inf; then every square takes one FMA, one exp2 and
        // one add per pair (a branch around the masking, no two-way split).
        float nl2 = lraw * -kLog2e;
        if ((uint32_t)(d0 - full_lo) > (uint32_t)fspan) {
          if (d0 + col >= S) nl2 = -__builtin_inff();
          // key row of register r of sub-tile j is ts + 32 j + 4*half +
          // 8*(r/4) + r%4: the pair is allowed when base - 32 j - (8*(r/4) +
          // r%4) lies in [0, la] (la = 2^31 - 1 without a lookahead)
          const int base = d0 + col - ts - window - 4 * half;
#pragma unroll
          for (int j = 0; j < KS; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int diff = base - 32 * j - (8 * (r >> 2) + (r & 3));
              acc[j][r] = (uint32_t)diff <= la ? acc[j][r] : -__builtin_inff();
            }
        }
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) macc[j][r] += fast_exp2(fmaf(acc[j][r], c, nl2));
      }
      if (PER_HEAD && (d0 + kQT == d_end || it == n_iter - 1)) {
        flush(cg);
#pragma unroll
        for (int j = 0; j < KS; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) macc[j][r] = 0.f;
      }
      d0 += kQT;
      if (d0 == d_end) {
        d0 = dt0;
        ++cg;
      }
    }
  };

  for (int left = n_st - 1; left >= 0; left -= kStages) {
    step(I0{}, left);
    if (left >= 1) step(I1{}, left - 1);
    if (kStages > 2 && left >= 2) step(I2{}, left - 2);
    if (kStages > 3 && left >= 3) step(I3{}, left - 3);
  }
  if (!PER_HEAD) flush(0);

  x += n_iter;
  if (x >= x_end) break;
  off = 0;
  do {  // next non-empty run
    if (++kb == geo.n_kb) {
      kb = 0;
      if (++ch == geo.n_chunks) {
        ch = 0;
        ++bh;
      }
    }
  } while (n_qtiles(geo, ch, kb) == 0);
  }
}

// Sum each key's pieces over chunks and workgroups in a fixed order,
// aggregate the group and apply count normalisation; writes every key
// (zeros where no query counts).
__global__ __launch_bounds__(256) void target_merge_kernel(
    const float* __restrict__ partial, const int* __restrict__ run_start,
    float* __restrict__ mass, float* __restrict__ mass_ph, int B, int Hq, int Hkv, int S,
    int window, int lookahead, TargetGeom geo, int agg, int count_normalize, int per_head) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)B * Hkv * S) return;
  const int t = (int)(idx % S);
  const int bh = (int)(idx / S);
  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  const int KB = geo.key_block;
  long nt = (long)S - t - window;
  if (nt < 0) nt = 0;
  if (lookahead >= 0 && nt > (long)lookahead + 1) nt = (long)lookahead + 1;
  const int kb = t / KB;
  const int kk = t - kb * KB;
  // sum of the pieces of run r, whose squares are [lo, lo + n) in the list
  auto run_sum = [&](int r, int lo, int n) {
    if (geo.item_mode) return partial[(size_t)r * KB + kk];  // one piece per run
    float v = 0.f;
    for (int w = lo / geo.share; w <= (lo + n - 1) / geo.share; ++w)
      v += partial[(size_t)(r + w) * KB + kk];
    return v;
  };
  float sum = 0.f, mx = 0.f;
  if (per_head) {
    for (int gl = 0; gl < G; ++gl) {
      float v = 0.f;
      for (int ch = 0; ch < geo.n_chunks; ++ch) {
        const int nq = n_qtiles(geo, ch, kb);
        if (nq == 0) continue;
        const int run = (bh * geo.n_chunks + ch) * geo.n_kb + kb;
        v += run_sum(run * G + gl, geo.item_mode ? 0 : run_start[run] + gl * nq, nq);
      }
      if (mass_ph)
        mass_ph[((size_t)b * Hq + h * G + gl) * S + t] = count_normalize ? (nt > 0 ? v / (float)nt : 0.f) : v;
      sum += v;
      mx = gl == 0 ? v : fmaxf(mx, v);
    }
  } else {
    for (int ch = 0; ch < geo.n_chunks; ++ch) {
      const int nq = n_qtiles(geo, ch, kb);
      if (nq == 0) continue;
      const int run = (bh * geo.n_chunks + ch) * geo.n_kb + kb;
      sum += run_sum(run, geo.item_mode ? 0 : run_start[run], G * nq);
    }
  }
  float out = agg == 0 ? sum : agg == 1 ? sum / (float)G : mx;
  if (count_normalize) out = nt > 0 ? out / (float)nt : 0.f;
  mass[idx] = out;
}

}  // namespace

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

static TargetGeom make_geometry(const AttnShape& s, const TargetPlan& p, int window, int lookahead,
                                int slots) {
  TargetGeom g;
  g.G = s.Hq / s.Hkv;
  g.S = s.S;
  g.window = window;
  g.key_block = p.key_block;
  g.kbt = p.key_block / 32;
  g.n_kb = p.n_kb;
  g.n_chunks = p.n_chunks;
  g.ct = p.chunk / 32;
  g.w_t = (window & ~31) / 32;
  g.s_t = (s.S + 31) / 32;
  g.la_t = lookahead < 0 ? (1 << 30)
                         : (int)(((long long)p.key_block + window + lookahead + 31) / 32);
  // squares per chunk of one (b, h), and of the launch, in 64 bits
  long long cpre[kTgtMaxChunks + 1];
  cpre[0] = 0;
  for (int ch = 0; ch < g.n_chunks; ++ch) {
    long long n = 0;
    for (int kb = 0; kb < g.n_kb; ++kb) n += n_qtiles(g, ch, kb);
    cpre[ch + 1] = cpre[ch] + n * g.G;
  }
  const long long per_bh = cpre[g.n_chunks];
  const long long total = per_bh * s.B * s.Hkv;
  // whole rounds of `slots` workgroups, each share at most the cap
  const long long cap = (long long)slots * KVPOP_TGT_SHARE_CAP;
  const long long rounds = std::max(1LL, (total + cap - 1) / cap);
  g.rounds = (int)rounds;  // the even split's: it bounds the workspace of any launch
  long long share = (total + (long long)slots * rounds - 1) / ((long long)slots * rounds);
  if (share < KVPOP_TGT_MIN_SHARE) share = KVPOP_TGT_MIN_SHARE;
  // one run per workgroup when there are many rounds of runs, or when the
  // list does not fit the 32-bit offsets the even split uses
  long long runs_ne = 0;
  for (int ch = 0; ch < g.n_chunks; ++ch)
    for (int kb = 0; kb < g.n_kb; ++kb) runs_ne += n_qtiles(g, ch, kb) > 0;
  runs_ne *= (long long)s.B * s.Hkv;
  g.item_mode = runs_ne >= (long long)KVPOP_TGT_ITEM_ROUNDS * slots || total >= (1LL << 30) ? 1 : 0;
  if (g.item_mode) {
    g.per_bh = g.total = g.share = 0;
    for (int ch = 0; ch <= kTgtMaxChunks; ++ch) g.cpre[ch] = 0;
    g.n_wg = s.B * s.Hkv * g.n_chunks * g.n_kb;
  } else {
    for (int ch = 0; ch <= kTgtMaxChunks; ++ch) g.cpre[ch] = (int)cpre[std::min(ch, g.n_chunks)];
    g.per_bh = (int)per_bh;
    g.total = (int)total;
    g.share = (int)share;
    g.n_wg = (int)((total + share - 1) / share);
  }
  return g;
}

// The D = 128 shapes: eight waves x one sub-tile, four waves x two.
constexpr int kW128 = 8, kKS128 = 1, kWideW = 4, kWideKS = 2;
static_assert(32 * kW128 * kKS128 == 32 * kWideW * kWideKS, "both shapes share the key block");

// Resident workgroups of the transposed pass on the whole device (all its
// variants for this head dim; the fewest, so a round of shares never
// exceeds what runs at once).
static int target_slots(int D) {
  static std::atomic<int> cached[64][2];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::atomic<int>& slot = cached[dev][D == 128];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  int per_cu = 0;
  auto occ = [&](const void* fn, int waves) {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, 64 * waves, 0) == hipSuccess && nb > 0)
      per_cu = per_cu == 0 ? nb : std::min(per_cu, nb);
  };
  if (D == 128) {
    occ((const void*)future_target_kernel<128, false, kW128, kKS128>, kW128);
    occ((const void*)future_target_kernel<128, true, kW128, kKS128>, kW128);
    if (KVPOP_TGT_WIDE_ITEMS) {
      occ((const void*)future_target_kernel<128, false, kWideW, kWideKS>, kWideW);
      occ((const void*)future_target_kernel<128, true, kWideW, kWideKS>, kWideW);
    }
  } else {
    occ((const void*)future_target_kernel<64, false, 4, 1>, 4);
    occ((const void*)future_target_kernel<64, true, 4, 1>, 4);
  }
  if (per_cu == 0) per_cu = D == 128 ? 2 : 4;  // fallback: four waves per SIMD
  n = device_cu_count() * per_cu;
  slot.store(n, std::memory_order_relaxed);
  return n;
}

TargetPlan plan_target(const AttnShape& s, int window) {
  TargetPlan p;
  // a 32-query tile is D / 16 1 KB loads: one per wave of eight (D = 128)
  // or of four (D = 64); four-wave workgroups of 32 keys per wave at
  // D = 128 (128-key blocks) measured 16% slower on the 4k layer.  The
  // plan's shape is the even split's (the wide shape has the same key
  // block and, at two workgroups per CU, the same slots).
  p.waves = s.D == 64 ? 4 : kW128;
  p.ksub = s.D == 64 ? 1 : kKS128;
  p.key_block = 32 * p.waves * p.ksub;
  p.n_kb = (s.S + p.key_block - 1) / p.key_block;
  const int G = s.Hq / s.Hkv;
  long long C = (long long)KVPOP_TGT_CHUNK_BYTES / ((long long)G * s.D * 2);
  C = std::max(256LL, C & ~31LL);
  const long long min_c = (((long long)s.S + kTgtMaxChunks - 1) / kTgtMaxChunks + 31) & ~31LL;
  C = std::max(C, min_c);
  p.chunk = (int)C;
  p.n_chunks = (int)((s.S + C - 1) / C);
  // the most workgroups any lookahead needs: a launch has at most rounds x
  // slots, and no lookahead gives the most squares and rounds
  const int slots = target_slots(s.D);
  p.max_wg = make_geometry(s, p, window, -1, slots).rounds * slots;
  p.runs = (size_t)s.B * s.Hkv * p.n_chunks * p.n_kb;
  p.partial_floats = (p.runs * G + (size_t)p.max_wg) * p.key_block;
  const size_t part_bytes = (p.partial_floats * sizeof(float) + 255) & ~(size_t)255;
  p.workspace_bytes = part_bytes + p.runs * sizeof(int);
  return p;
}

TargetGeom target_geometry(const AttnShape& s, const TargetPlan& p, int window, int lookahead) {
  return make_geometry(s, p, window, lookahead, target_slots(s.D));
}

hipError_t launch_future_target(const AttnShape& s, const void* q, const void* k,
                                const float* lse, int window, int lookahead, int agg,
                                int count_normalize, float* mass, float* mass_per_qhead,
                                float* workspace, hipStream_t st) {
  const TargetPlan p = plan_target(s, window);
  const TargetGeom geo = target_geometry(s, p, window, lookahead);
  int* run_start = reinterpret_cast<int*>(
      reinterpret_cast<char*>(workspace) + ((p.partial_floats * sizeof(float) + 255) & ~(size_t)255));
  const bool per_head = agg == 2 || mass_per_qhead != nullptr;
  const float c = s.scale * kLog2e;
  auto* qq = (const bf16_t*)q;
  auto* kk = (const bf16_t*)k;
  if (geo.n_wg > 0) {
    const dim3 grid(geo.n_wg);
#define KVPOP_TARGET_LAUNCH(DD, PH, WW, KS)                                                        \
  hipLaunchKernelGGL((future_target_kernel<DD, PH, WW, KS>), grid, dim3(64 * WW), 0, st, qq, kk,   \
                     lse, workspace, run_start, s.Hq, s.Hkv, s.S, window, lookahead, c, geo)
    if (s.D == 128 && KVPOP_TGT_WIDE_ITEMS && geo.item_mode) {
      if (per_head) { KVPOP_TARGET_LAUNCH(128, true, kWideW, kWideKS); }
      else { KVPOP_TARGET_LAUNCH(128, false, kWideW, kWideKS); }
    } else if (s.D == 128) {
      if (per_head) { KVPOP_TARGET_LAUNCH(128, true, kW128, kKS128); }
      else { KVPOP_TARGET_LAUNCH(128, false, kW128, kKS128); }
    } else {
      if (per_head) { KVPOP_TARGET_LAUNCH(64, true, 4, 1); } else { KVPOP_TARGET_LAUNCH(64, false, 4, 1); }
    }
#undef KVPOP_TARGET_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long n = (long)s.B * s.Hkv * s.S;
  hipLaunchKernelGGL(target_merge_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     workspace, run_start, mass, mass_per_qhead, s.B, s.Hq, s.Hkv, s.S, window,
                     lookahead, geo, agg, count_normalize, per_head ? 1 : 0);
  return hipGetLastError();
}

}  // namespace kvpop

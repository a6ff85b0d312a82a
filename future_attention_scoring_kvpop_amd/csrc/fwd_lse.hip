// fwd_lse.hip -- main causal pass emitting per-query log-normalizers.
//
// KVpop summary (arXiv 2607.05061v2), App. D.1 "dense target identity" and
// App. D.4, first step: the main attention pass yields one log-normalizer
// per query, which the transposed pass then reuses.
//   LSE[b][g][d] = log sum_{t <= d} exp(scale * q_d . k_t)
//
// gfx950 mapping
//   * A workgroup (4 waves) owns P = 128/G consecutive query positions of
//     every query head of one KV-head group, so all 128 of its query rows
//     share one causal key range and every K tile is read once per
//     workgroup for the whole group.
//   * Each wave keeps 32 query rows resident as MFMA B fragments and streams
//     64-key tiles of K as A fragments: v_mfma_f32_32x32x16_bf16 gives
//     S^T[key][query].  Dense LSE-only launches of many rounds keep two
//     groups of 32 query rows per wave instead (P = 256/G positions per
//     workgroup), so each K fragment read from LDS feeds two MFMAs.  K tiles reach LDS by direct buffer->LDS loads into a
//     ring of stages (one LDS object per stage, rows XOR-swizzled), requested
//     one tile ahead; the register budget allows four workgroups per CU.
//     A load's address is a 32-bit offset in the KV head's range (the
//     tile's scalar base plus a per-lane constant) and keys past S read as
//     zero, which took 4-5% off the pass against 64-bit per-lane addresses
//     with clamped rows.
//   * Softmax statistics are kept per lane (a lane owns one query column and
//     16 key rows of each 32-key sub-tile), in base 2 with the scale folded
//     into one FMA; the two half-waves of a column merge at the end.  A
//     tile's terms are taken relative to the running maximum as it stands,
//     and the maximum is only found again (and the sums rescaled) when some
//     lane's terms would sum past 2^64 or it has none yet: a score a little
//     past the maximum just gives a term above 1, so the common tile costs
//     one FMA, one exp2 and one add per score and no max.
//   * Causal rows grow with position, so when the launch holds too few row
//     blocks to occupy the chip the key range of long rows is split into
//     pieces of at most kmax keys; each piece writes a partial (max, sum) and
//     a small kernel merges them.
//   * Work items are issued longest first and renumbered so that each XCD
//     works through whole KV heads (their K stays in that XCD's L2).
//   * Sparse normalizer (App. D.3 with the running top-k mask of App. C.1):
//     key t takes part in row d only while t <= d < keep_until[t].
//     - Listed mode (a budget is given): keylist_kernel writes, per row
//       block [p0, p1), the keys still retained at p0: first those retained
//       through p1 - 1 (no test), then those leaving inside the block and
//       the block's own keys, padded to whole tiles with the position S.
//       With the running top-k mask at most budget + P keys qualify
//       (budget - 1 retained before p0, P new), so a block walks about
//       budget + P keys instead of its whole causal row.  K rows are
//       gathered through the list by the same DMA, one tile ahead; each
//       wave keeps its own copy of the tile's list and of the gathered
//       keep_until values, and only tiles past the unconditional keys test
//       each score (t <= d and d < keep_until[t]).  A block whose list
//       would not fit (keep_until not made with that budget) walks its
//       whole causal row through the same code with the list t = 0, 1, ...
//     - Masked mode (no budget): every causal tile is read as in the dense
//       pass and each score is tested against keep_until.
//   * Attention output (App. D.4 first step and App. I: the main pass is the
//     model's attention, dense or over the sparse mask): with V given, the
//     same pass also forms O = softmax(Q K^T) V.  A first kernel stores V
//     transposed (head-dim rows of keys) in the workspace, so each 64-key
//     tile of V^T reaches LDS by the same DMA as K, one stage beside it.
//     K rows are fed to the score MFMA in an order that leaves every lane
//     holding 8 consecutive keys per 16-key slice, which is the B operand of
//     the second MFMA (O^T[dim][query] += V^T[dim][key] P^T[key][query]),
//     so the probabilities go from registers to the matrix core as bf16
//     without an LDS round trip.  The two half-waves of a query column share
//     one running maximum (one lane swap per tile), so their partial sums
//     rescale together.  Rows are never split in this mode.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

#ifndef KVPOP_FWD_STAGES
#define KVPOP_FWD_STAGES 2
#endif
// waves per workgroup: the workgroup's 32 x waves query rows share each K tile
// (8 measured 1% faster on a 32k layer's LSE-only pass and 3% with the
// attention output, but 2-6% slower on the 4k layer)
#ifndef KVPOP_FWD_WAVES
#define KVPOP_FWD_WAVES 4
#endif
#ifndef KVPOP_FWD_MIN_BLOCKS
#define KVPOP_FWD_MIN_BLOCKS (16 / KVPOP_FWD_WAVES)
#endif
// Two query groups of 32 rows per wave (each K fragment read from LDS feeds
// two MFMAs; 187 registers, two workgroups per CU) for dense D = 128
// LSE-only launches of at least this many rounds of resident row blocks
// (1 on, 0 off): 3.94-3.98 -> 3.66 ms on a 32k layer; the masked sparse
// mode measured 1% slower with it and keeps one group
#ifndef KVPOP_FWD_WIDE
#define KVPOP_FWD_WIDE 1
#endif
#ifndef KVPOP_FWD_WIDE_ROUNDS
#define KVPOP_FWD_WIDE_ROUNDS 4
#endif
// Row blocks below which long causal rows are split into pieces (only
// launches that cannot occupy the chip gain from the extra merge).
#ifndef KVPOP_FWD_TARGET_ITEMS
#define KVPOP_FWD_TARGET_ITEMS 256
#endif

constexpr int kKT = 64;        // keys per LDS tile
constexpr int kWaves = KVPOP_FWD_WAVES;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup (G heads x P positions)
constexpr int kStages = KVPOP_FWD_STAGES;
static_assert(kStages >= 2 && kStages <= 4, "stage count");

// Wait until at most n of this wave's DMA instructions are in flight.
__device__ __forceinline__ void wait_inflight(int n) {
  if (n <= 0) wait_vmcnt<0>();
  else if (n <= 4) wait_vmcnt<4>();
  else if (n <= 8) wait_vmcnt<8>();
  else wait_vmcnt<12>();
}

enum { kDense = 0, kMasked = 1, kListed = 2 };

// Key lists of the listed sparse mode: one workgroup per (b, KV head, row
// block).  lists[blk][0, cap) receives the keys t < p0 with keep_until[t]
// >= p1 (in position order), then those with p0 < keep_until[t] < p1 and
// the block's own keys [p0, p1), then the padding S up to a whole tile;
// hdr[blk] = (tiles, first tile holding a conditional key), or (-1, 0)
// when the list does not fit in cap entries (or its conditional part in
// kPartMax).
constexpr int kPartMax = 256;
__global__ __launch_bounds__(256) void keylist_kernel(const int* __restrict__ keep_until,
                                                      int* __restrict__ lists,
                                                      int2* __restrict__ hdr, int S, int n_pb,
                                                      int P, int cap) {
  __shared__ int part[kPartMax];
  __shared__ int wcnt[2][4];
  // a block scans p0 keys: the longest (last) blocks of every row are
  // dispatched first, so no long block is left for the launch's tail
  // (5% off lists + pass on the 4k layer against position order)
  const int n_bh = gridDim.x / n_pb;
  const int bh = blockIdx.x % n_bh;
  const int pb = n_pb - 1 - blockIdx.x / n_bh;
  const int blk = bh * n_pb + pb;
  const int p0 = pb * P, p1 = min(S, p0 + P);
  const int* u = keep_until + (size_t)bh * S;
  int* list = lists + (size_t)blk * cap;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint64_t below = (1ull << lane) - 1;
  int n_full = 0, n_part = 0;  // same value in every thread
  constexpr int kU = 4;        // loads in flight per thread
  for (int base = 0; base < p0; base += 256 * kU) {
    int ut[kU];
#pragma unroll
    for (int x = 0; x < kU; ++x) {
      const int t = base + x * 256 + tid;
      ut[x] = t < p0 ? u[t] : 0;
    }
#pragma unroll
    for (int x = 0; x < kU; ++x) {
      const int t = base + x * 256 + tid;
      const bool full = t < p0 && ut[x] >= p1;
      const bool cond = t < p0 && ut[x] > p0 && ut[x] < p1;
      const uint64_t bf = __ballot(full), bc = __ballot(cond);
      if (lane == 0) {
        wcnt[0][w] = __popcll(bf);
        wcnt[1][w] = __popcll(bc);
      }
      __syncthreads();
      int of = 0, oc = 0, tf = 0, tc = 0;
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int cf = wcnt[0][y], cc = wcnt[1][y];
        if (y < w) {
          of += cf;
          oc += cc;
        }
        tf += cf;
        tc += cc;
      }
      if (full) {
        const int pos = n_full + of + __popcll(bf & below);
        if (pos < cap) list[pos] = t;
      }
      if (cond) {
        const int pos = n_part + oc + __popcll(bc & below);
        if (pos < kPartMax) part[pos] = t;
      }
      n_full += tf;
      n_part += tc;
      __syncthreads();  // wcnt is rewritten next round
    }
  }
  for (int t = p0 + tid; t < p1; t += 256) {
    const int pos = n_part + (t - p0);
    if (pos < kPartMax) part[pos] = t;
  }
  n_part += p1 - p0;
  __syncthreads();
  const int count = n_full + n_part;
  const bool fits = count <= cap && n_part <= kPartMax;
  const int n_t = (count + kKT - 1) / kKT;
  if (fits)
    for (int x = tid; x < n_t * kKT - n_full; x += 256) list[n_full + x] = x < n_part ? part[x] : S;
  if (tid == 0) hdr[blk] = fits ? make_int2(n_t, n_full / kKT) : make_int2(-1, 0);
}

// Workgroups per CU the kernel is built for: the output mode holds a V^T
// stage beside every K stage and 64 more accumulators per lane.
constexpr int kOutBlocks = 8 / kWaves;

// V [B*Hkv][S][D] -> V^T [B*Hkv][D][s_pad] (bf16, zero past S), one
// workgroup per (b, KV head, 64-key tile); rows of V^T are 64-key aligned so
// the output pass can DMA a tile of them like a tile of K.
template <int D>
__global__ __launch_bounds__(256) void transpose_v_kernel(const bf16_t* __restrict__ v,
                                                          bf16_t* __restrict__ vt, int S,
                                                          int s_pad) {
  constexpr int CPR = D / 8;  // 16-byte chunks per V row
  __shared__ uint16_t tile[kKT][D + 2];
  const int n_t = s_pad / kKT;
  const int bh = blockIdx.x / n_t, t0 = (blockIdx.x % n_t) * kKT;
  const bf16_t* src = v + (size_t)bh * S * D;
  for (int i = threadIdx.x; i < kKT * CPR; i += 256) {
    const int r = i / CPR, ch = i % CPR;
    const uint4 x = t0 + r < S ? ldg16(src + (size_t)(t0 + r) * D + ch * 8) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      tile[r][ch * 8 + 2 * j] = (uint16_t)(w[j] & 0xffffu);
      tile[r][ch * 8 + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
  bf16_t* dst = vt + (size_t)bh * D * s_pad + t0;
  for (int i = threadIdx.x; i < D * (kKT / 8); i += 256) {
    const int d = i / (kKT / 8), kc = i % (kKT / 8);
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
      w[j] = (uint32_t)tile[kc * 8 + 2 * j][d] | ((uint32_t)tile[kc * 8 + 2 * j + 1][d] << 16);
    stg16(dst + (size_t)d * s_pad + kc * 8, make_uint4(w[0], w[1], w[2], w[3]));
  }
}

template <int D, int MODE, bool OUT, int QG>
__global__ __launch_bounds__(kThreads, OUT ? kOutBlocks : (QG == 2 ? 2 : KVPOP_FWD_MIN_BLOCKS)) void fwd_lse_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ k, const int* __restrict__ keep_until,
    const int2* __restrict__ hdr, const int* __restrict__ lists, int cap, float* __restrict__ lse,
    float2* __restrict__ part, int B, int Hq, int Hkv, int S, float c, float scale, int n_pb,
    int kmax, int n_pieces, int n_items, int snake_cus, const bf16_t* __restrict__ vt, int s_pad,
    void* __restrict__ o_out, int o_bf16) {
  constexpr bool SPARSE = MODE != kDense;
  static_assert(MODE != kListed || kStages == 2, "the listed mode pairs list slots with stages");
  static_assert(!OUT || (MODE != kListed && kStages == 2), "the output mode: dense or masked, two stages");
  static_assert(QG == 1 || (QG == 2 && !OUT && MODE != kListed), "two query groups: LSE-only, dense or masked");
  constexpr int NS = D / 16;           // MFMA k-slices
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int ROWB = D * 2;          // bytes per K row
  constexpr int TILE = kKT * ROWB;     // bytes per K tile
  constexpr int LPW = TILE / 1024 / (kThreads / 64);  // 1 KB DMA instructions per wave
  constexpr int ROWS_PER_LOAD = 1024 / ROWB;
  static_assert(LPW >= 1, "tile split over waves");
  __shared__ __attribute__((aligned(1024))) uint8_t ks0[TILE], ks1[TILE], ks2[kStages > 2 ? TILE : 16],
      ks3[kStages > 3 ? TILE : 16];
  auto kst = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? ks0 : j == 1 ? ks1 : j == 2 ? ks2 : ks3;
  };
  // sparse mask: each wave's own copy of a stage's 64 keep_until values
  constexpr int US = SPARSE ? kKT * (kThreads / 64) : 1;
  __shared__ __attribute__((aligned(256))) int us0[US], us1[US], us2[kStages > 2 ? US : 1],
      us3[kStages > 3 ? US : 1];
  auto ust = [&](auto J) -> int* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? us0 : j == 1 ? us1 : j == 2 ? us2 : us3;
  };
  // listed mode: each wave's own copy of a tile's 64 list entries, in the
  // slot of the stage that tile is loaded into
  constexpr int LS = MODE == kListed ? kKT * (kThreads / 64) : 1;
  __shared__ __attribute__((aligned(256))) int lt0[LS], lt1[LS];
  auto lst = [&](auto J) -> int* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? lt0 : lt1;
  };
  // output mode: each stage's 64-key tile of V^T (D rows of 128 bytes, the
  // 16-byte chunks of row d XOR-swizzled by d & 7)
  __shared__ __attribute__((aligned(1024))) uint8_t vs0[OUT ? TILE : 16], vs1[OUT ? TILE : 16];
  auto vst = [&](auto J) -> uint8_t* {
    constexpr int j = decltype(J)::value;
    return j == 0 ? vs0 : vs1;
  };
  constexpr int VPW = OUT ? D * kKT * 2 / 1024 / (kThreads / 64) : 0;  // V^T DMAs per wave
  // DMAs per wave per stage
  constexpr int DPS = LPW + (SPARSE ? 1 : 0) + (MODE == kListed ? 1 : 0) + VPW;

  const int G = Hq / Hkv;
  const int P = kRows * QG / G;
  // Blocks go round robin over the 8 XCDs and, within an XCD, over its CUs.
  // Each XCD takes a contiguous range of items (longest first).  When the
  // whole launch is resident at once (snake_cus = CUs per XCD, else 0), the
  // range is dealt to the CUs in alternating direction per round, so every
  // CU gets a long and a short block in turn and the same total work.
  int item;
  {
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int q8 = n_items >> 3, r8 = n_items & 7;
    const int xstart = x * q8 + (x < r8 ? x : r8), xcount = q8 + (x < r8 ? 1 : 0);
    int jj = j;
    if (snake_cus > 0) {
      const int rnd = j / snake_cus, cu = j - rnd * snake_cus;
      if (rnd & 1) jj = rnd * snake_cus + (snake_cus - 1 - cu);
      if (jj >= xcount) jj = j;  // a partial last round keeps its order
    }
    item = xstart + jj;
  }
  const int bh = item / (n_pb * n_pieces);
  const int rest = item - bh * (n_pb * n_pieces);
  const int pb = n_pb - 1 - rest / n_pieces;  // longest rows first
  const int piece = rest % n_pieces;
  const int b = bh / Hkv, h = bh % Hkv;
  const int p0 = pb * P;
  const int n_keys = min(S, p0 + P);
  const int k_begin = piece * kmax;
  if (k_begin >= n_keys) return;  // this row block needs fewer pieces
  const int k_end = min(n_keys, k_begin + kmax);
  const int kt0 = k_begin / kKT;
  int n_kt = (k_end - k_begin + kKT - 1) / kKT;
  // listed mode: tiles of the block's list, first tile with a test, and
  // whether the list is the identity (a block whose list did not fit)
  int ft = 0;
  bool ident = true;
  const int* blist = nullptr;
  if constexpr (MODE == kListed) {
    const int blk = bh * n_pb + pb;
    const int2 hh = hdr[blk];
    if (hh.x >= 0) {
      n_kt = hh.x;
      ft = hh.y;
      ident = false;
      blist = lists + (size_t)blk * cap;
    }
  }

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31, half = lane >> 5;
  // query group qg of the wave: 32 query rows (a lane's column is one of
  // them), row wave * 32 * QG + 32 qg + col of the block's G x P rows
  int dposq[QG], gq[QG];
  bool validq[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int ci = (wave * QG + qg) * 32 + col;
    dposq[qg] = p0 + (ci % P);
    validq[qg] = dposq[qg] < S;
    gq[qg] = h * G + ci / P;
  }
  const int dpos = dposq[0], g = gq[0];
  const bool valid = validq[0];

  const bf16_t* kbase = k + ((size_t)b * Hkv + h) * (size_t)S * D;
  const bf16_t* vtbase = OUT ? vt + ((size_t)b * Hkv + h) * (size_t)D * s_pad : nullptr;
  const int* kuntil = SPARSE ? keep_until + ((size_t)b * Hkv + h) * (size_t)S : nullptr;
  // Tiles arrive by buffer->LDS loads: the (b, KV head)'s K, keep_until and
  // V^T are buffer ranges, a load's address is a 32-bit offset (the tile's
  // scalar base plus this lane's fixed offset), and keys past S read as
  // zero (their scores are masked in any case).
  const i32x4 rk = buffer_rsrc(kbase, (uint32_t)S * ROWB);
  const i32x4 ru = buffer_rsrc(kuntil, SPARSE ? (uint32_t)S * 4u : 0u);
  const i32x4 rv = buffer_rsrc(vtbase, OUT ? (uint32_t)(D * s_pad) * 2u : 0u);
  uint32_t koff[LPW];
#pragma unroll
  for (int j = 0; j < LPW; ++j) {
    const int I = wave * LPW + j;
    const int row = I * ROWS_PER_LOAD + lane / CPR;
    koff[j] = (uint32_t)(row * ROWB + (((lane % CPR) ^ (row & (CPR - 1))) << 4));
  }
  uint32_t voff_dma[OUT ? VPW : 1];
  if constexpr (OUT) {
#pragma unroll
    for (int j = 0; j < VPW; ++j) {
      const int row = (wave * VPW + j) * 8 + (lane >> 3);  // V^T rows 8 I .. 8 I + 7
      voff_dma[j] = (uint32_t)(row * s_pad * 2 + (((lane & 7) ^ (row & 7)) << 4));
    }
  }
  auto issue = [&](auto J, int kt) {
    uint8_t* dst = kst(J);
#pragma unroll
    for (int j = 0; j < LPW; ++j)
      bdma16(rk, (uint32_t)(kt * kKT * ROWB) + koff[j], dst + (wave * LPW + j) * 1024);
    if constexpr (SPARSE) bdma4(ru, (uint32_t)(kt * kKT + lane) * 4u, ust(J) + wave * 64);
    if constexpr (OUT) {
      uint8_t* vdst = vst(J);
#pragma unroll
      for (int j = 0; j < VPW; ++j)
        bdma16(rv, (uint32_t)(kt * kKT * 2) + voff_dma[j], vdst + (wave * VPW + j) * 1024);
    }
  };
  // listed mode: K rows and keep_until values of the tile whose list is in
  // slot J, gathered into stage J (list padding S reads as zero)
  auto issue_listed = [&](auto J) {
    uint8_t* dst = kst(J);
    const int* lw = lst(J) + wave * 64;
#pragma unroll
    for (int j = 0; j < LPW; ++j) {
      const int I = wave * LPW + j;
      const int row = I * ROWS_PER_LOAD + lane / CPR;
      bdma16(rk, (uint32_t)lw[row] * ROWB + (koff[j] - (uint32_t)(row * ROWB)), dst + I * 1024);
    }
    bdma4(ru, (uint32_t)lw[lane] * 4u, ust(J) + wave * 64);
  };
  // listed mode: list entries of tile i into slot J
  auto fill_list = [&](auto J, int i) {
    if (ident) {
      lst(J)[wave * 64 + lane] = i * kKT + lane;
    } else {
      wait_lgkmcnt0();  // this wave's reads of the slot are done before the DMA refills it
      dma4(blist + i * kKT + lane, lst(J) + wave * 64);
    }
  };

  bf16x8 bq[QG][NS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const bf16_t* qrow =
        q + (((size_t)b * Hq + gq[qg]) * S + (validq[qg] ? dposq[qg] : 0)) * D + 8 * half;
#pragma unroll
    for (int s = 0; s < NS; ++s)
      bq[qg][s] = as_bf16x8(validq[qg] ? ldg16(qrow + 16 * s) : make_uint4(0, 0, 0, 0));
  }

  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if constexpr (MODE == kListed) {
    fill_list(I0{}, 0);
    if (1 < n_kt) fill_list(I1{}, 1);
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    issue_listed(I0{});
  } else {
    if (0 < n_kt) issue(I0{}, kt0);
    if (1 < n_kt && kStages > 2) issue(I1{}, kt0 + 1);
    if (2 < n_kt && kStages > 3) issue(I2{}, kt0 + 2);
  }

  float mq[QG], lq[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    mq[qg] = -INFINITY;
    lq[qg] = 0.f;
  }
  float& m = mq[0];  // the output mode's (one query group)
  float& l = lq[0];
  // A-fragment row of this lane within a 32-key sub-tile.  The output mode
  // swaps bits 2 and 3 of the row, so that result register r of half h holds
  // key 16 (r / 8) + 8 h + r % 8 (eight consecutive keys per 16-key slice,
  // the B operand layout of the P.V product) instead of 8 (r / 4) + 4 h + r % 4.
  const int krow = OUT ? ((col & 19) | ((col & 4) << 1) | ((col & 8) >> 1)) : col;
  const int sw = krow & (CPR - 1);
  // byte offset of this lane's A fragment of k-slice s within a 32-key
  // sub-tile: loop-invariant, so each read is one ds_read whose immediate
  // offset holds the stage and sub-tile base
  uint32_t foff[NS];
#pragma unroll
  for (int s2 = 0; s2 < NS; ++s2) foff[s2] = krow * ROWB + (((2 * s2 + half) ^ sw) << 4);
  // key offset (within the 64-key tile) of result registers 4 r4 .. 4 r4 + 3
  // of sub-tile sub: four consecutive keys either way
  auto kb4 = [&](int sub, int r4) {
    return OUT ? 32 * sub + 16 * (r4 >> 1) + 8 * half + 4 * (r4 & 1) : 32 * sub + 8 * r4 + 4 * half;
  };
  // output mode: O^T accumulators (dims 32 db + 8 (r/4) + 4 h + r%4 of this
  // lane's query column) and the byte offsets of the V^T A fragments: rows
  // 32 db + col, keys 32 sub + 16 j + 8 h .. + 7 (chunk 4 sub + 2 j + h)
  constexpr int NDB = OUT ? D / 32 : 1;
  f32x16 oacc[NDB];
  uint32_t voff[2][2];
  if constexpr (OUT) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int j = 0; j < 2; ++j) voff[sub][j] = col * 128 + (((4 * sub + 2 * j + half) ^ (col & 7)) << 4);
  }
  auto step = [&](auto J, int i) {
    constexpr int j = decltype(J)::value;
    constexpr int jn = (j + kStages - 1) % kStages;
    wait_inflight(DPS * min(kStages - 2, n_kt - 1 - i));
    wait_lgkmcnt0();
    bare_barrier();  // tile i is in LDS for every wave; tile i-1's stage is free
    if (i + kStages - 1 < n_kt) {
      if constexpr (MODE == kListed) issue_listed(std::integral_constant<int, jn>{});
      else issue(std::integral_constant<int, jn>{}, kt0 + i + kStages - 1);
    }
    const int t0 = (kt0 + i) * kKT;
    const uint8_t* tile = kst(J);
    // each K fragment read from LDS feeds the MFMAs of every query group
    f32x16 accq[QG][2];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int r = 0; r < 16; ++r) accq[qg][sub][r] = 0.f;
      const uint8_t* sbase = tile + sub * 32 * ROWB;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>(sbase + foff[s]));
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) accq[qg][sub] = mfma32(a, bq[qg][s], accq[qg][sub]);
      }
    }
    f32x16(&acc)[2] = accq[0];  // the listed and output modes' (one query group)
    if constexpr (MODE == kListed) {
      // key of register r: entry 32 sub + 8 (r/4) + 4 half + r%4 of the
      // tile's list; tiles before ft hold only keys retained for the block
      if (ident || i >= ft) {
        const int* tl = lst(J) + wave * 64;
        const int* ut = ust(J) + wave * 64;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int4 tv = *reinterpret_cast<const int4*>(tl + sub * 32 + 8 * r4 + 4 * half);
            const int4 uv = *reinterpret_cast<const int4*>(ut + sub * 32 + 8 * r4 + 4 * half);
            acc[sub][4 * r4 + 0] = ((tv.x > dpos) | (dpos >= uv.x)) ? -INFINITY : acc[sub][4 * r4 + 0];
            acc[sub][4 * r4 + 1] = ((tv.y > dpos) | (dpos >= uv.y)) ? -INFINITY : acc[sub][4 * r4 + 1];
            acc[sub][4 * r4 + 2] = ((tv.z > dpos) | (dpos >= uv.z)) ? -INFINITY : acc[sub][4 * r4 + 2];
            acc[sub][4 * r4 + 3] = ((tv.w > dpos) | (dpos >= uv.w)) ? -INFINITY : acc[sub][4 * r4 + 3];
          }
      }
      // slot J is free again: the list of tile i + 2 goes there
      if (i + 2 < n_kt) fill_list(J, i + 2);
    } else if constexpr (SPARSE) {
      // key row of register r: t0 + 32 sub + 8 (r/4) + 4 half + r%4; its
      // keep_until values are four runs of four consecutive ints.  Below
      // the diagonal (and inside the piece) only keep_until can mask.
      const int* ut = ust(J) + wave * 64;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
      f32x16(&acc)[2] = accq[qg];
      const int dpos = dposq[qg];
      if (t0 + kKT - 1 > p0 || t0 + kKT > k_end) {  // diagonal, past S or past the piece
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int4 u = *reinterpret_cast<const int4*>(ut + kb4(sub, r4));
            const int uu[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int t = t0 + kb4(sub, r4) + e;
              acc[sub][4 * r4 + e] =
                  ((t > dpos) | (t >= k_end) | (dpos >= uu[e])) ? -INFINITY : acc[sub][4 * r4 + e];
            }
          }
      } else {
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int4 u = *reinterpret_cast<const int4*>(ut + kb4(sub, r4));
            acc[sub][4 * r4 + 0] = dpos >= u.x ? -INFINITY : acc[sub][4 * r4 + 0];
            acc[sub][4 * r4 + 1] = dpos >= u.y ? -INFINITY : acc[sub][4 * r4 + 1];
            acc[sub][4 * r4 + 2] = dpos >= u.z ? -INFINITY : acc[sub][4 * r4 + 2];
            acc[sub][4 * r4 + 3] = dpos >= u.w ? -INFINITY : acc[sub][4 * r4 + 3];
          }
      }
      }
    } else if (t0 + kKT - 1 > p0 || t0 + kKT > k_end) {  // diagonal, past S or past the piece
#pragma unroll
      for (int qg = 0; qg < QG; ++qg)
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = t0 + kb4(sub, r >> 2) + (r & 3);
            accq[qg][sub][r] = ((t > dposq[qg]) | (t >= k_end)) ? -INFINITY : accq[qg][sub][r];
          }
    }
    if constexpr (OUT) {
      // Terms relative to the running maximum m (one per query column,
      // shared by its two half-waves).  The maximum and the rescaling of the
      // sums are only taken again when a tile's terms would not stay small
      // (above 2^64 in some lane, or m not yet set: the sum is then inf or
      // NaN; query columns past S do not count); otherwise a term above 1
      // (a score past m) is kept as it is.
      float mc = m * c;
      float ts = 0.f;
      bf16x8 pb[2][2];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(fmaf(acc[sub][r], c, -mc));
          ts += p;
          pb[sub][r >> 3][r & 7] = (__bf16)p;
        }
      if (!__all(ts <= 0x1p64f || !valid)) {
        float mx = -INFINITY;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, acc[sub][r]);
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mn = fmaxf(m, mx);
        mc = mn > -INFINITY ? mn * c : 0.f;              // masked scores still give 0
        const float alpha = fast_exp2(fmaf(m, c, -mc));  // 0 while nothing was kept
        ts = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = fast_exp2(fmaf(acc[sub][r], c, -mc));
            ts += p;
            pb[sub][r >> 3][r & 7] = (__bf16)p;
          }
        l *= alpha;
        m = mn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      }
      l += ts;
      const uint8_t* vtile = vst(J);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int db = 0; db < NDB; ++db)
            oacc[db] = mfma32(as_bf16x8(*reinterpret_cast<const uint4*>(vtile + db * 32 * 128 +
                                                                         voff[sub][j])),
                              pb[sub][j], oacc[db]);
    } else {
      // terms relative to the running maximum m; the maximum is only taken
      // again when the tile's terms would not stay small (as above; query
      // columns past S never ask for it)
      float ts[QG];
      bool small = true;
#pragma unroll
      for (int qg = 0; qg < QG; ++qg) {
        const float mc = mq[qg] * c;
        ts[qg] = 0.f;
#pragma unroll
        for (int sub = 0; sub < 2; ++sub)
#pragma unroll
          for (int r = 0; r < 16; ++r) ts[qg] += fast_exp2(fmaf(accq[qg][sub][r], c, -mc));
        small = small && (ts[qg] <= 0x1p64f || !validq[qg]);
      }
      if (__all(small)) {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) lq[qg] += ts[qg];
      } else {
#pragma unroll
        for (int qg = 0; qg < QG; ++qg) {
          float mx = mq[qg];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, accq[qg][sub][r]);
          if (mx > -INFINITY) {
            const float mc = mx * c;
            float t = 0.f;
#pragma unroll
            for (int sub = 0; sub < 2; ++sub)
#pragma unroll
              for (int r = 0; r < 16; ++r) t += fast_exp2(fmaf(accq[qg][sub][r], c, -mc));
            lq[qg] = lq[qg] * fast_exp2(fmaf(mq[qg], c, -mc)) + t;
            mq[qg] = mx;
          }
        }
      }
    }
  };
  for (int i = 0; i < n_kt; i += kStages) {
    step(I0{}, i);
    if (i + 1 < n_kt) step(I1{}, i + 1);
    if (kStages > 2 && i + 2 < n_kt) step(I2{}, i + 2);
    if (kStages > 3 && i + 3 < n_kt) step(I3{}, i + 3);
  }

  if constexpr (OUT) {
    // both half-waves share m: their sums add; O = oacc / sum
    const float lt = l + __shfl_xor(l, 32);
    if (valid) {
      const size_t row = ((size_t)b * Hq + g) * S + dpos;
      if (half == 0) lse[row] = lt > 0.f ? m * scale + logf(lt) : -INFINITY;
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const int dim = 32 * db + 8 * r4 + 4 * half;
          const float o0 = oacc[db][4 * r4] * inv, o1 = oacc[db][4 * r4 + 1] * inv;
          const float o2 = oacc[db][4 * r4 + 2] * inv, o3 = oacc[db][4 * r4 + 3] * inv;
          if (o_bf16) {
            uint2 w;
            w.x = (uint32_t)f32_to_bf16_rne(o0) | ((uint32_t)f32_to_bf16_rne(o1) << 16);
            w.y = (uint32_t)f32_to_bf16_rne(o2) | ((uint32_t)f32_to_bf16_rne(o3) << 16);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(o_out) + row * D + dim) = w;
          } else {
            *reinterpret_cast<float4*>(reinterpret_cast<float*>(o_out) + row * D + dim) =
                make_float4(o0, o1, o2, o3);
          }
        }
    }
    return;
  }
  // merge the two half-waves that share a query column
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const float mm = mq[qg], ll = lq[qg];
    const float mo = __shfl_xor(mm, 32);
    const float lo = __shfl_xor(ll, 32);
    const float M = fmaxf(mm, mo);
    float L = 0.f;
    if (M > -INFINITY) {
      const float Mc = M * c;
      L = (mm > -INFINITY ? ll * fast_exp2(fmaf(mm, c, -Mc)) : 0.f) +
          (mo > -INFINITY ? lo * fast_exp2(fmaf(mo, c, -Mc)) : 0.f);
    }
    if (half == 0 && validq[qg]) {
      const size_t row = ((size_t)b * Hq + gq[qg]) * S + dposq[qg];
      if (n_pieces == 1) lse[row] = M * scale + logf(L);
      else part[(size_t)piece * B * Hq * S + row] = make_float2(M, L);
    }
  }
}

// Combine the pieces of each row: LSE = scale*M + ln(sum_j L_j 2^((M_j - M) c)).
__global__ __launch_bounds__(256) void fwd_lse_merge_kernel(const float2* __restrict__ part,
                                                            float* __restrict__ lse, int B, int Hq,
                                                            int S, float c, float scale, int P,
                                                            int kmax) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long rows = (long)B * Hq * S;
  if (idx >= rows) return;
  const int d = (int)(idx % S);
  const int n_keys = min(S, (d / P + 1) * P);
  const int n = (n_keys + kmax - 1) / kmax;
  float M = -INFINITY;
  for (int j = 0; j < n; ++j) M = fmaxf(M, part[(size_t)j * rows + idx].x);
  float L = 0.f;
  for (int j = 0; j < n; ++j) {
    const float2 v = part[(size_t)j * rows + idx];
    if (v.x > -INFINITY) L += v.y * fast_exp2((v.x - M) * c);
  }
  lse[idx] = M * scale + logf(L);
}

}  // namespace

// qg query groups of 32 rows per wave (1 or 2)
static FwdPlan plan_fwd_qg(const AttnShape& s, int qg) {
  FwdPlan p;
  const int G = s.Hq / s.Hkv;
  p.P = kRows * qg / G;
  p.n_pb = (s.S + p.P - 1) / p.P;
  const long rowblocks = (long)s.B * s.Hkv * p.n_pb;
  long want = (KVPOP_FWD_TARGET_ITEMS + rowblocks - 1) / rowblocks;
  const long cap = (s.S + 511) / 512;
  if (want > cap) want = cap;
  if (want < 1) want = 1;
  int kmax = (int)((s.S + want - 1) / want);
  kmax = (kmax + kKT - 1) / kKT * kKT;
  p.kmax = kmax;
  p.n_pieces = (s.S + kmax - 1) / kmax;
  p.partial_floats = p.n_pieces > 1 ? (size_t)2 * p.n_pieces * s.B * s.Hq * (size_t)s.S : 0;
  return p;
}

FwdPlan plan_fwd(const AttnShape& s) { return plan_fwd_qg(s, 1); }

SparsePlan plan_fwd_sparse(const AttnShape& s, int budget) {
  SparsePlan sp;
  const FwdPlan p = plan_fwd(s);
  sp.n_blocks = (long)s.B * s.Hkv * p.n_pb;
  const long keys = std::min<long>(s.S, (long)budget + p.P);
  sp.cap = (int)((keys + kKT - 1) / kKT * kKT);
  sp.list_offset = ((size_t)sp.n_blocks * sizeof(int2) + 255) / 256 * 256;
  sp.workspace_bytes = sp.list_offset + (size_t)sp.n_blocks * sp.cap * sizeof(int);
  return sp;
}

size_t fwd_out_workspace_bytes(const AttnShape& s) {
  const size_t s_pad = (size_t)(s.S + kKT - 1) / kKT * kKT;
  return (size_t)s.B * s.Hkv * s.D * s_pad * sizeof(bf16_t);
}

hipError_t launch_fwd_lse(const AttnShape& s, const void* q, const void* k, const int* keep_until,
                          int budget, float* lse, void* workspace, hipStream_t st, const void* v,
                          void* o, int o_bf16) {
  const bool out = v != nullptr;
  const bool listed = keep_until && budget > 0 && !out;
  FwdPlan p = plan_fwd(s);
  if (listed || out) {  // whole rows: a listed block walks about budget + P keys
    p.kmax = (s.S + kKT - 1) / kKT * kKT;
    p.n_pieces = 1;
  }
  const int cus = device_cu_count();
  // launches of many rounds of whole rows: two query groups per wave
  bool wide = KVPOP_FWD_WIDE && s.D == 128 && !keep_until && !out && p.n_pieces == 1 &&
              (long)s.B * s.Hkv * p.n_pb >= (long)KVPOP_FWD_WIDE_ROUNDS * cus * KVPOP_FWD_MIN_BLOCKS;
  if (wide) {
    const FwdPlan p2 = plan_fwd_qg(s, 2);
    if (p2.n_pieces == 1) p = p2;
    else wide = false;
  }
  const int n_items = s.B * s.Hkv * p.n_pb * p.n_pieces;
  const float c = s.scale * kLog2e;
  // one resident round: deal each XCD's blocks in a snake
  const int per_cu = out ? kOutBlocks : wide ? 2 : KVPOP_FWD_MIN_BLOCKS;
  const int snake_cus = n_items <= cus * per_cu && cus % 8 == 0 ? cus / 8 : 0;
  const int s_pad = (s.S + kKT - 1) / kKT * kKT;
  bf16_t* vt = nullptr;
  if (out) {  // V^T into the workspace
    vt = reinterpret_cast<bf16_t*>(workspace);
    const unsigned n_blk = (unsigned)(s.B * s.Hkv * (s_pad / kKT));
    if (s.D == 128)
      hipLaunchKernelGGL(transpose_v_kernel<128>, dim3(n_blk), dim3(256), 0, st, (const bf16_t*)v, vt,
                         s.S, s_pad);
    else
      hipLaunchKernelGGL(transpose_v_kernel<64>, dim3(n_blk), dim3(256), 0, st, (const bf16_t*)v, vt,
                         s.S, s_pad);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  dim3 grid(n_items), block(kThreads);
  float2* part = reinterpret_cast<float2*>(workspace);
  const int2* hdr = nullptr;
  const int* lists = nullptr;
  int cap = 0;
  if (listed) {
    const SparsePlan sp = plan_fwd_sparse(s, budget);
    int2* h = reinterpret_cast<int2*>(workspace);
    int* l = reinterpret_cast<int*>(reinterpret_cast<char*>(workspace) + sp.list_offset);
    hipLaunchKernelGGL(keylist_kernel, dim3((unsigned)sp.n_blocks), dim3(256), 0, st, keep_until,
                       l, h, s.S, p.n_pb, p.P, sp.cap);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hdr = h;
    lists = l;
    cap = sp.cap;
  }
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, grid, block, 0, st, (const bf16_t*)q, (const bf16_t*)k, keep_until,
                       hdr, lists, cap, lse, part, s.B, s.Hq, s.Hkv, s.S, c, s.scale, p.n_pb,
                       p.kmax, p.n_pieces, n_items, snake_cus, (const bf16_t*)vt, s_pad, o,
                       o_bf16);
  };
  if (s.D == 128) {
    if (out && keep_until) go(fwd_lse_kernel<128, kMasked, true, 1>);
    else if (out) go(fwd_lse_kernel<128, kDense, true, 1>);
    else if (listed) go(fwd_lse_kernel<128, kListed, false, 1>);
    else if (keep_until) go(fwd_lse_kernel<128, kMasked, false, 1>);
    else if (wide) go(fwd_lse_kernel<128, kDense, false, 2>);
    else go(fwd_lse_kernel<128, kDense, false, 1>);
  } else {
    if (out && keep_until) go(fwd_lse_kernel<64, kMasked, true, 1>);
    else if (out) go(fwd_lse_kernel<64, kDense, true, 1>);
    else if (listed) go(fwd_lse_kernel<64, kListed, false, 1>);
    else if (keep_until) go(fwd_lse_kernel<64, kMasked, false, 1>);
    else go(fwd_lse_kernel<64, kDense, false, 1>);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_pieces == 1) return e;
  const long rows = (long)s.B * s.Hq * s.S;
  hipLaunchKernelGGL(fwd_lse_merge_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, st,
                     part, lse, s.B, s.Hq, s.S, c, s.scale, p.P, p.kmax);
  return hipGetLastError();
}

}  // namespace kvpop

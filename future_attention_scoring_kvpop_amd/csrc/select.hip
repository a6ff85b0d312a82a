// select.hip -- fixed-budget retention: per-row top-k selection, canonical
// slot layout and compaction of K/V into the bounded cache.
//
// KVpop summary (arXiv 2607.05061v2), Sec. 3 "fixed-budget pruning" (keep
// sink tokens, a protected recent window and the top-k long-range tokens
// per head; attention then runs over the retained set only), App. C.1 (the
// budget is B = s + w + k) and App. F (ranking and selection in fp32).
//
// gfx950 mapping
//   * One 1024-thread workgroup per (b, h) row.  Scores are mapped to
//     order-preserving uint32 keys (NaN lowest, -0 == +0) and the k-th
//     largest key is found by an MSD radix select.
//   * Rows of up to 32K eligible tokens are read once, coalesced: each
//     wave keeps the scores of a contiguous run of 64 x (4..32) positions
//     in registers (slots past the row hold a NaN, whose key is never
//     kept).  Three passes of 12, 10 and 10 bits count into histograms
//     shared by the workgroup, in a few copies (lane l into copy l % copies)
//     whose rows are padded by 4 words, so that lanes of one atomic rarely
//     hit one address or one bank although keys cluster; each pass picks
//     its digit with one block scan.  (Four passes of 8 bits with per-wave
//     histograms took 15% longer on a 32K row: the first byte, sign and
//     exponent, barely splits clustered scores.)
//     Ties at the threshold key go to the lowest positions; since the kept
//     equal keys fill up in position order, one scan of the waves' packed
//     (equal, above) counts plus ballots within each wave give every kept
//     token its output slot, so the long-range slots come out in ascending
//     position with no sort.  The slots are staged in LDS (the histograms
//     are free by then) and written by consecutive threads, and the kept
//     scores come from registers, not from a second read of the row.
//   * Longer rows are streamed from memory: four 8-bit passes with per-wave
//     histograms, then two block scans per 8K-position chunk.
//   * The gather is a separate, fully coalesced 16-byte-per-lane copy with
//     non-temporal loads and stores (each byte moves once).  Launches with
//     at most half as many rows as CUs instead run every row's selection in
//     several workgroups (it is latency-bound, so the repeats cost little)
//     and let each copy a share of the row's slots: selection + compaction
//     41 -> 36 us on a 32k-prefill layer (8 rows), 12.7 -> 9.8 us on the 4k
//     layer.
#include <algorithm>

#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kVPT = 8;  // contiguous positions per thread per compaction chunk

// exclusive scan over the workgroup; returns the prefix, total in *total
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  if (wave == 0) {
    uint32_t s = lane < kSelWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kSelWaves; off <<= 1) {
      const uint32_t y = __shfl_up(s, off);
      if (lane >= off) s += y;
    }
    if (lane < kSelWaves) wsum[kSelWaves + lane] = s;  // inclusive wave prefix
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[kSelWaves + wave - 1] : 0u;
  *total = wsum[2 * kSelWaves - 1];
  __syncthreads();
  return before + x - v;
}

// Streamed path: 8-bit digits, one 256-bin histogram per wave; the row
// stride is padded by 4 words so that one bin of different waves' rows
// falls in different banks.
constexpr int kHistStride = 260;

// Register path: digits of 12, 10 and 10 bits (three passes).  Its
// histograms are shared by the workgroup in kSelCopies copies, lane l
// counting into copy l % kSelCopies: keys cluster (scores share a few
// exponents, and ties), and lanes of one atomic that hit one LDS address
// serialise.  The copies' rows are padded by 4 words so that one bin of
// different copies falls in different banks.
#ifndef KVPOP_SEL_COPIES
#define KVPOP_SEL_COPIES 4
#endif
constexpr int kSelCopies = KVPOP_SEL_COPIES;
constexpr int kRegBins0 = 4096, kRegStride0 = kRegBins0 + 4;  // bits 31..20
constexpr int kRegBins = 1024, kRegStride = kRegBins + 4;     // bits 19..10, 9..0
static_assert(kRegBins % kSelThreads == 0 && kRegBins0 % kSelThreads == 0, "bins per thread");

// The LDS array holds the histograms during the radix passes and the kept
// slots of the long-range region (8 bytes per slot) after them: at least
// enough for rows of 16 scores per lane, so those are always staged.
constexpr int kSelLdsWords = std::max({kSelWaves * kHistStride, kSelCopies * kRegStride0,
                                       2 * 16 * kSelThreads});
constexpr size_t kSelLdsBytes = sizeof(uint32_t) * kSelLdsWords;

// Lanes below this one whose bit is set in m (the rank of this lane among
// the set lanes), plus base.
__device__ __forceinline__ uint32_t lanes_below(unsigned long long m, uint32_t base) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, base));
}

// Wave 0 turns the per-wave digit histograms of one radix pass into the
// digit of the rem-th largest key (higher digits first) and the rank of
// that key among the keys with this digit.
__device__ __forceinline__ void radix_pick(const uint32_t (*hist)[kHistStride], uint32_t rem,
                                           uint32_t* sh_digit, uint32_t* sh_rem) {
  const int lane = threadIdx.x & 63;
  uint32_t cnt[4], tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t c = 0;
    for (int w = 0; w < kSelWaves; ++w) c += hist[w][4 * lane + i];
    cnt[i] = c;
    tot += c;
  }
  // inclusive suffix sum over lanes
  uint32_t x = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(x, off);
    if (lane + off < 64) x += y;
  }
  const uint32_t above = x - tot;
  if (above < rem && rem <= x) {
    uint32_t cum = above;
    for (int i = 3; i >= 0; --i) {
      if (cum + cnt[i] >= rem) {
        *sh_digit = 4 * lane + i;
        *sh_rem = rem - cum;
        break;
      }
      cum += cnt[i];
    }
  }
}

// The whole workgroup turns a histogram of NB bins (kSelCopies copies at
// stride cs; higher digits rank first) into the digit of the rem-th largest
// key and the rank of that key among the keys with this digit.  Thread t
// owns the NB / kSelThreads bins below NB - t * NB / kSelThreads, so one
// exclusive scan over the threads counts the keys in higher bins.  Needs
// 1 <= rem <= the number of keys counted; the results are valid after the
// caller's next barrier.
template <int NB>
__device__ __forceinline__ void block_pick(const uint32_t* h, int cs, uint32_t rem, uint32_t* wsum,
                                           uint32_t* sh_digit, uint32_t* sh_rem) {
  constexpr int BPT = NB / kSelThreads;
  const int b0 = NB - BPT * ((int)threadIdx.x + 1);
  uint32_t cnt[BPT], tot = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) {
    uint32_t c = 0;
#pragma unroll
    for (int k = 0; k < kSelCopies; ++k) c += h[k * cs + b0 + j];
    cnt[j] = c;
    tot += c;
  }
  uint32_t total;
  const uint32_t above = block_exclusive_scan(tot, wsum, &total);
  if (above < rem && rem <= above + tot) {
    uint32_t cum = above;
    bool found = false;
#pragma unroll
    for (int j = BPT - 1; j >= 0; --j) {
      if (!found && cum + cnt[j] >= rem) {
        *sh_digit = (uint32_t)(b0 + j);
        *sh_rem = rem - cum;
        found = true;
      }
      cum += cnt[j];
    }
  }
}

// VPT > 0: rows of at most VPT * kSelThreads eligible tokens, held in
// registers (VPT scores per lane) for the radix passes and the compaction;
// STAGE: the kept slots are staged in LDS (the launcher sets it only when
// 8 * kk bytes fit the histogram array).
// VPT == 0: longer rows, streamed from memory in chunks.
//
// GATHER (with VPT > 0 and STAGE): the launch has nsplit workgroups per row;
// each selects the whole row (the selection of a short launch is bound by
// latency, not work), part 0 writes slot_pos and slot_score, and part i
// then copies the K/V rows of slots [i, i + 1) * ceil(budget / nsplit) into
// the cache, so the compaction of a launch with few rows is spread over the
// chip without a second launch.
template <int VPT, bool STAGE, bool GATHER>
__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, int S, int n_sink, int window, int budget,
    const bf16_t* __restrict__ kg, const bf16_t* __restrict__ vg, bf16_t* __restrict__ kcg,
    bf16_t* __restrict__ vcg, int D, int nsplit) {
  static_assert(!GATHER || (VPT > 0 && STAGE), "the fused compaction reads the staged slots");
  __shared__ __attribute__((aligned(16))) uint32_t lds[kSelLdsWords];
  __shared__ uint32_t wsum[2 * kSelWaves];
  __shared__ uint32_t sh_digit, sh_rem;

  const int part = GATHER ? (int)(blockIdx.x % (unsigned)nsplit) : 0;
  const long row = GATHER ? (long)(blockIdx.x / (unsigned)nsplit) : (long)blockIdx.x;
  const bool writer = part == 0;
  const float* sc = scores + row * S;
  int32_t* sp = slot_pos + row * budget;
  float* ss = slot_score ? slot_score + row * budget : nullptr;
  const int tid = threadIdx.x, wave = tid >> 6;
  const int kk = budget - n_sink - window;
  const int e_lo = n_sink;
  const int e_hi = max(S - window, n_sink);
  const int n_e = e_hi - e_lo;
  const int n_keep = min(n_e, kk);

  // sinks, window ring and the padding of the long-range region
  const int w_lo = max(S - window, n_sink);
  auto ring_pos = [&](int j) {
    const int idx = j - n_sink - kk;  // ring index = p mod w
    const int cand = w_lo + ((idx - w_lo % window) % window + window) % window;
    return cand < S ? cand : -1;
  };
  if (writer) {
    for (int j = tid; j < budget; j += kSelThreads) {
      int p = -1;
      bool write = true;
      if (j < n_sink) {
        p = j < S ? j : -1;
      } else if (j < n_sink + kk) {
        write = j >= n_sink + n_keep;
      } else {
        p = ring_pos(j);
      }
      if (write) {
        sp[j] = p;
        if (ss) ss[j] = p >= 0 ? sc[p] : -INFINITY;
      }
    }
  }
  // the long-range slots come from the selection below unless every
  // eligible token is kept (or none can be)
  const bool select = n_keep > 0 && n_e > kk;
  if (n_keep > 0 && n_e <= kk && writer) {  // everything eligible is kept
    for (int i = tid; i < n_e; i += kSelThreads) {
      const int p = e_lo + i;
      sp[n_sink + i] = p;
      if (ss) ss[n_sink + i] = sc[p];
    }
  }

  if (!select) {
  } else if constexpr (VPT > 0) {
    // wave w owns the 64*VPT positions from e_lo + 64*VPT*w; its lane l
    // holds position e_lo + 64*(VPT*w + i) + l in slot i (coalesced loads)
    const int lane = tid & 63;
    const int p0 = e_lo + 64 * VPT * wave + lane;
    // Slots past the row hold a NaN, whose key is 0: they rank with the
    // lowest tokens and come after every real position, so with kk < n_e
    // none of them is ever kept and the counts stay consistent.
    // Only the scores stay in registers and the keys are recomputed where
    // they are used (a few ALU operations): keys, scores and positions side
    // by side at 32 per lane overflow the 128 registers of a 1024-thread
    // workgroup and spill.  The kept scores are written from the registers
    // with their own bits (keys merge -0/+0 and NaNs).
    float raw[VPT];
    if (e_lo + 64 * VPT * (wave + 1) <= e_hi) {  // the whole run is in the row
#pragma unroll
      for (int i = 0; i < VPT; ++i) raw[i] = sc[p0 + 64 * i];
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) raw[i] = sc[min(p0 + 64 * i, e_hi - 1)];
#pragma unroll
      for (int i = 0; i < VPT; ++i)
        if (p0 + 64 * i >= e_hi) raw[i] = __uint_as_float(0x7fc00000u);
    }
    // ---- radix select of the kk-th largest key: bits 31..20, then
    // 19..10 and 9..0 of the keys under the prefix chosen so far ----
    uint32_t prefix = 0, rem = (uint32_t)kk;
    const int copy = lane % kSelCopies;
    for (int pass = 0; pass < 3; ++pass) {
      const int stride = pass == 0 ? kRegStride0 : kRegStride;
      const int shift = pass == 0 ? 20 : 20 - 10 * pass;
      const uint32_t pmask = pass == 0 ? 0u : ~0u << (shift + 10);
      const uint32_t dmask = pass == 0 ? kRegBins0 - 1 : kRegBins - 1;
      // block_pick's reads of the previous histogram precede its barriers
      for (int i = tid; i < kSelCopies * stride / 4; i += kSelThreads)
        reinterpret_cast<uint4*>(lds)[i] = make_uint4(0, 0, 0, 0);
      __syncthreads();
      uint32_t* h = lds + copy * stride;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t key = rank_key(raw[i]);
        if ((key & pmask) == prefix) atomicAdd(&h[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      if (pass == 0)
        block_pick<kRegBins0>(lds, kRegStride0, rem, wsum, &sh_digit, &sh_rem);
      else
        block_pick<kRegBins>(lds, kRegStride, rem, wsum, &sh_digit, &sh_rem);
      __syncthreads();
      prefix |= sh_digit << shift;
      rem = sh_rem;
    }
    const uint32_t T = prefix;     // key of the kk-th best token
    const uint32_t need_eq = rem;  // tokens with key == T to keep (lowest positions)

    // ---- compaction in position order: tokens above T, and the first
    // need_eq tokens equal to T.  Counts before a wave come from one scan of
    // the waves' packed (equal, above) totals; within a wave, ballots order
    // the lanes; before any position, min(equal so far, need_eq) of the
    // equal tokens were kept. ----
    uint32_t w_gt = 0, w_eq = 0;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const uint32_t key = rank_key(raw[i]);
      w_gt += __popcll(__ballot(key > T));
      w_eq += __popcll(__ballot(key == T));
    }
    if (lane == 0) wsum[wave] = (w_eq << 16) | w_gt;
    __syncthreads();
    uint32_t pre = 0;
    for (int w = 0; w < wave; ++w) pre += wsum[w];
    // wave-uniform from here on: kept in scalar registers
    uint32_t eq_run = __builtin_amdgcn_readfirstlane(pre >> 16);
    uint32_t out = __builtin_amdgcn_readfirstlane((pre & 0xffffu) + min(pre >> 16, need_eq));
    // the positions are recomputed here from a copy of p0 the compiler
    // cannot see through; otherwise it keeps all VPT of them live from the
    // loads on
    int q0 = p0;
    asm volatile("" : "+v"(q0));
    // STAGE: the kept positions and scores are staged in LDS (the
    // histograms are free now) and then written with consecutive threads on
    // consecutive slots, instead of one scattered store per kept token
    int* stg_p = reinterpret_cast<int*>(lds);
    float* stg_s = reinterpret_cast<float*>(stg_p + kk);
    auto put = [&](int i, uint32_t o) {
      if constexpr (STAGE) {
        stg_p[o] = q0 + 64 * i;
        stg_s[o] = raw[i];
      } else {
        sp[n_sink + o] = q0 + 64 * i;
        if (ss) ss[n_sink + o] = raw[i];
      }
    };
    // A wave before the tie cut keeps all its keys equal to T, a wave after
    // it none: only the wave the cut falls in ranks its equal keys.
    const uint32_t w_eq_u = __builtin_amdgcn_readfirstlane(w_eq);
    if (eq_run + w_eq_u <= need_eq || eq_run >= need_eq) {
      const bool with_eq = eq_run + w_eq_u <= need_eq;
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t key = rank_key(raw[i]);
        const bool keep = key > T || (with_eq && key == T);
        const unsigned long long km = __ballot(keep);
        const uint32_t o = lanes_below(km, out);
        if (keep && o < (uint32_t)kk) put(i, o);
        out += (uint32_t)__popcll(km);
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        const uint32_t key = rank_key(raw[i]);
        const bool eq = key == T;
        const unsigned long long em = __ballot(eq);
        const bool keep = key > T || (eq && lanes_below(em, eq_run) < need_eq);
        const unsigned long long km = __ballot(keep);
        const uint32_t o = lanes_below(km, out);
        if (keep && o < (uint32_t)kk) put(i, o);
        out += (uint32_t)__popcll(km);
        eq_run += (uint32_t)__popcll(em);
      }
    }
    if constexpr (STAGE) {
      __syncthreads();
      if (writer) {
        for (int j = tid; j < kk; j += kSelThreads) {
          sp[n_sink + j] = stg_p[j];
          if (ss) ss[n_sink + j] = stg_s[j];
        }
      }
    }
  } else {
    // ---- radix select of the kk-th largest key, re-reading the scores ----
    uint32_t(*hist)[kHistStride] = reinterpret_cast<uint32_t(*)[kHistStride]>(lds);
    uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kk;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      for (int i = tid; i < kSelWaves * kHistStride; i += kSelThreads) (&hist[0][0])[i] = 0u;
      __syncthreads();
      for (int p = e_lo + tid; p < e_hi; p += kSelThreads) {
        const uint32_t key = rank_key(sc[p]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) radix_pick(hist, rem, &sh_digit, &sh_rem);
      __syncthreads();
      prefix |= sh_digit << shift;
      pmask |= 255u << shift;
      rem = sh_rem;
      __syncthreads();
    }
    const uint32_t T = prefix;
    const uint32_t need_eq = rem;

    // ---- compaction in position order, chunk by chunk ----
    uint32_t eq_run = 0, kept_run = 0, total;
    for (int base = e_lo; base < e_hi; base += kSelThreads * kVPT) {
      const int p0 = base + tid * kVPT;
      uint32_t keys[kVPT];
      uint32_t n_gt = 0, n_eq = 0;
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
        const int p = p0 + i;
        keys[i] = p < e_hi ? rank_key(sc[p]) : 0u;
        const bool in = p < e_hi;
        n_gt += (in && keys[i] > T) ? 1u : 0u;
        n_eq += (in && keys[i] == T) ? 1u : 0u;
      }
      const uint32_t eq_pre = eq_run + block_exclusive_scan(n_eq, wsum, &total);
      const uint32_t eq_tot = total;
      const uint32_t take = eq_pre >= need_eq ? 0u : min(n_eq, need_eq - eq_pre);
      const uint32_t kept_pre = kept_run + block_exclusive_scan(n_gt + take, wsum, &total);
      uint32_t out = n_sink + kept_pre, e = eq_pre;
#pragma unroll
      for (int i = 0; i < kVPT; ++i) {
        const int p = p0 + i;
        if (p >= e_hi) break;
        bool keep = keys[i] > T;
        if (keys[i] == T) {
          keep = e < need_eq;
          ++e;
        }
        if (keep && out < (uint32_t)(n_sink + kk)) {
          sp[out] = p;
          if (ss) ss[out] = sc[p];
          ++out;
        }
      }
      eq_run += eq_tot;
      kept_run += total;
    }
  }

  if constexpr (GATHER) {
    // this part's slots: sinks, the staged long-range slots (the selection
    // fills all kk of them), the window ring; 16 bytes of K and V per thread
    const int* stg_p = reinterpret_cast<const int*>(lds);
    const int per = (budget + nsplit - 1) / nsplit;
    const int j0 = part * per, j1 = min(budget, j0 + per);
    const int cpr = D / 8;
    for (int e = tid; e < (j1 - j0) * cpr; e += kSelThreads) {
      const int j = j0 + e / cpr, cc = e - (e / cpr) * cpr;
      int p;
      if (j < n_sink) {
        p = j < S ? j : -1;
      } else if (j < n_sink + kk) {
        const int i = j - n_sink;
        p = !select ? (i < n_keep ? e_lo + i : -1) : stg_p[i];
      } else {
        p = ring_pos(j);
      }
      uint4 a = make_uint4(0, 0, 0, 0), bv = make_uint4(0, 0, 0, 0);
      if (p >= 0) {
        const size_t src = ((size_t)row * S + p) * D + cc * 8;
        a = ldg16_nt(kg + src);
        bv = ldg16_nt(vg + src);
      }
      const size_t dst = ((size_t)row * budget + j) * D + cc * 8;
      stg16_nt(kcg + dst, a);
      stg16_nt(vcg + dst, bv);
    }
  }
}

// Non-temporal hints of the gather: 1 loads, 2 stores (bit mask; both
// measured 7-10% faster on the 512-row prefix compaction than neither).
#ifndef KVPOP_GATHER_NT
#define KVPOP_GATHER_NT 3
#endif

// One thread per 16-byte chunk of one cache row, for K and V.
__global__ __launch_bounds__(256) void gather_kernel(const int32_t* __restrict__ slot_pos,
                                                     const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v,
                                                     bf16_t* __restrict__ kc,
                                                     bf16_t* __restrict__ vc, int S, int D,
                                                     int budget, long n_chunks) {
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= n_chunks) return;
  const int cpr = D / 8;
  const long srow = gid / cpr;
  const int cc = (int)(gid % cpr);
  const long row = srow / budget;
  const int p = slot_pos[srow];
  uint4 a = make_uint4(0, 0, 0, 0), bv = make_uint4(0, 0, 0, 0);
  if (p >= 0 && p < S) {
    const size_t src = ((size_t)row * S + p) * D + cc * 8;
    a = KVPOP_GATHER_NT & 1 ? ldg16_nt(k + src) : ldg16(k + src);
    bv = KVPOP_GATHER_NT & 1 ? ldg16_nt(v + src) : ldg16(v + src);
  }
  if (KVPOP_GATHER_NT & 2) {
    stg16_nt(kc + (size_t)srow * D + cc * 8, a);
    stg16_nt(vc + (size_t)srow * D + cc * 8, bv);
  } else {
    stg16(kc + (size_t)srow * D + cc * 8, a);
    stg16(vc + (size_t)srow * D + cc * 8, bv);
  }
}

}  // namespace

hipError_t launch_select(int B, int Hkv, int S, int n_sink, int window, int budget,
                         const float* scores, int32_t* slot_pos, float* slot_score,
                         hipStream_t st) {
  const int n_e = std::max(S - window, n_sink) - n_sink;
  // staging holds 8 bytes per long-range slot; with n_e <= 16 * kSelThreads
  // the slots kept (fewer than n_e) always fit (kSelLdsWords)
  const size_t kk = (size_t)std::max(budget - n_sink - window, 0);
  const bool stage = kk * 8 <= kSelLdsBytes;
#define KVPOP_SEL(V, ST)                                                                      \
  hipLaunchKernelGGL((select_kernel<V, ST, false>), dim3(B * Hkv), dim3(kSelThreads), 0, st,  \
                     scores, slot_pos, slot_score, S, n_sink, window, budget, nullptr, nullptr, \
                     nullptr, nullptr, 0, 1)
  if (n_e <= 4 * kSelThreads)
    KVPOP_SEL(4, true);
  else if (n_e <= 8 * kSelThreads)
    KVPOP_SEL(8, true);
  else if (n_e <= 16 * kSelThreads)
    KVPOP_SEL(16, true);
  else if (n_e <= 32 * kSelThreads && stage)
    KVPOP_SEL(32, true);
  else if (n_e <= 32 * kSelThreads)
    KVPOP_SEL(32, false);
  else
    KVPOP_SEL(0, false);
#undef KVPOP_SEL
  return hipGetLastError();
}

hipError_t launch_select_gather(int B, int Hkv, int S, int D, int n_sink, int window, int budget,
                                const float* scores, int32_t* slot_pos, float* slot_score,
                                const void* k, const void* v, void* kc, void* vc, hipStream_t st) {
  // Launches with at most half as many rows as CUs select every row in
  // several workgroups, each also compacting a share of the row's slots;
  // larger ones select one row per workgroup and compact in a second launch.
  const long rows = (long)B * Hkv;
  const int cus = device_cu_count();
  const int n_e = std::max(S - window, n_sink) - n_sink;
  const size_t kk = (size_t)std::max(budget - n_sink - window, 0);
  const bool stage = kk * 8 <= kSelLdsBytes;
  const int nsplit = (int)std::min<long>({64, rows > 0 ? cus / rows : 1, budget});
  if (nsplit >= 2 && n_e <= 32 * kSelThreads && stage) {
    const dim3 grid((unsigned)(rows * nsplit));
#define KVPOP_SELG(V)                                                                           \
  hipLaunchKernelGGL((select_kernel<V, true, true>), grid, dim3(kSelThreads), 0, st, scores,    \
                     slot_pos, slot_score, S, n_sink, window, budget, (const bf16_t*)k,          \
                     (const bf16_t*)v, (bf16_t*)kc, (bf16_t*)vc, D, nsplit)
    if (n_e <= 4 * kSelThreads)
      KVPOP_SELG(4);
    else if (n_e <= 8 * kSelThreads)
      KVPOP_SELG(8);
    else if (n_e <= 16 * kSelThreads)
      KVPOP_SELG(16);
    else
      KVPOP_SELG(32);
#undef KVPOP_SELG
    return hipGetLastError();
  }
  hipError_t e = launch_select(B, Hkv, S, n_sink, window, budget, scores, slot_pos, slot_score, st);
  if (e != hipSuccess) return e;
  return launch_gather(B, Hkv, S, D, budget, slot_pos, k, v, kc, vc, st);
}

hipError_t launch_gather(int B, int Hkv, int S, int D, int budget, const int32_t* slot_pos,
                         const void* k, const void* v, void* kc, void* vc, hipStream_t st) {
  const long n = (long)B * Hkv * budget * (D / 8);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slot_pos,
                     (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)kc, (bf16_t*)vc, S, D, budget, n);
  return hipGetLastError();
}

}  // namespace kvpop

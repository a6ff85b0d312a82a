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
//     largest key is found by a 4-pass MSD radix select (8-bit digits,
//     per-wave LDS histograms, one wave-parallel suffix scan per pass).
//     Rows of 8K..32K eligible tokens hold their keys in registers (32 per
//     thread) across the four passes; shorter and longer rows re-read them.
//   * Ties at the threshold key go to the lowest positions: a block-wide
//     scan over the row in position order counts equal keys, and a second
//     scan gives every kept token its output slot, so the long-range slots
//     come out in ascending position with no sort.
//   * The gather is a separate, fully coalesced 16-byte-per-lane copy.
#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kVPT = 8;  // contiguous positions per thread per compaction chunk
constexpr int kRegKeys = 32;       // eligible keys per thread held in registers (32768 per row)
constexpr int kRegMin = 8 * 1024;  // rows longer than this keep their keys in registers

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

__global__ __launch_bounds__(kSelThreads) void select_kernel(
    const float* __restrict__ scores, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, int S, int n_sink, int window, int budget) {
  __shared__ uint32_t hist[kSelWaves][256];
  __shared__ uint32_t wsum[2 * kSelWaves];
  __shared__ uint32_t sh_digit, sh_rem;

  const long row = blockIdx.x;
  const float* sc = scores + row * S;
  int32_t* sp = slot_pos + row * budget;
  float* ss = slot_score ? slot_score + row * budget : nullptr;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = budget - n_sink - window;
  const int e_lo = n_sink;
  const int e_hi = max(S - window, n_sink);
  const int n_e = e_hi - e_lo;
  const int n_keep = min(n_e, kk);

  // sinks, window ring and the padding of the long-range region
  const int w_lo = max(S - window, n_sink);
  for (int j = tid; j < budget; j += kSelThreads) {
    int p = -1;
    bool write = true;
    if (j < n_sink) {
      p = j < S ? j : -1;
    } else if (j < n_sink + kk) {
      write = j >= n_sink + n_keep;
    } else {
      const int idx = j - n_sink - kk;  // ring index = p mod w
      const int cand = w_lo + ((idx - w_lo % window) % window + window) % window;
      p = cand < S ? cand : -1;
    }
    if (write) {
      sp[j] = p;
      if (ss) ss[j] = p >= 0 ? sc[p] : -INFINITY;
    }
  }
  if (n_keep <= 0) return;

  if (n_e <= kk) {  // everything eligible is kept
    for (int i = tid; i < n_e; i += kSelThreads) {
      const int p = e_lo + i;
      sp[n_sink + i] = p;
      if (ss) ss[n_sink + i] = sc[p];
    }
    return;
  }

  // ---- radix select of the kk-th largest key ----
  // Long rows (more than kRegMin eligible tokens, up to kRegKeys per
  // thread) read their keys once into registers for all four passes;
  // shorter rows, whose passes are latency-bound, re-read the scores.
  const bool in_regs = n_e > kRegMin && n_e <= kRegKeys * kSelThreads;
  uint32_t rk[kRegKeys];
  if (in_regs) {
#pragma unroll
    for (int i = 0; i < kRegKeys; ++i) {
      const int p = e_lo + tid + i * kSelThreads;
      rk[i] = p < e_hi ? rank_key(sc[p]) : 0u;
    }
  }
  uint32_t prefix = 0, pmask = 0, rem = (uint32_t)kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < kSelWaves * 256; i += kSelThreads) (&hist[0][0])[i] = 0u;
    __syncthreads();
    if (in_regs) {
#pragma unroll
      for (int i = 0; i < kRegKeys; ++i)
        if (tid + i * kSelThreads < n_e && (rk[i] & pmask) == prefix)
          atomicAdd(&hist[wave][(rk[i] >> shift) & 255u], 1u);
    } else {
      for (int p = e_lo + tid; p < e_hi; p += kSelThreads) {
        const uint32_t key = rank_key(sc[p]);
        if ((key & pmask) == prefix) atomicAdd(&hist[wave][(key >> shift) & 255u], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t cnt[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t c = 0;
        for (int w = 0; w < kSelWaves; ++w) c += hist[w][4 * lane + i];
        cnt[i] = c;
        tot += c;
      }
      // inclusive suffix sum over lanes (higher digits first)
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
            sh_digit = 4 * lane + i;
            sh_rem = rem - cum;
            break;
          }
          cum += cnt[i];
        }
      }
    }
    __syncthreads();
    prefix |= sh_digit << shift;
    pmask |= 255u << shift;
    rem = sh_rem;
    __syncthreads();
  }
  const uint32_t T = prefix;        // key of the kk-th best token
  const uint32_t need_eq = rem;     // tokens with key == T to keep (lowest positions)

  // ---- compaction in position order ----
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
  (void)lane;
}

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
    a = ldg16(k + src);
    bv = ldg16(v + src);
  }
  stg16(kc + (size_t)srow * D + cc * 8, a);
  stg16(vc + (size_t)srow * D + cc * 8, bv);
}

}  // namespace

hipError_t launch_select(int B, int Hkv, int S, int n_sink, int window, int budget,
                         const float* scores, int32_t* slot_pos, float* slot_score,
                         hipStream_t st) {
  hipLaunchKernelGGL(select_kernel, dim3(B * Hkv), dim3(kSelThreads), 0, st, scores, slot_pos,
                     slot_score, S, n_sink, window, budget);
  return hipGetLastError();
}

hipError_t launch_gather(int B, int Hkv, int S, int D, int budget, const int32_t* slot_pos,
                         const void* k, const void* v, void* kc, void* vc, hipStream_t st) {
  const long n = (long)B * Hkv * budget * (D / 8);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, slot_pos,
                     (const bf16_t*)k, (const bf16_t*)v, (bf16_t*)kc, (bf16_t*)vc, S, D, budget, n);
  return hipGetLastError();
}

}  // namespace kvpop

// running_topk.hip -- the running top-k retention mask and its cutoffs.
//
// KVpop summary (arXiv 2607.05061v2), App. C.1: at query d the fixed-budget
// mask keeps the sinks, the protected window (d-w, d] and the k best tokens
// of the eligible pool P_d = [s, d-w]; App. C.2: the per-query cutoffs of
// that running top-k (computed there with a Fenwick tree); Sec. 3 and
// App. B.3: a per-KV-head decay gamma_h turns into the static priority
// pi_t = sigma_t + lambda_h t with lambda_h = -ln gamma_h; App. F: ranking
// in fp32.
//
// The pool only grows, so token t (t >= s) is selected from query t+w
// until the query at which the k-th token that ranks before it has entered
// the pool, and is the pool's k-th best (the cutoff) from the entry of the
// (k-1)-th such token on.  With p_j = position of the j-th better-ranked
// token in position order:
//   keep_until[t] = min(S, max(t + w, p_k + w))     (S when p_k does not exist)
//   cutoff[d] = t  for d in [max(t + w, p_{k-1} + w), min(S, p_k + w))
// Every query whose pool holds at least k tokens lies in exactly one such
// interval; the others get -1.
//
// gfx950 mapping: two kernels.  Rows up to KVPOP_RT_LONG_MIN tokens take the
// counting kernel (O(S^2 / 64) compares, no workspace, one launch of many
// small workgroups); longer rows the O(S log S) kernel further below (sort,
// wavelet matrix, one workgroup per row, a workspace).  Counting kernel:
//   * A workgroup owns 64 consecutive tokens (one per lane) of one row; its
//     NSEG waves split the scanned positions [s, S) into NSEG segments of at
//     most 64 chunks of 64 positions.
//     Each wave ranks the 64 positions of a
//     chunk (one per lane), stores their keys in its own 256 bytes of LDS
//     and reads them back four at a time with broadcast ds_read_b128, so a
//     comparison of one position against the wave's 64 tokens costs one
//     VALU compare and one add.  The rows are L2-resident (4 bytes per
//     token).
//   * "Better" is the retention order: larger order-preserving uint32 key
//     first, the lower position on equal keys.  Keys are stored plus one so
//     that 0 marks positions outside the pool; before position t a token
//     with an equal key ranks first (>=), after it only a larger key does.
//   * The counting pass records each lane's count per chunk (one byte) and
//     per segment.  Then the wave whose segment holds a lane's (k-1)-th or
//     k-th better token walks that lane's chunk counts to the chunk and
//     rescans those 64 positions for the lane alone; the row is never read
//     a second time.
#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

// chunks of 64 positions per wave at most (sixteen waves: rows up to 65536)
constexpr int kRtChunksPerSeg = 64;
// rows longer than this take the O(S log S) kernel below (with a workspace);
// shorter ones the counting kernel, which needs none
#ifndef KVPOP_RT_LONG_MIN
#define KVPOP_RT_LONG_MIN 8192
#endif
static_assert(KVPOP_RT_LONG_MIN <= 16 * kRtChunksPerSeg * 64, "the counting kernel's longest row");
// the longest row either kernel takes
#define KVPOP_RT_MAX_LEN (1 << 24)

__device__ __forceinline__ uint32_t priority_key(float sigma, float lam, int t) {
  // pi = sigma + lambda * t, each operation rounded to fp32: contraction
  // into one FMA (a single rounding) would rank some ties differently
#pragma clang fp contract(off)
  const float age = lam * (float)t;
  const float pi = sigma + age;
  return rank_key(pi) + 1u;
}

__device__ __forceinline__ uint32_t order_key(const float* __restrict__ sc, float lam, int t) {
  return priority_key(sc[t], lam, t);
}

template <int NSEG, int CPS>
__global__ __launch_bounds__(64 * NSEG) void running_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ log_decay,
    int* __restrict__ keep_until, int* __restrict__ cutoff, int Hkv, int S, int n_sink,
    int window, int k, int blocks_per_row, int seg_chunks) {
  __shared__ __attribute__((aligned(16))) uint32_t keys[NSEG][64];
  __shared__ uint8_t ccount[NSEG][CPS][64];
  __shared__ int segtot[NSEG][64];
  __shared__ int found[2][64];  // positions of the (k-1)-th and k-th better token

  const int row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - row * blocks_per_row;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tb = blk * 64;  // the workgroup's first token
  const int t = tb + lane;
  const float lam = log_decay ? log_decay[row % Hkv] : 0.f;
  const float* sc = scores + (size_t)row * S;
  int* until = keep_until + (size_t)row * S;
  int* cut = cutoff ? cutoff + (size_t)row * S : nullptr;

  // queries whose pool holds fewer than k tokens have no cutoff
  if (wave == 0 && cut && t < S) {
    const long first_full = (long)n_sink + k - 1 + window;
    if (k == 0 || (long)t < first_full) cut[t] = -1;
  }
  // tokens that need no scan: sinks, tokens whose window reaches the end
  const bool scan = t < S && t >= n_sink && (long)t + window < S && k > 0;
  const bool any_scan = __syncthreads_or(scan) != 0;
  if (!any_scan) {
    if (wave == 0 && t < S) until[t] = (t >= n_sink && k == 0) ? min(S, t + window) : S;
    return;
  }
  const uint32_t kt = scan ? order_key(sc, lam, t) : 0u;
  const uint32_t thr_before = kt, thr_after = kt + 1u;  // kt <= 0xff800001: no wrap

  // ---- counting pass over this wave's segment ----
  const int c_first = n_sink & ~63;
  const int cbeg = c_first + wave * seg_chunks * 64;
  int cnt = 0, n_done = 0;
  for (int ci = 0; ci < seg_chunks; ++ci) {
    const int c0 = cbeg + ci * 64;
    if (c0 >= S) break;
    n_done = ci + 1;
    const int j = c0 + lane;
    keys[wave][lane] = (j >= n_sink && j < S) ? order_key(sc, lam, j) : 0u;
    __builtin_amdgcn_wave_barrier();
    const int before = cnt;
    if (c0 != tb) {
      const uint32_t thr = c0 < tb ? thr_before : thr_after;
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&keys[wave][i]);
        cnt += (v.x >= thr) + (v.y >= thr) + (v.z >= thr) + (v.w >= thr);
      }
    } else {  // the chunk of the workgroup's own tokens
#pragma unroll
      for (int i = 0; i < 64; i += 4) {
        const uint4 v = *reinterpret_cast<const uint4*>(&keys[wave][i]);
        cnt += (v.x >= (i + 0 < lane ? thr_before : thr_after)) +
               (v.y >= (i + 1 < lane ? thr_before : thr_after)) +
               (v.z >= (i + 2 < lane ? thr_before : thr_after)) +
               (v.w >= (i + 3 < lane ? thr_before : thr_after));
      }
    }
    ccount[wave][ci][lane] = (uint8_t)(cnt - before);
    __builtin_amdgcn_wave_barrier();
  }
  segtot[wave][lane] = cnt;
  if (wave == 0) found[0][lane] = found[1][lane] = -1;
  __syncthreads();

  // ---- locate the (k-1)-th and k-th better tokens of each lane ----
  int pre = 0;
  for (int w = 0; w < wave; ++w) pre += segtot[w][lane];
#pragma unroll
  for (int which = 0; which < 2; ++which) {
    const int target = which == 0 ? k - 1 : k;
    const bool mine = scan && target >= 1 && pre < target && target <= pre + cnt;
    if (__any(mine)) {
      int acc = pre, ci = 0;
      if (mine) {
        while (ci < n_done - 1 && acc + ccount[wave][ci][lane] < target)
          acc += ccount[wave][ci++][lane];
      }
      // rescan chunk ci of the segment for this lane alone: 16 loads at a
      // time (indices clamped into the row), each batch resolved branch-free
      const int c0 = cbeg + ci * 64;
      int pos = -1;
      if (mine) {
        for (int e0 = 0; e0 < 64; e0 += 16) {
          float v[16];
#pragma unroll
          for (int e = 0; e < 16; ++e) v[e] = sc[min(c0 + e0 + e, S - 1)];
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int p = c0 + e0 + e;
            const uint32_t kv = (p >= n_sink && p < S) ? priority_key(v[e], lam, p) : 0u;
            const int nacc = acc + (kv >= (p < t ? thr_before : thr_after));
            pos = (acc < target && nacc >= target) ? p : pos;
            acc = nacc;
          }
          if (acc >= target) break;
        }
        found[which][lane] = pos;
      }
    }
  }
  __syncthreads();

  // ---- outputs ----
  if (wave != 0 || t >= S) return;
  if (!scan) {
    until[t] = (t >= n_sink && k == 0) ? min(S, t + window) : S;
    return;
  }
  const int pk = found[1][lane], pk1 = found[0][lane];
  // the k-th better token enters the pool at query p_k + w; none: never
  const long leave = pk >= 0 ? (long)pk + window : (long)S + window;
  const long u = leave > (long)t + window ? leave : (long)t + window;
  until[t] = (int)(u < S ? u : S);
  if (cut) {
    // t is the pool's k-th best once k-1 better tokens are in the pool
    long d0 = k == 1 ? (long)t + window : (pk1 >= 0 ? (long)pk1 + window : (long)S);
    if (d0 < (long)t + window) d0 = (long)t + window;
    const long d1 = leave < S ? leave : S;
    for (long d = d0; d < d1; ++d) cut[d] = t;
  }
}

// ---------------------------------------------------------------------------
// Long rows in O(S log S).  App. C.2 takes the running cutoffs with a
// Fenwick tree in one sequential sweep per head; here one 1024-thread
// workgroup per row
//   1. ranks every token of [s, S) in the retention order by a stable LSD
//      radix sort of (complemented priority key, position) pairs: four
//      8-bit digits, counted by LDS atomics into per-wave rows; each wave
//      ranks its 64 lanes per step by eight ballots, so a pass needs
//      barriers only around its count scan;
//   2. builds a wavelet matrix over the ranks in position order: one stable
//      2-way partition per rank bit (most significant first), each level
//      keeping its bits and the zeros before every 32 of them;
//   3. (a second launch, many workgroups per row) takes the cutoff rank
//      c(d) = the k-th smallest rank among the first |P_d| pool positions
//      (the pool is a position prefix) by one descent of the matrix per
//      query; c(d) never increases with d;
//   4. (a third launch) finds keep_until[t] = the first d >= t + w with
//      c(d) < rank(t) by binary search (t stays selected while
//      rank(t) <= c(d)).
// The workspace holds the sort buffers, the ranks, the matrix and the
// cutoff ranks.
constexpr int kRsThreads = 1024;
constexpr int kRsWaves = kRsThreads / 64;
constexpr int kRsLdsWords = 2 * 256 * kRsWaves;  // per-wave digit counts and offsets
// steps of a wave loaded into registers a chunk ahead of their use; a
// wave's step count is a multiple of it, so no load needs a guard (guarded
// loads make the compiler wait for every earlier store before a use)
constexpr int kRsChunk = 8;
constexpr int kRsBatch = 8;  // queries and searches of a thread in flight together

struct RsLayout {
  int n, L, cw, nw;  // ranked tokens, matrix levels, elements per wave, words per level
  long kp0, kp1, rk, v0, v1, wb, wd, zt, cr, stride;  // offsets in 32-bit words
};

__host__ __device__ inline RsLayout rs_layout(int S, int n_sink) {
  RsLayout l;
  l.n = S > n_sink ? S - n_sink : 0;
  l.L = 1;
  while ((1L << l.L) < (long)l.n) ++l.L;
  const int span = kRsThreads * kRsChunk;  // elements of one chunk of steps over the workgroup
  l.cw = (l.n + span - 1) / span * 64 * kRsChunk;  // 16 cw >= n, cw / 64 a multiple of kRsChunk
  l.nw = kRsWaves * l.cw / 32 + 1;                 // one word past the elements
  const long N = (long)kRsWaves * l.cw;
  long o = 0;
  auto take = [&o](long words) {
    const long r = o;
    o += (words + 63) / 64 * 64;
    return r;
  };
  l.kp0 = take(2 * N);
  l.kp1 = take(2 * N);
  l.rk = take(N);
  l.v0 = take(N);
  l.v1 = take(N);
  l.wb = take((long)l.L * l.nw);
  l.wd = take((long)l.L * l.nw);
  l.zt = take(l.L);
  l.cr = take(S);
  l.stride = o;
  return l;
}

// exclusive prefix sum of v over the workgroup, and the total
__device__ uint32_t rs_block_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
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
    uint32_t s2 = lane < kRsWaves ? wsum[lane] : 0u;
#pragma unroll
    for (int off = 1; off < kRsWaves; off <<= 1) {
      const uint32_t y = __shfl_up(s2, off);
      if (lane >= off) s2 += y;
    }
    if (lane < kRsWaves) wsum[kRsWaves + lane] = s2;
  }
  __syncthreads();
  const uint32_t before = wave > 0 ? wsum[kRsWaves + wave - 1] : 0u;
  *total = wsum[2 * kRsWaves - 1];
  __syncthreads();
  return before + x - v;
}

// zeros among the first i elements of a matrix level
__device__ __forceinline__ uint32_t rs_rank0(const uint32_t* bits, const uint32_t* dir, uint32_t i) {
  const uint32_t wi = i >> 5, sh = i & 31u;
  const uint32_t below = sh ? (0xffffffffu >> (32u - sh)) : 0u;
  return dir[wi] + (uint32_t)__popc(~bits[wi] & below);
}

__global__ __launch_bounds__(kRsThreads) void running_topk_long_kernel(
    const float* __restrict__ scores, const float* __restrict__ log_decay,
    int* __restrict__ keep_until, int* __restrict__ cutoff, uint32_t* __restrict__ ws, int Hkv,
    int S, int n_sink, int window, int k) {
  __shared__ uint32_t lds[kRsLdsWords];
  __shared__ uint32_t wsum[2 * kRsWaves];
  const long row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const float lam = log_decay ? log_decay[row % Hkv] : 0.f;
  const float* sc = scores + row * S;
  int* until = keep_until + row * S;
  int* cut = cutoff ? cutoff + row * S : nullptr;
  const RsLayout ly = rs_layout(S, n_sink);
  const int n = ly.n, L = ly.L, nw = ly.nw;
  if (k == 0 || n == 0) {  // no pool ranking: tokens leave with the window
    for (int t = tid; t < S; t += kRsThreads) {
      until[t] = t >= n_sink ? min(S, t + window) : S;
      if (cut) cut[t] = -1;
    }
    return;
  }
  uint32_t* w = ws + row * ly.stride;
  uint2* kp0 = reinterpret_cast<uint2*>(w + ly.kp0);
  uint2* kp1 = reinterpret_cast<uint2*>(w + ly.kp1);
  uint32_t* rk = w + ly.rk;
  uint32_t* v0 = w + ly.v0;
  uint32_t* v1 = w + ly.v1;
  uint32_t* wb = w + ly.wb;
  uint32_t* wd = w + ly.wd;
  uint32_t* zt = w + ly.zt;
  const int steps = ly.cw / 64;  // a multiple of kRsChunk
  const int ebase = wave * ly.cw + lane;  // this lane's element of step m: ebase + 64 m
  const uint64_t lt = (1ull << lane) - 1ull;
  // Runs proc(m, value) over the wave's steps in order, the values of step
  // m loaded by load(m); each chunk's loads go out before the previous
  // chunk is processed.
  auto each = [&](auto load, auto proc) {
    using V = decltype(load(0));
    V cur[kRsChunk], nxt[kRsChunk];
#pragma unroll
    for (int j = 0; j < kRsChunk; ++j) cur[j] = load(j);
    for (int m0 = 0; m0 < steps; m0 += kRsChunk) {
      const int mn = m0 + kRsChunk < steps ? m0 + kRsChunk : m0;  // the last chunk reloads itself
#pragma unroll
      for (int j = 0; j < kRsChunk; ++j) nxt[j] = load(mn + j);
#pragma unroll
      for (int j = 0; j < kRsChunk; ++j) proc(m0 + j, cur[j]);
#pragma unroll
      for (int j = 0; j < kRsChunk; ++j) cur[j] = nxt[j];
    }
  };

  // 1. sort pairs (complemented priority key: ascending = best first;
  //    positions ascending on equal keys); slots past the row sort last
  each([&](int m) {
         const int i = ebase + 64 * m;
         return sc[n_sink + min(i, n - 1)];
       },
       [&](int m, float sg) {
         const int i = ebase + 64 * m;
         const int p = n_sink + i;
         kp0[i] = i < n ? make_uint2(~priority_key(sg, lam, p), (uint32_t)p)
                        : make_uint2(0xffffffffu, 0xffffffffu);
       });
  __syncthreads();
  uint32_t* cnt = lds;                    // [wave][digit] counts
  uint32_t* run = lds + 256 * kRsWaves;   // [wave][digit] running offsets
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 8 * pass;
    const uint2* src = (pass & 1) ? kp1 : kp0;
    uint2* dst = (pass & 1) ? kp0 : kp1;
#pragma unroll
    for (int q = 0; q < 4; ++q) cnt[wave * 256 + 64 * q + lane] = 0u;  // this wave's row
    each([&](int m) { return src[ebase + 64 * m].x; },
         [&](int, uint32_t kx) { atomicAdd(&cnt[wave * 256 + ((kx >> sh) & 255u)], 1u); });
    __syncthreads();
    // exclusive offsets in (digit, wave) order; thread t owns entries 4t..4t+3
    uint32_t e4[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * tid + q;  // digit e / 16, wave e % 16
      e4[q] = cnt[(e % kRsWaves) * 256 + e / kRsWaves];
      tot += e4[q];
    }
    uint32_t total;
    uint32_t at = rs_block_scan(tot, wsum, &total);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e = 4 * tid + q;
      run[(e % kRsWaves) * 256 + e / kRsWaves] = at;
      at += e4[q];
    }
    __syncthreads();
    each([&](int m) { return src[ebase + 64 * m]; },
         [&](int, uint2 e) {
           const uint32_t d = (e.x >> sh) & 255u;
           uint64_t mk = ~0ull;  // lanes of this step with the same digit
#pragma unroll
           for (int b = 0; b < 8; ++b) {
             const uint64_t bb = __ballot((d >> b) & 1u);
             mk &= ((d >> b) & 1u) ? bb : ~bb;
           }
           const uint32_t below = (uint32_t)__popcll(mk & lt);
           const uint32_t off = run[wave * 256 + d];
           dst[off + below] = e;
           if (below == 0) run[wave * 256 + d] = off + (uint32_t)__popcll(mk);
         });
    __syncthreads();
  }
  // four passes end in kp0: index = rank

  // 2. ranks in position order, then the wavelet matrix over them
  each([&](int m) { return kp0[ebase + 64 * m].y; },
       [&](int m, uint32_t p) {
         const int r = ebase + 64 * m;
         if (r < n) rk[p - (uint32_t)n_sink] = (uint32_t)r;
       });
  __syncthreads();
  each([&](int m) { return rk[min(ebase + 64 * m, n - 1)]; },
       [&](int m, uint32_t x) {
         const int i = ebase + 64 * m;
         v0[i] = i < n ? x : 0xffffffffu;
       });
  __syncthreads();
  uint32_t* wz = lds;  // zeros per wave
  for (int lv = 0; lv < L; ++lv) {
    const int bit = L - 1 - lv;
    const uint32_t* src = (lv & 1) ? v1 : v0;
    uint32_t* dst = (lv & 1) ? v0 : v1;
    uint32_t z = 0;
    each([&](int m) { return src[ebase + 64 * m]; },
         [&](int, uint32_t x) { z += (uint32_t)__popcll(~__ballot((x >> bit) & 1u)); });
    if (lane == 0) wz[wave] = z;
    __syncthreads();
    uint32_t zr = 0, Z = 0;
    for (int q = 0; q < kRsWaves; ++q) {
      const uint32_t zq = wz[q];
      zr += q < wave ? zq : 0u;
      Z += zq;
    }
    uint32_t orun = (uint32_t)(wave * ly.cw) - zr;
    uint32_t* bl = wb + (long)lv * nw;
    uint32_t* dl = wd + (long)lv * nw;
    each([&](int m) { return src[ebase + 64 * m]; },
         [&](int m, uint32_t x) {
           const bool one = (x >> bit) & 1u;
           const uint64_t B = __ballot(one);
           // lanes 0..3 write the two bit words and the two zero counts
           const int wi = (wave * ly.cw + 64 * m) >> 5;
           const uint32_t z0 = (uint32_t)__popc(~(uint32_t)B);
           if (lane < 4) {
             uint32_t* tp = lane < 2 ? bl : dl;
             const uint32_t val = lane == 0 ? (uint32_t)B : lane == 1 ? (uint32_t)(B >> 32)
                                : lane == 2 ? zr : zr + z0;
             tp[wi + (lane & 1)] = val;
           }
           if (one) dst[Z + orun + (uint32_t)__popcll(B & lt)] = x;
           else dst[zr + (uint32_t)__popcll(~B & lt)] = x;
           zr += (uint32_t)__popcll(~B);
           orun += (uint32_t)__popcll(B);
         });
    if (tid == 0) {
      bl[nw - 1] = 0xffffffffu;
      dl[nw - 1] = Z;
      zt[lv] = Z;
    }
    __syncthreads();
  }

}

// 3. cutoff ranks (n while the pool holds fewer than k tokens) and the
// cutoff tokens, by one descent of the matrix per query; kRsBatch queries
// of a thread descend together.  Many workgroups per row.
#ifndef KVPOP_RQ_THREADS
#define KVPOP_RQ_THREADS 128
#endif
#ifndef KVPOP_RQ_BATCH
#define KVPOP_RQ_BATCH 2
#endif
constexpr int kRqThreads = KVPOP_RQ_THREADS;
constexpr int kRqBatch = KVPOP_RQ_BATCH;  // queries (searches) of a thread in flight together
__global__ __launch_bounds__(kRqThreads) void running_topk_cut_kernel(
    int* __restrict__ cutoff, uint32_t* __restrict__ ws, int S, int n_sink, int window, int k,
    int blocks_per_row) {
  const long row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - (int)(row * blocks_per_row);
  const RsLayout ly = rs_layout(S, n_sink);
  const int n = ly.n, L = ly.L, nw = ly.nw;
  if (k == 0 || n == 0) return;  // the first kernel wrote the row
  uint32_t* w = ws + row * ly.stride;
  const uint2* kp0 = reinterpret_cast<const uint2*>(w + ly.kp0);
  const uint32_t* B = w + ly.wb;
  const uint32_t* Dd = w + ly.wd;
  const uint32_t* Zt = w + ly.zt;
  uint32_t* cr = w + ly.cr;
  int* cut = cutoff ? cutoff + row * S : nullptr;
  const uint32_t uk = (uint32_t)k;
  const int d0 = blk * kRqThreads * kRqBatch + (int)threadIdx.x;
  uint32_t lo[kRqBatch], hi[kRqBatch], kk[kRqBatch], val[kRqBatch];
  bool act[kRqBatch];
#pragma unroll
  for (int j = 0; j < kRqBatch; ++j) {
    const long d = (long)d0 + (long)j * kRqThreads;
    const long pool = min((long)n, max(0L, d - window - n_sink + 1));
    act[j] = d < S && pool >= (long)uk;
    lo[j] = 0;
    hi[j] = (uint32_t)pool;
    kk[j] = uk;
    val[j] = 0;
  }
  for (int lv = 0; lv < L; ++lv) {
    const uint32_t Z = Zt[lv];
    const uint32_t* Bl = B + (long)lv * nw;
    const uint32_t* Dl = Dd + (long)lv * nw;
#pragma unroll
    for (int j = 0; j < kRqBatch; ++j) {
      const uint32_t zl = rs_rank0(Bl, Dl, lo[j]), zh = rs_rank0(Bl, Dl, hi[j]);
      const uint32_t zc = zh - zl;
      const bool down = kk[j] <= zc;  // the k-th smallest has this bit clear
      kk[j] = down ? kk[j] : kk[j] - zc;
      lo[j] = down ? zl : Z + lo[j] - zl;
      hi[j] = down ? zh : Z + hi[j] - zh;
      val[j] |= down ? 0u : 1u << (L - 1 - lv);
    }
  }
  uint32_t tok[kRqBatch];
#pragma unroll
  for (int j = 0; j < kRqBatch; ++j) tok[j] = kp0[act[j] ? val[j] : 0u].y;
#pragma unroll
  for (int j = 0; j < kRqBatch; ++j) {
    const long d = (long)d0 + (long)j * kRqThreads;
    if (d < S) {
      cr[d] = act[j] ? val[j] : (uint32_t)n;
      if (cut) cut[d] = act[j] ? (int)tok[j] : -1;
    }
  }
}

// 4. keep_until[t] = the first d >= t + w with c(d) < rank(t) (c never
// increases), by binary search; kRqBatch tokens of a thread search together.
__global__ __launch_bounds__(kRqThreads) void running_topk_until_kernel(
    int* __restrict__ keep_until, const uint32_t* __restrict__ ws, int S, int n_sink, int window,
    int k, int blocks_per_row) {
  const long row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - (int)(row * blocks_per_row);
  const RsLayout ly = rs_layout(S, n_sink);
  const int n = ly.n;
  if (k == 0 || n == 0) return;
  const uint32_t* w = ws + row * ly.stride;
  const uint32_t* rk = w + ly.rk;
  const uint32_t* C = w + ly.cr;
  int* until = keep_until + row * S;
  const int t0 = blk * kRqThreads * kRqBatch + (int)threadIdx.x;
  int lo[kRqBatch], hi[kRqBatch];
  uint32_t r[kRqBatch];
#pragma unroll
  for (int j = 0; j < kRqBatch; ++j) {
    const int t = t0 + j * kRqThreads;
    const bool srch = t < S && t >= n_sink && (long)t + window < S;
    r[j] = rk[srch ? t - n_sink : 0];
    lo[j] = srch ? t + window : S;
    hi[j] = S;
  }
  for (int it = 0; it < 32; ++it) {  // intervals below 2^31 close within 31 halvings
    bool more = false;
#pragma unroll
    for (int j = 0; j < kRqBatch; ++j) {
      if (lo[j] < hi[j]) {
        const int mid = (lo[j] + hi[j]) >> 1;
        if (C[mid] >= r[j]) lo[j] = mid + 1;
        else hi[j] = mid;
      }
      more = more || lo[j] < hi[j];
    }
    if (!__any(more)) break;
  }
#pragma unroll
  for (int j = 0; j < kRqBatch; ++j) {
    const int t = t0 + j * kRqThreads;
    if (t < S) until[t] = lo[j];
  }
}

}  // namespace

int running_topk_max_len() { return KVPOP_RT_MAX_LEN; }

size_t running_topk_workspace_bytes(int B, int Hkv, int S, int n_sink) {
  if (S <= KVPOP_RT_LONG_MIN) return 0;
  return (size_t)B * Hkv * (size_t)rs_layout(S, n_sink).stride * sizeof(uint32_t);
}

hipError_t launch_running_topk(int B, int Hkv, int S, int n_sink, int window, int budget,
                               const float* scores, const float* log_decay, int* keep_until,
                               int* cutoff, void* workspace, hipStream_t st) {
  const int k = budget - n_sink - window;
  if (S > KVPOP_RT_LONG_MIN) {
    uint32_t* ws = static_cast<uint32_t*>(workspace);
    const long rows = (long)B * Hkv;
    hipLaunchKernelGGL(running_topk_long_kernel, dim3((unsigned)rows), dim3(kRsThreads), 0, st,
                       scores, log_decay, keep_until, cutoff, ws, Hkv, S, n_sink, window, k);
    const int bpr = (S + kRqThreads * kRqBatch - 1) / (kRqThreads * kRqBatch);
    hipLaunchKernelGGL(running_topk_cut_kernel, dim3((unsigned)(rows * bpr)), dim3(kRqThreads), 0,
                       st, cutoff, ws, S, n_sink, window, k, bpr);
    hipLaunchKernelGGL(running_topk_until_kernel, dim3((unsigned)(rows * bpr)), dim3(kRqThreads), 0,
                       st, keep_until, ws, S, n_sink, window, k, bpr);
    return hipGetLastError();
  }
  const int blocks_per_row = (S + 63) / 64;
  const long grid = (long)B * Hkv * blocks_per_row;
  const int n_chunks = (S - (n_sink & ~63) + 63) / 64;
  auto go = [&](auto kern, int nseg) {
    const int seg_chunks = (n_chunks + nseg - 1) / nseg;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(64 * nseg), 0, st, scores, log_decay,
                       keep_until, cutoff, Hkv, S, n_sink, window, k, blocks_per_row,
                       seg_chunks);
  };
  // the fewest waves per block whose segments hold at most 64 chunks; small
  // launches take more (shorter segments) while that keeps the launch under
  // about four waves per SIMD
  int nseg = n_chunks <= 4 * kRtChunksPerSeg ? 4 : n_chunks <= 8 * kRtChunksPerSeg ? 8 : 16;
  const long waves_cap = 4L * 4 * device_cu_count();
  while (nseg < 16 && grid * nseg * 2 <= waves_cap && n_chunks >= nseg * 4) nseg *= 2;
  if (nseg == 4) go(running_topk_kernel<4, kRtChunksPerSeg>, 4);
  else if (nseg == 8) go(running_topk_kernel<8, kRtChunksPerSeg>, 8);
  else go(running_topk_kernel<16, kRtChunksPerSeg>, 16);
  return hipGetLastError();
}

}  // namespace kvpop

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
// gfx950 mapping
//   * A workgroup owns 64 consecutive tokens (one per lane) of one row; its
//     NSEG waves split the scanned positions [s, S) into NSEG segments of at
//     most 64 chunks of 64 positions (128 chunks for rows past 65536).
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

// chunks of 64 positions per wave at most: 64, or 128 for rows past 65536
// positions (sixteen waves; the chunk counts then take 128 KB of LDS)
constexpr int kRtChunksPerSeg = 64;
constexpr int kRtChunksPerSegLong = 128;

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

}  // namespace

int running_topk_max_len() { return 16 * kRtChunksPerSegLong * 64; }

hipError_t launch_running_topk(int B, int Hkv, int S, int n_sink, int window, int budget,
                               const float* scores, const float* log_decay, int* keep_until,
                               int* cutoff, hipStream_t st) {
  const int k = budget - n_sink - window;
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
  if (n_chunks > 16 * kRtChunksPerSeg) go(running_topk_kernel<16, kRtChunksPerSegLong>, 16);
  else if (nseg == 4) go(running_topk_kernel<4, kRtChunksPerSeg>, 4);
  else if (nseg == 8) go(running_topk_kernel<8, kRtChunksPerSeg>, 8);
  else go(running_topk_kernel<16, kRtChunksPerSeg>, 16);
  return hipGetLastError();
}

}  // namespace kvpop

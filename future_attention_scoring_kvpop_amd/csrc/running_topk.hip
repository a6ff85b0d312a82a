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
//   * A wave owns 64 consecutive tokens (one per lane) and streams the row's
//     priority keys in chunks of 64: lane j loads and ranks token c0+j, and
//     v_readlane hands each key to the whole wave as a scalar operand, so a
//     comparison costs one VALU compare and one add.  The rows are L2-
//     resident (4 bytes per token), so every wave streams its own copy.
//   * "Better" is the retention order: larger order-preserving uint32 key
//     first, the lower position on equal keys.  Keys are stored plus one so
//     that 0 marks positions outside the pool; before position t a token
//     with an equal key ranks first (>=), after it only a larger key does.
//   * A wave stops once every lane has seen its k-th better token.
#include "common.h"
#include "launch.h"

namespace kvpop {
namespace {

constexpr int kRtThreads = 256;  // 4 waves x 64 tokens

__device__ __forceinline__ uint32_t order_key(const float* __restrict__ sc, float lam, int t) {
  // pi = sigma + lambda * t, each operation rounded to fp32: contraction
  // into one FMA (a single rounding) would rank some ties differently
#pragma clang fp contract(off)
  const float age = lam * (float)t;
  const float pi = sc[t] + age;
  return rank_key(pi) + 1u;
}

__global__ __launch_bounds__(kRtThreads) void running_topk_kernel(
    const float* __restrict__ scores, const float* __restrict__ log_decay,
    int* __restrict__ keep_until, int* __restrict__ cutoff, int Hkv, int S, int n_sink,
    int window, int k, int blocks_per_row) {
  const int row = blockIdx.x / blocks_per_row;
  const int blk = blockIdx.x - row * blocks_per_row;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tb = blk * kRtThreads + wave * 64;  // first token of this wave (wave-uniform)
  const int t = tb + lane;
  const float lam = log_decay ? log_decay[row % Hkv] : 0.f;
  const float* sc = scores + (size_t)row * S;
  int* until = keep_until + (size_t)row * S;
  int* cut = cutoff ? cutoff + (size_t)row * S : nullptr;

  // queries whose pool holds fewer than k tokens have no cutoff
  if (cut && t < S) {
    const long first_full = (long)n_sink + k - 1 + window;
    if (k == 0 || (long)t < first_full) cut[t] = -1;
  }
  if (tb >= S) return;

  // tokens that need no scan: sinks, tokens whose window reaches the end
  const bool scan = t < S && t >= n_sink && (long)t + window < S && k > 0;
  const uint32_t kt = scan ? order_key(sc, lam, t) : 0u;
  const uint32_t thr_before = kt, thr_after = kt + 1u;  // kt <= 0xff800001: no wrap
  // cnt = better-ranked tokens seen so far; p_j = the smallest position P
  // such that [s, P] holds j of them (while fewer are seen: one past the
  // last position scanned)
  int cnt = 0;
  const int c_first = n_sink & ~63;
  int p_k = c_first, p_k1 = c_first;

  if (__any(scan)) {
    for (int c0 = c_first; c0 < S; c0 += 64) {
      const int j = c0 + lane;
      const uint32_t kj = (j >= n_sink && j < S) ? order_key(sc, lam, j) : 0u;
      const bool own = c0 <= tb + 63 && c0 + 63 >= tb;  // chunk holds tokens of this wave
      if (!own && __all(!scan || cnt >= k || cnt + 64 < k - 1)) {
        // no lane reaches k-1 or k better tokens inside this chunk: count only
        const uint32_t thr = c0 < tb ? thr_before : thr_after;
#pragma unroll 16
        for (int i = 0; i < 64; ++i) cnt += (uint32_t)__builtin_amdgcn_readlane((int)kj, i) >= thr;
        if (cnt < k - 1) p_k1 = p_k = c0 + 64;
      } else {
#pragma unroll 8
        for (int i = 0; i < 64; ++i) {
          const uint32_t v = (uint32_t)__builtin_amdgcn_readlane((int)kj, i);
          const uint32_t thr = c0 + i < t ? thr_before : thr_after;
          cnt += v >= thr;
          p_k1 = cnt < k - 1 ? c0 + i + 1 : p_k1;
          p_k = cnt < k ? c0 + i + 1 : p_k;
        }
      }
      // every scanning lane has met its k-th better token
      if (!__any(scan && cnt < k)) break;
    }
  }
  if (t >= S) return;
  if (!scan) {
    until[t] = (t >= n_sink && k == 0) ? min(S, t + window) : S;
    return;
  }
  // the k-th better token enters the pool at query p_k + w; none: never
  const long leave = cnt >= k ? (long)p_k + window : (long)S + window;
  const long u = leave > (long)t + window ? leave : (long)t + window;
  until[t] = (int)(u < S ? u : S);
  if (cut) {
    // t is the pool's k-th best once k-1 better tokens are in the pool
    long d0 = k == 1 ? (long)t + window : (cnt >= k - 1 ? (long)p_k1 + window : (long)S);
    if (d0 < (long)t + window) d0 = (long)t + window;
    const long d1 = leave < S ? leave : S;
    for (long d = d0; d < d1; ++d) cut[d] = t;
  }
}

}  // namespace

hipError_t launch_running_topk(int B, int Hkv, int S, int n_sink, int window, int budget,
                               const float* scores, const float* log_decay, int* keep_until,
                               int* cutoff, hipStream_t st) {
  const int k = budget - n_sink - window;
  const int blocks_per_row = (S + kRtThreads - 1) / kRtThreads;
  const long grid = (long)B * Hkv * blocks_per_row;
  hipLaunchKernelGGL(running_topk_kernel, dim3((unsigned)grid), dim3(kRtThreads), 0, st, scores,
                     log_decay, keep_until, cutoff, Hkv, S, n_sink, window, k, blocks_per_row);
  return hipGetLastError();
}

}  // namespace kvpop

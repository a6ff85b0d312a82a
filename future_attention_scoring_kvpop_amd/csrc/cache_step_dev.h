// cache_step_dev.h -- device code of the bounded-cache decode step and the
// headwise MLP scorer, shared by the cache-step kernels and the fused
// decode step.
//
// KVpop summary (arXiv 2607.05061v2):
//   * App. E.2: stateless headwise MLP scorers score each token on its own
//     from cached quantities; here the input is the token's key, and the
//     scorer is W1 (hidden x D), GELU, then a scalar output layer.
//   * Sec. 3 and App. E.4: a token need not be scored when it enters the
//     cache; scoring may be deferred while it sits in the protected window,
//     and the keep-or-drop decision is taken when it leaves the window (at
//     query q the newly eligible token is u = q - w).
//   * App. C.1: the cache holds B = s + w + k entries per head.
//
// gfx950 mapping
//   * The MLP runs on one wave: lane j owns hidden unit j with its W1 row
//     in registers; the key's dwords are spread one per lane and handed to
//     the wave by v_readlane, so each weight costs one FMA and no LDS
//     access; the output layer is a fixed xor butterfly.  The prefix scorer
//     and the decode step share this code, so a key scores the same bits in
//     both.
//   * The decode step of a (b, h) row is one 256-thread workgroup: every
//     global read is issued first, one reduction finds the first empty slot
//     and the worst kept token, one thread takes the decision, and the same
//     threads move the exiting row and write the new row (16 bytes each),
//     so no thread reads global memory another thread of the step wrote.
#pragma once

#include "common.h"

namespace kvpop {
namespace csdev {

constexpr int kThreads = 256;

__device__ __forceinline__ float gelu_erf(float x) {
  return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

// The headwise scorer as one wave holds it: lane j owns hidden unit j
// (its W1 row, b1 and w2 entries); lanes j >= hidden own nothing.
template <int D>
struct ScorerLane {
  float w[D];
  float b, w2;
  bool unit;
};

template <int D>
__device__ __forceinline__ void load_scorer(ScorerLane<D>& sl, const float* __restrict__ w1,
                                            const float* __restrict__ b1,
                                            const float* __restrict__ w2, int h, int hidden,
                                            int lane) {
  sl.unit = lane < hidden;
  const size_t j = (size_t)h * hidden + (sl.unit ? lane : 0);
  const float* wr = w1 + j * D;
#pragma unroll
  for (int cc = 0; cc < D; ++cc) sl.w[cc] = wr[cc];
  sl.b = b1[j];
  sl.w2 = w2[j];
}

// This lane's term of one token's score: a_j = b1_j + sum_c W1[j][c] k_c as
// one FMA chain in c order, then w2_j * GELU(a_j).  kdw: lane i holds dword
// i of the bf16 key (elements 2i, 2i+1); v_readlane hands each dword to the
// whole wave.  Every scorer in this library goes through this function and
// wave_sum, so a key gets the same bits wherever it is scored.
template <int D>
__device__ __forceinline__ float scorer_term(const ScorerLane<D>& sl, uint32_t kdw) {
  float a = sl.b;
#pragma unroll
  for (int c2 = 0; c2 < D / 2; ++c2) {
    const uint32_t u = __builtin_amdgcn_readlane(kdw, c2);
    a = fmaf(sl.w[2 * c2], __uint_as_float(u << 16), a);
    a = fmaf(sl.w[2 * c2 + 1], __uint_as_float(u & 0xffff0000u), a);
  }
  return sl.unit ? fmaf(sl.w2, gelu_erf(a), 0.f) : 0.f;
}

// Sum over the wave by a fixed xor butterfly (every lane gets the same bits).
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = x + __shfl_xor(x, off);
  return x;
}

// Pool slots each thread scans per pass (loaded together, then reduced).
constexpr int kScanPer = 16;
// The bounded-cache decode step of one (b, h) row by one 256-thread
// workgroup; wave 0 holds the scorer when w1 is given.
template <int D>
__device__ __forceinline__ void cache_step_row(
    long row, int n_sink, int window, int budget, int delay, int pos_q,
    const bf16_t* __restrict__ k_new, const bf16_t* __restrict__ v_new,
    const float* __restrict__ w1, const float* __restrict__ b1, const float* __restrict__ w2,
    const float* __restrict__ b2, int hidden, const float* __restrict__ scores_r,
    bf16_t* __restrict__ kc, bf16_t* __restrict__ vc, int32_t* __restrict__ slot_pos,
    float* __restrict__ slot_score, int Hkv) {
  __shared__ int red_empty[kThreads / 64];
  __shared__ int red_slot[kThreads / 64];
  __shared__ uint32_t red_key[kThreads / 64];
  __shared__ int red_pos[kThreads / 64];
  __shared__ int sh_dst;

  const int h = (int)(row % Hkv);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kk = budget - n_sink - window;
  int32_t* sp = slot_pos + row * budget;
  float* ss = slot_score + row * budget;
  bf16_t* kr = kc + row * (size_t)budget * D;
  bf16_t* vr = vc + row * (size_t)budget * D;
  constexpr int cpr = D / 8;
  const int q = pos_q;
  const int u = q - window;               // the token leaving the window
  const bool exiting = u >= n_sink;
  const int ring_u = n_sink + kk + ((u % window) + window) % window;
  const int slot = q < n_sink ? q : n_sink + kk + (q % window);  // where q is written
  const int r = q - delay;                // the token scored at this step
  // no scorer given (neither weights nor a score): nothing is scored here
  const bool scoring = r >= n_sink && (w1 != nullptr || scores_r != nullptr);
  const int rslot = n_sink + kk + ((r % window) + window) % window;
  const bool use_mlp = scoring && w1 != nullptr;

  // ---- every global read first: one memory latency for the whole step ----
  // The loads are unconditional or under wave-uniform conditions (indices
  // clamped into the row), so they all go out before the first wait.
  // Rows: thread i < cpr owns 16-byte chunk i of K, cpr <= i < 2 cpr of V
  // (the other threads load a duplicate and store nothing); the exiting
  // row is read before the same thread overwrites its slot.  ring_u is a
  // ring slot even when no token exits.
  const bool row_thread = tid < 2 * cpr;
  const int rt = tid % (2 * cpr);
  const bool is_k = rt < cpr;
  const int chunk = is_k ? rt : rt - cpr;
  const uint4 old_row = ldg16((is_k ? kr : vr) + (size_t)ring_u * D + chunk * 8);
  const uint4 new_row = ldg16((is_k ? k_new : v_new) + row * D + chunk * 8);
  const int pos_u = sp[ring_u];
  const float score_u = ss[ring_u];
  const float given = scoring && !use_mlp ? scores_r[row] : 0.f;

  // first pass of the long-range scan (up to kThreads * kScanPer slots)
  const bool scan = exiting && kk > 0;
  int pv[kScanPer];
  float sv[kScanPer];
  if (scan) {
#pragma unroll
    for (int i = 0; i < kScanPer; ++i) {
      const int j = min(tid + i * kThreads, kk - 1);
      pv[i] = sp[n_sink + j];
      sv[i] = ss[n_sink + j];
    }
  }

  // wave 0 holds the scorer (its loads go out last: they are needed last)
  const bool wave0 = __builtin_amdgcn_readfirstlane(wave) == 0;
  ScorerLane<D> sl;
  uint32_t kdw = 0;
  if (use_mlp && wave0) {
    load_scorer<D>(sl, w1, b1, w2, h, hidden, lane);
    const bf16_t* ksrc = r == q ? k_new + row * D : kr + (size_t)rslot * D;
    kdw = reinterpret_cast<const uint32_t*>(ksrc)[lane % (D / 2)];
  }

  // ---- (a) scan of the long-range slots: first empty slot, worst kept token
  int first_empty = 0x7fffffff, worst = -1, wpos = 0;
  uint32_t wkey = 0;
  if (exiting) {
    for (int base = 0; base < kk; base += kThreads * kScanPer) {
      if (base > 0) {  // rows longer than one pass
#pragma unroll
        for (int i = 0; i < kScanPer; ++i) {
          const int j = min(base + tid + i * kThreads, kk - 1);
          pv[i] = sp[n_sink + j];
          sv[i] = ss[n_sink + j];
        }
      }
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) {
        const int j = base + tid + i * kThreads;
        if (j >= kk) continue;
        if (pv[i] < 0) {
          first_empty = min(first_empty, n_sink + j);
        } else {
          const uint32_t key = rank_key(sv[i]);
          if (worst < 0 || key < wkey || (key == wkey && pv[i] > wpos)) {
            worst = n_sink + j;
            wkey = key;
            wpos = pv[i];
          }
        }
      }
    }
    // worst = lowest rank key, ties to the later position (positions of kept
    // tokens are distinct, so the order is total)
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      first_empty = min(first_empty, __shfl_xor(first_empty, off));
      const int ow = __shfl_xor(worst, off);
      const uint32_t ok = (uint32_t)__shfl_xor((int)wkey, off);
      const int op = __shfl_xor(wpos, off);
      if (ow >= 0 && (worst < 0 || ok < wkey || (ok == wkey && op > wpos))) {
        worst = ow;
        wkey = ok;
        wpos = op;
      }
    }
    if (lane == 0) {
      red_empty[wave] = first_empty;
      red_slot[wave] = worst;
      red_key[wave] = wkey;
      red_pos[wave] = wpos;
    }
  }
  __syncthreads();

  // ---- decision (one thread): empty slot first, else strict evict-min ----
  if (tid == 0) {
    int dst = -1;
    if (exiting) {
      int fe = 0x7fffffff, wv = -1, wp = 0;
      uint32_t wk = 0;
      for (int w = 0; w < kThreads / 64; ++w) {
        fe = min(fe, red_empty[w]);
        const int cand = red_slot[w];
        if (cand >= 0 && (wv < 0 || red_key[w] < wk || (red_key[w] == wk && red_pos[w] > wp))) {
          wv = cand;
          wk = red_key[w];
          wp = red_pos[w];
        }
      }
      if (fe != 0x7fffffff) {
        dst = fe;
      } else if (wv >= 0) {
        const uint32_t uk = rank_key(score_u);
        if (uk > wk || (uk == wk && u < wp)) dst = wv;
      }
      if (dst >= 0) {
        sp[dst] = pos_u;
        ss[dst] = score_u;
      }
    }
    sh_dst = dst;
    // (b) the new token takes its ring slot, unscored for now
    sp[slot] = q;
    ss[slot] = __uint_as_float(0x7fc00000u);
  }
  __syncthreads();
  const int dst = sh_dst;
  if (row_thread) {
    bf16_t* base = is_k ? kr : vr;
    if (dst >= 0) stg16(base + (size_t)dst * D + chunk * 8, old_row);
    stg16(base + (size_t)slot * D + chunk * 8, new_row);
  }

  // ---- (c) delayed scoring of token r = q - delay ----
  if (scoring && wave == 0) {
    float sc = given;
    if (use_mlp) sc = wave_sum(scorer_term<D>(sl, kdw)) + b2[h];
    if (lane == 0) ss[rslot] = sc;  // after the NaN marker when r == q (same thread)
  }
}

}  // namespace csdev
}  // namespace kvpop

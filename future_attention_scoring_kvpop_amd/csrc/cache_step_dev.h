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
//   * The MLP of one token runs on one wave: lane j owns hidden units j,
//     j+64, ...; W1 is staged through LDS with a padded row so the lane-
//     varying reads are conflict free; the output layer is a fixed xor
//     butterfly, so every kernel that scores a token produces the same bits.
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

// Score of one key by one wave.  key: D floats in LDS; w1s: LDS copy of the
// head's W1 with row stride D+1.  Returns the same value in every lane.
__device__ __forceinline__ float mlp_wave(const float* key, const float* w1s, int D, int hidden,
                                          const float* __restrict__ b1,
                                          const float* __restrict__ w2, float b2, int lane) {
  float part = 0.f;
  for (int j = lane; j < hidden; j += 64) {
    const float* wr = w1s + j * (D + 1);
    float a = b1[j];
    for (int cc = 0; cc < D; ++cc) a = fmaf(wr[cc], key[cc], a);
    part = fmaf(w2[j], gelu_erf(a), part);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) part = part + __shfl_xor(part, off);
  return part + b2;
}

// LDS written by lanes of one wave becomes visible to the other lanes of the
// same wave (no workgroup barrier: waves of a block walk different tokens).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void stage_w1(float* w1s, const float* __restrict__ w1, int D,
                                         int hidden) {
  for (int e = threadIdx.x; e < hidden * D; e += blockDim.x) {
    const int j = e / D, cc = e % D;
    w1s[j * (D + 1) + cc] = w1[e];
  }
}

// Pool slots each thread scans per pass (loaded together, then reduced).
constexpr int kScanPer = 16;
// W1 elements per thread held in registers while staging (hidden * D <= 64 * 128).
constexpr int kW1Per = 64 * 128 / kThreads;

// The bounded-cache decode step of one (b, h) row by one 256-thread
// workgroup.  smem: hidden * (D+1) + D floats of LDS when w1 is given.
__device__ __forceinline__ void cache_step_row(
    long row, float* smem, int D, int n_sink, int window, int budget, int delay, int pos_q,
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
  const int cpr = D / 8;
  const int q = pos_q;
  const int u = q - window;               // the token leaving the window
  const bool exiting = u >= n_sink;
  const int ring_u = n_sink + kk + ((u % window) + window) % window;
  const int slot = q < n_sink ? q : n_sink + kk + (q % window);  // where q is written
  const int r = q - delay;                // the token scored at this step
  const bool scoring = r >= n_sink;
  const int rslot = n_sink + kk + ((r % window) + window) % window;
  const bool use_mlp = scoring && w1 != nullptr;

  // ---- every global read first: one memory latency for the whole step ----
  // rows: thread i < cpr owns 16-byte chunk i of K, cpr <= i < 2 cpr of V;
  // the exiting row is read before the same thread overwrites its slot
  const bool row_thread = tid < 2 * cpr;
  const bool is_k = tid < cpr;
  const int chunk = is_k ? tid : tid - cpr;
  uint4 old_row = make_uint4(0, 0, 0, 0), new_row = make_uint4(0, 0, 0, 0);
  if (row_thread) {
    if (exiting) old_row = ldg16((is_k ? kr : vr) + (size_t)ring_u * D + chunk * 8);
    new_row = ldg16((is_k ? k_new : v_new) + row * D + chunk * 8);
  }
  int pos_u = 0;
  float score_u = 0.f, given = 0.f;
  if (tid == 0) {
    if (exiting) {
      pos_u = sp[ring_u];
      score_u = ss[ring_u];
    }
    if (scoring && !use_mlp) given = scores_r[row];
  }
  float w1v[kW1Per];
  float keyv = 0.f;
  if (use_mlp) {
    const float* w1h = w1 + (size_t)h * hidden * D;
#pragma unroll
    for (int i = 0; i < kW1Per; ++i) {
      const int e = tid + i * kThreads;
      w1v[i] = e < hidden * D ? w1h[e] : 0.f;
    }
    const bf16_t* ksrc = r == q ? k_new + row * D : kr + (size_t)rslot * D;
    if (tid < D) keyv = __uint_as_float((uint32_t)ksrc[tid] << 16);
  }

  // ---- (a) scan of the long-range slots: first empty slot, worst kept token
  int first_empty = 0x7fffffff, worst = -1, wpos = 0;
  uint32_t wkey = 0;
  if (exiting) {
    for (int base = 0; base < kk; base += kThreads * kScanPer) {
      int pv[kScanPer];
      float sv[kScanPer];
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) {
        const int j = base + tid + i * kThreads;
        pv[i] = j < kk ? sp[n_sink + j] : -2;
        sv[i] = j < kk ? ss[n_sink + j] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < kScanPer; ++i) {
        const int j = n_sink + base + tid + i * kThreads;
        if (pv[i] == -2) continue;
        if (pv[i] < 0) {
          first_empty = min(first_empty, j);
        } else {
          const uint32_t key = rank_key(sv[i]);
          if (worst < 0 || key < wkey || (key == wkey && pv[i] > wpos)) {
            worst = j;
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
  float* w1s = smem;                         // hidden x (D+1)
  float* key = smem + (size_t)hidden * (D + 1);
  if (use_mlp) {
#pragma unroll
    for (int i = 0; i < kW1Per; ++i) {
      const int e = tid + i * kThreads;
      if (e < hidden * D) w1s[(e / D) * (D + 1) + e % D] = w1v[i];
    }
    if (tid < D) key[tid] = keyv;
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
    if (use_mlp)
      sc = mlp_wave(key, w1s, D, hidden, b1 + (size_t)h * hidden, w2 + (size_t)h * hidden, b2[h], lane);
    if (lane == 0) ss[rslot] = sc;  // after the NaN marker when r == q (same thread)
  }
}

}  // namespace csdev
}  // namespace kvpop

// decode_dev.h -- device code of GQA decode attention over the bounded
// per-head cache, shared by the decode kernel and the fused decode step.
//
// KVpop summary (arXiv 2607.05061v2), Sec. 3 (attention is computed only
// over the retained set) and App. C.1 (decoding attends directly over the
// retained cache entries).  One query per head; empty slots (slot_pos < 0)
// take no part.
//
// gfx950 mapping (HBM bound: every cache byte is read exactly once per step)
//   * Work item = (b, KV head, slot split).  Each K/V row is read once for
//     all G query heads of its group.
//   * A 16-lane quarter-wave owns one slot row at a time (16 bytes per lane,
//     fully coalesced 256-byte rows); the q.k partial dots are reduced with
//     four DPP adds inside the 16-lane row, so no LDS traffic in the loop.
//   * Softmax in base 2 with the scale folded into q; each quarter-wave keeps
//     an online (max, sum, o) state per head over blocks of 4 slots, and the
//     16 states of a workgroup are merged once through LDS.  The maximum is
//     only taken again (and l, o rescaled) when a block's terms would sum
//     past 2^64: a score a little past it just gives a term above 1.  Splits are
//     merged by a second small kernel with the same log-sum-exp rule.
//   * Each quarter-wave loads the next iteration's K/V rows before it
//     computes the current one, so a wave always has a row block in flight.
//     The loads carry the non-temporal hint (the cache is streamed once per
//     step): 142 -> 158 decode steps/s on the 64-sequence workload.
#pragma once

#include "common.h"

namespace kvpop {
namespace decdev {

constexpr int kThreads = 256;
// 1: the next iteration's K/V rows are loaded before this one is computed
#ifndef KVPOP_DEC_PREFETCH
#define KVPOP_DEC_PREFETCH 1
#endif
constexpr int kNB = 4;                    // slots per quarter-wave per iteration
constexpr int kSlotsPerIter = 16 * kNB;   // per workgroup

// sum over the 16 lanes of a DPP row; every lane receives the same value
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  return x;
}

template <int FPL>
__device__ __forceinline__ void unpack(const uint4& u, float* f);

template <>
__device__ __forceinline__ void unpack<8>(const uint4& u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}
template <>
__device__ __forceinline__ void unpack<4>(const uint4& u, float* f) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
}

// cache rows are read once per step: non-temporal loads (1) or plain (0)
#ifndef KVPOP_DEC_NT
#define KVPOP_DEC_NT 1
#endif

template <int FPL>
__device__ __forceinline__ uint4 load_row_part(const bf16_t* p) {
  if constexpr (FPL == 8) {
    return KVPOP_DEC_NT ? ldg16_nt(p) : ldg16(p);
  } else {
    const uint2 v = *reinterpret_cast<const uint2*>(p);
    return make_uint4(v.x, v.y, 0, 0);
  }
}

// Attention of the G queries of one (b, KV head) over slot split `split`
// by one 256-thread workgroup; with one split the result is final,
// otherwise the split's partial state goes to ws.
template <int D, int GC>
__device__ __forceinline__ void decode_row(
    int bh, int split, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc,
    const bf16_t* __restrict__ vc, const int32_t* __restrict__ slot_pos, float* __restrict__ ws,
    void* __restrict__ o_out, int o_bf16, float* __restrict__ lse_out, int Hq, int Hkv,
    int n_slots, int n_split, int sps, float c) {
  constexpr int FPL = D / 16;
  __shared__ float sm_m[16][GC], sm_l[16][GC];
  __shared__ float sm_o[16][GC][D];

  const int b = bh / Hkv, h = bh % Hkv;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, qw = tid >> 4, ql = tid & 15;
  const int j_begin = split * sps;
  const int j_end = min(n_slots, j_begin + sps);
  const size_t row0 = (size_t)bh * n_slots;

  for (int g0 = 0; g0 < G; g0 += GC) {
    float qv[GC][FPL];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      float t[8];
      unpack<FPL>(load_row_part<FPL>(q + ((size_t)b * Hq + h * G + g0 + g) * D + ql * FPL), t);
#pragma unroll
      for (int f = 0; f < FPL; ++f) qv[g][f] = t[f] * c;
    }
    float m[GC], l[GC], o[GC][FPL];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int f = 0; f < FPL; ++f) o[g][f] = 0.f;
    }

    // rows of iteration jb (prefetched one iteration ahead when enabled)
    uint4 kn[kNB], vn[kNB];
    int pn[kNB];
    auto fetch = [&](int jb) {
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const int j = jb + qw * kNB + i;
        const bool in = j < j_end;
        const size_t off = (row0 + (in ? j : j_begin)) * D + ql * FPL;
        kn[i] = load_row_part<FPL>(kc + off);
        vn[i] = load_row_part<FPL>(vc + off);
        pn[i] = in ? slot_pos[row0 + j] : -1;
      }
    };
    if (KVPOP_DEC_PREFETCH) fetch(j_begin);
    for (int jb = j_begin; jb < j_end; jb += kSlotsPerIter) {
      uint4 kr[kNB], vr[kNB];
      bool ok[kNB];
      if (!KVPOP_DEC_PREFETCH) fetch(jb);
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        kr[i] = kn[i];
        vr[i] = vn[i];
        ok[i] = pn[i] >= 0;
      }
      if (KVPOP_DEC_PREFETCH && jb + kSlotsPerIter < j_end) fetch(jb + kSlotsPerIter);
      float kf[kNB][8], vf[kNB][8];
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        unpack<FPL>(kr[i], kf[i]);
        unpack<FPL>(vr[i], vf[i]);
      }
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float s[kNB];
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
          float d = 0.f;
#pragma unroll
          for (int f = 0; f < FPL; ++f) d = fmaf(qv[g][f], kf[i][f], d);
          d = row16_sum(d);
          s[i] = ok[i] ? d : -INFINITY;
        }
        // Terms relative to the running maximum as it stands; the maximum
        // and the rescaling of l and o are only taken again when some
        // lane's terms would sum past 2^64 or it has no maximum yet (the
        // sum is then inf or NaN).
        float p[kNB], psum = 0.f;
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
          p[i] = fast_exp2(s[i] - m[g]);
          psum += p[i];
        }
        if (!__all(psum <= 0x1p64f)) {
          float mx = m[g];
#pragma unroll
          for (int i = 0; i < kNB; ++i) mx = fmaxf(mx, s[i]);
          const float alpha = mx > -INFINITY ? fast_exp2(m[g] - mx) : 1.f;
          const float ms = mx > -INFINITY ? mx : 0.f;  // masked slots still give 0
          psum = 0.f;
#pragma unroll
          for (int i = 0; i < kNB; ++i) {
            p[i] = fast_exp2(s[i] - ms);
            psum += p[i];
          }
          l[g] *= alpha;
#pragma unroll
          for (int f = 0; f < FPL; ++f) o[g][f] *= alpha;
          m[g] = mx;
        }
        l[g] += psum;
#pragma unroll
        for (int f = 0; f < FPL; ++f) {
          float acc = o[g][f];
#pragma unroll
          for (int i = 0; i < kNB; ++i) acc = fmaf(p[i], vf[i][f], acc);
          o[g][f] = acc;
        }
      }
    }

    // merge the 16 quarter-wave states of this workgroup
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      if (ql == 0) {
        sm_m[qw][g] = m[g];
        sm_l[qw][g] = l[g];
      }
#pragma unroll
      for (int f = 0; f < FPL; ++f) sm_o[qw][g][ql * FPL + f] = o[g][f];
    }
    __syncthreads();
    for (int e = tid; e < GC * D; e += kThreads) {
      const int g = e / D, f = e % D;
      float M = -INFINITY;
      for (int w = 0; w < 16; ++w) M = fmaxf(M, sm_m[w][g]);
      float L = 0.f, O = 0.f;
      if (M > -INFINITY) {
        for (int w = 0; w < 16; ++w) {
          const float mw = sm_m[w][g];
          if (mw == -INFINITY) continue;
          const float sc = fast_exp2(mw - M);
          L = fmaf(sm_l[w][g], sc, L);
          O = fmaf(sm_o[w][g][f], sc, O);
        }
      }
      const int gg = g0 + g;
      if (n_split == 1) {
        const size_t oi = ((size_t)b * Hq + h * G + gg) * D + f;
        const float val = L > 0.f ? O / L : 0.f;
        if (o_bf16) reinterpret_cast<uint16_t*>(o_out)[oi] = f32_to_bf16_rne(val);
        else reinterpret_cast<float*>(o_out)[oi] = val;
        if (f == 0 && lse_out)
          lse_out[(size_t)b * Hq + h * G + gg] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
      } else {
        float* pw = ws + (((size_t)bh * n_split + split) * G + gg) * (D + 2);
        pw[2 + f] = O;
        if (f == 0) {
          pw[0] = M;
          pw[1] = L;
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace decdev
}  // namespace kvpop

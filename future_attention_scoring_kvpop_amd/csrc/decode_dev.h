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
//   * q.k is taken with bf16 dot-product instructions (v_dot2c_f32_bf16:
//     K rows and q stay packed, fp32 accumulation, the scale applied to the
//     sum) and V rows are unpacked one slot at a time, which leaves the
//     registers free (216 for four query heads, two workgroups per CU).
//     Each quarter-wave issues the loads of the next iteration before it
//     computes the current one (two iterations ahead measured the same on
//     the 64-sequence workload: loads in flight are not what bounds it).
//     The loads carry the
//     non-temporal hint (the cache is streamed once per step): 142 -> 158
//     decode steps/s on the 64-sequence workload.
#pragma once

#include <type_traits>

#include "common.h"

namespace kvpop {
namespace decdev {

constexpr int kThreads = 256;
#ifndef KVPOP_DEC_NB
#define KVPOP_DEC_NB 4
#endif
constexpr int kNB = KVPOP_DEC_NB;         // slots per quarter-wave per iteration
constexpr int kSlotsPerIter = 16 * kNB;   // per workgroup
// iterations of K/V rows in flight ahead of the one being computed (1 or 2;
// 2 takes the four-head attention kernel past 256 registers), and the
// register ring that holds them
#ifndef KVPOP_DEC_DEPTH
#define KVPOP_DEC_DEPTH 1
#endif
constexpr int kDepth = KVPOP_DEC_DEPTH;
static_assert(kDepth == 1 || kDepth == 2, "prefetch depth");
constexpr int kRing = kDepth + 1;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

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

// slot positions of a quarter-wave's rows read by one 16-byte load (1)
#ifndef KVPOP_DEC_POS4
#define KVPOP_DEC_POS4 1
#endif
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
    // the group's queries as packed bf16 pairs: q.k is taken by bf16 dot
    // products with fp32 accumulation, and the scale applied to the sum
    uint32_t qp[GC][FPL / 2];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      const uint4 u = load_row_part<FPL>(q + ((size_t)b * Hq + h * G + g0 + g) * D + ql * FPL);
      qp[g][0] = u.x;
      qp[g][1] = u.y;
      if constexpr (FPL == 8) {
        qp[g][2] = u.z;
        qp[g][3] = u.w;
      }
    }
    float m[GC], l[GC], o[GC][FPL];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
      m[g] = -INFINITY;
      l[g] = 0.f;
#pragma unroll
      for (int f = 0; f < FPL; ++f) o[g][f] = 0.f;
    }

    // K/V rows of kDepth iterations in flight: ring slot r % kRing holds
    // iteration r's rows (slots past the split read row j_begin, masked)
    uint4 kb[kRing][kNB], vb[kRing][kNB];
    int pb[kRing][kNB];
    // the quarter-wave's kNB slot positions come as one 16-byte load when
    // they are aligned and inside the split
    const bool pos4 = KVPOP_DEC_POS4 && kNB == 4 && ((row0 + j_begin) & 3) == 0;
    auto fetch = [&](auto R, int jb) {
      constexpr int r = decltype(R)::value;
      const int jq = jb + qw * kNB;
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        const int j = jq + i;
        const bool in = j < j_end;
        const size_t off = (row0 + (in ? j : j_begin)) * D + ql * FPL;
        kb[r][i] = load_row_part<FPL>(kc + off);
        vb[r][i] = load_row_part<FPL>(vc + off);
      }
      if (pos4 && jq + kNB <= j_end) {
        const int4 pv = *reinterpret_cast<const int4*>(slot_pos + row0 + jq);
        pb[r][0] = pv.x;
        pb[r][1] = pv.y;
        pb[r][2] = pv.z;
        pb[r][3] = pv.w;
      } else {
#pragma unroll
        for (int i = 0; i < kNB; ++i) pb[r][i] = jq + i < j_end ? slot_pos[row0 + jq + i] : -1;
      }
    };
    auto bf2 = [](uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); };
    // one iteration on ring slot R: first the loads of the iteration
    // kDepth ahead go out, then this one's rows are consumed
    auto step = [&](auto R, int jb) {
      constexpr int r = decltype(R)::value;
      if (jb + kDepth * kSlotsPerIter < j_end)
        fetch(std::integral_constant<int, (r + kDepth) % kRing>{}, jb + kDepth * kSlotsPerIter);
      float p[GC][kNB];
#pragma unroll
      for (int g = 0; g < GC; ++g) {
        float sc[kNB];
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
          const uint32_t kw[4] = {kb[r][i].x, kb[r][i].y, kb[r][i].z, kb[r][i].w};
          float d = 0.f;
#pragma unroll
          for (int w = 0; w < FPL / 2; ++w) d = __builtin_amdgcn_fdot2_f32_bf16(bf2(qp[g][w]), bf2(kw[w]), d, false);
          d = row16_sum(d) * c;
          sc[i] = pb[r][i] >= 0 ? d : -INFINITY;
        }
        // Terms relative to the running maximum as it stands; the maximum
        // and the rescaling of l and o are only taken again when some
        // lane's terms would sum past 2^64 or it has no maximum yet (the
        // sum is then inf or NaN).
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < kNB; ++i) {
          p[g][i] = fast_exp2(sc[i] - m[g]);
          psum += p[g][i];
        }
        if (!__all(psum <= 0x1p64f)) {
          float mx = m[g];
#pragma unroll
          for (int i = 0; i < kNB; ++i) mx = fmaxf(mx, sc[i]);
          const float alpha = mx > -INFINITY ? fast_exp2(m[g] - mx) : 1.f;
          const float ms = mx > -INFINITY ? mx : 0.f;  // masked slots still give 0
          psum = 0.f;
#pragma unroll
          for (int i = 0; i < kNB; ++i) {
            p[g][i] = fast_exp2(sc[i] - ms);
            psum += p[g][i];
          }
          l[g] *= alpha;
#pragma unroll
          for (int f = 0; f < FPL; ++f) o[g][f] *= alpha;
          m[g] = mx;
        }
        l[g] += psum;
      }
      // o += p v, one V row part unpacked at a time (slot order per output)
#pragma unroll
      for (int i = 0; i < kNB; ++i) {
        float vf[8];
        unpack<FPL>(vb[r][i], vf);
#pragma unroll
        for (int g = 0; g < GC; ++g)
#pragma unroll
          for (int f = 0; f < FPL; ++f) o[g][f] = fmaf(p[g][i], vf[f], o[g][f]);
      }
    };
    using R0 = std::integral_constant<int, 0>;
    using R1 = std::integral_constant<int, 1>;
    using R2 = std::integral_constant<int, 2>;
    fetch(R0{}, j_begin);
    if (kDepth > 1 && j_begin + kSlotsPerIter < j_end) fetch(R1{}, j_begin + kSlotsPerIter);
    for (int jb = j_begin; jb < j_end; jb += kRing * kSlotsPerIter) {
      step(R0{}, jb);
      if (jb + kSlotsPerIter < j_end) step(R1{}, jb + kSlotsPerIter);
      if (kRing > 2 && jb + 2 * kSlotsPerIter < j_end) step(R2{}, jb + 2 * kSlotsPerIter);
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

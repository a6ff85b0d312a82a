// decode.hip -- decode attention launches: the split kernel, the merge of
// split partial states, and the plan that sizes the split (device code in
// decode_dev.h).
#include <atomic>
#include <mutex>

#include "decode_dev.h"
#include "kvpop.h"
#include "launch.h"

namespace kvpop {
namespace {

using decdev::kThreads;
using decdev::kSlotsPerIter;

template <int D, int GC>
__global__ __launch_bounds__(kThreads) void decode_kernel(
    const bf16_t* __restrict__ q, const bf16_t* __restrict__ kc, const bf16_t* __restrict__ vc,
    const int32_t* __restrict__ slot_pos, float* __restrict__ ws, void* __restrict__ o_out,
    int o_bf16, float* __restrict__ lse_out, int Hq, int Hkv, int n_slots, int n_split,
    int sps, float c) {
  decdev::decode_row<D, GC>(blockIdx.x / n_split, blockIdx.x % n_split, q, kc, vc, slot_pos, ws,
                            o_out, o_bf16, lse_out, Hq, Hkv, n_slots, n_split, sps, c);
}

// One workgroup per (b, query head) merges the split partial states
// (max, sum, D features each).  The splits' maxima and scales are reduced
// across the workgroup, so a thread issues its loads for many splits at once
// instead of walking every split twice in sequence: with 32 splits a
// one-thread-per-feature walk was a chain of L2 round trips, most of the
// merge's time.  Thread t sums feature t % D over the splits s with
// s % (kMergeThreads / D) == t / D; the groups are added in LDS.
constexpr int kMergeThreads = 256;
constexpr int kMergeChunk = 1024;  // splits whose scales are held in LDS at a time

__device__ __forceinline__ float block_max_merge(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) r = fmaxf(r, red[w]);
  return r;
}

__device__ __forceinline__ float block_sum_merge(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) r += red[w];
  return r;
}

__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(
    const float* __restrict__ ws, void* __restrict__ o_out, int o_bf16,
    float* __restrict__ lse_out, int Hq, int Hkv, int D, int n_split) {
  __shared__ float scl[kMergeChunk];
  __shared__ float red[kMergeThreads / 64];
  __shared__ float part[kMergeThreads];
  const int bg = blockIdx.x;  // b * Hq + g
  const int b = bg / Hq, g = bg % Hq;
  const int G = Hq / Hkv;
  const int h = g / G, gl = g % G;
  const size_t bh = (size_t)b * Hkv + h;
  const size_t stride = (size_t)G * (D + 2);  // floats from one split's state to the next
  const float* base = ws + (bh * n_split * G + gl) * (D + 2);
  const int tid = threadIdx.x;
  const int ng = kMergeThreads / D, grp = tid / D, f = tid % D;

  float m = -INFINITY;
  for (int sp = tid; sp < n_split; sp += kMergeThreads) m = fmaxf(m, base[sp * stride]);
  const float M = block_max_merge(m, red);
  float L = 0.f, O = 0.f;
  if (M > -INFINITY) {
    for (int c0 = 0; c0 < n_split; c0 += kMergeChunk) {
      const int nc = min(kMergeChunk, n_split - c0);
      __syncthreads();  // the previous chunk's scales are consumed
      for (int j = tid; j < nc; j += kMergeThreads) {
        const float* pw = base + (c0 + j) * stride;
        const float mw = pw[0];
        const float sc = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        scl[j] = sc;
        L = fmaf(pw[1], sc, L);
      }
      __syncthreads();
      if (grp < ng)
        for (int j = grp; j < nc; j += ng) O = fmaf(base[(c0 + j) * stride + 2 + f], scl[j], O);
    }
  }
  L = block_sum_merge(L, red);
  part[tid] = O;
  __syncthreads();
  if (tid < D) {
    float acc = part[tid];
    for (int k = 1; k < ng; ++k) acc += part[tid + k * D];
    const size_t oi = (size_t)bg * D + tid;
    const float val = L > 0.f ? acc / L : 0.f;
    if (o_bf16) reinterpret_cast<uint16_t*>(o_out)[oi] = f32_to_bf16_rne(val);
    else reinterpret_cast<float*>(o_out)[oi] = val;
    if (tid == 0 && lse_out) lse_out[bg] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
  }
}

// Split partials of the allocation-free entry point: a fixed array in device
// memory (each device the library runs on holds its own copy until the
// process ends).  Host code never passes this name to a kernel: the array's
// device address is looked up once per device (noalloc_scratch) and that
// address is what the kernels receive.
static __device__ __align__(256) float scratch[KVPOP_DECODE_NOALLOC_SCRATCH_BYTES / sizeof(float)];

}  // namespace

// rounds of resident workgroups a decode launch is split into
#ifndef KVPOP_DEC_ROUNDS
#define KVPOP_DEC_ROUNDS 1
#endif

// fewest slots a split of the decode attention covers
#ifndef KVPOP_DEC_MIN_SPLIT
#define KVPOP_DEC_MIN_SPLIT 256
#endif

// Resident decode workgroups on the current device for the group size used.
static int decode_slots(int D, int G) {
  static std::atomic<int> cached[64][2][4];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  const int gi = G >= 8 ? 3 : G >= 4 ? 2 : G >= 2 ? 1 : 0;
  std::atomic<int>& slot = cached[dev][D == 128][gi];
  int n = slot.load(std::memory_order_relaxed);
  if (n > 0) return n;
  const void* fn;
  if (D == 128) {
    const void* t[4] = {(const void*)decode_kernel<128, 1>, (const void*)decode_kernel<128, 2>,
                        (const void*)decode_kernel<128, 4>, (const void*)decode_kernel<128, 8>};
    fn = t[gi];
  } else {
    const void* t[4] = {(const void*)decode_kernel<64, 1>, (const void*)decode_kernel<64, 2>,
                        (const void*)decode_kernel<64, 4>, (const void*)decode_kernel<64, 8>};
    fn = t[gi];
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, fn, kThreads, 0) != hipSuccess || nb <= 0) nb = 2;
  n = device_cu_count() * nb;
  slot.store(n, std::memory_order_relaxed);
  return n;
}

DecodePlan plan_decode(const AttnShape& s) {
  DecodePlan p;
  const int units = s.B * s.Hkv;
  const int wgs = KVPOP_DEC_ROUNDS * decode_slots(s.D, s.Hq / s.Hkv);
  int want = (wgs + units - 1) / units;
  const int max_split = (s.S + KVPOP_DEC_MIN_SPLIT - 1) / KVPOP_DEC_MIN_SPLIT;
  p.n_split = want < 1 ? 1 : (want > max_split ? max_split : want);
  if (p.n_split < 1) p.n_split = 1;
  int sps = (s.S + p.n_split - 1) / p.n_split;
  sps = (sps + kSlotsPerIter - 1) / kSlotsPerIter * kSlotsPerIter;
  p.slots_per_split = sps;
  p.n_split = (s.S + sps - 1) / sps;
  const int G = s.Hq / s.Hkv;
  p.workspace_floats = p.n_split > 1 ? (size_t)units * p.n_split * G * (s.D + 2) : 0;
  return p;
}

hipError_t launch_decode(const AttnShape& s, const void* q, const void* kc, const void* vc,
                         const int32_t* slot_pos, void* o, int o_bf16, float* lse,
                         float* workspace, hipStream_t st) {
  const DecodePlan p = plan_decode(s);
  const int G = s.Hq / s.Hkv;
  const float c = s.scale * kLog2e;
  dim3 grid(s.B * s.Hkv * p.n_split), block(kThreads);
  auto* qq = (const bf16_t*)q;
  auto* kk = (const bf16_t*)kc;
  auto* vv = (const bf16_t*)vc;
#define KVPOP_DEC(DD, GG)                                                                        \
  hipLaunchKernelGGL((decode_kernel<DD, GG>), grid, block, 0, st, qq, kk, vv, slot_pos, workspace, \
                     o, o_bf16, lse, s.Hq, s.Hkv, s.S, p.n_split, p.slots_per_split, c)
  const int gc = G >= 8 ? 8 : G;
  if (s.D == 128) {
    switch (gc) {
      case 1: KVPOP_DEC(128, 1); break;
      case 2: KVPOP_DEC(128, 2); break;
      case 4: KVPOP_DEC(128, 4); break;
      default: KVPOP_DEC(128, 8); break;
    }
  } else {
    switch (gc) {
      case 1: KVPOP_DEC(64, 1); break;
      case 2: KVPOP_DEC(64, 2); break;
      case 4: KVPOP_DEC(64, 4); break;
      default: KVPOP_DEC(64, 8); break;
    }
  }
#undef KVPOP_DEC
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_split == 1) return e;
  static_assert(kMergeThreads % 128 == 0, "feature groups for D = 64 and 128");
  hipLaunchKernelGGL(decode_merge_kernel, dim3(s.B * s.Hq), dim3(kMergeThreads), 0, st, workspace,
                     o, o_bf16, lse, s.Hq, s.Hkv, s.D, p.n_split);
  return hipGetLastError();
}

// Device address of this device's scratch array, looked up on the first
// call on each device (with that device current) and kept per device.
static hipError_t noalloc_scratch(float** out) {
  static std::mutex mu;
  static std::atomic<float*> addr[64];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  float* p = addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(mu);
    p = addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* a = nullptr;
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!a) return hipErrorInvalidSymbol;
      p = static_cast<float*>(a);
      addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

size_t decode_noalloc_capacity() { return sizeof(scratch); }

hipError_t launch_decode_noalloc(const AttnShape& s, const void* q, const void* kc, const void* vc,
                                 const int32_t* slot_pos, void* o, int o_bf16, float* lse,
                                 hipStream_t st) {
  float* ws = nullptr;
  hipError_t e = noalloc_scratch(&ws);
  if (e != hipSuccess) return e;
  // every split writes all of its partial states before the merge reads
  // them, so the array needs no clearing between calls
  return launch_decode(s, q, kc, vc, slot_pos, o, o_bf16, lse, ws, st);
}

}  // namespace kvpop

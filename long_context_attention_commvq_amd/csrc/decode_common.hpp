// Device helpers shared by the decode kernels.
#pragma once

#include "commvq_internal.hpp"

namespace commvq {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// Phase e^{i m theta_p} of position m from the 64-bit fixed-point turn count
// F_p = theta_p / (2 pi) * 2^64: the top 32 bits of (m * F_p) mod 2^64 are the
// phase in turns, exact to 2^-32 turn for any m < 2^32.
__device__ __forceinline__ float2 phase_exact(uint32_t m, uint32_t flo, uint32_t fhi) {
  const uint32_t turns = m * fhi + __umulhi(m, flo);
  const float x = (float)(int32_t)turns * 0x1p-31f;  // angle / pi in [-1, 1)
  float s, c;
  sincospif(x, &s, &c);
  return make_float2(c, s);
}

// Wavefront reductions: butterfly over the 16 lanes of a row with DPP moves,
// then the four row results combined through scalar lane reads.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xb1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4e>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<0xb1>(v);
  v += dpp_f<0x4e>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x128>(v);
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
  const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
  return (r0 + r1) + (r2 + r3);
}

// Workspace layout: [counters: B*Hkv uint32, padded to 256 bytes][partials:
// B*Hq*n_chunks*(D+2) floats, each (max, sum, o[D]) of one chunk].
__host__ __device__ inline size_t counter_bytes(int B, int Hkv) {
  return ((size_t)B * Hkv * sizeof(uint32_t) + 255) & ~(size_t)255;
}

// Called by every thread of a workgroup after it stored its chunk partials for
// (b, h). The workgroup that arrives last for (b, h) merges every chunk of its NH
// query heads into `out`, o = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c, and
// re-arms the counter for the next call. `scratch` is LDS the caller no longer
// needs (cap floats); the chunk weights are staged there when they fit.
template <int NTHREADS>
__device__ void merge_if_last(const DecodeArgs& a, int b, int h, int NH, int D, uint32_t* flag_lds,
                              float* scratch, int cap) {
  uint32_t* counters = a.counters;
  // Every lane's partial stores are ordered before lane 0's release increment by
  // the barrier; one agent-scope release per workgroup publishes them all, and
  // only the last workgroup pays an acquire.
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(&counters[b * a.k.Hkv + h], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t last = (prev == (uint32_t)(a.n_chunks - 1)) ? 1u : 0u;
    if (last) __atomic_thread_fence(__ATOMIC_ACQUIRE);
    *flag_lds = last;
  }
  __syncthreads();
  if (*flag_lds == 0u) return;
  const size_t cs = (size_t)(D + 2);
  const size_t pstride = (size_t)a.n_chunks * cs;
  const int nc = a.n_chunks;
  const float* pb = a.part + ((size_t)b * a.Hq + h * NH) * pstride;
  float* outb = a.out + ((size_t)b * a.Hq + h * NH) * D;
  if (2 * NH * nc + 2 * NH <= cap) {
    float* wgt = scratch;               // [NH][nc] chunk maxima, then weights
    float* lsc = scratch + NH * nc;     // [NH][nc] chunk sums
    float* stat = scratch + 2 * NH * nc;  // [NH] max, [NH] total
    for (int i = threadIdx.x; i < NH * nc; i += NTHREADS) {
      const float* pc = pb + (size_t)(i / nc) * pstride + (size_t)(i % nc) * cs;
      wgt[i] = __builtin_nontemporal_load(pc);
      lsc[i] = __builtin_nontemporal_load(pc + 1);
    }
    __syncthreads();
    if ((int)threadIdx.x < NH) {
      float M = -INFINITY;
      for (int c = 0; c < nc; ++c) M = fmaxf(M, wgt[threadIdx.x * nc + c]);
      stat[threadIdx.x] = M;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NH * nc; i += NTHREADS) {
      const float M = stat[i / nc], mc = wgt[i];
      wgt[i] = (M > -INFINITY && mc > -INFINITY) ? __expf(mc - M) : 0.f;
    }
    __syncthreads();
    if ((int)threadIdx.x < NH) {
      float l = 0.f;
      for (int c = 0; c < nc; ++c) l = fmaf(wgt[threadIdx.x * nc + c], lsc[threadIdx.x * nc + c], l);
      stat[NH + threadIdx.x] = l;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NH * D; i += NTHREADS) {
      const int hh = i / D, d = i % D;
      const float* po = pb + (size_t)hh * pstride + 2 + d;
      const float* wh = wgt + hh * nc;
      float acc0 = 0.f, acc1 = 0.f, acc2 = 0.f, acc3 = 0.f;
      int c = 0;
      for (; c + 4 <= nc; c += 4) {
        const float o0 = __builtin_nontemporal_load(po + (size_t)c * cs);
        const float o1 = __builtin_nontemporal_load(po + (size_t)(c + 1) * cs);
        const float o2 = __builtin_nontemporal_load(po + (size_t)(c + 2) * cs);
        const float o3 = __builtin_nontemporal_load(po + (size_t)(c + 3) * cs);
        acc0 = fmaf(wh[c], o0, acc0);
        acc1 = fmaf(wh[c + 1], o1, acc1);
        acc2 = fmaf(wh[c + 2], o2, acc2);
        acc3 = fmaf(wh[c + 3], o3, acc3);
      }
      for (; c < nc; ++c) acc0 = fmaf(wh[c], __builtin_nontemporal_load(po + (size_t)c * cs), acc0);
      const float l = stat[NH + hh];
      outb[(size_t)hh * D + d] = l > 0.f ? ((acc0 + acc1) + (acc2 + acc3)) / l : 0.f;
    }
  } else {
    for (int i = threadIdx.x; i < NH * D; i += NTHREADS) {
      const int hh = i / D, d = i % D;
      const float* pr = pb + (size_t)hh * pstride;
      float M = -INFINITY;
      for (int c = 0; c < nc; ++c) M = fmaxf(M, __builtin_nontemporal_load(pr + (size_t)c * cs));
      float acc = 0.f, lsum = 0.f;
      if (M > -INFINITY) {
        for (int c = 0; c < nc; ++c) {
          const float* pc = pr + (size_t)c * cs;
          const float mc = __builtin_nontemporal_load(pc);
          if (mc > -INFINITY) {
            const float w = __expf(mc - M);
            lsum = fmaf(w, __builtin_nontemporal_load(pc + 1), lsum);
            acc = fmaf(w, __builtin_nontemporal_load(pc + 2 + d), acc);
          }
        }
      }
      outb[(size_t)hh * D + d] = lsum > 0.f ? acc / lsum : 0.f;
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(&counters[b * a.k.Hkv + h], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace commvq

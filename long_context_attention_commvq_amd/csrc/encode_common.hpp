// Greedy residual search of one group by one wavefront, shared by the kernels
// that encode few tokens (append, the generic and two-round decode steps):
// squared distance accumulated term by term in float32 with fmaf, lowest index
// on ties ("Pith review of CommVQ", "What carries the argument": one index
// shared by a group, R residual rounds). This is the fp32 bulk encoder's
// arithmetic; the matrix-core encoder and the one-round fused decode step rank
// entries by |c|^2/2 - e.c instead, so the paths can differ at near ties only
// (the tests accept a differing code only when its float64 distance is within
// 1e-5 relative of the minimum).
#pragma once

#include "commvq_internal.hpp"

namespace commvq {

// e: the group's g scalars (the running residual, updated in place);
// cbg: the group's [R][Nc][GS] fp16 entries. Every lane of the wavefront calls
// this with the same e; lane 0 stores round r's pick at out[r * out_stride].
template <int GS>
__device__ __forceinline__ void greedy_group_wave(float (&e)[GS], const _Float16* cbg, int Nc, int R, int lane,
                                                  uint8_t* out, int out_stride) {
  for (int r = 0; r < R; ++r) {
    const _Float16* c = cbg + (size_t)r * Nc * GS;
    float best = INFINITY;
    int bi = 0x7fffffff;
    for (int l = lane; l < Nc; l += 64) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < GS; ++i) {
        const float df = e[i] - (float)c[l * GS + i];
        d = fmaf(df, df, d);
      }
      if (d < best) {
        best = d;
        bi = l;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float od = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (od < best || (od == best && oi < bi)) {
        best = od;
        bi = oi;
      }
    }
    if (bi == 0x7fffffff) bi = 0;  // no distance below +inf (a NaN or infinite input): entry 0
#pragma unroll
    for (int i = 0; i < GS; ++i) e[i] -= (float)c[bi * GS + i];
    if (lane == 0) out[r * out_stride] = (uint8_t)bi;
  }
}

// The same search with 16 lanes per group (four groups per wavefront, one per
// 16-lane row), g = 8, Nc <= 256: each lane takes entries lane16 + 16 k. Used
// where every group of a token is searched at once (the fused decode step).
__device__ __forceinline__ void greedy_group_row16(float (&e)[8], const _Float16* cbg, int Nc, int R, int lane16,
                                                   uint8_t* out, int out_stride) {
  // An entry is read as one 16-byte vector of eight fp16 values and indexed
  // directly; the vector's halves are never re-split through 32-bit words.
  typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
  for (int r = 0; r < R; ++r) {
    const _Float16* c = cbg + (size_t)r * Nc * 8;
    float best = INFINITY;
    int bi = 0x7fffffff;
    h8_t ent[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int l = lane16 + 16 * k;
      ent[k] = l < Nc ? *reinterpret_cast<const h8_t*>(c + (size_t)l * 8) : h8_t{};
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int l = lane16 + 16 * k;
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float df = e[i] - (float)ent[k][i];
        d = fmaf(df, df, d);
      }
      if (l < Nc && d < best) {
        best = d;
        bi = l;
      }
    }
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) {
      const float od = __shfl_xor(best, o, 16);
      const int oi = __shfl_xor(bi, o, 16);
      if (od < best || (od == best && oi < bi)) {
        best = od;
        bi = oi;
      }
    }
    if (bi == 0x7fffffff) bi = 0;  // no distance below +inf (a NaN or infinite input): entry 0
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] -= (float)c[bi * 8 + i];
    if (lane16 == 0) out[r * out_stride] = (uint8_t)bi;
  }
}

}  // namespace commvq

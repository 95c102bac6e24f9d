// CommVQ decode attention on packed codes (any supported shape).
//
// Per workgroup: one (sequence b, KV head h, context chunk). For the NH query
// heads that read KV head h:
//   1. rotate q to its position and, for each (group j, round r), build the
//      query x codebook table T[a][l][p] = conj(q~_{a,p}) * z_{j,r,l,p} in LDS
//      ("Pith review of CommVQ", "What carries the argument": the query- and
//      codebook-dependent factors are computed once and reused for every
//      cached position);
//   2. every cached position m gathers T at its code and adds
//      Re(T * e^{i m theta_p}) to the score - the RoPE rotation of the key is a
//      phase because the codebook blocks commute with the rotation (paper Eq. 7);
//   3. softmax over the chunk (max and sum reduced across the workgroup);
//   4. the weights are scattered into per-code histograms (LDS integer atomics on
//      fixed-point weights) and the histograms are multiplied by the value
//      codebook (review, "If this is right", fourth bullet);
//   5. the chunk's (max, sum, unnormalised output) go to the workspace; a second
//      kernel (decode_merge_kernel) combines the chunks of each (b, query head).
// This kernel keeps the table in fp32; position phases come from the hardware
// sine and cosine of the exact turn count, or from sincospi of it in the
// exact-precision mode (a.exact_phase). It serves every supported shape.
// Positions' phases come from 64-bit fixed-point turn counts, exact for any
// position below 2^31.

#include <type_traits>

#include "decode_common.hpp"

namespace commvq {
namespace {

constexpr int kGenericChunk = 1024;  // positions per workgroup of the generic kernel
constexpr int kWideGroup = 32;  // group sizes from which keys are rebuilt per slice instead of tabled
// lanes per workgroup: 1024 (one position each) for wide groups and up to 4
// query heads per KV head, else 512 (two positions each; 8 query heads do not
// fit 128 registers per lane, and the table path measured slower at 1024)
__host__ __device__ constexpr int generic_threads(int nh, int gs) { return (gs >= kWideGroup && nh <= 4) ? 1024 : 512; }
constexpr int kHistShift = 20;  // fixed-point weights: w * 2^20 (chunk <= 1024 keeps sums < 2^31)
constexpr int kBitSub = 128;    // binary value codes: positions whose bit rows are staged in LDS at a time

// acc + the fp16 in the low (high) half of w, in one v_fma_mix_f32 (the
// conversion is exact and the product by 1 too: one rounding, as a convert
// then an fp32 add)
__device__ __forceinline__ float add_f16_lo(float acc, uint32_t w) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
  return acc;
}
__device__ __forceinline__ float add_f16_hi(float acc, uint32_t w) {
  asm("v_fma_mix_f32 %0, %1, 1.0, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w));
  return acc;
}

typedef __attribute__((address_space(3))) void lds_void_t;

// acc + x * (the fp16 in the low / high half of w), one v_fma_mix_f32 (exact
// conversion, one rounding: the same result as fmaf(x, (float)half, acc))
__device__ __forceinline__ float fma_f16_lo(float acc, uint32_t w, float x) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w), "v"(x));
  return acc;
}
__device__ __forceinline__ float fma_f16_hi(float acc, uint32_t w, float x) {
  asm("v_fma_mix_f32 %0, %1, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "+v"(acc) : "v"(w), "v"(x));
  return acc;
}

__device__ __forceinline__ int read_field(const uint8_t* rec, int f, int bits) {
  const int o = f * bits, byte = o >> 3, sh = o & 7;
  uint32_t v = rec[byte];
  if (sh + bits > 8) v |= (uint32_t)rec[byte + 1] << 8;
  return (int)((v >> sh) & ((1u << bits) - 1u));
}

// Value rounds per histogram pass of the generic kernel: all R where NH x R x Nc'
// bins fit in the LDS the key table (or slice) already takes, else 1.
__host__ __device__ inline int generic_hist_rounds(const CbShape& k, const CbShape& v, int NH) {
  const size_t table = k.g >= kWideGroup ? (size_t)k.R * k.Nc * 32 * 2 : (size_t)NH * k.Nc * (k.g / 2) * 8;
  return (size_t)NH * v.R * v.Nc * 4 <= table ? v.R : 1;
}

// Bytes of the region that holds the query x codebook table (or one slice of
// every round's entries, for wide groups) and, later, the value histograms.
__host__ __device__ inline size_t generic_uni_bytes(const CbShape& k, const CbShape& v, int NH) {
  const size_t table_bytes = k.g >= kWideGroup ? (size_t)k.R * k.Nc * 32 * sizeof(_Float16)  // one slice, all rounds
                                               : (size_t)NH * k.Nc * (k.g / 2) * sizeof(float2);
  const size_t hist_bytes = (size_t)NH * generic_hist_rounds(k, v, NH) * v.Nc * sizeof(uint32_t);
  return ((table_bytes > hist_bytes ? table_bytes : hist_bytes) + 15) / 16 * 16;
}

// Wide groups re-read every position's record once per (group, slice) and per
// value pass, one field per round: with records of at most 32 bytes the chunk's
// key and value records are copied to LDS once, so those reads wait on LDS
// instead of on memory.
// (only where they fit the LDS beside the rest)
__host__ __device__ inline size_t generic_base_fixed_bytes(const CbShape& k, int NH) {
  // rotated queries (float2 per pair), output accumulators, reductions
  const int P = k.D / 2, NW = generic_threads(NH, k.g) / 64;
  return (2 * NH * P + NH * k.D + ((NH * (NW > 2 ? NW : 2) + 2 * NH + 4) & ~3)) * sizeof(float);
}
// Wide groups with four query heads per KV head and D = 128 take their dot
// products on the matrix cores (phase split: the wavefront's block phase in the
// query, a lane-constant phase on the rebuilt key), with a table of the lane
// phases e^{i d theta_p}, d < 64, in LDS beside the staged slice, where it fits.
constexpr int kLanePhaseBytes = 64 * 64 * 8;  // [64 offsets][64 pairs] float2
// (never at the cost of the record staging below: that measured the larger gain)
__host__ __device__ inline bool generic_wide_mfma(const CbShape& k, const CbShape& v, int NH) {
  const size_t base = generic_base_fixed_bytes(k, NH) + generic_uni_bytes(k, v, NH);
  const bool stageable = k.bpt <= 32 && v.bpt <= 32 && base + (size_t)kGenericChunk * (k.bpt + v.bpt) <= 160 * 1024;
  return k.g >= kWideGroup && NH == 4 && k.D == 128 &&
         base + kLanePhaseBytes + (stageable ? (size_t)kGenericChunk * (k.bpt + v.bpt) : 0) <= 160 * 1024;
}
__host__ __device__ inline size_t generic_fixed_bytes(const CbShape& k, const CbShape& v, int NH) {
  return generic_base_fixed_bytes(k, NH) + (generic_wide_mfma(k, v, NH) ? kLanePhaseBytes : 0);
}
__host__ __device__ inline bool generic_stage_records(const CbShape& k, const CbShape& v, int NH) {
  return k.g >= kWideGroup && k.bpt <= 32 && v.bpt <= 32 &&
         generic_fixed_bytes(k, v, NH) + generic_uni_bytes(k, v, NH) + (size_t)kGenericChunk * (k.bpt + v.bpt) <=
             160 * 1024;
}
__host__ __device__ inline size_t generic_rec_bytes(const CbShape& k, const CbShape& v, int NH) {
  return generic_stage_records(k, v, NH) ? (size_t)kGenericChunk * (k.bpt + v.bpt) : 0;
}
// Wide groups on the matrix-core score path: a second slice buffer where it fits
// after everything else, so that the next slice is copied (straight into LDS)
// while the current one is used.
__host__ __device__ inline size_t generic_slice_bytes(const CbShape& k) { return (size_t)k.R * k.Nc * 32 * sizeof(_Float16); }
__host__ __device__ inline bool generic_dbl_slice(const CbShape& k, const CbShape& v, int NH) {
  return generic_wide_mfma(k, v, NH) && generic_fixed_bytes(k, v, NH) + generic_uni_bytes(k, v, NH) +
                                            generic_rec_bytes(k, v, NH) + generic_slice_bytes(k) <= 160 * 1024;
}

// n bytes from global memory to LDS, eight loads in flight per lane
template <int T>
__device__ __forceinline__ void copy_bytes(uint8_t* dst, const uint8_t* src, int n, int tid) {
  for (int i0 = 0; i0 < n; i0 += T * 8) {
    uint8_t tmp[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * T + tid;
      tmp[u] = i < n ? src[i] : (uint8_t)0;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * T + tid;
      if (i < n) dst[i] = tmp[u];
    }
  }
}

template <int NH, int GS, bool BITV>
__global__ __launch_bounds__(generic_threads(NH, GS)) void decode_generic_kernel(DecodeArgs a, PhaseTable ph) {
  constexpr int kThreads = generic_threads(NH, GS);
  constexpr int PP = GS / 2;
  constexpr int TPT = kGenericChunk / kThreads;
  constexpr int NW = kThreads / 64;
  extern __shared__ float4 dec_smem4[];
  float* sm = reinterpret_cast<float*>(dec_smem4);
  const CbShape K = a.k, V = a.v;
  const int D = K.D, P = D / 2, G = K.G;
  // KV head fastest in launch order: one head's chunks share an XCD's L2 (8 heads)
  const int h = blockIdx.x % a.k.Hkv, chunk_id = blockIdx.x / a.k.Hkv, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int m0 = chunk_id * a.chunk;
  const int hq0 = h * NH;
  const int red_floats = (NH * (NW > 2 ? NW : 2) + 2 * NH + 4) & ~3;
  const size_t pstride = (size_t)a.n_chunks * (D + 2);
  float* part = a.part + ((size_t)b * a.Hq + hq0) * pstride + (size_t)chunk_id * (D + 2);
  if (m0 >= L) {
    for (int i = tid; i < NH * (D + 2); i += kThreads) {
      const int hh = i / (D + 2), k = i % (D + 2);
      part[hh * pstride + k] = (k == 0) ? -INFINITY : 0.f;
    }
    return;
  }
  float2* qz = reinterpret_cast<float2*>(sm);  // [NH][P]
  float* oacc = sm + 2 * NH * P;               // [NH][D]
  float* red = oacc + NH * D;                  // [NH][NW]
  const bool wide_mfma = GS >= kWideGroup && NH == 4 && generic_wide_mfma(K, V, NH);
  float2* lph = reinterpret_cast<float2*>(red + red_floats);  // lane phases (wide_mfma)
  float* uni = red + red_floats + (wide_mfma ? kLanePhaseBytes / 4 : 0);  // table or histogram
  float2* table = reinterpret_cast<float2*>(uni);
  uint32_t* hist = reinterpret_cast<uint32_t*>(uni);

  const uint32_t qp = (uint32_t)max(a.q_pos[b], 0);
  for (int i = tid; i < NH * P; i += kThreads) {
    const int hh = i / P, p = i % P;
    const float* qrow = a.q + ((size_t)b * a.Hq + hq0 + hh) * D;
    const float x = qrow[2 * p], y = qrow[2 * p + 1];
    const float2 w = phase_exact(qp, ph.lo[p], ph.hi[p]);
    qz[i] = make_float2(x * w.x - y * w.y, x * w.y + y * w.x);
  }
  for (int i = tid; i < NH * D; i += kThreads) oacc[i] = 0.f;

  float s[TPT][NH];
#pragma unroll
  for (int t = 0; t < TPT; ++t)
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) s[t][hh] = 0.f;

  const uint8_t* kbase = a.kcodes + ((size_t)b * K.Hkv + h) * (size_t)a.cache_len * K.bpt;
  const uint8_t* vbase = a.vcodes + ((size_t)b * V.Hkv + h) * (size_t)a.cache_len * V.bpt;
  // the chunk's records in LDS (positions present in the cache only), after
  // the table region; the scores' first staging barrier orders these writes
  const bool staged = GS >= kWideGroup && generic_stage_records(K, V, NH);
  uint8_t* krl = reinterpret_cast<uint8_t*>(uni) + generic_uni_bytes(K, V, NH);
  uint8_t* vrl = krl + (size_t)kGenericChunk * K.bpt;
  if (staged) {
    const int n = min(a.chunk, a.cache_len - m0);
    copy_bytes<kThreads>(krl, kbase + (size_t)m0 * K.bpt, n * K.bpt, tid);
    if constexpr (!BITV) copy_bytes<kThreads>(vrl, vbase + (size_t)m0 * V.bpt, n * V.bpt, tid);
  }
  auto kfield = [&](int m, int f) {
    return staged ? read_field(krl + (size_t)(m - m0) * K.bpt, f, K.bits) : read_field(kbase + (size_t)m * K.bpt, f, K.bits);
  };
  auto vfield = [&](int m, int f) {
    return staged ? read_field(vrl + (size_t)(m - m0) * V.bpt, f, V.bits) : read_field(vbase + (size_t)m * V.bpt, f, V.bits);
  };

  // scores; the position phases are exact (sincospi of the exact turn count)
  // under COMMVQ_DECODE_EXACT, else from the hardware sine and cosine (turns)
  auto scores = [&](auto exc) {
    constexpr bool EX = decltype(exc)::value;
    if constexpr (GS >= kWideGroup) {
      // Wide groups (many pairs share an index): the key itself is rebuilt per
      // 32-scalar slice of a group - every round's entries of the slice staged in
      // LDS as fp16, summed in fp32 over the rounds - then rotated once per pair
      // and dotted with the rotated queries. A query x codebook table per (group,
      // round) would cost a phase and NH products per pair and round instead.
      constexpr int SL = 32, SP = SL / 2;
      // [R][Nc][SL]: entry e's 16-byte chunk v at chunk slot 4 e + ((v + e / 4) & 3),
      // so that lanes reading chunk v of different entries spread over the banks
      _Float16* cbs = reinterpret_cast<_Float16*>(uni);
      auto stage_slice = [&](int j, int sl) {
        __syncthreads();
        const _Float16* src = a.kcb + ((size_t)h * G + j) * K.R * K.Nc * GS + sl * SL;  // entry (r, l) at (r Nc + l) GS
        // four 16-byte loads in flight per lane
        const int nv = K.R * K.Nc * (SL / 8);
        for (int i0 = 0; i0 < nv; i0 += 4 * kThreads) {
          uint4 w[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads + tid;
            w[u] = i < nv ? *reinterpret_cast<const uint4*>(src + (size_t)(i / (SL / 8)) * GS + (i % (SL / 8)) * 8)
                          : make_uint4(0u, 0u, 0u, 0u);
          }
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int i = i0 + u * kThreads + tid, e = i / (SL / 8);
            if (i < nv) reinterpret_cast<uint4*>(cbs)[e * 4 + ((i + (e >> 2)) & 3)] = w[u];
          }
        }
        __syncthreads();
      };
      // kx[0 .. SL) += every round's entry of group j's staged slice at m's codes
      auto rebuild = [&](int m, int j, float (&kx)[SL], const _Float16* slice) {
        // each round's field is read during the previous round's additions
        int code_next = kfield(m, j);
        for (int r = 0; r < K.R; ++r) {
          const int code = code_next;
          if (r + 1 < K.R) code_next = kfield(m, (r + 1) * G + j);
          const int ei = r * K.Nc + code;
          const uint4* e = reinterpret_cast<const uint4*>(slice) + ei * 4;
#pragma unroll
          for (int v = 0; v < SL / 8; ++v) {
            const uint4 w = e[(v + (ei >> 2)) & 3];
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              kx[8 * v + 2 * u] = add_f16_lo(kx[8 * v + 2 * u], wd[u]);
              kx[8 * v + 2 * u + 1] = add_f16_hi(kx[8 * v + 2 * u + 1], wd[u]);
            }
          }
        }
      };
      // the slice copied straight into LDS (global_load_lds: lane l of a wavefront
      // writes 16-byte slot base + l), each slot loading the (entry, chunk) the
      // swizzled layout puts there; the caller waits (vmcnt) and synchronises
      auto stage_async = [&](int j, int sl, _Float16* dst) {
        const _Float16* src = a.kcb + ((size_t)h * G + j) * K.R * K.Nc * GS + sl * SL;
        const int nv = K.R * K.Nc * (SL / 8);
        for (int i0 = 0; i0 < nv; i0 += kThreads) {
          const int sig = i0 + tid;
          if (sig < nv) {
            const int e = sig >> 2, v = ((sig & 3) - (e >> 2)) & 3;
            __builtin_amdgcn_global_load_lds(src + (size_t)e * GS + v * 8,
                                             (lds_void_t*)(reinterpret_cast<uint4*>(dst) + i0 + 64 * wave), 16, 0, 0);
          }
        }
      };
      if constexpr (NH == 4 && !EX) {
        if (wide_mfma) {
          // Phase split (D = 128, one position per lane, m = m_b + d with m_b =
          // m0 + 64 w): s_m = Re sum_p conj(q~_p e^{-i m_b theta_p}) (k_p e^{i d theta_p}),
          // a real dot product over D between the wavefront's block-rotated query q'
          // and the rebuilt key rotated by lane-constant phases, on
          // v_mfma_f32_4x4x1f32: block b takes positions 4b..4b+3 of the wavefront
          // as columns and the four query heads as rows; K-step k (dimension k)
          // broadcasts block k % 16's A, so lane (block bq, row qi) holds head qi's
          // q' for dimensions bq + 16 t only. fp32 operands and sums throughout.
          // Lane phase table: chunk c (pairs 2c, 2c + 1) of row d at slot (c + d) & 31,
          // so that the 64 lanes reading chunk c of their own rows spread over the banks.
          const bool dbl = generic_dbl_slice(K, V, NH);
          _Float16* cbs2 = reinterpret_cast<_Float16*>(reinterpret_cast<uint8_t*>(uni) + generic_uni_bytes(K, V, NH) +
                                                       generic_rec_bytes(K, V, NH));
          if (dbl) stage_async(0, 0, cbs);  // (first slice in flight while the lane phases are built)
          for (int i = tid; i < 64 * 64; i += kThreads) {
            const int d = i >> 6, p = i & 63;
            lph[d * 64 + ((((p >> 1) + d) & 31) << 1) + (p & 1)] = phase_hw((uint32_t)d, ph.lo[p], ph.hi[p]);
          }
          if (dbl) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();  // (the rotated query too)
          const int qi = lane & 3, bq = lane >> 2;
          const uint32_t mb = (uint32_t)(m0 + 64 * wave);
          float qa[8];
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            const int k = bq + 16 * t, p = k >> 1;
            const float2 q0 = qz[qi * P + p];
            const float2 eb = phase_hw(mb, ph.lo[p], ph.hi[p]);
            qa[t] = (k & 1) ? fmaf(q0.y, eb.x, -q0.x * eb.y) : fmaf(q0.x, eb.x, q0.y * eb.y);
          }
          // every lane takes part in the products (a lane past the cache reads the
          // last record; positions past the sequence are masked after the scores)
          const int mr = min(m0 + tid, a.cache_len - 1);
          const float4* lph4 = reinterpret_cast<const float4*>(lph) + lane * 32;
          float4_t acc = {0.f, 0.f, 0.f, 0.f};
          constexpr int SPG = GS / SL;  // slices per group
          static_assert(GS % SL == 0 && (128 / GS) * SPG == 4, "four slices of D = 128");
          static_for<4>([&](auto sc) __attribute__((always_inline)) {
            constexpr int sI = decltype(sc)::value, j = sI / SPG, sl = sI % SPG;
            _Float16* cur = (dbl && (sI & 1)) ? cbs2 : cbs;
            if (dbl) {
              // the next slice into the other buffer (read by no wavefront since the
              // previous slice's closing barrier)
              if constexpr (sI + 1 < 4) stage_async((sI + 1) / SPG, (sI + 1) % SPG, (sI & 1) ? cbs : cbs2);
            } else {
              stage_slice(j, sl);
            }
            float kx[SL];
#pragma unroll
            for (int i = 0; i < SL; ++i) kx[i] = 0.f;
            rebuild(mr, j, kx, cur);
            static_for<SP / 2>([&](auto cc) __attribute__((always_inline)) {
              constexpr int c = decltype(cc)::value, p0 = j * PP + sl * SP + 2 * c;  // pairs p0, p0 + 1
              const float4 e2 = lph4[((p0 >> 1) + lane) & 31];
              const float ex[2] = {e2.x, e2.z}, ey[2] = {e2.y, e2.w};
              float kr[4];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const float x = kx[4 * c + 2 * u], y = kx[4 * c + 2 * u + 1];
                kr[2 * u] = x * ex[u] - y * ey[u];
                kr[2 * u + 1] = fmaf(x, ey[u], y * ex[u]);
              }
              // the wait takes the four values as operands: every product is issued
              // at least eight wait states after their last write
              asm volatile("s_nop 7" : "+v"(kr[0]), "+v"(kr[1]), "+v"(kr[2]), "+v"(kr[3]));
              static_for<4>([&](auto ic) __attribute__((always_inline)) {
                constexpr int i = decltype(ic)::value, k = 2 * p0 + i;
                acc = __builtin_amdgcn_mfma_f32_4x4x1f32(qa[k >> 4], kr[i], acc, 4, k & 15, 0);
              });
            });
            if (dbl) {
              // the next slice has landed (the compiler does not track these LDS
              // writes) and every wavefront is done with this one
              asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
              __syncthreads();
            }
          });
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) s[0][hh] = acc[hh];
          return;
        }
      }
      for (int j = 0; j < G; ++j) {
        for (int sl = 0; sl < GS / SL; ++sl) {
          stage_slice(j, sl);
#pragma unroll
          for (int t = 0; t < TPT; ++t) {  // (unrolled: s[t] stays in registers)
            const int m = m0 + tid + kThreads * t;
            if (m < L) {
              float kx[SL];
  #pragma unroll
              for (int i = 0; i < SL; ++i) kx[i] = 0.f;
              rebuild(m, j, kx, cbs);
  #pragma unroll
              for (int pp = 0; pp < SP; ++pp) {
                const int p = j * PP + sl * SP + pp;
                const float2 w = (EX ? phase_exact((uint32_t)m, ph.lo[p], ph.hi[p]) : phase_hw((uint32_t)m, ph.lo[p], ph.hi[p]));
                const float rx = kx[2 * pp] * w.x - kx[2 * pp + 1] * w.y, ry = kx[2 * pp] * w.y + kx[2 * pp + 1] * w.x;
  #pragma unroll
                for (int hh = 0; hh < NH; ++hh) {
                  const float2 qv = qz[hh * P + p];
                  s[t][hh] += qv.x * rx + qv.y * ry;  // Re(conj(q~) (R_m k))
                }
              }
            }
          }
        }
      }
    } else {
    for (int j = 0; j < G; ++j) {
      for (int r = 0; r < K.R; ++r) {
        __syncthreads();
        const _Float16* cbp = a.kcb + ((((size_t)h * G + j) * K.R + r) * K.Nc) * GS;
        for (int i = tid; i < NH * K.Nc * PP; i += kThreads) {
          const int hh = i / (K.Nc * PP), rem = i % (K.Nc * PP), l = rem / PP, pp = rem % PP;
          const float x = (float)cbp[l * GS + 2 * pp], y = (float)cbp[l * GS + 2 * pp + 1];
          const float2 qv = qz[hh * P + j * PP + pp];
          table[i] = make_float2(qv.x * x + qv.y * y, qv.x * y - qv.y * x);  // conj(q~) * z
        }
        __syncthreads();
        const int f = r * G + j;
  #pragma unroll
        for (int t = 0; t < TPT; ++t) {
          const int m = m0 + tid + kThreads * t;
          if (m < L) {
            const int code = read_field(kbase + (size_t)m * K.bpt, f, K.bits);
  #pragma unroll
            for (int pp = 0; pp < PP; ++pp) {
              const int p = j * PP + pp;
              const float2 w = (EX ? phase_exact((uint32_t)m, ph.lo[p], ph.hi[p]) : phase_hw((uint32_t)m, ph.lo[p], ph.hi[p]));
  #pragma unroll
              for (int hh = 0; hh < NH; ++hh) {
                const float2 T = table[(hh * K.Nc + code) * PP + pp];
                s[t][hh] += T.x * w.x - T.y * w.y;
              }
            }
          }
        }
      }
    }
    }

  };
  if (a.exact_phase)
    scores(std::true_type{});
  else
    scores(std::false_type{});

  // softmax over the chunk
  float M[NH], lsum[NH];
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TPT; ++t)
      if (m0 + tid + kThreads * t < L) mx = fmaxf(mx, s[t][hh] * a.sm_scale);
    mx = wave_max(mx);
    if (lane == 0) red[hh * NW + wave] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float mx = red[hh * NW];
    for (int w = 1; w < NW; ++w) mx = fmaxf(mx, red[hh * NW + w]);
    M[hh] = mx;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < TPT; ++t) {
      const bool ok = m0 + tid + kThreads * t < L;
      const float pw = ok ? __expf(s[t][hh] * a.sm_scale - M[hh]) : 0.f;
      s[t][hh] = pw;
      acc += pw;
    }
    acc = wave_sum(acc);
    if (lane == 0) red[hh * NW + wave] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int hh = 0; hh < NH; ++hh) {
    float acc = 0.f;
    for (int w = 0; w < NW; ++w) acc += red[hh * NW + w];
    lsum[hh] = acc;
    // (summed here: left to the end, the wavefront sums read above stay live in
    // registers through the value stage)
    asm volatile("" : "+v"(lsum[hh]));
  }

  if constexpr (BITV) {
    // Binary value codes (a token's whole value, all KV heads, is the sum of
    // the rows of C whose bits are set): u[hh][i] = sum_m p[hh][m] bit_i(m)
    // over the chunk, then o[hh] = u[hh]^T C[:, h D .. h D + D) - the weights
    // meet the codes before the codebook (review, "If this is right", fourth
    // bullet). Thread (slot, c) takes byte c of the bit rows (bits 8c .. 8c+7)
    // of every `slots`-th position; bit rows are staged in LDS kBitSub
    // positions at a time.
    const int NB = a.nbits, TB = NB / 8, slots = kThreads / TB;
    float* pw = uni;                                        // [NH][chunk] weights
    float* u = pw + NH * a.chunk;                           // [NH][NB]
    uint32_t* rows_l = reinterpret_cast<uint32_t*>(u + NH * NB);  // [kBitSub][TB / 4]
    __syncthreads();  // the score phase's table is no longer read
#pragma unroll
    for (int t = 0; t < TPT; ++t)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) pw[hh * a.chunk + tid + kThreads * t] = s[t][hh];  // 0 past the length
    for (int i = tid; i < NH * NB; i += kThreads) u[i] = 0.f;
    const int c = tid % TB, slot = tid / TB;
    float acc[8][NH];
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) acc[k][hh] = 0.f;
    const int n = min(L - m0, a.chunk);
    // range-major storage: ranges of RW dwords (16 bytes, or the whole string
    // when shorter), [B][ranges][cache_len][RW]
    const int RW = TB >= 16 ? 4 : TB / 4, NRG = (TB / 4) / RW;
    const uint32_t* bits_g = reinterpret_cast<const uint32_t*>(a.vbits) + (size_t)b * NRG * a.cache_len * RW;
    for (int s0 = 0; s0 < n; s0 += kBitSub) {
      const int ns = min(kBitSub, n - s0);
      __syncthreads();  // (the previous rows are read; the weights and u are written)
      for (int i = tid; i < ns * (TB / 4); i += kThreads) {
        const int p = i / (TB / 4), dw = i % (TB / 4), rr = dw / RW, k = dw % RW;
        rows_l[i] = bits_g[((size_t)rr * a.cache_len + m0 + s0 + p) * RW + k];
      }
      __syncthreads();
      const uint8_t* rb = reinterpret_cast<const uint8_t*>(rows_l);
      for (int tl = slot; tl < ns; tl += slots) {
        const uint32_t byte = rb[tl * TB + c];
        float w[NH];
#pragma unroll
        for (int hh = 0; hh < NH; ++hh) w[hh] = pw[hh * a.chunk + s0 + tl];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          const float bit = (float)((byte >> k) & 1u);
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) acc[k][hh] = fmaf(bit, w[hh], acc[k][hh]);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int hh = 0; hh < NH; ++hh) atomicAdd(&u[hh * NB + 8 * c + k], acc[k][hh]);
    __syncthreads();
    const _Float16* cv = a.vrows + (size_t)h * D;  // row i, column h D + d at cv[i * Hkv * D + d]
    const size_t ld = (size_t)K.Hkv * D;
    for (int i = tid; i < NH * D; i += kThreads) {
      const int hh = i / D, d = i % D;
      float o = 0.f;
      for (int r = 0; r < NB; ++r) o = fmaf(u[hh * NB + r], (float)cv[(size_t)r * ld + d], o);
      oacc[hh * D + d] = o;
    }
  } else {
  // value histograms and contraction with the value codebook: RB rounds of a
  // group per pass (all of them where their histograms fit the table's LDS),
  // bins [round][code][head]
  const int RB = generic_hist_rounds(K, V, NH);
  const int NBIN = RB * V.Nc;
  for (int j = 0; j < G; ++j) {
    for (int r = 0; r < V.R; r += RB) {
      // the pass's rounds of group j are consecutive in the codebook: bin b
      // (round r + b / Nc, code b % Nc) at cvp[b * GS]
      const _Float16* cvp = a.vcb + ((((size_t)h * G + j) * V.R + r) * V.Nc) * GS;
      // NO outputs (head, scalar), each a sum over the NBIN bins split over PARTS
      // lanes of one wavefront and added with shuffles
      constexpr int NO = NH * GS;
      constexpr int PARTS = NO >= kThreads ? 1 : (kThreads / NO > 64 ? 64 : kThreads / NO);
      // groups of 8 scalars: a lane takes 8 consecutive outputs of one head
      // (one 16-byte codebook read per bin) over every PV-th bin, and the PV
      // lanes of those outputs (adjacent, in one wavefront) are added with shuffles
      constexpr int NOV = NH * GS / 8;
      constexpr int PV = GS % 8 != 0 ? 0 : (kThreads / NOV > 64 ? 64 : kThreads / NOV);
      // Wide groups, where the wavefronts' partial sums fit the histogram's
      // region: the contraction on v_mfma_f32_16x16x16_f16 (below).
      constexpr int NHQ = (NH + 3) / 4;  // 16-row blocks of heads (rows of the A operand)
      const bool mc_on = GS >= kWideGroup && NBIN % 16 == 0 &&
                         (size_t)NW * 16 * NHQ * 16 <= generic_uni_bytes(K, V, NH);
      constexpr int MC_NT = GS / 16 > 0 ? GS / 16 : 1;    // output tiles of 16 columns
      constexpr int MC_WPT = NW / MC_NT > 0 ? NW / MC_NT : 1;  // wavefronts per tile
      static_assert(GS < kWideGroup || (NW % MC_NT == 0), "tiles per workgroup");
      // codebook bins per batch of loads
      constexpr int CBB = GS >= kWideGroup ? 8 : 4;
      const int pv_o = PV >= 2 ? tid / PV : 0, pv_part = PV >= 2 ? tid % PV : 0;
      const bool pv_on = PV >= 2 && pv_o < NOV;
      const int pv_ev = PV >= 2 ? pv_o % (GS / 8) : 0;
      auto load_bins = [&](int l0, uint4 (&w)[CBB]) {
#pragma unroll
        for (int u = 0; u < CBB; ++u) {
          const int l = l0 + u * PV;
          w[u] = l < NBIN ? *reinterpret_cast<const uint4*>(cvp + (size_t)l * GS + 8 * pv_ev) : make_uint4(0u, 0u, 0u, 0u);
        }
      };

      uint4 wpre[CBB];
      __syncthreads();
      for (int i = tid; i < NH * NBIN; i += kThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < TPT; ++t) {
        const int m = m0 + tid + kThreads * t;
        if (m < L) {
          uint32_t fx[NH];
#pragma unroll
          for (int hh = 0; hh < NH; ++hh) fx[hh] = (uint32_t)fmaf(s[t][hh], (float)(1 << kHistShift), 0.5f);
          int code_next = vfield(m, r * G + j);  // (each round's field read ahead)
          for (int rr = 0; rr < RB; ++rr) {
            const int bin = rr * V.Nc + code_next;
            if (rr + 1 < RB) code_next = vfield(m, (r + rr + 1) * G + j);
            if constexpr (NH % 2 == 0) {
              // two heads per 64-bit add: a head's bin sums to at most
              // 1024 * 2^20 < 2^32, so no half carries into its neighbour
#pragma unroll
              for (int hp = 0; hp < NH / 2; ++hp)
                __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(hist) + (size_t)bin * (NH / 2) + hp,
                                       (uint64_t)fx[2 * hp] | ((uint64_t)fx[2 * hp + 1] << 32), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
            } else {
#pragma unroll
              for (int hh = 0; hh < NH; ++hh) atomicAdd(&hist[bin * NH + hh], fx[hh]);
            }
          }
        }
      }
      __syncthreads();
      if constexpr (GS >= kWideGroup) {
        if (mc_on) {
          // o[head][dim] = sum_bin H[head][bin] CV[bin][dim] per 16-bin K-step.
          // A: row = head (lane & 15; rows past NH are 0), K = bins 4 kq .. 4 kq + 3
          // of the step, as the bins' fixed-point counts scaled to at most 1024 and
          // split into fp16 hi + lo parts (products keep ~22 bits). B: column n =
          // dimension 32 set + 2 n + par, the same bins, from one codebook dword
          // (two dimensions) per bin regrouped with byte permutes. Tile (set, par)
          // is shared by MC_WPT wavefronts taking every MC_WPT-th step, two steps'
          // codebook dwords in flight; their partial sums meet in LDS.
          const int tile = wave / MC_WPT, sub = wave % MC_WPT;
          const int set = tile >> 1, par = tile & 1, n = lane & 15, kq = lane >> 4, row = lane & 15;
          const int steps = NBIN / 16;
          const uint32_t* cv32 = reinterpret_cast<const uint32_t*>(cvp);  // bin b's dwords at b * GS / 2
          const uint32_t voff = (uint32_t)(4 * kq) * (GS / 2) + 16 * set + n;
          const uint32_t hoff = (uint32_t)(4 * kq) * NH + (row < NH ? row : 0);
          const bool hrow = row < NH;
          const uint32_t sel = par ? 0x07060302u : 0x05040100u;  // high or low halves: dim 2n + par
          auto load = [&](int st, uint32_t (&w)[4]) {
            const uint32_t* base = cv32 + (size_t)st * 16 * (GS / 2);  // (uniform)
#pragma unroll
            for (int u = 0; u < 4; ++u) w[u] = base[voff + u * (GS / 2)];
          };
          float4_t acc = {0.f, 0.f, 0.f, 0.f};
          auto step = [&](int st, const uint32_t (&w)[4]) {
            half4_t ahi, alo;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const uint32_t hv = hrow ? hist[(uint32_t)st * 16 * NH + hoff + u * NH] : 0u;
              const float x = (float)hv * (1.0f / (float)(1 << kHistShift));
              const _Float16 hi = (_Float16)x;
              ahi[u] = hi;
              alo[u] = (_Float16)(x - (float)hi);
            }
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const half4_t bop = __builtin_bit_cast(
                half4_t, (u32x2_t){__builtin_amdgcn_perm(w[1], w[0], sel), __builtin_amdgcn_perm(w[3], w[2], sel)});
            acc = __builtin_amdgcn_mfma_f32_16x16x16f16(ahi, bop, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x16f16(alo, bop, acc, 0, 0, 0);
          };
          uint32_t w0[4], w1[4];
          if (sub < steps) load(sub, w0);
          if (sub + MC_WPT < steps) load(sub + MC_WPT, w1);
          for (int st = sub; st < steps; st += 2 * MC_WPT) {
            step(st, w0);
            if (st + 2 * MC_WPT < steps) load(st + 2 * MC_WPT, w0);
            if (st + MC_WPT < steps) {
              step(st + MC_WPT, w1);
              if (st + 3 * MC_WPT < steps) load(st + 3 * MC_WPT, w1);
            }
          }
          __syncthreads();  // every wavefront is done with the histogram: its region takes the partial sums
          float* psum = uni;  // [wavefront][16 NHQ lanes][4]: rows 4 kq .. 4 kq + 3 of column n
          if (lane < 16 * NHQ) *reinterpret_cast<float4*>(psum + ((size_t)wave * 16 * NHQ + lane) * 4) = make_float4(acc[0], acc[1], acc[2], acc[3]);
          __syncthreads();
          for (int i = tid; i < NH * GS; i += kThreads) {
            const int hh = i / GS, d = i % GS;
            const int tile = (d >> 5) * 2 + (d & 1), l = (hh >> 2) * 16 + ((d & 31) >> 1);
            float sum = 0.f;
#pragma unroll
            for (int u = 0; u < MC_WPT; ++u) sum += psum[((size_t)(tile * MC_WPT + u) * 16 * NHQ + l) * 4 + (hh & 3)];
            oacc[hh * D + j * GS + d] += sum;
          }
        }
      }
      if constexpr (PV >= 2) {
        const int o = pv_o, part = pv_part;
        if (pv_on && !mc_on) {
          const int hh = o / (GS / 8), ev = pv_ev;
          float acc[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] = 0.f;
          auto consume = [&](const uint4 (&w)[CBB], int l0) {
#pragma unroll
            for (int u = 0; u < CBB; ++u) {
              const int l = l0 + u * PV;
              if (l < NBIN) {
                const float hv = (float)hist[l * NH + hh];
                const uint32_t wd[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                  acc[2 * k] = fma_f16_lo(acc[2 * k], wd[k], hv);
                  acc[2 * k + 1] = fma_f16_hi(acc[2 * k + 1], wd[k], hv);
                }
              }
            }
          };
          load_bins(part, wpre);
          consume(wpre, part);
#pragma unroll 1
          for (int l0 = part + CBB * PV; l0 < NBIN; l0 += CBB * PV) {
            uint4 w[CBB];
            load_bins(l0, w);
            consume(w, l0);
          }
          (void)ev;
          for (int off = PV / 2; off > 0; off >>= 1)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
          if (part == 0)
#pragma unroll
            for (int k = 0; k < 8; ++k) oacc[hh * D + j * GS + 8 * ev + k] += acc[k] * (1.0f / (float)(1 << kHistShift));
        }
      } else if constexpr (PARTS == 1) {
        for (int i = mc_on ? NO : tid; i < NO; i += kThreads) {
          const int hh = i / GS, e = i % GS;
          float acc = 0.f;
          for (int l = 0; l < NBIN; ++l) acc = fmaf((float)hist[l * NH + hh], (float)cvp[l * GS + e], acc);
          oacc[hh * D + j * GS + e] += acc * (1.0f / (float)(1 << kHistShift));
        }
      } else {
        const int o = tid / PARTS, part = tid % PARTS;
        if (o < NO && !mc_on) {  // whole groups of PARTS lanes
          const int hh = o / GS, e = o % GS;
          float acc = 0.f;
          for (int l = part; l < NBIN; l += PARTS) acc = fmaf((float)hist[l * NH + hh], (float)cvp[l * GS + e], acc);
#pragma unroll
          for (int off = PARTS / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
          if (part == 0) oacc[hh * D + j * GS + e] += acc * (1.0f / (float)(1 << kHistShift));
        }
      }
    }
  }
  }
  __syncthreads();
  if (tid == 0) {
#pragma unroll
    for (int hh = 0; hh < NH; ++hh) {
      red[2 * hh] = M[hh];
      red[2 * hh + 1] = lsum[hh];
    }
  }
  __syncthreads();
  for (int i = tid; i < NH * (D + 2); i += kThreads) {
    const int hh = i / (D + 2), k = i % (D + 2);
    part[hh * pstride + k] = k < 2 ? red[2 * hh + k] : oacc[hh * D + k - 2];
  }
}

template <int NH, int GS, bool BITV>
hipError_t launch_generic(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  const size_t smem = BITV ? decode_bitv_smem(a.k, a.nbits, NH) : decode_generic_smem(a.k, a.v, NH);
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&decode_generic_kernel<NH, GS, BITV>), configured);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_generic_kernel<NH, GS, BITV>), dim3(a.n_chunks * a.k.Hkv, a.B), dim3(generic_threads(NH, GS)), smem,
                     stream, a, ph);
  return hipGetLastError();
}

template <int NH, bool BITV>
hipError_t launch_generic_nh(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  switch (a.k.g) {
    case 2: return launch_generic<NH, 2, BITV>(a, ph, stream);
    case 4: return launch_generic<NH, 4, BITV>(a, ph, stream);
    case 8: return launch_generic<NH, 8, BITV>(a, ph, stream);
    case 16: return launch_generic<NH, 16, BITV>(a, ph, stream);
    case 32: return launch_generic<NH, 32, BITV>(a, ph, stream);
    case 64: return launch_generic<NH, 64, BITV>(a, ph, stream);
    case 128: return launch_generic<NH, 128, BITV>(a, ph, stream);
    default: return hipErrorInvalidValue;
  }
}

template <bool BITV>
hipError_t launch_generic_all(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  switch (a.NH) {
    case 1: return launch_generic_nh<1, BITV>(a, ph, stream);
    case 2: return launch_generic_nh<2, BITV>(a, ph, stream);
    case 4: return launch_generic_nh<4, BITV>(a, ph, stream);
    case 8: return launch_generic_nh<8, BITV>(a, ph, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t decode_bitv_smem(const CbShape& k, int nbits, int NH) {
  // the score phase's staging, or the weights [NH][chunk], u [NH][nbits] and
  // kBitSub positions' bit rows
  const size_t score = decode_generic_smem(k, k, NH);
  const size_t fixed = generic_fixed_bytes(k, k, NH);
  const size_t bitv = fixed + ((size_t)NH * kGenericChunk + (size_t)NH * nbits) * sizeof(float) +
                      (size_t)kBitSub * (nbits / 8);
  return score > bitv ? score : bitv;
}

size_t decode_generic_smem(const CbShape& k, const CbShape& v, int NH) {
  // rotated queries (float2 per pair), output accumulators, reductions, then
  // the query x codebook table of one (group, round) or a value histogram,
  // then (wide groups, short records) the chunk's key and value records
  return generic_fixed_bytes(k, v, NH) + generic_uni_bytes(k, v, NH) + generic_rec_bytes(k, v, NH) +
         (generic_dbl_slice(k, v, NH) ? generic_slice_bytes(k) : 0);
}

bool decode_fast_path(const CbShape& k, const CbShape& v, int NH, int flags) {
  return !(flags & 1) && k.D == 128 && k.g == 8 && k.Nc == 256 && v.Nc == 256 && k.R == v.R &&
         (k.R == 1 || k.R == 2) && NH == 4;
}

int decode_chunk_len(const CbShape& k, const CbShape& v, int B, int Hq, int max_len, int flags) {
  if (!decode_fast_path(k, v, Hq / k.Hkv, flags)) return kGenericChunk;
  // the longest chunk that still gives every compute unit a workgroup
  for (int c : {4096, 2048}) {
    const long long wgs = (long long)B * k.Hkv * ((max_len + c - 1) / c);
    if (wgs >= 256) return c;
  }
  return 1024;
}

size_t decode_newtok_offset(const CbShape& k, int B, int Hq, int max_len, int chunk) {
  // chunk partials [B][Hq][n_chunks][D + 2]: (max, sum, o[D]) of one chunk
  const size_t n_chunks = (size_t)(max_len + chunk - 1) / chunk;
  return ((size_t)B * Hq * n_chunks * (k.D + 2) * sizeof(float) + 255) / 256 * 256;
}

size_t decode_workspace_bytes(const CbShape& k, int B, int Hq, int max_len, int chunk) {
  // the partials, then a decode step's new-token area [B][Hkv][kFastNewTokFloats]
  return decode_newtok_offset(k, B, Hq, max_len, chunk) +
         ((size_t)B * k.Hkv * kFastNewTokFloats * sizeof(float) + 255) / 256 * 256;
}

hipError_t launch_decode_generic(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  return launch_generic_all<false>(a, ph, stream);
}

hipError_t launch_decode_bitv(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  if (a.nbits < 32 || a.nbits > 2048 || (a.nbits & (a.nbits - 1)) || a.chunk != kGenericChunk)
    return hipErrorInvalidValue;
  return launch_generic_all<true>(a, ph, stream);
}

}  // namespace commvq

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
__host__ __device__ inline size_t generic_fixed_bytes(const CbShape& k, int NH) {
  // rotated queries (float2 per pair), output accumulators, reductions
  const int P = k.D / 2, NW = generic_threads(NH, k.g) / 64;
  return (2 * NH * P + NH * k.D + ((NH * (NW > 2 ? NW : 2) + 2 * NH + 4) & ~3)) * sizeof(float);
}
__host__ __device__ inline bool generic_stage_records(const CbShape& k, const CbShape& v, int NH) {
  return k.g >= kWideGroup && k.bpt <= 32 && v.bpt <= 32 &&
         generic_fixed_bytes(k, NH) + generic_uni_bytes(k, v, NH) + (size_t)kGenericChunk * (k.bpt + v.bpt) <=
             160 * 1024;
}
__host__ __device__ inline size_t generic_rec_bytes(const CbShape& k, const CbShape& v, int NH) {
  return generic_stage_records(k, v, NH) ? (size_t)kGenericChunk * (k.bpt + v.bpt) : 0;
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
  float* uni = red + red_floats;  // table or histogram
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
      for (int j = 0; j < G; ++j) {
        for (int sl = 0; sl < GS / SL; ++sl) {
          __syncthreads();
          const _Float16* src = a.kcb + ((size_t)h * G + j) * K.R * K.Nc * GS + sl * SL;  // entry (r, l) at (r Nc + l) GS
          {
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
          }
          __syncthreads();
#pragma unroll
          for (int t = 0; t < TPT; ++t) {  // (unrolled: s[t] stays in registers)
            const int m = m0 + tid + kThreads * t;
            if (m < L) {
              float kx[SL];
  #pragma unroll
              for (int i = 0; i < SL; ++i) kx[i] = 0.f;
              for (int r = 0; r < K.R; ++r) {
                const int code = kfield(m, r * G + j);
                const int ei = r * K.Nc + code;
                const uint4* e = reinterpret_cast<const uint4*>(cbs) + ei * 4;
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
    const uint32_t* bits_g = reinterpret_cast<const uint32_t*>(a.vbits + ((size_t)b * a.cache_len + m0) * TB);
    for (int s0 = 0; s0 < n; s0 += kBitSub) {
      const int ns = min(kBitSub, n - s0);
      __syncthreads();  // (the previous rows are read; the weights and u are written)
      for (int i = tid; i < ns * (TB / 4); i += kThreads) rows_l[i] = bits_g[(size_t)s0 * (TB / 4) + i];
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
  // bins [head][round][code]
  const int RB = generic_hist_rounds(K, V, NH);
  const int NBIN = RB * V.Nc;
  for (int j = 0; j < G; ++j) {
    for (int r = 0; r < V.R; r += RB) {
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
          for (int rr = 0; rr < RB; ++rr) {
            const int code = vfield(m, (r + rr) * G + j);
#pragma unroll
            for (int hh = 0; hh < NH; ++hh) atomicAdd(&hist[hh * NBIN + rr * V.Nc + code], fx[hh]);
          }
        }
      }
      __syncthreads();
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
      if constexpr (PV >= 2) {
        const int o = tid / PV, part = tid % PV;
        if (o < NOV) {
          const int hh = o / (GS / 8), ev = o % (GS / 8);
          float acc[8];
#pragma unroll
          for (int k = 0; k < 8; ++k) acc[k] = 0.f;
#pragma unroll 4
          for (int l = part; l < NBIN; l += PV) {
            const uint4 w = *reinterpret_cast<const uint4*>(cvp + (size_t)l * GS + 8 * ev);
            const float hv = (float)hist[hh * NBIN + l];
            const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const half2_t xy = __builtin_bit_cast(half2_t, wd[u]);
              acc[2 * u] = fmaf(hv, (float)xy.x, acc[2 * u]);
              acc[2 * u + 1] = fmaf(hv, (float)xy.y, acc[2 * u + 1]);
            }
          }
#pragma unroll
          for (int off = PV / 2; off > 0; off >>= 1)
#pragma unroll
            for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
          if (part == 0)
#pragma unroll
            for (int k = 0; k < 8; ++k) oacc[hh * D + j * GS + 8 * ev + k] += acc[k] * (1.0f / (float)(1 << kHistShift));
        }
      } else if constexpr (PARTS == 1) {
        for (int i = tid; i < NO; i += kThreads) {
          const int hh = i / GS, e = i % GS;
          float acc = 0.f;
          for (int l = 0; l < NBIN; ++l) acc = fmaf((float)hist[hh * NBIN + l], (float)cvp[l * GS + e], acc);
          oacc[hh * D + j * GS + e] += acc * (1.0f / (float)(1 << kHistShift));
        }
      } else {
        const int o = tid / PARTS, part = tid % PARTS;
        if (o < NO) {  // whole groups of PARTS lanes
          const int hh = o / GS, e = o % GS;
          float acc = 0.f;
          for (int l = part; l < NBIN; l += PARTS) acc = fmaf((float)hist[hh * NBIN + l], (float)cvp[l * GS + e], acc);
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
  const int P = k.D / 2, NW = generic_threads(NH, k.g) / 64;
  const size_t fixed = (2 * NH * P + NH * k.D + ((NH * (NW > 2 ? NW : 2) + 2 * NH + 4) & ~3)) * sizeof(float);
  const size_t bitv = fixed + ((size_t)NH * kGenericChunk + (size_t)NH * nbits) * sizeof(float) +
                      (size_t)kBitSub * (nbits / 8);
  return score > bitv ? score : bitv;
}

size_t decode_generic_smem(const CbShape& k, const CbShape& v, int NH) {
  // rotated queries (float2 per pair), output accumulators, reductions, then
  // the query x codebook table of one (group, round) or a value histogram,
  // then (wide groups, short records) the chunk's key and value records
  return generic_fixed_bytes(k, NH) + generic_uni_bytes(k, v, NH) + generic_rec_bytes(k, v, NH);
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

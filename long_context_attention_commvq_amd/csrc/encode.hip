// CommVQ encoder: greedy residual nearest-codeword search and bit packing.
//
// Each (token, KV head, group of g scalars) is assigned, round by round, the
// codebook entry nearest to the running residual (squared Euclidean distance,
// lowest index on ties), and the residual is reduced by that entry ("Pith
// review of CommVQ", "What carries the argument": one index shared by a group,
// R residual rounds). The R*G fields of a record are packed round-major,
// LSB-first.
//
// Three kernels:
//  * encode_mfma_kernel (g = 8, Nc' = 256, R <= 2, the workload shape): the
//    distance search is a GEMM on the matrix cores. For an entry c and residual
//    e, score(c) = |c|^2 / 2 - e.c orders entries exactly as |e - c|^2 does.
//    One v_mfma_f32_16x16x32_f16 gives the scores of 16 entries for 16 tokens:
//    K = 32 holds [-c, -c, |c|^2/2 as three fp16 parts, 4096, 0...] against
//    [x, y, 1, 1, 1, C_h, 0...], where the residual is e = x + y with x the
//    fp16 input and y = 0 (round 0) or minus the round-0 entry (round 1), so
//    every product is exact and the sums are fp32. The per-token constant
//    4096 C_h >= |e|^2 / 2 makes the scores non-negative, so the argmin runs
//    on integer min3 over their bit patterns; the winner within a quad of four
//    entries is settled by rescoring the four in fp32.
//  * encode_kernel (any shape): distances accumulated term by term in fp32
//    with fmaf against the codebook of one (group, round) staged in LDS.
//  * encode_few_kernel (n <= 64 tokens, the decode-time append): one wavefront
//    per group, the same fp32 arithmetic as encode_kernel.
// The two arithmetic forms may pick different entries only where two
// distances agree to within fp32 rounding (a near tie).

#include "encode_common.hpp"

namespace commvq {
namespace {

template <int GS>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a, int tile) {
  extern __shared__ float enc_smem[];
  const CbShape s = a.s;
  const int R = s.R, Nc = s.Nc, G = s.G, D = s.D, RG = s.R * s.G;
  float* cbs = enc_smem;                                                // [Nc][GS]: one round
  uint8_t* codes_l = reinterpret_cast<uint8_t*>(cbs + (size_t)Nc * GS);  // [tile][R*G]
  const int tid = threadIdx.x;
  const int h = blockIdx.y;
  const int64_t t = (int64_t)blockIdx.x * tile + tid;
  bool valid = t < a.n_tokens;
  const _Float16* xp = nullptr;
  uint8_t* rec = nullptr;
  if (valid) {
    if (a.positions) {
      const int pos = a.positions[t];
      valid = pos >= 0 && pos < a.cache_len;
      xp = a.x + (t * s.Hkv + h) * (int64_t)D;
      rec = a.codes + t * a.code_token_stride + h * a.code_head_stride + (int64_t)pos * s.bpt;
    } else {
      xp = a.x + t * a.x_token_stride + (int64_t)h * D;
      rec = a.codes + t * a.code_token_stride + h * a.code_head_stride;
    }
  }
  for (int j = 0; j < G; ++j) {
    float e[GS];
    if (valid) {
#pragma unroll
      for (int i = 0; i < GS; ++i) e[i] = (float)xp[j * GS + i];
    }
    for (int r = 0; r < R; ++r) {
      __syncthreads();
      const _Float16* src = a.cb + (((int64_t)h * G + j) * R + r) * Nc * GS;
      for (int i = tid; i < Nc * GS; i += blockDim.x) cbs[i] = (float)src[i];
      __syncthreads();
      if (valid) {
        const float* c = cbs;
        float best = INFINITY;
        int bi = 0;
        for (int l = 0; l < Nc; ++l) {
          float d = 0.f;
#pragma unroll
          for (int i = 0; i < GS; ++i) {
            const float df = e[i] - c[l * GS + i];
            d = fmaf(df, df, d);
          }
          if (d < best) {
            best = d;
            bi = l;
          }
        }
#pragma unroll
        for (int i = 0; i < GS; ++i) e[i] -= c[bi * GS + i];
        codes_l[tid * RG + r * G + j] = (uint8_t)bi;
      }
    }
  }
  if (valid) {
    uint32_t acc = 0;
    int nacc = 0, out = 0;
    for (int f = 0; f < RG; ++f) {
      acc |= (uint32_t)codes_l[tid * RG + f] << nacc;
      nacc += s.bits;
      while (nacc >= 8) {
        rec[out++] = (uint8_t)acc;
        acc >>= 8;
        nacc -= 8;
      }
    }
    if (nacc > 0) rec[out++] = (uint8_t)acc;
  }
}

// Few-token variant (decode-time append): one workgroup per (token, KV head),
// one wavefront per group at a time, lanes spread over the codebook entries. The
// distance arithmetic is the bulk kernel's, term by term, so both pick the same
// entries; the wave-wide argmin keeps the lowest index on ties.
template <int GS>
__global__ __launch_bounds__(256) void encode_few_kernel(EncodeArgs a) {
  __shared__ uint8_t codes_l[4 * 128];  // [R][G], R*G <= 512
  const CbShape s = a.s;
  const int R = s.R, Nc = s.Nc, G = s.G, D = s.D;
  const int64_t t = blockIdx.x;
  const int h = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const _Float16* xp;
  uint8_t* rec;
  if (a.positions) {
    const int pos = a.positions[t];
    if (pos < 0 || pos >= a.cache_len) return;  // uniform over the workgroup
    xp = a.x + (t * s.Hkv + h) * (int64_t)D;
    rec = a.codes + t * a.code_token_stride + h * a.code_head_stride + (int64_t)pos * s.bpt;
  } else {
    xp = a.x + t * a.x_token_stride + (int64_t)h * D;
    rec = a.codes + t * a.code_token_stride + h * a.code_head_stride;
  }
  for (int j = wave; j < G; j += 4) {
    float e[GS];
#pragma unroll
    for (int i = 0; i < GS; ++i) e[i] = (float)xp[j * GS + i];
    greedy_group_wave<GS>(e, a.cb + ((int64_t)h * G + j) * R * Nc * GS, Nc, R, lane, codes_l + j, G);
  }
  __syncthreads();
  // byte k of the record collects record bits [8k, 8k + 8)
  for (int k = threadIdx.x; k < s.bpt; k += blockDim.x) {
    uint32_t v = 0;
    for (int i = 0; i < 8; ++i) {
      const int P = 8 * k + i, f = P / s.bits;
      if (f < R * G) v |= (((uint32_t)codes_l[f] >> (P % s.bits)) & 1u) << i;
    }
    rec[k] = (uint8_t)v;
  }
}

constexpr int MF_THREADS = 256;  // four wavefronts
constexpr int MF_TOKENS = 256;   // tokens per workgroup (16 MFMA columns of 16)

constexpr int MF_WAVES = MF_THREADS / 64;
constexpr int MF_NB = 2;  // token batches of 16 interleaved per iteration
constexpr float kMfCScale = 4096.f;  // the per-token constant enters the scores as kMfCScale * C_h

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Minimum of (v, i) over lanes l and l ^ S (S = 16 or 32), the lower lane's
// pair kept on equal v. A v_permlane{16,32}_swap of a register with itself
// leaves, in every lane, the lower lane's (l & ~S) value in its first result
// and the upper lane's (l | S) in its second, so both lanes keep the same
// pair. With i_pair set, the two lanes' indices are given instead of swapped.
template <int S, typename T>
__device__ __forceinline__ void min_lanes(T& v, int& i, bool i_pair = false, int i_lo = 0, int i_hi = 0) {
  static_assert(S == 16 || S == 32, "lane distance");
  const uint32_t vb = __builtin_bit_cast(uint32_t, v);
  uint32_t v0, v1;
  if constexpr (S == 16) {
    const auto pv = __builtin_amdgcn_permlane16_swap(vb, vb, false, false);
    v0 = pv[0], v1 = pv[1];
  } else {
    const auto pv = __builtin_amdgcn_permlane32_swap(vb, vb, false, false);
    v0 = pv[0], v1 = pv[1];
  }
  int i0 = i_lo, i1 = i_hi;
  if (!i_pair) {
    if constexpr (S == 16) {
      const auto pi = __builtin_amdgcn_permlane16_swap((uint32_t)i, (uint32_t)i, false, false);
      i0 = (int)pi[0], i1 = (int)pi[1];
    } else {
      const auto pi = __builtin_amdgcn_permlane32_swap((uint32_t)i, (uint32_t)i, false, false);
      i0 = (int)pi[0], i1 = (int)pi[1];
    }
  }
  const T a = __builtin_bit_cast(T, v0), b = __builtin_bit_cast(T, v1);
  const bool upper = b < a;
  v = upper ? b : a;
  i = upper ? i1 : i0;
}

// K slice q of a token's B operand: x (q 0), y (q 1), the constants (q 2), 0
// (q 3); m[k] is all ones in the lanes of slice k. Combined with bit masks, so
// that nothing moves into per-slice branches.
__device__ __forceinline__ h8_t b_operand(const uint32_t (&m)[3], const uint4 x, const uint4 y, const uint4 c) {
  auto pick = [&m](uint32_t xv, uint32_t yv, uint32_t cv) -> uint32_t {
    return (xv & m[0]) | (yv & m[1]) | (cv & m[2]);
  };
  typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
  const u4_t w = {pick(x.x, y.x, c.x), pick(x.y, y.y, c.y), pick(x.z, y.z, c.z), pick(x.w, y.w, c.w)};
  return __builtin_bit_cast(h8_t, w);
}

// A wavefront's LDS slot, in 16-byte units: its group's R x 256 negated
// entries, their fp32 |c|^2 / 2, and for R = 2 round 1's K-slice-2 operands
__host__ __device__ constexpr int mf_slot(int R) { return R * 256 + R * 64 + (R - 1) * 256; }

// |c|^2 / 2 in three fp16 parts, then the constant's scale: K slice 2 of an
// entry's A operand
__device__ __forceinline__ h8_t k_slice2(float v) {
  const _Float16 v0 = (_Float16)v;
  const float r1 = v - (float)v0;
  const _Float16 v1 = (_Float16)r1;
  const _Float16 v2 = (_Float16)(r1 - (float)v1);
  return h8_t{v0, v1, v2, (_Float16)kMfCScale, 0, 0, 0, 0};
}

// LDS of encode_mfma_kernel: four wavefront slots, then the tile's R * G
// one-byte codes per token
size_t encode_mfma_smem(const CbShape& s) {
  return (size_t)MF_WAVES * mf_slot(s.R) * 16 + (size_t)MF_TOKENS * s.R * s.G;
}

// sum of the eight fp16 products a_i b_i (each exact in fp32) onto acc
__device__ __forceinline__ float mf_dot8(const uint4 a, const uint4 b, float acc) {
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.x), __builtin_bit_cast(h2_t, b.x), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.y), __builtin_bit_cast(h2_t, b.y), acc, false);
  acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.z), __builtin_bit_cast(h2_t, b.z), acc, false);
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a.w), __builtin_bit_cast(h2_t, b.w), acc, false);
}

// Workgroup = (tile of 256 tokens, KV head). Wavefront w takes groups w, w+4,
// ...; for a group it stages the negated entries, their |c|^2 / 2 and round
// 1's K-slice-2 operands in its own LDS slot, keeps round 0's A operands (16
// blocks of 16 entries) in registers, reads round 1's from the slot per use,
// and streams the tile's tokens through them, two batches of 16 interleaved:
// lane (q = lane / 16, n = lane % 16) feeds K slice q of token n and receives
// the scores of entries 16 b + 4 q + i (i < 4) of block b for token n.
//
// The scores carry a per-token constant C >= |e|^2 / 2 (K slice 2 holds
// 4096 * C_h, C_h an fp16 rounded upward), which makes every score a
// non-negative half squared distance, |e - c|^2 / 2 + (C - |e|^2 / 2): fp32
// values >= 0 compare like their bit patterns as signed integers, so the
// search runs on integer min3. Per lane it keeps the smallest score and the
// block holding it; the four lanes of a token then agree on the quad of four
// entries (block, q) with the smallest score.
// Which entry of the quad won is settled by the four lanes rescoring one
// entry each in fp32 (fp16 products, exact, summed in fp32): the two
// evaluations can disagree only where two entries' scores agree to within
// fp32 rounding (a near tie).
template <int R, bool POS>
__global__ __launch_bounds__(MF_THREADS, 2) void encode_mfma_kernel(EncodeArgs a) {
  static_assert(R == 1 || R == 2, "one or two rounds");
  extern __shared__ uint4 mf_smem[];  // [waves] slots, then [MF_TOKENS][R * G] codes
  const CbShape s = a.s;
  const int G = s.G, RG = R * s.G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, n = lane & 15;
  uint4* ncw = mf_smem + wave * mf_slot(R);  // [R][256] negated entries
  float* nrw = reinterpret_cast<float*>(ncw + R * 256);  // [R][256] |c|^2 / 2
  uint4* k2w = ncw + R * 256 + R * 64;  // [R - 1][256] K slice 2 of round 1's A operands
  uint8_t* mf_rec = reinterpret_cast<uint8_t*>(mf_smem + MF_WAVES * mf_slot(R));
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * MF_TOKENS;
  const uint4 zero4 = {0u, 0u, 0u, 0u};
  const uint32_t qm[3] = {q == 0 ? ~0u : 0u, q == 1 ? ~0u : 0u, q == 2 ? ~0u : 0u};

  for (int j = wave; j < G; j += MF_WAVES) {
    // the slot is written and read by this wavefront only, in program order
    const uint4* cbj = reinterpret_cast<const uint4*>(a.cb + ((int64_t)h * G + j) * R * 256 * 8);
    for (int i = lane; i < R * 256; i += 64) {
      const h8_t c = __builtin_bit_cast(h8_t, cbj[i]);
      float v = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) v = fmaf((float)c[k], (float)c[k], v);
      v *= 0.5f;
      ncw[i] = __builtin_bit_cast(uint4, -c);
      nrw[i] = v;
      if (R == 2 && i >= 256) k2w[i - 256] = __builtin_bit_cast(uint4, k_slice2(v));
    }
    // A operands: rows = 16 entries of a block,
    // K = [-c (q 0), -c (q 1), |c|^2/2 as three parts and 4096 (q 2), 0 (q 3)];
    // round 0's in registers, round 1's read from the slot per use (the
    // lanes of K slice 3 read entries there: B is 0 in that slice)
    h8_t A0[16];
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int en = 16 * b + n;
      A0[b] = q < 2 ? __builtin_bit_cast(h8_t, ncw[en]) : (q == 2 ? k_slice2(nrw[en]) : h8_t{});
    }
    const uint4* a1 = (q == 2 ? k2w : ncw + 256) + n;
    // group j of token n of batch tb (zero for tokens past the end or
    // skipped); the input pointer advances by a fixed stride per batch. The
    // loads are unconditional (clamped to token 0) so that the batches'
    // instruction streams can interleave.
    const int64_t tok_stride = POS ? (int64_t)s.Hkv * s.D : a.x_token_stride;
    const _Float16* xg = a.x + (t0 + n) * tok_stride + (int64_t)h * s.D + 8 * j;
    const int64_t left = a.n_tokens - t0 - n;
    // (the raw load and its validity: the zeroing waits for the use)
    auto fetch = [&](int tb, bool& ok) -> uint4 {
      ok = 16 * tb < left;
      if constexpr (POS) {
        const int pos = a.positions[ok ? t0 + n + 16 * tb : 0];
        ok = ok && pos >= 0 && pos < a.cache_len;
      }
      return *reinterpret_cast<const uint4*>(ok ? xg + 16 * tb * tok_stride : a.x + 8 * j);
    };
    uint4 xnext[MF_NB];
    bool oknext[MF_NB];
#pragma unroll
    for (int u = 0; u < MF_NB; ++u) xnext[u] = fetch(u, oknext[u]);
#pragma unroll 1
    for (int tb = 0; tb < MF_TOKENS / 16; tb += MF_NB) {
      uint4 xw[MF_NB], yw[MF_NB];
      float xx[MF_NB], ee[MF_NB], slack[MF_NB];  // ee ~ |e|^2, slack >= its rounding error
      bool non_finite[MF_NB];
#pragma unroll
      for (int u = 0; u < MF_NB; ++u) {
        const uint32_t keep = oknext[u] ? ~0u : 0u;
        xw[u] = make_uint4(xnext[u].x & keep, xnext[u].y & keep, xnext[u].z & keep, xnext[u].w & keep);
        if (tb + MF_NB < MF_TOKENS / 16) xnext[u] = fetch(tb + MF_NB + u, oknext[u]);  // in flight during these batches
        // |x|^2 of finite fp16 values stays below 2^36; a NaN or an infinity
        // in the group makes it NaN or infinite, and such a group takes
        // entry 0 in every round (it has no finite distance to any entry)
        xx[u] = mf_dot8(xw[u], xw[u], 0.f);
        non_finite[u] = !(xx[u] <= 0x1p36f);
        // Round r's residual is e = x + y with y = 0 (round 0) or -c0
        // (round 1, c0 the round-0 entry): both fp16, so the products with an
        // entry are exact and e needs no splitting.
        yw[u] = zero4;
        ee[u] = xx[u];
        slack[u] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        h8_t bv[MF_NB];
#pragma unroll
        for (int u = 0; u < MF_NB; ++u) {
          // C_h >= |e|^2 / 8192: the 2^-8 factor covers the rounding of the
          // conversion, slack the cancellation in |x|^2 - 2 x.c0 + |c0|^2,
          // and the 2^-24 term the subnormal range
          const _Float16 ch = (_Float16)fmaf(ee[u], 0x1.01p-13f, slack[u] + 0x1p-24f);
          const h2_t one_c = {(_Float16)1.f, ch};
          const uint4 cw = make_uint4(0x3C003C00u, __builtin_bit_cast(uint32_t, one_c), 0u, 0u);
          bv[u] = b_operand(qm, xw[u], yw[u], cw);
        }
        int best[MF_NB], bb[MF_NB];
#pragma unroll
        for (int u = 0; u < MF_NB; ++u) best[u] = 0x7fffffff, bb[u] = 0;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const h8_t Ab = r == 0 ? A0[b] : __builtin_bit_cast(h8_t, a1[16 * b]);
#pragma unroll
          for (int u = 0; u < MF_NB; ++u) {
            const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ab, bv[u], (f4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            const int m3 = min(min(__float_as_int(d[0]), __float_as_int(d[1])), __float_as_int(d[2]));
            const int nb = min(min(best[u], m3), __float_as_int(d[3]));
            bb[u] = nb < best[u] ? b : bb[u];
            best[u] = nb;
          }
        }
#pragma unroll
        for (int u = 0; u < MF_NB; ++u) {
          // the four lanes of token n agree on the quad (4 block + q) with
          // the smallest score
          int quad = 4 * bb[u] + q;
          min_lanes<16>(best[u], quad);
          min_lanes<32>(best[u], quad);
          // entries 16 (quad / 4) + 4 (quad % 4) + i, i < 4: lane q rescoring entry i = q
          const int k0 = 16 * (quad >> 2) + 4 * (quad & 3);
          const uint4 cq = ncw[r * 256 + k0 + q];  // -c
          float dot = mf_dot8(cq, xw[u], 0.f);
          if (r > 0) dot = mf_dot8(cq, yw[u], dot);
          float sc = nrw[r * 256 + k0 + q] + dot;
          int ki = q;
          min_lanes<16>(sc, ki, true, q & 2, q | 1);
          min_lanes<32>(sc, ki);
          const int bi = non_finite[u] ? 0 : k0 + ki;
          // the token's four lanes store the same byte
          mf_rec[(16 * (tb + u) + n) * RG + r * G + j] = (uint8_t)bi;
          if (r + 1 < R) {
            yw[u] = ncw[bi];
            const float cc = 2.f * nrw[bi];
            ee[u] = fmaf(2.f, mf_dot8(xw[u], yw[u], 0.f), xx[u] + cc);
            slack[u] = (xx[u] + cc) * 0x1p-30f;
          }
        }
      }
    }
  }
  __syncthreads();
  // 8-bit fields: a record is its codes in order; one lane writes one token's
  for (int tl = tid; tl < MF_TOKENS; tl += MF_THREADS) {
    const int64_t t = t0 + tl;
    if (t >= a.n_tokens) break;
    uint8_t* rec;
    if (POS) {
      const int pos = a.positions[t];
      if (pos < 0 || pos >= a.cache_len) continue;
      rec = a.codes + t * a.code_token_stride + h * a.code_head_stride + (int64_t)pos * s.bpt;
    } else {
      rec = a.codes + t * a.code_token_stride + h * a.code_head_stride;
    }
    const uint8_t* src = mf_rec + tl * RG;
    if (((reinterpret_cast<uintptr_t>(rec) | (uintptr_t)RG) & 15) == 0) {
      for (int k = 0; k < RG; k += 16)
        *reinterpret_cast<uint4*>(rec + k) = *reinterpret_cast<const uint4*>(src + k);
    } else {
      for (int k = 0; k < RG; ++k) rec[k] = src[k];
    }
  }
}

template <int GS>
hipError_t launch_encode_g(const EncodeArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 64 && a.s.R * a.s.G <= 512) {
    hipLaunchKernelGGL(encode_few_kernel<GS>, dim3((unsigned)a.n_tokens, a.s.Hkv), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if constexpr (GS == 8) {
    if (encode_uses_matrix_cores(a.s)) {
      const int64_t nblk = (a.n_tokens + MF_TOKENS - 1) / MF_TOKENS;
      if (nblk > 0x7fffffff) return hipErrorInvalidValue;
      const size_t smem = encode_mfma_smem(a.s);
      static std::atomic<uint64_t> configured[4];
      const int v = (a.s.R == 2 ? 2 : 0) + (a.positions ? 1 : 0);
      const void* fns[4] = {reinterpret_cast<const void*>(&encode_mfma_kernel<1, false>),
                            reinterpret_cast<const void*>(&encode_mfma_kernel<1, true>),
                            reinterpret_cast<const void*>(&encode_mfma_kernel<2, false>),
                            reinterpret_cast<const void*>(&encode_mfma_kernel<2, true>)};
      if (smem > 64 * 1024) {
        const hipError_t e = allow_full_lds(fns[v], configured[v]);
        if (e != hipSuccess) return e;
      }
      const dim3 grid((unsigned)nblk, a.s.Hkv), block(MF_THREADS);
      switch (v) {
        case 0: hipLaunchKernelGGL((encode_mfma_kernel<1, false>), grid, block, smem, stream, a); break;
        case 1: hipLaunchKernelGGL((encode_mfma_kernel<1, true>), grid, block, smem, stream, a); break;
        case 2: hipLaunchKernelGGL((encode_mfma_kernel<2, false>), grid, block, smem, stream, a); break;
        default: hipLaunchKernelGGL((encode_mfma_kernel<2, true>), grid, block, smem, stream, a); break;
      }
      return hipGetLastError();
    }
  }
  const CbShape& s = a.s;
  const size_t cb_bytes = (size_t)s.Nc * GS * sizeof(float);  // one round at a time
  int tile = 256;
  while (tile > 64 && cb_bytes + (size_t)tile * s.R * s.G > 160 * 1024) tile /= 2;
  const size_t smem = cb_bytes + (size_t)tile * s.R * s.G;
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&encode_kernel<GS>), configured);
  if (e != hipSuccess) return e;
  const int64_t nblk = (a.n_tokens + tile - 1) / tile;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_kernel<GS>, dim3((unsigned)nblk, s.Hkv), dim3(tile), smem, stream, a, tile);
  return hipGetLastError();
}

}  // namespace

// The MFMA search covers g = 8, Nc' = 256 (8-bit fields) and R <= 2 when the
// wavefronts' codebook slots and the tile's codes fit the workgroup's LDS.
bool encode_uses_matrix_cores(const CbShape& s) {
  return s.g == 8 && s.Nc == 256 && s.R <= 2 && encode_mfma_smem(s) <= 160 * 1024;
}

// Near-tie diagnostic of an encoding already written: per (token, head, round,
// group) field, the relative margin between the two smallest squared distances
// of the round's residual to the group's entries,
//   gap = (d2 - d1) / max(d1, 1e-12 |e|^2)   (+inf when Nc' = 1),
// each round's residual taken after the encoder's own picks of the earlier
// rounds (read back from the record). Distances in fp32. One lane per
// (token, head, group); its residual lives in LDS (g <= 128 floats).
constexpr int kGapThreads = 64;

__device__ __forceinline__ int gap_read_field(const uint8_t* rec, int f, int bits) {
  const int o = f * bits, byte = o >> 3, sh = o & 7;
  uint32_t v = rec[byte];
  if (sh + bits > 8) v |= (uint32_t)rec[byte + 1] << 8;
  return (int)((v >> sh) & ((1u << bits) - 1u));
}

__global__ __launch_bounds__(kGapThreads) void encode_gaps_kernel(EncodeArgs a, float* gap) {
  extern __shared__ float gap_e[];
  const CbShape s = a.s;
  const int G = s.G, g = s.g, R = s.R, Nc = s.Nc, H = s.Hkv;
  const int64_t i = (int64_t)blockIdx.x * kGapThreads + threadIdx.x;  // (token, head, group)
  if (i >= a.n_tokens * H * G) return;
  const int j = (int)(i % G), h = (int)((i / G) % H);
  const int64_t t = i / ((int64_t)G * H);
  float* e = gap_e + threadIdx.x * g;
  const _Float16* xs = a.x + t * a.x_token_stride + (int64_t)h * s.D + (int64_t)j * g;
  for (int k = 0; k < g; ++k) e[k] = (float)xs[k];
  const uint8_t* rec = a.codes + t * a.code_token_stride + (int64_t)h * a.code_head_stride;
  for (int r = 0; r < R; ++r) {
    const _Float16* ent = a.cb + (((size_t)h * G + j) * R + r) * (size_t)Nc * g;
    float n2 = 0.f;
    for (int k = 0; k < g; ++k) n2 = fmaf(e[k], e[k], n2);
    float d1 = INFINITY, d2 = INFINITY;
    for (int l = 0; l < Nc; ++l) {
      float d = 0.f;
      for (int k = 0; k < g; ++k) {
        const float df = e[k] - (float)ent[(size_t)l * g + k];
        d = fmaf(df, df, d);
      }
      if (d < d1) {
        d2 = d1;
        d1 = d;
      } else if (d < d2) {
        d2 = d;
      }
    }
    gap[((t * H + h) * R + r) * G + j] = Nc > 1 ? (d2 - d1) / fmaxf(fmaxf(d1, 1e-12f * n2), 1e-30f) : INFINITY;
    const int code = gap_read_field(rec, r * G + j, s.bits);
    for (int k = 0; k < g; ++k) e[k] -= (float)ent[(size_t)code * g + k];
  }
}

hipError_t launch_encode_gaps(const EncodeArgs& a, float* gap, hipStream_t stream) {
  const int64_t n = a.n_tokens * a.s.Hkv * a.s.G;
  if (n <= 0) return hipSuccess;
  const int64_t nblk = (n + kGapThreads - 1) / kGapThreads;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_gaps_kernel, dim3((unsigned)nblk), dim3(kGapThreads), kGapThreads * a.s.g * sizeof(float),
                     stream, a, gap);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t stream) {
  switch (a.s.g) {
    case 2: return launch_encode_g<2>(a, stream);
    case 4: return launch_encode_g<4>(a, stream);
    case 6: return launch_encode_g<6>(a, stream);
    case 8: return launch_encode_g<8>(a, stream);
    case 10: return launch_encode_g<10>(a, stream);
    case 12: return launch_encode_g<12>(a, stream);
    case 14: return launch_encode_g<14>(a, stream);
    case 16: return launch_encode_g<16>(a, stream);
    case 32: return launch_encode_g<32>(a, stream);
    case 64: return launch_encode_g<64>(a, stream);
    case 128: return launch_encode_g<128>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace commvq

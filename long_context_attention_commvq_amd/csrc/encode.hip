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
//    K = 32 holds [-c, -c, |c|^2/2 as three fp16 parts, 0...] against
//    [e_hi, e_lo, 1, 1, 1, 0...], where e = e_hi + e_lo splits the fp32
//    residual into two fp16 values (products are exact, sums fp32). The argmin
//    compares the fp32 scores, lowest index on ties.
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

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));

// Workgroup = (tile of 256 tokens, KV head). Wavefront w takes groups w, w+4,
// ...; for a group it keeps the A operands of all R rounds (16 blocks of 16
// entries each) in registers and streams the tile's tokens through them, 16 at
// a time: lane (q = lane / 16, n = lane % 16) feeds K slice q of token n and
// receives the scores of entries 16 b + 4 q + i (i < 4) of block b for token n.
template <int R>
__global__ __launch_bounds__(MF_THREADS, 2) void encode_mfma_kernel(EncodeArgs a) {
  extern __shared__ uint8_t mf_rec[];  // [MF_TOKENS][R * G] codes of the tile
  const CbShape s = a.s;
  const int G = s.G, RG = R * s.G;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, q = lane >> 4, n = lane & 15;
  const int h = blockIdx.y;
  const int64_t t0 = (int64_t)blockIdx.x * MF_TOKENS;

  for (int j = wave; j < G; j += MF_THREADS / 64) {
    const _Float16* cbj = a.cb + ((int64_t)h * G + j) * R * 256 * 8;
    // A operands: rows = 16 entries of a block, K = [-c (q 0), -c (q 1), |c|^2/2 (q 2), 0 (q 3)]
    h8_t A[R][16];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const h8_t c = *reinterpret_cast<const h8_t*>(cbj + ((size_t)r * 256 + 16 * b + n) * 8);
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) v = fmaf((float)c[i], (float)c[i], v);
        v *= 0.5f;
        const _Float16 v0 = (_Float16)v;
        const float r1 = v - (float)v0;
        const _Float16 v1 = (_Float16)r1;
        const _Float16 v2 = (_Float16)(r1 - (float)v1);
        const h8_t nrm = {v0, v1, v2, 0, 0, 0, 0, 0};
        A[r][b] = q < 2 ? -c : (q == 2 ? nrm : h8_t{});
      }
    const h8_t ones = {1, 1, 1, 0, 0, 0, 0, 0};
#pragma unroll 1
    for (int tb = 0; tb < MF_TOKENS / 16; ++tb) {
      const int tl = 16 * tb + n;
      const int64_t t = t0 + tl;
      bool valid = t < a.n_tokens;
      const _Float16* xp = nullptr;
      if (valid) {
        if (a.positions) {
          const int pos = a.positions[t];
          valid = pos >= 0 && pos < a.cache_len;
          xp = a.x + (t * s.Hkv + h) * (int64_t)s.D;
        } else {
          xp = a.x + t * a.x_token_stride + (int64_t)h * s.D;
        }
      }
      float e[8];
      if (valid) {
        const h8_t xv = *reinterpret_cast<const h8_t*>(xp + 8 * j);
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (float)xv[i];
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = 0.f;
      }
#pragma unroll
      for (int r = 0; r < R; ++r) {
        h8_t hi, lo;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          hi[i] = (_Float16)e[i];
          lo[i] = (_Float16)(e[i] - (float)hi[i]);
        }
        const h8_t bv = q == 0 ? hi : (q == 1 ? lo : (q == 2 ? ones : h8_t{}));
        float best = INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int b = 0; b < 16; ++b) {
          const f4_t d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[r][b], bv, (f4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (d[i] < best) {
              best = d[i];
              bi = 16 * b + 4 * q + i;
            }
        }
        // the four lanes of token n hold disjoint entry sets
#pragma unroll
        for (int o = 16; o < 64; o <<= 1) {
          const float od = __shfl_xor(best, o, 64);
          const int oi = __shfl_xor(bi, o, 64);
          if (od < best || (od == best && oi < bi)) {
            best = od;
            bi = oi;
          }
        }
        if (bi == 0x7fffffff) bi = 0;  // no score compared below +inf (NaN input)
        if (q == 0) mf_rec[tl * RG + r * G + j] = (uint8_t)bi;
        if (r + 1 < R) {
          const h8_t c = *reinterpret_cast<const h8_t*>(cbj + ((size_t)r * 256 + bi) * 8);
#pragma unroll
          for (int i = 0; i < 8; ++i) e[i] -= (float)c[i];
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
    if (a.positions) {
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
      const size_t smem = (size_t)MF_TOKENS * a.s.R * a.s.G;
      if (a.s.R == 1)
        hipLaunchKernelGGL(encode_mfma_kernel<1>, dim3((unsigned)nblk, a.s.Hkv), dim3(MF_THREADS), smem, stream, a);
      else
        hipLaunchKernelGGL(encode_mfma_kernel<2>, dim3((unsigned)nblk, a.s.Hkv), dim3(MF_THREADS), smem, stream, a);
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
// tile's codes fit the workgroup's LDS.
bool encode_uses_matrix_cores(const CbShape& s) {
  return s.g == 8 && s.Nc == 256 && s.R <= 2 && (size_t)MF_TOKENS * s.R * s.G <= 64 * 1024;
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

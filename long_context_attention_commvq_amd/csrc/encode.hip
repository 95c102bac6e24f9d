// CommVQ encoder: greedy residual nearest-codeword search and bit packing.
//
// Each (token, KV head, group of g scalars) is assigned, round by round, the
// codebook entry nearest to the running residual (squared Euclidean distance,
// float32 arithmetic, lowest index on ties), and the residual is reduced by that
// entry ("Pith review of CommVQ", "What carries the argument": one index shared
// by a group, R residual rounds). The R*G fields of a record are packed
// round-major, LSB-first.
//
// Work split: one workgroup per (tile of tokens, KV head). The workgroup walks
// the groups; for each group the [R][Nc][g] codebook slice is staged in LDS as
// float and read by every lane at the same address (broadcast, no conflicts).
// Codes collect in LDS and each lane packs its own record at the end.

#include "encode_common.hpp"

namespace commvq {
namespace {

template <int GS>
__global__ __launch_bounds__(256) void encode_kernel(EncodeArgs a, int tile) {
  extern __shared__ float enc_smem[];
  const CbShape s = a.s;
  const int R = s.R, Nc = s.Nc, G = s.G, D = s.D, RG = s.R * s.G;
  float* cbs = enc_smem;                                                    // [R][Nc][GS]
  uint8_t* codes_l = reinterpret_cast<uint8_t*>(cbs + (size_t)R * Nc * GS);  // [tile][R*G]
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
    __syncthreads();
    const _Float16* src = a.cb + ((int64_t)h * G + j) * R * Nc * GS;
    for (int i = tid; i < R * Nc * GS; i += blockDim.x) cbs[i] = (float)src[i];
    __syncthreads();
    if (valid) {
      float e[GS];
#pragma unroll
      for (int i = 0; i < GS; ++i) e[i] = (float)xp[j * GS + i];
      for (int r = 0; r < R; ++r) {
        const float* c = cbs + (size_t)r * Nc * GS;
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

template <int GS>
hipError_t launch_encode_g(const EncodeArgs& a, hipStream_t stream) {
  if (a.n_tokens <= 64 && a.s.R * a.s.G <= 512) {
    hipLaunchKernelGGL(encode_few_kernel<GS>, dim3((unsigned)a.n_tokens, a.s.Hkv), dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  const CbShape& s = a.s;
  const size_t cb_bytes = (size_t)s.R * s.Nc * GS * sizeof(float);
  int tile = 256;
  while (tile > 64 && cb_bytes + (size_t)tile * s.R * s.G > 160 * 1024) tile /= 2;
  const size_t smem = cb_bytes + (size_t)tile * s.R * s.G;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&encode_kernel<GS>), configured);
  if (e != hipSuccess) return e;
  const int64_t nblk = (a.n_tokens + tile - 1) / tile;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(encode_kernel<GS>, dim3((unsigned)nblk, s.Hkv), dim3(tile), smem, stream, a, tile);
  return hipGetLastError();
}

}  // namespace

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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace commvq

// Codebook fitting: one EM iteration for one residual round of a codebook.
//
// The abstract says the codebook is trained with an Expectation-Maximization
// algorithm; the review ("Pith review of CommVQ", "Assumptions & free
// parameters") describes alternating assignment and update in the k-means
// manner with soft assignment and annealing, and ("Referee Report",
// Significance) a closed-form update. For round r of every (KV head, group):
//  E-step: each vector is reduced greedily by the nearest entry of rounds
//          0..r-1 (squared Euclidean distance in fp32, lowest index on ties, as
//          the encoder); for the residual e and the round's entries c_l,
//          d_l = |e - c_l|^2 and w_l = exp((min d - d_l) / T) / sum over l
//          (T > 0), or 1 for the nearest entry and 0 elsewhere (T = 0);
//  M-step: c_l = sum_n w_nl e_n / sum_n w_nl (kept where that mass is not
//          above min_mass).
// Launches: a fill of the fp32 accumulators; em_accumulate_kernel, or at
// temperature 0 for the shapes the encoder searches on the matrix cores the
// encoder (codes of a batch into the work buffer) and em_scatter_kernel per
// batch; then em_update_kernel.
//
// em_accumulate_kernel<g>: a workgroup per (1024 vectors, KV head) walks the
// groups; per group it stages rounds 0..r of the codebook (fp32), then for
// each tile of 256 vectors their residuals, in LDS. For 16 vectors at a time, thread l computes the
// distances to entry l; each wavefront reduces four vectors' rows (minimum
// and its lowest index). For an earlier round the residuals are then reduced
// by their nearest entries; for the fitted round at temperature 0 the
// wavefront adds the vector and a count of 1 to its nearest entry's sums in
// LDS (fp32 LDS atomics), and at temperature > 0 it also sums the row's soft
// weights, after which thread l adds w_nl e_n and w_nl in registers. The
// workgroup's sums go to the accumulators with fp32 atomics, once per group
// after its four tiles.

#include "decode_common.hpp"

namespace commvq {
namespace {

constexpr int kEmThreads = 256, kEmTokens = 256, kEmSub = 16;
constexpr int kEmTiles = 4;  // tiles of kEmTokens vectors per workgroup, one flush of the sums per group
constexpr size_t kEmCodeScratch = size_t(4) << 20;  // codes of one encoder batch (nearest-entry path)

// Wavefront minimum of (distance, entry) with the lowest entry on equal
// distances, on the 64-bit key (distance bits << 32 | entry): distances are
// non-negative (or +inf / NaN, which order above every finite one, as the
// scalar compare they replace never selects them), so their bits order as the
// values. DPP butterfly over each row of 16 lanes, then the four rows' results.
template <int CTRL>
__device__ __forceinline__ uint64_t em_dpp_u64(uint64_t k) {
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)k, CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(k >> 32), CTRL, 0xf, 0xf, false);
  return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}
__device__ __forceinline__ uint64_t em_wave_key_min(uint64_t k) {
  uint64_t o;
  o = em_dpp_u64<0xb1>(k);   // quad_perm [1,0,3,2]
  k = o < k ? o : k;
  o = em_dpp_u64<0x4e>(k);   // quad_perm [2,3,0,1]
  k = o < k ? o : k;
  o = em_dpp_u64<0x124>(k);  // row_ror:4
  k = o < k ? o : k;
  o = em_dpp_u64<0x128>(k);  // row_ror:8
  k = o < k ? o : k;
  uint64_t r = k;
#pragma unroll
  for (int row = 0; row < 4; ++row) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)k, 16 * row);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(k >> 32), 16 * row);
    const uint64_t rk = ((uint64_t)hi << 32) | lo;
    r = row == 0 ? rk : (rk < r ? rk : r);
  }
  return r;
}

// Minimum and sum over each 16-lane DPP row (every lane of the row ends with
// its row's result): quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_ror 4, row_ror 8.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}
__device__ __forceinline__ uint32_t row16_umin(uint32_t v) {
  v = min(v, dpp_u<0xb1>(v));
  v = min(v, dpp_u<0x4e>(v));
  v = min(v, dpp_u<0x124>(v));
  return min(v, dpp_u<0x128>(v));
}
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f<0xb1>(v);
  v += dpp_f<0x4e>(v);
  v += dpp_f<0x124>(v);
  return v + dpp_f<0x128>(v);
}

// g consecutive floats from LDS, 16 bytes at a time where g allows (rows of the
// codebook and of the residuals then start on 16-byte boundaries)
template <int GS>
__device__ __forceinline__ void lds_row(const float* p, float (&o)[GS]) {
  if constexpr (GS % 4 == 0) {
#pragma unroll
    for (int k = 0; k < GS; k += 4) {
      const float4 v = *reinterpret_cast<const float4*>(p + k);
      o[k] = v.x;
      o[k + 1] = v.y;
      o[k + 2] = v.z;
      o[k + 3] = v.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < GS; ++k) o[k] = p[k];
  }
}

__global__ __launch_bounds__(256) void em_fill_kernel(float* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.f;
}

template <int GS>
__global__ __launch_bounds__(kEmThreads) void em_accumulate_kernel(EmArgs a) {
  extern __shared__ __attribute__((aligned(16))) float em_smem[];
  const CbShape s = a.s;
  const int Nc = s.Nc, G = s.G, r = a.round;
  const int h = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t tw = (int64_t)blockIdx.x * kEmTokens * kEmTiles;
  float* cbf = em_smem;                          // [r + 1][Nc][GS]
  float* res = cbf + (size_t)(r + 1) * Nc * GS;  // [kEmTokens][GS]
  float* dist = res + kEmTokens * GS;            // [kEmSub][Nc]
  float* rmin = dist + kEmSub * Nc;              // [kEmSub]
  float* rsum = rmin + kEmSub;                   // [kEmSub]
  int* rarg = reinterpret_cast<int*>(rsum + kEmSub);
  float* hacc = rsum + 2 * kEmSub;               // [Nc][GS + 1]: nearest-entry sums (temperature 0 only)
  const bool soft = a.temperature > 0.f;
  const float invT = soft ? 1.f / a.temperature : 0.f;
  // exp((m - d) / T) = 2^((m - d) * log2(e) / T): one factor, then the hardware exp2
  const float kexp = invT * 1.44269504f;
  for (int j = 0; j < G; ++j) {
    __syncthreads();  // the previous group's reads of LDS are done
    const _Float16* cbj = a.cb + ((size_t)h * G + j) * s.R * Nc * GS;
    for (int i = tid; i < (r + 1) * Nc * GS; i += kEmThreads) cbf[i] = (float)cbj[i];
    if (!soft)
      for (int i = tid; i < Nc * (GS + 1); i += kEmThreads) hacc[i] = 0.f;
    float acc[GS + 1];
#pragma unroll
    for (int k = 0; k <= GS; ++k) acc[k] = 0.f;
    for (int tile = 0; tile < kEmTiles; ++tile) {
      const int64_t t0 = tw + (int64_t)tile * kEmTokens;
      if (t0 >= a.n_tokens) break;  // (uniform)
      const int nt = (int)min((int64_t)kEmTokens, a.n_tokens - t0);
      __syncthreads();  // the previous tile's reads of the residuals are done
      for (int i = tid; i < kEmTokens * GS; i += kEmThreads) {
        const int n = i / GS, k = i - n * GS;
        res[i] = n < nt ? (float)a.x[(t0 + n) * a.x_token_stride + (int64_t)h * s.D + j * GS + k] : 0.f;
      }
      __syncthreads();
      for (int n0 = 0; n0 < nt; n0 += kEmSub) {
        const int ns = min(kEmSub, nt - n0);
        for (int rr = 0; rr <= r; ++rr) {
          const float* cr = cbf + (size_t)rr * Nc * GS;
          const bool fitted = rr == r;
          // distances: thread l to entry l, for the sub-tile's vectors
          if (tid < Nc) {
            float c[GS];
            lds_row<GS>(cr + tid * GS, c);
#pragma unroll
            for (int n = 0; n < kEmSub; ++n) {
              float e[GS];
              lds_row<GS>(res + (n0 + n) * GS, e);
              float d = 0.f;
#pragma unroll
              for (int k = 0; k < GS; ++k) {
                const float df = e[k] - c[k];
                d = fmaf(df, df, d);
              }
              dist[n * Nc + tid] = d;
            }
          }
          __syncthreads();
          // rows: minimum and its lowest index; for the fitted round the soft
          // weights' sum, or (nearest entry) the vector added to its entry's sums
          static_assert(kEmSub == 4 * (kEmThreads / 64), "four rows per wavefront: one per 16-lane DPP row");
          if (fitted && soft && Nc == 256) {
            // the wavefront's four rows n = wave + 4 i, one per 16-lane DPP row
            // (i = lane / 16); lane j of it holds entries 4 j + 64 t + 0..3 in
            // registers (16-byte LDS accesses, a row's lanes contiguous). Only the
            // row's smallest distance is needed here: distances are non-negative,
            // +inf or NaN, so their bits order as unsigned integers with NaN above
            // +inf, never chosen (the minimum of the per-row loop below, exactly)
            const int n = wave + (kEmThreads / 64) * (lane >> 4);
            float4* drow = reinterpret_cast<float4*>(dist + n * Nc) + (lane & 15);
            float4 v[4];
            uint32_t mb = 0x7f800000u;  // +inf
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              v[t] = drow[16 * t];
              mb = min(mb, min(min(__builtin_bit_cast(uint32_t, v[t].x), __builtin_bit_cast(uint32_t, v[t].y)),
                               min(__builtin_bit_cast(uint32_t, v[t].z), __builtin_bit_cast(uint32_t, v[t].w))));
            }
            const float m = __builtin_bit_cast(float, row16_umin(mb));
            // each exponential is kept in place of its distance for the sums below
            float sm;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              float4 e;
              e.x = __builtin_amdgcn_exp2f((m - v[t].x) * kexp);
              e.y = __builtin_amdgcn_exp2f((m - v[t].y) * kexp);
              e.z = __builtin_amdgcn_exp2f((m - v[t].z) * kexp);
              e.w = __builtin_amdgcn_exp2f((m - v[t].w) * kexp);
              drow[16 * t] = e;
              sm = t == 0 ? e.x : sm + e.x;
              sm += e.y;
              sm += e.z;
              sm += e.w;
            }
            sm = row16_sum(sm);
            if ((lane & 15) == 0) {
              rmin[n] = m;
              rsum[n] = 1.f / sm;  // (sm >= 1: the nearest entry's term is 1)
            }
          } else
          for (int n = wave; n < kEmSub; n += kEmThreads / 64) {
            float m = INFINITY;
            int mi = 0;  // (a valid index even if every distance is infinite or NaN)
            // Nc' = 256: the lane's four distances stay in registers for the
            // exponentials below (the same values either way)
            const bool nc256 = Nc == 256;
            float v4[4];
            if (nc256) {
#pragma unroll
              for (int i = 0; i < 4; ++i) v4[i] = dist[n * Nc + lane + 64 * i];
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (v4[i] < m) m = v4[i], mi = lane + 64 * i;  // ascending entries: the first of equal ones is kept
            } else {
              for (int l = lane; l < Nc; l += 64) {
                const float v = dist[n * Nc + l];
                if (v < m) m = v, mi = l;  // a lane's entries ascend: the first of equal ones is kept
              }
            }
            {
              const uint64_t key = em_wave_key_min(((uint64_t)__builtin_bit_cast(uint32_t, m) << 32) | (uint32_t)mi);
              m = __builtin_bit_cast(float, (uint32_t)(key >> 32));
              mi = (int)(uint32_t)key;
            }
            if (fitted && soft) {
              // each exponential is kept in place of its distance for the sums below
              float sm = 0.f;
              if (nc256) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                  const float e = __builtin_amdgcn_exp2f((m - v4[i]) * kexp);
                  dist[n * Nc + lane + 64 * i] = e;
                  sm += e;
                }
              } else {
                for (int l = lane; l < Nc; l += 64) {
                  const float e = __builtin_amdgcn_exp2f((m - dist[n * Nc + l]) * kexp);
                  dist[n * Nc + l] = e;
                  sm += e;
                }
              }
              sm = wave_sum(sm);  // (DPP butterfly; the shuffle butterfly measured 8 % slower overall)
              if (lane == 0) {
                rmin[n] = m;
                rsum[n] = 1.f / sm;  // (sm >= 1: the nearest entry's term is 1)
              }
            } else if (fitted) {
              if (n < ns && lane <= GS) atomicAdd(&hacc[mi * (GS + 1) + lane], lane < GS ? res[(n0 + n) * GS + lane] : 1.f);
            } else if (lane == 0) {
              rarg[n] = mi;
            }
          }
          __syncthreads();
          if (!fitted) {
            for (int i = tid; i < ns * GS; i += kEmThreads) {
              const int n = i / GS, k = i - n * GS;
              res[(n0 + n) * GS + k] -= cr[rarg[n] * GS + k];
            }
            __syncthreads();
          } else if (soft && tid < Nc) {
            float rs[kEmSub];  // the rows' 1 / sum, 16 bytes at a time
#pragma unroll
            for (int n = 0; n < kEmSub; n += 4) {
              const float4 r4 = *reinterpret_cast<const float4*>(rsum + n);
              rs[n] = r4.x;
              rs[n + 1] = r4.y;
              rs[n + 2] = r4.z;
              rs[n + 3] = r4.w;
            }
#pragma unroll
            for (int n = 0; n < kEmSub; ++n) {
              if (n < ns) {
                // (no branch on w == 0: a weight that underflows adds exact zeros, and a
                // non-finite residual makes every weight of its row NaN, not 0)
                const float w = dist[n * Nc + tid] * rs[n];  // (the row pass's exponential)
                float e[GS];
                lds_row<GS>(res + (n0 + n) * GS, e);
#pragma unroll
                for (int k = 0; k < GS; ++k) acc[k] = fmaf(w, e[k], acc[k]);
                acc[GS] += w;
              }
            }
          }
        }
      }
    }
    if (!soft) {
      __syncthreads();  // every nearest-entry sum is in
      if (tid < Nc) {
#pragma unroll
        for (int k = 0; k <= GS; ++k) acc[k] = hacc[tid * (GS + 1) + k];
      }
    }
    if (tid < Nc) {
      float* wk = a.work + (((size_t)h * G + j) * Nc + tid) * (GS + 1);
#pragma unroll
      for (int k = 0; k <= GS; ++k)
        if (acc[k] != 0.f) atomicAdd(wk + k, acc[k]);
    }
  }
}

// Nearest-entry path (temperature 0, shapes the encoder searches on the matrix
// cores): the encoder writes a batch's codes, then this kernel adds every
// vector's round-r residual (x minus the chosen entries of rounds < r, in
// fp32 as the encoder subtracts them) with a count of 1 to its chosen entry's
// sums. A workgroup per (kScatterTokens vectors of the batch, KV head, group)
// sums in LDS (fp32 atomics) before one flush to the accumulators.
constexpr int kScatterTokens = 2048;

template <int GS>
__global__ __launch_bounds__(256) void em_scatter_kernel(EmArgs a, const uint8_t* codes, int64_t t_begin, int n_batch) {
  __shared__ float sums[256 * (GS + 1)];  // Nc' = 256
  const CbShape s = a.s;
  const int Nc = s.Nc, G = s.G, r = a.round;
  const int h = blockIdx.y, j = blockIdx.z, tid = threadIdx.x;
  const int n0 = blockIdx.x * kScatterTokens, n1 = min(n0 + kScatterTokens, n_batch);
  {
    for (int i = tid; i < Nc * (GS + 1); i += 256) sums[i] = 0.f;
    __syncthreads();
    for (int n = n0 + tid; n < n1; n += 256) {
      const uint8_t* rec = codes + ((size_t)n * s.Hkv + h) * s.bpt;  // 8-bit fields, round-major
      const _Float16* xp = a.x + (t_begin + n) * a.x_token_stride + (int64_t)h * s.D + j * GS;
      float e[GS];
#pragma unroll
      for (int k = 0; k < GS; ++k) e[k] = (float)xp[k];
      for (int rr = 0; rr < r; ++rr) {
        const _Float16* ce = a.cb + ((((size_t)h * G + j) * s.R + rr) * Nc + rec[rr * G + j]) * GS;
#pragma unroll
        for (int k = 0; k < GS; ++k) e[k] -= (float)ce[k];
      }
      float* dst = sums + rec[r * G + j] * (GS + 1);
#pragma unroll
      for (int k = 0; k < GS; ++k) atomicAdd(dst + k, e[k]);
      atomicAdd(dst + GS, 1.f);
    }
    __syncthreads();
    float* wk = a.work + ((size_t)h * G + j) * Nc * (GS + 1);
    for (int i = tid; i < Nc * (GS + 1); i += 256)
      if (sums[i] != 0.f) atomicAdd(wk + i, sums[i]);
  }
}

// One thread per (KV head, group, entry) of the fitted round.
template <int GS>
__global__ __launch_bounds__(256) void em_update_kernel(EmArgs a) {
  const CbShape s = a.s;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)s.Hkv * s.G * s.Nc) return;
  const int64_t hj = i / s.Nc;
  const int l = (int)(i - hj * s.Nc);
  const float* wk = a.work + i * (GS + 1);
  const float m = wk[GS];
  const size_t off = (((size_t)hj * s.R + a.round) * s.Nc + l) * GS;
  if (m > a.min_mass) {
#pragma unroll
    for (int k = 0; k < GS; ++k) a.new_cb[off + k] = (_Float16)(wk[k] / m);
  } else if (a.new_cb != a.cb) {
#pragma unroll
    for (int k = 0; k < GS; ++k) a.new_cb[off + k] = a.cb[off + k];
  }
  if (a.mass_out) a.mass_out[i] = m;
}

template <int GS>
hipError_t launch_em_g(const EmArgs& a, hipStream_t stream) {
  const CbShape& s = a.s;
  const size_t work_n = (size_t)s.Hkv * s.G * s.Nc * (GS + 1);
  const size_t fill_blocks = (work_n + 255) / 256 < 4096 ? (work_n + 255) / 256 : 4096;
  hipLaunchKernelGGL(em_fill_kernel, dim3((unsigned)fill_blocks), dim3(256), 0, stream, a.work, work_n);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t batch = em_code_batch(s);
  if (a.temperature == 0.f && batch > 0) {
    if constexpr (GS == 8) {
      uint8_t* codes = reinterpret_cast<uint8_t*>(a.work) + em_accum_bytes(s);
      for (int64_t t0 = 0; t0 < a.n_tokens; t0 += batch) {
        const int nb = (int)(a.n_tokens - t0 < batch ? a.n_tokens - t0 : batch);
        EncodeArgs ea{};
        ea.x = a.x + t0 * a.x_token_stride;
        ea.cb = a.cb;
        ea.codes = codes;
        ea.n_tokens = nb;
        ea.x_token_stride = a.x_token_stride;
        ea.code_token_stride = (int64_t)s.Hkv * s.bpt;
        ea.code_head_stride = s.bpt;
        ea.positions = nullptr;
        ea.cache_len = 0;
        ea.s = s;
        e = launch_encode(ea, stream);
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(em_scatter_kernel<8>, dim3((nb + kScatterTokens - 1) / kScatterTokens, s.Hkv, s.G),
                           dim3(256), 0, stream, a, codes, t0, nb);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
      }
      const int64_t entries = (int64_t)s.Hkv * s.G * s.Nc;
      hipLaunchKernelGGL((em_update_kernel<8>), dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, stream, a);
      return hipGetLastError();
    }
  }
  const size_t smem = em_accumulate_smem(s, a.round, a.temperature > 0.f);
  if (smem > 160 * 1024) return hipErrorInvalidValue;
  static std::atomic<uint64_t> configured{0};
  e = allow_full_lds(reinterpret_cast<const void*>(&em_accumulate_kernel<GS>), configured);
  if (e != hipSuccess) return e;
  const int64_t blocks = (a.n_tokens + kEmTokens * kEmTiles - 1) / (kEmTokens * kEmTiles);
  if (blocks > INT32_MAX || s.Hkv > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL((em_accumulate_kernel<GS>), dim3((unsigned)blocks, s.Hkv), dim3(kEmThreads), smem, stream, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t entries = (int64_t)s.Hkv * s.G * s.Nc;
  hipLaunchKernelGGL((em_update_kernel<GS>), dim3((unsigned)((entries + 255) / 256)), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

size_t em_accumulate_smem(const CbShape& s, int round, bool soft) {
  // rounds 0..round of the codebook (fp32), the residuals, one sub-tile's
  // distances, the rows' terms, and at temperature 0 the nearest-entry sums
  return ((size_t)(round + 1) * s.Nc * s.g + (size_t)kEmTokens * s.g + (size_t)kEmSub * s.Nc + 3 * kEmSub +
          (soft ? 0 : (size_t)s.Nc * (s.g + 1))) * sizeof(float);
}

size_t em_accum_bytes(const CbShape& s) {
  return ((size_t)s.Hkv * s.G * s.Nc * (s.g + 1) * sizeof(float) + 255) / 256 * 256;
}

int64_t em_code_batch(const CbShape& s) {
  // the nearest-entry path: shapes the encoder searches on the matrix cores,
  // codes of a batch of vectors in a 4 MiB scratch (at least 256 vectors)
  if (!encode_uses_matrix_cores(s) || s.Hkv > 65535) return 0;
  const int64_t batch = (int64_t)kEmCodeScratch / ((int64_t)s.Hkv * s.bpt);
  return batch >= 256 ? batch : 0;
}

size_t em_work_bytes(const CbShape& s) { return em_accum_bytes(s) + (em_code_batch(s) > 0 ? kEmCodeScratch : 0); }

hipError_t launch_em_step(const EmArgs& a, hipStream_t stream) {
  switch (a.s.g) {
    case 2: return launch_em_g<2>(a, stream);
    case 4: return launch_em_g<4>(a, stream);
    case 6: return launch_em_g<6>(a, stream);
    case 8: return launch_em_g<8>(a, stream);
    case 10: return launch_em_g<10>(a, stream);
    case 12: return launch_em_g<12>(a, stream);
    case 14: return launch_em_g<14>(a, stream);
    case 16: return launch_em_g<16>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace commvq

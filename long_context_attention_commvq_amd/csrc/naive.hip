// The comparison path: decoding "the naive way" on the same quantized cache.
// The review of CommVQ ("Pith review of CommVQ", "The pith") reports that the
// method's decode latency is several times lower than a naive implementation of
// the same quantization; the plain reading of "naive" taken here is: rebuild
// full fp16 keys (rotated to their positions) and values from the codes in HBM,
// then run ordinary dense decode attention over them. Two kernels:
//
//  * dequant_kv_kernel<g, lds>: a workgroup per (chunk of positions, KV head,
//    keys or values) stages the head's codebook in LDS (when it fits) and
//    writes, per (position, group), the group's g scalars: the sum over rounds
//    of the selected codebook entries (fp32, stored as fp16), keys rotated by
//    RoPE at their position. Streams 4*D bytes out per (position, KV head).
//  * dense_decode_kernel<NH>: split-context decode attention over fp16 keys and
//    values (D = 128). Scores of 16 positions x the NH query heads of a KV head
//    come from eight v_mfma_f32_16x16x32_f16 (the fp32 rotated query split into
//    two fp16 parts, hi + lo, so that its products with the fp16 keys are
//    exact and summed in fp32); the softmax-weighted value sum runs in fp32 on
//    the vector ALUs. Each workgroup
//    leaves (max, sum, o[D]) per query head for its chunk, which the merge kernel
//    combines.

#include "decode_common.hpp"

namespace commvq {
namespace {

typedef _Float16 h8n_t __attribute__((ext_vector_type(8)));

// Field f (log2 Nc' = bits wide, LSB first) of a packed record; a field spans at
// most two bytes since bits <= 8.
__device__ __forceinline__ uint32_t record_field(const uint8_t* rec, int f, int bits) {
  const int bit = f * bits, byte = bit >> 3, sh = bit & 7;
  uint32_t w = rec[byte];
  if (sh + bits > 8) w |= (uint32_t)rec[byte + 1] << 8;
  return (w >> sh) & ((1u << bits) - 1u);
}

// g/2 dwords (fp16 pairs) at p, with the widest accesses the alignment allows:
// p is a multiple of 2g bytes away from a 16-byte boundary.
template <int NP>
__device__ __forceinline__ void load_pairs(const void* p, uint32_t (&w)[NP]) {
  if constexpr (NP % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NP / 4; ++i) {
      const uint4 v = reinterpret_cast<const uint4*>(p)[i];
      w[4 * i] = v.x, w[4 * i + 1] = v.y, w[4 * i + 2] = v.z, w[4 * i + 3] = v.w;
    }
  } else if constexpr (NP % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NP / 2; ++i) {
      const uint2 v = reinterpret_cast<const uint2*>(p)[i];
      w[2 * i] = v.x, w[2 * i + 1] = v.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  }
}

template <int NP>
__device__ __forceinline__ void store_pairs(void* p, const uint32_t (&w)[NP]) {
  if constexpr (NP % 4 == 0) {
#pragma unroll
    for (int i = 0; i < NP / 4; ++i) reinterpret_cast<uint4*>(p)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else if constexpr (NP % 2 == 0) {
#pragma unroll
    for (int i = 0; i < NP / 2; ++i) reinterpret_cast<uint2*>(p)[i] = make_uint2(w[2 * i], w[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < NP; ++i) reinterpret_cast<uint32_t*>(p)[i] = w[i];
  }
}

__device__ __forceinline__ uint32_t pack_pair(float x, float y) {
  const half2_t v = {(_Float16)x, (_Float16)y};
  return __builtin_bit_cast(uint32_t, v);
}

constexpr int kDequantChunk = 4096;   // positions per workgroup
constexpr int kDequantThreads = 512;

// Workgroup x of (KV head y, sequence z) takes the keys (x even) or the values
// (x odd) of positions (x / 2) * kDequantChunk .. + kDequantChunk - 1. With
// CB_LDS the head's codebook is first copied to LDS (random 16-byte reads of a
// 64 KiB table through the vector L1 would each fetch a whole line from L2).
// Thread (tl, j), tl < tpb = 512 / G, does group j of positions tl + tpb * i:
// U positions per iteration, the first round's codes of the two next
// iterations requested before this one's are used.
template <int GS, bool CB_LDS>
__global__ __launch_bounds__(kDequantThreads) __attribute__((amdgpu_waves_per_eu(4)))
void dequant_kv_kernel(DequantArgs a, PhaseTable ph) {
  extern __shared__ uint4 dq_cb[];
  // U positions per thread and iteration (register budget: two workgroups per CU)
  constexpr int NP = GS / 2, U = GS <= 4 ? 8 : GS <= 8 ? 6 : GS <= 12 ? 4 : 2;
  const int is_v = blockIdx.x & 1;
  const CbShape S = is_v ? a.v : a.k;
  const uint8_t* codes = is_v ? a.vcodes : a.kcodes;
  _Float16* out = is_v ? a.vout : a.kout;
  const int G = S.G, tpb = kDequantThreads / G;
  const int b = blockIdx.z, h = blockIdx.y, tid = threadIdx.x;
  const int tl = tid / G, j = tid - tl * G;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int64_t c0 = (int64_t)(blockIdx.x >> 1) * kDequantChunk;
  if (c0 >= L) return;  // whole workgroup
  const size_t cb_elems = (size_t)G * S.R * S.Nc * GS;  // one head's codebook
  const _Float16* cbh = (is_v ? a.vcb : a.kcb) + (size_t)h * cb_elems;
  if constexpr (CB_LDS) {
    if ((cb_elems * 2) % 16 == 0) {
      for (int i = tid; i < (int)(cb_elems * 2 / 16); i += kDequantThreads)
        dq_cb[i] = reinterpret_cast<const uint4*>(cbh)[i];
    } else {
      uint32_t* d = reinterpret_cast<uint32_t*>(dq_cb);
      for (int i = tid; i < (int)(cb_elems / 2); i += kDequantThreads) d[i] = reinterpret_cast<const uint32_t*>(cbh)[i];
    }
    __syncthreads();
  }
  if (tl >= tpb) return;
  const int n = (int)min((int64_t)L - c0, (int64_t)kDequantChunk);
  const size_t head_row = ((size_t)b * S.Hkv + h) * (size_t)a.cache_len + (size_t)c0;
  const size_t jo = (size_t)j * S.R * S.Nc;  // entry index of (j, round 0, code 0)
  auto gather = [&](int r, uint32_t code, uint32_t (&e)[NP]) {
    const size_t ei = (jo + (size_t)r * S.Nc + code) * GS;
    if constexpr (CB_LDS)
      load_pairs<NP>(reinterpret_cast<const _Float16*>(dq_cb) + ei, e);
    else
      load_pairs<NP>(cbh + ei, e);
  };
  // (position offsets within a chunk fit 24-bit multiplies: pos < 4096, bpt <= 512, D <= 256)
  const uint8_t* rec0 = codes + head_row * S.bpt;
  _Float16* out0 = out + head_row * S.D + (size_t)j * GS;
  auto code_at = [&](int pos, int r) {
    return record_field(rec0 + __umul24((uint32_t)min(pos, n - 1), (uint32_t)S.bpt), r * G + j, S.bits);
  };
  // Key phases: the fraction of a turn t * F_P mod 2^64 (F_P = theta_P / 2pi
  // 2^64, exact in 64-bit integers) advances by tpb * F_P from one position of
  // this thread to its next; its top 32 bits feed the hardware cosine and sine
  // (input in turns), as in phase_hw.
  uint64_t turn[NP], tstep[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int P = j * NP + p;
    const uint64_t F = ((uint64_t)ph.hi[P] << 32) | ph.lo[P];
    turn[p] = (uint64_t)(uint32_t)(c0 + tl) * F;
    tstep[p] = (uint64_t)(uint32_t)tpb * F;
  }
  uint32_t nx1[U], nx2[U];
#pragma unroll
  for (int u = 0; u < U; ++u) nx1[u] = code_at(tl + tpb * u, 0);
#pragma unroll
  for (int u = 0; u < U; ++u) nx2[u] = code_at(tl + tpb * (U + u), 0);
  for (int p0 = tl; p0 < n; p0 += tpb * U) {
    uint32_t cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      cur[u] = nx1[u];
      nx1[u] = nx2[u];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) nx2[u] = code_at(p0 + tpb * (2 * U + u), 0);  // (clamped in range)
    float2 acc[U][NP];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t e[NP];
      gather(0, cur[u], e);
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const half2_t xy = __builtin_bit_cast(half2_t, e[p]);
        acc[u][p] = make_float2((float)xy.x, (float)xy.y);
      }
    }
    for (int r = 1; r < S.R; ++r) {
      uint32_t c[U];
#pragma unroll
      for (int u = 0; u < U; ++u) c[u] = code_at(p0 + tpb * u, r);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        uint32_t e[NP];
        gather(r, c[u], e);
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const half2_t xy = __builtin_bit_cast(half2_t, e[p]);
          acc[u][p].x += (float)xy.x;
          acc[u][p].y += (float)xy.y;
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int pos = p0 + tpb * u;
      uint32_t w[NP];
      if (is_v) {
#pragma unroll
        for (int p = 0; p < NP; ++p) w[p] = pack_pair(acc[u][p].x, acc[u][p].y);
      } else {
        // key: rotated to position c0 + pos, pair P = j g/2 + p by the angle (c0 + pos) theta_P
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          const float x = (float)(uint32_t)(turn[p] >> 32) * 0x1p-32f;
          const float cs = __builtin_amdgcn_cosf(x), sn = __builtin_amdgcn_sinf(x);
          turn[p] += tstep[p];
          w[p] = pack_pair(acc[u][p].x * cs - acc[u][p].y * sn, acc[u][p].x * sn + acc[u][p].y * cs);
        }
      }
      if (pos < n) store_pairs<NP>(out0 + __umul24((uint32_t)pos, (uint32_t)S.D), w);
    }
  }
}

constexpr int kDenseThreads = 256, kDenseWaves = kDenseThreads / 64, kDenseD = 128;

template <int NH>
__global__ __launch_bounds__(kDenseThreads) void dense_decode_kernel(DenseArgs a, PhaseTable ph) {
  constexpr int D = kDenseD, CH = kDenseChunk, NW = kDenseWaves, TILES = CH / 16, TPW = TILES / NW;
  static_assert(TPW % 4 == 0, "tiles per wavefront come in batches of 4 (scores) and 2 (values)");
  __shared__ float sc[NH][CH];  // scaled scores, then softmax weights
  __shared__ float red[2][NW][NH];
  __shared__ float osum[NW][NH][D];
  const int c = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, quarter = lane >> 4;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int c0 = c * CH;
  const size_t pstride = (size_t)a.n_chunks * (D + 2);
  float* part = a.part + (((size_t)b * a.Hq + (size_t)h * NH) * a.n_chunks + c) * (D + 2);
  if (c0 >= L) {
    for (int i = tid; i < NH * (D + 2); i += kDenseThreads) {
      const int k = i / (D + 2), e = i % (D + 2);
      part[k * pstride + e] = e == 0 ? -INFINITY : 0.f;
    }
    return;
  }
  const int n = min(L - c0, CH);

  // B operands: the rotated query of head `col` (zero for col >= NH) as fp16
  // hi + lo parts, dimensions 32 quarter + 8 i + (0..7) in MFMA i; the A
  // operand takes the same dimensions of position `col` of a 16-position tile.
  h8n_t qb[4], ql[4];
  {
    const uint32_t qp = (uint32_t)max(a.q_pos[b], 0);
    const float* qrow = a.q + ((size_t)b * a.Hq + (size_t)h * NH + (col < NH ? col : 0)) * D + 32 * quarter;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int P = 16 * quarter + 4 * i + p;
        const float x = qrow[8 * i + 2 * p], y = qrow[8 * i + 2 * p + 1];
        const float2 w = phase_exact(qp, ph.lo[P], ph.hi[P]);
        const float rx = col < NH ? x * w.x - y * w.y : 0.f, ry = col < NH ? x * w.y + y * w.x : 0.f;
        qb[i][2 * p] = (_Float16)rx;
        qb[i][2 * p + 1] = (_Float16)ry;
        ql[i][2 * p] = (_Float16)(rx - (float)qb[i][2 * p]);
        ql[i][2 * p + 1] = (_Float16)(ry - (float)qb[i][2 * p + 1]);
      }
  }

  // ---- scores: wavefront w takes tiles w, w + NW, ... ----------------------
  const _Float16* kb = a.k + ((size_t)b * a.Hkv + h) * (size_t)a.cache_len * D + 32 * quarter;
  float mx = -INFINITY;
#pragma unroll 1
  for (int i0 = 0; i0 < TPW; i0 += 4) {
    h8n_t ka[4][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tr = min(c0 + 16 * (wave + NW * (i0 + u)) + col, L - 1);  // rows past the length: any valid row
      const h8n_t* kp = reinterpret_cast<const h8n_t*>(kb + (size_t)tr * D);
#pragma unroll
      for (int i = 0; i < 4; ++i) ka[u][i] = kp[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int tl0 = 16 * (wave + NW * (i0 + u));
      float4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u][i], qb[i], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[u][i], ql[i], s, 0, 0, 0);
      }
      // s[r] = score of position tl0 + 4 quarter + r for head col
      if (col < NH) {
        float4_t o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = tl0 + 4 * quarter + r < n ? s[r] * a.sm_scale : -INFINITY;
          o[r] = v;
          mx = fmaxf(mx, v);
        }
        *reinterpret_cast<float4_t*>(&sc[col][tl0 + 4 * quarter]) = o;
      }
    }
  }
  mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (lane < NH) red[0][wave][lane] = mx;
  __syncthreads();

  // ---- softmax weights and their sums ---------------------------------------
  float M[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    M[k] = red[0][0][k];
#pragma unroll
    for (int w = 1; w < NW; ++w) M[k] = fmaxf(M[k], red[0][w][k]);
  }
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    float ls = 0.f;
#pragma unroll
    for (int t = tid; t < CH; t += kDenseThreads) {
      const float p = t < n ? __expf(sc[k][t] - M[k]) : 0.f;
      sc[k][t] = p;
      ls += p;
    }
    ls = wave_sum(ls);
    if (lane == 0) red[1][wave][k] = ls;
  }
  __syncthreads();

  // ---- weighted value sum: lane holds dimensions 8 slot .. 8 slot + 7 -------
  const int slot = lane & 15, tsub = lane >> 4;
  const _Float16* vb = a.v + ((size_t)b * a.Hkv + h) * (size_t)a.cache_len * D + 8 * slot;
  float acc[NH][8];
#pragma unroll
  for (int k = 0; k < NH; ++k)
#pragma unroll
    for (int d = 0; d < 8; ++d) acc[k][d] = 0.f;
  // two tiles (eight 16-byte reads per lane) requested per iteration
#pragma unroll 1
  for (int i = 0; i < TPW; i += 2) {
    const int tl0 = 16 * (wave + NW * i);
    if (tl0 >= n) break;  // wavefront-uniform
    h8n_t vv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tt = tl0 + tsub + 4 * (u & 3) + 16 * NW * (u >> 2);
      const int tr = min(c0 + tt, L - 1);  // weight 0 past the length
      vv[u] = *reinterpret_cast<const h8n_t*>(vb + (size_t)tr * D);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int tt = tl0 + tsub + 4 * (u & 3) + 16 * NW * (u >> 2);
      float pw[NH];
#pragma unroll
      for (int k = 0; k < NH; ++k) pw[k] = sc[k][tt];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const float x = (float)vv[u][d];
#pragma unroll
        for (int k = 0; k < NH; ++k) acc[k][d] = fmaf(pw[k], x, acc[k][d]);
      }
    }
  }
  // the four position subsets of a wavefront, then the wavefronts through LDS
#pragma unroll
  for (int k = 0; k < NH; ++k)
#pragma unroll
    for (int d = 0; d < 8; ++d) {
      acc[k][d] += __shfl_xor(acc[k][d], 16, 64);
      acc[k][d] += __shfl_xor(acc[k][d], 32, 64);
    }
  if (tsub == 0) {
#pragma unroll
    for (int k = 0; k < NH; ++k)
#pragma unroll
      for (int d = 0; d < 8; ++d) osum[wave][k][8 * slot + d] = acc[k][d];
  }
  __syncthreads();
  for (int i = tid; i < NH * D; i += kDenseThreads) {
    const int k = i / D, d = i % D;
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) o += osum[w][k][d];
    part[k * pstride + 2 + d] = o;
  }
  if (tid < NH) {
    float m = red[0][0][tid], l = 0.f;
#pragma unroll
    for (int w = 1; w < NW; ++w) m = fmaxf(m, red[0][w][tid]);
#pragma unroll
    for (int w = 0; w < NW; ++w) l += red[1][w][tid];
    part[tid * pstride] = m;
    part[tid * pstride + 1] = l;
  }
}

}  // namespace

template <int GS>
hipError_t launch_dequant_g(const DequantArgs& a, const PhaseTable& ph, hipStream_t stream) {
  const int64_t blocks = 2 * (((int64_t)a.max_len + kDequantChunk - 1) / kDequantChunk);  // keys and values
  if (a.k.G > kDequantThreads || blocks > INT32_MAX || a.k.Hkv > 65535 || a.B > 65535) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks, a.k.Hkv, a.B), block(kDequantThreads);
  const size_t kb = (size_t)a.k.G * a.k.R * a.k.Nc * GS * 2, vb = (size_t)a.v.G * a.v.R * a.v.Nc * GS * 2;
  const size_t cb_bytes = kb > vb ? kb : vb;
  if (cb_bytes <= 160 * 1024) {
    static std::atomic<uint64_t> configured{0};
    hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&dequant_kv_kernel<GS, true>), configured);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((dequant_kv_kernel<GS, true>), grid, block, cb_bytes, stream, a, ph);
  } else {
    hipLaunchKernelGGL((dequant_kv_kernel<GS, false>), grid, block, 0, stream, a, ph);
  }
  return hipGetLastError();
}

hipError_t launch_dequant_kv(const DequantArgs& a, const PhaseTable& ph, hipStream_t stream) {
  switch (a.k.g) {
    case 2: return launch_dequant_g<2>(a, ph, stream);
    case 4: return launch_dequant_g<4>(a, ph, stream);
    case 6: return launch_dequant_g<6>(a, ph, stream);
    case 8: return launch_dequant_g<8>(a, ph, stream);
    case 10: return launch_dequant_g<10>(a, ph, stream);
    case 12: return launch_dequant_g<12>(a, ph, stream);
    case 14: return launch_dequant_g<14>(a, ph, stream);
    case 16: return launch_dequant_g<16>(a, ph, stream);
    default: return hipErrorInvalidValue;
  }
}

size_t dense_workspace_bytes(int B, int Hq, int max_len) {
  const size_t n_chunks = ((size_t)max_len + kDenseChunk - 1) / kDenseChunk;
  return (size_t)B * Hq * n_chunks * (kDenseD + 2) * sizeof(float);
}

hipError_t launch_dense_decode(const DenseArgs& a, const PhaseTable& ph, hipStream_t stream) {
  if (a.Hkv > 65535 || a.B > 65535 || a.n_chunks < 1) return hipErrorInvalidValue;
  const dim3 grid(a.n_chunks, a.Hkv, a.B), block(kDenseThreads);
  switch (a.NH) {
    case 1: hipLaunchKernelGGL(dense_decode_kernel<1>, grid, block, 0, stream, a, ph); break;
    case 2: hipLaunchKernelGGL(dense_decode_kernel<2>, grid, block, 0, stream, a, ph); break;
    case 4: hipLaunchKernelGGL(dense_decode_kernel<4>, grid, block, 0, stream, a, ph); break;
    case 8: hipLaunchKernelGGL(dense_decode_kernel<8>, grid, block, 0, stream, a, ph); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  DecodeArgs m{};
  m.part = a.part;
  m.out = a.out;
  m.B = a.B;
  m.Hq = a.Hq;
  m.NH = a.NH;
  m.n_chunks = a.n_chunks;
  m.k.D = kDenseD;
  m.k.Hkv = a.Hkv;
  m.fold_new = 0;
  return launch_decode_merge(m, stream);
}

}  // namespace commvq

// Binary value codes on the matrix cores.
//
// The paper codes a token's value (all KV heads, d = Hkv * D scalars) as a bit
// string s in {0,1}^Nc and decodes it as s^T C ("Pith review of CommVQ",
// "Referee Report", minor comment 4). Attention then needs, per query head,
//   o = sum_m p_m s_m^T C = (sum_m p_m s_m)^T C = u^T C,
// the weights meeting the codes before the rows ("If this is right", fourth
// bullet). u[head][bit] = sum_m p[head][m] s[m][bit] is a product of the weight
// matrix with a 0/1 matrix: here it runs on v_mfma_f32_16x16x32_f16, all query
// heads of the sequence at once, so each code bit is expanded once per token
// (not once per KV head).
//
// The fast decode kernel has already written the weights e^{s - M} (fp16,
// [B][Hq][positions]) and each chunk's (M, l). One workgroup here takes one
// chunk of positions and one range of 128 code bits:
//   - wavefront w takes k-steps (32 positions) w, w + 8, ...; per k-step
//     A = 16 query heads x 32 positions of weights (one 16-byte load per lane),
//     B = 32 positions x 16 bits, for the 8 bit tiles of the range;
//   - the B operand is built in registers from the lane's 8 positions' 16 code
//     bytes (staged in LDS by direct copies, six k-steps ahead): a byte
//     permute moves the byte holding the lane's bit n of two positions'
//     half-words to the low bytes and a mask keeps that bit, which makes each
//     fp16 the subnormal 2^((n & 7) - 24) or 0 (exact in the products; the
//     scale is undone in fp32), so one operand dword costs two instructions;
//   - the eight wavefronts' u are added through LDS and written to the
//     (chunk, range) partial slot;
//   - the grid puts range r of chunk c at r * chunks + c; workgroups go to the
//     8 XCDs round-robin, so with a multiple of 8 chunks a chunk's ranges share
//     one XCD and its L2 copy of the chunk's weights.
// bitv_merge_kernel then combines the chunks on u (per query head) and forms
// o = u^T C once, in fp32.

#include "decode_common.hpp"

namespace commvq {
namespace {

constexpr int kBvThreads = 512;
constexpr int kBvWaves = kBvThreads / 64;
constexpr int kBvRange = 128;   // code bits per workgroup
constexpr int kBvRow = 132;     // LDS row stride (floats) of the wavefront partials: 4 rows of a store hit 4 bank groups
constexpr int kBvD = 128;       // head_dim of the fast path

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;

// NHT tiles of 16 query heads (Hq <= 16 NHT)
template <int NHT>
__global__ __launch_bounds__(kBvThreads, 1) void bitv_values_kernel(DecodeArgs a) {
  constexpr int HP = 16 * NHT;
  // the wavefront partials of u [w][head][bit]
  constexpr int R0 = kBvWaves * HP * kBvRow * 4;
  __shared__ __attribute__((aligned(16))) char r0[R0];
  float* usum = reinterpret_cast<float*>(r0);
  const int NR = a.nbits / kBvRange;
  const int npc = a.n_chunks / NR;
  // blockIdx.x = r * npc + c: consecutive workgroups (round-robin over the XCDs)
  // are consecutive chunks of one range
  const int r = blockIdx.x / npc, c = blockIdx.x % npc, b = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int m0 = c * a.chunk;
  if (m0 >= L) return;  // the score kernel wrote this chunk's empty partials
  const int nks = (min(m0 + a.chunk, L) - m0 + 31) / 32;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the k-step branches stay scalar
  const int n = lane & 15, kg = lane >> 4;
  // B operand half-words: the byte holding the lane's bit n of a code
  // half-word, moved to the low byte and masked to that bit, is the fp16
  // 2^((n & 7) - 24) (a subnormal, exact in the products) or 0
  const uint32_t jn = (uint32_t)(n >> 3);
  const uint32_t selh[2] = {0x0C040C00u + jn * 0x00010001u, 0x0C060C02u + jn * 0x00010001u};
  const uint32_t bmask = (1u << (n & 7)) * 0x00010001u;
  const size_t plen = (size_t)npc * a.chunk;
  // the range's 16 bytes of consecutive tokens are contiguous (range-major storage)
  const uint8_t* vb = a.vbits + ((size_t)b * NR + r) * a.cache_len * 16;
  const _Float16* pwb = a.pw + (size_t)b * a.Hq * plen;

  // operands of the wavefront's k-step kk (ks = wave + 8 kk, 32 positions):
  // the range's 16 code bytes of each position, copied straight into an LDS
  // slot of the wavefront's ring (lane l and l + 32 copy position l; clamped
  // into the cache, positions past the sequence have weight 0), and the
  // weights of heads 16 ht + n at positions kb..kb+7 into a register slot (a
  // head past Hq reads row 0; its rows of u are never stored). Every load is
  // unconditional, so the wait counts below are exact. kBvAhead k-steps are in
  // flight ahead of the one in use.
  constexpr int kBvAhead = 6;
  constexpr int kBvSlots = kBvAhead + 1;
  static_assert(kBvWaves * kBvSlots * 1024 <= R0, "bit rings fit the partials' LDS");
  char* ring = r0 + wave * (kBvSlots * 1024);
  h8_t wa[kBvSlots][NHT];
  auto issue = [&](int kk) {
    const int slot = kk % kBvSlots;
    const int kb0 = m0 + 32 * (wave + kBvWaves * kk);
    __builtin_amdgcn_global_load_lds(vb + (size_t)min(kb0 + (lane & 31), a.cache_len - 1) * 16,
                                     (lds_void_t*)(ring + slot * 1024), 16, 0, 0);
    const int kb = kb0 + 8 * kg;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = 16 * ht + n;
      wa[slot][ht] = *reinterpret_cast<const h8_t*>(pwb + (size_t)(head < a.Hq ? head : 0) * plen + kb);
    }
  };
  float4_t acc[NHT][8];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[ht][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto step = [&](const h8_t (&w)[NHT], const u32x4 (&x)[8]) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int q = t >> 1;
      const uint32_t sel = selh[t & 1];  // the low or high half-words of positions 2e, 2e + 1
      u32x4 bw;
#pragma unroll
      for (int e = 0; e < 4; ++e) bw[e] = __builtin_amdgcn_perm(x[2 * e + 1][q], x[2 * e][q], sel) & bmask;
      const h8_t bop = __builtin_bit_cast(h8_t, bw);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        acc[ht][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(w[ht], bop, acc[ht][t], 0, 0, 0);
    }
  };
  // A wavefront has at most 4096 / 32 / 8 = 16 k-steps; the loop is unrolled so
  // that the slots are fixed registers and LDS offsets.
  static_assert(4096 / 32 / kBvWaves == 16, "k-steps per wavefront");
#pragma unroll
  for (int kk = 0; kk < kBvAhead; ++kk)
    if (wave + kBvWaves * kk < nks) issue(kk);
#pragma unroll
  for (int kk = 0; kk < 16; ++kk) {
    const int ks = wave + kBvWaves * kk;
    if (ks >= nks) break;  // (uniform in the wavefront)
    const bool more = ks + kBvWaves * kBvAhead < nks;
    if (more) issue(kk + kBvAhead);
    // k-step kk's copy has landed once at most the later k-steps' loads (one
    // copy and NHT weight loads each) are outstanding; the compiler does not
    // track the copy's LDS writes, so the wait is explicit
    if (more)
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kBvAhead * (1 + NHT)) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    const char* sl = ring + (kk % kBvSlots) * 1024;
    u32x4 x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const u32x4*>(sl + (8 * kg + j) * 16);
    step(wa[kk % kBvSlots], x);
  }
  __syncthreads();  // the rings share LDS with the partials

  // lane holds u[16 ht + 4 kg + i][16 t + n] (times 2)
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) usum[(wave * HP + 16 * ht + 4 * kg + i) * kBvRow + 16 * t + n] = acc[ht][t][i];

  __syncthreads();
  // the slot's u (added over the wavefronts), bits in order
  float* pr = a.part + (((size_t)b * a.Hq) * a.n_chunks + (size_t)c * NR + r) * (kBvD + 2) + 2;
  for (int e = tid; e < a.Hq * kBvRange; e += kBvThreads) {
    const int head = e / kBvRange, bit = e % kBvRange;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kBvWaves; ++w) sum += usum[(w * HP + head) * kBvRow + bit];
    pr[(size_t)head * a.n_chunks * (kBvD + 2) + bit] = ldexpf(sum, 24 - (bit & 7));  // the bits entered as 2^((bit & 7) - 24)
  }
}

// Merge and contraction, one workgroup (1024 lanes) per (query head, sequence,
// quarter of the output dimensions; each quarter's workgroup forms all of U):
//   M = max_c M_c, L = sum_c e^{M_c - M} l_c,
//   U[128 r + i] = sum_c e^{M_c - M} u_{c,r}[i],   o = U^T C[:, kv D .. kv D + D) / L,
// the chunks' softmax partials combined on u (linear in the weights), so the
// rows of C meet one u per query head instead of one per chunk and range.
constexpr int kBmThreads = 1024;
__global__ __launch_bounds__(kBmThreads) void bitv_merge_kernel(DecodeArgs a) {
  __shared__ float U[2048];
  __shared__ float wsh[kBmThreads];
  __shared__ float red[2][kBmThreads / 64];
  constexpr int DQ = kBvD / 4;             // output dimensions per workgroup
  constexpr int NP = kBmThreads / (DQ / 2);  // parts of the rows (64)
  __shared__ float2 osum[NP][DQ / 2];
  const int hq = blockIdx.x, b = blockIdx.y, dq0 = blockIdx.z * DQ;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int NR = a.nbits / kBvRange, npc = a.n_chunks / NR;
  constexpr size_t cs = kBvD + 2;
  const float* pr = a.part + ((size_t)b * a.Hq + hq) * a.n_chunks * cs;
  // the rows of C this lane contracts, requested first: lane (part p, pair dp)
  // takes dimensions dq0 + 2 dp, dq0 + 2 dp + 1 of rows p * nbits / 64 ...
  const int dp = tid % (DQ / 2), p = tid / (DQ / 2);
  const int kv = hq / a.NH, dimc = a.k.Hkv * kBvD;
  const int rows = a.nbits / NP;  // 2 .. 32 rows per part
  const half2_t* col = reinterpret_cast<const half2_t*>(a.vrows + (size_t)(p * rows) * dimc + (size_t)kv * kBvD + dq0 + 2 * dp);
  half2_t cv[32];
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (i < rows) cv[i] = col[(size_t)i * (dimc / 2)];
  // the lane's bit i0 in the first kBmU chunks, requested before the chunk
  // statistics are reduced (the values do not depend on them)
  constexpr int kBmU = 32;
  const int i0 = tid, i1 = tid + kBmThreads;  // the lane's bits (nbits <= 2048)
  float u_first[kBmU];
  {
    const float* q = pr + (size_t)(i0 / kBvRange) * cs + 2 + i0 % kBvRange;
#pragma unroll
    for (int k = 0; k < kBmU; ++k) u_first[k] = i0 < a.nbits && k < npc ? q[(size_t)k * NR * cs] : 0.f;
  }
  // M = max_c M_c; the lane's chunk of the first kBmThreads keeps its (M_c, l_c)
  const float m_first = tid < npc ? pr[(size_t)tid * NR * cs] : -INFINITY;
  const float l_first = tid < npc ? pr[(size_t)tid * NR * cs + 1] : 0.f;
  float mx = m_first;
  for (int c = tid + kBmThreads; c < npc; c += kBmThreads) mx = fmaxf(mx, pr[(size_t)c * NR * cs]);
  mx = wave_max(mx);
  if (lane == 0) red[0][wave] = mx;
  __syncthreads();
  float M = red[0][0];
#pragma unroll
  for (int w = 1; w < kBmThreads / 64; ++w) M = fmaxf(M, red[0][w]);
  // U[i] = sum_c w_c u_c[i], w_c = e^{M_c - M} (0 for an empty chunk, whose
  // slots hold zeros), chunks taken kBmThreads at a time, their weights in LDS
  float ls = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int c0 = 0; c0 < npc; c0 += kBmThreads) {
    __syncthreads();
    {
      const int c = c0 + tid;
      float w = 0.f;
      if (c < npc) {
        const float mc = c0 == 0 ? m_first : pr[(size_t)c * NR * cs];
        if (mc > -INFINITY) {
          w = __expf(mc - M);
          ls = fmaf(w, c0 == 0 ? l_first : pr[(size_t)c * NR * cs + 1], ls);
        }
      }
      wsh[tid] = w;
    }
    __syncthreads();
    const int nc = min(kBmThreads, npc - c0);
    auto sweep = [&](int i, float& acc, int kfrom) {
      const int r = i / kBvRange, bit = i % kBvRange;
      const float* q = pr + ((size_t)c0 * NR + r) * cs + 2 + bit;
      for (int k0 = kfrom; k0 < nc; k0 += 16) {
        float uv[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) uv[k] = k0 + k < nc ? q[(size_t)(k0 + k) * NR * cs] : 0.f;
#pragma unroll
        for (int k = 0; k < 16; ++k) acc = fmaf(k0 + k < nc ? wsh[k0 + k] : 0.f, uv[k], acc);
      }
    };
    int kfrom = 0;
    if (c0 == 0) {  // the preloaded chunks (wsh is 0 past nc)
#pragma unroll
      for (int k = 0; k < kBmU; ++k) acc0 = fmaf(wsh[k], u_first[k], acc0);
      kfrom = kBmU;
    }
    if (i0 < a.nbits) sweep(i0, acc0, kfrom);
    if (i1 < a.nbits) sweep(i1, acc1, 0);
  }
  if (i0 < a.nbits) U[i0] = acc0;
  if (i1 < a.nbits) U[i1] = acc1;
  ls = wave_sum(ls);
  if (lane == 0) red[1][wave] = ls;
  __syncthreads();
  float Ls = 0.f;
#pragma unroll
  for (int w = 0; w < kBmThreads / 64; ++w) Ls += red[1][w];
  // o = U^T C / L over this lane's rows, then the 64 parts added
  float o0 = 0.f, o1 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i)
    if (i < rows) {
      const float u = U[p * rows + i];
      o0 = fmaf(u, (float)cv[i].x, o0);
      o1 = fmaf(u, (float)cv[i].y, o1);
    }
  osum[p][dp] = make_float2(o0, o1);
  __syncthreads();
  // wavefront w adds the 64 parts of dimensions 2 w and 2 w + 1, a part per lane
  static_assert(NP == 64 && DQ == 2 * (kBmThreads / 64), "a lane per part, two dimensions per wavefront");
  const float2 v = osum[lane][wave];
  const float ox = wave_sum(v.x), oy = wave_sum(v.y);
  if (lane == 0) {
    float* o = a.out + ((size_t)b * a.Hq + hq) * kBvD + dq0 + 2 * wave;
    o[0] = Ls > 0.f ? ox / Ls : 0.f;
    o[1] = Ls > 0.f ? oy / Ls : 0.f;
  }
}

}  // namespace

bool decode_bitv_fast_path(const CbShape& k, int nbits, int Hq, int flags) {
  return decode_fast_path(k, k, Hq / k.Hkv, flags) && nbits >= kBvRange && nbits % kBvRange == 0 && Hq <= 32;
}

size_t decode_bitv_pw_offset(const CbShape& k, int nbits, int B, int Hq, int max_len, int chunk) {
  // partials [B][Hq][chunks * nbits / 128][D + 2]
  const size_t slots = (size_t)(max_len + chunk - 1) / chunk * (nbits / kBvRange);
  return ((size_t)B * Hq * slots * (k.D + 2) * sizeof(float) + 255) / 256 * 256;
}

size_t decode_bitv_workspace_bytes(const CbShape& k, int nbits, int B, int Hq, int max_len) {
  // enough for either path: the generic kernel's partials, and where the fast
  // path applies its partial slots and weights
  const size_t generic = decode_workspace_bytes(k, B, Hq, max_len, decode_chunk_len(k, k, B, Hq, max_len, 1));
  if (!decode_bitv_fast_path(k, nbits, Hq, 0)) return generic;
  const int chunk = decode_chunk_len(k, k, B, Hq, max_len, 0);
  const size_t plen = (size_t)(max_len + chunk - 1) / chunk * chunk;
  const size_t fast = decode_bitv_pw_offset(k, nbits, B, Hq, max_len, chunk) + ((size_t)B * Hq * plen * 2 + 255) / 256 * 256;
  return fast > generic ? fast : generic;
}

hipError_t launch_bitv_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.k.D != kBvD || a.nbits < kBvRange || a.nbits > 2048 || a.nbits % kBvRange || a.n_chunks % (a.nbits / kBvRange))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(bitv_merge_kernel, dim3(a.Hq, a.B, 4), dim3(kBmThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_bitv_values(const DecodeArgs& a, hipStream_t stream) {
  if (a.k.D != kBvD || a.NH != 4 || a.Hq > 32 || a.nbits < kBvRange || a.nbits % kBvRange || a.chunk % 32 ||
      a.chunk > 4096 || a.n_chunks % (a.nbits / kBvRange) || !a.pw)
    return hipErrorInvalidValue;
  const dim3 grid(a.n_chunks, a.B);  // (ranges x chunks, sequences)
  if (a.Hq <= 16)
    hipLaunchKernelGGL(bitv_values_kernel<1>, grid, dim3(kBvThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(bitv_values_kernel<2>, grid, dim3(kBvThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace commvq

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
//     bytes: a rotate puts the lane's bit n of each half-word at bits 14 and
//     30, and a byte permute plus a mask makes each fp16 pair 2.0 or 0, so one
//     operand dword costs two instructions;
//   - the eight wavefronts' u are added through LDS, then thread (KV head,
//     dimension pair) forms o = u^T C over the range's 128 rows of C (fp32),
//     for the KV head's query heads, into the range's partial slot;
//   - the grid puts range r of chunk c at r * chunks + c; workgroups go to the
//     8 XCDs round-robin, so with a multiple of 8 chunks a chunk's ranges share
//     one XCD and its L2 copy of the chunk's weights.
// The merge kernel then combines the slots like any chunk partials (M equal
// across a chunk's ranges, l in the first only).

#include "decode_common.hpp"

namespace commvq {
namespace {

constexpr int kBvThreads = 512;
constexpr int kBvWaves = kBvThreads / 64;
constexpr int kBvRange = 128;   // code bits per workgroup
constexpr int kBvRow = 132;     // LDS row stride (floats) of the wavefront partials: 4 rows of a store hit 4 bank groups
constexpr int kBvURow = 36;     // LDS row stride (floats) of u [bit][head], 16-byte aligned rows
constexpr int kBvD = 128;       // head_dim of the fast path

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// NHT tiles of 16 query heads (Hq <= 16 NHT)
template <int NHT>
__global__ __launch_bounds__(kBvThreads, 1) void bitv_values_kernel(DecodeArgs a) {
  constexpr int HP = 16 * NHT;
  // region 0, in turn: the wavefront partials of u [w][head][bit]; the
  // contraction's partial outputs [row quarter][head][dim]
  constexpr int R0 = kBvWaves * 32 * kBvRow * 4;
  static_assert(4 * 32 * kBvD * 4 <= R0, "region 0");
  __shared__ __attribute__((aligned(16))) char r0[R0];
  __shared__ float ub[kBvRange * kBvURow];  // u [bit][head]
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
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 15, kg = lane >> 4;
  const uint32_t rot = (uint32_t)((n + 18) & 31);  // bit n -> 14, bit 16 + n -> 30
  const int nby = a.nbits / 8;
  const size_t plen = (size_t)npc * a.chunk;
  const uint8_t* vb = a.vbits + (size_t)b * a.cache_len * nby + 16 * r;
  const _Float16* pwb = a.pw + (size_t)b * a.Hq * plen;

  // operands of k-step ks (32 positions): the weights of heads 16 ht + n at
  // positions kb..kb+7 (a head past Hq reads row 0 and is zeroed by a select),
  // and the range's 16 code bytes of those 8 positions (clamped into the cache;
  // positions past the sequence have weight 0). Two k-steps are in flight ahead
  // of the one in use.
  struct Ops {
    h8_t a[NHT];
    u32x4 x[8];
  };
  auto load = [&](Ops& o, int ks) {
    const int kb = m0 + 32 * ks + 8 * kg;
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) {
      const int head = 16 * ht + n;
      const h8_t v = *reinterpret_cast<const h8_t*>(pwb + (size_t)(head < a.Hq ? head : 0) * plen + kb);
      o.a[ht] = head < a.Hq ? v : (h8_t){0, 0, 0, 0, 0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      o.x[j] = *reinterpret_cast<const u32x4*>(vb + (size_t)min(kb + j, a.cache_len - 1) * nby);
  };
  float4_t acc[NHT][8];
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[ht][t] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto step = [&](Ops& o, int ks) {
    uint32_t y[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) y[j][q] = __builtin_amdgcn_alignbit(o.x[j][q], o.x[j][q], rot);
    h8_t acur[NHT];
#pragma unroll
    for (int ht = 0; ht < NHT; ++ht) acur[ht] = o.a[ht];
    if (ks + 2 * kBvWaves < nks) load(o, ks + 2 * kBvWaves);  // refill this slot two k-steps ahead
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int q = t >> 1;
      const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;  // high or low half-words
      u32x4 bw;
#pragma unroll
      for (int e = 0; e < 4; ++e) bw[e] = __builtin_amdgcn_perm(y[2 * e + 1][q], y[2 * e][q], sel) & 0x40004000u;
      const h8_t bop = __builtin_bit_cast(h8_t, bw);
#pragma unroll
      for (int ht = 0; ht < NHT; ++ht)
        acc[ht][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(acur[ht], bop, acc[ht][t], 0, 0, 0);
    }
  };
  Ops o0, o1;
  if (wave < nks) load(o0, wave);
  if (wave + kBvWaves < nks) load(o1, wave + kBvWaves);
  for (int ks = wave; ks < nks; ks += 2 * kBvWaves) {
    step(o0, ks);
    if (ks + kBvWaves < nks) step(o1, ks + kBvWaves);
  }

  // lane holds u[16 ht + 4 kg + i][16 t + n] (times 2)
#pragma unroll
  for (int ht = 0; ht < NHT; ++ht)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) usum[(wave * HP + 16 * ht + 4 * kg + i) * kBvRow + 16 * t + n] = acc[ht][t][i];

  __syncthreads();
  // contraction operands, requested before the reduction (after the barrier,
  // so they do not share registers with the partials): thread (KV head kv, row
  // quarter qq, dimensions 8 d8 .. 8 d8 + 7) takes rows 32 qq .. 32 qq + 31 of
  // the range
  const int kv = tid >> 6, qq = (tid >> 4) & 3, d8 = tid & 15;
  const int dimc = a.k.Hkv * kBvD;
  const bool kv_ok = kv < a.k.Hkv;
  const _Float16* crow = a.vrows + (size_t)(kBvRange * r + 32 * qq) * dimc + (kv_ok ? kv : 0) * kBvD + 8 * d8;
  // four batches of 8 rows, each requested one batch ahead of its use (the
  // first before the reduction)
  h8_t cvb[2][8];
  auto load_rows = [&](h8_t (&dst)[8], int i0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = *reinterpret_cast<const h8_t*>(crow + (size_t)(i0 + i) * dimc);
  };
  load_rows(cvb[0], 0);
  for (int e = tid; e < HP * kBvRange; e += kBvThreads) {
    const int head = e / kBvRange, bit = e % kBvRange;
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kBvWaves; ++w) sum += usum[(w * HP + head) * kBvRow + bit];
    ub[bit * kBvURow + head] = 0.5f * sum;  // the bits entered as 2.0
  }
  __syncthreads();

  // o[4 kv + k][d] over the quarter's rows: sum_i u[4 kv + k][i] C[128 r + i][kv D + d]
  float o[4][8];
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[k][e] = 0.f;
#pragma unroll
  for (int bt = 0; bt < 4; ++bt) {
    if (bt < 3) load_rows(cvb[(bt + 1) & 1], 8 * (bt + 1));
    const h8_t (&cvh)[8] = cvb[bt & 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float4_t u4 = *reinterpret_cast<const float4_t*>(ub + (32 * qq + 8 * bt + i) * kBvURow + 4 * (kv_ok ? kv : 0));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float cf = (float)cvh[i][e];
#pragma unroll
        for (int k = 0; k < 4; ++k) o[k][e] = fmaf(u4[k], cf, o[k][e]);
      }
    }
  }
  float* osum = reinterpret_cast<float*>(r0);  // [quarter][head][dim] (u's partials are consumed)
  if (kv_ok) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      float* dst = osum + (qq * 32 + 4 * kv + k) * kBvD + 8 * d8;
      *reinterpret_cast<float4_t*>(dst) = (float4_t){o[k][0], o[k][1], o[k][2], o[k][3]};
      *reinterpret_cast<float4_t*>(dst + 4) = (float4_t){o[k][4], o[k][5], o[k][6], o[k][7]};
    }
  }
  __syncthreads();
  for (int e = tid; e < a.Hq * kBvD; e += kBvThreads) {
    const int hq = e / kBvD, d = e % kBvD;
    const float v = osum[hq * kBvD + d] + osum[(32 + hq) * kBvD + d] + osum[(64 + hq) * kBvD + d] +
                    osum[(96 + hq) * kBvD + d];
    a.part[(((size_t)b * a.Hq + hq) * a.n_chunks + (size_t)c * NR + r) * (kBvD + 2) + 2 + d] = v;
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

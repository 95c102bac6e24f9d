// Fast CommVQ decode attention for head_dim 128, g = 8, Nc' = 256, four query
// heads per KV head and R = 1 or 2 rounds (the 1-bit and 2-bit CommVQ of the
// LLaMA-3.1-8B layer shape).
//
// One workgroup (512 lanes, two wavefronts per SIMD) owns a chunk of C = 512*TL
// cached positions of one (sequence, KV head). Wavefront w handles blocks of 64
// consecutive positions m_b = m0 + 512 t + 64 w (t < TL), lane d taking m_b + d.
//
// Scores ("Pith review of CommVQ", "What carries the argument": the commuting
// codebook lets the query-dependent factor be formed once and reused for every
// cached position). With the phase split e^{i m theta} = e^{i m_b theta} e^{i d theta},
//   s = Re sum_p conj(q~_p e^{-i m_b theta_p}) (z_p e^{i d theta_p}),
// a real dot product over D between
//   q'_p = q~_p conj(e^{i m_b theta_p})   built once per block (fp16), and
//   k'_p = z_p e^{i d theta_p}           one codebook gather per group and a
//                                        rotation by lane-constant phases.
// No per-position phase is computed: block phases advance once per block, and
// the lane phases e^{i d theta_p}, d < 64, are constants. The dot products run
// on v_mfma_f32_4x4x4f16: block b of 16 takes positions 4b..4b+3 of the 64 as
// columns and the four query heads as rows, so lane d ends with its position's
// four scores; q' is broadcast from one block per instruction (CBSZ/ABID), so a
// lane holds it for two K-steps only. The key codebook of the head sits in LDS (64 KiB per
// round); k' is rotated in packed fp16 (v_pk_mul_f16 + v_pk_fma_f16).
// Values (review, "If this is right", fourth bullet: weights applied to the
// value codes before the codebook):
//   fixed-point weights are scattered into per-(round, code, group, head)
//   histograms with 64-bit LDS integer atomics (two heads per add); lanes
//   rotate over (group, head pair) to spread the adds over the banks. The
//   histogram is contracted with the value codebook on MFMA
//   (v_mfma_f32_4x4x4f16; per wavefront, 16 blocks = 2 groups x 8 bin segments
//   with two dimensions per lane; weights split into fp16 hi + lo parts).
// The chunk's (max, sum, o) go to the workspace; a second kernel merges the
// chunks of each (sequence, query head).

#include <type_traits>
#include <utility>

#include "decode_common.hpp"
#include "encode_common.hpp"

namespace commvq {
namespace {

constexpr int FT = 512;     // lanes per workgroup
constexpr int FW = FT / 64; // wavefronts per workgroup
constexpr int FNH = 4;      // query heads per KV head
constexpr int FD = 128;     // head_dim
constexpr int FG = 16;      // groups of g = 8
constexpr int FPR = 64;     // RoPE pairs
constexpr int FNC = 256;    // entries per codebook

template <int R>
struct FastCfg {
  static constexpr int BPT = 16 * R;                   // bytes per packed record
  static constexpr int KCB = R * FG * FNC * 16;        // key codebook bytes (64 KiB per round)
  static constexpr int HIST = R * FNC * FG * FNH * 4;  // histogram bytes (64 KiB per round)
  static constexpr int MAIN = 131072;                  // LDS region for both
  // R = 1: the histogram sits beside the key codebook, each wavefront clearing
  // its slice as it leaves the score loop; R = 2: it replaces the codebook once
  // all scores are done
  static constexpr int HOFF = R == 1 ? KCB : 0;
  static_assert(HOFF + HIST <= MAIN && KCB <= MAIN && (R == 2 || HOFF >= KCB), "layout");
};

// aux LDS: lane phases [64 offsets][64 pairs] fp16 (16-byte chunks swizzled),
// rotated query [4][64], reductions [64], and a decode step's new token:
// codes [2][2][16], scores [4], value [128]
constexpr int PHT_BYTES = 64 * FPR * 4;
// decode step, R = 1: per (sequence, KV head) the new key's group products
// q~.k~ [16 groups][4 heads], then its value [128]
constexpr int NEWTOK_FLOATS = kFastNewTokFloats;
static_assert(NEWTOK_FLOATS == FG * FNH + FD, "new-token record");
constexpr int NEW_BYTES = 64 + FNH * 4 + FD * 4;
constexpr int AUX_BYTES = PHT_BYTES + FNH * FPR * 8 + 64 * 4 + NEW_BYTES;
static_assert(131072 + AUX_BYTES <= 160 * 1024, "LDS budget");
static_assert(FT == FNH * FD && PHT_BYTES >= FW * FNH * FD * 4, "contraction: one output per lane, wavefront partials in the phase table's space");
static_assert(PHT_BYTES >= 4 * 4096, "value-codebook slabs reuse the lane phase table");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, half2_t));
}

// (x + iy)(c + is) on packed fp16 pairs z = (x, y), e = (c, s): t = (x c, y c),
// then (y, x) (-s, s) + t = (x c - y s, y c + x s); the compiler folds the swap,
// the broadcasts and the negation into operand selects of one v_pk_mul_f16 and
// one v_pk_fma_f16. The empty asm makes z an opaque register value: without it
// the swap of a vector's first element was materialised by a separate
// instruction.
__device__ __forceinline__ uint32_t rotate_h2(uint32_t z, uint32_t e) {
  asm("" : "+v"(z));
  const half2_t zz = __builtin_bit_cast(half2_t, z), ee = __builtin_bit_cast(half2_t, e);
  const half2_t t = zz * (half2_t){ee.x, ee.x};
  const half2_t zs = {zz.y, zz.x};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(zs, (half2_t){-ee.y, ee.y}, t));
}

// Packed fp16 sum of two (x, y) pairs. Elements of a 32-bit vector are passed
// to it by value: a bit cast applied directly to a vector element expression has
// been seen to read element 0 whatever the index.
__device__ __forceinline__ uint32_t add_h2(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) + __builtin_bit_cast(half2_t, b));
}

// 16 * byte B of w in one instruction (a byte-select operand); used for LDS
// gather offsets of 16-byte codebook entries.
template <int B>
__device__ __forceinline__ uint32_t byte_x16(uint32_t w) {
  uint32_t r;
  if constexpr (B == 0)
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  if constexpr (B == 1)
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  if constexpr (B == 2)
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  if constexpr (B == 3)
    asm("v_lshlrev_b32_sdwa %0, 4, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  return r;
}

__device__ __forceinline__ half4_t as_h4(uint32_t lo, uint32_t hi) {
  return __builtin_bit_cast(half4_t, (u32x2){lo, hi});
}

// Real and imaginary parts of z e + c for packed fp16 pairs z = (x, y) and
// e = (c, s), in fp32: v_dot2_f32_f16 forms both products exactly and adds them
// in fp32. The real part takes z as (x, -y), the imaginary part as (y, x).
__device__ __forceinline__ float cdot(uint32_t zv, uint32_t e, float c) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, zv), __builtin_bit_cast(half2_t, e), c, false);
}
__device__ __forceinline__ uint32_t conj_h2(uint32_t z) { return z ^ 0x80000000u; }       // (x, -y)
__device__ __forceinline__ uint32_t swap_h2(uint32_t z) { return __builtin_amdgcn_alignbit(z, z, 16); }  // (y, x)

// Largest standard deviation of the scaled scores over the valid positions of a
// wavefront beyond which its scores are recomputed in fp32 (see the precision
// guard in the kernel).
constexpr float kFastSigmaMax = 2.0f;

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));

// Decode step, R = 1: one group of the new token's key or value searched by a
// wavefront over entries l = lane + 64 k held in ent[k]. The input is fp16, so
// e.c and |c|^2 are fp32 sums of exact fp16 products (v_dot2_f32_f16), and
// score(c) = |c|^2 / 2 - e.c orders the entries as |e - c|^2; lowest index on
// ties. Returns the chosen entry and leaves its eight values in win (every lane).
__device__ __forceinline__ int search_row64_dot(const half2_t (&e2)[4], const h8_t (&ent)[4], int lane, u32x4& win) {
  float best = INFINITY;
  int bi = 0x7fffffff;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float ec = 0.f, cc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const half2_t c2 = {ent[k][2 * i], ent[k][2 * i + 1]};
      ec = __builtin_amdgcn_fdot2(e2[i], c2, ec, false);
      cc = __builtin_amdgcn_fdot2(c2, c2, cc, false);
    }
    const float sc = fmaf(cc, 0.5f, -ec);
    if (sc < best) {
      best = sc;
      bi = lane + 64 * k;
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
  if (bi == 0x7fffffff) bi = 0;  // (no score below +inf: non-finite input)
  // the winner's entry sits in lane bi % 64, slot bi / 64
  const int ks = bi >> 6;
  const u32x4 mine = __builtin_bit_cast(u32x4, ks == 0 ? ent[0] : ks == 1 ? ent[1] : ks == 2 ? ent[2] : ent[3]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t mi = mine[i];
    win[i] = (uint32_t)__shfl((int)mi, bi & 63, 64);
  }
  return bi;
}

// BV: binary value codes (a.vbits). The workgroup then stops after the
// softmax: it writes its positions' weights e^{s - M} (fp16, a.pw) and the
// chunk's (M, l) into each of its nbits / 128 partial slots (one per range of
// value-code bits; l in the first only); bitv_values_kernel adds each range's
// u.
template <int R, int TL, bool BV>
__global__ __launch_bounds__(FT, 1) void decode_fast_kernel(DecodeArgs a, PhaseTable ph) {
  using Cfg = FastCfg<R>;
  constexpr int BPT = Cfg::BPT;
  constexpr int C = FT * TL;
  constexpr int FXSHIFT = 31 - (C == 4096 ? 12 : C == 2048 ? 11 : 10);  // C * 2^FXSHIFT = 2^31
  static_assert(C <= 4096, "shape");

  __shared__ uint4 fsm[(131072 + AUX_BYTES) / 16];  // static: its LDS address (0) folds into offsets
  char* lds = reinterpret_cast<char*>(fsm);
  uint32_t* pht = reinterpret_cast<uint32_t*>(lds + Cfg::MAIN);       // [64][64] fp16 (cos, sin)
  float2* qz = reinterpret_cast<float2*>(lds + Cfg::MAIN + PHT_BYTES);  // [4][64] rotated query
  float* red = reinterpret_cast<float*>(qz + FNH * FPR);               // [64] reductions
  uint8_t* new_codes = reinterpret_cast<uint8_t*>(red + 64);         // [2][R][16]
  float* new_s = reinterpret_cast<float*>(new_codes + 64);           // [4] scaled scores
  float* new_v = new_s + FNH;                                        // [128]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are handed to the 8 XCDs round-robin in launch order; putting the
  // KV head in the fastest-varying position keeps one head's chunks (and its
  // codebooks) on one XCD's L2 when there are 8 KV heads.
  const int h = blockIdx.x % a.k.Hkv, chunk = blockIdx.x / a.k.Hkv, b = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int m0 = chunk * C;
  const int NR = BV ? a.nbits / 128 : 1;  // partial slots per chunk
  const size_t pstride = (size_t)a.n_chunks * (FD + 2);
  float* part = a.part + ((size_t)b * a.Hq + h * FNH) * pstride + (size_t)chunk * NR * (FD + 2);
  // the query pair this lane rotates (lanes < 256: head tid / 64, pair tid % 64),
  // requested before anything else
  const float2 qx = tid < FNH * FPR
                        ? *reinterpret_cast<const float2*>(a.q + ((size_t)b * a.Hq + h * FNH + (tid >> 6)) * FD +
                                                           2 * (tid & 63))
                        : make_float2(0.f, 0.f);
  const int qpos = a.q_pos[b];
  // turn counts of this lane's RoPE pair (pair = lane in the phase table and the
  // query rotation) and of the four pairs whose block phases it carries; loaded
  // first, the kernel-argument table being indexed per lane
  const uint32_t flo = ph.lo[lane], fhi = ph.hi[lane];
  uint32_t bflo[4], bfhi[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = 2 * (lane >> 2) + (u & 1) + 32 * (u >> 1);
    bflo[u] = ph.lo[p];
    bfhi[u] = ph.hi[p];
  }
  const uint8_t* kb = a.kcodes + ((size_t)b * a.k.Hkv + h) * (size_t)a.cache_len * BPT;
  // record of the lane's position in block t, clamped into the cache (not the
  // sequence, so the loads need not wait for seq_lens; positions past the
  // sequence are masked after the scores)
  auto load_rec = [&](int t, uint32_t (&cw)[R][4]) {
    const int mm = min(m0 + tid + FT * t, a.cache_len - 1);
    const u32x4* rec = reinterpret_cast<const u32x4*>(kb + (size_t)mm * BPT);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const u32x4 v = rec[r];
#pragma unroll
      for (int k = 0; k < 4; ++k) cw[r][k] = v[k];
    }
  };
  constexpr int NB = (R == 1) ? (TL < 3 ? TL : 3) : 2;  // records in flight
  constexpr int PD = (R == 1) ? 4 : 2;   // codebook gathers in flight (groups)
  uint32_t cw[NB][R][4];
#pragma unroll
  for (int t = 0; t < NB - (NB < TL ? 1 : 0); ++t) load_rec(t, cw[t]);

  // ---- per-workgroup constants ------------------------------------------
  // the head's key codebook, [G][R][Nc'][8] fp16 as in HBM: all loads are issued
  // before the lane phases are computed and stored to LDS after
  constexpr int NKCB = Cfg::KCB / 16 / FT;
  u32x4 kcv[NKCB];
  {
    const u32x4* src = reinterpret_cast<const u32x4*>(a.kcb + (size_t)h * FG * R * FNC * 8);
#pragma unroll
    for (int k = 0; k < NKCB; ++k) kcv[k] = src[tid + FT * k];
  }
  // decode step: the workgroup whose chunk holds the new position leaves that
  // position out of its table path (its record is being written). R = 2: that
  // workgroup encodes the new key and value of its KV head (all 32 group
  // searches at once, 16 lanes each), writes the records, and the token joins
  // the chunk's partial with an exact fp32 score at the end.
  const int pb = a.k_new ? a.positions[b] : -1;
  const bool appended = a.k_new && pb >= 0 && pb < a.cache_len;
  const int skip_pos = appended ? pb : -1;
  const bool owner = R != 1 && appended && chunk == min(pb / C, a.n_chunks - 1);
  // R = 1: the 32 searches (K, then V, of the 16 groups) are spread over the
  // head's workgroups: slot i of the workgroup of chunk c takes search
  // c + i * n_chunks, and wavefront w the slots w, w + 8, ... The first slot's
  // inputs are loaded here, the search runs after the set-up, and the results
  // go to the record and to the workspace, where the merge kernel adds the new
  // token as one more chunk (its score from the 16 group products, its value).
  auto row_of = [&](int it) { return chunk + (wave + FW * it) * a.n_chunks; };
  half2_t rx[4];
  h8_t rent[4];
  float2 rq = make_float2(0.f, 0.f);
  uint32_t rlo = 0, rhi = 0;
  auto row_load = [&](int rho) {
    const int rkv = rho >= FG ? 1 : 0, rj = rho & (FG - 1);
    const half2_t* x = reinterpret_cast<const half2_t*>((rkv ? a.v_new : a.k_new) + ((size_t)b * a.k.Hkv + h) * FD + rj * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) rx[i] = x[i];
    const _Float16* cbg = (rkv ? a.vcb : a.kcb) + ((size_t)h * FG + rj) * FNC * 8;
#pragma unroll
    for (int k = 0; k < 4; ++k) rent[k] = *reinterpret_cast<const h8_t*>(cbg + (size_t)(lane + 64 * k) * 8);
    if (!rkv && lane < 16) {  // lane (head lane / 4, pair 4 rj + lane % 4): the query pair and its turn counts
      const int p = 4 * rj + (lane & 3);
      rq = *reinterpret_cast<const float2*>(a.q + ((size_t)b * a.Hq + h * FNH + (lane >> 2)) * FD + 2 * p);
      rlo = ph.lo[p];
      rhi = ph.hi[p];
    }
  };
  auto row_job = [&]() {
    if (!(R == 1 && appended)) return;
    for (int it = 0; it < 4; ++it) {
      const int rho = row_of(it);
      if (rho >= 2 * FG) break;
      if (it > 0) row_load(rho);
      const int rkv = rho >= FG ? 1 : 0, rj = rho & (FG - 1);
      u32x4 win;
      const int code = search_row64_dot(rx, rent, lane, win);
      if (lane == 0) (rkv ? a.vcodes_w : a.kcodes_w)[(((size_t)b * a.k.Hkv + h) * a.cache_len + pb) * BPT + rj] = (uint8_t)code;
      float* nt = a.newtok + ((size_t)b * a.k.Hkv + h) * NEWTOK_FLOATS;
      if (rkv) {
        if (lane < 8) {
          const int u = lane >> 1;
          const uint32_t w2 = u == 0 ? win[0] : u == 1 ? win[1] : u == 2 ? win[2] : win[3];
          const half2_t vh = __builtin_bit_cast(half2_t, w2);  // (a scalar copy: bit_cast of a vector element misreads)
          nt[FG * FNH + 8 * rj + lane] = (float)((lane & 1) ? vh.y : vh.x);
        }
      } else {
        // q~_p k~_p for lane (head lane / 4, pair lane % 4), both rotations in fp32
        const int u = lane & 3;
        const uint32_t kw = u == 0 ? win[0] : u == 1 ? win[1] : u == 2 ? win[2] : win[3];
        const half2_t kp = __builtin_bit_cast(half2_t, kw);
        const float2 wq = phase_hw((uint32_t)max(qpos, 0), rlo, rhi), wk = phase_hw((uint32_t)pb, rlo, rhi);
        const float qx2 = rq.x * wq.x - rq.y * wq.y, qy2 = rq.x * wq.y + rq.y * wq.x;
        const float kx = (float)kp.x, ky = (float)kp.y;
        const float kx2 = kx * wk.x - ky * wk.y, ky2 = kx * wk.y + ky * wk.x;
        float c = qx2 * kx2 + qy2 * ky2;
        c += __shfl_xor(c, 1, 64);
        c += __shfl_xor(c, 2, 64);
        if (lane < 16 && u == 0) nt[rj * FNH + (lane >> 2)] = c;
      }
    }
  };
  if (owner) {
    const int row = tid >> 4, kv = row / FG, j = row % FG;
    const _Float16* x = (kv ? a.v_new : a.k_new) + ((size_t)b * a.k.Hkv + h) * FD + j * 8;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (float)x[i];
    const _Float16* cbg = (kv ? a.vcb : a.kcb) + ((size_t)h * FG + j) * R * FNC * 8;
    greedy_group_row16(e, cbg, FNC, R, tid & 15, new_codes + kv * R * FG + j, FG);
    __syncthreads();
    if (tid < 2 * BPT) {  // 8-bit fields: the record is the codes, round-major
      const int kv2 = tid / BPT, k = tid % BPT;
      uint8_t* cache = kv2 ? a.vcodes_w : a.kcodes_w;
      cache[(((size_t)b * a.k.Hkv + h) * a.cache_len + pb) * BPT + k] = new_codes[kv2 * BPT + k];
    }
  }

  // the decode step's first search inputs (after the loads that do not wait on
  // the step's positions)
  const bool rowjob = R == 1 && appended && row_of(0) < 2 * FG;
  if (rowjob) row_load(row_of(0));
  // a chunk wholly past the sequence contributes an empty partial (its loads were
  // issued before the length was known; they stay unused)
  if (m0 >= L) {
    // (uses of the set-up's loads on this path too, so that the compiler keeps
    // them ahead of the length test instead of sinking them past it)
#pragma unroll
    for (int k = 0; k < NKCB; ++k) asm volatile("" ::"v"(kcv[k]));
#pragma unroll
    for (int t = 0; t < NB - (NB < TL ? 1 : 0); ++t)
#pragma unroll
      for (int r = 0; r < R; ++r) asm volatile("" ::"v"(cw[t][r][0]), "v"(cw[t][r][1]), "v"(cw[t][r][2]), "v"(cw[t][r][3]));
    for (int i = tid; i < FNH * NR * (FD + 2); i += FT) {
      const int hh = i / (NR * (FD + 2)), k = i % (NR * (FD + 2));
      part[hh * pstride + k] = (k % (FD + 2) == 0) ? -INFINITY : 0.f;
    }
    row_job();
    return;
  }
  // lane phases e^{i d theta_p}, d < 64: 16-byte chunk c (pairs 4c..4c+3) of row d
  // at slot (c + d) & 15, so the 64 lanes reading chunk c hit 16 different slots.
  // Lane p (the pair) of wavefront w takes offsets d = w + 8 k: e^{i w theta}
  // from the hardware sine and cosine, then seven steps of e^{i 8 theta} in fp32.
  {
    static_assert(FT / 64 == 8, "eight offsets per lane");
    const float2 st = phase_hw(8u, flo, fhi);
    float2 e = phase_hw((uint32_t)wave, flo, fhi);
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int d = wave + 8 * k, p = lane;
      pht[d * 64 + (((p >> 2) + d) & 15) * 4 + (p & 3)] = pack_h2(e.x, e.y);
      e = make_float2(e.x * st.x - e.y * st.y, e.x * st.y + e.y * st.x);
    }
  }
#pragma unroll
  for (int k = 0; k < NKCB; ++k) reinterpret_cast<u32x4*>(lds)[tid + FT * k] = kcv[k];
  if (tid < FNH * FPR) {
    const float2 w = phase_hw((uint32_t)max(qpos, 0), flo, fhi);  // pair tid & 63 = lane
    qz[tid] = make_float2(qx.x * w.x - qx.y * w.y, qx.x * w.y + qx.y * w.x);
  }

  const bool fold = owner && pb < L;
  if (fold) {
    __syncthreads();  // rotated query visible
    if (wave == 0) {
      // exact fp32 score of the new key for the four query heads (lane = RoPE pair)
      const int p = lane, j = p >> 2, pp = p & 3;
      float kx = 0.f, ky = 0.f;
      for (int r = 0; r < R; ++r) {
        const _Float16* ce = a.kcb + ((((size_t)h * FG + j) * R + r) * FNC + new_codes[r * FG + j]) * 8 + 2 * pp;
        kx += (float)ce[0];
        ky += (float)ce[1];
      }
      const float2 wk = phase_hw((uint32_t)pb, flo, fhi);  // p = lane
      const float krx = kx * wk.x - ky * wk.y, kry = kx * wk.y + ky * wk.x;
#pragma unroll
      for (int k = 0; k < FNH; ++k) {
        const float2 qv = qz[k * FPR + p];
        const float sc = wave_sum(qv.x * krx + qv.y * kry);
        if (lane == 0) new_s[k] = sc * a.sm_scale;
      }
    } else if (tid >= 128 && tid < 256) {
      // its dequantised value, one dimension per lane
      const int d = tid - 128, j = d >> 3, ee = d & 7;
      float v = 0.f;
      for (int r = 0; r < R; ++r)
        v += (float)a.vcb[((((size_t)h * FG + j) * R + r) * FNC + new_codes[BPT + r * FG + j]) * 8 + ee];
      new_v[d] = v;
    }
  }
  __syncthreads();  // codebook, lane phases and rotated query visible
  row_job();

  // lane constants: e^{i lane theta_p} for the 64 pairs (packed fp16)
  uint32_t el[FPR];
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(pht + lane * 64 + ((c + lane) & 15) * 4);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      el[4 * c + k] = v[k];
      asm("" : "+v"(el[4 * c + k]));  // kept in registers, not re-read from LDS in the loop
    }
  }

  // ---- scores -------------------------------------------------------------
  // MFMA A operand (q'): instruction k (K-step k = pairs 2k, 2k+1) broadcasts
  // block k % 16's A to all 16 blocks (CBSZ = 4, ABID = k % 16), so lane
  // (block bq, row qi) only holds head qi's q' for K-steps bq and bq + 16: pairs
  // 2 bq, 2 bq + 1, 2 bq + 32, 2 bq + 33. They start from an exact block phase
  // and advance as q' <- q' conj(e^{i 512 theta_p}) per block (fp32).
  const int qi = lane & 3, bq = lane >> 2;
  float2 qf[4], stp[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int p = 2 * bq + (u & 1) + 32 * (u >> 1);
    const float2 qv = qz[qi * FPR + p];
    const float2 eb = phase_hw((uint32_t)(m0 + 64 * wave), bflo[u], bfhi[u]);
    qf[u] = make_float2(fmaf(qv.x, eb.x, qv.y * eb.y), fmaf(qv.y, eb.x, -qv.x * eb.y));
    stp[u] = phase_hw((uint32_t)FT, bflo[u], bfhi[u]);
  }
  float s[TL][FNH];
  // Two wavefronts share each SIMD. The scheduler favours the older one, which
  // would race ahead and leave the other to run alone (no latency hiding) at
  // the end; a wavefront's issue priority instead falls as it advances through
  // its blocks, so the pair stays interleaved.
  static_for<TL>([&](auto tc) {
    constexpr int t = decltype(tc)::value;
    __builtin_amdgcn_s_setprio(3 - (4 * t) / TL);
    if constexpr (NB < TL) {
      if (t + NB - 1 < TL) load_rec(t + NB - 1, cw[(t + NB - 1) % NB]);
    }
    const uint32_t (&cr)[R][4] = cw[t % NB];
    // codebook gathers run PD groups ahead of their use (rolling buffer), the
    // first PD issued before the block's q' is formed
    u32x4 zb[PD][R];
    auto gather = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const uint32_t off = byte_x16<j & 3>(cr[r][j >> 2]);  // code * 16
        zb[j % PD][r] = *reinterpret_cast<const u32x4*>(lds + (size_t)(j * R + r) * FNC * 16 + off);
      }
    };
    static_for<PD>(gather);
    if (t > 0) {
#pragma unroll
      for (int u = 0; u < 4; ++u)
        qf[u] = make_float2(fmaf(qf[u].x, stp[u].x, qf[u].y * stp[u].y), fmaf(qf[u].y, stp[u].x, -qf[u].x * stp[u].y));
    }
    // q' = q~ conj(e_b) as fp16 (re, im); qa[0..1]: K-step bq, qa[2..3]: K-step bq + 16
    uint32_t qa[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) qa[u] = pack_h2(qf[u].x, qf[u].y);
    const half4_t a_lo = as_h4(qa[0], qa[1]), a_hi = as_h4(qa[2], qa[3]);
    float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    static_for<FG>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      u32x4 z = zb[j % PD][0];
#pragma unroll
      for (int r = 1; r < R; ++r)
#pragma unroll
        for (int k = 0; k < 4; ++k) z[k] = add_h2(z[k], zb[j % PD][r][k]);
      if constexpr (j + PD < FG) gather(std::integral_constant<int, j + PD>{});
      const uint32_t k0 = rotate_h2(z[0], el[4 * j]), k1 = rotate_h2(z[1], el[4 * j + 1]);
      const uint32_t k2 = rotate_h2(z[2], el[4 * j + 2]), k3 = rotate_h2(z[3], el[4 * j + 3]);
      // K-steps 2j (pairs 4j, 4j+1) and 2j + 1 (pairs 4j+2, 4j+3)
      const half4_t aop = j < 8 ? a_lo : a_hi;
      acc0 = __builtin_amdgcn_mfma_f32_4x4x4f16(aop, as_h4(k0, k1), acc0, 4, (2 * j) & 15, 0);
      acc1 = __builtin_amdgcn_mfma_f32_4x4x4f16(aop, as_h4(k2, k3), acc1, 4, (2 * j + 1) & 15, 0);
    });
#pragma unroll
    for (int k = 0; k < FNH; ++k) s[t][k] = acc0[k] + acc1[k];
  });
  __builtin_amdgcn_s_setprio(0);

  // ---- precision guard ----------------------------------------------------
  // The fp16 roundings above (q', the lane phases, k') leave each score an error
  // of about 2^-11 of the spread of its terms, and the softmax passes it on the
  // more strongly the scores spread. When the standard deviation of a
  // wavefront's scaled scores (valid positions, any of the four heads) exceeds
  // kFastSigmaMax, the wavefront recomputes its scores: lane phases as fp16
  // hi + lo parts, k' formed in fp32 (exact fp16 products), q' in fp32 from an
  // exact block phase, and the dot products on v_mfma_f32_4x4x1f32.
  bool precise = false;
  {
    // per head, one pass: the sums of s and s^2 over the valid positions, taken
    // about one of the wavefront's scores (the spread does not depend on the
    // shift, and the sums of squares stay small)
    float wv[TL], nv = 0.f;
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const int mt = m0 + tid + FT * t;
      wv[t] = (mt < L && mt != skip_pos) ? 1.f : 0.f;
      nv += wv[t];
    }
    const float n = wave_sum(nv);
    if (n > 1.f) {
      float vmax = 0.f;
#pragma unroll
      for (int k = 0; k < FNH; ++k) {
        const float c0 = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, s[0][k])));
        float a1 = 0.f, a2 = 0.f;
#pragma unroll
        for (int t = 0; t < TL; ++t) {
          const float dv = wv[t] * (s[t][k] - c0);
          a1 += dv;
          a2 = fmaf(dv, dv, a2);
        }
        const float m1 = wave_sum(a1) / n;
        vmax = fmaxf(vmax, wave_sum(a2) / n - m1 * m1);
      }
      precise = vmax * a.sm_scale * a.sm_scale > kFastSigmaMax * kFastSigmaMax;
    }
  }
  if (precise) {
    // low parts of the lane phases: e^{i lane theta_p} (hardware sine and cosine
    // of the exact turn count) less its fp16 value el[p]
    uint32_t elo[FPR];
#pragma unroll
    for (int p = 0; p < FPR; ++p) {
      const float2 e = phase_hw((uint32_t)lane, ph.lo[p], ph.hi[p]);
      const half2_t hi = __builtin_bit_cast(half2_t, el[p]);
      elo[p] = pack_h2(e.x - (float)hi.x, e.y - (float)hi.y);
    }
    // MFMA A operand: instruction (pair p, part c) broadcasts block p % 16, whose
    // lane (block j, row qi) holds head qi's q'_p, p = j + 16 r, as qa[2 r + c]
    const int pj = lane >> 2;
    static_for<TL>([&](auto tc) __attribute__((always_inline)) {
      constexpr int t = decltype(tc)::value;
      uint32_t cr[R][4];
      load_rec(t, cr);
      const uint32_t mb = (uint32_t)(m0 + 64 * wave + FT * t);
      // (the rotated query and the turn counts are re-read per block, not kept
      // in registers across blocks)
      asm volatile("" ::: "memory");
      float qa[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = pj + 16 * r;
        const float2 q0 = qz[qi * FPR + p];
        const float2 eb = phase_hw(mb, ph.lo[p], ph.hi[p]);
        qa[2 * r] = fmaf(q0.x, eb.x, q0.y * eb.y);
        qa[2 * r + 1] = fmaf(q0.y, eb.x, -q0.x * eb.y);
      }
      float4_t acc[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
      static_for<FG>([&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        u32x4 z[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t off = byte_x16<j & 3>(cr[r][j >> 2]);  // code * 16
          z[r] = *reinterpret_cast<const u32x4*>(lds + (size_t)(j * R + r) * FNC * 16 + off);
        }
        // two pairs' four k' components first, then their four products: a
        // dot-product result must not reach the matrix core right after it is
        // written (read too soon, the product took a stale operand)
        static_for<2>([&](auto hc) __attribute__((always_inline)) {
          constexpr int hh = decltype(hc)::value;
          float kx[2], ky[2];
          static_for<2>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = 2 * hh + decltype(uc)::value, p = 4 * j + u, i = decltype(uc)::value;
            if constexpr (R == 1) {
              const uint32_t zc = conj_h2(z[0][u]), zw = swap_h2(z[0][u]);
              kx[i] = cdot(zc, el[p], cdot(zc, elo[p], 0.f));
              ky[i] = cdot(zw, el[p], cdot(zw, elo[p], 0.f));
            } else {
              // (z1 + z2) e: both rounds against the high part exactly, their
              // fp16 sum against the low part (its rounding scaled by 2^-12)
              const uint32_t zs = add_h2(z[0][u], z[1][u]);
              kx[i] = cdot(conj_h2(z[0][u]), el[p], cdot(conj_h2(z[1][u]), el[p], cdot(conj_h2(zs), elo[p], 0.f)));
              ky[i] = cdot(swap_h2(z[0][u]), el[p], cdot(swap_h2(z[1][u]), el[p], cdot(swap_h2(zs), elo[p], 0.f)));
            }
          });
          // the wait takes the four values as operands, so every product is
          // issued after it and at least eight wait states after the last write
          asm volatile("s_nop 7" : "+v"(kx[0]), "+v"(ky[0]), "+v"(kx[1]), "+v"(ky[1]));
          static_for<2>([&](auto uc) __attribute__((always_inline)) {
            constexpr int u = 2 * hh + decltype(uc)::value, p = 4 * j + u, i = decltype(uc)::value;
            acc[2 * i] = __builtin_amdgcn_mfma_f32_4x4x1f32(qa[2 * (p >> 4)], kx[i], acc[2 * i], 4, p & 15, 0);
            acc[2 * i + 1] = __builtin_amdgcn_mfma_f32_4x4x1f32(qa[2 * (p >> 4) + 1], ky[i], acc[2 * i + 1], 4, p & 15, 0);
          });
        });
      });
#pragma unroll
      for (int k = 0; k < FNH; ++k) s[t][k] = (acc[0][k] + acc[1][k]) + (acc[2][k] + acc[3][k]);
    });
  }

  // value records of the lane's positions, requested now so they arrive during
  // the softmax; dword k of round r is taken from slot (k + q4) & 3 (the lane's
  // rotation over groups in the histogram stage)
  const int g16 = tid & 15, h16 = (tid >> 4) & 1;
  const int q4 = (g16 >> 2) & 3, sh4 = g16 & 3;
  uint32_t ve[TL][R][4];  // (unused, and removed, when BV)
  if constexpr (!BV) {
    const uint8_t* vb = a.vcodes + ((size_t)b * a.v.Hkv + h) * (size_t)a.cache_len * BPT;
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const uint8_t* rec = vb + (size_t)min(m0 + tid + FT * t, a.cache_len - 1) * BPT;
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int k = 0; k < 4; ++k) ve[t][r][k] = *reinterpret_cast<const uint32_t*>(rec + r * 16 + 4 * ((k + q4) & 3));
    }
  }

  // ---- softmax over the chunk ---------------------------------------------
  // Each wavefront exponentiates against its own maximum M_w before the
  // workgroup's M is known (while slower wavefronts finish their scores); the
  // factor e^{M_w - M} then enters the fixed-point scale of the histogram stage,
  // and the wavefront sums are combined with it at the end.
  float M[FNH], fw[FNH], lsum[FNH];
  if constexpr (!BV && Cfg::HOFF >= Cfg::KCB) {
    uint4* hs = reinterpret_cast<uint4*>(lds + Cfg::HOFF) + wave * (Cfg::HIST / 16 / FW);
#pragma unroll
    for (int i = 0; i < Cfg::HIST / 16 / FT; ++i) hs[lane + 64 * i] = make_uint4(0, 0, 0, 0);
  }
#pragma unroll
  for (int t = 0; t < TL; ++t) {
    const int mt = m0 + tid + FT * t;
    const bool ok = mt < L && mt != skip_pos;
#pragma unroll
    for (int k = 0; k < FNH; ++k) s[t][k] = ok ? s[t][k] * a.sm_scale : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TL; ++t) mx = fmaxf(mx, s[t][k]);
    mx = wave_max(mx);
    fw[k] = mx;
    const float ref = mx == -INFINITY ? 0.f : mx;  // a wavefront may hold only masked positions
    float acc = 0.f;
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const float pw = __expf(s[t][k] - ref);  // exp(-inf) = 0 for masked positions
      s[t][k] = pw;
      acc += pw;
    }
    acc = wave_sum(acc);
    if (lane == 0) {
      red[k * FW + wave] = mx;
      red[32 + k * FW + wave] = acc;
    }
  }
  __syncthreads();  // also: every lane is done with the key codebook
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float mx = red[k * FW];
#pragma unroll
    for (int w = 1; w < FW; ++w) mx = fmaxf(mx, red[k * FW + w]);
    M[k] = mx;
    fw[k] = fw[k] == -INFINITY ? 0.f : __expf(fw[k] - mx);
  }
  // the chunk's sums: lane l < 32 scales wavefront l % 8's sum of head l / 8
  // from its own maximum, and the eight terms of a head are added in a row
  {
    const int kk = (lane >> 3) & 3, ww = lane & 7;
    const float mw = red[kk * FW + ww], mk = red[kk * FW];
    float mkx = mk;
#pragma unroll
    for (int w = 1; w < FW; ++w) mkx = fmaxf(mkx, red[kk * FW + w]);
    float term = (lane < 32 && mw != -INFINITY) ? red[32 + kk * FW + ww] * __expf(mw - mkx) : 0.f;
    term += dpp_f<0xb1>(term);   // quad_perm [1,0,3,2]
    term += dpp_f<0x4e>(term);   // quad_perm [2,3,0,1]
    term += __shfl_xor(term, 4, 64);
#pragma unroll
    for (int k = 0; k < FNH; ++k)
      lsum[k] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, term), 8 * k));
  }
  if constexpr (BV) {
    // weights e^{s - M} = e^{s - M_w} e^{M_w - M} of the lane's positions
    // (0 past the sequence), rows [B][Hq][n_pos_chunks * C]
    const size_t plen = (size_t)(a.n_chunks / NR) * C;
    _Float16* pwb = a.pw + ((size_t)b * a.Hq + h * FNH) * plen;
#pragma unroll
    for (int t = 0; t < TL; ++t)
#pragma unroll
      for (int k = 0; k < FNH; ++k) pwb[k * plen + m0 + tid + FT * t] = (_Float16)(s[t][k] * fw[k]);
    if (tid < FNH * NR) {
      const int hh = tid / NR, rr = tid % NR;
      float mk = M[0], lk = lsum[0];
#pragma unroll
      for (int k = 1; k < FNH; ++k)
        if (hh == k) {
          mk = M[k];
          lk = lsum[k];
        }
      part[hh * pstride + rr * (FD + 2)] = mk;
      part[hh * pstride + rr * (FD + 2) + 1] = rr == 0 ? lk : 0.f;
    }
    return;
  }
  if constexpr (Cfg::HOFF < Cfg::KCB) {
    // the histograms replace the key codebook
    for (int i = tid; i < Cfg::HIST / 16; i += FT) reinterpret_cast<uint4*>(lds + Cfg::HOFF)[i] = make_uint4(0, 0, 0, 0);
    __syncthreads();
  }

  // Value-codebook operands of the MFMA contraction at the end, requested a
  // slice per block of the histogram stage below, as that block's value records
  // free their registers (one head's codebook is shared by all its chunks, so
  // these mostly hit L2). Wavefront w contracts bins w * BPW .. + BPW - 1 (a bin
  // is a (round, code) pair, r * 256 + code) of all 16 groups: MFMA block grp
  // (lanes 4 grp .. 4 grp + 3) is group grp, its column mi two dimensions
  // (2 mi, 2 mi + 1; one dword per bin), and step st covers 4 bins.
  constexpr int NBIN = R * FNC, BPW = NBIN / FW, NSTEP = BPW / 4;
  static_assert(NSTEP % TL == 0, "codebook slices per block");
  const int mgrp = lane >> 2, mi = lane & 3;
  uint32_t cvw[NSTEP][4];
  const uint32_t* cvg =
      reinterpret_cast<const uint32_t*>(a.vcb + ((size_t)h * FG + mgrp) * R * FNC * 8) + (wave * BPW) * 4 + mi;

  // ---- value histograms (LDS integer atomics) -----------------------------
  // One 64-bit add carries two query heads' weights: a (round, code, group) bin
  // row holds heads 0..3 as consecutive dwords, and no 32-bit half can carry into
  // its neighbour since a chunk's weights sum to at most C * 2^FXSHIFT = 2^31.
  {
    uint32_t gb[FG];
#pragma unroll
    for (int kj = 0; kj < FG; ++kj) gb[kj] = (uint32_t)(((kj + g16) & 15) * 16);
    float fxk[FNH];  // fixed-point scale with the wavefront's factor e^{M_w - M}
#pragma unroll
    for (int k = 0; k < FNH; ++k) fxk[k] = (float)(1u << FXSHIFT) * fw[k];
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const int m = m0 + tid + FT * t;
      if (m < L && m != skip_pos) {
        const uint32_t (&e)[R][4] = ve[t];
        // pair word 0 goes to heads 2 h16, 2 h16 + 1; word 1 to the other pair
        const uint64_t p01 = (uint64_t)(uint32_t)fmaf(s[t][0], fxk[0], 0.5f) |
                             ((uint64_t)(uint32_t)fmaf(s[t][1], fxk[1], 0.5f) << 32);
        const uint64_t p23 = (uint64_t)(uint32_t)fmaf(s[t][2], fxk[2], 0.5f) |
                             ((uint64_t)(uint32_t)fmaf(s[t][3], fxk[3], 0.5f) << 32);
        const uint64_t pw[2] = {h16 ? p23 : p01, h16 ? p01 : p23};
        const uint32_t hoff0 = (uint32_t)(h16 * 8), hoff1 = (uint32_t)((1 - h16) * 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t x[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = __builtin_amdgcn_alignbyte(e[r][(k + 1) & 3], e[r][k], sh4);
#pragma unroll
          for (int kj = 0; kj < FG; ++kj) {
            const uint32_t code = (x[kj >> 2] >> (8 * (kj & 3))) & 0xffu;
            const uint32_t row = ((uint32_t)(r * FNC) + code) * 256u + gb[kj];
            __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(lds + Cfg::HOFF + row + hoff0), pw[0],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(lds + Cfg::HOFF + row + hoff1), pw[1],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      }
#pragma unroll
      for (int st = t * (NSTEP / TL); st < (t + 1) * (NSTEP / TL); ++st)
#pragma unroll
        for (int u = 0; u < 4; ++u) cvw[st][u] = cvg[(4 * st + u) * 4];
    }
  }
  __syncthreads();

  // ---- histogram x value codebook on MFMA ---------------------------------
  // Per group: o[head][dim] = sum_bin H[head][bin] CV[bin][dim], the fixed-point
  // bins split into fp16 hi + lo parts (v_mfma_f32_4x4x4f16: A = H rows = heads,
  // B = CV columns = dims, K = 4 bins per step; the dword of a bin holds the
  // lane's two dims, regrouped per dim with byte permutes). The 64 lanes of a
  // histogram read hit 16 groups x 4 heads, 64 distinct banks. The eight
  // wavefronts' partial sums are added through LDS (the lane phase table's
  // space, unused since the set-up).
  {
    const float inv = 1.0f / (float)(1u << FXSHIFT);
    float4_t acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const char* hrow = lds + Cfg::HOFF + mgrp * 16 + mi * 4 + (size_t)(wave * BPW) * 256;  // bin rl at rl * 256
    // all of the lane's bins read before the first is used (one LDS latency,
    // not one per step)
    uint32_t hvs[NSTEP][4];
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u) hvs[st][u] = *reinterpret_cast<const uint32_t*>(hrow + (size_t)(4 * st + u) * 256);
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int u = 0; u < 4; ++u) asm volatile("" : "+v"(hvs[st][u]));  // (keeps the reads together, ahead of the loop)
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      half4_t ahi, alo;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float x = (float)hvs[st][u] * inv;
        const _Float16 hi = (_Float16)x;
        ahi[u] = hi;
        alo[u] = (_Float16)(x - (float)hi);
      }
      const uint32_t(&w)[4] = cvw[st];
      const half4_t b0 = as_h4(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
      const half4_t b1 = as_h4(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
      acc0 = __builtin_amdgcn_mfma_f32_4x4x4f16(ahi, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_4x4x4f16(ahi, b1, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_4x4x4f16(alo, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_4x4x4f16(alo, b1, acc1, 0, 0, 0);
    }
    // acc0[k], acc1[k] = this wavefront's part of o[head k][8 mgrp + 2 mi], o[head k][8 mgrp + 2 mi + 1]
    float* osum = reinterpret_cast<float*>(pht);  // [wavefront][head][dim]
#pragma unroll
    for (int k = 0; k < FNH; ++k)
      *reinterpret_cast<float2*>(osum + (wave * FNH + k) * FD + 8 * mgrp + 2 * mi) = make_float2(acc0[k], acc1[k]);
    __syncthreads();
    // lane tid: head tid / 128, dimension tid % 128, summed over the wavefronts;
    // with the new token folded in (decode step owner): M' = max(M, s_new),
    // o' = o e^{M - M'} + v_new e^{s_new - M'}, l' = l e^{M - M'} + e^{s_new - M'}
    const int ok_ = tid >> 7, od = tid & (FD - 1);
    float o = 0.f;
#pragma unroll
    for (int w = 0; w < FW; ++w) o += osum[(w * FNH + ok_) * FD + od];
    float al[FNH], be[FNH], Mf[FNH];
#pragma unroll
    for (int k = 0; k < FNH; ++k) {
      if (fold) {
        const float sn = new_s[k];
        Mf[k] = fmaxf(M[k], sn);
        al[k] = M[k] == -INFINITY ? 0.f : __expf(M[k] - Mf[k]);
        be[k] = __expf(sn - Mf[k]);
      } else {
        Mf[k] = M[k];
        al[k] = 1.f;
        be[k] = 0.f;
      }
    }
    {
      const float vn = fold ? new_v[od] : 0.f;
      float alk = al[0], bek = be[0];
#pragma unroll
      for (int k = 1; k < FNH; ++k)
        if (ok_ == k) {
          alk = al[k];
          bek = be[k];
        }
      part[ok_ * pstride + 2 + od] = o * alk + vn * bek;
    }
    if (tid < FNH) {
      part[tid * pstride + 0] = Mf[tid];
      part[tid * pstride + 1] = lsum[tid] * al[tid] + be[tid];
    }
  }
}

template <int R, int TL, bool BV>
hipError_t launch_fast_t(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  const int npc = BV ? a.n_chunks / (a.nbits / 128) : a.n_chunks;  // chunks of positions
  hipLaunchKernelGGL((decode_fast_kernel<R, TL, BV>), dim3(npc * a.k.Hkv, a.B), dim3(FT), 0, stream, a, ph);
  return hipGetLastError();
}

template <int R, bool BV>
hipError_t launch_fast_r(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  switch (a.chunk) {
    case 4096: return launch_fast_t<R, 8, BV>(a, ph, stream);
    case 2048: return launch_fast_t<R, 4, BV>(a, ph, stream);
    case 1024: return launch_fast_t<R, 2, BV>(a, ph, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_fast(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  if (a.k.R == 1) return launch_fast_r<1, false>(a, ph, stream);
  if (a.k.R == 2) return launch_fast_r<2, false>(a, ph, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_decode_fast_bitv_scores(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream) {
  if (a.nbits < 128 || a.nbits % 128 || a.n_chunks % (a.nbits / 128) || !a.pw || a.k_new) return hipErrorInvalidValue;
  if (a.k.R == 1) return launch_fast_r<1, true>(a, ph, stream);
  if (a.k.R == 2) return launch_fast_r<2, true>(a, ph, stream);
  return hipErrorInvalidValue;
}

}  // namespace commvq

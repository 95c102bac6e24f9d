// Fast CommVQ decode attention for head_dim 128, g = 8, Nc' = 256, four query
// heads per KV head and R = 1 or 2 rounds (the 1-bit and 2-bit CommVQ of the
// LLaMA-3.1-8B layer shape).
//
// One workgroup (512 lanes, two wavefronts per SIMD) owns a chunk of C = 512*TL
// cached positions of one (sequence, KV head); lane `tid` owns positions
// m0 + tid + 512 t, t < TL.
//
// Scores ("Pith review of CommVQ", "What carries the argument": the commuting
// codebook lets query- and codebook-dependent factors be computed once and
// reused for every cached position):
//   T[a][j][r][l][p] = conj(q~_{a,p}) * z_{j,r,l,p} is built in LDS as fp16
//   (T_re, -T_im) pairs, in slices of J groups (the whole table does not fit).
//   A position adds dot2(T[code], (cos, sin)(m theta_p)) for every pair - a code
//   gather, a phase multiply-accumulate and a reduction, with fp32 accumulation.
//   Lanes visit the J groups of a slice in a lane-rotated order, so the 16-byte
//   gathers of neighbouring lanes fall in different LDS bank groups; each lane's
//   code bytes and phases are kept in that rotated order. Gathers are issued one
//   slot ahead of the multiply-accumulates that consume them.
//   Phases follow an fp32 recurrence over the lane's positions (step 512) that
//   starts from the product of two exactly computed phases (64-bit fixed point);
//   a lane keeps the state of four groups (16 pairs) at a time.
// Values (review, "If this is right", fourth bullet: weights applied to the
// value codes before the codebook):
//   fixed-point weights are scattered into per-(round, code, group, head)
//   histograms with LDS integer atomics; lanes rotate over (group, head) so the
//   64 lanes of an atomic hit 64 different banks. The histogram is contracted
//   with the value codebook on MFMA (v_mfma_f32_4x4x4f16, 16 blocks = 8 groups x
//   2 dim quads, weights split into fp16 hi + lo parts).
// The chunk's (max, sum, o) go to the workspace and the last workgroup of the
// (sequence, KV head) merges the chunks.

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
constexpr int HI_N = FT / 16;  // first-position phase table: tid = 16 hi + lo

template <int R>
struct FastCfg {
  static constexpr int J = 8 / R;                      // groups per table slice
  static constexpr int NPASS = FG / J;                 // table slices
  static constexpr int BPT = 16 * R;                   // bytes per packed record
  static constexpr int ROW = FNH * J * 16;             // bytes per (round, code) row of a slice
  static constexpr int TAB = R * FNC * ROW;            // slice bytes (128 KiB)
  static constexpr int HIST = R * FNC * FG * FNH * 4;  // histogram bytes (64 KiB per round)
  static_assert(TAB == 131072 && HIST <= TAB, "layout");
};

// aux LDS: phase tables [64][HI_N] + [64][16], step multipliers [64], rotated
// query [4][64], reductions [64], MFMA staging [2][64][4], flag, and a decode
// step's new token: codes [2][2][16], scores [4], value [128]
constexpr int EHI_BYTES = FPR * HI_N * 8;
constexpr int ELO_BYTES = FPR * 16 * 8;
constexpr int NEW_BYTES = 64 + FNH * 4 + FD * 4;
constexpr int AUX_BYTES = EHI_BYTES + ELO_BYTES + FPR * 8 + FNH * FPR * 8 + 64 * 4 + 2 * 64 * 4 * 4 + 16 + NEW_BYTES;
static_assert(131072 + AUX_BYTES <= 160 * 1024, "LDS budget");
static_assert(EHI_BYTES >= 4 * 4096, "value-codebook slabs reuse the phase table");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  typedef float f2v __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){lo, hi}, half2_t));
}

__device__ __forceinline__ float sel4(float v0, float v1, float v2, float v3, int i) {
  const float a = (i & 1) ? v1 : v0;
  const float b = (i & 1) ? v3 : v2;
  return (i & 2) ? b : a;
}

template <int R, int TL, bool HROT>
__global__ __launch_bounds__(FT, 1) void decode_fast_kernel(DecodeArgs a, PhaseTable ph, FastPhase fp) {
  using Cfg = FastCfg<R>;
  constexpr int J = Cfg::J, NPASS = Cfg::NPASS, BPT = Cfg::BPT, ROW = Cfg::ROW;
  constexpr int ROWSH = (J == 8) ? 9 : 8;  // log2(ROW)
  constexpr int C = FT * TL;
  constexpr int FXSHIFT = 31 - (C == 4096 ? 12 : C == 2048 ? 11 : 10);  // C * 2^FXSHIFT = 2^31
  constexpr int KH = 4;                   // slots whose phases a lane holds at once
  constexpr int NHALF = J / KH;
  static_assert(ROW == (1 << ROWSH) && C <= 4096, "shape");

  extern __shared__ uint4 fsm[];
  char* lds = reinterpret_cast<char*>(fsm);
  float2* ehi = reinterpret_cast<float2*>(lds + Cfg::TAB);  // [64][HI_N] e^{i (m0 + 16 u) theta_p}
  float2* elo = ehi + FPR * HI_N;                            // [64][16] e^{i u theta_p}
  float2* stp = elo + FPR * 16;                              // [64] e^{i 512 theta_p}
  float2* qz = stp + FPR;                                    // [4][64] rotated query
  float* red = reinterpret_cast<float*>(qz + FNH * FPR);     // [64] reductions
  float* stage = red + 64;                                   // [2][64][4] MFMA partials
  uint32_t* flag = reinterpret_cast<uint32_t*>(stage + 2 * 64 * 4);
  uint8_t* new_codes = reinterpret_cast<uint8_t*>(flag + 4);         // [2][R][16]
  float* new_s = reinterpret_cast<float*>(new_codes + 64);           // [4] scaled scores
  float* new_v = new_s + FNH;                                        // [128]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups are handed to the 8 XCDs round-robin in launch order; putting the
  // KV head in the fastest-varying position keeps one head's chunks (and its
  // codebooks) on one XCD's L2 when there are 8 KV heads.
  const int h = blockIdx.x % a.k.Hkv, chunk = blockIdx.x / a.k.Hkv, b = blockIdx.y;
  const int L = min(max(a.seq_lens[b], 0), a.max_len);
  const int m0 = chunk * C;
  const size_t pstride = (size_t)a.n_chunks * (FD + 2);
  float* part = a.part + ((size_t)b * a.Hq + h * FNH) * pstride + (size_t)chunk * (FD + 2);
  // decode step: the workgroup whose chunk holds the new position encodes the new
  // key and value of its KV head (all 32 group searches at once, 16 lanes each)
  // and writes the records; its table path leaves that position out and the
  // token joins the chunk's partial with an exact fp32 score at the end
  const int pb = a.k_new ? a.positions[b] : -1;
  const bool appended = a.k_new && pb >= 0 && pb < a.cache_len;
  const int skip_pos = appended ? pb : -1;
  const bool owner = appended && chunk == min(pb / C, a.n_chunks - 1);
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
  if (m0 >= L) {
    for (int i = tid; i < FNH * (FD + 2); i += FT) {
      const int hh = i / (FD + 2), k = i % (FD + 2);
      part[hh * pstride + k] = (k == 0) ? -INFINITY : 0.f;
    }
    merge_if_last<FT>(a, b, h, FNH, FD, flag, reinterpret_cast<float*>(lds), Cfg::TAB / 4);
    return;
  }

  const int gr = tid & (J - 1);                 // group rotation of this lane
  const uint8_t* kb = a.kcodes + ((size_t)b * a.k.Hkv + h) * (size_t)a.cache_len * BPT;

  // ---- scores -------------------------------------------------------------
  // A slice's code bytes of every owned position, rotated so that byte kj belongs
  // to group pass*J + ((kj + gr) & (J-1)).
  auto load_codes = [&](int pass, uint32_t (&cw)[TL][R][J / 4]) {
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const int mm = min(m0 + tid + FT * t, L - 1);
      const uint8_t* rec = kb + (size_t)mm * BPT + pass * J;
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if constexpr (J == 8) {
          const int q = (gr >> 2) & 1, sh = gr & 3;
          const uint32_t e0 = *reinterpret_cast<const uint32_t*>(rec + r * 16 + 4 * q);
          const uint32_t e1 = *reinterpret_cast<const uint32_t*>(rec + r * 16 + 4 * (1 - q));
          cw[t][r][0] = __builtin_amdgcn_alignbyte(e1, e0, sh);
          cw[t][r][1] = __builtin_amdgcn_alignbyte(e0, e1, sh);
        } else {
          const uint32_t d = *reinterpret_cast<const uint32_t*>(rec + r * 16);
          cw[t][r][0] = __builtin_amdgcn_alignbyte(d, d, gr);
        }
      }
    }
  };
  uint32_t cw[TL][R][J / 4];
  load_codes(0, cw);

  // ---- per-workgroup constants ------------------------------------------
  // exact phases of a lane's first position m0 + tid = m0 + 16 (tid >> 4) + (tid & 15)
  for (int i = tid; i < FPR * (HI_N + 16); i += FT) {
    if (i < FPR * HI_N) {
      const int p = i / HI_N, u = i % HI_N;
      ehi[i] = phase_exact((uint32_t)(m0 + 16 * u), ph.lo[p], ph.hi[p]);
    } else {
      const int k = i - FPR * HI_N, p = k >> 4, u = k & 15;
      elo[k] = phase_exact((uint32_t)u, ph.lo[p], ph.hi[p]);
    }
  }
  if (tid < FPR) stp[tid] = make_float2(fp.step_c[tid], fp.step_s[tid]);
  if (tid < FNH * FPR) {
    const int hh = tid >> 6, p = tid & 63;
    const float* qrow = a.q + ((size_t)b * a.Hq + h * FNH + hh) * FD;
    const float x = qrow[2 * p], y = qrow[2 * p + 1];
    const float2 w = phase_exact((uint32_t)max(a.q_pos[b], 0), ph.lo[p], ph.hi[p]);
    qz[tid] = make_float2(x * w.x - y * w.y, x * w.y + y * w.x);
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
      const float2 wk = phase_exact((uint32_t)pb, ph.lo[p], ph.hi[p]);
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

  float s[TL][FNH];
#pragma unroll
  for (int t = 0; t < TL; ++t)
#pragma unroll
    for (int k = 0; k < FNH; ++k) s[t][k] = 0.f;

  const int hr = HROT ? ((tid / J) & 3) : 0;    // head rotation of this lane
  uint32_t hoff[FNH];
#pragma unroll
  for (int k = 0; k < FNH; ++k) hoff[k] = (uint32_t)(((k + hr) & 3) * J * 16);

#pragma unroll 1
  for (int pass = 0; pass < NPASS; ++pass) {
    if (pass > 0) load_codes(pass, cw);  // in flight during the table build
    __syncthreads();  // previous slice fully consumed; constants visible
    {
      // table slice: this lane builds every (round, code) row of group pass*J + (tid % J)
      // for its four query heads; the codebook rows are loaded before any is used
      constexpr int NE = R * FNC * J / FT;
      const int jp = tid & (J - 1), j = pass * J + jp;
      float2 qv[FNH][4];
#pragma unroll
      for (int ah = 0; ah < FNH; ++ah)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) qv[ah][pp] = qz[ah * FPR + 4 * j + pp];
      u32x4 zr[NE];
      const _Float16* cbj = a.kcb + ((size_t)h * FG + j) * R * FNC * 8;
#pragma unroll
      for (int k = 0; k < NE; ++k) zr[k] = *reinterpret_cast<const u32x4*>(cbj + (size_t)((tid + FT * k) / J) * 8);
#pragma unroll
      for (int k = 0; k < NE; ++k) {
        const int rl = (tid + FT * k) / J;  // r * 256 + l
#pragma unroll
        for (int ah = 0; ah < FNH; ++ah) {
          u32x4 o;
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) {
            const half2_t z = as_h2(zr[k][pp]);
            const float x = (float)z.x, y = (float)z.y;
            o[pp] = pack_h2(fmaf(qv[ah][pp].x, x, qv[ah][pp].y * y), fmaf(qv[ah][pp].y, x, -qv[ah][pp].x * y));
          }
          *reinterpret_cast<u32x4*>(lds + (size_t)((rl * FNH + ah) * J + jp) * 16) = o;
        }
      }
    }
    __syncthreads();  // slice built

#pragma unroll
    for (int hf = 0; hf < NHALF; ++hf) {
      // phase state of slots KH*hf .. KH*hf + KH - 1 at the lane's first position
      float2 om[KH][4], w[KH][4];
#pragma unroll
      for (int ks = 0; ks < KH; ++ks)
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
          const int p = 4 * (pass * J + ((KH * hf + ks + gr) & (J - 1))) + pp;
          w[ks][pp] = stp[p];
          const float2 A = ehi[p * HI_N + (tid >> 4)], B = elo[p * 16 + (tid & 15)];
          om[ks][pp] = make_float2(A.x * B.x - A.y * B.y, A.x * B.y + A.y * B.x);
        }
      // gathers run one (position, slot) step ahead of their use
      auto gather = [&](int t, int ks, u32x4 (&T)[R][FNH]) {
        const int kj = KH * hf + ks;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const uint32_t code = (cw[t][r][kj >> 2] >> (8 * (kj & 3))) & 0xffu;
          const uint32_t row = (code << ROWSH) + (uint32_t)(r * FNC * ROW + ((kj + gr) & (J - 1)) * 16);
#pragma unroll
          for (int k = 0; k < FNH; ++k) T[r][k] = *reinterpret_cast<const u32x4*>(lds + row + hoff[k]);
        }
      };
      // R = 1: gathers run one (position, slot) step ahead of their use; R = 2
      // already has eight independent gathers per slot.
      constexpr int NB = (R == 1) ? 2 : 1;
      u32x4 T[NB][R][FNH];
      if constexpr (R == 1) gather(0, 0, T[0]);
#pragma unroll
      for (int t = 0; t < TL; ++t) {
        if (t > 0) {
#pragma unroll
          for (int ks = 0; ks < KH; ++ks)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              const float2 o = om[ks][pp], ww = w[ks][pp];
              om[ks][pp] = make_float2(fmaf(o.x, ww.x, -o.y * ww.y), fmaf(o.x, ww.y, o.y * ww.x));
            }
        }
#pragma unroll
        for (int ks = 0; ks < KH; ++ks) {
          const int step = t * KH + ks, cur = (R == 1) ? (step & 1) : 0;
          if constexpr (R == 1) {
            if (ks + 1 < KH) gather(t, ks + 1, T[cur ^ 1]);
            else if (t + 1 < TL) gather(t + 1, 0, T[cur ^ 1]);
          } else {
            gather(t, ks, T[0]);
          }
          half2_t phs[4];
#pragma unroll
          for (int pp = 0; pp < 4; ++pp) phs[pp] = as_h2(pack_h2(om[ks][pp].x, om[ks][pp].y));
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int k = 0; k < FNH; ++k) {
              float acc = s[t][k];
              acc = __builtin_amdgcn_fdot2(as_h2(T[cur][r][k][0]), phs[0], acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(T[cur][r][k][1]), phs[1], acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(T[cur][r][k][2]), phs[2], acc, false);
              acc = __builtin_amdgcn_fdot2(as_h2(T[cur][r][k][3]), phs[3], acc, false);
              s[t][k] = acc;
            }
        }
      }
    }
  }

  // ---- softmax over the chunk ---------------------------------------------
  float M[FNH], lsum[FNH];
#pragma unroll
  for (int t = 0; t < TL; ++t) {
    const int mt = m0 + tid + FT * t;
    const bool ok = mt < L && mt != skip_pos;
    float v[FNH];
#pragma unroll
    for (int k = 0; k < FNH; ++k) {
      const int src = HROT ? ((k - hr) & 3) : k;
      v[k] = HROT ? sel4(s[t][0], s[t][1], s[t][2], s[t][3], src) : s[t][k];
    }
#pragma unroll
    for (int k = 0; k < FNH; ++k) s[t][k] = ok ? v[k] * a.sm_scale : -INFINITY;
  }
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < TL; ++t) mx = fmaxf(mx, s[t][k]);
    mx = wave_max(mx);
    if (lane == 0) red[k * FW + wave] = mx;
  }
  __syncthreads();  // also: every lane is done with the last table slice
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float mx = red[k * FW];
#pragma unroll
    for (int w = 1; w < FW; ++w) mx = fmaxf(mx, red[k * FW + w]);
    M[k] = mx;
  }
  // zero the histograms while the weights are formed
  for (int i = tid; i < Cfg::HIST / 16; i += FT) reinterpret_cast<uint4*>(lds)[i] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float acc = 0.f;
    const float ref = M[k] == -INFINITY ? 0.f : M[k];  // a chunk may hold only the skipped new position
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const float pw = __expf(s[t][k] - ref);  // exp(-inf) = 0 for masked positions
      s[t][k] = pw;
      acc += pw;
    }
    acc = wave_sum(acc);
    if (lane == 0) red[32 + k * FW + wave] = acc;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < FNH; ++k) {
    float acc = 0.f;
#pragma unroll
    for (int w = 0; w < FW; ++w) acc += red[32 + k * FW + w];
    lsum[k] = acc;
  }

  // Value-codebook slab loader for the MFMA contraction below (waves 0..3): the
  // first slab is requested now so it arrives while the histograms fill.
  const bool mf_active = wave < 4;
  const int mf_sI = wave & 1, mf_kh = (wave >> 1) & 1;
  constexpr int NSLAB = R * FNC / 2 / 32;
  auto load_slab = [&](int sl, u32x4 (&cv)[4]) {
    const int rl0 = mf_kh * (R * FNC / 2) + sl * 32;
    const int r = rl0 / FNC, l0 = rl0 % FNC;
    const _Float16* src = a.vcb + ((((size_t)h * FG + 8 * mf_sI) * R + r) * FNC + l0) * 8;
    // element u = lane + 64 k of the slab: group u >> 5, bin u & 31
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int u = lane + 64 * k;
      cv[k] = *reinterpret_cast<const u32x4*>(src + ((size_t)(u >> 5) * R * FNC + (u & 31)) * 8);
    }
  };
  u32x4 cvn[4] = {};
  if (mf_active) load_slab(0, cvn);

  // ---- value histograms (LDS integer atomics) -----------------------------
  {
    const int g16 = tid & 15, h16 = (tid >> 4) & 3;
    uint32_t gb[FG];
#pragma unroll
    for (int kj = 0; kj < FG; ++kj) gb[kj] = (uint32_t)(((kj + g16) & 15) * 16);
    uint32_t hb[FNH];
#pragma unroll
    for (int k = 0; k < FNH; ++k) hb[k] = (uint32_t)(((k + h16) & 3) * 4);
    const uint8_t* vb = a.vcodes + ((size_t)b * a.v.Hkv + h) * (size_t)a.cache_len * BPT;
    const float fxs = (float)(1u << FXSHIFT);
    const int q4 = (g16 >> 2) & 3, sh4 = g16 & 3;
#pragma unroll
    for (int t = 0; t < TL; ++t) {
      const int m = m0 + tid + FT * t;
      if (m < L && m != skip_pos) {
        const uint8_t* rec = vb + (size_t)m * BPT;
        uint32_t e[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int k = 0; k < 4; ++k) e[r][k] = *reinterpret_cast<const uint32_t*>(rec + r * 16 + 4 * ((k + q4) & 3));
        uint32_t pf[FNH];
#pragma unroll
        for (int k = 0; k < FNH; ++k)
          pf[k] = (uint32_t)fmaf(sel4(s[t][0], s[t][1], s[t][2], s[t][3], (k + h16) & 3), fxs, 0.5f);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          uint32_t x[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) x[k] = __builtin_amdgcn_alignbyte(e[r][(k + 1) & 3], e[r][k], sh4);
#pragma unroll
          for (int kj = 0; kj < FG; ++kj) {
            const uint32_t code = (x[kj >> 2] >> (8 * (kj & 3))) & 0xffu;
            const uint32_t row = ((uint32_t)(r * FNC) + code) * 256u + gb[kj];
#pragma unroll
            for (int k = 0; k < FNH; ++k)
              __hip_atomic_fetch_add(reinterpret_cast<uint32_t*>(lds + row + hb[k]), pf[k], __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          }
        }
      }
    }
  }
  __syncthreads();

  // ---- histogram x value codebook on MFMA ---------------------------------
  // Waves 0..3 contract: wave w takes instruction set sI = w & 1 (groups 8 sI ..
  // 8 sI + 7) and half kh = w >> 1 of the (round, bin) range. Block bk = lane >> 2
  // covers group j = 8 sI + (bk >> 1), dims 4 (bk & 1) .. +3; within a block lane
  // i = lane & 3 supplies A row (head i) and B column (dim 4 (bk & 1) + i). The
  // value-codebook rows a wave needs are staged, 32 bins of its 8 groups at a
  // time, in its own 4 KiB of the (now unused) phase table.
  {
    const bool active = mf_active;
    const int sI = mf_sI, kh = mf_kh;
    const int bk = lane >> 2, i4 = lane & 3;
    const int g8 = bk >> 1, j = 8 * sI + g8;
    const int e = 4 * (bk & 1) + i4;
    const float inv = 1.0f / (float)(1u << FXSHIFT);
    _Float16* slab = reinterpret_cast<_Float16*>(ehi) + (wave & 3) * 2048;  // [8 groups][32 bins][8 dims]
    float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int sl = 0; sl < NSLAB; ++sl) {
      const int rl0 = kh * (R * FNC / 2) + sl * 32;  // first (round, bin) of the slab
      const int r = rl0 / FNC, l0 = rl0 % FNC;
      __syncthreads();  // previous slab consumed (and, first time, phase tables dead)
      if (active) {
#pragma unroll
        for (int k = 0; k < 4; ++k) reinterpret_cast<u32x4*>(slab)[lane + 64 * k] = cvn[k];
        if (sl + 1 < NSLAB) load_slab(sl + 1, cvn);
      }
      __syncthreads();
      if (active) {
#pragma unroll
        for (int st = 0; st < 8; ++st) {
          half4_t ahi, alo, bv;
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int l = l0 + 4 * st + u;
            const uint32_t hv = *reinterpret_cast<const uint32_t*>(lds + ((r * FNC + l) * 256 + j * 16 + i4 * 4));
            const float x = (float)hv * inv;
            const _Float16 hi = (_Float16)x;
            ahi[u] = hi;
            alo[u] = (_Float16)(x - (float)hi);
            bv[u] = slab[(g8 * 32 + 4 * st + u) * 8 + e];
          }
          acc = __builtin_amdgcn_mfma_f32_4x4x4f16(ahi, bv, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_4x4x4f16(alo, bv, acc, 0, 0, 0);
        }
      }
    }
    // acc[k] = partial o[head k][8 j + e]
    if (active && kh == 1) {
#pragma unroll
      for (int k = 0; k < 4; ++k) stage[(sI * 64 + lane) * 4 + k] = acc[k];
    }
    __syncthreads();
    // with the new token folded in (decode step owner): M' = max(M, s_new),
    // o' = o e^{M - M'} + v_new e^{s_new - M'}, l' = l e^{M - M'} + e^{s_new - M'}
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
    if (active && kh == 0) {
      const float vn = fold ? new_v[8 * j + e] : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        part[k * pstride + 2 + 8 * j + e] = (acc[k] + stage[(sI * 64 + lane) * 4 + k]) * al[k] + vn * be[k];
    }
    if (tid < FNH) {
      part[tid * pstride + 0] = Mf[tid];
      part[tid * pstride + 1] = lsum[tid] * al[tid] + be[tid];
    }
  }
  merge_if_last<FT>(a, b, h, FNH, FD, flag, reinterpret_cast<float*>(lds), Cfg::TAB / 4);
}

template <int R, int TL, bool HROT>
hipError_t launch_fast_t(const DecodeArgs& a, const PhaseTable& ph, const FastPhase& fp, hipStream_t stream) {
  const size_t smem = FastCfg<R>::TAB + AUX_BYTES;
  static std::atomic<uint64_t> configured{0};
  hipError_t e = allow_full_lds(reinterpret_cast<const void*>(&decode_fast_kernel<R, TL, HROT>), configured);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_fast_kernel<R, TL, HROT>), dim3(a.n_chunks * a.k.Hkv, a.B), dim3(FT), smem, stream, a,
                     ph, fp);
  return hipGetLastError();
}

template <int R, bool HROT>
hipError_t launch_fast_r(const DecodeArgs& a, const PhaseTable& ph, const FastPhase& fp, hipStream_t stream) {
  switch (a.chunk) {
    case 4096: return launch_fast_t<R, 8, HROT>(a, ph, fp, stream);
    case 2048: return launch_fast_t<R, 4, HROT>(a, ph, fp, stream);
    case 1024: return launch_fast_t<R, 2, HROT>(a, ph, fp, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_fast(const DecodeArgs& a, const PhaseTable& ph, const FastPhase& fp, hipStream_t stream) {
  // Head rotation costs an address add per gather; it pays when a slice has too
  // few groups (J = 4 at R = 2) to spread 16 lanes over distinct bank groups.
  if (a.k.R == 1) return launch_fast_r<1, false>(a, ph, fp, stream);
  if (a.k.R == 2) return launch_fast_r<2, true>(a, ph, fp, stream);
  return hipErrorInvalidValue;
}

}  // namespace commvq

// Internal interface between the C ABI (api.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace commvq {

constexpr int kMaxPairs = 128;  // D <= 256

// Validated shape of one codebook.
struct CbShape {
  int D, g, G, Nc, R, Hkv, bits, bpt;
};

struct EncodeArgs {
  const _Float16* x;
  const _Float16* cb;  // [Hkv][G][R][Nc][g]
  uint8_t* codes;
  int64_t n_tokens;
  int64_t x_token_stride;     // elements
  int64_t code_token_stride;  // bytes
  int64_t code_head_stride;   // bytes
  const int32_t* positions;   // append mode when non-null
  int32_t cache_len;
  CbShape s;
};

// Position phase: the RoPE angle m*theta_p is carried as a 64-bit fixed-point
// fraction of a turn, F_p = theta_p / (2 pi) * 2^64, so (m * F_p) mod 2^64 is the
// exact phase of position m to within 2^-64 turn per unit of m.
struct PhaseTable {
  uint32_t lo[kMaxPairs];
  uint32_t hi[kMaxPairs];
};

constexpr int kFastNewTokFloats = 16 * 4 + 128;

struct DecodeArgs {
  const float* q;
  const int32_t* q_pos;
  const uint8_t* kcodes;
  const uint8_t* vcodes;
  const int32_t* seq_lens;
  const _Float16* kcb;
  const _Float16* vcb;
  // fused decode step: when k_new is set, the new token of sequence b (fp16
  // [B][Hkv][D] keys / values) is encoded into the caches at positions[b]
  const _Float16* k_new;
  const _Float16* v_new;
  const int32_t* positions;
  uint8_t* kcodes_w;
  uint8_t* vcodes_w;
  float* part;         // [B][Hq][n_chunks][D + 2]: (max, sum, o[D]) per chunk
  // decode step on the fast R = 1 kernel: [B][Hkv][kFastNewTokFloats], the new
  // key's per-group products q~.k~ [16][4] and its value [128], which the merge
  // kernel adds as one more chunk (fold_new set)
  float* newtok;
  int fold_new;
  float* out;          // [B][Hq][D]
  // binary value codes (the generic kernel's bit-value variant): bits
  // [B][cache_len][nbits / 8] LSB-first, rows C fp16 [nbits][Hkv * D]
  const uint8_t* vbits;
  const _Float16* vrows;
  int nbits;
  // binary value codes on the fast kernel: softmax weights e^{s - M} of every
  // position, fp16 [B][Hq][n_chunks / (nbits / 128) * chunk]
  _Float16* pw;
  int B, Hq, NH, cache_len, max_len, n_chunks, chunk;
  float sm_scale;
  // generic kernel: 1 = exact position phases (COMMVQ_DECODE_EXACT), 0 = the
  // hardware sine and cosine of the exact turn count
  int exact_phase;
  CbShape k, v;
};

// Comparison path: packed records -> fp16 keys (rotated to their positions) and
// values, [B][Hkv][cache_len][D], for positions below the sequence length.
struct DequantArgs {
  const uint8_t* kcodes;
  const uint8_t* vcodes;
  const int32_t* seq_lens;
  const _Float16* kcb;
  const _Float16* vcb;
  _Float16* kout;
  _Float16* vout;
  int B, cache_len, max_len;
  CbShape k, v;
};

// Comparison path: dense decode attention over fp16 keys (already rotated) and
// values [B][Hkv][cache_len][128], chunks of kDenseChunk positions.
constexpr int kDenseChunk = 1024;
struct DenseArgs {
  const float* q;
  const int32_t* q_pos;
  const _Float16* k;
  const _Float16* v;
  const int32_t* seq_lens;
  float* part;  // [B][Hq][n_chunks][D + 2]
  float* out;   // [B][Hq][D]
  int B, Hq, Hkv, NH, cache_len, max_len, n_chunks;
  float sm_scale;
};

// Codebook fitting: one EM iteration for round `round` (fp32 accumulators
// work [Hkv][G][Nc][g + 1]: responsibility-weighted sums, then the mass).
struct EmArgs {
  const _Float16* x;          // token t, head h at x + t * x_token_stride + h * D
  int64_t n_tokens;
  int64_t x_token_stride;     // elements
  const _Float16* cb;         // [Hkv][G][R][Nc][g], read
  _Float16* new_cb;           // same layout; the fitted round's entries are written (may equal cb)
  float* work;
  float* mass_out;            // nullable [Hkv][G][Nc]
  int round;
  float temperature;          // 0: nearest entry
  float min_mass;
  CbShape s;
};

// Raises a kernel's dynamic-LDS limit to the whole 160 KiB of a CU, once per
// device: `done` is a per-kernel bit set of the devices already configured.
inline hipError_t allow_full_lds(const void* kernel, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev < 64 ? (uint64_t(1) << dev) : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

// Chunk length (tokens per workgroup) chosen for a decode shape; the workspace
// query and the launch use the same rule.
int decode_chunk_len(const CbShape& k, const CbShape& v, int B, int Hq, int max_len, int flags);
bool decode_fast_path(const CbShape& k, const CbShape& v, int NH, int flags);
// LDS bytes of the generic decode kernel for a shape (at most 160 KiB can run).
size_t decode_generic_smem(const CbShape& k, const CbShape& v, int NH);
// LDS bytes of the generic kernel's bit-value variant.
size_t decode_bitv_smem(const CbShape& k, int nbits, int NH);
// The generic kernel with binary value codes (a.vbits, a.vrows, a.nbits).
hipError_t launch_decode_bitv(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream);
// Binary value codes on the fast kernel's shapes (and nbits a multiple of 128,
// Hq <= 32): the fast kernel's scores and softmax write the weights a.pw and
// each chunk's (M, l); bitv_values_kernel forms each (chunk, 128-bit range)'s
// u on the matrix cores; bitv_merge_kernel combines the chunks and forms u^T C.
// a.n_chunks counts partial slots: chunks x nbits / 128.
bool decode_bitv_fast_path(const CbShape& k, int nbits, int Hq, int flags);
size_t decode_bitv_workspace_bytes(const CbShape& k, int nbits, int B, int Hq, int max_len);  // either path
// byte offset of the weights in the fast path's workspace (after the partials)
size_t decode_bitv_pw_offset(const CbShape& k, int nbits, int B, int Hq, int max_len, int chunk);
hipError_t launch_decode_fast_bitv_scores(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream);
hipError_t launch_bitv_values(const DecodeArgs& a, hipStream_t stream);
// the fast path's merge: chunks combined on u per (query head, sequence), then u^T C into a.out
hipError_t launch_bitv_merge(const DecodeArgs& a, hipStream_t stream);
size_t decode_workspace_bytes(const CbShape& k, int B, int Hq, int max_len, int chunk);
// Byte offset of the new-token area in the workspace (after the partials, 256-aligned).
size_t decode_newtok_offset(const CbShape& k, int B, int Hq, int max_len, int chunk);
hipError_t launch_decode_fast(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream);

hipError_t launch_encode(const EncodeArgs& a, hipStream_t stream);
// The near-tie diagnostic of an encoding already written (gap per field, [n][Hkv][R][G] fp32).
hipError_t launch_encode_gaps(const EncodeArgs& a, float* gap, hipStream_t stream);
// Whether launch_encode searches this shape on the matrix cores (more than 64 tokens).
bool encode_uses_matrix_cores(const CbShape& s);
hipError_t launch_decode_generic(const DecodeArgs& a, const PhaseTable& ph, hipStream_t stream);
hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_dequant_kv(const DequantArgs& a, const PhaseTable& ph, hipStream_t stream);
size_t dense_workspace_bytes(int B, int Hq, int max_len);
// dense_decode_kernel, then the chunk merge into a.out
hipError_t launch_dense_decode(const DenseArgs& a, const PhaseTable& ph, hipStream_t stream);
size_t em_work_bytes(const CbShape& s);
size_t em_accum_bytes(const CbShape& s);  // the fp32 accumulators, 256-byte padded
int64_t em_code_batch(const CbShape& s);  // vectors per encoder batch of the nearest-entry path (0: not used)
size_t em_accumulate_smem(const CbShape& s, int round, bool soft);
hipError_t launch_em_step(const EmArgs& a, hipStream_t stream);

}  // namespace commvq

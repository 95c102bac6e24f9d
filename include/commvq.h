/*
 * commvq.h - C ABI of the CommVQ quantized-KV hot path for AMD MI355X (gfx950).
 *
 * CommVQ stores each key/value vector of the KV cache as residual vector-quantizer
 * codes: the head dimension D is cut into groups of g scalars, every group shares
 * one index per round into an Nc'-entry codebook, and R rounds each encode the
 * residual the earlier rounds left ("Pith review of CommVQ", pith.science, section
 * "What carries the argument": index sharing over group size g, R residual rounds,
 * bit rate R*log2(Nc')/g, paper Eq. 21). Key codebook entries are blocks
 * [[x, y], [-y, x]] that commute with the RoPE rotation of each 2-D pair (same
 * section, paper Eq. 7; "Assumptions", Eqn 8), so a query-times-codebook table
 * built once per decode step serves every cached position. The softmax weights
 * are applied to the value codes before the value codebook (review, "If this is
 * right", fourth bullet).
 *
 * Conventions shared by every call:
 *  - Device pointers are HIP device allocations owned by the caller. The library
 *    allocates nothing and keeps no state besides a thread-local error string,
 *    and, for commvq_decode_step_noalloc, one static scratch array per GPU (with
 *    its device address, looked up once per device).
 *  - Every compute call is asynchronous on `stream` (a hipStream_t passed as
 *    void*; NULL is the default stream) and returns before the GPU work ends.
 *  - Calls return COMMVQ_OK (0) or a negative commvq_status; on error nothing is
 *    launched and commvq_last_error() describes the cause.
 *  - A codebook entry's pair (x, y) reconstructs the 2-vector (x, y) of one RoPE
 *    pair; RoPE pairs are the interleaved channels (2p, 2p+1) with frequency
 *    theta_p = theta_base^(-2p/D) and rotation [[cos, -sin], [sin, cos]].
 *  - Packed record of one (token, KV head): R*(D/g) fields of log2(Nc') bits,
 *    round-major (round outer, group inner), least significant bit first,
 *    padded to whole bytes: commvq_code_bytes_per_token() bytes.
 *  - Codes are chosen greedily per round: the entry nearest (squared Euclidean
 *    distance, float32 arithmetic) to the running residual, lowest index on ties.
 */
#ifndef COMMVQ_H
#define COMMVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define COMMVQ_ABI_VERSION 2

typedef enum commvq_status {
  COMMVQ_OK = 0,
  COMMVQ_ERR_INVALID_ARG = -1, /* bad descriptor, null pointer, bad size or stride */
  COMMVQ_ERR_UNSUPPORTED = -2, /* valid CommVQ shape that no kernel here handles */
  COMMVQ_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  COMMVQ_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed */
} commvq_status;

typedef enum commvq_dtype { COMMVQ_F16 = 1 } commvq_dtype;

/* commvq_decode_attention flags. By default shapes with head_dim 128, g = 8,
 * Nc' = 256, R = 1 or 2 and four query heads per KV head run a kernel that keeps
 * the query (per block of 64 positions), the position phases and the rotated
 * key entries in fp16 (products summed in fp32). Its score error is about 2^-11
 * of the spread of the score's terms, and the softmax passes it on more strongly
 * the more the scores spread. So the kernel measures, per wavefront (its 64 to
 * 512 positions), the standard deviation of the scaled scores (valid positions,
 * each of the four query heads); where it exceeds 2.0 the wavefront recomputes its
 * scores in fp32 (exact fp16 products, fp16 hi + lo phases, fp32 matrix-core
 * sums), at several times the cost of its score phase. Validated range (outputs
 * against an fp64 reference, worst row error over max |ref|): queries at 1 and
 * 2 times unit variance stay on the fp16 scores (1-bit: <= 8.9e-4, 2-bit:
 * <= 1.6e-3); from 4 times up to 16 times (tested) the recomputed scores give
 * <= 1e-4, at 4K to 128K positions. COMMVQ_DECODE_EXACT selects the fp32
 * generic kernel instead (slower still). The kernel for the other shapes (fp32
 * table or rebuilt keys) takes each position's phase from the hardware sine and
 * cosine of its exact turn count (within 2e-7), and from an exact sincospi under
 * COMMVQ_DECODE_EXACT. */
#define COMMVQ_DECODE_EXACT 1u

/* One codebook (keys or values) for all KV heads of one layer.
 * Pages: "What carries the argument" (codebook per subspace, group size g,
 * R rounds, Nc' entries). */
typedef struct commvq_codebook {
  int32_t head_dim;    /* D: even, 2..256 */
  int32_t group_size;  /* g scalars sharing one index: even, divides D, 2..128;
                          the kernels take even g <= 16, 32, 64 and 128 (other
                          values: COMMVQ_ERR_UNSUPPORTED from the compute calls) */
  int32_t n_entries;   /* Nc': power of two, 2..256 */
  int32_t n_rounds;    /* R: 1..32 */
  int32_t n_kv_heads;  /* 1 <= Hkv <= 65535 (larger: COMMVQ_ERR_UNSUPPORTED) */
  int32_t dtype;       /* COMMVQ_F16 */
  const void* entries; /* device fp16 [Hkv][D/g][R][Nc'][g]; within a group the
                          scalars are the interleaved (x, y) pairs */
} commvq_codebook;

/* RoPE description (review, "Assumptions": block-diagonal 2x2 rotations, Eqns 5-6). */
typedef struct commvq_rope {
  double theta_base; /* > 1; e.g. 500000 */
  int32_t pairing;   /* 0 = interleaved pairs (2p, 2p+1); other values are rejected */
  int32_t reserved;  /* must be 0 */
} commvq_rope;

/* ---- host-only queries (no GPU needed) --------------------------------- */

/* COMMVQ_ABI_VERSION of the library. */
int32_t commvq_abi_version(void);

/* Text of the last error on the calling thread ("" if none). Owned by the
 * library; valid until the thread's next call. */
const char* commvq_last_error(void);

/* Checks a descriptor's sizes (not its device pointer). COMMVQ_OK or
 * COMMVQ_ERR_INVALID_ARG. */
int32_t commvq_validate_codebook(const commvq_codebook* cb);

/* Average stored bits per scalar, R*log2(Nc')/g (paper Eq. 21 as quoted in the
 * review, "What carries the argument"); negative if the descriptor is invalid. */
double commvq_bits_per_scalar(const commvq_codebook* cb);

/* Bytes of one packed (token, KV head) record, ceil(R*(D/g)*log2(Nc')/8);
 * negative commvq_status if the descriptor is invalid. */
int64_t commvq_code_bytes_per_token(const commvq_codebook* cb);

/* Workspace bytes that commvq_decode_attention / commvq_decode_step need for
 * this shape: the split-context partials, (max, sum, o[D]) fp32 per (sequence,
 * query head, chunk of positions), then a decode step's new-token terms (192
 * fp32 per (sequence, KV head)), sized for every flags value; negative
 * commvq_status on invalid arguments. */
int64_t commvq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                      const commvq_codebook* kcb, const commvq_codebook* vcb);

/* ---- compute ------------------------------------------------------------ */

/* Encode n_tokens tokens of all KV heads into packed records.
 *   x      device fp16, token t head h scalar d at x[t*x_token_stride + h*D + d]
 *          (x_token_stride in elements, >= Hkv*D)
 *   codes  device bytes; record (t, h) starts at
 *          codes + t*code_token_stride + h*code_head_stride (strides in bytes);
 *          records must not overlap; every byte of each record is written.
 * n_tokens == 0 launches nothing. One round of one group's codebook (Nc' * g
 * fp32) plus 64 tokens' codes (64 * R * D/g bytes) must fit 160 KiB of LDS
 * (otherwise COMMVQ_ERR_UNSUPPORTED; commvq_append and commvq_decode_step
 * share the rule).
 *   gap_out  nullable device fp32 [n_tokens][Hkv][R][G], 4-byte aligned: when
 *          given, a second kernel (after the encoder, same stream) writes each
 *          field's near-tie diagnostic (d2 - d1) / max(d1, 1e-12 |e|^2), the
 *          relative margin between the two smallest squared distances of the
 *          round's residual e to the group's entries (fp32; +inf when Nc' = 1),
 *          with each round's residual taken after the encoder's own earlier
 *          picks. A field whose margin is below ~1e-5 is a near tie: another
 *          implementation may choose the other entry.
 * Pages: "What carries the argument" (shared index per group, R residual
 * rounds). */
int32_t commvq_encode(const commvq_codebook* cb, const void* x, int64_t n_tokens,
                      int64_t x_token_stride, uint8_t* codes, int64_t code_token_stride,
                      int64_t code_head_stride, float* gap_out, void* stream);

/* Encode one new token per sequence and write it into a contiguous cache at a
 * per-sequence position held on the device.
 *   x          device fp16 [batch][Hkv][D]
 *   positions  device int32 [batch]; a position outside [0, cache_len) skips
 *              that sequence (nothing written)
 *   cache      device bytes [batch][Hkv][cache_len][code_bytes_per_token] */
int32_t commvq_append(const commvq_codebook* cb, const void* x, int32_t batch,
                      const int32_t* positions, uint8_t* cache, int32_t cache_len, void* stream);

/* One decode step of grouped-query attention directly on packed codes.
 *   q        device fp32 [batch][n_q_heads][D], not yet rotated
 *   q_pos    device int32 [batch]: the query's RoPE position (normally len-1)
 *   kcodes, vcodes  device bytes [batch][Hkv][cache_len][bytes_per_token]
 *   seq_lens device int32 [batch]: keys at positions [0, seq_lens[b]) are
 *            attended; contract 1 <= seq_lens[b] <= max_seq_len <= cache_len.
 *            Lengths are clamped to [0, max_seq_len]; a length of 0 gives a
 *            zero output row.
 *   n_q_heads must be a multiple of Hkv; query head hq reads KV head
 *   hq / (n_q_heads / Hkv). n_q_heads / Hkv must be 1, 2, 4 or 8, group_size
 *   2, 4, 8, 16, 32, 64 or 128, batch <= 65535, ceil(max_seq_len / 1024) *
 *   Hkv < 2^31, and one (group, round)'s query x codebook table, NH * Nc' *
 *   g/2 complex fp32 values plus the queries, must fit 160 KiB of LDS
 *   (otherwise COMMVQ_ERR_UNSUPPORTED).
 *   sm_scale multiplies q.k (normally 1/sqrt(D)).
 *   out      device fp32 [batch][n_q_heads][D]
 *   workspace device, >= commvq_decode_workspace_bytes(batch, n_q_heads,
 *            max_seq_len, kcb, vcb) bytes, 256-byte aligned; its contents
 *            need no initialisation and are scratch after the call. Calls
 *            sharing one workspace must not overlap in time.
 *   flags    0 or COMMVQ_DECODE_EXACT.
 * Pages: "What carries the argument" (query-codebook factors computed once and
 * reused over cached positions); "If this is right", fourth bullet (weights
 * applied to value codes before the codebook). */
int32_t commvq_decode_attention(const commvq_codebook* kcb, const commvq_codebook* vcb,
                                const commvq_rope* rope, const float* q, const int32_t* q_pos,
                                const uint8_t* kcodes, const uint8_t* vcodes,
                                const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                int32_t cache_len, int32_t max_seq_len, float sm_scale,
                                float* out, void* workspace, size_t workspace_bytes,
                                uint32_t flags, void* stream);

/* One decode step: encode the new token's key and value (all KV heads), write
 * them into the caches at positions[b], then attend exactly as
 * commvq_decode_attention does over keys [0, seq_lens[b]).
 *   k_new, v_new device fp16 [batch][Hkv][D], 16-byte aligned
 *   positions    device int32 [batch]; a position outside [0, cache_len) skips
 *                the append for that sequence (attention still runs)
 *   kcodes, vcodes are written (the new records) and read.
 * Other arguments as commvq_decode_attention. For the shapes of the fast kernel
 * (D 128, g 8, Nc' 256, four query heads per KV head, R 1 or 2) the new token is
 * encoded inside the attention kernel (R = 1: its 32 group searches spread over
 * the KV head's workgroups, the token joining in the chunk merge; R = 2: by the
 * workgroup whose chunk holds the position): the step is that kernel plus the
 * chunk merge, as for commvq_decode_attention.
 * Pages: abstract (each new K/V vector is encoded to a low-bit code); "What
 * carries the argument" (shared index per group, R residual rounds, codebook
 * factors reused over cached positions). */
int32_t commvq_decode_step(const commvq_codebook* kcb, const commvq_codebook* vcb,
                           const commvq_rope* rope, const void* k_new, const void* v_new,
                           const int32_t* positions, const float* q, const int32_t* q_pos,
                           uint8_t* kcodes, uint8_t* vcodes, const int32_t* seq_lens,
                           int32_t batch, int32_t n_q_heads, int32_t cache_len,
                           int32_t max_seq_len, float sm_scale, float* out, void* workspace,
                           size_t workspace_bytes, uint32_t flags, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): commvq_decode_step with
 * no workspace argument. Its chunk partials and new-token terms live in a static
 * device array of COMMVQ_NOALLOC_SCRATCH_BYTES (16 MiB), one per GPU, held until
 * the process ends; the call allocates nothing. A shape whose
 * commvq_decode_workspace_bytes exceeds that size is rejected with
 * COMMVQ_ERR_WORKSPACE before any HIP call. The scratch is that of the device
 * current when the call is made (the stream must belong to it); its address is
 * looked up on the first call on each device. Nothing in it has to start at zero
 * (every call writes all it reads). All calls on one GPU share the one array:
 * calls that overlap in time on the same GPU (other streams, other host
 * threads) race. Arguments, outputs and errors as commvq_decode_step. */
#define COMMVQ_NOALLOC_SCRATCH_BYTES (16ull << 20)
int32_t commvq_decode_step_noalloc(const commvq_codebook* kcb, const commvq_codebook* vcb,
                                   const commvq_rope* rope, const void* k_new, const void* v_new,
                                   const int32_t* positions, const float* q, const int32_t* q_pos,
                                   uint8_t* kcodes, uint8_t* vcodes, const int32_t* seq_lens,
                                   int32_t batch, int32_t n_q_heads, int32_t cache_len,
                                   int32_t max_seq_len, float sm_scale, float* out, uint32_t flags,
                                   void* stream);

/* ---- binary value codes ------------------------------------------------------
 * The paper codes a value vector with a binary code s in {0,1}^Nc and decodes
 * it as s^T C ("Pith review of CommVQ", "Referee Report", minor comment 4;
 * "Assumptions & free parameters": Nc = 1024 rows for 1 bit, 2048 for 2 bits,
 * average bit width Nc/d). Here one code covers a token's whole value, all KV
 * heads (d = Hkv * D); keys keep the commutative residual codebook. Its learned
 * encoder is not part of this library; the decode side is. */
typedef struct commvq_bit_codebook {
  int32_t n_bits;      /* Nc: power of two, 32..2048 */
  int32_t dim;         /* d = Hkv * D of the key codebook it is used with */
  int32_t dtype;       /* COMMVQ_F16 */
  int32_t reserved;    /* must be 0 */
  const void* rows;    /* device fp16 [n_bits][dim], 16-byte aligned */
} commvq_bit_codebook;

/* Workspace bytes for commvq_decode_attention_bitv with these shapes, enough
 * for either of its paths (any flags); or a negative status for shapes it
 * rejects. */
int64_t commvq_decode_bitv_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                           const commvq_codebook* kcb, const commvq_bit_codebook* vcb);

/* Decode attention with binary value codes: as commvq_decode_attention for the
 * keys (kcb, kcodes, rope, q, q_pos, seq_lens, sizes, sm_scale, out), with the
 * value of position t of sequence b equal to the sum of the rows of vcb whose
 * bits are set in vbits[b][t] (bit i = bit i % 8 of byte i / 8); query head hq
 * reads columns [h D, h D + D) of that sum, h its KV head. The weights meet
 * the codes before the rows: u = sum_t p_t s_t, then u^T C.
 *   vbits     device bytes, 16-byte aligned: each token's bit string stored in
 *             ranges of 128 bits, range-major, [batch][n_bits / 128][cache_len][16]
 *             (bits 128 r .. 128 r + 127 of token t of sequence b are the 16
 *             bytes at ((b * n_bits / 128 + r) * cache_len + t) * 16); for
 *             n_bits < 128 one range of n_bits / 8 bytes, [batch][cache_len][n_bits / 8].
 *             One range of consecutive tokens is thus one contiguous stream
 *   workspace >= commvq_decode_bitv_workspace_bytes(...) bytes, 256-byte
 *             aligned, no initialisation needed
 *   flags     0 or COMMVQ_DECODE_EXACT
 * Paths: on the fast kernel's key shapes (D 128, g 8, Nc' 256, R 1 or 2, four
 * query heads per KV head), n_bits >= 128, n_q_heads <= 32 and flags 0, the
 * fast kernel computes the scores and softmax and writes fp16 weights, and a
 * second kernel forms u per chunk and range of 128 bits on the matrix cores
 * (fp16 weights times the 0/1 bits, fp32 sums); a third combines the chunks
 * on u and forms u^T C in fp32 per query head. Otherwise
 * the generic kernel runs (fp32 table or rebuilt keys, phases as above; shapes as
 * commvq_decode_attention's generic path). vcb->dim must equal Hkv * D (else
 * COMMVQ_ERR_INVALID_ARG). */
int32_t commvq_decode_attention_bitv(const commvq_codebook* kcb, const commvq_bit_codebook* vcb,
                                     const commvq_rope* rope, const float* q, const int32_t* q_pos,
                                     const uint8_t* kcodes, const uint8_t* vbits,
                                     const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                     int32_t cache_len, int32_t max_seq_len, float sm_scale,
                                     float* out, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, void* stream);

/* ---- comparison path: the "naive" decode of the same codes ----------------
 * The review ("Pith review of CommVQ", "The pith") compares the method's decode
 * latency with a naive implementation of the same quantization. These two calls
 * are that baseline, read plainly: rebuild fp16 keys and values from the codes
 * in HBM, then run dense attention over them. Same synchronisation, ownership
 * and error conventions as above. */

/* Dequantise the cached records of positions [0, min(seq_lens[b], max_seq_len))
 * into fp16 vectors:
 *   k_out[b][h][t][:] = RoPE_t( sum_r key entries selected by record (b, h, t) )
 *   v_out[b][h][t][:] = sum_r value entries selected by record (b, h, t)
 * (sums and rotation in fp32, rounded to fp16 once; the rotation angle of
 * pair p is t * theta_p, from the position's exact fraction of a turn and the
 * hardware sine and cosine, within 2e-7 of the exact values).
 *   kcodes, vcodes  device bytes [batch][Hkv][cache_len][bytes_per_token]
 *   seq_lens        device int32 [batch], clamped to [0, max_seq_len]
 *   k_out, v_out    device fp16 [batch][Hkv][cache_len][D], 16-byte aligned;
 *                   positions at or past the length are left untouched.
 * Codebooks as for commvq_decode_attention (same D, g and Hkv for K and V);
 * max_seq_len <= cache_len. Pages: "What carries the argument" (a vector is the
 * sum of its R rounds' entries; RoPE as 2x2 rotations of pairs). */
int32_t commvq_dequantize_kv(const commvq_codebook* kcb, const commvq_codebook* vcb,
                             const commvq_rope* rope, const uint8_t* kcodes, const uint8_t* vcodes,
                             const int32_t* seq_lens, int32_t batch, int32_t cache_len,
                             int32_t max_seq_len, void* k_out, void* v_out, void* stream);

/* Workspace bytes for commvq_dense_decode_attention: (max, sum, o[D]) fp32 per
 * (sequence, query head, chunk of 1024 positions); negative commvq_status on
 * invalid arguments (head_dim other than 128: COMMVQ_ERR_UNSUPPORTED). */
int64_t commvq_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                     int32_t head_dim, int32_t max_seq_len);

/* Dense grouped-query decode attention over fp16 keys that already carry their
 * rotation and fp16 values:
 *   out[b][hq] = sum_t softmax_t(sm_scale * qr . k[b][h][t]) v[b][h][t],
 *   t < min(seq_lens[b], max_seq_len), h = hq / (n_q_heads / n_kv_heads),
 *   qr = q[b][hq] rotated to position q_pos[b] (exact phase) in fp32, carried
 *   as two fp16 parts so that its products with the fp16 keys are exact; the
 *   products are summed in fp32 and the weighted value sum is fp32.
 *   q        device fp32 [batch][n_q_heads][head_dim]
 *   k, v     device fp16 [batch][n_kv_heads][cache_len][head_dim]
 *   out      device fp32 [batch][n_q_heads][head_dim]; a length of 0 gives zeros
 *   workspace >= commvq_dense_workspace_bytes(...), 256-byte aligned, no
 *            initialisation needed; calls sharing it must not overlap.
 * head_dim must be 128 and n_q_heads / n_kv_heads 1, 2, 4 or 8 (otherwise
 * COMMVQ_ERR_UNSUPPORTED); q, out, k and v 16-byte aligned. */
int32_t commvq_dense_decode_attention(const commvq_rope* rope, const float* q, const int32_t* q_pos,
                                      const void* k, const void* v, const int32_t* seq_lens,
                                      int32_t batch, int32_t n_q_heads, int32_t n_kv_heads,
                                      int32_t head_dim, int32_t cache_len, int32_t max_seq_len,
                                      float sm_scale, float* out, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---- codebook fitting ------------------------------------------------------
 * The codebook is trained with an Expectation-Maximization algorithm
 * (abstract); the review ("Assumptions & free parameters") describes it as
 * alternating assignment and update in the k-means manner, stabilised by soft
 * assignment and annealing, and ("Referee Report", Significance) notes the
 * closed-form update. One call is one iteration for one residual round; a
 * caller anneals by lowering the temperature over iterations and fits the
 * rounds in order. */

/* Bytes of the work buffer commvq_em_step needs for this codebook: the fp32
 * accumulators, Hkv * (D/g) * Nc' * (g + 1) * 4 rounded up to 256, plus, for
 * the shapes whose nearest-entry step reuses the matrix-core encoder (g = 8,
 * Nc' = 256, R <= 2, Hkv * R * 16 <= 16 KiB), a 4 MiB scratch for a batch of
 * codes; negative commvq_status if invalid. */
int64_t commvq_em_work_bytes(const commvq_codebook* cb);

/* One EM iteration fitting round `round` of `cb` to n_tokens vectors of every
 * KV head and group:
 *   E-step: each group of g scalars is reduced greedily by the nearest entry of
 *     rounds 0 .. round-1 (fp32 squared distance, lowest index on ties, as
 *     commvq_encode); for that residual e, d_l = |e - c_l|^2 over the round's
 *     entries and w_l = exp((min d - d_l) / temperature) / sum over l, or, for
 *     temperature 0, 1 on the nearest entry (lowest index on ties) and 0 else.
 *   M-step: c_l = sum w_l e / sum w_l over the vectors (fp32 sums, written as
 *     fp16); an entry whose mass sum w_l is not above min_mass keeps its value.
 *   At temperature 0 the E-step's choices for g = 8, Nc' = 256, R <= 2 are
 *   those of commvq_encode's matrix-core search (which may differ from the
 *   fp32 distance form only at near ties).
 *   x            device fp16, 4-byte aligned, token t head h scalar d at
 *                x[t * x_token_stride + h * D + d] (stride in elements, even,
 *                >= Hkv*D)
 *   new_entries  device fp16 with cb->entries' layout, 16-byte aligned: the
 *                round's entries are written, nothing else (it may be
 *                cb->entries itself: the update runs after every read)
 *   mass_out     NULL or device fp32 [Hkv][D/g][Nc']: sum w_l per entry
 *   work         device, >= commvq_em_work_bytes(cb), 256-byte aligned; no
 *                initialisation needed; calls sharing it must not overlap.
 * Requires n_tokens >= 1, 0 <= round < n_rounds, finite temperature >= 0 and
 * min_mass >= 0 (else COMMVQ_ERR_INVALID_ARG); the fitted round's staging
 * (round + 1) * Nc' * g + 256 * g + 16 * Nc' floats must fit 160 KiB of LDS
 * (else COMMVQ_ERR_HIP). */
int32_t commvq_em_step(const commvq_codebook* cb, const void* x, int64_t n_tokens,
                       int64_t x_token_stride, int32_t round, float temperature, float min_mass,
                       void* new_entries, float* mass_out, void* work, size_t work_bytes,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* COMMVQ_H */

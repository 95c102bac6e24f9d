// C ABI of libcommvq: argument validation, size queries, dispatch to kernels.
// Validation runs entirely on the host before any HIP call, so every error path
// is testable without a GPU.

#include <climits>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "../../include/commvq.h"
#include "decode_common.hpp"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int ilog2(int64_t v) {
  int b = 0;
  while ((int64_t(1) << b) < v) ++b;
  return b;
}

// Shape checks shared by every entry point (descriptor sizes only).
int32_t check_shape(const commvq_codebook* cb, const char* name, commvq::CbShape* out) {
  if (!cb) return fail(COMMVQ_ERR_INVALID_ARG, "%s: null codebook descriptor", name);
  const int D = cb->head_dim, g = cb->group_size, Nc = cb->n_entries, R = cb->n_rounds;
  if (D < 2 || D > 2 * commvq::kMaxPairs || (D & 1))
    return fail(COMMVQ_ERR_INVALID_ARG, "%s: head_dim %d must be even and in [2, %d]", name, D,
                2 * commvq::kMaxPairs);
  if (g < 2 || g > 128 || (g & 1) || D % g)
    return fail(COMMVQ_ERR_INVALID_ARG, "%s: group_size %d must be even, in [2, 128] and divide head_dim %d",
                name, g, D);
  if (!is_pow2(Nc) || Nc < 2 || Nc > 256)
    return fail(COMMVQ_ERR_INVALID_ARG, "%s: n_entries %d must be a power of two in [2, 256]", name, Nc);
  if (R < 1 || R > 32) return fail(COMMVQ_ERR_INVALID_ARG, "%s: n_rounds %d must be in [1, 32]", name, R);
  if (cb->n_kv_heads < 1) return fail(COMMVQ_ERR_INVALID_ARG, "%s: n_kv_heads %d < 1", name, cb->n_kv_heads);
  if (cb->n_kv_heads > 65535) return fail(COMMVQ_ERR_UNSUPPORTED, "%s: n_kv_heads %d > 65535", name, cb->n_kv_heads);
  if (cb->dtype != COMMVQ_F16) return fail(COMMVQ_ERR_INVALID_ARG, "%s: dtype %d is not COMMVQ_F16", name, cb->dtype);
  if (out) {
    out->D = D;
    out->g = g;
    out->G = D / g;
    out->Nc = Nc;
    out->R = R;
    out->Hkv = cb->n_kv_heads;
    out->bits = ilog2(Nc);
    out->bpt = (R * (D / g) * out->bits + 7) / 8;
  }
  return COMMVQ_OK;
}

// Group sizes the encoder and the generic decode kernel are built for.
bool kernel_group_size(int g) { return g <= 16 || g == 32 || g == 64 || g == 128; }

// The encoder keeps a tile's codes (R * D/g bytes per token, tile >= 64 tokens)
// and one round of one group's codebook in LDS.
int32_t check_encodable(const commvq::CbShape& s, const char* name) {
  if (!kernel_group_size(s.g))
    return fail(COMMVQ_ERR_UNSUPPORTED, "%s: group_size %d: the kernels take even sizes up to 16, 32, 64 or 128", name,
                s.g);
  if ((size_t)s.Nc * s.g * 4 + (size_t)64 * s.R * s.G > 160 * 1024)
    return fail(COMMVQ_ERR_UNSUPPORTED, "%s: %d rounds x %d groups of codes do not fit the encoder's LDS", name, s.R,
                s.G);
  return COMMVQ_OK;
}

int32_t check_entries(const commvq_codebook* cb, const char* name) {
  if (!cb->entries) return fail(COMMVQ_ERR_INVALID_ARG, "%s: null entries pointer", name);
  if (reinterpret_cast<uintptr_t>(cb->entries) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "%s: entries pointer must be 16-byte aligned", name);
  return COMMVQ_OK;
}

int32_t hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return COMMVQ_OK;
  return fail(COMMVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Scratch of commvq_decode_step_noalloc: a static device array, one copy per
// GPU, held until the process ends. In host code its name is only a stand-in:
// the device address is looked up once per device (with that device current)
// and that address is what kernels and copies receive.
constexpr int kNoAllocMaxDevices = 64;
__device__ __align__(256) unsigned char scratch[COMMVQ_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
void* g_scratch_addr[kNoAllocMaxDevices] = {};

int32_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "commvq_decode_step_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(COMMVQ_ERR_UNSUPPORTED, "commvq_decode_step_noalloc: device %d beyond the %d with a scratch address",
                dev, kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "commvq_decode_step_noalloc: hipGetSymbolAddress");
    if (!ptr) return fail(COMMVQ_ERR_HIP, "commvq_decode_step_noalloc: null scratch address");
    g_scratch_addr[dev] = ptr;
  }
  *out = g_scratch_addr[dev];
  return COMMVQ_OK;
}

int32_t decode_shapes(const commvq_codebook* kcb, const commvq_codebook* vcb, int32_t batch,
                      int32_t n_q_heads, int32_t max_seq_len, commvq::CbShape* k, commvq::CbShape* v) {
  int32_t st = check_shape(kcb, "key codebook", k);
  if (st) return st;
  st = check_shape(vcb, "value codebook", v);
  if (st) return st;
  if (k->D != v->D || k->g != v->g || k->Hkv != v->Hkv)
    return fail(COMMVQ_ERR_INVALID_ARG, "key and value codebooks disagree on head_dim, group_size or n_kv_heads");
  if (batch < 1) return fail(COMMVQ_ERR_INVALID_ARG, "batch %d < 1", batch);
  if (n_q_heads < 1 || n_q_heads % k->Hkv)
    return fail(COMMVQ_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d", n_q_heads,
                k->Hkv);
  const int NH = n_q_heads / k->Hkv;
  if (NH != 1 && NH != 2 && NH != 4 && NH != 8)
    return fail(COMMVQ_ERR_UNSUPPORTED, "query heads per KV head %d not in {1, 2, 4, 8}", NH);
  if (max_seq_len < 1) return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d < 1", max_seq_len);
  // launch grid: (context chunks x KV heads, batch); chunks are at least 1024 positions
  if (batch > 65535) return fail(COMMVQ_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  if ((int64_t)((max_seq_len + 1023) / 1024) * k->Hkv > INT32_MAX)
    return fail(COMMVQ_ERR_UNSUPPORTED, "max_seq_len %d x n_kv_heads %d exceeds the launch grid", max_seq_len, k->Hkv);
  if (k->g != 2 && k->g != 4 && k->g != 8 && k->g != 16 && k->g != 32 && k->g != 64 && k->g != 128)
    return fail(COMMVQ_ERR_UNSUPPORTED, "decode supports group_size 2, 4, 8, 16, 32, 64 or 128, not %d", k->g);
  if (commvq::decode_generic_smem(*k, *v, NH) > 160 * 1024)
    return fail(COMMVQ_ERR_UNSUPPORTED,
                "decode's LDS staging for %d query heads, %d entries, %d rounds, group size %d exceeds 160 KiB", NH, k->Nc,
                k->R, k->g);
  return COMMVQ_OK;
}


void phase_table(double base, int D, commvq::PhaseTable* ph) {
  // F_p = frac(theta_p / 2pi) * 2^64 with theta_p = base^(-2p/D), in long double.
  const long double two_pi = 6.283185307179586476925286766559L;
  for (int p = 0; p < D / 2; ++p) {
    long double theta = powl((long double)base, -2.0L * p / D);
    long double turns = theta / two_pi;
    turns -= floorl(turns);
    long double f = ldexpl(turns, 64);
    unsigned long long F = f >= 18446744073709551615.0L ? ~0ULL : (unsigned long long)f;
    ph->lo[p] = (uint32_t)(F & 0xffffffffULL);
    ph->hi[p] = (uint32_t)(F >> 32);
  }
}

// The phase constants of one (theta_base, head_dim), kept per thread for the
// next call with the same rotary base (one model reuses it every step).
struct PhaseConsts {
  double base = 0.0;
  int D = 0;
  commvq::PhaseTable ph;
};

const PhaseConsts& phase_consts(double base, int D) {
  thread_local PhaseConsts c;
  if (c.base != base || c.D != D) {
    phase_table(base, D, &c.ph);
    c.base = base;
    c.D = D;
  }
  return c;
}

}  // namespace

extern "C" {

int32_t commvq_abi_version(void) { return COMMVQ_ABI_VERSION; }

const char* commvq_last_error(void) { return g_err; }

int32_t commvq_validate_codebook(const commvq_codebook* cb) {
  g_err[0] = 0;
  return check_shape(cb, "codebook", nullptr);
}

double commvq_bits_per_scalar(const commvq_codebook* cb) {
  g_err[0] = 0;
  commvq::CbShape s;
  int32_t st = check_shape(cb, "codebook", &s);
  if (st) return (double)st;
  return (double)s.R * (double)s.bits / (double)s.g;
}

int64_t commvq_code_bytes_per_token(const commvq_codebook* cb) {
  g_err[0] = 0;
  commvq::CbShape s;
  int32_t st = check_shape(cb, "codebook", &s);
  if (st) return st;
  return s.bpt;
}

int64_t commvq_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                      const commvq_codebook* kcb, const commvq_codebook* vcb) {
  g_err[0] = 0;
  commvq::CbShape k, v;
  int32_t st = decode_shapes(kcb, vcb, batch, n_q_heads, max_seq_len, &k, &v);
  if (st) return st;
  // the smallest chunk any path uses bounds the partials
  return (int64_t)commvq::decode_workspace_bytes(k, batch, n_q_heads, max_seq_len, 1024);
}

int32_t commvq_encode(const commvq_codebook* cb, const void* x, int64_t n_tokens, int64_t x_token_stride,
                      uint8_t* codes, int64_t code_token_stride, int64_t code_head_stride, float* gap_out,
                      void* stream) {
  g_err[0] = 0;
  commvq::CbShape s;
  int32_t st = check_shape(cb, "codebook", &s);
  if (st) return st;
  st = check_encodable(s, "codebook");
  if (st) return st;
  if (n_tokens < 0) return fail(COMMVQ_ERR_INVALID_ARG, "n_tokens %lld < 0", (long long)n_tokens);
  if (n_tokens == 0) return COMMVQ_OK;
  st = check_entries(cb, "codebook");
  if (st) return st;
  if (!x || !codes) return fail(COMMVQ_ERR_INVALID_ARG, "null x or codes pointer");
  if (reinterpret_cast<uintptr_t>(x) & 3) return fail(COMMVQ_ERR_INVALID_ARG, "x must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(gap_out) & 3) return fail(COMMVQ_ERR_INVALID_ARG, "gap_out must be 4-byte aligned");
  if (x_token_stride < (int64_t)s.Hkv * s.D || (x_token_stride & 1))
    return fail(COMMVQ_ERR_INVALID_ARG, "x_token_stride %lld must be even and >= n_kv_heads*head_dim",
                (long long)x_token_stride);
  if (code_token_stride < 0 || code_head_stride < 0)
    return fail(COMMVQ_ERR_INVALID_ARG, "negative code strides are not supported");
  {
    // Records (t, h) at t*ts + h*hs must be at least a record apart: either heads
    // nest inside tokens (hs >= bpt, ts >= Hkv*hs) or tokens inside heads.
    const int64_t ts = code_token_stride, hs = code_head_stride, n = n_tokens, H = s.Hkv, r = s.bpt;
    const bool heads_inner = (H == 1 || hs >= r) && (n == 1 || ts >= H * (H == 1 ? r : hs));
    const bool tokens_inner = (n == 1 || ts >= r) && (H == 1 || hs >= n * (n == 1 ? r : ts));
    if (!heads_inner && !tokens_inner)
      return fail(COMMVQ_ERR_INVALID_ARG, "code strides (token %lld, head %lld) make %d-byte records overlap",
                  (long long)ts, (long long)hs, s.bpt);
  }
  commvq::EncodeArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.cb = static_cast<const _Float16*>(cb->entries);
  a.codes = codes;
  a.n_tokens = n_tokens;
  a.x_token_stride = x_token_stride;
  a.code_token_stride = code_token_stride;
  a.code_head_stride = code_head_stride;
  a.positions = nullptr;
  a.cache_len = 0;
  a.s = s;
  hipError_t e = commvq::launch_encode(a, static_cast<hipStream_t>(stream));
  if (e == hipSuccess && gap_out) e = commvq::launch_encode_gaps(a, gap_out, static_cast<hipStream_t>(stream));
  return hip_status(e, "commvq_encode launch");
}

int32_t commvq_append(const commvq_codebook* cb, const void* x, int32_t batch, const int32_t* positions,
                      uint8_t* cache, int32_t cache_len, void* stream) {
  g_err[0] = 0;
  commvq::CbShape s;
  int32_t st = check_shape(cb, "codebook", &s);
  if (st) return st;
  st = check_encodable(s, "codebook");
  if (st) return st;
  if (batch < 0) return fail(COMMVQ_ERR_INVALID_ARG, "batch %d < 0", batch);
  if (batch == 0) return COMMVQ_OK;
  st = check_entries(cb, "codebook");
  if (st) return st;
  if (!x || !positions || !cache) return fail(COMMVQ_ERR_INVALID_ARG, "null x, positions or cache pointer");
  if (reinterpret_cast<uintptr_t>(x) & 3) return fail(COMMVQ_ERR_INVALID_ARG, "x must be 4-byte aligned");
  if (cache_len < 1) return fail(COMMVQ_ERR_INVALID_ARG, "cache_len %d < 1", cache_len);
  commvq::EncodeArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.cb = static_cast<const _Float16*>(cb->entries);
  a.codes = cache;
  a.n_tokens = batch;
  a.x_token_stride = (int64_t)s.Hkv * s.D;
  a.code_token_stride = (int64_t)s.Hkv * cache_len * s.bpt;
  a.code_head_stride = (int64_t)cache_len * s.bpt;
  a.positions = positions;
  a.cache_len = cache_len;
  a.s = s;
  return hip_status(commvq::launch_encode(a, static_cast<hipStream_t>(stream)), "commvq_append launch");
}

}  // extern "C"

namespace {

struct StepArgs {
  const void* k_new;
  const void* v_new;
  const int32_t* positions;
};

int32_t decode_impl(const commvq_codebook* kcb, const commvq_codebook* vcb, const commvq_rope* rope, const float* q,
                    const int32_t* q_pos, const uint8_t* kcodes, const uint8_t* vcodes, const int32_t* seq_lens,
                    int32_t batch, int32_t n_q_heads, int32_t cache_len, int32_t max_seq_len, float sm_scale,
                    float* out, void* workspace, size_t workspace_bytes, uint32_t flags, const StepArgs* step,
                    void* stream, bool static_scratch = false) {
  g_err[0] = 0;
  commvq::CbShape k, v;
  int32_t st = decode_shapes(kcb, vcb, batch, n_q_heads, max_seq_len, &k, &v);
  if (st) return st;
  if (!rope) return fail(COMMVQ_ERR_INVALID_ARG, "null rope descriptor");
  if (!(rope->theta_base > 1.0) || !std::isfinite(rope->theta_base))
    return fail(COMMVQ_ERR_INVALID_ARG, "rope theta_base must be finite and > 1");
  if (rope->pairing != 0 || rope->reserved != 0)
    return fail(COMMVQ_ERR_UNSUPPORTED, "rope pairing %d: only interleaved pairs (0) are supported", rope->pairing);
  if (cache_len < max_seq_len)
    return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds cache_len %d", max_seq_len, cache_len);
  if (!std::isfinite(sm_scale)) return fail(COMMVQ_ERR_INVALID_ARG, "sm_scale is not finite");
  if (flags & ~(uint32_t)COMMVQ_DECODE_EXACT) return fail(COMMVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  st = check_entries(kcb, "key codebook");
  if (st) return st;
  st = check_entries(vcb, "value codebook");
  if (st) return st;
  if (!q || !q_pos || !kcodes || !vcodes || !seq_lens || !out)
    return fail(COMMVQ_ERR_INVALID_ARG, "null q, q_pos, codes, seq_lens or out pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(kcodes) | reinterpret_cast<uintptr_t>(vcodes)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "code caches must be 16-byte aligned");
  if (step) {
    st = check_encodable(k, "key codebook");
    if (st) return st;
    st = check_encodable(v, "value codebook");
    if (st) return st;
    if (!step->k_new || !step->v_new || !step->positions)
      return fail(COMMVQ_ERR_INVALID_ARG, "null k_new, v_new or positions pointer");
    if ((reinterpret_cast<uintptr_t>(step->k_new) | reinterpret_cast<uintptr_t>(step->v_new)) & 15)
      return fail(COMMVQ_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  }
  const int64_t need = commvq_decode_workspace_bytes(batch, n_q_heads, max_seq_len, kcb, vcb);
  if (need < 0) return (int32_t)need;
  if (static_scratch) {
    // every argument is checked above, before the first HIP call
    if ((uint64_t)need > (uint64_t)COMMVQ_NOALLOC_SCRATCH_BYTES)
      return fail(COMMVQ_ERR_WORKSPACE,
                  "commvq_decode_step_noalloc: this shape needs %lld bytes of scratch, beyond the static %llu",
                  (long long)need, (unsigned long long)COMMVQ_NOALLOC_SCRATCH_BYTES);
    st = noalloc_scratch(&workspace);
    if (st) return st;
    workspace_bytes = COMMVQ_NOALLOC_SCRATCH_BYTES;
  }
  if (!workspace || workspace_bytes < (size_t)need)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %lld required", workspace_bytes,
                (long long)need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  commvq::DecodeArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.kcodes = kcodes;
  a.vcodes = vcodes;
  a.seq_lens = seq_lens;
  a.kcb = static_cast<const _Float16*>(kcb->entries);
  a.vcb = static_cast<const _Float16*>(vcb->entries);
  a.part = static_cast<float*>(workspace);
  a.newtok = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      commvq::decode_newtok_offset(k, batch, n_q_heads, max_seq_len, 1024));
  a.out = out;
  a.B = batch;
  a.Hq = n_q_heads;
  a.NH = n_q_heads / k.Hkv;
  a.cache_len = cache_len;
  a.max_len = max_seq_len;
  a.chunk = commvq::decode_chunk_len(k, v, batch, n_q_heads, max_seq_len, (int)flags);
  a.n_chunks = (max_seq_len + a.chunk - 1) / a.chunk;
  a.sm_scale = sm_scale;
  a.exact_phase = (flags & COMMVQ_DECODE_EXACT) ? 1 : 0;
  a.k = k;
  a.v = v;
  const PhaseConsts& pc = phase_consts(rope->theta_base, k.D);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool fast = commvq::decode_fast_path(k, v, a.NH, (int)flags);
  hipError_t e = hipSuccess;
  if (step && fast) {
    // the fast kernel encodes the new token inside the workgroup that reads it
    a.k_new = static_cast<const _Float16*>(step->k_new);
    a.v_new = static_cast<const _Float16*>(step->v_new);
    a.positions = step->positions;
    a.kcodes_w = const_cast<uint8_t*>(kcodes);
    a.vcodes_w = const_cast<uint8_t*>(vcodes);
    a.fold_new = k.R == 1 ? 1 : 0;  // R = 1: the merge kernel adds the new token
  } else if (step) {
    for (int kv = 0; kv < 2 && e == hipSuccess; ++kv) {
      const commvq::CbShape& sh = kv ? v : k;
      commvq::EncodeArgs ea{};
      ea.x = static_cast<const _Float16*>(kv ? step->v_new : step->k_new);
      ea.cb = static_cast<const _Float16*>(kv ? vcb->entries : kcb->entries);
      ea.codes = const_cast<uint8_t*>(kv ? vcodes : kcodes);
      ea.n_tokens = batch;
      ea.x_token_stride = (int64_t)sh.Hkv * sh.D;
      ea.code_token_stride = (int64_t)sh.Hkv * cache_len * sh.bpt;
      ea.code_head_stride = (int64_t)cache_len * sh.bpt;
      ea.positions = step->positions;
      ea.cache_len = cache_len;
      ea.s = sh;
      e = commvq::launch_encode(ea, s);
    }
  }
  if (e == hipSuccess) {
    if (fast) {
      e = commvq::launch_decode_fast(a, pc.ph, s);
    } else {
      e = commvq::launch_decode_generic(a, pc.ph, s);
    }
  }
  if (e == hipSuccess) e = commvq::launch_decode_merge(a, s);
  return hip_status(e, step ? "commvq_decode_step launch" : "commvq_decode_attention launch");
}

}  // namespace

extern "C" {

int32_t commvq_decode_attention(const commvq_codebook* kcb, const commvq_codebook* vcb, const commvq_rope* rope,
                                const float* q, const int32_t* q_pos, const uint8_t* kcodes,
                                const uint8_t* vcodes, const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                int32_t cache_len, int32_t max_seq_len, float sm_scale, float* out,
                                void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  return decode_impl(kcb, vcb, rope, q, q_pos, kcodes, vcodes, seq_lens, batch, n_q_heads, cache_len, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, flags, nullptr, stream);
}

int32_t commvq_decode_step(const commvq_codebook* kcb, const commvq_codebook* vcb, const commvq_rope* rope,
                           const void* k_new, const void* v_new, const int32_t* positions, const float* q,
                           const int32_t* q_pos, uint8_t* kcodes, uint8_t* vcodes, const int32_t* seq_lens,
                           int32_t batch, int32_t n_q_heads, int32_t cache_len, int32_t max_seq_len, float sm_scale,
                           float* out, void* workspace, size_t workspace_bytes, uint32_t flags, void* stream) {
  StepArgs st{k_new, v_new, positions};
  return decode_impl(kcb, vcb, rope, q, q_pos, kcodes, vcodes, seq_lens, batch, n_q_heads, cache_len, max_seq_len,
                     sm_scale, out, workspace, workspace_bytes, flags, &st, stream);
}

int32_t commvq_decode_step_noalloc(const commvq_codebook* kcb, const commvq_codebook* vcb, const commvq_rope* rope,
                                   const void* k_new, const void* v_new, const int32_t* positions, const float* q,
                                   const int32_t* q_pos, uint8_t* kcodes, uint8_t* vcodes, const int32_t* seq_lens,
                                   int32_t batch, int32_t n_q_heads, int32_t cache_len, int32_t max_seq_len,
                                   float sm_scale, float* out, uint32_t flags, void* stream) {
  StepArgs st{k_new, v_new, positions};
  return decode_impl(kcb, vcb, rope, q, q_pos, kcodes, vcodes, seq_lens, batch, n_q_heads, cache_len, max_seq_len,
                     sm_scale, out, nullptr, 0, flags, &st, stream, true);
}

}  // extern "C"

// ---- comparison path: dequantise, then dense attention ---------------------

namespace {

int32_t check_rope(const commvq_rope* rope) {
  if (!rope) return fail(COMMVQ_ERR_INVALID_ARG, "null rope descriptor");
  if (!(rope->theta_base > 1.0) || !std::isfinite(rope->theta_base))
    return fail(COMMVQ_ERR_INVALID_ARG, "rope theta_base must be finite and > 1");
  if (rope->pairing != 0 || rope->reserved != 0)
    return fail(COMMVQ_ERR_UNSUPPORTED, "rope pairing %d: only interleaved pairs (0) are supported", rope->pairing);
  return COMMVQ_OK;
}

int32_t dense_shapes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t max_seq_len) {
  if (batch < 1) return fail(COMMVQ_ERR_INVALID_ARG, "batch %d < 1", batch);
  if (n_kv_heads < 1) return fail(COMMVQ_ERR_INVALID_ARG, "n_kv_heads %d < 1", n_kv_heads);
  if (n_q_heads < 1 || n_q_heads % n_kv_heads)
    return fail(COMMVQ_ERR_INVALID_ARG, "n_q_heads %d must be a positive multiple of n_kv_heads %d", n_q_heads,
                n_kv_heads);
  if (max_seq_len < 1) return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d < 1", max_seq_len);
  if (head_dim < 2 || (head_dim & 1)) return fail(COMMVQ_ERR_INVALID_ARG, "head_dim %d must be even and >= 2", head_dim);
  if (head_dim != 128) return fail(COMMVQ_ERR_UNSUPPORTED, "dense attention supports head_dim 128, not %d", head_dim);
  const int NH = n_q_heads / n_kv_heads;
  if (NH != 1 && NH != 2 && NH != 4 && NH != 8)
    return fail(COMMVQ_ERR_UNSUPPORTED, "query heads per KV head %d not in {1, 2, 4, 8}", NH);
  if (batch > 65535 || n_kv_heads > 65535)
    return fail(COMMVQ_ERR_UNSUPPORTED, "batch %d or n_kv_heads %d > 65535", batch, n_kv_heads);
  return COMMVQ_OK;
}

}  // namespace

extern "C" {

int32_t commvq_dequantize_kv(const commvq_codebook* kcb, const commvq_codebook* vcb, const commvq_rope* rope,
                             const uint8_t* kcodes, const uint8_t* vcodes, const int32_t* seq_lens, int32_t batch,
                             int32_t cache_len, int32_t max_seq_len, void* k_out, void* v_out, void* stream) {
  g_err[0] = 0;
  commvq::CbShape k, v;
  int32_t st = check_shape(kcb, "key codebook", &k);
  if (st) return st;
  st = check_shape(vcb, "value codebook", &v);
  if (st) return st;
  if (k.D != v.D || k.g != v.g || k.Hkv != v.Hkv)
    return fail(COMMVQ_ERR_INVALID_ARG, "key and value codebooks disagree on head_dim, group_size or n_kv_heads");
  if (k.g > 16) return fail(COMMVQ_ERR_UNSUPPORTED, "dequantisation supports group_size up to 16, not %d", k.g);
  st = check_rope(rope);
  if (st) return st;
  if (batch < 1) return fail(COMMVQ_ERR_INVALID_ARG, "batch %d < 1", batch);
  if (max_seq_len < 1) return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d < 1", max_seq_len);
  if (cache_len < max_seq_len)
    return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds cache_len %d", max_seq_len, cache_len);
  if (batch > 65535) return fail(COMMVQ_ERR_UNSUPPORTED, "batch %d > 65535", batch);
  st = check_entries(kcb, "key codebook");
  if (st) return st;
  st = check_entries(vcb, "value codebook");
  if (st) return st;
  if (!kcodes || !vcodes || !seq_lens || !k_out || !v_out)
    return fail(COMMVQ_ERR_INVALID_ARG, "null codes, seq_lens or output pointer");
  if ((reinterpret_cast<uintptr_t>(k_out) | reinterpret_cast<uintptr_t>(v_out)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "k_out and v_out must be 16-byte aligned");
  commvq::DequantArgs a{};
  a.kcodes = kcodes;
  a.vcodes = vcodes;
  a.seq_lens = seq_lens;
  a.kcb = static_cast<const _Float16*>(kcb->entries);
  a.vcb = static_cast<const _Float16*>(vcb->entries);
  a.kout = static_cast<_Float16*>(k_out);
  a.vout = static_cast<_Float16*>(v_out);
  a.B = batch;
  a.cache_len = cache_len;
  a.max_len = max_seq_len;
  a.k = k;
  a.v = v;
  const PhaseConsts& pc = phase_consts(rope->theta_base, k.D);
  return hip_status(commvq::launch_dequant_kv(a, pc.ph, static_cast<hipStream_t>(stream)),
                    "commvq_dequantize_kv launch");
}

int64_t commvq_dense_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                     int32_t max_seq_len) {
  g_err[0] = 0;
  const int32_t st = dense_shapes(batch, n_q_heads, n_kv_heads, head_dim, max_seq_len);
  if (st) return st;
  return (int64_t)commvq::dense_workspace_bytes(batch, n_q_heads, max_seq_len);
}

int32_t commvq_dense_decode_attention(const commvq_rope* rope, const float* q, const int32_t* q_pos, const void* k,
                                      const void* v, const int32_t* seq_lens, int32_t batch, int32_t n_q_heads,
                                      int32_t n_kv_heads, int32_t head_dim, int32_t cache_len, int32_t max_seq_len,
                                      float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                      void* stream) {
  g_err[0] = 0;
  int32_t st = dense_shapes(batch, n_q_heads, n_kv_heads, head_dim, max_seq_len);
  if (st) return st;
  st = check_rope(rope);
  if (st) return st;
  if (cache_len < max_seq_len)
    return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds cache_len %d", max_seq_len, cache_len);
  if (!std::isfinite(sm_scale)) return fail(COMMVQ_ERR_INVALID_ARG, "sm_scale is not finite");
  if (!q || !q_pos || !k || !v || !seq_lens || !out)
    return fail(COMMVQ_ERR_INVALID_ARG, "null q, q_pos, k, v, seq_lens or out pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out) | reinterpret_cast<uintptr_t>(k) |
       reinterpret_cast<uintptr_t>(v)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "q, out, k and v must be 16-byte aligned");
  const int64_t need = commvq_dense_workspace_bytes(batch, n_q_heads, n_kv_heads, head_dim, max_seq_len);
  if (need < 0) return (int32_t)need;
  if (!workspace || workspace_bytes < (size_t)need)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %lld required", workspace_bytes,
                (long long)need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  commvq::DenseArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.k = static_cast<const _Float16*>(k);
  a.v = static_cast<const _Float16*>(v);
  a.seq_lens = seq_lens;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = batch;
  a.Hq = n_q_heads;
  a.Hkv = n_kv_heads;
  a.NH = n_q_heads / n_kv_heads;
  a.cache_len = cache_len;
  a.max_len = max_seq_len;
  a.n_chunks = (max_seq_len + commvq::kDenseChunk - 1) / commvq::kDenseChunk;
  a.sm_scale = sm_scale;
  const PhaseConsts& pc = phase_consts(rope->theta_base, head_dim);
  return hip_status(commvq::launch_dense_decode(a, pc.ph, static_cast<hipStream_t>(stream)),
                    "commvq_dense_decode_attention launch");
}

}  // extern "C"

// ---- codebook fitting --------------------------------------------------------

extern "C" {

int64_t commvq_em_work_bytes(const commvq_codebook* cb) {
  g_err[0] = 0;
  commvq::CbShape s;
  const int32_t st = check_shape(cb, "codebook", &s);
  if (st) return st;
  return (int64_t)commvq::em_work_bytes(s);
}

int32_t commvq_em_step(const commvq_codebook* cb, const void* x, int64_t n_tokens, int64_t x_token_stride,
                       int32_t round, float temperature, float min_mass, void* new_entries, float* mass_out,
                       void* work, size_t work_bytes, void* stream) {
  g_err[0] = 0;
  commvq::CbShape s;
  int32_t st = check_shape(cb, "codebook", &s);
  if (st) return st;
  if (n_tokens < 1) return fail(COMMVQ_ERR_INVALID_ARG, "n_tokens %lld < 1", (long long)n_tokens);
  if (round < 0 || round >= s.R) return fail(COMMVQ_ERR_INVALID_ARG, "round %d not in [0, %d)", round, s.R);
  if (s.g > 16) return fail(COMMVQ_ERR_UNSUPPORTED, "codebook fitting supports group_size up to 16, not %d", s.g);
  if (commvq::em_accumulate_smem(s, round, temperature > 0.f) > 160 * 1024)
    return fail(COMMVQ_ERR_UNSUPPORTED, "rounds 0..%d of %d entries x %d scalars exceed the fitting kernel's LDS", round,
                s.Nc, s.g);
  if (!std::isfinite(temperature) || temperature < 0.f)
    return fail(COMMVQ_ERR_INVALID_ARG, "temperature must be finite and >= 0");
  if (!std::isfinite(min_mass) || min_mass < 0.f) return fail(COMMVQ_ERR_INVALID_ARG, "min_mass must be finite and >= 0");
  if (x_token_stride < (int64_t)s.Hkv * s.D)
    return fail(COMMVQ_ERR_INVALID_ARG, "x_token_stride %lld < n_kv_heads*head_dim", (long long)x_token_stride);
  st = check_entries(cb, "codebook");
  if (st) return st;
  if (!x || !new_entries) return fail(COMMVQ_ERR_INVALID_ARG, "null x or new_entries pointer");
  if (reinterpret_cast<uintptr_t>(x) & 3) return fail(COMMVQ_ERR_INVALID_ARG, "x must be 4-byte aligned");
  if (x_token_stride & 1) return fail(COMMVQ_ERR_INVALID_ARG, "x_token_stride must be even");
  if (reinterpret_cast<uintptr_t>(new_entries) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "new_entries must be 16-byte aligned");
  if (mass_out && (reinterpret_cast<uintptr_t>(mass_out) & 3))
    return fail(COMMVQ_ERR_INVALID_ARG, "mass_out must be 4-byte aligned");
  const size_t need = commvq::em_work_bytes(s);
  if (!work || work_bytes < need)
    return fail(COMMVQ_ERR_WORKSPACE, "work buffer of %zu bytes is smaller than the %zu required", work_bytes, need);
  if (reinterpret_cast<uintptr_t>(work) & 255) return fail(COMMVQ_ERR_WORKSPACE, "work must be 256-byte aligned");
  if ((n_tokens + 255) / 256 > INT32_MAX) return fail(COMMVQ_ERR_UNSUPPORTED, "n_tokens exceeds the launch grid");
  commvq::EmArgs a{};
  a.x = static_cast<const _Float16*>(x);
  a.n_tokens = n_tokens;
  a.x_token_stride = x_token_stride;
  a.cb = static_cast<const _Float16*>(cb->entries);
  a.new_cb = static_cast<_Float16*>(new_entries);
  a.work = static_cast<float*>(work);
  a.mass_out = mass_out;
  a.round = round;
  a.temperature = temperature;
  a.min_mass = min_mass;
  a.s = s;
  return hip_status(commvq::launch_em_step(a, static_cast<hipStream_t>(stream)), "commvq_em_step launch");
}

}  // extern "C"

// ---- binary value codes --------------------------------------------------------

extern "C" {

// Shapes of a binary-value decode: the key codebook as for decode attention,
// the bit codebook's descriptor (rows not checked).
static int32_t bitv_shapes(const commvq_codebook* kcb, const commvq_bit_codebook* vcb, int32_t batch,
                           int32_t n_q_heads, int32_t max_seq_len, uint32_t flags, commvq::CbShape* k) {
  commvq::CbShape kk;
  int32_t st = decode_shapes(kcb, kcb, batch, n_q_heads, max_seq_len, k, &kk);
  if (st) return st;
  if (flags & ~(uint32_t)COMMVQ_DECODE_EXACT) return fail(COMMVQ_ERR_INVALID_ARG, "unknown flags 0x%x", flags);
  if (!vcb) return fail(COMMVQ_ERR_INVALID_ARG, "null binary value codebook");
  const int nb = vcb->n_bits;
  if (nb < 32 || nb > 2048 || (nb & (nb - 1)))
    return fail(COMMVQ_ERR_INVALID_ARG, "n_bits %d must be a power of two in [32, 2048]", nb);
  if ((int64_t)vcb->dim != (int64_t)k->Hkv * k->D)
    return fail(COMMVQ_ERR_INVALID_ARG, "binary value codebook dim %d must equal n_kv_heads*head_dim %d", vcb->dim,
                k->Hkv * k->D);
  if (vcb->dtype != COMMVQ_F16 || vcb->reserved != 0)
    return fail(COMMVQ_ERR_INVALID_ARG, "binary value codebook: dtype must be COMMVQ_F16, reserved 0");
  return COMMVQ_OK;
}

int64_t commvq_decode_bitv_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t max_seq_len,
                                           const commvq_codebook* kcb, const commvq_bit_codebook* vcb) {
  g_err[0] = 0;
  commvq::CbShape k;
  const int32_t st = bitv_shapes(kcb, vcb, batch, n_q_heads, max_seq_len, 0, &k);
  if (st) return st;
  return (int64_t)commvq::decode_bitv_workspace_bytes(k, vcb->n_bits, batch, n_q_heads, max_seq_len);
}

int32_t commvq_decode_attention_bitv(const commvq_codebook* kcb, const commvq_bit_codebook* vcb,
                                     const commvq_rope* rope, const float* q, const int32_t* q_pos,
                                     const uint8_t* kcodes, const uint8_t* vbits, const int32_t* seq_lens,
                                     int32_t batch, int32_t n_q_heads, int32_t cache_len, int32_t max_seq_len,
                                     float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                     uint32_t flags, void* stream) {
  g_err[0] = 0;
  commvq::CbShape k;
  int32_t st = bitv_shapes(kcb, vcb, batch, n_q_heads, max_seq_len, flags, &k);
  if (st) return st;
  const int nb = vcb->n_bits;
  if (!vcb->rows || (reinterpret_cast<uintptr_t>(vcb->rows) & 15))
    return fail(COMMVQ_ERR_INVALID_ARG, "binary value codebook rows must be non-null and 16-byte aligned");
  st = check_rope(rope);
  if (st) return st;
  if (cache_len < max_seq_len)
    return fail(COMMVQ_ERR_INVALID_ARG, "max_seq_len %d exceeds cache_len %d", max_seq_len, cache_len);
  if (!std::isfinite(sm_scale)) return fail(COMMVQ_ERR_INVALID_ARG, "sm_scale is not finite");
  st = check_entries(kcb, "key codebook");
  if (st) return st;
  if (!q || !q_pos || !kcodes || !vbits || !seq_lens || !out)
    return fail(COMMVQ_ERR_INVALID_ARG, "null q, q_pos, codes, bits, seq_lens or out pointer");
  if ((reinterpret_cast<uintptr_t>(q) | reinterpret_cast<uintptr_t>(out)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "q and out must be 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(kcodes) | reinterpret_cast<uintptr_t>(vbits)) & 15)
    return fail(COMMVQ_ERR_INVALID_ARG, "kcodes and vbits must be 16-byte aligned");
  const int NH = n_q_heads / k.Hkv;
  const bool fast = commvq::decode_bitv_fast_path(k, nb, n_q_heads, (int)flags);
  if (!fast && commvq::decode_bitv_smem(k, nb, NH) > 160 * 1024)
    return fail(COMMVQ_ERR_UNSUPPORTED, "binary value decode's LDS staging for %d query heads and %d bits exceeds 160 KiB",
                NH, nb);
  const int64_t need = (int64_t)commvq::decode_bitv_workspace_bytes(k, nb, batch, n_q_heads, max_seq_len);
  if (!workspace || workspace_bytes < (size_t)need)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %lld required", workspace_bytes,
                (long long)need);
  if (reinterpret_cast<uintptr_t>(workspace) & 255)
    return fail(COMMVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  commvq::DecodeArgs a{};
  a.q = q;
  a.q_pos = q_pos;
  a.kcodes = kcodes;
  a.seq_lens = seq_lens;
  a.kcb = static_cast<const _Float16*>(kcb->entries);
  a.vbits = vbits;
  a.vrows = static_cast<const _Float16*>(vcb->rows);
  a.nbits = nb;
  a.part = static_cast<float*>(workspace);
  a.out = out;
  a.B = batch;
  a.Hq = n_q_heads;
  a.NH = NH;
  a.cache_len = cache_len;
  a.max_len = max_seq_len;
  a.chunk = commvq::decode_chunk_len(k, k, batch, n_q_heads, max_seq_len, fast ? (int)flags : COMMVQ_DECODE_EXACT);
  a.n_chunks = (max_seq_len + a.chunk - 1) / a.chunk;
  a.sm_scale = sm_scale;
  a.exact_phase = (flags & COMMVQ_DECODE_EXACT) ? 1 : 0;
  a.k = k;
  a.v = k;
  const PhaseConsts& pc = phase_consts(rope->theta_base, k.D);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (fast) {
    // weights and chunk statistics, then o per (chunk, 128-bit range) slot
    a.pw = reinterpret_cast<_Float16*>(static_cast<char*>(workspace) +
                                       commvq::decode_bitv_pw_offset(k, nb, batch, n_q_heads, max_seq_len, a.chunk));
    a.n_chunks *= nb / 128;
    e = commvq::launch_decode_fast_bitv_scores(a, pc.ph, s);
    if (e == hipSuccess) e = commvq::launch_bitv_values(a, s);
    if (e == hipSuccess) e = commvq::launch_bitv_merge(a, s);
  } else {
    e = commvq::launch_decode_bitv(a, pc.ph, s);
    if (e == hipSuccess) e = commvq::launch_decode_merge(a, s);
  }
  return hip_status(e, "commvq_decode_attention_bitv launch");
}

}  // extern "C"

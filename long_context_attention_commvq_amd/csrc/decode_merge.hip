// Split-context combine: the decode kernels leave, per (sequence, query head,
// chunk of positions), the chunk's running max m_c, its sum of exponentials
// l_c and its unnormalised output o_c. The merged output is
//   o = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c,  M = max_c m_c,
// the standard combination of softmax partials over disjoint position ranges.
// Running it as its own kernel (ordered after the decode kernel on the stream)
// publishes the partials at the kernel boundary, instead of one release per
// workgroup across the XCDs' separate L2 caches. In a decode step on the fast
// 1-bit kernel the new token enters here as one more chunk: m = its scaled
// score (the sum of its 16 group products), l = 1, o = its value.

#include "decode_common.hpp"

namespace commvq {
namespace {

// One workgroup (T lanes) per (sequence, query head). Lane t takes dimension
// t % D and the chunks c = t / D (mod T / D), loading 16 of them at a time
// before using any (one memory round trip per batch; batches are combined with
// a running max and rescaling). The lanes sharing a dimension are combined the
// same way through LDS. T = 1024 when there are many partials (the binary-value
// path's chunk x bit-range slots), so that fewer batches run in a row.
template <int T>
__global__ __launch_bounds__(T) void decode_merge_kernel(DecodeArgs a) {
  constexpr int kMergeThreads = T;
  __shared__ float sm[3][kMergeThreads];
  __shared__ float sc_new;
  const float* __restrict__ part = a.part;
  const int n_chunks = a.n_chunks, D = a.k.D, Hq = a.Hq;
  // Workgroups go to the XCDs round-robin in launch order, and the decode
  // kernels put KV head h's chunks on XCD h mod 8 (KV head fastest). Workgroup
  // k Hkv + h merges query head h NH + k, on the XCD that wrote its partials.
  const int hq = (blockIdx.x % a.k.Hkv) * a.NH + blockIdx.x / a.k.Hkv, b = blockIdx.y, tid = threadIdx.x;
  const size_t cs = (size_t)D + 2;
  const float* pr = part + ((size_t)b * Hq + hq) * (size_t)n_chunks * cs;
  const int lpd = kMergeThreads / D;  // lanes per dimension (D <= 256)
  const int d = tid % D, sub = tid / D;
  const bool active = sub < lpd;
  float M = -INFINITY, l = 0.f, acc = 0.f;
  // the decode step's new token (fast 1-bit kernel): its terms are requested
  // with the partials (lanes 0..15 one group product each, lane d its value
  // dimension) and used after them, so its fold costs no second round trip
  float v_new = 0.f, scj = 0.f;
  int pbv = -1, Lv = 0;
  if (a.fold_new) {
    const int h = hq / a.NH, kk = hq % a.NH;
    const float* nt = a.newtok + ((size_t)b * a.k.Hkv + h) * kFastNewTokFloats;
    if (active && sub == 0) v_new = nt[64 + d];
    if (tid < 16) scj = nt[tid * 4 + kk];
    // vector loads (an opaque zero index), so that no scalar wait for them
    // stands before the partials' loads
    int z = 0;
    asm volatile("" : "+v"(z));
    pbv = a.positions[b + z];
    Lv = a.seq_lens[b + z];
  }
  if (active) {
    constexpr int KB = 16;  // chunks loaded per batch, all before any is used
    for (int c0 = sub; c0 < n_chunks; c0 += KB * lpd) {
      float mc[KB], lc[KB], oc[KB];
#pragma unroll
      for (int k = 0; k < KB; ++k) {
        const int c = c0 + k * lpd;
        const float* p = pr + (size_t)(c < n_chunks ? c : 0) * cs;
        mc[k] = c < n_chunks ? p[0] : -INFINITY;
        lc[k] = p[1];
        oc[k] = p[2 + d];
      }
      float Mb = M;
#pragma unroll
      for (int k = 0; k < KB; ++k) Mb = fmaxf(Mb, mc[k]);
      if (Mb > -INFINITY) {
        const float a = M > -INFINITY ? __expf(M - Mb) : 0.f;
        l *= a;
        acc *= a;
#pragma unroll
        for (int k = 0; k < KB; ++k) {
          const float w = mc[k] > -INFINITY ? __expf(mc[k] - Mb) : 0.f;
          l = fmaf(w, lc[k], l);
          acc = fmaf(w, oc[k], acc);
        }
        M = Mb;
      }
    }
  }
  sm[0][tid] = M;
  sm[1][tid] = l;
  sm[2][tid] = acc;
  if (a.fold_new && tid < 64) {
    // sum of the 16 group products (lanes 0..15; the other lanes hold 0)
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) scj += __shfl_xor(scj, o, 64);
    if (tid == 0) sc_new = scj;
  }
  __syncthreads();
  if (active && sub == 0) {
    auto add = [&](float mk, float lk, float ok) {
      if (mk > -INFINITY) {
        const float Mn = fmaxf(M, mk);
        const float sa = M > -INFINITY ? __expf(M - Mn) : 0.f, w = __expf(mk - Mn);
        l = fmaf(l, sa, w * lk);
        acc = fmaf(acc, sa, w * ok);
        M = Mn;
      }
    };
    for (int k = 1; k < lpd; ++k) add(sm[0][tid + k * D], sm[1][tid + k * D], sm[2][tid + k * D]);
    if (a.fold_new) {
      asm volatile("" : "+v"(Lv), "+v"(pbv));  // (used here, not where loaded)
      const int L = min(max(Lv, 0), a.max_len);
      if (pbv >= 0 && pbv < a.cache_len && pbv < L) add(sc_new * a.sm_scale, 1.f, v_new);
    }
    a.out[((size_t)b * Hq + hq) * D + d] = l > 0.f ? acc / l : 0.f;
  }
}

}  // namespace

hipError_t launch_decode_merge(const DecodeArgs& a, hipStream_t stream) {
  if (a.k.D > 256) return hipErrorInvalidValue;
  if (a.k.Hkv < 1 || a.NH * a.k.Hkv != a.Hq) return hipErrorInvalidValue;  // (the head remap is a bijection)
  if (a.fold_new && (a.k.D != 128 || a.NH != 4)) return hipErrorInvalidValue;  // the fast kernel's shape
  if (a.n_chunks > 64)
    hipLaunchKernelGGL(decode_merge_kernel<1024>, dim3(a.Hq, a.B), dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL(decode_merge_kernel<256>, dim3(a.Hq, a.B), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace commvq

// C-ABI entry points of libkla.so (declared in include/kla.h): argument
// validation on the host, then one kernel launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "../../include/kla.h"
#include "kla_internal.h"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};
Range range(const void *p, int64_t bytes) {
  const uintptr_t b = reinterpret_cast<uintptr_t>(p);
  return {b, b + static_cast<uintptr_t>(bytes > 0 ? bytes : 0)};
}
bool overlap(Range a, Range b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

bool supported_dim(int32_t dk, int32_t dv) { return dk == dv && (dk == 64 || dk == 128); }

constexpr int32_t kla_max_splits = 1024;

}  // namespace

extern "C" {

const char *kla_status_string(kla_status s) {
  switch (s) {
    case KLA_OK: return "ok";
    case KLA_ERR_INVALID_ARG: return "invalid argument";
    case KLA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case KLA_ERR_WORKSPACE: return "workspace too small";
    case KLA_ERR_HIP: return "HIP runtime error";
    default: break;
  }
  return "unknown status";
}

const char *kla_version(void) { return "0.1.0 gfx950"; }

size_t kla_fwd_chunked_workspace_size(int32_t n_seqs, int64_t, int32_t, int32_t, int32_t,
                                      int32_t) {
  // the longest-first order of packed sequences (int32 per sequence), used
  // when cu_seqlens is given for 2 .. kSeqOrderMax sequences
  if (n_seqs < 2 || n_seqs > kla::kSeqOrderMax) return 0;
  return ((size_t)n_seqs * 4 + 255) / 256 * 256;
}

size_t kla_fwd_chunked_split_workspace_size(int32_t n_seqs, int32_t H, int32_t dk, int32_t dv,
                                            int32_t n_splits) {
  if (n_seqs <= 0 || H <= 0 || n_splits <= 1 || !supported_dim(dk, dv)) return 0;
  // A and B maps for segments 0..P-2, start states for segments 0..P-1
  const size_t per = (size_t)dk * dv * sizeof(float);
  return (size_t)n_seqs * H * per * (size_t)(3 * n_splits - 2);
}

namespace {
kla_status fwd_impl(const void *q, const void *k, const void *v, const float *alpha,
                    const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                    int64_t total_tok, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                    float eps, kla_dtype dtype, kla_beta_mode beta_mode, int32_t n_splits,
                    const float *initial_state, float *o, float *final_state,
                    void *workspace, size_t workspace_bytes, void *stream,
                    bool channel_decay = false, bool noalloc = false) {
  if (n_seqs <= 0 || H <= 0 || total_tok < 0 || !std::isfinite(eps) || eps < 0.f)
    return KLA_ERR_INVALID_ARG;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_dim(dk, dv) || chunk != 64) return KLA_ERR_UNSUPPORTED;
  if (!cu_seqlens && total_tok % n_seqs != 0) return KLA_ERR_INVALID_ARG;
  if (n_splits < 1 || n_splits > kla_max_splits) return KLA_ERR_INVALID_ARG;
  if (channel_decay && n_splits != 1) return KLA_ERR_UNSUPPORTED;
  // one pass over packed sequences: their longest-first order
  const bool order = n_splits == 1 && !channel_decay && cu_seqlens && total_tok > 0;
  const size_t ws_need = n_splits > 1
      ? kla_fwd_chunked_split_workspace_size(n_seqs, H, dk, dv, n_splits)
      : order ? kla_fwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk) : 0;
  // no-allocation variant: the library's static scratch array stands in for
  // the workspace (its device address is taken after every other check)
  if (noalloc) workspace_bytes = KLA_NOALLOC_SCRATCH_BYTES;
  if (workspace_bytes < ws_need) return KLA_ERR_WORKSPACE;
  if (!noalloc && ws_need > 0 && (!workspace || !aligned16(workspace))) return KLA_ERR_INVALID_ARG;
  const bool have_tokens = total_tok > 0;
  if (have_tokens && (!q || !k || !v || !eta || !o)) return KLA_ERR_INVALID_ARG;
  if (have_tokens && channel_decay && !alpha) return KLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(initial_state) || !aligned16(final_state) || (channel_decay && !aligned16(alpha)))
    return KLA_ERR_INVALID_ARG;

  const int64_t esz = dtype == KLA_BF16 ? 2 : 4;
  const int64_t th = total_tok * H;
  const Range rq = range(q, th * dk * esz), rk = range(k, th * dk * esz),
              rv = range(v, th * dv * esz),
              ra = range(alpha, alpha ? th * 4 * (channel_decay ? dk : 1) : 0), re = range(eta, th * 4),
              ro = range(o, th * dv * 4),
              rcu = range(cu_seqlens, cu_seqlens ? (int64_t)(n_seqs + 1) * 4 : 0),
              rs0 = range(initial_state, initial_state ? (int64_t)n_seqs * H * dk * dv * 4 : 0),
              rs1 = range(final_state, final_state ? (int64_t)n_seqs * H * dk * dv * 4 : 0);
  const Range rws = range(noalloc ? nullptr : workspace, noalloc ? 0 : (int64_t)ws_need);
  for (const Range &in : {rq, rk, rv, ra, re, rcu, rs0, rs1, rws})
    if (overlap(ro, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rcu, rs0, rs1})
    if (overlap(rws, in)) return KLA_ERR_INVALID_ARG;
  if (final_state) {
    for (const Range &in : {rq, rk, rv, ra, re, rcu})
      if (overlap(rs1, in)) return KLA_ERR_INVALID_ARG;
    if (initial_state && initial_state != final_state && overlap(rs0, rs1))
      return KLA_ERR_INVALID_ARG;
  }

  kla::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.eta = eta;
  a.cu_seqlens = cu_seqlens;
  a.n_seqs = n_seqs;
  a.seq_len_dense = cu_seqlens ? 0 : total_tok / n_seqs;
  a.H = H;
  a.D = dk;
  a.eps = eps;
  a.beta_direct = beta_mode == KLA_BETA_DIRECT;
  a.initial_state = initial_state;
  a.o = o;
  a.final_state = final_state;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (channel_decay)
    return kla::launch_prefill_kda(a, dtype == KLA_BF16, st) == hipSuccess ? KLA_OK : KLA_ERR_HIP;
  auto run = [&]() {
    return dtype == KLA_BF16 ? kla::launch_prefill_bf16(a, st) : kla::launch_prefill_f32(a, st);
  };
  if (order && ws_need > 0) {
    int32_t *ord = static_cast<int32_t *>(workspace);
    if (kla::launch_seq_order(cu_seqlens, n_seqs, ord, st) != hipSuccess) return KLA_ERR_HIP;
    a.seq_order = ord;
  }
  if (n_splits == 1 || total_tok == 0) return run() == hipSuccess ? KLA_OK : KLA_ERR_HIP;
  if (noalloc && kla::noalloc_scratch(&workspace) != hipSuccess) return KLA_ERR_HIP;
  // split sequences: segment maps, scan of the maps, then every segment
  const size_t mat = (size_t)n_seqs * H * dk * dv;
  float *ws = static_cast<float *>(workspace);
  a.n_splits = n_splits;
  a.ws_a = ws;
  a.ws_b = ws + mat * (n_splits - 1);
  a.ws_s = ws + 2 * mat * (n_splits - 1);
  hipError_t e = kla::launch_split_identity(a, st);
  if (e == hipSuccess) {
    a.seg_mode = 1;
    e = run();
  }
  if (e == hipSuccess) e = kla::launch_split_scan(a, st);
  if (e == hipSuccess) {
    a.seg_mode = 2;
    e = run();
  }
  return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}
}  // namespace

kla_status kla_fwd_chunked_ex(const void *q, const void *k, const void *v, const float *alpha,
                              const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                              int64_t total_tok, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                              float eps, kla_dtype dtype, kla_beta_mode beta_mode,
                              const float *initial_state, float *o, float *final_state,
                              void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk, eps, dtype,
                  beta_mode, 1, initial_state, o, final_state, workspace, workspace_bytes, stream);
}

kla_status kla_fwd_chunked_split(const void *q, const void *k, const void *v, const float *alpha,
                                 const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                                 int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                                 int32_t chunk, float eps, kla_dtype dtype,
                                 kla_beta_mode beta_mode, int32_t n_splits,
                                 const float *initial_state, float *o, float *final_state,
                                 void *workspace, size_t workspace_bytes, void *stream) {
  return fwd_impl(q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk, eps, dtype,
                  beta_mode, n_splits, initial_state, o, final_state, workspace, workspace_bytes,
                  stream);
}

kla_status kla_fwd_chunked_split_noalloc(const void *q, const void *k, const void *v,
                                         const float *alpha, const float *eta,
                                         const int32_t *cu_seqlens, int32_t n_seqs,
                                         int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                                         int32_t chunk, float eps, kla_dtype dtype,
                                         kla_beta_mode beta_mode, int32_t n_splits,
                                         const float *initial_state, float *o,
                                         float *final_state, void *stream) {
  return fwd_impl(q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk, eps, dtype,
                  beta_mode, n_splits, initial_state, o, final_state, nullptr, 0, stream, false,
                  true);
}

kla_status kla_fwd_chunked(const void *q, const void *k, const void *v, const float *alpha,
                           const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                           int64_t total_tok, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           float eps, kla_dtype dtype, const float *initial_state, float *o,
                           float *final_state, void *workspace, size_t workspace_bytes,
                           void *stream) {
  return kla_fwd_chunked_ex(q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk,
                            eps, dtype, KLA_BETA_KACZMARZ, initial_state, o, final_state,
                            workspace, workspace_bytes, stream);
}

kla_status kla_fwd_chunked_kda(const void *q, const void *k, const void *v, const float *alpha,
                               const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                               int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                               int32_t chunk, float eps, kla_dtype dtype,
                               kla_beta_mode beta_mode, const float *initial_state, float *o,
                               float *final_state, void *workspace, size_t workspace_bytes,
                               void *stream) {
  return fwd_impl(q, k, v, alpha, eta, cu_seqlens, n_seqs, total_tok, H, dk, dv, chunk, eps, dtype,
                  beta_mode, 1, initial_state, o, final_state, workspace, workspace_bytes, stream,
                  true);
}

namespace {
kla_status decode_impl(const void *q, const void *k, const void *v, const float *alpha,
                       const float *eta, float *state, float *o, int32_t n_seqs, int32_t H,
                       int32_t dk, int32_t dv, float eps, kla_dtype dtype,
                       kla_beta_mode beta_mode, void *stream, bool channel_decay) {
  if (n_seqs <= 0 || H <= 0 || !std::isfinite(eps) || eps < 0.f) return KLA_ERR_INVALID_ARG;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_dim(dk, dv)) return KLA_ERR_UNSUPPORTED;
  if (!q || !k || !v || !eta || !state || !o) return KLA_ERR_INVALID_ARG;
  if (channel_decay && !alpha) return KLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(o) ||
      (channel_decay && !aligned16(alpha)))
    return KLA_ERR_INVALID_ARG;
  const int64_t esz = dtype == KLA_BF16 ? 2 : 4;
  const int64_t nh = (int64_t)n_seqs * H;
  const Range rq = range(q, nh * dk * esz), rk = range(k, nh * dk * esz),
              rv = range(v, nh * dv * esz),
              ra = range(alpha, alpha ? nh * 4 * (channel_decay ? dk : 1) : 0), re = range(eta, nh * 4),
              rs = range(state, nh * dk * dv * 4), ro = range(o, nh * dv * 4);
  for (const Range &in : {rq, rk, rv, ra, re, rs})
    if (overlap(ro, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re})
    if (overlap(rs, in)) return KLA_ERR_INVALID_ARG;

  kla::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.eta = eta;
  a.state = state;
  a.o = o;
  a.n_seqs = n_seqs;
  a.H = H;
  a.D = dk;
  a.eps = eps;
  a.beta_direct = beta_mode == KLA_BETA_DIRECT;
  a.channel_decay = channel_decay;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e =
      dtype == KLA_BF16 ? kla::launch_decode_bf16(a, st) : kla::launch_decode_f32(a, st);
  return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}
}  // namespace

kla_status kla_decode_step_ex(const void *q, const void *k, const void *v, const float *alpha,
                              const float *eta, float *state, float *o, int32_t n_seqs, int32_t H,
                              int32_t dk, int32_t dv, float eps, kla_dtype dtype,
                              kla_beta_mode beta_mode, void *stream) {
  return decode_impl(q, k, v, alpha, eta, state, o, n_seqs, H, dk, dv, eps, dtype, beta_mode,
                     stream, false);
}

kla_status kla_decode_step_kda(const void *q, const void *k, const void *v, const float *alpha,
                               const float *eta, float *state, float *o, int32_t n_seqs,
                               int32_t H, int32_t dk, int32_t dv, float eps, kla_dtype dtype,
                               kla_beta_mode beta_mode, void *stream) {
  return decode_impl(q, k, v, alpha, eta, state, o, n_seqs, H, dk, dv, eps, dtype, beta_mode,
                     stream, true);
}

kla_status kla_decode_step(const void *q, const void *k, const void *v, const float *alpha,
                           const float *eta, float *state, float *o, int32_t n_seqs, int32_t H,
                           int32_t dk, int32_t dv, float eps, kla_dtype dtype, void *stream) {
  return kla_decode_step_ex(q, k, v, alpha, eta, state, o, n_seqs, H, dk, dv, eps, dtype,
                            KLA_BETA_KACZMARZ, stream);
}

}  // extern "C"

// ---- curvature-conditioned read ---------------------------------------------
namespace {
constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ccq_record(int32_t dk) { return (int64_t)dk * dk + dk + 4; }
}  // namespace

extern "C" {

size_t kla_ccq_state_floats(int32_t dk) { return dk > 0 ? (size_t)ccq_record(dk) : 0; }

size_t kla_fwd_chunked_ccq_workspace_size(int64_t total_tok, int32_t H, int32_t dk, int32_t dv,
                                          kla_dtype dtype) {
  if (total_tok <= 0 || H <= 0 || !supported_dim(dk, dv)) return 0;
  const size_t th = (size_t)total_tok * H;
  if (dtype == KLA_BF16)  // q_clean hi and lo (bf16), the half-sequence sums' rows (fp32)
    return 2 * round_up(th * dk * 2) + round_up(th * dv * 4);
  return round_up(th * dk * 4);  // q_clean (fp32)
}

size_t kla_decode_step_ccq_workspace_size(int32_t n_seqs, int32_t H, int32_t dk) {
  if (n_seqs <= 0 || H <= 0 || dk <= 0) return 0;
  return round_up((size_t)n_seqs * H * dk * 4);
}

kla_status kla_fwd_chunked_ccq(const void *q, const void *k, const void *v, const float *alpha,
                               const float *eta, const float *lambda, const int32_t *cu_seqlens,
                               int32_t n_seqs, int64_t total_tok, int32_t H, int32_t dk,
                               int32_t dv, int32_t chunk, float eps, kla_dtype dtype,
                               kla_beta_mode beta_mode, const float *initial_state,
                               const float *ccq_in, float *o, float *final_state, float *ccq_out,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (n_seqs <= 0 || H <= 0 || total_tok < 0 || !std::isfinite(eps) || eps < 0.f)
    return KLA_ERR_INVALID_ARG;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_dim(dk, dv) || chunk != 64) return KLA_ERR_UNSUPPORTED;
  if (!cu_seqlens && total_tok % n_seqs != 0) return KLA_ERR_INVALID_ARG;
  const size_t ws_need = kla_fwd_chunked_ccq_workspace_size(total_tok, H, dk, dv, dtype);
  if (workspace_bytes < ws_need) return KLA_ERR_WORKSPACE;
  if (ws_need > 0 && (!workspace || !aligned16(workspace))) return KLA_ERR_INVALID_ARG;
  if (total_tok > 0 && (!q || !k || !v || !eta || !lambda || !o)) return KLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      !aligned16(initial_state) || !aligned16(final_state) || !aligned16(ccq_in) ||
      !aligned16(ccq_out))
    return KLA_ERR_INVALID_ARG;
  const int64_t esz = dtype == KLA_BF16 ? 2 : 4;
  const int64_t th = total_tok * H, rec = (int64_t)n_seqs * H * ccq_record(dk) * 4;
  const Range rq = range(q, th * dk * esz), rk = range(k, th * dk * esz),
              rv = range(v, th * dv * esz), ra = range(alpha, alpha ? th * 4 : 0),
              re = range(eta, th * 4), rl = range(lambda, th * 4), ro = range(o, th * dv * 4),
              rcu = range(cu_seqlens, cu_seqlens ? (int64_t)(n_seqs + 1) * 4 : 0),
              rs0 = range(initial_state, initial_state ? (int64_t)n_seqs * H * dk * dv * 4 : 0),
              rs1 = range(final_state, final_state ? (int64_t)n_seqs * H * dk * dv * 4 : 0),
              rc0 = range(ccq_in, ccq_in ? rec : 0), rc1 = range(ccq_out, ccq_out ? rec : 0),
              rws = range(workspace, (int64_t)ws_need);
  for (const Range &in : {rq, rk, rv, ra, re, rl, rcu, rs0, rs1, rc0, rc1, rws})
    if (overlap(ro, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rl, rcu, rs0, rs1, rc0, rc1})
    if (overlap(rws, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rl, rcu, rs0, rs1, rc0})
    if (overlap(rc1, in)) return KLA_ERR_INVALID_ARG;  // the end sums: a buffer of their own
  if (final_state) {
    for (const Range &in : {rq, rk, rv, ra, re, rl, rcu, rc0})
      if (overlap(rs1, in)) return KLA_ERR_INVALID_ARG;
    if (initial_state && initial_state != final_state && overlap(rs0, rs1))
      return KLA_ERR_INVALID_ARG;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  kla::CcqArgs c;
  c.q = q;
  c.k = k;
  c.lambda = lambda;
  c.cu_seqlens = cu_seqlens;
  c.n_seqs = n_seqs;
  c.seq_len_dense = cu_seqlens ? 0 : total_tok / n_seqs;
  c.H = H;
  c.D = dk;
  c.bf16_inputs = dtype == KLA_BF16;
  c.ccq_in = ccq_in;
  c.ccq_out = ccq_out;
  c.qh = ws;
  c.ql = dtype == KLA_BF16 ? ws + round_up((size_t)th * dk * 2) : nullptr;
  // the third part of the workspace holds the sums of the first halves of
  // long sequences (each in its own token rows) for the cleaning pass
  c.half_sums = dtype == KLA_BF16 ? reinterpret_cast<float *>(ws + 2 * round_up((size_t)th * dk * 2))
                                  : nullptr;
  hipError_t e = kla::launch_ccq_query(c, st);

  kla::PrefillArgs a;
  a.k = k;
  a.v = v;
  a.alpha = alpha;
  a.eta = eta;
  a.cu_seqlens = cu_seqlens;
  a.n_seqs = n_seqs;
  a.seq_len_dense = c.seq_len_dense;
  a.H = H;
  a.D = dk;
  a.eps = eps;
  a.beta_direct = beta_mode == KLA_BETA_DIRECT;
  a.initial_state = initial_state;
  // With no tokens the kernels only copy the start state and sums to the end
  // ones (workspace and query pointers are then never dereferenced).
  if (dtype == KLA_BF16) {
    // one state pass that reads with both bf16 parts of the cleaned query:
    // o = S^T (q_hi + q_lo)
    a.q = c.qh;
    a.q_lo = c.ql;
    a.o = o;
    a.final_state = final_state;
    if (e == hipSuccess) e = kla::launch_prefill_bf16(a, st);
  } else {
    a.q = c.qh;
    a.o = o;
    a.final_state = final_state;
    if (e == hipSuccess) e = kla::launch_prefill_f32(a, st);
  }
  return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

kla_status kla_decode_step_ccq(const void *q, const void *k, const void *v, const float *alpha,
                               const float *eta, const float *lambda, float *state,
                               float *ccq_state, float *o, int32_t n_seqs, int32_t H, int32_t dk,
                               int32_t dv, float eps, kla_dtype dtype, kla_beta_mode beta_mode,
                               void *workspace, size_t workspace_bytes, void *stream) {
  if (n_seqs <= 0 || H <= 0 || !std::isfinite(eps) || eps < 0.f) return KLA_ERR_INVALID_ARG;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_dim(dk, dv)) return KLA_ERR_UNSUPPORTED;
  const size_t ws_need = kla_decode_step_ccq_workspace_size(n_seqs, H, dk);
  if (workspace_bytes < ws_need) return KLA_ERR_WORKSPACE;
  if (!q || !k || !v || !eta || !lambda || !state || !ccq_state || !o || !workspace)
    return KLA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(state) || !aligned16(o) ||
      !aligned16(ccq_state) || !aligned16(workspace))
    return KLA_ERR_INVALID_ARG;
  const int64_t esz = dtype == KLA_BF16 ? 2 : 4;
  const int64_t nh = (int64_t)n_seqs * H;
  const Range rq = range(q, nh * dk * esz), rk = range(k, nh * dk * esz),
              rv = range(v, nh * dv * esz), ra = range(alpha, alpha ? nh * 4 : 0),
              re = range(eta, nh * 4), rl = range(lambda, nh * 4), rs = range(state, nh * dk * dv * 4),
              rc = range(ccq_state, nh * ccq_record(dk) * 4), ro = range(o, nh * dv * 4),
              rws = range(workspace, (int64_t)ws_need);
  for (const Range &in : {rq, rk, rv, ra, re, rl, rs, rc, rws})
    if (overlap(ro, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rl, rc, rws})
    if (overlap(rs, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rl, rws})
    if (overlap(rc, in)) return KLA_ERR_INVALID_ARG;
  for (const Range &in : {rq, rk, rv, ra, re, rl})
    if (overlap(rws, in)) return KLA_ERR_INVALID_ARG;

  kla::CcqDecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lambda = lambda;
  a.alpha = alpha;
  a.eta = eta;
  a.ccq_state = ccq_state;
  a.state = state;
  a.o = o;
  a.q_clean = static_cast<float *>(workspace);
  a.n_seqs = n_seqs;
  a.H = H;
  a.D = dk;
  a.eps = eps;
  a.beta_direct = beta_mode == KLA_BETA_DIRECT;
  a.bf16_inputs = dtype == KLA_BF16;
  const hipError_t e = kla::launch_ccq_decode_step(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? KLA_OK : KLA_ERR_HIP;
}

namespace {
// Workspace sections of the backward, in floats, each rounded up to 64.
struct BwdWs {
  size_t ckpt, dq, dk, db, c, kk, fin, total;
};
size_t up64(size_t x) { return (x + 63) / 64 * 64; }
BwdWs bwd_ws(int32_t n_seqs, int64_t total_tok, int32_t H, int32_t d) {
  BwdWs w;
  const size_t th = (size_t)total_tok * H, ns = (size_t)d / 16;
  w.ckpt = up64(((size_t)total_tok / 64 + n_seqs) * H * d * d);
  w.dq = up64(ns * th * d);
  w.dk = w.dq;
  w.db = up64(ns * th);
  w.c = w.db;
  w.kk = up64(th);
  w.fin = up64((size_t)n_seqs * H * d * d);
  w.total = w.ckpt + w.dq + w.dk + w.db + w.c + w.kk + w.fin;
  return w;
}
}  // namespace

size_t kla_bwd_chunked_workspace_size(int32_t n_seqs, int64_t total_tok, int32_t H, int32_t dk,
                                      int32_t dv, int32_t chunk) {
  if (n_seqs <= 0 || H <= 0 || total_tok < 0 || !supported_dim(dk, dv) || chunk != 64) return 0;
  return bwd_ws(n_seqs, total_tok, H, dk).total * sizeof(float);
}

kla_status kla_bwd_chunked(const void *q, const void *k, const void *v, const float *alpha,
                           const float *eta, const int32_t *cu_seqlens, int32_t n_seqs,
                           int64_t total_tok, int32_t H, int32_t dk, int32_t dv, int32_t chunk,
                           float eps, kla_dtype dtype, kla_beta_mode beta_mode,
                           const float *initial_state, const float *d_o, const float *d_final,
                           float *dq, float *dk_out, float *dv_out, float *d_alpha, float *d_eta,
                           float *d_initial, void *workspace, size_t workspace_bytes,
                           void *stream) {
  if (n_seqs <= 0 || H <= 0 || total_tok < 0 || !std::isfinite(eps) || eps < 0.f)
    return KLA_ERR_INVALID_ARG;
  if (beta_mode != KLA_BETA_KACZMARZ && beta_mode != KLA_BETA_DIRECT) return KLA_ERR_INVALID_ARG;
  if (dtype != KLA_F32 && dtype != KLA_BF16) return KLA_ERR_UNSUPPORTED;
  if (!supported_dim(dk, dv) || chunk != 64) return KLA_ERR_UNSUPPORTED;
  if (!cu_seqlens && total_tok % n_seqs != 0) return KLA_ERR_INVALID_ARG;
  const size_t ws_need = kla_bwd_chunked_workspace_size(n_seqs, total_tok, H, dk, dv, chunk);
  if (workspace_bytes < ws_need) return KLA_ERR_WORKSPACE;
  if (!workspace || !aligned16(workspace)) return KLA_ERR_INVALID_ARG;
  const bool have_tokens = total_tok > 0;
  if (have_tokens && (!q || !k || !v || !eta || !d_o || !dq || !dk_out || !dv_out || !d_eta ||
                      (alpha && !d_alpha)))
    return KLA_ERR_INVALID_ARG;
  for (const void *ptr : {q, k, v, (const void *)d_o, (const void *)dq, (const void *)dk_out,
                          (const void *)dv_out, (const void *)initial_state,
                          (const void *)d_final, (const void *)d_initial})
    if (!aligned16(ptr)) return KLA_ERR_INVALID_ARG;

  const int64_t esz = dtype == KLA_BF16 ? 2 : 4;
  const int64_t th = total_tok * H, st = (int64_t)n_seqs * H * dk * dv * 4;
  const Range in[] = {range(q, th * dk * esz), range(k, th * dk * esz), range(v, th * dv * esz),
                      range(alpha, alpha ? th * 4 : 0), range(eta, th * 4),
                      range(cu_seqlens, cu_seqlens ? (int64_t)(n_seqs + 1) * 4 : 0),
                      range(initial_state, initial_state ? st : 0), range(d_o, th * dv * 4),
                      range(d_final, d_final ? st : 0)};
  const Range out[] = {range(dq, th * dk * 4), range(dk_out, th * dk * 4), range(dv_out, th * dv * 4),
                       range(alpha ? d_alpha : nullptr, alpha ? th * 4 : 0), range(d_eta, th * 4),
                       range(d_initial, d_initial ? st : 0), range(workspace, (int64_t)ws_need)};
  for (size_t a = 0; a < sizeof(out) / sizeof(out[0]); ++a) {
    for (const Range &r : in)
      if (overlap(out[a], r)) return KLA_ERR_INVALID_ARG;
    for (size_t b = a + 1; b < sizeof(out) / sizeof(out[0]); ++b)
      if (overlap(out[a], out[b])) return KLA_ERR_INVALID_ARG;
  }

  const BwdWs w = bwd_ws(n_seqs, total_tok, H, dk);
  float *ws = static_cast<float *>(workspace);
  kla::BwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.alpha = alpha;
  p.eta = eta;
  p.cu_seqlens = cu_seqlens;
  p.n_seqs = n_seqs;
  p.seq_len_dense = cu_seqlens ? 0 : total_tok / n_seqs;
  p.total_tok = total_tok;
  p.H = H;
  p.D = dk;
  p.eps = eps;
  p.beta_direct = beta_mode == KLA_BETA_DIRECT;
  p.initial_state = initial_state;
  p.d_o = d_o;
  p.d_final = d_final;
  p.dq = dq;
  p.dk = dk_out;
  p.dv = dv_out;
  p.d_alpha = alpha ? d_alpha : nullptr;
  p.d_eta = d_eta;
  p.d_initial = d_initial;
  p.ws_ckpt = ws;
  p.ws_dq = p.ws_ckpt + w.ckpt;
  p.ws_dk = p.ws_dq + w.dq;
  p.ws_db = p.ws_dk + w.dk;
  p.ws_c = p.ws_db + w.db;
  p.ws_kk = p.ws_c + w.c;
  p.ws_fin = p.ws_kk + w.kk;
  return kla::launch_bwd(p, dtype == KLA_BF16, static_cast<hipStream_t>(stream)) == hipSuccess
             ? KLA_OK
             : KLA_ERR_HIP;
}

}  // extern "C"

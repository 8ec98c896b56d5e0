// C ABI of libgdn: argument validation and dispatch to the kernels.
// Every check runs before anything is enqueued, so an error return means no
// kernel was launched and no output was written.
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

thread_local char g_last_error[512];

int fail(int status, const char *fmt, const char *what) {
  snprintf(g_last_error, sizeof(g_last_error), fmt, what);
  return status;
}

bool misaligned(const void *p, uintptr_t a = 16) {
  return p && (reinterpret_cast<uintptr_t>(p) & (a - 1)) != 0;
}

bool head_size_ok(int d) { return d == 64 || d == 128; }

bool dtype_ok(int t) { return t == GDN_F32 || t == GDN_BF16 || t == GDN_F16; }

size_t esize(int t) { return t == GDN_F32 ? 4 : 2; }

// half-open byte ranges [a, a+na) and [b, b+nb) overlap?
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

int hip_status(hipError_t e, const char *where) {
  if (e == hipSuccess) return GDN_OK;
  snprintf(g_last_error, sizeof(g_last_error), "%s: %s", where, hipGetErrorString(e));
  return GDN_ERR_HIP;
}

}  // namespace

extern "C" {

GDN_API const char *gdn_status_string(int status) {
  switch (status) {
    case GDN_OK: return "GDN_OK";
    case GDN_ERR_INVALID_ARG: return "GDN_ERR_INVALID_ARG";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED";
    case GDN_ERR_MISALIGNED: return "GDN_ERR_MISALIGNED";
    case GDN_ERR_HIP: return "GDN_ERR_HIP";
    default: return "GDN_ERR_UNKNOWN";
  }
}

GDN_API const char *gdn_last_error(void) { return g_last_error; }

GDN_API int gdn_version(void) { return 100; }

GDN_API int32_t gdn_prefill_state_columns(int32_t N, int32_t H, int32_t dk, int32_t dv,
                                          int32_t in_dtype) {
  if (N < 0 || H <= 0 || !head_size_ok(dk) || !head_size_ok(dv) || !dtype_ok(in_dtype)) return 0;
  gdn::ChunkArgs a{};
  a.N = N;
  a.H = H;
  a.dk = dk;
  a.dv = dv;
  a.in_dtype = in_dtype;
  return gdn::chunk_fwd_state_columns(a);
}

}  // extern "C"

namespace {

// Shared by gdn_chunk_fwd (A == null: gates given as log alpha and beta) and
// gdn_chunk_fwd_gated (raw pre-activations plus per-head A and b_alpha).
int chunk_fwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *A, const float *b_alpha, const float *S0,
                   void *y, float *S_T, const int32_t *cu_seqlens, int32_t N, int32_t T,
                   int32_t H, int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                   void *stream, const char *name, gdn::ChunkArgs *prepared = nullptr) {
  g_last_error[0] = '\0';
  if (N < 0 || T < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N, T must be >= 0 and H > 0");
  if (!head_size_ok(dk) || !head_size_ok(dv))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dk and dv must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (static_cast<int64_t>(N) * H > (int64_t{1} << 31) / 8)
    return fail(GDN_ERR_INVALID_ARG, "%s", "N * H too large");
  if (rows * H * (dk > dv ? dk : dv) >= (int64_t{1} << 40))
    return fail(GDN_ERR_INVALID_ARG, "%s", "input too large");
  const bool any_rows = rows > 0;
  if (any_rows && (!q || !k || !v || !log_alpha || !beta || !y))
    return fail(GDN_ERR_INVALID_ARG, "%s", "null input or output pointer");
  if (N > 0 && !S_T && !y) return fail(GDN_ERR_INVALID_ARG, "%s", "no output requested");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(y) || misaligned(S0) ||
      misaligned(S_T) || misaligned(log_alpha, 4) || misaligned(beta, 4) ||
      misaligned(cu_seqlens, 4))
    return fail(GDN_ERR_MISALIGNED, "%s", "q, k, v, y, S0, S_T need 16-byte alignment, the rest 4");
  const size_t in_b = esize(in_dtype);
  const size_t nq = static_cast<size_t>(rows) * H * dk * in_b;
  const size_t nv = static_cast<size_t>(rows) * H * dv * in_b;
  const size_t ny = static_cast<size_t>(rows) * H * dv * esize(out_dtype);
  const size_t ns = static_cast<size_t>(N) * H * dk * dv * 4;
  const size_t ng = static_cast<size_t>(rows) * H * 4;
  const void *ins[5] = {q, k, v, log_alpha, beta};
  const size_t in_n[5] = {nq, nq, nv, ng, ng};
  for (int i = 0; i < 5; ++i) {
    if (overlap(ins[i], in_n[i], y, ny) || overlap(ins[i], in_n[i], S_T, ns))
      return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output");
  }
  if (overlap(y, ny, S_T, ns)) return fail(GDN_ERR_INVALID_ARG, "%s", "y overlaps S_T");
  if (S0 && S0 != S_T && overlap(S0, ns, S_T, ns))
    return fail(GDN_ERR_INVALID_ARG, "%s", "S0 partially overlaps S_T");
  if (S0 && overlap(S0, ns, y, ny)) return fail(GDN_ERR_INVALID_ARG, "%s", "S0 overlaps y");
  if (A) {
    if (misaligned(A, 4) || misaligned(b_alpha, 4))
      return fail(GDN_ERR_MISALIGNED, "%s", "A and b_alpha need 4-byte alignment");
    const size_t nh = static_cast<size_t>(H) * 4;
    if (overlap(A, nh, y, ny) || overlap(A, nh, S_T, ns) || overlap(b_alpha, nh, y, ny) ||
        overlap(b_alpha, nh, S_T, ns))
      return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output");
  }

  gdn::ChunkArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.A = A;
  a.b_alpha = A ? b_alpha : nullptr;
  a.S0 = S0;
  a.y = y;
  a.S_T = S_T;
  a.cu_seqlens = cu_seqlens;
  a.N = N;
  a.T = T;
  a.H = H;
  a.dk = dk;
  a.dv = dv;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  if (prepared) {  // validated only: the caller launches
    *prepared = a;
    return GDN_OK;
  }
  char where[64];
  snprintf(where, sizeof(where), "%s launch", name);
  return hip_status(gdn::launch_chunk_fwd(a), where);
}

// Workspace of gdn_chunk_fwd_segmented, byte offsets (each 256-aligned):
// segment bounds, the zero-start final states of segments 0 .. P-2, the true
// initial states of segments 1 .. P-1 and the transitions of segments
// 1 .. P-2, per sequence. Every byte is written before it is read.
struct SegLayout {
  size_t cu, nst, sin, mst, total;
};

SegLayout seg_layout(int N, int H, int dk, int dv, int P) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  const size_t per = static_cast<size_t>(H) * dk * dv * 4;
  const size_t mper = static_cast<size_t>(H) * dk * dk * 4;
  const size_t nm = P > 2 ? static_cast<size_t>(P - 2) : 0;
  SegLayout L;
  size_t off = 0;
  L.cu = off;
  off += al(static_cast<size_t>(N) * (P + 1) * 4);
  L.nst = off;
  off += al(static_cast<size_t>(N) * (P - 1) * per);
  L.sin = off;
  off += al(static_cast<size_t>(N) * (P - 1) * per);
  L.mst = off;
  off += al(static_cast<size_t>(N) * nm * mper);
  L.total = off;
  return L;
}

// Shared by every decode entry point. state_idx (may be null) is an int32
// table [N, idx_cols]: column 0 is the slot each sequence reads; with
// idx_cols = 1 + n_tok, column 1 + j is the slot the state after token j is
// written to; with idx_cols = 1 the final state goes back to the read slot.
// front end and output gate of the fused decode
struct DecodeFusion {
  const float *conv_w;
  void *conv_state;
  const void *z;
  const float *norm_w;
  float l2_eps, rms_eps;
};

int decode_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                const float *beta, const float *A, const float *b_alpha, float *S,
                const int32_t *state_idx, int32_t idx_cols, int32_t n_slots, void *y, int32_t N,
                int32_t n_tok, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype,
                int32_t out_dtype, void *stream, const char *name,
                const DecodeFusion *fx = nullptr) {
  g_last_error[0] = '\0';
  if (N < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N must be >= 0 and H > 0");
  if (n_tok < 1 || n_tok > gdn::kDecodeMaxTok)
    return fail(GDN_ERR_INVALID_ARG, "%s", "n_tok must be in [1, 8]");
  if (!head_size_ok(dk) || !head_size_ok(dv))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dk and dv must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  if (static_cast<int64_t>(N) * H * n_tok >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "N * H * n_tok too large");
  if (state_idx && n_slots < 0) return fail(GDN_ERR_INVALID_ARG, "%s", "n_slots must be >= 0");
  if (state_idx && static_cast<int64_t>(n_slots) * H >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "n_slots * H too large");
  const int64_t slots = state_idx ? n_slots : N;
  if (N > 0 && (!q || !k || !v || !log_alpha || !beta || !y || (slots > 0 && !S)))
    return fail(GDN_ERR_INVALID_ARG, "%s", "null pointer");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(y) || misaligned(S) ||
      misaligned(log_alpha, 4) || misaligned(beta, 4) || misaligned(A, 4) ||
      misaligned(b_alpha, 4) || misaligned(state_idx, 4))
    return fail(GDN_ERR_MISALIGNED, "%s", "q, k, v, y, S need 16-byte alignment, the rest 4");
  const size_t in_b = esize(in_dtype);
  const size_t rows = static_cast<size_t>(N) * n_tok * H;
  const size_t ns = static_cast<size_t>(slots) * H * dk * dv * 4;
  const size_t ny = rows * dv * esize(out_dtype);
  const size_t nh = static_cast<size_t>(H) * 4;
  const void *ins[8] = {q, k, v, log_alpha, beta, A, A ? b_alpha : nullptr, state_idx};
  const size_t in_n[8] = {rows * dk * in_b, rows * dk * in_b, rows * dv * in_b, rows * 4,
                          rows * 4, nh, nh, static_cast<size_t>(N) * idx_cols * 4};
  for (int i = 0; i < 8; ++i) {
    if (overlap(ins[i], in_n[i], S, ns) || overlap(ins[i], in_n[i], y, ny))
      return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output");
  }
  if (overlap(S, ns, y, ny)) return fail(GDN_ERR_INVALID_ARG, "%s", "S overlaps y");
  if (fx) {
    if (dk != dv) return fail(GDN_ERR_UNSUPPORTED, "%s", "the fused decode needs dk == dv");
    if (!(fx->l2_eps >= 0.0f) || !(fx->rms_eps >= 0.0f))
      return fail(GDN_ERR_INVALID_ARG, "%s", "l2_eps and rms_eps must be >= 0");
    if (N > 0 && (!fx->conv_w || !fx->z || (slots > 0 && !fx->conv_state)))
      return fail(GDN_ERR_INVALID_ARG, "%s", "null pointer");
    if (misaligned(fx->conv_w) || misaligned(fx->z) || misaligned(fx->conv_state) ||
        misaligned(fx->norm_w, 4))
      return fail(GDN_ERR_MISALIGNED, "%s",
                  "conv_w, z and conv_state need 16-byte alignment, norm_w 4");
    const size_t ncs = static_cast<size_t>(slots) * H * 9 * dk * in_b;
    const size_t nw = static_cast<size_t>(3) * H * dk * 4 * 4;
    const void *fin[3] = {fx->conv_w, fx->z, fx->norm_w};
    const size_t fin_n[3] = {nw, rows * dv * in_b, static_cast<size_t>(dv) * 4};
    for (int i = 0; i < 3; ++i)
      if (overlap(fin[i], fin_n[i], S, ns) || overlap(fin[i], fin_n[i], y, ny) ||
          overlap(fin[i], fin_n[i], fx->conv_state, ncs))
        return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output");
    for (int i = 0; i < 8; ++i)
      if (overlap(ins[i], in_n[i], fx->conv_state, ncs))
        return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps conv_state");
    if (overlap(fx->conv_state, ncs, S, ns) || overlap(fx->conv_state, ncs, y, ny))
      return fail(GDN_ERR_INVALID_ARG, "%s", "conv_state overlaps an output");
  }

  gdn::DecodeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.A = A;
  a.b_alpha = A ? b_alpha : nullptr;
  a.S = S;
  a.read_idx = state_idx;
  a.r_stride = idx_cols;
  a.write_idx = (state_idx && idx_cols > 1) ? state_idx + 1 : nullptr;
  a.w_stride = idx_cols;
  a.n_slots = static_cast<int>(slots);
  a.y = y;
  a.N = N;
  a.n_tok = n_tok;
  a.H = H;
  a.dk = dk;
  a.dv = dv;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  if (fx) {
    a.conv_w = fx->conv_w;
    a.conv_state = fx->conv_state;
    a.z = fx->z;
    a.norm_w = fx->norm_w;
    a.l2_eps = fx->l2_eps;
    a.rms_eps = fx->rms_eps;
  }
  char where[64];
  snprintf(where, sizeof(where), "%s launch", name);
  return hip_status(fx ? gdn::launch_decode_fused(a) : gdn::launch_decode_step(a), where);
}

}  // namespace

extern "C" {

GDN_API int gdn_chunk_fwd(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *beta, const float *S0, void *y, float *S_T,
                          const int32_t *cu_seqlens, int32_t N, int32_t T, int32_t H,
                          int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                          void *stream) {
  return chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, nullptr, S0, y, S_T, cu_seqlens, N,
                        T, H, dk, dv, in_dtype, out_dtype, stream, "gdn_chunk_fwd");
}

GDN_API int gdn_chunk_fwd_gated(const void *q, const void *k, const void *v, const float *a,
                                const float *b, const float *A, const float *b_alpha,
                                const float *S0, void *y, float *S_T, const int32_t *cu_seqlens,
                                int32_t N, int32_t T, int32_t H, int32_t dk, int32_t dv,
                                int32_t in_dtype, int32_t out_dtype, void *stream) {
  g_last_error[0] = '\0';
  if (H > 0 && !A) return fail(GDN_ERR_INVALID_ARG, "%s", "A is required");
  return chunk_fwd_impl(q, k, v, a, b, A, b_alpha, S0, y, S_T, cu_seqlens, N, T, H, dk, dv,
                        in_dtype, out_dtype, stream, "gdn_chunk_fwd_gated");
}

GDN_API size_t gdn_chunk_fwd_segmented_workspace_size(int64_t rows, int32_t N, int32_t H,
                                                      int32_t dk, int32_t dv, int32_t segments,
                                                      int32_t in_dtype) {
  if (rows < 0 || N < 0 || H <= 0 || !head_size_ok(dk) || !head_size_ok(dv) || segments < 2 ||
      segments > 64 || !dtype_ok(in_dtype))
    return 0;
  return seg_layout(N, H, dk, dv, segments).total;
}

// The segment-parallel prefill with its workspace given (validated here).
int segmented_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *S0, void *y, float *S_T,
                   const int32_t *cu_seqlens, int32_t N, int32_t T, int32_t H, int32_t dk,
                   int32_t dv, int32_t segments, void *workspace, size_t workspace_bytes,
                   int32_t in_dtype, int32_t out_dtype, void *stream, const char *name) {
  const int P = segments;
  if (P < 2 || P > 64) return fail(GDN_ERR_INVALID_ARG, "%s", "segments must be in [2, 64]");
  gdn::ChunkArgs base;
  const int st = chunk_fwd_impl(q, k, v, log_alpha, beta, nullptr, nullptr, S0, y, S_T,
                                cu_seqlens, N, T, H, dk, dv, in_dtype, out_dtype, stream, name,
                                &base);
  if (st != GDN_OK) return st;
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (rows >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "more than 2^31 - 1 rows");
  const SegLayout L = seg_layout(N, H, dk, dv, P);
  if (!workspace || workspace_bytes < L.total)
    return fail(GDN_ERR_INVALID_ARG, "%s", "workspace missing or smaller than "
                                           "gdn_chunk_fwd_segmented_workspace_size");
  if (misaligned(workspace, 256))
    return fail(GDN_ERR_MISALIGNED, "%s", "workspace needs 256-byte alignment");
  {
    const size_t nq = static_cast<size_t>(rows) * H * dk * esize(in_dtype);
    const size_t nv = static_cast<size_t>(rows) * H * dv * esize(in_dtype);
    const size_t ng = static_cast<size_t>(rows) * H * 4;
    const size_t ny = static_cast<size_t>(rows) * H * dv * esize(out_dtype);
    const size_t ns = static_cast<size_t>(N) * H * dk * dv * 4;
    const void *args[9] = {q, k, v, log_alpha, beta, S0, y, S_T, cu_seqlens};
    const size_t sizes[9] = {nq, nq, nv, ng, ng, ns, ny, ns, static_cast<size_t>(N + 1) * 4};
    for (int i = 0; i < 9; ++i)
      if (overlap(workspace, L.total, args[i], sizes[i]))
        return fail(GDN_ERR_INVALID_ARG, "%s", "the workspace overlaps an argument");
  }
  if (N == 0) return GDN_OK;

  char *w = static_cast<char *>(workspace);
  int32_t *cu_seg = reinterpret_cast<int32_t *>(w + L.cu);
  float *nst = reinterpret_cast<float *>(w + L.nst);
  float *sinit = reinterpret_cast<float *>(w + L.sin);
  float *mst = reinterpret_cast<float *>(w + L.mst);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  gdn::SegPrepArgs pa;
  pa.cu_seqlens = cu_seqlens;
  pa.N = N;
  pa.T = T;
  pa.P = P;
  pa.cu_seg = cu_seg;
  pa.stream = s;
  hipError_t e = gdn::launch_seg_prep(pa);
  if (e != hipSuccess) return hip_status(e, "segment bounds");

  const size_t per = static_cast<size_t>(H) * dk * dv;  // floats per state
  const size_t mper = static_cast<size_t>(H) * dk * dk;
  const int32_t Tall = static_cast<int32_t>(rows);      // row bound of the packed form
  for (int n = 0; n < N; ++n) {
    int32_t *cu_n = cu_seg + static_cast<size_t>(n) * (P + 1);
    float *nst_n = nst + static_cast<size_t>(n) * (P - 1) * per;
    float *sin_n = sinit + static_cast<size_t>(n) * (P - 1) * per;
    float *mst_n = mst + static_cast<size_t>(n) * (P > 2 ? P - 2 : 0) * mper;
    // segments 0 .. P-2 from zero, segment 0 from S0: their final states N,
    // and y of segment 0 (only)
    gdn::ChunkArgs a = base;
    a.cu_seqlens = cu_n;
    a.N = P - 1;
    a.T = Tall;
    a.S0 = S0 ? S0 + static_cast<size_t>(n) * per : nullptr;
    a.seg.s0_nseq = 1;
    a.seg.y_nseq = 1;
    a.S_T = nst_n;
    e = gdn::launch_chunk_fwd(a);
    if (e != hipSuccess) return hip_status(e, "segment summaries");
    // transitions M of segments 1 .. P-2: from the identity with v = 0, no y
    if (P > 2) {
      gdn::ChunkArgs b = base;
      b.dv = dk;
      b.S0 = nullptr;
      b.seg.s0_ident = 1;
      b.seg.v_zero = 1;
      b.y = nullptr;
      b.S_T = mst_n;
      b.cu_seqlens = cu_n + 1;
      b.N = P - 2;
      b.T = Tall;
      e = gdn::launch_chunk_fwd(b);
      if (e != hipSuccess) return hip_status(e, "segment transitions");
    }
    e = gdn::launch_seg_combine(nst_n, mst_n, sin_n, H, dk, dv, P, s);
    if (e != hipSuccess) return hip_status(e, "segment chain");
    // segments 1 .. P-1 again from their true initial states: their y, and
    // the last one's final state into S_T
    gdn::ChunkArgs c = base;
    c.cu_seqlens = cu_n + 1;
    c.N = P - 1;
    c.T = Tall;
    c.S0 = sin_n;
    c.S_T = S_T ? S_T + static_cast<size_t>(n) * per : nullptr;
    c.seg.st_first = P - 2;
    e = gdn::launch_chunk_fwd(c);
    if (e != hipSuccess) return hip_status(e, "segment outputs");
  }
  return GDN_OK;
}

GDN_API int gdn_chunk_fwd_segmented(const void *q, const void *k, const void *v,
                                    const float *log_alpha, const float *beta, const float *S0,
                                    void *y, float *S_T, const int32_t *cu_seqlens, int32_t N,
                                    int32_t T, int32_t H, int32_t dk, int32_t dv,
                                    int32_t segments, void *workspace, size_t workspace_bytes,
                                    int32_t in_dtype, int32_t out_dtype, void *stream) {
  g_last_error[0] = '\0';
  return segmented_impl(q, k, v, log_alpha, beta, S0, y, S_T, cu_seqlens, N, T, H, dk, dv,
                        segments, workspace, workspace_bytes, in_dtype, out_dtype, stream,
                        "gdn_chunk_fwd_segmented");
}

// Scratch of gdn_chunk_fwd_segmented_noalloc: a fixed device array, one copy
// on every GPU the library runs on, held until the process ends. In host code
// `scratch` names a host-side stand-in, not a device address: its address on
// a device comes from hipGetSymbolAddress with that device current, looked up
// once per device and kept in g_scratch_ptr.
constexpr size_t kNoAllocScratch = GDN_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratch];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

int scratch_of_current_device(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GDN_ERR_UNSUPPORTED, "%s", "device ordinal beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_status(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}
}  // namespace

GDN_API int gdn_chunk_fwd_segmented_noalloc(const void *q, const void *k, const void *v,
                                            const float *log_alpha, const float *beta,
                                            const float *S0, void *y, float *S_T,
                                            const int32_t *cu_seqlens, int32_t N, int32_t T,
                                            int32_t H, int32_t dk, int32_t dv, int32_t segments,
                                            int32_t in_dtype, int32_t out_dtype, void *stream) {
  g_last_error[0] = '\0';
  if (segments < 2 || segments > 64)
    return fail(GDN_ERR_INVALID_ARG, "%s", "segments must be in [2, 64]");
  if (N < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N must be >= 0 and H > 0");
  if (!head_size_ok(dk) || !head_size_ok(dv))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dk and dv must be 64 or 128");
  const size_t need = seg_layout(N, H, dk, dv, segments).total;
  if (need > kNoAllocScratch) {
    char msg[160];
    snprintf(msg, sizeof(msg), "needs %zu bytes of scratch, more than the fixed %zu "
             "(fewer sequences, heads or segments per call)", need, kNoAllocScratch);
    return fail(GDN_ERR_INVALID_ARG, "%s", msg);
  }
  void *ws = nullptr;
  const int rc = scratch_of_current_device(&ws);
  if (rc != GDN_OK) return rc;
  return segmented_impl(q, k, v, log_alpha, beta, S0, y, S_T, cu_seqlens, N, T, H, dk, dv,
                        segments, ws, kNoAllocScratch, in_dtype, out_dtype, stream,
                        "gdn_chunk_fwd_segmented_noalloc");
}

GDN_API int gdn_decode_step(const void *q, const void *k, const void *v, const float *log_alpha,
                            const float *beta, float *S, void *y, int32_t N, int32_t H,
                            int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                            void *stream) {
  return decode_impl(q, k, v, log_alpha, beta, nullptr, nullptr, S, nullptr, 1, 0, y, N, 1, H,
                     dk, dv, in_dtype, out_dtype, stream, "gdn_decode_step");
}

GDN_API int gdn_decode_step_gated(const void *q, const void *k, const void *v, const float *a,
                                  const float *b, const float *A, const float *b_alpha,
                                  float *S, const int32_t *state_idx, int32_t n_slots, void *y,
                                  int32_t N, int32_t H, int32_t dk, int32_t dv,
                                  int32_t in_dtype, int32_t out_dtype, void *stream) {
  g_last_error[0] = '\0';
  if (H > 0 && !A) return fail(GDN_ERR_INVALID_ARG, "%s", "A is required");
  return decode_impl(q, k, v, a, b, A, b_alpha, S, state_idx, 1, n_slots, y, N, 1, H, dk, dv,
                     in_dtype, out_dtype, stream, "gdn_decode_step_gated");
}

GDN_API int gdn_decode_fused(const void *q_raw, const void *k_raw, const void *v_raw,
                             const float *conv_w, void *conv_state, const float *g_a,
                             const float *g_b, const float *A, const float *b_alpha, float *S,
                             const int32_t *state_idx, int32_t n_slots, const void *z,
                             const float *norm_w, float l2_eps, float rms_eps, void *o,
                             int32_t N, int32_t n_tok, int32_t H, int32_t d, int32_t in_dtype,
                             int32_t out_dtype, void *stream) {
  const DecodeFusion fx{conv_w, conv_state, z, norm_w, l2_eps, rms_eps};
  return decode_impl(q_raw, k_raw, v_raw, g_a, g_b, A, b_alpha, S, state_idx, 1 + n_tok, n_slots,
                     o, N, n_tok, H, d, d, in_dtype, out_dtype, stream, "gdn_decode_fused", &fx);
}

GDN_API int gdn_decode_multi(const void *q, const void *k, const void *v, const float *g_a,
                             const float *g_b, const float *A, const float *b_alpha, float *S,
                             const int32_t *state_idx, int32_t n_slots, void *y, int32_t N,
                             int32_t n_tok, int32_t H, int32_t dk, int32_t dv, int32_t in_dtype,
                             int32_t out_dtype, void *stream) {
  return decode_impl(q, k, v, g_a, g_b, A, b_alpha, S, state_idx, 1 + n_tok, n_slots, y, N,
                     n_tok, H, dk, dv, in_dtype, out_dtype, stream, "gdn_decode_multi");
}

GDN_API int gdn_frontend_qkv(const void *q_raw, const void *k_raw, const void *v_raw,
                             const float *conv_w, const int32_t *cu_seqlens, int32_t N, int32_t T,
                             int32_t H, int32_t d, float l2_eps, void *q, void *k, void *v,
                             int32_t in_dtype, int32_t out_dtype, void *stream) {
  g_last_error[0] = '\0';
  if (N < 0 || T < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N, T must be >= 0 and H > 0");
  if (!head_size_ok(d)) return fail(GDN_ERR_UNSUPPORTED, "%s", "d must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  if (!(l2_eps >= 0.0f)) return fail(GDN_ERR_INVALID_ARG, "%s", "l2_eps must be >= 0");
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (rows * H * d >= (int64_t{1} << 40)) return fail(GDN_ERR_INVALID_ARG, "%s", "input too large");
  if ((rows + 63) / 64 * H * 3 >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "too many rows");
  if (rows > 0 && (!q_raw || !k_raw || !v_raw || !conv_w || !q || !k || !v))
    return fail(GDN_ERR_INVALID_ARG, "%s", "null pointer");
  if (misaligned(q_raw) || misaligned(k_raw) || misaligned(v_raw) || misaligned(conv_w) ||
      misaligned(q) || misaligned(k) || misaligned(v) || misaligned(cu_seqlens, 4))
    return fail(GDN_ERR_MISALIGNED, "%s", "tensors need 16-byte alignment, cu_seqlens 4");
  const size_t nin = static_cast<size_t>(rows) * H * d * esize(in_dtype);
  const size_t nout = static_cast<size_t>(rows) * H * d * esize(out_dtype);
  const void *ins[4] = {q_raw, k_raw, v_raw, conv_w};
  const size_t in_n[4] = {nin, nin, nin, static_cast<size_t>(3) * H * d * 4 * 4};
  const void *outs[3] = {q, k, v};
  for (int i = 0; i < 4; ++i)
    for (int j = 0; j < 3; ++j)
      if (overlap(ins[i], in_n[i], outs[j], nout))
        return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output");
  if (overlap(q, nout, k, nout) || overlap(q, nout, v, nout) || overlap(k, nout, v, nout))
    return fail(GDN_ERR_INVALID_ARG, "%s", "outputs overlap");
  gdn::FrontendArgs a;
  a.xq = q_raw;
  a.xk = k_raw;
  a.xv = v_raw;
  a.conv_w = conv_w;
  a.cu_seqlens = cu_seqlens;
  a.N = N;
  a.T = T;
  a.rows = rows;
  a.H = H;
  a.d = d;
  a.eps = l2_eps;
  a.q = q;
  a.k = k;
  a.v = v;
  a.in_dtype = in_dtype;
  a.out_dtype = out_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  if (cu_seqlens == nullptr && T == 0) return GDN_OK;
  return hip_status(gdn::launch_frontend(a), "gdn_frontend_qkv launch");
}

GDN_API int gdn_output_gate(const void *y, const void *z, const float *norm_w, float rms_eps,
                            void *o, int64_t rows, int32_t d, int32_t y_dtype, int32_t z_dtype,
                            int32_t out_dtype, void *stream) {
  const int32_t in_dtype = y_dtype;
  g_last_error[0] = '\0';
  if (rows < 0) return fail(GDN_ERR_INVALID_ARG, "%s", "rows must be >= 0");
  if (!head_size_ok(d)) return fail(GDN_ERR_UNSUPPORTED, "%s", "d must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(z_dtype) || !dtype_ok(out_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  if (!(rms_eps >= 0.0f)) return fail(GDN_ERR_INVALID_ARG, "%s", "rms_eps must be >= 0");
  if (rows / 64 >= (int64_t{1} << 31)) return fail(GDN_ERR_INVALID_ARG, "%s", "too many rows");
  if (rows > 0 && (!y || !z || !o)) return fail(GDN_ERR_INVALID_ARG, "%s", "null pointer");
  if (misaligned(y) || misaligned(z) || misaligned(o) || misaligned(norm_w, 4))
    return fail(GDN_ERR_MISALIGNED, "%s", "y, z, o need 16-byte alignment, norm_w 4");
  const size_t nin = static_cast<size_t>(rows) * d * esize(in_dtype);
  const size_t nz = static_cast<size_t>(rows) * d * esize(z_dtype);
  const size_t nout = static_cast<size_t>(rows) * d * esize(out_dtype);
  if (overlap(y, nin, o, nout) || overlap(z, nz, o, nout) ||
      overlap(norm_w, static_cast<size_t>(d) * 4, o, nout))
    return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps the output");
  gdn::GateArgs a;
  a.y = y;
  a.z = z;
  a.norm_w = norm_w;
  a.eps = rms_eps;
  a.o = o;
  a.rows = rows;
  a.d = d;
  a.in_dtype = in_dtype;
  a.z_dtype = z_dtype;
  a.out_dtype = out_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_output_gate(a), "gdn_output_gate launch");
}

namespace {

size_t pad256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

// byte offsets of the fused call's intermediates inside the workspace
struct FusedLayout {
  size_t qkv_bytes, y_bytes, q, k, v, y, total;
  FusedLayout(int64_t rows, int32_t H, int32_t d) {
    qkv_bytes = static_cast<size_t>(rows) * H * d * 2;
    y_bytes = static_cast<size_t>(rows) * H * d * 2;
    q = 0;
    k = q + pad256(qkv_bytes);
    v = k + pad256(qkv_bytes);
    y = v + pad256(qkv_bytes);
    total = rows > 0 ? y + pad256(y_bytes) : 0;
  }
};

}  // namespace

GDN_API size_t gdn_fused_workspace_size(int64_t rows, int32_t H, int32_t d) {
  if (rows < 0 || H <= 0 || !head_size_ok(d) || rows * H * d >= (int64_t{1} << 40)) return 0;
  return FusedLayout(rows, H, d).total;
}

GDN_API int gdn_chunk_fwd_fused(const void *q_raw, const void *k_raw, const void *v_raw,
                                const float *conv_w, const float *log_alpha, const float *beta,
                                const float *S0, const void *z, const float *norm_w,
                                float l2_eps, float rms_eps, void *o, float *S_T,
                                const int32_t *cu_seqlens, int32_t N, int32_t T, int32_t H,
                                int32_t dk, int32_t dv, int32_t in_dtype, int32_t out_dtype,
                                void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error[0] = '\0';
  if (N < 0 || T < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N, T must be >= 0 and H > 0");
  if (dk != dv) return fail(GDN_ERR_UNSUPPORTED, "%s", "the fused prefill needs dk == dv");
  const int32_t d = dk;
  if (!head_size_ok(d)) return fail(GDN_ERR_UNSUPPORTED, "%s", "d must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  // q, k, v and y pass between the stages in fp16: fp32 inputs would lose
  // the precision they are given for, so they take the three separate calls
  if (in_dtype == GDN_F32)
    return fail(GDN_ERR_UNSUPPORTED, "%s",
                "the fused prefill takes 16-bit inputs (fp32: gdn_frontend_qkv, gdn_chunk_fwd, "
                "gdn_output_gate)");
  if (!(l2_eps >= 0.0f) || !(rms_eps >= 0.0f))
    return fail(GDN_ERR_INVALID_ARG, "%s", "l2_eps and rms_eps must be >= 0");
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (static_cast<int64_t>(N) * H > (int64_t{1} << 31) / 8)
    return fail(GDN_ERR_INVALID_ARG, "%s", "N * H too large");
  if (rows * H * d >= (int64_t{1} << 40)) return fail(GDN_ERR_INVALID_ARG, "%s", "input too large");
  if ((rows + 63) / 64 * H * 3 >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "too many rows");
  const FusedLayout lay(rows, H, d);
  if (rows > 0) {
    if (!q_raw || !k_raw || !v_raw || !conv_w || !log_alpha || !beta || !z || !o)
      return fail(GDN_ERR_INVALID_ARG, "%s", "null input or output pointer");
    if (!workspace || workspace_bytes < lay.total)
      return fail(GDN_ERR_INVALID_ARG, "%s", "workspace missing or smaller than gdn_fused_workspace_size()");
  }
  if (misaligned(q_raw) || misaligned(k_raw) || misaligned(v_raw) || misaligned(conv_w) ||
      misaligned(z) || misaligned(o) || misaligned(S0) || misaligned(S_T) ||
      misaligned(workspace, 256) || misaligned(log_alpha, 4) || misaligned(beta, 4) ||
      misaligned(norm_w, 4) || misaligned(cu_seqlens, 4))
    return fail(GDN_ERR_MISALIGNED, "%s",
                "tensors need 16-byte alignment, the workspace 256, gates/norm_w/cu_seqlens 4");
  const size_t nin = static_cast<size_t>(rows) * H * d * esize(in_dtype);
  const size_t no = static_cast<size_t>(rows) * H * d * esize(out_dtype);
  const size_t ng = static_cast<size_t>(rows) * H * 4;
  const size_t ns = static_cast<size_t>(N) * H * d * d * 4;
  const void *ins[9] = {q_raw, k_raw, v_raw, z, conv_w, log_alpha, beta, norm_w, cu_seqlens};
  const size_t in_n[9] = {nin, nin, nin, nin, static_cast<size_t>(3) * H * d * 16, ng, ng,
                          static_cast<size_t>(d) * 4, static_cast<size_t>(N + 1) * 4};
  for (int i = 0; i < 9; ++i) {
    if (overlap(ins[i], in_n[i], o, no) || overlap(ins[i], in_n[i], S_T, ns) ||
        overlap(ins[i], in_n[i], workspace, lay.total))
      return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output or the workspace");
  }
  if (overlap(o, no, S_T, ns) || overlap(o, no, workspace, lay.total) ||
      overlap(S_T, ns, workspace, lay.total))
    return fail(GDN_ERR_INVALID_ARG, "%s", "o, S_T and the workspace must not overlap");
  if (S0 && S0 != S_T && overlap(S0, ns, S_T, ns))
    return fail(GDN_ERR_INVALID_ARG, "%s", "S0 partially overlaps S_T");
  if (S0 && (overlap(S0, ns, o, no) || overlap(S0, ns, workspace, lay.total)))
    return fail(GDN_ERR_INVALID_ARG, "%s", "S0 overlaps o or the workspace");

  const hipStream_t st = static_cast<hipStream_t>(stream);
  char *ws = static_cast<char *>(workspace);
  void *q = ws + lay.q, *k = ws + lay.k, *v = ws + lay.v, *y = ws + lay.y;
  if (rows > 0) {
    gdn::FrontendArgs f;
    f.xq = q_raw;
    f.xk = k_raw;
    f.xv = v_raw;
    f.conv_w = conv_w;
    f.cu_seqlens = cu_seqlens;
    f.N = N;
    f.T = T;
    f.rows = rows;
    f.H = H;
    f.d = d;
    f.eps = l2_eps;
    f.q = q;
    f.k = k;
    f.v = v;
    f.in_dtype = in_dtype;
    f.out_dtype = GDN_F16;
    f.stream = st;
    const int rc = hip_status(gdn::launch_frontend(f), "gdn_chunk_fwd_fused front end");
    if (rc != GDN_OK) return rc;
  }
  gdn::ChunkArgs c;
  c.q = q;
  c.k = k;
  c.v = v;
  c.log_alpha = log_alpha;
  c.beta = beta;
  c.S0 = S0;
  c.y = y;
  c.S_T = S_T;
  c.cu_seqlens = cu_seqlens;
  c.N = N;
  c.T = T;
  c.H = H;
  c.dk = d;
  c.dv = d;
  c.in_dtype = GDN_F16;
  c.out_dtype = GDN_F16;
  c.stream = st;
  int rc = hip_status(gdn::launch_chunk_fwd(c), "gdn_chunk_fwd_fused prefill");
  if (rc != GDN_OK || rows == 0) return rc;
  gdn::GateArgs g;
  g.y = y;
  g.z = z;
  g.norm_w = norm_w;
  g.eps = rms_eps;
  g.o = o;
  g.rows = rows * H;
  g.d = d;
  g.in_dtype = GDN_F16;
  g.z_dtype = in_dtype;
  g.out_dtype = out_dtype;
  g.stream = st;
  return hip_status(gdn::launch_output_gate(g), "gdn_chunk_fwd_fused output gate");
}

GDN_API size_t gdn_chunk_bwd_workspace_size(int64_t rows, int32_t N, int32_t H, int32_t dk,
                                            int32_t dv, int32_t in_dtype) {
  if (rows < 0 || N < 0 || H <= 0 || !head_size_ok(dk) || !head_size_ok(dv) ||
      !dtype_ok(in_dtype) || rows * H * (dk > dv ? dk : dv) >= (int64_t{1} << 40))
    return 0;
  return gdn::chunk_bwd_workspace_size(rows, N, H, dk, dv, in_dtype);
}

}  // extern "C"

namespace {

int chunk_bwd_impl(const void *q, const void *k, const void *v, const float *log_alpha,
                   const float *beta, const float *A, const float *b_alpha, const float *S0,
                   const void *dy, const float *dS_T, const int32_t *cu_seqlens, int32_t N,
                   int32_t T, int32_t H, int32_t dk, int32_t dv, void *dq, void *dk_out,
                   void *dv_out, float *dlog_alpha, float *dbeta, float *dA, float *db_alpha,
                   float *dS0, int32_t in_dtype, int32_t grad_dtype, void *workspace,
                   size_t workspace_bytes, void *stream, const char *name) {
  if (N < 0 || T < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N, T must be >= 0 and H > 0");
  if (!head_size_ok(dk) || !head_size_ok(dv))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dk and dv must be 64 or 128");
  if (!dtype_ok(in_dtype) || !dtype_ok(grad_dtype))
    return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (static_cast<int64_t>(N) * H > (int64_t{1} << 31) / 8)
    return fail(GDN_ERR_INVALID_ARG, "%s", "N * H too large");
  if (rows * H * (dk > dv ? dk : dv) >= (int64_t{1} << 40))
    return fail(GDN_ERR_INVALID_ARG, "%s", "input too large");
  const size_t need = gdn::chunk_bwd_workspace_size(rows, N, H, dk, dv, in_dtype);
  if (N > 0 && (!workspace || workspace_bytes < need))
    return fail(GDN_ERR_INVALID_ARG, "%s",
                "workspace missing or smaller than gdn_chunk_bwd_workspace_size()");
  const bool any_rows = rows > 0;
  if (any_rows && (!q || !k || !v || !log_alpha || !beta || !dy || !dq || !dk_out || !dv_out ||
                   !dlog_alpha || !dbeta))
    return fail(GDN_ERR_INVALID_ARG, "%s", "null input or output pointer");
  if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(dy) || misaligned(S0) ||
      misaligned(dS_T) || misaligned(dq) || misaligned(dk_out) || misaligned(dv_out) ||
      misaligned(dS0) || misaligned(workspace, 256) || misaligned(log_alpha, 4) ||
      misaligned(beta, 4) || misaligned(dlog_alpha, 4) || misaligned(dbeta, 4) ||
      misaligned(cu_seqlens, 4))
    return fail(GDN_ERR_MISALIGNED, "%s",
                "tensors need 16-byte alignment, the workspace 256, gates and cu_seqlens 4");
  const size_t in_b = esize(in_dtype), g_b = esize(grad_dtype);
  const size_t nqk = static_cast<size_t>(rows) * H * dk, nv = static_cast<size_t>(rows) * H * dv;
  const size_t ng = static_cast<size_t>(rows) * H * 4;
  const size_t ns = static_cast<size_t>(N) * H * dk * dv * 4;
  const void *ins[9] = {q, k, v, log_alpha, beta, S0, dy, dS_T, cu_seqlens};
  const size_t in_n[9] = {nqk * in_b, nqk * in_b, nv * in_b, ng, ng, ns, nv * g_b, ns,
                          static_cast<size_t>(N + 1) * 4};
  const void *outs[7] = {dq, dk_out, dv_out, dlog_alpha, dbeta, dS0, workspace};
  const size_t out_n[7] = {nqk * g_b, nqk * g_b, nv * g_b, ng, ng, ns, N > 0 ? need : 0};
  for (int i = 0; i < 9; ++i)
    for (int j = 0; j < 7; ++j)
      if (overlap(ins[i], in_n[i], outs[j], out_n[j]))
        return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps an output or the workspace");
  for (int i = 0; i < 7; ++i)
    for (int j = i + 1; j < 7; ++j)
      if (overlap(outs[i], out_n[i], outs[j], out_n[j]))
        return fail(GDN_ERR_INVALID_ARG, "%s", "outputs overlap");
  if (A) {
    if (!dA || !db_alpha) return fail(GDN_ERR_INVALID_ARG, "%s", "dA and db_alpha are required");
    if (misaligned(A, 4) || misaligned(b_alpha, 4) || misaligned(dA, 4) ||
        misaligned(db_alpha, 4))
      return fail(GDN_ERR_MISALIGNED, "%s", "A, b_alpha, dA, db_alpha need 4-byte alignment");
    const size_t nh = static_cast<size_t>(H) * 4;
    const void *hin[2] = {A, b_alpha};
    const void *hout[2] = {dA, db_alpha};
    for (int i = 0; i < 2; ++i) {
      for (int j = 0; j < 7; ++j)
        if (overlap(hin[i], nh, outs[j], out_n[j]) || overlap(hout[i], nh, outs[j], out_n[j]))
          return fail(GDN_ERR_INVALID_ARG, "%s", "per-head gate arguments overlap an output");
      for (int j = 0; j < 9; ++j)
        if (overlap(hout[i], nh, ins[j], in_n[j]))
          return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps dA or db_alpha");
      for (int j = 0; j < 2; ++j)
        if (overlap(hout[i], nh, hin[j], nh) || (i != j && overlap(hout[i], nh, hout[j], nh)))
          return fail(GDN_ERR_INVALID_ARG, "%s", "per-head gate arguments overlap");
    }
  }

  gdn::BwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.log_alpha = log_alpha;
  a.beta = beta;
  a.S0 = S0;
  a.dy = dy;
  a.dS_T = dS_T;
  a.cu_seqlens = cu_seqlens;
  a.N = N;
  a.T = T;
  a.H = H;
  a.dk_size = dk;
  a.dv_size = dv;
  a.rows = rows;
  a.dq = dq;
  a.dk = dk_out;
  a.dv = dv_out;
  a.dlog_alpha = dlog_alpha;
  a.dbeta = dbeta;
  a.dS0 = dS0;
  a.ws_states = static_cast<float *>(workspace);
  const gdn::BwdLayout lay = gdn::chunk_bwd_layout(rows, N, H, dk, dv, in_dtype);
  a.ws_part = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.part);
  a.ws_carry = reinterpret_cast<float *>(static_cast<char *>(workspace) + lay.carry);
  a.run_off = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) + lay.table);
  a.A = A;
  a.b_alpha = A ? b_alpha : nullptr;
  a.dA = dA;
  a.db_alpha = db_alpha;
  a.in_dtype = in_dtype;
  a.grad_dtype = grad_dtype;
  a.stream = static_cast<hipStream_t>(stream);
  char where[64];
  snprintf(where, sizeof(where), "%s launch", name);
  return hip_status(gdn::launch_chunk_bwd(a), where);
}

}  // namespace

extern "C" {

GDN_API int gdn_chunk_bwd(const void *q, const void *k, const void *v, const float *log_alpha,
                          const float *beta, const float *S0, const void *dy, const float *dS_T,
                          const int32_t *cu_seqlens, int32_t N, int32_t T, int32_t H, int32_t dk,
                          int32_t dv, void *dq, void *dk_out, void *dv_out, float *dlog_alpha,
                          float *dbeta, float *dS0, int32_t in_dtype, int32_t grad_dtype,
                          void *workspace, size_t workspace_bytes, void *stream) {
  g_last_error[0] = '\0';
  return chunk_bwd_impl(q, k, v, log_alpha, beta, nullptr, nullptr, S0, dy, dS_T, cu_seqlens, N,
                        T, H, dk, dv, dq, dk_out, dv_out, dlog_alpha, dbeta, nullptr, nullptr,
                        dS0, in_dtype, grad_dtype, workspace, workspace_bytes, stream,
                        "gdn_chunk_bwd");
}

GDN_API int gdn_chunk_bwd_gated(const void *q, const void *k, const void *v, const float *a,
                                const float *b, const float *A, const float *b_alpha,
                                const float *S0, const void *dy, const float *dS_T,
                                const int32_t *cu_seqlens, int32_t N, int32_t T, int32_t H,
                                int32_t dk, int32_t dv, void *dq, void *dk_out, void *dv_out,
                                float *da, float *db, float *dA, float *db_alpha, float *dS0,
                                int32_t in_dtype, int32_t grad_dtype, void *workspace,
                                size_t workspace_bytes, void *stream) {
  g_last_error[0] = '\0';
  if (H > 0 && !A) return fail(GDN_ERR_INVALID_ARG, "%s", "A is required");
  return chunk_bwd_impl(q, k, v, a, b, A, b_alpha, S0, dy, dS_T, cu_seqlens, N, T, H, dk, dv, dq,
                        dk_out, dv_out, da, db, dA, db_alpha, dS0, in_dtype, grad_dtype,
                        workspace, workspace_bytes, stream, "gdn_chunk_bwd_gated");
}

GDN_API int gdn_conv_state_from_prefill(const void *q_raw, const void *k_raw, const void *v_raw,
                                        const int32_t *cu_seqlens, int32_t N, int32_t T,
                                        int32_t H, int32_t d, const int32_t *slot_idx,
                                        int32_t n_slots, void *conv_state, int32_t dtype,
                                        void *stream) {
  g_last_error[0] = '\0';
  if (N < 0 || T < 0 || H <= 0) return fail(GDN_ERR_INVALID_ARG, "%s", "N, T must be >= 0 and H > 0");
  if (!head_size_ok(d)) return fail(GDN_ERR_UNSUPPORTED, "%s", "d must be 64 or 128");
  if (!dtype_ok(dtype)) return fail(GDN_ERR_UNSUPPORTED, "%s", "dtype must be GDN_F32, GDN_BF16 or GDN_F16");
  const int64_t slots = slot_idx ? n_slots : N;
  if (slots < 0) return fail(GDN_ERR_INVALID_ARG, "%s", "n_slots must be >= 0");
  const int64_t rows = cu_seqlens ? static_cast<int64_t>(T) : static_cast<int64_t>(N) * T;
  if (rows * H * d >= (int64_t{1} << 40) || static_cast<int64_t>(N) * H >= (int64_t{1} << 31))
    return fail(GDN_ERR_INVALID_ARG, "%s", "input too large");
  if (N > 0 && (!q_raw || !k_raw || !v_raw || (slots > 0 && !conv_state)))
    return fail(GDN_ERR_INVALID_ARG, "%s", "null pointer");
  if (misaligned(cu_seqlens, 4) || misaligned(slot_idx, 4) || misaligned(conv_state, 4))
    return fail(GDN_ERR_MISALIGNED, "%s", "cu_seqlens, slot_idx and conv_state need 4-byte alignment");
  const size_t eb = esize(dtype);
  const size_t nin = static_cast<size_t>(rows) * H * d * eb;
  const size_t ncs = static_cast<size_t>(slots) * H * 9 * d * eb;
  const void *ins[5] = {q_raw, k_raw, v_raw, cu_seqlens, slot_idx};
  const size_t in_n[5] = {nin, nin, nin, static_cast<size_t>(N + 1) * 4, static_cast<size_t>(N) * 4};
  for (int i = 0; i < 5; ++i)
    if (overlap(ins[i], in_n[i], conv_state, ncs))
      return fail(GDN_ERR_INVALID_ARG, "%s", "an input overlaps conv_state");
  gdn::ConvStateArgs a;
  a.xq = q_raw;
  a.xk = k_raw;
  a.xv = v_raw;
  a.cu_seqlens = cu_seqlens;
  a.slot_idx = slot_idx;
  a.N = N;
  a.T = T;
  a.H = H;
  a.d = d;
  a.n_slots = static_cast<int>(slots);
  a.elem_bytes = static_cast<int>(eb);
  a.conv_state = conv_state;
  a.stream = static_cast<hipStream_t>(stream);
  return hip_status(gdn::launch_conv_state(a), "gdn_conv_state_from_prefill launch");
}

}  // extern "C"

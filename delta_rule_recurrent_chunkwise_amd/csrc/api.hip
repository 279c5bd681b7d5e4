// api.hip -- the extern "C" entry points of liblinattn.so.  Each validates
// its arguments on the host (no HIP call happens before validation passes),
// then enqueues one kernel on the caller's stream.  Declarations, argument
// meaning and layouts are documented in include/linattn.h.
#include <limits.h>
#include <stdint.h>

#include "../../include/linattn.h"
#include "launch.hpp"

namespace {

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
bool dtype_ok(int dt) { return dt == LA_DTYPE_F32 || dt == LA_DTYPE_BF16; }

// Element counts must stay addressable and the grid within one dimension:
// B*H and the chunk count B*H*ceil(T/64) fit an int, and every tensor (T
// rounded up to whole chunks) and the state hold fewer than 2^50 elements.
// t = 0 is allowed where the caller says so (a prefill over no tokens).
// Each bound is checked by division, so no product here can overflow.
bool sizes_ok(long long b, long long h, long long t, int dk, int dv, bool allow_empty = false) {
  const long long lim = 1LL << 50;
  const long long mx = (dk > dv ? dk : dv);  // callers pass dims >= 1
  if (b <= 0 || h <= 0 || t < (allow_empty ? 0 : 1)) return false;
  if (b > INT_MAX / h) return false;
  const long long bh = b * h;
  if (t > INT_MAX - 64) return false;  // the chunk count rounds t up to 64
  const long long nch = (t + 63) / 64;
  if (nch > 0 && bh > INT_MAX / nch) return false;  // one workgroup per chunk in some kernels
  const long long tp = nch * 64;
  if (tp > 0 && bh * nch > lim / 64 / mx) return false;
  return bh <= lim / ((long long)dk * dv);
}

int launch_rc(hipError_t e) { return e == hipSuccess ? LA_OK : LA_ERR_LAUNCH; }

// A workspace is needed only when its size is not 0: then it must be given,
// be at least that large, and start on a 256-byte boundary.
int workspace_rc(size_t need, const void* ws, size_t have) {
  if (need == 0) return LA_OK;
  if (ws == nullptr || have < need) return LA_ERR_WORKSPACE;
  if (((uintptr_t)ws & 255u) != 0) return LA_ERR_ALIGN;
  return LA_OK;
}

// The checks every prefill entry point shares, in the order the header
// documents them; LA_OK when the call may proceed to its workspace check.
int prefill_args_rc(int dtype, int B, int H, int T, int dk, int dv) {
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(B, H, T, dk > 0 ? dk : 1, dv > 0 ? dv : 1, true)) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  return LA_OK;
}

size_t prefill_ws(int mode, int B, int H, int T, int dk, int dv, int dtype) {
  if (prefill_args_rc(dtype, B, H, T, dk, dv) != LA_OK) return 0;
  linattn::PrefillArgs a{};
  a.B = B;
  a.H = H;
  a.T = T;
  a.dv = dv;
  return linattn::prefill_workspace_bytes(mode, dtype == LA_DTYPE_BF16, dk, a);
}

size_t backward_ws(int gated, int B, int H, int T, int dk, int dv, int dtype) {
  if (prefill_args_rc(dtype, B, H, T, dk, dv) != LA_OK) return 0;
  if (dtype == LA_DTYPE_F32 && (dk > 64 || dv > 64)) return 0;  // not supported
  linattn::BackwardArgs a{};
  a.B = B;
  a.H = H;
  a.T = T;
  a.dk_ = dk;
  a.dv_ = dv;
  static const char one = 0;
  a.g = gated ? &one : nullptr;  // only its presence matters here
  return linattn::delta_backward_workspace_bytes(dtype == LA_DTYPE_BF16, a);
}

size_t kda_ws(int B, int H, int T, int dk, int dv, int dtype) {
  if (prefill_args_rc(dtype, B, H, T, dk, dv) != LA_OK) return 0;
  if (dtype != LA_DTYPE_BF16) return 0;  // not supported
  linattn::BackwardArgs a{};
  a.B = B;
  a.H = H;
  a.T = T;
  a.dk_ = dk;
  a.dv_ = dv;
  return linattn::kda_backward_workspace_bytes(a);
}

// Segmented prefill: the prefill mode of a gate kind (-1 for none valid).
int seg_mode(int gate) {
  return gate == 0 ? linattn::PF_DELTA : gate == 1 ? linattn::PF_GATED : gate == 2 ? linattn::PF_SGATED : -1;
}

// The segment count a call uses (0: chosen by the library); 0 when the
// arguments are invalid for it.  Every check here precedes any HIP call.
int seg_count(int B, int H, int T, int dv, int segments) {
  if (segments < 0) return 0;
  if (segments == 0) return linattn::segmented_auto_segments(B, H, T, dv);
  return segments;
}

// The checks of deltanet_prefill_segmented after its pointers: LA_OK when
// the call may proceed to its alignment and workspace checks.
int seg_args_rc(int gate, int dtype, int B, int H, int T, int dk, int dv, int P) {
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (seg_mode(gate) < 0 || P < 1) return LA_ERR_SHAPE;
  if (P > 1) {
    if (T % P != 0) return LA_ERR_SHAPE;
    // (this also bounds the fix-up's one-dimensional grid, B*H*(P-1) times
    // ceil(T/P / 256) blocks, below 2^31)
    if ((long long)H * P > INT_MAX || !sizes_ok(B, (long long)H * P, T / P, dk, dv, true)) return LA_ERR_SHAPE;
  }
  if (dtype != LA_DTYPE_BF16) return LA_ERR_UNSUPPORTED_DIM;
  return LA_OK;
}

size_t seg_ws(int gate, int B, int H, int T, int dk, int dv, int dtype, int segments) {
  if (prefill_args_rc(dtype, B, H, T, dk, dv) != LA_OK) return 0;
  const int P = seg_count(B, H, T, dv, segments);
  if (P == 0 || seg_args_rc(gate, dtype, B, H, T, dk, dv, P) != LA_OK) return 0;
  if (P == 1) return gate == 1 ? prefill_ws(linattn::PF_GATED, B, H, T, dk, dv, dtype) : 0;
  if (T == 0) return 0;
  linattn::PrefillArgs a{};
  a.B = B;
  a.H = H;
  a.T = T;
  a.dv = dv;
  return linattn::segmented_layout(seg_mode(gate), dk, a, P).total;
}

}  // namespace

extern "C" {

const char* la_strerror(int code) {
  switch (code) {
    case LA_OK: return "success";
    case LA_ERR_NULL: return "a required pointer argument is NULL";
    case LA_ERR_SHAPE:
      return "invalid shape: B, H, N must be positive, T >= 0 for prefill, "
             "and sizes within range";
    case LA_ERR_DTYPE: return "dtype must be LA_DTYPE_F32 (0) or LA_DTYPE_BF16 (1)";
    case LA_ERR_UNSUPPORTED_DIM:
      return "unsupported head dimension: dk and dv must each be 16, 32, 64 or 128 "
             "(float32: dk <= 64 for deltanet_prefill with a per-channel gate, "
             "dk and dv <= 64 for the backward entry points; "
             "bf16 only for kda_prefill_backward and deltanet_prefill_segmented)";
    case LA_ERR_LAUNCH: return "the HIP runtime rejected a kernel launch";
    case LA_ERR_WORKSPACE:
      return "the workspace is NULL or smaller than the matching *_workspace_bytes() query returns";
    case LA_ERR_SCRATCH_LIMIT:
      return "la_prefill_noalloc: the call needs more scratch memory than the library's fixed "
             "LA_NOALLOC_SCRATCH_BYTES (64 MiB) array holds; use la_prefill with a workspace";
    case LA_ERR_ALIGN:
      return "q, k, v and o (prefill; and dO, dq, dk, dv, backward; q and k in and out, prologue) "
             "and S (decode) must be 16-byte aligned, and a workspace 256-byte aligned";
    default: return "unknown error code";
  }
}

size_t la_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  return prefill_ws(linattn::PF_LA, B, H, T, dk, dv, dtype);
}

int la_prefill(const void* q, const void* k, const void* v, void* o, float* S, float* z,
               int use_initial_state, int B, int H, int T, int dk, int dv, int dtype,
               void* workspace, size_t workspace_bytes, void* stream) {
  if (!S || !z || (T != 0 && (!q || !k || !v || !o))) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  if (int rc = workspace_rc(la_prefill_workspace_bytes(B, H, T, dk, dv, dtype), workspace,
                            workspace_bytes))
    return rc;
  linattn::PrefillArgs a{q, k, v, nullptr, nullptr, o, S, z, B, H, T, dv, use_initial_state ? 1 : 0};
  return launch_rc(linattn::launch_prefill(linattn::PF_LA, dtype == LA_DTYPE_BF16, dk, a, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int la_decode_step(const void* q, const void* k, const void* v, void* o, float* S, float* z,
                   int N, int H, int dk, int dv, int dtype, void* stream) {
  if (!q || !k || !v || !o || !S || !z) return LA_ERR_NULL;
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(N, H, 1, dk > 0 ? dk : 1, dv > 0 ? dv : 1)) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(S)) return LA_ERR_ALIGN;
  linattn::DecodeArgs a{q, k, v, nullptr, nullptr, o, S, z, N * H};
  return launch_rc(linattn::launch_decode(linattn::DEC_LA, dtype == LA_DTYPE_BF16, dk, dv, a,
                                          static_cast<hipStream_t>(stream)));
}

size_t deltanet_prefill_workspace_bytes(int gated, int B, int H, int T, int dk, int dv, int dtype) {
  return prefill_ws(gated ? linattn::PF_GATED : linattn::PF_DELTA, B, H, T, dk, dv, dtype);
}

int deltanet_prefill(const void* q, const void* k, const void* v, const void* beta,
                     const void* g, void* o, float* S, int use_initial_state, int B, int H,
                     int T, int dk, int dv, int dtype, void* workspace, size_t workspace_bytes,
                     void* stream) {
  if (!S || (T != 0 && (!q || !k || !v || !beta || !o))) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (g && dtype == LA_DTYPE_F32 && dk > 64) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  if (int rc = workspace_rc(deltanet_prefill_workspace_bytes(g != nullptr, B, H, T, dk, dv, dtype),
                            workspace, workspace_bytes))
    return rc;
  linattn::PrefillArgs a{q, k, v, beta, g, o, S, nullptr, B, H, T, dv, use_initial_state ? 1 : 0};
  return launch_rc(linattn::launch_prefill(g ? linattn::PF_GATED : linattn::PF_DELTA, dtype == LA_DTYPE_BF16, dk, a,
                                           workspace, static_cast<hipStream_t>(stream)));
}

int deltanet_decode_step(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, void* o, float* S, int N, int H, int dk, int dv,
                         int dtype, void* stream) {
  if (!q || !k || !v || !beta || !o || !S) return LA_ERR_NULL;
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(N, H, 1, dk > 0 ? dk : 1, dv > 0 ? dv : 1)) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(S)) return LA_ERR_ALIGN;
  linattn::DecodeArgs a{q, k, v, beta, g, o, S, nullptr, N * H};
  return launch_rc(linattn::launch_decode(g ? linattn::DEC_GATED : linattn::DEC_DELTA, dtype == LA_DTYPE_BF16, dk, dv, a,
                                          static_cast<hipStream_t>(stream)));
}

int gated_deltanet_prefill(const void* q, const void* k, const void* v, const void* beta,
                           const void* g, void* o, float* S, int use_initial_state, int B,
                           int H, int T, int dk, int dv, int dtype, void* stream) {
  if (!S || (T != 0 && (!q || !k || !v || !beta || !g || !o))) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  linattn::PrefillArgs a{q, k, v, beta, g, o, S, nullptr, B, H, T, dv, use_initial_state ? 1 : 0};
  return launch_rc(linattn::launch_prefill(linattn::PF_SGATED, dtype == LA_DTYPE_BF16, dk, a, nullptr,
                                           static_cast<hipStream_t>(stream)));
}

int gated_deltanet_decode_step(const void* q, const void* k, const void* v, const void* beta,
                               const void* g, void* o, float* S, int N, int H, int dk, int dv,
                               int dtype, void* stream) {
  if (!q || !k || !v || !beta || !g || !o || !S) return LA_ERR_NULL;
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(N, H, 1, dk > 0 ? dk : 1, dv > 0 ? dv : 1)) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(S)) return LA_ERR_ALIGN;
  linattn::DecodeArgs a{q, k, v, beta, g, o, S, nullptr, N * H};
  return launch_rc(linattn::launch_decode(linattn::DEC_SGATED, dtype == LA_DTYPE_BF16, dk, dv, a,
                                          static_cast<hipStream_t>(stream)));
}

size_t gla_prefill_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  return prefill_ws(linattn::PF_GLA, B, H, T, dk, dv, dtype);
}

int gla_prefill(const void* q, const void* k, const void* v, const void* g, void* o, float* S,
                int use_initial_state, int B, int H, int T, int dk, int dv, int dtype,
                void* workspace, size_t workspace_bytes, void* stream) {
  if (!S || (T != 0 && (!q || !k || !v || !o))) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  if (int rc = workspace_rc(gla_prefill_workspace_bytes(B, H, T, dk, dv, dtype), workspace,
                            workspace_bytes))
    return rc;
  linattn::PrefillArgs a{q, k, v, nullptr, g, o, S, nullptr, B, H, T, dv, use_initial_state ? 1 : 0};
  return launch_rc(linattn::launch_prefill(linattn::PF_GLA, dtype == LA_DTYPE_BF16, dk, a, workspace,
                                           static_cast<hipStream_t>(stream)));
}

int gla_decode_step(const void* q, const void* k, const void* v, const void* g, void* o,
                    float* S, int N, int H, int dk, int dv, int dtype, void* stream) {
  if (!q || !k || !v || !o || !S) return LA_ERR_NULL;
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(N, H, 1, dk > 0 ? dk : 1, dv > 0 ? dv : 1)) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(S)) return LA_ERR_ALIGN;
  linattn::DecodeArgs a{q, k, v, nullptr, g, o, S, nullptr, N * H};
  return launch_rc(linattn::launch_decode(linattn::DEC_GLA, dtype == LA_DTYPE_BF16, dk, dv, a,
                                          static_cast<hipStream_t>(stream)));
}

size_t deltanet_prefill_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  return backward_ws(0, B, H, T, dk, dv, dtype);
}

int deltanet_prefill_backward(const void* q, const void* k, const void* v, const void* beta,
                              const float* S0, const void* dO, const float* dST, void* dq, void* dk_out,
                              void* dv_out, void* dbeta, float* dS0, int B, int H, int T, int dk,
                              int dv, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  if (T != 0 && (!q || !k || !v || !beta || !dO || !dq || !dk_out || !dv_out || !dbeta)) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (dtype == LA_DTYPE_F32 && (dk > 64 || dv > 64)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk_out) ||
      !aligned16(dv_out))
    return LA_ERR_ALIGN;
  if (int rc = workspace_rc(backward_ws(0, B, H, T, dk, dv, dtype), workspace, workspace_bytes)) return rc;
  linattn::BackwardArgs a{q, k, v, beta, S0, dO, dST, dq, dk_out, dv_out, dbeta, dS0, B, H, T, dk, dv};
  return launch_rc(linattn::launch_delta_backward(dtype == LA_DTYPE_BF16, a, workspace,
                                                  static_cast<hipStream_t>(stream)));
}

size_t gated_deltanet_prefill_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  return backward_ws(1, B, H, T, dk, dv, dtype);
}

int gated_deltanet_prefill_backward(const void* q, const void* k, const void* v, const void* beta,
                                    const void* g, const float* S0, const void* dO, const float* dST,
                                    void* dq, void* dk_out, void* dv_out, void* dbeta, void* dg, float* dS0,
                                    int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (T != 0 && (!q || !k || !v || !beta || !g || !dO || !dq || !dk_out || !dv_out || !dbeta || !dg))
    return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (dtype == LA_DTYPE_F32 && (dk > 64 || dv > 64)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk_out) ||
      !aligned16(dv_out))
    return LA_ERR_ALIGN;
  if (int rc = workspace_rc(backward_ws(1, B, H, T, dk, dv, dtype), workspace, workspace_bytes)) return rc;
  linattn::BackwardArgs a{q, k, v, beta, S0, dO, dST, dq, dk_out, dv_out, dbeta, dS0, B, H, T, dk, dv, g, dg};
  return launch_rc(linattn::launch_delta_backward(dtype == LA_DTYPE_BF16, a, workspace,
                                                  static_cast<hipStream_t>(stream)));
}

size_t kda_prefill_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int dtype) {
  return kda_ws(B, H, T, dk, dv, dtype);
}

int kda_prefill_backward(const void* q, const void* k, const void* v, const void* beta, const void* g,
                         const float* S0, const void* dO, const float* dST, void* dq, void* dk_out, void* dv_out,
                         void* dbeta, void* dg, float* dS0, int B, int H, int T, int dk, int dv, int dtype,
                         void* workspace, size_t workspace_bytes, void* stream) {
  if (T != 0 && (!q || !k || !v || !beta || !g || !dO || !dq || !dk_out || !dv_out || !dbeta || !dg))
    return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (dtype != LA_DTYPE_BF16) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dO) || !aligned16(dq) || !aligned16(dk_out) ||
      !aligned16(dv_out))
    return LA_ERR_ALIGN;
  if (int rc = workspace_rc(kda_ws(B, H, T, dk, dv, dtype), workspace, workspace_bytes)) return rc;
  linattn::BackwardArgs a{q, k, v, beta, S0, dO, dST, dq, dk_out, dv_out, dbeta, dS0, B, H, T, dk, dv, g, dg};
  return launch_rc(linattn::launch_kda_backward(a, workspace, static_cast<hipStream_t>(stream)));
}

size_t deltanet_prefill_segmented_workspace_bytes(int gate, int B, int H, int T, int dk, int dv,
                                                  int dtype, int segments) {
  return seg_ws(gate, B, H, T, dk, dv, dtype, segments);
}

int deltanet_prefill_segments(int B, int H, int T, int dk, int dv) {
  if (prefill_args_rc(LA_DTYPE_BF16, B, H, T, dk, dv) != LA_OK) return 0;
  return linattn::segmented_auto_segments(B, H, T, dv);
}

int deltanet_prefill_segmented(const void* q, const void* k, const void* v, const void* beta,
                               const void* g, int gate, void* o, float* S, int use_initial_state,
                               int B, int H, int T, int dk, int dv, int dtype, int segments,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!S || (T != 0 && (!q || !k || !v || !beta || !o))) return LA_ERR_NULL;
  if (gate != 0 && T != 0 && !g) return LA_ERR_NULL;
  if (int rc = prefill_args_rc(dtype, B, H, T, dk, dv)) return rc;
  if (gate == 0 && g) return LA_ERR_SHAPE;
  const int P = seg_count(B, H, T, dv, segments);
  if (P == 0) return LA_ERR_SHAPE;
  if (int rc = seg_args_rc(gate, dtype, B, H, T, dk, dv, P)) return rc;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  if (int rc = workspace_rc(seg_ws(gate, B, H, T, dk, dv, dtype, segments), workspace, workspace_bytes))
    return rc;
  const int mode = seg_mode(gate);
  linattn::PrefillArgs a{q, k, v, beta, g, o, S, nullptr, B, H, T, dv, use_initial_state ? 1 : 0};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (P == 1 || T == 0) return launch_rc(linattn::launch_prefill(mode, 1, dk, a, workspace, st));
  return launch_rc(linattn::launch_segmented(mode, dk, a, P, workspace, st));
}

int deltanet_prologue(const void* q_in, const void* k_in, const void* beta_logits, void* q_out,
                      void* k_out, void* beta_out, int B, int H, int T, int dk, int beta_heads,
                      int apply_silu, float q_scale, int dtype, void* stream) {
  if (T != 0 && (!q_in || !k_in || !q_out || !k_out)) return LA_ERR_NULL;
  if (T != 0 && (beta_logits != nullptr) != (beta_out != nullptr)) return LA_ERR_NULL;
  if (!dtype_ok(dtype)) return LA_ERR_DTYPE;
  if (!sizes_ok(B, H, T, dk > 0 ? dk : 1, 1, true)) return LA_ERR_SHAPE;
  if (beta_logits && beta_heads != 1 && beta_heads != H) return LA_ERR_SHAPE;
  if (!dim_ok(dk)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q_in) || !aligned16(k_in) || !aligned16(q_out) || !aligned16(k_out)) return LA_ERR_ALIGN;
  linattn::PrologueArgs a{q_in, k_in, beta_logits, q_out, k_out, beta_out, B, H, T, dk,
                          beta_logits ? beta_heads : H, apply_silu ? 1 : 0, q_scale};
  return launch_rc(linattn::launch_prologue(dtype == LA_DTYPE_BF16, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// launch.hpp -- internal interface between the C-ABI entry points (api.hip)
// and the kernel launchers (decode.hip, prefill.hip, ...): argument structs,
// launcher declarations, and the workspace sizes (host-only arithmetic, so
// the validation in api.hip builds without the device compiler).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace linattn {

// DEC_GATED: decay per key channel; DEC_SGATED: one decay per token (Gated
// DeltaNet); DEC_GLA: gated linear attention, S <- a S + k^T v, o = q S.
enum DecodeKind { DEC_DELTA = 0, DEC_GATED = 1, DEC_LA = 2, DEC_SGATED = 3, DEC_GLA = 4 };
// PF_GATED: gated delta rule, decay per key channel; PF_SGATED: one decay per
// token (Gated DeltaNet); PF_GLA: gated linear attention (one decay per token).
enum PrefillMode { PF_LA = 0, PF_DELTA = 1, PF_GATED = 2, PF_GLA = 3, PF_SGATED = 4 };

struct DecodeArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;  // delta / gated only
  const void* g;     // gated only: [N*H][dk]; [N*H] for DEC_SGATED, DEC_GLA (may be NULL)
  void* o;
  float* S;
  float* z;          // linear attention only
  int nheads;        // N * H
};

struct PrefillArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;  // delta / gated only
  const void* g;     // gated only: log-decay [B,H,T,dk] (PF_GATED) or [B,H,T]
  void* o;
  float* S;
  float* z;          // linear attention only
  int B, H, T, dv, use_init;
  // backward pass only: when set, the state entering every chunk is written
  // to Sc [B*H][ceil(T/64)][dk][dv] in the input type (generic kernel:
  // neither o nor the final state is written then)
  float* Sc;
};

// Enqueue one kernel on `st`; returns hipGetLastError() of the launch, or
// hipErrorInvalidValue for a combination with no kernel.
hipError_t launch_decode(int kind, int bf16, int dk, int dv, const DecodeArgs& a,
                         hipStream_t st);
// The prefill with a workspace of at least prefill_workspace_bytes() bytes,
// 256-byte aligned (may be NULL when that is 0).
hipError_t launch_prefill(int mode, int bf16, int dk, const PrefillArgs& a, void* workspace,
                          hipStream_t st);
// The generic prefill kernel only (used by the backward pass with a.Sc set).
hipError_t launch_prefill_generic(int mode, int bf16, int dk, const PrefillArgs& a, hipStream_t st);
// Gradient of the ungated delta rule (backward.hip): see deltanet_prefill_backward.
struct BackwardArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const float* S0;   // initial state or NULL
  const void* dO;
  const float* dST;  // gradient of the final state or NULL
  void* dq;
  void* dk;
  void* dv;
  void* dbeta;
  float* dS0;        // gradient of the initial state or NULL
  int B, H, T, dk_, dv_;
  const void* g;     // one log-decay per token [B,H,T] (gated rule) or NULL
  void* dg;          // its gradient [B,H,T] (with g)
};
hipError_t launch_delta_backward(int bf16, const BackwardArgs& a, void* workspace, hipStream_t st);
// Gradient of the per-key-channel gated rule (bf16; a.g [B,H,T,dk], a.dg
// likewise): see kda_prefill_backward.
hipError_t launch_kda_backward(const BackwardArgs& a, void* workspace, hipStream_t st);
// The layer prologue (prologue.hip): see deltanet_prologue.
struct PrologueArgs {
  const void* q_in;
  const void* k_in;
  const void* beta_logits;  // [B, beta_heads, T] or NULL
  void* q_out;
  void* k_out;
  void* beta_out;           // [B, H, T]
  int B, H, T, dk, beta_heads, silu;
  float q_scale;
};
hipError_t launch_prologue(int bf16, const PrologueArgs& a, hipStream_t st);
// The software-pipelined delta-rule prefill for bf16, dk = 128, dv % 32 == 0:
// plain (a.g == NULL, no workspace) or gated (needs a workspace of
// gated_pipe_workspace_bytes(a) bytes).
hipError_t launch_prefill_pipe(const PrefillArgs& a, void* workspace, hipStream_t st);
// The per-key-channel gate pre-pass (bf16, dk in {16, 32, 64, 128}): for
// n = B*H*ceil(T/64) chunks, Gam Q, Gam K, K / Gam as bf16 [n][64][dk] each,
// then Gam_C as fp32 [n][dk], into `workspace` (gate_prep_bytes); Gam_C = -1
// in every channel marks a chunk whose decay leaves the factored form's
// range, whose three tiles then hold the raw q, k and g.
hipError_t launch_gate_prep(int dk, const PrefillArgs& a, void* workspace, hipStream_t st);
// The pipelined gated kernel (dk = 128) on the pre-pass's output `prep`; with
// a.Sc set it captures the chunk states (and writes neither o nor S).
hipError_t launch_prefill_pipe_prepped(const PrefillArgs& a, const void* prep, hipStream_t st);
// ... and with one decay per token (a.g [B,H,T]; no workspace).
hipError_t launch_prefill_pipe_token(const PrefillArgs& a, hipStream_t st);

// Chunk-parallel linear attention (bf16): every chunk's phi(K)^T V and
// colsum phi(K) into a workspace of la_par_workspace_bytes bytes, then their
// exclusive prefix in place (the chunk-start states) and the final S, z.
// gla: gated linear attention instead (no feature map or normaliser; a decay
// per token).
hipError_t launch_la_par_states(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st);
// ... then every chunk's output from its chunk-start state (bf16).
hipError_t launch_la_par_outputs(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st);

// The delta rule (mode PF_DELTA, PF_GATED or PF_SGATED, bf16) over each
// head's sequence cut into P >= 2 segments of T / P tokens that run side by
// side (segmented.hip): a pass from the caller's state over every segment, a
// pass from the identity with v = 0 (each segment's transition), a scan of the
// segments' incoming states, and a fix-up of the outputs.  The workspace is
// segmented_layout(...).total bytes, 256-byte aligned.
hipError_t launch_segmented(int mode, int dk, const PrefillArgs& a, int P, void* workspace,
                            hipStream_t st);

// ---------------------------------------------------------------------------
// Workspace sizes (C = ceil(T/64) chunks per head)
// ---------------------------------------------------------------------------
inline size_t workspace_round256(size_t n) { return (n + 255) / 256 * 256; }
inline size_t workspace_chunks(long B, long H, long T) { return (size_t)B * H * ((T + 63) / 64); }

// Chunk-parallel linear attention: [dS: fp32 chunks x dk x dv][dz, then z_c
// (or Gam_C): fp32 chunks x dk][S_c: bf16 chunks x dk x dv].
inline size_t la_par_workspace_bytes(int dk, const PrefillArgs& a) {
  const size_t n = workspace_chunks(a.B, a.H, a.T);
  return n * ((size_t)dk * a.dv + dk) * sizeof(float) + n * dk * a.dv * sizeof(uint16_t);
}

// Per-channel gate pre-pass: Gam Q, Gam K, K / Gam in bf16 (64 rows per
// chunk) and Gam_C in fp32.
inline size_t gate_prep_bytes(int dk, long B, long H, long T) {
  const size_t n = workspace_chunks(B, H, T);
  return 3 * n * 64 * dk * sizeof(uint16_t) + n * dk * sizeof(float);
}
inline size_t gated_pipe_workspace_bytes(const PrefillArgs& a) { return gate_prep_bytes(128, a.B, a.H, a.T); }

// Device memory a prefill needs beyond its inputs and outputs (0 for most
// paths): the chunk-parallel bf16 linear-attention kernels keep per-chunk
// states; the per-channel gated pipelined kernel reads the pre-pass's
// decay-scaled q and k.
inline size_t prefill_workspace_bytes(int mode, int bf16, int dk, const PrefillArgs& a) {
  if (a.T == 0 || !bf16) return 0;
  if (mode == PF_LA || mode == PF_GLA) return la_par_workspace_bytes(dk, a);
  if (mode == PF_GATED && dk == 128 && a.dv % 32 == 0) return gated_pipe_workspace_bytes(a);
  return 0;
}

// Segmented prefill with P segments (segment-heads n = B*H*P, Tp = T/P), each
// region on a 256-byte boundary:
//   Sz   fp32 [n][dk][dv]   every segment's final state from its own start
//   M    fp32 [n][dk][dk]   every segment's transition (from the identity)
//   oB   bf16 [n][Tp][dk]   the transition pass's outputs (rows M_t^T q_t)
//   v0   bf16 [n][Tp][dk]   zeros: the transition pass's values
//   F    bf16 [B*H][P-1][2][ceil(dk/32)][dv/16][64][8]: the incoming state of
//        segments 1 .. P-1 as bf16 high and low parts, in MFMA B-operand order
//   MF   bf16 [n][dk/16][2][ceil(dk/32)][64][8]: the transitions as high and
//        low parts, in MFMA A-operand order
//   prep the two passes' own workspace (the per-channel gate's pre-pass).
struct SegmentedLayout {
  size_t sz, m, ob, v0, f, mf, prep, total;
};
inline SegmentedLayout segmented_layout(int mode, int dk, const PrefillArgs& a, int P) {
  SegmentedLayout L{};
  const size_t n = (size_t)a.B * a.H * P, tp = (size_t)(a.T / P);
  const size_t k32 = (size_t)(dk + 31) / 32;
  PrefillArgs av = a, at = a;
  av.H = at.H = a.H * P;
  av.T = at.T = a.T / P;
  at.dv = dk;
  const size_t prep = prefill_workspace_bytes(mode, 1, dk, av) > prefill_workspace_bytes(mode, 1, dk, at)
                          ? prefill_workspace_bytes(mode, 1, dk, av)
                          : prefill_workspace_bytes(mode, 1, dk, at);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at_ = off;
    off += workspace_round256(bytes);
    return at_;
  };
  L.sz = take(n * dk * a.dv * sizeof(float));
  L.m = take(n * dk * dk * sizeof(float));
  L.ob = take(n * tp * dk * sizeof(uint16_t));
  L.v0 = take(n * tp * dk * sizeof(uint16_t));
  L.f = take((size_t)a.B * a.H * (P - 1) * 2 * k32 * (a.dv / 16) * 512 * sizeof(uint16_t));
  L.mf = take(n * (dk / 16) * 2 * k32 * 512 * sizeof(uint16_t));
  L.prep = take(prep);
  L.total = off;
  return L;
}

// The segment count chosen when the caller asks for it to be chosen: the
// largest power of two P <= 64 for which one pass over the segments (as
// B*H*P heads of 32 value columns per workgroup) still fits one wave of
// workgroups on the 256 compute units, with at least 512 tokens per segment
// and T % P == 0; 1 (one pass over the whole sequence) when that P is below 4,
// since the two passes then cost more than the idle compute units.
inline int segmented_auto_segments(int B, int H, int T, int dv) {
  const long long units = (long long)B * H * (((long long)dv + 31) / 32);
  int best = 1;
  for (int P = 2; P <= 64; P *= 2) {
    if (units * P > 256 || T % P != 0 || T / P < 512) break;
    best = P;
  }
  return best >= 4 ? best : 1;
}

// Backward: each region starting on a 256-byte boundary,
//   Sc, dSc   fp32 [chunks][dk][dv] each (the chunk states and their
//             gradients; bf16 paths use the first half of each);
//   gC        fp32 [chunks] (gated rule only: the decay of every chunk);
//   P, R^T    bf16 [chunks][dk][dk] and [chunks][dk][64] (bf16 only).
inline size_t delta_backward_workspace_bytes(int bf16, const BackwardArgs& a) {
  if (a.T == 0) return 0;
  const size_t n = workspace_chunks(a.B, a.H, a.T);
  size_t w = 2 * workspace_round256(n * a.dk_ * a.dv_ * sizeof(float));
  if (a.g) w += workspace_round256(n * sizeof(float));
  if (bf16) w += workspace_round256(n * a.dk_ * (a.dk_ + 64) * sizeof(uint16_t));
  return w;
}

// Per-channel gated backward, each region on a 256-byte boundary:
//   the gate pre-pass's tiles (gate_prep_bytes);
//   Sc, dSc   bf16 [chunks][dk][dv] each;
//   P, R^T    bf16 [chunks][dk][dk] and [chunks][dk][64].
inline size_t kda_backward_workspace_bytes(const BackwardArgs& a) {
  if (a.T == 0) return 0;
  const size_t n = workspace_chunks(a.B, a.H, a.T);
  size_t w = workspace_round256(gate_prep_bytes(a.dk_, a.B, a.H, a.T));
  w += 2 * workspace_round256(n * a.dk_ * a.dv_ * sizeof(uint16_t));
  w += workspace_round256(n * a.dk_ * (a.dk_ + 64) * sizeof(uint16_t));
  return w;
}

}  // namespace linattn

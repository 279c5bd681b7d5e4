// launch.hpp -- internal interface between the C-ABI entry points (api.hip)
// and the kernel launchers (decode.hip, prefill.hip).
#pragma once
#include <hip/hip_runtime.h>

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
// Device memory a prefill needs beyond its inputs and outputs (0 for most
// paths), and the prefill itself with a workspace of at least that many
// bytes, 256-byte aligned (may be NULL when the size is 0).
size_t prefill_workspace_bytes(int mode, int bf16, int dk, const PrefillArgs& a);
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
size_t delta_backward_workspace_bytes(int bf16, const BackwardArgs& a);
hipError_t launch_delta_backward(int bf16, const BackwardArgs& a, void* workspace, hipStream_t st);
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
size_t gated_pipe_workspace_bytes(const PrefillArgs& a);
hipError_t launch_prefill_pipe(const PrefillArgs& a, void* workspace, hipStream_t st);
// ... and with one decay per token (a.g [B,H,T]; no workspace).
hipError_t launch_prefill_pipe_token(const PrefillArgs& a, hipStream_t st);

// Chunk-parallel linear attention (bf16): every chunk's phi(K)^T V and
// colsum phi(K) into a workspace of la_par_workspace_bytes bytes, then their
// exclusive prefix in place (the chunk-start states) and the final S, z.
// gla: gated linear attention instead (no feature map or normaliser; a decay
// per token).
size_t la_par_workspace_bytes(int dk, const PrefillArgs& a);
hipError_t launch_la_par_states(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st);
// ... then every chunk's output from its chunk-start state (bf16).
hipError_t launch_la_par_outputs(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st);

}  // namespace linattn

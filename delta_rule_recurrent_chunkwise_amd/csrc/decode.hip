// decode.hip -- one-token decode steps that update each head's fp32 state in
// place: the delta rule (optionally with a per-key-channel decay) and ELU+1
// linear attention with its normaliser.
//
// Delta rule, from the layer forward of the article "From GPT-2 to Kimi K3,
// explained", section "DeltaNet (Fast Weight Programmers)", at one token:
//   (gated, sections "Gated Delta Net" / "KDA / Kimi Linear") S' = diag(a) S
//   r = k S',  u = beta (v - r),  S <- S' + k^T u,  o = q S = q S' + (q.k) u.
// Linear attention, section "Linear Attention", cached forward at one token:
//   S <- S + phi(k)^T v, z <- z + phi(k),
//   o = phi(q) S / phi(q).z = (phi(q) S_old + (phi(q).phi(k)) v)
//                             / (phi(q).z_old + phi(q).phi(k)).
// Writing the output through the old state lets each state element be read
// once and written once: the step is a pure streaming read-modify-write of
// the state, so the kernel is bound by HBM bandwidth.
//
// Layout of the work: a head's state is dk x dv fp32, row-major.  A thread
// owns 4 consecutive value columns (one float4) of RPT rows spaced RG apart,
// so one wave-wide load instruction reads whole contiguous rows.  The column
// sums over key rows (k S, q S) are finished across the RG row groups in LDS.
#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {

template <int DK, int DV>
struct DecodeShape {
  static constexpr int CQ = DV / 4;               // float4 column groups
  static constexpr int RPT = DK < 16 ? DK : 16;  // rows per thread
  static constexpr int RG = DK / RPT;             // row groups
  static constexpr int TPH = CQ * RG;             // threads per head
  static constexpr int HPB = 256 / TPH;           // heads per block
  static_assert(TPH <= 256 && 256 % TPH == 0, "bad decode shape");
};

__device__ __forceinline__ float elu_plus_one(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int DK, int DV, class E, int KIND>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
  typedef DecodeShape<DK, DV> Sh;
  typedef typename E::T T;
  constexpr int CQ = Sh::CQ, RPT = Sh::RPT, RG = Sh::RG, TPH = Sh::TPH, HPB = Sh::HPB;

  __shared__ float s_q[HPB][DK];
  __shared__ float s_k[HPB][DK];
  __shared__ float s_a[KIND == DEC_GATED ? HPB : 1][KIND == DEC_GATED ? DK : 1];
  __shared__ float s_z[KIND == DEC_LA ? HPB : 1][KIND == DEC_LA ? DK : 1];
  __shared__ float4 s_red0[HPB][RG][CQ];
  __shared__ float4 s_red1[HPB][RG][CQ];
  __shared__ float2 s_red2[HPB][RG][CQ];

  const int hb = threadIdx.x / TPH;
  const int tl = threadIdx.x % TPH;
  const int cq = tl % CQ;
  const int rg = tl / CQ;
  const long head = (long)blockIdx.x * HPB + hb;
  const bool active = head < a.nheads;
  const long hc = active ? head : 0;  // clamped index for address arithmetic

  float4* S4 = reinterpret_cast<float4*>(a.S) + hc * (DK * CQ);

  // Issue the state loads first: they are the bulk of the traffic.
  float4 s[RPT];
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    s[j] = active ? S4[(rg + RG * j) * CQ + cq] : make_float4(0.f, 0.f, 0.f, 0.f);
  }

  // Stage this block's per-row vectors (q, k, decay, z) in LDS as fp32.
  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* kg = reinterpret_cast<const T*>(a.k);
  for (int i = threadIdx.x; i < HPB * DK; i += 256) {
    const int h = i / DK, d = i % DK;
    const long hh = (long)blockIdx.x * HPB + h;
    float qv = 0.f, kv = 0.f;
    if (hh < a.nheads) {
      qv = E::ld(qg + hh * DK + d);
      kv = E::ld(kg + hh * DK + d);
    }
    if (KIND == DEC_LA) {
      qv = elu_plus_one(qv);
      kv = elu_plus_one(kv);
      s_z[h][d] = hh < a.nheads ? a.z[hh * DK + d] : 0.f;
    }
    if (KIND == DEC_GATED) {
      const T* gg = reinterpret_cast<const T*>(a.g);
      s_a[h][d] = hh < a.nheads ? __expf(E::ld(gg + hh * DK + d)) : 1.f;
    }
    s_q[h][d] = qv;
    s_k[h][d] = kv;
  }
  __syncthreads();

  // Partial column sums over this thread's rows.
  float4 r4 = make_float4(0.f, 0.f, 0.f, 0.f);   // k S' (delta) | unused (LA)
  float4 s4 = make_float4(0.f, 0.f, 0.f, 0.f);   // q S'          | phi(q) S
  float sc = 0.f;                                // q.k           | phi(q).phi(k)
  float sz = 0.f;                                // unused        | phi(q).z_old
#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    const float kr = s_k[hb][row];
    const float qr = s_q[hb][row];
    if (KIND == DEC_GATED) {
      const float ar = s_a[hb][row];
      s[j].x *= ar; s[j].y *= ar; s[j].z *= ar; s[j].w *= ar;
    }
    if (KIND != DEC_LA) {
      r4.x += kr * s[j].x; r4.y += kr * s[j].y; r4.z += kr * s[j].z; r4.w += kr * s[j].w;
    }
    s4.x += qr * s[j].x; s4.y += qr * s[j].y; s4.z += qr * s[j].z; s4.w += qr * s[j].w;
    if (cq == 0) {
      sc += qr * kr;
      if (KIND == DEC_LA) sz += qr * s_z[hb][row];
    }
  }
  if (RG > 1) {
    s_red0[hb][rg][cq] = r4;
    s_red1[hb][rg][cq] = s4;
    s_red2[hb][rg][cq] = make_float2(sc, sz);
    __syncthreads();
    r4 = make_float4(0.f, 0.f, 0.f, 0.f);
    s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    sc = 0.f;
    sz = 0.f;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      const float4 x = s_red0[hb][i][cq];
      const float4 y = s_red1[hb][i][cq];
      r4.x += x.x; r4.y += x.y; r4.z += x.z; r4.w += x.w;
      s4.x += y.x; s4.y += y.y; s4.z += y.z; s4.w += y.w;
      sc += s_red2[hb][i][0].x;
      sz += s_red2[hb][i][0].y;
    }
  } else {
    // a single row group: every thread of the head already holds the full
    // column sums; the scalar sum lives in the cq == 0 thread.
    s_red2[hb][0][cq] = make_float2(sc, sz);
    __syncthreads();
    sc = s_red2[hb][0][0].x;
    sz = s_red2[hb][0][0].y;
  }
  if (!active) return;

  const T* vg = reinterpret_cast<const T*>(a.v) + hc * DV + 4 * cq;
  const float4 v4 = make_float4(E::ld(vg), E::ld(vg + 1), E::ld(vg + 2), E::ld(vg + 3));
  float4 u4, o4;
  if (KIND == DEC_LA) {
    u4 = v4;
    const float inv = 1.f / (sz + sc);
    o4 = make_float4((s4.x + sc * v4.x) * inv, (s4.y + sc * v4.y) * inv,
                     (s4.z + sc * v4.z) * inv, (s4.w + sc * v4.w) * inv);
  } else {
    const float b = E::ld(reinterpret_cast<const T*>(a.beta) + hc);
    u4 = make_float4(b * (v4.x - r4.x), b * (v4.y - r4.y), b * (v4.z - r4.z),
                     b * (v4.w - r4.w));
    o4 = make_float4(s4.x + sc * u4.x, s4.y + sc * u4.y, s4.z + sc * u4.z,
                     s4.w + sc * u4.w);
  }

#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    const float kr = s_k[hb][row];
    s[j].x += kr * u4.x; s[j].y += kr * u4.y; s[j].z += kr * u4.z; s[j].w += kr * u4.w;
    S4[row * CQ + cq] = s[j];
  }
  if (KIND == DEC_LA && cq == 0) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int row = rg + RG * j;
      a.z[hc * DK + row] = s_z[hb][row] + s_k[hb][row];
    }
  }
  if (rg == 0) {
    T* og = reinterpret_cast<T*>(a.o) + hc * DV + 4 * cq;
    og[0] = E::cvt(o4.x);
    og[1] = E::cvt(o4.y);
    og[2] = E::cvt(o4.z);
    og[3] = E::cvt(o4.w);
  }
}

template <int DK, int DV, class E, int KIND>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  typedef DecodeShape<DK, DV> Sh;
  const int blocks = (a.nheads + Sh::HPB - 1) / Sh::HPB;
  hipLaunchKernelGGL((decode_kernel<DK, DV, E, KIND>), dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

template <class E, int KIND>
static hipError_t launch_decode_e(int dk, int dv, const DecodeArgs& a, hipStream_t st) {
#define LINATTN_DV(DKV)                                                   \
  switch (dv) {                                                           \
    case 16: return launch_decode_t<DKV, 16, E, KIND>(a, st);             \
    case 32: return launch_decode_t<DKV, 32, E, KIND>(a, st);             \
    case 64: return launch_decode_t<DKV, 64, E, KIND>(a, st);             \
    case 128: return launch_decode_t<DKV, 128, E, KIND>(a, st);           \
    default: return hipErrorInvalidValue;                                 \
  }
  switch (dk) {
    case 16: LINATTN_DV(16)
    case 32: LINATTN_DV(32)
    case 64: LINATTN_DV(64)
    case 128: LINATTN_DV(128)
    default: return hipErrorInvalidValue;
  }
#undef LINATTN_DV
}

hipError_t launch_decode(int kind, int bf16, int dk, int dv, const DecodeArgs& a,
                         hipStream_t st) {
  if (bf16) {
    if (kind == DEC_DELTA) return launch_decode_e<BF16, DEC_DELTA>(dk, dv, a, st);
    if (kind == DEC_GATED) return launch_decode_e<BF16, DEC_GATED>(dk, dv, a, st);
    return launch_decode_e<BF16, DEC_LA>(dk, dv, a, st);
  }
  if (kind == DEC_DELTA) return launch_decode_e<F32, DEC_DELTA>(dk, dv, a, st);
  if (kind == DEC_GATED) return launch_decode_e<F32, DEC_GATED>(dk, dv, a, st);
  return launch_decode_e<F32, DEC_LA>(dk, dv, a, st);
}

}  // namespace linattn

// decode.hip -- one-token decode steps that update each head's fp32 state in
// place: the delta rule (optionally with a decay per key channel or per
// token), ELU+1 linear attention with its normaliser, and gated linear
// attention.
//
// Delta rule, from the layer forward of the article "From GPT-2 to Kimi K3,
// explained", section "DeltaNet (Fast Weight Programmers)", at one token:
//   (gated, sections "Gated Delta Net" / "KDA / Kimi Linear") S' = diag(a) S
//   r = k S',  u = beta (v - r),  S <- S' + k^T u,  o = q S = q S' + (q.k) u.
// Linear attention, section "Linear Attention", cached forward at one token:
//   S <- S + phi(k)^T v, z <- z + phi(k),
//   o = phi(q) S / phi(q).z = (phi(q) S_old + (phi(q).phi(k)) v)
//                             / (phi(q).z_old + phi(q).phi(k)).
// Gated linear attention, section "Gated Delta Net" (the additive cache with
// a forgetting factor): S' = a S, S <- S' + k^T v, o = q S' + (q.k) v.
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

// RPTT: target rows per thread.  Fewer rows per thread means more threads
// per head and fewer bytes per thread in flight between the load and the
// store of the state, which streams better.
template <int DK, int DV, int RPTT>
struct DecodeShape {
  static constexpr int CQ = DV / 4;                    // float4 column groups
  static constexpr int RPT = DK < RPTT ? DK : RPTT;    // rows per thread
  static constexpr int RG = DK / RPT;                  // row groups
  static constexpr int TPH = CQ * RG;                  // threads per head
  static constexpr int NTB = TPH > 256 ? TPH : 256;    // threads per block
  static constexpr int HPB = NTB / TPH;                // heads per block
  static_assert(TPH <= 1024 && NTB % TPH == 0, "bad decode shape");
};

template <bool NT>
__device__ __forceinline__ float4 ld_state(const float4* p) {
  if constexpr (NT) {
    typedef float fx4 __attribute__((ext_vector_type(4)));
    const fx4 v = __builtin_nontemporal_load(reinterpret_cast<const fx4*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  } else {
    return *p;
  }
}
template <bool NT>
__device__ __forceinline__ void st_state(float4* p, float4 x) {
  if constexpr (NT) {
    typedef float fx4 __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store(fx4{x.x, x.y, x.z, x.w}, reinterpret_cast<fx4*>(p));
  } else {
    *p = x;
  }
}

__device__ __forceinline__ float elu_plus_one(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int DK, int DV, class E, int KIND, int RPTT, bool NT, int WPE>
__global__ __launch_bounds__((DecodeShape<DK, DV, RPTT>::NTB))
__attribute__((amdgpu_waves_per_eu(WPE))) void decode_kernel(DecodeArgs a) {
  typedef DecodeShape<DK, DV, RPTT> Sh;
  typedef typename E::T T;
  constexpr int CQ = Sh::CQ, RPT = Sh::RPT, RG = Sh::RG, TPH = Sh::TPH, HPB = Sh::HPB;
  constexpr int NTB = Sh::NTB;
  constexpr bool kDecay = KIND == DEC_GATED || KIND == DEC_SGATED || KIND == DEC_GLA;
  constexpr bool kDelta = KIND == DEC_DELTA || KIND == DEC_GATED || KIND == DEC_SGATED;

  __shared__ float s_q[HPB][DK];
  __shared__ float s_k[HPB][DK];
  __shared__ float s_a[kDecay ? HPB : 1][kDecay ? DK : 1];
  __shared__ float s_z[KIND == DEC_LA ? HPB : 1][KIND == DEC_LA ? DK : 1];
  __shared__ float4 s_red0[HPB][RG][CQ];
  __shared__ float4 s_red1[HPB][RG][CQ];
  __shared__ float2 s_red2[HPB][RG][CQ];
  __shared__ float4 s_u[HPB][CQ];

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
    s[j] = ld_state<NT>(&S4[(rg + RG * j) * CQ + cq]);  // hc is clamped: always in bounds
  }

  // Stage this block's per-row vectors (q, k, decay, z) in LDS as fp32.
  const T* qg = reinterpret_cast<const T*>(a.q);
  const T* kg = reinterpret_cast<const T*>(a.k);
  for (int i = threadIdx.x; i < HPB * DK; i += NTB) {
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
    if (kDecay) {  // per key channel, or one value per head (and none: a = 1)
      const T* gg = reinterpret_cast<const T*>(a.g);
      const long gi = KIND == DEC_GATED ? hh * DK + d : hh;
      s_a[h][d] = hh < a.nheads && gg ? __expf(E::ld(gg + gi)) : 1.f;
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
    if (kDecay) {
      const float ar = s_a[hb][row];
      s[j].x *= ar; s[j].y *= ar; s[j].z *= ar; s[j].w *= ar;
    }
    if (kDelta) {
      r4.x += kr * s[j].x; r4.y += kr * s[j].y; r4.z += kr * s[j].z; r4.w += kr * s[j].w;
    }
    s4.x += qr * s[j].x; s4.y += qr * s[j].y; s4.z += qr * s[j].z; s4.w += qr * s[j].w;
    if (cq == 0) {
      sc += qr * kr;
      if (KIND == DEC_LA) sz += qr * s_z[hb][row];
    }
  }
  // Cross-row-group reduction: every thread posts its partial sums; the
  // threads of row group 0 add them up, form u and o, and hand u back to the
  // other row groups through LDS.
  s_red0[hb][rg][cq] = r4;
  s_red1[hb][rg][cq] = s4;
  s_red2[hb][rg][cq] = make_float2(sc, sz);
  __syncthreads();
  float4 u4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (rg == 0) {
    r4 = make_float4(0.f, 0.f, 0.f, 0.f);
    s4 = make_float4(0.f, 0.f, 0.f, 0.f);
    sc = 0.f;
    sz = 0.f;
#pragma unroll 4
    for (int i = 0; i < RG; ++i) {
      const float4 x = s_red0[hb][i][cq];
      const float4 y = s_red1[hb][i][cq];
      const float2 w = s_red2[hb][i][0];  // scalar sums live in the cq == 0 threads
      r4.x += x.x; r4.y += x.y; r4.z += x.z; r4.w += x.w;
      s4.x += y.x; s4.y += y.y; s4.z += y.z; s4.w += y.w;
      sc += w.x;
      sz += w.y;
    }
    if (active) {
      const T* vg = reinterpret_cast<const T*>(a.v) + hc * DV + 4 * cq;
      const float4 v4 = make_float4(E::ld(vg), E::ld(vg + 1), E::ld(vg + 2), E::ld(vg + 3));
      float4 o4;
      if (KIND == DEC_LA) {
        u4 = v4;
        const float inv = 1.f / (sz + sc);
        o4 = make_float4((s4.x + sc * v4.x) * inv, (s4.y + sc * v4.y) * inv,
                         (s4.z + sc * v4.z) * inv, (s4.w + sc * v4.w) * inv);
      } else if (KIND == DEC_GLA) {
        u4 = v4;
        o4 = make_float4(s4.x + sc * v4.x, s4.y + sc * v4.y, s4.z + sc * v4.z, s4.w + sc * v4.w);
      } else {
        const float b = E::ld(reinterpret_cast<const T*>(a.beta) + hc);
        u4 = make_float4(b * (v4.x - r4.x), b * (v4.y - r4.y), b * (v4.z - r4.z),
                         b * (v4.w - r4.w));
        o4 = make_float4(s4.x + sc * u4.x, s4.y + sc * u4.y, s4.z + sc * u4.z,
                         s4.w + sc * u4.w);
      }
      T* og = reinterpret_cast<T*>(a.o) + hc * DV + 4 * cq;
      og[0] = E::cvt(o4.x);
      og[1] = E::cvt(o4.y);
      og[2] = E::cvt(o4.z);
      og[3] = E::cvt(o4.w);
      if (RG > 1) s_u[hb][cq] = u4;
    }
  }
  if (RG > 1) {
    __syncthreads();
    u4 = s_u[hb][cq];
  }
  if (!active) return;

#pragma unroll
  for (int j = 0; j < RPT; ++j) {
    const int row = rg + RG * j;
    const float kr = s_k[hb][row];
    s[j].x += kr * u4.x; s[j].y += kr * u4.y; s[j].z += kr * u4.z; s[j].w += kr * u4.w;
    st_state<NT>(&S4[row * CQ + cq], s[j]);
  }
  if (KIND == DEC_LA && cq == 0) {
#pragma unroll
    for (int j = 0; j < RPT; ++j) {
      const int row = rg + RG * j;
      a.z[hc * DK + row] = s_z[hb][row] + s_k[hb][row];
    }
  }
}

template <int DK, int DV, class E, int KIND, int RPTT = 4, bool NT = true, int WPE = 8>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  typedef DecodeShape<DK, DV, RPTT> Sh;
  const int blocks = (a.nheads + Sh::HPB - 1) / Sh::HPB;
  hipLaunchKernelGGL((decode_kernel<DK, DV, E, KIND, RPTT, NT, WPE>), dim3(blocks), dim3(Sh::NTB), 0,
                     st, a);
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

template <class E>
static hipError_t launch_decode_kind(int kind, int dk, int dv, const DecodeArgs& a, hipStream_t st) {
  switch (kind) {
    case DEC_DELTA: return launch_decode_e<E, DEC_DELTA>(dk, dv, a, st);
    case DEC_GATED: return launch_decode_e<E, DEC_GATED>(dk, dv, a, st);
    case DEC_LA: return launch_decode_e<E, DEC_LA>(dk, dv, a, st);
    case DEC_SGATED: return launch_decode_e<E, DEC_SGATED>(dk, dv, a, st);
    case DEC_GLA: return launch_decode_e<E, DEC_GLA>(dk, dv, a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(int kind, int bf16, int dk, int dv, const DecodeArgs& a,
                         hipStream_t st) {
  return bf16 ? launch_decode_kind<BF16>(kind, dk, dv, a, st) : launch_decode_kind<F32>(kind, dk, dv, a, st);
}

}  // namespace linattn

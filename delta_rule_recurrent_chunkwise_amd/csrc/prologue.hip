// prologue.hip -- the steps just before the delta rule in the layer of the
// article "From GPT-2 to Kimi K3, explained", section "DeltaNet (Fast Weight
// Programmers)": q and k each go through silu and an L2 normalisation over
// the head dimension (x / max(|x|_2, 1e-12), torch's F.normalize), q
// optionally times a scale, and beta = sigmoid(logits), one logit per token
// shared by every head or one per head.
//
// HBM-bound elementwise and row work, so one pass that reads each row once
// and writes it once: a row of d elements is n = d * sizeof(T) / 16 lanes of
// 16-byte vectors; the sum of squares is reduced over those n lanes with
// xor shuffles.  q rows, k rows and beta are three slices of one grid (one
// launch); each thread takes NR rows (all loads first), so that enough bytes
// are in flight.  The rows are touched once, so loads and stores are
// nontemporal.
#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

template <class E>
union Vec16P {
  Vec16 v;
  typename E::T e[E::kVec];
};

constexpr int NR = 4;  // rows per thread

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// beta[b, h, t] = sigmoid(logits[b, hb ? h : 0, t]) for the block's elements
// i0 + l, l = threadIdx.x + 256 j < NB
template <class E, int NB>
__device__ __forceinline__ void beta_part(const typename E::T* __restrict__ logits, typename E::T* __restrict__ beta,
                                          long i0, int B, int Hb, int H, int T) {
  const long n = (long)B * H * T;
#pragma unroll
  for (int j = 0; j < (NB + 255) / 256; ++j) {
    const int l = threadIdx.x + 256 * j;
    const long i = i0 + l;
    if (l >= NB || i >= n) return;
    const int t = (int)(i % T);
    const long bh = i / T;
    const int h = (int)(bh % H), b = (int)(bh / H);
    const float z = E::tof(logits[((size_t)b * Hb + (Hb == 1 ? 0 : h)) * T + t]);
    beta[i] = E::cvt(1.f / (1.f + __expf(-z)));
  }
}

// blockIdx.y: 0 q rows, 1 k rows, 2 beta (blocks of RPB * NR elements)
template <int D, class E, bool SILU>
__global__ __launch_bounds__(256) void qk_prologue(const typename E::T* q_in,
                                                   const typename E::T* k_in,
                                                   typename E::T* q_out,
                                                   typename E::T* k_out, long rows, float q_scale,
                                                   const typename E::T* logits, typename E::T* beta,
                                                   int B, int Hb, int H, int T) {
  constexpr int KV = E::kVec;
  constexpr int LPR = D / KV;        // lanes per row
  constexpr int RPB = 256 / LPR;     // rows per block and step
  if (blockIdx.y == 2) {
    beta_part<E, RPB * NR>(logits, beta, (long)blockIdx.x * RPB * NR, B, Hb, H, T);
    return;
  }
  const int sub = threadIdx.x % LPR;
  const bool isq = blockIdx.y == 0;
  const typename E::T* in = isq ? q_in : k_in;
  typename E::T* out = isq ? q_out : k_out;
  const float scale = isq ? q_scale : 1.f;
  long row[NR];
  Vec16P<E> x[NR];
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    row[j] = ((long)blockIdx.x * NR + j) * RPB + threadIdx.x / LPR;
    const long rr = row[j] < rows ? row[j] : rows - 1;  // every lane loads; extra rows are not stored
    x[j].v = __builtin_bit_cast(Vec16, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(in + (size_t)rr * D + sub * KV)));
  }
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float y[KV];
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < KV; ++e) {
      const float xv = E::tof(x[j].e[e]);
      // x / (1 + e^-x) with the hardware reciprocal (about 1 ulp) in place
      // of an IEEE division, about ten instructions per element
      y[e] = SILU ? xv * __builtin_amdgcn_rcpf(1.f + __expf(-xv)) : xv;
      ss += y[e] * y[e];
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off, LPR);
    const float s = scale / fmaxf(sqrtf(ss), 1e-12f);
#pragma unroll
    for (int e = 0; e < KV; ++e) x[j].e[e] = E::cvt(y[e] * s);
    if (row[j] < rows)
      __builtin_nontemporal_store(__builtin_bit_cast(u32x4, x[j].v), reinterpret_cast<u32x4*>(out + (size_t)row[j] * D + sub * KV));
  }
}

template <int D, class E>
hipError_t launch_qk(const PrologueArgs& a, hipStream_t st) {
  constexpr int RPB = 256 / (D / E::kVec);
  const long rows = (long)a.B * a.H * a.T;  // also the number of beta elements
  const dim3 grid((unsigned)((rows + RPB * NR - 1) / (RPB * NR)), a.beta_logits ? 3 : 2);
  typedef typename E::T T;
  const T* qi = reinterpret_cast<const T*>(a.q_in);
  const T* ki = reinterpret_cast<const T*>(a.k_in);
  T* qo = reinterpret_cast<T*>(a.q_out);
  T* ko = reinterpret_cast<T*>(a.k_out);
  const T* lg = reinterpret_cast<const T*>(a.beta_logits);
  T* bo = reinterpret_cast<T*>(a.beta_out);
  if (a.silu)
    hipLaunchKernelGGL((qk_prologue<D, E, true>), grid, dim3(256), 0, st, qi, ki, qo, ko, rows, a.q_scale, lg, bo,
                       a.B, a.beta_heads, a.H, a.T);
  else
    hipLaunchKernelGGL((qk_prologue<D, E, false>), grid, dim3(256), 0, st, qi, ki, qo, ko, rows, a.q_scale, lg, bo,
                       a.B, a.beta_heads, a.H, a.T);
  return hipGetLastError();
}

template <class E>
hipError_t launch_prologue_e(const PrologueArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_qk<16, E>(a, st);
    case 32: return launch_qk<32, E>(a, st);
    case 64: return launch_qk<64, E>(a, st);
    case 128: return launch_qk<128, E>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prologue(int bf16, const PrologueArgs& a, hipStream_t st) {
  if (a.T == 0) return hipSuccess;
  return bf16 ? launch_prologue_e<BF16>(a, st) : launch_prologue_e<F32>(a, st);
}

}  // namespace linattn

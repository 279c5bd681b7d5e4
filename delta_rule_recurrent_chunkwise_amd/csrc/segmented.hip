// segmented.hip -- the delta rule over a long sequence cut into segments that
// run side by side: the sequence-parallel chunk-state scan.
//
// With the tokens fixed, one step of the rule, S <- (I - b k k^T) diag(a) S +
// b k v^T, is affine in the state, and so is any run of steps: a segment maps
// its incoming state S_in to M S_in + S_z, where M (dk x dk) is the product of
// the steps' linear parts and S_z the state the segment reaches from zero.
// Every output is affine in S_in too: o_t = o_t(S_in = 0) + S_in^T (M_t^T q_t),
// M_t the product up to token t.  (Article "From GPT-2 to Kimi K3, explained",
// section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)": each
// chunk's output is computed from the state the previous chunk leaves; the
// same argument carries the state across segments.  Sections "Gated Delta
// Net" and "KDA / Kimi Linear" for the decays.)
//
// A head's sequence of T tokens is read as P segments of Tp = T / P tokens,
// i.e. [B, H, T, d] as [B, H*P, Tp, d] (no copy), and:
//
// 1. every segment from its own start state through the library's prefill:
//    segment 0 of each head from the caller's state, the others from zero;
//    the outputs go straight to the caller's o, the final states to Sz;
// 2. every segment from the identity with v = 0 (the state is dk x dk): its
//    final state is M, its outputs the rows M_t^T q_t (oB);
// 3. seg_mfrag, seg_scan: S_in[1] = Sz[0], S_in[p+1] = M[p] S_in[p] + Sz[p], and the
//    caller's final state M[P-1] S_in[P-1] + Sz[P-1] (fp32 accumulation);
// 4. seg_fixup: o += oB S_in[p] for every segment p >= 1, one pass over o.
//
// The two passes each run B*H*P heads, so a call with few heads fills the
// GPU where one pass over the whole sequence leaves most compute units idle.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

// A workgroup barrier that orders LDS accesses only: outstanding global loads
// (the next step's operands) stay in flight across it, where __syncthreads()
// would wait for them.  Waves exchange data here through LDS alone.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Zeros for the transition pass's values, the identity as its start state,
// and (with a caller's state) the first pass's start states: segment 0 of
// every head from S0, the other segments from zero.  blockIdx.y picks the job.
__global__ __launch_bounds__(256) void seg_prepare(uint4* __restrict__ v0, size_t nv0,
                                                  float* __restrict__ M, size_t nm, int dk,
                                                  float* __restrict__ Sz, const float* __restrict__ S0,
                                                  size_t nsz, int P, size_t dkdv) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (blockIdx.y == 0) {
    for (size_t i = i0; i < nv0; i += stride) v0[i] = make_uint4(0u, 0u, 0u, 0u);
  } else if (blockIdx.y == 1) {
    const size_t dd = (size_t)dk * dk;
    for (size_t i = i0; i < nm; i += stride) {
      const size_t e = i % dd;
      M[i] = (e / dk == e % dk) ? 1.f : 0.f;
    }
  } else {
    // Sz[(bh * P + p) * dkdv + e] = p == 0 ? S0[bh * dkdv + e] : 0
    for (size_t i = i0; i < nsz; i += stride) {
      const size_t sh = i / dkdv, e = i % dkdv;
      Sz[i] = (sh % P == 0) ? S0[(sh / P) * dkdv + e] : 0.f;
    }
  }
}

// x (8 floats) -> its bf16 high part hi = bf16(x) and low part lo = bf16(x - hi)
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int e2 = 0; e2 < 4; ++e2) {
    hw[e2] = pack2(x[2 * e2], x[2 * e2 + 1]);
    lw[e2] = pack2(x[2 * e2] - __uint_as_float(hw[e2] << 16),
                   x[2 * e2 + 1] - __uint_as_float(hw[e2] & 0xffff0000u));
  }
  hi = words_to_bf16x8(hw[0], hw[1], hw[2], hw[3]);
  lo = words_to_bf16x8(lw[0], lw[1], lw[2], lw[3]);
}

// Every segment's transition M as bf16 high and low A-operand fragments:
// workgroup (sh, rt), one wave, rows 16rt .. 16rt+15 of M[sh]; lane (c, g)
// holds M[sh][16rt + c][32s + 8g + e], e = 0..7 (zero past DK), fragment
// ((sh * DK/16 + rt) * 2 + part) * K32 + s.  Done once for all segments, so
// that the scan's sequential steps only load them.
template <int DK>
__global__ __launch_bounds__(64) void seg_mfrag(const float* __restrict__ M, uint4* __restrict__ MF) {
  constexpr int K32 = (DK + 31) / 32, NRT = DK / 16;
  const size_t sh = blockIdx.x;
  const int rt = blockIdx.y, lane = threadIdx.x, c = lane & 15, g = lane >> 4;
  const float* mrow = M + (sh * DK + 16 * rt + c) * DK;
  uint4* out = MF + ((sh * NRT + rt) * 2) * K32 * 64;
#pragma unroll
  for (int s = 0; s < K32; ++s) {
    const int k0 = 32 * s + 8 * g;
    float x[8];
    if (k0 < DK) {
      const float4 a = *reinterpret_cast<const float4*>(mrow + k0);
      const float4 b = *reinterpret_cast<const float4*>(mrow + k0 + 4);
      x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
      x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
    }
    bf16x8 hi, lo;
    split8(x, hi, lo);
    out[(0 * K32 + s) * 64 + lane] = __builtin_bit_cast(uint4, hi);
    out[(1 * K32 + s) * 64 + lane] = __builtin_bit_cast(uint4, lo);
  }
}

// The scan over the segments of one head, for 16 value columns: workgroup
// (bh, n), DK / 16 waves, wave w owning rows 16w .. 16w+15 of the state.
// Each step is S_in[p+1] = M[p] S_in[p] + Sz[p] with fp32 accumulation and the
// product in three 32-deep bf16 MFMAs per k-step, M_hi S_hi + M_hi S_lo +
// M_lo S_hi (hi = bf16(x), lo = bf16(x - hi)); the dropped M_lo S_lo and the
// rounding of the low parts leave a relative error of about 2^-17 per step.
// The current S_in columns live in LDS as those high and low B-operand
// fragments: lane (c, g) of fragment (part, s) holds S_in[32s + 8g + e][16n + c].
// A wave's new rows 16w + 4g + i are elements e = 4(g % 2) + i of lane
// (c, 2(w % 2) + g / 2) of k-step w / 2, one 8-byte store per part.  The same
// fragments are the fix-up's B operands: waves w < K32 copy k-step w out.
template <int DK>
__global__ __launch_bounds__(64 * (DK / 16)) void seg_scan(const uint4* __restrict__ MF,
                                                          const float* __restrict__ Sz,
                                                          uint4* __restrict__ F,
                                                          float* __restrict__ S, int P, int dv) {
  constexpr int K32 = (DK + 31) / 32, NRT = DK / 16;
  __shared__ uint4 frag[2][K32][64];
  const int bh = blockIdx.x, n = blockIdx.y, NT = dv / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;
  const size_t seg0 = (size_t)bh * P;  // segment-head index of segment 0
  const size_t dkdv = (size_t)DK * dv;
  const int row0 = 16 * w + 4 * g, col = 16 * n + c;
  // where this lane's four new rows go in the fragments (in bf16 units)
  const int fs = w >> 1, fl = 16 * (2 * (w & 1) + (g >> 1)) + c, fe = 4 * (g & 1);
  auto put_rows = [&](float r0, float r1, float r2, float r3) {
    const uint32_t h0 = pack2(r0, r1), h1 = pack2(r2, r3);
    const uint32_t l0 = pack2(r0 - __uint_as_float(h0 << 16), r1 - __uint_as_float(h0 & 0xffff0000u));
    const uint32_t l1 = pack2(r2 - __uint_as_float(h1 << 16), r3 - __uint_as_float(h1 & 0xffff0000u));
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(&frag[0][fs][fl]) + fe) = make_uint2(h0, h1);
    *reinterpret_cast<uint2*>(reinterpret_cast<bf16_t*>(&frag[1][fs][fl]) + fe) = make_uint2(l0, l1);
  };
  if (DK < 32) {  // k-steps past DK stay zero
    for (int i = threadIdx.x; i < 2 * K32 * 64; i += 64 * NRT) (&frag[0][0][0])[i] = make_uint4(0u, 0u, 0u, 0u);
    lds_barrier();
  }
  // S_in[1]: the final state of segment 0, which started from the caller's state
  {
    const float* sz = Sz + seg0 * dkdv;
    put_rows(sz[(size_t)(row0 + 0) * dv + col], sz[(size_t)(row0 + 1) * dv + col],
             sz[(size_t)(row0 + 2) * dv + col], sz[(size_t)(row0 + 3) * dv + col]);
  }
  // step p's operands, loaded three steps ahead into a ring of three register
  // slots (slot (p + 2) % 3; the loop is unrolled by three so that slot
  // indices are static): Sz[p] rows 16w + 4g + i at column 16n + c, and M[p]'s
  // fragments for rows 16w ..  Every trip of every step issues its load (past
  // the last step it re-reads step P - 1, unused), and the first three loads
  // are made by trips of the same loop (steps -2 .. 0 only load): a path
  // without the load, or loads before the loop, made the compiler copy the
  // ring's registers at the loop's back edge, which waits for every load in
  // flight.
  constexpr int NSLOT = 3;
  floatx4 szn[NSLOT];
  uint4 mf[NSLOT][2][K32];
  auto load_step = [&](int p, auto slotc) {
    constexpr int SL = decltype(slotc)::value;
    const float* sz = Sz + (seg0 + p) * dkdv;
#pragma unroll
    for (int i = 0; i < 4; ++i) szn[SL][i] = sz[(size_t)(row0 + i) * dv + col];
    const uint4* src = MF + (((seg0 + p) * NRT + w) * 2) * K32 * 64 + lane;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int s = 0; s < K32; ++s) mf[SL][h][s] = src[(h * K32 + s) * 64];
  };
  lds_barrier();
  auto step = [&](int p, auto slotc) {
    constexpr int SL = decltype(slotc)::value;
    if (p >= 1 && p < P) {
      floatx4 acc = szn[SL], a1 = zero4(), a2 = zero4();
      bf16x8 ah[K32], al[K32];
#pragma unroll
      for (int s = 0; s < K32; ++s) {
        ah[s] = __builtin_bit_cast(bf16x8, mf[SL][0][s]);
        al[s] = __builtin_bit_cast(bf16x8, mf[SL][1][s]);
      }
      uint4* fb = F + ((size_t)bh * (P - 1) + (p - 1)) * 2 * K32 * NT * 64;
#pragma unroll
      for (int s = 0; s < K32; ++s) {
        const uint4 bhw = frag[0][s][lane], blw = frag[1][s][lane];
        if (w == s) {  // S_in[p] for the fix-up
          fb[((size_t)(0 * K32 + s) * NT + n) * 64 + lane] = bhw;
          fb[((size_t)(1 * K32 + s) * NT + n) * 64 + lane] = blw;
        }
        const bf16x8 bh8 = __builtin_bit_cast(bf16x8, bhw), bl8 = __builtin_bit_cast(bf16x8, blw);
        acc = mfma_k32(ah[s], bh8, acc);
        a1 = mfma_k32(ah[s], bl8, a1);
        a2 = mfma_k32(al[s], bh8, a2);
      }
      acc += a1 + a2;
      lds_barrier();  // every wave has read S_in[p]
      put_rows(acc[0], acc[1], acc[2], acc[3]);
      if (p == P - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i) S[((size_t)bh * DK + row0 + i) * dv + col] = acc[i];
      }
      lds_barrier();
    }
    const int q = p + NSLOT;
    load_step(q < 1 ? 1 : (q < P ? q : P - 1), slotc);
  };
  for (int p = 1 - NSLOT; p < P; p += NSLOT) {
    step(p, std::integral_constant<int, 0>{});
    step(p + 1, std::integral_constant<int, 1>{});
    step(p + 2, std::integral_constant<int, 2>{});
  }
}

// o += oB S_in[p] for segment p >= 1 of one head: workgroup (f, y) with f =
// bh * (P-1) + p - 1 covers tokens 256y .. 256y+255 of the segment, wave w
// (of 8) two 16-token tiles.  oB (bf16, exact) is the A operand; S_in enters
// as its bf16 high and low parts, two 32-deep bf16 MFMAs per k-step, so the
// product carries about 16 bits of S_in (the fp32 accumulator adds the rest).
// The fp32 result passes through LDS so that o is read and written in 16-byte
// row vectors.
constexpr int kFixWaves = 8;
constexpr int kFixRows = 32 * kFixWaves;

template <int DK, int DV>
__global__ __launch_bounds__(64 * kFixWaves) void seg_fixup(const bf16_t* __restrict__ oB,
                                                           const uint4* __restrict__ F,
                                                           bf16_t* __restrict__ o, int P, int Tp) {
  constexpr int K32 = (DK + 31) / 32, NT = DV / 16, NF = 2 * K32 * NT * 64;
  constexpr int SP = DV + 4;  // row stride of the staging tile (floats)
  // the B fragments, and after the products the output staging tile, share
  // one LDS buffer (at most 67.6 KB: two workgroups per compute unit)
  constexpr int NSTAGE = kFixWaves * 16 * SP / 4;  // in 16-byte units
  __shared__ uint4 smem[NF > NSTAGE ? NF : NSTAGE];
  uint4* sb = smem;
  float(*stage)[16][SP] = reinterpret_cast<float(*)[16][SP]>(smem);
  // one flat index (a grid's second dimension is limited to 65535 blocks),
  // segment fastest: consecutive blocks take the same rows of every segment
  // (1.3 us faster per call than a segment's row blocks in a row)
  const int nrb = (Tp + kFixRows - 1) / kFixRows;
  const int nf = (int)(gridDim.x / nrb);
  const int rb = (int)(blockIdx.x / nf), f = (int)(blockIdx.x - (unsigned)rb * nf);
  const int bh = f / (P - 1), p = f % (P - 1) + 1;
  const size_t sh = (size_t)bh * P + p;  // segment-head index
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, c = lane & 15, g = lane >> 4;

  // A operands: rows r0 + 16rt + c of oB (a row past the segment re-reads
  // the last one and is not stored); requested before the fragments are staged
  const int r0 = rb * kFixRows + 32 * w;
  bf16x8 fa[2][K32];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int row = min(r0 + 16 * rt + c, Tp - 1);
    const bf16_t* src = oB + (sh * Tp + row) * DK;
#pragma unroll
    for (int s = 0; s < K32; ++s) {
      if (32 * s + 8 * g < DK) {
        fa[rt][s] = *reinterpret_cast<const bf16x8*>(src + 32 * s + 8 * g);
      } else {
        fa[rt][s] = bf16x8{};
      }
    }
  }
  const uint4* fsrc = F + (size_t)f * NF;
  for (int i = threadIdx.x; i < NF; i += 64 * kFixWaves) sb[i] = fsrc[i];
  lds_barrier();
  floatx4 acc[2][NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    acc[0][nt] = zero4();
    acc[1][nt] = zero4();
#pragma unroll
    for (int s = 0; s < K32; ++s) {
      const bf16x8 bhi = __builtin_bit_cast(bf16x8, sb[((0 * K32 + s) * NT + nt) * 64 + lane]);
      const bf16x8 blo = __builtin_bit_cast(bf16x8, sb[((1 * K32 + s) * NT + nt) * 64 + lane]);
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        acc[rt][nt] = mfma_k32(fa[rt][s], bhi, acc[rt][nt]);
        acc[rt][nt] = mfma_k32(fa[rt][s], blo, acc[rt][nt]);
      }
    }
  }
  lds_barrier();  // every wave is done with the fragments: the buffer becomes the staging tile
  // per 16-token tile: accumulators -> LDS -> o (row vectors of 8 columns)
  constexpr int VPR = DV / 8;  // 16-byte vectors per row
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) stage[w][4 * g + i][16 * nt + c] = acc[rt][nt][i];
    lds_barrier();
#pragma unroll
    for (int j = 0; j < (16 * VPR + 63) / 64; ++j) {
      const int vv = lane + 64 * j;
      const int rr = vv / VPR, cv = vv % VPR;
      const int row = r0 + 16 * rt + rr;
      if (vv < 16 * VPR && row < Tp) {
        bf16_t* dst = o + (sh * Tp + row) * DV + 8 * cv;
        const uint4 old = *reinterpret_cast<const uint4*>(dst);
        const float4 a0 = *reinterpret_cast<const float4*>(&stage[w][rr][8 * cv]);
        const float4 a1 = *reinterpret_cast<const float4*>(&stage[w][rr][8 * cv + 4]);
        uint4 nw;
        nw.x = pack2(__uint_as_float(old.x << 16) + a0.x, __uint_as_float(old.x & 0xffff0000u) + a0.y);
        nw.y = pack2(__uint_as_float(old.y << 16) + a0.z, __uint_as_float(old.y & 0xffff0000u) + a0.w);
        nw.z = pack2(__uint_as_float(old.z << 16) + a1.x, __uint_as_float(old.z & 0xffff0000u) + a1.y);
        nw.w = pack2(__uint_as_float(old.w << 16) + a1.z, __uint_as_float(old.w & 0xffff0000u) + a1.w);
        *reinterpret_cast<uint4*>(dst) = nw;
      }
    }
    lds_barrier();
  }
}

template <int DK>
hipError_t launch_scan(const float* M, uint4* MF, const float* Sz, uint4* F, float* S, int BH, int P,
                       int dv, hipStream_t st) {
  hipLaunchKernelGGL(seg_mfrag<DK>, dim3((unsigned)BH * P, DK / 16), dim3(64), 0, st, M, MF);
  if (hipError_t e = hipGetLastError()) return e;
  hipLaunchKernelGGL(seg_scan<DK>, dim3(BH, dv / 16), dim3(64 * (DK / 16)), 0, st, MF, Sz, F, S, P, dv);
  return hipGetLastError();
}

template <int DK, int DV>
hipError_t launch_fixup_t(const bf16_t* oB, const uint4* F, bf16_t* o, int BH, int P, int Tp,
                          hipStream_t st) {
  const dim3 grid((unsigned)((long)BH * (P - 1) * ((Tp + kFixRows - 1) / kFixRows)));
  hipLaunchKernelGGL((seg_fixup<DK, DV>), grid, dim3(64 * kFixWaves), 0, st, oB, F, o, P, Tp);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_fixup(int dv, const bf16_t* oB, const uint4* F, bf16_t* o, int BH, int P, int Tp,
                        hipStream_t st) {
  switch (dv) {
    case 16: return launch_fixup_t<DK, 16>(oB, F, o, BH, P, Tp, st);
    case 32: return launch_fixup_t<DK, 32>(oB, F, o, BH, P, Tp, st);
    case 64: return launch_fixup_t<DK, 64>(oB, F, o, BH, P, Tp, st);
    case 128: return launch_fixup_t<DK, 128>(oB, F, o, BH, P, Tp, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_segmented(int mode, int dk, const PrefillArgs& a, int P, void* workspace,
                            hipStream_t st) {
  if (P < 2 || a.T % P != 0 || a.T == 0) return hipErrorInvalidValue;
  if (dk != 16 && dk != 32 && dk != 64 && dk != 128) return hipErrorInvalidValue;
  const SegmentedLayout L = segmented_layout(mode, dk, a, P);
  char* ws = static_cast<char*>(workspace);
  float* Sz = reinterpret_cast<float*>(ws + L.sz);
  float* M = reinterpret_cast<float*>(ws + L.m);
  bf16_t* oB = reinterpret_cast<bf16_t*>(ws + L.ob);
  bf16_t* v0 = reinterpret_cast<bf16_t*>(ws + L.v0);
  uint4* F = reinterpret_cast<uint4*>(ws + L.f);
  uint4* MF = reinterpret_cast<uint4*>(ws + L.mf);
  void* prep = ws + L.prep;
  const int BH = a.B * a.H, HP = a.H * P, Tp = a.T / P;
  const size_t nseg = (size_t)BH * P, dkdv = (size_t)dk * a.dv;

  // zeros, identity, start states
  {
    const size_t nv0 = nseg * Tp * dk * sizeof(bf16_t) / 16;
    const size_t nm = nseg * dk * dk;
    const size_t nsz = a.use_init ? nseg * dkdv : 0;
    hipLaunchKernelGGL(seg_prepare, dim3(1024, a.use_init ? 3 : 2), dim3(256), 0, st,
                       reinterpret_cast<uint4*>(v0), nv0, M, nm, dk, Sz, a.S, nsz, P, dkdv);
    if (hipError_t e = hipGetLastError()) return e;
  }
  // 1. every segment from its start state: outputs into the caller's o
  PrefillArgs av = a;
  av.H = HP;
  av.T = Tp;
  av.S = Sz;
  av.z = nullptr;
  av.Sc = nullptr;
  // 2. every segment's transition: from the identity, v = 0, state dk x dk
  PrefillArgs at = av;
  at.v = v0;
  at.o = oB;
  at.S = M;
  at.dv = dk;
  at.use_init = 1;
  if (mode == PF_GATED && dk == 128 && a.dv % 32 == 0) {
    // both passes on the pipelined kernel: its gate pre-pass (decay-scaled q
    // and k, which do not depend on v) runs once for the two
    if (hipError_t e = launch_gate_prep(128, av, prep, st)) return e;
    if (hipError_t e = launch_prefill_pipe_prepped(av, prep, st)) return e;
    if (hipError_t e = launch_prefill_pipe_prepped(at, prep, st)) return e;
  } else {
    if (hipError_t e = launch_prefill(mode, 1, dk, av, prep, st)) return e;
    if (hipError_t e = launch_prefill(mode, 1, dk, at, prep, st)) return e;
  }
  // 3. scan over the segments: S_in fragments and the caller's final state
  hipError_t e;
  switch (dk) {
    case 16: e = launch_scan<16>(M, MF, Sz, F, a.S, BH, P, a.dv, st); break;
    case 32: e = launch_scan<32>(M, MF, Sz, F, a.S, BH, P, a.dv, st); break;
    case 64: e = launch_scan<64>(M, MF, Sz, F, a.S, BH, P, a.dv, st); break;
    default: e = launch_scan<128>(M, MF, Sz, F, a.S, BH, P, a.dv, st); break;
  }
  if (e != hipSuccess) return e;
  // 4. o += oB S_in for segments 1 .. P-1
  bf16_t* o = static_cast<bf16_t*>(a.o);
  switch (dk) {
    case 16: return launch_fixup<16>(a.dv, oB, F, o, BH, P, Tp, st);
    case 32: return launch_fixup<32>(a.dv, oB, F, o, BH, P, Tp, st);
    case 64: return launch_fixup<64>(a.dv, oB, F, o, BH, P, Tp, st);
    default: return launch_fixup<128>(a.dv, oB, F, o, BH, P, Tp, st);
  }
}

}  // namespace linattn

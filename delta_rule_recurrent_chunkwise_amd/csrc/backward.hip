// backward.hip -- gradient of the chunkwise delta rule (ungated).
//
// The article "From GPT-2 to Kimi K3, explained" gives the chunk form of
// section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)" as
// the way to train the delta rule in linear time.  Per 64-token chunk with
// incoming state S (dk x dv), L = tril(diag(beta) K K^T, -1), T = (I + L)^-1:
//   X = diag(beta)(V - K S),  u = T X,  A = tril(Q K^T),
//   O = Q S + A u,            S' = S + K^T u.
// For the loss sum(dO * O) + sum(dS' * S') the chain rule gives, with
// dS' the gradient of the state leaving the chunk (dSn below):
//   du = A^T dO + K dSn            (O through u, and S' through u)
//   dX = T^T du                    ((I + L) u = X)
//   dL = -tril(dX u^T, -1),  dA = tril(dO u^T)
//   dV = diag(beta) dX
//   dbeta = rowsum((V - K S) * dX) + rowsum(dL * K K^T)
//   dQ = dO S^T + dA K
//   dK = dA^T Q + u dSn^T - diag(beta) dX S^T + (diag(beta) dL) K + (diag(beta) dL)^T K
//   dS = dSn + Q^T dO - K^T diag(beta) dX   (the gradient of the state entering)
//
// Passes:
//   1. the forward chunk recurrence (the pipelined kernel for bf16 with
//      dk = 128 and dv % 32 == 0, the generic one otherwise) writes the state
//      entering every chunk to a workspace, in the input type;
//   2. bf16: bwd_transition forms every chunk's P = W^T K and R = Q - A W at
//      once, and bwd_chain_mat walks the chunks backwards with
//      dS <- dS - P dS + R^T dO (see there); fp32: bwd_chain walks them with
//      the formulas above.  One workgroup per (batch, head, slice of value
//      columns) -- the columns of dS are independent, as those of S are
//      forward -- and dSn of every chunk goes to a workspace;
//   3. bwd_grads forms every chunk's dQ, dK, dV, dbeta at once, one workgroup
//      per chunk, from its S and dSn.
// Inputs and outputs have the input dtype; the products run on bf16 MFMA
// (fp32 MFMA for fp32 inputs) with fp32 accumulation, like the forward.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

constexpr int kC = 64;
constexpr int kThreads = 256;        // default staging width
constexpr int kChainThreads = 512;   // bwd_chain: 8 waves, so the products spread wider
constexpr int kGradThreads = 512;    // bwd_grads: likewise
constexpr int LTL = kC + 4;  // fp32 row stride of T and its transpose

__device__ __forceinline__ int xcd_remap_b(int bid, int n) {
  if (n % 8 != 0) return bid;
  return (bid % 8) * (n / 8) + bid / 8;
}

// Gated rule (one log-decay g per token): G_r = g_t0 + ... + g_(t0+r), the
// log-decay summed from the chunk start, r = 0..63 (rows past the end add
// nothing, so they keep G of the last row).  Called by a whole wave; lane r
// returns G_r.
template <class E>
__device__ __forceinline__ float chunk_logdecay(const typename E::T* gh, int t0, int nrow, int lane) {
  return scan64_up(lane < nrow ? E::tof(gh[t0 + lane]) : 0.f);
}
// exp(G_r - G_c) for c <= r (a decay ratio, at most 1), else 0
__device__ __forceinline__ float decay_ratio(const float* sG, int r, int c) {
  return c <= r ? __expf(sG[r] - sG[c]) : 0.f;
}

// T = (I + L)^-1 in the lower triangle (diagonal included) of sTL, from L
// stored transposed in its strictly upper triangle (sTL[c][r] = L[r][c],
// c < r).  Diagonal 16 x 16 blocks by forward substitution, one lane per
// column; then block row by block row, T[bi][bj] = -T[bi][bi] sum_m L[bi][m]
// T[m][bj].  The strictly upper triangle is cleared.  Every thread calls it.
template <bool kBf16, int NTH>
__device__ void form_T(float* sTL, int tid, int wave, int lane) {
  const int lc = lane & 15, lg = lane >> 4;
  if (wave == NTH / 64 - 1) {
    const int b0 = 16 * lg;
    float tv[16];
    // right-looking: once tv[m] is known it is folded into the partial sums of
    // every later row, so one multiply-add separates tv[m] from tv[m+1]
    float ps[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ps[i] = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      tv[m] = m < lc ? 0.f : (m == lc ? 1.f : -ps[m]);
#pragma unroll
      for (int i = m + 1; i < 16; ++i) ps[i] += sTL[(b0 + m) * LTL + b0 + i] * tv[m];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (i >= lc) sTL[(b0 + i) * LTL + b0 + lc] = tv[i];
  }
  __syncthreads();
  for (int bi = 1; bi < 4; ++bi) {
    if (wave < bi) {
      const int bj = wave;
      floatx4 R = zero4();
      for (int m = bj; m < bi; ++m) {
        float av[4], bv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int kk = 4 * lg + e;
          av[e] = sTL[(16 * m + kk) * LTL + 16 * bi + lc];
          bv[e] = (m > bj || kk >= lc) ? sTL[(16 * m + kk) * LTL + 16 * bj + lc] : 0.f;
        }
        if constexpr (kBf16) {
          R = mfma_k16(words_to_shortx4(pack2(av[0], av[1]), pack2(av[2], av[3])),
                       words_to_shortx4(pack2(bv[0], bv[1]), pack2(bv[2], bv[3])), R);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) R = mfma_f32(av[e], bv[e], R);
        }
      }
      float tv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kk = 4 * lg + e;
        tv[e] = kk <= lc ? sTL[(16 * bi + lc) * LTL + 16 * bi + kk] : 0.f;
      }
      floatx4 Y = zero4();
      if constexpr (kBf16) {
        Y = mfma_k16(words_to_shortx4(pack2(tv[0], tv[1]), pack2(tv[2], tv[3])), acc_to_b16(R), Y);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) Y = mfma_f32(tv[e], R[e], Y);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sTL[(16 * bi + 4 * lg + i) * LTL + 16 * bj + lc] = -Y[i];
    }
    __syncthreads();
  }
  for (int i = tid; i < kC * kC; i += NTH) {
    const int r = i >> 6, c = i & 63;
    if (c > r) sTL[r * LTL + c] = 0.f;
  }
  __syncthreads();
}

// acc (one 16 x 16 tile) += A[r, 0:K] B[c, 0:K]^T, both row-major in LDS
template <bool kBf16, class T>
__device__ __forceinline__ floatx4 rowrow(floatx4 acc, const T* arow, const T* brow, int K, int lane) {
  if constexpr (kBf16) return mm_rowrow_bf16(acc, arow, brow, K, lane);
  else return mm_rowrow_f32(acc, arow, brow, K, lane);
}
// acc += A[r, 0:16 nt] X, X given as nt accumulator tiles (nt even, or 1)
template <bool kBf16, class EA>
__device__ __forceinline__ floatx4 accB(floatx4 acc, const EA* arow, const floatx4* xt, int nt, int lane) {
  if constexpr (kBf16) return mm_accB_bf16(acc, arow, xt, nt, lane);
  else return mm_accB_f32(acc, reinterpret_cast<const float*>(arow), xt, nt, lane);
}

// acc += A X with A's row r (r = lane % 16 of the tile) read as column r of a
// row-major matrix M (A[r][k] = M[k][r]): col = &M[0][r], ld = M's row
// stride.  Same k order as mm_accB_bf16 / mm_accB_f32, so X is given as nt
// accumulator tiles (nt even, or 1, for bf16).  Consecutive lanes read
// consecutive addresses.
template <bool kBf16, class EM>
__device__ __forceinline__ floatx4 accB_col(floatx4 acc, const EM* col, int ld, const floatx4* xt, int nt, int lane) {
  const int g = lane >> 4;
  auto ldf = [&](int k) { return (float)(sizeof(EM) == 2 ? bf2f(*reinterpret_cast<const bf16_t*>(col + (size_t)k * ld))
                                                        : *reinterpret_cast<const float*>(col + (size_t)k * ld)); };
  if constexpr (kBf16) {
    int t = 0;
    for (; t + 1 < nt; t += 2) {
      const int k0 = 16 * t + 4 * g, k1 = 16 * t + 16 + 4 * g;
      const bf16x8 a = words_to_bf16x8(pack2(ldf(k0), ldf(k0 + 1)), pack2(ldf(k0 + 2), ldf(k0 + 3)),
                                       pack2(ldf(k1), ldf(k1 + 1)), pack2(ldf(k1 + 2), ldf(k1 + 3)));
      acc = mfma_k32(a, acc_pair_to_b(xt[t], xt[t + 1]), acc);
    }
    if (t < nt) {
      const int k0 = 16 * t + 4 * g;
      acc = mfma_k16(words_to_shortx4(pack2(ldf(k0), ldf(k0 + 1)), pack2(ldf(k0 + 2), ldf(k0 + 3))),
                     acc_to_b16(xt[t]), acc);
    }
  } else {
    for (int t = 0; t < nt; ++t) {
      const int k0 = 16 * t + 4 * g;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mfma_f32(ldf(k0 + e), xt[t][e], acc);
    }
  }
  return acc;
}

template <class E>
union Vec16U {
  Vec16 v;
  typename E::T e[E::kVec];
};

// Stage D columns of rows [t0, t0 + 64) of a row-major tensor (source row
// stride sld elements, 16-byte aligned rows) into LDS, rows past the end as
// zeros: row-major (dst[r][d], stride ld, 16-byte aligned rows) and/or
// transposed (dstT[d][r], stride ldT).  Every thread first issues all of its
// 16-byte loads (rows past the end re-read the last row), then stores.
// With a transposed copy, consecutive lanes take consecutive rows, so the
// transposed stores of one instruction are consecutive addresses (no bank
// conflicts); otherwise consecutive lanes take consecutive vectors of a row.
template <class E, int D, int NTH = kThreads>
__device__ __forceinline__ void stage_rows(const typename E::T* src, int sld, int t0, int nrow, typename E::T* dst,
                                           int ld, typename E::T* dstT, int ldT, int tid) {
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  constexpr int KV = E::kVec;
  constexpr int VPR = D / KV;  // 16-byte vectors per row
  constexpr int NV = kC * VPR;
  constexpr int NPT = (NV + NTH - 1) / NTH;
  const bool rows_fast = dstT != nullptr;
  w4 buf[NPT];  // plain vectors: a union selected per lane would go through scratch memory
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i = min(tid + NTH * j, NV - 1);
    const int r = min(rows_fast ? i % kC : i / VPR, nrow - 1);
    const int vc = rows_fast ? i / kC : i % VPR;
    buf[j] = *reinterpret_cast<const w4*>(src + (size_t)(t0 + r) * sld + vc * KV);
  }
  const w4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NPT; ++j) {
    const int i = tid + NTH * j;
    if (NV % NTH != 0 && i >= NV) continue;
    const int r = rows_fast ? i % kC : i / VPR, d = (rows_fast ? i / kC : i % VPR) * KV;
    const w4 w = r < nrow ? buf[j] : z;
    if (dst) *reinterpret_cast<w4*>(dst + r * ld + d) = w;
    if (dstT) {
      Vec16U<E> x;
      x.v = __builtin_bit_cast(Vec16, w);
#pragma unroll
      for (int e = 0; e < KV; ++e) dstT[(d + e) * ldT + r] = x.e[e];
    }
  }
}

// The same staging split in two, so that the loads of the next chunk can be
// in flight while the current one is computed: load() issues the 16-byte
// loads into registers, store() writes them to LDS.  RF: rows-fast lane
// mapping (for a transposed copy), as in stage_rows.
template <class E, int D, bool RF, int NTH>
struct RowTile {
  typedef typename E::T T;
  static constexpr int KV = E::kVec, VPR = D / KV, NV = kC * VPR, NPT = (NV + NTH - 1) / NTH;
  typedef uint32_t w4 __attribute__((ext_vector_type(4)));
  // plain vectors: an array of unions went through scratch memory, whose
  // accesses the compiler then waited for between the loads
  w4 buf[NPT];
  __device__ __forceinline__ void load(const T* src, int sld, int t0, int nrow, int tid) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i = min(tid + NTH * j, NV - 1);
      const int r = min(RF ? i % kC : i / VPR, nrow - 1);
      buf[j] = *reinterpret_cast<const w4*>(src + (size_t)(t0 + r) * sld + (RF ? i / kC : i % VPR) * KV);
    }
  }
  __device__ __forceinline__ void store(int nrow, T* dst, int ld, T* dstT, int ldT, int tid) {
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i = tid + NTH * j;
      if (NV % NTH != 0 && i >= NV) continue;
      const int r = RF ? i % kC : i / VPR, d = (RF ? i / kC : i % VPR) * KV;
      const w4 z = {0u, 0u, 0u, 0u};
      const w4 w = r < nrow ? buf[j] : z;
      if (dst) *reinterpret_cast<w4*>(dst + r * ld + d) = w;
      if (dstT) {  // elements through one local union, as in stage_rows
        Vec16U<E> x;
        x.v = __builtin_bit_cast(Vec16, w);
#pragma unroll
        for (int e = 0; e < KV; ++e) dstT[(d + e) * ldT + r] = x.e[e];
      }
    }
  }
};

// ---------------------------------------------------------------------------
// Pass 2: the reverse chain.  One workgroup per (batch, head, DVS value
// columns); NCW = DVS / 16 chain waves hold dS[:, 16 columns] as accumulator
// tiles.  Per chunk (last to first): write dSn, stage Q, K, dO, beta; the
// other waves form tril(Q K^T) and L; all form T; the chain forms
// du = A^T dO + K dSn, dX = T^T du (A and T read by columns) and
// dS = dSn + Q^T dO - K^T diag(beta) dX.
// ---------------------------------------------------------------------------
template <int DK, class E, int DVS>
struct ChainLayout {
  typedef typename E::T T;
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int LQ = DK + PAD;   // rows of Q, K
  static constexpr int LKT = kC + PAD;  // rows of Q^T, K^T, dO^T, A
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kC * LQ * (int)sizeof(T);
  static constexpr int oQt = oK + kC * LQ * (int)sizeof(T);
  static constexpr int oKt = oQt + DK * LKT * (int)sizeof(T);
  static constexpr int oDOt = oKt + DK * LKT * (int)sizeof(T);
  static constexpr int oAt = oDOt + DVS * LKT * (int)sizeof(T);
  static constexpr int oTL = oAt + kC * LKT * (int)sizeof(T);
  static constexpr int oB = oTL + kC * LTL * 4;
  static constexpr int oG = oB + kC * 4;  // gated: G_r
  static constexpr int total = oG + kC * 4;
};

// GATE (one log-decay per token, G_r summed from the chunk start, decay
// ratios exp(G_r - G_c) in A and L):
//   du = A^T dO + diag(exp(G_C - G)) K dSn,
//   dS = exp(G_C) dSn + Q^T diag(exp(G)) dO - K^T diag(beta exp(G)) dX.
template <int DK, class E, int DVS, bool GATE>
__global__ __launch_bounds__(kChainThreads) void bwd_chain(BackwardArgs a, float* __restrict__ dSc) {
  constexpr int NTH = kChainThreads, NW = NTH / 64;
  typedef ChainLayout<DK, E, DVS> L;
  typedef typename E::T T;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int NCW = DVS / 16, NKT = DK / 16;
  constexpr int LQ = L::LQ, LKT = L::LKT;
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sQt = reinterpret_cast<T*>(smem + L::oQt);
  T* sKt = reinterpret_cast<T*>(smem + L::oKt);
  T* sDOt = reinterpret_cast<T*>(smem + L::oDOt);
  T* sA = reinterpret_cast<T*>(smem + L::oAt);  // tril(Q K^T), row-major
  float* sTL = reinterpret_cast<float*>(smem + L::oTL);
  float* sB = reinterpret_cast<float*>(smem + L::oB);
  float* sG = reinterpret_cast<float*>(smem + L::oG);

  const int dv = a.dv_;
  const int nsl = dv / DVS;
  const int w = xcd_remap_b(blockIdx.x, gridDim.x);
  const int bh = w / nsl, sl = w - bh * nsl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int Tn = a.T, nch = (Tn + kC - 1) / kC;
  const T* qh = reinterpret_cast<const T*>(a.q) + (size_t)bh * Tn * DK;
  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)bh * Tn * DK;
  const T* doh = reinterpret_cast<const T*>(a.dO) + (size_t)bh * Tn * dv + sl * DVS;
  const T* bth = reinterpret_cast<const T*>(a.beta) + (size_t)bh * Tn;
  const bool chain = wave < NCW;
  const int col = sl * DVS + 16 * wave + lc;  // value column of a chain lane

  floatx4 st[NKT];  // dS[:, 16 columns] of a chain wave
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    st[kt] = zero4();
    if (chain && a.dST) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[kt][i] = a.dST[((size_t)bh * DK + 16 * kt + 4 * lg + i) * dv + col];
    }
  }

  // chunk c's Q, K, dO slice and beta are loaded into registers while chunk
  // c + 1 is computed
  RowTile<E, DK, true, NTH> pq, pk;
  RowTile<E, DVS, true, NTH> pdo;
  float pb = 0.f;
  auto prefetch = [&](int cc) {
    const int t0 = cc * kC, nrow = min(kC, Tn - t0);
    pq.load(qh, DK, t0, nrow, tid);
    pk.load(kh, DK, t0, nrow, tid);
    pdo.load(doh, dv, t0, nrow, tid);
    if (tid < kC) pb = E::tof(bth[t0 + min(tid, nrow - 1)]);
  };
  prefetch(nch - 1);
  for (int c = nch - 1; c >= 0; --c) {
    const int t0 = c * kC, nrow = min(kC, Tn - t0);
    if (chain) {  // dSn of chunk c
      float* out = dSc + ((size_t)bh * nch + c) * DK * dv;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) out[(size_t)(16 * kt + 4 * lg + i) * dv + col] = st[kt][i];
    }
    __syncthreads();  // the previous chunk's readers are done
    pq.store(nrow, sQ, LQ, sQt, LKT, tid);
    pk.store(nrow, sK, LQ, sKt, LKT, tid);
    pdo.store(nrow, nullptr, 0, sDOt, LKT, tid);  // the dO slice, transposed
    if (tid < kC) sB[tid] = tid < nrow ? pb : 0.f;
    if constexpr (GATE) {
      if (wave == 0) sG[lane] = chunk_logdecay<E>(reinterpret_cast<const T*>(a.g) + (size_t)bh * Tn, t0, nrow, lane);
    }
    prefetch(c > 0 ? c - 1 : 0);  // issued on every trip (the last one re-reads chunk 0)
    __syncthreads();

    floatx4 kds[4];
    if (chain) {  // K dSn while the other waves form the products
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        kds[mt] = accB<kBf16>(zero4(), sK + (16 * mt + lc) * LQ, st, NKT, lane);
        if constexpr (GATE) {
#pragma unroll
          for (int i = 0; i < 4; ++i) kds[mt][i] *= __expf(sG[63] - sG[16 * mt + 4 * lg + i]);
        }
      }
    } else {
      // jobs 0..9: tiles (i, j <= i) of tril(Q K^T); jobs 10..19: the same
      // tiles of K K^T -> L (strictly lower, rows scaled by beta), stored
      // transposed in T's upper triangle
      for (int jb = wave - NCW; jb < 20; jb += NW - NCW) {
        const bool isA = jb < 10;
        const int t = isA ? jb : jb - 10;
        const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        const int tj = t - ti * (ti + 1) / 2;
        floatx4 acc =
            rowrow<kBf16>(zero4(), (isA ? sQ : sK) + (16 * ti + lc) * LQ, sK + (16 * tj + lc) * LQ, DK, lane);
        const int cc = 16 * tj + lc;
        if constexpr (GATE) {
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[i] *= decay_ratio(sG, 16 * ti + 4 * lg + i, cc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * lg + i;
          if (isA) sA[r * LKT + cc] = E::cvt(cc <= r ? acc[i] : 0.f);
          else if (cc < r) sTL[cc * LTL + r] = sB[r] * acc[i];
        }
      }
      // tiles above the diagonal (ti < tj) are never written: zero them
      for (int i = tid - 64 * NCW; i >= 0 && i < kC * kC; i += NTH - 64 * NCW) {
        const int r = i >> 6, cc = i & 63;
        if ((cc >> 4) > (r >> 4)) sA[r * LKT + cc] = E::cvt(0.f);
      }
    }
    __syncthreads();
    form_T<kBf16, NTH>(sTL, tid, wave, lane);
    if (chain) {
      floatx4 dOt[4], du[4], dx[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {  // dO tiles over tokens: lane holds rows 16t + 4lg + i
        const T* p = sDOt + (16 * wave + lc) * LKT + 16 * t + 4 * lg;
#pragma unroll
        for (int i = 0; i < 4; ++i) dOt[t][i] = E::tof(p[i]);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)  // a fresh accumulator: K dSn may come from the 16-deep opcode
        du[mt] = kds[mt] + accB_col<kBf16>(zero4(), sA + 16 * mt + lc, LKT, dOt, 4, lane);  // A^T dO
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        dx[mt] = accB_col<kBf16>(zero4(), sTL + 16 * mt + lc, LTL, du, 4, lane);  // T^T du
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // -diag(beta) dX (gated: times exp(G_r))
          const int r = 16 * mt + 4 * lg + i;
          dx[mt][i] *= GATE ? -sB[r] * __expf(sG[r]) : -sB[r];
        }
      }
      floatx4 dOg[4];  // diag(exp(G)) dO
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) dOg[t][i] = GATE ? dOt[t][i] * __expf(sG[16 * t + 4 * lg + i]) : dOt[t][i];
      const float gc = GATE ? __expf(sG[63]) : 1.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        floatx4 g1 = accB<kBf16>(zero4(), sQt + (16 * kt + lc) * LKT, dOg, 4, lane);
        floatx4 g2 = accB<kBf16>(zero4(), sKt + (16 * kt + lc) * LKT, dx, 4, lane);
        st[kt] = gc * st[kt] + g1 + g2;
      }
    }
  }
  if (chain && a.dS0) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) a.dS0[((size_t)bh * DK + 16 * kt + 4 * lg + i) * dv + col] = st[kt][i];
  }
}

// ---------------------------------------------------------------------------
// bf16: the reverse chain as one product per chunk.  With W = T diag(beta) K,
// i.e. (I + L) W = diag(beta) K, the gradient of the state entering a chunk
// is
//   dS = dSn + Q^T dO - W^T (A^T dO + K dSn) = dSn - P dSn + R^T dO,
//   P = W^T K (dk x dk),  R = Q - A W (64 x dk),
// and P, R depend on the chunk's inputs only.  bwd_transition forms them for
// every chunk at once; bwd_chain_mat walks the chunks backwards with
// dS <- dS - P dS + R^T dO, one barrier per chunk.
// ---------------------------------------------------------------------------
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ bf16x8 ld_frag(const bf16_t* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ __forceinline__ shortx4 ld_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4*)((__attribute__((address_space(3))) bf16_t*)(p)));
}
__device__ __forceinline__ bf16x8 cat_tr(shortx4 lo, shortx4 hi) {
  typedef short shortx8_t __attribute__((ext_vector_type(8)));
  const shortx8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}
// Operand of a 32-deep product over tokens t0 .. t0 + 31, read with the LDS
// transpose read from a row-major (token x column) bf16 tile: lane (lc, G)
// receives column c0 + lc of tokens t0 + 4G + e and t0 + 16 + 4G + e,
// e = 0..3 (lane 16G + 4a + b receives element b of the 8-byte runs addressed
// by lanes 16G + a + 4e).  As an A operand its rows are columns c0 .. c0+15;
// as a B operand, its columns.
__device__ __forceinline__ bf16x8 tok_frag(const bf16_t* tile, int ld, int t0, int c0, int lane) {
  const int trow = 4 * (lane >> 4) + ((lane >> 2) & 3), tcol = 4 * (lane & 3);
  return cat_tr(ld_tr(tile + (t0 + trow) * ld + c0 + tcol), ld_tr(tile + (t0 + 16 + trow) * ld + c0 + tcol));
}
// The token order of tok_frag as a column permutation, for tiles read with
// plain 16-byte fragment reads against it: token 32b + 16h + 4g + i is kept
// in column 32b + 8g + 4h + i.
__device__ __forceinline__ int tperm(int x) {
  return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ void st4_bf16(bf16_t* p, float a0, float a1, float a2, float a3) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack2(a0, a1), pack2(a2, a3));
}

// Per-key-channel gate (KDA): the gate pre-pass's tiles (Q~ = Gam Q,
// K~ = Gam K, K^ = K / Gam, bf16 [chunk][64][dk]; Gam_C fp32 [chunk][dk], -1
// for a chunk walked token by token, whose tiles hold the raw q, k, g).
struct KdaPtrs {
  const bf16_t* qt;
  const bf16_t* kt;
  const bf16_t* kht;
  const float* gc;
};

template <int DK, bool KDA = false>
struct TransLayout {
  static constexpr int LQ = DK + 16;  // rows of Q, K
  static constexpr int LT = kC + 16;  // rows of A and W^T (token columns permuted by tperm)
  static constexpr int LD = 20;       // fp32 rows of a diagonal block of L
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kC * LQ * 2;
  static constexpr int oKh = oK + kC * LQ * 2;                  // KDA: K^ (and, walked, g)
  static constexpr int oA = oKh + (KDA ? kC * LQ * 2 : 0);
  static constexpr int oWt = oA + kC * LT * 2;
  static constexpr int oLo = oWt + DK * LT * 2;   // L_bj, b > j: bf16 [6][16][16], row-major
  static constexpr int oD = oLo + 6 * 256 * 2;    // D_b = (I + L_bb)^-1: bf16 [4][16][16]
  static constexpr int oLd = oD + 4 * 256 * 2;    // L_bb: fp32 [4][16][LD], strictly lower
  static constexpr int oB = oLd + 4 * 16 * LD * 4;
  static constexpr int oG = oB + kC * 4;          // gated: G_r (fp32)
  static constexpr int total = oG + kC * 4;
};

constexpr int kTransThreads = 512;

// One workgroup (8 waves) per (batch, head, chunk): P = W^T K and R = Q - A W.
//   1. stage Q, K, beta;
//   2. tril(Q K^T) -> A (bf16, token columns permuted) and the blocks of
//      L = tril(diag(beta) K K^T, -1): off the diagonal in bf16, on it fp32;
//   3. D_b = (I + L_bb)^-1 (one lane per block column, fp32);
//   4. W by block forward substitution, W_b = D_b (beta K_b - sum_{j<b} L_bj W_j),
//      one wave per 16-column tile of W, stored as W^T (token columns permuted);
//   5. P and R^T (token columns permuted) to global memory, in the order the
//      chain's MFMA fragments are read: P as [dk/16][dk/32][64 lanes][8],
//      fragment (w, kb), lane (lc, lg) = P[16w + lc][32kb + 8lg .. +7]
//      (dk = 16: [1][64][4], P[lc][4lg .. +3]); R^T as [dk/16][2][64][8]
//      likewise.  A wave's store of one tile then covers 512 contiguous bytes.
// GATE (one log-decay per token, G_r summed from the chunk start): A and L
// take the decay ratios exp(G_r - G_c), W solves (I + L) W = diag(beta
// exp(G)) K, P = W^T diag(exp(G_C - G)) K and R = diag(exp(G)) Q - A W, and
// exp(G_C) of the chunk goes to gC; the chain then takes
// dS <- exp(G_C) dS - P dS + R^T dO.
// KDA (a decay per key channel; the tiles of the gate pre-pass): A =
// tril(Q~ K^^T), L = tril(diag(beta) K~ K^^T, -1), W solves (I + L) W =
// diag(beta) K~, P = W^T (K^ diag(Gam_C)) and R = Q~ - A W; the chain takes
// dS <- diag(Gam_C) dS - P dS + R^T dO.  A chunk walked token by token gets
// its transition from the recurrence itself: X <- (I - beta k k^T) diag(a) X
// from X = I over its tokens (the delta rule with v = 0 and the identity as
// the state), R_t = q_t^T X_t and P = -X^T, and its Gam_C marker makes the
// chain use 0 for the decay, so that the chain's step is dS <- X^T dS + R^T dO
// (with P = I - X^T and a decay of 1, dS - P dS would leave the bf16
// rounding of the operand dS behind where X is small).
template <int DK, bool GATE, bool KDA = false>
__global__ __launch_bounds__(kTransThreads) void bwd_transition(BackwardArgs a, bf16_t* __restrict__ Pg,
                                                                bf16_t* __restrict__ Rg, float* __restrict__ gC,
                                                                KdaPtrs kp = KdaPtrs{}) {
  static_assert(!(GATE && KDA), "one gate kind at a time");
  typedef TransLayout<DK, KDA> LY;
  constexpr int NTH = kTransThreads, NW = NTH / 64, LQ = LY::LQ, LT = LY::LT, LD = LY::LD, NT = DK / 16;
  __shared__ __attribute__((aligned(16))) char smem[LY::total];
  bf16_t* sQ = reinterpret_cast<bf16_t*>(smem + LY::oQ);
  bf16_t* sK = reinterpret_cast<bf16_t*>(smem + LY::oK);
  bf16_t* sKh = reinterpret_cast<bf16_t*>(smem + LY::oKh);
  bf16_t* sA = reinterpret_cast<bf16_t*>(smem + LY::oA);
  bf16_t* sWt = reinterpret_cast<bf16_t*>(smem + LY::oWt);
  bf16_t* sLo = reinterpret_cast<bf16_t*>(smem + LY::oLo);
  bf16_t* sD = reinterpret_cast<bf16_t*>(smem + LY::oD);
  float* sLd = reinterpret_cast<float*>(smem + LY::oLd);
  float* sB = reinterpret_cast<float*>(smem + LY::oB);
  float* sG = reinterpret_cast<float*>(smem + LY::oG);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int Tn = a.T, nch = (Tn + kC - 1) / kC;
  const size_t chunk = blockIdx.x;
  const int bh = (int)(chunk / nch), c = (int)(chunk - (size_t)bh * nch);
  const int t0 = c * kC, nrow = min(kC, Tn - t0);
  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q) + (size_t)bh * Tn * DK;
  const bf16_t* kh = reinterpret_cast<const bf16_t*>(a.k) + (size_t)bh * Tn * DK;
  const bf16_t* bth = reinterpret_cast<const bf16_t*>(a.beta) + (size_t)bh * Tn;

  // 1. staging (rows past the end as zeros); A starts cleared, as its tiles
  // above the diagonal are read as zeros.  KDA: Q~, K~, K^ from the gate
  // pre-pass (64 rows per chunk, zero past the end).
  constexpr int NV = kC * DK / 8, VPT = (NV + NTH - 1) / NTH;
  u32x4 bq[VPT], bk[VPT], bkh[KDA ? VPT : 1];
  const bool walked = KDA && kp.gc[chunk * DK] < 0.f;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = min(tid + NTH * j, NV - 1);
    if constexpr (KDA) {
      const size_t off = chunk * kC * DK + (size_t)v * 8;
      bq[j] = *reinterpret_cast<const u32x4*>(kp.qt + off);
      bk[j] = *reinterpret_cast<const u32x4*>(kp.kt + off);
      bkh[j] = *reinterpret_cast<const u32x4*>(kp.kht + off);
    } else {
      const size_t off = (size_t)(t0 + min(v / (DK / 8), nrow - 1)) * DK + (v % (DK / 8)) * 8;
      bq[j] = *reinterpret_cast<const u32x4*>(qh + off);
      bk[j] = *reinterpret_cast<const u32x4*>(kh + off);
    }
  }
  const float bt = bf2f(bth[t0 + min(tid & 63, nrow - 1)]);
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  for (int i = tid; i < kC * LT / 8; i += NTH) reinterpret_cast<u32x4*>(sA)[i] = z4;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    const int v = tid + NTH * j;
    if (NV % NTH != 0 && v >= NV) continue;
    const int r = v / (DK / 8), c8 = (v % (DK / 8)) * 8;
    *reinterpret_cast<u32x4*>(sQ + r * LQ + c8) = r < nrow ? bq[j] : z4;
    *reinterpret_cast<u32x4*>(sK + r * LQ + c8) = r < nrow ? bk[j] : z4;
    if constexpr (KDA) *reinterpret_cast<u32x4*>(sKh + r * LQ + c8) = r < nrow ? bkh[j] : z4;
  }
  if (tid < kC) sB[tid] = tid < nrow ? bt : 0.f;
  if constexpr (GATE) {
    if (wave == 0) {
      const float G = chunk_logdecay<BF16>(reinterpret_cast<const bf16_t*>(a.g) + (size_t)bh * Tn, t0, nrow, lane);
      sG[lane] = G;
      if (lane == 63) gC[chunk] = __expf(G);
    }
  }
  __syncthreads();
  const size_t cb = (size_t)bh * nch + c;
  bf16_t* Pc = Pg + cb * DK * DK;
  bf16_t* Rc = Rg + cb * DK * kC;
  if constexpr (KDA) {
    if (walked) {  // uniform over the workgroup: the transition by the recurrence
      bf16_t* sR = sA;  // R, rows of LQ, where A and W^T would be
      if (wave < NT) {
        const int col = 16 * wave + lc;
        float x[NT][4];  // X[16 t + 4 lg + i][col]
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[t][i] = 16 * t + 4 * lg + i == col ? 1.f : 0.f;
        for (int tau = 0; tau < kC; ++tau) {
          float kk[NT][4], qq[NT][4];
          float r = 0.f;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const int o = tau * LQ + 16 * t + 4 * lg;
            const uint2 kw = *reinterpret_cast<const uint2*>(sK + o);
            const uint2 qw = *reinterpret_cast<const uint2*>(sQ + o);
            const uint2 gw = *reinterpret_cast<const uint2*>(sKh + o);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const uint32_t kx = i < 2 ? kw.x : kw.y, qx = i < 2 ? qw.x : qw.y, gx = i < 2 ? gw.x : gw.y;
              const int sh = (i & 1) * 16;
              kk[t][i] = bf2f((bf16_t)(kx >> sh));
              qq[t][i] = bf2f((bf16_t)(qx >> sh));
              x[t][i] *= __expf(bf2f((bf16_t)(gx >> sh)));
              r += kk[t][i] * x[t][i];
            }
          }
          r = xsum32(xsum16(r));
          const float u = -sB[tau] * r;  // v = 0
          float o = 0.f;
#pragma unroll
          for (int t = 0; t < NT; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[t][i] += kk[t][i] * u;
              o += qq[t][i] * x[t][i];
            }
          o = xsum32(xsum16(o));
          if (lg == 0) sR[tau * LQ + col] = f2bf(o);
        }
        // P = -X^T: lane (column col of X) writes row col of P, in the
        // fragment order of the product path below
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          float pv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pv[i] = -x[t][i];
          const size_t o = DK == 16 ? ((size_t)lc + 16 * lg) * 4
                                    : (((size_t)wave * (DK / 32) + (t >> 1)) * 64 + lc + 16 * (2 * (t & 1) + (lg >> 1))) * 8 +
                                          4 * (lg & 1);
          st4_bf16(Pc + o, pv[0], pv[1], pv[2], pv[3]);
        }
      }
      __syncthreads();
      for (int jb = wave; jb < 4 * NT; jb += NW) {  // R^T, as below
        const int rt = jb / NT, dt = jb - rt * NT;
        float rv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) rv[i] = bf2f(sR[(16 * rt + 4 * lg + i) * LQ + 16 * dt + lc]);
        st4_bf16(Rc + (((size_t)dt * 2 + (rt >> 1)) * 64 + lc + 16 * lg) * 8 + 4 * (rt & 1), rv[0], rv[1], rv[2], rv[3]);
      }
      return;
    }
  }

  // 2. jobs 0..9: tiles (ti >= tj) of tril(Q K^T); 10..19: of L.  The
  // transposed products, so that a lane holds row 16 ti + lc and the four
  // consecutive columns 16 tj + 4 lg + i.
  for (int jb = wave; jb < 20; jb += NW) {
    const bool isA = jb < 10;
    const int t = isA ? jb : jb - 10;
    const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int tj = t - ti * (ti + 1) / 2;
    floatx4 acc = mm_rowrow_bf16(zero4(), (KDA ? sKh : sK) + (16 * tj + lc) * LQ, (isA ? sQ : sK) + (16 * ti + lc) * LQ,
                                 DK, lane);
    const int r = 16 * ti + lc, c0 = 16 * tj + 4 * lg;
    if constexpr (GATE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= decay_ratio(sG, r, c0 + i);
    }
    if (isA) {
      st4_bf16(sA + r * LT + tperm(c0), c0 <= r ? acc[0] : 0.f, c0 + 1 <= r ? acc[1] : 0.f,
               c0 + 2 <= r ? acc[2] : 0.f, c0 + 3 <= r ? acc[3] : 0.f);
    } else {
      const float br = sB[r];
      if (ti == tj) {
        float4 v;
        v.x = c0 < r ? br * acc[0] : 0.f;
        v.y = c0 + 1 < r ? br * acc[1] : 0.f;
        v.z = c0 + 2 < r ? br * acc[2] : 0.f;
        v.w = c0 + 3 < r ? br * acc[3] : 0.f;
        *reinterpret_cast<float4*>(sLd + (16 * ti + lc) * LD + 4 * lg) = v;
      } else {
        st4_bf16(sLo + ((ti * (ti - 1) / 2 + tj) * 16 + lc) * 16 + 4 * lg, br * acc[0], br * acc[1], br * acc[2],
                 br * acc[3]);
      }
    }
  }
  __syncthreads();

  // 3. D_b: lane (block lg, column lc) solves (I + L_bb) x = e_lc
  // (right-looking: once x_m is known it is folded into the partial sums of
  // every later row, so one multiply-add separates x_m from x_{m+1})
  if (wave == 0) {
    const float* lb = sLd + 16 * lg * LD;
    float x[16], ps[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) ps[i] = 0.f;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      x[m] = m < lc ? 0.f : (m == lc ? 1.f : -ps[m]);
#pragma unroll
      for (int i = m + 1; i < 16; ++i) ps[i] += lb[i * LD + m] * x[m];
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) sD[(16 * lg + i) * 16 + lc] = f2bf(x[i]);
  }
  __syncthreads();

  // 4. W, one wave per 16-column tile (k16 products of 16 x 16 blocks; the B
  // operands are accumulator tiles)
  if (wave < NT) {
    const int dt = wave;
    auto blk = [&](const bf16_t* b) { return *reinterpret_cast<const shortx4*>(b + lc * 16 + 4 * lg); };
    floatx4 xb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * b + 4 * lg + i;
        xb[b][i] = sB[r] * bf2f(sK[r * LQ + 16 * dt + lc]);
        if constexpr (GATE) xb[b][i] *= __expf(sG[r]);
      }
    floatx4 w[4];
    w[0] = mfma_k16(blk(sD), acc_to_b16(xb[0]), zero4());
    const shortx4 w0 = acc_to_b16(w[0]);
    w[1] = mfma_k16(blk(sD + 256), acc_to_b16(xb[1] - mfma_k16(blk(sLo), w0, zero4())), zero4());
    const shortx4 w1 = acc_to_b16(w[1]);
    w[2] = mfma_k16(blk(sD + 512),
                    acc_to_b16(xb[2] - mfma_k16(blk(sLo + 512), w1, mfma_k16(blk(sLo + 256), w0, zero4()))), zero4());
    const shortx4 w2 = acc_to_b16(w[2]);
    w[3] = mfma_k16(blk(sD + 768),
                    acc_to_b16(xb[3] - mfma_k16(blk(sLo + 1280), w2,
                                                mfma_k16(blk(sLo + 1024), w1, mfma_k16(blk(sLo + 768), w0, zero4())))),
                    zero4());
#pragma unroll
    for (int b = 0; b < 4; ++b)
      st4_bf16(sWt + (16 * dt + lc) * LT + tperm(16 * b + 4 * lg), w[b][0], w[b][1], w[b][2], w[b][3]);
  }
  __syncthreads();
  if constexpr (GATE) {  // K's rows times exp(G_C - G_r): P's operand
    constexpr int NKV = kC * DK / 8;
    for (int v = tid; v < NKV; v += NTH) {
      const int r = v / (DK / 8), c8 = (v % (DK / 8)) * 8;
      u32x4* p = reinterpret_cast<u32x4*>(sK + r * LQ + c8);
      const u32x4 x = *p;
      const float f = __expf(sG[63] - sG[r]);
      u32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e) y[e] = pack2(f * __uint_as_float(x[e] << 16), f * __uint_as_float(x[e] & 0xffff0000u));
      *p = y;
    }
    __syncthreads();
  }
  if constexpr (KDA) {  // K^ diag(Gam_C): P's operand
    constexpr int NKV = kC * DK / 8;
    const float* gcc = kp.gc + chunk * DK;
    for (int v = tid; v < NKV; v += NTH) {
      const int r = v / (DK / 8), c8 = (v % (DK / 8)) * 8;
      u32x4* p = reinterpret_cast<u32x4*>(sKh + r * LQ + c8);
      const u32x4 x = *p;
      u32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = pack2(gcc[c8 + 2 * e] * __uint_as_float(x[e] << 16), gcc[c8 + 2 * e + 1] * __uint_as_float(x[e] & 0xffff0000u));
      *p = y;
    }
    __syncthreads();
  }

  // 5. P (from P^T = K^T W: lane holds P[16 dt + lc][16 et + 4 lg + i]) and
  // R = Q - A W (lane holds R[16 rt + 4 lg + i][16 dt + lc]); A's row block rt
  // reaches tokens <= 16 rt + 15 only
  constexpr int NPJ = NT * NT, NRJ = 4 * NT;
  for (int jb = wave; jb < NPJ + NRJ; jb += NW) {
    if (jb < NPJ) {
      const int et = jb / NT, dt = jb - et * NT;
      floatx4 acc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        acc = mfma_k32(tok_frag(KDA ? sKh : sK, LQ, 32 * kb, 16 * et, lane),
                       ld_frag(sWt + (16 * dt + lc) * LT + 32 * kb + 8 * lg), acc);
      // P[16 dt + lc][16 et + 4 lg .. +3]: fragment (dt, et / 2), lane
      // lc + 16 (2 (et % 2) + lg / 2), half lg % 2
      const size_t o = DK == 16 ? ((size_t)dt * 64 + lc + 16 * lg) * 4
                                : (((size_t)dt * (DK / 32) + (et >> 1)) * 64 + lc + 16 * (2 * (et & 1) + (lg >> 1))) * 8 +
                                      4 * (lg & 1);
      st4_bf16(Pc + o, acc[0], acc[1], acc[2], acc[3]);
    } else {
      const int t = jb - NPJ, rt = t / NT, dt = t - rt * NT;
      floatx4 acc = zero4();
      for (int kb = 0; kb <= (rt >> 1); ++kb)
        acc = mfma_k32(ld_frag(sA + (16 * rt + lc) * LT + 32 * kb + 8 * lg),
                       ld_frag(sWt + (16 * dt + lc) * LT + 32 * kb + 8 * lg), acc);
      float rv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * rt + 4 * lg + i;
        rv[i] = bf2f(sQ[r * LQ + 16 * dt + lc]) * (GATE ? __expf(sG[r]) : 1.f) - acc[i];
      }
      // R^T[16 dt + lc][tperm(16 rt + 4 lg) .. +3]: fragment (dt, rt / 2),
      // lane lc + 16 lg, half rt % 2
      st4_bf16(Rc + (((size_t)dt * 2 + (rt >> 1)) * 64 + lc + 16 * lg) * 8 + 4 * (rt & 1), rv[0], rv[1], rv[2], rv[3]);
    }
  }
}

// One workgroup per (batch, head, DVS value columns), DK / 16 waves: wave w
// keeps dS rows 16w .. 16w + 15 of the slice as DVS / 16 accumulator tiles.
// Per chunk (last to first): write dSn for the gradient pass (bf16, the
// precision that pass reads it in, in accumulator-tile order: tile (kt, jt)
// of chunk c at ((c * dk/16 + kt) * dv/16 + jt) * 256, lane l's four rows
// at 4l), then
// dS <- dS - P dS + R^T dO with the fragments of P and R^T loaded straight
// into registers (NS chunks ahead; bwd_transition stores them in fragment
// order, so a wave's load is 1 KB contiguous) and dS^T, the dO slice read
// from LDS (double buffered, one barrier per chunk).
// GATE: dS <- exp(G_C) dS - P dS + R^T dO, exp(G_C) of each chunk from gC.
// KDA: dS <- diag(Gam_C) dS - P dS + R^T dO, Gam_C per key channel from gC
// ([chunk][dk]; the marker -1 of a chunk walked token by token stands for 0,
// its P being minus the transposed transition).
template <int DK, int DVS, bool GATE, bool KDA = false>
__global__ __launch_bounds__(DK * 4) void bwd_chain_mat(BackwardArgs a, const bf16_t* __restrict__ Pg,
                                                        const bf16_t* __restrict__ Rg, bf16_t* __restrict__ dSt,
                                                        const float* __restrict__ gC) {
  constexpr int NTH = DK * 4, NJ = DVS / 16, LDT = DK + 16, LVO = DVS + 16, NS = 4;  // NS: chunks in flight (the prologue issues four)
  constexpr int KP = DK >= 32 ? DK / 32 : 1;
  constexpr int NVO = kC * DVS / 8, VPT = (NVO + NTH - 1) / NTH;
  __shared__ __attribute__((aligned(16))) bf16_t sDt[2][DVS][LDT];
  __shared__ __attribute__((aligned(16))) bf16_t sDO[2][kC][LVO];
  const int dv = a.dv_, nsl = dv / DVS;
  const int wid = xcd_remap_b(blockIdx.x, gridDim.x);
  const int bh = wid / nsl, sl = wid - bh * nsl;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const int Tn = a.T, nch = (Tn + kC - 1) / kC;
  const bf16_t* doh = reinterpret_cast<const bf16_t*>(a.dO) + (size_t)bh * Tn * dv + sl * DVS;

  // register slots of NS chunks: P fragments, R^T fragments, the dO slice;
  // every lane issues every load (clamped to valid rows and chunks), and
  // slots are indexed at compile time only
  u32x4 sp[NS][KP], sr[NS][2], so[NS][VPT];
  float sgc[NS];
  floatx4 sgk[KDA ? NS : 1];  // KDA: Gam_C of this wave's four rows
  auto issue = [&](int x, auto slotc) {
    constexpr int S = decltype(slotc)::value;
    const size_t cb = (size_t)bh * nch + x;
    sgc[S] = GATE ? gC[cb] : 1.f;
    if constexpr (KDA) {
      const float4 g4 = *reinterpret_cast<const float4*>(gC + cb * DK + 16 * wave + 4 * lg);
      sgk[S] = floatx4{g4.x, g4.y, g4.z, g4.w};
    }
    // fragment (wave, kb) of P and of R^T: 64 lanes x 16 bytes, contiguous
#pragma unroll
    for (int kb = 0; kb < KP; ++kb) {
      if constexpr (DK == 16) {
        const uint2 h = *reinterpret_cast<const uint2*>(Pg + cb * DK * DK + (size_t)lane * 4);
        sp[S][kb] = u32x4{h.x, h.y, 0u, 0u};
      } else {
        sp[S][kb] = *reinterpret_cast<const u32x4*>(Pg + cb * DK * DK + (((size_t)wave * KP + kb) * 64 + lane) * 8);
      }
    }
    const bf16_t* rr = Rg + cb * DK * kC + (size_t)wave * 2 * 64 * 8 + (size_t)lane * 8;
    sr[S][0] = *reinterpret_cast<const u32x4*>(rr);
    sr[S][1] = *reinterpret_cast<const u32x4*>(rr + 64 * 8);
    const int t0 = x * kC, nrow = min(kC, Tn - t0);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = min(tid + NTH * j, NVO - 1);
      const int r = min(v / (DVS / 8), nrow - 1);
      so[S][j] = *reinterpret_cast<const u32x4*>(doh + (size_t)(t0 + r) * dv + (v % (DVS / 8)) * 8);
    }
  };
  auto store_do = [&](int x, auto slotc, int buf) {
    constexpr int S = decltype(slotc)::value;
    const int nrow = min(kC, Tn - x * kC);
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int v = tid + NTH * j;
      if (NVO % NTH != 0 && v >= NVO) continue;
      const int r = v / (DVS / 8), c8 = (v % (DVS / 8)) * 8;
      const u32x4 z = {0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(&sDO[buf][r][c8]) = r < nrow ? so[S][j] : z;
    }
  };
  floatx4 st[NJ];
  auto put_dst = [&](int buf) {  // dS^T, bf16: lane writes 4 consecutive rows of column 16 jt + lc
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) st4_bf16(&sDt[buf][16 * jt + lc][16 * wave + 4 * lg], st[jt][0], st[jt][1], st[jt][2], st[jt][3]);
  };
  const int col0 = sl * DVS + lc;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt) {
    st[jt] = zero4();
    if (a.dST) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[jt][i] = a.dST[((size_t)bh * DK + 16 * wave + 4 * lg + i) * dv + col0 + 16 * jt];
    }
  }
  issue(max(nch - 1, 0), std::integral_constant<int, 0>{});
  issue(max(nch - 2, 0), std::integral_constant<int, 1>{});
  issue(max(nch - 3, 0), std::integral_constant<int, 2>{});
  issue(max(nch - 4, 0), std::integral_constant<int, 3>{});
  put_dst(0);
  store_do(nch - 1, std::integral_constant<int, 0>{}, 0);
  lds_barrier();

  auto body = [&](const int i, auto slotc) {
    constexpr int S = decltype(slotc)::value, NXT = (S + 1) % NS, buf = S & 1;
    const int x = nch - 1 - i;
    // every LDS fragment of the chunk first, then the products
    bf16x8 fd[KP][NJ], fo[2][NJ];
#pragma unroll
    for (int kb = 0; kb < KP; ++kb)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        if constexpr (DK == 16) {
          const shortx4 h = *reinterpret_cast<const shortx4*>(&sDt[buf][16 * jt + lc][4 * lg]);
          fd[kb][jt] = __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(uint2, h).x, __builtin_bit_cast(uint2, h).y, 0u, 0u});
        } else {
          fd[kb][jt] = ld_frag(&sDt[buf][16 * jt + lc][32 * kb + 8 * lg]);
        }
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) fo[kb][jt] = tok_frag(&sDO[buf][0][0], LVO, 32 * kb, 16 * jt, lane);
    bf16_t* out = dSt + ((((size_t)bh * nch + x) * (DK / 16) + wave) * (dv / 16) + sl * NJ) * 256 + 4 * lane;
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) st4_bf16(out + 256 * jt, st[jt][0], st[jt][1], st[jt][2], st[jt][3]);
    floatx4 cp[NJ], cr[NJ];
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt) { cp[jt] = zero4(); cr[jt] = zero4(); }
    if constexpr (DK == 16) {  // one 16-deep product
      const shortx4 pa = words_to_shortx4(sp[S][0][0], sp[S][0][1]);
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        const u32x4 w = __builtin_bit_cast(u32x4, fd[0][jt]);
        cp[jt] = mfma_k16(pa, words_to_shortx4(w[0], w[1]), cp[jt]);
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < KP; ++kb) {
        const bf16x8 pa = __builtin_bit_cast(bf16x8, sp[S][kb]);
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) cp[jt] = mfma_k32(pa, fd[kb][jt], cp[jt]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bf16x8 ra = __builtin_bit_cast(bf16x8, sr[S][kb]);
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) cr[jt] = mfma_k32(ra, fo[kb][jt], cr[jt]);
    }
    if constexpr (KDA) {
      const floatx4 gk = sgk[S][0] < 0.f ? floatx4{0.f, 0.f, 0.f, 0.f} : sgk[S];
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) st[jt] = gk * st[jt] - cp[jt] + cr[jt];
    } else {
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) st[jt] = (GATE ? sgc[S] * st[jt] : st[jt]) - cp[jt] + cr[jt];
    }
    // the next chunk's dS^T and dO slice go to the other buffers (past the
    // first chunk this writes unused data)
    put_dst(buf ^ 1);
    store_do(max(x - 1, 0), std::integral_constant<int, NXT>{}, buf ^ 1);
    issue(max(x - NS, 0), slotc);
    lds_barrier();
  };
  int i = 0;
  for (; i + NS <= nch; i += NS) {
    body(i, std::integral_constant<int, 0>{});
    body(i + 1, std::integral_constant<int, 1>{});
    body(i + 2, std::integral_constant<int, 2>{});
    body(i + 3, std::integral_constant<int, 3>{});
  }
  if (i < nch) body(i, std::integral_constant<int, 0>{});
  if (i + 1 < nch) body(i + 1, std::integral_constant<int, 1>{});
  if (i + 2 < nch) body(i + 2, std::integral_constant<int, 2>{});
  if (a.dS0) {
#pragma unroll
    for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) a.dS0[((size_t)bh * DK + 16 * wave + 4 * lg + i2) * dv + col0 + 16 * jt] = st[jt][i2];
  }
}

// ---------------------------------------------------------------------------
// Pass 3: one workgroup per (batch, head, chunk).  Phases (barriers between),
// with LDS regions reused as operands die:
//   A  stage Q, K; tril(Q K^T) and K K^T -> L; bf16: the blocks of L and
//      D_b = (I + L_bb)^-1, also transposed; fp32: T (A and T are read by
//      columns where their transposes are needed)
//   B  per 16-column slice of dv (one wave each): X, u, du, dX from S and
//      dSn held as accumulator tiles (bf16: u and dX by block forward and
//      back substitution with those blocks, fp32: products with T); write dV; rowsum((V - K S) * dX) into
//      dbeta; u and dX rows to LDS
//   C  stage dO; dA = tril(dO u^T), dL = -tril(dX u^T, -1) (+ its rowsum
//      against K K^T into dbeta), both also transposed
//   D  stage K^T: dQ = dA K and dK = (bL) K + (bL)^T K, bL = diag(beta) dL;
//      then Q^T over bL: dK += dA^T Q (all kept in registers)
//   E  stage S, dSn rows; dQ += dO S^T, dK += u dSn^T - diag(beta) dX S^T;
//      write dQ, dK, dbeta
// ---------------------------------------------------------------------------
template <int DK, int DV, class E, bool GATE = false, bool KDA = false>
struct GradLayout {
  typedef typename E::T T;
  static constexpr int ES = (int)sizeof(T);
  static constexpr int PAD = 16 / ES;
  static constexpr int LQ = DK + PAD;   // rows of Q, K
  static constexpr int LV = DV + PAD;   // rows of u, dX, dO
  static constexpr int LS = DV + PAD;   // rows of S, dSn (key rows)
  static constexpr int LKT = kC + PAD;  // rows of A, dA, bL and their transposes, K^T, Q^T
  static constexpr int ROWQ = kC * LQ * ES, ROWV = kC * LV * ES, TRI = kC * LKT * ES;
  static constexpr int TQ = DK * LKT * ES, ST = DK * LS * ES, FT = kC * LTL * 4;
  // persistent: u, dX, K K^T (fp32), beta, dbeta
  static constexpr int oU = 0;
  static constexpr int oDX = oU + ROWV;
  static constexpr int oKK = oDX + ROWV;
  static constexpr int oB = oKK + FT;
  static constexpr int oDB = oB + kC * 4;
  static constexpr int oG = oDB + kC * 4;   // gated: G_r
  static constexpr int oDG = oG + kC * 4;   // gated: the gradient of G_r
  static constexpr int oGC = oDG + kC * 4;  // KDA: Gam_C per key channel
  static constexpr int oCC = oGC + (KDA ? DK * 4 : 0);  // KDA: the chunk decay's gradient per channel
  static constexpr int oW = oCC + (KDA ? DK * 4 : 0);  // phase-dependent work area
  // phases A, B
  static constexpr int aQ = oW, aK = aQ + ROWQ, aAt = aK + ROWQ, aTL = aAt + TRI;
  // bf16 inputs: the blocks of L (off the diagonal bf16, on it fp32) and
  // D_b = (I + L_bb)^-1, the bf16 ones also transposed, and A^T; the fp32 T
  // region aTL is not used then
  static constexpr int aLoT = aTL + FT, aDT = aLoT + 6 * 256 * 2, aAtt = aDT + 4 * 256 * 2;
  static constexpr int aLo = aAtt + TRI, aD = aLo + 6 * 256 * 2, aLd = aD + 4 * 256 * 2;
  static constexpr int endAB = ES == 2 ? aLd + 4 * 16 * 20 * 4 : aTL + FT;
  // KDA (bf16): K^ where the fp32 T region would be
  static constexpr int aKh = aTL;
  static_assert(!KDA || (ES == 2 && ROWQ <= FT), "KDA: K^ must fit the unused fp32 T region");
  // phases C, D: dO, dA, dA^T, bL, bL^T, K^T; then Q^T where bL was
  static constexpr int cDO = oW, cDA = cDO + ROWV, cDAt = cDA + TRI, cBL = cDAt + TRI, cBLt = cBL + TRI;
  static constexpr int dKt = cBLt + TRI, dQt = cBL;
  static_assert(TQ <= 2 * TRI, "Q^T must fit where bL and its transpose were");
  // bf16: K and Q row-major after the four 64 x 64 tiles
  static constexpr int dKr = cBLt + TRI, dQr = dKr + ROWQ;
  static constexpr int dKtr = dQr + ROWQ;  // KDA: K~ row-major as well
  static constexpr int endCD = ES == 2 ? dKtr + (KDA ? ROWQ : 0) : dKt + TQ;
  // phase E: dO (kept), S, dSn
  static constexpr int eS = cDA, eDS = eS + ST;
  static constexpr int endE = eDS + ST;
  static constexpr int endAll = endAB > endCD ? (endAB > endE ? endAB : endE) : (endCD > endE ? endCD : endE);
  // gated: the strictly lower part of the ten lower 16 x 16 tiles of the
  // gated A, kept from phase A to phase C: after everything (bf16), or
  // where K^T is staged in phase D (fp32; no phase before D uses it)
  static constexpr int oAg = ES == 2 ? endAll : dKt;
  static constexpr int endAg = oAg + (GATE ? 10 * 256 * ES : 0);
  static constexpr int total = endAll > endAg ? endAll : endAg;
  static_assert(ES == 2 || dKt >= endAB, "fp32: the kept A tiles must not overlap phases A and B");
};

// GATE (one log-decay per token, G_r summed from the chunk start): A, L and
// their gradients take the decay ratios exp(G_r - G_c); X = diag(beta)(V -
// diag(exp(G)) K S), du = A^T dO + diag(exp(G_C - G)) K dSn,
// dQ = diag(exp(G)) dO S^T + dA K, dK = ... + diag(exp(G_C - G)) u dSn^T -
// diag(beta exp(G)) dX S^T.  G enters the chunk at X (through exp(G_r) K S),
// at A and L (through the ratios), at O (exp(G_r) Q S) and at the state
// leaving it, so the gradient of G_r is
//   - beta_r exp(G_r) (K S)_r . dX_r + sum_j (dA * A)_rj - sum_i (dA * A)_ir
//   + k_r . (bL K - bL^T K)_r + exp(G_r) q_r . (dO S^T)_r
//   - exp(G_C - G_r) k_r . (u dSn^T)_r
// plus, on the last row, exp(G_C) <S, dSn> + sum_j exp(G_C - G_j) k_j .
// (u dSn^T)_j (dA, A, bL with the ratios).  Pairs that cancel exactly (the
// diagonal of dA * A, the last row's own k . (u dSn^T)) are left out, so
// every term carries a decay and dg keeps its relative accuracy when the
// decays are strong.  g_t enters G_r for r >= t of its own chunk only, so
// dg_t = sum of dG_r over r >= t in the chunk.
// KDA (bf16; a decay per key channel, the gate pre-pass's tiles): with
// dSn' = diag(Gam_C) dSn, the formulas above with Q~ for Q, K~ for K on the
// left of K S and of L (and W), K^ on the right of A and L and in the state
// update, and dSn' for dSn; the gradients of the three tiles are kept apart,
//   dQ~ = dO S^T + dA K^,  dK~ = (b dL) K^ - diag(beta) dX S^T,
//   dK^ = dA^T Q~ + (b dL)^T K~ + u dSn'^T.
// With G the log-decay summed from the chunk start (per channel, formed
// again here from g), Q~ = e^G q, K~ = e^G k, K^ = e^-G k and
// Gam_C = e^(G_C):  dq = e^G dQ~,  dk = e^G dK~ + e^-G dK^, and
//   dG = q e^G dQ~ + k e^G dK~ - k e^-G dK^  (elementwise),
// plus, on the chunk's last row, <S_i + (K^^T u)_i, dSn'_i> per channel i
// (Gam_C's part).  g_t enters G_r for r >= t of its own chunk only, so
// dg_t = sum of dG_r over r >= t; as the last row's term is in every such
// sum, it is added to every row.  A chunk walked token by token is left to
// kda_walk_grads.
template <int DK, int DV, class E, bool GATE, bool KDA = false>
__global__ __launch_bounds__(kGradThreads) void bwd_grads(BackwardArgs a, const float* __restrict__ Sc,
                                                     const float* __restrict__ dSc, KdaPtrs kp = KdaPtrs{}) {
  static_assert(!(GATE && KDA), "one gate kind at a time");
  typedef GradLayout<DK, DV, E, GATE, KDA> L;
  typedef typename E::T T;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int NTH = kGradThreads, NW = NTH / 64;
  constexpr int NKT = DK / 16;
  constexpr int NVT = DV / 16;
  constexpr int LQ = L::LQ, LV = L::LV, LS = L::LS, LKT = L::LKT;
  __shared__ __attribute__((aligned(16))) char smem[L::total];
  T* sU = reinterpret_cast<T*>(smem + L::oU);
  T* sDX = reinterpret_cast<T*>(smem + L::oDX);
  float* sKK = reinterpret_cast<float*>(smem + L::oKK);
  float* sB = reinterpret_cast<float*>(smem + L::oB);
  float* sDB = reinterpret_cast<float*>(smem + L::oDB);
  float* sG = reinterpret_cast<float*>(smem + L::oG);
  float* sDG = reinterpret_cast<float*>(smem + L::oDG);
  T* sAg = reinterpret_cast<T*>(smem + L::oAg);  // gated: [10][16][16], tile t = ti (ti + 1) / 2 + tj
  float* sGC = reinterpret_cast<float*>(smem + L::oGC);
  float* sCC = reinterpret_cast<float*>(smem + L::oCC);

  const int chunk = blockIdx.x;  // over B * H * nch
  if constexpr (KDA) {
    static_assert(sizeof(typename E::T) == 2, "KDA gradients: bf16 only");
    if (kp.gc[(size_t)chunk * DK] < 0.f) return;  // walked token by token (uniform)
  }
  const int Tn = a.T, nch = (Tn + kC - 1) / kC;
  const int bh = chunk / nch, c = chunk - bh * nch;
  const int t0 = c * kC, nrow = min(kC, Tn - t0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  const T* qh = reinterpret_cast<const T*>(a.q) + (size_t)bh * Tn * DK;
  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)bh * Tn * DK;
  const T* vh = reinterpret_cast<const T*>(a.v) + (size_t)bh * Tn * DV;
  const T* doh = reinterpret_cast<const T*>(a.dO) + (size_t)bh * Tn * DV;
  const T* bth = reinterpret_cast<const T*>(a.beta) + (size_t)bh * Tn;
  // S: fp32 row-major (fp32 inputs), or bf16 in accumulator-tile order
  const T* S = reinterpret_cast<const T*>(Sc) + (size_t)chunk * DK * DV;
  // dSn: fp32 row-major (fp32 inputs), or bf16 in accumulator-tile order
  // (bf16 inputs; written so by bwd_chain_mat)
  const float* dSn = dSc + (size_t)chunk * DK * DV;
  const bf16_t* dSt = reinterpret_cast<const bf16_t*>(dSc) + (size_t)chunk * DK * DV;

  // bf16, dv = 128 (eight 16-column slices, one per wave), no per-channel
  // decay: this wave's slice of S and dSn, loaded with phase A's loads
  // (after them, so that storing the staged tiles does not wait for these),
  // read by phase B and staged into LDS for phase E without a second load.
  // (With a per-channel decay the kernel has no registers to spare for it
  // and measured no gain.)
  constexpr bool kHold = kBf16 && !KDA && NVT == NW;
  uint2 hS[kHold ? NKT : 1], hD[kHold ? NKT : 1];
  // and (the same kernels) the V and dO entries phase B reads, rows 16mt +
  // 4lg + i of column 16 wave + lc: loaded at the start, they arrive while
  // phase A runs instead of holding up phase B's first product
  T hV[kHold ? 16 : 1], hO[kHold ? 16 : 1];

  // ---- phase A ----
  T* sQ = reinterpret_cast<T*>(smem + L::aQ);
  T* sK = reinterpret_cast<T*>(smem + L::aK);
  T* sA = reinterpret_cast<T*>(smem + L::aAt);  // tril(Q K^T), row-major
  float* sTL = reinterpret_cast<float*>(smem + L::aTL);
  bf16_t* sLoT = reinterpret_cast<bf16_t*>(smem + L::aLoT);
  bf16_t* sDT = reinterpret_cast<bf16_t*>(smem + L::aDT);
  bf16_t* sAtt = reinterpret_cast<bf16_t*>(smem + L::aAtt);
  bf16_t* sLo = reinterpret_cast<bf16_t*>(smem + L::aLo);
  bf16_t* sD = reinterpret_cast<bf16_t*>(smem + L::aD);
  float* sLd = reinterpret_cast<float*>(smem + L::aLd);
  T* sKh = reinterpret_cast<T*>(smem + L::aKh);
  const size_t tile0 = (size_t)chunk * kC * DK;  // KDA: this chunk's rows of the pre-pass tiles
  // Every staging load is issued before any of them is stored (one round
  // trip to memory instead of one per tile), and every lane issues each of
  // them: a load under a per-lane condition would make the compiler wait
  // for all outstanding loads.
  static_assert(DK <= NTH, "one Gam_C entry per thread");
  RowTile<E, DK, false, NTH> tq, tk, tkh;
  float gcv = 0.f;
  if constexpr (KDA) {
    tq.load(reinterpret_cast<const T*>(kp.qt + tile0), DK, 0, nrow, tid);
    tk.load(reinterpret_cast<const T*>(kp.kt + tile0), DK, 0, nrow, tid);
    tkh.load(reinterpret_cast<const T*>(kp.kht + tile0), DK, 0, nrow, tid);
    gcv = kp.gc[(size_t)chunk * DK + tid % DK];
  } else {
    tq.load(qh, DK, t0, nrow, tid);
    tk.load(kh, DK, t0, nrow, tid);
  }
  const T btv = bth[t0 + min(lane, nrow - 1)];
  // keep the early S and dSn loads behind these in the issue order (the
  // scheduler would otherwise hoist them), so that the stores below wait
  // for the tiles only
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (kHold) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) {
      hD[kt] = *reinterpret_cast<const uint2*>(dSt + (kt * NVT + wave) * 256 + 4 * lane);
      hS[kt] = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(S) + (kt * NVT + wave) * 256 + 4 * lane);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int rr = min(16 * (e >> 2) + 4 * lg + (e & 3), nrow - 1);  // rows past the end: zeroed in phase B
      hV[e] = vh[(size_t)(t0 + rr) * DV + 16 * wave + lc];
      hO[e] = doh[(size_t)(t0 + rr) * DV + 16 * wave + lc];
    }
  }
  tq.store(nrow, sQ, LQ, nullptr, 0, tid);
  tk.store(nrow, sK, LQ, nullptr, 0, tid);
  if constexpr (KDA) {
    tkh.store(nrow, sKh, LQ, nullptr, 0, tid);
    if (tid < DK) {
      sGC[tid] = gcv;
      sCC[tid] = 0.f;
    }
  }
  if (tid < kC) {
    sB[tid] = tid < nrow ? E::tof(btv) : 0.f;
    sDB[tid] = 0.f;
  }
  if constexpr (GATE) {
    if (wave == 0) {
      sG[lane] = chunk_logdecay<E>(reinterpret_cast<const T*>(a.g) + (size_t)bh * Tn, t0, nrow, lane);
      sDG[lane] = 0.f;
    }
  }
  for (int i = tid; i < kC * kC; i += NTH) {  // tiles above the diagonal stay zero
    const int r = i >> 6, cc = i & 63;
    if ((cc >> 4) > (r >> 4)) {
      sA[r * LKT + cc] = E::cvt(0.f);
      if constexpr (kBf16) sAtt[cc * LKT + r] = E::cvt(0.f);
    }
  }
  __syncthreads();
  for (int jb = wave; jb < 20; jb += NW) {
    const bool isA = jb < 10;
    const int t = isA ? jb : jb - 10;
    const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int tj = t - ti * (ti + 1) / 2;
    floatx4 acc = rowrow<kBf16>(zero4(), (isA ? sQ : sK) + (16 * ti + lc) * LQ, (KDA ? sKh : sK) + (16 * tj + lc) * LQ,
                                DK, lane);
    const int cc = 16 * tj + lc;
    if constexpr (GATE) {
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] *= decay_ratio(sG, 16 * ti + 4 * lg + i, cc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ti + 4 * lg + i;
      if (isA) {
        if constexpr (GATE) sAg[t * 256 + (4 * lg + i) * 16 + lc] = E::cvt(cc < r ? acc[i] : 0.f);
        sA[r * LKT + cc] = E::cvt(cc <= r ? acc[i] : 0.f);
        if constexpr (kBf16) sAtt[cc * LKT + r] = E::cvt(cc <= r ? acc[i] : 0.f);
      } else {
        if (cc < r) sKK[r * LTL + cc] = acc[i];
        if constexpr (kBf16) {
          const float l = cc < r ? sB[r] * acc[i] : 0.f;
          if (ti == tj) sLd[(16 * ti + 4 * lg + i) * 20 + lc] = l;
          else sLo[((ti * (ti - 1) / 2 + tj) * 16 + 4 * lg + i) * 16 + lc] = f2bf(l);
        } else if (cc < r) {
          sTL[cc * LTL + r] = sB[r] * acc[i];
        }
      }
    }
    if constexpr (kBf16) {
      if (!isA && ti != tj) {  // L_ti,tj transposed: row lc of it is column cc of the block
        const float* bt = sB + 16 * ti + 4 * lg;
        st4_bf16(sLoT + ((ti * (ti - 1) / 2 + tj) * 16 + lc) * 16 + 4 * lg, bt[0] * acc[0], bt[1] * acc[1],
                 bt[2] * acc[2], bt[3] * acc[3]);
      }
    }
  }
  __syncthreads();
  if constexpr (kBf16) {
    // D_b: lane (block lg, column lc) solves (I + L_bb) x = e_lc
    if (wave == 0) {
      // right-looking: once x_m is known it is folded into the partial sums
      // of every later row, so one multiply-add separates x_m from x_{m+1}
      // (x_m = 0 for m < lc, x_lc = 1)
      const float* lb = sLd + 16 * lg * 20;
      float x[16], ps[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) ps[i] = 0.f;
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        x[m] = m < lc ? 0.f : (m == lc ? 1.f : -ps[m]);
#pragma unroll
        for (int i = m + 1; i < 16; ++i) ps[i] += lb[i * 20 + m] * x[m];
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sD[(16 * lg + i) * 16 + lc] = f2bf(x[i]);
#pragma unroll
      for (int i = 0; i < 16; i += 4) st4_bf16(sDT + (16 * lg + lc) * 16 + i, x[i], x[i + 1], x[i + 2], x[i + 3]);
    }
    __syncthreads();
  } else {
    form_T<kBf16, NTH>(sTL, tid, wave, lane);
  }
  // an A operand from a 16 x 16 bf16 block stored row-major
  auto blk16 = [&](const bf16_t* b) { return *reinterpret_cast<const shortx4*>(b + lc * 16 + 4 * lg); };

  // ---- phase B: 16-column slices of dv, one per wave at a time ----
  for (int s = wave; s < NVT; s += NW) {
    const int col = 16 * s + lc;
    floatx4 Sv[NKT], dSv[NKT], vt[4], dOt[4];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (!kBf16) {
          Sv[kt][i] = S[(size_t)(16 * kt + 4 * lg + i) * DV + col];
          dSv[kt][i] = dSn[(size_t)(16 * kt + 4 * lg + i) * DV + col];
        }
      }
    if constexpr (kBf16) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const uint2 w = kHold ? hD[kHold ? kt : 0]
                              : *reinterpret_cast<const uint2*>(dSt + (kt * NVT + s) * 256 + 4 * lane);
        const uint2 v = kHold ? hS[kHold ? kt : 0]
                              : *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(S) + (kt * NVT + s) * 256 + 4 * lane);
        dSv[kt][0] = bf2f((bf16_t)(w.x & 0xffffu));
        dSv[kt][1] = bf2f((bf16_t)(w.x >> 16));
        dSv[kt][2] = bf2f((bf16_t)(w.y & 0xffffu));
        dSv[kt][3] = bf2f((bf16_t)(w.y >> 16));
        Sv[kt][0] = bf2f((bf16_t)(v.x & 0xffffu));
        Sv[kt][1] = bf2f((bf16_t)(v.x >> 16));
        Sv[kt][2] = bf2f((bf16_t)(v.y & 0xffffu));
        Sv[kt][3] = bf2f((bf16_t)(v.y >> 16));
      }
    }
    if constexpr (KDA) {  // dSn' = diag(Gam_C) dSn; <S_i, dSn'_i> over this slice, per channel
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * kt + 4 * lg + i;
          dSv[kt][i] *= sGC[ch];
          float p = Sv[kt][i] * dSv[kt][i];
          p = sum16(p);
          if (lc == 0) atomicAdd(&sCC[ch], p);
        }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * lg + i;
        const int rr = min(r, nrow - 1);  // every lane loads; rows past the end are zeroed
        const float vx = E::tof(kHold ? hV[kHold ? 4 * mt + i : 0] : vh[(size_t)(t0 + rr) * DV + col]);
        const float ox = E::tof(kHold ? hO[kHold ? 4 * mt + i : 0] : doh[(size_t)(t0 + rr) * DV + col]);
        vt[mt][i] = r < nrow ? vx : 0.f;
        dOt[mt][i] = r < nrow ? ox : 0.f;
      }
    floatx4 res[4], xx[4], ut[4], du[4], dx[4], gy[4];  // gy: exp(G) K S (gated)
    if constexpr (GATE) {  // exp(G_C) <S, dSn> over this slice, to the last row
      float p = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) p += Sv[kt][i] * dSv[kt][i];
      p = sum64(p);
      if (lane == 0) atomicAdd(&sDG[nrow - 1], __expf(sG[63]) * p);
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      floatx4 y = accB<kBf16>(zero4(), sK + (16 * mt + lc) * LQ, Sv, NKT, lane);
      if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] *= __expf(sG[16 * mt + 4 * lg + i]);
        gy[mt] = y;
      }
      res[mt] = vt[mt] - y;  // V - K S
#pragma unroll
      for (int i = 0; i < 4; ++i) xx[mt][i] = sB[16 * mt + 4 * lg + i] * res[mt][i];
    }
    if constexpr (kBf16) {
      // u = (I + L)^-1 X by block forward substitution, as in the forward:
      // u_b = D_b (X_b - sum_{j<b} L_bj u_j)
      shortx4 ub[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        floatx4 acc = xx[b];
        if (b > 0) {
          floatx4 t = zero4();
#pragma unroll
          for (int j = 0; j < b; ++j) t = mfma_k16(blk16(sLo + (b * (b - 1) / 2 + j) * 256), ub[j], t);
          acc = xx[b] - t;
        }
        ut[b] = mfma_k16(blk16(sD + 256 * b), acc_to_b16(acc), zero4());
        ub[b] = acc_to_b16(ut[b]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      floatx4 d1;
      if constexpr (kBf16) {
        d1 = accB<kBf16>(zero4(), sAtt + (16 * mt + lc) * LKT, dOt, 4, lane);  // A^T dO
      } else {
        ut[mt] = accB<kBf16>(zero4(), sTL + (16 * mt + lc) * LTL, xx, mt + 1, lane);
        d1 = accB_col<kBf16>(zero4(), sA + 16 * mt + lc, LKT, dOt, 4, lane);  // A^T dO
      }
      floatx4 d2 = accB<kBf16>(zero4(), (KDA ? sKh : sK) + (16 * mt + lc) * LQ, dSv, NKT, lane);
      if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) d2[i] *= __expf(sG[63] - sG[16 * mt + 4 * lg + i]);
      }
      du[mt] = d1 + d2;
    }
    if constexpr (kBf16) {
      // dX = (I + L)^-T du by block back substitution:
      // dX_b = D_b^T (du_b - sum_{j>b} L_jb^T dX_j)
      shortx4 xb[4];
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        floatx4 acc = du[b];
        if (b < 3) {
          floatx4 t = zero4();
#pragma unroll
          for (int j = b + 1; j < 4; ++j) t = mfma_k16(blk16(sLoT + (j * (j - 1) / 2 + b) * 256), xb[j], t);
          acc = du[b] - t;
        }
        dx[b] = mfma_k16(blk16(sDT + 256 * b), acc_to_b16(acc), zero4());
        xb[b] = acc_to_b16(dx[b]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if constexpr (!kBf16) dx[mt] = accB_col<kBf16>(zero4(), sTL + 16 * mt + lc, LTL, du, 4, lane);  // T^T du
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * lg + i;
        if constexpr (!kBf16) {
          if (r < nrow) reinterpret_cast<T*>(a.dv)[((size_t)bh * Tn + t0 + r) * DV + col] = E::cvt(sB[r] * dx[mt][i]);
        }
        sU[r * LV + col] = E::cvt(ut[mt][i]);
        sDX[r * LV + col] = E::cvt(dx[mt][i]);
        float p = res[mt][i] * dx[mt][i];  // rowsum over this slice's 16 columns
        p = sum16(p);
        if (lc == 0) atomicAdd(&sDB[r], p);
        if constexpr (GATE) {  // - beta_r exp(G_r) (K S)_r . dX_r
          float pv = gy[mt][i] * sB[r] * dx[mt][i];
          pv = sum16(pv);
          if (lc == 0) atomicAdd(&sDG[r], -pv);
        }
      }
    }
  }
  __syncthreads();
  // phase C's dO tile, requested before the dV stores go out
  RowTile<E, DV, false, NTH> tdo;
  tdo.load(doh, DV, t0, nrow, tid);
  if constexpr (kBf16) {  // dV = diag(beta) dX, from its rows in LDS with 16-byte stores
    constexpr int NVD = kC * DV / 8;
    for (int v = tid; v < NVD; v += NTH) {
      const int r = v / (DV / 8), c8 = (v % (DV / 8)) * 8;
      if (r >= nrow) continue;
      const u32x4 x = *reinterpret_cast<const u32x4*>(reinterpret_cast<const bf16_t*>(sDX) + r * LV + c8);
      const float br = sB[r];
      u32x4 y;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        y[e] = pack2(br * __uint_as_float(x[e] << 16), br * __uint_as_float(x[e] & 0xffff0000u));
      *reinterpret_cast<u32x4*>(reinterpret_cast<bf16_t*>(a.dv) + ((size_t)bh * Tn + t0 + r) * DV + c8) = y;
    }
  }

  // ---- phase C ----
  T* sDO = reinterpret_cast<T*>(smem + L::cDO);
  T* sDA = reinterpret_cast<T*>(smem + L::cDA);
  T* sDAt = reinterpret_cast<T*>(smem + L::cDAt);
  T* sBL = reinterpret_cast<T*>(smem + L::cBL);
  T* sBLt = reinterpret_cast<T*>(smem + L::cBLt);
  tdo.store(nrow, sDO, LV, nullptr, 0, tid);
  // bf16: phase D's row-major K and Q tiles (KDA: K^, Q~ and K~), requested
  // now so that phase C covers their latency
  RowTile<E, DK, false, NTH> tdk, tdq, tdk2;
  if constexpr (kBf16) {
    if constexpr (KDA) {
      tdk.load(reinterpret_cast<const T*>(kp.kht + tile0), DK, 0, nrow, tid);
      tdq.load(reinterpret_cast<const T*>(kp.qt + tile0), DK, 0, nrow, tid);
      tdk2.load(reinterpret_cast<const T*>(kp.kt + tile0), DK, 0, nrow, tid);
    } else {
      tdk.load(kh, DK, t0, nrow, tid);
      tdq.load(qh, DK, t0, nrow, tid);
    }
  }
  // bf16: sDAt and sBLt hold dA and diag(beta) dL with their token columns
  // permuted by tperm (A operands against the transpose reads of phase D);
  // fp32: the transposes
  for (int i = tid; i < kC * kC; i += NTH) {  // tiles above the diagonal stay zero
    const int r = i >> 6, cc = i & 63;
    if ((cc >> 4) > (r >> 4)) {
      const T z = E::cvt(0.f);
      sDA[r * LKT + cc] = z;
      sBL[r * LKT + cc] = z;
      if constexpr (kBf16) {
        sDAt[r * LKT + tperm(cc)] = z;
        sBLt[r * LKT + tperm(cc)] = z;
      } else {
        sDAt[cc * LKT + r] = z;
        sBLt[cc * LKT + r] = z;
      }
    }
  }
  __syncthreads();
  for (int jb = wave; jb < 20; jb += NW) {
    const bool isA = jb < 10;  // dA, else dL
    const int t = isA ? jb : jb - 10;
    const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
    const int tj = t - ti * (ti + 1) / 2;
    if constexpr (kBf16) {
      // the transposed product: lane holds row r = 16 ti + lc, columns
      // c0 .. c0 + 3 of dA = dO u^T (or of dX u^T), 8-byte stores
      const floatx4 acc =
          rowrow<kBf16>(zero4(), sU + (16 * tj + lc) * LV, (isA ? sDO : sDX) + (16 * ti + lc) * LV, DV, lane);
      const int r = 16 * ti + lc, c0 = 16 * tj + 4 * lg;
      float gm[4] = {1.f, 1.f, 1.f, 1.f};
      if constexpr (GATE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) gm[i] = decay_ratio(sG, r, c0 + i);
      }
      if (isA) {
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = c0 + i <= r ? acc[i] * gm[i] : 0.f;
        if constexpr (GATE) {
          // A's part of the gradient of G: row sums minus column sums of
          // dA * A below the diagonal (on it the two cancel exactly)
          const uint2 w = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(sAg) + t * 256 + lc * 16 + 4 * lg);
          const float ag[4] = {bf2f((bf16_t)(w.x & 0xffffu)), bf2f((bf16_t)(w.x >> 16)), bf2f((bf16_t)(w.y & 0xffffu)),
                               bf2f((bf16_t)(w.y >> 16))};
          float m[4], rs = 0.f;
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // dA (without the ratios) times the gated A
            m[i] = acc[i] * ag[i];
            rs += m[i];
          }
          rs = xsum32(xsum16(rs));
          if (lg == 0) atomicAdd(&sDG[r], rs);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m[i] = sum16(m[i]);
            if (lc == 0) atomicAdd(&sDG[c0 + i], -m[i]);
          }
        }
        st4_bf16(reinterpret_cast<bf16_t*>(sDA) + r * LKT + c0, v[0], v[1], v[2], v[3]);
        st4_bf16(reinterpret_cast<bf16_t*>(sDAt) + r * LKT + tperm(c0), v[0], v[1], v[2], v[3]);
      } else {
        float dl[4], p = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          dl[i] = c0 + i < r ? -acc[i] : 0.f;
          p += c0 + i < r ? dl[i] * sKK[r * LTL + c0 + i] : 0.f;  // rowsum(dL * K K^T)
        }
        p = xsum32(xsum16(p));
        if (lg == 0) atomicAdd(&sDB[r], p);
        const float br = sB[r];
#pragma unroll
        for (int i = 0; i < 4; ++i) dl[i] *= gm[i];
        st4_bf16(reinterpret_cast<bf16_t*>(sBL) + r * LKT + c0, br * dl[0], br * dl[1], br * dl[2], br * dl[3]);
        st4_bf16(reinterpret_cast<bf16_t*>(sBLt) + r * LKT + tperm(c0), br * dl[0], br * dl[1], br * dl[2],
                 br * dl[3]);
      }
      continue;
    }
    const floatx4 acc =
        rowrow<kBf16>(zero4(), (isA ? sDO : sDX) + (16 * ti + lc) * LV, sU + (16 * tj + lc) * LV, DV, lane);
    const int cc = 16 * tj + lc;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ti + 4 * lg + i;
      const float gm = GATE ? decay_ratio(sG, r, cc) : 1.f;
      if (isA) {
        const T x = E::cvt(cc <= r ? acc[i] * gm : 0.f);
        sDA[r * LKT + cc] = x;
        sDAt[cc * LKT + r] = x;
        if constexpr (GATE) {  // dA * A below the diagonal: + row sum, - column sum
          float m = acc[i] * E::tof(sAg[t * 256 + (4 * lg + i) * 16 + lc]);  // dA times the gated A
          float rs = m;
          rs = sum16(rs);
          if (lc == 0) atomicAdd(&sDG[r], rs);
          m = xsum32(xsum16(m));
          if (lg == 0) atomicAdd(&sDG[cc], -m);
        }
      } else {
        const float dl = cc < r ? -acc[i] : 0.f;
        float p = cc < r ? dl * sKK[r * LTL + cc] : 0.f;  // rowsum(dL * K K^T)
        p = sum16(p);
        if (lc == 0) atomicAdd(&sDB[r], p);
        const T x = E::cvt(sB[r] * dl * gm);
        sBL[r * LKT + cc] = x;
        sBLt[cc * LKT + r] = x;
      }
    }
  }
  __syncthreads();

  // ---- phase D: each wave owns output tiles id = wave + 4 n of the 4 x NKT grid ----
  constexpr int NTILE = 4 * NKT, NOWN = (NTILE + NW - 1) / NW;  // output tiles, per wave
  floatx4 gq[NOWN], gk[NOWN], gkh[KDA ? NOWN : 1];  // KDA: dK~ in gk, dK^ in gkh
  // KDA: this lane's g, q, k for its output tiles of phase E (row 16 ti + lc,
  // channels d0 .. d0 + 3), loaded now so that phase D covers their latency
  uint2 rg[KDA ? NOWN : 1], rq[KDA ? NOWN : 1], rk[KDA ? NOWN : 1];
  if constexpr (KDA) {
    const bf16_t* ghh = reinterpret_cast<const bf16_t*>(a.g) + ((size_t)bh * Tn + t0) * DK;
#pragma unroll
    for (int n = 0; n < NOWN; ++n) {
      const int id = min(wave + NW * n, NTILE - 1), ti = id / NKT, tk = id - ti * NKT;
      const size_t o = (size_t)min(16 * ti + lc, nrow - 1) * DK + 16 * tk + 4 * lg;  // in bounds for every lane
      rg[n] = *reinterpret_cast<const uint2*>(ghh + o);
      rq[n] = *reinterpret_cast<const uint2*>(qh + (size_t)t0 * DK + o);
      rk[n] = *reinterpret_cast<const uint2*>(kh + (size_t)t0 * DK + o);
    }
  }
  float gpre[KDA ? NOWN : 1][4], dsuf[KDA ? NOWN : 1][4];
  float* sTotG = sKK;            // KDA, [4][DK]: per tile, the sum of its rows' g
  float* sTotD = sKK + 4 * DK;   // KDA, [4][DK]: per tile, the sum of its rows' dG
  if constexpr (kBf16) {
    // K and Q row-major; every product over tokens reads them (and dA,
    // diag(beta) dL) with the transpose read or against the permuted copies.
    // Tiles are computed transposed: lane holds output row r = 16 ti + lc,
    // columns 16 tk + 4 lg .. +3.
    bf16_t* sKr = reinterpret_cast<bf16_t*>(smem + L::dKr);
    bf16_t* sQr = reinterpret_cast<bf16_t*>(smem + L::dQr);
    bf16_t* sKtr = reinterpret_cast<bf16_t*>(smem + L::dKtr);  // KDA: K~ (sKr holds K^, sQr Q~)
    tdk.store(nrow, reinterpret_cast<T*>(sKr), LQ, nullptr, 0, tid);
    tdq.store(nrow, reinterpret_cast<T*>(sQr), LQ, nullptr, 0, tid);
    if constexpr (KDA) tdk2.store(nrow, reinterpret_cast<T*>(sKtr), LQ, nullptr, 0, tid);
    __syncthreads();
    const bf16_t* bDA = reinterpret_cast<const bf16_t*>(sDA);
    const bf16_t* bDAp = reinterpret_cast<const bf16_t*>(sDAt);
    const bf16_t* bBL = reinterpret_cast<const bf16_t*>(sBL);
    const bf16_t* bBLp = reinterpret_cast<const bf16_t*>(sBLt);
#pragma unroll
    for (int n = 0; n < NOWN; ++n) {
      const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
      if (NTILE % NW != 0 && id >= NTILE) continue;
      // gated: (b dL) K and (b dL)^T K kept apart (xk, xb) for the gradient of G
      floatx4 xq = zero4(), xk = zero4(), xb = zero4(), xc = zero4();
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = tok_frag(sKr, LQ, 32 * kb, 16 * tk, lane);
        xq = mfma_k32(kf, ld_frag(bDAp + (16 * ti + lc) * LKT + 32 * kb + 8 * lg), xq);           // dA K
        xk = mfma_k32(kf, ld_frag(bBLp + (16 * ti + lc) * LKT + 32 * kb + 8 * lg), xk);           // (b dL) K
        if constexpr (KDA) {
          xb = mfma_k32(tok_frag(sKtr, LQ, 32 * kb, 16 * tk, lane), tok_frag(bBL, LKT, 32 * kb, 16 * ti, lane), xb);
        } else if constexpr (GATE) {
          xb = mfma_k32(kf, tok_frag(bBL, LKT, 32 * kb, 16 * ti, lane), xb);  // (b dL)^T K
        } else {
          xk = mfma_k32(kf, tok_frag(bBL, LKT, 32 * kb, 16 * ti, lane), xk);
        }
        const bf16x8 qf = tok_frag(sQr, LQ, 32 * kb, 16 * tk, lane), af = tok_frag(bDA, LKT, 32 * kb, 16 * ti, lane);
        if constexpr (GATE || KDA) xc = mfma_k32(qf, af, xc);  // dA^T Q
        else xk = mfma_k32(qf, af, xk);
      }
      if constexpr (GATE) {  // k_r . (bL K - bL^T K)_r, four columns per lane
        const int r = 16 * ti + lc, d0 = 16 * tk + 4 * lg;
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) p += bf2f(sKr[r * LQ + d0 + i]) * (xk[i] - xb[i]);
        p = xsum32(xsum16(p));
        if (lg == 0) atomicAdd(&sDG[r], p);
        xk += xb + xc;
      }
      gq[n] = xq;
      gk[n] = xk;
      if constexpr (KDA) gkh[n] = xb + xc;
    }
    if constexpr (KDA) {
      // the log-decay G_r summed from the chunk start, per key channel, for
      // this lane's rows and channels: a prefix over the tile's 16 rows by
      // shuffles now, plus the totals of the tiles above (through LDS, in the
      // K K^T region, free since phase C) in phase E
#pragma unroll
      for (int n = 0; n < NOWN; ++n) {
        const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
        const bool own = NTILE % NW == 0 || id < NTILE;
        const int r = 16 * ti + lc, d0 = 16 * tk + 4 * lg;
        float x[4];
        x[0] = bf2f((bf16_t)(rg[n].x & 0xffffu));
        x[1] = bf2f((bf16_t)(rg[n].x >> 16));
        x[2] = bf2f((bf16_t)(rg[n].y & 0xffffu));
        x[3] = bf2f((bf16_t)(rg[n].y >> 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (r >= nrow) x[i] = 0.f;
          x[i] = scan16_up(x[i]);
          gpre[n][i] = x[i];
          if (own && lc == 15) sTotG[ti * DK + d0 + i] = x[i];
        }
      }
    }
    __syncthreads();
  } else {
  T* sKt = reinterpret_cast<T*>(smem + L::dKt);
  T* sQt = reinterpret_cast<T*>(smem + L::dQt);
  stage_rows<E, DK, NTH>(kh, DK, t0, nrow, nullptr, 0, sKt, LKT, tid);
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NOWN; ++n) {
    const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
    if (NTILE % NW != 0 && id >= NTILE) continue;
    gq[n] = rowrow<kBf16>(zero4(), sDA + (16 * ti + lc) * LKT, sKt + (16 * tk + lc) * LKT, kC, lane);
    const floatx4 x = rowrow<kBf16>(zero4(), sBL + (16 * ti + lc) * LKT, sKt + (16 * tk + lc) * LKT, kC, lane);
    const floatx4 xt = rowrow<kBf16>(zero4(), sBLt + (16 * ti + lc) * LKT, sKt + (16 * tk + lc) * LKT, kC, lane);
    gk[n] = x + xt;
    if constexpr (GATE) {  // k_r . (bL K - bL^T K)_r over the tile's 16 columns
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * ti + 4 * lg + i, d = 16 * tk + lc;
        float p = r < nrow ? E::tof(sKt[d * LKT + r]) * (x[i] - xt[i]) : 0.f;
        p = sum16(p);
        if (lc == 0) atomicAdd(&sDG[r], p);
      }
    }
  }
  __syncthreads();  // bL is dead: Q^T goes in its place
  stage_rows<E, DK, NTH>(qh, DK, t0, nrow, nullptr, 0, sQt, LKT, tid);
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NOWN; ++n) {
    const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
    if (NTILE % NW != 0 && id >= NTILE) continue;
    gk[n] += rowrow<kBf16>(zero4(), sDAt + (16 * ti + lc) * LKT, sQt + (16 * tk + lc) * LKT, kC, lane);
  }
  __syncthreads();
  }

  // ---- phase E ----
  T* sS = reinterpret_cast<T*>(smem + L::eS);
  T* sDS = reinterpret_cast<T*>(smem + L::eDS);
  if constexpr (kBf16) {
    // S and dSn in accumulator-tile order: lane-tile i (tile i / 64, lane
    // i % 64) holds four rows of one column; all loads first
    constexpr int NLT = DK * DV / 4, NPT = (NLT + NTH - 1) / NTH;
    uint2 bs[NPT], bd[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      if constexpr (kHold) {  // lane-tile tid + NTH j is tile (j, wave), lane `lane`: the held words
        bs[j] = hS[kHold ? j : 0];
        bd[j] = hD[kHold ? j : 0];
      } else {
        const int i = min(tid + NTH * j, NLT - 1);
        bs[j] = *reinterpret_cast<const uint2*>(reinterpret_cast<const bf16_t*>(S) + 4 * i);
        bd[j] = *reinterpret_cast<const uint2*>(dSt + 4 * i);
      }
    }
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i = tid + NTH * j;
      if (NLT % NTH != 0 && i >= NLT) continue;
      const int tile = i >> 6, ln = i & 63, kt = tile / NVT, jt = tile - kt * NVT;
      const int o = (16 * kt + 4 * (ln >> 4)) * LS + 16 * jt + (ln & 15);
      bf16_t* ps = reinterpret_cast<bf16_t*>(sS) + o;
      bf16_t* pd = reinterpret_cast<bf16_t*>(sDS) + o;
      if constexpr (KDA) {  // dSn' = diag(Gam_C) dSn: rows are key channels
        const float* gr = sGC + 16 * kt + 4 * (ln >> 4);
        bd[j] = make_uint2(pack2(gr[0] * bf2f((bf16_t)(bd[j].x & 0xffffu)), gr[1] * bf2f((bf16_t)(bd[j].x >> 16))),
                           pack2(gr[2] * bf2f((bf16_t)(bd[j].y & 0xffffu)), gr[3] * bf2f((bf16_t)(bd[j].y >> 16))));
      }
      ps[0] = (bf16_t)(bs[j].x & 0xffffu); ps[LS] = (bf16_t)(bs[j].x >> 16);
      ps[2 * LS] = (bf16_t)(bs[j].y & 0xffffu); ps[3 * LS] = (bf16_t)(bs[j].y >> 16);
      pd[0] = (bf16_t)(bd[j].x & 0xffffu); pd[LS] = (bf16_t)(bd[j].x >> 16);
      pd[2 * LS] = (bf16_t)(bd[j].y & 0xffffu); pd[3 * LS] = (bf16_t)(bd[j].y >> 16);
    }
  } else {  // fp32 rows
    constexpr int NV4 = DK * DV / 4, NPT = NV4 / NTH > 0 ? NV4 / NTH : 1;
    float4 bs[NPT], bd[NPT];
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i = min(tid + NTH * j, NV4 - 1);
      bs[j] = reinterpret_cast<const float4*>(S)[i];
      bd[j] = reinterpret_cast<const float4*>(dSn)[i];
    }
#pragma unroll
    for (int j = 0; j < NPT; ++j) {
      const int i = tid + NTH * j;
      if (i >= NV4) continue;
      const int r = (4 * i) / DV, d = (4 * i) % DV;
      T* ps = sS + r * LS + d;
      T* pd = sDS + r * LS + d;
      ps[0] = E::cvt(bs[j].x); ps[1] = E::cvt(bs[j].y); ps[2] = E::cvt(bs[j].z); ps[3] = E::cvt(bs[j].w);
      pd[0] = E::cvt(bd[j].x); pd[1] = E::cvt(bd[j].y); pd[2] = E::cvt(bd[j].z); pd[3] = E::cvt(bd[j].w);
    }
  }
  T* dqo = reinterpret_cast<T*>(a.dq) + ((size_t)bh * Tn + t0) * DK;
  T* dko = reinterpret_cast<T*>(a.dk) + ((size_t)bh * Tn + t0) * DK;
  __syncthreads();
#pragma unroll
  for (int n = 0; n < NOWN; ++n) {
    const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
    if (NTILE % NW != 0 && id >= NTILE) continue;
    if constexpr (kBf16) {  // transposed tiles, as gq and gk: row r = 16 ti + lc
      const floatx4 q1 = rowrow<kBf16>(zero4(), sS + (16 * tk + lc) * LS, sDO + (16 * ti + lc) * LV, DV, lane);
      const floatx4 k1 = rowrow<kBf16>(zero4(), sDS + (16 * tk + lc) * LS, sU + (16 * ti + lc) * LV, DV, lane);
      const floatx4 k2 = rowrow<kBf16>(zero4(), sS + (16 * tk + lc) * LS, sDX + (16 * ti + lc) * LV, DV, lane);
      const int r = 16 * ti + lc, d0 = 16 * tk + 4 * lg;
      const float br = sB[r];
      if constexpr (KDA) {
        // with Q~ = e^G q, K~ = e^G k, K^ = e^-G k (fp32 from the inputs):
        //   dq = e^G dQ~,  dk = e^G dK~ + e^-G dK^,
        //   dG = q e^G dQ~ + k e^G dK~ - k e^-G dK^;
        // and the sum over tokens of K^ (u dSn'^T) per channel, the part of
        // the decay's gradient through Gam_C that phase B did not form
        float qv[4] = {0.f, 0.f, 0.f, 0.f}, kv[4] = {0.f, 0.f, 0.f, 0.f};
        if (r < nrow) {
          qv[0] = bf2f((bf16_t)(rq[n].x & 0xffffu)); qv[1] = bf2f((bf16_t)(rq[n].x >> 16));
          qv[2] = bf2f((bf16_t)(rq[n].y & 0xffffu)); qv[3] = bf2f((bf16_t)(rq[n].y >> 16));
          kv[0] = bf2f((bf16_t)(rk[n].x & 0xffffu)); kv[1] = bf2f((bf16_t)(rk[n].x >> 16));
          kv[2] = bf2f((bf16_t)(rk[n].y & 0xffffu)); kv[3] = bf2f((bf16_t)(rk[n].y >> 16));
        }
        float dq4[4], dk4[4], dG[4], p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float G = gpre[n][i];
          for (int t2 = 0; t2 < ti; ++t2) G += sTotG[t2 * DK + d0 + i];
          const float e = __expf(G), ie = __expf(-G);
          const float dqt = gq[n][i] + q1[i], dkt = gk[n][i] - br * k2[i], dkh = gkh[n][i] + k1[i];
          dq4[i] = e * dqt;
          dk4[i] = e * dkt + ie * dkh;
          dG[i] = qv[i] * e * dqt + kv[i] * e * dkt - kv[i] * ie * dkh;
          p[i] = kv[i] * ie * k1[i];
        }
        if (r < nrow) {
          st4_bf16(reinterpret_cast<bf16_t*>(dqo) + (size_t)r * DK + d0, dq4[0], dq4[1], dq4[2], dq4[3]);
          st4_bf16(reinterpret_cast<bf16_t*>(dko) + (size_t)r * DK + d0, dk4[0], dk4[1], dk4[2], dk4[3]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[i] = sum16(p[i]);
          dG[i] = scan16_down(dG[i]);  // suffix over the tile's rows
          if (lc == 0) {
            atomicAdd(&sCC[d0 + i], p[i]);
            sTotD[ti * DK + d0 + i] = dG[i];
          }
          dsuf[n][i] = dG[i];
        }
        continue;
      }
      // gated: dO S^T and beta dX S^T times exp(G_r), u dSn^T times exp(G_C - G_r)
      const float e1 = GATE ? __expf(sG[r]) : 1.f, e2 = GATE ? __expf(sG[63] - sG[r]) : 1.f;
      float dq4[4], dk4[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dq4[i] = gq[n][i] + e1 * q1[i];
        dk4[i] = gk[n][i] + e2 * k1[i] - br * e1 * k2[i];
      }
      if (r < nrow) {
        st4_bf16(reinterpret_cast<bf16_t*>(dqo) + (size_t)r * DK + d0, dq4[0], dq4[1], dq4[2], dq4[3]);
        st4_bf16(reinterpret_cast<bf16_t*>(dko) + (size_t)r * DK + d0, dk4[0], dk4[1], dk4[2], dk4[3]);
      }
      if constexpr (GATE) {  // exp(G_r) q . (dO S^T) - exp(G_C - G_r) k . (u dSn^T), four columns
        float p = 0.f, pk = 0.f;
        if (r < nrow) {
          const uint2 w = *reinterpret_cast<const uint2*>(qh + (size_t)(t0 + r) * DK + d0);
          const uint2 x = *reinterpret_cast<const uint2*>(kh + (size_t)(t0 + r) * DK + d0);
          const float qv[4] = {bf2f((bf16_t)(w.x & 0xffffu)), bf2f((bf16_t)(w.x >> 16)), bf2f((bf16_t)(w.y & 0xffffu)),
                               bf2f((bf16_t)(w.y >> 16))};
          const float kv[4] = {bf2f((bf16_t)(x.x & 0xffffu)), bf2f((bf16_t)(x.x >> 16)), bf2f((bf16_t)(x.y & 0xffffu)),
                               bf2f((bf16_t)(x.y >> 16))};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p += qv[i] * q1[i];
            pk += kv[i] * k1[i];
          }
          // on the last row (e2 = 1) the term cancels against its share of
          // the chunk sum: both are left out
          pk = r < nrow - 1 ? e2 * pk : 0.f;
          p = e1 * p - pk;
        }
        p = xsum32(xsum16(p));
        if (lg == 0) atomicAdd(&sDG[r], p);
        // the same k . (u dSn^T) terms summed over the chunk, on its last row
        pk = sum64(pk);
        if (lane == 0) atomicAdd(&sDG[nrow - 1], pk);
      }
      continue;
    }
    const floatx4 q1 = rowrow<kBf16>(zero4(), sDO + (16 * ti + lc) * LV, sS + (16 * tk + lc) * LS, DV, lane);
    const floatx4 k1 = rowrow<kBf16>(zero4(), sU + (16 * ti + lc) * LV, sDS + (16 * tk + lc) * LS, DV, lane);
    const floatx4 k2 = rowrow<kBf16>(zero4(), sDX + (16 * ti + lc) * LV, sS + (16 * tk + lc) * LS, DV, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * ti + 4 * lg + i, d = 16 * tk + lc;
      const float e1 = GATE ? __expf(sG[r]) : 1.f, e2 = GATE ? __expf(sG[63] - sG[r]) : 1.f;
      const float dqv = gq[n][i] + e1 * q1[i];
      if (r < nrow) {
        dqo[(size_t)r * DK + d] = E::cvt(dqv);
        dko[(size_t)r * DK + d] = E::cvt(gk[n][i] + e2 * k1[i] - sB[r] * e1 * k2[i]);
      }
      if constexpr (GATE) {  // exp(G_r) q . (dO S^T) - exp(G_C - G_r) k . (u dSn^T), 16 columns
        float p = 0.f, pk = 0.f;
        if (r < nrow) {  // the last row's own term and its share of the chunk sum cancel
          pk = r < nrow - 1 ? e2 * E::tof(kh[(size_t)(t0 + r) * DK + d]) * k1[i] : 0.f;
          p = e1 * E::tof(qh[(size_t)(t0 + r) * DK + d]) * q1[i] - pk;
        }
        p = sum16(p);
        if (lc == 0) atomicAdd(&sDG[r], p);
        pk = sum64(pk);
        if (lane == 0) atomicAdd(&sDG[nrow - 1], pk);
      }
    }
  }
  if (tid < nrow) reinterpret_cast<T*>(a.dbeta)[(size_t)bh * Tn + t0 + tid] = E::cvt(sDB[tid]);
  if constexpr (KDA) {  // dg_t = sum of dG_r over r >= t, plus the decay's part through Gam_C
    __syncthreads();
    bf16_t* dgo = reinterpret_cast<bf16_t*>(a.dg) + ((size_t)bh * Tn + t0) * DK;
#pragma unroll
    for (int n = 0; n < NOWN; ++n) {
      const int id = wave + NW * n, ti = id / NKT, tk = id - ti * NKT;
      if (NTILE % NW != 0 && id >= NTILE) continue;
      const int r = 16 * ti + lc, d0 = 16 * tk + 4 * lg;
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[i] = dsuf[n][i] + sCC[d0 + i];
        for (int t2 = ti + 1; t2 < 4; ++t2) v[i] += sTotD[t2 * DK + d0 + i];
      }
      if (r < nrow) st4_bf16(dgo + (size_t)r * DK + d0, v[0], v[1], v[2], v[3]);
    }
  }
  if constexpr (GATE) {  // dg_t: the sums of dG_r over r >= t in the chunk
    __syncthreads();
    if (wave == 0) {
      float x = lane < nrow ? sDG[lane] : 0.f;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_down(x, off, 64);
        if (lane + off < 64) x += o;
      }
      if (lane < nrow) reinterpret_cast<T*>(a.dg)[(size_t)bh * Tn + t0 + lane] = E::cvt(x);
    }
  }
}

// ---------------------------------------------------------------------------
// KDA, a chunk whose decay leaves the factored form's range: the gradients
// by the recurrence itself, token by token and backwards.  Per token t, with
// S' = diag(a_t) S_{t-1}, r = S'^T k_t, u = beta_t (v_t - r),
// S_t = S' + k_t u^T, o_t = S_t^T q_t, and dS the gradient of S_t from the
// tokens after it (dSn for the chunk's last token):
//   dS += q_t dO_t^T;  dq_t = S_t dO_t;  du = dS^T k_t;
//   dk_t = dS u - beta_t S' du;  dv_t = beta_t du;  dbeta_t = du . (v_t - r);
//   dS' = dS - beta_t k_t du^T;  dg_t = rowsum(dS' * S');  dS <- diag(a_t) dS'.
// S_{t-1} is formed again from the chunk's entry state for every t (64
// dependent steps at most, no per-token states kept).  One workgroup per
// chunk; wave w < dv/16 holds 16 value columns of S and dS (rows 16 kt +
// 4 lg + i, column 16 w + lc); the sums over value columns go through LDS.
// ---------------------------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(512) void kda_walk_grads(BackwardArgs a, const bf16_t* __restrict__ Sc,
                                                      const bf16_t* __restrict__ dSc, KdaPtrs kp) {
  constexpr int NKT = DK / 16, NVW = DV / 16, LQ = DK + 8, LV = DV + 8, NRED = 3 * DK + 1;
  __shared__ __attribute__((aligned(16))) bf16_t sq[kC][LQ];
  __shared__ __attribute__((aligned(16))) bf16_t sk[kC][LQ];
  __shared__ __attribute__((aligned(16))) float sa[kC][DK];  // e^g
  __shared__ __attribute__((aligned(16))) bf16_t sv[kC][LV];
  __shared__ __attribute__((aligned(16))) bf16_t sdo[kC][LV];
  __shared__ float sb[kC];
  __shared__ float red[NVW][NRED];
  const size_t chunk = blockIdx.x;
  if (!(kp.gc[chunk * DK] < 0.f)) return;  // factored chunks are done elsewhere (uniform)
  const int Tn = a.T, nch = (Tn + kC - 1) / kC;
  const int bh = (int)(chunk / nch), t0 = (int)(chunk - (size_t)bh * nch) * kC, nrow = min(kC, Tn - t0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lc = lane & 15, lg = lane >> 4;
  // stage the chunk: raw q, k, g from the pre-pass's slots (zero past the end)
  const size_t tb = chunk * kC * DK;
  for (int i = tid; i < kC * DK; i += 512) {
    const int r = i / DK, d = i - r * DK;
    sq[r][d] = kp.qt[tb + i];
    sk[r][d] = kp.kt[tb + i];
    sa[r][d] = __expf(bf2f(kp.kht[tb + i]));
  }
  const bf16_t* vh = reinterpret_cast<const bf16_t*>(a.v) + ((size_t)bh * Tn + t0) * DV;
  const bf16_t* doh = reinterpret_cast<const bf16_t*>(a.dO) + ((size_t)bh * Tn + t0) * DV;
  for (int i = tid; i < kC * DV; i += 512) {
    const int r = i / DV, d = i - r * DV;
    sv[r][d] = r < nrow ? vh[(size_t)r * DV + d] : f2bf(0.f);
    sdo[r][d] = r < nrow ? doh[(size_t)r * DV + d] : f2bf(0.f);
  }
  if (tid < kC) sb[tid] = tid < nrow ? bf2f(reinterpret_cast<const bf16_t*>(a.beta)[(size_t)bh * Tn + t0 + tid]) : 0.f;
  __syncthreads();
  const bool act = wave < NVW;
  const int col = 16 * wave + lc;
  float s0[NKT][4], ds[NKT][4];  // entry state and the running gradient (tile order in Sc, dSc)
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    const size_t o = chunk * DK * DV + ((size_t)kt * NVW + (act ? wave : 0)) * 256 + 4 * lane;
    const uint2 w0 = *reinterpret_cast<const uint2*>(Sc + o);
    const uint2 w1 = *reinterpret_cast<const uint2*>(dSc + o);
    s0[kt][0] = bf2f((bf16_t)(w0.x & 0xffffu));
    s0[kt][1] = bf2f((bf16_t)(w0.x >> 16));
    s0[kt][2] = bf2f((bf16_t)(w0.y & 0xffffu));
    s0[kt][3] = bf2f((bf16_t)(w0.y >> 16));
    ds[kt][0] = bf2f((bf16_t)(w1.x & 0xffffu));
    ds[kt][1] = bf2f((bf16_t)(w1.x >> 16));
    ds[kt][2] = bf2f((bf16_t)(w1.y & 0xffffu));
    ds[kt][3] = bf2f((bf16_t)(w1.y >> 16));
  }
  // one forward step of token tau on x (a wave's 16 columns); returns r and
  // leaves S' in sp when asked
  auto step = [&](float (&x)[NKT][4], int tau, float (*sp)[4]) {
    float r = 0.f;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ch = 16 * kt + 4 * lg + i;
        x[kt][i] *= sa[tau][ch];
        if (sp) sp[kt][i] = x[kt][i];
        r += bf2f(sk[tau][ch]) * x[kt][i];
      }
    r = xsum32(xsum16(r));
    const float u = sb[tau] * (bf2f(sv[tau][col]) - r);
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[kt][i] += bf2f(sk[tau][16 * kt + 4 * lg + i]) * u;
    return r;
  };
  bf16_t* dqo = reinterpret_cast<bf16_t*>(a.dq) + ((size_t)bh * Tn + t0) * DK;
  bf16_t* dko = reinterpret_cast<bf16_t*>(a.dk) + ((size_t)bh * Tn + t0) * DK;
  bf16_t* dgo = reinterpret_cast<bf16_t*>(a.dg) + ((size_t)bh * Tn + t0) * DK;
  bf16_t* dvo = reinterpret_cast<bf16_t*>(a.dv) + ((size_t)bh * Tn + t0) * DV;
  for (int tau = nrow - 1; tau >= 0; --tau) {
    if (act) {
      float x[NKT][4], sp[NKT][4];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) x[kt][i] = s0[kt][i];
      for (int s2 = 0; s2 < tau; ++s2) step(x, s2, nullptr);
      const float r = step(x, tau, sp);  // x = S_tau, sp = S'
      const float u = sb[tau] * (bf2f(sv[tau][col]) - r);
      const float dOj = bf2f(sdo[tau][col]);
      float du = 0.f;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * kt + 4 * lg + i;
          ds[kt][i] += bf2f(sq[tau][ch]) * dOj;
          du += bf2f(sk[tau][ch]) * ds[kt][i];
        }
      du = xsum32(xsum16(du));
      const float bt = sb[tau];
      if (lg == 0) dvo[(size_t)tau * DV + col] = f2bf(bt * du);
      float pb = lg == 0 ? du * (bf2f(sv[tau][col]) - r) : 0.f;
      pb = sum16(pb);
      if (lane == 0) red[wave][3 * DK] = pb;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int ch = 16 * kt + 4 * lg + i;
          float pk = ds[kt][i] * u - bt * sp[kt][i] * du;               // dk partial
          const float dsp = ds[kt][i] - bt * bf2f(sk[tau][ch]) * du;    // dS'
          float pg = dsp * sp[kt][i];                                   // dg partial
          float p1 = x[kt][i] * dOj;                                    // dq partial
          p1 = sum16(p1);
          pk = sum16(pk);
          pg = sum16(pg);
          if (lc == 0) {
            red[wave][ch] = p1;
            red[wave][DK + ch] = pk;
            red[wave][2 * DK + ch] = pg;
          }
          ds[kt][i] = sa[tau][ch] * dsp;
        }
    }
    __syncthreads();
    for (int i = tid; i < NRED; i += 512) {
      float t = 0.f;
#pragma unroll
      for (int w2 = 0; w2 < NVW; ++w2) t += red[w2][i];
      if (i < DK) dqo[(size_t)tau * DK + i] = f2bf(t);
      else if (i < 2 * DK) dko[(size_t)tau * DK + i - DK] = f2bf(t);
      else if (i < 3 * DK) dgo[(size_t)tau * DK + i - 2 * DK] = f2bf(t);
      else reinterpret_cast<bf16_t*>(a.dbeta)[(size_t)bh * Tn + t0 + tau] = f2bf(t);
    }
    __syncthreads();
  }
}

template <int DK, int DV, class E, bool GATE>
hipError_t launch_grads(const BackwardArgs& a, const float* Sc, const float* dSc, long nchunks,
                        hipStream_t st) {
  static_assert(GradLayout<DK, DV, E, GATE>::total <= 160 * 1024, "backward gradient kernel exceeds the LDS of a CU");
  hipLaunchKernelGGL((bwd_grads<DK, DV, E, GATE>), dim3((unsigned)nchunks), dim3(kGradThreads), 0, st, a, Sc, dSc);
  return hipGetLastError();
}

template <int DK, class E, bool GATE>
hipError_t launch_grads_dk(const BackwardArgs& a, const float* Sc, const float* dSc, long nchunks,
                           hipStream_t st) {
  switch (a.dv_) {
    case 16: return launch_grads<DK, 16, E, GATE>(a, Sc, dSc, nchunks, st);
    case 32: return launch_grads<DK, 32, E, GATE>(a, Sc, dSc, nchunks, st);
    case 64: return launch_grads<DK, 64, E, GATE>(a, Sc, dSc, nchunks, st);
    case 128:
      if constexpr (sizeof(typename E::T) == 2) return launch_grads<DK, 128, E, GATE>(a, Sc, dSc, nchunks, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int DK, class E, bool GATE>
hipError_t launch_chain_dk(const BackwardArgs& a, float* dSc, hipStream_t st) {
  const long bh = (long)a.B * a.H;
  if (a.dv_ % 32 == 0) {
    hipLaunchKernelGGL((bwd_chain<DK, E, 32, GATE>), dim3((unsigned)(bh * (a.dv_ / 32))), dim3(kChainThreads), 0, st,
                       a, dSc);
  } else {
    hipLaunchKernelGGL((bwd_chain<DK, E, 16, GATE>), dim3((unsigned)(bh * (a.dv_ / 16))), dim3(kChainThreads), 0, st,
                       a, dSc);
  }
  return hipGetLastError();
}

// bf16: P and R for every chunk, then the one-product chain
template <int DK, bool GATE>
hipError_t launch_chain_mat(const BackwardArgs& a, bf16_t* Pg, bf16_t* Rg, float* dSc, float* gC, hipStream_t st) {
  bf16_t* dSt = reinterpret_cast<bf16_t*>(dSc);  // bf16 tile order (see bwd_chain_mat)
  static_assert(TransLayout<DK>::total <= 80 * 1024, "two transition workgroups should fit a CU");
  const long nchunks = (long)a.B * a.H * ((a.T + kC - 1) / kC);
  hipLaunchKernelGGL((bwd_transition<DK, GATE>), dim3((unsigned)nchunks), dim3(kTransThreads), 0, st, a, Pg, Rg, gC);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long bh = (long)a.B * a.H;
  if (a.dv_ % 32 == 0)
    hipLaunchKernelGGL((bwd_chain_mat<DK, 32, GATE>), dim3((unsigned)(bh * (a.dv_ / 32))), dim3(DK * 4), 0, st, a, Pg,
                       Rg, dSt, gC);
  else
    hipLaunchKernelGGL((bwd_chain_mat<DK, 16, GATE>), dim3((unsigned)(bh * (a.dv_ / 16))), dim3(DK * 4), 0, st, a, Pg,
                       Rg, dSt, gC);
  return hipGetLastError();
}

// gC: exp(G_C) of every chunk (gated rule, bf16)
template <class E, bool GATE>
hipError_t launch_backward_e(const BackwardArgs& a, float* Sc, float* dSc, bf16_t* Pg, bf16_t* Rg, float* gC,
                             hipStream_t st) {
  const long nchunks = (long)a.B * a.H * ((a.T + kC - 1) / kC);
  hipError_t e;
  constexpr bool kB = sizeof(typename E::T) == 2;
  switch (a.dk_) {
    case 16: e = kB ? launch_chain_mat<16, GATE>(a, Pg, Rg, dSc, gC, st) : launch_chain_dk<16, E, GATE>(a, dSc, st); break;
    case 32: e = kB ? launch_chain_mat<32, GATE>(a, Pg, Rg, dSc, gC, st) : launch_chain_dk<32, E, GATE>(a, dSc, st); break;
    case 64: e = kB ? launch_chain_mat<64, GATE>(a, Pg, Rg, dSc, gC, st) : launch_chain_dk<64, E, GATE>(a, dSc, st); break;
    case 128:
      if constexpr (kB) {
        e = launch_chain_mat<128, GATE>(a, Pg, Rg, dSc, gC, st);
        break;
      }
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  switch (a.dk_) {
    case 16: return launch_grads_dk<16, E, GATE>(a, Sc, dSc, nchunks, st);
    case 32: return launch_grads_dk<32, E, GATE>(a, Sc, dSc, nchunks, st);
    case 64: return launch_grads_dk<64, E, GATE>(a, Sc, dSc, nchunks, st);
    case 128:
      if constexpr (sizeof(typename E::T) == 2) return launch_grads_dk<128, E, GATE>(a, Sc, dSc, nchunks, st);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

// KDA (bf16): the transition and chain with a decay per key channel, then
// the gradients (factored chunks: bwd_grads; walked chunks: kda_walk_grads;
// each kernel leaves the other kind of chunk alone)
template <int DK, int DV>
hipError_t launch_kda_grads(const BackwardArgs& a, const bf16_t* Sc, const bf16_t* dSt, const KdaPtrs& kp,
                            long nchunks, hipStream_t st) {
  static_assert(GradLayout<DK, DV, BF16, false, true>::total <= 160 * 1024,
                "backward gradient kernel exceeds the LDS of a CU");
  hipLaunchKernelGGL((bwd_grads<DK, DV, BF16, false, true>), dim3((unsigned)nchunks), dim3(kGradThreads), 0, st, a,
                     reinterpret_cast<const float*>(Sc), reinterpret_cast<const float*>(dSt), kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((kda_walk_grads<DK, DV>), dim3((unsigned)nchunks), dim3(512), 0, st, a, Sc, dSt, kp);
  return hipGetLastError();
}

template <int DK>
hipError_t launch_kda_passes(const BackwardArgs& a, const bf16_t* Sc, bf16_t* dSt, bf16_t* Pg, bf16_t* Rg,
                             const KdaPtrs& kp, hipStream_t st) {
  static_assert(TransLayout<DK, true>::total <= 160 * 1024, "transition kernel exceeds the LDS of a CU");
  const long nchunks = (long)a.B * a.H * ((a.T + kC - 1) / kC);
  hipLaunchKernelGGL((bwd_transition<DK, false, true>), dim3((unsigned)nchunks), dim3(kTransThreads), 0, st, a, Pg, Rg,
                     static_cast<float*>(nullptr), kp);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long bh = (long)a.B * a.H;
  if (a.dv_ % 32 == 0)
    hipLaunchKernelGGL((bwd_chain_mat<DK, 32, false, true>), dim3((unsigned)(bh * (a.dv_ / 32))), dim3(DK * 4), 0, st,
                       a, Pg, Rg, dSt, kp.gc);
  else
    hipLaunchKernelGGL((bwd_chain_mat<DK, 16, false, true>), dim3((unsigned)(bh * (a.dv_ / 16))), dim3(DK * 4), 0, st,
                       a, Pg, Rg, dSt, kp.gc);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  switch (a.dv_) {
    case 16: return launch_kda_grads<DK, 16>(a, Sc, dSt, kp, nchunks, st);
    case 32: return launch_kda_grads<DK, 32>(a, Sc, dSt, kp, nchunks, st);
    case 64: return launch_kda_grads<DK, 64>(a, Sc, dSt, kp, nchunks, st);
    case 128: return launch_kda_grads<DK, 128>(a, Sc, dSt, kp, nchunks, st);
    default: return hipErrorInvalidValue;
  }
}

__global__ __launch_bounds__(256) void zero_state(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.f;
}

bool pass1_pipelined(int bf16, const BackwardArgs& a) { return bf16 && a.dk_ == 128 && a.dv_ % 32 == 0; }

}  // namespace

// Workspace layout: see delta_backward_workspace_bytes (launch.hpp).
hipError_t launch_delta_backward(int bf16, const BackwardArgs& a, void* workspace, hipStream_t st) {
  if (a.T == 0) {  // no tokens: the state's gradient passes through
    if (!a.dS0) return hipSuccess;
    const size_t n = (size_t)a.B * a.H * a.dk_ * a.dv_;
    if (a.dST) return hipMemcpyAsync(a.dS0, a.dST, n * sizeof(float), hipMemcpyDeviceToDevice, st);
    const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(zero_state, dim3((unsigned)blocks), dim3(256), 0, st, a.dS0, n);
    return hipGetLastError();
  }
  const size_t nchunks = (size_t)a.B * a.H * ((a.T + kC - 1) / kC);
  const size_t nst = nchunks * a.dk_ * a.dv_;
  char* ws = static_cast<char*>(workspace);
  float* Sc = reinterpret_cast<float*>(ws);
  ws += workspace_round256(nst * sizeof(float));
  float* dSc = reinterpret_cast<float*>(ws);
  ws += workspace_round256(nst * sizeof(float));
  float* gC = nullptr;
  if (a.g) {
    gC = reinterpret_cast<float*>(ws);
    ws += workspace_round256(nchunks * sizeof(float));
  }
  bf16_t* Pg = bf16 ? reinterpret_cast<bf16_t*>(ws) : nullptr;
  bf16_t* Rg = bf16 ? Pg + nchunks * a.dk_ * a.dk_ : nullptr;
  // pass 1: the state entering every chunk, from a forward kernel that
  // writes only those (no output, no final state; S0 is only read)
  PrefillArgs f{};
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.beta = a.beta;
  f.g = a.g;
  f.S = const_cast<float*>(a.S0);
  f.B = a.B;
  f.H = a.H;
  f.T = a.T;
  f.dv = a.dv_;
  f.use_init = a.S0 != nullptr;
  f.Sc = Sc;
  hipError_t e;
  if (pass1_pipelined(bf16, a))
    e = a.g ? launch_prefill_pipe_token(f, st) : launch_prefill_pipe(f, nullptr, st);
  else
    e = launch_prefill_generic(a.g ? PF_SGATED : PF_DELTA, bf16, a.dk_, f, st);
  // passes 2 and 3
  if (e == hipSuccess) {
    if (a.g)
      e = bf16 ? launch_backward_e<BF16, true>(a, Sc, dSc, Pg, Rg, gC, st)
               : launch_backward_e<F32, true>(a, Sc, dSc, Pg, Rg, gC, st);
    else
      e = bf16 ? launch_backward_e<BF16, false>(a, Sc, dSc, Pg, Rg, gC, st)
               : launch_backward_e<F32, false>(a, Sc, dSc, Pg, Rg, gC, st);
  }
  return e;
}

// Workspace layout: see kda_backward_workspace_bytes (launch.hpp).
hipError_t launch_kda_backward(const BackwardArgs& a, void* workspace, hipStream_t st) {
  if (a.T == 0) {  // no tokens: the state's gradient passes through
    if (!a.dS0) return hipSuccess;
    const size_t n = (size_t)a.B * a.H * a.dk_ * a.dv_;
    if (a.dST) return hipMemcpyAsync(a.dS0, a.dST, n * sizeof(float), hipMemcpyDeviceToDevice, st);
    const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(zero_state, dim3((unsigned)blocks), dim3(256), 0, st, a.dS0, n);
    return hipGetLastError();
  }
  const size_t nchunks = workspace_chunks(a.B, a.H, a.T);
  const size_t ntile = nchunks * kC * a.dk_;
  char* ws = static_cast<char*>(workspace);
  char* prep = ws;
  ws += workspace_round256(gate_prep_bytes(a.dk_, a.B, a.H, a.T));
  bf16_t* Sc = reinterpret_cast<bf16_t*>(ws);
  ws += workspace_round256(nchunks * a.dk_ * a.dv_ * sizeof(bf16_t));
  bf16_t* dSt = reinterpret_cast<bf16_t*>(ws);
  ws += workspace_round256(nchunks * a.dk_ * a.dv_ * sizeof(bf16_t));
  bf16_t* Pg = reinterpret_cast<bf16_t*>(ws);
  bf16_t* Rg = Pg + nchunks * a.dk_ * a.dk_;
  KdaPtrs kp{};
  kp.qt = reinterpret_cast<const bf16_t*>(prep);
  kp.kt = kp.qt + ntile;
  kp.kht = kp.kt + ntile;
  kp.gc = reinterpret_cast<const float*>(kp.kht + ntile);
  // the gate pre-pass, then pass 1: the state entering every chunk (no
  // output, no final state; S0 is only read)
  PrefillArgs f{};
  f.q = a.q;
  f.k = a.k;
  f.v = a.v;
  f.beta = a.beta;
  f.g = a.g;
  f.S = const_cast<float*>(a.S0);
  f.B = a.B;
  f.H = a.H;
  f.T = a.T;
  f.dv = a.dv_;
  f.use_init = a.S0 != nullptr;
  f.Sc = reinterpret_cast<float*>(Sc);
  hipError_t e = launch_gate_prep(a.dk_, f, prep, st);
  if (e != hipSuccess) return e;
  if (a.dk_ == 128 && a.dv_ % 32 == 0)
    e = launch_prefill_pipe_prepped(f, prep, st);
  else
    e = launch_prefill_generic(PF_GATED, 1, a.dk_, f, st);
  if (e != hipSuccess) return e;
  switch (a.dk_) {
    case 16: return launch_kda_passes<16>(a, Sc, dSt, Pg, Rg, kp, st);
    case 32: return launch_kda_passes<32>(a, Sc, dSt, Pg, Rg, kp, st);
    case 64: return launch_kda_passes<64>(a, Sc, dSt, Pg, Rg, kp, st);
    case 128: return launch_kda_passes<128>(a, Sc, dSt, Pg, Rg, kp, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace linattn

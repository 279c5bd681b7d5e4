// prefill.hip -- chunkwise prefill of causal linear attention with a fixed
// dk x dv fp32 state: ELU+1 linear attention with normaliser, the delta rule,
// the gated delta rule (decay per key channel or per token), and gated
// linear attention (additive cache with a per-token forgetting factor).
//
// Method (article "From GPT-2 to Kimi K3, explained"):
//  * section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)":
//    the sequence is cut into chunks of C = 64 tokens; inside a chunk the
//    masked product tril(Q K^T) is formed directly, across chunks everything
//    is folded into the state S.  For the delta rule the chunk's corrections
//    come from the UT/WY form: with L = tril(diag(beta) K K^T, -1) and
//    T = (I + L)^{-1},  u = T diag(beta) (V - K S),  O = Q S + tril(Q K^T) u,
//    S <- S + K^T u.  (The article forms W = T diag(beta) K and U = T diag(beta) V
//    first; u = U - W S is the same quantity.)
//  * section "Linear Attention": phi(x) = elu(x) + 1 on q and k, and the
//    output divided by phi(q).z; chunkwise the denominator is
//    phi(Q) z + rowsum(tril(phi(Q) phi(K)^T)), and z += sum of phi(k).
//  * sections "Gated Delta Net" and "KDA / Kimi Linear": a decay per key
//    channel applied to S before each read.  Within a chunk, with the
//    cumulative decay Gam_t = prod_{s<=t} a_s (per channel, from the chunk
//    start) -- the article's gamma^r / gamma^i ratios -- the same UT/WY form
//    holds with K~ = Gam*K, K^ = K/Gam, Q~ = Gam*Q:
//      L = tril(diag(beta) K~ K^^T, -1), u = T diag(beta) (V - K~ S),
//      O = Q~ S + tril(Q~ K^^T) u,  S <- diag(Gam_C) S + (K*Gam_C/Gam)^T u.
//  * one decay per token (section "Gated Delta Net"): with G_t the summed
//    log-decay from the chunk start, the same products are formed from the
//    plain Q and K, and each entry (r, c) of tril(Q K^T) and L is scaled by
//    exp(G_r - G_c) <= 1; the rows of Q S and K S by exp(G_r); the state by
//    exp(G_C) and the rows of u by exp(G_C - G_r) before S += K^T u.  No
//    factor exceeds 1, so any decay is representable.
//  * section "Gated Delta Net", first step: the additive cache with a
//    forgetting factor, S <- a_t S + k^T v, o = q S (q, k as given).  It is
//    the per-token gated form with u = V: no beta, no L, no normaliser.
//
// Mapping to gfx950.  One workgroup (4 waves) owns one (batch, head) and a
// slice of DVS value columns (32, or 16 when dv = 16): the value columns of
// the state evolve independently given T and the chunk's keys, so slicing dv
// multiplies the number of independent serial chains.  Inside the workgroup
// NCW = DVS/16 "chain" waves each keep S[:, 16 columns] in MFMA accumulator
// registers for the whole sequence (fp32); the other waves form the
// S-independent products of the chunk.  The chain never moves S through LDS:
// an accumulator tile is used directly as the B operand of the next product
// (see device_common.hpp), so the serial work per chunk is five small MFMA
// contractions per chain wave.  Per chunk the whole 64-token tile of q, k and
// the slice of v are staged in LDS once.
#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {

constexpr int kC = 64;         // chunk length in tokens
constexpr int kThreads = 256;  // 4 waves
// Per-channel gate: the factored chunk form divides keys by the decay summed
// from the chunk start; a chunk where that sum leaves [-kGateRange,
// kGateRange] for some channel is computed token by token instead.
constexpr float kGateRange = 64.f;
constexpr int kWaves = kThreads / 64;

// kGate: decay per key channel, decayed operands (K~, K^, Q~) staged;
// kScal: one decay per token, applied to the products' entries and rows;
// kSolve: beta, L and T = (I + L)^-1 (the delta-rule modes).
template <int MODE>
struct ModeTraits {
  static constexpr bool kGate = MODE == PF_GATED;
  static constexpr bool kScal = MODE == PF_SGATED || MODE == PF_GLA;
  static constexpr bool kSolve = MODE == PF_DELTA || MODE == PF_GATED || MODE == PF_SGATED;
};

template <int DK, class E, int MODE, int DVS>
struct PrefillLayout {
  typedef typename E::T T;
  static constexpr bool kGate = ModeTraits<MODE>::kGate;
  static constexpr int PAD = 16 / (int)sizeof(T);  // one 16-byte vector of padding
  static constexpr int LQ = DK + PAD;               // row stride: sQ, sK, sKh
  static constexpr int LKT = kC + PAD;              // row stride: sKt, sVt, sA
  static constexpr int LTL = kC + 4;                // row stride: sTL (fp32)
  static constexpr int oQ = 0;
  static constexpr int oK = oQ + kC * LQ * (int)sizeof(T);
  static constexpr int oKh = oK + kC * LQ * (int)sizeof(T);
  static constexpr int oKt = oKh + (kGate ? kC * LQ * (int)sizeof(T) : 0);
  static constexpr int oVt = oKt + DK * LKT * (int)sizeof(T);
  static constexpr int oA = oVt + DVS * LKT * (int)sizeof(T);
  static constexpr int oTL = oA + kC * LKT * (int)sizeof(T);
  static constexpr int oRow = oTL + (ModeTraits<MODE>::kSolve ? kC * LTL * 4 : 0);  // beta or den
  static constexpr int oVec = oRow + kC * 4;                            // Gam_C or z
  static constexpr int oPart = oVec + DK * 4;                           // scan partials
  static constexpr int oG = oPart + (kGate ? kThreads * 4 : 0);         // per-token G_t
  static constexpr int total = oG + (ModeTraits<MODE>::kScal ? kC * 4 : 0);
};

// Workgroup i runs on XCD i % 8.  Give consecutive logical indices (the dv
// slices of one head, which read the same q and k) to one XCD so they share
// its L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if (n % 8 != 0) return bid;
  return (bid % 8) * (n / 8) + bid / 8;
}

__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <class E>
union VecU {
  Vec16 v;
  typename E::T e[E::kVec];
};

template <int DK, class E, int MODE, int DVS>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  typedef PrefillLayout<DK, E, MODE, DVS> L;
  typedef typename E::T T;
  constexpr bool kBf16 = sizeof(T) == 2;
  constexpr int kVec = E::kVec;
  constexpr int NCW = DVS / 16;  // chain waves
  constexpr int NKT = DK / 16;   // 16-row tiles of S per chain wave
  constexpr int LQ = L::LQ, LKT = L::LKT, LTL = L::LTL;
  constexpr bool kGate = ModeTraits<MODE>::kGate;
  constexpr bool kScal = ModeTraits<MODE>::kScal;
  constexpr bool kSolve = ModeTraits<MODE>::kSolve;

  __shared__ __attribute__((aligned(16))) char smem[L::total];
  __shared__ int sWide;  // per-channel gate: this chunk's decay leaves the factored form's range
  T* sQ = reinterpret_cast<T*>(smem + L::oQ);
  T* sK = reinterpret_cast<T*>(smem + L::oK);
  T* sKh = kGate ? reinterpret_cast<T*>(smem + L::oKh) : sK;
  T* sKt = reinterpret_cast<T*>(smem + L::oKt);
  T* sVt = reinterpret_cast<T*>(smem + L::oVt);
  T* sA = reinterpret_cast<T*>(smem + L::oA);
  float* sTL = reinterpret_cast<float*>(smem + L::oTL);
  float* sRow = reinterpret_cast<float*>(smem + L::oRow);  // beta (delta rule), or 1 / den (LA)
  float* sVec = reinterpret_cast<float*>(smem + L::oVec);  // Gam_C (gated) / z (LA)
  float* sPart = reinterpret_cast<float*>(smem + L::oPart);
  float* sG = reinterpret_cast<float*>(smem + L::oG);  // per-token modes: G_t

  const int nsl = a.dv / DVS;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / nsl;
  const int sl = w - bh * nsl;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int Tn = a.T;
  const int dv = a.dv;

  const T* qh = reinterpret_cast<const T*>(a.q) + (size_t)bh * Tn * DK;
  const T* kh = reinterpret_cast<const T*>(a.k) + (size_t)bh * Tn * DK;
  const T* vh = reinterpret_cast<const T*>(a.v) + (size_t)bh * Tn * dv + sl * DVS;
  const T* bth = reinterpret_cast<const T*>(a.beta) + (size_t)bh * Tn;
  // log-decay: [T][DK] per key channel, [T] per token, or none (gated
  // linear attention without a decay)
  const T* gh = a.g ? reinterpret_cast<const T*>(a.g) + (size_t)bh * Tn * (kGate ? DK : 1) : nullptr;
  T* oh = reinterpret_cast<T*>(a.o) + (size_t)bh * Tn * dv + sl * DVS;
  float* Sh = a.S + (size_t)bh * DK * dv + sl * DVS;

  for (int i = tid; i < kC * LKT; i += kThreads) sA[i] = E::cvt(0.f);
  if (MODE == PF_LA) {
    for (int d = tid; d < DK; d += kThreads) sVec[d] = a.use_init ? a.z[(size_t)bh * DK + d] : 0.f;
  }

  const bool chain = wave < NCW;
  const int cw = wave;
  floatx4 st[NKT];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt) {
    st[kt] = zero4();
    if (chain && a.use_init) {
#pragma unroll
      for (int i = 0; i < 4; ++i) st[kt][i] = Sh[(size_t)(16 * kt + 4 * lg + i) * dv + 16 * cw + lc];
    }
  }

  // A partial last chunk: loads past the last token re-read it, and the
  // staged rows past the end get k = 0, v = 0, beta = 0 and (gated) g = 0,
  // so they add nothing to the state, the normaliser or the outputs of the
  // tokens that exist; their own outputs are not stored.
  const int nchunks = (Tn + kC - 1) / kC;
  const int tlast = Tn - 1;

  // Non-gated modes: the chunk's q, k and v-slice vectors (and beta) are
  // loaded into registers one chunk ahead, so their latency overlaps the
  // previous chunk's work.  Thread tid owns vectors tid + kThreads j of the
  // chunk (q, then k, then v); every thread issues every load (a vector past
  // the end re-reads vector 0 and is not stored).
  constexpr int VPRQ = DK / kVec;          // 16-byte vectors per q/k row
  constexpr int NQV = kC * VPRQ;
  constexpr int VPRS = DVS / kVec;         // per row of the v slice
  constexpr int NTOT = 2 * NQV + kC * VPRS;
  constexpr int NPT = (NTOT + kThreads - 1) / kThreads;
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));  // a register array of
  u32x4v pre[kGate ? 1 : NPT];                        // structs would go to memory
  float preb = 0.f, preg = 0.f;
  auto prefetch = [&](int c) {
    if constexpr (!kGate) {
      const T* const pq = qh;
      const T* const pk = kh;
      const T* const pv = vh;
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int i0 = tid + kThreads * j;
        const int i = i0 < NTOT ? i0 : 0;
        const T* src;
        if (i < 2 * NQV) {
          const int ii = i < NQV ? i : i - NQV;
          src = (i < NQV ? pq : pk) + (size_t)min(c * kC + ii / VPRQ, tlast) * DK + (ii % VPRQ) * kVec;
        } else {
          const int ii = i - 2 * NQV;
          src = pv + (size_t)min(c * kC + ii / VPRS, tlast) * dv + (ii % VPRS) * kVec;
        }
        pre[j] = *reinterpret_cast<const u32x4v*>(src);
      }
      if (kSolve && tid < kC) preb = E::ld(bth + min(c * kC + tid, tlast));
      if (kScal && tid < kC) preg = gh ? E::ld(gh + min(c * kC + tid, tlast)) : 0.f;
    }
  };
  prefetch(0);

  for (int c = 0; c < nchunks; ++c) {
    const int t0 = c * kC;
    if (a.Sc && chain) {  // the state entering chunk c, for the backward pass
      // in the input type (the precision the gradient pass reads it in):
      // fp32 row-major; bf16 in accumulator-tile order (tile (kt, jt) of the
      // chunk at (kt * dv/16 + jt) * 256, lane l's four rows at 4l)
      typename E::T* sc = reinterpret_cast<typename E::T*>(a.Sc) + ((size_t)bh * nchunks + c) * DK * dv;
      if constexpr (sizeof(typename E::T) == 2) {
        const int jt = (sl * DVS + 16 * cw) / 16;
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
          *reinterpret_cast<uint2*>(sc + ((size_t)kt * (dv / 16) + jt) * 256 + 4 * lane) =
              make_uint2(pack2(st[kt][0], st[kt][1]), pack2(st[kt][2], st[kt][3]));
      } else {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) sc[(size_t)(16 * kt + 4 * lg + i) * dv + sl * DVS + 16 * cw + lc] = st[kt][i];
      }
    }
    __syncthreads();  // the previous chunk's readers of LDS are done

    // ---------------- stage the chunk in LDS ----------------
    if (!kGate) {
#pragma unroll
      for (int j = 0; j < NPT; ++j) {
        const int i = tid + kThreads * j;
        if (i >= NTOT) continue;
        if (i >= 2 * NQV) {  // v slice, stored transposed
          const int ii = i - 2 * NQV;
          const int r = ii / VPRS, cv = ii % VPRS;
          VecU<E> vv;
          vv.v = __builtin_bit_cast(Vec16, pre[j]);
          if (t0 + r > tlast) vv.v = Vec16{};
#pragma unroll
          for (int e = 0; e < kVec; ++e) sVt[(cv * kVec + e) * LKT + r] = vv.e[e];
          continue;
        }
        const bool isq = i < NQV;
        const int ii = isq ? i : i - NQV;
        const int r = ii / VPRQ, cv = ii % VPRQ;
        VecU<E> xv;
        xv.v = __builtin_bit_cast(Vec16, pre[j]);
        if (MODE == PF_LA) {
#pragma unroll
          for (int e = 0; e < kVec; ++e) xv.e[e] = E::cvt(phi_elu1(E::tof(xv.e[e])));
        }
        if (isq) {
          *reinterpret_cast<Vec16*>(sQ + r * LQ + cv * kVec) = xv.v;
        } else {
          if (t0 + r > tlast) xv.v = Vec16{};  // after the feature map: phi(0) = 1
          *reinterpret_cast<Vec16*>(sK + r * LQ + cv * kVec) = xv.v;
#pragma unroll
          for (int e = 0; e < kVec; ++e) sKt[(cv * kVec + e) * LKT + r] = xv.e[e];
        }
      }
      if (kSolve && tid < kC) sRow[tid] = t0 + tid <= tlast ? preb : 0.f;
      if (kScal && tid < kC) {
        // wave 0 (one lane per token): G_t = sum_{s<=t} g_s over the chunk
        sG[tid] = scan64_up(t0 + tid <= tlast ? preg : 0.f);
      }
      if (c + 1 < nchunks) prefetch(c + 1);
    }
    if (kGate) {
      // cumulative log-decay per key channel over the chunk, then the scaled
      // operands Q~ = Gam Q, K~ = Gam K, K^ = K / Gam, (K Gam_C / Gam)^T
      constexpr int NP = kThreads / DK;  // token parts
      constexpr int TPP = kC / NP;       // tokens per part
      const int d = tid % DK;
      const int part = tid / DK;
      float gl[TPP];
      float run = 0.f;
#pragma unroll
      for (int j = 0; j < TPP; ++j) {
        const int t = t0 + part * TPP + j;
        if (t <= tlast) run += E::ld(gh + (size_t)t * DK + d);
        gl[j] = run;
      }
      sPart[part * DK + d] = run;
      if (tid == 0) sWide = 0;
      __syncthreads();
      float off = 0.f, tot = 0.f;
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        const float x = sPart[p * DK + d];
        if (p < part) off += x;
        tot += x;
      }
      // K / Gam must stay in the float range: a chunk in which some channel's
      // summed log-decay leaves [-kGateRange, kGateRange] is walked token by
      // token instead, on raw q, k and g staged in the same places
      float mx = 0.f;
#pragma unroll
      for (int j = 0; j < TPP; ++j) mx = fmaxf(mx, fabsf(off + gl[j]));
      if (!(mx <= kGateRange)) sWide = 1;  // also for NaN
      __syncthreads();
      const bool wide = sWide != 0;
      if (part == 0) sVec[d] = __expf(tot);
#pragma unroll
      for (int j = 0; j < TPP; ++j) {
        const int r = part * TPP + j;
        const float G = off + gl[j];
        const bool in = t0 + r <= tlast;
        const float qv = in ? E::ld(qh + (size_t)(t0 + r) * DK + d) : 0.f;
        const float kv = in ? E::ld(kh + (size_t)(t0 + r) * DK + d) : 0.f;
        if (wide) {
          const float gv = in ? E::ld(gh + (size_t)(t0 + r) * DK + d) : 0.f;
          sQ[r * LQ + d] = E::cvt(qv);
          sK[r * LQ + d] = E::cvt(kv);
          sKh[r * LQ + d] = E::cvt(gv);
        } else {
          const float eg = __expf(G), emg = __expf(-G), dec = __expf(tot - G);
          sQ[r * LQ + d] = E::cvt(qv * eg);
          sK[r * LQ + d] = E::cvt(kv * eg);
          sKh[r * LQ + d] = E::cvt(kv * emg);
          sKt[d * LKT + r] = E::cvt(kv * dec);
        }
      }
    }
    if (kGate) {
      constexpr int VPRV = DVS / kVec;
      for (int i = tid; i < kC * VPRV; i += kThreads) {
        const int r = i / VPRV, cv = i - (i / VPRV) * VPRV;
        VecU<E> vv;
        vv.v = t0 + r <= tlast ? *reinterpret_cast<const Vec16*>(vh + (size_t)(t0 + r) * dv + cv * kVec) : Vec16{};
#pragma unroll
        for (int e = 0; e < kVec; ++e) sVt[(cv * kVec + e) * LKT + r] = vv.e[e];
      }
      if (kSolve && tid < kC) sRow[tid] = t0 + tid <= tlast ? E::ld(bth + t0 + tid) : 0.f;
    }
    __syncthreads();
    if (kGate && sWide) {
      // the recurrence itself, token by token, S <- diag(a_t) S, u = beta_t
      // (v_t - k_t S), S += k_t^T u, o_t = q_t S: lane (lc, lg) of a chain
      // wave holds column 16cw + lc of rows (key channels) 16kt + 4lg + i;
      // sums over channels are completed across the four lanes of a column
      if (chain) {
        for (int tau = 0; tau < kC; ++tau) {
          float kk[NKT][4], qq[NKT][4];
          float r = 0.f;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int ch = 16 * kt + 4 * lg + i;
              kk[kt][i] = E::tof(sK[tau * LQ + ch]);
              qq[kt][i] = E::tof(sQ[tau * LQ + ch]);
              st[kt][i] *= __expf(E::tof(sKh[tau * LQ + ch]));
              r += kk[kt][i] * st[kt][i];
            }
          r = xsum32(xsum16(r));
          const float u = sRow[tau] * (E::tof(sVt[(16 * cw + lc) * LKT + tau]) - r);
          float o = 0.f;
#pragma unroll
          for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              st[kt][i] += kk[kt][i] * u;
              o += qq[kt][i] * st[kt][i];
            }
          o = xsum32(xsum16(o));
          if (lg == 0 && !a.Sc && t0 + tau <= tlast) oh[(size_t)(t0 + tau) * dv + 16 * cw + lc] = E::cvt(o);
        }
      }
      continue;  // uniform over the workgroup
    }

    // -------- chain waves: products with the incoming state; others: the
    // -------- chunk's pairwise products
    floatx4 ox[4], xx[4];
    if (chain) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const T* qrow = sQ + (16 * mt + lc) * LQ;
        if constexpr (kBf16) ox[mt] = mm_accB_bf16(zero4(), qrow, st, NKT, lane);
        else ox[mt] = mm_accB_f32(zero4(), qrow, st, NKT, lane);
        const T* vp = sVt + (16 * cw + lc) * LKT + 16 * mt + 4 * lg;
        floatx4 vv;
#pragma unroll
        for (int i = 0; i < 4; ++i) vv[i] = E::tof(vp[i]);
        floatx4 dec = {1.f, 1.f, 1.f, 1.f};  // per-token decay exp(G_r) of rows r
        if constexpr (kScal) {
#pragma unroll
          for (int i = 0; i < 4; ++i) dec[i] = __expf(sG[16 * mt + 4 * lg + i]);
#pragma unroll
          for (int i = 0; i < 4; ++i) ox[mt][i] *= dec[i];
        }
        if (!kSolve) {
          xx[mt] = vv;
        } else {
          const T* krow = sK + (16 * mt + lc) * LQ;
          floatx4 y;
          if constexpr (kBf16) y = mm_accB_bf16(zero4(), krow, st, NKT, lane);
          else y = mm_accB_f32(zero4(), krow, st, NKT, lane);
#pragma unroll
          for (int i = 0; i < 4; ++i) xx[mt][i] = sRow[16 * mt + 4 * lg + i] * (vv[i] - dec[i] * y[i]);
        }
      }
    } else {
      // jobs 0..9: tiles (i, j<=i) of tril(Q K^^T) -> sA
      // jobs 10..19: tiles (i, j<=i) of K~ K^^T -> L = beta_row * (.) strictly
      //              below the diagonal, stored transposed in sTL's upper part
      const int njobs = kSolve ? 20 : 10;
      for (int jb = wave - NCW; jb < njobs; jb += kWaves - NCW) {
        const bool isA = jb < 10;
        const int t = isA ? jb : jb - 10;
        const int ti = t >= 6 ? 3 : t >= 3 ? 2 : t >= 1 ? 1 : 0;
        const int tj = t - ti * (ti + 1) / 2;
        const T* left = (isA ? sQ : sK) + (16 * ti + lc) * LQ;
        const T* right = sKh + (16 * tj + lc) * LQ;
        floatx4 acc;
        if constexpr (kBf16) acc = mm_rowrow_bf16(zero4(), left, right, DK, lane);
        else acc = mm_rowrow_f32(zero4(), left, right, DK, lane);
        const int cc = 16 * tj + lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * ti + 4 * lg + i;
          float x = acc[i];
          if constexpr (kScal) x *= cc <= r ? __expf(sG[r] - sG[cc]) : 0.f;  // decay from c to r
          if (isA) sA[r * LKT + cc] = E::cvt(cc <= r ? x : 0.f);
          else if (cc < r) sTL[cc * LTL + r] = sRow[r] * x;
        }
      }
    }
    __syncthreads();

    if (MODE == PF_LA) {
      // denominators phi(Q) z + rowsum(tril(phi(Q) phi(K)^T)), then z += sum phi(k)
      // (lane = row r; 16-byte row reads of phi(Q), tril(.) and phi(K)^T)
      if (wave == NCW) {
        float den0 = 0.f, den1 = 0.f;
#pragma unroll
        for (int d8 = 0; d8 < DK; d8 += kVec) {
          VecU<E> x;
          x.v = *reinterpret_cast<const Vec16*>(sQ + lane * LQ + d8);
#pragma unroll
          for (int e = 0; e < kVec; ++e) den0 += E::tof(x.e[e]) * sVec[d8 + e];
        }
#pragma unroll
        for (int c8 = 0; c8 < kC; c8 += kVec) {
          VecU<E> x;
          x.v = *reinterpret_cast<const Vec16*>(sA + lane * LKT + c8);
#pragma unroll
          for (int e = 0; e < kVec; ++e) den1 += E::tof(x.e[e]);
        }
        float zs[DK > 64 ? 2 : 1];
#pragma unroll
        for (int h = 0; h * 64 < DK; ++h) {
          const int d = lane + 64 * h;
          float acc = 0.f;
          if (d < DK) {
#pragma unroll
            for (int r8 = 0; r8 < kC; r8 += kVec) {
              VecU<E> x;
              x.v = *reinterpret_cast<const Vec16*>(sKt + d * LKT + r8);
#pragma unroll
              for (int e = 0; e < kVec; ++e) acc += E::tof(x.e[e]);
            }
          }
          zs[h] = acc;
        }
        // every lane has read z (sVec) before it is updated: one wave, LDS
        // operations in program order
        sRow[lane] = 1.f / (den0 + den1);  // reciprocal: one division per row
#pragma unroll
        for (int h = 0; h * 64 < DK; ++h)
          if (lane + 64 * h < DK) sVec[lane + 64 * h] += zs[h];
      }
      __syncthreads();
    } else if constexpr (kSolve) {
      // T = (I + L)^{-1}.  Diagonal 16x16 blocks by forward substitution (one
      // lane per column), then off-diagonal blocks block-row by block-row:
      // T[bi][bj] = -T[bi][bi] * sum_{bj<=m<bi} L[bi][m] T[m][bj].
      // T is stored row-major in the lower triangle of sTL (diagonal included).
      if (wave == kWaves - 1) {
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
              av[e] = sTL[(16 * m + kk) * LTL + 16 * bi + lc];  // L[16bi+lc][16m+kk]
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
            tv[e] = kk <= lc ? sTL[(16 * bi + lc) * LTL + 16 * bi + kk] : 0.f;  // T[16bi+lc][16bi+kk]
          }
          floatx4 Y = zero4();
          if constexpr (kBf16) {
            Y = mfma_k16(words_to_shortx4(pack2(tv[0], tv[1]), pack2(tv[2], tv[3])),
                         acc_to_b16(R), Y);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) Y = mfma_f32(tv[e], R[e], Y);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sTL[(16 * bi + 4 * lg + i) * LTL + 16 * bj + lc] = -Y[i];
        }
        __syncthreads();
      }
      // clear the strictly upper triangle (it held L) so rows read as T
      for (int i = tid; i < kC * kC; i += kThreads) {
        const int r = i >> 6, cidx = i & 63;
        if (cidx > r) sTL[r * LTL + cidx] = 0.f;
      }
      __syncthreads();
    }

    // ---------------- chain waves: finish the chunk ----------------
    if (chain) {
      floatx4 ut[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (!kSolve) {
          ut[mt] = xx[mt];
        } else {
          // T is lower triangular: row tile mt needs column tiles 0..mt.  The
          // bf16 path rounds that up to an even count (the extra tile of T is
          // exactly zero) so one accumulation chain never mixes the 32-deep
          // and 16-deep MFMA opcodes.
          const float* trow = sTL + (16 * mt + lc) * LTL;
          if constexpr (kBf16) ut[mt] = mm_accB_bf16(zero4(), trow, xx, (mt | 1) + 1, lane);
          else ut[mt] = mm_accB_f32(zero4(), trow, xx, mt + 1, lane);
        }
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const T* arow = sA + (16 * mt + lc) * LKT;  // tiles above the diagonal are zero
        if constexpr (kBf16) ox[mt] = mm_accB_bf16(ox[mt], arow, ut, (mt | 1) + 1, lane);
        else ox[mt] = mm_accB_f32(ox[mt], arow, ut, mt + 1, lane);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 16 * mt + 4 * lg + i;
          float val = ox[mt][i];
          if (MODE == PF_LA) val = val * sRow[r];
          if (!a.Sc && t0 + r <= tlast) oh[(size_t)(t0 + r) * dv + 16 * cw + lc] = E::cvt(val);
        }
      }
      if (kGate) {
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[kt][i] *= sVec[16 * kt + 4 * lg + i];
      }
      if constexpr (kScal) {
        // S <- exp(G_C) S + K^T (u * exp(G_C - G_r)): row r of u decays from
        // token r to the chunk end
        const float gC = sG[kC - 1];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int i = 0; i < 4; ++i) ut[mt][i] *= __expf(gC - sG[16 * mt + 4 * lg + i]);
        const float eC = __expf(gC);
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i) st[kt][i] *= eC;
      }
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const T* krow = sKt + (16 * kt + lc) * LKT;
        if constexpr (kBf16) st[kt] = mm_accB_bf16(st[kt], krow, ut, 4, lane);
        else st[kt] = mm_accB_f32(st[kt], krow, ut, 4, lane);
      }
    }
  }

  if (chain && !a.Sc) {
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sh[(size_t)(16 * kt + 4 * lg + i) * dv + 16 * cw + lc] = st[kt][i];
  }
  if (MODE == PF_LA && sl == 0 && !a.Sc) {
    __syncthreads();
    for (int d = tid; d < DK; d += kThreads) a.z[(size_t)bh * DK + d] = sVec[d];
  }
}

// T = 0 without an initial state: the final state is zero.  A kernel rather
// than a memset, so the call can be captured in a graph.
__global__ __launch_bounds__(256) void zero_fill(float* __restrict__ p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0.f;
}

static hipError_t zero_floats(float* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
  hipLaunchKernelGGL(zero_fill, dim3((unsigned)blocks), dim3(256), 0, st, p, n);
  return hipGetLastError();
}

template <int DK, class E, int MODE, int DVS>
static hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t st) {
  const long blocks = (long)a.B * a.H * (a.dv / DVS);
  hipLaunchKernelGGL((prefill_kernel<DK, E, MODE, DVS>), dim3((unsigned)blocks),
                     dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

template <int DK, class E, int MODE>
static hipError_t launch_prefill_dk(const PrefillArgs& a, hipStream_t st) {
  if (a.dv % 32 == 0) return launch_prefill_t<DK, E, MODE, 32>(a, st);
  return launch_prefill_t<DK, E, MODE, 16>(a, st);
}

template <class E, int MODE>
static hipError_t launch_prefill_e(int dk, const PrefillArgs& a, hipStream_t st) {
  switch (dk) {
    case 16: return launch_prefill_dk<16, E, MODE>(a, st);
    case 32: return launch_prefill_dk<32, E, MODE>(a, st);
    case 64: return launch_prefill_dk<64, E, MODE>(a, st);
    case 128:
      if constexpr (ModeTraits<MODE>::kGate && sizeof(typename E::T) == 4) {
        return hipErrorInvalidValue;  // LDS footprint exceeds one CU
      } else {
        return launch_prefill_dk<128, E, MODE>(a, st);
      }
    default: return hipErrorInvalidValue;
  }
}

// The chunk-parallel linear-attention kernels (bf16) keep per-chunk states in
// the workspace; the per-channel gated pipelined kernel reads the pre-pass's
// decay-scaled q and k from it.  Every other path needs none.
hipError_t launch_prefill(int mode, int bf16, int dk, const PrefillArgs& a, void* workspace,
                          hipStream_t st) {
  if (a.T == 0) {  // no tokens: the state passes through unchanged
    if (a.use_init) return hipSuccess;
    const size_t nbh = (size_t)a.B * a.H;
    hipError_t e = zero_floats(a.S, nbh * dk * a.dv, st);
    if (e == hipSuccess && mode == PF_LA) e = zero_floats(a.z, nbh * dk, st);
    return e;
  }
  if (bf16 && (mode == PF_LA || mode == PF_GLA)) {
    // Linear attention, chunk-parallel: the chunk-start states come from a
    // prefix over per-chunk phi(K)^T V (gated: decayed); then every chunk's
    // output is formed independently from its own start state.
    hipError_t e = launch_la_par_states(dk, a, workspace, mode == PF_GLA, st);
    if (e == hipSuccess) e = launch_la_par_outputs(dk, a, workspace, mode == PF_GLA, st);
    return e;
  }
  if (bf16 && dk == 128 && a.dv % 32 == 0) {
    if (mode == PF_DELTA) return launch_prefill_pipe(a, nullptr, st);
    if (mode == PF_SGATED) return launch_prefill_pipe_token(a, st);
    // the gate pre-pass writes Gam Q, Gam K, K / Gam and Gam_C to the workspace
    if (mode == PF_GATED) return launch_prefill_pipe(a, workspace, st);
  }
  return launch_prefill_generic(mode, bf16, dk, a, st);
}

hipError_t launch_prefill_generic(int mode, int bf16, int dk, const PrefillArgs& a, hipStream_t st) {
  if (bf16) {
    switch (mode) {
      case PF_LA: return launch_prefill_e<BF16, PF_LA>(dk, a, st);
      case PF_DELTA: return launch_prefill_e<BF16, PF_DELTA>(dk, a, st);
      case PF_GATED: return launch_prefill_e<BF16, PF_GATED>(dk, a, st);
      case PF_GLA: return launch_prefill_e<BF16, PF_GLA>(dk, a, st);
      case PF_SGATED: return launch_prefill_e<BF16, PF_SGATED>(dk, a, st);
      default: return hipErrorInvalidValue;
    }
  }
  switch (mode) {
    case PF_LA: return launch_prefill_e<F32, PF_LA>(dk, a, st);
    case PF_DELTA: return launch_prefill_e<F32, PF_DELTA>(dk, a, st);
    case PF_GATED: return launch_prefill_e<F32, PF_GATED>(dk, a, st);
    case PF_GLA: return launch_prefill_e<F32, PF_GLA>(dk, a, st);
    case PF_SGATED: return launch_prefill_e<F32, PF_SGATED>(dk, a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace linattn

// la_par.hip -- chunk-parallel pieces of the linear-attention prefill.
//
// Article "From GPT-2 to Kimi K3, explained", section "Linear Attention":
// the state is S_t = S_{t-1} + phi(k_t) v_t^T and the normaliser
// z_t = z_{t-1} + phi(k_t), phi = elu + 1.  Neither update depends on the
// state, so with 64-token chunks the state entering chunk c is
//   S_c = S_0 + sum_{c' < c} phi(K_c')^T V_c',   z_c = z_0 + sum_{c' < c} colsum phi(K_c').
// la_chunk_state forms every chunk's phi(K)^T V and colsum phi(K) in
// parallel; la_state_scan turns them into S_c (bf16, the precision the
// output products read it in) and z_c (fp32, in place) and writes the final
// state; the chunk outputs are then independent.
//
// Gated linear attention (section "Gated Delta Net", the additive cache with
// a forgetting factor; q and k as given, no normaliser) has the same
// structure with a decay per token: with G_t the log-decay summed from the
// chunk start and Gam_C = exp(G_63),
//   dS_c = (K * exp(G_63 - G_t))^T V,   S_{c+1} = Gam_C S_c + dS_c,
//   O = diag(exp(G_t)) Q S_c + (tril(Q K^T) * exp(G_r - G_c)) V,
// every factor at most 1.  The kernels take it as the template flag GLA.
//
// Chunks are numbered over (batch, head, chunk) with nch = ceil(T / 64)
// chunks per head; inputs have T rows per head.  A partial last chunk is
// staged with zero rows past the end (phi(k) = 0 there: no contribution to
// the state or the normaliser), and its missing outputs are not stored.
#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

constexpr int kC = 64;
typedef short shortx4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

// Loads of a tile of N 16-byte vectors, all issued before any is used:
// thread tid takes vectors tid + 256 j; idx(i) gives the element offset of
// vector i (already clamped to valid rows by the caller).
template <int N, class F>
__device__ __forceinline__ void load_vecs(u32x4 (&buf)[(N + 255) / 256], const bf16_t* base, int tid, F idx) {
#pragma unroll
  for (int j = 0; j < (N + 255) / 256; ++j) {
    const int i = min(tid + 256 * j, N - 1);
    buf[j] = *reinterpret_cast<const u32x4*>(base + idx(i));
  }
}

// Wave 0 of a chunk's workgroup: G_t = sum_{s<=t} g_s over the chunk (lane =
// token; tokens past the end and a missing gate count as 0).
__device__ __forceinline__ float chunk_log_decay(const bf16_t* gc, int lane, int nrow) {
  return scan64_up((gc && lane < nrow) ? bf2f(gc[min(lane, nrow - 1)]) : 0.f);
}

__device__ __forceinline__ shortx4_t ld_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4_t*)((__attribute__((address_space(3))) bf16_t*)(p)));
}
__device__ __forceinline__ bf16x8 cat_tr(shortx4_t lo, shortx4_t hi) {
  typedef short shortx8_t __attribute__((ext_vector_type(8)));
  const shortx8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// One workgroup (4 waves) per (batch, head, chunk): dS[chunk] = phi(K)^T V
// (dk x dv, fp32) and dz[chunk] = colsum phi(K) (dk), bf16 inputs.  Output
// tile (16 key channels x 16 value columns) = sum over the 64 tokens, two
// 32-deep MFMAs; both operands are read from the row-major LDS tiles with
// the transpose read (lane 16G + 4a + b receives element b of the 8-byte runs
// addressed by lanes 16G + a + 4e), so that the k-index of element (g, e) is
// token 4g + e (e < 4) or 16 + 4g + e - 4.  The column sums are the same
// product with V replaced by ones.
// GLA: K rows are scaled by exp(G_63 - G_t) instead of phi, there is no
// column sum, and dz[chunk] receives Gam_C = exp(G_63) instead.
template <int DK, int DV, bool GLA>
__global__ __launch_bounds__(256) void la_chunk_state(const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v,
                                                      const bf16_t* __restrict__ g,
                                                      float* __restrict__ dS, float* __restrict__ dz, int T,
                                                      int nch) {
  constexpr int LK = DK + 16, LV = DV + 16;  // row strides (bf16)
  __shared__ __attribute__((aligned(16))) bf16_t sk[kC][LK];
  __shared__ __attribute__((aligned(16))) bf16_t sv[kC][LV];
  __shared__ float sw[GLA ? kC : 1];
  const size_t chunk = blockIdx.x;
  const int bh = (int)(chunk / nch), t0 = (int)(chunk - (size_t)bh * nch) * kC;
  const int nrow = min(kC, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16_t* kc = k + ((size_t)bh * T + t0) * DK;
  const bf16_t* vc = v + ((size_t)bh * T + t0) * DV;
  if constexpr (GLA) {
    if (wave == 0) {
      const float G = chunk_log_decay(g ? g + (size_t)bh * T + t0 : nullptr, lane, nrow);
      const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(G), kC - 1));
      sw[lane] = __expf(gC - G);
      if (lane == 0) dz[chunk] = __expf(gC);
    }
    __syncthreads();
  }
  // rows past the end re-read the last row and are zeroed after phi
  constexpr int NK = kC * DK / 8, NV = kC * DV / 8;
  u32x4 bk[(NK + 255) / 256], bv[(NV + 255) / 256];
  load_vecs<NK>(bk, kc, tid, [&](int i) { return (size_t)min(i / (DK / 8), nrow - 1) * DK + (i % (DK / 8)) * 8; });
  load_vecs<NV>(bv, vc, tid, [&](int i) { return (size_t)min(i / (DV / 8), nrow - 1) * DV + (i % (DV / 8)) * 8; });
#pragma unroll
  for (int j = 0; j < (NK + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (NK % 256 != 0 && i >= NK) continue;
    const int r = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
    u32x4 w = bk[j];
    const float wr = GLA ? sw[GLA ? r : 0] : 1.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float x0 = bf2f((bf16_t)(w[e] & 0xffffu)), x1 = bf2f((bf16_t)(w[e] >> 16));
      const float lo = GLA ? x0 * wr : phi_elu1(x0);
      const float hi = GLA ? x1 * wr : phi_elu1(x1);
      w[e] = r < nrow ? pack2(lo, hi) : 0u;
    }
    *reinterpret_cast<u32x4*>(&sk[r][c8]) = w;
  }
#pragma unroll
  for (int j = 0; j < (NV + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (NV % 256 != 0 && i >= NV) continue;
    const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
    *reinterpret_cast<u32x4*>(&sv[r][c8]) = r < nrow ? bv[j] : u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  constexpr int NDT = DK / 16, NJT = DV / 16 + (GLA ? 0 : 1);  // the extra column tile gives dz
  const int trow = 4 * (lane >> 4) + ((lane >> 2) & 3);
  const int tcol = 4 * (lane & 3);
  const int lc = lane & 15, lg = lane >> 4;
  const bf16_t one = f2bf(1.f);
  const bf16x8 ones = {__builtin_bit_cast(__bf16, one), __builtin_bit_cast(__bf16, one),
                       __builtin_bit_cast(__bf16, one), __builtin_bit_cast(__bf16, one),
                       __builtin_bit_cast(__bf16, one), __builtin_bit_cast(__bf16, one),
                       __builtin_bit_cast(__bf16, one), __builtin_bit_cast(__bf16, one)};
  for (int tile = wave; tile < NDT * NJT; tile += 4) {
    const int dt = tile / NJT, jt = tile % NJT;
    floatx4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int t0 = 32 * kb;
      const bf16x8 a = cat_tr(ld_tr(&sk[t0 + trow][16 * dt + tcol]), ld_tr(&sk[t0 + 16 + trow][16 * dt + tcol]));
      const bf16x8 b = (GLA || jt < NJT - 1)
                           ? cat_tr(ld_tr(&sv[t0 + trow][16 * jt + tcol]), ld_tr(&sv[t0 + 16 + trow][16 * jt + tcol]))
                           : ones;
      acc = mfma_k32(a, b, acc);
    }
    // lane (lc, lg) holds rows 16dt + 4lg + i, column 16jt + lc
    if (GLA || jt < NJT - 1) {
      float* out = dS + chunk * DK * DV;
#pragma unroll
      for (int i = 0; i < 4; ++i) out[(size_t)(16 * dt + 4 * lg + i) * DV + 16 * jt + lc] = acc[i];
    } else if (lc == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) dz[chunk * DK + 16 * dt + 4 * lg + i] = acc[i];
    }
  }
}

// Per (batch, head) and state element: the exclusive prefix over chunks,
// starting from the initial state (or zero); the total is the final state.
// Thread e of a (batch, head) owns element e of [S (dk*dv), z (dk)].  The
// prefix of S goes to Sb in bf16 (rounded to nearest even); that of z
// replaces dz in place.
// GLA: S only (dk = 0 here), and each step first decays the running state
// by the chunk's Gam_C, held in dz[chunk]: S_{c+1} = Gam_C S_c + dS_c.
template <bool GLA>
__global__ __launch_bounds__(256) void la_state_scan(const float* __restrict__ dS, float* __restrict__ dz,
                                                     bf16_t* __restrict__ Sb, float* S, float* z, int nch,
                                                     int dkdv, int dk, int use_init) {
  const long bh = blockIdx.x;  // heads in the first grid dimension (the second is limited to 65535)
  const int e = blockIdx.y * 256 + threadIdx.x;
  if (e >= dkdv + dk) return;
  const float* gam = GLA ? dz + (size_t)bh * nch : nullptr;
  const bool isz = e >= dkdv;
  const int idx = isz ? e - dkdv : e;
  const int stride = isz ? dk : dkdv;
  const float* base = isz ? dz + (size_t)bh * nch * dk + idx : dS + (size_t)bh * nch * dkdv + idx;
  float* zout = dz + (size_t)bh * nch * dk + idx;
  bf16_t* sout = Sb + (size_t)bh * nch * dkdv + idx;
  float* fin = isz ? z + (size_t)bh * dk + idx : S + (size_t)bh * dkdv + idx;
  float run = use_init ? *fin : 0.f;
  auto put = [&](int c, float val) {
    if (isz) zout[(size_t)c * stride] = val;
    else sout[(size_t)c * stride] = f2bf(val);
  };
  int c = 0;
  for (; c + 8 <= nch; c += 8) {  // eight loads in flight
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = base[(size_t)(c + i) * stride];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      put(c + i, run);
      run = GLA ? run * gam[c + i] + t[i] : run + t[i];
    }
  }
  for (; c < nch; ++c) {
    const float t = base[(size_t)c * stride];
    put(c, run);
    run = GLA ? run * gam[c] + t : run + t;
  }
  *fin = run;
}

// One workgroup (4 waves) per (batch, head, chunk): with S_c (bf16), z_c the
// state entering the chunk (from la_state_scan),
//   O = (phi(Q) S_c + tril(phi(Q) phi(K)^T) V) / (phi(Q) z_c + rowsum tril(...)).
// Wave w owns tokens 16w .. 16w+15.  A operands (phi(Q) rows, rows of the
// masked score block) are 16-byte LDS reads in natural k order; B operands
// over tokens or key channels (V, S_c) are LDS transpose reads addressing
// rows 8G + e and 8G + 4 + e, which gives the same natural order.
// GLA: q and k as given, no denominator; scores scaled by exp(G_r - G_c)
// and the rows of phi(Q) S_c -> Q S_c by exp(G_r).
template <int DK, int DV, bool GLA>
__global__ __launch_bounds__(256) void la_chunk_out(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                    const bf16_t* __restrict__ v, const bf16_t* __restrict__ g,
                                                    const bf16_t* __restrict__ Sc,
                                                    const float* __restrict__ zc, bf16_t* __restrict__ o, int T,
                                                    int nch) {
  constexpr int LQ = DK + 16, LV = DV + 16, LA = kC + 16;
  __shared__ __attribute__((aligned(16))) bf16_t sq[kC][LQ];
  __shared__ __attribute__((aligned(16))) bf16_t sk[kC][LQ];
  __shared__ __attribute__((aligned(16))) bf16_t sv[kC][LV];
  __shared__ __attribute__((aligned(16))) bf16_t ss[DK][LV];   // S_c in bf16
  __shared__ __attribute__((aligned(16))) bf16_t sa[kC][LA];   // masked scores, bf16
  __shared__ float sz[DK];
  __shared__ float sden[kC];
  __shared__ float sg[GLA ? kC : 1];
  const size_t chunk = blockIdx.x;
  const int bh = (int)(chunk / nch), t0 = (int)(chunk - (size_t)bh * nch) * kC;
  const int nrow = min(kC, T - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lc = lane & 15, lg = lane >> 4;
  const bf16_t* qc = q + ((size_t)bh * T + t0) * DK;
  const bf16_t* kc = k + ((size_t)bh * T + t0) * DK;
  const bf16_t* vc = v + ((size_t)bh * T + t0) * DV;
  // every load first (rows past the end re-read the last row; phi(q) =
  // phi(k) = 0 there), then phi and the LDS stores
  constexpr int NQ = kC * DK / 8, NV = kC * DV / 8, NS = DK * DV / 8;
  const bf16_t* sc = Sc + chunk * DK * DV;
  u32x4 bq[(NQ + 255) / 256], bk[(NQ + 255) / 256], bv[(NV + 255) / 256], bs[(NS + 255) / 256];
  auto qk_idx = [&](int i) { return (size_t)min(i / (DK / 8), nrow - 1) * DK + (i % (DK / 8)) * 8; };
  load_vecs<NQ>(bq, qc, tid, qk_idx);
  load_vecs<NQ>(bk, kc, tid, qk_idx);
  load_vecs<NV>(bv, vc, tid, [&](int i) { return (size_t)min(i / (DV / 8), nrow - 1) * DV + (i % (DV / 8)) * 8; });
  load_vecs<NS>(bs, sc, tid, [&](int i) { return (size_t)i * 8; });
#pragma unroll
  for (int j = 0; j < (NQ + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (NQ % 256 != 0 && i >= NQ) continue;
    const int r = i / (DK / 8), c8 = (i % (DK / 8)) * 8;
    u32x4 wq = bq[j], wk = bk[j];
    if constexpr (!GLA) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        wq[e] = pack2(phi_elu1(bf2f((bf16_t)(wq[e] & 0xffffu))), phi_elu1(bf2f((bf16_t)(wq[e] >> 16))));
        wk[e] = pack2(phi_elu1(bf2f((bf16_t)(wk[e] & 0xffffu))), phi_elu1(bf2f((bf16_t)(wk[e] >> 16))));
      }
    }
    if (r >= nrow) wq = wk = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&sq[r][c8]) = wq;
    *reinterpret_cast<u32x4*>(&sk[r][c8]) = wk;
  }
#pragma unroll
  for (int j = 0; j < (NV + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (NV % 256 != 0 && i >= NV) continue;
    const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
    *reinterpret_cast<u32x4*>(&sv[r][c8]) = r < nrow ? bv[j] : u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int j = 0; j < (NS + 255) / 256; ++j) {
    const int i = tid + 256 * j;
    if (NS % 256 != 0 && i >= NS) continue;
    const int r = i / (DV / 8), c8 = (i % (DV / 8)) * 8;
    *reinterpret_cast<u32x4*>(&ss[r][c8]) = bs[j];
  }
  if constexpr (GLA) {
    if (wave == 0) sg[lane] = chunk_log_decay(g ? g + (size_t)bh * T + t0 : nullptr, lane, nrow);
  } else {
    for (int i = tid; i < DK; i += 256) sz[i] = zc[chunk * DK + i];
  }
  __syncthreads();

  const int mt = wave;  // token row block
  // masked scores of the row block: tiles j <= mt; rowsum on the way
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (j > mt) break;
    floatx4 acc = zero4();
    if constexpr (DK == 16) {  // one 16-deep product
      acc = mfma_k16(*reinterpret_cast<const shortx4_t*>(&sq[16 * mt + lc][4 * lg]),
                     *reinterpret_cast<const shortx4_t*>(&sk[16 * j + lc][4 * lg]), acc);
    } else {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        acc = mfma_k32(*reinterpret_cast<const bf16x8*>(&sq[16 * mt + lc][32 * kb + 8 * lg]),
                       *reinterpret_cast<const bf16x8*>(&sk[16 * j + lc][32 * kb + 8 * lg]), acc);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 16 * mt + 4 * lg + i, cc = 16 * j + lc;
      float x = acc[i];
      if constexpr (GLA) x *= cc <= r ? __expf(sg[GLA ? r : 0] - sg[GLA ? cc : 0]) : 0.f;
      x = cc <= r ? x : 0.f;
      sa[r][cc] = f2bf(x);
      rs[i] += x;
    }
  }
  for (int j = mt + 1; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[16 * mt + 4 * lg + i][16 * j + lc] = 0;
  // denominators: phi(q_r).z_c (lane lc takes channels lc, lc + 16, ...)
  // plus the row sum, summed over the 16 lanes of a lane group
#pragma unroll
  for (int i = 0; i < (GLA ? 0 : 4); ++i) {
    const int r = 16 * mt + 4 * lg + i;
    float x = rs[i];
#pragma unroll
    for (int c = lc; c < DK; c += 16) x += bf2f(sq[r][c]) * sz[c];
    x = sum16(x);
    if (lc == 0) sden[r] = x;
  }
  // one wave wrote its own score rows and denominators: wave-local ordering
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  const int trow = 8 * lg + ((lane >> 2) & 3);
  const int tcol = 4 * (lane & 3);
  bf16_t* oc = o + ((size_t)bh * T + t0) * DV;
  // the output tiles are formed transposed (operands swapped): lane (lc, lg)
  // holds token r = 16 mt + lc, value columns 16 jt + 4 lg .. +3, so one
  // scale per lane and one 8-byte store
  const int r = 16 * mt + lc;
  // decay of Q S_c, or the reciprocal of the denominator (one division per
  // lane instead of one per output element)
  const float rs_r = GLA ? __expf(sg[GLA ? r : 0]) : 1.f / sden[GLA ? 0 : r];
#pragma unroll
  for (int jt = 0; jt < DV / 16; ++jt) {
    // phi(Q) S_c (a separate accumulator: the 16-deep and 32-deep opcodes
    // must not share one accumulation chain)
    floatx4 aqs = zero4();
    if constexpr (DK == 16) {
      aqs = mfma_k16(ld_tr(&ss[4 * lg + ((lane >> 2) & 3)][16 * jt + tcol]),
                     *reinterpret_cast<const shortx4_t*>(&sq[16 * mt + lc][4 * lg]), aqs);
    } else {
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const bf16x8 b = cat_tr(ld_tr(&ss[32 * kb + trow][16 * jt + tcol]), ld_tr(&ss[32 * kb + 4 + trow][16 * jt + tcol]));
        aqs = mfma_k32(b, *reinterpret_cast<const bf16x8*>(&sq[16 * mt + lc][32 * kb + 8 * lg]), aqs);
      }
    }
    // tril(.) V over tokens 0 .. 16 mt + 15
    floatx4 acc = zero4();
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (32 * kb > 16 * mt + 15) break;
      const bf16x8 b = cat_tr(ld_tr(&sv[32 * kb + trow][16 * jt + tcol]), ld_tr(&sv[32 * kb + 4 + trow][16 * jt + tcol]));
      acc = mfma_k32(b, *reinterpret_cast<const bf16x8*>(&sa[16 * mt + lc][32 * kb + 8 * lg]), acc);
    }
    float v4[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = GLA ? acc[i] + aqs[i] * rs_r : (acc[i] + aqs[i]) * rs_r;
    if (r < nrow)
      *reinterpret_cast<uint2*>(oc + (size_t)r * DV + 16 * jt + 4 * lg) =
          make_uint2(pack2(v4[0], v4[1]), pack2(v4[2], v4[3]));
  }
}

template <int DK, bool GLA>
hipError_t launch_state_dk(int dv, const PrefillArgs& a, float* dS, float* dz, long nchunks, int nch,
                           hipStream_t st) {
  const bf16_t* k = reinterpret_cast<const bf16_t*>(a.k);
  const bf16_t* v = reinterpret_cast<const bf16_t*>(a.v);
  const bf16_t* g = reinterpret_cast<const bf16_t*>(a.g);
  const dim3 grid((unsigned)nchunks), block(256);
  switch (dv) {
    case 16: hipLaunchKernelGGL((la_chunk_state<DK, 16, GLA>), grid, block, 0, st, k, v, g, dS, dz, a.T, nch); break;
    case 32: hipLaunchKernelGGL((la_chunk_state<DK, 32, GLA>), grid, block, 0, st, k, v, g, dS, dz, a.T, nch); break;
    case 64: hipLaunchKernelGGL((la_chunk_state<DK, 64, GLA>), grid, block, 0, st, k, v, g, dS, dz, a.T, nch); break;
    case 128: hipLaunchKernelGGL((la_chunk_state<DK, 128, GLA>), grid, block, 0, st, k, v, g, dS, dz, a.T, nch); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int DK, bool GLA>
hipError_t launch_out_dk(int dv, const PrefillArgs& a, const bf16_t* Sc, const float* zc, long nchunks, int nch,
                         hipStream_t st) {
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
  const bf16_t* k = reinterpret_cast<const bf16_t*>(a.k);
  const bf16_t* v = reinterpret_cast<const bf16_t*>(a.v);
  const bf16_t* g = reinterpret_cast<const bf16_t*>(a.g);
  bf16_t* o = reinterpret_cast<bf16_t*>(a.o);
  const dim3 grid((unsigned)nchunks), block(256);
  switch (dv) {
    case 16: hipLaunchKernelGGL((la_chunk_out<DK, 16, GLA>), grid, block, 0, st, q, k, v, g, Sc, zc, o, a.T, nch); break;
    case 32: hipLaunchKernelGGL((la_chunk_out<DK, 32, GLA>), grid, block, 0, st, q, k, v, g, Sc, zc, o, a.T, nch); break;
    case 64: hipLaunchKernelGGL((la_chunk_out<DK, 64, GLA>), grid, block, 0, st, q, k, v, g, Sc, zc, o, a.T, nch); break;
    case 128: hipLaunchKernelGGL((la_chunk_out<DK, 128, GLA>), grid, block, 0, st, q, k, v, g, Sc, zc, o, a.T, nch); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool GLA>
hipError_t launch_outputs(int dk, const PrefillArgs& a, void* workspace, hipStream_t st) {
  const int nch = (a.T + kC - 1) / kC;
  const long nchunks = (long)a.B * a.H * nch;
  const float* dS = reinterpret_cast<const float*>(workspace);
  const float* zc = dS + (size_t)nchunks * dk * a.dv;
  const bf16_t* Sc = reinterpret_cast<const bf16_t*>(zc + (size_t)nchunks * dk);
  switch (dk) {
    case 16: return launch_out_dk<16, GLA>(a.dv, a, Sc, zc, nchunks, nch, st);
    case 32: return launch_out_dk<32, GLA>(a.dv, a, Sc, zc, nchunks, nch, st);
    case 64: return launch_out_dk<64, GLA>(a.dv, a, Sc, zc, nchunks, nch, st);
    case 128: return launch_out_dk<128, GLA>(a.dv, a, Sc, zc, nchunks, nch, st);
    default: return hipErrorInvalidValue;
  }
}

template <bool GLA>
hipError_t launch_states(int dk, const PrefillArgs& a, void* workspace, hipStream_t st) {
  const int nch = (a.T + kC - 1) / kC;
  const long nchunks = (long)a.B * a.H * nch;
  float* dS = reinterpret_cast<float*>(workspace);
  float* dz = dS + (size_t)nchunks * dk * a.dv;
  hipError_t e;
  switch (dk) {
    case 16: e = launch_state_dk<16, GLA>(a.dv, a, dS, dz, nchunks, nch, st); break;
    case 32: e = launch_state_dk<32, GLA>(a.dv, a, dS, dz, nchunks, nch, st); break;
    case 64: e = launch_state_dk<64, GLA>(a.dv, a, dS, dz, nchunks, nch, st); break;
    case 128: e = launch_state_dk<128, GLA>(a.dv, a, dS, dz, nchunks, nch, st); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  const int nz = GLA ? 0 : dk;  // gated linear attention has no normaliser
  const int n = dk * a.dv + nz;
  bf16_t* Sb = reinterpret_cast<bf16_t*>(dz + (size_t)nchunks * dk);
  hipLaunchKernelGGL((la_state_scan<GLA>), dim3((unsigned)(a.B * a.H), (unsigned)((n + 255) / 256)), dim3(256),
                     0, st, dS, dz, Sb, a.S, a.z, nch, dk * a.dv, nz, a.use_init);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_la_par_states(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st) {
  return gla ? launch_states<true>(dk, a, workspace, st) : launch_states<false>(dk, a, workspace, st);
}

hipError_t launch_la_par_outputs(int dk, const PrefillArgs& a, void* workspace, bool gla, hipStream_t st) {
  return gla ? launch_outputs<true>(dk, a, workspace, st) : launch_outputs<false>(dk, a, workspace, st);
}

}  // namespace linattn

// prefill_pipe.hip -- software-pipelined chunkwise delta-rule prefill for
// bf16 inputs with dk = 128 and dv a multiple of 32 (the throughput path).
//
// The arithmetic is that of the article "From GPT-2 to Kimi K3, explained",
// section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)":
// per 64-token chunk, with L = tril(diag(beta) K K^T, -1) and T = (I + L)^-1,
//   u = T diag(beta) (V - K S),   O = Q S + tril(Q K^T) u,   S <- S + K^T u.
// It is the same computation as prefill.hip; this kernel only organises it
// for throughput on one CU.  T is never formed: with I + L split into 16x16
// token blocks, u is obtained by block forward substitution,
//   u_b = D_b (X_b - sum_{j<b} L_bj u_j),   D_b = (I + L_bb)^-1,
// where X = diag(beta) (V - K S).
//
// Work split inside a workgroup (8 waves; one (batch, head) and 32 value
// columns per workgroup):
//   waves 0-1  "chain": each keeps S[:, 16 columns] in MFMA accumulators and
//              runs only the S-dependent products of chunk c.
//   waves 2,3,7 products of chunk c+1: K K^T (giving L) in phase 1 and
//              tril(Q K^T) in phase 2.
//   wave 6     the diagonal-block inverses D_b of chunk c+1 by fp32 forward
//              substitution (one lane per column; phase 2).
//   wave 4     writes the output tile of chunk c-1 to memory (phase 1).
//   waves 2-7  the global loads of q, k and the v slice, issued three
//              chunks ahead into registers and written to LDS two chunks
//              ahead.
// Each iteration has two phases separated by LDS-only barriers, so global
// loads stay in flight across them.
//
// Index conventions.  K, Q and the v slice are stored row-major (tokens x
// channels) in natural column order.  The chain's 32-deep MFMA pairs two
// accumulator tiles; the k-index order that pairing implies is absorbed by a
// fixed permutation of S's rows: the accumulator row rho = 32b + 16h + 4g + i
// of a chain wave holds logical key channel d = 32b + 8g + 4h + i (perm32
// below).  tril(Q K^T), used as an A operand against paired tiles over
// tokens, stores its token columns permuted the same way, so each of its
// fragments is one 16-byte LDS read.  The transposed operands K^T (for
// S += K^T u) and the accumulator-layout V are read straight from the
// row-major tiles with the LDS transpose read (ds_read_b64_tr_b16): lane
// 16G + 4a + b receives element b of the 8-byte runs addressed by lanes
// 16G + a + 4e, e = 0..3.  The 16x16 blocks D_b and L_bj are stored
// transposed (16 bf16 per row, unpadded) and read the same way as the A
// operands of the 16-deep MFMA.
//
// Row strides are 8 (mod 32) dwords: 16-byte fragment reads of 16 rows and
// transpose reads of 4-8 rows then fall in distinct LDS banks.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

constexpr int kC = 64;
constexpr int kDK = 128;
constexpr int kDVS = 32;
constexpr int kThreads = 512;

constexpr int kLQ = kDK + 16;  // bf16 row stride of q, k (72 dwords)
constexpr int kLT = kC + 16;   // bf16 row stride of tril(QK^T) (40 dwords)
constexpr int kLV = kDVS + 16; // bf16 row stride of the v slice (24 dwords)
constexpr int kLL = kC + 4;    // fp32 row stride of L (diagonal blocks)
constexpr int kLO = kDVS + 8;  // bf16 row stride of the output tile

struct __attribute__((aligned(16))) Smem {
  bf16_t q[2][kC][kLQ];
  bf16_t k[3][kC][kLQ];    // chunk x in buffer x mod 3: K(c) is read in both phases
  bf16_t a[2][kC][kLT];
  bf16_t lb[2][6][16][16]; // off-diagonal blocks L_bj (b > j), transposed
  bf16_t d[2][4][16][16];  // diagonal-block inverses D_b, transposed
  bf16_t v[2][kC][kLV];    // the v slice, row-major
  bf16_t o[kC][kLO];       // output tile of one chunk
  float l[kC][kLL];
  float beta[2][kC];
};

// 32b + 16h + 4g + i  ->  32b + 8g + 4h + i
__device__ __forceinline__ int perm32(int x) {
  return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}
// inverse: 32b + 8g + 4h + i  ->  32b + 16h + 4g + i
__device__ __forceinline__ int perm32_inv(int x) {
  return (x & ~31) | (((x >> 2) & 1) << 4) | (((x >> 3) & 3) << 2) | (x & 3);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int mod3(int x) { return (x + 3) % 3; }  // x >= -3

__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if (n % 8 != 0) return bid;
  return (bid % 8) * (n / 8) + bid / 8;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 ld_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

typedef short shortx4_t __attribute__((ext_vector_type(4)));
// LDS transpose read of four bf16 (see the index conventions above).
__device__ __forceinline__ shortx4_t ld_tr(const bf16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) shortx4_t*)(
          (__attribute__((address_space(3))) bf16_t*)(p)));
}
__device__ __forceinline__ bf16x8 cat_tr(shortx4_t lo, shortx4_t hi) {
  typedef short shortx8_t __attribute__((ext_vector_type(8)));
  const shortx8_t x = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, x);
}

// 16x16 fp32 accumulator tile used as a 16-deep bf16 MFMA operand.  As B it
// is the tile itself; as A it is the tile's transpose.
}  // namespace

__global__ __launch_bounds__(kThreads) void prefill_delta_pipe(PrefillArgs a) {
  __shared__ Smem sm;

  const int nsl = a.dv / kDVS;
  const int w = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = w / nsl;
  const int sl = w - bh * nsl;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lc = lane & 15;
  const int lg = lane >> 4;
  const int Tn = a.T;
  const int dv = a.dv;
  const int nch = Tn / kC;

  const bf16_t* qh = reinterpret_cast<const bf16_t*>(a.q) + (size_t)bh * Tn * kDK;
  const bf16_t* kh = reinterpret_cast<const bf16_t*>(a.k) + (size_t)bh * Tn * kDK;
  const bf16_t* vh = reinterpret_cast<const bf16_t*>(a.v) + (size_t)bh * Tn * dv + sl * kDVS;
  const bf16_t* bth = reinterpret_cast<const bf16_t*>(a.beta) + (size_t)bh * Tn;
  bf16_t* oh = reinterpret_cast<bf16_t*>(a.o) + (size_t)bh * Tn * dv + sl * kDVS;
  float* Sh = a.S + (size_t)bh * kDK * dv + sl * kDVS;

  // Tiles above the diagonal of tril(QK^T) are read as zeros.
  {
    uint32_t* z = reinterpret_cast<uint32_t*>(&sm.a[0][0][0]);
    for (int i = tid; i < (int)(sizeof(sm.a) / 4); i += kThreads) z[i] = 0u;
  }

  // ---- register prefetch by waves 2..7 (the chain waves keep their
  // registers for the state).  A chunk is 2304 16-byte vectors: 0..1023 q,
  // 1024..2047 k, 2048..2303 the 64 x 32 slice of v; loader thread
  // u = tid - 128 owns vectors u + 384 j.  beta is loaded by wave 4.
  constexpr int kLoaders = kThreads - 128;
  constexpr int kPerLoader = 2304 / kLoaders;  // 6
  const int lu = tid - 128;
  auto issue_loads = [&](int chunk, u32x4 (&dst)[kPerLoader], uint32_t& bdst) {
#pragma unroll
    for (int j = 0; j < kPerLoader; ++j) {
      const int v = lu + kLoaders * j;
      const bf16_t* src;
      if (v < 2048) {
        const int vv = v & 1023;
        src = (v < 1024 ? qh : kh) + (size_t)(chunk * kC + (vv >> 4)) * kDK + (vv & 15) * 8;
      } else {
        const int vv = v - 2048;
        src = vh + (size_t)(chunk * kC + (vv >> 2)) * dv + (vv & 3) * 8;
      }
      dst[j] = *reinterpret_cast<const u32x4*>(src);
    }
    if (wave == 4) bdst = bth[chunk * kC + lane];  // converted when stored
  };
  auto store_loads = [&](int buf, int kbuf, const u32x4 (&src)[kPerLoader], uint32_t bsrc) {
#pragma unroll
    for (int j = 0; j < kPerLoader; ++j) {
      const int v = lu + kLoaders * j;
      if (v < 2048) {
        const int vv = v & 1023;
        bf16_t* dstp = (v < 1024 ? &sm.q[buf][vv >> 4][(vv & 15) * 8] : &sm.k[kbuf][vv >> 4][(vv & 15) * 8]);
        *reinterpret_cast<u32x4*>(dstp) = src[j];
      } else {
        const int vv = v - 2048;
        *reinterpret_cast<u32x4*>(&sm.v[buf][vv >> 2][(vv & 3) * 8]) = src[j];
      }
    }
    if (wave == 4) sm.beta[buf][lane] = bf2f((bf16_t)bsrc);
  };

  // Every role below runs its own copy of the chunk loop: iteration c
  // (c = -1 .. nch-1) has two phases, each closed by one LDS barrier, so all
  // waves meet at the same barriers while each role keeps only its own state
  // live.  In iteration c the chain works on chunk c, products and T on
  // chunk c+1; every wave writes its share of chunk c+2 to LDS (loaded one
  // iteration earlier) and issues its global loads of chunk c+3.
  // `body(c, P, phase1, phase2)` runs one iteration with P = c & 1 known at
  // compile time, so every buffer and register-slot index is static.
  auto run = [&](auto phase1, auto phase2) {
    const bool loader = wave >= 2;
    u32x4 pf[2][kPerLoader];
    uint32_t pfb[2] = {0u, 0u};
    if (loader) {
      issue_loads(0, pf[0], pfb[0]);
      store_loads(0, 0, pf[0], pfb[0]);
      if (nch > 1) issue_loads(1, pf[1], pfb[1]);
    }
    lds_barrier();
    auto body = [&](const int c, auto parity) {
      constexpr int P = decltype(parity)::value;
      phase1(c, parity);
      if (loader && c + 3 < nch) issue_loads(c + 3, pf[1 - P], pfb[1 - P]);
      lds_barrier();
      phase2(c, parity);
      if (loader && c + 2 < nch) store_loads(P, mod3(c + 2), pf[P], pfb[P]);
      lds_barrier();
    };
    for (int c = -1; c < nch; c += 2) {
      body(c, std::integral_constant<int, 1>{});
      if (c + 1 < nch) body(c + 1, std::integral_constant<int, 0>{});
    }
  };

  if (wave < 2) {
    // ======================= chain waves =======================
    const int col = 16 * wave + lc;  // value column within the slice
    floatx4 st[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      st[t] = zero4();
      if (a.use_init) {
#pragma unroll
        for (int i = 0; i < 4; ++i) st[t][i] = Sh[(size_t)perm32(16 * t + 4 * lg + i) * dv + col];
      }
    }
    floatx4 xx[4], ox[4];
    run(
        [&](const int c, auto parity) {
          constexpr int P = decltype(parity)::value;
          if (c < 0) return;
          const int kc = mod3(c);
          // Y = K S and O = Q S (shared S fragments), X = beta (V - Y).
          // The fragments of k-step kb+1 are loaded while kb computes.
          floatx4 y[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) { y[mt] = zero4(); ox[mt] = zero4(); }
          bf16x8 fk[2][4], fq[2][4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            fk[0][mt] = ld_frag(&sm.k[kc][16 * mt + lc][8 * lg]);
            fq[0][mt] = ld_frag(&sm.q[P][16 * mt + lc][8 * lg]);
          }
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            if (kb < 3) {
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) {
                fk[(kb + 1) & 1][mt] = ld_frag(&sm.k[kc][16 * mt + lc][32 * (kb + 1) + 8 * lg]);
                fq[(kb + 1) & 1][mt] = ld_frag(&sm.q[P][16 * mt + lc][32 * (kb + 1) + 8 * lg]);
              }
            }
            const bf16x8 b = acc_pair_to_b(st[2 * kb], st[2 * kb + 1]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              y[mt] = mfma_k32(fk[kb & 1][mt], b, y[mt]);
              ox[mt] = mfma_k32(fq[kb & 1][mt], b, ox[mt]);
            }
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            // lane (lg, lc) gets V[16 mt + 4 lg + i][col], i = 0..3
            const shortx4_t vw = ld_tr(&sm.v[P][16 * mt + 4 * lg + ((lane >> 2) & 3)][16 * wave + 4 * (lane & 3)]);
            const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[P][16 * mt + 4 * lg]);
            xx[mt][0] = bt.x * (bf2f((bf16_t)vw[0]) - y[mt][0]);
            xx[mt][1] = bt.y * (bf2f((bf16_t)vw[1]) - y[mt][1]);
            xx[mt][2] = bt.z * (bf2f((bf16_t)vw[2]) - y[mt][2]);
            xx[mt][3] = bt.w * (bf2f((bf16_t)vw[3]) - y[mt][3]);
          }
        },
        [&](const int c, auto parity) {
          constexpr int P = decltype(parity)::value;
          if (c < 0) return;
          const int kc = mod3(c);
          // u by block forward substitution; the D_b, L_bj and tril(Q K^T)
          // fragments are requested up front.
          auto fr16 = [&](const bf16_t* blk) {  // A operand of a transposed 16x16 block
            return ld_tr(blk + (4 * lg + ((lane >> 2) & 3)) * 16 + 4 * (lane & 3));
          };
          shortx4_t fd[4], fl[6];
#pragma unroll
          for (int b = 0; b < 4; ++b) fd[b] = fr16(&sm.d[P][b][0][0]);
#pragma unroll
          for (int x = 0; x < 6; ++x) fl[x] = fr16(&sm.lb[P][x][0][0]);
          bf16x8 fa[6];
          fa[0] = ld_frag(&sm.a[P][lc][8 * lg]);
          fa[1] = ld_frag(&sm.a[P][16 + lc][8 * lg]);
          fa[2] = ld_frag(&sm.a[P][32 + lc][8 * lg]);
          fa[3] = ld_frag(&sm.a[P][32 + lc][32 + 8 * lg]);
          fa[4] = ld_frag(&sm.a[P][48 + lc][8 * lg]);
          fa[5] = ld_frag(&sm.a[P][48 + lc][32 + 8 * lg]);
          // blocks L_bj stored in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
          floatx4 ut[4];
          ut[0] = mfma_k16(fd[0], acc_to_b16(xx[0]), zero4());
          const shortx4_t u0 = acc_to_b16(ut[0]);
          ut[1] = mfma_k16(fd[1], acc_to_b16(xx[1] - mfma_k16(fl[0], u0, zero4())), zero4());
          const shortx4_t u1 = acc_to_b16(ut[1]);
          ut[2] = mfma_k16(fd[2], acc_to_b16(xx[2] - mfma_k16(fl[2], u1, mfma_k16(fl[1], u0, zero4()))),
                           zero4());
          const shortx4_t u2 = acc_to_b16(ut[2]);
          ut[3] = mfma_k16(fd[3], acc_to_b16(xx[3] - mfma_k16(fl[5], u2, mfma_k16(fl[4], u1, mfma_k16(fl[3], u0, zero4())))),
                           zero4());
          // K^T fragments: row 16t + c of the A operand is key channel
          // perm32(16t + c); its k-elements are the tokens of u's pairing.
          const int trow = 4 * lg + ((lane >> 2) & 3);
          auto kt_frag = [&](int t, int tok0) {
            const int col = 32 * (t >> 1) + 4 * (t & 1) + 8 * (lane & 3);
            return cat_tr(ld_tr(&sm.k[kc][tok0 + trow][col]), ld_tr(&sm.k[kc][tok0 + 16 + trow][col]));
          };
          bf16x8 fkt[2][8];
#pragma unroll
          for (int t = 0; t < 8; ++t) fkt[0][t] = kt_frag(t, 0);
          const bf16x8 u01 = acc_pair_to_b(ut[0], ut[1]);
          const bf16x8 u23 = acc_pair_to_b(ut[2], ut[3]);
          // O += tril(Q K^T) u
          ox[0] = mfma_k32(fa[0], u01, ox[0]);
          ox[1] = mfma_k32(fa[1], u01, ox[1]);
          ox[2] = mfma_k32(fa[3], u23, mfma_k32(fa[2], u01, ox[2]));
          ox[3] = mfma_k32(fa[5], u23, mfma_k32(fa[4], u01, ox[3]));
#pragma unroll
          for (int t = 0; t < 8; ++t) fkt[1][t] = kt_frag(t, 32);
          // S += K^T u
#pragma unroll
          for (int t = 0; t < 8; ++t) st[t] = mfma_k32(fkt[0][t], u01, st[t]);
#pragma unroll
          for (int t = 0; t < 8; ++t) st[t] = mfma_k32(fkt[1][t], u23, st[t]);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) sm.o[16 * mt + 4 * lg + i][col] = f2bf(ox[mt][i]);
        });
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) Sh[(size_t)perm32(16 * t + 4 * lg + i) * dv + col] = st[t][i];
  } else if (wave == 6) {
    // ======================= D wave =======================
    // Diagonal 16x16 blocks of I + L for chunk c+1 (phase 2): lane (block lg,
    // column lc) solves (I + L_bb) x = e_lc by forward substitution in fp32;
    // x is column lc of D_b = (I + L_bb)^-1, stored as row lc of D_b^T.
    run([&](const int c, auto parity) {},
        [&](const int c, auto parity) {
          constexpr int nb = 1 - decltype(parity)::value;
          if (c + 1 >= nch) return;
          const int b0 = 16 * lg;
          float4 lr[16][4];  // strictly-lower rows of L_bb, requested up front
#pragma unroll
          for (int i = 1; i < 16; ++i)
#pragma unroll
            for (int m4 = 0; m4 < i; m4 += 4)
              lr[i][m4 >> 2] = *reinterpret_cast<const float4*>(&sm.l[b0 + i][b0 + m4]);
          float tv[16];
#pragma unroll
          for (int m = 0; m < 16; ++m) tv[m] = m == lc ? 1.f : 0.f;
#pragma unroll
          for (int i = 1; i < 16; ++i) {
            float s0 = 0.f, s1 = 0.f;
#pragma unroll
            for (int m = 0; m < i; ++m) {
              const float4 q4 = lr[i][m >> 2];
              const float lv = (m & 3) == 0 ? q4.x : (m & 3) == 1 ? q4.y : (m & 3) == 2 ? q4.z : q4.w;
              if (m & 1) s1 += lv * tv[m];
              else s0 += lv * tv[m];
            }
            if (i > lc) tv[i] = -(s0 + s1);
          }
          u32x4 w0, w1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = pack2(tv[2 * e], tv[2 * e + 1]);
            w1[e] = pack2(tv[8 + 2 * e], tv[9 + 2 * e]);
          }
          *reinterpret_cast<u32x4*>(&sm.d[nb][lg][lc][0]) = w0;
          *reinterpret_cast<u32x4*>(&sm.d[nb][lg][lc][8]) = w1;
        });
  } else if (wave == 2 || wave == 3 || wave == 7) {
    // ======================= product waves =======================
    // Row blocks I0..I1 of K K^T (phase 1) and tril(Q K^T) (phase 2) of
    // chunk c+1, tile lists fixed at compile time: wave 2 row 3, wave 3
    // row 2, wave 7 rows 0 and 1.  All fragments of a row block are
    // requested before its MFMAs.
    auto prod = [&](auto i0c, auto i1c) {
      constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
      run(
          [&](const int c, auto parity) {
            constexpr int nb = 1 - decltype(parity)::value;  // buffer of chunk c+1
            if (c + 1 >= nch) return;
            const int kn = mod3(c + 1);
            // K K^T -> L = diag(beta) (.) strictly below the diagonal
#pragma unroll
            for (int i = I0; i <= I1; ++i) {
              bf16x8 fb[4][4];
#pragma unroll
              for (int j = 0; j <= i; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fb[j][kb] = ld_frag(&sm.k[kn][16 * j + lc][32 * kb + 8 * lg]);
              floatx4 acc[4];
#pragma unroll
              for (int j = 0; j <= i; ++j) {
                acc[j] = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc[j] = mfma_k32(fb[i][kb], fb[j][kb], acc[j]);
              }
              // diagonal tile: fp32 strictly-lower part for the D wave;
              // off-diagonal tiles: bf16, transposed (lane writes row lc,
              // columns 4 lg .. 4 lg + 3 of L_ij^T)
              const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[nb][16 * i + 4 * lg]);
#pragma unroll
              for (int j = 0; j < i; ++j) {
                uint2 w;
                w.x = pack2(bt.x * acc[j][0], bt.y * acc[j][1]);
                w.y = pack2(bt.z * acc[j][2], bt.w * acc[j][3]);
                *reinterpret_cast<uint2*>(&sm.lb[nb][i * (i - 1) / 2 + j][lc][4 * lg]) = w;
              }
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) {
                const int r = 16 * i + 4 * lg + ii, cc = 16 * i + lc;
                if (cc < r) sm.l[r][cc] = (ii == 0 ? bt.x : ii == 1 ? bt.y : ii == 2 ? bt.z : bt.w) * acc[i][ii];
              }
            }
          },
          [&](const int c, auto parity) {
            constexpr int nb = 1 - decltype(parity)::value;
            if (c + 1 >= nch) return;
            const int kn = mod3(c + 1);
            // tril(Q K^T), token columns permuted
#pragma unroll
            for (int i = I0; i <= I1; ++i) {
              bf16x8 fq[4], fb[4][4];
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) fq[kb] = ld_frag(&sm.q[nb][16 * i + lc][32 * kb + 8 * lg]);
#pragma unroll
              for (int j = 0; j <= i; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fb[j][kb] = ld_frag(&sm.k[kn][16 * j + lc][32 * kb + 8 * lg]);
              floatx4 acc[4];
#pragma unroll
              for (int j = 0; j <= i; ++j) {
                acc[j] = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc[j] = mfma_k32(fq[kb], fb[j][kb], acc[j]);
              }
#pragma unroll
              for (int j = 0; j <= i; ++j)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                  const int r = 16 * i + 4 * lg + ii, cc = 16 * j + lc;
                  sm.a[nb][r][perm32(cc)] = f2bf(cc <= r ? acc[j][ii] : 0.f);
                }
            }
          });
    };
    if (wave == 2) prod(std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{});
    else if (wave == 3) prod(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
    else prod(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  } else {
    // ======================= output waves (4, 5) =======================
    // Wave 4 writes the output tile of chunk c-1 (left in LDS by the chain
    // waves) to memory with 16-byte stores; both waves also load.
    const int sw = tid - 256;  // 0..127
    auto store_o = [&](int chunk) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int v = sw + 64 * j;
        const int r = v >> 2, c8 = (v & 3) * 8;
        *reinterpret_cast<u32x4*>(oh + (size_t)(chunk * kC + r) * dv + c8) =
            *reinterpret_cast<const u32x4*>(&sm.o[r][c8]);
      }
    };
    run([&](const int c, auto parity) {
          if (wave == 4 && c >= 1) store_o(c - 1);
        },
        [&](const int c, auto parity) {});
    if (wave == 4) store_o(nch - 1);
  }
}

hipError_t launch_prefill_pipe(const PrefillArgs& a, hipStream_t st) {
  const long blocks = (long)a.B * a.H * (a.dv / kDVS);
  hipLaunchKernelGGL(prefill_delta_pipe, dim3((unsigned)blocks), dim3(kThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace linattn

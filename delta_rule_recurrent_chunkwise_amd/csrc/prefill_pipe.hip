// prefill_pipe.hip -- software-pipelined chunkwise delta-rule prefill, plain
// and with a per-key-channel gate, for bf16 inputs with dk = 128 and dv a
// multiple of 32.
//
// Arithmetic (article "From GPT-2 to Kimi K3, explained"):
//  * section "DeltaNet (Parallelizing Linear Transformers with Delta Rule)":
//    per 64-token chunk, with L = tril(diag(beta) K K^T, -1),
//      u = (I + L)^-1 diag(beta) (V - K S),  O = Q S + tril(Q K^T) u,
//      S <- S + K^T u.
//  * sections "Gated Delta Net" and "KDA / Kimi Linear": a decay a_t[i] per
//    key channel scales row i of S before each read.  With the decay
//    accumulated from the chunk start, Gam_t = prod_{s<=t} a_s, the same
//    form holds with K~ = Gam K, K^ = K / Gam, Q~ = Gam Q (row-wise):
//      L = tril(diag(beta) K~ K^^T, -1),  u = (I + L)^-1 diag(beta) (V - K~ S),
//      O = Q~ S + tril(Q~ K^^T) u,  S <- diag(Gam_C) (S + K^^T u),
//    since (K Gam_C / Gam)^T u = diag(Gam_C) K^^T u.  A pre-pass (gate_prep
//    below) forms K~, K^, Q~ and Gam_C for every chunk; the main kernel is
//    the plain one with K~ in place of K on the left of every product, K^ on
//    the right, and the row scaling by Gam_C.
//  * one decay per token (Gated DeltaNet): the same identity with scalar
//    Gam_t = exp(G_t), G_t the log-decay summed from the chunk start, is
//    applied to the products' entries instead of the operands: entry (r, c)
//    of tril(Q K^T) and of L is scaled by exp(G_r - G_c), the rows of Q S and
//    K S by exp(G_r), the state by exp(G_C) and the rows of u by
//    exp(G_C - G_r) before S += K^T u.  No factor exceeds 1, there is no
//    pre-pass, and the kernel is otherwise the plain one.
//
// (I + L)^-1 is never formed: with I + L cut into 16x16 token blocks, u is
// obtained by block forward substitution,
//   u_b = D_b (X_b - sum_{j<b} L_bj u_j),   D_b = (I + L_bb)^-1.
//
// Work split inside a workgroup (8 waves; one (batch, head) and 32 value
// columns per workgroup).  Iteration x has two phases, each closed by an
// LDS-only barrier:
//   waves 0-1    "chain": each keeps S[:, 16 columns] in MFMA accumulators.
//                Phase 1: Y = K S, O = Q S, X = beta (V - Y) for chunk x.
//                Phase 2: u, O += tril(Q K^T) u, S += K^T u for chunk x.
//   waves 2,3,7  products.  Phase 1: tril(Q K^T) of chunk x.  Phase 2: L of
//                chunk x+1 (diagonal blocks fp32, the others bf16).
//   wave 6       D_b of chunk x from L's diagonal blocks (phase 1).
//   wave 4       writes the output tile of chunk x-1 to memory (phase 1).
//   loaders      write chunk x+1 to LDS in phase 1 of iteration x and issue
//                the global loads of chunk x+3 into the freed registers.
// Chunk y lives in LDS buffer y & 1: it is written in phase 1 of iteration
// y-1 and last read in phase 2 of iteration y.  (Tiles stored two chunks
// ahead in phase 2 take three buffers, or two if not read in phase 2 of their
// own chunk; a tile read only in phase 1 and stored in phase 2 takes one.)
//
// Index conventions.  Q, K (and K^) and the v slice are stored row-major
// (tokens x channels).  The chain's 32-deep MFMA pairs two accumulator
// tiles; the k-index order of that pairing is absorbed by a fixed
// permutation of S's rows: accumulator row rho = 32b + 16h + 4g + i of a
// chain wave holds key channel perm32(rho) = 32b + 8g + 4h + i.
// tril(Q K^T), an A operand against paired tiles over tokens, stores its
// token columns permuted the same way.  K^T (for S += K^T u), V in
// accumulator layout, and the 16x16 blocks D_b, L_bj (stored transposed) are
// read with the LDS transpose read ds_read_b64_tr_b16: lane 16G + 4a + b
// receives element b of the 8-byte runs addressed by lanes 16G + a + 4e,
// e = 0..3.  Row strides are 8 (mod 32) dwords, which keeps 16-byte fragment
// reads of 16 rows and transpose reads of 4-8 rows in distinct LDS banks.
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace linattn {
namespace {

constexpr int kC = 64;
constexpr int kDK = 128;
constexpr int kThreads = 512;

constexpr int kLQ = kDK + 16;   // bf16 row stride of q, k, k^ (72 dwords)
constexpr int kLT = kC + 16;    // bf16 row stride of tril(QK^T) (40 dwords)
constexpr int kLR = 20;         // fp32 row stride inside a diagonal block of L
constexpr int kLB = 16 * kLR + 16;  // fp32 stride between diagonal blocks

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Buffer access for the loader and output waves: a resource whose base is
// the chunk's first row and whose size ends at the chunk's last row that
// exists.  A 16-byte access then needs only its lane's offset (loop-invariant,
// with compile-time parts folded into the instruction's immediate) and no
// per-access address arithmetic; accesses past the size read zeros and write
// nothing (the hardware's range check on the vector offset).  0x00020000 is
// the resource's fourth word for gfx9-family targets.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load16(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(decltype(__builtin_amdgcn_raw_buffer_load_b128(r, 0, 0, 0)), v), r, off, 0, 0);
}
typedef short shortx4_t __attribute__((ext_vector_type(4)));

// DVS: value columns per workgroup (32, or 16 when there are too few
// (batch, head) pairs to fill the GPU with 32-column slices).
// GM: 0 plain, 1 decay per key channel (operands from the pre-pass), 2 one
// decay per token.
template <int GM, int DVS>
struct __attribute__((aligned(16))) Smem2 {
  static constexpr bool GATED = GM == 1;
  static constexpr bool TOKG = GM == 2;
  static constexpr int kLV = DVS + 16;  // bf16 row stride of the v slice
  static constexpr int kLO = DVS + 8;   // bf16 row stride of the output tile
  // Buffers per tile (see the loader schedule).  Gated with 16-column
  // slices (three tile waves): Q stored in phase 2 for the next chunk (one
  // buffer), Gam K and K / Gam two chunks ahead in phase 2 (two and three).
  static constexpr bool kShift = GATED && DVS == 16;
  static constexpr int NQB = kShift ? 1 : 2;
  static constexpr int NKH = GATED ? (kShift ? 3 : 2) : 1;
  static constexpr int RKH = GATED ? kC : 1;
  static constexpr int NKB = GATED ? 2 : 3;
  // K first: its buffer is chosen at run time, and fragment offsets from one
  // base register stay within the 16-bit immediate of the LDS instructions
  bf16_t k[NKB][kC][kLQ];     // K (gated: Gam K)
  bf16_t q[NQB][kC][kLQ];     // Q (gated: Gam Q)
  bf16_t kh[NKH][RKH][kLQ];   // gated: K / Gam
  bf16_t a[kC][kLT];          // tril(Q K^T), token columns permuted
  bf16_t lb[2][6][16][16];    // L_bj (b > j), transposed
  bf16_t d[4][16][16];        // D_b, transposed
  bf16_t v[2][kC][kLV];       // v slice
  bf16_t o[2][kC][kLO];       // output tile of chunk c in buffer c & 1
  float l[4 * kLB];           // diagonal blocks of L (strictly lower parts)
  float beta[2][kC];
  float gc[GATED ? 2 : 1][kDK];  // gated: Gam_C per key channel, chunk c in buffer c & 1
  // per-token decay of chunk c in buffer c & 1: G_t, exp(G_t), exp(G_63 - G_t)
  float gs[TOKG ? 2 : 1][3][TOKG ? kC : 1];
};

// 32b + 16h + 4g + i  ->  32b + 8g + 4h + i
__device__ __forceinline__ int perm32(int x) {
  return (x & ~31) | (((x >> 2) & 3) << 3) | (((x >> 4) & 1) << 2) | (x & 3);
}

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Consecutive logical workgroups (the dv slices of one head, which read the
// same q and k) go to one XCD, so they share its L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  if (n % 8 != 0) return bid;
  return (bid % 8) * (n / 8) + bid / 8;
}

__device__ __forceinline__ bf16x8 ld_frag(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
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

struct PipeArgs {
  const bf16_t* q;     // Q, or Gam Q
  const bf16_t* k;     // K, or Gam K
  const bf16_t* kh;    // gated: K / Gam
  const float* gc;     // gated: Gam_C, [B*H][ceil(T/64)][dk]
  const bf16_t* g;     // per-token gate: log-decay [B*H][T]
  const bf16_t* v;
  const bf16_t* beta;
  bf16_t* o;
  float* S;
  int T, dv, use_init;
  int Tq;              // rows per head of q, k, k^: T, or T rounded up to 64 (gated)
  float* Sc;           // if set: the state entering every chunk, bf16, [B*H][nch] x dk x dv in accumulator-tile order
};

// Loads.  Each tile-loader wave owns whole tiles (Q, K, and, gated, K^) and
// lane `lane` of it loads 16-byte vectors lane + 64 j of a tile (rows 4j +
// lane/16, 8 columns each).  Wave 7 loads the v slice, beta and (gated)
// Gam_C.  Every lane issues every load of its slots: a per-lane condition
// around a load would make the compiler wait for all outstanding loads.
//   plain:            wave 4 Q, wave 5 K; two register slots.
//   gated, 16 cols:   wave 1 (no chain work) Q, wave 4 K, wave 5 K^; two slots;
//                     K and K^ are stored two chunks ahead, in phase 2.
//   gated, 32 cols:   wave 4 Q + half of K^, wave 5 K + the other half; one
//                     slot (96 registers).
// With two slots the loads of chunk y are issued in iteration y-3 and stored
// in iteration y-1 (y-4 and y-2 for a tile stored two chunks ahead); with
// one, issued in iteration y-2.
template <bool GATED, int DVS>
struct LoadPlan {
  static constexpr bool kThree = GATED && DVS == 16;           // three tile waves
  static constexpr int NT = (GATED && !kThree) ? 24 : 16;      // tile vectors per lane
  static constexpr int NSLOT = NT > 16 ? 1 : 2;
  static constexpr int NS = NT;                                // registers per slot
  __device__ static bool is_tile_wave(int wave) { return wave == 4 || wave == 5 || (kThree && wave == 1); }
  // tile (0 Q, 1 K, 2 K^) and vector index within it of slot j
  __device__ static int tile_of(int wave, int j) {
    if (kThree) return wave == 1 ? 0 : (wave == 4 ? 1 : 2);
    if (GATED && j >= 16) return 2;
    return wave == 4 ? 0 : 1;
  }
  __device__ static int vec_of(int wave, int lane, int j) {
    if (GATED && !kThree && j >= 16) return 512 * (wave - 4) + lane + 64 * (j - 16);
    return lane + 64 * j;
  }
};

// CAP: also write the state entering every chunk to a.Sc (backward pass,
// which passes a.o = NULL: then neither the output nor the final state is
// written; a run-time test, which kept the register allocation free of
// spills where the compile-time one did not).  The output itself is not
// formed under CAP (compile time): no Q tiles, no Q S, no tril(Q K^T), no
// O += tril(Q K^T) u; the state needs K, V and beta only.
template <int GM, int DVS, bool CAP = false>
__global__ __launch_bounds__(kThreads) void prefill_pipe(PipeArgs a) {
  constexpr bool GATED = GM == 1;  // per key channel, operands from the pre-pass
  constexpr bool TOKG = GM == 2;   // one decay per token
  typedef Smem2<GM, DVS> Sm;
  constexpr bool kShift = Sm::kShift;  // gated, 16 columns: one Q buffer, K^ chunk c in buffer c % 3
  constexpr bool kOut = !CAP;          // the output is formed (not when only the chunk states are wanted)
  constexpr int kDVS = DVS;
  constexpr int NCW = DVS / 16;        // chain waves
  constexpr int VPRV = DVS / 8;        // 16-byte vectors per row of the v slice
  constexpr int NVL = kC * VPRV / 64;  // v-slice vectors per lane of wave 7
  typedef LoadPlan<GATED, DVS> LP;
  __shared__ Sm sm;

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
  const int nch = (Tn + kC - 1) / kC;
  // A last chunk with fewer than 64 tokens: loads of rows past the end
  // re-read the last row (every lane still issues every load), and those
  // rows get beta = 0 where they are staged in LDS.  Then their rows of L
  // and of X = beta (V - K S) vanish, so their u rows are zero and they
  // change neither S nor the outputs of earlier tokens; their own outputs
  // are not stored.  (The gate pre-pass gives them zero log-decay.)
  const int qlast = a.Tq - 1, tlast = Tn - 1;

  const bf16_t* qh = a.q + (size_t)bh * a.Tq * kDK;
  const bf16_t* kh = a.k + (size_t)bh * a.Tq * kDK;
  const bf16_t* khh = GATED ? a.kh + (size_t)bh * a.Tq * kDK : nullptr;
  const float* gch = GATED ? a.gc + (size_t)bh * nch * kDK : nullptr;
  const bf16_t* vh = a.v + (size_t)bh * Tn * dv + sl * kDVS;
  const bf16_t* bth = a.beta + (size_t)bh * Tn;
  const bf16_t* gth = TOKG ? a.g + (size_t)bh * Tn : nullptr;
  bf16_t* oh = a.o + (size_t)bh * Tn * dv + sl * kDVS;
  float* Sh = a.S + (size_t)bh * kDK * dv + sl * kDVS;

  // Tiles above the diagonal of tril(QK^T) are read as zeros.
  {
    uint32_t* z = reinterpret_cast<uint32_t*>(&sm.a[0][0]);
    for (int i = tid; i < (int)(sizeof(sm.a) / 4); i += kThreads) z[i] = 0u;
  }

  // load kind of a role, fixed at compile time: 0 none, 1 tiles (q, k, k^),
  // 2 wave 7's v slice, beta and Gam_C
  constexpr int NSMALL = NVL + (GATED ? 1 : 0);
  auto issue_loads = [&](auto kindc, int chunk, auto& dst, uint32_t* bdst) {
    constexpr int KIND = decltype(kindc)::value;
    if constexpr (KIND == 1) {
      // rows of the chunk that exist (chunk <= nch - 1: at least one); rows
      // past them read zeros, which get beta = 0 where they are staged
      const int rows = min(qlast + 1 - chunk * kC, kC);
      const uint32_t nb = (uint32_t)rows * kDK * 2;
      const size_t cb = (size_t)chunk * kC * kDK;
      const rsrc_t r0 = buf_rsrc(qh + cb, nb), r1 = buf_rsrc(kh + cb, nb);
      const rsrc_t r2 = GATED ? buf_rsrc(khh + cb, nb) : r1;
#pragma unroll
      for (int j = 0; j < LP::NT; ++j) {
        const int t = LP::tile_of(wave, j);
        const int vv = LP::vec_of(wave, lane, j);
        dst[j] = buf_load16(t == 0 ? r0 : (t == 1 ? r1 : r2), (uint32_t)((vv >> 4) * kDK + (vv & 15) * 8) * 2);
      }
    } else if constexpr (KIND == 2) {  // wave 7
#pragma unroll
      for (int j = 0; j < NVL; ++j) {
        const int vv = lane + 64 * j;  // row vv / VPRV, eight columns
        const int row = min(chunk * kC + vv / VPRV, tlast);
        dst[j] = *reinterpret_cast<const u32x4*>(vh + (size_t)row * dv + (vv % VPRV) * 8);
      }
      if constexpr (GATED) dst[NVL] = *reinterpret_cast<const u32x4*>(gch + (size_t)chunk * kDK + 4 * (lane & 31));
      const int row = min(chunk * kC + lane, tlast);
      bdst[0] = bth[row];  // converted when stored
      if constexpr (TOKG) bdst[1] = gth[row];
    }
  };
  auto store_loads = [&](auto kindc, int chunk, int buf, int kbi, const auto& src, const uint32_t* bsrc) {
    constexpr int KIND = decltype(kindc)::value;
    if constexpr (KIND == 1) {
#pragma unroll
      for (int j = 0; j < LP::NT; ++j) {
        const int t = LP::tile_of(wave, j);
        bf16_t(*tile)[kLQ] = t == 0 ? sm.q[kShift ? 0 : buf]
                                    : (t == 1 ? sm.k[kbi] : sm.kh[GATED ? (kShift ? chunk % 3 : buf) : 0]);
        const int vv = LP::vec_of(wave, lane, j);
        *reinterpret_cast<u32x4*>(&tile[vv >> 4][(vv & 15) * 8]) = src[j];
      }
    } else if constexpr (KIND == 2) {  // wave 7
#pragma unroll
      for (int j = 0; j < NVL; ++j) {
        const int vv = lane + 64 * j;
        *reinterpret_cast<u32x4*>(&sm.v[buf][vv / VPRV][(vv % VPRV) * 8]) = src[j];
      }
      if constexpr (GATED) {
        if (lane < 32) *reinterpret_cast<u32x4*>(&sm.gc[GATED ? buf : 0][4 * lane]) = src[NVL];
      }
      const bool in = chunk * kC + lane <= tlast;
      sm.beta[buf][lane] = in ? bf2f((bf16_t)bsrc[0]) : 0.f;
      if constexpr (TOKG) {
        // G_t = sum_{s<=t} g_s over the chunk (lane = token), then the
        // factors exp(G_t) and exp(G_63 - G_t), both at most 1
        const float x = scan64_up(in ? bf2f((bf16_t)bsrc[1]) : 0.f);
        const float gC = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), kC - 1));
        sm.gs[TOKG ? buf : 0][0][lane] = x;
        sm.gs[TOKG ? buf : 0][1][lane] = __expf(x);
        sm.gs[TOKG ? buf : 0][2][lane] = __expf(gC - x);
      }
    }
  };

  // K buffer of chunk c: three in rotation (plain), two by parity (gated)
  auto kidx = [&](int c) { return GATED ? (c & 1) : (c % 3); };

  // Every role runs its own copy of the chunk loop (the same barriers, only
  // its own registers live).  body(x, parity) runs iteration x with
  // parity = x & 1 known at compile time, so buffer and register-slot
  // indices are static.  A loader's schedule SCH: 0 stores chunk x+1 in
  // phase 1 of iteration x; 1 stores it in phase 2; 2 stores chunk x+2 in
  // phase 2 (chunk 0 goes to LDS before the loop).  Phase 1 carries most of
  // the LDS reads, so stores moved out of it wait less.
  auto run = [&](auto phase1, auto phase2, auto kindc, auto schc) {
    constexpr int KIND = decltype(kindc)::value;
    constexpr int SCH = decltype(schc)::value;
    constexpr int LEAD = SCH == 2 ? 2 : 1;
    constexpr bool loader = KIND != 0;
    constexpr int NSL = KIND == 1 ? LP::NSLOT : 2;
    constexpr int NREG = KIND == 1 ? LP::NT : (KIND == 2 ? NSMALL : 1);
    static_assert(LEAD == 1 || NSL == 2, "a two-chunk lead needs two register slots");
    u32x4 pf[NSL][NREG];
    uint32_t pfb[NSL][2] = {};  // beta and (per-token gate) g of each slot
    if (loader) {
      issue_loads(kindc, 0, pf[0], pfb[0]);
      if constexpr (LEAD == 2) {
        store_loads(kindc, 0, 0, 0, pf[0], pfb[0]);
        issue_loads(kindc, nch > 1 ? 1 : 0, pf[1], pfb[1]);
        issue_loads(kindc, nch > 2 ? 2 : nch - 1, pf[0], pfb[0]);
      } else if (NSL == 2) {
        issue_loads(kindc, nch > 1 ? 1 : 0, pf[NSL - 1], pfb[NSL - 1]);
      }
    }
    // The loads are issued on every path (past the last chunk they re-read
    // it and the registers are not stored): a path without them would make
    // the compiler assume the slot being stored holds the newest loads and
    // wait for every outstanding load and store of the wave.
    auto body = [&](const int x, auto parity) {
      constexpr int P = decltype(parity)::value;
      constexpr int PC = (P + LEAD) & 1;             // parity of chunk x + LEAD
      constexpr int SL = NSL == 2 ? PC : 0;          // its register slot
      auto move = [&] {
        const int c = x + LEAD;
        if (c < nch) store_loads(kindc, c, PC, kidx(c), pf[SL], pfb[SL]);
        issue_loads(kindc, c + NSL < nch ? c + NSL : nch - 1, pf[SL], pfb[SL]);
      };
      phase1(x, parity);
      if (loader && SCH == 0) move();
      lds_barrier();
      phase2(x, parity);
      if (loader && SCH != 0) move();
      lds_barrier();
    };
    // Both bodies run on every trip (no path back to the loop head skips
    // the second one's loads); an odd chunk left over runs after the loop.
    int x = -1;
    for (; x + 1 < nch; x += 2) {
      body(x, std::integral_constant<int, 1>{});
      body(x + 1, std::integral_constant<int, 0>{});
    }
    if (x < nch) body(x, std::integral_constant<int, 1>{});
  };

  if (wave < NCW) {
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
    // Without the per-channel gate ox[mt] holds the output tile transposed
    // (the output products take their operands in swapped order): lane
    // (lc, lg) has token 16mt + lc, value columns 16wave + 4lg .. +3, one
    // 8-byte LDS store instead of four 2-byte ones.  The per-channel gated
    // kernel keeps the untransposed tile (the swap made it spill).
    constexpr bool kOT = !GATED;
    floatx4 xx[4], ox[4];
    // Per-channel gate, a chunk the pre-pass marked (Gam_C < 0): its decay
    // leaves the range of the factored form, so it is walked token by token
    // with the recurrence itself, S <- diag(a_t) S, u = beta_t (v_t - k_t S),
    // S += k_t^T u, o_t = q_t S, on the raw q, k and g the pre-pass staged in
    // its slots.  Lane (lc, lg) holds column col of rows 16t + 4lg + i, i.e.
    // key channels perm32(16t + 4lg) + i; the sums over channels are
    // completed across the four lanes that share a column.
    auto token_walk = [&](const int x, auto parity) {
      constexpr int P = decltype(parity)::value;
      for (int tau = 0; tau < kC; ++tau) {
        float kk[8][4], qq[8][4];
        float r = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int c0 = perm32(16 * t + 4 * lg);
          const uint2 kw = *reinterpret_cast<const uint2*>(&sm.k[GATED ? P : 0][tau][c0]);
          const uint2 qw = *reinterpret_cast<const uint2*>(&sm.q[kShift ? 0 : P][tau][c0]);
          const uint2 gw = *reinterpret_cast<const uint2*>(&sm.kh[GATED ? (kShift ? x % 3 : P) : 0][GATED ? tau : 0][c0]);
          const uint32_t kv[2] = {kw.x, kw.y}, qv[2] = {qw.x, qw.y}, gv[2] = {gw.x, gw.y};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint32_t sh = (i & 1) ? 16u : 0u;
            kk[t][i] = bf2f((bf16_t)(kv[i >> 1] >> sh));
            qq[t][i] = bf2f((bf16_t)(qv[i >> 1] >> sh));
            st[t][i] *= __expf(bf2f((bf16_t)(gv[i >> 1] >> sh)));
            r += kk[t][i] * st[t][i];
          }
        }
        r = xsum32(xsum16(r));
        const float u = sm.beta[P][tau] * (bf2f(sm.v[P][tau][col]) - r);
        float o = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            st[t][i] += kk[t][i] * u;
            o += qq[t][i] * st[t][i];
          }
        if constexpr (kOut) {
          o = xsum32(xsum16(o));
          if (lg == 0) sm.o[P][tau][col] = f2bf(o);
        }
      }
    };
    run(
        [&](const int x, auto parity) {
          constexpr int P = decltype(parity)::value;
          if (x < 0) return;
          if constexpr (CAP) {  // the state entering chunk x, for the backward pass
            // row perm32(16t + 4lg + i) = 8lg + 32(t / 2) + 4(t % 2) + i: one
            // lane-dependent base, offsets uniform across the wave
            // (bf16, the precision the gradient pass reads it in), in
            // accumulator-tile order: tile (kt, jt) of chunk x at
            // ((x * dk/16 + kt) * dv/16 + jt) * 256, lane l's four rows at 4l.
            // Accumulator rows 16t + 4lg + i hold key channels 32(t/2) + 8lg +
            // 4(t%2) + i: tile 2(t/2) + lg/2, lane group 2(lg%2) + t%2.
            bf16_t* scb = reinterpret_cast<bf16_t*>(a.Sc) + ((size_t)bh * nch + x) * kDK * dv;
            const int jt = sl * (kDVS / 16) + wave;
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const int kt = 2 * (t >> 1) + (lg >> 1), lgt = 2 * (lg & 1) + (t & 1);
              *reinterpret_cast<uint2*>(scb + ((size_t)kt * (dv / 16) + jt) * 256 + 4 * (16 * lgt + lc)) =
                  make_uint2(pack2(st[t][0], st[t][1]), pack2(st[t][2], st[t][3]));
            }
          }
          if constexpr (GATED) {
            if (sm.gc[P][0] < 0.f) {
              token_walk(x, parity);
              return;
            }
          }
          // Y = K S and O = Q S (shared S fragments), X = beta (V - Y); the
          // fragments of k-step kb+1 are loaded while kb computes.
          floatx4 y[4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) { y[mt] = zero4(); ox[mt] = zero4(); }
          const bf16_t(*kx)[kLQ] = sm.k[GATED ? P : kidx(x)];
          bf16x8 fk[2][4], fq[2][4];
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            fk[0][mt] = ld_frag(&kx[16 * mt + lc][8 * lg]);
            if constexpr (kOut) fq[0][mt] = ld_frag(&sm.q[kShift ? 0 : P][16 * mt + lc][8 * lg]);
          }
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            if (kb < 3) {
#pragma unroll
              for (int mt = 0; mt < 4; ++mt) {
                fk[(kb + 1) & 1][mt] = ld_frag(&kx[16 * mt + lc][32 * (kb + 1) + 8 * lg]);
                if constexpr (kOut)
                  fq[(kb + 1) & 1][mt] = ld_frag(&sm.q[kShift ? 0 : P][16 * mt + lc][32 * (kb + 1) + 8 * lg]);
              }
            }
            const bf16x8 b = acc_pair_to_b(st[2 * kb], st[2 * kb + 1]);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              y[mt] = mfma_k32(fk[kb & 1][mt], b, y[mt]);
              if constexpr (kOut)
                ox[mt] = kOT ? mfma_k32(b, fq[kb & 1][mt], ox[mt]) : mfma_k32(fq[kb & 1][mt], b, ox[mt]);
            }
          }
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) {
            // lane (lg, lc) gets V[16 mt + 4 lg + i][col], i = 0..3
            const shortx4_t vw =
                ld_tr(&sm.v[P][16 * mt + 4 * lg + ((lane >> 2) & 3)][16 * wave + 4 * (lane & 3)]);
            const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[P][16 * mt + 4 * lg]);
            if constexpr (TOKG) {  // rows of K S and Q S decay by exp(G_r)
              const float4 dc = *reinterpret_cast<const float4*>(&sm.gs[TOKG ? P : 0][1][16 * mt + 4 * lg]);
              y[mt][0] *= dc.x; y[mt][1] *= dc.y; y[mt][2] *= dc.z; y[mt][3] *= dc.w;
              if constexpr (kOut) ox[mt] *= sm.gs[TOKG ? P : 0][1][16 * mt + lc];  // the lane's token
            }
            xx[mt][0] = bt.x * (bf2f((bf16_t)vw[0]) - y[mt][0]);
            xx[mt][1] = bt.y * (bf2f((bf16_t)vw[1]) - y[mt][1]);
            xx[mt][2] = bt.z * (bf2f((bf16_t)vw[2]) - y[mt][2]);
            xx[mt][3] = bt.w * (bf2f((bf16_t)vw[3]) - y[mt][3]);
          }
        },
        [&](const int x, auto parity) {
          constexpr int P = decltype(parity)::value;
          if (x < 0) return;
          if constexpr (GATED) {
            if (sm.gc[P][0] < 0.f) return;  // walked token by token in phase 1
          }
          auto fr16 = [&](const bf16_t* blk) {  // A operand of a transposed 16x16 block
            return ld_tr(blk + (4 * lg + ((lane >> 2) & 3)) * 16 + 4 * (lane & 3));
          };
          shortx4_t fd[4], fl[6];
#pragma unroll
          for (int b = 0; b < 4; ++b) fd[b] = fr16(&sm.d[b][0][0]);
#pragma unroll
          for (int i = 0; i < 6; ++i) fl[i] = fr16(&sm.lb[P][i][0][0]);
          bf16x8 fa[6];
          if constexpr (kOut) {
            fa[0] = ld_frag(&sm.a[lc][8 * lg]);
            fa[1] = ld_frag(&sm.a[16 + lc][8 * lg]);
            fa[2] = ld_frag(&sm.a[32 + lc][8 * lg]);
            fa[3] = ld_frag(&sm.a[32 + lc][32 + 8 * lg]);
            fa[4] = ld_frag(&sm.a[48 + lc][8 * lg]);
            fa[5] = ld_frag(&sm.a[48 + lc][32 + 8 * lg]);
          }
          if constexpr (TOKG) {  // S <- exp(G_C) S before K^T u is added
            const float eC = sm.gs[TOKG ? P : 0][1][kC - 1];
#pragma unroll
            for (int t = 0; t < 8; ++t) st[t] *= eC;
          }
          // blocks L_bj stored in the order (1,0) (2,0) (2,1) (3,0) (3,1) (3,2)
          floatx4 ut[4];
          ut[0] = mfma_k16(fd[0], acc_to_b16(xx[0]), zero4());
          const shortx4_t u0 = acc_to_b16(ut[0]);
          ut[1] = mfma_k16(fd[1], acc_to_b16(xx[1] - mfma_k16(fl[0], u0, zero4())), zero4());
          const shortx4_t u1 = acc_to_b16(ut[1]);
          ut[2] = mfma_k16(fd[2], acc_to_b16(xx[2] - mfma_k16(fl[2], u1, mfma_k16(fl[1], u0, zero4()))),
                           zero4());
          const shortx4_t u2 = acc_to_b16(ut[2]);
          ut[3] = mfma_k16(
              fd[3], acc_to_b16(xx[3] - mfma_k16(fl[5], u2, mfma_k16(fl[4], u1, mfma_k16(fl[3], u0, zero4())))),
              zero4());
          // K^T fragments (K^ when gated): row 16t + c of the A operand is key
          // channel perm32(16t + c); its k-elements are the tokens of u's pairing.
          const bf16_t(*kt)[kLQ] = GATED ? sm.kh[GATED ? (kShift ? x % 3 : P) : 0] : sm.k[kidx(x)];
          // one lane base per chunk; every fragment is a compile-time offset
          // from it (an immediate of the read).  The empty asm makes the base
          // opaque: otherwise the compiler kept one loop-invariant address per
          // fragment in a register and rebuilt all 32 from the chunk's buffer
          // offset in every iteration (two vector operations each).
          uint32_t ktb = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const bf16_t*)
              &kt[4 * lg + ((lane >> 2) & 3)][8 * (lane & 3)];
          asm volatile("" : "+v"(ktb));
          const bf16_t* ktl = (const bf16_t*)(__attribute__((address_space(3))) const bf16_t*)(uintptr_t)ktb;
          auto kt_frag = [&](int t, int tok0) {
            const int cc = 32 * (t >> 1) + 4 * (t & 1);
            return cat_tr(ld_tr(ktl + tok0 * kLQ + cc), ld_tr(ktl + (tok0 + 16) * kLQ + cc));
          };
          bf16x8 fkt[2][8];
#pragma unroll
          for (int t = 0; t < 8; ++t) fkt[0][t] = kt_frag(t, 0);
          const bf16x8 u01 = acc_pair_to_b(ut[0], ut[1]);
          const bf16x8 u23 = acc_pair_to_b(ut[2], ut[3]);
          // O += tril(Q K^T) u
          if constexpr (!kOut) {
          } else if constexpr (kOT) {
            ox[0] = mfma_k32(u01, fa[0], ox[0]);
            ox[1] = mfma_k32(u01, fa[1], ox[1]);
            ox[2] = mfma_k32(u23, fa[3], mfma_k32(u01, fa[2], ox[2]));
            ox[3] = mfma_k32(u23, fa[5], mfma_k32(u01, fa[4], ox[3]));
          } else {
            ox[0] = mfma_k32(fa[0], u01, ox[0]);
            ox[1] = mfma_k32(fa[1], u01, ox[1]);
            ox[2] = mfma_k32(fa[3], u23, mfma_k32(fa[2], u01, ox[2]));
            ox[3] = mfma_k32(fa[5], u23, mfma_k32(fa[4], u01, ox[3]));
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) fkt[1][t] = kt_frag(t, 32);
          // S += K^T u (per-token gate: rows of u decay by exp(G_C - G_r))
          bf16x8 s01 = u01, s23 = u23;
          if constexpr (TOKG) {
            floatx4 us[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
              const float4 rm = *reinterpret_cast<const float4*>(&sm.gs[TOKG ? P : 0][2][16 * mt + 4 * lg]);
              us[mt][0] = ut[mt][0] * rm.x; us[mt][1] = ut[mt][1] * rm.y;
              us[mt][2] = ut[mt][2] * rm.z; us[mt][3] = ut[mt][3] * rm.w;
            }
            s01 = acc_pair_to_b(us[0], us[1]);
            s23 = acc_pair_to_b(us[2], us[3]);
          }
#pragma unroll
          for (int t = 0; t < 8; ++t) st[t] = mfma_k32(fkt[0][t], s01, st[t]);
#pragma unroll
          for (int t = 0; t < 8; ++t) st[t] = mfma_k32(fkt[1][t], s23, st[t]);
          if constexpr (GATED) {
            // S <- diag(Gam_C) S; accumulator rows 16t + 4lg + i are the
            // consecutive channels perm32(16t + 4lg) + i
#pragma unroll
            for (int t = 0; t < 8; ++t) {
              const float4 gv = *reinterpret_cast<const float4*>(&sm.gc[P][perm32(16 * t + 4 * lg)]);
              st[t][0] *= gv.x;
              st[t][1] *= gv.y;
              st[t][2] *= gv.z;
              st[t][3] *= gv.w;
            }
          }
          if constexpr (!kOut) {
          } else if constexpr (kOT) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
              *reinterpret_cast<uint2*>(&sm.o[P][16 * mt + lc][16 * wave + 4 * lg]) =
                  make_uint2(pack2(ox[mt][0], ox[mt][1]), pack2(ox[mt][2], ox[mt][3]));
          } else {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
              for (int i = 0; i < 4; ++i) sm.o[P][16 * mt + 4 * lg + i][col] = f2bf(ox[mt][i]);
          }
        },
        std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    if (a.o != nullptr) {  // the backward pass (no output) needs only the chunk states
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) Sh[(size_t)perm32(16 * t + 4 * lg + i) * dv + col] = st[t][i];
    }
  } else if (wave == 6) {
    // ======================= D wave =======================
    // D_b = (I + L_bb)^-1 of chunk x (phase 1): lane (block lg, column lc)
    // solves (I + L_bb) x = e_lc by forward substitution in fp32; x is column
    // lc of D_b, stored as row lc of D_b^T.
    run(
        [&](const int x, auto parity) {
          if (x < 0) return;
          const float* lbk = &sm.l[lg * kLB];
          float4 lr[16][4];  // strictly-lower rows of L_bb, requested up front
#pragma unroll
          for (int i = 1; i < 16; ++i)
#pragma unroll
            for (int m4 = 0; m4 < i; m4 += 4)
              lr[i][m4 >> 2] = *reinterpret_cast<const float4*>(lbk + i * kLR + m4);
          // right-looking: once x_m is known it is folded into the partial
          // sums of every later row, so one multiply-add separates x_m from
          // x_{m+1} (x_m = 0 for m < lc, x_lc = 1)
          float tv[16], ps[16];
#pragma unroll
          for (int i = 0; i < 16; ++i) ps[i] = 0.f;
#pragma unroll
          for (int m = 0; m < 16; ++m) {
            tv[m] = m < lc ? 0.f : (m == lc ? 1.f : -ps[m]);
#pragma unroll
            for (int i = m + 1; i < 16; ++i) {
              const float4 q4 = lr[i][m >> 2];
              const float lv = (m & 3) == 0 ? q4.x : (m & 3) == 1 ? q4.y : (m & 3) == 2 ? q4.z : q4.w;
              ps[i] += lv * tv[m];
            }
          }
          u32x4 w0, w1;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            w0[e] = pack2(tv[2 * e], tv[2 * e + 1]);
            w1[e] = pack2(tv[8 + 2 * e], tv[9 + 2 * e]);
          }
          *reinterpret_cast<u32x4*>(&sm.d[lg][lc][0]) = w0;
          *reinterpret_cast<u32x4*>(&sm.d[lg][lc][8]) = w1;
        },
        [&](const int x, auto parity) {}, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
  } else if (wave == 2 || wave == 3 || wave == 7) {
    // ======================= product waves =======================
    // Row blocks I0..I1: tril(Q K^T) of chunk x in phase 1, L of chunk x+1
    // in phase 2 (K^ on the right when gated).  Wave 2 row 3, wave 3 row 2,
    // wave 7 rows 0 and 1.  All fragments of a row block are requested
    // before its MFMAs.
    auto prod = [&](auto i0c, auto i1c) {
      constexpr int I0 = decltype(i0c)::value, I1 = decltype(i1c)::value;
      run(
          [&](const int x, auto parity) {
            constexpr int P = decltype(parity)::value;
            if (x < 0 || !kOut) return;  // tril(Q K^T) serves the output only
            const bf16_t(*rt)[kLQ] = GATED ? sm.kh[GATED ? (kShift ? x % 3 : P) : 0] : sm.k[kidx(x)];
#pragma unroll
            for (int i = I0; i <= I1; ++i) {
              bf16x8 fq[4], fb[4][4];
#pragma unroll
              for (int kb = 0; kb < 4; ++kb) fq[kb] = ld_frag(&sm.q[kShift ? 0 : P][16 * i + lc][32 * kb + 8 * lg]);
#pragma unroll
              for (int j = 0; j <= i; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fb[j][kb] = ld_frag(&rt[16 * j + lc][32 * kb + 8 * lg]);
              // the transposed product K Q^T: lane (lc, lg) gets row 16i + lc,
              // columns 16j + 4lg .. +3, which the token-column permutation
              // for the chain's pairing keeps contiguous: one 8-byte store
              floatx4 acc[4];
#pragma unroll
              for (int j = 0; j <= i; ++j) {
                acc[j] = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) acc[j] = mfma_k32(fb[j][kb], fq[kb], acc[j]);
              }
#pragma unroll
              for (int j = 0; j <= i; ++j) {
                const int r = 16 * i + lc, c0 = 16 * j + 4 * lg;
                if constexpr (TOKG) {  // decay from token c to token r (c <= r)
                  const float gr = sm.gs[TOKG ? P : 0][0][r];
                  const float4 gcl = *reinterpret_cast<const float4*>(&sm.gs[TOKG ? P : 0][0][c0]);
                  acc[j][0] *= c0 <= r ? __expf(gr - gcl.x) : 0.f;
                  acc[j][1] *= c0 + 1 <= r ? __expf(gr - gcl.y) : 0.f;
                  acc[j][2] *= c0 + 2 <= r ? __expf(gr - gcl.z) : 0.f;
                  acc[j][3] *= c0 + 3 <= r ? __expf(gr - gcl.w) : 0.f;
                }
                const float e0 = c0 <= r ? acc[j][0] : 0.f, e1 = c0 + 1 <= r ? acc[j][1] : 0.f;
                const float e2 = c0 + 2 <= r ? acc[j][2] : 0.f, e3 = c0 + 3 <= r ? acc[j][3] : 0.f;
                *reinterpret_cast<uint2*>(&sm.a[r][perm32(c0)]) = make_uint2(pack2(e0, e1), pack2(e2, e3));
              }
            }
          },
          [&](const int x, auto parity) {
            constexpr int nb = 1 - decltype(parity)::value;  // buffer of chunk x+1
            if (x + 1 >= nch) return;
            const bf16_t(*rt)[kLQ] = GATED ? sm.kh[GATED ? (kShift ? (x + 1) % 3 : nb) : 0] : sm.k[kidx(x + 1)];
#pragma unroll
            for (int i = I0; i <= I1; ++i) {
              bf16x8 fl[4], fb[4][4];
#pragma unroll
              for (int j = 0; j <= i; ++j)
#pragma unroll
                for (int kb = 0; kb < 4; ++kb) fb[j][kb] = ld_frag(&rt[16 * j + lc][32 * kb + 8 * lg]);
#pragma unroll
              for (int kb = 0; kb < 4; ++kb)  // left operand: K (gated: Gam K)
                fl[kb] = GATED ? ld_frag(&sm.k[GATED ? nb : 0][16 * i + lc][32 * kb + 8 * lg]) : fb[i][kb];
              // off-diagonal blocks as L (stored transposed below); the
              // diagonal block as the transposed product, so that a lane holds
              // four consecutive columns of one row (one 16-byte store)
              floatx4 acc[4];
#pragma unroll
              for (int j = 0; j <= i; ++j) {
                acc[j] = zero4();
#pragma unroll
                for (int kb = 0; kb < 4; ++kb)
                  acc[j] = j < i ? mfma_k32(fl[kb], fb[j][kb], acc[j]) : mfma_k32(fb[j][kb], fl[kb], acc[j]);
              }
              // L = diag(beta) (.): the diagonal tile's strictly-lower part in
              // fp32 for the D wave; off-diagonal tiles bf16, transposed (the
              // lane writes row lc, columns 4lg .. 4lg+3 of L_ij^T)
              const float4 bt = *reinterpret_cast<const float4*>(&sm.beta[nb][16 * i + 4 * lg]);
              if constexpr (TOKG) {  // decay from token c to token r
                const float4 grw = *reinterpret_cast<const float4*>(&sm.gs[TOKG ? nb : 0][0][16 * i + 4 * lg]);
#pragma unroll
                for (int j = 0; j < i; ++j) {  // rows 16i + 4lg + n, column 16j + lc
                  const float gcl = sm.gs[TOKG ? nb : 0][0][16 * j + lc];
                  acc[j][0] *= __expf(grw.x - gcl);
                  acc[j][1] *= __expf(grw.y - gcl);
                  acc[j][2] *= __expf(grw.z - gcl);
                  acc[j][3] *= __expf(grw.w - gcl);
                }
                // diagonal block: row 16i + lc, columns 16i + 4lg + n; only
                // the strictly lower entries are read
                const float gr = sm.gs[TOKG ? nb : 0][0][16 * i + lc];
                const float4 gcd = *reinterpret_cast<const float4*>(&sm.gs[TOKG ? nb : 0][0][16 * i + 4 * lg]);
                acc[i][0] *= 4 * lg < lc ? __expf(gr - gcd.x) : 0.f;
                acc[i][1] *= 4 * lg + 1 < lc ? __expf(gr - gcd.y) : 0.f;
                acc[i][2] *= 4 * lg + 2 < lc ? __expf(gr - gcd.z) : 0.f;
                acc[i][3] *= 4 * lg + 3 < lc ? __expf(gr - gcd.w) : 0.f;
              }
#pragma unroll
              for (int j = 0; j < i; ++j) {
                uint2 wv;
                wv.x = pack2(bt.x * acc[j][0], bt.y * acc[j][1]);
                wv.y = pack2(bt.z * acc[j][2], bt.w * acc[j][3]);
                *reinterpret_cast<uint2*>(&sm.lb[nb][i * (i - 1) / 2 + j][lc][4 * lg]) = wv;
              }
              // lane (lc, lg): row lc, columns 4lg .. 4lg+3 of the diagonal
              // block; entries on and above the diagonal are not read
              const float bl = sm.beta[nb][16 * i + lc];
              *reinterpret_cast<float4*>(&sm.l[i * kLB + lc * kLR + 4 * lg]) =
                  make_float4(bl * acc[i][0], bl * acc[i][1], bl * acc[i][2], bl * acc[i][3]);
            }
          },
          std::integral_constant<int, (I0 == 0 && I1 == 1) ? 2 : 0>{},  // wave 7 loads v, beta
          std::integral_constant<int, 0>{});
    };
    if (wave == 2) prod(std::integral_constant<int, 3>{}, std::integral_constant<int, 3>{});
    else if (wave == 3) prod(std::integral_constant<int, 2>{}, std::integral_constant<int, 2>{});
    else prod(std::integral_constant<int, 0>{}, std::integral_constant<int, 1>{});
  } else {
    // ============ output / load waves (4, 5; wave 1 idles when NCW = 1) ============
    // Wave 4 writes the output tile of chunk x-1 (left in LDS by the chain
    // waves) to memory with 16-byte stores, in phase 2 of iteration x, while
    // the chain waves fill the other buffer with chunk x.
    // Only the last chunk can be partial: it is stored after the loop, the
    // one place where rows past the end are skipped.
    const int sw = tid - 256;  // 0..63 on wave 4
    auto store_o = [&](int chunk, auto tailc) {
      // the resource ends at the last element of the slice's last row that
      // exists, so rows past the end are not written (and the tail skips them)
      const int rows = min(Tn - chunk * kC, kC);
      const rsrc_t ro = buf_rsrc(oh + (size_t)chunk * kC * dv, (uint32_t)((rows - 1) * dv + kDVS) * 2);
#pragma unroll
      for (int j = 0; j < kC * VPRV / 64; ++j) {
        const int vi = sw + 64 * j;
        const int r = vi / VPRV, c8 = (vi % VPRV) * 8;
        if (decltype(tailc)::value && chunk * kC + r > tlast) continue;
        buf_store16(ro, (uint32_t)(r * dv + c8) * 2, *reinterpret_cast<const u32x4*>(&sm.o[chunk & 1][r][c8]));
      }
    };
    auto ph1 = [&](const int x, auto parity) {};
    auto ph2 = [&](const int x, auto parity) {
      if (kOut && a.o != nullptr && wave == 4 && x >= 1) store_o(x - 1, std::false_type{});
    };
    // plain: Q of chunk x+1 and K of chunk x+2 are stored in phase 2 of x
    // (K(x+1) is read then, for L(x+1)); gated: K and K^ in phase 1, and
    // Q of chunk x+1 in phase 2 where a wave of its own loads it (16-column
    // slices)
    if (!GATED && wave == 4) run(ph1, ph2, std::integral_constant<int, kOut ? 1 : 0>{}, std::integral_constant<int, GATED ? 0 : 1>{});
    else if (!GATED && wave == 5) run(ph1, ph2, std::integral_constant<int, 1>{}, std::integral_constant<int, GATED ? 0 : 2>{});
    else if (LP::kThree && wave == 1)  // Q only: none without the output
      run(ph1, ph2, std::integral_constant<int, kOut ? 1 : 0>{}, std::integral_constant<int, LP::kThree ? 1 : 0>{});
    else if (LP::is_tile_wave(wave))  // gated K and K^: two chunks ahead in phase 2 (16 columns), else phase 1
      run(ph1, ph2, std::integral_constant<int, 1>{}, std::integral_constant<int, kShift ? 2 : 0>{});
    else run(ph1, ph2, std::integral_constant<int, 0>{}, std::integral_constant<int, 0>{});
    if (kOut && a.o != nullptr && wave == 4) store_o(nch - 1, std::true_type{});
  }
}

// Gate pre-pass: for each (batch, head, chunk) and key channel d, the
// cumulative log-decay G_t = sum_{s<=t} g_s over the chunk (fp32), then
// Gam Q, Gam K, K / Gam in bf16 and Gam_C = e^{G_63}.  One workgroup of 256
// threads per chunk: thread (w, l) holds channels 2l, 2l+1 of tokens
// TPS w .. TPS w + TPS - 1 (TPS = 16 at dk = 128, fewer rows per thread and
// more row groups at smaller dk); the row groups' partial sums are combined
// through LDS.  Inputs have T rows per head; the outputs have nch * 64, and
// rows past T (a partial last chunk) get g = 0 and q = k = 0, so Gam_C is the
// decay over the tokens that exist.
// A chunk in which some |G_t| exceeds kGateRange (a channel decays by more
// than e^-64 within it, so K / Gam would leave the float range) is not
// scaled: its q, k and g are copied as they are into the Gam Q, Gam K and
// K / Gam slots, and Gam_C is set to -1, which tells the main kernel (and the
// backward pass) to walk that chunk token by token.
constexpr float kGateRange = 64.f;

template <int DK>
__global__ __launch_bounds__(256) void gate_prep(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                 const bf16_t* __restrict__ g, bf16_t* __restrict__ qt,
                                                 bf16_t* __restrict__ kt, bf16_t* __restrict__ kht,
                                                 float* __restrict__ gcum, int T, int nch) {
  constexpr int NCOL = DK / 2, NSEG = 256 / NCOL, TPS = kC / NSEG;
  __shared__ float2 part[NSEG][NCOL];
  __shared__ int wide;
  const int chunk = blockIdx.x;  // over B*H*nch
  const int bh = chunk / nch, t0 = (chunk - bh * nch) * kC;
  const int w = threadIdx.x / NCOL, l = threadIdx.x % NCOL;
  const size_t base = (size_t)chunk * kC * DK;                  // outputs
  const size_t ibase = ((size_t)bh * T + t0) * DK;              // inputs
  const int nrow = min(kC, T - t0);                             // rows that exist
  const uint32_t* g2 = reinterpret_cast<const uint32_t*>(g + ibase);
  uint32_t gw[TPS];
#pragma unroll
  for (int t = 0; t < TPS; ++t) gw[t] = g2[min(TPS * w + t, nrow - 1) * NCOL + l];  // masked below
  // every q and k load of the thread too, in flight with g's: the compiler
  // cannot move a load above a store to the outputs, so loads next to the
  // stores below would each wait for the previous row's round trip
  const uint32_t* q2 = reinterpret_cast<const uint32_t*>(q + ibase);
  const uint32_t* k2 = reinterpret_cast<const uint32_t*>(k + ibase);
  uint32_t qv[TPS], kv[TPS];
#pragma unroll
  for (int t = 0; t < TPS; ++t) {
    const int iidx = min(TPS * w + t, nrow - 1) * NCOL + l;  // in bounds for every lane
    qv[t] = q2[iidx];
    kv[t] = k2[iidx];
  }
  float2 run = make_float2(0.f, 0.f);
  float2 gl[TPS];
#pragma unroll
  for (int t = 0; t < TPS; ++t) {
    const uint32_t gv = TPS * w + t < nrow ? gw[t] : 0u;
    run.x += bf2f((bf16_t)(gv & 0xffffu));
    run.y += bf2f((bf16_t)(gv >> 16));
    gl[t] = run;
  }
  part[w][l] = run;
  if (threadIdx.x == 0) wide = 0;
  __syncthreads();
  float2 off = make_float2(0.f, 0.f), tot = make_float2(0.f, 0.f);
#pragma unroll
  for (int p = 0; p < NSEG; ++p) {
    const float2 x = part[p][l];
    if (p < w) { off.x += x.x; off.y += x.y; }
    tot.x += x.x;
    tot.y += x.y;
  }
  // does any channel leave [-kGateRange, kGateRange] within the chunk?
  float mx = 0.f;
#pragma unroll
  for (int t = 0; t < TPS; ++t) mx = fmaxf(mx, fmaxf(fabsf(off.x + gl[t].x), fabsf(off.y + gl[t].y)));
  if (!(mx <= kGateRange)) wide = 1;  // also for NaN
  __syncthreads();
  uint32_t* qt2 = reinterpret_cast<uint32_t*>(qt + base);
  uint32_t* kt2 = reinterpret_cast<uint32_t*>(kt + base);
  uint32_t* kh2 = reinterpret_cast<uint32_t*>(kht + base);
  if (wide) {  // uniform over the workgroup: raw q, k, g and the marker
    if (w == 0) reinterpret_cast<float2*>(gcum + (size_t)chunk * DK)[l] = make_float2(-1.f, -1.f);
#pragma unroll
    for (int t = 0; t < TPS; ++t) {
      const int idx = (TPS * w + t) * NCOL + l;
      const bool in = TPS * w + t < nrow;
      qt2[idx] = in ? qv[t] : 0u;
      kt2[idx] = in ? kv[t] : 0u;
      kh2[idx] = in ? gw[t] : 0u;
    }
    return;
  }
  if (w == 0) reinterpret_cast<float2*>(gcum + (size_t)chunk * DK)[l] = make_float2(__expf(tot.x), __expf(tot.y));
#pragma unroll
  for (int t = 0; t < TPS; ++t) {
    const int idx = (TPS * w + t) * NCOL + l;
    const bool in = TPS * w + t < nrow;
    const uint32_t qw = in ? qv[t] : 0u, kw = in ? kv[t] : 0u;
    const float G0 = off.x + gl[t].x, G1 = off.y + gl[t].y;
    const float e0 = __expf(G0), e1 = __expf(G1), r0 = __expf(-G0), r1 = __expf(-G1);
    const float q0 = bf2f((bf16_t)(qw & 0xffffu)), q1 = bf2f((bf16_t)(qw >> 16));
    const float k0 = bf2f((bf16_t)(kw & 0xffffu)), k1 = bf2f((bf16_t)(kw >> 16));
    qt2[idx] = pack2(q0 * e0, q1 * e1);
    kt2[idx] = pack2(k0 * e0, k1 * e1);
    kh2[idx] = pack2(k0 * r0, k1 * r1);
  }
}

}  // namespace

namespace {

template <int GM, bool CAP = false>
hipError_t launch_pipe_t(const PipeArgs& p, long bh, int dv, hipStream_t st) {
  // 32 value columns per workgroup, or 16 when 32-column slices would leave
  // compute units idle (few (batch, head) pairs, as with long sequences)
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    cus = 256;
  if (bh * (dv / 32) < cus && dv % 16 == 0) {
    hipLaunchKernelGGL((prefill_pipe<GM, 16, CAP>), dim3((unsigned)(bh * (dv / 16))), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((prefill_pipe<GM, 32, CAP>), dim3((unsigned)(bh * (dv / 32))), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

namespace {
PipeArgs pipe_args(const PrefillArgs& a) {
  PipeArgs p{};
  p.v = reinterpret_cast<const bf16_t*>(a.v);
  p.beta = reinterpret_cast<const bf16_t*>(a.beta);
  p.o = reinterpret_cast<bf16_t*>(a.o);
  p.S = a.S;
  p.T = a.T;
  p.dv = a.dv;
  p.use_init = a.use_init;
  p.Tq = a.T;
  p.Sc = a.Sc;
  return p;
}
}  // namespace

hipError_t launch_gate_prep(int dk, const PrefillArgs& a, void* workspace, hipStream_t st) {
  const int nch = (a.T + kC - 1) / kC;
  const size_t n = (size_t)a.B * a.H * nch * kC * dk;
  bf16_t* qt = reinterpret_cast<bf16_t*>(workspace);
  bf16_t* kt = qt + n;
  bf16_t* kht = kt + n;
  float* gcum = reinterpret_cast<float*>(kht + n);
  const dim3 grid((unsigned)(a.B * a.H * nch)), block(256);
  const bf16_t* q = reinterpret_cast<const bf16_t*>(a.q);
  const bf16_t* k = reinterpret_cast<const bf16_t*>(a.k);
  const bf16_t* g = reinterpret_cast<const bf16_t*>(a.g);
  switch (dk) {
    case 16: hipLaunchKernelGGL(gate_prep<16>, grid, block, 0, st, q, k, g, qt, kt, kht, gcum, a.T, nch); break;
    case 32: hipLaunchKernelGGL(gate_prep<32>, grid, block, 0, st, q, k, g, qt, kt, kht, gcum, a.T, nch); break;
    case 64: hipLaunchKernelGGL(gate_prep<64>, grid, block, 0, st, q, k, g, qt, kt, kht, gcum, a.T, nch); break;
    case 128: hipLaunchKernelGGL(gate_prep<128>, grid, block, 0, st, q, k, g, qt, kt, kht, gcum, a.T, nch); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill_pipe_prepped(const PrefillArgs& a, const void* prep, hipStream_t st) {
  const int nch = (a.T + kC - 1) / kC;
  const size_t n = (size_t)a.B * a.H * nch * kC * kDK;
  PipeArgs p = pipe_args(a);
  p.q = reinterpret_cast<const bf16_t*>(prep);
  p.k = p.q + n;
  p.kh = p.k + n;
  p.gc = reinterpret_cast<const float*>(p.kh + n);
  p.Tq = nch * kC;
  const long bh = (long)a.B * a.H;
  return a.Sc ? launch_pipe_t<1, true>(p, bh, a.dv, st) : launch_pipe_t<1>(p, bh, a.dv, st);
}

hipError_t launch_prefill_pipe(const PrefillArgs& a, void* workspace, hipStream_t st) {
  if (a.g == nullptr) {
    PipeArgs p = pipe_args(a);
    p.q = reinterpret_cast<const bf16_t*>(a.q);
    p.k = reinterpret_cast<const bf16_t*>(a.k);
    const long bh = (long)a.B * a.H;
    return a.Sc ? launch_pipe_t<0, true>(p, bh, a.dv, st) : launch_pipe_t<0>(p, bh, a.dv, st);
  }
  const hipError_t e = launch_gate_prep(kDK, a, workspace, st);
  if (e != hipSuccess) return e;
  return launch_prefill_pipe_prepped(a, workspace, st);
}

hipError_t launch_prefill_pipe_token(const PrefillArgs& a, hipStream_t st) {
  PipeArgs p = pipe_args(a);
  p.q = reinterpret_cast<const bf16_t*>(a.q);
  p.k = reinterpret_cast<const bf16_t*>(a.k);
  p.g = reinterpret_cast<const bf16_t*>(a.g);
  return a.Sc ? launch_pipe_t<2, true>(p, (long)a.B * a.H, a.dv, st) : launch_pipe_t<2>(p, (long)a.B * a.H, a.dv, st);
}

}  // namespace linattn

// abi_driver.cpp -- runs the C ABI's argument validation and dispatch under
// AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.
//
// It is linked with api.hip (built as plain C++: the entry points do only host
// work before a launch) and with the stub launchers below, which count calls
// and never touch the pointers they get, so every entry point can be driven
// all the way to its launch without a GPU.  Valid calls must reach a launcher
// and return LA_OK; invalid ones must return their documented code without
// reaching one; a seeded sweep over extreme shapes, dims, dtypes, pointers and
// workspace sizes must finish without any sanitizer report.
#include <limits.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/linattn.h"
#include "../../delta_rule_recurrent_chunkwise_amd/csrc/launch.hpp"

static long g_launches = 0;

namespace linattn {
hipError_t launch_decode(int, int, int, int, const DecodeArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill(int, int, int, const PrefillArgs&, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_generic(int, int, int, const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_delta_backward(int, const BackwardArgs&, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_kda_backward(const BackwardArgs&, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prologue(int, const PrologueArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_pipe(const PrefillArgs&, void*, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_prefill_pipe_token(const PrefillArgs&, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_la_par_states(int, const PrefillArgs&, void*, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_la_par_outputs(int, const PrefillArgs&, void*, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_segmented(int, int, const PrefillArgs&, int, void*, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace linattn

static int failures = 0;
#define EXPECT(cond)                                                          \
  do {                                                                        \
    if (!(cond)) {                                                            \
      fprintf(stderr, "%s:%d: expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++failures;                                                             \
    }                                                                         \
  } while (0)

static void* const F = (void*)(uintptr_t)0x1000;   // aligned, never dereferenced
static void* const M = (void*)(uintptr_t)0x1002;   // misaligned
static const size_t BIG = (size_t)1 << 60;

// A call that validates must reach a launcher and return LA_OK.
static void expect_ok(int rc, long before, bool launches) {
  EXPECT(rc == LA_OK);
  EXPECT(launches ? g_launches > before : g_launches == before);
}

static uint64_t rng = 0x9E3779B97F4A7C15ull;
static uint64_t next() {  // xorshift64*
  rng ^= rng >> 12; rng ^= rng << 25; rng ^= rng >> 27;
  return rng * 2685821657736338717ull;
}
static int pick_int() {
  static const int v[] = {INT_MIN, -65, -1, 0, 1, 2, 3, 15, 16, 17, 31, 32, 48, 63, 64, 65, 96, 100, 127,
                          128, 129, 192, 255, 256, 1000, 4096, 32768, 65536, 1 << 20, INT_MAX - 64,
                          INT_MAX - 63, INT_MAX};
  return v[next() % (sizeof v / sizeof v[0])];
}
static void* pick_ptr() {
  switch (next() % 4) { case 0: return nullptr; case 1: return M; default: return F; }
}

int main() {
  // ---- valid calls reach their launchers ----
  for (int dt = 0; dt < 2; ++dt)
    for (int dk : {16, 32, 64, 128})
      for (int dv : {16, 32, 64, 128}) {
        const size_t la_ws = la_prefill_workspace_bytes(2, 3, 130, dk, dv, dt);
        long n = g_launches;
        expect_ok(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 2, 3, 130, dk, dv, dt, la_ws ? F : nullptr, la_ws,
                             nullptr), n, true);
        n = g_launches;
        expect_ok(la_decode_step(F, F, F, F, (float*)F, (float*)F, 5, 3, dk, dv, dt, nullptr), n, true);
        for (int gated = 0; gated < 2; ++gated) {
          if (gated && dt == LA_DTYPE_F32 && dk > 64) continue;
          const size_t ws = deltanet_prefill_workspace_bytes(gated, 2, 3, 130, dk, dv, dt);
          n = g_launches;
          expect_ok(deltanet_prefill(F, F, F, F, gated ? F : nullptr, F, (float*)F, 1, 2, 3, 130, dk, dv, dt,
                                     ws ? F : nullptr, ws, nullptr), n, true);
          n = g_launches;
          expect_ok(deltanet_decode_step(F, F, F, F, gated ? F : nullptr, F, (float*)F, 5, 3, dk, dv, dt, nullptr), n,
                    true);
        }
        n = g_launches;
        expect_ok(gated_deltanet_prefill(F, F, F, F, F, F, (float*)F, 0, 2, 3, 130, dk, dv, dt, nullptr), n, true);
        n = g_launches;
        expect_ok(gated_deltanet_decode_step(F, F, F, F, F, F, (float*)F, 5, 3, dk, dv, dt, nullptr), n, true);
        const size_t gws = gla_prefill_workspace_bytes(2, 3, 130, dk, dv, dt);
        n = g_launches;
        expect_ok(gla_prefill(F, F, F, F, F, (float*)F, 0, 2, 3, 130, dk, dv, dt, gws ? F : nullptr, gws, nullptr), n,
                  true);
        n = g_launches;
        expect_ok(gla_decode_step(F, F, F, nullptr, F, (float*)F, 5, 3, dk, dv, dt, nullptr), n, true);
        if (dt == LA_DTYPE_F32 && (dk > 64 || dv > 64)) continue;
        const size_t bws = deltanet_prefill_backward_workspace_bytes(2, 3, 130, dk, dv, dt);
        n = g_launches;
        expect_ok(deltanet_prefill_backward(F, F, F, F, nullptr, F, nullptr, F, F, F, F, nullptr, 2, 3, 130, dk, dv,
                                            dt, F, bws, nullptr), n, true);
        const size_t gbws = gated_deltanet_prefill_backward_workspace_bytes(2, 3, 130, dk, dv, dt);
        EXPECT(gbws > bws);
        n = g_launches;
        expect_ok(gated_deltanet_prefill_backward(F, F, F, F, F, nullptr, F, nullptr, F, F, F, F, F, nullptr, 2, 3, 130,
                                                  dk, dv, dt, F, gbws, nullptr), n, true);
        if (dt == LA_DTYPE_BF16) {
          const size_t kws = kda_prefill_backward_workspace_bytes(2, 3, 130, dk, dv, dt);
          EXPECT(kws > 0);
          n = g_launches;
          expect_ok(kda_prefill_backward(F, F, F, F, F, nullptr, F, nullptr, F, F, F, F, F, nullptr, 2, 3, 130, dk, dv,
                                         dt, F, kws, nullptr), n, true);
        }
        n = g_launches;
        expect_ok(deltanet_prologue(F, F, F, F, F, F, 2, 3, 130, dk, 1, 1, 0.5f, dt, nullptr), n, true);
        if (dt == LA_DTYPE_BF16) {
          for (int gate = 0; gate < 3; ++gate)
            for (int segs : {0, 1, 2, 5, 10}) {
              const size_t sws = deltanet_prefill_segmented_workspace_bytes(gate, 2, 3, 130, dk, dv, dt, segs);
              EXPECT(segs < 2 || sws > 0);
              n = g_launches;
              expect_ok(deltanet_prefill_segmented(F, F, F, F, gate ? F : nullptr, gate, F, (float*)F, 1, 2, 3, 130,
                                                   dk, dv, dt, segs, F, sws, nullptr),
                        n, true);
            }
        }
      }
  // T = 0 with the initial state kept: valid with NULL token arrays and no
  // workspace (the launcher then enqueues nothing)
  long n0 = g_launches;
  expect_ok(la_prefill(nullptr, nullptr, nullptr, nullptr, (float*)F, (float*)F, 1, 1, 1, 0, 64, 64, 1, nullptr, 0,
                       nullptr), n0, true);

  // ---- invalid calls return their code before any launch ----
  const long before = g_launches;
  EXPECT(la_prefill(nullptr, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 64, 64, 1, F, BIG, nullptr) == LA_ERR_NULL);
  EXPECT(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 64, 64, 7, F, BIG, nullptr) == LA_ERR_DTYPE);
  EXPECT(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 0, 1, 64, 64, 64, 1, F, BIG, nullptr) == LA_ERR_SHAPE);
  EXPECT(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 96, 64, 1, F, BIG, nullptr) ==
         LA_ERR_UNSUPPORTED_DIM);
  EXPECT(la_prefill(M, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 64, 64, 1, F, BIG, nullptr) == LA_ERR_ALIGN);
  EXPECT(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 64, 64, 1, nullptr, BIG, nullptr) ==
         LA_ERR_WORKSPACE);
  EXPECT(la_prefill(F, F, F, F, (float*)F, (float*)F, 0, 1, 1, 64, 64, 64, 1, (void*)(uintptr_t)0x1010, BIG,
                    nullptr) == LA_ERR_ALIGN);
  EXPECT(deltanet_prefill(F, F, F, F, F, F, (float*)F, 0, 1, 1, 64, 128, 128, 0, nullptr, 0, nullptr) ==
         LA_ERR_UNSUPPORTED_DIM);
  EXPECT(deltanet_prefill_backward(F, F, F, F, nullptr, F, nullptr, F, F, F, F, nullptr, 1, 1, 64, 64, 64, 1,
                                   nullptr, 0, nullptr) == LA_ERR_WORKSPACE);
  EXPECT(deltanet_prefill_segmented(F, F, F, F, nullptr, 1, F, (float*)F, 0, 1, 1, 64, 64, 64, 1, 2, F, BIG,
                                    nullptr) == LA_ERR_NULL);
  EXPECT(deltanet_prefill_segmented(F, F, F, F, F, 0, F, (float*)F, 0, 1, 1, 64, 64, 64, 1, 2, F, BIG, nullptr) ==
         LA_ERR_SHAPE);
  EXPECT(deltanet_prefill_segmented(F, F, F, F, nullptr, 0, F, (float*)F, 0, 1, 1, 64, 64, 64, 1, 3, F, BIG,
                                    nullptr) == LA_ERR_SHAPE);
  EXPECT(deltanet_prefill_segmented(F, F, F, F, nullptr, 0, F, (float*)F, 0, 1, 1, 64, 64, 64, 0, 2, F, BIG,
                                    nullptr) == LA_ERR_UNSUPPORTED_DIM);
  EXPECT(deltanet_prefill_segmented(F, F, F, F, nullptr, 0, F, (float*)F, 0, 1, 1, 64, 64, 64, 1, 2, nullptr, 0,
                                    nullptr) == LA_ERR_WORKSPACE);
  EXPECT(g_launches == before);

  // ---- a seeded sweep over extreme arguments: any outcome, no UB ----
  for (int it = 0; it < 200000; ++it) {
    const int B = pick_int(), H = pick_int(), T = pick_int(), dk = pick_int(), dv = pick_int();
    const int dt = (int)(next() % 4) - 1, gated = (int)(next() % 2);
    void* p[8];
    for (auto& x : p) x = pick_ptr();
    const size_t wsn = (next() % 2) ? BIG : (size_t)(next() % 4096);
    void* ws = (next() % 3) ? F : nullptr;
    (void)la_prefill_workspace_bytes(B, H, T, dk, dv, dt);
    (void)gla_prefill_workspace_bytes(B, H, T, dk, dv, dt);
    (void)deltanet_prefill_workspace_bytes(gated, B, H, T, dk, dv, dt);
    (void)deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dt);
    (void)gated_deltanet_prefill_backward_workspace_bytes(B, H, T, dk, dv, dt);
    (void)kda_prefill_backward_workspace_bytes(B, H, T, dk, dv, dt);
    const int segs = pick_int(), gate = (int)(next() % 5) - 1;
    (void)deltanet_prefill_segmented_workspace_bytes(gate, B, H, T, dk, dv, dt, segs);
    (void)deltanet_prefill_segments(B, H, T, dk, dv);
    int rc[13];
    rc[0] = la_prefill(p[0], p[1], p[2], p[3], (float*)p[4], (float*)p[5], gated, B, H, T, dk, dv, dt, ws, wsn, nullptr);
    rc[1] = la_decode_step(p[0], p[1], p[2], p[3], (float*)p[4], (float*)p[5], B, H, dk, dv, dt, nullptr);
    rc[2] = deltanet_prefill(p[0], p[1], p[2], p[3], gated ? p[6] : nullptr, p[4], (float*)p[5], gated, B, H, T, dk,
                             dv, dt, ws, wsn, nullptr);
    rc[3] = deltanet_decode_step(p[0], p[1], p[2], p[3], gated ? p[6] : nullptr, p[4], (float*)p[5], B, H, dk, dv,
                                 dt, nullptr);
    rc[4] = gated_deltanet_prefill(p[0], p[1], p[2], p[3], p[6], p[4], (float*)p[5], gated, B, H, T, dk, dv, dt,
                                   nullptr);
    rc[5] = gated_deltanet_decode_step(p[0], p[1], p[2], p[3], p[6], p[4], (float*)p[5], B, H, dk, dv, dt, nullptr);
    rc[6] = gla_prefill(p[0], p[1], p[2], p[6], p[4], (float*)p[5], gated, B, H, T, dk, dv, dt, ws, wsn, nullptr);
    rc[7] = gla_decode_step(p[0], p[1], p[2], p[6], p[4], (float*)p[5], B, H, dk, dv, dt, nullptr);
    rc[8] = deltanet_prefill_backward(p[0], p[1], p[2], p[3], nullptr, p[4], nullptr, p[5], p[6], p[7], p[0],
                                      nullptr, B, H, T, dk, dv, dt, ws, wsn, nullptr);
    rc[9] = gated_deltanet_prefill_backward(p[0], p[1], p[2], p[3], p[6], nullptr, p[4], nullptr, p[5], p[6], p[7],
                                            p[0], p[1], nullptr, B, H, T, dk, dv, dt, ws, wsn, nullptr);
    rc[10] = deltanet_prologue(p[0], p[1], p[2], p[3], p[4], p[5], B, H, T, dk, (int)(next() % 3), gated, 1.f, dt,
                               nullptr);
    rc[11] = kda_prefill_backward(p[0], p[1], p[2], p[3], p[6], nullptr, p[4], nullptr, p[5], p[6], p[7], p[0], p[1],
                                  nullptr, B, H, T, dk, dv, dt, ws, wsn, nullptr);
    rc[12] = deltanet_prefill_segmented(p[0], p[1], p[2], p[3], gated ? p[6] : nullptr, gate, p[4], (float*)p[5],
                                        gated, B, H, T, dk, dv, dt, segs, ws, wsn, nullptr);
    for (int r : rc) EXPECT(r <= 0 && r >= LA_ERR_WORKSPACE);
  }
  for (int code = -10; code <= 2; ++code) EXPECT(la_strerror(code) != nullptr);
  if (failures) {
    fprintf(stderr, "%d expectation(s) failed\n", failures);
    return 1;
  }
  printf("abi driver: %ld launches reached, no sanitizer report\n", g_launches);
  return 0;
}

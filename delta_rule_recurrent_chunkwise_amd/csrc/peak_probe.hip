// Peak-rate probes for the measurement harness (not part of the linattn
// ABI): a dense bf16 MFMA loop and streaming device copies, so that the
// kernels' rates can be stated as fractions of what this GPU sustains in the
// same run, next to the published peaks.  Built into its own library,
// libpeak_probe.so.
#include <hip/hip_runtime.h>

#include <cstddef>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float fx4 __attribute__((ext_vector_type(4)));

// Every wave runs `iters` rounds of 4 independent 32x32x16 bf16 MFMAs on
// register operands (32768 flops each).  On gfx950 this shape sustains a
// higher rate than 16x16x32 (measured 2.48 against 2.15 PFLOP/s).  Operands
// come from `seed` so the compiler cannot fold them; one float per thread is
// written to `sink`.
__global__ __launch_bounds__(256) void mfma_loop(const float* __restrict__ seed, float* __restrict__ sink,
                                                 int iters) {
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const float s = seed[threadIdx.x & 63];
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(s * (float)(i + 1));
    b[i] = (__bf16)(s - (float)i);
  }
  // named accumulators: an array of them made the compiler copy
  // accumulator registers around every iteration
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const floatx16 t = (c0 + c1) + (c2 + c3);
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += t[i];
  sink[tid] = r;
}

// One workgroup per tile of 256 * U 16-byte vectors; each thread moves U
// vectors, all loads before all stores, nontemporal (the data is touched
// once).  RMW = false copies src to dst (U = 8); RMW = true updates src in
// place (adds 1 to every float; U = 4), the access pattern of an in-place
// state update.  Back-to-back launches of these sustained 6.4 (copy) and
// 6.1 (in place) TB/s over 512 MiB on MI355X, more than other shapes tried
// (grid-stride loops, plain loads and stores, 1 GiB).
template <bool RMW, int U>
__global__ __launch_bounds__(256) void stream_tile(const fx4* src, fx4* dst) {
  const size_t base = (size_t)blockIdx.x * 256 * U + threadIdx.x;
  fx4 v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(src + base + 256 * u);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if (RMW) v[u] += 1.0f;
    __builtin_nontemporal_store(v[u], dst + base + 256 * u);
  }
}

constexpr size_t kStreamQuantum = 256 * 8 * 16;  // bytes: one copy tile (32 KiB)

}  // namespace

// Launches `blocks` workgroups of 256 threads, each wave doing iters * 4
// MFMAs of 32768 flops; `seed` holds 64 floats, `sink` blocks * 256 floats
// (device pointers owned by the caller).  Returns 0, -1 for bad arguments,
// or the HIP error code of the launch.  Flops per launch:
// blocks * 4 * iters * 4 * 32768.
extern "C" int peak_probe_mfma_bf16(const float* seed, float* sink, int blocks, int iters, void* stream) {
  if (!seed || !sink || blocks <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_loop, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, seed, sink, iters);
  return (int)hipGetLastError();
}

// Streams `bytes` (a multiple of 32 KiB; 16-byte aligned device memory owned
// by the caller): in_place = 0 copies src to dst (not overlapping),
// in_place = 1 updates src in place (dst unused; every float grows by 1).
// Returns 0, -1 for bad arguments, or the HIP error code of the launch.
// Bytes moved per launch: 2 * bytes (read + write).
extern "C" int peak_probe_stream(void* src, void* dst, size_t bytes, int in_place, void* stream) {
  if (!src || (!in_place && !dst) || bytes == 0 || bytes % kStreamQuantum != 0) return -1;
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16 != 0) return -1;
  fx4* s = reinterpret_cast<fx4*>(src);
  if (in_place)
    hipLaunchKernelGGL((stream_tile<true, 4>), dim3((unsigned)(bytes / (256 * 4 * 16))), dim3(256), 0,
                       (hipStream_t)stream, s, s);
  else
    hipLaunchKernelGGL((stream_tile<false, 8>), dim3((unsigned)(bytes / (256 * 8 * 16))), dim3(256), 0,
                       (hipStream_t)stream, s, reinterpret_cast<fx4*>(dst));
  return (int)hipGetLastError();
}

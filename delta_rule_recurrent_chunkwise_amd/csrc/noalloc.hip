// noalloc.hip -- la_prefill_noalloc: la_prefill for callers that cannot
// allocate device memory (code under stream capture, tight serving loops,
// harnesses that forbid allocation).  The chunk-parallel bf16 kernels keep
// per-chunk states in scratch memory; here that scratch is a fixed array in
// the library's own device memory instead of a caller workspace.
//
// `scratch` is a file-scope __device__ array: every GPU the library is loaded
// on holds its own copy, at its own address, until the process ends.  In
// host code its name is only a stand-in for the symbol, never a device
// address, so its address on each device is looked up once with
// hipGetSymbolAddress (with that device current) and only that pointer is
// handed to kernels.  Calls on one GPU share its array: calls that overlap
// on one GPU (different streams without ordering between them) race on it.
// The kernels write every scratch element they read in the same call, so the
// previous call's contents need no clearing.
#include <hip/hip_runtime.h>
#include <mutex>
#include <stdint.h>

#include "../../include/linattn.h"
#include "launch.hpp"

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // LA_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == LA_NOALLOC_SCRATCH_BYTES, "header and library disagree");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mutex;

// The current device's copy of `scratch` (looked up on the first call on
// that device), or nullptr if the runtime cannot provide it.
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

}  // namespace

extern "C" int la_prefill_noalloc(const void* q, const void* k, const void* v, void* o, float* S, float* z,
                                  int use_initial_state, int B, int H, int T, int dk, int dv, int dtype,
                                  void* stream) {
  if (!S || !z || (T != 0 && (!q || !k || !v || !o))) return LA_ERR_NULL;
  if (dtype != LA_DTYPE_F32 && dtype != LA_DTYPE_BF16) return LA_ERR_DTYPE;
  // the shape checks of la_prefill, through its workspace query (0 for a
  // rejected shape) and then la_prefill's own validation below
  if (B <= 0 || H <= 0 || T < 0) return LA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return LA_ERR_UNSUPPORTED_DIM;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return LA_ERR_ALIGN;
  const size_t need = la_prefill_workspace_bytes(B, H, T, dk, dv, dtype);
  if (need > kScratchBytes) return LA_ERR_SCRATCH_LIMIT;
  void* ws = nullptr;
  if (need > 0) {
    ws = scratch_on_current_device();
    if (ws == nullptr) return LA_ERR_LAUNCH;
  }
  // la_prefill repeats the validation (and rejects sizes the checks above
  // let through), then launches the same kernels on the fixed scratch
  return la_prefill(q, k, v, o, S, z, use_initial_state, B, H, T, dk, dv, dtype, ws, need, stream);
}

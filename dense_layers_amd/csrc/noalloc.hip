// Softmax cross-entropy for callers that cannot allocate device memory (code
// under stream-graph capture, tight serving loops, harnesses that forbid
// allocation).  It runs the same kernels as softmax_xent_fwd_bwd; the one
// scratch buffer those kernels need -- the per-row losses the fixed-order
// mean reads, when the caller does not ask for them -- lives in a
// file-scope device array instead of a caller workspace.
//
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  Host code never hands the array's name to a kernel (on the
// host it is only a stand-in symbol): the first call on a device, with that
// device current, looks up the device address with hipGetSymbolAddress and
// keeps it per device, and every later use goes through that address.
// Calls on one GPU share its array: two calls that overlap in time on one
// GPU (different streams, or threads) race on it.  The cross-entropy writes
// every row's loss before the mean reads it, so nothing needs clearing
// between calls.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/dense_layers_amd.h"
#include "common.hpp"

namespace {

constexpr int64_t kNoAllocMaxRows = DL_XENT_NOALLOC_MAX_ROWS;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kNoAllocMaxRows];

std::once_flag g_once[kMaxDevices];
float* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's `scratch`, looked up once per device.
hipError_t scratch_of(int dev, float** out) {
  std::call_once(g_once[dev], [dev] {
    float* ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress((void**)&ptr, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *out = g_ptr[dev];
  return g_err[dev];
}

bool overlaps(const void* a, size_t an, const void* b, size_t bn) {
  if (a == nullptr || b == nullptr || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

int fail(int code, const char* fmt, long long a = 0, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), fmt, a, b);
  return dl::api_fail(code, buf);
}

}  // namespace

extern "C" int softmax_xent_fwd_bwd_noalloc(void* stream, int64_t B, int64_t C,
                                            const float* logits, const int32_t* labels,
                                            float* loss, float* row_loss, float* dlogits) {
  if (B <= 0 || B > 0x7fffffff || C <= 0 || C > 0x7fffffff)
    return fail(DL_INVALID_ARGUMENT,
                "softmax_xent_fwd_bwd_noalloc: sizes must be in [1, 2^31): B=%lld C=%lld", B, C);
  if (!logits || !labels || !loss || !dlogits)
    return fail(DL_INVALID_ARGUMENT,
                "softmax_xent_fwd_bwd_noalloc: logits, labels, loss and dlogits are required");
  if (row_loss == nullptr && B > kNoAllocMaxRows)
    return fail(DL_WORKSPACE_TOO_SMALL,
                "softmax_xent_fwd_bwd_noalloc: B=%lld rows exceed the %lld-row scratch "
                "(pass row_loss, or use softmax_xent_fwd_bwd with a workspace)",
                B, kNoAllocMaxRows);
  const size_t nz = (size_t)B * C * 4;
  if ((dlogits != logits && overlaps(dlogits, nz, logits, nz)) ||
      overlaps(dlogits, nz, labels, B * 4) || overlaps(dlogits, nz, loss, 4) ||
      overlaps(dlogits, nz, row_loss, B * 4) || overlaps(loss, 4, logits, nz) ||
      overlaps(row_loss, B * 4, logits, nz))
    return fail(DL_ALIASING,
                "softmax_xent_fwd_bwd_noalloc: outputs overlap inputs (dlogits may equal logits)");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(DL_HIP_ERROR, "softmax_xent_fwd_bwd_noalloc: hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DL_UNSUPPORTED, "softmax_xent_fwd_bwd_noalloc: device %lld past the %lld supported",
                dev, kMaxDevices);
  float* rl = row_loss;
  if (rl == nullptr) {
    e = scratch_of(dev, &rl);
    if (e != hipSuccess || rl == nullptr)
      return fail(DL_HIP_ERROR,
                  "softmax_xent_fwd_bwd_noalloc: hipGetSymbolAddress of the scratch failed");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  e = dl::launch_xent(B, C, logits, labels, rl, dlogits, loss, s);
  if (e != hipSuccess) return fail(DL_HIP_ERROR, "softmax_xent_fwd_bwd_noalloc: launch failed");
  return DL_OK;
}

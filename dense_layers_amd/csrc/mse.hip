// Mean squared error, forward and backward in one pass (MuNet page, "Python
// training": the compiled step's mse_loss; noeira.nn docs, package layout:
// MSE among the losses):
//   loss = (1/n) sum (p - t)^2,  dpred = (p - t) (2/n),  n = B C.
// HBM-bound: 8 bytes read and 4 written per element.  Each workgroup adds
// the squares of its units in float64 (differences formed in float64, exact
// for float32 inputs) and leaves one partial; one workgroup adds the partials
// in a fixed order, so the loss is bit-reproducible.  The grid is two
// workgroups per CU walking the units, and dpred is written with
// non-temporal stores (nothing reads it back in this kernel): on [16384,
// 4096] 141 us against 151 us with 8 workgroups per CU and plain stores.
#include "common.hpp"

namespace dl {
namespace {

__device__ __forceinline__ double block_sum_d(double acc) {
  __shared__ double red[kOptBlock / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < kOptBlock / 64; ++w) t += red[w];
  return t;
}

// Units of kStatUnit elements; thread t takes the float4 groups at
// t*4 + {0, 1, 2, 3} * 1024.  Full aligned units go through a software
// pipeline (the next unit's loads are issued before the current one is
// used); the array's last, partial unit is done element by element.  dpred
// may equal pred: every element is read and then written by the same thread.
__device__ __forceinline__ void mse_fetch(const float* pred, const float* target, int64_t base,
                                          f32x4 (&p)[4], f32x4 (&t)[4]) {
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    p[it] = *reinterpret_cast<const f32x4*>(pred + base + it * 1024);
    t[it] = *reinterpret_cast<const f32x4*>(target + base + it * 1024);
  }
}

__global__ void __launch_bounds__(kOptBlock)
mse_kernel(int64_t n, const float* pred, const float* __restrict__ target, float* dpred,
           double* __restrict__ part, float two_over_n, int vec, const float* dscale) {
  if (dscale != nullptr) two_over_n *= *dscale;  // loss scale
  double acc = 0.0;
  const int64_t units = (n + kStatUnit - 1) / kStatUnit;
  // units whose every thread's 16 elements exist (all but a partial last one)
  const int64_t full_units = vec ? n / kStatUnit : 0;
  int64_t u = blockIdx.x;
  f32x4 p[4], t[4];
  if (u < full_units) mse_fetch(pred, target, u * kStatUnit + (int64_t)threadIdx.x * 4, p, t);
  while (u < full_units) {
    const int64_t un = u + gridDim.x;
    f32x4 pn[4], tn[4];
    if (un < full_units) mse_fetch(pred, target, un * kStatUnit + (int64_t)threadIdx.x * 4, pn, tn);
    const int64_t base = u * kStatUnit + (int64_t)threadIdx.x * 4;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d = (double)p[it][e] - (double)t[it][e];
        acc += d * d;
      }
      if (dpred != nullptr)
        __builtin_nontemporal_store((p[it] - t[it]) * two_over_n,
                                    reinterpret_cast<f32x4*>(dpred + base + it * 1024));
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      p[it] = pn[it];
      t[it] = tn[it];
    }
    u = un;
  }
  for (; u < units; u += gridDim.x) {
    const int64_t base = u * kStatUnit + (int64_t)threadIdx.x * 4;
    for (int it = 0; it < 4; ++it)
      for (int e = 0; e < 4; ++e) {
        const int64_t i = base + it * 1024 + e;
        if (i >= n) continue;
        const float pi = pred[i], ti = target[i];
        const double d = (double)pi - (double)ti;
        acc += d * d;
        if (dpred != nullptr) dpred[i] = (pi - ti) * two_over_n;
      }
  }
  const double r = block_sum_d(acc);
  if (threadIdx.x == 0) part[blockIdx.x] = r;
}

__global__ void __launch_bounds__(kOptBlock)
mse_finish_kernel(const double* __restrict__ part, int parts, int64_t n, float* __restrict__ loss) {
  double acc = 0.0;
  for (int i = threadIdx.x; i < parts; i += kOptBlock) acc += part[i];
  const double t = block_sum_d(acc);
  if (threadIdx.x == 0) loss[0] = (float)(t / (double)n);
}

}  // namespace

// Two workgroups per CU of the 256-CU chip.
constexpr int kMseBlocks = 512;

int mse_grid(int64_t n) {
  const int64_t units = (n + kStatUnit - 1) / kStatUnit;
  return (int)(units < kMseBlocks ? units : kMseBlocks);
}

hipError_t launch_mse(int64_t n, const float* pred, const float* target, float* dpred,
                      double* part, float* loss, hipStream_t s, const float* dscale) {
  const int grid = mse_grid(n);
  const int vec = ((reinterpret_cast<uintptr_t>(pred) | reinterpret_cast<uintptr_t>(target) |
                    reinterpret_cast<uintptr_t>(dpred)) & 15) == 0;
  hipLaunchKernelGGL(mse_kernel, dim3((unsigned)grid), dim3(kOptBlock), 0, s, n, pred, target,
                     dpred, part, (float)(2.0 / (double)n), vec, dscale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mse_finish_kernel, dim3(1), dim3(kOptBlock), 0, s, part, grid, n, loss);
  return hipGetLastError();
}

}  // namespace dl

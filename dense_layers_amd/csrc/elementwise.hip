// Small streaming kernels around the GEMMs:
//   * split-K reduction of weight-gradient partials (and the fused db partials),
//     summed in slice order so the result is bit-reproducible;
//   * G = dY * act'(saved) for a vjp whose upstream gradient was not already
//     masked by the previous dX epilogue;
//   * float32 -> bf16 round-to-nearest-even working copies.
#include "common.hpp"

namespace dl {
namespace {

// dW (contiguous [M, N]) = sum over slices of partial[s][M][N].  Four lanes
// share a group of 4 consecutive elements: lane q adds slices q, q+4, ... in
// order and the quad combines its partial sums in the fixed tree
// (p0 + p1) + (p2 + p3), so each thread walks a quarter of the slices and
// the result is bit-reproducible.
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(int64_t MN, int splits, const float* __restrict__ partial, float* __restrict__ C,
                     int vec) {
  const int q = threadIdx.x & 3;
  const int64_t e0 = ((int64_t)blockIdx.x * 64 + (threadIdx.x >> 2)) * 4;
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  if (vec && e0 + 3 < MN) {
#pragma unroll 4
    for (int s = q; s < splits; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(partial + s * MN + e0);
      g[0] += x[0]; g[1] += x[1]; g[2] += x[2]; g[3] += x[3];
    }
  } else {
    for (int s = q; s < splits; s += 4)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e0 + e < MN) g[e] += partial[s * MN + e0 + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    g[e] += __shfl_xor(g[e], 1);
    g[e] += __shfl_xor(g[e], 2);
  }
  if (e0 + q < MN) C[e0 + q] = g[q];
}

template <typename T>
__global__ void __launch_bounds__(256)
act_mask_kernel(int act, int64_t n, const T* __restrict__ dY, const T* __restrict__ saved,
                T* __restrict__ G) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const float g = Elem<T>::load(dY, i) * act_deriv(act, Elem<T>::load(saved, i));
    Elem<T>::store(G, i, g);
  }
}

__global__ void __launch_bounds__(256)
cast_bf16_kernel(int64_t n, const float* __restrict__ src, bf16_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = f32_to_bf16(src[i]);
}

// src [rows, cols] float32 -> dst = bf16(src) (same layout) and/or
// dst_t = bf16(src)^T [cols, rows], through a 64 x 64 LDS tile so both the
// reads and the transposed writes are row-contiguous.
constexpr int kTT = 64;
__global__ void __launch_bounds__(256)
cast_bf16_t_kernel(int64_t rows, int64_t cols, const float* __restrict__ src,
                   bf16_t* __restrict__ dst, bf16_t* __restrict__ dst_t) {
  __shared__ bf16_t tile[kTT][kTT + 2];
  const int64_t r0 = (int64_t)blockIdx.y * kTT, c0 = (int64_t)blockIdx.x * kTT;
  const int tx = threadIdx.x % kTT, ty = threadIdx.x / kTT;  // 64 x 4
#pragma unroll
  for (int k = 0; k < kTT; k += 4) {
    const int64_t r = r0 + ty + k, c = c0 + tx;
    bf16_t v = 0;
    if (r < rows && c < cols) {
      v = f32_to_bf16(src[r * cols + c]);
      if (dst != nullptr) dst[r * cols + c] = v;
    }
    tile[ty + k][tx] = v;
  }
  if (dst_t == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTT; k += 4) {
    const int64_t c = c0 + ty + k, r = r0 + tx;  // output row c, column r
    if (c < cols && r < rows) dst_t[c * rows + r] = tile[tx][ty + k];
  }
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_splitk_reduce(int M, int N, int splits, const float* partial,
                                const float* db_partial, float* C, int64_t ldc, float* db,
                                hipStream_t s) {
  if (ldc != N) return hipErrorInvalidValue;
  const int64_t MN = (int64_t)M * N;
  const int vec = (MN % 4 == 0) && ((reinterpret_cast<uintptr_t>(partial) & 15) == 0);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((MN + 255) / 256)), dim3(256), 0, s, MN,
                     splits, partial, C, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || db == nullptr) return e;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, s,
                     (int64_t)M, splits, db_partial, db, 0);
  return hipGetLastError();
}

hipError_t launch_act_mask(int dtype, int act, int64_t rows, int64_t cols, const void* dY,
                           const void* saved, void* G, hipStream_t s) {
  const int64_t n = rows * cols;
  if (dtype == 0)
    hipLaunchKernelGGL(act_mask_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, act, n,
                       static_cast<const float*>(dY), static_cast<const float*>(saved),
                       static_cast<float*>(G));
  else
    hipLaunchKernelGGL(act_mask_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, s, act, n,
                       static_cast<const bf16_t*>(dY), static_cast<const bf16_t*>(saved),
                       static_cast<bf16_t*>(G));
  return hipGetLastError();
}

hipError_t launch_cast_bf16_t(int64_t rows, int64_t cols, const float* src, bf16_t* dst,
                              bf16_t* dst_t, hipStream_t s) {
  const dim3 grid((unsigned)((cols + kTT - 1) / kTT), (unsigned)((rows + kTT - 1) / kTT));
  hipLaunchKernelGGL(cast_bf16_t_kernel, grid, dim3(256), 0, s, rows, cols, src, dst, dst_t);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(int64_t n, const float* src, bf16_t* dst, hipStream_t s) {
  hipLaunchKernelGGL(cast_bf16_kernel, dim3(grid_for(n)), dim3(256), 0, s, n, src, dst);
  return hipGetLastError();
}

}  // namespace dl

// Small streaming kernels around the GEMMs:
//   * split-K reduction of weight-gradient partials (and the fused db partials),
//     summed in slice order so the result is bit-reproducible;
//   * G = dY * act'(saved) for a vjp whose upstream gradient was not already
//     masked by the previous dX epilogue;
//   * float32 -> bf16 round-to-nearest-even working copies, or half copies
//     (nearest-even, clamped to +-65504; the MuNet page, "Configuration").
#include "common.hpp"

namespace dl {
namespace {

// out[0 .. n) = sum over slices s = 0 .. S - 1 of p[s * n + (0 .. n)], added in
// slice order (bit-reproducible).  One thread per 4 consecutive outputs
// reads all of its slices, so a thread has many independent loads in flight.
__device__ __forceinline__ void reduce_slices(int64_t n, int S, const float* __restrict__ p,
                                              float* __restrict__ out, bool vec, unsigned blk) {
  const int64_t e0 = ((int64_t)blk * 256 + threadIdx.x) * 4;
  if (e0 >= n) return;
  if (vec && e0 + 3 < n) {
    f32x4 a = *reinterpret_cast<const f32x4*>(p + e0);
#pragma unroll 8
    for (int sl = 1; sl < S; ++sl) a += *reinterpret_cast<const f32x4*>(p + sl * n + e0);
    *reinterpret_cast<f32x4*>(out + e0) = a;
  } else {
    for (int e = 0; e < 4 && e0 + e < n; ++e) {
      float a = p[e0 + e];
      for (int sl = 1; sl < S; ++sl) a += p[sl * n + e0 + e];
      out[e0 + e] = a;
    }
  }
}

// Split-K finish of the weight gradient: blocks [0, wblocks) sum the dW
// slices partial[s][M][N] into C, the rest the db slices db_partial[s][M].
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(int64_t MN, int64_t M, int splits, const float* __restrict__ partial,
                     const float* __restrict__ db_partial, float* __restrict__ C,
                     float* __restrict__ db, int vec, int vec_db, unsigned wblocks) {
  if (blockIdx.x < wblocks) reduce_slices(MN, splits, partial, C, vec != 0, blockIdx.x);
  else reduce_slices(M, splits, db_partial, db, vec_db != 0, blockIdx.x - wblocks);
}

// Forward product split along K: Y[m, n] = act(b[n] + sum over slices s of
// partial[s][m][n]), the slices added in order; one thread per 4 consecutive
// outputs of a row.
__global__ void __launch_bounds__(256)
splitk_finish_fwd_kernel(int64_t MN, int N, int splits, const float* __restrict__ partial,
                         const float* __restrict__ bias, int act, float* __restrict__ Y,
                         int vec) {
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= MN) return;
  if (vec) {  // N % 4 == 0: the 4 outputs share a row
    f32x4 a = *reinterpret_cast<const f32x4*>(partial + e0);
#pragma unroll 8
    for (int sl = 1; sl < splits; ++sl) a += *reinterpret_cast<const f32x4*>(partial + sl * MN + e0);
    const int n = (int)(e0 % N);
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = act_apply(act, a[e] + (bias ? bias[n + e] : 0.f));
    *reinterpret_cast<f32x4*>(Y + e0) = o;
  } else {
    for (int e = 0; e < 4 && e0 + e < MN; ++e) {
      float a = partial[e0 + e];
      for (int sl = 1; sl < splits; ++sl) a += partial[sl * MN + e0 + e];
      Y[e0 + e] = act_apply(act, a + (bias ? bias[(e0 + e) % N] : 0.f));
    }
  }
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

template <int HK>
__global__ void __launch_bounds__(256)
cast_bf16_kernel(int64_t n, const float* __restrict__ src, bf16_t* __restrict__ dst) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = HalfOps<HK>::one(src[i]);
}

// src [rows, cols] float32 -> dst = bf16(src) (same layout) and/or
// dst_t = bf16(src)^T [cols, rows], through a 64 x 64 LDS tile so both the
// reads and the transposed writes are row-contiguous.
constexpr int kTT = 64;
template <int HK>
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
      v = HalfOps<HK>::one(src[r * cols + c]);
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

// The same for rows and cols multiples of 4 with 16-byte aligned float rows
// and 8-byte aligned bf16 rows: each thread moves 4 consecutive elements at a
// time (a float4 in, 8 bytes out) on both sides of the transpose.
template <int HK>
__global__ void __launch_bounds__(256)
cast_bf16_t_vec_kernel(int64_t rows, int64_t cols, const float* __restrict__ src,
                       bf16_t* __restrict__ dst, bf16_t* __restrict__ dst_t) {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  __shared__ __attribute__((aligned(16))) bf16_t tile[kTT][kTT + 4];
  const int64_t r0 = (int64_t)blockIdx.y * kTT, c0 = (int64_t)blockIdx.x * kTT;
  const int q = threadIdx.x % 16, p = threadIdx.x / 16;  // 16 quads x 16 rows
#pragma unroll
  for (int k = 0; k < kTT; k += 16) {
    const int64_t r = r0 + p + k, c = c0 + 4 * q;
    u32x2v w = {0u, 0u};
    if (r < rows && c < cols) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + r * cols + c);
      w = u32x2v{HalfOps<HK>::pack2(x[0], x[1]), HalfOps<HK>::pack2(x[2], x[3])};
      if (dst != nullptr) *reinterpret_cast<u32x2v*>(dst + r * cols + c) = w;
    }
    *reinterpret_cast<u32x2v*>(&tile[p + k][4 * q]) = w;
  }
  if (dst_t == nullptr) return;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kTT; k += 16) {
    const int64_t c = c0 + p + k, r = r0 + 4 * q;  // output row c, columns r .. r + 3
    if (c < cols && r < rows) {
      const uint32_t lo = (uint32_t)tile[4 * q][p + k] | ((uint32_t)tile[4 * q + 1][p + k] << 16);
      const uint32_t hi = (uint32_t)tile[4 * q + 2][p + k] | ((uint32_t)tile[4 * q + 3][p + k] << 16);
      *reinterpret_cast<u32x2v*>(dst_t + c * rows + r) = u32x2v{lo, hi};
    }
  }
}

// Half copy with a power-of-two scale (mixed_safe): the largest finite |x|
// is found (per-workgroup maxima, then one workgroup), s = 2^(14 - floor(log2
// m)) (m = 0: s = 1; exponent capped at 127) puts it in [2^14, 2^15), and
// dst = half(x s) with saturation; x s is exact in float32.  The maxima are
// order-independent, so the result is deterministic.
constexpr int kAmaxUnit = 4096;  // elements per workgroup per round, 4 float4 per thread
constexpr int kAmaxBlocks = 2048;

__global__ void __launch_bounds__(256)
absmax_kernel(int64_t n, const float* __restrict__ x, float* __restrict__ part, int vec) {
  __shared__ float red[4];
  float m = 0.f;
  const int64_t units = (n + kAmaxUnit - 1) / kAmaxUnit;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t base = u * kAmaxUnit + (int64_t)threadIdx.x * 4;
    if (vec && base + 3 * 1024 + 3 < n) {
      f32x4 a[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) a[it] = *reinterpret_cast<const f32x4*>(x + base + it * 1024);
#pragma unroll
      for (int it = 0; it < 4; ++it)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (__builtin_isfinite(a[it][e])) m = fmaxf(m, fabsf(a[it][e]));
    } else {
      for (int it = 0; it < 4; ++it)
        for (int e = 0; e < 4; ++e) {
          const int64_t i = base + it * 1024 + e;
          if (i < n && __builtin_isfinite(x[i])) m = fmaxf(m, fabsf(x[i]));
        }
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

__global__ void __launch_bounds__(256)
safe_scale_kernel(const float* __restrict__ part, int parts, float* __restrict__ scale) {
  __shared__ float red[4];
  float m = 0.f;
  for (int i = threadIdx.x; i < parts; i += 256) m = fmaxf(m, part[i]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x != 0) return;
  m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  float s = 1.f;
  if (m > 0.f) {
    int e;
    frexpf(m, &e);  // m = f 2^e, f in [0.5, 1): floor(log2 m) = e - 1
    s = ldexpf(1.f, min(15 - e, 127));
  }
  scale[0] = s;
}

__global__ void __launch_bounds__(256)
cast_f16_scaled_kernel(int64_t n, const float* __restrict__ src, const float* __restrict__ scale,
                       bf16_t* __restrict__ dst) {
  const float s = scale[0];
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = HalfOps<HK_F16>::one(src[i] * s);
}

unsigned grid_for(int64_t n) {
  int64_t b = (n + 255) / 256;
  if (b > 65536) b = 65536;
  if (b < 1) b = 1;
  return (unsigned)b;
}

}  // namespace

int safe_scale_parts(int64_t n) {
  const int64_t units = (n + kAmaxUnit - 1) / kAmaxUnit;
  return (int)(units < kAmaxBlocks ? units : kAmaxBlocks);
}

hipError_t launch_cast_f16_scaled(int64_t n, const float* src, bf16_t* dst, float* scale,
                                  float* part, hipStream_t s) {
  const int parts = safe_scale_parts(n);
  const int vec = (reinterpret_cast<uintptr_t>(src) & 15) == 0;
  hipLaunchKernelGGL(absmax_kernel, dim3((unsigned)parts), dim3(256), 0, s, n, src, part, vec);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(safe_scale_kernel, dim3(1), dim3(256), 0, s, part, parts, scale);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cast_f16_scaled_kernel, dim3(grid_for(n)), dim3(256), 0, s, n, src, scale, dst);
  return hipGetLastError();
}

hipError_t launch_splitk_reduce(int M, int N, int splits, const float* partial,
                                const float* db_partial, float* C, int64_t ldc, float* db,
                                hipStream_t s) {
  if (ldc != N) return hipErrorInvalidValue;
  const int64_t MN = (int64_t)M * N;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const int vec = (MN % 4 == 0) && al16(partial) && al16(C);
  const int vec_db = db != nullptr && (M % 4 == 0) && al16(db_partial) && al16(db);
  const int64_t wblocks = (MN + 1023) / 1024;
  const int64_t dblocks = db != nullptr ? ((int64_t)M + 1023) / 1024 : 0;
  if (wblocks + dblocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)(wblocks + dblocks)), dim3(256), 0, s,
                     MN, (int64_t)M, splits, partial, db_partial, C, db, vec, vec_db,
                     (unsigned)wblocks);
  return hipGetLastError();
}

hipError_t launch_splitk_finish_fwd(int M, int N, int splits, const float* partial,
                                    const float* bias, int act, float* Y, hipStream_t s) {
  const int64_t MN = (int64_t)M * N;
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const int vec = N % 4 == 0 && al16(partial) && al16(Y);
  const int64_t blocks = (MN + 1023) / 1024;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(splitk_finish_fwd_kernel, dim3((unsigned)blocks), dim3(256), 0, s, MN, N, splits,
                     partial, bias, act, Y, vec);
  return hipGetLastError();
}

hipError_t launch_act_mask(int dtype, int act, int64_t rows, int64_t cols, const void* dY,
                           const void* saved, void* G, hipStream_t s) {
  const int64_t n = rows * cols;
  if (dtype == 0)
    hipLaunchKernelGGL(act_mask_kernel<float>, dim3(grid_for(n)), dim3(256), 0, s, act, n,
                       static_cast<const float*>(dY), static_cast<const float*>(saved),
                       static_cast<float*>(G));
  else if (dtype == 2)
    hipLaunchKernelGGL(act_mask_kernel<f16_t>, dim3(grid_for(n)), dim3(256), 0, s, act, n,
                       static_cast<const f16_t*>(dY), static_cast<const f16_t*>(saved),
                       static_cast<f16_t*>(G));
  else
    hipLaunchKernelGGL(act_mask_kernel<bf16_t>, dim3(grid_for(n)), dim3(256), 0, s, act, n,
                       static_cast<const bf16_t*>(dY), static_cast<const bf16_t*>(saved),
                       static_cast<bf16_t*>(G));
  return hipGetLastError();
}

hipError_t launch_cast_bf16_t(int64_t rows, int64_t cols, const float* src, bf16_t* dst,
                              bf16_t* dst_t, hipStream_t s, int half_kind) {
  const dim3 grid((unsigned)((cols + kTT - 1) / kTT), (unsigned)((rows + kTT - 1) / kTT));
  auto al = [](const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; };
  const bool vec = rows % 4 == 0 && cols % 4 == 0 && al(src, 16) && (dst == nullptr || al(dst, 8)) &&
                   (dst_t == nullptr || al(dst_t, 8));
  const bool f16 = half_kind == HK_F16;
  if (vec && f16)
    hipLaunchKernelGGL(cast_bf16_t_vec_kernel<HK_F16>, grid, dim3(256), 0, s, rows, cols, src, dst,
                       dst_t);
  else if (vec)
    hipLaunchKernelGGL(cast_bf16_t_vec_kernel<HK_BF16>, grid, dim3(256), 0, s, rows, cols, src, dst,
                       dst_t);
  else if (f16)
    hipLaunchKernelGGL(cast_bf16_t_kernel<HK_F16>, grid, dim3(256), 0, s, rows, cols, src, dst, dst_t);
  else
    hipLaunchKernelGGL(cast_bf16_t_kernel<HK_BF16>, grid, dim3(256), 0, s, rows, cols, src, dst,
                       dst_t);
  return hipGetLastError();
}

hipError_t launch_cast_bf16(int64_t n, const float* src, bf16_t* dst, hipStream_t s, int half_kind) {
  if (half_kind == HK_F16)
    hipLaunchKernelGGL(cast_bf16_kernel<HK_F16>, dim3(grid_for(n)), dim3(256), 0, s, n, src, dst);
  else
    hipLaunchKernelGGL(cast_bf16_kernel<HK_BF16>, dim3(grid_for(n)), dim3(256), 0, s, n, src, dst);
  return hipGetLastError();
}

// An empty kernel: the cost of a launch and nothing else, for the launch
// floor of latency-bound steps.
__global__ void __launch_bounds__(64) empty_kernel() {}

hipError_t launch_empty(hipStream_t s) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, s);
  return hipGetLastError();
}

}  // namespace dl

// Gradient control of an optimizer step: the global 2-norm for clipping
// (MuNet page, "What runs today": gradient clipping) and the finite check of
// dynamic loss scaling (Orthon page, "Core capabilities": the loss scaler
// tests the gradients for Inf / NaN, drops such a step, and lowers the scale
// after one and raises it after a run of good steps).
//
// One reading pass over every gradient (finishing split-K slice sums into
// their gradient arrays on the way) leaves per-workgroup float64 sums of
// squares and non-finite counts; one workgroup then adds them in a fixed
// order, forms norm = sqrt(sum) / S, the clip coefficient
// min(1, max_norm / (norm + 1e-6)) and the skip decision, updates the loss
// scale and ticks the device step count.  Everything stays on the device:
// the optimizer reads the result from memory, so a step needs no host
// synchronisation.  The grid of the reading pass depends only on the array
// sizes, so the sums are bit-reproducible.
#include "common.hpp"

namespace dl {
namespace {

// Sum over the workgroup's 256 threads in a fixed order: a shuffle tree per
// wave, then the four waves in order.  Result valid in thread 0.
__device__ __forceinline__ void block_sum(double& acc, int& bad) {
  __shared__ double red[kOptBlock / 64];
  __shared__ int redb[kOptBlock / 64];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    acc += __shfl_xor(acc, o);
    bad += __shfl_xor(bad, o);
  }
  if ((threadIdx.x & 63) == 0) {
    red[threadIdx.x >> 6] = acc;
    redb[threadIdx.x >> 6] = bad;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    acc = 0.0;
    bad = 0;
    for (int w = 0; w < kOptBlock / 64; ++w) {
      acc += red[w];
      bad += redb[w];
    }
  }
}

__device__ __forceinline__ void account(float g, double& acc, int& bad) {
  acc += (double)g * (double)g;
  bad += __builtin_isfinite(g) ? 0 : 1;
}

__device__ __forceinline__ int seg_of(const OptSegs& segs, int64_t u) {
  int s = 0;
  while (s + 1 < segs.count && u >= segs.start_block[s + 1]) ++s;
  return s;
}

// Unit u of a segment: elements [u * kStatUnit, +kStatUnit); thread t takes
// the float4 groups at t*4 + {0, 1, 2, 3} * 1024.
struct UnitPos {
  int s;
  int64_t n, base;
};
__device__ __forceinline__ UnitPos unit_pos(const OptSegs& segs, int64_t u) {
  const int s = seg_of(segs, u);
  return UnitPos{s, segs.n[s], (u - segs.start_block[s]) * kStatUnit + (int64_t)threadIdx.x * 4};
}

// The thread's 16 gradient values of unit u; places past the array's end
// read as 0 (which adds nothing to the sum of squares and is finite).
__device__ __forceinline__ void fetch_unit(const OptSegs& segs, int64_t u, f32x4 (&a)[4]) {
  const UnitPos q = unit_pos(segs, u);
  const float* g = segs.g[q.s];
  if (q.base + 3 * 1024 + 3 < q.n && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
#pragma unroll
    for (int it = 0; it < 4; ++it) a[it] = *reinterpret_cast<const f32x4*>(g + q.base + it * 1024);
  } else {
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t i = q.base + it * 1024 + e;
        a[it][e] = i < q.n ? g[i] : 0.f;
      }
  }
}

// Plain gradients: software-pipelined, the next unit's loads are issued
// before the current unit is added up.
__global__ void __launch_bounds__(kOptBlock)
grad_stats_kernel(OptSegs segs, int64_t units, double* __restrict__ part_sq,
                  int* __restrict__ part_bad) {
  double acc = 0.0;
  int bad = 0;
  int64_t u = blockIdx.x;
  f32x4 cur[4];
  if (u < units) fetch_unit(segs, u, cur);
  while (u < units) {
    const int64_t un = u + gridDim.x;
    f32x4 nxt[4];
    if (un < units) fetch_unit(segs, un, nxt);
#pragma unroll
    for (int it = 0; it < 4; ++it)
#pragma unroll
      for (int e = 0; e < 4; ++e) account(cur[it][e], acc, bad);
#pragma unroll
    for (int it = 0; it < 4; ++it) cur[it] = nxt[it];
    u = un;
  }
  block_sum(acc, bad);
  if (threadIdx.x == 0) {
    part_sq[blockIdx.x] = acc;
    part_bad[blockIdx.x] = bad;
  }
}

// Split-K segments present (the MLP step): the slices of each element are
// added in slice order and the sum is stored to the segment's gradient
// array before it is accounted.
__global__ void __launch_bounds__(kOptBlock)
grad_stats_split_kernel(OptSegs segs, int64_t units, double* __restrict__ part_sq,
                        int* __restrict__ part_bad) {
  double acc = 0.0;
  int bad = 0;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const UnitPos q = unit_pos(segs, u);
    const int64_t n = q.n, base = q.base;
    const int S = segs.splits[q.s];
    const float* src = S > 1 ? segs.part[q.s] : segs.g[q.s];
    const int64_t stride = S > 1 ? segs.part_stride[q.s] : 0;
    float* out = segs.g_out[q.s];
    const bool full = base + 3 * 1024 + 3 < n;
    const bool vec = full && ((reinterpret_cast<uintptr_t>(src) |
                               static_cast<uintptr_t>(stride * 4) |
                               (S > 1 ? reinterpret_cast<uintptr_t>(out) : 0)) & 15) == 0;
    if (vec) {
      f32x4 a[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) a[it] = *reinterpret_cast<const f32x4*>(src + base + it * 1024);
      for (int k = 1; k < S; ++k) {
        f32x4 b[4];
#pragma unroll
        for (int it = 0; it < 4; ++it)
          b[it] = *reinterpret_cast<const f32x4*>(src + (int64_t)k * stride + base + it * 1024);
#pragma unroll
        for (int it = 0; it < 4; ++it) a[it] += b[it];
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        if (S > 1) *reinterpret_cast<f32x4*>(out + base + it * 1024) = a[it];
#pragma unroll
        for (int e = 0; e < 4; ++e) account(a[it][e], acc, bad);
      }
    } else {
      for (int it = 0; it < 4; ++it)
        for (int e = 0; e < 4; ++e) {
          const int64_t i = base + it * 1024 + e;
          if (i >= n) continue;
          float a = src[i];
          for (int k = 1; k < S; ++k) a += src[(int64_t)k * stride + i];
          if (S > 1) out[i] = a;
          account(a, acc, bad);
        }
    }
  }
  block_sum(acc, bad);
  if (threadIdx.x == 0) {
    part_sq[blockIdx.x] = acc;
    part_bad[blockIdx.x] = bad;
  }
}

__global__ void __launch_bounds__(kOptBlock) grad_ctl_kernel(CtlArgs a) {
  double acc = 0.0;
  int bad = 0;
  for (int i = threadIdx.x; i < a.parts; i += kOptBlock) {
    acc += a.part_sq[i];
    bad += a.part_bad[i];
  }
  block_sum(acc, bad);
  if (threadIdx.x != 0) return;
  const double S = a.scale != nullptr ? (double)a.scale[0] : 1.0;
  const bool nonfinite = bad > 0 || !__builtin_isfinite(acc);
  const double norm = sqrt(acc) / S;
  double coef = 1.0;
  if (a.max_norm > 0.0) {
    coef = a.max_norm / (norm + 1e-6);
    if (!(coef < 1.0)) coef = 1.0;
  }
  const bool skip = a.scale != nullptr && nonfinite;
  GradCtl c;
  c.mul = (float)(coef / S);
  c.skip = skip ? 1 : 0;
  c.norm = (float)norm;
  c.pad = 0;
  *a.ctl = c;
  if (a.norm_out != nullptr) a.norm_out[0] = (float)norm;
  if (a.clip_coef != nullptr) a.clip_coef[0] = (float)coef;
  if (a.scale != nullptr) {
    a.found_inf[0] = nonfinite ? 1 : 0;
    if (nonfinite) {
      a.scale[0] = (float)(S * a.backoff_factor);
      a.growth_tracker[0] = 0;
    } else {
      int t = a.growth_tracker[0] + 1;
      if (t == a.growth_interval) {
        a.scale[0] = (float)(S * a.growth_factor);
        t = 0;
      }
      a.growth_tracker[0] = t;
    }
  }
  if (a.step_dev != nullptr && !skip) a.step_dev[0] = a.step_dev[0] + 1;
}

// g *= c for every gradient of the segments, only when c < 1 (c = 1 leaves
// every value unchanged, so the pass is skipped).
__global__ void __launch_bounds__(kOptBlock)
scale_kernel(OptSegs segs, int64_t units, const float* __restrict__ coef) {
  const float c = coef[0];
  if (!(c < 1.0f)) return;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int s = seg_of(segs, u);
    const int64_t n = segs.n[s];
    const int64_t base = (u - segs.start_block[s]) * kStatUnit + (int64_t)threadIdx.x * 4;
    float* g = segs.w[s];
    if (base + 3 * 1024 + 3 < n && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
      f32x4 a[4];
#pragma unroll
      for (int it = 0; it < 4; ++it) a[it] = *reinterpret_cast<const f32x4*>(g + base + it * 1024);
#pragma unroll
      for (int it = 0; it < 4; ++it) *reinterpret_cast<f32x4*>(g + base + it * 1024) = a[it] * c;
    } else {
      for (int it = 0; it < 4; ++it)
        for (int e = 0; e < 4; ++e) {
          const int64_t i = base + it * 1024 + e;
          if (i < n) g[i] *= c;
        }
    }
  }
}

}  // namespace

int64_t stat_units(const OptSegs& segs) {
  return segs.start_block[segs.count];
}

int stat_grid(int64_t units) {
  return (int)(units < kStatBlocks ? units : kStatBlocks);
}

hipError_t launch_grad_stats(const OptSegs& segs, int64_t units, double* part_sq, int* part_bad,
                             hipStream_t s) {
  if (units <= 0) return hipSuccess;
  bool split = false;
  for (int k = 0; k < segs.count; ++k) split = split || segs.splits[k] > 1;
  if (split)
    hipLaunchKernelGGL(grad_stats_split_kernel, dim3((unsigned)stat_grid(units)), dim3(kOptBlock),
                       0, s, segs, units, part_sq, part_bad);
  else
    hipLaunchKernelGGL(grad_stats_kernel, dim3((unsigned)stat_grid(units)), dim3(kOptBlock), 0, s,
                       segs, units, part_sq, part_bad);
  return hipGetLastError();
}

hipError_t launch_grad_ctl(const CtlArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(grad_ctl_kernel, dim3(1), dim3(kOptBlock), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_scale_by(const OptSegs& segs, const float* coef, hipStream_t s) {
  const int64_t units = stat_units(segs);
  if (units <= 0) return hipSuccess;
  hipLaunchKernelGGL(scale_kernel, dim3((unsigned)stat_grid(units)), dim3(kOptBlock), 0, s, segs,
                     units, coef);
  return hipGetLastError();
}

}  // namespace dl

// SGD and AdamW updates (MuNet page, "What runs today": SGD and AdamW;
// noeira.nn docs, "The design in one page": Adam's m and v live with the
// parameter).  Pure streaming kernels: 16-byte loads and stores, each thread
// handles four float4 groups so a workgroup moves 16 KB per array.
//
// AdamW, per element (decoupled decay first, then the bias-corrected Adam
// step; decay = 1 - lr wd, omb1 = 1 - b1, omb2 = 1 - b2, step_size =
// lr / (1 - b1^t) and inv_sqrt_bc2 = 1 / sqrt(1 - b2^t) are formed on the host
// in double and rounded once):
//   w *= decay;  m = b1 m + omb1 g;  v = b2 v + omb2 g^2;
//   w -= step_size m / (sqrt(v) inv_sqrt_bc2 + eps)
#include "common.hpp"

namespace dl {
namespace {

using AdamParams = OptConsts;

__device__ __forceinline__ void adam_elem(float& w, float g, float& m, float& v,
                                          const AdamParams& p) {
  w *= p.decay;
  m = p.b1 * m + p.omb1 * g;
  v = p.b2 * v + p.omb2 * (g * g);
  w -= p.step_size * m / (sqrtf(v) * p.inv_sqrt_bc2 + p.eps);
}

// Where an array's gradient comes from: a plain array, or split-K partial
// slices summed in slice order (then also written to `out`).
struct GradSrc {
  const float* g;
  const float* part;
  int64_t stride;
  int splits;
  float* out;
};

__device__ __forceinline__ float grad1(const GradSrc& s, int64_t i) {
  if (s.splits <= 1) return s.g[i];
  float acc = s.part[i];
#pragma unroll 8
  for (int k = 1; k < s.splits; ++k) acc += s.part[(int64_t)k * s.stride + i];
  s.out[i] = acc;
  return acc;
}

__device__ __forceinline__ f32x4 grad4(const GradSrc& s, int64_t i) {
  if (s.splits <= 1) return *reinterpret_cast<const f32x4*>(s.g + i);
  f32x4 acc = *reinterpret_cast<const f32x4*>(s.part + i);
#pragma unroll 8
  for (int k = 1; k < s.splits; ++k)
    acc += *reinterpret_cast<const f32x4*>(s.part + (int64_t)k * s.stride + i);
  *reinterpret_cast<f32x4*>(s.out + i) = acc;
  return acc;
}

// Process elements [base, base + kOptElemsPerBlock) of one array.  In the
// full-block vector path every load of the thread's four float4 groups (w, g
// and for AdamW m, v) is issued before the first store, so a thread keeps 8
// or 16 loads in flight instead of waiting once per group.
template <int KIND>
__device__ __forceinline__ void opt_block(int64_t n, int64_t base, float* __restrict__ w,
                                          const GradSrc& gs, float* __restrict__ m,
                                          float* __restrict__ v, const AdamParams& p,
                                          bool vec) {
  const int64_t end = min(n, base + (int64_t)kOptElemsPerBlock);
  if (vec && end - base == kOptElemsPerBlock) {
    f32x4 wv[4], gv[4], mv[4], vv[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      wv[it] = *reinterpret_cast<const f32x4*>(w + i);
      if (gs.splits <= 1) gv[it] = *reinterpret_cast<const f32x4*>(gs.g + i);
      if (KIND) {
        mv[it] = *reinterpret_cast<const f32x4*>(m + i);
        vv[it] = *reinterpret_cast<const f32x4*>(v + i);
      }
    }
    if (gs.splits > 1) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
        gv[it] = grad4(gs, base + ((int64_t)it * kOptBlock + threadIdx.x) * 4);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      if (KIND == 0) {
        wv[it] -= p.lr * gv[it];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float we = wv[it][e], me = mv[it][e], ve = vv[it][e];
          adam_elem(we, gv[it][e], me, ve, p);
          wv[it][e] = we; mv[it][e] = me; vv[it][e] = ve;
        }
        *reinterpret_cast<f32x4*>(m + i) = mv[it];
        *reinterpret_cast<f32x4*>(v + i) = vv[it];
      }
      *reinterpret_cast<f32x4*>(w + i) = wv[it];
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < end; i += kOptBlock) {
      const float g = grad1(gs, i);
      if (KIND == 0) {
        w[i] -= p.lr * g;
      } else {
        float we = w[i], me = m[i], ve = v[i];
        adam_elem(we, g, me, ve, p);
        w[i] = we; m[i] = me; v[i] = ve;
      }
    }
  }
}

template <int KIND>
__global__ void __launch_bounds__(kOptBlock)
opt_single_kernel(int64_t n, float* w, const float* g, float* m, float* v, AdamParams p, int vec) {
  const GradSrc gs{g, nullptr, 0, 1, nullptr};
  opt_block<KIND>(n, (int64_t)blockIdx.x * kOptElemsPerBlock, w, gs, m, v, p, vec);
}

// Split-K segments: the slices are summed by 4 lanes per 4-element group,
// lane q taking slices q, q+4, q+8, ... in order, then the 4 partial sums are
// combined in a fixed tree ((p0 + p1) + (p2 + p3)) with lane shuffles, so a
// thread walks a quarter of the slices and the result is bit-reproducible.
constexpr int kSplitElemsPerBlock = kOptSplitElemsPerBlock;  // one 4-element group per 4 lanes

template <int KIND>
__device__ __forceinline__ void opt_split_block(int64_t n, int64_t base, float* __restrict__ w,
                                                const GradSrc& gs, float* __restrict__ m,
                                                float* __restrict__ v, const AdamParams& p,
                                                bool vec) {
  const int q = threadIdx.x & 3;
  const int64_t e0 = base + (int64_t)(threadIdx.x >> 2) * 4;
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  const bool full = vec && e0 + 3 < n;
  if (full) {
#pragma unroll 4
    for (int k = q; k < gs.splits; k += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(gs.part + (int64_t)k * gs.stride + e0);
      g[0] += x[0]; g[1] += x[1]; g[2] += x[2]; g[3] += x[3];
    }
  } else {
    for (int k = q; k < gs.splits; k += 4)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e0 + e < n) g[e] += gs.part[(int64_t)k * gs.stride + e0 + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    g[e] += __shfl_xor(g[e], 1);
    g[e] += __shfl_xor(g[e], 2);
  }
  // every lane of the quad now holds the same sum; lane q updates element q
  const int64_t i = e0 + q;
  if (i >= n) return;
  const float gi = g[q];
  gs.out[i] = gi;
  if (KIND == 0) {
    w[i] -= p.lr * gi;
  } else {
    float we = w[i], me = m[i], ve = v[i];
    adam_elem(we, gi, me, ve, p);
    w[i] = we; m[i] = me; v[i] = ve;
  }
}

// Segments with many slices (more than kOptWideSplits): a whole wave per
// 4-element group, lane q summing slices q, q+64, ... in order, then a fixed
// 64-lane shuffle tree; four groups per workgroup.
template <int KIND>
__device__ __forceinline__ void opt_wide_split_block(int64_t n, int64_t base,
                                                     float* __restrict__ w, const GradSrc& gs,
                                                     float* __restrict__ m, float* __restrict__ v,
                                                     const AdamParams& p, bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t e0 = base + (int64_t)(threadIdx.x >> 6) * 4;
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  if (vec && e0 + 3 < n) {
#pragma unroll 2
    for (int k = lane; k < gs.splits; k += 64) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(gs.part + (int64_t)k * gs.stride + e0);
      g[0] += x[0]; g[1] += x[1]; g[2] += x[2]; g[3] += x[3];
    }
  } else {
    for (int k = lane; k < gs.splits; k += 64)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e0 + e < n) g[e] += gs.part[(int64_t)k * gs.stride + e0 + e];
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1)
#pragma unroll
    for (int e = 0; e < 4; ++e) g[e] += __shfl_xor(g[e], o);
  if (lane >= 4) return;
  const int64_t i = e0 + lane;
  if (i >= n) return;
  const float gi = g[lane];
  gs.out[i] = gi;
  if (KIND == 0) {
    w[i] -= p.lr * gi;
  } else {
    float we = w[i], me = m[i], ve = v[i];
    adam_elem(we, gi, me, ve, p);
    w[i] = we; m[i] = me; v[i] = ve;
  }
}

// One launch over several arrays: block b belongs to the segment whose
// prefix range [start_block[s], start_block[s+1]) contains it; a segment's
// elements per block are opt_elems_per_block(splits).
// Mean of the per-row losses by one workgroup: thread t takes rows t, t+256,
// ... in chunks of 8 (loaded together, added in order, float64), then a fixed
// shuffle tree and the 4 waves in order.
__device__ __forceinline__ void loss_mean_block(int64_t rows, const float* __restrict__ row_loss,
                                                float* __restrict__ loss) {
  __shared__ double red[kOptBlock / 64];
  double acc = 0.0;
  for (int64_t i0 = threadIdx.x; i0 < rows; i0 += 8 * kOptBlock) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + (int64_t)u * kOptBlock;
      x[u] = i < rows ? row_loss[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc += (double)x[u];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kOptBlock / 64; ++w) t += red[w];
    loss[0] = (float)(t / (double)rows);
  }
}

// The bias corrections of step t, in double, rounded once (the host forms
// the same expressions from its own step count).
__device__ __forceinline__ void device_step_consts(AdamParams& p) {
  const double t = (double)*p.step_dev;
  p.step_size = (float)(p.lr_d / (1.0 - pow(p.beta1_d, t)));
  p.inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - pow(p.beta2_d, t)));
}

__global__ void step_tick_kernel(int64_t* step_dev) {
  if (threadIdx.x == 0) step_dev[0] = step_dev[0] + 1;
}

template <int KIND>
__global__ void __launch_bounds__(kOptBlock)
opt_multi_kernel(OptSegs segs, AdamParams p) {
  if (KIND == 1 && p.step_dev != nullptr) device_step_consts(p);
  int64_t b = blockIdx.x;
  if (segs.rows > 0) {  // workgroup 0 (dispatched first) takes the loss mean
    if (b == 0) {
      loss_mean_block(segs.rows, segs.row_loss, segs.loss);
      return;
    }
    --b;
  }
  int s = 0;
  while (s + 1 < segs.count && b >= segs.start_block[s + 1]) ++s;
  const int64_t local = b - segs.start_block[s];
  const GradSrc gs{segs.g[s], segs.part[s], segs.part_stride[s], segs.splits[s], segs.g_out[s]};
  if (gs.splits > 1) {
    const bool vec = ((reinterpret_cast<uintptr_t>(gs.part) |
                       static_cast<uintptr_t>(gs.stride * 4)) & 15) == 0;
    if (gs.splits > kOptWideSplits)
      opt_wide_split_block<KIND>(segs.n[s], local * kOptWideElemsPerBlock, segs.w[s], gs,
                                 segs.m[s], segs.v[s], p, vec);
    else
      opt_split_block<KIND>(segs.n[s], local * kSplitElemsPerBlock, segs.w[s], gs, segs.m[s],
                            segs.v[s], p, vec);
    return;
  }
  uintptr_t addr = reinterpret_cast<uintptr_t>(segs.w[s]) | reinterpret_cast<uintptr_t>(gs.g);
  if (KIND) addr |= reinterpret_cast<uintptr_t>(segs.m[s]) | reinterpret_cast<uintptr_t>(segs.v[s]);
  opt_block<KIND>(segs.n[s], local * kOptElemsPerBlock, segs.w[s], gs, segs.m[s], segs.v[s], p,
                  (addr & 15) == 0);
}

}  // namespace

hipError_t launch_sgd(int64_t n, float* w, const float* g, const OptConsts& p, hipStream_t s) {
  const int64_t blocks = (n + kOptElemsPerBlock - 1) / kOptElemsPerBlock;
  const int vec = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(g)) & 15) == 0;
  hipLaunchKernelGGL(opt_single_kernel<0>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, n, w, g,
                     nullptr, nullptr, p, vec);
  return hipGetLastError();
}

hipError_t launch_adamw(int64_t n, float* w, const float* g, float* m, float* v,
                        const OptConsts& p, hipStream_t s) {
  const int64_t blocks = (n + kOptElemsPerBlock - 1) / kOptElemsPerBlock;
  const int vec = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(g) |
                    reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15) == 0;
  hipLaunchKernelGGL(opt_single_kernel<1>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, n, w, g,
                     m, v, p, vec);
  return hipGetLastError();
}

hipError_t launch_step_tick(int64_t* step_dev, hipStream_t s) {
  hipLaunchKernelGGL(step_tick_kernel, dim3(1), dim3(64), 0, s, step_dev);
  return hipGetLastError();
}

hipError_t launch_opt_multi(const OptSegs& segs, int kind, const OptConsts& p, hipStream_t s) {
  const int64_t blocks = segs.start_block[segs.count] + (segs.rows > 0 ? 1 : 0);
  if (blocks <= 0) return hipSuccess;
  if (kind == 0)
    hipLaunchKernelGGL(opt_multi_kernel<0>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, segs, p);
  else
    hipLaunchKernelGGL(opt_multi_kernel<1>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, segs, p);
  return hipGetLastError();
}

}  // namespace dl

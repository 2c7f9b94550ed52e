// SGD, AdamW and Adam updates (MuNet page, "What runs today": SGD and AdamW;
// noeira.nn docs, "Optimizers & losses": Adam; noeira.nn docs, "The design in
// one page": Adam's m and v live with the parameter).  Pure streaming
// kernels: 16-byte loads and stores, each thread handles four float4 groups
// so a workgroup moves 16 KB per array.
//
// Per element (decay = 1 - lr wd, omb1 = 1 - b1, omb2 = 1 - b2, step_size =
// lr / (1 - b1^t) and inv_sqrt_bc2 = 1 / sqrt(1 - b2^t) are formed in double
// and rounded once, on the host or, with a device step count, on the device):
//   AdamW: w *= decay;  Adam: g += wd w;  then
//   m = b1 m + omb1 g;  v = b2 v + omb2 g^2;  w -= step_size m / (sqrt(v) inv_sqrt_bc2 + eps)
// The fused options of the multi-array form: the gradient multiplied by the
// gradient control's factor (clip coefficient / loss scale) or the whole
// update skipped, e <- d e + (1 - d) w for the parameter average (MuNet page,
// "What runs today": EMA), and the bf16 RNE copy of the updated w.
#include "common.hpp"

namespace dl {
namespace {

using AdamParams = OptConsts;
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// One element of the update.  AdamW decays w before the Adam step; Adam adds
// the decay to the gradient (coupled), so it passes through both moments.
template <int KIND>
__device__ __forceinline__ void update_elem(float& w, float g, float& m, float& v,
                                            const AdamParams& p) {
  if (KIND == OPT_SGD) {
    w -= p.lr * g;
    return;
  }
  if (KIND == OPT_ADAMW)
    w *= p.decay;
  else
    g += p.wd * w;
  m = p.b1 * m + p.omb1 * g;
  v = p.b2 * v + p.omb2 * (g * g);
  w -= p.step_size * m / (sqrtf(v) * p.inv_sqrt_bc2 + p.eps);
}

// Per-array extras of the fused update: the parameter average and the bf16
// copy of the updated value (either may be null).
struct Extras {
  float* e;
  bf16_t* wb;
};

// Update element i with gradient gi (scalar paths).
template <int KIND, bool EXT>
__device__ __forceinline__ void update_one(int64_t i, float gi, float* __restrict__ w,
                                           float* __restrict__ m, float* __restrict__ v,
                                           const Extras& x, const AdamParams& p) {
  float we = w[i], me = 0.f, ve = 0.f;
  if (KIND != OPT_SGD) {
    me = m[i];
    ve = v[i];
  }
  update_elem<KIND>(we, gi, me, ve, p);
  w[i] = we;
  if (KIND != OPT_SGD) {
    m[i] = me;
    v[i] = ve;
  }
  if (EXT) {
    if (x.e != nullptr) x.e[i] = p.ema_d * x.e[i] + p.ema_omd * we;
    if (x.wb != nullptr) x.wb[i] = f32_to_bf16(we);
  }
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
// and for Adam m, v, and the average) is issued before the first store, so a
// thread keeps 8 to 20 loads in flight instead of waiting once per group.
// `mul` multiplies every gradient (the gradient control's factor; 1 without).
template <int KIND, bool EXT>
__device__ __forceinline__ void opt_block(int64_t n, int64_t base, float* __restrict__ w,
                                          const GradSrc& gs, float* __restrict__ m,
                                          float* __restrict__ v, const Extras& x, float mul,
                                          const AdamParams& p, bool vec) {
  const int64_t end = min(n, base + (int64_t)kOptElemsPerBlock);
  if (vec && end - base == kOptElemsPerBlock) {
    f32x4 wv[4], gv[4], mv[4], vv[4], ev[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      wv[it] = *reinterpret_cast<const f32x4*>(w + i);
      if (gs.splits <= 1) gv[it] = *reinterpret_cast<const f32x4*>(gs.g + i);
      if (KIND != OPT_SGD) {
        mv[it] = *reinterpret_cast<const f32x4*>(m + i);
        vv[it] = *reinterpret_cast<const f32x4*>(v + i);
      }
      if (EXT && x.e != nullptr) ev[it] = *reinterpret_cast<const f32x4*>(x.e + i);
    }
    if (gs.splits > 1) {
#pragma unroll
      for (int it = 0; it < 4; ++it)
        gv[it] = grad4(gs, base + ((int64_t)it * kOptBlock + threadIdx.x) * 4);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      if (EXT) gv[it] *= mul;
      if (KIND == OPT_SGD) {
        wv[it] -= p.lr * gv[it];
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float we = wv[it][e], me = mv[it][e], ve = vv[it][e];
          update_elem<KIND>(we, gv[it][e], me, ve, p);
          wv[it][e] = we; mv[it][e] = me; vv[it][e] = ve;
        }
        *reinterpret_cast<f32x4*>(m + i) = mv[it];
        *reinterpret_cast<f32x4*>(v + i) = vv[it];
      }
      *reinterpret_cast<f32x4*>(w + i) = wv[it];
      if (EXT && x.e != nullptr)
        *reinterpret_cast<f32x4*>(x.e + i) = p.ema_d * ev[it] + p.ema_omd * wv[it];
      if (EXT && x.wb != nullptr) {
        const u32x2v h = {pack_bf16x2(wv[it][0], wv[it][1]), pack_bf16x2(wv[it][2], wv[it][3])};
        *reinterpret_cast<u32x2v*>(x.wb + i) = h;
      }
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < end; i += kOptBlock) {
      float g = grad1(gs, i);
      if (EXT) g *= mul;
      update_one<KIND, EXT>(i, g, w, m, v, x, p);
    }
  }
}

template <int KIND>
__global__ void __launch_bounds__(kOptBlock)
opt_single_kernel(int64_t n, float* w, const float* g, float* m, float* v, AdamParams p, int vec) {
  const GradSrc gs{g, nullptr, 0, 1, nullptr};
  opt_block<KIND, false>(n, (int64_t)blockIdx.x * kOptElemsPerBlock, w, gs, m, v,
                         Extras{nullptr, nullptr}, 1.f, p, vec);
}

// Split-K segments of 5 to 32 slices: the slices are summed by 4 lanes per
// 4-element group, lane q taking slices q, q+4, q+8, ... in order, then the
// 4 partial sums are combined in a fixed tree ((p0 + p1) + (p2 + p3)) with
// lane shuffles, so a thread walks a quarter of the slices and the result is
// bit-reproducible.  (Up to 4 slices: opt_few_split_block, the same sums.)
constexpr int kSplitElemsPerBlock = kOptSplitElemsPerBlock;  // one 4-element group per 4 lanes

template <int KIND, bool EXT>
__device__ __forceinline__ void opt_split_block(int64_t n, int64_t base, float* __restrict__ w,
                                                const GradSrc& gs, float* __restrict__ m,
                                                float* __restrict__ v, const Extras& x,
                                                const AdamParams& p, bool vec) {
  const int q = threadIdx.x & 3;
  const int64_t e0 = base + (int64_t)(threadIdx.x >> 2) * 4;
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  const bool full = vec && e0 + 3 < n;
  if (full) {
#pragma unroll 4
    for (int k = q; k < gs.splits; k += 4) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(gs.part + (int64_t)k * gs.stride + e0);
      g[0] += xv[0]; g[1] += xv[1]; g[2] += xv[2]; g[3] += xv[3];
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
  update_one<KIND, EXT>(i, gi, w, m, v, x, p);
}

// Segments of 2 to 4 slices: one thread per 4-element group, four groups a
// thread as in opt_block, each slice of a group one float4 load (a missing
// slice reads slice 0 and counts as zero), all loads in flight together.
// The sum (s0 + s1) + (s2 + s3) is the 4-lane tree of opt_split_block when
// each lane holds one slice, so both forms give the same bits.
template <int KIND, bool EXT>
__device__ __forceinline__ void opt_few_split_block(int64_t n, int64_t base, float* __restrict__ w,
                                                    const GradSrc& gs, float* __restrict__ m,
                                                    float* __restrict__ v, const Extras& x,
                                                    const AdamParams& p, bool vec) {
  const int64_t end = min(n, base + (int64_t)kOptElemsPerBlock);
  if (vec && end - base == kOptElemsPerBlock) {
    f32x4 wv[4], mv[4], vv[4], ev[4], sv[4][4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int kk = k < gs.splits ? k : 0;
        sv[it][k] = *reinterpret_cast<const f32x4*>(gs.part + (int64_t)kk * gs.stride + i);
      }
      wv[it] = *reinterpret_cast<const f32x4*>(w + i);
      if (KIND != OPT_SGD) {
        mv[it] = *reinterpret_cast<const f32x4*>(m + i);
        vv[it] = *reinterpret_cast<const f32x4*>(v + i);
      }
      if (EXT && x.e != nullptr) ev[it] = *reinterpret_cast<const f32x4*>(x.e + i);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      // each lane's partial starts from +0 as in the 4-lane tree
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      const f32x4 s2 = gs.splits > 2 ? zero + sv[it][2] : zero;
      const f32x4 s3 = gs.splits > 3 ? zero + sv[it][3] : zero;
      const f32x4 gv = ((zero + sv[it][0]) + (zero + sv[it][1])) + (s2 + s3);
      *reinterpret_cast<f32x4*>(gs.out + i) = gv;
      if (KIND == OPT_SGD) {
        wv[it] -= p.lr * gv;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float we = wv[it][e], me = mv[it][e], ve = vv[it][e];
          update_elem<KIND>(we, gv[e], me, ve, p);
          wv[it][e] = we; mv[it][e] = me; vv[it][e] = ve;
        }
        *reinterpret_cast<f32x4*>(m + i) = mv[it];
        *reinterpret_cast<f32x4*>(v + i) = vv[it];
      }
      *reinterpret_cast<f32x4*>(w + i) = wv[it];
      if (EXT && x.e != nullptr)
        *reinterpret_cast<f32x4*>(x.e + i) = p.ema_d * ev[it] + p.ema_omd * wv[it];
      if (EXT && x.wb != nullptr) {
        const u32x2v h = {pack_bf16x2(wv[it][0], wv[it][1]), pack_bf16x2(wv[it][2], wv[it][3])};
        *reinterpret_cast<u32x2v*>(x.wb + i) = h;
      }
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < end; i += kOptBlock) {
      float s[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) s[k] = k < gs.splits ? 0.f + gs.part[(int64_t)k * gs.stride + i] : 0.f;
      const float gi = (s[0] + s[1]) + (s[2] + s[3]);
      gs.out[i] = gi;
      update_one<KIND, EXT>(i, gi, w, m, v, x, p);
    }
  }
}

// Segments with many slices (more than kOptWideSplits): a whole wave per
// 4-element group, lane q summing slices q, q+64, ... in order, then a fixed
// 64-lane shuffle tree; four groups per workgroup.
template <int KIND, bool EXT>
__device__ __forceinline__ void opt_wide_split_block(int64_t n, int64_t base,
                                                     float* __restrict__ w, const GradSrc& gs,
                                                     float* __restrict__ m, float* __restrict__ v,
                                                     const Extras& x, const AdamParams& p,
                                                     bool vec) {
  const int lane = threadIdx.x & 63;
  const int64_t e0 = base + (int64_t)(threadIdx.x >> 6) * 4;
  float g[4] = {0.f, 0.f, 0.f, 0.f};
  if (vec && e0 + 3 < n) {
#pragma unroll 2
    for (int k = lane; k < gs.splits; k += 64) {
      const f32x4 xv = *reinterpret_cast<const f32x4*>(gs.part + (int64_t)k * gs.stride + e0);
      g[0] += xv[0]; g[1] += xv[1]; g[2] += xv[2]; g[3] += xv[3];
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
  update_one<KIND, EXT>(i, gi, w, m, v, x, p);
}

// One launch over several arrays: block b belongs to the segment whose
// prefix range [start_block[s], start_block[s+1]) contains it; a segment's
// elements per block are opt_elems_per_block(splits).
// The learning rate (scheduled) and bias corrections of step t, in double,
// rounded once (the host forms the same expressions from its own step count).
template <int KIND>
__device__ __forceinline__ void device_step_consts(AdamParams& p) {
  const int64_t t = *p.step_dev;
  const double lr = lr_schedule(p.sched, p.lr_d, t);
  p.lr = (float)lr;
  if (KIND != OPT_SGD) {
    p.decay = (float)(1.0 - lr * p.wd_d);
    p.step_size = (float)(lr / (1.0 - pow(p.beta1_d, (double)t)));
    p.inv_sqrt_bc2 = (float)(1.0 / sqrt(1.0 - pow(p.beta2_d, (double)t)));
  }
}

__global__ void step_tick_kernel(int64_t* step_dev) {
  if (threadIdx.x == 0) step_dev[0] = step_dev[0] + 1;
}

// EXT: the gradient control (a skipped step returns at once, every gradient
// is multiplied by its factor), the parameter averages and the bf16 copies.
// The gradient pass has already finished any split sums when the control is
// on, so a segment with slices never meets a multiplier.
template <int KIND, bool EXT>
__global__ void __launch_bounds__(kOptBlock)
opt_multi_kernel(OptSegs segs, AdamParams p) {
  int64_t b = blockIdx.x;
  if (segs.rows > 0) {  // workgroup 0 (dispatched first) takes the loss mean
    if (b == 0) {
      loss_mean_block(segs.rows, segs.row_loss, segs.loss);
      return;
    }
    --b;
  }
  float mul = 1.f;
  if (EXT && p.ctl != nullptr) {
    if (p.ctl->skip) return;
    mul = p.ctl->mul;
  }
  if (p.step_dev != nullptr) device_step_consts<KIND>(p);
  int s = 0;
  while (s + 1 < segs.count && b >= segs.start_block[s + 1]) ++s;
  const int64_t local = b - segs.start_block[s];
  const GradSrc gs{segs.g[s], segs.part[s], segs.part_stride[s], segs.splits[s], segs.g_out[s]};
  const Extras x{EXT ? segs.ema[s] : nullptr, EXT ? segs.wb[s] : nullptr};
  if (gs.splits > 1) {
    const bool vec = ((reinterpret_cast<uintptr_t>(gs.part) |
                       static_cast<uintptr_t>(gs.stride * 4)) & 15) == 0;
    if (gs.splits > kOptWideSplits)
      opt_wide_split_block<KIND, EXT>(segs.n[s], local * kOptWideElemsPerBlock, segs.w[s], gs,
                                      segs.m[s], segs.v[s], x, p, vec);
    else if (gs.splits <= kOptFewSplits) {
      uintptr_t addr = reinterpret_cast<uintptr_t>(segs.w[s]) | reinterpret_cast<uintptr_t>(gs.out);
      if (KIND != OPT_SGD)
        addr |= reinterpret_cast<uintptr_t>(segs.m[s]) | reinterpret_cast<uintptr_t>(segs.v[s]);
      addr |= reinterpret_cast<uintptr_t>(x.e);
      const bool vec4 = vec && (addr & 15) == 0 && (reinterpret_cast<uintptr_t>(x.wb) & 7) == 0;
      opt_few_split_block<KIND, EXT>(segs.n[s], local * kOptElemsPerBlock, segs.w[s], gs,
                                     segs.m[s], segs.v[s], x, p, vec4);
    } else
      opt_split_block<KIND, EXT>(segs.n[s], local * kSplitElemsPerBlock, segs.w[s], gs,
                                 segs.m[s], segs.v[s], x, p, vec);
    return;
  }
  uintptr_t addr = reinterpret_cast<uintptr_t>(segs.w[s]) | reinterpret_cast<uintptr_t>(gs.g);
  if (KIND != OPT_SGD)
    addr |= reinterpret_cast<uintptr_t>(segs.m[s]) | reinterpret_cast<uintptr_t>(segs.v[s]);
  addr |= reinterpret_cast<uintptr_t>(x.e);
  bool vec = (addr & 15) == 0 && (reinterpret_cast<uintptr_t>(x.wb) & 7) == 0;
  opt_block<KIND, EXT>(segs.n[s], local * kOptElemsPerBlock, segs.w[s], gs, segs.m[s], segs.v[s],
                       x, mul, p, vec);
}

__global__ void __launch_bounds__(kOptBlock)
ema_kernel(int64_t n, float* __restrict__ e, const float* __restrict__ w, float d, float omd,
           int vec) {
  const int64_t base = (int64_t)blockIdx.x * kOptElemsPerBlock;
  const int64_t end = min(n, base + (int64_t)kOptElemsPerBlock);
  if (vec && end - base == kOptElemsPerBlock) {
    f32x4 ev[4], wv[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      ev[it] = *reinterpret_cast<const f32x4*>(e + i);
      wv[it] = *reinterpret_cast<const f32x4*>(w + i);
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int64_t i = base + ((int64_t)it * kOptBlock + threadIdx.x) * 4;
      *reinterpret_cast<f32x4*>(e + i) = d * ev[it] + omd * wv[it];
    }
  } else {
    for (int64_t i = base + threadIdx.x; i < end; i += kOptBlock) e[i] = d * e[i] + omd * w[i];
  }
}

}  // namespace

hipError_t launch_sgd(int64_t n, float* w, const float* g, const OptConsts& p, hipStream_t s) {
  const int64_t blocks = (n + kOptElemsPerBlock - 1) / kOptElemsPerBlock;
  const int vec = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(g)) & 15) == 0;
  hipLaunchKernelGGL(opt_single_kernel<OPT_SGD>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, n,
                     w, g, nullptr, nullptr, p, vec);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_adam_kind(int64_t n, float* w, const float* g, float* m, float* v,
                            const OptConsts& p, hipStream_t s) {
  const int64_t blocks = (n + kOptElemsPerBlock - 1) / kOptElemsPerBlock;
  const int vec = ((reinterpret_cast<uintptr_t>(w) | reinterpret_cast<uintptr_t>(g) |
                    reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v)) & 15) == 0;
  hipLaunchKernelGGL(opt_single_kernel<KIND>, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, n, w,
                     g, m, v, p, vec);
  return hipGetLastError();
}

hipError_t launch_adamw(int64_t n, float* w, const float* g, float* m, float* v,
                        const OptConsts& p, hipStream_t s) {
  return launch_adam_kind<OPT_ADAMW>(n, w, g, m, v, p, s);
}

hipError_t launch_adam(int64_t n, float* w, const float* g, float* m, float* v,
                       const OptConsts& p, hipStream_t s) {
  return launch_adam_kind<OPT_ADAM>(n, w, g, m, v, p, s);
}

hipError_t launch_ema(int64_t n, float* e, const float* w, float d, float omd, hipStream_t s) {
  const int64_t blocks = (n + kOptElemsPerBlock - 1) / kOptElemsPerBlock;
  const int vec = ((reinterpret_cast<uintptr_t>(e) | reinterpret_cast<uintptr_t>(w)) & 15) == 0;
  hipLaunchKernelGGL(ema_kernel, dim3((unsigned)blocks), dim3(kOptBlock), 0, s, n, e, w, d, omd,
                     vec);
  return hipGetLastError();
}

hipError_t launch_step_tick(int64_t* step_dev, hipStream_t s) {
  hipLaunchKernelGGL(step_tick_kernel, dim3(1), dim3(64), 0, s, step_dev);
  return hipGetLastError();
}

template <int KIND>
hipError_t launch_multi_kind(const OptSegs& segs, bool ext, const OptConsts& p, dim3 grid,
                             hipStream_t s) {
  if (ext)
    hipLaunchKernelGGL((opt_multi_kernel<KIND, true>), grid, dim3(kOptBlock), 0, s, segs, p);
  else
    hipLaunchKernelGGL((opt_multi_kernel<KIND, false>), grid, dim3(kOptBlock), 0, s, segs, p);
  return hipGetLastError();
}

hipError_t launch_opt_multi(const OptSegs& segs, int kind, const OptConsts& p, hipStream_t s) {
  const int64_t blocks = segs.start_block[segs.count] + (segs.rows > 0 ? 1 : 0);
  if (blocks <= 0) return hipSuccess;
  bool ext = p.ctl != nullptr;
  for (int k = 0; k < segs.count; ++k) ext = ext || segs.ema[k] != nullptr || segs.wb[k] != nullptr;
  const dim3 grid((unsigned)blocks);
  if (kind == OPT_SGD) return launch_multi_kind<OPT_SGD>(segs, ext, p, grid, s);
  if (kind == OPT_ADAMW) return launch_multi_kind<OPT_ADAMW>(segs, ext, p, grid, s);
  return launch_multi_kind<OPT_ADAM>(segs, ext, p, grid, s);
}

}  // namespace dl

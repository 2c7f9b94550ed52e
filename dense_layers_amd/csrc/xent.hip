// Softmax cross-entropy forward and backward in a single pass over the
// logits, with no log-probability tensor in between (Orthon page, "Selected
// Orthon vs. PyTorch results"; that page ties the gain to the number of
// classes, so here the lanes that own a row are chosen per class-count
// range).
//
// A row of C logits is owned by TPR consecutive threads (a lane group inside a
// wave for TPR <= 64, the whole workgroup of 1024 threads for wide rows).  Each
// thread keeps its slice of the row in registers, so HBM sees one read and
// one write per logit; row max, sum of exponentials and the label's logit are
// combined with cross-lane shuffles (plus LDS across waves when a workgroup
// owns the row).
//   lse = max + log(sum exp(z - max)),  loss_i = lse - z[y_i],
//   dlogits = (exp(z - max) / sum - [c == y_i]) / B.
// Per-row losses go to a buffer and a single workgroup sums them in a fixed
// order, so the mean is bit-reproducible.
#include "common.hpp"

namespace dl {
namespace {

constexpr int kXentBlock = 256;

template <int TPR, int BLOCK>
__device__ __forceinline__ float group_max(float v, float* red) {
  if (TPR <= 64) {
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < BLOCK / 64; ++w) r = fmaxf(r, red[w]);
    __syncthreads();
    return r;
  }
}

template <int TPR, int BLOCK>
__device__ __forceinline__ void group_sum2(float& a, float& b, float* red) {
  if (TPR <= 64) {
#pragma unroll
    for (int o = TPR / 2; o > 0; o >>= 1) {
      a += __shfl_xor(a, o);
      b += __shfl_xor(b, o);
    }
  } else {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      a += __shfl_xor(a, o);
      b += __shfl_xor(b, o);
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
      red[2 * wave] = a;
      red[2 * wave + 1] = b;
    }
    __syncthreads();
    a = 0.f;
    b = 0.f;
#pragma unroll
    for (int w = 0; w < BLOCK / 64; ++w) {
      a += red[2 * w];
      b += red[2 * w + 1];
    }
  }
}

// VEC: items are float4 (C % 4 == 0, 16-byte aligned rows), else floats.
// NI:  items cached per thread; the kernel is only launched with
//      C <= TPR * NI * (VEC ? 4 : 1).  BLOCK: threads per workgroup.
template <int TPR, int NI, bool VEC, int BLOCK = kXentBlock>
__global__ void __launch_bounds__(BLOCK)
xent_rows_kernel(int64_t B, int C, const float* logits, const int32_t* __restrict__ labels,
                 float* __restrict__ row_loss, float* dlogits, float invB,
                 const float* dscale) {
  if (dscale != nullptr) invB *= *dscale;  // loss scale
  constexpr int RPB = BLOCK / TPR;
  constexpr int W = VEC ? 4 : 1;
  __shared__ float red[2 * BLOCK / 64];
  const int lr = threadIdx.x % TPR;
  const int64_t row = (int64_t)blockIdx.x * RPB + threadIdx.x / TPR;
  const bool active = row < B;
  const int64_t base = (active ? row : 0) * (int64_t)C;
  const int y = active ? labels[row] : 0;
  const bool valid = (y >= 0) && (y < C);

  float v[NI][W];
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int c0 = (lr + j * TPR) * W;
    if (VEC) {
      f32x4 x = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
      if (active && c0 < C) x = *reinterpret_cast<const f32x4*>(logits + base + c0);
#pragma unroll
      for (int e = 0; e < W; ++e) v[j][e] = x[e];
    } else {
      v[j][0] = (active && c0 < C) ? logits[base + c0] : -INFINITY;
    }
#pragma unroll
    for (int e = 0; e < W; ++e) m = fmaxf(m, v[j][e]);
  }
  m = group_max<TPR, BLOCK>(m, red);

  float s = 0.f, zy = 0.f;
#pragma unroll
  for (int j = 0; j < NI; ++j)
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const int c = (lr + j * TPR) * W + e;
      const float x = v[j][e];
      if (c < C) {
        const float ex = __expf(x - m);
        v[j][e] = ex;
        s += ex;
        if (c == y) zy = x;
      }
    }
  group_sum2<TPR, BLOCK>(s, zy, red);

  const float inv_s = 1.0f / s;
  if (active && lr == 0)
    row_loss[row] = valid ? (m + __logf(s)) - zy : __builtin_nanf("");
  if (!active) return;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int c0 = (lr + j * TPR) * W;
    if (c0 >= C) continue;
    float o[W];
#pragma unroll
    for (int e = 0; e < W; ++e) {
      const float onehot = (c0 + e == y) ? 1.0f : 0.0f;
      o[e] = (v[j][e] * inv_s - onehot) * invB;
    }
    if (VEC) {
      f32x4 x = {o[0], o[W > 1 ? 1 : 0], o[W > 2 ? 2 : 0], o[W > 3 ? 3 : 0]};
      *reinterpret_cast<f32x4*>(dlogits + base + c0) = x;
    } else {
      dlogits[base + c0] = o[0];
    }
  }
}

// One row per workgroup of BLOCK threads (C % 4 == 0, C <= BLOCK * NI * 4),
// NI float4 of the row per thread, addressed through buffer resources over
// the row (base and size in scalar registers, no 64-bit address per item).
// An item past the row gets the per-lane offset C * 4 (the range check
// applies to the per-lane offset, not to the uniform one): its load returns
// zero, kept out of the max, and its store is dropped.  The loads carry the
// non-temporal cache hint (each logit is read once); the stores do not (the
// hint on the stores, alone or with the loads, measured slower).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kNontemporal = 2;  // cache-policy operand of a buffer access: nt
template <int BLOCK, int NI>
__global__ void __launch_bounds__(BLOCK)
xent_row_wg_kernel(int C, const float* logits, const int32_t* __restrict__ labels,
                   float* __restrict__ row_loss, float* dlogits, float invB,
                   const float* dscale) {
  if (dscale != nullptr) invB *= *dscale;  // loss scale
  __shared__ float red[2 * BLOCK / 64];
  const int64_t row = blockIdx.x;
  const int y = labels[row];
  const bool valid = (y >= 0) && (y < C);
  const __amdgpu_buffer_rsrc_t in = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(logits + row * C), 0, C * 4, 0x00020000);
  const __amdgpu_buffer_rsrc_t out =
      __builtin_amdgcn_make_buffer_rsrc(dlogits + row * C, 0, C * 4, 0x00020000);
  auto item_off = [&](int j) {
    const int c0 = (int)(threadIdx.x + j * BLOCK) * 4;
    return c0 < C ? c0 * 4 : C * 4;
  };
  f32x4 v[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j)
    v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(in, item_off(j), 0, kNontemporal));
  float m = -INFINITY;
#pragma unroll
  for (int j = 0; j < NI; ++j)
    if ((int)(threadIdx.x + j * BLOCK) * 4 < C)
      m = fmaxf(fmaxf(m, fmaxf(v[j][0], v[j][1])), fmaxf(v[j][2], v[j][3]));
  m = group_max<BLOCK, BLOCK>(m, red);
  float s = 0.f, zy = 0.f;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int c0 = (int)(threadIdx.x + j * BLOCK) * 4;
    if (c0 < C) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (c0 + e == y) zy = v[j][e];
        v[j][e] = __expf(v[j][e] - m);
        s += v[j][e];
      }
    }
  }
  group_sum2<BLOCK, BLOCK>(s, zy, red);
  if (threadIdx.x == 0) row_loss[row] = valid ? (m + __logf(s)) - zy : __builtin_nanf("");
  const float inv_s = 1.0f / s;
#pragma unroll
  for (int j = 0; j < NI; ++j) {
    const int c0 = (int)(threadIdx.x + j * BLOCK) * 4;
    f32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = (v[j][e] * inv_s - (c0 + e == y ? 1.0f : 0.0f)) * invB;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), out, item_off(j), 0, 0);
  }
}

// Rows too wide to cache in registers: one workgroup per row, two passes
// (the second read normally hits L2 / the 256 MB Infinity Cache).
__global__ void __launch_bounds__(kXentBlock)
xent_rows_wide_kernel(int64_t B, int64_t C, const float* logits, const int32_t* __restrict__ labels,
                      float* __restrict__ row_loss, float* dlogits, float invB,
                 const float* dscale) {
  if (dscale != nullptr) invB *= *dscale;  // loss scale
  __shared__ float red[2 * kXentBlock / 64];
  const int64_t row = blockIdx.x;
  const int64_t base = row * C;
  const int y = labels[row];
  const bool valid = (y >= 0) && (y < C);
  float m = -INFINITY;
  for (int64_t c = threadIdx.x; c < C; c += kXentBlock) m = fmaxf(m, logits[base + c]);
  m = group_max<kXentBlock, kXentBlock>(m, red);
  float s = 0.f, zy = 0.f;
  for (int64_t c = threadIdx.x; c < C; c += kXentBlock) {
    const float x = logits[base + c];
    s += __expf(x - m);
    if (c == y) zy = x;
  }
  group_sum2<kXentBlock, kXentBlock>(s, zy, red);
  if (threadIdx.x == 0) row_loss[row] = valid ? (m + __logf(s)) - zy : __builtin_nanf("");
  __syncthreads();  // every read of this row precedes the first in-place write
  const float inv_s = 1.0f / s;
  for (int64_t c = threadIdx.x; c < C; c += kXentBlock) {
    const float x = logits[base + c];
    dlogits[base + c] = (__expf(x - m) * inv_s - (c == y ? 1.0f : 0.0f)) * invB;
  }
}

// Mean of the per-row losses: one workgroup of 1024 threads, fixed summation
// order (each thread a strided slice, then a tree), float64 accumulation.
constexpr int kMeanThreads = 1024;
__global__ void __launch_bounds__(kMeanThreads)
loss_mean_kernel(int64_t B, const float* __restrict__ row_loss, float* __restrict__ loss) {
  __shared__ double red[kMeanThreads / 64];
  double acc = 0.0;
  int64_t i = threadIdx.x;
  for (; i + 3 * kMeanThreads < B; i += 4 * kMeanThreads) {
    const float a = row_loss[i], b = row_loss[i + kMeanThreads];
    const float c = row_loss[i + 2 * kMeanThreads], d = row_loss[i + 3 * kMeanThreads];
    acc += ((double)a + (double)b) + ((double)c + (double)d);
  }
  for (; i < B; i += kMeanThreads) acc += (double)row_loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    double t = 0.0;
    for (int w = 0; w < kMeanThreads / 64; ++w) t += red[w];
    loss[0] = (float)(t / (double)B);
  }
}

// Fused classifier head, after its forward GEMM: row i's log-sum-exp from the
// T column tiles' (max, sum exp(z - max)) pairs part[2 (t B + i)]:
//   m = max_t m_t,  s = sum_t s_t exp(m_t - m),  lse = m + log s,
// and its loss lse - z[i, y_i] (NaN for a label outside [0, C)).  A
// workgroup of kLseWaves waves takes 64 rows (a lane per row, so each read of
// a tile is 512 contiguous bytes); wave w takes the tiles w, w + kLseWaves,
// ..., keeping them in registers when T <= kLseWaves kLseMaxPer (else it
// reads them twice).  The maxima combine exactly in any order; the sums are
// added in tile order within a wave, then the waves' sums in wave order.
constexpr int kLseWaves = 8;
constexpr int kLseMaxPer = 32;
__global__ void __launch_bounds__(kLseWaves * 64)
xent_lse_kernel(int64_t B, int64_t C, int T, const float* __restrict__ part,
                const float* __restrict__ logits, const int32_t* __restrict__ labels,
                float* __restrict__ lse, float* __restrict__ row_loss) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  __shared__ float red[kLseWaves][64];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = (int64_t)blockIdx.x * 64 + lane;
  const bool ok = row < B;
  const f32x2* p = reinterpret_cast<const f32x2*>(part) + (ok ? row : 0);  // rows past B: row 0
  float m = -INFINITY, s = 0.f;
  if (T <= kLseWaves * kLseMaxPer) {
    f32x2 v[kLseMaxPer];
#pragma unroll
    for (int i = 0; i < kLseMaxPer; ++i) {
      const int t = w + kLseWaves * i;
      v[i] = t < T ? p[(int64_t)t * B] : f32x2{-INFINITY, 0.f};
    }
#pragma unroll
    for (int i = 0; i < kLseMaxPer; ++i) m = fmaxf(m, v[i][0]);
    red[w][lane] = m;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kLseWaves; ++x) m = fmaxf(m, red[x][lane]);
#pragma unroll
    for (int i = 0; i < kLseMaxPer; ++i)
      if (w + kLseWaves * i < T) s += v[i][1] * __expf(v[i][0] - m);
  } else {
    for (int t = w; t < T; t += kLseWaves) m = fmaxf(m, p[(int64_t)t * B][0]);
    red[w][lane] = m;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < kLseWaves; ++x) m = fmaxf(m, red[x][lane]);
    for (int t = w; t < T; t += kLseWaves) {
      const f32x2 v = p[(int64_t)t * B];
      s += v[1] * __expf(v[0] - m);
    }
  }
  __syncthreads();  // every wave has read the maxima
  red[w][lane] = s;
  __syncthreads();
  if (w != 0 || !ok) return;
  s = red[0][lane];
#pragma unroll
  for (int x = 1; x < kLseWaves; ++x) s += red[x][lane];
  const float l = m + logf(s);
  lse[row] = l;
  const int32_t y = labels[row];
  row_loss[row] = (y >= 0 && (int64_t)y < C) ? l - logits[row * C + y] : __builtin_nanf("");
}

constexpr int kLseBlock = 256;  // the row-record pass

// Per-row records of the fused head's backward: exponent offset and label.
__global__ void __launch_bounds__(kLseBlock)
xent_rows_pack_kernel(int64_t B, const float* __restrict__ lse, const int32_t* __restrict__ labels,
                      float log2B, float* __restrict__ rows) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const int64_t i = (int64_t)blockIdx.x * kLseBlock + threadIdx.x;
  if (i >= B) return;
  constexpr float kLog2e = 1.4426950408889634f;
  const f32x2 rec = {fmaf(lse[i], kLog2e, log2B), __int_as_float(labels[i])};
  reinterpret_cast<f32x2*>(rows)[i] = rec;
}

// Labels outside [0, C): one workgroup strides over the batch, counts per
// thread, then a fixed-order tree; one lane stores the count.
__global__ void __launch_bounds__(kMeanThreads)
label_check_kernel(int64_t B, int64_t C, const int32_t* __restrict__ labels, int* __restrict__ bad) {
  __shared__ int red[kMeanThreads / 64];
  int n = 0;
  for (int64_t i = threadIdx.x; i < B; i += kMeanThreads) {
    const int32_t y = labels[i];
    n += (y < 0 || (int64_t)y >= C) ? 1 : 0;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = n;
  __syncthreads();
  if (threadIdx.x == 0) {
    int t = 0;
    for (int w = 0; w < kMeanThreads / 64; ++w) t += red[w];
    bad[0] = t;
  }
}

template <int TPR, int NI, bool VEC, int BLOCK = kXentBlock>
hipError_t launch_rows(int64_t B, int64_t C, const float* logits, const int32_t* labels,
                       float* row_loss, float* dlogits, const float* dscale, hipStream_t s) {
  constexpr int RPB = BLOCK / TPR;
  const int64_t blocks = (B + RPB - 1) / RPB;
  hipLaunchKernelGGL((xent_rows_kernel<TPR, NI, VEC, BLOCK>), dim3((unsigned)blocks), dim3(BLOCK), 0,
                     s, B, (int)C, logits, labels, row_loss, dlogits, (float)(1.0 / (double)B),
                     dscale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_xent(int64_t B, int64_t C, const float* logits, const int32_t* labels,
                       float* row_loss, float* dlogits, float* loss, hipStream_t s,
                       const float* dscale) {
  const bool vec = (C % 4 == 0) && ((reinterpret_cast<uintptr_t>(logits) & 15) == 0) &&
                   ((reinterpret_cast<uintptr_t>(dlogits) & 15) == 0);
  hipError_t e;
  if (C <= 32)
    e = launch_rows<8, 4, false>(B, C, logits, labels, row_loss, dlogits, dscale, s);
  else if (C <= 256)
    e = vec ? launch_rows<32, 2, true>(B, C, logits, labels, row_loss, dlogits, dscale, s)
            : launch_rows<32, 8, false>(B, C, logits, labels, row_loss, dlogits, dscale, s);
  else if (C <= 2048)
    e = vec ? launch_rows<64, 8, true>(B, C, logits, labels, row_loss, dlogits, dscale, s)
            : launch_rows<64, 32, false>(B, C, logits, labels, row_loss, dlogits, dscale, s);
  else if (vec && C <= 32768) {  // a workgroup of 1024 threads per row, 8 float4 each
    hipLaunchKernelGGL((xent_row_wg_kernel<1024, 8>), dim3((unsigned)B), dim3(1024), 0, s, (int)C,
                       logits, labels, row_loss, dlogits, (float)(1.0 / (double)B), dscale);
    e = hipGetLastError();
  }
  else {
    hipLaunchKernelGGL(xent_rows_wide_kernel, dim3((unsigned)B), dim3(kXentBlock), 0, s, B, C,
                       logits, labels, row_loss, dlogits, (float)(1.0 / (double)B), dscale);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  return launch_loss_mean(B, row_loss, loss, s);
}

hipError_t launch_xent_lse(int64_t B, int64_t C, int T, const float* part, const float* logits,
                           const int32_t* labels, float* lse, float* row_loss, hipStream_t s) {
  const int64_t blocks = (B + 63) / 64;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(xent_lse_kernel, dim3((unsigned)blocks), dim3(kLseWaves * 64), 0, s, B, C, T,
                     part, logits, labels, lse, row_loss);
  return hipGetLastError();
}

hipError_t launch_xent_rows(int64_t B, const float* lse, const int32_t* labels, float log2B,
                            float* rows, hipStream_t s) {
  const int64_t blocks = (B + kLseBlock - 1) / kLseBlock;
  hipLaunchKernelGGL(xent_rows_pack_kernel, dim3((unsigned)blocks), dim3(kLseBlock), 0, s, B, lse,
                     labels, log2B, rows);
  return hipGetLastError();
}

hipError_t launch_label_check(int64_t B, int64_t C, const int32_t* labels, int* bad,
                              hipStream_t s) {
  hipLaunchKernelGGL(label_check_kernel, dim3(1), dim3(kMeanThreads), 0, s, B, C, labels, bad);
  return hipGetLastError();
}

hipError_t launch_loss_mean(int64_t B, const float* row_loss, float* loss, hipStream_t s) {
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(kMeanThreads), 0, s, B, row_loss, loss);
  return hipGetLastError();
}

}  // namespace dl

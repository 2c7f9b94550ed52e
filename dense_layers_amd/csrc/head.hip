// Narrow classifier head of the MLP step in one pass over the rows: the last
// Linear (identity activation), the fused softmax cross-entropy and the vjp of
// that Linear, for C <= 16 classes and in <= 256 features.
//
// The pieces are those of the step (noeira.nn docs, "The design in one page":
// LinearAct forward and vjp, the backward pass as their composition; the
// cross-entropy read once, Orthon page, "Selected Orthon vs. PyTorch
// results").  With so few classes every product is a short dot product per
// row, so a workgroup takes 32 rows of the head's input H, keeps them and W in
// LDS and computes, per row,
//   z = W h + b,  loss = logsumexp(z) - z[y],  g = (softmax(z) - onehot(y)) / B,
//   dh = (W^T g) * act'(h)                 (written over h, like the dX fold)
// and, over its rows, the partial sums dW_s = sum_r g_r h_r^T and
// db_s = sum_r g_r (rows in order; a workgroup loops over several 32-row
// tiles and keeps its slice in registers, at most 256 slices).  The logits
// never reach HBM.  The slices of all workgroups are added in slice order by
// the optimizer kernel of the step, exactly as split-K partials are.
#include "common.hpp"

namespace dl {
namespace {

constexpr int kHeadThreads = 512;
constexpr int kHeadTPR = 16;                       // threads per row
constexpr int kHeadRows = kHeadThreads / kHeadTPR;  // rows per tile
constexpr int kHeadCMax = 16;
constexpr int kHeadKMax = 256;
constexpr int kHeadMaxSlices = 256;                // workgroups (dW / db partial slices)
constexpr int kHeadPairs = kHeadKMax * (kHeadCMax / 4) / kHeadThreads;  // (k, 4 classes) per thread
constexpr int kHeadLoads = kHeadRows * kHeadKMax / kHeadThreads;       // tile floats per thread

// DPP move of v from the lane CTRL selects within its row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each row of 16 lanes, left in every lane of the row, by DPP
// moves (swap neighbours, swap pairs, mirror each half of 8, mirror the 16)
// instead of LDS-routed shuffles.  Each lane adds the same two operands at
// every step (in swapped order), so all 16 results are bit-identical.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Workgroup b takes row tiles [b * tiles_per, (b + 1) * tiles_per).  VEC:
// K % 4 == 0 and H, dH 16-byte aligned (tile moved as float4).
template <bool VEC>
__global__ void __launch_bounds__(kHeadThreads)
head_xent_kernel(int64_t B, int K, int C, int64_t tiles_per, const float* H, float* dH,
                 int prev_act, const float* __restrict__ W, const float* __restrict__ bias,
                 const int32_t* __restrict__ labels, float* __restrict__ row_loss,
                 float* __restrict__ dW_part, float* __restrict__ db_part, float invB,
                 const float* dscale) {
  if (dscale != nullptr) invB *= *dscale;  // loss scale
  constexpr int KP = kHeadKMax + 1;  // padded row stride of the row tiles
  // W transposed, classes padded to 16 with zeros: Wt[k][c]
  __shared__ __attribute__((aligned(16))) float Wt[kHeadKMax * kHeadCMax];
  __shared__ float Hs[kHeadRows * KP];
  __shared__ float Gs[kHeadRows * KP];
  __shared__ __attribute__((aligned(16))) float Ds[kHeadRows * kHeadCMax];
  const int tid = threadIdx.x;
  const int r = tid / kHeadTPR, lr = tid % kHeadTPR;
  {
    // all loads of W in flight before the first LDS store
    float wr[kHeadKMax * kHeadCMax / kHeadThreads];
#pragma unroll
    for (int j = 0; j < kHeadKMax * kHeadCMax / kHeadThreads; ++j) {
      const int i = tid + j * kHeadThreads;
      const int k = i / kHeadCMax, c = i % kHeadCMax;
      wr[j] = (k < K && c < C) ? W[(int64_t)c * K + k] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < kHeadKMax * kHeadCMax / kHeadThreads; ++j) Wt[tid + j * kHeadThreads] = wr[j];
  }
  float bc[kHeadCMax];
#pragma unroll
  for (int c = 0; c < kHeadCMax; ++c) bc[c] = c < C ? bias[c] : 0.f;

  // this thread's (k, 4-class group) pairs of the dW slice
  int pk[kHeadPairs], pc[kHeadPairs];
  float acc[kHeadPairs][4];
#pragma unroll
  for (int j = 0; j < kHeadPairs; ++j) {
    const int p = tid + j * kHeadThreads;
    pk[j] = p % K;
    pc[j] = p < K * (kHeadCMax / 4) ? (p / K) * 4 : -1;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
  }
  float dbacc = 0.f;  // threads < C: db of class tid

  const int64_t ntiles = (B + kHeadRows - 1) / kHeadRows;
  const int64_t t_end = min<int64_t>(ntiles, ((int64_t)blockIdx.x + 1) * tiles_per);
  for (int64_t t = (int64_t)blockIdx.x * tiles_per; t < t_end; ++t) {
    const int64_t r0 = t * kHeadRows;
    const int nrows = (int)min<int64_t>(kHeadRows, B - r0);
    const int n = nrows * K;  // the tile is one contiguous run of H
    const float* src = H + r0 * K;
    // every load of the tile (and the row's label) in flight before the
    // first LDS store
    const bool active = r < nrows;
    const int y = active ? labels[r0 + r] : -1;
    float v[kHeadLoads];
    if (VEC) {
#pragma unroll
      for (int j = 0; j < kHeadLoads / 4; ++j) {
        const int e = (tid + j * kHeadThreads) * 4;
        f32x4 x = {0.f, 0.f, 0.f, 0.f};
        if (e < n) x = *reinterpret_cast<const f32x4*>(src + e);
        v[4 * j] = x[0]; v[4 * j + 1] = x[1]; v[4 * j + 2] = x[2]; v[4 * j + 3] = x[3];
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHeadLoads; ++j) {
        const int e = tid + j * kHeadThreads;
        v[j] = e < n ? src[e] : 0.f;
      }
    }
    __syncthreads();  // the previous tile's LDS reads are done
    if (VEC) {
#pragma unroll
      for (int j = 0; j < kHeadLoads / 4; ++j) {
        const int e = (tid + j * kHeadThreads) * 4;
        if (e < kHeadRows * K) {
          const int q = e / K, k = e - q * K;
#pragma unroll
          for (int u = 0; u < 4; ++u) Hs[q * KP + k + u] = v[4 * j + u];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < kHeadLoads; ++j) {
        const int e = tid + j * kHeadThreads;
        if (e < kHeadRows * K) {
          const int q = e / K;
          Hs[q * KP + e - q * K] = v[j];
        }
      }
    }
    __syncthreads();

    const bool valid = y >= 0 && y < C;
    float z[kHeadCMax];
#pragma unroll
    for (int c = 0; c < kHeadCMax; ++c) z[c] = 0.f;
#pragma unroll
    for (int kk = 0; kk < kHeadKMax / kHeadTPR; ++kk) {
      const int k = lr + kk * kHeadTPR;
      if (k >= K) break;
      const float h = Hs[r * KP + k];
#pragma unroll
      for (int c4 = 0; c4 < kHeadCMax / 4; ++c4) {
        const f32x4 w = *reinterpret_cast<const f32x4*>(&Wt[k * kHeadCMax + c4 * 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) z[c4 * 4 + e] += h * w[e];
      }
    }
    float m = -INFINITY;
#pragma unroll
    for (int c = 0; c < kHeadCMax; ++c) {
      z[c] = row16_sum(z[c]);
      z[c] += bc[c];
      if (c < C) m = fmaxf(m, z[c]);
    }
    float s = 0.f, zy = 0.f;
#pragma unroll
    for (int c = 0; c < kHeadCMax; ++c) {
      if (c == y) zy = z[c];
      z[c] = c < C ? __expf(z[c] - m) : 0.f;
      s += z[c];
    }
    const float inv_s = 1.0f / s;
    if (active && lr == 0) row_loss[r0 + r] = valid ? (m + __logf(s)) - zy : __builtin_nanf("");
    float g[kHeadCMax];
#pragma unroll
    for (int c = 0; c < kHeadCMax; ++c)
      g[c] = (active && c < C) ? (z[c] * inv_s - (c == y ? 1.0f : 0.0f)) * invB : 0.f;
    if (lr < kHeadCMax / 4) {
      // lane lr of the row stores classes 4 lr .. 4 lr + 3
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c4 = 0; c4 < kHeadCMax / 4; ++c4)
        if (c4 == lr) x = f32x4{g[4 * c4], g[4 * c4 + 1], g[4 * c4 + 2], g[4 * c4 + 3]};
      *reinterpret_cast<f32x4*>(&Ds[r * kHeadCMax + lr * 4]) = x;
    }
    if (dH != nullptr) {
#pragma unroll
      for (int kk = 0; kk < kHeadKMax / kHeadTPR; ++kk) {
        const int k = lr + kk * kHeadTPR;
        if (k >= K) break;
        float d = 0.f;
#pragma unroll
        for (int c4 = 0; c4 < kHeadCMax / 4; ++c4) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(&Wt[k * kHeadCMax + c4 * 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) d += g[c4 * 4 + e] * w[e];
        }
        Gs[r * KP + k] = d * act_deriv(prev_act, Hs[r * KP + k]);
      }
    }
    __syncthreads();

    // this tile's rows, in order, into the workgroup's dW / db slice
#pragma unroll
    for (int j = 0; j < kHeadPairs; ++j) {
      if (pc[j] < 0) continue;
      float a0 = acc[j][0], a1 = acc[j][1], a2 = acc[j][2], a3 = acc[j][3];
#pragma unroll 8
      for (int q = 0; q < kHeadRows; ++q) {
        const float h = Hs[q * KP + pk[j]];
        const f32x4 d = *reinterpret_cast<const f32x4*>(&Ds[q * kHeadCMax + pc[j]]);
        a0 += d[0] * h; a1 += d[1] * h; a2 += d[2] * h; a3 += d[3] * h;
      }
      acc[j][0] = a0; acc[j][1] = a1; acc[j][2] = a2; acc[j][3] = a3;
    }
    if (tid < C)
      for (int q = 0; q < kHeadRows; ++q) dbacc += Ds[q * kHeadCMax + tid];
    if (dH != nullptr) {
      float* dst = dH + r0 * K;
      if (VEC) {
#pragma unroll
        for (int j = 0; j < kHeadLoads / 4; ++j) {
          const int e = (tid + j * kHeadThreads) * 4;
          if (e < n) {
            const int q = e / K, k = e - q * K;
            const f32x4 x = {Gs[q * KP + k], Gs[q * KP + k + 1], Gs[q * KP + k + 2],
                             Gs[q * KP + k + 3]};
            *reinterpret_cast<f32x4*>(dst + e) = x;
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < kHeadLoads; ++j) {
          const int e = tid + j * kHeadThreads;
          if (e < n) {
            const int q = e / K;
            dst[e] = Gs[q * KP + e - q * K];
          }
        }
      }
    }
  }

  float* dWp = dW_part + (int64_t)blockIdx.x * C * K;
#pragma unroll
  for (int j = 0; j < kHeadPairs; ++j) {
    if (pc[j] < 0) continue;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (pc[j] + e < C) dWp[(int64_t)(pc[j] + e) * K + pk[j]] = acc[j][e];
  }
  if (tid < C) db_part[(int64_t)blockIdx.x * C + tid] = dbacc;
}

}  // namespace

int64_t head_xent_slices(int64_t B) {
  const int64_t ntiles = (B + kHeadRows - 1) / kHeadRows;
  const int64_t per = (ntiles + kHeadMaxSlices - 1) / kHeadMaxSlices;
  return (ntiles + per - 1) / per;
}

bool head_xent_fits(int64_t K, int64_t C) {
  return C >= 1 && C <= kHeadCMax && K >= 1 && K <= kHeadKMax;
}

hipError_t launch_head_xent(int64_t B, int K, int C, const float* H, float* dH, int prev_act,
                            const float* W, const float* bias, const int32_t* labels,
                            float* row_loss, float* dW_part, float* db_part, hipStream_t s,
                            const float* dscale) {
  if (!head_xent_fits(K, C) || B < 1) return hipErrorInvalidValue;
  const int64_t ntiles = (B + kHeadRows - 1) / kHeadRows;
  const int64_t per = (ntiles + kHeadMaxSlices - 1) / kHeadMaxSlices;
  const int64_t blocks = (ntiles + per - 1) / per;
  const bool vec = K % 4 == 0 && ((reinterpret_cast<uintptr_t>(H) | reinterpret_cast<uintptr_t>(dH)) & 15) == 0;
  if (vec)
    hipLaunchKernelGGL(head_xent_kernel<true>, dim3((unsigned)blocks), dim3(kHeadThreads), 0, s, B,
                       K, C, per, H, dH, prev_act, W, bias, labels, row_loss, dW_part, db_part,
                       (float)(1.0 / (double)B), dscale);
  else
    hipLaunchKernelGGL(head_xent_kernel<false>, dim3((unsigned)blocks), dim3(kHeadThreads), 0, s, B,
                       K, C, per, H, dH, prev_act, W, bias, labels, row_loss, dW_part, db_part,
                       (float)(1.0 / (double)B), dscale);
  return hipGetLastError();
}

}  // namespace dl

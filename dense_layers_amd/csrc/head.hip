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
#include "head_rows.hpp"

namespace dl {
namespace {

constexpr int kHeadLoads = kHeadRows * kHeadKMax / kHeadThreads;  // tile floats per thread
constexpr int KP = kHeadKMax + 1;  // padded row stride of the row tiles

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
  // W transposed, classes padded to 16 with zeros: Wt[k][c]
  __shared__ __attribute__((aligned(16))) float Wt[kHeadKMax * kHeadCMax];
  __shared__ float Hs[kHeadRows * KP];
  __shared__ float Gs[kHeadRows * KP];
  __shared__ __attribute__((aligned(16))) float Ds[kHeadRows * kHeadCMax];
  __shared__ float Bc[kHeadCMax];
  const int tid = threadIdx.x;
  const int r = tid / kHeadTPR, lr = tid % kHeadTPR;
  head_load_wt(W, Wt, tid, K, C);
  if (tid < kHeadCMax) Bc[tid] = tid < C ? bias[tid] : 0.f;
  HeadSlice sl;
  sl.init(tid, K);

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

    float g[kHeadCMax];
    head_row_loss<KP>(Hs, Wt, Bc, Ds, r, lr, K, C, y, active, invB, row_loss, r0 + r, g);
    if (dH != nullptr) head_row_dx<KP>(Hs, Wt, Gs, r, lr, K, prev_act, g);
    __syncthreads();

    // this tile's rows, in order, into the workgroup's dW / db slice
    sl.add_tile<KP>(Hs, Ds, tid, C);
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

  sl.store(dW_part, db_part, blockIdx.x, tid, K, C);
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

// Row-wise pieces of the narrow classifier head (last Linear with C <= 16
// classes and K <= 256 inputs, softmax cross-entropy and its vjp), shared by
// the head kernel and the MLP-step tail kernel, so that both compute every
// value with the same operations in the same order.
//
// The pieces follow the LinearAct forward / vjp of the noeira.nn docs ("The
// design in one page") and the fused cross-entropy of the Orthon page
// ("Selected Orthon vs. PyTorch results"): per row,
//   z = W h + b,  loss = logsumexp(z) - z[y],  g = (softmax(z) - onehot(y)) / B,
//   dh = (W^T g) * act'(h),
// and over a tile's rows, in order, the partial sums dW += g h^T, db += g.
// A workgroup of kHeadThreads threads takes kHeadRows rows, kHeadTPR threads
// per row (the narrow-batch tail: 16 rows, 32 threads per row); the row tile
// H sits in LDS with row stride S, W transposed in LDS as Wt[k][16] (classes
// padded to 16 with zeros).
#pragma once
#include "common.hpp"

namespace dl {

constexpr int kHeadThreads = 512;
constexpr int kHeadTPR = 16;                        // threads per row
constexpr int kHeadRows = kHeadThreads / kHeadTPR;  // rows per tile
constexpr int kHeadCMax = 16;
constexpr int kHeadKMax = 256;
constexpr int kHeadMaxSlices = 256;                 // workgroups (dW / db partial slices)
constexpr int kHeadPairs = kHeadKMax * (kHeadCMax / 4) / kHeadThreads;  // (k, 4 classes) per thread

// DPP move of v from the lane CTRL selects within its row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float head_dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Sum over each row of 16 lanes, left in every lane of the row, by DPP
// moves (swap neighbours, swap pairs, mirror each half of 8, mirror the 16)
// instead of LDS-routed shuffles.  Each lane adds the same two operands at
// every step (in swapped order), so all 16 results are bit-identical.
__device__ __forceinline__ float row16_sum(float v) {
  v += head_dpp_mov<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += head_dpp_mov<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += head_dpp_mov<0x141>(v);  // row_half_mirror
  v += head_dpp_mov<0x140>(v);  // row_mirror
  return v;
}

// Sum over the TPR (16 or 32) lanes of a row: with 32, the two rows of 16
// add their sums (each lane the same two operands, so again bit-identical).
template <int TPR>
__device__ __forceinline__ float row_sum(float v) {
  static_assert(TPR == 16 || TPR == 32, "16 or 32 threads per row");
  v = row16_sum(v);
  if (TPR == 32) v += __shfl_xor(v, 16);
  return v;
}

// Row r (thread lr of the row's TPR): the logits from H[r][0..K), the
// row's loss (row_loss[row], written by lane 0 of an active row; NaN for a
// label outside [0, C)), and g = (softmax - onehot) * invB in g[0..C)
// (zeros past C and for an inactive row).  Lanes lr < 4 store g of classes
// 4 lr .. 4 lr + 3 to Ds[r][16].
template <int S, int TPR = kHeadTPR>
__device__ __forceinline__ void head_row_loss(const float* Hs, const float* Wt, const float* bias16,
                                              float* Ds, int r, int lr, int K, int C, int y,
                                              bool active, float invB, float* __restrict__ row_loss,
                                              int64_t row, float (&g)[kHeadCMax]) {
  const bool valid = y >= 0 && y < C;
  float z[kHeadCMax];
#pragma unroll
  for (int c = 0; c < kHeadCMax; ++c) z[c] = 0.f;
#pragma unroll
  for (int kk = 0; kk < kHeadKMax / TPR; ++kk) {
    const int k = lr + kk * TPR;
    if (k >= K) break;
    const float h = Hs[r * S + k];
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
    z[c] = row_sum<TPR>(z[c]);
    z[c] += bias16[c];
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
  if (active && lr == 0) row_loss[row] = valid ? (m + __logf(s)) - zy : __builtin_nanf("");
#pragma unroll
  for (int c = 0; c < kHeadCMax; ++c)
    g[c] = (active && c < C) ? (z[c] * inv_s - (c == y ? 1.0f : 0.0f)) * invB : 0.f;
  if (lr < kHeadCMax / 4) {
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c4 = 0; c4 < kHeadCMax / 4; ++c4)
      if (c4 == lr) x = f32x4{g[4 * c4], g[4 * c4 + 1], g[4 * c4 + 2], g[4 * c4 + 3]};
    *reinterpret_cast<f32x4*>(&Ds[r * kHeadCMax + lr * 4]) = x;
  }
}

// Row r: dh[k] = (sum_c g_c W[c][k]) * act'(H[r][k]) for k < K, into Gs[r][k].
template <int S, int TPR = kHeadTPR>
__device__ __forceinline__ void head_row_dx(const float* Hs, const float* Wt, float* Gs, int r,
                                            int lr, int K, int act, const float (&g)[kHeadCMax]) {
#pragma unroll
  for (int kk = 0; kk < kHeadKMax / TPR; ++kk) {
    const int k = lr + kk * TPR;
    if (k >= K) break;
    float d = 0.f;
#pragma unroll
    for (int c4 = 0; c4 < kHeadCMax / 4; ++c4) {
      const f32x4 w = *reinterpret_cast<const f32x4*>(&Wt[k * kHeadCMax + c4 * 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) d += g[c4 * 4 + e] * w[e];
    }
    Gs[r * S + k] = d * act_deriv(act, Hs[r * S + k]);
  }
}

// The workgroup's dW / db slice: the tile's rows, in order, added to this
// thread's (k, 4 classes) pairs and (threads < C) to db of class tid.
struct HeadSlice {
  int pk[kHeadPairs], pc[kHeadPairs];
  float acc[kHeadPairs][4];
  float db;

  __device__ __forceinline__ void init(int tid, int K) {
#pragma unroll
    for (int j = 0; j < kHeadPairs; ++j) {
      const int p = tid + j * kHeadThreads;
      pk[j] = p % K;
      pc[j] = p < K * (kHeadCMax / 4) ? (p / K) * 4 : -1;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[j][e] = 0.f;
    }
    db = 0.f;
  }
  template <int S, int ROWS = kHeadRows>
  __device__ __forceinline__ void add_tile(const float* Hs, const float* Ds, int tid, int C) {
#pragma unroll
    for (int j = 0; j < kHeadPairs; ++j) {
      if (pc[j] < 0) continue;
      float a0 = acc[j][0], a1 = acc[j][1], a2 = acc[j][2], a3 = acc[j][3];
#pragma unroll 8
      for (int q = 0; q < ROWS; ++q) {
        const float h = Hs[q * S + pk[j]];
        const f32x4 d = *reinterpret_cast<const f32x4*>(&Ds[q * kHeadCMax + pc[j]]);
        a0 += d[0] * h; a1 += d[1] * h; a2 += d[2] * h; a3 += d[3] * h;
      }
      acc[j][0] = a0; acc[j][1] = a1; acc[j][2] = a2; acc[j][3] = a3;
    }
    if (tid < C)
      for (int q = 0; q < ROWS; ++q) db += Ds[q * kHeadCMax + tid];
  }
  // Slice `slice` of dW_part [S][C][K] and db_part [S][C].
  __device__ __forceinline__ void store(float* dW_part, float* db_part, int64_t slice, int tid,
                                        int K, int C) const {
    float* dWp = dW_part + slice * C * K;
#pragma unroll
    for (int j = 0; j < kHeadPairs; ++j) {
      if (pc[j] < 0) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (pc[j] + e < C) dWp[(int64_t)(pc[j] + e) * K + pk[j]] = acc[j][e];
    }
    if (tid < C) db_part[slice * C + tid] = db;
  }
};

// W [C, K] transposed into Wt[k][16] (classes past C and k past K zero), all
// loads of a thread in flight before its LDS stores.
__device__ __forceinline__ void head_load_wt(const float* __restrict__ W, float* Wt, int tid, int K,
                                             int C) {
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

}  // namespace dl

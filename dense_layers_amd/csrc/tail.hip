// The tail of the MLP step in one pass over the rows: the forward of the
// last hidden layer, the narrow classifier head after it (last Linear,
// softmax cross-entropy and its vjp) and the dX of that hidden layer.
//
// The pieces are the LinearAct forward / vjp and the composed backward pass
// of the noeira.nn docs ("The design in one page"), with the cross-entropy
// read once (Orthon page, "Selected Orthon vs. PyTorch results").  For the
// layers h -> n -> C at the end of a network (h, n <= 256, C <= 16) a
// workgroup takes 32 rows of the hidden layer's input Hin and, keeping
// everything in LDS,
//   H   = act1(Hin W1^T + b1)                     (matrix cores)
//   z   = W2 h + b2, loss = logsumexp(z) - z[y], g = (softmax(z) - onehot) / B
//   G1  = (W2^T g) * act1'(H)                     (the head's dX, masked)
//   dH  = (G1 W1) * act0'(Hin)                    (matrix cores)
// and writes only G1 and dH (the inputs of the two weight gradients that
// follow) and the per-row losses; H and the logits never reach HBM.  The
// head's dW2 / db2 leave as per-workgroup slices (rows added in order), which
// the optimizer adds in slice order.
//
// Every product runs in the order of the standalone kernels: each 32x32
// block accumulates its whole contraction in one wave, k ascending in groups
// of 8 (lane half h supplies k = 8 kg + 4 h + s at MFMA step s), and the
// bias, activation and masks are applied with the same operations, so the
// results equal those of the forward GEMM, the head kernel and the dX GEMM
// run one after the other.  A forward wave requests all of its W1 fragments
// (at most 128 registers) when the workgroup starts and keeps them for every
// row tile, so its chain of MFMAs never waits on memory; the dX operand
// streams in chunks, the first requested before the head runs.
#include "head_rows.hpp"

namespace dl {
namespace {

constexpr int kTailThreads = kHeadThreads;  // the head's 16 threads per row of 32
constexpr int kTailRows = kHeadRows;
constexpr int kTailDMax = 256;              // h and n
constexpr int kTailMaxSlices = kHeadMaxSlices;
constexpr int kTS = kTailDMax + 4;  // LDS row stride (floats): 16-byte aligned rows
constexpr int kTailVecs = kTailRows * kTailDMax / 4 / kTailThreads;  // float4 per thread per tile
constexpr int kGroups = kTailDMax / 8;  // k groups of 8 in the longest contraction
constexpr int kChunk = 4;               // k groups per streamed dX operand chunk
static_assert(kTailRows == 32, "one 32x32 MFMA block of rows per tile");

// The thread index made opaque, so that the row / column of each element in
// the copies below is computed where it is used rather than hoisted out of
// the row-tile loop and kept live through every phase.
__device__ __forceinline__ int fresh(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Moves a [nrows x D] row-major block between global memory and an LDS tile
// of row stride kTS (D % 4 == 0, 16-byte aligned rows); rows past nrows are
// filled with zeros on the way in and skipped on the way out.
__device__ __forceinline__ void tile_load(const float* __restrict__ src, int n,
                                          f32x4 (&v)[kTailVecs], int tid) {
  tid = fresh(tid);
#pragma unroll
  for (int j = 0; j < kTailVecs; ++j) {
    const int e = (tid + j * kTailThreads) * 4;
    v[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (e < n) v[j] = *reinterpret_cast<const f32x4*>(src + e);
  }
}
__device__ __forceinline__ void tile_put(float* lds, const f32x4 (&v)[kTailVecs], int D, int tid) {
  tid = fresh(tid);
#pragma unroll
  for (int j = 0; j < kTailVecs; ++j) {
    const int e = (tid + j * kTailThreads) * 4;
    if (e < kTailRows * D) {
      const int q = e / D, k = e - q * D;
      *reinterpret_cast<f32x4*>(lds + q * kTS + k) = v[j];
    }
  }
}
__device__ __forceinline__ void tile_store(const float* lds, float* __restrict__ dst, int n, int D,
                                           int tid) {
  tid = fresh(tid);
#pragma unroll
  for (int j = 0; j < kTailVecs; ++j) {
    const int e = (tid + j * kTailThreads) * 4;
    if (e < n) {
      const int q = e / D, k = e - q * D;
      *reinterpret_cast<f32x4*>(dst + e) = *reinterpret_cast<const f32x4*>(lds + q * kTS + k);
    }
  }
}

// Buffer resource over `bytes` bytes at p: loads past the end return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const float* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p), 0, bytes, 0x00020000);
}

// A fragment of k group kg (row lane % 32 at arow, k = 8 kg + 4 h .. + 3).
__device__ __forceinline__ f32x4 afrag(const float* arow, int kg) {
  return *reinterpret_cast<const f32x4*>(arow + kg * 8);
}

// The 4 MFMAs of one k group: lane half h supplies k = 8 kg + 4 h + s at
// step s of both fragments.
__device__ __forceinline__ void mfma4(f32x16& acc, f32x4 a, f32x4 b) {
#pragma unroll
  for (int s = 0; s < 4; ++s) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[s], b[s], acc, 0, 0, 0);
}

// The dX operand of one 32-column block: W1 read as [N1, K1] (4 loads per k
// group, one per k, consecutive columns across the lanes), streamed in
// chunks of kChunk groups, each requested one chunk ahead.  The per-lane
// offset is fixed and the k offset uniform; groups past the end and columns
// past K1 read zeros (their offset points past the buffer).
struct DxOperand {
  __amdgpu_buffer_rsrc_t res;
  int voff, oob, ldb4, groups;
  f32x4 q0[kChunk], q1[kChunk];

  __device__ __forceinline__ void fetch(f32x4 (&b)[kChunk], int kg0) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      const int kg = kg0 + i;
      const int vo = kg < groups ? voff : oob;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        b[i][t] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(res, vo, (kg * 8 + t) * ldb4, 0));
    }
  }
  // The MFMAs of one chunk; each group's A fragment is read while the
  // previous group's MFMAs run (a holds group kg0's on entry, group
  // kg0 + kChunk's, clamped to the last, on exit).
  __device__ __forceinline__ void chunk(f32x16& acc, const float* arow, const f32x4 (&b)[kChunk],
                                        int kg0, f32x4& a) {
#pragma unroll
    for (int i = 0; i < kChunk; ++i) {
      if (kg0 + i >= groups) break;
      const f32x4 cur = a;
      a = afrag(arow, min(kg0 + i + 1, groups - 1));
      mfma4(acc, cur, b[i]);
    }
  }
  // The whole contraction of a compile-time G groups (G == groups), fully
  // unrolled: no branches between the MFMAs, and each group's A fragment is
  // read into registers of its own while the previous group's MFMAs run.
  // The first chunk was requested with fetch(q0, 0).
  template <int G>
  __device__ __forceinline__ f32x16 run_fixed(const float* arow) {
    static_assert(G % (2 * kChunk) == 0, "whole chunk pairs");
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    f32x4 a = afrag(arow, 0);
#pragma unroll
    for (int c = 0; c < G / kChunk; ++c) {
      f32x4(&cur)[kChunk] = (c & 1) ? q1 : q0;
      f32x4(&nxt)[kChunk] = (c & 1) ? q0 : q1;
      if (c + 1 < G / kChunk) fetch(nxt, (c + 1) * kChunk);
#pragma unroll
      for (int i = 0; i < kChunk; ++i) {
        const int kg = c * kChunk + i;
        const f32x4 an = kg + 1 < G ? afrag(arow, kg + 1) : a;
        mfma4(acc, a, cur[i]);
        a = an;
      }
    }
    return acc;
  }
  // Any group count: the first chunk was requested with fetch(q0, 0).
  __device__ __forceinline__ f32x16 run(const float* arow) {
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    f32x4 a = afrag(arow, 0);
    for (int kg0 = 0; kg0 < groups; kg0 += 2 * kChunk) {
      if (kg0 + kChunk < groups) fetch(q1, kg0 + kChunk);
      chunk(acc, arow, q0, kg0, a);
      if (kg0 + kChunk >= groups) break;
      if (kg0 + 2 * kChunk < groups) fetch(q0, kg0 + 2 * kChunk);
      chunk(acc, arow, q1, kg0 + kChunk, a);
    }
    return acc;
  }
};

// Row of accumulator register r of lane half h in a 32x32 block (the lane's
// column is lane % 32).
__device__ __forceinline__ int acc_row(int r, int h) { return (r >> 2) * 8 + h * 4 + (r & 3); }

// Workgroup b takes row tiles [b tiles_per, (b + 1) tiles_per).  Hin, W1,
// G1, dH 16-byte aligned; K1 (h) and N1 (n) multiples of 8.  KGF / KGX: the
// forward / dX contraction lengths in groups of 8 (K1 / 8, N1 / 8) when
// known at compile time (fully unrolled loops), else 0.
template <bool HAS_DX, int KGF, int KGX>
__global__ void __launch_bounds__(kTailThreads)
mlp_tail_kernel(int64_t B, int K1, int N1, int C, int64_t tiles_per,
                const float* __restrict__ Hin, const float* __restrict__ W1,
                const float* __restrict__ b1, int act1, int act0, const float* __restrict__ W2,
                const float* __restrict__ b2, const int32_t* __restrict__ labels,
                float* __restrict__ row_loss, float* __restrict__ G1, float* __restrict__ dH,
                float* __restrict__ dW_part, float* __restrict__ db_part, float invB,
                const float* dscale) {
  __shared__ __attribute__((aligned(16))) float Xs[kTailRows * kTS];  // Hin, then dH
  __shared__ __attribute__((aligned(16))) float Hs[kTailRows * kTS];  // H
  __shared__ __attribute__((aligned(16))) float Gs[kTailRows * kTS];  // G1
  __shared__ __attribute__((aligned(16))) float Wt[kHeadKMax * kHeadCMax];
  __shared__ __attribute__((aligned(16))) float Ds[kTailRows * kHeadCMax];
  __shared__ float Bc[kHeadCMax];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, h = lane >> 5;
  const int r = tid / kHeadTPR, lr = tid % kHeadTPR;
  const int K = N1;  // the head's input width
  const int w1bytes = N1 * K1 * 4;
  const __amdgpu_buffer_rsrc_t w1res = buffer_of(W1, w1bytes);

  // forward: wave w owns columns 32 w .. 32 w + 31 of H; all of its W1
  // fragments are requested first and kept for every row tile
  const int KG = K1 / 8;
  const bool f_has = wave * 32 < N1;
  const int fcol = wave * 32 + l32;
  constexpr int kBf = KGF > 0 ? KGF : kGroups;
  f32x4 bf[kBf];
  if (f_has) {
    const int vo = fcol < N1 ? (fcol * K1 + 4 * h) * 4 : w1bytes;
#pragma unroll
    for (int kg = 0; kg < kBf; ++kg)
      bf[kg] = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(w1res, kg < KG ? vo : w1bytes, kg * 32, 0));
  }
  const float fbias = (f_has && fcol < N1) ? b1[fcol] : 0.f;
  if (dscale != nullptr) invB *= *dscale;  // loss scale
  head_load_wt(W2, Wt, tid, K, C);
  if (tid < kHeadCMax) Bc[tid] = tid < C ? b2[tid] : 0.f;

  // dX: wave w owns columns 32 w .. 32 w + 31 of dH
  const bool x_has = HAS_DX && wave * 32 < K1;
  const int xcol = wave * 32 + l32;
  DxOperand xo;
  xo.res = w1res;
  xo.oob = w1bytes;
  xo.ldb4 = K1 * 4;
  xo.groups = N1 / 8;
  xo.voff = xcol < K1 ? (4 * h * K1 + xcol) * 4 : w1bytes;

  HeadSlice sl;
  sl.init(tid, K);
  const float* arow_x = Xs + l32 * kTS + 4 * h;
  const float* arow_g = Gs + l32 * kTS + 4 * h;

  const int64_t ntiles = (B + kTailRows - 1) / kTailRows;
  const int64_t t_end = min<int64_t>(ntiles, ((int64_t)blockIdx.x + 1) * tiles_per);
  for (int64_t t = (int64_t)blockIdx.x * tiles_per; t < t_end; ++t) {
    const int64_t r0 = t * kTailRows;
    const int nrows = (int)min<int64_t>(kTailRows, B - r0);
    const bool active = r < nrows;
    const int y = active ? labels[r0 + r] : -1;
    {
      f32x4 v[kTailVecs];
      tile_load(Hin + r0 * K1, nrows * K1, v, tid);
      __syncthreads();  // the previous tile's LDS reads are done
      tile_put(Xs, v, K1, tid);
    }
    __syncthreads();

    // ---- forward of the hidden layer: H = act1(Hin W1^T + b1)
    if (f_has) {
      f32x16 acc;
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[q] = 0.f;
      // each group's A fragment is read while the previous group's MFMAs run
      f32x4 a = afrag(arow_x, 0);
      if (KGF > 0) {
#pragma unroll
        for (int kg = 0; kg < kBf; ++kg) {
          const f32x4 an = kg + 1 < kBf ? afrag(arow_x, kg + 1) : a;
          mfma4(acc, a, bf[kg]);
          a = an;
        }
      } else {
#pragma unroll
        for (int kg = 0; kg < kBf; ++kg)
          if (kg < KG) {
            const f32x4 cur = a;
            a = afrag(arow_x, min(kg + 1, KG - 1));
            mfma4(acc, cur, bf[kg]);
          }
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const float z = acc[q] + fbias;
        Hs[acc_row(q, h) * kTS + fcol] = fcol < N1 ? act_apply(act1, z) : 0.f;
      }
    }
    if (x_has) xo.fetch(xo.q0, 0);
    __syncthreads();

    // ---- head: logits, softmax cross-entropy, g, G1 = (W2^T g) act1'(H)
    {
      float g[kHeadCMax];
      head_row_loss<kTS>(Hs, Wt, Bc, Ds, r, lr, K, C, y, active, invB, row_loss, r0 + r, g);
      head_row_dx<kTS>(Hs, Wt, Gs, r, lr, K, act1, g);
    }
    __syncthreads();

    // this tile's rows, in order, into the workgroup's dW2 / db2 slice
    sl.add_tile<kTS>(Hs, Ds, tid, C);
    tile_store(Gs, G1 + r0 * N1, nrows * N1, N1, tid);

    // ---- dX of the hidden layer: dH = (G1 W1) act0'(Hin), over Hin in LDS
    if (HAS_DX) {
      if (x_has) {
        const f32x16 acc = KGX > 0 ? xo.template run_fixed<KGX>(arow_g) : xo.run(arow_g);
        if (xcol < K1) {
#pragma unroll
          for (int q = 0; q < 16; ++q) {
            float* p = &Xs[acc_row(q, h) * kTS + xcol];
            *p = acc[q] * act_deriv(act0, *p);
          }
        }
      }
      __syncthreads();
      tile_store(Xs, dH + r0 * K1, nrows * K1, K1, tid);
    }
  }

  sl.store(dW_part, db_part, blockIdx.x, tid, K, C);
}

// ---- the narrow-batch form ---------------------------------------------------
// With a small batch the 32-row tiles leave all but a few CUs idle, and each
// wave's product is one chain of dependent 32x32x2 MFMAs (128 of them for a
// 256-long forward), so the step waits on chain latency.  The narrow form
// gives each workgroup one tile of 16 rows (a 64-row batch spreads over 4
// CUs) and runs both products on the 16x16x4 MFMA: H (16 x N1) is N1/16
// blocks and dH (16 x K1) K1/16 blocks over 8 waves, each block a chain of
// half as many MFMAs as a 32-row block, each taking half as long.  Inside a
// block, MFMA step s of k group q takes k = 16 q + 4 g + s from lane group g
// (lanes 16 g .. 16 g + 15), so a lane reads the A operand of 4 steps as one
// float4.  The head runs
// on the same MFMA (logits, the head's dX and its dW slice are 16 x 16 x 16
// products per 16-column block), with the softmax on 16 lanes per row.  The
// sums run in another order than the 32-row form and the standalone kernels
// (the same products, rounded differently).
//
// Optionally the workgroup also finishes the split-K forward of the layer
// before it: Hin = act0(sum of the K-slices in slice order + b0), as the
// finishing kernel of that forward computes it, written out for the weight
// gradient that reads it and kept in LDS.

// Identity or ReLU, the hidden activations of the MLP step, as selects
// rather than branches: the values of act_apply / act_deriv for those two
// (a NaN maps to 0 under ReLU, as there).
__device__ __forceinline__ float relu_or_id(bool relu, float z) {
  return (relu && !(z > 0.0f)) ? 0.0f : z;
}
__device__ __forceinline__ float relu_or_id_deriv(bool relu, float z) {
  return (relu && !(z > 0.0f)) ? 0.0f : 1.0f;
}

// Maximum over each row of 16 lanes, left in every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, head_dpp_mov<0xB1>(v));
  v = fmaxf(v, head_dpp_mov<0x4E>(v));
  v = fmaxf(v, head_dpp_mov<0x141>(v));
  v = fmaxf(v, head_dpp_mov<0x140>(v));
  return v;
}

constexpr int kNarrowRows = 16;
constexpr int kNarrowThreads = kHeadThreads;

template <bool HAS_DX, int K1, int N1>
__global__ void __launch_bounds__(kNarrowThreads)
mlp_tail_narrow_kernel(int64_t B, int C, float* __restrict__ Hin, const float* __restrict__ fold_part,
                       int fold_splits, const float* __restrict__ b0, const float* __restrict__ W1,
                       const float* __restrict__ b1, int act1, int act0,
                       const float* __restrict__ W2, const float* __restrict__ b2,
                       const int32_t* __restrict__ labels, float* __restrict__ row_loss,
                       float* __restrict__ G1, float* __restrict__ dH, float* __restrict__ dW_part,
                       float* __restrict__ db_part, float invB, const float* dscale) {
  static_assert(K1 % 128 == 0 && N1 % 128 == 0 && K1 <= kHeadKMax && N1 <= kHeadKMax,
                "16-column blocks spread evenly over 8 waves");
  constexpr int NBF = N1 / 128;  // forward blocks per wave
  constexpr int NBX = K1 / 128;  // dX blocks per wave
  constexpr int TX = K1 + 4;     // LDS row strides (floats): 16-byte aligned rows
  constexpr int TH = N1 + 4;
  // With N1 = 128 the forward operand (all of W1, 128 KB) is staged in LDS:
  // requested as whole 128-byte lines (a wave reads one row per request),
  // where the MFMA layout read straight from memory would take half a line
  // per row and request, which measured about twice as slow.  The head's
  // arrays reuse that space once the forward is done.
  constexpr bool STAGE = N1 == 128;
  constexpr int TW = K1 + 4;
  constexpr int kHeadFloats = 2 * kNarrowRows * TH + N1 * kHeadCMax + 9 * kNarrowRows * kHeadCMax;
  constexpr int kRegion = STAGE && N1 * TW > kHeadFloats ? N1 * TW : kHeadFloats;
  __shared__ __attribute__((aligned(16))) float pool[kNarrowRows * TX + kRegion];
  float* const Xs = pool;                            // Hin [16][TX]
  float* const W1s = pool + kNarrowRows * TX;        // W1 [N1][TW] (staged forward operand)
  float* const Hs = W1s;                             // H [16][TH], after the forward
  float* const Gs = Hs + kNarrowRows * TH;           // G1 [16][TH]
  float* const Wt = Gs + kNarrowRows * TH;           // W2^T [N1][16]
  float* const Zp = Wt + N1 * kHeadCMax;             // logit parts [8][16][16]
  float* const Gm = Zp + 8 * kNarrowRows * kHeadCMax;  // g [16][16]
  __shared__ float Bc[kHeadCMax];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  // the head's softmax: threads 0..255, one (row, class) each, 16 lanes per row
  const int r = tid >> 4, cls = tid & 15;
  const int64_t r0 = (int64_t)blockIdx.x * kNarrowRows;
  const int nrows = (int)min<int64_t>(kNarrowRows, B - r0);

  const bool relu0 = act0 == ACT_RELU, relu1 = act1 == ACT_RELU;
  if (dscale != nullptr) invB *= *dscale;  // loss scale

  // ---- every load of the prologue is requested before the first is used.
  // Except the forward operand, they go through buffer resources whose
  // range check turns a lane's out-of-range offset into a zero, so no load
  // sits behind a branch (the compiler waits for the loads before a branch).
  // The row tile of Hin first: each thread's float4 groups, or with a fold
  // the K-slices of a group of kFoldGroup (slice s of the rows from r0 on
  // starts s B K1 floats further; rows past the batch and slices past the
  // last read as zeros).
  constexpr int XV = kNarrowRows * K1 / 4 / kNarrowThreads;
  constexpr int kFoldGroup = N1 > 128 ? 4 : 8;  // registers: the forward operand is in flight too
  const int tile_bytes = nrows * K1 * 4;        // from row r0 on
  const int slice_bytes = (int)(B * K1 * 4);
  int vo[XV];  // byte offset of the thread's float4 (tile_bytes: past the batch)
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int f = tid + j * kNarrowThreads;
    const int row = f / (K1 / 4), c = (f % (K1 / 4)) * 4;
    vo[j] = row < nrows ? (row * K1 + c) * 4 : tile_bytes;
  }
  const __amdgpu_buffer_rsrc_t hres =
      fold_splits > 0 ? buffer_of(fold_part + r0 * K1, (fold_splits - 1) * slice_bytes + tile_bytes)
                      : buffer_of(Hin + r0 * K1, tile_bytes);
  f32x4 v[XV];
  f32x4 p[XV][kFoldGroup];
  auto fold_fetch = [&](int s0) {
#pragma unroll
    for (int j = 0; j < XV; ++j)
#pragma unroll
      for (int u = 0; u < kFoldGroup; ++u) {
        const int o = (s0 + u < fold_splits && vo[j] < tile_bytes)
                          ? vo[j] + (s0 + u) * slice_bytes : 0x7ffffff0;
        p[j][u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, o, 0, 0));
      }
  };
  // slice order, as the finishing kernel of the split forward adds them
  auto fold_add = [&](int s0) {
#pragma unroll
    for (int j = 0; j < XV; ++j)
#pragma unroll
      for (int u = 0; u < kFoldGroup; ++u)
        if (s0 + u < fold_splits) v[j] = s0 + u == 0 ? p[j][u] : v[j] + p[j][u];
  };
  if (fold_splits > 0) {
    fold_fetch(0);
  } else {
#pragma unroll
    for (int j = 0; j < XV; ++j)
      v[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, vo[j], 0, 0));
  }
  // the fold's bias b0 at the thread's columns
  float bb[XV][4];
  {
    // (no fold: an empty range over b1, read as zeros and unused)
    const __amdgpu_buffer_rsrc_t b0res =
        fold_splits > 0 ? buffer_of(b0, K1 * 4) : buffer_of(b1, 0);
#pragma unroll
    for (int j = 0; j < XV; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        bb[j][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            b0res, ((tid + j * kNarrowThreads) % (K1 / 4) * 4 + e) * 4, 0, 0));
  }
  // W2 transposed into Wt[k][16] (classes past C zero), b2, the labels
  constexpr int WV = N1 * kHeadCMax / kNarrowThreads;
  float wr[WV];
  {
    const int w2bytes = C * N1 * 4;
    const __amdgpu_buffer_rsrc_t w2res = buffer_of(W2, w2bytes);
#pragma unroll
    for (int j = 0; j < WV; ++j) {
      const int i = tid + j * kNarrowThreads;
      const int k = i / kHeadCMax, c = i % kHeadCMax;
      const int o = c < C ? (c * N1 + k) * 4 : w2bytes;
      wr[j] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(w2res, o, 0, 0));
    }
  }
  const float bc = __uint_as_float(
      __builtin_amdgcn_raw_buffer_load_b32(buffer_of(b2, C * 4), tid * 4, 0, 0));
  const bool active = tid < kNarrowRows * kHeadCMax && r < nrows;
  int y = (int)__builtin_amdgcn_raw_buffer_load_b32(
      buffer_of(reinterpret_cast<const float*>(labels + r0), nrows * 4),
      active ? r * 4 : nrows * 4, 0, 0);
  if (!active) y = -1;

  // The forward operand, requested last: waits are in request order, so the
  // fold and the LDS stores below do not wait for it.  Staged: thread t takes
  // the float4s t + 512 i of W1 (row-major, whole lines per wave).  Else the
  // MFMA layout straight into registers: rows n = 16 (wave + 8 j) + li, the
  // float4 at k = 16 q + 4 lg, each k group used as it arrives.
  constexpr int WL = STAGE ? N1 * K1 / 4 / kNarrowThreads : 1;
  f32x4 wl[WL];
  f32x4 bf[STAGE ? 1 : NBF][STAGE ? 1 : K1 / 16];
  float fb[NBF];
  if (STAGE) {
#pragma unroll
    for (int i = 0; i < WL; ++i)
      wl[i] = *reinterpret_cast<const f32x4*>(W1 + (int64_t)(tid + i * kNarrowThreads) * 4);
  } else {
#pragma unroll
    for (int j = 0; j < NBF; ++j)
#pragma unroll
      for (int q = 0; q < K1 / 16; ++q)
        bf[j][q] = *reinterpret_cast<const f32x4*>(
            W1 + (int64_t)(16 * (wave + 8 * j) + li) * K1 + 16 * q + 4 * lg);
  }
#pragma unroll
  for (int j = 0; j < NBF; ++j) fb[j] = b1[16 * (wave + 8 * j) + li];

  // ---- finish the fold: act0(sum + b0), written out and kept in LDS
  if (fold_splits > 0) {
    fold_add(0);
    for (int s0 = kFoldGroup; s0 < fold_splits; s0 += kFoldGroup) {
      fold_fetch(s0);
      fold_add(s0);
    }
#pragma unroll
    for (int j = 0; j < XV; ++j) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[j][e] = relu_or_id(relu0, v[j][e] + bb[j][e]);
      if (vo[j] < tile_bytes) *reinterpret_cast<f32x4*>(Hin + r0 * K1 + vo[j] / 4) = v[j];
    }
  }
#pragma unroll
  for (int j = 0; j < XV; ++j) {
    const int f = tid + j * kNarrowThreads;
    // rows past the batch hold zeros (a fold's act0(b0) is not kept for them)
    const f32x4 x = vo[j] < tile_bytes ? v[j] : f32x4{0.f, 0.f, 0.f, 0.f};
    *reinterpret_cast<f32x4*>(Xs + (f / (K1 / 4)) * TX + (f % (K1 / 4)) * 4) = x;
  }
  if (STAGE) {
#pragma unroll
    for (int i = 0; i < WL; ++i) {
      const int f = tid + i * kNarrowThreads;
      *reinterpret_cast<f32x4*>(W1s + (f / (K1 / 4)) * TW + (f % (K1 / 4)) * 4) = wl[i];
    }
  }
  __syncthreads();

  // dX operand: W1[n][col] for col = 16 (wave + 8 j) + li and n = 16 q + 4 lg
  // + st.  With N1 = 128 it is requested now and arrives during the forward
  // and the head; with N1 = 256 (128 registers) it waits until the head is
  // done.
  float bx[HAS_DX ? NBX : 1][HAS_DX ? N1 / 16 : 1][4];
  auto load_bx = [&] {
#pragma unroll
    for (int j = 0; j < NBX; ++j)
#pragma unroll
      for (int q = 0; q < N1 / 16; ++q)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          bx[j][q][st] = W1[(int64_t)(16 * q + 4 * lg + st) * K1 + 16 * (wave + 8 * j) + li];
  };
  if (HAS_DX && N1 <= 128) load_bx();

  // ---- forward: H = act1(Hin W1^T + b1), the NBF chains of a wave interleaved
  f32x4 facc[NBF];
#pragma unroll
  for (int j = 0; j < NBF; ++j) facc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int q = 0; q < K1 / 16; ++q) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(Xs + li * TX + 16 * q + 4 * lg);
#pragma unroll
    for (int j = 0; j < NBF; ++j) {
      const f32x4 b = STAGE ? *reinterpret_cast<const f32x4*>(
                                  W1s + (16 * (wave + 8 * j) + li) * TW + 16 * q + 4 * lg)
                            : bf[STAGE ? 0 : j][STAGE ? 0 : q];
#pragma unroll
      for (int st = 0; st < 4; ++st)
        facc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[st], facc[j], 0, 0, 0);
    }
  }
  __syncthreads();  // every wave is done with W1s, whose space the head reuses
#pragma unroll
  for (int j = 0; j < NBF; ++j) {
    const int n = 16 * (wave + 8 * j) + li;
#pragma unroll
    for (int e = 0; e < 4; ++e) Hs[(4 * lg + e) * TH + n] = relu_or_id(relu1, facc[j][e] + fb[j]);
  }
#pragma unroll
  for (int j = 0; j < WV; ++j) Wt[tid + j * kNarrowThreads] = wr[j];
  if (tid < kHeadCMax) Bc[tid] = bc;
  __syncthreads();

  // ---- head on the matrix cores (classes padded to 16 with zero weights).
  // Logits Z = H W2^T: wave w adds k in [16 w, 16 w + 16) (+128 for N1 = 256)
  // into a 16x16 part, and the 8 parts are added in wave order.
  {
    f32x4 zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < N1; kb += 128) {
      const int k0 = kb + 16 * wave + 4 * lg;
      const f32x4 a = *reinterpret_cast<const f32x4*>(Hs + li * TH + k0);
#pragma unroll
      for (int st = 0; st < 4; ++st)
        zacc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], Wt[(k0 + st) * kHeadCMax + li], zacc, 0,
                                                    0, 0);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) Zp[(wave * kNarrowRows + 4 * lg + e) * kHeadCMax + li] = zacc[e];
  }
  __syncthreads();
  // softmax cross-entropy of row r, class cls: loss = logsumexp(z) - z[y],
  // g = (softmax(z) - onehot(y)) / B (zero past C and for rows past the batch)
  if (tid < kNarrowRows * kHeadCMax) {
    float z = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) z += Zp[(w * kNarrowRows + r) * kHeadCMax + cls];
    z += Bc[cls];
    const bool in_c = cls < C;
    const float m = row16_max(in_c ? z : -INFINITY);
    const float ez = in_c ? __expf(z - m) : 0.f;
    const float sum = row16_sum(ez);
    const float zy = row16_sum(cls == y ? z : 0.f);  // one term
    const bool valid = y >= 0 && y < C;
    if (active && cls == 0) row_loss[r0 + r] = valid ? (m + __logf(sum)) - zy : __builtin_nanf("");
    const float inv_s = 1.0f / sum;
    Gm[r * kHeadCMax + cls] = (active && in_c) ? (ez * inv_s - (cls == y ? 1.0f : 0.0f)) * invB : 0.f;
  }
  __syncthreads();
  // G1 = (g W2) act1'(H) and the slice dW2 = g^T H on the wave's forward
  // blocks, db2 = the column sums of g (rows in order)
#pragma unroll
  for (int j = 0; j < NBF; ++j) {
    const int cb = wave + 8 * j;
    const int n = 16 * cb + li;
    const f32x4 a = *reinterpret_cast<const f32x4*>(Gm + li * kHeadCMax + 4 * lg);
    const f32x4 b = *reinterpret_cast<const f32x4*>(Wt + n * kHeadCMax + 4 * lg);
    f32x4 gacc = {0.f, 0.f, 0.f, 0.f}, wacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      gacc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[st], gacc, 0, 0, 0);
      const int row = 4 * lg + st;
      wacc = __builtin_amdgcn_mfma_f32_16x16x4f32(Gm[row * kHeadCMax + li], Hs[row * TH + n], wacc,
                                                  0, 0, 0);
    }
    float* dWp = dW_part + (int64_t)blockIdx.x * C * N1;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int row = 4 * lg + e;  // a row of G1, a class of dW2
      Gs[row * TH + n] = gacc[e] * relu_or_id_deriv(relu1, Hs[row * TH + n]);
      if (row < C) dWp[(int64_t)row * N1 + n] = wacc[e];
    }
  }
  if (tid < C) {
    float db = 0.f;
    for (int q = 0; q < kNarrowRows; ++q) db += Gm[q * kHeadCMax + tid];
    db_part[(int64_t)blockIdx.x * C + tid] = db;
  }
  __syncthreads();
  if (HAS_DX && N1 > 128) load_bx();
  constexpr int GV = kNarrowRows * N1 / 4 / kNarrowThreads;
#pragma unroll
  for (int j = 0; j < GV; ++j) {
    const int f = tid + j * kNarrowThreads;
    const int row = f / (N1 / 4), c = (f % (N1 / 4)) * 4;
    if (row < nrows)
      *reinterpret_cast<f32x4*>(G1 + (r0 + row) * N1 + c) =
          *reinterpret_cast<const f32x4*>(Gs + row * TH + c);
  }

  // ---- dX of the hidden layer: dH = (G1 W1) act0'(Hin)
  if (HAS_DX) {
    f32x4 acc[NBX];
#pragma unroll
    for (int j = 0; j < NBX; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < N1 / 16; ++q) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Gs + li * TH + 16 * q + 4 * lg);
#pragma unroll
      for (int st = 0; st < 4; ++st)
#pragma unroll
        for (int j = 0; j < NBX; ++j)
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], bx[j][q][st], acc[j], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NBX; ++j) {
      const int col = 16 * (wave + 8 * j) + li;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = 4 * lg + e;
        if (row < nrows)
          dH[(r0 + row) * K1 + col] = acc[j][e] * relu_or_id_deriv(relu0, Xs[row * TX + col]);
      }
    }
  }
}

// ---- the small-batch forward before the narrow tail ---------------------------
// K-slices of Y = X W^T (no bias or activation: the narrow tail adds the
// slices in order and applies them) for a batch of a few 16-row tiles and a
// long contraction: workgroup (row tile, 64-column block, slice) stages its
// 16 rows of X and 64 rows of W over the slice's k range in LDS (whole-line
// loads, rows past the batch or N and k past K read as zero) and its 4 waves
// each run one 16x16 block on the 16x16x4 MFMA, k = 16 q + 4 g + s as in the
// narrow tail.  Slice s covers k in [s kps, min(K, (s + 1) kps)) and goes to
// slices[s][B][N].
constexpr int kFwdNarrowCols = 64;
constexpr int kFwdNarrowMaxK = 256;

__global__ void __launch_bounds__(256)
mlp_fwd_narrow_kernel(int B, int K, int N, int kps, const float* __restrict__ X,
                      const float* __restrict__ W, float* __restrict__ slices) {
  constexpr int TS = kFwdNarrowMaxK + 4;  // LDS row stride (floats)
  __shared__ __attribute__((aligned(16))) float Xs[kNarrowRows * TS];
  __shared__ __attribute__((aligned(16))) float Ws[kFwdNarrowCols * TS];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 15, lg = lane >> 4;
  const int tiles_r = (B + kNarrowRows - 1) / kNarrowRows;
  const int tiles_c = (N + kFwdNarrowCols - 1) / kFwdNarrowCols;
  const int bid = blockIdx.x;
  const int sl = bid / (tiles_r * tiles_c);
  const int rc = bid % (tiles_r * tiles_c);
  const int r0 = (rc % tiles_r) * kNarrowRows, c0 = (rc / tiles_r) * kFwdNarrowCols;
  const int k0 = sl * kps;
  const int kn = min(K, k0 + kps) - k0;  // k in this slice (> 0)
  const int kv = kps / 4;                 // float4 per staged row

  // stage the 16 rows of X and 64 of W: every load issued before the first
  // store, through buffer resources whose range check reads an out-of-range
  // lane as zero (no load behind a branch)
  constexpr int kXV = kNarrowRows * kFwdNarrowMaxK / 4 / 256;
  constexpr int kWV = kFwdNarrowCols * kFwdNarrowMaxK / 4 / 256;
  const int xbytes = B * K * 4, wbytes = N * K * 4;
  const __amdgpu_buffer_rsrc_t xres = buffer_of(X, xbytes), wres = buffer_of(W, wbytes);
  f32x4 xv[kXV], wv[kWV];
  auto offset = [&](int f, int rows, int g0, int glim, int oob) {
    const int row = f / kv, c = (f % kv) * 4;
    return (f < rows * kv && c < kn && g0 + row < glim) ? ((g0 + row) * K + k0 + c) * 4 : oob;
  };
#pragma unroll
  for (int j = 0; j < kXV; ++j)
    xv[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          xres, offset(tid + j * 256, kNarrowRows, r0, B, xbytes), 0, 0));
#pragma unroll
  for (int j = 0; j < kWV; ++j)
    wv[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                          wres, offset(tid + j * 256, kFwdNarrowCols, c0, N, wbytes), 0, 0));
#pragma unroll
  for (int j = 0; j < kXV; ++j) {
    const int f = tid + j * 256;
    if (f < kNarrowRows * kv) *reinterpret_cast<f32x4*>(Xs + (f / kv) * TS + (f % kv) * 4) = xv[j];
  }
#pragma unroll
  for (int j = 0; j < kWV; ++j) {
    const int f = tid + j * 256;
    if (f < kFwdNarrowCols * kv) *reinterpret_cast<f32x4*>(Ws + (f / kv) * TS + (f % kv) * 4) = wv[j];
  }
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const float* xa = Xs + li * TS + 4 * lg;
  const float* wb = Ws + (16 * wave + li) * TS + 4 * lg;
  for (int q = 0; q < kps / 16; ++q) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(xa + 16 * q);
    const f32x4 b = *reinterpret_cast<const f32x4*>(wb + 16 * q);
#pragma unroll
    for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[st], b[st], acc, 0, 0, 0);
  }
  const int col = c0 + 16 * wave + li;
  float* out = slices + (int64_t)sl * B * N;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = r0 + 4 * lg + e;
    if (row < B && col < N) out[(int64_t)row * N + col] = acc[e];
  }
}

}  // namespace

bool mlp_tail_fits(int64_t K1, int64_t N1, int64_t C) {
  return C >= 1 && C <= kHeadCMax && K1 >= 8 && K1 <= kTailDMax && K1 % 8 == 0 && N1 >= 8 &&
         N1 <= kTailDMax && N1 % 8 == 0;
}

hipError_t launch_mlp_tail(int64_t B, int K1, int N1, int C, const float* Hin, const float* W1,
                           const float* b1, int act1, int act0, const float* W2, const float* b2,
                           const int32_t* labels, float* row_loss, float* G1, float* dH,
                           float* dW_part, float* db_part, hipStream_t s, const float* dscale) {
  if (!mlp_tail_fits(K1, N1, C) || B < 1) return hipErrorInvalidValue;
  const uintptr_t al = reinterpret_cast<uintptr_t>(Hin) | reinterpret_cast<uintptr_t>(W1) |
                       reinterpret_cast<uintptr_t>(G1) | reinterpret_cast<uintptr_t>(dH);
  if ((al & 15) != 0) return hipErrorNotSupported;
  // the head kernel's slicing (32-row tiles, at most 256 slices), so the
  // optimizer finds head_xent_slices(B) slices either way
  const int64_t ntiles = (B + kTailRows - 1) / kTailRows;
  const int64_t per = (ntiles + kTailMaxSlices - 1) / kTailMaxSlices;
  const int64_t blocks = (ntiles + per - 1) / per;
  const float invB = (float)(1.0 / (double)B);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(kTailThreads), 0, s, B, K1, N1, C, per,
                       Hin, W1, b1, act1, act0, W2, b2, labels, row_loss, G1, dH, dW_part, db_part,
                       invB, dscale);
  };
  // the MLP shapes with a 256-wide hidden input get fully unrolled loops
  const bool fixed = K1 == 256 && (N1 == 128 || N1 == 256);
  if (dH != nullptr) {
    if (fixed && N1 == 128) go(mlp_tail_kernel<true, 32, 16>);
    else if (fixed) go(mlp_tail_kernel<true, 32, 32>);
    else go(mlp_tail_kernel<true, 0, 0>);
  } else {
    if (fixed && N1 == 128) go(mlp_tail_kernel<false, 32, 16>);
    else if (fixed) go(mlp_tail_kernel<false, 32, 32>);
    else go(mlp_tail_kernel<false, 0, 0>);
  }
  return hipGetLastError();
}

// Up to this batch the narrow form is the faster one (measured at 8192 rows
// through the 256 -> 128 layer: 24 us against 30 us for the 32-row form,
// whose workgroups load W1 once for several tiles); its head leaves one
// dW / db slice per 16 rows.
constexpr int64_t kNarrowMaxRows = 8192;

bool mlp_tail_narrow_fits(int64_t B, int64_t K1, int64_t N1, int64_t C) {
  return mlp_tail_fits(K1, N1, C) && K1 == 256 && (N1 == 128 || N1 == 256) && B >= 1 &&
         B <= kNarrowMaxRows;
}

int64_t mlp_tail_narrow_slices(int64_t B) { return (B + kNarrowRows - 1) / kNarrowRows; }

bool mlp_fwd_narrow_fits(int64_t B, int64_t K, int64_t N, int kps) {
  // byte offsets of X and W in 31 bits (buffer loads)
  return B >= 1 && B <= 4096 && N >= 1 && K % 4 == 0 && kps % 16 == 0 && kps > 0 &&
         kps <= kFwdNarrowMaxK && B * K * 4 < (int64_t)1 << 31 && N * K * 4 < (int64_t)1 << 31;
}

hipError_t launch_mlp_fwd_narrow(int B, int K, int N, int splits, int kps, const float* X,
                                 const float* W, float* slices, hipStream_t s) {
  if (!mlp_fwd_narrow_fits(B, K, N, kps) || splits < 1 || (int64_t)(splits - 1) * kps >= K ||
      (int64_t)splits * kps < K)
    return hipErrorInvalidValue;
  if (((reinterpret_cast<uintptr_t>(X) | reinterpret_cast<uintptr_t>(W)) & 15) != 0)
    return hipErrorNotSupported;
  const int64_t blocks = (int64_t)((B + kNarrowRows - 1) / kNarrowRows) *
                         ((N + kFwdNarrowCols - 1) / kFwdNarrowCols) * splits;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mlp_fwd_narrow_kernel, dim3((unsigned)blocks), dim3(256), 0, s, B, K, N, kps,
                     X, W, slices);
  return hipGetLastError();
}

hipError_t launch_mlp_tail_narrow(int64_t B, int K1, int N1, int C, float* Hin,
                                  const float* fold_part, int fold_splits, const float* b0,
                                  const float* W1, const float* b1, int act1, int act0,
                                  const float* W2, const float* b2, const int32_t* labels,
                                  float* row_loss, float* G1, float* dH, float* dW_part,
                                  float* db_part, hipStream_t s, const float* dscale) {
  auto hidden_act = [](int a) { return a == ACT_IDENTITY || a == ACT_RELU; };
  if (!mlp_tail_narrow_fits(B, K1, N1, C) || fold_splits < 0 ||
      (fold_splits > 0 && (fold_part == nullptr || b0 == nullptr)) || !hidden_act(act0) ||
      !hidden_act(act1))
    return hipErrorInvalidValue;
  const uintptr_t al = reinterpret_cast<uintptr_t>(Hin) | reinterpret_cast<uintptr_t>(W1) |
                       reinterpret_cast<uintptr_t>(G1) | reinterpret_cast<uintptr_t>(fold_part);
  if ((al & 15) != 0) return hipErrorNotSupported;
  const float invB = (float)(1.0 / (double)B);
  auto go = [&](auto kern) {
    hipLaunchKernelGGL(kern, dim3((unsigned)mlp_tail_narrow_slices(B)), dim3(kNarrowThreads), 0, s,
                       B, C, Hin, fold_part, fold_splits, b0, W1, b1, act1, act0, W2, b2, labels,
                       row_loss, G1, dH, dW_part, db_part, invB, dscale);
  };
  if (dH != nullptr) {
    if (N1 == 128) go(mlp_tail_narrow_kernel<true, 256, 128>);
    else go(mlp_tail_narrow_kernel<true, 256, 256>);
  } else {
    if (N1 == 128) go(mlp_tail_narrow_kernel<false, 256, 128>);
    else go(mlp_tail_narrow_kernel<false, 256, 256>);
  }
  return hipGetLastError();
}

}  // namespace dl

// Shared device-side helpers for the gfx950 kernels: vector types, bf16
// conversion, activations and the launch descriptors used between the C ABI
// layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dl {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // storage type of one bfloat16

enum Act { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };
enum Layout { K_MAJOR = 0, MN_MAJOR = 1 };
enum Epi { EPI_FWD = 0, EPI_DX = 1, EPI_DW = 2 };

// ---- bf16 <-> f32 -----------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even; NaN stays NaN (quietened).  bf16 is the upper half
// of an IEEE float32, so rounding adds half an ulp of the lower half plus the
// parity of the kept part and truncates.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<bf16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<bf16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};

// ---- activations ------------------------------------------------------------
// GELU (tanh form): 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3).
// tanh(u) = 1 - 2 / (1 + exp(2u)); exp saturates to 0 or inf for large |u|,
// which yields exactly -1 or 1, so no range reduction is needed here.

constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCubic = 0.044715f;

__device__ __forceinline__ float tanh_from_exp(float u) {
  float e = __expf(2.0f * u);
  return 1.0f - 2.0f / (1.0f + e);
}

__device__ __forceinline__ float act_apply(int act, float z) {
  if (act == ACT_RELU) return z > 0.0f ? z : 0.0f;
  if (act == ACT_GELU_TANH) {
    float t = tanh_from_exp(kSqrt2OverPi * (z + kGeluCubic * z * z * z));
    return 0.5f * z * (1.0f + t);
  }
  return z;
}

// Derivative of act at pre-activation z.  For ReLU the saved value may be Y
// instead of Z: Y > 0 exactly when Z > 0.
__device__ __forceinline__ float act_deriv(int act, float z) {
  if (act == ACT_RELU) return z > 0.0f ? 1.0f : 0.0f;
  if (act == ACT_GELU_TANH) {
    float z2 = z * z;
    float t = tanh_from_exp(kSqrt2OverPi * (z + kGeluCubic * z2 * z));
    float du = kSqrt2OverPi * (1.0f + 3.0f * kGeluCubic * z2);
    return 0.5f * (1.0f + t) + 0.5f * z * (1.0f - t * t) * du;
  }
  return 1.0f;
}

// ---- workgroup -> tile mapping ------------------------------------------------
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Remap so every XCD receives a contiguous run of tiles,
// then walk the tiles in bands of 8 tile-rows so that neighbouring workgroups
// share A rows and B columns in L2.  Returns (split, tm, tn).
__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& split,
                                            int& tm, int& tn) {
  const int nwg = gridDim.x;
  int id = blockIdx.x;
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  const int ntiles = tiles_m * tiles_n;
  split = id / ntiles;
  const int tile = id - split * ntiles;
  constexpr int GROUP = 8;
  const int band = tile / (GROUP * tiles_n);
  const int first_m = band * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int in_band = tile - band * GROUP * tiles_n;
  tm = first_m + in_band % gsz;
  tn = in_band / gsz;
}

// ---- GEMM launch descriptor ---------------------------------------------
// C[M, N] = A[M, K] * B[K, N] with
//   A K_MAJOR : element (m, k) at A[m * lda + k]     (rows of A contiguous in k)
//   A MN_MAJOR: element (m, k) at A[k * lda + m]
//   B K_MAJOR : element (k, n) at B[n * ldb + k]
//   B MN_MAJOR: element (k, n) at B[k * ldb + n]
// and an epilogue:
//   EPI_FWD: z = acc + bias[n]; C = act(z); Z[m, n] = z if Z != null
//   EPI_DX : C = acc * act'(mask_src[m, n]) (act' = 1 for identity)
//   EPI_DW : C (float) = acc; db[m] = sum_k A(m, k) when db != null.
//            With split-K (splits > 1) slice s writes partial[s][M][N] and
//            db_partial[s][M]; a reduce kernel finishes both.
struct GemmDesc {
  int M, N, K;
  const void* A; int64_t lda; int a_layout;
  const void* B; int64_t ldb; int b_layout;
  void* C; int64_t ldc;
  int epi;
  const float* bias; int act; void* Z;
  int mask_act; const void* mask_src;
  float* db;
  int splits; int k_per_split;
  float* partial; float* db_partial;
};

// Host-side launchers (defined in the kernel files).
hipError_t launch_gemm_f32(const GemmDesc& d, int tile, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmDesc& d, int tile, hipStream_t s);
hipError_t launch_splitk_reduce(int M, int N, int splits, const float* partial,
                                const float* db_partial, float* C, int64_t ldc,
                                float* db, hipStream_t s);
hipError_t launch_act_mask(int dtype, int act, int64_t rows, int64_t cols,
                           const void* dY, const void* saved, void* G,
                           hipStream_t s);
hipError_t launch_cast_bf16(int64_t n, const float* src, bf16_t* dst,
                            hipStream_t s);
hipError_t launch_xent(int64_t B, int64_t C, const float* logits,
                       const int32_t* labels, float* row_loss, float* dlogits,
                       float* loss, hipStream_t s);
// Optimizer constants, each formed in double on the host and rounded once.
struct OptConsts {
  float lr;            // SGD step
  float decay;         // 1 - lr wd
  float b1, omb1;      // beta1, 1 - beta1
  float b2, omb2;      // beta2, 1 - beta2
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
};
hipError_t launch_sgd(int64_t n, float* w, const float* g, const OptConsts& c,
                      hipStream_t s);
hipError_t launch_adamw(int64_t n, float* w, const float* g, float* m, float* v,
                        const OptConsts& c, hipStream_t s);

constexpr int kMaxSegs = 32;
// Multi-tensor optimizer: one launch updates up to kMaxSegs arrays.  The
// gradient of segment k is g[k] when splits[k] <= 1; otherwise it is the
// split-K partial sum  sum_s part[k][s * part_stride[k] + i]  (added in slice
// order), which is also stored to g_out[k] -- the optimizer finishes the
// weight-gradient reduction instead of a separate pass.
struct OptSegs {
  int count;
  int64_t start_block[kMaxSegs + 1];  // prefix sums of blocks per segment
  int64_t n[kMaxSegs];
  float* w[kMaxSegs];
  const float* g[kMaxSegs];
  float* m[kMaxSegs];
  float* v[kMaxSegs];
  const float* part[kMaxSegs];
  int64_t part_stride[kMaxSegs];
  int splits[kMaxSegs];
  float* g_out[kMaxSegs];
};
constexpr int kOptBlock = 256;
constexpr int kOptElemsPerBlock = kOptBlock * 4 * 4;  // 4 float4 per thread
hipError_t launch_opt_multi(const OptSegs& segs, int kind, const OptConsts& c,
                            hipStream_t s);

}  // namespace dl

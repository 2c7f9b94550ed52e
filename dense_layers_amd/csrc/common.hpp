// Shared device-side helpers for the gfx950 kernels: vector types, bf16
// conversion, activations and the launch descriptors used between the C ABI
// layer (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace dl {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint16_t bf16_t;  // storage type of one bfloat16
typedef _Float16 f16_t;   // storage type of one IEEE half
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

enum Act { ACT_IDENTITY = 0, ACT_RELU = 1, ACT_GELU_TANH = 2 };
enum Layout { K_MAJOR = 0, MN_MAJOR = 1 };
enum Epi { EPI_FWD = 0, EPI_DX = 1, EPI_DW = 2 };

// ---- bf16 <-> f32 -----------------------------------------------------------

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// Round-to-nearest-even (the hardware conversion, v_cvt_pk_bf16_f32); NaN
// stays NaN.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// Two floats to a packed pair of bf16 (low half = a), one conversion.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
  const f2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf2));
}

// ---- half (fp16) <-> f32 ------------------------------------------------------
// The mixed-precision input convention of the MuNet page ("Configuration"):
// nearest-even rounding, clamped to +-65504 instead of overflowing to
// infinity, NaN kept.  Clamping first gives the saturation (values past
// 65504 would otherwise round to 65504 or to infinity); NaN skips the clamp.
__device__ __forceinline__ float f16_sat(float f) {
  return __builtin_isnan(f) ? f : fminf(fmaxf(f, -65504.f), 65504.f);
}
__device__ __forceinline__ f16_t f32_to_f16(float f) { return (f16_t)f16_sat(f); }
__device__ __forceinline__ float f16_to_f32(f16_t h) { return (float)h; }
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const f2 v = {f16_sat(a), f16_sat(b)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
}

// The two 16-bit operand formats of the matrix-core GEMMs, both moved as
// 16-bit words: the float32 view of one word, the packing of two floats, and
// the 32x32x16 MFMA of eight-element fragments.
enum HalfKind { HK_BF16 = 0, HK_F16 = 1 };
template <int HK> struct HalfOps;
template <> struct HalfOps<HK_BF16> {
  using T = bf16_t;
  __device__ static __forceinline__ float to_f32(uint32_t w) { return __uint_as_float(w << 16); }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) { return pack_bf16x2(a, b); }
  __device__ static __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ float elem(bf16x8 a, int e) { return static_cast<float>(a[e]); }
  __device__ static __forceinline__ uint16_t one(float x) { return f32_to_bf16(x); }
};
template <> struct HalfOps<HK_F16> {
  using T = f16_t;
  __device__ static __forceinline__ float to_f32(uint32_t w) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)w);
  }
  __device__ static __forceinline__ uint32_t pack2(float a, float b) { return pack_f16x2(a, b); }
  __device__ static __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  __device__ static __forceinline__ float elem(bf16x8 a, int e) {
    return static_cast<float>(__builtin_bit_cast(f16x8, a)[e]);
  }
  __device__ static __forceinline__ uint16_t one(float x) {
    return __builtin_bit_cast(uint16_t, f32_to_f16(x));
  }
};

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static __forceinline__ float load(const float* p, int64_t i) { return p[i]; }
  __device__ static __forceinline__ void store(float* p, int64_t i, float v) { p[i] = v; }
};
template <> struct Elem<bf16_t> {
  __device__ static __forceinline__ float load(const bf16_t* p, int64_t i) { return bf16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(bf16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }
};
template <> struct Elem<f16_t> {
  __device__ static __forceinline__ float load(const f16_t* p, int64_t i) { return f16_to_f32(p[i]); }
  __device__ static __forceinline__ void store(f16_t* p, int64_t i, float v) { p[i] = f32_to_f16(v); }
};

// ---- activations ------------------------------------------------------------
// GELU (tanh form): 0.5 z (1 + tanh(u)), u = sqrt(2/pi) (z + 0.044715 z^3).
// With r = 1 / (1 + exp(2u)):  tanh(u) = 1 - 2r, so
//   gelu(z)  = z (1 - r)
//   gelu'(z) = 0.5 (1 + t) + 0.5 z (1 - t^2) u'   (t = tanh u, u' = du/dz)
//            = (1 - r) (1 + 2 z r u'),   u' = sqrt(2/pi) (1 + 3 * 0.044715 z^2).
// exp(2u) is one hardware exp2 of 2u log2(e); it saturates to 0 or +inf for
// large |u|, giving r = 1 or 0 and the exact limits, so no range reduction is
// needed.  The reciprocal is the hardware one (about 1 ulp), well inside the
// float32 tolerance of the results.

// 2u log2(e) = z (kX0 + kX2 z^2) and 2u' = kD0 + kD2 z^2, each constant
// formed in double and rounded once, so that each polynomial is one fused
// multiply-add.
constexpr double kSqrt2OverPi = 0.7978845608028654;
constexpr double kGeluCubic = 0.044715;
constexpr double kTwoLog2e = 2.8853900817779268;  // 2 / ln 2
constexpr float kX0 = (float)(kTwoLog2e * kSqrt2OverPi);
constexpr float kX2 = (float)(kTwoLog2e * kSqrt2OverPi * kGeluCubic);
constexpr float kD0 = (float)(2.0 * kSqrt2OverPi);
constexpr float kD2 = (float)(2.0 * kSqrt2OverPi * 3.0 * kGeluCubic);

__device__ __forceinline__ float gelu_r(float z, float z2) {
  const float x = z * fmaf(kX2, z2, kX0);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x));
}

__device__ __forceinline__ float act_apply(int act, float z) {
  if (act == ACT_RELU) return z > 0.0f ? z : 0.0f;
  if (act == ACT_GELU_TANH) return fmaf(-z, gelu_r(z, z * z), z);
  return z;
}

// Derivative of act at pre-activation z.  For ReLU the saved value may be Y
// instead of Z: Y > 0 exactly when Z > 0.
__device__ __forceinline__ float act_deriv(int act, float z) {
  if (act == ACT_RELU) return z > 0.0f ? 1.0f : 0.0f;
  if (act == ACT_GELU_TANH) {
    const float z2 = z * z;
    const float r = gelu_r(z, z2);
    const float t = z * fmaf(kD2, z2, kD0);  // 2 z u'
    return (1.0f - r) * fmaf(t, r, 1.0f);
  }
  return 1.0f;
}

// ---- workgroup -> tile mapping ------------------------------------------------
// Consecutive workgroup ids are dispatched round-robin over the 8 XCDs, each
// with its own L2.  Remap so every XCD receives a contiguous run of tiles,
// then walk the tiles in bands of 8 tile-rows so that neighbouring workgroups
// share A rows and B columns in L2.  Returns (split, tm, tn).
// Position `id` in that band order -> (split, tm, tn).
__device__ __forceinline__ void band_coords(int id, int tiles_m, int tiles_n, int& split, int& tm,
                                            int& tn) {
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

// Workgroup `id` of `nwg` working on one product -> (split, tm, tn).
__device__ __forceinline__ void tile_coords_at(int id, int nwg, int tiles_m, int tiles_n,
                                               int& split, int& tm, int& tn) {
  if ((nwg & 7) == 0) id = (id & 7) * (nwg >> 3) + (id >> 3);
  band_coords(id, tiles_m, tiles_n, split, tm, tn);
}

__device__ __forceinline__ void tile_coords(int tiles_m, int tiles_n, int& split,
                                            int& tm, int& tn) {
  tile_coords_at(blockIdx.x, gridDim.x, tiles_m, tiles_n, split, tm, tn);
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
  int half_kind;  // 16-bit operands: HK_BF16 or HK_F16
  // weight-gradient products (dW, db) whose gradient operand was handed over
  // times s (device float32 [1], a power of two): the float32 results are
  // divided by s before they are stored.  dX products keep the scale (dX is
  // the next layer's gradient operand).  Null: no scale.
  const float* out_scale;
  // Fused classifier head over many classes (float32 kernels only).
  // Forward: with xent_part set, the epilogue also leaves, for every output
  // row and column tile tn, the tile's (max z, sum exp(z - max)) over its
  // columns as two floats at xent_part[2 (tn M + row)].
  float* xent_part;
  // dX / dW of the head: with xent_rows set, the A operand holds the logits
  // [rows, C] and becomes the loss gradient
  //   g = 2^(z log2 e - o_i) - [class == y_i] xent_invB  (= exp(z - lse_i) / B - ...)
  // as it is staged into LDS (rows are batch rows, classes the head's
  // outputs; elements past the operand's K range stay zero).  xent_rows
  // holds one 8-byte record per batch row i: the exponent offset
  // o_i = lse_i log2 e + log2 B, and the label y_i (its int32 bits).
  const float* xent_rows;
  float xent_invB;
  // Weight gradient with one K slice: with sgd_w set, the epilogue also
  // takes the SGD step on the parameters at the same places,
  // sgd_w[m][n] -= sgd_lr dW[m][n] (sgd_w with leading dimension ldc), and
  // with sgd_b set, sgd_b[m] -= sgd_lr db[m], as the optimizer kernel would
  // from the stored dW and db.
  float* sgd_w;
  float* sgd_b;
  float sgd_lr;
};

// 1 / s of a descriptor's gradient-operand scale (1 without one).
__device__ __forceinline__ float unscale_factor(const GemmDesc& d) {
  return d.out_scale != nullptr ? 1.0f / d.out_scale[0] : 1.0f;
}

// ---- GEMM epilogue through LDS ------------------------------------------------
// The 32x32 MFMA result leaves each lane one column of 16 rows, so direct
// stores would be 2- or 4-byte scatters.  Instead the whole BM x BN tile is
// staged as float32 in LDS, then the workgroup streams it out
// row-contiguously: 4 outputs per thread (8-byte bf16 or 16-byte float32
// stores), with the bias, activation, derivative mask and bf16 rounding
// applied on the way.  `stage` must hold stage_floats<BM, BN, WGM>() floats
// and may alias the K-loop buffers (the caller has passed a barrier after
// its last LDS read).
//   out_vec: C (and Z / mask_src) allow aligned 4-wide access (pointer and
//   leading dimension), checked by the launcher.

template <typename T> struct Store4;
template <> struct Store4<float> {
  __device__ static __forceinline__ void vec(float* p, const float v[4]) {
    f32x4 x = {v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(p) = x;
  }
  __device__ static __forceinline__ void load_vec(const float* p, float v[4]) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(p);
    v[0] = x[0]; v[1] = x[1]; v[2] = x[2]; v[3] = x[3];
  }
};
template <> struct Store4<bf16_t> {
  __device__ static __forceinline__ void vec(bf16_t* p, const float v[4]) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    u32x2v x = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    *reinterpret_cast<u32x2v*>(p) = x;
  }
  __device__ static __forceinline__ void load_vec(const bf16_t* p, float v[4]) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v x = *reinterpret_cast<const u32x2v*>(p);
    v[0] = __uint_as_float(x[0] << 16); v[1] = __uint_as_float(x[0] & 0xffff0000u);
    v[2] = __uint_as_float(x[1] << 16); v[3] = __uint_as_float(x[1] & 0xffff0000u);
  }
};

template <> struct Store4<f16_t> {
  __device__ static __forceinline__ void vec(f16_t* p, const float v[4]) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    u32x2v x = {pack_f16x2(v[0], v[1]), pack_f16x2(v[2], v[3])};
    *reinterpret_cast<u32x2v*>(p) = x;
  }
  __device__ static __forceinline__ void load_vec(const f16_t* p, float v[4]) {
    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
    const u32x2v x = *reinterpret_cast<const u32x2v*>(p);
    v[0] = HalfOps<HK_F16>::to_f32(x[0] & 0xffffu); v[1] = HalfOps<HK_F16>::to_f32(x[0] >> 16);
    v[2] = HalfOps<HK_F16>::to_f32(x[1] & 0xffffu); v[3] = HalfOps<HK_F16>::to_f32(x[1] >> 16);
  }
};

// Four consecutive elements kept in their storage format (one 16-byte or
// 8-byte register group) until they are used.
template <typename T> struct Raw4;
template <> struct Raw4<float> {
  f32x4 v = {0.f, 0.f, 0.f, 0.f};
  __device__ __forceinline__ void load_vec(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ void set(int e, float x) { v[e] = x; }
  __device__ __forceinline__ float get(int e) const { return v[e]; }
};
template <> struct Raw4<bf16_t> {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v v = {0u, 0u};
  __device__ __forceinline__ void load_vec(const bf16_t* p) { v = *reinterpret_cast<const u32x2v*>(p); }
  __device__ __forceinline__ void set(int e, float x) {
    const uint32_t h = f32_to_bf16(x);
    v[e >> 1] = (e & 1) ? ((v[e >> 1] & 0xffffu) | (h << 16)) : ((v[e >> 1] & 0xffff0000u) | h);
  }
  __device__ __forceinline__ float get(int e) const {
    return (e & 1) ? __uint_as_float(v[e >> 1] & 0xffff0000u) : __uint_as_float(v[e >> 1] << 16);
  }
};
template <> struct Raw4<f16_t> {
  typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
  u32x2v v = {0u, 0u};
  __device__ __forceinline__ void load_vec(const f16_t* p) { v = *reinterpret_cast<const u32x2v*>(p); }
  __device__ __forceinline__ void set(int e, float x) {
    const uint32_t h = __builtin_bit_cast(uint16_t, f32_to_f16(x));
    v[e >> 1] = (e & 1) ? ((v[e >> 1] & 0xffffu) | (h << 16)) : ((v[e >> 1] & 0xffff0000u) | h);
  }
  __device__ __forceinline__ float get(int e) const {
    return HalfOps<HK_F16>::to_f32((e & 1) ? v[e >> 1] >> 16 : v[e >> 1] & 0xffffu);
  }
};

// Max / sum over groups of N consecutive lanes (N = 16 or 32), left in every
// lane of the group: DPP moves within each row of 16 lanes (swap neighbours,
// swap pairs, mirror each half of 8, mirror the 16), then for N = 32 one
// exchange with the other row.  Each step combines the same two values in
// every lane (in swapped order), so all lanes of a group end bit-identical.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, true));
}
template <int N>
__device__ __forceinline__ float lanes_max(float v) {
  static_assert(N == 16 || N == 32, "groups of 16 or 32 lanes");
  v = fmaxf(v, dpp_mov<0xB1>(v));
  v = fmaxf(v, dpp_mov<0x4E>(v));
  v = fmaxf(v, dpp_mov<0x141>(v));
  v = fmaxf(v, dpp_mov<0x140>(v));
  if (N == 32) v = fmaxf(v, __shfl_xor(v, 16));
  return v;
}
template <int N>
__device__ __forceinline__ float lanes_sum(float v) {
  static_assert(N == 16 || N == 32, "groups of 16 or 32 lanes");
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  if (N == 32) v += __shfl_xor(v, 16);
  return v;
}

// A tile whose float32 staging copy exceeds kStageBudget bytes is staged in
// WGM passes of BM / WGM rows (the rows of one row of waves each).
constexpr int kStageBudget = 80 * 1024;
// LDS of one CU (and the most one workgroup may allocate).
constexpr int kLdsBytes = 160 * 1024;
template <int BM, int BN, int WGM>
constexpr int stage_passes() { return BM * (BN + 4) * 4 <= kStageBudget ? 1 : WGM; }
template <int BM, int BN, int WGM>
constexpr int stage_floats() { return BM / stage_passes<BM, BN, WGM>() * (BN + 4); }

// Rows handled per thread in one staging pass, and the load of the dX
// epilogue's saved activations for one pass (kept in their storage format).
template <int BM, int BN, int WGM, int WGN>
struct EpiShape {
  static constexpr int NT = WGM * WGN * 64;
  static constexpr int CPR = BN / 4;  // 4-wide chunks per tile row
  static constexpr int PASSES = stage_passes<BM, BN, WGM>();
  static constexpr int PR = BM / PASSES;  // tile rows per pass
  static constexpr int RPT = PR / (NT / CPR);
};

template <typename TO, int BM, int BN, int WGM, int WGN, int RPT>
__device__ __forceinline__ void load_mask_pass(Raw4<TO> (&ms)[RPT], const GemmDesc& d, int tm,
                                               int tn, int pass, int out_vec) {
  using G = EpiShape<BM, BN, WGM, WGN>;  // RPT == G::RPT where a mask is used
  const int tid = threadIdx.x;
  const int c4 = (tid % G::CPR) * 4;
  const int col = tn * BN + c4;
  const int nv = col < d.N ? min(4, d.N - col) : 0;
  const bool colfull = out_vec && nv == 4;
  const TO* __restrict__ msrc = static_cast<const TO*>(d.mask_src);
#pragma unroll
  for (int it = 0; it < G::RPT; ++it) {
    const int row = tm * BM + pass * G::PR + tid / G::CPR + it * (G::NT / G::CPR);
    const int64_t o = (int64_t)row * d.ldc + col;
    if (row < d.M && nv > 0) {
      if (colfull) ms[it].load_vec(msrc + o);
      else for (int e = 0; e < nv; ++e) ms[it].set(e, Elem<TO>::load(msrc, o + e));
    }
  }
}

// With PRE the caller has already loaded pass 0's saved activations into
// `pre` (dX epilogue with a derivative mask); otherwise they are loaded here.
// The saved activations of pass p + 1 are requested while pass p is written.
template <typename TOut, int BM, int BN, int WGM, int WGN, int EPI, int FM, int FN, bool PRE,
          typename TO, int NPRE>
__device__ __forceinline__ void store_tile_impl(const f32x16 (&acc)[FM][FN],
                                                float* __restrict__ stage, const GemmDesc& d,
                                                int tm, int tn, int split, int out_vec,
                                                Raw4<TO> (&pre)[NPRE]) {
  static_assert(std::is_same<TO, typename std::conditional<EPI == EPI_DW, float, TOut>::type>::value,
                "storage type");
  using G = EpiShape<BM, BN, WGM, WGN>;
  constexpr int NT = G::NT;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int SS = BN + 4;
  constexpr int CPR = G::CPR;
  constexpr int PASSES = G::PASSES;
  constexpr int PR = G::PR;
  static_assert(NT % CPR == 0, "each thread keeps the same columns");
  static_assert(PR % (NT / CPR) == 0, "rows per pass not divisible among threads");
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, h = lane >> 5;
  const int M = d.M, N = d.N;
  TO* __restrict__ out = static_cast<TO*>(d.C);
  int64_t ld = d.ldc;
  if (EPI == EPI_DW && d.splits > 1) {
    out = reinterpret_cast<TO*>(d.partial + (int64_t)split * M * N);
    ld = N;
  }
  TO* __restrict__ zout = static_cast<TO*>(d.Z);

  // every chunk this thread handles has the same 4 columns, pass-local rows
  // tid / CPR + it * (NT / CPR)
  constexpr int RPT = G::RPT;
  const int c4 = (tid % CPR) * 4;
  const int col = tn * BN + c4;
  const int nv = col < N ? min(4, N - col) : 0;
  const bool colfull = out_vec && nv == 4;
  float bias[4] = {0.f, 0.f, 0.f, 0.f};
  if (EPI == EPI_FWD && d.bias != nullptr)
    for (int e = 0; e < nv; ++e) bias[e] = d.bias[col + e];
  const bool masked = EPI == EPI_DX && d.mask_act != ACT_IDENTITY;
  const float osc = EPI == EPI_DW ? unscale_factor(d) : 1.0f;

  Raw4<TO> ms[EPI == EPI_DX ? RPT : 1];
  if (masked) {
    if (PRE) {
#pragma unroll
      for (int it = 0; it < (RPT < NPRE ? RPT : NPRE); ++it) ms[it] = pre[it];
    } else {
      load_mask_pass<TO, BM, BN, WGM, WGN>(ms, d, tm, tn, 0, out_vec);
    }
  }

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    const int prow0 = tm * BM + pass * PR;
    if (PASSES == 1 || wm == pass) {
      const int r0 = PASSES == 1 ? wm * WM : 0;
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            stage[(r0 + i * 32 + (r >> 2) * 8 + h * 4 + (r & 3)) * SS + wn * WN + j * 32 + l32] =
                acc[i][j][r];
    }
    __syncthreads();

    Raw4<TO> ms_next[EPI == EPI_DX && PASSES > 1 ? RPT : 1];
    if (masked && pass + 1 < PASSES)
      load_mask_pass<TO, BM, BN, WGM, WGN>(ms_next, d, tm, tn, pass + 1, out_vec);

    // (the row statistics are reduced over lane groups of at most 32, so
    // tiles of up to 128 columns write them; the launcher sends the fused
    // head's forward to no wider tile)
    constexpr bool kXent = EPI == EPI_FWD && CPR <= 32;
    const bool xent = kXent && d.xent_part != nullptr;
    if constexpr (kXent) if (xent) {
      // Logits and, for a fused softmax over many classes, each row's max
      // and sum of exp(z - max) over this tile's columns, from the same
      // float32 z = acc + bias the logits are stored as.  The CPR lanes
      // sharing a row (consecutive lanes of one wave) reduce across lanes;
      // every lane takes part (columns past N count as -inf, rows past M
      // are computed and not stored), and the group's first lane stores.
#pragma unroll
      for (int it = 0; it < RPT; ++it) {
        const int rl = tid / CPR + it * (NT / CPR);
        const int row = prow0 + rl;
        float v[4];
        Store4<float>::load_vec(stage + rl * SS + c4, v);
        float mx = -INFINITY;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] += bias[e];
          if (e < nv) mx = fmaxf(mx, v[e]);
        }
        if (row < M && nv > 0) {
          const int64_t o = (int64_t)row * ld + col;
          if (colfull) Store4<TO>::vec(out + o, v);
          else for (int e = 0; e < nv; ++e) Elem<TO>::store(out, o + e, v[e]);
        }
        mx = lanes_max<CPR>(mx);
        float se = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e < nv) se += __expf(v[e] - mx);
        se = lanes_sum<CPR>(se);
        if ((tid % CPR) == 0 && row < M)
          *reinterpret_cast<f32x2*>(d.xent_part + 2 * ((int64_t)tn * M + row)) = f32x2{mx, se};
      }
    }
    if (!xent && nv > 0) {
#pragma unroll
      for (int it = 0; it < RPT; ++it) {
        const int rl = tid / CPR + it * (NT / CPR);
        const int row = prow0 + rl;
        if (row >= M) continue;
        float v[4];
        Store4<float>::load_vec(stage + rl * SS + c4, v);
        const int64_t o = (int64_t)row * ld + col;
        if (EPI == EPI_FWD) {
          float z[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            z[e] = v[e] + bias[e];
            v[e] = act_apply(d.act, z[e]);
          }
          if (colfull) {
            Store4<TO>::vec(out + o, v);
            if (zout != nullptr) Store4<TO>::vec(zout + o, z);
          } else {
            for (int e = 0; e < nv; ++e) {
              Elem<TO>::store(out, o + e, v[e]);
              if (zout != nullptr) Elem<TO>::store(zout, o + e, z[e]);
            }
          }
        } else if (EPI == EPI_DX) {
          if (masked) {
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] *= act_deriv(d.mask_act, ms[it].get(e));
          }
          if (colfull) Store4<TO>::vec(out + o, v);
          else for (int e = 0; e < nv; ++e) Elem<TO>::store(out, o + e, v[e]);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= osc;
          if (colfull) Store4<TO>::vec(out + o, v);
          else for (int e = 0; e < nv; ++e) Elem<TO>::store(out, o + e, v[e]);
          if (EPI == EPI_DW && d.sgd_w != nullptr) {
            float* wp = d.sgd_w + o;
            if (colfull) {
              float w[4];
              Store4<float>::load_vec(wp, w);
#pragma unroll
              for (int e = 0; e < 4; ++e) w[e] -= d.sgd_lr * v[e];
              Store4<float>::vec(wp, w);
            } else {
              for (int e = 0; e < nv; ++e) wp[e] -= d.sgd_lr * v[e];
            }
          }
        }
      }
    }
    if (masked && pass + 1 < PASSES) {
#pragma unroll
      for (int it = 0; it < RPT; ++it) ms[it] = ms_next[it];
    }
    if (PASSES > 1 && pass + 1 < PASSES) __syncthreads();
  }
}

template <typename TOut, int BM, int BN, int WGM, int WGN, int EPI, int FM, int FN>
__device__ __forceinline__ void store_tile(const f32x16 (&acc)[FM][FN], float* __restrict__ stage,
                                           const GemmDesc& d, int tm, int tn, int split,
                                           int out_vec) {
  using TO = typename std::conditional<EPI == EPI_DW, float, TOut>::type;
  Raw4<TO> none[EpiShape<BM, BN, WGM, WGN>::RPT];
  store_tile_impl<TOut, BM, BN, WGM, WGN, EPI, FM, FN, false>(acc, stage, d, tm, tn, split,
                                                              out_vec, none);
}

// Host-side launchers (defined in the kernel files).
hipError_t launch_gemm_f32(const GemmDesc& d, int tile, hipStream_t s);
hipError_t launch_gemm_bf16(const GemmDesc& d, int tile, hipStream_t s);
// Weight gradient (M/N-major operands) and dX (K-major G, N-major W) of one
// small float32 layer in one launch, 64x64 tiles for both.
hipError_t launch_gemm_f32_dw_dx(const GemmDesc& dw, const GemmDesc& dx, hipStream_t s);
// Direct-to-LDS bf16 GEMM; hipErrorNotSupported when the operands do not
// meet its alignment / K-multiple requirements (nothing is launched then).
hipError_t launch_gemm_bf16_dma(const GemmDesc& d, int tile, hipStream_t s);
hipError_t launch_splitk_reduce(int M, int N, int splits, const float* partial,
                                const float* db_partial, float* C, int64_t ldc,
                                float* db, hipStream_t s);
// Y = act(b + slice-order sum of the float32 K-slices partial[S][M][N]).
hipError_t launch_splitk_finish_fwd(int M, int N, int splits, const float* partial,
                                    const float* bias, int act, float* Y, hipStream_t s);
hipError_t launch_act_mask(int dtype, int act, int64_t rows, int64_t cols,
                           const void* dY, const void* saved, void* G,
                           hipStream_t s);
// float32 -> 16-bit copies (half_kind HK_BF16 or HK_F16; the 16-bit words of
// either are moved as bf16_t)
hipError_t launch_cast_bf16(int64_t n, const float* src, bf16_t* dst,
                            hipStream_t s, int half_kind = HK_BF16);
hipError_t launch_cast_bf16_t(int64_t rows, int64_t cols, const float* src, bf16_t* dst,
                              bf16_t* dst_t, hipStream_t s, int half_kind = HK_BF16);
// dscale (optional, device float32 [1]): dlogits are multiplied by it (the
// loss scale).
// dst = half(src s) with the power-of-two scale s chosen from the largest
// finite |src| (written to scale[0]); part holds safe_scale_parts(n) floats.
int safe_scale_parts(int64_t n);
hipError_t launch_cast_f16_scaled(int64_t n, const float* src, bf16_t* dst, float* scale,
                                  float* part, hipStream_t s);
// Fused classifier head: lse and the per-row losses from the forward's
// per-tile partials ([T][B] pairs of max and sum exp), in tile order.
hipError_t launch_xent_lse(int64_t B, int64_t C, int T, const float* part, const float* logits,
                           const int32_t* labels, float* lse, float* row_loss, hipStream_t s);
// The fused head's per-row records for its backward GEMMs: rows[2 i] =
// lse[i] log2 e + log2B, rows[2 i + 1] = the bits of labels[i].
hipError_t launch_xent_rows(int64_t B, const float* lse, const int32_t* labels, float log2B,
                            float* rows, hipStream_t s);
hipError_t launch_xent(int64_t B, int64_t C, const float* logits,
                       const int32_t* labels, float* row_loss, float* dlogits,
                       float* loss, hipStream_t s, const float* dscale = nullptr);
// One launch of an empty kernel (the launch floor).
hipError_t launch_empty(hipStream_t s);
// Sets the calling thread's last-error message (dense_last_error) and
// returns `code` (defined with the C ABI in api.cpp).
int api_fail(int code, const char* msg);
// Number of labels outside [0, C) into bad[0] (one workgroup, no atomics).
hipError_t launch_label_check(int64_t B, int64_t C, const int32_t* labels, int* bad,
                              hipStream_t s);
// Fixed-order float64 mean of the per-row losses (one workgroup).
hipError_t launch_loss_mean(int64_t B, const float* row_loss, float* loss, hipStream_t s);
// Narrow classifier head of the MLP step (C <= 16 classes, K <= 256 inputs):
// last Linear + softmax-xent + its vjp in one pass; dH (may alias H, or null
// for a single-layer network) receives (W^T g) * act'(H); dW / db leave as
// head_xent_slices(B) partial slices [S][C][K] and [S][C].
bool head_xent_fits(int64_t K, int64_t C);
int64_t head_xent_slices(int64_t B);
hipError_t launch_head_xent(int64_t B, int K, int C, const float* H, float* dH, int prev_act,
                            const float* W, const float* bias, const int32_t* labels,
                            float* row_loss, float* dW_part, float* db_part, hipStream_t s,
                            const float* dscale = nullptr);
// The MLP step's tail in one kernel: the forward of a hidden layer
// [K1 -> N1] (act1), the narrow head after it [N1 -> C] with softmax-xent
// and its vjp, and the hidden layer's dX masked by act0' of its input (dH
// null: no dX).  Writes G1 [B, N1] (the hidden layer's output gradient, times
// act1'), dH [B, K1], the per-row losses and the head's dW / db as
// head_xent_slices(B) slices.  hipErrorNotSupported when Hin, W1, G1 or dH is
// not 16-byte aligned (nothing launched).
bool mlp_tail_fits(int64_t K1, int64_t N1, int64_t C);
hipError_t launch_mlp_tail(int64_t B, int K1, int N1, int C, const float* Hin, const float* W1,
                           const float* b1, int act1, int act0, const float* W2, const float* b2,
                           const int32_t* labels, float* row_loss, float* G1, float* dH,
                           float* dW_part, float* db_part, hipStream_t s,
                           const float* dscale = nullptr);
// The same tail for a smaller batch (K1 = 256, N1 = 128 or 256, B <= 8192):
// 16-row tiles on the 16x16x4 MFMA, one per workgroup, dW / db as
// mlp_tail_narrow_slices(B) slices.  With fold_splits > 0, Hin is first
// formed as act0(sum of fold_splits K-slices fold_part[s][B][K1] + b0) and
// written to Hin; else it is read from Hin.  hipErrorNotSupported when Hin,
// W1, G1 or fold_part is not 16-byte aligned (nothing launched).
bool mlp_tail_narrow_fits(int64_t B, int64_t K1, int64_t N1, int64_t C);
// The K-slices slices[s][B][N] of X [B, K] W^T (W [N, K]) for a small batch,
// slice s over k in [s kps, min(K, (s + 1) kps)), on 16-row x 64-column
// tiles and the 16x16x4 MFMA (the narrow tail then adds them with the bias
// and activation).  Needs K % 4 == 0, kps a multiple of 16 up to 256, and
// splits slices covering K exactly; hipErrorNotSupported when X or W is not
// 16-byte aligned (nothing launched).
bool mlp_fwd_narrow_fits(int64_t B, int64_t K, int64_t N, int kps);
hipError_t launch_mlp_fwd_narrow(int B, int K, int N, int splits, int kps, const float* X,
                                 const float* W, float* slices, hipStream_t s);
int64_t mlp_tail_narrow_slices(int64_t B);
hipError_t launch_mlp_tail_narrow(int64_t B, int K1, int N1, int C, float* Hin,
                                  const float* fold_part, int fold_splits, const float* b0,
                                  const float* W1, const float* b1, int act1, int act0,
                                  const float* W2, const float* b2, const int32_t* labels,
                                  float* row_loss, float* G1, float* dH, float* dW_part,
                                  float* db_part, hipStream_t s, const float* dscale = nullptr);
// Two float32 weight gradients (M/N-major operands, 64x64 tiles) in one
// launch; with fin, also the sgd_finish_wgs(*fin) workgroups of
// sgd_finish_block (a descriptor with sgd_w set then needs one K slice, db
// and sgd_b, and sgd_w at the alignment of C modulo 16 bytes).
struct SgdFinish;
hipError_t launch_gemm_f32_dw_dw(const GemmDesc& a, const GemmDesc& b, hipStream_t s,
                                 const SgdFinish* fin = nullptr);
// Optimizer kinds (the values of enum dl_opt_kind).
enum OptKind { OPT_SGD = 0, OPT_ADAMW = 1, OPT_ADAM = 2 };

// Learning-rate schedule (the fields of dl_lr_schedule_t); kind 0 = constant.
struct LrSched {
  int kind;
  int64_t warmup, total, step_size;
  double min_lr, gamma;
};

// The learning rate of step t >= 1: k = t - 1 scheduler steps; a linear
// warmup to lr over `warmup` steps, then a cosine or linear decay to min_lr
// reached at k = total, or lr gamma^floor(k / step_size).  Double precision;
// the same code runs on the host (host step count) and on the device
// (device step count).
__host__ __device__ inline double lr_schedule(const LrSched& s, double lr, int64_t t) {
  const int64_t k = t - 1;
  if (s.kind == 1) return lr * pow(s.gamma, (double)(k / s.step_size));
  if (s.kind == 2 || s.kind == 3) {
    if (k < s.warmup) return lr * (double)(k + 1) / (double)s.warmup;
    const int64_t T = s.total - s.warmup;
    if (T <= 0) return s.min_lr;
    const int64_t j = k - s.warmup < T ? k - s.warmup : T;
    if (s.kind == 2)
      return s.min_lr + (lr - s.min_lr) * (1.0 + cos(3.141592653589793 * (double)j / (double)T)) / 2.0;
    return s.min_lr + (lr - s.min_lr) * (double)(T - j) / (double)T;
  }
  return lr;
}

// What the gradient pass leaves for the optimizer (device memory): every
// gradient is used multiplied by `mul` (clip coefficient / loss scale), and
// with `skip` set the update is not applied at all.
struct GradCtl {
  float mul;
  int skip;
  float norm;
  int pad;
};

// Optimizer constants, each formed in double on the host and rounded once.
struct OptConsts {
  float lr;            // SGD step
  float decay;         // AdamW: 1 - lr wd
  float wd;            // Adam: coupled decay
  float b1, omb1;      // beta1, 1 - beta1
  float b2, omb2;      // beta2, 1 - beta2
  float step_size;     // lr / (1 - beta1^t)
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^t)
  float eps;
  float ema_d, ema_omd;  // parameter averages: d, 1 - d
  // With a device step count: t = *step_dev, and lr (scheduled), decay,
  // step_size and inv_sqrt_bc2 are formed on the device from these doubles
  const int64_t* step_dev;
  double lr_d, beta1_d, beta2_d, wd_d;
  LrSched sched;
  const GradCtl* ctl;  // gradient control of this step, or null
};
// Adds 1 to a device step count (one lane, a vector store).
hipError_t launch_step_tick(int64_t* step_dev, hipStream_t s);
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
  float* ema[kMaxSegs];   // parameter average, or null
  bf16_t* wb[kMaxSegs];   // bf16 copy of the updated w, or null
  // optional: one extra workgroup (the first) writes loss = mean(row_loss[0 ..
  // rows)) (float64, fixed order)
  const float* row_loss;
  int64_t rows;
  float* loss;
};
constexpr int kOptBlock = 256;
constexpr int kOptElemsPerBlock = kOptBlock * 4 * 4;  // 4 float4 per thread
constexpr int kOptSplitElemsPerBlock = kOptBlock;      // split-K segments: 4 lanes per 4 elements
constexpr int kOptWideSplits = 32;                     // more slices: a wave per 4 elements
constexpr int kOptWideElemsPerBlock = kOptBlock / 16;
constexpr int kOptFewSplits = 4;                       // up to 4 slices: a thread per 4 elements
inline int64_t opt_elems_per_block(int splits) {
  return splits > kOptWideSplits ? kOptWideElemsPerBlock
                                 : (splits > kOptFewSplits ? kOptSplitElemsPerBlock : kOptElemsPerBlock);
}
hipError_t launch_opt_multi(const OptSegs& segs, int kind, const OptConsts& c,
                            hipStream_t s);
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

// SGD of one layer whose dW / db are the split-K or row-tile slices of a
// fused kernel (or, with one slice, already final), by
// kOptBlock-thread workgroups that also form the loss mean: each element's
// slices are added as the multi-array optimizer adds them (slice k into
// partial sum k mod 4, in slice order, then (p0 + p1) + (p2 + p3)), the sum
// stored as the gradient, and w -= lr g.
struct SgdFinish {
  float* W;
  float* b;
  float* dW;
  float* db;
  const float* dW_part;  // [slices][n_w], or null with one slice
  const float* db_part;  // [slices][n_b]
  int64_t n_w;
  int n_b, slices;
  float lr;
  int64_t rows;  // the loss mean: rows of row_loss into loss
  const float* row_loss;
  float* loss;
};
// Finishing workgroup `part` of sgd_finish_wgs(f): elements [part kOptBlock,
// +kOptBlock) of W then b, one per thread with all its slices requested
// before the first is added; part 0 also forms the loss mean.
__device__ __forceinline__ void sgd_finish_block(const SgdFinish& f, int part) {
  if (part == 0) loss_mean_block(f.rows, f.row_loss, f.loss);
  const int64_t i = (int64_t)part * kOptBlock + threadIdx.x;
  if (i >= f.n_w + f.n_b) return;
  const bool isw = i < f.n_w;
  const int64_t j = isw ? i : i - f.n_w;
  float* w = isw ? f.W : f.b;
  float* g_out = isw ? f.dW : f.db;
  float g;
  if (f.slices > 1) {
    const float* part_p = (isw ? f.dW_part : f.db_part) + j;
    const int64_t stride = isw ? f.n_w : (int64_t)f.n_b;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    int k = 0;
    for (; k + 4 <= f.slices; k += 4) {
      float x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = part_p[(int64_t)(k + u) * stride];
#pragma unroll
      for (int u = 0; u < 4; ++u) a[u] += x[u];
    }
    for (int u = 0; k + u < f.slices; ++u) a[u] += part_p[(int64_t)(k + u) * stride];
    g = (a[0] + a[1]) + (a[2] + a[3]);
    g_out[j] = g;
  } else {
    g = g_out[j];
  }
  w[j] -= f.lr * g;
}
inline int sgd_finish_wgs(const SgdFinish& f) {
  return (int)((f.n_w + f.n_b + kOptBlock - 1) / kOptBlock);
}

hipError_t launch_adam(int64_t n, float* w, const float* g, float* m, float* v,
                       const OptConsts& c, hipStream_t s);
hipError_t launch_ema(int64_t n, float* e, const float* w, float d, float omd, hipStream_t s);

// ---- gradient control (global norm, finite check, loss scale) ---------------
// The gradient pass reads every gradient once (finishing split-K sums into
// g_out on the way) and leaves per-workgroup float64 sums of squares and
// non-finite counts; the control kernel (one workgroup) adds them in a fixed
// order and writes the GradCtl, updates the loss scaler and ticks the
// device step count.  The segments' start_block holds prefix sums of units of
// kStatUnit elements (stat_units: their total); at most kStatBlocks
// workgroups per launch (stat_grid), each taking units b, b + grid, ...
constexpr int kStatUnit = kOptElemsPerBlock;
constexpr int kStatBlocks = 2048;
int64_t stat_units(const OptSegs& segs);
int stat_grid(int64_t units);
hipError_t launch_grad_stats(const OptSegs& segs, int64_t units, double* part_sq, int* part_bad,
                             hipStream_t s);
struct CtlArgs {
  const double* part_sq;
  const int* part_bad;
  int parts;
  double max_norm;          // <= 0: no clipping
  float* scale;             // loss scale, or null
  int* growth_tracker;
  int* found_inf;
  double growth_factor, backoff_factor;
  int growth_interval;
  int64_t* step_dev;        // ticked when the step is applied, or null
  float* norm_out;          // optional
  GradCtl* ctl;
  float* clip_coef;         // optional: min(1, max_norm / (norm + 1e-6))
};
hipError_t launch_grad_ctl(const CtlArgs& a, hipStream_t s);
// g *= *coef where *coef < 1 (clip_grad_norm's in-place scaling).
hipError_t launch_scale_by(const OptSegs& segs, const float* coef, hipStream_t s);

// ---- mean squared error --------------------------------------------------------
int mse_grid(int64_t n);
// dscale (optional, device float32 [1]): dpred is multiplied by it (the loss
// scale).
hipError_t launch_mse(int64_t n, const float* pred, const float* target, float* dpred,
                      double* part, float* loss, hipStream_t s, const float* dscale = nullptr);

}  // namespace dl

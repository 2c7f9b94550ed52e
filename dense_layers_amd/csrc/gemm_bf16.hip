// 16-bit-operand GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16,
// or _f16 for IEEE half operands, whose outputs round with saturation at
// +-65504; float32 accumulation) with the dense-layer epilogues fused in.
//
// Same three products as the float32 kernel (forward, dX, dW; the fused
// LinearAct of the noeira.nn docs, "The design in one page") for operands
// held as bf16 working copies (the FP32-master-weight scheme of the Orthon
// page, "Mixed-precision training on CUDA"; round-to-nearest-even copies as in
// the MuNet page, "Configuration").  Forward and dX results are stored as
// bf16, dW and db as float32.
//
// LDS holds every operand K-contiguous: each tile row (one m or n) is BK = 64
// bf16 = 128 bytes, eight 16-byte units, and a lane's MFMA fragment (8
// consecutive k of one row) is one 16-byte LDS read.  Units are XOR-swizzled
// by row, unit' = unit ^ ((row ^ row >> 3) & 7), so the 8 lanes that read
// rows r..r+7 of one unit, and the 8 lanes that store rows 8 apart in the
// transposing path, all land on different banks.
//
// K-major operands are copied in 16-byte vectors.  M/N-major operands
// (dW's A and B, dX's B) are transposed on the way in: a thread loads a
// 4 (k) x 8 (m) block as four 16-byte row pieces, regroups them in registers
// into eight 4-k column pieces and stores each with one 8-byte LDS write.
//
// As in the float32 kernel, which k a lane supplies inside an MFMA is free as
// long as A and B agree: at k-step ks, lane half h supplies k = 16 ks + 8 h +
// (0..7).
#include "common.hpp"

namespace dl {
namespace {

constexpr int BK = 64;           // k per LDS tile
constexpr int kRowElems = BK;    // bf16 per LDS row (no padding; swizzled)

__device__ __forceinline__ int swz(int row, int unit) {
  return unit ^ ((row ^ (row >> 3)) & 7);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int ROWS, int LAY, int NT>
struct TileLoaderBf16 {
  static constexpr int kLdsSize = ROWS * kRowElems;  // bf16 elements
  // K-major: ROWS x 8 vectors of 8 bf16.  MN-major: (BK/4) x (ROWS/8) blocks.
  static constexpr int kItems = (LAY == K_MAJOR) ? ROWS * (BK / 8) : (BK / 4) * (ROWS / 8);
  static_assert(kItems % NT == 0, "tile not divisible among threads");
  static constexpr int kPer = kItems / NT;
  static constexpr int kRegs = (LAY == K_MAJOR) ? kPer : kPer * 4;

  u32x4 r[kRegs];

  // The per-thread part of the full K steps' load addresses, fixed for a
  // tile: item i's row and 16-byte unit at k = 0 (K-major), or its first k
  // row and m (M/N-major).  A K step then adds k0, or k0 ld and j ld for the
  // rows of a block, which the whole workgroup shares, instead of forming
  // each address's 64-bit product again.  Rows past the end (edge tiles) are
  // clamped to a valid row: they only feed output rows / columns that are
  // never stored.  For an M/N-major operand this needs nrows % 8 == 0 so that
  // no vector straddles the end (checked by the caller).
  struct Origin {
    const bf16_t* p[kPer];
  };
  __device__ __forceinline__ static Origin origin(const bf16_t* __restrict__ base, int64_t ld,
                                                  int row0, int nrows, int tid) {
    Origin o;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * NT;
      if (LAY == K_MAJOR) {
        const int row = min(row0 + q / (BK / 8), nrows - 1);
        o.p[i] = base + (int64_t)row * ld + (q % (BK / 8)) * 8;
      } else {
        int m = row0 + (q % (ROWS / 8)) * 8;
        m = m < nrows ? m : 0;
        o.p[i] = base + (int64_t)(q / (ROWS / 8) * 4) * ld + m;
      }
    }
    return o;
  }

  // Full K step, 16-byte aligned rows: plain vector loads with no
  // per-element control flow, so the loads of a K step stay in flight
  // together.
  __device__ __forceinline__ void load_fast(const Origin& o, int64_t ld, int k0) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (LAY == K_MAJOR) {
        r[i] = *reinterpret_cast<const u32x4*>(o.p[i] + k0);
      } else {
        const bf16_t* q = o.p[i] + (int64_t)k0 * ld;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[i * 4 + j] = *reinterpret_cast<const u32x4*>(q + j * ld);
      }
    }
  }

  // Edge tiles: element loads, zero outside [0, nrows) x [k0, kend).
  __device__ __forceinline__ static u32x4 load_row8(const bf16_t* __restrict__ p, int valid) {
    u32x4 x = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t e = (j < valid) ? static_cast<uint32_t>(p[j]) : 0u;
      x[j >> 1] |= e << ((j & 1) * 16);
    }
    return x;
  }

  __device__ __forceinline__ void load_safe(const bf16_t* __restrict__ base, int64_t ld, int row0,
                                            int nrows, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * NT;
      if (LAY == K_MAJOR) {
        const int row = row0 + q / (BK / 8);
        const int k = k0 + (q % (BK / 8)) * 8;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row < nrows && k < kend) x = load_row8(base + (int64_t)row * ld + k, kend - k);
        r[i] = x;
      } else {
        const int mg = q % (ROWS / 8);
        const int kq = q / (ROWS / 8);
        const int m = row0 + mg * 8;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int k = k0 + kq * 4 + j;
          u32x4 x = {0u, 0u, 0u, 0u};
          if (k < kend && m < nrows) x = load_row8(base + (int64_t)k * ld + m, nrows - m);
          r[i * 4 + j] = x;
        }
      }
    }
  }

  __device__ __forceinline__ void store(bf16_t* __restrict__ lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int q = tid + i * NT;
      if (LAY == K_MAJOR) {
        const int row = q / (BK / 8);
        const int unit = q % (BK / 8);
        *reinterpret_cast<u32x4*>(lds + row * kRowElems + swz(row, unit) * 8) = r[i];
      } else {
        const int mg = q % (ROWS / 8);
        const int kq = q / (ROWS / 8);
        // rows j = 0..3 of the block hold k = 4kq + j; element c of a row is
        // m = 8mg + c.  Column c gathers element c of the 4 rows: one byte
        // permute per pair of rows (low or high halves of word c / 2).
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int w = c >> 1;
          const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
          u32x2 col = {__builtin_amdgcn_perm(r[i * 4 + 1][w], r[i * 4 + 0][w], sel),
                       __builtin_amdgcn_perm(r[i * 4 + 3][w], r[i * 4 + 2][w], sel)};
          const int row = mg * 8 + c;
          const int unit = kq >> 1;
          *reinterpret_cast<u32x2*>(lds + row * kRowElems + swz(row, unit) * 8 + (kq & 1) * 4) = col;
        }
      }
    }
  }

  // 8 bf16 of tile row `row` at k-step ks (16 k), lane half h.
  __device__ __forceinline__ static bf16x8 frag(const bf16_t* __restrict__ lds, int row, int ks,
                                                int h) {
    const u32x4 x = *reinterpret_cast<const u32x4*>(lds + row * kRowElems + swz(row, ks * 2 + h) * 8);
    return __builtin_bit_cast(bf16x8, x);
  }
};

template <int BM, int BN, int WGM, int WGN, int ALAY, int BLAY, int EPI, int HK>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_bf16_kernel(GemmDesc d, int tiles_m, int tiles_n, int a_vec, int b_vec, int out_vec) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 1, "bad tile");
  using LA = TileLoaderBf16<BM, ALAY, NT>;
  using LB = TileLoaderBf16<BN, BLAY, NT>;
  constexpr int kSmemAB = (2 * LA::kLdsSize + 2 * LB::kLdsSize) * 2;  // bytes
  constexpr int kStage = stage_floats<BM, BN, WGM>() * 4;
  __shared__ __attribute__((aligned(16))) char smem[kSmemAB > kStage ? kSmemAB : kStage];
  // buffer b of A at b * LA::kLdsSize, of B after both A buffers
  auto As = [&](int b) { return reinterpret_cast<bf16_t*>(smem) + b * LA::kLdsSize; };
  auto Bs = [&](int b) {
    return reinterpret_cast<bf16_t*>(smem) + 2 * LA::kLdsSize + b * LB::kLdsSize;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, h = lane >> 5;

  int split, tm, tn;
  tile_coords(tiles_m, tiles_n, split, tm, tn);

  const int M = d.M, N = d.N;
  const int kbeg = split * d.k_per_split;
  const int kend = min(d.K, kbeg + d.k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const bf16_t* __restrict__ A = static_cast<const bf16_t*>(d.A);
  const bf16_t* __restrict__ B = static_cast<const bf16_t*>(d.B);

  LA la;
  LB lb;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const bool do_db = (EPI == EPI_DW) && (d.db != nullptr || d.db_partial != nullptr) &&
                     tn == 0 && wn == 0;
  float dbacc[FM];
#pragma unroll
  for (int i = 0; i < FM; ++i) dbacc[i] = 0.f;

  // When both operands allow 16-byte loads, the full K steps run with
  // branch-free vector loads (edge rows clamped); a last partial K step, or
  // operands that do not allow vector loads, go through the bounds-checked
  // loads.  The two
  // loops are kept apart so that no join of the two load paths sits inside
  // the loop where the compiler would have to drain the loads in flight.
  const bool fast = a_vec && b_vec && (ALAY == K_MAJOR || M % 8 == 0) &&
                    (BLAY == K_MAJOR || N % 8 == 0);
  const int nk_full = fast ? (kend - kbeg) / BK : 0;

  auto compute = [&](int cur) {
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) a[i] = LA::frag(As(cur), wm * WM + i * 32 + l32, ks, h);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[j] = LB::frag(Bs(cur), wn * WN + j * 32 + l32, ks, h);
      if (do_db) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < 8; ++e) s += HalfOps<HK>::elem(a[i], e);
          dbacc[i] += s;
        }
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
          acc[i][j] = HalfOps<HK>::mfma(a[i], b[j], acc[i][j]);
    }
  };

  // Loads run two K steps ahead: register set 1 (la, lb) and set 2 (la2,
  // lb2) alternate, so each load has two steps of MFMA work to land in.
  // Invariant at the top of a trip: LDS buffer (kt & 1) holds step kt and
  // set 2 holds step kt + 1 in flight.
  LA la2;
  LB lb2;
  const typename LA::Origin oa = LA::origin(A, d.lda, tm * BM, M, tid);
  const typename LB::Origin ob = LB::origin(B, d.ldb, tn * BN, N, tid);
  if (nk > 0) {
    if (nk_full > 0) {
      la.load_fast(oa, d.lda, kbeg);
      lb.load_fast(ob, d.ldb, kbeg);
    } else {
      la.load_safe(A, d.lda, tm * BM, M, kbeg, kend, tid);
      lb.load_safe(B, d.ldb, tn * BN, N, kbeg, kend, tid);
    }
    la.store(As(0), tid);
    lb.store(Bs(0), tid);
    if (nk_full >= 2) {
      la2.load_fast(oa, d.lda, kbeg + BK);
      lb2.load_fast(ob, d.ldb, kbeg + BK);
    }
  }
  __syncthreads();

  int kt = 0;
  for (; kt + 3 < nk_full; kt += 2) {
    la.load_fast(oa, d.lda, kbeg + (kt + 2) * BK);
    lb.load_fast(ob, d.ldb, kbeg + (kt + 2) * BK);
    // keep the loads ahead of the MFMAs (the scheduler would otherwise sink
    // them next to their LDS stores)
    __builtin_amdgcn_sched_barrier(0);
    compute(0);
    __builtin_amdgcn_sched_barrier(0);
    la2.store(As(1), tid);
    lb2.store(Bs(1), tid);
    __syncthreads();
    la2.load_fast(oa, d.lda, kbeg + (kt + 3) * BK);
    lb2.load_fast(ob, d.ldb, kbeg + (kt + 3) * BK);
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    __builtin_amdgcn_sched_barrier(0);
    la.store(As(0), tid);
    lb.store(Bs(0), tid);
    __syncthreads();
  }
  if (kt + 1 < nk_full) {  // drain set 2
    __builtin_amdgcn_sched_barrier(0);
    compute(kt & 1);
    __builtin_amdgcn_sched_barrier(0);
    la2.store(As((kt + 1) & 1), tid);
    lb2.store(Bs((kt + 1) & 1), tid);
    __syncthreads();
    ++kt;
  }
  for (; kt + 1 < nk_full; ++kt) {
    const int cur = kt & 1;
    const int k0 = kbeg + (kt + 1) * BK;
    la.load_fast(oa, d.lda, k0);
    lb.load_fast(ob, d.ldb, k0);
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
    __builtin_amdgcn_sched_barrier(0);
    la.store(As(cur ^ 1), tid);
    lb.store(Bs(cur ^ 1), tid);
    __syncthreads();
  }
  for (; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      const int k0 = kbeg + (kt + 1) * BK;
      la.load_safe(A, d.lda, tm * BM, M, k0, kend, tid);
      lb.load_safe(B, d.ldb, tn * BN, N, k0, kend, tid);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(cur);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      la.store(As(cur ^ 1), tid);
      lb.store(Bs(cur ^ 1), tid);
    }
    __syncthreads();
  }

  // ---- epilogue -------------------------------------------------------------
  if (EPI == EPI_DW && do_db) {
    const int row_base = tm * BM + wm * WM;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float v = (dbacc[i] + __shfl_xor(dbacc[i], 32)) * unscale_factor(d);
      const int row = row_base + i * 32 + l32;
      if (h == 0 && row < M) {
        if (d.splits > 1) d.db_partial[(int64_t)split * M + row] = v;
        else d.db[row] = v;
      }
    }
  }
  store_tile<typename HalfOps<HK>::T, BM, BN, WGM, WGN, EPI>(acc, reinterpret_cast<float*>(smem),
                                                              d, tm, tn, split, out_vec);
}

template <int BM, int BN, int WGM, int WGN, int ALAY, int BLAY, int EPI, int HK>
hipError_t launch_tile(const GemmDesc& d, hipStream_t s) {
  const int tiles_m = (d.M + BM - 1) / BM;
  const int tiles_n = (d.N + BN - 1) / BN;
  const int64_t nwg = (int64_t)tiles_m * tiles_n * d.splits;
  if (nwg <= 0 || nwg > 0x7fffffff) return hipErrorInvalidValue;
  auto aligned = [](const void* p, int64_t ld) {
    return ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (ld % 8 == 0);
  };
  const int a_vec = aligned(d.A, d.lda);
  const int b_vec = aligned(d.B, d.ldb);
  // output: float32 (dW) needs 16-byte rows of 4, bf16 needs 8-byte rows of 4
  auto out_ok = [](const void* p, int64_t ld, int bytes) {
    return ((reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0) && (ld % 4 == 0);
  };
  int out_vec;
  if (EPI == EPI_DW)
    out_vec = d.splits > 1 ? out_ok(d.partial, d.N, 16) : out_ok(d.C, d.ldc, 16);
  else
    out_vec = out_ok(d.C, d.ldc, 8) && (d.Z == nullptr || out_ok(d.Z, d.ldc, 8)) &&
              (d.mask_src == nullptr || out_ok(d.mask_src, d.ldc, 8));
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, WGM, WGN, ALAY, BLAY, EPI, HK>), dim3((unsigned)nwg),
                     dim3(WGM * WGN * 64), 0, s, d, tiles_m, tiles_n, a_vec, b_vec, out_vec);
  return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int HK>
hipError_t dispatch_layout(const GemmDesc& d, hipStream_t s) {
  if (d.epi == EPI_FWD && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_tile<BM, BN, WGM, WGN, K_MAJOR, K_MAJOR, EPI_FWD, HK>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == MN_MAJOR)
    return launch_tile<BM, BN, WGM, WGN, K_MAJOR, MN_MAJOR, EPI_DX, HK>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_tile<BM, BN, WGM, WGN, K_MAJOR, K_MAJOR, EPI_DX, HK>(d, s);
  if (d.epi == EPI_DW && d.a_layout == MN_MAJOR && d.b_layout == MN_MAJOR)
    return launch_tile<BM, BN, WGM, WGN, MN_MAJOR, MN_MAJOR, EPI_DW, HK>(d, s);
  return hipErrorInvalidValue;
}

}  // namespace

// Forward and dX products go to the direct-to-LDS kernel (tile 0: 256x256,
// tile 1: 128x128) when the operands allow it; weight gradients (both
// operands M/N-major), and operands it declines, run the general kernel at
// 128x128 (4 waves of 64x64, two workgroups per CU).  For the weight
// gradients this kernel's transpose in registers, which leaves both operands
// K-contiguous in LDS for 16-byte fragment reads, measured faster than the
// direct-to-LDS kernel's transposing 8-byte reads (the 32768-token
// transformer MLP's two weight gradients: 326-342 against 395-401 us).
hipError_t launch_gemm_bf16(const GemmDesc& d, int tile, hipStream_t s) {
  if ((tile == 0 || tile == 1) && d.epi != EPI_DW) {
    const hipError_t e = launch_gemm_bf16_dma(d, tile, s);
    if (e != hipErrorNotSupported) return e;
  }
  return d.half_kind == HK_F16 ? dispatch_layout<128, 128, 2, 2, HK_F16>(d, s)
                                : dispatch_layout<128, 128, 2, 2, HK_BF16>(d, s);
}

}  // namespace dl

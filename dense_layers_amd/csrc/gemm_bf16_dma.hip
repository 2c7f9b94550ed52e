// 16-bit-operand GEMM for large, aligned problems: operand tiles go from HBM
// straight into LDS (global_load_lds_dwordx4, no staging registers), the
// matrix cores read them back as MFMA fragments (v_mfma_f32_32x32x16_bf16, or
// _f16 for IEEE half operands; float32 accumulation), and the dense-layer
// epilogues (bias + activation, act' masking, float32 weight-gradient slices)
// are applied on the way out.  bf16 and half take the same path: only the
// MFMA, the output rounding (half saturates at +-65504) and the reading of
// saved activations differ (HalfOps).
//
// The products are those of the fused LinearAct (noeira.nn docs, "The
// design in one page"): forward Z = X W^T + b and dX = (dY o act') W, on the
// bf16 working copies of the FP32-master-weight scheme (Orthon page,
// "Mixed-precision training on CUDA").  The kernel's weight-gradient form
// dW = (dY o act')^T X (float32 slices, the db sums) is kept in the template
// but no longer launched: the register-staged kernel of gemm_bf16.hip
// measured faster for those products, whose operands are both M/N-major.
//
// Pipeline: STAGES LDS buffers of BK k each.  The loads of stage
// g + STAGES - 1 are issued during stage g (spread over its k-steps), so each
// load has about STAGES - 2 stages of matrix-core work to land in; nothing is
// staged in VGPRs.  One barrier per stage publishes the next stage (see the
// loop).  Work items are (split, tile) pairs; in the persistent form a
// workgroup walks several items with one continuous pipeline.
//
// A direct load writes 64 lanes x 16 bytes to 1 KB of consecutive LDS, so the
// LDS layout is chosen by which global 16-byte unit each lane fetches:
//  * K-major operand (rows contiguous in k): LDS row r holds the BK k of tile
//    row r as BK / 8 16-byte units, unit u at position u ^ ksw(r).  A lane's
//    fragment (8 consecutive k of one row) is one 16-byte LDS read; the 16
//    lanes of one read phase land on distinct banks.
//  * M/N-major operand (rows contiguous in m): LDS k-row k holds the tile's
//    ROWS m of that k, 16-byte unit u at position u ^ (4 (k & 3)).  Fragments
//    come from the gfx950 transposing read ds_read_b64_tr_b16: in each group
//    of 16 lanes, lane i receives element i % 4 of the 8-byte piece addressed
//    by lane 4 t + i / 4 as its element t.  Lane 4 t + q of the group
//    addresses k-row (k0 + t), m = m0 + 4 q, so lane i gets k0 .. k0 + 3 of
//    column m0 + i; two reads give the 8 k of a fragment.  The 4 k-rows read
//    together sit in different 64-byte bank groups.
// Which k a lane supplies inside an MFMA is free as long as A and B agree: at
// k-step ks, lane half h supplies k = 16 ks + 8 h + (0..7) for both layouts.
//
// Requirements (checked by the launcher, which reports hipErrorNotSupported
// otherwise so the caller can use the general kernel): A and B 16-byte
// aligned with leading dimensions a multiple of 8, K and the split length
// multiples of 64, and M (N) a multiple of 8 when A (B) is M/N-major.  Tile
// rows past M or N are clamped to a valid row; they only feed outputs that are
// never stored.
#include "common.hpp"

namespace dl {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// s_waitcnt immediate that waits for at most n outstanding vector-memory
// operations and leaves the LDS and export counters alone.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// K-major swizzle: 16-byte unit u of tile row r sits at position u ^ ksw(r).
// With BK = 64 a row is 8 units (128 bytes), with BK = 32 it is 4 units and
// four consecutive rows share a 256-byte bank window.
template <int BK>
__device__ __forceinline__ int ksw(int row) {
  return BK == 64 ? ((row ^ (row >> 3)) & 7) : ((row >> 2) & 3);
}
__device__ __forceinline__ int msw(int k) { return (k & 3) << 2; }

template <int ROWS, int LAY, int NT, int BK>
struct DmaOperand {
  static constexpr int kBytes = ROWS * BK * 2;  // one stage
  static constexpr int kUnits = ROWS * BK / 8;  // 16-byte units per stage
  static constexpr int kUPR = BK / 8;           // units per K-major row
  static constexpr int kWaves = NT / 64;
  static constexpr int kInst = kUnits / (64 * kWaves);  // loads per wave per stage
  static_assert(kUnits % (64 * kWaves) == 0, "stage not divisible among waves");
  static_assert(LAY == K_MAJOR || ROWS % 128 == 0, "M/N-major tiles need 16+ units per k-row");
  static_assert(BK == 32 || BK == 64, "BK");

  const bf16_t* ptr[kInst];  // this lane's source for load i of the next stage
  int64_t step;              // elements between consecutive stages

  __device__ __forceinline__ void init(const bf16_t* __restrict__ base, int64_t ld, int row0,
                                       int nrows, int k0, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < kInst; ++i) {
      const int U = (i * kWaves + wave) * 64 + lane;  // LDS position of this lane's unit
      if (LAY == K_MAJOR) {
        const int row = U / kUPR;
        const int u = (U % kUPR) ^ ksw<BK>(row);
        const int grow = min(row0 + row, nrows - 1);
        ptr[i] = base + (int64_t)grow * ld + k0 + u * 8;
      } else {
        constexpr int UPR = ROWS / 8;
        const int kr = U / UPR;
        const int u = (U % UPR) ^ msw(kr);
        int m = row0 + u * 8;
        if (m >= nrows) m = row0;
        ptr[i] = base + (int64_t)(k0 + kr) * ld + m;
      }
    }
    step = LAY == K_MAJOR ? BK : (int64_t)BK * ld;
  }

  // Issue this wave's load i of the next stage into `lds` (the operand's
  // buffer) and advance to the stage after it.
  __device__ __forceinline__ void issue_one(char* lds, int wave, int i) {
    __builtin_amdgcn_global_load_lds(
        (__attribute__((address_space(1))) void*)ptr[i],
        (__attribute__((address_space(3))) void*)(lds + (i * kWaves + wave) * 1024), 16, 0, 0);
    ptr[i] += step;
  }

  // After the last stage: later loads repeat that stage, so that every stage
  // issues the same number of loads; the buffers they fill are never read.
  __device__ __forceinline__ void park() {
#pragma unroll
    for (int i = 0; i < kInst; ++i) ptr[i] -= step;
    step = 0;
  }

  // Fragment of tile rows mb .. mb + 31 at k-step ks: this lane's 8 k.
  __device__ __forceinline__ static bf16x8 frag(const char* lds, int mb, int ks, int lane) {
    if (LAY == K_MAJOR) {
      const int row = mb + (lane & 31);
      const int pos = (2 * ks + (lane >> 5)) ^ ksw<BK>(row);
      return *reinterpret_cast<const bf16x8*>(lds + row * (BK * 2) + pos * 16);
    } else {
      const int g = (lane >> 4) & 1, h = lane >> 5, t = (lane >> 2) & 3, q = lane & 3;
      const int m = mb + 16 * g + 4 * q;
      const int k0 = ks * 16 + 8 * h + t;
      const int off = ((m >> 3) ^ (t << 2)) * 16 + ((m >> 2) & 1) * 8;
      typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(lds + k0 * (ROWS * 2) + off));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(lds + (k0 + 4) * (ROWS * 2) + off));
      const s16x8 x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      return __builtin_bit_cast(bf16x8, x);
    }
  }
};

// Scheduling hint for one k-step: its MFMAs interleaved with the LDS reads of
// the next fragments and with NV global loads.
template <int kMfma, int kReads, int NV>
__device__ __forceinline__ void sched_interleave() {
#pragma unroll
  for (int r = 0; r < kMfma; ++r) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (r < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    if (r < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
  }
  if (kReads > kMfma) __builtin_amdgcn_sched_group_barrier(0x100, kReads > kMfma ? kReads - kMfma : 1, 0);
  if (NV > kMfma) __builtin_amdgcn_sched_group_barrier(0x020, NV > kMfma ? NV - kMfma : 1, 0);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---- epilogue ------------------------------------------------------------------
// The matrix cores form each 32x32 block transposed (the B fragment is the
// MFMA's first operand), so lane l holds tile row 32 i + l % 32 of block
// (i, j) and, in register group g (registers 4 g .. 4 g + 3), the 4
// consecutive columns 8 g + 4 h + (0..3), h = l / 32.  Exchanging groups
// 0 <-> 2 and 1 <-> 3 between the wave halves (v_permlane32_swap) leaves
// each lane with the 16 consecutive columns 16 h + c, c = 0..15, of its row,
// column c in register col_reg(c).
//
// Each wave then finishes its own WM x WN sub-tile through a private LDS
// region (the stage buffers, free after the main loop): lanes write their
// 16-value row pieces, and read back whole rows, so that every global store
// instruction writes 8 rows x 128 bytes (bf16) or 4 rows x 256 bytes
// (float32).  Row r of the region keeps its 16-byte pieces at position
// piece ^ (r mod pieces-per-row), which makes both the column-wise writes and
// the row-wise reads free of bank conflicts.  No workgroup barrier is needed
// beyond the one that retires the stage buffers.
__device__ __forceinline__ int col_reg(int c) { return (c & 3) | ((c & 4) << 1) | ((c & 8) >> 1); }

template <int FM, int FN>
__device__ __forceinline__ void swap_halves(f32x16 (&acc)[FM][FN]) {
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][j][r]),
                                                        __float_as_uint(acc[i][j][r + 8]), false,
                                                        false);
        acc[i][j][r] = __uint_as_float(p[0]);
        acc[i][j][r + 8] = __uint_as_float(p[1]);
      }
}

// One lane's row and first column of block (i, j) in the output.
struct BlockPos {
  int row, col;
};
template <int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ BlockPos block_pos(int tm, int tn, int wm, int wn, int i, int j,
                                              int lane) {
  constexpr int WM = BM / WGM, WN = BN / WGN;
  return {tm * BM + wm * WM + i * 32 + (lane & 31), tn * BN + wn * WN + j * 32 + 16 * (lane >> 5)};
}

// Edge handling in the epilogue.  `full` (the same for the whole wave):
// every column of the wave's sub-tile is inside the matrix and the output
// allows 16-byte accesses, so no lane needs a per-element path.  It is
// tested first, as a branch of the whole wave.  On the other side the count
// of valid columns passes through an empty asm statement, which the
// compiler may not move or compute ahead of its branch: otherwise it
// evaluates the per-element column tests of every block in the common code
// and keeps them live in scalar registers, spilled, across the epilogue.
__device__ __forceinline__ int cols_left(int n) {
  asm volatile("" : "+v"(n));
  return n;
}

// The 16 saved bf16 activations at a lane's block position (zeros outside
// the matrix), as they are stored.
__device__ __forceinline__ void load_mask16(u32x4 (&m)[2], const bf16_t* __restrict__ src,
                                            int64_t ld, BlockPos p, int M, int N, bool vec,
                                            bool full) {
  m[0] = u32x4{0u, 0u, 0u, 0u};
  m[1] = m[0];
  if (p.row >= M) return;
  const bf16_t* q = src + (int64_t)p.row * ld + p.col;
  if (full) {
    m[0] = *reinterpret_cast<const u32x4*>(q);
    m[1] = *reinterpret_cast<const u32x4*>(q + 8);
    return;
  }
  const int lim = cols_left(N - p.col);
  if (vec && lim >= 16) {
    m[0] = *reinterpret_cast<const u32x4*>(q);
    m[1] = *reinterpret_cast<const u32x4*>(q + 8);
  } else {
#pragma unroll
    for (int c = 0; c < 16; ++c)
      if (c < lim) m[c >> 3][(c >> 1) & 3] |= (uint32_t)q[c] << (16 * (c & 1));
  }
}
template <int HK>
__device__ __forceinline__ float mask_at(const u32x4 (&m)[2], int c) {
  const uint32_t w = m[c >> 3][(c >> 1) & 3];
  return HalfOps<HK>::to_f32((c & 1) ? (w >> 16) : (w & 0xffffu));
}

// Orders this wave's LDS accesses (no other wave touches its region).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Writes a lane's 16 values (columns 16 h .. 16 h + 15 of block column j, row
// r of the region) in storage format.
template <typename TO, int WN, int HK>
__device__ __forceinline__ void region_put(char* region, int r, int j, int h, const float (&v)[16]) {
  constexpr int ES = sizeof(TO), PPR = WN * ES / 16;  // 16-byte pieces per row
  char* row = region + r * (WN * ES);
  if constexpr (ES == 2) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int q = 4 * j + 2 * h + k;
      using H = HalfOps<HK>;
      const u32x4 x = {H::pack2(v[8 * k], v[8 * k + 1]), H::pack2(v[8 * k + 2], v[8 * k + 3]),
                       H::pack2(v[8 * k + 4], v[8 * k + 5]), H::pack2(v[8 * k + 6], v[8 * k + 7])};
      *reinterpret_cast<u32x4*>(row + ((q ^ (r % PPR)) * 16)) = x;
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int q = 8 * j + 4 * h + k;
      *reinterpret_cast<f32x4*>(row + ((q ^ (r % PPR)) * 16)) =
          f32x4{v[4 * k], v[4 * k + 1], v[4 * k + 2], v[4 * k + 3]};
    }
  }
}

// Copies region rows 0 .. ROWS - 1 to out rows row0 .., columns col0 ..
// col0 + WN - 1 (clipped to M x N), one 16-byte piece per lane per step.
template <typename TO, int WN, int ROWS>
__device__ __forceinline__ void region_flush(const char* region, TO* __restrict__ out, int64_t ld,
                                             int row0, int col0, int M, int N, bool vec, bool full,
                                             int lane) {
  constexpr int ES = sizeof(TO), PPR = WN * ES / 16, EPP = 16 / ES, RPS = 64 / PPR;
  const int p = lane % PPR;
  const int col = col0 + p * EPP;
  if (full) {  // all columns inside: rows tested alone
#pragma unroll
    for (int t = 0; t < ROWS / RPS; ++t) {
      const int r = t * RPS + lane / PPR;
      const u32x4 x =
          *reinterpret_cast<const u32x4*>(region + r * (WN * ES) + ((p ^ (r % PPR)) * 16));
      if (row0 + r < M) *reinterpret_cast<u32x4*>(out + (int64_t)(row0 + r) * ld + col) = x;
    }
    return;
  }
  const int lim = cols_left(N - col);
#pragma unroll
  for (int t = 0; t < ROWS / RPS; ++t) {
    const int r = t * RPS + lane / PPR;
    const u32x4 x = *reinterpret_cast<const u32x4*>(region + r * (WN * ES) + ((p ^ (r % PPR)) * 16));
    const int row = row0 + r;
    if (row >= M || lim <= 0) continue;
    TO* q = out + (int64_t)row * ld + col;
    if (vec && lim >= EPP) {
      *reinterpret_cast<u32x4*>(q) = x;
    } else {
#pragma unroll
      for (int e = 0; e < EPP; ++e) {
        if (e >= lim) break;
        if constexpr (ES == 2) q[e] = (bf16_t)(x[e >> 1] >> (16 * (e & 1)));
        else q[e] = __uint_as_float(x[e]);
      }
    }
  }
}

// Largest power-of-two divisor of fm that is at most cap (at least 1).
constexpr int block_rows_per_round(int cap, int fm) {
  int r = 1;
  while (2 * r <= cap && fm % (2 * r) == 0) r *= 2;
  return r;
}

// Epilogue of one wave, on accumulators already passed through swap_halves:
// forward (bias, act; with ZOUT also Z = acc + bias), dX (times act' of the
// saved activations, read here one round ahead), or dW (float32, to C or to
// split `split`'s partial).  `region` is this wave's LDS area of kRegion
// bytes; the wave's rows go through it in rounds of IR block rows.
template <int BM, int BN, int WGM, int WGN, int EPI, int ACT, bool ZOUT, int FM, int FN,
          int kRegion, int HK>
__device__ __forceinline__ void store_epilogue(const f32x16 (&acc)[FM][FN], const GemmDesc& d,
                                               int tm, int tn, int split, int wm, int wn, int lane,
                                               bool vec, char* region) {
  using TO = typename std::conditional<EPI == EPI_DW, float, bf16_t>::type;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int ES = sizeof(TO);
  static_assert(WN == 32 * FN && WM == 32 * FM, "wave tile");
  constexpr bool kZ = ZOUT && EPI == EPI_FWD;
  constexpr int NOUT = kZ ? 2 : 1;
  constexpr int kOutBytes = kRegion / NOUT;  // region part of one output
  // (one block row per round when saved activations ride along, to bound
  // the registers they take)
  constexpr int IR = block_rows_per_round(
      EPI == EPI_DX && ACT != ACT_IDENTITY ? 1 : kOutBytes / (32 * WN * ES), FM);
  static_assert(kOutBytes >= 32 * WN * ES, "region too small for one block row");
  constexpr bool kMasked = EPI == EPI_DX && ACT != ACT_IDENTITY;
  const int M = d.M, N = d.N;
  const int h = lane >> 5, l32 = lane & 31;
  TO* __restrict__ out = static_cast<TO*>(d.C);
  int64_t ld = d.ldc;
  if (EPI == EPI_DW && d.splits > 1) {
    out = reinterpret_cast<TO*>(d.partial + (int64_t)split * M * N);
    ld = N;
  }
  const int row0 = tm * BM + wm * WM, col0 = tn * BN + wn * WN;
  // the same for every lane of the wave (tm, tn, wm, wn and the flags are)
  const bool full = vec && col0 + WN <= N;

  float bias[FN][16];
#pragma unroll
  for (int j = 0; j < FN; ++j)
#pragma unroll
    for (int c = 0; c < 16; ++c) bias[j][c] = 0.f;
  if (EPI == EPI_FWD && d.bias != nullptr) {
    const bool bias_vec = (reinterpret_cast<uintptr_t>(d.bias) & 15) == 0;
    auto bias16 = [&](int j, int col) {
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 x = *reinterpret_cast<const f32x4*>(d.bias + col + 4 * k);
        bias[j][4 * k] = x[0]; bias[j][4 * k + 1] = x[1];
        bias[j][4 * k + 2] = x[2]; bias[j][4 * k + 3] = x[3];
      }
    };
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = col0 + 32 * j + 16 * h;
      if (full && bias_vec) {
        bias16(j, col);
      } else {
        const int lim = cols_left(N - col);
        if (vec && lim >= 16 && bias_vec) {
          bias16(j, col);
        } else {
#pragma unroll
          for (int c = 0; c < 16; ++c)
            if (c < lim) bias[j][c] = d.bias[col + c];
        }
      }
    }
  }

  TO* __restrict__ zout = static_cast<TO*>(d.Z);
  const float osc = EPI == EPI_DW ? unscale_factor(d) : 1.0f;
  // saved activations of the current round's blocks (ii, j) at ii FN + j
  u32x4 mk[kMasked ? IR * FN : 1][2];
  auto load_masks = [&](int i0) {
#pragma unroll
    for (int ii = 0; ii < IR; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        load_mask16(mk[ii * FN + j], static_cast<const bf16_t*>(d.mask_src), d.ldc,
                    block_pos<BM, BN, WGM, WGN>(tm, tn, wm, wn, i0 + ii, j, lane), M, N, vec,
                    full);
  };
  if constexpr (kMasked) load_masks(0);
#pragma unroll
  for (int i0 = 0; i0 < FM; i0 += IR) {
#pragma unroll
    for (int ii = 0; ii < IR; ++ii)
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        float v[16];
#pragma unroll
        for (int c = 0; c < 16; ++c) v[c] = acc[i0 + ii][j][col_reg(c)];
        if constexpr (EPI == EPI_DW) {
#pragma unroll
          for (int c = 0; c < 16; ++c) v[c] *= osc;
        }
        if constexpr (EPI == EPI_FWD) {
          float z[16];
#pragma unroll
          for (int c = 0; c < 16; ++c) {
            z[c] = v[c] + bias[j][c];
            v[c] = act_apply(ACT, z[c]);
          }
          if constexpr (kZ) region_put<TO, WN, HK>(region + kOutBytes, ii * 32 + l32, j, h, z);
        } else if constexpr (kMasked) {
#pragma unroll
          for (int c = 0; c < 16; ++c) v[c] *= act_deriv(ACT, mask_at<HK>(mk[ii * FN + j], c));
        }
        region_put<TO, WN, HK>(region, ii * 32 + l32, j, h, v);
      }
    if constexpr (kMasked) {
      if (i0 + IR < FM) load_masks(i0 + IR);
    }
    wave_lds_order();
    region_flush<TO, WN, IR * 32>(region, out, ld, row0 + i0 * 32, col0, M, N, vec, full, lane);
    if constexpr (kZ)
      region_flush<TO, WN, IR * 32>(region + kOutBytes, zout, ld, row0 + i0 * 32, col0, M, N, vec,
                                    full, lane);
    wave_lds_order();
  }
}

// Work items are (split, tile) pairs, numbered in the XCD-aware band order
// of tile_coords.  Workgroup b of P takes its k-th item at item_pos(b, k):
// the 32 workgroups of one XCD walk that XCD's contiguous share of the items
// together, so they work on neighbouring tiles at any time.  -1: no more.
__device__ __forceinline__ int item_pos(int b, int k, int P, int T) {
  if ((P & 7) == 0 && (T & 7) == 0) {
    const int per = T >> 3, w = (b >> 3) + k * (P >> 3);
    return w < per ? (b & 7) * per + w : -1;
  }
  const int id = b + k * P;
  return id < T ? id : -1;
}

struct Item {
  int split, tm, tn, kbeg, nk;
};

// PERSIST: the grid holds one workgroup per CU and each walks several items
// with one continuous pipeline: the loads of the next item's first stages are
// issued during the current item's last stages, and the epilogue, which works
// in LDS regions of its own, runs while they land.  Otherwise the grid holds
// one workgroup per item and the epilogue reuses the stage buffers.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int ALAY, int BLAY, int EPI,
          bool PERSIST, int HK>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_bf16_dma_kernel(GemmDesc d, int tiles_m, int tiles_n, int out_vec) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int NW = NT / 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int KS = BK / 16;  // MFMA k-steps per stage
  static_assert(FM >= 1 && FN >= 1, "bad tile");
  static_assert(STAGES >= 2, "stages");
  static_assert(KS % 2 == 0, "fragment double buffer assumes an even k-step count");
  using OA = DmaOperand<BM, ALAY, NT, BK>;
  using OB = DmaOperand<BN, BLAY, NT, BK>;
  constexpr int kStageBytes = OA::kBytes + OB::kBytes;
  constexpr int kLoads = OA::kInst + OB::kInst;  // per wave per stage
  constexpr int kStageArea = STAGES * kStageBytes;
  constexpr int kRegion = PERSIST ? (kLdsBytes - kStageArea) / NW / 1024 * 1024 : kStageArea / NW;
  constexpr int kSmem = PERSIST ? kStageArea + NW * kRegion : kStageArea;
  static_assert(kSmem <= kLdsBytes, "LDS");
  __shared__ __attribute__((aligned(1024))) char smem[kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int h = lane >> 5;
  const int M = d.M, N = d.N;
  const int T = tiles_m * tiles_n * d.splits;
  const int P = gridDim.x, b = blockIdx.x;

  auto make_item = [&](int pos) {
    Item it;
    band_coords(pos, tiles_m, tiles_n, it.split, it.tm, it.tn);
    it.kbeg = it.split * d.k_per_split;
    const int kend = min(d.K, it.kbeg + d.k_per_split);
    it.nk = (kend - it.kbeg) / BK;
    return it;
  };

  // ---- loader: which item and stage the next issued loads belong to
  OA oa;
  OB ob;
  int ld_k = 0, ld_kt = 0, lg = 0;  // item index, its stage, global stage
  bool lpast = false;               // past the last stage of the last item
  Item ld = make_item(item_pos(b, 0, P, T));
  auto load_init = [&]() {
    oa.init(static_cast<const bf16_t*>(d.A), d.lda, ld.tm * BM, M, ld.kbeg, wave, lane);
    ob.init(static_cast<const bf16_t*>(d.B), d.ldb, ld.tn * BN, N, ld.kbeg, wave, lane);
  };
  load_init();
  // loads j0 .. j1 - 1 of global stage lg (A's loads first, then B's)
  auto issue_parts = [&](int j0, int j1) {
    char* p = smem + (lg % STAGES) * kStageBytes;
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      if (j < OA::kInst) oa.issue_one(p, wave, j);
      else ob.issue_one(p + OA::kBytes, wave, j - OA::kInst);
    }
  };
  auto next_load_stage = [&]() {
    ++lg;
    ++ld_kt;
    if (!lpast && ld_kt == ld.nk) {
      const int pos = PERSIST ? item_pos(b, ++ld_k, P, T) : -1;
      if (pos < 0) {
        lpast = true;
        oa.park();
        ob.park();
      } else {
        ld = make_item(pos);
        ld_kt = 0;
        load_init();
      }
    }
  };

  // ---- compute state
  Item cur = ld;
  int ck = 0;
  f32x16 acc[FM][FN];
  float dbacc[FM];
  auto clear_acc = [&]() {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      dbacc[i] = 0.f;
#pragma unroll
      for (int j = 0; j < FN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    }
  };
  clear_acc();
  const bool want_db = (EPI == EPI_DW) && (d.db != nullptr || d.db_partial != nullptr) && wn == 0;
  bool do_db = want_db && cur.tn == 0;

  auto read_frags = [&](const char* buf, int ks, bf16x8 (&a)[FM], bf16x8 (&bb)[FN]) {
#pragma unroll
    for (int i = 0; i < FM; ++i) a[i] = OA::frag(buf, wm * WM + i * 32, ks, lane);
#pragma unroll
    for (int j = 0; j < FN; ++j) bb[j] = OB::frag(buf + OA::kBytes, wn * WN + j * 32, ks, lane);
  };
  auto mfmas = [&](const bf16x8 (&a)[FM], const bf16x8 (&bb)[FN]) {
    if (do_db) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        float sum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += HalfOps<HK>::elem(a[i], e);
        dbacc[i] += sum;
      }
    }
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = HalfOps<HK>::mfma(bb[j], a[i], acc[i][j]);
  };
  auto stage_buf = [&](int g) { return smem + (g % STAGES) * kStageBytes; };

  // Fragments are double-buffered in registers (set ks & 1 holds k-step ks),
  // so the reads of one k-step are in flight while the MFMAs of the previous
  // one run.  The barrier of global stage g sits before its last k-step: by
  // then every wave holds its last fragments of stage g in registers, so
  // after the barrier the first fragments of stage g + 1 are read while the
  // last MFMAs of stage g run, and the matrix cores do not idle at the
  // barrier.  Each wave drains its LDS reads before that barrier, so once past
  // it no wave reads stage g's buffer again; the loads of stage g + STAGES
  // (same buffer), issued during stage g + 1, may then overwrite it.
  //
  // With three or more stages the loads of stage g + STAGES - 1 are spread
  // over the k-steps of stage g, interleaved with the MFMAs, and every stage
  // issues kLoads loads (repeats past the end), so at the barrier of stage g
  // the loads still allowed in flight are those of the stages after g + 1:
  // (STAGES - 2) kLoads minus the part of stage g + STAGES - 1 not yet
  // issued.  With two stages the loads of stage g + 1 all go first (they must
  // land by the barrier of stage g) and none are allowed in flight.  Stores
  // and saved-activation loads of an epilogue are younger than the loads of
  // the stage that follows it, so the next barrier also waits for them.
  bf16x8 fa[2][FM], fb[2][FN];
  constexpr int kReads = (ALAY == K_MAJOR ? FM : 2 * FM) + (BLAY == K_MAJOR ? FN : 2 * FN);
  constexpr int kMfma = FM * FN;
  // loads per k-step (three or more stages): kMid in each, the remainder in
  // the last
  constexpr int kMid = STAGES == 2 ? 0 : kLoads / KS;
  constexpr int kLast = STAGES == 2 ? 0 : kLoads - (KS - 1) * kMid;
  constexpr int kAllowed = (STAGES - 2) * kLoads - kLast;
  auto part = [](int ks) { return ks * kMid; };

  const bool vec = out_vec != 0;
  const int act = EPI == EPI_FWD ? d.act : EPI == EPI_DX ? d.mask_act : ACT_IDENTITY;
  char* region = smem + (PERSIST ? kStageArea : 0) + wave * kRegion;

#pragma unroll
  for (int st = 0; st < STAGES - 1; ++st) {
    issue_parts(0, kLoads);
    next_load_stage();
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((STAGES - 2) * kLoads));
  __builtin_amdgcn_s_barrier();
  read_frags(stage_buf(0), 0, fa[0], fb[0]);

  // One stage: k-steps, barrier, the rest of the next stage's loads; the
  // first fragments of the next stage are read unless LAST (the item's last
  // stage, after which the epilogue runs and the next item starts).
  int g = 0;
  auto run_stage = [&](auto last_tag) {
    constexpr bool LAST = decltype(last_tag)::value;
    const char* cbuf = stage_buf(g);
    if (STAGES == 2) {
      issue_parts(0, kLoads);
      next_load_stage();
    }
#pragma unroll
    for (int ks = 0; ks + 1 < KS; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
      if (STAGES > 2) issue_parts(part(ks), part(ks + 1));
      read_frags(cbuf, ks + 1, fa[(ks + 1) & 1], fb[(ks + 1) & 1]);
      mfmas(fa[ks & 1], fb[ks & 1]);
      sched_interleave<kMfma, kReads, kMid>();
      __builtin_amdgcn_sched_barrier(0);
    }
    // own reads of stage g complete; stage g + 1 landed for this wave
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(kAllowed));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    if (STAGES > 2) {
      issue_parts(part(KS - 1), kLoads);
      next_load_stage();
    }
    if (!LAST) read_frags(stage_buf(g + 1), 0, fa[0], fb[0]);
    mfmas(fa[1], fb[1]);
    sched_interleave<kMfma, kReads, LAST ? 0 : kLast>();
    __builtin_amdgcn_sched_barrier(0);
    ++g;
  };

  while (true) {
    for (int kt = 0; kt + 1 < cur.nk; ++kt) run_stage(std::false_type{});
    run_stage(std::true_type{});

    // ---- epilogue of item `cur`
    if (!PERSIST) {
      // the repeated loads past the last stage still write LDS, and other
      // waves may still read the stage buffers the regions reuse
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __syncthreads();
    }
    if (EPI == EPI_DW && do_db) {
      const int row_base = cur.tm * BM + wm * WM;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const float v = (dbacc[i] + __shfl_xor(dbacc[i], 32)) * unscale_factor(d);
        const int row = row_base + i * 32 + (lane & 31);
        if (h == 0 && row < M) {
          if (d.splits > 1) d.db_partial[(int64_t)cur.split * M + row] = v;
          else d.db[row] = v;
        }
      }
    }
    swap_halves(acc);
#define DL_EPILOGUE(A, Z)                                                                 \
  store_epilogue<BM, BN, WGM, WGN, EPI, A, Z, FM, FN, kRegion, HK>(                       \
      acc, d, cur.tm, cur.tn, cur.split, wm, wn, lane, vec, region)
    if (EPI == EPI_FWD && d.Z != nullptr) {
      if constexpr (EPI != EPI_FWD) {
      } else if (act == ACT_GELU_TANH) DL_EPILOGUE(ACT_GELU_TANH, true);
      else if (act == ACT_RELU) DL_EPILOGUE(ACT_RELU, true);
      else DL_EPILOGUE(ACT_IDENTITY, true);
    } else {
      if (act == ACT_GELU_TANH) DL_EPILOGUE(ACT_GELU_TANH, false);
      else if (act == ACT_RELU) DL_EPILOGUE(ACT_RELU, false);
      else DL_EPILOGUE(ACT_IDENTITY, false);
    }
#undef DL_EPILOGUE

    // ---- next item: its first stage landed before the last barrier
    const int pos = item_pos(b, ++ck, P, T);
    if (!PERSIST || pos < 0) break;
    cur = make_item(pos);
    do_db = want_db && cur.tn == 0;
    clear_acc();
    read_frags(stage_buf(g), 0, fa[0], fb[0]);
  }
  // nothing may still write this workgroup's LDS when it retires
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int ALAY, int BLAY, int EPI,
          bool PERSIST, int HK>
hipError_t launch_dma(const GemmDesc& d, hipStream_t s) {
  auto aligned = [](const void* p, int64_t ld) {
    return ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (ld % 8 == 0);
  };
  if (!aligned(d.A, d.lda) || !aligned(d.B, d.ldb)) return hipErrorNotSupported;
  if (d.K % 64 != 0 || d.k_per_split % 64 != 0 || d.k_per_split <= 0) return hipErrorNotSupported;
  if (ALAY == MN_MAJOR && d.M % 8 != 0) return hipErrorNotSupported;
  if (BLAY == MN_MAJOR && d.N % 8 != 0) return hipErrorNotSupported;
  const int tiles_m = (d.M + BM - 1) / BM;
  const int tiles_n = (d.N + BN - 1) / BN;
  const int64_t items = (int64_t)tiles_m * tiles_n * d.splits;
  if (items <= 0 || items > 0x7fffffff) return hipErrorInvalidValue;
  int64_t nwg = items;
  if (PERSIST) {  // one workgroup per CU (the kernel's LDS admits no more)
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    nwg = std::min<int64_t>(items, std::max(cus, 1));
  }
  auto out_ok = [](const void* p, int64_t ld, int bytes) {
    return ((reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0) && (ld % 4 == 0);
  };
  int out_vec;
  if (EPI == EPI_DW)
    out_vec = d.splits > 1 ? out_ok(d.partial, d.N, 16) : out_ok(d.C, d.ldc, 16);
  else
    out_vec = out_ok(d.C, d.ldc, 16) && d.ldc % 8 == 0 &&
              (d.Z == nullptr || out_ok(d.Z, d.ldc, 16)) &&
              (d.mask_src == nullptr || out_ok(d.mask_src, d.ldc, 16));
  hipLaunchKernelGGL((gemm_bf16_dma_kernel<BM, BN, BK, STAGES, WGM, WGN, ALAY, BLAY, EPI, PERSIST, HK>),
                     dim3((unsigned)nwg), dim3(WGM * WGN * 64), 0, s, d, tiles_m, tiles_n,
                     out_vec);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, bool PERSIST, int HK>
hipError_t dma_layout(const GemmDesc& d, hipStream_t s) {
  if (d.epi == EPI_FWD && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_dma<BM, BN, BK, STAGES, WGM, WGN, K_MAJOR, K_MAJOR, EPI_FWD, PERSIST, HK>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_dma<BM, BN, BK, STAGES, WGM, WGN, K_MAJOR, K_MAJOR, EPI_DX, PERSIST, HK>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == MN_MAJOR)
    return launch_dma<BM, BN, BK, STAGES, WGM, WGN, K_MAJOR, MN_MAJOR, EPI_DX, PERSIST, HK>(d, s);
  return hipErrorNotSupported;  // weight gradients run the register-staged kernel
}

}  // namespace

// The 256x256 tile runs persistent (three stages, separate epilogue LDS)
// when every CU gets at least kPersistItems items: there the pipeline fill
// and the epilogue of each item are the costs it hides.  With fewer items per
// CU the one-workgroup-per-item form with four stages measured faster.
constexpr int kPersistItems = 4;

template <int HK>
hipError_t launch_tile(const GemmDesc& d, int tile, hipStream_t s) {
  switch (tile) {
    case 0: {
      int dev = 0, cus = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
      const int64_t items = (int64_t)((d.M + 255) / 256) * ((d.N + 255) / 256) * d.splits;
      if (items >= (int64_t)kPersistItems * cus) return dma_layout<256, 256, 32, 3, 2, 4, true, HK>(d, s);
      return dma_layout<256, 256, 32, 4, 2, 4, false, HK>(d, s);
    }
    case 1: return dma_layout<128, 128, 64, 2, 2, 2, false, HK>(d, s);
    default: return hipErrorNotSupported;
  }
}

hipError_t launch_gemm_bf16_dma(const GemmDesc& d, int tile, hipStream_t s) {
  return d.half_kind == HK_F16 ? launch_tile<HK_F16>(d, tile, s) : launch_tile<HK_BF16>(d, tile, s);
}

}  // namespace dl

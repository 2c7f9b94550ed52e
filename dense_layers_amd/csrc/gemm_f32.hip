// Float32 GEMM on the CDNA4 matrix cores (v_mfma_f32_32x32x2_f32) with the
// dense-layer epilogues fused in.
//
// One kernel template covers the three products of a dense layer:
//   forward  Z = X W^T        A = X  [B, in]  K-major, B = W [out, in] K-major
//   dX       dX = G W         A = G  [B, out] K-major, B = W [out, in] N-major
//   dW       dW = G^T X       A = G  [B, out] M-major, B = X [B, in]   N-major
// (the fused Linear / LinearAct of the noeira.nn docs, "The design in one
// page", with bias and activation in the GEMM epilogue, and split-K for the
// long-K weight gradient as in its package layout's split-K GEMM).
//
// Structure: a workgroup of WGM x WGN waves owns a BM x BN output tile; each
// wave owns a (BM/WGM) x (BN/WGN) sub-tile made of 32x32 MFMA blocks whose
// accumulators stay in registers for the whole K loop.  Operand tiles go
// global -> registers -> LDS (double-buffered, one barrier per K step); the
// global loads of the K step two ahead are issued before the current step's
// MFMAs so their latency hides behind the matrix work.  LDS keeps the global layout
// (no transpose on the store side); fragments are read as one 16-byte load
// (K-major) or four 4-byte loads (M/N-major).
//
// The sum over k inside an MFMA does not depend on which k each lane
// supplies, as long as A and B agree.  Within a group of 8 k values, lane
// half h (lanes 0-31 / 32-63) supplies k = 4h + s at MFMA step s, so a
// K-major fragment is 4 consecutive floats.
#include "common.hpp"

namespace dl {
namespace {

constexpr int kPad = 4;  // floats of padding per LDS row

// XF: the operand holds logits [batch rows, classes] of a fused classifier
// head and is turned into the softmax cross-entropy gradient
//   g = (exp(z - lse[i]) - [c == label[i]]) * invB
// on its way to LDS (in store(), when the loads have landed, so the loads
// of the next K step stay in flight meanwhile).  Each float4 holds four
// classes of one batch row: for a K-major operand (dX = G W) the batch row
// is the tile row and the classes run along K; for an M-major operand
// (dW = G^T X) the batch row is the K index and the classes are the tile
// rows.  Each batch row's (exponent offset, label) pair comes from an 8-byte
// record (xent_rows): for a K-major operand the rows do not change along K
// and the records are loaded once per tile (prime), for an M-major operand
// one record per vector is loaded with the logits.  Elements past the K
// range (zero-filled by the bounds-checked load) stay zero.
template <int ROWS, int BK, int LAY, int NT, bool XF = false>
struct TileLoader {
  // A tile is ROWS (M or N) x BK (K) elements, moved as float4 vectors.
  static constexpr int kVecs = ROWS * BK / 4;
  static_assert(kVecs % NT == 0, "tile not divisible among threads");
  static constexpr int kPer = kVecs / NT;
  static constexpr int kLdsStride = (LAY == K_MAJOR) ? (BK + kPad) : (ROWS + kPad);
  static constexpr int kLdsSize = (LAY == K_MAJOR) ? ROWS * (BK + kPad) : BK * (ROWS + kPad);

  f32x4 r[kPer];
  // XF state: the batch row's exponent offset (lse log2 e + log2 B) and
  // label per vector, the K range and first tile row of the last load, and
  // the operand's constants.
  float xl[XF ? kPer : 1];
  int xy[XF ? kPer : 1];
  int xk0 = 0, xkend = 0, xrow0 = 0;
  bool xsafe = false;
  const f32x2* xrec = nullptr;
  float xinvB = 0.f;

  __device__ __forceinline__ void bind(const GemmDesc& d) {
    xrec = reinterpret_cast<const f32x2*>(d.xent_rows);
    xinvB = d.xent_invB;
  }

  // (offset, label) of vector i's batch row (XF only); `brow` is in range.
  __device__ __forceinline__ void load_row_stats(int i, int brow) {
    const f32x2 rec = xrec[brow];
    xl[i] = rec[0];
    xy[i] = __float_as_int(rec[1]);
  }

  // K-major XF operand: the batch rows of this thread's vectors for the
  // tile starting at row0 (the same in every K step).
  __device__ __forceinline__ void prime(int row0, int nrows, int tid) {
    if (!XF || LAY != K_MAJOR) return;
#pragma unroll
    for (int i = 0; i < kPer; ++i) load_row_stats(i, min(row0 + vec(i, tid) / (BK / 4), nrows - 1));
  }

  // Which vector of the tile load i of thread tid moves.  In general
  // consecutive threads take consecutive vectors (tid + i NT).  An M-major
  // XF operand instead gives each group of kVPR threads (one k-row's
  // vectors) kPer consecutive k-rows, so a thread's vectors lie in adjacent
  // batch rows and one load brings all their records.  Only which thread
  // moves a vector changes: the LDS tile is the same.
  static constexpr int kVPR = ROWS / 4;  // vectors per k-row (M-major)
  static constexpr bool kGroupK = XF && LAY == MN_MAJOR;
  static_assert(!kGroupK || (NT % kVPR == 0 && (NT / kVPR) * kPer == BK && kPer <= 2),
                "grouped k-rows");
  __device__ __forceinline__ static int vec(int i, int tid) {
    return kGroupK ? (tid % kVPR) + kVPR * (kPer * (tid / kVPR) + i) : tid + i * NT;
  }

  // M-major XF operand: the records of this thread's kPer consecutive batch
  // rows from k0 on, in one load (the record buffer holds one spare record
  // past the batch, so the pair may reach one row past kend).
  __device__ __forceinline__ void load_group_stats(int k0, int kend, int tid) {
    const int kb = min(k0 + kPer * (tid / kVPR), kend - 1);
    if constexpr (XF && kPer == 2) {
      const f32x4 rec = *reinterpret_cast<const f32x4*>(xrec + kb);
      xl[0] = rec[0];
      xy[0] = __float_as_int(rec[1]);
      xl[1] = rec[2];
      xy[1] = __float_as_int(rec[3]);
    } else {
      load_row_stats(0, kb);
    }
  }

  // The per-thread part of the full K steps' load addresses, fixed for a
  // tile: vector i's row and k offset at k = 0 (K-major), or its k row and
  // first tile row (M/N-major).  A K step then adds k0, or k0 ld, which the
  // whole workgroup shares, instead of forming each address's 64-bit
  // product again.  Rows past the end (edge tiles) are clamped to a valid
  // row: they only feed output rows / columns that are never stored.  For
  // an M/N-major operand this needs nrows % 4 == 0 so that no vector
  // straddles the end (checked by the caller).
  struct Origin {
    const float* p[kPer];
  };
  __device__ __forceinline__ static Origin origin(const float* __restrict__ base, int64_t ld,
                                                  int row0, int nrows, int tid) {
    Origin o;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = vec(i, tid);
      if (LAY == K_MAJOR) {
        const int row = min(row0 + v / (BK / 4), nrows - 1);
        o.p[i] = base + (int64_t)row * ld + (v % (BK / 4)) * 4;
      } else {
        int row = row0 + (v % (ROWS / 4)) * 4;
        row = row < nrows ? row : 0;
        o.p[i] = base + (int64_t)(v / (ROWS / 4)) * ld + row;
      }
    }
    return o;
  }

  // Full K step, 16-byte aligned rows: plain vector loads with no
  // per-element control flow, so the loads of a K step stay in flight
  // together.  `row0` is the tile's first row, as given to origin().
  __device__ __forceinline__ void load_fast(const Origin& o, int64_t ld, int row0, int k0,
                                            int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      if (LAY == K_MAJOR) r[i] = *reinterpret_cast<const f32x4*>(o.p[i] + k0);
      else r[i] = *reinterpret_cast<const f32x4*>(o.p[i] + (int64_t)k0 * ld);
    }
    if (XF) {
      if (kGroupK) load_group_stats(k0, k0 + BK, tid);
      xk0 = k0;
      xkend = k0 + BK;
      xrow0 = row0;
      xsafe = false;
    }
  }

  // The same loads with every address formed in full.
  __device__ __forceinline__ void load_fast(const float* __restrict__ base, int64_t ld,
                                            int row0, int nrows, int k0, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = vec(i, tid);
      if (LAY == K_MAJOR) {
        const int row = min(row0 + v / (BK / 4), nrows - 1);
        const int k = k0 + (v % (BK / 4)) * 4;
        r[i] = *reinterpret_cast<const f32x4*>(base + (int64_t)row * ld + k);
      } else {
        const int k = k0 + v / (ROWS / 4);
        int row = row0 + (v % (ROWS / 4)) * 4;
        row = row < nrows ? row : 0;
        r[i] = *reinterpret_cast<const f32x4*>(base + (int64_t)k * ld + row);
      }
    }
    if (XF) {
      if (kGroupK) load_group_stats(k0, k0 + BK, tid);
      xk0 = k0;
      xkend = k0 + BK;
      xrow0 = row0;
      xsafe = false;
    }
  }

  // Edge tiles: element loads, zero outside [0, nrows) x [k0, kend).
  __device__ __forceinline__ void load_safe(const float* __restrict__ base, int64_t ld,
                                            int row0, int nrows, int k0, int kend, int tid) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = vec(i, tid);
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (LAY == K_MAJOR) {
        const int row = row0 + v / (BK / 4);
        const int k = k0 + (v % (BK / 4)) * 4;
        if (row < nrows) {
          const float* p = base + (int64_t)row * ld + k;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (k + j < kend) x[j] = p[j];
        }
      } else {
        const int k = k0 + v / (ROWS / 4);
        const int row = row0 + (v % (ROWS / 4)) * 4;
        if (k < kend) {
          const float* p = base + (int64_t)k * ld + row;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (row + j < nrows) x[j] = p[j];
        }
      }
      r[i] = x;
    }
    if (XF) {
      if (kGroupK) load_group_stats(k0, kend, tid);
      xk0 = k0;
      xkend = kend;
      xrow0 = row0;
      xsafe = true;
    }
  }

  // XF: the loss gradient of vector i (see the struct comment), formed as
  // one base-2 exponential per element: exp(z - lse) / B =
  // 2^(z log2(e) - (lse log2(e) + log2 B)) with the row's offset from its
  // record; the one-hot lands on at most one element of a vector.
  __device__ __forceinline__ f32x4 xent_grad(int i, int v) const {
    constexpr float kLog2e = 1.4426950408889634f;
    f32x4 x = r[i];
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = __builtin_amdgcn_exp2f(fmaf(x[j], kLog2e, -xl[i]));
    const int c0 = LAY == K_MAJOR ? xk0 + (v % (BK / 4)) * 4 : xrow0 + (v % (ROWS / 4)) * 4;
    const unsigned dj = (unsigned)(xy[i] - c0);
    if (dj < 4u) {  // the label is one of these 4 classes: rare, so a branch
#pragma unroll
      for (int j = 0; j < 4; ++j) x[j] = dj == (unsigned)j ? x[j] - xinvB : x[j];
    }
    if (xsafe) {  // bounds-checked load: elements past the K range stay zero
      if (LAY == K_MAJOR) {
#pragma unroll
        for (int j = 0; j < 4; ++j) x[j] = c0 + j < xkend ? x[j] : 0.0f;
      } else if (xk0 + v / (ROWS / 4) >= xkend) {
        x = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return x;
  }

  __device__ __forceinline__ void store(float* __restrict__ lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int v = vec(i, tid);
      int off;
      if (LAY == K_MAJOR)
        off = (v / (BK / 4)) * kLdsStride + (v % (BK / 4)) * 4;
      else
        off = (v / (ROWS / 4)) * kLdsStride + (v % (ROWS / 4)) * 4;
      *reinterpret_cast<f32x4*>(lds + off) = XF ? xent_grad(i, v) : r[i];
    }
  }

  // Fragment for a 32-row MFMA block starting at tile row `row` (this lane's
  // row already added), k group kg (8 values), lane half h.
  __device__ __forceinline__ void frag(const float* __restrict__ lds, int row,
                                       int kg, int h, float out[4]) const {
    if (LAY == K_MAJOR) {
      f32x4 x = *reinterpret_cast<const f32x4*>(lds + row * kLdsStride + kg * 8 + h * 4);
      out[0] = x[0]; out[1] = x[1]; out[2] = x[2]; out[3] = x[3];
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) out[s] = lds[(kg * 8 + h * 4 + s) * kLdsStride + row];
    }
  }
};

// LDS floats of one workgroup: two stages of both operand tiles, or the
// epilogue's staging tile, whichever is larger.
template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY>
constexpr int f32_smem_floats() {
  constexpr int NT = WGM * WGN * 64;
  constexpr int ab = 2 * TileLoader<BM, BK, ALAY, NT>::kLdsSize + 2 * TileLoader<BN, BK, BLAY, NT>::kLdsSize;
  constexpr int st = stage_floats<BM, BN, WGM>();
  return ab > st ? ab : st;
}

// One output tile (K slice `split`, tile row tm, tile column tn) of the
// GEMM `d`, LDS at `smem`.
template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY, int EPI, bool XF = false>
__device__ __forceinline__ void gemm_f32_tile(const GemmDesc& d, int split, int tm, int tn,
                                              int a_vec, int b_vec, int out_vec, float* smem) {
  constexpr int NT = WGM * WGN * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  static_assert(FM >= 1 && FN >= 1 && BK % 8 == 0, "bad tile");
  using LA = TileLoader<BM, BK, ALAY, NT, XF>;
  using LB = TileLoader<BN, BK, BLAY, NT>;
  // buffer b of A at smem + b * LA::kLdsSize, of B after both A buffers
  auto As = [&](int b) { return smem + b * LA::kLdsSize; };
  auto Bs = [&](int b) { return smem + 2 * LA::kLdsSize + b * LB::kLdsSize; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l32 = lane & 31, h = lane >> 5;

  const int M = d.M, N = d.N;
  const int kbeg = split * d.k_per_split;
  const int kend = min(d.K, kbeg + d.k_per_split);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

  const float* __restrict__ A = static_cast<const float*>(d.A);
  const float* __restrict__ B = static_cast<const float*>(d.B);

  LA la;
  LB lb;
  if (XF) {
    la.bind(d);
    la.prime(tm * BM, M, tid);
  }
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
  const bool fast = a_vec && b_vec && (ALAY == K_MAJOR || M % 4 == 0) &&
                    (BLAY == K_MAJOR || N % 4 == 0);
  const int nk_full = fast ? (kend - kbeg) / BK : 0;

  auto compute = [&](int cur) {
#pragma unroll
    for (int kg = 0; kg < BK / 8; ++kg) {
      float a[FM][4], b[FN][4];
#pragma unroll
      for (int i = 0; i < FM; ++i) la.frag(As(cur), wm * WM + i * 32 + l32, kg, h, a[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) lb.frag(Bs(cur), wn * WN + j * 32 + l32, kg, h, b[j]);
      if (do_db) {
#pragma unroll
        for (int i = 0; i < FM; ++i) dbacc[i] += (a[i][0] + a[i][1]) + (a[i][2] + a[i][3]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][s], b[j][s], acc[i][j], 0, 0, 0);
    }
  };
  // The same K step with every fragment read issued first and `mid` (the
  // LDS stores of a later step's operands) placed after the first k group's
  // MFMAs, so a wait for those operands' loads overlaps matrix work.
  auto compute_mid = [&](int cur, auto&& mid) {
    float a[BK / 8][FM][4], b[BK / 8][FN][4];
#pragma unroll
    for (int kg = 0; kg < BK / 8; ++kg) {
#pragma unroll
      for (int i = 0; i < FM; ++i) la.frag(As(cur), wm * WM + i * 32 + l32, kg, h, a[kg][i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) lb.frag(Bs(cur), wn * WN + j * 32 + l32, kg, h, b[kg][j]);
    }
#pragma unroll
    for (int kg = 0; kg < BK / 8; ++kg) {
      if (do_db) {
#pragma unroll
        for (int i = 0; i < FM; ++i)
          dbacc[i] += (a[kg][i][0] + a[kg][i][1]) + (a[kg][i][2] + a[kg][i][3]);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[kg][i][s], b[kg][j][s], acc[i][j],
                                                             0, 0, 0);
      if (kg == 0) {
        __builtin_amdgcn_sched_barrier(0);
        mid();
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Loads run two K steps ahead: register set 1 (la, lb) and set 2 (la2,
  // lb2) alternate, so each load has two steps of MFMA work to land in.
  // Invariant at the top of a trip: LDS buffer (kt & 1) holds step kt and
  // set 2 holds step kt + 1 in flight.
  LA la2;
  LB lb2;
  if (XF) {
    la2.bind(d);
    la2.prime(tm * BM, M, tid);
  }
  // Full K steps load from per-tile origins, except in the loss-gradient
  // products (XF), whose loads form every address in full: their walking
  // kernel has no registers to spare, and the origins measured slower there.
  struct NoOrigin {};
  using OA = typename std::conditional<XF, NoOrigin, typename LA::Origin>::type;
  using OB = typename std::conditional<XF, NoOrigin, typename LB::Origin>::type;
  OA oa;
  OB ob;
  if constexpr (!XF) {
    oa = LA::origin(A, d.lda, tm * BM, M, tid);
    ob = LB::origin(B, d.ldb, tn * BN, N, tid);
  }
#define DL_FAST_A(l, k0)                                                    \
  do {                                                                      \
    if constexpr (XF) l.load_fast(A, d.lda, tm * BM, M, k0, tid);           \
    else l.load_fast(oa, d.lda, tm * BM, k0, tid);                          \
  } while (0)
#define DL_FAST_B(l, k0)                                                    \
  do {                                                                      \
    if constexpr (XF) l.load_fast(B, d.ldb, tn * BN, N, k0, tid);           \
    else l.load_fast(ob, d.ldb, tn * BN, k0, tid);                          \
  } while (0)
  if (nk > 0) {
    if (nk_full > 0) {
      DL_FAST_A(la, kbeg);
      DL_FAST_B(lb, kbeg);
    } else {
      la.load_safe(A, d.lda, tm * BM, M, kbeg, kend, tid);
      lb.load_safe(B, d.ldb, tn * BN, N, kbeg, kend, tid);
    }
    la.store(As(0), tid);
    lb.store(Bs(0), tid);
    if (nk_full >= 2) {
      DL_FAST_A(la2, kbeg + BK);
      DL_FAST_B(lb2, kbeg + BK);
    }
  }
  __syncthreads();

  // Each half of a trip stores the register set loaded one half earlier into
  // the buffer the other half reads (the data has had a whole half to land),
  // and the stores no longer sit between the MFMAs and the barrier.  The
  // barrier at the end of each half orders every wave's reads of a buffer
  // before the next stores into it.  Forward-shaped products (both operands
  // K-major, K step 16) place those stores after the first k group's MFMAs,
  // so that a wait for their loads overlaps matrix work (measured: the wide
  // MLP's 4096-wide forwards 1.4% and the classifier head's forward 2.7%
  // faster); the other products store before their MFMAs (the later
  // placement measured 6% slower for the head's weight gradient and slower
  // for the 64 x 128 tile).
  int kt = 0;
  constexpr bool kMid = BK == 16 && ALAY == K_MAJOR && BLAY == K_MAJOR && !XF;
  for (; kt + 3 < nk_full; kt += 2) {
    DL_FAST_A(la, kbeg + (kt + 2) * BK);
    DL_FAST_B(lb, kbeg + (kt + 2) * BK);
    // keep the loads ahead of the MFMAs (the scheduler would otherwise sink
    // them next to their LDS stores)
    __builtin_amdgcn_sched_barrier(0);
    if (kMid) {
      compute_mid(0, [&] {
        la2.store(As(1), tid);
        lb2.store(Bs(1), tid);
      });
    } else {
      la2.store(As(1), tid);
      lb2.store(Bs(1), tid);
      __builtin_amdgcn_sched_barrier(0);
      compute(0);
    }
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    DL_FAST_A(la2, kbeg + (kt + 3) * BK);
    DL_FAST_B(lb2, kbeg + (kt + 3) * BK);
    __builtin_amdgcn_sched_barrier(0);
    if (kMid) {
      compute_mid(1, [&] {
        la.store(As(0), tid);
        lb.store(Bs(0), tid);
      });
    } else {
      la.store(As(0), tid);
      lb.store(Bs(0), tid);
      __builtin_amdgcn_sched_barrier(0);
      compute(1);
    }
    __builtin_amdgcn_sched_barrier(0);
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
    DL_FAST_A(la, k0);
    DL_FAST_B(lb, k0);
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
#undef DL_FAST_A
#undef DL_FAST_B

  // ---- epilogue -------------------------------------------------------------
  if (EPI == EPI_DW && do_db) {
    const int row_base = tm * BM + wm * WM;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      float v = (dbacc[i] + __shfl_xor(dbacc[i], 32)) * unscale_factor(d);
      const int row = row_base + i * 32 + l32;
      if (h == 0 && row < M) {
        if (d.splits > 1) {
          d.db_partial[(int64_t)split * M + row] = v;
        } else {
          d.db[row] = v;
          if (d.sgd_b != nullptr) d.sgd_b[row] -= d.sgd_lr * v;
        }
      }
    }
  }
  store_tile<float, BM, BN, WGM, WGN, EPI>(acc, smem, d, tm, tn, split, out_vec);
}

// Workgroup `wg` of `nwg` working on the GEMM `d`: its tile in the XCD-aware
// band order of tile_coords.
template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY, int EPI, bool XF = false>
__device__ __forceinline__ void gemm_f32_body(const GemmDesc& d, int tiles_m, int tiles_n,
                                              int a_vec, int b_vec, int out_vec, int wg, int nwg,
                                              float* smem) {
  int split, tm, tn;
  tile_coords_at(wg, nwg, tiles_m, tiles_n, split, tm, tn);
  gemm_f32_tile<BM, BN, BK, WGM, WGN, ALAY, BLAY, EPI, XF>(d, split, tm, tn, a_vec, b_vec,
                                                           out_vec, smem);
}

template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY, int EPI, bool XF = false>
__global__ void __launch_bounds__(WGM * WGN * 64)
gemm_f32_kernel(GemmDesc d, int tiles_m, int tiles_n, int a_vec, int b_vec, int out_vec) {
  __shared__ __attribute__((aligned(16))) float smem[f32_smem_floats<BM, BN, BK, WGM, WGN, ALAY, BLAY>()];
  gemm_f32_body<BM, BN, BK, WGM, WGN, ALAY, BLAY, EPI, XF>(d, tiles_m, tiles_n, a_vec, b_vec,
                                                           out_vec, blockIdx.x, gridDim.x, smem);
}

// Waves per SIMD the walking grid is sized for (the tiles it runs fit two in
// registers and LDS): two workgroups of 4 waves, or one of 8, per CU.
constexpr int kRowsWaves = 2;

// Long-K products with few tile columns (the classifier head's dX and dW,
// K = 32000 and 65536 over N = 768): a grid the chip holds at once (a
// multiple of 8 workgroups, kRowsWaves waves per SIMD), each walking tiles.
// Workgroup b runs on XCD b % 8, and the workgroups of XCD x take, round
// after round, the tiles of tile rows x, x + 8, x + 16, ... in row order, so
// the tiles of one row (which read the same A rows over the whole K loop)
// run side by side on one XCD and meet that operand in its L2.  In a grid of
// one workgroup per tile they drift apart as workgroups of later dispatch
// rounds start whenever a slot frees.  One K slice.
template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY, int EPI, bool XF = false>
__global__ void __launch_bounds__(WGM * WGN * 64, kRowsWaves)
gemm_f32_rows_kernel(GemmDesc d, int tiles_m, int tiles_n, int a_vec, int b_vec, int out_vec) {
  __shared__ __attribute__((aligned(16))) float smem[f32_smem_floats<BM, BN, BK, WGM, WGN, ALAY, BLAY>()];
  const int x = blockIdx.x & 7, per = gridDim.x >> 3;
  for (int q = blockIdx.x >> 3;; q += per) {
    const int tm = x + 8 * (q / tiles_n), tn = q % tiles_n;
    if (tm >= tiles_m) break;
    gemm_f32_tile<BM, BN, BK, WGM, WGN, ALAY, BLAY, EPI, XF>(d, 0, tm, tn, a_vec, b_vec, out_vec,
                                                             smem);
    __syncthreads();  // the epilogue's LDS reads before the next tile's stores
  }
}

// Two small products in one launch (64x64 tiles of 4 waves for both):
// workgroups [0, a.nwg) take the weight-gradient items of job a, the next
// b.nwg the items of job b (the same layer's dX, or another layer's weight
// gradient).  The two products only read common inputs, so they may run side
// by side; neither may write over the other's inputs.  With fin.W set, more
// workgroups take the loss mean and the SGD step of a third layer from its
// gradient slices (the weight gradients then take their own SGD steps in the
// epilogue).
struct F32Job {
  GemmDesc d;
  int tiles_m, tiles_n, a_vec, b_vec, out_vec, nwg;
};
template <int ALAY2, int BLAY2, int EPI2>
__global__ void __launch_bounds__(256)
gemm_f32_pair_kernel(F32Job a, F32Job b, SgdFinish fin) {
  constexpr int kA = f32_smem_floats<64, 64, 32, 2, 2, MN_MAJOR, MN_MAJOR>();
  constexpr int kB = f32_smem_floats<64, 64, 32, 2, 2, ALAY2, BLAY2>();
  __shared__ __attribute__((aligned(16))) float smem[kA > kB ? kA : kB];
  const int w = blockIdx.x;
  if (w < a.nwg)
    gemm_f32_body<64, 64, 32, 2, 2, MN_MAJOR, MN_MAJOR, EPI_DW>(
        a.d, a.tiles_m, a.tiles_n, a.a_vec, a.b_vec, a.out_vec, w, a.nwg, smem);
  else if (w < a.nwg + b.nwg)
    gemm_f32_body<64, 64, 32, 2, 2, ALAY2, BLAY2, EPI2>(
        b.d, b.tiles_m, b.tiles_n, b.a_vec, b.b_vec, b.out_vec, w - a.nwg, b.nwg, smem);
  else
    sgd_finish_block(fin, w - a.nwg - b.nwg);
}

// Grid shape and vector-access flags of one GEMM on a BM x BN tile.
template <int BM, int BN>
hipError_t make_job(const GemmDesc& d, F32Job& j) {
  j.d = d;
  j.tiles_m = (d.M + BM - 1) / BM;
  j.tiles_n = (d.N + BN - 1) / BN;
  const int64_t nwg = (int64_t)j.tiles_m * j.tiles_n * d.splits;
  if (nwg <= 0 || nwg > 0x3fffffff) return hipErrorInvalidValue;
  j.nwg = (int)nwg;
  auto aligned = [](const void* p, int64_t ld) {
    return ((reinterpret_cast<uintptr_t>(p) & 15) == 0) && (ld % 4 == 0);
  };
  j.a_vec = aligned(d.A, d.lda);
  j.b_vec = aligned(d.B, d.ldb);
  if (d.epi == EPI_DW && d.splits > 1)
    j.out_vec = aligned(d.partial, d.N);
  else
    j.out_vec = aligned(d.C, d.ldc) && (d.Z == nullptr || aligned(d.Z, d.ldc)) &&
                (d.mask_src == nullptr || aligned(d.mask_src, d.ldc));
  return hipSuccess;
}

hipError_t cu_count(int& cus) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  return e;
}

template <int BM, int BN, int BK, int WGM, int WGN, int ALAY, int BLAY, int EPI, bool XF = false>
hipError_t launch_tile(const GemmDesc& d, hipStream_t s) {
  F32Job j;
  const hipError_t e = make_job<BM, BN>(d, j);
  if (e != hipSuccess) return e;
  if constexpr (XF && BM == 128 && (BN == 128 || BN == 256)) {
    int cus = 0;
    const hipError_t e2 = cu_count(cus);
    if (e2 != hipSuccess) return e2;
    const int64_t slots = (int64_t)(kRowsWaves * 4 / (WGM * WGN)) * cus / 8 * 8;
    if (d.splits == 1 && slots >= 8 && j.nwg > slots) {
      hipLaunchKernelGGL((gemm_f32_rows_kernel<BM, BN, BK, WGM, WGN, ALAY, BLAY, EPI, XF>),
                         dim3((unsigned)slots), dim3(WGM * WGN * 64), 0, s, d, j.tiles_m,
                         j.tiles_n, j.a_vec, j.b_vec, j.out_vec);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_f32_kernel<BM, BN, BK, WGM, WGN, ALAY, BLAY, EPI, XF>),
                     dim3((unsigned)j.nwg), dim3(WGM * WGN * 64), 0, s, d, j.tiles_m,
                     j.tiles_n, j.a_vec, j.b_vec, j.out_vec);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WGM, int WGN>
hipError_t dispatch_layout(const GemmDesc& d, hipStream_t s) {
  if (d.xent_rows != nullptr) {  // the fused head's dX and dW: A is the logits
    if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == MN_MAJOR && d.mask_act == ACT_IDENTITY)
      return launch_tile<BM, BN, BK, WGM, WGN, K_MAJOR, MN_MAJOR, EPI_DX, true>(d, s);
    if (d.epi == EPI_DW && d.a_layout == MN_MAJOR && d.b_layout == MN_MAJOR)
      return launch_tile<BM, BN, BK, WGM, WGN, MN_MAJOR, MN_MAJOR, EPI_DW, true>(d, s);
    return hipErrorInvalidValue;
  }
  if (d.epi == EPI_FWD && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_tile<BM, BN, BK, WGM, WGN, K_MAJOR, K_MAJOR, EPI_FWD>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == MN_MAJOR)
    return launch_tile<BM, BN, BK, WGM, WGN, K_MAJOR, MN_MAJOR, EPI_DX>(d, s);
  if (d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_tile<BM, BN, BK, WGM, WGN, K_MAJOR, K_MAJOR, EPI_DX>(d, s);
  if (d.epi == EPI_DW && d.a_layout == MN_MAJOR && d.b_layout == MN_MAJOR)
    return launch_tile<BM, BN, BK, WGM, WGN, MN_MAJOR, MN_MAJOR, EPI_DW>(d, s);
  // float32 K-slices of a forward product (the MLP step's split forward)
  if (d.epi == EPI_DW && d.a_layout == K_MAJOR && d.b_layout == K_MAJOR)
    return launch_tile<BM, BN, BK, WGM, WGN, K_MAJOR, K_MAJOR, EPI_DW>(d, s);
  return hipErrorInvalidValue;
}

// Tile 0.  The forward (without the fused head's row statistics, which are
// laid out per 128 columns) and dX products run on 128x256 tiles of 8 waves
// of 64x64, one workgroup per CU, when every CU still gets two tiles: a
// workgroup then stages 128 + 256 operand rows per K step where two 128x128
// tiles stage 512, and the fused head's dX forms its loss gradient for half
// as many tiles (the wide MLP's forwards 1.7% and its dX 1.5% faster, the
// head's dX 2.5%).  Weight gradients and the rest stay on 128x128 tiles of 4
// waves, two workgroups per CU (the 8-wave tile measured 2% slower for the
// head's weight gradient).
hipError_t launch_tile0(const GemmDesc& d, hipStream_t s) {
  const bool fwd = d.epi == EPI_FWD && d.xent_part == nullptr && d.a_layout == K_MAJOR &&
                   d.b_layout == K_MAJOR;
  const bool dx = d.epi == EPI_DX && d.a_layout == K_MAJOR && d.b_layout == MN_MAJOR &&
                  (d.xent_rows == nullptr || d.mask_act == ACT_IDENTITY);
  if (fwd || dx) {
    int cus = 0;
    const hipError_t e = cu_count(cus);
    if (e != hipSuccess) return e;
    const int64_t tiles = (int64_t)((d.M + 127) / 128) * ((d.N + 255) / 256) * d.splits;
    if (tiles >= 2 * (int64_t)cus) {
      if (fwd) return launch_tile<128, 256, 16, 2, 4, K_MAJOR, K_MAJOR, EPI_FWD>(d, s);
      if (d.xent_rows != nullptr)
        return launch_tile<128, 256, 16, 2, 4, K_MAJOR, MN_MAJOR, EPI_DX, true>(d, s);
      return launch_tile<128, 256, 16, 2, 4, K_MAJOR, MN_MAJOR, EPI_DX>(d, s);
    }
  }
  return dispatch_layout<128, 128, 16, 2, 2>(d, s);
}

}  // namespace

// tile 0: 128x128, K step 16 (4 waves of 64x64; 128x256 of 8 waves for
// large forward and dX products); tile 1: 64x64, K step 32 (4 waves of
// 32x32); tile 2: 64x128, K step 32 (8 waves of 32x32: one workgroup loads
// 64 + 128 operand rows per K step where two 64x64 tiles load 256)
hipError_t launch_gemm_f32(const GemmDesc& d, int tile, hipStream_t s) {
  switch (tile) {
    case 0: return launch_tile0(d, s);
    case 1: return dispatch_layout<64, 64, 32, 2, 2>(d, s);
    case 2: return dispatch_layout<64, 128, 32, 2, 4>(d, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_gemm_f32_dw_dx(const GemmDesc& dw, const GemmDesc& dx, hipStream_t s) {
  if (dw.epi != EPI_DW || dw.a_layout != MN_MAJOR || dw.b_layout != MN_MAJOR ||
      dx.epi != EPI_DX || dx.a_layout != K_MAJOR || dx.b_layout != MN_MAJOR)
    return hipErrorInvalidValue;
  F32Job a, b;
  hipError_t e = make_job<64, 64>(dw, a);
  if (e == hipSuccess) e = make_job<64, 64>(dx, b);
  if (e != hipSuccess) return e;
  const SgdFinish none{};
  hipLaunchKernelGGL((gemm_f32_pair_kernel<K_MAJOR, MN_MAJOR, EPI_DX>),
                     dim3((unsigned)(a.nwg + b.nwg)), dim3(256), 0, s, a, b, none);
  return hipGetLastError();
}

hipError_t launch_gemm_f32_dw_dw(const GemmDesc& dw_a, const GemmDesc& dw_b, hipStream_t s,
                                 const SgdFinish* fin) {
  auto ok = [](const GemmDesc& d) {
    return d.epi == EPI_DW && d.a_layout == MN_MAJOR && d.b_layout == MN_MAJOR;
  };
  if (!ok(dw_a) || !ok(dw_b)) return hipErrorInvalidValue;
  // the epilogue's SGD step needs the final gradient (one K slice) and the
  // parameters at the same 16-byte alignment as dW
  auto sgd_ok = [](const GemmDesc& d) {
    if (d.sgd_w == nullptr) return d.sgd_b == nullptr;
    return d.splits == 1 && d.db != nullptr && d.sgd_b != nullptr &&
           ((reinterpret_cast<uintptr_t>(d.sgd_w) ^ reinterpret_cast<uintptr_t>(d.C)) & 15) == 0;
  };
  if (!sgd_ok(dw_a) || !sgd_ok(dw_b)) return hipErrorInvalidValue;
  F32Job a, b;
  hipError_t e = make_job<64, 64>(dw_a, a);
  if (e == hipSuccess) e = make_job<64, 64>(dw_b, b);
  if (e != hipSuccess) return e;
  SgdFinish f{};
  if (fin != nullptr) f = *fin;
  const unsigned extra = f.W != nullptr ? (unsigned)sgd_finish_wgs(f) : 0u;
  hipLaunchKernelGGL((gemm_f32_pair_kernel<MN_MAJOR, MN_MAJOR, EPI_DW>),
                     dim3((unsigned)(a.nwg + b.nwg) + extra), dim3(256), 0, s, a, b, f);
  return hipGetLastError();
}

}  // namespace dl

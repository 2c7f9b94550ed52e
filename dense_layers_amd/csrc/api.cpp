// C ABI of the dense-layer training path: argument validation (everything is
// checked before the first launch, so a rejected call touches no output),
// workspace planning, GEMM tile / split-K planning, and the composition of
// the kernels into the forward, vjp, loss, optimizer and whole-MLP-step calls.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/dense_layers_amd.h"
#include "common.hpp"

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(DL_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

}  // namespace

namespace dl {
// The last-error message of the calling thread, for entry points defined in
// other files.
int api_fail(int code, const char* msg) { return fail(code, "%s", msg); }
}  // namespace dl

namespace {

// ---- optional per-launch timing ----------------------------------------------
struct ProfRec {
  const char* name;
  hipEvent_t start, stop;
};
struct Prof {
  bool on = false;
  int capacity = 0;
  int seen = 0;
  std::vector<ProfRec> recs;
};
thread_local Prof g_prof;

// How much of the MLP step runs fused (dl_set_mlp_fusion): 2 = the tail
// kernel when the network ends in a small hidden layer and a narrow head,
// 1 = the head kernel alone.
thread_local int g_mlp_fusion = 2;

// Run `launch` (one kernel launch on stream s), timed when profiling is on.
template <class F>
hipError_t timed(const char* name, hipStream_t s, F&& launch) {
  if (!g_prof.on) return launch();
  ++g_prof.seen;
  if ((int)g_prof.recs.size() >= g_prof.capacity) return launch();
  ProfRec r{name, nullptr, nullptr};
  if (hipEventCreate(&r.start) != hipSuccess) return launch();
  if (hipEventCreate(&r.stop) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    return launch();
  }
  // a launch whose events could not be recorded runs untimed
  if (hipEventRecord(r.start, s) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    return launch();
  }
  hipError_t e = launch();
  if (hipEventRecord(r.stop, s) != hipSuccess) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
    return e;
  }
  g_prof.recs.push_back(r);
  return e;
}

// Validate mode (dl_set_validate): label ranges are checked on the device
// before a cross-entropy runs, which costs a stream synchronisation.
thread_local int g_validate = 0;

// In validate mode: count the labels outside [0, C) into the 4-byte device
// slot `slot` (part of the call's workspace, not yet in use), wait for the
// count and fail with DL_LABEL_OUT_OF_RANGE when there are any.  Nothing else
// has been launched when it fails.
int check_labels(const char* who, hipStream_t s, int64_t B, int64_t C, const int32_t* labels,
                 void* slot) {
  if (!g_validate) return DL_OK;
  hipError_t e = dl::launch_label_check(B, C, labels, static_cast<int*>(slot), s);
  if (e != hipSuccess) return hip_fail(e, who);
  int bad = 0;
  e = hipMemcpyAsync(&bad, slot, sizeof(int), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, who);
  if (bad > 0)
    return fail(DL_LABEL_OUT_OF_RANGE, "%s: %d label(s) outside [0, %lld)", who, bad,
                (long long)C);
  return DL_OK;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t esize(int dtype) { return dtype == DL_F32 ? 4 : 2; }

bool dtype_ok(int dtype) { return dtype == DL_F32 || dtype == DL_BF16 || dtype == DL_F16; }

bool overlap(const void* a, size_t an, const void* b, size_t bn) {
  if (a == nullptr || b == nullptr || an == 0 || bn == 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + bn && b0 < a0 + an;
}

bool dim_ok(int64_t v) { return v > 0 && v <= 0x7fffffff; }

// ---- GEMM planning ----------------------------------------------------------
// float32 tiles {0: 128x128x16, 1: 64x64x32, 2: 64x128x32 with 8 waves}:
// tile 0 when it alone yields at least one workgroup per CU (256); else, for
// forward and dX products, 64x128 when that does; otherwise 64x64.  (The
// launcher runs large tile-0 forward and dX products on 128x256 tiles of 8
// waves.)
// 16-bit tiles {0: 256x256 of 8 waves, 1: 128x128} of the direct-to-LDS
// kernel (K a multiple of 64) for forward and dX products: tile 0 with at
// least one such tile per CU, 128x128 otherwise; weight gradients, and
// operands the direct-load kernel cannot take (unaligned, K not a multiple
// of 64), run on the register-staged 128x128 kernel.  Only the
// weight-gradient product (K = batch) is split along K, when it has fewer
// than two workgroups per CU, into a power-of-two number of slices (at most
// 64, each keeping at least four K tiles): for 16-bit operands the smallest
// count that gives at least two workgroups per CU (the transformer-MLP
// block's weight gradients: 2 slices, 4 measured the same, none slower); for
// float32 the largest count that keeps the launch within one round of four
// workgroups per CU (fewer slices mean less fixed cost per slice and a
// shorter sum over them in the optimizer, and a second, partial round costs
// more than it hides).

constexpr int kCUs = 256;

struct Plan {
  int tile;
  int splits;
  int k_per_split;
};

void tile_shape(int dtype, int tile, int& bm, int& bn, int& bk) {
  if (dtype != DL_F32) {  // 16-bit operands
    bm = bn = tile == 1 ? 128 : 256;
    bk = 64;
  } else {
    bm = tile == 0 ? 128 : 64;
    bn = tile == 1 ? 64 : 128;
    bk = tile == 0 ? 16 : 32;
  }
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

Plan plan_gemm(int dtype, int epi, int64_t M, int64_t N, int64_t K) {
  Plan p{0, 1, (int)K};
  int bm, bn, bk;
  tile_shape(dtype, 0, bm, bn, bk);
  int64_t tiles = ceil_div(M, bm) * ceil_div(N, bn);
  // 16-bit weight gradients run on the register-staged kernel's 128x128
  // tile, split along K for about two workgroups per CU (four K-slices
  // measured the same, one slower); float32 ones aim at four per CU.
  int64_t per_cu = 4;
  if (dtype != DL_F32 && epi == dl::EPI_DW) per_cu = 2;
  if (tiles < kCUs || (dtype != DL_F32 && epi == dl::EPI_DW)) {
    p.tile = 1;
    if (dtype == DL_F32 && epi != dl::EPI_DW && ceil_div(M, 64) * ceil_div(N, 128) >= kCUs)
      p.tile = 2;
    tile_shape(dtype, p.tile, bm, bn, bk);
    tiles = ceil_div(M, bm) * ceil_div(N, bn);
  }
  if (epi == dl::EPI_DW && tiles < 2 * kCUs) {
    int64_t want = 1;  // a power of two: even slices of power-of-two batches
    if (dtype == DL_F32) {
      while (2 * want * tiles <= per_cu * kCUs) want *= 2;
    } else {
      while (want * tiles < per_cu * kCUs) want *= 2;
    }
    const int64_t max_by_k = std::max<int64_t>(1, K / (4 * bk));
    want = std::min<int64_t>(std::min<int64_t>(want, max_by_k), 64);
    int64_t kps = ceil_div(ceil_div(K, want), bk) * bk;
    p.k_per_split = (int)kps;
    p.splits = (int)ceil_div(K, kps);
  }
  if (p.splits <= 1) {
    p.splits = 1;
    p.k_per_split = (int)K;
  }
  return p;
}

size_t splitk_bytes(const Plan& p, int64_t M, int64_t N) {
  if (p.splits <= 1) return 0;
  return align_up((size_t)p.splits * M * N * 4) + align_up((size_t)p.splits * M * 4);
}

hipError_t run_gemm(int dtype, const dl::GemmDesc& d, int tile, hipStream_t s) {
  if (dtype == DL_F32) return dl::launch_gemm_f32(d, tile, s);
  dl::GemmDesc h = d;
  h.half_kind = dtype == DL_F16 ? dl::HK_F16 : dl::HK_BF16;
  return dl::launch_gemm_bf16(h, tile, s);
}

dl::GemmDesc blank_desc() {
  dl::GemmDesc d;
  memset(&d, 0, sizeof(d));
  d.splits = 1;
  return d;
}

// Forward GEMM with bias + activation epilogue.
hipError_t fwd_gemm(int dtype, int act, int64_t B, int64_t in, int64_t out, const void* X,
                    const void* W, const float* b, void* Y, void* Z, hipStream_t s) {
  dl::GemmDesc d = blank_desc();
  d.M = (int)B; d.N = (int)out; d.K = (int)in;
  d.A = X; d.lda = in; d.a_layout = dl::K_MAJOR;
  d.B = W; d.ldb = in; d.b_layout = dl::K_MAJOR;
  d.C = Y; d.ldc = out;
  d.epi = dl::EPI_FWD;
  d.bias = b; d.act = act; d.Z = Z;
  const Plan p = plan_gemm(dtype, dl::EPI_FWD, B, out, in);
  d.k_per_split = (int)in;
  return timed("fwd_gemm", s, [&] { return run_gemm(dtype, d, p.tile, s); });
}

// dW = G^T X (+ db = column sums of G), split-K partials in `partial_ws`.
// With reduce = false and a split plan, the partial slices are left for the
// caller (the optimizer kernel of the MLP step adds them up).
dl::GemmDesc dw_desc(int dtype, int64_t B, int64_t in, int64_t out, const void* G, const void* X,
                     float* dW, float* db, void* partial_ws, const Plan& p) {
  dl::GemmDesc d = blank_desc();
  d.M = (int)out; d.N = (int)in; d.K = (int)B;
  d.A = G; d.lda = out; d.a_layout = dl::MN_MAJOR;
  d.B = X; d.ldb = in; d.b_layout = dl::MN_MAJOR;
  d.C = dW; d.ldc = in;
  d.epi = dl::EPI_DW;
  d.splits = p.splits;
  d.k_per_split = p.k_per_split;
  if (p.splits > 1) {
    char* base = static_cast<char*>(partial_ws);
    d.partial = reinterpret_cast<float*>(base);
    d.db_partial = db ? reinterpret_cast<float*>(base + align_up((size_t)p.splits * out * in * 4))
                      : nullptr;
    d.db = nullptr;
  } else {
    d.db = db;
  }
  (void)dtype;
  return d;
}

hipError_t dw_gemm(int dtype, int64_t B, int64_t in, int64_t out, const void* G, const void* X,
                   float* dW, float* db, void* partial_ws, hipStream_t s, bool reduce = true,
                   const float* out_scale = nullptr, const Plan* plan = nullptr) {
  const Plan p = plan ? *plan : plan_gemm(dtype, dl::EPI_DW, out, in, B);
  dl::GemmDesc d = dw_desc(dtype, B, in, out, G, X, dW, db, partial_ws, p);
  d.out_scale = out_scale;
  hipError_t e = timed("dw_gemm", s, [&] { return run_gemm(dtype, d, p.tile, s); });
  if (e != hipSuccess || p.splits == 1 || !reduce) return e;
  return timed("splitk_reduce", s, [&] {
    return dl::launch_splitk_reduce((int)out, (int)in, p.splits, d.partial, d.db_partial, dW, in,
                                    db, s);
  });
}

// dX = G W, optionally times mask_act'(mask_src).  With Wt (W transposed,
// [in, out]) the B operand is read along K.
dl::GemmDesc dx_desc(int64_t B, int64_t in, int64_t out, const void* G, const void* W,
                     const void* Wt, void* dX, int mask_act, const void* mask_src) {
  dl::GemmDesc d = blank_desc();
  d.M = (int)B; d.N = (int)in; d.K = (int)out;
  d.A = G; d.lda = out; d.a_layout = dl::K_MAJOR;
  if (Wt != nullptr) {
    d.B = Wt; d.ldb = out; d.b_layout = dl::K_MAJOR;
  } else {
    d.B = W; d.ldb = in; d.b_layout = dl::MN_MAJOR;
  }
  d.C = dX; d.ldc = in;
  d.epi = dl::EPI_DX;
  d.mask_act = mask_act; d.mask_src = mask_src;
  d.k_per_split = (int)out;
  return d;
}

hipError_t dx_gemm(int dtype, int64_t B, int64_t in, int64_t out, const void* G, const void* W,
                   const void* Wt, void* dX, int mask_act, const void* mask_src, hipStream_t s,
                   const float* out_scale = nullptr) {
  dl::GemmDesc d = dx_desc(B, in, out, G, W, Wt, dX, mask_act, mask_src);
  d.out_scale = out_scale;
  const Plan p = plan_gemm(dtype, dl::EPI_DX, B, in, out);
  return timed("dx_gemm", s, [&] { return run_gemm(dtype, d, p.tile, s); });
}

size_t vjp_ws(int dtype, int act, int64_t B, int64_t in, int64_t out) {
  size_t ws = 0;
  if (act != DL_ACT_IDENTITY) ws += align_up((size_t)B * out * esize(dtype));
  ws += splitk_bytes(plan_gemm(dtype, dl::EPI_DW, out, in, B), out, in);
  return ws;
}

bool act_ok(int act) { return act == DL_ACT_IDENTITY || act == DL_ACT_RELU || act == DL_ACT_GELU_TANH; }

}  // namespace

extern "C" {

const char* dl_last_error(void) { return g_last_error.c_str(); }

const char* dense_last_error(void) { return g_last_error.c_str(); }

int dl_empty_launches(void* stream, int n) {
  if (n < 0) return fail(DL_INVALID_ARGUMENT, "dl_empty_launches: negative count");
  hipStream_t s = static_cast<hipStream_t>(stream);
  for (int i = 0; i < n; ++i) {
    const hipError_t e = dl::launch_empty(s);
    if (e != hipSuccess) return hip_fail(e, "dl_empty_launches");
  }
  return DL_OK;
}

int dl_set_validate(int on) {
  const int prev = g_validate;
  g_validate = on != 0;
  return prev;
}

const char* dl_build_target(void) { return "gfx950"; }

int dl_set_mlp_fusion(int level) {
  if (level != 1 && level != 2)
    return -fail(DL_INVALID_ARGUMENT, "dl_set_mlp_fusion: level must be 1 or 2");
  const int prev = g_mlp_fusion;
  g_mlp_fusion = level;
  return prev;
}

int dl_profile_begin(int capacity) {
  if (capacity < 0) return fail(DL_INVALID_ARGUMENT, "dl_profile_begin: negative capacity");
  for (auto& r : g_prof.recs) {
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.recs.clear();
  g_prof.recs.reserve(capacity);
  g_prof.capacity = capacity;
  g_prof.seen = 0;
  g_prof.on = true;
  return DL_OK;
}

int dl_profile_end(int max, float* ms, char* names) {
  g_prof.on = false;
  int err = 0;
  int i = 0;
  for (auto& r : g_prof.recs) {
    float t = 0.f;
    if (hipEventSynchronize(r.stop) != hipSuccess || hipEventElapsedTime(&t, r.start, r.stop) != hipSuccess)
      err = 1;
    if (i < max) {
      if (ms) ms[i] = t;
      if (names) {
        strncpy(names + (size_t)i * 48, r.name, 47);
        names[(size_t)i * 48 + 47] = 0;
      }
    }
    ++i;
    (void)hipEventDestroy(r.start);
    (void)hipEventDestroy(r.stop);
  }
  g_prof.recs.clear();
  if (err) {
    fail(DL_HIP_ERROR, "dl_profile_end: event query failed");
    return -DL_HIP_ERROR;
  }
  return g_prof.seen;
}

int dense_act_fwd(void* stream, int dtype, int act, int64_t B, int64_t in, int64_t out,
                  const void* X, const void* W, const float* b, void* Y, void* Z) {
  if (!dtype_ok(dtype)) return fail(DL_INVALID_ARGUMENT, "dense_act_fwd: bad dtype %d", dtype);
  if (!act_ok(act)) return fail(DL_INVALID_ARGUMENT, "dense_act_fwd: bad activation %d", act);
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(out))
    return fail(DL_INVALID_ARGUMENT, "dense_act_fwd: sizes must be in [1, 2^31): B=%lld in=%lld out=%lld",
                (long long)B, (long long)in, (long long)out);
  if (!X || !W || !Y) return fail(DL_INVALID_ARGUMENT, "dense_act_fwd: X, W and Y are required");
  const size_t es = esize(dtype);
  const size_t nX = (size_t)B * in * es, nW = (size_t)out * in * es, nY = (size_t)B * out * es;
  if (overlap(Y, nY, X, nX) || overlap(Y, nY, W, nW) || overlap(Y, nY, b, out * 4) ||
      overlap(Z, nY, Y, nY) || overlap(Z, nY, X, nX) || overlap(Z, nY, W, nW) ||
      overlap(Z, nY, b, out * 4))
    return fail(DL_ALIASING, "dense_act_fwd: Y/Z overlap an input or each other");
  hipError_t e = fwd_gemm(dtype, act, B, in, out, X, W, b, Y, Z, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "dense_act_fwd");
  return DL_OK;
}

size_t dense_act_vjp_workspace_size(int dtype, int act, int64_t B, int64_t in, int64_t out) {
  if (!dtype_ok(dtype) || !act_ok(act) || !dim_ok(B) || !dim_ok(in) ||
      !dim_ok(out))
    return 0;
  return vjp_ws(dtype, act, B, in, out);
}

static int vjp_impl(void* stream, int dtype, int act, int64_t B, int64_t in, int64_t out,
                    const void* dY, const void* saved, const void* X, const void* W,
                    const void* Wt, void* dX, float* dW, float* db, int dx_act,
                    const void* dx_saved, void* ws, size_t ws_bytes, const float* dy_scale) {
  if (!dtype_ok(dtype)) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: bad dtype %d", dtype);
  if (!act_ok(act) || !act_ok(dx_act)) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: bad activation");
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(out))
    return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: sizes must be in [1, 2^31)");
  if (!dY) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: dY is required");
  if (act != DL_ACT_IDENTITY && !saved)
    return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: saved Z/Y is required for a non-identity activation");
  if ((dW || db) && !X) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: X is required for dW/db");
  if (dX && !W && !Wt) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: W or Wt is required for dX");
  if (db && !dW) return fail(DL_UNSUPPORTED, "dense_act_vjp: db is reduced inside the dW kernel; pass dW too");
  if (dx_act != DL_ACT_IDENTITY && (!dX || !dx_saved))
    return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: dx_act needs dX and dx_saved");
  const size_t need = vjp_ws(dtype, act, B, in, out);
  if (need > 0 && (ws == nullptr || ws_bytes < need))
    return fail(DL_WORKSPACE_TOO_SMALL, "dense_act_vjp: workspace %zu bytes, need %zu", ws_bytes, need);
  if (ws && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DL_INVALID_ARGUMENT, "dense_act_vjp: workspace must be 256-byte aligned");
  const size_t es = esize(dtype);
  const size_t nY = (size_t)B * out * es, nX = (size_t)B * in * es, nW = (size_t)out * in * es;
  const size_t ndW = (size_t)out * in * 4, ndb = (size_t)out * 4;
  // dX may be X itself and/or dx_saved itself (dW and db are finished first).
  if (dX && (overlap(dX, nX, dY, nY) || overlap(dX, nX, W, nW) || overlap(dX, nX, Wt, nW) ||
             overlap(dX, nX, saved, nY) ||
             overlap(dX, nX, ws, need) || overlap(dX, nX, dW, ndW) || overlap(dX, nX, db, ndb) ||
             (dX != X && overlap(dX, nX, X, nX)) ||
             (dX != dx_saved && overlap(dX, nX, dx_saved, nX))))
    return fail(DL_ALIASING, "dense_act_vjp: dX overlaps an input it must not");
  if (dW && (overlap(dW, ndW, dY, nY) || overlap(dW, ndW, X, nX) || overlap(dW, ndW, W, nW) ||
             overlap(dW, ndW, saved, nY) || overlap(dW, ndW, ws, need) || overlap(dW, ndW, db, ndb)))
    return fail(DL_ALIASING, "dense_act_vjp: dW overlaps an input or db");
  if (db && (overlap(db, ndb, dY, nY) || overlap(db, ndb, X, nX) || overlap(db, ndb, W, nW) ||
             overlap(db, ndb, saved, nY) || overlap(db, ndb, ws, need)))
    return fail(DL_ALIASING, "dense_act_vjp: db overlaps an input");

  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsp = static_cast<char*>(ws);
  const void* G = dY;
  hipError_t e;
  if (act != DL_ACT_IDENTITY) {
    e = timed("act_mask", s, [&] { return dl::launch_act_mask(dtype, act, B, out, dY, saved, wsp, s); });
    if (e != hipSuccess) return hip_fail(e, "dense_act_vjp (mask)");
    G = wsp;
    wsp += align_up((size_t)B * out * es);
  }
  if (dW) {
    e = dw_gemm(dtype, B, in, out, G, X, dW, db, wsp, s, true, dy_scale);
    if (e != hipSuccess) return hip_fail(e, "dense_act_vjp (dW)");
  }
  if (dX) {
    e = dx_gemm(dtype, B, in, out, G, W, Wt, dX, dx_act, dx_saved, s, dy_scale);
    if (e != hipSuccess) return hip_fail(e, "dense_act_vjp (dX)");
  }
  return DL_OK;
}

int dense_act_vjp(void* stream, int dtype, int act, int64_t B, int64_t in, int64_t out,
                  const void* dY, const void* saved, const void* X, const void* W,
                  const void* Wt, void* dX, float* dW, float* db, int dx_act,
                  const void* dx_saved, void* ws, size_t ws_bytes) {
  return vjp_impl(stream, dtype, act, B, in, out, dY, saved, X, W, Wt, dX, dW, db, dx_act,
                  dx_saved, ws, ws_bytes, nullptr);
}

int dense_act_vjp_scaled(void* stream, int dtype, int act, int64_t B, int64_t in, int64_t out,
                         const void* dY, const void* saved, const void* X, const void* W,
                         const void* Wt, void* dX, float* dW, float* db, int dx_act,
                         const void* dx_saved, void* ws, size_t ws_bytes,
                         const float* dy_scale) {
  if (!dy_scale) return fail(DL_INVALID_ARGUMENT, "dense_act_vjp_scaled: dy_scale is required");
  const size_t nY = (size_t)B * out * esize(dtype);
  if (dim_ok(B) && dim_ok(out) && (overlap(dy_scale, 4, dX, (size_t)B * in * esize(dtype)) ||
                                   overlap(dy_scale, 4, dW, (size_t)out * in * 4) ||
                                   overlap(dy_scale, 4, db, (size_t)out * 4) ||
                                   overlap(dy_scale, 4, ws, ws_bytes) || overlap(dy_scale, 4, dY, nY)))
    return fail(DL_ALIASING, "dense_act_vjp_scaled: dy_scale overlaps an output or the workspace");
  return vjp_impl(stream, dtype, act, B, in, out, dY, saved, X, W, Wt, dX, dW, db, dx_act,
                  dx_saved, ws, ws_bytes, dy_scale);
}

size_t softmax_xent_workspace_size(int64_t B, int64_t C) {
  if (B <= 0 || C <= 0) return 0;
  return align_up((size_t)B * 4);
}

int softmax_xent_fwd_bwd(void* stream, int64_t B, int64_t C, const float* logits,
                         const int32_t* labels, float* loss, float* row_loss, float* dlogits,
                         void* ws, size_t ws_bytes) {
  if (!dim_ok(B) || !dim_ok(C)) return fail(DL_INVALID_ARGUMENT, "softmax_xent_fwd_bwd: sizes must be in [1, 2^31)");
  if (!logits || !labels || !loss || !dlogits)
    return fail(DL_INVALID_ARGUMENT, "softmax_xent_fwd_bwd: logits, labels, loss and dlogits are required");
  const size_t need = softmax_xent_workspace_size(B, C);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "softmax_xent_fwd_bwd: workspace %zu bytes, need %zu", ws_bytes, need);
  const size_t nz = (size_t)B * C * 4;
  if ((dlogits != logits && overlap(dlogits, nz, logits, nz)) || overlap(dlogits, nz, labels, B * 4) ||
      overlap(dlogits, nz, loss, 4) || overlap(dlogits, nz, row_loss, B * 4) ||
      overlap(loss, 4, logits, nz) || overlap(row_loss, B * 4, logits, nz) ||
      overlap(dlogits, nz, ws, need))
    return fail(DL_ALIASING, "softmax_xent_fwd_bwd: outputs overlap inputs (dlogits may equal logits)");
  float* rl = row_loss ? row_loss : static_cast<float*>(ws);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int vs = check_labels("softmax_xent_fwd_bwd", st, B, C, labels, ws);
  if (vs != DL_OK) return vs;
  hipError_t e = timed("xent", st, [&] { return dl::launch_xent(B, C, logits, labels, rl, dlogits, loss, st); });
  if (e != hipSuccess) return hip_fail(e, "softmax_xent_fwd_bwd");
  return DL_OK;
}

// ---- fused classifier head over many classes ----------------------------------
// Forward: one GEMM writes the logits and, per row and column tile, the tile's
// (max, sum exp) pair; a row pass forms lse and the row losses, and the fixed
// order mean follows.  Backward: the dX and dW GEMMs read the logits and form
// the loss gradient from them and lse as they stage them (the gradient never
// reaches HBM, and no pass over the logits runs between the two GEMMs).

static int xent_tiles(int64_t B, int64_t in, int64_t C) {
  const Plan p = plan_gemm(DL_F32, dl::EPI_FWD, B, C, in);
  int bm, bn, bk;
  tile_shape(DL_F32, p.tile, bm, bn, bk);
  return (int)ceil_div(C, bn);
}

size_t dense_xent_fwd_workspace_size(int64_t B, int64_t in, int64_t C) {
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(C)) return 0;
  return align_up((size_t)xent_tiles(B, in, C) * B * 8) + align_up((size_t)B * 4);
}

int dense_xent_fwd(void* stream, int64_t B, int64_t in, int64_t C, const float* X,
                   const float* W, const float* b, const int32_t* labels, float* logits,
                   float* lse, float* loss, float* row_loss, void* ws, size_t ws_bytes) {
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(C))
    return fail(DL_INVALID_ARGUMENT, "dense_xent_fwd: sizes must be in [1, 2^31)");
  if (!X || !W || !labels || !logits || !lse || !loss)
    return fail(DL_INVALID_ARGUMENT, "dense_xent_fwd: X, W, labels, logits, lse and loss are required");
  const size_t need = dense_xent_fwd_workspace_size(B, in, C);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "dense_xent_fwd: workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DL_INVALID_ARGUMENT, "dense_xent_fwd: workspace must be 256-byte aligned");
  const size_t nz = (size_t)B * C * 4, nX = (size_t)B * in * 4, nW = (size_t)C * in * 4;
  const struct { const void* p; size_t n; } outs[] = {{logits, nz}, {lse, (size_t)B * 4},
                                                      {loss, 4}, {row_loss, (size_t)B * 4},
                                                      {ws, need}};
  const struct { const void* p; size_t n; } ins[] = {{X, nX}, {W, nW}, {b, (size_t)C * 4},
                                                     {labels, (size_t)B * 4}};
  for (size_t i = 0; i < 5; ++i) {
    for (size_t j = 0; j < 4; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
        return fail(DL_ALIASING, "dense_xent_fwd: an output overlaps an input");
    for (size_t j = i + 1; j < 5; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(DL_ALIASING, "dense_xent_fwd: two outputs overlap");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* wsp = static_cast<char*>(ws);
  const int T = xent_tiles(B, in, C);
  float* part = reinterpret_cast<float*>(wsp);
  float* rl = row_loss ? row_loss : reinterpret_cast<float*>(wsp + align_up((size_t)T * B * 8));
  const int vs = check_labels("dense_xent_fwd", s, B, C, labels, wsp);
  if (vs != DL_OK) return vs;
  dl::GemmDesc d = blank_desc();
  d.M = (int)B; d.N = (int)C; d.K = (int)in;
  d.A = X; d.lda = in; d.a_layout = dl::K_MAJOR;
  d.B = W; d.ldb = in; d.b_layout = dl::K_MAJOR;
  d.C = logits; d.ldc = C;
  d.epi = dl::EPI_FWD;
  d.bias = b; d.act = DL_ACT_IDENTITY;
  d.k_per_split = (int)in;
  d.xent_part = part;
  const Plan p = plan_gemm(DL_F32, dl::EPI_FWD, B, C, in);
  hipError_t e = timed("xent_fwd_gemm", s, [&] { return dl::launch_gemm_f32(d, p.tile, s); });
  if (e == hipSuccess)
    e = timed("xent_lse", s, [&] { return dl::launch_xent_lse(B, C, T, part, logits, labels, lse, rl, s); });
  if (e == hipSuccess)
    e = timed("loss_mean", s, [&] { return dl::launch_loss_mean(B, rl, loss, s); });
  if (e != hipSuccess) return hip_fail(e, "dense_xent_fwd");
  return DL_OK;
}

size_t dense_xent_vjp_workspace_size(int64_t B, int64_t in, int64_t C) {
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(C)) return 0;
  // the per-row records (and one spare), then the dW split-K slices
  return align_up((size_t)(B + 1) * 8) +
         splitk_bytes(plan_gemm(DL_F32, dl::EPI_DW, C, in, B), C, in);
}

int dense_xent_vjp(void* stream, int64_t B, int64_t in, int64_t C, const float* logits,
                   const float* lse, const int32_t* labels, const float* X, const float* W,
                   float* dX, float* dW, float* db, void* ws, size_t ws_bytes) {
  if (!dim_ok(B) || !dim_ok(in) || !dim_ok(C))
    return fail(DL_INVALID_ARGUMENT, "dense_xent_vjp: sizes must be in [1, 2^31)");
  if (!logits || !lse || !labels)
    return fail(DL_INVALID_ARGUMENT, "dense_xent_vjp: logits, lse and labels are required");
  if ((dW || db) && !X) return fail(DL_INVALID_ARGUMENT, "dense_xent_vjp: X is required for dW/db");
  if (dX && !W) return fail(DL_INVALID_ARGUMENT, "dense_xent_vjp: W is required for dX");
  if (db && !dW) return fail(DL_UNSUPPORTED, "dense_xent_vjp: db is reduced inside the dW kernel; pass dW too");
  const size_t need = dense_xent_vjp_workspace_size(B, in, C);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "dense_xent_vjp: workspace %zu bytes, need %zu", ws_bytes, need);
  if (ws && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DL_INVALID_ARGUMENT, "dense_xent_vjp: workspace must be 256-byte aligned");
  const size_t nz = (size_t)B * C * 4, nX = (size_t)B * in * 4, nW = (size_t)C * in * 4;
  const struct { const void* p; size_t n; } outs[] = {{dX, nX}, {dW, nW}, {db, (size_t)C * 4},
                                                      {ws, need}};
  const struct { const void* p; size_t n; } ins[] = {{logits, nz}, {lse, (size_t)B * 4},
                                                     {labels, (size_t)B * 4}, {X, nX}, {W, nW}};
  for (size_t i = 0; i < 4; ++i) {
    for (size_t j = 0; j < 5; ++j)
      if (overlap(outs[i].p, outs[i].n, ins[j].p, ins[j].n))
        return fail(DL_ALIASING, "dense_xent_vjp: an output overlaps an input");
    for (size_t j = i + 1; j < 4; ++j)
      if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n))
        return fail(DL_ALIASING, "dense_xent_vjp: two outputs overlap");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const float invB = (float)(1.0 / (double)B);
  const float log2B = (float)std::log2((double)B);
  char* wsp = static_cast<char*>(ws);
  float* rows = reinterpret_cast<float*>(wsp);
  hipError_t e = timed("xent_rows", s, [&] {
    return dl::launch_xent_rows(B, lse, labels, log2B, rows, s);
  });
  if (e != hipSuccess) return hip_fail(e, "dense_xent_vjp (rows)");
  if (dW) {
    const Plan p = plan_gemm(DL_F32, dl::EPI_DW, C, in, B);
    dl::GemmDesc d = dw_desc(DL_F32, B, in, C, logits, X, dW, db,
                             wsp + align_up((size_t)(B + 1) * 8), p);
    d.xent_rows = rows; d.xent_invB = invB;
    e = timed("xent_dw_gemm", s, [&] { return dl::launch_gemm_f32(d, p.tile, s); });
    if (e == hipSuccess && p.splits > 1)
      e = timed("splitk_reduce", s, [&] {
        return dl::launch_splitk_reduce((int)C, (int)in, p.splits, d.partial, d.db_partial, dW, in,
                                        db, s);
      });
    if (e != hipSuccess) return hip_fail(e, "dense_xent_vjp (dW)");
  }
  if (dX) {
    dl::GemmDesc d = dx_desc(B, in, C, logits, W, nullptr, dX, DL_ACT_IDENTITY, nullptr);
    d.xent_rows = rows; d.xent_invB = invB;
    const Plan p = plan_gemm(DL_F32, dl::EPI_DX, B, in, C);
    e = timed("xent_dx_gemm", s, [&] { return dl::launch_gemm_f32(d, p.tile, s); });
    if (e != hipSuccess) return hip_fail(e, "dense_xent_vjp (dX)");
  }
  return DL_OK;
}

// ---- optimizers ---------------------------------------------------------------

static dl::LrSched to_sched(const dl_lr_schedule_t* s) {
  dl::LrSched r;
  memset(&r, 0, sizeof(r));
  r.step_size = 1;
  r.gamma = 1.0;
  if (s != nullptr) {
    r.kind = s->kind;
    r.warmup = s->warmup;
    r.total = s->total;
    r.step_size = s->step_size;
    r.min_lr = s->min_lr;
    r.gamma = s->gamma;
  }
  return r;
}

static const char* sched_problem(const dl_lr_schedule_t* s) {
  if (s == nullptr) return nullptr;
  if (s->kind < DL_LR_CONSTANT || s->kind > DL_LR_WARMUP_LINEAR) return "bad schedule kind";
  if (s->kind == DL_LR_STEP && s->step_size < 1) return "a step schedule needs step_size >= 1";
  if (s->warmup < 0) return "warmup must be >= 0";
  return nullptr;
}

double dl_lr_at(const dl_lr_schedule_t* s, double lr, int64_t step) {
  if (step < 1 || sched_problem(s) != nullptr) return NAN;
  return dl::lr_schedule(to_sched(s), lr, step);
}

// Constants of step t (t < 1: the bias corrections are left at 1, for SGD or
// when the device forms them).
static dl::OptConsts opt_consts(const dl_opt_t& o, int64_t t) {
  dl::OptConsts c;
  memset(&c, 0, sizeof(c));
  c.sched = to_sched(o.schedule);
  c.lr_d = o.lr;
  c.beta1_d = o.beta1;
  c.beta2_d = o.beta2;
  c.wd_d = o.weight_decay;
  const double lr = t >= 1 ? dl::lr_schedule(c.sched, o.lr, t) : o.lr;
  c.lr = (float)lr;
  c.decay = (float)(1.0 - lr * o.weight_decay);
  c.wd = (float)o.weight_decay;
  c.b1 = (float)o.beta1;
  c.omb1 = (float)(1.0 - o.beta1);
  c.b2 = (float)o.beta2;
  c.omb2 = (float)(1.0 - o.beta2);
  const double bc1 = t >= 1 ? 1.0 - std::pow(o.beta1, (double)t) : 1.0;
  const double bc2 = t >= 1 ? 1.0 - std::pow(o.beta2, (double)t) : 1.0;
  c.step_size = (float)(lr / bc1);
  c.inv_sqrt_bc2 = (float)(1.0 / std::sqrt(bc2));
  c.eps = (float)o.eps;
  c.ema_d = (float)o.ema_decay;
  c.ema_omd = (float)(1.0 - o.ema_decay);
  return c;
}

static dl_opt_t plain_opt(int kind, double lr, double beta1, double beta2, double eps, double wd,
                          int64_t step) {
  dl_opt_t o;
  memset(&o, 0, sizeof(o));
  o.kind = kind;
  o.lr = lr;
  o.beta1 = beta1;
  o.beta2 = beta2;
  o.eps = eps;
  o.weight_decay = wd;
  o.step = step;
  return o;
}

static bool betas_ok(double b1, double b2) { return b1 >= 0.0 && b1 < 1.0 && b2 >= 0.0 && b2 < 1.0; }

// The checks of dl_opt_t that optimizer_step and mlp_train_step share.
static int check_opt(const dl_opt_t* o, const char* who, bool any_ema) {
  if (o->kind != DL_OPT_SGD && o->kind != DL_OPT_ADAMW && o->kind != DL_OPT_ADAM)
    return fail(DL_INVALID_ARGUMENT, "%s: bad optimizer kind %d", who, o->kind);
  const bool adam = o->kind != DL_OPT_SGD;
  if (adam && !betas_ok(o->beta1, o->beta2))
    return fail(DL_INVALID_ARGUMENT, "%s: betas must be in [0, 1)", who);
  if (const char* p = sched_problem(o->schedule)) return fail(DL_INVALID_ARGUMENT, "%s: %s", who, p);
  const bool needs_t = adam || o->schedule != nullptr;
  if (needs_t && o->step_dev == nullptr && o->step < 1)
    return fail(DL_INVALID_ARGUMENT, "%s: step counts from 1", who);
  if (any_ema && !(o->ema_decay >= 0.0 && o->ema_decay <= 1.0))
    return fail(DL_INVALID_ARGUMENT, "%s: ema_decay must be in [0, 1]", who);
  if (o->max_grad_norm != o->max_grad_norm)
    return fail(DL_INVALID_ARGUMENT, "%s: max_grad_norm is NaN", who);
  if (o->scaler != nullptr) {
    const dl_loss_scaler_t& sc = *o->scaler;
    if (!sc.scale || !sc.growth_tracker || !sc.found_inf)
      return fail(DL_INVALID_ARGUMENT, "%s: the loss scaler needs scale, growth_tracker and found_inf", who);
    if (!(sc.growth_factor > 0.0) || !(sc.backoff_factor > 0.0) || sc.growth_interval < 1)
      return fail(DL_INVALID_ARGUMENT, "%s: bad loss-scaler factors or interval", who);
    if (needs_t && o->step_dev == nullptr)
      return fail(DL_INVALID_ARGUMENT,
                  "%s: a loss scaler needs a device step count (a skipped step must not advance t)", who);
  }
  return DL_OK;
}

// Byte ranges that must not overlap one another (null or empty ones are
// ignored): sorted by start, neighbours compared.
struct Span {
  uintptr_t a;
  size_t n;
};
static bool spans_overlap(std::vector<Span> v) {
  v.erase(std::remove_if(v.begin(), v.end(), [](const Span& x) { return x.a == 0 || x.n == 0; }),
          v.end());
  std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) { return x.a < y.a; });
  for (size_t i = 1; i < v.size(); ++i)
    if (v[i - 1].a + v[i - 1].n > v[i].a) return true;
  return false;
}
static Span span(const void* p, size_t n) { return Span{reinterpret_cast<uintptr_t>(p), n}; }

// Multi-array calls take their arrays kMaxSegs to a launch.  The gradient
// pass of a chunk leaves stat_grid(units of the chunk) partials.
constexpr int kMaxArrays = 4096;
static int64_t units_of(int64_t n) { return (n + dl::kStatUnit - 1) / dl::kStatUnit; }
extern "C++" {
template <class N>
static int64_t stat_parts(int count, N n_of) {
  int64_t parts = 0;
  for (int c0 = 0; c0 < count; c0 += dl::kMaxSegs) {
    int64_t units = 0;
    for (int k = c0; k < std::min(count, c0 + dl::kMaxSegs); ++k) units += units_of(n_of(k));
    parts += dl::stat_grid(units);
  }
  return parts;
}
}
// Workspace of the gradient control: the GradCtl and clip coefficient, then
// the float64 partial sums and the int partial counts.
static size_t ctl_bytes(int64_t parts) {
  return kAlign + align_up((size_t)parts * 8) + align_up((size_t)parts * 4);
}
struct CtlMem {
  dl::GradCtl* ctl;
  float* coef;
  double* sq;
  int* bad;
};
static CtlMem ctl_mem(void* ws, int64_t parts) {
  char* b = static_cast<char*>(ws);
  CtlMem m;
  m.ctl = reinterpret_cast<dl::GradCtl*>(b);
  m.coef = reinterpret_cast<float*>(b + sizeof(dl::GradCtl));
  m.sq = reinterpret_cast<double*>(b + kAlign);
  m.bad = reinterpret_cast<int*>(b + kAlign + align_up((size_t)parts * 8));
  return m;
}
static dl::OptSegs blank_segs() {
  dl::OptSegs segs;
  memset(&segs, 0, sizeof(segs));
  return segs;
}
// Appends one array to segs with start_block in units (gradient pass) or in
// optimizer blocks (update).
static void add_seg(dl::OptSegs& segs, int64_t& blocks, bool units, int64_t n, float* w,
                    const float* g, float* m, float* v, float* e, void* wb, const float* part,
                    int splits, float* g_out) {
  const int k = segs.count++;
  segs.start_block[k] = blocks;
  segs.n[k] = n;
  segs.w[k] = w;
  segs.g[k] = g;
  segs.m[k] = m;
  segs.v[k] = v;
  segs.ema[k] = e;
  segs.wb[k] = static_cast<dl::bf16_t*>(wb);
  segs.part[k] = splits > 1 ? part : nullptr;
  segs.part_stride[k] = n;
  segs.splits[k] = splits;
  segs.g_out[k] = g_out;
  const int64_t per = units ? dl::kStatUnit : dl::opt_elems_per_block(splits);
  blocks += (n + per - 1) / per;
  segs.start_block[segs.count] = blocks;
}

static dl::CtlArgs ctl_args(const dl_opt_t* o, const CtlMem& m, int64_t parts) {
  dl::CtlArgs a;
  memset(&a, 0, sizeof(a));
  a.part_sq = m.sq;
  a.part_bad = m.bad;
  a.parts = (int)parts;
  a.max_norm = o->max_grad_norm;
  if (o->scaler != nullptr) {
    a.scale = o->scaler->scale;
    a.growth_tracker = o->scaler->growth_tracker;
    a.found_inf = o->scaler->found_inf;
    a.growth_factor = o->scaler->growth_factor;
    a.backoff_factor = o->scaler->backoff_factor;
    a.growth_interval = o->scaler->growth_interval;
  }
  a.step_dev = o->step_dev;
  a.norm_out = o->grad_norm;
  a.ctl = m.ctl;
  a.clip_coef = m.coef;
  return a;
}

int sgd_step(void* stream, int64_t n, float* w, const float* g, double lr) {
  if (n <= 0) return fail(DL_INVALID_ARGUMENT, "sgd_step: n must be positive");
  if (!w || !g) return fail(DL_INVALID_ARGUMENT, "sgd_step: w and g are required");
  if (overlap(w, n * 4, g, n * 4)) return fail(DL_ALIASING, "sgd_step: w overlaps g");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dl::OptConsts oc = opt_consts(plain_opt(DL_OPT_SGD, lr, 0, 0, 0, 0, 0), 0);
  hipError_t e = timed("sgd", st, [&] { return dl::launch_sgd(n, w, g, oc, st); });
  if (e != hipSuccess) return hip_fail(e, "sgd_step");
  return DL_OK;
}

static int adam_like(const char* who, int kind, void* stream, int64_t n, float* w, const float* g,
                     float* m, float* v, double lr, double beta1, double beta2, double eps,
                     double weight_decay, int64_t step) {
  if (n <= 0) return fail(DL_INVALID_ARGUMENT, "%s: n must be positive", who);
  if (!w || !g || !m || !v) return fail(DL_INVALID_ARGUMENT, "%s: w, g, m and v are required", who);
  if (step < 1) return fail(DL_INVALID_ARGUMENT, "%s: step counts from 1", who);
  if (!betas_ok(beta1, beta2)) return fail(DL_INVALID_ARGUMENT, "%s: betas must be in [0, 1)", who);
  const size_t nb = (size_t)n * 4;
  if (overlap(w, nb, g, nb) || overlap(w, nb, m, nb) || overlap(w, nb, v, nb) ||
      overlap(g, nb, m, nb) || overlap(g, nb, v, nb) || overlap(m, nb, v, nb))
    return fail(DL_ALIASING, "%s: w, g, m, v must be distinct", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const dl::OptConsts oc = opt_consts(plain_opt(kind, lr, beta1, beta2, eps, weight_decay, step), step);
  hipError_t e = timed(kind == DL_OPT_ADAM ? "adam" : "adamw", st, [&] {
    return kind == DL_OPT_ADAM ? dl::launch_adam(n, w, g, m, v, oc, st)
                               : dl::launch_adamw(n, w, g, m, v, oc, st);
  });
  if (e != hipSuccess) return hip_fail(e, who);
  return DL_OK;
}

int adamw_step(void* stream, int64_t n, float* w, const float* g, float* m, float* v, double lr,
               double beta1, double beta2, double eps, double weight_decay, int64_t step) {
  return adam_like("adamw_step", DL_OPT_ADAMW, stream, n, w, g, m, v, lr, beta1, beta2, eps,
                   weight_decay, step);
}

int adam_step(void* stream, int64_t n, float* w, const float* g, float* m, float* v, double lr,
              double beta1, double beta2, double eps, double weight_decay, int64_t step) {
  return adam_like("adam_step", DL_OPT_ADAM, stream, n, w, g, m, v, lr, beta1, beta2, eps,
                   weight_decay, step);
}

int ema_update(void* stream, int64_t n, float* ema, const float* w, double decay) {
  if (n <= 0) return fail(DL_INVALID_ARGUMENT, "ema_update: n must be positive");
  if (!ema || !w) return fail(DL_INVALID_ARGUMENT, "ema_update: ema and w are required");
  if (!(decay >= 0.0 && decay <= 1.0)) return fail(DL_INVALID_ARGUMENT, "ema_update: decay must be in [0, 1]");
  if (overlap(ema, n * 4, w, n * 4)) return fail(DL_ALIASING, "ema_update: ema overlaps w");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed("ema", st, [&] {
    return dl::launch_ema(n, ema, w, (float)decay, (float)(1.0 - decay), st);
  });
  if (e != hipSuccess) return hip_fail(e, "ema_update");
  return DL_OK;
}

size_t clip_grad_norm_workspace_size(int32_t count, const int64_t* n) {
  if (count < 1 || count > kMaxArrays || !n) return 0;
  for (int k = 0; k < count; ++k)
    if (n[k] <= 0) return 0;
  return ctl_bytes(stat_parts(count, [&](int k) { return n[k]; }));
}

int clip_grad_norm(void* stream, int32_t count, float* const* grads, const int64_t* n,
                   double max_norm, float* total_norm, void* ws, size_t ws_bytes) {
  if (count < 1 || count > kMaxArrays || !grads || !n)
    return fail(DL_INVALID_ARGUMENT, "clip_grad_norm: count must be in [1, %d] with grads and n", kMaxArrays);
  if (!(max_norm > 0.0)) return fail(DL_INVALID_ARGUMENT, "clip_grad_norm: max_norm must be positive");
  std::vector<Span> spans;
  for (int k = 0; k < count; ++k) {
    if (!grads[k] || n[k] <= 0) return fail(DL_INVALID_ARGUMENT, "clip_grad_norm: array %d is empty or null", k);
    spans.push_back(span(grads[k], (size_t)n[k] * 4));
  }
  const int64_t parts = stat_parts(count, [&](int k) { return n[k]; });
  const size_t need = ctl_bytes(parts);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "clip_grad_norm: workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DL_INVALID_ARGUMENT, "clip_grad_norm: workspace must be 256-byte aligned");
  spans.push_back(span(ws, need));
  spans.push_back(span(total_norm, 4));
  if (spans_overlap(spans)) return fail(DL_ALIASING, "clip_grad_norm: arrays overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const CtlMem mem = ctl_mem(ws, parts);
  int64_t off = 0;
  hipError_t e = hipSuccess;
  for (int c0 = 0; c0 < count && e == hipSuccess; c0 += dl::kMaxSegs) {
    dl::OptSegs segs = blank_segs();
    int64_t units = 0;
    for (int k = c0; k < std::min(count, c0 + dl::kMaxSegs); ++k)
      add_seg(segs, units, true, n[k], grads[k], grads[k], nullptr, nullptr, nullptr, nullptr,
              nullptr, 1, nullptr);
    e = timed("grad_stats", s, [&] {
      return dl::launch_grad_stats(segs, units, mem.sq + off, mem.bad + off, s);
    });
    off += dl::stat_grid(units);
  }
  dl_opt_t o = plain_opt(DL_OPT_SGD, 0, 0, 0, 0, 0, 0);
  o.max_grad_norm = max_norm;
  o.grad_norm = total_norm;
  const dl::CtlArgs a = ctl_args(&o, mem, parts);
  if (e == hipSuccess) e = timed("grad_ctl", s, [&] { return dl::launch_grad_ctl(a, s); });
  for (int c0 = 0; c0 < count && e == hipSuccess; c0 += dl::kMaxSegs) {
    dl::OptSegs segs = blank_segs();
    int64_t units = 0;
    for (int k = c0; k < std::min(count, c0 + dl::kMaxSegs); ++k)
      add_seg(segs, units, true, n[k], grads[k], grads[k], nullptr, nullptr, nullptr, nullptr,
              nullptr, 1, nullptr);
    e = timed("clip_scale", s, [&] { return dl::launch_scale_by(segs, mem.coef, s); });
  }
  if (e != hipSuccess) return hip_fail(e, "clip_grad_norm");
  return DL_OK;
}

size_t optimizer_step_workspace_size(int32_t count, const dl_param_t* params) {
  if (count < 1 || count > kMaxArrays || !params) return 0;
  for (int k = 0; k < count; ++k)
    if (params[k].n <= 0) return 0;
  return ctl_bytes(stat_parts(count, [&](int k) { return params[k].n; }));
}

int optimizer_step(void* stream, const dl_opt_t* opt, int32_t count, const dl_param_t* params,
                   void* ws, size_t ws_bytes) {
  if (!opt || !params || count < 1 || count > kMaxArrays)
    return fail(DL_INVALID_ARGUMENT, "optimizer_step: opt, params and count in [1, %d] are required", kMaxArrays);
  const bool adam = opt->kind == DL_OPT_ADAM || opt->kind == DL_OPT_ADAMW;
  bool any_ema = false;
  std::vector<Span> spans;
  for (int k = 0; k < count; ++k) {
    const dl_param_t& p = params[k];
    if (p.n <= 0 || !p.w || !p.g) return fail(DL_INVALID_ARGUMENT, "optimizer_step: param %d needs n > 0, w and g", k);
    if (adam && (!p.m || !p.v)) return fail(DL_INVALID_ARGUMENT, "optimizer_step: param %d needs m and v", k);
    const size_t nb = (size_t)p.n * 4;
    spans.push_back(span(p.w, nb));
    spans.push_back(span(p.g, nb));
    if (adam) {
      spans.push_back(span(p.m, nb));
      spans.push_back(span(p.v, nb));
    }
    spans.push_back(span(p.ema, nb));
    spans.push_back(span(p.w_bf16, (size_t)p.n * 2));
    any_ema = any_ema || p.ema != nullptr;
  }
  if (int st = check_opt(opt, "optimizer_step", any_ema)) return st;
  const bool ctl_on = opt->max_grad_norm > 0.0 || opt->scaler != nullptr;
  const int64_t parts = ctl_on ? stat_parts(count, [&](int k) { return params[k].n; }) : 0;
  const size_t need = ctl_on ? ctl_bytes(parts) : 0;
  if (ctl_on) {
    if (!ws || ws_bytes < need)
      return fail(DL_WORKSPACE_TOO_SMALL, "optimizer_step: workspace %zu bytes, need %zu", ws_bytes, need);
    if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
      return fail(DL_INVALID_ARGUMENT, "optimizer_step: workspace must be 256-byte aligned");
    spans.push_back(span(ws, need));
  }
  if (spans_overlap(spans)) return fail(DL_ALIASING, "optimizer_step: arrays overlap");
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool dev_step = opt->step_dev != nullptr;
  hipError_t e = hipSuccess;
  if (dev_step && !ctl_on) e = dl::launch_step_tick(opt->step_dev, s);
  CtlMem mem{};
  if (ctl_on) {
    mem = ctl_mem(ws, parts);
    int64_t off = 0;
    for (int c0 = 0; c0 < count && e == hipSuccess; c0 += dl::kMaxSegs) {
      dl::OptSegs segs = blank_segs();
      int64_t units = 0;
      for (int k = c0; k < std::min(count, c0 + dl::kMaxSegs); ++k)
        add_seg(segs, units, true, params[k].n, params[k].w, params[k].g, nullptr, nullptr,
                nullptr, nullptr, nullptr, 1, nullptr);
      e = timed("grad_stats", s, [&] {
        return dl::launch_grad_stats(segs, units, mem.sq + off, mem.bad + off, s);
      });
      off += dl::stat_grid(units);
    }
    const dl::CtlArgs a = ctl_args(opt, mem, parts);
    if (e == hipSuccess) e = timed("grad_ctl", s, [&] { return dl::launch_grad_ctl(a, s); });
  }
  dl::OptConsts oc = opt_consts(*opt, dev_step ? 0 : opt->step);
  if (dev_step) oc.step_dev = opt->step_dev;
  if (ctl_on) oc.ctl = mem.ctl;
  for (int c0 = 0; c0 < count && e == hipSuccess; c0 += dl::kMaxSegs) {
    dl::OptSegs segs = blank_segs();
    int64_t blocks = 0;
    for (int k = c0; k < std::min(count, c0 + dl::kMaxSegs); ++k) {
      const dl_param_t& p = params[k];
      add_seg(segs, blocks, false, p.n, p.w, p.g, p.m, p.v, p.ema, p.w_bf16, nullptr, 1, nullptr);
    }
    e = timed("opt_multi", s, [&] { return dl::launch_opt_multi(segs, opt->kind, oc, s); });
  }
  if (e != hipSuccess) return hip_fail(e, "optimizer_step");
  return DL_OK;
}

// ---- mean squared error ------------------------------------------------------------

size_t mse_loss_workspace_size(int64_t B, int64_t C) {
  if (B <= 0 || C <= 0) return 0;
  return align_up((size_t)dl::mse_grid(B * C) * 8);
}

int mse_loss_fwd_bwd(void* stream, int64_t B, int64_t C, const float* pred, const float* target,
                     float* loss, float* dpred, void* ws, size_t ws_bytes) {
  if (B <= 0 || C <= 0 || B > (int64_t(1) << 40) / C)
    return fail(DL_INVALID_ARGUMENT, "mse_loss_fwd_bwd: B, C must be positive (B C <= 2^40)");
  if (!pred || !target || !loss) return fail(DL_INVALID_ARGUMENT, "mse_loss_fwd_bwd: pred, target and loss are required");
  const int64_t n = B * C;
  const size_t need = mse_loss_workspace_size(B, C);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "mse_loss_fwd_bwd: workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) % 8) != 0)
    return fail(DL_INVALID_ARGUMENT, "mse_loss_fwd_bwd: workspace must be 8-byte aligned");
  const size_t nb = (size_t)n * 4;
  if ((dpred != pred && overlap(dpred, nb, pred, nb)) || overlap(dpred, nb, target, nb) ||
      overlap(loss, 4, pred, nb) || overlap(loss, 4, target, nb) || overlap(loss, 4, dpred, nb) ||
      overlap(ws, need, pred, nb) || overlap(ws, need, target, nb) || overlap(ws, need, dpred, nb) ||
      overlap(ws, need, loss, 4))
    return fail(DL_ALIASING, "mse_loss_fwd_bwd: outputs overlap inputs (dpred may equal pred)");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = timed("mse", s, [&] {
    return dl::launch_mse(n, pred, target, dpred, static_cast<double*>(ws), loss, s);
  });
  if (e != hipSuccess) return hip_fail(e, "mse_loss_fwd_bwd");
  return DL_OK;
}

static int cast_half(const char* who, const char* label, int half_kind, void* stream, int64_t n,
                     const float* src, void* dst) {
  if (n <= 0) return fail(DL_INVALID_ARGUMENT, "%s: n must be positive", who);
  if (!src || !dst) return fail(DL_INVALID_ARGUMENT, "%s: src and dst are required", who);
  if (overlap(src, n * 4, dst, n * 2)) return fail(DL_ALIASING, "%s: src overlaps dst", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed(label, st, [&] {
    return dl::launch_cast_bf16(n, src, static_cast<dl::bf16_t*>(dst), st, half_kind);
  });
  if (e != hipSuccess) return hip_fail(e, who);
  return DL_OK;
}

static int cast_half_t(const char* who, const char* label, int half_kind, void* stream,
                       int64_t rows, int64_t cols, const float* src, void* dst, void* dst_t) {
  if (!dim_ok(rows) || !dim_ok(cols)) return fail(DL_INVALID_ARGUMENT, "%s: sizes must be in [1, 2^31)", who);
  if (!src || (!dst && !dst_t)) return fail(DL_INVALID_ARGUMENT, "%s: src and an output are required", who);
  const size_t n = (size_t)rows * cols;
  if (overlap(src, n * 4, dst, n * 2) || overlap(src, n * 4, dst_t, n * 2) || overlap(dst, n * 2, dst_t, n * 2))
    return fail(DL_ALIASING, "%s: buffers overlap", who);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed(label, st, [&] {
    return dl::launch_cast_bf16_t(rows, cols, src, static_cast<dl::bf16_t*>(dst),
                                  static_cast<dl::bf16_t*>(dst_t), st, half_kind);
  });
  if (e != hipSuccess) return hip_fail(e, who);
  return DL_OK;
}

int dense_cast_bf16(void* stream, int64_t n, const float* src, void* dst) {
  return cast_half("dense_cast_bf16", "cast_bf16", dl::HK_BF16, stream, n, src, dst);
}

int dense_cast_bf16_t(void* stream, int64_t rows, int64_t cols, const float* src, void* dst,
                      void* dst_t) {
  return cast_half_t("dense_cast_bf16_t", "cast_bf16_t", dl::HK_BF16, stream, rows, cols, src, dst,
                     dst_t);
}

size_t dense_cast_f16_scaled_workspace_size(int64_t n) {
  if (n <= 0) return 0;
  return align_up((size_t)dl::safe_scale_parts(n) * 4);
}

int dense_cast_f16_scaled(void* stream, int64_t n, const float* src, void* dst, float* scale,
                          void* ws, size_t ws_bytes) {
  if (n <= 0) return fail(DL_INVALID_ARGUMENT, "dense_cast_f16_scaled: n must be positive");
  if (!src || !dst || !scale) return fail(DL_INVALID_ARGUMENT, "dense_cast_f16_scaled: src, dst and scale are required");
  const size_t need = dense_cast_f16_scaled_workspace_size(n);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "dense_cast_f16_scaled: workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) % 4) != 0)
    return fail(DL_INVALID_ARGUMENT, "dense_cast_f16_scaled: workspace must be 4-byte aligned");
  if (overlap(src, n * 4, dst, n * 2) || overlap(scale, 4, src, n * 4) || overlap(scale, 4, dst, n * 2) ||
      overlap(ws, need, src, n * 4) || overlap(ws, need, dst, n * 2) || overlap(ws, need, scale, 4))
    return fail(DL_ALIASING, "dense_cast_f16_scaled: buffers overlap");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = timed("cast_f16_scaled", st, [&] {
    return dl::launch_cast_f16_scaled(n, src, static_cast<dl::bf16_t*>(dst), scale,
                                      static_cast<float*>(ws), st);
  });
  if (e != hipSuccess) return hip_fail(e, "dense_cast_f16_scaled");
  return DL_OK;
}

int dense_cast_f16(void* stream, int64_t n, const float* src, void* dst) {
  return cast_half("dense_cast_f16", "cast_f16", dl::HK_F16, stream, n, src, dst);
}

int dense_cast_f16_t(void* stream, int64_t rows, int64_t cols, const float* src, void* dst,
                     void* dst_t) {
  return cast_half_t("dense_cast_f16_t", "cast_f16_t", dl::HK_F16, stream, rows, cols, src, dst,
                     dst_t);
}

// ---- whole MLP step ---------------------------------------------------------
// Workspace: per-layer outputs Y_l [B, out_l] (the last one holds the logits,
// then dlogits in place), the per-row losses, one split-K partial buffer
// per layer whose weight gradient is split along the batch, the K-slices of
// a split forward, and the gradient buffers of paired layers.  During the
// backward pass the dX epilogue of layer l writes
// G_{l-1} = (G_l W_l) * relu'(Y_{l-1}) over Y_{l-1} in place, after layer l's
// dW has consumed Y_{l-1}; a layer whose dW and dX share one launch writes
// G_{l-1} to a gradient buffer instead.  Split weight gradients are not reduced by a pass
// of their own: the optimizer kernel adds the slices, stores dW / db and
// applies the update in one read.

// Whether the last layer runs as the fused narrow head (last Linear +
// softmax-xent + its vjp in one kernel).
static bool mlp_fused_head(int32_t L, const dl_layer_t* layers, bool xent) {
  return xent && dl::head_xent_fits(layers[L - 1].in, layers[L - 1].out);
}

// Whether the last hidden layer, the narrow head and the hidden layer's dX
// fit the tail kernel (shapes only; the step also checks alignment).
static bool mlp_tail_shape(int32_t L, const dl_layer_t* layers, bool xent) {
  return L >= 2 && mlp_fused_head(L, layers, xent) &&
         dl::mlp_tail_fits(layers[L - 2].in, layers[L - 2].out, layers[L - 1].out);
}

// Weight-gradient plan of layer l inside the MLP step.  When the tail
// kernel's hidden layer is layer 1 of a network that fits it, its weight
// gradient shares a launch with the first layer's: it then takes the largest
// power-of-two slice count that keeps both within one round of four
// workgroups per CU (fewer, longer slices for the optimizer to add).  Both
// fusion levels use this plan, so their results stay identical.
static Plan mlp_dw_plan(int64_t B, int32_t L, const dl_layer_t* layers, int l, bool xent) {
  Plan p = plan_gemm(DL_F32, dl::EPI_DW, layers[l].out, layers[l].in, B);
  if (l != 1 || L != 3 || !mlp_tail_shape(L, layers, xent) || p.tile != 1 || p.splits <= 1)
    return p;
  const Plan p0 = plan_gemm(DL_F32, dl::EPI_DW, layers[0].out, layers[0].in, B);
  if (p0.tile != 1) return p;
  const int64_t tiles = ceil_div(layers[l].out, 64) * ceil_div(layers[l].in, 64);
  const int64_t budget = 4 * kCUs - ceil_div(layers[0].out, 64) * ceil_div(layers[0].in, 64) * p0.splits;
  int64_t want = 1;
  while (2 * want <= p.splits && 2 * want * tiles <= budget) want *= 2;
  const int64_t kps = ceil_div(ceil_div(B, want), 32) * 32;
  p.k_per_split = (int)kps;
  p.splits = (int)ceil_div(B, kps);
  if (p.splits <= 1) {
    p.splits = 1;
    p.k_per_split = (int)B;
  }
  return p;
}

// Whether the tail fits its narrow-batch form (16-row tiles; shapes only).
static bool mlp_tail_narrow(int64_t B, int32_t L, const dl_layer_t* layers, bool xent) {
  return mlp_tail_shape(L, layers, xent) &&
         dl::mlp_tail_narrow_fits(B, layers[L - 2].in, layers[L - 2].out, layers[L - 1].out);
}

// Gradient slices a layer's dW / db leave for the optimizer to add up: the
// split-K slices of its weight-gradient GEMM, or the fused head's slices (one
// per 16 rows with the narrow-batch tail, else one per 32-row tile group).
static int64_t mlp_slices(int64_t B, int32_t L, const dl_layer_t* layers, int l, bool xent,
                          bool narrow = false) {
  if (l == L - 1 && mlp_fused_head(L, layers, xent))
    return narrow ? dl::mlp_tail_narrow_slices(B) : dl::head_xent_slices(B);
  return mlp_dw_plan(B, L, layers, l, xent).splits;
}

// Forward of a layer split along K: when its forward product has few tiles
// (a small batch) but a long contraction, the product leaves float32
// K-slices and a finishing kernel adds them in slice order with the bias and
// activation.  The 64-row batch through the 784-input layer: 4 tiles, 5
// slices of 160.
constexpr int kFwdSplitTile = 1;  // 64x64, K step 32
static Plan mlp_fwd_plan(int64_t B, const dl_layer_t& ly) {
  Plan p{kFwdSplitTile, 1, (int)ly.in};
  const int64_t tiles = ceil_div(B, 64) * ceil_div(ly.out, 64);
  const int bk = 32;
  if (tiles > 16 || ly.in < 16 * bk) return p;
  int64_t want = 1;
  while (want * tiles < 64) want *= 2;
  want = std::min<int64_t>(want, ly.in / (4 * bk));
  const int64_t kps = ceil_div(ceil_div(ly.in, want), bk) * bk;
  p.k_per_split = (int)kps;
  p.splits = (int)ceil_div(ly.in, kps);
  if (p.splits <= 1) p = Plan{kFwdSplitTile, 1, (int)ly.in};
  return p;
}

// Whether layer l (l > 0) runs its weight gradient and its dX as one launch:
// both products small (the weight gradient on the 64x64 tile, the dX at
// most 2^33 flop), so that one launch fills the GPU with both.  The dX then
// goes to a gradient buffer of its own, since the weight gradient still reads
// the layer input that the in-place form would overwrite.
static bool mlp_pair(int64_t B, const dl_layer_t& ly) {
  const Plan p = plan_gemm(DL_F32, dl::EPI_DW, ly.out, ly.in, B);
  return p.tile == 1 && 2.0 * (double)B * (double)ly.in * (double)ly.out <= 8589934592.0;
}

// Whether layer l (l > 0, not paired) can take a plain SGD step inside its
// weight-gradient launch: one K slice, so each tile holds its finished dW and
// the epilogue can step W (and b) with it.  Its dX then runs first, into a
// gradient buffer of its own: dX reads W, and the weight gradient still reads
// the layer input that the in-place dX would overwrite.  (Shapes only; the
// step also needs plain SGD with no gradient pass, averages or device step
// count.)
static bool mlp_sgd_in_dw_shape(int64_t B, int32_t L, const dl_layer_t* layers, int l, bool xent) {
  return l > 0 && !mlp_pair(B, layers[l]) && mlp_dw_plan(B, L, layers, l, xent).splits == 1;
}

// Gradient-control partials of the MLP step: one gradient pass over all W and
// b (at most 32 arrays, one launch).
static int64_t mlp_stat_parts(int32_t L, const dl_layer_t* layers) {
  int64_t units = 0;
  for (int l = 0; l < L; ++l) units += units_of(layers[l].out * layers[l].in) + units_of(layers[l].out);
  return dl::stat_grid(units);
}

// `xent`: the loss is softmax cross-entropy (a narrow last layer then runs as
// the fused head); otherwise MSE, whose partial sums take the per-row loss
// region.
static size_t mlp_layout(int64_t B, int32_t L, const dl_layer_t* layers, bool xent,
                         size_t* y_off, size_t* rl_off, size_t* part_off, size_t* fwd_off,
                         size_t* g_off, size_t* g_bytes, size_t* ctl_off) {
  size_t off = 0;
  for (int l = 0; l < L; ++l) {
    y_off[l] = off;
    off += align_up((size_t)B * layers[l].out * 4);
  }
  *rl_off = off;
  off += std::max(align_up((size_t)B * 4), xent ? 0 : align_up((size_t)dl::mse_grid(B * layers[L - 1].out) * 8));
  for (int l = 0; l < L; ++l) {
    part_off[l] = off;
    // room for the slices of either tail form (the form is chosen per call)
    const int64_t S = std::max(mlp_slices(B, L, layers, l, xent),
                               mlp_slices(B, L, layers, l, xent, mlp_tail_narrow(B, L, layers, xent)));
    if (S > 1)
      off += align_up((size_t)S * layers[l].out * layers[l].in * 4) +
             align_up((size_t)S * layers[l].out * 4);
  }
  // the split forwards' K-slices (one layer at a time)
  *fwd_off = off;
  size_t fwd = 0;
  for (int l = 0; l < L; ++l) {
    const Plan p = mlp_fwd_plan(B, layers[l]);
    if (p.splits > 1) fwd = std::max(fwd, align_up((size_t)p.splits * B * layers[l].out * 4));
  }
  off += fwd;
  // gradient buffers of the paired layers (two alternate when several pair)
  const int last_gemm = mlp_fused_head(L, layers, xent) ? L - 2 : L - 1;
  int pairs = 0;
  size_t gb = 0;
  if (L >= 3 && mlp_tail_shape(L, layers, xent)) {  // the tail kernel's dX
    ++pairs;
    gb = align_up((size_t)B * layers[L - 2].in * 4);
  }
  for (int l = 1; l <= last_gemm; ++l)
    if (mlp_pair(B, layers[l]) || mlp_sgd_in_dw_shape(B, L, layers, l, xent)) {
      ++pairs;
      gb = std::max(gb, align_up((size_t)B * layers[l].in * 4));
    }
  *g_off = off;
  *g_bytes = gb;
  off += (size_t)std::min(pairs, 2) * gb;
  *ctl_off = off;
  return off + ctl_bytes(mlp_stat_parts(L, layers));
}

size_t mlp_train_step_workspace_size(int64_t B, int32_t n_layers, const dl_layer_t* layers) {
  if (!dim_ok(B) || n_layers < 1 || n_layers > 16 || !layers) return 0;
  for (int l = 0; l < n_layers; ++l)
    if (!dim_ok(layers[l].in) || !dim_ok(layers[l].out)) return 0;
  size_t y_off[16], rl, part[16], fwd, g_off, g_bytes, ctl_off;
  // the larger of the cross-entropy and the MSE layouts, so one workspace
  // serves both steps
  const size_t a = mlp_layout(B, n_layers, layers, true, y_off, &rl, part, &fwd, &g_off, &g_bytes,
                              &ctl_off);
  const size_t b = mlp_layout(B, n_layers, layers, false, y_off, &rl, part, &fwd, &g_off, &g_bytes,
                              &ctl_off);
  return std::max(a, b);
}

}  // extern "C"

// The whole step for either loss: softmax cross-entropy against `labels`, or
// (labels null) the mean squared error against `targets`.
static int mlp_step(void* stream, int64_t B, int32_t n_layers, const dl_layer_t* layers,
                    const float* X, const int32_t* labels, const float* targets,
                    const dl_opt_t* opt, float* loss, void* ws, size_t ws_bytes) {
  const bool xent = labels != nullptr;
  if (!dim_ok(B)) return fail(DL_INVALID_ARGUMENT, "mlp_train_step: B must be in [1, 2^31)");
  if (n_layers < 1 || n_layers > 16 || !layers)
    return fail(DL_INVALID_ARGUMENT, "mlp_train_step: n_layers must be in [1, 16]");
  if (!X || (!labels && !targets) || !opt || !loss)
    return fail(DL_INVALID_ARGUMENT, "mlp_train_step: X, labels (targets), opt and loss are required");
  const bool any_ema = layers && n_layers >= 1 && layers[0].eW != nullptr;
  if (int st = check_opt(opt, "mlp_train_step", any_ema)) return st;
  const bool adam = opt->kind != DL_OPT_SGD;
  int n_tensors = 0;
  for (int l = 0; l < n_layers; ++l) {
    const dl_layer_t& ly = layers[l];
    if (!dim_ok(ly.in) || !dim_ok(ly.out)) return fail(DL_INVALID_ARGUMENT, "mlp_train_step: layer %d has a bad shape", l);
    if (l > 0 && ly.in != layers[l - 1].out)
      return fail(DL_INVALID_ARGUMENT, "mlp_train_step: layer %d in=%lld != layer %d out=%lld", l,
                  (long long)ly.in, l - 1, (long long)layers[l - 1].out);
    if (ly.act != DL_ACT_IDENTITY && ly.act != DL_ACT_RELU)
      return fail(ly.act == DL_ACT_GELU_TANH ? DL_UNSUPPORTED : DL_INVALID_ARGUMENT,
                  "mlp_train_step: layer %d activation %d (identity or ReLU only)", l, ly.act);
    if (!ly.W || !ly.b || !ly.dW || !ly.db)
      return fail(DL_INVALID_ARGUMENT, "mlp_train_step: layer %d needs W, b, dW and db", l);
    if (adam && (!ly.mW || !ly.vW || !ly.mb || !ly.vb))
      return fail(DL_INVALID_ARGUMENT, "mlp_train_step: layer %d needs Adam moments", l);
    if ((ly.eW != nullptr) != any_ema || (ly.eb != nullptr) != any_ema)
      return fail(DL_INVALID_ARGUMENT, "mlp_train_step: parameter averages for all layers or none");
    if (overlap(ly.dW, ly.out * ly.in * 4, ly.W, ly.out * ly.in * 4) || overlap(ly.db, ly.out * 4, ly.b, ly.out * 4))
      return fail(DL_ALIASING, "mlp_train_step: layer %d gradient overlaps its parameters", l);
    n_tensors += 2;
  }
  if (n_tensors > dl::kMaxSegs) return fail(DL_UNSUPPORTED, "mlp_train_step: too many layers");
  // The loss pass overwrites the logits with dlogits, so the last layer has no
  // activation of its own (its derivative would need the overwritten output).
  if (layers[n_layers - 1].act != DL_ACT_IDENTITY)
    return fail(DL_UNSUPPORTED, "mlp_train_step: the last layer must be the identity");
  if (!xent && overlap(targets, (size_t)B * layers[n_layers - 1].out * 4, X,
                       (size_t)B * layers[0].in * 4))
    return fail(DL_ALIASING, "mlp_train_step: targets overlap X");
  size_t y_off[16], rl_off, part_off[16], fwd_off, g_off, g_bytes, ctl_off;
  const size_t need = mlp_layout(B, n_layers, layers, xent, y_off, &rl_off, part_off, &fwd_off,
                                 &g_off, &g_bytes, &ctl_off);
  if (!ws || ws_bytes < need)
    return fail(DL_WORKSPACE_TOO_SMALL, "mlp_train_step: workspace %zu bytes, need %zu", ws_bytes, need);
  if ((reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(DL_INVALID_ARGUMENT, "mlp_train_step: workspace must be 256-byte aligned");

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (xent) {  // the per-row loss region is free until the loss runs
    const int vs = check_labels("mlp_train_step", s, B, layers[n_layers - 1].out, labels,
                                static_cast<char*>(ws) + rl_off);
    if (vs != DL_OK) return vs;
  }
  char* base = static_cast<char*>(ws);
  const bool dev_step = opt->step_dev != nullptr;
  // with clipping or loss scaling a gradient pass precedes the update and its
  // control kernel advances the device step count (unless the step is skipped)
  const bool ctl_on = opt->max_grad_norm > 0.0 || opt->scaler != nullptr;
  const float* dscale = opt->scaler != nullptr ? opt->scaler->scale : nullptr;
  if (dev_step && !ctl_on) {
    hipError_t et = dl::launch_step_tick(opt->step_dev, s);
    if (et != hipSuccess) return hip_fail(et, "mlp_train_step (step count)");
  }
  float* Y[16];
  for (int l = 0; l < n_layers; ++l) Y[l] = reinterpret_cast<float*>(base + y_off[l]);
  float* row_loss = reinterpret_cast<float*>(base + rl_off);
  const int L = n_layers;
  const int64_t C = layers[L - 1].out;
  hipError_t e;

  // With a narrow last layer the logits never reach HBM: one kernel runs its
  // forward, the softmax-xent and its vjp (dX written over Y[L-2], dW / db as
  // slices for the optimizer).
  const bool fused = mlp_fused_head(L, layers, xent);
  // With a small last hidden layer the tail kernel also runs that layer's
  // forward and dX, so its output never reaches HBM either: it writes the
  // layer's output gradient into Y[L-2] and the dX into a gradient buffer.
  auto al16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; };
  const bool tail = g_mlp_fusion >= 2 && mlp_tail_shape(L, layers, xent) &&
                    al16(layers[L - 2].W) && (L >= 3 || al16(X));
  // a small batch takes the tail's narrow form, which also finishes the
  // split-K forward of the layer before it
  const bool narrow = tail && mlp_tail_narrow(B, L, layers, xent);
  const float* fold_part = nullptr;
  int fold_splits = 0;
  const int last_gemm = tail ? L - 3 : fused ? L - 2 : L - 1;
  float* gbuf[2] = {reinterpret_cast<float*>(base + g_off),
                    reinterpret_cast<float*>(base + g_off + g_bytes)};
  // forward
  for (int l = 0; l <= last_gemm; ++l) {
    const dl_layer_t& ly = layers[l];
    const float* in = l == 0 ? X : Y[l - 1];
    const Plan fp = mlp_fwd_plan(B, ly);
    if (fp.splits > 1) {
      float* slices = reinterpret_cast<float*>(base + fwd_off);
      dl::GemmDesc d = blank_desc();
      d.M = (int)B; d.N = (int)ly.out; d.K = (int)ly.in;
      d.A = in; d.lda = ly.in; d.a_layout = dl::K_MAJOR;
      d.B = ly.W; d.ldb = ly.in; d.b_layout = dl::K_MAJOR;
      d.C = slices; d.ldc = ly.out;
      d.epi = dl::EPI_DW;  // float32 slices, no column sums
      d.splits = fp.splits; d.k_per_split = fp.k_per_split;
      d.partial = slices;
      // before the narrow tail: the slices on 16-row tiles (the tail adds them)
      const bool fwd_narrow =
          narrow && l == last_gemm && dl::mlp_fwd_narrow_fits(B, ly.in, ly.out, fp.k_per_split) &&
          al16(in) && al16(ly.W);
      e = timed("fwd_gemm", s, [&] {
        return fwd_narrow ? dl::launch_mlp_fwd_narrow((int)B, (int)ly.in, (int)ly.out, fp.splits,
                                                      fp.k_per_split, in, ly.W, slices, s)
                          : dl::launch_gemm_f32(d, fp.tile, s);
      });
      if (narrow && l == last_gemm) {  // the tail finishes it
        fold_part = slices;
        fold_splits = fp.splits;
      } else if (e == hipSuccess)
        e = timed("fwd_finish", s, [&] {
          return dl::launch_splitk_finish_fwd((int)B, (int)ly.out, fp.splits, slices, ly.b, ly.act,
                                              Y[l], s);
        });
    } else {
      e = fwd_gemm(DL_F32, ly.act, B, ly.in, ly.out, in, ly.W, ly.b, Y[l], nullptr, s);
    }
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (forward)");
  }
  if (tail) {
    const dl_layer_t& hl = layers[L - 2];
    const dl_layer_t& ly = layers[L - 1];
    const int64_t S = mlp_slices(B, L, layers, L - 1, xent, narrow);
    char* pb = base + part_off[L - 1];
    float* dWp = S > 1 ? reinterpret_cast<float*>(pb) : ly.dW;
    float* dbp = S > 1 ? reinterpret_cast<float*>(pb + align_up((size_t)S * ly.out * ly.in * 4))
                       : ly.db;
    const float* Hin = L >= 3 ? Y[L - 3] : X;
    float* dH = L >= 3 ? gbuf[0] : nullptr;
    const int act0 = L >= 3 ? layers[L - 3].act : DL_ACT_IDENTITY;
    if (narrow) {
      // with a fold the kernel writes Y[L-3]; without one it only reads Hin
      e = timed("mlp_tail", s, [&] {
        return dl::launch_mlp_tail_narrow(B, (int)hl.in, (int)hl.out, (int)ly.out,
                                          const_cast<float*>(Hin), fold_part, fold_splits,
                                          fold_splits > 0 ? layers[L - 3].b : nullptr, hl.W, hl.b,
                                          hl.act, act0, ly.W, ly.b, labels, row_loss, Y[L - 2], dH,
                                          dWp, dbp, s, dscale);
      });
    } else {
      e = timed("mlp_tail", s, [&] {
        return dl::launch_mlp_tail(B, (int)hl.in, (int)hl.out, (int)ly.out, Hin, hl.W, hl.b,
                                   hl.act, act0, ly.W, ly.b, labels, row_loss, Y[L - 2], dH, dWp,
                                   dbp, s, dscale);
      });
    }
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (tail)");
  } else if (fused) {
    const dl_layer_t& ly = layers[L - 1];
    const int64_t S = dl::head_xent_slices(B);
    // one slice (B <= 32): straight into dW / db, where the optimizer reads it
    char* pb = base + part_off[L - 1];
    float* dWp = S > 1 ? reinterpret_cast<float*>(pb) : ly.dW;
    float* dbp = S > 1 ? reinterpret_cast<float*>(pb + align_up((size_t)S * ly.out * ly.in * 4))
                       : ly.db;
    const float* H = L > 1 ? Y[L - 2] : X;
    float* dH = L > 1 ? Y[L - 2] : nullptr;
    const int prev_act = L > 1 ? layers[L - 2].act : DL_ACT_IDENTITY;
    e = timed("head_xent", s, [&] {
      return dl::launch_head_xent(B, (int)ly.in, (int)ly.out, H, dH, prev_act, ly.W, ly.b, labels,
                                  row_loss, dWp, dbp, s, dscale);
    });
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (head)");
  } else if (xent) {
    // loss + dlogits (in place over the logits)
    e = timed("xent", s, [&] {
      return dl::launch_xent(B, C, Y[L - 1], labels, row_loss, Y[L - 1], loss, s, dscale);
    });
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (xent)");
  } else {
    // MSE + dpred (in place over the predictions); its partial sums use the
    // per-row loss region
    e = timed("mse", s, [&] {
      return dl::launch_mse(B * C, Y[L - 1], targets, Y[L - 1], reinterpret_cast<double*>(row_loss),
                            loss, s, dscale);
    });
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (mse)");
  }
  // backward; G holds the current layer's output gradient
  const float* G = last_gemm >= 0 ? Y[last_gemm] : nullptr;
  int first_bwd = last_gemm;
  bool sgd_in_dw = false;  // the SGD step ran inside the weight-gradient launch
  if (tail) {
    // the weight gradient of the tail's hidden layer (its output gradient in
    // Y[L-2]), in one launch with the first layer's when that layer comes
    // right before it (the first layer has no dX)
    const int lh = L - 2;
    const dl_layer_t& hl = layers[lh];
    const float* Hin = lh >= 1 ? Y[lh - 1] : X;
    const Plan ph = mlp_dw_plan(B, L, layers, lh, xent);
    const Plan p0 = mlp_dw_plan(B, L, layers, 0, xent);
    if (lh == 1 && ph.tile == 1 && p0.tile == 1) {
      dl::GemmDesc d0 = dw_desc(DL_F32, B, layers[0].in, layers[0].out, gbuf[0], X, layers[0].dW,
                                layers[0].db, base + part_off[0], p0);
      dl::GemmDesc dh = dw_desc(DL_F32, B, hl.in, hl.out, Y[lh], Hin, hl.dW, hl.db,
                                base + part_off[lh], ph);
      // Plain SGD of the three-layer network: the two weight gradients take
      // their SGD steps in their epilogue and one more workgroup of the same
      // launch adds up the head's slices, steps the head and forms the loss
      // mean, so the step needs no optimizer launch (the same arithmetic as
      // that launch, so the same results).
      auto same16 = [](const void* a, const void* b) {
        return ((reinterpret_cast<uintptr_t>(a) ^ reinterpret_cast<uintptr_t>(b)) & 15) == 0;
      };
      sgd_in_dw = L == 3 && opt->kind == DL_OPT_SGD && !ctl_on && !dev_step && !any_ema &&
                  p0.splits == 1 && ph.splits == 1 && same16(layers[0].W, layers[0].dW) &&
                  same16(hl.W, hl.dW);
      dl::SgdFinish fin{};
      if (sgd_in_dw) {
        const float lr = opt_consts(*opt, opt->step).lr;
        d0.sgd_w = layers[0].W; d0.sgd_b = layers[0].b; d0.sgd_lr = lr;
        dh.sgd_w = hl.W; dh.sgd_b = hl.b; dh.sgd_lr = lr;
        const dl_layer_t& ly = layers[L - 1];
        const int64_t S = mlp_slices(B, L, layers, L - 1, xent, narrow);
        char* pb = base + part_off[L - 1];
        fin.W = ly.W; fin.b = ly.b; fin.dW = ly.dW; fin.db = ly.db;
        fin.dW_part = S > 1 ? reinterpret_cast<const float*>(pb) : nullptr;
        fin.db_part = S > 1 ? reinterpret_cast<const float*>(pb + align_up((size_t)S * ly.out * ly.in * 4))
                            : nullptr;
        fin.n_w = ly.out * ly.in;
        fin.n_b = (int)ly.out;
        fin.slices = (int)S;
        fin.lr = lr;
        fin.rows = B;
        fin.row_loss = row_loss;
        fin.loss = loss;
      }
      e = timed("dwdw_gemm", s, [&] {
        return dl::launch_gemm_f32_dw_dw(d0, dh, s, sgd_in_dw ? &fin : nullptr);
      });
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dW + dW)");
      first_bwd = -1;
    } else {
      e = dw_gemm(DL_F32, B, hl.in, hl.out, Y[lh], Hin, hl.dW, hl.db, base + part_off[lh], s,
                  /*reduce=*/false, nullptr, &ph);
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dW)");
      G = gbuf[0];
    }
  }
  // plain SGD: layers whose weight gradient has one K slice step W and b in
  // its epilogue (the same arithmetic as the optimizer launch), after their dX
  const bool sgd_epi = opt->kind == DL_OPT_SGD && !ctl_on && !dev_step && !any_ema;
  const float sgd_lr = sgd_epi ? opt_consts(*opt, opt->step).lr : 0.0f;
  bool stepped[16] = {};
  for (int l = first_bwd; l >= 0; --l) {
    const dl_layer_t& ly = layers[l];
    const float* in = l == 0 ? X : Y[l - 1];
    if (sgd_epi && mlp_sgd_in_dw_shape(B, L, layers, l, xent) &&
        ((reinterpret_cast<uintptr_t>(ly.W) ^ reinterpret_cast<uintptr_t>(ly.dW)) & 15) == 0) {
      float* Gn = G == gbuf[0] ? gbuf[1] : gbuf[0];
      e = dx_gemm(DL_F32, B, ly.in, ly.out, G, ly.W, nullptr, Gn, layers[l - 1].act, Y[l - 1], s);
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dX)");
      const Plan pl = mlp_dw_plan(B, L, layers, l, xent);
      dl::GemmDesc d = dw_desc(DL_F32, B, ly.in, ly.out, G, in, ly.dW, ly.db, nullptr, pl);
      d.sgd_w = ly.W;
      d.sgd_b = ly.b;
      d.sgd_lr = sgd_lr;
      e = timed("dw_gemm", s, [&] { return run_gemm(DL_F32, d, pl.tile, s); });
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dW + SGD)");
      stepped[l] = true;
      G = Gn;
      continue;
    }
    if (l > 0 && mlp_pair(B, ly)) {
      float* Gn = G == gbuf[0] ? gbuf[1] : gbuf[0];
      const Plan p = mlp_dw_plan(B, L, layers, l, xent);
      const dl::GemmDesc dw = dw_desc(DL_F32, B, ly.in, ly.out, G, in, ly.dW, ly.db,
                                      base + part_off[l], p);
      const dl::GemmDesc dx = dx_desc(B, ly.in, ly.out, G, ly.W, nullptr, Gn, layers[l - 1].act,
                                      Y[l - 1]);
      e = timed("dwdx_gemm", s, [&] { return dl::launch_gemm_f32_dw_dx(dw, dx, s); });
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dW + dX)");
      G = Gn;
      continue;
    }
    const Plan pl = mlp_dw_plan(B, L, layers, l, xent);
    e = dw_gemm(DL_F32, B, ly.in, ly.out, G, in, ly.dW, ly.db, base + part_off[l], s,
                /*reduce=*/false, nullptr, &pl);
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dW)");
    if (l > 0) {
      e = dx_gemm(DL_F32, B, ly.in, ly.out, G, ly.W, nullptr, Y[l - 1], layers[l - 1].act,
                  Y[l - 1], s);
      if (e != hipSuccess) return hip_fail(e, "mlp_train_step (dX)");
      G = Y[l - 1];
    }
  }
  if (sgd_in_dw) return DL_OK;
  // optimizer over every W and b in one launch (finishing split-K sums, or,
  // with the gradient control on, after the gradient pass has finished them)
  dl::OptSegs segs = blank_segs();
  dl::OptSegs stat = blank_segs();
  int64_t blocks = 0, units = 0;
  for (int l = 0; l < L; ++l) {
    if (stepped[l]) continue;  // stepped inside its weight-gradient launch
    const dl_layer_t& ly = layers[l];
    const int64_t S = mlp_slices(B, L, layers, l, xent, narrow);
    char* pb = base + part_off[l];
    float* ws_[2] = {ly.W, ly.b};
    float* gs_[2] = {ly.dW, ly.db};
    float* ms_[2] = {ly.mW, ly.mb};
    float* vs_[2] = {ly.vW, ly.vb};
    float* es_[2] = {ly.eW, ly.eb};
    const int64_t ns_[2] = {ly.out * ly.in, ly.out};
    const float* ps_[2] = {reinterpret_cast<float*>(pb),
                           reinterpret_cast<float*>(pb + align_up((size_t)S * ly.out * ly.in * 4))};
    for (int t = 0; t < 2; ++t) {
      if (ctl_on) {
        add_seg(stat, units, true, ns_[t], ws_[t], gs_[t], nullptr, nullptr, nullptr, nullptr,
                ps_[t], (int)S, gs_[t]);
        add_seg(segs, blocks, false, ns_[t], ws_[t], gs_[t], ms_[t], vs_[t], es_[t], nullptr,
                nullptr, 1, gs_[t]);
      } else {
        add_seg(segs, blocks, false, ns_[t], ws_[t], gs_[t], ms_[t], vs_[t], es_[t], nullptr,
                ps_[t], (int)S, gs_[t]);
      }
    }
  }
  if (fused) {  // the loss mean rides on the optimizer launch
    segs.row_loss = row_loss;
    segs.rows = B;
    segs.loss = loss;
  }
  dl::OptConsts oc = opt_consts(*opt, dev_step ? 0 : opt->step);
  if (dev_step) oc.step_dev = opt->step_dev;
  if (ctl_on) {
    const int64_t parts = mlp_stat_parts(L, layers);
    const CtlMem mem = ctl_mem(base + ctl_off, parts);
    e = timed("grad_stats", s, [&] { return dl::launch_grad_stats(stat, units, mem.sq, mem.bad, s); });
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (gradient pass)");
    const dl::CtlArgs a = ctl_args(opt, mem, parts);
    e = timed("grad_ctl", s, [&] { return dl::launch_grad_ctl(a, s); });
    if (e != hipSuccess) return hip_fail(e, "mlp_train_step (gradient control)");
    oc.ctl = mem.ctl;
  }
  static const char* const kOptNames[3] = {"sgd_multi", "adamw_multi", "adam_multi"};
  e = timed(kOptNames[opt->kind], s, [&] { return dl::launch_opt_multi(segs, opt->kind, oc, s); });
  if (e != hipSuccess) return hip_fail(e, "mlp_train_step (optimizer)");
  return DL_OK;
}

extern "C" {

int mlp_train_step(void* stream, int64_t B, int32_t n_layers, const dl_layer_t* layers,
                   const float* X, const int32_t* labels, const dl_opt_t* opt, float* loss,
                   void* ws, size_t ws_bytes) {
  if (!labels) return fail(DL_INVALID_ARGUMENT, "mlp_train_step: labels are required");
  return mlp_step(stream, B, n_layers, layers, X, labels, nullptr, opt, loss, ws, ws_bytes);
}

int mlp_train_step_mse(void* stream, int64_t B, int32_t n_layers, const dl_layer_t* layers,
                       const float* X, const float* targets, const dl_opt_t* opt, float* loss,
                       void* ws, size_t ws_bytes) {
  if (!targets) return fail(DL_INVALID_ARGUMENT, "mlp_train_step_mse: targets are required");
  return mlp_step(stream, B, n_layers, layers, X, nullptr, targets, opt, loss, ws, ws_bytes);
}

}  // extern "C"

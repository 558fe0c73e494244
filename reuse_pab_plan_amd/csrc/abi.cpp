// abi.cpp -- exported attention and MSE entry points: argument validation
// (before any HIP call), error text, and dispatch to the kernel launchers.
#include "abi.hpp"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "launch.hpp"

namespace pab {

namespace {
thread_local std::string g_last_error;

constexpr int64_t kMaxElems = (int64_t)1 << 40;  // sanity bound on tensor sizes

bool dims_ok(std::initializer_list<int64_t> dims, int64_t* total) {
  int64_t t = 1;
  for (int64_t d : dims) {
    if (d <= 0) return false;
    if (t > kMaxElems / d) return false;
    t *= d;
  }
  *total = t;
  return true;
}

bool d_supported(int32_t D) { return D >= 8 && D <= 128 && D % 8 == 0; }

}  // namespace

std::string fmt(const char* f, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, f);
  vsnprintf(buf, sizeof buf, f, ap);
  va_end(ap);
  return buf;
}

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}
int ok() {
  g_last_error.clear();
  return PAB_OK;
}
int device_error(const char* what, int hip_err) {
  return fail(PAB_ERR_DEVICE, fmt("%s: HIP error %d (%s)", what, hip_err,
                                  hipGetErrorString((hipError_t)hip_err)));
}

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

size_t dtype_size(int32_t dtype) { return dtype == PAB_BF16 ? 2 : (dtype == PAB_F32 ? 4 : 0); }

static int check_common(const char* fn, int32_t D, int32_t dtype, float scale) {
  if (dtype != PAB_BF16 && dtype != PAB_F32)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: unsupported dtype %d", fn, dtype));
  if (!d_supported(D))
    return fail(PAB_ERR_UNSUPPORTED,
                fmt("%s: head dim D=%d unsupported (need a multiple of 8 in [8, 128])", fn, D));
  if (!(scale >= 0.f) || !std::isfinite(scale))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: softmax_scale must be finite and >= 0", fn));
  return PAB_OK;
}

int check_video_attn(const char* fn, const void* q, const void* k, const void* v, const void* o,
                     int32_t B, int32_t H, int32_t F, int32_t S, int32_t D, int32_t dtype,
                     float scale, bool temporal) {
  if (!q || !k || !v || !o) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: pointers must be 16-byte aligned", fn));
  int64_t n = 0;
  if (!dims_ok({B, H, F, S, D}, &n))
    return fail(PAB_ERR_INVALID_ARG,
                fmt("%s: bad shape B=%d H=%d F=%d S=%d D=%d", fn, B, H, F, S, D));
  int st = check_common(fn, D, dtype, scale);
  if (st) return st;
  if (temporal && F > 64)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: F=%d frames unsupported (max 64)", fn, F));
  // The bf16 kernels address one (b, h) slab (temporal) or one sequence
  // (spatial) with 32-bit byte offsets.
  const int64_t slab = temporal ? (int64_t)F * S * D * 2 : (int64_t)S * D * 2;
  if (dtype == PAB_BF16 && slab >= ((int64_t)1 << 32))
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: %s of %lld bytes exceeds 4 GiB", fn,
                                         temporal ? "(b, h) slab" : "sequence", (long long)slab));
  const size_t bytes = (size_t)n * dtype_size(dtype);
  if (ranges_overlap(o, bytes, q, bytes) || ranges_overlap(o, bytes, k, bytes) ||
      ranges_overlap(o, bytes, v, bytes))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: output overlaps an input", fn));
  return PAB_OK;
}

int check_cross_attn(const void* q, const void* kt, const void* vt, const void* o, int32_t B,
                     int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype, float scale,
                     const int32_t* text_len) {
  const char* fn = text_len ? "pab_attn_cross_masked" : "pab_attn_cross";
  if (!q || !kt || !vt || !o) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (!aligned16(q) || !aligned16(kt) || !aligned16(vt) || !aligned16(o))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: pointers must be 16-byte aligned", fn));
  int64_t nq_el = 0, nk_el = 0;
  if (!dims_ok({B, H, Nq, D}, &nq_el) || !dims_ok({B, H, L, D}, &nk_el))
    return fail(PAB_ERR_INVALID_ARG,
                fmt("%s: bad shape B=%d H=%d Nq=%lld L=%d D=%d", fn, B, H, (long long)Nq, L, D));
  int st = check_common(fn, D, dtype, scale);
  if (st) return st;
  if (L > 128) return fail(PAB_ERR_UNSUPPORTED, fmt("%s: L=%d text tokens unsupported (max 128)", fn, L));
  if (text_len)
    for (int32_t b = 0; b < B; ++b)
      if (text_len[b] < 1 || text_len[b] > L)
        return fail(PAB_ERR_INVALID_ARG,
                    fmt("%s: text_len[%d]=%d outside [1, L=%d]", fn, b, text_len[b], L));
  if (Nq > ((int64_t)1 << 31) * 32)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: Nq too large", fn));
  const size_t es = dtype_size(dtype);
  const size_t qb = (size_t)nq_el * es, kb = (size_t)nk_el * es;
  if (ranges_overlap(o, qb, q, qb) || ranges_overlap(o, qb, kt, kb) || ranges_overlap(o, qb, vt, kb))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: output overlaps an input", fn));
  return PAB_OK;
}

int check_mse(const void* a, const void* b, int64_t n, int32_t dtype, const double* out,
              const void* ws, size_t ws_bytes) {
  const char* fn = "pab_attn_diff_mse";
  if (!a || !b || !out || !ws) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (!aligned16(a) || !aligned16(b) || !aligned16(ws) || ((uintptr_t)out & 7u))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: misaligned pointer", fn));
  if (n < 1 || n > kMaxElems) return fail(PAB_ERR_INVALID_ARG, fmt("%s: bad n=%lld", fn, (long long)n));
  if (dtype != PAB_BF16 && dtype != PAB_F32)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: unsupported dtype %d", fn, dtype));
  const size_t need = pab_mse_workspace_bytes(n);
  if (ws_bytes < need)
    return fail(PAB_ERR_CAPACITY, fmt("%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need));
  return PAB_OK;
}

static float resolve_scale(float scale, int32_t D) {
  return scale == 0.f ? (float)(1.0 / std::sqrt((double)D)) : scale;
}

int run_spatial(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                int32_t F, int32_t S, int32_t D, int32_t dtype, float scale, void* stream,
                const DiffOut* diff) {
  const float c = resolve_scale(scale, D);
  hipError_t e;
  if (diff && diff->nparts) *diff->nparts = 0;
  if (dtype == PAB_BF16) {
    e = launch_spatial_bf16(q, k, v, o, (int64_t)B * H * F, S, D, c, diff ? *diff : DiffOut{},
                            (hipStream_t)stream);
  } else {
    SeqLayout lay{(int64_t)B * H * F, 1, (int64_t)S * D, 0, D, (int64_t)S * D, 0, D, S, S};
    e = launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lay, D, c,
                        (hipStream_t)stream);
  }
  return e == hipSuccess ? ok() : device_error("pab_attn_spatial launch", e);
}

int run_temporal(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                 int32_t F, int32_t S, int32_t D, int32_t dtype, float scale, void* stream,
                 const DiffOut* diff) {
  const float c = resolve_scale(scale, D);
  hipError_t e;
  if (diff && diff->nparts) *diff->nparts = 0;
  if (dtype == PAB_BF16) {
    e = launch_temporal_bf16(q, k, v, o, (int64_t)B * H, F, S, D, c, diff ? *diff : DiffOut{},
                             (hipStream_t)stream);
  } else {
    const int64_t fs = (int64_t)F * S * D;
    SeqLayout lay{(int64_t)B * H * S, S, fs, D, (int64_t)S * D, fs, D, (int64_t)S * D, F, F};
    e = launch_attn_f32((const float*)q, (const float*)k, (const float*)v, (float*)o, lay, D, c,
                        (hipStream_t)stream);
  }
  return e == hipSuccess ? ok() : device_error("pab_attn_temporal launch", e);
}

int run_cross(const void* q, const void* kt, const void* vt, void* o, int32_t B, int32_t H,
              int64_t Nq, int32_t L, int32_t D, int32_t dtype, float scale,
              const int32_t* text_len, void* stream, const DiffOut* diff) {
  const float c = resolve_scale(scale, D);
  if (diff && diff->nparts) *diff->nparts = 0;
  bool full = true;
  if (text_len)
    for (int32_t b = 0; b < B; ++b) full = full && text_len[b] == L;
  const size_t es = dtype_size(dtype);
  // All text tokens real: one launch.  Otherwise one launch per batch entry,
  // each over that entry's real tokens (rows stay L apart in memory).  With a
  // fused difference each launch writes its partials after the previous
  // one's; if one of them cannot (workspace), none counts and the caller
  // takes the difference in a separate pass.
  const int32_t parts = full ? 1 : B;
  const bool fuse = diff && diff->prev && diff->nparts && dtype == PAB_BF16;
  int64_t total_parts = 0;
  bool all_fused = true;
  for (int32_t b = 0; b < parts; ++b) {
    const int64_t nbh = full ? (int64_t)B * H : H;
    const int32_t len = full ? L : text_len[b];
    const size_t qo = full ? 0 : (size_t)b * H * Nq * D * es;
    const size_t ko = full ? 0 : (size_t)b * H * L * D * es;
    const char* qb = (const char*)q + qo;
    const char* kb = (const char*)kt + ko;
    const char* vb = (const char*)vt + ko;
    char* ob = (char*)o + qo;
    hipError_t e;
    if (dtype == PAB_BF16) {
      DiffOut db;
      int np = 0;
      if (fuse) {
        db.prev = (const char*)diff->prev + qo;
        db.partials = diff->partials + total_parts;
        db.capacity = diff->capacity - total_parts;
        db.nparts = &np;
      }
      e = launch_cross_bf16(qb, kb, vb, ob, nbh, Nq, len, L, D, c, db, (hipStream_t)stream);
      if (fuse) {
        all_fused = all_fused && np > 0;
        total_parts += np;
      }
    } else {
      SeqLayout lay{nbh, 1, Nq * D, 0, D, (int64_t)L * D, 0, D, Nq, len};
      e = launch_attn_f32((const float*)qb, (const float*)kb, (const float*)vb, (float*)ob, lay, D,
                          c, (hipStream_t)stream);
    }
    if (e != hipSuccess) return device_error("pab_attn_cross launch", e);
  }
  if (fuse && all_fused) *diff->nparts = (int)total_parts;
  return ok();
}

int run_mse(const void* a, const void* b, int64_t n, int32_t dtype, double* out, void* ws,
            void* stream) {
  hipError_t e = launch_mse(a, b, n, dtype, out, (double*)ws, (hipStream_t)stream);
  return e == hipSuccess ? ok() : device_error("pab_attn_diff_mse launch", e);
}

int run_mse_final(const double* partials, int nparts, int64_t n, double* out, void* stream) {
  hipError_t e = launch_mse_final(partials, nparts, n, out, (hipStream_t)stream);
  return e == hipSuccess ? ok() : device_error("pab_step_dispatch(attention difference)", e);
}


int check_proj(const char* fn, const void* x, const void* w, void* const outs[3], int32_t n_out,
               int32_t B, int32_t F, int32_t S, int32_t H, int32_t D, int32_t dtype, bool in) {
  if (!x || !w) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (n_out < 1 || n_out > 3)
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: n_out must be 1, 2 or 3", fn));
  for (int i = 0; i < n_out; ++i)
    if (!outs[i] || !aligned16(outs[i]))
      return fail(PAB_ERR_INVALID_ARG, fmt("%s: output %d NULL or not 16-byte aligned", fn, i));
  if (!aligned16(x) || !aligned16(w))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: pointers must be 16-byte aligned", fn));
  int64_t n = 0;
  if (!dims_ok({B, H, F, S, D}, &n))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: bad shape B=%d H=%d F=%d S=%d D=%d", fn, B, H, F, S, D));
  if (dtype != PAB_BF16)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: only bf16 projections are built", fn));
  if (!d_supported(D)) return fail(PAB_ERR_UNSUPPORTED, fmt("%s: head dim D=%d unsupported", fn, D));
  const int64_t C = (int64_t)H * D;
  if (C % 32 != 0 || C > 16384)
    return fail(PAB_ERR_UNSUPPORTED,
                fmt("%s: hidden size H*D=%lld must be a multiple of 32, <= 16384", fn, (long long)C));
  const size_t bytes = (size_t)n * 2;
  if (bytes >= ((size_t)1 << 32))
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: tensors of 4 GiB or more are not supported", fn));
  const size_t wbytes = (size_t)(in ? n_out : 1) * C * C * 2;
  for (int i = 0; i < n_out; ++i) {
    if (ranges_overlap(outs[i], bytes, x, bytes) || ranges_overlap(outs[i], bytes, w, wbytes))
      return fail(PAB_ERR_INVALID_ARG, fmt("%s: output %d overlaps an input", fn, i));
    for (int j = 0; j < i; ++j)
      if (ranges_overlap(outs[i], bytes, outs[j], bytes))
        return fail(PAB_ERR_INVALID_ARG, fmt("%s: outputs %d and %d overlap", fn, j, i));
  }
  return PAB_OK;
}

int run_proj_in(const void* x, const void* w, void* const outs[3], int32_t n_out, int32_t B,
                int32_t F, int32_t S, int32_t H, int32_t D, void* stream) {
  const int64_t C = (int64_t)H * D, T = (int64_t)F * S;
  void* o3[3] = {outs[0], n_out > 1 ? outs[1] : nullptr, n_out > 2 ? outs[2] : nullptr};
  hipError_t e = launch_proj_bf16(x, w, o3, (int64_t)B * T, (int)(n_out * C), (int)C, (int)T, H,
                                  D, false, true, (hipStream_t)stream);
  return e == hipSuccess ? ok() : device_error("pab_proj_in launch", e);
}

int run_proj_out(const void* o, const void* w, void* y, int32_t B, int32_t F, int32_t S, int32_t H,
                 int32_t D, void* stream) {
  const int64_t C = (int64_t)H * D, T = (int64_t)F * S;
  void* outs[3] = {y, nullptr, nullptr};
  hipError_t e = launch_proj_bf16(o, w, outs, (int64_t)B * T, (int)C, (int)C, (int)T, H, D, true,
                                  false, (hipStream_t)stream);
  return e == hipSuccess ? ok() : device_error("pab_proj_out launch", e);
}
}  // namespace pab

using namespace pab;

extern "C" {

int pab_attn_spatial(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                     int32_t F, int32_t S, int32_t D, int32_t dtype, float softmax_scale,
                     void* stream) {
  int st = check_video_attn("pab_attn_spatial", q, k, v, o, B, H, F, S, D, dtype, softmax_scale, false);
  if (st) return st;
  return run_spatial(q, k, v, o, B, H, F, S, D, dtype, softmax_scale, stream);
}

int pab_attn_temporal(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                      int32_t F, int32_t S, int32_t D, int32_t dtype, float softmax_scale,
                      void* stream) {
  int st = check_video_attn("pab_attn_temporal", q, k, v, o, B, H, F, S, D, dtype, softmax_scale, true);
  if (st) return st;
  return run_temporal(q, k, v, o, B, H, F, S, D, dtype, softmax_scale, stream);
}

int pab_attn_cross(const void* q, const void* k_text, const void* v_text, void* o, int32_t B,
                   int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype,
                   float softmax_scale, void* stream) {
  int st = check_cross_attn(q, k_text, v_text, o, B, H, Nq, L, D, dtype, softmax_scale, nullptr);
  if (st) return st;
  return run_cross(q, k_text, v_text, o, B, H, Nq, L, D, dtype, softmax_scale, nullptr, stream);
}

int pab_attn_cross_masked(const void* q, const void* k_text, const void* v_text, void* o,
                          int32_t B, int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype,
                          float softmax_scale, const int32_t* text_len, void* stream) {
  if (!text_len) return fail(PAB_ERR_INVALID_ARG, "pab_attn_cross_masked: NULL text_len");
  int st = check_cross_attn(q, k_text, v_text, o, B, H, Nq, L, D, dtype, softmax_scale, text_len);
  if (st) return st;
  return run_cross(q, k_text, v_text, o, B, H, Nq, L, D, dtype, softmax_scale, text_len, stream);
}

int pab_proj_in(const void* x, const void* w, void* out0, void* out1, void* out2, int32_t n_out,
                int32_t B, int32_t F, int32_t S, int32_t H, int32_t D, int32_t dtype,
                void* stream) {
  void* outs[3] = {out0, out1, out2};
  int st = check_proj("pab_proj_in", x, w, outs, n_out, B, F, S, H, D, dtype, true);
  if (st) return st;
  return run_proj_in(x, w, outs, n_out, B, F, S, H, D, stream);
}

int pab_proj_out(const void* o, const void* w, void* y, int32_t B, int32_t F, int32_t S,
                 int32_t H, int32_t D, int32_t dtype, void* stream) {
  void* outs[3] = {y, nullptr, nullptr};
  int st = check_proj("pab_proj_out", o, w, outs, 1, B, F, S, H, D, dtype, false);
  if (st) return st;
  return run_proj_out(o, w, y, B, F, S, H, D, stream);
}

size_t pab_mse_workspace_bytes(int64_t n) {
  if (n < 1) return 0;
  // Enough partials for either dtype's grid, and for one per block of the
  // attention kernels that fuse the difference into their output pass (the
  // dispatcher falls back to the separate reduction when a launch has more
  // blocks than this holds), rounded to 256 bytes.
  int64_t blocks = mse_num_blocks(n, PAB_F32) > mse_num_blocks(n, PAB_BF16)
                       ? mse_num_blocks(n, PAB_F32)
                       : mse_num_blocks(n, PAB_BF16);
  if (n / 1024 + 64 > blocks) blocks = n / 1024 + 64;
  return ((size_t)blocks * sizeof(double) + 255) / 256 * 256;
}

int pab_attn_diff_mse(const void* a, const void* b, int64_t n, int32_t dtype, double* out_dev,
                      void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_mse(a, b, n, dtype, out_dev, workspace, workspace_bytes);
  if (st) return st;
  return run_mse(a, b, n, dtype, out_dev, workspace, stream);
}

int pab_attn_diff_mse_noalloc(const void* a, const void* b, int64_t n, int32_t dtype,
                              double* out_dev, void* stream) {
  const char* fn = "pab_attn_diff_mse_noalloc";
  if (!a || !b || !out_dev) return fail(PAB_ERR_INVALID_ARG, fmt("%s: NULL pointer", fn));
  if (!aligned16(a) || !aligned16(b) || ((uintptr_t)out_dev & 7u))
    return fail(PAB_ERR_INVALID_ARG, fmt("%s: misaligned pointer", fn));
  if (n < 1 || n > kMaxElems) return fail(PAB_ERR_INVALID_ARG, fmt("%s: bad n=%lld", fn, (long long)n));
  if (dtype != PAB_BF16 && dtype != PAB_F32)
    return fail(PAB_ERR_UNSUPPORTED, fmt("%s: unsupported dtype %d", fn, dtype));
  const int parts = mse_num_blocks(n, dtype);
  if (parts > mse_scratch_partials())
    return fail(PAB_ERR_CAPACITY, fmt("%s: n=%lld needs %d partials, the scratch holds %d", fn,
                                      (long long)n, parts, mse_scratch_partials()));
  double* partials = nullptr;
  hipError_t e = mse_scratch(&partials);
  if (e != hipSuccess) return device_error("pab_attn_diff_mse_noalloc (scratch address)", e);
  e = launch_mse(a, b, n, dtype, out_dev, partials, (hipStream_t)stream);
  return e == hipSuccess ? ok() : device_error("pab_attn_diff_mse_noalloc launch", e);
}

const char* pab_last_error(void) { return g_last_error.c_str(); }

const char* pab_version(void) { return "pab-mi355x 0.1 (gfx950)"; }

}  // extern "C"

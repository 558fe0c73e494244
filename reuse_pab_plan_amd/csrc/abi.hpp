// abi.hpp -- internal helpers of the C ABI layer: the thread-local error
// text and the argument checks shared by the entry points.
#pragma once

#include <stdint.h>

#include <string>

#include "../../include/pab.h"
#include "launch.hpp"

namespace pab {

std::string fmt(const char* f, ...) __attribute__((format(printf, 1, 2)));  // printf to string
int fail(int status, const std::string& msg);  // records msg, returns status
int ok();                                       // clears the error, returns PAB_OK
int device_error(const char* what, int hip_err);

bool aligned16(const void* p);
bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn);
size_t dtype_size(int32_t dtype);

// Validation of the attention calls, with no HIP call (shared by the direct
// entry points and the step dispatcher).
int check_video_attn(const char* fn, const void* q, const void* k, const void* v, const void* o,
                     int32_t B, int32_t H, int32_t F, int32_t S, int32_t D, int32_t dtype,
                     float scale, bool temporal);
// text_len: host array of B real text-token counts in [1, L], or NULL (all L).
int check_cross_attn(const void* q, const void* kt, const void* vt, const void* o, int32_t B,
                     int32_t H, int64_t Nq, int32_t L, int32_t D, int32_t dtype, float scale,
                     const int32_t* text_len);
int check_mse(const void* a, const void* b, int64_t n, int32_t dtype, const double* out,
              const void* ws, size_t ws_bytes);

// Launch without re-validating (arguments already checked).
// diff (optional, bf16 only): fuse the attention difference against
// diff->prev into the output pass when the workspace holds a partial per
// block (see DiffOut); with padded prompts cross attention launches once per
// batch entry and the partials of the launches follow one another.
int run_spatial(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                int32_t F, int32_t S, int32_t D, int32_t dtype, float scale, void* stream,
                const DiffOut* diff = nullptr);
int run_temporal(const void* q, const void* k, const void* v, void* o, int32_t B, int32_t H,
                 int32_t F, int32_t S, int32_t D, int32_t dtype, float scale, void* stream,
                 const DiffOut* diff = nullptr);
int run_cross(const void* q, const void* kt, const void* vt, void* o, int32_t B, int32_t H,
              int64_t Nq, int32_t L, int32_t D, int32_t dtype, float scale,
              const int32_t* text_len, void* stream, const DiffOut* diff = nullptr);
int run_mse(const void* a, const void* b, int64_t n, int32_t dtype, double* out, void* ws,
            void* stream);
int run_mse_final(const double* partials, int nparts, int64_t n, double* out, void* stream);

// Projections around an attention (bf16).  in = true: input projection
// (x token-major [B, F*S, C] -> n_out head-major tensors); false: output
// projection (head-major x -> outs[0] token-major).
int check_proj(const char* fn, const void* x, const void* w, void* const outs[3], int32_t n_out,
               int32_t B, int32_t F, int32_t S, int32_t H, int32_t D, int32_t dtype, bool in);
int run_proj_in(const void* x, const void* w, void* const outs[3], int32_t n_out, int32_t B,
                int32_t F, int32_t S, int32_t H, int32_t D, void* stream);
int run_proj_out(const void* o, const void* w, void* y, int32_t B, int32_t F, int32_t S, int32_t H,
                 int32_t D, void* stream);

}  // namespace pab

// dispatch.cpp -- one denoising step of one block under the broadcast cache.
//
// PAB article, Figure 2 caption: an attention result is broadcast to the
// next few steps, which then skip the attention computation.  Here a type
// that recomputes at this step launches its kernel into its next cache slot;
// a type that reuses launches nothing at all, and the slot that its last
// recompute wrote is handed back as this step's output (zero bytes moved,
// bit-identical by construction).  With two slots per type the previous
// output survives the recompute, so the attention difference between the two
// (PAB article, Figure 1 caption: measured by the MSE) can be taken on the
// device.  The dispatcher is stateless: slot parity is the number of
// recomputes so far, read off the schedule.  A type may also be a whole
// attention module (projections around the attention); its recompute then
// runs the module and a broadcast step skips all of it.
#include <stdint.h>

#include <initializer_list>

#include "abi.hpp"

using namespace pab;

namespace {

size_t output_elems(const pab_type_desc& t) {
  return (size_t)t.B * t.H * t.F * t.S * t.D;
}

// The attention module of a type (input projection, attention, output
// projection), checked as the three calls it makes.
int check_module(const pab_step_desc* d, const pab_type_desc& t) {
  if (!t.w_in || !t.w_out || !t.scratch[0] || !t.scratch[1] || !t.scratch[2] || !t.scratch[3])
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: a module needs w_in, w_out and 4 scratch buffers");
  void* qkv[3] = {t.scratch[0], t.scratch[1], t.scratch[2]};
  void* slot[3] = {t.slot[0], nullptr, nullptr};
  int st;
  if (t.kind == PAB_CROSS) {
    if (t.x_text && !t.w_kv)
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: a cross module with x_text needs w_kv");
    st = check_proj("pab_step_dispatch(proj q)", t.x, t.w_in, qkv, 1, t.B, t.F, t.S, t.H, t.D,
                    d->dtype, true);
    if (st) return st;
    if (t.x_text) {  // else scratch[1], scratch[2] already hold the projected text K/V
      void* kv[3] = {t.scratch[1], t.scratch[2], nullptr};
      st = check_proj("pab_step_dispatch(proj kv)", t.x_text, t.w_kv, kv, 2, t.B, 1, t.L, t.H,
                      t.D, d->dtype, true);
      if (st) return st;
    }
    st = check_cross_attn(t.scratch[0], t.scratch[1], t.scratch[2], t.scratch[3], t.B, t.H,
                          (int64_t)t.F * t.S, t.L, t.D, d->dtype, d->softmax_scale, t.text_len);
  } else {
    st = check_proj("pab_step_dispatch(proj qkv)", t.x, t.w_in, qkv, 3, t.B, t.F, t.S, t.H, t.D,
                    d->dtype, true);
    if (st) return st;
    st = check_video_attn("pab_step_dispatch(module attention)", t.scratch[0], t.scratch[1],
                          t.scratch[2], t.scratch[3], t.B, t.H, t.F, t.S, t.D, d->dtype,
                          d->softmax_scale, t.kind == PAB_TEMPORAL);
  }
  if (st) return st;
  st = check_proj("pab_step_dispatch(proj out)", t.scratch[3], t.w_out, slot, 1, t.B, t.F, t.S,
                  t.H, t.D, d->dtype, false);
  return st;
}

// A type that reuses its slot at this step launches nothing and reads none
// of its inputs (they may be NULL, e.g. when a trajectory resumes at a
// broadcast step): only what locating the slot needs is checked.
int check_reuse(const pab_step_desc* d, int a) {
  const pab_type_desc& t = d->types[a];
  if (t.kind != PAB_SPATIAL && t.kind != PAB_TEMPORAL && t.kind != PAB_CROSS)
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: unknown attention kind");
  if (dtype_size(d->dtype) == 0)
    return fail(PAB_ERR_UNSUPPORTED, fmt("pab_step_dispatch: unsupported dtype %d", d->dtype));
  if (t.B < 1 || t.H < 1 || t.F < 1 || t.S < 1 || t.D < 1)
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: bad shape");
  if (!t.slot[0] || !aligned16(t.slot[0]) || (t.slot[1] && !aligned16(t.slot[1])))
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slots must be non-NULL and 16-byte aligned");
  const uint64_t kMaxElems = (uint64_t)1 << 40;
  uint64_t elems = 1;
  for (int32_t dim : {t.B, t.H, t.F, t.S, t.D}) {
    if (elems > kMaxElems / (uint64_t)dim)
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: shape too large");
    elems *= (uint64_t)dim;
  }
  const size_t bytes = output_elems(t) * dtype_size(d->dtype);
  if (t.slot[1] && ranges_overlap(t.slot[0], bytes, t.slot[1], bytes))
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slots overlap");
  return PAB_OK;
}

int check_type(const pab_step_desc* d, int a) {
  const pab_type_desc& t = d->types[a];
  if (t.x) {
    if (t.kind != PAB_SPATIAL && t.kind != PAB_TEMPORAL && t.kind != PAB_CROSS)
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: unknown attention kind");
    int st = check_module(d, t);
    if (st) return st;
    if (t.slot[1] && !aligned16(t.slot[1]))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slot[1] must be 16-byte aligned");
    const size_t bytes = output_elems(t) * dtype_size(d->dtype);
    if (t.slot[1] && ranges_overlap(t.slot[0], bytes, t.slot[1], bytes))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slots overlap");
    // Scratch: q and the attention output are O-sized; a cross module's k, v
    // hold the text tokens only.
    const size_t kv_bytes = t.kind == PAB_CROSS
                                ? (size_t)t.B * t.H * t.L * t.D * dtype_size(d->dtype)
                                : bytes;
    const size_t scratch_bytes[4] = {bytes, kv_bytes, kv_bytes, bytes};
    for (int s = 0; s < 2; ++s)
      for (int i = 0; t.slot[s] && i < 4; ++i)
        if (ranges_overlap(t.slot[s], bytes, t.scratch[i], scratch_bytes[i]))
          return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: a slot overlaps a scratch buffer");
    if (t.drift && t.slot[1]) {
      if ((uintptr_t)t.drift & 7u)
        return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: misaligned drift");
      if (!d->workspace || !aligned16(d->workspace))
        return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: drift needs a 16-byte aligned workspace");
      if (d->workspace_bytes < pab_mse_workspace_bytes((int64_t)output_elems(t)))
        return fail(PAB_ERR_CAPACITY, "pab_step_dispatch: workspace too small for the drift MSE");
    }
    return PAB_OK;
  }
  const void* probe_out = t.slot[0];
  int st;
  switch (t.kind) {
    case PAB_SPATIAL:
      st = check_video_attn("pab_step_dispatch(spatial)", t.q, t.k, t.v, probe_out, t.B, t.H, t.F,
                            t.S, t.D, d->dtype, d->softmax_scale, false);
      break;
    case PAB_TEMPORAL:
      st = check_video_attn("pab_step_dispatch(temporal)", t.q, t.k, t.v, probe_out, t.B, t.H, t.F,
                            t.S, t.D, d->dtype, d->softmax_scale, true);
      break;
    case PAB_CROSS:
      st = check_cross_attn(t.q, t.k, t.v, probe_out, t.B, t.H, (int64_t)t.F * t.S, t.L, t.D,
                            d->dtype, d->softmax_scale, t.text_len);
      break;
    default:
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: unknown attention kind");
  }
  if (st) return st;
  if (t.slot[1]) {
    if (!aligned16(t.slot[1]))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slot[1] must be 16-byte aligned");
    const size_t bytes = output_elems(t) * dtype_size(d->dtype);
    if (ranges_overlap(t.slot[0], bytes, t.slot[1], bytes))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slots overlap");
    const size_t qbytes = bytes;
    if (ranges_overlap(t.slot[1], bytes, t.q, qbytes) ||
        (t.kind != PAB_CROSS && (ranges_overlap(t.slot[1], bytes, t.k, qbytes) ||
                                 ranges_overlap(t.slot[1], bytes, t.v, qbytes))))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: slot[1] overlaps an input");
  }
  if (t.drift && t.slot[1]) {
    if ((uintptr_t)t.drift & 7u) return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: misaligned drift");
    const int64_t n = (int64_t)output_elems(t);
    if (!d->workspace || !aligned16(d->workspace))
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: drift needs a 16-byte aligned workspace");
    if (d->workspace_bytes < pab_mse_workspace_bytes(n))
      return fail(PAB_ERR_CAPACITY, "pab_step_dispatch: workspace too small for the drift MSE");
  }
  return PAB_OK;
}

}  // namespace

extern "C" int pab_step_dispatch(const pab_step_desc* desc, int32_t step, uint32_t* recomputed_mask,
                                 void** outputs) {
  if (!desc || !desc->recompute || !desc->types)
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: NULL descriptor");
  const int nt = desc->num_types;
  if (nt < 1 || nt > 32) return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: num_types in [1, 32]");
  if (desc->num_steps < 1 || step < 0 || step >= desc->num_steps)
    return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: step out of range");

  // Slot of the latest output per type: recomputes in steps 0..step.
  int32_t count[32];
  for (int a = 0; a < nt; ++a) {
    count[a] = 0;
    for (int i = 0; i <= step; ++i) count[a] += desc->recompute[(size_t)i * nt + a] ? 1 : 0;
    if (count[a] == 0)
      return fail(PAB_ERR_INVALID_ARG, "pab_step_dispatch: type reused before any recompute");
    int st = desc->recompute[(size_t)step * nt + a] ? check_type(desc, a) : check_reuse(desc, a);
    if (st) return st;
  }

  uint32_t mask = 0;
  for (int a = 0; a < nt; ++a) {
    const pab_type_desc& t = desc->types[a];
    const bool two = t.slot[1] != nullptr;
    void* cur = two ? t.slot[(count[a] - 1) & 1] : t.slot[0];
    if (outputs) outputs[a] = cur;
    if (!desc->recompute[(size_t)step * nt + a]) continue;  // broadcast: no work at all
    mask |= 1u << a;
    int st;
    // The attention difference against the previous computation of this
    // type (when asked for): bf16 attention kernels fold it into their output
    // pass (partial sums per block in the workspace, then one final
    // reduction); otherwise a separate MSE pass follows.
    const bool want_diff = two && t.drift && count[a] >= 2;
    const void* prev = want_diff ? t.slot[count[a] & 1] : nullptr;
    int nparts = 0;
    DiffOut diff;
    if (want_diff && !t.x && desc->dtype == PAB_BF16) {
      diff.prev = prev;
      diff.partials = (double*)desc->workspace;
      diff.capacity = (int64_t)(desc->workspace_bytes / sizeof(double));
      diff.nparts = &nparts;
    }
    if (t.x) {
      // The whole attention module: projections around the attention.
      void* qkv[3] = {t.scratch[0], t.scratch[1], t.scratch[2]};
      if (t.kind == PAB_CROSS) {
        void* q1[3] = {t.scratch[0], nullptr, nullptr};
        void* kv[3] = {t.scratch[1], t.scratch[2], nullptr};
        st = run_proj_in(t.x, t.w_in, q1, 1, t.B, t.F, t.S, t.H, t.D, desc->stream);
        if (!st && t.x_text)
          st = run_proj_in(t.x_text, t.w_kv, kv, 2, t.B, 1, t.L, t.H, t.D, desc->stream);
        if (!st)
          st = run_cross(t.scratch[0], t.scratch[1], t.scratch[2], t.scratch[3], t.B, t.H,
                         (int64_t)t.F * t.S, t.L, t.D, desc->dtype, desc->softmax_scale,
                         t.text_len, desc->stream);
      } else {
        st = run_proj_in(t.x, t.w_in, qkv, 3, t.B, t.F, t.S, t.H, t.D, desc->stream);
        if (!st && t.kind == PAB_SPATIAL)
          st = run_spatial(qkv[0], qkv[1], qkv[2], t.scratch[3], t.B, t.H, t.F, t.S, t.D,
                           desc->dtype, desc->softmax_scale, desc->stream);
        if (!st && t.kind == PAB_TEMPORAL)
          st = run_temporal(qkv[0], qkv[1], qkv[2], t.scratch[3], t.B, t.H, t.F, t.S, t.D,
                            desc->dtype, desc->softmax_scale, desc->stream);
      }
      if (!st) st = run_proj_out(t.scratch[3], t.w_out, cur, t.B, t.F, t.S, t.H, t.D, desc->stream);
    } else {
      switch (t.kind) {
        case PAB_SPATIAL:
          st = run_spatial(t.q, t.k, t.v, cur, t.B, t.H, t.F, t.S, t.D, desc->dtype,
                           desc->softmax_scale, desc->stream, &diff);
          break;
        case PAB_TEMPORAL:
          st = run_temporal(t.q, t.k, t.v, cur, t.B, t.H, t.F, t.S, t.D, desc->dtype,
                            desc->softmax_scale, desc->stream, &diff);
          break;
        default:
          st = run_cross(t.q, t.k, t.v, cur, t.B, t.H, (int64_t)t.F * t.S, t.L, t.D, desc->dtype,
                         desc->softmax_scale, t.text_len, desc->stream, &diff);
          break;
      }
    }
    if (st) return st;
    if (want_diff) {
      st = nparts > 0
               ? run_mse_final((const double*)desc->workspace, nparts, (int64_t)output_elems(t),
                               t.drift + step, desc->stream)
               : run_mse(cur, prev, (int64_t)output_elems(t), desc->dtype, t.drift + step,
                         desc->workspace, desc->stream);
      if (st) return st;
    }
  }
  if (recomputed_mask) *recomputed_mask = mask;
  return ok();
}

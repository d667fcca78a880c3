// ssd_api.cpp -- the C ABI of libssd (declared in include/ssd.h).
//
// Every entry point validates its arguments on the host before any HIP call,
// then enqueues the stage kernels on the caller's stream.  No allocation, no
// host synchronisation, no global mutable state.
#include <climits>
#include <cstddef>
#include <cstdint>

#include "ssd.h"
#include "ssd_launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Required pointer: non-null and 16-byte aligned.
bool ok_ptr(const void* p) { return p != nullptr && aligned16(p); }
// Optional pointer: null, or 16-byte aligned.
bool ok_opt(const void* p) { return p == nullptr || aligned16(p); }

ssd_status check_dims(const ssd_dims* d, ssd::Shape* out) {
  if (d == nullptr) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t v[7] = {d->batch, d->seqlen, d->nheads, d->headdim,
                        d->dstate, d->ngroups, d->chunk_size};
  for (int64_t e : v)
    if (e < 1 || e > INT32_MAX) return SSD_ERR_INVALID_ARGUMENT;
  if (d->nheads % d->ngroups != 0) return SSD_ERR_INVALID_ARGUMENT;
  // Index arithmetic inside the kernels uses 32-bit block ids and token
  // counts; keep every launch and every (batch * seqlen) within range.
  const int64_t nc = (d->seqlen + d->chunk_size - 1) / d->chunk_size;
  if (d->batch * d->seqlen > INT32_MAX) return SSD_ERR_INVALID_ARGUMENT;
  // (batch * per_head_blocks <= 2^34 here, so only the last factor needs a
  // division to stay clear of 64-bit overflow)
  const int64_t per_head_blocks = nc * 4 > 8 ? nc * 4 : 8;
  if (d->batch * per_head_blocks > INT32_MAX / d->nheads) return SSD_ERR_INVALID_ARGUMENT;
  if (d->headdim != 64) return SSD_ERR_UNSUPPORTED;
  // Kernels address each sequence with 32-bit byte offsets (up to one chunk
  // past its end).
  const int64_t span = d->seqlen + d->chunk_size;
  if (span * d->nheads * d->headdim * 4 >= INT32_MAX ||
      span * d->ngroups * d->dstate * 4 >= INT32_MAX)
    return SSD_ERR_UNSUPPORTED;
  if (d->dstate != 64 && d->dstate != 128) return SSD_ERR_UNSUPPORTED;
  if (d->chunk_size != 64 && d->chunk_size != 128 && d->chunk_size != 256)
    return SSD_ERR_UNSUPPORTED;
  if (out) {
    *out = ssd::Shape{d->batch, d->seqlen, d->nheads, d->headdim,
                      d->dstate, d->ngroups, d->chunk_size};
  }
  return SSD_OK;
}

bool ok_dtype(ssd_dtype t) { return t == SSD_F32 || t == SSD_BF16; }

ssd_status check_gdn_dims(const ssd_gdn_dims* d, ssd::GdnShape* out) {
  if (d == nullptr) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t v[6] = {d->batch, d->seqlen, d->nheads, d->dk, d->dv, d->chunk_size};
  for (int64_t e : v)
    if (e < 1 || e > INT32_MAX) return SSD_ERR_INVALID_ARGUMENT;
  if (d->batch * d->seqlen > INT32_MAX) return SSD_ERR_INVALID_ARGUMENT;
  const int64_t nt = (d->seqlen + 63) / 64;
  if (d->batch * (nt > 8 ? nt : 8) > INT32_MAX / d->nheads) return SSD_ERR_INVALID_ARGUMENT;
  if (d->chunk_size != 64) return SSD_ERR_UNSUPPORTED;
  if ((d->dk != 64 && d->dk != 128) || (d->dv != 64 && d->dv != 128))
    return SSD_ERR_UNSUPPORTED;
  // Each sequence is addressed with 32-bit byte offsets, up to two chunks
  // past its end.
  const int64_t span = d->seqlen + 128;
  const int64_t wide = d->dk > d->dv ? d->dk : d->dv;
  if (span * d->nheads * wide * 4 >= INT32_MAX) return SSD_ERR_UNSUPPORTED;
  if (out) *out = ssd::GdnShape{d->batch, d->seqlen, d->nheads, d->dk, d->dv};
  return SSD_OK;
}

ssd_status from_hip(int err) { return err == 0 ? SSD_OK : SSD_ERR_HIP; }

// Whether two byte ranges of length n starting at a and b (either may be
// null) share any byte.
bool overlap(const void* a, const void* b, size_t n) {
  if (a == nullptr || b == nullptr || n == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + n && y < x + n;
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status status) {
  switch (status) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_INVALID_ARGUMENT: return "SSD_ERR_INVALID_ARGUMENT";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE";
    case SSD_ERR_HIP: return "SSD_ERR_HIP";
  }
  return "SSD_ERR_UNKNOWN";
}

size_t ssd_forward_workspace_bytes(const ssd_dims* dims) {
  if (check_dims(dims, nullptr) != SSD_OK) return 0;
  return 2 * sizeof(float) * (size_t)dims->batch * (size_t)dims->nheads *
         (size_t)dims->seqlen;
}

ssd_status ssd_chunk_cumsum(const float* dt, const float* A, float* g,
                            float* dt_t, const ssd_dims* dims, void* stream) {
  if (dims == nullptr) return SSD_ERR_INVALID_ARGUMENT;
  // Stage 1 reads only batch, seqlen, nheads and chunk_size; check those with
  // a shape whose other fields are fixed to a supported value.
  ssd_dims d1 = *dims;
  d1.headdim = 64;
  d1.dstate = 64;
  d1.ngroups = 1;
  ssd::Shape s;
  const ssd_status st = check_dims(&d1, &s);
  if (st != SSD_OK) return st;
  if (!ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(g) || !ok_ptr(dt_t))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_chunk_cumsum(dt, A, g, dt_t, s, stream));
}

ssd_status ssd_fwd_pass_state(const void* x, const void* B, const float* dt_t,
                              const float* g, const float* init_state,
                              float* states, float* final_state, ssd_dtype in_dtype,
                              const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(B) || !ok_ptr(dt_t) || !ok_ptr(g) || !ok_ptr(states) ||
      !ok_opt(init_state) || !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_fwd_pass_state(x, B, dt_t, g, init_state, states,
                                             final_state, in_dtype == SSD_BF16,
                                             s, stream));
}

ssd_status ssd_chunk_state(const void* x, const void* B, const float* dt_t, const float* g,
                           float* states, float* final_state, ssd_dtype in_dtype,
                           const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(B) || !ok_ptr(dt_t) || !ok_ptr(g) || !ok_ptr(states) ||
      !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_chunk_state(x, B, dt_t, g, states, final_state,
                                          in_dtype == SSD_BF16, false, s, stream));
}

ssd_status ssd_state_passing(const float* g, const float* init_state, float* states,
                             float* final_state, const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_ptr(g) || !ok_opt(init_state) || !ok_ptr(states) || !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  // final_state holds the last chunk's contribution on entry, so it cannot
  // also be the initial state here.
  const size_t sbytes = sizeof(float) * (size_t)(s.batch * s.nheads * s.headdim * s.dstate);
  if (overlap(init_state, final_state, sbytes)) return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(
      ssd::launch_state_passing(g, init_state, states, final_state, false, s, stream));
}

ssd_status ssd_compute_out(const void* x, const void* B, const void* C,
                           const float* dt_t, const float* g,
                           const float* states, const float* D, void* y,
                           ssd_dtype in_dtype, ssd_dtype y_dtype, const ssd_dims* dims,
                           void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(y_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(B) || !ok_ptr(C) || !ok_ptr(dt_t) || !ok_ptr(g) ||
      !ok_ptr(states) || !ok_ptr(D) || !ok_ptr(y))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_compute_out(x, B, C, dt_t, g, states, D, y,
                                          in_dtype == SSD_BF16,
                                          y_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_state_and_out(const void* x, const void* B, const void* C,
                             const float* dt_t, const float* g, const float* D,
                             const float* init_state, void* y, float* states,
                             float* final_state, ssd_dtype in_dtype, ssd_dtype y_dtype,
                             const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(y_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(B) || !ok_ptr(C) || !ok_ptr(dt_t) || !ok_ptr(g) ||
      !ok_ptr(D) || !ok_ptr(y) || !ok_ptr(states) || !ok_opt(init_state) ||
      !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_state_and_out(x, B, C, dt_t, g, D, init_state, states,
                                            final_state, y, in_dtype == SSD_BF16,
                                            y_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_forward(const void* x, const float* dt, const float* A,
                       const void* B, const void* C, const float* D,
                       const float* init_state, void* y, float* states,
                       float* final_state, void* workspace,
                       size_t workspace_bytes, ssd_dtype in_dtype, ssd_dtype y_dtype,
                       const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(y_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C) ||
      !ok_ptr(D) || !ok_ptr(y) || !ok_ptr(states) || !ok_opt(init_state) ||
      !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  if (workspace == nullptr || !aligned16(workspace) ||
      workspace_bytes < ssd_forward_workspace_bytes(dims))
    return SSD_ERR_WORKSPACE;
  float* g = static_cast<float*>(workspace);
  float* dt_t = g + (size_t)s.batch * s.nheads * s.seqlen;
  const bool bf16 = in_dtype == SSD_BF16;
  int err = ssd::launch_chunk_cumsum(dt, A, g, dt_t, s, stream);
  if (err == 0)
    err = ssd::launch_state_and_out(x, B, C, dt_t, g, D, init_state, states, final_state, y,
                                    bf16, y_dtype == SSD_BF16, s, stream);
  return from_hip(err);
}

ssd_status ssd_forward_noalloc(const void* x, const float* dt, const float* A, const void* B,
                               const void* C, const float* D, const float* init_state, void* y,
                               float* states, float* final_state, ssd_dtype in_dtype,
                               ssd_dtype y_dtype, const ssd_dims* dims, void* stream) {
  ssd::Shape s;
  const ssd_status st = check_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(y_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C) ||
      !ok_ptr(D) || !ok_ptr(y) || !ok_ptr(states) || !ok_opt(init_state) ||
      !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  if (ssd_forward_workspace_bytes(dims) > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_WORKSPACE;
  return from_hip(ssd::launch_forward_noalloc(x, dt, A, B, C, D, init_state, y, states,
                                              final_state, in_dtype == SSD_BF16,
                                              y_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_decode_step(const void* x, const float* dt, const float* A,
                           const void* B, const void* C, const float* D, float* state,
                           void* y, ssd_dtype in_dtype, ssd_dtype y_dtype, const ssd_dims* dims,
                           void* stream) {
  if (dims == nullptr) return SSD_ERR_INVALID_ARGUMENT;
  // One token: seqlen and chunk_size are not read; check the rest with
  // those two fixed to supported values.
  ssd_dims d1 = *dims;
  d1.seqlen = 1;
  d1.chunk_size = 64;
  ssd::Shape s;
  const ssd_status st = check_dims(&d1, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(y_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(dt) || !ok_ptr(A) || !ok_ptr(B) || !ok_ptr(C) || !ok_ptr(D) ||
      !ok_ptr(state) || !ok_ptr(y))
    return SSD_ERR_INVALID_ARGUMENT;
  return from_hip(ssd::launch_decode_step(x, dt, A, B, C, D, state, y, in_dtype == SSD_BF16,
                                          y_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_gdn_chunk_fwd_h(const void* k, const void* w, const void* u, const float* g,
                               const float* h0, float* h, void* v_new, float* final_state,
                               ssd_dtype in_dtype, ssd_dtype v_dtype, const ssd_gdn_dims* dims,
                               void* stream) {
  ssd::GdnShape s;
  const ssd_status st = check_gdn_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(v_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(k) || !ok_ptr(w) || !ok_ptr(u) || !ok_ptr(g) || !ok_opt(h0) || !ok_ptr(h) ||
      !ok_ptr(v_new) || !ok_opt(final_state))
    return SSD_ERR_INVALID_ARGUMENT;
  if (in_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_gdn_fwd_h(k, w, u, g, h0, h, v_new, final_state,
                                        v_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_gdn_chunk_fwd_o(const void* q, const void* k, const void* v_new, const float* h,
                               const float* g, void* o, float scale, ssd_dtype in_dtype, ssd_dtype v_dtype,
                               ssd_dtype o_dtype, const ssd_gdn_dims* dims, void* stream) {
  ssd::GdnShape s;
  const ssd_status st = check_gdn_dims(dims, &s);
  if (st != SSD_OK) return st;
  if (!ok_dtype(in_dtype) || !ok_dtype(v_dtype) || !ok_dtype(o_dtype))
    return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(v_new) || !ok_ptr(h) || !ok_ptr(g) || !ok_ptr(o))
    return SSD_ERR_INVALID_ARGUMENT;
  if (in_dtype != SSD_BF16 || v_dtype != SSD_BF16) return SSD_ERR_UNSUPPORTED;
  return from_hip(
      ssd::launch_gdn_fwd_o(q, k, v_new, h, g, o, scale, o_dtype == SSD_BF16, s, stream));
}

ssd_status ssd_causal_conv1d(const void* x, const float* weight, const float* bias, void* out,
                             int64_t batch, int64_t dim, int64_t seqlen, int64_t width,
                             ssd_dtype x_dtype, ssd_dtype out_dtype, void* stream) {
  if (batch < 1 || dim < 1 || seqlen < 1 || width < 1) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_dtype(x_dtype) || !ok_dtype(out_dtype)) return SSD_ERR_INVALID_ARGUMENT;
  if (!ok_ptr(x) || !ok_ptr(weight) || !ok_opt(bias) || !ok_ptr(out))
    return SSD_ERR_INVALID_ARGUMENT;
  if (width > 4) return SSD_ERR_UNSUPPORTED;
  // A row is addressed with 32-bit byte offsets (fp32 rows plus one
  // wavefront run of slack); the element count must not overflow.
  if (seqlen > ((int64_t)1 << 29) - (1 << 14)) return SSD_ERR_UNSUPPORTED;
  if (batch > ((int64_t)1 << 40) / dim || batch * dim > ((int64_t)1 << 44) / seqlen)
    return SSD_ERR_UNSUPPORTED;
  return from_hip(ssd::launch_causal_conv1d(x, weight, bias, out, batch, dim, seqlen,
                                            (int)width, x_dtype == SSD_BF16,
                                            out_dtype == SSD_BF16, stream));
}

}  // extern "C"

// ssd_launch.h -- host-side launchers of the kernels (internal to
// libssd).  Arguments arrive already validated by the C ABI layer; each
// launcher returns the hipError_t of its launch as an int (0 = success).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "ssd.h"

namespace ssd {

// Size of the per-device scratch array behind ssd_forward_noalloc (holds g
// and dt_t: 8 bytes per (batch, token, head)).
constexpr size_t kNoallocScratchBytes = SSD_NOALLOC_SCRATCH_BYTES;

struct Shape {
  int64_t batch, seqlen, nheads, headdim, dstate, ngroups, chunk;
  int64_t nchunks() const { return (seqlen + chunk - 1) / chunk; }
};

int launch_chunk_cumsum(const float* dt, const float* A, float* g,
                        float* dt_t, const Shape& s, void* stream);

int launch_fwd_pass_state(const void* x, const void* B, const float* dt_t,
                          const float* g, const float* init_state,
                          float* states, float* final_state, bool bf16_in,
                          const Shape& s, void* stream);

int launch_compute_out(const void* x, const void* B, const void* C,
                       const float* dt_t, const float* g, const float* states,
                       const float* D, void* y, bool bf16_in, bool bf16_out,
                       const Shape& s, void* stream);

// Stage 2 for fp32 inputs with 64-token chunks, N = 64, an even group size
// and at least one (b, head pair) per compute unit: one workgroup per head
// pair sharing each staged B tile, on bf16 matrix instructions with exact
// three-term splits (launch_fwd_pass_state takes it where it applies).
bool state_pair_f32_applies(const Shape& s, bool bf16_in);
int launch_state_pair_f32(const float* x, const float* B, const float* dt_t, const float* g,
                          const float* init, float* states, float* fin, const Shape& s,
                          void* stream);

// Stages 2 and 3 of ssd_forward: the fused single-pass kernel where it
// applies (fp32 inputs, 64-token chunks, N = 64, at least one (b, head pair)
// per compute unit), otherwise launch_fwd_pass_state then
// launch_compute_out.  Outputs are the same either way.
int launch_state_and_out(const void* x, const void* B, const void* C, const float* dt_t,
                         const float* g, const float* D, const float* init_state, float* states,
                         float* final_state, void* y, bool bf16_in, bool bf16_out,
                         const Shape& s, void* stream);

// Stages 2 and 3 as one pass for bf16 inputs with N = 128 and an even group
// size (heads taken in pairs): a run pass and a run passing (when the chains
// are cut into runs), then the fused head-pair kernel.  The states buffer
// holds the runs' intermediate results until the fused kernel overwrites
// them, so no other memory is used.
bool fused_bf16_applies(const Shape& s, bool bf16_in);
int launch_fused_bf16(const void* x, const void* B, const void* C, const float* dt_t,
                      const float* g, const float* D, const float* init, float* states,
                      float* fin, void* y, bool bf16_out, const Shape& s, void* stream);

// The two-level form of stage 2 (chunk_state writes each chunk's zero-state
// contribution into the slot of the state it feeds; state_passing turns the
// slots into the states in place).  With park / parked, the last chunk's
// contribution goes through the states[0] slot instead of final_state, so
// init_state may alias final_state.
int launch_chunk_state(const void* x, const void* B, const float* dt_t, const float* g,
                       float* states, float* fin, bool bf16_in, bool park, const Shape& s,
                       void* stream);
int launch_state_passing(const float* g, const float* init, float* states, float* fin,
                         bool parked, const Shape& s, void* stream);

// ssd_forward with g and dt_t in the library's per-device scratch array;
// the shape must need at most kNoallocScratchBytes of it.
int launch_forward_noalloc(const void* x, const float* dt, const float* A, const void* B,
                           const void* C, const float* D, const float* init_state, void* y,
                           float* states, float* final_state, bool bf16_in, bool bf16_out,
                           const Shape& s, void* stream);

int launch_decode_step(const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, float* state, void* y, bool bf16_in,
                       bool bf16_out, const Shape& s, void* stream);

// Gated DeltaNet shapes: q, k, w [b, L, H, K]; u, v_new, o [b, L, H, V];
// chunks of 64 tokens.
struct GdnShape {
  int64_t batch, seqlen, nheads, dk, dv;
  int64_t nchunks() const { return (seqlen + 63) / 64; }
};

int launch_gdn_fwd_h(const void* k, const void* w, const void* u, const float* g,
                     const float* h0, float* hout, void* vnew, float* fin, bool vbf16,
                     const GdnShape& s, void* stream);

int launch_gdn_fwd_o(const void* q, const void* k, const void* vnew, const float* h,
                     const float* g, void* o, float scale, bool obf16, const GdnShape& s,
                     void* stream);

int launch_causal_conv1d(const void* x, const float* weight, const float* bias, void* out,
                         int64_t batch, int64_t dim, int64_t seqlen, int width, bool bf16_in,
                         bool bf16_out, void* stream);

}  // namespace ssd

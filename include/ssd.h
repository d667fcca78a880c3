/*
 * ssd.h -- C ABI of libssd: the Mamba-2 SSD chunked forward pass on one
 * AMD Instinct MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [P1] "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in
 *        NVIDIA CUDA Tile" (trishampatil.com)
 *   [P2] the zhiding.cn rendering of the same write-up, section
 *        "Mamba-2架构" (where the display formulas survive)
 *   [P3] the Helion hackathon project gallery (cerebralvalley.ai)
 *
 * The method.  Per batch b and head h, with group g = h / (nheads/ngroups):
 *     S_t = exp(A_h dt_t) S_{t-1} + dt_t x_t B_t^T      (state, headdim x dstate)
 *     y_t = S_t C_t + D_h x_t
 * [P1 "The Mamba-2 Recurrence"; P2 "Mamba-2架构"], evaluated chunk by chunk
 * in three stages [P1 "From the Math to Three Kernels"]:
 *   1. ssd_chunk_cumsum    g = log2(e) * per-chunk inclusive cumsum of A dt
 *   2. ssd_fwd_pass_state  per-chunk starting states by the jump
 *                          S_next = 2^{g_last} S + X^T (dt 2^{g_last-g} B)
 *   3. ssd_compute_out     Y = 2^{g} (C S^T) + ((C B^T) o 2^{g_i-g_j} o M)(dt X) + D X
 * and ssd_forward runs the three in order.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers to contiguous row-major arrays in the
 *   layouts given below, each 16-byte aligned.  The caller owns every buffer;
 *   the library allocates nothing, keeps no mutable global state and may be
 *   called concurrently on different streams.
 * - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   Every call is stream-ordered and asynchronous: it only enqueues kernels
 *   and never synchronises the host.
 * - Every argument is checked on the host BEFORE any HIP call; a failed check
 *   returns SSD_ERR_INVALID_ARGUMENT or SSD_ERR_UNSUPPORTED and touches
 *   nothing.  A failed kernel launch returns SSD_ERR_HIP.  Faults during
 *   execution surface at the caller's next synchronisation.
 * - Dimensions: batch, seqlen, nheads, headdim (P), dstate (N), ngroups (G),
 *   chunk_size (T), all >= 1, nheads % ngroups == 0.  seqlen need not be a
 *   multiple of chunk_size: a ragged last chunk is handled as the recurrence
 *   defines it.  Supported: P = 64; N in {64, 128}; T in {64, 128, 256};
 *   x/B/C in fp32 or bf16.  Anything else returns SSD_ERR_UNSUPPORTED.
 * - nc = ceil(seqlen / chunk_size) is the number of chunks.
 * - Element types: x, B, C share `in_dtype`; y has `y_dtype`; dt, dt_t, A,
 *   D, g, states, final_state and init_state are always fp32.
 * - Stage 1 also writes dt_t, dt transposed to [b, H, L]: with g it is what
 *   stages 2 and 3 read, so every per-head token run they load is contiguous.
 * - Per-sequence byte extents must stay below 2 GiB:
 *   (seqlen + chunk_size) * nheads * headdim * 4 and the same with
 *   ngroups * dstate, else SSD_ERR_UNSUPPORTED.
 */
#ifndef SSD_H_
#define SSD_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SSD_OK = 0,
    SSD_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad dim, misalignment   */
    SSD_ERR_UNSUPPORTED = 2,      /* valid but not built: (P, N, T, dtype)  */
    SSD_ERR_WORKSPACE = 3,        /* workspace null or smaller than needed  */
    SSD_ERR_HIP = 4               /* a HIP launch reported an error         */
} ssd_status;

typedef enum { SSD_F32 = 0, SSD_BF16 = 1 } ssd_dtype;

/* Problem shape; field names follow the problem statement of the pages'
 * benchmark example [P1 "Mamba-2 Forward Pass Benchmarks: cuTile vs Triton
 * on NVIDIA B300"] (batch size, tokens, groups, heads, state size, head
 * size, chunk size). */
typedef struct {
    int64_t batch;      /* b                                           */
    int64_t seqlen;     /* L, tokens per sequence                       */
    int64_t nheads;     /* H                                            */
    int64_t headdim;    /* P, size of x_t per head                      */
    int64_t dstate;     /* N, size of B_t and C_t (the state size)      */
    int64_t ngroups;    /* G, B/C shared by nheads/ngroups heads         */
    int64_t chunk_size; /* T                                            */
} ssd_dims;

/* Human-readable name of a status code (static storage; never NULL). */
const char *ssd_status_string(ssd_status status);

/* Bytes of device workspace ssd_forward needs: the stage-1 outputs g and
 * dt_t, 8 * batch * nheads * seqlen.  Returns 0 when dims is NULL or
 * invalid. */
size_t ssd_forward_workspace_bytes(const ssd_dims *dims);

/*
 * Stage 1 [P1 "Kernel 1: chunk_cumsum, the Cumulative Decay Sums"]:
 *   g[b,h,t] = log2(e) * sum_{s = T*floor(t/T)}^{t} A[h] * dt[b,s,h]
 * the within-chunk inclusive cumsum of a = A dt, scaled so later stages use
 * exp2.  g and a transposed copy of dt are stored head-major, [b, H, L], so
 * per-head token runs are contiguous: the layout change the pages apply to
 * both decay_cumsum and dt [P2 "Mamba-2性能优化", the global-memory layout
 * item; P1 "Mamba-2 Performance Optimizations in cuTile"].
 *   dt [b, L, H] fp32 (read)     A [H] fp32 (read)
 *   g [b, H, L] fp32 (written)   dt_t [b, H, L] fp32 (written; dt_t[b,h,t] = dt[b,t,h])
 * Only batch, seqlen, nheads and chunk_size of `dims` are read.
 */
ssd_status ssd_chunk_cumsum(const float *dt, const float *A, float *g,
                            float *dt_t, const ssd_dims *dims, void *stream);

/*
 * Stage 2 [P1 "Kernel 2: fwd_pass_state, Carrying the State Between Chunks";
 * P1 "Step 3: Add Back the Decay, Safely, in Log-Space"]: for every (b, h),
 * S = init_state[b,h] (zeros if init_state is NULL); for each chunk c in
 * order: states[b,h,c] = S, then
 *   S = 2^{g_last} S + X_c^T (w o B_c),   w_t = dt_t 2^{g_last - g_t}
 * with g_last the value of g at the chunk's last token.  final_state = S
 * after the last chunk.
 *   x [b, L, H, P] in_dtype      B [b, L, G, N] in_dtype
 *   dt_t, g [b, H, L] fp32 (from ssd_chunk_cumsum)
 *   init_state [b, H, P, N] fp32 or NULL
 *   states [b, H, nc, P, N] fp32 (written)   final_state [b, H, P, N] or NULL
 * init_state and final_state may be the same buffer (a sequence continued in
 * place); no other output may overlap an input.
 */
ssd_status ssd_fwd_pass_state(const void *x, const void *B, const float *dt_t,
                              const float *g, const float *init_state,
                              float *states, float *final_state, ssd_dtype in_dtype,
                              const ssd_dims *dims, void *stream);

/*
 * Stage 2 in two levels [P1 "Step 1: Jump the State Across a Chunk with One
 * Matmul"]: the jump S_{c+1} = 2^{g_last(c)} S_c + P_c, with P_c =
 * X_c^T (w o B_c) the contribution of chunk c from a zero state, split into
 * a fully parallel part and a short sequential one.  The two calls below,
 * in this order, compute the states and final_state ssd_fwd_pass_state
 * computes (equal up to the order of fp32 roundings); with bf16 inputs
 * ssd_fwd_pass_state itself takes this form for long chains on few heads,
 * where it is faster than the one-pass kernel.
 *
 * ssd_chunk_state: every P_c at once, written into the slot of the state it
 * feeds: states[b,h,c+1] = P_c for c < nc-1, and final_state = P_{nc-1}
 * (skipped when final_state is NULL).  states[b,h,0] is not touched.
 *   x, B, dt_t, g, states, final_state as for ssd_fwd_pass_state; in_dtype
 *   bf16 or fp32.
 *
 * ssd_state_passing: in place, element by element over the state:
 *   states[b,h,0] = init (zeros if init_state is NULL);
 *   states[b,h,c] = 2^{g_last(c-1)} states[b,h,c-1] + states[b,h,c], c >= 1;
 *   final_state = 2^{g_last(nc-1)} states[b,h,nc-1] + final_state (if not NULL).
 *   g [b, H, L] fp32 from ssd_chunk_cumsum; states, init, final fp32.
 * In this two-call form final_state carries P_{nc-1} from the first call to
 * the second, so init_state must not overlap final_state
 * (SSD_ERR_INVALID_ARGUMENT); ssd_fwd_pass_state has no such restriction.
 */
ssd_status ssd_chunk_state(const void *x, const void *B, const float *dt_t,
                           const float *g, float *states, float *final_state,
                           ssd_dtype in_dtype, const ssd_dims *dims, void *stream);
ssd_status ssd_state_passing(const float *g, const float *init_state,
                             float *states, float *final_state,
                             const ssd_dims *dims, void *stream);

/*
 * Stage 3 [P1 "Kernel 3: compute_out, the Fused Output Kernel"; P1 "Step 2:
 * Compute a Chunk of Outputs from One State"]: for every (b, c, h), with S_c
 * = states[b,h,c], rows i and columns j tokens of chunk c:
 *   Y = 2^{g_i} (C S_c^T) + L' X + D_h X,
 *   L'[i,j] = (C B^T)[i,j] 2^{g_i - g_j} dt_j  for i >= j, else 0
 * The masked entries are selected away, never multiplied by zero, so the
 * positive exponents above the diagonal cannot turn into NaN [P1 "Step 3"].
 * The chunk x chunk matrix never reaches memory.
 *   x, B, C as above; dt_t, g as above; states [b, H, nc, P, N] fp32 (read)
 *   D [H] fp32; y [b, L, H, P] in y_dtype (written)
 */
ssd_status ssd_compute_out(const void *x, const void *B, const void *C,
                           const float *dt_t, const float *g,
                           const float *states, const float *D, void *y,
                           ssd_dtype in_dtype, ssd_dtype y_dtype, const ssd_dims *dims,
                           void *stream);

/*
 * Stages 2 and 3 in one call: ssd_fwd_pass_state then ssd_compute_out on the
 * same arguments, with the same results (equal up to the order of fp32
 * roundings).  Two shape classes run as one pass that carries each head's
 * state from chunk to chunk in registers, so x is read once and the states
 * are written but not read back (the pages' two kernels, fused; [P1
 * "Kernel 2"; P1 "Kernel 3"]):
 *   - fp32 inputs, 64-token chunks and dstate 64, when the batch holds at
 *     least one (b, head pair) per compute unit;
 *   - bf16 inputs with dstate 128 and an even number of heads per group;
 *     the chains of chunks are cut into runs walked at once, each run
 *     starting from a state that two short kernels compute first (they
 *     use the states buffer as their only working memory).
 *   x, B, C, dt_t, g, D as for the two stages; init_state [b, H, P, N] fp32
 *   or NULL; states [b, H, nc, P, N] fp32 (written); final_state [b, H, P, N]
 *   fp32 or NULL; y [b, L, H, P] in y_dtype (written).
 * init_state and final_state may be the same buffer; no other output may
 * overlap an input.
 */
ssd_status ssd_state_and_out(const void *x, const void *B, const void *C,
                             const float *dt_t, const float *g, const float *D,
                             const float *init_state, void *y, float *states,
                             float *final_state, ssd_dtype in_dtype, ssd_dtype y_dtype,
                             const ssd_dims *dims, void *stream);

/*
 * The whole forward [P1 "From the Math to Three Kernels"]: stage 1 (g, dt_t)
 * into the caller's workspace (at least ssd_forward_workspace_bytes(dims)
 * bytes, else
 * SSD_ERR_WORKSPACE), then stages 2 and 3, all on `stream`.  Returns y, the
 * per-chunk starting states and (if final_state != NULL) the final state,
 * which a later call can take back as init_state to continue the sequence
 * (init_state and final_state may be the same buffer).
 */
ssd_status ssd_forward(const void *x, const float *dt, const float *A,
                       const void *B, const void *C, const float *D,
                       const float *init_state, void *y, float *states,
                       float *final_state, void *workspace,
                       size_t workspace_bytes, ssd_dtype in_dtype, ssd_dtype y_dtype,
                       const ssd_dims *dims, void *stream);

/*
 * ssd_forward without allocation: for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments and results as
 * ssd_forward minus the workspace; g and dt_t (8 * batch * nheads * seqlen
 * bytes) go to a scratch array the library holds on each GPU it runs on,
 * SSD_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU for the life of the process.
 * Shapes that need more return SSD_ERR_WORKSPACE before any HIP call; use
 * ssd_forward with a workspace for those.  The call allocates nothing and
 * calls no allocating routine.  All calls on one GPU share its array, so
 * calls that overlap in time on one GPU (other streams, other host threads)
 * race: order them on one stream.
 */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
ssd_status ssd_forward_noalloc(const void *x, const float *dt, const float *A,
                               const void *B, const void *C, const float *D,
                               const float *init_state, void *y, float *states,
                               float *final_state, ssd_dtype in_dtype,
                               ssd_dtype y_dtype, const ssd_dims *dims,
                               void *stream);

/*
 * The streaming decode step [P1 "The Mamba-2 Recurrence"; P1 "Why Would a
 * Trading Firm Care About Mamba-2 Kernels?" (at inference the fixed-size
 * state is carried forward and updated per new event); P1 "Kernel 2" (the
 * final state is the next call's init_state)]: one token through the
 * recurrence for every (b, h), with the state updated in place:
 *   state = exp(A_h dt) state + dt x B^T;   y = state C + D_h x
 * (y reads the updated state, as in the forward pass).  `state` is the
 * final_state of a previous ssd_forward (or any [b, H, P, N] fp32 state) and
 * holds the state after this token on return.
 *   x [b, H, P] in_dtype       dt [b, H] fp32 (already softplus'd)
 *   A [H] fp32                 B, C [b, G, N] in_dtype      D [H] fp32
 *   state [b, H, P, N] fp32 (read and written)   y [b, H, P] in y_dtype
 * These are the layouts of one token of the forward pass's tensors.  Only
 * batch, nheads, headdim, dstate and ngroups of `dims` are read.
 */
ssd_status ssd_decode_step(const void *x, const float *dt, const float *A,
                           const void *B, const void *C, const float *D,
                           float *state, void *y, ssd_dtype in_dtype, ssd_dtype y_dtype,
                           const ssd_dims *dims, void *stream);

/*
 * Gated DeltaNet, chunked forward [P3, the gated_deltanet_chunk_fwd_h and
 * gated_deltanet_chunk_fwd_o entries].  Problem shape: batch b, seqlen L,
 * nheads H, key size dk (K), value size dv (V), chunk_size (C).  Supported:
 * K and V in {64, 128}, C = 64, bf16 q/k/w/u; anything else valid returns
 * SSD_ERR_UNSUPPORTED.  (L + 128) * H * max(K, V) * 4 must stay below 2 GiB.
 */
typedef struct {
    int64_t batch;      /* b                                     */
    int64_t seqlen;     /* L, tokens per sequence                 */
    int64_t nheads;     /* H                                      */
    int64_t dk;         /* K, key size (rows of the state)        */
    int64_t dv;         /* V, value size (columns of the state)   */
    int64_t chunk_size; /* C                                      */
} ssd_gdn_dims;

/*
 * The inter-chunk state pass [P3, chunk_fwd_h]: per (b, h), h = h0 (zeros if
 * NULL); for each chunk c of C tokens (the last may be shorter), in order:
 *   h_out[b,h,c] = h
 *   v_new[t] = u[t] - w[t] h                       (t in the chunk)
 *   h = exp(g_last) h + sum_t k[t]^T (exp(g_last - g[t]) v_new[t])
 * with g_last = g at the chunk's last valid token; final_state = h at the
 * end.  g is the chunk-local cumulative sum of the per-token log-gates
 * (natural log); w and u are the WY-transformed keys and values.
 *   k, w [b, L, H, K] in_dtype      u [b, L, H, V] in_dtype     g [b, L, H] fp32
 *   h0 [b, H, K, V] fp32 or NULL    h [b, H, nt, K, V] fp32 (written), nt = ceil(L / C)
 *   v_new [b, L, H, V] v_dtype (written)   final_state [b, H, K, V] fp32 or NULL
 * Arithmetic is fp32 (the fp32 state enters the matrix products as bf16
 * hi + lo pairs).
 */
ssd_status ssd_gdn_chunk_fwd_h(const void *k, const void *w, const void *u,
                               const float *g, const float *h0, float *h,
                               void *v_new, float *final_state, ssd_dtype in_dtype,
                               ssd_dtype v_dtype, const ssd_gdn_dims *dims,
                               void *stream);

/*
 * The output [P3, chunk_fwd_o]: for every (b, chunk c, h) and token t of the
 * chunk,
 *   o[t] = scale * ( exp(g[t]) q[t] h[b,h,c]
 *                    + sum_{j in chunk, j <= t} (q[t] . k[j]) exp(g[t] - g[j]) v_new[j] )
 * (scale = 1 is the gallery's formula).  Entries with j > t are replaced by
 * zero after their exponent is formed (a select, never a multiply by a 0/1
 * mask).
 *   q, k [b, L, H, K] in_dtype    v_new [b, L, H, V] v_dtype (from chunk_fwd_h)
 *   h [b, H, nt, K, V] fp32 (from chunk_fwd_h)    g [b, L, H] fp32
 *   o [b, L, H, V] o_dtype (written)
 * Supported: in_dtype and v_dtype bf16; o_dtype fp32 or bf16.
 */
ssd_status ssd_gdn_chunk_fwd_o(const void *q, const void *k, const void *v_new,
                               const float *h, const float *g, void *o,
                               float scale, ssd_dtype in_dtype, ssd_dtype v_dtype,
                               ssd_dtype o_dtype, const ssd_gdn_dims *dims,
                               void *stream);

/*
 * The causal depthwise conv1d of the Mamba block, upstream of the SSD [P3,
 * the causal_conv1d entries]: each channel row is filtered on its own over
 * the current and the width-1 previous tokens, with zeros before the first
 * token:
 *   out[b,d,t] = bias[d] + sum_{k=0}^{width-1} weight[d,k] x[b,d,t-width+1+k]
 * No activation is applied.  Arithmetic is fp32.
 *   x [batch, dim, seqlen] x_dtype (read)       weight [dim, width] fp32
 *   bias [dim] fp32 or NULL (no bias)           out [batch, dim, seqlen] out_dtype
 * The size arguments replace ssd_dims (this op has no heads or state).
 * Supported: width 1..4 (the gallery's filters have 3 or 4 taps) and seqlen
 * up to 2^29 - 2^14; wider filters or longer rows return
 * SSD_ERR_UNSUPPORTED.  out must not overlap x.  Any seqlen works; rows
 * whose byte length is a multiple of 16 take the vectorised kernel.
 */
ssd_status ssd_causal_conv1d(const void *x, const float *weight,
                             const float *bias, void *out, int64_t batch,
                             int64_t dim, int64_t seqlen, int64_t width,
                             ssd_dtype x_dtype, ssd_dtype out_dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SSD_H_ */

// Stage 2: the inter-chunk state pass.
//
// For every (b, h): S = init (or 0); for chunk c = 0, 1, ...:
//   states[b,h,c] = S
//   S = 2^{g_last} S + X_c^T (w o B_c),   w_t = dt_t 2^{g_last - g_t}
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", sections "Step 1: Jump the State Across a Chunk with One Matmul",
// "Step 3: Add Back the Decay, Safely, in Log-Space" and "Kernel 2:
// fwd_pass_state": the state is stored before each chunk's update, and the
// sequential dependence stays inside one program.)  Every kept exponent
// g_last - g_t is <= 0 because A dt <= 0, so nothing here can overflow.
//
// MI355X design.
// * One workgroup (4 waves) owns the state slice S[0:64, n0:n0+BN] of one
//   (b, h) and walks the chunks in order; slices of all (b, h, n-tile) run in
//   parallel.  Wave w owns rows p in [16w, 16w+16).
// * The slice is computed transposed, S^T[n][p], so each lane's four
//   accumulator registers are four consecutive n at one p: the per-chunk state
//   store and the final store are 16-byte writes straight from registers.
// * A chunk's contribution P_c = X_c^T (w o B_c) does not depend on the
//   carried state, so it is accumulated in fresh registers and the only
//   sequential step is S = 2^{g_last} S + P_c.  Everything else is streamed:
//   the global loads of chunk c + D are issued while chunk c is processed
//   (a D-deep register ring; the chunk loop is unrolled D times so every ring
//   slot is a fixed set of registers), the LDS operand tiles are double
//   buffered, and the per-token weights w of chunk c + 1 are formed while
//   chunk c is processed, so one barrier per chunk suffices.
// * The contraction runs over tokens, which are the slow axis of both x and
//   B in memory.  Each chunk's X and w o B tiles are therefore written to LDS
//   token-contiguous ([p][t] and [n][t]) by the threads that load them, so
//   every matrix operand is one 16-byte LDS read.
// * bf16 inputs: X is an exact bf16 operand; w o B is a computed fp32 value,
//   split into bf16 hi + lo (two MFMAs) so the product keeps ~16 mantissa bits
//   under fp32 accumulation; a single bf16 rounding of it loses the output
//   tolerance.  fp32 inputs use the fp32 matrix instruction directly.
// * Block ids are remapped so the n-tiles of one (b, h) land on one XCD and
//   share its L2 for the X chunk they all read.
// HBM traffic per (b, h, chunk): x (e*T*64) + B (e*T*N, shared by the heads
// of a group) + dt, g (8*T) + the stored state (4*64*N); the stored states
// dominate, so the stage is HBM-bound.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// A byte offset past every buffer range used here (reads return zero).
constexpr uint32_t kPastRange = 0x7FFFFFF0u;

// Map the hardware block id so consecutive logical tiles run on one XCD
// (blocks are dealt to the 8 XCDs round-robin).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  if (total % 8) return bid;
  return (bid % 8) * (total / 8) + bid / 8;
}

// ---------------------------------------------------------------- bf16 path
// Workgroup tile: HB heads of one group x 16 RS state rows (p0..) x BN state
// columns (n0..n0+BN-1); one wave per (head, 16-row slice, NBW blocks of 16
// columns).
// The chunk is streamed in token tiles of TK = 128 tokens: a chunk of 256
// spans two tiles, a tile holds two chunks of 64 (halving the sequential
// steps, whose fixed cost dominates at small batch x heads).  Per tile, the
// B columns n0..n0+BN-1 are staged once, exact, and serve all HB heads; the
// decay weight is folded into x instead:
//   P^T[n][p] = sum_t B[t][n] (w_t x_t[p]),  w_t = dt_t 2^{g_last - g_t},
// with w o x a computed fp32 value split into bf16 hi + lo (two MFMAs), so
// the product keeps ~16 mantissa bits under fp32 accumulation.  With 16-row
// slices (RS = 1) a workgroup reads 16 columns of x per head and shares one
// B tile among its heads, which keeps 256 equal tiles even at few (b, h)
// pairs; with many pairs, whole heads (RS = 4, 128 columns) use every byte of
// each x line they fetch.
// Both operand tiles sit in LDS token-major ([t][n], [t][p]) and the matrix
// operands are read with the LDS transpose read.  k-slot map of one 32-token
// step kk for lane group lq: slots 0..3 <-> tokens 32kk + 4lq + 0..3, slots
// 4..7 <-> tokens 32kk + 16 + 4lq + 0..3 (both operands alike).  Row strides
// are chosen so each 32-lane pass of a transpose read touches every LDS bank
// once.
template <int N>
struct BfTileStride {
  static constexpr int value = N == 16 ? 16 : N + 16;
};

template <int HB, int RS, int BN, int NBW>
struct BfTile {
  static constexpr int WPH = BN / (16 * NBW);   // waves per 16-row slice of a head
  static constexpr int NTHR = 64 * HB * RS * WPH;
};

template <int T, int N, int HB, int RS, int BN, int NBW, int Q>
__global__ __launch_bounds__(64 * HB * RS * (BN / (16 * NBW))) void state_pass_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dt_t, const float* __restrict__ g,
    const float* __restrict__ init, float* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int G, int nc) {
  constexpr int TK = 128;                      // tokens per tile
  constexpr int R = T > TK ? T / TK : 1;       // tiles per chunk
  constexpr int CPT = T < TK ? TK / T : 1;     // chunks per tile
  constexpr int WPH = BfTile<HB, RS, BN, NBW>::WPH;
  constexpr int NTHR = BfTile<HB, RS, BN, NBW>::NTHR;
  constexpr int XS = BfTileStride<16 * RS>::value;  // w o x row stride (bf16)
  constexpr int BS = BfTileStride<BN>::value;  // B row stride (bf16)
  constexpr int kXUnits = HB * TK * 2 * RS;    // (head, token, 8 of the 16 RS p)
  constexpr int XU = (kXUnits + NTHR - 1) / NTHR;
  constexpr int kBUnits = TK * (BN / 8);       // (token, 8 n)
  constexpr int BU = (kBUnits + NTHR - 1) / NTHR;
  __shared__ __attribute__((aligned(16))) uint16_t bts[2][TK * BS];
  __shared__ __attribute__((aligned(16))) uint16_t whs[2][HB * TK * XS];
  __shared__ __attribute__((aligned(16))) uint16_t wls[2][HB * TK * XS];

  constexpr int NT = N / BN;
  constexpr int NPS = kHeadDim / (16 * RS);    // row tiles of the state
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int ntile = logical % NT;
  const int ps = (logical / NT) % NPS;
  const int hblk = logical / (NT * NPS);
  const int nhb = H / HB;
  const int b = hblk / nhb, h0 = (hblk % nhb) * HB;
  const int grp = h0 / (H / G);
  const int n0 = ntile * BN, p0 = 16 * RS * ps;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int hh = wave / (RS * WPH);            // this wave's head in the block
  const int rs = (wave / WPH) % RS;            // its 16-row slice of the tile
  const int nb0 = (wave % WPH) * NBW;          // its first 16-column block
  const int h = h0 + hh;
  const int ntiles = R > 1 ? nc * R : (nc + CPT - 1) / CPT;

  // Buffer descriptors.  x and B: reads past the sequence's last token
  // return zero.  g and dt_t: the HB heads' rows, [hh][L]; token indices at
  // or past L are redirected past the range.
  const uint32_t xrow = (uint32_t)(H * kHeadDim), brow = (uint32_t)(G * N);
  const rsrc_t xr = make_rsrc(x + (size_t)b * L * H * kHeadDim, (uint32_t)L * xrow * 2u);
  const rsrc_t br = make_rsrc(Bm + ((size_t)b * L * G + grp) * N,
                              ((uint32_t)(L - 1) * brow + N) * 2u);
  const size_t grow = ((size_t)b * H + h0) * L;
  const rsrc_t gr = make_rsrc(g + grow, (uint32_t)(HB * L) * 4u);
  const rsrc_t dr = make_rsrc(dt_t + grow, (uint32_t)(HB * L) * 4u);

  // State block of this wave: acc[j] holds
  // S_h[p0 + 16 rs + lr][n0 + 16 (nb0 + j) + 4 lq + 0..3].
  f32x4 acc[NBW];
  const size_t sbase = ((size_t)b * H + h) * kHeadDim * N + (size_t)(p0 + 16 * rs + lr) * N +
                       n0 + 16 * nb0 + 4 * lq;
#pragma unroll
  for (int j = 0; j < NBW; ++j)
    acc[j] = init ? *(const f32x4*)(init + sbase + 16 * j) : (f32x4){0, 0, 0, 0};
  // Let the initial state land before the pipeline starts, so waits inside
  // the loop only ever concern tile loads.
  __builtin_amdgcn_s_waitcnt(0);

  // Staging units of this thread.  x unit u: head u / (2 RS TK), token
  // (u / (2 RS)) % TK, columns p0 + 8 (u % (2 RS)) .. + 7.  B unit u: token
  // u / (BN/8), columns n0 + 8 (u % (BN/8)) .. + 7.  Idle units read past the
  // range, so every thread issues the same loads.
  uint32_t xoff[XU], gtok[XU], ghead[XU], boff[BU];
  int xlds[XU], blds[BU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = tid + NTHR * i;
    const bool on = u < kXUnits;
    const int uh = on ? u / (2 * RS * TK) : 0, t = (u / (2 * RS)) % TK, half = u % (2 * RS);
    xoff[i] = on ? (((uint32_t)t * H + h0 + uh) * kHeadDim + p0 + 8 * half) * 2u : kPastRange;
    gtok[i] = on ? (uint32_t)t : (uint32_t)L;    // token within the tile (L: never valid)
    ghead[i] = (uint32_t)uh * L;
    xlds[i] = (uh * TK + t) * XS + 8 * half;
  }
#pragma unroll
  for (int i = 0; i < BU; ++i) {
    const int u = tid + NTHR * i;
    const int t = u / (BN / 8), c8 = u % (BN / 8);
    boff[i] = u < kBUnits ? ((uint32_t)t * brow + n0 + 8 * c8) * 2u : kPastRange;
    blds[i] = t * BS + 8 * c8;
  }
  const uint32_t xstep = xrow * 2u, bstep = brow * 2u;   // bytes per token

  // Raw global data of one tile: x units with their token's g and dt and
  // their head's g at the chunk's last token; B units; and g at the chunk's
  // last token for this wave's own head (its decay).
  struct Tile {
    u32x4 x[XU];
    float g[XU], dt[XU], gl[XU];
    u32x4 b[BU];
    float dl[CPT];
  };

  auto issue = [&](int k, Tile& tl) {
    // the tile's first chunk; a token t of the tile lies in chunk c + t / T
    const int c = R > 1 ? k / R : k * CPT;
    const uint32_t t0 = (uint32_t)(k * TK);
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      tl.x[i] = load_b128(xr, xoff[i] + t0 * xstep);
      const uint32_t tt = t0 + gtok[i];
      const uint32_t go = tt < (uint32_t)L ? (ghead[i] + tt) * 4u : kPastRange;
      tl.g[i] = load_f32(gr, go);
      tl.dt[i] = load_f32(dr, go);
      const int cu = c + (CPT > 1 ? (int)(gtok[i] % TK) / T : 0);
      const uint32_t tlast = (uint32_t)(min(cu * T + T, L) - 1);
      tl.gl[i] = load_f32(gr, (ghead[i] + tlast) * 4u);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) tl.b[i] = load_b128(br, boff[i] + t0 * bstep);
#pragma unroll
    for (int part = 0; part < CPT; ++part)
      tl.dl[part] = load_f32(gr, ((uint32_t)hh * L + (uint32_t)(min((c + part) * T + T, L) - 1)) * 4u);
  };

  // B (as loaded) and the split w o x of a tile into LDS buffer `buf`.
  // Tokens past the end read dt = g = 0 and x = 0, so w o x = 0.
  auto commit = [&](int buf, const Tile& tl) {
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      if (tid + NTHR * i < kXUnits) {
        const float w = tl.dt[i] * exp2_hw(tl.gl[i] - tl.g[i]);
        uint32_t hv[4], lv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          split_bf16(bf16_lo(tl.x[i][e]) * w, bf16_hi(tl.x[i][e]) * w, hv[e], lv[e]);
        *(u32x4*)(whs[buf] + xlds[i]) = make_u32x4(hv);
        *(u32x4*)(wls[buf] + xlds[i]) = make_u32x4(lv);
      }
    }
#pragma unroll
    for (int i = 0; i < BU; ++i)
      if (tid + NTHR * i < kBUnits) *(u32x4*)(bts[buf] + blds[i]) = tl.b[i];
  };

  // Transpose-read addresses of this lane (element offsets within a tile).
  const int rsel = 4 * lq + (lr >> 2), csel = 4 * (lr & 3);
  const int wrd = (hh * TK + rsel) * XS + 16 * rs + csel;
  const int brd = rsel * BS + 16 * nb0 + csel;

  f32x4 ph[NBW], pl[NBW];
  // One step of the sequential pass for tile k: for each chunk part of the
  // tile, the state store at a chunk start, the part's matrix products from
  // LDS buffer k & 1 and the state update S = 2^{g_last} S + P at a chunk
  // end; then the staging of tile k + 1 into the other buffer and one
  // barrier.
  auto step = [&](int k, const Tile& cur, const Tile& next) {
    const int buf = k & 1;
    // The tile's token k-steps: part `part` (one chunk of T tokens when a
    // tile holds several chunks) covers k-steps [part T/32, (part+1) T/32).
    constexpr int KPP = TK / 32 / CPT;
#pragma unroll
    for (int part = 0; part < CPT; ++part) {
      const int c = R > 1 ? k / R : k * CPT + part;      // chunk of this part
      const bool first = R > 1 ? k % R == 0 : true;      // the chunk starts here
      const bool last = R > 1 ? k % R == R - 1 : true;   // the chunk ends here
      if (c < nc) {
        if (first) {
          float* dst = states + (((size_t)b * H + h) * nc + c) * kHeadDim * N +
                       (size_t)(p0 + 16 * rs + lr) * N + n0 + 16 * nb0 + 4 * lq;
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            *(f32x4*)(dst + 16 * j) = acc[j];
            ph[j] = pl[j] = (f32x4){0, 0, 0, 0};
          }
        }
#pragma unroll
        for (int kq = 0; kq < KPP; ++kq) {
          const int kk = part * KPP + kq;
          const u32x2 a0 = lds_read_tr16(whs[buf] + wrd + 32 * kk * XS);
          const u32x2 a1 = lds_read_tr16(whs[buf] + wrd + (32 * kk + 16) * XS);
          const u32x2 c0 = lds_read_tr16(wls[buf] + wrd + 32 * kk * XS);
          const u32x2 c1 = lds_read_tr16(wls[buf] + wrd + (32 * kk + 16) * XS);
          const u32x4 wxh = {a0[0], a0[1], a1[0], a1[1]};
          const u32x4 wxl = {c0[0], c0[1], c1[0], c1[1]};
#pragma unroll
          for (int j = 0; j < NBW; ++j) {
            const int o0 = brd + 32 * kk * BS + 16 * j;
            const u32x2 e0 = lds_read_tr16(bts[buf] + o0);
            const u32x2 e1 = lds_read_tr16(bts[buf] + o0 + 16 * BS);
            const u32x4 bv = {e0[0], e0[1], e1[0], e1[1]};
            ph[j] = mfma_bf16(bv, wxh, ph[j]);
            pl[j] = mfma_bf16(bv, wxl, pl[j]);
          }
        }
        if (last) {
          const float decay = exp2_hw(cur.dl[part]);
#pragma unroll
          for (int j = 0; j < NBW; ++j) acc[j] = decay * acc[j] + (ph[j] + pl[j]);
        }
      }
    }
    if (k + 1 < ntiles) commit(buf ^ 1, next);
    __syncthreads();
  };

  // Two groups of Q tiles: one group is consumed while the other group's
  // loads are in flight, then the roles swap.  Within one pass of the loop
  // body the code is straight-line, so the compiler's memory-wait counts let
  // the other group's loads stay outstanding; scheduling barriers pin each
  // group's loads in place so they are issued in the same order on every
  // path into the loop.  Tiles past the end are issued too (their loads fall
  // outside every range and cost nothing).
  Tile ga[Q], gb[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) issue(q, ga[q]);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int q = 0; q < Q; ++q) issue(Q + q, gb[q]);
  __builtin_amdgcn_sched_barrier(0);
  commit(0, ga[0]);
  __syncthreads();
  for (int k0 = 0; k0 < ntiles; k0 += 2 * Q) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (k0 + q < ntiles) step(k0 + q, ga[q], q + 1 < Q ? ga[q + 1] : gb[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < Q; ++q) issue(k0 + 2 * Q + q, ga[q]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (k0 + Q + q < ntiles) step(k0 + Q + q, gb[q], q + 1 < Q ? gb[q + 1] : ga[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = 0; q < Q; ++q) issue(k0 + 3 * Q + q, gb[q]);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (final_state) {
#pragma unroll
    for (int j = 0; j < NBW; ++j) *(f32x4*)(final_state + sbase + 16 * j) = acc[j];
  }
}

// ---------------------------------------------------------------- fp32 path
// Token tiles of TK = 64.  k-map for v_mfma_f32_16x16x4_f32: step (u, v)
// gives lane group lq the token 16u + 4lq + v of the tile, so each lane reads
// four steps' operands at once.  Staging units are (4 columns x 4 tokens).
template <int T, int N, int BN, int D>
__global__ __launch_bounds__(256) void state_pass_f32(
    const float* __restrict__ x, const float* __restrict__ Bm,
    const float* __restrict__ dt_t, const float* __restrict__ g,
    const float* __restrict__ init, float* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int G, int nc) {
  static_assert(D >= 2, "the weights of tile k+1 come from another ring slot");
  constexpr int TK = 64;
  constexpr int R = T / TK;
  constexpr int NB = BN / 16;
  constexpr int XS = TK + 4;                   // LDS row stride (floats)
  constexpr int XU = TK / 64;                  // X units per thread
  constexpr int kBUnits = (BN / 4) * (TK / 4);
  constexpr int BU = (kBUnits + 255) / 256;
  __shared__ __attribute__((aligned(16))) float xs[2][64 * XS];
  __shared__ __attribute__((aligned(16))) float bs[2][BN * XS];
  __shared__ __attribute__((aligned(16))) float ws[2][TK];

  constexpr int NT = N / BN;
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int ntile = logical % NT;
  const int bh_idx = logical / NT;
  const int b = bh_idx / H, h = bh_idx % H, grp = h / (H / G);
  const int n0 = ntile * BN;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int p = 16 * wave + lr;
  const int ntiles = nc * R;

  const float* gh = g + (size_t)bh_idx * L;
  const uint32_t xrow = (uint32_t)(H * kHeadDim), brow = (uint32_t)(G * N);
  const rsrc_t xr = make_rsrc(x + ((size_t)b * L * H + h) * kHeadDim,
                              ((uint32_t)(L - 1) * xrow + kHeadDim) * 4u);
  const rsrc_t br = make_rsrc(Bm + ((size_t)b * L * G + grp) * N,
                              ((uint32_t)(L - 1) * brow + N) * 4u);
  const rsrc_t gr = make_rsrc(gh, (uint32_t)L * 4u);
  const rsrc_t dr = make_rsrc(dt_t + (size_t)bh_idx * L, (uint32_t)L * 4u);

  f32x4 acc[NB];
  const size_t sbase = (size_t)bh_idx * kHeadDim * N + (size_t)p * N + n0 + 4 * lq;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    acc[nb] = init ? *(const f32x4*)(init + sbase + 16 * nb) : (f32x4){0, 0, 0, 0};
  // Let the initial state land before the tile ring starts, so waits inside
  // the loop only ever concern ring loads.
  __builtin_amdgcn_s_waitcnt(0);

  struct Slot {
    f32x4 x[XU][4];
    f32x4 b[BU][4];
    float g, dt, glast;
  };
  Slot ring[D];

  uint32_t xoff[XU], boff[BU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int u = tid + 256 * i;
    xoff[i] = ((uint32_t)(4 * (u >> 4)) * xrow + 4 * (u & 15)) * 4u;
  }
#pragma unroll
  for (int i = 0; i < BU; ++i) {
    const int u = tid + 256 * i;
    boff[i] = u < kBUnits
        ? ((uint32_t)(4 * (u / (BN / 4))) * brow + n0 + 4 * (u % (BN / 4))) * 4u
        : kPastRange;
  }
  const uint32_t xstep = xrow * 4u, bstep = brow * 4u;

  auto issue = [&](int k, Slot& sl) {
    const int c = k / R;
    const uint32_t t0 = (uint32_t)(k * TK);
#pragma unroll
    for (int i = 0; i < XU; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sl.x[i][r] = load_f32x4(xr, xoff[i] + (t0 + r) * xstep);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sl.b[i][r] = load_f32x4(br, boff[i] + (t0 + r) * bstep);
    }
    sl.g = load_f32(gr, (t0 + tid) * 4u);
    sl.dt = load_f32(dr, (t0 + tid) * 4u);
    sl.glast = load_f32(gr, (uint32_t)(min(c * T + T, L) - 1) * 4u);
  };

  auto commit_w = [&](int k, const Slot& sl, float& decay) {
    if (tid < TK) ws[k & 1][tid] = sl.dt * exp2_hw(sl.glast - sl.g);
    decay = exp2_hw(sl.glast);
  };

  auto commit_xb = [&](int k, const Slot& sl) {
    const int buf = k & 1;
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + 256 * i;
      const int pq = u & 15, tq = u >> 4;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(xs[buf] + (4 * pq + e) * XS + 4 * tq) =
            (f32x4){sl.x[i][0][e], sl.x[i][1][e], sl.x[i][2][e], sl.x[i][3][e]};
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
      const int u = tid + 256 * i;
      if (u < kBUnits) {
        const int nq = u % (BN / 4), tq = u / (BN / 4);
        const f32x4 w = *(const f32x4*)(ws[buf] + 4 * tq);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          *(f32x4*)(bs[buf] + (4 * nq + e) * XS + 4 * tq) =
              (f32x4){sl.b[i][0][e] * w[0], sl.b[i][1][e] * w[1],
                      sl.b[i][2][e] * w[2], sl.b[i][3][e] * w[3]};
      }
    }
  };

  // Tiles past the end are issued too: their loads fall outside every
  // buffer range, cost no memory traffic and keep the wait counts exact.
#pragma unroll
  for (int s = 0; s < D; ++s) issue(s, ring[s]);
  float decay_cur = 1.0f, decay_next = 1.0f;
  commit_w(0, ring[0], decay_cur);
  __syncthreads();

  f32x4 pc[NB];
  for (int k0 = 0; k0 < ntiles; k0 += D) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      const int k = k0 + s;
      if (k >= ntiles) break;
      const int sub = k % R;
      if (sub == 0) {
        float* dst = states + ((size_t)bh_idx * nc + k / R) * kHeadDim * N + (size_t)p * N + n0 + 4 * lq;
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          *(f32x4*)(dst + 16 * nb) = acc[nb];
          pc[nb] = (f32x4){0, 0, 0, 0};
        }
      }
      commit_xb(k, ring[s]);
      float dnext = decay_next;
      if (k + 1 < ntiles) commit_w(k + 1, ring[(s + 1) % D], dnext);
      issue(k + D, ring[s]);
      __syncthreads();

      const int buf = k & 1;
#pragma unroll
      for (int u = 0; u < TK / 16; ++u) {
        const f32x4 xv = *(const f32x4*)(xs[buf] + p * XS + 16 * u + 4 * lq);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const f32x4 bv = *(const f32x4*)(bs[buf] + (16 * nb + lr) * XS + 16 * u + 4 * lq);
#pragma unroll
          for (int v = 0; v < 4; ++v) pc[nb] = mfma_f32(bv[v], xv[v], pc[nb]);
        }
      }
      if (sub == R - 1) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) acc[nb] = decay_cur * acc[nb] + pc[nb];
      }
      if (k + 1 < ntiles && (k + 1) % R == 0) decay_cur = dnext;
      decay_next = dnext;
    }
  }
  if (final_state) {
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) *(f32x4*)(final_state + sbase + 16 * nb) = acc[nb];
  }
}

// ------------------------------------------------------------- launching
// bf16 workgroup tiles (heads HB, state columns BN, 16-column blocks per
// wave NBW), in order of preference: the first that divides the heads of a
// group (so the heads of a tile share B) and still gives one workgroup per
// CU is used, else the one with the most workgroups.  Measured on MI355X:
// tiles with 64 columns (each B row one 128-byte line) beat narrower ones
// with fewer bytes but more partial lines, and among those more heads per
// tile (fewer x and B requests per state element) is faster.
struct BfCfg {
  int hb, rs, bn, nbw;
};
// Workgroup tiles (heads, 16-row slices, columns, column blocks per wave).
constexpr BfCfg kBfCfgs[] = {{4, 1, 64, 2}, {3, 1, 64, 1}, {2, 1, 64, 1}, {1, 1, 64, 1},
                             {2, 1, 32, 1}, {1, 1, 32, 1}, {1, 1, 16, 1}, {1, 4, 128, 4},
                             {1, 4, 64, 1}};
constexpr int kWholeHeadCfg = 7;
constexpr int kHalfHeadCfg = 8;
constexpr int kNumBfCfgs = sizeof(kBfCfgs) / sizeof(kBfCfgs[0]);

int64_t bf_cfg_wgs(const BfCfg& c, const Shape& s) {
  return s.batch * (s.nheads / c.hb) * (kHeadDim / (16 * c.rs)) * (s.dstate / c.bn);
}

int choose_bf_cfg(const Shape& s, int cus) {
  // Whole-head tiles (64 rows x 128 columns) read each x line once per
  // workgroup instead of once per 16-row slice; they win once there are
  // enough (b, h) pairs to occupy most CUs (measured: 190 -> 163 us on the
  // 2 x 8192-token, 80-head layer; slower with 96 or 32 pairs).
  const int64_t pairs = s.batch * s.nheads;
  if (s.dstate == 128 && pairs * 5 >= (int64_t)cus * 3) return kWholeHeadCfg;
  // Half-head tiles (64 rows x 64 columns, 16 waves) also read whole x
  // lines; with 3/8 to 1/2 as many (b, h) pairs as CUs they give one tile
  // per CU on 3/4 of the chip or more, and beat 16-row tiles on every CU
  // (measured: 51.8 -> 47.3 us on the 4 x 2048-token, 24-head layer).
  if (s.dstate == 128 && pairs * 8 >= (int64_t)cus * 3 && pairs * 2 <= (int64_t)cus)
    return kHalfHeadCfg;
  const int64_t hpg = s.nheads / s.ngroups;
  int most = -1;
  int64_t most_wgs = -1;
  for (int i = 0; i < kNumBfCfgs; ++i) {
    const BfCfg c = kBfCfgs[i];
    if (c.rs != 1 || hpg % c.hb != 0 || c.bn > s.dstate) continue;
    const int64_t wgs = bf_cfg_wgs(c, s);
    if (wgs >= cus) return i;
    if (wgs > most_wgs) {
      most = i;
      most_wgs = wgs;
    }
  }
  return most;
}

// Compute units of the current device (the MI355X count if the query fails;
// only the tile choice depends on it), cached per device.
int device_cus() {
  static PerDeviceInt cache;
  const int cus = cache.get(query_cus);
  return cus > 0 ? cus : 256;
}

template <int T, int N, int HB, int RS, int BN, int NBW>
int launch_bf(const uint16_t* x, const uint16_t* B, const float* dt_t, const float* g,
              const float* init, float* states, float* fin, const Shape& s,
              hipStream_t st) {
  if constexpr (BN > N) {
    return (int)hipErrorInvalidValue;   // never chosen: the chooser checks BN <= N
  } else {
    constexpr int NTHR = BfTile<HB, RS, BN, NBW>::NTHR;
    // tiles per group: two, unless one tile's registers are many (deeper
    // groups measured no faster)
    constexpr int CPT = T < 128 ? 128 / T : 1;
    constexpr int XU = (HB * 128 * 2 * RS + NTHR - 1) / NTHR;
    constexpr int BU = (128 * (BN / 8) + NTHR - 1) / NTHR;
    constexpr int Q = 7 * XU + 4 * BU + CPT <= 24 ? 2 : 1;
    const unsigned blocks =
        (unsigned)(s.batch * (s.nheads / HB) * (kHeadDim / (16 * RS)) * (N / BN));
    hipLaunchKernelGGL((state_pass_bf16<T, N, HB, RS, BN, NBW, Q>), dim3(blocks), dim3(NTHR),
                       0, st, x, B, dt_t, g, init, states, fin, (int)s.seqlen, (int)s.nheads,
                       (int)s.ngroups, (int)s.nchunks());
    return (int)hipGetLastError();
  }
}

template <int T, int N>
int launch_bf_n(const void* x, const void* B, const float* dt_t, const float* g,
                const float* init, float* states, float* fin, const Shape& s,
                hipStream_t st) {
  const uint16_t* xb = (const uint16_t*)x;
  const uint16_t* bb = (const uint16_t*)B;
  switch (choose_bf_cfg(s, device_cus())) {
    case 0: return launch_bf<T, N, 4, 1, 64, 2>(xb, bb, dt_t, g, init, states, fin, s, st);
    case 1: return launch_bf<T, N, 3, 1, 64, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    case 2: return launch_bf<T, N, 2, 1, 64, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    case 3: return launch_bf<T, N, 1, 1, 64, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    case 4: return launch_bf<T, N, 2, 1, 32, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    case 5: return launch_bf<T, N, 1, 1, 32, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    case kWholeHeadCfg:
      return launch_bf<T, N, 1, 4, 128, 4>(xb, bb, dt_t, g, init, states, fin, s, st);
    case kHalfHeadCfg:
      return launch_bf<T, N, 1, 4, 64, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
    default: return launch_bf<T, N, 1, 1, 16, 1>(xb, bb, dt_t, g, init, states, fin, s, st);
  }
}

// fp32 n-tile width: the widest tile that still gives >= 1024 workgroups
// (four per CU), else the narrowest.
int choose_bn(const Shape& s) {
  const int64_t pairs = s.batch * s.nheads;
  for (int bn : {64, 32}) {
    if (bn <= s.dstate && pairs * (s.dstate / bn) >= 1024) return bn;
  }
  return 16;
}

template <int T, int N, int BN>
int launch_f32(const void* x, const void* B, const float* dt_t, const float* g,
               const float* init, float* states, float* fin, const Shape& s,
               hipStream_t st) {
  constexpr int D = BN >= 32 ? 2 : 4;   // register ring depth
  const unsigned blocks = (unsigned)(s.batch * s.nheads * (N / BN));
  hipLaunchKernelGGL((state_pass_f32<T, N, BN, D>), dim3(blocks), dim3(256), 0, st,
                     (const float*)x, (const float*)B, dt_t, g, init, states, fin,
                     (int)s.seqlen, (int)s.nheads, (int)s.ngroups, (int)s.nchunks());
  return (int)hipGetLastError();
}

template <int T, int N>
int launch_f32_n(const void* x, const void* B, const float* dt_t, const float* g,
                 const float* init, float* states, float* fin, const Shape& s,
                 hipStream_t st) {
  switch (choose_bn(s)) {
    case 64: return launch_f32<T, N, 64>(x, B, dt_t, g, init, states, fin, s, st);
    case 32: return launch_f32<T, N, 32>(x, B, dt_t, g, init, states, fin, s, st);
    default: return launch_f32<T, N, 16>(x, B, dt_t, g, init, states, fin, s, st);
  }
}

template <bool BF16, int T>
int launch_n(const void* x, const void* B, const float* dt_t, const float* g,
             const float* init, float* states, float* fin, const Shape& s,
             hipStream_t st) {
  if constexpr (BF16) {
    if (s.dstate == 64) return launch_bf_n<T, 64>(x, B, dt_t, g, init, states, fin, s, st);
    return launch_bf_n<T, 128>(x, B, dt_t, g, init, states, fin, s, st);
  } else {
    if (s.dstate == 64) return launch_f32_n<T, 64>(x, B, dt_t, g, init, states, fin, s, st);
    return launch_f32_n<T, 128>(x, B, dt_t, g, init, states, fin, s, st);
  }
}

template <bool BF16>
int launch_chunk(const void* x, const void* B, const float* dt_t, const float* g,
                 const float* init, float* states, float* fin, const Shape& s,
                 hipStream_t st) {
  switch (s.chunk) {
    case 64: return launch_n<BF16, 64>(x, B, dt_t, g, init, states, fin, s, st);
    case 128: return launch_n<BF16, 128>(x, B, dt_t, g, init, states, fin, s, st);
    default: return launch_n<BF16, 256>(x, B, dt_t, g, init, states, fin, s, st);
  }
}

// The two-level form (chunk_state, then state_passing) moves about twice the
// bytes of the one-pass kernel but has no chain per workgroup.  It wins
// where the one-pass grid is long chains on few waves: measured on the
// 65536-token, 32-head sequence (512 chunks, four waves per CU) it takes
// about 395 us against 400-490 (the one-pass time varies from run to run);
// with 32 chunks (small and large layers) it loses (80 vs 53 us, 166 vs
// 159 us).
bool use_two_level(const Shape& s, int cus) {
  const int c = choose_bf_cfg(s, cus);
  if (c < 0) return false;
  const BfCfg k = kBfCfgs[c];
  const int64_t chain_tiles = s.chunk > 128 ? s.nchunks() * (s.chunk / 128)
                                            : (s.nchunks() * s.chunk + 127) / 128;
  const int64_t waves = bf_cfg_wgs(k, s) * k.hb * k.rs * (k.bn / (16 * k.nbw));
  return chain_tiles >= 128 && waves <= 8 * (int64_t)cus;
}

}  // namespace

int launch_fwd_pass_state(const void* x, const void* B, const float* dt_t,
                          const float* g, const float* init_state,
                          float* states, float* final_state, bool bf16_in,
                          const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (bf16_in && use_two_level(s, device_cus())) {
    // P_{nc-1} is parked in the states[0] slot rather than in final_state,
    // so init_state may be the final_state buffer (a sequence continued in
    // place), as it may for the one-pass kernels.
    const int r = launch_chunk_state(x, B, dt_t, g, states, final_state, true, true, s, stream);
    if (r != 0) return r;
    return launch_state_passing(g, init_state, states, final_state, true, s, stream);
  }
  if (bf16_in)
    return launch_chunk<true>(x, B, dt_t, g, init_state, states, final_state, s, st);
  if (state_pair_f32_applies(s, false))
    return launch_state_pair_f32((const float*)x, (const float*)B, dt_t, g, init_state, states,
                                 final_state, s, stream);
  return launch_chunk<false>(x, B, dt_t, g, init_state, states, final_state, s, st);
}

}  // namespace ssd

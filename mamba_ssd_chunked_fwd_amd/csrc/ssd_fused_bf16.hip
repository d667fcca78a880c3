// Stages 2 and 3 in one pass for bf16 inputs (N = 128 state columns, heads
// of 64, chunks of 64, 128 or 256 tokens), with each (b, h) chain of chunks
// cut into runs so that enough workgroups walk chains at once.
//
// For each (b, h) the state entering chunk c is S_c and
//   S_{c+1} = 2^{g_last(c)} S_c + sum_{t in c} 2^{g_last(c) - g_t} dt_t x_t B_t^T
//   Y_c     = 2^{g_i} (C S_c^T) + L' X + D_h X
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile": the recurrence of "Kernel 2: fwd_pass_state" and the output of
// "Kernel 3: compute_out, the Fused Output Kernel" with "Step 2" and
// "Step 3").  As in the fp32 fused pass, walking the chunks of a (b, h) in
// order with the state in registers writes every S_c once and never reads
// one back, and reads x once.  The bf16 layers have too few (b, h) pairs for
// one walk per pair to fill the chip (96, 160 and 32 of them), so the chunks
// of a chain are cut into runs, walked at once: a lead run of R0 chunks and
// nr - 1 runs of R chunks (1 <= R0 <= R), R being the chunk steps per CU if
// the whole walk were spread evenly over the CUs.  The (b, head pair) lead
// runs that do not get a CU of their own share the spare ones, a few per
// workgroup, so no workgroup walks much more than R chunks:
//
// 1. run_state_bf16: for every run r but the last, E_r = the state after the
//    run from a zero start, parked in the states slot of the next run's
//    first chunk.
// 2. run_passing: S at the run starts, S_{c(r+1)} = 2^{d_r} S_{c(r)} + E_r
//    with c(r) the run's first chunk and d_r the sum of its g_last, in
//    place.  The same jump as stage 2's, over a run instead of one chunk.
// 3. fused_pair_bf16: one workgroup per (b, head pair, run) -- or per few
//    lead runs -- starting from each run's first state and walking its
//    chunks in 64-token blocks.
// With one run per chain (enough pairs for the chip) 1 and 2 do not run.
//
// A chunk of 128 or 256 tokens is evaluated as 2 or 4 blocks of 64 tokens
// with the state carried between them in registers: for the tokens of a
// block, the earlier tokens of the chunk act through the state at the block's
// start exactly as the earlier chunks act through S_c, so y and the states
// at chunk boundaries are the same sums, in another order.  g is the
// chunk's cumulative sum; a block that starts inside a chunk subtracts g of
// the token before it, which turns g into the block's own cumulative sum.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

#include <type_traits>

namespace ssd {
namespace {

constexpr int kN = 128;   // state columns of the bf16 fused pass
constexpr int kTB = 64;   // tokens per block
constexpr int kNontemporal = 2;   // cache-policy operand of a buffer store: the nt bit

// Consecutive logical items on one XCD (blocks are dealt round-robin).
__device__ __forceinline__ int xcd_map(int bid, int total) {
  if (total % 8) return bid;
  return (bid % 8) * (total / 8) + bid / 8;
}

// k-slot order of the columns of C (and the second copy of B): slot
// position of state column n, as the accumulator layout of S sets it.
__device__ __forceinline__ int kpos(int c) {
  return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3);
}

// eight consecutive fp32 values split into bf16 hi + lo fragments
__device__ __forceinline__ void split8_2(const f32x4& v0, const f32x4& v1, u32x4& hi,
                                         u32x4& lo) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t h, l;
    split_bf16(v0[2 * q], v0[2 * q + 1], h, l);
    hi[q] = h;
    lo[q] = l;
    split_bf16(v1[2 * q], v1[2 * q + 1], h, l);
    hi[2 + q] = h;
    lo[2 + q] = l;
  }
}

// ------------------------------------------------------------------ 1
// One workgroup (4 waves per head) per (b, run k, block of HB heads);
// wave 4 hh + w owns rows 16w..16w+15 of head hh and all N columns, transposed in the
// accumulators as in the other state kernels (lane: column p, four
// consecutive n).  The run is consumed in 64-token tiles through two
// LDS buffers: while the waves multiply tile s out of one, they stage tile
// s + 1 (x of both heads as loaded, B, and the weights w_t = dt_t
// 2^{g_last - g_t}) into the other from registers, and the loads of tile
// s + 3 go out; one barrier per tile.  Each wave reads its x columns with
// the transpose read, scales them by w and splits them (hi + lo) itself, as
// the fused kernel's update does.  At each chunk start the accumulated
// state is decayed by the chunk's 2^{g_last} before the chunk's tokens add.
// The runs it walks lie before the last run, so every chunk is whole.
template <int N, int HB>
__global__ __launch_bounds__(256 * HB) void run_state_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dt_t, const float* __restrict__ g, float* __restrict__ states,
    int L, int H, int G, int T, int nc, int R, int R0, int nsub) {
  constexpr int NT = 256 * HB, ST = 64;
  constexpr int XS = kHeadDim + 16;   // x row stride (bf16)
  constexpr int BS = N + 16;          // B row stride (bf16)
  constexpr int NB = N / 16;
  constexpr int PPT = 8 * HB;         // 16-byte pieces of x per token
  constexpr int BU = ST * N / 8 / NT; // 16-byte units of B per thread
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][HB][ST * XS];   // [buffer][head]
  __shared__ __attribute__((aligned(16))) uint16_t bts[2][ST * BS];
  __shared__ __attribute__((aligned(16))) float wts[2][HB][ST];          // [buffer][head]

  const int npr = H / HB;
  const int item = xcd_map(blockIdx.x, gridDim.x);
  const int h0 = (item % npr) * HB;
  const int k = (item / npr) % nsub;   // the run
  const int b = item / (npr * nsub);
  const int c0 = k == 0 ? 0 : R0 + (k - 1) * R;   // its first chunk
  const int rl = k == 0 ? R0 : R;                  // its chunks
  const int grp = h0 / (H / G);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = wave >> 2, wr = wave & 3;
  const int lr = lane & 15, lq = lane >> 4;
  const int spc = T / ST;          // tiles per chunk (1, 2 or 4)
  const int lgspc = 31 - __builtin_clz((unsigned)spc);
  const int nst = rl * spc;        // tiles of the run
  const int tb = c0 * T;           // its first token

  const uint32_t xrow = (uint32_t)H * kHeadDim * 2, brow = (uint32_t)G * N * 2;
  const uint32_t span = (uint32_t)(rl * T);
  const rsrc_t xr = make_rsrc(x + ((size_t)(b * (size_t)L + tb) * H + h0) * kHeadDim,
                              (span - 1) * xrow + HB * kHeadDim * 2);
  const rsrc_t br = make_rsrc(Bm + ((size_t)(b * (size_t)L + tb) * G + grp) * N,
                              (span - 1) * brow + N * 2);
  // x unit e = tid + NT u: token e / PPT, 16-byte piece e % PPT of the
  // block's HB adjacent 128-byte head rows (head piece / 8, columns
  // 8 (piece % 8)..); B unit e: token e / 16, piece e % 16.  The thread's
  // head picks its g and dt row by offset, so the descriptors stay uniform.
  // One thread in eight (piece % 8 == 0) also forms w_t of its (head, token).
  const int th = HB == 1 ? 0 : (tid % PPT) >> 3;
  const bool wthr = (tid & 7) == 0;
  const size_t grow = ((size_t)b * H + h0) * L + tb;
  const rsrc_t gr = make_rsrc(g + grow, ((uint32_t)L + span) * 4);
  const rsrc_t dr = make_rsrc(dt_t + grow, ((uint32_t)L + span) * 4);

  uint32_t xo[2], bo[BU], go[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + NT * u;
    xo[u] = (uint32_t)(e / PPT) * xrow + 16 * (e % PPT);
    go[u] = 4 * ((uint32_t)(e / PPT) + (uint32_t)th * L);
  }
#pragma unroll
  for (int u = 0; u < BU; ++u) {
    const int e = tid + NT * u;
    bo[u] = (uint32_t)(e >> 4) * brow + 16 * (e & 15);
  }
  const uint32_t gl_lane = 4 * (uint32_t)th * L;
  const uint32_t gl_wave = 4 * (uint32_t)hh * L;

  struct Regs {
    u32x4 xv[2], bv[BU];
    float gv[2], dv[2], gl;   // g, dt of the thread's units; g_last of their head's chunk
    float glw;                // g_last of this wave's head's chunk
  };
  // loads of tile s; past the run they read zero (x, B) or words of the
  // same rows (g, dt) that are never used
  auto issue = [&](int s, Regs& r) {
    const uint32_t t0 = (uint32_t)(s * ST);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      r.xv[u] = load_b128(xr, t0 * xrow + xo[u]);
      r.gv[u] = load_f32(gr, 4 * t0 + go[u]);
      r.dv[u] = load_f32(dr, 4 * t0 + go[u]);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) r.bv[u] = load_b128(br, t0 * brow + bo[u]);
    const uint32_t tl = 4u * (uint32_t)((s >> lgspc) * T + T - 1);   // the chunk's last token
    r.gl = load_f32(gr, gl_lane + tl);
    r.glw = load_f32(gr, gl_wave + tl);
  };
  auto stage = [&](const Regs& r, int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + NT * u, t = e / PPT;
      *(u32x4*)(xs[buf][th] + t * XS + 8 * (e & 7)) = r.xv[u];
      if (wthr) wts[buf][th][t] = r.dv[u] * exp2_hw(r.gl - r.gv[u]);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int e = tid + NT * u;
      *(u32x4*)(bts[buf] + (e >> 4) * BS + 8 * (e & 15)) = r.bv[u];
    }
  };

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0, 0, 0, 0};
  const int rsel = 4 * lq + (lr >> 2), csel = 4 * (lr & 3);

  // g_last of the chunk of the tile being multiplied (this wave's head),
  // taken from the tile's registers when it is staged
  float glw_cur = 0.0f;

  // tile s from buffer s & 1; stage tile s + 1 from rn into the other
  // buffer, then load tile s + 3 into rn
  auto step = [&](int s, Regs& rn) {
    const int buf = s & 1;
    const float glw = glw_cur;
    stage(rn, buf ^ 1);
    glw_cur = rn.glw;
    issue(s + 3, rn);
    if (s > 0 && (s & (spc - 1)) == 0) {
      const float dec = exp2_hw(glw);
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] *= dec;
    }
#pragma unroll
    for (int kk = 0; kk < ST / 32; ++kk) {
      // this wave's x columns, tokens 32 kk + 16 (e / 4) + 4 lq + e % 4,
      // scaled by w and split
      const int xo2 = (32 * kk + rsel) * XS + 16 * wr + csel;
      const u32x2 a0 = lds_read_tr16(xs[buf][hh] + xo2);
      const u32x2 a1 = lds_read_tr16(xs[buf][hh] + xo2 + 16 * XS);
      const f32x4 w0 = *(const f32x4*)(&wts[buf][hh][32 * kk + 4 * lq]);
      const f32x4 w1 = *(const f32x4*)(&wts[buf][hh][32 * kk + 16 + 4 * lq]);
      const f32x4 x0 = {bf16_lo(a0[0]) * w0[0], bf16_hi(a0[0]) * w0[1], bf16_lo(a0[1]) * w0[2],
                        bf16_hi(a0[1]) * w0[3]};
      const f32x4 x1 = {bf16_lo(a1[0]) * w1[0], bf16_hi(a1[0]) * w1[1], bf16_lo(a1[1]) * w1[2],
                        bf16_hi(a1[1]) * w1[3]};
      u32x4 bt[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int bb = (32 * kk + rsel) * BS + 16 * j + csel;
        const u32x2 e0 = lds_read_tr16(bts[buf] + bb), e1 = lds_read_tr16(bts[buf] + bb + 16 * BS);
        bt[j] = (u32x4){e0[0], e0[1], e1[0], e1[1]};
      }
      u32x4 wxh, wxl;
      split8_2(x0, x1, wxh, wxl);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        acc[j] = mfma_bf16(bt[j], wxh, acc[j]);
        acc[j] = mfma_bf16(bt[j], wxl, acc[j]);
      }
    }
    __syncthreads();   // tile s + 1 is staged; tile s's reads are done
  };

  Regs ra, rb;
  issue(0, ra);
  issue(1, rb);
  stage(ra, 0);
  glw_cur = ra.glw;
  issue(2, ra);
  __syncthreads();
  // steps alternate register sets: step s stages tile s + 1 from the set
  // that holds it (rb for even s) and reloads that set with tile s + 3
#pragma unroll 1
  for (int s = 0; s + 1 < nst; s += 2) {
    step(s, rb);
    step(s + 1, ra);
  }
  if (nst & 1) step(nst - 1, rb);

  // E_k into the slot of the chunk after the run
  float* dst = states + (((size_t)b * H + h0 + hh) * nc + (size_t)(c0 + rl)) * kHeadDim * N;
  const int p = 16 * wr + lr;
#pragma unroll
  for (int j = 0; j < NB; ++j) *(f32x4*)(dst + (size_t)p * N + 16 * j + 4 * lq) = acc[j];
}

// ------------------------------------------------------------------ 2
// A thread owns one 16-byte unit (four consecutive n of one row p) of one
// (b, h) and walks the runs: S_0 = init (or zero) is written to slot 0,
// then S_{c(r+1)} = 2^{d_r} S_{c(r)} + E_r into the slot of run r + 1's
// first chunk, where E_r is parked.  The runs' decay sums d_r (sums of their
// chunks' g_last) are formed first, one run per thread, into LDS.  Run r
// starts at chunk c(r) = 0 for r = 0, else R0 + (r - 1) R, and has R0
// chunks for r = 0, else R; nsub runs precede the last one.
template <int N>
__global__ __launch_bounds__(256) void run_passing_kernel(
    const float* __restrict__ g, const float* __restrict__ init, float* __restrict__ states,
    int L, int T, int nc, int R, int R0, int nsub) {
  constexpr int UNITS = kHeadDim * N / 4;
  constexpr int WPB = UNITS / 256;
  constexpr int D = 4;
  constexpr int MAXS = 1024;   // runs per pass over the decay sums
  __shared__ float dsum[MAXS];
  const int bh = blockIdx.x / WPB;
  const int u = (blockIdx.x % WPB) * 256 + threadIdx.x;
  const size_t ss = (size_t)kHeadDim * N;
  float* st = states + (size_t)bh * nc * ss + 4 * (size_t)u;
  const float* gh = g + (size_t)bh * L;
  f32x4 s = init ? *(const f32x4*)(init + bh * ss + 4 * (size_t)u) : (f32x4){0, 0, 0, 0};
  *(f32x4*)st = s;
  // slot of run k + 1's first chunk, where E_k is parked and S goes
  auto slot = [&](int k) { return (size_t)(R0 + k * R) * ss; };
#pragma unroll 1
  for (int k0 = 0; k0 < nsub; k0 += MAXS) {
    const int kn = min(MAXS, nsub - k0);
    __syncthreads();
    for (int k = threadIdx.x; k < kn; k += 256) {
      const int r = k0 + k, c0 = r == 0 ? 0 : R0 + (r - 1) * R, rl = r == 0 ? R0 : R;
      const float* q = gh + (size_t)c0 * T + T - 1;
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
      int c = 0;
      for (; c + 4 <= rl; c += 4) {
        s0 += q[(size_t)c * T];
        s1 += q[(size_t)(c + 1) * T];
        s2 += q[(size_t)(c + 2) * T];
        s3 += q[(size_t)(c + 3) * T];
      }
      for (; c < rl; ++c) s0 += q[(size_t)c * T];
      dsum[k] = (s0 + s1) + (s2 + s3);
    }
    __syncthreads();
#pragma unroll 1
    for (int j0 = 0; j0 < kn; j0 += D) {
      f32x4 e[D];
#pragma unroll
      for (int j = 0; j < D; ++j)
        e[j] = j0 + j < kn ? *(const f32x4*)(st + slot(k0 + j0 + j)) : (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < D; ++j) {
        if (j0 + j < kn) {
          s = exp2_hw(dsum[j0 + j]) * s + e[j];
          *(f32x4*)(st + slot(k0 + j0 + j)) = s;
        }
      }
    }
  }
}

// ------------------------------------------------------------------ 3
// Head-pair form (8 waves, two per SIMD): waves 4q..4q+3 on head q of the
// pair, wave 4q + w owning rows p = 16w..16w+15 of that head's state and of
// its Y^T[p][i] over the block's 64 tokens.
// * The state stays in accumulators, S[p][16 nb + 4 lq + rr] in lane
//   (p, lq), and feeds C S^T directly after a hi + lo split: its k slots
//   follow that layout, n = 32 kk + 16 (e / 4) + 4 lq + e % 4, and C is
//   staged with its columns in that order.
// * x of both heads, B and C are staged once per block; x is read back with
//   the transpose read straight into the operand of X^T L'^T (exact bf16)
//   and, scaled by w_t = dt_t 2^{g_last - g_t} and split, of the update.
// * Each of the ten lower 16x16 blocks of C B^T (exact bf16 operands) is
//   formed once, by one wave (two for waves 0 and 1), and turned into L' of
//   both heads (hi + lo) in LDS.
// * Every step's operands are loaded two steps ahead into one of two
//   register sets, staged after the step's L' barrier while the other waves
//   multiply by L'.  Within a step each product's LDS fragments are read
//   one group ahead of it (scheduling barriers keep the reads early), so a
//   wave waits on LDS once per phase rather than once per product.
// * Uniform address parts go into the buffer descriptors; their ranges end
//   at the sequence, so rows past it read zero and their stores are dropped.
// * Work items are (b, head pair, run) with the runs r >= 1 first (pairs
//   fastest) and then the lead runs.  Workgroup w < (number of runs r >= 1)
//   takes that one item; each of the others takes ks consecutive lead runs
//   (ks = 0: every workgroup takes items with a stride of the grid size).
//   A run's blocks are the steps.
template <bool YBF16>
__global__ __launch_bounds__(512) void fused_pair_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ dt_t, const float* __restrict__ g,
    const float* __restrict__ Dv, const float* __restrict__ init, float* __restrict__ states,
    float* __restrict__ final_state, void* __restrict__ y, int L, int H, int G, int T, int nc,
    int R, int R0, int nr, int chains, int ks) {
  constexpr int NT = 512, TB = kTB, N = kN, NIB = TB / 16, KN = N / 32;
  constexpr int XS = kHeadDim + 16;   // x tile row stride (bf16)
  constexpr int BS = N + 16;          // B row stride (bf16), natural column order
  constexpr int CS = N + 16;          // C and B row stride (bf16), columns in k-slot order
  // (16-byte reads of 16 rows x 4 column groups hit no bank twice when the
  // row stride is an odd multiple of 32 bytes: 288 here; at 272 every such
  // read took two passes)
  constexpr int LS = TB + 16;         // L' row stride (bf16), columns in k-slot order
  // (160 bytes: the 16-byte reads of X^T L'^T hit no bank twice; the fewer
  // 8-byte L' writes take more passes than at 144, which measured slower)
  constexpr uint32_t kYB = YBF16 ? 2 : 4;
  constexpr uint32_t kStateBytes = kHeadDim * N * 4;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][TB * XS];
  __shared__ __attribute__((aligned(16))) uint16_t bp[TB * BS];
  __shared__ __attribute__((aligned(16))) uint16_t bq[TB * CS];
  __shared__ __attribute__((aligned(16))) uint16_t cp[TB * CS];
  __shared__ __attribute__((aligned(16))) uint16_t lp[2][2][TB * LS];
  __shared__ __attribute__((aligned(16))) float gs[2][TB], ds[2][TB];
  __shared__ __attribute__((aligned(16))) float ws[2][TB];   // w_t = dt_t 2^{g_last - g_t}
  constexpr int YS = 2 * kHeadDim + 4;   // Y tile row stride (fp32): both heads' 64 columns
  __shared__ __attribute__((aligned(16))) float ys[TB * YS];

  const int nwg = gridDim.x;
  const int wg = xcd_map(blockIdx.x, nwg);
  // this workgroup's items: it0 + istride j, j < icount
  const int n_long = chains * (nr - 1), total = n_long + chains;
  int it0 = wg, istride = nwg, icount = wg < total ? (total - 1 - wg) / nwg + 1 : 0;
  if (ks > 0) {
    istride = 1;
    if (wg < n_long) {
      icount = 1;
    } else {
      it0 = n_long + (wg - n_long) * ks;
      icount = max(0, min(ks, total - it0));
    }
  }
  if (icount <= 0) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = wave >> 2, w = wave & 3;
  const int lr = lane & 15, lq = lane >> 4;
  const int hpg = H / G, npr = H / 2;
  const int lgT = 31 - __builtin_clz((unsigned)T);   // T is 64, 128 or 256
  const uint32_t xrow = (uint32_t)H * kHeadDim * 2;   // bytes per token of x
  const uint32_t brow = (uint32_t)G * N * 2;          // bytes per token of B and C
  const int p = 16 * w + lr;   // this lane's state row (operand row)

  // run r: first chunk, blocks
  auto run_c0 = [&](int r) { return r == 0 ? 0 : R0 + (r - 1) * R; };
  auto run_blocks = [&](int r) {
    const int tb = run_c0(r) * T, te = min(tb + (r == 0 ? R0 : R) * T, L);
    return (te - tb + TB - 1) / TB;
  };
  const int nrm = max(nr - 1, 1);
  auto item_run = [&](int it) { return it < n_long ? 1 + (it / npr) % nrm : 0; };
  int nsteps = 0;
  for (int j = 0; j < icount; ++j) nsteps += run_blocks(item_run(it0 + istride * j));

  // loop-invariant lane offsets (bytes) from each step's descriptor bases:
  // unit e = tid + 512 u is token e >> 4, 16-byte piece e & 15 of the row
  // (for x: the pair's two 128-byte head rows side by side)
  uint32_t xo_lane[2], bo_lane[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int e = tid + NT * u;
    xo_lane[u] = (uint32_t)(e >> 4) * xrow + 16 * (e & 15);
    bo_lane[u] = (uint32_t)(e >> 4) * brow + 16 * (e & 15);
  }
  const uint32_t gd_lane = 4 * (uint32_t)lane;
  const uint32_t so_lane = ((uint32_t)p * N + 4 * lq) * 4;

  // this wave's blocks (ib, jb) of C B^T: waves 0-3 (3, 3-w), waves 4-6
  // (2, 6-w), wave 7 (1, 0); waves 0 and 1 also (w, w)
  const int ncb = wave < 2 ? 2 : 1;
  auto blk_i = [&](int sl) { return sl == 1 ? wave : (wave < 4 ? 3 : (wave < 7 ? 2 : 1)); };
  auto blk_j = [&](int sl) {
    return sl == 1 ? wave : (wave < 4 ? 3 - wave : (wave < 7 ? 6 - wave : 0));
  };

  struct StepP {
    int b, h0, grp, r, t0;
    bool live, first;
  };
  struct Cursor {
    int k, blk, nb, j;   // step, block of the item, its blocks, item of the workgroup
    StepP st;
  };
  auto at_item = [&](Cursor& cu) {
    const int it = it0 + istride * cu.j;
    const int q = it < n_long ? it : it - n_long;
    const int pr = q % npr;
    cu.st.r = item_run(it);
    cu.st.b = it < n_long ? q / (npr * nrm) : q / npr;
    cu.st.h0 = 2 * pr;
    cu.st.grp = cu.st.h0 / hpg;
    cu.nb = run_blocks(cu.st.r);
  };
  auto set_step = [&](Cursor& cu) {
    cu.st.t0 = run_c0(cu.st.r) * T + TB * cu.blk;
    cu.st.first = cu.blk == 0;
    cu.st.live = cu.k < nsteps;
  };
  auto advance = [&](Cursor& cu) {
    ++cu.k;
    if (++cu.blk == cu.nb) {
      cu.blk = 0;
      ++cu.j;
      if (cu.k < nsteps) at_item(cu);
    }
    set_step(cu);
  };

  struct Regs {
    u32x4 xu[2], bu[2], cu[2];
    float gv, dv;   // g and dt (waves 0 and 2: heads 0 and 1)
    StepP st;       // the step these registers were loaded for
  };
  constexpr int NLOAD = 8;
  struct Src {
    rsrc_t xr, br, crr, gr, dr;
  };
  const bool gwave = wave == 0 || wave == 2;
  auto prepare = [&](const StepP& st, Src& sc) {
    const int t0 = st.t0;
    const uint32_t rows = (uint32_t)(L - t0);
    sc.xr = make_rsrc(x + (((size_t)st.b * L + t0) * H + st.h0) * kHeadDim,
                      st.live ? (rows * H - st.h0) * (kHeadDim * 2) : 0u);
    const size_t bcb = (((size_t)st.b * L + t0) * G + st.grp) * N;
    const uint32_t bcr = st.live ? (rows * G - st.grp) * (N * 2) : 0u;
    sc.br = make_rsrc(Bm + bcb, bcr);
    sc.crr = make_rsrc(Cm + bcb, bcr);
    // g and dt of both heads: wave 0 head 0, wave 2 head 1
    const size_t gro = ((size_t)st.b * H + st.h0 + ((wave >> 1) & 1)) * L + t0;
    const bool gl = st.live && gwave;
    sc.gr = make_rsrc(g + gro, gl ? rows * 4 : 0u);
    sc.dr = make_rsrc(dt_t + gro, gl ? rows * 4 : 0u);
  };
  auto issue_slot = [&](int j, const Src& sc, Regs& r) {
    if (j < 2) {
      r.xu[j] = load_b128(sc.xr, xo_lane[j]);
    } else if (j < 4) {
      r.bu[j - 2] = load_b128(sc.br, bo_lane[j - 2]);
    } else if (j < 6) {
      r.cu[j - 4] = load_b128(sc.crr, bo_lane[j - 4]);
    } else if (j == 6) {
      r.gv = load_f32(sc.gr, gd_lane);
    } else {
      r.dv = load_f32(sc.dr, gd_lane);
    }
  };

  f32x4 sacc[N / 16];   // S[p][16 nb + 4 lq + rr] of this wave's head
  f32x4 cbr[2];         // (B C^T)[16 jb + 4 lq + rr][16 ib + lr] of this wave's blocks

  // L' blocks that stay zero: (ib 0, jb 1) and (ib 2, jb 3), read as the
  // upper halves of 32-token k-steps on the diagonal
  for (int e = tid; e < 2 * 2 * 16 * 16; e += NT) {
    const int hh = e >> 9, blk = (e >> 8) & 1, r = (e >> 4) & 15, c = e & 15;
    const int i = blk == 0 ? r : 32 + r, j = blk == 0 ? 16 + c : 48 + c;
    lp[hh][0][i * LS + kpos(j)] = 0;
    lp[hh][1][i * LS + kpos(j)] = 0;
  }

  // D_h of the pair's heads for the step being computed (set when a step is
  // staged: an item's first step reads them); raw g of the last token of
  // the staged block (waves 0 and 2), the g before the next block when
  // that block continues a chunk
  float dcur[2] = {0.0f, 0.0f};
  float gprev = 0.0f;

  Regs ra, rb;
  Cursor cur;
  cur.k = 0;
  cur.blk = 0;
  cur.j = 0;
  at_item(cur);
  set_step(cur);
  {
    Src sc;
    prepare(cur.st, sc);
    ra.st = cur.st;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, ra);
    advance(cur);
    prepare(cur.st, sc);
    rb.st = cur.st;
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, rb);
    advance(cur);
  }

  // Staging of a step from its registers: x, B, C, g, dt and w of both
  // heads; the run's first state into the accumulators at a run start; S
  // to the states at a chunk start.  It runs in the previous step's last
  // phase, which reads only the L' planes.
  auto commit = [&](const Regs& r) {
    const StepP st = r.st;
    const size_t hrow = (size_t)st.b * H + st.h0 + hq;
    if (st.first) {
      dcur[0] = Dv[st.h0];
      dcur[1] = Dv[st.h0 + 1];
      // the run's first state: init_state (or zero: an empty range) for a
      // single run, else the slot the run passing wrote
      rsrc_t ires;
      if (nr > 1)
        ires = make_rsrc(states + (hrow * nc + (size_t)run_c0(st.r)) * (kHeadDim * N),
                         kStateBytes);
      else
        ires = init ? make_rsrc(init + hrow * (kHeadDim * N), kStateBytes)
                    : make_rsrc(states, 0u);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) sacc[nb] = load_f32x4(ires, so_lane + 64 * nb);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int e = tid + NT * u, t = e >> 4, c = e & 15;
      *(u32x4*)(xs[(e >> 3) & 1] + t * XS + 8 * (e & 7)) = r.xu[u];
      *(u32x4*)(bp + t * BS + 8 * c) = r.bu[u];
      const int o0 = t * CS + kpos(8 * c), o1 = t * CS + kpos(8 * c + 4);
      *(u32x2*)(bq + o0) = (u32x2){r.bu[u][0], r.bu[u][1]};
      *(u32x2*)(bq + o1) = (u32x2){r.bu[u][2], r.bu[u][3]};
      *(u32x2*)(cp + o0) = (u32x2){r.cu[u][0], r.cu[u][1]};
      *(u32x2*)(cp + o1) = (u32x2){r.cu[u][2], r.cu[u][3]};
    }
    if (gwave) {
      // g relative to the block, dt and the update weight of one head:
      // lane = token; tokens past the end read g = dt = 0 (w = 0) and get
      // g = 0
      const int hh = wave >> 1;
      const int nt = min(TB, L - st.t0);
      const int gl = __builtin_amdgcn_readlane(__float_as_int(r.gv), nt - 1);
      // a block inside a chunk follows a whole block of the same chunk
      const float gb = (st.t0 & (T - 1)) != 0 ? gprev : 0.0f;
      gprev = __int_as_float(gl);
      gs[hh][lane] = lane < nt ? r.gv - gb : 0.0f;
      ds[hh][lane] = r.dv;
      ws[hh][lane] = r.dv * exp2_hw(__int_as_float(gl) - r.gv);
    }
    if ((st.t0 & (T - 1)) == 0) {
      const rsrc_t sres =
          make_rsrc(states + (hrow * nc + (st.t0 >> lgT)) * (kHeadDim * N), kStateBytes);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[nb]), sres,
                                               so_lane + 64 * nb, 0, 0);
    }
  };
  commit(ra);
  __syncthreads();

  // step k from the registers r (staged already); rn holds step k + 1
  auto body = [&](Regs& r, const Regs& rn, bool has_next) {
    const StepP st = r.st;
    const int h = st.h0 + hq;
    const int t0 = st.t0;
    const int nt = min(TB, L - t0);
    const size_t hrow = (size_t)st.b * H + h;
    const float Dh[2] = {dcur[0], dcur[1]};
    Src nxt;
    prepare(cur.st, nxt);
    r.st = cur.st;
    advance(cur);
    // every operand of the step two ahead, in one burst
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, nxt, r);

    // ---- operands read ahead of their products: the first C B^T block's
    //      fragments and this head's x tile as X^T fragments (lane (p, lq)
    //      holds tokens 32 s + 16 (e / 4) + 4 lq + e % 4 of column p)
    auto cb_frags = [&](int sl, u32x4 (&bf)[KN], u32x4 (&cf)[KN]) {
      const int ib = blk_i(sl), jb = blk_j(sl);
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        bf[kk] = *(const u32x4*)(bq + (16 * jb + lr) * CS + 32 * kk + 8 * lq);
        cf[kk] = *(const u32x4*)(cp + (16 * ib + lr) * CS + 32 * kk + 8 * lq);
      }
    };
    u32x4 cbb[KN], cbc[KN];
    cb_frags(0, cbb, cbc);
    u32x4 xa[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int xo = (32 * s + 4 * lq + (lr >> 2)) * XS + 16 * w + 4 * (lr & 3);
      const u32x2 a0 = lds_read_tr16(xs[hq] + xo);
      const u32x2 a1 = lds_read_tr16(xs[hq] + xo + 16 * XS);
      xa[s] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) acc = mfma_bf16(cbb[kk], cbc[kk], acc);
      cbr[0] = acc;
    }
    if (ncb > 1) {
      cb_frags(1, cbb, cbc);
      __builtin_amdgcn_sched_barrier(0);
      f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) acc = mfma_bf16(cbb[kk], cbc[kk], acc);
      cbr[1] = acc;
    }
    // C fragments of the first k-step of C S^T, in flight while L' is formed
    auto c_frag = [&](int kk, int ib) {
      return *(const u32x4*)(cp + (16 * ib + lr) * CS + 32 * kk + 8 * lq);
    };
    u32x4 cfa[NIB], cfb[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) cfa[ib] = c_frag(0, ib);
    __builtin_amdgcn_sched_barrier(0);

    // ---- L' of both heads from this wave's blocks -> LDS
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl < ncb) {
        const int ib = blk_i(sl), jb = blk_j(sl);
        const int i = 16 * ib + lr, j0 = 16 * jb + 4 * lq;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const float gi = gs[hh][i];
          const f32x4 gj = *(const f32x4*)(&gs[hh][j0]);
          const f32x4 dj = *(const f32x4*)(&ds[hh][j0]);
          f32x4 v;
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int j = j0 + rr;
            float wv = cbr[sl][rr] * (exp2_hw(gi - gj[rr]) * dj[rr]);
            if (j == i) wv += Dh[hh];
            v[rr] = j <= i ? wv : 0.0f;
          }
          uint32_t h0, l0, h1, l1;
          split_bf16(v[0], v[1], h0, l0);
          split_bf16(v[2], v[3], h1, l1);
          const int o = i * LS + kpos(j0);
          *(u32x2*)(lp[hh][0] + o) = (u32x2){h0, h1};
          *(u32x2*)(lp[hh][1] + o) = (u32x2){l0, l1};
        }
      }
    }

    // ---- Y^T = S C^T, A = S from the accumulators (hi + lo), B = C rows;
    //      the next k-step's C fragments are read during this one's products
    f32x4 yacc[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) yacc[ib] = (f32x4){0, 0, 0, 0};
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
      u32x4(&cur)[NIB] = (kk & 1) ? cfb : cfa;
      u32x4(&nxt)[NIB] = (kk & 1) ? cfa : cfb;
      if (kk + 1 < KN) {
#pragma unroll
        for (int ib = 0; ib < NIB; ++ib) nxt[ib] = c_frag(kk + 1, ib);
      }
      u32x4 sh, sl;
      split8_2(sacc[2 * kk], sacc[2 * kk + 1], sh, sl);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        yacc[ib] = mfma_bf16(sh, cur[ib], yacc[ib]);
        yacc[ib] = mfma_bf16(sl, cur[ib], yacc[ib]);
      }
    }
    const float* gsh = gs[hq];
    const float* wsh = ws[hq];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) yacc[ib] *= exp2_hw(gsh[16 * ib + lr]);

    // ---- state: S <- 2^{g_last} S + B^T X', X' = w o x on this lane's tokens;
    //      each 32-token half's B^T fragments are read ahead of its products
    auto b_frag = [&](int s, int nb) {
      const int bo = (32 * s + 4 * lq + (lr >> 2)) * BS + 4 * (lr & 3) + 16 * nb;
      const u32x2 a0 = lds_read_tr16(bp + bo);
      const u32x2 a1 = lds_read_tr16(bp + bo + 16 * BS);
      return (u32x4){a0[0], a0[1], a1[0], a1[1]};
    };
    u32x4 bf0[N / 16], bf1[N / 16];
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) bf0[nb] = b_frag(0, nb);
    const float dec = exp2_hw(gsh[nt - 1]);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) sacc[nb] *= dec;
    auto wx_split = [&](int s, u32x4& xh, u32x4& xl) {
      const f32x4 w0 = *(const f32x4*)(&wsh[32 * s + 4 * lq]);
      const f32x4 w1 = *(const f32x4*)(&wsh[32 * s + 16 + 4 * lq]);
      const f32x4 x0 = {bf16_lo(xa[s][0]) * w0[0], bf16_hi(xa[s][0]) * w0[1],
                        bf16_lo(xa[s][1]) * w0[2], bf16_hi(xa[s][1]) * w0[3]};
      const f32x4 x1 = {bf16_lo(xa[s][2]) * w1[0], bf16_hi(xa[s][2]) * w1[1],
                        bf16_lo(xa[s][3]) * w1[2], bf16_hi(xa[s][3]) * w1[3]};
      split8_2(x0, x1, xh, xl);
    };
    {
      u32x4 xh, xl;
      wx_split(0, xh, xl);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        sacc[nb] = mfma_bf16(bf0[nb], xh, sacc[nb]);
        sacc[nb] = mfma_bf16(bf0[nb], xl, sacc[nb]);
        if (nb == 1) {
#pragma unroll
          for (int q = 0; q < N / 16; ++q) bf1[q] = b_frag(1, q);
        }
      }
    }
    {
      u32x4 xh, xl;
      wx_split(1, xh, xl);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        sacc[nb] = mfma_bf16(bf1[nb], xh, sacc[nb]);
        sacc[nb] = mfma_bf16(bf1[nb], xl, sacc[nb]);
      }
    }
    if (t0 + TB >= L && final_state) {
      const rsrc_t fres = make_rsrc(final_state + hrow * (kHeadDim * N), kStateBytes);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[nb]), fres,
                                               so_lane + 64 * nb, 0, 0);
    }
    __syncthreads();  // every wave's L' blocks are in LDS; x, B, C, g, dt reads are done

    // L' fragments of the first three row blocks, in flight during the staging
    uint16_t(*lph)[TB * LS] = lp[hq];
    auto l_frag = [&](int ib, int s, int q) {
      return *(const u32x4*)(lph[q] + (16 * ib + lr) * LS + 32 * s + 8 * lq);
    };
    u32x4 lf[4][2][2];   // [ib][s][hi, lo]
#pragma unroll
    for (int ib = 0; ib < 3; ++ib) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (2 * s <= ib) {
          lf[ib][s][0] = l_frag(ib, s, 0);
          lf[ib][s][1] = l_frag(ib, s, 1);
        }
      }
    }

    // the next step's operands, while the other waves multiply by L'
    if (has_next) commit(rn);
    __builtin_amdgcn_sched_barrier(0);

    // ---- Y^T += X^T L'^T over the 32-token k-steps on or below the
    //      diagonal, into the block's Y tile in LDS (token rows, both heads'
    //      columns side by side)
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
      if (ib == 1) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          lf[3][s][0] = l_frag(3, s, 0);
          lf[3][s][1] = l_frag(3, s, 1);
        }
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (2 * s <= ib) {
          yacc[ib] = mfma_bf16(xa[s], lf[ib][s][0], yacc[ib]);
          yacc[ib] = mfma_bf16(xa[s], lf[ib][s][1], yacc[ib]);
        }
      }
      *(f32x4*)(ys + (16 * ib + lr) * YS + hq * kHeadDim + p - lr + 4 * lq) = yacc[ib];
    }
    __syncthreads();  // the next step's operands and the Y tile are staged; L' reads are done

    // ---- the Y tile to y in whole rows: the pair's two head rows of a
    //      token are one 512-byte run (256 with bf16 y), so a wave writes two
    //      such runs per instruction; rows past the end of the sequence fall
    //      outside the range.  (The tile is rewritten only after the next
    //      step's first barrier, which every wave reaches after these reads.)
    //      The stores are nontemporal: y is written once and not read back.
    const rsrc_t yres =
        make_rsrc((char*)y + (((size_t)st.b * L + t0) * H + st.h0) * kHeadDim * kYB,
                  ((uint32_t)(L - t0) * H - st.h0) * kHeadDim * kYB);
#pragma unroll
    for (int j = 0; j < TB * 2 * kHeadDim / 4 / NT; ++j) {
      const int c = tid + NT * j, i = c >> 5, c4 = c & 31;
      const f32x4 v = *(const f32x4*)(ys + i * YS + 4 * c4);
      const uint32_t yo = ((uint32_t)i * H * kHeadDim + 4 * c4) * kYB;
      if constexpr (YBF16) {
        __builtin_amdgcn_raw_buffer_store_b64(
            (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])}, yres, yo, 0, kNontemporal);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), yres, yo, 0,
                                               kNontemporal);
      }
    }
  };

  for (int k = 0; k < nsteps; k += 2) {
    body(ra, rb, k + 1 < nsteps);
    if (k + 1 < nsteps) body(rb, ra, k + 2 < nsteps);
  }
}

// Runs per chain for the shape: R = the chunk steps per CU if every chain's
// walk were spread evenly over the CUs; a lead run of R0 = nc - (nr - 1) R
// chunks (1 <= R0 <= R) and nr - 1 runs of R.  nr = 1 when there are enough
// (b, head pair) chains for the CUs.
struct RunPlan {
  int nr, R, R0;
};

RunPlan plan_runs(const Shape& s, int cus) {
  const int nc = (int)s.nchunks();
  const int64_t pairs = s.batch * s.nheads / 2;
  const int64_t per = (pairs * nc + cus - 1) / cus;
  if (per >= nc) return RunPlan{1, nc, nc};
  const int R = (int)per;
  const int nr = 1 + (nc - 1) / R;
  return RunPlan{nr, R, nc - (nr - 1) * R};
}

template <bool YBF16>
int launch_pair_bf16(const void* x, const void* B, const void* C, const float* dt_t,
                     const float* g, const float* D, const float* init, float* states,
                     float* fin, void* y, const Shape& s, const RunPlan& pl, hipStream_t st) {
  static PerDeviceInt resident;
  const int slots = resident.get([&](int dev) {
    return resident_slots((const void*)fused_pair_bf16<YBF16>, 512, dev);
  });
  if (slots <= 0) return (int)hipErrorInvalidDevice;
  const int chains = (int)(s.batch * (s.nheads / 2));
  const int items = chains * pl.nr;
  const int grid = items < slots ? items : slots;
  // lead runs per spare workgroup (0: a stride of the grid over all items)
  const int n_long = chains * (pl.nr - 1), spare = grid - n_long;
  const int ks = pl.nr > 1 && spare > 0 ? (chains + spare - 1) / spare : 0;
  hipLaunchKernelGGL((fused_pair_bf16<YBF16>), dim3((unsigned)grid), dim3(512), 0, st,
                     (const uint16_t*)x, (const uint16_t*)B, (const uint16_t*)C, dt_t, g, D,
                     init, states, fin, y, (int)s.seqlen, (int)s.nheads, (int)s.ngroups,
                     (int)s.chunk, (int)s.nchunks(), pl.R, pl.R0, pl.nr, chains, ks);
  return (int)hipGetLastError();
}

}  // namespace

bool fused_bf16_applies(const Shape& s, bool bf16_in) {
  return bf16_in && s.dstate == kN && s.headdim == kHeadDim &&
         (s.chunk == 64 || s.chunk == 128 || s.chunk == 256) &&
         (s.nheads / s.ngroups) % 2 == 0;
}

int launch_fused_bf16(const void* x, const void* B, const void* C, const float* dt_t,
                      const float* g, const float* D, const float* init, float* states,
                      float* fin, void* y, bool bf16_out, const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  static PerDeviceInt cus_cache;
  int cus = cus_cache.get(query_cus);
  if (cus <= 0) cus = 256;
  const RunPlan pl = plan_runs(s, cus);
  if (pl.nr > 1) {
    const int nc = (int)s.nchunks();
    // head pairs sharing each staged B tile (8 waves, one workgroup per CU):
    // with the read-ahead fused kernel, 2-4% faster than one head per
    // workgroup at two workgroups per CU (interleaved same-box timings)
    const int nsub = pl.nr - 1;   // the runs before the last
    const unsigned g1 = (unsigned)(s.batch * (s.nheads / 2) * nsub);
    hipLaunchKernelGGL((run_state_bf16<kN, 2>), dim3(g1), dim3(512), 0, st, (const uint16_t*)x,
                       (const uint16_t*)B, dt_t, g, states, (int)s.seqlen, (int)s.nheads,
                       (int)s.ngroups, (int)s.chunk, nc, pl.R, pl.R0, nsub);
    int err = (int)hipGetLastError();
    if (err) return err;
    const unsigned g2 = (unsigned)(s.batch * s.nheads * (kHeadDim * kN / 4 / 256));
    hipLaunchKernelGGL((run_passing_kernel<kN>), dim3(g2), dim3(256), 0, st, g, init, states,
                       (int)s.seqlen, (int)s.chunk, nc, pl.R, pl.R0, nsub);
    err = (int)hipGetLastError();
    if (err) return err;
  }
  if (bf16_out) return launch_pair_bf16<true>(x, B, C, dt_t, g, D, init, states, fin, y, s, pl, st);
  return launch_pair_bf16<false>(x, B, C, dt_t, g, D, init, states, fin, y, s, pl, st);
}

}  // namespace ssd

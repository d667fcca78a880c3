// Stage 2, the inter-chunk state pass, for fp32 inputs with many (batch,
// head pair) chains: both heads of a pair per workgroup, sharing each staged
// B tile.
//
// For every (b, h): S = init (or 0); for chunk c = 0, 1, ...:
//   states[b,h,c] = S
//   S = 2^{g_last} S + sum_t 2^{g_last - g_t} dt_t x_t B_t^T
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", sections "Step 1: Jump the State Across a Chunk with One Matmul"
// and "Kernel 2: fwd_pass_state": the state is stored before each chunk's
// update, and the sequential dependence stays inside one program.)
//
// MI355X design.  The fp32-instruction kernel (state_pass_f32) gives every
// (b, h) its own workgroup, so B -- shared by the heads of a group -- is
// fetched and staged once per head, and its fp32 16x16x4 matrix instructions
// take 2.7 times the matrix time of bf16 ones for the same product.  Here:
// * Work items are (b, pair of adjacent heads of one group); persistent
//   workgroups take them with a stride of the grid, so the workgroups of an
//   XCD walk consecutive pairs of a group at once and share B in its L2.
// * 8 waves: waves 4q..4q+3 on head q of the pair, wave 4q + w owning state
//   rows p = 16w..16w+15 and all 64 columns, transposed in the accumulators
//   (lane (p, lq) of block nb holds S[p][16 nb + 4 lq + 0..3]).  State
//   stores pass through the wave's own rows of an x^T buffer it is done
//   with, so each store instruction writes four whole 256-byte rows instead
//   of 16 rows x 64 bytes (2% faster).
// * The chunk's B tile is staged once for both heads, split exactly into
//   three bf16 planes (v = hi + mid + lo); the update reads its transpose
//   with the LDS transpose read.  The decay weight w_t = dt_t 2^{g_last - g_t}
//   multiplies x instead of B, so B stays shared.  x is read in whole lines
//   (32 lanes take a token's 512 bytes for both heads), staged transposed
//   ([p][t], fp32) through the 4 x 4 register transpose that each thread's
//   four tokens give, and each lane reads its 8 tokens of column p as two
//   16-byte LDS reads, scales them by w_t and splits them like B.  (Loading
//   each lane's own (token, p) values from memory instead takes twice the
//   read requests, 64-byte pieces of each row, and was 7% slower.)  Six bf16
//   products per pair of split operands keep every term of relative size
//   2^-16 or more: fp32 accuracy.
// * Every operand of a step is loaded two steps ahead into one of two
//   register sets; B planes, x^T and the weights are double-buffered in LDS
//   (129 KB, one workgroup per CU), so one barrier per step suffices.
// * Chunks of 64 tokens only (one step per chunk); the ranges of the buffer
//   descriptors end at the sequence, so rows past it read zero (x = B = 0,
//   g = dt = 0, w = 0) and a ragged last chunk needs no special case.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// the six products of a split pair: acc += a * b to fp32 accuracy
__device__ __forceinline__ f32x4 mfma_split6(const u32x4 (&a)[3], const u32x4 (&b)[3],
                                             f32x4 acc) {
  acc = mfma_bf16(a[0], b[0], acc);
  acc = mfma_bf16(a[0], b[1], acc);
  acc = mfma_bf16(a[1], b[0], acc);
  acc = mfma_bf16(a[0], b[2], acc);
  acc = mfma_bf16(a[1], b[1], acc);
  acc = mfma_bf16(a[2], b[0], acc);
  return acc;
}

// eight fp32 values split exactly into three bf16 fragments
__device__ __forceinline__ void split8_3(const f32x4& v0, const f32x4& v1, u32x4 (&f)[3]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t h, m, l;
    split3_bf16(v0[2 * q], v0[2 * q + 1], h, m, l);
    f[0][q] = h; f[1][q] = m; f[2][q] = l;
    split3_bf16(v1[2 * q], v1[2 * q + 1], h, m, l);
    f[0][2 + q] = h; f[1][2 + q] = m; f[2][2 + q] = l;
  }
}

__global__ __launch_bounds__(512) void state_pair_f32(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ init, float* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int G, int nc, int pairs) {
  constexpr int NT = 512;
  constexpr int T = 64, N = 64;
  constexpr int BS = 80;                 // B plane row stride (bf16): 160 bytes
  constexpr int XT = T + 4;              // x^T row stride (fp32)
  constexpr int BU = T * 16 / NT;        // 16-byte units of the B tile per thread
  constexpr uint32_t kStateBytes = kHeadDim * N * 4;
  __shared__ __attribute__((aligned(16))) uint16_t bp[2][3][T * BS];
  __shared__ __attribute__((aligned(16))) float xt[2][2][kHeadDim * XT];   // [buffer][head] x^T
  __shared__ __attribute__((aligned(16))) float ws[2][2][T];   // [buffer][head] w_t
  __shared__ float gls[2][2];                                   // [buffer][head] g_last

  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  if (wg >= pairs) return;
  const int mine = (pairs - 1 - wg) / nwg + 1;
  const int nsteps = mine * nc;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = wave >> 2, w = wave & 3;     // head of the pair, row block
  const int lr = lane & 15, lq = lane >> 4;
  const int hpg = H / G, npr = H / 2;
  const uint32_t xrow = (uint32_t)H * kHeadDim * 4;   // bytes per token of x
  const uint32_t brow = (uint32_t)G * N * 4;          // bytes per token of B
  const int p = 16 * w + lr;                  // this lane's state row
  const bool gwave = w == 0;   // the first wave of each head loads its g and dt

  // x unit of this thread: tokens 4 tq + 0..3, 16-byte piece `xpc` of the
  // pair's two adjacent 256-byte head rows (head xpc / 16, columns
  // 4 (xpc % 16) + 0..3): each token's 512 bytes are read by 32 lanes in one
  // instruction, whole lines
  const int tq = tid >> 5, xpc = tid & 31;
  const uint32_t xo_lane = (uint32_t)(4 * tq) * xrow + 16 * (uint32_t)xpc;
  uint32_t bo_lane[BU];
#pragma unroll
  for (int u = 0; u < BU; ++u) {
    const int e = tid + NT * u;
    bo_lane[u] = (uint32_t)(e >> 4) * brow + 16 * (e & 15);
  }
  const uint32_t gd_lane = 4 * (uint32_t)lane;
  const uint32_t so_lane = ((uint32_t)p * N + 4 * lq) * 4;

  // Work steps are (pair, chunk), chunks fastest; a cursor walks them in
  // order, dividing only when it moves to the next pair.
  struct StepP {
    int b, c, h0, grp;
    bool live;
  };
  struct Cursor {
    int k, c, it;
    StepP st;
  };
  auto at_pair = [&](Cursor& cu) {
    cu.st.b = cu.it / npr;
    cu.st.h0 = (cu.it - cu.st.b * npr) * 2;
    cu.st.grp = cu.st.h0 / hpg;
  };
  auto advance = [&](Cursor& cu) {
    ++cu.k;
    if (++cu.c == nc) {
      cu.c = 0;
      cu.it += nwg;
      if (cu.k < nsteps) at_pair(cu);
    }
    cu.st.c = cu.c;
    cu.st.live = cu.k < nsteps;
  };

  struct Regs {
    f32x4 xq[4];    // x of tokens 4 tq + r, the unit's four columns
    f32x4 bt[BU];
    float gv, dv;   // g and dt (the first wave of each head), lane = token
    StepP st;       // the step these registers were loaded for
  };
  // Every load of step st into r, in one burst.
  auto issue = [&](const StepP& st, Regs& r) {
    const int t0 = st.c * T;
    const uint32_t rows = (uint32_t)(L - t0);
    const rsrc_t xr = make_rsrc(x + (((size_t)st.b * L + t0) * H + st.h0) * kHeadDim,
                                st.live ? (rows * H - st.h0) * (kHeadDim * 4) : 0u);
    const rsrc_t br = make_rsrc(Bm + (((size_t)st.b * L + t0) * G + st.grp) * N,
                                st.live ? (rows * G - st.grp) * (N * 4) : 0u);
    const size_t gro = ((size_t)st.b * H + st.h0 + hq) * L + t0;
    const uint32_t grr = st.live && gwave ? rows * 4 : 0u;
    const rsrc_t gr = make_rsrc(g + gro, grr), dr = make_rsrc(dt_t + gro, grr);
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) r.xq[r4] = load_f32x4(xr, xo_lane + (uint32_t)r4 * xrow);
#pragma unroll
    for (int u = 0; u < BU; ++u) r.bt[u] = load_f32x4(br, bo_lane[u]);
    r.gv = load_f32(gr, gd_lane);
    r.dv = load_f32(dr, gd_lane);
    r.st = st;
  };

  f32x4 sacc[N / 16];   // S[p][16 nb + 4 lq + rr] of this wave's head

  Regs ra, rb;
  Cursor cur;
  cur.k = 0;
  cur.c = 0;
  cur.it = wg;
  at_pair(cur);
  cur.st.c = 0;
  cur.st.live = true;
  issue(cur.st, ra);
  advance(cur);
  issue(cur.st, rb);
  advance(cur);

  // Staging of a step into LDS buffer `buf`: B as three exact bf16 planes
  // (row = token, natural column order, for the transposed reads), x of both
  // heads transposed ([p][t], fp32, through the 4 x 4 register transpose the
  // unit's four tokens give), and the weights w_t and g_last of both heads.
  auto stage = [&](const Regs& r, int buf) {
    const StepP st = r.st;
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int e = tid + NT * u, row = e >> 4, c4 = e & 15;
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(r.bt[u][0], r.bt[u][1], h0, m0, l0);
      split3_bf16(r.bt[u][2], r.bt[u][3], h1, m1, l1);
      const int ob = row * BS + 4 * c4;
      *(u32x2*)(bp[buf][0] + ob) = (u32x2){h0, h1};
      *(u32x2*)(bp[buf][1] + ob) = (u32x2){m0, m1};
      *(u32x2*)(bp[buf][2] + ob) = (u32x2){l0, l1};
    }
    {
      float* xh = xt[buf][xpc >> 4] + 4 * (xpc & 15) * XT + 4 * tq;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(xh + e * XT) = (f32x4){r.xq[0][e], r.xq[1][e], r.xq[2][e], r.xq[3][e]};
    }
    if (gwave) {
      // lane = token; tokens past the end read g = dt = 0, so w = 0
      const int nt = min(T, L - st.c * T);
      const int gl = __builtin_amdgcn_readlane(__float_as_int(r.gv), nt - 1);
      ws[buf][hq][lane] = r.dv * exp2_hw(__int_as_float(gl) - r.gv);
      if (lane == 0) gls[buf][hq] = __int_as_float(gl);
    }
  };
  // The state entering a step's chunk: init_state (or zero) at a pair's
  // first chunk, else the accumulators as the previous step left them;
  // stored to states.  The store goes through this wave's own 16 rows of
  // x^T buffer fb (no other wave reads them, and the wave is done with
  // them): each lane writes its accumulator blocks there, then reads back
  // 16-byte pieces of whole 256-byte state rows, so each store instruction
  // writes four consecutive rows, 1 KB of consecutive bytes, rather than
  // 16 rows x 64 bytes.
  auto enter = [&](const StepP& st, int fb) {
    const size_t hrow = (size_t)st.b * H + st.h0 + hq;
    if (st.c == 0) {
      // no initial state: an empty range, every load reads zero
      const rsrc_t ires = init ? make_rsrc(init + hrow * (kHeadDim * N), kStateBytes)
                               : make_rsrc(states, 0u);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) sacc[nb] = load_f32x4(ires, so_lane + 64 * nb);
    }
    float* reg = xt[fb][hq] + 16 * w * XT;
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) *(f32x4*)(reg + lr * XT + 16 * nb + 4 * lq) = sacc[nb];
    __builtin_amdgcn_wave_barrier();
    const rsrc_t sres = make_rsrc(states + (hrow * nc + st.c) * (kHeadDim * N), kStateBytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i + (lane >> 4), c = lane & 15;
      const f32x4 v = *(const f32x4*)(reg + r * XT + 4 * c);
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), sres,
                                             (uint32_t)((16 * w + r) * N + 4 * c) * 4, 0, 0);
    }
  };

  stage(ra, 0);
  enter(ra.st, 1);
  __syncthreads();

  // step k (staged in buffer buf); r held it and is reloaded with step
  // k + 2 once rn (step k + 1) is staged into the other buffer
  auto body = [&](Regs& r, const Regs& rn, bool has_next, int buf) {
    const StepP st = r.st;
    if (has_next) stage(rn, buf ^ 1);
    issue(cur.st, r);
    advance(cur);

    // ---- S <- 2^{g_last} S + B^T X', X' = w o x on this lane's tokens
    //      (k slot e of step s: token 32 s + 16 (e / 4) + 4 lq + e % 4)
    auto b_frags = [&](int s, int nb, u32x4 (&bt)[3]) {
      const int bo = (32 * s + 4 * lq + (lr >> 2)) * BS + 4 * (lr & 3) + 16 * nb;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const u32x2 a0 = lds_read_tr16(bp[buf][q] + bo);
        const u32x2 a1 = lds_read_tr16(bp[buf][q] + bo + 16 * BS);
        bt[q] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
      }
    };
    u32x4 btr[2][3];
    b_frags(0, 0, btr[0]);
    const float* wsh = ws[buf][hq];
    const float* xh = xt[buf][hq] + p * XT;
    const float dec = exp2_hw(gls[buf][hq]);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) sacc[nb] *= dec;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 w0 = *(const f32x4*)(&wsh[32 * s + 4 * lq]);
      const f32x4 w1 = *(const f32x4*)(&wsh[32 * s + 16 + 4 * lq]);
      const f32x4 x0 = *(const f32x4*)(xh + 32 * s + 4 * lq) * w0;
      const f32x4 x1 = *(const f32x4*)(xh + 32 * s + 16 + 4 * lq) * w1;
      u32x4 xp[3];
      split8_3(x0, x1, xp);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        const int gi = s * (N / 16) + nb;
        if (gi + 1 < 2 * (N / 16)) b_frags((gi + 1) / (N / 16), (gi + 1) % (N / 16), btr[(gi + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        sacc[nb] = mfma_split6(btr[gi & 1], xp, sacc[nb]);
      }
    }
    if (st.c == nc - 1 && final_state) {
      const size_t hrow = (size_t)st.b * H + st.h0 + hq;
      const rsrc_t fres = make_rsrc(final_state + hrow * (kHeadDim * N), kStateBytes);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[nb]), fres,
                                               so_lane + 64 * nb, 0, 0);
    }
    // the state entering the next step's chunk
    if (has_next) enter(rn.st, buf);
    __syncthreads();  // buffer buf ^ 1 is staged; buffer buf's reads are done
  };

  for (int k = 0; k < nsteps; k += 2) {
    body(ra, rb, k + 1 < nsteps, 0);
    if (k + 1 < nsteps) body(rb, ra, k + 2 < nsteps, 1);
  }
}

}  // namespace

// Whether the head-pair kernel takes this shape: fp32 inputs, 64-token
// chunks, N = 64, an even group size, and at least one (b, head pair) per
// compute unit.
bool state_pair_f32_applies(const Shape& s, bool bf16_in) {
  if (bf16_in || s.chunk != 64 || s.dstate != 64 || s.headdim != kHeadDim) return false;
  if ((s.nheads / s.ngroups) % 2 != 0) return false;
  static PerDeviceInt cus_cache;
  int cus = cus_cache.get(query_cus);
  if (cus <= 0) cus = 256;
  return s.batch * s.nheads / 2 >= cus;
}

int launch_state_pair_f32(const float* x, const float* B, const float* dt_t, const float* g,
                          const float* init, float* states, float* fin, const Shape& s,
                          void* stream) {
  static PerDeviceInt resident;
  const int slots = resident.get(
      [&](int dev) { return resident_slots((const void*)state_pair_f32, 512, dev); });
  if (slots <= 0) return (int)hipErrorInvalidDevice;
  const int pairs = (int)(s.batch * s.nheads / 2);
  const unsigned grid = (unsigned)(pairs < slots ? pairs : slots);
  hipLaunchKernelGGL(state_pair_f32, dim3(grid), dim3(512), 0, (hipStream_t)stream, x, B, dt_t,
                     g, init, states, fin, (int)s.seqlen, (int)s.nheads, (int)s.ngroups,
                     (int)s.nchunks(), pairs);
  return (int)hipGetLastError();
}

}  // namespace ssd

// The two-level form of stage 2: per-chunk local states computed for every
// chunk in parallel, then a short sequential pass that carries the state
// across chunks element by element.
//
// With P_c = X_c^T (w o B_c), w_t = dt_t 2^{g_last(c) - g_t}, the chunk's
// contribution from a zero state, the jump of stage 2 is
//   S_{c+1} = 2^{g_last(c)} S_c + P_c
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", "Step 1: Jump the State Across a Chunk with One Matmul" and
// "Kernel 2: fwd_pass_state").  Chunk-state computes every P_c at once (no
// chain), writing P_c into the slot of the state it feeds, states[c+1] (the
// last one into final); state-passing then turns those slots into the states
// in place: states[0] = init, states[c] = 2^{g_last(c-1)} states[c-1] +
// states[c], final = 2^{g_last(nc-1)} states[nc-1] + final.
//
// MI355X design.
// * chunk_state: one workgroup per (b, chunk, block of HB heads of one
//   group), four waves per head; wave (hh, w) owns rows 16w..16w+15 of head
//   hh and all N columns (N/16 accumulator blocks of P^T[n][p], lane: column
//   p, four consecutive n, so stores are 16 bytes).  The HB heads share one
//   staged B tile.
//   The chunk is consumed in sub-tiles (64 tokens, 32 with several heads, so
//   the LDS stays near 46 KB for two heads): x (as w o x, split bf16 hi +
//   lo) and B staged in LDS, operands read with the LDS transpose read, the
//   same k-slot map as the fused pass.  No state is carried, so every
//   (b, chunk, head) is independent and the grid has b * nc * H / HB
//   workgroups.
// * state_passing: a pure element-wise stream.  A thread owns one 16-byte
//   unit (four consecutive n of one row p) of one (b, h) and walks the
//   chunks in blocks of D.  The loads do not depend on the carried value,
//   so the next block's loads are in flight while a block is combined.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr uint32_t kPastRange = 0x7FFFFFF0u;

// Consecutive logical items on one XCD (blocks are dealt round-robin).
__device__ __forceinline__ int xcd_item(int bid, int total) {
  if (total % 8) return bid;
  return (bid % 8) * (total / 8) + bid / 8;
}

template <int N>
struct TlStride {
  static constexpr int value = N + 16;
};

template <int T, int N, int HB>
__global__ __launch_bounds__(256 * HB) void chunk_state_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const float* __restrict__ dt_t, const float* __restrict__ g, float* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int G, int nc, int park) {
  constexpr int ST = HB == 1 ? 64 : 32;        // tokens per sub-tile
  constexpr int NSUB = T / ST;
  constexpr int XS = kHeadDim + 16;            // w o x row stride (bf16)
  constexpr int BS = TlStride<N>::value;       // B row stride (bf16)
  constexpr int NB = N / 16;                   // accumulator blocks per wave
  constexpr int NTHR = 256 * HB;
  constexpr int XU = HB * ST * kHeadDim / 8 / NTHR;  // 16-byte x units per thread
  constexpr int BUN = ST * N / 8;                     // 16-byte B units per sub-tile
  constexpr int BU = (BUN + NTHR - 1) / NTHR;         // ... per thread (the last partial)
  static_assert(XU * NTHR == HB * ST * kHeadDim / 8, "x units");
  __shared__ __attribute__((aligned(16))) uint16_t whs[HB * ST * XS];
  __shared__ __attribute__((aligned(16))) uint16_t wls[HB * ST * XS];
  __shared__ __attribute__((aligned(16))) uint16_t bts[ST * BS];

  // blocks: (b, c, block of HB heads of one group) with the head block
  // fastest; the HB heads share the staged B tile.  Consecutive items are
  // remapped onto one XCD (blocks are dealt to the 8 XCDs round-robin), so
  // the head blocks of a chunk read its B rows through one L2.
  const int nhb = H / HB;
  const int item = xcd_item(blockIdx.x, gridDim.x);
  const int h0 = (item % nhb) * HB;
  const int c = (item / nhb) % nc;
  const int b = item / (nhb * nc);
  const int grp = h0 / (H / G);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int hh = wave >> 2, wr = wave & 3;      // this wave's head and 16-row slice
  const int h = h0 + hh;

  const uint32_t xrow = (uint32_t)(H * kHeadDim), brow = (uint32_t)(G * N);
  const rsrc_t xr = make_rsrc(x + ((size_t)b * L * H + h0) * kHeadDim,
                              ((uint32_t)(L - 1) * xrow + (uint32_t)HB * kHeadDim) * 2u);
  const rsrc_t br = make_rsrc(Bm + ((size_t)b * L * G + grp) * N,
                              ((uint32_t)(L - 1) * brow + N) * 2u);
  // g and dt_t rows of the HB heads, [hh][L]
  const size_t grow = ((size_t)b * H + h0) * L;
  const rsrc_t gr = make_rsrc(g + grow, (uint32_t)(HB * L) * 4u);
  const rsrc_t dr = make_rsrc(dt_t + grow, (uint32_t)(HB * L) * 4u);
  const int tlast = min(c * T + T, L) - 1;

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0, 0, 0, 0};

  // transpose-read offsets: rows t = 4 lq + (lr >> 2) (+32 kk, +16), column
  // c0 + 4 (lr & 3)
  const int rsel = 4 * lq + (lr >> 2), csel = 4 * (lr & 3);
  // Loads of a sub-tile (x units: head, token, 8 p; B units: token, 8 n)
  // land in registers; the next sub-tile's are issued before the current
  // one is consumed from LDS.  Each x unit carries its head's g_last.
  u32x4 xv[XU], bv[BU];
  float gv[XU], dv[XU], glv[XU];
#pragma unroll
  for (int i = 0; i < XU; ++i) {
    const int uh = (tid + NTHR * i) / (ST * 8);
    glv[i] = g[grow + (size_t)uh * L + tlast];
  }
  auto issue = [&](int sub) {
    const uint32_t t0 = (uint32_t)(c * T + sub * ST);
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + NTHR * i, uh = u / (ST * 8), t = (u >> 3) % ST, c8 = u & 7;
      xv[i] = load_b128(xr, ((t0 + t) * xrow + uh * kHeadDim + 8 * c8) * 2u);
      const uint32_t go = t0 + t < (uint32_t)L ? ((uint32_t)uh * L + t0 + t) * 4u : kPastRange;
      gv[i] = load_f32(gr, go);
      dv[i] = load_f32(dr, go);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
      const int u = tid + NTHR * i, t = u / (N / 8), c8 = u % (N / 8);
      if (BUN % NTHR == 0 || u < BUN) bv[i] = load_b128(br, ((t0 + t) * brow + 8 * c8) * 2u);
    }
  };
  issue(0);
#pragma unroll 1
  for (int sub = 0; sub < NSUB; ++sub) {
    if (sub > 0) __syncthreads();  // the previous sub-tile's reads are done
#pragma unroll
    for (int i = 0; i < XU; ++i) {
      const int u = tid + NTHR * i, uh = u / (ST * 8), t = (u >> 3) % ST, c8 = u & 7;
      // tokens past the end read dt = g = 0 and x = 0, so w o x = 0
      const float w = dv[i] * exp2_hw(glv[i] - gv[i]);
      uint32_t hv[4], lv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        split_bf16(bf16_lo(xv[i][e]) * w, bf16_hi(xv[i][e]) * w, hv[e], lv[e]);
      *(u32x4*)(whs + (uh * ST + t) * XS + 8 * c8) = make_u32x4(hv);
      *(u32x4*)(wls + (uh * ST + t) * XS + 8 * c8) = make_u32x4(lv);
    }
#pragma unroll
    for (int i = 0; i < BU; ++i) {
      const int u = tid + NTHR * i, t = u / (N / 8), c8 = u % (N / 8);
      if (BUN % NTHR == 0 || u < BUN) *(u32x4*)(bts + t * BS + 8 * c8) = bv[i];
    }
    if (sub + 1 < NSUB) issue(sub + 1);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < ST / 32; ++kk) {
      const int wo = (hh * ST + 32 * kk + rsel) * XS + 16 * wr + csel;
      const u32x2 a0 = lds_read_tr16(whs + wo), a1 = lds_read_tr16(whs + wo + 16 * XS);
      const u32x2 c0 = lds_read_tr16(wls + wo), c1 = lds_read_tr16(wls + wo + 16 * XS);
      const u32x4 wxh = {a0[0], a0[1], a1[0], a1[1]};
      const u32x4 wxl = {c0[0], c0[1], c1[0], c1[1]};
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int bo = (32 * kk + rsel) * BS + 16 * j + csel;
        const u32x2 e0 = lds_read_tr16(bts + bo), e1 = lds_read_tr16(bts + bo + 16 * BS);
        const u32x4 bb = {e0[0], e0[1], e1[0], e1[1]};
        acc[j] = mfma_bf16(bb, wxh, acc[j]);
        acc[j] = mfma_bf16(bb, wxl, acc[j]);
      }
    }
  }

  // P_c into the slot of the state it feeds: states[c + 1], or final (or,
  // with `park`, the not yet written states[0]).
  float* dst = nullptr;
  if (c + 1 < nc) {
    dst = states + (((size_t)b * H + h) * nc + c + 1) * kHeadDim * N;
  } else if (final_state) {
    dst = park ? states + ((size_t)b * H + h) * nc * kHeadDim * N
               : final_state + ((size_t)b * H + h) * kHeadDim * N;
  }
  if (dst) {
    const int p = 16 * wr + lr;
#pragma unroll
    for (int j = 0; j < NB; ++j) *(f32x4*)(dst + (size_t)p * N + 16 * j + 4 * lq) = acc[j];
  }
}

// fp32 inputs: one workgroup (4 waves) per (b, chunk, head), wave w owning
// rows 16w..16w+15 and all N columns as in the bf16 kernel.  The fp32 matrix
// instruction takes one k value per lane, so both operands are loaded
// straight from memory into their lanes (no staging): lane (lr, lq) of a
// 4-token step holds B[t][16j + lr] and (w o x)[t][16w + lr] for token
// t = t0 + lq.  Four steps (16 tokens) of loads are issued before their
// products.
template <int T, int N>
__global__ __launch_bounds__(256) void chunk_state_f32(
    const float* __restrict__ x, const float* __restrict__ Bm,
    const float* __restrict__ dt_t, const float* __restrict__ g, float* __restrict__ states,
    float* __restrict__ final_state, int L, int H, int G, int nc, int park) {
  constexpr int NB = N / 16;
  const int item = xcd_item(blockIdx.x, gridDim.x);   // as in the bf16 kernel
  const int h = item % H;
  const int c = (item / H) % nc;
  const int b = item / (H * nc);
  const int grp = h / (H / G);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lq = lane >> 4;

  const uint32_t xrow = (uint32_t)(H * kHeadDim), brow = (uint32_t)(G * N);
  const rsrc_t xr = make_rsrc(x + ((size_t)b * L * H + h) * kHeadDim,
                              ((uint32_t)(L - 1) * xrow + kHeadDim) * 4u);
  const rsrc_t br = make_rsrc(Bm + ((size_t)b * L * G + grp) * N,
                              ((uint32_t)(L - 1) * brow + N) * 4u);
  const size_t grow = ((size_t)b * H + h) * L;
  const rsrc_t gr = make_rsrc(g + grow, (uint32_t)L * 4u);
  const rsrc_t dr = make_rsrc(dt_t + grow, (uint32_t)L * 4u);
  const int tlast = min(c * T + T, L) - 1;
  const float gl = g[grow + tlast];

  f32x4 acc[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) acc[j] = (f32x4){0, 0, 0, 0};
#pragma unroll 1
  for (int s0 = 0; s0 < T; s0 += 16) {
    float wx[4], bv[4][NB];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t t = (uint32_t)(c * T + s0 + 4 * u + lq);
      // tokens past the end read dt = g = 0 and x = B = 0, so w o x = 0
      const uint32_t go = t < (uint32_t)L ? t * 4u : kPastRange;
      const float gv = load_f32(gr, go), dv = load_f32(dr, go);
      const float xv = load_f32(xr, (t * xrow + 16 * wave + lr) * 4u);
      wx[u] = dv * exp2_hw(gl - gv) * xv;
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[u][j] = load_f32(br, (t * brow + 16 * j + lr) * 4u);
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[j] = mfma_f32(bv[u][j], wx[u], acc[j]);
  }

  float* dst = nullptr;
  if (c + 1 < nc) {
    dst = states + (((size_t)b * H + h) * nc + c + 1) * kHeadDim * N;
  } else if (final_state) {
    dst = park ? states + ((size_t)b * H + h) * nc * kHeadDim * N
               : final_state + ((size_t)b * H + h) * kHeadDim * N;
  }
  if (dst) {
    const int p = 16 * wave + lr;
#pragma unroll
    for (int j = 0; j < NB; ++j) *(f32x4*)(dst + (size_t)p * N + 16 * j + 4 * lq) = acc[j];
  }
}

// ---------------------------------------------------------------- passing
template <int N, int D>
__global__ __launch_bounds__(256) void state_passing_kernel(
    const float* __restrict__ g, const float* __restrict__ init, float* __restrict__ states,
    float* __restrict__ final_state, int L, int T, int nc, int parked) {
  constexpr int UNITS = kHeadDim * N / 4;      // 16-byte units per state
  constexpr int WPB = UNITS / 256;             // workgroups per (b, h)
  const int bh = blockIdx.x / WPB;
  const int u = (blockIdx.x % WPB) * 256 + threadIdx.x;
  const size_t sstride = (size_t)kHeadDim * N;
  float* st = states + (size_t)bh * nc * sstride + 4 * (size_t)u;
  const float* gh = g + (size_t)bh * L;

  f32x4 s = init ? *(const f32x4*)(init + bh * sstride + 4 * (size_t)u) : (f32x4){0, 0, 0, 0};
  // P_{nc-1}: in the final slot, or parked in states[0] (read before the
  // slot is overwritten; each unit is read and written by its own thread,
  // so init_state may then be the final_state buffer).
  f32x4 plast = (f32x4){0, 0, 0, 0};
  if (parked) plast = *(const f32x4*)st;
  *(f32x4*)st = s;
  // Chunks 1 .. nc-1 in blocks of D, software-pipelined over two register
  // blocks: the loads of block j+1 are issued before block j is combined.
  // Chunks past the end are clamped to the last one (a harmless re-read).
  auto load_block = [&](int c0, f32x4 (&v)[D], float (&dec)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = min(c0 + d, nc - 1);
      v[d] = *(const f32x4*)(st + (size_t)c * sstride);
      dec[d] = exp2_hw(gh[min(c * T, L) - 1]);   // g_last of chunk c - 1
    }
  };
  auto combine_block = [&](int c0, const f32x4 (&v)[D], const float (&dec)[D]) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int c = c0 + d;
      if (c < nc) {
        s = dec[d] * s + v[d];
        *(f32x4*)(st + (size_t)c * sstride) = s;
      }
    }
  };
  f32x4 va[D], vb[D];
  float da[D], db[D];
  if (nc > 1) load_block(1, va, da);
#pragma unroll 1
  for (int c0 = 1; c0 < nc; c0 += 2 * D) {
    if (c0 + D < nc) load_block(c0 + D, vb, db);
    combine_block(c0, va, da);
    if (c0 + 2 * D < nc) load_block(c0 + 2 * D, va, da);
    if (c0 + D < nc) combine_block(c0 + D, vb, db);
  }
  if (final_state) {
    float* f = final_state + bh * sstride + 4 * (size_t)u;
    const float dec = exp2_hw(gh[min(nc * T, L) - 1]);
    if (!parked) plast = *(const f32x4*)f;
    *(f32x4*)f = dec * s + plast;
  }
}

template <int T, int N, int HB>
int launch_cs_hb(const void* x, const void* B, const float* dt_t, const float* g,
                 float* states, float* fin, bool park, const Shape& s, hipStream_t st) {
  const int nc = (int)s.nchunks();
  const unsigned blocks = (unsigned)(s.batch * nc * (s.nheads / HB));
  hipLaunchKernelGGL((chunk_state_bf16<T, N, HB>), dim3(blocks), dim3(256 * HB), 0, st,
                     (const uint16_t*)x, (const uint16_t*)B, dt_t, g, states, fin,
                     (int)s.seqlen, (int)s.nheads, (int)s.ngroups, nc, (int)park);
  return (int)hipGetLastError();
}

// Heads per workgroup: two (sharing one staged B tile) when the heads of a
// group pair up and the grid keeps at least one workgroup per CU, else one.
// Measured on MI355X, two heads beat one and four at every layer shape
// (4 x 2048 tokens, 24 heads: 31.8 us against 33.9 and 34.1; 2 x 8192, 80
// heads: 85.6 against 98.8 and 92.1; 65536 tokens, 32 heads: 183 against
// 197 and 196): four heads need 83 KB of LDS, one workgroup per CU.
template <int T, int N>
int launch_cs(const void* x, const void* B, const float* dt_t, const float* g, float* states,
              float* fin, bool park, const Shape& s, hipStream_t st) {
  const int64_t hpg = s.nheads / s.ngroups;
  const int64_t items = s.batch * s.nchunks() * s.nheads;
  if (hpg % 2 == 0 && items / 2 >= 256)
    return launch_cs_hb<T, N, 2>(x, B, dt_t, g, states, fin, park, s, st);
  return launch_cs_hb<T, N, 1>(x, B, dt_t, g, states, fin, park, s, st);
}

template <int T, int N>
int launch_cs_f32(const void* x, const void* B, const float* dt_t, const float* g,
                  float* states, float* fin, bool park, const Shape& s, hipStream_t st) {
  const int nc = (int)s.nchunks();
  const unsigned blocks = (unsigned)(s.batch * nc * s.nheads);
  hipLaunchKernelGGL((chunk_state_f32<T, N>), dim3(blocks), dim3(256), 0, st, (const float*)x,
                     (const float*)B, dt_t, g, states, fin, (int)s.seqlen, (int)s.nheads,
                     (int)s.ngroups, nc, (int)park);
  return (int)hipGetLastError();
}

template <int N>
int launch_sp(const float* g, const float* init, float* states, float* fin, bool parked,
              const Shape& s, hipStream_t st) {
  constexpr int UNITS = kHeadDim * N / 4;
  const unsigned blocks = (unsigned)(s.batch * s.nheads * (UNITS / 256));
  // D = 4 chunks per register block (measured on the 65536-token sequence:
  // 183 us against 265, 192 and 193 for D = 2, 8 and 16)
  hipLaunchKernelGGL((state_passing_kernel<N, 4>), dim3(blocks), dim3(256), 0, st, g, init,
                     states, fin, (int)s.seqlen, (int)s.chunk, (int)s.nchunks(), (int)parked);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_state(const void* x, const void* B, const float* dt_t, const float* g,
                       float* states, float* fin, bool bf16_in, bool park, const Shape& s,
                       void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (!bf16_in) {
    if (s.dstate == 64) {
      switch (s.chunk) {
        case 64: return launch_cs_f32<64, 64>(x, B, dt_t, g, states, fin, park, s, st);
        case 128: return launch_cs_f32<128, 64>(x, B, dt_t, g, states, fin, park, s, st);
        default: return launch_cs_f32<256, 64>(x, B, dt_t, g, states, fin, park, s, st);
      }
    }
    switch (s.chunk) {
      case 64: return launch_cs_f32<64, 128>(x, B, dt_t, g, states, fin, park, s, st);
      case 128: return launch_cs_f32<128, 128>(x, B, dt_t, g, states, fin, park, s, st);
      default: return launch_cs_f32<256, 128>(x, B, dt_t, g, states, fin, park, s, st);
    }
  }
  if (s.dstate == 64) {
    switch (s.chunk) {
      case 64: return launch_cs<64, 64>(x, B, dt_t, g, states, fin, park, s, st);
      case 128: return launch_cs<128, 64>(x, B, dt_t, g, states, fin, park, s, st);
      default: return launch_cs<256, 64>(x, B, dt_t, g, states, fin, park, s, st);
    }
  }
  switch (s.chunk) {
    case 64: return launch_cs<64, 128>(x, B, dt_t, g, states, fin, park, s, st);
    case 128: return launch_cs<128, 128>(x, B, dt_t, g, states, fin, park, s, st);
    default: return launch_cs<256, 128>(x, B, dt_t, g, states, fin, park, s, st);
  }
}

int launch_state_passing(const float* g, const float* init, float* states, float* fin,
                         bool parked, const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  return s.dstate == 64 ? launch_sp<64>(g, init, states, fin, parked, s, st)
                        : launch_sp<128>(g, init, states, fin, parked, s, st);
}

}  // namespace ssd

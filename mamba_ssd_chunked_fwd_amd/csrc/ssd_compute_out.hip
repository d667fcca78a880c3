// Stage 3: the fused per-chunk output.
//
// For every (b, chunk c, head h), rows i and columns j tokens of the chunk,
// S_c = states[b,h,c]:
//   Y = 2^{g_i} (C S_c^T) + L' X + D_h X,
//   L'[i,j] = (C B^T)[i,j] 2^{g_i - g_j} dt_j   for i >= j, else 0
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", sections "Step 2: Compute a Chunk of Outputs from One State",
// "Step 3: Add Back the Decay, Safely, in Log-Space" and "Kernel 3:
// compute_out, the Fused Output Kernel").  The chunk x chunk matrix lives in
// registers only.  Entries above the diagonal are replaced by zero with a
// select after they are formed, never multiplied by a 0/1 mask, so the
// positive exponents there cannot produce Inf * 0 = NaN.
//
// MI355X design.
// * Persistent workgroups.  The work items are the (b, c, h) triples, h
//   fastest; the grid holds as many workgroups as fit on the chip at once
//   and each takes one contiguous run of items, so every workgroup does the
//   same amount of work and runs of heads share one chunk.  Consecutive runs
//   are placed on the same XCD (blocks are dealt to the 8 XCDs round-robin).
// * Software pipeline across items: while item k is computed from LDS, the
//   x tile, state, g and dt of item k+1 are already in flight into
//   registers.  C B^T and the C fragments depend only on (b, c, group), so
//   they are formed once and reused for every head of the group in the run
//   (the pages compute C B^T once per group as well).
// * One workgroup covers the whole chunk.  Wave w owns query-row block w
//   (16 rows) and, for 256-token chunks (8 waves, 16 blocks), also block
//   NIB-1-w, so every wave has the same share of the causal triangle.
//   128-token chunks take 8 waves of one block each: the waves' shares of
//   the triangle differ, but half the registers per wave allow twice the
//   waves per CU, which measured faster (365 -> 325 us on the 65536-token
//   sequence) than 4 balanced waves of two blocks.  Y is computed
//   transposed (Y^T[p][i]) so each lane's accumulators are four consecutive
//   p of one token: 16-byte stores of y.
// * C B^T is computed transposed (B C^T, rows j, columns i), only for 16x16
//   blocks on or below the diagonal.  In that accumulator layout a lane
//   holds, for its query column i, exactly the j values the next product's
//   operand needs, so L'^T goes from accumulator to matrix operand with no
//   data movement: the decay, dt_j, the causal select and the D_h skip term
//   (folded onto the diagonal, L'[i,i] += D_h) are applied in registers.
// * bf16 inputs: C, B and X are exact bf16 operands; S_c and L' are computed
//   fp32 values, split into bf16 hi + lo (two matrix instructions each).
//   X is staged row-major in LDS and read with the LDS transpose read.
//   fp32 inputs use the fp32 matrix instruction with X staged transposed.
// HBM traffic per item: the x tile, the state S_c (4*64*N bytes), dt, g and
// y; B and C once per (b, c, group) run.  The stage is HBM-bound at every
// supported shape by algorithmic count.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// A byte offset past every buffer range used here (reads return zero).
constexpr uint32_t kPastRange = 0x7FFFFFF0u;

template <bool YBF16>
__device__ __forceinline__ void store_y(void* y, size_t off, f32x4 v) {
  if constexpr (YBF16) {
    *(u32x2*)((uint16_t*)y + off) = (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
    *(f32x4*)((float*)y + off) = v;
  }
}

// Geometry shared by both element types.
template <int T>
struct Geo {
  static constexpr int NIB = T / 16;             // 16-token blocks per chunk
  static constexpr int NW = T >= 128 ? 8 : 4;    // waves per workgroup
  static constexpr int NTHR = 64 * NW;
  static constexpr int MB = NIB / NW;            // query-row blocks per wave
  static_assert(MB == 1 || MB == 2, "one or two row blocks per wave");
};

// bf16 geometry: 8 waves for 128- and 256-token chunks (one or two row
// blocks per wave), 4 for 64-token chunks (one each).  (Measured on the
// small layer: 8 waves that split a 64-token chunk's output columns in two
// took 47.2 against 43.5 us.)
template <int T>
struct GeoB {
  static constexpr int NIB = T / 16;
  static constexpr int NW = T == 64 ? 4 : 8;
  static constexpr int NTHR = 64 * NW;
  static constexpr int MB = NIB / NW;                 // row blocks per wave
  static_assert(MB == 1 || MB == 2, "one or two row blocks per wave");
};

// Row block of slot m (0 or 1) of wave w: w and NIB-1-w.
template <int T>
__device__ __forceinline__ int row_block(int w, int m) {
  return m == 0 ? w : Geo<T>::NIB - 1 - w;
}

template <int T>
__device__ __forceinline__ int row_block_b(int w, int m) {
  return m == 0 ? w : GeoB<T>::NIB - 1 - w;
}

struct Item {
  int b, c, h, grp;
};
__device__ __forceinline__ Item decode_item(int k, int H, int nc, int hpg) {
  Item it;
  it.h = k % H;
  k /= H;
  it.c = k % nc;
  it.b = k / nc;
  it.grp = it.h / hpg;
  return it;
}

// This workgroup's contiguous run of items [k0, k1).
__device__ __forceinline__ void item_range(int items, int& k0, int& k1) {
  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  k0 = (int)((int64_t)wg * items / nwg);
  k1 = (int)((int64_t)(wg + 1) * items / nwg);
}

// ---------------------------------------------------------------- bf16 path
// cb entries: row slot 0 keeps its blocks 0..ib0 at entries 0..ib0; row slot
// 1 keeps block k at entry NE-1-k.  Each row's block count is padded to
// even (the 32-token k-step covers two blocks), padding entries stay zero;
// with ib0 + ib1 = NIB - 1 the two padded counts add up to NIB + 2.
template <int T, int N, bool YBF16>
__global__ __launch_bounds__(GeoB<T>::NTHR) void compute_out_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ Dv, void* __restrict__ y, int L, int H, int G,
    int nc, int items) {
  using Gm = GeoB<T>;
  constexpr int NTHR = Gm::NTHR, MB = Gm::MB, NIB = Gm::NIB;
  constexpr int KN = N / 32;            // k-steps over the state index
  constexpr int XS = 80;                // X tile row stride (bf16), 64 + 16
  constexpr int SS = N + 8;             // state-half row stride (bf16)
  constexpr int XU = T * 8 / NTHR;      // 16-byte x units per thread
  constexpr int SU = 16 * N / NTHR;     // 16-byte state units per thread
  constexpr int NE = MB == 1 ? NIB : NIB + 2;
  static_assert(XU >= 1 && SU >= 1 && 2 * T <= NTHR, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t xs[T * XS];
  __shared__ __attribute__((aligned(16))) uint16_t sh[64 * SS];
  __shared__ __attribute__((aligned(16))) uint16_t sl[64 * SS];
  __shared__ float gs[T], ds[T];
  // per wave: 2^{g_e - g_j} dt_j for the 32 tokens j of one k-step, e its
  // last token
  __shared__ __attribute__((aligned(16))) float cw[Gm::NW][32];

  int k0, k1;
  item_range(items, k0, k1);
  if (k0 >= k1) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int hpg = H / G;
  const uint32_t xbytes = (uint32_t)L * H * kHeadDim * 2;
  const uint32_t bcbytes = (uint32_t)L * G * N * 2;
  const rsrc_t drs = make_rsrc(Dv, (uint32_t)H * 4);

  // ---- per-item operands, prefetched into registers
  struct Regs {
    u32x4 x[XU];
    f32x4 s[SU];
    float gd, dh;
  } r;
  // The loads of one item, as NLOAD single-instruction slots that the
  // compute of the previous item interleaves (see the item loop).  An item
  // index past this workgroup's run gets empty buffer ranges: its loads
  // return zero without touching memory, so every slot is issued on every
  // pass and the loop body has no branch around them.
  constexpr int NLOAD = XU + SU + 2;
  struct Src {
    rsrc_t xr, sr, gdr;
    uint32_t xo[XU], gdo;
    int h;
  };
  auto prepare = [&](int k, Src& sc) {
    const bool live = k < k1;
    const Item it = decode_item(live ? k : k0, H, nc, hpg);
    sc.xr = make_rsrc(x + (size_t)it.b * L * H * kHeadDim, live ? xbytes : 0u);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, row = e >> 3, c8 = e & 7;
      sc.xo[u] = ((uint32_t)(it.c * T + row) * H + it.h) * (kHeadDim * 2) + 16 * c8;
    }
    sc.sr = make_rsrc(states + (((size_t)it.b * H + it.h) * nc + it.c) * kHeadDim * N,
                      live ? kHeadDim * N * 4u : 0u);
    // waves [0, T/64) read g, waves [T/64, 2T/64) read dt (a uniform choice)
    const size_t row = ((size_t)it.b * H + it.h) * L;
    const bool wave_g = __builtin_amdgcn_readfirstlane(tid >> 6) < T / 64;
    sc.gdr = make_rsrc((wave_g ? g : dt_t) + row, live ? (uint32_t)L * 4 : 0u);
    sc.gdo = tid < 2 * T ? 4 * (uint32_t)(it.c * T + (tid % T)) : kPastRange;
    sc.h = it.h;
  };
  auto issue_slot = [&](int j, const Src& sc) {
    if (j < XU) {
      r.x[j] = load_b128(sc.xr, sc.xo[j]);
    } else if (j < XU + SU) {
      r.s[j - XU] = load_f32x4(sc.sr, 16 * (tid + NTHR * (j - XU)));
    } else if (j == XU + SU) {
      r.gd = load_f32(sc.gdr, sc.gdo);
    } else {
      r.dh = load_f32(drs, 4 * sc.h);
    }
  };
  auto commit = [&]() {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, row = e >> 3, c8 = e & 7;
      *(u32x4*)(xs + row * XS + 8 * c8) = r.x[u];
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = tid + NTHR * u, row = e / (N / 4), col = 4 * (e % (N / 4));
      uint32_t h0, l0, h1, l1;
      split_bf16(r.s[u][0], r.s[u][1], h0, l0);
      split_bf16(r.s[u][2], r.s[u][3], h1, l1);
      *(u32x2*)(sh + row * SS + col) = (u32x2){h0, h1};
      *(u32x2*)(sl + row * SS + col) = (u32x2){l0, l1};
    }
    if (tid < T) {
      gs[tid] = r.gd;
    } else if (tid < 2 * T) {
      ds[tid - T] = r.gd;
    }
  };

  // ---- C fragments (k = state index 32kk + 8lq + e) and C B^T blocks,
  //      cb[entry][rr] = (C B^T)[i][16 jb + 4 lq + rr]
  u32x4 cf[MB][KN];
  f32x4 cb[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) cb[e] = (f32x4){0, 0, 0, 0};
  auto form_cb = [&](const Item& it) {
    const rsrc_t cr = make_rsrc(Cm + (size_t)it.b * L * G * N, bcbytes);
    const rsrc_t br = make_rsrc(Bm + (size_t)it.b * L * G * N, bcbytes);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int i = 16 * row_block_b<T>(wave, m) + lr;
      const uint32_t off = ((uint32_t)(it.c * T + i) * G + it.grp) * (N * 2) + 16 * lq;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) cf[m][kk] = load_b128(cr, off + 64 * kk);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block_b<T>(wave, m);
#pragma unroll
      for (int k = 0; k < NIB; ++k) {
        if (k <= ib) {
          const uint32_t off =
              ((uint32_t)(it.c * T + 16 * k + lr) * G + it.grp) * (N * 2) + 16 * lq;
          f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
          for (int kk = 0; kk < KN; ++kk) acc = mfma_bf16(load_b128(br, off + 64 * kk), cf[m][kk], acc);
          if (m == 0) {
            if (k < NE) cb[k] = acc;
          } else {
            if (NE - 1 - k >= 0) cb[NE - 1 - k] = acc;
          }
        }
      }
    }
  };

  {
    Src sc;
    prepare(k0, sc);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc);
  }
  int key = -1;
  for (int k = k0; k < k1; ++k) {
    const Item it = decode_item(k, H, nc, hpg);
    const int nkey = (it.b * nc + it.c) * G + it.grp;
    if (nkey != key) {
      form_cb(it);
      key = nkey;
    }
    __syncthreads();  // the previous item's LDS reads are done
    commit();
    const float Dh = r.dh;
    Src nxt;
    prepare(k + 1, nxt);
    __syncthreads();

    const int t0 = it.c * T;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block_b<T>(wave, m);
      const int i = 16 * ib + lr;
      // Y^T = S C^T (state split hi + lo), then column i scaled by 2^{g_i}
      f32x4 yacc[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          // the next item's loads, one per pair of matrix instructions
          if (m == 0 && 4 * kk + pb < NLOAD) issue_slot(4 * kk + pb, nxt);
          const int off = (16 * pb + lr) * SS + 32 * kk + 8 * lq;
          yacc[pb] = mfma_bf16(*(const u32x4*)(sh + off), cf[m][kk], yacc[pb]);
          yacc[pb] = mfma_bf16(*(const u32x4*)(sl + off), cf[m][kk], yacc[pb]);
        }
      }
      if (m == 0) {
#pragma unroll
        for (int j = 4 * KN; j < NLOAD; ++j) issue_slot(j, nxt);
      }
      const float gi = gs[i];
      const float ei = exp2_hw(gi);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

      // Y^T += X^T L'^T over 32-token k-steps s: slots 0..3 carry tokens
      // 32s + 4lq + rr and slots 4..7 tokens 32s + 16 + 4lq + rr.
      // A step wholly below the row block (every j <= e = 32s + 31 < i)
      // factors the decay as 2^{g_i - g_e} 2^{g_e - g_j}, both exponents
      // <= 0: the wave forms the 32 column factors once (one exponential
      // per lane) and shares them through its own LDS row, each lane adds
      // one exponential for its row, and no causal select is needed.  The
      // step that meets the diagonal takes the entries one by one.
      const bool row_in = t0 + i < L;
#pragma unroll
      for (int s = 0; s < NE / 2; ++s) {
        if (2 * s <= ib) {
          const int e0 = m == 0 ? 2 * s : NE - 1 - 2 * s;
          const int e1 = m == 0 ? 2 * s + 1 : NE - 2 - 2 * s;
          float v[8];
          if (2 * s + 2 <= ib) {
            const float ge = gs[32 * s + 31];
            const int jl = 32 * s + (lane & 31);
            const float cl = exp2_hw(ge - gs[jl]) * ds[jl];
            if (lane < 32) cw[wave][lane] = cl;
            // rows past the sequence's end are never stored
            const float ai = row_in ? exp2_hw(gi - ge) : 0.0f;
            const f32x4 c0 = *(const f32x4*)(&cw[wave][4 * lq]);
            const f32x4 c1 = *(const f32x4*)(&cw[wave][16 + 4 * lq]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              v[rr] = cb[e0][rr] * (c0[rr] * ai);
              v[4 + rr] = cb[e1][rr] * (c1[rr] * ai);
            }
          } else {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const f32x4 cbv = half ? cb[e1] : cb[e0];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int j = 32 * s + 16 * half + 4 * lq + rr;
                float w = cbv[rr] * exp2_hw(gi - gs[j]) * ds[j];
                if (j == i) w += Dh;
                v[4 * half + rr] = j <= i ? w : 0.0f;
              }
            }
          }
          uint32_t lh4[4], ll4[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) split_bf16(v[2 * q], v[2 * q + 1], lh4[q], ll4[q]);
          const u32x4 lh = make_u32x4(lh4), ll = make_u32x4(ll4);
          const uint16_t* xp = xs + (32 * s + 4 * lq + (lr >> 2)) * XS + 4 * (lr & 3);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) {
            const u32x2 a0 = lds_read_tr16(xp + 16 * pb);
            const u32x2 a1 = lds_read_tr16(xp + 16 * XS + 16 * pb);
            const u32x4 xa = (u32x4){a0[0], a0[1], a1[0], a1[1]};
            yacc[pb] = mfma_bf16(xa, lh, yacc[pb]);
            yacc[pb] = mfma_bf16(xa, ll, yacc[pb]);
          }
        }
      }
      if (t0 + i < L) {
        const size_t off = (((size_t)it.b * L + t0 + i) * H + it.h) * kHeadDim + 4 * lq;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
      }
    }
  }
}

// ------------------------------------------------ fp32 via split bf16
// fp32 inputs on the bf16 matrix instructions: every operand is split into
// three bf16 terms, exactly (hi + mid + lo), and each product keeps its six
// terms of relative size 2^-16 or more (hh, hm, mh, hl, mm, lh), which is
// fp32 accuracy at 6 x 16 cycles per 32-step of k instead of 8 x 32 with the
// fp32 instruction.  Same geometry, item order, prefetch and operand layouts
// as compute_out_bf16: the x tile and the state are staged in LDS as three
// bf16 planes each, C and B fragments are split in registers, and L' is
// split where it is formed.
template <int T, int N, bool YBF16>
__global__ __launch_bounds__(GeoB<T>::NTHR) void compute_out_f32s(
    const float* __restrict__ x, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ Dv, void* __restrict__ y, int L, int H, int G,
    int nc, int items) {
  using Gm = GeoB<T>;
  constexpr int NTHR = Gm::NTHR, MB = Gm::MB, NIB = Gm::NIB;
  constexpr int KN = N / 32;            // k-steps over the state index
  constexpr int XS = 80;                // x plane row stride (bf16), 64 + 16
  constexpr int SS = N + 8;             // state plane row stride (bf16)
  constexpr int XU = T * 16 / NTHR;     // 16-byte fp32 x units per thread
  constexpr int SU = 16 * N / NTHR;     // 16-byte state units per thread
  constexpr int NE = MB == 1 ? NIB : NIB + 2;
  static_assert(XU >= 1 && SU >= 1 && 2 * T <= NTHR, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t xs[3][T * XS];
  __shared__ __attribute__((aligned(16))) uint16_t ss[3][64 * SS];
  __shared__ float gs[T], ds[T];
  __shared__ __attribute__((aligned(16))) float cw[Gm::NW][32];

  int k0, k1;
  item_range(items, k0, k1);
  if (k0 >= k1) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int hpg = H / G;
  const uint32_t xbytes = (uint32_t)L * H * kHeadDim * 4;
  const uint32_t bcbytes = (uint32_t)L * G * N * 4;
  const rsrc_t drs = make_rsrc(Dv, (uint32_t)H * 4);

  struct Regs {
    f32x4 x[XU];
    f32x4 s[SU];
    float gd, dh;
  };
  Regs ra, rb;
  constexpr int NLOAD = XU + SU + 2;
  struct Src {
    rsrc_t xr, sr, gdr;
    uint32_t xo[XU], gdo;
    int h;
  };
  auto prepare = [&](int k, Src& sc) {
    const bool live = k < k1;
    const Item it = decode_item(live ? k : k0, H, nc, hpg);
    sc.xr = make_rsrc(x + (size_t)it.b * L * H * kHeadDim, live ? xbytes : 0u);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, row = e >> 4, c4 = e & 15;
      sc.xo[u] = ((uint32_t)(it.c * T + row) * H + it.h) * (kHeadDim * 4) + 16 * c4;
    }
    sc.sr = make_rsrc(states + (((size_t)it.b * H + it.h) * nc + it.c) * kHeadDim * N,
                      live ? kHeadDim * N * 4u : 0u);
    const size_t row = ((size_t)it.b * H + it.h) * L;
    const bool wave_g = __builtin_amdgcn_readfirstlane(tid >> 6) < T / 64;
    sc.gdr = make_rsrc((wave_g ? g : dt_t) + row, live ? (uint32_t)L * 4 : 0u);
    sc.gdo = tid < 2 * T ? 4 * (uint32_t)(it.c * T + (tid % T)) : kPastRange;
    sc.h = it.h;
  };
  auto issue_slot = [&](int j, const Src& sc, Regs& r) {
    if (j < XU) {
      r.x[j] = load_f32x4(sc.xr, sc.xo[j]);
    } else if (j < XU + SU) {
      r.s[j - XU] = load_f32x4(sc.sr, 16 * (tid + NTHR * (j - XU)));
    } else if (j == XU + SU) {
      r.gd = load_f32(sc.gdr, sc.gdo);
    } else {
      r.dh = load_f32(drs, 4 * sc.h);
    }
  };
  auto commit = [&](const Regs& r) {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, row = e >> 4, c4 = e & 15;
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(r.x[u][0], r.x[u][1], h0, m0, l0);
      split3_bf16(r.x[u][2], r.x[u][3], h1, m1, l1);
      const int o = row * XS + 4 * c4;
      *(u32x2*)(xs[0] + o) = (u32x2){h0, h1};
      *(u32x2*)(xs[1] + o) = (u32x2){m0, m1};
      *(u32x2*)(xs[2] + o) = (u32x2){l0, l1};
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = tid + NTHR * u, row = e / (N / 4), col = 4 * (e % (N / 4));
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(r.s[u][0], r.s[u][1], h0, m0, l0);
      split3_bf16(r.s[u][2], r.s[u][3], h1, m1, l1);
      const int o = row * SS + col;
      *(u32x2*)(ss[0] + o) = (u32x2){h0, h1};
      *(u32x2*)(ss[1] + o) = (u32x2){m0, m1};
      *(u32x2*)(ss[2] + o) = (u32x2){l0, l1};
    }
    if (tid < T) {
      gs[tid] = r.gd;
    } else if (tid < 2 * T) {
      ds[tid - T] = r.gd;
    }
  };
  // the six products of a split pair: acc += a * b to fp32 accuracy
  auto mfma6 = [](const u32x4 (&a)[3], const u32x4 (&b)[3], f32x4 acc) {
    acc = mfma_bf16(a[0], b[0], acc);
    acc = mfma_bf16(a[0], b[1], acc);
    acc = mfma_bf16(a[1], b[0], acc);
    acc = mfma_bf16(a[0], b[2], acc);
    acc = mfma_bf16(a[1], b[1], acc);
    acc = mfma_bf16(a[2], b[0], acc);
    return acc;
  };
  // eight consecutive fp32 values split into three bf16 fragments
  auto split8 = [](const f32x4& v0, const f32x4& v1, u32x4 (&f)[3]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      uint32_t h, m, l;
      split3_bf16(v0[2 * q], v0[2 * q + 1], h, m, l);
      f[0][q] = h; f[1][q] = m; f[2][q] = l;
      split3_bf16(v1[2 * q], v1[2 * q + 1], h, m, l);
      f[0][2 + q] = h; f[1][2 + q] = m; f[2][2 + q] = l;
    }
  };

  // ---- C fragments (k = state index 32kk + 8lq + e, three planes) and
  //      C B^T blocks, cb[entry][rr] = (C B^T)[i][16 jb + 4 lq + rr]
  u32x4 cf[MB][KN][3];
  f32x4 cb[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) cb[e] = (f32x4){0, 0, 0, 0};
  auto form_cb = [&](const Item& it) {
    const rsrc_t cr = make_rsrc(Cm + (size_t)it.b * L * G * N, bcbytes);
    const rsrc_t br = make_rsrc(Bm + (size_t)it.b * L * G * N, bcbytes);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int i = 16 * row_block_b<T>(wave, m) + lr;
      const uint32_t off = ((uint32_t)(it.c * T + i) * G + it.grp) * (N * 4) + 32 * lq;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk)
        split8(load_f32x4(cr, off + 128 * kk), load_f32x4(cr, off + 128 * kk + 16), cf[m][kk]);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block_b<T>(wave, m);
#pragma unroll
      for (int k = 0; k < NIB; ++k) {
        if (k <= ib) {
          const uint32_t off =
              ((uint32_t)(it.c * T + 16 * k + lr) * G + it.grp) * (N * 4) + 32 * lq;
          f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
          for (int kk = 0; kk < KN; ++kk) {
            u32x4 bf[3];
            split8(load_f32x4(br, off + 128 * kk), load_f32x4(br, off + 128 * kk + 16), bf);
            acc = mfma6(bf, cf[m][kk], acc);
          }
          if (m == 0) {
            if (k < NE) cb[k] = acc;
          } else {
            if (NE - 1 - k >= 0) cb[NE - 1 - k] = acc;
          }
        }
      }
    }
  };

  // Two items of prefetch: the loads of items k0 and k0 + 1 go out first;
  // item k is committed from its register set, which then takes the loads
  // of item k + 2 while item k is computed.
  {
    Src sc;
    prepare(k0, sc);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, ra);
    prepare(k0 + 1, sc);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, rb);
  }
  int key = -1;
  auto body = [&](int k, Regs& r) {
    const Item it = decode_item(k, H, nc, hpg);
    const int nkey = (it.b * nc + it.c) * G + it.grp;
    if (nkey != key) {
      form_cb(it);
      key = nkey;
    }
    __syncthreads();  // the previous item's LDS reads are done
    commit(r);
    const float Dh = r.dh;
    Src nxt;
    prepare(k + 2, nxt);
    __syncthreads();

    const int t0 = it.c * T;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block_b<T>(wave, m);
      const int i = 16 * ib + lr;
      // Y^T = S C^T (both split), then column i scaled by 2^{g_i}
      f32x4 yacc[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          if (m == 0 && 4 * kk + pb < NLOAD) issue_slot(4 * kk + pb, nxt, r);
          const int off = (16 * pb + lr) * SS + 32 * kk + 8 * lq;
          const u32x4 sa[3] = {*(const u32x4*)(ss[0] + off), *(const u32x4*)(ss[1] + off),
                               *(const u32x4*)(ss[2] + off)};
          yacc[pb] = mfma6(sa, cf[m][kk], yacc[pb]);
        }
      }
      if (m == 0) {
#pragma unroll
        for (int j = 4 * KN; j < NLOAD; ++j) issue_slot(j, nxt, r);
      }
      const float gi = gs[i];
      const float ei = exp2_hw(gi);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

      // Y^T += X^T L'^T over 32-token k-steps, the decay factored below the
      // diagonal exactly as in compute_out_bf16
      const bool row_in = t0 + i < L;
#pragma unroll
      for (int s = 0; s < NE / 2; ++s) {
        if (2 * s <= ib) {
          const int e0 = m == 0 ? 2 * s : NE - 1 - 2 * s;
          const int e1 = m == 0 ? 2 * s + 1 : NE - 2 - 2 * s;
          float v[8];
          if (2 * s + 2 <= ib) {
            const float ge = gs[32 * s + 31];
            const int jl = 32 * s + (lane & 31);
            const float cl = exp2_hw(ge - gs[jl]) * ds[jl];
            if (lane < 32) cw[wave][lane] = cl;
            const float ai = row_in ? exp2_hw(gi - ge) : 0.0f;
            const f32x4 c0 = *(const f32x4*)(&cw[wave][4 * lq]);
            const f32x4 c1 = *(const f32x4*)(&cw[wave][16 + 4 * lq]);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
              v[rr] = cb[e0][rr] * (c0[rr] * ai);
              v[4 + rr] = cb[e1][rr] * (c1[rr] * ai);
            }
          } else {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
              const f32x4 cbv = half ? cb[e1] : cb[e0];
#pragma unroll
              for (int rr = 0; rr < 4; ++rr) {
                const int j = 32 * s + 16 * half + 4 * lq + rr;
                float w = cbv[rr] * exp2_hw(gi - gs[j]) * ds[j];
                if (j == i) w += Dh;
                v[4 * half + rr] = j <= i ? w : 0.0f;
              }
            }
          }
          u32x4 lf[3];
          split8((f32x4){v[0], v[1], v[2], v[3]}, (f32x4){v[4], v[5], v[6], v[7]}, lf);
          const int xo = (32 * s + 4 * lq + (lr >> 2)) * XS + 4 * (lr & 3);
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) {
            u32x4 xa[3];
#pragma unroll
            for (int q = 0; q < 3; ++q) {
              const u32x2 a0 = lds_read_tr16(xs[q] + xo + 16 * pb);
              const u32x2 a1 = lds_read_tr16(xs[q] + xo + 16 * XS + 16 * pb);
              xa[q] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
            }
            yacc[pb] = mfma6(xa, lf, yacc[pb]);
          }
        }
      }
      if (t0 + i < L) {
        const size_t off = (((size_t)it.b * L + t0 + i) * H + it.h) * kHeadDim + 4 * lq;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
      }
    }
  };
  for (int k = k0; k < k1; k += 2) {
    body(k, ra);
    if (k + 1 < k1) body(k + 1, rb);
  }
}

// ---------------------------------------------------------------- fp32 path
// k-map over the state index n for v_mfma_f32_16x16x4_f32: step (u, v)
// gives lane group lq the index 16u + 4lq + v; over tokens j: step (jb, rr)
// gives 16jb + 4lq + rr, which is exactly the j of accumulator element rr.
// cb entries: row slot 0 block k at entry k, row slot 1 block k at entry
// NE-1-k; the two rows have NIB + 1 blocks together.
template <int T, int N, bool YBF16>
__global__ __launch_bounds__(Geo<T>::NTHR) void compute_out_f32(
    const float* __restrict__ x, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ Dv, void* __restrict__ y, int L, int H, int G,
    int nc, int items) {
  using Gm = Geo<T>;
  constexpr int NTHR = Gm::NTHR, MB = Gm::MB, NIB = Gm::NIB;
  constexpr int KU = N / 16;            // groups of four k-steps over n
  constexpr int XS = T + 4;             // X^T row stride (floats)
  constexpr int SS = N + 4;             // state row stride (floats)
  constexpr int XU = 4 * T / NTHR;      // (4 tokens x 4 p) x units per thread
  constexpr int SU = 16 * N / NTHR;     // 16-byte state units per thread
  constexpr int NE = MB == 1 ? NIB : NIB + 1;
  static_assert(XU >= 1 && SU >= 1 && 2 * T <= NTHR, "tile split");
  __shared__ __attribute__((aligned(16))) float xT[64 * XS];
  __shared__ __attribute__((aligned(16))) float ss[64 * SS];
  __shared__ float gs[T], ds[T];

  int k0, k1;
  item_range(items, k0, k1);
  if (k0 >= k1) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int hpg = H / G;
  const uint32_t xbytes = (uint32_t)L * H * kHeadDim * 4;
  const uint32_t bcbytes = (uint32_t)L * G * N * 4;
  const rsrc_t drs = make_rsrc(Dv, (uint32_t)H * 4);

  struct Regs {
    f32x4 x[XU][4];
    f32x4 s[SU];
    float gd, dh;
  } r;
  auto issue = [&](int k) {
    const Item it = decode_item(k, H, nc, hpg);
    const rsrc_t xr = make_rsrc(x + (size_t)it.b * L * H * kHeadDim, xbytes);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, pq = e & 15, tq = e >> 4;
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        r.x[u][rr] = load_f32x4(
            xr, ((uint32_t)(it.c * T + 4 * tq + rr) * H + it.h) * (kHeadDim * 4) + 16 * pq);
    }
    const rsrc_t sr = make_rsrc(
        states + (((size_t)it.b * H + it.h) * nc + it.c) * kHeadDim * N, kHeadDim * N * 4);
#pragma unroll
    for (int u = 0; u < SU; ++u) r.s[u] = load_f32x4(sr, 16 * (tid + NTHR * u));
    const size_t row = ((size_t)it.b * H + it.h) * L;
    const uint32_t toff = 4 * (uint32_t)(it.c * T + (tid % T));
    if (tid < T) {
      r.gd = load_f32(make_rsrc(g + row, (uint32_t)L * 4), toff);
    } else if (tid < 2 * T) {
      r.gd = load_f32(make_rsrc(dt_t + row, (uint32_t)L * 4), toff);
    }
    r.dh = load_f32(drs, 4 * it.h);
  };
  auto commit = [&]() {
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + NTHR * u, pq = e & 15, tq = e >> 4;
#pragma unroll
      for (int ee = 0; ee < 4; ++ee)
        *(f32x4*)(xT + (4 * pq + ee) * XS + 4 * tq) =
            (f32x4){r.x[u][0][ee], r.x[u][1][ee], r.x[u][2][ee], r.x[u][3][ee]};
    }
#pragma unroll
    for (int u = 0; u < SU; ++u) {
      const int e = tid + NTHR * u, row = e / (N / 4), col = 4 * (e % (N / 4));
      *(f32x4*)(ss + row * SS + col) = r.s[u];
    }
    if (tid < T) {
      gs[tid] = r.gd;
    } else if (tid < 2 * T) {
      ds[tid - T] = r.gd;
    }
  };

  f32x4 cf[MB][KU];
  f32x4 cb[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) cb[e] = (f32x4){0, 0, 0, 0};
  auto form_cb = [&](const Item& it) {
    const rsrc_t cr = make_rsrc(Cm + (size_t)it.b * L * G * N, bcbytes);
    const rsrc_t br = make_rsrc(Bm + (size_t)it.b * L * G * N, bcbytes);
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int i = 16 * row_block<T>(wave, m) + lr;
      const uint32_t off = ((uint32_t)(it.c * T + i) * G + it.grp) * (N * 4) + 16 * lq;
#pragma unroll
      for (int u = 0; u < KU; ++u) cf[m][u] = load_f32x4(cr, off + 64 * u);
    }
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block<T>(wave, m);
#pragma unroll
      for (int k = 0; k < NIB; ++k) {
        if (k <= ib) {
          const uint32_t off =
              ((uint32_t)(it.c * T + 16 * k + lr) * G + it.grp) * (N * 4) + 16 * lq;
          f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
          for (int u = 0; u < KU; ++u) {
            const f32x4 bv = load_f32x4(br, off + 64 * u);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc = mfma_f32(bv[v], cf[m][u][v], acc);
          }
          if (m == 0) {
            if (k < NE) cb[k] = acc;
          } else {
            if (NE - 1 - k >= 0) cb[NE - 1 - k] = acc;
          }
        }
      }
    }
  };

  issue(k0);
  int key = -1;
  for (int k = k0; k < k1; ++k) {
    const Item it = decode_item(k, H, nc, hpg);
    const int nkey = (it.b * nc + it.c) * G + it.grp;
    if (nkey != key) {
      form_cb(it);
      key = nkey;
    }
    __syncthreads();
    commit();
    const float Dh = r.dh;
    if (k + 1 < k1) issue(k + 1);
    __syncthreads();

    const int t0 = it.c * T;
#pragma unroll
    for (int m = 0; m < MB; ++m) {
      const int ib = row_block<T>(wave, m);
      const int i = 16 * ib + lr;
      f32x4 yacc[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        yacc[pb] = (f32x4){0, 0, 0, 0};
        const float* srow = ss + (16 * pb + lr) * SS + 4 * lq;
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const f32x4 sv = *(const f32x4*)(srow + 16 * u);
#pragma unroll
          for (int v = 0; v < 4; ++v) yacc[pb] = mfma_f32(sv[v], cf[m][u][v], yacc[pb]);
        }
      }
      const float gi = gs[i];
      const float ei = exp2_hw(gi);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

#pragma unroll
      for (int kb = 0; kb < NIB; ++kb) {
        if (kb <= ib) {
          const int e = m == 0 ? kb : NE - 1 - kb;
          if (e < 0 || e >= NE) continue;
          float w[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int j = 16 * kb + 4 * lq + rr;
            float v = cb[e][rr] * exp2_hw(gi - gs[j]) * ds[j];
            if (j == i) v += Dh;
            w[rr] = j <= i ? v : 0.0f;
          }
#pragma unroll
          for (int pb = 0; pb < 4; ++pb) {
            const f32x4 xv = *(const f32x4*)(xT + (16 * pb + lr) * XS + 16 * kb + 4 * lq);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) yacc[pb] = mfma_f32(xv[rr], w[rr], yacc[pb]);
          }
        }
      }
      if (t0 + i < L) {
        const size_t off = (((size_t)it.b * L + t0 + i) * H + it.h) * kHeadDim + 4 * lq;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
      }
    }
  }
}

// ------------------------------------------------------------- launching
template <bool BF16, int T, int N, bool YBF16>
int launch_t(const void* x, const void* B, const void* C, const float* dt_t,
             const float* g, const float* states, const float* D, void* y,
             const Shape& s, hipStream_t st) {
  constexpr int NTHR = BF16 ? GeoB<T>::NTHR : Geo<T>::NTHR;
  const int nc = (int)s.nchunks();
  const int L = (int)s.seqlen, H = (int)s.nheads, G = (int)s.ngroups;
  const int items = (int)(s.batch * nc * s.nheads);
  // fp32 inputs: the split-bf16 kernel for chunks of 64 and 128 tokens (its
  // three x planes of 256 tokens would not fit the LDS beside the state)
  constexpr bool SPLIT = !BF16 && T <= 128;
  constexpr int NTHR_K = SPLIT ? GeoB<T>::NTHR : NTHR;
  const void* kern;
  if constexpr (BF16) kern = (const void*)compute_out_bf16<T, N, YBF16>;
  else if constexpr (SPLIT) kern = (const void*)compute_out_f32s<T, N, YBF16>;
  else kern = (const void*)compute_out_f32<T, N, YBF16>;
  // the persistent grid: as many workgroups as are resident on the device
  static PerDeviceInt resident;
  const int slots = resident.get([&](int dev) { return resident_slots(kern, NTHR_K, dev); });
  if (slots <= 0) return (int)hipErrorInvalidDevice;
  const unsigned grid = (unsigned)(items < slots ? items : slots);
  if constexpr (BF16) {
    hipLaunchKernelGGL((compute_out_bf16<T, N, YBF16>), dim3(grid), dim3(NTHR), 0, st,
                       (const uint16_t*)x, (const uint16_t*)B, (const uint16_t*)C, dt_t, g,
                       states, D, y, L, H, G, nc, items);
  } else if constexpr (SPLIT) {
    hipLaunchKernelGGL((compute_out_f32s<T, N, YBF16>), dim3(grid), dim3(NTHR_K), 0, st,
                       (const float*)x, (const float*)B, (const float*)C, dt_t, g, states,
                       D, y, L, H, G, nc, items);
  } else {
    hipLaunchKernelGGL((compute_out_f32<T, N, YBF16>), dim3(grid), dim3(NTHR), 0, st,
                       (const float*)x, (const float*)B, (const float*)C, dt_t, g, states,
                       D, y, L, H, G, nc, items);
  }
  return (int)hipGetLastError();
}

template <bool BF16, int T, int N>
int launch_y(const void* x, const void* B, const void* C, const float* dt_t,
             const float* g, const float* states, const float* D, void* y,
             bool ybf16, const Shape& s, hipStream_t st) {
  if (ybf16) return launch_t<BF16, T, N, true>(x, B, C, dt_t, g, states, D, y, s, st);
  return launch_t<BF16, T, N, false>(x, B, C, dt_t, g, states, D, y, s, st);
}

template <bool BF16, int T>
int launch_n(const void* x, const void* B, const void* C, const float* dt_t,
             const float* g, const float* states, const float* D, void* y,
             bool ybf16, const Shape& s, hipStream_t st) {
  if (s.dstate == 64) return launch_y<BF16, T, 64>(x, B, C, dt_t, g, states, D, y, ybf16, s, st);
  return launch_y<BF16, T, 128>(x, B, C, dt_t, g, states, D, y, ybf16, s, st);
}

template <bool BF16>
int launch_chunk(const void* x, const void* B, const void* C, const float* dt_t,
                 const float* g, const float* states, const float* D, void* y,
                 bool ybf16, const Shape& s, hipStream_t st) {
  switch (s.chunk) {
    case 64: return launch_n<BF16, 64>(x, B, C, dt_t, g, states, D, y, ybf16, s, st);
    case 128: return launch_n<BF16, 128>(x, B, C, dt_t, g, states, D, y, ybf16, s, st);
    default: return launch_n<BF16, 256>(x, B, C, dt_t, g, states, D, y, ybf16, s, st);
  }
}

}  // namespace

int launch_compute_out(const void* x, const void* B, const void* C,
                       const float* dt_t, const float* g, const float* states,
                       const float* D, void* y, bool bf16_in, bool bf16_out,
                       const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (bf16_in) return launch_chunk<true>(x, B, C, dt_t, g, states, D, y, bf16_out, s, st);
  return launch_chunk<false>(x, B, C, dt_t, g, states, D, y, bf16_out, s, st);
}

}  // namespace ssd

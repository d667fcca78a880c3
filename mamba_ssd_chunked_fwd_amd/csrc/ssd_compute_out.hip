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
// * One workgroup (4 waves) per (b, c, 64-row tile q of the chunk, h); wave
//   w owns the 16 query rows i in block ib = 4q + w and all 64 columns p of
//   y, computed transposed (Y^T[p][i]) so each lane's accumulators are four
//   consecutive p of one token: 16-byte stores of y.
// * C B^T is computed transposed as well (B C^T, rows j, columns i), only for
//   16x16 blocks on or below the diagonal.  In that accumulator layout a lane
//   holds, for its query column i, exactly the eight j values the next
//   product's operand needs, so L'^T goes from accumulator to matrix operand
//   with no data movement: the decay, dt_j, the causal select and the D_h
//   skip term (folded onto the diagonal, L'[i,i] += D_h) are applied in
//   registers.
// * X is staged in LDS token-contiguous ([p][j]) for the L' X product; the
//   state S_c is staged in LDS row-major.  The C fragments of a wave's rows
//   are the B operand of both C S^T and B C^T and are loaded once.
// * bf16 inputs: C, B and X are exact bf16 operands; S_c and L' are computed
//   fp32 values and are split into bf16 hi + lo (two MFMAs each).  fp32
//   inputs use the fp32 matrix instruction.
// HBM traffic per (b, h, chunk): x, C and B tiles, dt and g, the state
// S_c (4*64*N) and y; the stage is HBM-bound at every supported shape by
// algorithmic count.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

template <bool BF16>
struct In;
template <>
struct In<true> { using T = uint16_t; };
template <>
struct In<false> { using T = float; };

template <bool YBF16>
__device__ __forceinline__ void store_y(void* y, size_t off, f32x4 v) {
  if constexpr (YBF16) {
    *(u32x2*)((uint16_t*)y + off) = (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
    *(f32x4*)((float*)y + off) = v;
  }
}

// Decode the flat block id: h fastest, then the row tile, chunk and batch.
struct OutTile {
  int h, q, c, b;
};
__device__ __forceinline__ OutTile decode_tile(int bid, int H, int NQ, int nc) {
  OutTile t;
  t.h = bid % H;
  bid /= H;
  t.q = bid % NQ;
  bid /= NQ;
  t.c = bid % nc;
  t.b = bid / nc;
  return t;
}

// ---------------------------------------------------------------- bf16 path
template <int T, int N, bool YBF16>
__global__ __launch_bounds__(256) void compute_out_bf16(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Bm,
    const uint16_t* __restrict__ Cm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ Dv, void* __restrict__ y, int L, int H, int G,
    int nc) {
  constexpr int NQ = T / 64;
  constexpr int XS = T + 8;   // xT row stride (bf16)
  constexpr int SS = N + 8;   // state row stride (bf16)
  constexpr int KN = N / 32;  // k-steps over the state index
  constexpr int NJB = T / 16; // 16-token blocks per chunk
  __shared__ __attribute__((aligned(16))) uint16_t xT[64 * XS];
  __shared__ __attribute__((aligned(16))) uint16_t sh[64 * SS];
  __shared__ __attribute__((aligned(16))) uint16_t sl[64 * SS];
  __shared__ float gs[T], ds[T];

  const OutTile tile = decode_tile(blockIdx.x, H, NQ, nc);
  const int h = tile.h, q = tile.q, c = tile.c, b = tile.b;
  const int grp = h / (H / G);
  const int t0 = c * T;
  const int nvalid = min(T, L - t0);
  const int bh_idx = b * H + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int ib = 4 * q + wave;
  const int i = 16 * ib + lr;          // this lane's query token in the chunk

  // ---- stage X^T (tokens [0, 64(q+1))), the state split, g and dt in LDS
  {
    const int pp = tid & 31, xtb = tid >> 5;
    for (int it = 0; it <= q; ++it) {
      uint32_t xr[8];
#pragma unroll
      for (int r = 0; r < 8; ++r) {
        const int t = 8 * (xtb + 8 * it) + r;
        xr[r] = t < nvalid
            ? *(const uint32_t*)(x + (((size_t)b * L + t0 + t) * H + h) * kHeadDim + 2 * pp)
            : 0u;
      }
      u32x4 lo, hi;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        lo[k] = lo_halves(xr[2 * k], xr[2 * k + 1]);
        hi[k] = hi_halves(xr[2 * k], xr[2 * k + 1]);
      }
      const int tcol = 8 * (xtb + 8 * it);
      *(u32x4*)(xT + (2 * pp) * XS + tcol) = lo;
      *(u32x4*)(xT + (2 * pp + 1) * XS + tcol) = hi;
    }
    const float* S = states + ((size_t)bh_idx * nc + c) * kHeadDim * N;
#pragma unroll
    for (int u = tid; u < kHeadDim * N / 8; u += 256) {
      const int row = u / (N / 8), col = 8 * (u % (N / 8));
      const f32x4 a = *(const f32x4*)(S + (size_t)row * N + col);
      const f32x4 a2 = *(const f32x4*)(S + (size_t)row * N + col + 4);
      uint32_t hv[4], lv[4];
      split_bf16(a[0], a[1], hv[0], lv[0]);
      split_bf16(a[2], a[3], hv[1], lv[1]);
      split_bf16(a2[0], a2[1], hv[2], lv[2]);
      split_bf16(a2[2], a2[3], hv[3], lv[3]);
      *(u32x4*)(sh + row * SS + col) = make_u32x4(hv);
      *(u32x4*)(sl + row * SS + col) = make_u32x4(lv);
    }
    for (int t = tid; t < T; t += 256) {
      const bool ok = t < nvalid;
      gs[t] = ok ? g[(size_t)bh_idx * L + t0 + t] : 0.0f;
      ds[t] = ok ? dt_t[(size_t)bh_idx * L + t0 + t] : 0.0f;
    }
  }

  // ---- C fragments of this lane's query token (k = state index 32kk+8lq+e)
  u32x4 cf[KN];
  {
    const bool ok = i < nvalid;
    const uint16_t* crow = Cm + (((size_t)b * L + t0 + i) * G + grp) * N + 8 * lq;
#pragma unroll
    for (int kk = 0; kk < KN; ++kk)
      cf[kk] = ok ? *(const u32x4*)(crow + 32 * kk) : (u32x4){0, 0, 0, 0};
  }

  // ---- (B C^T) blocks on or below the diagonal: cb[jb][r] = (C B^T)[i][j],
  //      j = 16 jb + 4 lq + r
  f32x4 cb[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    cb[jb] = (f32x4){0, 0, 0, 0};
    if (jb <= ib) {
      const int j = 16 * jb + lr;
      const bool ok = j < nvalid;
      const uint16_t* brow = Bm + (((size_t)b * L + t0 + j) * G + grp) * N + 8 * lq;
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
        const u32x4 bv = ok ? *(const u32x4*)(brow + 32 * kk) : (u32x4){0, 0, 0, 0};
        cb[jb] = mfma_bf16(bv, cf[kk], cb[jb]);
      }
    }
  }
  __syncthreads();

  // ---- Y^T = S C^T (state split hi + lo), then scale column i by 2^{g_i}
  f32x4 yacc[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) yacc[pb] = (f32x4){0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const int off = (16 * pb + lr) * SS + 32 * kk + 8 * lq;
      yacc[pb] = mfma_bf16(*(const u32x4*)(sh + off), cf[kk], yacc[pb]);
      yacc[pb] = mfma_bf16(*(const u32x4*)(sl + off), cf[kk], yacc[pb]);
    }
  }
  const float gi = gs[i];
  const float ei = exp2_hw(gi);
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

  // ---- Y^T += X^T L'^T over 32-token k-steps; slots 0..3 carry tokens
  //      32kj + 4lq + r and slots 4..7 tokens 32kj + 16 + 4lq + r.
  const float Dh = Dv[h];
#pragma unroll
  for (int kj = 0; kj < T / 32; ++kj) {
    if (2 * kj <= ib) {
      float v[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int jb = 2 * kj + half;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = 16 * jb + 4 * lq + r;
          float w = cb[jb][r] * exp2_hw(gi - gs[j]) * ds[j];
          if (j == i) w += Dh;
          v[4 * half + r] = (jb <= ib && j <= i) ? w : 0.0f;
        }
      }
      uint32_t lh4[4], ll4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) split_bf16(v[2 * k], v[2 * k + 1], lh4[k], ll4[k]);
      const u32x4 lh = make_u32x4(lh4), ll = make_u32x4(ll4);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        const int off = (16 * pb + lr) * XS + 32 * kj + 4 * lq;
        const u32x2 a0 = *(const u32x2*)(xT + off);
        const u32x2 a1 = *(const u32x2*)(xT + off + 16);
        const u32x4 xa = (u32x4){a0[0], a0[1], a1[0], a1[1]};
        yacc[pb] = mfma_bf16(xa, lh, yacc[pb]);
        yacc[pb] = mfma_bf16(xa, ll, yacc[pb]);
      }
    }
  }

  if (i < nvalid) {
    const size_t off = (((size_t)b * L + t0 + i) * H + h) * kHeadDim + 4 * lq;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
  }
}

// ---------------------------------------------------------------- fp32 path
// k-map over the state index n for v_mfma_f32_16x16x4_f32: step (u, v)
// gives lane group lq the index 16u + 4lq + v; over tokens j: step (jb, r)
// gives 16jb + 4lq + r, which is exactly the j of accumulator element r.
template <int T, int N, bool YBF16>
__global__ __launch_bounds__(256) void compute_out_f32(
    const float* __restrict__ x, const float* __restrict__ Bm,
    const float* __restrict__ Cm, const float* __restrict__ dt_t,
    const float* __restrict__ g, const float* __restrict__ states,
    const float* __restrict__ Dv, void* __restrict__ y, int L, int H, int G,
    int nc) {
  constexpr int NQ = T / 64;
  constexpr int XS = T + 4;   // xT row stride (floats)
  constexpr int KU = N / 16;  // groups of four k-steps over n
  constexpr int NJB = T / 16;
  __shared__ __attribute__((aligned(16))) float xT[64 * XS];
  __shared__ float gs[T], ds[T];

  const OutTile tile = decode_tile(blockIdx.x, H, NQ, nc);
  const int h = tile.h, q = tile.q, c = tile.c, b = tile.b;
  const int grp = h / (H / G);
  const int t0 = c * T;
  const int nvalid = min(T, L - t0);
  const int bh_idx = b * H + h;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int ib = 4 * q + wave;
  const int i = 16 * ib + lr;

  {
    const int pq = tid & 15, xtb = tid >> 4;
    for (int it = 0; it <= q; ++it) {
      f32x4 xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 4 * (xtb + 16 * it) + r;
        xr[r] = t < nvalid
            ? *(const f32x4*)(x + (((size_t)b * L + t0 + t) * H + h) * kHeadDim + 4 * pq)
            : (f32x4){0, 0, 0, 0};
      }
      const int tcol = 4 * (xtb + 16 * it);
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *(f32x4*)(xT + (4 * pq + e) * XS + tcol) = (f32x4){xr[0][e], xr[1][e], xr[2][e], xr[3][e]};
    }
    for (int t = tid; t < T; t += 256) {
      const bool ok = t < nvalid;
      gs[t] = ok ? g[(size_t)bh_idx * L + t0 + t] : 0.0f;
      ds[t] = ok ? dt_t[(size_t)bh_idx * L + t0 + t] : 0.0f;
    }
  }

  f32x4 cf[KU];
  {
    const bool ok = i < nvalid;
    const float* crow = Cm + (((size_t)b * L + t0 + i) * G + grp) * N + 4 * lq;
#pragma unroll
    for (int u = 0; u < KU; ++u) cf[u] = ok ? *(const f32x4*)(crow + 16 * u) : (f32x4){0, 0, 0, 0};
  }

  f32x4 cb[NJB];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    cb[jb] = (f32x4){0, 0, 0, 0};
    if (jb <= ib) {
      const int j = 16 * jb + lr;
      const bool ok = j < nvalid;
      const float* brow = Bm + (((size_t)b * L + t0 + j) * G + grp) * N + 4 * lq;
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const f32x4 bv = ok ? *(const f32x4*)(brow + 16 * u) : (f32x4){0, 0, 0, 0};
#pragma unroll
        for (int v = 0; v < 4; ++v) cb[jb] = mfma_f32(bv[v], cf[u][v], cb[jb]);
      }
    }
  }

  f32x4 yacc[4];
  const float* S = states + ((size_t)bh_idx * nc + c) * kHeadDim * N + 4 * lq;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) {
    yacc[pb] = (f32x4){0, 0, 0, 0};
    const float* srow = S + (size_t)(16 * pb + lr) * N;
#pragma unroll
    for (int u = 0; u < KU; ++u) {
      const f32x4 sv = *(const f32x4*)(srow + 16 * u);
#pragma unroll
      for (int v = 0; v < 4; ++v) yacc[pb] = mfma_f32(sv[v], cf[u][v], yacc[pb]);
    }
  }
  __syncthreads();

  const float gi = gs[i];
  const float ei = exp2_hw(gi);
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

  const float Dh = Dv[h];
#pragma unroll
  for (int jb = 0; jb < NJB; ++jb) {
    if (jb <= ib) {
      float w[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * jb + 4 * lq + r;
        float v = cb[jb][r] * exp2_hw(gi - gs[j]) * ds[j];
        if (j == i) v += Dh;
        w[r] = (j <= i) ? v : 0.0f;
      }
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) {
        const f32x4 xv = *(const f32x4*)(xT + (16 * pb + lr) * XS + 16 * jb + 4 * lq);
#pragma unroll
        for (int r = 0; r < 4; ++r) yacc[pb] = mfma_f32(xv[r], w[r], yacc[pb]);
      }
    }
  }

  if (i < nvalid) {
    const size_t off = (((size_t)b * L + t0 + i) * H + h) * kHeadDim + 4 * lq;
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
  }
}

// ------------------------------------------------------------- launching
template <bool BF16, int T, int N, bool YBF16>
int launch_t(const void* x, const void* B, const void* C, const float* dt_t,
             const float* g, const float* states, const float* D, void* y,
             const Shape& s, hipStream_t st) {
  const int nc = (int)s.nchunks();
  const unsigned blocks = (unsigned)(s.batch * nc * (T / 64) * s.nheads);
  const int L = (int)s.seqlen, H = (int)s.nheads, G = (int)s.ngroups;
  using E = typename In<BF16>::T;
  if constexpr (BF16) {
    hipLaunchKernelGGL((compute_out_bf16<T, N, YBF16>), dim3(blocks), dim3(256), 0, st,
                       (const E*)x, (const E*)B, (const E*)C, dt_t, g, states, D, y, L,
                       H, G, nc);
  } else {
    hipLaunchKernelGGL((compute_out_f32<T, N, YBF16>), dim3(blocks), dim3(256), 0, st,
                       (const E*)x, (const E*)B, (const E*)C, dt_t, g, states, D, y, L,
                       H, G, nc);
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
  hipStream_t st = (hipStream_t)stream;
  if (bf16_in) return launch_chunk<true>(x, B, C, dt_t, g, states, D, y, bf16_out, s, st);
  return launch_chunk<false>(x, B, C, dt_t, g, states, D, y, bf16_out, s, st);
}

}  // namespace ssd

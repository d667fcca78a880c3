// Stages 2 and 3 in one pass, for fp32 inputs with many (batch, head) pairs.
//
// For each (b, h) the chunks are visited in order and the state is carried
// in matrix-core accumulators from one chunk to the next:
//   states[b,h,c] = S_c                                  (state entering chunk c)
//   Y_c = 2^{g_i} (C S_c^T) + L' X + D_h X               (stage 3, as in compute_out)
//   S_{c+1} = 2^{g_last} S_c + sum_t 2^{g_last - g_t} dt_t x_t B_t^T
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile": the recurrence of "Kernel 2: fwd_pass_state" and the output of
// "Kernel 3: compute_out, the Fused Output Kernel" with sections "Step 2" and
// "Step 3").  The pages run them as two kernels with the states between them
// in memory; when the batch holds enough (b, h) pairs to fill the chip one
// sequential walk per pair is parallel enough, and fusing the two saves the
// second read of x and the read of every state back from HBM: per (b, c, h)
// x is read once, B and C once per head pair, and y and S_c are written.
//
// MI355X design (fp32 values on bf16 matrix instructions, three-term exact
// splits and six products per pair as in compute_out_f32s: fp32 accuracy).
// Two kernels, both with persistent workgroups that take (b, head pair)
// work items with a stride of the grid size, so that at any moment the
// workgroups of one XCD work on consecutive pairs -- the heads of a group --
// and share B and C in that XCD's L2; both prefetch a step's operands two
// steps ahead into one of two register sets, and both run 8 waves (two per
// SIMD) because their LDS admits one workgroup per CU.
// * fused_pair_f32 (groups of an even number of heads): both heads of a pair
//   at once, every wave owning 16 state rows of one head; see its comment.
// * fused_state_out_f32 (odd group sizes: one head per work item): four
//   waves compute the output by query rows as compute_out_f32s does, four
//   carry the state rows; x, B and S_c pass through LDS as bf16 planes.
//   The state waves hold S transposed in accumulators: lane (r, q) of block
//   nb holds S[16w + r][16 nb + 4q + 0..3], the layout both a 16-byte store
//   of S_c and its bf16 planes want.  The update's operands are B^T
//   (transposed LDS reads of the B planes) and X' = w o x, where the x
//   fragment of the output's LDS reads is rebuilt in fp32 (the three planes
//   sum to x exactly), scaled by w_t = dt_t 2^{g_last - g_t} <= dt_t and
//   split again.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

#include <type_traits>

namespace ssd {
namespace {

constexpr uint32_t kPastRange = 0x7FFFFFF0u;
constexpr int kThreads = 512;

template <bool YBF16>
__device__ __forceinline__ void store_y(void* y, size_t off, f32x4 v) {
  if constexpr (YBF16) {
    *(u32x2*)((uint16_t*)y + off) = (u32x2){pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
  } else {
    *(f32x4*)((float*)y + off) = v;
  }
}

// the six products of a split pair: acc += a * b to fp32 accuracy
__device__ __forceinline__ f32x4 mfma6(const u32x4 (&a)[3], const u32x4 (&b)[3], f32x4 acc) {
  acc = mfma_bf16(a[0], b[0], acc);
  acc = mfma_bf16(a[0], b[1], acc);
  acc = mfma_bf16(a[1], b[0], acc);
  acc = mfma_bf16(a[0], b[2], acc);
  acc = mfma_bf16(a[1], b[1], acc);
  acc = mfma_bf16(a[2], b[0], acc);
  return acc;
}

// eight consecutive fp32 values split into three bf16 fragments
__device__ __forceinline__ void split8(const f32x4& v0, const f32x4& v1, u32x4 (&f)[3]) {
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    uint32_t h, m, l;
    split3_bf16(v0[2 * q], v0[2 * q + 1], h, m, l);
    f[0][q] = h; f[1][q] = m; f[2][q] = l;
    split3_bf16(v1[2 * q], v1[2 * q + 1], h, m, l);
    f[0][2 + q] = h; f[1][2 + q] = m; f[2][2 + q] = l;
  }
}

// Work decode: pair `it` of (b, head pair), head q of the pair.
struct Step {
  int b, c, h, grp, q;
};

// T = 64-token chunks, N = 64 state columns, HB heads (1 or 2) per pair.
// Waves 0-3 compute the output (wave w: query rows 16w..16w+15), waves 4-7
// carry the state (wave 4+w: state rows 16w..16w+15), so each SIMD runs one
// wave of each kind; all 8 stage the step's tiles into LDS.
template <int HB, bool YBF16>
__global__ __launch_bounds__(kThreads) void fused_state_out_f32(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ Cm,
    const float* __restrict__ dt_t, const float* __restrict__ g, const float* __restrict__ Dv,
    const float* __restrict__ init, float* __restrict__ states, float* __restrict__ final_state,
    void* __restrict__ y, int L, int H, int G, int nc, int pairs) {
  constexpr int T = 64, N = 64, NIB = 4, KN = N / 32;
  constexpr int XS = 80;                 // x plane row stride (bf16)
  constexpr int BS = 80;                 // B plane row stride (bf16)
  constexpr int SS = N + 8;              // state plane row stride (bf16)
  constexpr int XU = T * 16 / kThreads;  // 16-byte x units per thread
  constexpr int BU = T * (N / 4) / kThreads;
  constexpr int NE = NIB;
  static_assert(HB == 1 || HB == 2, "one or two heads per pair");
  static_assert(XU >= 1 && BU >= 1, "tile split");
  __shared__ __attribute__((aligned(16))) uint16_t xs[3][T * XS];
  __shared__ __attribute__((aligned(16))) uint16_t bp[3][T * BS];
  __shared__ __attribute__((aligned(16))) uint16_t ss[3][64 * SS];
  __shared__ __attribute__((aligned(16))) float gs[T], ds[T];
  __shared__ __attribute__((aligned(16))) float cw[4][32];

  const int nwg = gridDim.x;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  if (wg >= pairs) return;
  const int mine = (pairs - 1 - wg) / nwg + 1;   // pairs of this workgroup
  const int nsteps = mine * nc * HB;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const bool ywave = __builtin_amdgcn_readfirstlane(wave) < 4;   // output or state role
  const int w4 = wave & 3;
  const int hpg = H / G, npr = H / HB;
  const uint32_t xbytes = (uint32_t)L * H * kHeadDim * 4;
  const uint32_t bcbytes = (uint32_t)L * G * N * 4;
  const rsrc_t drs = make_rsrc(Dv, (uint32_t)H * 4);
  const int ib = w4, i = 16 * ib + lr;        // output waves: this lane's query row
  const int p = 16 * w4 + lr;                 // state waves: this lane's state row

  auto decode = [&](int k) {
    Step st;
    st.q = k % HB;
    k /= HB;
    st.c = k % nc;
    const int it = wg + (k / nc) * nwg;
    st.b = it / npr;
    st.h = (it % npr) * HB + st.q;
    st.grp = st.h / hpg;
    return st;
  };

  struct Regs {
    f32x4 x[XU];
    f32x4 bt[BU];       // the chunk's B tile (first head of a pair only)
    f32x4 cr[2 * KN];   // output waves: this lane's C row (first head of a pair only)
    float gd, dh;
  };
  constexpr int NLOAD = XU + BU + 2 * KN + 2;
  struct Src {
    rsrc_t xr, br, crr, gdr;
    uint32_t xo[XU], bo[BU], co, gdo;
    int h;
  };
  auto prepare = [&](int k, Src& sc) {
    const bool live = k < nsteps;
    const Step st = decode(live ? k : 0);
    const bool first = live && st.q == 0;
    sc.xr = make_rsrc(x + (size_t)st.b * L * H * kHeadDim, live ? xbytes : 0u);
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + kThreads * u, row = e >> 4, c4 = e & 15;
      sc.xo[u] = ((uint32_t)(st.c * T + row) * H + st.h) * (kHeadDim * 4) + 16 * c4;
    }
    sc.br = make_rsrc(Bm + (size_t)st.b * L * G * N, first ? bcbytes : 0u);
    sc.crr = make_rsrc(Cm + (size_t)st.b * L * G * N, first && ywave ? bcbytes : 0u);
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int e = tid + kThreads * u, row = e / (N / 4), c4 = e % (N / 4);
      sc.bo[u] = ((uint32_t)(st.c * T + row) * G + st.grp) * (N * 4) + 16 * c4;
    }
    sc.co = ((uint32_t)(st.c * T + i) * G + st.grp) * (N * 4) + 32 * lq;
    const bool wave_g = __builtin_amdgcn_readfirstlane(wave) == 0;
    sc.gdr = make_rsrc((wave_g ? g : dt_t) + ((size_t)st.b * H + st.h) * L,
                       live ? (uint32_t)L * 4 : 0u);
    sc.gdo = tid < 2 * T ? 4 * (uint32_t)(st.c * T + (tid % T)) : kPastRange;
    sc.h = st.h;
  };
  auto issue_slot = [&](int j, const Src& sc, Regs& r) {
    if (j < XU) {
      r.x[j] = load_f32x4(sc.xr, sc.xo[j]);
    } else if (j < XU + BU) {
      r.bt[j - XU] = load_f32x4(sc.br, sc.bo[j - XU]);
    } else if (j < XU + BU + 2 * KN) {
      const int jj = j - XU - BU;
      if (ywave) r.cr[jj] = load_f32x4(sc.crr, sc.co + 128 * (jj >> 1) + 16 * (jj & 1));
    } else if (j == XU + BU + 2 * KN) {
      r.gd = load_f32(sc.gdr, sc.gdo);
    } else {
      if (ywave) r.dh = load_f32(drs, 4 * sc.h);
    }
  };

  // state waves: each head's state, S[p][16 nb + 4 lq + rr] in sacc[q][nb][rr]
  f32x4 sacc[HB][N / 16];
  // output waves: C fragments of this lane's query row (k = 32 kk + 8 lq + e)
  // and (C B^T)[i][16 jb + 4 lq + rr] in cb[jb][rr], jb <= ib
  u32x4 cf[KN][3];
  f32x4 cb[NE];
#pragma unroll
  for (int e = 0; e < NE; ++e) cb[e] = (f32x4){0, 0, 0, 0};

  Regs ra, rb;
  {
    Src sc;
    prepare(0, sc);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, ra);
    prepare(1, sc);
#pragma unroll
    for (int j = 0; j < NLOAD; ++j) issue_slot(j, sc, rb);
  }

  auto body = [&](auto qtag, int k, Regs& r) {
    constexpr int Q = decltype(qtag)::value;
    const Step st = decode(k);
    const size_t hrow = (size_t)st.b * H + st.h;
    const int t0 = st.c * T;
    const int nt = min(T, L - t0);
    // a pair's walk starts from the initial state (or zero)
    if (!ywave && st.c == 0) {
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        sacc[Q][nb] = init ? *(const f32x4*)(init + hrow * kHeadDim * N + (size_t)p * N +
                                             16 * nb + 4 * lq)
                           : (f32x4){0, 0, 0, 0};
    }
    __syncthreads();  // the previous step's LDS reads are done

    // ---- commit: x planes, g, dt; B planes and C fragments at a pair's
    //      first head; S_c to the states and to its planes
#pragma unroll
    for (int u = 0; u < XU; ++u) {
      const int e = tid + kThreads * u, row = e >> 4, c4 = e & 15;
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(r.x[u][0], r.x[u][1], h0, m0, l0);
      split3_bf16(r.x[u][2], r.x[u][3], h1, m1, l1);
      const int o = row * XS + 4 * c4;
      *(u32x2*)(xs[0] + o) = (u32x2){h0, h1};
      *(u32x2*)(xs[1] + o) = (u32x2){m0, m1};
      *(u32x2*)(xs[2] + o) = (u32x2){l0, l1};
    }
    if (Q == 0) {
#pragma unroll
      for (int u = 0; u < BU; ++u) {
        const int e = tid + kThreads * u, row = e / (N / 4), c4 = e % (N / 4);
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(r.bt[u][0], r.bt[u][1], h0, m0, l0);
        split3_bf16(r.bt[u][2], r.bt[u][3], h1, m1, l1);
        const int o = row * BS + 4 * c4;
        *(u32x2*)(bp[0] + o) = (u32x2){h0, h1};
        *(u32x2*)(bp[1] + o) = (u32x2){m0, m1};
        *(u32x2*)(bp[2] + o) = (u32x2){l0, l1};
      }
      if (ywave) {
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) split8(r.cr[2 * kk], r.cr[2 * kk + 1], cf[kk]);
      }
    }
    if (tid < T) {
      gs[tid] = r.gd;
    } else if (tid < 2 * T) {
      ds[tid - T] = r.gd;
    }
    if (!ywave) {
      float* dst = states + (hrow * nc + st.c) * kHeadDim * N + (size_t)p * N + 4 * lq;
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        *(f32x4*)(dst + 16 * nb) = sacc[Q][nb];
        uint32_t h0, m0, l0, h1, m1, l1;
        split3_bf16(sacc[Q][nb][0], sacc[Q][nb][1], h0, m0, l0);
        split3_bf16(sacc[Q][nb][2], sacc[Q][nb][3], h1, m1, l1);
        const int o = p * SS + 16 * nb + 4 * lq;
        *(u32x2*)(ss[0] + o) = (u32x2){h0, h1};
        *(u32x2*)(ss[1] + o) = (u32x2){m0, m1};
        *(u32x2*)(ss[2] + o) = (u32x2){l0, l1};
      }
    }
    const float Dh = r.dh;
    Src nxt;
    prepare(k + 2, nxt);
    __syncthreads();

    if (ywave) {
      // ---- C B^T blocks of this wave's query rows, once per chunk
      if (Q == 0) {
#pragma unroll
        for (int jb = 0; jb < NIB; ++jb) {
          if (jb <= ib) {
            f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
            for (int kk = 0; kk < KN; ++kk) {
              const int o = (16 * jb + lr) * BS + 32 * kk + 8 * lq;
              const u32x4 bf[3] = {*(const u32x4*)(bp[0] + o), *(const u32x4*)(bp[1] + o),
                                   *(const u32x4*)(bp[2] + o)};
              acc = mfma6(bf, cf[kk], acc);
            }
            cb[jb] = acc;
          }
        }
      }

      // ---- output: Y^T = S C^T scaled by 2^{g_i}, plus X^T L'^T
      f32x4 yacc[4];
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < KN; ++kk) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) {
          if (4 * kk + pb < NLOAD) issue_slot(4 * kk + pb, nxt, r);
          const int off = (16 * pb + lr) * SS + 32 * kk + 8 * lq;
          const u32x4 sa[3] = {*(const u32x4*)(ss[0] + off), *(const u32x4*)(ss[1] + off),
                               *(const u32x4*)(ss[2] + off)};
          yacc[pb] = mfma6(sa, cf[kk], yacc[pb]);
        }
      }
#pragma unroll
      for (int j = 4 * KN; j < NLOAD; ++j) issue_slot(j, nxt, r);
      const float gi = gs[i];
      const float ei = exp2_hw(gi);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) yacc[pb] *= ei;

      const bool row_in = t0 + i < L;
#pragma unroll
      for (int s = 0; s < NE / 2; ++s) {
        if (2 * s <= ib) {
          const int e0 = 2 * s, e1 = 2 * s + 1;
          float v[8];
          if (2 * s + 2 <= ib) {
            // a block below the diagonal block: 2^{g_i - g_j} factored
            // through the block's last token, both factors at most 1
            const float ge = gs[32 * s + 31];
            const int jl = 32 * s + (lane & 31);
            const float cl = exp2_hw(ge - gs[jl]) * ds[jl];
            if (lane < 32) cw[w4][lane] = cl;
            const float ai = row_in ? exp2_hw(gi - ge) : 0.0f;
            const f32x4 c0 = *(const f32x4*)(&cw[w4][4 * lq]);
            const f32x4 c1 = *(const f32x4*)(&cw[w4][16 + 4 * lq]);
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
      if (row_in) {
        const size_t off = (((size_t)st.b * L + t0 + i) * H + st.h) * kHeadDim + 4 * lq;
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) store_y<YBF16>(y, off + 16 * pb, yacc[pb]);
      }
    } else {
      // ---- state: S <- 2^{g_last} S + B^T X', X' = w o x over this wave's rows
      const float glast = gs[nt - 1];
      const float dec = exp2_hw(glast);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) sacc[Q][nb] *= dec;
#pragma unroll
      for (int s = 0; s < T / 32; ++s) {
        // k slot e of lane group lq carries token 32 s + 16 (e / 4) + 4 lq + e % 4
        const int xo = (32 * s + 4 * lq + (lr >> 2)) * XS + 4 * (lr & 3) + 16 * w4;
        u32x4 xa[3];
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          const u32x2 a0 = lds_read_tr16(xs[q] + xo);
          const u32x2 a1 = lds_read_tr16(xs[q] + xo + 16 * XS);
          xa[q] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
        }
        const f32x4 g0 = *(const f32x4*)(&gs[32 * s + 4 * lq]);
        const f32x4 g1 = *(const f32x4*)(&gs[32 * s + 16 + 4 * lq]);
        const f32x4 d0 = *(const f32x4*)(&ds[32 * s + 4 * lq]);
        const f32x4 d1 = *(const f32x4*)(&ds[32 * s + 16 + 4 * lq]);
        float xv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int wd = e >> 1;
          const float hv = (e & 1) ? bf16_hi(xa[0][wd]) : bf16_lo(xa[0][wd]);
          const float mv = (e & 1) ? bf16_hi(xa[1][wd]) : bf16_lo(xa[1][wd]);
          const float lv = (e & 1) ? bf16_hi(xa[2][wd]) : bf16_lo(xa[2][wd]);
          const float gt = e < 4 ? g0[e] : g1[e - 4];
          const float dt = e < 4 ? d0[e] : d1[e - 4];
          xv[e] = ((hv + mv) + lv) * (dt * exp2_hw(glast - gt));
        }
        u32x4 xp[3];
        split8((f32x4){xv[0], xv[1], xv[2], xv[3]}, (f32x4){xv[4], xv[5], xv[6], xv[7]}, xp);
        const int bo = (32 * s + 4 * lq + (lr >> 2)) * BS + 4 * (lr & 3);
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb) {
          if (4 * s + nb < NLOAD) issue_slot(4 * s + nb, nxt, r);
          u32x4 bt[3];
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            const u32x2 a0 = lds_read_tr16(bp[q] + bo + 16 * nb);
            const u32x2 a1 = lds_read_tr16(bp[q] + bo + 16 * BS + 16 * nb);
            bt[q] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
          }
          sacc[Q][nb] = mfma6(bt, xp, sacc[Q][nb]);
        }
      }
#pragma unroll
      for (int j = 4 * (T / 32); j < NLOAD; ++j) issue_slot(j, nxt, r);
      if (st.c == nc - 1 && final_state) {
        float* dst = final_state + hrow * kHeadDim * N + (size_t)p * N + 4 * lq;
#pragma unroll
        for (int nb = 0; nb < N / 16; ++nb) *(f32x4*)(dst + 16 * nb) = sacc[Q][nb];
      }
    }
  };

  // steps alternate between the two register sets; with two heads per
  // pair the even steps are the first head, the odd ones the second
  for (int k = 0; k < nsteps; k += 2) {
    body(std::integral_constant<int, 0>{}, k, ra);
    if (k + 1 < nsteps) body(std::integral_constant<int, HB - 1>{}, k + 1, rb);
  }
}

// Head-pair form (8 waves, two per SIMD), for groups of an even number of
// heads: both heads of a pair at once, waves 4q..4q+3 on head q, wave 4q + w
// owning rows p = 16w..16w+15 of that head's state and of its Y^T[p][i]
// over every token i of the chunk, so the waves carry equal work.
// * The state stays in accumulators, S[p][16 nb + 4 lq + rr] in lane (p, lq),
//   and feeds C S^T directly: its k slots follow that layout, n = 32 kk +
//   16 (e / 4) + 4 lq + e % 4, and C is staged with its columns in that
//   order.
// * x never passes through LDS: each lane loads the 16 (token, p) values its
//   fragments carry (token 32 s + 16 (e / 4) + 4 lq + e % 4, column p),
//   splits them for X^T L'^T and scales them by w_t for the state update.
// * B and C are staged once per chunk for both heads.  Each of the ten lower
//   16x16 blocks of C B^T is formed once, by one wave (two for waves 0 and 1,
//   one for the others), which turns it into L' of both heads in LDS.
// * Addresses: every per-step part is uniform and goes into the buffer
//   descriptors (scalar arithmetic); the lanes' offsets are loop-invariant.
//   The ranges end at the sequence, so rows past its end read zero and their
//   stores are dropped.
// * Each product's LDS fragments are read one group ahead of it (scheduling
//   barriers keep the reads early), so a wave waits on LDS once per group
//   of products with the next group's reads already in flight.
template <bool YBF16>
__global__ __launch_bounds__(512) void fused_pair_f32(
    const float* __restrict__ x, const float* __restrict__ Bm, const float* __restrict__ Cm,
    const float* __restrict__ dt_t, const float* __restrict__ g, const float* __restrict__ Dv,
    const float* __restrict__ init, float* __restrict__ states, float* __restrict__ final_state,
    void* __restrict__ y, int L, int H, int G, int nc, int pairs) {
  constexpr int NT = 512;
  constexpr int T = 64, N = 64, NIB = 4, KN = N / 32;
  constexpr int BS = 80;                 // B plane row stride (bf16)
  constexpr int CS = N + 16;             // C plane row stride (bf16), columns in k-slot order
  // (160 bytes: 16-byte reads of 16 rows x 4 column groups then hit no bank
  // twice, where 144 took two passes)
  constexpr int LS = T + 8;              // L' plane row stride (bf16), columns in k-slot order
  constexpr int BU = T * 16 / NT;        // 16-byte units of the B and C tiles per thread
  constexpr int XV = 16;                 // x values per lane
  constexpr uint32_t kYB = YBF16 ? 2 : 4;
  constexpr uint32_t kStateBytes = kHeadDim * N * 4;
  __shared__ __attribute__((aligned(16))) uint16_t bp[3][T * BS];
  __shared__ __attribute__((aligned(16))) uint16_t cp[3][T * CS];
  __shared__ __attribute__((aligned(16))) uint16_t bq[3][T * CS];   // B, columns in k-slot order
  __shared__ __attribute__((aligned(16))) uint16_t lp[2][3][T * LS];
  __shared__ __attribute__((aligned(16))) float gs[2][T], ds[2][T];
  __shared__ __attribute__((aligned(16))) float ws[2][T];   // w_t = dt_t 2^{g_last - g_t}

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
  const uint32_t brow = (uint32_t)G * N * 4;          // bytes per token of B and C
  const rsrc_t drs = make_rsrc(Dv, (uint32_t)H * 4);
  const int p = 16 * w + lr;                  // this lane's state row (operand row)

  // loop-invariant lane offsets (bytes) from each step's descriptor bases
  const uint32_t xo_lane = 4 * (uint32_t)p + 4 * (uint32_t)lq * xrow;
  uint32_t bo_lane[BU];
#pragma unroll
  for (int u = 0; u < BU; ++u) {
    const int e = tid + NT * u;
    bo_lane[u] = (uint32_t)(e >> 4) * brow + 16 * (e & 15);
  }
  const uint32_t gd_lane = 4 * (uint32_t)(tid & 63);
  const uint32_t so_lane = ((uint32_t)p * N + 4 * lq) * 4;

  auto kpos = [](int c) { return (c & ~31) + 8 * ((c >> 2) & 3) + 4 * ((c >> 4) & 1) + (c & 3); };
  // uniform part of the token of x value v (v = 8 s + e): 32 s + 16 (e / 4) + e % 4
  auto xtok_u = [](int v) { return 32 * (v >> 3) + 16 * ((v >> 2) & 1) + (v & 3); };

  // this wave's blocks (ib, jb) of C B^T: waves 0-3 (3, 3-w), waves 4-6
  // (2, 6-w), wave 7 (1, 0); waves 0 and 1 also (w, w)
  const int nblk = wave < 2 ? 2 : 1;
  auto blk_i = [&](int sl) { return sl == 1 ? wave : (wave < 4 ? 3 : (wave < 7 ? 2 : 1)); };
  auto blk_j = [&](int sl) {
    return sl == 1 ? wave : (wave < 4 ? 3 - wave : (wave < 7 ? 6 - wave : 0));
  };

  // Work steps are (pair, chunk), chunks fastest.  A cursor walks them in
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
    float xv[XV];
    f32x4 bt[BU], ct[BU];
    float gv, dv, dh[2];   // g and dt (waves 0 and 2: heads 0 and 1), D_h of both heads
    StepP st;              // the step these registers were loaded for
  };
  constexpr int NLOAD = XV + 2 * BU + 4;
  struct Src {
    rsrc_t xr, br, crr, gr, dr;
    int h0;
  };
  auto prepare = [&](const StepP& st, Src& sc) {
    const int t0 = st.c * T, h = st.h0 + hq;
    const uint32_t rows = (uint32_t)(L - t0);
    sc.xr = make_rsrc(x + (((size_t)st.b * L + t0) * H + h) * kHeadDim,
                      st.live ? (rows * H - h) * (kHeadDim * 4) : 0u);
    const size_t bcb = (((size_t)st.b * L + t0) * G + st.grp) * N;
    const uint32_t bcr = st.live ? (rows * G - st.grp) * (N * 4) : 0u;
    sc.br = make_rsrc(Bm + bcb, bcr);
    sc.crr = make_rsrc(Cm + bcb, bcr);
    // g and dt of both heads: wave 0 head 0, wave 2 head 1
    const size_t gro = ((size_t)st.b * H + st.h0 + (wave >> 1)) * L + t0;
    const uint32_t grr = st.live && (wave == 0 || wave == 2) ? rows * 4 : 0u;
    sc.gr = make_rsrc(g + gro, grr);
    sc.dr = make_rsrc(dt_t + gro, grr);
    sc.h0 = st.h0;
  };
  auto issue_slot = [&](int j, const Src& sc, Regs& r) {
    if (j < XV) {
      r.xv[j] = load_f32(sc.xr, xo_lane + (uint32_t)xtok_u(j) * xrow);
    } else if (j < XV + BU) {
      r.bt[j - XV] = load_f32x4(sc.br, bo_lane[j - XV]);
    } else if (j < XV + 2 * BU) {
      r.ct[j - XV - BU] = load_f32x4(sc.crr, bo_lane[j - XV - BU]);
    } else if (j == XV + 2 * BU) {
      r.gv = load_f32(sc.gr, gd_lane);
    } else if (j == XV + 2 * BU + 1) {
      r.dv = load_f32(sc.dr, gd_lane);
    } else {
      const int q = j - XV - 2 * BU - 2;
      r.dh[q] = load_f32(drs, 4 * (sc.h0 + q));
    }
  };
  auto store3 = [](uint16_t* p0, uint16_t* p1, uint16_t* p2, int o, const f32x4& v) {
    uint32_t h0, m0, l0, h1, m1, l1;
    split3_bf16(v[0], v[1], h0, m0, l0);
    split3_bf16(v[2], v[3], h1, m1, l1);
    *(u32x2*)(p0 + o) = (u32x2){h0, h1};
    *(u32x2*)(p1 + o) = (u32x2){m0, m1};
    *(u32x2*)(p2 + o) = (u32x2){l0, l1};
  };

  f32x4 sacc[N / 16];   // S[p][16 nb + 4 lq + rr] of this wave's head
  f32x4 cbr[2];         // (B C^T)[16 jb + 4 lq + rr][16 ib + lr] of this wave's blocks

  // L' blocks that stay zero: (ib 0, jb 1) and (ib 2, jb 3), read as the
  // upper halves of 32-token k-steps on the diagonal
  for (int e = tid; e < 2 * 2 * 16 * 16; e += NT) {
    const int hh = e >> 9, blk = (e >> 8) & 1, r = (e >> 4) & 15, c = e & 15;
    const int i = blk == 0 ? r : 32 + r, j = blk == 0 ? 16 + c : 48 + c;
#pragma unroll
    for (int q = 0; q < 3; ++q) lp[hh][q][i * LS + kpos(j)] = 0;
  }

  Regs ra, rb;
  Cursor cur;
  cur.k = 0;
  cur.c = 0;
  cur.it = wg;
  at_pair(cur);
  cur.st.c = 0;
  cur.st.live = true;
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

  // Staging of a step from its registers: B and C planes, g and dt of both
  // heads, and S_c (the state entering the chunk, after the previous
  // chunk's update or from init_state) to the states.  It runs in the
  // previous step's last phase, which reads only the L' planes, so it
  // overlaps the other waves' X^T L'^T.
  auto commit = [&](const Regs& r) {
    const StepP st = r.st;
    const size_t hrow = (size_t)st.b * H + st.h0 + hq;
    if (st.c == 0) {
      // no initial state: an empty range, every load reads zero
      const rsrc_t ires = init ? make_rsrc(init + hrow * (kHeadDim * N), kStateBytes)
                               : make_rsrc(states, 0u);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) sacc[nb] = load_f32x4(ires, so_lane + 64 * nb);
    }
#pragma unroll
    for (int u = 0; u < BU; ++u) {
      const int e = tid + NT * u, row = e >> 4, c4 = e & 15;
      uint32_t h0, m0, l0, h1, m1, l1;
      split3_bf16(r.bt[u][0], r.bt[u][1], h0, m0, l0);
      split3_bf16(r.bt[u][2], r.bt[u][3], h1, m1, l1);
      const int ob = row * BS + 4 * c4, oq = row * CS + kpos(4 * c4);
      *(u32x2*)(bp[0] + ob) = (u32x2){h0, h1};
      *(u32x2*)(bp[1] + ob) = (u32x2){m0, m1};
      *(u32x2*)(bp[2] + ob) = (u32x2){l0, l1};
      *(u32x2*)(bq[0] + oq) = (u32x2){h0, h1};
      *(u32x2*)(bq[1] + oq) = (u32x2){m0, m1};
      *(u32x2*)(bq[2] + oq) = (u32x2){l0, l1};
      store3(cp[0], cp[1], cp[2], oq, r.ct[u]);
    }
    if (wave == 0 || wave == 2) {
      // g, dt and the state-update weight w of one head: lane = token;
      // tokens past the end read g = dt = 0, so w = 0
      const int hh = wave >> 1;
      const int nt = min(T, L - st.c * T);
      const int gl = __builtin_amdgcn_readlane(__float_as_int(r.gv), nt - 1);
      gs[hh][lane] = r.gv;
      ds[hh][lane] = r.dv;
      ws[hh][lane] = r.dv * exp2_hw(__int_as_float(gl) - r.gv);
    }
    const rsrc_t sres = make_rsrc(states + (hrow * nc + st.c) * (kHeadDim * N), kStateBytes);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[nb]), sres,
                                             so_lane + 64 * nb, 0, 0);
  };
  commit(ra);
  __syncthreads();

  // step k from the registers r (staged already); rn holds step k + 1
  auto body = [&](Regs& r, const Regs& rn, bool has_next) {
    const StepP st = r.st;
    const int h = st.h0 + hq;
    const int t0 = st.c * T;
    const int nt = min(T, L - t0);
    const size_t hrow = (size_t)st.b * H + h;
    // this lane's x values split into the X^T fragments
    u32x4 xa[2][3];
#pragma unroll
    for (int s = 0; s < 2; ++s)
      split8((f32x4){r.xv[8 * s], r.xv[8 * s + 1], r.xv[8 * s + 2], r.xv[8 * s + 3]},
             (f32x4){r.xv[8 * s + 4], r.xv[8 * s + 5], r.xv[8 * s + 6], r.xv[8 * s + 7]},
             xa[s]);
    const float Dh[2] = {r.dh[0], r.dh[1]};
    Src nxt;
    prepare(cur.st, nxt);
    r.st = cur.st;
    advance(cur);
    // B, C, g, dt and D of the step two ahead (their registers were staged
    // already); x follows once this step's x is consumed
#pragma unroll
    for (int j = XV; j < NLOAD; ++j) issue_slot(j, nxt, r);

    // ---- this wave's blocks of C B^T (A = B rows j, B = C rows i, k slots
    //      in accumulator order) and from them L' of both heads -> LDS; a
    //      block's fragments are all read before its products
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl < nblk) {
        const int ib = blk_i(sl), jb = blk_j(sl);
        u32x4 bf[KN][3], cf[KN][3];
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) {
          const int ob = (16 * jb + lr) * CS + 32 * kk + 8 * lq;
          const int oc = (16 * ib + lr) * CS + 32 * kk + 8 * lq;
#pragma unroll
          for (int q = 0; q < 3; ++q) {
            bf[kk][q] = *(const u32x4*)(bq[q] + ob);
            cf[kk][q] = *(const u32x4*)(cp[q] + oc);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = (f32x4){0, 0, 0, 0};
#pragma unroll
        for (int kk = 0; kk < KN; ++kk) acc = mfma6(bf[kk], cf[kk], acc);
        cbr[sl] = acc;
      }
    }
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl < nblk) {
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
          store3(lp[hh][0], lp[hh][1], lp[hh][2], i * LS + kpos(j0), v);
        }
      }
    }

    // ---- Y^T = S C^T, A = S from the accumulators (split), B = C rows; each
    //      row block's C fragments are read during the previous one's products
    f32x4 yacc[NIB];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) yacc[ib] = (f32x4){0, 0, 0, 0};
    auto c_frags = [&](int kk, int ib, u32x4 (&cf)[3]) {
      const int oc = (16 * ib + lr) * CS + 32 * kk + 8 * lq;
#pragma unroll
      for (int q = 0; q < 3; ++q) cf[q] = *(const u32x4*)(cp[q] + oc);
    };
    u32x4 cfr[2][3];
    c_frags(0, 0, cfr[0]);
#pragma unroll
    for (int kk = 0; kk < KN; ++kk) {
      u32x4 sf[3];
      split8(sacc[2 * kk], sacc[2 * kk + 1], sf);
#pragma unroll
      for (int ib = 0; ib < NIB; ++ib) {
        const int g = kk * NIB + ib;
        if (g + 1 < KN * NIB) c_frags((g + 1) / NIB, (g + 1) % NIB, cfr[(g + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        yacc[ib] = mfma6(sf, cfr[g & 1], yacc[ib]);
      }
    }
    const float* gsh = gs[hq];
    const float* wsh = ws[hq];
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) yacc[ib] *= exp2_hw(gsh[16 * ib + lr]);

    // ---- state: S <- 2^{g_last} S + B^T X', X' = w o x on this lane's tokens
    auto b_frags = [&](int s, int nb, u32x4 (&bt)[3]) {
      const int bo = (32 * s + 4 * lq + (lr >> 2)) * BS + 4 * (lr & 3) + 16 * nb;
#pragma unroll
      for (int q = 0; q < 3; ++q) {
        const u32x2 a0 = lds_read_tr16(bp[q] + bo);
        const u32x2 a1 = lds_read_tr16(bp[q] + bo + 16 * BS);
        bt[q] = (u32x4){a0[0], a0[1], a1[0], a1[1]};
      }
    };
    u32x4 btr[2][3];
    b_frags(0, 0, btr[0]);
    const float glast = gsh[nt - 1];
    const float dec = exp2_hw(glast);
#pragma unroll
    for (int nb = 0; nb < N / 16; ++nb) sacc[nb] *= dec;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const f32x4 w0 = *(const f32x4*)(&wsh[32 * s + 4 * lq]);
      const f32x4 w1 = *(const f32x4*)(&wsh[32 * s + 16 + 4 * lq]);
      f32x4 x0, x1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x0[e] = r.xv[8 * s + e] * w0[e];
        x1[e] = r.xv[8 * s + 4 + e] * w1[e];
      }
      u32x4 xp[3];
      split8(x0, x1, xp);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb) {
        const int g = s * (N / 16) + nb;
        if (g + 1 < 2 * (N / 16)) b_frags((g + 1) / (N / 16), (g + 1) % (N / 16), btr[(g + 1) & 1]);
        __builtin_amdgcn_sched_barrier(0);
        sacc[nb] = mfma6(btr[g & 1], xp, sacc[nb]);
      }
    }
    // x of the step two ahead, now that this step's x is consumed
#pragma unroll
    for (int j = 0; j < XV; ++j) issue_slot(j, nxt, r);
    if (st.c == nc - 1 && final_state) {
      const rsrc_t fres = make_rsrc(final_state + hrow * (kHeadDim * N), kStateBytes);
#pragma unroll
      for (int nb = 0; nb < N / 16; ++nb)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, sacc[nb]), fres,
                                               so_lane + 64 * nb, 0, 0);
    }
    __syncthreads();  // every wave's L' blocks are in LDS; B, C, g, dt reads are done

    // the next step's operands, while the other waves multiply by L'
    if (has_next) commit(rn);

    // ---- Y^T += X^T L'^T over the 32-token k-steps on or below the
    //      diagonal; rows past the end of the sequence fall outside the range
    const rsrc_t yres =
        make_rsrc((char*)y + (((size_t)st.b * L + t0) * H + h) * kHeadDim * kYB,
                  ((uint32_t)(L - t0) * H - h) * kHeadDim * kYB);
    uint16_t(*lph)[T * LS] = lp[hq];
    // the six (row block, k-step) pairs on or below the diagonal, in order
    constexpr int kIb[6] = {0, 1, 2, 2, 3, 3}, kS[6] = {0, 0, 0, 1, 0, 1};
    auto l_frags = [&](int g, u32x4 (&lf)[3]) {
      const int ol = (16 * kIb[g] + lr) * LS + 32 * kS[g] + 8 * lq;
#pragma unroll
      for (int q = 0; q < 3; ++q) lf[q] = *(const u32x4*)(lph[q] + ol);
    };
    u32x4 lfr[2][3];
    l_frags(0, lfr[0]);
#pragma unroll
    for (int ib = 0; ib < NIB; ++ib) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (2 * s <= ib) {
          const int g = ib == 0 ? 0 : (ib == 1 ? 1 : 2 * ib - 2 + s);
          if (g + 1 < 6) l_frags(g + 1, lfr[(g + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          yacc[ib] = mfma6(xa[s], lfr[g & 1], yacc[ib]);
        }
      }
      const uint32_t yo = ((uint32_t)(16 * ib + lr) * H * kHeadDim + p - lr + 4 * lq) * kYB;
      if constexpr (YBF16) {
        __builtin_amdgcn_raw_buffer_store_b64(
            (u32x2){pack_bf16(yacc[ib][0], yacc[ib][1]), pack_bf16(yacc[ib][2], yacc[ib][3])},
            yres, yo, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, yacc[ib]), yres, yo, 0,
                                               0);
      }
    }
    __syncthreads();  // the next step's operands are staged; this step's L' reads are done
  };

  for (int k = 0; k < nsteps; k += 2) {
    body(ra, rb, k + 1 < nsteps);
    if (k + 1 < nsteps) body(rb, ra, k + 2 < nsteps);
  }
}

template <int HB, bool YBF16>
int launch_hb(const float* x, const float* B, const float* C, const float* dt_t, const float* g,
              const float* D, const float* init, float* states, float* fin, void* y,
              const Shape& s, hipStream_t st) {
  // two heads per pair: the head-pair kernel; one: the output/state-wave kernel
  const void* kern = HB == 2 ? (const void*)fused_pair_f32<YBF16>
                             : (const void*)fused_state_out_f32<HB, YBF16>;
  const int threads = HB == 2 ? 512 : kThreads;
  static PerDeviceInt resident;
  const int slots = resident.get([&](int dev) { return resident_slots(kern, threads, dev); });
  if (slots <= 0) return (int)hipErrorInvalidDevice;
  const int pairs = (int)(s.batch * s.nheads / HB);
  const unsigned grid = (unsigned)(pairs < slots ? pairs : slots);
  if (HB == 2)
    hipLaunchKernelGGL((fused_pair_f32<YBF16>), dim3(grid), dim3(threads), 0, st, x, B, C, dt_t,
                       g, D, init, states, fin, y, (int)s.seqlen, (int)s.nheads, (int)s.ngroups,
                       (int)s.nchunks(), pairs);
  else
    hipLaunchKernelGGL((fused_state_out_f32<HB, YBF16>), dim3(grid), dim3(threads), 0, st, x,
                       B, C, dt_t, g, D, init, states, fin, y, (int)s.seqlen, (int)s.nheads,
                       (int)s.ngroups, (int)s.nchunks(), pairs);
  return (int)hipGetLastError();
}

// Heads per pair: two when the group size allows.
int heads_per_pair(const Shape& s) { return (s.nheads / s.ngroups) % 2 == 0 ? 2 : 1; }

// Whether the fused kernel takes this shape.
bool fused_applies(const Shape& s, bool bf16_in) {
  if (bf16_in || s.chunk != 64 || s.dstate != 64 || s.headdim != kHeadDim) return false;
  static PerDeviceInt cus_cache;
  int cus = cus_cache.get(query_cus);
  if (cus <= 0) cus = 256;
  // one sequential walk per pair: enough pairs to give every CU one
  return s.batch * s.nheads / heads_per_pair(s) >= cus;
}

int launch_fused(const float* x, const float* B, const float* C, const float* dt_t,
                 const float* g, const float* D, const float* init, float* states, float* fin,
                 void* y, bool bf16_out, const Shape& s, hipStream_t st) {
  if (heads_per_pair(s) == 2) {
    if (bf16_out) return launch_hb<2, true>(x, B, C, dt_t, g, D, init, states, fin, y, s, st);
    return launch_hb<2, false>(x, B, C, dt_t, g, D, init, states, fin, y, s, st);
  }
  if (bf16_out) return launch_hb<1, true>(x, B, C, dt_t, g, D, init, states, fin, y, s, st);
  return launch_hb<1, false>(x, B, C, dt_t, g, D, init, states, fin, y, s, st);
}

}  // namespace

int launch_state_and_out(const void* x, const void* B, const void* C, const float* dt_t,
                         const float* g, const float* D, const float* init_state, float* states,
                         float* final_state, void* y, bool bf16_in, bool bf16_out,
                         const Shape& s, void* stream) {
  if (fused_applies(s, bf16_in)) {
    clear_launch_error();
    return launch_fused((const float*)x, (const float*)B, (const float*)C, dt_t, g, D,
                        init_state, states, final_state, y, bf16_out, s, (hipStream_t)stream);
  }
  if (fused_bf16_applies(s, bf16_in))
    return launch_fused_bf16(x, B, C, dt_t, g, D, init_state, states, final_state, y, bf16_out,
                             s, stream);
  int err = launch_fwd_pass_state(x, B, dt_t, g, init_state, states, final_state, bf16_in, s,
                                  stream);
  if (err == 0)
    err = launch_compute_out(x, B, C, dt_t, g, states, D, y, bf16_in, bf16_out, s, stream);
  return err;
}

}  // namespace ssd

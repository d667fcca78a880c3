// Gated DeltaNet, chunked forward: the inter-chunk state pass (chunk_fwd_h)
// and the per-chunk output (chunk_fwd_o), as the Helion hackathon gallery
// describes them (its gated_deltanet_chunk_fwd_h and chunk_fwd_o entries).
// The state h is K x V per (batch, head); chunks have C = 64 tokens.  Per
// chunk, with g the chunk-local cumulative log-gate and g_last its value at
// the chunk's last (valid) token:
//   h_out[c] = h;   v_new = u - w h;   h = e^{g_last} h + k^T (e^{g_last - g} o v_new)
//   o = scale (e^{g} o (q h_out[c]) + causal(q k^T o e^{g_i - g_j}) v_new)
// w and u are the WY-transformed keys and values; they are inputs here.
//
// MI355X design (bf16 inputs; fp32 state and accumulation).
// chunk_fwd_h: one workgroup owns the state columns of one (b, h) v-tile of
// 16 NW columns and walks the chunks in order; wave w owns 16 columns, all
// K rows, as K/16 accumulator blocks H[K][v] (lane: column v, four
// consecutive K).  Both products of a chunk take an operand straight from
// accumulators:
//   v_new = u - w h: for lane group q the k-slots carry K = 32kk + 4q + 0..3
//     and 32kk + 16 + 4q + 0..3, exactly the rows two state blocks hold, so
//     the state (split bf16 hi + lo) is the B operand as it sits; w is read
//     from LDS as two 8-byte pieces per lane.
//   h += k^T v_gated: the v_new accumulator blocks hold, per lane, four
//     consecutive tokens of one column, again the k-slot map, so the gated
//     v_new (split hi + lo) is the B operand as it sits; k^T comes from the
//     LDS transpose read.
// So the sequential chain of a wave never leaves registers except for the
// stores.  The state and v_new are written with 16-byte stores after a
// per-wave transpose through LDS.  The w, k and u tiles of the next chunk
// are loaded into registers while the current one is processed, then staged
// into the other half of a double-buffered LDS tile set (one barrier per
// chunk).

#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr uint32_t kPastRange = 0x7FFFFFF0u;
constexpr int kGdnC = 64;    // tokens per chunk
constexpr int kTrS = 20;     // row stride (floats) of the per-wave transpose scratch

__device__ __forceinline__ int gdn_xcd_remap(int bid, int total) {
  if (total % 8) return bid;
  return (bid % 8) * (total / 8) + bid / 8;
}

// hi/lo bf16 split of eight fp32 values (slots 0..3 from a, 4..7 from b).
__device__ __forceinline__ void split8(const f32x4& a, const f32x4& b, u32x4& hi, u32x4& lo) {
  uint32_t h[4], l[4];
  split_bf16(a[0], a[1], h[0], l[0]);
  split_bf16(a[2], a[3], h[1], l[1]);
  split_bf16(b[0], b[1], h[2], l[2]);
  split_bf16(b[2], b[3], h[3], l[3]);
  hi = make_u32x4(h);
  lo = make_u32x4(l);
}

template <int K, int V, int NW, bool VBF16>
__global__ __launch_bounds__(64 * NW) void gdn_fwd_h_kernel(
    const uint16_t* __restrict__ kin, const uint16_t* __restrict__ win,
    const uint16_t* __restrict__ uin, const float* __restrict__ g,
    const float* __restrict__ h0, float* __restrict__ hout, void* __restrict__ vnew,
    float* __restrict__ fin, int L, int H) {
  constexpr int C = kGdnC;
  constexpr int BV = 16 * NW;
  constexpr int NTHR = 64 * NW;
  constexpr int NKB = K / 16;                  // state row blocks per wave
  constexpr int NKK = K / 32;                  // 32-wide k-steps over K
  constexpr int WS = K + 8;                    // w tile row stride (bf16)
  constexpr int KSt = K + 16;                  // k tile row stride (bf16)
  constexpr int US = BV + 16;                  // u tile row stride (bf16)
  constexpr int TRR = K > C ? K : C;           // transpose scratch rows
  constexpr int kWUnits = C * K / 8;           // 16-byte units of a w (or k) tile
  constexpr int WU = (kWUnits + NTHR - 1) / NTHR;
  constexpr int kUUnits = C * BV / 8;
  constexpr int UU = (kUUnits + NTHR - 1) / NTHR;
  __shared__ __attribute__((aligned(16))) uint16_t ws_[2][C * WS];
  __shared__ __attribute__((aligned(16))) uint16_t ks_[2][C * KSt];
  __shared__ __attribute__((aligned(16))) uint16_t us_[2][C * US];
  __shared__ __attribute__((aligned(16))) float gs_[2][C];
  __shared__ __attribute__((aligned(16))) float tr_[NW][TRR * kTrS];

  const int nvt = V / BV;
  const int logical = gdn_xcd_remap(blockIdx.x, gridDim.x);
  const int vt = logical % nvt;
  const int bh = logical / nvt;
  const int b = bh / H, h = bh % H;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const int v0 = vt * BV + 16 * wave;          // this wave's first state column
  const int nt = (L + C - 1) / C;

  // Per-sequence buffer descriptors: reads past the last token return zero.
  const uint32_t krow = (uint32_t)(H * K), urow = (uint32_t)(H * V);
  const rsrc_t kr = make_rsrc(kin + ((size_t)b * L * H + h) * K, ((uint32_t)(L - 1) * krow + K) * 2u);
  const rsrc_t wr = make_rsrc(win + ((size_t)b * L * H + h) * K, ((uint32_t)(L - 1) * krow + K) * 2u);
  const rsrc_t ur = make_rsrc(uin + ((size_t)b * L * H + h) * V, ((uint32_t)(L - 1) * urow + V) * 2u);
  const rsrc_t gr = make_rsrc(g + (size_t)b * L * H + h, ((uint32_t)(L - 1) * H + 1) * 4u);
  constexpr int VES = VBF16 ? 2 : 4;
  const rsrc_t vr = make_rsrc((char*)vnew + ((size_t)b * L * H + h) * V * VES,
                              ((uint32_t)(L - 1) * urow + V) * VES);

  // State blocks: acc[kb][r] = h[16 kb + 4 lq + r][v0 + lr].
  f32x4 acc[NKB];
  const size_t sbase = (size_t)bh * K * V;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[kb][r] = h0 ? h0[sbase + (size_t)(16 * kb + 4 * lq + r) * V + v0 + lr] : 0.0f;
  }
  __builtin_amdgcn_s_waitcnt(0);

  // Staging units of this thread (idle units read past the range).
  uint32_t woff[WU], uoff[UU];
  int wlds[WU], klds[WU], ulds[UU];
#pragma unroll
  for (int i = 0; i < WU; ++i) {
    const int u = tid + NTHR * i;
    const int t = u / (K / 8), c8 = u % (K / 8);
    woff[i] = u < kWUnits ? ((uint32_t)t * krow + 8 * c8) * 2u : kPastRange;
    wlds[i] = t * WS + 8 * c8;
    klds[i] = t * KSt + 8 * c8;
  }
#pragma unroll
  for (int i = 0; i < UU; ++i) {
    const int u = tid + NTHR * i;
    const int t = u / (BV / 8), c8 = u % (BV / 8);
    uoff[i] = u < kUUnits ? ((uint32_t)t * urow + vt * BV + 8 * c8) * 2u : kPastRange;
    ulds[i] = t * US + 8 * c8;
  }

  struct Tile {
    u32x4 w[WU], k[WU], u[UU];
    float g;
  };
  auto issue = [&](int c, Tile& tl) {
    const uint32_t t0 = (uint32_t)(c * C);
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      tl.w[i] = load_b128(wr, woff[i] + t0 * krow * 2u);
      tl.k[i] = load_b128(kr, woff[i] + t0 * krow * 2u);
    }
#pragma unroll
    for (int i = 0; i < UU; ++i) tl.u[i] = load_b128(ur, uoff[i] + t0 * urow * 2u);
    const uint32_t tt = t0 + (uint32_t)tid;
    tl.g = load_f32(gr, (tid < C && tt < (uint32_t)L) ? tt * (uint32_t)H * 4u : kPastRange);
  };
  auto commit = [&](int buf, const Tile& tl) {
#pragma unroll
    for (int i = 0; i < WU; ++i) {
      if (tid + NTHR * i < kWUnits) {
        *(u32x4*)(ws_[buf] + wlds[i]) = tl.w[i];
        *(u32x4*)(ks_[buf] + klds[i]) = tl.k[i];
      }
    }
#pragma unroll
    for (int i = 0; i < UU; ++i)
      if (tid + NTHR * i < kUUnits) *(u32x4*)(us_[buf] + ulds[i]) = tl.u[i];
    if (tid < C) gs_[buf][tid] = tl.g;
  };

  float* tr = tr_[wave];
  // The wave's 16 state columns (all K rows) as 16-byte rows of 4 columns.
  auto store_state = [&](float* dst) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) tr[(16 * kb + 4 * lq + r) * kTrS + lr] = acc[kb][r];
    }
#pragma unroll
    for (int i = 0; i < K / 16; ++i) {
      const int row = 16 * i + (lane >> 2), cg = lane & 3;
      *(f32x4*)(dst + (size_t)row * V + v0 + 4 * cg) = *(const f32x4*)(tr + row * kTrS + 4 * cg);
    }
  };

  auto step = [&](int c, const Tile& next) {
    const int buf = c & 1;
    const uint16_t* wsb = ws_[buf];
    const uint16_t* ksb = ks_[buf];
    const uint16_t* usb = us_[buf];
    const float* gsb = gs_[buf];
    const int n = min(C, L - c * C);            // valid tokens of the chunk

    // (1) the state at the chunk start
    store_state(hout + ((size_t)bh * nt + c) * K * V);

    // (2) v_new = u - w h, as -(w h - u); rows t = 16 tb + 4 lq + r, column v0 + lr
    u32x4 hh[NKK], hl[NKK];
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) split8(acc[2 * kk], acc[2 * kk + 1], hh[kk], hl[kk]);
    f32x4 vn[4];
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
      const u32x2 uu = lds_read_tr16(usb + (16 * tb + 4 * lq + (lr >> 2)) * US + 16 * wave +
                                     4 * (lr & 3));
      vn[tb] = -(f32x4){bf16_lo(uu[0]), bf16_hi(uu[0]), bf16_lo(uu[1]), bf16_hi(uu[1])};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const uint16_t* wp = wsb + (16 * tb + lr) * WS + 32 * kk + 4 * lq;
        const u32x2 a0 = *(const u32x2*)wp;
        const u32x2 a1 = *(const u32x2*)(wp + 16);
        const u32x4 av = {a0[0], a0[1], a1[0], a1[1]};
        vn[tb] = mfma_bf16(av, hh[kk], vn[tb]);
        vn[tb] = mfma_bf16(av, hl[kk], vn[tb]);
      }
      vn[tb] = -vn[tb];
    }

    // (3) v_new out, 16-byte rows of 4 columns (tokens past the end fall
    //     outside the buffer range and are dropped)
#pragma unroll
    for (int tb = 0; tb < 4; ++tb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) tr[(16 * tb + 4 * lq + r) * kTrS + lr] = vn[tb][r];
    }
    const uint32_t t0 = (uint32_t)(c * C);
#pragma unroll
    for (int i = 0; i < C / 16; ++i) {
      const int row = 16 * i + (lane >> 2), cg = lane & 3;
      const f32x4 vv = *(const f32x4*)(tr + row * kTrS + 4 * cg);
      const uint32_t off = ((t0 + row) * urow + v0 + 4 * cg) * VES;
      if constexpr (VBF16) {
        __builtin_amdgcn_raw_buffer_store_b64(
            (u32x2){pack_bf16(vv[0], vv[1]), pack_bf16(vv[2], vv[3])}, vr, (int)off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, vv), vr, (int)off, 0,
                                               0);
      }
    }

    // (4) gate and (5) update: h = e^{g_last} h + k^T (e^{g_last - g} o v_new).
    //     Tokens past the end have u = w = 0, so v_new = 0 there.
    const float gl = gsb[n - 1];
    const float decay = exp2_hw(gl * kLog2e);
    u32x4 gh[2], glo[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x4 e[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int tb = 2 * kk + s;
        const f32x4 gv = *(const f32x4*)(gsb + 16 * tb + 4 * lq);
#pragma unroll
        for (int r = 0; r < 4; ++r) e[s][r] = vn[tb][r] * exp2_hw((gl - gv[r]) * kLog2e);
      }
      split8(e[0], e[1], gh[kk], glo[kk]);
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      acc[kb] = decay * acc[kb];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const uint16_t* kp = ksb + (32 * kk + 4 * lq + (lr >> 2)) * KSt + 16 * kb + 4 * (lr & 3);
        const u32x2 e0 = lds_read_tr16(kp);
        const u32x2 e1 = lds_read_tr16(kp + 16 * KSt);
        const u32x4 kv = {e0[0], e0[1], e1[0], e1[1]};
        acc[kb] = mfma_bf16(kv, gh[kk], acc[kb]);
        acc[kb] = mfma_bf16(kv, glo[kk], acc[kb]);
      }
    }
    if (c + 1 < nt) commit(buf ^ 1, next);
    __syncthreads();
  };

  // Two register tiles: one is staged while the other's loads are in flight.
  Tile ga, gb;
  issue(0, ga);
  __builtin_amdgcn_sched_barrier(0);
  issue(1, gb);
  __builtin_amdgcn_sched_barrier(0);
  commit(0, ga);
  __syncthreads();
  for (int c0 = 0; c0 < nt; c0 += 2) {
    step(c0, gb);
    __builtin_amdgcn_sched_barrier(0);
    issue(c0 + 2, ga);
    __builtin_amdgcn_sched_barrier(0);
    if (c0 + 1 < nt) step(c0 + 1, ga);
    __builtin_amdgcn_sched_barrier(0);
    issue(c0 + 3, gb);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (fin) store_state(fin + sbase);
}

template <int K, int V, int NW, bool VBF16>
int launch_h(const void* k, const void* w, const void* u, const float* g, const float* h0,
             float* hout, void* vnew, float* fin, const GdnShape& s, hipStream_t st) {
  const unsigned blocks = (unsigned)(s.batch * s.nheads * (V / (16 * NW)));
  hipLaunchKernelGGL((gdn_fwd_h_kernel<K, V, NW, VBF16>), dim3(blocks), dim3(64 * NW), 0, st,
                     (const uint16_t*)k, (const uint16_t*)w, (const uint16_t*)u, g, h0, hout,
                     vnew, fin, (int)s.seqlen, (int)s.nheads);
  return (int)hipGetLastError();
}

template <int K, int V>
int launch_h_kv(const void* k, const void* w, const void* u, const float* g, const float* h0,
                float* hout, void* vnew, float* fin, bool vbf16, const GdnShape& s,
                hipStream_t st) {
  // four waves (64 columns) per workgroup when that still gives a workgroup
  // per CU, else two
  const bool wide = V >= 64 && s.batch * s.nheads * (V / 64) >= 256;
  if (wide)
    return vbf16 ? launch_h<K, V, 4, true>(k, w, u, g, h0, hout, vnew, fin, s, st)
                 : launch_h<K, V, 4, false>(k, w, u, g, h0, hout, vnew, fin, s, st);
  return vbf16 ? launch_h<K, V, 2, true>(k, w, u, g, h0, hout, vnew, fin, s, st)
               : launch_h<K, V, 2, false>(k, w, u, g, h0, hout, vnew, fin, s, st);
}

// ------------------------------------------------------------ chunk_fwd_o
// Work items are (b, chunk, head, 64-column block of V), the column block
// fastest.  A persistent workgroup takes one contiguous run of items and
// prefetches: while item i is computed from LDS and registers, item i+1's
// state block, v_new block, g and (when its (b, chunk, head) differs from
// item i's) its k tile and q rows are already loading into registers.  The
// column blocks of one (b, chunk, head) share k and q, so the second block
// loads neither.  Wave w owns the 16 tokens t of block w and computes
// o^T[v][t] for the item's columns, so each lane's accumulators are four
// consecutive v of one token (16-byte stores).  Per wave:
//   (i)   D = k q^T over K for the key blocks j <= t (rows j, columns t); with
//         the decay e^{g_t - g_j} and the causal select (j <= t, applied
//         after the exponent is formed) it is A^T, and a lane holds exactly
//         the four consecutive j of the k-slot map, so A^T (split hi + lo)
//         is the B operand of the next product as it sits;
//   (ii)  o^T = h^T q^T (the state from LDS as bf16 hi + lo, read with the
//         transpose read), scaled per token by e^{g_t};
//   (iii) o^T += v_new^T A^T (v_new from LDS with the transpose read).
// q stays in registers (each wave reads only its own 16 rows); k, v_new and
// the state are staged in LDS.  The LDS footprint lets two workgroups share
// a CU.
template <int K, int V, bool OBF16>
__global__ __launch_bounds__(256) void gdn_fwd_o_kernel(
    const uint16_t* __restrict__ qin, const uint16_t* __restrict__ kin,
    const uint16_t* __restrict__ vnin, const float* __restrict__ hin,
    const float* __restrict__ g, void* __restrict__ out, float scale, int L, int H, int nt,
    int items) {
  constexpr int C = kGdnC;
  constexpr int VB = 64;                       // columns of V per item
  constexpr int NVB = VB / 16;
  constexpr int NKK = K / 32;
  constexpr int HS = VB + 16;                  // state tile row stride (bf16)
  constexpr int KS = K + 8;                    // k tile row stride (bf16)
  constexpr int VS = VB + 16;                  // v_new tile row stride (bf16)
  constexpr int kHUnits = K * VB / 4;          // 16-byte fp32 units of the state tile
  constexpr int HU = kHUnits / 256;
  constexpr int kKUnits = C * K / 8;
  constexpr int KU = kKUnits / 256;
  constexpr int kVUnits = C * VB / 8;
  constexpr int VU = kVUnits / 256;
  static_assert(HU * 256 == kHUnits && KU * 256 == kKUnits && VU * 256 == kVUnits, "units");
  __shared__ __attribute__((aligned(16))) uint16_t hhi[K * HS];
  __shared__ __attribute__((aligned(16))) uint16_t hlo[K * HS];
  __shared__ __attribute__((aligned(16))) uint16_t ks[C * KS];
  __shared__ __attribute__((aligned(16))) uint16_t vs[C * VS];
  __shared__ __attribute__((aligned(16))) float gs[C];

  constexpr int NVH = V / VB;
  // this workgroup's run [i0, i1); consecutive runs on one XCD
  int i0, i1;
  {
    const int nwg = gridDim.x;
    const int wg = gdn_xcd_remap(blockIdx.x, nwg);
    i0 = (int)((int64_t)wg * items / nwg);
    i1 = (int)((int64_t)(wg + 1) * items / nwg);
  }
  if (i0 >= i1) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lr = lane & 15, lq = lane >> 4;
  const uint32_t krow = (uint32_t)(H * K), vrow = (uint32_t)(H * V);

  struct Item {
    int b, c, h, vh;
  };
  auto decode = [&](int i) {
    Item it;
    it.vh = i % NVH;
    const int r = i / NVH;
    it.h = r % H;
    it.c = (r / H) % nt;
    it.b = r / (H * nt);
    return it;
  };
  // An item loads k and q unless the item before it in the run has the same
  // (b, chunk, head).
  auto loads_kq = [&](int i) { return i == i0 || i % NVH == 0; };

  // One item's raw data.  A dead item (past the run) gets empty buffer
  // ranges: its loads return zero without touching memory.
  struct Ld {
    f32x4 h[HU];
    u32x4 k[KU], v[VU], q[NKK];
    float g;
  };
  auto issue = [&](int i, bool live, bool kq, Ld& d) {
    const Item it = decode(i);
    const uint32_t t0 = (uint32_t)(it.c * C);
    const rsrc_t hr = make_rsrc(hin + (((size_t)it.b * H + it.h) * nt + it.c) * K * V + it.vh * VB,
                                live ? ((uint32_t)(K - 1) * V + VB) * 4u : 0u);
#pragma unroll
    for (int j = 0; j < HU; ++j) {
      const int u = tid + 256 * j, row = u / (VB / 4), c4 = u % (VB / 4);
      d.h[j] = load_f32x4(hr, ((uint32_t)row * V + 4 * c4) * 4u);
    }
    if (kq) {
      const rsrc_t kr = make_rsrc(kin + ((size_t)it.b * L * H + it.h) * K,
                                  live ? ((uint32_t)(L - 1) * krow + K) * 2u : 0u);
#pragma unroll
      for (int j = 0; j < KU; ++j) {
        const int u = tid + 256 * j, t = u / (K / 8), c8 = u % (K / 8);
        d.k[j] = load_b128(kr, ((t0 + t) * krow + 8 * c8) * 2u);
      }
      // q: this wave's 16 tokens, in the k-slot map (K = 32kk + 4lq + 0..3
      // and 32kk + 16 + 4lq + 0..3), straight into operand registers
      const rsrc_t qr = make_rsrc(qin + ((size_t)it.b * L * H + it.h) * K,
                                  live ? ((uint32_t)(L - 1) * krow + K) * 2u : 0u);
      const uint32_t tq = t0 + 16 * wave + lr;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x2 a = load_b64(qr, (tq * krow + 32 * kk + 4 * lq) * 2u);
        const u32x2 bq = load_b64(qr, (tq * krow + 32 * kk + 16 + 4 * lq) * 2u);
        d.q[kk] = (u32x4){a[0], a[1], bq[0], bq[1]};
      }
    }
    const rsrc_t vr = make_rsrc(vnin + ((size_t)it.b * L * H + it.h) * V,
                                live ? ((uint32_t)(L - 1) * vrow + V) * 2u : 0u);
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = tid + 256 * j, t = u / (VB / 8), c8 = u % (VB / 8);
      d.v[j] = load_b128(vr, ((t0 + t) * vrow + it.vh * VB + 8 * c8) * 2u);
    }
    const rsrc_t gr = make_rsrc(g + (size_t)it.b * L * H + it.h,
                                live ? ((uint32_t)(L - 1) * H + 1) * 4u : 0u);
    d.g = load_f32(gr, (tid < C && t0 + tid < (uint32_t)L) ? (t0 + tid) * (uint32_t)H * 4u
                                                          : kPastRange);
  };

  Ld nx;
  u32x4 qf[NKK];
  issue(i0, true, true, nx);
  for (int i = i0; i < i1; ++i) {
    const Item it = decode(i);
    const bool kq = loads_kq(i);
    __syncthreads();  // the previous item's LDS reads are done
    // Stage: the state split into bf16 hi + lo, k and v_new as loaded, g.
#pragma unroll
    for (int j = 0; j < HU; ++j) {
      const int u = tid + 256 * j, row = u / (VB / 4), c4 = u % (VB / 4);
      uint32_t hh0, hl0, hh1, hl1;
      split_bf16(nx.h[j][0], nx.h[j][1], hh0, hl0);
      split_bf16(nx.h[j][2], nx.h[j][3], hh1, hl1);
      *(u32x2*)(hhi + row * HS + 4 * c4) = (u32x2){hh0, hh1};
      *(u32x2*)(hlo + row * HS + 4 * c4) = (u32x2){hl0, hl1};
    }
    if (kq) {
#pragma unroll
      for (int j = 0; j < KU; ++j) {
        const int u = tid + 256 * j, t = u / (K / 8), c8 = u % (K / 8);
        *(u32x4*)(ks + t * KS + 8 * c8) = nx.k[j];
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) qf[kk] = nx.q[kk];
    }
#pragma unroll
    for (int j = 0; j < VU; ++j) {
      const int u = tid + 256 * j, t = u / (VB / 8), c8 = u % (VB / 8);
      *(u32x4*)(vs + t * VS + 8 * c8) = nx.v[j];
    }
    if (tid < C) gs[tid] = nx.g;
    // the next item's loads
    {
      const bool live = i + 1 < i1;
      issue(live ? i + 1 : i, live, live && loads_kq(i + 1), nx);
    }
    __syncthreads();

    const int tl = 16 * wave + lr;               // this lane's token in the chunk
    const float gt = gs[tl];

    // (ii) inter term: o^T = h^T q^T, then e^{g_t} per token.
    f32x4 oa[NVB];
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      oa[vb] = (f32x4){0, 0, 0, 0};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const int o0 = (32 * kk + 4 * lq + (lr >> 2)) * HS + 16 * vb + 4 * (lr & 3);
        const u32x2 a0 = lds_read_tr16(hhi + o0), a1 = lds_read_tr16(hhi + o0 + 16 * HS);
        const u32x2 c0 = lds_read_tr16(hlo + o0), c1 = lds_read_tr16(hlo + o0 + 16 * HS);
        oa[vb] = mfma_bf16((u32x4){a0[0], a0[1], a1[0], a1[1]}, qf[kk], oa[vb]);
        oa[vb] = mfma_bf16((u32x4){c0[0], c0[1], c1[0], c1[1]}, qf[kk], oa[vb]);
      }
      oa[vb] = exp2_hw(gt * kLog2e) * oa[vb];
    }

    // (i) A^T blocks for key blocks jb <= wave, then (iii) o^T += v_new^T A^T
    // in pairs of key blocks (32 keys per matrix step).
#pragma unroll
    for (int kp = 0; kp < 2; ++kp) {
      if (2 * kp > wave) break;
      f32x4 at[2];
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const int jb = 2 * kp + s2;
        at[s2] = (f32x4){0, 0, 0, 0};
        if (jb <= wave) {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const uint16_t* kp0 = ks + (16 * jb + lr) * KS + 32 * kk + 4 * lq;
            const u32x2 a = *(const u32x2*)kp0;
            const u32x2 bb = *(const u32x2*)(kp0 + 16);
            at[s2] = mfma_bf16((u32x4){a[0], a[1], bb[0], bb[1]}, qf[kk], at[s2]);
          }
          const f32x4 gj = *(const f32x4*)(gs + 16 * jb + 4 * lq);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int j = 16 * jb + 4 * lq + r;
            const float e = at[s2][r] * exp2_hw((gt - gj[r]) * kLog2e);
            at[s2][r] = j <= tl ? e : 0.0f;
          }
        }
      }
      u32x4 bh, bl;
      split8(at[0], at[1], bh, bl);
#pragma unroll
      for (int vb = 0; vb < NVB; ++vb) {
        const int o0 = (32 * kp + 4 * lq + (lr >> 2)) * VS + 16 * vb + 4 * (lr & 3);
        const u32x2 e0 = lds_read_tr16(vs + o0), e1 = lds_read_tr16(vs + o0 + 16 * VS);
        const u32x4 av = {e0[0], e0[1], e1[0], e1[1]};
        oa[vb] = mfma_bf16(av, bh, oa[vb]);
        oa[vb] = mfma_bf16(av, bl, oa[vb]);
      }
    }

    // o[t][v .. v+3] for v = 64 vh + 16 vb + 4 lq; tokens past the end are
    // outside the buffer range and dropped.
    constexpr int OES = OBF16 ? 2 : 4;
    const rsrc_t orr = make_rsrc((char*)out + ((size_t)it.b * L * H + it.h) * V * OES,
                                 ((uint32_t)(L - 1) * vrow + V) * OES);
    const uint32_t tq = (uint32_t)(it.c * C) + 16 * wave + lr;
#pragma unroll
    for (int vb = 0; vb < NVB; ++vb) {
      const f32x4 ov = scale * oa[vb];
      const uint32_t off = (tq * vrow + it.vh * VB + 16 * vb + 4 * lq) * OES;
      if constexpr (OBF16) {
        __builtin_amdgcn_raw_buffer_store_b64((u32x2){pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3])},
                                              orr, (int)off, 0, 0);
      } else {
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, ov), orr, (int)off, 0, 0);
      }
    }
  }
}

template <int K, int V, bool OBF16>
int launch_o(const void* q, const void* k, const void* vnew, const float* h, const float* g,
             void* o, float scale, const GdnShape& s, hipStream_t st) {
  const int nt = (int)s.nchunks();
  const int items = (int)(s.batch * nt * s.nheads * (V / 64));
  // the persistent grid: as many workgroups as are resident on the device
  static PerDeviceInt resident;
  const int slots = resident.get([](int dev) {
    return resident_slots((const void*)gdn_fwd_o_kernel<K, V, OBF16>, 256, dev);
  });
  if (slots <= 0) return (int)hipErrorInvalidDevice;
  const unsigned grid = (unsigned)(items < slots ? items : slots);
  hipLaunchKernelGGL((gdn_fwd_o_kernel<K, V, OBF16>), dim3(grid), dim3(256), 0, st,
                     (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)vnew, h, g, o, scale,
                     (int)s.seqlen, (int)s.nheads, nt, items);
  return (int)hipGetLastError();
}

template <int K, int V>
int launch_o_kv(const void* q, const void* k, const void* vnew, const float* h, const float* g,
                void* o, float scale, bool obf16, const GdnShape& s, hipStream_t st) {
  if (obf16) return launch_o<K, V, true>(q, k, vnew, h, g, o, scale, s, st);
  return launch_o<K, V, false>(q, k, vnew, h, g, o, scale, s, st);
}

}  // namespace

int launch_gdn_fwd_o(const void* q, const void* k, const void* vnew, const float* h,
                     const float* g, void* o, float scale, bool obf16, const GdnShape& s,
                     void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (s.dk == 64)
    return s.dv == 64 ? launch_o_kv<64, 64>(q, k, vnew, h, g, o, scale, obf16, s, st)
                      : launch_o_kv<64, 128>(q, k, vnew, h, g, o, scale, obf16, s, st);
  return s.dv == 64 ? launch_o_kv<128, 64>(q, k, vnew, h, g, o, scale, obf16, s, st)
                    : launch_o_kv<128, 128>(q, k, vnew, h, g, o, scale, obf16, s, st);
}

int launch_gdn_fwd_h(const void* k, const void* w, const void* u, const float* g,
                     const float* h0, float* hout, void* vnew, float* fin, bool vbf16,
                     const GdnShape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (s.dk == 64)
    return s.dv == 64 ? launch_h_kv<64, 64>(k, w, u, g, h0, hout, vnew, fin, vbf16, s, st)
                      : launch_h_kv<64, 128>(k, w, u, g, h0, hout, vnew, fin, vbf16, s, st);
  return s.dv == 64 ? launch_h_kv<128, 64>(k, w, u, g, h0, hout, vnew, fin, vbf16, s, st)
                    : launch_h_kv<128, 128>(k, w, u, g, h0, hout, vnew, fin, vbf16, s, st);
}

}  // namespace ssd

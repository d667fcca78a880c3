// Stage 1: per-chunk, log2-scaled cumulative sum of the decay.
//
//   g[b,h,t] = log2(e) * sum_{s = T*floor(t/T)}^{t} A[h] * dt[b,s,h]
//
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", section "Kernel 1: chunk_cumsum, the Cumulative Decay Sums":
// the sum restarts at every chunk; the log2(e) factor lets later stages use
// exp2.)  dt arrives token-major [b, L, H]; g and a transposed copy of dt
// leave head-major [b, H, L] so the later stages read each head's chunk as
// one contiguous run (the pages transpose both decay_cumsum and dt to
// [batch, head, token] among their optimizations).
//
// MI355X design.  The dt values of one (b, chunk) are one contiguous slab of
// T rows of H floats.  A workgroup (4 waves) owns the slab's columns for a
// block of HB consecutive heads: all of its loads are issued at once, as
// 16-byte vectors where the columns allow (so with HB = H every byte of
// every fetched line is used, and consecutive threads read consecutive 16
// bytes), and land in LDS as [token][head] with an odd row stride.  Then each
// wave scans whole heads, two at a time: lane l reads its T/64 consecutive
// tokens of the head's column and scans them serially, and a wavefront scan
// of the lane totals by DPP row shifts and row broadcasts (register moves
// between lanes, no LDS round trip) gives the lane's offset.  g and dt_t rows leave as
// contiguous vector stores.  The host picks the head block so the grid has
// at least one workgroup per CU (the slab count alone is 64 on the 2 x 8192
// token, 256-token-chunk layer), and the largest block that does, so reads
// stay as wide as the slab allows.  Consecutive blocks are placed on one
// XCD, so the head blocks of a slab share its lines in one L2.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
// LDS floats for one slab block: T rows of (HB + 1) floats.
constexpr int kSlabFloats = 8448;

// Largest head block that fits the LDS slab for chunk size T.
constexpr int max_head_block(int T) { return kSlabFloats / T - 1; }

// One DPP move of v across lanes (gfx9 encodings): lanes with no source, or
// in rows outside ROWS, read 0.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143, kWaveShr1 = 0x138;

// Inclusive scan across the 64 lanes: shifts by 1, 2, 4, 8 within each row
// of 16 lanes, then lane 15 of rows 0 and 2 added into rows 1 and 3, then
// lane 31 into rows 2 and 3.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp0<kRowShr1, 0xF>(x);
  x += dpp0<kRowShr2, 0xF>(x);
  x += dpp0<kRowShr4, 0xF>(x);
  x += dpp0<kRowShr8, 0xF>(x);
  x += dpp0<kRowBcast15, 0xA>(x);
  x += dpp0<kRowBcast31, 0xC>(x);
  return x;
}

template <int T, int VW>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ g, float* __restrict__ dt_t, int L, int H, int nc,
    int HB, int nhb) {
  constexpr int kPer = T / kWave;            // tokens per lane in the scan
  constexpr int kBatch = 8;                  // loads in flight per thread
  __shared__ float slab[kSlabFloats];

  int blk = blockIdx.x;
  if (gridDim.x % 8 == 0) blk = (blk % 8) * (gridDim.x / 8) + blk / 8;
  const int hb = blk % nhb;
  const int c = (blk / nhb) % nc;
  const int b = blk / (nhb * nc);
  const int h0 = hb * HB;
  const int nh = min(HB, H - h0);            // heads in this block
  const int t0 = c * T;
  const int nt = min(T, L - t0);             // valid tokens in this chunk
  const int S = HB + 1;                      // LDS row stride (odd when HB is even)
  const int tid = threadIdx.x, wave = tid / kWave, lane = tid % kWave;

  // ---- load: units of VW consecutive heads of one token row; rows past the
  // end of the sequence read zero through the buffer range
  const rsrc_t dr = make_rsrc(dt + (size_t)b * L * H, (uint32_t)L * H * 4u);
  const int upr = (nh + VW - 1) / VW;        // units per row
  const int nunits = T * upr;
  for (int u0 = 0; u0 < nunits; u0 += kBatch * kThreads) {
    float v[kBatch][VW];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int u = u0 + k * kThreads + tid;
      const int row = u / upr, col = (u % upr) * VW;
      const uint32_t off = u < nunits ? ((uint32_t)(t0 + row) * H + h0 + col) * 4u : 0x7FFFFFF0u;
      if constexpr (VW == 4) {
        const f32x4 q = load_f32x4(dr, off);
#pragma unroll
        for (int j = 0; j < 4; ++j) v[k][j] = q[j];
      } else {
        v[k][0] = load_f32(dr, off);
      }
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int u = u0 + k * kThreads + tid;
      if (u < nunits) {
        const int row = u / upr, col = (u % upr) * VW;
#pragma unroll
        for (int j = 0; j < VW; ++j) slab[row * S + col + j] = v[k][j];
      }
    }
  }
  __syncthreads();

  // ---- scan: each wave takes two heads at a time (independent chains)
  const bool full = lane * kPer + kPer <= nt;
  const bool vst = kPer > 1 && L % kPer == 0 && full;
  constexpr int kWaves = kThreads / kWave;
  for (int j0 = wave; j0 < nh; j0 += 2 * kWaves) {
    float d[2][kPer], v[2][kPer], excl[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = min(j0 + q * kWaves, nh - 1);
      const float a = A[h0 + j];
      float run = 0.0f;
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        d[q][k] = slab[(lane * kPer + k) * S + j];
        run += a * d[q][k];
        v[q][k] = run;
      }
      // the lane's offset: the inclusive scan of the lane totals, shifted
      // one lane up (lane 0 gets 0)
      excl[q] = dpp0<kWaveShr1, 0xF>(wave_inclusive_scan(run));
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int j = j0 + q * kWaves;
      if (j >= nh) break;
      const size_t row = ((size_t)b * H + h0 + j) * L + t0 + lane * kPer;
      if (vst) {
        if constexpr (kPer == 4) {
          *(f32x4*)(g + row) =
              (f32x4){(excl[q] + v[q][0]) * kLog2e, (excl[q] + v[q][1]) * kLog2e,
                      (excl[q] + v[q][2]) * kLog2e, (excl[q] + v[q][3]) * kLog2e};
          *(f32x4*)(dt_t + row) = (f32x4){d[q][0], d[q][1], d[q][2], d[q][3]};
        } else if constexpr (kPer == 2) {
          *(f32x2*)(g + row) = (f32x2){(excl[q] + v[q][0]) * kLog2e, (excl[q] + v[q][1]) * kLog2e};
          *(f32x2*)(dt_t + row) = (f32x2){d[q][0], d[q][1]};
        }
      } else {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          if (lane * kPer + k < nt) {
            g[row + k] = (excl[q] + v[q][k]) * kLog2e;
            dt_t[row + k] = d[q][k];
          }
        }
      }
    }
  }
}

// Head block for a grid of at least one workgroup per CU: the fewest blocks
// that reach the CU count (or one block per head) and fit the LDS slab.
int choose_head_block(const Shape& s, int T, int cus) {
  const int64_t slabs = s.batch * s.nchunks();
  const int64_t H = s.nheads;
  int64_t nb = (H + max_head_block(T) - 1) / max_head_block(T);
  const int64_t want = (cus + slabs - 1) / slabs;
  if (want > nb) nb = want;
  if (nb > H) nb = H;
  return (int)((H + nb - 1) / nb);
}

template <int T>
int launch_t(const float* dt, const float* A, float* g, float* dt_t, const Shape& s,
             hipStream_t st) {
  static PerDeviceInt cus_cache;
  int cus = cus_cache.get(query_cus);
  if (cus <= 0) cus = 256;
  const int HB = choose_head_block(s, T, cus);
  const int nhb = (int)((s.nheads + HB - 1) / HB);
  const int nc = (int)s.nchunks();
  const dim3 grid((unsigned)(s.batch * nc * nhb));
  const int L = (int)s.seqlen, H = (int)s.nheads;
  // 16-byte units need 16-byte aligned rows and blocks
  if (H % 4 == 0 && HB % 4 == 0)
    hipLaunchKernelGGL((chunk_cumsum_kernel<T, 4>), grid, dim3(kThreads), 0, st, dt, A, g,
                       dt_t, L, H, nc, HB, nhb);
  else
    hipLaunchKernelGGL((chunk_cumsum_kernel<T, 1>), grid, dim3(kThreads), 0, st, dt, A, g,
                       dt_t, L, H, nc, HB, nhb);
  return (int)hipGetLastError();
}

}  // namespace

int launch_chunk_cumsum(const float* dt, const float* A, float* g,
                        float* dt_t, const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  switch (s.chunk) {
    case 64: return launch_t<64>(dt, A, g, dt_t, s, st);
    case 128: return launch_t<128>(dt, A, g, dt_t, s, st);
    case 256: return launch_t<256>(dt, A, g, dt_t, s, st);
    default: return (int)hipErrorInvalidValue;
  }
}

}  // namespace ssd

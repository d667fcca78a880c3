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
// One wavefront per (chunk, 4 consecutive heads, batch), four per workgroup.
// Lane l owns tokens T/64 * l .. + T/64 - 1 of the chunk and loads each
// token's 4 head values at once (one 16-byte load when H % 4 == 0, else
// four 4-byte loads); all of a lane's loads are in flight together.  Each
// head is then scanned as before: a serial inclusive scan over the lane's
// tokens, and a wavefront inclusive scan of the lane totals (shuffles)
// supplies the lane's offset.  No LDS and no barrier: the 4 heads' scans
// run side by side in registers.  Output rows are written contiguously
// (16 bytes per lane where the rows allow it).  The stage moves 12 bytes per
// (token, head) and is HBM-bound.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kHeadsPerWave = 4;
constexpr int kWavesPerBlock = 4;

template <int T, bool VEC>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ g, float* __restrict__ dt_t, int L, int H, int nc,
    int nhq, int nwaves) {
  constexpr int kPer = T / kWave;  // tokens per lane
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  // Flat wave id: head quad fastest (the quads of one token row share its
  // cache lines), then chunk, then batch.  Blocks are dealt to the 8 XCDs
  // round-robin, so consecutive logical blocks are remapped onto one XCD:
  // the quads of a row then meet in one L2 instead of fetching its lines
  // from memory once per XCD.
  int blk = blockIdx.x;
  if (gridDim.x % 8 == 0) blk = (blk % 8) * (gridDim.x / 8) + blk / 8;
  const int wid = blk * kWavesPerBlock + wave;
  if (wid >= nwaves) return;   // the last workgroup's spare waves
  const int hq = wid % nhq;
  const int c = (wid / nhq) % nc;
  const int b = wid / (nc * nhq);
  const int h0 = hq * kHeadsPerWave;
  const int t0 = c * T;
  const int nt = min(T, L - t0);
  const int nh = min(kHeadsPerWave, H - h0);

  // d[k][j]: dt of token lane*kPer + k, head h0 + j (0 past the end)
  const rsrc_t dr = make_rsrc(dt + (size_t)b * L * H, (uint32_t)L * H * 4u);
  float d[kPer][kHeadsPerWave];
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const uint32_t row = (uint32_t)(t0 + lane * kPer + k) * H + h0;
    if constexpr (VEC) {
      const f32x4 q = load_f32x4(dr, row * 4u);
#pragma unroll
      for (int j = 0; j < kHeadsPerWave; ++j) d[k][j] = q[j];
    } else {
#pragma unroll
      for (int j = 0; j < kHeadsPerWave; ++j)
        d[k][j] = load_f32(dr, j < nh ? (row + j) * 4u : 0x7FFFFFF0u);
    }
  }

  // Rows start 16-byte aligned when L % 4 == 0 (8-byte when L is even), so
  // a lane whose tokens are all real stores them as one vector.
  const bool full = lane * kPer + kPer <= nt;
  const bool vst = kPer > 1 && L % kPer == 0 && full;
#pragma unroll
  for (int j = 0; j < kHeadsPerWave; ++j) {
    if (j >= nh) break;
    const float a = A[h0 + j];
    float v[kPer];
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      run += a * d[k][j];
      v[k] = run;
    }
    // Inclusive scan of the lane totals across the wavefront.
    float incl = run;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const float o = __shfl_up(incl, off, kWave);
      if (lane >= off) incl += o;
    }
    float excl = __shfl_up(incl, 1, kWave);
    if (lane == 0) excl = 0.0f;
    const size_t row = ((size_t)b * H + h0 + j) * L + t0 + lane * kPer;
    if (vst) {
      if constexpr (kPer == 4) {
        *(f32x4*)(g + row) = (f32x4){(excl + v[0]) * kLog2e, (excl + v[1]) * kLog2e,
                                     (excl + v[2]) * kLog2e, (excl + v[3]) * kLog2e};
        *(f32x4*)(dt_t + row) = (f32x4){d[0][j], d[1][j], d[2][j], d[3][j]};
      } else if constexpr (kPer == 2) {
        *(f32x2*)(g + row) = (f32x2){(excl + v[0]) * kLog2e, (excl + v[1]) * kLog2e};
        *(f32x2*)(dt_t + row) = (f32x2){d[0][j], d[1][j]};
      }
    } else {
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        if (lane * kPer + k < nt) {
          g[row + k] = (excl + v[k]) * kLog2e;
          dt_t[row + k] = d[k][j];
        }
      }
    }
  }
}

}  // namespace

int launch_chunk_cumsum(const float* dt, const float* A, float* g,
                        float* dt_t, const Shape& s, void* stream) {
  clear_launch_error();
  const int nc = (int)s.nchunks();
  const int nhq = (int)((s.nheads + kHeadsPerWave - 1) / kHeadsPerWave);
  const int64_t nwaves = s.batch * nc * nhq;
  const dim3 grid((unsigned)((nwaves + kWavesPerBlock - 1) / kWavesPerBlock));
  const dim3 block(kWave * kWavesPerBlock);
  hipStream_t st = (hipStream_t)stream;
  const int L = (int)s.seqlen, H = (int)s.nheads;
  const bool vec = H % 4 == 0;
#define SSD_CUMSUM_LAUNCH(TT)                                                              \
  if (vec)                                                                                 \
    hipLaunchKernelGGL((chunk_cumsum_kernel<TT, true>), grid, block, 0, st, dt, A, g, dt_t, \
                       L, H, nc, nhq, (int)nwaves);                                        \
  else                                                                                     \
    hipLaunchKernelGGL((chunk_cumsum_kernel<TT, false>), grid, block, 0, st, dt, A, g,      \
                       dt_t, L, H, nc, nhq, (int)nwaves);
  switch (s.chunk) {
    case 64: SSD_CUMSUM_LAUNCH(64) break;
    case 128: SSD_CUMSUM_LAUNCH(128) break;
    case 256: SSD_CUMSUM_LAUNCH(256) break;
    default:
      return (int)hipErrorInvalidValue;
  }
#undef SSD_CUMSUM_LAUNCH
  return (int)hipGetLastError();
}

}  // namespace ssd

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
// One workgroup per (chunk, 16-head tile, batch).  The [T x 16] dt tile is
// read with coalesced row loads into LDS (the transpose), then each wave
// scans one head at a time: every lane owns T/64 consecutive tokens, does a
// serial inclusive scan over them, and a wavefront inclusive scan of the lane
// totals (shuffles) supplies each lane's offset.  Output rows are written
// contiguously.  The stage moves 12 bytes per (token, head) and is
// HBM-bound.
#include "ssd_device.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

constexpr int kHeadTile = 16;

template <int T>
__global__ __launch_bounds__(256) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const float* __restrict__ A,
    float* __restrict__ g, float* __restrict__ dt_t, int L, int H, int nc,
    int nht) {
  constexpr int kPer = T / kWave;  // tokens per lane
  __shared__ float tile[T][kHeadTile + 1];

  // Flat block id: chunk fastest, then head tile, then batch.
  const int c = blockIdx.x % nc;
  const int h0 = (blockIdx.x / nc) % nht * kHeadTile;
  const int b = blockIdx.x / (nc * nht);
  const int t0 = c * T;
  const int nt = min(T, L - t0);
  const int nh = min(kHeadTile, H - h0);

  const float* src = dt + ((size_t)b * L + t0) * H + h0;
  for (int e = threadIdx.x; e < T * kHeadTile; e += blockDim.x) {
    const int t = e / kHeadTile, hh = e % kHeadTile;
    tile[t][hh] = (t < nt && hh < nh) ? src[(size_t)t * H + hh] : 0.0f;
  }
  __syncthreads();

  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  for (int hh = wave; hh < nh; hh += blockDim.x / kWave) {
    const float a = A[h0 + hh];
    float v[kPer], d[kPer];
    float run = 0.0f;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      d[k] = tile[lane * kPer + k][hh];
      run += a * d[k];
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
    const size_t row = ((size_t)b * H + h0 + hh) * L + t0;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int t = lane * kPer + k;
      if (t < nt) {
        g[row + t] = (excl + v[k]) * kLog2e;
        dt_t[row + t] = d[k];
      }
    }
  }
}

}  // namespace

int launch_chunk_cumsum(const float* dt, const float* A, float* g,
                        float* dt_t, const Shape& s, void* stream) {
  const int nc = (int)s.nchunks();
  const int nht = (int)((s.nheads + kHeadTile - 1) / kHeadTile);
  const dim3 grid((unsigned)(s.batch * nc * nht));
  const dim3 block(256);
  hipStream_t st = (hipStream_t)stream;
  const int L = (int)s.seqlen, H = (int)s.nheads;
  switch (s.chunk) {
    case 64:
      hipLaunchKernelGGL(chunk_cumsum_kernel<64>, grid, block, 0, st, dt, A, g, dt_t, L, H, nc, nht);
      break;
    case 128:
      hipLaunchKernelGGL(chunk_cumsum_kernel<128>, grid, block, 0, st, dt, A, g, dt_t, L, H, nc, nht);
      break;
    case 256:
      hipLaunchKernelGGL(chunk_cumsum_kernel<256>, grid, block, 0, st, dt, A, g, dt_t, L, H, nc, nht);
      break;
    default:
      return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

}  // namespace ssd

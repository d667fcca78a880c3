// The streaming decode step: one token through the recurrence with a carried
// state, for every (b, h):
//   S = exp(A_h dt) S + dt x B^T        (S: P x N, fp32, updated in place)
//   y = S C + D_h x
// ("Accelerating Mamba-2 with High-Performance Forward Pass Kernels in NVIDIA
// CUDA Tile", sections "The Mamba-2 Recurrence" and "Why Would a Trading Firm
// Care About Mamba-2 Kernels?": at inference the fixed-size state is carried
// forward and updated with each new event; "Kernel 2: fwd_pass_state": the
// final state of a call is the next call's init_state.)  y reads the state
// after the update, as in the forward pass.
//
// MI355X design.  The step reads and writes the state once (8 P N bytes per
// head) and touches little else, so it is HBM-bound; the kernel is a
// coalesced stream over the state.  One workgroup (256 threads) per (b, h,
// block of 64/RB state rows), RB = 1, 2 or 4 chosen so that small batches
// still spread over all CUs (rows are independent: y_p reads row p only).
// Thread t owns the 16-byte units t + 256 i of its row block, so every load
// and store instruction covers 4 KB of contiguous state.  Unit u sits in row
// p = u / (N/4), columns 4 (u % (N/4)) .. + 3; since 256 is a multiple of
// N/4, a thread's columns are the same for every i, so its four values of B
// and C are loaded once.  A row's N/4 units belong to N/4 consecutive lanes
// of one wave, so the row sum for y is a lane reduction.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

template <bool BF16>
struct DecIn;
template <>
struct DecIn<true> {
  using T = uint16_t;
  static __device__ __forceinline__ f32x4 load4(const uint16_t* p) {
    const u32x2 v = *(const u32x2*)p;
    return (f32x4){bf16_lo(v[0]), bf16_hi(v[0]), bf16_lo(v[1]), bf16_hi(v[1])};
  }
  static __device__ __forceinline__ float load1(const uint16_t* p) {
    return __uint_as_float((uint32_t)*p << 16);
  }
};
template <>
struct DecIn<false> {
  using T = float;
  static __device__ __forceinline__ f32x4 load4(const float* p) { return *(const f32x4*)p; }
  static __device__ __forceinline__ float load1(const float* p) { return *p; }
};

template <int N, int RB, bool BF16, bool YBF16>
__global__ __launch_bounds__(256) void decode_step_kernel(
    const void* __restrict__ xv, const float* __restrict__ dt, const float* __restrict__ A,
    const void* __restrict__ Bv, const void* __restrict__ Cv, const float* __restrict__ Dv,
    float* __restrict__ state, void* __restrict__ y, int H, int G) {
  using In = DecIn<BF16>;
  using E = typename In::T;
  constexpr int UPR = N / 4;                 // 16-byte units per state row
  constexpr int ROWS = kHeadDim / RB;        // state rows of this workgroup
  constexpr int NU = ROWS * N / 4;           // units per workgroup
  constexpr int IT = NU / 256;               // units per thread
  static_assert(256 % UPR == 0 && NU % 256 == 0, "unit split");
  __shared__ float xs[ROWS];

  const int bh = blockIdx.x / RB, rb = blockIdx.x % RB;
  const int b = bh / H, h = bh % H, grp = h / (H / G);
  const int tid = threadIdx.x;
  const int p0 = rb * ROWS;
  const E* x = (const E*)xv + (size_t)bh * kHeadDim + p0;
  if (tid < ROWS) xs[tid] = In::load1(x + tid);

  const float d = dt[bh];
  const float decay = exp2_hw(A[h] * d * kLog2e);
  const float Dh = Dv[h];
  const int col = 4 * (tid % UPR);
  const size_t bc = ((size_t)b * G + grp) * N + col;
  const f32x4 Bq = In::load4((const E*)Bv + bc) * d;
  const f32x4 Cq = In::load4((const E*)Cv + bc);
  float* S = state + ((size_t)bh * kHeadDim + p0) * N;
  f32x4 s[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) s[i] = *(const f32x4*)(S + 4 * (tid + 256 * i));
  __syncthreads();

  float part[IT];
#pragma unroll
  for (int i = 0; i < IT; ++i) {
    const int p = (tid + 256 * i) / UPR;
    const float xp = xs[p];
    s[i] = decay * s[i] + xp * Bq;
    part[i] = s[i][0] * Cq[0] + s[i][1] * Cq[1] + s[i][2] * Cq[2] + s[i][3] * Cq[3];
    *(f32x4*)(S + 4 * (tid + 256 * i)) = s[i];
  }
  // Row sums over the UPR lanes that hold a row (lane groups aligned to UPR).
#pragma unroll
  for (int i = 0; i < IT; ++i) {
#pragma unroll
    for (int off = UPR / 2; off > 0; off >>= 1) part[i] += __shfl_xor(part[i], off, 64);
  }
  if (tid % UPR == 0) {
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const int p = (tid + 256 * i) / UPR;
      const float yv = part[i] + Dh * xs[p];
      const size_t o = (size_t)bh * kHeadDim + p0 + p;
      if constexpr (YBF16) {
        ((uint16_t*)y)[o] = (uint16_t)(pack_bf16(yv, 0.0f) & 0xFFFFu);
      } else {
        ((float*)y)[o] = yv;
      }
    }
  }
}

template <int N, int RB, bool BF16>
int launch_rb(const void* x, const float* dt, const float* A, const void* B, const void* C,
              const float* D, float* state, void* y, bool ybf16, const Shape& s,
              hipStream_t st) {
  const dim3 grid((unsigned)(s.batch * s.nheads * RB)), block(256);
  const int H = (int)s.nheads, G = (int)s.ngroups;
  if (ybf16)
    hipLaunchKernelGGL((decode_step_kernel<N, RB, BF16, true>), grid, block, 0, st, x, dt, A, B,
                       C, D, state, y, H, G);
  else
    hipLaunchKernelGGL((decode_step_kernel<N, RB, BF16, false>), grid, block, 0, st, x, dt, A,
                       B, C, D, state, y, H, G);
  return (int)hipGetLastError();
}

// Row blocks per head: enough workgroups for two per CU where the state
// allows (a workgroup keeps at least 256 units of 16 bytes).
template <int N, bool BF16>
int launch_y(const void* x, const float* dt, const float* A, const void* B, const void* C,
             const float* D, float* state, void* y, bool ybf16, const Shape& s,
             hipStream_t st) {
  const int64_t pairs = s.batch * s.nheads;
  if (pairs >= 512) return launch_rb<N, 1, BF16>(x, dt, A, B, C, D, state, y, ybf16, s, st);
  if (pairs >= 256) return launch_rb<N, 2, BF16>(x, dt, A, B, C, D, state, y, ybf16, s, st);
  return launch_rb<N, 4, BF16>(x, dt, A, B, C, D, state, y, ybf16, s, st);
}

}  // namespace

int launch_decode_step(const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, float* state, void* y, bool bf16_in,
                       bool bf16_out, const Shape& s, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (s.dstate == 64) {
    return bf16_in ? launch_y<64, true>(x, dt, A, B, C, D, state, y, bf16_out, s, st)
                   : launch_y<64, false>(x, dt, A, B, C, D, state, y, bf16_out, s, st);
  }
  return bf16_in ? launch_y<128, true>(x, dt, A, B, C, D, state, y, bf16_out, s, st)
                 : launch_y<128, false>(x, dt, A, B, C, D, state, y, bf16_out, s, st);
}

}  // namespace ssd

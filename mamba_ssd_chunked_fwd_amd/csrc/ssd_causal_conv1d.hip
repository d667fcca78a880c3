// The causal depthwise conv1d of the Mamba block, the step that feeds the SSD
// its x, B and C (the Helion hackathon gallery on NVIDIA B200, its
// causal_conv1d entries): every channel row is filtered on its own with a
// W-tap filter over the current and W-1 previous tokens, zeros before the
// first token:
//   out[b,d,t] = bias[d] + sum_{k<W} weight[d,k] x[b,d,t-W+1+k]
// x and out are [batch, dim, seqlen] with time contiguous; weight [dim, W]
// and bias [dim] are fp32; arithmetic is fp32 with the taps added in k order
// onto the bias.
//
// MI355X design.  The op reads x once and writes out once, so it is a pure
// HBM stream; the gallery entries say as much (the filter fits in registers,
// bandwidth decides).  The work unit is one 16-byte vector of a row (8 bf16
// or 4 fp32 tokens).  A wavefront owns a run of 64 * VPT consecutive units of
// one row: lane l handles units u0 + 64 j + l, j < VPT, so every load and
// store instruction of the wave covers 1 KB of contiguous row.  The W-1
// tokens before a unit belong to the previous unit, which lane l-1 holds:
// they arrive by a lane rotation (ds_bpermute), lane 0 taking lane 63's value
// of the previous j, and only lane 0 of the first j loads one extra unit
// (the run's left neighbour).  Rows are addressed through buffer descriptors
// whose range is the row itself: the unit before a row's first token and the
// units past its last read as zero, which is the causal padding and the
// ragged tail, and stores past the row are dropped by the same range check.
// Rows whose byte length is not a multiple of 16 take a plain per-token
// kernel instead.
#include "ssd_device.h"
#include "ssd_host.h"
#include "ssd_launch.h"

namespace ssd {
namespace {

// Byte offset past any row's range: reads there return zero.
constexpr uint32_t kPastRange = 0x7FFFFFF0u;
// Units per lane: 4 for bf16 rows, 1 for fp32 rows (measured on MI355X: fp32
// rows stream about 10% faster in 1 KB runs, bf16 rows are indifferent).
template <bool XBF16>
constexpr int conv_vpt() { return XBF16 ? 4 : 1; }
constexpr int kConvWaves = 4;       // wavefronts per workgroup
constexpr int kConvMaxBlocks = 1 << 20;

__device__ __forceinline__ void store_b128(rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0);
}
__device__ __forceinline__ void store_b64(rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)off, 0, 0);
}

// E tokens of one 16-byte unit as floats.
template <bool BF16>
__device__ __forceinline__ void unpack_unit(u32x4 u, float* v) {
  if constexpr (BF16) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[2 * k] = bf16_lo(u[k]);
      v[2 * k + 1] = bf16_hi(u[k]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __uint_as_float(u[k]);
  }
}

template <int W, bool XBF16, bool OBF16>
__global__ __launch_bounds__(kWave * kConvWaves) void conv_vec_kernel(
    const void* __restrict__ x, const float* __restrict__ weight,
    const float* __restrict__ bias, void* __restrict__ out, int64_t dim, int64_t nseg,
    int segs_per_row, uint32_t row_in_bytes, uint32_t row_out_bytes) {
  constexpr int E = XBF16 ? 8 : 4;       // tokens per unit
  constexpr int NP = W - 1;              // tokens needed from the previous unit
  constexpr int OB = OBF16 ? 2 : 4;      // output bytes per token
  constexpr int VPT = conv_vpt<XBF16>();
  const int lane = threadIdx.x % kWave;
  const int src = (lane + kWave - 1) % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  int64_t seg = (int64_t)blockIdx.x * kConvWaves + wave;
  const int64_t stride = (int64_t)gridDim.x * kConvWaves;

  for (; seg < nseg; seg += stride) {
    const int64_t row = seg / segs_per_row;
    const uint32_t u0 = (uint32_t)(seg % segs_per_row) * (kWave * VPT);
    const int64_t d = row % dim;
    float w[W];
#pragma unroll
    for (int k = 0; k < W; ++k) w[k] = weight[d * W + k];
    const float b0 = bias ? bias[d] : 0.0f;
    const rsrc_t xr = make_rsrc((const char*)x + row * row_in_bytes, row_in_bytes);
    const rsrc_t orr = make_rsrc((char*)out + row * row_out_bytes, row_out_bytes);

    u32x4 raw[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) raw[j] = load_b128(xr, (u0 + kWave * j + lane) * 16u);
    u32x4 left = {0u, 0u, 0u, 0u};
    if (NP > 0) {
      const uint32_t off = (lane == 0 && u0 > 0) ? (u0 - 1) * 16u : kPastRange;
      left = load_b128(xr, off);
    }

    // The previous unit's dwords, rotated one lane up.
    u32x4 prev = left;
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      u32x4 rot = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        // Only the dwords holding the last NP tokens are needed.
        if (NP > 0 && k >= 4 - (XBF16 ? (NP + 1) / 2 : NP)) rot[k] = __shfl(raw[j][k], src, kWave);
      }
      const u32x4 pu = (lane == 0) ? prev : rot;
      prev = rot;  // lane 0 of the next j takes lane 63 of this one

      float z[NP + E];
      float pv[E];
      unpack_unit<XBF16>(pu, pv);
#pragma unroll
      for (int k = 0; k < NP; ++k) z[k] = pv[E - NP + k];
      unpack_unit<XBF16>(raw[j], z + NP);
      float o[E];
#pragma unroll
      for (int i = 0; i < E; ++i) {
        float acc = b0;
#pragma unroll
        for (int k = 0; k < W; ++k) acc = __builtin_fmaf(w[k], z[i + k], acc);
        o[i] = acc;
      }
      const uint32_t u = u0 + kWave * j + lane;
      if constexpr (OBF16) {
        if constexpr (E == 8) {
          store_b128(orr, u * 16u, (u32x4){pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                                           pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7])});
        } else {
          store_b64(orr, u * 8u, (u32x2){pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])});
        }
      } else {
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          store_b128(orr, u * (uint32_t)(E * OB) + 16u * h,
                     (u32x4){__float_as_uint(o[4 * h]), __float_as_uint(o[4 * h + 1]),
                             __float_as_uint(o[4 * h + 2]), __float_as_uint(o[4 * h + 3])});
        }
      }
    }
  }
}

// Any row length: one thread per output token, grid-stride.
template <int W, bool XBF16, bool OBF16>
__global__ __launch_bounds__(256) void conv_scalar_kernel(
    const void* __restrict__ x, const float* __restrict__ weight,
    const float* __restrict__ bias, void* __restrict__ out, int64_t dim, int64_t seqlen,
    int64_t total) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    const int64_t row = i / seqlen, t = i % seqlen, d = row % dim;
    float acc = bias ? bias[d] : 0.0f;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int64_t s = t - (W - 1) + k;
      float v = 0.0f;
      if (s >= 0) {
        const int64_t e = row * seqlen + s;
        v = XBF16 ? __uint_as_float((uint32_t)((const uint16_t*)x)[e] << 16)
                  : ((const float*)x)[e];
      }
      acc = __builtin_fmaf(weight[d * W + k], v, acc);
    }
    if constexpr (OBF16) {
      ((uint16_t*)out)[i] = (uint16_t)(pack_bf16(acc, 0.0f) & 0xFFFFu);
    } else {
      ((float*)out)[i] = acc;
    }
  }
}

template <int W, bool XBF16, bool OBF16>
int launch_w(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
             int64_t dim, int64_t seqlen, hipStream_t st) {
  constexpr int E = XBF16 ? 8 : 4;
  const int64_t rows = batch * dim;
  if (seqlen % E == 0) {
    const int64_t units = seqlen / E;
    const int64_t per_seg = (int64_t)kWave * conv_vpt<XBF16>();
    const int64_t segs_per_row = (units + per_seg - 1) / per_seg;
    const int64_t nseg = rows * segs_per_row;
    int64_t blocks = (nseg + kConvWaves - 1) / kConvWaves;
    if (blocks > kConvMaxBlocks) blocks = kConvMaxBlocks;
    hipLaunchKernelGGL((conv_vec_kernel<W, XBF16, OBF16>), dim3((unsigned)blocks),
                       dim3(kWave * kConvWaves), 0, st, x, weight, bias, out, dim, nseg,
                       (int)segs_per_row, (uint32_t)(seqlen * (XBF16 ? 2 : 4)),
                       (uint32_t)(seqlen * (OBF16 ? 2 : 4)));
  } else {
    const int64_t total = rows * seqlen;
    int64_t blocks = (total + 255) / 256;
    if (blocks > kConvMaxBlocks) blocks = kConvMaxBlocks;
    hipLaunchKernelGGL((conv_scalar_kernel<W, XBF16, OBF16>), dim3((unsigned)blocks), dim3(256),
                       0, st, x, weight, bias, out, dim, seqlen, total);
  }
  return (int)hipGetLastError();
}

template <bool XBF16, bool OBF16>
int launch_t(const void* x, const float* weight, const float* bias, void* out, int64_t batch,
             int64_t dim, int64_t seqlen, int width, hipStream_t st) {
  switch (width) {
    case 1: return launch_w<1, XBF16, OBF16>(x, weight, bias, out, batch, dim, seqlen, st);
    case 2: return launch_w<2, XBF16, OBF16>(x, weight, bias, out, batch, dim, seqlen, st);
    case 3: return launch_w<3, XBF16, OBF16>(x, weight, bias, out, batch, dim, seqlen, st);
    default: return launch_w<4, XBF16, OBF16>(x, weight, bias, out, batch, dim, seqlen, st);
  }
}

}  // namespace

int launch_causal_conv1d(const void* x, const float* weight, const float* bias, void* out,
                         int64_t batch, int64_t dim, int64_t seqlen, int width, bool bf16_in,
                         bool bf16_out, void* stream) {
  clear_launch_error();
  hipStream_t st = (hipStream_t)stream;
  if (bf16_in)
    return bf16_out ? launch_t<true, true>(x, weight, bias, out, batch, dim, seqlen, width, st)
                    : launch_t<true, false>(x, weight, bias, out, batch, dim, seqlen, width, st);
  return bf16_out ? launch_t<false, true>(x, weight, bias, out, batch, dim, seqlen, width, st)
                  : launch_t<false, false>(x, weight, bias, out, batch, dim, seqlen, width, st);
}

}  // namespace ssd

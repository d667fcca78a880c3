// ssd_device.h -- device-side building blocks shared by the three stage
// kernels of libssd (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (64-lane wavefront, lane l):
//   v_mfma_f32_16x16x32_bf16  D[16x16] += A[16x32] * B[32x16]
//     A: lane l holds row (l % 16), eight k values (bf16x8)
//     B: lane l holds column (l % 16), eight k values
//     D: lane l holds column (l % 16), rows 4*(l/16) + r, r = 0..3
//   v_mfma_f32_16x16x4_f32    D[16x16] += A[16x4] * B[4x16]
//     A: lane l holds row (l % 16), one k value; B: column (l % 16), one k
//     D: as above
// The hardware pairs the k slots of A and B identically, so which token or
// state index a slot carries is our choice as long as both operands agree;
// every kernel documents the k <-> index map it uses.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kHeadDim = 64;  // P: the only head size built
// log2(e): exp(v) = exp2(v * log2(e)).
constexpr float kLog2e = 1.4426950408889634f;

// ---- raw buffer loads
// A buffer descriptor (base, byte range) lives in scalar registers; each lane
// passes a 32-bit byte offset.  Reads at or beyond the range return zero
// without touching memory, which is how token tiles that run past the end
// of a sequence are masked.  Offsets must stay below 2^31.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kBufferConfig = 0x00020000;  // raw 32-bit dwords (gfx9 family)

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes,
                                           kBufferConfig);
}
__device__ __forceinline__ uint32_t load_b32(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}
__device__ __forceinline__ u32x2 load_b64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ u32x4 load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ float load_f32(rsrc_t r, uint32_t off) {
  return __uint_as_float(load_b32(r, off));
}
__device__ __forceinline__ f32x4 load_f32x4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, load_b128(r, off));
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
      __builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32).  Large negative arguments
// underflow to 0, which the method tolerates: those are decays below 2^-126.
__device__ __forceinline__ float exp2_hw(float v) {
  return __builtin_amdgcn_exp2f(v);
}

// Round two floats to bf16 (nearest-even) and pack: `a` in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 r = __builtin_convertvector((f32x2){a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) {
  return __uint_as_float(w << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}

// c - h_lo and c - h_hi for the two bf16 halves of h, as fp32, with the bf16
// dot product (v_dot2c_f32_bf16, c + h . m with m = (-1, 0) or (0, -1)): one
// instruction instead of an unpack and a subtraction, and exact wherever the
// difference is representable in fp32, as it is in the splits below.  The
// multiplier pairs are held in scalar registers: the compiler would encode
// (-1, 0) as the inline constant -1.0, which the hardware reads as the fp32
// bit pattern, i.e. the pair (0, -1), and the first half would come out wrong.
__device__ __forceinline__ float sub_bf16_lo(float c, uint32_t h) {
  uint32_t m = 0x0000BF80u;   // (-1, 0)
  asm("" : "+s"(m));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, h),
                                         __builtin_bit_cast(bf16x2, m), c, false);
}
__device__ __forceinline__ float sub_bf16_hi(float c, uint32_t h) {
  uint32_t m = 0xBF800000u;   // (0, -1)
  asm("" : "+s"(m));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, h),
                                         __builtin_bit_cast(bf16x2, m), c, false);
}

// Two-term bf16 split of fp32 values: v ~= hi + lo with |v - hi - lo| about
// 2^-17 |v|.  A product with an exact bf16 operand then costs two bf16 matrix
// instructions and keeps ~16 mantissa bits, which the fp32 accumulate keeps.
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi,
                                           uint32_t& lo) {
  hi = pack_bf16(a, b);
  lo = pack_bf16(sub_bf16_lo(a, hi), sub_bf16_hi(b, hi));
}

// Three-term bf16 split of fp32 values, exact: v = hi + mid + lo.  hi is v
// rounded to bf16; v - hi is exact in fp32 and keeps at most 16 significant
// bits, mid takes the top 8 of them, and the remaining at most 8 bits fit lo
// exactly.  (Values near the bottom of the fp32 range, where bf16 goes
// subnormal, are the exception; their products are far below fp32
// resolution of any sum they join.)  The product of two split values, kept
// to its six terms of relative size 2^-16 or more, is exact to about 2^-23:
// fp32 accuracy from bf16 matrix instructions.
__device__ __forceinline__ void split3_bf16(float a, float b, uint32_t& hi, uint32_t& mid,
                                            uint32_t& lo) {
  hi = pack_bf16(a, b);
  const float ra = sub_bf16_lo(a, hi), rb = sub_bf16_hi(b, hi);
  mid = pack_bf16(ra, rb);
  lo = pack_bf16(sub_bf16_lo(ra, mid), sub_bf16_hi(rb, mid));
}

__device__ __forceinline__ u32x4 make_u32x4(const uint32_t (&a)[4]) {
  return (u32x4){a[0], a[1], a[2], a[3]};
}

// ---- LDS transpose read (ds_read_b64_tr_b16)
// Within each 16-lane group, if lane i points at row R0 + i/4, column
// C0 + 4*(i%4) of a row-major bf16 tile in LDS, lane j receives the four
// elements (R0 + k, C0 + j), k = 0..3: one column, four consecutive rows --
// the layout of a matrix-instruction operand whose k index runs along rows.
// `p` must point into LDS.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_bit_cast(
      u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)const_cast<uint16_t*>(p)));
}

// Low / high bf16 halves of two words, packed: (lo16(a), lo16(b)) and
// (hi16(a), hi16(b)).  Used to transpose 2x2 blocks of bf16.
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
  return (a & 0xFFFFu) | (b << 16);
}
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xFFFF0000u);
}

}  // namespace ssd

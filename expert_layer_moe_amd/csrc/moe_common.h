// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_kernels.h"

namespace moe {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float floatx4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// two fp32 -> packed bf16 pair (a in the low half), round to nearest even
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Four consecutive values of an expert output row y: fp32 (16 bytes), or
// bf16 (8 bytes, round to nearest even) in fp8-weight layers.
template <bool YB>
__device__ __forceinline__ void store_y4(void* y, size_t idx, floatx4 v) {
  if constexpr (YB)
    *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(y) + idx) =
        u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
  else
    *reinterpret_cast<floatx4*>(static_cast<float*>(y) + idx) = v;
}

// y rows as 24-bit floats: the top three bytes of the fp32, rounded to
// nearest even (bf16's range, 15 mantissa bits; NaN stays NaN).  Four
// consecutive values take 12 bytes: a | b << 24, b >> 8 | c << 16,
// c >> 16 | d << 8.
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));

__device__ __forceinline__ uint32_t f32_to_f24_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 8) | 0x4000u;
  return (u + 0x7fu + ((u >> 8) & 1u)) >> 8;
}

// four consecutive y values at element idx of a 24-bit y buffer
__device__ __forceinline__ void store_y24(void* y, size_t idx, floatx4 v) {
  const uint32_t a = f32_to_f24_bits(v[0]), b = f32_to_f24_bits(v[1]);
  const uint32_t c = f32_to_f24_bits(v[2]), d = f32_to_f24_bits(v[3]);
  *reinterpret_cast<u32x3*>(static_cast<uint8_t*>(y) + idx * 3) =
      u32x3{a | (b << 24), (b >> 8) | (c << 16), (c >> 16) | (d << 8)};
}

__device__ __forceinline__ floatx4 unpack_y24(u32x3 w) {
  return floatx4{__uint_as_float(w[0] << 8),
                 __uint_as_float(((w[0] >> 24) | (w[1] << 8)) << 8),
                 __uint_as_float(((w[1] >> 16) | (w[2] << 16)) << 8),
                 __uint_as_float(w[2] & 0xffffff00u)};
}

// Eight consecutive values of y (a then b): fp32 (32 bytes) or bf16 (16).
template <bool YB>
__device__ __forceinline__ void store_y8(void* y, size_t idx, floatx4 a, floatx4 b) {
  if constexpr (YB) {
    *reinterpret_cast<u32x4*>(static_cast<uint16_t*>(y) + idx) =
        u32x4{pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
              pack_bf16x2(b[2], b[3])};
  } else {
    *reinterpret_cast<floatx4*>(static_cast<float*>(y) + idx) = a;
    *reinterpret_cast<floatx4*>(static_cast<float*>(y) + idx + 4) = b;
  }
}

// 8 OCP e4m3fn codes (two dwords) -> 8 bf16, exact (every e4m3 value is a
// bf16 value).  gfx950's scaled converter applies only the exponent of its
// scale, so the scale here is 1 and block scales are applied elsewhere.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// D(16x16, fp32) += A(16x32) * B(32x16), bf16 inputs.  Lane l holds
//   A[l%16][8*(l/16) + i], B[8*(l/16) + i][l%16]  (i < 8)
//   D[4*(l/16) + i][l%16]                          (i < 4)
// The K order inside the 32-wide step is free as long as A and B agree.
__device__ __forceinline__ floatx4 mfma16x16x32(bf16x8 a, bf16x8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float floatx16;

// D(32x32, fp32) += A(32x16) * B(16x32), bf16 inputs.  Lane l holds
//   A[l%32][8*(l/32) + i], B[8*(l/32) + i][l%32]  (i < 8)
//   D[8*(r/4) + 4*(l/32) + r%4][l%32]               (r < 16)
__device__ __forceinline__ floatx16 mfma32x32x16(bf16x8 a, bf16x8 b, floatx16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float silu_mul(float g, float u) {
  return __fdividef(g, 1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x2 ld8(const void* p) {
  return *reinterpret_cast<const u32x2*>(p);
}

// Raises the completion signals (BlockSignals) of a down-projection unit.
// Called by every thread of a block once the block has stored ncols columns
// of y for rows [r0, r0 + nrows) of segment seg (r0 a multiple of 64).  Each
// wave waits for its own stores, then one release at agent scope (the write
// back of this XCD's L2) orders all of them before the counts grow.
__device__ __forceinline__ void signal_rows_done(BlockSignals bs, int seg, int r0, int nrows,
                                                 int ncols) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0 && nrows > 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    for (int b = r0 >> 6; b <= (r0 + nrows - 1) >> 6; ++b)
      __hip_atomic_fetch_add(bs.sig + (size_t)seg * bs.nb64 + b, ncols, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
  }
}

// MFMA fragment order of a [rows, K] bf16 matrix in 16-row tiles: tile t
// holds K/32 steps of 64 lanes x 8 elements, lane 16 g + m carrying row
// 16 t + m, columns 32 s + 8 g .. + 7 of step s.  A wave then fetches a whole
// fragment as 1 KB contiguous instead of 16 rows x 64 B.
__device__ __forceinline__ size_t frag_index(int row, int col, int K) {
  return (size_t)(row >> 4) * 16 * K + (size_t)((col >> 5) * 64 + ((col >> 3) & 3) * 16 + (row & 15)) * 8 +
         (col & 7);
}

}  // namespace moe

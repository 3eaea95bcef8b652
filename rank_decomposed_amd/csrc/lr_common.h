// Device helpers shared by the HIP kernels of the low-rank hot path (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return f2bf(lo) | (f2bf(hi) << 16);
}

// 16 bytes of bf16 viewed as the 8-element MFMA operand.
__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// D = A(16x32) * B(32x16) + C on bf16 inputs, fp32 accumulate.
// Operand lanes: lane l supplies row (l % 16) of A / column (l % 16) of B and
// the k-group (l / 16) of 8 consecutive k.  Result: lane l holds
// C[4 * (l / 16) + v][l % 16], v = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// Non-temporal 16-byte load for weights streamed exactly once.
__device__ __forceinline__ u32x4 ldg16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Branch-free variant of mask_tail for hot loops (selects, no early exit).
__device__ __forceinline__ u32x4 mask_tail_nb(u32x4 v, int k0, int kmax) {
  const int valid = kmax - k0;
  u32x4 m;
  m.x = (0 < valid ? 0x0000ffffu : 0u) | (1 < valid ? 0xffff0000u : 0u);
  m.y = (2 < valid ? 0x0000ffffu : 0u) | (3 < valid ? 0xffff0000u : 0u);
  m.z = (4 < valid ? 0x0000ffffu : 0u) | (5 < valid ? 0xffff0000u : 0u);
  m.w = (6 < valid ? 0x0000ffffu : 0u) | (7 < valid ? 0xffff0000u : 0u);
  return v & m;
}

// Zero the bf16 elements of a 16-byte chunk whose index (k0 + e) >= kmax.
__device__ __forceinline__ u32x4 mask_tail(u32x4 v, int k0, int kmax) {
  int valid = kmax - k0;
  if (valid >= 8) return v;
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    int e = 2 * i;
    uint32_t m = (e < valid ? 0x0000ffffu : 0u) | (e + 1 < valid ? 0xffff0000u : 0u);
    w[i] &= m;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// ---------------------------------------------------------------- buffer loads
// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero, so tiles past a matrix edge need no branches.  Word 3 is the
// gfx9-family raw-buffer configuration.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

// Bytes of a row-major bf16 view [rows, cols] with pitch ld (elements), from
// its first element to the end of the 16-byte granule holding its last one.
// As a buffer extent it keeps every load inside the view's own rows: the
// padding after the last row is never read, wherever the allocation ends.
__device__ __forceinline__ uint64_t view_bytes(int64_t rows, int64_t cols, int64_t ld) {
  return rows <= 0 || cols <= 0 ? 0 : ((((uint64_t)(rows - 1) * ld + cols) * 2 + 15) & ~15ull);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}

// NB 16-row MFMA fragments of one 32-wide k-step of a row-major bf16 matrix:
// lane l gets row row0 + nb*16 + (l & 15), elements k + 8*(l >> 4) .. +8.
template <int NB>
__device__ __forceinline__ void frag_load(u32x4 (&f)[NB], __amdgpu_buffer_rsrc_t rs, int64_t ld,
                                          int row0, int k, int lane) {
  const int row = lane & 15, kk = k + (lane >> 4) * 8;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
    f[nb] = bload(rs, (uint32_t)(((int64_t)(row0 + nb * 16 + row) * ld + kk) * 2));
}

// Zero the elements >= kmax of fragments loaded at k-step base k.
template <int NB>
__device__ __forceinline__ void frag_mask(u32x4 (&f)[NB], int k, int kmax, int lane) {
  const int kk = k + (lane >> 4) * 8;
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) f[nb] = mask_tail(f[nb], kk, kmax);
}

template <int MB, int NB>
__device__ __forceinline__ void frag_mma(f32x4 (&acc)[MB][NB], const u32x4 (&a)[MB],
                                         const u32x4 (&b)[NB]) {
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
}

__device__ __forceinline__ u32x4 lds16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace lr

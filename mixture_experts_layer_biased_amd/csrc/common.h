// Device-side helpers shared by the lcmoe kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcmoe {

constexpr int kWave = 64;

// MFMA operand / accumulator vector types.
typedef short bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Unpack a 32-bit word holding two bf16 values (low half first).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = (__bf16)lo;
  v.y = (__bf16)hi;
  return *reinterpret_cast<uint32_t*>(&v);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  __bf16 b = (__bf16)f;
  return *reinterpret_cast<uint16_t*>(&b);
}

// Four E4M3FN codes (one 32-bit word, byte 0 first) -> four fp32 values.
// gfx950 converts the OCP E4M3FN encoding in hardware; every code is exact.
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float out[4]) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  out[0] = lo[0];
  out[1] = lo[1];
  out[2] = hi[0];
  out[3] = hi[1];
}

// Eight E4M3FN codes (two words) times a block scale -> eight bf16 values
// (one 16-byte MFMA operand), each rounded once: bf16(fl32(q * s)).
__device__ __forceinline__ uint4 fp8x8_scaled_to_bf16x8(uint32_t w0, uint32_t w1, float s) {
  float a[4], b[4];
  fp8x4_to_f32(w0, a);
  fp8x4_to_f32(w1, b);
  uint4 r;
  r.x = pack_bf16x2(a[0] * s, a[1] * s);
  r.y = pack_bf16x2(a[2] * s, a[3] * s);
  r.z = pack_bf16x2(b[0] * s, b[1] * s);
  r.w = pack_bf16x2(b[2] * s, b[3] * s);
  return r;
}

// fp32 -> three bf16 planes with w = hi + mid + lo exactly: each residual of
// a round-to-nearest bf16 conversion is exact in fp32 and the last one fits
// in 8 bits (Henry, Tang & Heinecke, ARITH 2019). Products of a bf16 value
// with each plane are exact in an fp32 MFMA accumulator.
__device__ __forceinline__ void split3(float w, uint16_t& h, uint16_t& m, uint16_t& l) {
  __bf16 bh = (__bf16)w;
  float r1 = w - (float)bh;
  __bf16 bm = (__bf16)r1;
  float r2 = r1 - (float)bm;
  __bf16 bl = (__bf16)r2;
  h = *reinterpret_cast<uint16_t*>(&bh);
  m = *reinterpret_cast<uint16_t*>(&bm);
  l = *reinterpret_cast<uint16_t*>(&bl);
}

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) {
  return *reinterpret_cast<bf16x8_t*>(&v);
}

// ---- wave-level reductions (64 lanes, fixed butterfly order) ----
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, kWave);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, kWave);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}
// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    int o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  return v;
}

// gfx950 LDS has 64 four-byte banks (256 bytes per cycle): a 16-byte-per-
// lane access is conflict-free when each group of 16 lanes covers all 16
// 16-byte bank slots of a 256-byte window.
//
// Swizzled offset (in 16-byte chunks) for an LDS tile whose rows are 8
// chunks (128 bytes) wide: chunk c of row r lives at c ^ ((r >> 1) & 7), so
// sixteen consecutive rows read at the same logical chunk hit distinct slots.
__device__ __forceinline__ int swz128(int row, int chunk) {
  return row * 8 + (chunk ^ ((row >> 1) & 7));
}

}  // namespace lcmoe

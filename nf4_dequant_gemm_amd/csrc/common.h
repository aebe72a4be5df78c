// Device-side helpers shared by the HIP kernels of the NF4 QLoRA library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4q {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

// The NF4 levels and their decision thresholds, passed by value as a kernel argument.
struct Tables {
  float level[16];
  float thresh[15];
};

// Weight descriptor as the kernels see it.
struct WDesc {
  const uint8_t *codes;   // [n*k/2]
  const void *absmax;     // float[nblk] (dq == 0) or int8[nblk]
  const float *scale;     // [ceil(nblk/256)] when dq
  int64_t n, k;
  int dq;                 // 0 or 1 (runs of 256)
};

// Two floats -> packed bf16 pair (low half = lo), round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Block constant a' of flattened block index b.
__device__ __forceinline__ float block_absmax(const WDesc &w, int64_t b) {
  if (w.dq) {
    const int8_t q = reinterpret_cast<const int8_t *>(w.absmax)[b];
    return float(q) * w.scale[b >> 8];
  }
  return reinterpret_cast<const float *>(w.absmax)[b];
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8 &a, const bf16x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace nf4q

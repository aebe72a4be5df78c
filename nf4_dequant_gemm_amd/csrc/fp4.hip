// 4-bit floating-point (E2M1) weights with FP8 (E4M3) group scales (gfx950): quantise and
// dequantise. The format is the codebook variant of the NF4 layer [NVFP4 update article, "NVFP4:
// A Quantization Format for the Next Generation of Hardware": E2M1 elements, 1 sign, 2 exponent
// and 1 mantissa bits, magnitudes up to 6; groups of 16 or 32 sharing one FP8 scale].
//
//   E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6; code = sign << 3 | magnitude index.
//   Tensor scale  S   = fl32(max |w| / 2688)            (2688 = 6 * 448, E4M3's largest value)
//   Group scale   s_g = E4M3(fl32(max_g |w| / fl32(6 S)))   nearest, ties to even, saturating
//   Element code      = E2M1(fl32(w / fl32(s_g S)))         nearest, ties to even, saturating
//   Dequantised   w'  = fl32(fl32(e2m1 * s_g) * S)          (the inner product is exact)
// Groups are 16 consecutive elements of the row-major weight; codes are packed two per byte,
// the first element in the high nibble.
//
// Quantisation runs in three launches: a grid-wide maximum (per-workgroup maxima combined with
// one atomic max per workgroup on the float bits, which order like unsigned integers for
// non-negative floats; the maximum does not depend on the order), S from it (one thread), then
// one thread per group. Every launch is HBM-bound and one-off (a frozen weight is quantised once).
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr float kTscaleDiv = 2688.f;

// 8 consecutive input values (bf16 or float32) as floats.
__device__ __forceinline__ void load8(const void *w, bool f32_in, int64_t i8, float v[8]) {
  if (f32_in) {
    const float4 a = reinterpret_cast<const float4 *>(w)[2 * i8];
    const float4 b = reinterpret_cast<const float4 *>(w)[2 * i8 + 1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint4 a = reinterpret_cast<const uint4 *>(w)[i8];
    const uint32_t p[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = bf16_lo(p[j]);
      v[2 * j + 1] = bf16_hi(p[j]);
    }
  }
}

__global__ __launch_bounds__(256) void fp4_zero_kernel(uint32_t *slot) { *slot = 0u; }

__global__ __launch_bounds__(256) void fp4_amax_kernel(const void *__restrict__ w, bool f32_in,
                                                       int64_t n8, uint32_t *__restrict__ slot) {
  __shared__ float red[256];
  float m = 0.f;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n8;
       i += (int64_t)gridDim.x * blockDim.x) {
    float v[8];
    load8(w, f32_in, i, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
  }
  red[threadIdx.x] = m;
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + h]);
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(slot, __float_as_uint(red[0]));
}

__global__ __launch_bounds__(256) void fp4_tscale_kernel(float *slot) {
  *slot = __uint_as_float(*reinterpret_cast<uint32_t *>(slot)) / kTscaleDiv;
}

// E4M3 value nearest to t >= 0 (ties to the even mantissa), saturating at 448.
__device__ __forceinline__ float e4m3_round(float t) {
  if (t < 0x1p-6f) return rintf(t * 512.f) * 0x1p-9f;   // subnormals (multiples of 2^-9)
  uint32_t b = __float_as_uint(t);
  b = (b + 0x7FFFFu + ((b >> 20) & 1u)) & 0xFFF00000u;  // round the mantissa to 3 bits
  return fminf(__uint_as_float(b), 448.f);
}

// Byte of an E4M3 value v >= 0 produced by e4m3_round.
__device__ __forceinline__ uint32_t e4m3_byte(float v) {
  if (v < 0x1p-6f) return (uint32_t)(v * 512.f);
  return (__float_as_uint(v) >> 20) - (120u << 3);
}

// Magnitude index of the E2M1 value nearest to a >= 0: one comparison per midpoint, strict where
// the tie goes down (to the even mantissa below) and inclusive where it goes up.
__device__ __forceinline__ uint32_t e2m1_index(float a) {
  return (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
         (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.f);
}

__global__ __launch_bounds__(256) void fp4_quantize_kernel(const void *__restrict__ w, bool f32_in,
                                                           int64_t ngroups,
                                                           const float *__restrict__ tscale,
                                                           uint8_t *__restrict__ codes,
                                                           uint8_t *__restrict__ scales) {
  const float S = *tscale;
  const float six_S = 6.f * S;
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < ngroups;
       g += (int64_t)gridDim.x * blockDim.x) {
    float v[16];
    load8(w, f32_in, 2 * g, v);
    load8(w, f32_in, 2 * g + 1, v + 8);
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) amax = fmaxf(amax, fabsf(v[j]));
    const float s = S > 0.f ? e4m3_round(amax / six_S) : 0.f;
    const float d = s * S;
    uint32_t out[2] = {0u, 0u};
    if (d > 0.f) {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float x = v[j] / d;
        const uint32_t c = e2m1_index(fabsf(x)) | (x < 0.f ? 8u : 0u);
        // byte j / 2 of the group: element j even in bits 7..4, odd in bits 3..0
        out[j >> 3] |= c << (8 * ((j >> 1) & 3) + ((j & 1) ? 0 : 4));
      }
    }
    reinterpret_cast<uint2 *>(codes)[g] = make_uint2(out[0], out[1]);
    scales[g] = (uint8_t)e4m3_byte(s);
  }
}

__global__ __launch_bounds__(256) void fp4_dequantize_kernel(WDesc w, void *__restrict__ out,
                                                             bool f32_out) {
  const int64_t ngroups = w.n * w.k / 16;
  const float S = *w.scale;
  const uint8_t *sc = reinterpret_cast<const uint8_t *>(w.absmax);
  for (int64_t g = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; g < ngroups;
       g += (int64_t)gridDim.x * blockDim.x) {
    const uint2 cw = reinterpret_cast<const uint2 *>(w.codes)[g];
    const float s = e4m3_to_f32(sc[g]);
    float v[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const uint32_t word = (j < 8) ? cw.x : cw.y;
      const uint32_t c = (word >> (8 * ((j >> 1) & 3) + ((j & 1) ? 0 : 4))) & 15u;
      const uint32_t mi = c & 7u;
      // magnitude index -> value: 0, 0.5, 1, 1.5 (index / 2) and 2, 3, 4, 6
      const float mag = mi < 4 ? 0.5f * float(mi) : (mi == 4 ? 2.f : mi == 5 ? 3.f : mi == 6 ? 4.f : 6.f);
      const float inner = mag * s;                         // exact
      const float val = inner * S;
      v[j] = (c & 8u) ? -val : val;
    }
    if (f32_out) {
      float4 *o = reinterpret_cast<float4 *>(out) + 4 * g;
#pragma unroll
      for (int q = 0; q < 4; ++q) o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
    } else {
      uint4 *o = reinterpret_cast<uint4 *>(out) + 2 * g;
      o[0] = make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                        pack_bf16x2(v[6], v[7]));
      o[1] = make_uint4(pack_bf16x2(v[8], v[9]), pack_bf16x2(v[10], v[11]),
                        pack_bf16x2(v[12], v[13]), pack_bf16x2(v[14], v[15]));
    }
  }
}

unsigned grid_for(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 8192) b = 8192;   // 32 workgroups per CU, grid-stride beyond
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_fp4_quantize(const void *w, bool f32_in, int64_t nelem, uint8_t *codes,
                               uint8_t *scales, float *tscale, hipStream_t st) {
  if (nelem % 16) return hipErrorInvalidValue;
  uint32_t *slot = reinterpret_cast<uint32_t *>(tscale);
  fp4_zero_kernel<<<1, 1, 0, st>>>(slot);
  fp4_amax_kernel<<<dim3(grid_for(nelem / 8) < 2048 ? grid_for(nelem / 8) : 2048), dim3(256), 0, st>>>(
      w, f32_in, nelem / 8, slot);
  fp4_tscale_kernel<<<1, 1, 0, st>>>(tscale);
  fp4_quantize_kernel<<<dim3(grid_for(nelem / 16)), dim3(256), 0, st>>>(w, f32_in, nelem / 16, tscale,
                                                                       codes, scales);
  return hipGetLastError();
}

hipError_t launch_fp4_dequantize(const WDesc &w, void *out, bool f32_out, hipStream_t st) {
  fp4_dequantize_kernel<<<dim3(grid_for(w.n * w.k / 16)), dim3(256), 0, st>>>(w, out, f32_out);
  return hipGetLastError();
}

}  // namespace nf4q

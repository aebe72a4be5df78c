// NF4 quantiser and dequantiser kernels (gfx950).
//
// The quantiser encodes a weight into 4-bit NormalFloat codes with a float32 absmax per block of
// 64 and, optionally, double-quantises the block constants to int8 in runs of 256 with one
// float32 scale per run [Unsloth v0.1.463-beta release article, "About the Unsloth Project":
// 4-bit NF4 base, double quantisation of the quantisation constants]. One workgroup owns one
// run of 256 blocks (16384 elements), so the double quantisation needs no second pass, no
// workspace and no atomics: the result is bit-exact and deterministic.
#include "common.h"
#include "launch.h"

namespace nf4q {

constexpr int kQuantThreads = 256;   // 4 waves; one workgroup = one run of 256 blocks

template <bool kF32In>
__device__ __forceinline__ void load8(const void *w, int64_t e, float v[8]) {
  if (kF32In) {
    const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(w) + e);
    float4 a = p[0], b = p[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    uint4 u = *reinterpret_cast<const uint4 *>(reinterpret_cast<const uint16_t *>(w) + e);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  }
}

// Encode one value against block constant a (a > 0): number of thresholds below fl32(v / a).
__device__ __forceinline__ uint32_t encode1(float w, float a, const Tables &t) {
  const float v = w / a;   // IEEE correctly rounded division (no fast-math in this build)
  uint32_t c = 0;
#pragma unroll
  for (int j = 0; j < 15; ++j) c += (v > t.thresh[j]) ? 1u : 0u;
  return c;
}

template <bool kF32In>
__global__ __launch_bounds__(kQuantThreads) void quantize_kernel(const void *__restrict__ w,
                                                                uint32_t *__restrict__ codes,
                                                                void *__restrict__ absmax,
                                                                float *__restrict__ scale,
                                                                int64_t nblk, int dq, Tables t) {
  __shared__ float sh_a[256];
  __shared__ float sh_max[4];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t run = blockIdx.x;
  const int sub = lane >> 3;   // block within the wave's group of 8
  const int part = lane & 7;   // which 8 elements of the block this lane holds

#pragma unroll 1
  for (int it = 0; it < 8; ++it) {
    const int local = (wave * 8 + it) * 8 + sub;  // 0..255 within the run
    const int64_t b = run * 256 + local;
    const bool live = b < nblk;
    float v[8];
    if (live) {
      load8<kF32In>(w, b * 64 + part * 8, v);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = 0.f;
    }
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
    m = fmaxf(m, __shfl_xor(m, 1));
    m = fmaxf(m, __shfl_xor(m, 2));
    m = fmaxf(m, __shfl_xor(m, 4));
    uint32_t word = 0;
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const uint32_t c0 = (m > 0.f) ? encode1(v[i], m, t) : 7u;
      const uint32_t c1 = (m > 0.f) ? encode1(v[i + 1], m, t) : 7u;
      word |= ((c0 << 4) | c1) << (8 * (i >> 1));
    }
    if (live) {
      codes[b * 8 + part] = word;
      if (part == 0) {
        sh_a[local] = m;
        if (!dq) reinterpret_cast<float *>(absmax)[b] = m;
      }
    } else if (part == 0) {
      sh_a[local] = 0.f;
    }
  }
  if (!dq) return;

  // Double quantisation of this run's 256 block constants.
  __syncthreads();
  const int tid = threadIdx.x;
  const float a = sh_a[tid];
  float m = a;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) sh_max[wave] = m;
  __syncthreads();
  m = fmaxf(fmaxf(sh_max[0], sh_max[1]), fmaxf(sh_max[2], sh_max[3]));
  const float S = m / 127.0f;
  const int64_t b = run * 256 + tid;
  if (b < nblk) {
    int q = 0;
    if (S > 0.f) {
      const float r = rintf(a / S);
      q = (int)fminf(fmaxf(r, 0.f), 127.f);
    }
    reinterpret_cast<int8_t *>(absmax)[b] = (int8_t)q;
  }
  if (tid == 0) scale[run] = S;
}

// Dequantise: each thread expands one 32-bit word of codes (8 elements).
template <bool kF32Out>
__global__ __launch_bounds__(256) void dequantize_kernel(WDesc w, void *__restrict__ out,
                                                         int64_t nwords, Tables t) {
  __shared__ float lv[16];
  if (threadIdx.x < 16) lv[threadIdx.x] = t.level[threadIdx.x];
  __syncthreads();
  const uint32_t *cw = reinterpret_cast<const uint32_t *>(w.codes);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nwords;
       i += (int64_t)gridDim.x * blockDim.x) {
    const uint32_t word = cw[i];
    const float a = block_absmax(w, i >> 3);
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t byte = (word >> (8 * j)) & 0xFFu;
      v[2 * j] = lv[byte >> 4] * a;
      v[2 * j + 1] = lv[byte & 15u] * a;
    }
    if (kF32Out) {
      float4 *o = reinterpret_cast<float4 *>(reinterpret_cast<float *>(out) + i * 8);
      o[0] = make_float4(v[0], v[1], v[2], v[3]);
      o[1] = make_float4(v[4], v[5], v[6], v[7]);
    } else {
      uint4 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      u.z = pack_bf16x2(v[4], v[5]);
      u.w = pack_bf16x2(v[6], v[7]);
      reinterpret_cast<uint4 *>(out)[i] = u;
    }
  }
}

hipError_t launch_quantize(const void *w, bool f32_in, uint8_t *codes, void *absmax, float *scale,
                           int64_t nblk, int dq, const Tables &t, hipStream_t st) {
  const int64_t runs = (nblk + 255) / 256;
  if (f32_in)
    quantize_kernel<true><<<dim3((unsigned)runs), dim3(kQuantThreads), 0, st>>>(
        w, reinterpret_cast<uint32_t *>(codes), absmax, scale, nblk, dq, t);
  else
    quantize_kernel<false><<<dim3((unsigned)runs), dim3(kQuantThreads), 0, st>>>(
        w, reinterpret_cast<uint32_t *>(codes), absmax, scale, nblk, dq, t);
  return hipGetLastError();
}

hipError_t launch_dequantize(const WDesc &w, void *out, bool f32_out, const Tables &t,
                             hipStream_t st) {
  const int64_t nwords = w.n * w.k / 8;
  int64_t blocks = (nwords + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (f32_out)
    dequantize_kernel<true><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(w, out, nwords, t);
  else
    dequantize_kernel<false><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(w, out, nwords, t);
  return hipGetLastError();
}

}  // namespace nf4q

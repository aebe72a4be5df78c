// Rank-r LoRA kernels of the QLoRA layer (gfx950, bf16 MFMA).
//
// The pages give the adapter algebra (Delta W = B A at rank r, only A and B are trained)
// [Unsloth v0.1.463-beta release article, "About the Unsloth Project"]. Besides the fused GEMM,
// the layer needs three thin products whose cost is reading one [M, L] activation once:
//   rowproj : T = X A^T (forward) and U = dY B (backward), out [M, r]
//   mreduce : dA = s U^T X and dB = s dY^T T, sums over the M rows
// Sums over M are split across workgroups into float32 partials and reduced in a fixed order,
// so the results are deterministic (no atomics).
#include "common.h"
#include "launch.h"

namespace nf4q {

__device__ __forceinline__ int swz8(int row, int c) { return row * 8 + (c ^ (row & 7)); }
__device__ __forceinline__ int swz16(int row, int c) { return row * 16 + (c ^ (row & 7)); }

// ------------------------------------------------------------------------------------ rowproj
// Workgroup: 64 rows of `in` (one 16-row MFMA tile per wave) x all r (<= 128) columns; the
// reduction [l_begin, l_end) of this split runs in steps of 64. p is staged in LDS per step.
template <int TN>
__global__ __launch_bounds__(256) void rowproj_kernel(const uint16_t *__restrict__ in, int64_t ldin,
                                                      const uint16_t *__restrict__ p, int64_t ldp,
                                                      int64_t M, int64_t L, int r, int64_t lsplit,
                                                      float *__restrict__ part,
                                                      uint16_t *__restrict__ out) {
  __shared__ uint4 sP[TN * 16 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m = (int64_t)blockIdx.x * 64 + wave * 16 + (lane & 15);
  const int split = blockIdx.y;
  const int64_t lb = split * lsplit;
  const int64_t le = (lb + lsplit < L) ? lb + lsplit : L;

  f32x4 acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll 1
  for (int64_t l0 = lb; l0 < le; l0 += 64) {
    // stage p[j][l0 .. l0+63] for j < TN*16
#pragma unroll
    for (int i = 0; i < (TN * 16 * 8 + 255) / 256; ++i) {
      const int q = tid + 256 * i;
      if (q < TN * 16 * 8) {
        const int j = q >> 3, c = q & 7;
        const int64_t l = l0 + c * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < r && l < le) v = *reinterpret_cast<const uint4 *>(p + (int64_t)j * ldp + l);
        sP[swz8(j, c)] = v;
      }
    }
    bf16x8 af[2];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int64_t l = l0 + kk * 32 + (lane >> 4) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m < M && l < le) v = *reinterpret_cast<const uint4 *>(in + m * ldin + l);
      af[kk] = __builtin_bit_cast(bf16x8, v);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const bf16x8 bf =
            __builtin_bit_cast(bf16x8, sP[swz8(t * 16 + (lane & 15), kk * 4 + (lane >> 4))]);
        acc[t] = mfma16x16x32(af[kk], bf, acc[t]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = (int64_t)blockIdx.x * 64 + wave * 16 + 4 * (lane >> 4) + v;
      const int j = t * 16 + (lane & 15);
      if (row < M && j < r) {
        if (part)
          part[((int64_t)split * M + row) * r + j] = acc[t][v];
        else
          out[row * r + j] = (uint16_t)(pack_bf16x2(acc[t][v], 0.f) & 0xFFFFu);
      }
    }
}

__global__ void rowproj_reduce_kernel(const float *__restrict__ part, int64_t n, int splits,
                                      uint16_t *__restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float a = 0.f;
    for (int s = 0; s < splits; ++s) a += part[(int64_t)s * n + i];
    out[i] = (uint16_t)(pack_bf16x2(a, 0.f) & 0xFFFFu);
  }
}

int rowproj_splits(int64_t M, int64_t L) {
  const int64_t wgs = (M + 63) / 64;
  int64_t s = (1024 + wgs - 1) / wgs;
  const int64_t maxs = (L + 255) / 256;   // keep at least 256 reduction elements per split
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_rowproj(const uint16_t *in, int64_t ldin, const uint16_t *p, int64_t ldp,
                          int64_t M, int64_t L, int r, int splits, float *part, uint16_t *out,
                          hipStream_t st) {
  int64_t lsplit = (L + splits - 1) / splits;
  lsplit = (lsplit + 63) / 64 * 64;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)splits);
  float *pp = splits > 1 ? part : nullptr;
  const int tn = (r + 15) / 16;
  switch (tn) {
#define RP_CASE(T) \
  case T: rowproj_kernel<T><<<grid, dim3(256), 0, st>>>(in, ldin, p, ldp, M, L, r, lsplit, pp, out); break;
    RP_CASE(1) RP_CASE(2) RP_CASE(3) RP_CASE(4) RP_CASE(5) RP_CASE(6) RP_CASE(7) RP_CASE(8)
#undef RP_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n = M * r;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  rowproj_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(part, n, splits, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ mreduce
// Workgroup: 128 output columns c x all r (<= 128) rows, over one split of the M rows in steps of
// 128. Both operands are transposed through LDS so that MFMA fragments read 8 consecutive m.
template <int TJ>
__global__ __launch_bounds__(256) void mreduce_kernel(const uint16_t *__restrict__ P,
                                                      const uint16_t *__restrict__ Q, int64_t ldq,
                                                      int64_t M, int64_t C, int r, int64_t msplit,
                                                      float *__restrict__ part) {
  __shared__ uint4 sPt[TJ * 32 * 16];   // [j][128 m]
  __shared__ uint4 sQt[128 * 16];       // [c][128 m]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * 128;
  const int split = blockIdx.y;
  const int64_t mb = split * msplit;
  const int64_t me = (mb + msplit < M) ? mb + msplit : M;

  f32x16 acc[TJ];
#pragma unroll
  for (int t = 0; t < TJ; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[t][v] = 0.f;

  const int mg = tid & 15;     // m-group of 8
  const int cg = tid >> 4;     // c-group (Q) / j-group (P) of 8
#pragma unroll 1
  for (int64_t ms = mb; ms < me; ms += 128) {
    // Q tile: 8 rows x 8 columns per thread, transposed into sQt[c][m]
    {
      uint4 rows[8];
      const int64_t c = c0 + cg * 8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t m = ms + mg * 8 + i;
        rows[i] = (m < me && c < C) ? *reinterpret_cast<const uint4 *>(Q + m * ldq + c)
                                    : make_uint4(0, 0, 0, 0);
      }
      const uint32_t *w = reinterpret_cast<const uint32_t *>(rows);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        uint32_t h[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) h[i] = (w[i * 4 + (e >> 1)] >> ((e & 1) * 16)) & 0xFFFFu;
        sQt[swz16(cg * 8 + e, mg)] =
            make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16));
      }
    }
    // P tile: 8 rows x 8 j per thread, transposed into sPt[j][m]
    if (cg < TJ * 4) {
      uint32_t h[8][8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int64_t m = ms + mg * 8 + i;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = cg * 8 + e;
          h[e][i] = (m < me && j < r) ? P[m * r + j] : 0u;
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e)
        sPt[swz16(cg * 8 + e, mg)] = make_uint4(h[e][0] | (h[e][1] << 16), h[e][2] | (h[e][3] << 16),
                                                h[e][4] | (h[e][5] << 16), h[e][6] | (h[e][7] << 16));
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int c = kk * 2 + (lane >> 5);
      const bf16x8 bq = __builtin_bit_cast(bf16x8, sQt[swz16(wave * 32 + (lane & 31), c)]);
#pragma unroll
      for (int t = 0; t < TJ; ++t) {
        const bf16x8 ap = __builtin_bit_cast(bf16x8, sPt[swz16(t * 32 + (lane & 31), c)]);
        acc[t] = mfma32x32x16(ap, bq, acc[t]);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int t = 0; t < TJ; ++t)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int j = t * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      const int64_t c = c0 + wave * 32 + (lane & 31);
      if (j < r && c < C) part[((int64_t)split * r + j) * C + c] = acc[t][v];
    }
}

__global__ void mreduce_final_kernel(const float *__restrict__ part, int64_t C, int r, int splits,
                                     float s, bool transposed, uint16_t *__restrict__ out) {
  const int64_t n = (int64_t)r * C;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    float a = 0.f;
    for (int sp = 0; sp < splits; ++sp) a += part[(int64_t)sp * n + i];
    const uint16_t v = (uint16_t)(pack_bf16x2(s * a, 0.f) & 0xFFFFu);
    const int64_t j = i / C, c = i % C;
    if (transposed)
      out[c * r + j] = v;
    else
      out[i] = v;
  }
}

int mreduce_splits(int64_t M, int64_t C) {
  const int64_t ct = (C + 127) / 128;
  int64_t s = (1024 + ct - 1) / ct;
  const int64_t maxs = (M + 127) / 128;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_mreduce(const uint16_t *P, const uint16_t *Q, int64_t ldq, int64_t M, int64_t C,
                          int r, float s, int splits, float *part, uint16_t *out,
                          bool transposed_out, hipStream_t st) {
  int64_t msplit = (M + splits - 1) / splits;
  msplit = (msplit + 127) / 128 * 128;
  const dim3 grid((unsigned)((C + 127) / 128), (unsigned)splits);
  const int tj = (r + 31) / 32;
  switch (tj) {
#define MR_CASE(T) \
  case T: mreduce_kernel<T><<<grid, dim3(256), 0, st>>>(P, Q, ldq, M, C, r, msplit, part); break;
    MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4)
#undef MR_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)r * C;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  mreduce_final_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(part, C, r, splits, s,
                                                                     transposed_out, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------- transpose
__global__ void transpose_kernel(const uint16_t *__restrict__ src, int64_t L, int r,
                                 uint16_t *__restrict__ dst) {
  const int64_t n = L * r;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / L, l = i % L;
    dst[i] = src[l * r + j];
  }
}

hipError_t launch_transpose(const uint16_t *src, int64_t L, int r, uint16_t *dst, hipStream_t st) {
  const int64_t n = L * r;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  transpose_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(src, L, r, dst);
  return hipGetLastError();
}

}  // namespace nf4q

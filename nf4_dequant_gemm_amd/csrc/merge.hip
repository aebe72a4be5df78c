// LoRA merge of the QLoRA layer (gfx950): W' = bf16(deq(W) + s B A), the adapters folded into
// the base for a merged save, to be re-quantised by nf4_quantize for a compressed export
// [pyshine Unsloth code tour, the save.py walkthrough: merged saves, LoRA weights merged layer by
// layer; NVFP4 update article, "A More Flexible Quantization Export Pipeline"].
//
// One workgroup (4 waves) owns a 32 (n) x 128 (k) tile of W'. The rank-r product B A runs on the
// matrix cores with MFMA 16x16x32 over r (zero-padded to a multiple of 32): A [r, k] is staged in
// LDS row-major and read with the transposing LDS load ds_read_b64_tr_b16 (each lane receives 4
// consecutive rows r of one column k, the operand layout with r as the reduction index), B [n, r]
// is staged row-major and read 16 bytes per lane. The tile's codes (one 16-byte load per thread)
// and its block constants are staged in LDS as well: loaded per lane, 2 bytes at a time, they
// made the kernel request-bound (1.35 TB/s). For an E2M1 weight the constants are the tile's E4M3
// group scales (8 per row), the levels the E2M1 values, and the dequantised element is
// fl32(fl32(e2m1 * s_g) * S) with S the tensor scale. With A as the first operand, a lane holds 4
// consecutive columns k of one row n; it adds fl32(level * a') of those 4 elements (codes, block
// constant and a 16-entry level table from LDS) to s times the fp32 sum, rounds to bf16 and
// stages the tile in LDS, from which rows leave in 16-byte pieces. The work is the weight stream:
// 0.52 bytes read and 2 bytes written per element.
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kTN = 32, kTK = 128, kThreads = 256;
constexpr int kNT = kTN / 16;     // 16-row MFMA tiles per workgroup tile
constexpr int kMaxR = 128;

typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ s16x4 lds_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
// bf16 index of 8-byte unit u (4 columns) of staged A row j (rows of 128 columns = 32 units); the
// XOR puts the 8 rows x 32 bytes of a transposing read on distinct banks
__device__ __forceinline__ int aunit(int j, int u) {
  return j * kTK + ((u ^ (4 * ((j + 4 * (j >> 3)) & 7))) << 2);
}

template <bool kFP4>
__global__ __launch_bounds__(kThreads) void merge_kernel(WDesc w, const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B, int r,
                                                         float s, Tables t, uint16_t *__restrict__ out) {
  // LDS sized to the rank (dynamic): the output tile, codes, block constants and levels, then A
  // (rp rows of 128 columns) and B (32 rows of rp + 8 ranks); 21 KB at r <= 32, seven workgroups
  // per CU. The kernel is latency-bound (each workgroup loads, computes and stores in turn), so
  // occupancy sets its rate: on a 4096 x 14336 weight, r = 32, a fixed 128-rank layout with 64-row
  // tiles (2 workgroups per CU) ran 93 us, rank-sized 64-row tiles 64 us, 32-row tiles 61 us.
  extern __shared__ __align__(16) uint8_t smem[];
  const int rp = (r + 31) / 32 * 32;
  const int bstride = rp + 8;
  uint16_t *sO = reinterpret_cast<uint16_t *>(smem);                    // kTN * kTK bf16
  uint8_t *sC = smem + kTN * kTK * 2;                                    // kTN * kTK / 2 bytes
  float *sAbs = reinterpret_cast<float *>(sC + kTN * kTK / 2);          // 2 (NF4) or 8 per row
  float *sLv = sAbs + kTN * kTK / 16;                                    // 16 levels
  uint16_t *sA = reinterpret_cast<uint16_t *>(sLv + 16);                 // rp * kTK bf16
  uint16_t *sB = sA + rp * kTK;                                          // kTN * bstride bf16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int64_t N = w.n, K = w.k;
  const int64_t n0 = (int64_t)blockIdx.y * kTN, k0 = (int64_t)blockIdx.x * kTK;
  if (tid < 16) {
    if (kFP4) {   // E2M1 value of code tid: sign bit 3, magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6
      const int mi = tid & 7;
      const float mag = mi < 4 ? 0.5f * float(mi) : (mi == 4 ? 2.f : mi == 5 ? 3.f : mi == 6 ? 4.f : 6.f);
      sLv[tid] = (tid & 8) ? -mag : mag;
    } else {
      sLv[tid] = t.level[tid];
    }
  }
  const float tsc = kFP4 ? *w.scale : 1.f;
  // the tile's codes (one 16-byte load per thread of the first 128; rows past N read as zero) and
  // block constants
  {
    const __amdgpu_buffer_rsrc_t rC = make_rsrc(w.codes, N * K / 2);
    const int row = tid >> 2, piece = tid & 3;
    const int64_t n = n0 + row;
    const uint32_t off = row < kTN && n < N ? (uint32_t)((n * K + k0) / 2 + 16 * piece) : 0x80000000u;
    if (row < kTN)
      *reinterpret_cast<u32x4 *>(sC + row * (kTK / 2) + 16 * piece) =
          __builtin_amdgcn_raw_buffer_load_b128(rC, off, 0, 0);
    if (kFP4) {
      // 8 group scales per row: thread t takes row t / 8, group t % 8
      const int64_t bn = n0 + (tid >> 3), bk = k0 + 16 * (tid & 7);
      sAbs[tid] = (tid < kTN * kTK / 16 && bn < N && bk < K)
                      ? e4m3_to_f32(reinterpret_cast<const uint8_t *>(w.absmax)[(bn * K + bk) / 16])
                      : 0.f;
    } else if (tid < kTN * kTK / 64) {
      const int64_t bn = n0 + (tid >> 1), bk = k0 + 64 * (tid & 1);
      sAbs[tid] = (bn < N && bk < K) ? block_absmax(w, (bn * K + bk) / 64) : 0.f;
    }
  }
  // stage A rows 0 .. rp-1, columns k0 .. k0+127 (zero past r and past K) and B rows n0 .. n0+31,
  // ranks 0 .. rp-1 (zero past r and past N), 16 bytes at a time
  for (int i = tid; i < rp * (kTK / 8); i += kThreads) {
    const int j = i / (kTK / 8), c = i % (kTK / 8);
    const int64_t k = k0 + 8 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && k < K) v = *reinterpret_cast<const uint4 *>(A + (int64_t)j * K + k);
    *reinterpret_cast<uint2 *>(sA + aunit(j, 2 * c)) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2 *>(sA + aunit(j, 2 * c + 1)) = make_uint2(v.z, v.w);
  }
  for (int i = tid; i < kTN * (rp / 8); i += kThreads) {
    const int row = i / (rp / 8), c = i % (rp / 8);
    const int64_t n = n0 + row;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (n < N && 8 * c < r) {
      // ranks 8c .. 8c+7; r % 8 != 0 leaves a partial last piece, read element by element
      if (8 * c + 8 <= r && (r & 7) == 0) {
        v = *reinterpret_cast<const uint4 *>(B + n * r + 8 * c);
      } else {
        uint32_t e[4] = {0, 0, 0, 0};
        for (int q = 0; q < 8 && 8 * c + q < r; ++q)
          e[q >> 1] |= (uint32_t)B[n * r + 8 * c + q] << (16 * (q & 1));
        v = make_uint4(e[0], e[1], e[2], e[3]);
      }
    }
    *reinterpret_cast<uint4 *>(sB + row * bstride + 8 * c) = v;
  }
  __syncthreads();

  // wave w: columns 32 w .. 32 w + 31 (2 tiles of 16) x the tile's rows (kNT tiles of 16)
  f32x4 acc[2][kNT];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < kNT; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int ks = 0; ks < rp / 32; ++ks) {
    bf16x8 af[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int j = 32 * ks + 8 * g16 + (l16 >> 2);
      const int u = (32 * wave + 16 * kt) / 4 + (l16 & 3);
      const s16x4 lo = lds_tr16(sA + aunit(j, u));
      const s16x4 hi = lds_tr16(sA + aunit(j + 4, u));
      const short v8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      af[kt] = __builtin_bit_cast(bf16x8, v8);
    }
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      const bf16x8 bf = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4 *>(sB + (16 * nt + l16) * bstride + 32 * ks + 8 * g16));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[kt][nt] = mfma16x16x32(af[kt], bf, acc[kt][nt]);
    }
  }

  // lane: row n = n0 + 16 nt + l16, columns k .. k+3 with k = k0 + 32 w + 16 kt + 4 g16
#pragma unroll
  for (int nt = 0; nt < kNT; ++nt) {
    const int row = 16 * nt + l16;
    const int64_t n = n0 + row;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = 32 * wave + 16 * kt + 4 * g16;
      const int64_t k = k0 + kk;
      uint32_t o[2] = {0, 0};
      if (n < N && k < K) {
        // codes of k .. k+3 (two bytes, high nibble first) and the constant of their block
        const uint32_t cw = *reinterpret_cast<const uint16_t *>(sC + row * (kTK / 2) + kk / 2);
        const float a = kFP4 ? sAbs[8 * row + kk / 16] : sAbs[2 * row + kk / 64];
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t byte = (cw >> (8 * (e >> 1))) & 0xFFu;
          const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
          const float dq = kFP4 ? (sLv[code] * a) * tsc : sLv[code] * a;   // E2M1: inner product exact
          v[e] = r > 0 ? dq + s * acc[kt][nt][e] : dq;
        }
        o[0] = pack_bf16x2(v[0], v[1]);
        o[1] = pack_bf16x2(v[2], v[3]);
      }
      *reinterpret_cast<uint2 *>(sO + (16 * nt + l16) * kTK + kk) = make_uint2(o[0], o[1]);
    }
  }
  __syncthreads();
  // rows of the tile leave in 16-byte pieces (K % 64 == 0: a piece is wholly inside or past K)
  for (int i = tid; i < kTN * (kTK / 8); i += kThreads) {
    const int row = i / (kTK / 8), c = i % (kTK / 8);
    const int64_t n = n0 + row, k = k0 + 8 * c;
    if (n < N && k < K)
      *reinterpret_cast<uint4 *>(out + n * K + k) = *reinterpret_cast<const uint4 *>(sO + row * kTK + 8 * c);
  }
}

}  // namespace

hipError_t launch_merge(const WDesc &w, const uint16_t *A, const uint16_t *B, int r, float s,
                        const Tables &t, uint16_t *out, hipStream_t st) {
  if (r < 0 || r > kMaxR || w.k % 64) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((w.k + kTK - 1) / kTK), (unsigned)((w.n + kTN - 1) / kTN));
  const int rp = (r + 31) / 32 * 32;
  const size_t lds = (size_t)kTN * kTK * 2 + kTN * kTK / 2 + 4 * (kTN * kTK / 16 + 16) +
                     2 * ((size_t)rp * kTK + (size_t)kTN * (rp + 8));
  const void *fn = w.fp4 ? reinterpret_cast<const void *>(merge_kernel<true>)
                         : reinterpret_cast<const void *>(merge_kernel<false>);
  if (lds > 65536) {   // above the default dynamic-LDS limit: opt in (gfx950 has 160 KB per CU)
    const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  if (w.fp4)
    merge_kernel<true><<<grid, dim3(kThreads), lds, st>>>(w, A, B, r, s, t, out);
  else
    merge_kernel<false><<<grid, dim3(kThreads), lds, st>>>(w, A, B, r, s, t, out);
  return hipGetLastError();
}

}  // namespace nf4q

// LoRA merge of the QLoRA layer (gfx950): W' = bf16(deq(W) + s B A), the adapters folded into
// the base for a merged save, to be re-quantised by nf4_quantize for a compressed export
// [pyshine Unsloth code tour, the save.py walkthrough: merged saves, LoRA weights merged layer by
// layer; NVFP4 update article, "A More Flexible Quantization Export Pipeline"].
//
// One workgroup (4 waves) owns a 64 (n) x 128 (k) tile of W'. The rank-r product B A runs on the
// matrix cores with MFMA 16x16x32 over r (zero-padded to a multiple of 32): A [r, k] is staged in
// LDS row-major and read with the transposing LDS load ds_read_b64_tr_b16 (each lane receives 4
// consecutive rows r of one column k, the operand layout with r as the reduction index), B [n, r]
// is staged row-major and read 16 bytes per lane. With A as the first operand, a lane holds 4
// consecutive columns k of one row n; it adds fl32(level * a') of those 4 elements (the codes, the
// block constant and a 16-entry level table in LDS) to s times the fp32 sum, rounds to bf16 and
// stages the tile in LDS, from which rows leave in 16-byte pieces. The work is the weight stream:
// 0.52 bytes read and 2 bytes written per element.
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kTN = 64, kTK = 128, kThreads = 256;
constexpr int kMaxR = 128;
constexpr int kBStride = kMaxR + 8;   // bf16 per staged B row (16 bytes of padding)

typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ s16x4 lds_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}
// bf16 index of 8-byte unit u (4 columns) of staged A row j (rows of 128 columns = 32 units); the
// XOR puts the 8 rows x 32 bytes of a transposing read on distinct banks
__device__ __forceinline__ int aunit(int j, int u) {
  return j * kTK + ((u ^ (4 * ((j + 4 * (j >> 3)) & 7))) << 2);
}

__global__ __launch_bounds__(kThreads) void merge_kernel(WDesc w, const uint16_t *__restrict__ A,
                                                         const uint16_t *__restrict__ B, int r,
                                                         float s, Tables t, uint16_t *__restrict__ out) {
  __shared__ __align__(16) uint16_t sA[kMaxR * kTK];
  __shared__ __align__(16) uint16_t sB[kTN * kBStride];
  __shared__ __align__(16) uint16_t sO[kTN * kTK];
  __shared__ float sLv[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int64_t N = w.n, K = w.k;
  const int64_t n0 = (int64_t)blockIdx.y * kTN, k0 = (int64_t)blockIdx.x * kTK;
  const int rp = (r + 31) / 32 * 32;
  if (tid < 16) sLv[tid] = t.level[tid];
  // stage A rows 0 .. rp-1, columns k0 .. k0+127 (zero past r and past K) and B rows n0 .. n0+63,
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
    *reinterpret_cast<uint4 *>(sB + row * kBStride + 8 * c) = v;
  }
  __syncthreads();

  // wave w: columns 32 w .. 32 w + 31 (2 tiles of 16) x rows 0 .. 63 (4 tiles of 16)
  f32x4 acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    for (int nt = 0; nt < 4; ++nt) {
      const bf16x8 bf = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4 *>(sB + (16 * nt + l16) * kBStride + 32 * ks + 8 * g16));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[kt][nt] = mfma16x16x32(af[kt], bf, acc[kt][nt]);
    }
  }

  // lane: row n = n0 + 16 nt + l16, columns k .. k+3 with k = k0 + 32 w + 16 kt + 4 g16
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(w.codes, N * K / 2);
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t n = n0 + 16 * nt + l16;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int kk = 32 * wave + 16 * kt + 4 * g16;
      const int64_t k = k0 + kk;
      uint32_t o[2] = {0, 0};
      if (n < N && k < K) {
        const int64_t e0 = n * K + k;                 // even: codes of k, k+1 in one byte
        const uint32_t cw = __builtin_amdgcn_raw_buffer_load_b16(rC, (uint32_t)(e0 / 2), 0, 0);
        const float a = block_absmax(w, e0 / 64);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t byte = (cw >> (8 * (e >> 1))) & 0xFFu;
          const uint32_t code = (e & 1) ? (byte & 15u) : (byte >> 4);
          const float dq = sLv[code] * a;
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
  merge_kernel<<<grid, dim3(kThreads), 0, st>>>(w, A, B, r, s, t, out);
  return hipGetLastError();
}

}  // namespace nf4q

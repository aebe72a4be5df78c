// LoRA merge of the QLoRA layer (gfx950): W' = bf16(deq(W) + s B A), the adapters folded into
// the base for a merged save, to be re-quantised by nf4_quantize for a compressed export
// [pyshine Unsloth code tour, the save.py walkthrough: merged saves, LoRA weights merged layer by
// layer; NVFP4 update article, "A More Flexible Quantization Export Pipeline"].
//
// The work is the weight stream: 0.52 bytes read and 2 bytes written per element, so the kernel
// is built like a plain streaming pass. A workgroup (4 waves) owns a strip of 128 columns k and
// stages A [r, those columns] in LDS once; after that each wave works alone, with no barrier, on
// units of 16 rows x 128 columns: lane (g, l) takes row l of the unit and the 32 consecutive
// columns 32 g .. 32 g + 31, loads their 16 bytes of codes, their block constant and its 16-byte
// pieces of B row l directly into registers (the next two units' loads are in flight while a
// unit is computed and written) and puts its 64 bytes of W' in the wave's own 4 KB of LDS, from
// which the unit leaves as 4 rows x 256 contiguous bytes per store instruction (straight from the
// registers, each instruction would write 64 pieces of 16 bytes 64 bytes apart: half the rate).
// The rank-r product runs on the matrix cores: 8 MFMA 16x16x32 per 32 ranks, B as the second
// operand (lane: 8 ranks of row l) and A as the first, read from LDS with the transposing load
// ds_read_b64_tr_b16 (each lane receives 4 consecutive ranks of one column). MFMA m's output rows
// are mapped to the columns 32 q + 4 m + (0..3), q = 0..3, so that a lane, which receives output
// rows 4 g .. 4 g + 3 of every MFMA, ends up with the 32 consecutive columns above: A is staged
// with its 4-column groups permuted accordingly. Per element the lane adds fl32(level * a') (codes
// and block constant from its registers, the 16 levels from LDS) to s times the float32 sum and
// rounds once to bf16. For an E2M1 weight the constants are the E4M3 group scales (two per lane),
// the levels the E2M1 values, and the dequantised element is fl32(fl32(e2m1 * s_g) * S) with S
// the tensor scale.
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kTK = 128;          // columns of a strip
constexpr int kUnit = 16;         // rows of a unit
constexpr int kThreads = 256;
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
// LDS place of the strip's 4-column group c (0..31): MFMA m reads places 4 m .. 4 m + 3 as its
// output rows, which are to be the groups m, m + 8, m + 16, m + 24
__device__ __forceinline__ int aplace(int c) { return 4 * (c & 7) + (c >> 3); }

// LDS bytes of the kernel for padded rank rp: the 16 levels, each wave's output unit (16 rows of
// 256 bytes) and A (rp rows of 128 columns)
__host__ __device__ constexpr size_t merge_lds_bytes(int rp) {
  return 64 + 4 * kUnit * kTK * 2 + 2 * (size_t)rp * kTK;
}

// One unit's inputs as loaded into registers: the lane's 16 bytes of codes, its block constant
// words (NF4: the int8 code or the float bits, and the run scale; E2M1: the two group-scale
// bytes) and its kBQ 16-byte pieces of B (ranks 32 q + 8 g .. + 7 of row l); kBQ = rp / 32
// rounded up to 1, 2 or 4, a template parameter so that the registers in flight are those the
// rank needs.
template <int kBQ>
struct UnitIn {
  u32x4 c;
  uint32_t q, sc;
  u32x4 b[kBQ];
};

// Waves per SIMD the kernel is built for (its register budget: 128, 168 or 256 VGPRs), by kBQ.
__host__ __device__ constexpr int merge_occupancy(int bq) { return bq == 1 ? 4 : bq == 2 ? 3 : 2; }

template <bool kFP4, int kBQ>
__global__ __launch_bounds__(kThreads, merge_occupancy(kBQ)) void merge_kernel(
    WDesc w, const uint16_t *__restrict__ A, const uint16_t *__restrict__ B, int r, float s, Tables t,
    uint16_t *__restrict__ out, int per) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int rp = (r + 31) / 32 * 32;
  float *sLv = reinterpret_cast<float *>(smem);                          // 16 levels
  uint4 *sO = reinterpret_cast<uint4 *>(smem + 64);                      // 4 x 16 rows x 16 pieces
  uint16_t *sA = reinterpret_cast<uint16_t *>(smem + 64 + 4 * kUnit * kTK * 2);   // rp * kTK bf16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, g16 = lane >> 4;
  const int64_t N = w.n, K = w.k;
  const int strips = (int)((K + kTK - 1) / kTK);
  const int nun = (int)((N + kUnit - 1) / kUnit);
  // Workgroups are dealt round-robin to the 8 XCDs; each XCD gets a contiguous range of work
  // items (item = strip + strips * run), so that neighbouring strips, which read the two halves
  // of the same 128-byte lines of codes, and the strips of one run, which read the same rows of
  // B, share an L2.
  const int items = (int)gridDim.x, xcd = (int)blockIdx.x & 7;
  const int item = xcd * (items >> 3) + (xcd < (items & 7) ? xcd : (items & 7)) + ((int)blockIdx.x >> 3);
  const int64_t k0 = (int64_t)(item % strips) * kTK;
  const int ubeg = (item / strips) * per;
  const int uend = ubeg + per < nun ? ubeg + per : nun;

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
  // A rows 0 .. rp-1 of the strip's columns (zero past r and past K), 16 bytes (two 4-column
  // groups) at a time, each group at its LDS place
  for (int i = tid; i < rp * (kTK / 8); i += kThreads) {
    const int j = i / (kTK / 8), c = i % (kTK / 8);
    const int64_t k = k0 + 8 * c;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (j < r && k < K) v = *reinterpret_cast<const uint4 *>(A + (int64_t)j * K + k);
    *reinterpret_cast<uint2 *>(sA + aunit(j, aplace(2 * c))) = make_uint2(v.x, v.y);
    *reinterpret_cast<uint2 *>(sA + aunit(j, aplace(2 * c + 1))) = make_uint2(v.z, v.w);
  }
  __syncthreads();

  // Buffer resources: loads past the end of a buffer return zero (rows past N and columns past K
  // read through out-of-range offsets)
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(w.codes, N * K / 2);
  const __amdgpu_buffer_rsrc_t rQ =
      kFP4 ? make_rsrc(w.absmax, N * K / 16) : make_rsrc(w.absmax, w.dq ? N * K / 64 : N * K / 16);
  const int64_t nruns = (N * (K / 64) + 255) / 256;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(w.scale, (!kFP4 && w.dq) ? nruns * 4 : 0);
  const __amdgpu_buffer_rsrc_t rB = make_rsrc(B, r > 0 ? N * r * 2 : 0);
  constexpr uint32_t kOut = 0x80000000u;
  const int nks = rp / 32;   // 32-rank slices (0 .. kBQ)
  const bool bvec = (r & 7) == 0;
  const int64_t kl = k0 + 32 * g16;   // the lane's first column
  const bool kin = kl < K;            // K % 64 == 0: the lane's 32 columns are all inside or all past K

  auto load = [&](int u, UnitIn<kBQ> &in) {
    const int64_t n = (int64_t)u * kUnit + l16;
    const bool ok = n < N && kin;
    in.c = __builtin_amdgcn_raw_buffer_load_b128(rC, ok ? (uint32_t)((n * K + kl) / 2) : kOut, 0, 0);
    if (kFP4) {
      in.q = __builtin_amdgcn_raw_buffer_load_b16(rQ, ok ? (uint32_t)((n * K + kl) / 16) : kOut, 0, 0);
    } else {
      const int64_t b = n * (K / 64) + kl / 64;
      if (w.dq) {
        in.q = __builtin_amdgcn_raw_buffer_load_b8(rQ, ok ? (uint32_t)b : kOut, 0, 0);
        in.sc = __builtin_amdgcn_raw_buffer_load_b32(rS, ok ? (uint32_t)((b >> 8) * 4) : kOut, 0, 0);
      } else {
        in.q = __builtin_amdgcn_raw_buffer_load_b32(rQ, ok ? (uint32_t)(b * 4) : kOut, 0, 0);
      }
    }
    const uint32_t boff = n < N ? (uint32_t)(n * r * 2) : kOut;
#pragma unroll
    for (int q = 0; q < kBQ; ++q) {
      if (q < nks) {
        const int j0 = 32 * q + 8 * g16;   // the piece's first rank
        if (bvec) {
          in.b[q] = __builtin_amdgcn_raw_buffer_load_b128(rB, j0 < r ? boff + 2 * j0 : kOut, 0, 0);
        } else {   // a rank that is not a multiple of 8: element by element
          uint32_t e[4] = {0, 0, 0, 0};
          if (n < N)
            for (int x = 0; x < 8 && j0 + x < r; ++x)
              e[x >> 1] |= (uint32_t)B[n * r + j0 + x] << (16 * (x & 1));
          in.b[q] = u32x4{e[0], e[1], e[2], e[3]};
        }
      }
    }
  };

  auto unit = [&](int u, const UnitIn<kBQ> &in) {
    // the lane's block constant (E2M1: the scales of its two groups of 16)
    float a0, a1;
    if (kFP4) {
      a0 = e4m3_to_f32(in.q & 0xFFu);
      a1 = e4m3_to_f32((in.q >> 8) & 0xFFu);
    } else {
      a0 = a1 = w.dq ? int8_code(in.q) * __uint_as_float(in.sc) : __uint_as_float(in.q);
    }
    // Piece p (columns kl + 8 p .. + 7) takes MFMAs 2 p and 2 p + 1 (acc[h][v]: column
    // kl + 8 p + 4 h + v of row l), then goes through the wave's LDS: 16-byte piece c of row i at
    // place c ^ i (the 16 rows of a write and the 16 pieces of a row read hit distinct banks).
    uint4 *ob = sO + wave * (kUnit * 16);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < kBQ; ++ks) {
        if (ks < nks) {
          const bf16x8 bf = __builtin_bit_cast(bf16x8, in.b[ks]);
          const int j = 32 * ks + 8 * g16 + (l16 >> 2);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int pu = 4 * (2 * p + h) + (l16 & 3);
            const s16x4 lo = lds_tr16(sA + aunit(j, pu));
            const s16x4 hi = lds_tr16(sA + aunit(j + 4, pu));
            const short v8[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            acc[h] = mfma16x16x32(__builtin_bit_cast(bf16x8, v8), bf, acc[h]);
          }
        }
      }
      uint32_t o[4];
#pragma unroll
      for (int x = 0; x < 8; x += 2) {
        // columns kl + 8 p + x, + 1: code byte 4 p + x / 2, high nibble first
        const uint32_t byte = (in.c[p] >> (8 * (x >> 1))) & 0xFFu;
        const float a = p < 2 ? a0 : a1;
        float v[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const uint32_t code = h ? (byte & 15u) : (byte >> 4);
          const float dq = kFP4 ? (sLv[code] * a) * tsc : sLv[code] * a;   // E2M1: inner product exact
          v[h] = r > 0 ? dq + s * acc[(x + h) >> 2][(x + h) & 3] : dq;
        }
        o[x >> 1] = pack_bf16x2(v[0], v[1]);
      }
      ob[l16 * 16 + ((4 * g16 + p) ^ l16)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
    const int c = lane & 15;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = (lane >> 4) + 4 * q;
      const int64_t nr = (int64_t)u * kUnit + row, k = k0 + 8 * c;
      const uint4 v = ob[row * 16 + (c ^ row)];
      if (nr < N && k < K)
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4 *>(out + nr * K + k));
    }
  };

  // wave w takes the units ubeg + w, ubeg + w + 4, ...; two units' loads in flight ahead of the
  // unit being computed
  UnitIn<kBQ> in0, in1;
  int u = ubeg + wave;
  if (u < uend) load(u, in0);
  if (u + 4 < uend) load(u + 4, in1);
#pragma unroll 1
  for (; u + 4 < uend; u += 8) {
    unit(u, in0);
    if (u + 8 < uend) load(u + 8, in0);
    unit(u + 4, in1);
    if (u + 12 < uend) load(u + 12, in1);
  }
  if (u < uend) unit(u, in0);
}

}  // namespace

hipError_t launch_merge(const WDesc &w, const uint16_t *A, const uint16_t *B, int r, float s,
                        const Tables &t, uint16_t *out, hipStream_t st) {
  if (r < 0 || r > kMaxR || w.k % 64) return hipErrorInvalidValue;
  const int rp = (r + 31) / 32 * 32;
  const size_t lds = merge_lds_bytes(rp);
  const int bq = rp <= 32 ? 1 : rp <= 64 ? 2 : 4;
  // Workgroups of a launch: about as many per CU as the kernel's register budget lets run at
  // once, each column strip's units split into runs of `per`.
  int dev = 0, cus = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
    cus = 256;
  const int64_t strips = (w.k + kTK - 1) / kTK, nun = (w.n + kUnit - 1) / kUnit;
  const int64_t runs = std::max<int64_t>(1, std::min<int64_t>((nun + 3) / 4, (int64_t)cus * merge_occupancy(bq) / strips));
  const int64_t per = (nun + runs - 1) / runs;
  const int64_t grid = strips * ((nun + per - 1) / per);
  const dim3 gd((unsigned)grid), bd(kThreads);
  const int p = (int)per;
  if (w.fp4) {
    if (bq == 1) merge_kernel<true, 1><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
    else if (bq == 2) merge_kernel<true, 2><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
    else merge_kernel<true, 4><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
  } else {
    if (bq == 1) merge_kernel<false, 1><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
    else if (bq == 2) merge_kernel<false, 2><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
    else merge_kernel<false, 4><<<gd, bd, lds, st>>>(w, A, B, r, s, t, out, p);
  }
  return hipGetLastError();
}

}  // namespace nf4q

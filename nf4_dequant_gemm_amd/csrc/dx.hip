// Fused input-gradient kernel of the QLoRA layer: dX = dY deq(W) + s U A (gfx950).
//
// The backward pass of the frozen-base QLoRA layer needs the gradient through the dequantised
// base weight and through the adapters; W itself gets no gradient [Unsloth v0.1.463-beta release
// article, "About the Unsloth Project": the 4-bit base is frozen, only the adapters train; the
// Unsloth kernels rewrite the backward pass]. As in the forward kernel, the NF4 weight is decoded
// on the fly into LDS and the rank-r term runs as extra reduction steps into the same tile.
//
// Work split. One workgroup (4 waves, 2 x 2) owns a 256 x 256 tile of dX (rows m, columns k) and
// walks the reduction index n in steps of 64. The reduction runs over the weight's ROW index,
// so the decoded weight tile is stored transposed in LDS (256 k-rows of 64 n). Thread t decodes
// two weight rows (n, n+1) x 32 columns per step through two 16-entry bf16 tables (one per row
// and block), pairs the rows per column with byte permutes and writes 4-byte (n, n+1) words.
//
// Pipeline per step s: the dY tile of step s+1 goes straight to LDS buffer (s+1) & 1 by DMA
// (buffer_load ... lds, issued at the start of the step, so its latency hides behind a whole
// step) and the codes of step s+2 are loaded into registers; the 64 MFMAs of step s run on LDS
// buffer s & 1 while the decoded, transposed weight of step s+1 is written to buffer (s+1) & 1
// between MFMA issues.
//
// LDS: the dY tile has rows of 64 bf16 = 8 chunks of 16 bytes, chunk c of row r at slot
// c ^ ((r >> 1) & 7). The transposed weight tile pads its rows to 144 bytes (conflict-free for
// both the 4-byte writes and the 16-byte fragment reads) and keeps column k in row
// k ^ ((k / 32) & 1).
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kT = 256;
constexpr int kS = 64;
constexpr int kThreads = 256;
constexpr int kChunks = kT * kS / 8;

__device__ __forceinline__ int swzd(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }
// Transposed weight tile: row p(k) of column k (0..255) holds 64 n-values in 144 bytes (128 bytes
// of data, 16 of padding). p(k) flips the lowest bit of k in odd groups of 32 columns, so the two
// half-waves of a write (columns k and k + 32) land in different halves of the bank window.
constexpr int kWRow = 36;    // 32-bit words per transposed row (144 bytes)
__device__ __forceinline__ int prow(int k) { return k ^ ((k >> 5) & 1); }

__device__ __forceinline__ int tile_remap(int hw, int tiles) {
  const int per = tiles >> 3, rem = tiles & 7, x = hw & 7;
  return x * per + (x < rem ? x : rem) + (hw >> 3);
}

struct CStage2 {
  u32x4 c[2];        // 16 bytes of codes (32 columns) of rows n and n+1
  uint32_t q[2];     // block constants (int8 or float bits)
  uint32_t sc[2];    // run scale bits (double quantisation)
};

// LoRA step staging: A-side U columns jb..jb+63 (rows m), B-side s * A^T (rows k, columns j).
__device__ void stage_lora_dx(const GemmArgs &g, int64_t m0, int64_t k0, int jb, uint4 *sA, uint32_t *sB) {
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int i = 0; i < 8; ++i) {
    const int q = tid + kThreads * i;
    const int row = q >> 3, c = q & 7;
    uint32_t wa[4], wb[4];
    const int64_t m = m0 + row, k = k0 + row;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int j0 = jb + c * 8 + e, j1 = j0 + 1;
      uint32_t lo = 0, hi = 0;
      if (m < g.M) {
        if (j0 < g.r) lo = g.lora_a[m * g.r + j0];
        if (j1 < g.r) hi = g.lora_a[m * g.r + j1];
      }
      wa[e >> 1] = lo | (hi << 16);
      float b0 = 0.f, b1 = 0.f;
      if (k < g.C) {
        if (j0 < g.r) b0 = bf16_to_f32(g.lora_b[(int64_t)j0 * g.C + k]);
        if (j1 < g.r) b1 = bf16_to_f32(g.lora_b[(int64_t)j1 * g.C + k]);
      }
      wb[e >> 1] = pack_bf16x2(g.s * b0, g.s * b1);
    }
    sA[swzd(row, c)] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    reinterpret_cast<uint4 *>(sB)[prow(row) * (kWRow / 4) + c] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  }
}

template <bool kDQ>
__global__ __launch_bounds__(kThreads, 1) void dx_fused_kernel(GemmArgs g) {
  // dY tiles [m][n], two separate arrays: the compiler then knows that reads of one do not
  // alias the DMA in flight into the other (one array of two would make it wait for the DMA)
  __shared__ uint4 sY0[kChunks], sY1[kChunks];
  auto ybuf = [&](int P) { return P ? sY1 : sY0; };
  __shared__ uint32_t sW[2][kT * kWRow];   // decoded weight tiles, transposed [p(k)][n], padded

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wk = wave & 1;
  const int tiles_k = (int)((g.C + kT - 1) / kT);
  const int logical = tile_remap(blockIdx.x, gridDim.x);
  const int64_t m0 = (int64_t)(logical / tiles_k) * kT;
  const int64_t k0 = (int64_t)(logical % tiles_k) * kT;
  const int64_t K = g.w.k, N = g.w.n;
  const int64_t rows_m = (g.M - m0 < kT) ? g.M - m0 : kT;
  const int kblk = (int)(K / kS);
  const int nsteps = (int)((N + kS - 1) / kS);
  const int last = nsteps - 1;

  // dY rows m0.. (reduction index n contiguous). Chunks past n = N read the next row's values
  // (finite) and meet weight rows past N, which decode to exact zeros (codes and constants read
  // past the end of their buffers are 0), so they add nothing.
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(g.a_side + m0 * N, rows_m * N * 2);
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.w.codes, N * (K / 2));
  const __amdgpu_buffer_rsrc_t rQ =
      kDQ ? make_rsrc(g.w.absmax, N * kblk) : make_rsrc(g.w.absmax, N * kblk * 4);
  const int64_t nruns = (N * kblk + 255) / 256;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.w.scale, kDQ ? nruns * 4 : 0);

  // dY DMA: instruction i of wave w fills the 1 KB of the tile holding rows 8 (8 w + i) .. +7;
  // lane L writes physical chunk L % 8 of row 8 (8 w + i) + L / 8, i.e. logical chunk
  // (L % 8) ^ ((row >> 1) & 7) (the same swizzle as swzd).
  uint32_t yoff[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * (8 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    yoff[i] = (uint32_t)(row * N * 2 + c * 16);
  }
  // Weight rows n = 64 s + 2 np + {0, 1}, columns k0 + 32 kq .. + 31.
  const int np = tid & 31, kq = tid >> 5;
  const int64_t kcol = k0 + kq * 32;
  const bool kvalid = kcol < K;
  const uint32_t coff = (uint32_t)((2 * np) * (K / 2) + (kvalid ? kcol / 2 : 0));
  const uint32_t crow = (uint32_t)(K / 2);
  const uint32_t qoff = (uint32_t)((2 * np) * kblk + (kvalid ? kcol / 64 : 0));

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  auto dma_y = [&](int s, uint4 *sA) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rY, (__attribute__((address_space(3))) void *)(sA + (8 * wave + i) * 64), 16, yoff[i],
          s * 128, 0, 0);
  };
  constexpr int kCodeLoads = 2 * (kDQ ? 3 : 2);   // loads issued by load_c
  auto load_c = [&](int s, CStage2 &c) {
    const uint32_t rowbase = (uint32_t)(s * kS);   // first weight row of the step
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      c.c[r] = __builtin_amdgcn_raw_buffer_load_b128(rC, coff + (rowbase + r) * crow, 0, 0);
      const uint32_t b = qoff + (rowbase + r) * (uint32_t)kblk;
      if (kDQ) {
        c.q[r] = __builtin_amdgcn_raw_buffer_load_b8(rQ, b, 0, 0);
        c.sc[r] = __builtin_amdgcn_raw_buffer_load_b32(rS, (b >> 8) * 4, 0, 0);
      } else {
        c.q[r] = __builtin_amdgcn_raw_buffer_load_b32(rQ, b * 4, 0, 0);
      }
    }
  };
  auto absmax_of = [&](const CStage2 &c, int r) {
    const float a = kDQ ? int8_code(c.q[r]) * __uint_as_float(c.sc[r]) : __uint_as_float(c.q[r]);
    return kvalid ? a : 0.f;
  };
  auto cword = [](const CStage2 &c, int r, int w) {
    const u32x4 &v = c.c[r];
    return w == 0 ? v.x : w == 1 ? v.y : w == 2 ? v.z : v.w;
  };
  // Transposed weight write: the 4-byte word (n, n+1) of column k = kq * 32 + kl.
  auto write_w = [&](uint32_t *sB, int kl, uint32_t v) { sB[prow(kq * 32 + kl) * kWRow + np] = v; };
  auto decode_all = [&](const CStage2 &c, uint32_t *sB) {
    RowTable t[2];
#pragma unroll
    for (int r = 0; r < 2; ++r) t[r] = make_row_table(absmax_of(c, r), g.t);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t o[2][4];
#pragma unroll
      for (int r = 0; r < 2; ++r) decode8(t[r], cword(c, r, w), o[r]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        write_w(sB, w * 8 + 2 * q, perm(o[1][q], o[0][q], 0x05040100u));
        write_w(sB, w * 8 + 2 * q + 1, perm(o[1][q], o[0][q], 0x07060302u));
      }
    }
  };
  auto wfrag = [&](const uint32_t *sB, int t, int c) {
    return __builtin_bit_cast(
        bf16x8, reinterpret_cast<const uint4 *>(sB)[prow(wk * 128 + t * 32 + (lane & 31)) * (kWRow / 4) + c]);
  };
  auto read_frags = [&](const uint4 *sA, const uint32_t *sB, int kk, bf16x8 af[4], bf16x8 bw[4]) {
    const int c = kk * 2 + (lane >> 5);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      af[t] = __builtin_bit_cast(bf16x8, sA[swzd(wm * 128 + t * 32 + (lane & 31), c)]);
      bw[t] = wfrag(sB, t, c);
    }
  };
  auto mma = [&](const uint4 *sA, const uint32_t *sB) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[4], bw[4];
      read_frags(sA, sB, kk, af, bw);
#pragma unroll
      for (int tk = 0; tk < 4; ++tk)
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tk][tm] = mfma32x32x16(bw[tk], af[tm], acc[tk][tm]);
    }
  };

  // One step: MFMAs on buffer P; dY chunks (yn) and the transposed weight (decoded from cn) of
  // step s+1 go to buffer P^1 in between; loads of step s+2 go to ym / cm.
  auto body = [&](int s, int P, CStage2 &cm, CStage2 &cn) {
    const int s1 = s + 1 < last ? s + 1 : last;
    const int s2 = s + 2 < last ? s + 2 : last;
    dma_y(s1, ybuf(P ^ 1));
    __builtin_amdgcn_sched_barrier(0);   // the DMA stays ahead of the code loads (see the wait)
    load_c(s2, cm);
    const uint4 *A = ybuf(P);
    const uint32_t *B = sW[P];
    uint32_t *Bn = sW[P ^ 1];
    bf16x8 af[2][4], bw[2][4];
    read_frags(A, B, 0, af[0], bw[0]);

    float a[2];
    a[0] = absmax_of(cn, 0);
    a[1] = absmax_of(cn, 1);
    uint32_t pk[2][8];
    RowTable t[2];
    Dec8 dx[2];
    uint32_t o[2][4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int tk = i >> 2, tm = i & 3;
        const int slot = kk * 16 + i;
        acc[tk][tm] = mfma32x32x16(bw[kk & 1][tk], af[kk & 1][tm], acc[tk][tm]);
        if (kk < 3 && i < 4) {
          const int c = (kk + 1) * 2 + (lane >> 5);
          af[(kk + 1) & 1][i] = __builtin_bit_cast(bf16x8, A[swzd(wm * 128 + i * 32 + (lane & 31), c)]);
          bw[(kk + 1) & 1][i] = wfrag(B, i, c);
        }
        if (slot < 8) {
          // tables: slot = 4 r + quarter
          const int r = slot >> 2, qq = slot & 3;
          pk[r][2 * qq] = pack_bf16x2(g.t.level[4 * qq] * a[r], g.t.level[4 * qq + 1] * a[r]);
          pk[r][2 * qq + 1] = pack_bf16x2(g.t.level[4 * qq + 2] * a[r], g.t.level[4 * qq + 3] * a[r]);
          t[r].L[qq] = perm(pk[r][2 * qq + 1], pk[r][2 * qq], 0x06040200u);
          t[r].H[qq] = perm(pk[r][2 * qq + 1], pk[r][2 * qq], 0x07050301u);
        } else {
          // word w: slots 8 + 14 w .. : pieces of rows 0 and 1 interleaved (10 slots), then the
          // 4 transposed pairs (4 slots)
          const int w = (slot - 8) / 14, u = (slot - 8) % 14;
          if (u < 10) {
            const int r = u & 1, p = u >> 1;
            if (p == 0) dx[r].d = cword(cn, r, w);
            dec_piece(t[r], dx[r], p, o[r]);
          } else {
            const int q = u - 10;
            write_w(Bn, w * 8 + 2 * q, perm(o[1][q], o[0][q], 0x05040100u));
            write_w(Bn, w * 8 + 2 * q + 1, perm(o[1][q], o[0][q], 0x07060302u));
          }
        }
      }
    }
    // the dY DMA of step s+1 (older than the code loads of step s+2) has landed
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCodeLoads) : "memory");
  };

  CStage2 c0, c1;
  dma_y(0, ybuf(0));
  load_c(0, c0);
  load_c(nsteps > 1 ? 1 : 0, c1);
  decode_all(c0, sW[0]);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int s = 0;
#pragma unroll 1
  for (; s + 2 <= nsteps; s += 2) {
    body(s, 0, c0, c1);
    body(s + 1, 1, c1, c0);
  }
  if (s < nsteps) body(s, 0, c0, c1);
  __syncthreads();

  const int nlora = (g.r + kS - 1) / kS;
#pragma unroll 1
  for (int j = 0; j < nlora; ++j) {
    const int buf = j & 1;
    stage_lora_dx(g, m0, k0, j * kS, ybuf(buf), sW[buf]);
    __syncthreads();
    mma(ybuf(buf), sW[buf]);
    __syncthreads();
  }

  // Epilogue: with the weight tile as the MFMA A operand, a lane holds columns k..k+3 of row m.
#pragma unroll
  for (int tk = 0; tk < 4; ++tk)
#pragma unroll
    for (int tm = 0; tm < 4; ++tm) {
      const int64_t m = m0 + wm * 128 + tm * 32 + (lane & 31);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + wk * 128 + tk * 32 + 8 * q + 4 * (lane >> 5);
        if (m < g.M && k < g.C) {
          const uint2 v = make_uint2(pack_bf16x2(acc[tk][tm][4 * q], acc[tk][tm][4 * q + 1]),
                                     pack_bf16x2(acc[tk][tm][4 * q + 2], acc[tk][tm][4 * q + 3]));
          *reinterpret_cast<uint2 *>(g.out + m * g.ldo + k) = v;
        }
      }
    }
}

}  // namespace

hipError_t launch_gemm_dx(const GemmArgs &g, hipStream_t st) {
  const int64_t tiles = ((g.C + kT - 1) / kT) * ((g.M + kT - 1) / kT);
  if (g.w.dq)
    dx_fused_kernel<true><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else
    dx_fused_kernel<false><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace nf4q

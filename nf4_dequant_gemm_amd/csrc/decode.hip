// Decode-shaped (M <= 64) forward kernel: dequantise-on-the-fly GEMV of the NF4 weight with the
// LoRA correction, Y = X deq(W)^T + s T B^T, bound by the weight stream [pyshine Unsloth code
// tour, "Why You Need This": dequantize-on-the-fly GEMV for NF4 weights; "Inside Unsloth"
// listing, "What You'll Learn", "LoRA and QLoRA": dequant, matmul and LoRA correction in one
// launch; NVFP4 update article, "NVFP4: A Quantization Format for the Next Generation of
// Hardware": a separate dequantisation step eats into the bandwidth that 4-bit storage saves].
//
// With M <= 64 rows of X the work is the 0.52 bytes per weight element streamed from HBM, so the
// kernel is organised around the stream and around the vector-memory pipeline of the CU, whose
// L1 tag lookups (not HBM) limit a naive version:
//   * codes reach LDS by DMA (buffer_load ... lds) in fully coalesced 1 KB pieces, two stages
//     ahead in a three-slot ring; a row's 16-byte chunks are XOR-swizzled by the row index so
//     the MFMA-layout reads below hit 64 distinct banks;
//   * the block constants of a stage (int8 codes and run scales of the double quantisation, or
//     fp32 values) reach LDS by DMA too, one coalesced piece per row; every LDS byte arrives by
//     DMA, so no LDS store waits for the DMA stages still in flight;
//   * X fragments are read straight from global memory (L2-resident: every workgroup reads the
//     same X), each instruction covering whole 64-byte pieces of 16 rows;
//   * a code byte (two elements) becomes a pair of bf16 NF4 levels through a 256-entry table
//     replicated 16 times in LDS: one LDS read and two address instructions per two elements
//     (a register decode with byte permutes costs about 29 vector instructions per 8 elements,
//     and a wave64 vector instruction occupies the SIMD for 4 cycles, so the vector ALU is the
//     scarcer unit here); the table reads of the next row group are issued before the MFMAs of
//     the current one;
//   * MFMA 16x16x32 multiplies the unscaled levels by X; the block constant a (per weight row and
//     64-element block) is applied to the block's fp32 partial sum afterwards:
//         Y[m][n] += a(n, b) * sum_{k in block b} X[m][k] * level(code[n][k]).
// Workgroup: 64 weight rows, 8 waves; wave w takes block w of each 8-block stage for all 64 rows
// (two waves per SIMD per workgroup hide one another's LDS and barrier waits), and the partial
// sums are added through LDS at the end.
// Numerics: this path rounds the NF4 level (not level * a) to bf16 before the product, so it is
// not bit-identical to the large-M kernel; both stay within the layer's tolerance.
// Requires K % 256 == 0 (a whole number of 4-block groups per row keeps the block-constant DMA
// dword-aligned and each group inside one scale run); the host sends other shapes to the
// large-M kernel.
#include <type_traits>

#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kRows = 64;          // weight rows per workgroup
constexpr int kWaves = 8;          // = blocks per stage
constexpr int kThreads = kWaves * 64;
constexpr int kBlkPerStage = kWaves;                      // 64-element blocks per stage
constexpr int kStages = 3;
constexpr int kStageBytes = kRows * kBlkPerStage * 32;   // 16 KB
constexpr int kCopies = 16;        // level-pair table copies: lane l reads copy l % 16
constexpr int kTabBytes = 256 * kCopies * 4;              // 16 KB
// block constants of a stage: 64 rows x 8 blocks, as int8 codes + one scale per row and 4-block
// half (each copied twice, see the DMA below), or as fp32: 2 KB either way
constexpr int kConstBytes = kRows * kBlkPerStage * 4;

struct DecArgs {
  const uint16_t *X;
  const uint16_t *T;
  const uint16_t *B;
  WDesc w;
  int64_t M;
  int r;
  float s;
  uint16_t *Y;
  Tables t;
};

template <int MT, int kFmt>
__device__ __forceinline__ void decode_body(const DecArgs &g) {
  constexpr bool kDQ = kFmt == 1;
  // [0, 16 KB) level-pair table, then the ring of kStages slots (16 KB of codes + the stage's
  // block constants). After the main loop the area from 0 holds the cross-wave reduction.
  constexpr int kSlot = kStageBytes + kConstBytes;
  constexpr int kRedBytes = 4 * MT * 16 * 64 * 4;
  constexpr int kArea = kTabBytes + kStages * kSlot;
  static_assert(kRedBytes <= kArea, "reduction area");
  __shared__ __align__(16) uint8_t smem[kArea];
  uint8_t *stab = smem;
  uint8_t *sring = smem + kTabBytes;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = g.w.k, N = g.w.n;
  const int kblk = (int)(K / 64);
  const int nst = (kblk + kBlkPerStage - 1) / kBlkPerStage;
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t rows = (N - n0 < kRows) ? N - n0 : kRows;
  // Workgroups walk the stages in rotated order (logical stage st is stage (st + rot) % nst of
  // K), so that at any moment they read different parts of the shared X and spread over the L2
  // channels instead of all hitting the same few lines.
  const int rot = (int)(blockIdx.x % (unsigned)nst);
  auto ph = [&](int st) { const int p = st + rot; return p >= nst ? p - nst : p; };

  // byte -> (level[hi nibble], level[lo nibble]) as a packed bf16 pair (the high nibble is the
  // earlier element); threads e and e + 256 write copies 0..7 and 8..15 of byte e
  {
    const int e = tid & 255;
    const uint32_t v = pack_bf16x2(g.t.level[e >> 4], g.t.level[e & 15]);
    uint4 *dst = reinterpret_cast<uint4 *>(stab + e * kCopies * 4 + (tid >> 8) * (kCopies * 2));
#pragma unroll
    for (int c = 0; c < kCopies / 8; ++c) dst[c] = make_uint4(v, v, v, v);
  }

  const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.w.codes + n0 * (K / 2), rows * (K / 2));
  const __amdgpu_buffer_rsrc_t rQ =
      kDQ ? make_rsrc(reinterpret_cast<const int8_t *>(g.w.absmax) + n0 * kblk, rows * kblk)
          : make_rsrc(reinterpret_cast<const float *>(g.w.absmax) + n0 * kblk, rows * kblk * 4);
  const int64_t nruns = (N * kblk + 255) / 256;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.w.scale, kDQ ? nruns * 4 : 0);
  const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.X, g.M * K * 2);

  // Code DMA: instruction i of wave w fills stage bytes [(2w + i) KB, +1 KB) = rows
  // 4 (2w + i) .. +3 (256 bytes each); lane L writes physical chunk L % 16 of row (L / 16), which
  // holds logical chunk (L % 16) ^ (row % 16) of that row's 256-byte stage slice. Rows at or
  // past N read as zero (outside the buffer resource).
  uint32_t doff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = (wave * 2 + i) * 4 + (lane >> 4);
    const int lc = (lane & 15) ^ (row & 15);
    doff[i] = (uint32_t)(row * (K / 2) + lc * 16);
  }
  // Block-constant DMA, one 64-lane instruction per wave and stage:
  //   double quantisation: waves 0..3 copy the int8 codes, lane l -> dword (l % 2) of the 8
  //     codes of row 16 w + (l % 32) / 2; waves 4..7 copy the scales, lane l -> run scale of
  //     4-block half (l % 2) of row 16 (w - 4) + (l % 32) / 2 (a 4-aligned group of 4 blocks
  //     never straddles a run). Lanes 32..63 repeat lanes 0..31 into the second half of the
  //     wave's 256-byte piece (a branch around them would make the count of loads in flight
  //     unknown to the compiler).
  //   fp32: wave w, lane l -> value (64 w + l) % 8 of row (64 w + l) / 8.
  const __amdgpu_buffer_rsrc_t rCst = kDQ ? (wave < 4 ? rQ : rS) : rQ;
  uint32_t coff;
  if (kDQ) {
    const int row = (wave & 3) * 16 + ((lane & 31) >> 1), h = lane & 1;
    coff = wave < 4 ? (uint32_t)(row * kblk + 4 * h)                     // + 8 st
                    : (uint32_t)((n0 + row) * kblk + 4 * h);             // block, not yet >> 8
  } else {
    const int idx = 64 * wave + lane;
    coff = (uint32_t)(((idx >> 3) * kblk + (idx & 7)) * 4);              // + 32 st
  }
  auto dma = [&](int st) {
    uint8_t *dst = sring + (st % kStages) * kSlot;
    st = ph(st);
#pragma unroll
    for (int i = 0; i < 2; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rC, (__attribute__((address_space(3))) void *)(dst + (wave * 2 + i) * 1024), 16,
          doff[i] + st * (kBlkPerStage * 32), 0, 0, 0);
    uint8_t *cdst = dst + kStageBytes;
    if (kDQ) {
      const uint32_t o = wave < 4 ? coff + st * kBlkPerStage
                                  : ((coff + st * kBlkPerStage) >> 8) * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rCst, (__attribute__((address_space(3))) void *)(cdst + wave * 256), 4, o, 0, 0, 0);
    } else {
      // fp32 constants: 8 blocks x 4 bytes per row and stage
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rQ, (__attribute__((address_space(3))) void *)(cdst + wave * 256), 4,
          coff + st * (kBlkPerStage * 4), 0, 0, 0);
    }
  };
  constexpr int kDmaPerStage = 3;

  const int nl = lane & 15, gl = lane >> 4;   // MFMA lane: column (weight row) and k-group

  // This wave's X fragments of a stage, loaded one stage ahead (lane: row mt*16 + nl, columns
  // kbase + 32 t + 8 gl .. +7 of the wave's block). Every load is issued, so a stage issues
  // exactly 2 MT of them, which the stage waits below count.
  struct Opnd {
    bf16x8 x[MT][2];
  };
  // lane part of the X offsets (bytes); the stage's column base goes in the scalar offset
  uint32_t xoff[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int t = 0; t < 2; ++t) xoff[mt][t] = (uint32_t)(((mt * 16 + nl) * K + t * 32 + gl * 8) * 2);
  auto load_opnd = [&](int st, Opnd &o) {
    const int kb2 = (ph(st) * kBlkPerStage + wave) * 128;   // column base in bytes
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        o.x[mt][t] = __builtin_bit_cast(
            bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rX, xoff[mt][t], kb2, 0));
  };
  constexpr int kXPerStage = 2 * MT;

  f32x4 acc[MT][4];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Prologue (K >= 256, so nst >= 1). Stage 1 is requested even when nst == 1: it then reads
  // beyond the row or outside the buffer into a slot nobody reads, and the number of loads in
  // flight stays the same on every path into the stage loop.
  Opnd o0, o1;
  dma(0);
  load_opnd(0, o0);
  __builtin_amdgcn_sched_barrier(0);
  dma(1);

  const uint32_t lane_off = (uint32_t)(lane & (kCopies - 1)) * 4;
  // One stage: the X operands of st are in cur; with kNext those of st + 1 are loaded into nxt,
  // with kDma the codes and constants of st + 2 are requested. Both roles are compile-time so
  // every path is straight-line code with a fixed number of loads in flight. The loop runs two
  // stages per trip so cur and nxt swap roles without register copies (a copy would wait for
  // the loads).
  auto stage = [&](auto next_tag, auto dma_tag, int st, const Opnd &cur, Opnd &nxt) {
    constexpr bool kNext = decltype(next_tag)::value, kDma = decltype(dma_tag)::value;
    // Issue order per stage: X of st + 1, then the DMA of st + 2, so the newest loads are
    // [DMA st+2, X st+1, DMA st+1, X st]; everything older, the DMA of st included, must be done
    // before the barrier that opens the stage (the table writes too: lgkmcnt).
    if constexpr (kNext) load_opnd(st + 1, nxt);
    __builtin_amdgcn_sched_barrier(0);   // keep the X loads ahead of the DMA
    if constexpr (kDma) {
      dma(st + 2);
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * kDmaPerStage + 2 * kXPerStage)
                   : "memory");
    } else if constexpr (kNext) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kDmaPerStage + 2 * kXPerStage)
                   : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const uint8_t *S = sring + (st % kStages) * kSlot;
    const uint8_t *C = S + kStageBytes;
    // the lane's code dwords of (row 16 rg + nl, the wave's block, half t): logical bytes
    // 32 w + 16 t + 4 gl .. +3 of the row's stage slice, in chunk (2 w + t) stored at
    // chunk ^ (row % 16)
    uint32_t cw[4][2];
#pragma unroll
    for (int rg = 0; rg < 4; ++rg)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int row = rg * 16 + nl, chunk = wave * 2 + t;
        cw[rg][t] = *reinterpret_cast<const uint32_t *>(
            S + row * 256 + ((chunk ^ (row & 15)) << 4) + gl * 4);
      }
    // block constants a(row 16 rg + nl, the wave's block); blocks past K get zero
    float ca[4];
    const bool live = ph(st) * kBlkPerStage + wave < kblk;
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int row = rg * 16 + nl;
      float a;
      if (kDQ) {
        // int8 code times the scale of the row's 4-block half
        const int q = reinterpret_cast<const int8_t *>(C)[(row >> 4) * 256 + (row & 15) * 8 + wave];
        const float sc = *reinterpret_cast<const float *>(
            C + 1024 + (row >> 4) * 256 + ((row & 15) * 2 + (wave >> 2)) * 4);
        a = float(q) * sc;
      } else {
        a = *reinterpret_cast<const float *>(C + (row * 8 + wave) * 4);
      }
      ca[rg] = live ? a : 0.f;
    }
    // table reads of row group rg (both halves of the block); those of rg + 1 are issued
    // before the MFMAs of rg
    auto lookups = [&](int rg, uint32_t o[8]) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          o[4 * t + j] = *reinterpret_cast<const uint32_t *>(
              stab + ((((cw[rg][t] >> (8 * j)) & 0xFFu) << 6) | lane_off));
    };
    uint32_t lk[2][8];
    lookups(0, lk[0]);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      if (rg + 1 < 4) lookups(rg + 1, lk[(rg + 1) & 1]);
      const uint32_t *o = lk[rg & 1];
      const bf16x8 b0 = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
      const bf16x8 b1 = __builtin_bit_cast(bf16x8, make_uint4(o[4], o[5], o[6], o[7]));
      {
        f32x4 part[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          part[mt] = mfma16x16x32(cur.x[mt][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
          part[mt] = mfma16x16x32(cur.x[mt][1], b1, part[mt]);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[mt][rg][v] += ca[rg] * part[mt][v];
      }
    }
    // every wave is done with this ring slot
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  using T1 = std::true_type;
  using F0 = std::false_type;

  int st = 0;
#pragma unroll 1
  for (; st + 3 < nst; st += 2) {
    stage(T1{}, T1{}, st, o0, o1);
    stage(T1{}, T1{}, st + 1, o1, o0);
  }
  // 0 to 3 stages remain; the operands of stage st are in o0
  if (nst - st == 3) {
    stage(T1{}, T1{}, st, o0, o1);
    stage(T1{}, F0{}, st + 1, o1, o0);
    stage(F0{}, F0{}, st + 2, o0, o1);
  } else if (nst - st == 2) {
    stage(T1{}, F0{}, st, o0, o1);
    stage(F0{}, F0{}, st + 1, o1, o0);
  } else if (nst - st == 1) {
    stage(F0{}, F0{}, st, o0, o1);
  }

  // LoRA term on the matrix cores: wave w < 4 adds s * T[m][:] . B[n][:] for the 16 output
  // columns n = 16 w + (lane % 16) to its partial sums, in steps of 32 ranks (A operand: T row
  // m, B operand: B row n, both k-contiguous; ranks at or past r, rows past M or N read as zero).
  if (g.r > 0 && wave < 4) {
    const int r = g.r;
    const float sl = g.s;
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(g.T, g.M * r * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + n0 * r, rows * r * 2);
    const int nrow = wave * 16 + nl;
#pragma unroll 1
    for (int j0 = 0; j0 < r; j0 += 32) {
      uint32_t tb[MT][8], bb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int j = j0 + gl * 8 + e;
        const bool in = j < r;
        bb[e] = in ? __builtin_amdgcn_raw_buffer_load_b16(rB, (uint32_t)((nrow * r + j) * 2), 0, 0) : 0u;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          tb[mt][e] = in ? __builtin_amdgcn_raw_buffer_load_b16(
                               rT, (uint32_t)(((mt * 16 + nl) * r + j) * 2), 0, 0)
                         : 0u;
      }
      u32x4 bw;
#pragma unroll
      for (int q = 0; q < 4; ++q) bw[q] = (bb[2 * q] & 0xFFFFu) | (bb[2 * q + 1] << 16);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        u32x4 tw;
#pragma unroll
        for (int q = 0; q < 4; ++q) tw[q] = (tb[mt][2 * q] & 0xFFFFu) | (tb[mt][2 * q + 1] << 16);
        const f32x4 lp = mfma16x16x32(__builtin_bit_cast(bf16x8, tw), __builtin_bit_cast(bf16x8, bw),
                                      f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int rg = 0; rg < 4; ++rg)   // acc[mt][wave], without a dynamic register index
          if (rg == wave)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[mt][rg][v] += sl * lp[v];
      }
    }
  }

  // Sum the 8 waves' partial sums through LDS: waves 4..7 store theirs, waves 0..3 add them and
  // store the pair sums, then every thread adds the 4 pair sums of its outputs and stores Y.
  // acc[mt][rg] holds D[m][n] for m = mt*16 + 4 (lane / 16) + v, n = rg*16 + lane % 16.
  float *red = reinterpret_cast<float *>(smem);     // [4][MT*16 m][64 n]
  const int wq = wave & 3;
  if (wave >= 4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          red[(wq * MT * 16 + mt * 16 + 4 * gl + v) * 64 + rg * 16 + nl] = acc[mt][rg][v];
  }
  __syncthreads();
  if (wave < 4) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          float &cell = red[(wq * MT * 16 + mt * 16 + 4 * gl + v) * 64 + rg * 16 + nl];
          cell = acc[mt][rg][v] + cell;
        }
  }
  __syncthreads();
  for (int i = tid; i < MT * 16 * 64; i += kThreads) {
    const int m = i / 64, n = i % 64;
    float y = red[m * 64 + n] + red[(MT * 16 + m) * 64 + n] +
              red[(2 * MT * 16 + m) * 64 + n] + red[(3 * MT * 16 + m) * 64 + n];
    const int64_t gm = m, gn = n0 + n;
    if (gm < g.M && gn < N) g.Y[gm * N + gn] = (uint16_t)(pack_bf16x2(y, 0.f) & 0xFFFFu);
  }
}

template <int MT, int kFmt>
__global__ __launch_bounds__(kThreads) void decode_fwd_kernel(DecArgs g) {
  decode_body<MT, kFmt>(g);
}

}  // namespace

hipError_t launch_decode_fwd(const GemmArgs &ga, hipStream_t st) {
  DecArgs g;
  g.X = ga.a_side;
  g.T = ga.lora_a;
  g.B = ga.lora_b;
  g.w = ga.w;
  g.M = ga.M;
  g.r = ga.r;
  g.s = ga.s;
  g.Y = ga.out;
  g.t = ga.t;
  const unsigned grid = (unsigned)((ga.w.n + kRows - 1) / kRows);
  const int mt = (int)((ga.M + 15) / 16);
  if (ga.w.fp4) return hipErrorInvalidValue;   // E2M1 takes the stream kernel (decode16.hip)
#define DEC_CASE(T)                                                              \
  case T:                                                                        \
    if (ga.w.dq)                                                                 \
      decode_fwd_kernel<T, 1><<<dim3(grid), dim3(kThreads), 0, st>>>(g);         \
    else                                                                         \
      decode_fwd_kernel<T, 0><<<dim3(grid), dim3(kThreads), 0, st>>>(g);         \
    break;
  switch (mt) {
    DEC_CASE(1) DEC_CASE(2) DEC_CASE(3)
    default: return hipErrorInvalidValue;
  }
#undef DEC_CASE
  return hipGetLastError();
}

}  // namespace nf4q

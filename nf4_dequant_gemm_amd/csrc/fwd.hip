// Fused forward kernel of the QLoRA layer: Y = X deq(W)^T + s T B^T in one launch (gfx950).
//
// NF4 dequantisation, the base GEMM and the rank-r LoRA correction run in the same kernel and the
// same output tile; the weight is decoded on the fly and never written to HBM [Unsloth pages:
// "Inside Unsloth" listing, "What You'll Learn", "LoRA and QLoRA" (dequant, matmul and LoRA
// correction fused into a single launch); pyshine code tour, "Why You Need This" (LoRA delta computed
// inside the matmul instead of two extra matmuls); v0.1.463-beta release article, "About the
// Unsloth Project" (no redundant buffers during dequantisation)].
//
// Work split. One workgroup of 8 waves (2 x 4) owns a 256 x 256 tile of Y and walks K in steps of
// 64 = one NF4 block per weight row. Each wave accumulates 128 (m) x 64 (n) with MFMA 16x16x32
// (32 tiles), which keeps it within 256 registers so that two waves share each SIMD: the NF4
// decode of one wave (vector ALU) then runs while the other wave's MFMAs execute (a lone wave
// overlaps only a fraction of its own vector work with its MFMAs).
// Threads 2r and 2r+1 own weight row n0 + r of the tile, 32 elements each: per step they turn
// 16 bytes of codes and the block constant into bf16 values through a 16-entry table of
// bf16(level_i * a) held in registers (byte-select lookups, no LDS lookups, no per-element
// multiply).
//
// Pipeline per step s (one workgroup barrier per step):
//   * the X tile of step s+1 is requested by DMA straight into LDS buffer (s+1) & 1
//     (buffer_load ... lds: no registers, no LDS store instructions; its latency hides behind the
//     whole step), and the codes and block constant of step s+2 are loaded into registers,
//   * the 64 MFMAs of step s run on LDS buffer s & 1 in 16 groups (k-slice, m-tile) of 4, each
//     X fragment read two groups before its MFMAs and the second k-slice's weight fragments four
//     groups before theirs,
//   * between MFMA issues, the W half-rows of step s+1 (codes loaded one step earlier) are decoded
//     and written to LDS buffer (s+1) & 1.
// LDS rows hold 64 bf16 as 8 chunks of 16 bytes; chunk c of row r sits at slot c ^ x(r) with
// x(r) = ((r >> 1) ^ 2 (r & 1)) & 7. Measured on gfx950, a 16-byte LDS read serves 16 lanes per
// 256-byte bank window and a 16-byte write 8 lanes per 128 bytes: x keeps the 16 consecutive rows
// of a fragment read on distinct slots of the 256-byte window, and the 4 rows x 2 chunks of a
// decode write on distinct slots of the 128-byte window (the plain (r >> 1) & 7 left those writes
// 2-way conflicted).
//
// The same body serves three more forms (template parameters of fwd_body): the grouped launch of a
// mixture-of-experts layer [NVFP4 update article, "Comprehensive Improvements in Training
// Performance and Stability": grouped MoE with LoRA on the experts], the gate/up pair with its
// SwiGLU activation in the epilogue [pyshine Unsloth code tour, "Why You Need This": the fused
// gated-MLP activation], and the E2M1 weight format with FP8 group scales [NVFP4 update article,
// "NVFP4: A Quantization Format for the Next Generation of Hardware"].
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kT = 256;      // output tile rows and columns
constexpr int kS = 64;       // reduction step = NF4 block
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kChunks = kT * kS / 8;

__device__ __forceinline__ int rowx(int row) { return ((row >> 1) ^ ((row & 1) << 1)) & 7; }
__device__ __forceinline__ int swzf(int row, int c) { return row * 8 + (c ^ rowx(row)); }

// Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous range of tiles so
// the n-tiles of one m-block (which share X) run on one XCD and share its L2.
__device__ __forceinline__ int tile_remap(int hw, int tiles) {
  const int per = tiles >> 3, rem = tiles & 7, x = hw & 7;
  return x * per + (x < rem ? x : rem) + (hw >> 3);
}

struct CStage {
  u32x4 c;           // 16 bytes of codes (32 elements) of the thread's half-row
  uint32_t q, sc;    // block constant (int8 or float bits) and run scale bits
  uint16_t q16;      // E2M1: the two group scales (kept 16-bit: a widening of the just-loaded
                     // value would make the compiler wait for every load in flight)
};

// LoRA step staging: A side T columns jb..jb+63, B side s * B (rows n), zero-padded; only the
// first nch 8-column chunks are written (the MFMAs of the step read no further). Thread t stages
// chunk t % 8 of rows t / 8 + 64 i. When r is a multiple of 8 and T and B are 16-byte aligned,
// each chunk is one 16-byte buffer load (rows past the tile edge and chunks past r read as zero);
// otherwise values are read one at a time.
__device__ void stage_lora(const GemmArgs &g, float sb, int64_t m0, int64_t n0, int64_t rows_n,
                           int64_t n1, int64_t rows_n1, int64_t rows_m, int jb, int nch, uint4 *sA,
                           uint4 *sB) {
  // m0: first row of T; tile rows 0..127 take B rows n0.. (rows_n of them valid), tile rows
  // 128..255 B rows n1.. (rows_n1 valid; the plain tile has n1 = n0 + 128, rows_n1 = rows_n - 128);
  // rows past the valid ones are zero; B is staged times sb
  const int tid = threadIdx.x;
  const int c = tid & 7, row0 = tid >> 3;
  if (c >= nch) return;
  const int j0 = jb + c * 8;
  const bool vec = (g.r & 7) == 0 &&
                   ((reinterpret_cast<uintptr_t>(g.lora_a) | reinterpret_cast<uintptr_t>(g.lora_b)) & 15) == 0;
  if (vec) {
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.lora_a + m0 * g.r, rows_m * g.r * 2);
    const int64_t v0 = rows_n < 128 ? (rows_n > 0 ? rows_n : 0) : 128;
    const int64_t v1 = rows_n1 < 128 ? (rows_n1 > 0 ? rows_n1 : 0) : 128;
    const __amdgpu_buffer_rsrc_t rB0 = make_rsrc(g.lora_b + n0 * g.r, v0 * g.r * 2);
    const __amdgpu_buffer_rsrc_t rB1 = make_rsrc(g.lora_b + n1 * g.r, v1 * g.r * 2);
    u32x4 ta[kChunks / kThreads], tb[kChunks / kThreads];
#pragma unroll
    for (int i = 0; i < kChunks / kThreads; ++i) {
      const int row = row0 + 64 * i;
      const uint32_t off = j0 < g.r ? (uint32_t)(row * g.r + j0) * 2 : 0x80000000u;
      const uint32_t offb = j0 < g.r ? (uint32_t)((row & 127) * g.r + j0) * 2 : 0x80000000u;
      ta[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
      tb[i] = __builtin_amdgcn_raw_buffer_load_b128(i < 2 ? rB0 : rB1, offb, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kChunks / kThreads; ++i) {
      const int row = row0 + 64 * i;
      uint32_t wb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) wb[e] = pack_bf16x2(sb * bf16_lo(tb[i][e]), sb * bf16_hi(tb[i][e]));
      sA[swzf(row, c)] = make_uint4(ta[i][0], ta[i][1], ta[i][2], ta[i][3]);
      sB[swzf(row, c)] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    }
    return;
  }
#pragma unroll 1
  for (int i = 0; i < kChunks / kThreads; ++i) {
    const int row = row0 + 64 * i;
    uint32_t wa[4], wb[4];
    const int64_t m = m0 + row, n = row < 128 ? n0 + row : n1 + (row - 128);
    const bool nvalid = row < 128 ? row < rows_n : row - 128 < rows_n1;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ja = j0 + e, jc = ja + 1;
      uint32_t lo = 0, hi = 0;
      if (row < rows_m) {
        if (ja < g.r) lo = g.lora_a[m * g.r + ja];
        if (jc < g.r) hi = g.lora_a[m * g.r + jc];
      }
      wa[e >> 1] = lo | (hi << 16);
      float b0 = 0.f, b1 = 0.f;
      if (nvalid) {
        if (ja < g.r) b0 = bf16_to_f32(g.lora_b[n * g.r + ja]);
        if (jc < g.r) b1 = bf16_to_f32(g.lora_b[n * g.r + jc]);
      }
      wb[e >> 1] = pack_bf16x2(sb * b0, sb * b1);
    }
    sA[swzf(row, c)] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    sB[swzf(row, c)] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  }
}

// LoRA step staging of the gate/up pair. The A side is T as in stage_lora (columns jb .. of the
// 2 r' ranks [X Ag^T | X Au^T]); on the B side tile rows 0..127 take Bg row n0 + row at ranks
// 0 .. r' - 1 and rows 128..255 Bu row n0 + row - 128 at ranks r' .. 2 r' - 1, zero at the other
// half's ranks: the block-diagonal [[Bg, 0], [0, Bu]] without storing it (r' = g.r / 2).
__device__ void stage_lora_pair(const GemmArgs &g, float sb, int64_t m0, int64_t n0, int64_t rows_n,
                                int64_t rows_m, int jb, int nch, uint4 *sA, uint4 *sB) {
  const int tid = threadIdx.x;
  const int c = tid & 7, row0 = tid >> 3;
  if (c >= nch) return;
  const int j0 = jb + c * 8;
  const int rh = g.r / 2;
  const bool vec = (rh & 7) == 0 &&
                   ((reinterpret_cast<uintptr_t>(g.lora_a) | reinterpret_cast<uintptr_t>(g.lora_b) |
                     reinterpret_cast<uintptr_t>(g.lora_b2)) & 15) == 0;
  if (vec) {
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.lora_a + m0 * g.r, rows_m * g.r * 2);
    const int64_t v = rows_n < 128 ? (rows_n > 0 ? rows_n : 0) : 128;
    const __amdgpu_buffer_rsrc_t rBg = make_rsrc(g.lora_b + n0 * rh, v * rh * 2);
    const __amdgpu_buffer_rsrc_t rBu = make_rsrc(g.lora_b2 + n0 * rh, v * rh * 2);
    u32x4 ta[kChunks / kThreads], tb[kChunks / kThreads];
#pragma unroll
    for (int i = 0; i < kChunks / kThreads; ++i) {
      const int row = row0 + 64 * i;
      const int jj = i < 2 ? j0 : j0 - rh;   // rank within the row's own half (rows 128.. are up)
      const uint32_t off = j0 < g.r ? (uint32_t)(row * g.r + j0) * 2 : 0x80000000u;
      const uint32_t offb = jj >= 0 && jj < rh ? (uint32_t)((row & 127) * rh + jj) * 2 : 0x80000000u;
      ta[i] = __builtin_amdgcn_raw_buffer_load_b128(rA, off, 0, 0);
      tb[i] = __builtin_amdgcn_raw_buffer_load_b128(i < 2 ? rBg : rBu, offb, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kChunks / kThreads; ++i) {
      const int row = row0 + 64 * i;
      uint32_t wb[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) wb[e] = pack_bf16x2(sb * bf16_lo(tb[i][e]), sb * bf16_hi(tb[i][e]));
      sA[swzf(row, c)] = make_uint4(ta[i][0], ta[i][1], ta[i][2], ta[i][3]);
      sB[swzf(row, c)] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
    }
    return;
  }
#pragma unroll 1
  for (int i = 0; i < kChunks / kThreads; ++i) {
    const int row = row0 + 64 * i;
    const bool up = row >= 128;
    const uint16_t *Bh = up ? g.lora_b2 : g.lora_b;
    const int64_t m = m0 + row, n = n0 + (row & 127);
    const bool nvalid = (row & 127) < rows_n;
    uint32_t wa[4], wb[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ja = j0 + e, jc = ja + 1;
      uint32_t lo = 0, hi = 0;
      if (row < rows_m) {
        if (ja < g.r) lo = g.lora_a[m * g.r + ja];
        if (jc < g.r) hi = g.lora_a[m * g.r + jc];
      }
      wa[e >> 1] = lo | (hi << 16);
      const int ka = up ? ja - rh : ja, kc = ka + 1;
      float b0 = 0.f, b1 = 0.f;
      if (nvalid) {
        if (ka >= 0 && ka < rh) b0 = bf16_to_f32(Bh[n * rh + ka]);
        if (kc >= 0 && kc < rh) b1 = bf16_to_f32(Bh[n * rh + kc]);
      }
      wb[e >> 1] = pack_bf16x2(sb * b0, sb * b1);
    }
    sA[swzf(row, c)] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    sB[swzf(row, c)] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  }
}

// The kernel body, shared by the plain launch and the grouped (mixture-of-experts) launch. With
// kGrp, the tiles of every expert follow one another: the workgroup finds its expert e from the
// first-tile table, takes rows m_off[e] .. m_off[e+1] of X, T and Y, and rows e N .. of the stacked
// weight and of the stacked B (N = g.C); everything else is the plain kernel.
// kFmt: 0 NF4 with float32 block constants, 1 NF4 with double-quantised constants, 2 E2M1 with
// E4M3 group scales (groups of 16: the two groups of a thread's 32 elements get a table each) and
// a float32 tensor scale S. E2M1 values times group scales are exact in bf16, so the weight
// operand is decoded without rounding and S multiplies the accumulators in the epilogue; the
// LoRA steps stage B times s / S to share the accumulators.
// kPair: the gate/up pair with its SwiGLU epilogue. The weight is the stacked [Wg; Wu] [2N, K]
// (N = g.C), the up projection the block-diagonal [[Bg, 0], [0, Bu]] (stage_lora_pair); a tile's
// 256 columns are gate columns n0 .. n0 + 127 (weight rows n0 .., Bg rows n0 ..) and the up
// columns of the same indices (weight rows N + n0 .., Bu rows n0 ..),
// so the epilogue holds Yg and Yu of the same columns: it writes both to g.out ([M, 2N], gate then
// up) and H = silu(Yg) * Yu, from their float32 sums, to g.hout ([M, N], row stride g.ldh).
template <int kFmt, bool kGrp, bool kPair = false>
__device__ __forceinline__ void fwd_body(const GemmArgs &g, const GroupArgs &gr) {
  constexpr bool kDQ = kFmt == 1, kFP4 = kFmt == 2;
  constexpr int kTN = kPair ? kT / 2 : kT;   // columns of each output a tile advances by
  // X and W tiles as separate arrays: the compiler then knows that LDS accesses to one do not
  // alias the DMA in flight into another (one array of two would make it wait for the DMA)
  __shared__ uint4 sX0[kChunks], sX1[kChunks];
  __shared__ uint4 sW0[kChunks], sW1[kChunks];
  auto xbuf = [&](int P) { return P ? sX1 : sX0; };
  auto wbuf = [&](int P) { return P ? sW1 : sW0; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int tiles_n = (int)((g.C + kTN - 1) / kTN);
  int local;
  int64_t m_lo = 0, m_hi = g.M, wbase = 0;
  if (kGrp) {
    // a grid sized by an upper bound (routing on the device) has workgroups past the last tile
    const int total = grp_tile_off(gr, gr.E);
    if ((int)blockIdx.x >= total) return;
    local = tile_remap(blockIdx.x, total);
    const int e = find_group(gr, local);
    local -= grp_tile_off(gr, e);
    m_lo = grp_m_off(gr, e);
    m_hi = grp_m_off(gr, e + 1);
    wbase = (int64_t)e * g.C;
  } else {
    local = tile_remap(blockIdx.x, gridDim.x);
  }
  const int64_t m0 = m_lo + (int64_t)(local / tiles_n) * kT;
  const int64_t n0 = (int64_t)(local % tiles_n) * kTN;   // columns of Y
  const int64_t wn0 = wbase + n0;                         // rows of the (stacked) weight and B
  const int64_t K = g.w.k;
  const int64_t rows_m = (m_hi - m0 < kT) ? m_hi - m0 : kT;
  const int64_t rows_n = (g.C - n0 < kTN) ? g.C - n0 : kTN;   // valid columns (of each half)
  const int kblk = (int)(K / kS);
  const int last = kblk - 1;
  // The tiles of one row block start their walk over K at step rot (and wrap around), tiles of
  // different row blocks at different steps, so that the workgroups of a launch do not all
  // request the same K offsets at once. rot depends on the row block only: every output element
  // still sums its K steps in an order fixed by its row (the pair and grouped forms agree).
  const int rot = (int)(((m0 - m_lo) / kT) * 5 % kblk);
  auto phys = [&](int s) { return s + rot < kblk ? s + rot : s + rot - kblk; };

  const __amdgpu_buffer_rsrc_t rX = make_rsrc(g.a_side + m0 * K, rows_m * K * 2);
  // pair: the buffers span the whole stacked weight, rows addressed per thread (rows past N read
  // as zero through out-of-range offsets)
  const int64_t wrows = kPair ? 2 * g.C : rows_n;
  const int64_t wfirst = kPair ? 0 : wn0;
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.w.codes + wfirst * (K / 2), wrows * (K / 2));
  const __amdgpu_buffer_rsrc_t rQ =
      kFP4  ? make_rsrc(reinterpret_cast<const uint8_t *>(g.w.absmax) + wfirst * (K / 16), wrows * (K / 16))
      : kDQ ? make_rsrc(reinterpret_cast<const int8_t *>(g.w.absmax) + wfirst * kblk, wrows * kblk)
            : make_rsrc(reinterpret_cast<const float *>(g.w.absmax) + wfirst * kblk, wrows * kblk * 4);
  const int64_t nruns = (g.w.n * kblk + 255) / 256;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.w.scale, kDQ ? nruns * 4 : 0);
  // E2M1: the tensor scale (1 for an all-zero weight, whose group scales are all 0), read where
  // it is used so that no register holds it through the main loop
  auto tscale = [&]() {
    const float S = *g.w.scale;
    return S > 0.f ? S : 1.f;
  };

  // X DMA: instruction i of wave w fills the 1 KB of the tile holding rows 8 (4 w + i) .. +7;
  // lane L writes physical chunk L % 8 of row 8 (4 w + i) + L / 8, i.e. logical chunk
  // (L % 8) ^ rowx(row) (the same swizzle as swzf).
  uint32_t xoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ rowx(row);
    xoff[i] = (uint32_t)(row * K * 2 + c * 16);
  }
  // Decode ownership: weight row wr of the tile, elements 32 wh .. 32 wh + 31 of each step.
  const int wr = tid >> 1, wh = tid & 1;
  // In the pipelined steps the two threads of a row split its table: thread wh builds entries
  // 8 wh .. 8 wh + 7 (levels lvh) and takes the other half from the partner lane; the select masks
  // of the decode are complemented for wh = 1, whose own half is the upper one.
  float lvh[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) lvh[i] = wh ? g.t.level[8 + i] : g.t.level[i];
  const uint32_t mhi = (wh && !kFP4) ? 0u : 0xFFFFFFFFu, mlo = (wh && !kFP4) ? 0xFFFFFFFFu : 0u;
  // weight row of tile row wr (pair: gate rows n0 + wr, up rows N + n0 + wr - 128), and whether
  // it holds data (a pair tile past N reads zeros)
  const int64_t wrow = kPair ? (wr < 128 ? n0 + wr : g.C + n0 + (wr - 128)) : wr;
  const bool wvalid = !kPair || n0 + (wr & 127) < g.C;
  const uint32_t coff = wvalid ? (uint32_t)(wrow * (K / 2) + wh * 16) : 0x80000000u;
  // E2M1: the two group scales of the thread's 32 elements (bytes 4 s + 2 wh, + 1 of its row)
  // (out of range: 0x80000000 bytes, or that many after the float32 constants' scaling by 4)
  const uint32_t qoff = !wvalid ? ((kFP4 || kDQ) ? 0x80000000u : 0x20000000u)
                        : kFP4  ? (uint32_t)(wrow * (K / 16) + 2 * wh)
                                : (uint32_t)(wrow * kblk);
  const int64_t sbase = (kPair ? wrow : wn0 + wr) * kblk;

  const int g16 = lane >> 4, l16 = lane & 15;
  f32x4 acc[4][8];   // [n-tile][m-tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto dma_x = [&](int s, uint4 *sA) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rX, (__attribute__((address_space(3))) void *)(sA + (4 * wave + i) * 64), 16, xoff[i],
          s * 128, 0, 0);
  };
  constexpr int kCodeLoads = kDQ ? 3 : 2;   // loads issued by load_c
  auto load_c = [&](int s, CStage &c) {
    c.c = __builtin_amdgcn_raw_buffer_load_b128(rC, coff + s * 32, 0, 0);
    if (kFP4) {
      c.q16 = __builtin_amdgcn_raw_buffer_load_b16(rQ, qoff + 4 * s, 0, 0);
    } else if (kDQ) {
      c.q = __builtin_amdgcn_raw_buffer_load_b8(rQ, qoff + s, 0, 0);
      c.sc = __builtin_amdgcn_raw_buffer_load_b32(rS, (uint32_t)(((sbase + s) >> 8) * 4), 0, 0);
    } else {
      c.q = __builtin_amdgcn_raw_buffer_load_b32(rQ, (qoff + s) * 4, 0, 0);
    }
  };
  auto absmax_of = [&](const CStage &c) {
    return kDQ ? int8_code(c.q) * __uint_as_float(c.sc) : __uint_as_float(c.q);
  };
  auto word = [](const CStage &c, int j) {
    return j == 0 ? c.c.x : j == 1 ? c.c.y : j == 2 ? c.c.z : c.c.w;
  };
  auto decode_half = [&](const CStage &c, uint4 *sB) {
    RowTable t = kFP4 ? make_e2m1_table(e4m3_to_f32(c.q16 & 0xFFu)) : make_row_table(absmax_of(c), g.t);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o[4];
      if (kFP4 && j == 2) t = make_e2m1_table(e4m3_to_f32((c.q16 >> 8) & 0xFFu));
      if (kFP4) decode8_e2m1(t, word(c, j), o); else decode8(t, word(c, j), o);
      sB[swzf(wr, 4 * wh + j)] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  };
  // MFMA operands of k-slice ks (32 columns k): lane (g16, l16) takes 8 consecutive k
  // (32 ks + 8 g16 ..) of weight row wn*64 + 16 nt + l16 or of X row wm*128 + 16 mt + l16.
  auto wfrag = [&](const uint4 *sB, int ks, int nt) {
    return __builtin_bit_cast(bf16x8, sB[swzf(wn * 64 + nt * 16 + l16, ks * 4 + g16)]);
  };
  auto xfrag = [&](const uint4 *sA, int ks, int mt) {
    return __builtin_bit_cast(bf16x8, sA[swzf(wm * 128 + mt * 16 + l16, ks * 4 + g16)]);
  };
  // Plain MFMA pass over k-slice ks of one step (used for the LoRA steps).
  auto mma = [&](const uint4 *sA, const uint4 *sB, int ks) {
    bf16x8 aw[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aw[nt] = wfrag(sB, ks, nt);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bf16x8 b = xfrag(sA, ks, mt);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt][mt] = mfma16x16x32(aw[nt], b, acc[nt][mt]);
    }
  };

  // One step: MFMAs on buffer P; the X tile of step s+1 arrives in buffer P^1 by DMA and the W
  // half-rows of step s+1 (decoded from cn) are written there in between; codes of step s+2 go to
  // cm. 16 groups (k-slice, m-tile) of 4 MFMAs; decode pieces go between groups.
  auto body = [&](int s, int P, CStage &cm, CStage &cn) {
    const int s1 = s + 1 < last ? s + 1 : last;
    const int s2 = s + 2 < last ? s + 2 : last;
    dma_x(phys(s1), xbuf(P ^ 1));
    __builtin_amdgcn_sched_barrier(0);   // the DMA stays ahead of the code loads (see the wait)
    load_c(phys(s2), cm);
    const uint4 *A = xbuf(P);
    const uint4 *B = wbuf(P);
    uint4 *Bn = wbuf(P ^ 1);
    // LDS operands: the first k-slice's weight fragments and the first two X fragments now; the
    // NF4 table of step s+1 is built while they arrive; later X fragments are read two groups
    // ahead and the second k-slice's weight fragments four groups ahead, so an MFMA rarely waits
    // for an LDS read.
    bf16x8 aw0[4], aw1[4], xb[3];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) aw0[nt] = wfrag(B, 0, nt);
    xb[0] = xfrag(A, 0, 0);
    xb[1] = xfrag(A, 0, 1);

    // this thread's half of the table in L[0..1], H[0..1]; the partner lane's half by DPP
    // (E2M1: the whole table of the thread's first group)
    RowTable t;
    if (kFP4) {
      t = make_e2m1_table(e4m3_to_f32(cn.q16 & 0xFFu));
    } else {
      const float a = absmax_of(cn);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const uint32_t p0 = pack_bf16x2(lvh[4 * q] * a, lvh[4 * q + 1] * a);
        const uint32_t p1 = pack_bf16x2(lvh[4 * q + 2] * a, lvh[4 * q + 3] * a);
        t.L[q] = perm(p1, p0, 0x06040200u);
        t.H[q] = perm(p1, p0, 0x07050301u);
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        t.L[2 + q] = swap_adjacent_lanes(t.L[q]);
        t.H[2 + q] = swap_adjacent_lanes(t.H[q]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
    Dec8 dx;
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) {
      const int mt = grp & 7, ks = grp >> 3;
      if (grp == 4) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) aw1[nt] = wfrag(B, 1, nt);
      }
      if (grp + 2 < 16) xb[(grp + 2) % 3] = xfrag(A, (grp + 2) >> 3, (grp + 2) & 7);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        acc[nt][mt] = mfma16x16x32(ks ? aw1[nt] : aw0[nt], xb[grp % 3], acc[nt][mt]);
      // decode of step s+1: word j = grp / 3 in pieces over three groups (pieces 0-1, 2-3,
      // 4 + store), groups 0..11
      if (grp < 12) {
        const int j = grp / 3, ph = grp % 3;
        uint32_t o[4];
        if (ph == 0) {
          dx.d = word(cn, j);
          kFP4 ? dec_piece_e2m1(t, dx, 0, o) : dec_piece(t, dx, 0, o, mhi, mlo);
          kFP4 ? dec_piece_e2m1(t, dx, 1, o) : dec_piece(t, dx, 1, o, mhi, mlo);
        } else if (ph == 1) {
          kFP4 ? dec_piece_e2m1(t, dx, 2, o) : dec_piece(t, dx, 2, o, mhi, mlo);
          kFP4 ? dec_piece_e2m1(t, dx, 3, o) : dec_piece(t, dx, 3, o, mhi, mlo);
        } else {
          kFP4 ? dec_piece_e2m1(t, dx, 4, o) : dec_piece(t, dx, 4, o, mhi, mlo);
          Bn[swzf(wr, 4 * wh + j)] = make_uint4(o[0], o[1], o[2], o[3]);
          // E2M1: words 2 and 3 belong to the thread's second group. The empty asm keeps this
          // table from being hoisted above the groups before (two live tables spill registers).
          if (kFP4 && j == 1) {
            uint16_t q2 = cn.q16;
            asm volatile("" : "+v"(q2));
            t = make_e2m1_table(e4m3_to_f32((q2 >> 8) & 0xFFu));
          }
        }
      }
      // keep each group's loads and decode work in place (hoisting them stretches register
      // lifetimes past the 256 a wave may use with two waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
    // This wave's LDS writes are done and the X DMA of step s+1 (older than the code loads of
    // step s+2, which stay in flight) has landed; the barrier publishes buffer P^1.
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCodeLoads) : "memory");
  };

  CStage c0, c1;
  dma_x(phys(0), xbuf(0));
  load_c(phys(0), c0);
  load_c(phys(kblk > 1 ? 1 : 0), c1);
  decode_half(c0, wbuf(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int s = 0;
#pragma unroll 1
  for (; s + 2 <= kblk; s += 2) {
    body(s, 0, c0, c1);
    body(s + 1, 1, c1, c0);
  }
  if (s < kblk) body(s, 0, c0, c1);
  __syncthreads();

  // LoRA steps: [T | s B] as extra reduction steps of the same tile; a k-slice of 32 columns
  // that lies wholly past r is skipped. The pair: when r' = r / 2 is a multiple of 32, every
  // k-slice holds ranks of one half only (gate: below r'), and the waves of the other half
  // (waves wn < 2 hold gate columns) skip it: their B there is zero.
  const int nlora = (g.r + kS - 1) / kS;
  auto pair_skips = [&](int j, int ks) {
    return kPair && (g.r / 2) % 32 == 0 && ((j * kS + 32 * ks < g.r / 2) != (wn < 2));
  };
#pragma unroll 1
  for (int j = 0; j < nlora; ++j) {
    const int buf = j & 1;
    const int nks = g.r - j * kS > kS / 2 ? 2 : 1;
    if (kPair)
      stage_lora_pair(g, kFP4 ? g.s / tscale() : g.s, m0, n0, rows_n, rows_m, j * kS, 4 * nks,
                      xbuf(buf), wbuf(buf));
    else
      stage_lora(g, kFP4 ? g.s / tscale() : g.s, m0, wn0, rows_n, wn0 + 128, rows_n - 128, rows_m,
                 j * kS, 4 * nks, xbuf(buf), wbuf(buf));
    __syncthreads();
    if (!pair_skips(j, 0)) mma(xbuf(buf), wbuf(buf), 0);
    if (nks > 1 && !pair_skips(j, 1)) mma(xbuf(buf), wbuf(buf), 1);
    __syncthreads();
  }

  // Epilogue. With the weight tile as the MFMA A operand, a lane holds columns n..n+3 of row m.
  // Each wave packs its 128 x 64 block to bf16 in 16 KB of the (now idle) LDS and writes it out as
  // whole 128-byte row pieces, 16 bytes per lane, with non-temporal stores (Y is not read again by
  // this kernel, and streaming it out measured faster than write-back cached stores). Rows of Y
  // are 16-byte aligned and the column count is a multiple of 8 (checked at launch), so a 16-byte
  // piece lies wholly inside or wholly past the last column.
  // E2M1: the sums are in units of the tensor scale S
  if (kFP4) {
    const float tsc = tscale();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) acc[nt][mt] *= tsc;
  }
  uint4 *blk = (wave >> 1) == 0 ? sX0 : (wave >> 1) == 1 ? sX1 : (wave >> 1) == 2 ? sW0 : sW1;
  blk += (wave & 1) * (kChunks / 2);
  uint2 *b2 = reinterpret_cast<uint2 *>(blk);
  const int c = lane & 7;
  // output column of this wave's piece c (pair: gate or up half of [M, 2N])
  const int64_t ncol = kPair ? n0 + (wn & 1) * 64 + c * 8 : n0 + wn * 64 + c * 8;
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
      b2[swzf(mt * 16 + l16, 2 * nt + (g16 >> 1)) * 2 + (g16 & 1)] =
          make_uint2(pack_bf16x2(acc[nt][mt][0], acc[nt][mt][1]),
                     pack_bf16x2(acc[nt][mt][2], acc[nt][mt][3]));
  __syncthreads();
  {
    const int64_t n = kPair ? (wn < 2 ? ncol : g.C + ncol) : ncol;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int64_t m = m0 + wm * 128 + row;
      const uint4 v = blk[swzf(row, c)];
      if (wm * 128 + row < rows_m && ncol < g.C)
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4 *>(g.out + m * g.ldo + n));
    }
  }
  if (kPair) {
    // H = silu(Yg) * Yu from the float32 sums. Wave (wm, wn) with wn < 2 holds Yg of tile
    // columns 64 wn ..; wave (wm, wn + 2) holds Yu of the same columns in the same register
    // positions. The up waves park their float32 accumulators in LDS (32 KB each: the four fill
    // the 128 KB), the gate waves read them at their own positions and turn their accumulators
    // into H, which they then stage and write like Y.
    __syncthreads();
    f32x4 *park = reinterpret_cast<f32x4 *>(wm == 0 ? (wn & 1 ? sX1 : sX0) : (wn & 1 ? sW1 : sW0));
    if (wn >= 2) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) park[(nt * 8 + mt) * 64 + lane] = acc[nt][mt];
    }
    __syncthreads();
    if (wn < 2) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const f32x4 u = park[(nt * 8 + mt) * 64 + lane];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float gv = acc[nt][mt][e], uv = u[e];
            // the activation kernel's expression, in float32 on the unrounded sums
            acc[nt][mt][e] = gv * (1.f / (1.f + __expf(-gv))) * uv;
          }
        }
    }
    __syncthreads();
    if (wn < 2) {
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
          b2[swzf(mt * 16 + l16, 2 * nt + (g16 >> 1)) * 2 + (g16 & 1)] =
              make_uint2(pack_bf16x2(acc[nt][mt][0], acc[nt][mt][1]),
                         pack_bf16x2(acc[nt][mt][2], acc[nt][mt][3]));
    }
    __syncthreads();
    if (wn < 2) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int row = 8 * i + (lane >> 3);
        const int64_t m = m0 + wm * 128 + row;
        const uint4 v = blk[swzf(row, c)];
        if (wm * 128 + row < rows_m && ncol < g.C)
          __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                      reinterpret_cast<u32x4 *>(g.hout + m * g.ldh + ncol));
      }
    }
  }
}

template <int kFmt>
__global__ __launch_bounds__(kThreads) void fwd_fused_kernel(GemmArgs g) {
  fwd_body<kFmt, false>(g, GroupArgs{});
}

template <int kFmt>
__global__ __launch_bounds__(kThreads) void fwd_grouped_kernel(GemmArgs g, GroupArgs gr) {
  fwd_body<kFmt, true>(g, gr);
}

template <int kFmt>
__global__ __launch_bounds__(kThreads) void fwd_pair_kernel(GemmArgs g) {
  fwd_body<kFmt, false, true>(g, GroupArgs{});
}

}  // namespace

hipError_t launch_gemm_fwd(const GemmArgs &g, hipStream_t st) {
  if (((g.C | g.ldo) & 7) != 0 || (reinterpret_cast<uintptr_t>(g.out) & 15) != 0)
    return hipErrorInvalidValue;   // the epilogue writes 16-byte pieces of 8 columns
  const int64_t tiles = ((g.C + kT - 1) / kT) * ((g.M + kT - 1) / kT);
  if (g.w.fp4)
    fwd_fused_kernel<2><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else if (g.w.dq)
    fwd_fused_kernel<1><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else
    fwd_fused_kernel<0><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd_grouped(const GemmArgs &g, const GroupArgs &gr, hipStream_t st) {
  if (((g.C | g.ldo) & 7) != 0 || (reinterpret_cast<uintptr_t>(g.out) & 15) != 0 || gr.E < 1 ||
      gr.E > kMaxExperts)
    return hipErrorInvalidValue;
  const int64_t tiles = gr.grid;
  if (tiles < 1) return hipSuccess;
  if (g.w.fp4)
    fwd_grouped_kernel<2><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g, gr);
  else if (g.w.dq)
    fwd_grouped_kernel<1><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g, gr);
  else
    fwd_grouped_kernel<0><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g, gr);
  return hipGetLastError();
}

hipError_t launch_gemm_fwd_pair(const GemmArgs &g, hipStream_t st) {
  if (((g.C | g.ldo | g.ldh) & 7) != 0 || g.ldo < 2 * g.C || g.ldh < g.C || g.w.n != 2 * g.C ||
      ((reinterpret_cast<uintptr_t>(g.out) | reinterpret_cast<uintptr_t>(g.hout)) & 15) != 0 ||
      (g.r > 0 && ((g.r & 1) != 0 || !g.lora_a || !g.lora_b || !g.lora_b2)))
    return hipErrorInvalidValue;
  const int64_t tiles = ((g.C + kT / 2 - 1) / (kT / 2)) * ((g.M + kT - 1) / kT);
  if (g.w.fp4)
    fwd_pair_kernel<2><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else if (g.w.dq)
    fwd_pair_kernel<1><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else
    fwd_pair_kernel<0><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace nf4q

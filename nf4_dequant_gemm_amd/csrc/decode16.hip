// Decode-shaped forward for at most 16 rows of X and double-quantised block constants:
// dequantise-on-the-fly GEMV of the NF4 weight with the LoRA correction, Y = X deq(W)^T + s T B^T
// [pyshine Unsloth code tour, "Why You Need This": dequantize-on-the-fly GEMV for NF4 weights;
// "Inside Unsloth" listing, "What You'll Learn", "LoRA and QLoRA": dequant, matmul and LoRA
// correction in one launch; NVFP4 update article, "NVFP4: A Quantization Format for the Next
// Generation of Hardware": a separate dequantisation step eats into the bandwidth that 4-bit
// storage saves].
//
// The work is the 0.52 bytes per weight element streamed from HBM, and on this GPU the rate of a
// stream is set by how many bytes each memory request carries: a 16-row MFMA operand loaded
// straight from the row-major codes touches 16 cache lines for 512 bytes. So every byte the
// kernel reads from memory (codes, X and block constants) goes to LDS by DMA in whole 128-byte
// lines and is read from there in the matrix-core layout:
//   * one workgroup per CU takes 112 weight rows (7 MFMA column tiles; 256 workgroups for the
//     28672-row projections) and walks K in stages of one 4-block group (128 bytes of each row);
//   * a stage is 14 KB of codes, the 8 KB X slice (shared by all 7 tiles) and the int8 block codes
//     and run scales of the double quantisation, all by `buffer_load ... lds`; four stage slots,
//     three stages in flight, one barrier per stage;
//   * a code byte (two elements) becomes a pair of bf16 NF4 levels through a 256-entry table in
//     LDS replicated 64 times: entry e of copy c sits at byte 256 e + 4 c, so the lookup address
//     of byte j of a code word is one v_perm_b32 (code byte into bits 15..8, the lane's copy
//     offset into bits 7..0) and every lane reads its own bank;
//   * MFMA 16x16x32 multiplies the unscaled levels by X; the block constant a (per weight row and
//     64-element block) scales the fp32 block partial sum afterwards:
//         Y[m][n] += a(n, b) * sum_{k in block b} X[m][k] * level(code[n][k]);
//   * wave (g, j) takes block j of every stage for tiles 4g .. 4g + 3 (3 tiles for g = 1), so each
//     X fragment is read from LDS once per block and serves every tile of the wave; the four
//     partial sums of a tile meet in LDS at the end;
//   * one group of four waves issues every copy, the other none, which leaves its vector-memory
//     counter to loads the compiler tracks. With the adapter A given (NF4) the copies go to the
//     3-tile waves (g = 1) and the 4-tile waves form T = X A^T themselves: wave (0, j) multiplies
//     the X fragments of block j it already holds by A's matching 16-byte pieces, loaded straight
//     into registers two stages ahead (2 MFMAs per rank tile of 16 and stage), and the four block
//     sums of T meet in LDS at the end, so the decode forward needs no separate launch for T.
//     Without it (T given or as split partials) the NF4 form gives the copies to the 4-tile waves
//     (measured faster: 28.6-28.9 against 30.3 us on the 28672 x 8192 weight); The E2M1 form's 4-tile waves are
//     at the register limit (the same work cost it 8 us of a 34 us launch); it has LDS to spare,
//     so there (r <= 16) the copying waves also copy A's slice of each stage next to X's, in the
//     same layout, and form T from LDS with the X fragments they hold.
// LDS layouts are XOR-swizzled so the matrix-core reads hit distinct banks; the swizzle is applied
// on the DMA source side (the DMA writes 1 KB contiguously).
// Numerics: the NF4 level (not level * a) is rounded to bf16 before the product, as in the other
// decode-shaped kernel; within the layer's tolerance of the definition.
// Requires M <= 16, double quantisation, K % 256 == 0; the host sends other shapes elsewhere.
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kTiles = 7;
constexpr int kRows = 16 * kTiles;           // weight rows per workgroup
constexpr int kWaves = 8;                    // wave (g, j): tiles 4g .. 4g+3 (< 7), block j of a stage
constexpr int kThreads = kWaves * 64;
constexpr int kCodeBytes = kRows * 128;      // a stage: 4 blocks x 32 bytes of each row
constexpr int kXOff = kCodeBytes;            // X slice: 16 rows x 256 elements
constexpr int kSOff = kXOff + 16 * 512;      // run scale of each row's group: 128 rows x 4
constexpr int kSlotBytes = kSOff + 512;
constexpr int kQWinBytes = 128 * 16;         // int8 block codes of 4 stages: 128 rows x 16
constexpr int kTabBytes = 256 * 64 * 4;      // 64 KB
// Copies (buffer_load ... lds) each of the kDmaWaves copying waves (4..7) issues per stage, and the
// extra one waves 4 and 5 issue in the stages that also fetch a window of block codes. dma() below
// issues exactly these, and the stage waits are derived from them: a stage waits until only the
// copies of the two stages after it are in flight.
constexpr int kDmaWaves = 4;
constexpr int kStageCopies = 6;
constexpr int kWindowCopies = 1;
// and, in the E2M1 form that forms T, the pieces of A's slice for the stage
constexpr int kACopies = 2;

struct Dec16Args {
  const uint16_t *X;
  const uint16_t *T;
  const uint16_t *B;
  WDesc w;
  int64_t M;
  int r;
  float s;
  uint16_t *Y;
  Tables t;
  const float *tpart;   // T = X A^T as split partials [M][r][tsplits] (NULL: T is given)
  int tsplits;
  uint16_t *tout;       // with tpart or A: T (bf16 [M][r]) written by workgroup 0
  const uint16_t *A;    // adapter A [r][K] when the kernel forms T itself (kQ > 0)
};

// Roles of the two wave groups in the stage loop (see the header comment).
struct CopyRole {
  static constexpr bool copies = true;
};
struct TRole {
  static constexpr bool copies = false;
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource words for the DMA below (same layout as make_rsrc: raw buffer, no stride,
// loads at or past `bytes` return 0).
__device__ __forceinline__ i32x4 rsrc_words(const void *p, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)((a >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

template <typename T>
__device__ __forceinline__ uint32_t lds_addr(T *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) T *)p;
}

// LDS read at a byte address.
template <typename T>
__device__ __forceinline__ T lds_ld(uint32_t a) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T *>((uintptr_t)a);
}

// A slot's LDS base address as a value the compiler cannot fold: the slots lie above the 64 KB
// reach of the LDS instruction offset, so each read needs base + lane offset in a register; kept
// opaque, that add happens at the read instead of as one hoisted register per slot and offset.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+s"(v));
  return v;
}

// HBM -> LDS copies (buffer_load ... lds): 64 lanes x 16 (or 4) bytes from per-lane offsets into
// 1 KB (256 bytes) of LDS at `lds`, in lane order. Written as inline assembly so that the compiler
// does not track them: it cannot tell the stage slots apart across loop iterations and would wait
// for every copy in flight before each LDS read. The stage loop waits for them itself (vmcnt).
__device__ __forceinline__ void dma16(const i32x4 &rs, uint32_t lds, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               ::"s"(lds), "v"(voff), "s"(rs), "s"(soff) : "memory");
}
__device__ __forceinline__ void dma4(const i32x4 &rs, uint32_t lds, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               ::"s"(lds), "v"(voff), "s"(rs) : "memory");
}

template <int N>
struct TileCount {
  static constexpr int n = N;
};

// Two E2M1 values (byte kByte of w) as a bf16 pair, low nibble -> low half. The conversion's
// scale operand contributes only its power of two (measured on gfx950: the mantissa of the
// scale is ignored), so it is 1 here and the E4M3 group scales are applied to the sums.
template <int kByte>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, kByte));
}

// kFP4: E2M1 codes with an E4M3 scale per group of 16 and a float32 tensor scale S (block 16 of
// the weight descriptor). A stage then carries the 16 group-scale bytes of each row (4 blocks x 4
// groups) in place of the run scales, and needs no windows of block codes and no level table
// (the codes convert to bf16 in one instruction per byte). Each lane takes 8 consecutive
// elements of a 32-element slice, so a slice holds two groups split by lane half; each group's
// product is its own MFMA (the X operand masked to that half), times its scale, and the sums are
// in units of S, which multiplies the tile at the end.
// kQ: rank tiles of 16 of T = X A^T formed in the kernel (0: T given, or added from split
// partials; E2M1 at most 1).
template <bool kFP4, int kQ>
__global__ __launch_bounds__(kThreads) void decode16_fwd_kernel(Dec16Args g) {
  static_assert(!kFP4 || kQ <= 1, "the E2M1 form forms T for r <= 16 only");
  // E2M1 forming T: A's slice (16 ranks x 256 elements, laid out as X's) follows the group scales
  // in each slot, copied by the copying waves, which form T
  constexpr bool kTlds = kFP4 && kQ > 0;
  constexpr int kAOff = kSOff + kRows * 16;
  constexpr int kCopies = kStageCopies + (kTlds ? kACopies : 0);   // per copying wave and stage
  constexpr int kPending = 2 * kCopies;
  // Four stage slots, two windows of block codes and the level-pair table, which holds the
  // cross-wave sums at the end (and after them the block sums of T).
  constexpr int kSlot = kFP4 ? kAOff + (kTlds ? 16 * 512 : 0) : kSlotBytes;
  constexpr int kQWin = kFP4 ? 16 : kQWinBytes;
  __shared__ __align__(16) uint8_t slot0[kSlot];
  __shared__ __align__(16) uint8_t slot1[kSlot];
  __shared__ __align__(16) uint8_t slot2[kSlot];
  __shared__ __align__(16) uint8_t slot3[kSlot];
  __shared__ __align__(16) uint8_t qwin0[kQWin];
  __shared__ __align__(16) uint8_t qwin1[kQWin];
  // E2M1: no level table; the area holds only the cross-wave sums (7 tiles x 4 blocks x 1 KB).
  // With kQ > 0, T's block sums (4 blocks x kQ tiles x 1 KB) follow the cross-wave sums.
  constexpr int kRed = kTiles * 4 * 64 * 16;
  constexpr int kTab = kFP4 ? kRed + 4 * kQ * 64 * 16 : kTabBytes;
  static_assert(kRed + 4 * kQ * 64 * 16 <= kTab, "cross-wave sums exceed the table area");
  __shared__ __align__(16) uint32_t stab[kTab / 4];
  auto slot = [&](int i) -> uint8_t * {
    return i == 0 ? slot0 : i == 1 ? slot1 : i == 2 ? slot2 : slot3;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = g.w.k, N = g.w.n;
  const int kblk = (int)(K / 64);
  const int nst = kblk / 4;                        // stages = 4-block groups of a row
  const int64_t n0 = (int64_t)blockIdx.x * kRows;
  const int64_t rows = (N - n0 < kRows) ? N - n0 : kRows;

  // Buffer resources: rows at or past N (codes, block codes) and rows of X at or past M read as
  // zero. Run indices are taken relative to run0 = floor(n0 * kblk / 256), the run of the
  // workgroup's first block, with that block's offset in its run (boff) added back.
  const i32x4 rC = rsrc_words(g.w.codes + n0 * (K / 2), rows * (K / 2));
  // NF4: int8 block codes; E2M1: the E4M3 group scales (K / 16 bytes per row)
  const i32x4 rQ = kFP4 ? rsrc_words(reinterpret_cast<const uint8_t *>(g.w.absmax) + n0 * (K / 16), rows * (K / 16))
                        : rsrc_words(reinterpret_cast<const int8_t *>(g.w.absmax) + n0 * kblk, rows * kblk);
  const int64_t b0 = n0 * kblk;                    // flattened index of the first block
  const int64_t run0 = b0 >> 8;
  const int boff = (int)(b0 & 255);
  const int64_t nruns = (N * kblk + 255) / 256;
  const i32x4 rS = rsrc_words(g.w.scale + run0, kFP4 ? 0 : (nruns - run0) * 4);
  const i32x4 rX = rsrc_words(g.X, g.M * K * 2);
  const i32x4 rAw = rsrc_words(g.A, kTlds ? (int64_t)g.r * K * 2 : 0);   // ranks past r read as zero

  // Copy roles, per stage (6 copies for each wave of the copying group, none for the other), with
  // w = wave % 4:
  // the codes are 14 pieces of 1 KB, rows 8 i .. 8 i + 7: lane L -> row 8 i + L / 8, LDS chunk
  // L % 8, which holds the row's 16-byte chunk (L % 8) ^ ((row / 2) % 8); wave w copies pieces w,
  // w + 4, w + 8 and, for w < 2, w + 12. X is 8 pieces, rows 2 i, 2 i + 1: lane L -> row
  // 2 i + L / 32, LDS chunk L % 32 holding chunk (L % 32) ^ (row % 16) of the row's 512 bytes; wave
  // w copies pieces w and w + 4. Waves w = 2, 3 copy the run scale of the stage's group for rows
  // 64 (w - 2) + L. Once every 4 stages, waves w = 0, 1 also copy the int8 codes of the next 4
  // groups (16 bytes) for rows 64 w + L into a code window. (Used by the copying group only.)
  const int cw = wave & 3;
  auto code_voff = [&](int i) {
    const int r = 8 * i + (lane >> 3);
    return (uint32_t)(r * (K / 2) + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
  };
  // pieces w + 4 c lie 32 c rows below piece w with the same chunk placement: one lane offset,
  // 16 K c bytes more in the scalar offset
  const uint32_t cvoff = code_voff(cw);
  uint32_t xvoff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int xrow = 2 * (cw + 4 * h) + (lane >> 5);
    xvoff[h] = (uint32_t)(xrow * K * 2 + 16 * ((lane & 31) ^ (xrow & 15)));
  }
  const int krow = 64 * (wave & 1) + lane;          // row of the block constants copied
  const uint32_t qvoff = (uint32_t)(krow * kblk);
  // E2M1: waves 2, 3 copy the 16 scale bytes of the stage for rows 64 (w - 2) + L; the lanes of
  // rows past the 112 (wave 3, lanes 48 ..) copy nothing (their LDS bytes would lie past the slot)
  const uint32_t gvoff = (uint32_t)(krow * (K / 16));
  const bool gcopy = !kFP4 || cw == 2 || lane < kRows - 64;
  const uint32_t sdst = kSOff + 256 * (wave & 1), qdst = 1024 * (wave & 1);

  // Workgroups start at different groups of K (in steps of 4, which keeps the code windows
  // aligned): stage st reads group (st + rot) % nst. All workgroups walking K in step would send
  // their requests to the same few memory channels at a time (measured: the DMA stream alone runs
  // at 4.1 TB/s in step and 5.0 TB/s staggered).
  const int rot = (nst >= 8 && nst % 4 == 0) ? (int)(blockIdx.x % (unsigned)(nst / 4)) * 4 : 0;
  // Copies of stage st into slot dst (look-ahead past the end re-reads the last stage into a slot
  // nobody reads any more); with the window flag, waves w = 0, 1 also copy the block codes of
  // stages st .. st + 3 into window qw. Stage numbers here are the workgroup's own order; the
  // group of K they read is rotated by rot. Called by the copying group only.
  auto group_of = [&](int st) {
    st = st < nst ? st : nst - 1;
    st += rot;
    return st < nst ? st : st - nst;
  };
  auto dma = [&](int st, uint32_t dst, bool window, uint32_t qw) {
    st = group_of(st);
    // kStageCopies = 6 copies: codes (3, and a 4th for w = 0, 1), X (2) (and A, kACopies), then the
    // run scales or E2M1 group scales (w = 2, 3)
#pragma unroll
    for (int c = 0; c < 3; ++c) dma16(rC, dst + 1024 * (cw + 4 * c), cvoff, (uint32_t)(st * 128 + c * 16 * K));
    if (cw < 2) dma16(rC, dst + 1024 * (cw + 12), cvoff, (uint32_t)(st * 128 + 48 * K));
#pragma unroll
    for (int h = 0; h < 2; ++h) dma16(rX, dst + kXOff + 1024 * (cw + 4 * h), xvoff[h], (uint32_t)(st * 512));
    // kACopies more (E2M1 forming T): A's pieces in X's layout (rank rows at X's row offsets)
    if constexpr (kTlds) {
#pragma unroll
      for (int h = 0; h < kACopies; ++h)
        dma16(rAw, dst + kAOff + 1024 * (cw + 4 * h), xvoff[h], (uint32_t)(st * 512));
    }
    if (cw >= 2) {
      if constexpr (kFP4) {
        if (gcopy) dma16(rQ, dst + kSOff + 1024 * (cw - 2), gvoff, (uint32_t)(st * 16));
      } else {
        const uint32_t run = (uint32_t)((boff + krow * kblk + 4 * st) >> 8);
        dma4(rS, dst + sdst, run * 4);
      }
    }
    // kWindowCopies more: the block codes of stages st .. st + 3 (w = 0, 1; NF4 only)
#pragma unroll
    for (int c = 0; c < kWindowCopies; ++c)
      if (!kFP4 && window && cw < 2) dma16(rQ, qw + qdst, qvoff + 4 * st, 0);
  };

  // LoRA operands of the tile this wave finishes (tile 4 g + j below, g = wave / 4,
  // j = wave % 4), loaded now so that their latency hides under the main loop: rank steps of 32,
  // lane (nl, gl) holds ranks 32 s + 8 gl .. + 7 of T row nl and of B row 16 t + nl (16-byte loads
  // when r % 8 == 0; ranks at or past r, rows past M or N read as zero). Issued before the first
  // copies, so the first stage wait covers them.
  const int tfin = 4 * (wave >> 2) + (wave & 3);
  const int nlf = lane & 15, glf = lane >> 4;
  const bool lvec = g.r > 0 && g.r % 8 == 0 && tfin < kTiles;
  u32x4 tpre[4], bpre[4];
  {
    // every load is issued (no branch, no register copies that would wait for them); those not
    // needed read outside the buffers and return zero (T is read from LDS at the end when the
    // kernel forms it)
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(g.T, lvec && !g.tpart ? g.M * g.r * 2 : 0);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (lvec ? n0 * g.r : 0), lvec ? rows * g.r * 2 : 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 32 * q + 8 * glf;
      const uint32_t off = j0 < g.r ? 0u : 0x80000000u;   // ranks past r: outside both buffers
      if constexpr (kQ == 0)
        tpre[q] = __builtin_amdgcn_raw_buffer_load_b128(rT, (uint32_t)((nlf * g.r + j0) * 2) | off, 0, 0);
      else
        tpre[q] = u32x4{0u, 0u, 0u, 0u};
      bpre[q] = __builtin_amdgcn_raw_buffer_load_b128(rB, (uint32_t)(((16 * tfin + nlf) * g.r + j0) * 2) | off, 0, 0);
    }
  }

  // In-kernel T (kQ > 0). NF4, waves 0..3: wave (0, jb) holds, per rank tile q, the pieces of A
  // rows 16 q + nl that match its X fragments of block jb (the same 8 elements per lane as the
  // weight operand: 16 gl + 8 h), loaded two stages ahead into abuf[stage % 2] (one stage ahead,
  // the wait for them measured 2.5 us of a 33 us launch). E2M1, waves 4..7: the same pieces from
  // the stage's A slice in LDS (tmma below). Either way tacc[q] sums X A^T over the stages for
  // block jb (lane (nl, gl): T[4 gl + v][16 q + nl]). Ranks past r and rows of X past M read as
  // zero.
  const int grp = wave >> 2, jb = wave & 3;
  // the copying wave group: the 4-tile waves (0) for NF4 with T given, else the 3-tile waves (1)
  // (E2M1's 4-tile waves spill with the copies; NF4 forming T costs 3.3 us on the 3-tile waves)
  constexpr int kCopyGrp = (!kFP4 && kQ == 0) ? 0 : 1;
  // Each stage's instructions kept in the stage (the compiler otherwise moves MFMAs of one stage
  // past the next stage's barrier): measured faster in these two forms (NF4 with T given 28.3-28.6
  // against 28.7-28.8 us, E2M1 forming T 35.5 against 36.4 us), slower in E2M1 with T given (34.0
  // against 33.2-33.6 us) and equal in NF4 forming T.
  constexpr bool kPin = (!kFP4 && kQ == 0) || kTlds;
  const int nl = lane & 15, gl = lane >> 4;
  f32x4 tacc[kQ > 0 ? kQ : 1];
  u32x4 abuf[2][kQ > 0 ? kQ : 1][2];
  uint32_t avoff[kQ > 0 ? kQ : 1];
  const __amdgpu_buffer_rsrc_t rA = make_rsrc(g.A, kQ > 0 ? (int64_t)g.r * K * 2 : 0);
  auto aload = [&](int st) {
    const uint32_t soff = (uint32_t)(group_of(st) * 512);
    const int b = st & 1;
#pragma unroll
    for (int q = 0; q < kQ; ++q)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        abuf[b][q][h] = __builtin_amdgcn_raw_buffer_load_b128(rA, avoff[q] + 16u * h, soff, 0);
  };
  if constexpr (kQ > 0) {
#pragma unroll
    for (int q = 0; q < kQ; ++q) {
      tacc[q] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int64_t j = 16 * q + nl;
      avoff[q] = (uint32_t)((j * K + 64 * jb + 16 * gl) * 2);
    }
  }

  if (grp == kCopyGrp) {
    dma(0, lds_addr(slot0), true, lds_addr(qwin0));
    dma(1, lds_addr(slot1), false, 0);
    dma(2, lds_addr(slot2), false, 0);
  }

  // Table (NF4): uint4 i holds four copies of entry e = i / 16: (level[e >> 4], level[e & 15]) as
  // a bf16 pair (the high nibble is the earlier element). The 16 levels go through LDS (the start
  // of slot 3, whose first copy is issued after the first stage barrier) so that the indexed reads
  // are LDS reads, not memory loads that would join the copies in flight.
  if constexpr (!kFP4) {
    float *lv = reinterpret_cast<float *>(slot3);
    if (tid == 0) {
#pragma unroll
      for (int j = 0; j < 16; ++j) lv[j] = g.t.level[j];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    for (int i = tid; i < kTabBytes / 16; i += kThreads) {
      const int e = i >> 4;
      const uint32_t v = pack_bf16x2(lv[e >> 4], lv[e & 15]);
      reinterpret_cast<uint4 *>(stab)[i] = make_uint4(v, v, v, v);
    }
  }

  // T from split partials: every workgroup adds them (in split order, as the separate reduction
  // does) into bf16 T in LDS (slot 3, after the levels), workgroup 0 also stores T, and the
  // finishing waves take their LoRA operands from LDS. The partial loads wait for the copies
  // issued above too (the compiler does not see those), which costs little: the first stage waits
  // for them anyway.
  if (kQ == 0 && g.tpart) {
    uint16_t *tl = reinterpret_cast<uint16_t *>(slot3 + 1024);
    const int r = g.r;
    for (int idx = tid; idx < 16 * r; idx += kThreads) {
      const int m = idx / r, j = idx - m * r;
      float a = 0.f;
      if (m < g.M) {
        const float *pp = g.tpart + ((int64_t)m * r + j) * g.tsplits;
        int q = 0;
        // loads issued 32 (then 8) at a time, added in split order
        for (; q + 32 <= g.tsplits; q += 32) {
          float v[32];
#pragma unroll
          for (int e = 0; e < 32; ++e) v[e] = pp[q + e];
#pragma unroll
          for (int e = 0; e < 32; ++e) a += v[e];
        }
        for (; q + 8 <= g.tsplits; q += 8) {
          float v[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) v[e] = pp[q + e];
#pragma unroll
          for (int e = 0; e < 8; ++e) a += v[e];
        }
        for (; q < g.tsplits; ++q) a += pp[q];
      }
      const uint16_t tb = (uint16_t)(pack_bf16x2(a, 0.f) & 0xFFFFu);
      tl[idx] = tb;
      if (blockIdx.x == 0 && m < g.M) g.tout[idx] = tb;
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (lvec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j0 = 32 * q + 8 * glf;
        tpre[q] = j0 < r ? *reinterpret_cast<const u32x4 *>(tl + nlf * r + j0) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }

  // This wave's operands: block jb of each stage for tiles t = 4 g + tt. MFMA lanes: nl = column
  // (weight row 16 t + nl) and X row, gl = k-group: the lane takes bytes 8 gl .. 8 gl + 7 of the
  // row's block (elements 16 gl .. 16 gl + 15; the first 8 feed MFMA 0, the next 8 MFMA 1) and the
  // same elements of X.
  const int ntiles = grp == 0 ? 4 : kTiles - 4;
  // E2M1: the lane takes bytes 16 h + 4 gl .. + 3 of the block for slice h (elements
  // 32 h + 8 gl .. + 7; lanes gl = 0, 1 hold the slice's first group, gl = 2, 3 its second), the
  // same elements of X, and the block's 4 group scales (saddr).
  uint32_t caddr[4], qaddr[4], saddr[4], xaddr[2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int row = 16 * (4 * grp + tt) + nl;
    caddr[tt] = kFP4 ? (uint32_t)(row * 128 + 16 * ((2 * jb) ^ ((row >> 1) & 7)) + 4 * gl)
                     : (uint32_t)(row * 128 + 16 * ((2 * jb + (gl >> 1)) ^ ((row >> 1) & 7)) + 8 * (gl & 1));
    qaddr[tt] = (uint32_t)(row * 16 + jb);          // in the window, + 4 * (stage % 4)
    saddr[tt] = kFP4 ? (uint32_t)(kSOff + row * 16 + 4 * jb) : (uint32_t)(kSOff + row * 4);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    xaddr[hh] = kFP4 ? (uint32_t)(kXOff + nl * 512 + 16 * ((8 * jb + 4 * hh + gl) ^ nl))
                     : (uint32_t)(kXOff + nl * 512 + 16 * ((8 * jb + 2 * gl + hh) ^ nl));
  const uint32_t lane_off = (uint32_t)lane * 4;
  const char *ctab = reinterpret_cast<const char *>(stab);

  f32x4 acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // T's products for this stage's block jb, after the wave's tiles. NF4 (waves 0..3): from
  // abuf[tpar] (tpar = stage % 2): the A pieces were loaded two stages ago, and they are the only
  // vector-memory loads these waves have in flight, so the compiler's wait for them is exact.
  // E2M1 (waves 4..7): from the stage's A slice in LDS, at the X fragments' addresses.
  int tpar = 0;
  auto tmma = [&](const bf16x8 &x0, const bf16x8 &x1, uint32_t sb, auto role) {
    if constexpr (!kFP4 && kQ > 0 && !decltype(role)::copies) {
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        tacc[q] = mfma16x16x32(x0, __builtin_bit_cast(bf16x8, abuf[tpar][q][0]), tacc[q]);
        tacc[q] = mfma16x16x32(x1, __builtin_bit_cast(bf16x8, abuf[tpar][q][1]), tacc[q]);
      }
    }
    if constexpr (kTlds && decltype(role)::copies) {
      const bf16x8 a0 = lds_ld<bf16x8>(sb + xaddr[0] + (kAOff - kXOff));
      const bf16x8 a1 = lds_ld<bf16x8>(sb + xaddr[1] + (kAOff - kXOff));
      tacc[0] = mfma16x16x32(x0, a0, tacc[0]);
      tacc[0] = mfma16x16x32(x1, a1, tacc[0]);
    }
  };
  // One stage from slot base sb and window base qb (LDS byte addresses).
  // nt: the wave's tile count as a constant (TileCount<4> for waves 0..3, TileCount<3> for 4..7)
  auto consume = [&](uint32_t sb, uint32_t qb, auto nt, auto role) {
    const bf16x8 x0 = lds_ld<bf16x8>(sb + xaddr[0]);
    const bf16x8 x1 = lds_ld<bf16x8>(sb + xaddr[1]);
    if constexpr (kFP4) {
      // X with the halves of each dword swapped (element 2 i + 1 low, 2 i high, as the codes
      // convert), masked to one group each: xs[q] keeps the lanes holding group q of the block
      // (slice q / 2, lanes gl < 2 for even q, gl >= 2 for odd q) and zeroes the rest
      const uint32_t lm = gl < 2 ? 0xFFFFFFFFu : 0u;
      u32x4 u0 = __builtin_bit_cast(u32x4, x0), u1 = __builtin_bit_cast(u32x4, x1);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u0[e] = __builtin_amdgcn_alignbit(u0[e], u0[e], 16);
        u1[e] = __builtin_amdgcn_alignbit(u1[e], u1[e], 16);
      }
      const bf16x8 xs[4] = {__builtin_bit_cast(bf16x8, u0 & lm), __builtin_bit_cast(bf16x8, u0 & ~lm),
                            __builtin_bit_cast(bf16x8, u1 & lm), __builtin_bit_cast(bf16x8, u1 & ~lm)};
#pragma unroll
      for (int tt = 0; tt < decltype(nt)::n; ++tt) {
        const uint32_t cw0 = lds_ld<uint32_t>(sb + caddr[tt]);
        const uint32_t cw1 = lds_ld<uint32_t>(sb + (caddr[tt] ^ 16u));
        const uint32_t sc = lds_ld<uint32_t>(sb + saddr[tt]);
        const bf16x8 w0 = __builtin_bit_cast(
            bf16x8, u32x4{cvt_fp4x2<0>(cw0), cvt_fp4x2<1>(cw0), cvt_fp4x2<2>(cw0), cvt_fp4x2<3>(cw0)});
        const bf16x8 w1 = __builtin_bit_cast(
            bf16x8, u32x4{cvt_fp4x2<0>(cw1), cvt_fp4x2<1>(cw1), cvt_fp4x2<2>(cw1), cvt_fp4x2<3>(cw1)});
        // group q's partial sum times its scale (byte q of sc, E4M3)
        const float sg[4] = {__builtin_amdgcn_cvt_f32_fp8((int)sc, 0), __builtin_amdgcn_cvt_f32_fp8((int)sc, 1),
                             __builtin_amdgcn_cvt_f32_fp8((int)sc, 2), __builtin_amdgcn_cvt_f32_fp8((int)sc, 3)};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 pg = mfma16x16x32(xs[q], q < 2 ? w0 : w1, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[tt][v] += sg[q] * pg[v];
        }
      }
      tmma(x0, x1, sb, role);
      return;
    }
#pragma unroll
    for (int tt = 0; tt < decltype(nt)::n; ++tt) {
      const u32x2 cw = lds_ld<u32x2>(sb + caddr[tt]);
      const float a = float(lds_ld<int8_t>(qb + qaddr[tt])) * lds_ld<float>(sb + saddr[tt]);
      uint32_t o[8];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t addr = perm(cw[hh], lane_off, 0x0C0C0400u | ((4u + i) << 8));
          o[4 * hh + i] = *reinterpret_cast<const uint32_t *>(ctab + addr);
        }
      const bf16x8 w0 = __builtin_bit_cast(bf16x8, make_uint4(o[0], o[1], o[2], o[3]));
      const bf16x8 w1 = __builtin_bit_cast(bf16x8, make_uint4(o[4], o[5], o[6], o[7]));
      f32x4 part = mfma16x16x32(x0, w0, f32x4{0.f, 0.f, 0.f, 0.f});
      part = mfma16x16x32(x1, w1, part);
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[tt][v] += a * part[v];
    }
    tmma(x0, x1, sb, role);
  };

  // Stage st (slot st % 4, code window st / 4 % 2). The copying group: wait until this wave's
  // copies of st have landed (those of st + 1 and st + 2 may stay in flight), barrier (everyone's
  // copies of st have landed and everyone is done with stage st - 1, whose slot the next copies
  // overwrite), copies of st + 3, then the stage's MFMAs. The other group: the barrier, the
  // stage's MFMAs, then (NF4, kQ > 0) the A pieces of stage st + 2 into the buffer the stage has
  // just used. The window of stages 4 j .. 4 j + 3 is copied with stage 4 j (issued in stage
  // 4 j - 3, after window j - 2 was last read in stage 4 j - 5).
  auto stage = [&](int st, int i, int win, auto nt, auto role) {
    const uint32_t sb = opaque(lds_addr(slot(i)));
    const uint32_t qb = opaque(lds_addr(win ? qwin1 : qwin0) + 4 * i);   // 4 codes of each row
    if constexpr (decltype(role)::copies) {
      // copies issued in the two stages before st (phases (i + 2) % 4 and (i + 3) % 4 issue the
      // copies of phases i + 1 and i + 2 = (i + 1) % 4, (i + 2) % 4; the window goes with phase 0)
      const bool w1 = ((i + 1) & 3) == 0, w2 = ((i + 2) & 3) == 0;
      if (!kFP4 && (w1 || w2) && cw < 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPending + kWindowCopies) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kPending) : "memory");
      const int in = (i + 3) & 3;                      // phase of stage st + 3
      dma(st + 3, lds_addr(slot(in)), in == 0, lds_addr(win ? qwin0 : qwin1));
      consume(sb, qb, nt, role);
      if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      tpar = st & 1;
      consume(sb, qb, nt, role);
      if constexpr (!kFP4 && kQ > 0) aload(st + 2);
      if constexpr (kPin) __builtin_amdgcn_sched_barrier(0);
    }
  };
  // One stage loop per wave group (each runs nst stages with one barrier each).
  auto walk = [&](auto role, auto nt) {
    int st = 0;
    if constexpr (kFP4) {   // no code windows: a loop over the four slots
#pragma unroll 1
      for (; st + 4 <= nst; st += 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) stage(st + j, j, 0, nt, role);
      }
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (st + j < nst) stage(st + j, j, 0, nt, role);
    } else {
#pragma unroll 1
      for (; st + 8 <= nst; st += 8) {
#pragma unroll
        for (int j = 0; j < 8; ++j) stage(st + j, j & 3, j >> 2, nt, role);
      }
#pragma unroll
      for (int j = 0; j < 7; ++j)
        if (st + j < nst) stage(st + j, j & 3, j >> 2, nt, role);
    }
  };
  if (grp == kCopyGrp) {
    if constexpr (kCopyGrp == 0) walk(CopyRole{}, TileCount<4>{}); else walk(CopyRole{}, TileCount<3>{});
  } else {
    // the first A pieces (stages 0 and 1) here, on this branch only: issued before the branch, the
    // compiler would count them as possibly in flight on the copying waves' path too and wait for
    // them there
    if constexpr (!kFP4 && kQ > 0) { aload(0); aload(1); }
    if constexpr (kCopyGrp == 0) walk(TRole{}, TileCount<3>{}); else walk(TRole{}, TileCount<4>{});
    // the look-ahead A pieces of the last two stages retired here, as the compiler sees it (an
    // s_waitcnt it emits itself, vmcnt(0)), so that no path into the copying waves' loop carries
    // loads it would wait for there
    if constexpr (!kFP4 && kQ > 0) __builtin_amdgcn_s_waitcnt(0x0F70);
  }

  // Every wave past its last stage (and every DMA landed: the look-ahead loads wrote into slots
  // nobody reads any more) before the table area is reused for the cross-wave sums.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // Partial sums red[tile][block][lane]; wave (g, jb) then finishes tile 4 g + jb (7 tiles).
  f32x4 *red = reinterpret_cast<f32x4 *>(stab);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    if (tt < ntiles) red[((4 * grp + tt) * 4 + jb) * 64 + lane] = acc[tt];
  // and T's block sums tp[block][rank tile][lane] after them
  f32x4 *tp = red + kTiles * 4 * 64;
  if constexpr (kQ > 0) {
    if (grp == (kFP4 ? 1 : 0)) {   // the waves that formed T
#pragma unroll
      for (int q = 0; q < kQ; ++q) tp[(jb * kQ + q) * 64 + lane] = tacc[q];
    }
  }
  __syncthreads();
  if constexpr (kQ > 0) {
    // T[m][j]: the four block sums added in block order, rounded to bf16, into LDS (slot 0, free
    // now) for the LoRA term below; workgroup 0 also stores T. Each workgroup sums T in its own
    // walk order over K; workgroup 0's (rot = 0) is the plain order.
    uint16_t *tl = reinterpret_cast<uint16_t *>(slot0);
    const int r = g.r;
    for (int idx = tid; idx < 16 * r; idx += kThreads) {
      const int m = idx / r, j = idx - m * r;
      const int li = (j & 15) + 16 * (m >> 2), q = j >> 4, v = m & 3;
      float a = tp[q * 64 + li][v];
#pragma unroll
      for (int b = 1; b < 4; ++b) a += tp[(b * kQ + q) * 64 + li][v];
      const uint16_t tb = (uint16_t)(pack_bf16x2(a, 0.f) & 0xFFFFu);
      tl[idx] = tb;
      if (blockIdx.x == 0 && m < g.M) g.tout[idx] = tb;
    }
    __syncthreads();
    if (lvec) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j0 = 32 * q + 8 * glf;
        tpre[q] = j0 < r ? *reinterpret_cast<const u32x4 *>(tl + nlf * r + j0) : u32x4{0u, 0u, 0u, 0u};
      }
    }
  }
  const int t = 4 * grp + jb;
  if (t >= kTiles) return;
  const int row = 16 * t + nl;
  f32x4 y = red[(t * 4) * 64 + lane];
#pragma unroll
  for (int jj = 1; jj < 4; ++jj) y += red[(t * 4 + jj) * 64 + lane];
  if (kFP4) {   // the sums are in units of the tensor scale (1 for an all-zero weight)
    const float S = *g.w.scale;
    y *= S > 0.f ? S : 1.f;
  }

  // LoRA term on the matrix cores: s * T[m][:] . B[n][:] for the tile's 16 columns, in steps of
  // 32 ranks (A operand: T row m, B operand: B row n, both rank-contiguous). With r % 8 == 0 the
  // operands were loaded before the main loop; otherwise they are read here element by element.
  if (lvec) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      if (32 * q < g.r) {
        const f32x4 lp = mfma16x16x32(__builtin_bit_cast(bf16x8, tpre[q]),
                                      __builtin_bit_cast(bf16x8, bpre[q]), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int v = 0; v < 4; ++v) y[v] += g.s * lp[v];
      }
  } else if (g.r > 0) {
    const int r = g.r;
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(g.T, g.M * r * 2);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + n0 * r, rows * r * 2);
#pragma unroll 1
    for (int j0 = 0; j0 < r; j0 += 32) {
      uint32_t tb[8], bb[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int jr = j0 + gl * 8 + e;
        const bool in = jr < r;
        bb[e] = in ? __builtin_amdgcn_raw_buffer_load_b16(rB, (uint32_t)((row * r + jr) * 2), 0, 0) : 0u;
        tb[e] = in ? __builtin_amdgcn_raw_buffer_load_b16(rT, (uint32_t)((nl * r + jr) * 2), 0, 0) : 0u;
      }
      u32x4 bw, tw;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bw[q] = (bb[2 * q] & 0xFFFFu) | (bb[2 * q + 1] << 16);
        tw[q] = (tb[2 * q] & 0xFFFFu) | (tb[2 * q + 1] << 16);
      }
      const f32x4 lp = mfma16x16x32(__builtin_bit_cast(bf16x8, tw), __builtin_bit_cast(bf16x8, bw),
                                    f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int v = 0; v < 4; ++v) y[v] += g.s * lp[v];
    }
  }

  // y[v] = Y[m][n] for m = 4 gl + v, n = n0 + 16 t + nl
  const int64_t gn = n0 + row;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t m = 4 * gl + v;
    if (m < g.M && gn < N) g.Y[m * N + gn] = (uint16_t)(pack_bf16x2(y[v], 0.f) & 0xFFFFu);
  }
}

}  // namespace

namespace {
Dec16Args dec16_args(const GemmArgs &ga) {
  Dec16Args g;
  g.X = ga.a_side;
  g.T = ga.lora_a;
  g.B = ga.lora_b;
  g.w = ga.w;
  g.M = ga.M;
  g.r = ga.r;
  g.s = ga.s;
  g.Y = ga.out;
  g.t = ga.t;
  g.tpart = nullptr;
  g.tsplits = 0;
  g.tout = nullptr;
  g.A = nullptr;
  return g;
}

template <int kQ>
hipError_t launch_dec16(const Dec16Args &g, hipStream_t st) {
  const unsigned grid = (unsigned)((g.w.n + kRows - 1) / kRows);
  if constexpr (kQ <= 1) {
    if (g.w.fp4) {
      decode16_fwd_kernel<true, kQ><<<dim3(grid), dim3(kThreads), 0, st>>>(g);
      return hipGetLastError();
    }
  }
  decode16_fwd_kernel<false, kQ><<<dim3(grid), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_decode16_fwd(const GemmArgs &ga, hipStream_t st) {
  if (ga.M > 16 || !(ga.w.dq || ga.w.fp4) || ga.w.k % 256 != 0) return hipErrorInvalidValue;
  return launch_dec16<0>(dec16_args(ga), st);
}

hipError_t launch_decode16_fwd_tpart(const GemmArgs &ga, const float *tpart, int tsplits,
                                     uint16_t *tout, hipStream_t st) {
  if (ga.M > 16 || !(ga.w.dq || ga.w.fp4) || ga.w.k % 256 != 0 || ga.r % 8 != 0 || !tpart || tsplits < 1)
    return hipErrorInvalidValue;
  Dec16Args g = dec16_args(ga);
  g.tpart = tpart;
  g.tsplits = tsplits;
  g.tout = tout;
  return launch_dec16<0>(g, st);
}

hipError_t launch_decode16_fwd_tin(const GemmArgs &ga, const uint16_t *A, uint16_t *tout, hipStream_t st) {
  const int maxr = ga.w.fp4 ? kDecode16MaxTinRankE2M1 : kDecode16MaxTinRank;
  if (ga.M > 16 || !(ga.w.dq || ga.w.fp4) || ga.w.k % 256 != 0 || ga.r < 8 || ga.r > maxr || ga.r % 8 != 0 ||
      !A || !tout)
    return hipErrorInvalidValue;
  Dec16Args g = dec16_args(ga);
  g.T = nullptr;
  g.A = A;
  g.tout = tout;
  if (ga.r <= 16) return launch_dec16<1>(g, st);
  if (ga.r <= 32) return launch_dec16<2>(g, st);
  return launch_dec16<4>(g, st);
}

}  // namespace nf4q

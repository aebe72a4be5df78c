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
//     partial sums of a tile meet in LDS at the end.
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
  uint16_t *tout;       // with tpart: T (bf16 [M][r]) written by workgroup 0
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

__global__ __launch_bounds__(kThreads) void decode16_fwd_kernel(Dec16Args g) {
  // Four stage slots, two windows of block codes and the level-pair table, which holds the
  // cross-wave sums at the end.
  __shared__ __align__(16) uint8_t slot0[kSlotBytes];
  __shared__ __align__(16) uint8_t slot1[kSlotBytes];
  __shared__ __align__(16) uint8_t slot2[kSlotBytes];
  __shared__ __align__(16) uint8_t slot3[kSlotBytes];
  __shared__ __align__(16) uint8_t qwin0[kQWinBytes];
  __shared__ __align__(16) uint8_t qwin1[kQWinBytes];
  __shared__ __align__(16) uint32_t stab[kTabBytes / 4];
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
  const i32x4 rQ = rsrc_words(reinterpret_cast<const int8_t *>(g.w.absmax) + n0 * kblk, rows * kblk);
  const int64_t b0 = n0 * kblk;                    // flattened index of the first block
  const int64_t run0 = b0 >> 8;
  const int boff = (int)(b0 & 255);
  const int64_t nruns = (N * kblk + 255) / 256;
  const i32x4 rS = rsrc_words(g.w.scale + run0, (nruns - run0) * 4);
  const i32x4 rX = rsrc_words(g.X, g.M * K * 2);

  // DMA roles, per stage (3 copies per wave): the codes are 14 pieces of 1 KB, rows 8 i .. 8 i + 7;
  // lane L -> row 8 i + L / 8, LDS chunk L % 8, which holds the row's 16-byte chunk
  // (L % 8) ^ ((row / 2) % 8). Wave w copies pieces w and, for w < 6, w + 8. X is 8 pieces,
  // rows 2 w, 2 w + 1: lane L -> row 2 w + L / 32, LDS chunk L % 32 holding chunk
  // (L % 32) ^ (row % 16) of the row's 512 bytes; wave w copies piece w. Waves 6, 7 copy the run
  // scale of the stage's group for rows 64 (w - 6) + L. Once every 4 stages, waves 0, 1 also copy
  // the int8 codes of the next 4 groups (16 bytes) for rows 64 w + L into a code window.
  auto code_voff = [&](int i) {
    const int r = 8 * i + (lane >> 3);
    return (uint32_t)(r * (K / 2) + 16 * ((lane & 7) ^ ((r >> 1) & 7)));
  };
  const uint32_t cvoff0 = code_voff(wave), cvoff1 = code_voff(wave < 6 ? wave + 8 : wave);
  const int xrow = 2 * wave + (lane >> 5);
  const uint32_t xvoff = (uint32_t)(xrow * K * 2 + 16 * ((lane & 31) ^ (xrow & 15)));
  const int krow = 64 * (wave & 1) + lane;          // row of the block constants copied
  const uint32_t qvoff = (uint32_t)(krow * kblk);
  const uint32_t cdst0 = 1024 * wave, cdst1 = 1024 * (wave + 8), xdst = kXOff + 1024 * wave;
  const uint32_t sdst = kSOff + 256 * (wave & 1), qdst = 1024 * (wave & 1);

  // Workgroups start at different groups of K (in steps of 4, which keeps the code windows
  // aligned): stage st reads group (st + rot) % nst. All workgroups walking K in step would send
  // their requests to the same few memory channels at a time (measured: the DMA stream alone runs
  // at 4.1 TB/s in step and 5.0 TB/s staggered).
  const int rot = (nst >= 8 && nst % 4 == 0) ? (int)(blockIdx.x % (unsigned)(nst / 4)) * 4 : 0;
  // Copies of stage st into slot dst (look-ahead past the end re-reads the last stage into a slot
  // nobody reads any more); with the window flag, waves 8, 9 also copy the block codes of stages
  // st .. st + 3 into window qw. Stage numbers here are the workgroup's own order; the group of
  // K they read is rotated by rot.
  auto dma = [&](int st, uint32_t dst, bool window, uint32_t qw) {
    st = st < nst ? st : nst - 1;
    st += rot;
    st = st < nst ? st : st - nst;
    dma16(rC, dst + cdst0, cvoff0, (uint32_t)(st * 128));
    dma16(rX, dst + xdst, xvoff, (uint32_t)(st * 512));
    if (wave < 6) {
      dma16(rC, dst + cdst1, cvoff1, (uint32_t)(st * 128));
      if (window && wave < 2) dma16(rQ, qw + qdst, qvoff + 4 * st, 0);
    } else {
      const uint32_t run = (uint32_t)((boff + krow * kblk + 4 * st) >> 8);
      dma4(rS, dst + sdst, run * 4);
    }
  };
  // Copies this wave issues in one stage's DMA (the count the stage waits below rely on).
  auto ndma = [&](bool window) { return 3 + (int)(window && wave < 2); };

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
    // needed read outside the buffers and return zero
    const __amdgpu_buffer_rsrc_t rT = make_rsrc(g.T, lvec && !g.tpart ? g.M * g.r * 2 : 0);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(g.B + (lvec ? n0 * g.r : 0), lvec ? rows * g.r * 2 : 0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int j0 = 32 * q + 8 * glf;
      const uint32_t off = j0 < g.r ? 0u : 0x80000000u;   // ranks past r: outside both buffers
      tpre[q] = __builtin_amdgcn_raw_buffer_load_b128(rT, (uint32_t)((nlf * g.r + j0) * 2) | off, 0, 0);
      bpre[q] = __builtin_amdgcn_raw_buffer_load_b128(rB, (uint32_t)(((16 * tfin + nlf) * g.r + j0) * 2) | off, 0, 0);
    }
  }

  dma(0, lds_addr(slot0), true, lds_addr(qwin0));
  dma(1, lds_addr(slot1), false, 0);
  dma(2, lds_addr(slot2), false, 0);

  // Table: uint4 i holds four copies of entry e = i / 16: (level[e >> 4], level[e & 15]) as a
  // bf16 pair (the high nibble is the earlier element). The 16 levels go through LDS (the start of
  // slot 3, whose first copy is issued after the first stage barrier) so that the indexed reads
  // are LDS reads, not memory loads that would join the copies in flight.
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

  // T from split partials: every workgroup adds them (in split order, as the separate reduction
  // does) into bf16 T in LDS (slot 3, after the levels), workgroup 0 also stores T, and the
  // finishing waves take their LoRA operands from LDS. The partial loads wait for the copies
  // issued above too (the compiler does not see those), which costs little: the first stage waits
  // for them anyway.
  if (g.tpart) {
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
  const int grp = wave >> 2, jb = wave & 3;
  const int ntiles = grp == 0 ? 4 : kTiles - 4;
  const int nl = lane & 15, gl = lane >> 4;
  uint32_t caddr[4], qaddr[4], saddr[4], xaddr[2];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) {
    const int row = 16 * (4 * grp + tt) + nl;
    caddr[tt] = (uint32_t)(row * 128 + 16 * ((2 * jb + (gl >> 1)) ^ ((row >> 1) & 7)) + 8 * (gl & 1));
    qaddr[tt] = (uint32_t)(row * 16 + jb);          // in the window, + 4 * (stage % 4)
    saddr[tt] = (uint32_t)(kSOff + row * 4);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
    xaddr[hh] = (uint32_t)(kXOff + nl * 512 + 16 * ((8 * jb + 2 * gl + hh) ^ nl));
  const uint32_t lane_off = (uint32_t)lane * 4;
  const char *ctab = reinterpret_cast<const char *>(stab);

  f32x4 acc[4];
#pragma unroll
  for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // One stage from slot base sb and window base qb (LDS byte addresses).
  auto consume = [&](uint32_t sb, uint32_t qb) {
    const bf16x8 x0 = lds_ld<bf16x8>(sb + xaddr[0]);
    const bf16x8 x1 = lds_ld<bf16x8>(sb + xaddr[1]);
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      if (tt == 3 && ntiles == 3) break;
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
  };

  // Stage st (slot st % 4, code window st / 4 % 2): wait until this wave's copies of st have
  // landed (those of st + 1 and st + 2 may stay in flight), barrier (everyone's copies of st have
  // landed and everyone is done with stage st - 1, whose slot the next copies overwrite), copies
  // of st + 3, then the stage's MFMAs. The window of stages 4 j .. 4 j + 3 is copied with stage
  // 4 j (issued in stage 4 j - 3, after window j - 2 was last read in stage 4 j - 5).
  auto stage = [&](int st, int i, int win) {
    // copies issued in the two stages before st (phases (i + 2) % 4 and (i + 3) % 4 issue the
    // copies of phases i + 1 and i + 2 = (i + 1) % 4, (i + 2) % 4; the window goes with phase 0)
    const bool w1 = ((i + 1) & 3) == 0, w2 = ((i + 2) & 3) == 0;
    const int pending = ndma(w1) + ndma(w2);
    if (pending == 7)
      asm volatile("s_waitcnt vmcnt(7) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(6) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int in = (i + 3) & 3;                      // phase of stage st + 3
    dma(st + 3, lds_addr(slot(in)), in == 0, lds_addr(win ? qwin0 : qwin1));
    consume(opaque(lds_addr(slot(i))), opaque(lds_addr(win ? qwin1 : qwin0) + 4 * i));  // 4 codes of each row
  };
  int st = 0;
#pragma unroll 1
  for (; st + 8 <= nst; st += 8) {
#pragma unroll
    for (int j = 0; j < 8; ++j) stage(st + j, j & 3, j >> 2);
  }
#pragma unroll
  for (int j = 0; j < 7; ++j)
    if (st + j < nst) stage(st + j, j & 3, j >> 2);

  // Every wave past its last stage (and every DMA landed: the look-ahead loads wrote into slots
  // nobody reads any more) before the table area is reused for the cross-wave sums.
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // Partial sums red[tile][block][lane]; wave (g, jb) then finishes tile 4 g + jb (7 tiles).
  f32x4 *red = reinterpret_cast<f32x4 *>(stab);
#pragma unroll
  for (int tt = 0; tt < 4; ++tt)
    if (tt < ntiles) red[((4 * grp + tt) * 4 + jb) * 64 + lane] = acc[tt];
  __syncthreads();
  const int t = 4 * grp + jb;
  if (t >= kTiles) return;
  const int row = 16 * t + nl;
  f32x4 y = red[(t * 4) * 64 + lane];
#pragma unroll
  for (int jj = 1; jj < 4; ++jj) y += red[(t * 4 + jj) * 64 + lane];

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

hipError_t launch_decode16_fwd(const GemmArgs &ga, hipStream_t st) {
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
  if (ga.M > 16 || !ga.w.dq || ga.w.k % 256 != 0) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((ga.w.n + kRows - 1) / kRows);
  decode16_fwd_kernel<<<dim3(grid), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_decode16_fwd_tpart(const GemmArgs &ga, const float *tpart, int tsplits,
                                     uint16_t *tout, hipStream_t st) {
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
  g.tpart = tpart;
  g.tsplits = tsplits;
  g.tout = tout;
  if (ga.M > 16 || !ga.w.dq || ga.w.k % 256 != 0 || ga.r % 8 != 0 || !tpart || tsplits < 1)
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((ga.w.n + kRows - 1) / kRows);
  decode16_fwd_kernel<<<dim3(grid), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace nf4q

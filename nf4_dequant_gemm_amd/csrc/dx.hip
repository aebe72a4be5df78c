// Fused input-gradient kernel of the QLoRA layer: dX = dY deq(W) + s U A (gfx950).
//
// The backward pass of the frozen-base QLoRA layer needs the gradient through the dequantised
// base weight and through the adapters; W itself gets no gradient [Unsloth v0.1.463-beta release
// article, "About the Unsloth Project": the 4-bit base is frozen, only the adapters train; the
// Unsloth kernels rewrite the backward pass]. As in the forward kernel, the NF4 weight is decoded
// on the fly into LDS and the rank-r term runs as extra reduction steps into the same tile.
//
// Work split. One workgroup of 8 waves (2 x 4) owns a 256 x 256 tile of dX (rows m, columns k)
// and walks the reduction index n in steps of 64; each wave accumulates 128 (m) x 64 (k) with
// MFMA 16x16x32 (within 256 registers, so two waves share each SIMD and one wave's decode
// overlaps the other's MFMAs). The reduction runs over the weight's ROW index, so the MFMA needs
// the decoded tile transposed: the tile is stored in LDS as it is decoded (64 rows n x 256
// columns k, 16-byte stores) and read with the gfx950 transposing LDS load ds_read_b64_tr_b16,
// which hands each lane 4 consecutive rows of one column -- the operand layout with n as the
// reduction index. Eight threads decode each weight row of the step, 32 columns each, through
// a register table of bf16(level_i * a) (byte permutes, no LDS lookups).
//
// Pipeline per step s: the dY tile of step s+1 goes straight to LDS buffer (s+1) & 1 by DMA
// (buffer_load ... lds, issued at the start of the step, so its latency hides behind a whole
// step) and the codes of step s+2 are loaded into registers; the 64 MFMAs of step s run on LDS
// buffer s & 1 while the weight rows of step s+1 are decoded into buffer (s+1) & 1 between MFMA
// issues.
//
// LDS: the dY tile has rows of 64 bf16 = 8 chunks of 16 bytes, chunk c of row r at slot
// c ^ ((r >> 1) & 7). The weight tile has rows of 256 bf16 = 64 units of 8 bytes, unit u of row
// r at u ^ (4 ((r + 4 (r / 8)) % 8) + 2 ((r / 4) % 2)). Measured on gfx950, a transposing 8-byte
// read serves 32 lanes per 256-byte bank window and a 16-byte write 8 lanes per 128 bytes. The
// multiple of 4 units puts the 8 rows x 32 bytes of every transposing read on distinct banks; the
// 2-unit term (which only permutes units inside a 32-byte group, so reads keep their banks) and
// the decode ownership (the 8 lanes of a write pass take 8 different rows) put every decode write
// on distinct banks. (Eight lanes of one row, the plain mapping, conflicted 4 ways.)
//
// The same body serves the grouped launch of a mixture-of-experts layer [NVFP4 update article,
// "Comprehensive Improvements in Training Performance and Stability"] and the E2M1 weight format
// with FP8 group scales [NVFP4 update article, "NVFP4: A Quantization Format for the Next
// Generation of Hardware"] (template parameters of dx_body).
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

constexpr int kT = 256;
constexpr int kS = 64;
constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr int kYChunks = kT * kS / 8;   // dY tile: 2048 chunks of 16 bytes
constexpr int kWElems = kS * kT;        // weight tile: 64 x 256 bf16
constexpr int kGroupM = 4;              // row blocks per tile group (see the tile order)

__device__ __forceinline__ int swzd(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }
// bf16 index of 8-byte unit u of weight-tile row r
__device__ __forceinline__ int wunit(int r, int u) {
  return r * kT + ((u ^ (4 * ((r + 4 * (r >> 3)) & 7) + 2 * ((r >> 2) & 1))) << 2);
}
// Weight-tile ownership of thread t: row 8 (t / 64) + t % 8, 32-column segment (t / 8) % 8, so
// that the 8 lanes of a write pass hold 8 different rows.
__device__ __forceinline__ int own_row(int t) { return ((t >> 6) << 3) | (t & 7); }
__device__ __forceinline__ int own_seg(int t) { return (t >> 3) & 7; }

__device__ __forceinline__ int tile_remap(int hw, int tiles) {
  const int per = tiles >> 3, rem = tiles & 7, x = hw & 7;
  return x * per + (x < rem ? x : rem) + (hw >> 3);
}

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
__device__ __forceinline__ s16x4 lds_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(p));
}

struct CStage {
  u32x4 c;           // 16 bytes of codes (32 columns) of the thread's weight row
  uint32_t q, sc;    // block constant (int8 or float bits) and run scale bits
};

// LoRA step staging: the weight side gets s * A rows j = jb .. jb + nrows - 1 (columns k0 ..),
// laid out like a decoded weight tile; the dY side gets U columns jb .. (rows m0 ..), chunks of 8
// columns 0 .. nch - 1; both zero-padded (the MFMAs of the step read no further). U chunks are
// one 16-byte buffer load each when r is a multiple of 8 and U is 16-byte aligned (rows past the
// tile edge and chunks past r read as zero), single values otherwise.
__device__ void stage_lora_dx(const GemmArgs &g, float sa, const uint16_t *A, int64_t m0, int64_t k0,
                              int64_t rows_m, int jb, int nrows, int nch, uint4 *sY, uint16_t *sW) {
  const int tid = threadIdx.x;
  {
    const int row = own_row(tid), seg = own_seg(tid);
    const int j = jb + row;
    if (row < nrows) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t k = k0 + seg * 32 + q * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (j < g.r && k < g.C) {
          const uint4 a = *reinterpret_cast<const uint4 *>(A + (int64_t)j * g.C + k);
          const uint32_t w[4] = {a.x, a.y, a.z, a.w};
          uint32_t o[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = pack_bf16x2(sa * bf16_lo(w[e]), sa * bf16_hi(w[e]));
          v = make_uint4(o[0], o[1], o[2], o[3]);
        }
        *reinterpret_cast<uint4 *>(sW + wunit(row, seg * 8 + 2 * q)) = v;
      }
    }
  }
  const int c = tid & 7, row0 = tid >> 3;
  if (c >= nch) return;
  const int j0 = jb + c * 8;
  if ((g.r & 7) == 0 && (reinterpret_cast<uintptr_t>(g.lora_a) & 15) == 0) {
    const __amdgpu_buffer_rsrc_t rU = make_rsrc(g.lora_a + m0 * g.r, rows_m * g.r * 2);
    u32x4 u[kYChunks / kThreads];
#pragma unroll
    for (int i = 0; i < kYChunks / kThreads; ++i) {
      const int row = row0 + 64 * i;
      const uint32_t off = j0 < g.r ? (uint32_t)(row * g.r + j0) * 2 : 0x80000000u;
      u[i] = __builtin_amdgcn_raw_buffer_load_b128(rU, off, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < kYChunks / kThreads; ++i)
      sY[swzd(row0 + 64 * i, c)] = make_uint4(u[i][0], u[i][1], u[i][2], u[i][3]);
    return;
  }
#pragma unroll 1
  for (int i = 0; i < kYChunks / kThreads; ++i) {
    const int row = row0 + 64 * i;
    const int64_t m = m0 + row;
    uint32_t wa[4];
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const int ja = j0 + e, jc = ja + 1;
      uint32_t lo = 0, hi = 0;
      if (row < rows_m) {
        if (ja < g.r) lo = g.lora_a[m * g.r + ja];
        if (jc < g.r) hi = g.lora_a[m * g.r + jc];
      }
      wa[e >> 1] = lo | (hi << 16);
    }
    sY[swzd(row, c)] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
  }
}

// kGrp: the grouped (mixture-of-experts) form. The weight holds E experts' [N, K] blocks stacked
// ([E N, K]), A their [r, K] blocks ([E r, K]); the rows of dY, U and dX are grouped by expert
// (rows m_off[e] .. m_off[e+1] - 1 belong to expert e), and expert e's tiles are the logical
// tiles tile_off[e] .. tile_off[e+1] - 1 of the launch.
// kFmt: 0 NF4 with float32 block constants, 1 NF4 double-quantised, 2 E2M1 with E4M3 group
// scales of 16 (a thread's 32 columns are two groups, each with its own whole table; the operand
// is exact in bf16) and a float32 tensor scale applied in the epilogue (the LoRA steps stage
// s / S times A).
// Origin (m0, k0) of tile `logical` of a group of rows m_lo .. m_hi: tiles in groups of kGroupM
// row blocks, consecutive logical tiles walking the row blocks of a group first.
__device__ __forceinline__ void dx_origin(int64_t m_lo, int64_t m_hi, int tiles_k, int logical, int64_t &m0,
                                          int64_t &k0) {
  const int tiles_m = (int)((m_hi - m_lo + kT - 1) / kT);
  const int gsz = kGroupM * tiles_k, grp0 = logical / gsz, gin = logical % gsz;
  const int gm = tiles_m - grp0 * kGroupM < kGroupM ? tiles_m - grp0 * kGroupM : kGroupM;
  m0 = m_lo + (int64_t)(grp0 * kGroupM + gin % gm) * kT;
  k0 = (int64_t)(gin / gm) * kT;
}

template <int kFmt, bool kGrp>
__device__ __forceinline__ void dx_body(const GemmArgs &g, const GroupArgs &gr) {
  constexpr bool kDQ = kFmt == 1, kFP4 = kFmt == 2;
  // separate LDS arrays per buffer: the compiler then knows that accesses to one do not alias
  // the DMA in flight into another (one array of two would make it wait for the DMA)
  __shared__ uint4 sY0[kYChunks], sY1[kYChunks];
  __shared__ uint4 sW0[kWElems / 8], sW1[kWElems / 8];
  __shared__ __attribute__((aligned(16))) float sLv[16];
  auto ybuf = [&](int P) { return P ? sY1 : sY0; };
  auto wbuf = [&](int P) { return reinterpret_cast<uint16_t *>(P ? sW1 : sW0); };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wk = wave & 3;
  const int g16 = lane >> 4, l16 = lane & 15;
  const int tiles_k = (int)((g.C + kT - 1) / kT);
  // Tiles in groups of kGroupM row blocks: consecutive logical tiles walk the row blocks of a group
  // first, so the 32 workgroups an XCD runs at once cover 4 row blocks x 8 column tiles and
  // share 4 dY row blocks and 8 weight column tiles in its L2 (one row block x 32 column tiles
  // re-fetched the whole weight from beyond L2 once per row block).
  int logical;
  int64_t m_lo = 0, m_hi = g.M, wbase = 0;
  const int nsteps = (int)((g.R + kS - 1) / kS);
  // Grouped launches may split the tiles of a last, partly filled round (dx_split): workgroup
  // full + tail_i * S + piece runs steps [sbeg, send) of tail tile tail_i and writes its float32
  // sums to gr.part; a second launch (dx_tail_kernel) adds the pieces.
  int piece = -1, tail_i = 0;
  DxSplit sp{0, 0, 1};
  if (kGrp) {
    // a grid sized by an upper bound (routing on the device) has workgroups past the last tile
    const int total = grp_tile_off(gr, gr.E);
    sp = dx_split(gr.width, gr.smax, gr.part != nullptr, total, nsteps);
    const int b = (int)blockIdx.x;
    if (b >= sp.full + sp.tail * sp.S) return;
    if (b < sp.full) {
      logical = tile_remap(b, sp.full);
    } else {
      tail_i = (b - sp.full) / sp.S;
      piece = (b - sp.full) - tail_i * sp.S;
      logical = sp.full + tail_i;
    }
    const int e = find_group(gr, logical);
    logical -= grp_tile_off(gr, e);
    m_lo = grp_m_off(gr, e);
    m_hi = grp_m_off(gr, e + 1);
    wbase = (int64_t)e * g.R;
  } else {
    logical = tile_remap(blockIdx.x, gridDim.x);
  }
  const int sbeg = piece < 0 ? 0 : piece * nsteps / sp.S;
  const int send = piece < 0 ? nsteps : (piece + 1) * nsteps / sp.S;
  int64_t m0, k0;
  dx_origin(m_lo, m_hi, tiles_k, logical, m0, k0);
  const int64_t K = g.w.k, N = g.R;   // N: the reduction length (one expert's rows of the weight)
  const int64_t rows_m = (m_hi - m0 < kT) ? m_hi - m0 : kT;
  const int kblk = (int)(K / kS);
  const int last = send - 1;

  // dY rows m0.. (reduction index n contiguous). Chunks past n = N read the next row's values
  // (finite) and meet weight rows past N, which decode to exact zeros (codes and constants read
  // past the end of the expert's part of their buffers are 0), so they add nothing. The run
  // scales of the double quantisation are indexed by the block's place in the whole tensor
  // (qb0 + block), since a run may straddle two experts.
  const int64_t qb0 = wbase * kblk;
  const __amdgpu_buffer_rsrc_t rC = make_rsrc(g.w.codes + wbase * (K / 2), N * (K / 2));
  const __amdgpu_buffer_rsrc_t rQ =
      kFP4  ? make_rsrc(reinterpret_cast<const uint8_t *>(g.w.absmax) + wbase * (K / 16), N * (K / 16))
      : kDQ ? make_rsrc(reinterpret_cast<const int8_t *>(g.w.absmax) + qb0, N * kblk)
            : make_rsrc(reinterpret_cast<const float *>(g.w.absmax) + qb0, N * kblk * 4);
  // E2M1: the tensor scale (1 for an all-zero weight, whose group scales are all 0), read where
  // it is used so that no register holds it through the main loop
  auto tscale = [&]() {
    const float S = *g.w.scale;
    return S > 0.f ? S : 1.f;
  };
  const int64_t nruns = (g.w.n * kblk + 255) / 256;
  const __amdgpu_buffer_rsrc_t rS = make_rsrc(g.w.scale, kDQ ? nruns * 4 : 0);
  const __amdgpu_buffer_rsrc_t rY = make_rsrc(g.a_side + m0 * N, rows_m * N * 2);

  // dY DMA: instruction i of wave w fills the 1 KB of the tile holding rows 8 (4 w + i) .. +7;
  // lane L writes physical chunk L % 8 of row 8 (4 w + i) + L / 8, i.e. logical chunk
  // (L % 8) ^ ((row >> 1) & 7) (the same swizzle as swzd).
  uint32_t yoff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = 8 * (4 * wave + i) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    yoff[i] = (uint32_t)(row * N * 2 + c * 16);
  }
  // Decode ownership: weight row n = 64 s + wr of step s, columns k0 + 32 seg .. + 31.
  const int wr = own_row(tid), seg = own_seg(tid);
  // In the pipelined steps the two threads of a 64-column block (segments 2b and 2b + 1, lanes l
  // and l ^ 8) split its table: the thread with segment parity h builds entries 8 h .. 8 h + 7
  // (levels lvh) and takes the other half from the partner lane; the select masks of the decode
  // are complemented for h = 1, whose own half is the upper one.
  // The levels are read from LDS four at a time when the table is built (eight per-lane
  // registers held across the loop would not fit beside the accumulators).
  const int sh = kFP4 ? 0 : (seg & 1);
  const uint32_t mhi = sh ? 0u : 0xFFFFFFFFu, mlo = sh ? 0xFFFFFFFFu : 0u;
  if (tid < 16) sLv[tid] = g.t.level[tid];
  const f32x4 *lvq = reinterpret_cast<const f32x4 *>(sLv) + 2 * sh;
  const int64_t kcol = k0 + seg * 32;
  const bool kvalid = kcol < K;
  const uint32_t coff = (uint32_t)(wr * (K / 2) + (kvalid ? kcol / 2 : 0));
  const uint32_t cstep = (uint32_t)(kS * (K / 2));
  // E2M1: the two group scales of the thread's 32 columns, bytes kcol / 16 and + 1 of its row
  const uint32_t qoff = kFP4 ? (uint32_t)(wr * (K / 16) + (kvalid ? kcol / 16 : 0))
                             : (uint32_t)(wr * kblk + (kvalid ? kcol / 64 : 0));
  const uint32_t qstep = kFP4 ? (uint32_t)(kS * (K / 16)) : (uint32_t)(kS * kblk);

  f32x4 acc[4][8];   // [k-tile][m-tile]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto dma_y = [&](int s, uint4 *sA) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rY, (__attribute__((address_space(3))) void *)(sA + (4 * wave + i) * 64), 16, yoff[i],
          s * 128, 0, 0);
  };
  constexpr int kCodeLoads = kDQ ? 3 : 2;   // loads issued by load_c
  auto load_c = [&](int s, CStage &c) {
    c.c = __builtin_amdgcn_raw_buffer_load_b128(rC, coff + s * cstep, 0, 0);
    const uint32_t b = qoff + s * qstep;
    if (kFP4) {
      c.q = __builtin_amdgcn_raw_buffer_load_b16(rQ, b, 0, 0);
    } else if (kDQ) {
      c.q = __builtin_amdgcn_raw_buffer_load_b8(rQ, b, 0, 0);
      c.sc = __builtin_amdgcn_raw_buffer_load_b32(rS, (uint32_t)((qb0 + b) >> 8) * 4, 0, 0);
    } else {
      c.q = __builtin_amdgcn_raw_buffer_load_b32(rQ, b * 4, 0, 0);
    }
  };
  auto absmax_of = [&](const CStage &c) {
    const float a = kDQ ? int8_code(c.q) * __uint_as_float(c.sc) : __uint_as_float(c.q);
    return kvalid ? a : 0.f;
  };
  auto word = [](const CStage &c, int j) {
    return j == 0 ? c.c.x : j == 1 ? c.c.y : j == 2 ? c.c.z : c.c.w;
  };
  // columns 32 seg + 8 j .. +7 of the thread's weight row = 8-byte units 8 seg + 2 j, +1
  auto wstore = [&](uint16_t *sW, int j, const uint32_t o[4]) {
    *reinterpret_cast<uint4 *>(sW + wunit(wr, seg * 8 + 2 * j)) = make_uint4(o[0], o[1], o[2], o[3]);
  };
  // E2M1 table of the thread's group h (0, 1); zero past K
  auto fp4_table = [&](const CStage &c, int h) {
    return make_e2m1_table(kvalid ? e4m3_to_f32((c.q >> (8 * h)) & 0xFFu) : 0.f);
  };
  auto decode_all = [&](const CStage &c, uint16_t *sW) {
    RowTable t = kFP4 ? fp4_table(c, 0) : make_row_table(absmax_of(c), g.t);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t o[4];
      if (kFP4 && j == 2) t = fp4_table(c, 1);
      if (kFP4) decode8_e2m1(t, word(c, j), o); else decode8(t, word(c, j), o);
      wstore(sW, j, o);
    }
  };
  // MFMA operands of k-slice ks (32 rows n): the weight side, transposed on the fly -- lane
  // (g16, l16) gets rows 32 ks + 8 g16 .. + 7 of column wk*64 + 16 kt + l16 -- and the dY side,
  // row wm*128 + 16 mt + l16, reduction elements 32 ks + 8 g16 .. + 7.
  auto wfrag = [&](const uint16_t *sW, int ks, int kt) {
    const int row = ks * 32 + g16 * 8 + (l16 >> 2);
    const int u = (wk * 64 + kt * 16) / 4 + (l16 & 3);
    const s16x4 lo = lds_tr16(sW + wunit(row, u));
    const s16x4 hi = lds_tr16(sW + wunit(row + 4, u));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };
  auto yfrag = [&](const uint4 *sA, int ks, int mt) {
    return __builtin_bit_cast(bf16x8, sA[swzd(wm * 128 + mt * 16 + l16, ks * 4 + g16)]);
  };
  // Plain MFMA pass over k-slice ks of one step (used for the LoRA steps).
  auto mma = [&](const uint4 *sA, const uint16_t *sW, int ks) {
    bf16x8 aw[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) aw[kt] = wfrag(sW, ks, kt);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      const bf16x8 b = yfrag(sA, ks, mt);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc[kt][mt] = mfma16x16x32(aw[kt], b, acc[kt][mt]);
    }
  };

  // One step: MFMAs on buffer P; the dY tile of step s+1 arrives in buffer P^1 by DMA and the
  // weight rows of step s+1 (decoded from cn) are written there in between; codes of step s+2
  // go to cm. 16 groups (k-slice, m-tile) of 4 MFMAs; decode pieces go between groups.
  auto body = [&](int s, int P, CStage &cm, CStage &cn) {
    const int s1 = s + 1 < last ? s + 1 : last;
    const int s2 = s + 2 < last ? s + 2 : last;
    dma_y(s1, ybuf(P ^ 1));
    __builtin_amdgcn_sched_barrier(0);   // the DMA stays ahead of the code loads (see the wait)
    load_c(s2, cm);
    const uint4 *Y = ybuf(P);
    const uint16_t *W = wbuf(P);
    uint16_t *Wn = wbuf(P ^ 1);
    bf16x8 aw[4], yb[2];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) aw[kt] = wfrag(W, 0, kt);
    yb[0] = yfrag(Y, 0, 0);

    const float a = absmax_of(cn);
    RowTable t;
    Dec8 dx;
#pragma unroll
    for (int grp = 0; grp < 16; ++grp) {
      const int ks = grp >> 3, mt = grp & 7;
      // the second k-slice's weight fragments replace the first's (one exposed LDS latency per
      // step, which keeps the wave within 256 registers); the next m-tile's dY fragment is read
      // one group ahead
      if (grp == 8) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) aw[kt] = wfrag(W, 1, kt);
      }
      if (grp + 1 < 16) yb[(grp + 1) & 1] = yfrag(Y, (grp + 1) >> 3, (grp + 1) & 7);
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) acc[kt][mt] = mfma16x16x32(aw[kt], yb[grp & 1], acc[kt][mt]);
      // decode of step s+1: table in groups 0..3, then word j = (grp - 4) / 3 in pieces over
      // three groups (pieces 0-1, 2-3, 4 + store)
      if (kFP4 && grp < 4) {
        if (grp == 0) t = fp4_table(cn, 0);       // the whole table of the first group
      } else if (grp < 4) {
        // this thread's half of the table in L[0..1], H[0..1] (groups 0, 1); the partner lane's
        // half by DPP (groups 1, 2)
        if (grp < 2) {
          const f32x4 lv = lvq[grp];
          const uint32_t p0 = pack_bf16x2(lv[0] * a, lv[1] * a);
          const uint32_t p1 = pack_bf16x2(lv[2] * a, lv[3] * a);
          t.L[grp] = perm(p1, p0, 0x06040200u);
          t.H[grp] = perm(p1, p0, 0x07050301u);
        }
        if (grp == 1 || grp == 2) {
          t.L[grp + 1] = swap_lane_octets(t.L[grp - 1]);
          t.H[grp + 1] = swap_lane_octets(t.H[grp - 1]);
        }
      } else {
        const int j = (grp - 4) / 3, ph = (grp - 4) % 3;
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
          wstore(Wn, j, o);
          if (kFP4 && j == 1) t = fp4_table(cn, 1);   // words 2, 3: the second group
        }
      }
      // keep each group's loads and decode work in place (hoisting them stretches register
      // lifetimes past the 256 a wave may use with two waves per SIMD)
      __builtin_amdgcn_sched_barrier(0);
    }
    // the dY DMA of step s+1 (older than the code loads of step s+2) has landed and this wave's
    // LDS stores are done; the barrier publishes buffer P^1
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(kCodeLoads) : "memory");
  };

  CStage c0, c1;
  dma_y(sbeg, ybuf(0));
  load_c(sbeg, c0);
  load_c(send - sbeg > 1 ? sbeg + 1 : sbeg, c1);
  decode_all(c0, wbuf(0));
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  int s = sbeg;
#pragma unroll 1
  for (; s + 2 <= send; s += 2) {
    body(s, 0, c0, c1);
    body(s + 1, 1, c1, c0);
  }
  if (s < send) body(s, 0, c0, c1);
  __syncthreads();

  // LoRA steps (a split tile's last piece only); a k-slice of 32 rows j that lies wholly past r
  // is skipped.
  const int nlora = piece < sp.S - 1 && piece >= 0 ? 0 : (g.r + kS - 1) / kS;
  const uint16_t *Ae = g.lora_b + (kGrp ? (wbase / g.R) * g.r * K : 0);   // the expert's A
#pragma unroll 1
  for (int j = 0; j < nlora; ++j) {
    const int buf = j & 1;
    const int nks = g.r - j * kS > kS / 2 ? 2 : 1;
    stage_lora_dx(g, kFP4 ? g.s / tscale() : g.s, Ae, m0, k0, rows_m, j * kS, 32 * nks, 4 * nks, ybuf(buf),
                  wbuf(buf));
    __syncthreads();
    mma(ybuf(buf), wbuf(buf), 0);
    if (nks > 1) mma(ybuf(buf), wbuf(buf), 1);
    __syncthreads();
  }

  // A piece of a split tile: its float32 sums, [wave][k-tile * 8 + m-tile][lane] as f32x4, for
  // dx_tail_kernel to add.
  if (kGrp && piece >= 0) {
    f32x4 *pp = reinterpret_cast<f32x4 *>(gr.part + ((int64_t)tail_i * sp.S + piece) * kDxPieceFloats) +
                wave * 32 * 64 + lane;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) pp[(kt * 8 + mt) * 64] = acc[kt][mt];
    return;
  }

  // Epilogue. With the weight as the MFMA A operand, a lane holds columns k..k+3 of row m. Each
  // wave packs its 128 x 64 block to bf16 in 16 KB of the (now idle) LDS and writes it out as whole
  // 128-byte row pieces, 16 bytes per lane, with non-temporal stores (dX is not read again by this
  // kernel, and streaming it out measured faster than write-back cached stores). Rows of dX are
  // 16-byte aligned and the column count is a multiple of 8 (checked at launch).
  {
    uint4 *blk = (wave >> 1) == 0 ? sY0 : (wave >> 1) == 1 ? sY1 : (wave >> 1) == 2 ? sW0 : sW1;
    blk += (wave & 1) * (kYChunks / 2);
    uint2 *b2 = reinterpret_cast<uint2 *>(blk);
    const float tsc = kFP4 ? tscale() : 1.f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
        b2[swzd(mt * 16 + l16, 2 * kt + (g16 >> 1)) * 2 + (g16 & 1)] =
            kFP4 ? make_uint2(pack_bf16x2(tsc * acc[kt][mt][0], tsc * acc[kt][mt][1]),
                              pack_bf16x2(tsc * acc[kt][mt][2], tsc * acc[kt][mt][3]))
                 : make_uint2(pack_bf16x2(acc[kt][mt][0], acc[kt][mt][1]),
                              pack_bf16x2(acc[kt][mt][2], acc[kt][mt][3]));
    __syncthreads();
    const int c = lane & 7;
    const int64_t k = k0 + wk * 64 + c * 8;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = 8 * i + (lane >> 3);
      const int64_t m = m0 + wm * 128 + row;
      const uint4 v = blk[swzd(row, c)];
      if (m < m_hi && k < g.C)
        __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w},
                                    reinterpret_cast<u32x4 *>(g.out + m * g.ldo + k));
    }
  }
}

template <int kFmt>
__global__ __launch_bounds__(kThreads) void dx_fused_kernel(GemmArgs g) {
  dx_body<kFmt, false>(g, GroupArgs{});
}
template <int kFmt>
__global__ __launch_bounds__(kThreads) void dx_grouped_kernel(GemmArgs g, GroupArgs gr) {
  dx_body<kFmt, true>(g, gr);
}

// The split tiles of a grouped dX launch: workgroups 4 i .. 4 i + 3 add the S float32 pieces of
// tail tile i in piece order (a fixed order: the result does not depend on which piece finished
// first), each a quarter of the tile (8 of the 32 accumulator blocks of every wave), scale E2M1
// sums by the tensor scale, round to bf16 and write the tile. Workgroups past the tail (a grid
// sized by an upper bound) exit at once.
template <int kFmt>
__global__ __launch_bounds__(kThreads) void dx_tail_kernel(GemmArgs g, GroupArgs gr) {
  const int nsteps = (int)((g.R + kS - 1) / kS);
  const int total = grp_tile_off(gr, gr.E);
  const DxSplit sp = dx_split(gr.width, gr.smax, gr.part != nullptr, total, nsteps);
  const int i = (int)blockIdx.x >> 2, quarter = (int)blockIdx.x & 3;
  if (i >= sp.tail) return;
  int logical = sp.full + i;
  const int e = find_group(gr, logical);
  logical -= grp_tile_off(gr, e);
  const int64_t m_lo = grp_m_off(gr, e), m_hi = grp_m_off(gr, e + 1);
  const int tiles_k = (int)((g.C + kT - 1) / kT);
  int64_t m0, k0;
  dx_origin(m_lo, m_hi, tiles_k, logical, m0, k0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wk = wave & 3, g16 = lane >> 4, l16 = lane & 15;
  float tsc = 1.f;
  if (kFmt == 2) {
    const float S = *g.w.scale;
    tsc = S > 0.f ? S : 1.f;
  }
  const f32x4 *pp = reinterpret_cast<const f32x4 *>(gr.part + (int64_t)i * sp.S * kDxPieceFloats) +
                    wave * 32 * 64 + lane;
  constexpr int kPiece = kDxPieceFloats / 4;   // f32x4 per piece
#pragma unroll 4
  for (int q = 8 * quarter; q < 8 * quarter + 8; ++q) {   // q = k-tile * 8 + m-tile
    f32x4 a = pp[q * 64];
    for (int p = 1; p < sp.S; ++p) a += pp[p * kPiece + q * 64];
    const int kt = q >> 3, mt = q & 7;
    const int64_t m = m0 + wm * 128 + mt * 16 + l16;
    const int64_t k = k0 + wk * 64 + kt * 16 + 4 * g16;
    if (m < m_hi && k < g.C)
      *reinterpret_cast<uint2 *>(g.out + m * g.ldo + k) =
          make_uint2(pack_bf16x2(tsc * a[0], tsc * a[1]), pack_bf16x2(tsc * a[2], tsc * a[3]));
  }
}

}  // namespace

hipError_t launch_gemm_dx_grouped(const GemmArgs &g, const GroupArgs &gr, hipStream_t st) {
  if (((g.C | g.ldo) & 7) != 0 || (reinterpret_cast<uintptr_t>(g.out) & 15) != 0 || gr.E < 1 ||
      gr.E > kMaxExperts || g.w.n != (int64_t)gr.E * g.R || gr.width < 0 || gr.width > kDxMaxWidth ||
      gr.smax < 1)
    return hipErrorInvalidValue;
  const int nsteps = (int)((g.R + kS - 1) / kS);
  const bool split = gr.width > 0 && gr.part != nullptr;
  int64_t grid = gr.grid, tail_grid = 0;
  if (split) {
    if (gr.dtile_off) {   // device routing: upper bounds (the split adds fewer than width pieces)
      grid += gr.width;
      tail_grid = gr.width;
    } else {
      const DxSplit d = dx_split(gr.width, gr.smax, true, gr.tile_off[gr.E], nsteps);
      grid = d.full + (int64_t)d.tail * d.S;
      tail_grid = d.tail;
    }
  }
  if (grid < 1) return hipSuccess;
  if (g.w.fp4)
    dx_grouped_kernel<2><<<dim3((unsigned)grid), dim3(kThreads), 0, st>>>(g, gr);
  else if (g.w.dq)
    dx_grouped_kernel<1><<<dim3((unsigned)grid), dim3(kThreads), 0, st>>>(g, gr);
  else
    dx_grouped_kernel<0><<<dim3((unsigned)grid), dim3(kThreads), 0, st>>>(g, gr);
  if (tail_grid > 0) {
    tail_grid *= 4;   // four workgroups per tile
    if (g.w.fp4)
      dx_tail_kernel<2><<<dim3((unsigned)tail_grid), dim3(kThreads), 0, st>>>(g, gr);
    else if (g.w.dq)
      dx_tail_kernel<1><<<dim3((unsigned)tail_grid), dim3(kThreads), 0, st>>>(g, gr);
    else
      dx_tail_kernel<0><<<dim3((unsigned)tail_grid), dim3(kThreads), 0, st>>>(g, gr);
  }
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmArgs &g, hipStream_t st) {
  if (((g.C | g.ldo) & 7) != 0 || (reinterpret_cast<uintptr_t>(g.out) & 15) != 0 || g.R != g.w.n)
    return hipErrorInvalidValue;   // the epilogue writes 16-byte pieces of 8 columns
  const int64_t tiles = ((g.C + kT - 1) / kT) * ((g.M + kT - 1) / kT);
  if (g.w.fp4)
    dx_fused_kernel<2><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else if (g.w.dq)
    dx_fused_kernel<1><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  else
    dx_fused_kernel<0><<<dim3((unsigned)tiles), dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

}  // namespace nf4q

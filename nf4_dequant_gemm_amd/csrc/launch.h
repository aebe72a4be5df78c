// Internal launch wrappers of the NF4 QLoRA kernels (host-callable, not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace nf4q {

hipError_t launch_quantize(const void *w, bool f32_in, uint8_t *codes, void *absmax, float *scale,
                           int64_t nblk, int dq, const Tables &t, hipStream_t st);
hipError_t launch_dequantize(const WDesc &w, void *out, bool f32_out, const Tables &t,
                             hipStream_t st);
// The E2M1 variant (fp4.hip): codes, E4M3 group scales (one per 16 elements) and the float32
// tensor scale of nelem values; nelem % 16 == 0.
hipError_t launch_fp4_quantize(const void *w, bool f32_in, int64_t nelem, uint8_t *codes,
                               uint8_t *scales, float *tscale, hipStream_t st);
hipError_t launch_fp4_dequantize(const WDesc &w, void *out, bool f32_out, hipStream_t st);

// out[m][c] = bf16( sum_red a_side[m][red] * deq-side[c][red] + sum_j lora_a[m][j] * s*lora_b(c, j) )
//   fwd: a_side = X [M,K], weight rows c = n (reduction over k), lora_a = T [M,r], lora_b = B [N,r]
//   dx:  a_side = dY [M,N], weight columns c = k (reduction over n), lora_a = U [M,r], lora_b = A [r,K]
struct GemmArgs {
  const uint16_t *a_side;
  int64_t lda;
  const uint16_t *lora_a;   // [M, r] or NULL when r == 0
  const uint16_t *lora_b;   // fwd: B [N, r]; dx: A [r, K]
  WDesc w;
  int64_t M;                // rows of out
  int64_t C;                // columns of out (N for fwd, K for dx)
  int64_t R;                // reduction length (K for fwd, N for dx)
  int r;
  float s;
  uint16_t *out;
  int64_t ldo;
  Tables t;
  uint16_t *hout = nullptr;   // gate/up pair only: H [M, C], row stride ldh
  int64_t ldh = 0;
  const uint16_t *lora_b2 = nullptr;   // gate/up pair only: Bu [C, r / 2] (lora_b is Bg [C, r / 2])
};

hipError_t launch_gemm_fwd(const GemmArgs &g, hipStream_t st);
// The gate/up pair with the SwiGLU epilogue: g.w the stacked [Wg; Wu] [2C, K], g.lora_a T
// [M, r] (r = 2 r': [X Ag^T | X Au^T]), g.lora_b Bg and g.lora_b2 Bu [C, r'] each (the up
// projection is the block-diagonal [[Bg, 0], [0, Bu]], applied without storing it), g.out Ygu
// [M, 2C] (row stride ldo), g.hout H = silu(Yg) * Yu [M, C] (row stride ldh) from the float32
// sums of Yg and Yu.
hipError_t launch_gemm_fwd_pair(const GemmArgs &g, hipStream_t st);

// Grouped (mixture-of-experts) forward: E experts, rows m_off[e] .. m_off[e+1] of X, T and Y
// belong to expert e, whose weight rows are e N .. e N + N - 1 of the stacked weight g.w and whose
// B rows are the same rows of g.lora_b (N = g.C). tile_off[e] = sum over e' < e of
// ceil(rows_e' / 256) * ceil(N / 256): one launch runs every expert's tiles.
// The table is either held in the arguments (routing known on the host) or, with dm_off set, in
// device memory (routing computed on the device: launch_moe_plan writes it, and the launch's
// grid is an upper bound; workgroups past tile_off[E] exit at once).
constexpr int kMaxExperts = 256;
struct GroupArgs {
  int E;
  int64_t grid;                 // workgroups of the launch (x): tile_off[E] or an upper bound
  const int64_t *dm_off;        // device table [E + 1], or NULL: m_off below
  const int32_t *dtile_off;     // device table [E + 1], or NULL: tile_off below
  int64_t m_off[kMaxExperts + 1];
  int32_t tile_off[kMaxExperts + 1];
  // Grouped dX only: the tiles of a last, partly filled round of `width` workgroups (one per CU)
  // are split along the reduction into up to `smax` pieces that write float32 partial sums to
  // `part`; a second launch adds them (dx_split below). width 0 or part NULL: no split.
  int width = 0, smax = 1;
  float *part = nullptr;
};

// The split of a grouped dX launch of `total` tiles with `nsteps` reduction steps per tile: the
// first `full` tiles run whole (whole rounds of `width` workgroups); each of the `tail` others
// becomes S pieces of consecutive steps (S >= 2, S <= smax, S * tail <= width, S <= nsteps), or
// none is split (tail 0, S 1). The workgroups of a launch: full + tail * S. Only a tail behind
// at least one full round is split: a launch of at most one round keeps whole tiles, as the
// plain dX launch does (a grouped launch with one expert then equals it bit for bit).
struct DxSplit {
  int full, tail, S;
};
__host__ __device__ inline DxSplit dx_split(int width, int smax, bool enabled, int total, int nsteps) {
  DxSplit d{total, 0, 1};
  if (!enabled || width <= 0 || total <= width) return d;
  const int tail = total % width;
  if (tail == 0) return d;
  int S = width / tail;
  S = S < smax ? S : smax;
  S = S < nsteps ? S : nsteps;
  if (S >= 2) {
    d.full = total - tail;
    d.tail = tail;
    d.S = S;
  }
  return d;
}
// Float32 values of one piece (a 256 x 256 tile); a split launch writes at most width pieces,
// and width is at most kDxMaxWidth (the workspace is sized for that).
constexpr int64_t kDxPieceFloats = 256 * 256;
constexpr int kDxMaxWidth = 256;
constexpr int kDxMaxPieces = 8;
// Table entries, for a group index the same in every lane (kept in scalar registers: values
// derived from it address every tile load).
__device__ __forceinline__ int64_t grp_m_off(const GroupArgs &g, int e) {
  const int64_t v = g.dm_off ? g.dm_off[e] : g.m_off[e];
  const uint64_t u = (uint64_t)v;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)u);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(u >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ int grp_tile_off(const GroupArgs &g, int e) {
  return __builtin_amdgcn_readfirstlane(g.dtile_off ? g.dtile_off[e] : g.tile_off[e]);
}
// The group holding logical tile `local` (tile_off[e] <= local < tile_off[e + 1]; empty groups
// hold none): every thread tests some groups, the match goes through LDS. Call with the whole
// workgroup; `local` is the same in every lane, and so is the result.
__device__ __forceinline__ int find_group(const GroupArgs &g, int local) {
  __shared__ int s_group;
  for (int t = threadIdx.x; t < g.E; t += blockDim.x) {
    const int lo = g.dtile_off ? g.dtile_off[t] : g.tile_off[t];
    const int hi = g.dtile_off ? g.dtile_off[t + 1] : g.tile_off[t + 1];
    if (local >= lo && local < hi) s_group = t;
  }
  __syncthreads();
  return __builtin_amdgcn_readfirstlane(s_group);
}

// Device group tables of a grouped layer from expert row counts held in device memory (int64
// [E]): m_off int64 [E + 1], then int32 [E + 1] first-tile tables for 256-row tiles times tiles_n
// (forward) and times tiles_k (dX) column tiles, and for 64-row blocks. Negative counts count as
// 0 and the row offsets are clipped at m, so no row past m is ever read or written. One
// workgroup; the table takes moe_table_bytes(E) bytes.
size_t moe_table_bytes(int E);
hipError_t launch_moe_plan(const int64_t *dcounts, int E, int64_t m, int64_t tiles_n,
                           int64_t tiles_k, void *table, hipStream_t st);
__host__ __device__ inline int64_t *moe_table_m_off(void *t) { return reinterpret_cast<int64_t *>(t); }
__host__ __device__ inline int32_t *moe_table_tiles(void *t, int E, int which) {   // 0 forward, 1 dX, 2 64-row blocks
  return reinterpret_cast<int32_t *>(reinterpret_cast<char *>(t) + 8 * (E + 1)) + which * (E + 1);
}
hipError_t launch_gemm_fwd_grouped(const GemmArgs &g, const GroupArgs &gr, hipStream_t st);
// Forward for M <= 48 and K % 256 == 0 (weight-stream bound): codes streamed by LDS DMA, table
// decode of unscaled levels, block constant applied to the per-block partial sums.
hipError_t launch_decode_fwd(const GemmArgs &g, hipStream_t st);
constexpr int64_t kDecodeMaxM = 48;
// Forward for M <= 16, double-quantised W and K % 256 == 0: codes, X and block constants all
// staged by LDS DMA in whole lines, 112 weight rows per workgroup.
hipError_t launch_decode16_fwd(const GemmArgs &g, hipStream_t st);
// The same with T = X A^T given as split partials (float [M][r][tsplits], see launch_rowproj):
// every workgroup adds them in split order for its LoRA term and workgroup 0 writes T (bf16) to
// tout. Requires r % 8 == 0.
hipError_t launch_decode16_fwd_tpart(const GemmArgs &g, const float *tpart, int tsplits,
                                     uint16_t *tout, hipStream_t st);
// The same with T = X A^T formed inside the launch from A bf16 [r, K] (g.lora_a unused): every
// workgroup sums T for its own LoRA term and workgroup 0 writes T (bf16 [M][r]) to tout.
// Requires r % 8 == 0 and 8 <= r <= kDecode16MaxTinRank (double-quantised NF4) or
// kDecode16MaxTinRankE2M1 (E2M1).
hipError_t launch_decode16_fwd_tin(const GemmArgs &g, const uint16_t *A, uint16_t *tout, hipStream_t st);
constexpr int kDecode16MaxTinRank = 64;
constexpr int kDecode16MaxTinRankE2M1 = 16;
hipError_t launch_gemm_dx(const GemmArgs &g, hipStream_t st);
// dX of every expert in one launch: g.R = N (one expert's rows of the stacked weight, the
// reduction), g.w.n = E N, g.lora_b = the stacked A [E r, K]; rows of dY, U, dX grouped by
// expert as gr.m_off says; gr.tile_off[e] = sum over e' < e of ceil(rows_e' / 256) * ceil(K / 256).
// With gr.width (the workgroups that run at once, <= kDxMaxWidth) and gr.part (kDxMaxWidth *
// kDxPieceFloats float32) set, the tiles of a last, partly filled round are split along the
// reduction (dx_split) and a second, small launch adds the pieces.
hipError_t launch_gemm_dx_grouped(const GemmArgs &g, const GroupArgs &gr, hipStream_t st);

// out[m][j] = sum_l in[m][l] * p[j][l] for j < r (p row-major [r][L], leading dim ldp).
// With splits > 1 the partial sums go to part and are added in split order: by a second launch
// into out, from split-major partials (float [splits][M][r]); or, with out == NULL, by their
// consumer, from partials with the splits of one output contiguous (float [M][r][splits]).
hipError_t launch_rowproj(const uint16_t *in, int64_t ldin, const uint16_t *p, int64_t ldp,
                          int64_t M, int64_t L, int r, int splits, float *part, uint16_t *out,
                          hipStream_t st);
int rowproj_splits(int64_t M, int64_t L);

// out = bf16(s * sum over m of P[m][j] * Q[m][c]); P [M][r] (ld r), Q [M][C] (ld ldq).
// transposed_out: out[c][j] (ld r) else out[j][c] (ld C). part: float [splits][r][C].
hipError_t launch_mreduce(const uint16_t *P, const uint16_t *Q, int64_t ldq, int64_t M, int64_t C,
                          int r, float s, int splits, float *part, uint16_t *out,
                          bool transposed_out, hipStream_t st);
int mreduce_splits(int64_t M, int64_t C, int r, int E = 1);

// dst[j][l] = src[l][j] for a bf16 [L][r] matrix.
hipError_t launch_transpose(const uint16_t *src, int64_t L, int r, uint16_t *dst, hipStream_t st);
// Grouped forms (rows grouped by expert as gr.m_off says). Row projection: expert e's p is
// p + e * pstride, gr.tile_off[e] = its first 64-row block, partials need splits * M * r floats.
// M-reduction: one [r][C] sum per expert over its own rows, written at out + e r C (transposed:
// [C][r] there); partials need E * splits * r * C floats.
hipError_t launch_rowproj_grouped(const uint16_t *in, int64_t ldin, const uint16_t *p, int64_t pstride,
                                  int64_t ldp, int64_t M, int64_t L, int r, int splits, float *part,
                                  uint16_t *out, const GroupArgs &gr, hipStream_t st);
hipError_t launch_mreduce_grouped(const uint16_t *P, const uint16_t *Q, int64_t ldq, int64_t C, int r,
                                  float s, int splits, float *part, uint16_t *out,
                                  bool transposed_out, const GroupArgs &gr, hipStream_t st);

// Gate/up SwiGLU pair (swiglu.hip). ygu / dygu rows: the gate block then the up block, 2n columns.
hipError_t launch_swiglu_fwd(const uint16_t *ygu, int64_t m, int64_t n, uint16_t *h, hipStream_t st);
hipError_t launch_swiglu_bwd(const uint16_t *dh, const uint16_t *ygu, int64_t m, int64_t n,
                             uint16_t *dygu, hipStream_t st);
hipError_t launch_blockdiag(const uint16_t *bg, const uint16_t *bu, int64_t n, int r, uint16_t *b2,
                            hipStream_t st);
hipError_t launch_diagblocks(const uint16_t *db2, int64_t n, int r, uint16_t *dbg, uint16_t *dbu,
                             hipStream_t st);

// LoRA merge (merge.hip): out bf16 [n, k] = bf16(deq(W) + s B A), 0 <= r <= 128, k % 64 == 0.
hipError_t launch_merge(const WDesc &w, const uint16_t *A, const uint16_t *B, int r, float s,
                        const Tables &t, uint16_t *out, hipStream_t st);

}  // namespace nf4q

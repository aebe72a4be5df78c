// Rank-r LoRA kernels of the QLoRA layer (gfx950, bf16 MFMA).
//
// The pages give the adapter algebra (Delta W = B A at rank r, only A and B are trained)
// [Unsloth v0.1.463-beta release article, "About the Unsloth Project"]. Besides the fused GEMM,
// the layer needs three thin products whose cost is reading one [M, L] activation once:
//   rowproj : T = X A^T (forward) and U = dY B (backward), out [M, r]
//   mreduce : dA = s U^T X and dB = s dY^T T, sums over the M rows
// Sums over M are split across workgroups into float32 partials and reduced in a fixed order,
// so the results are deterministic (no atomics).
#include "common.h"
#include "launch.h"

namespace nf4q {


// ------------------------------------------------------------------------------------ rowproj
// out[m][j] = sum over l of in[m][l] * p[j][l]  (T: in = X, p = A;  U: in = dY, p = B^T).
// Workgroup: 64 rows of `in` (one 16-row MFMA 16x16x32 tile per wave) x all r (<= 128) columns,
// over one split of the reduction in steps of 64. Each step's in-tile (64 rows x 128 bytes) and
// p-tile (r rows x 128 bytes) are loaded with fully coalesced 16-byte loads (8 lanes per
// 128-byte row), two steps ahead, and staged in LDS (rows of 8 chunks, chunk c of row i at slot
// c ^ ((i >> 1) & 7)), from where the fragments are read.
__device__ __forceinline__ int swzr(int row, int c) { return row * 8 + (c ^ ((row >> 1) & 7)); }

// kGrp: rows grouped by expert (rows gr.m_off[e] .. gr.m_off[e+1] - 1 of `in` and `out` belong
// to expert e, whose p is p + e * pstride); the launch's 64-row blocks are every expert's blocks
// in turn (expert e's first block is gr.tile_off[e]). The partial-sum layout is over all M rows.
template <int TN, bool kGrp>
__device__ __forceinline__ void rowproj_body(const uint16_t *__restrict__ in, int64_t ldin,
                                             const uint16_t *__restrict__ p, int64_t ldp, int64_t M,
                                             int64_t L, int r, int64_t lsplit,
                                             float *__restrict__ part, int smajor,
                                             uint16_t *__restrict__ out, const GroupArgs &gr,
                                             int64_t pstride) {
  constexpr int PCH = TN * 16 * 8;                 // p-tile chunks per step
  constexpr int PPT = (PCH + 255) / 256;           // p-tile chunks per thread
  __shared__ uint4 sI[2][64 * 8];
  __shared__ uint4 sP[2][TN * 16 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t mbase = (int64_t)blockIdx.x * 64, mhi = M;
  if (kGrp) {
    // a grid sized by an upper bound (routing on the device) has blocks past the last one
    if ((int)blockIdx.x >= grp_tile_off(gr, gr.E)) return;
    const int e = find_group(gr, (int)blockIdx.x);
    mbase = grp_m_off(gr, e) + (int64_t)((int)blockIdx.x - grp_tile_off(gr, e)) * 64;
    mhi = grp_m_off(gr, e + 1);
    p += e * pstride;
  }
  const int split = blockIdx.y;
  const int64_t lb = split * lsplit;
  const int64_t le = (lb + lsplit < L) ? lb + lsplit : L;

  f32x4 acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    uint4 x[2];
    uint4 q[PPT];
  };
  auto load = [&](int64_t l0, Stage &st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qd = tid + 256 * i;
      const int row = qd >> 3, c = qd & 7;
      const int64_t m = mbase + row, l = l0 + c * 8;
      st.x[i] = (m < mhi && l < le) ? *reinterpret_cast<const uint4 *>(in + m * ldin + l) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int qd = tid + 256 * i;
      const int j = qd >> 3, c = qd & 7;
      const int64_t l = l0 + c * 8;
      st.q[i] = (qd < PCH && j < r && l < le) ? *reinterpret_cast<const uint4 *>(p + (int64_t)j * ldp + l)
                                              : make_uint4(0, 0, 0, 0);
    }
  };
  auto store = [&](const Stage &st, int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int qd = tid + 256 * i;
      sI[buf][swzr(qd >> 3, qd & 7)] = st.x[i];
    }
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
      const int qd = tid + 256 * i;
      if (qd < PCH) sP[buf][swzr(qd >> 3, qd & 7)] = st.q[i];
    }
  };
  auto mma = [&](int buf) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int c = kk * 4 + (lane >> 4);
      const bf16x8 a = __builtin_bit_cast(bf16x8, sI[buf][swzr(wave * 16 + (lane & 15), c)]);
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const bf16x8 b = __builtin_bit_cast(bf16x8, sP[buf][swzr(t * 16 + (lane & 15), c)]);
        acc[t] = mfma16x16x32(a, b, acc[t]);
      }
    }
  };

  Stage s0, s1;
  const int64_t nst = (le - lb + 63) / 64;
  if (nst > 0) load(lb, s0);
  if (nst > 1) load(lb + 64, s1);
  if (nst > 0) store(s0, 0);
  __syncthreads();
  // step i: MFMAs on buffer i & 1; loads of step i+2; stores of step i+1 into the other buffer
#pragma unroll 1
  for (int64_t i = 0; i < nst; i += 2) {
    if (i + 2 < nst) load(lb + (i + 2) * 64, s0);
    mma(0);
    if (i + 1 < nst) store(s1, 1);
    __syncthreads();
    if (i + 1 >= nst) break;
    if (i + 3 < nst) load(lb + (i + 3) * 64, s1);
    mma(1);
    if (i + 2 < nst) store(s0, 0);
    __syncthreads();
  }

  // D[m][j]: lane l holds column j = l % 16 and rows 4 (l / 16) + v.
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = mbase + wave * 16 + 4 * (lane >> 4) + v;
      const int j = t * 16 + (lane & 15);
      if (row < mhi && j < r) {
        if (part && smajor)   // [split][M][r]: a workgroup's partials form one contiguous block
          part[((int64_t)split * M + row) * r + j] = acc[t][v];
        else if (part)        // [M][r][split]: the splits of one output form one contiguous run
          part[((int64_t)row * r + j) * gridDim.y + split] = acc[t][v];
        else
          out[row * r + j] = (uint16_t)(pack_bf16x2(acc[t][v], 0.f) & 0xFFFFu);
      }
    }
}

template <int TN>
__global__ __launch_bounds__(256) void rowproj_kernel(const uint16_t *__restrict__ in, int64_t ldin,
                                                      const uint16_t *__restrict__ p, int64_t ldp,
                                                      int64_t M, int64_t L, int r, int64_t lsplit,
                                                      float *__restrict__ part, int smajor,
                                                      uint16_t *__restrict__ out) {
  rowproj_body<TN, false>(in, ldin, p, ldp, M, L, r, lsplit, part, smajor, out, GroupArgs{}, 0);
}

template <int TN>
__global__ __launch_bounds__(256) void rowproj_grouped_kernel(
    const uint16_t *__restrict__ in, int64_t ldin, const uint16_t *__restrict__ p, int64_t ldp,
    int64_t M, int64_t L, int r, int64_t lsplit, float *__restrict__ part, int smajor,
    uint16_t *__restrict__ out, GroupArgs gr, int64_t pstride) {
  rowproj_body<TN, true>(in, ldin, p, ldp, M, L, r, lsplit, part, smajor, out, gr, pstride);
}

// The same product for at most 16 rows (decode shapes), where the reduction is short and a
// workgroup has little to stream: latency, not bandwidth, sets the time. Each wave takes 32-column
// slices 4 u + wave of its split and issues all of its loads (straight into MFMA operand registers,
// 16 bytes per lane) before its MFMAs: one memory round trip per workgroup. The four waves' sums
// are added in wave order in LDS. Rows past M and ranks past r read as zero (buffer bounds);
// requires L % 8 == 0 (every reduction length here: K % 64 == 0, N % 8 == 0).
template <int TN>
__global__ __launch_bounds__(256) void rowproj16_kernel(const uint16_t *__restrict__ in, int64_t ldin,
                                                        const uint16_t *__restrict__ p, int64_t ldp,
                                                        int64_t M, int64_t L, int r, int64_t lsplit,
                                                        float *__restrict__ part, int smajor,
                                                        uint16_t *__restrict__ out) {
  __shared__ f32x4 red[4][TN][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int split = blockIdx.x;
  const int64_t lb = split * lsplit;
  const int64_t le = (lb + lsplit < L) ? lb + lsplit : L;
  const __amdgpu_buffer_rsrc_t rI = make_rsrc(in, M * ldin * 2);
  const __amdgpu_buffer_rsrc_t rP = make_rsrc(p, (int64_t)r * ldp * 2);
  const int nl = lane & 15, kg = lane >> 4;
  f32x4 acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int64_t k0 = lb + 32 * wave; k0 < le; k0 += 256) {
    // two slices per pass: k0 and k0 + 128. A lane reads 8 columns from c = k + 8 kg; L (and so
    // le) is a multiple of 8, so such a chunk lies wholly inside or wholly past the split, and a
    // chunk past it (which would otherwise read the next row's values) reads as zero.
    const int64_t c0 = k0 + 8 * kg, c1 = k0 + 128 + 8 * kg;
    const uint32_t oob = 0x80000000u;
    const uint32_t xo0 = c0 < le ? (uint32_t)((nl * ldin + c0) * 2) : oob;
    const uint32_t xo1 = c1 < le ? (uint32_t)((nl * ldin + c1) * 2) : oob;
    const u32x4 x0 = __builtin_amdgcn_raw_buffer_load_b128(rI, xo0, 0, 0);
    const u32x4 x1 = __builtin_amdgcn_raw_buffer_load_b128(rI, xo1, 0, 0);
    u32x4 a0[TN], a1[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      const int64_t j = 16 * t + nl;
      a0[t] = __builtin_amdgcn_raw_buffer_load_b128(rP, c0 < le ? (uint32_t)((j * ldp + c0) * 2) : oob, 0, 0);
      a1[t] = __builtin_amdgcn_raw_buffer_load_b128(rP, c1 < le ? (uint32_t)((j * ldp + c1) * 2) : oob, 0, 0);
    }
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      acc[t] = mfma16x16x32(__builtin_bit_cast(bf16x8, x0), __builtin_bit_cast(bf16x8, a0[t]), acc[t]);
      acc[t] = mfma16x16x32(__builtin_bit_cast(bf16x8, x1), __builtin_bit_cast(bf16x8, a1[t]), acc[t]);
    }
  }
#pragma unroll
  for (int t = 0; t < TN; ++t) red[wave][t][lane] = acc[t];
  __syncthreads();
  // D[m][j]: lane l holds column j = l % 16 and rows 4 (l / 16) + v; wave w finishes tiles w, w + 4
  for (int t = wave; t < TN; t += 4) {
    f32x4 v4 = red[0][t][lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) v4 += red[w][t][lane];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t row = 4 * kg + v;
      const int j = 16 * t + nl;
      if (row < M && j < r) {
        if (part && smajor)
          part[((int64_t)split * M + row) * r + j] = v4[v];
        else if (part)
          part[((int64_t)row * r + j) * gridDim.x + split] = v4[v];
        else
          out[row * r + j] = (uint16_t)(pack_bf16x2(v4[v], 0.f) & 0xFFFFu);
      }
    }
  }
}

__global__ void rowproj_reduce_kernel(const float *__restrict__ part, int64_t n, int splits,
                                      uint16_t *__restrict__ out) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    // sequential sum over the splits (fixed order) of the split-major partials, its loads issued
    // eight at a time
    const float *pi = part + i;
    float a = 0.f;
    int s = 0;
    for (; s + 8 <= splits; s += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = pi[(int64_t)(s + j) * n];
#pragma unroll
      for (int j = 0; j < 8; ++j) a += v[j];
    }
    for (; s < splits; ++s) a += pi[(int64_t)s * n];
    out[i] = (uint16_t)(pack_bf16x2(a, 0.f) & 0xFFFFu);
  }
}

int rowproj_splits(int64_t M, int64_t L) {
  const int64_t wgs = (M + 63) / 64;
  int64_t s = (1024 + wgs - 1) / wgs;
  const int64_t maxs = (L + 255) / 256;   // keep at least 256 reduction elements per split
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_rowproj(const uint16_t *in, int64_t ldin, const uint16_t *p, int64_t ldp,
                          int64_t M, int64_t L, int r, int splits, float *part, uint16_t *out,
                          hipStream_t st) {
  int64_t lsplit = (L + splits - 1) / splits;
  lsplit = (lsplit + 63) / 64 * 64;
  const dim3 grid((unsigned)((M + 63) / 64), (unsigned)splits);
  float *pp = splits > 1 ? part : nullptr;
  const int smajor = out != nullptr;   // a reduction launch follows: split-major partials
  const int tn = (r + 15) / 16;
  if (M <= 16) {
    switch (tn) {
#define RP_CASE(T) \
  case T: rowproj16_kernel<T><<<dim3((unsigned)splits), dim3(256), 0, st>>>(in, ldin, p, ldp, M, L, r, lsplit, pp, smajor, out); break;
      RP_CASE(1) RP_CASE(2) RP_CASE(3) RP_CASE(4) RP_CASE(5) RP_CASE(6) RP_CASE(7) RP_CASE(8)
#undef RP_CASE
      default: return hipErrorInvalidValue;
    }
  } else {
    switch (tn) {
#define RP_CASE(T) \
  case T: rowproj_kernel<T><<<grid, dim3(256), 0, st>>>(in, ldin, p, ldp, M, L, r, lsplit, pp, smajor, out); break;
      RP_CASE(1) RP_CASE(2) RP_CASE(3) RP_CASE(4) RP_CASE(5) RP_CASE(6) RP_CASE(7) RP_CASE(8)
#undef RP_CASE
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1 || !out) return e;
  const int64_t n = M * r;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  rowproj_reduce_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(part, n, splits, out);
  return hipGetLastError();
}

hipError_t launch_rowproj_grouped(const uint16_t *in, int64_t ldin, const uint16_t *p, int64_t pstride,
                                  int64_t ldp, int64_t M, int64_t L, int r, int splits, float *part,
                                  uint16_t *out, const GroupArgs &gr, hipStream_t st) {
  const int64_t blocks = gr.grid;
  if (blocks < 1) return hipSuccess;
  int64_t lsplit = (L + splits - 1) / splits;
  lsplit = (lsplit + 63) / 64 * 64;
  const dim3 grid((unsigned)blocks, (unsigned)splits);
  float *pp = splits > 1 ? part : nullptr;
  const int tn = (r + 15) / 16;
  switch (tn) {
#define RP_CASE(T) \
  case T: rowproj_grouped_kernel<T><<<grid, dim3(256), 0, st>>>(in, ldin, p, ldp, M, L, r, lsplit, pp, 1, out, gr, pstride); break;
    RP_CASE(1) RP_CASE(2) RP_CASE(3) RP_CASE(4) RP_CASE(5) RP_CASE(6) RP_CASE(7) RP_CASE(8)
#undef RP_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  const int64_t n = M * r;
  int64_t nb = (n + 255) / 256;
  if (nb > 4096) nb = 4096;
  rowproj_reduce_kernel<<<dim3((unsigned)nb), dim3(256), 0, st>>>(part, n, splits, out);
  return hipGetLastError();
}

// ------------------------------------------------------------------- group tables (routing on the device)
size_t moe_table_bytes(int E) { return 8 * (size_t)(E + 1) + 3 * 4 * (size_t)(E + 1); }

__global__ __launch_bounds__(256) void moe_plan_kernel(const int64_t *__restrict__ dcounts, int E,
                                                       int64_t m, int64_t tiles_n, int64_t tiles_k,
                                                       void *table) {
  __shared__ int64_t cnt[kMaxExperts];
  const int t = threadIdx.x;
  if (t < E) {   // each count clamped to [0, m] first, so the running sums below cannot overflow
    const int64_t c = dcounts[t];
    cnt[t] = c > 0 ? (c < m ? c : m) : 0;
  }
  __syncthreads();
  if (t != 0) return;
  int64_t *mo = moe_table_m_off(table);
  int32_t *tf = moe_table_tiles(table, E, 0), *td = moe_table_tiles(table, E, 1);
  int32_t *tb = moe_table_tiles(table, E, 2);
  int64_t off = 0, a = 0, b = 0, c = 0;
  mo[0] = 0;
  tf[0] = td[0] = tb[0] = 0;
  for (int e = 0; e < E; ++e) {
    const int64_t hi = off + cnt[e] < m ? off + cnt[e] : m;
    const int64_t blocks = (hi - off + 255) / 256;
    a += blocks * tiles_n;
    b += blocks * tiles_k;
    c += (hi - off + 63) / 64;
    off = hi;
    mo[e + 1] = off;
    tf[e + 1] = (int32_t)a;
    td[e + 1] = (int32_t)b;
    tb[e + 1] = (int32_t)c;
  }
}

hipError_t launch_moe_plan(const int64_t *dcounts, int E, int64_t m, int64_t tiles_n,
                           int64_t tiles_k, void *table, hipStream_t st) {
  if (E < 1 || E > kMaxExperts || !dcounts || !table) return hipErrorInvalidValue;
  moe_plan_kernel<<<dim3(1), dim3(256), 0, st>>>(dcounts, E, m, tiles_n, tiles_k, table);
  return hipGetLastError();
}

// ------------------------------------------------------------------------------------ mreduce
// out[j][c] = sum over m of P[m][j] * Q[m][c]  (dA: P = U, Q = X;  dB: P = T, Q = dY).
// Workgroup: 128 columns c x all r (<= 128) rows j, over one split of the M rows in stages of 64,
// loaded two stages ahead with coalesced 16-byte loads (16 lanes per 256-byte row).
// Both tiles are staged row-major in LDS (rows padded by 32 bytes so that the 4 rows a 16-lane
// group touches fall in different bank ranges) and read with the gfx950 transposing LDS load
// ds_read_b64_tr_b16, which hands each lane 4 consecutive rows (m) of one column: exactly the
// MFMA 16x16x32 operand layout with m as the reduction index.
constexpr int kMR_BM = 64;                 // m per stage
constexpr int kMR_BC = 128;                // columns per workgroup
constexpr int kMR_QROW = kMR_BC + 16;      // Q row stride in bf16 (288 bytes)

typedef __attribute__((ext_vector_type(4))) short s16x4;

__device__ __forceinline__ s16x4 lds_tr16(const uint16_t *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4 *)(p));
}

// kGrp: one sum per expert over its own rows (expert blockIdx.z: rows gr.m_off[z] ..
// gr.m_off[z+1] - 1, cut into gridDim.y splits of whole 64-row stages); partials
// [expert][split][r][C].
template <int TJ, bool kGrp>
__device__ __forceinline__ void mreduce_body(const uint16_t *__restrict__ P,
                                             const uint16_t *__restrict__ Q, int64_t ldq, int64_t M,
                                             int64_t C, int r, int64_t msplit,
                                             float *__restrict__ part, const GroupArgs &gr) {
  constexpr int PROW = TJ * 16 + 16;          // P row stride in bf16 (padded by 32 bytes)
  __shared__ uint16_t sQ[2][kMR_BM * kMR_QROW];
  __shared__ uint16_t sP[2][kMR_BM * PROW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kMR_BC;
  const int split = blockIdx.y;
  int64_t lo = 0, hi = M;
  if (kGrp) {
    lo = grp_m_off(gr, blockIdx.z);
    hi = grp_m_off(gr, blockIdx.z + 1);
    msplit = (hi - lo + gridDim.y - 1) / gridDim.y;
    msplit = (msplit + kMR_BM - 1) / kMR_BM * kMR_BM;
  }
  const int64_t mb = lo + split * msplit;
  const int64_t me = (mb + msplit < hi) ? mb + msplit : hi;
  const bool pvec = (r & 7) == 0;

  f32x4 acc[TJ][2];
#pragma unroll
  for (int t = 0; t < TJ; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u) acc[t][u] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging registers: Q 4 chunks of 16 bytes, P up to TJ / 2 chunks (vector path)
  struct Stage {
    uint4 q[4];
    uint4 p[(TJ + 1) / 2];
  };
  auto load = [&](int64_t ms, Stage &st) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 4, ch = q & 15;
      const int64_t m = ms + row, c = c0 + ch * 8;
      st.q[i] = (m < me && c < C) ? *reinterpret_cast<const uint4 *>(Q + m * ldq + c)
                                  : make_uint4(0, 0, 0, 0);
    }
    if (pvec) {
#pragma unroll
      for (int i = 0; i < (TJ + 1) / 2; ++i) {
        const int q = tid + 256 * i;               // chunk q of the P tile: row q / (2 TJ)
        const int row = q / (2 * TJ), ch = q % (2 * TJ);
        const int64_t m = ms + row;
        const int j = ch * 8;
        st.p[i] = (row < kMR_BM && m < me && j < r) ? *reinterpret_cast<const uint4 *>(P + m * r + j)
                                                    : make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto store = [&](int64_t ms, const Stage &st, int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int q = tid + 256 * i;
      const int row = q >> 4, ch = q & 15;
      *reinterpret_cast<uint4 *>(&sQ[buf][row * kMR_QROW + ch * 8]) = st.q[i];
    }
    if (pvec) {
#pragma unroll
      for (int i = 0; i < (TJ + 1) / 2; ++i) {
        const int q = tid + 256 * i;
        const int row = q / (2 * TJ), ch = q % (2 * TJ);
        if (row < kMR_BM) *reinterpret_cast<uint4 *>(&sP[buf][row * PROW + ch * 8]) = st.p[i];
      }
    } else {
      for (int q = tid; q < kMR_BM * TJ * 16; q += 256) {
        const int row = q / (TJ * 16), j = q % (TJ * 16);
        const int64_t m = ms + row;
        sP[buf][row * PROW + j] = (m < me && j < r) ? P[m * r + j] : (uint16_t)0;
      }
    }
  };

  // transposing fragment reads: lane i of a 16-lane group gets rows 4 i' .. of its column
  const int g16 = lane >> 4, l16 = lane & 15;
  auto frag = [&](const uint16_t *S, int rowstride, int colbase, int kslice) {
    // 8 consecutive m (= 8 g16 .. + 7 of the k-slice) of column colbase + l16, as two 4-row reads
    const int m0 = kslice * 32 + g16 * 8 + (l16 >> 2);
    const int col = colbase + 4 * (l16 & 3);
    const s16x4 lo = lds_tr16(S + m0 * rowstride + col);
    const s16x4 hi = lds_tr16(S + (m0 + 4) * rowstride + col);
    typedef __attribute__((ext_vector_type(8))) short s16x8;
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  auto mma = [&](int buf) {
    const uint16_t *Sq = sQ[buf];
    const uint16_t *Sp = sP[buf];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 bq[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) bq[u] = frag(Sq, kMR_QROW, wave * 32 + u * 16, ks);
#pragma unroll
      for (int t = 0; t < TJ; ++t) {
        const bf16x8 ap = frag(Sp, PROW, t * 16, ks);
#pragma unroll
        for (int u = 0; u < 2; ++u) acc[t][u] = mfma16x16x32(ap, bq[u], acc[t][u]);
      }
    }
  };

  // stage i: MFMAs on buffer i & 1; loads of stage i+2; stores of stage i+1 into the other buffer
  const int64_t nst = (me > mb) ? (me - mb + kMR_BM - 1) / kMR_BM : 0;
  Stage s0, s1;
  if (nst > 0) load(mb, s0);
  if (nst > 1) load(mb + kMR_BM, s1);
  if (nst > 0) store(mb, s0, 0);
  __syncthreads();
#pragma unroll 1
  for (int64_t i = 0; i < nst; i += 2) {
    if (i + 2 < nst) load(mb + (i + 2) * kMR_BM, s0);
    mma(0);
    if (i + 1 < nst) store(mb + (i + 1) * kMR_BM, s1, 1);
    __syncthreads();
    if (i + 1 >= nst) break;
    if (i + 3 < nst) load(mb + (i + 3) * kMR_BM, s1);
    mma(1);
    if (i + 2 < nst) store(mb + (i + 2) * kMR_BM, s0, 0);
    __syncthreads();
  }

  // D[j][c] (16 x 16 blocks): lane l holds column c = l % 16 and rows j = 4 (l / 16) + v.
#pragma unroll
  for (int t = 0; t < TJ; ++t)
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = t * 16 + 4 * g16 + v;
        const int64_t c = c0 + wave * 32 + u * 16 + l16;
        if (j < r && c < C)
          part[(((int64_t)blockIdx.z * gridDim.y + split) * r + j) * C + c] = acc[t][u][v];
      }
}

template <int TJ>
__global__ __launch_bounds__(256) void mreduce_kernel(const uint16_t *__restrict__ P,
                                                      const uint16_t *__restrict__ Q, int64_t ldq,
                                                      int64_t M, int64_t C, int r, int64_t msplit,
                                                      float *__restrict__ part) {
  mreduce_body<TJ, false>(P, Q, ldq, M, C, r, msplit, part, GroupArgs{});
}

template <int TJ>
__global__ __launch_bounds__(256) void mreduce_grouped_kernel(const uint16_t *__restrict__ P,
                                                              const uint16_t *__restrict__ Q,
                                                              int64_t ldq, int64_t C, int r,
                                                              float *__restrict__ part, GroupArgs gr) {
  mreduce_body<TJ, true>(P, Q, ldq, 0, C, r, 0, part, gr);
}

// out = s * (sum over splits of part), for E blocks of [r][C] (E = 1 unless grouped); block e of
// the output is [r][C] at out + e r C, or [C][r] there when transposed.
__global__ void mreduce_final_kernel(const float *__restrict__ part, int64_t C, int r, int splits,
                                     int E, float s, bool transposed, uint16_t *__restrict__ out) {
  const int64_t n = (int64_t)r * C;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n * E;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t e = i / n, ie = i - e * n;
    const float *pe = part + e * splits * n + ie;
    float a = 0.f;
    int sp = 0;
    for (; sp + 8 <= splits; sp += 8) {   // fixed-order sum, loads issued eight at a time
      float v8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) v8[j] = pe[(int64_t)(sp + j) * n];
#pragma unroll
      for (int j = 0; j < 8; ++j) a += v8[j];
    }
    for (; sp < splits; ++sp) a += pe[(int64_t)sp * n];
    const uint16_t v = (uint16_t)(pack_bf16x2(s * a, 0.f) & 0xFFFFu);
    const int64_t j = ie / C, c = ie % C;
    if (transposed)
      out[e * n + c * r + j] = v;
    else
      out[i] = v;
  }
}

// Splits of the M-reduction over C / 128 column tiles. One layer: as many as let ONE round of
// workgroups fill the GPU, so that each workgroup streams the longest run of rows and no partial
// round trails (measured: the backward's rank-r part of the mlp_up shape 0.153 -> 0.130 ms). A
// round is the 256 CUs times the workgroups one CU holds, which the LDS staging of a workgroup sets
// (two 64-row stages of Q and of P: 45-74 KB by the rank): 3 for up to 32 ranks, 2 up to 64, 1
// above (gfx950, hipcc's resource report). E > 1 experts: about 1024 workgroups, more than a
// round, since a split covers part of one expert's rows, whose count varies with the routing, and
// shorter splits keep the largest expert's from setting the time (one round measured 1-3% slower
// on the grouped backward). One expert gives the single layer's count.
int mreduce_splits(int64_t M, int64_t C, int r, int E) {
  const int tj = (r + 15) / 16;
  const int64_t round = 256 * (tj <= 2 ? 3 : tj <= 4 ? 2 : 1);
  const int64_t tiles = (C + kMR_BC - 1) / kMR_BC * (E > 0 ? E : 1);
  int64_t s = E > 1 ? (1024 + tiles - 1) / tiles : round / tiles;
  const int64_t maxs = (M + kMR_BM - 1) / kMR_BM;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_mreduce(const uint16_t *P, const uint16_t *Q, int64_t ldq, int64_t M, int64_t C,
                          int r, float s, int splits, float *part, uint16_t *out,
                          bool transposed_out, hipStream_t st) {
  int64_t msplit = (M + splits - 1) / splits;
  msplit = (msplit + kMR_BM - 1) / kMR_BM * kMR_BM;
  const dim3 grid((unsigned)((C + kMR_BC - 1) / kMR_BC), (unsigned)splits);
  const int tj = (r + 15) / 16;
  switch (tj) {
#define MR_CASE(T) \
  case T: mreduce_kernel<T><<<grid, dim3(256), 0, st>>>(P, Q, ldq, M, C, r, msplit, part); break;
    MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4) MR_CASE(5) MR_CASE(6) MR_CASE(7) MR_CASE(8)
#undef MR_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)r * C;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  mreduce_final_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(part, C, r, splits, 1, s,
                                                                     transposed_out, out);
  return hipGetLastError();
}

hipError_t launch_mreduce_grouped(const uint16_t *P, const uint16_t *Q, int64_t ldq, int64_t C, int r,
                                  float s, int splits, float *part, uint16_t *out,
                                  bool transposed_out, const GroupArgs &gr, hipStream_t st) {
  const dim3 grid((unsigned)((C + kMR_BC - 1) / kMR_BC), (unsigned)splits, (unsigned)gr.E);
  const int tj = (r + 15) / 16;
  switch (tj) {
#define MR_CASE(T) \
  case T: mreduce_grouped_kernel<T><<<grid, dim3(256), 0, st>>>(P, Q, ldq, C, r, part, gr); break;
    MR_CASE(1) MR_CASE(2) MR_CASE(3) MR_CASE(4) MR_CASE(5) MR_CASE(6) MR_CASE(7) MR_CASE(8)
#undef MR_CASE
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = (int64_t)gr.E * r * C;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  mreduce_final_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(part, C, r, splits, gr.E, s,
                                                                     transposed_out, out);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------- transpose
__global__ void transpose_kernel(const uint16_t *__restrict__ src, int64_t L, int r,
                                 uint16_t *__restrict__ dst) {
  const int64_t n = L * r;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t j = i / L, l = i % L;
    dst[i] = src[l * r + j];
  }
}

hipError_t launch_transpose(const uint16_t *src, int64_t L, int r, uint16_t *dst, hipStream_t st) {
  const int64_t n = L * r;
  int64_t blocks = (n + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  transpose_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(src, L, r, dst);
  return hipGetLastError();
}

}  // namespace nf4q

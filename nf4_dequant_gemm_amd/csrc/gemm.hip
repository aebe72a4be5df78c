// Fused NF4-dequant GEMM with the LoRA correction in the same output tile (gfx950, bf16 MFMA).
//
// One kernel template serves both dense contractions of the QLoRA layer:
//   forward  Y  = X  deq(W)^T + s T B^T    (reduction over k; weight rows are output columns)
//   backward dX = dY deq(W)   + s U A      (reduction over n; weight columns are output columns)
// The NF4 weight is decoded on the fly into LDS and never written to HBM; the rank-r LoRA
// product runs as extra reduction steps over [T | U] and s*[B | A^T] into the same
// accumulators, so the layer needs no second matmul and no separate add [Unsloth pages: "Inside
// Unsloth" listing, "What You'll Learn", "LoRA and QLoRA" (one fused launch for dequant, matmul
// and LoRA correction); pyshine code tour, "Detailed view" (LoRA delta computed inside the
// matmul); v0.1.463-beta release article, "About the Unsloth Project" (no redundant
// dequantisation buffers)].
//
// Tiling: 256 x 256 output tile per workgroup of 4 waves (2 x 2), 128 x 128 per wave as 4 x 4
// MFMA 32x32x16 tiles; reduction steps of 64 (one NF4 absmax block), double-buffered in LDS
// (2 x 64 KB). LDS rows hold 64 bf16 as 8 chunks of 16 bytes, XOR-swizzled by (row & 7) so that
// 8 consecutive rows reading the same logical chunk hit 8 different bank groups.
#include "common.h"
#include "launch.h"

namespace nf4q {

constexpr int kTile = 256;            // output tile rows and columns
constexpr int kStep = 64;             // reduction step (= NF4 block)
constexpr int kThreads = 256;
constexpr int kTileChunks = kTile * kStep / 8;   // 2048 chunks of 8 bf16

__device__ __forceinline__ int swz(int row, int c) { return row * 8 + (c ^ (row & 7)); }

__device__ __forceinline__ uint32_t nib(uint32_t d, int j) {
  // element j (0..7) of a 32-bit word of packed codes: byte j/2, high nibble first
  return (d >> (8 * (j >> 1) + ((j & 1) ? 0 : 4))) & 15u;
}

template <bool kDx>
struct Stage {
  uint4 a[8];         // A-side chunks (X or dY)
  uint32_t c[8];      // codes: fwd uses c[0..7] as the row's 32 bytes, dx one word per row
  float am[8];        // block constants: fwd uses am[0], dx one per row
};

template <bool kDx>
__device__ __forceinline__ void load_base(const GemmArgs &g, int64_t m0, int64_t c0, int step,
                                          Stage<kDx> &st) {
  const int tid = threadIdx.x;
  const int64_t red0 = (int64_t)step * kStep;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + kThreads * i;
    const int row = q >> 3, c = q & 7;
    const int64_t m = m0 + row, red = red0 + c * 8;
    if (m < g.M && red < g.R)
      st.a[i] = *reinterpret_cast<const uint4 *>(g.a_side + m * g.lda + red);
    else
      st.a[i] = make_uint4(0, 0, 0, 0);
  }
  const int64_t K = g.w.k;
  if (!kDx) {
    const int64_t n = c0 + tid;
    if (n < g.w.n) {
      const uint4 *p = reinterpret_cast<const uint4 *>(g.w.codes + n * (K / 2) + red0 / 2);
      const uint4 x = p[0], y = p[1];
      st.c[0] = x.x; st.c[1] = x.y; st.c[2] = x.z; st.c[3] = x.w;
      st.c[4] = y.x; st.c[5] = y.y; st.c[6] = y.z; st.c[7] = y.w;
      st.am[0] = block_absmax(g.w, n * (K / kStep) + step);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) st.c[j] = 0x77777777u;   // code 7 = exact zero
      st.am[0] = 0.f;
    }
  } else {
    const int kg = tid >> 3, ng = tid & 7;
    const int64_t k = c0 + kg * 8;
    const uint32_t *cw = reinterpret_cast<const uint32_t *>(g.w.codes);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t n = red0 + ng * 8 + i;
      if (n < g.w.n && k < K) {
        st.c[i] = cw[(n * K + k) >> 3];
        st.am[i] = block_absmax(g.w, n * (K / kStep) + (k >> 6));
      } else {
        st.c[i] = 0x77777777u;
        st.am[i] = 0.f;
      }
    }
  }
}

template <bool kDx>
__device__ __forceinline__ void store_base(const Stage<kDx> &st, uint4 *sA, uint4 *sB,
                                           const float *lv) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + kThreads * i;
    sA[swz(q >> 3, q & 7)] = st.a[i];
  }
  if (!kDx) {
    const float a = st.am[0];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t d = st.c[j];
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = lv[nib(d, e)] * a;
      uint4 u;
      u.x = pack_bf16x2(v[0], v[1]);
      u.y = pack_bf16x2(v[2], v[3]);
      u.z = pack_bf16x2(v[4], v[5]);
      u.w = pack_bf16x2(v[6], v[7]);
      sB[swz(tid, j)] = u;
    }
  } else {
    const int kg = tid >> 3, ng = tid & 7;
    float v[8][8];   // [n row i][k element j]
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) v[i][j] = lv[nib(st.c[i], j)] * st.am[i];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint4 u;
      u.x = pack_bf16x2(v[0][j], v[1][j]);
      u.y = pack_bf16x2(v[2][j], v[3][j]);
      u.z = pack_bf16x2(v[4][j], v[5][j]);
      u.w = pack_bf16x2(v[6][j], v[7][j]);
      sB[swz(kg * 8 + j, ng)] = u;
    }
  }
}

// LoRA reduction step: A-side = [T | U] columns jb..jb+63, B-side = s * (B rows | A^T rows).
template <bool kDx>
__device__ __forceinline__ void store_lora(const GemmArgs &g, int64_t m0, int64_t c0, int jb,
                                           uint4 *sA, uint4 *sB) {
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int i = 0; i < 8; ++i) {
    const int q = tid + kThreads * i;
    const int row = q >> 3, c = q & 7;
    uint32_t wa[4], wb[4];
    const int64_t m = m0 + row;
    const int64_t cc = c0 + row;
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
      if (cc < g.C) {
        if (!kDx) {
          if (j0 < g.r) b0 = bf16_to_f32(g.lora_b[cc * g.r + j0]);
          if (j1 < g.r) b1 = bf16_to_f32(g.lora_b[cc * g.r + j1]);
        } else {
          if (j0 < g.r) b0 = bf16_to_f32(g.lora_b[(int64_t)j0 * g.C + cc]);
          if (j1 < g.r) b1 = bf16_to_f32(g.lora_b[(int64_t)j1 * g.C + cc]);
        }
      }
      wb[e >> 1] = pack_bf16x2(g.s * b0, g.s * b1);
    }
    sA[swz(row, c)] = make_uint4(wa[0], wa[1], wa[2], wa[3]);
    sB[swz(row, c)] = make_uint4(wb[0], wb[1], wb[2], wb[3]);
  }
}

template <bool kDx>
__global__ __launch_bounds__(kThreads, 1) void gemm_kernel(GemmArgs g) {
  __shared__ uint4 smA[2][kTileChunks];
  __shared__ uint4 smB[2][kTileChunks];
  __shared__ float lv[16];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = (int64_t)blockIdx.y * kTile;
  const int64_t c0 = (int64_t)blockIdx.x * kTile;
  if (tid < 16) lv[tid] = g.t.level[tid];

  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

  const int nbase = (int)(g.R / kStep) + ((g.R % kStep) ? 1 : 0);
  const int nsteps = nbase + (g.r + kStep - 1) / kStep;

  Stage<kDx> st;
  if (nbase > 0) load_base<kDx>(g, m0, c0, 0, st);
  __syncthreads();   // lv ready
  if (nbase > 0)
    store_base<kDx>(st, smA[0], smB[0], lv);
  else
    store_lora<kDx>(g, m0, c0, 0, smA[0], smB[0]);
  __syncthreads();

#pragma unroll 1
  for (int s = 0; s < nsteps; ++s) {
    const int cur = s & 1;
    const bool next_base = (s + 1) < nbase;
    if (next_base) load_base<kDx>(g, m0, c0, s + 1, st);

    const uint4 *sA = smA[cur];
    const uint4 *sB = smB[cur];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 af[4], bfr[4];
      const int c = kk * 2 + (lane >> 5);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        af[t] = __builtin_bit_cast(bf16x8, sA[swz(wm * 128 + t * 32 + (lane & 31), c)]);
        bfr[t] = __builtin_bit_cast(bf16x8, sB[swz(wn * 128 + t * 32 + (lane & 31), c)]);
      }
#pragma unroll
      for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) acc[tm][tn] = mfma32x32x16(af[tm], bfr[tn], acc[tm][tn]);
    }

    if (s + 1 < nsteps) {
      if (next_base)
        store_base<kDx>(st, smA[cur ^ 1], smB[cur ^ 1], lv);
      else
        store_lora<kDx>(g, m0, c0, (s + 1 - nbase) * kStep, smA[cur ^ 1], smB[cur ^ 1]);
    }
    __syncthreads();
  }

  // Epilogue: fp32 accumulators -> bf16 (round to nearest even).
#pragma unroll
  for (int tm = 0; tm < 4; ++tm)
#pragma unroll
    for (int tn = 0; tn < 4; ++tn)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 128 + tm * 32 + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        const int64_t col = c0 + wn * 128 + tn * 32 + (lane & 31);
        if (row < g.M && col < g.C)
          g.out[row * g.ldo + col] = (uint16_t)(pack_bf16x2(acc[tm][tn][v], 0.f) & 0xFFFFu);
      }
}

static hipError_t launch_gemm(const GemmArgs &g, bool dx, hipStream_t st) {
  const dim3 grid((unsigned)((g.C + kTile - 1) / kTile), (unsigned)((g.M + kTile - 1) / kTile));
  if (dx)
    gemm_kernel<true><<<grid, dim3(kThreads), 0, st>>>(g);
  else
    gemm_kernel<false><<<grid, dim3(kThreads), 0, st>>>(g);
  return hipGetLastError();
}

hipError_t launch_gemm_dx(const GemmArgs &g, hipStream_t st) { return launch_gemm(g, true, st); }

}  // namespace nf4q

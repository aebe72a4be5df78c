// Gate/up pair of QLoRA projections joined by the SwiGLU activation (gfx950): the elementwise
// parts. The pages name a fused gated-MLP activation whose backward reuses its input buffers
// [pyshine Unsloth code tour, "Why You Need This": swiglu.py; "Inside Unsloth" listing, "What
// You'll Learn", "Triton Kernel Internals"]; the activation is read as the Llama gated MLP,
// H = silu(Yg) * Yu with silu(x) = x / (1 + exp(-x)).
//
// The two projections run as ONE stacked QLoRA layer (the existing fused kernels): the base
// weight is the stacked NF4 tensor [Wg; Wu] [2n, k], the adapters are [Ag; Au] [2r, k] and the
// block-diagonal [[Bg, 0], [0, Bu]] [2n, 2r], so one forward yields Ygu = [Yg | Yu] per row and
// one backward with dY = [dYg | dYu] yields dX, [dAg; dAu] and, on its diagonal blocks, dBg, dBu.
// The kernels here are what that composition adds: the activation, its backward, and the
// block-diagonal B and its gradient's diagonal blocks. Above the decode shapes the forward runs
// the fused kernel's pair form instead, with the activation in its epilogue (fwd.hip);
// swiglu_fwd_kernel serves the decode shapes (M <= 48). All are HBM-bound streams; rows are read
// and written in 16-byte pieces of 8 columns (n % 8 == 0), consecutive lanes on consecutive
// pieces.
#include "common.h"
#include "launch.h"

namespace nf4q {
namespace {

__device__ __forceinline__ float sigmoid(float x) { return 1.f / (1.f + __expf(-x)); }

// H[i][c] = silu(Yg[i][c]) * Yu[i][c]; Ygu rows hold Yg then Yu (2n columns).
__global__ __launch_bounds__(256) void swiglu_fwd_kernel(const uint16_t *__restrict__ ygu,
                                                         int64_t m, int64_t n,
                                                         uint16_t *__restrict__ h) {
  const int64_t pieces = n / 8, total = m * pieces;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / pieces, c = (i - row * pieces) * 8;
    const u32x4 g = *reinterpret_cast<const u32x4 *>(ygu + row * 2 * n + c);
    const u32x4 u = *reinterpret_cast<const u32x4 *>(ygu + row * 2 * n + n + c);
    u32x4 o;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g0 = bf16_lo(g[e]), g1 = bf16_hi(g[e]);
      o[e] = pack_bf16x2(g0 * sigmoid(g0) * bf16_lo(u[e]), g1 * sigmoid(g1) * bf16_hi(u[e]));
    }
    *reinterpret_cast<u32x4 *>(h + row * n + c) = o;
  }
}

// dYg = dH * Yu * silu'(Yg), silu'(x) = sigma(x) (1 + x (1 - sigma(x))); dYu = dH * silu(Yg).
// Written as one [m, 2n] gradient, dYg then dYu in each row (the stacked layer's dY).
__global__ __launch_bounds__(256) void swiglu_bwd_kernel(const uint16_t *__restrict__ dh,
                                                         const uint16_t *__restrict__ ygu,
                                                         int64_t m, int64_t n,
                                                         uint16_t *__restrict__ dygu) {
  const int64_t pieces = n / 8, total = m * pieces;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / pieces, c = (i - row * pieces) * 8;
    const u32x4 d = *reinterpret_cast<const u32x4 *>(dh + row * n + c);
    const u32x4 g = *reinterpret_cast<const u32x4 *>(ygu + row * 2 * n + c);
    const u32x4 u = *reinterpret_cast<const u32x4 *>(ygu + row * 2 * n + n + c);
    u32x4 og, ou;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float rg[2], ru[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const float dv = hh ? bf16_hi(d[e]) : bf16_lo(d[e]);
        const float gv = hh ? bf16_hi(g[e]) : bf16_lo(g[e]);
        const float uv = hh ? bf16_hi(u[e]) : bf16_lo(u[e]);
        const float sg = sigmoid(gv);
        rg[hh] = dv * uv * (sg * (1.f + gv * (1.f - sg)));
        ru[hh] = dv * (gv * sg);
      }
      og[e] = pack_bf16x2(rg[0], rg[1]);
      ou[e] = pack_bf16x2(ru[0], ru[1]);
    }
    *reinterpret_cast<u32x4 *>(dygu + row * 2 * n + c) = og;
    *reinterpret_cast<u32x4 *>(dygu + row * 2 * n + n + c) = ou;
  }
}

// B2 [2n, 2r] = [[Bg, 0], [0, Bu]] from Bg, Bu [n, r].
__global__ __launch_bounds__(256) void blockdiag_kernel(const uint16_t *__restrict__ bg,
                                                        const uint16_t *__restrict__ bu, int64_t n,
                                                        int r, uint16_t *__restrict__ b2) {
  const int64_t total = 2 * n * 2 * r;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / (2 * r);
    const int j = (int)(i - row * 2 * r);
    uint16_t v = 0;
    if (row < n && j < r) v = bg[row * r + j];
    else if (row >= n && j >= r) v = bu[(row - n) * r + (j - r)];
    b2[i] = v;
  }
}

// dBg = dB2[0:n, 0:r], dBu = dB2[n:2n, r:2r].
__global__ __launch_bounds__(256) void diagblocks_kernel(const uint16_t *__restrict__ db2,
                                                         int64_t n, int r,
                                                         uint16_t *__restrict__ dbg,
                                                         uint16_t *__restrict__ dbu) {
  const int64_t total = n * r;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / r;
    const int j = (int)(i - row * r);
    dbg[i] = db2[row * 2 * r + j];
    dbu[i] = db2[(n + row) * 2 * r + r + j];
  }
}

unsigned grid_for(int64_t items) {
  int64_t b = (items + 255) / 256;
  if (b > 8192) b = 8192;   // 32 workgroups per CU, grid-stride beyond
  return (unsigned)(b < 1 ? 1 : b);
}

}  // namespace

hipError_t launch_swiglu_fwd(const uint16_t *ygu, int64_t m, int64_t n, uint16_t *h, hipStream_t st) {
  if (n % 8) return hipErrorInvalidValue;
  swiglu_fwd_kernel<<<dim3(grid_for(m * n / 8)), dim3(256), 0, st>>>(ygu, m, n, h);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const uint16_t *dh, const uint16_t *ygu, int64_t m, int64_t n,
                             uint16_t *dygu, hipStream_t st) {
  if (n % 8) return hipErrorInvalidValue;
  swiglu_bwd_kernel<<<dim3(grid_for(m * n / 8)), dim3(256), 0, st>>>(dh, ygu, m, n, dygu);
  return hipGetLastError();
}

hipError_t launch_blockdiag(const uint16_t *bg, const uint16_t *bu, int64_t n, int r, uint16_t *b2,
                            hipStream_t st) {
  blockdiag_kernel<<<dim3(grid_for(4 * n * r)), dim3(256), 0, st>>>(bg, bu, n, r, b2);
  return hipGetLastError();
}

hipError_t launch_diagblocks(const uint16_t *db2, int64_t n, int r, uint16_t *dbg, uint16_t *dbu,
                             hipStream_t st) {
  diagblocks_kernel<<<dim3(grid_for(n * r)), dim3(256), 0, st>>>(db2, n, r, dbg, dbu);
  return hipGetLastError();
}

}  // namespace nf4q

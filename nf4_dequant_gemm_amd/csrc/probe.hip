// Measured-achievable matrix-core rate on this chip (a measurement aid for bench.py, not part of
// the layer): every wave runs back-to-back bf16 MFMA 16x16x32 on register operands read once from
// caller data, eight independent accumulators, no memory traffic in the loop. With realistic
// operand values this measures the dense bf16 rate the chip sustains under its power limit,
// against which the fused kernels' rate can be read.
#include <hip/hip_runtime.h>
#include <cstdint>

#include "probe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kAcc = 8;

__global__ __launch_bounds__(256) void mfma_loop_kernel(const uint4 *__restrict__ a,
                                                        const uint4 *__restrict__ b, int64_t n16,
                                                        int iters, float *__restrict__ out) {
  const int64_t gt = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8 av[4], bv[2];
#pragma unroll
  for (int i = 0; i < 4; ++i) av[i] = __builtin_bit_cast(bf16x8, a[(gt * 4 + i) % n16]);
#pragma unroll
  for (int i = 0; i < 2; ++i) bv[i] = __builtin_bit_cast(bf16x8, b[(gt * 2 + i) % n16]);
  f32x4 acc[kAcc];
#pragma unroll
  for (int i = 0; i < kAcc; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // one asm block per iteration pins each accumulator to its registers (the compiler otherwise
  // rotates them through copies inside the loop)
#pragma unroll 1
  for (int it = 0; it < iters; ++it) {
    asm volatile(
        "v_mfma_f32_16x16x32_bf16 %0, %8, %12, %0\n\t"
        "v_mfma_f32_16x16x32_bf16 %1, %9, %12, %1\n\t"
        "v_mfma_f32_16x16x32_bf16 %2, %10, %12, %2\n\t"
        "v_mfma_f32_16x16x32_bf16 %3, %11, %12, %3\n\t"
        "v_mfma_f32_16x16x32_bf16 %4, %8, %13, %4\n\t"
        "v_mfma_f32_16x16x32_bf16 %5, %9, %13, %5\n\t"
        "v_mfma_f32_16x16x32_bf16 %6, %10, %13, %6\n\t"
        "v_mfma_f32_16x16x32_bf16 %7, %11, %13, %7"
        : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
          "+v"(acc[6]), "+v"(acc[7])
        : "v"(av[0]), "v"(av[1]), "v"(av[2]), "v"(av[3]), "v"(bv[0]), "v"(bv[1]));
  }
  // the accumulators are read only after the last MFMA has had time to complete
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+v"(acc[0]), "+v"(acc[1]), "+v"(acc[2]), "+v"(acc[3]), "+v"(acc[4]), "+v"(acc[5]),
                 "+v"(acc[6]), "+v"(acc[7]));
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kAcc; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
  out[gt] = s;
}

}  // namespace

extern "C" int nf4probe_mfma_loop(const void *a, const void *b, int64_t bytes, int64_t workgroups,
                                  int32_t iters, float *out, void *stream) {
  if (!a || !b || !out || bytes < 16 || workgroups <= 0 || iters <= 0) return -1;
  mfma_loop_kernel<<<dim3((unsigned)workgroups), dim3(256), 0, (hipStream_t)stream>>>(
      static_cast<const uint4 *>(a), static_cast<const uint4 *>(b), bytes / 16, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" double nf4probe_mfma_loop_flops(int64_t workgroups, int32_t iters) {
  return (double)workgroups * 4 /* waves */ * iters * kAcc * 16.0 * 16.0 * 32.0 * 2.0;
}

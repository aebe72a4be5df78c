/* Measurement aid beside the QLoRA layer library (libnf4probe.so, built with it): a matrix-core
 * loop that measures the dense bf16 MFMA rate the chip sustains, the "measured-achievable" peak
 * that the fused GEMM rates are compared with. Not part of the layer's interface.
 *
 * nf4probe_mfma_loop: launches `workgroups` workgroups of 4 waves on `stream` (a hipStream_t, 0 =
 * default); every wave runs `iters` iterations of 8 independent bf16 MFMA 16x16x32 on operands read
 * once from the device buffers a and b (`bytes` each, >= 16; lanes read 16-byte pieces modulo that
 * size), then writes one float per thread to the device buffer out [workgroups * 256] (so that the
 * work is not optimised away). The caller owns every buffer. Returns 0, -1 for an invalid argument
 * (nothing launched) or -3 for a HIP launch error.
 * nf4probe_mfma_loop_flops: the algorithmic flops of one such launch. */
#ifndef NF4PROBE_H
#define NF4PROBE_H
#include <stdint.h>
#ifdef __cplusplus
extern "C" {
#endif
int nf4probe_mfma_loop(const void *a, const void *b, int64_t bytes, int64_t workgroups,
                       int32_t iters, float *out, void *stream);
double nf4probe_mfma_loop_flops(int64_t workgroups, int32_t iters);
#ifdef __cplusplus
}
#endif
#endif

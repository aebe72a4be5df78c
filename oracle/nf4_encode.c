/* NF4 encoder of the CPU oracle -- test infrastructure only (see oracle/__init__.py).
 *
 * The same plain definition as oracle/nf4.py's numpy encode, written as a C loop so that the
 * full-size weights of the benchmark workloads can be encoded in seconds: for every element,
 * v = fl32(w / a) (IEEE single-precision division; built without fast-math, SSE arithmetic) and
 * the code is the index of the nearest of the 16 levels, distances taken in double, ties to the
 * lower index; a block constant of 0 gives code 7 (the exact zero level). Blocks are 64
 * consecutive elements [Unsloth v0.1.463-beta release article, "About the Unsloth Project": 4-bit
 * NormalFloat base weight; block size, rounding and tie rule are the oracle's stated readings].
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared oracle/nf4_encode.c -o oracle/libnf4oracle.so -lm
 */
#include <math.h>
#include <stdint.h>

void oracle_nf4_encode(const float *w, const float *absmax, int64_t count, const float *levels,
                       uint8_t *codes) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < count; ++i) {
    const float a = absmax[i / 64];
    if (a == 0.0f) {
      codes[i] = 7;
      continue;
    }
    const float v = w[i] / a;
    int best = 0;
    double best_d = fabs((double)v - (double)levels[0]);
    for (int j = 1; j < 16; ++j) {
      const double d = fabs((double)v - (double)levels[j]);
      if (d < best_d) {
        best_d = d;
        best = j;
      }
    }
    codes[i] = (uint8_t)best;
  }
}

// Device-side helpers shared by the HIP kernels of the NF4 QLoRA library (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nf4q {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// The NF4 levels and their decision thresholds, passed by value as a kernel argument.
struct Tables {
  float level[16];
  float thresh[15];
};

// Weight descriptor as the kernels see it.
struct WDesc {
  const uint8_t *codes;   // [n*k/2]
  const void *absmax;     // float[nblk] (dq == 0) or int8[nblk]
  const float *scale;     // [ceil(nblk/256)] when dq
  int64_t n, k;
  int dq;                 // 0 or 1 (runs of 256)
  int fp4;                // 1: E2M1 codes, absmax = uint8 E4M3 scale per group of 16,
                          //    scale = float[1] tensor scale (see fp4.hip)
};

// Two floats -> packed bf16 pair (low half = lo), round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Block constant a' of flattened block index b.
__device__ __forceinline__ float block_absmax(const WDesc &w, int64_t b) {
  if (w.dq) {
    const int8_t q = reinterpret_cast<const int8_t *>(w.absmax)[b];
    return float(q) * w.scale[b >> 8];
  }
  return reinterpret_cast<const float *>(w.absmax)[b];
}

// Buffer resource over [p, p + bytes): loads past the end return 0 (raw buffer, no stride).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint32_t bitsel(uint32_t m, uint32_t a, uint32_t b) {
  return (m & a) | (~m & b);
}

// NF4 decode table of one 64-element block: the 16 values bf16(level_i * a) split into byte
// planes L (low bytes) and H (high bytes), four entries per 32-bit word.
// The int8 block code of the double quantisation (low byte of q) as a float. Written as
// (low 7 bits) - (sign bit) rather than a sign-extending cast: the cast lets the compiler fold
// the extension into the byte load and then move that load next to this use, after the waits
// of the software pipeline, so it stalls on memory.
__device__ __forceinline__ float int8_code(uint32_t q) {
  return float(q & 0x7Fu) - float(q & 0x80u);
}

struct RowTable {
  uint32_t L[4], H[4];
};

__device__ __forceinline__ RowTable make_row_table(float a, const Tables &t) {
  uint32_t pk[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pk[j] = pack_bf16x2(t.level[2 * j] * a, t.level[2 * j + 1] * a);
  RowTable r;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    r.L[q] = perm(pk[2 * q + 1], pk[2 * q], 0x06040200u);
    r.H[q] = perm(pk[2 * q + 1], pk[2 * q], 0x07050301u);
  }
  return r;
}

// Look up 4 codes at once: s7 = the codes' low 3 bits (one per byte), m = 0xFF bytes where the
// code is >= 8. Returns the table's low (L) or high (H) bytes of the 4 entries.
__device__ __forceinline__ uint32_t lookup4(const uint32_t P[4], uint32_t s7, uint32_t m) {
  return bitsel(m, perm(P[3], P[2], s7), perm(P[1], P[0], s7));
}

// Decode one 32-bit word of packed codes (8 elements; byte b = element 2b in bits 7..4 and
// element 2b+1 in bits 3..0) into 4 words of bf16 pairs in element order.
__device__ __forceinline__ void decode8(const RowTable &t, uint32_t d, uint32_t out[4]) {
  const uint32_t se7 = (d >> 4) & 0x07070707u;                             // even elements
  const uint32_t so7 = d & 0x07070707u;                                    // odd elements
  const uint32_t me = perm(0u, 0u, ((d >> 7) & 0x01010101u) | 0x0C0C0C0Cu); // bit 3 of even codes
  const uint32_t mo = perm(0u, 0u, ((d >> 3) & 0x01010101u) | 0x0C0C0C0Cu); // bit 3 of odd codes
  const uint32_t Le = lookup4(t.L, se7, me), He = lookup4(t.H, se7, me);
  const uint32_t Lo = lookup4(t.L, so7, mo), Ho = lookup4(t.H, so7, mo);
  const uint32_t E01 = perm(He, Le, 0x05010400u), E23 = perm(He, Le, 0x07030602u);
  const uint32_t O01 = perm(Ho, Lo, 0x05010400u), O23 = perm(Ho, Lo, 0x07030602u);
  out[0] = perm(O01, E01, 0x05040100u);
  out[1] = perm(O01, E01, 0x07060302u);
  out[2] = perm(O23, E23, 0x05040100u);
  out[3] = perm(O23, E23, 0x07060302u);
}

// decode8 split into five pieces of about six VALU instructions each, so the decode of a chunk
// can be spread between MFMA issues. The select masks come from byte permutes of (mhi, mlo) by
// selector bytes 0 / 4 (bit 3 of the code clear / set): (0xFFFFFFFF, 0) gives 0xFF where the code
// is >= 8 (the table's upper half sits in L[2..3], H[2..3]); (0, 0xFFFFFFFF) gives the complement,
// for a table whose halves are stored the other way round.
struct Dec8 {
  uint32_t d, se7, so7, me, mo, Le, He, Lo, Ho, E01, E23;
};

__device__ __forceinline__ void dec_piece(const RowTable &t, Dec8 &x, int piece, uint32_t out[4],
                                          uint32_t mhi, uint32_t mlo) {
  switch (piece) {
    case 0:
      x.se7 = (x.d >> 4) & 0x07070707u;
      x.so7 = x.d & 0x07070707u;
      x.me = perm(mhi, mlo, (x.d >> 5) & 0x04040404u);
      break;
    case 1:
      x.mo = perm(mhi, mlo, (x.d >> 1) & 0x04040404u);
      x.Le = lookup4(t.L, x.se7, x.me);
      break;
    case 2:
      x.He = lookup4(t.H, x.se7, x.me);
      x.Lo = lookup4(t.L, x.so7, x.mo);
      break;
    case 3:
      x.Ho = lookup4(t.H, x.so7, x.mo);
      x.E01 = perm(x.He, x.Le, 0x05010400u);
      x.E23 = perm(x.He, x.Le, 0x07030602u);
      break;
    default: {
      const uint32_t O01 = perm(x.Ho, x.Lo, 0x05010400u), O23 = perm(x.Ho, x.Lo, 0x07030602u);
      out[0] = perm(O01, x.E01, 0x05040100u);
      out[1] = perm(O01, x.E01, 0x07060302u);
      out[2] = perm(O23, x.E23, 0x05040100u);
      out[3] = perm(O23, x.E23, 0x07060302u);
    }
  }
}

// ---- 4-bit float (E2M1) weights with FP8 (E4M3) group scales --------------------------------
// Value of a non-negative E4M3 byte (bias 7, exponent field 0 subnormal: m * 2^-9). The sign bit
// is ignored (group scales are never negative).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  const uint32_t e = (b >> 3) & 15u;
  return e ? __uint_as_float(((b & 0x7Fu) << 20) + (120u << 23)) : float(b & 7u) * 0x1p-9f;
}

// Decode table of one group of 16: the 8 magnitudes bf16(e2m1[i] * s), i = 0..7, as byte planes
// (L[0..1] low bytes, H[0..1] high bytes, four entries per word). The products are exact (at most
// 6 significant bits), so the bf16 conversion does not round. The sign (code bit 3) is not in the
// table: decode_e2m1 sets the bf16 sign bit from the code. L[2..3], H[2..3] are unused.
__device__ __forceinline__ RowTable make_e2m1_table(float s) {
  const uint32_t p0 = pack_bf16x2(0.f, 0.5f * s), p1 = pack_bf16x2(s, 1.5f * s);
  const uint32_t p2 = pack_bf16x2(2.f * s, 3.f * s), p3 = pack_bf16x2(4.f * s, 6.f * s);
  RowTable r;
  r.L[0] = perm(p1, p0, 0x06040200u);
  r.H[0] = perm(p1, p0, 0x07050301u);
  r.L[1] = perm(p3, p2, 0x06040200u);
  r.H[1] = perm(p3, p2, 0x07050301u);
  r.L[2] = r.L[3] = r.H[2] = r.H[3] = 0u;
  return r;
}

// decode8 / dec_piece for E2M1 codes (same five-piece split and output order): one byte permute
// per plane looks up the magnitude of 4 codes at once (3-bit index into 8 bytes), and the code's
// sign bit is moved onto bit 7 of the high byte (the bf16 sign): bit 7 of each code byte for the
// even elements, bit 3 (shifted left by 4) for the odd ones.
__device__ __forceinline__ void dec_piece_e2m1(const RowTable &t, Dec8 &x, int piece, uint32_t out[4]) {
  switch (piece) {
    case 0:
      x.se7 = (x.d >> 4) & 0x07070707u;
      x.so7 = x.d & 0x07070707u;
      break;
    case 1:
      x.Le = perm(t.L[1], t.L[0], x.se7);
      x.He = perm(t.H[1], t.H[0], x.se7) | (x.d & 0x80808080u);
      break;
    case 2:
      x.Lo = perm(t.L[1], t.L[0], x.so7);
      x.Ho = perm(t.H[1], t.H[0], x.so7) | ((x.d << 4) & 0x80808080u);
      break;
    case 3:
      x.E01 = perm(x.He, x.Le, 0x05010400u);
      x.E23 = perm(x.He, x.Le, 0x07030602u);
      break;
    default: {
      const uint32_t O01 = perm(x.Ho, x.Lo, 0x05010400u), O23 = perm(x.Ho, x.Lo, 0x07030602u);
      out[0] = perm(O01, x.E01, 0x05040100u);
      out[1] = perm(O01, x.E01, 0x07060302u);
      out[2] = perm(O23, x.E23, 0x05040100u);
      out[3] = perm(O23, x.E23, 0x07060302u);
    }
  }
}

__device__ __forceinline__ void decode8_e2m1(const RowTable &t, uint32_t d, uint32_t out[4]) {
  Dec8 x;
  x.d = d;
#pragma unroll
  for (int p = 0; p < 5; ++p) dec_piece_e2m1(t, x, p, out);
}

// Value of v in lane l ^ 1 (DPP quad permutation 1, 0, 3, 2).
__device__ __forceinline__ uint32_t swap_adjacent_lanes(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
}
// Value of v in lane l ^ 8 within each row of 16 lanes (DPP row rotation by 8).
__device__ __forceinline__ uint32_t swap_lane_octets(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x128, 0xF, 0xF, true);
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

}  // namespace nf4q

// Device helpers shared by the QKV-quant kernel, the packed-K/V attention kernel
// and the test kernels: vector types, bf16/f16 conversions, the 128-point Hadamard
// butterfly and the group quantiser/packer, all working on one register layout.
//
// The "column layout" used throughout is the output layout of a 32x32 MFMA block
// as seen from one head: 128 values of one vector (one token's head, or one
// query's output) are spread over a lane pair (lane, lane ^ 32) and four 32-row
// blocks.  Lane L holds, in u[b][i] (b = 0..3, i = 0..15), element
//     e(b, i, L) = 32 b + 8 (i >> 2) + 4 (L >> 5) + (i & 3)
// of the vector whose index is L & 31 within the block of 32 vectors.  Element
// bits 0-1 and 3-4 are register bits, bit 2 is the lane-pair bit, and bits 5-6
// are the block index, so every 128-point transform or 32-value group reduction
// needs at most one exchange with lane ^ 32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace sqg {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kHeadDim = 128;
constexpr int kGroup = 32;
// word 3 of a raw buffer resource descriptor on gfx9-family GPUs (32-bit data format)
constexpr int kBufferWord3 = 0x00020000;
// 1/sqrt(128) rounded to fp32
constexpr float kInvSqrtHeadDim = 0.0883883461356163f;


// ----------------------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp32 -> fp16 bits, IEEE round to nearest even (v_cvt_f16_f32 in the default mode)
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

// v / sqrt(128) rounded to fp32 through one fp64 product: for exactly representable
// Hadamard outputs (integer inputs) this rounds like the fp64 definition r = fp32(u H / sqrt(128))
__device__ __forceinline__ float scale_inv_sqrt128(float v) {
  return (float)((double)v * 0.08838834764831845);
}

// value held by lane ^ 32
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32); }
__device__ __forceinline__ uint32_t xor32u(uint32_t v) { return (uint32_t)__shfl_xor((int)v, 32); }

__device__ __forceinline__ bool upper_half() { return (threadIdx.x & 32) != 0; }

// ----------------------------------------------------------------------------- Hadamard
// Unnormalised 128-point Walsh-Hadamard transform (Sylvester / natural order) of the
// vector held in column layout: out[e] = sum_j (-1)^popcount(e & j) in[j].
// Six butterfly stages are register-local, one crosses the lane pair.
__device__ __forceinline__ void fwht128_cols(float (&u)[4][16]) {
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int bit = 1; bit < 16; bit <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i & bit) continue;
        float x = u[b][i], y = u[b][i | bit];
        u[b][i] = x + y;
        u[b][i | bit] = x - y;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float x0 = u[0][i], x1 = u[1][i], x2 = u[2][i], x3 = u[3][i];
    float s01 = x0 + x1, d01 = x0 - x1, s23 = x2 + x3, d23 = x2 - x3;
    u[0][i] = s01 + s23;
    u[1][i] = d01 + d23;
    u[2][i] = s01 - s23;
    u[3][i] = d01 - d23;
  }
  const bool hi = upper_half();
#pragma unroll
  for (int b = 0; b < 4; ++b) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float p = xor32(u[b][i]);
      u[b][i] = hi ? (p - u[b][i]) : (u[b][i] + p);
    }
  }
}

// ----------------------------------------------------------------------------- quantise + pack
// The group scales of the two integer formats, from a group's fp32 absmax a:
//   INT4: a / 7 (IEEE fp32 division) rounded UP to 8 significant bits, stored as fp16
//     (exact).  Three code bits plus eight scale bits fit fp16's eleven, so the
//     attention kernel's f16 decode code * scale is exact for INT4 tiles; the round-up
//     enlarges the step by less than 2^-7, the page's own enlargement of its int8 scale.
//   INT8: VRAM Lab page, kvi8r section (`_Int8KV.store`): a * fp32((1 + 2^-7) / 127) in
//     fp32, rounded to nearest fp16.  The enlargement keeps |r / s| below 127 whatever
//     the fp16 rounding does.
constexpr float kInt8ScaleFactor = 0x1.04081p-7f;   // fp32((1 + 2^-7) / 127)

template <int FMT>
__device__ __forceinline__ uint32_t group_scale_bits(float a) {
  if (FMT == FMT_INT4) {
    uint32_t t = __float_as_uint(a / 7.0f);
    constexpr uint32_t kMask = (1u << (24 - 8)) - 1u;
    if (t & kMask) t = (t | kMask) + 1u;
    return f32_to_f16_bits(__uint_as_float(t));
  }
  // the product is rounded to fp32 first: the barrier keeps the compiler from fusing
  // multiply and conversion into one mixed-precision FMA, which rounds once (to f16)
  // and differs from the rule where the fp32 rounding moves a value across an f16 tie
  float t = __fmul_rn(a, kInt8ScaleFactor);
  asm volatile("" : "+v"(t));
  return f32_to_f16_bits(t);
}

// Group quantisation of one rotated 128-vector per lane pair (column layout), then
// packing and storing its codes and scales.  Group g is block b = g.
//   a = max |r| over the 32 values; s = group_scale_bits<FMT>(a) (fp16);
//   code = 0 if s == 0, else clamp(rne(r / fp32(s)), -qmax, qmax)
// INT4 rows are 64 bytes (code 2i in the low nibble of byte i), INT8 rows 128 bytes.
// `row` points at the vector's code row, `scales` at its 4 fp16 scales; only lanes
// with `valid` store.  All lanes must execute this function (lane-pair exchanges).
template <int FMT>
__device__ __forceinline__ void quant_pack_store(const float (&r)[4][16], uint8_t* row,
                                                 uint16_t* scales, bool valid) {
  constexpr float qmax = (FMT == FMT_INT4) ? 7.0f : 127.0f;
  const bool hi = upper_half();
  uint32_t sbits[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fmaxf(a, fabsf(r[b][i]));
    a = fmaxf(a, xor32(a));
    sbits[b] = group_scale_bits<FMT>(a);
    const float s = f16_bits_to_f32(sbits[b]);
    int c[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float t = (s == 0.0f) ? 0.0f : rintf(r[b][i] / s);
      t = fminf(fmaxf(t, -qmax), qmax);
      c[i] = (int)t;
    }
    if (FMT == FMT_INT4) {
      // halfword q holds elements 8q + 4h + {0..3}: byte offset 4q + 2h of the block's 16
      uint32_t hw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        hw[q] = (uint32_t)(c[4 * q] & 15) | ((uint32_t)(c[4 * q + 1] & 15) << 4) |
                ((uint32_t)(c[4 * q + 2] & 15) << 8) | ((uint32_t)(c[4 * q + 3] & 15) << 12);
      }
      // the lower lane keeps words 0,1 of the block, the upper lane words 2,3
      const uint32_t send = hi ? (hw[0] | (hw[1] << 16)) : (hw[2] | (hw[3] << 16));
      const uint32_t recv = xor32u(send);
      u32x2 out;
      if (!hi) {
        out[0] = hw[0] | ((recv & 0xffffu) << 16);
        out[1] = hw[1] | (recv & 0xffff0000u);
      } else {
        out[0] = (recv & 0xffffu) | (hw[2] << 16);
        out[1] = (recv >> 16) | (hw[3] << 16);
      }
      if (valid) *reinterpret_cast<u32x2*>(row + 16 * b + 8 * (hi ? 1 : 0)) = out;
    } else {
      // word q holds elements 8q + 4h + {0..3}: byte offset 8q + 4h of the block's 32
      uint32_t w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        w[q] = (uint32_t)(c[4 * q] & 255) | ((uint32_t)(c[4 * q + 1] & 255) << 8) |
               ((uint32_t)(c[4 * q + 2] & 255) << 16) | ((uint32_t)(c[4 * q + 3] & 255) << 24);
      }
      // the lower lane stores bytes 0-15 (words q = 0, 1), the upper lane bytes 16-31
      const uint32_t s0 = hi ? w[0] : w[2];
      const uint32_t s1 = hi ? w[1] : w[3];
      const uint32_t r0 = xor32u(s0);
      const uint32_t r1 = xor32u(s1);
      u32x4 out;
      if (!hi) {
        out[0] = w[0]; out[1] = r0; out[2] = w[1]; out[3] = r1;
      } else {
        out[0] = r0; out[1] = w[2]; out[2] = r1; out[3] = w[3];
      }
      if (valid) *reinterpret_cast<u32x4*>(row + 32 * b + 16 * (hi ? 1 : 0)) = out;
    }
  }
  if (valid && !hi) {
    u32x2 sv;
    sv[0] = sbits[0] | (sbits[1] << 16);
    sv[1] = sbits[2] | (sbits[3] << 16);
    *reinterpret_cast<u32x2*>(scales) = sv;
  }
}

// Format, row bytes and first byte of head h's rows in segment sg (see SegTable):
// an INT4 segment's INT8 heads take 64 bytes more per row than the others.
__device__ __forceinline__ int head_format(const SegTable& t, int sg, int h) {
  return (t.fmt[sg] == FMT_INT4 && ((t.int8_heads[sg] >> h) & 1ull)) ? FMT_INT8 : t.fmt[sg];
}
__device__ __forceinline__ int format_row_bytes(int fmt) {
  return fmt == FMT_INT4 ? 64 : (fmt == FMT_INT8 ? 128 : 256);
}
__device__ __forceinline__ int64_t head_rows_offset(const SegTable& t, int sg, int h) {
  int64_t units = (int64_t)format_row_bytes(t.fmt[sg]) * h;
  const uint64_t below = t.int8_heads[sg] & ((1ull << h) - 1ull);
  units += 64 * (int64_t)__popcll(below);
  return t.offset[sg] + (t.end[sg] - t.begin[sg]) * units;
}

// One rotated 128-vector per lane pair (column layout) rounded to bf16 (RNE) and
// stored as 128 consecutive bf16 values; the group scales of such a row are zero.
__device__ __forceinline__ void bf16_row_store(const float (&r)[4][16], uint8_t* row,
                                               uint16_t* scales, bool valid) {
  const int h4 = upper_half() ? 4 : 0;
  if (!valid) return;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x2 v;
      v[0] = f32_to_bf16_bits(r[b][4 * q]) | (f32_to_bf16_bits(r[b][4 * q + 1]) << 16);
      v[1] = f32_to_bf16_bits(r[b][4 * q + 2]) | (f32_to_bf16_bits(r[b][4 * q + 3]) << 16);
      *reinterpret_cast<u32x2*>(row + 2 * (32 * b + 8 * q + h4)) = v;
    }
  if (!upper_half()) {
    u32x2 z = {0u, 0u};
    *reinterpret_cast<u32x2*>(scales) = z;
  }
}

// segment of a token (the table is small and uniform across the wave)
__device__ __forceinline__ int find_segment(const SegTable& t, int64_t tok) {
  int s = 0;
  for (int k = 1; k < t.n; ++k)
    if (tok >= t.begin[k]) s = k;
  return s;
}

}  // namespace sqg

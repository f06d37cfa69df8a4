// Flash-style attention over a packed rotated INT4/INT8 K/V store, for gfx950.
//
// Feature request "Streamed QKV Projection and Packed Low-Bit K/V Support",
// sections "Proposed backend capability" and "Dense fallback is important":
// attention consumes Q in bf16 and K/V as packed low-bit codes, decoding K/V
// only tile by tile inside the kernel.  VRAM Lab page, kvi8r section
// (`_Int8KV`, `_blockwise_attention_q`, `_online_combine`): K/V stay in the
// orthonormal Hadamard basis; the query tile is rotated once, scores and P.V run
// in that basis (q.k = (qH).(kH), P.V = (P.(VH)).H^T), partial results combine by
// online softmax, and the output is rotated back once.  That page also measured
// that the rotated basis needs fp16 operands rather than bf16 (rotation spreads
// every value to the same magnitude), so both products use f16 MFMA with fp32
// accumulation.  Where softmax is sharp the scores need more than the 11 bits an
// f16 query carries, so the rotated query is split into an f16 high part and a
// remainder (about 2^-12 of it), and the scores are
//   S = K_f16 q_hi  (f16 MFMA)  +  K_6 q_lo6  (block-scaled fp6 MFMA)
// with K_6 and q_lo6 the keys and the remainder in fp6 E2M3 with one E8M0 exponent
// per group of 32 dims (the store's quantisation groups).  The fp6 product runs at
// four times the f16 rate and carries the remainder to ~2^-4, so the scores keep
// ~16 bits for 1/8 more matrix work instead of 1/2.  INT4 keys are exact in f16 (the
// store's INT4 scales have 8 significant bits); INT8 keys are not (kvi8r scales are
// full fp16), so INT8 tiles add K_lo q_hi with K_lo = code * scale - f16(code * scale),
// exact in f16.
//
// Workgroup: 256 queries of one head, eight waves of 32 queries (two waves per
// SIMD, so one wave's softmax and dequantisation overlap the other's MFMAs).
// Per 64-key tile the workgroup loads the packed codes and fp16 scales once (waves
// 0-3 the K codes, waves 4-7 the V codes: one 32-value group of one key per thread,
// one code load and one scale load), dequantises them to f16 in LDS (K and V both
// row-major; the P.V operands come out of LDS through transposing reads), and
// every wave computes
//   S^T = K_r Q_r^T        (keys x queries, 32x32x16 f16 MFMA)
//   online softmax down each query column (one lane-pair exchange per tile)
//   O^T += V_r^T P^T       (dims x queries)
// The transposed products keep a query's scores and its 128 output values in one
// lane pair, so the softmax statistics and the final inverse rotation are
// register-local apart from one exchange with lane ^ 32 (v_permlane32_swap inside
// the loop).  The query is prescaled by softmax scale * log2(e) before the split, and
// each tile's score accumulators start at minus the running reference maximum, so the
// MFMAs deliver the exponent of P = exp2(S) directly.  The query's f16 high part stays
// in registers and its fp6 remainder in LDS (one copy per wave).  QK^T and P.V read
// their LDS fragments one MFMA group ahead, with scheduling fences between the groups
// so that the compiler cannot sink a read next to the MFMA that consumes it.  The
// running maximum is only moved (and O rescaled) when a column's maximum grows by more
// than 2^8, so most tiles skip the rescale; P then stays below 256, well inside f16.
// One launch walks every key of the call: continuing (m, l, O) across a key-block
// boundary is the log-sum-exp merge of the blocks (VRAM Lab page, kvi8r section,
// `_online_combine`), so KV blocking costs nothing here.
#include "device_common.h"
#include "internal.h"

namespace sqg {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBQ = 32 * kWaves;      // queries per workgroup
constexpr int kBKV = 64;              // keys per tile
constexpr int kKB = kBKV / 32;        // 32-key MFMA blocks per tile
constexpr int kKStride = 128 + 8;     // f16 per K row in LDS (272 B)
constexpr int kKTile = kBKV * kKStride;
// V rows: 160 f16 per key (80 dwords: consecutive keys start 16 banks apart), and dim
// bits 3-4 XORed with bits 0-1 of the key, so that the decode's 16-byte row writes (4
// keys x 4 groups per 16-lane phase) and the transposing 8-byte reads (8 keys x 16
// dims per instruction) each fall in distinct banks of the 64-bank LDS.
constexpr int kVStride = kHeadDim + 32;
constexpr int kVTile = kBKV * kVStride;
__device__ __forceinline__ int vcol(int k, int d) { return d ^ ((k & 3) << 3); }
constexpr float kRescaleLog2 = 8.0f;  // move the running max only past this growth


// 8 f16 values code * scale from 8 INT4 codes (one dword, code j in bits 4j..4j+3)
__device__ __forceinline__ void dequant_int4x8(uint32_t w, uint32_t s2, uint32_t (&out)[4]) {
  const uint32_t b = w ^ 0x88888888u;          // nibble = code + 8
  const uint32_t lo = b & 0x0f0f0f0fu;         // codes 0, 2, 4, 6 in bytes 0..3
  const uint32_t hi = (b >> 4) & 0x0f0f0f0fu;  // codes 1, 3, 5, 7
  const f16x2 bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const f16x2 sc = __builtin_bit_cast(f16x2, s2);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    // f16 bit pattern 0x6400 | u is 1024 + u exactly
    const uint32_t sel = (uint32_t)p | 0x0c00u | ((uint32_t)(4 + p) << 16) | 0x0c000000u;
    const uint32_t pr = __builtin_amdgcn_perm(hi, lo, sel) | 0x64006400u;
    f16x2 v = __builtin_bit_cast(f16x2, pr) + bias;  // exact code
    v = v * sc;                                       // exact: the scale has few bits
    out[p] = __builtin_bit_cast(uint32_t, v);
  }
}

// Transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane c
// supplies the address of 4 consecutive f16 values (chunk c) and lane i receives
// element i % 4 of chunks i / 4 + 4 j, j = 0..3.
__device__ __forceinline__ f16x4 tr_read_f16x4(const _Float16* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)p);
  return __builtin_bit_cast(f16x4, r);
}

// two bf16 values (one dword) as two f16 values, each rounded to nearest
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w) {
  const f16x2 h = {(_Float16)__uint_as_float(w << 16), (_Float16)__uint_as_float(w & 0xffff0000u)};
  return __builtin_bit_cast(uint32_t, h);
}

// 4 f16 values code * scale from 4 INT8 codes (one dword, code j in byte j)
__device__ __forceinline__ void dequant_int8x4(uint32_t w, uint32_t s2, uint32_t (&out)[2]) {
  const uint32_t b = w ^ 0x80808080u;  // byte = code + 128
  const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 sc = __builtin_bit_cast(f16x2, s2);
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t sel = (uint32_t)(2 * p) | 0x0c00u | ((uint32_t)(2 * p + 1) << 16) | 0x0c000000u;
    const uint32_t pr = __builtin_amdgcn_perm(0u, b, sel) | 0x64006400u;
    f16x2 v = __builtin_bit_cast(f16x2, pr) + bias;
    v = v * sc;
    out[p] = __builtin_bit_cast(uint32_t, v);
  }
}

// The remainders code * scale - f16(code * scale) of 4 INT8 codes (one dword, code j in
// byte j), as 4 f16 values: code * scale has at most 7 + 11 significant bits, so it is
// exact in fp32 and its remainder after the f16 rounding is exact in f16 (outside the
// f16 subnormal range)
__device__ __forceinline__ void dequant_int8x4_rem(uint32_t w, uint32_t s2, uint32_t (&out)[2]) {
  const uint32_t b = w ^ 0x80808080u;
  const f16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const f16x2 sc = __builtin_bit_cast(f16x2, s2);
  const float sf = (float)sc[0];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t sel = (uint32_t)(2 * p) | 0x0c00u | ((uint32_t)(2 * p + 1) << 16) | 0x0c000000u;
    const uint32_t pr = __builtin_amdgcn_perm(0u, b, sel) | 0x64006400u;
    const f16x2 c = __builtin_bit_cast(f16x2, pr) + bias;   // exact codes
    const f16x2 v = c * sc;                                  // as stored in the K tile
    const f16x2 r = {(_Float16)((float)c[0] * sf - (float)v[0]), (_Float16)((float)c[1] * sf - (float)v[1])};
    out[p] = __builtin_bit_cast(uint32_t, r);
  }
}

// E8M0 exponent for fp6 E2M3 values (largest magnitude 7.5): the smallest e with
// a <= 7.5 * 2^e for a finite a >= 0 (a = 1.m * 2^E: e = E - 2 if 1.m <= 1.875, else
// E - 1), clamped to [-126, 127] so that 2^e is a normal fp32 scale.
__device__ __forceinline__ int fp6_exponent(float a) {
  const uint32_t b = __float_as_uint(a);
  const int e = (int)(b >> 23) - 129 + ((b & 0x7fffffu) > 0x700000u ? 1 : 0);
  return e < -126 ? -126 : (e > 127 ? 127 : e);
}
__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

typedef _Float16 f16x32 __attribute__((ext_vector_type(32)));
typedef uint32_t u32x6 __attribute__((ext_vector_type(6)));

// 32 f16 values as fp6 E2M3 codes of value / 2^e (round to nearest even, value i in
// bits 6i .. 6i + 5 of the six dwords)
__device__ __forceinline__ u32x6 to_fp6(const f16x32 v, int e) {
  return __builtin_amdgcn_cvt_scalef32_pk32_fp6_f16(v, pow2f(e));
}

// Packed codes and the group scale one thread moves per tile: 32 values of one key
// (16 B INT4 in c0, 32 B INT8 in c0, c1); BF16 tiles are read later, in store_tile,
// from the tile's byte offset crow.
struct TileRegs {
  u32x4 c0, c1;
  uint32_t scale;
  int fmt;
  uint32_t crow;
};

// E8M0 exponent of a block whose largest magnitude is a (a finite fp32 >= 0): the
// smallest e with a <= 448 * 2^e, from the bit pattern (a = 1.m * 2^(ef - 127), and
// 448 = 1.75 * 2^8), clamped to [-127, 127]; -127 for a zero block.
__device__ __forceinline__ int e8m0_exponent(float a) {
  const uint32_t b = __float_as_uint(a);
  if (a <= 0.0f) return -127;
  const int e = (int)(b >> 23) - 135 + ((b & 0x7fffffu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef short s16x2 __attribute__((ext_vector_type(2)));

// fp8 K rows in LDS: 128 codes of one key, dim d at byte swap(bits 3, 4 of d) so that
// a lane's 16-byte halves of a 64-dim chunk are the dims the scaled MFMA pairs with
// the query bytes held in registers (see the QK^T step)
constexpr int kK8Stride = 128 + 16;
// fp6 K rows in LDS: the four groups of one key, 24 bytes each (32 E2M3 codes in
// dim order), then 24 bytes of padding: consecutive keys start 15 eight-byte slots
// apart, so the 32 keys of one 8-byte operand read fall in distinct bank pairs and
// the decode's writes conflict at most 2-way.
constexpr int kK6Stride = 120;

template <bool kFp8QK>
__global__ __launch_bounds__(kThreads, 1) void packed_attention_kernel(const AttnParams p) {
  __shared__ __attribute__((aligned(16))) _Float16 sK[2][kKTile];
  __shared__ __attribute__((aligned(16))) _Float16 sV[2][kVTile];
  // exact tier: the keys as fp6 for the remainder term, and the f16 remainders of INT8 keys
  __shared__ __attribute__((aligned(16))) uint8_t sK6[kFp8QK ? 1 : 2][kFp8QK ? 16 : kBKV * kK6Stride];
  __shared__ __attribute__((aligned(16))) _Float16 sKlo[kFp8QK ? 1 : 2][kFp8QK ? 8 : kKTile];
  // exact tier: each wave's fp6 query remainder, [chunk][lane][6 dwords]
  __shared__ __attribute__((aligned(16))) uint32_t sQ6[kFp8QK ? 1 : kWaves][kFp8QK ? 2 : 2 * 64 * 6];
  __shared__ uint32_t sKe[2][kBKV];   // the four E8M0 exponents of each key (byte g = group g)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l32 = lane & 31;
  const int hsel = lane >> 5;
  const int head = blockIdx.y;
  const int64_t N = p.n_tokens;

  // ---- query tile: rotate once, keep as MFMA B operands: f16 high part + remainder,
  // or (fp8 QK) E4M3 codes with one E8M0 exponent per group of 32 dims
  const int64_t qrow = p.q_begin + (int64_t)blockIdx.x * kBQ + 32 * wave + l32;
  const bool qvalid = qrow < p.q_end;
  f16x8 qf[8];
  i32x8 q8[2];        // fp8 tier: the E4M3 query (the exact tier keeps its fp6 remainder in LDS)
  uint32_t q8e[2];    // the E8M0 exponent byte this lane supplies for each 64-dim chunk
  {
    const uint16_t* src = p.q + ((qvalid ? qrow : p.q_begin) - p.q_row0) * p.ldq + head * kHeadDim + 8 * hsel;
    // element e(ks, j) = 16 ks + 8 hsel + j: bits 0-2 = j, bit 3 = lane pair, bits 4-6 = ks.
    // The fp8 tier quantises the rotated query, so there the transform runs in fp64:
    // the sum of 128 bf16 values is then exact and one fp64 product rounded to fp32
    // gives the correctly rounded rotated value, on which the quantiser decides.
    float v[8][8];
    if constexpr (kFp8QK) {
      double w[8][8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qvalid) raw = *reinterpret_cast<const u32x4*>(src + 16 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          w[ks][2 * j] = (double)bf16_lo(raw[j]);
          w[ks][2 * j + 1] = (double)bf16_hi(raw[j]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j & bit) continue;
            const double x = w[ks][j], y = w[ks][j | bit];
            w[ks][j] = x + y;
            w[ks][j | bit] = x - y;
          }
#pragma unroll
      for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks & bit) continue;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const double x = w[ks][j], y = w[ks | bit][j];
            w[ks][j] = x + y;
            w[ks | bit][j] = x - y;
          }
        }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint64_t b = __builtin_bit_cast(uint64_t, w[ks][j]);
          const uint64_t pb = (uint64_t)xor32u((uint32_t)b) | ((uint64_t)xor32u((uint32_t)(b >> 32)) << 32);
          const double pr = __builtin_bit_cast(double, pb);
          v[ks][j] = (float)((hsel ? (pr - w[ks][j]) : (w[ks][j] + pr)) * 0.08838834764831845);
        }
    } else {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qvalid) raw = *reinterpret_cast<const u32x4*>(src + 16 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          v[ks][2 * j] = bf16_lo(raw[j]);
          v[ks][2 * j + 1] = bf16_hi(raw[j]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            if (j & bit) continue;
            const float x = v[ks][j], y = v[ks][j | bit];
            v[ks][j] = x + y;
            v[ks][j | bit] = x - y;
          }
#pragma unroll
      for (int bit = 1; bit < 8; bit <<= 1)
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          if (ks & bit) continue;
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = v[ks][j], y = v[ks | bit][j];
            v[ks][j] = x + y;
            v[ks | bit][j] = x - y;
          }
        }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float pr = xor32(v[ks][j]);
          v[ks][j] = (hsel ? (pr - v[ks][j]) : (v[ks][j] + pr)) * kInvSqrtHeadDim;
        }
    }
    if constexpr (!kFp8QK) {
      // the exact tier splits the query prescaled by softmax scale * log2(e), so its
      // scores come out of the MFMAs in the base-2 units of the softmax
      f16x8 ql[8];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) v[ks][j] *= p.scale_log2;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const _Float16 hi = (_Float16)v[ks][j];
          qf[ks][j] = hi;
          ql[ks][j] = (_Float16)(v[ks][j] - (float)hi);
        }
      // fp6 operand of the remainder: for chunk c (dims 64 c .. + 63) this lane supplies
      // group 2 c + hsel whole, 32 values in dim order.  It holds the half of that group
      // with dim bit 3 = hsel; the partner lane sends the other half.
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        f16x8 got[2];   // the partner's half of this lane's group, k-steps 4 c + 2 hsel + t
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const u32x4 snd = __builtin_bit_cast(u32x4, hsel ? ql[4 * c + t] : ql[4 * c + 2 + t]);
          u32x4 rcv;
#pragma unroll
          for (int k = 0; k < 4; ++k) rcv[k] = xor32u(snd[k]);
          got[t] = __builtin_bit_cast(f16x8, rcv);
        }
        f16x32 g;
        float amax = 0.0f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const f16x8 mine = hsel ? ql[4 * c + 2 + t] : ql[4 * c + t];
          const f16x8 lo8 = hsel ? got[t] : mine;   // dims 16 t + 0 .. 7 of the group
          const f16x8 hi8 = hsel ? mine : got[t];   // dims 16 t + 8 .. 15
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            g[16 * t + j] = lo8[j];
            g[16 * t + 8 + j] = hi8[j];
            amax = fmaxf(amax, fmaxf(fabsf((float)lo8[j]), fabsf((float)hi8[j])));
          }
        }
        const int e = fp6_exponent(amax);
        const u32x6 w6 = to_fp6(g, e);
        u32x2* q6 = reinterpret_cast<u32x2*>(&sQ6[wave][(c * 64 + lane) * 6]);
        q6[0] = u32x2{w6[0], w6[1]};
        q6[1] = u32x2{w6[2], w6[3]};
        q6[2] = u32x2{w6[4], w6[5]};
        q8e[c] = (uint32_t)(e + 127);
      }
    } else {
      // group g = dims 32 g .. + 31 = k-steps 2 g, 2 g + 1 of both lanes of the pair
      int eg[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float a = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fmaxf(fabsf(v[2 * g][j]), fabsf(v[2 * g + 1][j])));
        eg[g] = e8m0_exponent(fmaxf(a, xor32(a)));
      }
      // B operand of chunk c (dims 64 c .. + 63): byte b = element (k-step 4 c + b / 8, b % 8)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const int ks = 4 * c + kk;
          const int e = eg[ks >> 1];
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            int w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[ks][4 * h], -e), ldexpf(v[ks][4 * h + 1], -e), 0, false);
            w = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(v[ks][4 * h + 2], -e), ldexpf(v[ks][4 * h + 3], -e), w, true);
            q8[c][2 * kk + h] = w;
          }
        }
        q8e[c] = (uint32_t)(eg[2 * c + hsel] + 127);   // this lane supplies block hsel's exponent
      }
    }
  }

  // ---- per-thread maps for the K/V tile loads (64 keys per tile, 512 threads): waves
  // 0-3 bring K, waves 4-7 bring V; thread (key, grp) moves group grp (32 values) of one
  // key: one code load and one scale load per tile.
  const bool vside = wave >= kWaves / 2;   // wave-uniform
  const int tkey = (tid & 255) >> 2;
  const int tgrp = tid & 3;
  const uint32_t c_off4 = (uint32_t)(tkey * 64 + 16 * tgrp);
  const uint32_t c_off8 = (uint32_t)(tkey * 128 + 32 * tgrp);
  const uint32_t c_off16 = (uint32_t)(tkey * 256 + 64 * tgrp);
  const uint32_t s_off = (uint32_t)(2 * (tkey * 4 + tgrp));

  // Tile loads go through buffer resources that cover this head's rows of one
  // segment (codes) or of the whole sequence (scales); rows past the end read as
  // zero.  The load cursor below follows the segment of the next tile to load in
  // scalar registers, so a tile costs a few scalar adds and one vector add per base.
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((vside ? p.vscale : p.kscale) + (int64_t)head * p.kv_n * 4), 0, (int32_t)(p.kv_n * 8),
      kBufferWord3);
  const uint8_t* const cbase = vside ? p.vpack : p.kpack;
  int ld_seg = -1;
  int64_t ld_sb = 0, ld_se = 0;
  int ld_fmt = FMT_INT4;
  __amdgpu_buffer_rsrc_t cr = sr;
  auto load_tile = [&](int64_t key0, TileRegs& r) {
    while (key0 >= ld_se) {  // the tile starts a new segment (rare)
      ++ld_seg;
      ld_sb = p.seg.begin[ld_seg];
      ld_se = p.seg.end[ld_seg];
      ld_fmt = head_format(p.seg, ld_seg, head);
      const int64_t rb = format_row_bytes(ld_fmt);
      const int64_t base = head_rows_offset(p.seg, ld_seg, head);
      const int32_t bytes = (int32_t)((ld_se - ld_sb) * rb);
      cr = __builtin_amdgcn_make_buffer_rsrc((void*)(cbase + base), 0, bytes, kBufferWord3);
    }
    r.fmt = ld_fmt;
    r.scale = __builtin_amdgcn_raw_buffer_load_b16(sr, s_off + (uint32_t)((key0 - p.kv_row0) * 8), 0, 0);
    if (ld_fmt == FMT_INT4) {
      r.c0 = __builtin_amdgcn_raw_buffer_load_b128(cr, c_off4 + (uint32_t)((key0 - ld_sb) * 64), 0, 0);
    } else if (ld_fmt == FMT_INT8) {
      const uint32_t crow = (uint32_t)((key0 - ld_sb) * 128);
      r.c0 = __builtin_amdgcn_raw_buffer_load_b128(cr, c_off8 + crow, 0, 0);
      r.c1 = __builtin_amdgcn_raw_buffer_load_b128(cr, c_off8 + crow + 16, 0, 0);
    } else {
      r.crow = (uint32_t)((key0 - ld_sb) * 256);
    }
  };

  // decode one thread's 32 values into row tkey, elements 32 tgrp .. + 31, of the K or V
  // tile (both row-major: key rows of 128 dims)
  auto store_tile = [&](const TileRegs& r, int stage) {
    _Float16* dst = (vside ? sV[stage] : sK[stage]) + tkey * kKStride + 32 * tgrp;
    const int fmt = __builtin_amdgcn_readfirstlane(r.fmt);
    const uint32_t s2 = r.scale | (r.scale << 16);
    constexpr bool kSplit = !kFp8QK;   // exact tier: INT8 keys carry their f16 remainder
    uint32_t o[16];
    if (fmt == FMT_INT4) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t a[4];
        dequant_int4x8(r.c0[w], s2, a);
#pragma unroll
        for (int i = 0; i < 4; ++i) o[4 * w + i] = a[i];
      }
    } else if (fmt == FMT_INT8) {
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        uint32_t a[2];
        dequant_int8x4(w < 4 ? r.c0[w] : r.c1[w - 4], s2, a);
        o[2 * w] = a[0];
        o[2 * w + 1] = a[1];
      }
    } else {
      // bf16 rows, read now: bf16 -> fp32 is a shift, fp32 -> f16 rounds to nearest
      // (exact for the 8 significant bits of bf16 within f16's normal range)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(cr, c_off16 + r.crow + 16 * i, 0, 0);
#pragma unroll
        for (int w = 0; w < 4; ++w) o[4 * i + w] = bf16x2_to_f16x2(b[w]);
      }
    }
    if (kFp8QK && !vside) {
      // K as E4M3 codes of value / 2^e with e the group's E8M0 exponent; bytes of dims
      // 8..15 and 16..23 of the group trade places (the swap of dim bits 3 and 4).  The
      // codes are taken from the exact decoded value: INT4 and BF16 keys are exact in
      // f16, INT8 keys (code * scale, up to 18 significant bits) are formed in fp32.
      uint32_t w[8];
      int e;
      if (fmt != FMT_INT8) {
        f16x2 m2 = {(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
        for (int i = 0; i < 16; ++i) m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(__builtin_bit_cast(f16x2, o[i])));
        const float a = fmaxf((float)m2[0], (float)m2[1]);
        e = e8m0_exponent(a);
        const float sc = a > 0.0f ? ldexpf(1.0f, e) : 1.0f;
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          const s16x2 zero = {0, 0};
          s16x2 r2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(zero, __builtin_bit_cast(f16x2, o[2 * d]), sc, false);
          r2 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(r2, __builtin_bit_cast(f16x2, o[2 * d + 1]), sc, true);
          w[d] = __builtin_bit_cast(uint32_t, r2);
        }
      } else {
        const float sf = f16_bits_to_f32(r.scale & 0xffffu);
        float a = 0.0f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t cw = q < 4 ? r.c0[q] : r.c1[q - 4];
#pragma unroll
          for (int j = 0; j < 4; ++j) a = fmaxf(a, fabsf((float)(int8_t)(cw >> (8 * j)) * sf));
        }
        e = e8m0_exponent(a);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const uint32_t cw = q < 4 ? r.c0[q] : r.c1[q - 4];
          float v[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) v[j] = ldexpf((float)(int8_t)(cw >> (8 * j)) * sf, -e);
          int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
          x = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], x, true);
          w[q] = (uint32_t)x;
        }
      }
      uint8_t* k8 = reinterpret_cast<uint8_t*>(sK[stage]) + tkey * kK8Stride + 32 * tgrp;
      const u32x4 lo = {w[0], w[1], w[4], w[5]};
      const u32x4 hi = {w[2], w[3], w[6], w[7]};
      *reinterpret_cast<u32x4*>(k8) = lo;
      *reinterpret_cast<u32x4*>(k8 + 16) = hi;
      reinterpret_cast<uint8_t*>(sKe[stage])[4 * tkey + tgrp] = (uint8_t)(e + 127);
    } else if (vside) {
      _Float16* vrow = sV[stage] + tkey * kVStride;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = {o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
        *reinterpret_cast<u32x4*>(vrow + vcol(tkey, 32 * tgrp + 8 * i)) = v;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4 v = {o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
        *reinterpret_cast<u32x4*>(dst + 8 * i) = v;
      }
      if constexpr (kSplit) {
        // the group as fp6 for the remainder term; its exponent covers the group's
        // largest magnitude: 7 s (INT4) or 127 s (INT8) from the scale, else the values
        float amax;
        if (fmt == FMT_BF16) {
          f16x2 m2 = {(_Float16)0.0f, (_Float16)0.0f};
#pragma unroll
          for (int i = 0; i < 16; ++i) m2 = __builtin_elementwise_max(m2, __builtin_elementwise_abs(__builtin_bit_cast(f16x2, o[i])));
          amax = fmaxf((float)m2[0], (float)m2[1]);
        } else {
          amax = f16_bits_to_f32(r.scale & 0xffffu) * (fmt == FMT_INT4 ? 7.0f : 127.0f);
        }
        const int e = fp6_exponent(amax);
        f16x32 g;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const f16x2 h = __builtin_bit_cast(f16x2, o[i]);
          g[2 * i] = h[0];
          g[2 * i + 1] = h[1];
        }
        const u32x6 w6 = to_fp6(g, e);
        u32x2* k6 = reinterpret_cast<u32x2*>(sK6[stage] + tkey * kK6Stride + 24 * tgrp);
        k6[0] = u32x2{w6[0], w6[1]};
        k6[1] = u32x2{w6[2], w6[3]};
        k6[2] = u32x2{w6[4], w6[5]};
        reinterpret_cast<uint8_t*>(sKe[stage])[4 * tkey + tgrp] = (uint8_t)(e + 127);
        if (fmt == FMT_INT8) {
          // second pass over the codes: the f16 remainders of the INT8 keys
          _Float16* lrow = sKlo[stage] + tkey * kKStride + 32 * tgrp;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            uint32_t a[2], b[2];
            dequant_int8x4_rem(i < 2 ? r.c0[2 * i] : r.c1[2 * i - 4], s2, a);
            dequant_int8x4_rem(i < 2 ? r.c0[2 * i + 1] : r.c1[2 * i - 3], s2, b);
            const u32x4 v = {a[0], a[1], b[0], b[1]};
            *reinterpret_cast<u32x4*>(lrow + 8 * i) = v;
          }
        }
      }
    }
  };

  // ---- state
  f32x16 oacc[4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[a][e] = 0.0f;
  float m_run = -INFINITY;  // reference max of scale*log2e*score for this query column
  // exact tier: the score accumulators start at -m_ref (the reference max, 0 before the
  // first tile), so they come out as scale*log2e*score - m_ref and P = exp2(S) needs no
  // per-score arithmetic; a rescale moves m_ref with the running max
  float m_ref = 0.0f;
  f32x16 negm = {};
  float l_run = 0.0f;       // lane-partial sum of the f16 P values
  const float c = p.scale_log2;
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};

  const int64_t kv0 = p.kv_begin;
  const int n_tiles = (int)((p.kv_end - kv0 + kBKV - 1) / kBKV);
  TileRegs regs;
  load_tile(kv0, regs);
  store_tile(regs, 0);
  if (n_tiles > 1) load_tile(kv0 + kBKV, regs);
  __syncthreads();

  // Waves 0-3 and 4-7 share the four SIMDs (one of each per SIMD).  Between two
  // barriers both run the same four steps, rotated by one for the second group so
  // that on a SIMD one wave's MFMA step meets the other's VALU step:
  //   waves 0-3: QK(j)    SM(j)    PV(j)    DQ(j+1)
  //   waves 4-7: DQ(j+1)  QK(j)    SM(j)    PV(j)
  // (QK = scores, SM = softmax, PV = output update, DQ = dequantise the next tile
  // into the other LDS stage and start loading the one after.)
  const bool lead = wave < kWaves / 2;

  auto do_qk = [&](int stage, int kfmt, f32x16 (&s)[kKB]) {
    const _Float16* K = sK[stage];
    // Software pipeline over LDS: reads are issued in groups, each group one group of
    // MFMAs ahead of its use, with scheduling fences between the groups so that the
    // compiler cannot sink a read next to its MFMA (which would expose the LDS latency
    // at every MFMA).  Order: the fp6 remainder MFMAs (chunk c = 0, then 1), then the
    // 16 f16 MFMAs of the high part in groups of four.
    // fp6 remainder: lane (key, hsel) supplies group 2 c + hsel of its key and that
    // group's exponent; the query side comes from this wave's LDS copy
    auto k6_read = [&](int kb, int c) -> i32x8 {
      const uint8_t* row = sK6[stage] + (32 * kb + l32) * kK6Stride + 24 * hsel + 48 * c;
      const u32x2 a0 = *reinterpret_cast<const u32x2*>(row);
      const u32x2 a1 = *reinterpret_cast<const u32x2*>(row + 8);
      const u32x2 a2 = *reinterpret_cast<const u32x2*>(row + 16);
      return i32x8{(int)a0[0], (int)a0[1], (int)a1[0], (int)a1[1], (int)a2[0], (int)a2[1], 0, 0};
    };
    auto q6_read = [&](int c) -> i32x8 {
      const u32x2* q6 = reinterpret_cast<const u32x2*>(&sQ6[kFp8QK ? 0 : wave][(c * 64 + lane) * 6]);
      const u32x2 b0 = q6[0], b1 = q6[1], b2 = q6[2];
      return i32x8{(int)b0[0], (int)b0[1], (int)b1[0], (int)b1[1], (int)b2[0], (int)b2[1], 0, 0};
    };
    auto kf_read = [&](int i) -> f16x8 {   // fragment i: k-step i / 2, key block i % 2
      return *reinterpret_cast<const f16x8*>(K + (32 * (i & 1) + l32) * kKStride + 16 * (i >> 1) + 8 * hsel);
    };
    uint32_t ew[kKB];
    i32x8 A[kKB], B;
    f16x8 kf[16];
    // group: chunk-0 fp6 operands and the first four K fragments
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      ew[kb] = sKe[stage][32 * kb + l32];
      A[kb] = k6_read(kb, 0);
    }
    B = q6_read(0);
#pragma unroll
    for (int i = 0; i < 4; ++i) kf[i] = kf_read(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
      s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[kb], B, negm, 2, 2, 0,
                                                               (int)((ew[kb] >> (8 * hsel)) & 0xffu), 0, (int)q8e[0]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) A[kb] = k6_read(kb, 1);
    B = q6_read(1);
#pragma unroll
    for (int i = 4; i < 8; ++i) kf[i] = kf_read(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
      s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A[kb], B, s[kb], 2, 2, 0,
                                                               (int)((ew[kb] >> (8 * (2 + hsel))) & 0xffu), 0, (int)q8e[1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      if (g + 2 < 4) {
#pragma unroll
        for (int i = 4 * (g + 2); i < 4 * (g + 3); ++i) kf[i] = kf_read(i);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 4 * g; i < 4 * g + 4; ++i)
        s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf[i], qf[i >> 1], s[i & 1], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (kfmt == FMT_INT8) {
      const _Float16* Kl = sKlo[stage];
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb) {
          const f16x8 kf = *reinterpret_cast<const f16x8*>(Kl + (32 * kb + l32) * kKStride + 16 * ks + 8 * hsel);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[ks], s[kb], 0, 0, 0);
        }
      }
    }
  };

  // fp8 QK^T: per 32-key block and 64-dim chunk one block-scaled MFMA.  A lane's
  // operand bytes are k slots 16 hsel + b % 16 + 32 (b / 16); slot k carries dim k with
  // bits 3 and 4 swapped on both sides (the query bytes by construction, the key bytes
  // by their LDS order), so the MFMA's 32-slot scale blocks are exactly the groups.
  auto do_qk8 = [&](int stage, f32x16 (&s)[kKB]) {
    const uint8_t* K8 = reinterpret_cast<const uint8_t*>(sK[stage]);
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb) {
      const uint32_t ew = sKe[stage][32 * kb + l32];
      const uint8_t* row = K8 + (32 * kb + l32) * kK8Stride + 16 * hsel;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(row + 64 * c);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(row + 64 * c + 32);
        const i32x8 A = __builtin_bit_cast(i32x8, __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7));
        const int ea = (int)((ew >> (8 * (2 * c + hsel))) & 0xffu);
        const f32x16 acc = c == 0 ? f32x16{} : s[kb];
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A, q8[c], acc, 0, 0, 0, ea, 0, (int)q8e[c]);
      }
    }
  };

  auto do_softmax = [&](int64_t key0, f32x16 (&s)[kKB], f16x8 (&pf)[2 * kKB]) {
    if (key0 + kBKV > p.kv_end) {
      // keys past the end of the range: element e of block kb is key
      // key0 + 32 kb + 8 (e >> 2) + 4 hsel + (e & 3); compare its offset within the tile
      // (a literal) with one per-lane limit
      const int lim = (int)(p.kv_end - key0) - 4 * hsel;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (32 * kb + 8 * (e >> 2) + (e & 3) >= lim) s[kb][e] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      // the tile's largest scale*log2e*score (the exact tier's scores carry -m_ref)
      mx = kFp8QK ? mx * c : mx + m_ref;
    }
    if (__any(mx > m_run + kRescaleLog2)) {  // wave-uniform: move every column's max
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[db][e] *= alpha;
      if constexpr (!kFp8QK) {
        const float delta = m_new - m_ref;
        m_ref = m_new;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kb][e] -= delta;
#pragma unroll
        for (int e = 0; e < 16; ++e) negm[e] = -m_new;
      }
    }
#pragma unroll
    for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        const float p0 = __builtin_amdgcn_exp2f(kFp8QK ? s[kb][e] * c - m_run : s[kb][e]);
        const float p1 = __builtin_amdgcn_exp2f(kFp8QK ? s[kb][e + 1] * c - m_run : s[kb][e + 1]);
        const f16x2 h2 = {(_Float16)p0, (_Float16)p1};
        l_run = __builtin_amdgcn_fdot2(h2, ones, l_run, false);
        pf[2 * kb + (e >> 3)][e & 7] = h2[0];
        pf[2 * kb + (e >> 3)][(e & 7) + 1] = h2[1];
      }
  };

  // P.V: O^T += V^T P^T.  The V^T fragments of the first k-step are read by pv_begin
  // (called before the softmax, so their LDS latency hides behind it), the rest inside
  // do_pv, one k-step ahead of their MFMAs.
  const int pv_vk = 4 * hsel + ((lane & 15) >> 2);
  const int pv_vd = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  auto vf_read = [&](int stage, int ks, int db) -> f16x8 {
    // A operand (V^T) by transposing LDS reads: lane L gets dim 32 db + L % 32 of keys
    // 16 ks + 4 hsel + 0..3 and 16 ks + 8 + 4 hsel + 0..3 (the MFMA's k slots 8 hsel + e
    // with bits 2 and 3 swapped, matching the key order of the P operand).  Each 16-lane
    // group reads 4 keys x 16 dims: lane c points at key (c / 4), dims 4 (c % 4) .. + 3.
    // key k = 16 ks + 8 half + vk (vk = 4 hsel + (lane % 16) / 4), so bits 0-1 of k (the
    // column swizzle) are those of vk for every ks and half: one base per half, ks and
    // db as offsets
    const _Float16* V = sV[stage];
    const _Float16* vb0 = V + pv_vk * kVStride + vcol(pv_vk, pv_vd);
    const _Float16* vb1 = V + (pv_vk + 8) * kVStride + vcol(pv_vk + 8, pv_vd);
    const f16x4 lo = tr_read_f16x4(vb0 + 16 * ks * kVStride + 32 * db);
    const f16x4 hi = tr_read_f16x4(vb1 + 16 * ks * kVStride + 32 * db);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto pv_begin = [&](int stage, f16x8 (&vf0)[4]) {
#pragma unroll
    for (int db = 0; db < 4; ++db) vf0[db] = vf_read(stage, 0, db);
  };
  auto do_pv = [&](int stage, const f16x8 (&pf)[2 * kKB], const f16x8 (&vf0)[4]) {
    f16x8 vf[2 * kKB][4];
#pragma unroll
    for (int db = 0; db < 4; ++db) vf[0][db] = vf0[db];
#pragma unroll
    for (int ks = 0; ks < 2 * kKB; ++ks) {
      if (ks + 1 < 2 * kKB) {
#pragma unroll
        for (int db = 0; db < 4; ++db) vf[ks + 1][db] = vf_read(stage, ks + 1, db);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int db = 0; db < 4; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf[ks][db], pf[ks], oacc[db], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  auto do_dq = [&](int it) {   // dequantise tile it + 1, then start loading tile it + 2
    if (it + 1 < n_tiles) store_tile(regs, (it + 1) & 1);
    if (it + 2 < n_tiles) load_tile(kv0 + (int64_t)(it + 2) * kBKV, regs);
  };

  // format of the K tile being multiplied, followed in scalar registers (tiles never
  // straddle two segments: boundaries and kv_begin are multiples of 128)
  int qk_seg = -1;
  int64_t qk_se = 0;
  int qk_fmt = FMT_INT4;
  for (int it = 0; it < n_tiles; ++it) {
    const int stage = it & 1;
    const int64_t key0 = kv0 + (int64_t)it * kBKV;
    while (key0 >= qk_se) {
      ++qk_seg;
      qk_se = p.seg.end[qk_seg];
      qk_fmt = head_format(p.seg, qk_seg, head);
    }
    if (!lead) do_dq(it);
    f32x16 s[kKB];
    f16x8 pf[2 * kKB];
    if constexpr (kFp8QK)
      do_qk8(stage, s);
    else
      do_qk(stage, qk_fmt, s);
    f16x8 vf0[4];
    pv_begin(stage, vf0);
    do_softmax(key0, s, pf);
    do_pv(stage, pf, vf0);
    if (lead) do_dq(it);
    __syncthreads();
  }

  // ---- epilogue: normalise, rotate back, merge, store
  const float l_tot = l_run + xor32(l_run);
  const float inv = 1.0f / l_tot;
  float u[4][16];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) u[db][e] = oacc[db][e] * inv;
  fwht128_cols(u);
  float lse = (m_run + log2f(l_tot)) * 0.6931471805599453f;
  const int64_t rr = qvalid ? qrow : 0;
  if (p.accumulate) {
    const float* orow = reinterpret_cast<const float*>(p.o) + rr * p.ldo + head * kHeadDim + 4 * hsel;
    const float lse_old = p.lse[(int64_t)head * N + rr];
    const float mxl = fmaxf(lse_old, lse);
    const float lse_new = mxl + logf(expf(lse_old - mxl) + expf(lse - mxl));
    const float w_old = expf(lse_old - lse_new);
    const float w_new = expf(lse - lse_new) * kInvSqrtHeadDim;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 prev = {0.f, 0.f, 0.f, 0.f};
        if (qvalid) prev = *reinterpret_cast<const f32x4*>(orow + 32 * db + 8 * q);
#pragma unroll
        for (int j = 0; j < 4; ++j) u[db][4 * q + j] = prev[j] * w_old + u[db][4 * q + j] * w_new;
      }
    lse = lse_new;
  } else {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) u[db][e] *= kInvSqrtHeadDim;
  }
  if (!qvalid) return;
  if (p.o_dtype == 0) {
    float* orow = reinterpret_cast<float*>(p.o) + qrow * p.ldo + head * kHeadDim + 4 * hsel;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        f32x4 v = {u[db][4 * q], u[db][4 * q + 1], u[db][4 * q + 2], u[db][4 * q + 3]};
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * q) = v;
      }
  } else {
    uint16_t* orow = reinterpret_cast<uint16_t*>(p.o) + qrow * p.ldo + head * kHeadDim + 4 * hsel;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        u32x2 v;
        if (p.o_dtype == 1) {
          v[0] = f32_to_bf16_bits(u[db][4 * q]) | (f32_to_bf16_bits(u[db][4 * q + 1]) << 16);
          v[1] = f32_to_bf16_bits(u[db][4 * q + 2]) | (f32_to_bf16_bits(u[db][4 * q + 3]) << 16);
        } else {
          v[0] = f32_to_f16_bits(u[db][4 * q]) | (f32_to_f16_bits(u[db][4 * q + 1]) << 16);
          v[1] = f32_to_f16_bits(u[db][4 * q + 2]) | (f32_to_f16_bits(u[db][4 * q + 3]) << 16);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * q) = v;
      }
  }
  if (p.lse && hsel == 0) p.lse[(int64_t)head * N + qrow] = lse;
}

}  // namespace

int launch_packed_attention(const AttnParams& p, void* stream) {
  const int64_t nq = p.q_end - p.q_begin;
  if (nq <= 0 || p.kv_end <= p.kv_begin) return 0;
  const int64_t tiles = (nq + kBQ - 1) / kBQ;
  if (p.qk_mode == 1)
    hipLaunchKernelGGL(packed_attention_kernel<true>, dim3((unsigned)tiles, (unsigned)p.n_heads),
                       dim3(kThreads), 0, (hipStream_t)stream, p);
  else
    hipLaunchKernelGGL(packed_attention_kernel<false>, dim3((unsigned)tiles, (unsigned)p.n_heads),
                       dim3(kThreads), 0, (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace sqg

// Streamed QKV projection with a quantising epilogue, for gfx950.
//
// Computes, for the token rows of one chunk, the transposed projection tile
// y^T[col, token] = sum_k W[k, col] x[token, k] on bf16 MFMA (fp32 accumulation)
// and consumes it in registers: the fused [N, 3d] tensor is never written
// (feature request "Streamed QKV Projection and Packed Low-Bit K/V Support",
// section "Proposed backend capability").  Per 128-column head of the tile:
//   q columns : optional RMSNorm + split-half RoPE, bf16 store (model basis);
//   k columns : optional RMSNorm + RoPE, Hadamard rotation, group quantisation,
//               nibble (or byte) packing into the K store;
//   v columns : Hadamard rotation, quantisation, packing into the V store.
// (VRAM Lab page, block section `_phase1_kv`: projection -> split -> norm/RoPE ->
// store; kvi8r section: rotated store.)
//
// Workgroup tile: 256 output columns (2 heads) x 256 tokens, K-step 64, four
// waves in a 2 x 2 grid, each wave owning one head x 128 tokens.  Slices of x and
// W are fetched with range-checked buffer loads two K-steps ahead of their LDS
// store (two register sets), LDS is double-buffered, and scheduling groups thread
// the next step's operand reads between each step's MFMAs.  The transposed
// product puts one token per lane column of each 32x32 MFMA block, so the head's
// 128 values of a token sit in one lane pair: the Hadamard, the RMSNorm sum and the
// group absmax each need a single exchange with lane ^ 32 (device_common.h).
#include "device_common.h"
#include "internal.h"

namespace sqg {
namespace {

constexpr int kBM = 256;        // output columns per workgroup
constexpr int kBN = 256;        // tokens per workgroup
constexpr int kBK = 64;         // reduction slice per stage
constexpr int kStride = kBK + 8;  // bf16 per LDS row (144 B: conflict-free 16-byte reads)
constexpr int kTileElems = 256 * kStride;
constexpr int kGroupRows = 32;  // token tiles per raster group (L2 reuse of W and x)

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi_src, uint32_t lo_src, uint32_t sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}

// RMSNorm of one head vector in column layout: u * w / sqrt(mean(u^2) + eps)
__device__ __forceinline__ void rms_norm_cols(float (&u)[4][16], const float* __restrict__ w,
                                              float eps) {
  float ss = 0.0f;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) ss += u[b][i] * u[b][i];
  ss += xor32(ss);
  const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + eps);
  const int h4 = (threadIdx.x & 32) ? 4 : 0;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 wv = *reinterpret_cast<const f32x4*>(w + 32 * b + 8 * q + h4);
#pragma unroll
      for (int j = 0; j < 4; ++j) u[b][4 * q + j] = u[b][4 * q + j] * inv * wv[j];
    }
}

// split-half RoPE: element pairs (e, e + 64) = blocks (b, b + 2) rotate by table row `t`
__device__ __forceinline__ void rope_cols(float (&u)[4][16], const float* __restrict__ cs,
                                          const float* __restrict__ sn, int64_t t, bool valid) {
  const int h4 = (threadIdx.x & 32) ? 4 : 0;
  const int64_t base = valid ? t * 64 : 0;
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 c = *reinterpret_cast<const f32x4*>(cs + base + 32 * b + 8 * q + h4);
      const f32x4 s = *reinterpret_cast<const f32x4*>(sn + base + 32 * b + 8 * q + h4);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = u[b][4 * q + j], x1 = u[b + 2][4 * q + j];
        u[b][4 * q + j] = x0 * c[j] - x1 * s[j];
        u[b + 2][4 * q + j] = x1 * c[j] + x0 * s[j];
      }
    }
}

__global__ __launch_bounds__(256, 1) void qkv_quant_kernel(const QkvParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][kTileElems];  // [stage][A=W^T, B=x]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hsel = lane >> 5;

  // ---- raster: groups of kGroupRows token tiles sweep all column tiles
  const int n_col_tiles = p.n_col_tiles;
  const int64_t rows = p.row_end - p.row_begin;
  const int n_tok_tiles = (int)((rows + kBN - 1) / kBN);
  const int lin = blockIdx.x;
  const int per_group = kGroupRows * n_col_tiles;
  const int group = lin / per_group;
  const int first_tok = group * kGroupRows;
  const int gsize = min(kGroupRows, n_tok_tiles - first_tok);
  const int in_group = lin - group * per_group;
  const int tok_tile = first_tok + in_group % gsize;
  const int col_tile = p.col_tile0 + in_group / gsize;

  const int col0 = col_tile * kBM;
  const int64_t tok0 = p.row_begin + (int64_t)tok_tile * kBN;

  // ---- global -> register staging maps
  // x tile [256 tokens][64 k]: thread loads 16 B chunk (tid & 7) of rows (tid >> 3) + 32 i
  const int xc = tid & 7;
  const int xr = tid >> 3;
  // W tile [64 k][256 cols]: thread loads an 8 k x 8 col block: k rows 8 (tid & 7) + i,
  // cols 8 (tid >> 3) .. + 7, and writes it transposed (k contiguous per column)
  const int wk = tid & 7;
  const int wcb = tid >> 3;

  // x rows past the end of the sequence read as zero through the buffer's size
  const int64_t rows_valid = min((int64_t)kBN, p.n_tokens - tok0);
  const __amdgpu_buffer_rsrc_t xr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.x + tok0 * p.ldx), 0, (int32_t)(rows_valid * p.ldx * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + col0), 0, (int32_t)0x7fffffff, kBufferWord3);
  const uint32_t x_off = (uint32_t)((xr * p.ldx + 8 * xc) * 2);
  const uint32_t x_rowstep = (uint32_t)(32 * p.ldx * 2);
  const uint32_t w_off = (uint32_t)(((8 * wk) * p.ldw + 8 * wcb) * 2);
  const uint32_t w_rowstep = (uint32_t)(p.ldw * 2);

  u32x4 xregs[2][8], wregs[2][8];
  auto load_tiles = [&](int kt, u32x4 (&xreg)[8], u32x4 (&wreg)[8]) {
    const int32_t kx = kt * kBK * 2;                       // byte offset along k in x rows
    const int32_t kw = (int32_t)((int64_t)kt * kBK * p.ldw * 2);  // byte offset of k rows in W
#pragma unroll
    for (int i = 0; i < 8; ++i)
      xreg[i] = __builtin_amdgcn_raw_buffer_load_b128(xr_rsrc, x_off + i * x_rowstep, kx, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i)
      wreg[i] = __builtin_amdgcn_raw_buffer_load_b128(wr_rsrc, w_off + i * w_rowstep, kw, 0);
  };
  auto store_tiles = [&](int stage, const u32x4 (&xreg)[8], const u32x4 (&wreg)[8]) {
    uint16_t* sA = lds[stage][0];
    uint16_t* sB = lds[stage][1];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<u32x4*>(sB + (xr + 32 * i) * kStride + 8 * xc) = xreg[i];
    // 8x8 transpose of bf16: column c gets (k=2j, k=2j+1) pairs from rows 2j, 2j+1
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int m = c >> 1;
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      u32x4 o;
#pragma unroll
      for (int j = 0; j < 4; ++j) o[j] = perm_b32(wreg[2 * j + 1][m], wreg[2 * j][m], sel);
      *reinterpret_cast<u32x4*>(sA + (8 * wcb + c) * kStride + 8 * wk) = o;
    }
  };

  // ---- main loop
  const int wc = wave & 1;   // column half: head 2 col_tile + wc
  const int wt = wave >> 1;  // token half
  f32x16 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  const int nk = p.d_model / kBK;   // a multiple of 4 (d is a multiple of 256)
  load_tiles(0, xregs[0], wregs[0]);
  load_tiles(1, xregs[1], wregs[1]);
  store_tiles(0, xregs[0], wregs[0]);
  load_tiles(2, xregs[0], wregs[0]);
  __syncthreads();
  const int a_row = (128 * wc + l32) * kStride + 8 * hsel;
  const int b_row = (128 * wt + l32) * kStride + 8 * hsel;
  // slices are loaded two iterations before they are written to LDS: at the end of
  // iteration kt the registers holding slice kt + 1 are stored, then reloaded with
  // slice kt + 3 (clamped to the last slice near the end)
  auto iteration = [&](int kt, u32x4 (&xreg)[8], u32x4 (&wreg)[8]) {
    const int stage = kt & 1;
    const uint16_t* sA = lds[stage][0];
    const uint16_t* sB = lds[stage][1];
    bf16x8 af[2][4], bfr[2][4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      af[0][c] = *reinterpret_cast<const bf16x8*>(sA + a_row + 32 * c * kStride);
      bfr[0][c] = *reinterpret_cast<const bf16x8*>(sB + b_row + 32 * c * kStride);
    }
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
      const int cur = ks & 1;
      if (ks + 1 < kBK / 16) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          af[cur ^ 1][c] = *reinterpret_cast<const bf16x8*>(sA + a_row + 32 * c * kStride + 16 * (ks + 1));
          bfr[cur ^ 1][c] = *reinterpret_cast<const bf16x8*>(sB + b_row + 32 * c * kStride + 16 * (ks + 1));
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[c][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[cur][c], bfr[cur][t], acc[c][t], 0, 0, 0);
    }
    store_tiles(stage ^ 1, xreg, wreg);
    load_tiles(min(kt + 3, nk - 1), xreg, wreg);
    // schedule: first-step fragments; then per step its 16 MFMAs with the next step's
    // 8 fragment reads threaded between them; LDS writes and global loads last
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
    for (int ks = 0; ks < kBK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (ks + 1 < kBK / 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    }
    __syncthreads();
  };
  for (int kt = 0; kt < nk; kt += 2) {
    iteration(kt, xregs[1], wregs[1]);
    iteration(kt + 1, xregs[0], wregs[0]);
  }

  // ---- epilogue: one head x 128 tokens per wave
  const int head_all = (col0 >> 7) + wc;   // head index over q | k | v
  const int section = head_all / p.n_heads;  // 0 q, 1 k, 2 v
  const int h = head_all - section * p.n_heads;
  const int64_t wtok0 = tok0 + 128 * wt;
  if (wtok0 >= p.row_end) return;          // wave-uniform
  const int seg = find_segment(p.seg, wtok0);
  const int fmt = head_format(p.seg, seg, h);
  const int64_t head_base = head_rows_offset(p.seg, seg, h);
  const int row_bytes = format_row_bytes(fmt);

  // The token-block loop stays rolled (its body is large); the accumulator column
  // is picked with static indices so the accumulators never leave registers.
#pragma nounroll
  for (int tb = 0; tb < 4; ++tb) {
    const int64_t t = wtok0 + 32 * tb + l32;
    const bool valid = t < p.row_end;
    float u[4][16];
    switch (tb) {
#define SQG_TAKE_COLUMN(TB)                                    \
      case TB:                                                 \
        _Pragma("unroll") for (int b = 0; b < 4; ++b)          \
        _Pragma("unroll") for (int i = 0; i < 16; ++i) u[b][i] = acc[b][TB][i]; \
        break;
      SQG_TAKE_COLUMN(0)
      SQG_TAKE_COLUMN(1)
      SQG_TAKE_COLUMN(2)
      default:
      SQG_TAKE_COLUMN(3)
#undef SQG_TAKE_COLUMN
    }

    if (section == 0) {
      if (p.q_norm_w) rms_norm_cols(u, p.q_norm_w, p.eps);
      if (p.rope_cos) rope_cols(u, p.rope_cos, p.rope_sin, t, valid);
      if (valid) {
        uint16_t* qrow = p.q + (t - p.q_row0) * p.ldq + h * kHeadDim + 4 * hsel;
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            u32x2 v;
            v[0] = f32_to_bf16_bits(u[b][4 * q]) | (f32_to_bf16_bits(u[b][4 * q + 1]) << 16);
            v[1] = f32_to_bf16_bits(u[b][4 * q + 2]) | (f32_to_bf16_bits(u[b][4 * q + 3]) << 16);
            *reinterpret_cast<u32x2*>(qrow + 32 * b + 8 * q) = v;
          }
      }
    } else {
      if (section == 1) {
        if (p.k_norm_w) rms_norm_cols(u, p.k_norm_w, p.eps);
        if (p.rope_cos) rope_cols(u, p.rope_cos, p.rope_sin, t, valid);
      }
      fwht128_cols(u);
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) u[b][i] = scale_inv_sqrt128(u[b][i]);
      uint8_t* store = (section == 1) ? p.kpack : p.vpack;
      uint16_t* scl = (section == 1) ? p.kscale : p.vscale;
      const int64_t tt = valid ? t : wtok0;
      uint8_t* row = store + head_base + (tt - p.seg.begin[seg]) * row_bytes;
      uint16_t* srow = scl + ((int64_t)h * p.kv_n + (tt - p.kv_row0)) * 4;
      if (fmt == FMT_INT4)
        quant_pack_store<FMT_INT4>(u, row, srow, valid);
      else if (fmt == FMT_INT8)
        quant_pack_store<FMT_INT8>(u, row, srow, valid);
      else
        bf16_row_store(u, row, srow, valid);
    }
  }
}

}  // namespace

int launch_qkv_quant(const QkvParams& p, void* stream) {
  const int64_t rows = p.row_end - p.row_begin;
  const int64_t n_tok_tiles = (rows + kBN - 1) / kBN;
  const int64_t blocks = n_tok_tiles * p.n_col_tiles;
  if (blocks <= 0) return 0;
  hipLaunchKernelGGL(qkv_quant_kernel, dim3((unsigned)blocks), dim3(256), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace sqg

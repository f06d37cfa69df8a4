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
// Workgroup tile: 256 output columns (2 heads) x 256 tokens, K-step 64, eight
// waves (two per SIMD) in a 2 x 4 grid, each wave owning one head x 64 tokens
// (128 accumulator registers), so one wave's MFMAs run through the other's
// barrier and operand-read gaps.  The x and W
// slices of a K-step go from HBM straight into LDS (range-checked buffer loads with
// the LDS bit, no register staging), into two stages; W stays k-major there and
// its MFMA operand comes out through transposing LDS reads.  One barrier per
// K-step sits before the step's last k-substep, whose 8 MFMAs per wave run beside the
// loads of the slices two steps ahead and the next step's first operand reads;
// scheduling groups thread each substep's operand reads between the MFMAs of the
// substep before.  The transposed
// product puts one token per lane column of each 32x32 MFMA block, so the head's
// 128 values of a token sit in one lane pair: the Hadamard, the RMSNorm sum and the
// group absmax each need a single exchange with lane ^ 32 (device_common.h).
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace sqg {
namespace {

constexpr int kBM = 256;        // output columns per workgroup
constexpr int kBN = 256;        // tokens per workgroup
constexpr int kBK = 64;         // reduction slice per stage
constexpr int kXBytes = kBN * kBK * 2;          // x slice [256 tokens][64 k]: 32 KiB
constexpr int kStageBytes = kXBytes + kBK * kBM * 2;  // + W slice [64 k][256 cols]
constexpr int kTB = 2;          // 32-token blocks per wave (eight waves: 2 heads x 4 token quarters)
constexpr int kGroupRows = 32;  // token tiles per raster group (L2 reuse of W and x)

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

__global__ __launch_bounds__(512, 1) void qkv_quant_kernel(const QkvParams p) {
  // two stages as two arrays, so that the compiler sees that a stage being filled and
  // the stage being read never alias (no wait on the fills before the reads)
  __shared__ __attribute__((aligned(1024))) uint8_t lds0[kStageBytes];
  __shared__ __attribute__((aligned(1024))) uint8_t lds1[kStageBytes];

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

  // ---- operand slices go from HBM straight into LDS (buffer loads with the LDS bit:
  // lane L of a wave's load writes bytes [16 L, 16 L + 16) of a 1 KiB LDS block), two
  // stages of 64 KiB, each holding the x slice [256 tokens][64 k] (128-byte rows) and
  // the W slice [64 k][256 cols] (512-byte rows).  Each 16-byte chunk is placed at an
  // XOR-swizzled slot of its row (the lane loads the chunk that belongs in its slot), so
  // the MFMA operand reads below hit distinct LDS banks:
  //   x row t, chunk c (k 8c .. 8c + 7)     at slot c ^ ((t >> 1) & 7)
  //   W row k, chunk c (cols 8c .. 8c + 7)  at slot c ^ (4 (k & 3))
  const int64_t rows_valid = min((int64_t)kBN, p.n_tokens - tok0);
  const __amdgpu_buffer_rsrc_t xr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.x + tok0 * p.ldx), 0, (int32_t)(rows_valid * p.ldx * 2), kBufferWord3);
  const __amdgpu_buffer_rsrc_t wr_rsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.w + col0), 0, (int32_t)0x7fffffff, kBufferWord3);
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  // wave wv moves x rows 32 wv .. + 31 and W rows 8 wv .. + 7: four 1 KiB loads each
  uint32_t xoff[4], woff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int xrow = 32 * wv + 8 * i + (lane >> 3);
    const int xc = (lane & 7) ^ ((xrow >> 1) & 7);
    xoff[i] = (uint32_t)(xrow * p.ldx * 2 + 16 * xc);
    const int wrow = 8 * wv + 2 * i + (lane >> 5);
    const int wch = (lane & 31) ^ (4 * (wrow & 3));
    woff[i] = (uint32_t)(wrow * p.ldw * 2 + 16 * wch);
  }
  auto issue_loads = [&](int kt, int stage) {
    uint8_t* xs = (stage ? lds1 : lds0) + wv * 4096;
    uint8_t* ws = xs + kXBytes;
    const uint32_t kx = (uint32_t)(kt * kBK * 2);
    const uint32_t kw = (uint32_t)((int64_t)kt * kBK * p.ldw * 2);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr_rsrc, (__attribute__((address_space(3))) void*)(xs + 1024 * i),
                                               16, xoff[i], kx, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_rsrc, (__attribute__((address_space(3))) void*)(ws + 1024 * i),
                                               16, woff[i], kw, 0, 0);
  };

  // ---- main loop
  const int wc = wave & 1;   // column half: head 2 col_tile + wc
  const int wt = wave >> 1;  // token quarter
  f32x16 acc[4][kTB];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < kTB; ++b)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[a][b][e] = 0.0f;

  // A operand (W^T: 32 cols x 16 k per MFMA) by transposing reads: within a 16-lane
  // group, lane g4 + 4 j points at 4 columns 4 (lane % 4) .. of W row k0 + j and lane i
  // receives column i of rows k0 .. k0 + 3; two reads (k0, k0 + 4) give the 8 k values
  // of lanes 0-31 (k 0-7) and 32-63 (k 8-15).
  const int g16 = lane >> 4, c16 = lane & 15, a4 = c16 & 3, j4 = c16 >> 2;
  uint32_t abase[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
    abase[cb] = (uint32_t)((8 * (g16 >> 1) + j4) * 512 +
                           16 * (16 * wc + 4 * (cb ^ j4) + 2 * (g16 & 1) + (a4 >> 1)) + 8 * (a4 & 1));
  // B operand (x: 16 k x 32 tokens per MFMA): lane = token, 16 contiguous bytes
  const int bswz = (l32 >> 1) & 7;
  uint32_t bbase[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) bbase[ks] = (uint32_t)((32 * kTB * wt + l32) * 128 + 16 * ((2 * ks + hsel) ^ bswz));

  const int nk = p.d_model / kBK;   // a multiple of 2 (d is a multiple of 256)
  bf16x8 af[2][4], bfr[2][kTB];
  auto rd = [&](const uint8_t* xs, int ks, int b) {   // operands of k-substep ks into set b
    const uint8_t* ws = xs + kXBytes;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      typedef short v4s __attribute__((ext_vector_type(4)));
      const v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(ws + abase[cb] + ks * 8192));
      const v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) v4s*)(ws + abase[cb] + ks * 8192 + 2048));
      af[b][cb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int tb = 0; tb < kTB; ++tb)
      bfr[b][tb] = *reinterpret_cast<const bf16x8*>(xs + bbase[ks] + tb * 4096);
  };
  auto mm = [&](int b) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int t = 0; t < kTB; ++t)
        acc[c][t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[b][c], bfr[b][t], acc[c][t], 0, 0, 0);
  };
  // every wave's slices of the stage about to be read have landed, and every wave has
  // read its operands of the other stage
  auto sync_point = [&]() {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  auto interleave = [&](int n_vmem) {     // 8 MFMAs, each with up to one load and two reads
#pragma unroll
    for (int i = 0; i < 4 * kTB; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (i < n_vmem) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      if (i < 5) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };
  // Step kt reads stage kt & 1.  Its first operands were read before it starts; the
  // barrier sits before the last k-substep's MFMAs, after which the slices of step kt + 2
  // go into this stage and the first operands of step kt + 1 are read, both while those
  // MFMAs (8 per wave) run.
  auto step = [&](int kt, int stage, auto loads, auto more) {
    const uint8_t* xs = stage ? lds1 : lds0;
    const uint8_t* xn = stage ? lds0 : lds1;
    __builtin_amdgcn_sched_barrier(0);
    rd(xs, 1, 1);
    mm(0);
    interleave(0);
    __builtin_amdgcn_sched_barrier(0);
    rd(xs, 2, 0);
    mm(1);
    interleave(0);
    __builtin_amdgcn_sched_barrier(0);
    rd(xs, 3, 1);
    mm(0);
    interleave(0);
    __builtin_amdgcn_sched_barrier(0);
    sync_point();
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (decltype(loads)::value) issue_loads(kt + 2, stage);
    if constexpr (decltype(more)::value) rd(xn, 0, 0);
    mm(1);
    interleave(decltype(loads)::value ? 8 : 0);
    __builtin_amdgcn_sched_barrier(0);
  };
  issue_loads(0, 0);
  sync_point();
  if (nk > 1) issue_loads(1, 1);
  rd(lds0, 0, 0);
  const std::true_type yes;
  const std::false_type no;
  for (int kt = 0; kt < nk - 2; kt += 2) {
    step(kt, 0, yes, yes);
    step(kt + 1, 1, yes, yes);
  }
  step(nk - 2, 0, no, yes);
  step(nk - 1, 1, no, no);

  // ---- epilogue: one head x 64 tokens per wave
  const int head_all = (col0 >> 7) + wc;   // head index over q | k | v
  const int section = head_all / p.n_heads;  // 0 q, 1 k, 2 v
  const int h = head_all - section * p.n_heads;
  const int64_t wtok0 = tok0 + 32 * kTB * wt;
  if (wtok0 >= p.row_end) return;          // wave-uniform
  const int seg = find_segment(p.seg, wtok0);
  const int fmt = head_format(p.seg, seg, h);
  const int64_t head_base = head_rows_offset(p.seg, seg, h);
  const int row_bytes = format_row_bytes(fmt);

  // The two token blocks are unrolled, so the first block's accumulators are free
  // registers while the second is processed (rolled, both stay live and spill).
#pragma unroll
  for (int tb = 0; tb < kTB; ++tb) {
    const int64_t t = wtok0 + 32 * tb + l32;
    const bool valid = t < p.row_end;
    float u[4][16];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) u[b][i] = acc[b][tb][i];

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
  hipLaunchKernelGGL(qkv_quant_kernel, dim3((unsigned)blocks), dim3(512), 0,
                     (hipStream_t)stream, p);
  return (int)hipGetLastError();
}

}  // namespace sqg

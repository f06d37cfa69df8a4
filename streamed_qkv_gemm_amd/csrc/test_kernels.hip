// Test entry kernels: run the production epilogue steps (the quantise/pack step and
// the 128-point Hadamard butterfly of device_common.h) on caller-supplied fp32
// vectors, so that parity tests can check those steps bit for bit in isolation.
// Each wave takes 32 vectors and holds them in the same column layout the
// QKV-quant kernel's accumulators have.
#include "device_common.h"
#include "internal.h"

namespace sqg {
namespace {

__device__ __forceinline__ void load_cols(const float* __restrict__ base, int64_t row, bool valid,
                                          float (&u)[4][16]) {
  const int h4 = (threadIdx.x & 32) ? 4 : 0;
  const float* src = base + (valid ? row : 0) * kHeadDim + h4;
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v = {0.f, 0.f, 0.f, 0.f};
      if (valid) v = *reinterpret_cast<const f32x4*>(src + 32 * b + 8 * q);
#pragma unroll
      for (int j = 0; j < 4; ++j) u[b][4 * q + j] = v[j];
    }
}

__global__ __launch_bounds__(64) void test_quant_pack_kernel(const float* r, int64_t rows, int fmt,
                                                             uint8_t* codes, uint16_t* scales) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x & 31);
  const bool valid = row < rows;
  float u[4][16];
  load_cols(r, row, valid, u);
  const int64_t rr = valid ? row : 0;
  if (fmt == FMT_INT4)
    quant_pack_store<FMT_INT4>(u, codes + rr * 64, scales + rr * 4, valid);
  else
    quant_pack_store<FMT_INT8>(u, codes + rr * 128, scales + rr * 4, valid);
}

__global__ __launch_bounds__(64) void test_fwht_kernel(const float* in, float* out, int64_t rows,
                                                       int normalize) {
  const int64_t row = (int64_t)blockIdx.x * 32 + (threadIdx.x & 31);
  const bool valid = row < rows;
  float u[4][16];
  load_cols(in, row, valid, u);
  fwht128_cols(u);
  if (!valid) return;
  if (normalize) {
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) u[b][i] = scale_inv_sqrt128(u[b][i]);
  }
  float* dst = out + row * kHeadDim + ((threadIdx.x & 32) ? 4 : 0);
#pragma unroll
  for (int b = 0; b < 4; ++b)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      f32x4 v = {u[b][4 * q], u[b][4 * q + 1], u[b][4 * q + 2], u[b][4 * q + 3]};
      *reinterpret_cast<f32x4*>(dst + 32 * b + 8 * q) = v;
    }
}

}  // namespace

int launch_test_quant_pack(const float* r, int64_t rows, int32_t fmt, void* codes, void* scales,
                           void* stream) {
  if (rows <= 0) return 0;
  const int64_t blocks = (rows + 31) / 32;
  hipLaunchKernelGGL(test_quant_pack_kernel, dim3((unsigned)blocks), dim3(64), 0,
                     (hipStream_t)stream, r, rows, (int)fmt, (uint8_t*)codes, (uint16_t*)scales);
  return (int)hipGetLastError();
}

int launch_test_fwht(const float* in, float* out, int64_t rows, int32_t normalize, void* stream) {
  if (rows <= 0) return 0;
  const int64_t blocks = (rows + 31) / 32;
  hipLaunchKernelGGL(test_fwht_kernel, dim3((unsigned)blocks), dim3(64), 0, (hipStream_t)stream,
                     in, out, rows, (int)normalize);
  return (int)hipGetLastError();
}

}  // namespace sqg

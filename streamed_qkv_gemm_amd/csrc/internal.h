// Host-side interface between the C-ABI entry points (sqg_api.cpp) and the kernel
// launchers (one .hip file per kernel).  Not part of the public ABI; plain C++ so
// the host side builds without HIP headers.
#pragma once

#include <stdint.h>

namespace sqg {

enum { FMT_INT4 = 0, FMT_INT8 = 1, FMT_BF16 = 2 };

// Token-range segments of the packed store (at most 16).  Within segment s, head h
// uses format FMT_INT8 if fmt[s] is FMT_INT4 and bit h of int8_heads[s] is set, else
// fmt[s]; its rows start at offset[s] + (end - begin) * (bytes of the rows of the
// heads before it) and follow each other.
struct SegTable {
  int32_t n;
  int32_t fmt[16];
  int64_t begin[16];
  int64_t end[16];
  int64_t offset[16];      // byte offset of the segment in the packed store
  uint64_t int8_heads[16];
};

// One launch of the streamed QKV-quant kernel over rows [row_begin, row_end).
struct QkvParams {
  const uint16_t* x;       // bf16 [N, ldx]
  const uint16_t* w;       // bf16 [d, ldw]
  uint16_t* q;             // bf16 [N, ldq]
  uint8_t* kpack;
  uint8_t* vpack;
  uint16_t* kscale;        // fp16 [H, kv_n, 4]
  uint16_t* vscale;
  const float* q_norm_w;   // [128] or null
  const float* k_norm_w;
  const float* rope_cos;   // [N, 64] or null
  const float* rope_sin;
  int64_t ldx, ldw, ldq;
  int64_t n_tokens;
  int64_t row_begin, row_end;
  int64_t q_row0;          // token t's Q goes to row t - q_row0 of q
  int64_t kv_row0, kv_n;   // the K/V store holds tokens [kv_row0, kv_row0 + kv_n)
  int32_t d_model, n_heads;
  float eps;
  int32_t col_tile0;       // first 256-column tile of [q | k | v] this launch covers
  int32_t n_col_tiles;     // number of column tiles it covers
  int32_t pad_;
  SegTable seg;
};

// One launch of the packed-K/V attention kernel: queries [q_begin, q_end) against
// keys [kv_begin, kv_end); accumulate merges into the existing (o, lse).
struct AttnParams {
  const uint16_t* q;       // bf16 [N, ldq]
  const uint8_t* kpack;
  const uint8_t* vpack;
  const uint16_t* kscale;  // fp16 [H, kv_n, 4]
  const uint16_t* vscale;
  void* o;                 // [N, ldo] of o_dtype
  float* lse;              // [H, N] or null
  int64_t ldq, ldo;
  int64_t n_tokens;
  int64_t q_begin, q_end;
  int64_t q_row0;          // query row r is row r - q_row0 of q
  int64_t kv_row0, kv_n;   // the K/V store holds keys [kv_row0, kv_row0 + kv_n)
  int64_t kv_begin, kv_end;
  int32_t d_model, n_heads;
  int32_t o_dtype;
  int32_t accumulate;
  float scale_log2;        // softmax scale * log2(e)
  int32_t qk_mode;         // 0: f16 high + remainder query; 1: block-scaled fp8 QK^T
  SegTable seg;
};

int launch_qkv_quant(const QkvParams& p, void* stream);       // returns a hipError_t value
int launch_packed_attention(const AttnParams& p, void* stream);
int launch_test_quant_pack(const float* r, int64_t rows, int32_t fmt, void* codes, void* scales,
                           void* stream);
int launch_test_fwht(const float* in, float* out, int64_t rows, int32_t normalize, void* stream);
const char* hip_error_text(int err);

// Device scratch of the allocation-free Q-recompute entry point: kScratchBytes on every
// device, shared by all calls on that device.  scratch_for_current_device returns its
// address on the calling thread's current device (a hipError_t value, 0 on success).
constexpr int64_t kScratchBytes = 64ll << 20;
int scratch_for_current_device(void** ptr);

// Asynchronous copy on `stream` (hipMemcpyAsync); returns a hipError_t value.
enum CopyKind { kHostToDevice = 1, kDeviceToHost = 2 };
int copy_async(void* dst, const void* src, int64_t bytes, CopyKind kind, void* stream);

// Events ordering work across two streams (timing disabled); each returns a hipError_t value.
int event_create(void** ev);
int event_destroy(void* ev);
int event_record(void* ev, void* stream);
int stream_wait_event(void* stream, void* ev);

}  // namespace sqg

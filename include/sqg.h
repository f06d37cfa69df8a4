/*
 * sqg.h -- C ABI of libsqg.so: streamed QKV-quant and packed-K/V attention for
 * AMD Instinct MI355X (gfx950).
 *
 * What the library computes comes from two pages:
 *   [FR] feature request "Streamed QKV Projection and Packed Low-Bit K/V Support
 *        for Extreme Long-Sequence Attention" (comfy-kitchen issue and mirror);
 *   [VL] "VRAM Lab" module page (ComfyUI-MAINodes vram_lab.py).
 *
 * Conventions shared by every call
 *   - Pointers marked "device" are HIP device pointers; "host" pointers are read
 *     during the call only.  The caller owns every buffer.  The library never
 *     allocates or frees device memory, keeps no pointer after returning, never
 *     synchronises the stream, and holds no mutable global state except a
 *     thread-local error message.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is
 *     enqueued on it and the call returns without waiting.
 *   - Device pointers must be 16-byte aligned and row strides (in elements) must be
 *     multiples of 8, so that every tile is moved with 128-bit accesses.
 *   - Every argument is checked on the host before the first launch: a call that
 *     returns an error has enqueued nothing.  sqg_last_error() then describes it.
 *   - head_dim is 128 and the quantisation group is 32 values along head_dim.
 */
#ifndef SQG_H
#define SQG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(SQG_BUILDING_LIBRARY)
#define SQG_API __attribute__((visibility("default")))
#else
#define SQG_API
#endif

#define SQG_VERSION 140          /* 1.4.0 */
#define SQG_HEAD_DIM 128
#define SQG_GROUP 32
#define SQG_MAX_SEGMENTS 16

typedef enum sqg_status {
  SQG_OK = 0,
  SQG_ERR_INVALID_ARGUMENT = -1,   /* null pointer, bad size, bad range policy ... */
  SQG_ERR_UNSUPPORTED = -2,        /* shape outside what the kernels implement */
  SQG_ERR_MISALIGNED = -3,         /* pointer not 16-byte aligned or stride not a multiple of 8 */
  SQG_ERR_WORKSPACE_TOO_SMALL = -4,/* a workspace (or the device scratch) cannot hold what the call needs */
  SQG_ERR_HIP = -5                 /* a HIP launch reported an error */
} sqg_status;

/* K/V storage format of a token range.  [FR] "Quality-oriented low-bit format"
 * (fixed-width rotated INT4 with per-group scales) and "Mixed precision for
 * conditioning" (BF16 or 8-bit K/V for conditioning ranges).  The integer formats
 * hold codes of the Hadamard-rotated vector with one fp16 scale per group of 32
 * values; BF16 holds the rotated vector itself. */
typedef enum sqg_kv_format {
  SQG_INT4_ROT = 0,   /* codes in [-7, 7], two per byte, code 2i in bits 0-3 */
  SQG_INT8_ROT = 1,   /* codes in [-127, 127], one per byte (two's complement) */
  SQG_BF16_ROT = 2    /* the rotated values rounded to bf16 (RNE), 128 per row, little
                         endian; no scales (their entries are written as zero).  [FR]
                         "Mixed precision for conditioning" keeps conditioning ranges
                         at BF16 or INT8. */
} sqg_kv_format;

typedef enum sqg_out_dtype { SQG_F32 = 0, SQG_BF16 = 1, SQG_F16 = 2 } sqg_out_dtype;

/* Precision of the scores QK^T in attention.
 * SQG_QK_EXACT: the parity tier.  The rotated query, prescaled by softmax_scale *
 *   log2(e), is split into an f16 high part and its remainder; the scores are the f16
 *   MFMA of the high part against the dequantised f16 keys plus the block-scaled fp6
 *   (E2M3, one E8M0 exponent per group of 32 dims) MFMA of the remainder against the
 *   keys, fp32 accumulation.  INT4 and BF16 keys are exact in f16; INT8 keys add the
 *   f16 remainder of code * scale against the high part.
 * SQG_QK_FP8: [VL] kvi8s section (an approximation tier: rotated Q and K, QK^T on
 *   low-precision matrix cores straight from the store).  The rotated query and the
 *   decoded keys are quantised per group of 32 dims to OCP E4M3 values with one E8M0
 *   exponent (the smallest e with max |x| <= 448 * 2^e); the scores are the
 *   block-scaled fp8 MFMA of those operands.  P.V is unchanged (f16).  Not bit-equal
 *   to the exact tier. */
typedef enum sqg_qk_mode { SQG_QK_EXACT = 0, SQG_QK_FP8 = 1 } sqg_qk_mode;

/* What one sqg_streamed_qkv_quant call writes.  [VL] block section (the three-phase
 * streamed block): phase 1 keeps only K and V for the whole sequence and phase 2
 * recomputes Q chunk by chunk; SQG_EMIT_KV is that phase 1, SQG_EMIT_Q the Q part of
 * phase 2 (see sqg_packed_kv_attention_qrecompute). */
typedef enum sqg_emit {
  SQG_EMIT_QKV = 0,   /* Q and the packed K/V store */
  SQG_EMIT_Q = 1,     /* Q only: kpack, vpack, kscale, vscale may be NULL */
  SQG_EMIT_KV = 2     /* the packed K/V store only: q may be NULL */
} sqg_emit;

/* One token range [begin, end) of the precision policy. */
typedef struct sqg_range {
  int64_t begin;
  int64_t end;
  int32_t fmt;          /* sqg_kv_format */
  int32_t reserved;     /* must be 0 */
  uint64_t int8_heads;  /* INT4 ranges only (else 0): bit h set = head h of this range
                           is stored SQG_INT8_ROT ([VL] kvmix section: per-head 4/8-bit
                           split); bits at or above n_heads must be 0 */
} sqg_range;

/* Byte layout of the packed K (and, identically, V) store, filled by sqg_kv_layout.
 * Segment s covers tokens [seg_begin[s], seg_end[s]) in format seg_fmt[s], except that
 * in an INT4 segment the heads set in seg_int8_heads[s] are INT8.  Row bytes are 64
 * (INT4), 128 (INT8) and 256 (BF16); seg_row_bytes[s] is that of seg_fmt[s].  Within
 * a segment the heads' rows follow each other, head by head: the row of (head h,
 * token t) starts at byte
 *   seg_offset[s] + L * (sum of the row bytes of heads 0 .. h-1) + (t - seg_begin[s]) * rb(h)
 * of the kpack (vpack) buffer, L = seg_end[s] - seg_begin[s]; sqg_kv_row_offset
 * computes it.  With no INT8 heads this is
 *   seg_offset[s] + (h * L + (t - seg_begin[s])) * seg_row_bytes[s].
 * Scales are fp16 [n_heads, n_tokens, 4]: group g of (h, t) at element (h*N + t)*4 + g.
 * A block store (sqg_kv_block_layout) holds only keys [k0, k1): n_tokens = k1 - k0, the
 * segments are the policy's clipped to [k0, k1) (seg_begin/seg_end stay absolute token
 * indices, seg_begin[0] = k0), and token t's scales sit at row t - k0. */
typedef struct sqg_layout {
  int64_t n_tokens;
  int32_t n_heads;
  int32_t n_segments;
  int64_t seg_begin[SQG_MAX_SEGMENTS];
  int64_t seg_end[SQG_MAX_SEGMENTS];
  int64_t seg_offset[SQG_MAX_SEGMENTS];
  int32_t seg_fmt[SQG_MAX_SEGMENTS];
  int32_t seg_row_bytes[SQG_MAX_SEGMENTS];
  uint64_t seg_int8_heads[SQG_MAX_SEGMENTS];
  int64_t q_bytes;        /* bf16 Q [N, d] */
  int64_t pack_bytes;     /* bytes of kpack, and of vpack */
  int64_t scale_bytes;    /* bytes of kscale, and of vscale */
  int64_t bf16_qkv_bytes; /* the fused bf16 [N, 3d] tensor this layout replaces */
} sqg_layout;

/* Arguments of sqg_streamed_qkv_quant. */
typedef struct sqg_qkv_args {
  int64_t n_tokens;            /* N >= 0 (0 is a no-op) */
  int32_t d_model;             /* d = 128 * n_heads, a multiple of 256 */
  int32_t n_heads;
  const void* x;               /* device, bf16 [N, ldx] row-major */
  int64_t ldx;
  const void* w_qkv;           /* device, bf16 [d, 3d] row-major: columns q | k | v, head h at 128h */
  int64_t ldw;                 /* >= 3d */
  const float* q_norm_w;       /* device, fp32 [128] or NULL: per-head RMSNorm gain of q */
  const float* k_norm_w;       /* device, fp32 [128] or NULL (both or neither) */
  float eps;                   /* RMSNorm epsilon */
  const float* rope_cos;       /* device, fp32 [N, 64] or NULL (both or neither); see sqg_rope_table */
  const float* rope_sin;
  const sqg_range* ranges;     /* host; NULL with n_ranges 0 = all INT4 */
  int32_t n_ranges;
  int32_t emit;                /* sqg_emit (0 = Q and K/V) */
  int64_t chunk_rows;          /* rows per launch (multiple of 128); 0 = one launch */
  int64_t min_tail;            /* a last chunk shorter than this joins the previous one; <0 = 512 */
  void* q;                     /* device, bf16 [N, ldq] out (model basis) */
  int64_t ldq;
  void* kpack;                 /* device, layout.pack_bytes out */
  void* vpack;
  void* kscale;                /* device, fp16 [H, N, 4] out */
  void* vscale;
} sqg_qkv_args;

/* Arguments of sqg_packed_kv_attention. */
typedef struct sqg_attn_args {
  int64_t n_tokens;            /* N: rows of Q and keys in the store */
  int32_t d_model;
  int32_t n_heads;
  const void* q;               /* device, bf16 [N, ldq] (model basis) */
  int64_t ldq;
  const void* kpack;           /* device, as written by sqg_streamed_qkv_quant */
  const void* vpack;
  const void* kscale;          /* device, fp16 [H, N, 4] */
  const void* vscale;
  const sqg_range* ranges;     /* host: the policy the store was written with */
  int32_t n_ranges;
  int32_t o_dtype;             /* sqg_out_dtype */
  int64_t q_begin, q_end;      /* query rows [q_begin, q_end); q_end 0 = N */
  int64_t kv_begin, kv_end;    /* keys [kv_begin, kv_end); kv_end 0 = N; kv_begin % 128 == 0 */
  int64_t kv_block;            /* 0 = one pass; > 0 = key blocks of this many keys (multiple of
                                  128, last block shorter than 512 folded) merged by log-sum-exp,
                                  in one launch (see sqg_packed_kv_attention) */
  int32_t accumulate;          /* 1 = merge into the existing (O, lse) instead of overwriting */
  float softmax_scale;         /* 0 = 1/sqrt(128) */
  void* o;                     /* device, [N, ldo] of o_dtype, out (model basis) */
  int64_t ldo;
  float* lse;                  /* device, fp32 [H, N] natural-log LSE out, or NULL;
                                  required when accumulate or kv_block > 0 */
  int32_t qk_mode;             /* sqg_qk_mode (0 = exact tier) */
  int32_t reserved;            /* must be 0 */
} sqg_attn_args;

/* A K/V store held in host memory as consecutive block stores ([VL] module docstring:
 * the host-staged ("turtle") K/V the pages name as the real fix for the K/V peak).
 * Keys are split into blocks of block_rows (sqg_chunk_ranges(N, block_rows, 512):
 * a last block shorter than 512 keys joins the previous one).  Block b is a block store
 * (sqg_kv_block_layout) whose codes start at host_kpack + (sum of the pack_bytes of
 * blocks before b), and whose scales start at host_kscale + (sum of their scale_bytes);
 * likewise for V.  Two device staging block stores carry blocks between host and
 * kernels.  sqg_staged_sizes gives every buffer size.  With copy_stream NULL the copies
 * run in order on the call's stream; with a second stream (default priority, same
 * device) they run there, ordered against the kernels by events, so a block's copy
 * overlaps the neighbouring block's kernel (a staging slot is refilled only after the
 * kernel that used it, a kernel starts only after its block's copy).  The copy stream
 * first waits for the work already on the call's stream, and a staged QKV-quant call
 * leaves the call's stream waiting for its last copies, so either way the caller sees
 * the same ordering as with in-order copies.  Calls that share one copy stream must not
 * overlap in time. */
typedef struct sqg_staged_kv {
  int64_t block_rows;          /* keys per block, a positive multiple of 128 */
  void* host_kpack;            /* pinned host (hipHostMalloc / pinned torch tensors) */
  void* host_vpack;
  void* host_kscale;
  void* host_vscale;
  void* dev_kpack[2];          /* device staging */
  void* dev_vpack[2];
  void* dev_kscale[2];
  void* dev_vscale[2];
  void* copy_stream;           /* hipStream_t for the copies, or NULL (copies in order) */
} sqg_staged_kv;

/* Arguments of sqg_packed_kv_attention_qrecompute. */
typedef struct sqg_qrecompute_args {
  sqg_attn_args attn;          /* as for sqg_packed_kv_attention, except that attn.q and attn.ldq
                                  are ignored: Q is recomputed into the workspace */
  const void* x;               /* device, bf16 [N, ldx]: the rows the K/V store was built from */
  int64_t ldx;
  const void* w_qkv;           /* device, bf16 [d, 3d] row-major (only the q columns are read) */
  int64_t ldw;
  const float* q_norm_w;       /* device, fp32 [128] or NULL: per-head RMSNorm gain of q */
  const float* rope_cos;       /* device, fp32 [N, 64] or NULL (both or neither) */
  const float* rope_sin;
  float eps;                   /* RMSNorm epsilon */
  int32_t reserved;            /* must be 0 */
  int64_t q_chunk_rows;        /* query rows per chunk, a multiple of 128; 0 = the larger of
                                  16384 and 256 * ceil(2048 / n_heads); a last chunk shorter
                                  than 512 joins the previous one */
  void* workspace;             /* device, bf16 Q of one chunk; at least
                                  sqg_qrecompute_workspace_bytes(...) bytes */
  int64_t workspace_bytes;
} sqg_qrecompute_args;

/* Library version (SQG_VERSION of the build). */
SQG_API int sqg_version(void);

/* Fixed text for a status code. */
SQG_API const char* sqg_status_string(int status);

/* Detail of the last error on the calling thread ("" after a successful call). */
SQG_API const char* sqg_last_error(void);

/* sizeof of the argument structs, so bindings can check their mirrors:
 * which = 0 sqg_range, 1 sqg_layout, 2 sqg_qkv_args, 3 sqg_attn_args,
 * 4 sqg_qrecompute_args, 5 sqg_staged_kv; else -1. */
SQG_API int64_t sqg_struct_size(int which);

/* Host only.  Row chunks of `size` rows over [0, n); a last chunk shorter than
 * `min_tail` joins the previous one; size <= 0 or size >= n gives one chunk
 * ([VL] helpers section, `_ranges`).  Writes at most `cap` (begin, end) pairs to
 * `begins`/`ends` (host) and the total count to *count. */
SQG_API int sqg_chunk_ranges(int64_t n, int64_t size, int64_t min_tail, int64_t* begins,
                             int64_t* ends, int32_t cap, int32_t* count);

/* Host only.  Validates a token-range precision policy ([FR] "Mixed precision for
 * conditioning") and fills the packed-store layout.  Ranges must be sorted,
 * contiguous, non-empty, cover [0, n_tokens), have interior boundaries that are
 * multiples of 128, and number at most SQG_MAX_SEGMENTS; n_ranges 0 = all INT4.
 * d_model must be 128 * n_heads, n_heads at most 64. */
SQG_API int sqg_kv_layout(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                          const sqg_range* ranges, int32_t n_ranges, sqg_layout* out);

/* Host only.  Byte offset of the row of (head, token) in the kpack (vpack) buffer
 * laid out by *layout (a full or a block store); -1 if the head or the token is
 * outside the layout. */
SQG_API int64_t sqg_kv_row_offset(const sqg_layout* layout, int32_t head, int64_t token);

/* Host only.  Layout of the block store that holds keys [key_begin, key_end) of the
 * sequence the policy describes (see sqg_layout).  key_begin must be a multiple of 128
 * and 0 <= key_begin < key_end <= n_tokens. */
SQG_API int sqg_kv_block_layout(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                                const sqg_range* ranges, int32_t n_ranges, int64_t key_begin,
                                int64_t key_end, sqg_layout* out);

/* Host only.  Buffer sizes of a host-staged store with blocks of block_rows keys:
 * sizes[0] = bytes of host_kpack (and of host_vpack), sizes[1] = bytes of host_kscale
 * (and host_vscale), sizes[2] = bytes of each dev_kpack / dev_vpack staging buffer (the
 * largest block), sizes[3] = bytes of each dev_kscale / dev_vscale staging buffer;
 * *n_blocks = the number of blocks. */
SQG_API int sqg_staged_sizes(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                             const sqg_range* ranges, int32_t n_ranges, int64_t block_rows,
                             int64_t sizes[4], int32_t* n_blocks);

/* Host only.  Split-half RoPE tables for positions [pos0, pos0 + n): cos and sin of
 * pos * theta^(-2i/128), i in [0, 64), computed in fp64 and rounded to fp32, into the
 * host arrays cos_out / sin_out ([n, 64] each). */
SQG_API int sqg_rope_table(int64_t pos0, int64_t n, double theta, float* cos_out, float* sin_out);

/* The streamed QKV projection with its quantising epilogue ([FR] "Proposed backend
 * capability"; [VL] block section `_phase1_kv`).  For the rows of each chunk of
 * `chunk_rows` it computes y = x W (bf16 inputs, fp32 accumulation), never storing
 * the fused [N, 3d] tensor:
 *   - q = y[:, 0:d], k = y[:, d:2d], v = y[:, 2d:3d], per head of 128;
 *   - if norm weights are given: per-head RMSNorm of q and k; if RoPE tables are
 *     given: split-half RoPE of q and k ([VL] helpers `_norm_rope`);
 *   - Q = bf16(q) stored in the model basis;
 *   - K and V: r = u H / sqrt(128) (Sylvester Hadamard, [VL] kvi8r `_hadamard`),
 *     per group of 32 with a = max|r|: INT4 s = fp16(a / 7 in fp32, rounded up to 8
 *     significant bits), INT8 s = fp16(a * fp32((1 + 2^-7) / 127)) (round to nearest
 *     even); code = clamp(rne(r / s), +-qmax) with qmax 7 (INT4) or 127 (INT8 ranges),
 *     IEEE fp32 division; packed per sqg_kv_layout.
 * Chunks only partition the launches: results do not depend on chunk_rows.  `emit`
 * restricts the launch to Q or to the K/V store; what it writes is identical to the
 * same part of a full call. */
SQG_API int sqg_streamed_qkv_quant(const sqg_qkv_args* args, void* stream);

/* Flash-style attention that reads the packed K/V tile by tile ([FR] "Proposed
 * backend capability", "Dense fallback is important"; [VL] kvi8r
 * `_blockwise_attention_q`): each query tile is rotated once by H/sqrt(128),
 * scores and P.V run against K/V dequantised in on-chip memory in the rotated
 * basis, blocks combine by online softmax, and the output is rotated back once.
 * Non-causal, no mask.  O = softmax(scale * Q K^T) V and lse = ln sum exp(scale * Q K^T)
 * over keys [kv_begin, kv_end).  kv_block > 0 names the pages' key blocks ([VL] kvi8r
 * `_online_combine`): one launch walks every block, and continuing the running
 * maximum, sum and output across a block boundary is the log-sum-exp merge of the
 * blocks' partial (O, lse), so the result equals the merge of per-block passes up to
 * fp32 rounding; kv_block is validated (multiple of 128) and requires lse.
 * accumulate = 1 merges into the (O, lse) already in the buffers (requires
 * o_dtype SQG_F32).  Errors are reported before anything is enqueued; a store whose
 * code bytes of one (segment, head), or whose scales of one head, exceed 2 GiB is
 * SQG_ERR_UNSUPPORTED (the kernel's 32-bit buffer ranges). */
SQG_API int sqg_packed_kv_attention(const sqg_attn_args* args, void* stream);

/* Host only.  Bytes of the Q workspace sqg_packed_kv_attention_qrecompute needs for
 * query rows [q_begin, q_end) (n_query_rows = q_end - q_begin) in chunks of
 * q_chunk_rows (0 = the default of sqg_qrecompute_args) at d_model: the largest chunk's
 * rows * d_model * 2.  Returns -1 for invalid arguments. */
SQG_API int64_t sqg_qrecompute_workspace_bytes(int64_t n_query_rows, int64_t q_chunk_rows,
                                               int32_t d_model);

/* Attention with Q recomputed per query chunk ([VL] block sections `_phase2_q_attn`
 * and the three-phase streamed block): for each chunk of q_chunk_rows query rows,
 * Q = bf16 of the projection of those rows (with the same RMSNorm / RoPE as
 * sqg_streamed_qkv_quant) is written to the workspace and the chunk attends to the
 * packed store exactly as sqg_packed_kv_attention does.  With a store written by
 * SQG_EMIT_KV, no [N, d] Q buffer exists: the device working set is the K/V store
 * plus one chunk of Q.  Results equal sqg_streamed_qkv_quant (SQG_EMIT_Q) followed by
 * sqg_packed_kv_attention bit for bit. */
SQG_API int sqg_packed_kv_attention_qrecompute(const sqg_qrecompute_args* args, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sqg_packed_kv_attention_qrecompute
 * with the one-chunk Q workspace taken from a fixed device scratch of
 * sqg_noalloc_scratch_bytes() bytes (64 MiB) that the library holds on every GPU it runs
 * on until the process ends.  args->workspace must be NULL and args->workspace_bytes 0.
 * With q_chunk_rows 0 the chunk is the default one shrunk to the largest multiple of 256
 * rows whose chunks (a folded tail of up to 511 rows included) fit the scratch: 4096 rows at
 * d_model 7168.  An explicit q_chunk_rows whose chunks do not fit, or a d_model for which
 * 256 rows do not, returns SQG_ERR_WORKSPACE_TOO_SMALL.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine); the scratch's
 * device address is looked up once per device (hipGetSymbolAddress) on the first call
 * with that device current.  Every call on one GPU shares that GPU's scratch, which keeps
 * the last call's contents (each chunk's Q is written before it is read, so nothing needs
 * clearing): calls that overlap in time on one GPU (other streams, other threads) race
 * and must not be issued.  Results equal sqg_packed_kv_attention_qrecompute bit for bit. */
SQG_API int sqg_packed_kv_attention_qrecompute_noalloc(const sqg_qrecompute_args* args, void* stream);

/* Bytes of the device scratch sqg_packed_kv_attention_qrecompute_noalloc uses. */
SQG_API int64_t sqg_noalloc_scratch_bytes(void);

/* sqg_streamed_qkv_quant with the packed K/V kept in host memory: for each key block,
 * the kernel writes the block's K/V into a device staging block store (alternating
 * between the two) and an asynchronous copy moves it to the block's place in the host
 * store.  args->kpack, vpack, kscale and vscale are ignored; Q (unless emit is
 * SQG_EMIT_KV) goes to args->q as usual; chunk_rows and min_tail are ignored (each block
 * is one launch).  Every copy and launch is enqueued on `stream`, in order; the host
 * store is complete once the stream has reached the end of the call.  emit
 * SQG_EMIT_Q is rejected (there is no K/V to stage). */
SQG_API int sqg_streamed_qkv_quant_staged(const sqg_qkv_args* args, const sqg_staged_kv* staged,
                                          void* stream);

/* sqg_packed_kv_attention against a host-staged store: for each block that meets
 * [kv_begin, kv_end), an asynchronous copy brings the block into a device staging
 * block store and the attention kernel processes its keys, merged into (O, LSE)
 * through the log-sum-exp ([VL] kvi8r section, `_online_combine`).  The blocks take
 * the place of kv_block (args->kv_block is ignored), so with more than one block an
 * lse buffer and SQG_F32 output are required.  args->kpack, vpack, kscale, vscale are
 * ignored.  Results equal one sqg_packed_kv_attention call per block on the device
 * store (keys [block begin, block end), accumulate after the first) bit for bit, and
 * the single-launch device path with kv_block = block_rows up to fp32 rounding.  The
 * device never holds more than two blocks of K/V. */
SQG_API int sqg_packed_kv_attention_staged(const sqg_attn_args* args, const sqg_staged_kv* staged,
                                           void* stream);

/* Test entry: runs the kernels' own quantise-and-pack step on fp32 rotated vectors
 * r (device, [rows, 128]) with format fmt for every row; writes codes (device,
 * [rows, 64] bytes for INT4 or [rows, 128] for INT8) and scales (device, fp16
 * [rows, 4]).  rows >= 0. */
SQG_API int sqg_test_quant_pack_f32(const float* r, int64_t rows, int32_t fmt, void* codes,
                                    void* scales, void* stream);

/* Test entry: runs the kernels' own in-register 128-point Hadamard butterfly on
 * in (device, fp32 [rows, 128]) into out; normalize = 1 multiplies by 1/sqrt(128). */
SQG_API int sqg_test_fwht_f32(const float* in, float* out, int64_t rows, int32_t normalize,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SQG_H */

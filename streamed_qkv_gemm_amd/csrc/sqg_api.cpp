// C-ABI entry points of libsqg.so: argument checking, the packed-store layout, the
// token-range policy, the row-chunk scheduler and the launch loops.  Plain C++17
// with no HIP headers: every check runs on the host before anything is enqueued,
// and the kernels are reached only through the launchers in internal.h.
#define SQG_BUILDING_LIBRARY 1
#include "../../include/sqg.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.h"

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int ok() {
  g_last_error.clear();
  return SQG_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Row chunks of `size` over [0, n) with a short remainder folded (VRAM Lab page, helpers
// section, `_ranges`: a last chunk under min_tail rows joins the one before it).  The
// last chunk starts at the last multiple of `size` below n, or one chunk earlier when
// fewer than min_tail rows would follow it; every chunk before it is `size` rows.
std::vector<std::pair<int64_t, int64_t>> chunk_plan(int64_t n, int64_t size, int64_t min_tail) {
  std::vector<std::pair<int64_t, int64_t>> out;
  if (size <= 0 || size >= n) {
    out.emplace_back(0, n);
    return out;
  }
  int64_t last = ((n - 1) / size) * size;
  if (last > 0 && n - last < min_tail) last -= size;
  for (int64_t b = 0; b < last; b += size) out.emplace_back(b, b + size);
  out.emplace_back(last, n);
  return out;
}

int format_row_bytes(int32_t fmt) { return fmt == SQG_INT4_ROT ? 64 : (fmt == SQG_INT8_ROT ? 128 : 256); }

// Bytes of one token's rows over heads [0, h) of segment s: INT8 heads of an INT4
// segment take 64 bytes more than the others.
int64_t segment_row_units(const sqg_layout& L, int s, int h) {
  const uint64_t below = h >= 64 ? L.seg_int8_heads[s] : (L.seg_int8_heads[s] & ((1ull << h) - 1ull));
  return (int64_t)L.seg_row_bytes[s] * h + 64 * (int64_t)__builtin_popcountll(below);
}

int build_layout(int64_t n, int32_t d, int32_t heads, const sqg_range* ranges, int32_t n_ranges,
                 sqg_layout* L) {
  if (n < 0) return fail(SQG_ERR_INVALID_ARGUMENT, "n_tokens must be >= 0 (got %lld)", (long long)n);
  if (heads < 1 || d != heads * SQG_HEAD_DIM)
    return fail(SQG_ERR_INVALID_ARGUMENT, "d_model (%d) must equal 128 * n_heads (%d)", d, heads);
  if (heads > 64) return fail(SQG_ERR_UNSUPPORTED, "at most 64 heads (got %d)", heads);
  if (n_ranges < 0 || n_ranges > SQG_MAX_SEGMENTS)
    return fail(SQG_ERR_INVALID_ARGUMENT, "n_ranges must be in [0, %d] (got %d)", SQG_MAX_SEGMENTS,
                n_ranges);
  if (n_ranges > 0 && !ranges) return fail(SQG_ERR_INVALID_ARGUMENT, "ranges is NULL");
  std::memset(L, 0, sizeof *L);
  L->n_tokens = n;
  L->n_heads = heads;
  if (n_ranges == 0) {
    if (n > 0) {
      L->n_segments = 1;
      L->seg_begin[0] = 0;
      L->seg_end[0] = n;
      L->seg_fmt[0] = SQG_INT4_ROT;
    }
  } else {
    int64_t pos = 0;
    for (int i = 0; i < n_ranges; ++i) {
      const sqg_range& r = ranges[i];
      if (r.fmt != SQG_INT4_ROT && r.fmt != SQG_INT8_ROT && r.fmt != SQG_BF16_ROT)
        return fail(SQG_ERR_INVALID_ARGUMENT, "range %d: unknown format %d", i, r.fmt);
      if (r.reserved != 0) return fail(SQG_ERR_INVALID_ARGUMENT, "range %d: reserved field not 0", i);
      if (r.int8_heads != 0 && r.fmt != SQG_INT4_ROT)
        return fail(SQG_ERR_INVALID_ARGUMENT, "range %d: int8_heads applies to INT4 ranges only", i);
      if (heads < 64 && (r.int8_heads >> heads) != 0)
        return fail(SQG_ERR_INVALID_ARGUMENT, "range %d: int8_heads names a head >= n_heads", i);
      if (r.begin != pos)
        return fail(SQG_ERR_INVALID_ARGUMENT,
                    "range %d begins at %lld, expected %lld (ranges must be sorted and contiguous)",
                    i, (long long)r.begin, (long long)pos);
      if (r.end <= r.begin)
        return fail(SQG_ERR_INVALID_ARGUMENT, "range %d is empty or reversed", i);
      if (r.end < n && r.end % 128 != 0)
        return fail(SQG_ERR_INVALID_ARGUMENT, "range %d: interior boundary %lld is not a multiple of 128",
                    i, (long long)r.end);
      L->seg_begin[i] = r.begin;
      L->seg_end[i] = r.end;
      L->seg_fmt[i] = r.fmt;
      L->seg_int8_heads[i] = r.int8_heads;
      pos = r.end;
    }
    if (pos != n)
      return fail(SQG_ERR_INVALID_ARGUMENT, "ranges end at %lld, not at n_tokens %lld", (long long)pos,
                  (long long)n);
    L->n_segments = n_ranges;
  }
  int64_t off = 0;
  for (int s = 0; s < L->n_segments; ++s) {
    L->seg_row_bytes[s] = format_row_bytes(L->seg_fmt[s]);
    L->seg_offset[s] = off;
    off += (L->seg_end[s] - L->seg_begin[s]) * segment_row_units(*L, s, heads);
  }
  L->pack_bytes = off;
  L->scale_bytes = n * heads * 4 * 2;
  L->q_bytes = n * (int64_t)d * 2;
  L->bf16_qkv_bytes = 3 * L->q_bytes;
  return SQG_OK;
}

// Block store of keys [k0, k1): the policy's segments clipped to the block, packed one
// after another as in a full store of k1 - k0 tokens.
int build_block_layout(const sqg_layout& full, int32_t d, int64_t k0, int64_t k1, sqg_layout* B) {
  if (k0 < 0 || k1 <= k0 || k1 > full.n_tokens)
    return fail(SQG_ERR_INVALID_ARGUMENT, "key block [%lld, %lld) is empty or outside [0, %lld]",
                (long long)k0, (long long)k1, (long long)full.n_tokens);
  if (k0 % 128 != 0) return fail(SQG_ERR_INVALID_ARGUMENT, "key block start %lld is not a multiple of 128",
                                 (long long)k0);
  std::memset(B, 0, sizeof *B);
  B->n_tokens = k1 - k0;
  B->n_heads = full.n_heads;
  int64_t off = 0;
  for (int s = 0; s < full.n_segments; ++s) {
    const int64_t b = full.seg_begin[s] > k0 ? full.seg_begin[s] : k0;
    const int64_t e = full.seg_end[s] < k1 ? full.seg_end[s] : k1;
    if (b >= e) continue;
    const int i = B->n_segments++;
    B->seg_begin[i] = b;
    B->seg_end[i] = e;
    B->seg_fmt[i] = full.seg_fmt[s];
    B->seg_row_bytes[i] = full.seg_row_bytes[s];
    B->seg_int8_heads[i] = full.seg_int8_heads[s];
    B->seg_offset[i] = off;
    off += (e - b) * segment_row_units(full, s, full.n_heads);
  }
  B->pack_bytes = off;
  B->scale_bytes = B->n_tokens * full.n_heads * 4 * 2;
  B->q_bytes = B->n_tokens * (int64_t)d * 2;
  B->bf16_qkv_bytes = 3 * B->q_bytes;
  return SQG_OK;
}

// Blocks of a host-staged store with their layouts and host offsets.
struct StagedBlock {
  int64_t k0, k1;
  int64_t pack_off, scale_off;  // byte offsets in the host buffers
  sqg_layout L;
};

int staged_plan(const sqg_layout& full, int32_t d, int64_t block_rows, std::vector<StagedBlock>* out) {
  if (block_rows <= 0 || block_rows % 128 != 0)
    return fail(SQG_ERR_INVALID_ARGUMENT, "block_rows must be a positive multiple of 128 (got %lld)",
                (long long)block_rows);
  out->clear();
  if (full.n_tokens == 0) return SQG_OK;
  int64_t po = 0, so = 0;
  for (const auto& c : chunk_plan(full.n_tokens, block_rows, 512)) {
    StagedBlock b;
    b.k0 = c.first;
    b.k1 = c.second;
    b.pack_off = po;
    b.scale_off = so;
    const int st = build_block_layout(full, d, b.k0, b.k1, &b.L);
    if (st != SQG_OK) return st;
    po += b.L.pack_bytes;
    so += b.L.scale_bytes;
    out->push_back(b);
  }
  return SQG_OK;
}

int check_staged(const sqg_staged_kv* s) {
  if (!s) return fail(SQG_ERR_INVALID_ARGUMENT, "staged is NULL");
  if (!s->host_kpack || !s->host_vpack || !s->host_kscale || !s->host_vscale)
    return fail(SQG_ERR_INVALID_ARGUMENT, "a host buffer of the staged store is NULL");
  for (int i = 0; i < 2; ++i) {
    const void* d[] = {s->dev_kpack[i], s->dev_vpack[i], s->dev_kscale[i], s->dev_vscale[i]};
    for (const void* ptr : d) {
      if (!ptr) return fail(SQG_ERR_INVALID_ARGUMENT, "a device staging buffer is NULL");
      if (!aligned16(ptr)) return fail(SQG_ERR_MISALIGNED, "staging buffer %p is not 16-byte aligned", ptr);
    }
  }
  return SQG_OK;
}

sqg::SegTable seg_table(const sqg_layout& L) {
  sqg::SegTable t;
  std::memset(&t, 0, sizeof t);
  t.n = L.n_segments;
  for (int s = 0; s < L.n_segments; ++s) {
    t.fmt[s] = L.seg_fmt[s];
    t.begin[s] = L.seg_begin[s];
    t.end[s] = L.seg_end[s];
    t.offset[s] = L.seg_offset[s];
    t.int8_heads[s] = L.seg_int8_heads[s];
  }
  return t;
}

int launch_status(int hip_err, const char* what) {
  if (hip_err != 0)
    return fail(SQG_ERR_HIP, "%s: HIP error %d (%s)", what, hip_err, sqg::hip_error_text(hip_err));
  return SQG_OK;
}

// Events of one staged call with a copy stream: the entry point on the call's stream,
// and per staging slot the kernel that last used it and its last copy.  Destroyed on
// return, pending or not (the runtime releases them once they complete).
struct StageEvents {
  void* ev[5] = {nullptr, nullptr, nullptr, nullptr, nullptr};
  ~StageEvents() {
    for (void* e : ev) sqg::event_destroy(e);
  }
  int create() {
    for (void*& e : ev) {
      const int r = sqg::event_create(&e);
      if (r) return r;
    }
    return 0;
  }
  void* start() const { return ev[0]; }
  void* kernel(int slot) const { return ev[1 + slot]; }
  void* copy(int slot) const { return ev[3 + slot]; }
};

// With a copy stream: create the events and let the copy stream wait for the work
// already enqueued on the call's stream.
int stage_begin(StageEvents& E, void* copy_stream, void* stream) {
  int st = launch_status(E.create(), "staging events");
  if (st != SQG_OK) return st;
  st = launch_status(sqg::event_record(E.start(), stream), "staging event record");
  if (st != SQG_OK) return st;
  return launch_status(sqg::stream_wait_event(copy_stream, E.start()), "staging stream wait");
}

// `waiter` waits for `ev` after recording it on `recorder` (no-op without a copy stream)
int stage_order(void* ev, void* recorder, void* waiter) {
  int st = launch_status(sqg::event_record(ev, recorder), "staging event record");
  if (st != SQG_OK) return st;
  return launch_status(sqg::stream_wait_event(waiter, ev), "staging stream wait");
}

// Checks the attention arguments and fills the kernel parameters.  With check_q false
// the caller supplies Q itself (a->q and a->ldq are ignored).  *empty is set when there
// is nothing to compute.
int attn_prepare(const sqg_attn_args* a, bool check_q, sqg::AttnParams* p, int64_t* kv_end_out,
                 bool* empty) {
  *empty = false;
  sqg_layout L;
  int st = build_layout(a->n_tokens, a->d_model, a->n_heads, a->ranges, a->n_ranges, &L);
  if (st != SQG_OK) return st;
  const int64_t N = a->n_tokens;
  const int64_t d = a->d_model;
  if (a->o_dtype != SQG_F32 && a->o_dtype != SQG_BF16 && a->o_dtype != SQG_F16)
    return fail(SQG_ERR_INVALID_ARGUMENT, "unknown o_dtype %d", a->o_dtype);
  const int64_t q_end = a->q_end == 0 ? N : a->q_end;
  const int64_t kv_end = a->kv_end == 0 ? N : a->kv_end;
  if (a->q_begin < 0 || a->q_begin > q_end || q_end > N)
    return fail(SQG_ERR_INVALID_ARGUMENT, "query range [%lld, %lld) is outside [0, %lld]",
                (long long)a->q_begin, (long long)q_end, (long long)N);
  if (a->kv_block < 0 || a->kv_block % 128 != 0)
    return fail(SQG_ERR_INVALID_ARGUMENT, "kv_block must be 0 or a positive multiple of 128");
  if (a->accumulate != 0 && a->accumulate != 1)
    return fail(SQG_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1");
  if ((a->accumulate || a->kv_block > 0) && (!a->lse || a->o_dtype != SQG_F32))
    return fail(SQG_ERR_INVALID_ARGUMENT,
                "accumulate and kv_block > 0 need an lse buffer and o_dtype SQG_F32");
  if (!(std::isfinite(a->softmax_scale) && a->softmax_scale >= 0.0f))
    return fail(SQG_ERR_INVALID_ARGUMENT, "softmax_scale must be finite and >= 0");
  if (a->qk_mode != SQG_QK_EXACT && a->qk_mode != SQG_QK_FP8)
    return fail(SQG_ERR_INVALID_ARGUMENT, "unknown qk_mode %d", a->qk_mode);
  if (a->reserved != 0) return fail(SQG_ERR_INVALID_ARGUMENT, "attention reserved field not 0");
  // the kernel reads each (segment, head) block of codes and each head's scale rows
  // through buffer resources whose byte length is a 32-bit field
  if (N * 8 > 0x7fffffffLL)
    return fail(SQG_ERR_UNSUPPORTED, "a head's scales span %lld bytes, more than a 2 GiB buffer resource",
                (long long)(N * 8));
  for (int s = 0; s < L.n_segments; ++s) {
    const int64_t rows = L.seg_end[s] - L.seg_begin[s];
    for (int h = 0; h < L.n_heads; ++h) {
      const bool int8 = L.seg_fmt[s] == SQG_INT4_ROT && ((L.seg_int8_heads[s] >> h) & 1ull);
      const int64_t bytes = rows * (int8 ? 128 : L.seg_row_bytes[s]);
      if (bytes > 0x7fffffffLL)
        return fail(SQG_ERR_UNSUPPORTED,
                    "range %d holds %lld bytes of codes per head, more than a 2 GiB buffer resource",
                    s, (long long)bytes);
    }
  }
  if (N == 0 || q_end == a->q_begin) {
    *empty = true;
    return SQG_OK;
  }
  if (a->kv_begin < 0 || a->kv_begin >= kv_end || kv_end > N)
    return fail(SQG_ERR_INVALID_ARGUMENT, "key range [%lld, %lld) is empty or outside [0, %lld]",
                (long long)a->kv_begin, (long long)kv_end, (long long)N);
  if (a->kv_begin % 128 != 0)
    return fail(SQG_ERR_INVALID_ARGUMENT, "kv_begin must be a multiple of 128");
  if ((check_q && !a->q) || !a->kpack || !a->vpack || !a->kscale || !a->vscale || !a->o)
    return fail(SQG_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if ((check_q && a->ldq < d) || a->ldo < d)
    return fail(SQG_ERR_INVALID_ARGUMENT, "row strides must be >= d_model");
  if ((check_q && a->ldq % 8) || a->ldo % 8)
    return fail(SQG_ERR_MISALIGNED, "row strides must be multiples of 8");
  const void* ptrs[] = {check_q ? a->q : nullptr, a->kpack, a->vpack, a->kscale, a->vscale, a->o, a->lse};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(SQG_ERR_MISALIGNED, "device pointer %p is not 16-byte aligned", ptr);

  std::memset(p, 0, sizeof *p);
  p->q = static_cast<const uint16_t*>(a->q);
  p->kpack = static_cast<const uint8_t*>(a->kpack);
  p->vpack = static_cast<const uint8_t*>(a->vpack);
  p->kscale = static_cast<const uint16_t*>(a->kscale);
  p->vscale = static_cast<const uint16_t*>(a->vscale);
  p->o = a->o;
  p->lse = a->lse;
  p->ldq = a->ldq;
  p->ldo = a->ldo;
  p->n_tokens = N;
  p->q_begin = a->q_begin;
  p->q_end = q_end;
  p->q_row0 = 0;
  p->kv_row0 = 0;
  p->kv_n = N;
  p->d_model = a->d_model;
  p->n_heads = a->n_heads;
  p->o_dtype = a->o_dtype;
  p->qk_mode = a->qk_mode;
  const double scale = a->softmax_scale > 0.0f ? (double)a->softmax_scale : 1.0 / std::sqrt(128.0);
  p->scale_log2 = (float)(scale * 1.4426950408889634);
  p->seg = seg_table(L);
  *kv_end_out = kv_end;
  return SQG_OK;
}

// Checks the QKV-quant arguments and fills the kernel parameters (all rows, the whole
// store).  With check_store false the K/V store pointers are not checked (the caller
// substitutes its own).  *empty is set when there is nothing to compute.
int qkv_prepare(const sqg_qkv_args* a, bool check_store, sqg::QkvParams* pp, sqg_layout* Lout,
                bool* empty) {
  *empty = false;
  sqg_layout& L = *Lout;
  int st = build_layout(a->n_tokens, a->d_model, a->n_heads, a->ranges, a->n_ranges, &L);
  if (st != SQG_OK) return st;
  const int64_t N = a->n_tokens;
  const int64_t d = a->d_model;
  if (d % 256 != 0)
    return fail(SQG_ERR_UNSUPPORTED, "d_model must be a multiple of 256 (got %lld)", (long long)d);
  if (d * a->ldw * 2 > 0x7fffffffLL || 256 * a->ldx * 2 > 0x7fffffffLL)
    return fail(SQG_ERR_UNSUPPORTED, "W (or a 256-row slice of x) exceeds the 2 GiB a buffer resource addresses");
  if (a->emit != SQG_EMIT_QKV && a->emit != SQG_EMIT_Q && a->emit != SQG_EMIT_KV)
    return fail(SQG_ERR_INVALID_ARGUMENT, "unknown emit mode %d", a->emit);
  const bool want_q = a->emit != SQG_EMIT_KV;
  const bool want_kv = a->emit != SQG_EMIT_Q && check_store;
  if ((a->q_norm_w == nullptr) != (a->k_norm_w == nullptr))
    return fail(SQG_ERR_INVALID_ARGUMENT, "q_norm_w and k_norm_w must both be set or both be NULL");
  if ((a->rope_cos == nullptr) != (a->rope_sin == nullptr))
    return fail(SQG_ERR_INVALID_ARGUMENT, "rope_cos and rope_sin must both be set or both be NULL");
  if (a->q_norm_w && !(a->eps >= 0.0f && std::isfinite(a->eps)))
    return fail(SQG_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (a->chunk_rows < 0 || a->chunk_rows % 128 != 0)
    return fail(SQG_ERR_INVALID_ARGUMENT, "chunk_rows must be 0 or a positive multiple of 128 (got %lld)",
                (long long)a->chunk_rows);
  if (N == 0) {
    *empty = true;
    return SQG_OK;
  }
  if (!a->x || !a->w_qkv || (want_q && !a->q) ||
      (want_kv && (!a->kpack || !a->vpack || !a->kscale || !a->vscale)))
    return fail(SQG_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  const int64_t ldq = want_q ? a->ldq : d;
  if (a->ldx < d || a->ldw < 3 * d || ldq < d)
    return fail(SQG_ERR_INVALID_ARGUMENT, "row strides must be >= the row length (ldx %lld, ldw %lld, ldq %lld)",
                (long long)a->ldx, (long long)a->ldw, (long long)ldq);
  if (a->ldx % 8 || a->ldw % 8 || ldq % 8)
    return fail(SQG_ERR_MISALIGNED, "row strides must be multiples of 8 elements");
  const void* ptrs[] = {a->x, a->w_qkv, want_q ? a->q : nullptr,
                        want_kv ? a->kpack : nullptr, want_kv ? a->vpack : nullptr,
                        want_kv ? a->kscale : nullptr, want_kv ? a->vscale : nullptr,
                        a->q_norm_w, a->k_norm_w, a->rope_cos, a->rope_sin};
  for (const void* p : ptrs)
    if (p && !aligned16(p)) return fail(SQG_ERR_MISALIGNED, "device pointer %p is not 16-byte aligned", p);

  sqg::QkvParams& p = *pp;
  std::memset(&p, 0, sizeof p);
  p.x = static_cast<const uint16_t*>(a->x);
  p.w = static_cast<const uint16_t*>(a->w_qkv);
  p.q = want_q ? static_cast<uint16_t*>(a->q) : nullptr;
  p.kpack = want_kv ? static_cast<uint8_t*>(a->kpack) : nullptr;
  p.vpack = want_kv ? static_cast<uint8_t*>(a->vpack) : nullptr;
  p.kscale = want_kv ? static_cast<uint16_t*>(a->kscale) : nullptr;
  p.vscale = want_kv ? static_cast<uint16_t*>(a->vscale) : nullptr;
  p.q_norm_w = a->q_norm_w;
  p.k_norm_w = a->k_norm_w;
  p.rope_cos = a->rope_cos;
  p.rope_sin = a->rope_sin;
  p.ldx = a->ldx;
  p.ldw = a->ldw;
  p.ldq = ldq;
  p.n_tokens = N;
  p.q_row0 = 0;
  p.d_model = a->d_model;
  p.n_heads = a->n_heads;
  p.eps = a->eps;
  p.col_tile0 = want_q ? 0 : (int32_t)(d / 256);
  p.n_col_tiles = (int32_t)((want_q ? d / 256 : 0) + (a->emit != SQG_EMIT_Q ? 2 * d / 256 : 0));
  p.seg = seg_table(L);
  p.kv_row0 = 0;
  p.kv_n = N;
  p.row_begin = 0;
  p.row_end = N;
  return SQG_OK;
}

// One attention pass of p's query rows over keys [kv_begin, kv_end) (`accumulate` merges
// into the (O, LSE) already in the buffers), as one launch whatever kv_block is.  The
// kernel walks the key range tile by tile keeping the running maximum, sum and
// unnormalised O of each query in registers; merging a block's partial (o_b, lse_b)
// into (o, lse) by the log-sum-exp rule of VRAM Lab's `_online_combine` gives exactly
// what continuing that running state over the block's keys gives (both are
// sum_j e^(s_j) v_j / sum_j e^(s_j) over the keys so far), so the KV blocks are merged
// in registers as the walk crosses them, and O, LSE and Q are read and written once.
int attn_launch_blocks(sqg::AttnParams p, int64_t kv_begin, int64_t kv_end, int32_t accumulate,
                       void* stream) {
  p.kv_begin = kv_begin;
  p.kv_end = kv_end;
  p.accumulate = accumulate;
  return launch_status(sqg::launch_packed_attention(p, stream), "packed_kv_attention launch");
}

// Default query chunk of the Q-recompute mode: 16384 rows, or more when there are few
// heads, so that one attention launch still has at least 2048 workgroups (8 per CU).
int64_t default_q_chunk(int64_t heads) {
  const int64_t rows = 256 * ((2048 + heads - 1) / heads);
  return rows > 16384 ? rows : 16384;
}

}  // namespace

extern "C" {

SQG_API int sqg_version(void) { return SQG_VERSION; }

SQG_API const char* sqg_status_string(int status) {
  switch (status) {
    case SQG_OK: return "ok";
    case SQG_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SQG_ERR_UNSUPPORTED: return "unsupported shape";
    case SQG_ERR_MISALIGNED: return "misaligned pointer or stride";
    case SQG_ERR_WORKSPACE_TOO_SMALL: return "workspace too small";
    case SQG_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

SQG_API const char* sqg_last_error(void) { return g_last_error.c_str(); }

SQG_API int64_t sqg_struct_size(int which) {
  switch (which) {
    case 0: return (int64_t)sizeof(sqg_range);
    case 1: return (int64_t)sizeof(sqg_layout);
    case 2: return (int64_t)sizeof(sqg_qkv_args);
    case 3: return (int64_t)sizeof(sqg_attn_args);
    case 4: return (int64_t)sizeof(sqg_qrecompute_args);
    case 5: return (int64_t)sizeof(sqg_staged_kv);
    default: return -1;
  }
}

SQG_API int sqg_chunk_ranges(int64_t n, int64_t size, int64_t min_tail, int64_t* begins,
                             int64_t* ends, int32_t cap, int32_t* count) {
  if (n < 0) return fail(SQG_ERR_INVALID_ARGUMENT, "n must be >= 0");
  if (!count) return fail(SQG_ERR_INVALID_ARGUMENT, "count is NULL");
  if (cap > 0 && (!begins || !ends)) return fail(SQG_ERR_INVALID_ARGUMENT, "output arrays are NULL");
  const auto plan = chunk_plan(n, size, min_tail);
  *count = (int32_t)plan.size();
  for (size_t i = 0; i < plan.size() && (int32_t)i < cap; ++i) {
    begins[i] = plan[i].first;
    ends[i] = plan[i].second;
  }
  return ok();
}

SQG_API int sqg_kv_layout(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                          const sqg_range* ranges, int32_t n_ranges, sqg_layout* out) {
  if (!out) return fail(SQG_ERR_INVALID_ARGUMENT, "out is NULL");
  const int st = build_layout(n_tokens, d_model, n_heads, ranges, n_ranges, out);
  return st == SQG_OK ? ok() : st;
}

SQG_API int64_t sqg_kv_row_offset(const sqg_layout* L, int32_t head, int64_t token) {
  if (!L || head < 0 || head >= L->n_heads) return -1;
  for (int s = 0; s < L->n_segments; ++s) {
    if (token < L->seg_begin[s] || token >= L->seg_end[s]) continue;
    const bool int8 = L->seg_fmt[s] == SQG_INT4_ROT && ((L->seg_int8_heads[s] >> head) & 1ull);
    const int64_t rb = int8 ? 128 : L->seg_row_bytes[s];
    return L->seg_offset[s] + (L->seg_end[s] - L->seg_begin[s]) * segment_row_units(*L, s, head) +
           (token - L->seg_begin[s]) * rb;
  }
  return -1;
}

SQG_API int sqg_kv_block_layout(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                                const sqg_range* ranges, int32_t n_ranges, int64_t key_begin,
                                int64_t key_end, sqg_layout* out) {
  if (!out) return fail(SQG_ERR_INVALID_ARGUMENT, "out is NULL");
  sqg_layout L;
  int st = build_layout(n_tokens, d_model, n_heads, ranges, n_ranges, &L);
  if (st != SQG_OK) return st;
  st = build_block_layout(L, d_model, key_begin, key_end, out);
  return st == SQG_OK ? ok() : st;
}

SQG_API int sqg_staged_sizes(int64_t n_tokens, int32_t d_model, int32_t n_heads,
                             const sqg_range* ranges, int32_t n_ranges, int64_t block_rows,
                             int64_t sizes[4], int32_t* n_blocks) {
  if (!sizes || !n_blocks) return fail(SQG_ERR_INVALID_ARGUMENT, "sizes or n_blocks is NULL");
  sqg_layout L;
  int st = build_layout(n_tokens, d_model, n_heads, ranges, n_ranges, &L);
  if (st != SQG_OK) return st;
  std::vector<StagedBlock> blocks;
  st = staged_plan(L, d_model, block_rows, &blocks);
  if (st != SQG_OK) return st;
  int64_t mp = 0, ms = 0;
  for (const auto& b : blocks) {
    mp = b.L.pack_bytes > mp ? b.L.pack_bytes : mp;
    ms = b.L.scale_bytes > ms ? b.L.scale_bytes : ms;
  }
  sizes[0] = L.pack_bytes;
  sizes[1] = L.scale_bytes;
  sizes[2] = mp;
  sizes[3] = ms;
  *n_blocks = (int32_t)blocks.size();
  return ok();
}

SQG_API int sqg_rope_table(int64_t pos0, int64_t n, double theta, float* cos_out, float* sin_out) {
  if (n < 0 || pos0 < 0) return fail(SQG_ERR_INVALID_ARGUMENT, "n and pos0 must be >= 0");
  if (n > 0 && (!cos_out || !sin_out)) return fail(SQG_ERR_INVALID_ARGUMENT, "output is NULL");
  if (!(theta > 1.0)) return fail(SQG_ERR_INVALID_ARGUMENT, "theta must be > 1");
  double inv[64];
  for (int i = 0; i < 64; ++i) inv[i] = std::pow(theta, -2.0 * i / 128.0);
  for (int64_t r = 0; r < n; ++r) {
    const double pos = (double)(pos0 + r);
    for (int i = 0; i < 64; ++i) {
      const double a = pos * inv[i];
      cos_out[r * 64 + i] = (float)std::cos(a);
      sin_out[r * 64 + i] = (float)std::sin(a);
    }
  }
  return ok();
}

SQG_API int sqg_streamed_qkv_quant(const sqg_qkv_args* a, void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  sqg::QkvParams p;
  sqg_layout L;
  bool empty = false;
  int st = qkv_prepare(a, true, &p, &L, &empty);
  if (st != SQG_OK) return st;
  if (empty) return ok();
  const int64_t min_tail = a->min_tail < 0 ? 512 : a->min_tail;
  for (const auto& c : chunk_plan(a->n_tokens, a->chunk_rows, min_tail)) {
    p.row_begin = c.first;
    p.row_end = c.second;
    st = launch_status(sqg::launch_qkv_quant(p, stream), "streamed_qkv_quant launch");
    if (st != SQG_OK) return st;
  }
  return ok();
}

SQG_API int sqg_packed_kv_attention(const sqg_attn_args* a, void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  sqg::AttnParams p;
  int64_t kv_end = 0;
  bool empty = false;
  int st = attn_prepare(a, true, &p, &kv_end, &empty);
  if (st != SQG_OK) return st;
  if (empty) return ok();
  st = attn_launch_blocks(p, a->kv_begin, kv_end, a->accumulate, stream);
  return st == SQG_OK ? ok() : st;
}

SQG_API int64_t sqg_qrecompute_workspace_bytes(int64_t n_query_rows, int64_t q_chunk_rows,
                                               int32_t d_model) {
  if (n_query_rows < 0 || q_chunk_rows < 0 || q_chunk_rows % 128 != 0 || d_model <= 0 ||
      d_model % SQG_HEAD_DIM != 0)
    return -1;
  const int64_t size = q_chunk_rows == 0 ? default_q_chunk(d_model / SQG_HEAD_DIM) : q_chunk_rows;
  int64_t rows = 0;
  for (const auto& c : chunk_plan(n_query_rows, size, 512))
    rows = c.second - c.first > rows ? c.second - c.first : rows;
  return rows * d_model * 2;
}

namespace {

// Q-recompute attention with the given Q workspace (the caller's, or the device scratch
// of the allocation-free entry); `scratch` chooses which the argument checks describe.
int qrecompute_run(const sqg_qrecompute_args* a, void* workspace, int64_t workspace_bytes,
                   bool scratch, void* stream) {
  const sqg_attn_args& at = a->attn;
  sqg::AttnParams ap;
  int64_t kv_end = 0;
  bool empty = false;
  int st = attn_prepare(&at, false, &ap, &kv_end, &empty);
  if (st != SQG_OK) return st;
  const int64_t d = at.d_model;
  if (d % 256 != 0)
    return fail(SQG_ERR_UNSUPPORTED, "d_model must be a multiple of 256 (got %lld)", (long long)d);
  if (a->reserved != 0) return fail(SQG_ERR_INVALID_ARGUMENT, "reserved field not 0");
  if (a->q_chunk_rows < 0 || a->q_chunk_rows % 128 != 0)
    return fail(SQG_ERR_INVALID_ARGUMENT, "q_chunk_rows must be 0 or a positive multiple of 128 (got %lld)",
                (long long)a->q_chunk_rows);
  if ((a->rope_cos == nullptr) != (a->rope_sin == nullptr))
    return fail(SQG_ERR_INVALID_ARGUMENT, "rope_cos and rope_sin must both be set or both be NULL");
  if (a->q_norm_w && !(a->eps >= 0.0f && std::isfinite(a->eps)))
    return fail(SQG_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
  if (scratch && (a->workspace || a->workspace_bytes))
    return fail(SQG_ERR_INVALID_ARGUMENT,
                "the allocation-free entry uses its own device scratch: workspace must be NULL and "
                "workspace_bytes 0");
  // chunk rows: the caller's, else the default; the scratch entry shrinks the default to
  // the largest multiple of 256 rows whose chunks fit its scratch (a last chunk may run
  // up to 511 rows longer, the folded tail)
  int64_t size = a->q_chunk_rows == 0 ? default_q_chunk(at.n_heads) : a->q_chunk_rows;
  if (scratch && a->q_chunk_rows == 0) {
    const int64_t fit_rows = workspace_bytes / (2 * d);
    const int64_t fit = fit_rows > 511 ? (fit_rows - 511) / 256 * 256 : 0;
    if (fit < size) size = fit;
    if (size <= 0)
      return fail(SQG_ERR_WORKSPACE_TOO_SMALL,
                  "chunks of 256 query rows (and a folded tail) of d_model %lld need %lld bytes, more "
                  "than the %lld-byte device scratch",
                  (long long)d, (long long)(767 * 2 * d), (long long)workspace_bytes);
  }
  if (empty) return ok();
  const int64_t n_q = ap.q_end - ap.q_begin;
  const int64_t need = sqg_qrecompute_workspace_bytes(n_q, size, at.d_model);
  if (!a->x || !a->w_qkv || (!scratch && !workspace))
    return fail(SQG_ERR_INVALID_ARGUMENT, "a required device pointer is NULL");
  if (workspace_bytes < need)
    return fail(SQG_ERR_WORKSPACE_TOO_SMALL, "%s holds %lld bytes, %lld needed for chunks of %lld rows",
                scratch ? "the device scratch" : "workspace", (long long)workspace_bytes,
                (long long)need, (long long)size);
  if (a->ldx < d || a->ldw < 3 * d)
    return fail(SQG_ERR_INVALID_ARGUMENT, "row strides must be >= the row length (ldx %lld, ldw %lld)",
                (long long)a->ldx, (long long)a->ldw);
  if (a->ldx % 8 || a->ldw % 8) return fail(SQG_ERR_MISALIGNED, "row strides must be multiples of 8 elements");
  if (d * a->ldw * 2 > 0x7fffffffLL || 256 * a->ldx * 2 > 0x7fffffffLL)
    return fail(SQG_ERR_UNSUPPORTED, "W (or a 256-row slice of x) exceeds the 2 GiB a buffer resource addresses");
  const void* ptrs[] = {a->x, a->w_qkv, workspace, a->q_norm_w, a->rope_cos, a->rope_sin};
  for (const void* ptr : ptrs)
    if (ptr && !aligned16(ptr)) return fail(SQG_ERR_MISALIGNED, "device pointer %p is not 16-byte aligned", ptr);
  if (scratch) {   // every argument is valid: the scratch's address on this device
    st = launch_status(sqg::scratch_for_current_device(&workspace), "device scratch lookup");
    if (st != SQG_OK) return st;
  }

  // Q-only projection of one chunk into the workspace (row t at row t - chunk start)
  sqg::QkvParams qp;
  std::memset(&qp, 0, sizeof qp);
  qp.x = static_cast<const uint16_t*>(a->x);
  qp.w = static_cast<const uint16_t*>(a->w_qkv);
  qp.q = static_cast<uint16_t*>(workspace);
  qp.q_norm_w = a->q_norm_w;
  qp.rope_cos = a->rope_cos;
  qp.rope_sin = a->rope_sin;
  qp.ldx = a->ldx;
  qp.ldw = a->ldw;
  qp.ldq = d;
  qp.n_tokens = at.n_tokens;
  qp.kv_row0 = 0;
  qp.kv_n = at.n_tokens;
  qp.d_model = at.d_model;
  qp.n_heads = at.n_heads;
  qp.eps = a->eps;
  qp.col_tile0 = 0;
  qp.n_col_tiles = (int32_t)(d / 256);
  qp.seg = ap.seg;

  ap.q = static_cast<const uint16_t*>(workspace);
  ap.ldq = d;
  for (const auto& c : chunk_plan(n_q, size, 512)) {
    const int64_t c0 = ap.q_begin + c.first;  // chunk offsets are relative to the range start
    const int64_t c1 = ap.q_begin + c.second;
    qp.row_begin = c0;
    qp.row_end = c1;
    qp.q_row0 = c0;
    st = launch_status(sqg::launch_qkv_quant(qp, stream), "q recompute launch");
    if (st != SQG_OK) return st;
    sqg::AttnParams cp = ap;
    cp.q_begin = c0;
    cp.q_end = c1;
    cp.q_row0 = c0;
    st = attn_launch_blocks(cp, at.kv_begin, kv_end, at.accumulate, stream);
    if (st != SQG_OK) return st;
  }
  return ok();
}

}  // namespace

SQG_API int sqg_packed_kv_attention_qrecompute(const sqg_qrecompute_args* a, void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  return qrecompute_run(a, a->workspace, a->workspace_bytes, false, stream);
}

SQG_API int sqg_packed_kv_attention_qrecompute_noalloc(const sqg_qrecompute_args* a, void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  return qrecompute_run(a, nullptr, sqg::kScratchBytes, true, stream);
}

SQG_API int64_t sqg_noalloc_scratch_bytes(void) { return sqg::kScratchBytes; }

SQG_API int sqg_streamed_qkv_quant_staged(const sqg_qkv_args* a, const sqg_staged_kv* sk,
                                          void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  if (a->emit == SQG_EMIT_Q)
    return fail(SQG_ERR_INVALID_ARGUMENT, "emit SQG_EMIT_Q writes no K/V to stage");
  sqg::QkvParams p;
  sqg_layout L;
  bool empty = false;
  int st = qkv_prepare(a, false, &p, &L, &empty);
  if (st != SQG_OK) return st;
  st = check_staged(sk);
  if (st != SQG_OK) return st;
  std::vector<StagedBlock> blocks;
  st = staged_plan(L, a->d_model, sk->block_rows, &blocks);
  if (st != SQG_OK) return st;
  if (empty) return ok();
  void* const cs = sk->copy_stream;
  void* const copy_stream = cs ? cs : stream;
  StageEvents E;
  if (cs) {
    st = stage_begin(E, cs, stream);
    if (st != SQG_OK) return st;
  }
  for (size_t i = 0; i < blocks.size(); ++i) {
    const StagedBlock& b = blocks[i];
    const int j = (int)(i & 1);
    if (cs && i >= 2) {   // slot j's previous block has left the device
      st = launch_status(sqg::stream_wait_event(stream, E.copy(j)), "staging stream wait");
      if (st != SQG_OK) return st;
    }
    p.kpack = static_cast<uint8_t*>(sk->dev_kpack[j]);
    p.vpack = static_cast<uint8_t*>(sk->dev_vpack[j]);
    p.kscale = static_cast<uint16_t*>(sk->dev_kscale[j]);
    p.vscale = static_cast<uint16_t*>(sk->dev_vscale[j]);
    p.seg = seg_table(b.L);
    p.kv_row0 = b.k0;
    p.kv_n = b.k1 - b.k0;
    p.row_begin = b.k0;
    p.row_end = b.k1;
    st = launch_status(sqg::launch_qkv_quant(p, stream), "streamed_qkv_quant launch");
    if (st != SQG_OK) return st;
    if (cs) {   // the copies start once this block's kernel is done
      st = stage_order(E.kernel(j), stream, cs);
      if (st != SQG_OK) return st;
    }
    char* hk = static_cast<char*>(sk->host_kpack) + b.pack_off;
    char* hv = static_cast<char*>(sk->host_vpack) + b.pack_off;
    char* hks = static_cast<char*>(sk->host_kscale) + b.scale_off;
    char* hvs = static_cast<char*>(sk->host_vscale) + b.scale_off;
    const int rc[4] = {
        sqg::copy_async(hk, sk->dev_kpack[j], b.L.pack_bytes, sqg::kDeviceToHost, copy_stream),
        sqg::copy_async(hv, sk->dev_vpack[j], b.L.pack_bytes, sqg::kDeviceToHost, copy_stream),
        sqg::copy_async(hks, sk->dev_kscale[j], b.L.scale_bytes, sqg::kDeviceToHost, copy_stream),
        sqg::copy_async(hvs, sk->dev_vscale[j], b.L.scale_bytes, sqg::kDeviceToHost, copy_stream)};
    for (int r : rc) {
      st = launch_status(r, "staging copy to host");
      if (st != SQG_OK) return st;
    }
    if (cs) {
      st = launch_status(sqg::event_record(E.copy(j), cs), "staging event record");
      if (st != SQG_OK) return st;
    }
  }
  if (cs) {   // the call's stream continues once the host store is complete
    for (size_t j = 0; j < blocks.size() && j < 2; ++j) {
      st = launch_status(sqg::stream_wait_event(stream, E.copy((int)j)), "staging stream wait");
      if (st != SQG_OK) return st;
    }
  }
  return ok();
}

SQG_API int sqg_packed_kv_attention_staged(const sqg_attn_args* a, const sqg_staged_kv* sk,
                                           void* stream) {
  if (!a) return fail(SQG_ERR_INVALID_ARGUMENT, "args is NULL");
  int st = check_staged(sk);
  if (st != SQG_OK) return st;
  // the store pointers are ignored: check the rest with the staging buffers in their place
  sqg_attn_args c = *a;
  c.kpack = sk->dev_kpack[0];
  c.vpack = sk->dev_vpack[0];
  c.kscale = sk->dev_kscale[0];
  c.vscale = sk->dev_vscale[0];
  c.kv_block = 0;
  sqg::AttnParams p;
  int64_t kv_end = 0;
  bool empty = false;
  st = attn_prepare(&c, true, &p, &kv_end, &empty);
  if (st != SQG_OK) return st;
  sqg_layout L;
  st = build_layout(a->n_tokens, a->d_model, a->n_heads, a->ranges, a->n_ranges, &L);
  if (st != SQG_OK) return st;
  std::vector<StagedBlock> blocks;
  st = staged_plan(L, a->d_model, sk->block_rows, &blocks);
  if (st != SQG_OK) return st;
  if (empty) return ok();
  std::vector<const StagedBlock*> meet;
  for (const auto& b : blocks)
    if (b.k1 > a->kv_begin && b.k0 < kv_end) meet.push_back(&b);
  if (meet.size() > 1 && (!a->lse || a->o_dtype != SQG_F32))
    return fail(SQG_ERR_INVALID_ARGUMENT, "the key range spans %d blocks: merging needs an lse buffer and o_dtype SQG_F32",
                (int)meet.size());
  void* const cs = sk->copy_stream;
  void* const copy_stream = cs ? cs : stream;
  StageEvents E;
  if (cs && !meet.empty()) {
    st = stage_begin(E, cs, stream);
    if (st != SQG_OK) return st;
  }
  for (size_t i = 0; i < meet.size(); ++i) {
    const StagedBlock& b = *meet[i];
    const int j = (int)(i & 1);
    if (cs && i >= 2) {   // the kernel that read slot j (two blocks back) is done
      st = launch_status(sqg::stream_wait_event(cs, E.kernel(j)), "staging stream wait");
      if (st != SQG_OK) return st;
    }
    const char* hk = static_cast<const char*>(sk->host_kpack) + b.pack_off;
    const char* hv = static_cast<const char*>(sk->host_vpack) + b.pack_off;
    const char* hks = static_cast<const char*>(sk->host_kscale) + b.scale_off;
    const char* hvs = static_cast<const char*>(sk->host_vscale) + b.scale_off;
    const int rc[4] = {
        sqg::copy_async(sk->dev_kpack[j], hk, b.L.pack_bytes, sqg::kHostToDevice, copy_stream),
        sqg::copy_async(sk->dev_vpack[j], hv, b.L.pack_bytes, sqg::kHostToDevice, copy_stream),
        sqg::copy_async(sk->dev_kscale[j], hks, b.L.scale_bytes, sqg::kHostToDevice, copy_stream),
        sqg::copy_async(sk->dev_vscale[j], hvs, b.L.scale_bytes, sqg::kHostToDevice, copy_stream)};
    for (int r : rc) {
      st = launch_status(r, "staging copy to device");
      if (st != SQG_OK) return st;
    }
    if (cs) {   // this block's kernel starts once its copies have landed
      st = stage_order(E.copy(j), cs, stream);
      if (st != SQG_OK) return st;
    }
    p.kpack = static_cast<const uint8_t*>(sk->dev_kpack[j]);
    p.vpack = static_cast<const uint8_t*>(sk->dev_vpack[j]);
    p.kscale = static_cast<const uint16_t*>(sk->dev_kscale[j]);
    p.vscale = static_cast<const uint16_t*>(sk->dev_vscale[j]);
    p.seg = seg_table(b.L);
    p.kv_row0 = b.k0;
    p.kv_n = b.k1 - b.k0;
    p.kv_begin = b.k0 > a->kv_begin ? b.k0 : a->kv_begin;
    p.kv_end = b.k1 < kv_end ? b.k1 : kv_end;
    p.accumulate = i == 0 ? a->accumulate : 1;
    st = launch_status(sqg::launch_packed_attention(p, stream), "packed_kv_attention launch");
    if (st != SQG_OK) return st;
    if (cs) {
      st = launch_status(sqg::event_record(E.kernel(j), stream), "staging event record");
      if (st != SQG_OK) return st;
    }
  }
  return ok();
}

SQG_API int sqg_test_quant_pack_f32(const float* r, int64_t rows, int32_t fmt, void* codes,
                                    void* scales, void* stream) {
  if (rows < 0) return fail(SQG_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (fmt != SQG_INT4_ROT && fmt != SQG_INT8_ROT)
    return fail(SQG_ERR_INVALID_ARGUMENT, "unknown format %d", fmt);
  if (rows == 0) return ok();
  if (!r || !codes || !scales) return fail(SQG_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
  if (!aligned16(r) || !aligned16(codes) || ((uintptr_t)scales & 7u))
    return fail(SQG_ERR_MISALIGNED, "r and codes must be 16-byte aligned, scales 8-byte aligned");
  const int st = launch_status(sqg::launch_test_quant_pack(r, rows, fmt, codes, scales, stream),
                               "test_quant_pack launch");
  return st == SQG_OK ? ok() : st;
}

SQG_API int sqg_test_fwht_f32(const float* in, float* out, int64_t rows, int32_t normalize,
                              void* stream) {
  if (rows < 0) return fail(SQG_ERR_INVALID_ARGUMENT, "rows must be >= 0");
  if (rows == 0) return ok();
  if (!in || !out) return fail(SQG_ERR_INVALID_ARGUMENT, "a device pointer is NULL");
  if (!aligned16(in) || !aligned16(out)) return fail(SQG_ERR_MISALIGNED, "pointers must be 16-byte aligned");
  const int st = launch_status(sqg::launch_test_fwht(in, out, rows, normalize, stream), "test_fwht launch");
  return st == SQG_OK ? ok() : st;
}

}  // extern "C"

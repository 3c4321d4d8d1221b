// Host-side part of libpa: error channel, descriptor checks, version, and the
// step metadata builder (slot_mapping and cu_seqlens).
#include <cstdarg>
#include <cstring>

#include "common.hpp"

namespace pa {

namespace {
thread_local char g_error[512] = {0};
}

void set_error(const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
}

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof(g_error), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_error[0] = 0; }

int check_desc(const pa_desc* d) {
  if (!d) return fail(PA_ERR_INVALID_ARG, "desc is NULL");
  if (d->num_q_heads <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0 || d->block_size <= 0 ||
      d->num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARG, "desc: sizes must be positive (H_q=%d H_kv=%d d=%d B=%d N=%lld)",
                d->num_q_heads, d->num_kv_heads, d->head_dim, d->block_size,
                (long long)d->num_blocks);
  if (d->num_q_heads % d->num_kv_heads)
    return fail(PA_ERR_INVALID_ARG, "desc: num_q_heads %d is not a multiple of num_kv_heads %d",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not built (64, 128)", d->head_dim);
  if (d->block_size < kMinBlockSize || d->block_size > kMaxBlockSize ||
      (d->block_size & (d->block_size - 1)))
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not built (powers of two, 16..1024)",
                d->block_size);
  const int g = d->num_q_heads / d->num_kv_heads;
  if (g > 16) return fail(PA_ERR_UNSUPPORTED, "GQA group size %d not built (1 .. 16)", g);
  return PA_OK;
}

}  // namespace pa

extern "C" const char* pa_last_error(void) { return pa::g_error; }

extern "C" const char* pa_version(void) { return "0.1.0"; }

// Slot of every position a step computes, in batch order, plus the varlen
// prefix sums. The two-step map: logical block p / B through the table, then
// offset p % B inside the physical block.
extern "C" int64_t pa_build_metadata(const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* starts, const int32_t* ends,
                                     int32_t num_seqs, int32_t block_size,
                                     int32_t* slot_mapping, int64_t slot_capacity,
                                     int32_t* cu_seqlens_q, int32_t* cu_seqlens_k) {
  using pa::fail;
  if (num_seqs < 0 || block_size <= 0 || max_blocks_per_seq < 0 || slot_capacity < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: negative size");
  if (num_seqs > 0 && (!block_tables || !starts || !ends))
    return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: NULL input");
  int64_t n = 0;
  int64_t cq = 0, ck = 0;
  if (cu_seqlens_q) cu_seqlens_q[0] = 0;
  if (cu_seqlens_k) cu_seqlens_k[0] = 0;
  for (int32_t b = 0; b < num_seqs; ++b) {
    const int32_t s = starts[b], e = ends[b];
    if (s < 0 || e < s)
      return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: seq %d has start %d end %d", b, s, e);
    if (((int64_t)e + block_size - 1) / block_size > max_blocks_per_seq)
      return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: seq %d needs more than %d blocks", b,
                  max_blocks_per_seq);
    if (n + (e - s) > slot_capacity)
      return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: slot_mapping capacity %lld too small",
                  (long long)slot_capacity);
    const int32_t* row = block_tables + (int64_t)b * max_blocks_per_seq;
    for (int32_t p = s; p < e; ++p) {
      const int32_t blk = row[p / block_size];
      if (blk < 0)
        return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: seq %d position %d hits table padding",
                    b, p);
      const int64_t slot = (int64_t)blk * block_size + p % block_size;
      if (slot > INT32_MAX)
        return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: slot exceeds int32");
      slot_mapping[n++] = (int32_t)slot;
    }
    cq += e - s;
    ck += e;
    if (cq > INT32_MAX || ck > INT32_MAX)
      return fail(PA_ERR_INVALID_ARG, "pa_build_metadata: cu_seqlens exceed int32");
    if (cu_seqlens_q) cu_seqlens_q[b + 1] = (int32_t)cq;
    if (cu_seqlens_k) cu_seqlens_k[b + 1] = (int32_t)ck;
  }
  pa::clear_error();
  return n;
}

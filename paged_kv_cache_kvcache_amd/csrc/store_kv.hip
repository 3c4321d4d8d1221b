// pa_store_kv: scatter each new token's K/V row into the paged cache at its
// slot ("12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.6 store kernel;
// slot protocol from "Nano-vLLM 源码解读 - 3. PagedAttention", §4).
//
// Pure data movement: a token row is H_kv*d bf16 values (2 KiB at 8 kv heads
// x 128). Each lane moves 16 bytes of K and 16 of V per iteration, so a wave
// covers 1 KiB of a row per instruction with fully coalesced loads and stores.
// Slots are read once per lane (they are uniform across the lanes of a row
// and served from the scalar/vector cache).
#include "common.hpp"

namespace pa {
namespace {

constexpr int kStoreThreads = 256;

// 16-byte path: rows, strides and base pointers are 16-byte aligned.
__global__ __launch_bounds__(kStoreThreads) void store_kv_vec16_kernel(
    const uint4* __restrict__ k, int64_t k_stride_vec, const uint4* __restrict__ v,
    int64_t v_stride_vec, uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
    const int32_t* __restrict__ slots, int32_t n_tokens, int32_t row_vecs, int64_t num_slots) {
  const int64_t total = (int64_t)n_tokens * row_vecs;
  const int64_t step = (int64_t)gridDim.x * kStoreThreads;
  for (int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x; i < total; i += step) {
    const int32_t tok = (int32_t)(i / row_vecs);
    const int32_t c = (int32_t)(i - (int64_t)tok * row_vecs);
    const int32_t slot = slots[tok];
    // -1 is padding; anything else outside the pool is a broken precondition
    // and is dropped rather than written out of bounds.
    if (slot < 0 || slot >= num_slots) continue;
    const uint4 kv = k[(int64_t)tok * k_stride_vec + c];
    const uint4 vv = v[(int64_t)tok * v_stride_vec + c];
    k_cache[(int64_t)slot * row_vecs + c] = kv;
    v_cache[(int64_t)slot * row_vecs + c] = vv;
  }
}

// Any-alignment path, one bf16 element per lane.
__global__ __launch_bounds__(kStoreThreads) void store_kv_elem_kernel(
    const uint16_t* __restrict__ k, int64_t k_stride, const uint16_t* __restrict__ v,
    int64_t v_stride, uint16_t* __restrict__ k_cache, uint16_t* __restrict__ v_cache,
    const int32_t* __restrict__ slots, int32_t n_tokens, int32_t row_elems, int64_t num_slots) {
  const int64_t total = (int64_t)n_tokens * row_elems;
  const int64_t step = (int64_t)gridDim.x * kStoreThreads;
  for (int64_t i = (int64_t)blockIdx.x * kStoreThreads + threadIdx.x; i < total; i += step) {
    const int32_t tok = (int32_t)(i / row_elems);
    const int32_t c = (int32_t)(i - (int64_t)tok * row_elems);
    const int32_t slot = slots[tok];
    if (slot < 0 || slot >= num_slots) continue;
    k_cache[(int64_t)slot * row_elems + c] = k[(int64_t)tok * k_stride + c];
    v_cache[(int64_t)slot * row_elems + c] = v[(int64_t)tok * v_stride + c];
  }
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace pa

extern "C" int pa_store_kv(const void* k, int64_t k_row_stride, const void* v,
                           int64_t v_row_stride, void* k_cache, void* v_cache,
                           const int32_t* slot_mapping, int32_t n_tokens, const pa_desc* desc,
                           void* stream) {
  using namespace pa;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (n_tokens < 0) return fail(PA_ERR_INVALID_ARG, "pa_store_kv: n_tokens %d < 0", n_tokens);
  if (n_tokens == 0) return PA_OK;
  if (!k || !v || !k_cache || !v_cache || !slot_mapping)
    return fail(PA_ERR_INVALID_ARG, "pa_store_kv: NULL pointer");
  const int32_t row = desc->num_kv_heads * desc->head_dim;
  if (k_row_stride < row || v_row_stride < row)
    return fail(PA_ERR_INVALID_ARG, "pa_store_kv: row stride (%lld, %lld) < H_kv*d = %d",
                (long long)k_row_stride, (long long)v_row_stride, row);
  const int64_t num_slots = desc->num_blocks * desc->block_size;
  hipStream_t s = (hipStream_t)stream;
  if (debug_enabled()) {
    rc = debug_check_slots("pa_store_kv", slot_mapping, n_tokens, num_slots, s);
    if (rc) return rc;
  }
  const bool vec = aligned16(k) && aligned16(v) && aligned16(k_cache) && aligned16(v_cache) &&
                   (k_row_stride % 8 == 0) && (v_row_stride % 8 == 0) && (row % 8 == 0);
  if (vec) {
    const int32_t row_vecs = row / 8;
    const int64_t total = (int64_t)n_tokens * row_vecs;
    const int64_t blocks = std::min<int64_t>((total + kStoreThreads - 1) / kStoreThreads, 65536);
    hipLaunchKernelGGL(store_kv_vec16_kernel, dim3((unsigned)blocks), dim3(kStoreThreads), 0, s,
                       (const uint4*)k, k_row_stride / 8, (const uint4*)v, v_row_stride / 8,
                       (uint4*)k_cache, (uint4*)v_cache, slot_mapping, n_tokens, row_vecs,
                       num_slots);
  } else {
    const int64_t total = (int64_t)n_tokens * row;
    const int64_t blocks = std::min<int64_t>((total + kStoreThreads - 1) / kStoreThreads, 65536);
    hipLaunchKernelGGL(store_kv_elem_kernel, dim3((unsigned)blocks), dim3(kStoreThreads), 0, s,
                       (const uint16_t*)k, k_row_stride, (const uint16_t*)v, v_row_stride,
                       (uint16_t*)k_cache, (uint16_t*)v_cache, slot_mapping, n_tokens, row,
                       num_slots);
  }
  return launch_status("pa_store_kv");
}

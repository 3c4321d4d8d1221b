// Debug mode: checks of the device-resident preconditions before any kernel
// that relies on them runs.
//
// The attention and store kernels take slots, block tables and sequence
// lengths from device memory and never read them back on the host ("Nano-vLLM
// 源码解读 - 3. PagedAttention", §4: -1 marks a padding slot; §3: entries of a
// table past the sequence's last block are padding). In normal operation a
// broken entry is only kept from becoming an out-of-bounds access (read as
// block 0 or dropped). With debug mode on (environment variable PA_DEBUG set
// to anything but "0", or pa_set_debug(1)), every entry point first runs the
// kernels below on its stream, waits for them, and returns PA_ERR_INVALID_ARG
// with the first violation it finds instead of launching its own kernels:
//   * slots: in [-1, N*B), and no slot twice (an all-pairs comparison, tiled
//     through LDS; skipped above 16M tokens);
//   * lengths: 0 <= n <= max_context_len and ceil(n / B) <= max_blocks_per_seq;
//   * block tables: the entries of blocks 0 .. ceil(n / B) - 1 in [0, N);
//   * varlen batches: cu_seqlens_q/k non-decreasing from 0, k_len >= q_len,
//     q_len <= max_seqlen_q, k_len <= max_seqlen_k, and q_len == 1 for the
//     decode rows of a mixed batch.
// Debug mode synchronises the stream, so it cannot be used under graph
// capture, and concurrent debug calls on one device share the violation
// record below.
#include <atomic>
#include <cstdlib>
#include <cstring>

#include <vector>

#include "common.hpp"

namespace pa {
namespace {

enum Kind : int {
  kSlotRange = 1,
  kSlotDuplicate,
  kLength,
  kTableEntry,
  kCuQ,
  kCuK,
  kKShort,
  kQLong,
  kKLong,
  kDecodeRow,
};

// The first violation: kind, two indices and the offending value.
struct Record {
  int kind;
  int i;
  int j;
  int pad;
  long long value;
};

__device__ int g_found;
__device__ Record g_record;

__device__ void report(int kind, int i, int j, long long value) {
  if (atomicCAS(&g_found, 0, 1) == 0) {
    g_record.kind = kind;
    g_record.i = i;
    g_record.j = j;
    g_record.value = value;
    __threadfence();
  }
}

__global__ void reset_kernel() {
  g_found = 0;
  g_record.kind = 0;
}

constexpr int kTile = 256;

__global__ __launch_bounds__(kTile) void slot_range_kernel(const int32_t* slots, int32_t n,
                                                           int64_t num_slots) {
  for (int64_t i = (int64_t)blockIdx.x * kTile + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * kTile) {
    const int32_t s = slots[i];
    if (s < -1 || s >= num_slots) report(kSlotRange, (int)i, 0, s);
  }
}

// Tile (blockIdx.x, blockIdx.y) compares slots of tile x with those of tile
// y >= x; every pair i < j is compared once.
__global__ __launch_bounds__(kTile) void slot_unique_kernel(const int32_t* slots, int32_t n) {
  if (blockIdx.y < blockIdx.x) return;
  __shared__ int32_t other[kTile];
  const int j0 = blockIdx.y * kTile;
  const int jt = j0 + threadIdx.x;
  other[threadIdx.x] = jt < n ? slots[jt] : -1;
  __syncthreads();
  const int i = blockIdx.x * kTile + threadIdx.x;
  if (i >= n) return;
  const int32_t s = slots[i];
  if (s < 0) return;
  const int jn = min(kTile, n - j0);
  for (int k = 0; k < jn; ++k)
    if (j0 + k > i && other[k] == s) report(kSlotDuplicate, i, j0 + k, s);
}

// One thread per (sequence, table column).
__global__ __launch_bounds__(kTile) void table_kernel(const int32_t* bt, int32_t max_blocks,
                                                      const int32_t* lens, const int32_t* cu_k,
                                                      int32_t num_seqs, int32_t max_ctx,
                                                      int32_t block_size, int64_t num_blocks) {
  const int64_t total = (int64_t)num_seqs * max(max_blocks, 1);
  for (int64_t x = (int64_t)blockIdx.x * kTile + threadIdx.x; x < total;
       x += (int64_t)gridDim.x * kTile) {
    const int b = (int)(x / max(max_blocks, 1));
    const int t = (int)(x % max(max_blocks, 1));
    const int n = lens ? lens[b] : cu_k[b + 1] - cu_k[b];
    const int64_t need = n <= 0 ? 0 : ((int64_t)n + block_size - 1) / block_size;
    if (t == 0 && (n < 0 || n > max_ctx || need > max_blocks)) report(kLength, b, 0, n);
    if (t < need && t < max_blocks) {
      const int32_t e = bt[(int64_t)b * max_blocks + t];
      if (e < 0 || e >= num_blocks) report(kTableEntry, b, t, e);
    }
  }
}

__global__ __launch_bounds__(kTile) void cu_kernel(const int32_t* cu_q, const int32_t* cu_k,
                                                   int32_t num_seqs, int32_t max_q, int32_t max_k,
                                                   int32_t decode_rows) {
  for (int b = blockIdx.x * kTile + threadIdx.x; b < num_seqs; b += gridDim.x * kTile) {
    if (b == 0 && cu_q[0] != 0) report(kCuQ, 0, 0, cu_q[0]);
    if (b == 0 && cu_k[0] != 0) report(kCuK, 0, 0, cu_k[0]);
    const int q_len = cu_q[b + 1] - cu_q[b];
    const int k_len = cu_k[b + 1] - cu_k[b];
    if (q_len < 0) report(kCuQ, b + 1, 0, cu_q[b + 1]);
    if (k_len < 0) report(kCuK, b + 1, 0, cu_k[b + 1]);
    if (k_len < q_len) report(kKShort, b, q_len, k_len);
    if (q_len > max_q) report(kQLong, b, 0, q_len);
    if (k_len > max_k) report(kKLong, b, 0, k_len);
    if (b < decode_rows && q_len != 1) report(kDecodeRow, b, 0, q_len);
  }
}

unsigned grid_for(int64_t items) {
  return (unsigned)std::min<int64_t>((items + kTile - 1) / kTile, 4096);
}

std::atomic<int> g_debug{-1};

// Waits for the check kernels queued on s and turns a recorded violation
// into an error status and message.
int finish(const char* who, hipStream_t s) {
  int rc = launch_status(who);
  if (rc) return rc;
  int found = 0;
  Record r{};
  if (hipMemcpyFromSymbolAsync(&found, HIP_SYMBOL(g_found), sizeof(found), 0,
                               hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipMemcpyFromSymbolAsync(&r, HIP_SYMBOL(g_record), sizeof(r), 0, hipMemcpyDeviceToHost,
                               s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: debug check: %s", who, hipGetErrorString(hipGetLastError()));
  if (!found) return PA_OK;
  switch (r.kind) {
    case kSlotRange:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: slot_mapping[%d] = %lld is outside [-1, N*B)",
                  who, r.i, r.value);
    case kSlotDuplicate:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: slot %lld appears twice (slot_mapping[%d] "
                  "and [%d])", who, r.value, r.i, r.j);
    case kLength:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: sequence %d has length %lld, outside "
                  "[0, max_context_len] or beyond its table row", who, r.i, r.value);
    case kTableEntry:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: block_tables[%d][%d] = %lld is outside "
                  "[0, num_blocks) and the sequence reaches that block", who, r.i, r.j, r.value);
    case kCuQ:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: cu_seqlens_q[%d] = %lld breaks a "
                  "non-decreasing prefix sum from 0", who, r.i, r.value);
    case kCuK:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: cu_seqlens_k[%d] = %lld breaks a "
                  "non-decreasing prefix sum from 0", who, r.i, r.value);
    case kKShort:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: sequence %d has k_len %lld < q_len %d",
                  who, r.i, r.value, r.j);
    case kQLong:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: sequence %d has q_len %lld > max_seqlen_q",
                  who, r.i, r.value);
    case kKLong:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: sequence %d has k_len %lld > max_seqlen_k",
                  who, r.i, r.value);
    case kDecodeRow:
      return fail(PA_ERR_INVALID_ARG, "%s: debug check: decode row %d has q_len %lld (must be 1)",
                  who, r.i, r.value);
  }
  return fail(PA_ERR_INVALID_ARG, "%s: debug check: violation %d", who, r.kind);
}

}  // namespace

bool debug_enabled() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = std::getenv("PA_DEBUG");
    const int want = (e && *e && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, want);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v > 0;
}

int debug_check_slots(const char* who, const int32_t* slots, int32_t n, int64_t num_slots,
                      hipStream_t s) {
  if (n <= 0) return PA_OK;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(slot_range_kernel, dim3(grid_for(n)), dim3(kTile), 0, s, slots, n, num_slots);
  const int64_t tiles = ((int64_t)n + kTile - 1) / kTile;
  if (tiles <= 65535)
    hipLaunchKernelGGL(slot_unique_kernel, dim3((unsigned)tiles, (unsigned)tiles), dim3(kTile), 0,
                       s, slots, n);
  return finish(who, s);
}

int debug_check_tables(const char* who, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, const int32_t* cu_k, int32_t num_seqs,
                       int32_t max_context_len, const pa_desc* d, hipStream_t s) {
  if (num_seqs <= 0) return PA_OK;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(table_kernel, dim3(grid_for((int64_t)num_seqs * std::max(max_blocks, 1))),
                     dim3(kTile), 0, s, block_tables, max_blocks, context_lens, cu_k, num_seqs,
                     max_context_len, d->block_size, d->num_blocks);
  return finish(who, s);
}

int debug_check_varlen(const char* who, const int32_t* cu_q, const int32_t* cu_k,
                       int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t decode_rows, hipStream_t s) {
  if (num_seqs <= 0) return PA_OK;
  hipLaunchKernelGGL(reset_kernel, dim3(1), dim3(1), 0, s);
  hipLaunchKernelGGL(cu_kernel, dim3(grid_for(num_seqs)), dim3(kTile), 0, s, cu_q, cu_k,
                     num_seqs, max_seqlen_q, max_seqlen_k, decode_rows);
  return finish(who, s);
}

int debug_check_zero(const char* who, const void* p, size_t bytes, hipStream_t s) {
  if (!bytes) return PA_OK;
  std::vector<unsigned char> h(bytes);
  if (hipMemcpyAsync(h.data(), p, bytes, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(PA_ERR_HIP, "%s: debug check: %s", who, hipGetErrorString(hipGetLastError()));
  for (size_t i = 0; i < bytes; ++i)
    if (h[i])
      return fail(PA_ERR_WORKSPACE, "%s: debug check: workspace byte %zu of the counter header "
                  "is not zero (zero the workspace before its first use)", who, i);
  return PA_OK;
}

}  // namespace pa

extern "C" int pa_set_debug(int on) {
  const int prev = pa::debug_enabled() ? 1 : 0;
  pa::g_debug.store(on ? 1 : 0);
  return prev;
}

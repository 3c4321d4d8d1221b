// Shared helpers of libpa (device and host): bf16 bit handling, cross-lane
// reductions for gfx950 wave64, argument checks and the error channel.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/pa.h"

namespace pa {

constexpr int kWave = 64;
constexpr int kMinBlockSize = 16;    // block sizes: powers of two in [16, 1024]
constexpr int kMaxBlockSize = 1024;
inline int log2_int(int v) { int s = 0; while ((1 << s) < v) ++s; return s; }

// ------------------------------------------------------------------ errors

void set_error(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Validate a descriptor; returns PA_OK or an error code (message set).
int check_desc(const pa_desc* d);

inline int launch_status(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PA_OK;
}

// ------------------------------------------- debug-mode checks (validate.hip)

// True when debug mode is on (PA_DEBUG in the environment, or pa_set_debug).
bool debug_enabled();
// Each queues its check kernels on s, waits for them and returns PA_OK or
// PA_ERR_INVALID_ARG with the first violation in the message.
int debug_check_slots(const char* who, const int32_t* slots, int32_t n, int64_t num_slots,
                      hipStream_t s);
int debug_check_tables(const char* who, const int32_t* block_tables, int32_t max_blocks,
                       const int32_t* context_lens, const int32_t* cu_k, int32_t num_seqs,
                       int32_t max_context_len, const pa_desc* d, hipStream_t s);
int debug_check_varlen(const char* who, const int32_t* cu_q, const int32_t* cu_k,
                       int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                       int32_t decode_rows, hipStream_t s);
// PA_ERR_WORKSPACE unless the first `bytes` bytes at device address p are zero.
int debug_check_zero(const char* who, const void* p, size_t bytes, hipStream_t s);

// ------------------------------------------------- decode launch (decode.hip)

struct NewTokens {  // the fused store's inputs (null for plain decode)
  const void* k;
  int64_t k_stride;
  const void* v;
  int64_t v_stride;
  const int32_t* slot_mapping;
};

// Split-K decode of num_seqs rows; lengths from context_lens, or (when it is
// null) from cu_k[b+1] - cu_k[b]. Validates its arguments; returns a status.
// use_scratch: the workspace is the library's own device array (the caller's
// workspace arguments are ignored), refused if the batch needs more.
int launch_decode(const char* who, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, const int32_t* cu_k, int32_t num_seqs,
                  int32_t max_context_len, float scale, void* out, void* workspace,
                  size_t workspace_bytes, int32_t partition_blocks, const pa_desc* desc,
                  void* stream, const NewTokens* nt, bool use_scratch = false);
size_t decode_workspace_bytes(const pa_desc* desc, int32_t num_seqs, int32_t max_context_len);

// ------------------------------------------------------------- bf16 bits

// bf16 -> fp32 is exact: the bf16 pattern is the top half of the fp32 one.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ------------------------------------------------------- cross-lane (DPP)

// DPP controls of the GCN/CDNA "dpp_ctrl" field.
constexpr int kDppQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each 16-lane row
constexpr int kDppRowRor8 = 0x128;        // rotate a 16-lane row by 8 (= lane xor 8)

template <int Ctrl>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N = 8 or 16); every lane of a group
// ends with the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 8 || N == 16, "group of 8 or 16 lanes");
  x += dpp<kDppQuadXor1>(x);
  x += dpp<kDppQuadXor2>(x);
  x += dpp<kDppRowHalfMirror>(x);
  if constexpr (N == 16) x += dpp<kDppRowMirror>(x);
  return x;
}

// Lane-exact xor exchange for offsets >= 8 (whole groups of lanes swap).
__device__ __forceinline__ float xor_lane(float x, int mask) { return __shfl_xor(x, mask, kWave); }

}  // namespace pa

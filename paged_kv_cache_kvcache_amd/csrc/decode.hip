// pa_decode: paged GQA decode attention for gfx950.
//
// What is computed: for each sequence and q-head, softmax(scale * q . K_t) V_t
// over the sequence's tokens, K/V read through its block table
// ("12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.6 decode branch;
// "vLLM 深度解读", §3 kernel sketch: block-table lookup per block, online
// softmax with max/sum rescaling; two-step address of
// "Nano-vLLM 源码解读 - 3. PagedAttention", §3).
//
// How (MI355X design, not the sketch's):
//   * split-K: a work item is (sequence, kv-head, partition of whole 256-token
//     blocks), one wave64 each, so a 256-sequence batch with 16x spread in
//     length still yields tens of thousands of equal-sized items; a second
//     kernel merges the partitions' (max, sum, unnormalised output) triples.
//     Sequences that fit one partition are finished by the first kernel.
//   * GQA: the wave loads each K/V row of its kv-head once and applies it to
//     all G q-heads of the group held in registers (one load, G uses).
//   * loads: 16 bytes per lane; d/8 lanes cover one token's 2*d-byte head
//     vector, so a wave instruction reads 64/(d/8) whole token vectors
//     (4 at d = 128). Eight such loads of K and eight of V are in flight per
//     wave before any arithmetic.
//   * q.k: v_dot2_f32_bf16 on the raw bf16 pairs (exact products, fp32 sum),
//     then a DPP butterfly over the d/8 lanes of the token (no LDS traffic).
//   * softmax: base-2 exponent with scale*log2(e) folded into the score; each
//     token-row of lanes keeps its own running max so no cross-row exchange
//     is needed inside the loop; rows are merged once at the end.
//   * V: bf16 -> fp32 by shift/mask (exact), fp32 FMA accumulation.
#include <cmath>

#include "common.hpp"

namespace pa {
namespace {

constexpr int kUnroll = 8;          // token loads in flight per wave per chunk
constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  float* ws_o;   // [num_seqs, H_q, max_parts, d] fp32 unnormalised partial outputs
  float* ws_ml;  // [num_seqs, H_q, max_parts, 2]  (running max in log2 units, sum)
  uint16_t* out;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t part_tokens;
  int32_t max_parts;
  float scale_log2;
};

__device__ __forceinline__ float dot8_bf16(const uint4& k, const uint32_t (&q)[4], float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.x),
                                        __builtin_bit_cast(bf16x2, q[0]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.y),
                                        __builtin_bit_cast(bf16x2, q[1]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.z),
                                        __builtin_bit_cast(bf16x2, q[2]), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, k.w),
                                        __builtin_bit_cast(bf16x2, q[3]), acc, false);
  return acc;
}

__device__ __forceinline__ int clamp_len(int n, int max_blocks) {
  return max(0, min(n, max_blocks * kBlockSize));
}

template <int D, int G>
__global__ __launch_bounds__(kWave) void decode_split_kernel(DecodeArgs a) {
  constexpr int LPT = D / 8;            // lanes per token vector
  constexpr int TPI = kWave / LPT;      // tokens per wave load instruction
  constexpr int CHUNK = TPI * kUnroll;  // tokens per loop iteration
  static_assert(kBlockSize % CHUNK == 0, "a chunk never straddles a block");

  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * G;
  int idx = blockIdx.x;
  const int g = idx % H_kv;
  idx /= H_kv;
  const int b = idx % a.num_seqs;
  const int part = idx / a.num_seqs;
  const int lane = threadIdx.x;
  const int sub = lane % LPT;  // which 8 elements of the head vector
  const int row = lane / LPT;  // which token of a load instruction

  const int n = clamp_len(a.context_lens[b], a.max_blocks);
  const int nparts = min((n + a.part_tokens - 1) / a.part_tokens, a.max_parts);
  const int64_t head0 = (int64_t)b * H_q + (int64_t)g * G;  // first q-head of the group

  if (n == 0) {  // padding row: defined as zeros, nothing read
    if (part == 0 && row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h)
        *reinterpret_cast<uint4*>(a.out + (head0 + h) * D + sub * 8) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  if (part >= nparts) return;
  const int start = part * a.part_tokens;
  const int end = min(n, start + a.part_tokens);

  uint32_t qv[G][4];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = *reinterpret_cast<const uint4*>(a.q + (head0 + h) * D + sub * 8);
    qv[h][0] = t.x; qv[h][1] = t.y; qv[h][2] = t.z; qv[h][3] = t.w;
  }
  float m[G], l[G], acc[G][8];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
  }

  const int64_t row_elems = (int64_t)H_kv * D;  // elements per token row of the cache
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  for (int c = start; c < end; c += CHUNK) {
    const int blk = bt[c / kBlockSize];
    const bool blk_ok = blk >= 0 && blk < a.num_blocks;  // broken table entry: read nothing
    const int64_t base =
        ((int64_t)(blk_ok ? blk : 0) * kBlockSize + (c % kBlockSize)) * row_elems + g * D + sub * 8;
    const int last = end - 1 - c;  // last valid token index inside this chunk (>= 0)

    uint4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      // tokens past the end re-read the last valid token (finite data) and
      // are masked below, so poisoned rows never enter the sums
      const int t = min(u * TPI + row, last);
      kr[u] = *reinterpret_cast<const uint4*>(a.k_cache + base + t * row_elems);
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int t = min(u * TPI + row, last);
      vr[u] = *reinterpret_cast<const uint4*>(a.v_cache + base + t * row_elems);
    }

    float s[kUnroll][G];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const bool valid = blk_ok && (u * TPI + row <= last);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float d = group_sum<LPT>(dot8_bf16(kr[u], qv[h], 0.f));
        s[u][h] = valid ? d * a.scale_log2 : -INFINITY;
      }
    }

    float msafe[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float mx = s[0][h];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mx = fmaxf(mx, s[u][h]);
      const float mnew = fmaxf(m[h], mx);
      msafe[h] = (mnew == -INFINITY) ? 0.f : mnew;  // row saw no token yet
      const float alpha = exp2f(m[h] - msafe[h]);
      l[h] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] *= alpha;
      m[h] = mnew;
    }

#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vf[8];
      vf[0] = bf16_lo(vr[u].x); vf[1] = bf16_hi(vr[u].x);
      vf[2] = bf16_lo(vr[u].y); vf[3] = bf16_hi(vr[u].y);
      vf[4] = bf16_lo(vr[u].z); vf[5] = bf16_hi(vr[u].z);
      vf[6] = bf16_lo(vr[u].w); vf[7] = bf16_hi(vr[u].w);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = exp2f(s[u][h] - msafe[h]);
        l[h] += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(p, vf[e], acc[h][e]);
      }
    }
  }

  // Merge the TPI token-rows (each has its own running max).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = m[h];
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) M = fmaxf(M, xor_lane(M, off));
    const float w = (m[h] == -INFINITY) ? 0.f : exp2f(m[h] - M);
    float lh = l[h] * w;
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) lh += xor_lane(lh, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float o = acc[h][e] * w;
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) o += xor_lane(o, off);
      acc[h][e] = o;
    }
    m[h] = M;
    l[h] = lh;
  }

  if (nparts == 1) {
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = 1.f / l[h];
        uint4 o;
        o.x = pack_bf16x2(acc[h][0] * inv, acc[h][1] * inv);
        o.y = pack_bf16x2(acc[h][2] * inv, acc[h][3] * inv);
        o.z = pack_bf16x2(acc[h][4] * inv, acc[h][5] * inv);
        o.w = pack_bf16x2(acc[h][6] * inv, acc[h][7] * inv);
        *reinterpret_cast<uint4*>(a.out + (head0 + h) * D + sub * 8) = o;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t wi = (head0 + h) * a.max_parts + part;
      if (row == 0) {
        float4* dst = reinterpret_cast<float4*>(a.ws_o + wi * D + sub * 8);
        dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
        dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
      }
      if (lane == 0) *reinterpret_cast<float2*>(a.ws_ml + wi * 2) = make_float2(m[h], l[h]);
    }
  }
}

// Exact log-sum-exp merge of a sequence's partitions:
// M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p 2^(m_p - M) / L.
template <int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeArgs a, int H_q) {
  constexpr int EPL = D / kWave;  // output elements per lane
  const int h = blockIdx.x % H_q;
  const int b = blockIdx.x / H_q;
  const int n = clamp_len(a.context_lens[b], a.max_blocks);
  const int nparts = min((n + a.part_tokens - 1) / a.part_tokens, a.max_parts);
  if (nparts <= 1) return;
  const int64_t w0 = ((int64_t)b * H_q + h) * a.max_parts;
  const int lane = threadIdx.x;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, a.ws_ml[(w0 + p) * 2]);
  float L = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + (w0 + p) * 2);
    const float w = (ml.x == -INFINITY) ? 0.f : exp2f(ml.x - M);
    L = fmaf(ml.y, w, L);
    const float* src = a.ws_o + (w0 + p) * D + lane * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = fmaf(src[e], w, o[e]);
  }
  const float inv = 1.f / L;
  uint16_t* dst = a.out + ((int64_t)b * H_q + h) * D + lane * EPL;
  if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else {
    dst[0] = (uint16_t)f32_to_bf16_rne(o[0] * inv);
  }
}

using SplitFn = void (*)(DecodeArgs);

template <int D>
SplitFn pick_split(int G) {
  switch (G) {
    case 1: return decode_split_kernel<D, 1>;
    case 2: return decode_split_kernel<D, 2>;
    case 4: return decode_split_kernel<D, 4>;
    case 8: return decode_split_kernel<D, 8>;
  }
  return nullptr;
}

int default_partition_blocks(const pa_desc*, int32_t, int32_t) { return 1; }

struct Plan {
  int part_tokens;
  int max_parts;
  size_t ws_bytes;
};

Plan make_plan(const pa_desc* d, int32_t num_seqs, int32_t max_ctx, int32_t part_blocks) {
  if (part_blocks <= 0) part_blocks = default_partition_blocks(d, num_seqs, max_ctx);
  Plan p;
  p.part_tokens = part_blocks * kBlockSize;
  p.max_parts = max(1, (max_ctx + p.part_tokens - 1) / p.part_tokens);
  p.ws_bytes = p.max_parts <= 1 ? 0
                                : (size_t)num_seqs * d->num_q_heads * p.max_parts *
                                      (size_t)(d->head_dim + 2) * sizeof(float);
  return p;
}

}  // namespace
}  // namespace pa

extern "C" size_t pa_decode_workspace_size_ex(const pa_desc* desc, int32_t num_seqs,
                                              int32_t max_context_len, int32_t partition_blocks) {
  if (pa::check_desc(desc) != PA_OK || num_seqs < 0 || max_context_len < 0 ||
      partition_blocks < 0)
    return 0;
  return pa::make_plan(desc, num_seqs, max_context_len, partition_blocks).ws_bytes;
}

extern "C" size_t pa_decode_workspace_size(const pa_desc* desc, int32_t num_seqs,
                                           int32_t max_context_len) {
  return pa_decode_workspace_size_ex(desc, num_seqs, max_context_len, 0);
}

extern "C" int pa_decode_partitioned(const void* q, const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t max_context_len, float scale, void* out,
                                     void* workspace, size_t workspace_bytes,
                                     int32_t partition_blocks, const pa_desc* desc,
                                     void* stream) {
  using namespace pa;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0 || partition_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: negative size");
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: NULL pointer");
  if ((int64_t)max_blocks_per_seq * kBlockSize < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: max_context_len %d exceeds %d table entries",
                max_context_len, max_blocks_per_seq);
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15u)
    return fail(PA_ERR_INVALID_ARG, "pa_decode: q, caches and out must be 16-byte aligned");
  const Plan plan = make_plan(desc, num_seqs, max_context_len, partition_blocks);
  if (plan.ws_bytes) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace %zu bytes < %zu needed",
                  workspace ? workspace_bytes : (size_t)0, plan.ws_bytes);
    if ((uintptr_t)workspace & 15u)
      return fail(PA_ERR_WORKSPACE, "pa_decode: workspace must be 16-byte aligned");
  }
  const int G = desc->num_q_heads / desc->num_kv_heads;
  const int D = desc->head_dim;
  const int64_t items = (int64_t)num_seqs * desc->num_kv_heads * plan.max_parts;
  if (items > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "pa_decode: grid too large");

  DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  const size_t o_floats = (size_t)num_seqs * desc->num_q_heads * plan.max_parts * D;
  a.ws_o = plan.ws_bytes ? (float*)workspace : nullptr;
  a.ws_ml = plan.ws_bytes ? (float*)workspace + o_floats : nullptr;
  a.out = (uint16_t*)out;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_kv_heads = desc->num_kv_heads;
  a.part_tokens = plan.part_tokens;
  a.max_parts = plan.max_parts;
  a.scale_log2 = scale * kLog2e;

  hipStream_t s = (hipStream_t)stream;
  SplitFn split = D == 128 ? pick_split<128>(G) : pick_split<64>(G);
  hipLaunchKernelGGL(split, dim3((unsigned)items), dim3(kWave), 0, s, a);
  rc = launch_status("pa_decode split");
  if (rc) return rc;
  if (plan.max_parts > 1) {
    const unsigned rows = (unsigned)num_seqs * desc->num_q_heads;
    if (D == 128)
      hipLaunchKernelGGL(decode_reduce_kernel<128>, dim3(rows), dim3(kWave), 0, s, a,
                         desc->num_q_heads);
    else
      hipLaunchKernelGGL(decode_reduce_kernel<64>, dim3(rows), dim3(kWave), 0, s, a,
                         desc->num_q_heads);
    rc = launch_status("pa_decode reduce");
    if (rc) return rc;
  }
  return PA_OK;
}

extern "C" int pa_decode(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                         const int32_t* context_lens, int32_t num_seqs, int32_t max_context_len,
                         float scale, void* out, void* workspace, size_t workspace_bytes,
                         const pa_desc* desc, void* stream) {
  return pa_decode_partitioned(q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                               context_lens, num_seqs, max_context_len, scale, out, workspace,
                               workspace_bytes, 0, desc, stream);
}

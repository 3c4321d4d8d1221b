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
//     blocks; 4 blocks by default), one wave64 each; a second kernel merges
//     the partitions' (max, sum, unnormalised output) triples exactly.
//     Sequences that fit one partition are finished by the first kernel.
//     Items are dispatched highest partition first, so the grid drains on the
//     first partitions that every sequence has instead of on a few long ones.
//   * GQA: the wave loads each K/V row of its kv-head once and applies it to
//     all G q-heads of the group held in registers (one load, G uses).
//   * loads: 16 bytes per lane, nontemporal (K/V are read once); d/8 lanes
//     cover one token's 2*d-byte head vector, so a wave instruction reads
//     64/(d/8) whole token vectors (4 at d = 128). Eight such loads of K and
//     eight of V are in flight per wave before any arithmetic; full chunks
//     address them from a wave-uniform base plus one per-lane offset.
//   * q.k: v_dot2_f32_bf16 on the raw bf16 pairs (exact products, fp32 sum),
//     then a DPP butterfly over the d/8 lanes of the token (no LDS traffic).
//   * softmax: base-2 exponent (raw v_exp_f32) with scale*log2(e) folded into
//     one FMA; each token-row of lanes keeps its own running max so no
//     cross-row exchange is needed inside the loop; rows merge once at the end.
//   * V: bf16 -> fp32 by shift/mask (exact), fp32 FMA accumulation.
#include <cmath>

#include "common.hpp"

namespace pa {
namespace {

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

#ifndef PA_DECODE_UNROLL
#define PA_DECODE_UNROLL 8
#endif
#ifndef PA_DECODE_NT
#define PA_DECODE_NT 1
#endif
#ifndef PA_DECODE_WAVES
#define PA_DECODE_WAVES 2
#endif
#ifndef PA_DECODE_PIPE
#define PA_DECODE_PIPE 0
#endif

// K/V rows are read exactly once per call: nontemporal loads keep them from
// displacing reusable lines (tables, q) in the caches.
__device__ __forceinline__ uint4 load16(const char* p) {
#if PA_DECODE_NT
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
#else
  return *reinterpret_cast<const uint4*>(p);
#endif
}

// Raw v_exp_f32 (2^x). Arguments are <= 0 here; results below the normal
// range flush to zero, which is what a softmax weight that small should be.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Per-wave state of one work item.
template <int D, int G, int U>
struct SplitState {
  static constexpr int LPT = D / 8;            // lanes per token vector
  static constexpr int TPI = kWave / LPT;      // tokens per wave load instruction
  static constexpr int CHUNK = TPI * U;        // tokens per chunk
  uint32_t qv[G][4];
  float m[G], l[G], acc[G][8];  // running max (log2 units), sum, unnormalised output
};

// Loads of one chunk. A full chunk reads tokens c .. c+CHUNK-1 from a
// wave-uniform base plus one per-lane offset; the tail chunk clamps every
// token index to the last valid one (masked later), so no address ever
// leaves the sequence's blocks.
template <int D, int G, int U, bool TAIL>
__device__ __forceinline__ void issue_chunk(const char* kbase, const char* vbase, int64_t row_bytes,
                                            int lane_off, int row, int last, uint4 (&kr)[U],
                                            uint4 (&vr)[U]) {
  using S = SplitState<D, G, U>;
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (TAIL) {
      const int t = min(u * S::TPI + row, last);
      kr[u] = load16(kbase + t * row_bytes + lane_off);
    } else {
      kr[u] = load16(kbase + (int64_t)u * S::TPI * row_bytes + lane_off);
    }
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    if constexpr (TAIL) {
      const int t = min(u * S::TPI + row, last);
      vr[u] = load16(vbase + t * row_bytes + lane_off);
    } else {
      vr[u] = load16(vbase + (int64_t)u * S::TPI * row_bytes + lane_off);
    }
  }
}

#ifndef PA_DECODE_LAZY
#define PA_DECODE_LAZY 0
#endif
// Lazy rescaling: a row's reference max m is raised only when a score
// exceeds it by more than 2^kLazyLog2, so weights 2^(s-m) stay <= 256 and the
// accumulator rescale (G*8 multiplies + exps) runs only on those rare tokens.
// The result is the same softmax: numerator and denominator share m.
constexpr float kLazyLog2 = 8.f;

template <int D, int G, int U, bool TAIL>
__device__ __forceinline__ void compute_chunk(SplitState<D, G, U>& st, float scale_log2, int row,
                                              int nvalid, const uint4 (&kr)[U],
                                              const uint4 (&vr)[U]) {
  using S = SplitState<D, G, U>;
#if PA_DECODE_LAZY
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const bool valid = !TAIL || (u * S::TPI + row < nvalid);
    float sc[G];
    float over = -INFINITY;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      sc[h] = group_sum<S::LPT>(dot8_bf16(kr[u], st.qv[h], 0.f)) * scale_log2;
      over = fmaxf(over, sc[h] - st.m[h]);  // +inf before the row's first token
    }
    if (valid && over > kLazyLog2) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mnew = fmaxf(st.m[h], sc[h]);
        const float alpha = fast_exp2(st.m[h] - mnew);  // 0 on the first token
        st.l[h] *= alpha;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
        st.m[h] = mnew;
      }
    }
    float vf[8];
    vf[0] = bf16_lo(vr[u].x); vf[1] = bf16_hi(vr[u].x);
    vf[2] = bf16_lo(vr[u].y); vf[3] = bf16_hi(vr[u].y);
    vf[4] = bf16_lo(vr[u].z); vf[5] = bf16_hi(vr[u].z);
    vf[6] = bf16_lo(vr[u].w); vf[7] = bf16_hi(vr[u].w);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float p = fast_exp2(sc[h] - st.m[h]);
      if constexpr (TAIL) p = valid ? p : 0.f;
      st.l[h] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] = fmaf(p, vf[e], st.acc[h][e]);
    }
  }
#else
  float s[U][G];  // raw q.k (unscaled)
#pragma unroll
  for (int u = 0; u < U; ++u) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float d = group_sum<S::LPT>(dot8_bf16(kr[u], st.qv[h], 0.f));
      if constexpr (TAIL) {
        s[u][h] = (u * S::TPI + row < nvalid) ? d : -INFINITY;
      } else {
        s[u][h] = d;
      }
    }
  }
  float negm[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float mx = s[0][h];
#pragma unroll
    for (int u = 1; u < U; ++u) mx = fmaxf(mx, s[u][h]);
    const float mnew = fmaxf(st.m[h], mx * scale_log2);  // scale > 0 commutes with max
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;  // this row has seen no token yet
    const float alpha = fast_exp2(st.m[h] - msafe);
    st.l[h] *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
    st.m[h] = mnew;
    negm[h] = -msafe;
  }
#pragma unroll
  for (int u = 0; u < U; ++u) {
    float vf[8];
    vf[0] = bf16_lo(vr[u].x); vf[1] = bf16_hi(vr[u].x);
    vf[2] = bf16_lo(vr[u].y); vf[3] = bf16_hi(vr[u].y);
    vf[4] = bf16_lo(vr[u].z); vf[5] = bf16_hi(vr[u].z);
    vf[6] = bf16_lo(vr[u].w); vf[7] = bf16_hi(vr[u].w);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = fast_exp2(fmaf(s[u][h], scale_log2, negm[h]));
      st.l[h] += p;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] = fmaf(p, vf[e], st.acc[h][e]);
    }
  }
#endif
}

template <int D, int G>
__global__ __launch_bounds__(kWave) __attribute__((amdgpu_waves_per_eu(PA_DECODE_WAVES)))
void decode_split_kernel(DecodeArgs a) {
  constexpr int U = PA_DECODE_UNROLL;
  using S = SplitState<D, G, U>;
  constexpr int LPT = S::LPT;
  constexpr int CHUNK = S::CHUNK;
  static_assert(kBlockSize % CHUNK == 0, "a chunk never straddles a block");

  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * G;
#ifndef PA_DECODE_ORDER
#define PA_DECODE_ORDER 1
#endif
  int idx = blockIdx.x;
#if PA_DECODE_ORDER == 2
  // partition fastest: a sequence's items are dispatched together
  const int part = idx % a.max_parts;
  idx /= a.max_parts;
  const int g = idx % H_kv;
  const int b = idx / H_kv;
#else
  const int g = idx % H_kv;
  idx /= H_kv;
  const int b = idx % a.num_seqs;
#if PA_DECODE_ORDER == 1
  // highest partitions first: the items dispatched last are the first
  // partitions, which every sequence has, so the grid drains evenly
  const int part = a.max_parts - 1 - idx / a.num_seqs;
#else
  const int part = idx / a.num_seqs;
#endif
#endif
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
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  S st;
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const uint4 t = *reinterpret_cast<const uint4*>(a.q + (head0 + h) * D + sub * 8);
    st.qv[h][0] = t.x; st.qv[h][1] = t.y; st.qv[h][2] = t.z; st.qv[h][3] = t.w;
    st.m[h] = -INFINITY;
    st.l[h] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
  }

  const int64_t row_bytes = (int64_t)H_kv * D * 2;  // bytes per token row of a cache
  const int lane_off = row * (int)row_bytes + (g * D + sub * 8) * 2;
  const int tail_lane_off = (g * D + sub * 8) * 2;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  const int nfull = (end - start) / CHUNK;  // chunks with no token past the end
  // base byte offset of full chunk i; a broken table entry reads block 0 and
  // the chunk is skipped
  auto chunk_off = [&](int i, bool& ok) -> int64_t {
    const int cc = start + i * CHUNK;
    const int blk = bt[cc / kBlockSize];
    ok = blk >= 0 && blk < a.num_blocks;
    return ((int64_t)(ok ? blk : 0) * kBlockSize + (cc % kBlockSize)) * row_bytes;
  };
#if PA_DECODE_PIPE
  // Two register buffers: chunk i+1's loads are in flight while chunk i is
  // computed. The prefetch index is clamped to the last full chunk, so every
  // issue is unconditional and the memory-counter waits are static.
  if (nfull > 0) {
    uint4 ka[U], va[U], kb[U], vb[U];
    bool oka, okb;
    int64_t off = chunk_off(0, oka);
    issue_chunk<D, G, U, false>(kc + off, vc + off, row_bytes, lane_off, row, 0, ka, va);
    for (int i = 0; i < nfull; i += 2) {
      off = chunk_off(min(i + 1, nfull - 1), okb);
      issue_chunk<D, G, U, false>(kc + off, vc + off, row_bytes, lane_off, row, 0, kb, vb);
      if (oka) compute_chunk<D, G, U, false>(st, a.scale_log2, row, CHUNK, ka, va);
      if (i + 1 >= nfull) break;
      off = chunk_off(min(i + 2, nfull - 1), oka);
      issue_chunk<D, G, U, false>(kc + off, vc + off, row_bytes, lane_off, row, 0, ka, va);
      if (okb) compute_chunk<D, G, U, false>(st, a.scale_log2, row, CHUNK, kb, vb);
    }
  }
#else
  for (int i = 0; i < nfull; ++i) {
    bool ok;
    const int64_t off = chunk_off(i, ok);
    if (!ok) continue;
    uint4 kr[U], vr[U];
    issue_chunk<D, G, U, false>(kc + off, vc + off, row_bytes, lane_off, row, 0, kr, vr);
    compute_chunk<D, G, U, false>(st, a.scale_log2, row, CHUNK, kr, vr);
  }
#endif
  const int c = start + nfull * CHUNK;
  if (c < end) {
    const int blk = bt[c / kBlockSize];
    if (blk >= 0 && blk < a.num_blocks) {
      const int64_t off = ((int64_t)blk * kBlockSize + (c % kBlockSize)) * row_bytes;
      uint4 kr[U], vr[U];
      issue_chunk<D, G, U, true>(kc + off, vc + off, row_bytes, tail_lane_off, row, end - 1 - c,
                                 kr, vr);
      compute_chunk<D, G, U, true>(st, a.scale_log2, row, end - c, kr, vr);
    }
  }

  // Merge the token-rows of lanes (each has its own running max).
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float M = st.m[h];
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) M = fmaxf(M, xor_lane(M, off));
    const float w = (st.m[h] == -INFINITY) ? 0.f : exp2f(st.m[h] - M);
    float lh = st.l[h] * w;
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) lh += xor_lane(lh, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float o = st.acc[h][e] * w;
#pragma unroll
      for (int off = LPT; off < kWave; off <<= 1) o += xor_lane(o, off);
      st.acc[h][e] = o;
    }
    st.m[h] = M;
    st.l[h] = lh;
  }

  if (nparts == 1) {
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float inv = 1.f / st.l[h];
        uint4 o;
        o.x = pack_bf16x2(st.acc[h][0] * inv, st.acc[h][1] * inv);
        o.y = pack_bf16x2(st.acc[h][2] * inv, st.acc[h][3] * inv);
        o.z = pack_bf16x2(st.acc[h][4] * inv, st.acc[h][5] * inv);
        o.w = pack_bf16x2(st.acc[h][6] * inv, st.acc[h][7] * inv);
        *reinterpret_cast<uint4*>(a.out + (head0 + h) * D + sub * 8) = o;
      }
    }
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const int64_t wi = (head0 + h) * a.max_parts + part;
      if (row == 0) {
        float4* dst = reinterpret_cast<float4*>(a.ws_o + wi * D + sub * 8);
        dst[0] = make_float4(st.acc[h][0], st.acc[h][1], st.acc[h][2], st.acc[h][3]);
        dst[1] = make_float4(st.acc[h][4], st.acc[h][5], st.acc[h][6], st.acc[h][7]);
      }
      if (lane == 0) *reinterpret_cast<float2*>(a.ws_ml + wi * 2) = make_float2(st.m[h], st.l[h]);
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

int default_partition_blocks(const pa_desc*, int32_t, int32_t) { return 4; }

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

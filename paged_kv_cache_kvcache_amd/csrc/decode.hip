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
//   * split-K: a work item is (sequence, group of KPW adjacent kv-heads,
//     partition of up to 16 units of 256 tokens, sized from the batch), one
//     wave64 each; a second kernel merges the partitions' (max, sum,
//     unnormalised output) triples exactly. Sequences that fit one
//     partition are finished by the first kernel.
//   * dispatch: when the grid has more items than CUs, a one-workgroup
//     kernel first ranks them longest first and lays the ranks out so each
//     CU gets long and short items in turn; the bandwidth-bound grid then
//     drains on short items. Batches of more than 4,096 sequences keep the
//     plain order (highest partition first).
//   * loads in flight: at full occupancy a wave waits for a chunk's loads
//     before issuing the next chunk's; with fewer waves two chunks overlap
//     (the host picks the kernel).
//   * GQA: each lane holds the G q-heads of its kv-head, so one K/V load
//     serves G heads.
//   * loads: 16 bytes per lane, nontemporal (K/V are read once); d/8 lanes
//     cover one kv-head vector and KPW adjacent kv-heads make a 512-byte
//     contiguous piece of a token row. A chunk is eight loads of K and
//     eight of V, and the next chunk's
//     loads are issued before the current chunk is multiplied (two register
//     buffers; block-table entries are read two chunks ahead).
//   * q.k: v_dot2_f32_bf16 on the raw bf16 pairs (exact products, fp32 sum),
//     then DPP exchanges (no LDS); at d = 128 a transposed butterfly leaves
//     each lane with one token's full score.
//   * softmax: base-2 exponent (raw v_exp_f32) with scale*log2(e) folded into
//     one FMA; each token-row of lanes keeps its own running max; rows merge
//     once at the end.
//   * P.V: weights rounded to bf16 pairs, v_dot2_f32_bf16 on paired V rows,
//     fp32 accumulation; the sum adds the same rounded weights.
//   * 8 or more q-heads per kv-head (and group sizes that are not powers of
//     two): the vector work per byte grows with the group and would bound
//     the kernel, so both products run on
//     the matrix cores instead (v_mfma_f32_16x16x32_bf16, the q-heads as
//     the 16 columns), with each chunk's K rows and V^T staged through a
//     per-wave LDS region (compute_chunk_mf). Loads, pipeline and dispatch
//     are the same.
#include <cmath>
#include <mutex>
#include <type_traits>

#include "common.hpp"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;  // null: lengths are cu_k[b+1] - cu_k[b]
  const int32_t* cu_k;
  float* ws_o;   // [num_seqs, H_q, max_parts, d] fp32 unnormalised partial outputs
  float* ws_ml;  // [num_seqs, H_q, max_parts, 2]  (running max in log2 units, sum)
  uint16_t* out;
  // fused store (pa_decode_step): the newest token of each sequence comes
  // from k_new/v_new and is written to the cache at slot_mapping[b]
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_cache_w;  // the caches, written only by the fused store
  uint16_t* v_cache_w;
  const int32_t* slot_mapping;
  int64_t k_new_stride;  // elements between tokens of k_new / v_new
  int64_t v_new_stride;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t part_tokens;
  int32_t max_parts;
  int32_t block_size;   // tokens per physical block (power of two)
  int32_t block_shift;  // log2(block_size)
  int32_t* order;  // dispatch order (decode_order_kernel), or null: plain order
  // partition length chosen by decode_order_kernel (null: part_tokens)
  int32_t* part_dev;
  int32_t group;   // q-heads per kv-head
  int32_t max_ctx;  // host bound of the lengths (the stream grid cuts longer ones there)
  // layout of a partial's o[d] (see decode_piece): 0 = element order (the
  // matrix-core path), else the lanes per head vector of the vector path
  int32_t vec_lpt;
  int32_t* counters;  // stream grid: arrival count per (sequence, kv-head), zero between calls
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

__device__ __forceinline__ int seq_len(const DecodeArgs& a, int b) {
  return a.context_lens ? a.context_lens[b] : a.cu_k[b + 1] - a.cu_k[b];
}

__device__ __forceinline__ int clamp_len(int n, int max_blocks, int block_size) {
  return (int)max((int64_t)0, min((int64_t)n, (int64_t)max_blocks * block_size));
}

// How a sequence of n tokens is cut into work items: k = ceil(n / P)
// partitions of P tokens (at most max_parts; a length past max_parts * P is
// cut there), the last one shorter. (Cutting a sequence into k parts of
// equal length instead measured 3% slower at the Qwen3-8B batch.)
struct Parts {
  int n;  // tokens covered
  int k;  // parts
};

__device__ __forceinline__ Parts split_parts(int n, int P, int max_parts) {
  Parts r;
  r.n = min(n, max_parts * P);
  r.k = (r.n + P - 1) / P;
  return r;
}

// Partition lengths are counted in units of 256 tokens, whatever the block size.
constexpr int kPartUnit = 256;
// Longest partition (units): 2^30 tokens, the longest context accepted.
constexpr int kMaxPartUnits = 1 << 22;
constexpr int32_t kMaxContext = kMaxPartUnits * kPartUnit;

// Tokens per partition of this call: the host's, or the order kernel's
// choice when it ran (never shorter than the grid and workspace allow).
__device__ __forceinline__ int part_tokens(const DecodeArgs& a) {
  return a.part_dev ? __builtin_amdgcn_readfirstlane(*a.part_dev) : a.part_tokens;
}

// Byte offset in a cache of token `pos` of a sequence, given the table entry
// blk of its block: the physical block, then the offset inside it. A broken
// entry (precondition violated) reads block 0: the result is then
// meaningless, but the access stays inside the pool.
__device__ __forceinline__ int64_t block_offset(const DecodeArgs& a, int blk, int pos,
                                                int64_t row_bytes) {
  blk = (blk >= 0 && blk < a.num_blocks) ? blk : 0;
  return (((int64_t)blk << a.block_shift) + (pos & (a.block_size - 1))) * row_bytes;
}

__device__ __forceinline__ int64_t token_offset(const DecodeArgs& a, const int32_t* bt, int pos,
                                                int64_t row_bytes) {
  return block_offset(a, bt[pos >> a.block_shift], pos, row_bytes);
}

// Load instructions per chunk on the vector path (group sizes 1, 2, 4).
constexpr int kVecUnroll = 8;
// Waves per SIMD the split kernel is compiled for (its register budget).
constexpr int kSplitWavesPerSimd = 2;

// K/V rows are read exactly once per call: nontemporal loads keep them from
// displacing reusable lines (tables, q) in the caches.
__device__ __forceinline__ uint4 load16(const char* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(r.x, r.y, r.z, r.w);
}

// Before a chunk's loads are issued (U loads each of K and V), optionally
// wait until the previous chunk's loads have all arrived (s_waitcnt
// vmcnt(0); the export and LDS/scalar counters are left alone), so a wave
// has one chunk of loads in flight while it multiplies the chunk before.
// Without the wait the compiler's partial waits inside the multiply let two
// chunks' loads overlap. With every wave slot of the chip filled, the
// overlap only adds requests to already full memory queues (measured 5%
// slower at the Qwen3-8B batch); with fewer waves it is what keeps enough
// bytes in flight (waiting here measured up to twice as slow at one wave
// per SIMD), so the host picks the kernel, and a kernel built with the wait
// may skip it at run time (`on`, wave-uniform). Chunks of 4 loads never
// wait.
template <int U, bool DRAIN>
__device__ __forceinline__ void drain_loads(bool on) {
  if constexpr (DRAIN && U == 8) {
    __builtin_amdgcn_sched_barrier(0);  // not hoisted into the multiply before it
    if (on) __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), acc, false);
}

// Two fp32 -> packed bf16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack2_bf16_hw(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Raw v_exp_f32 (2^x). Arguments are <= 0 here; results below the normal
// range flush to zero, which is what a softmax weight that small should be.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane geometry: d/8 lanes hold one kv-head's vector of a token (16 bytes
// each); KPW adjacent kv-heads of the same token form one contiguous segment
// of KPW * 2d bytes, and a wave load instruction covers TPI tokens of it.
template <int D, int KPW>
struct Lanes {
  static constexpr int LPT = D / 8;             // lanes per kv-head vector
  static constexpr int SEG = LPT * KPW;         // lanes per token segment
  static constexpr int TPI = kWave / SEG;       // tokens per wave load instruction
  static_assert(kWave % SEG == 0, "segments tile the wave");
};

// Per-wave state of one work item.
template <int D, int G>
struct SplitState {
  uint32_t qv[G][4];
  float m[G], l[G], acc[G][8];  // running max (log2 units), sum, unnormalised output
};

// Loads of a full chunk inside one block: tokens c .. c+CHUNK-1 from a
// wave-uniform base plus one per-lane offset.
template <class S, int U>
__device__ __forceinline__ void issue_chunk(const char* kbase, const char* vbase, int64_t row_bytes,
                                            int lane_off, uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) kr[u] = load16(kbase + (int64_t)u * S::TPI * row_bytes + lane_off);
#pragma unroll
  for (int u = 0; u < U; ++u) vr[u] = load16(vbase + (int64_t)u * S::TPI * row_bytes + lane_off);
}

// Loads of a full chunk whose load groups (TPI tokens each) may lie in
// different blocks: one base offset per group.
template <int U>
__device__ __forceinline__ void issue_chunk_groups(const char* kc, const char* vc,
                                                   const int64_t (&off)[U], int lane_off,
                                                   uint4 (&kr)[U], uint4 (&vr)[U]) {
#pragma unroll
  for (int u = 0; u < U; ++u) kr[u] = load16(kc + off[u] + lane_off);
#pragma unroll
  for (int u = 0; u < U; ++u) vr[u] = load16(vc + off[u] + lane_off);
}

// DPP lane maps inside a 16-lane row (checked on gfx950): lane i reads lane
// i^1, i^2, i^7 (mirror inside each 8-lane half) or i^8 (rotate by 8), or
// lane n of its row (broadcast).
constexpr int kDppXor1 = kDppQuadXor1;
constexpr int kDppXor2 = kDppQuadXor2;
constexpr int kDppXor7 = kDppRowHalfMirror;
constexpr int kDppXor8 = kDppRowRor8;
constexpr int kDppBcast0 = 0x150;  // row_newbcast:n is kDppBcast0 + n

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, Ctrl, 0xF, 0xF, true);
}

// keep + the partner's `send`, where a lane whose selector bit is set keeps
// the upper value of the pair and sends the lower one (and the reverse).
template <int Ctrl>
__device__ __forceinline__ float fold(float lo, float hi, bool sel) {
  const float keep = sel ? hi : lo;
  const float send = sel ? lo : hi;
  return keep + dpp<Ctrl>(send);
}

// compute_chunk for 16 lanes per kv-head vector (d = 128) and 4 or 8 loads
// per chunk: the 16-lane sums of the U partial dot products are folded so
// that each lane ends with the full score of ONE token (a transposed
// butterfly: every exchange halves the values a lane keeps), so the softmax
// runs one exponential per lane and head instead of U. With lane bits
// b0, b1, b2 of the lane inside its 8-lane half, the lane holds token
//   U = 8: u = 4*b2 + 2*b1 + b0      U = 4: u = 2*b2 + b0.
// Tokens 2k and 2k+1 sit in lanes i and i^1: their weights are packed into
// one bf16 pair there and broadcast to the row for the P.V products.
template <class S, int D, int G, int U, bool TAIL>
__device__ __forceinline__ void compute_chunk_t(SplitState<D, G>& st, float scale_log2, int lane,
                                                int row, int nvalid, const uint4 (&kr)[U],
                                                const uint4 (&vr)[U]) {
  static_assert(S::LPT == 16 && (U == 4 || U == 8), "16-lane vectors, 4 or 8 loads");
  const bool b0 = lane & 1, b1 = lane & 2, b2 = lane & 4;
  const int u_me = U == 8 ? (b2 ? 4 : 0) + (b1 ? 2 : 0) + (b0 ? 1 : 0) : (b2 ? 2 : 0) + (b0 ? 1 : 0);
  float sc[G];  // this lane's token's raw q.k per head
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float x[U];
#pragma unroll
    for (int u = 0; u < U; ++u) x[u] = dot8_bf16(kr[u], st.qv[h], 0.f);
    float y;
    if constexpr (U == 8) {
      float y1[4], y2[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) y1[k] = fold<kDppXor7>(x[k], x[k + 4], b2);   // u bit 2
#pragma unroll
      for (int k = 0; k < 2; ++k) y2[k] = fold<kDppXor2>(y1[k], y1[k + 2], b1);  // u bit 1
      y = fold<kDppXor1>(y2[0], y2[1], b0);                                        // u bit 0
    } else {
      float y1[2];
#pragma unroll
      for (int k = 0; k < 2; ++k) y1[k] = fold<kDppXor7>(x[k], x[k + 2], b2);  // u bit 1
      y = fold<kDppXor1>(y1[0], y1[1], b0);                                      // u bit 0
      y += dpp<kDppXor2>(y);
    }
    y += dpp<kDppXor8>(y);
    if constexpr (TAIL) y = (u_me * S::TPI + row < nvalid) ? y : -INFINITY;
    sc[h] = y;
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    // chunk max over the row's tokens (all 8 lanes of the half row)
    float mx = fmaxf(sc[h], dpp<kDppXor1>(sc[h]));
    if constexpr (U == 8) mx = fmaxf(mx, dpp<kDppXor2>(mx));
    mx = fmaxf(mx, dpp<kDppXor7>(mx));
    const float mnew = fmaxf(st.m[h], mx * scale_log2);  // scale > 0 commutes with max
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;  // this row has seen no token yet
    const float alpha = fast_exp2(st.m[h] - msafe);
    st.l[h] *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) st.acc[h][e] *= alpha;
    st.m[h] = mnew;
    const float p = fast_exp2(fmaf(sc[h], scale_log2, -msafe));
    // (p of token 2k, p of token 2k+1) as one bf16 pair, then to every lane
    const float pp = dpp<kDppXor1>(p);
    const uint32_t pk = pack2_bf16_hw(b0 ? pp : p, b0 ? p : pp);
    uint32_t ppair[U / 2];
    if constexpr (U == 8) {
      ppair[0] = dpp_u32<kDppBcast0 + 0>(pk);
      ppair[1] = dpp_u32<kDppBcast0 + 2>(pk);
      ppair[2] = dpp_u32<kDppBcast0 + 4>(pk);
      ppair[3] = dpp_u32<kDppBcast0 + 6>(pk);
    } else {
      ppair[0] = dpp_u32<kDppBcast0 + 0>(pk);
      ppair[1] = dpp_u32<kDppBcast0 + 4>(pk);
    }
    // P.V on token pairs with v_dot2_f32_bf16; the sum adds the same rounded
    // weights, so the output stays an exact weighted mean
#pragma unroll
    for (int k = 0; k < U / 2; ++k) {
      st.l[h] += bf16_lo(ppair[k]) + bf16_hi(ppair[k]);
      const uint32_t a4[4] = {vr[2 * k].x, vr[2 * k].y, vr[2 * k].z, vr[2 * k].w};
      const uint32_t c4[4] = {vr[2 * k + 1].x, vr[2 * k + 1].y, vr[2 * k + 1].z, vr[2 * k + 1].w};
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t lo = __builtin_amdgcn_perm(c4[w], a4[w], 0x05040100u);  // element 2w
        const uint32_t hi = __builtin_amdgcn_perm(c4[w], a4[w], 0x07060302u);  // element 2w+1
        st.acc[h][2 * w] = dot2_bf16(lo, ppair[k], st.acc[h][2 * w]);
        st.acc[h][2 * w + 1] = dot2_bf16(hi, ppair[k], st.acc[h][2 * w + 1]);
      }
    }
  }
}

template <class S, int D, int G, int U, bool TAIL>
__device__ __forceinline__ void compute_chunk_v(SplitState<D, G>& st, float scale_log2, int lane,
                                              int row, int nvalid, const uint4 (&kr)[U],
                                              const uint4 (&vr)[U]) {
  if constexpr (S::LPT == 16 && (U == 4 || U == 8)) {
    compute_chunk_t<S, D, G, U, TAIL>(st, scale_log2, lane, row, nvalid, kr, vr);
    return;
  }
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
  if constexpr (U % 2 == 0) {
  // P.V on token pairs with v_dot2_f32_bf16: (V[t][e], V[t+1][e]) packed by
  // v_perm, weights rounded to bf16 as the MFMA prefill does. The sum l adds
  // the same rounded weights, so the output stays an exact weighted mean.
  // (A single token -- the fused step's newest one at d = 64 -- takes the
  // fp32 form below.)
#pragma unroll
  for (int u = 0; u < U; u += 2) {
    uint32_t ppair[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p0 = fast_exp2(fmaf(s[u][h], scale_log2, negm[h]));
      const float p1 = fast_exp2(fmaf(s[u + 1][h], scale_log2, negm[h]));
      ppair[h] = pack2_bf16_hw(p0, p1);
      st.l[h] += bf16_lo(ppair[h]) + bf16_hi(ppair[h]);
    }
    const uint32_t a[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
    const uint32_t c[4] = {vr[u + 1].x, vr[u + 1].y, vr[u + 1].z, vr[u + 1].w};
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = __builtin_amdgcn_perm(c[w], a[w], 0x05040100u);  // element 2w
      const uint32_t hi = __builtin_amdgcn_perm(c[w], a[w], 0x07060302u);  // element 2w+1
#pragma unroll
      for (int h = 0; h < G; ++h) {
        st.acc[h][2 * w] = dot2_bf16(lo, ppair[h], st.acc[h][2 * w]);
        st.acc[h][2 * w + 1] = dot2_bf16(hi, ppair[h], st.acc[h][2 * w + 1]);
      }
    }
  }
  } else {
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
  }
}

// ---- matrix-core variant (one kv-head per wave, up to 16 q-heads)
//
// The chunk's 32 tokens go through a per-wave LDS region so that both
// products run on v_mfma_f32_16x16x32_bf16 with the q-heads as the 16
// columns: S^T = K Q^T, then O^T += V^T P^T. In the MFMA layouts lane
// (g, i) = (lane / 16, lane % 16); the S^T accumulator of 16-token tile T
// gives it, in register c, the score of q-head i for K row 4g + c of the
// tile. The loads are placed so that those 8 scores (two tiles) are the 8
// keys of lane group g in the B operand of the P.V product, and V^T is staged
// in the same key order (slot 8g + 4T + c), so P stays in registers:
//   d = 128: lane (r, s) = (lane / 16, lane % 16) loaded token 4u + r,
//     elements 8s .., u = 0..7; tile u >> 2, row 4r + (u & 3), so (T, g, c)
//     is token 16T + 4c + g;
//   d = 64: lane (r, s) = (lane / 8, lane % 8) loaded token 8u + r, u = 0..3;
//     tile r >> 2, row 4(r & 3) + u, so (T, g, c) is token 8c + 4T + g.
// Columns past G carry zero queries and are never written.
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <int D>
struct MfState {
  bf16x8 qf[D / 32];  // Q^T operand of k-step j: lane (g, i) = q-head i, elements 32j + 8g ..
  f32x4 o[D / 16];    // O^T tile mt: lane (g, i), register c = element 16mt + 4g + c of q-head i
  float m;            // column i's running max (log2 units); equal in the column's 4 lanes
  float l;            // this lane's share of column i's sum (its tokens only)
};

constexpr int mf_kbytes(int D) { return 2 * 16 * 2 * D; }  // two 16-token K tiles
constexpr int kMfVRow = 80;                                // V^T row: 32 keys x 2 B, padded
constexpr int mf_bytes(int D) { return mf_kbytes(D) + D * kMfVRow; }  // LDS per wave
// A column's reference max moves only when a score exceeds it by more than
// kMfLazy in log2 units, so a weight stays below 2^8: far inside the bf16 and
// fp32 ranges, and most chunks skip the rescale.
constexpr float kMfLazy = 8.f;

// acc + lo + hi of a packed bf16 pair, summed in fp32 (v_dot2_f32_bf16 with
// the pair (1, 1)).
__device__ __forceinline__ float sum_pair_bf16(uint32_t pair, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

// LDS rows are swizzled so that the accesses below are free of bank
// conflicts (V^T writes at d = 64: two-way): K block b of row rho sits at
// b ^ (rho mod the blocks per row); the V^T 16-byte group of lane group g in
// row d sits at g ^ ((d >> 4) & 3).
template <int D, bool TAIL>
__device__ __forceinline__ void compute_chunk_mf(MfState<D>& st, char* lds, float scale_log2,
                                                 int lane, int nvalid, const uint4 (&kr)[D / 16],
                                                 const uint4 (&vr)[D / 16]) {
  constexpr int U = D / 16;          // loads per chunk (32 tokens)
  constexpr int LPT = D / 8;         // lanes per token vector (16-byte blocks per row)
  constexpr int ROW = 2 * D;         // bytes per K row
  constexpr int TILE = 16 * ROW;     // bytes per 16-token K tile
  const int g = lane >> 4, i = lane & 15;      // MFMA roles
  const int r = lane / LPT, s = lane % LPT;    // load roles: token r of an instruction, block s
  char* vt = lds + mf_kbytes(D);
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int T = D == 128 ? u >> 2 : r >> 2;
    const int rho = D == 128 ? 4 * r + (u & 3) : 4 * (r & 3) + u;
    *reinterpret_cast<uint4*>(lds + T * TILE + rho * ROW + ((s ^ (rho & (LPT - 1))) << 4)) = kr[u];
  }
  // V^T: a dword holds tokens u = 2k (low) and 2k + 1 of the lane's row r
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t c[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t x4[4] = {vr[u].x, vr[u].y, vr[u].z, vr[u].w};
      c[u] = x4[w];
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t sel = e ? 0x07060302u : 0x05040100u;  // element 2w + e of both tokens
      const int d = 8 * s + 2 * w + e;
      if constexpr (D == 128) {  // slots 8r .. 8r+7: the whole 16-byte group
        uint4 x;
        x.x = __builtin_amdgcn_perm(c[1], c[0], sel);
        x.y = __builtin_amdgcn_perm(c[3], c[2], sel);
        x.z = __builtin_amdgcn_perm(c[5], c[4], sel);
        x.w = __builtin_amdgcn_perm(c[7], c[6], sel);
        *reinterpret_cast<uint4*>(vt + d * kMfVRow + ((r ^ ((d >> 4) & 3)) << 4)) = x;
      } else {  // slots 8(r & 3) + 4(r >> 2) .. +3: half of group r & 3
        uint2 x;
        x.x = __builtin_amdgcn_perm(c[1], c[0], sel);
        x.y = __builtin_amdgcn_perm(c[3], c[2], sel);
        *reinterpret_cast<uint2*>(vt + d * kMfVRow + (((r & 3) ^ ((d >> 4) & 3)) << 4) +
                                  8 * (r >> 2)) = x;
      }
    }
  }
  // a wave's LDS operations execute in order: only the compiler must keep
  // the reads below after the writes above
  asm volatile("" ::: "memory");
  f32x4 sc[2];
#pragma unroll
  for (int T = 0; T < 2; ++T) {
    sc[T] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const bf16x8 av = __builtin_bit_cast(
          bf16x8, *reinterpret_cast<const uint4*>(lds + T * TILE + i * ROW +
                                                  (((4 * j + g) ^ (i & (LPT - 1))) << 4)));
      sc[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, st.qf[j], sc[T], 0, 0, 0);
    }
  }
  float sv[8];  // K row 4g + c of tile T at index 4T + c
#pragma unroll
  for (int T = 0; T < 2; ++T)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float x = sc[T][c];
      const int t = D == 128 ? 16 * T + 4 * c + g : 8 * c + 4 * T + g;  // token in the chunk
      sv[4 * T + c] = (!TAIL || t < nvalid) ? x : -INFINITY;
    }
  float mx = sv[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) mx = fmaxf(mx, sv[k]);
  mx = fmaxf(mx, xor_lane(mx, 16));
  mx = fmaxf(mx, xor_lane(mx, 32));
  mx *= scale_log2;  // scale > 0 commutes with max
  if (mx > st.m + kMfLazy) {  // the column's 4 lanes agree
    const float mnew = fmaxf(st.m, mx);
    const float alpha = fast_exp2(st.m - mnew);  // 0 on the first chunk
    st.m = mnew;
    st.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] *= alpha;
  }
  const float negm = (st.m == -INFINITY) ? 0.f : -st.m;
  float p[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) p[k] = fast_exp2(fmaf(sv[k], scale_log2, negm));
  uint4 pk;
  pk.x = pack2_bf16_hw(p[0], p[1]);
  pk.y = pack2_bf16_hw(p[2], p[3]);
  pk.z = pack2_bf16_hw(p[4], p[5]);
  pk.w = pack2_bf16_hw(p[6], p[7]);
  // the sum adds the rounded weights the products see (an exact weighted mean)
  st.l = sum_pair_bf16(pk.x, st.l);
  st.l = sum_pair_bf16(pk.y, st.l);
  st.l = sum_pair_bf16(pk.z, st.l);
  st.l = sum_pair_bf16(pk.w, st.l);
  const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) {
    const int d = 16 * mt + i;
    const bf16x8 av = __builtin_bit_cast(
        bf16x8, *reinterpret_cast<const uint4*>(vt + d * kMfVRow + ((g ^ (mt & 3)) << 4)));
    st.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pf, st.o[mt], 0, 0, 0);
  }
  // the next chunk's LDS writes stay after these reads
  asm volatile("" ::: "memory");
}

// One chunk on either path: the matrix-core state takes chunks of 32 tokens
// (a single fused token is widened to a masked chunk of copies).
template <class L, int D, int G, int U, bool TAIL, class St>
__device__ __forceinline__ void compute_chunk(St& st, char* lds, float scale_log2, int lane,
                                              int row, int nvalid, const uint4 (&kr)[U],
                                              const uint4 (&vr)[U]) {
  if constexpr (std::is_same<St, MfState<D>>::value) {
    constexpr int UM = D / 16;
    if constexpr (U == UM) {
      compute_chunk_mf<D, TAIL>(st, lds, scale_log2, lane, nvalid, kr, vr);
    } else {
      uint4 kw[UM], vw[UM];
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        kw[u] = kr[u % U];
        vw[u] = vr[u % U];
      }
      compute_chunk_mf<D, true>(st, lds, scale_log2, lane, nvalid, kw, vw);
    }
  } else {
    compute_chunk_v<L, D, G, U, TAIL>(st, scale_log2, lane, row, nvalid, kr, vr);
  }
}

// Dispatch order of the split kernel's work items, longest first. The
// kernel is bandwidth-bound and its items differ in length (a sequence's
// last partition is partial), so handing out the longest items first lets
// the grid drain on short ones instead of ending on a few long stragglers.
// Items are ranked by length bucket (32 buckets of part_tokens/32 tokens;
// full partitions in the top one; empty sequences, which only write zeros,
// last). One workgroup ranks them before the split kernel runs (a histogram
// of the buckets, then each item takes the next rank of its bucket) and
// writes order[slot] = part << 12 | sequence, -1 past the last item (slot:
// the rank laid out by dispatch_slot), and the partition length it chose
// to the workspace; a split wave reads its one entry. (Each wave ranking
// the items itself from the lengths cost it 8-24 us: every wave read the
// same lengths.)
constexpr int kOrderMaxSeqs = 4096;  // sequence ids must fit 12 bits
constexpr int kOrderBuckets = 32;
constexpr int kOrderThreads = 1024;

__device__ __forceinline__ int len_bucket(int len, int part_tokens) {
  return 1 + (int)(((int64_t)(len - 1) * kOrderBuckets) / part_tokens);  // 1..32
}


// Where rank r goes in the dispatch order. Workgroups are dealt to the CUs
// in launch order, a round of `round` items (one per CU) at a time; in
// ranked order every CU would get the same place in each round, so the
// first CU would get the longest item of every round. Odd rounds are
// reversed, so each CU gets a long and a short item in turn.
__device__ __forceinline__ int dispatch_slot(int r, int round, int max_items) {
  const int k = r / round;
  const int start = k * round;
  const int len = min(round, max_items - start);
  return (k & 1) ? start + len - 1 - (r - start) : r;
}

// PartRule: the host's partition heuristic (default_partition_blocks), which
// estimates the mean length as half the longest. The order kernel reads
// every length and applies it to the tokens themselves (a short sequence
// counts its tokens, not a whole partition), between min_units and
// auto_units. auto_units = 0: the caller fixed the partition length.
struct PartRule {
  int auto_units;  // longest partition tried, in units of 256 tokens (0: keep the host's)
  int min_units;   // shortest allowed: the workspace and grid hold that many partitions
  int waves;       // waves per sequence and partition
  int fill;        // waves that count as filling the chip
};

__global__ __launch_bounds__(kOrderThreads) void decode_order_kernel(DecodeArgs a, int max_items,
                                                                     int round, PartRule rule) {
  constexpr int NB = kOrderBuckets + 1;
  __shared__ int next[NB];  // counts, then the next free rank of each bucket
  __shared__ int total;
  // each length read once from memory (the host orders at most this many)
  __shared__ int lens[kOrderMaxSeqs];
  __shared__ unsigned long long sum_len;
  __shared__ int chosen;
  const int t = threadIdx.x;
  if (t == 0) sum_len = 0;
  __syncthreads();
  unsigned long long mine = 0;
  for (int s = t; s < a.num_seqs; s += kOrderThreads) {
    const int n = clamp_len(seq_len(a, s), a.max_blocks, a.block_size);
    lens[s] = n;
    mine += (unsigned long long)n;
  }
  if (rule.auto_units > 0) {
    // one LDS atomic per wave
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) mine += __shfl_xor(mine, off, kWave);
    if (t % kWave == 0 && mine) atomicAdd(&sum_len, mine);
  }
  __syncthreads();
  if (t == 0) {
    // the host's rule on the true mean length (the longest partition whose
    // item count fills the chip), shortened further when the tokens
    // themselves would fill less than half of it (one long sequence among
    // short ones: each short one counts as a whole item but holds little
    // work), no shorter than the workspace and grid allow
    int P = a.part_tokens;
    if (rule.auto_units > 0) {
      const double mean = fmax(1.0, floor((double)sum_len / a.num_seqs));
      int by_items = rule.min_units, by_tokens = rule.min_units;
      for (int u = rule.auto_units; u > rule.min_units; u >>= 1) {
        const double per_seq = ceil(mean / (u * kPartUnit));
        if ((double)a.num_seqs * rule.waves * per_seq >= rule.fill) {
          by_items = u;
          break;
        }
      }
      for (int u = rule.auto_units; u > rule.min_units; u >>= 1) {
        if (2.0 * (double)sum_len * rule.waves >= (double)rule.fill * u * kPartUnit) {
          by_tokens = u;
          break;
        }
      }
      P = min(by_items, by_tokens) * kPartUnit;
    }
    chosen = P;
    *a.part_dev = P;
  }
  __syncthreads();
  const int P = chosen;
  // a sequence's items: `bulk` full partitions in bucket kb (the top one),
  // then its last part in bucket kl (an empty sequence: one item, in bucket 0)
  auto items = [&](int s, int& bulk, int& kb, int& kl) {
    const int n = lens[s];
    if (n == 0) {
      bulk = 0;
      kb = 0;
      kl = 0;
      return;
    }
    const Parts q = split_parts(n, P, a.max_parts);
    bulk = q.k - 1;
    kb = kOrderBuckets;
    kl = len_bucket(q.n - bulk * P, P);
  };
  if (t < NB) next[t] = 0;
  __syncthreads();
  for (int s = t; s < a.num_seqs; s += kOrderThreads) {
    int bulk, kb, kl;
    items(s, bulk, kb, kl);
    if (bulk) atomicAdd(&next[kb], bulk);
    atomicAdd(&next[kl], 1);
  }
  __syncthreads();
  if (t == 0) {
    int run = 0;
    for (int k = kOrderBuckets; k >= 0; --k) {
      const int c = next[k];
      next[k] = run;
      run += c;
    }
    total = run;
  }
  __syncthreads();
  // every item takes the next rank of its bucket (the order inside a bucket
  // does not matter: each item's result is the same whoever computes it)
  int32_t* order = a.order;
  for (int s = t; s < a.num_seqs; s += kOrderThreads) {
    int bulk, kb, kl;
    items(s, bulk, kb, kl);
    if (bulk) {
      const int pos = atomicAdd(&next[kb], bulk);
      for (int j = 0; j < bulk; ++j)
        order[dispatch_slot(pos + j, round, max_items)] = (j << 12) | s;
    }
    order[dispatch_slot(atomicAdd(&next[kl], 1), round, max_items)] = (bulk << 12) | s;
  }
  for (int r = total + t; r < max_items; r += kOrderThreads)
    order[dispatch_slot(r, round, max_items)] = -1;
}

// Partials are written and read with agent-scope atomic accesses (sc1:
// written through to, and read from, the level where every CU of the GPU
// sees the same data, past the per-XCD L2s), so a wave can publish its
// partial by waiting for its own stores to complete, without a release
// fence (which writes back the whole L2 of its XCD: about +100 us per call
// when every wave did it) or an acquire fence (which invalidates it).
__device__ __forceinline__ void store_agent(float* p, float x, float y) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                     __builtin_bit_cast(uint64_t, make_float2(x, y)), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float2 load_agent(const float* p) {
  return __builtin_bit_cast(float2, __hip_atomic_load(reinterpret_cast<const uint64_t*>(p),
                                                      __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// One piece of work: tokens [start, end) of sequence b (n tokens) for the
// wave's kv-heads. `direct`: the piece is the whole sequence, and the
// normalised output is written to out; otherwise the unnormalised partial
// (o, m, l) goes to workspace row `slot`, q-head h at index slot * H_q + h.
// SMALL: blocks hold fewer tokens than a chunk, so each load group looks up
// its own block; otherwise a chunk lies inside one block.
// Vector path (G = 1, 2, 4): one wave per workgroup (VS = 1), KPW adjacent
// kv-heads per wave.
// MF: the matrix-core variant (KPW = 1, G <= 16; G = 0 takes the group
// size from the arguments); with VS > 1 its waves take VS adjacent kv-heads,
// one each.
template <int D, int G, int KPW, bool FUSED, bool SMALL, bool DRAIN, int VS, bool MF>
__device__ __forceinline__ void decode_piece(const DecodeArgs& a, char* lds, int tid, int b,
                                             int n, int start, int end, bool direct,
                                             int64_t slot, bool drain_on = true) {
  static_assert(!MF || (KPW == 1 && G <= 16 && VS <= 4), "matrix-core geometry");
  static_assert(MF || G > 0, "the vector path is built per group size");
  const int Gn = G ? G : a.group;  // q-heads per kv-head
  constexpr bool kPair = MF && VS > 1;  // one kv-head per wave, VS per workgroup
  constexpr int U = MF ? D / 16 : kVecUnroll;  // matrix cores: chunks of 32 tokens
  using S = typename std::conditional<MF, MfState<D>, SplitState<D, (G ? G : 1)>>::type;
  using L = Lanes<D, KPW>;
  constexpr int LPT = L::LPT;
  constexpr int SEG = L::SEG;
  constexpr int TPI = L::TPI;
  constexpr int CHUNK = TPI * U;  // tokens per chunk
  static_assert(kMinBlockSize % TPI == 0, "a load group never straddles a block");

  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * Gn * (kPair ? 1 : VS);
  // kv-head groups (the host checks divisibility)
  const int n_groups = H_kv / (kPair ? VS : KPW);
  const int gw = blockIdx.x % n_groups;  // the kv-head groups of one item are adjacent
  const int lane = tid % kWave;
  // which G q-heads of the kv-head (or, kPair, which kv-head of the VS)
  const int half = VS == 1 ? 0 : tid / kWave;
  const int sub = lane % LPT;                 // which 8 elements of the head vector
  const int g = kPair ? gw * VS + half : gw * KPW + (lane / LPT) % KPW;  // this lane's kv-head
  const int row = lane / SEG;                 // which token of a load instruction
  const int64_t head0 = kPair ? (int64_t)b * H_q + (int64_t)g * Gn
                              : (int64_t)b * H_q + (int64_t)g * Gn * VS + half * Gn;  // first q-head
  const int64_t wrow = slot * H_q + (head0 - (int64_t)b * H_q);  // its partial row

  if (n == 0) {  // padding row: defined as zeros, nothing read
    if (row == 0) {
#pragma unroll
      for (int h = 0; h < Gn; ++h)
        *reinterpret_cast<uint4*>(a.out + (head0 + h) * D + sub * 8) = make_uint4(0, 0, 0, 0);
    }
    return;
  }
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  S st;
  if constexpr (MF) {
    // lane (g, i): q-head i (zeros past G), elements 32j + 8g .. +8
    const int qg = lane >> 4, qi = lane & 15;
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      uint4 t = make_uint4(0, 0, 0, 0);
      if (qi < Gn) t = *reinterpret_cast<const uint4*>(a.q + (head0 + qi) * D + 32 * j + 8 * qg);
      st.qf[j] = __builtin_bit_cast(bf16x8, t);
    }
    st.m = -INFINITY;
    st.l = 0.f;
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) st.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const uint4 t = *reinterpret_cast<const uint4*>(a.q + (head0 + h) * D + sub * 8);
      st.qv[h][0] = t.x; st.qv[h][1] = t.y; st.qv[h][2] = t.z; st.qv[h][3] = t.w;
      st.m[h] = -INFINITY;
      st.l[h] = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) st.acc[h][e] = 0.f;
    }
  }

  const int64_t row_bytes = (int64_t)H_kv * D * 2;  // bytes per token row of a cache
  const int lane_off = row * (int)row_bytes + (g * D + sub * 8) * 2;
  const int tail_lane_off = (g * D + sub * 8) * 2;
  const char* kc = reinterpret_cast<const char*>(a.k_cache);
  const char* vc = reinterpret_cast<const char*>(a.v_cache);
  // With the fused store the newest token (position n-1) is taken from
  // k_new/v_new instead of the cache: full chunks cover only [start, cend),
  // and the tail chunk, which then always exists, loads that token from the
  // inputs in the same round of loads as its cache rows.
  const bool has_new = FUSED && end == n;
  const int cend = has_new ? n - 1 : end;
  const int nfull = (cend - start) / CHUNK;  // chunks with no token past cend
  // Full chunk i: its first token and the table entries of its blocks (one
  // when the chunk lies in one block, else one per load group of TPI
  // tokens). i is clamped to the last full chunk, so a lookup ahead never
  // reads past the sequence's table entries. The entries are raw: the
  // offsets are formed in issue(), so a lookup ahead does not wait for its
  // table read.
  struct Lookup {
    int pos;
    int blk[SMALL ? U : 1];
  };
  auto lookup = [&](int i) {
    Lookup r;
    r.pos = start + min(i, nfull - 1) * CHUNK;
#pragma unroll
    for (int u = 0; u < (SMALL ? U : 1); ++u) r.blk[u] = bt[(r.pos + u * TPI) >> a.block_shift];
    return r;
  };
  auto issue = [&](const Lookup& t, uint4 (&kr)[U], uint4 (&vr)[U]) {
    if constexpr (!SMALL) {
      const int64_t off = block_offset(a, t.blk[0], t.pos, row_bytes);
      issue_chunk<L, U>(kc + off, vc + off, row_bytes, lane_off, kr, vr);
    } else {
      int64_t off[U];
#pragma unroll
      for (int u = 0; u < U; ++u) off[u] = block_offset(a, t.blk[u], t.pos + u * TPI, row_bytes);
      issue_chunk_groups<U>(kc, vc, off, lane_off, kr, vr);
    }
  };
  // Software pipeline over two register buffers: chunk i+1's loads are in
  // flight while chunk i is multiplied, and the table entry of chunk i+2 is
  // read before chunk i+1's loads are issued, so it has arrived by the time
  // it is needed (a table read right before its chunk's loads would put its
  // latency in front of every chunk; after a drain the compiler makes table
  // reads vector loads, which complete in order behind the chunk's loads).
  // The loop body has no branches. The last one or two chunks are finished
  // after the loop, so no chunk is loaded twice.
  if (nfull > 0) {
    uint4 ka[U], va[U], kb[U], vb[U];
    issue(lookup(0), ka, va);
    Lookup next = lookup(1);
    int i = 0;
    for (; i + 2 < nfull; i += 2) {
      drain_loads<U, DRAIN>(drain_on);
      const Lookup after = lookup(i + 2);
      issue(next, kb, vb);  // chunk i+1
      __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the multiply
      compute_chunk<L, D, G, U, false>(st, lds, a.scale_log2, lane, row, CHUNK, ka, va);
      drain_loads<U, DRAIN>(drain_on);
      next = lookup(i + 3);
      issue(after, ka, va);  // chunk i+2 (clamped)
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk<L, D, G, U, false>(st, lds, a.scale_log2, lane, row, CHUNK, kb, vb);
    }
    if (i + 1 < nfull) {
      drain_loads<U, DRAIN>(drain_on);
      issue(next, kb, vb);  // chunk i+1
      __builtin_amdgcn_sched_barrier(0);
      compute_chunk<L, D, G, U, false>(st, lds, a.scale_log2, lane, row, CHUNK, ka, va);
      compute_chunk<L, D, G, U, false>(st, lds, a.scale_log2, lane, row, CHUNK, kb, vb);
    } else if (i < nfull) {
      compute_chunk<L, D, G, U, false>(st, lds, a.scale_log2, lane, row, CHUNK, ka, va);
    }
  }
  const int c = start + nfull * CHUNK;
  if (c < end) {
    // tail: every lane finds its own token's row (clamped to the last valid
    // token, which is masked out again in compute_chunk); the newest token's
    // row comes from k_new/v_new
    const char* kn = nullptr;
    const char* vn = nullptr;
    const int slot_new = has_new ? a.slot_mapping[b] : -1;  // read early, used last
    if constexpr (FUSED) {
      kn = reinterpret_cast<const char*>(a.k_new + (int64_t)b * a.k_new_stride + g * D + sub * 8);
      vn = reinterpret_cast<const char*>(a.v_new + (int64_t)b * a.v_new_stride + g * D + sub * 8);
    }
    uint4 kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = min(u * TPI + row, end - 1 - c);
      const bool fresh = has_new && c + t == n - 1;  // per lane: one load either way
      const int64_t off = fresh ? 0 : token_offset(a, bt, c + t, row_bytes) + tail_lane_off;
      kr[u] = load16(fresh ? kn : kc + off);
      vr[u] = load16(fresh ? vn : vc + off);
    }
    compute_chunk<L, D, G, U, true>(st, lds, a.scale_log2, lane, row, end - c, kr, vr);
    if (has_new) {
      // write the newest token to its slot (no piece of this call reads that
      // cache row) from the lanes whose last load holds it: token e of the
      // tail is load U-1 of row max(0, e - (U-1) * TPI)
      const int e = end - 1 - c;
      if (row == max(0, e - (U - 1) * TPI) && (kPair || half == 0) && slot_new >= 0 &&
          slot_new < (a.num_blocks << a.block_shift)) {
        const int64_t dst = (int64_t)slot_new * H_kv * D + g * D + sub * 8;
        *reinterpret_cast<uint4*>(a.k_cache_w + dst) = kr[U - 1];
        *reinterpret_cast<uint4*>(a.v_cache_w + dst) = vr[U - 1];
      }
    }
  }

  if constexpr (MF) {
    // column sums across the 4 lane groups; the max is already common
    const int lg = lane >> 4, li = lane & 15;
    float lt = st.l;
    lt += xor_lane(lt, 16);
    lt += xor_lane(lt, 32);
    if (li < Gn) {
      if (direct) {
        const float inv = 1.f / lt;
        uint16_t* dst = a.out + (head0 + li) * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
          uint2 v;
          v.x = pack_bf16x2(st.o[mt][0] * inv, st.o[mt][1] * inv);
          v.y = pack_bf16x2(st.o[mt][2] * inv, st.o[mt][3] * inv);
          *reinterpret_cast<uint2*>(dst + 16 * mt) = v;
        }
      } else {
        const int64_t wi = wrow + li;
        float* dst = a.ws_o + wi * D + 4 * lg;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) {
          store_agent(dst + 16 * mt, st.o[mt][0], st.o[mt][1]);
          store_agent(dst + 16 * mt + 2, st.o[mt][2], st.o[mt][3]);
        }
        if (lg == 0) store_agent(a.ws_ml + wi * 2, st.m, lt);
      }
    }
  } else {
    // Merge the token-rows of lanes (each has its own running max); lanes
    // SEG apart hold the same kv-head.
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float M = st.m[h];
#pragma unroll
      for (int off = SEG; off < kWave; off <<= 1) M = fmaxf(M, xor_lane(M, off));
      const float w = (st.m[h] == -INFINITY) ? 0.f : exp2f(st.m[h] - M);
      float lh = st.l[h] * w;
#pragma unroll
      for (int off = SEG; off < kWave; off <<= 1) lh += xor_lane(lh, off);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float o = st.acc[h][e] * w;
#pragma unroll
        for (int off = SEG; off < kWave; off <<= 1) o += xor_lane(o, off);
        st.acc[h][e] = o;
      }
      st.m[h] = M;
      st.l[h] = lh;
    }

    if (direct) {
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
        const int64_t wi = wrow + h;
        // o[d] is stored pair-major (element pair k of lane group sub at
        // 2 LPT k + 2 sub), so each store instruction writes LPT * 8
        // contiguous bytes: element order would leave every 8-byte store 32
        // bytes from its neighbour, and partial lines cost more to write
        // through than their data
        if (row == 0) {
          float* dst = a.ws_o + wi * D + sub * 2;
#pragma unroll
          for (int k = 0; k < 4; ++k)
            store_agent(dst + 2 * LPT * k, st.acc[h][2 * k], st.acc[h][2 * k + 1]);
        }
        if (row == 0 && sub == 0) store_agent(a.ws_ml + wi * 2, st.m[h], st.l[h]);
      }
    }
  }
}

// Exact log-sum-exp merge of the partials of one sequence, for q-heads
// h0 .. h0+nh-1 of sequence b, partial rows slot0 .. slot0+np-1:
// M = max m_p, L = sum l_p 2^(m_p - M), out = sum o_p 2^(m_p - M) / L.
// One wave; HP (a power of two, at least nh) heads share it, 64/HP lanes
// per head, each with D*HP/64 adjacent elements. The partials are read KP
// at a time (one round of loads for up to that many) and folded into a
// running max, so a merge of up to KP partials waits for memory once.
// Where element d of a partial's o[] sits: element order, or pair-major for
// the vector path (pair (d mod 8) / 2 of lane group d / 8 at 2 lpt pair +
// 2 group; pairs (d, d + 1), d even, stay adjacent).
__device__ __forceinline__ int partial_pos(int lpt, int d) {
  return lpt ? ((d & 7) >> 1) * 2 * lpt + (d >> 3) * 2 + (d & 1) : d;
}

template <int D, int HP>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int H_q, int b, int h0, int nh,
                                             int64_t slot0, int np) {
  constexpr int LPH = kWave / HP;  // lanes per head
  constexpr int EPL = D / LPH;     // elements per lane
  static_assert(LPH >= 1 && EPL >= 1 && EPL <= 32, "merge geometry");
  constexpr int KP = EPL >= 32 ? 4 : 8;  // up to 128 registers of partials per round (8 at a
                                         // time: 32 x 16,384 tokens, 341 -> 336 us)
  const int lane = threadIdx.x % kWave;
  const int h = lane / LPH;
  if (h >= nh) return;
  const int e0 = (lane % LPH) * EPL;
  float M = -INFINITY, Lsum = 0.f;
  float o[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) o[e] = 0.f;
  for (int p0 = 0; p0 < np; p0 += KP) {
    float2 ml[KP];
    float src[KP][EPL];
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const int p = min(p0 + k, np - 1);  // past the last: re-read it, weight 0 below
      const int64_t wi = (slot0 + p) * H_q + h0 + h;
      ml[k] = load_agent(a.ws_ml + wi * 2);
      const float* s = a.ws_o + wi * D;
      if constexpr (EPL % 2 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 2) {
          const float2 v = load_agent(s + partial_pos(a.vec_lpt, e0 + e));
          src[k][e] = v.x;
          src[k][e + 1] = v.y;
        }
      } else {
        src[k][0] = __hip_atomic_load(s + partial_pos(a.vec_lpt, e0), __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    float Mc = M;
#pragma unroll
    for (int k = 0; k < KP; ++k)
      if (p0 + k < np) Mc = fmaxf(Mc, ml[k].x);
    const float r = (M == -INFINITY) ? 0.f : exp2f(M - Mc);  // rescale what came before
    Lsum *= r;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] *= r;
#pragma unroll
    for (int k = 0; k < KP; ++k) {
      const float w = (p0 + k >= np || ml[k].x == -INFINITY) ? 0.f : exp2f(ml[k].x - Mc);
      Lsum = fmaf(ml[k].y, w, Lsum);
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[e] = fmaf(src[k][e], w, o[e]);
    }
    M = Mc;
  }
  const float inv = 1.f / Lsum;
  uint16_t* dst = a.out + ((int64_t)b * H_q + h0 + h) * D + e0;
  if constexpr (EPL == 1) {
    dst[0] = (uint16_t)f32_to_bf16_rne(o[0] * inv);
  } else if constexpr (EPL == 2) {
    *reinterpret_cast<uint32_t*>(dst) = pack_bf16x2(o[0] * inv, o[1] * inv);
  } else if constexpr (EPL == 4) {
    *reinterpret_cast<uint2*>(dst) =
        make_uint2(pack_bf16x2(o[0] * inv, o[1] * inv), pack_bf16x2(o[2] * inv, o[3] * inv));
  } else {
#pragma unroll
    for (int e = 0; e < EPL; e += 8) {
      uint4 v;
      v.x = pack_bf16x2(o[e] * inv, o[e + 1] * inv);
      v.y = pack_bf16x2(o[e + 2] * inv, o[e + 3] * inv);
      v.z = pack_bf16x2(o[e + 4] * inv, o[e + 5] * inv);
      v.w = pack_bf16x2(o[e + 6] * inv, o[e + 7] * inv);
      *reinterpret_cast<uint4*>(dst + e) = v;
    }
  }
}

// ---- partitioned grid (explicit partition length, or batches too large
// for the arrival counters): one work item per (sequence, kv-head group,
// partition), in the order of decode_order_kernel, merged by
// decode_reduce_kernel. Partial row of (sequence b, partition p):
// b * max_parts + p.
template <int D, int G, int KPW, bool FUSED, bool SMALL, bool DRAIN, int VS = 1, bool MF = false>
__global__ __launch_bounds__(kWave * VS) __attribute__((amdgpu_waves_per_eu(kSplitWavesPerSimd)))
void decode_split_kernel(DecodeArgs a, int /*unused: the stream kernel's signature*/) {
  constexpr bool kPair = MF && VS > 1;
  const int n_groups = a.num_kv_heads / (kPair ? VS : KPW);
  int b, part, P = a.part_tokens;  // P: tokens per partition
  if (a.order) {
    // items longest first (decode_order_kernel)
    const int v = a.order[blockIdx.x / n_groups];
    if (v < 0) return;
    b = __builtin_amdgcn_readfirstlane(v & 4095);
    part = __builtin_amdgcn_readfirstlane((v >> 12) & 4095);
    P = part_tokens(a);  // the length the order kernel chose
  } else {
    // highest partition first
    const int idx = blockIdx.x / n_groups;
    b = idx % a.num_seqs;
    part = a.max_parts - 1 - idx / a.num_seqs;
  }
  const int n = clamp_len(seq_len(a, b), a.max_blocks, a.block_size);
  const Parts parts = split_parts(n, P, a.max_parts);
  if (n == 0 ? part != 0 : part >= parts.k) return;
  char* lds = nullptr;
  if constexpr (MF) {
    __shared__ __attribute__((aligned(16))) char mf_lds[VS * mf_bytes(D)];
    lds = mf_lds + (VS == 1 ? 0 : threadIdx.x / kWave) * mf_bytes(D);
  }
  const int start = part * P;
  decode_piece<D, G, KPW, FUSED, SMALL, DRAIN, VS, MF>(
      a, lds, threadIdx.x, b, n, start, min(parts.n, start + P), parts.k <= 1,
      (int64_t)b * a.max_parts + part);
}

// Merge of the partitioned grid's partials: one wave per (sequence, q-head)
// (4 waves per workgroup measured no faster than 1).
template <int D>
__global__ __launch_bounds__(kWave) void decode_reduce_kernel(DecodeArgs a, int H_q) {
  const int h = blockIdx.x % H_q;
  const int b = blockIdx.x / H_q;
  const int n = clamp_len(seq_len(a, b), a.max_blocks, a.block_size);
  const int nparts = split_parts(n, part_tokens(a), a.max_parts).k;
  if (nparts <= 1) return;
  merge_pieces<D, 1>(a, H_q, b, h, 1, (int64_t)b * a.max_parts, nparts);
}

// ---- stream grid (the default): one launch, no dispatch order, no merge
// kernel.
//
// Every sequence is cut into units of CHUNK tokens (max(1, ceil(n/CHUNK))
// units; an empty sequence has one, which writes its zeros). For each
// kv-head group, the units of all sequences, in batch order, are cut into W
// contiguous grabs of equal size, one wave (workgroup) each, all resident
// at once (one wave per SIMD), so every wave streams the same number of
// bytes whatever the length mix: one long context among short ones is
// spread over as many waves as its share of the bytes.
// A grab covers the end of one sequence, whole sequences, and the start of
// another; a sequence inside one grab is finished there, the others leave a
// partial per grab (row j + b for grab j and sequence b: unique, since
// grabs are consecutive intervals and consecutive sequences share at most
// one grab), and the wave that completes a sequence's last piece merges
// them. Completion is counted per (sequence, kv-head) in the workspace's
// header: each wave publishes its partial (agent-scope stores, waited for)
// and then increments the counter; the wave whose increment completes the
// count reads the partials (agent-scope loads), merges, and sets the
// counter back to zero, so every call leaves the header zero (the caller
// zeroes it once).
// What bounds it: the waves of one launch finish up to 15-25% apart, by
// their own timestamps (the HBM fabric serves waves unevenly: XCD means
// differ by ~8%, and CUs within an XCD more), and the launch ends with the
// slowest. Balancing by a queue of small grabs taken with atomics, or by
// oversubscribing the grid with smaller grabs in later levels, both
// measured slower: each extra grab costs a chain of dependent round trips
// (queue, lengths, table, K/V, counter) under a loaded memory system.
// Resident waves of the split kernels on an MI355X: 256 CUs x 8 waves. A
// fixed constant (not a device query) so the workspace size is a pure
// function of the arguments.
constexpr int64_t kComputeUnits = 256;
constexpr int64_t kResidentItems = kComputeUnits * 8;
// Waves of the stream grid: one per SIMD (2 per SIMD measured 4% slower at
// the Qwen3-0.6B batch and 9% at 32 x 16,384 tokens).
constexpr int kStreamWaves = 1024;
constexpr int kMinPieceTokens = 256;  // shortest grab when the batch is small (128: the
// 1 x 8,192 + 255 x 100 batch 5% slower; 512: 40% slower)
// Grabs of fewer units than this keep two chunks of loads in flight (a
// short grab is latency-bound); longer ones wait for each chunk's loads
// before issuing the next (see drain_loads).
constexpr int kDrainUnits = 16;
// fixed cost of a piece, in units (0: the Qwen3-0.6B batch 2% slower, the
// Qwen3-8B batch 1%; 4 and 8 no better)
constexpr int kPieceCost = 2;

// The grabs of one kv-head group: units [lo(j), lo(j + 1)) for grab j < W.
struct Sched {
  int C;  // units in all
  int W;  // grabs (waves in use), at most C
  __device__ __forceinline__ int lo(int j) const { return (int)((int64_t)j * C / W); }
  // the grab holding unit x (< C)
  __device__ __forceinline__ int grab_of(int x) const {
    return (int)(((int64_t)(x + 1) * W - 1) / C);
  }
};

template <int CHUNK>
__device__ __forceinline__ int seq_units(const DecodeArgs& a, int s) {
  const int n = min(clamp_len(seq_len(a, s), a.max_blocks, a.block_size), a.max_ctx);
  return n <= 0 ? 1 : (n + CHUNK - 1) / CHUNK;
}

__device__ __forceinline__ int wave_sum(int x) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) x += __shfl_xor(x, off, kWave);
  return x;
}

__device__ __forceinline__ int wave_inclusive_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off, kWave);
    if (lane >= off) x += y;
  }
  return x;
}

template <int CHUNK>
__device__ __forceinline__ int units_of(int n) {
  return n <= 0 ? 1 : (n + CHUNK - 1) / CHUNK;
}

// The cost of a sequence in the split: its units plus kPieceCost, the
// fixed cost of starting a piece (its length, q and table reads and the
// first loads, in units of streaming time), placed before its first unit.
// Grabs of equal unit counts took up to 40% apart at the Qwen3-0.6B batch,
// in the same order on every run: grabs holding more sequence starts were
// the slow ones.
template <int CHUNK>
__device__ __forceinline__ int cost_of(int n) {
  return units_of<CHUNK>(n) + kPieceCost;
}

// Where grab j starts: the batch's schedule, the sequence b holding unit lo
// (its first unit S and length n). Every length is read once (4 x 64 per
// round, a wave-wide sum); the first 256 stay in registers for the search
// (a wave-wide scan, then the first lane past lo), so a batch of up to 256
// sequences costs one round trip. Wave-uniform: kept in scalar registers.
struct GrabStart {
  int b, S, n;
};

template <int CHUNK>
__device__ __forceinline__ Sched stream_locate(const DecodeArgs& a, int slots, int j,
                                               GrabStart& at) {
  constexpr int KB = 4;
  const int lane = threadIdx.x % kWave;
  const int ns = a.num_seqs;
  int keep[KB];  // lengths of sequences 64k + lane
  int C = 0;
  for (int base = 0; base < ns; base += KB * kWave) {
    int n[KB], u = 0;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int s = base + k * kWave + lane;
      n[k] = s < ns ? min(clamp_len(seq_len(a, s), a.max_blocks, a.block_size), a.max_ctx) : -1;
      u += n[k] < 0 ? 0 : cost_of<CHUNK>(n[k]);
    }
    if (base == 0) {
#pragma unroll
      for (int k = 0; k < KB; ++k) keep[k] = n[k];
    }
    C += wave_sum(u);
  }
  Sched sc;
  sc.C = __builtin_amdgcn_readfirstlane(C);
  sc.W = max(1, min(slots, sc.C / max(1, kMinPieceTokens / CHUNK)));
  at.b = ns;
  at.S = 0;
  at.n = 0;
  if (j >= sc.W) return sc;
  const int x = sc.lo(j);
  int S = 0;
  for (int base = 0; base < ns; base += kWave) {
    int n;
    if (base < KB * kWave) {
      const int k = base / kWave;
      n = k == 0 ? keep[0] : k == 1 ? keep[1] : k == 2 ? keep[2] : keep[3];
    } else {
      const int s = base + lane;
      n = s < ns ? min(clamp_len(seq_len(a, s), a.max_blocks, a.block_size), a.max_ctx) : -1;
    }
    const int u = n < 0 ? 0 : cost_of<CHUNK>(n);
    const int incl = wave_inclusive_scan(u, lane);
    const uint64_t past = __ballot(S + incl > x);
    if (past) {
      const int l = __ffsll((long long)past) - 1;
      at.b = __builtin_amdgcn_readfirstlane(base + l);
      at.S = __builtin_amdgcn_readfirstlane(S + __shfl(incl - u, l, kWave));
      at.n = __builtin_amdgcn_readfirstlane(__shfl(n, l, kWave));
      return sc;
    }
    S = __builtin_amdgcn_readfirstlane(S + __shfl(incl, kWave - 1, kWave));
  }
  return sc;  // not reached: lo < C
}

template <int D, int G, int KPW, bool FUSED, bool SMALL, bool DRAIN, int VS = 1, bool MF = false>
__global__ __launch_bounds__(kWave * VS) __attribute__((amdgpu_waves_per_eu(kSplitWavesPerSimd)))
void decode_stream_kernel(DecodeArgs a, int slots) {
  constexpr bool kPair = MF && VS > 1;
  using L = Lanes<D, KPW>;
  constexpr int CHUNK = L::TPI * (MF ? D / 16 : kVecUnroll);
  // q-heads merged per wave, rounded up to a power of two
  constexpr int HW = MF ? 16 : KPW * G;
  constexpr int HP = (MF && G > 0 && G <= 8) ? 8 : HW;
  const int Gn = G ? G : a.group;
  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * Gn;
  const int n_groups = H_kv / (kPair ? VS : KPW);
  const int gw = blockIdx.x % n_groups;
  const int j = blockIdx.x / n_groups;  // this workgroup's grab
  const int half = VS == 1 ? 0 : threadIdx.x / kWave;
  // this wave's first kv-head and its q-heads
  const int g0 = kPair ? gw * VS + half : gw * KPW * VS + half;
  const int h0 = g0 * Gn;
  const int nh = MF ? Gn : KPW * G;
  char* lds_base = nullptr;
  if constexpr (MF) {
    __shared__ __attribute__((aligned(16))) char mf_lds[VS * mf_bytes(D)];
    lds_base = mf_lds;
  }

  GrabStart at;
  const Sched sc = stream_locate<CHUNK>(a, slots, j, at);
  if (j >= sc.W) return;  // a small batch leaves some workgroups idle
  const int lo = sc.lo(j), hi = sc.lo(j + 1);
  const int lane = threadIdx.x % kWave;
  const bool drain_on = sc.C / sc.W >= kDrainUnits;
  // the sequence holding cost position u, where its cost starts, and its
  // length; its units are cost positions [S + kPieceCost, S + kPieceCost + c)
  int b = at.b, S = at.S, n_next = at.n;
  const int b0 = b, S0 = S;
  // Only a grab's first and last pieces can be part of a longer sequence,
  // so a grab completes at most two sequences (bit 0: its first sequence's,
  // bit 1: its last piece's); they are merged after it, so the merge's
  // registers stay out of the streaming loop.
  int complete = 0;
  int bl = b, Sl = S;  // the last piece's sequence and where its cost starts
  for (int u = lo; u < hi && b < a.num_seqs; ++b) {
    const int n = n_next;
    const int c = units_of<CHUNK>(n);
    const int f = S + kPieceCost;  // cost position of its first unit
    const int u1 = min(hi, f + c);
    // the next piece's length, read now so that it has arrived when needed
    if (u1 < hi && b + 1 < a.num_seqs)
      n_next = min(clamp_len(seq_len(a, b + 1), a.max_blocks, a.block_size), a.max_ctx);
    const int p0 = max(u, f);  // this grab's units of the sequence: [p0, u1)
    if (p0 < u1) {
      const int first = sc.grab_of(f), last = sc.grab_of(f + c - 1);
      const bool direct = first == last;
      // the thread id, opaque to the compiler in each piece: what
      // decode_piece derives from it (lane roles, load and LDS offsets) is
      // computed in the piece, not hoisted out of this loop where it would
      // hold registers across every piece's streaming loop
      int tid = threadIdx.x;
      asm volatile("" : "+v"(tid));
      char* lds = MF ? lds_base + (VS == 1 ? 0 : tid / kWave) * mf_bytes(D) : nullptr;
      decode_piece<D, G, KPW, FUSED, SMALL, DRAIN, VS, MF>(
          a, lds, tid, b, n, (p0 - f) * CHUNK, min((u1 - f) * CHUNK, n), direct,
          (int64_t)j + b, drain_on);
      if (!direct) {
        // publish the partial (its agent-scope stores complete), then count it
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        int before = 0;
        if (lane == 0)
          before = __hip_atomic_fetch_add(a.counters + (int64_t)b * H_kv + g0, 1,
                                          __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (__builtin_amdgcn_readfirstlane(before) == last - first)  // every other piece is in
          complete |= b == b0 ? 1 : 2;
      }
      bl = b;
      Sl = S;
    }
    u = u1;
    S = f + c;
  }
  for (int k = 0; k < 2; ++k) {
    if (!(complete & (1 << k))) continue;
    const int mb = k ? bl : b0;
    const int mf = (k ? Sl : S0) + kPieceCost;
    const int first = sc.grab_of(mf), last = sc.grab_of(mf + seq_units<CHUNK>(a, mb) - 1);
    merge_pieces<D, HP>(a, H_q, mb, h0, nh, (int64_t)first + mb, last - first + 1);
    if (lane == 0)
      __hip_atomic_store(a.counters + (int64_t)mb * H_kv + g0, 0, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

using SplitFn = void (*)(DecodeArgs, int);

// ST: the stream grid's kernel, else the partitioned grid's.
template <bool ST, int D, int G, int KPW, bool FUSED, bool SMALL, bool DRAIN, int VS = 1,
          bool MF = false>
SplitFn kernel_of() {
  if constexpr (ST) return decode_stream_kernel<D, G, KPW, FUSED, SMALL, DRAIN, VS, MF>;
  else return decode_split_kernel<D, G, KPW, FUSED, SMALL, DRAIN, VS, MF>;
}

// DRAIN is built only where it changes the code: chunks of 8 loads (G < 8)
// inside one block.
template <bool ST, int D, int KPW, bool FUSED, bool SMALL, bool DRAIN>
SplitFn pick_split(int G) {
  constexpr bool kD = DRAIN && !SMALL;
  switch (G) {
    case 1: return kernel_of<ST, D, 1, KPW, FUSED, SMALL, kD>();
    case 2: return kernel_of<ST, D, 2, KPW, FUSED, SMALL, kD>();
    case 4: return kernel_of<ST, D, 4, KPW, FUSED, SMALL, kD>();
  }
  return nullptr;
}

// The matrix-core variant (one kv-head per wave, VS waves per workgroup):
// group sizes 8 and 16 built as such, the others (up to 16) take G from the
// arguments.
template <bool ST, int D, bool FUSED, bool SMALL, bool DRAIN, int VS>
SplitFn pick_split_mf(int G) {
  constexpr bool kD = DRAIN && !SMALL;
  switch (G) {
    case 8: return kernel_of<ST, D, 8, 1, FUSED, SMALL, kD, VS, true>();
    case 16: return kernel_of<ST, D, 16, 1, FUSED, SMALL, kD, VS, true>();
  }
  return G >= 1 && G <= 16 ? kernel_of<ST, D, 0, 1, FUSED, SMALL, kD, VS, true>() : nullptr;
}

template <bool ST, int D, bool FUSED, int VS>
SplitFn pick_split_mf(int G, bool small, bool drain) {
  if (small) return pick_split_mf<ST, D, FUSED, true, false, VS>(G);
  return drain ? pick_split_mf<ST, D, FUSED, false, true, VS>(G)
               : pick_split_mf<ST, D, FUSED, false, false, VS>(G);
}

template <bool ST, int D, bool FUSED>
SplitFn pick_split_mf(int G, bool small, bool drain, int waves) {
  switch (waves) {
    case 1: return pick_split_mf<ST, D, FUSED, 1>(G, small, drain);
    case 2: return pick_split_mf<ST, D, FUSED, 2>(G, small, drain);
  }
  return nullptr;
}

template <bool ST, int D, int KPW, bool FUSED>
SplitFn pick_split(int G, bool small, bool drain) {
  if (small) return pick_split<ST, D, KPW, FUSED, true, false>(G);
  return drain ? pick_split<ST, D, KPW, FUSED, false, true>(G)
               : pick_split<ST, D, KPW, FUSED, false, false>(G);
}

template <bool ST, int D, int KPW>
SplitFn pick_split(int G, bool fused, bool small, bool drain) {
  return fused ? pick_split<ST, D, KPW, true>(G, small, drain)
               : pick_split<ST, D, KPW, false>(G, small, drain);
}

constexpr int kSegmentBytes = 512;

// kv-heads per wave: as many adjacent heads as make a kSegmentBytes-byte
// contiguous piece of each token row (on MI355X 512-byte pieces stream about
// 7% faster than 256-byte ones), when the head count allows it; else one.
// The matrix-core variant takes one kv-head per wave.
// Group sizes from 8 up, and those that are not powers of two, run on the
// matrix cores (at both head dims); 1, 2 and 4 on the vector path.
bool mf_group(int /*head_dim*/, int G) { return G >= 8 || (G & (G - 1)) != 0; }
bool use_mf(const pa_desc* d) { return mf_group(d->head_dim, d->num_q_heads / d->num_kv_heads); }
// Matrix-core items: two adjacent kv-heads (one when the head count is odd),
// one wave each, in one workgroup.
int mf_waves(const pa_desc* d) {
  if (!use_mf(d)) return 0;
  int w = 2;
  while (w > 1 && d->num_kv_heads % w) w >>= 1;
  return w;
}
// Waves per split-kernel workgroup.
int kv_split(const pa_desc* d) { return use_mf(d) ? mf_waves(d) : 1; }

// Work-item groups per sequence: kv-heads over kv-heads per wave.
int item_groups(const pa_desc* d);

int kv_heads_per_wave(int head_dim, int num_q_heads, int num_kv_heads) {
  if (mf_group(head_dim, num_q_heads / num_kv_heads)) return 1;
  const int want = kSegmentBytes / (2 * head_dim);
  return (want > 1 && num_kv_heads % want == 0) ? want : 1;
}

int item_groups(const pa_desc* d) {
  if (use_mf(d)) return d->num_kv_heads / mf_waves(d);
  return d->num_kv_heads / kv_heads_per_wave(d->head_dim, d->num_q_heads, d->num_kv_heads);
}



// Longest partition (16, 8, 4, 2 or 1 units of 256 tokens) whose wave count
// still fills the chip, estimating the mean context as max_context_len / 2
// (the order kernel, when it runs, applies the same rule to the true mean
// and may lengthen the partitions). Long partitions amortise each item's
// set-up and keep its loads streaming (fewer concurrent streams also read
// HBM more efficiently); short ones keep small batches spread over the whole
// chip.
// The heuristic's inputs: longest partition tried (16 units for multi-head
// waves and the matrix-core variant, else 8), waves per sequence and
// partition (a matrix-core item is one wave per kv-head), and the waves that
// count as filling the chip (matrix-core items of two waves keep long
// partitions down to a quarter of the slots: 64 q / 8 kv heads at batch 64,
// 186 us with 4,096 tokens, 195 us with 2,048).
PartRule part_rule(const pa_desc* d) {
  const int kpw = kv_heads_per_wave(d->head_dim, d->num_q_heads, d->num_kv_heads);
  const bool mf = use_mf(d);
  PartRule r;
  r.auto_units = (kpw > 1 || mf) ? 16 : 8;
  r.min_units = 1;
  r.waves = mf ? d->num_kv_heads : item_groups(d);
  r.fill = (int)(mf && mf_waves(d) > 1 ? kResidentItems / 4 : kResidentItems / 2);
  return r;
}

int default_partition_blocks(const pa_desc* d, int32_t num_seqs, int32_t max_ctx) {
  const int64_t mean_ctx = max(1, max_ctx / 2);
  const PartRule r = part_rule(d);
  for (int p = r.auto_units; p > 1; p >>= 1) {
    const int64_t per_seq = (mean_ctx + (int64_t)p * kPartUnit - 1) / ((int64_t)p * kPartUnit);
    if ((int64_t)num_seqs * r.waves * per_seq >= r.fill) return p;
  }
  return 1;
}

// Workspace: the partitions' (o[d], m, l) fp32 partials when a sequence can
// span more than one partition, then the dispatch order (one int32 per
// sequence and partition, 16-byte rounded) and the partition length the
// order kernel chose (16 bytes) when the grid has more items than CUs. The order
// matters even when every item is resident at once: a CU's share of HBM
// bandwidth is bounded, and longest first deals the long items out across
// the CUs instead of stacking some on a few.
// The dispatch order is computed when the grid has more items than CUs and
// an order entry can hold a sequence id and a partition index (12 bits each).
bool ordered_grid(const pa_desc* d, int32_t num_seqs, int max_parts) {
  return num_seqs <= kOrderMaxSeqs && max_parts <= 4096 &&
         (int64_t)num_seqs * max_parts * item_groups(d) > kComputeUnits;
}

// Workspace layout, the same for every plan, so that one workspace serves
// calls of any shape in turn: a fixed header of kMaxCounters words (the
// stream grid's arrival counters, one per (sequence, kv-head); zero before
// the first call, and every call leaves it zero), then the partials (o[d]
// fp32, then (m, l) pairs), then, for the partitioned grid, the dispatch
// order and the chosen partition length.
constexpr int kMaxCounters = 1 << 16;  // (sequence, kv-head) pairs of a stream-grid call
constexpr size_t kHeaderBytes = (size_t)kMaxCounters * sizeof(int32_t);

// Tokens per chunk of the split kernels.
int chunk_tokens(const pa_desc* d) {
  if (use_mf(d)) return 32;
  const int kpw = kv_heads_per_wave(d->head_dim, d->num_q_heads, d->num_kv_heads);
  return (kWave / (d->head_dim / 8 * kpw)) * kVecUnroll;
}

// Grabs per kv-head group of the stream grid: its waves over the waves of
// one grab (a matrix-core grab is a workgroup of VS waves).
int stream_ranges(const pa_desc* d) {
  return (int)max((int64_t)1, (int64_t)kStreamWaves / ((int64_t)item_groups(d) * kv_split(d)));
}

struct Plan {
  bool stream;  // the stream grid (else the partitioned one)
  int ranges;   // stream grid: ranges per kv-head group
  int part_tokens;
  int min_units;  // shortest partition the order kernel may choose, in 256 tokens
  int max_parts;
  bool ordered;
  bool auto_part;  // the partition length is the library's to choose
  size_t partial_rows;  // partial rows (one per q-head each)
  size_t partial_bytes;
  size_t order_bytes;  // ranks, 16-byte rounded
  size_t ws_bytes;
};

Plan make_plan(const pa_desc* d, int32_t num_seqs, int32_t max_ctx, int32_t part_blocks) {
  Plan p;
  p.auto_part = part_blocks <= 0;
  // The stream grid needs a counter per (sequence, kv-head) and a unit count
  // of the batch that fits an int.
  const int64_t units = ((int64_t)max(1, max_ctx) + chunk_tokens(d) - 1) / chunk_tokens(d) +
                        kPieceCost;
  p.stream = p.auto_part && (int64_t)num_seqs * d->num_kv_heads <= kMaxCounters &&
             (int64_t)num_seqs * units < ((int64_t)1 << 30);
  if (p.stream) {
    p.ranges = stream_ranges(d);
    p.part_tokens = 0;
    p.min_units = 0;
    p.max_parts = 0;
    p.ordered = false;
    // row j + b for grab j < W
    p.partial_rows = (size_t)p.ranges + max(1, num_seqs) - 1;
    p.partial_bytes = p.partial_rows * d->num_q_heads * (size_t)(d->head_dim + 2) * sizeof(float);
    p.order_bytes = 0;
    p.ws_bytes = kHeaderBytes + p.partial_bytes;
    return p;
  }
  p.ranges = 0;
  if (part_blocks <= 0) part_blocks = default_partition_blocks(d, num_seqs, max_ctx);
  // A partition at least as long as the longest context holds every
  // sequence whole, whatever its length: longer requests are cut to that.
  const int64_t whole = max((int64_t)1, min(((int64_t)max_ctx + kPartUnit - 1) / kPartUnit,
                                            (int64_t)kMaxPartUnits));
  part_blocks = (int)min((int64_t)part_blocks, whole);
  p.part_tokens = part_blocks * kPartUnit;
  p.min_units = part_blocks;
  p.max_parts = max(1, (max_ctx + p.part_tokens - 1) / p.part_tokens);
  if (p.auto_part && ordered_grid(d, num_seqs, p.max_parts)) {
    // the order kernel may cut down to a quarter of the estimate: room for
    // that many partitions (a grid 4x the items it fills measured no slower;
    // 16x cost 1.6% at the Qwen3-8B batch)
    const int units4 = max(1, part_blocks / 4);
    const int parts = max(1, (max_ctx + units4 * kPartUnit - 1) / (units4 * kPartUnit));
    if (ordered_grid(d, num_seqs, parts)) {
      p.min_units = units4;
      p.max_parts = parts;
    }
  }
  p.partial_rows = p.max_parts <= 1 ? 0 : (size_t)num_seqs * p.max_parts;  // row b * max_parts + p
  p.partial_bytes = p.partial_rows * d->num_q_heads * (size_t)(d->head_dim + 2) * sizeof(float);
  const int64_t ranks = (int64_t)num_seqs * p.max_parts;
  p.ordered = ordered_grid(d, num_seqs, p.max_parts);
  p.order_bytes = p.ordered ? (size_t)((ranks * 4 + 15) & ~15) : 0;
  // then the partition length the order kernel chose (16 bytes)
  const size_t body = p.partial_bytes + p.order_bytes + (p.ordered ? 16 : 0);
  p.ws_bytes = body ? kHeaderBytes + body : 0;
  return p;
}

// Workspace in a library-owned device array, for callers that cannot
// allocate (pa_decode_noalloc). Each GPU the library runs on holds its own
// copy of the array until the process ends; every call on that GPU shares
// it, so calls that overlap on one GPU race. The array starts as zeros
// (static storage), which is the state the counter header needs; every
// call leaves the header zero, and writes every other byte it later reads.
constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;  // per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of this device's `scratch` (its host-side name is only a
// stand-in and is never passed to a kernel), looked up once per device with
// that device current.
int scratch_address(const char* who, void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: hipGetDevice: %s", who, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(PA_ERR_UNSUPPORTED, "%s: device %d beyond %d", who, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", who,
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

int launch_decode(const char* who, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                  const int32_t* context_lens, const int32_t* cu_k, int32_t num_seqs,
                  int32_t max_context_len,
                  float scale, void* out, void* workspace, size_t workspace_bytes,
                  int32_t partition_blocks, const pa_desc* desc, void* stream,
                  const NewTokens* nt, bool use_scratch) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (num_seqs < 0 || max_context_len < 0 || max_blocks_per_seq < 0 || partition_blocks < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", who);
  if (max_context_len > kMaxContext)
    return fail(PA_ERR_INVALID_ARG, "%s: max_context_len %d above %d", who, max_context_len,
                kMaxContext);
  // the kernels take the maximum of the raw scores and scale it afterwards,
  // which equals the maximum of the scaled scores only for a positive scale
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale %g must be positive and finite", who,
                (double)scale);
  if (num_seqs == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !(context_lens || cu_k) || !out)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if ((int64_t)max_blocks_per_seq * desc->block_size < max_context_len)
    return fail(PA_ERR_INVALID_ARG, "%s: max_context_len %d exceeds %d table entries", who,
                max_context_len, max_blocks_per_seq);
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15u)
    return fail(PA_ERR_INVALID_ARG, "%s: q, caches and out must be 16-byte aligned", who);
  const int G = desc->num_q_heads / desc->num_kv_heads;
  const int D = desc->head_dim;
  const int row = desc->num_kv_heads * D;
  if (nt) {
    if (!nt->k || !nt->v || !nt->slot_mapping)
      return fail(PA_ERR_INVALID_ARG, "%s: NULL new-token pointer", who);
    if (nt->k_stride < row || nt->v_stride < row || (nt->k_stride % 8) || (nt->v_stride % 8) ||
        (((uintptr_t)nt->k | (uintptr_t)nt->v) & 15u))
      return fail(PA_ERR_INVALID_ARG,
                  "%s: k_new/v_new need 16-byte aligned rows with stride >= H_kv*d", who);
  }
  const Plan plan = make_plan(desc, num_seqs, max_context_len, partition_blocks);
  if (use_scratch) {  // the library's array replaces the caller's workspace
    if (plan.ws_bytes > kScratchBytes)
      return fail(PA_ERR_WORKSPACE,
                  "%s: this batch needs %zu bytes of workspace; the library's scratch holds %zu "
                  "(use pa_decode with a caller-owned workspace)", who, plan.ws_bytes,
                  kScratchBytes);
    workspace = nullptr;
    workspace_bytes = 0;
    if (plan.ws_bytes) {
      rc = scratch_address(who, &workspace);
      if (rc) return rc;
      workspace_bytes = kScratchBytes;
    }
  }
  if (plan.ws_bytes) {
    if (!workspace || workspace_bytes < plan.ws_bytes)
      return fail(PA_ERR_WORKSPACE, "%s: workspace %zu bytes < %zu needed", who,
                  workspace ? workspace_bytes : (size_t)0, plan.ws_bytes);
    if ((uintptr_t)workspace & 15u)
      return fail(PA_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", who);
  }
  const int kpw = kv_heads_per_wave(desc->head_dim, desc->num_q_heads, desc->num_kv_heads);
  const int64_t items = plan.stream ? (int64_t)item_groups(desc) * plan.ranges
                                    : (int64_t)num_seqs * item_groups(desc) * plan.max_parts;
  if (items > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "%s: grid too large", who);
  if (debug_enabled()) {
    rc = debug_check_tables(who, block_tables, max_blocks_per_seq, context_lens, cu_k, num_seqs,
                            max_context_len, desc, (hipStream_t)stream);
    if (!rc && nt)
      rc = debug_check_slots(who, nt->slot_mapping, num_seqs,
                             desc->num_blocks * desc->block_size, (hipStream_t)stream);
    if (!rc && plan.stream)
      rc = debug_check_zero(who, workspace, kHeaderBytes, (hipStream_t)stream);
    if (rc) return rc;
  }

  DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.cu_k = cu_k;
  const size_t o_floats = plan.partial_rows * desc->num_q_heads * D;
  float* partials = plan.ws_bytes ? (float*)((char*)workspace + kHeaderBytes) : nullptr;
  a.ws_o = partials;
  a.ws_ml = partials ? partials + o_floats : nullptr;
  a.out = (uint16_t*)out;
  a.k_new = nt ? (const uint16_t*)nt->k : nullptr;
  a.v_new = nt ? (const uint16_t*)nt->v : nullptr;
  a.k_cache_w = nt ? (uint16_t*)k_cache : nullptr;
  a.v_cache_w = nt ? (uint16_t*)v_cache : nullptr;
  a.slot_mapping = nt ? nt->slot_mapping : nullptr;
  a.k_new_stride = nt ? nt->k_stride : 0;
  a.v_new_stride = nt ? nt->v_stride : 0;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_kv_heads = desc->num_kv_heads;
  a.part_tokens = plan.part_tokens;
  a.max_parts = plan.max_parts;
  a.block_size = desc->block_size;
  a.block_shift = log2_int(desc->block_size);
  a.scale_log2 = scale * kLog2e;
  char* after_partials = plan.ws_bytes ? (char*)workspace + kHeaderBytes + plan.partial_bytes
                                       : nullptr;
  a.order = plan.ordered ? (int32_t*)after_partials : nullptr;
  a.part_dev = plan.ordered ? (int32_t*)(after_partials + plan.order_bytes) : nullptr;
  a.group = G;
  a.max_ctx = max_context_len;
  a.vec_lpt = use_mf(desc) ? 0 : D / 8;
  a.counters = plan.stream ? (int32_t*)workspace : nullptr;

  hipStream_t s = (hipStream_t)stream;
  const bool mf = use_mf(desc);
  const int chunk = chunk_tokens(desc);
  const bool small = desc->block_size < chunk;
  const bool fused = nt != nullptr;
  // the wave slots are full (2 per SIMD): one chunk of loads in flight per
  // wave (the stream grid decides on the device, from the grab length)
  const bool drain = plan.stream || items >= kResidentItems;
  SplitFn split = nullptr;
  auto pick = [&](auto st) -> SplitFn {
    constexpr bool ST = decltype(st)::value;
    if (mf) {
      const int waves = mf_waves(desc);
      if (D == 128)
        return fused ? pick_split_mf<ST, 128, true>(G, small, drain, waves)
                     : pick_split_mf<ST, 128, false>(G, small, drain, waves);
      return fused ? pick_split_mf<ST, 64, true>(G, small, drain, waves)
                   : pick_split_mf<ST, 64, false>(G, small, drain, waves);
    }
    if (D == 128)
      return kpw == 2 ? pick_split<ST, 128, 2>(G, fused, small, drain)
                      : pick_split<ST, 128, 1>(G, fused, small, drain);
    return kpw == 4   ? pick_split<ST, 64, 4>(G, fused, small, drain)
           : kpw == 2 ? pick_split<ST, 64, 2>(G, fused, small, drain)
                      : pick_split<ST, 64, 1>(G, fused, small, drain);
  };
  split = plan.stream ? pick(std::true_type{}) : pick(std::false_type{});
  if (!split || (D == 128 && kpw > 2))
    return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for %d kv-heads per wave", who, kpw);
  if (plan.stream) {
    // the vector path's workgroups (one wave) ask for a quarter of the LDS
    // they do not use, so that four fit a CU: one wave per SIMD
    hipLaunchKernelGGL(split, dim3((unsigned)items), dim3(kWave * kv_split(desc)), 0, s, a,
                       plan.ranges);
    return launch_status(who);
  }
  if (plan.ordered) {
    const int round = (int)max((int64_t)1, kComputeUnits / item_groups(desc));
    PartRule rule = part_rule(desc);
    rule.min_units = plan.min_units;
    if (!plan.auto_part) rule.auto_units = 0;
    hipLaunchKernelGGL(decode_order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a,
                       num_seqs * plan.max_parts, round, rule);
    rc = launch_status(who);
    if (rc) return rc;
  }
  hipLaunchKernelGGL(split, dim3((unsigned)items), dim3(kWave * kv_split(desc)), 0, s, a, 0);
  rc = launch_status(who);
  if (rc) return rc;
  if (plan.max_parts > 1) {
    const unsigned wgs = (unsigned)num_seqs * desc->num_q_heads;
    if (D == 128)
      hipLaunchKernelGGL(decode_reduce_kernel<128>, dim3(wgs), dim3(kWave), 0, s, a,
                         desc->num_q_heads);
    else
      hipLaunchKernelGGL(decode_reduce_kernel<64>, dim3(wgs), dim3(kWave), 0, s, a,
                         desc->num_q_heads);
    rc = launch_status(who);
    if (rc) return rc;
  }
  return PA_OK;
}

size_t decode_workspace_bytes(const pa_desc* desc, int32_t num_seqs, int32_t max_context_len) {
  if (check_desc(desc) != PA_OK || num_seqs < 0 || max_context_len < 0) return 0;
  return make_plan(desc, num_seqs, max_context_len, 0).ws_bytes;
}

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
  return pa::launch_decode("pa_decode", q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                           context_lens, nullptr, num_seqs, max_context_len, scale, out, workspace,
                           workspace_bytes, partition_blocks, desc, stream, nullptr);
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

extern "C" int pa_decode_step(const void* q, const void* k_new, int64_t k_row_stride,
                              const void* v_new, int64_t v_row_stride, void* k_cache,
                              void* v_cache, const int32_t* slot_mapping,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t max_context_len, float scale, void* out, void* workspace,
                              size_t workspace_bytes, const pa_desc* desc, void* stream) {
  const pa::NewTokens nt{k_new, k_row_stride, v_new, v_row_stride, slot_mapping};
  return pa::launch_decode("pa_decode_step", q, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, nullptr, num_seqs, max_context_len,
                           scale,
                           out, workspace, workspace_bytes, 0, desc, stream, &nt);
}


extern "C" int pa_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t num_seqs,
                                 int32_t max_context_len, float scale, void* out,
                                 const pa_desc* desc, void* stream) {
  return pa::launch_decode("pa_decode_noalloc", q, k_cache, v_cache, block_tables,
                           max_blocks_per_seq, context_lens, nullptr, num_seqs, max_context_len,
                           scale, out, nullptr, 0, 0, desc, stream, nullptr, true);
}

// pa_prefill_varlen: causal varlen prefill over paged K/V, bf16 MFMA on gfx950.
//
// What is computed ("12. 推理加速(二): nano-vllm — 1200 行手写 vLLM", §12.6,
// prefill branch with prefix cache and the cu_seqlens notes): sequence b has
// q_len new tokens packed at rows cu_q[b].., and k_len keys read through its
// block table (cached prefix plus the new tokens, stored beforehand). Query i
// sits at position k_len - q_len + i and attends to keys 0 .. that position.
//
// How (MI355X design):
//   * Work item = workgroup of 8 waves for (sequence, kv-head, block of
//     256/G query positions). Its 16 MFMA column tiles (two per wave) are 16
//     positions x 1 q-head each, covering all G q-heads of the kv-head, so
//     every K/V tile staged in LDS serves the whole GQA group.
//   * Scores are computed transposed, S^T = K Q^T, with
//     v_mfma_f32_16x16x32_bf16: A = K rows from LDS, B = Q held in registers
//     for the whole loop. The accumulator layout of S^T (one query column per
//     lane, keys down the lane groups) is exactly the B-operand layout of the
//     next product O^T += V^T P^T once the 32 keys of a step are numbered in
//     the order the lanes hold them, so P never goes through LDS. V is staged
//     transposed (d-major) in LDS in that key order.
//   * Online softmax per query column: base-2 exponent with scale*log2(e)
//     folded in, running max exchanged across the 4 lane groups of a column,
//     P rounded to bf16 for the MFMA (the row sum adds the same rounded
//     weights), fp32 accumulation, bf16 output.
//   * Keys are staged 64 at a time (with blocks of 64 tokens or more a stage
//     never straddles a block, so one block-table lookup per stage),
//     double-buffered in LDS with register staging one stage ahead of LDS.
//   * Causal work skipping: stages past the work item's last query are never
//     loaded; a wave skips the stages that lie after all its queries; only
//     stages that cross the diagonal apply the mask.
//   * Grid order: per sequence the last position blocks (the most keys) come
//     first; consecutive workgroups differ in kv-head so one (sequence,
//     kv-head)'s blocks, which re-read the same K/V, land on the same XCD.
#include <cmath>

#include "common.hpp"

namespace pa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 8;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kNT = 2;     // 16-column tiles per wave
constexpr int kTiles = kNT * kWaves;      // 16-column tiles per workgroup
constexpr int kCols = 16 * kTiles;        // (position, q-head) columns per workgroup
// Lazy rescaling: a column's reference max moves only when a score exceeds
// it by more than 2^kLazyLog2 (weights stay <= 256, well inside bf16/fp32).
constexpr float kLazyLog2 = 8.f;
constexpr int kKT = 64;          // keys per LDS stage

struct PrefillArgs {
  const uint16_t* q;
  const uint16_t* k_cache;
  const uint16_t* v_cache;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* block_tables;
  uint16_t* out;
  int64_t num_blocks;
  int32_t max_blocks;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t max_rblocks;  // position blocks of the longest sequence
  int32_t block_size;   // tokens per physical block (power of two)
  int32_t block_shift;  // log2(block_size)
  int32_t group;        // q-heads per kv-head
  float scale_log2;
};

// Query positions per workgroup: its tiles cover floor(kTiles / G) blocks of
// 16 positions for all G q-heads (every tile when G divides kTiles).
__host__ __device__ constexpr int positions_per_workgroup(int G) { return 16 * (kTiles / G); }

template <int D>
struct Geo {
  static constexpr int KROW = D * 2 + 16;    // bytes per staged K row (padded)
  static constexpr int VROW = kKT * 2 + 16;  // bytes per staged V^T row (padded)
  static constexpr int KBYTES = kKT * KROW;
  static constexpr int VBYTES = D * VROW;
  static constexpr int STAGE = KBYTES + VBYTES;
  static constexpr int KCHUNKS = kKT * D / 8 / kThreads;  // 16-byte K loads per thread
  static constexpr int VGROUPS = kThreads / 32;           // d ranges per key pair
  static constexpr int VW = D / VGROUPS;                  // V elements per thread per key
  static_assert(KCHUNKS >= 1 && (VW == 4 || VW == 8 || VW == 16), "stage split");
};

template <int VW> struct VVec;
template <> struct VVec<4> { typedef __attribute__((ext_vector_type(2))) unsigned int T; };
template <> struct VVec<8> { typedef __attribute__((ext_vector_type(4))) unsigned int T; };
template <> struct VVec<16> { typedef __attribute__((ext_vector_type(8))) unsigned int T; };

// Position of key k (0..31) of a 32-key step in the order the MFMA lanes hold
// it: lane group j holds keys 4j..4j+3 (first 16-key tile) then 16+4j..16+4j+3.
__device__ __forceinline__ int key_slot(int k) {
  return ((k & 15) >> 2) * 8 + (k >> 4) * 4 + (k & 3);
}

// acc + lo + hi of a packed bf16 pair, summed in fp32 (v_dot2_f32_bf16 with
// the pair (1.0, 1.0)).
__device__ __forceinline__ float sum_pair_bf16(uint32_t pair, float acc) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pair),
                                         __builtin_bit_cast(bf16x2, 0x3F803F80u), acc, false);
}

// Two fp32 -> packed bf16 (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// Row offset (in elements) of key position p of a sequence in a cache. A
// broken table entry (precondition violated) reads block 0: the result is
// then meaningless, but the access stays inside the pool.
__device__ __forceinline__ int64_t key_row(const PrefillArgs& a, const int32_t* bt, int p,
                                           int64_t row_elems) {
  const int blk_raw = bt[p >> a.block_shift];
  const int64_t blk = (blk_raw >= 0 && blk_raw < a.num_blocks) ? blk_raw : 0;
  return ((blk << a.block_shift) + (p & (a.block_size - 1))) * row_elems;
}

// Register loads of stage `stage` (keys [64*stage, 64*stage + 64)). Keys at
// or past kmax are never visible; they re-read the last needed one. SMALL:
// blocks hold fewer keys than a stage, so every key looks up its own block;
// otherwise the whole stage lies in one block (one lookup).
template <int D, bool SMALL>
__device__ __forceinline__ void load_stage(const PrefillArgs& a, const int32_t* bt, int g, int kmax,
                                           int stage, u32x4 (&kreg)[Geo<D>::KCHUNKS],
                                           typename VVec<Geo<D>::VW>::T (&vreg)[2]) {
  using GG = Geo<D>;
  const int t = threadIdx.x;
  const int kbase = stage * kKT;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const uint16_t* kc = a.k_cache + (int64_t)g * D;
  const uint16_t* vc = a.v_cache + (int64_t)g * D;
  int64_t base = 0;
  if constexpr (!SMALL) base = key_row(a, bt, kbase, row_elems) - (int64_t)kbase * row_elems;
  // row offset of key position p (base + p rows when the stage is in one block)
  auto row_of = [&](int p) -> int64_t {
    if constexpr (SMALL) return key_row(a, bt, p, row_elems);
    else return base + (int64_t)p * row_elems;
  };
#pragma unroll
  for (int i = 0; i < GG::KCHUNKS; ++i) {
    const int c = t + i * kThreads;
    const int key = c / (D / 8);
    const int ch = c % (D / 8);
    const int kp = min(kbase + key, kmax - 1);
    kreg[i] = *reinterpret_cast<const u32x4*>(kc + row_of(kp) + ch * 8);
  }
  typedef typename VVec<GG::VW>::T VT;
  const int pair = t % 32;  // keys 2*pair, 2*pair+1 of the stage
  const int dg = t / 32;    // d range [dg*VW, dg*VW+VW)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int kp = min(kbase + 2 * pair + s, kmax - 1);
    vreg[s] = *reinterpret_cast<const VT*>(vc + row_of(kp) + dg * GG::VW);
  }
}

template <int D>
__device__ __forceinline__ void store_stage(char* lds, const u32x4 (&kreg)[Geo<D>::KCHUNKS],
                                            const typename VVec<Geo<D>::VW>::T (&vreg)[2]) {
  using GG = Geo<D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < GG::KCHUNKS; ++i) {
    const int c = t + i * kThreads;
    const int key = c / (D / 8);
    const int ch = c % (D / 8);
    *reinterpret_cast<u32x4*>(lds + key * GG::KROW + ch * 16) = kreg[i];
  }
  // V^T[d][slot]: a dword holds the pair (V[2p][d], V[2p+1][d]); an even key
  // and its odd neighbour occupy adjacent slots
  const int pair = t % 32;
  const int dg = t / 32;
  const int key0 = 2 * pair;
  const int slot = (key0 / 32) * 32 + key_slot(key0 % 32);
  char* vt = lds + GG::KBYTES + slot * 2;
#pragma unroll
  for (int w = 0; w < GG::VW / 2; ++w) {
    const int d = dg * GG::VW + 2 * w;
    // element d: low halves; element d+1: high halves
    const uint32_t e0 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
    const uint32_t e1 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
    *reinterpret_cast<uint32_t*>(vt + d * GG::VROW) = e0;
    *reinterpret_cast<uint32_t*>(vt + (d + 1) * GG::VROW) = e1;
  }
}

// G_ = 0: the group size is taken from the arguments (any G up to kTiles).
template <int D, int G_, bool SMALL>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillArgs a) {
  using GG = Geo<D>;
  const int G = G_ ? G_ : a.group;
  const int QB = positions_per_workgroup(G);  // query positions per workgroup
  const int used = (kTiles / G) * G;          // tiles with columns of their own
  constexpr int KSTEPS = D / 32;             // MFMA k-steps over head_dim
  constexpr int MT = D / 16;                 // 16-row tiles of O^T over head_dim
  __shared__ __attribute__((aligned(16))) char lds[2 * GG::STAGE];

  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * G;
  int idx = blockIdx.x;
  const int g = idx % H_kv;
  idx /= H_kv;
  // A sequence's position blocks are consecutive (last positions first) and
  // kv-head is fastest, so the blocks of one (sequence, kv-head), which read
  // the same K/V, run together on one XCD and share its L2.
  const int r = idx % a.max_rblocks;  // position block counted from the end
  const int b = idx / a.max_rblocks;

  const int q0 = a.cu_q[b];
  const int q_len = a.cu_q[b + 1] - q0;
  int k_len = a.cu_k[b + 1] - a.cu_k[b];
  k_len = (int)min((int64_t)k_len, (int64_t)a.max_blocks * a.block_size);
  if (q_len <= 0 || k_len < q_len) return;  // nothing to do / broken precondition
  const int p_end = q_len - r * QB;         // positions [p_end - QB, p_end)
  if (p_end <= 0) return;
  const int p0 = p_end - QB;
  const int off = k_len - q_len;  // query i is the token at position off + i
  const int kmax = off + p_end;   // keys this workgroup can see: [0, kmax)
  const int n_stages = (kmax + kKT - 1) / kKT;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  const int col = lane % 16;
  const int grp = lane / 16;

  int head[kNT], pbase[kNT];
  bool own[kNT];  // a spare tile (when G does not divide kTiles) repeats a used one, unwritten
  int wmax = -1;  // last position any column of this wave holds
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int T = wave * kNT + j;
    own[j] = T < used;
    const int Tu = own[j] ? T : T - used;
    head[j] = g * G + Tu % G;
    pbase[j] = p0 + (Tu / G) * 16;
    wmax = max(wmax, pbase[j] + 15);
  }
  wmax = min(wmax, p_end - 1);

  // Q^T operands for all k-steps (rows outside the sequence re-read row 0;
  // their columns are never written)
  bf16x8 qf[kNT][KSTEPS];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    const int pos = max(pbase[j] + col, 0);
    const uint16_t* qp = a.q + ((int64_t)(q0 + pos) * H_q + head[j]) * D + grp * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[j][ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 32));
  }

  f32x4 o[kNT][MT];
  float m[kNT], l[kNT];
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) o[j][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // S^T = K Q^T for the 64 keys of the stage held in `kst` x (kNT x 16) columns
  auto scores = [&](const char* kst, f32x4 (&sc)[kKT / 16][kNT]) {
#pragma unroll
    for (int kt = 0; kt < kKT / 16; ++kt) {
#pragma unroll
      for (int j = 0; j < kNT; ++j) sc[kt][j] = f32x4{0.f, 0.f, 0.f, 0.f};
      const char* arow = kst + (kt * 16 + col) * GG::KROW + grp * 16;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 av =
            __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(arow + ks * 64));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          sc[kt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qf[j][ks], sc[kt][j], 0, 0, 0);
      }
    }
  };
  // Online softmax of the stage's scores per column, then O^T += V^T P^T
  // with the stage's V^T held in `vst` (two 32-key products).
  auto softmax_pv = [&](int key0, const f32x4 (&sc)[kKT / 16][kNT], const char* vst) {
    // P^T operands for the two 32-key products (lane order of key_slot)
    bf16x8 pf[kNT][kKT / 32];
#pragma unroll
    for (int j = 0; j < kNT; ++j) {
      const int qpos = off + pbase[j] + col;  // absolute position of this column's query
      float sv[kKT / 4];
#pragma unroll
      for (int kt = 0; kt < kKT / 16; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[kt * 4 + i] = sc[kt][j][i];
      if (key0 + kKT - 1 > off + pbase[j]) {  // the stage crosses some column's diagonal
#pragma unroll
        for (int i = 0; i < kKT / 4; ++i) {
          const int kpos = key0 + (i >> 2) * 16 + grp * 4 + (i & 3);
          if (kpos > qpos) sv[i] = -INFINITY;
        }
      }
      float mx = sv[0];
#pragma unroll
      for (int i = 1; i < kKT / 4; ++i) mx = fmaxf(mx, sv[i]);
      mx = fmaxf(mx, xor_lane(mx, 16));
      mx = fmaxf(mx, xor_lane(mx, 32));
      mx *= a.scale_log2;
      // all lanes of a column see the same mx and m, so they agree on it
      if (mx > m[j] + kLazyLog2) {
        const float mnew = fmaxf(m[j], mx);
        const float alpha = __builtin_amdgcn_exp2f(m[j] - mnew);  // 0 on the first step
        m[j] = mnew;
        l[j] *= alpha;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) o[j][mt] *= alpha;
      }
      const float negm = (m[j] == -INFINITY) ? 0.f : -m[j];
#pragma unroll
      for (int h = 0; h < kKT / 32; ++h) {
        float p[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
          p[i] = __builtin_amdgcn_exp2f(fmaf(sv[h * 8 + i], a.scale_log2, negm));
        uint4 pk;
        pk.x = pack2_bf16(p[0], p[1]);
        pk.y = pack2_bf16(p[2], p[3]);
        pk.z = pack2_bf16(p[4], p[5]);
        pk.w = pack2_bf16(p[6], p[7]);
        // the sum adds the rounded weights the MFMA sees (an exact weighted
        // mean): a dot product of each packed pair with (1, 1)
        l[j] = sum_pair_bf16(pk.x, l[j]);
        l[j] = sum_pair_bf16(pk.y, l[j]);
        l[j] = sum_pair_bf16(pk.z, l[j]);
        l[j] = sum_pair_bf16(pk.w, l[j]);
        pf[j][h] = __builtin_bit_cast(bf16x8, pk);
      }
    }
#pragma unroll
    for (int h = 0; h < kKT / 32; ++h) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const char* vrow = vst + (mt * 16 + col) * GG::VROW + (h * 32 + grp * 8) * 2;
        const bf16x8 av = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(vrow));
#pragma unroll
        for (int j = 0; j < kNT; ++j)
          o[j][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pf[j][h], o[j][mt], 0, 0, 0);
      }
    }
  };

  // Register staging one stage ahead of LDS: at iteration st, stage st+1
  // (loaded during the previous iteration) is copied into the LDS buffer of
  // stage st-1, which every wave finished with before the last barrier, and
  // stage st+2 is issued into the same registers, so its loads land while
  // stage st is multiplied. Stage indices are clamped, so every issue is
  // unconditional and the memory counter waits stay static.
  u32x4 kr[GG::KCHUNKS];
  typename VVec<GG::VW>::T vr[2];
  load_stage<D, SMALL>(a, bt, g, kmax, 0, kr, vr);
  store_stage<D>(lds, kr, vr);
  load_stage<D, SMALL>(a, bt, g, kmax, min(1, n_stages - 1), kr, vr);
  __syncthreads();
  for (int st = 0; st < n_stages; ++st) {
    if (st + 1 < n_stages) store_stage<D>(lds + ((st + 1) & 1) * GG::STAGE, kr, vr);
    load_stage<D, SMALL>(a, bt, g, kmax, min(st + 2, n_stages - 1), kr, vr);
    const char* ks_lds = lds + (st & 1) * GG::STAGE;
    const int key0 = st * kKT;  // absolute position of the stage's first key
    if (key0 <= off + wmax) {   // else every key is after every query of the wave
      f32x4 s[kKT / 16][kNT];
      scores(ks_lds, s);
      softmax_pv(key0, s, ks_lds + GG::KBYTES);
    }
    __syncthreads();
  }

  // ---- epilogue: column sums across the 4 lane groups, normalise, store
#pragma unroll
  for (int j = 0; j < kNT; ++j) {
    float lt = l[j];
    lt += xor_lane(lt, 16);
    lt += xor_lane(lt, 32);
    const int pos = pbase[j] + col;
    if (!own[j] || pos < 0 || pos >= p_end) continue;
    const float inv = 1.f / lt;
    uint16_t* dst = a.out + ((int64_t)(q0 + pos) * H_q + head[j]) * D + grp * 4;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      uint2 v;
      v.x = pack_bf16x2(o[j][mt][0] * inv, o[j][mt][1] * inv);
      v.y = pack_bf16x2(o[j][mt][2] * inv, o[j][mt][3] * inv);
      *reinterpret_cast<uint2*>(dst + mt * 16) = v;
    }
  }
}

using PrefillFn = void (*)(PrefillArgs);

template <int D, bool SMALL>
PrefillFn pick(int G) {
  switch (G) {
    case 1: return prefill_kernel<D, 1, SMALL>;
    case 2: return prefill_kernel<D, 2, SMALL>;
    case 4: return prefill_kernel<D, 4, SMALL>;
    case 8: return prefill_kernel<D, 8, SMALL>;
    case 16: return prefill_kernel<D, 16, SMALL>;
  }
  return G >= 1 && G <= kTiles ? prefill_kernel<D, 0, SMALL> : nullptr;  // other group sizes
}

}  // namespace
}  // namespace pa

namespace pa {
namespace {

int launch_prefill(const char* who, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs,
                   int32_t max_seqlen_q, int32_t max_seqlen_k, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, float scale, void* out, const pa_desc* desc,
                   void* stream, bool debug_varlen) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (num_seqs < 0 || max_seqlen_q < 0 || max_seqlen_k < 0 || max_blocks_per_seq < 0)
    return fail(PA_ERR_INVALID_ARG, "%s: negative size", who);
  // the kernel takes the maximum of the raw scores and scales it afterwards,
  // which equals the maximum of the scaled scores only for a positive scale
  if (!(scale > 0.f) || !std::isfinite(scale))
    return fail(PA_ERR_INVALID_ARG, "%s: scale %g must be positive and finite", who,
                (double)scale);
  if (num_seqs == 0 || max_seqlen_q == 0) return PA_OK;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !cu_seqlens_k || !block_tables || !out)
    return fail(PA_ERR_INVALID_ARG, "%s: NULL pointer", who);
  if (max_seqlen_q > max_seqlen_k)
    return fail(PA_ERR_INVALID_ARG, "%s: max_seqlen_q %d > max_seqlen_k %d", who, max_seqlen_q,
                max_seqlen_k);
  if ((int64_t)max_blocks_per_seq * desc->block_size < max_seqlen_k)
    return fail(PA_ERR_INVALID_ARG, "%s: max_seqlen_k %d exceeds %d table entries", who,
                max_seqlen_k, max_blocks_per_seq);
  if (((uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)out) & 15u)
    return fail(PA_ERR_INVALID_ARG, "%s: q, caches and out must be 16-byte aligned", who);
  if (debug_enabled()) {
    // debug_varlen: the batch is the caller's whole cu_seqlens (else a mixed
    // batch's prefill rows, whose prefix sums were checked as a whole)
    if (debug_varlen)
      rc = debug_check_varlen(who, cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q,
                              max_seqlen_k, 0, (hipStream_t)stream);
    if (!rc)
      rc = debug_check_tables(who, block_tables, max_blocks_per_seq, nullptr, cu_seqlens_k,
                              num_seqs, max_seqlen_k, desc, (hipStream_t)stream);
    if (rc) return rc;
  }
  const int G = desc->num_q_heads / desc->num_kv_heads;
  const int D = desc->head_dim;
  const int QB = positions_per_workgroup(G);
  const int64_t rblocks = (max_seqlen_q + QB - 1) / QB;
  const int64_t blocks = (int64_t)num_seqs * desc->num_kv_heads * rblocks;
  if (blocks > INT32_MAX) return fail(PA_ERR_INVALID_ARG, "%s: grid too large", who);

  PrefillArgs a;
  a.q = (const uint16_t*)q;
  a.k_cache = (const uint16_t*)k_cache;
  a.v_cache = (const uint16_t*)v_cache;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.block_tables = block_tables;
  a.out = (uint16_t*)out;
  a.num_blocks = desc->num_blocks;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_kv_heads = desc->num_kv_heads;
  a.max_rblocks = (int32_t)rblocks;
  a.block_size = desc->block_size;
  a.block_shift = log2_int(desc->block_size);
  a.group = G;
  a.scale_log2 = scale * kLog2e;
  const bool small = desc->block_size < kKT;
  PrefillFn fn = D == 128 ? (small ? pick<128, true>(G) : pick<128, false>(G))
                          : (small ? pick<64, true>(G) : pick<64, false>(G));
  if (!fn) return fail(PA_ERR_UNSUPPORTED, "%s: no kernel for group size %d", who, G);
  hipLaunchKernelGGL(fn, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream, a);
  return launch_status(who);
}

}  // namespace
}  // namespace pa

extern "C" int pa_prefill_varlen(const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                 int32_t num_seqs, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 float scale, void* out, const pa_desc* desc, void* stream) {
  return pa::launch_prefill("pa_prefill_varlen", q, k_cache, v_cache, cu_seqlens_q,
                            cu_seqlens_k, num_seqs, max_seqlen_q, max_seqlen_k, block_tables,
                            max_blocks_per_seq, scale, out, desc, stream, true);
}

extern "C" size_t pa_mixed_workspace_size(const pa_desc* desc, int32_t num_decode_rows,
                                          int32_t max_seqlen_k) {
  return pa::decode_workspace_bytes(desc, num_decode_rows, max_seqlen_k);
}

// The first num_decode_rows sequences of the varlen batch have one query
// each: they go through the split-K decode kernels (lengths from
// cu_seqlens_k); the remaining rows go through the MFMA prefill kernel.
extern "C" int pa_mixed_varlen(const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t num_seqs, int32_t num_decode_rows, int32_t max_seqlen_q,
                               int32_t max_seqlen_k, const int32_t* block_tables,
                               int32_t max_blocks_per_seq, float scale, void* out,
                               void* workspace, size_t workspace_bytes, const pa_desc* desc,
                               void* stream) {
  using namespace pa;
  int rc = check_desc(desc);
  if (rc) return rc;
  if (num_decode_rows < 0 || num_decode_rows > num_seqs)
    return fail(PA_ERR_INVALID_ARG, "pa_mixed_varlen: num_decode_rows %d outside [0, %d]",
                num_decode_rows, num_seqs);
  if (debug_enabled() && num_seqs > 0 && cu_seqlens_q && cu_seqlens_k) {
    // the prefix sums as a whole; each launch below checks its rows' tables
    rc = debug_check_varlen("pa_mixed_varlen", cu_seqlens_q, cu_seqlens_k, num_seqs,
                            max_seqlen_q, max_seqlen_k, num_decode_rows, (hipStream_t)stream);
    if (rc) return rc;
  }
  if (num_decode_rows > 0) {
    rc = launch_decode("pa_mixed_varlen", q, k_cache, v_cache, block_tables, max_blocks_per_seq,
                       nullptr, cu_seqlens_k, num_decode_rows, max_seqlen_k, scale, out,
                       workspace, workspace_bytes, 0, desc, stream, nullptr);
    if (rc) return rc;
  }
  const int32_t rest = num_seqs - num_decode_rows;
  if (rest > 0) {
    if (!cu_seqlens_q || !cu_seqlens_k || !block_tables)
      return fail(PA_ERR_INVALID_ARG, "pa_mixed_varlen: NULL pointer");
    rc = launch_prefill("pa_mixed_varlen", q, k_cache, v_cache, cu_seqlens_q + num_decode_rows,
                        cu_seqlens_k + num_decode_rows, rest, max_seqlen_q, max_seqlen_k,
                        block_tables + (int64_t)num_decode_rows * max_blocks_per_seq,
                        max_blocks_per_seq, scale, out, desc, stream, false);
  }
  return rc;
}

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
//     256/G query positions). Its 16 column tiles (two per wave) are 16
//     positions x 1 q-head each, covering all G q-heads of the kv-head, so
//     every K/V stage staged in LDS serves the whole GQA group. A wave takes
//     its two tiles as one 32-column tile of v_mfma_f32_32x32x16_bf16.
//   * Scores are computed transposed, S^T = K Q^T: A = K rows from LDS, B =
//     Q held in registers for the whole loop. The accumulator layout of S^T
//     (one query column per lane pair, keys down the registers) is the
//     B-operand layout of the next product O^T += V^T P^T once the keys of a
//     16-key step are renumbered, so P never goes through LDS; V is staged
//     transposed (d-major) in LDS in that key order.
//   * Online softmax per query column: base-2 exponent with scale*log2(e)
//     folded in, lazily rescaled running max, P rounded to bf16 for the MFMA
//     (the row sum adds the same rounded weights), fp32 accumulation, bf16
//     output.
//   * Keys are staged 64 at a time (with blocks of 64 tokens or more a stage
//     never straddles a block, so one block-table lookup per stage), K one
//     stage ahead of V in LDS so that each wave multiplies the next stage's
//     scores while it runs the current stage's softmax; register staging
//     brings each stage in a whole iteration before it is stored.
//   * Causal work skipping: stages past the work item's last query are never
//     loaded; only stages that cross the diagonal apply the mask.
//   * Grid order: per sequence the last position blocks (the most keys) come
//     first; consecutive workgroups differ in kv-head so one (sequence,
//     kv-head)'s blocks, which re-read the same K/V, land on the same XCD.
#include <cmath>

#include "common.hpp"

namespace pa {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 8;  // waves per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kNT = 2;     // 16-column tiles per wave
constexpr int kTiles = kNT * kWaves;      // 16-column tiles per workgroup
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

// ---- 32 x 32 tiles (v_mfma_f32_32x32x16_bf16), software-pipelined
//
// Each wave's two 16-column tiles are taken as one 32-column tile: column j
// of a wave is column j % 16 of its tile j / 16. A 32 x 32 x 16 product
// reads a 1 KiB A operand for 32 K FLOP, twice the work per LDS byte of a
// 16 x 16 x 32 one. Lane layouts (checked on the GPU): A[i][k] in lane i + 32 (k / 8),
// B[k][j] in lane j + 32 (k / 8), both 8 consecutive k; D[i][j] in lane
// j + 32 h, register r, for i = 8 (r / 4) + 4 h + r % 4.
//   * S^T = K Q^T per 32-key tile: A = 32 K rows from LDS, B = Q held in
//     registers (8 d per lane per 16-d step).
//   * Lane j + 32 h holds the scores of column j for keys 8q + 4h + c; its
//     registers 8s .. 8s + 7 of a stage are the B operand of k-step s of
//     O^T += V^T P^T when the 16 keys of a k-step are numbered with bits 2
//     and 3 swapped: V^T is staged in that order (swap23), and P stays in
//     registers.
//   * A column's two lanes are the two halves of the wave: its max and sum
//     are exchanged with v_permlane32_swap.
//   * Pipelining: while the softmax of stage st runs on the vector ALU, the
//     scores of stage st + 1 are already being multiplied, so each wave
//     keeps the matrix unit fed on its own. K is therefore staged one stage
//     ahead of V: at iteration st the LDS holds K of stage st + 1 and V of
//     stage st, the registers bring in K of stage st + 3 and V of stage
//     st + 2, and one barrier per stage guards both double buffers. The
//     loop is unrolled twice so the two score arrays swap roles in place.
__device__ __forceinline__ int swap23(int x) { return (x & ~12) | ((x & 4) << 1) | ((x & 8) >> 1); }

// Both lanes of a column (lanes c and c + 32) get max / sum of their values.
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Physical block of the block holding key position p (a broken table entry
// reads block 0: the result is then meaningless, but the access stays
// inside the pool).
__device__ __forceinline__ int64_t block_of(const PrefillArgs& a, const int32_t* bt, int p) {
  const int raw = bt[p >> a.block_shift];
  return (raw >= 0 && raw < a.num_blocks) ? raw : 0;
}

// Cache row of key position p when blocks hold fewer keys than a stage: each
// key looks its block up on its own.
__device__ __forceinline__ int64_t small_block_row(const PrefillArgs& a, const int32_t* bt, int p) {
  return (block_of(a, bt, p) << a.block_shift) + (p & (a.block_size - 1));
}

// Register loads of K (resp. V) of stage `stage` for blocks smaller than a
// stage; keys at or past kmax are never visible and re-read the last needed
// one. (Larger blocks use scalar stage bases, in the kernel.)
template <int D>
__device__ __forceinline__ void load_k_small(const PrefillArgs& a, const int32_t* bt, int g,
                                             int kmax, int stage,
                                             u32x4 (&kreg)[Geo<D>::KCHUNKS]) {
  const int t = threadIdx.x;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const uint16_t* kc = a.k_cache + (int64_t)g * D;
#pragma unroll
  for (int i = 0; i < Geo<D>::KCHUNKS; ++i) {
    const int c = t + i * kThreads;
    const int kp = min(stage * kKT + c / (D / 8), kmax - 1);
    kreg[i] = *reinterpret_cast<const u32x4*>(kc + small_block_row(a, bt, kp) * row_elems +
                                              (c % (D / 8)) * 8);
  }
}

template <int D>
__device__ __forceinline__ void load_v_small(const PrefillArgs& a, const int32_t* bt, int g,
                                             int kmax, int stage,
                                             typename VVec<Geo<D>::VW>::T (&vreg)[2]) {
  typedef typename VVec<Geo<D>::VW>::T VT;
  const int t = threadIdx.x;
  const int64_t row_elems = (int64_t)a.num_kv_heads * D;
  const uint16_t* vc = a.v_cache + (int64_t)g * D;
  const int pair = t % 32;  // keys 2 pair, 2 pair + 1 of the stage
  const int dg = t / 32;    // d range [dg VW, dg VW + VW)
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int kp = min(stage * kKT + 2 * pair + s, kmax - 1);
    vreg[s] = *reinterpret_cast<const VT*>(vc + small_block_row(a, bt, kp) * row_elems +
                                           dg * Geo<D>::VW);
  }
}

template <int D>
__device__ __forceinline__ void store_k32(char* kst, const u32x4 (&kreg)[Geo<D>::KCHUNKS]) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Geo<D>::KCHUNKS; ++i) {
    const int c = t + i * kThreads;
    *reinterpret_cast<u32x4*>(kst + (c / (D / 8)) * Geo<D>::KROW + (c % (D / 8)) * 16) = kreg[i];
  }
}

// V^T[d][slot]: a dword holds the pair (V[2p][d], V[2p+1][d]); swap23 keeps
// an even key and its odd neighbour in adjacent slots
template <int D>
__device__ __forceinline__ void store_v32(char* vst, const typename VVec<Geo<D>::VW>::T (&vreg)[2]) {
  using GG = Geo<D>;
  const int t = threadIdx.x;
  const int key0 = 2 * (t % 32);
  const int slot = (key0 & ~15) + swap23(key0 & 15);
  char* vt = vst + slot * 2;
#pragma unroll
  for (int w = 0; w < GG::VW / 2; ++w) {
    const int d = (t / 32) * GG::VW + 2 * w;
    const uint32_t e0 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x05040100u);
    const uint32_t e1 = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], 0x07060302u);
    *reinterpret_cast<uint32_t*>(vt + d * GG::VROW) = e0;
    *reinterpret_cast<uint32_t*>(vt + (d + 1) * GG::VROW) = e1;
  }
}

template <int D, int G_, bool SMALL>
__global__ __launch_bounds__(kThreads) void prefill32_kernel(PrefillArgs a) {
  using GG = Geo<D>;
  typedef __attribute__((ext_vector_type(16))) float f32x16;
  const int G = G_ ? G_ : a.group;
  const int QB = positions_per_workgroup(G);  // query positions per workgroup
  const int used = (kTiles / G) * G;          // tiles with columns of their own
  constexpr int KSTEPS = D / 16;              // 16-d steps of S^T
  constexpr int DT = D / 32;                  // 32-row tiles of O^T over head_dim
  // K buffers, then V^T buffers
  __shared__ __attribute__((aligned(16))) char lds[2 * GG::STAGE];
  char* const kbuf = lds;
  char* const vbuf = lds + 2 * GG::KBYTES;

  const int H_kv = a.num_kv_heads;
  const int H_q = H_kv * G;
  int idx = blockIdx.x;
  const int g = idx % H_kv;
  idx /= H_kv;
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
  const int j = lane % 32;  // this lane's column
  const int h = lane / 32;  // which 8 of each 16 keys / d it holds
  const int jt = j / 16;

  int head[kNT], pbase[kNT];
  bool own[kNT];  // a spare tile (when G does not divide kTiles) repeats a used one, unwritten
#pragma unroll
  for (int t2 = 0; t2 < kNT; ++t2) {
    const int T = wave * kNT + t2;
    own[t2] = T < used;
    const int Tu = own[t2] ? T : T - used;
    head[t2] = g * G + Tu % G;
    pbase[t2] = p0 + (Tu / G) * 16;
  }
  const int wmin = min(pbase[0], pbase[1]);  // first position any column holds
  const int mypos = (jt ? pbase[1] : pbase[0]) + j % 16;
  const int myhead = jt ? head[1] : head[0];
  const bool myown = jt ? own[1] : own[0];
  // First stage whose last key lies after the query of some column of the
  // wave (wave-uniform, read into a scalar register for a scalar branch).
  // From there on the mask runs, so a stage after all of the wave's queries
  // (at most one: its positions span less than a stage) adds nothing.
  const int diag_st = __builtin_amdgcn_readfirstlane(max(off + wmin + 1, 0) / kKT);

  // Q^T operand for all 16-d steps (rows outside the sequence re-read row
  // 0; their columns are never written)
  bf16x8 qf[KSTEPS];
  {
    const uint16_t* qp = a.q + ((int64_t)(q0 + max(mypos, 0)) * H_q + myhead) * D + h * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + ks * 16));
  }

  f32x16 o[DT];
  float m = -INFINITY, l = 0.f;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[dt][i] = 0.f;

  // S^T of the two 32-key tiles of the K stage at `kst`
  auto scores = [&](const char* kst, f32x16 (&sc)[2]) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[kt][i] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(kst + (kt * 32 + j) * GG::KROW + ks * 32 +
                                                    h * 16));
        sc[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], sc[kt], 0, 0, 0);
      }
    }
  };

  // ---- register staging: kr holds K of stage st + 2, vr V of stage st + 1
  // when iteration st starts; the iteration stores them and brings in K of
  // stage st + 3 and V of stage st + 2. Stage indices are clamped, so every
  // load and store is unconditional: a buffer written past the last stage
  // is never read. With blocks of at least a stage, the stage lies in one
  // block, so a load is a scalar base plus a per-thread offset fixed for the
  // whole loop, and the block's table entry is read an iteration ahead. K
  // rows past kmax are read as they are (same block, and the mask removes
  // their scores); V rows past kmax re-read row kmax - 1, since a zero
  // weight times a non-finite stale value would not vanish. Smaller blocks
  // look every key up on its own (load_k_small / load_v_small).
  typedef typename VVec<GG::VW>::T VT;
  const int row_e = H_kv * D;           // elements per cache row
  const int pair = threadIdx.x % 32;    // V: keys 2 pair, 2 pair + 1 of a stage
  const int dg = threadIdx.x / 32;      // V: d range [dg VW, dg VW + VW)
  uint32_t koff[GG::KCHUNKS], voff[2];  // element offsets from a stage's first row
#pragma unroll
  for (int i = 0; i < GG::KCHUNKS; ++i) {
    const int c = threadIdx.x + i * kThreads;
    koff[i] = (uint32_t)((c / (D / 8)) * row_e + (c % (D / 8)) * 8);
  }
#pragma unroll
  for (int s = 0; s < 2; ++s) voff[s] = (uint32_t)((2 * pair + s) * row_e + dg * GG::VW);
  u32x4 kr[GG::KCHUNKS];
  VT vr[2];
  // K of stage sk (in block bk) and V of stage sv (in block bv)
  auto load_kv = [&](int sk, int64_t bk, int sv, int64_t bv) {
    if constexpr (SMALL) {
      load_k_small<D>(a, bt, g, kmax, sk, kr);
      load_v_small<D>(a, bt, g, kmax, sv, vr);
    } else {
      const int kb = sk * kKT, vb = sv * kKT;
      const uint16_t* kp =
          a.k_cache + ((bk << a.block_shift) + (kb & (a.block_size - 1))) * row_e + g * D;
      const uint16_t* vp =
          a.v_cache + ((bv << a.block_shift) + (vb & (a.block_size - 1))) * row_e + g * D;
#pragma unroll
      for (int i = 0; i < GG::KCHUNKS; ++i) kr[i] = *reinterpret_cast<const u32x4*>(kp + koff[i]);
      // (selected only on the last stage, where kmax - 1 - vb < 64; clamped so
      // the product stays in range on the others)
      const uint32_t vlast = (uint32_t)(min(kmax - 1 - vb, kKT - 1) * row_e + dg * GG::VW);
#pragma unroll
      for (int s = 0; s < 2; ++s)
        vr[s] = *reinterpret_cast<const VT*>(vp + (vb + 2 * pair + s < kmax ? voff[s] : vlast));
    }
  };
  int64_t bk = 0, bv = 0;  // blocks of the iteration's K and V loads
  int raw_next = 0;        // table entry of the next iteration's K block
  auto staging = [&](int st) {
    const int64_t bk_now =
        SMALL ? 0 : ((raw_next >= 0 && raw_next < a.num_blocks) ? raw_next : 0);
    if constexpr (!SMALL) raw_next = bt[(min(st + 4, n_stages - 1) * kKT) >> a.block_shift];
    bv = bk;
    bk = bk_now;
    store_k32<D>(kbuf + (st & 1) * GG::KBYTES, kr);
    store_v32<D>(vbuf + ((st + 1) & 1) * GG::VBYTES, vr);
    load_kv(min(st + 3, n_stages - 1), bk, min(st + 2, n_stages - 1), bv);
  };

  // One stage: softmax of `cur` (stage st), scores of stage st + 1 into
  // `nxt`, O^T += V^T P^T of stage st. The next scores are computed even on
  // the wave's last stage (the result is then never read): that keeps the
  // stage one straight run of code the scheduler can interleave.
  auto step = [&](int st, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    if (st >= diag_st) {  // the stage crosses some column's diagonal
      // (kept a branch: the mask is not worth running on every stage)
      asm volatile("" ::: "memory");
      // key 32 kt + 8 (r / 4) + 4 h + r % 4 of the stage at cur[kt][r]
      const int thr = off + mypos - st * kKT - 4 * h;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int c = (i >> 4) * 32 + ((i & 15) >> 2) * 8 + (i & 3);
        if (c > thr) cur[i >> 4][i & 15] = -INFINITY;
      }
    }
    float mx = cur[0][0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, cur[i >> 4][i & 15]);
    mx = halves_max(mx) * a.scale_log2;
    // both lanes of a column see the same mx and m, so they agree on it
    const bool need = mx > m + kLazyLog2;
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float mnew = need ? fmaxf(m, mx) : m;
      const float alpha = need ? __builtin_amdgcn_exp2f(m - mnew) : 1.f;  // 0 on the first step
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    const float negm = (m == -INFINITY) ? 0.f : -m;
    staging(st);
    scores(kbuf + ((st + 1) & 1) * GG::KBYTES, nxt);
    const char* vst = vbuf + (st & 1) * GG::VBYTES;
#pragma unroll
    for (int s = 0; s < kKT / 16; ++s) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        p[e] = __builtin_amdgcn_exp2f(fmaf(cur[s >> 1][(s & 1) * 8 + e], a.scale_log2, negm));
      uint4 pk;
      pk.x = pack2_bf16(p[0], p[1]);
      pk.y = pack2_bf16(p[2], p[3]);
      pk.z = pack2_bf16(p[4], p[5]);
      pk.w = pack2_bf16(p[6], p[7]);
      // the sum adds the rounded weights the MFMA sees (an exact weighted mean)
      l = sum_pair_bf16(pk.x, l);
      l = sum_pair_bf16(pk.y, l);
      l = sum_pair_bf16(pk.z, l);
      l = sum_pair_bf16(pk.w, l);
      const bf16x8 pf = __builtin_bit_cast(bf16x8, pk);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 av = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const uint4*>(vst + (dt * 32 + j) * GG::VROW +
                                                    (s * 16 + h * 8) * 2));
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, pf, o[dt], 0, 0, 0);
      }
    }
  };
  auto iterate = [&](int st, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    step(st, cur, nxt);
    __syncthreads();
  };

  // Prologue: K and V of stage 0 to LDS, scores of stage 0, K of stage 1 to
  // LDS; kr, vr then hold K of stage 2 and V of stage 1.
  f32x16 sa[2], sb[2];
  {
    const int s1 = min(1, n_stages - 1), s2 = min(2, n_stages - 1), s3 = min(3, n_stages - 1);
    const int64_t b0 = SMALL ? 0 : block_of(a, bt, 0);
    const int64_t b1 = SMALL ? 0 : block_of(a, bt, s1 * kKT);
    const int64_t b2 = SMALL ? 0 : block_of(a, bt, s2 * kKT);
    load_kv(0, b0, 0, b0);
    store_k32<D>(kbuf, kr);
    store_v32<D>(vbuf, vr);
    load_kv(s1, b1, s1, b1);
    __syncthreads();
    scores(kbuf, sa);
    store_k32<D>(kbuf + GG::KBYTES, kr);
    load_kv(s2, b2, s1, b1);  // vr: V of stage 1 again
    bk = b2;                  // iteration 0 loads V of stage 2 from it
    if constexpr (!SMALL) raw_next = bt[(s3 * kKT) >> a.block_shift];
    __syncthreads();
  }
  for (int st = 0; st < n_stages; st += 2) {
    iterate(st, sa, sb);
    if (st + 1 < n_stages) iterate(st + 1, sb, sa);
  }

  // ---- epilogue: column sum across the two lanes, normalise, store
  const float lt = halves_sum(l);
  if (!myown || mypos < 0 || mypos >= p_end) return;
  const float inv = 1.f / lt;
  uint16_t* dst = a.out + ((int64_t)(q0 + mypos) * H_q + myhead) * D + h * 4;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      uint2 v;
      v.x = pack2_bf16(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv);
      v.y = pack2_bf16(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv);
      *reinterpret_cast<uint2*>(dst + dt * 32 + q4 * 8) = v;
    }
}

using PrefillFn = void (*)(PrefillArgs);

template <int D, int G_, bool SMALL>
PrefillFn kernel_for() {
  return prefill32_kernel<D, G_, SMALL>;
}

template <int D, bool SMALL>
PrefillFn pick(int G) {
  switch (G) {
    case 1: return kernel_for<D, 1, SMALL>();
    case 2: return kernel_for<D, 2, SMALL>();
    case 4: return kernel_for<D, 4, SMALL>();
    case 8: return kernel_for<D, 8, SMALL>();
    case 16: return kernel_for<D, 16, SMALL>();
  }
  return G >= 1 && G <= kTiles ? kernel_for<D, 0, SMALL>() : nullptr;  // other group sizes
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

// Block-sparse attention over the static stripe-sort pattern.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention,
// static-pattern bullet: after the stripe-sort permutation the N x N map is a 4 x 4
// mosaic of banded sub-maps plus a small global keep-set; the pattern is fixed, so a
// FlashAttention-2-style kernel runs it with no mask built at run time. Here the
// plan's tile list (CSR: kept key tiles of every query tile) is that pattern; every
// kept tile is computed whole and nothing inside a tile is masked.
//
// Kernels:
//  * attn_mfma64_kernel (bf16, head_dim 64, B = 64, stripes a multiple of 64 long):
//    persistent 512-thread workgroups walk units = (work item, segment, head), longest
//    first. A work item is a group of up to four query tiles with identical kept-key
//    lists (one per stripe at the same offset) against that list; every K and V^T
//    tile is loaded into LDS once for the group. S^T = K Q^T and O^T = V^T P^T run on
//    v_mfma_f32_32x32x16_bf16, so a lane holds one query's scores (the row max needs
//    one permlane swap with lane ^ 32) and one query's output column. K tile rows are
//    stored in a permuted order so that the S^T accumulator already has the layout of
//    the P^T operand. Online softmax in fp32 with exp2: Q carries the scale and
//    log2(e), a fifth MFMA k-step subtracts the bf16-exact running reference, so a
//    probability costs one v_exp_f32; the reference moves (and O is rescaled) only on
//    the first tile and when a lane's probability sum passes 2^64. The unit is a
//    template on the key-parity count, so the per-step tile loads have no branches.
//  * attn_d80_kernel: the same work items for head_dim 80 (running max with a 2^8
//    slack, denominators from a ones row of the third V^T block).
//  * attn_win_kernel: short segments (windows, N <= 256), one workgroup per (segment,
//    head). Key tiles kept by the same query tiles share consecutive LDS slots cut into
//    16-key blocks; query positions keeping the same key tiles form groups of 16; each
//    group runs on v_mfma_f32_16x16x32_bf16 over exactly its kept key blocks (1.04x the
//    kept pairs of a ViT-B window, where whole 32 x 32 blocks are 3.0x).
//  * attn_short_kernel: short segments whose key classes do not fit the window kernel's
//    256 slots: K and V^T in LDS by position, whole 32 x 32 blocks, the static mask as
//    one or two extra MFMA k-steps over key classes.
//  * attn_combine_kernel: merges the partial results of rows split over several
//    work items (none at ViT sizes).
//  * attn_simt_kernel (fp32 or bf16 storage, any pattern and head_dim <= 128): one to
//    sixteen threads per query (each a share of the keys, merged at the end), V rows
//    staged in LDS, K rows read through the scalar cache when one thread serves a query
//    and staged with V otherwise; the exact path for small configs.
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

// ---------------------------------------------------------------- MFMA kernel (D = 64, B = 64)

constexpr int kTile = 64;
constexpr int kTileBytes = kTile * 128;          // one swizzled 64 x 64 bf16 tile
constexpr int kParityBytes = 4 * kTileBytes;     // K ring (2 slots) + V^T ring (2 slots)
constexpr int kAttnWaves = 8;                    // wavefronts per workgroup: 4 x (two query halves)
constexpr int kAttnLds = 4 * kParityBytes;       // up to four key parities: 128 KiB
// partial record of a split row (floats): O[D], m, l, pad
__host__ __device__ constexpr int part_ld(int D) { return D + 4; }

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// The running max of the online softmax is the reference of exp2(); moving it costs a
// rescale of the output accumulators. The result does not depend on the reference, so
// it only moves when a new score exceeds it by more than this many binary orders:
// probabilities then stay below 2^8, far inside the fp32 and bf16 range.
constexpr float kRescaleSlack = 8.0f;

// The D = 64 kernel moves its reference even more lazily: only when a lane's sum of 32
// probabilities passes 2^64 (so every probability stays below 2^64, and a row's O and
// l below 2^64 * 4096 * max |v|, far inside fp32).
constexpr float kOverflowGuard = 18446744073709551616.0f;  // 2^64

// Relative-position bias in the D = 64 kernel (attn_mfma64_rel_kernel). A query's bias
// table row (k_relpos.hip) has 128 fp16 entries: key rows 0..63, key columns at 64..127.
// The bias enters S^T through eight more MFMA k-steps (fp16 operands, 2^-11 relative
// rounding of the bias instead of bf16's 2^-8) whose K operand is one-hot in the key's
// row (k-steps 0..3) or column (4..7) and whose Q^T operand is the query's table row. LDS past the rings: the query halves' table rows (8 KiB each; with P parities the
// G = 4 / P members need at most 16 KiB after 128 KiB of rings, 64 KiB after 32), then
// 17 one-hot fp16 rows of 16 bytes (row 8 + e: 1.0 at element e; the others zero) and the
// key coordinates of every K slot, [slot][parity][64 keys].
constexpr int kRelTj = 128;
constexpr int kRelTqBytes = 32 * kRelTj * 2;
constexpr int kRelOneHot = 4 * kParityBytes + 2 * kRelTqBytes;
constexpr int kRelKc = kRelOneHot + 512;
constexpr int kRelLds = kRelKc + 2 * 4 * 64 * 4;
static_assert(kRelLds <= 160 * 1024, "bias layout fits the LDS");

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;

// acc + a + b for two bf16 values, in one dot product with (1, 1)
__device__ __forceinline__ float sum_bf16_pair(bf16_t a, bf16_t b, float acc) {
  const bf16x2 ab = {a, b}, one = {to_bf16(1.0f), to_bf16(1.0f)};
  return __builtin_amdgcn_fdot2_f32_bf16(ab, one, acc, false);
}

// eight bf16 values times s, rounded back to bf16
__device__ __forceinline__ bf16x8 scale_bf16x8(bf16x8 v, float s) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = to_bf16(to_f32(v[e]) * s);
  return r;
}

// max of three floats; the compiler forms v_max3_f32 (and, unlike inline assembly,
// inserts the wait states a read of fresh MFMA results needs)
__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// key row held by row r of a K tile in LDS: rows 4..7 and 8..11 of each 16-row group
// are exchanged (an involution)
__device__ __forceinline__ int kperm16(int r) {
  const int q = r & 12;
  return q == 4 ? r + 4 : q == 8 ? r - 4 : r;
}

// max over lanes l and l ^ 32 (one permlane swap, no LDS round trip)
__device__ __forceinline__ float max_xor32(float v) {
  const unsigned u = __float_as_uint(v);
  const auto t = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(t[0]), __uint_as_float(t[1]));
}

// One work item: a group of G <= 4 query tiles whose kept key-tile lists are identical
// (the 4 x 4 mosaic repeats one band in every sub-map, so the same tile index in each
// stripe has the same list), against the kept key tiles col_idx[kb..ke) of that list,
// at most kAttnItemTiles (<= 64) of them. The eight wavefronts are G tiles x two query
// halves x P = 4 / G key parities (G = 3: P = 1, one pair idle but loading): parity p
// walks list entries p, p + P, ...; the parities merge through LDS at the end. Every K
// and V^T tile is loaded into LDS once for the whole group. Longer lists (none at
// ViT sizes) are split over G = 1 items that write an unnormalised partial (O,
// running max, running sum) to `partial` at `slot` for a combine pass.
//
// Item record (two int4): {kb, ke, slot or -1, G | P << 4}, {query tile of each member}.
//
// Pipeline of a wavefront (its j-th tile is list entry p + P j): each parity has a
// two-slot ring for K and one for V^T. Step j computes S_j = K_j Q^T on the matrix
// cores from K fragments read into registers in step j - 1 (tile t's in register set
// t & 1), so the MFMAs start right after the barrier; then the softmax of S_j and
// O^T += V_j^T P_j^T. Meanwhile the step reads K_{j+1}'s fragments for the next step
// and V_j's for its own O^T update, and the workgroup issues the direct-to-LDS loads
// of K_{j+2} and V_{j+1} of every parity (wavefront w loads row group w of each tile)
// into the slots of K_j and V_{j-1}, whose fragments were read in step j - 1. One
// barrier per step, after each wavefront's own loads and LDS reads are complete, both
// publishes K_{j+1} and V_j and retires the slots the step overwrites. (Loading more
// steps ahead through deeper rings measured slower.)
static_assert(kAttnItemTiles <= 64, "one key tile per lane");
// P: key parities of the item (1, 2 or 4): the load code has no run-time loop. REL: add
// the relative-position bias from rel_t (bias table rows) and rel_kc (key coordinates).
template <int P, bool REL>
__device__ __forceinline__ void attn_mfma64_unit(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt,
                                                 const bf16_t* __restrict__ VT, bf16_t* __restrict__ O,
                                                 const int4* __restrict__ items, const int* __restrict__ col_idx,
                                                 const int* __restrict__ tile_start, int n, int n_pad, int heads,
                                                 int seg_heads, float c_log2, float* __restrict__ partial, int item,
                                                 int sh, char* smem, const f16_t* __restrict__ rel_t,
                                                 const int* __restrict__ rel_kc) {
  constexpr int D = 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int4 it0 = items[2 * item], it1 = items[2 * item + 1];
  const int kb = __builtin_amdgcn_readfirstlane(it0.x), ke = __builtin_amdgcn_readfirstlane(it0.y);
  const int slot = __builtin_amdgcn_readfirstlane(it0.z), gp = __builtin_amdgcn_readfirstlane(it0.w);
  const int G = gp & 15;
  const int qh = wave & 1, pr = wave >> 1;  // query half; wavefront pair 0..3
  const int gi = pr % G, kp = pr / G;       // member of the group; key parity
  const bool active = kp < P;               // false only for the spare pair of a G = 3 group
  const int qt = gi == 0 ? it1.x : gi == 1 ? it1.y : gi == 2 ? it1.z : it1.w;
  const int seg = sh / heads, h = sh - seg * heads;
  const bf16_t* q_base = Q + (size_t)sh * n * D;
  const bf16_t* k_base = Kt + (size_t)sh * n * D;
  const bf16_t* v_base = VT + (size_t)sh * D * n_pad;
  constexpr int R = 2;                            // ring slots per parity
  constexpr int ring_bytes = 2 * R * kTileBytes;  // K ring then V^T ring
  char* ring = smem + (active ? kp : 0) * ring_bytes;
  char* tq = smem + P * ring_bytes + (gi * 2 + qh) * kRelTqBytes;  // this query half's bias rows

  // Every tile of these plans is 64 tokens long (stripes are multiples of 64), so tile t
  // starts at token 64 t and no offset table is read. The key offsets are requested
  // first and Q after them: the first direct loads below wait only for the offsets, and
  // the barrier before the loop for Q.
  const int total = ke - kb;
  // first token of the item's i-th key tile, held by lane i and read with readlane, so
  // the loop never waits on a dependent index load
  const int koff = lane < total ? col_idx[kb + lane] * kTile : 0;
  const int q_local = qh * 32 + (lane & 31);
  const int my_q = qt * kTile + q_local;
  // Q^T operand: lane holds Q[my_q][16 ks + 8 (lane / 32) .. + 7], times the softmax
  // scale and log2(e), so that the matrix cores deliver scores in exp2 units
  bf16x8 qf[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
    qf[ks] = scale_bf16x8(*reinterpret_cast<const bf16x8*>(q_base + (size_t)my_q * D + ks * 16 + (lane >> 5) * 8),
                          c_log2);

  // Direct-to-LDS tile loads: wavefront w fills row group w (rows 8 w .. 8 w + 7) of
  // every tile; lane L fetches the chunk that the swizzle places at byte 16 L.
  const int krow = 8 * wave + (lane >> 3), kch = (lane & 7) ^ swz_key(8 * wave + (lane >> 3));
  // K tile row r holds key kperm(r): rows 4..7 and 8..11 of every 16-row group are
  // swapped, so that the S^T accumulator hands lane half h of every 16-key group keys
  // 8h .. 8h+7 in order -- the layout of the P^T operand -- with no lane exchange
  const int k_src = kperm16(krow) * D + kch * 8, v_src = krow * n_pad + kch * 8;
  // Entries past the list are clamped to its last tile: the loads stay unconditional
  // (no branch in the step) and land in slots no wavefront reads.
  auto issue_k = [&](int j) {  // K tiles of step j (every parity) into K slot j mod R
    char* dst = smem + (j & (R - 1)) * kTileBytes + wave * 1024;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k0 = __builtin_amdgcn_readlane(koff, min(p + P * j, total - 1));
      __builtin_amdgcn_global_load_lds((const void*)(k_base + (size_t)k0 * D + k_src),
                                       (__attribute__((address_space(3))) void*)(dst + p * ring_bytes), 16, 0, 0);
    }
    if constexpr (REL) {
      if (wave == 0) {  // the tiles' key coordinates, one dword per lane
#pragma unroll
        for (int p = 0; p < P; ++p) {
          const int k0 = __builtin_amdgcn_readlane(koff, min(p + P * j, total - 1));
          __builtin_amdgcn_global_load_lds(
              (const void*)(rel_kc + (size_t)seg * n + k0 + lane),
              (__attribute__((address_space(3))) void*)(smem + kRelKc + ((j & (R - 1)) * 4 + p) * 256), 4, 0, 0);
        }
      }
    }
  };
  auto issue_v = [&](int j) {  // V^T tiles of step j (every parity) into V slot j mod R
    char* dst = smem + (R + (j & (R - 1))) * kTileBytes + wave * 1024;
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int k0 = __builtin_amdgcn_readlane(koff, min(p + P * j, total - 1));
      __builtin_amdgcn_global_load_lds((const void*)(v_base + k0 + v_src),
                                       (__attribute__((address_space(3))) void*)(dst + p * ring_bytes), 16, 0, 0);
    }
  };
  // wait until this wavefront's tile loads and LDS reads are complete, then meet the
  // other wavefronts
  auto ready = [&]() {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0) & lgkmcnt0_mask());
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // fragments of the K tile in slot s (A operand of S^T = K Q^T: two 32-key blocks) and
  // of the V^T tile in slot s (A operand of O^T = V^T P^T: two 32-channel blocks)
  auto read_k = [&](int j, bf16x8 (&kf)[4][2]) {
    const char* Ks = ring + (j & (R - 1)) * kTileBytes;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        kf[ks][mb] = *reinterpret_cast<const bf16x8*>(Ks + swz(mb * 32 + (lane & 31), ks * 2 + (lane >> 5)));
  };
  // coordinates (row | column << 16) of the keys this lane's K fragment rows hold
  auto read_kc = [&](int j, int (&kcv)[2]) {
    const int* kcs = reinterpret_cast<const int*>(smem + kRelKc) + ((j & (R - 1)) * 4 + kp) * 64;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) kcv[mb] = kcs[kperm16(mb * 32 + (lane & 31))];
  };
  auto read_v = [&](int j, bf16x8 (&vf)[4][2]) {
    const char* Vs = ring + (R + (j & (R - 1))) * kTileBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int md = 0; md < 2; ++md)
        vf[kk][md] = *reinterpret_cast<const bf16x8*>(Vs + swz(md * 32 + (lane & 31), kk * 2 + (lane >> 5)));
  };
  // Reference of exp2 (the online softmax's running max, in exp2 units): m_run, -inf
  // before the first tile. It enters the scores through a fifth k-step of S^T = K Q^T
  // whose K operand is a column of ones (dimension 64 of every key: element 0 of lanes
  // 0..31) and whose Q^T operand holds -m_run (element 0 of lane q < 32), so the
  // accumulator already holds c s - m_run and each probability costs one exp2. The
  // reference is kept bf16-exact for that.
  float m_run = -INFINITY, l_run = 0.0f;
  bf16x8 kx, qx;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    kx[e] = to_bf16(e == 0 && lane < 32 ? 1.0f : 0.0f);
    qx[e] = to_bf16(0.0f);
  }
  // S^T = K Q^T - m_run; the two accumulation chains alternate, so each MFMA depends on
  // the one two back
  auto scores = [&](const bf16x8 (&kf)[4][2], const int (&kcv)[2], f32x16 (&sc)[2]) {
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[mb][e] = 0.0f;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kx, qx, sc[mb], 0, 0, 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
        sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks][mb], qf[ks], sc[mb], 0, 0, 0);
    if constexpr (REL) {
      // table columns 16 ks + 8 h .. + 7 of this lane's query (chunk c of row q sits at
      // chunk c ^ (q & 15)) against the one-hot row of its key's row or column
      const int q = lane & 31, hf = lane >> 5;
      const char* oh = smem + kRelOneHot;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const f16x8 tf = *reinterpret_cast<const f16x8*>(tq + q * (kRelTj * 2) + (((2 * ks + hf) ^ (q & 15)) * 16));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int jj = ks < 4 ? (kcv[mb] & 0xffff) : (kcv[mb] >> 16);
          const int row = min(max(jj - 16 * ks - 8 * hf + 8, 0), 16);
          const f16x8 af = *reinterpret_cast<const f16x8*>(oh + row * 16);
          sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, tf, sc[mb], 0, 0, 0);
        }
      }
    }
  };

  // O^T accumulators: blocks 0 and 1 hold channels 0..63
  f32x16 oacc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.0f;

  // P^T operand of key group kk (keys 16 kk .. + 15) from the scores minus `shift`: with
  // the permuted K rows, accumulator elements 8 (kk & 1) .. + 7 of block kk / 2 are keys
  // 8 h .. 8 h + 7 of the group for lane half h, in order. Returns this lane's sum of
  // the 32 bf16 probabilities (the ones the output is weighted with), by bf16 dot
  // products with (1, 1).
  auto probs = [&](const f32x16 (&sc)[2], bf16x8 (&pf)[4], float shift) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = to_bf16(__builtin_amdgcn_exp2f(sc[kk >> 1][(kk & 1) * 8 + e] - shift));
      pf[kk] = v;
      s0 = sum_bf16_pair(v[0], v[1], s0);
      s1 = sum_bf16_pair(v[2], v[3], s1);
      s0 = sum_bf16_pair(v[4], v[5], s0);
      s1 = sum_bf16_pair(v[6], v[7], s1);
    }
    return s0 + s1;
  };
  // Online softmax of S_j (this lane's query: 32 of the tile's 64 scores, the rest in
  // lane ^ 32) into the P^T operand. The reference moves only on the first tile and
  // when some probability may pass 2^kOverflowLog2 (the lane sum bounds every one of
  // its 32): the row max is then taken, O and l rescaled, and P recomputed (a
  // wave-uniform branch, rare after the first tile).
  auto softmax = [&](const f32x16 (&sc)[2], bf16x8 (&pf)[4], bool first) {
    float sum = probs(sc, pf, 0.0f);
    if (first || __builtin_amdgcn_ballot_w64(sum > kOverflowGuard) != 0) {
      float t[11];
#pragma unroll
      for (int i = 0; i < 10; ++i)
        t[i] = max3f(sc[(3 * i) >> 4][(3 * i) & 15], sc[(3 * i + 1) >> 4][(3 * i + 1) & 15],
                     sc[(3 * i + 2) >> 4][(3 * i + 2) & 15]);
      t[10] = fmaxf(sc[1][14], sc[1][15]);
      float mx = max3f(max3f(t[0], t[1], t[2]), max3f(t[3], t[4], t[5]), max3f(t[6], t[7], max3f(t[8], t[9], t[10])));
      mx = max_xor32(mx);  // relative to the reference the scores carry
      const float base = first ? 0.0f : m_run;
      const float m_new = to_f32(to_bf16(base + (first ? mx : fmaxf(mx, 0.0f))));
      if (!first) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int md = 0; md < 2; ++md)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[md][e] *= alpha;
        l_run *= alpha;
      }
      m_run = m_new;
      qx[0] = to_bf16(lane < 32 ? -m_new : 0.0f);
      sum = probs(sc, pf, m_new - base);
    }
    l_run += sum;
  };
  // O^T += V^T P^T over four 16-key steps
  auto pv = [&](const bf16x8 (&vf)[4][2], const bf16x8 (&pf)[4]) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int md = 0; md < 2; ++md)
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[kk][md], pf[kk], oacc[md], 0, 0, 0);
  };

  const int nj = active ? (total - kp + P - 1) / P : 0;  // tiles of this wavefront's parity
  const int niter = (total + P - 1) / P;                  // steps (parity 0 has the most)
  f32x16 sacc[2];
  bf16x8 kb2[2][4][2];
  int kc2[2][2] = {{0, 0}, {0, 0}};
  // With the bias the registers do not hold a second set of K fragments: K is then
  // loaded one step ahead, like V, and read in the step that uses it.
  issue_k(0);
  if constexpr (!REL) issue_k(1);
  issue_v(0);
  if constexpr (REL) {
    // this query half's 32 bias rows (256 bytes each), once per member: lane L of load i
    // brings row 4 i + L / 16, logical chunk (L % 16) ^ (row & 15)
    if (active && kp == 0) {
      const f16_t* trow = rel_t + ((size_t)sh * n + qt * kTile + qh * 32) * kRelTj;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4), c = (lane & 15) ^ (r & 15);
        __builtin_amdgcn_global_load_lds((const void*)(trow + r * kRelTj + c * 8),
                                         (__attribute__((address_space(3))) void*)(tq + i * 1024), 16, 0, 0);
      }
    }
  }
  ready();
  if constexpr (!REL)
    if (nj > 0) read_k(0, kb2[0]);
  auto step = [&](int j, bf16x8 (&k_use)[4][2], bf16x8 (&k_next)[4][2], int (&kc_use)[2]) {
    ready();
    if constexpr (REL) {
      issue_k(j + 1);
      issue_v(j + 1);
    } else {
      issue_k(j + 2);
      issue_v(j + 1);
      if (j + 1 < nj) read_k(j + 1, k_next);
    }
    if (j < nj) {
      bf16x8 vf[4][2], pf[4];
      if constexpr (REL) {
        read_k(j, k_use);
        read_kc(j, kc_use);
      }
      read_v(j, vf);
      scores(k_use, kc_use, sacc);
      softmax(sacc, pf, j == 0);
      pv(vf, pf);
    }
  };
  for (int j = 0; j < niter; j += 2) {
    if constexpr (REL) {
      step(j, kb2[0], kb2[0], kc2[0]);
      if (j + 1 < niter) step(j + 1, kb2[0], kb2[0], kc2[0]);
    } else {
      step(j, kb2[0], kb2[1], kc2[0]);
      if (j + 1 < niter) step(j + 1, kb2[1], kb2[0], kc2[0]);
    }
  }
  // every wavefront is done with the rings before the exchange area reuses them
  __syncthreads();

  // merge parities 1 .. P-1 into parity 0 through LDS, in parity order (same lane ->
  // same queries); exchange record: [parity - 1][member][query half][lane][m, l, O[32]]
  float* xch = reinterpret_cast<float*>(smem);
  auto rec_of = [&](int p) { return xch + ((((size_t)(p - 1) * G + gi) * 2 + qh) * 64 + lane) * 34; };
  if (active && kp > 0) {
    float* r = rec_of(kp);
    r[0] = m_run;
    r[1] = l_run;
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int e = 0; e < 16; ++e) r[2 + md * 16 + e] = oacc[md][e];
  }
  __syncthreads();
  if (!active || kp > 0) return;  // this wavefront's part of the unit is done
  for (int p = 1; p < P; ++p) {
    const float* r = rec_of(p);
    const float m1 = r[0], l1 = r[1];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[md][e] = oacc[md][e] * a0 + r[2 + md * 16 + e] * a1;
    m_run = mm;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (slot < 0) {
    const float inv_l = 1.0f / l_tot;
    bf16_t* o_row = O + ((size_t)seg * n + my_q) * ((size_t)heads * D) + (size_t)h * D;
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = md * 32 + g4 * 8 + (lane >> 5) * 4;
        bf16x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = to_bf16(oacc[md][g4 * 4 + e] * inv_l);
        *reinterpret_cast<bf16x4*>(o_row + d) = v4;
      }
  } else {
    float* rec = partial + (((size_t)slot * seg_heads + sh) * kTile + q_local) * part_ld(D);
#pragma unroll
    for (int md = 0; md < 2; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = md * 32 + g4 * 8 + (lane >> 5) * 4;
        *reinterpret_cast<f32x4*>(rec + d) =
            f32x4{oacc[md][g4 * 4], oacc[md][g4 * 4 + 1], oacc[md][g4 * 4 + 2], oacc[md][g4 * 4 + 3]};
      }
    if (lane < 32) {
      rec[D] = m_run;
      rec[D + 1] = l_tot;
    }
  }
}

// Unit of workgroup w in round r of a persistent launch of `nwg` workgroups, units u =
// item * seg_heads + segment-head, items longest first; returns `total` when w is done.
//  - More units than workgroups: the workgroups walk the units in snake order, u = r *
//    nwg + (r even ? w : nwg - 1 - w): long units land on every workgroup in the first
//    round and the shortest ones fill in after the shortest first-round units, which
//    evens out the work per workgroup without any atomics.
//  - One round (a workgroup per unit, the ViT-B global block at batch 1): the workgroups
//    of one XCD (w % 8) take consecutive units in segment-head-major order, so a head's
//    items share one or two XCDs' L2 and its K and V^T tiles are fetched once per such
//    XCD (item-major, workgroup 12 i + h sat on XCD (4 i + h) mod 8: every head on two).
//  - head_major (several rounds, chosen by the host when the static schedule is no less
//    balanced than the snake's): round r takes the head-major units r * nwg .., each
//    XCD's workgroups a consecutive run of them, so the items of a segment-head run in
//    one round on one or two XCDs and share its K and V^T tiles in L2 (in the snake
//    order each item of a head runs in another round and fetches the head's tiles again).
__device__ __forceinline__ int attn_unit(int r, int w, int nwg, int total, int n_items, int seg_heads,
                                         int head_major) {
  if (total <= nwg || head_major) {
    if (total <= nwg && r > 0) return total;
    const int x = w % kXcds, j = w / kXcds;
    const int up = r * nwg + x * (nwg / kXcds) + min(x, nwg % kXcds) + j;  // head-major index
    if (up >= total) return total;
    const int sh = up / n_items, item = up - sh * n_items;
    return item * seg_heads + sh;
  }
  return r * nwg + ((r & 1) ? nwg - 1 - w : w);
}

// Persistent launch: `nwg` workgroups (as many as stay resident) walk the units in the
// order attn_unit gives.
__global__ void __launch_bounds__(64 * kAttnWaves) attn_mfma64_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt,
                                                          const bf16_t* __restrict__ VT, bf16_t* __restrict__ O,
                                                          const int4* __restrict__ items,
                                                          const int* __restrict__ col_idx,
                                                          const int* __restrict__ tile_start, int n, int n_pad,
                                                          int heads, int seg_heads, int n_items, float c_log2,
                                                          float* __restrict__ partial, int head_major) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nwg = gridDim.x, w = blockIdx.x;
  const int total = n_items * seg_heads;
  for (int r = 0;; ++r) {
    const int u = attn_unit(r, w, nwg, total, n_items, seg_heads, head_major);
    if (u >= total) break;
    if (r > 0) __syncthreads();  // the previous unit's merge has read its LDS exchange
    const int item = u / seg_heads;
    const int parities = __builtin_amdgcn_readfirstlane(items[2 * item].w) >> 4;
    if (parities == 1)
      attn_mfma64_unit<1, false>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                 partial, item, u - item * seg_heads, smem, nullptr, nullptr);
    else if (parities == 2)
      attn_mfma64_unit<2, false>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                 partial, item, u - item * seg_heads, smem, nullptr, nullptr);
    else
      attn_mfma64_unit<4, false>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                 partial, item, u - item * seg_heads, smem, nullptr, nullptr);
  }
}

// The same kernel with the relative-position bias (bias table rows rel_t [segment,
// head, position, 128] fp16 in exp2 units, key coordinates rel_kc [segment, position]).
__global__ void __launch_bounds__(64 * kAttnWaves) attn_mfma64_rel_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ VT,
    bf16_t* __restrict__ O, const int4* __restrict__ items, const int* __restrict__ col_idx,
    const int* __restrict__ tile_start, int n, int n_pad, int heads, int seg_heads, int n_items, float c_log2,
    float* __restrict__ partial, const f16_t* __restrict__ rel_t, const int* __restrict__ rel_kc, int head_major) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the one-hot rows, written once; the first unit's barrier publishes them
  if (threadIdx.x < 68) {
    const int row = threadIdx.x >> 2, i = threadIdx.x & 3, e = row - 8;
    const uint32_t v = e == 2 * i ? 0x3C00u : e == 2 * i + 1 ? 0x3C000000u : 0u;  // fp16 1.0
    reinterpret_cast<uint32_t*>(smem + kRelOneHot)[threadIdx.x] = v;
  }
  const int nwg = gridDim.x, w = blockIdx.x;
  const int total = n_items * seg_heads;
  for (int r = 0;; ++r) {
    const int u = attn_unit(r, w, nwg, total, n_items, seg_heads, head_major);
    if (u >= total) break;
    if (r > 0) __syncthreads();
    const int item = u / seg_heads;
    const int parities = __builtin_amdgcn_readfirstlane(items[2 * item].w) >> 4;
    if (parities == 1)
      attn_mfma64_unit<1, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                partial, item, u - item * seg_heads, smem, rel_t, rel_kc);
    else if (parities == 2)
      attn_mfma64_unit<2, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                partial, item, u - item * seg_heads, smem, rel_t, rel_kc);
    else
      attn_mfma64_unit<4, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2,
                                partial, item, u - item * seg_heads, smem, rel_t, rel_kc);
  }
}

// ---------------------------------------------------------------- long segments, head_dim 80

// The same work items, wavefront roles and parity merge as attn_mfma64_kernel, for
// head_dim 80 (ViT-H). A K tile is 64 rows of 160 bytes, its 10 chunks of row r
// rotated by r / 8 so that 16 consecutive rows of one logical chunk fall in distinct
// bank groups; a V^T tile is 80 rows of the swizzled 128-byte layout. Both arrive by
// direct-to-LDS loads into two-slot rings per parity (160 KiB for four parities), one
// step ahead; S^T = K Q^T takes five 16-channel steps and O^T = V^T P^T three 32-row
// blocks, rows 80..95 zero in registers. No S-ahead pipelining here: the registers are
// taken by the wider operands.
constexpr int kD80 = 80;
constexpr int kD80Tile = kTile * kD80 * 2;         // bytes of one K or V^T tile (10 KiB)
constexpr int kD80Parity = 4 * kD80Tile;           // K ring + V^T ring, two slots each
constexpr int kD80Lds = 4 * kD80Parity;            // four parities: 160 KiB
__device__ __forceinline__ int k80_off(int r, int c) { return r * 160 + ((c + (r >> 3)) % 10) * 16; }

// With the relative-position bias (REL) the unit walks at most two key parities (the
// rings of four would fill the LDS): a four-parity item runs with wavefront pairs 2 and 3
// idle. After the rings: the query halves' bias table rows (8 KiB each), the 17 one-hot
// rows and the key coordinates, as in the head_dim-64 kernel; the scores are taken to
// exp2 units before the bias k-steps.
constexpr int kD80RelOneHot = 2 * kD80Parity + 4 * kRelTqBytes;
constexpr int kD80RelKc = kD80RelOneHot + 512;
constexpr int kD80RelLds = kD80RelKc + 2 * 4 * 64 * 4;
static_assert(kD80RelLds <= 160 * 1024, "head_dim-80 bias layout fits the LDS");

template <int P, bool REL = false>  // key parities of the item (1, 2 or 4)
__device__ __forceinline__ void attn_d80_unit(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt,
                                              const bf16_t* __restrict__ VT, bf16_t* __restrict__ O,
                                              const int4* __restrict__ items, const int* __restrict__ col_idx,
                                              const int* __restrict__ tile_start, int n, int n_pad, int heads,
                                              int seg_heads, float c_log2, float* __restrict__ partial, int item,
                                              int sh, char* smem, const f16_t* __restrict__ rel_t = nullptr,
                                              const int* __restrict__ rel_kc = nullptr) {
  constexpr int D = kD80, KS = D / 16, MD = 3;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int4 it0 = items[2 * item], it1 = items[2 * item + 1];
  const int kb = __builtin_amdgcn_readfirstlane(it0.x), ke = __builtin_amdgcn_readfirstlane(it0.y);
  const int slot = __builtin_amdgcn_readfirstlane(it0.z), gp = __builtin_amdgcn_readfirstlane(it0.w);
  const int G = gp & 15;
  const int qh = wave & 1, pr = wave >> 1;
  constexpr int PP = REL && P > 2 ? 2 : P;  // parities walked
  const int gi = pr % G, kp = pr / G;
  const bool active = kp < PP;
  const int qt = gi == 0 ? it1.x : gi == 1 ? it1.y : gi == 2 ? it1.z : it1.w;
  const int seg = sh / heads, h = sh - seg * heads;
  const bf16_t* q_base = Q + (size_t)sh * n * D;
  const bf16_t* k_base = Kt + (size_t)sh * n * D;
  const bf16_t* v_base = VT + (size_t)sh * D * n_pad;
  char* ring = smem + (active ? kp : 0) * kD80Parity;
  char* tq = smem + PP * kD80Parity + (gi * 2 + qh) * kRelTqBytes;  // this query half's bias rows
  const int hi = lane >> 5, l32 = lane & 31;

  // 64-token tiles: tile t starts at token 64 t (no offset table); offsets first, then Q
  const int total = ke - kb;
  const int koff = lane < total ? col_idx[kb + lane] * kTile : 0;
  const int q_local = qh * 32 + l32;
  const int my_q = qt * kTile + q_local;
  bf16x8 qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = *reinterpret_cast<const bf16x8*>(q_base + (size_t)my_q * D + ks * 16 + hi * 8);

  // loads: 10 groups of 1 KiB per tile (K and V^T alike); wavefront w takes groups w
  // and w + 8 (< 10). K: physical chunk 64 g + L is row (64 g + L) / 10, position
  // (64 g + L) % 10, which holds logical chunk (position - row / 8) mod 10. V^T: row
  // 8 g + L / 8, position L % 8 holding logical chunk (L % 8) ^ swz_key(row).
  int k_src[2], v_src[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = wave + 8 * i;
    const int pc = 64 * g + lane, kr = pc / 10, kpos = pc - (pc / 10) * 10;
    const int kc = (kpos + 10 - ((kr >> 3) % 10)) % 10;
    k_src[i] = kr * D + kc * 8;
    const int vr = 8 * g + (lane >> 3), vc = (lane & 7) ^ swz_key(8 * g + (lane >> 3));
    v_src[i] = vr * n_pad + vc * 8;
  }
  const bool two_groups = wave + 8 < 10;
  // K and V^T tiles of step j (every parity) into slot s; entries past the list are
  // clamped to its last tile (unconditional loads into slots no wavefront reads)
  auto issue = [&](int j, int s) {
#pragma unroll
    for (int p = 0; p < PP; ++p) {
      const int k0 = __builtin_amdgcn_readlane(koff, min(p + PP * j, total - 1));
      if constexpr (REL) {
        if (wave == 0)  // the tile's key coordinates, one dword per lane
          __builtin_amdgcn_global_load_lds(
              (const void*)(rel_kc + (size_t)seg * n + k0 + lane),
              (__attribute__((address_space(3))) void*)(smem + kD80RelKc + (s * 4 + p) * 256), 4, 0, 0);
      }
      char* base = smem + p * kD80Parity;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (i == 1 && !two_groups) break;
        const int g = wave + 8 * i;
        __builtin_amdgcn_global_load_lds((const void*)(k_base + (size_t)k0 * D + k_src[i]),
                                         (__attribute__((address_space(3))) void*)(base + s * kD80Tile + g * 1024),
                                         16, 0, 0);
        __builtin_amdgcn_global_load_lds(
            (const void*)(v_base + k0 + v_src[i]),
            (__attribute__((address_space(3))) void*)(base + (2 + s) * kD80Tile + g * 1024), 16, 0, 0);
      }
    }
  };

  f32x16 oacc[MD];
#pragma unroll
  for (int i = 0; i < MD; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[i][e] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  auto tile_step = [&](int s) {
    const char* Ks = ring + s * kD80Tile;
    const char* Vs = ring + (2 + s) * kD80Tile;
    f32x16 sc[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[mb][e] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + k80_off(mb * 32 + l32, ks * 2 + hi));
        sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc[mb], 0, 0, 0);
      }
    if constexpr (REL) {
      // K tile rows are in key order here: row mb * 32 + l32 holds that key
      const int* kcs = reinterpret_cast<const int*>(smem + kD80RelKc) + (s * 4 + kp) * 64;
      const int kcv[2] = {kcs[l32], kcs[32 + l32]};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[mb][e] *= c_log2;
      const char* oh = smem + kD80RelOneHot;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const f16x8 tf = *reinterpret_cast<const f16x8*>(tq + l32 * (kRelTj * 2) + (((2 * ks + hi) ^ (l32 & 15)) * 16));
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const int jj = ks < 4 ? (kcv[mb] & 0xffff) : (kcv[mb] >> 16);
          const int row = min(max(jj - 16 * ks - 8 * hi + 8, 0), 16);
          const f16x8 af = *reinterpret_cast<const f16x8*>(oh + row * 16);
          sc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, tf, sc[mb], 0, 0, 0);
        }
      }
    }
    float mx = sc[0][0];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[mb][e]);
    mx = max_xor32(mx);
    const float m_new = fmaxf(m_run, REL ? mx : mx * c_log2);
    if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
      for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[md][e] *= alpha;
      m_run = m_new;
    }
    bf16x8 pf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      bf16x8 v;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        v[e] = to_bf16(__builtin_amdgcn_exp2f(REL ? sc[kk >> 1][(kk & 1) * 8 + e] - m_run
                                                  : __builtin_fmaf(sc[kk >> 1][(kk & 1) * 8 + e], c_log2, -m_run)));
      u32x4 r = __builtin_bit_cast(u32x4, v);
      const auto s02 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
      const auto s13 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
      r = u32x4{s02[0], s13[0], s02[1], s13[1]};
      pf[kk] = __builtin_bit_cast(bf16x8, r);
    }
    // rows 80..95 of the third block: row 80 is all ones (it accumulates the softmax
    // denominators on the matrix cores), the rest zero
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const int d = md * 32 + l32;
        bf16x8 vf;
        if (md < 2 || d < D) {
          vf = *reinterpret_cast<const bf16x8*>(Vs + swz(min(d, D - 1), kk * 2 + hi));
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) vf[i] = to_bf16(d == D ? 1.0f : 0.0f);
        }
        oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], oacc[md], 0, 0, 0);
      }
  };

  const int nj = active ? (total - kp + PP - 1) / PP : 0;
  const int niter = (total + PP - 1) / PP;
  issue(0, 0);
  if constexpr (REL) {
    // 32 bias rows of this query half (256 bytes each), once per member: lane L of load i
    // brings row 4 i + L / 16, logical chunk (L % 16) ^ (row & 15)
    if (active && kp == 0) {
      const f16_t* trow = rel_t + ((size_t)sh * n + qt * kTile + qh * 32) * kRelTj;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4), c = (lane & 15) ^ (r & 15);
        __builtin_amdgcn_global_load_lds((const void*)(trow + r * kRelTj + c * 8),
                                         (__attribute__((address_space(3))) void*)(tq + i * 1024), 16, 0, 0);
      }
    }
  }
  for (int j = 0; j < niter; ++j) {
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    issue(j + 1, (j + 1) & 1);  // into the slot read in step j - 1
    if (j < nj) tile_step(j & 1);
  }
  __syncthreads();
  l_run = oacc[2][8];  // row 80: lane q < 32 holds the denominator of query q, lanes 32..63 0

  float* xch = reinterpret_cast<float*>(smem);
  constexpr int RL = 2 + 16 * MD;  // exchange record: m, l, O[48]
  auto rec_of = [&](int p) { return xch + ((((size_t)(p - 1) * G + gi) * 2 + qh) * 64 + lane) * RL; };
  if (active && kp > 0) {
    float* r = rec_of(kp);
    r[0] = m_run;
    r[1] = l_run;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int e = 0; e < 16; ++e) r[2 + md * 16 + e] = oacc[md][e];
  }
  __syncthreads();
  if (!active || kp > 0) return;
  for (int p = 1; p < PP; ++p) {
    const float* r = rec_of(p);
    const float m1 = r[0], l1 = r[1];
    const float mm = fmaxf(m_run, m1);
    const float a0 = __builtin_amdgcn_exp2f(m_run - mm), a1 = __builtin_amdgcn_exp2f(m1 - mm);
    l_run = l_run * a0 + l1 * a1;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[md][e] = oacc[md][e] * a0 + r[2 + md * 16 + e] * a1;
    m_run = mm;
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (slot < 0) {
    const float inv_l = 1.0f / l_tot;
    bf16_t* o_row = O + ((size_t)seg * n + my_q) * ((size_t)heads * D) + (size_t)h * D;
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = md * 32 + g4 * 8 + hi * 4;
        if (d < D) {
          bf16x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = to_bf16(oacc[md][g4 * 4 + e] * inv_l);
          *reinterpret_cast<bf16x4*>(o_row + d) = v4;
        }
      }
  } else {
    float* rec = partial + (((size_t)slot * seg_heads + sh) * kTile + q_local) * part_ld(D);
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = md * 32 + g4 * 8 + hi * 4;
        if (d < D)
          *reinterpret_cast<f32x4*>(rec + d) =
              f32x4{oacc[md][g4 * 4], oacc[md][g4 * 4 + 1], oacc[md][g4 * 4 + 2], oacc[md][g4 * 4 + 3]};
      }
    if (lane < 32) {
      rec[D] = m_run;
      rec[D + 1] = l_tot;
    }
  }
}

__global__ void __launch_bounds__(64 * kAttnWaves) attn_d80_kernel(const bf16_t* __restrict__ Q,
                                                                  const bf16_t* __restrict__ Kt,
                                                                  const bf16_t* __restrict__ VT, bf16_t* __restrict__ O,
                                                                  const int4* __restrict__ items,
                                                                  const int* __restrict__ col_idx,
                                                                  const int* __restrict__ tile_start, int n, int n_pad,
                                                                  int heads, int seg_heads, int n_items, float c_log2,
                                                                  float* __restrict__ partial, int head_major) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nwg = gridDim.x, w = blockIdx.x;
  const int total = n_items * seg_heads;
  for (int r = 0;; ++r) {
    const int u = attn_unit(r, w, nwg, total, n_items, seg_heads, head_major);
    if (u >= total) break;
    if (r > 0) __syncthreads();
    const int item = u / seg_heads;
    const int parities = __builtin_amdgcn_readfirstlane(items[2 * item].w) >> 4;
    if (parities == 1)
      attn_d80_unit<1>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial, item,
                          u - item * seg_heads, smem);
    else if (parities == 2)
      attn_d80_unit<2>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial, item,
                          u - item * seg_heads, smem);
    else
      attn_d80_unit<4>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial, item,
                          u - item * seg_heads, smem);
  }
}

// The head_dim-80 kernel with the relative-position bias (rel_t: bias table rows
// [segment, head, position, 128] fp16 in exp2 units; rel_kc: key coordinates).
__global__ void __launch_bounds__(64 * kAttnWaves) attn_d80_rel_kernel(
    const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ VT,
    bf16_t* __restrict__ O, const int4* __restrict__ items, const int* __restrict__ col_idx,
    const int* __restrict__ tile_start, int n, int n_pad, int heads, int seg_heads, int n_items, float c_log2,
    float* __restrict__ partial, const f16_t* __restrict__ rel_t, const int* __restrict__ rel_kc, int head_major) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  if (threadIdx.x < 68) {  // one-hot rows, published by the first unit's barrier
    const int row = threadIdx.x >> 2, i = threadIdx.x & 3, e = row - 8;
    const uint32_t v = e == 2 * i ? 0x3C00u : e == 2 * i + 1 ? 0x3C000000u : 0u;
    reinterpret_cast<uint32_t*>(smem + kD80RelOneHot)[threadIdx.x] = v;
  }
  const int nwg = gridDim.x, w = blockIdx.x;
  const int total = n_items * seg_heads;
  for (int r = 0;; ++r) {
    const int u = attn_unit(r, w, nwg, total, n_items, seg_heads, head_major);
    if (u >= total) break;
    if (r > 0) __syncthreads();
    const int item = u / seg_heads;
    const int parities = __builtin_amdgcn_readfirstlane(items[2 * item].w) >> 4;
    if (parities == 1)
      attn_d80_unit<1, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial,
                             item, u - item * seg_heads, smem, rel_t, rel_kc);
    else if (parities == 2)
      attn_d80_unit<2, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial,
                             item, u - item * seg_heads, smem, rel_t, rel_kc);
    else
      attn_d80_unit<4, true>(Q, Kt, VT, O, items, col_idx, tile_start, n, n_pad, heads, seg_heads, c_log2, partial,
                             item, u - item * seg_heads, smem, rel_t, rel_kc);
  }
}

// Merge the partials of split rows: O = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c.
// One wavefront per (split row, segment-head, query); lane d is channel d (and d + 64).
template <int D>
__global__ void __launch_bounds__(256) attn_combine_kernel(const float* __restrict__ partial,
                                                           const int* __restrict__ splits,
                                                           const int* __restrict__ tile_start, bf16_t* __restrict__ O,
                                                           int n, int heads, int seg_heads, int total) {
  constexpr int LD = part_ld(D);
  const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (w >= total) return;
  const int q = w % kTile, rs = w / kTile;
  const int sh = rs % seg_heads, r = rs / seg_heads;
  const int qt = splits[3 * r], slot0 = splits[3 * r + 1], nch = splits[3 * r + 2];
  const int seg = sh / heads, h = sh - seg * heads;
  float mm = -INFINITY;
  for (int c = 0; c < nch; ++c) mm = fmaxf(mm, partial[(((size_t)(slot0 + c) * seg_heads + sh) * kTile + q) * LD + D]);
  for (int d = lane; d < D; d += 64) {
    float num = 0.0f, den = 0.0f;
    for (int c = 0; c < nch; ++c) {
      const float* rec = partial + (((size_t)(slot0 + c) * seg_heads + sh) * kTile + q) * LD;
      const float a = __builtin_amdgcn_exp2f(rec[D] - mm);
      num += a * rec[d];
      den += a * rec[D + 1];
    }
    O[((size_t)seg * n + tile_start[qt] + q) * ((size_t)heads * D) + (size_t)h * D + d] = to_bf16(num / den);
  }
}

// ---------------------------------------------------------------- short segments (windows)

// Segments of at most 256 tokens (the 14 x 14 windows): one 512-thread workgroup per
// (segment, head) holds the segment's whole K and V^T in LDS (keys past n zero) and
// wavefront w takes the 32-query block w. The pattern's blocks (16 tokens, ragged at
// stripe ends) do not align with 32-token MFMA blocks, so each 32 x 32 block is computed
// whole and masked by the plan's static mask (added on the matrix cores, below); blocks
// without any kept pair are skipped. S^T = K Q^T and O^T = V^T P^T on
// v_mfma_f32_32x32x16_bf16 as in the long-segment kernel; head_dim 80 runs V^T as
// three 32-row blocks with rows 80..95 zero in registers.
constexpr int kMaxShortBlocks = 8;  // 32-token blocks of a short segment
static_assert(kShortMaxN <= 32 * kMaxShortBlocks, "short segments fit the unrolled block loop");

constexpr int kShortOneHotBytes = 17 * 16;  // 17 one-hot rows of eight 16-bit entries
constexpr int kShortWaves = 8;               // one wavefront per 32-query block (nt32 <= 8)
constexpr int kShortThreads = 64 * kShortWaves;

template <int D>
struct ShortLds {
  static constexpr int KLD = D + 8;        // K row stride (bf16): 16-byte pad, conflict-free reads
  static constexpr int MD = (D + 31) / 32;  // 32-row blocks of V^T
  // K rows, V^T rows, the fp16 (bias) and bf16 (mask) one-hot tables, then two ints per
  // key (mask class; coordinates for the bias)
  static size_t bytes(int nt32) {
    const int nk = nt32 * 32;
    return (size_t)nk * KLD * 2 + (size_t)D * (nk + 8) * 2 + 2 * kShortOneHotBytes + (size_t)nk * 8;
  }
};

// REL: add the relative-position bias. Short segments are at most 16 x 16, so a query's
// table row (rel_t, fp16, exp2 units) has 32 entries, key rows at 0..15 and key columns
// at 16..31: two fp16 MFMA k-steps whose K operand is one-hot in the key's row (k-step 0)
// or column (k-step 1), from 17 one-hot rows after the K and V^T tiles in LDS. The
// scores are then taken to exp2 units before the bias is added.
//
// The mask rides on the matrix cores too: MK bf16 k-steps add, to the score of a query
// in tile tq and a key of class c, mask_row[tq][c] (0 kept, -2^100 masked), with a
// one-hot K operand from 17 bf16 one-hot rows. A masked score is then -2^100 (times the
// scale): its probability is exactly 0 against any kept reference. A row whose blocks so
// far hold no kept key takes such a score as its reference; its first kept block then
// rescales by exp2(-huge) = 0, which leaves exactly what starting there would have.
//
// Four wavefronts per SIMD (two workgroups per CU) are asked of the compiler: the
// head_dim-80 variant with the bias then fits 128 VGPRs (a few spills) instead of 142 at
// one workgroup per CU -- ViT-H window attention 559 -> 441 us with the bias, 294 -> 255
// us without.
template <int D, bool REL, int MK>
__global__ void __launch_bounds__(kShortThreads) __attribute__((amdgpu_waves_per_eu(4))) attn_short_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt,
                                                         const bf16_t* __restrict__ VT, bf16_t* __restrict__ O,
                                                         const int* __restrict__ pos_tile,
                                                         const int* __restrict__ mask_class,
                                                         const int* __restrict__ mask_row,
                                                         const int* __restrict__ any32, int n, int n_pad, int nt32,
                                                         int heads, float c_log2, const f16_t* __restrict__ rel_t,
                                                         const int* __restrict__ rel_kc) {
  using L = ShortLds<D>;
  constexpr int KS = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nk = nt32 * 32, vld = nk + 8;  // V^T row stride (bf16)
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Vs = Ks + (size_t)nk * L::KLD;
  const int sh = blockIdx.x;
  const int seg = sh / heads, h = sh - seg * heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const bf16_t* q_base = Q + (size_t)sh * n * D;
  const bf16_t* k_base = Kt + (size_t)sh * n * D;
  const bf16_t* v_base = VT + (size_t)sh * D * n_pad;

  // Every load of the fill is issued before any LDS store (fixed trip counts, nk <=
  // 256), so the workgroup waits for one memory latency instead of one per chunk.
  // K rows 0..nk-1 (zero past n), 8 channels per 16-byte chunk: chunk c = tid + 512 i.
  constexpr int KCH = D / 8, KIT = 256 * KCH / kShortThreads;  // nk * KCH / 512 <= KIT
  i32x4 kv[KIT];
  // (loads are unconditional, from clamped in-bounds addresses; rows and keys past n
  // are zeroed in registers)
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int c = tid + kShortThreads * i, r = c / KCH, ch = c - (c / KCH) * KCH;
    kv[i] = *reinterpret_cast<const i32x4*>(k_base + (size_t)min(r, n - 1) * D + ch * 8);
  }
  // V^T rows d = tid / 32 + 16 i, 16-byte key chunk tid % 32 (of nk / 8 <= 32): keys
  // past n read as zero. The chunk read lies inside the n_pad-long row.
  const int vch = tid & 31, kc = vch * 8, kc_in = min(kc, (n - 1) & ~7);
  constexpr int VIT = D / 16;
  bf16x8 vv[VIT];
#pragma unroll
  for (int i = 0; i < VIT; ++i)
    vv[i] = *reinterpret_cast<const bf16x8*>(v_base + (size_t)((tid >> 5) + 16 * i) * n_pad + kc_in);
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int c = tid + kShortThreads * i, r = c / KCH, ch = c - (c / KCH) * KCH;
    if (r < nk) *reinterpret_cast<i32x4*>(Ks + r * L::KLD + ch * 8) = r < n ? kv[i] : i32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int i = 0; i < VIT; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (kc + e >= n) vv[i][e] = (bf16_t)0.0f;
  if (kc < nk) {
#pragma unroll
    for (int i = 0; i < VIT; ++i) *reinterpret_cast<bf16x8*>(Vs + ((tid >> 5) + 16 * i) * vld + kc) = vv[i];
  }
  // one-hot rows (row 8 + e: 1.0 at element e, the other rows zero): fp16 for the bias,
  // bf16 for the mask
  const char* onehot = reinterpret_cast<const char*>(Vs + (size_t)D * vld);
  const char* onehot_m = onehot + kShortOneHotBytes;
  int* key_cls = reinterpret_cast<int*>(const_cast<char*>(onehot_m + kShortOneHotBytes));  // [nk]
  int* key_rc = key_cls + nk;                                                              // [nk]
  // per key: mask class (pads their own) and, for the bias, the coordinates
  // (row | (16 + column) << 16)
  if (tid < nk) {
    key_cls[tid] = mask_class[tid];
    if constexpr (REL) key_rc[tid] = rel_kc[(size_t)seg * n + min(tid, n - 1)];
  }
  if (tid < 136) {
    const int t = tid < 68 ? tid : tid - 68;
    const int row = t >> 2, i = t & 3, e = row - 8;
    const uint32_t one = tid < 68 ? 0x3C00u : 0x3F80u;
    const uint32_t v = e == 2 * i ? one : e == 2 * i + 1 ? one << 16 : 0u;
    if (REL || tid >= 68) reinterpret_cast<uint32_t*>(const_cast<char*>(tid < 68 ? onehot : onehot_m))[t] = v;
  }
  __syncthreads();

  const int hi = lane >> 5, l32 = lane & 31;
  constexpr bool kSumRow = L::MD * 32 > D;  // spare accumulator rows: denominators on the matrix cores
  for (int qt = wave; qt < nt32; qt += kShortWaves) {
    const int qpos = qt * 32 + l32;
    const int qrow = min(qpos, n - 1);
    const int tq = pos_tile[qrow];
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = *reinterpret_cast<const bf16x8*>(q_base + (size_t)qrow * D + ks * 16 + hi * 8);
    f16x8 tf[2];  // this query's bias entries 16 ks + 8 hi .. + 7
    if constexpr (REL) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        tf[ks] = *reinterpret_cast<const f16x8*>(rel_t + ((size_t)sh * n + qrow) * 32 + ks * 16 + hi * 8);
    }
    // this query's mask entries 16 ks + 8 hi .. + 7 (the B operand of the mask k-steps)
    bf16x8 mq[MK];
#pragma unroll
    for (int ks = 0; ks < MK; ++ks)
      mq[ks] = *reinterpret_cast<const bf16x8*>(mask_row + ((size_t)tq * MK * 16 + ks * 16 + hi * 8) / 2);
    f32x16 oacc[L::MD];
#pragma unroll
    for (int md = 0; md < L::MD; ++md)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[md][e] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    const int any = any32[qt];
#pragma unroll
    for (int kt = 0; kt < kMaxShortBlocks; ++kt) {
      if (kt >= nt32 || !((any >> kt) & 1)) continue;  // no kept pair in this 32 x 32 block
      const int kcl = key_cls[kt * 32 + l32];
      const int kcs = REL ? key_rc[kt * 32 + l32] : 0;
      // S^T block: keys kt*32 + 8 (e / 4) + 4 hi + (e % 4) of this lane's query
      f32x16 sc;
#pragma unroll
      for (int e = 0; e < 16; ++e) sc[e] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(Ks + (kt * 32 + l32) * L::KLD + ks * 16 + hi * 8);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], sc, 0, 0, 0);
      }
      if constexpr (REL) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sc[e] *= c_log2;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int jj = ks == 0 ? (kcs & 0xffff) : (kcs >> 16);
          const int row = min(max(jj - 16 * ks - 8 * hi + 8, 0), 16);
          const f16x8 af = *reinterpret_cast<const f16x8*>(onehot + row * 16);
          sc = __builtin_amdgcn_mfma_f32_32x32x16_f16(af, tf[ks], sc, 0, 0, 0);
        }
      }
      // the mask: -2^100 on masked scores, 0 on kept ones
#pragma unroll
      for (int ks = 0; ks < MK; ++ks) {
        const int row = min(max(kcl - 16 * ks - 8 * hi + 8, 0), 16);
        const bf16x8 af = *reinterpret_cast<const bf16x8*>(onehot_m + row * 16);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, mq[ks], sc, 0, 0, 0);
      }
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, sc[e]);
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, REL ? mx : mx * c_log2);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack) != 0) {
        // a lane whose reference does not move keeps alpha = 1 (also when both are -inf)
        const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        if constexpr (!kSumRow) l_run *= alpha;
#pragma unroll
        for (int md = 0; md < L::MD; ++md)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[md][e] *= alpha;
        m_run = m_new;
      }
      // branch-free probabilities: the reference is clamped to -FLT_MAX, so a masked score
      // (-inf) gives exp2(-inf) = 0 even while no key of the row has been kept (the
      // reference is then -inf); otherwise the reference is finite and unchanged
      const float mref = fmaxf(m_run, -3.40282347e38f);
      float ps = 0.0f;
      bf16x8 pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8 v;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = sc[kk * 8 + e];
          v[e] = to_bf16(__builtin_amdgcn_exp2f(REL ? x - mref : __builtin_fmaf(x, c_log2, -mref)));
        }
        // the denominator sums exactly the bf16 probabilities V is multiplied with
        if constexpr (!kSumRow) {
#pragma unroll
          for (int e = 0; e < 8; e += 2) ps = sum_bf16_pair(v[e], v[e + 1], ps);
        }
        u32x4 r = __builtin_bit_cast(u32x4, v);
        const auto s02 = __builtin_amdgcn_permlane32_swap(r[0], r[2], false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(r[1], r[3], false, false);
        r = u32x4{s02[0], s13[0], s02[1], s13[1]};
        pf[kk] = __builtin_bit_cast(bf16x8, r);
      }
      if constexpr (!kSumRow) l_run += ps;
      // O^T += V^T P^T: rows d = 32 md + l32 (zero past D; row D all ones when the last
      // block has spare rows, so the matrix cores sum the denominators), keys kt*32 +
      // 16 kk + 8 hi ..
#pragma unroll
      for (int md = 0; md < L::MD; ++md) {
        const int d = md * 32 + l32;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          bf16x8 vf;
          if (md * 32 + 32 <= D || d < D)
            vf = *reinterpret_cast<const bf16x8*>(Vs + (size_t)min(d, D - 1) * vld + kt * 32 + kk * 16 + hi * 8);
          if (!(md * 32 + 32 <= D) && d >= D) {
#pragma unroll
            for (int i = 0; i < 8; ++i) vf[i] = to_bf16(d == D ? 1.0f : 0.0f);
          }
          oacc[md] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kk], oacc[md], 0, 0, 0);
        }
      }
    }
    if constexpr (kSumRow) {
      // row D sits at row r = D % 32 of the last block; block row 8 (e / 4) + 4 hi + e % 4
      // is element e of lane half hi, so row r is element 4 (r / 8) + r % 4 of the lanes
      // with hi = (r / 4) % 2
      constexpr int r = D % 32;
      l_run = ((r >> 2) & 1) == hi ? oacc[L::MD - 1][4 * (r >> 3) + (r & 3)] : 0.0f;
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (qpos < n) {
      const float inv_l = 1.0f / l_tot;
      bf16_t* o_row = O + ((size_t)seg * n + qpos) * ((size_t)heads * D) + (size_t)h * D;
#pragma unroll
      for (int md = 0; md < L::MD; ++md)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = md * 32 + g4 * 8 + hi * 4;
          if (d < D) {
            bf16x4 v4;
#pragma unroll
            for (int e = 0; e < 4; ++e) v4[e] = to_bf16(oacc[md][g4 * 4 + e] * inv_l);
            *reinterpret_cast<bf16x4*>(o_row + d) = v4;
          }
        }
    }
  }
}

// ---------------------------------------------------------------- window kernel on 16-key blocks

// Short segments without the bias (the windows), computed on the kept pairs only. The
// plan (see the window tables in api.hip) packs the segment for the kernel:
//  - key blocks: key tiles kept by the same set of query tiles form a class; a class's
//    positions are stored consecutively in LDS slots and cut into blocks of 16 slots
//    (the last one of a class partly empty, its empty slots masked);
//  - query groups: query positions whose tiles keep the same key tiles, up to 16 per
//    group, each with the list of its key blocks (exactly the kept keys of its queries).
// One workgroup of eight wavefronts per (segment, head); each wavefront takes a list of
// groups (balanced over the wavefronts by the plan) and walks a group's key blocks two at
// a time on v_mfma_f32_16x16x32_bf16: S^T = K Q^T per block (lane = query l % 16, keys
// 4 (l / 16) .. + 3 of the block), online softmax in exp2 units with a reference that
// moves only past kRescaleSlack, and O^T += V^T P^T over the 32 keys of the pair, whose
// k order (four keys of each block per lane group) is the one the S^T lanes already hold,
// so P needs no lane exchange. K rows are stored by slot (every load issued before any
// LDS store); V^T columns are gathered by slot (an empty slot reads a real key of its
// class, whose probability is 0).
constexpr int kWinThreads = 64 * kWinWaves;
// group record (kWinGroupInts ints): {first key block, end, queries, 0}, then 16 query
// positions (-1: none)

template <int D>
struct WinLds {
  static constexpr int KLD = D + 8;  // K row stride (bf16): 16-byte pad
  // K rows, V^T rows; with the bias, 17 fp16 one-hot rows and each slot's key coordinates
  static size_t bytes(int nslots, bool rel) {
    return (size_t)nslots * KLD * 2 + (size_t)D * (nslots + 8) * 2 + (rel ? kShortOneHotBytes + (size_t)nslots * 4 : 0);
  }
};

// REL: add the relative-position bias. A query's table row (rel_t, fp16, exp2 units)
// holds 32 entries, key rows at 0..15 and key columns at 16..31; one fp16 k-step of 32
// per key block adds it, its K operand one-hot in the key's row (lane groups 0, 1) or
// column (groups 2, 3), from 17 one-hot rows in LDS, the scores taken to exp2 units first.
template <int D, bool REL>
__global__ void __launch_bounds__(kWinThreads) __attribute__((amdgpu_waves_per_eu(4)))
attn_win_kernel(const bf16_t* __restrict__ Q, const bf16_t* __restrict__ Kt, const bf16_t* __restrict__ VT,
                bf16_t* __restrict__ O, const int* __restrict__ pos_slot, const int* __restrict__ slot_pos,
                const int* __restrict__ groups, const int* __restrict__ kblocks, const int* __restrict__ wave_begin,
                int n, int n_pad, int nslots, int heads, float c_log2, const f16_t* __restrict__ rel_t,
                const int* __restrict__ rel_kc) {
  using L = WinLds<D>;
  constexpr int KCH = D / 8;                                 // 16-byte chunks of a K row
  constexpr int KIT = (kShortMaxN * KCH + kWinThreads - 1) / kWinThreads;
  constexpr int VIT = (D * 32 + kWinThreads - 1) / kWinThreads;  // V^T chunks of 8 slots, 32 per row
  constexpr int KS = (D + 31) / 32;  // 32-wide k-steps of Q K^T; in the last one of D = 80
                                     // the lanes past D hold zeros in both operands
  constexpr int MD = D / 16;                                 // 16-row blocks of O^T
  static_assert(D % 16 == 0 && kShortMaxN <= kWinMaxSlots, "window kernel shapes");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int vld = nslots + 8;
  bf16_t* Ks = reinterpret_cast<bf16_t*>(smem);
  bf16_t* Vs = Ks + (size_t)nslots * L::KLD;
  const int sh = blockIdx.x;
  const int seg = sh / heads, h = sh - seg * heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, g = lane >> 4;
  const bf16_t* q_base = Q + (size_t)sh * n * D;
  const bf16_t* k_base = Kt + (size_t)sh * n * D;
  const bf16_t* v_base = VT + (size_t)sh * D * n_pad;

  // This wavefront's groups: the first group's query fragments (and bias row) are
  // requested before the fill, each next group's while the current one is computed.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int gb = wave_begin[wv], ge = wave_begin[wv + 1];
  bf16x8 qf[KS];
  f16x8 tf{};  // the query's bias entries 8 g .. + 7
  auto load_q = [&](int gi, int& qp, bf16x8* f, f16x8& t) {
    qp = groups[(size_t)gi * kWinGroupInts + 4 + r16];
    const int qrow = qp < 0 ? 0 : qp;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int d0 = ks * 32 + g * 8;
      f[ks] = *reinterpret_cast<const bf16x8*>(q_base + (size_t)qrow * D + min(d0, D - 8));
      if (d0 >= D) f[ks] = bf16x8{};
    }
    if constexpr (REL) t = *reinterpret_cast<const f16x8*>(rel_t + ((size_t)sh * n + qrow) * 32 + g * 8);
  };
  int qp = -1;
  if (gb < ge) load_q(gb, qp, qf, tf);

  // Fill, every load issued before any LDS store. K rows by position: chunk c = tid +
  // 512 i is position c / KCH, channels 8 (c % KCH), stored at the position's slot.
  i32x4 kv[KIT];
  int ks_slot[KIT];
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int c = tid + kWinThreads * i, p = min(c / KCH, n - 1), ch = c - (c / KCH) * KCH;
    kv[i] = *reinterpret_cast<const i32x4*>(k_base + (size_t)p * D + ch * 8);
    ks_slot[i] = pos_slot[p];
  }
  // V^T by position: chunk c = tid + 512 i is row c / 32, positions 8 (c % 32) .. + 7,
  // each element stored at its position's slot
  bf16x8 vv[VIT];
  i32x4 vs[VIT][2];
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int c = tid + kWinThreads * i, d = min(c >> 5, D - 1), j = c & 31;
    vv[i] = *reinterpret_cast<const bf16x8*>(v_base + (size_t)d * n_pad + min(8 * j, n_pad - 8));
    vs[i][0] = *reinterpret_cast<const i32x4*>(pos_slot + 8 * j);
    vs[i][1] = *reinterpret_cast<const i32x4*>(pos_slot + 8 * j + 4);
  }
  char* onehot = reinterpret_cast<char*>(Vs + (size_t)D * vld);
  int* key_rc = reinterpret_cast<int*>(onehot + kShortOneHotBytes);  // [nslots]: row | (16 + column) << 16
  int kc_own = 0;
  if constexpr (REL) {
    if (tid < nslots) kc_own = rel_kc[(size_t)seg * n + slot_pos[tid]];
  }
  // V^T rows zeroed first (the empty slots of a class's last block must hold finite
  // values: their probabilities are 0), while the loads are in flight; only LDS
  // operations are waited for before this barrier
  for (int i = tid; i < D * vld / 8; i += kWinThreads) reinterpret_cast<i32x4*>(Vs)[i] = i32x4{0, 0, 0, 0};
  asm volatile("" ::: "memory");  // the zero stores stay above the wait and the barrier
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(63) & lgkmcnt0_mask());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int i = 0; i < KIT; ++i) {
    const int c = tid + kWinThreads * i, ch = c - (c / KCH) * KCH;
    if (c / KCH < n) *reinterpret_cast<i32x4*>(Ks + ks_slot[i] * L::KLD + ch * 8) = kv[i];
  }
#pragma unroll
  for (int i = 0; i < VIT; ++i) {
    const int c = tid + kWinThreads * i, d = c >> 5, j = c & 31;
    if (d < D) {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (8 * j + e < n) Vs[d * vld + vs[i][e >> 2][e & 3]] = vv[i][e];
    }
  }
  if constexpr (REL) {
    if (tid < nslots) key_rc[tid] = kc_own;
    if (tid < 68) {  // row 8 + e: fp16 1.0 at element e; rows 0..7 and 16 zero
      const int row = tid >> 2, i = tid & 3, e = row - 8;
      reinterpret_cast<uint32_t*>(onehot)[tid] = (e == 2 * i ? 0x3C00u : 0u) | (e == 2 * i + 1 ? 0x3C000000u : 0u);
    }
  }
  __syncthreads();

  for (int gi = gb; gi < ge; ++gi) {
    const int* gr = groups + (size_t)gi * kWinGroupInts;
    const int kb_first = gr[0], kb_end = gr[1];
    int qp_next = -1;
    bf16x8 qf_next[KS] = {};
    f16x8 tf_next{};
    if (gi + 1 < ge) load_q(gi + 1, qp_next, qf_next, tf_next);
    f32x4 oacc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) oacc[md] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    float m_run = -INFINITY, l_run = 0.0f;
    // S^T of key block b for this lane's query: keys 16 b + 4 g .. + 3 (with the bias: in
    // exp2 units)
    auto scores = [&](int b) {
      f32x4 s{0.0f, 0.0f, 0.0f, 0.0f};
      const bf16_t* krow = Ks + (16 * b + r16) * L::KLD;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int d0 = ks * 32 + g * 8;
        bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + min(d0, D - 8));
        if (d0 >= D) kf = bf16x8{};
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[ks], s, 0, 0, 0);
      }
      if constexpr (REL) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] *= c_log2;
        const int kcs = key_rc[16 * b + r16];
        const int jj = g < 2 ? (kcs & 0xffff) : (kcs >> 16);
        const int row = min(max(jj - 8 * g + 8, 0), 16);
        const f16x8 af = *reinterpret_cast<const f16x8*>(onehot + row * 16);
        s = __builtin_amdgcn_mfma_f32_16x16x32_f16(af, tf, s, 0, 0, 0);
      }
      return s;
    };
    for (int kb = kb_first; kb < kb_end; kb += 2) {
      const bool two = kb + 1 < kb_end;
      const int e0 = kblocks[kb], e1 = two ? kblocks[kb + 1] : e0;
      const int b0 = e0 & 0xffff, b1 = e1 & 0xffff;
      f32x4 s0 = scores(b0), s1;
      if (two) {
        s1 = scores(b1);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) s1[i] = -INFINITY;
      }
      // empty slots of a block: masked (their K rows are not stored)
      const unsigned v0 = (unsigned)e0 >> 16, v1 = (unsigned)e1 >> 16;
      if (v0 != 0xffffu) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((v0 >> (4 * g + i)) & 1u)) s0[i] = -INFINITY;
      }
      if (two && v1 != 0xffffu) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (!((v1 >> (4 * g + i)) & 1u)) s1[i] = -INFINITY;
      }
      float mx = fmaxf(max3f(s0[0], s0[1], s0[2]), max3f(s0[3], s1[0], s1[1]));
      mx = max3f(mx, s1[2], s1[3]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = max_xor32(mx);
      const float m_new = fmaxf(m_run, REL ? mx : mx * c_log2);
      if (__builtin_amdgcn_ballot_w64(m_new > m_run + kRescaleSlack) != 0) {
        const float alpha = m_new > m_run ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;
        l_run *= alpha;
#pragma unroll
        for (int md = 0; md < MD; ++md)
#pragma unroll
          for (int i = 0; i < 4; ++i) oacc[md][i] *= alpha;
        m_run = m_new;
      }
      const float mref = fmaxf(m_run, -3.40282347e38f);
      bf16x8 pf;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pf[i] = to_bf16(__builtin_amdgcn_exp2f(REL ? s0[i] - mref : __builtin_fmaf(s0[i], c_log2, -mref)));
        pf[4 + i] = to_bf16(__builtin_amdgcn_exp2f(REL ? s1[i] - mref : __builtin_fmaf(s1[i], c_log2, -mref)));
      }
      // the denominator sums exactly the bf16 probabilities V is multiplied with
#pragma unroll
      for (int i = 0; i < 8; i += 2) l_run = sum_bf16_pair(pf[i], pf[i + 1], l_run);
      // O^T += V^T P^T: rows d = 16 md + l % 16, k order = keys 4 g .. + 3 of b0, then of b1
#pragma unroll
      for (int md = 0; md < MD; ++md) {
        const bf16_t* vrow = Vs + (16 * md + r16) * vld + 4 * g;
        const bf16x4 va = *reinterpret_cast<const bf16x4*>(vrow + 16 * b0);
        const bf16x4 vb = *reinterpret_cast<const bf16x4*>(vrow + 16 * b1);
        const bf16x8 vf = {va[0], va[1], va[2], va[3], vb[0], vb[1], vb[2], vb[3]};
        oacc[md] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, oacc[md], 0, 0, 0);
      }
    }
    float l_tot = l_run + __shfl_xor(l_run, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    // O rows in 16-byte pieces: lanes g and g ^ 1 (same query) trade halves, so that for
    // the blocks md, md + 1 an even lane holds d = 16 md + 4 g .. + 7 and an odd lane
    // d = 16 (md + 1) + 4 (g - 1) .. + 7 (with an odd MD the last block is written by
    // the even lanes alone)
    const float inv_l = 1.0f / l_tot;
    const bool odd = g & 1;
    bf16_t* o_row = O + ((size_t)seg * n + (qp < 0 ? 0 : qp)) * ((size_t)heads * D) + (size_t)h * D;
#pragma unroll
    for (int mp = 0; mp < MD; mp += 2) {
      const int m0 = mp, m1 = mp + 1 < MD ? mp + 1 : mp;
      bf16x4 a, b;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = to_bf16(oacc[m0][i] * inv_l);
        b[i] = to_bf16(oacc[m1][i] * inv_l);
      }
      const i32x2 ai = __builtin_bit_cast(i32x2, a), bi = __builtin_bit_cast(i32x2, b);
      const int r0 = __shfl_xor(odd ? ai[0] : bi[0], 16, 64);
      const int r1 = __shfl_xor(odd ? ai[1] : bi[1], 16, 64);
      const i32x4 w = odd ? i32x4{r0, r1, bi[0], bi[1]} : i32x4{ai[0], ai[1], r0, r1};
      const int d = odd ? 16 * m1 + 4 * (g - 1) : 16 * m0 + 4 * g;
      if (qp >= 0 && (mp + 1 < MD || !odd)) *reinterpret_cast<i32x4*>(o_row + d) = w;
    }
    qp = qp_next;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = qf_next[ks];
    if constexpr (REL) tf = tf_next;
  }
}

// ---------------------------------------------------------------- SIMT kernel (any pattern)

// REL: add the relative-position bias, rel_t[sh, query, kc & 0xffff] +
// rel_t[sh, query, kc >> 16] for the key's coordinates kc = rel_kc[seg, key] (fp32
// tables of rel_tj entries per query, exp2 units).
template <typename T, int D, bool REL>
__global__ void __launch_bounds__(64) attn_simt_kernel(const T* __restrict__ Q, const T* __restrict__ Kt,
                                                       const T* __restrict__ VT, T* __restrict__ O,
                                                       const int* __restrict__ row_ptr,
                                                       const int* __restrict__ col_idx,
                                                       const int* __restrict__ tile_start,
                                                       const int* __restrict__ tile_len, int n, int n_pad, int heads,
                                                       int chunks, int qpw, float c_log2, const float* __restrict__ rel_t,
                                                       const int* __restrict__ rel_kc, int tj) {
  const int qt = blockIdx.x / chunks, chunk = blockIdx.x - (blockIdx.x / chunks) * chunks;
  const int h = blockIdx.y, seg = blockIdx.z;
  const int len = tile_len[qt];
  const size_t sh = (size_t)seg * heads + h;
  float qv[D], acc[D];
  // qpw queries per workgroup (64, 32 or 4), each served by kpar = 64 / qpw threads that
  // take every kpar-th key and merge their softmax states at the end
  const int kpar = 64 / qpw, part = threadIdx.x / qpw;
  const int local = chunk * qpw + (threadIdx.x - part * qpw);
  const bool active = local < len;
  const int qi = tile_start[qt] + (active ? local : 0);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = active ? (float)Q[(sh * n + qi) * D + d] : 0.0f;
    acc[d] = 0.0f;
  }
  float m_run = -INFINITY, l_run = 0.0f;
  const float* trow = REL ? rel_t + (sh * n + qi) * (size_t)tj : nullptr;
  // The V rows of a kept tile's keys (from the V^T columns), in chunks of up to KCH keys,
  // are staged in LDS and read by every thread as 16-byte broadcasts. With one thread
  // per query (kpar = 1) every lane reads the same K row, so K comes straight from
  // global memory (uniform addresses: scalar loads, which measured faster than LDS
  // broadcasts); with several threads per query the lanes read kpar different rows, so
  // the chunk's K rows are staged too. A thread issues 16 of its staging loads before it
  // stores any (one round trip per 16 values; storing each value as it arrived cost a
  // round trip per value).
  constexpr int KCH = D <= 80 ? 64 : 32;  // keys per staged chunk (LDS: 2 KCH D floats)
  __shared__ __attribute__((aligned(16))) float vs[KCH][D];
  __shared__ __attribute__((aligned(16))) float ks[KCH][D];
  const bool stage_k = kpar > 1;
  for (int t = row_ptr[qt]; t < row_ptr[qt + 1]; ++t) {
    const int kt = col_idx[t];
    const int k0 = tile_start[kt], kl = tile_len[kt];
    for (int c0 = 0; c0 < kl; c0 += KCH) {
      const int cl = min(KCH, kl - c0);
      __syncthreads();  // the previous chunk has been read
      {
        // V^T rows dv, columns k0 + c0 + iv: thread (g, iv) takes iv = t mod cl and
        // channels g, g + G, ... (G = 64 / cl groups; coalesced along iv)
        const int G = 64 / cl, iv = threadIdx.x % cl, g = threadIdx.x / cl;
        if (g < G) {
          const T* vcol = VT + sh * D * n_pad + k0 + c0 + iv;
          for (int db = g; db < D; db += 16 * G) {
            float v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
              const int dv = db + u * G;
              v[u] = dv < D ? (float)vcol[(size_t)dv * n_pad] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 16; ++u)
              if (db + u * G < D) vs[iv][db + u * G] = v[u];
          }
        }
      }
      if (stage_k) {
        const T* kc = Kt + (sh * n + k0 + c0) * D;  // the chunk's K rows are contiguous
        for (int eb = threadIdx.x; eb < cl * D; eb += 16 * 64) {
          float v[16];
#pragma unroll
          for (int u = 0; u < 16; ++u) v[u] = eb + 64 * u < cl * D ? (float)kc[eb + 64 * u] : 0.0f;
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            const int e = eb + 64 * u;
            if (e < cl * D) ks[e / D][e % D] = v[u];
          }
        }
      }
      __syncthreads();
      for (int j = part; j < cl; j += kpar) {
        const int kj = k0 + c0 + j;
        float sc = 0.0f;
        if (stage_k) {
          // four partial sums (channels d mod 4), added in a fixed order
          const f32x4* kr4 = reinterpret_cast<const f32x4*>(&ks[j][0]);
          float s4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int d4 = 0; d4 < D / 4; ++d4) {
            const f32x4 k4 = kr4[d4];
#pragma unroll
            for (int e = 0; e < 4; ++e) s4[e] = fmaf(qv[4 * d4 + e], k4[e], s4[e]);
          }
          sc = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        } else {
          const T* kr = Kt + (sh * n + kj) * D;
#pragma unroll
          for (int d = 0; d < D; ++d) sc = fmaf(qv[d], (float)kr[d], sc);
        }
        sc *= c_log2;
        if constexpr (REL) {
          const int kc = rel_kc[(size_t)seg * n + kj];
          sc += trow[kc & 0xffff] + trow[kc >> 16];
        }
        const float m_new = fmaxf(m_run, sc);
        const float alpha = exp2f(m_run - m_new);
        const float p = exp2f(sc - m_new);
        l_run = l_run * alpha + p;
        m_run = m_new;
        const f32x4* vr = reinterpret_cast<const f32x4*>(&vs[j][0]);
#pragma unroll
        for (int d4 = 0; d4 < D / 4; ++d4) {
          const f32x4 v4 = vr[d4];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * d4 + e] = fmaf(p, v4[e], acc[4 * d4 + e] * alpha);
        }
      }
    }
  }
  // merge the kpar partial states of a query (lanes q, q + qpw, ...) in a fixed
  // butterfly order; a part that saw no key (m = -inf) carries weight 0
  for (int o = qpw; o < 64; o <<= 1) {
    const float m_o = __shfl_xor(m_run, o, 64), l_o = __shfl_xor(l_run, o, 64);
    const float mm = fmaxf(m_run, m_o);
    const float a0 = m_run == -INFINITY ? 0.0f : exp2f(m_run - mm);
    const float a1 = m_o == -INFINITY ? 0.0f : exp2f(m_o - mm);
#pragma unroll
    for (int d = 0; d < D; ++d) acc[d] = acc[d] * a0 + __shfl_xor(acc[d], o, 64) * a1;
    l_run = l_run * a0 + l_o * a1;
    m_run = mm;
  }
  if (!active || part != 0) return;
  T* orow = O + ((size_t)seg * n + qi) * ((size_t)heads * D) + (size_t)h * D;
  const float inv_l = 1.0f / l_run;
#pragma unroll
  for (int d = 0; d < D; ++d) orow[d] = from_f32<T>(acc[d] * inv_l);
}

// ---------------------------------------------------------------- launchers

// workgroups of the long-segment kernel for head_dim (64 or 80) resident at once
int attn_long_resident_wgs(int device, int head_dim) {
  const void* kern = head_dim == 80 ? (const void*)attn_d80_kernel : (const void*)attn_mfma64_kernel;
  const int lds = head_dim == 80 ? kD80Lds : kAttnLds;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess) return 0;
  if (hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 64 * kAttnWaves, lds) != hipSuccess) return 0;
  return cus * per_cu;
}

bool attn_long_supported(const sparsesam_plan& p) {
  return p.desc.dtype == SPARSESAM_BF16 && (p.desc.head_dim == 64 || p.desc.head_dim == 80) && p.desc.block == 64 &&
         p.s % 64 == 0 && p.nt32 == 0;
}

size_t attn_partial_bytes(const sparsesam_plan& p, int segments) {
  if (!attn_long_supported(p)) return 0;
  return (size_t)p.n_slots * segments * p.desc.heads * kTile * part_ld(p.desc.head_dim) * sizeof(float);
}

template <typename T, int D, bool REL = false>
static hipError_t run_simt(const sparsesam_plan& p, int segments, const T* q, const T* k, const T* vt, T* o,
                           float c_log2, hipStream_t st, const float* rel_t = nullptr, const int* rel_kc = nullptr) {
  // queries per workgroup: 64 for 64-token tiles, 32 or 16 for tiles up to 32 tokens, and
  // 4 (16 threads per query, four workgroups per 16-token tile) for tiles of at most 16,
  // so that short tiles keep every thread busy with a share of the keys and spread over
  // more CUs
  const int qpw = p.desc.block >= 64 ? 64 : p.desc.block > 16 ? 32 : 4;
  const int chunks = (p.desc.block + qpw - 1) / qpw;
  dim3 grid(p.tiles * chunks, p.desc.heads, segments);
  hipLaunchKernelGGL((attn_simt_kernel<T, D, REL>), grid, dim3(64), 0, st, q, k, vt, o, p.d_row_ptr, p.d_col_idx,
                     p.d_tile_start, p.d_tile_len, p.n, p.n_pad, p.desc.heads, chunks, qpw, c_log2, rel_t, rel_kc,
                     p.rel_tj);
  return hipGetLastError();
}

// The short-segment kernel for a plan: one workgroup per (segment, head), the mask in
// one or two k-steps.
template <int D, bool REL>
static hipError_t launch_short(const sparsesam_plan& p, int units, const bf16_t* q, const bf16_t* k,
                               const bf16_t* vt, bf16_t* o, float c_log2, const f16_t* tb, const int* kc,
                               hipStream_t st) {
  const size_t lds = ShortLds<D>::bytes(p.nt32);
  auto kern = p.mask_ksteps == 2 ? attn_short_kernel<D, REL, 2> : attn_short_kernel<D, REL, 1>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(kShortThreads), lds, st, q, k, vt, o, p.d_pos_tile, p.d_mask_class,
                     p.d_mask_row, p.d_any32, p.n, p.n_pad, p.nt32, p.desc.heads, c_log2, tb, kc);
  return hipGetLastError();
}

// Unit order of a launch of several rounds: the head-major order (attn_unit) when the
// work it gives the busiest workgroup is no more than the snake order gives, from each
// item's steps (tiles / key parities; a four-parity step loads four tiles, 1.25 steps'
// time) plus 2.6 steps of prologue and epilogue per unit. Units are assigned statically,
// so both schedules are known here.
static bool attn_head_major(const sparsesam_plan& p, int seg_heads, int nwg) {
  const int total = p.n_items * seg_heads;
  if (nwg <= 0 || total <= nwg) return false;
  std::vector<double> cost(p.n_items);
  for (int i = 0; i < p.n_items; ++i) {
    const int* it = &p.items[(size_t)8 * i];
    const int par = std::max(1, it[3] >> 4);
    cost[i] = (double)((it[1] - it[0] + par - 1) / par) * (par == 4 ? 1.25 : 1.0) + 2.6;
  }
  double snake = 0.0, head = 0.0;
  for (int w = 0; w < nwg; ++w) {
    double a = 0.0, b = 0.0;
    for (int r = 0;; ++r) {
      const int u = r * nwg + ((r & 1) ? nwg - 1 - w : w);
      if (u >= total) break;
      a += cost[u / seg_heads];
    }
    const int x = w % kXcds, off = x * (nwg / kXcds) + std::min(x, nwg % kXcds) + w / kXcds;
    for (int up = off; up < total; up += nwg) b += cost[up % p.n_items];
    snake = std::max(snake, a);
    head = std::max(head, b);
  }
  return head <= snake * 1.001;
}

// The window kernel on 16-key blocks: one workgroup per (segment, head).
template <int D, bool REL>
static hipError_t launch_win(const sparsesam_plan& p, int units, const bf16_t* q, const bf16_t* k, const bf16_t* vt,
                             bf16_t* o, float c_log2, const f16_t* tb, const int* kc, hipStream_t st) {
  const size_t lds = WinLds<D>::bytes(p.win_nslots, REL);
  auto kern = attn_win_kernel<D, REL>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)units), dim3(kWinThreads), lds, st, q, k, vt, o, p.d_win_pos_slot,
                     p.d_win_slot_pos, p.d_win_groups, p.d_win_kb, p.d_win_wave, p.n, p.n_pad, p.win_nslots,
                     p.desc.heads, c_log2, tb, kc);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attention(const sparsesam_plan& p, int segments, const T* q, const T* k, const T* vt, T* o,
                            float scale, void* partial, hipStream_t st) {
  if (segments <= 0) return hipSuccess;
  const float c_log2 = scale * 1.4426950408889634f;
  if constexpr (sizeof(T) == 2) {
    if ((p.win_nslots > 0 || p.nt32 > 0) && (p.desc.head_dim == 64 || p.desc.head_dim == 80)) {
      const int units = segments * p.desc.heads;
      const auto* qb = reinterpret_cast<const bf16_t*>(q);
      const auto* kb = reinterpret_cast<const bf16_t*>(k);
      const auto* vb = reinterpret_cast<const bf16_t*>(vt);
      auto* ob = reinterpret_cast<bf16_t*>(o);
      if (p.win_nslots > 0)
        return p.desc.head_dim == 64 ? launch_win<64, false>(p, units, qb, kb, vb, ob, c_log2, nullptr, nullptr, st)
                                     : launch_win<80, false>(p, units, qb, kb, vb, ob, c_log2, nullptr, nullptr, st);
      return p.desc.head_dim == 64 ? launch_short<64, false>(p, units, qb, kb, vb, ob, c_log2, nullptr, nullptr, st)
                                   : launch_short<80, false>(p, units, qb, kb, vb, ob, c_log2, nullptr, nullptr, st);
    }
    if (attn_long_supported(p)) {
      const bool d80 = p.desc.head_dim == 80;
      const void* kern = d80 ? (const void*)attn_d80_kernel : (const void*)attn_mfma64_kernel;
      const int lds = d80 ? kD80Lds : kAttnLds;
      const int seg_heads = segments * p.desc.heads;
      hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      const int units = p.n_items * seg_heads;
      dim3 grid((unsigned)std::min(units, std::max(1, p.attn_resident_wgs)));
      const int hm = attn_head_major(p, seg_heads, (int)grid.x) ? 1 : 0;
      const auto* items = reinterpret_cast<const int4*>(p.d_items);
      if (d80)
        hipLaunchKernelGGL(attn_d80_kernel, grid, dim3(64 * kAttnWaves), lds, st, q, k, vt, o, items, p.d_col_idx,
                           p.d_tile_start, p.n, p.n_pad, p.desc.heads, seg_heads, p.n_items, c_log2,
                           static_cast<float*>(partial), hm);
      else
        hipLaunchKernelGGL(attn_mfma64_kernel, grid, dim3(64 * kAttnWaves), lds, st, q, k, vt, o, items,
                           p.d_col_idx, p.d_tile_start, p.n, p.n_pad, p.desc.heads, seg_heads, p.n_items, c_log2,
                           static_cast<float*>(partial), hm);
      e = hipGetLastError();
      if (e != hipSuccess || p.n_split_rows == 0) return e;
      const int waves = p.n_split_rows * seg_heads * kTile;
      if (d80)
        hipLaunchKernelGGL(attn_combine_kernel<80>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                           static_cast<const float*>(partial), p.d_splits, p.d_tile_start, o, p.n, p.desc.heads,
                           seg_heads, waves);
      else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                           static_cast<const float*>(partial), p.d_splits, p.d_tile_start, o, p.n, p.desc.heads,
                           seg_heads, waves);
      return hipGetLastError();
    }
  }
  switch (p.desc.head_dim) {
    case 64: return run_simt<T, 64>(p, segments, q, k, vt, o, c_log2, st);
    case 80: return run_simt<T, 80>(p, segments, q, k, vt, o, c_log2, st);
    case 32: return run_simt<T, 32>(p, segments, q, k, vt, o, c_log2, st);
    case 128: return run_simt<T, 128>(p, segments, q, k, vt, o, c_log2, st);
    default: return hipErrorInvalidValue;
  }
}

bool attn_relpos_fused(const sparsesam_plan& p) {
  return p.desc.dtype == SPARSESAM_BF16 && (p.desc.head_dim == 64 || p.desc.head_dim == 80) &&
         attn_long_supported(p) && p.rel_tj == kRelTj && p.rel_xoff == 64;
}

template <typename T>
hipError_t launch_attention_relpos(const sparsesam_plan& p, int segments, const T* q, const T* k, const T* vt, T* o,
                                   float scale, const int* perm, const float* rel_h, const float* rel_w, void* table,
                                   int* kc, void* partial, hipStream_t st) {
  if (segments <= 0) return hipSuccess;
  if (p.rel_tj <= 0) return hipErrorInvalidValue;
  const float c_log2 = scale * 1.4426950408889634f;
  if constexpr (sizeof(T) == 2) {
    if (attn_relpos_fused(p)) {
      auto* tb = static_cast<f16_t*>(table);
      hipError_t e = launch_relpos_table<bf16_t, f16_t>(p, segments, reinterpret_cast<const bf16_t*>(q), perm,
                                                         rel_h, rel_w, tb, kc, st);
      if (e != hipSuccess) return e;
      const bool d80 = p.desc.head_dim == 80;
      const void* kern = d80 ? (const void*)attn_d80_rel_kernel : (const void*)attn_mfma64_rel_kernel;
      const int lds = d80 ? kD80RelLds : kRelLds;
      e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
      if (e != hipSuccess) return e;
      const int seg_heads = segments * p.desc.heads;
      const int units = p.n_items * seg_heads;
      dim3 grid((unsigned)std::min(units, std::max(1, p.attn_resident_wgs)));
      const int hm = attn_head_major(p, seg_heads, (int)grid.x) ? 1 : 0;
      const auto* items = reinterpret_cast<const int4*>(p.d_items);
      const auto* qb = reinterpret_cast<const bf16_t*>(q);
      const auto* kb = reinterpret_cast<const bf16_t*>(k);
      const auto* vb = reinterpret_cast<const bf16_t*>(vt);
      auto* ob = reinterpret_cast<bf16_t*>(o);
      if (d80)
        hipLaunchKernelGGL(attn_d80_rel_kernel, grid, dim3(64 * kAttnWaves), lds, st, qb, kb, vb, ob, items,
                           p.d_col_idx, p.d_tile_start, p.n, p.n_pad, p.desc.heads, seg_heads, p.n_items, c_log2,
                           static_cast<float*>(partial), tb, kc, hm);
      else
        hipLaunchKernelGGL(attn_mfma64_rel_kernel, grid, dim3(64 * kAttnWaves), lds, st, qb, kb, vb, ob, items,
                           p.d_col_idx, p.d_tile_start, p.n, p.n_pad, p.desc.heads, seg_heads, p.n_items, c_log2,
                           static_cast<float*>(partial), tb, kc, hm);
      e = hipGetLastError();
      if (e != hipSuccess || p.n_split_rows == 0) return e;
      const int waves = p.n_split_rows * seg_heads * kTile;
      if (d80)
        hipLaunchKernelGGL(attn_combine_kernel<80>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                           static_cast<const float*>(partial), p.d_splits, p.d_tile_start, ob, p.n, p.desc.heads,
                           seg_heads, waves);
      else
        hipLaunchKernelGGL(attn_combine_kernel<64>, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st,
                           static_cast<const float*>(partial), p.d_splits, p.d_tile_start, ob, p.n, p.desc.heads,
                           seg_heads, waves);
      return hipGetLastError();
    }
  }
  if constexpr (sizeof(T) == 2) {
    if ((p.nt32 > 0 || p.win_nslots > 0) && p.rel_tj == 32 && (p.desc.head_dim == 64 || p.desc.head_dim == 80)) {
      auto* tb = static_cast<f16_t*>(table);
      hipError_t e = launch_relpos_table<bf16_t, f16_t>(p, segments, reinterpret_cast<const bf16_t*>(q), perm,
                                                         rel_h, rel_w, tb, kc, st);
      if (e != hipSuccess) return e;
      const int units = segments * p.desc.heads;
      const auto* qb = reinterpret_cast<const bf16_t*>(q);
      const auto* kb = reinterpret_cast<const bf16_t*>(k);
      const auto* vb = reinterpret_cast<const bf16_t*>(vt);
      auto* ob = reinterpret_cast<bf16_t*>(o);
      if (p.win_nslots > 0)
        return p.desc.head_dim == 80 ? launch_win<80, true>(p, units, qb, kb, vb, ob, c_log2, tb, kc, st)
                                     : launch_win<64, true>(p, units, qb, kb, vb, ob, c_log2, tb, kc, st);
      return p.desc.head_dim == 80 ? launch_short<80, true>(p, units, qb, kb, vb, ob, c_log2, tb, kc, st)
                                   : launch_short<64, true>(p, units, qb, kb, vb, ob, c_log2, tb, kc, st);
    }
  }
  // every other plan: fp32 tables and the SIMT kernel
  auto* tf = static_cast<float*>(table);
  hipError_t e = launch_relpos_table<T, float>(p, segments, q, perm, rel_h, rel_w, tf, kc, st);
  if (e != hipSuccess) return e;
  switch (p.desc.head_dim) {
    case 64: return run_simt<T, 64, true>(p, segments, q, k, vt, o, c_log2, st, tf, kc);
    case 80: return run_simt<T, 80, true>(p, segments, q, k, vt, o, c_log2, st, tf, kc);
    case 32: return run_simt<T, 32, true>(p, segments, q, k, vt, o, c_log2, st, tf, kc);
    case 128: return run_simt<T, 128, true>(p, segments, q, k, vt, o, c_log2, st, tf, kc);
    default: return hipErrorInvalidValue;
  }
}

template hipError_t launch_attention_relpos<float>(const sparsesam_plan&, int, const float*, const float*,
                                                   const float*, float*, float, const int*, const float*,
                                                   const float*, void*, int*, void*, hipStream_t);
template hipError_t launch_attention_relpos<bf16_t>(const sparsesam_plan&, int, const bf16_t*, const bf16_t*,
                                                    const bf16_t*, bf16_t*, float, const int*, const float*,
                                                    const float*, void*, int*, void*, hipStream_t);

template hipError_t launch_attention<float>(const sparsesam_plan&, int, const float*, const float*, const float*,
                                            float*, float, void*, hipStream_t);
template hipError_t launch_attention<bf16_t>(const sparsesam_plan&, int, const bf16_t*, const bf16_t*, const bf16_t*,
                                             bf16_t*, float, void*, hipStream_t);

}  // namespace sparsesam

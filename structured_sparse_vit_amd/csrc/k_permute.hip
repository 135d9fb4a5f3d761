// Stripe-sort permutation and keep-set of every segment of an image.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention,
// stripe-sort bullet: tokens are sorted by importance, the sorted list is viewed as
// a matrix and transposed before flattening, which spreads the important tokens over
// the whole sequence. Part 2 (Residual-Consistency MLP), token routing bullet: the
// keep-set is the top of the same deterministic order.
//
// The order is total: importance descending (-0.0 == +0.0, NaN after every number,
// pad slots after every real slot), then slot ascending -- or, for the plan's other
// orderings (Z-order, Hilbert, seeded random; the same page's abstract and the method
// registry of the SparseSAM README name them), an ascending position-derived key with
// the same tie and pad rules. A slot's rank is therefore
// the number of slots that precede it, and everything follows from the rank alone:
// rank rho sits at stripe rho % g, offset rho / g, i.e. position (rho % g) * S + rho / g,
// and the slot is in the keep-set iff rho < K, at index rho of the segment's part of
// the keep-set list. No sorted list is ever materialised.
//
// The same kernel selects the keep-set of plans whose routing follows a score (the
// squared attention update of a block): the score takes the place of importance (with
// the importance order forced), it may arrive as `parts` partial sums per token that the
// key fill adds in order, and perm / inv are not written.
//
// rank_kernel: one workgroup per (segment, chunk of slots). Its lanes count, for the
// chunk's slots, the preceding slots within shares of the segment's keys (held in LDS
// as 64-bit order words); lanes of one slot fold their counts with shuffles, the
// wavefronts' shares are summed in LDS, and one lane per slot writes perm, inv and --
// when the rank is below K -- the keep-set entry. The split is chosen so a single
// image's 4096 slots still spread over 256 workgroups.
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));

// 32-bit key that orders descending importance ascending: larger value -> smaller key.
__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0xFFFFFFFEu;       // NaN: after every number
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0.0 -> +0.0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
constexpr uint32_t kPadKey = 0xFFFFFFFFu;  // pad slots: after every real slot

// Ascending keys of the other token orders (sparsesam_ordering), from a slot's position
// (y, x) in its segment. All stay below kPadKey.
// Z-order: bit b of x at bit 2b, bit b of y at bit 2b + 1.
__device__ __forceinline__ uint32_t zorder_key(uint32_t y, uint32_t x) {
  uint32_t c = 0;
#pragma unroll
  for (int b = 0; b < 16; ++b) c |= (((x >> b) & 1u) << (2 * b)) | (((y >> b) & 1u) << (2 * b + 1));
  return c;
}
// Hilbert curve over a side x side square (a power of two), from the coarsest level down:
// the quadrants are visited (x, y) = (lo, lo), (lo, hi), (hi, hi), (hi, lo); inside the
// first one the half-size curve is mirrored in the main diagonal, inside the last one in
// the anti-diagonal, so the cell's coordinates are mapped the same way before the next
// level.
__device__ __forceinline__ uint32_t hilbert_key(int side, int y, int x) {
  uint32_t d = 0;
  for (int h = side >> 1; h >= 1; h >>= 1) {
    const int qx = x >= h, qy = y >= h;
    int lx = x - h * qx, ly = y - h * qy, q;
    if (qy) {
      q = qx ? 2 : 1;
    } else if (!qx) {
      q = 0;
      const int t = lx;  // main-diagonal mirror
      lx = ly;
      ly = t;
    } else {
      q = 3;
      const int t = h - 1 - ly;  // anti-diagonal mirror
      ly = h - 1 - lx;
      lx = t;
    }
    d += (uint32_t)(q * h * h);
    x = lx;
    y = ly;
  }
  return d;
}
// Seeded random order: top 31 bits of the first SplitMix64 output (Steele, Lea and Flood,
// OOPSLA 2014) from state seed * 2^32 + slot.
__device__ __forceinline__ uint32_t random_key(uint32_t seed, uint32_t slot) {
  uint64_t z = (((uint64_t)seed << 32) | slot) + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  z ^= z >> 31;
  return (uint32_t)(z >> 33);
}

// rank_kernel layout: a workgroup of kw wavefronts ranks tpw slots of one segment
// (tpw = 16 or 64). The segment's keys sit in LDS as 64-bit words (order key << 32 |
// slot), so "slot j precedes slot s" is one unsigned compare of two words and every
// 16-byte read brings two keys. Lane l of a wavefront serves slot l % tpw and key pair
// residue class l / tpw (mod 64 / tpw); wavefront w takes the w-th share of the keys.
// For N = 4096 that is 256 workgroups of 16 wavefronts, every lane comparing 64 keys.
//
// NV > 0 (one wavefront per slot: tpw == kw == 16) also writes the block's first
// LayerNorm: wavefront w loads the token row of slot chunk * 16 + w (C = 256 NV
// channels) while the keys are ranked, and once the slot's stripe-sorted position p is
// known writes LayerNorm(row) as bf16 to ln_out[seg * n + p] -- the rows the gathered
// LayerNorm would write through perm, bit for bit (the same LnRow code).
constexpr int kMaxRankWaves = 16;

struct RankLn {
  const float* x = nullptr;
  long long x_rows = 0;
  const float* gamma = nullptr;
  const float* beta = nullptr;
  bf16_t* out = nullptr;
};

template <int NV>
__global__ void __launch_bounds__(64 * kMaxRankWaves) rank_kernel(const float* __restrict__ imp, SegmentMap map,
                                                                  int n, int stripes, int chunks, int tpw,
                                                                  const int* __restrict__ seg_k,
                                                                  const int* __restrict__ seg_off,
                                                                  int routed_per_image, int* __restrict__ perm,
                                                                  int* __restrict__ inv, int* __restrict__ routed,
                                                                  int ordering, uint32_t seed, int seg_w,
                                                                  int hilbert_side, int parts,
                                                                  float* __restrict__ score_out, RankLn ln) {
  extern __shared__ __attribute__((aligned(16))) uint64_t key_lds[];  // padded to a multiple of 64
  __shared__ int part[kMaxRankWaves * 64];
  __shared__ int pos_lds[kMaxRankWaves];
  const int seg = blockIdx.x / chunks, chunk = blockIdx.x - (blockIdx.x / chunks) * chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = blockDim.x >> 6;
  const int tokens = map.grid_h * map.grid_w;
  const int img = map.f_spi.div(seg);
  const float* im = imp + (size_t)img * tokens * parts;
  // a token's key value: imp[token], or the in-order sum of its `parts` partials
  auto value = [&](int tok) {
    if (parts == 1) return im[tok];
    const float* pp = im + (size_t)tok * parts;
    float v = pp[0];
    for (int c = 1; c < parts; ++c) v = v + pp[c];
    return v;
  };
  const int n64 = (n + 63) & ~63;
  // keys past n are pad keys with index >= n: they never precede a real slot. Four
  // slots per thread at a time, their importance loads all issued before the first
  // key is formed (the index is clamped to a real token; pads discard the value).
  constexpr int kFillUnroll = 4;
  for (int base = 0; base < n64; base += kFillUnroll * (int)blockDim.x) {
    int rows[kFillUnroll];
    float vals[kFillUnroll];
#pragma unroll
    for (int u = 0; u < kFillUnroll; ++u) {
      const int s = base + tid + u * (int)blockDim.x;
      rows[u] = s < n ? map.row_of(seg, s) : -1;
      vals[u] = 0.0f;
      if (ordering == SPARSESAM_ORDER_IMPORTANCE && parts == 1) vals[u] = im[max(rows[u] - img * tokens, 0)];
    }
    if (parts > 1) {
#pragma unroll
      for (int u = 0; u < kFillUnroll; ++u)
        if (rows[u] >= 0) vals[u] = value(rows[u] - img * tokens);
    }
#pragma unroll
    for (int u = 0; u < kFillUnroll; ++u) {
      const int s = base + tid + u * (int)blockDim.x;
      if (s >= n64) break;
      uint32_t k = kPadKey;
      if (rows[u] >= 0) {
        if (ordering == SPARSESAM_ORDER_IMPORTANCE) {
          k = desc_key(vals[u]);
        } else {
          const int y = s / seg_w, x = s - (s / seg_w) * seg_w;
          k = ordering == SPARSESAM_ORDER_ZORDER    ? zorder_key((uint32_t)y, (uint32_t)x)
              : ordering == SPARSESAM_ORDER_HILBERT ? hilbert_key(hilbert_side, y, x)
                                                    : random_key(seed, (uint32_t)s);
        }
      }
      key_lds[s] = ((uint64_t)k << 32) | (uint32_t)s;
    }
  }
  // the LayerNorm row of this wavefront's slot, requested after the fill's importance
  // loads (loads retire in order), so that it arrives during the LDS-only ranking loop
  LnRow<(NV > 0 ? NV : 1)> lrow;
  int ln_src = -1;
  if constexpr (NV > 0) {
    const int sl = chunk * tpw + wave;
    ln_src = sl < n ? map.row_of(seg, sl) : -1;
    if (ln_src >= ln.x_rows) ln_src = -1;
    if (ln_src >= 0) lrow.load(ln.x + (size_t)ln_src * (NV * 256), ln.gamma, ln.beta, lane);
  }
  __syncthreads();
  const int subs = 64 / tpw;  // lanes per slot
  const int slot = chunk * tpw + (lane % tpw);
  const int sub = lane / tpw;
  const uint64_t mine = slot < n ? key_lds[slot] : 0ull;
  // this wavefront's share of the keys: [j0, j1), a multiple of 64 long
  const int per = ((n64 / 64 + kw - 1) / kw) * 64;
  const int j0 = wave * per, j1 = min(n64, j0 + per);
  int cnt = 0;
  // each lane reads key pairs jb + 2 (sub + subs u) (16 bytes) for u = 0..3
  for (int jb = j0; jb < j1; jb += 8 * subs) {
    uint64_t kk[8];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const auto v = *reinterpret_cast<const u64x2*>(key_lds + jb + 2 * (sub + subs * u));
      kk[2 * u] = v[0];
      kk[2 * u + 1] = v[1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) cnt += kk[u] < mine;
  }
  // the 64 / tpw lanes of one slot are tpw apart: fold them
  for (int o = tpw; o < 64; o <<= 1) cnt += __shfl_xor(cnt, o, 64);
  if (lane < tpw) part[wave * 64 + lane] = cnt;
  __syncthreads();
  // slot chunk * tpw + tid's rank and stripe-sorted position (threads tid < tpw); with
  // NV > 0 the positions are published first, so that the LayerNorm rows do not wait
  // for the index writes
  const int sl_me = chunk * tpw + tid;
  const bool slot_thread = tid < tpw && sl_me < n;
  int rank = 0, p = 0;
  if (slot_thread) {
#pragma unroll 4
    for (int w = 0; w < kw; ++w) rank += part[w * 64 + tid];
    const int S = n / stripes;
    p = (rank % stripes) * S + rank / stripes;
    if constexpr (NV > 0) pos_lds[tid] = p;
  }
  if constexpr (NV > 0) __syncthreads();  // every slot's position is in pos_lds
  if (slot_thread) {
    const size_t base = (size_t)seg * n;
    if (perm) {
      perm[base + p] = sl_me;
      inv[base + sl_me] = p;
    }
    const int w_img = seg - img * map.segs_per_img;
    if (score_out) {
      const int row = map.row_of(seg, sl_me);
      if (row >= 0) score_out[row] = value(row - img * tokens);
    }
    if (rank < seg_k[w_img])  // K <= real slots, so never a pad
      routed[(size_t)img * routed_per_image + seg_off[w_img] + rank] = map.row_of(seg, sl_me);
  }
  if constexpr (NV > 0) {
    const int sl = chunk * tpw + wave;
    if (sl < n) {
      bf16_t* o = ln.out + ((size_t)seg * n + pos_lds[wave]) * (NV * 256);
      if (ln_src >= 0)
        lrow.store(o, lane);
      else
        LnRow<NV>::zero(o, lane);
    }
  }
}

size_t permute_lds_bytes(const sparsesam_plan& p) { return (size_t)((p.n + 63) & ~63) * 8; }

static hipError_t launch_rank(const sparsesam_plan& p, const float* imp, int parts, int batch, int* perm, int* inv,
                              int* routed, float* score_out, int ordering, hipStream_t st, RankLn ln = RankLn{}) {
  // long segments: 16 slots per workgroup and up to 16 wavefronts splitting the keys;
  // short ones (windows): 64 slots per workgroup, one wavefront per 256 keys
  const int tpw = p.n >= 1024 ? 16 : 64;
  const int kw = std::max(1, std::min(kMaxRankWaves, (p.n + 255) / 256));
  const int chunks = (p.n + tpw - 1) / tpw;
  const int segs = batch * p.segs_per_img;
  const size_t key_bytes = permute_lds_bytes(p);
  const int nv = ln.out ? p.desc.channels / 256 : 0;
  if (ln.out && (tpw != 16 || kw != 16 || p.desc.channels % 256 != 0 || nv < 3 || nv > 5))
    return hipErrorInvalidValue;
  auto kern = nv == 3 ? rank_kernel<3> : nv == 4 ? rank_kernel<4> : nv == 5 ? rank_kernel<5> : rank_kernel<0>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)key_bytes);
  if (e != hipSuccess) return e;
  // segment shape for the position-based orders: the grid, or one window
  const int seg_h = p.desc.window ? p.desc.window : p.desc.grid_h;
  const int seg_w = p.desc.window ? p.desc.window : p.desc.grid_w;
  int side = 1;
  while (side < std::max(seg_h, seg_w)) side *= 2;
  hipLaunchKernelGGL(kern, dim3((unsigned)(segs * chunks)), dim3(64 * kw), key_bytes, st, imp, p.segmap(), p.n,
                     p.desc.stripes, chunks, tpw, p.d_seg_k, p.d_seg_off, p.routed_per_image, perm, inv, routed,
                     ordering, p.desc.order_seed, seg_w, side, parts, score_out, ln);
  return hipGetLastError();
}

hipError_t launch_permute(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                          hipStream_t st) {
  return launch_rank(p, imp, 1, batch, perm, inv, routed, nullptr, (int)p.desc.ordering, st);
}

bool permute_ln_fusable(const sparsesam_plan& p) {
  const int tpw = p.n >= 1024 ? 16 : 64;
  const int kw = std::max(1, std::min(kMaxRankWaves, (p.n + 255) / 256));
  const int nv = p.desc.channels / 256;
  return p.desc.dtype == SPARSESAM_BF16 && tpw == 16 && kw == 16 && p.desc.channels % 256 == 0 && nv >= 3 &&
         nv <= 5;
}

hipError_t launch_permute_ln(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                             const float* x, long long x_rows, const float* gamma, const float* beta, bf16_t* out,
                             hipStream_t st) {
  RankLn ln;
  ln.x = x;
  ln.x_rows = x_rows;
  ln.gamma = gamma;
  ln.beta = beta;
  ln.out = out;
  return launch_rank(p, imp, 1, batch, perm, inv, routed, nullptr, (int)p.desc.ordering, st, ln);
}

hipError_t launch_route_topk(const sparsesam_plan& p, const float* score, int parts, int batch, int* routed,
                             float* score_out, hipStream_t st) {
  return launch_rank(p, score, parts, batch, nullptr, nullptr, routed, score_out, SPARSESAM_ORDER_IMPORTANCE, st);
}

}  // namespace sparsesam

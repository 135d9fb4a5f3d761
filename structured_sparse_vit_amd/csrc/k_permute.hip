// Stripe-sort permutation and keep-set of every segment of an image.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention,
// stripe-sort bullet: tokens are sorted by importance, the sorted list is viewed as
// a matrix and transposed before flattening, which spreads the important tokens over
// the whole sequence. Part 2 (Residual-Consistency MLP), token routing bullet: the
// keep-set follows the same deterministic order.
//
// The order is total: importance descending (-0.0 == +0.0, NaN after every number,
// pad slots after every real slot), then slot ascending. A slot's rank is therefore
// the number of slots that precede it, and its stripe-sorted position follows from
// the rank alone: rank rho sits at stripe rho % g, offset rho / g, i.e. position
// (rho % g) * S + rho / g. No sorted list is ever materialised.
//
//  * rank_kernel: one workgroup per (segment, chunk of slots). Its lanes count, for
//    the chunk's slots, the preceding slots within shares of the segment's keys (held
//    in LDS as 32-bit order keys); the shares are summed in LDS and one lane per slot
//    writes perm and inv. The split is chosen so a single image's 4096 slots still
//    spread over 256 workgroups.
//  * keepset_kernel: one workgroup per image reads each real token's rank back from
//    inv, flags the K first of its segment, and compacts the flags in raster order
//    (block-wide scan), which gives the keep-set ascending.
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

// 32-bit key that orders descending importance ascending: larger value -> smaller key.
__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0xFFFFFFFEu;       // NaN: after every number
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;  // -0.0 -> +0.0
  const uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;
}
constexpr uint32_t kPadKey = 0xFFFFFFFFu;  // pad slots: after every real slot

// rank_kernel layout: a workgroup of kw wavefronts ranks tpw slots of one segment
// (tpw = 16 or 64). Lane l of a wavefront serves slot l % tpw and key residue class
// l / tpw (mod 64 / tpw); wavefront w takes the w-th share of the keys. For N = 4096
// that is 256 workgroups of 16 wavefronts, every lane comparing 64 keys.
constexpr int kMaxRankWaves = 16;

__global__ void __launch_bounds__(64 * kMaxRankWaves) rank_kernel(const float* __restrict__ imp, SegmentMap map,
                                                                  int n, int stripes, int chunks, int tpw,
                                                                  int* __restrict__ perm, int* __restrict__ inv) {
  extern __shared__ uint32_t key_lds[];  // keys of the segment, padded to a multiple of 64
  __shared__ int part[kMaxRankWaves * 64];
  const int seg = blockIdx.x / chunks, chunk = blockIdx.x - (blockIdx.x / chunks) * chunks;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int kw = blockDim.x >> 6;
  const int tokens = map.grid_h * map.grid_w;
  const int img = seg / map.segs_per_img;
  const float* im = imp + (size_t)img * tokens;
  const int n64 = (n + 63) & ~63;
  // keys past n are pad keys with index >= n: they never precede a real slot
#pragma unroll 4
  for (int s = tid; s < n64; s += blockDim.x) {
    const int row = s < n ? map.row_of(seg, s) : -1;
    key_lds[s] = row >= 0 ? desc_key(im[row - img * tokens]) : kPadKey;
  }
  __syncthreads();
  const int subs = 64 / tpw;                 // lanes per slot
  const int slot = chunk * tpw + (lane % tpw);
  const int sub = lane / tpw;
  const bool valid = slot < n;
  const uint32_t mine = valid ? key_lds[slot] : 0u;
  // this wavefront's share of the keys: [j0, j1), a multiple of 64 long
  const int per = ((n64 / 64 + kw - 1) / kw) * 64;
  const int j0 = wave * per, j1 = min(n64, j0 + per);
  int cnt = 0;
  for (int jb = j0; jb < j1; jb += 4 * subs) {
    // four keys per lane per step: jb + sub + subs * u, u = 0..3
    uint32_t kk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) kk[u] = key_lds[jb + sub + subs * u];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int jj = jb + sub + subs * u;
      cnt += (kk[u] < mine) | ((kk[u] == mine) & (jj < slot));
    }
  }
  part[wave * 64 + lane] = cnt;
  __syncthreads();
  if (tid < tpw) {
    const int sl = chunk * tpw + tid;
    if (sl < n) {
      int rank = 0;
      for (int w = 0; w < kw; ++w)
        for (int u = 0; u < subs; ++u) rank += part[w * 64 + u * tpw + tid];
      const int S = n / stripes;
      const int p = (rank % stripes) * S + rank / stripes;
      const size_t base = (size_t)seg * n;
      perm[base + p] = sl;
      inv[base + sl] = p;
    }
  }
}

__global__ void __launch_bounds__(1024) keepset_kernel(const int* __restrict__ inv, SegmentMap map, int segs, int n,
                                                       int stripes, const int* __restrict__ seg_k,
                                                       int routed_per_image, int* __restrict__ routed) {
  extern __shared__ unsigned char flag[];
  __shared__ int wave_tot[16];
  const int img = blockIdx.x;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int tokens = map.grid_h * map.grid_w;
  const int S = n / stripes;
  for (int t = tid; t < tokens; t += nth) flag[t] = 0;
  __syncthreads();
#pragma unroll 4
  for (int i = tid; i < segs * n; i += nth) {
    const int sg = i / n, s = i - sg * n;
    const int row = map.row_of(img * segs + sg, s) - img * tokens;
    if (row < 0 || row >= tokens) continue;  // pad slot
    const int p = inv[((size_t)img * segs + sg) * n + s];
    const int rank = stripes * (p % S) + p / S;
    if (rank < seg_k[sg]) flag[row] = 1;
  }
  __syncthreads();
  // compact the flags in raster order (block-wide exclusive scan)
  const int per = (tokens + nth - 1) / nth;
  const int t0 = tid * per;
  int cnt = 0;
  for (int t = t0; t < t0 + per && t < tokens; ++t) cnt += flag[t];
  const int lane = tid & 63, wv = tid >> 6;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_tot[wv] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wv; ++w) before += wave_tot[w];
  int pos = before + incl - cnt;
  int* out = routed + (size_t)img * routed_per_image;
  for (int t = t0; t < t0 + per && t < tokens; ++t) {
    if (flag[t]) {
      if (pos < routed_per_image) out[pos] = img * tokens + t;
      ++pos;
    }
  }
}

size_t permute_lds_bytes(const sparsesam_plan& p) {
  const size_t tokens = (size_t)p.desc.grid_h * p.desc.grid_w;
  return std::max((size_t)((p.n + 63) & ~63) * 4, tokens);
}

hipError_t launch_permute(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                          hipStream_t st) {
  // long segments: 16 slots per workgroup and up to 16 wavefronts splitting the keys;
  // short ones (windows): 64 slots per workgroup, one wavefront per 256 keys
  const int tpw = p.n >= 1024 ? 16 : 64;
  const int kw = std::max(1, std::min(kMaxRankWaves, (p.n + 255) / 256));
  const int chunks = (p.n + tpw - 1) / tpw;
  const int segs = batch * p.segs_per_img;
  const size_t key_bytes = (size_t)((p.n + 63) & ~63) * 4;
  hipError_t e = hipFuncSetAttribute((const void*)rank_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)key_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(rank_kernel, dim3((unsigned)(segs * chunks)), dim3(64 * kw), key_bytes, st, imp, p.segmap(),
                     p.n, p.desc.stripes, chunks, tpw, perm, inv);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t flag_bytes = (size_t)p.desc.grid_h * p.desc.grid_w;
  e = hipFuncSetAttribute((const void*)keepset_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)flag_bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(keepset_kernel, dim3(batch), dim3(1024), flag_bytes, st, inv, p.segmap(), p.segs_per_img, p.n,
                     p.desc.stripes, p.d_seg_k, p.routed_per_image, routed);
  return hipGetLastError();
}

}  // namespace sparsesam

// Stripe-sort permutation and keep-set of every segment of an image.
//
// "Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention,
// stripe-sort bullet: tokens are sorted by importance, the sorted list is viewed as
// a matrix and transposed before flattening, which spreads the important tokens over
// the whole sequence. Part 2 (Residual-Consistency MLP), token routing bullet: the
// keep-set follows the same deterministic order.
//
// One workgroup (1024 threads) per image does everything in LDS:
//  1. builds one 64-bit key per segment slot: the high word orders importance
//     descending (-0.0 == +0.0, NaN after every number, pad slots after NaN), the low
//     word is the slot, so the order is total and the result unique;
//  2. bitonic-sorts every segment's keys in place (segments are padded to a power of
//     two with keys that sort last);
//  3. writes perm[p] = sorted[g * (p % S) + p / S] and inv[perm[p]] = p;
//  4. flags the first K slots of each segment's order in an image-wide token map and
//     compacts the flags in raster order, which gives the keep-set ascending.
#include "internal.hpp"

namespace sparsesam {

__device__ __forceinline__ uint32_t desc_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 0xFFFFFFFEu;          // NaN: after every number
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;     // -0.0 -> +0.0
  uint32_t asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ~asc;                              // larger value -> smaller key
}

__global__ void __launch_bounds__(1024) stripe_permute_kernel(const float* __restrict__ imp, SegmentMap map,
                                                              int segs, int n, int p2, int stripes,
                                                              const int* __restrict__ seg_k, int routed_per_image,
                                                              int* __restrict__ perm, int* __restrict__ inv,
                                                              int* __restrict__ routed) {
  extern __shared__ unsigned long long smem_keys[];
  __shared__ int wave_tot[16];
  const int img = blockIdx.x;
  const int tid = threadIdx.x, nth = blockDim.x;
  const int tokens = map.grid_h * map.grid_w;
  const int total = segs * p2;
  unsigned long long* keys = smem_keys;
  unsigned char* flag = reinterpret_cast<unsigned char*>(smem_keys + total);
  const float* im = imp + (size_t)img * tokens;

  for (int i = tid; i < total; i += nth) {
    int sg = i / p2, slot = i - sg * p2;
    uint32_t hi = 0xFFFFFFFFu;
    if (slot < n) {
      int row = map.row_of(img * segs + sg, slot);
      if (row >= 0) hi = desc_key(im[row - img * tokens]);
    }
    keys[i] = ((unsigned long long)hi << 32) | (uint32_t)slot;
  }
  for (int t = tid; t < tokens; t += nth) flag[t] = 0;
  __syncthreads();

  // Bitonic sort of each p2-long run, ascending by key. Pair t of a stage with stride j
  // compares keys i = (t / j) * 2j + t % j and i + j. For j <= 32 the 64 pairs of one
  // wavefront lie inside one 128-key block that no other wavefront touches, so those
  // stages need only a wavefront fence; a workgroup barrier precedes every stage with a
  // larger stride (its pairs cross wavefronts) and the first stride-32 stage after one.
  const int half = total >> 1;
  for (int k = 2, lk = 1; k <= p2; k <<= 1, ++lk) {
    for (int j = k >> 1, lj = lk - 1; j > 0; j >>= 1, --lj) {
      if (j >= 32) __syncthreads();
      for (int t = tid; t < half; t += nth) {
        const int i = ((t >> lj) << (lj + 1)) | (t & (j - 1));
        const int l = i + j;
        const unsigned long long a = keys[i], b = keys[l];
        // direction from the index inside the segment, so every segment ends ascending
        const bool up = (((i & (p2 - 1)) & k) == 0);
        if ((a > b) == up) {
          keys[i] = b;
          keys[l] = a;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
      __builtin_amdgcn_wave_barrier();
    }
  }
  __syncthreads();

  // Stripe transpose, inverse, and keep-set flags.
  const int S = n / stripes;
  for (int i = tid; i < segs * n; i += nth) {
    int sg = i / n, p = i - sg * n;
    int rank = stripes * (p % S) + p / S;
    int slot = (int)(uint32_t)keys[sg * p2 + rank];
    size_t base = ((size_t)img * segs + sg) * n;
    perm[base + p] = slot;
    inv[base + slot] = p;
    if (p < seg_k[sg]) {  // rank p of the plain order is in the keep-set
      int slot_r = (int)(uint32_t)keys[sg * p2 + p];
      int row = map.row_of(img * segs + sg, slot_r) - img * tokens;
      if (row >= 0 && row < tokens) flag[row] = 1;
    }
  }
  __syncthreads();

  // Compact the flags in raster order (block-wide exclusive scan).
  const int per = (tokens + nth - 1) / nth;
  const int t0 = tid * per;
  int cnt = 0;
  for (int t = t0; t < t0 + per && t < tokens; ++t) cnt += flag[t];
  const int lane = tid & 63, wv = tid >> 6;
  int incl = cnt;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int v = __shfl_up(incl, o, 64);
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
  size_t tokens = (size_t)p.desc.grid_h * p.desc.grid_w;
  return (size_t)p.segs_per_img * p.sort_pow2 * 8 + ((tokens + 15) & ~size_t(15));
}

hipError_t launch_permute(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                          hipStream_t st) {
  size_t lds = permute_lds_bytes(p);
  hipError_t e = hipFuncSetAttribute((const void*)stripe_permute_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(stripe_permute_kernel, dim3(batch), dim3(1024), lds, st, imp, p.segmap(), p.segs_per_img,
                     p.n, p.sort_pow2, p.desc.stripes, p.d_seg_k, p.routed_per_image, perm, inv, routed);
  return hipGetLastError();
}

}  // namespace sparsesam

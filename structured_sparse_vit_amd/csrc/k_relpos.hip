// Decomposed relative-position bias tables for the attention kernels.
//
// SAM's image encoder (Kirillov et al., "Segment Anything", 2023, after Li et al.,
// MViTv2, CVPR 2022) adds to the logit of a query at segment coordinates (y, x) and a
// key at (y', x') the two terms <q, Rh[y - y' + Sh - 1]> and <q, Rw[x - x' + Sw - 1]>,
// with the unscaled query and tables shared by the heads of a block. The SparseSAM
// pages name fused "FA2 + rel-pos" kernels without defining the term; this is the
// reading taken.
//
// A query's bias depends on the key only through y' and x', so each query gets one
// table row T[j] in exp2 units: j < Sh holds the term of key row y' = j, j in
// [xoff, xoff + Sw) the term of key column x' = j - xoff, the rest is zero. The
// attention kernels add T[y'] + T[xoff + x'] to the logit of every kept key. The key
// side needs only (y', x') per position: kc[seg][p] = y' | (xoff + x') << 16.
//
// relpos_table_kernel: one 256-thread workgroup per (segment, head, 64 positions). It
// forms G[p][r] = <q_p, R[r]> for all 2 Sh - 1 rows of Rh and 2 Sw - 1 rows of Rw
// (a 64 x 256 x D product in fp32 from LDS, 4 positions x 16 rows per thread), stores
// G in LDS and writes T[p][j] = log2(e) * G[p][y_p - j + Sh - 1] (or the Rw part) along
// rows, in the table type (fp16 for the matrix-core kernel, clamped to the fp16 range;
// fp32 for the SIMT one).
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

constexpr int kRelRows = 256;           // G columns: Rh rows at 0.., Rw rows at 128..
constexpr int kRelLd = kRelRows + 4;    // LDS row stride of R^T and G (16-byte aligned)
constexpr int kRelQLd = 64 + 4;         // LDS row stride of Q^T
constexpr int kRelPos = 64;             // positions per workgroup

template <typename TT>
__device__ __forceinline__ TT to_table(float v) {
  return v;
}
template <>
__device__ __forceinline__ f16_t to_table<f16_t>(float v) {
  return (f16_t)fminf(fmaxf(v, -65504.0f), 65504.0f);
}

template <typename T, typename TT>
__global__ void __launch_bounds__(256) relpos_table_kernel(const T* __restrict__ Q, const int* __restrict__ perm,
                                                           const float* __restrict__ rel_h,
                                                           const float* __restrict__ rel_w, int n, int heads, int D,
                                                           int seg_h, int seg_w, int xoff, int tj,
                                                           TT* __restrict__ table, int* __restrict__ kc) {
  extern __shared__ __attribute__((aligned(16))) float rl[];
  float* Rt = rl;                   // [D][kRelLd]: Rt[d][r] = R[r][d]; later G[p][kRelLd]
  float* Qt = rl + D * kRelLd;      // [D][kRelQLd]: Qt[d][p] = q_p[d]
  const int tid = threadIdx.x;
  const int sh = blockIdx.y, seg = sh / heads, h = sh - seg * heads;
  const int p0 = blockIdx.x * kRelPos;
  const int nh = 2 * seg_h - 1, nw = 2 * seg_w - 1;
  for (int i = tid; i < kRelRows * D; i += 256) {
    const int r = i / D, d = i - (i / D) * D;
    float v = 0.0f;
    if (r < 128) {
      if (r < nh) v = rel_h[(size_t)r * D + d];
    } else if (r - 128 < nw) {
      v = rel_w[(size_t)(r - 128) * D + d];
    }
    Rt[d * kRelLd + r] = v;
  }
  const T* qs = Q + ((size_t)sh * n + p0) * D;
  for (int i = tid; i < kRelPos * D; i += 256) {
    const int p = i / D, d = i - (i / D) * D;
    Qt[d * kRelQLd + p] = p0 + p < n ? (float)qs[(size_t)p * D + d] : 0.0f;
  }
  __syncthreads();
  const int pg = tid >> 4, rg = tid & 15;  // positions 4 pg .. + 3, rows 16 rg .. + 15
  float acc[4][16];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 16; ++b) acc[a][b] = 0.0f;
#pragma unroll 2
  for (int d = 0; d < D; ++d) {
    const f32x4 qv = *reinterpret_cast<const f32x4*>(Qt + d * kRelQLd + 4 * pg);
    f32x4 rv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rv[i] = *reinterpret_cast<const f32x4*>(Rt + d * kRelLd + 16 * rg + 4 * i);
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 16; ++b) acc[a][b] = fmaf(qv[a], rv[b >> 2][b & 3], acc[a][b]);
  }
  __syncthreads();  // every thread is done with R^T and Q^T
  float* G = rl;    // [kRelPos][kRelLd]
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<f32x4*>(G + (4 * pg + a) * kRelLd + 16 * rg + 4 * i) =
          f32x4{acc[a][4 * i], acc[a][4 * i + 1], acc[a][4 * i + 2], acc[a][4 * i + 3]};
  __syncthreads();
  // four threads per position, each a quarter of the row
  const int p = tid >> 2, part = tid & 3;
  if (p0 + p >= n) return;
  const int slot = min(max(perm[(size_t)seg * n + p0 + p], 0), seg_h * seg_w - 1);
  const int y = slot / seg_w, x = slot - (slot / seg_w) * seg_w;
  if (h == 0 && part == 0) kc[(size_t)seg * n + p0 + p] = y | ((xoff + x) << 16);
  const float log2e = 1.4426950408889634f;
  const float* g = G + p * kRelLd;
  TT* trow = table + ((size_t)sh * n + p0 + p) * tj;
  const int per = tj / 4;
  for (int j = part * per; j < (part + 1) * per; ++j) {
    float v = 0.0f;
    if (j < seg_h)
      v = g[y - j + seg_h - 1];
    else if (j >= xoff && j < xoff + seg_w)
      v = g[128 + x - (j - xoff) + seg_w - 1];
    trow[j] = to_table<TT>(v * log2e);
  }
}

// R^T and Q^T, or G over the same memory afterwards, whichever is larger
size_t relpos_lds_bytes(int head_dim) {
  return std::max((size_t)head_dim * (kRelLd + kRelQLd), (size_t)kRelPos * kRelLd) * sizeof(float);
}

template <typename T, typename TT>
hipError_t launch_relpos_table(const sparsesam_plan& p, int segments, const T* q, const int* perm,
                               const float* rel_h, const float* rel_w, TT* table, int* kc, hipStream_t st) {
  const int D = p.desc.head_dim;
  const size_t lds = relpos_lds_bytes(D);
  auto kern = relpos_table_kernel<T, TT>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((p.n + kRelPos - 1) / kRelPos), (unsigned)(segments * p.desc.heads));
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q, perm, rel_h, rel_w, p.n, p.desc.heads, D, p.rel_seg_h,
                     p.rel_seg_w, p.rel_xoff, p.rel_tj, table, kc);
  return hipGetLastError();
}

template hipError_t launch_relpos_table<bf16_t, f16_t>(const sparsesam_plan&, int, const bf16_t*, const int*,
                                                       const float*, const float*, f16_t*, int*, hipStream_t);
template hipError_t launch_relpos_table<bf16_t, float>(const sparsesam_plan&, int, const bf16_t*, const int*,
                                                       const float*, const float*, float*, int*, hipStream_t);
template hipError_t launch_relpos_table<float, float>(const sparsesam_plan&, int, const float*, const int*,
                                                      const float*, const float*, float*, int*, hipStream_t);

}  // namespace sparsesam

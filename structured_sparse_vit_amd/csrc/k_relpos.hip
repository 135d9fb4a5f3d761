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
// relpos_table_kernel (head_dim D = 32, 64 or 80): one 256-thread workgroup per
// (segment, head, 64 positions). It forms G[p][r] = <q_p, R[r]> for all 2 Sh - 1 rows
// of Rh and 2 Sw - 1 rows of Rw (a 64 x 256 x D product in fp32 from LDS, 4 positions x
// 16 rows per thread), stages log2(e) G in LDS, already in the table type (fp16 for the
// matrix-core attention kernels, clamped to its range: the one rounding of the entry;
// fp32 for the SIMT one), and writes T[p][j] = that staged G[p][y_p - j + Sh - 1] (or
// the Rw part) along rows. fp16 staging halves the LDS of a workgroup, so all of them
// stay resident at once on the ViT-B global grid.
#include <algorithm>

#include "internal.hpp"

namespace sparsesam {

constexpr int kRelRows = 256;           // G columns: Rh rows at 0.., Rw rows at 128..
constexpr int kRelLd = kRelRows + 4;    // LDS row stride of R^T and G (16-byte aligned)
constexpr int kRelQLd = 64 + 4;         // LDS row stride of Q^T
constexpr int kRelPos = 64;             // positions per workgroup

// a table entry from its fp32 value in exp2 units: fp16 clamped to its range, or fp32
template <typename TT>
__device__ __forceinline__ TT table_entry(float v);
template <>
__device__ __forceinline__ float table_entry<float>(float v) {
  return v;
}
template <>
__device__ __forceinline__ f16_t table_entry<f16_t>(float v) {
  return (f16_t)fminf(fmaxf(v, -65504.0f), 65504.0f);
}

// four consecutive table entries in one store (8 bytes fp16, 16 bytes fp32)
template <typename TT>
__device__ __forceinline__ void store4(TT* dst, const TT (&v)[4]);
template <>
__device__ __forceinline__ void store4<float>(float* dst, const float (&v)[4]) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
}
template <>
__device__ __forceinline__ void store4<f16_t>(f16_t* dst, const f16_t (&v)[4]) {
  typedef __attribute__((__vector_size__(4 * sizeof(_Float16)))) _Float16 f16x4;
  *reinterpret_cast<f16x4*>(dst) = f16x4{v[0], v[1], v[2], v[3]};
}

constexpr float kLog2e = 1.4426950408889634f;

// Table rows are the rows of [segment][head][position] taken flat: row r is position
// r mod n of segment-head r / n, and its Q row and table row sit at index r.
template <typename TT>
__device__ __forceinline__ void write_rows(const TT* G, int slot_raw, long long r0, long long r_end, int n,
                                           int heads, int seg_h, int seg_w, int xoff, int tj,
                                           TT* __restrict__ table, int* __restrict__ kc);
// slot of the position whose row this thread writes in write_rows (row r0 + threadIdx.x /
// 4, clamped to the last row), loaded up front so that its latency overlaps the product
__device__ __forceinline__ int row_slot(const int* __restrict__ perm, long long r0, long long r_end, int n,
                                        int heads) {
  const long long r = min(r0 + (long long)(threadIdx.x >> 2), r_end - 1);
  const long long sh = r / n;
  return perm[(sh / heads) * n + (r - sh * n)];
}

template <typename T, typename TT, int D>
__global__ void __launch_bounds__(256) relpos_table_kernel(const T* __restrict__ Q, const int* __restrict__ perm,
                                                           const float* __restrict__ rel_h,
                                                           const float* __restrict__ rel_w, int n, int heads,
                                                           int seg_h, int seg_w, int xoff, int tj,
                                                           TT* __restrict__ table, int* __restrict__ kc) {
  extern __shared__ __attribute__((aligned(16))) float rl[];
  float* Rt = rl;                   // [D][kRelLd]: Rt[d][r] = R[r][d]; later G[p][kRelLd]
  float* Qt = rl + D * kRelLd;      // [D][kRelQLd]: Qt[d][p] = q_p[d]
  const int tid = threadIdx.x;
  const int sh = blockIdx.y;
  const int p0 = blockIdx.x * kRelPos;
  const int nh = 2 * seg_h - 1, nw = 2 * seg_w - 1;
  // every load of the R and Q tiles is issued before the first LDS store (addresses
  // clamped to a real row; rows past the tables and positions past n store zero)
  constexpr int RI = kRelRows * D / 256, QI = kRelPos * D / 256;
  float rv[RI], qv0[QI];
#pragma unroll
  for (int k = 0; k < RI; ++k) {
    const int i = tid + 256 * k, r = i / D, d = i - (i / D) * D;
    rv[k] = r < 128 ? rel_h[(size_t)min(r, nh - 1) * D + d] : rel_w[(size_t)min(r - 128, nw - 1) * D + d];
  }
  const T* qs = Q + ((size_t)sh * n + p0) * D;
  const int prow = n - 1 - p0;  // last real position of this workgroup, relative to p0
#pragma unroll
  for (int k = 0; k < QI; ++k) {
    const int i = tid + 256 * k, p = i / D, d = i - (i / D) * D;
    qv0[k] = (float)qs[(size_t)min(p, prow) * D + d];
  }
#pragma unroll
  for (int k = 0; k < RI; ++k) {
    const int i = tid + 256 * k, r = i / D, d = i - (i / D) * D;
    const bool real = r < 128 ? r < nh : r - 128 < nw;
    Rt[d * kRelLd + r] = real ? rv[k] : 0.0f;
  }
#pragma unroll
  for (int k = 0; k < QI; ++k) {
    const int i = tid + 256 * k, p = i / D, d = i - (i / D) * D;
    Qt[d * kRelQLd + p] = p <= prow ? qv0[k] : 0.0f;
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
  __syncthreads();                         // every thread is done with R^T and Q^T
  TT* G = reinterpret_cast<TT*>(rl);       // [kRelPos][kRelLd], log2(e) G as table entries
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 16; ++b) G[(4 * pg + a) * kRelLd + 16 * rg + b] = table_entry<TT>(acc[a][b] * kLog2e);
  __syncthreads();
  const long long r0 = (long long)sh * n + p0, r_end = (long long)sh * n + n;
  write_rows<TT>(G, row_slot(perm, r0, r_end, n, heads), r0, r_end, n, heads, seg_h, seg_w, xoff, tj, table, kc);
}

// Table rows r0 .. r0 + 63 (those below r_end) from the staged entries G[r - r0][c] in
// LDS (row stride kRelLd): four threads per row; store i of thread `part` covers entries
// 4 (4 i + part) .. + 3, so the four threads of a row write one contiguous piece per
// store. Each entry reads the one staged value it takes (index clamped into the row,
// zero outside both parts). Rows of head 0 also write their position's key coordinates.
template <typename TT>
__device__ __forceinline__ void write_rows(const TT* G, int slot_raw, long long r0, long long r_end, int n,
                                           int heads, int seg_h, int seg_w, int xoff, int tj,
                                           TT* __restrict__ table, int* __restrict__ kc) {
  const int tid = threadIdx.x;
  const int p = tid >> 2, part = tid & 3;
  const long long r = r0 + p;
  if (r >= r_end) return;
  const long long sh = r / n;
  const int pos = (int)(r - sh * n);
  const long long seg = sh / heads;
  const int slot = min(max(slot_raw, 0), seg_h * seg_w - 1);
  const int y = slot / seg_w, x = slot - (slot / seg_w) * seg_w;
  if (sh - seg * heads == 0 && part == 0) kc[seg * n + pos] = y | ((xoff + x) << 16);
  const TT* g = G + p * kRelLd;
  TT* trow = table + r * tj;
  // tj is a multiple of 16 and at most 128: tj / 16 <= 8 stores of 4 entries per thread
#pragma unroll
  for (int it = 0; it < 8; ++it) {
    const int j0 = 4 * part + 16 * it;
    if (j0 >= tj) break;
    TT v4[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j0 + e;
      const bool in_w = j >= xoff && j < xoff + seg_w;
      const int idx = j < seg_h ? y - j + seg_h - 1 : 128 + x - (j - xoff) + seg_w - 1;
      const TT v = g[min(max(idx, 0), 255)];
      v4[e] = (j < seg_h || in_w) ? v : (TT)0.0f;
    }
    store4<TT>(trow + j0, v4);
  }
}

// bf16 queries: G = Q R^T on the matrix cores (v_mfma_f32_32x32x16_bf16). R is fp32, so
// each R fragment goes in as bf16 hi + lo parts (R - hi rounded again), two MFMAs per
// k-step: G carries about 2^-16 relative error, far below the table's own rounding.
// One workgroup per 64 flat table rows (so short segments, such as 196-token windows,
// leave no idle positions). Wavefront w forms G for the 64 rows and R rows 64 w ..
// 64 w + 63 straight from global memory (Q rows and R rows are each read by the lanes
// that need them) and stages it in LDS; a wavefront whose R rows are all past the tables
// (w = 1 for Sh <= 32, w = 3 for Sw <= 32) does nothing, as no entry reads its columns.
// The workgroup then writes the table rows as above.
template <typename TT, int D>
__global__ void __launch_bounds__(256) relpos_table_mfma_kernel(const bf16_t* __restrict__ Q,
                                                                const int* __restrict__ perm,
                                                                const float* __restrict__ rel_h,
                                                                const float* __restrict__ rel_w, int n, int heads,
                                                                long long rows, int seg_h, int seg_w, int xoff,
                                                                int tj, TT* __restrict__ table,
                                                                int* __restrict__ kc) {
  extern __shared__ __attribute__((aligned(16))) float rl[];
  constexpr int KS = D / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long long r0 = (long long)blockIdx.x * kRelPos;
  const int nh = 2 * seg_h - 1, nw = 2 * seg_w - 1;
  const int l32 = lane & 31, k8 = (lane >> 5) * 8;
  const int slot_raw = row_slot(perm, r0, rows, n, heads);
  const bool live = w < 2 ? 64 * w < nh : 64 * (w - 2) < nw;
  if (live) {
    // A operand: Q rows r0 + 32 pb + l32 (clamped to the last row), d = 16 ks + k8 ..
    bf16x8 qa[2][KS];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb) {
      const long long row = min(r0 + 32 * pb + l32, rows - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[pb][ks] = *reinterpret_cast<const bf16x8*>(Q + row * D + 16 * ks + k8);
    }
    // B operand: R rows r = 64 w + 32 rb + l32 (rel_h below 128, rel_w above), as hi / lo
    f32x4 rf[2][KS][2];
    bool real[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const int r = 64 * w + 32 * rb + l32;
      real[rb] = r < 128 ? r < nh : r - 128 < nw;
      const float* src = r < 128 ? rel_h + (size_t)min(r, nh - 1) * D : rel_w + (size_t)min(r - 128, nw - 1) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        rf[rb][ks][0] = *reinterpret_cast<const f32x4*>(src + 16 * ks + k8);
        rf[rb][ks][1] = *reinterpret_cast<const f32x4*>(src + 16 * ks + k8 + 4);
      }
    }
    f32x16 acc[2][2];
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[pb][rb][e] = 0.0f;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = real[rb] ? rf[rb][ks][e >> 2][e & 3] : 0.0f;
          hi[e] = to_bf16(v);
          lo[e] = to_bf16(v - to_f32(hi[e]));
        }
#pragma unroll
        for (int pb = 0; pb < 2; ++pb) {
          acc[pb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[pb][ks], hi, acc[pb][rb], 0, 0, 0);
          acc[pb][rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[pb][ks], lo, acc[pb][rb], 0, 0, 0);
        }
      }
    // C[row = table row][col = R row]: lane l holds column l32, rows 8 (i / 4) + 4 (l / 32) + i % 4
    TT* G = reinterpret_cast<TT*>(rl);
#pragma unroll
    for (int pb = 0; pb < 2; ++pb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int p = 32 * pb + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
          G[p * kRelLd + 64 * w + 32 * rb + l32] = table_entry<TT>(acc[pb][rb][i] * kLog2e);
        }
  }
  __syncthreads();
  write_rows<TT>(reinterpret_cast<const TT*>(rl), slot_raw, r0, rows, n, heads, seg_h, seg_w, xoff, tj, table, kc);
}

// R^T and Q^T, or G over the same memory afterwards, whichever is larger
size_t relpos_lds_bytes(int head_dim) {
  return std::max((size_t)head_dim * (kRelLd + kRelQLd), (size_t)kRelPos * kRelLd) * sizeof(float);
}

template <typename T, typename TT>
hipError_t launch_relpos_table(const sparsesam_plan& p, int segments, const T* q, const int* perm,
                               const float* rel_h, const float* rel_w, TT* table, int* kc, hipStream_t st) {
  const int D = p.desc.head_dim;
  dim3 grid((unsigned)((p.n + kRelPos - 1) / kRelPos), (unsigned)(segments * p.desc.heads));
  if constexpr (sizeof(T) == 2) {
    const long long rows = (long long)segments * p.desc.heads * p.n;
    if (rows <= 0) return hipSuccess;
    const size_t lds = (size_t)kRelPos * kRelLd * sizeof(TT);
    auto kern = D == 32 ? relpos_table_mfma_kernel<TT, 32> : D == 80 ? relpos_table_mfma_kernel<TT, 80>
                                                                     : relpos_table_mfma_kernel<TT, 64>;
    if (D != 32 && D != 64 && D != 80) return hipErrorInvalidValue;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3((unsigned)((rows + kRelPos - 1) / kRelPos)), dim3(256), lds, st, q, perm, rel_h,
                       rel_w, p.n, p.desc.heads, rows, p.rel_seg_h, p.rel_seg_w, p.rel_xoff, p.rel_tj, table, kc);
    return hipGetLastError();
  }
  const size_t lds = relpos_lds_bytes(D);
  auto kern = D == 32 ? relpos_table_kernel<T, TT, 32> : D == 80 ? relpos_table_kernel<T, TT, 80>
                                                                 : relpos_table_kernel<T, TT, 64>;
  if (D != 32 && D != 64 && D != 80) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q, perm, rel_h, rel_w, p.n, p.desc.heads, p.rel_seg_h,
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

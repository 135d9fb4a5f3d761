// GEMMs of the block, C = A W^T, with fused epilogues.
//
// The QKV, output projection and MLP products stay dense over the rows they are
// given (the method sparsifies attention and routes MLP rows; it does not prune
// weights). bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation); the fp32 path is a plain SIMT kernel for small exact checks.
//
// bf16 kernel: 128 x 128 output tile per 256-thread workgroup, K step 64. A and W
// tiles are staged through LDS (rows padded by 16 bytes so the 16-byte fragment
// reads of 32 consecutive rows hit distinct banks); the next K step is prefetched
// into registers while the current one is multiplied. Each wavefront owns a 64 x 64
// quarter as 2 x 2 MFMA blocks. Workgroups whose columns are all V columns of the QKV
// product swap the MFMA operands so each lane holds consecutive tokens of one
// channel, which is the layout of the transposed V the attention kernel reads.
#include "internal.hpp"

namespace sparsesam {

// ---------------------------------------------------------------- epilogues

template <typename T>
struct QKVStore {
  const float* bias;
  T *q, *k, *vt;
  int n, n_pad, heads, D, C;
  // One unconditional store through a selected base pointer and index. (A three-way
  // if / else-if / else with a store in each arm was compiled for gfx950 into code
  // that sent the V^T stores through the k pointer; selects avoid that shape.)
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    v += bias[c];
    const int which = c / C;
    const int cc = c - which * C;
    const int h = cc / D, d = cc - h * D;
    const int seg = r / n, p = r - seg * n;
    const size_t sh = (size_t)seg * heads + h;
    const bool is_v = which >= 2;
    const size_t idx = is_v ? (sh * D + d) * (size_t)n_pad + p : (sh * n + p) * (size_t)D + d;
    T* base = is_v ? vt : (which == 0 ? q : k);
    base[idx] = from_f32<T>(v);
  }
  // Column tile [c0, c0 + BN) is all V: store it transposed.
  __device__ __forceinline__ bool transposed_tile(int c0) const { return c0 >= 2 * C; }
};

template <typename T>
struct GeluStore {
  const float* bias;
  T* out;
  int ld;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    out[(size_t)r * ld + c] = from_f32<T>(gelu_erf(v + bias[c]));
  }
  __device__ __forceinline__ bool transposed_tile(int) const { return false; }
};

struct ResidualAdd {
  const float* bias;
  float* x;
  const int* perm;
  const int* list;
  SegmentMap map;
  int ldx;
  long long x_rows;
  __device__ __forceinline__ int dst_row(int r) const {
    if (list) return list[r];
    return map.row_of(r / map.n, perm[r]);
  }
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    int row = dst_row(r);
    if (row < 0 || row >= x_rows) return;
    float* px = x + (size_t)row * ldx + c;
    *px = *px + (v + bias[c]);
  }
  __device__ __forceinline__ bool transposed_tile(int) const { return false; }
};

// Partial sums of a split-K product: part[z][r][c].
struct PartialStore {
  float* part;
  int m, n;
  int z;
  __device__ __forceinline__ void operator()(int r, int c, float v) const {
    part[((size_t)z * m + r) * n + c] = v;
  }
  __device__ __forceinline__ bool transposed_tile(int) const { return false; }
};

// ---------------------------------------------------------------- bf16 MFMA GEMM

constexpr int BM = 128, BN = 128, BK = 64, LDS_LD = BK + 8;

template <class Epi, bool kPartial>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, int k_split, Epi epi, float* part) {
  __shared__ __attribute__((aligned(16))) bf16_t As[BM * LDS_LD];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[BN * LDS_LD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n0 = blockIdx.x * BN, m0 = blockIdx.y * BM;
  const int kz = blockIdx.z;
  const int kb = kz * k_split, ke = min(K, kb + k_split);
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // global -> register staging: 4 x 16 bytes of A and of W per thread
  i32x4 ra[4], rb[4];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      int row = c >> 3, col = (c & 7) * 8;
      int gm = m0 + row, gn = n0 + row;
      ra[i] = (gm < M) ? *reinterpret_cast<const i32x4*>(A + (size_t)gm * K + k0 + col) : i32x4{0, 0, 0, 0};
      rb[i] = (gn < N) ? *reinterpret_cast<const i32x4*>(W + (size_t)gn * K + k0 + col) : i32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int c = tid + 256 * i;
      int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<i32x4*>(As + row * LDS_LD + col) = ra[i];
      *reinterpret_cast<i32x4*>(Bs + row * LDS_LD + col) = rb[i];
    }
  };

  const bool tr = epi.transposed_tile(n0);
  if (kb < ke) load_tile(kb);
  for (int k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (k0 + BK < ke) load_tile(k0 + BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        int ar = wm * 64 + i * 32 + (lane & 31);
        int br = wn * 64 + i * 32 + (lane & 31);
        int col = ks * 16 + (lane >> 5) * 8;
        af[i] = *reinterpret_cast<const bf16x8*>(As + ar * LDS_LD + col);
        bfr[i] = *reinterpret_cast<const bf16x8*>(Bs + br * LDS_LD + col);
      }
      if (!tr) {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
      }
    }
  }

  // epilogue: lane holds column (lane & 31) of four row quads of each 32 x 32 block
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        int inner = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        int outer = lane & 31;
        int m, n;
        if (!tr) {
          m = m0 + wm * 64 + i * 32 + inner;
          n = n0 + wn * 64 + j * 32 + outer;
        } else {
          n = n0 + wn * 64 + j * 32 + inner;
          m = m0 + wm * 64 + i * 32 + outer;
        }
        if (m < M && n < N) {
          if (kPartial) {
            part[((size_t)kz * M + m) * N + n] = acc[i][j][e];
          } else {
            epi(m, n, acc[i][j][e]);
          }
        }
      }
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

constexpr int FT = 64, FK = 16;

template <class Epi, bool kPartial>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       int M, int N, int K, int k_split, Epi epi, float* part) {
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * FT, m0 = blockIdx.y * FT;
  const int kz = blockIdx.z;
  const int kb = kz * k_split, ke = min(K, kb + k_split);
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  for (int k0 = kb; k0 < ke; k0 += FK) {
    for (int i = tid; i < FT * FK; i += 256) {
      int row = i / FK, kk = i % FK;
      int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      As[kk][row] = (gm < M && gk < ke) ? A[(size_t)gm * K + gk] : 0.0f;
      Bs[kk][row] = (gn < N && gk < ke) ? W[(size_t)gn * K + gk] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < FK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = As[kk][tr + 16 * i];
        b[i] = Bs[kk][tc + 16 * i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      int m = m0 + tr + 16 * i, n = n0 + tc + 16 * j;
      if (m < M && n < N) {
        if (kPartial)
          part[((size_t)kz * M + m) * N + n] = acc[i][j];
        else
          epi(m, n, acc[i][j]);
      }
    }
}

// ---------------------------------------------------------------- split-K reduction

__global__ void __launch_bounds__(256) splitk_residual_kernel(const float* __restrict__ part, int splits, int M, int N,
                                                              ResidualAdd epi) {
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)M * N) return;
  int r = (int)(i / N), c = (int)(i - (size_t)r * N);
  float s = part[i];
  for (int z = 1; z < splits; ++z) s += part[(size_t)z * M * N + i];
  epi(r, c, s);
}

// ---------------------------------------------------------------- launchers

template <typename T>
struct GemmOp;
template <>
struct GemmOp<bf16_t> {
  template <class Epi, bool P>
  static hipError_t run(const bf16_t* a, const bf16_t* w, int m, int n, int k, int splits, const Epi& e, float* part,
                        hipStream_t st) {
    int ksplit = ((k / splits + BK - 1) / BK) * BK;
    dim3 grid((n + BN - 1) / BN, (m + BM - 1) / BM, splits);
    hipLaunchKernelGGL((gemm_bf16_kernel<Epi, P>), grid, dim3(256), 0, st, a, w, m, n, k, ksplit, e, part);
    return hipGetLastError();
  }
};
template <>
struct GemmOp<float> {
  template <class Epi, bool P>
  static hipError_t run(const float* a, const float* w, int m, int n, int k, int splits, const Epi& e, float* part,
                        hipStream_t st) {
    int ksplit = ((k / splits + FK - 1) / FK) * FK;
    dim3 grid((n + FT - 1) / FT, (m + FT - 1) / FT, splits);
    hipLaunchKernelGGL((gemm_f32_kernel<Epi, P>), grid, dim3(256), 0, st, a, w, m, n, k, ksplit, e, part);
    return hipGetLastError();
  }
};

template <typename T>
hipError_t launch_gemm_qkv(const T* a, const T* w, int m, int k, const EpiQKV& e, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  QKVStore<T> s{e.bias, (T*)e.q, (T*)e.k, (T*)e.vt, e.n, e.n_pad, e.heads, e.head_dim, e.channels};
  return GemmOp<T>::template run<QKVStore<T>, false>(a, w, m, 3 * e.channels, k, 1, s, nullptr, st);
}

template <typename T>
hipError_t launch_gemm_gelu(const T* a, const T* w, int m, int n, int k, const EpiGelu& e, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  GeluStore<T> s{e.bias, (T*)e.out, e.ld};
  return GemmOp<T>::template run<GeluStore<T>, false>(a, w, m, n, k, 1, s, nullptr, st);
}

template <typename T>
hipError_t launch_gemm_residual(const T* a, const T* w, int m, int n, int k, const EpiResidualScatter& e, int splits,
                                float* part, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  ResidualAdd s{e.bias, e.x, e.perm, e.list, e.map, e.ldx, e.x_rows};
  if (splits <= 1) return GemmOp<T>::template run<ResidualAdd, false>(a, w, m, n, k, 1, s, nullptr, st);
  hipError_t err = GemmOp<T>::template run<ResidualAdd, true>(a, w, m, n, k, splits, s, part, st);
  if (err != hipSuccess) return err;
  size_t total = (size_t)m * n;
  hipLaunchKernelGGL(splitk_residual_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, part, splits, m,
                     n, s);
  return hipGetLastError();
}

template hipError_t launch_gemm_qkv<bf16_t>(const bf16_t*, const bf16_t*, int, int, const EpiQKV&, hipStream_t);
template hipError_t launch_gemm_qkv<float>(const float*, const float*, int, int, const EpiQKV&, hipStream_t);
template hipError_t launch_gemm_gelu<bf16_t>(const bf16_t*, const bf16_t*, int, int, int, const EpiGelu&, hipStream_t);
template hipError_t launch_gemm_gelu<float>(const float*, const float*, int, int, int, const EpiGelu&, hipStream_t);
template hipError_t launch_gemm_residual<bf16_t>(const bf16_t*, const bf16_t*, int, int, int,
                                                 const EpiResidualScatter&, int, float*, hipStream_t);
template hipError_t launch_gemm_residual<float>(const float*, const float*, int, int, int, const EpiResidualScatter&,
                                                int, float*, hipStream_t);

}  // namespace sparsesam

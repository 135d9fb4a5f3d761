// Gathered LayerNorm: the prologue of the QKV and fc1 GEMMs.
//
// out[r] = LayerNorm(x[src(r)]) with fp32 statistics (two passes over the row held
// in registers, biased variance, eps 1e-6), written in the GEMM operand type. The
// source row is the stripe-sorted position's token (through perm and the segment
// map; window pads give a zero row) or an explicit row list (the keep-set).
// One wavefront per row; memory-bound: 4C bytes read and 2C (bf16) written per row.
#include "internal.hpp"

namespace sparsesam {

constexpr int kMaxPerLane = 24;  // C <= 1536

template <typename T>
__global__ void __launch_bounds__(256) gather_ln_kernel(const float* __restrict__ x, int x_rows, int rows_out, int C,
                                                        const int* __restrict__ perm, const int* __restrict__ list,
                                                        SegmentMap map, const float* __restrict__ g,
                                                        const float* __restrict__ b, T* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
  if (r >= rows_out) return;
  int src;
  if (list) {
    src = list[r];
  } else if (perm) {
    int seg = map.seg_of(r), slot = perm[r];
    src = map.row_of(seg, slot);
  } else {
    src = map.pad_position(r) ? -1 : r;
  }
  T* o = out + (size_t)r * C;
  if (src < 0 || src >= x_rows) {
    for (int c = lane; c < C; c += 64) o[c] = from_f32<T>(0.0f);
    return;
  }
  const float* xr = x + (size_t)src * C;
  float v[kMaxPerLane];
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int c = lane + 64 * i;
    v[i] = (c < C) ? xr[c] : 0.0f;
    s += v[i];
  }
  const float mean = wave_sum(s) / (float)C;
  float q = 0.0f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int c = lane + 64 * i;
    float d = (c < C) ? v[i] - mean : 0.0f;
    q += d * d;
  }
  const float rstd = rsqrtf(wave_sum(q) / (float)C + 1e-6f);
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    int c = lane + 64 * i;
    if (c < C) o[c] = from_f32<T>((v[i] - mean) * rstd * g[c] + b[c]);
  }
}

// Vector form for bf16 output and C a multiple of 256: each lane holds NV float4 chunks
// (16-byte loads) and writes four bf16 per chunk (8-byte stores), through LnRow.
template <int NV>
__global__ void __launch_bounds__(256) gather_ln_vec_kernel(const float* __restrict__ x, int x_rows, int rows_out,
                                                            const int* __restrict__ perm,
                                                            const int* __restrict__ list, SegmentMap map,
                                                            const float* __restrict__ g, const float* __restrict__ b,
                                                            bf16_t* __restrict__ out) {
  constexpr int C = NV * 256;
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows_out) return;
  int src;
  if (list) {
    src = list[r];
  } else if (perm) {
    const int seg = map.seg_of(r), slot = perm[r];
    src = map.row_of(seg, slot);
  } else {
    src = map.pad_position(r) ? -1 : r;
  }
  bf16_t* o = out + (size_t)r * C;
  if (src < 0 || src >= x_rows) {
    LnRow<NV>::zero(o, lane);
    return;
  }
  LnRow<NV> row;
  row.load(x + (size_t)src * C, g, b, lane);
  row.store(o, lane);
}

template <typename T>
hipError_t launch_gather_ln(const sparsesam_plan& p, const float* x, int x_rows, int rows_out, const int* perm,
                            const int* list, const float* g, const float* b, T* out, hipStream_t st) {
  if (rows_out <= 0) return hipSuccess;
  const int C = p.desc.channels;
  dim3 grid((rows_out + 3) / 4);
  if constexpr (sizeof(T) == 2) {
    auto* o = reinterpret_cast<bf16_t*>(out);
    switch (C) {
      case 768:
        hipLaunchKernelGGL(gather_ln_vec_kernel<3>, grid, dim3(256), 0, st, x, x_rows, rows_out, perm, list,
                           p.segmap(), g, b, o);
        return hipGetLastError();
      case 1024:
        hipLaunchKernelGGL(gather_ln_vec_kernel<4>, grid, dim3(256), 0, st, x, x_rows, rows_out, perm, list,
                           p.segmap(), g, b, o);
        return hipGetLastError();
      case 1280:
        hipLaunchKernelGGL(gather_ln_vec_kernel<5>, grid, dim3(256), 0, st, x, x_rows, rows_out, perm, list,
                           p.segmap(), g, b, o);
        return hipGetLastError();
      default:
        break;
    }
  }
  hipLaunchKernelGGL(gather_ln_kernel<T>, grid, dim3(256), 0, st, x, x_rows, rows_out, C, perm, list, p.segmap(), g, b,
                     out);
  return hipGetLastError();
}

template hipError_t launch_gather_ln<float>(const sparsesam_plan&, const float*, int, int, const int*, const int*,
                                            const float*, const float*, float*, hipStream_t);
template hipError_t launch_gather_ln<bf16_t>(const sparsesam_plan&, const float*, int, int, const int*, const int*,
                                             const float*, const float*, bf16_t*, hipStream_t);

}  // namespace sparsesam

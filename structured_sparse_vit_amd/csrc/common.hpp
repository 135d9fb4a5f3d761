// Device-side helpers shared by the SparseSAM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparsesam {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef _Float16 f16_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

constexpr int kWave = 64;

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (other
// counters unconstrained), in the gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits [15:14].
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }
// AND-ed into a vmcnt_imm value: also wait until no LDS read is outstanding (lgkmcnt 0)
constexpr int lgkmcnt0_mask() { return ~(15 << 8); }

// fp32 -> bf16, round to nearest even (the hardware conversion on gfx950).
__device__ __forceinline__ bf16_t to_bf16(float f) { return (bf16_t)f; }
__device__ __forceinline__ float to_f32(bf16_t b) { return (float)b; }

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return to_bf16(f); }

template <typename T>
__device__ __forceinline__ float load_f32(const T* p) { return (float)(*p); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each with its
// own L2. xcd_remap turns the hardware workgroup id into a logical work index such that
// every XCD receives one contiguous range [x * per, (x + 1) * per) of the logical order
// (per = ceil(total / 8)). Grids are launched with 8 * per workgroups; ids that land
// past `total` return -1 and the workgroup exits.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_remap(int hw_id, int total) {
  const int per = (total + kXcds - 1) / kXcds;
  const int logical = (hw_id % kXcds) * per + hw_id / kXcds;
  return logical < total ? logical : -1;
}
__host__ __device__ inline int xcd_grid(int total) { return kXcds * ((total + kXcds - 1) / kXcds); }

// Swizzled LDS tiles: 128-byte rows (64 bf16), the 16-byte chunk c of row r stored at
// chunk position c ^ ((r >> 1) & 7). gfx950 serves a 16-byte read for 16 lanes at a
// time from 16 groups of banks (group = address / 16 mod 16); 16 consecutive rows of one
// logical chunk then land in 16 distinct groups (no bank conflicts). A wavefront's
// direct-to-LDS load -- 64 lanes x 16 bytes into one contiguous 1 KiB block, lane L at
// byte 16 L -- fills 8 whole rows when lane L fetches the chunk that belongs there.
__device__ __forceinline__ int swz_key(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int swz(int r, int c) { return r * 128 + ((c ^ swz_key(r)) << 4); }

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula 7.1.26:
// erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2), t = 1 / (1 + p x) for
// x >= 0 (odd symmetry otherwise), absolute error below 1.5e-7. Branch-free, one
// reciprocal and one exp2, against a two-branch library erff.
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  const float poly =
      fmaf(fmaf(fmaf(fmaf(1.061405429f, t, -1.453152027f), t, 1.421413741f), t, -0.284496736f), t, 0.254829592f) * t;
  const float e = __builtin_amdgcn_exp2f(-(ax * ax) * 1.4426950408889634f);
  return copysignf(fmaf(-poly, e, 1.0f), x);
}

// GELU with the Gaussian CDF, 0.5 z (1 + erf(z / sqrt 2)).
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erf_as(z * 0.70710678118654752f)); }

// Division by a divisor fixed on the host, by multiplication (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994, round-up method): for
// 0 <= x < 2^31, x / d = (umulhi(x, mul) + x) >> shift with shift = ceil(log2 d) and
// mul = floor(2^32 (2^shift - d) / d) + 1. Three VALU operations instead of a
// division sequence. The default object divides by 1.
struct FastDiv {
  uint32_t d = 1, mul = 0, shift = 0;
  FastDiv() = default;
  __host__ explicit FastDiv(uint32_t divisor) : d(divisor ? divisor : 1) {
    while ((1ull << shift) < d) ++shift;
    mul = (uint32_t)((((1ull << 32) * ((1ull << shift) - d)) / d) + 1);
  }
  __device__ __forceinline__ int div(int x) const {
    return (int)((__umulhi((uint32_t)x, mul) + (uint32_t)x) >> shift);
  }
};

// Image-token row of a segment slot. Global segments map slot -> token directly;
// windowed segments map (window, slot) through the padded window grid. Returns -1
// for a pad slot. The divisions use host-prepared FastDiv divisors.
struct SegmentMap {
  int grid_h, grid_w, window, nwx, segs_per_img, n;
  FastDiv f_spi, f_nwx, f_win, f_n;  // by segs_per_img, nwx, window (or 1), n
  int stripes, s;                    // g and the stripe length S = n / g
  FastDiv f_s;                       // by S

  // Row r of a stream kept in stripe-sorted order holds a window pad iff the rank it
  // holds, (p % S) * g + p / S, is at least the window's real-token count: pads sort
  // after every real slot, so this needs no permutation load. Global segments have no pads.
  __device__ __forceinline__ bool pad_position(int r) const {
    if (window == 0) return false;
    const int seg = seg_of(r), p = r - seg * n;
    const int w = seg - f_spi.div(seg) * segs_per_img;
    const int wy = f_nwx.div(w), wx = w - wy * nwx;
    const int ry = min(window, grid_h - wy * window), rx = min(window, grid_w - wx * window);
    const int a = f_s.div(p), u = p - a * s;
    return u * stripes + a >= ry * rx;
  }

  // segment of a stripe-sorted segment row r (rows are segment-major, n per segment)
  __device__ __forceinline__ int seg_of(int r) const { return f_n.div(r); }

  __device__ __forceinline__ int row_of(int seg, int slot) const {
    const int img = f_spi.div(seg);
    int tok;
    if (window == 0) {
      tok = slot;
    } else {
      const int w = seg - img * segs_per_img;
      const int wy = f_nwx.div(w), wx = w - wy * nwx;
      const int ly = f_win.div(slot), lx = slot - ly * window;
      const int y = wy * window + ly, x = wx * window + lx;
      if (y >= grid_h || x >= grid_w) return -1;
      tok = y * grid_w + x;
    }
    return img * grid_h * grid_w + tok;
  }
};

// One LayerNorm row of C = 256 NV fp32 channels held by a wavefront: lane l holds the
// float4 chunks l + 64 i. load() issues the row's and the affine parameters' loads;
// store() forms the fp32 statistics (two passes over the registers, biased variance, eps
// 1e-6) and writes the normalised row as bf16. The gathered LayerNorm and the fused
// permutation kernel both use it, so their rows are bit-identical.
template <int NV>
struct LnRow {
  f32x4 v[NV], g[NV], b[NV];
  __device__ __forceinline__ void load(const float* __restrict__ xrow, const float* __restrict__ gamma,
                                       const float* __restrict__ beta, int lane) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      g[i] = *reinterpret_cast<const f32x4*>(gamma + 4 * (lane + 64 * i));
      b[i] = *reinterpret_cast<const f32x4*>(beta + 4 * (lane + 64 * i));
    }
    const f32x4* xr = reinterpret_cast<const f32x4*>(xrow);
#pragma unroll
    for (int i = 0; i < NV; ++i) v[i] = xr[lane + 64 * i];
  }
  __device__ __forceinline__ void store(bf16_t* __restrict__ out, int lane) const {
    constexpr int C = NV * 256;
    float s = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i) s += (v[i][0] + v[i][1]) + (v[i][2] + v[i][3]);
    const float mean = wave_sum(s) * (1.0f / C);
    float q = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float d = v[i][e] - mean;
        q += d * d;
      }
    const float rstd = rsqrtf(wave_sum(q) * (1.0f / C) + 1e-6f);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = to_bf16((v[i][e] - mean) * rstd * g[i][e] + b[i][e]);
      *reinterpret_cast<bf16x4*>(out + 4 * (lane + 64 * i)) = w;
    }
  }
  // a zero row (window pads, rows outside x)
  static __device__ __forceinline__ void zero(bf16_t* __restrict__ out, int lane) {
#pragma unroll
    for (int i = 0; i < NV; ++i) *reinterpret_cast<bf16x4*>(out + 4 * (lane + 64 * i)) = bf16x4{};
  }
};

}  // namespace sparsesam

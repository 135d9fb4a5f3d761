// Device-side helpers shared by the SparseSAM kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sparsesam {

typedef __bf16 bf16_t;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;
typedef __attribute__((__vector_size__(2 * sizeof(int)))) int i32x2;

constexpr int kWave = 64;

// s_waitcnt immediate for "at most n vector-memory operations outstanding" (other
// counters unconstrained), in the gfx9 encoding: vmcnt[3:0], expcnt[6:4],
// lgkmcnt[11:8], vmcnt[5:4] in bits [15:14].
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

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

// GELU with the exact Gaussian CDF.
__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }

// Image-token row of a segment slot. Global segments map slot -> token directly;
// windowed segments map (window, slot) through the padded window grid. Returns -1
// for a pad slot.
struct SegmentMap {
  int grid_h, grid_w, window, nwx, segs_per_img, n;

  __device__ __forceinline__ int row_of(int seg, int slot) const {
    int img = seg / segs_per_img;
    int tok;
    if (window == 0) {
      tok = slot;
    } else {
      int w = seg - img * segs_per_img;
      int wy = w / nwx, wx = w - wy * nwx;
      int ly = slot / window, lx = slot - ly * window;
      int y = wy * window + ly, x = wx * window + lx;
      if (y >= grid_h || x >= grid_w) return -1;
      tok = y * grid_w + x;
    }
    return img * grid_h * grid_w + tok;
  }
};

}  // namespace sparsesam

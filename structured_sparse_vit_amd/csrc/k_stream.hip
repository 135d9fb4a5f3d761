// Residual stream kept in stripe-sorted order across the blocks of an encoder.
//
// "Technische Samenvatting: SparseSAM", Methodologie, closing paragraph of part 2: one
// precomputed permutation set serves every layer, so the per-layer overhead stays
// negligible; the Probleemstelling's token-merging bullet names the per-layer
// scatter-gather passes as what sinks token merging. With the stream kept in the
// stripe-sorted order of the current block type, a block reads its rows in place (no
// gather through perm, pads found from their rank alone) and its residual epilogues
// write them in place (no scatter). Only a change of block type moves the stream, by
// one composed gather: every destination row finds its token through the destination
// layout's perm and that token's row in the source layout through the source inv.
//
// reorder_kernel: one wavefront per destination row, 16-byte copies; pad rows of a
// windowed layout are written as zeros.
#include "internal.hpp"

namespace sparsesam {

// Image row (image * tokens + token) held by stream row r, or -1 for a window pad.
__device__ __forceinline__ int stream_token(const StreamLayout& L, int r) {
  if (!L.perm) return r;
  return L.map.row_of(L.map.seg_of(r), L.perm[r]);
}

// Stream row holding image row t.
__device__ __forceinline__ int stream_row(const StreamLayout& L, int t) {
  if (!L.perm) return t;
  const SegmentMap& m = L.map;
  const int tokens = m.grid_h * m.grid_w;
  const int img = t / tokens, tok = t - img * tokens;
  int seg = img, slot = tok;
  if (m.window) {
    const int y = tok / m.grid_w, x = tok - (tok / m.grid_w) * m.grid_w;
    const int wy = y / m.window, wx = x / m.window;
    seg = img * m.segs_per_img + wy * m.nwx + wx;
    slot = (y - wy * m.window) * m.window + (x - wx * m.window);
  }
  return seg * m.n + L.inv[(size_t)seg * m.n + slot];
}

__global__ void __launch_bounds__(256) reorder_kernel(float* __restrict__ dst, const float* __restrict__ src,
                                                      int rows, int C, StreamLayout to, StreamLayout from) {
  const int lane = threadIdx.x & 63;
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int t = stream_token(to, r);
  f32x4* o = reinterpret_cast<f32x4*>(dst + (size_t)r * C);
  const int c4 = C / 4;
  if (t < 0) {
    for (int i = lane; i < c4; i += 64) o[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    return;
  }
  const f32x4* s = reinterpret_cast<const f32x4*>(src + (size_t)stream_row(from, t) * C);
  for (int i = lane; i < c4; i += 64) o[i] = s[i];
}

hipError_t launch_reorder(float* dst, const float* src, int rows, int C, const StreamLayout& to,
                          const StreamLayout& from, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(reorder_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, dst, src, rows, C, to, from);
  return hipGetLastError();
}

}  // namespace sparsesam

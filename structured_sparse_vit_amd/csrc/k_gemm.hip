// GEMMs of the block, C = A W^T, with fused epilogues.
//
// The QKV, output projection and MLP products stay dense over the rows they are
// given (the method sparsifies attention and routes MLP rows; it does not prune
// weights). bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation); the fp32 path is a plain SIMT kernel for small exact checks.
//
// bf16 kernel: BM x BN output tile (128 x 64 or 64 x 64) per 256-thread workgroup,
// K step 64, four wavefronts in a 2 x 2 layout each owning a (BM/2) x (BN/2) block of
// 32 x 32 MFMA tiles. A and W tiles go straight from global memory into LDS
// (global_load_lds_dwordx4, no register staging) through an ST-stage ring of swizzled
// 128-byte rows, with an explicit vmcnt wait and one barrier per K step; ST - 1 steps
// of loads stay in flight while one step multiplies. The tile grid is cut into one
// rectangle per XCD (each XCD's L2 then holds only the A and W rows it needs).
//
// Epilogue: the fp32 tile is staged in LDS, then written out as 16-byte chunks along
// the destination's contiguous axis -- 8 channels of one token for q, k, the MLP
// hidden activation and the residual stream, 8 tokens of one channel for the
// transposed V the attention kernel reads -- so every store is a full vector store
// and the index decoding (token -> segment, column -> head) runs once per chunk.
// (Storing straight from the accumulators, 4-element pieces of 32 rows per
// instruction, measured slower: four times the memory transactions.)
#include "internal.hpp"

namespace sparsesam {

// ---------------------------------------------------------------- epilogues

template <typename T>
__device__ __forceinline__ void store8(T* dst, const float* v);
template <>
__device__ __forceinline__ void store8<bf16_t>(bf16_t* dst, const float* v) {
  bf16x8 p;
#pragma unroll
  for (int i = 0; i < 8; ++i) p[i] = to_bf16(v[i]);
  *reinterpret_cast<bf16x8*>(dst) = p;
}
template <>
__device__ __forceinline__ void store8<float>(float* dst, const float* v) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

// Batched epilogues. Each thread of a tile owns a fixed 8-column chunk c..c+7 of ITER
// rows (row-major destinations) or a fixed 8-token chunk of ITER channels (V^T). What
// the epilogue reads from global memory -- the bias chunk, the residual rows' source
// indices -- is requested before the K loop (row_prefetch / col_prefetch), and the
// residual stream is read for all ITER rows before any of them is written, so the
// latency of those loads is paid once per tile instead of once per row in sequence.
template <int ITER>
struct RowPre {
  float b[8];
  int raw[ITER];
};

__device__ __forceinline__ void load_bias8(const float* bias, int c, int N, float* b) {
  if (c + 8 <= N) {
    const f32x4 b0 = *reinterpret_cast<const f32x4*>(bias + c);
    const f32x4 b1 = *reinterpret_cast<const f32x4*>(bias + c + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      b[i] = b0[i];
      b[4 + i] = b1[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = c + i < N ? bias[c + i] : 0.0f;
  }
}

// q, k [seg, H, N, D] and V^T [seg, H, D, N_pad] from the columns of the QKV product.
// Token r of the stripe-sorted rows is slot p of segment seg; column c is channel d of
// head h of part `which` (q, k, v). Divisions by n, C and D use FastDiv.
template <typename T>
struct QKVStore {
  const float* bias;
  T *q, *k, *vt;
  int n, n_pad, heads, D, C;
  FastDiv f_n, f_C, f_D;

  // One store through a selected base pointer and index. (A three-way if / else-if /
  // else with a store in each arm was compiled for gfx950 into code that sent the V^T
  // stores through the k pointer; selects avoid that shape.)
  __device__ __forceinline__ void elem(int r, int c, float v) const {
    v += bias[c];
    const int which = f_C.div(c);
    const int cc = c - which * C;
    const int h = f_D.div(cc), d = cc - h * D;
    const int seg = f_n.div(r), p = r - seg * n;
    const size_t sh = (size_t)seg * heads + h;
    const bool is_v = which >= 2;
    const size_t idx = is_v ? (sh * D + d) * (size_t)n_pad + p : (sh * n + p) * (size_t)D + d;
    T* base = is_v ? vt : (which == 0 ? q : k);
    base[idx] = from_f32<T>(v);
  }
  // Tiles whose columns are all V columns are written along tokens.
  __device__ __forceinline__ bool col_tile(int c0) const { return c0 >= 2 * C; }
  // Eight channels c..c+7 of token r (c % 8 == 0 and D % 8 == 0: one head, one part).
  __device__ __forceinline__ void row8(int r, int c, const float* v) const {
    const int which = f_C.div(c);
    if (which >= 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) elem(r, c + i, v[i]);
      return;
    }
    const int cc = c - which * C;
    const int h = f_D.div(cc), d = cc - h * D;
    const int seg = f_n.div(r), p = r - seg * n;
    const size_t sh = (size_t)seg * heads + h;
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = v[i] + bias[c + i];
    T* base = which == 0 ? q : k;
    store8<T>(base + (sh * n + p) * (size_t)D + d, w);
  }
  // Eight tokens r..r+7 (r % 8 == 0, count of them below M) of channel c.
  __device__ __forceinline__ void col8(int r, int c, const float* v, int count) const {
    const int seg = f_n.div(r), p = r - seg * n;
    const int which = f_C.div(c);
    if (which == 2 && count == 8 && p + 8 <= n && (p & 7) == 0) {
      const int cc = c - 2 * C;
      const int h = f_D.div(cc), d = cc - h * D;
      const size_t sh = (size_t)seg * heads + h;
      const float b = bias[c];
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = v[i] + b;
      store8<T>(vt + (sh * D + d) * (size_t)n_pad + p, w);
      return;
    }
    for (int i = 0; i < count; ++i) elem(r + i, c, v[i]);
  }

  template <int ITER>
  __device__ __forceinline__ void row_prefetch(RowPre<ITER>& pre, const int*, int c, int, int N) const {
    if (c < N) load_bias8(bias, c, N, pre.b);
  }
  template <int ITER>
  __device__ __forceinline__ void row_store(const RowPre<ITER>& pre, const int* ms, int c, const float (*v)[8], int M,
                                            int N) const {
    if (c >= N) return;
    const int which = f_C.div(c);
    if (c + 8 > N || which >= 2) {  // not a whole chunk of one q / k head: element by element
#pragma unroll
      for (int it = 0; it < ITER; ++it)
        if (ms[it] < M)
          for (int i = 0; i < 8 && c + i < N; ++i) elem(ms[it], c + i, v[it][i]);
      return;
    }
    const int cc = c - which * C;
    const int h = f_D.div(cc), d = cc - h * D;
    T* base = (which == 0 ? q : k) + (size_t)h * n * D + d;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int m = ms[it];
      if (m >= M) continue;
      const int seg = f_n.div(m), p = m - seg * n;
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = v[it][i] + pre.b[i];
      store8<T>(base + ((size_t)seg * heads * n + p) * (size_t)D, w);
    }
  }
  __device__ __forceinline__ float col_bias(int c, int N) const { return c < N ? bias[c] : 0.0f; }
  // Eight tokens r..r+7 of channel c with the channel's bias b already loaded.
  __device__ __forceinline__ void col8b(int r, int c, const float* v, int count, float b) const {
    const int seg = f_n.div(r), p = r - seg * n;
    const int which = f_C.div(c);
    if (which == 2 && count == 8 && p + 8 <= n && (p & 7) == 0) {
      const int cc = c - 2 * C;
      const int h = f_D.div(cc), d = cc - h * D;
      const size_t sh = (size_t)seg * heads + h;
      float w[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) w[i] = v[i] + b;
      store8<T>(vt + (sh * D + d) * (size_t)n_pad + p, w);
      return;
    }
    for (int i = 0; i < count; ++i) elem(r + i, c, v[i]);
  }
};

// Hidden activation of the routed MLP: out[r, c] = GELU(acc + bias).
template <typename T>
struct GeluStore {
  const float* bias;
  T* out;
  int ld;
  __device__ __forceinline__ void elem(int r, int c, float v) const {
    out[(size_t)r * ld + c] = from_f32<T>(gelu_erf(v + bias[c]));
  }
  __device__ __forceinline__ bool col_tile(int) const { return false; }
  __device__ __forceinline__ void row8(int r, int c, const float* v) const {
    float w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = gelu_erf(v[i] + bias[c + i]);
    store8<T>(out + (size_t)r * ld + c, w);
  }
  __device__ __forceinline__ void col8(int r, int c, const float* v, int count) const {
    for (int i = 0; i < count; ++i) elem(r + i, c, v[i]);
  }
  template <int ITER>
  __device__ __forceinline__ void row_prefetch(RowPre<ITER>& pre, const int*, int c, int, int N) const {
    if (c < N) load_bias8(bias, c, N, pre.b);
  }
  template <int ITER>
  __device__ __forceinline__ void row_store(const RowPre<ITER>& pre, const int* ms, int c, const float (*v)[8], int M,
                                            int N) const {
    if (c >= N) return;
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const int m = ms[it];
      if (m >= M) continue;
      if (c + 8 <= N) {
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = gelu_erf(v[it][i] + pre.b[i]);
        store8<T>(out + (size_t)m * ld + c, w);
      } else {
        for (int i = 0; c + i < N; ++i) elem(m, c + i, v[it][i]);
      }
    }
  }
  __device__ __forceinline__ float col_bias(int, int) const { return 0.0f; }
  __device__ __forceinline__ void col8b(int r, int c, const float* v, int count, float) const { col8(r, c, v, count); }
};

// Residual update of the fp32 stream: x[dst(r), c] += acc + bias, where dst maps a
// stripe-sorted row back to its token (through perm and the segment map; pads have
// no destination) or takes it from an explicit row list (the keep-set).
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
    return map.row_of(map.seg_of(r), perm[r]);
  }
  __device__ __forceinline__ void elem(int r, int c, float v) const {
    const int row = dst_row(r);
    if (row < 0 || row >= x_rows) return;
    float* px = x + (size_t)row * ldx + c;
    *px = *px + (v + bias[c]);
  }
  __device__ __forceinline__ bool col_tile(int) const { return false; }
  __device__ __forceinline__ void row8(int r, int c, const float* v) const {
    const int row = dst_row(r);
    if (row < 0 || row >= x_rows) return;
    f32x4* px = reinterpret_cast<f32x4*>(x + (size_t)row * ldx + c);
    f32x4 a = px[0], b = px[1];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = a[i] + (v[i] + bias[c + i]);
      b[i] = b[i] + (v[4 + i] + bias[c + 4 + i]);
    }
    px[0] = a;
    px[1] = b;
  }
  __device__ __forceinline__ void col8(int r, int c, const float* v, int count) const {
    for (int i = 0; i < count; ++i) elem(r + i, c, v[i]);
  }
  template <int ITER>
  __device__ __forceinline__ void row_prefetch(RowPre<ITER>& pre, const int* ms, int c, int M, int N) const {
    if (c < N) load_bias8(bias, c, N, pre.b);
#pragma unroll
    for (int it = 0; it < ITER; ++it) pre.raw[it] = ms[it] < M ? (list ? list[ms[it]] : perm[ms[it]]) : -1;
  }
  template <int ITER>
  __device__ __forceinline__ void row_store(const RowPre<ITER>& pre, const int* ms, int c, const float (*v)[8], int M,
                                            int N) const {
    if (c >= N) return;
    if (c + 8 > N) {
#pragma unroll
      for (int it = 0; it < ITER; ++it)
        if (ms[it] < M)
          for (int i = 0; c + i < N; ++i) elem(ms[it], c + i, v[it][i]);
      return;
    }
    // destination rows, then every row's current values, then the updates
    long long off[ITER];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      int row = -1;
      if (ms[it] < M && pre.raw[it] >= 0) row = list ? pre.raw[it] : map.row_of(map.seg_of(ms[it]), pre.raw[it]);
      off[it] = (row < 0 || row >= x_rows) ? -1 : (long long)row * ldx + c;
    }
    f32x4 cur[ITER][2];
#pragma unroll
    for (int it = 0; it < ITER; ++it)
      if (off[it] >= 0) {
        cur[it][0] = *reinterpret_cast<const f32x4*>(x + off[it]);
        cur[it][1] = *reinterpret_cast<const f32x4*>(x + off[it] + 4);
      }
#pragma unroll
    for (int it = 0; it < ITER; ++it)
      if (off[it] >= 0) {
        f32x4 a = cur[it][0], b = cur[it][1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[i] = a[i] + (v[it][i] + pre.b[i]);
          b[i] = b[i] + (v[it][4 + i] + pre.b[4 + i]);
        }
        *reinterpret_cast<f32x4*>(x + off[it]) = a;
        *reinterpret_cast<f32x4*>(x + off[it] + 4) = b;
      }
  }
  __device__ __forceinline__ float col_bias(int, int) const { return 0.0f; }
  __device__ __forceinline__ void col8b(int r, int c, const float* v, int count, float) const { col8(r, c, v, count); }
};

// ---------------------------------------------------------------- bf16 MFMA GEMM

constexpr int BK = 64;  // K step: one 128-byte row of bf16 per tile row

// ST: LDS pipeline depth (ST - 1 K steps in flight while one is multiplied).
template <int BM, int BN, int ST>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave block (2 x 2 waves)
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int GROUPS = (BM + BN) / 8;     // 1 KiB groups (8 rows x 128 B) per stage
  static constexpr int LOADS = GROUPS / 4;         // direct-to-LDS loads per wave per stage
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int CT_LD = BN + 4;             // fp32 epilogue tile row stride
  static constexpr int CTT_LD = BM + 4;            // ... of the transposed tile (V^T tiles)
  static constexpr int CT_BYTES = (BM * CT_LD > BN * CTT_LD ? BM * CT_LD : BN * CTT_LD) * 4;
  static constexpr int PIPE_BYTES = ST * STAGE_BYTES;
  static constexpr int LDS_BYTES = PIPE_BYTES > CT_BYTES ? PIPE_BYTES : CT_BYTES;
};

// Tiles live in LDS in the swizzled 128-byte-row layout of swz() (common.hpp).

// wait until at most n of this wavefront's tile loads are in flight, then meet the
// other wavefronts; the empty asm keeps the compiler from moving LDS reads above it
template <int N>
__device__ __forceinline__ void stage_ready() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The main loop and epilogue of one tile. TR: the tile's columns are written along
// tokens (V^T), so the MFMA operands are swapped and the block accumulates C^T.
template <int BM, int BN, int ST, bool TR, class Epi>
__device__ __forceinline__ void gemm_bf16_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, int M,
                                               int N, int K, const Epi& epi, char* smem, int m0, int n0) {
  using TL = Tile<BM, BN, ST>;
  constexpr int kStages = ST;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[TL::MI][TL::NI];
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

  // Global source of this lane for each of its groups, as a byte offset from the tile's
  // first A row or W row (a scalar base that advances by one K step per step). Group
  // g < BM/8 holds A rows 8g..8g+7, the rest W rows; lane L fills row 8g + L/8 at chunk
  // position L%8, which holds logical chunk (L%8) ^ swz_key(8g + L/8). Rows past M or N
  // are clamped to the last row: the loads stay unconditional and those rows only reach
  // accumulators that are never stored.
  uint32_t voff[TL::LOADS];
#pragma unroll
  for (int i = 0; i < TL::LOADS; ++i) {
    const int g = wave + 4 * i;
    const int r = lane >> 3, lc = (lane & 7) ^ swz_key(8 * g + r);
    if (g < BM / 8) {
      const int gm = min(m0 + g * 8 + r, M - 1);
      voff[i] = (uint32_t)(((gm - m0) * K + lc * 8) * 2);
    } else {
      const int gn = min(n0 + (g - BM / 8) * 8 + r, N - 1);
      voff[i] = (uint32_t)(((gn - n0) * K + lc * 8) * 2);
    }
  }
  const char* a_base = reinterpret_cast<const char*>(A + (size_t)m0 * K);
  const char* w_base = reinterpret_cast<const char*>(W + (size_t)n0 * K);
  auto issue = [&](int kt) {
    char* base = smem + (kt % kStages) * TL::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < TL::LOADS; ++i) {
      const int g = wave + 4 * i;
      const char* src = (g < BM / 8 ? a_base : w_base) + kt * (BK * 2);
      __builtin_amdgcn_global_load_lds((const void*)(src + voff[i]),
                                       (__attribute__((address_space(3))) void*)(base + g * 1024), 16, 0, 0);
    }
  };

  // epilogue inputs requested now, consumed after the K loop (see RowPre)
  constexpr int CPR = BN / 8, ITER = BM * CPR / 256;  // row path: chunks per row, chunks per thread
  constexpr int RPC = BM / 8, ITERT = BN * RPC / 256;  // V^T path: chunks per channel, per thread
  static_assert(256 % CPR == 0 && 256 % RPC == 0, "fixed chunk per thread");
  const int ec = n0 + (tid % CPR) * 8;
  int ems[ITER];
#pragma unroll
  for (int it = 0; it < ITER; ++it) ems[it] = m0 + tid / CPR + it * (256 / CPR);
  RowPre<ITER> rpre;
  const int tm = m0 + (tid % RPC) * 8;
  float tb[ITERT];
  if constexpr (!TR) {
    epi.row_prefetch(rpre, ems, ec, M, N);
  } else {
#pragma unroll
    for (int it = 0; it < ITERT; ++it) tb[it] = epi.col_bias(n0 + tid / RPC + it * (256 / RPC), N);
  }

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s)
    if (s < nk) issue(s);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt must be complete; the later stages already issued (at most
    // kStages - 2 of them) may stay in flight
    static_assert(kStages >= 2 && kStages <= 5, "pipeline depth");
    const int later = min(kStages - 2, nk - 1 - kt);
    if (later <= 0)
      stage_ready<0>();
    else if (later == 1)
      stage_ready<TL::LOADS>();
    else if (later == 2)
      stage_ready<2 * TL::LOADS>();
    else
      stage_ready<3 * TL::LOADS>();
    if (kt + kStages - 1 < nk) issue(kt + kStages - 1);  // into the buffer read last step
    const char* As = smem + (kt % kStages) * TL::STAGE_BYTES;
    const char* Bs = As + BM * 128;
    // every fragment of the K step is requested before the first MFMA
    bf16x8 af[BK / 16][TL::MI], bfr[BK / 16][TL::NI];
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int c = ks * 2 + (lane >> 5);
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
        af[ks][i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * TL::WM + i * 32 + (lane & 31), c));
#pragma unroll
      for (int j = 0; j < TL::NI; ++j)
        bfr[ks][j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * TL::WN + j * 32 + (lane & 31), c));
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
#pragma unroll
      for (int i = 0; i < TL::MI; ++i)
#pragma unroll
        for (int j = 0; j < TL::NI; ++j) {
          if constexpr (!TR)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks][i], bfr[ks][j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[ks][j], af[ks][i], acc[i][j], 0, 0, 0);
        }
    }
  }
  // every wavefront is done reading the pipeline buffers before they become the
  // epilogue tile
  __syncthreads();

  // Stage the fp32 tile in LDS. A lane holds one column of four row quads per 32 x 32
  // block; on transposed tiles the block holds C^T, and the tile is staged as C^T
  // ([BN][BM + 4]) so both the stores here and the chunk reads below run along rows.
  float* ct = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < TL::MI; ++i)
#pragma unroll
    for (int j = 0; j < TL::NI; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int inner = (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
        const int outer = lane & 31;
        if constexpr (!TR)
          ct[(wm * TL::WM + i * 32 + inner) * TL::CT_LD + wn * TL::WN + j * 32 + outer] = acc[i][j][e];
        else
          ct[(wn * TL::WN + j * 32 + inner) * TL::CTT_LD + wm * TL::WM + i * 32 + outer] = acc[i][j][e];
      }
  __syncthreads();
  if constexpr (!TR) {
    float v[ITER][8];
#pragma unroll
    for (int it = 0; it < ITER; ++it) {
      const float* src = ct + (ems[it] - m0) * TL::CT_LD + (ec - n0);
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[it][i] = a[i];
        v[it][4 + i] = b[i];
      }
    }
    epi.row_store(rpre, ems, ec, v, M, N);
  } else {
#pragma unroll
    for (int it = 0; it < ITERT; ++it) {
      const int n = n0 + tid / RPC + it * (256 / RPC);
      if (tm >= M || n >= N) continue;
      const float* src = ct + (n - n0) * TL::CTT_LD + (tm - m0);
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 b = *reinterpret_cast<const f32x4*>(src + 4);
      const float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      epi.col8b(tm, n, v, min(8, M - tm), tb[it]);
    }
  }
}

// XCD rectangles: the (mt x nt) tile grid is cut into xa bands of tile rows times xb
// bands of tile columns (xa * xb = 8), one rectangle per XCD, so each XCD's L2 holds
// the A rows and W rows of its own rectangle. Workgroup hw runs on XCD hw % 8 and takes
// the (hw / 8)-th tile of that rectangle, tile rows fastest.
struct XcdRect {
  int xa, xb, mb, nb;  // bands, and tiles per band (ceil)
};

template <int BM, int BN, int ST, class Epi>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, Epi epi, XcdRect xr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nt = (N + BN - 1) / BN, mt = (M + BM - 1) / BM;
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  const int ra = x / xr.xb, rb = x - (x / xr.xb) * xr.xb;
  const int mi = ra * xr.mb + j % xr.mb, ni = rb * xr.nb + j / xr.mb;
  if (j >= xr.mb * xr.nb || mi >= mt || ni >= nt) return;
  const int m0 = mi * BM, n0 = ni * BN;
  if (epi.col_tile(n0))
    gemm_bf16_tile<BM, BN, ST, true>(A, W, M, N, K, epi, smem, m0, n0);
  else
    gemm_bf16_tile<BM, BN, ST, false>(A, W, M, N, K, epi, smem, m0, n0);
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

constexpr int FT = 64, FK = 16;

template <class Epi>
__global__ void __launch_bounds__(256) gemm_f32_kernel(const float* __restrict__ A, const float* __restrict__ W,
                                                       int M, int N, int K, Epi epi) {
  __shared__ float As[FK][FT + 1];
  __shared__ float Bs[FK][FT + 1];
  const int tid = threadIdx.x;
  const int n0 = blockIdx.x * FT, m0 = blockIdx.y * FT;
  const int ke = K;
  const int tr = tid / 16, tc = tid % 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < ke; k0 += FK) {
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
      if (m < M && n < N) epi.elem(m, n, acc[i][j]);
    }
}

// ---------------------------------------------------------------- launchers

template <int BM, int BN, int ST, class Epi>
static hipError_t run_bf16(const bf16_t* a, const bf16_t* w, int m, int n, int k, const Epi& e, hipStream_t st) {
  using TL = Tile<BM, BN, ST>;
  auto kern = gemm_bf16_kernel<BM, BN, ST, Epi>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, TL::LDS_BYTES);
  if (err != hipSuccess) return err;
  // pick the XCD split with the fewest tiles on the busiest XCD, then the smallest
  // per-XCD working set (A rows + W rows of a rectangle)
  const int mt = (m + BM - 1) / BM, nt = (n + BN - 1) / BN;
  XcdRect best{8, 1, (mt + 7) / 8, nt};
  long best_load = -1, best_ws = 0;
  for (int xa = 1; xa <= 8; xa *= 2) {
    const int xb = 8 / xa;
    const int mb = (mt + xa - 1) / xa, nb = (nt + xb - 1) / xb;
    const long load = (long)mb * nb;
    const long ws = (long)mb * BM + (long)nb * BN;
    if (best_load < 0 || load < best_load || (load == best_load && ws < best_ws)) {
      best = XcdRect{xa, xb, mb, nb};
      best_load = load;
      best_ws = ws;
    }
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)(kXcds * best_load)), dim3(256), TL::LDS_BYTES, st, a, w, m, n, k, e,
                     best);
  return hipGetLastError();
}

// Tile choice (measured on the ViT-B shapes): wide products (QKV, fc1) take 128 x 64
// tiles at two stages (48 KiB of LDS, three workgroups per CU); narrow ones (N <= 1024:
// the projection) 64 x 64 tiles, twice the workgroups; long K (fc2) 64 x 64 tiles with
// three steps in flight (64 KiB, two workgroups per CU). Resident workgroups matter
// more than pipeline depth at K = 768.
template <class Epi>
static hipError_t run(const bf16_t* a, const bf16_t* w, int m, int n, int k, const Epi& e, hipStream_t st) {
  if (k >= 2048) return run_bf16<64, 64, 4>(a, w, m, n, k, e, st);
  if (n <= 1024) return run_bf16<64, 64, 2>(a, w, m, n, k, e, st);
  return run_bf16<128, 64, 2>(a, w, m, n, k, e, st);
}

template <class Epi>
static hipError_t run(const float* a, const float* w, int m, int n, int k, const Epi& e, hipStream_t st) {
  dim3 grid((n + FT - 1) / FT, (m + FT - 1) / FT);
  hipLaunchKernelGGL(gemm_f32_kernel<Epi>, grid, dim3(256), 0, st, a, w, m, n, k, e);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm_qkv(const T* a, const T* w, int m, int k, const EpiQKV& e, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  QKVStore<T> s{e.bias, (T*)e.q, (T*)e.k, (T*)e.vt, e.n, e.n_pad, e.heads, e.head_dim, e.channels,
                FastDiv((uint32_t)e.n), FastDiv((uint32_t)e.channels), FastDiv((uint32_t)e.head_dim)};
  return run(a, w, m, 3 * e.channels, k, s, st);
}

template <typename T>
hipError_t launch_gemm_gelu(const T* a, const T* w, int m, int n, int k, const EpiGelu& e, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  GeluStore<T> s{e.bias, (T*)e.out, e.ld};
  return run(a, w, m, n, k, s, st);
}

template <typename T>
hipError_t launch_gemm_residual(const T* a, const T* w, int m, int n, int k, const EpiResidualScatter& e,
                                hipStream_t st) {
  if (m <= 0) return hipSuccess;
  ResidualAdd s{e.bias, e.x, e.perm, e.list, e.map, e.ldx, e.x_rows};
  return run(a, w, m, n, k, s, st);
}

template hipError_t launch_gemm_qkv<bf16_t>(const bf16_t*, const bf16_t*, int, int, const EpiQKV&, hipStream_t);
template hipError_t launch_gemm_qkv<float>(const float*, const float*, int, int, const EpiQKV&, hipStream_t);
template hipError_t launch_gemm_gelu<bf16_t>(const bf16_t*, const bf16_t*, int, int, int, const EpiGelu&, hipStream_t);
template hipError_t launch_gemm_gelu<float>(const float*, const float*, int, int, int, const EpiGelu&, hipStream_t);
template hipError_t launch_gemm_residual<bf16_t>(const bf16_t*, const bf16_t*, int, int, int,
                                                 const EpiResidualScatter&, hipStream_t);
template hipError_t launch_gemm_residual<float>(const float*, const float*, int, int, int, const EpiResidualScatter&,
                                                hipStream_t);

}  // namespace sparsesam

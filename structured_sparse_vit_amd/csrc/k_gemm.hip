// GEMMs of the block, C = A W^T, with fused epilogues.
//
// The QKV, output projection and MLP products stay dense over the rows they are
// given (the method sparsifies attention and routes MLP rows; it does not prune
// weights). bf16 operands run on the gfx950 matrix cores (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation); the fp32 path is a plain SIMT kernel for small exact checks.
//
// bf16 kernel: one BM x BN output tile per 256-thread workgroup, K step 64, four
// wavefronts in a 2 x 2 layout, each owning a (BM/2) x (BN/2) block of 32 x 32 MFMA
// tiles. Large products take large tiles (192 x 128 or 256 x 128) because an MI355X CU
// gets about 64 bytes per clock through L1 from its XCD's L2: a 128 x 64 tile needs 94
// bytes per clock at the matrix-core rate, a 192 x 128 tile 53. Short products take
// small tiles at several workgroups per CU (see pick_tile).
//
// A and W tiles go straight from global memory into LDS (global_load_lds_dwordx4, no
// register staging) through an ST-slot ring of swizzled 128-byte rows; every slot is
// filled before the first step, and a slot is refilled with step kt + ST as soon as
// step kt has been read out of it. The operand fragments of the next 16-wide K slice
// are read from LDS while the MFMAs of the current one run, across step boundaries
// too, so one wavefront per SIMD keeps its matrix core fed.
//
// Epilogue: after a barrier (every wavefront done with the ring), each wavefront stages
// its accumulators, one 32-row block at a time, in a private LDS area and reads them
// back so that every lane holds eight consecutive columns of one row and the lanes of
// a store instruction cover whole row segments; the epilogue then writes them as
// 16-byte (bf16) or 32-byte (fp32) chunks. Tiles written along tokens (the transposed
// V tiles of the QKV product) skip the staging: one v_permlane32_swap per register
// pair gives every lane eight consecutive tokens of one channel straight from the
// accumulators.
#include <algorithm>
#include <cmath>
#include <type_traits>

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

// Epilogue interface. rows(): a lane holds MR rows r[i] and NC column chunks c[j]
// (eight consecutive columns c[j] .. c[j] + 7, c[j] % 8 == 0), values v[i][j][0..7];
// rows >= M and columns >= N are not stored. cols(): the transposed form, NCOL columns
// c[j] and RC row chunks r[i] (eight consecutive rows), values v[j][i][0..7].
// col_tile(n0): the tile starting at column n0 is written along rows (cols()).

// q, k [seg, H, N, D] and V^T [seg, H, D, N_pad] from the columns of the QKV product.
// Row r of the stripe-sorted rows is slot p of segment seg; column c is channel d of
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
  static constexpr bool kRowSq = false;
  // Tiles whose columns are all V columns are written along tokens.
  __device__ __forceinline__ bool col_tile(int c0) const { return c0 >= 2 * C; }

  template <int MR, int NC>
  __device__ __forceinline__ void rows(const int (&r)[MR], const int (&c)[NC], float (&v)[MR][NC][8], int M,
                                       int N) const {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (c[j] >= N) continue;
      const int which = f_C.div(c[j]);
      if (c[j] + 8 > N || which >= 2) {  // not a whole chunk of one q / k head: element by element
#pragma unroll
        for (int i = 0; i < MR; ++i)
          if (r[i] < M)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (c[j] + e < N) elem(r[i], c[j] + e, v[i][j][e]);
        continue;
      }
      const int cc = c[j] - which * C;
      const int h = f_D.div(cc), d = cc - h * D;
      T* base = (which == 0 ? q : k) + (size_t)h * n * D + d;
      float b[8];
      load_bias8(bias, c[j], N, b);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        if (r[i] >= M) continue;
        const int seg = f_n.div(r[i]), p = r[i] - seg * n;
        float w[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) w[e] = v[i][j][e] + b[e];
        store8<T>(base + ((size_t)seg * heads * n + p) * (size_t)D, w);
      }
    }
  }
  template <int NCOL, int RC>
  __device__ __forceinline__ void cols(const int (&c)[NCOL], const int (&r)[RC], float (&v)[NCOL][RC][8], int M,
                                       int N) const {
#pragma unroll
    for (int j = 0; j < NCOL; ++j) {
      if (c[j] >= N) continue;
      const int cc = c[j] - 2 * C;
      const int h = f_D.div(cc), d = cc - h * D;
      const float b = bias[c[j]];
#pragma unroll
      for (int i = 0; i < RC; ++i) {
        if (r[i] >= M) continue;
        const int seg = f_n.div(r[i]), p = r[i] - seg * n;
        if (r[i] + 8 <= M && p + 8 <= n && (p & 7) == 0) {
          float w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = v[j][i][e] + b;
          store8<T>(vt + (((size_t)seg * heads + h) * D + d) * (size_t)n_pad + p, w);
        } else if constexpr (sizeof(T) == 2) {
          // Segments of a length 4 (mod 8) (the 196-token windows) start at multiples of
          // four rows, so each half of the chunk (rows r .. r+3, r+4 .. r+7; r a multiple of
          // 8) lies in one segment at a four-aligned position: one 8-byte store per half.
          if (r[i] + 8 <= M && (n & 3) == 0) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              const int rr = r[i] + 4 * hh;
              const int sg = f_n.div(rr), pp = rr - sg * n;
              bf16x4 w4;
#pragma unroll
              for (int e = 0; e < 4; ++e) w4[e] = to_bf16(v[j][i][4 * hh + e] + b);
              *reinterpret_cast<bf16x4*>(vt + (((size_t)sg * heads + h) * D + d) * (size_t)n_pad + pp) = w4;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (r[i] + e < M) elem(r[i] + e, c[j], v[j][i][e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (r[i] + e < M) elem(r[i] + e, c[j], v[j][i][e]);
        }
      }
    }
  }
};

// Hidden activation of the routed MLP: out[r, c] = GELU(acc + bias).
template <typename T>
struct GeluStore {
  const float* bias;
  T* out;
  int ld;
  static constexpr bool kRowSq = false;
  __device__ __forceinline__ void elem(int r, int c, float v) const {
    out[(size_t)r * ld + c] = from_f32<T>(gelu_erf(v + bias[c]));
  }
  __device__ __forceinline__ bool col_tile(int) const { return false; }
  template <int MR, int NC>
  __device__ __forceinline__ void rows(const int (&r)[MR], const int (&c)[NC], float (&v)[MR][NC][8], int M,
                                       int N) const {
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (c[j] >= N) continue;
      float b[8];
      load_bias8(bias, c[j], N, b);
#pragma unroll
      for (int i = 0; i < MR; ++i) {
        if (r[i] >= M) continue;
        if (c[j] + 8 <= N) {
          float w[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) w[e] = gelu_erf(v[i][j][e] + b[e]);
          store8<T>(out + (size_t)r[i] * ld + c[j], w);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (c[j] + e < N) elem(r[i], c[j] + e, v[i][j][e]);
        }
      }
    }
  }
  template <int NCOL, int RC>
  __device__ __forceinline__ void cols(const int (&c)[NCOL], const int (&r)[RC], float (&v)[NCOL][RC][8], int M,
                                       int N) const {
#pragma unroll
    for (int j = 0; j < NCOL; ++j)
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c[j] < N && r[i] + e < M) elem(r[i] + e, c[j], v[j][i][e]);
  }
};

// Residual update of the fp32 stream: x[dst(r), c] += acc + bias, where dst maps a
// stripe-sorted row back to its token (through perm and the segment map; pads have
// no destination) or takes it from an explicit row list (the keep-set). Optionally
// also the squared-update partial sums of each destination row (sq_part, the dynamic
// keep-set's scores) and the updates themselves by GEMM row (upd, the merge).
struct ResidualAdd {
  const float* bias;
  float* x;
  const int* perm;
  const int* list;
  SegmentMap map;
  int ldx;
  long long x_rows;
  float* sq_part;
  int sq_ld;
  float* upd;
  static constexpr bool kRowSq = true;
  __device__ __forceinline__ int dst_row(int r) const {
    if (list) return list[r];
    if (!perm) return r;  // stream in stripe-sorted order
    return map.row_of(map.seg_of(r), perm[r]);
  }
  __device__ __forceinline__ void elem(int r, int c, float v) const {
    const float u = v + bias[c];
    if (upd) upd[(size_t)r * ldx + c] = u;
    const int row = dst_row(r);
    if (row < 0 || row >= x_rows) return;
    float* px = x + (size_t)row * ldx + c;
    *px = *px + u;
  }
  // Squared-update partial sums of the staged epilogue: a lane holds eight columns c0..c0+7
  // of rows r[t]; the CPR consecutive lanes of one row cover the wavefront's column block
  // [cb0, cb0 + W) (W = 8 CPR, 32 or 64). Each lane squares and adds its eight updates in
  // order, the lanes of a row fold by xor shuffles (offsets 1, 2, ...), and the block's
  // first lane writes the sum (and, for W = 64, a zero into the second 32-column slot).
  template <int CPR, int MR>
  __device__ __forceinline__ void row_sq(const int (&r)[MR], int c0, float (&v)[MR][1][8], int M, int N,
                                         int cb0) const {
    float b[8];
    load_bias8(bias, c0, N, b);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int t = 0; t < MR; ++t) {
      float s = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float u = c0 + e < N ? v[t][0][e] + b[e] : 0.0f;
        s = s + u * u;
      }
#pragma unroll
      for (int o = 1; o < CPR; o <<= 1) s += __shfl_xor(s, o, 64);
      if (lane % CPR == 0 && r[t] < M) {
        const int row = dst_row(r[t]);
        if (row >= 0 && row < x_rows) {
          float* dst = sq_part + (size_t)row * sq_ld + cb0 / 32;
          dst[0] = s;
          if (CPR == 8 && cb0 / 32 + 1 < sq_ld) dst[1] = 0.0f;
        }
      }
    }
  }
  __device__ __forceinline__ bool col_tile(int) const { return false; }
  // destination rows, then every chunk's current values, then the updates: the loads
  // of a lane's whole tile part are in flight together
  template <int MR, int NC>
  __device__ __forceinline__ void rows(const int (&r)[MR], const int (&c)[NC], float (&v)[MR][NC][8], int M,
                                       int N) const {
    int raw[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) raw[i] = r[i] < M ? (list ? list[r[i]] : perm ? perm[r[i]] : r[i]) : -1;
    long long off[MR];
#pragma unroll
    for (int i = 0; i < MR; ++i) {
      int row = -1;
      if (raw[i] >= 0) row = (list || !perm) ? raw[i] : map.row_of(map.seg_of(r[i]), raw[i]);
      off[i] = (row < 0 || row >= x_rows) ? -1 : (long long)row * ldx;
    }
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      if (c[j] >= N) continue;
      if (c[j] + 8 > N) {
#pragma unroll
        for (int i = 0; i < MR; ++i)
          if (r[i] < M)
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (c[j] + e < N) {
                const float u = v[i][j][e] + bias[c[j] + e];
                if (upd) upd[(size_t)r[i] * ldx + c[j] + e] = u;
                if (off[i] >= 0) x[off[i] + c[j] + e] += u;
              }
        continue;
      }
      float b[8];
      load_bias8(bias, c[j], N, b);
      f32x4 cur[MR][2];
#pragma unroll
      for (int i = 0; i < MR; ++i)
        if (off[i] >= 0) {
          cur[i][0] = *reinterpret_cast<const f32x4*>(x + off[i] + c[j]);
          cur[i][1] = *reinterpret_cast<const f32x4*>(x + off[i] + c[j] + 4);
        }
#pragma unroll
      for (int i = 0; i < MR; ++i)
        if (off[i] >= 0) {
          f32x4 a = cur[i][0], d = cur[i][1];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = a[e] + (v[i][j][e] + b[e]);
            d[e] = d[e] + (v[i][j][4 + e] + b[4 + e]);
          }
          *reinterpret_cast<f32x4*>(x + off[i] + c[j]) = a;
          *reinterpret_cast<f32x4*>(x + off[i] + c[j] + 4) = d;
        }
      if (upd) {
#pragma unroll
        for (int i = 0; i < MR; ++i)
          if (r[i] < M) {
            float* pu = upd + (size_t)r[i] * ldx + c[j];
            *reinterpret_cast<f32x4*>(pu) =
                f32x4{v[i][j][0] + b[0], v[i][j][1] + b[1], v[i][j][2] + b[2], v[i][j][3] + b[3]};
            *reinterpret_cast<f32x4*>(pu + 4) =
                f32x4{v[i][j][4] + b[4], v[i][j][5] + b[5], v[i][j][6] + b[6], v[i][j][7] + b[7]};
          }
      }
    }
  }
  template <int NCOL, int RC>
  __device__ __forceinline__ void cols(const int (&c)[NCOL], const int (&r)[RC], float (&v)[NCOL][RC][8], int M,
                                       int N) const {
#pragma unroll
    for (int j = 0; j < NCOL; ++j)
#pragma unroll
      for (int i = 0; i < RC; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (c[j] < N && r[i] + e < M) elem(r[i] + e, c[j], v[j][i][e]);
  }
};

// ---------------------------------------------------------------- bf16 MFMA GEMM

constexpr int BK = 64;  // K step: one 128-byte row of bf16 per tile row

// ST: LDS ring slots (up to ST - 1 K steps in flight while one is multiplied).
template <int BM, int BN, int ST>
struct Tile {
  static constexpr int WM = BM / 2, WN = BN / 2;  // wave block (2 x 2 waves)
  static constexpr int MI = WM / 32, NI = WN / 32;
  static constexpr int LOADS = (BM + BN) / 32;     // 1 KiB groups (8 rows x 128 B) per wave per step
  static constexpr int STAGE_BYTES = (BM + BN) * 128;
  static constexpr int LDS_BYTES = ST * STAGE_BYTES;
  static_assert(WM % 32 == 0 && WN % 32 == 0 && (BM + BN) % 32 == 0, "tile shape");
  static_assert(ST >= 2 && ST <= 8, "ring depth");
};

// Tiles live in LDS in the swizzled 128-byte-row layout of swz() (common.hpp).

// Wait until at most n of this wavefront's tile loads are in flight and its LDS reads
// have returned, then meet the other wavefronts; the empty asm keeps the compiler from
// moving LDS reads above the barrier.
template <int N>
__device__ __forceinline__ void ring_sync() {
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(N) & lgkmcnt0_mask());
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
template <int LOADS, int ST>
__device__ __forceinline__ void ring_sync_n(int later) {  // later: whole steps allowed in flight
  static_assert(ST <= 8, "ring depth");
  switch (later) {
    case 0: ring_sync<0>(); break;
    case 1: ring_sync<(ST > 1 ? LOADS : 0)>(); break;
    case 2: ring_sync<(ST > 2 ? 2 * LOADS : 0)>(); break;
    case 3: ring_sync<(ST > 3 ? 3 * LOADS : 0)>(); break;
    case 4: ring_sync<(ST > 4 ? 4 * LOADS : 0)>(); break;
    case 5: ring_sync<(ST > 5 ? 5 * LOADS : 0)>(); break;
    default: ring_sync<(ST > 6 ? 6 * LOADS : 0)>(); break;
  }
}

// Eight consecutive outputs per lane from a 32 x 32 accumulator. A lane holds outer
// index l % 32 and inner indices 8 g + 4 (l / 32) + t for register 4 g + t; swapping
// groups 2p + 1 of the low half with groups 2p of the high half gives the low lanes
// inner 16p .. 16p + 7 and the high lanes 16p + 8 .. 16p + 15.
__device__ __forceinline__ void acc_chunk(const f32x16& a, int p, float* out) {
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a[8 * p + t]), __float_as_uint(a[8 * p + 4 + t]),
                                                    false, false);
    out[t] = __uint_as_float(s[0]);
    out[4 + t] = __uint_as_float(s[1]);
  }
}

// The K loop and epilogue of one tile. TR: the tile's columns are written along rows
// (V^T), so the accumulators hold C (lane = column) instead of C^T (lane = row).
template <int BM, int BN, int ST, bool TR, class Epi>
__device__ __forceinline__ void gemm_bf16_tile(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W, int M,
                                               int N, int K, const Epi& epi, char* smem, int m0, int n0) {
  using TL = Tile<BM, BN, ST>;
  constexpr int MI = TL::MI, NI = TL::NI;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
  const int wm = wave >> 1, wn = wave & 1;

  f32x16 acc[MI][NI];
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NI; ++j)
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
  // direct-to-LDS loads [i0, i1) of this wavefront's groups for step kt into `slot`
  auto issue = [&](int kt, int slot, int i0, int i1) {
    char* base = smem + slot * TL::STAGE_BYTES;
#pragma unroll
    for (int i = 0; i < TL::LOADS; ++i) {
      if (i < i0 || i >= i1) continue;
      const int g = wave + 4 * i;
      const char* src = (g < BM / 8 ? a_base : w_base) + kt * (BK * 2);
      __builtin_amdgcn_global_load_lds((const void*)(src + voff[i]),
                                       (__attribute__((address_space(3))) void*)(base + g * 1024), 16, 0, 0);
    }
  };
  const int nk = K / BK;
  // Fragments of 16-wide K slice ks of the step held in `slot`, one register set per
  // slice.
  bf16x8 fa[BK / 16][MI], fb[BK / 16][NI];
  auto read = [&](int slot, int ks) {
    const char* As = smem + slot * TL::STAGE_BYTES;
    const char* Bs = As + BM * 128;
    const int c = ks * 2 + hi;
#pragma unroll
    for (int i = 0; i < MI; ++i)
      fa[ks][i] = *reinterpret_cast<const bf16x8*>(As + swz(wm * TL::WM + i * 32 + l32, c));
#pragma unroll
    for (int j = 0; j < NI; ++j)
      fb[ks][j] = *reinterpret_cast<const bf16x8*>(Bs + swz(wn * TL::WN + j * 32 + l32, c));
  };
  // MFMA q (in (i, j) order) of slice ks
  auto mfma = [&](int ks, int q) {
    const int i = q / NI, j = q % NI;
    if constexpr (!TR)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[ks][i], fb[ks][j], acc[i][j], 0, 0, 0);
  };
  constexpr int QN = MI * NI;
  constexpr int Q1 = QN >= 4 ? 2 : 1;  // MFMAs issued ahead of a group's reads / barrier
  constexpr int SPOTS = 2 * (QN - Q1);  // places for the step's direct loads (slices 0, 1)
  // One K step kt. Every MFMA of the step is issued between the other instructions, so
  // the matrix core stays busy while the wavefront feeds LDS and its registers:
  //  - slice 0: the reads of slice 1, then the direct loads of step kt + ST - 1 (into
  //    the slot step kt - 1 used) spread one or two per MFMA;
  //  - slice 1: the reads of slices 2 and 3 (the whole step is then in registers), the
  //    rest of the direct loads;
  //  - slice 2: the ring barrier (step kt + 1 landed; every wavefront done with step
  //    kt), then the reads of slice 0 of step kt + 1;
  //  - slice 3: MFMAs only.
  // sched_barrier keeps the compiler from regrouping the pieces.
  auto step = [&](auto dma_tag, int kt, int later) {
    constexpr bool DMA = decltype(dma_tag)::value;
    const int slot = kt % ST;
    const int dslot = (kt + ST - 1) % ST;
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
      for (int q = 0; q < Q1; ++q) mfma(g, q);
      __builtin_amdgcn_sched_barrier(0);
      if (g == 0) {
        read(slot, 1);
        if constexpr (DMA && SPOTS == 0) issue(kt + ST - 1, dslot, 0, TL::LOADS);
      } else {
        read(slot, 2);
        read(slot, 3);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = Q1; q < QN; ++q) {
        mfma(g, q);
        if constexpr (DMA) {
          const int spot = g * (QN - Q1) + (q - Q1);
          const int i0 = spot * TL::LOADS / (SPOTS > 0 ? SPOTS : 1), i1 = (spot + 1) * TL::LOADS / (SPOTS > 0 ? SPOTS : 1);
          if (i1 > i0) {
            __builtin_amdgcn_sched_barrier(0);
            issue(kt + ST - 1, dslot, i0, i1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < Q1; ++q) mfma(2, q);
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      // step kt + 1 must have landed (`later` steps after it may stay in flight) and
      // every wavefront must be done reading step kt before its slot is refilled
      if constexpr (DMA)
        ring_sync<(ST - 2) * TL::LOADS>();
      else
        ring_sync_n<TL::LOADS, ST>(later);
      read((kt + 1) % ST, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int q = Q1; q < QN; ++q) mfma(2, q);
#pragma unroll
    for (int q = 0; q < QN; ++q) mfma(3, q);
  };

  // slots 0 .. ST - 2 are filled up front; step kt fills slot (kt + ST - 1) % ST
#pragma unroll
  for (int s = 0; s < ST - 1; ++s)
    if (s < nk) issue(s, s, 0, TL::LOADS);
  ring_sync_n<TL::LOADS, ST>(min(ST - 2, nk - 1));
  read(0, 0);
  int kt = 0;
  for (; kt + ST - 1 < nk; ++kt) step(std::true_type{}, kt, ST - 2);
  for (; kt < nk; ++kt) step(std::false_type{}, kt, min(ST - 2, nk - 2 - kt));

  if constexpr (!TR) {
    // Staged through LDS, one 32-row block per wavefront at a time: the accumulators
    // (lane = row l32, four consecutive columns per register group) go into a private
    // [32][WN + 4] fp32 area, then every lane takes an eight-column chunk of R rows in
    // row-contiguous lane order, so a store instruction covers 64 / CPR whole row
    // segments (full cache lines) instead of 32 short pieces.
    constexpr int SLD = TL::WN + 4;
    constexpr int CPR = TL::WN / 8, RPI = 64 / CPR, R = 32 / RPI;
    static_assert(64 % CPR == 0 && 32 % RPI == 0, "staging layout");
    __syncthreads();  // every wavefront is done reading the ring
    float* stg = reinterpret_cast<float*>(smem) + wave * 32 * SLD;
    const int ch = lane % CPR, r0 = lane / CPR;
    int cc[1] = {n0 + wn * TL::WN + ch * 8};
#pragma unroll
    for (int i = 0; i < MI; ++i) {
#pragma unroll
      for (int j = 0; j < NI; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(stg + l32 * SLD + j * 32 + 8 * g + 4 * hi) =
              f32x4{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
      int r[R];
      float v[R][1][8];
#pragma unroll
      for (int t = 0; t < R; ++t) {
        const int row = r0 + t * RPI;
        r[t] = m0 + wm * TL::WM + i * 32 + row;
        const f32x4 a = *reinterpret_cast<const f32x4*>(stg + row * SLD + ch * 8);
        const f32x4 b = *reinterpret_cast<const f32x4*>(stg + row * SLD + ch * 8 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[t][0][e] = a[e];
          v[t][0][4 + e] = b[e];
        }
      }
      epi.rows(r, cc, v, M, N);
      if constexpr (Epi::kRowSq) {
        if (epi.sq_part) epi.template row_sq<CPR>(r, cc[0], v, M, N, n0 + wn * TL::WN);
      }
    }
  } else {
    // lane: column wn*WN + 32j + l32; rows wm*WM + 32i + 16p + 8hi .. + 7
    int r[MI * 2];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int p = 0; p < 2; ++p) r[i * 2 + p] = m0 + wm * TL::WM + i * 32 + 16 * p + 8 * hi;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int c[1] = {n0 + wn * TL::WN + j * 32 + l32};
      float v[1][MI * 2][8];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int p = 0; p < 2; ++p) acc_chunk(acc[i][j], p, v[0][i * 2 + p]);
      epi.cols(c, r, v, M, N);
    }
  }
}

// XCD rectangles: the (mt x nt) tile grid is cut into xa bands of tile rows times xb
// bands of tile columns (xa * xb = 8), one rectangle per XCD, so each XCD's L2 holds
// the A rows and W rows of its own rectangle. Workgroup hw runs on XCD hw % 8 and takes
// the (hw / 8)-th tile of that rectangle. The rectangle is walked in groups of gm tile
// rows, tile rows fastest inside a group, so the workgroups resident on an XCD at one
// time cover about gm rows by (resident / gm) columns of tiles and share their A and W
// panels in the L2 (walking a whole band of rows at a time made every column of tiles
// fetch the band's A rows again).
struct XcdRect {
  int xa, xb, mb, nb;  // bands, and tiles per band (ceil)
  int gm;              // tile rows per group, 1 .. mb
};

template <int BM, int BN, int ST, class Epi>
__global__ void __launch_bounds__(256) gemm_bf16_kernel(const bf16_t* __restrict__ A, const bf16_t* __restrict__ W,
                                                        int M, int N, int K, Epi epi, XcdRect xr) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int nt = (N + BN - 1) / BN, mt = (M + BM - 1) / BM;
  const int x = blockIdx.x % kXcds, j = blockIdx.x / kXcds;
  if (j >= xr.mb * xr.nb) return;
  const int ra = x / xr.xb, rb = x - (x / xr.xb) * xr.xb;
  const int grp = xr.gm * xr.nb, gi = j / grp, jj = j - gi * grp;
  const int rows = min(xr.gm, xr.mb - gi * xr.gm);  // tile rows of this group
  const int mi = ra * xr.mb + gi * xr.gm + jj % rows, ni = rb * xr.nb + jj / rows;
  if (mi >= mt || ni >= nt) return;
  const int m0 = mi * BM, n0 = ni * BN;
  if (epi.col_tile(n0))
    gemm_bf16_tile<BM, BN, ST, true>(A, W, M, N, K, epi, smem, m0, n0);
  else
    gemm_bf16_tile<BM, BN, ST, false>(A, W, M, N, K, epi, smem, m0, n0);
}

// ---------------------------------------------------------------- fp32 SIMT GEMM

// 64 x 64 tiles, 256 threads (4 x 4 outputs each), K in slices of FK: a slice's A and W
// values are loaded into registers while the previous slice is multiplied, then stored to
// LDS (the loads of a slice are all issued before the first store, so a slice costs one
// round trip to memory, overlapped with the previous slice's arithmetic). Each output
// adds its K products in ascending k.
constexpr int FT = 64, FK = 32;
constexpr int FV = FT * FK / 256;  // values of A (and of W) per thread per slice

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
  float ra[FV], rb[FV];
  // value u of this thread in a slice: tile row (i / FK), slice column (i % FK), i = tid + 256 u
  auto fetch = [&](int k0) {
#pragma unroll
    for (int u = 0; u < FV; ++u) {
      const int i = tid + 256 * u, row = i / FK, kk = i % FK;
      const int gm = m0 + row, gn = n0 + row, gk = k0 + kk;
      ra[u] = (gm < M && gk < ke) ? A[(size_t)gm * K + gk] : 0.0f;
      rb[u] = (gn < N && gk < ke) ? W[(size_t)gn * K + gk] : 0.0f;
    }
  };
  fetch(0);
  for (int k0 = 0; k0 < ke; k0 += FK) {
#pragma unroll
    for (int u = 0; u < FV; ++u) {
      const int i = tid + 256 * u, row = i / FK, kk = i % FK;
      As[kk][row] = ra[u];
      Bs[kk][row] = rb[u];
    }
    __syncthreads();
    if (k0 + FK < ke) fetch(k0 + FK);  // the next slice, in flight during this one
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
  if constexpr (std::is_same_v<Epi, ResidualAdd>) {
    // the residual update: every current value requested before the first store (the
    // stores could alias later loads, so elem() by elem() would serialise them)
    long long off[4];
    float cur[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + tr + 16 * i;
      const int row = m < M ? epi.dst_row(m) : -1;
      off[i] = (row < 0 || row >= epi.x_rows) ? -1 : (long long)row * epi.ldx;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tc + 16 * j;
        cur[i][j] = (off[i] >= 0 && n < N) ? epi.x[off[i] + n] : 0.0f;
      }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int m = m0 + tr + 16 * i, n = n0 + tc + 16 * j;
        if (m >= M || n >= N) continue;
        const float u = acc[i][j] + epi.bias[n];
        if (epi.upd) epi.upd[(size_t)m * epi.ldx + n] = u;
        if (off[i] >= 0) epi.x[off[i] + n] = cur[i][j] + u;
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        int m = m0 + tr + 16 * i, n = n0 + tc + 16 * j;
        if (m < M && n < N) epi.elem(m, n, acc[i][j]);
      }
  }
  if constexpr (Epi::kRowSq) {
    // squared-update partial sums over the tile's 64 columns: each thread adds its four
    // columns in order, the 16 consecutive lanes of a row fold by xor shuffles, and lane
    // tc = 0 writes the sum into the slot of column n0 and a zero into the next one
    if (epi.sq_part) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = m0 + tr + 16 * i;
        float s = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + tc + 16 * j;
          const float u = n < N ? acc[i][j] + epi.bias[n] : 0.0f;
          s = s + u * u;
        }
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, 64);
        if (tc == 0 && m < M) {
          const int row = epi.dst_row(m);
          if (row >= 0 && row < epi.x_rows) {
            float* dst = epi.sq_part + (size_t)row * epi.sq_ld + n0 / 32;
            dst[0] = s;
            if (n0 / 32 + 1 < epi.sq_ld) dst[1] = 0.0f;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- launchers

template <int BM, int BN, int ST, class Epi>
static hipError_t run_bf16(const bf16_t* a, const bf16_t* w, int m, int n, int k, const Epi& e, hipStream_t st) {
  using TL = Tile<BM, BN, ST>;
  auto kern = gemm_bf16_kernel<BM, BN, ST, Epi>;
  hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, TL::LDS_BYTES);
  if (err != hipSuccess) return err;
  // XCD split: among the splits whose busiest XCD holds at most 5 % more tiles than the
  // fewest possible, the one that fetches the least (each row band of A is read by the
  // xb XCDs of its band, each column band of W by xa: m xb + n xa rows of K), then the
  // smallest per-XCD working set (A rows + W rows of a rectangle)
  const int mt = (m + BM - 1) / BM, nt = (n + BN - 1) / BN;
  long min_load = -1;
  for (int xa = 1; xa <= 8; xa *= 2) {
    const long load = (long)((mt + xa - 1) / xa) * ((nt + 8 / xa - 1) / (8 / xa));
    if (min_load < 0 || load < min_load) min_load = load;
  }
  XcdRect best{8, 1, (mt + 7) / 8, nt, 1};
  long best_load = -1, best_fetch = 0, best_ws = 0;
  for (int xa = 1; xa <= 8; xa *= 2) {
    const int xb = 8 / xa;
    const int mb = (mt + xa - 1) / xa, nb = (nt + xb - 1) / xb;
    const long load = (long)mb * nb;
    if (load * 20 > min_load * 21) continue;
    const long fetch = (long)m * xb + (long)n * xa;
    const long ws = (long)mb * BM + (long)nb * BN;
    if (best_load < 0 || fetch < best_fetch || (fetch == best_fetch && ws < best_ws)) {
      best = XcdRect{xa, xb, mb, nb, 1};
      best_load = load;
      best_fetch = fetch;
      best_ws = ws;
    }
  }
  // group height: the resident workgroups of an XCD (32 CUs times the workgroups the LDS
  // allows per CU) as a gm x (resident / gm) block that reads the fewest panel bytes,
  // gm ~ sqrt(resident BN / BM)
  const int per_cu = std::max(1, std::min(8, (int)((160 * 1024) / TL::LDS_BYTES)));
  const double g = std::sqrt(32.0 * per_cu * BN / BM);
  best.gm = std::max(1, std::min(best.mb, (int)(g + 0.5)));
  hipLaunchKernelGGL(kern, dim3((unsigned)(kXcds * best_load)), dim3(256), TL::LDS_BYTES, st, a, w, m, n, k, e,
                     best);
  return hipGetLastError();
}

// Tile shapes and ring depths. 256 x 128 with three slots takes 144 KiB of LDS (one
// workgroup per CU); 192 x 128 with two slots 80 KiB (two per CU, so one tile's
// epilogue and the next one's first loads overlap the other's K loop); 128 x 64 and
// 64 x 64 with two slots 48 and 32 KiB (three to five per CU); 128 x 64 with six slots
// 144 KiB and 192 x 128 with three slots 120 KiB (one per CU, deeper prefetch for long
// K).
enum class TileShape { t64x64, t128x64s2, t128x64, t192x128s2, t256x128, t64x128s4, t192x128s3 };

// Shape choice. Long K over few tiles (the ViT-B second MLP product, 1638 x 768 x 3072)
// takes 64 x 128 with four slots (two workgroups per CU; 3 % faster for that MLP than
// 128 x 64 with six slots at one per CU, which in turn beat 64 x 64, 64 x 64 with six
// slots and 128 x 64 with three); long K over at most one round of 192 x 128 tiles (the
// windowed ViT-B second MLP product, 6554 x 768 x 3072) takes 192 x 128 with three slots
// (3 % faster for the c3 block than the model's 128 x 64, in a sweep of eleven shapes
// over every product of the ViT-B/L/H blocks, where the model's choice was otherwise
// within noise of the fastest); narrow short products 64 x 64. Otherwise each shape's time is estimated as
// (rounds of resident workgroups) x (tile area per CU per round) / (efficiency), the
// efficiencies -- 1.0, 1.3, 0.8 and 0.3 for 256 x 128, 192 x 128, 128 x 64 and 64 x 64
// -- fitted to timings of every shape on MI355X over 25 ViT-B/L/H products (M x N x K
// from 1638 x 768 x 3072 to 78400 x 1280 x 1280); the fitted choice is within 3 % of
// the fastest shape on 20 of them and within 14 % on all.
// `align`: tiles must not straddle multiples of it (the QKV parts), 0 = no constraint.
static TileShape pick_tile(int m, int n, int k, int align) {
  auto tiles = [&](int bm, int bn) { return (long)((m + bm - 1) / bm) * ((n + bn - 1) / bn); };
  if (k >= 2048 && tiles(128, 64) <= 320 && align == 0) return TileShape::t64x128s4;
  if (k >= 2048 && tiles(192, 128) <= 256 && align == 0) return TileShape::t192x128s3;
  // narrow short products (the ViT-B projection, 4096 x 768 x 768): 64 x 64 measured
  // fastest, by 7 % to 15 % depending on the epilogue
  if (n <= 768 && (double)m * n * k < 1e10) return TileShape::t64x64;
  struct Cand {
    TileShape s;
    int bm, bn, per_cu;
    double eff;
  };
  const Cand cands[] = {{TileShape::t256x128, 256, 128, 1, 1.0},
                        {TileShape::t192x128s2, 192, 128, 2, 1.3},
                        {TileShape::t128x64s2, 128, 64, 3, 0.8},
                        {TileShape::t64x64, 64, 64, 5, 0.3}};
  TileShape best = TileShape::t128x64s2;
  double best_cost = -1.0;
  for (const Cand& c : cands) {
    if (align > 0 && align % c.bn != 0) continue;
    const long slots = 256L * c.per_cu;
    const long rounds = (tiles(c.bm, c.bn) + slots - 1) / slots;
    const double cost = (double)rounds * c.per_cu * c.bm * c.bn / c.eff;
    if (best_cost < 0 || cost < best_cost) {
      best = c.s;
      best_cost = cost;
    }
  }
  return best;
}

template <class Epi>
static hipError_t run(const bf16_t* a, const bf16_t* w, int m, int n, int k, const Epi& e, hipStream_t st,
                      int align = 0) {
  switch (pick_tile(m, n, k, align)) {
    case TileShape::t256x128: return run_bf16<256, 128, 3>(a, w, m, n, k, e, st);
    case TileShape::t192x128s2: return run_bf16<192, 128, 2>(a, w, m, n, k, e, st);
    case TileShape::t64x64: return run_bf16<64, 64, 2>(a, w, m, n, k, e, st);
    case TileShape::t128x64s2: return run_bf16<128, 64, 2>(a, w, m, n, k, e, st);
    case TileShape::t64x128s4: return run_bf16<64, 128, 4>(a, w, m, n, k, e, st);
    case TileShape::t192x128s3: return run_bf16<192, 128, 3>(a, w, m, n, k, e, st);
    default: return run_bf16<128, 64, 6>(a, w, m, n, k, e, st);
  }
}

template <class Epi>
static hipError_t run(const float* a, const float* w, int m, int n, int k, const Epi& e, hipStream_t st,
                      int = 0) {
  dim3 grid((n + FT - 1) / FT, (m + FT - 1) / FT);
  hipLaunchKernelGGL(gemm_f32_kernel<Epi>, grid, dim3(256), 0, st, a, w, m, n, k, e);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_gemm_qkv(const T* a, const T* w, int m, int k, const EpiQKV& e, hipStream_t st) {
  if (m <= 0) return hipSuccess;
  QKVStore<T> s{e.bias, (T*)e.q, (T*)e.k, (T*)e.vt, e.n, e.n_pad, e.heads, e.head_dim, e.channels,
                FastDiv((uint32_t)e.n), FastDiv((uint32_t)e.channels), FastDiv((uint32_t)e.head_dim)};
  return run(a, w, m, 3 * e.channels, k, s, st, e.channels);
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
  ResidualAdd s{e.bias, e.x, e.perm, e.list, e.map, e.ldx, e.x_rows, e.sq_part, e.sq_ld, e.upd};
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

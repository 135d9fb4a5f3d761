// Host-side plan and kernel launch interfaces of libsparsesam (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <string>
#include <vector>

#include "sparsesam.h"
#include "common.hpp"

// Longest key-tile list of one matrix-core attention work item; longer rows are split.
constexpr int kAttnItemTiles = 64;
// Segments up to this length (the windows) take the short-segment attention kernel.
constexpr int kShortMaxN = 256;
// The window kernel on 16-key blocks: wavefronts per workgroup, LDS slots at most, ints
// per query-group record.
constexpr int kWinWaves = 8;
constexpr int kWinMaxSlots = 256;
constexpr int kWinGroupInts = 20;

struct sparsesam_plan {
  sparsesam_plan_desc desc;
  int n = 0;              // tokens per segment (pads included)
  int n_pad = 0;          // n rounded up to a multiple of 8 (row stride of V^T)
  int s = 0;              // stripe length n / g
  int nbs = 0;            // tiles per stripe
  int tiles = 0;          // g * nbs
  int radius = 0;
  int segs_per_img = 1;
  int nwx = 1, nwy = 1;
  int tiles_kept = 0;
  long long pairs_kept = 0;
  double density = 0.0;
  int routed_per_image = 0;
  size_t block_ws = 0, mlp_ws = 0;

  // host copies of the static tables
  std::vector<int> row_ptr, col_idx;  // CSR of kept key tiles per query tile
  std::vector<int> tile_start, tile_len;
  std::vector<int> order;             // query tiles, longest row first
  std::vector<int> seg_k;             // keep-set size of each segment of an image
  std::vector<int> seg_off;           // exclusive prefix sum of seg_k (offset in the image's keep-set)
  // matrix-core attention work list, two int4 per item: {first, end kept-key index,
  // partial slot or -1, G | P << 4}, {query tiles of the G members}; members share one
  // kept-key list. Longest first; lists longer than the chunk limit are split into
  // single-tile items that write partials, merged per (query tile, first slot, chunks)
  // in `splits`
  std::vector<int> items, splits;
  int n_items = 0, n_split_rows = 0, n_slots = 0;
  int attn_resident_wgs = 0;          // workgroups of the attention kernel resident at once
  // short segments (n <= 256, the windows): tile of every position; for each 32-query
  // block the 32-key blocks holding any kept pair. The mask goes to the matrix cores:
  // key tiles with the same kept column form one class (pad keys a class of their own);
  // mask_class[k] is the class of key position k (nt32 * 32 entries), mask_row[t] the
  // bias of query tile t against each class (16 * mask_ksteps bf16: 0 kept, -2^100
  // masked, two per int). nt32 = 0: no short-segment kernel (more than 32 classes).
  std::vector<int> pos_tile, any32, mask_class, mask_row;
  int nt32 = 0, mask_ksteps = 0;
  // short segments on 16-key blocks (attn_win_kernel): key tiles kept by the same query
  // tiles form a class stored in consecutive LDS slots, cut into blocks of 16 (empty
  // slots masked); query positions with the same kept key tiles form groups of up to 16.
  // win_pos_slot[p] / win_slot_pos[s]: slot of position p and position of slot s (an
  // empty slot holds a real key of its class), both padded to 256 entries; win_groups:
  // kWinGroupInts ints per group (first key block, end, queries, 0, 16 positions or -1);
  // win_kb: key blocks (block | valid-slot mask << 16); win_wave: groups of wavefront w
  // are [win_wave[w], win_wave[w + 1]). win_nslots = 0: not available.
  std::vector<int> win_pos_slot, win_slot_pos, win_groups, win_kb, win_wave;
  int win_nslots = 0;
  // relative-position bias: segment shape (grid or window) and the bias table row of a
  // query: key rows at 0 .. rel_seg_h - 1, key columns at rel_xoff .., rel_tj entries
  // (0 when the segment is larger than 64 x 64: no bias support)
  int rel_seg_h = 0, rel_seg_w = 0, rel_xoff = 0, rel_tj = 0;

  // device copy (one allocation) on `device`
  int device = -1;
  void* dev = nullptr;
  const int* d_row_ptr = nullptr;
  const int* d_col_idx = nullptr;
  const int* d_tile_start = nullptr;
  const int* d_tile_len = nullptr;
  const int* d_order = nullptr;
  const int* d_seg_k = nullptr;
  const int* d_seg_off = nullptr;
  const int* d_items = nullptr;
  const int* d_splits = nullptr;
  const int* d_pos_tile = nullptr;
  const int* d_any32 = nullptr;
  const int* d_mask_class = nullptr;
  const int* d_mask_row = nullptr;
  const int* d_win_pos_slot = nullptr;
  const int* d_win_slot_pos = nullptr;
  const int* d_win_groups = nullptr;
  const int* d_win_kb = nullptr;
  const int* d_win_wave = nullptr;
  // keep-set of a stream kept in stripe-sorted order: the positions of ranks 0 .. K - 1
  // of every segment, (seg * n) + (rank % g) * S + rank / g, for max_batch images in
  // the keep-set layout (static: the keep-set is the first K ranks)
  std::vector<int> keep_pos;
  const int* d_keep_pos = nullptr;

  sparsesam::SegmentMap segmap() const {
    sparsesam::SegmentMap m;
    m.grid_h = desc.grid_h;
    m.grid_w = desc.grid_w;
    m.window = desc.window;
    m.nwx = nwx;
    m.segs_per_img = segs_per_img;
    m.n = n;
    m.f_spi = sparsesam::FastDiv((uint32_t)segs_per_img);
    m.f_nwx = sparsesam::FastDiv((uint32_t)nwx);
    m.f_win = sparsesam::FastDiv((uint32_t)(desc.window > 0 ? desc.window : 1));
    m.f_n = sparsesam::FastDiv((uint32_t)n);
    m.stripes = desc.stripes;
    m.s = s;
    m.f_s = sparsesam::FastDiv((uint32_t)s);
    return m;
  }
};

namespace sparsesam {

void set_error(const std::string& msg);
sparsesam_status hip_fail(hipError_t e, const char* where);

// Workspace carve-up of sparsesam_block / sparsesam_mlp.
struct BlockLayout {
  size_t h = 0, q = 0, k = 0, vt = 0, o = 0, part = 0, rel_table = 0, rel_kc = 0, total_attn = 0;
  // dynamic routing: squared-update partials [x rows, sq_ld] after the attention region
  // (read by the keep-set selection before the MLP region is written)
  size_t sq = 0, total_dyn = 0;
  int sq_ld = 0;
  size_t a2 = 0, hid = 0, total_mlp = 0;
  // merging: the keep-set's updates [routed rows, C] fp32 after the MLP region
  size_t upd = 0, total_merge = 0;
  size_t total() const { return std::max(std::max(total_attn, total_dyn), std::max(total_mlp, total_merge)); }
};
BlockLayout block_layout(const sparsesam_plan& p, int batch);
// Workspace carve-up of the relative-position bias: tables (sized for fp32 entries),
// key coordinates, then the attention partials.
struct RelLayout {
  size_t table = 0, kc = 0, part = 0, total = 0;
};
RelLayout relpos_layout(const sparsesam_plan& p, int segments);
size_t mlp_workspace(const sparsesam_plan& p, int routed_rows, size_t* a2, size_t* hid);

// ---- launches (each returns hipSuccess or the launch error) ----
hipError_t launch_importance(const float* img, int batch, int height, int width, int patch, float* imp,
                             hipStream_t st);
hipError_t launch_permute(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                          hipStream_t st);
// The permutation plus the block's first LayerNorm (bf16 rows in stripe-sorted order,
// the rows launch_gather_ln writes through perm), for plans where the ranking runs one
// wavefront per slot (bf16, N > 3840 tokens per segment, C = 768, 1024 or 1280).
bool permute_ln_fusable(const sparsesam_plan& p);
hipError_t launch_permute_ln(const sparsesam_plan& p, const float* imp, int batch, int* perm, int* inv, int* routed,
                             const float* x, long long x_rows, const float* gamma, const float* beta, bf16_t* out,
                             hipStream_t st);
// Keep-set of every segment by score (descending, ties to the lower slot, pads last):
// score [batch, tokens, parts] partial sums added in order; score_out (optional)
// receives each token's summed score.
hipError_t launch_route_topk(const sparsesam_plan& p, const float* score, int parts, int batch, int* routed,
                             float* score_out, hipStream_t st);
// Row order of a residual stream: raster image rows (perm null), or the stripe-sorted
// segment rows of a plan (its segment map, perm and inv for the batch).
struct StreamLayout {
  SegmentMap map;
  const int* perm = nullptr;
  const int* inv = nullptr;
};
// dst[r] = src[row of the same token in `from`] for the rows of layout `to` (C % 4 == 0);
// window pad rows of `to` become zero rows.
hipError_t launch_reorder(float* dst, const float* src, int rows, int C, const StreamLayout& to,
                          const StreamLayout& from, hipStream_t st);
// The merge of mlp_merge plans: every real token of a segment outside its keep-set gets
// the mean of the keep-set's updates upd [batch * routed_per_image, C] (rows in the
// keep-set's layout).
hipError_t launch_merge(const sparsesam_plan& p, float* x, int batch, const int* routed, const float* upd,
                        hipStream_t st);

// LayerNorm of gathered rows: out[r] = LN(x[src(r)]) for r < rows_out, zero rows for pads.
// Row source: stripe-sorted segment rows through perm; an explicit list; or, with both
// null, the row itself (x already in stripe-sorted order; pads by map.pad_position).
template <typename T>
hipError_t launch_gather_ln(const sparsesam_plan& p, const float* x, int x_rows, int rows_out, const int* perm,
                            const int* list, const float* g, const float* b, T* out, hipStream_t st);

// GEMM C = A W^T with fused epilogues (bf16 matrix cores or fp32 SIMT).
struct EpiQKV {  // q, k [seg, H, N, D]; vt [seg, H, D, N_pad]
  const float* bias;
  void* q;
  void* k;
  void* vt;
  int n, n_pad, heads, head_dim, channels;
};
struct EpiResidualScatter {  // x[map(r)] += acc + bias
  const float* bias;
  float* x;
  const int* perm;  // stripe-sorted rows -> slot (mode 0), or null
  const int* list;  // explicit row list (mode 1), or null
  SegmentMap map;
  int ldx;
  long long x_rows;  // rows of x; destination rows outside [0, x_rows) are skipped
  // with perm and list both null the destination is the row itself (a stream kept in
  // stripe-sorted order)
  // optional: squared-update partial sums, sq_part[dst row * sq_ld + column / 32] = the sum of
  // (acc + bias)^2 over a block of 32 or 64 columns starting at that column (a 64-column
  // block writes 0 into its second slot); sq_ld = ceil(N / 32)
  float* sq_part = nullptr;
  int sq_ld = 0;
  // optional: upd[r * ldx + c] = acc + bias (the update itself, by GEMM row r)
  float* upd = nullptr;
};
struct EpiGelu {  // out[r, c] = GELU(acc + bias)
  const float* bias;
  void* out;
  int ld;
};

template <typename T>
hipError_t launch_gemm_qkv(const T* a, const T* w, int m, int k, const EpiQKV& e, hipStream_t st);
template <typename T>
hipError_t launch_gemm_gelu(const T* a, const T* w, int m, int n, int k, const EpiGelu& e, hipStream_t st);
// Residual GEMM: x[dst(r)] += A W^T + bias, each element written once (deterministic).
template <typename T>
hipError_t launch_gemm_residual(const T* a, const T* w, int m, int n, int k, const EpiResidualScatter& e,
                                hipStream_t st);

template <typename T>
hipError_t launch_attention(const sparsesam_plan& p, int segments, const T* q, const T* k, const T* vt, T* o,
                            float scale, void* partial, hipStream_t st);
// The same attention with the relative-position bias of each segment added to the
// logits: `perm` gives each position's slot, rel_h / rel_w the fp32 tables; `table`,
// `kc` and `partial` are the RelLayout regions of the workspace.
template <typename T>
hipError_t launch_attention_relpos(const sparsesam_plan& p, int segments, const T* q, const T* k, const T* vt, T* o,
                                   float scale, const int* perm, const float* rel_h, const float* rel_w, void* table,
                                   int* kc, void* partial, hipStream_t st);
// bias tables T[segment, head, position, rel_tj] (exp2 units; TT fp16 or fp32) and key
// coordinates
template <typename T, typename TT>
hipError_t launch_relpos_table(const sparsesam_plan& p, int segments, const T* q, const int* perm,
                               const float* rel_h, const float* rel_w, TT* table, int* kc, hipStream_t st);
size_t relpos_lds_bytes(int head_dim);
bool attn_relpos_fused(const sparsesam_plan& p);
bool attn_long_supported(const sparsesam_plan& p);
int attn_long_resident_wgs(int device, int head_dim);
size_t attn_partial_bytes(const sparsesam_plan& p, int segments);

}  // namespace sparsesam

/*
 * sparsesam.h -- C ABI of the SparseSAM encoder-block hot path on MI355X (gfx950).
 *
 * The method: "SparseSAM: Structured Sparsification of Activations in Segment
 * Anything Models" (arXiv 2605.17633). Stripe-Sort Attention orders the tokens
 * of an image by Sobel gradient magnitude, stripe-sorts them, and runs attention
 * over a static banded block pattern; the Residual-Consistency MLP runs the MLP
 * only on the most important tokens and passes the others through the residual.
 * The steps are described in "Technische Samenvatting: SparseSAM" (gist.science),
 * section Methodologie, parts 1 (Stripe-Sort Attention) and 2 (Residual-Consistency
 * MLP), and in the arXiv abstract.
 *
 * Conventions for every call below.
 *  - Pointers are device pointers unless the comment says "host".
 *  - The caller owns every buffer; the library never frees caller memory and the
 *    five compute calls never allocate: scratch memory comes from the caller's
 *    workspace, sized by sparsesam_plan_get_info().
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream). Compute
 *    calls only enqueue work on it and never synchronise the host.
 *  - Host-side validation runs before any launch; a call that returns an error has
 *    enqueued nothing and written nothing. Launch failures return SPARSESAM_ERR_HIP.
 *    Device faults surface at the caller's next synchronisation, as for any HIP call.
 *  - sparsesam_last_error() returns a thread-local message for the last failure.
 *  - Matrices are row-major. Weight matrices are [out, in] (the layout of a
 *    torch.nn.Linear weight). Biases and LayerNorm parameters are always fp32. The
 *    residual stream x is always fp32.
 *  - A plan is immutable after creation and may be shared across threads and streams.
 *    Its device copy lives on the device that was current at creation; compute calls
 *    must run with that device current.
 */
#ifndef SPARSESAM_H
#define SPARSESAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sparsesam_status {
  SPARSESAM_OK = 0,
  SPARSESAM_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad size, inconsistent shapes */
  SPARSESAM_ERR_UNSUPPORTED = 2,      /* valid request that this build has no kernel for */
  SPARSESAM_ERR_WORKSPACE = 3,        /* workspace smaller than the plan requires */
  SPARSESAM_ERR_OUT_OF_MEMORY = 4,    /* host or device allocation in plan creation failed */
  SPARSESAM_ERR_HIP = 5,              /* a HIP runtime call or launch failed */
  SPARSESAM_ERR_NO_DEVICE = 6         /* the plan has no device copy (no GPU, or another device) */
} sparsesam_status;

typedef enum sparsesam_dtype {
  SPARSESAM_F32 = 0,  /* fp32 weights and activations everywhere (small configs, exactness) */
  SPARSESAM_BF16 = 1  /* bf16 weights and matrix-core operands, fp32 accumulation and residual */
} sparsesam_dtype;

typedef struct sparsesam_plan* sparsesam_plan_t;

/*
 * Token order ahead of the stripe-sort. "Technische Samenvatting: SparseSAM" (gist.science)
 * orders tokens by Sobel importance (method section, 1. Stripe-Sort Attention) and also
 * calls the ordering a Z-order (Morton) one (abstract); the SparseSAM README's method
 * registry lists random and Hilbert-curve orders beside it. The variants replace only the
 * sort key (ascending key, ties to the lower slot, window pads last); the stripe-sort, the
 * pattern and the keep-set (the first K of the same order) are unchanged. Keys come from a
 * slot's position in its segment ((y, x) on the grid, (ly, lx) in a window):
 *   ZORDER:  bit b of x at bit 2b, bit b of y at bit 2b + 1;
 *   HILBERT: index along the Hilbert curve of the smallest power-of-two square covering the
 *            segment, starting at (0, 0), quadrants visited (x, y) = (lo, lo), (lo, hi),
 *            (hi, hi), (hi, lo);
 *   RANDOM:  top 31 bits of the first SplitMix64 output from state order_seed * 2^32 + slot
 *            (the same order in every segment and image).
 */
typedef enum sparsesam_ordering {
  SPARSESAM_ORDER_IMPORTANCE = 0,
  SPARSESAM_ORDER_ZORDER = 1,
  SPARSESAM_ORDER_HILBERT = 2,
  SPARSESAM_ORDER_RANDOM = 3
} sparsesam_ordering;

/*
 * How a block picks the MLP keep-set of each segment ("Technische Samenvatting: SparseSAM",
 * Methodologie, 2. Residual-Consistency MLP: the token-routing bullet partitions the tokens by
 * the deterministic permutation order; the selective-computation bullet describes the keep-set
 * as the tokens of high feature dissimilarity or update magnitude). K is the same in both.
 *   IMPORTANCE: the first K tokens of the segment's importance order, computed once per image
 *               by sparsesam_permute and reused by every block of the plan.
 *   UPDATE:     per block, the K tokens whose update by this block's attention sub-block,
 *               x1 - x, has the largest squared L2 norm (fp32, ties to the lower slot, pads
 *               never chosen); blocks of such plans run through sparsesam_block_dynamic.
 */
typedef enum sparsesam_routing {
  SPARSESAM_ROUTE_IMPORTANCE = 0,
  SPARSESAM_ROUTE_UPDATE = 1
} sparsesam_routing;

/*
 * What one plan describes: the segments of an image (one global segment of
 * grid_h*grid_w tokens, or window x window windows over the grid padded up to
 * multiples of `window`), the stripe-sort and its static attention pattern, the
 * MLP keep-set size and the block's dimensions.
 *
 * Pattern ("Technische Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort
 * Attention, static-pattern bullet: a 4 x 4 mosaic of sub-maps with a banded
 * diagonal plus a small global keep-set). Reading used here: a segment of N tokens
 * is stripe-sorted into g = `stripes` stripes of S = N/g positions; position p is in
 * stripe a = p / S at offset u = p % S, in stripe-local block j = u / B (B = `block`,
 * the last block of a stripe may be shorter). The pair (p, q) is kept when
 * |j_p - j_q| <= r, or when p or q is global (a == 0 and u < G, G = `global_tokens`).
 * r = `band_radius`, or, when it is -1, the smallest r whose kept share of the
 * N x N map reaches `attn_density`.
 *
 * Keep-set (same page, 2. Residual-Consistency MLP): per segment the K most important
 * real tokens, K = floor(mlp_density * n_real + 0.5) computed in double, at least 1.
 */
typedef struct sparsesam_plan_desc {
  int32_t grid_h, grid_w;  /* token grid of one image (64 x 64 for SAM at 1024 px) */
  int32_t window;          /* 0: one global segment per image; w > 0: w x w windows */
  int32_t stripes;         /* g >= 1; N must be a multiple of g */
  int32_t block;           /* B: pattern tile in tokens, 1..S */
  int32_t global_tokens;   /* G: 0 <= G <= S */
  int32_t band_radius;     /* r >= 0, or -1 to derive r from attn_density */
  float attn_density;      /* in (0, 1] */
  float mlp_density;       /* in (0, 1] */
  int32_t channels;        /* C = heads * head_dim */
  int32_t heads;
  int32_t head_dim;
  int32_t mlp_hidden;
  int32_t max_batch;       /* largest batch a call will pass; sizes the workspace */
  int32_t dtype;           /* sparsesam_dtype */
  int32_t ordering;        /* sparsesam_ordering: the token order ahead of the stripe-sort (0 = importance) */
  uint32_t order_seed;     /* seed of SPARSESAM_ORDER_RANDOM */
  int32_t rel_pos;         /* 1: blocks add the relative-position bias (block weights rel_pos_h,
                              rel_pos_w; segments of at most 64 x 64); 0: no bias */
  int32_t routing;         /* sparsesam_routing: how a block picks its MLP keep-set */
  int32_t mlp_merge;       /* 1: a segment's tokens outside the keep-set receive the mean MLP update of
                              its keep-set (block calls only, segments of at most 16384 tokens);
                              0: they stay bitwise unchanged */
} sparsesam_plan_desc;

typedef struct sparsesam_plan_info {
  int32_t seq_len;              /* N: tokens per segment, pads included */
  int32_t segments_per_image;   /* 1, or the number of windows */
  int32_t band_radius;          /* r in use */
  int32_t tiles_per_stripe;     /* ceil(S / B) */
  int32_t tiles;                /* T = g * tiles_per_stripe (query tiles = key tiles) */
  int32_t tiles_kept;           /* kept (query tile, key tile) pairs of one segment */
  int64_t pairs_kept;           /* kept token pairs of one segment */
  double realised_density;      /* pairs_kept / N^2 */
  int32_t routed_per_image;     /* keep-set size summed over the segments of one image */
  int32_t reserved0;
  size_t block_workspace_bytes; /* workspace sparsesam_block needs at max_batch */
  size_t mlp_workspace_bytes;   /* workspace sparsesam_mlp needs for max_batch images' keep-sets */
  size_t attn_workspace_bytes;  /* workspace sparsesam_attn needs for max_batch images' segments
                                   (0 when the plan's attention needs none) */
  int32_t has_device_copy;      /* 1 when the plan can run on the current device */
  int32_t device;               /* HIP device of the device copy, -1 when none */
  size_t relpos_workspace_bytes; /* workspace sparsesam_attn_relpos needs for max_batch images'
                                    segments (0 when the segments exceed 64 x 64) */
} sparsesam_plan_info;

/* Plan lifecycle. sparsesam_plan_create validates the description, builds the
 * static tile list on the host and copies it to the current device when one is
 * present (host-only plans can be queried but not run). */
sparsesam_status sparsesam_plan_create(const sparsesam_plan_desc* desc /* host */, sparsesam_plan_t* out /* host */);
sparsesam_status sparsesam_plan_get_info(sparsesam_plan_t plan, sparsesam_plan_info* info /* host */);
/* The kept key tiles of every query tile, in CSR form: row_ptr[T + 1] and
 * col_idx[tiles_kept] (host buffers the caller sizes from the info). Tile t covers
 * stripe t / tiles_per_stripe, stripe-local block t % tiles_per_stripe. */
sparsesam_status sparsesam_plan_tile_list(sparsesam_plan_t plan, int32_t* row_ptr /* host */, int32_t* col_idx /* host */);
void sparsesam_plan_destroy(sparsesam_plan_t plan);
/* The same two queries under the names of the boundary's original listing: identical
 * arguments, behaviour and errors (sparsesam_plan_info_get = sparsesam_plan_get_info,
 * sparsesam_plan_block_list = sparsesam_plan_tile_list; a "block" of the pattern is one
 * B x B tile). */
sparsesam_status sparsesam_plan_info_get(sparsesam_plan_t plan, sparsesam_plan_info* info /* host */);
sparsesam_status sparsesam_plan_block_list(sparsesam_plan_t plan, int32_t* row_ptr /* host */,
                                           int32_t* col_idx /* host */);

const char* sparsesam_status_string(sparsesam_status status);
const char* sparsesam_last_error(void);

/*
 * (1) Token importance: per-pixel L2 magnitude of the unnormalised Sobel gradient
 * with zero padding, averaged over each patch x patch tile ("Technische
 * Samenvatting: SparseSAM", Methodologie, 1. Stripe-Sort Attention, the
 * gradient-based ordering bullet: a parameter-free Sobel operator measures local
 * information density).
 *   img [batch, height, width] fp32 grayscale; imp [batch, (height/patch) * (width/patch)]
 *   fp32, tokens in raster order. height and width must be multiples of patch.
 * Every operation rounds once to fp32 in a fixed order, so the result is exactly
 * reproducible: gx = ((P[y-1][x+1] + 2P[y][x+1]) + P[y+1][x+1]) - ((P[y-1][x-1] +
 * 2P[y][x-1]) + P[y+1][x-1]), gy likewise with rows, m = sqrt(gx*gx + gy*gy) correctly
 * rounded; each tile row is summed left to right, the row sums top to bottom, and
 * the total divided by patch^2.
 */
sparsesam_status sparsesam_importance(const float* img, int32_t batch, int32_t height, int32_t width,
                                      int32_t patch, float* imp, void* stream);

/*
 * (2) Stripe-sort permutation and keep-set of every segment of `batch` images
 * (same page, stripe-sort bullet; 2. Residual-Consistency MLP, token routing).
 *   imp    [batch, grid_h * grid_w] fp32.
 *   perm   [batch * segments_per_image, N] int32: segment-local slot at each position
 *          of the stripe-sorted sequence (slot = token index in raster order within the
 *          global grid or within the window).
 *   inv    [batch * segments_per_image, N] int32: inv[perm[p]] = p.
 *   routed [batch * routed_per_image] int32: global row ids (image * grid_h * grid_w +
 *          token) of the keep-set. Per image, segment by segment (segment w starts at
 *          the sum of the keep-set sizes of segments 0..w-1), each segment's K tokens in
 *          the order below: most important first.
 * Order (plan ordering IMPORTANCE): importance descending, ties by lower slot, -0.0 ==
 * +0.0, NaN after every number, window pad slots after every real slot (so no pad enters
 * the keep-set); the other orderings replace the importance key as described at
 * sparsesam_ordering (imp is then not read). The
 * stripe-sort reads the sorted list as an (N/g) x g matrix, transposes it and
 * flattens it: perm[p] = sorted[g * (p % S) + p / S]. All outputs are integers and
 * exactly determined.
 */
sparsesam_status sparsesam_permute(sparsesam_plan_t plan, const float* imp, int32_t batch, int32_t* perm,
                                   int32_t* inv, int32_t* routed, void* stream);

/*
 * (3) Block-sparse attention over the plan's static pattern, on already
 * stripe-sorted tokens (same page, static-pattern bullet: the pattern is fixed, so
 * no mask is built at run time). For each segment s and head h:
 *   o[s, p, h, :] = sum_q softmax_q(scale * <q[s,h,p,:], k[s,h,q,:]>) v[s,h,q,:]
 * over the kept positions q of row p only.
 *   q, k [segments, heads, N, head_dim]       (plan dtype)
 *   vt   [segments, heads, head_dim, N_pad]   (plan dtype; V transposed, N_pad = N
 *                                              rounded up to a multiple of 8; columns
 *                                              N..N_pad-1 are never read)
 *   o    [segments, N, heads * head_dim]      (plan dtype)
 * `scale` must be positive; usually head_dim^-0.5. Rows with long key lists may be split
 * into pieces whose partial results go through `workspace` (fp32 partial sums, running
 * max and running sum); it must hold attn_workspace_bytes scaled to `segments`
 * (attn_workspace_bytes / (max_batch * segments_per_image) bytes per segment) and may
 * be NULL when that is 0.
 */
sparsesam_status sparsesam_attn(sparsesam_plan_t plan, int32_t segments, const void* q, const void* k,
                                const void* vt, void* o, float scale, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * (3b) The attention (3) with SAM's decomposed relative-position bias added to every
 * kept logit. The SparseSAM README's repository layout names fused "FA2 + rel-pos"
 * kernels; the pages do not define the bias, and the reading taken is SAM's image
 * encoder's (Kirillov et al. 2023, after MViTv2, Li et al. 2022). For a query at
 * segment coordinates (y, x) and a key at (y', x'):
 *   logit = scale * <q, k> + <q, rel_h[y - y' + Sh - 1]> + <q, rel_w[x - x' + Sw - 1]>
 * with the unscaled q, Sh x Sw the segment shape (grid_h x grid_w, or window x window
 * with pads at their padded-window coordinates) and a slot's coordinates
 * (slot / Sw, slot % Sw).
 *   perm   [segments, N] int32: the slot at each position (sparsesam_permute's perm of
 *          the same segments); values are clamped into [0, N).
 *   rel_h  [2 Sh - 1, head_dim] fp32, rel_w [2 Sw - 1, head_dim] fp32 (shared by heads),
 *          16-byte aligned.
 *   q, k, vt, o, scale as in (3). Sh and Sw must be at most 64 and head_dim at most 80
 *   (UNSUPPORTED otherwise).
 * The bias is evaluated once per (segment, head, position) into a table in fp32 from
 * the stored q; bf16 plans with head_dim 64 and a 64 x 64 grid keep the table in fp16
 * (clamped to +-65504) and run it on the matrix cores, the others use fp32 tables. workspace must hold
 * relpos_workspace_bytes scaled to `segments` (bytes per segment =
 * relpos_workspace_bytes / (max_batch * segments_per_image)).
 */
sparsesam_status sparsesam_attn_relpos(sparsesam_plan_t plan, int32_t segments, const void* q, const void* k,
                                       const void* vt, void* o, float scale, const int32_t* perm,
                                       const float* rel_h, const float* rel_w, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * (4) Residual-Consistency MLP, in place on the fp32 residual stream (same page,
 * 2. Residual-Consistency MLP: the MLP runs on the keep-set only; every other token
 * passes through the residual unchanged). For each row t in routed:
 *   x[t] += fc2(GELU(fc1(LayerNorm(x[t]))))   (exact-erf GELU, LayerNorm eps 1e-6)
 * Rows not in `routed` are never read or written.
 * Plans with mlp_merge = 1 are not taken (UNSUPPORTED): the merge needs the segments, which
 * the block calls have.
 *   x [rows, C] fp32; routed [routed_count] int32 distinct row ids in [0, rows);
 *   ln_g, ln_b [C] fp32; w1 [hidden, C], w2 [C, hidden] (plan dtype); b1 [hidden],
 *   b2 [C] fp32. routed_count must not exceed max_batch * routed_per_image;
 *   workspace >= mlp_workspace_bytes.
 */
sparsesam_status sparsesam_mlp(sparsesam_plan_t plan, float* x, int64_t rows, const int32_t* routed,
                               int32_t routed_count, const float* ln_g, const float* ln_b, const void* w1,
                               const float* b1, const void* w2, const float* b2, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * (4b) Keep-set selection by score: for each segment of `batch` images, the K tokens with the
 * largest score (same page, selective-computation bullet; the selection of
 * SPARSESAM_ROUTE_UPDATE plans), ranked like importance in sparsesam_permute: descending,
 * -0.0 == +0.0, NaN after every number, ties to the lower slot, window pads never chosen.
 *   score  [batch, grid_h * grid_w] fp32, tokens in raster order.
 *   routed [batch * routed_per_image] int32: global row ids, segment by segment as in
 *          sparsesam_permute, each segment's K tokens largest score first.
 * Integer output, exactly determined by the scores. Works for plans of either routing.
 */
sparsesam_status sparsesam_route_topk(sparsesam_plan_t plan, const float* score, int32_t batch, int32_t* routed,
                                      void* stream);

/* Parameters of one pre-LN ViT block. Matrices in the plan dtype, [out, in]. */
typedef struct sparsesam_block_weights {
  const float* ln1_g;  /* [C] */
  const float* ln1_b;  /* [C] */
  const void* w_qkv;   /* [3C, C]: rows 0..C-1 give q, C..2C-1 k, 2C..3C-1 v; head h uses h*D..h*D+D-1 */
  const float* b_qkv;  /* [3C] */
  const void* w_proj;  /* [C, C] */
  const float* b_proj; /* [C] */
  const float* ln2_g;  /* [C] */
  const float* ln2_b;  /* [C] */
  const void* w1;      /* [hidden, C] */
  const float* b1;     /* [hidden] */
  const void* w2;      /* [C, hidden] */
  const float* b2;     /* [C] */
  const float* rel_pos_h; /* [2 Sh - 1, head_dim] relative-position table (3b) when the plan has
                             rel_pos = 1, else NULL */
  const float* rel_pos_w; /* [2 Sw - 1, head_dim], likewise */
} sparsesam_block_weights;

/*
 * (5) One SparseSAM encoder block, in place on x [batch, grid_h, grid_w, C] fp32 in
 * raster order, with the perm and routed outputs of sparsesam_permute for the same
 * plan and images (one permutation set serves every block of a type: same page,
 * closing paragraph of part 2):
 *   h  = LayerNorm1(x) gathered into stripe-sorted order (window pads: h = 0)
 *   qkv = h W_qkv^T + b_qkv
 *   o  = sparse attention (3) per segment and head, scale head_dim^-0.5 (with the
 *        relative-position bias (3b) when the plan has rel_pos = 1)
 *   x  = x + o W_proj^T + b_proj          scattered back to raster order, pads dropped
 *   x  = the routed MLP (4) on the keep-set
 * With mlp_merge = 1, every real token of a segment outside its keep-set then adds the mean
 * of the keep-set's MLP updates (the reading of the residual-propagation bullet's
 * y_i = x_i + eps_i taken for merging).
 * workspace >= block_workspace_bytes; batch <= max_batch. Plans with routing = UPDATE are
 * rejected (INVALID_ARGUMENT): their keep-set is chosen inside the block, see (5c).
 */
sparsesam_status sparsesam_block(sparsesam_plan_t plan, const sparsesam_block_weights* weights /* host */,
                                 float* x, int32_t batch, const int32_t* perm, const int32_t* routed,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * (5d) The whole hot path of one block step: importance (1) of img [batch, height, width]
 * fp32 into imp, the permutation (2) into perm / inv / routed, then the block (5) in place
 * on x -- the three calls in one, with the same results bit for bit. ("Technische
 * Samenvatting: SparseSAM", Methodologie: importance-guided reordering ahead of the
 * block's attention and MLP.) height = grid_h * patch, width = grid_w * patch. Where the
 * ranking runs one wavefront per slot (bf16 plans with more than 3840 tokens per segment
 * and C = 768, 1024 or 1280: the ViT global grids), the permutation kernel also writes
 * the block's first LayerNorm rows, so the block skips its gather launch.
 * All pointers are device pointers; workspace as in (5). Plans with routing = UPDATE are
 * rejected (INVALID_ARGUMENT); other validation as in (1), (2) and (5).
 */
sparsesam_status sparsesam_forward(sparsesam_plan_t plan, const sparsesam_block_weights* weights /* host */,
                                   const float* img, int32_t batch, int32_t height, int32_t width, int32_t patch,
                                   float* x, float* imp, int32_t* perm, int32_t* inv, int32_t* routed,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * (5c) One block of a plan with routing = SPARSESAM_ROUTE_UPDATE: as (5), except that after
 * the attention sub-block (x1 = x + o W_proj^T + b_proj) each segment's keep-set is the K
 * tokens with the largest ||x1[t] - x[t]||^2, chosen as by (4b), and the MLP (and the merge,
 * when mlp_merge = 1) runs on that set.
 *   routed_out [batch * routed_per_image] int32: receives the keep-set (layout of (4b)).
 *   score_out  [batch, grid_h * grid_w] fp32 or NULL: receives every token's score.
 *   perm as in (5); workspace >= block_workspace_bytes.
 * The squared norms are summed in a fixed order, so the keep-set is reproducible run to run;
 * it is exactly the (4b) selection of score_out.
 */
sparsesam_status sparsesam_block_dynamic(sparsesam_plan_t plan, const sparsesam_block_weights* weights /* host */,
                                         float* x, int32_t batch, const int32_t* perm, int32_t* routed_out,
                                         float* score_out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * (6) Encoder: a stack of n_layers blocks (5) in place on x, layer l a global block
 * (kinds[l] = 1, global_plan, perm_global / routed_global) or a windowed block
 * (kinds[l] = 0, window_plan, perm_window / routed_window). The permutations depend on
 * the image only, so one set per block type, computed once by sparsesam_permute, serves
 * every layer of that type ("Technische Samenvatting: SparseSAM", Methodologie, closing
 * paragraph of part 2; SAM's encoders place four global blocks among windowed ones).
 *   layers [n_layers] host array; kinds [n_layers] host uint8 in {0, 1}.
 *   global_plan and window_plan share grid, channels, heads, head_dim, mlp_hidden,
 *   dtype and device; either may be null when no layer uses it.
 *   workspace >= the block_workspace_bytes of every plan used, batch <= their max_batch.
 * Plans with routing = UPDATE are not taken (UNSUPPORTED): their blocks run through (5c).
 * Every layer is validated before the first launch: on INVALID_ARGUMENT, UNSUPPORTED,
 * NO_DEVICE or WORKSPACE nothing runs and x is untouched. A launch failure in layer l
 * returns ERR_HIP with layers 0..l-1 applied.
 */
sparsesam_status sparsesam_encoder(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                   const sparsesam_block_weights* layers /* host */, const uint8_t* kinds /* host */,
                                   int32_t n_layers, float* x, int32_t batch, const int32_t* perm_global,
                                   const int32_t* routed_global, const int32_t* perm_window,
                                   const int32_t* routed_window, void* workspace, size_t workspace_bytes,
                                   void* stream);

/*
 * (5b) sparsesam_block (5) for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. Instead of a
 * caller workspace it uses a fixed scratch array held by the library, one per GPU, of
 * sparsesam_noalloc_scratch_bytes() bytes (64 MiB) for the life of the process; the call
 * itself allocates nothing. The caller still passes x, perm, routed and the weights as in
 * (5), and the results are those of (5).
 *   Limit: the plan's block workspace at `batch` (block_workspace_bytes at max_batch is an
 *   upper bound) must fit the scratch; larger requests return SPARSESAM_ERR_WORKSPACE with
 *   nothing launched. Every other error is reported as by (5).
 *   All calls on one GPU share that GPU's scratch, which keeps the last call's contents:
 *   calls that overlap on one GPU (other streams, other threads) race and give undefined
 *   results. Serialise them, e.g. on one stream.
 */
size_t sparsesam_noalloc_scratch_bytes(void);
sparsesam_status sparsesam_block_noalloc(sparsesam_plan_t plan, const sparsesam_block_weights* weights /* host */,
                                         float* x, int32_t batch, const int32_t* perm, const int32_t* routed,
                                         void* stream);

/*
 * (6b) The encoder (6) with the residual stream kept in stripe-sorted order ("Technische
 * Samenvatting: SparseSAM", Methodologie, closing paragraph of part 2: one precomputed
 * permutation set reused by every layer; Probleemstelling, token-merging bullet: per-layer
 * scatter-gather passes are the overhead to avoid). The stream is gathered once into the
 * order of the first block's type; consecutive blocks of that type read and write their
 * rows in place (no gather through perm, no scatter back; pads and keep-set positions follow
 * from the plan alone); a change of block type moves the stream by one composed gather
 * (window order -> global order or back); after the last block it returns to raster order
 * in x. The arithmetic of every block is that of (6), so the result equals (6) bit for bit.
 *   perm_* / inv_*: sparsesam_permute's perm and inv of each block type used (the keep-set
 *   is not passed: in stripe-sorted order it is the plan's first K ranks of each segment).
 *   workspace >= sparsesam_encoder_permuted_workspace(global_plan, window_plan, batch): two
 *   stream buffers plus the largest block workspace.
 * Plans with routing = UPDATE or mlp_merge = 1 are not taken (UNSUPPORTED). Validation as in (6).
 */
sparsesam_status sparsesam_encoder_permuted_workspace(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                                      int32_t batch, size_t* bytes /* host */);
sparsesam_status sparsesam_encoder_permuted(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                            const sparsesam_block_weights* layers /* host */,
                                            const uint8_t* kinds /* host */, int32_t n_layers, float* x,
                                            int32_t batch, const int32_t* perm_global, const int32_t* inv_global,
                                            const int32_t* perm_window, const int32_t* inv_window, void* workspace,
                                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSESAM_H */

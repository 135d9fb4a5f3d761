// C ABI of libsparsesam: plans, validation and the five hot-path entry points.
#include <algorithm>
#include <map>
#include <mutex>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.hpp"

namespace sparsesam {

static thread_local std::string g_error;

void set_error(const std::string& msg) { g_error = msg; }

sparsesam_status hip_fail(hipError_t e, const char* where) {
  set_error(std::string(where) + ": " + hipGetErrorString(e));
  return SPARSESAM_ERR_HIP;
}

static sparsesam_status invalid(const std::string& msg) {
  set_error(msg);
  return SPARSESAM_ERR_INVALID_ARGUMENT;
}

static sparsesam_status unsupported(const std::string& msg) {
  set_error(msg);
  return SPARSESAM_ERR_UNSUPPORTED;
}

size_t permute_lds_bytes(const sparsesam_plan& p);

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

static size_t elem_size(const sparsesam_plan& p) { return p.desc.dtype == SPARSESAM_BF16 ? 2 : 4; }

size_t mlp_workspace(const sparsesam_plan& p, int rows, size_t* a2, size_t* hid) {
  const size_t es = elem_size(p);
  size_t off = 0;
  *a2 = off;
  off += align256((size_t)rows * p.desc.channels * es);
  *hid = off;
  off += align256((size_t)rows * p.desc.mlp_hidden * es);
  return off;
}

RelLayout relpos_layout(const sparsesam_plan& p, int segments) {
  RelLayout R;
  const size_t segs = (size_t)std::max(segments, 0);
  // every region is a whole number of 256-byte-aligned per-segment parts, so the total is
  // proportional to the segment count (callers scale it per segment)
  R.table = 0;
  R.kc = segs * align256((size_t)p.desc.heads * p.n * (size_t)p.rel_tj * sizeof(float));
  R.part = R.kc + segs * align256((size_t)p.n * sizeof(int));
  R.total = R.part + segs * align256(attn_partial_bytes(p, 1));
  return R;
}

BlockLayout block_layout(const sparsesam_plan& p, int batch) {
  BlockLayout L;
  const size_t es = elem_size(p);
  const size_t segs = (size_t)batch * p.segs_per_img;
  const size_t M = segs * p.n;
  const size_t C = p.desc.channels;
  size_t off = 0;
  L.h = off;
  off += align256(M * C * es);
  L.q = off;
  off += align256(M * C * es);
  L.k = off;
  off += align256(M * C * es);
  L.vt = off;
  off += align256(segs * p.desc.heads * p.desc.head_dim * (size_t)p.n_pad * es);
  L.o = off;
  off += align256(M * C * es);
  L.part = off;
  off += align256(attn_partial_bytes(p, (int)segs));
  if (p.desc.rel_pos) {
    const RelLayout R = relpos_layout(p, (int)segs);
    L.rel_table = off;
    off += R.kc;
    L.rel_kc = off;
    off += R.part - R.kc;
  }
  L.total_attn = off;
  if (p.desc.routing == SPARSESAM_ROUTE_UPDATE) {
    L.sq_ld = (int)((C + 31) / 32);
    L.sq = off;
    off += align256((size_t)batch * p.desc.grid_h * p.desc.grid_w * L.sq_ld * sizeof(float));
    L.total_dyn = off;
  }
  L.total_mlp = mlp_workspace(p, batch * p.routed_per_image, &L.a2, &L.hid);
  if (p.desc.mlp_merge) {
    L.upd = L.total_mlp;
    L.total_merge = L.upd + align256((size_t)batch * p.routed_per_image * C * sizeof(float));
  }
  return L;
}

static sparsesam_status check_device(const sparsesam_plan* p) {
  if (!p) return invalid("plan is null");
  if (!p->dev) {
    set_error("plan has no device copy (no GPU was present when it was created)");
    return SPARSESAM_ERR_NO_DEVICE;
  }
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) {
    set_error("current device " + std::to_string(dev) + " differs from the plan's device " +
              std::to_string(p->device));
    return SPARSESAM_ERR_NO_DEVICE;
  }
  return SPARSESAM_OK;
}

static sparsesam_status validate_desc(const sparsesam_plan_desc& d) {
  if (d.grid_h <= 0 || d.grid_w <= 0) return invalid("grid_h and grid_w must be positive");
  if (d.window < 0) return invalid("window must be >= 0");
  const long long n = d.window > 0 ? (long long)d.window * d.window : (long long)d.grid_h * d.grid_w;
  if (n > (1 << 20)) return invalid("segment too long");
  if (d.stripes < 1 || n % d.stripes != 0) return invalid("stripes must be >= 1 and divide the segment length");
  const long long S = n / d.stripes;
  if (d.block < 1 || d.block > S) return invalid("block must be in [1, N / stripes]");
  if (d.global_tokens < 0 || d.global_tokens > S) return invalid("global_tokens must be in [0, N / stripes]");
  if (d.global_tokens % d.block != 0) return invalid("global_tokens must be a multiple of block");
  if (d.band_radius < -1) return invalid("band_radius must be >= -1");
  if (!(d.attn_density > 0.0f && d.attn_density <= 1.0f)) return invalid("attn_density must be in (0, 1]");
  if (!(d.mlp_density > 0.0f && d.mlp_density <= 1.0f)) return invalid("mlp_density must be in (0, 1]");
  if (d.heads < 1 || d.head_dim < 1 || d.channels != d.heads * d.head_dim)
    return invalid("channels must equal heads * head_dim");
  if (d.mlp_hidden < 1) return invalid("mlp_hidden must be positive");
  if (d.max_batch < 1) return invalid("max_batch must be >= 1");
  if (d.dtype != SPARSESAM_F32 && d.dtype != SPARSESAM_BF16) return invalid("dtype must be SPARSESAM_F32 or SPARSESAM_BF16");
  if (d.ordering < SPARSESAM_ORDER_IMPORTANCE || d.ordering > SPARSESAM_ORDER_RANDOM)
    return invalid("ordering must be a sparsesam_ordering value");
  if (d.rel_pos != 0 && d.rel_pos != 1) return invalid("rel_pos must be 0 or 1");
  if (d.routing != SPARSESAM_ROUTE_IMPORTANCE && d.routing != SPARSESAM_ROUTE_UPDATE)
    return invalid("routing must be a sparsesam_routing value");
  if (d.mlp_merge != 0 && d.mlp_merge != 1) return invalid("mlp_merge must be 0 or 1");
  if (d.mlp_merge && n > 16384) return unsupported("mlp_merge needs segments of at most 16384 tokens");
  if (d.channels > 1536) return unsupported("channels above 1536 are not supported");
  if (d.head_dim != 32 && d.head_dim != 64 && d.head_dim != 80 && d.head_dim != 128)
    return unsupported("head_dim must be 32, 64, 80 or 128");
  if (d.dtype == SPARSESAM_BF16) {
    if (d.channels % 128 != 0 || d.mlp_hidden % 128 != 0)
      return unsupported("bf16 plans need channels and mlp_hidden multiples of 128");
    if (d.head_dim != 64 && d.head_dim != 80) return unsupported("bf16 plans need head_dim 64 or 80");
  }
  return SPARSESAM_OK;
}

static void build_tiles(sparsesam_plan& p, int radius) {
  const int g = p.desc.stripes, B = p.desc.block, G = p.desc.global_tokens;
  p.nbs = (p.s + B - 1) / B;
  p.tiles = g * p.nbs;
  p.tile_start.resize(p.tiles);
  p.tile_len.resize(p.tiles);
  for (int t = 0; t < p.tiles; ++t) {
    int a = t / p.nbs, j = t % p.nbs;
    p.tile_start[t] = a * p.s + j * B;
    p.tile_len[t] = std::min(B, p.s - j * B);
  }
  auto global_tile = [&](int t) { return (t / p.nbs) == 0 && (t % p.nbs) * B < G; };
  p.row_ptr.assign(p.tiles + 1, 0);
  p.col_idx.clear();
  p.pairs_kept = 0;
  for (int t1 = 0; t1 < p.tiles; ++t1) {
    for (int t2 = 0; t2 < p.tiles; ++t2) {
      int j1 = t1 % p.nbs, j2 = t2 % p.nbs;
      bool keep = std::abs(j1 - j2) <= radius || global_tile(t1) || global_tile(t2);
      if (keep) {
        p.col_idx.push_back(t2);
        p.pairs_kept += (long long)p.tile_len[t1] * p.tile_len[t2];
      }
    }
    p.row_ptr[t1 + 1] = (int)p.col_idx.size();
  }
  p.tiles_kept = (int)p.col_idx.size();
  p.density = (double)p.pairs_kept / ((double)p.n * (double)p.n);
  p.radius = radius;
}

// Tables of the window kernel on 16-key blocks (attn_win_kernel) for segments of at most
// kShortMaxN tokens: key classes in consecutive slots, query groups with their key-block
// lists, the groups balanced over the wavefronts (longest first onto the least loaded).
// Leaves win_nslots = 0 when the segment does not fit kWinMaxSlots slots.
static void build_window_tables(sparsesam_plan& p) {
  p.win_nslots = 0;
  p.win_pos_slot.clear();
  p.win_slot_pos.clear();
  p.win_groups.clear();
  p.win_kb.clear();
  p.win_wave.clear();
  if (p.n > kShortMaxN || p.desc.stripes * p.s != p.n) return;
  const int T = p.tiles;
  std::vector<char> kept((size_t)T * T, 0);
  for (int t = 0; t < T; ++t)
    for (int c = p.row_ptr[t]; c < p.row_ptr[t + 1]; ++c) kept[(size_t)t * T + p.col_idx[c]] = 1;
  // key classes: tiles with the same kept column, in first-appearance order
  std::map<std::vector<char>, int> cls_of;
  std::vector<int> tile_cls(T);
  std::vector<std::vector<int>> cls_tiles;
  for (int t2 = 0; t2 < T; ++t2) {
    std::vector<char> col(T);
    for (int t1 = 0; t1 < T; ++t1) col[t1] = kept[(size_t)t1 * T + t2];
    auto f = cls_of.emplace(col, (int)cls_tiles.size());
    if (f.second) cls_tiles.emplace_back();
    tile_cls[t2] = f.first->second;
    cls_tiles[f.first->second].push_back(t2);
  }
  const int ncls = (int)cls_tiles.size();
  std::vector<int> pos_slot(kWinMaxSlots, 0), slot_pos(kWinMaxSlots, 0), blk_mask;
  std::vector<int> cls_b0(ncls), cls_b1(ncls);
  int slot = 0;
  for (int c = 0; c < ncls; ++c) {
    cls_b0[c] = slot / 16;
    const int first = p.tile_start[cls_tiles[c][0]];
    for (int t : cls_tiles[c])
      for (int i = 0; i < p.tile_len[t]; ++i, ++slot) {
        if (slot >= kWinMaxSlots) return;
        slot_pos[slot] = p.tile_start[t] + i;
        pos_slot[p.tile_start[t] + i] = slot;
      }
    const int end = (slot + 15) / 16 * 16;
    if (end > kWinMaxSlots) return;
    for (int b = cls_b0[c]; b < end / 16; ++b) {
      int m = 0;
      for (int i = 0; i < 16; ++i)
        if (16 * b + i < slot) m |= 1 << i;
      blk_mask.push_back(m);
    }
    for (; slot < end; ++slot) slot_pos[slot] = first;  // empty: a real key, masked
    cls_b1[c] = end / 16;
  }
  // query groups: tiles whose kept key tiles form the same set of classes
  std::map<std::vector<int>, int> set_of;
  std::vector<std::vector<int>> set_tiles, set_cls;
  for (int t1 = 0; t1 < T; ++t1) {
    std::vector<int> cs;
    for (int c = p.row_ptr[t1]; c < p.row_ptr[t1 + 1]; ++c) cs.push_back(tile_cls[p.col_idx[c]]);
    std::sort(cs.begin(), cs.end());
    cs.erase(std::unique(cs.begin(), cs.end()), cs.end());
    if (cs.empty()) continue;  // a query tile with no kept key has no output here
    auto f = set_of.emplace(cs, (int)set_tiles.size());
    if (f.second) {
      set_tiles.emplace_back();
      set_cls.push_back(cs);
    }
    set_tiles[f.first->second].push_back(t1);
  }
  struct Group { int kb0, kb1, nq; int q[16]; };
  std::vector<Group> gs;
  for (size_t st = 0; st < set_tiles.size(); ++st) {
    const int kb0 = (int)p.win_kb.size();
    for (int c : set_cls[st])
      for (int b = cls_b0[c]; b < cls_b1[c]; ++b) p.win_kb.push_back(b | (blk_mask[b] << 16));
    const int kb1 = (int)p.win_kb.size();
    std::vector<int> qs;
    for (int t : set_tiles[st])
      for (int i = 0; i < p.tile_len[t]; ++i) qs.push_back(p.tile_start[t] + i);
    for (size_t q0 = 0; q0 < qs.size(); q0 += 16) {
      Group g{kb0, kb1, (int)std::min<size_t>(16, qs.size() - q0), {}};
      for (int i = 0; i < 16; ++i) g.q[i] = q0 + i < qs.size() ? qs[q0 + i] : -1;
      gs.push_back(g);
    }
  }
  // longest first onto the least loaded wavefront (cost: key blocks + 1 for the query
  // loads and stores)
  std::vector<int> idx(gs.size());
  for (size_t i = 0; i < gs.size(); ++i) idx[i] = (int)i;
  std::stable_sort(idx.begin(), idx.end(),
                   [&](int a, int b) { return gs[a].kb1 - gs[a].kb0 > gs[b].kb1 - gs[b].kb0; });
  std::vector<int> load(kWinWaves, 0);
  std::vector<std::vector<int>> wl(kWinWaves);
  for (int i : idx) {
    const int w = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[w] += gs[i].kb1 - gs[i].kb0 + 1;
    wl[w].push_back(i);
  }
  p.win_wave.push_back(0);
  for (int w = 0; w < kWinWaves; ++w) {
    for (int i : wl[w]) {
      const Group& g = gs[i];
      p.win_groups.insert(p.win_groups.end(), {g.kb0, g.kb1, g.nq, 0});
      p.win_groups.insert(p.win_groups.end(), g.q, g.q + 16);
    }
    p.win_wave.push_back((int)(p.win_groups.size() / kWinGroupInts));
  }
  p.win_pos_slot = pos_slot;
  p.win_slot_pos = slot_pos;
  p.win_nslots = slot;
}

}  // namespace sparsesam

using namespace sparsesam;

extern "C" {

const char* sparsesam_status_string(sparsesam_status s) {
  switch (s) {
    case SPARSESAM_OK: return "ok";
    case SPARSESAM_ERR_INVALID_ARGUMENT: return "invalid argument";
    case SPARSESAM_ERR_UNSUPPORTED: return "unsupported";
    case SPARSESAM_ERR_WORKSPACE: return "workspace too small";
    case SPARSESAM_ERR_OUT_OF_MEMORY: return "out of memory";
    case SPARSESAM_ERR_HIP: return "HIP error";
    case SPARSESAM_ERR_NO_DEVICE: return "no device copy for the current device";
  }
  return "unknown status";
}

const char* sparsesam_last_error(void) { return g_error.c_str(); }

sparsesam_status sparsesam_plan_create(const sparsesam_plan_desc* desc, sparsesam_plan_t* out) {
  if (!desc || !out) return invalid("desc and out must not be null");
  *out = nullptr;
  sparsesam_status st = validate_desc(*desc);
  if (st != SPARSESAM_OK) return st;
  sparsesam_plan* p = new (std::nothrow) sparsesam_plan();
  if (!p) {
    set_error("host allocation failed");
    return SPARSESAM_ERR_OUT_OF_MEMORY;
  }
  p->desc = *desc;
  const sparsesam_plan_desc& d = p->desc;
  if (d.window > 0) {
    p->nwy = (d.grid_h + d.window - 1) / d.window;
    p->nwx = (d.grid_w + d.window - 1) / d.window;
    p->segs_per_img = p->nwy * p->nwx;
    p->n = d.window * d.window;
  } else {
    p->n = d.grid_h * d.grid_w;
  }
  p->n_pad = (p->n + 7) & ~7;
  p->s = p->n / d.stripes;
  p->rel_seg_h = d.window > 0 ? d.window : d.grid_h;
  p->rel_seg_w = d.window > 0 ? d.window : d.grid_w;
  if (p->rel_seg_h <= 64 && p->rel_seg_w <= 64 && d.head_dim <= 80) {  // table kernel's LDS
    p->rel_xoff = 16 * ((p->rel_seg_h + 15) / 16);
    p->rel_tj = p->rel_xoff + 16 * ((p->rel_seg_w + 15) / 16);
  }
  if (d.rel_pos && p->rel_tj == 0) {
    delete p;
    return unsupported("the relative-position bias needs segments of at most 64 x 64 tokens and head_dim <= 80");
  }
  int radius = d.band_radius;
  const int last = (p->s - 1) / d.block;
  if (radius < 0) {
    for (radius = 0; radius <= last; ++radius) {
      build_tiles(*p, radius);
      if (p->density >= (double)d.attn_density) break;
    }
    if (radius > last) radius = last;
  }
  build_tiles(*p, radius);
  // longest tile row first
  p->order.resize(p->tiles);
  for (int t = 0; t < p->tiles; ++t) p->order[t] = t;
  std::stable_sort(p->order.begin(), p->order.end(), [&](int a, int b) {
    return (p->row_ptr[a + 1] - p->row_ptr[a]) > (p->row_ptr[b + 1] - p->row_ptr[b]);
  });
  // Matrix-core attention work list. Query tiles with identical kept-key lists form
  // groups of at most four (one item each, G members, P = 4 / G key parities; G = 3
  // runs one parity); lists longer than kAttnItemTiles are split into single-tile items
  // with partial slots, merged per (query tile, first slot, chunks) in `splits`. Items
  // are ordered by steps (list length / P), longest first. Record: {kb, ke, slot, G |
  // P << 4}, {members' query tiles, -1 padded}.
  {
    const int kChunk = kAttnItemTiles;
    struct Item { int kb, ke, slot, g, pq; int qt[4]; };
    std::vector<Item> v;
    p->splits.clear();
    p->n_slots = 0;
    std::map<std::vector<int>, std::vector<int>> by_list;
    std::vector<std::vector<int>> lists;  // first-appearance order
    for (int qt = 0; qt < p->tiles; ++qt) {
      std::vector<int> key(p->col_idx.begin() + p->row_ptr[qt], p->col_idx.begin() + p->row_ptr[qt + 1]);
      auto f = by_list.find(key);
      if (f == by_list.end()) {
        lists.push_back(key);
        by_list[key] = {qt};
      } else {
        f->second.push_back(qt);
      }
    }
    for (const std::vector<int>& key : lists) {
      const std::vector<int>& members = by_list[key];
      const int rb = p->row_ptr[members[0]], len = (int)key.size();
      if (len > kChunk) {
        for (int qt : members) {
          const int rq = p->row_ptr[qt];
          const int nch = (len + kChunk - 1) / kChunk;
          p->splits.insert(p->splits.end(), {qt, p->n_slots, nch});
          for (int c = 0; c < nch; ++c)
            v.push_back({rq + (int)((long long)c * len / nch), rq + (int)((long long)(c + 1) * len / nch),
                         p->n_slots++, 1, 4, {qt, -1, -1, -1}});
        }
        continue;
      }
      for (size_t m0 = 0; m0 < members.size(); m0 += 4) {
        const int g = (int)std::min<size_t>(4, members.size() - m0);
        Item it{rb, rb + len, -1, g, g == 1 ? 4 : g == 2 ? 2 : 1, {-1, -1, -1, -1}};
        for (int i = 0; i < g; ++i) it.qt[i] = members[m0 + i];
        v.push_back(it);
      }
    }
    auto steps = [](const Item& it) { return (it.ke - it.kb + it.pq - 1) / it.pq; };
    std::stable_sort(v.begin(), v.end(), [&](const Item& a, const Item& b) { return steps(a) > steps(b); });
    p->items.clear();
    for (const Item& it : v)
      p->items.insert(p->items.end(), {it.kb, it.ke, it.slot, it.g | (it.pq << 4), it.qt[0], it.qt[1], it.qt[2],
                                       it.qt[3]});
    p->n_items = (int)v.size();
    p->n_split_rows = (int)p->splits.size() / 3;
  }
  // short-segment attention tables (n <= 256)
  p->pos_tile.clear();
  p->any32.clear();
  p->mask_class.clear();
  p->mask_row.clear();
  p->nt32 = 0;
  p->mask_ksteps = 0;
  if (p->n <= kShortMaxN) {
    const int nt32 = (p->n + 31) / 32;
    p->pos_tile.assign(p->n, 0);
    for (int t = 0; t < p->tiles; ++t)
      for (int i = 0; i < p->tile_len[t]; ++i) p->pos_tile[p->tile_start[t] + i] = t;
    // kept[t1][t2], then the classes of key tiles with equal columns (first appearance)
    std::vector<char> kept((size_t)p->tiles * p->tiles, 0);
    for (int t = 0; t < p->tiles; ++t)
      for (int c = p->row_ptr[t]; c < p->row_ptr[t + 1]; ++c) kept[(size_t)t * p->tiles + p->col_idx[c]] = 1;
    std::map<std::vector<char>, int> cls_of;
    std::vector<int> tile_cls(p->tiles), cls_tile;
    for (int t2 = 0; t2 < p->tiles; ++t2) {
      std::vector<char> col(p->tiles);
      for (int t1 = 0; t1 < p->tiles; ++t1) col[t1] = kept[(size_t)t1 * p->tiles + t2];
      auto f = cls_of.emplace(col, (int)cls_tile.size());
      if (f.second) cls_tile.push_back(t2);
      tile_cls[t2] = f.first->second;
    }
    const int pad_cls = (int)cls_tile.size(), ncls = pad_cls + 1;
    if (ncls <= 32) {
      const int ks = ncls <= 16 ? 1 : 2;
      p->nt32 = nt32;
      p->mask_ksteps = ks;
      p->mask_class.assign((size_t)nt32 * 32, pad_cls);
      for (int k = 0; k < p->n; ++k) p->mask_class[k] = tile_cls[p->pos_tile[k]];
      const uint16_t kMasked = 0xF180;  // bf16 -2^100
      p->mask_row.assign((size_t)p->tiles * ks * 8, 0);
      for (int t1 = 0; t1 < p->tiles; ++t1)
        for (int c = 0; c < 16 * ks; ++c) {
          const bool masked = c == pad_cls || (c < pad_cls && !kept[(size_t)t1 * p->tiles + cls_tile[c]]);
          if (masked) p->mask_row[(size_t)t1 * ks * 8 + c / 2] |= (int)((uint32_t)kMasked << (16 * (c & 1)));
        }
      p->any32.assign(nt32, 0);
      for (int q = 0; q < p->n; ++q)
        for (int k = 0; k < p->n; ++k)
          if (kept[(size_t)p->pos_tile[q] * p->tiles + p->pos_tile[k]]) p->any32[q / 32] |= 1 << (k / 32);
    }
  }
  build_window_tables(*p);
  // keep-set size per segment
  p->seg_k.resize(p->segs_per_img);
  p->seg_off.resize(p->segs_per_img);
  p->routed_per_image = 0;
  for (int w = 0; w < p->segs_per_img; ++w) {
    int n_real = p->n;
    if (d.window > 0) {
      int wy = w / p->nwx, wx = w % p->nwx;
      int ry = std::min(d.window, d.grid_h - wy * d.window);
      int rx = std::min(d.window, d.grid_w - wx * d.window);
      n_real = ry * rx;
    }
    int k = (int)std::floor((double)d.mlp_density * (double)n_real + 0.5);
    k = std::max(1, std::min(k, n_real));
    p->seg_k[w] = k;
    p->seg_off[w] = p->routed_per_image;
    p->routed_per_image += k;
  }
  // keep-set positions of a stream kept in stripe-sorted order (max_batch images)
  p->keep_pos.clear();
  p->keep_pos.reserve((size_t)d.max_batch * p->routed_per_image);
  for (int img = 0; img < d.max_batch; ++img)
    for (int w = 0; w < p->segs_per_img; ++w)
      for (int rho = 0; rho < p->seg_k[w]; ++rho)
        p->keep_pos.push_back((img * p->segs_per_img + w) * p->n + (rho % d.stripes) * p->s + rho / d.stripes);
  if (permute_lds_bytes(*p) > 160 * 1024) {
    delete p;
    return unsupported("a segment's keys or an image's token flags do not fit the permutation kernels' 160 KiB of LDS");
  }
  BlockLayout L = block_layout(*p, d.max_batch);
  p->block_ws = L.total();
  size_t a2, hid;
  p->mlp_ws = mlp_workspace(*p, d.max_batch * p->routed_per_image, &a2, &hid);

  // device copy, when a device is present
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) == hipSuccess && ndev > 0) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) dev = 0;
    std::vector<int> blob;
    auto put = [&](const std::vector<int>& v) {
      while (blob.size() % 4) blob.push_back(0);  // 16-byte alignment for int4 reads
      size_t o = blob.size();
      blob.insert(blob.end(), v.begin(), v.end());
      return o;
    };
    size_t o_rp = put(p->row_ptr), o_ci = put(p->col_idx), o_ts = put(p->tile_start), o_tl = put(p->tile_len),
           o_or = put(p->order), o_sk = put(p->seg_k), o_so = put(p->seg_off), o_it = put(p->items),
           o_sp = put(p->splits), o_pt = put(p->pos_tile), o_a32 = put(p->any32), o_mc = put(p->mask_class),
           o_mr = put(p->mask_row), o_kp = put(p->keep_pos), o_wps = put(p->win_pos_slot),
           o_wsp = put(p->win_slot_pos), o_wg = put(p->win_groups), o_wkb = put(p->win_kb),
           o_ww = put(p->win_wave);
    blob.push_back(0);
    void* dptr = nullptr;
    hipError_t e = hipMalloc(&dptr, blob.size() * sizeof(int));
    if (e != hipSuccess) {
      delete p;
      set_error(std::string("hipMalloc of the tile list failed: ") + hipGetErrorString(e));
      return SPARSESAM_ERR_OUT_OF_MEMORY;
    }
    e = hipMemcpy(dptr, blob.data(), blob.size() * sizeof(int), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(dptr);
      delete p;
      return hip_fail(e, "hipMemcpy of the tile list");
    }
    const int* b = static_cast<const int*>(dptr);
    p->dev = dptr;
    p->device = dev;
    p->d_row_ptr = b + o_rp;
    p->d_col_idx = b + o_ci;
    p->d_tile_start = b + o_ts;
    p->d_tile_len = b + o_tl;
    p->d_order = b + o_or;
    p->d_seg_k = b + o_sk;
    p->d_seg_off = b + o_so;
    p->d_items = b + o_it;
    p->d_splits = b + o_sp;
    p->d_pos_tile = b + o_pt;
    p->d_any32 = b + o_a32;
    p->d_mask_class = b + o_mc;
    p->d_mask_row = b + o_mr;
    p->d_keep_pos = b + o_kp;
    p->d_win_pos_slot = b + o_wps;
    p->d_win_slot_pos = b + o_wsp;
    p->d_win_groups = b + o_wg;
    p->d_win_kb = b + o_wkb;
    p->d_win_wave = b + o_ww;
    p->attn_resident_wgs = attn_long_supported(*p) ? attn_long_resident_wgs(dev, p->desc.head_dim) : 0;
    (void)hipGetLastError();
  } else {
    (void)hipGetLastError();
  }
  *out = p;
  return SPARSESAM_OK;
}

sparsesam_status sparsesam_plan_get_info(sparsesam_plan_t p, sparsesam_plan_info* info) {
  if (!p || !info) return invalid("plan and info must not be null");
  std::memset(info, 0, sizeof(*info));
  info->seq_len = p->n;
  info->segments_per_image = p->segs_per_img;
  info->band_radius = p->radius;
  info->tiles_per_stripe = p->nbs;
  info->tiles = p->tiles;
  info->tiles_kept = p->tiles_kept;
  info->pairs_kept = p->pairs_kept;
  info->realised_density = p->density;
  info->routed_per_image = p->routed_per_image;
  info->block_workspace_bytes = p->block_ws;
  info->mlp_workspace_bytes = p->mlp_ws;
  info->attn_workspace_bytes = attn_partial_bytes(*p, p->desc.max_batch * p->segs_per_img);
  info->relpos_workspace_bytes =
      p->rel_tj > 0 ? relpos_layout(*p, p->desc.max_batch * p->segs_per_img).total : 0;
  info->has_device_copy = p->dev ? 1 : 0;
  info->device = p->dev ? p->device : -1;
  return SPARSESAM_OK;
}

sparsesam_status sparsesam_plan_tile_list(sparsesam_plan_t p, int32_t* row_ptr, int32_t* col_idx) {
  if (!p || !row_ptr || !col_idx) return invalid("plan, row_ptr and col_idx must not be null");
  std::memcpy(row_ptr, p->row_ptr.data(), p->row_ptr.size() * sizeof(int32_t));
  std::memcpy(col_idx, p->col_idx.data(), p->col_idx.size() * sizeof(int32_t));
  return SPARSESAM_OK;
}

sparsesam_status sparsesam_plan_info_get(sparsesam_plan_t p, sparsesam_plan_info* info) {
  return sparsesam_plan_get_info(p, info);
}

sparsesam_status sparsesam_plan_block_list(sparsesam_plan_t p, int32_t* row_ptr, int32_t* col_idx) {
  return sparsesam_plan_tile_list(p, row_ptr, col_idx);
}

void sparsesam_plan_destroy(sparsesam_plan_t p) {
  if (!p) return;
  if (p->dev) {
    int cur = -1;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    (void)hipFree(p->dev);
    if (cur >= 0 && cur != p->device) (void)hipSetDevice(cur);
  }
  delete p;
}

sparsesam_status sparsesam_importance(const float* img, int32_t batch, int32_t height, int32_t width, int32_t patch,
                                      float* imp, void* stream) {
  if (batch < 0) return invalid("batch must be >= 0");
  if (patch < 1 || patch > 32) return unsupported("patch must be in [1, 32]");
  if (height <= 0 || width <= 0 || height % patch || width % patch)
    return invalid("height and width must be positive multiples of patch");
  if (batch > 65535 || height / patch > 65535 || width / patch > (1 << 30)) return invalid("grid too large");
  if (batch == 0) return SPARSESAM_OK;
  if (!img || !imp) return invalid("img and imp must not be null");
  hipError_t e = launch_importance(img, batch, height, width, patch, imp, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_importance launch");
}

sparsesam_status sparsesam_permute(sparsesam_plan_t p, const float* imp, int32_t batch, int32_t* perm, int32_t* inv,
                                   int32_t* routed, void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (batch < 0) return invalid("batch must be >= 0");
  if (batch == 0) return SPARSESAM_OK;
  if (!perm || !inv || !routed) return invalid("perm, inv and routed must not be null");
  if (!imp && p->desc.ordering == SPARSESAM_ORDER_IMPORTANCE) return invalid("imp must not be null");
  hipError_t e = launch_permute(*p, imp, batch, perm, inv, routed, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_permute launch");
}

sparsesam_status sparsesam_attn(sparsesam_plan_t p, int32_t segments, const void* q, const void* k, const void* vt,
                                void* o, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (segments < 0) return invalid("segments must be >= 0");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return invalid("scale must be positive and finite");
  if (segments == 0) return SPARSESAM_OK;
  if (!q || !k || !vt || !o) return invalid("q, k, vt and o must not be null");
  const size_t need = attn_partial_bytes(*p, segments);
  if (need > 0 && (!workspace || workspace_bytes < need)) {
    set_error("attention workspace needs " + std::to_string(need) + " bytes for " + std::to_string(segments) +
              " segments");
    return SPARSESAM_ERR_WORKSPACE;
  }
  hipError_t e;
  if (p->desc.dtype == SPARSESAM_BF16)
    e = launch_attention<bf16_t>(*p, segments, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt, (bf16_t*)o, scale,
                                 workspace, (hipStream_t)stream);
  else
    e = launch_attention<float>(*p, segments, (const float*)q, (const float*)k, (const float*)vt, (float*)o, scale,
                                workspace, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_attn launch");
}

sparsesam_status sparsesam_attn_relpos(sparsesam_plan_t p, int32_t segments, const void* q, const void* k,
                                       const void* vt, void* o, float scale, const int32_t* perm,
                                       const float* rel_h, const float* rel_w, void* workspace,
                                       size_t workspace_bytes, void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (segments < 0) return invalid("segments must be >= 0");
  if (!(scale > 0.0f) || !std::isfinite(scale)) return invalid("scale must be positive and finite");
  if (p->rel_tj <= 0)
    return unsupported("the relative-position bias needs segments of at most 64 x 64 tokens and head_dim <= 80");
  if (segments == 0) return SPARSESAM_OK;
  if (!q || !k || !vt || !o || !perm || !rel_h || !rel_w)
    return invalid("q, k, vt, o, perm, rel_h and rel_w must not be null");
  if (((uintptr_t)rel_h | (uintptr_t)rel_w) & 15) return invalid("rel_h and rel_w must be 16-byte aligned");
  const RelLayout R = relpos_layout(*p, segments);
  if (!workspace || workspace_bytes < R.total) {
    set_error("relative-position attention workspace needs " + std::to_string(R.total) + " bytes for " +
              std::to_string(segments) + " segments");
    return SPARSESAM_ERR_WORKSPACE;
  }
  char* ws = static_cast<char*>(workspace);
  hipError_t e;
  if (p->desc.dtype == SPARSESAM_BF16)
    e = launch_attention_relpos<bf16_t>(*p, segments, (const bf16_t*)q, (const bf16_t*)k, (const bf16_t*)vt,
                                        (bf16_t*)o, scale, perm, rel_h, rel_w, ws + R.table,
                                        reinterpret_cast<int*>(ws + R.kc), ws + R.part, (hipStream_t)stream);
  else
    e = launch_attention_relpos<float>(*p, segments, (const float*)q, (const float*)k, (const float*)vt, (float*)o,
                                       scale, perm, rel_h, rel_w, ws + R.table, reinterpret_cast<int*>(ws + R.kc),
                                       ws + R.part, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_attn_relpos launch");
}

}  // extern "C"

template <typename T>
static hipError_t run_mlp(const sparsesam_plan& p, float* x, int64_t x_rows, const int32_t* routed, int rows,
                          const float* ln_g,
                          const float* ln_b, const void* w1, const float* b1, const void* w2, const float* b2,
                          char* ws, hipStream_t st) {
  size_t o_a2, o_hid;
  mlp_workspace(p, rows, &o_a2, &o_hid);
  T* a2 = reinterpret_cast<T*>(ws + o_a2);
  T* hid = reinterpret_cast<T*>(ws + o_hid);
  const int C = p.desc.channels, Hm = p.desc.mlp_hidden;
  hipError_t e = launch_gather_ln<T>(p, x, (int)x_rows, rows, nullptr, routed, ln_g, ln_b, a2, st);
  if (e != hipSuccess) return e;
  EpiGelu eg{b1, hid, Hm};
  e = launch_gemm_gelu<T>(a2, (const T*)w1, rows, Hm, C, eg, st);
  if (e != hipSuccess) return e;
  EpiResidualScatter er{b2, x, nullptr, routed, p.segmap(), C, x_rows};
  return launch_gemm_residual<T>(hid, (const T*)w2, rows, C, Hm, er, st);
}

extern "C" {

sparsesam_status sparsesam_mlp(sparsesam_plan_t p, float* x, int64_t rows, const int32_t* routed, int32_t routed_count,
                               const float* ln_g, const float* ln_b, const void* w1, const float* b1, const void* w2,
                               const float* b2, void* workspace, size_t workspace_bytes, void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (rows < 0 || routed_count < 0) return invalid("rows and routed_count must be >= 0");
  if ((int64_t)routed_count > rows) return invalid("routed_count exceeds rows");
  if ((int64_t)routed_count > (int64_t)p->desc.max_batch * p->routed_per_image)
    return invalid("routed_count exceeds max_batch * routed_per_image");
  if (p->desc.mlp_merge)
    return unsupported("sparsesam_mlp does not take mlp_merge plans: the merge needs the block calls' segments");
  if (routed_count == 0) return SPARSESAM_OK;
  if (!x || !routed || !ln_g || !ln_b || !w1 || !b1 || !w2 || !b2) return invalid("null pointer argument");
  size_t a2, hid;
  size_t need = mlp_workspace(*p, routed_count, &a2, &hid);
  if (!workspace || workspace_bytes < need) {
    set_error("mlp workspace needs " + std::to_string(need) + " bytes");
    return SPARSESAM_ERR_WORKSPACE;
  }
  hipError_t e;
  if (p->desc.dtype == SPARSESAM_BF16)
    e = run_mlp<bf16_t>(*p, x, rows, routed, routed_count, ln_g, ln_b, w1, b1, w2, b2, (char*)workspace, (hipStream_t)stream);
  else
    e = run_mlp<float>(*p, x, rows, routed, routed_count, ln_g, ln_b, w1, b1, w2, b2, (char*)workspace, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_mlp launch");
}

}  // extern "C"

// One block. routed: the keep-set (input) or, for dynamic plans, where the block writes
// the keep-set it selects (score_out optional).
// stream_sorted: x is the residual stream in this plan's stripe-sorted order ([segments *
// N, C], pads included) instead of raster order; the block then reads and writes its
// rows in place and its keep-set is the plan's static list of keep-set positions.
template <typename T>
// ln1_ready: the first LayerNorm's rows are already in the workspace (written by the
// fused permutation of sparsesam_forward).
static hipError_t run_block(const sparsesam_plan& p, const sparsesam_block_weights& w, float* x, int batch,
                            const int32_t* perm, int32_t* routed, float* score_out, char* ws, hipStream_t st,
                            bool stream_sorted = false, bool ln1_ready = false) {
  BlockLayout L = block_layout(p, batch);
  const int segs = batch * p.segs_per_img;
  const int M = segs * p.n;
  const int C = p.desc.channels;
  T* h = reinterpret_cast<T*>(ws + L.h);
  T* q = reinterpret_cast<T*>(ws + L.q);
  T* k = reinterpret_cast<T*>(ws + L.k);
  T* vt = reinterpret_cast<T*>(ws + L.vt);
  T* o = reinterpret_cast<T*>(ws + L.o);
  const long long x_rows = stream_sorted ? (long long)M : (long long)batch * p.desc.grid_h * p.desc.grid_w;
  const int32_t* row_perm = stream_sorted ? nullptr : perm;  // null: rows in place
  if (stream_sorted) routed = const_cast<int32_t*>(p.d_keep_pos);
  hipError_t e = hipSuccess;
  if (!ln1_ready) e = launch_gather_ln<T>(p, x, (int)x_rows, M, row_perm, nullptr, w.ln1_g, w.ln1_b, h, st);
  if (e != hipSuccess) return e;
  EpiQKV eq{w.b_qkv, q, k, vt, p.n, p.n_pad, p.desc.heads, p.desc.head_dim, C};
  e = launch_gemm_qkv<T>(h, (const T*)w.w_qkv, M, C, eq, st);
  if (e != hipSuccess) return e;
  const float scale = 1.0f / std::sqrt((float)p.desc.head_dim);
  if (p.desc.rel_pos)
    e = launch_attention_relpos<T>(p, segs, q, k, vt, o, scale, perm, w.rel_pos_h, w.rel_pos_w, ws + L.rel_table,
                                   reinterpret_cast<int*>(ws + L.rel_kc), ws + L.part, st);
  else
    e = launch_attention<T>(p, segs, q, k, vt, o, scale, ws + L.part, st);
  if (e != hipSuccess) return e;
  const bool dynamic = p.desc.routing == SPARSESAM_ROUTE_UPDATE;
  EpiResidualScatter er{w.b_proj, x, row_perm, nullptr, p.segmap(), C, x_rows};
  if (dynamic) {  // the projection epilogue also sums each token's squared update
    er.sq_part = reinterpret_cast<float*>(ws + L.sq);
    er.sq_ld = L.sq_ld;
  }
  e = launch_gemm_residual<T>(o, (const T*)w.w_proj, M, C, C, er, st);
  if (e != hipSuccess) return e;
  if (dynamic) {
    e = launch_route_topk(p, reinterpret_cast<const float*>(ws + L.sq), L.sq_ld, batch, routed, score_out, st);
    if (e != hipSuccess) return e;
  }
  const int rows = batch * p.routed_per_image;
  T* a2 = reinterpret_cast<T*>(ws + L.a2);
  T* hid = reinterpret_cast<T*>(ws + L.hid);
  e = launch_gather_ln<T>(p, x, (int)x_rows, rows, nullptr, routed, w.ln2_g, w.ln2_b, a2, st);
  if (e != hipSuccess) return e;
  EpiGelu eg{w.b1, hid, p.desc.mlp_hidden};
  e = launch_gemm_gelu<T>(a2, (const T*)w.w1, rows, p.desc.mlp_hidden, C, eg, st);
  if (e != hipSuccess) return e;
  EpiResidualScatter e2{w.b2, x, nullptr, routed, p.segmap(), C, x_rows};
  if (p.desc.mlp_merge) e2.upd = reinterpret_cast<float*>(ws + L.upd);  // keep the updates for the merge
  e = launch_gemm_residual<T>(hid, (const T*)w.w2, rows, C, p.desc.mlp_hidden, e2, st);
  if (e != hipSuccess || !p.desc.mlp_merge) return e;
  return launch_merge(p, x, batch, routed, reinterpret_cast<const float*>(ws + L.upd), st);
}

// Validation of one block call (no launch, no side effects).
static sparsesam_status block_check(sparsesam_plan_t p, const sparsesam_block_weights* w, const float* x,
                                    int32_t batch, const int32_t* perm, const int32_t* routed, const void* workspace,
                                    size_t workspace_bytes) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (!w) return invalid("weights must not be null");
  if (batch < 0 || batch > p->desc.max_batch) return invalid("batch must be in [0, max_batch]");
  if (batch == 0) return SPARSESAM_OK;
  if (!x || !perm || !routed) return invalid("x, perm and routed must not be null");
  if (!w->ln1_g || !w->ln1_b || !w->w_qkv || !w->b_qkv || !w->w_proj || !w->b_proj || !w->ln2_g || !w->ln2_b ||
      !w->w1 || !w->b1 || !w->w2 || !w->b2)
    return invalid("a weight pointer is null");
  if (p->desc.rel_pos && (!w->rel_pos_h || !w->rel_pos_w))
    return invalid("the plan has rel_pos = 1: rel_pos_h and rel_pos_w must not be null");
  if (((uintptr_t)w->rel_pos_h | (uintptr_t)w->rel_pos_w) & 15)
    return invalid("rel_pos_h and rel_pos_w must be 16-byte aligned");
  if (!p->desc.rel_pos && (w->rel_pos_h || w->rel_pos_w))
    return invalid("rel_pos_h / rel_pos_w given to a plan created with rel_pos = 0");
  BlockLayout L = block_layout(*p, batch);
  size_t need = L.total();
  if (!workspace || workspace_bytes < need) {
    set_error("block workspace needs " + std::to_string(need) + " bytes");
    return SPARSESAM_ERR_WORKSPACE;
  }
  return SPARSESAM_OK;
}

// routed: the keep-set for static plans, the keep-set output for dynamic ones
static sparsesam_status block_impl(sparsesam_plan_t p, const sparsesam_block_weights* w, float* x, int32_t batch,
                                   const int32_t* perm, int32_t* routed, float* score_out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  sparsesam_status st = block_check(p, w, x, batch, perm, routed, workspace, workspace_bytes);
  if (st != SPARSESAM_OK || batch == 0) return st;
  hipError_t e;
  if (p->desc.dtype == SPARSESAM_BF16)
    e = run_block<bf16_t>(*p, *w, x, batch, perm, routed, score_out, (char*)workspace, (hipStream_t)stream);
  else
    e = run_block<float>(*p, *w, x, batch, perm, routed, score_out, (char*)workspace, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_block launch");
}

static sparsesam_status static_plan(sparsesam_plan_t p, const char* what) {
  if (p && p->desc.routing == SPARSESAM_ROUTE_UPDATE) {
    set_error(std::string(what) + ": the plan chooses its keep-set per block (routing = UPDATE); "
              "run its blocks through sparsesam_block_dynamic");
    return SPARSESAM_ERR_INVALID_ARGUMENT;
  }
  return SPARSESAM_OK;
}

extern "C" {

sparsesam_status sparsesam_block(sparsesam_plan_t p, const sparsesam_block_weights* w, float* x, int32_t batch,
                                 const int32_t* perm, const int32_t* routed, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  sparsesam_status st = static_plan(p, "sparsesam_block");
  if (st != SPARSESAM_OK) return st;
  // a static plan's block only reads the keep-set
  return block_impl(p, w, x, batch, perm, const_cast<int32_t*>(routed), nullptr, workspace, workspace_bytes, stream);
}

sparsesam_status sparsesam_forward(sparsesam_plan_t p, const sparsesam_block_weights* w, const float* img,
                                   int32_t batch, int32_t height, int32_t width, int32_t patch, float* x, float* imp,
                                   int32_t* perm, int32_t* inv, int32_t* routed, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  sparsesam_status st = static_plan(p, "sparsesam_forward");
  if (st != SPARSESAM_OK) return st;
  st = block_check(p, w, x, batch, perm, routed, workspace, workspace_bytes);
  if (st != SPARSESAM_OK || batch == 0) return st;
  if (!img || !imp || !inv) return invalid("img, imp and inv must not be null");
  if (patch < 1 || patch > 32) return unsupported("patch must be in [1, 32]");
  if (height != p->desc.grid_h * patch || width != p->desc.grid_w * patch)
    return invalid("height and width must be the plan's grid times patch");
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_importance(img, batch, height, width, patch, imp, s);
  if (e != hipSuccess) return hip_fail(e, "sparsesam_forward importance launch");
  const bool fused = permute_ln_fusable(*p);
  if (fused) {
    const BlockLayout L = block_layout(*p, batch);
    e = launch_permute_ln(*p, imp, batch, perm, inv, routed, x, (long long)batch * p->desc.grid_h * p->desc.grid_w,
                          w->ln1_g, w->ln1_b, reinterpret_cast<bf16_t*>((char*)workspace + L.h), s);
  } else {
    e = launch_permute(*p, imp, batch, perm, inv, routed, s);
  }
  if (e != hipSuccess) return hip_fail(e, "sparsesam_forward permutation launch");
  if (p->desc.dtype == SPARSESAM_BF16)
    e = run_block<bf16_t>(*p, *w, x, batch, perm, routed, nullptr, (char*)workspace, s, false, fused);
  else
    e = run_block<float>(*p, *w, x, batch, perm, routed, nullptr, (char*)workspace, s);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_forward block launch");
}

sparsesam_status sparsesam_block_dynamic(sparsesam_plan_t p, const sparsesam_block_weights* w, float* x,
                                         int32_t batch, const int32_t* perm, int32_t* routed_out, float* score_out,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (p && p->desc.routing != SPARSESAM_ROUTE_UPDATE)
    return invalid("sparsesam_block_dynamic needs a plan with routing = SPARSESAM_ROUTE_UPDATE");
  return block_impl(p, w, x, batch, perm, routed_out, score_out, workspace, workspace_bytes, stream);
}

sparsesam_status sparsesam_route_topk(sparsesam_plan_t p, const float* score, int32_t batch, int32_t* routed,
                                      void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (batch < 0) return invalid("batch must be >= 0");
  if (batch == 0) return SPARSESAM_OK;
  if (!score || !routed) return invalid("score and routed must not be null");
  hipError_t e = launch_route_topk(*p, score, 1, batch, routed, nullptr, (hipStream_t)stream);
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_route_topk launch");
}

}  // extern "C"

// Scratch memory of sparsesam_block_noalloc: the block workspace, held by the library for
// callers that cannot allocate. Each GPU the library runs on holds one copy until the
// process ends. Host code never passes the array's name to a kernel (on the host it is
// only a stand-in for the symbol): the device address comes from hipGetSymbolAddress,
// once per device, with that device current, and is kept in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

static std::mutex g_scratch_mu;
static std::vector<void*> g_scratch_ptr;  // per device index; null until looked up

// Device address of `scratch` on device `dev` (the current device).
static sparsesam_status scratch_address(int dev, void** out) {
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (dev < 0) return invalid("bad device index");
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize((size_t)dev + 1, nullptr);
  if (!g_scratch_ptr[(size_t)dev]) {
    void* ptr = nullptr;
    hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the no-alloc scratch");
    if (!ptr) {
      set_error("hipGetSymbolAddress returned a null scratch address");
      return SPARSESAM_ERR_HIP;
    }
    g_scratch_ptr[(size_t)dev] = ptr;
  }
  *out = g_scratch_ptr[(size_t)dev];
  return SPARSESAM_OK;
}

extern "C" {

size_t sparsesam_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

sparsesam_status sparsesam_block_noalloc(sparsesam_plan_t p, const sparsesam_block_weights* w, float* x,
                                         int32_t batch, const int32_t* perm, const int32_t* routed, void* stream) {
  sparsesam_status st = check_device(p);
  if (st != SPARSESAM_OK) return st;
  if (batch < 0 || batch > p->desc.max_batch) return invalid("batch must be in [0, max_batch]");
  if (batch == 0) return block_check(p, w, x, 0, perm, routed, nullptr, 0);
  const BlockLayout L = block_layout(*p, batch);
  const size_t need = L.total();
  if (need > kNoAllocScratchBytes) {
    set_error("sparsesam_block_noalloc: this block needs " + std::to_string(need) +
              " bytes of scratch at batch " + std::to_string(batch) + ", above the library's fixed " +
              std::to_string(kNoAllocScratchBytes) + " bytes; use sparsesam_block with a workspace");
    return SPARSESAM_ERR_WORKSPACE;
  }
  st = static_plan(p, "sparsesam_block_noalloc");
  if (st != SPARSESAM_OK) return st;
  void* ws = nullptr;
  st = scratch_address(p->device, &ws);
  if (st != SPARSESAM_OK) return st;
  // the kernels write every scratch byte they read (no region has to start at zero)
  return block_impl(p, w, x, batch, perm, const_cast<int32_t*>(routed), nullptr, ws, kNoAllocScratchBytes, stream);
}

}  // extern "C"

// Checks shared by both encoder entry points: layer kinds, plans present and of one
// shape, no dynamic-routing plan.
static sparsesam_status encoder_plans_check(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                            const sparsesam_block_weights* layers, const uint8_t* kinds,
                                            int32_t n_layers) {
  if (!layers || !kinds) return invalid("layers and kinds must not be null");
  bool any_global = false, any_window = false;
  for (int l = 0; l < n_layers; ++l) {
    if (kinds[l] > 1) return invalid("kinds must hold 1 (global block) or 0 (windowed block)");
    if (kinds[l])
      any_global = true;
    else
      any_window = true;
  }
  if (any_global && !global_plan) return invalid("a global layer needs global_plan");
  if (any_window && !window_plan) return invalid("a windowed layer needs window_plan");
  for (sparsesam_plan_t pl : {global_plan, window_plan})
    if (pl && pl->desc.routing == SPARSESAM_ROUTE_UPDATE)
      return unsupported("the encoders do not take plans with routing = UPDATE; run their blocks through "
                         "sparsesam_block_dynamic");
  if (any_global && any_window) {
    const sparsesam_plan_desc &g = global_plan->desc, &w = window_plan->desc;
    if (g.grid_h != w.grid_h || g.grid_w != w.grid_w || g.channels != w.channels || g.heads != w.heads ||
        g.head_dim != w.head_dim || g.mlp_hidden != w.mlp_hidden || g.dtype != w.dtype ||
        global_plan->device != window_plan->device)
      return invalid("global_plan and window_plan must share grid, channels, heads, head_dim, mlp_hidden, dtype "
                     "and device");
  }
  return SPARSESAM_OK;
}

extern "C" {

sparsesam_status sparsesam_encoder(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                   const sparsesam_block_weights* layers, const uint8_t* kinds, int32_t n_layers,
                                   float* x, int32_t batch, const int32_t* perm_global, const int32_t* routed_global,
                                   const int32_t* perm_window, const int32_t* routed_window, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (n_layers < 0) return invalid("n_layers must be >= 0");
  if (n_layers == 0) return SPARSESAM_OK;
  sparsesam_status pst = encoder_plans_check(global_plan, window_plan, layers, kinds, n_layers);
  if (pst != SPARSESAM_OK) return pst;
  // every layer is validated before the first launch: no partial run on bad input
  for (int l = 0; l < n_layers; ++l) {
    sparsesam_status st = block_check(kinds[l] ? global_plan : window_plan, &layers[l], x, batch,
                                      kinds[l] ? perm_global : perm_window, kinds[l] ? routed_global : routed_window,
                                      workspace, workspace_bytes);
    if (st != SPARSESAM_OK) return st;
  }
  for (int l = 0; l < n_layers; ++l) {
    sparsesam_status st = block_impl(kinds[l] ? global_plan : window_plan, &layers[l], x, batch,
                                     kinds[l] ? perm_global : perm_window,
                                     const_cast<int32_t*>(kinds[l] ? routed_global : routed_window), nullptr,
                                     workspace, workspace_bytes, stream);
    if (st != SPARSESAM_OK) return st;
  }
  return SPARSESAM_OK;
}

}  // extern "C"

// Workspace of sparsesam_encoder_permuted: two stream buffers (rows of the larger layout)
// then the largest block workspace of the plans used.
struct PermutedEncoderLayout {
  size_t stream_bytes = 0, a = 0, b = 0, block = 0, total = 0;
};
static PermutedEncoderLayout permuted_encoder_layout(sparsesam_plan_t gp, sparsesam_plan_t wp, int batch) {
  PermutedEncoderLayout E;
  size_t rows = 0, block = 0;
  for (sparsesam_plan_t pl : {gp, wp}) {
    if (!pl) continue;
    rows = std::max(rows, (size_t)batch * pl->segs_per_img * pl->n);
    rows = std::max(rows, (size_t)batch * pl->desc.grid_h * pl->desc.grid_w);
    block = std::max(block, block_layout(*pl, batch).total());
  }
  const size_t C = gp ? gp->desc.channels : (wp ? wp->desc.channels : 0);
  E.stream_bytes = align256(rows * C * sizeof(float));
  E.a = 0;
  E.b = E.stream_bytes;
  E.block = 2 * E.stream_bytes;
  E.total = E.block + block;
  return E;
}

static StreamLayout stream_layout(const sparsesam_plan* pl, const int32_t* perm, const int32_t* inv) {
  StreamLayout L;
  L.map = pl->segmap();
  L.perm = perm;
  L.inv = inv;
  return L;
}

extern "C" {

sparsesam_status sparsesam_encoder_permuted_workspace(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                                      int32_t batch, size_t* bytes) {
  if (!bytes) return invalid("bytes must not be null");
  if (!global_plan && !window_plan) return invalid("at least one plan is needed");
  if (batch < 0) return invalid("batch must be >= 0");
  *bytes = permuted_encoder_layout(global_plan, window_plan, batch).total;
  return SPARSESAM_OK;
}

sparsesam_status sparsesam_encoder_permuted(sparsesam_plan_t global_plan, sparsesam_plan_t window_plan,
                                            const sparsesam_block_weights* layers, const uint8_t* kinds,
                                            int32_t n_layers, float* x, int32_t batch, const int32_t* perm_global,
                                            const int32_t* inv_global, const int32_t* perm_window,
                                            const int32_t* inv_window, void* workspace, size_t workspace_bytes,
                                            void* stream) {
  if (n_layers < 0) return invalid("n_layers must be >= 0");
  if (n_layers == 0) return SPARSESAM_OK;
  sparsesam_status st = encoder_plans_check(global_plan, window_plan, layers, kinds, n_layers);
  if (st != SPARSESAM_OK) return st;
  for (sparsesam_plan_t pl : {global_plan, window_plan})
    if (pl && pl->desc.mlp_merge)
      return unsupported("sparsesam_encoder_permuted does not take mlp_merge plans");
  if (batch < 0) return invalid("batch must be >= 0");
  if (batch == 0) return SPARSESAM_OK;
  const PermutedEncoderLayout E = permuted_encoder_layout(global_plan, window_plan, batch);
  if (!workspace || workspace_bytes < E.total) {
    set_error("sparsesam_encoder_permuted needs " + std::to_string(E.total) + " bytes of workspace");
    return SPARSESAM_ERR_WORKSPACE;
  }
  bool any_global = false, any_window = false;
  for (int l = 0; l < n_layers; ++l) (kinds[l] ? any_global : any_window) = true;
  if ((any_global && (!perm_global || !inv_global)) || (any_window && (!perm_window || !inv_window)))
    return invalid("each block type used needs its perm and inv");
  const sparsesam_plan* ref0 = global_plan ? global_plan : window_plan;
  if (ref0->desc.channels % 4) return unsupported("channels must be a multiple of 4");
  if (!x) return invalid("x must not be null");
  char* ws = static_cast<char*>(workspace);
  char* blk = ws + E.block;
  const size_t blk_bytes = workspace_bytes - E.block;
  // every layer validated before the first launch (the block workspace and the in-place
  // stream; the keep-set comes from the plan)
  for (int l = 0; l < n_layers; ++l) {
    sparsesam_plan_t pl = kinds[l] ? global_plan : window_plan;
    st = block_check(pl, &layers[l], x, batch, kinds[l] ? perm_global : perm_window, pl->d_keep_pos, blk,
                     blk_bytes);
    if (st != SPARSESAM_OK) return st;
  }
  const sparsesam_plan* ref = global_plan ? global_plan : window_plan;
  const int C = ref->desc.channels;
  const int raster_rows = batch * ref->desc.grid_h * ref->desc.grid_w;
  hipStream_t hs = (hipStream_t)stream;
  StreamLayout raster;
  raster.map = ref->segmap();
  float* bufs[2] = {reinterpret_cast<float*>(ws + E.a), reinterpret_cast<float*>(ws + E.b)};
  int cur = -1;   // block kind the stream is ordered for (-1: not yet gathered)
  int which = 0;  // buffer holding the stream
  hipError_t e = hipSuccess;
  for (int l = 0; l < n_layers && e == hipSuccess; ++l) {
    const int kind = kinds[l];
    sparsesam_plan_t pl = kind ? global_plan : window_plan;
    const int32_t* perm = kind ? perm_global : perm_window;
    const int32_t* inv = kind ? inv_global : inv_window;
    if (kind != cur) {  // one composed gather into the new block type's order
      const StreamLayout to = stream_layout(pl, perm, inv);
      const int rows = batch * pl->segs_per_img * pl->n;
      if (cur < 0) {
        e = launch_reorder(bufs[which], x, rows, C, to, raster, hs);
      } else {
        sparsesam_plan_t prev = cur ? global_plan : window_plan;
        const StreamLayout from = stream_layout(prev, cur ? perm_global : perm_window, cur ? inv_global : inv_window);
        e = launch_reorder(bufs[1 - which], bufs[which], rows, C, to, from, hs);
        which = 1 - which;
      }
      cur = kind;
      if (e != hipSuccess) break;
    }
    if (pl->desc.dtype == SPARSESAM_BF16)
      e = run_block<bf16_t>(*pl, layers[l], bufs[which], batch, perm, nullptr, nullptr, blk, hs, true);
    else
      e = run_block<float>(*pl, layers[l], bufs[which], batch, perm, nullptr, nullptr, blk, hs, true);
  }
  if (e == hipSuccess) {  // back to raster order
    sparsesam_plan_t prev = cur ? global_plan : window_plan;
    const StreamLayout from = stream_layout(prev, cur ? perm_global : perm_window, cur ? inv_global : inv_window);
    e = launch_reorder(x, bufs[which], raster_rows, C, raster, from, hs);
  }
  return e == hipSuccess ? SPARSESAM_OK : hip_fail(e, "sparsesam_encoder_permuted launch");
}

}  // extern "C"

// Host check of the tables the window attention kernel on 16-key blocks (attn_win_kernel)
// reads, built by sparsesam_plan_create for short segments. For every plan shape below
// it verifies, against the plan's own kept-tile list:
//  - the slot map: every position has one slot, slots are unique and inverse to the
//    slot -> position table, and every table entry the kernel may read is in range;
//  - the key blocks: a block's valid-slot mask marks exactly the occupied slots;
//  - the query groups: every position is in exactly one group, and the keys a group's
//    blocks hold (valid slots only) are exactly the kept keys of each of its queries, so
//    the kernel computes every kept pair once and no other pair;
//  - the wavefront lists partition the groups.
// Tables are absent exactly when the classes need more than the 256 slots (those plans
// run the 32 x 32-block kernel, or the SIMT kernel past 31 classes). A sweep over a grid
// of plan shapes repeats every check. Prints "all ok" and exits 0 when every check holds.
#include <cstdio>
#include <set>
#include <vector>

#include "internal.hpp"

static int fails = 0;
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      ++fails;                        \
      std::printf("FAIL %s: ", name); \
      std::printf(__VA_ARGS__);       \
      std::printf("\n");              \
      return;                         \
    }                                 \
  } while (0)

// Slots the key classes need (each class rounded up to whole 16-slot blocks), counted
// from the plan's tile list: tiles kept by the same query tiles form one class.
static int class_slots(const sparsesam_plan& p) {
  std::vector<std::vector<char>> cols;
  std::vector<int> size;
  for (int t2 = 0; t2 < p.tiles; ++t2) {
    std::vector<char> col(p.tiles, 0);
    for (int t1 = 0; t1 < p.tiles; ++t1)
      for (int c = p.row_ptr[t1]; c < p.row_ptr[t1 + 1]; ++c)
        if (p.col_idx[c] == t2) col[t1] = 1;
    size_t k = 0;
    while (k < cols.size() && cols[k] != col) ++k;
    if (k == cols.size()) {
      cols.push_back(col);
      size.push_back(0);
    }
    size[k] += p.tile_len[t2];
  }
  int slots = 0;
  for (int s : size) slots += (s + 15) / 16 * 16;
  return slots;
}

static void check_plan(const char* name, const sparsesam_plan& p, bool expect_tables, bool named) {
  const int n = p.n, ns = p.win_nslots;
  if (!expect_tables) {
    CHECK(ns == 0 && p.win_groups.empty(), "tables built for a plan whose classes overflow the slots");
    CHECK(class_slots(p) > kWinMaxSlots, "no tables although the classes need %d slots", class_slots(p));
    if (named) CHECK(p.nt32 > 0, "no 32 x 32-block kernel for an overflowing plan");
    return;
  }
  CHECK(ns == class_slots(p), "%d slots against %d the classes need", ns, class_slots(p));
  CHECK(ns > 0 && ns % 16 == 0 && ns <= kWinMaxSlots, "slot count %d", ns);
  CHECK(p.win_pos_slot.size() == (size_t)kWinMaxSlots && p.win_slot_pos.size() == (size_t)kWinMaxSlots,
        "table sizes");
  std::vector<int> owner(ns, -1);
  for (int q = 0; q < n; ++q) {
    const int s = p.win_pos_slot[q];
    CHECK(s >= 0 && s < ns, "slot of position %d out of range", q);
    CHECK(owner[s] < 0, "slot %d used twice", s);
    owner[s] = q;
    CHECK(p.win_slot_pos[s] == q, "slot table not inverse at slot %d", s);
  }
  for (int s = 0; s < kWinMaxSlots; ++s)
    CHECK(p.win_slot_pos[s] >= 0 && p.win_slot_pos[s] < n, "position of slot %d out of range", s);
  std::vector<int> tile_of(n, -1);
  for (int t = 0; t < p.tiles; ++t)
    for (int i = 0; i < p.tile_len[t]; ++i) tile_of[p.tile_start[t] + i] = t;
  const int ng = (int)p.win_groups.size() / kWinGroupInts;
  CHECK(p.win_groups.size() == (size_t)ng * kWinGroupInts, "group table size");
  CHECK(p.win_wave.size() == (size_t)kWinWaves + 1 && p.win_wave[0] == 0 && p.win_wave[kWinWaves] == ng,
        "wavefront lists");
  for (int w = 0; w < kWinWaves; ++w) CHECK(p.win_wave[w] <= p.win_wave[w + 1], "wavefront list order");
  std::vector<int> seen(n, 0);
  long long pairs = 0;
  for (int gi = 0; gi < ng; ++gi) {
    const int* g = &p.win_groups[(size_t)gi * kWinGroupInts];
    CHECK(g[0] >= 0 && g[0] < g[1] && g[1] <= (int)p.win_kb.size(), "key-block range of group %d", gi);
    CHECK(g[2] >= 1 && g[2] <= 16, "queries of group %d", gi);
    std::set<int> keys;
    for (int kb = g[0]; kb < g[1]; ++kb) {
      const int e = p.win_kb[kb], b = e & 0xffff;
      const unsigned m = (unsigned)e >> 16;
      CHECK(b >= 0 && b < ns / 16 && m != 0, "key block entry %d", kb);
      for (int i = 0; i < 16; ++i) {
        const bool occ = owner[16 * b + i] >= 0;
        CHECK(occ == (bool)((m >> i) & 1u), "valid mask of block %d slot %d", b, i);
        if (occ) CHECK(keys.insert(owner[16 * b + i]).second, "key %d twice in group %d", owner[16 * b + i], gi);
      }
    }
    for (int i = 0; i < 16; ++i) {
      const int q = g[4 + i];
      if (i >= g[2]) {
        CHECK(q == -1, "unused query entry of group %d", gi);
        continue;
      }
      CHECK(q >= 0 && q < n && !seen[q], "query %d of group %d", q, gi);
      seen[q] = 1;
      std::set<int> want;
      const int t1 = tile_of[q];
      for (int c = p.row_ptr[t1]; c < p.row_ptr[t1 + 1]; ++c)
        for (int j = 0; j < p.tile_len[p.col_idx[c]]; ++j) want.insert(p.tile_start[p.col_idx[c]] + j);
      CHECK(want == keys, "keys of query %d differ from its kept keys", q);
      pairs += (long long)keys.size();
    }
  }
  for (int q = 0; q < n; ++q) CHECK(seen[q], "position %d in no group", q);
  CHECK(pairs == p.pairs_kept, "pairs %lld against %lld kept", pairs, p.pairs_kept);
}

// expect_tables: 1 tables required, 0 tables must be absent, -1 either (a sweep case:
// tables absent only when the classes overflow the slots)
static void check(const char* name, int gh, int gw, int window, int stripes, int block, int G, float density,
                  int heads, int head_dim, int expect_tables) {
  sparsesam_plan_desc d{};
  d.grid_h = gh;
  d.grid_w = gw;
  d.window = window;
  d.stripes = stripes;
  d.block = block;
  d.global_tokens = G;
  d.band_radius = -1;
  d.attn_density = density;
  d.mlp_density = 0.4f;
  d.heads = heads;
  d.head_dim = head_dim;
  d.channels = heads * head_dim;
  d.mlp_hidden = 4 * d.channels;
  d.max_batch = 1;
  d.dtype = SPARSESAM_BF16;
  sparsesam_plan_t h = nullptr;
  if (sparsesam_plan_create(&d, &h) != SPARSESAM_OK) {
    if (expect_tables < 0) return;  // a sweep shape the plan rules reject
    ++fails;
    std::printf("FAIL %s: plan_create: %s\n", name, sparsesam_last_error());
    return;
  }
  if (expect_tables >= 0 || h->n <= kShortMaxN)
    check_plan(name, *h, expect_tables < 0 ? h->win_nslots > 0 : expect_tables != 0, expect_tables >= 0);
  sparsesam_plan_destroy(h);
}

// Every short-segment plan of a grid of shapes: grids and windows, stripe counts, tile
// lengths, global token counts and densities.
static int sweep() {
  int plans = 0;
  const int grids[][2] = {{8, 8}, {12, 12}, {14, 14}, {16, 16}, {16, 15}, {15, 17}, {18, 18}, {28, 28}};
  for (const auto& gr : grids)
    for (int window : {0, 7, 8, 14})
      for (int stripes : {1, 2, 4, 7})
        for (int block : {4, 8, 12, 16, 32})
          for (int gm : {0, 1, 2})
            for (float dens : {0.2f, 0.4f, 1.0f}) {
              const int seg = window > 0 ? window * window : gr[0] * gr[1];
              if (seg > kShortMaxN || seg % stripes != 0 || block > seg / stripes) continue;
              char name[160];
              std::snprintf(name, sizeof(name), "sweep grid %dx%d window %d stripes %d block %d G %d d %.1f", gr[0],
                            gr[1], window, stripes, block, gm * block, dens);
              const int before = fails;
              check(name, gr[0], gr[1], window, stripes, block, gm * block, dens, 2, 64, -1);
              ++plans;
              if (fails > before + 5) return plans;
            }
  return plans;
}

int main() {
  check("ViT-B windows d 0.4", 64, 64, 14, 4, 16, 16, 0.4f, 12, 64, 1);
  check("ViT-B windows d 0.3", 64, 64, 14, 4, 16, 16, 0.3f, 12, 64, 1);
  check("ViT-B windows d 1.0", 64, 64, 14, 4, 16, 16, 1.0f, 12, 64, 1);
  check("ViT-H windows d 0.4", 64, 64, 14, 4, 16, 16, 0.4f, 16, 80, 1);
  check("18 x 18 grid, partial windows", 18, 18, 14, 4, 16, 16, 0.4f, 2, 64, 1);
  check("16 x 16 global, one stripe", 16, 16, 0, 1, 16, 16, 0.3f, 2, 64, 1);
  check("16 x 16 global, four stripes", 16, 16, 0, 4, 16, 16, 0.4f, 2, 64, 1);
  check("windows of 14, seven stripes of 4-token tiles", 28, 28, 14, 7, 4, 0, 0.5f, 2, 64, 1);
  check("windows of 8", 16, 16, 8, 4, 16, 16, 0.4f, 2, 64, 1);
  check("one stripe of one tile", 14, 14, 14, 1, 49, 49, 1.0f, 2, 64, 1);
  check("30 classes of 8 tokens (overflow)", 16, 15, 0, 1, 8, 8, 0.3f, 2, 64, 0);
  check("15 classes of 17 tokens (overflow)", 15, 17, 0, 1, 17, 17, 0.3f, 8, 80, 0);
  const int swept = sweep();
  std::printf("%d sweep plans\n", swept);
  std::printf(fails ? "%d failures\n" : "all ok\n", fails);
  return fails != 0;
}

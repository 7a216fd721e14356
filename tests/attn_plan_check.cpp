// Host check of the attention work plan (folded_tensor_sequence_amd/csrc/
// attn_plan.h, the code the attention and merge kernels run): for many rank
// shapes, both token partitions, both row-block sizes and both pairings,
// every (row block, sequence x q-head, key tile) is computed by exactly one
// work unit, every local row lies in exactly one block at the position the
// partition gives it (written out here on its own), each block's key tiles
// end with the tile of its last row's position, no unit is empty, a block is
// either computed whole by one unit or split into pieces with distinct
// consecutive workspace slots, and the merge kernel finds every split block
// with the first slot and piece count the attention units used.  Prints
// "ok <cases>" or the first failure.
#include <algorithm>
#include <cstdio>
#include <vector>

#include "attn_plan.h"

using namespace tsp;

static int fail(const char* what, int B, int S, int D, int r, int part, int Hq, int rbr, long long target,
                int pair) {
  std::printf("FAIL %s: B=%d S=%d D=%d r=%d part=%d Hq=%d rb=%d target=%lld pair=%d\n", what, B, S, D, r, part, Hq,
              rbr, target, pair);
  return 1;
}

// Global position of local row t: zigzag (chunks r and 2D-1-r of length c)
// or striped (t D + r).
static int position(int c, int D, int r, int part, int t) {
  if (part == 1) return t * D + r;
  return t < c ? r * c + t : (2 * D - 1 - r) * c + (t - c);
}

static int check(int B, int S, int D, int r, int part, int Hq, int rbr, long long slots, long long target,
                 int pair_req) {
  const int c = S / (2 * D);
  const PlanKey k = plan_key(c, D, r, part, B, Hq, rbr, slots, target, pair_req);
  const PlanCounts n = plan_counts(k);
  const int per_bh = B * Hq;
  const int nb = 2 * k.nrb;
#define FAIL(what) return fail(what, B, S, D, r, part, Hq, rbr, target, pair_req)
  // rows: each of the 2c local rows in exactly one block, at its position
  std::vector<int> row_seen(2 * c, 0);
  int max_nkt = 0;
  for (int bi = 0; bi < nb; ++bi) {
    const BlockGeo g = block_rows(c, D, r, part, rbr, k.nrb, bi);
    int last = -1;
    for (int t = g.t0; t < g.t0 + rbr && t < g.row_end; ++t) {
      ++row_seen[t];
      const int pos = g.gstart + (t - g.row_begin) * g.pstride;
      if (pos != position(c, D, r, part, t)) FAIL("row position");
      if (pos <= last) FAIL("positions not increasing");
      last = pos;
    }
    if (g.nkt > max_nkt) max_nkt = g.nkt;
    // the key tiles end with the tile holding the block's last position
    if (g.nkt * 64 <= last || (g.nkt - 1) * 64 > last) FAIL("key range");
  }
  for (int t = 0; t < 2 * c; ++t)
    if (row_seen[t] != 1) FAIL("rows");
  // units: every (block, bh, key tile) exactly once; each split block's
  // partial states in consecutive workspace slots, one per piece
  std::vector<int> cover((size_t)nb * per_bh * max_nkt, 0);
  std::vector<int> slot_used((size_t)(n.pieces > 0 ? n.pieces : 1) * per_bh, 0);
  std::vector<int> first_slot(nb, 1 << 30), last_slot(nb, -1), pieces_of(nb, 0), whole(nb, 0);
  const long long units = n.units_per_bh * per_bh;
  for (long long u = 0; u < units; ++u) {
    const UnitPos p = unit_of(k, per_bh, (int)u);
    if (p.piece < 0 || p.piece >= p.g.ns || p.bh < 0 || p.bh >= per_bh) FAIL("unit decode");
    const PieceSplit q = piece_split(k, p.g, p.bi);
    int nonempty = 0;
    for (int which = 0; which < 2; ++which) {
      BlockGeo g;
      int kb, ke, slot;
      bool split;
      if (!unit_part(k, p.g, p.bi, q, p.piece, which, g, kb, ke, split, slot)) continue;
      ++nonempty;
      const int bi = which == 0 ? p.bi : nb - 1 - p.bi;
      if (g.t0 != block_rows(c, D, r, part, rbr, k.nrb, bi).t0) FAIL("part block");
      if (kb < 0 || ke > g.nkt) FAIL("part range");
      for (int kt = kb; kt < ke; ++kt) ++cover[((size_t)bi * per_bh + p.bh) * max_nkt + kt];
      if (split) {
        const long long s = (long long)(p.piece_base + slot) * per_bh + p.bh;
        if (s < 0 || s >= (long long)n.pieces * per_bh) FAIL("piece slot range");
        ++slot_used[s];
        if (p.bh == 0) {
          first_slot[bi] = std::min(first_slot[bi], p.piece_base + slot);
          last_slot[bi] = std::max(last_slot[bi], p.piece_base + slot);
          ++pieces_of[bi];
        }
      } else {
        if (kb != 0 || ke != g.nkt) FAIL("whole block not whole");
        if (p.bh == 0) ++whole[bi];
      }
    }
    if (nonempty == 0) FAIL("empty unit");
  }
  for (int bi = 0; bi < nb; ++bi) {
    if (whole[bi] + (pieces_of[bi] > 0 ? 1 : 0) != 1) FAIL("block both whole and split");
    if (pieces_of[bi] == 1) FAIL("split block with one piece");
    if (pieces_of[bi] > 1 && last_slot[bi] - first_slot[bi] + 1 != pieces_of[bi]) FAIL("slots not consecutive");
  }
  for (int bi = 0; bi < nb; ++bi) {
    const int nkt = block_rows(c, D, r, part, rbr, k.nrb, bi).nkt;
    for (int bh = 0; bh < per_bh; ++bh)
      for (int kt = 0; kt < max_nkt; ++kt)
        if (cover[((size_t)bi * per_bh + bh) * max_nkt + kt] != (kt < nkt ? 1 : 0)) FAIL("tile coverage");
  }
  for (long long i = 0; i < (long long)n.pieces * per_bh; ++i)
    if (slot_used[i] != 1) FAIL("piece slots");
  // merge: work groups of 256 items, 32 items (4 head-dim columns each) per row
  const long long ipb = (long long)per_bh * rbr * 32;
  const long long total = (long long)n.split_rows * per_bh * 32;
  std::vector<int> merged(nb, 0);
  // the host's table of split blocks: when it holds the plan, entry e is the
  // block merge_block_of finds for the items of the e-th split block
  const MergeTab tab = merge_table(k);
  int split_blocks = 0;
  for (int bi = 0; bi < nb; ++bi) split_blocks += pieces_of[bi] > 1 ? 1 : 0;
  if (tab.n >= 0 ? tab.n != split_blocks : split_blocks <= kMergeTab) FAIL("merge table size");
  for (long long item = 0; item < total; item += 256) {
    const MergePos m = merge_block_of(k, ipb, item);
    if (m.bi < 0 || m.bi >= nb || pieces_of[m.bi] < 2) FAIL("merge block");
    if (m.piece_base != first_slot[m.bi] || m.npieces != pieces_of[m.bi]) FAIL("merge pieces");
    if (m.g.t0 != block_rows(c, D, r, part, rbr, k.nrb, m.bi).t0) FAIL("merge rows");
    if (m.item < 0 || m.item + 256 > ipb) FAIL("merge item");
    if (m.item == 0) ++merged[m.bi];
    if (tab.n >= 0) {
      const long long e = item / ipb;
      if (e >= tab.n || tab.bi[e] != m.bi || tab.base[e] != m.piece_base || tab.np[e] != m.npieces ||
          item - e * ipb != m.item)
        FAIL("merge table entry");
    }
  }
  for (int bi = 0; bi < nb; ++bi)
    if (merged[bi] != (pieces_of[bi] > 1 ? 1 : 0)) FAIL("merge misses a split block");
  if (merge_block_of(k, ipb, total).bi != -1) FAIL("merge end");
#undef FAIL
  return 0;
}

int main() {
  struct Case {
    int B, S, D, Hq;
  };
  // the test and benchmark shapes, plus a grid of small ones
  std::vector<Case> cases = {{1, 256, 2, 4},     {1, 512, 4, 16},    {2, 384, 2, 16},   {1, 256, 4, 8},
                             {1, 128, 1, 2},     {1, 16, 8, 8},      {1, 96, 2, 4},     {1, 1024, 2, 8},
                             {2, 320, 2, 8},     {1, 4096, 2, 2},    {2, 2048, 2, 4},   {1, 8192, 8, 32},
                             {2, 16384, 8, 32},  {1, 32768, 8, 64},  {1, 131072, 8, 32}, {1, 384, 3, 6},
                             {1, 600, 5, 5},     {2, 768, 6, 12},    {1, 4480, 7, 7}};
  for (int D = 1; D <= 8; D *= 2)
    for (int c = 1; c <= 1200; c = c * 3 + 7)
      for (int Hq = 1; Hq <= 16; Hq *= 4) cases.push_back({1 + (c & 1), 2 * D * c, D, Hq});
  int checked = 0;
  for (const Case& cs : cases)
    for (int r = 0; r < cs.D; ++r)
      for (int part = 0; part < 2; ++part)
        for (int rbr : {128, 256})
          for (long long target : {512LL, 256LL, 97LL, 2000LL})
            for (int pair = 0; pair < 2; ++pair) {
              const long long slots = rbr == 128 ? 512 : 256;
              if (check(cs.B, cs.S, cs.D, r, part, cs.Hq, rbr, slots, target, pair)) return 1;
              ++checked;
            }
  std::printf("ok %d\n", checked);
  return 0;
}

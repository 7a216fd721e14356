// Work plan of the attention kernels: which rows and key tiles each work
// group processes.  Plain integer code shared by the attention kernel, the
// merge kernel and the host plan, and compiled on its own by the host test
// of the plan (so no HIP header is needed here).
//
// A rank's T = 2c local rows form two halves of c rows.  Zigzag partition
// (Zyphra TSP article on ai-trends.today, section "How to Fold a Book"): the
// halves are chunk r, whose queries see keys [0, (r + 1) c), and chunk
// 2D-1-r, whose queries see keys up to (2D - r) c; positions step by 1 along
// a half.  Striped partition (r007.github.io "Распределенное обучение",
// section "Параллелизм по контексту: Ring Attention против Ulysses", item 1,
// names it beside zigzag): local row t sits at position tD + r, so positions
// step by D and the second half sees the longer key prefixes.  Rows are
// grouped in blocks of rb rows; block index bi in [0, 2 nrb) lists the later
// half's blocks first, last rows first.
#pragma once

#ifndef TSP_HD
#define TSP_HD __host__ __device__
#endif

namespace tsp {

struct BlockGeo {
  int row_begin, row_end;  // local rows of the half
  int gstart;              // global position of the half's first row
  int pstride;             // position step from one local row to the next
  int t0;                  // first local row of the block
  int nkt;                 // key tiles (64 keys) the block needs
  int ns;                  // pieces (0: the block runs inside its partner's last piece)
  int tper;                // key tiles per piece (the last piece may hold fewer)
};

// Rows and key range of block bi (half length c, degree D, rank r,
// partition part: 0 zigzag, 1 striped; rb rows per block, nrb blocks per
// half), not cut into pieces.
TSP_HD inline BlockGeo block_rows(int c, int D, int r, int part, int rbr, int nrb, int bi) {
  BlockGeo g;
  const int late = bi < nrb ? 1 : 0;
  const int rbi = nrb - 1 - (late ? bi : bi - nrb);  // row block within the half
  g.row_begin = late * c;
  g.row_end = g.row_begin + c;
  if (part == 1) {
    g.gstart = late * c * D + r;
    g.pstride = D;
  } else {
    g.gstart = (late ? (2 * D - 1 - r) : r) * c;
    g.pstride = 1;
  }
  g.t0 = g.row_begin + rbi * rbr;
  const int last = g.t0 + rbr - 1 < g.row_end ? g.t0 + rbr - 1 : g.row_end - 1;
  g.nkt = (g.gstart + (last - g.row_begin) * g.pstride + 64) / 64;
  g.ns = 1;
  g.tper = g.nkt;
  return g;
}

// Pieces along the keys.  Unpaired: every block is cut into pieces of at
// most kt_max tiles.  Paired: the later-half block bi (heavy) and the
// earlier-half block 2 nrb - 1 - bi (light) share their work units: their key
// ranges, the heavy block's tiles followed by the light block's, form one
// combined range cut into ns pieces of tper tiles, so every unit of the pair
// weighs the same.  A piece may end in the heavy block, start in the light
// one, or straddle the two; either block is split (partial states merged
// afterwards) when more than one piece touches it.  Light blocks get ns = 0.
TSP_HD inline BlockGeo block_geo(int c, int D, int r, int part, int rbr, int nrb, int kt_max, int pair, int bi) {
  BlockGeo g = block_rows(c, D, r, part, rbr, nrb, bi);
  if (!pair) {
    g.ns = (g.nkt + kt_max - 1) / kt_max;
    g.tper = (g.nkt + g.ns - 1) / g.ns;
  } else if (bi >= nrb) {
    g.ns = 0;
  } else {
    const int tot = g.nkt + block_rows(c, D, r, part, rbr, nrb, 2 * nrb - 1 - bi).nkt;
    g.ns = (tot + kt_max - 1) / kt_max;
    g.tper = (tot + g.ns - 1) / g.ns;
  }
  return g;
}

// Parameters that fix a plan.
struct PlanKey {
  int c, D, r, part, rbr, nrb, kt_max, pair;
};

// How the pieces of block bi (geometry g from block_geo) fall on the blocks
// it computes: nh pieces touch the block itself; paired, the light partner
// has nkt_l tiles and is touched by nl pieces, the first of them piece p0.
// A block is split when more than one piece touches it; its partial states
// then take one workspace slot per piece.
struct PieceSplit {
  int nh, nkt_l, p0, nl;
  int slots;  // workspace slots the block (and its light partner) use
};

TSP_HD inline PieceSplit piece_split(const PlanKey& k, const BlockGeo& g, int bi) {
  PieceSplit q;
  q.nkt_l = 0;
  q.p0 = 0;
  q.nl = 0;
  if (g.ns == 0) {
    q.nh = 0;
    q.slots = 0;
    return q;
  }
  if (!k.pair) {
    q.nh = g.ns;
    q.slots = g.ns > 1 ? g.ns : 0;
    return q;
  }
  q.nkt_l = block_rows(k.c, k.D, k.r, k.part, k.rbr, k.nrb, 2 * k.nrb - 1 - bi).nkt;
  q.nh = (g.nkt + g.tper - 1) / g.tper;
  q.p0 = g.nkt / g.tper;
  q.nl = g.ns - q.p0;
  q.slots = (q.nh > 1 ? q.nh : 0) + (q.nl > 1 ? q.nl : 0);
  return q;
}

// Part `which` of unit piece `piece` of block bi: 0 = the block's own key
// tiles, 1 = the light partner's (paired plans).  Fills the block computed
// (geometry pg), its key tiles [kb, ke), whether its state is partial
// (split) and, if so, its workspace slot relative to the pair's first slot.
// Returns false when the part is empty.
TSP_HD inline bool unit_part(const PlanKey& k, const BlockGeo& g, int bi, const PieceSplit& q, int piece,
                             int which, BlockGeo& pg, int& kb, int& ke, bool& split, int& slot) {
  if (!k.pair) {
    if (which != 0) return false;
    pg = g;
    kb = piece * g.tper;
    ke = kb + g.tper < g.nkt ? kb + g.tper : g.nkt;
    split = g.ns > 1;
    slot = piece;
    return kb < ke;
  }
  const int tot = g.nkt + q.nkt_l;
  const int c0 = piece * g.tper;
  const int c1 = c0 + g.tper < tot ? c0 + g.tper : tot;
  if (which == 0) {
    if (c0 >= g.nkt) return false;
    pg = g;
    kb = c0;
    ke = c1 < g.nkt ? c1 : g.nkt;
    split = q.nh > 1;
    slot = piece;
    return kb < ke;
  }
  if (c1 <= g.nkt) return false;
  pg = block_rows(k.c, k.D, k.r, k.part, k.rbr, k.nrb, 2 * k.nrb - 1 - bi);
  kb = (c0 > g.nkt ? c0 : g.nkt) - g.nkt;
  ke = c1 - g.nkt;
  split = q.nl > 1;
  slot = (q.nh > 1 ? q.nh : 0) + (piece - q.p0);
  return kb < ke;
}

// Work unit u of the attention kernel: block bi, key piece `piece` of
// (sequence, q-head) pair bh; piece_base = workspace slots taken by the
// blocks listed before bi (the index of the block's first slot).
struct UnitPos {
  BlockGeo g;
  int bi, piece, bh, piece_base;
};

TSP_HD inline UnitPos unit_of(const PlanKey& k, int per_bh, int u) {
  UnitPos p;
  p.bi = 0;
  p.piece_base = 0;
  p.g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, 0);
  for (;;) {
    const int n = p.g.ns * per_bh;
    if (u < n || p.bi + 1 >= 2 * k.nrb) break;
    u -= n;
    p.piece_base += piece_split(k, p.g, p.bi).slots;
    ++p.bi;
    p.g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, p.bi);
  }
  p.piece = u / per_bh;
  p.bh = u - p.piece * per_bh;
  return p;
}

// The split block holding merge item `item` when every split block holds
// items_per_block items, in workspace slot order: its geometry, index, first
// slot, number of pieces and the item within it; bi = -1 past the last one.
struct MergePos {
  BlockGeo g;
  int bi, piece_base, npieces;
  long long item;
};

TSP_HD inline MergePos merge_block_of(const PlanKey& k, long long items_per_block, long long item) {
  MergePos m;
  int base = 0;
  for (int bi = 0; bi < 2 * k.nrb; ++bi) {
    const BlockGeo g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, bi);
    const PieceSplit q = piece_split(k, g, bi);
    for (int which = 0; which < 2; ++which) {
      const int n = which == 0 ? q.nh : q.nl;
      if (n <= 1) continue;
      if (item >= items_per_block) {
        item -= items_per_block;
        base += n;
        continue;
      }
      m.g = which == 0 ? g : block_rows(k.c, k.D, k.r, k.part, k.rbr, k.nrb, 2 * k.nrb - 1 - bi);
      m.bi = which == 0 ? bi : 2 * k.nrb - 1 - bi;
      m.piece_base = base;
      m.npieces = n;
      m.item = item;
      return m;
    }
  }
  m.bi = -1;
  m.item = item;
  return m;
}

// The split blocks in workspace slot order, as merge_block_of walks them,
// for the merge kernels (passed as a kernel argument so that no work group
// repeats the walk): entry e is block bi[e] with pieces [base[e], base[e] +
// np[e]).  n = -1 when the plan has more split blocks than the table holds
// (the merge then walks the plan itself).
constexpr int kMergeTab = 32;
struct MergeTab {
  int n;
  int bi[kMergeTab], base[kMergeTab], np[kMergeTab];
};

TSP_HD inline MergeTab merge_table(const PlanKey& k) {
  MergeTab t;
  t.n = 0;
  int base = 0;
  for (int bi = 0; bi < 2 * k.nrb; ++bi) {
    const BlockGeo g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, bi);
    const PieceSplit q = piece_split(k, g, bi);
    for (int which = 0; which < 2; ++which) {
      const int n = which == 0 ? q.nh : q.nl;
      if (n <= 1) continue;
      if (t.n >= kMergeTab) {
        t.n = -1;
        return t;
      }
      t.bi[t.n] = which == 0 ? bi : 2 * k.nrb - 1 - bi;
      t.base[t.n] = base;
      t.np[t.n] = n;
      ++t.n;
      base += n;
    }
  }
  return t;
}

// Whole-plan counts: work units per (sequence, q-head) pair, workspace slots
// of the split blocks, rows of the split blocks.
struct PlanCounts {
  long long units_per_bh;
  int pieces, split_rows;
};

TSP_HD inline PlanCounts plan_counts(const PlanKey& k) {
  PlanCounts n{0, 0, 0};
  for (int bi = 0; bi < 2 * k.nrb; ++bi) {
    const BlockGeo g = block_geo(k.c, k.D, k.r, k.part, k.rbr, k.nrb, k.kt_max, k.pair, bi);
    const PieceSplit q = piece_split(k, g, bi);
    n.units_per_bh += g.ns;
    n.pieces += q.slots;
    n.split_rows += (q.nh > 1 ? k.rbr : 0) + (q.nl > 1 ? k.rbr : 0);
  }
  return n;
}

// kt_max and pairing for a rank: blocks are split only when there are fewer
// than 2 x slots of them (slots = work groups resident on the GPU at once);
// pieces then hold about tiles / target key tiles (at least 16).  pair_req:
// 0 or 1 when blocks are split (ignored otherwise).
TSP_HD inline PlanKey plan_key(int c, int D, int r, int part, int B, int Hq, int rbr, long long slots,
                               long long target, int pair_req) {
  PlanKey k;
  k.c = c;
  k.D = D;
  k.r = r;
  k.part = part;
  k.rbr = rbr;
  k.nrb = (c + rbr - 1) / rbr;
  const long long blocks = 2LL * k.nrb * B * Hq;
  long long tiles = 0;
  for (int bi = 0; bi < 2 * k.nrb; ++bi) tiles += block_rows(c, D, r, part, rbr, k.nrb, bi).nkt;
  tiles *= (long long)B * Hq;
  if (blocks >= 2 * slots) {
    k.kt_max = 1 << 30;
    k.pair = 0;
  } else {
    const long long kt = (tiles + target - 1) / target;
    k.kt_max = (int)(kt < 16 ? 16 : kt);
    k.pair = pair_req;
  }
  return k;
}

}  // namespace tsp

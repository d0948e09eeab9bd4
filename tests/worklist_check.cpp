// Host-only check of the work lists that libdkv's scheduler builds (no GPU needed):
// the library's source is included so that its internal list builders can be called.
//
// For seeded random shapes (prompt groups with empty prompts and empty groups, ragged
// and empty responses, windows, GQA ratios, head dims, split mode) it checks:
//   * forward / dQ items: every (kv head, sequence, query tile) exactly once, with the
//     sequence's rows and its own group's prompt rows;
//   * dK/dV items: every (kv head, sequence, own key tile) exactly once; every
//     (kv head, prompt key tile, sequence of the prompt's group whose rows see the
//     tile) exactly once in atomic mode; in split mode every (kv head, prompt key tile,
//     slice) exactly once, its sequence range inside both the slice's chunk and the
//     tile's group;
//   * layout items: every output row written exactly once, all rows in bounds;
//   * the kernels' own walks (dkv_walks.h, the device code itself compiled for the
//     host): a query item's key tiles cover the keys its rows see (KeyTiles), and a key
//     item's row walk visits each sequence's visible rows exactly once (RowSteps).
// Exit status 0 and "ok <n>" on success; the first violation is printed otherwise.
#include "../shared_prompt_exact_dkv_amd/csrc/dkv_api.cpp"
#include "../shared_prompt_exact_dkv_amd/csrc/dkv_walks.h"

#include <map>
#include <random>
#include <tuple>

#define REQUIRE(c, ...)                          \
  do {                                           \
    if (!(c)) {                                  \
      printf("FAIL %s: ", #c);                   \
      printf(__VA_ARGS__);                       \
      printf("\n");                              \
      exit(1);                                   \
    }                                            \
  } while (0)


// The key tiles a query item visits (KeyTiles, as the forward and dQ kernels walk them,
// tiles of BN keys): within each region (prompt, then own keys) aligned tiles in order,
// together covering every key some row of the item sees and none wholly outside them.
template <int BN> static void check_key_tiles(int P, int wl, int t0, int nt, int seqlen) {
  dkv::KeyTiles<BN> kt;
  kt.init(P, wl, t0, nt);
  const long c_lo = wl >= 0 ? std::max(0, P + t0 - wl) : 0, c_hi = P;   // prompt keys seen
  const long o_lo = wl >= 0 ? std::max(0, t0 - wl) : 0, o_hi = t0 + nt;  // own keys seen
  long c_at = c_lo < c_hi ? c_lo : -1, o_at = o_lo;
  for (int i = 0; i < kt.n; ++i) {
    int nrows, kpos0;
    kt.at(i, P, seqlen, nrows, kpos0);
    if (kt.in_ctx(i)) {
      const int k0 = kt.ctx_start(i);
      REQUIRE(k0 % BN == 0 && k0 <= c_at && k0 + BN > c_at && k0 < c_hi, "prompt tile %d at %d (want %ld)", i, k0, c_at);
      REQUIRE(nrows == P - k0 && kpos0 == k0, "prompt tile rows");
      c_at = std::min<long>(c_hi, k0 + BN);
    } else {
      const int k0 = kt.own_start(i);
      REQUIRE(k0 % BN == 0 && k0 <= o_at && k0 + BN > o_at && k0 < o_hi, "own tile %d at %d (want %ld)", i, k0, o_at);
      REQUIRE(nrows == seqlen - k0 && kpos0 == P + k0, "own tile rows");
      o_at = std::min<long>(o_hi, k0 + BN);
    }
  }
  REQUIRE(c_at == -1 || c_at == c_hi, "prompt keys end at %ld of %ld", c_at, c_hi);
  REQUIRE(o_at == o_hi, "own keys end at %ld of %ld", o_at, o_hi);
}

// The device's row walk run on the host: sequence bounds read from host memory.
struct HostCu {
  static int32_t load(const int32_t *cu, int i) { return cu[i]; }
};

// A key item's row walk (RowSteps, as the dK/dV kernels run it, 32-row steps, with the
// windowed own-key rotation for tiles of rot_bn keys or without it) visits, for each
// sequence whose rows see the item's keys, exactly the flattened rows the scheduler
// counts as visible (kv_rows_visible, cut to the item's row chunk): whole aligned steps
// whose in-range parts tile those rows once, sequences from the last down; a rotated
// walk over a whole band visits step r at position -r mod L.
static void check_walk(const Shape &s, const KVItem &it, int rot_bn) {
  constexpr int BM = 32;
  const bool ctx = it.region == kRegionCtx;
  const int P = it.ctx_len;
  const int nkeys = ctx ? P - it.key_start : s.cu[it.seq_lo + 1] - s.cu[it.seq_lo] - it.key_start;
  const int nk = std::min(s.kv_tile, nkeys);
  dkv::RowSteps<BM, HostCu> rs;
  rs.init(s.cu.data(), it, nk, P, s.wl, s.G, ctx, rot_bn);
  std::map<int, std::vector<std::pair<int, int>>> runs;   // sequence -> (flo, fend) in visit order
  std::map<int, std::vector<int>> steps;
  int last_seq = it.seq_hi, guard = 0;
  while (!rs.done) {
    REQUIRE(++guard < 1 << 22, "walk does not end");
    const int sq = rs.cs;
    REQUIRE(sq >= it.seq_lo && sq < it.seq_hi && sq <= last_seq, "walk sequence %d", sq);
    last_seq = sq;
    REQUIRE(rs.cs0 == s.cu[sq] && rs.clen == s.cu[sq + 1] - s.cu[sq], "cursor bounds");
    int f0, flo, fend;
    rs.advance(f0, flo, fend);
    REQUIRE(f0 % BM == 0 && f0 <= flo && flo < fend && fend <= f0 + BM, "step %d [%d, %d)", f0, flo, fend);
    runs[sq].push_back({flo, fend});
    steps[sq].push_back(f0 / BM);
  }
  for (int i = it.seq_lo; i < it.seq_hi; ++i) {
    const int len = s.cu[i + 1] - s.cu[i];
    long fa, fb;
    if (ctx) {
      fa = 0;
      fb = kv_rows_visible(s, true, it.key_start, nk, len, P) * s.G;
    } else {
      fa = (long)it.key_start * s.G;
      fb = fa + kv_rows_visible(s, false, it.key_start, nk, len, 0) * s.G;
    }
    if (it.row_hi > 0) {
      fa = std::max<long>(fa, it.row_hi - kRowChunk);
      fb = std::max<long>(fa, std::min<long>(fb, it.row_hi));
    }
    std::vector<std::pair<int, int>> r = runs.count(i) ? runs[i] : std::vector<std::pair<int, int>>{};
    std::sort(r.begin(), r.end());
    long at = fa;
    for (auto &x : r) {
      REQUIRE(x.first == at, "seq %d rows: run at %d, want %ld (rows [%ld, %ld))", i, x.first, at, fa, fb);
      at = x.second;
    }
    REQUIRE(at == fb, "seq %d rows end at %ld, want %ld", i, at, fb);
    if (rot_bn > 0 && !ctx && s.wl >= 0 && it.row_hi == 0 && !steps[i].empty()) {
      const int L = ((rot_bn + s.wl) * s.G + BM - 1) / BM;
      const std::vector<int> &v = steps[i];
      if ((int)v.size() == L && fa % BM == 0)
        for (int t = 0; t < L; ++t)
          REQUIRE(((t + v[t]) % L) == 0, "rotated walk: step %d at position %d of %d", v[t], t, L);
    }
  }
}

int main(int argc, char **argv) {
  const int trials = argc > 1 ? atoi(argv[1]) : 400;
  std::mt19937 rng(2026);
  long checked = 0;
  for (int trial = 0; trial < trials; ++trial) {
    const int ng = 1 + rng() % 4;
    // one trial in four has long sequences, whose key tiles split into row chunks
    const int maxlen = (rng() % 4 == 0) ? 3000 : 300;
    std::vector<int> ctx{0}, seq{0}, cu{0};
    for (int j = 0; j < ng; ++j) {
      const int P = (rng() % 4 == 0) ? 0 : rng() % 400;
      const int n = rng() % 5;
      ctx.push_back(ctx.back() + P);
      seq.push_back(seq.back() + n);
      for (int i = 0; i < n; ++i) cu.push_back(cu.back() + ((rng() % 5 == 0) ? rng() % 2 : rng() % maxlen));
    }
    const int hds[6] = {64, 96, 128, 192, 256, 512};
    const int Gs[5] = {1, 2, 3, 4, 8};
    dkv_params p{};
    p.num_seqs = seq.back();
    p.ctx_len = ctx.back();
    p.num_heads_kv = 1 + rng() % 4;
    p.num_heads_q = p.num_heads_kv * Gs[rng() % 5];
    p.head_dim = hds[rng() % 6];
    p.window_left = (rng() % 3 == 0) ? (int)(rng() % 200) : -1;
    p.dtype = DKV_BF16;
    p.cu_seqlens_host = cu.data();
    p.cu_seqlens_dev = cu.data();   // never dereferenced here
    p.num_groups = (ng > 1 || rng() % 2) ? ng : 0;
    p.ctx_cu_host = ctx.data();
    p.group_seq_cu_host = seq.data();
    Shape s;
    REQUIRE(check_params(&p, false, &s) == DKV_OK, "%s", dkv_last_error());
    const int N = s.N;
    auto len = [&](int i) { return s.cu[i + 1] - s.cu[i]; };
    auto group_of = [&](int i) {
      int j = 0;
      while (s.gseq[j + 1] <= i) ++j;
      return j;
    };

    // ---- query-parallel items (forward, dQ)
    for (int bm : {s.bm_tok, s.bm_tok_dq}) {
      std::map<std::tuple<int, int, int>, int> seen;
      for (const QItem &it : build_q_items(s, bm, kFwdBN)) {
        int i = 0;
        while (i < N && !(s.cu[i] == it.seq_start && len(i) == it.seq_len && len(i) > 0)) ++i;
        REQUIRE(i < N, "item with seq_start %d len %d", it.seq_start, it.seq_len);
        // several sequences may share a start (empty ones); take the non-empty one
        REQUIRE(it.g >= 0 && it.g < s.Hkv, "g %d", it.g);
        REQUIRE(it.tile >= 0 && (long)it.tile * bm < it.seq_len, "tile %d", it.tile);
        const int j = group_of(i);
        REQUIRE(it.ctx_start == s.gctx[j] && it.ctx_len == s.gctx[j + 1] - s.gctx[j],
                "prompt of seq %d", i);
        REQUIRE(++seen[std::make_tuple(it.g, i, it.tile)] == 1, "q item repeated");
        const int t0 = it.tile * bm, nt = std::min(bm, it.seq_len - t0);
        check_key_tiles<64>(it.ctx_len, s.wl, t0, nt, it.seq_len);
        check_key_tiles<32>(it.ctx_len, s.wl, t0, nt, it.seq_len);
      }
      long want = 0;
      for (int i = 0; i < N; ++i) want += (long)((len(i) + bm - 1) / bm) * s.Hkv;
      REQUIRE((long)seen.size() == want, "q items %zu of %ld", seen.size(), want);
    }

    // ---- key-parallel items (dK/dV), atomic and split modes
    for (int split = 0; split < 2; ++split) {
      std::map<std::tuple<int, int, int>, int> own, ctxc, slice;
      const int cs = split ? split_chunk(s) : 1;
      for (const KVItem &it : build_kv_items(s, true, split)) {
        REQUIRE(it.g >= 0 && it.g < s.Hkv, "g");
        check_walk(s, it, 0);
        check_walk(s, it, s.kv_tile);
        REQUIRE(it.seq_lo >= 0 && it.seq_lo <= it.seq_hi && it.seq_hi <= N, "range");
        if (it.region == kRegionOwn) {
          REQUIRE(it.seq_hi == it.seq_lo + 1, "own item spans sequences");
          const int i = it.seq_lo, j = group_of(i);
          REQUIRE(it.key_start >= 0 && it.key_start < len(i), "own key tile");
          REQUIRE(it.ctx_start == s.gctx[j] && it.ctx_len == s.gctx[j + 1] - s.gctx[j], "own prompt");
          REQUIRE(++own[std::make_tuple(it.g, i, it.key_start)] == 1, "own item repeated");
        } else {
          REQUIRE(it.region == kRegionCtx, "region");
          // the group whose (non-empty) prompt the item names: prompts of positive
          // length have distinct first rows
          int j = 0;
          while (j < (int)s.gseq.size() - 1 &&
                 !(s.gctx[j] == it.ctx_start && s.gctx[j + 1] - s.gctx[j] == it.ctx_len))
            ++j;
          REQUIRE(j < (int)s.gseq.size() - 1, "ctx item group");
          const int Pg = s.gctx[j + 1] - s.gctx[j];
          REQUIRE(it.ctx_len == Pg && Pg > 0, "ctx prompt length");
          REQUIRE(it.key_start >= 0 && it.key_start < Pg && it.key_start % s.kv_tile == 0, "ctx key tile");
          if (it.seq_hi > it.seq_lo)
            REQUIRE(it.seq_lo >= s.gseq[j] && it.seq_hi <= s.gseq[j + 1], "ctx range outside group");
          if (split) {
            const int c = it.seq_lo / cs;
            REQUIRE(it.seq_hi <= (c + 1) * cs, "split range outside chunk");
            REQUIRE(++slice[std::make_tuple(it.g, s.gctx[j] + it.key_start, c)] == 1, "slice item repeated");
          } else {
            for (int i = it.seq_lo; i < it.seq_hi; ++i)
              REQUIRE(++ctxc[std::make_tuple(it.g, s.gctx[j] + it.key_start, i)] == 1, "ctx pair repeated");
          }
        }
      }
      long want_own = 0;
      for (int i = 0; i < N; ++i) want_own += (long)((len(i) + s.kv_tile - 1) / s.kv_tile) * s.Hkv;
      REQUIRE((long)own.size() == want_own, "own items %zu of %ld", own.size(), want_own);
      for (int j = 0; j + 1 < (int)s.gseq.size(); ++j) {
        const int Pg = s.gctx[j + 1] - s.gctx[j];
        for (int g = 0; g < s.Hkv; ++g)
          for (int k0 = 0; k0 < Pg; k0 += s.kv_tile) {
            const int nk = std::min(s.kv_tile, Pg - k0);
            if (split) {
              for (int c = 0; c < split_slices(s); ++c)
                REQUIRE(slice.count(std::make_tuple(g, s.gctx[j] + k0, c)) == 1, "slice %d of tile missing", c);
            } else {
              for (int i = s.gseq[j]; i < s.gseq[j + 1]; ++i) {
                // a chunk of sequences may include some that do not see the tile (their
                // walk has no rows); every one that does is covered exactly once
                const bool sees = kv_rows_visible(s, true, k0, nk, len(i), Pg) > 0;
                const size_t c = ctxc.count(std::make_tuple(g, s.gctx[j] + k0, i));
                REQUIRE(sees ? c == 1u : c <= 1u,
                        "ctx pair (g %d, key %d, seq %d) coverage", g, s.gctx[j] + k0, i);
              }
            }
          }
      }
    }

    // ---- own key tiles split into row chunks (a call that adds them into the
    // accumulator): a split tile's chunks sit on the kRowChunk grid and cover the
    // flattened rows that see it exactly once; an unsplit tile is one item (row_hi 0)
    for (int chunk = 0; chunk < 2; ++chunk) {
      std::map<std::tuple<int, int, int>, std::vector<int>> tiles;
      const std::vector<KVItem> items = build_kv_items(s, false, false, chunk);
      for (const KVItem &it : items) {
        REQUIRE(it.region == kRegionOwn && it.seq_hi == it.seq_lo + 1, "own item");
        check_walk(s, it, 0);
        check_walk(s, it, s.kv_tile);
        REQUIRE(it.row_hi >= 0 && it.row_hi % kRowChunk == 0, "row_hi %d", it.row_hi);
        tiles[std::make_tuple(it.g, it.seq_lo, it.key_start)].push_back(it.row_hi);
      }
      long want = 0;
      for (int i = 0; i < N; ++i) want += (long)((len(i) + s.kv_tile - 1) / s.kv_tile) * s.Hkv;
      REQUIRE((long)tiles.size() == want, "chunked own tiles %zu of %ld", tiles.size(), want);
      for (auto &t : tiles) {
        const int i = std::get<1>(t.first), k0 = std::get<2>(t.first);
        const int nk = std::min(s.kv_tile, len(i) - k0);
        const long fa = (long)k0 * s.G, fb = fa + kv_rows_visible(s, false, k0, nk, len(i), 0) * s.G;
        std::vector<int> &hs = t.second;
        std::sort(hs.begin(), hs.end());
        if (hs.size() == 1 && hs[0] == 0) {
          REQUIRE(!chunk || fb - fa <= kRowChunk, "unsplit long tile");
          continue;
        }
        REQUIRE(chunk && fb - fa > kRowChunk, "split tile");
        long c = fa / kRowChunk;
        for (int h : hs) {
          REQUIRE(h == (c + 1) * kRowChunk, "chunk grid: row_hi %d, want %ld", h, (c + 1) * kRowChunk);
          ++c;
        }
        REQUIRE((c - 1) * kRowChunk < fb && c * kRowChunk >= fb, "chunks end at the rows' end");
      }
      REQUIRE(plan_bwd(s, false, false, chunk).st.n_kv >= items.size(), "plan bound");
      // the workspace size sizes for the chunks whenever a call may split (the policy)
      if (!chunk || chunk_own_rows(s))
        REQUIRE(plan_bwd(s, false, false, chunk_own_rows(s)).st.n_kv >= items.size(),
                "workspace bound");
    }

    // ---- layout items
    Shape sl;
    REQUIRE(check_layout(&p, DKV_PACK, 64, &sl) == DKV_OK, "%s", dkv_last_error());
    for (int op = DKV_PACK; op <= DKV_FIRST_TOKEN_SCATTER; ++op) {
      LayoutPlan pl = plan_layout(sl, op);
      std::vector<int> cover(pl.out_rows, 0);
      for (const RowItem &it : pl.items) {
        REQUIRE(it.nrows >= 1 && it.nrows <= kRowsPerItem && it.ndst >= 1, "layout item, op %d", op);
        REQUIRE(it.tab_off >= 0 && it.tab_off + it.nsrc + it.ndst <= (int)pl.src.size(), "layout table");
        for (int k = 0; k < it.nsrc; ++k) {
          const int st = pl.src[it.tab_off + k];
          REQUIRE(st >= 0 && st + it.nrows <= pl.in_rows, "layout src, op %d", op);
        }
        for (int k = 0; k < it.ndst; ++k) {
          const int d = pl.src[it.tab_off + it.nsrc + k];
          REQUIRE(d >= 0 && d + it.nrows <= pl.out_rows, "layout dst, op %d", op);
          for (int r = 0; r < it.nrows; ++r) cover[d + r]++;
        }
      }
      for (long r = 0; r < pl.out_rows; ++r)
        REQUIRE(cover[r] == 1, "layout op %d row %ld written %d times", op, r, cover[r]);
    }
    ++checked;
  }
  printf("ok %ld\n", checked);
  return 0;
}

// Host checks of libmac's integer logic, compiled from the library's own
// headers: the KV tile permutations are bijections onto the tile; the
// natural-row tiles' loads, LDS rows and read-back give every lane the
// elements the tile layout gives it; and the split-K plan partitions the
// fresh range [lo, n) into slices that never straddle p_new, with every
// slice non-empty and at most max_slices of them.
#include <cstdio>
#include <cstdlib>
#include <algorithm>
#include <random>
#include <vector>

#include "../../kv_cache_reuse_amd/csrc/mac_dev.h"
#include "../../kv_cache_reuse_amd/csrc/merge_map.h"
#include "../../kv_cache_reuse_amd/csrc/rows_map.h"

static int fails = 0;
#define CHECK(c, ...)                         \
  do {                                        \
    if (!(c)) {                               \
      if (fails < 20) {                       \
        std::printf("FAIL %s: ", #c);         \
        std::printf(__VA_ARGS__);             \
        std::printf("\n");                    \
      }                                       \
      ++fails;                                \
    }                                         \
  } while (0)

template <typename T>
void check_tiles(int D) {
  std::vector<int> seen_k(16 * D, 0), seen_v(16 * D, 0);
  for (int tok = 0; tok < 16; ++tok)
    for (int d = 0; d < D; ++d) {
      int ko = mac::k_tile_offset<T>(tok, d), vo = mac::v_tile_offset<T>(tok, d);
      CHECK(ko >= 0 && ko < 16 * D, "k offset %d (tok %d dim %d D %d)", ko, tok, d, D);
      CHECK(vo >= 0 && vo < 16 * D, "v offset %d (tok %d dim %d D %d)", vo, tok, d, D);
      if (ko >= 0 && ko < 16 * D) seen_k[ko]++;
      if (vo >= 0 && vo < 16 * D) seen_v[vo]++;
    }
  for (int i = 0; i < 16 * D; ++i) {
    CHECK(seen_k[i] == 1, "k slot %d hit %d times (D %d)", i, seen_k[i], D);
    CHECK(seen_v[i] == 1, "v slot %d hit %d times (D %d)", i, seen_v[i], D);
  }
  // lane view: lane l of 1 KiB block j reads elements [64 E j + E l, +E)
  constexpr int E = 16 / sizeof(T);
  for (int tok = 0; tok < 16; ++tok)
    for (int d = 0; d < D; ++d) {
      int ko = mac::k_tile_offset<T>(tok, d);
      int j = ko / (64 * E), lane = (ko % (64 * E)) / E, e = ko % E;
      CHECK(lane % 16 == tok, "k lane %d holds token %d", lane, tok);
      CHECK(d == E * (4 * j + lane / 16) + e, "k lane %d block %d elem %d holds dim %d", lane, j, e, d);
      int vo = mac::v_tile_offset<T>(tok, d);
      int i = vo / (64 * E), vl = (vo % (64 * E)) / E, ve = vo % E;
      CHECK(vl % 16 == d % 16, "v lane %d holds dim %d", vl, d);
      CHECK(tok == 4 * (vl / 16) + ve % 4, "v lane %d elem %d holds token %d", vl, ve, tok);
      CHECK(d / 16 == (E / 4) * i + ve / 4, "v block %d elem %d holds column tile of dim %d", i, ve, d);
    }
}

void check_plan(int lo, int n, int band, int S, int first) {
  mac::Plan p = mac::make_plan(lo, n, band, S, first);
  const int mid = n - band > 0 ? n - band : 0;
  CHECK(p.mid == mid && p.hi == n, "mid/hi");
  CHECK(p.n_pre + p.n_post <= S, "too many slices %d + %d > %d", p.n_pre, p.n_post, S);
  // with a second round, what a hit needs (the slices after p_new and the
  // first one before it) stays below first - 1, the workgroup that copies
  // the reused states
  if (first < S) CHECK(p.n_post <= (first - 2 > 1 ? first - 2 : 1), "%d slices after p_new, first %d", p.n_post, first);
  CHECK((p.lo < p.mid) == (p.n_pre > 0), "pre slices %d for [%d, %d)", p.n_pre, p.lo, p.mid);
  CHECK((p.mid < p.hi) == (p.n_post > 0), "post slices %d for [%d, %d)", p.n_post, p.mid, p.hi);
  // walk the slices in key order: pre slices (indices n_post ..), then post
  // slices (indices 0 .. n_post - 1)
  int cur = p.lo;
  for (int q = 0; q < p.n_pre + p.n_post; ++q) {
    const int i = q < p.n_pre ? p.n_post + q : q - p.n_pre;
    int a, e;
    mac::slice_range(p, i, &a, &e);
    CHECK(mac::slice_is_pre(p, i) == (q < p.n_pre), "slice %d classified wrongly", i);
    if (q == p.n_pre) CHECK(cur == p.mid, "pre slices end at %d, not mid %d", cur, p.mid);
    CHECK(a == cur, "slice %d starts at %d, expected %d (lo %d n %d B %d S %d)", i, a, cur, lo, n, band, S);
    CHECK(e > a, "slice %d empty [%d, %d) (lo %d n %d B %d S %d)", i, a, e, lo, n, band, S);
    if (q < p.n_pre) CHECK(e <= p.mid, "pre slice passes mid");
    else CHECK(a >= p.mid, "post slice before mid");
    bool interior_end = (q != p.n_pre - 1) && (q != p.n_pre + p.n_post - 1);
    if (interior_end) CHECK(e % 16 == 0, "interior bound %d not on a tile edge", e);
    cur = e;
  }
  // the slice holding the last key (the fused append's token)
  if (p.n_pre + p.n_post > 0) {
    const int last = p.n_post > 0 ? p.n_post - 1 : p.n_pre + p.n_post - 1;
    int a, e;
    mac::slice_range(p, last, &a, &e);
    CHECK(e == (p.n_post ? p.hi : p.mid), "slice %d does not hold the last key", last);
  }
  CHECK(cur == (p.n_post ? p.hi : p.mid), "slices end at %d", cur);
}

// Every (group, slice) of the step launch gets exactly one workgroup id;
// padding ids are the only ones left over; the chunks of a wide group's
// slice share an XCD (ids congruent mod 8).  With a sequence order (narrow
// launches, hkv heads per sequence, `first` slices in the first round), the
// first round keeps the slice-major ids and the second round's ids visit
// the sequences in the order given.
void check_coords(int groups, int nchunk, int S, int hkv = 1, int first = 0,
                  const std::vector<unsigned char>* ord = nullptr) {
  const int grid = mac::step_grid(groups, nchunk, S);
  std::vector<int> seen((size_t)groups * S, 0), xcd((size_t)groups * S, -1);
  unsigned long long word = 0;   // nibble k: the sequence of rank k
  if (ord)
    for (size_t k = 0; k < ord->size(); ++k) word |= (unsigned long long)(*ord)[k] << (4 * k);
  int pad = 0, prev_rank = 0;
  for (int id = 0; id < grid; ++id) {
    int g = -1, s = -1;
    const bool real = mac::step_coords(id, groups, nchunk, S, &g, &s, hkv, first,
                                       ord != nullptr, word);
    if (ord && real) {
      if (id < groups * first) {
        CHECK(g == id % groups && s == id / groups, "first-round id %d -> (%d, %d)", id, g, s);
      } else {
        CHECK(s >= first, "second-round id %d -> slice %d < first %d", id, s, first);
        int rank = 0;
        while (rank < (int)ord->size() && (*ord)[rank] != g / hkv) ++rank;
        CHECK(rank >= prev_rank, "id %d: sequence rank %d after rank %d", id, rank, prev_rank);
        prev_rank = rank;
      }
    }
    if (!real) {
      CHECK(s == S && g >= 0 && g < groups, "padding id %d -> (%d, %d)", id, g, s);
      ++pad;
      continue;
    }
    CHECK(g >= 0 && g < groups && s >= 0 && s < S, "id %d -> (%d, %d) out of range (G %d C %d S %d)",
          id, g, s, groups, nchunk, S);
    if (g < 0 || g >= groups || s < 0 || s >= S) continue;
    seen[(size_t)g * S + s]++;
    xcd[(size_t)g * S + s] = id % mac::kXcds;
  }
  for (size_t i = 0; i < seen.size(); ++i)
    CHECK(seen[i] == 1, "(group %zu, slice %zu) taken %d times (G %d C %d S %d)", i / S, i % S,
          seen[i], groups, nchunk, S);
  CHECK(pad < nchunk * mac::kXcds, "%d padding ids", pad);
  if (nchunk > 1)
    for (int g = 0; g < groups; ++g)
      for (int s = 0; s < S; ++s) {
        const int first = xcd[(size_t)(g - g % nchunk) * S + s];
        CHECK(xcd[(size_t)g * S + s] == first, "chunks of group %d slice %d on different XCDs", g, s);
      }
}

// Every (query head, dim part) of the merge launch gets exactly one id, the
// head's group is the one it belongs to, and with a multiple of 8 groups
// every merge workgroup of a group is on the XCD of the group's step
// workgroups (ids congruent mod 8 to the group's step ids).
void check_merge_coords(int batch, int hkv, int group, int parts, int S) {
  const int hq = hkv * group, n = batch * hq * parts, groups = batch * hkv;
  std::vector<int> seen((size_t)n, 0);
  for (int id = 0; id < n; ++id) {
    const mac::MergeCoords m = mac::merge_coords(id, batch, hkv, group, parts);
    const bool ok = m.b >= 0 && m.b < batch && m.h >= 0 && m.h < hq && m.q >= 0 && m.q < parts &&
                    m.hi == m.h % group && m.grp == m.b * hkv + m.h / group;
    CHECK(ok, "merge id %d -> (b %d, h %d, hi %d, q %d, grp %d)", id, m.b, m.h, m.hi, m.q, m.grp);
    if (!ok) continue;
    seen[((size_t)m.b * hq + m.h) * parts + m.q]++;
    if (groups % mac::kXcds == 0) {
      int g = -1, s = -1;
      mac::step_coords(m.grp + groups * (S - 1), groups, 1, S, &g, &s);
      CHECK(g == m.grp && id % mac::kXcds == (m.grp + groups * (S - 1)) % mac::kXcds,
            "merge id %d of group %d on another XCD", id, m.grp);
    }
  }
  for (int i = 0; i < n; ++i) CHECK(seen[i] == 1, "merge (head, part) %d taken %d times", i, seen[i]);
}

// Natural-row tiles.  A tile's element (token, dim) sits at token * D + dim
// of the row tile and at k_tile_offset / v_tile_offset of a library tile; a
// wave load j gives lane l the 16 bytes at element E (64 j + l) of either.
// The row path writes each load's piece into the LDS rows and reads the
// operands back (bf16 values through a model of the transposing LDS read:
// in each block of 16 lanes, lane B + i takes element i mod 4 of the 4 at
// the address of lane B + 4 r + i / 4 as its element r); every operand
// element must be the one the tile path loads into that lane and slot.
template <typename T>
void check_rows(int D) {
  const int E = 16 / (int)sizeof(T);
  const int NL = D * (int)sizeof(T) / 64;
  const int PR = 4 * NL;
  const int RS = D + (sizeof(T) == 2 ? mac::kRowsPadBf16 : mac::kRowsPadF32);
  std::vector<int> kinv(16 * D, -1), vinv(16 * D, -1);
  for (int tok = 0; tok < 16; ++tok)
    for (int d = 0; d < D; ++d) {
      kinv[mac::k_tile_offset<T>(tok, d)] = tok * D + d;
      vinv[mac::v_tile_offset<T>(tok, d)] = tok * D + d;
    }
  std::vector<int> lds(16 * RS, -1);
  for (int j = 0; j < NL; ++j)
    for (int lane = 0; lane < 64; ++lane) {
      const int row = mac::rows_load_row(j, lane, PR), piece = mac::rows_load_piece(j, lane, PR);
      CHECK(row >= 0 && row < 16 && piece >= 0 && piece < PR, "load %d lane %d -> row %d piece %d", j, lane, row, piece);
      for (int e = 0; e < E; ++e) {
        const int label = E * (64 * j + lane) + e;   // the row tile's element there
        CHECK(label == row * D + E * piece + e, "load %d lane %d e %d: row %d piece %d", j, lane, e, row, piece);
        CHECK(lds[row * RS + E * piece + e] == -1, "LDS slot written twice (row %d piece %d)", row, piece);
        lds[row * RS + E * piece + e] = label;
      }
    }
  for (int j = 0; j < NL; ++j)
    for (int lane = 0; lane < 64; ++lane)
      for (int e = 0; e < E; ++e) {
        const int got = lds[mac::rows_key_row(lane) * RS + E * mac::rows_key_piece(j, lane) + e];
        CHECK(got == kinv[E * (64 * j + lane) + e], "key j %d lane %d e %d: %d vs %d (D %d)", j, lane, e, got,
              kinv[E * (64 * j + lane) + e], D);
      }
  for (int i = 0; i < NL; ++i)
    for (int lane = 0; lane < 64; ++lane) {
      if (sizeof(T) == 2) {
        const int B = lane & ~15, ii = lane % 16;
        for (int th = 0; th < 2; ++th)
          for (int r = 0; r < 4; ++r) {
            const int src = B + 4 * r + ii / 4;
            const int col = 32 * i + 16 * th + mac::tr16_col(src);
            CHECK(col + 3 < D, "transposing read past the row (col %d, D %d)", col, D);
            const int got = lds[mac::tr16_row(src) * RS + col + ii % 4];
            const int want = vinv[E * (64 * i + lane) + 4 * th + r];
            CHECK(got == want, "value i %d lane %d th %d r %d: %d vs %d (D %d)", i, lane, th, r, got, want, D);
          }
      } else {
        for (int r = 0; r < 4; ++r) {
          const int got = lds[(4 * (lane / 16) + r) * RS + 16 * i + lane % 16];
          const int want = vinv[4 * (64 * i + lane) + r];
          CHECK(got == want, "value i %d lane %d r %d: %d vs %d (D %d)", i, lane, r, got, want, D);
        }
      }
    }
  // the fused-append patch of row r touches each of its pieces once
  for (int r = 0; r < 16; ++r) {
    std::vector<int> seen(PR, 0);
    for (int j = 0; j < NL; ++j)
      for (int lane = 0; lane < 64; ++lane)
        if (mac::rows_load_row(j, lane, PR) == r) seen[mac::rows_load_piece(j, lane, PR)]++;
    for (int p = 0; p < PR; ++p) CHECK(seen[p] == 1, "patch of row %d: piece %d taken %d times", r, p, seen[p]);
  }
}

int main() {
  check_tiles<uint16_t>(64);
  check_tiles<uint16_t>(128);
  check_tiles<float>(64);
  check_tiles<float>(128);
  check_rows<uint16_t>(64);
  check_rows<uint16_t>(128);
  check_rows<float>(64);
  check_rows<float>(128);
  std::mt19937 rng(123);
  const int Ss[] = {2, 3, 8, 16, 34, 128, 1024};
  for (int it = 0; it < 200000; ++it) {
    int n = 1 + rng() % (it % 3 == 0 ? 300 : 200000);
    int band = rng() % 4 == 0 ? 0 : rng() % 600;
    int mid = n - band > 0 ? n - band : 0;
    int lo = rng() % 2 ? 0 : (int)(rng() % (mid + 1));
    int S = Ss[rng() % 7];
    // one round, or a first round of about half the slices
    int first = rng() % 2 ? S : (S / 2 > 0 ? S / 2 : 1);
    check_plan(lo, n, band, S, first);
  }
  for (int groups : {1, 2, 3, 8, 16, 64})
    for (int S : {2, 5, 32, 128, 1024}) check_coords(groups, 1, S);
  for (int batch : {1, 2, 3, 8})
    for (int hkv : {1, 2, 8})
      for (int group : {1, 4, 8, 16, 32})
        for (int parts : {4, 8}) check_merge_coords(batch, hkv, group, parts, 32);
  // second-round orders: batch x hkv groups, first < S, random permutations
  std::mt19937 orng(7);
  for (int batch : {2, 3, 8, 11, 16})
    for (int hkv : {1, 2, 8})
      for (int S : {2, 5, 8, 16}) {
        std::vector<unsigned char> ord(batch);
        for (int b = 0; b < batch; ++b) ord[b] = (unsigned char)b;
        std::shuffle(ord.begin(), ord.end(), orng);
        for (int first = 1; first < S; first += (S > 4 ? 3 : 1))
          check_coords(batch * hkv, 1, S, hkv, first, &ord);
      }
  for (int real : {1, 2, 3, 8})
    for (int nc : {2, 3, 4})
      for (int S : {2, 5, 13, 64, 128}) check_coords(real * nc, nc, S);
  check_plan(0, 131072 + 512, 256, 128, 128);
  check_plan(131072 + 300 - 256 - 1, 131072 + 300, 256, 128, 128);
  check_plan(131072 + 300 - 256 - 1, 131072 + 300, 256, 8, 4);
  if (fails) {
    std::printf("%d failures\n", fails);
    return 1;
  }
  std::printf("OK\n");
  return 0;
}

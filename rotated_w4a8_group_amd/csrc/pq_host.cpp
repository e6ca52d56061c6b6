// Host-side parts of the C ABI: version, error state, partition validation and the rotation
// record builder.
//
// Record building follows "ParoQuant (PARO) W4A8 on gfx1201 — engineering log", section
// "Format" (pairs [8, K] local to each 128-group, one f16 angle per pair) and section
// "Design" item 3 (8-byte records {i | j << 8, cos f16, sin f16}). The lane order inside
// each (layer, group) is this library's own: it makes the prologue's in-place LDS updates
// free of bank conflicts (see order_layer below).
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "pq_internal.h"

namespace pq {

static thread_local std::string g_last_error;

int set_error(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int check_partitions(int P, int pb1, int pb2, int N) {
  if (P < 1 || P > PQ_MAX_PARTITIONS)
    return set_error(PQ_ERR_PARTITION, "P=%d must be in 1..3", P);
  // boundaries at or past N do not split anything
  const bool b1 = pb1 < N, b2 = pb2 < N;
  if (b2 && !b1) return set_error(PQ_ERR_PARTITION, "pb2=%d < N but pb1=%d is not", pb2, pb1);
  if (b1 && (pb1 <= 0 || pb1 % PQ_GROUP))
    return set_error(PQ_ERR_PARTITION, "pb1=%d must be a positive multiple of 128", pb1);
  if (b2 && (pb2 <= pb1 || pb2 % PQ_GROUP))
    return set_error(PQ_ERR_PARTITION, "pb2=%d must be a multiple of 128 above pb1=%d", pb2, pb1);
  const int expect = 1 + (b1 ? 1 : 0) + (b2 ? 1 : 0);
  if (P != expect)
    return set_error(PQ_ERR_PARTITION, "P=%d but the boundaries (%d, %d) split N=%d into %d parts",
                     P, pb1, pb2, N, expect);
  return PQ_OK;
}

// IEEE binary16 round-to-nearest-even of a double, done on the bits (no double rounding).
static uint16_t f16_from_double(double v) {
  uint64_t b;
  std::memcpy(&b, &v, 8);
  const uint16_t sign = static_cast<uint16_t>((b >> 48) & 0x8000);
  const double a = std::fabs(v);
  if (std::isnan(v)) return sign | 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;  // rounds to infinity
  int e;
  std::frexp(a, &e);                        // a = f * 2^e, f in [0.5, 1)
  int exp16 = e - 1;                        // a in [2^exp16, 2^(exp16+1))
  if (a == 0.0) return sign;
  if (exp16 < -14) exp16 = -14;             // subnormal spacing 2^-24
  const double ulp = std::ldexp(1.0, exp16 - 10);
  const double q = a / ulp;                 // exact: power-of-two scaling
  double n = std::floor(q);
  const double rem = q - n;
  if (rem > 0.5 || (rem == 0.5 && std::fmod(n, 2.0) != 0.0)) n += 1.0;
  // n * ulp, re-encoded
  const double r = n * ulp;
  if (r >= 65520.0) return sign | 0x7C00;
  if (r < std::ldexp(1.0, -14)) return sign | static_cast<uint16_t>(n);  // subnormal (n < 1024)
  int e2;
  const double f2 = std::frexp(r, &e2);     // r = f2 * 2^e2, f2 in [0.5, 1)
  const uint16_t mant = static_cast<uint16_t>(std::ldexp(f2, 11) - 1024.0);
  const uint16_t exp = static_cast<uint16_t>(e2 - 1 + 15);
  return sign | static_cast<uint16_t>(exp << 10) | mant;
}

static double f16_to_double(uint16_t h) {
  const int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = std::ldexp(m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = std::ldexp(1024 + m, e - 25);
  return s ? -v : v;
}

// Lane order for the 64 pairs of the first layer of a group (later layers follow from it, see
// chain_group).
//
// The prologue keeps 4 tokens of a token-group in LDS token-minor: channel c occupies the
// 16-byte row lds_row(c) = c + c/8 (one padding row per 8 channels). In each layer lane l reads
// the row of its pair's first channel ("tail"), then the row of the second ("head"), rotates
// the 4 tokens and writes both rows back. A 16-byte access by 64 lanes is served in passes of
// 16 lanes over 64 banks or 8 lanes over 32 banks, so it is conflict-free when, in every block of
// 16 lanes, the tails' rows are distinct mod 16 and the heads' rows too, and in every half-block
// of 8 lanes they are distinct mod 8. This picks each pair's orientation (listing a pair as
// (j, i) is the same rotation with sin negated) and its lane so that both hold.
//
// Residues u = lds_row(c) mod 16 take each value for exactly 8 channels, so the pairs are the
// edges of an 8-regular multigraph on 16 residues. Orienting every edge along an Euler circuit
// gives each residue 4 outgoing and 4 incoming edges; the bipartite graph (outgoing side x
// incoming side) is then 4-regular and splits into 4 perfect matchings, each one a block whose
// 16 tails and 16 heads are all distinct residues. Inside a block, edges whose tails differ by 8
// are linked, and so are edges whose heads differ by 8; the links form even alternating cycles,
// and colouring each cycle alternately gives two half-blocks distinct mod 8.
static int lds_row(int c) { return c + (c >> 3); }

// Returns false only if a step that cannot fail for a valid pairing did (never expected).
static bool order_layer(const int* pi, const int* pj, int* tail, int* head, int* lane_of) {
  // residue multigraph and an Euler orientation (Hierholzer, iterative)
  int ru[64], rv[64];
  for (int q = 0; q < 64; ++q) { ru[q] = lds_row(pi[q]) & 15; rv[q] = lds_row(pj[q]) & 15; }
  std::vector<int> adj[16];
  for (int q = 0; q < 64; ++q) { adj[ru[q]].push_back(q); if (rv[q] != ru[q]) adj[rv[q]].push_back(q); else adj[ru[q]].push_back(q); }
  bool used[64] = {false};
  size_t ptr[16] = {0};
  int from[64];   // residue the oriented edge leaves
  for (int s = 0; s < 16; ++s) {
    // walk circuits from s until all its edges are used; orientation = direction of travel
    std::vector<int> stack{s};
    while (!stack.empty()) {
      const int v = stack.back();
      while (ptr[v] < adj[v].size() && used[adj[v][ptr[v]]]) ++ptr[v];
      if (ptr[v] == adj[v].size()) { stack.pop_back(); continue; }
      const int q = adj[v][ptr[v]];
      used[q] = true;
      from[q] = v;
      stack.push_back(ru[q] == v ? rv[q] : ru[q]);
    }
  }
  int tr[64], hr[64];   // tail / head residue of each oriented edge
  for (int q = 0; q < 64; ++q) {
    const bool fwd = from[q] == ru[q];
    tail[q] = fwd ? pi[q] : pj[q];
    head[q] = fwd ? pj[q] : pi[q];
    tr[q] = lds_row(tail[q]) & 15;
    hr[q] = lds_row(head[q]) & 15;
  }
  // split into 4 perfect matchings of the 4-regular bipartite multigraph tail residue -> head residue
  int block[64];
  bool taken[64] = {false};
  for (int b = 0; b < 4; ++b) {
    int match_h[16], match_t[16];   // head residue -> edge, tail residue -> edge
    for (int r = 0; r < 16; ++r) match_h[r] = match_t[r] = -1;
    for (int u = 0; u < 16; ++u) {
      // augmenting path from tail residue u (Kuhn's algorithm over the untaken edges)
      int prev_edge[16];
      bool seen[16] = {false};
      std::vector<int> queue{u};
      int found = -1;
      for (size_t qi = 0; qi < queue.size() && found < 0; ++qi) {
        const int t = queue[qi];
        for (int q = 0; q < 64 && found < 0; ++q) {
          if (taken[q] || tr[q] != t || seen[hr[q]]) continue;
          seen[hr[q]] = true;
          prev_edge[hr[q]] = q;
          if (match_h[hr[q]] < 0) found = hr[q];
          else queue.push_back(tr[match_h[hr[q]]]);
        }
      }
      // a regular bipartite graph always has a perfect matching, so the path exists
      if (found < 0) return false;
      for (int h = found; h >= 0;) {
        const int q = prev_edge[h];
        const int t = tr[q];
        const int next = match_t[t] >= 0 ? hr[match_t[t]] : -1;
        match_h[h] = q;
        match_t[t] = q;
        h = (t == u) ? -1 : next;
      }
    }
    for (int r = 0; r < 16; ++r) { taken[match_t[r]] = true; block[match_t[r]] = b; }
  }
  // halves of each block: alternate colours along tail-mate / head-mate cycles
  for (int b = 0; b < 4; ++b) {
    int by_t[16], by_h[16];
    for (int q = 0; q < 64; ++q)
      if (block[q] == b) { by_t[tr[q]] = q; by_h[hr[q]] = q; }
    int color[64];
    for (int q = 0; q < 64; ++q) color[q] = -1;
    int n[2] = {0, 0};
    for (int r0 = 0; r0 < 16; ++r0) {
      int q = by_t[r0];
      if (color[q] >= 0) continue;
      int c = 0;
      bool via_tail = true;
      while (color[q] < 0) {
        color[q] = c;
        lane_of[q] = 16 * b + 8 * c + n[c]++;
        q = via_tail ? by_t[tr[q] ^ 8] : by_h[hr[q] ^ 8];
        via_tail = !via_tail;
        c ^= 1;
      }
    }
    if (n[0] != 8 || n[1] != 8) return false;
  }
  return true;
}

// Proper edge colouring of a bipartite multigraph in which every node has degree deg: n left
// and n right nodes, edge e joins left[e] and right[e]. Colour c's edges form a perfect matching
// (found by augmenting paths among the uncoloured edges; a regular bipartite multigraph always
// has one, and removing it leaves a regular one). Returns false only if that fails.
static bool colour_regular(int n, int deg, const int* left, const int* right, int* colour) {
  const int E = n * deg;
  for (int e = 0; e < E; ++e) colour[e] = -1;
  for (int c = 0; c < deg; ++c) {
    std::vector<int> match_r(n, -1), match_l(n, -1);   // node -> edge
    for (int u = 0; u < n; ++u) {
      std::vector<int> prev_edge(n, -1);
      std::vector<bool> seen(n, false);
      std::vector<int> queue{u};
      int found = -1;
      for (size_t qi = 0; qi < queue.size() && found < 0; ++qi) {
        const int a = queue[qi];
        for (int e = 0; e < E && found < 0; ++e) {
          if (colour[e] >= 0 || left[e] != a || seen[right[e]]) continue;
          seen[right[e]] = true;
          prev_edge[right[e]] = e;
          if (match_r[right[e]] < 0) found = right[e];
          else queue.push_back(left[match_r[right[e]]]);
        }
      }
      if (found < 0) return false;
      for (int b = found; b >= 0;) {
        const int e = prev_edge[b];
        const int a = left[e];
        const int next = match_l[a] >= 0 ? right[match_l[a]] : -1;
        match_r[b] = e;
        match_l[a] = e;
        b = (a == u) ? -1 : next;
      }
    }
    for (int a = 0; a < n; ++a) colour[match_l[a]] = c;
  }
  return true;
}

// The record chain of one group (8 layers x 64 lanes), see pq_build_records: pi[r][q], pj[r][q]
// are the channels of pair q of layer r. Layer 0 takes order_layer's lanes. From each layer to
// the next, the two pairings form even cycles; keeping alternate channels along each cycle gives
// every lane one output it consumes itself in the next layer (that layer's first operand) and one
// it hands to another lane through an LDS row, chosen so that both the writes and the reads are
// free of bank conflicts. A handed-off value may travel negated (the lane computes f1*v - f2*u
// for either output it hands on); neg_v records that for the reader. Returns false only on an
// internal failure.
struct LaneRec {
  int u, v;          // the lane's pair as it computes it: u the first operand, v the second
  int rslot, wslot;  // hand-off rows read (layers 1..7) and written (layers 0..6)
  bool keep_v;       // the output kept in registers for the next layer is v's (layers 0..6)
  bool neg_v;        // the second operand arrives negated (layers 1..7)
};
static bool chain_group(const int (*pi)[64], const int (*pj)[64], LaneRec (*out)[64]) {
  // layer 0: lane order and orientation from order_layer (conflict-free reads of the image)
  {
    int tail[64], head[64], lane_of[64];
    if (!order_layer(pi[0], pj[0], tail, head, lane_of)) return false;
    for (int q = 0; q < 64; ++q) out[0][lane_of[q]] = LaneRec{tail[q], head[q], 0, 0, false, false};
  }
  for (int r = 0; r + 1 < PQ_LAYERS; ++r) {
    int nxt[128], lane_at[128];
    for (int q = 0; q < 64; ++q) { nxt[pi[r + 1][q]] = pj[r + 1][q]; nxt[pj[r + 1][q]] = pi[r + 1][q]; }
    for (int l = 0; l < 64; ++l) { lane_at[out[r][l].u] = l; lane_at[out[r][l].v] = l; }
    // Along each cycle of layer r's and layer r+1's pairings, keep alternate ends: every pair of
    // layer r then keeps one channel and every pair of layer r+1 contains exactly one kept one.
    int keep[64];
    bool done[64] = {false};
    for (int l0 = 0; l0 < 64; ++l0) {
      if (done[l0]) continue;
      int l = l0, k = out[r][l0].u;
      while (true) {
        done[l] = true;
        keep[l] = k;
        const int x = nxt[k];             // handed off by its layer-r lane
        const int lx = lane_at[x];
        if (lx == l0) {
          if (x != (out[r][l0].u == keep[l0] ? out[r][l0].v : out[r][l0].u)) return false;
          break;
        }
        if (done[lx]) return false;
        l = lx;
        k = (out[r][l].u == x) ? out[r][l].v : out[r][l].u;
      }
    }
    // layer r+1: lane l continues with its kept channel as the first operand
    for (int l = 0; l < 64; ++l) {
      out[r][l].keep_v = keep[l] == out[r][l].v;
      out[r + 1][l] = LaneRec{keep[l], nxt[keep[l]], 0, 0, false, false};
    }
    // hand-off slots: writer lane l (8-lane block l/8) -> reader lane l2 (16-lane block l2/16);
    // slot = 16 (l2/16) + rho with rho distinct in each reader block (reads: rows distinct mod 16)
    // and rho mod 8 distinct in each writer block (writes: rows distinct mod 8)
    int reader[64], wl[64], hr[64], col[64];
    for (int l2 = 0; l2 < 64; ++l2) reader[lane_at[out[r + 1][l2].v]] = l2;   // v of l2 is handed off by its layer-r lane
    int seen_rb[4] = {0, 0, 0, 0};
    for (int l = 0; l < 64; ++l) {
      const int rb = reader[l] / 16;
      wl[l] = l / 8;
      hr[l] = 2 * rb + (seen_rb[rb]++ < 8 ? 0 : 1);   // halves of the reader block, 8 edges each
    }
    if (!colour_regular(8, 8, wl, hr, col)) return false;
    for (int l = 0; l < 64; ++l) {
      const int slot = 16 * (reader[l] / 16) + col[l] + 8 * (hr[l] & 1);
      out[r][l].wslot = slot;
      out[r + 1][reader[l]].rslot = slot;
      // the handed output carries the writer's operand sign, flipped once more when v's output
      // is the one kept (see pq_build_records)
      out[r + 1][reader[l]].neg_v = out[r][l].neg_v != out[r][l].keep_v;
    }
  }
  return true;
}

}  // namespace pq

extern "C" {

int pq_abi_version(void) { return PQ_ABI_VERSION; }

const char* pq_last_error(void) { return pq::g_last_error.c_str(); }

int pq_build_records(const int16_t* pairs_h, const uint16_t* theta_h, int K, void* rec_h) {
  using namespace pq;
  clear_error();
  if (!pairs_h || !theta_h || !rec_h) return set_error(PQ_ERR_NULL, "pq_build_records: NULL pointer");
  if (K <= 0 || K % PQ_GROUP) return set_error(PQ_ERR_SHAPE, "pq_build_records: K=%d must be a positive multiple of 128", K);
  const int G = K / PQ_GROUP, half = K / 2;
  for (int r = 0; r < PQ_LAYERS; ++r)
    for (int g = 0; g < G; ++g) {
      bool seen[128] = {false};
      for (int c = 0; c < PQ_GROUP; ++c) {
        const int v = pairs_h[static_cast<size_t>(r) * K + g * PQ_GROUP + c];
        if (v < 0 || v >= PQ_GROUP || seen[v])
          return set_error(PQ_ERR_RECORDS, "pairs layer %d group %d is not a permutation of 0..127", r, g);
        seen[v] = true;
      }
    }
  std::vector<uint8_t> out(static_cast<size_t>(PQ_LAYERS) * half * 8);
  for (int g = 0; g < G; ++g) {
    int pi[PQ_LAYERS][64], pj[PQ_LAYERS][64];
    uint16_t c16[PQ_LAYERS][64], s16[PQ_LAYERS][64];
    int pair_of[PQ_LAYERS][128];
    for (int r = 0; r < PQ_LAYERS; ++r)
      for (int q = 0; q < 64; ++q) {
        const size_t pidx = static_cast<size_t>(r) * K + g * PQ_GROUP + 2 * q;
        pi[r][q] = pairs_h[pidx];
        pj[r][q] = pairs_h[pidx + 1];
        pair_of[r][pi[r][q]] = q;
        pair_of[r][pj[r][q]] = q;
        const double th = f16_to_double(theta_h[static_cast<size_t>(r) * half + g * 64 + q]);
        c16[r][q] = f16_from_double(std::cos(th));
        s16[r][q] = f16_from_double(std::sin(th));
      }
    LaneRec lr[PQ_LAYERS][64];
    if (!chain_group(pi, pj, lr))
      return set_error(PQ_ERR_RECORDS, "pairs group %d: lane ordering failed", g);
    for (int r = 0; r < PQ_LAYERS; ++r)
      for (int l = 0; l < 64; ++l) {
        const LaneRec& e = lr[r][l];
        const int q = pair_of[r][e.u];
        // (c, s) of the pair listed as (u, v): listing it as (j, i) negates sin
        const uint16_t c = c16[r][q];
        const uint16_t sn = (pi[r][q] == e.u) ? s16[r][q] : static_cast<uint16_t>(s16[r][q] ^ 0x8000);
        // The lane reads w = t v (t = -1 when neg_v) and computes keep = f1 u + f2 w and
        // hand = f1 w - f2 u:
        //   kept output u: (f1, f2) = (c, t s): keep = c u + s v,  hand = t (c v - s u)
        //   kept output v: (f1, f2) = (-s, t c): keep = c v - s u, hand = -t (c u + s v)
        // so a handed value is the other output times t, negated again when v's is kept. The last
        // layer keeps u's output and writes t * hand, v's output, to the image.
        const bool kv = (r + 1 < PQ_LAYERS) && e.keep_v;
        const uint16_t t = e.neg_v ? 0x8000 : 0;
        const uint16_t f1 = kv ? static_cast<uint16_t>(sn ^ 0x8000) : c;
        const uint16_t f2 = static_cast<uint16_t>((kv ? c : sn) ^ t);
        const uint32_t w = static_cast<uint32_t>(e.u) | (e.neg_v ? 0x80u : 0u) | (static_cast<uint32_t>(e.v) << 8) |
                           (kv ? 0x8000u : 0u) | (static_cast<uint32_t>(r > 0 ? e.rslot : 0) << 16) |
                           (static_cast<uint32_t>(r + 1 < PQ_LAYERS ? e.wslot : 0) << 24);
        uint8_t* dst = out.data() + (static_cast<size_t>(r) * half + g * 64 + l) * 8;
        std::memcpy(dst, &w, 4);
        std::memcpy(dst + 4, &f1, 2);
        std::memcpy(dst + 6, &f2, 2);
      }
  }
  std::memcpy(rec_h, out.data(), out.size());
  return PQ_OK;
}

int pq_plan_partitions(int J, const int* ncols_h, const int16_t* const* pairs_h,
                       const uint16_t* const* theta_h, const uint16_t* const* cs_h, int K,
                       int* P_out, int* pb_out, int* rep_out) {
  using namespace pq;
  clear_error();
  if (!ncols_h || !pairs_h || !theta_h || !cs_h || !P_out || !pb_out || !rep_out)
    return set_error(PQ_ERR_NULL, "pq_plan_partitions: NULL pointer");
  if (J < 1 || J > 64) return set_error(PQ_ERR_SHAPE, "pq_plan_partitions: J=%d must be in 1..64", J);
  if (K <= 0 || K % PQ_GROUP) return set_error(PQ_ERR_SHAPE, "pq_plan_partitions: K=%d must be a positive multiple of 128", K);
  for (int j = 0; j < J; ++j) {
    if (ncols_h[j] <= 0 || ncols_h[j] % 16)
      return set_error(PQ_ERR_SHAPE, "pq_plan_partitions: projection %d has %d columns (positive multiple of 16)", j, ncols_h[j]);
    if (!pairs_h[j] || !theta_h[j] || !cs_h[j]) return set_error(PQ_ERR_NULL, "pq_plan_partitions: NULL rotation data for projection %d", j);
  }
  const size_t pb = sizeof(int16_t) * PQ_LAYERS * K, tb = sizeof(uint16_t) * PQ_LAYERS * (K / 2),
               cb = sizeof(uint16_t) * K;
  auto same = [&](int a, int b) {
    return std::memcmp(pairs_h[a], pairs_h[b], pb) == 0 && std::memcmp(theta_h[a], theta_h[b], tb) == 0 &&
           std::memcmp(cs_h[a], cs_h[b], cb) == 0;
  };
  // runs of adjacent projections with identical rotation data
  int P = 0, rep[PQ_MAX_PARTITIONS], bound[PQ_MAX_PARTITIONS];
  int64_t col = 0;
  for (int j = 0; j < J; ++j) {
    if (j == 0 || !same(j - 1, j)) {
      if (P == PQ_MAX_PARTITIONS)
        return set_error(PQ_ERR_PARTITION, "pq_plan_partitions: more than %d runs of distinct rotations", PQ_MAX_PARTITIONS);
      if (P > 0 && col % PQ_GROUP)
        return set_error(PQ_ERR_PARTITION, "pq_plan_partitions: a partition boundary at column %lld is not a multiple of 128",
                         static_cast<long long>(col));
      rep[P] = j;
      bound[P] = static_cast<int>(col);
      ++P;
    }
    col += ncols_h[j];
    if (col > (1 << 24)) return set_error(PQ_ERR_SHAPE, "pq_plan_partitions: too many columns");
  }
  *P_out = P;
  pb_out[0] = P > 1 ? bound[1] : PQ_NO_BOUNDARY;
  pb_out[1] = P > 2 ? bound[2] : PQ_NO_BOUNDARY;
  for (int q = 0; q < PQ_MAX_PARTITIONS; ++q) rep_out[q] = q < P ? rep[q] : -1;
  return PQ_OK;
}

}  // extern "C"

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

// Lane order for the 64 pairs of one (layer, group).
//
// The prologue keeps a token's 128 channels in LDS in channel order (word c at bank c mod 64
// and c mod 32) and updates a layer in place: lane l reads channel t_l, then channel h_l,
// rotates, and writes both back. This picks for each pair which channel is read first
// (t = "tail") and which lane it goes to so that
//   * across the 64 lanes the tails are distinct mod 64 and so are the heads, and
//   * within each half-wave (lanes 0-31, 32-63) tails and heads are distinct mod 32,
// which makes every read and write conflict-free whether the LDS serves a wave in one pass
// over 64 banks or in two half-wave passes over 32 banks.
//
// Tails mod 64: channels c and c^64 share a 64-bank; pair edges plus these sibling links form
// even alternating cycles, so walking each cycle and taking every second channel as a tail
// gives one tail per 64-bank. Halves: each 32-residue is then the tail of exactly two pairs
// and the head of exactly two; linking pairs that share a tail residue or a head residue
// gives even cycles again, and colouring each cycle alternately splits the pairs into two
// halves of 32 with distinct residues.
static void order_layer(const int* pi, const int* pj, int* tail, int* head, int* lane_of) {
  int partner[128];
  for (int q = 0; q < 64; ++q) { partner[pi[q]] = pj[q]; partner[pj[q]] = pi[q]; }
  int pair_of[128];
  for (int q = 0; q < 64; ++q) { pair_of[pi[q]] = q; pair_of[pj[q]] = q; }
  bool done[64] = {false};
  for (int q0 = 0; q0 < 64; ++q0) {
    if (done[q0]) continue;
    int t = pi[q0];
    while (true) {
      const int q = pair_of[t];
      if (done[q]) break;
      done[q] = true;
      tail[q] = t;
      head[q] = partner[t];
      t = head[q] ^ 64;  // the sibling of a head must be a tail
    }
  }
  // tail-mate / head-mate links by residue mod 32
  int tmate[64], hmate[64];
  int first_t[32], first_h[32];
  for (int r = 0; r < 32; ++r) first_t[r] = first_h[r] = -1;
  for (int q = 0; q < 64; ++q) {
    const int rt = tail[q] & 31, rh = head[q] & 31;
    if (first_t[rt] < 0) first_t[rt] = q; else { tmate[q] = first_t[rt]; tmate[first_t[rt]] = q; }
    if (first_h[rh] < 0) first_h[rh] = q; else { hmate[q] = first_h[rh]; hmate[first_h[rh]] = q; }
  }
  int color[64];
  for (int q = 0; q < 64; ++q) color[q] = -1;
  for (int q0 = 0; q0 < 64; ++q0) {
    if (color[q0] >= 0) continue;
    int q = q0, c = 0;
    bool via_tail = true;
    while (color[q] < 0) {
      color[q] = c;
      q = via_tail ? tmate[q] : hmate[q];
      via_tail = !via_tail;
      c ^= 1;
    }
  }
  int n0 = 0, n1 = 32;
  for (int q = 0; q < 64; ++q) lane_of[q] = color[q] == 0 ? n0++ : n1++;
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
  for (int r = 0; r < PQ_LAYERS; ++r)
    for (int g = 0; g < G; ++g) {
      int pi[64], pj[64], tail[64], head[64], lane_of[64];
      uint16_t c16[64], s16[64];
      for (int q = 0; q < 64; ++q) {
        const size_t pidx = static_cast<size_t>(r) * K + g * PQ_GROUP + 2 * q;
        pi[q] = pairs_h[pidx];
        pj[q] = pairs_h[pidx + 1];
        const double th = f16_to_double(theta_h[static_cast<size_t>(r) * half + g * 64 + q]);
        c16[q] = f16_from_double(std::cos(th));
        s16[q] = f16_from_double(std::sin(th));
      }
      order_layer(pi, pj, tail, head, lane_of);
      for (int q = 0; q < 64; ++q) {
        // listing the pair as (j, i) is the same rotation with sin negated
        const uint16_t s = (tail[q] == pi[q]) ? s16[q] : static_cast<uint16_t>(s16[q] ^ 0x8000);
        const uint32_t ij = static_cast<uint32_t>(tail[q]) | (static_cast<uint32_t>(head[q]) << 8);
        uint8_t* dst = out.data() + (static_cast<size_t>(r) * half + g * 64 + lane_of[q]) * 8;
        std::memcpy(dst, &ij, 4);
        std::memcpy(dst + 4, &c16[q], 2);
        std::memcpy(dst + 6, &s, 2);
      }
    }
  std::memcpy(rec_h, out.data(), out.size());
  return PQ_OK;
}

}  // extern "C"

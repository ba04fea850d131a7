// Host-side validation of the rotation parameters and construction of the
// per-segment schedule that the gfx950 rotation kernel executes.
//
// What is computed follows the ParoQuant paper notes, section "关键设计":
// K stages of independent Givens rotations on disjoint channel pairs inside
// each quantization group, preceded by the channel scaling diag(alpha); the
// 2x2 update is the CSDN article's section 2.2 matrix [[c, -s], [s, c]] on
// (v_i, v_j). On the activation side the scaling is 1/alpha and the stages run
// in the same order with the same update (x T^-1 for a row x).
#include <algorithm>
#include <cmath>
#include <cstring>

#include "paro_internal.h"

namespace paro {
namespace {

constexpr int kMaxK = 32;

uint32_t fbits(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return u;
}

// v_perm_b32 byte selectors (result byte k <- byte sel[k] of {src0:src1}).
constexpr uint32_t kSelLoadKeep = 0x03020100u;  // kept channel is the low half
constexpr uint32_t kSelLoadSwap = 0x01000302u;  // kept channel is the high half
constexpr uint32_t kSelStoreX = 0x03020100u;    // packed (X low, fetched high) as is
constexpr uint32_t kSelStoreB = 0x01000302u;    // halves swapped: fetched low, X high

// One segment's sequence of pairings: index 0 is the natural pairing before
// stage 0, 1..K are the stages, K+1 is the natural pairing after the last
// stage. partner[tt][ch] is the other member of ch's pair; first[tt][ch] is
// 1 when ch is the pair's first member (the "i" of (i, j)); cs[tt][ch] holds
// the pair's fp64 cos and sin.
struct SegPairings {
  int C = 0;
  std::vector<std::vector<int>> partner;
  std::vector<std::vector<uint8_t>> first;
  std::vector<std::vector<double>> c, s;
};

// Identity pairs for the factored stage form, which cannot swap the members of
// an identity pair: a lane that holds one has to keep the channel it kept at
// the exchange before. On entry S holds the segment's rotations at stages
// 1..KA (partner -1 where a stage leaves a channel free) and the natural
// pairings of stages 0 and KA+1 that load and store it.
//
// Every rotation, and every natural pair of stage 0, is a node with one bit:
// whether its lower channel is the one that stays in its lane at the exchange
// right after it. A channel's standing at exchange tau is then fixed by the
// last node it belongs to up to stage tau (an identity pair changes nothing).
// The lanes work out when every pair of stage tau+1 has one member that stays
// and one that does not; for a rotation, or a natural pair of stage KA+1, that
// ties the bits of its members' previous nodes with a parity. A node meets at
// most two such ties, one through each member, so the ties form paths and
// cycles; going once round a cycle enters and leaves every node through
// different members, the parities cancel, and the ties always have a solution
// (found with a union-find that tracks parities). Free bits go, in stage order,
// to whichever keeps the larger of a rotation's |cos| and |sin| on the register
// it stays in. With the bits fixed, the channels a stage leaves free split
// evenly into those that stay at the exchange before it and those that do not;
// pairing one half with the other gives identity pairs whose lanes keep their
// registers. kset[tau][ch] says whether ch stays at exchange tau.
bool fill_kept(SegPairings& S, int KA, double tiny, std::vector<std::vector<uint8_t>>& kset) {
  const int C = S.C;
  struct Node { int stage, lo, hi, prev_lo, prev_hi; };
  std::vector<Node> nodes;
  std::vector<int> uf_par, uf_x;
  auto add_node = [&](Node n) {
    uf_par.push_back((int)nodes.size());
    uf_x.push_back(0);
    nodes.push_back(n);
    return (int)nodes.size() - 1;
  };
  auto find = [&](int v, int& parity) {
    int p = 0, u = v;
    while (uf_par[u] != u) {
      p ^= uf_x[u];
      u = uf_par[u];
    }
    for (int w = v, pw = p; uf_par[w] != w;) {  // path compression
      const int nx = uf_par[w], xw = uf_x[w];
      uf_par[w] = u;
      uf_x[w] = pw;
      pw ^= xw;
      w = nx;
    }
    parity = p;
    return u;
  };
  std::vector<int> node_of(C);
  std::vector<std::vector<int>> node_at(KA + 1, std::vector<int>(C, -1));
  for (int ch = 0; ch < C; ch += 2) node_of[ch] = node_of[ch + 1] = add_node({0, ch, ch + 1, -1, -1});
  for (int ch = 0; ch < C; ++ch) node_at[0][ch] = node_of[ch];
  for (int tt = 1; tt <= KA + 1; ++tt) {
    for (int u = 0; u < C; ++u) {
      const int w = S.partner[tt][u];
      if (w < u) continue;  // free (-1), or visited from the lower member
      const int nu = node_of[u], nw = node_of[w];
      // stays(ch) = bit(node) ^ (ch is not the node's lower member); one of u, w stays
      const int rel = 1 ^ (u != nodes[nu].lo) ^ (w != nodes[nw].lo);
      int pu, pw;
      const int ru = find(nu, pu), rw = find(nw, pw);
      if (ru == rw) {
        if ((pu ^ pw) != rel) return false;
      } else {
        uf_par[ru] = rw;
        uf_x[ru] = pu ^ pw ^ rel;
      }
      if (tt <= KA) node_of[u] = node_of[w] = node_at[tt][u] = node_at[tt][w] = add_node({tt, u, w, nu, nw});
    }
  }
  // a rotation whose cos (or sin) is below `tiny` has to keep (or swap) the
  // channel in its register: a tie with the previous node of its lower member
  // (these extra ties can contradict the others; the caller then falls back)
  for (size_t n = 0; n < nodes.size(); ++n) {
    const Node& nd = nodes[n];
    if (nd.stage == 0) continue;
    const double c = std::fabs(S.c[nd.stage][nd.lo]), s = std::fabs(S.s[nd.stage][nd.lo]);
    if (c >= tiny && s >= tiny) continue;
    // lo stays at both exchanges iff bit(n) ^ bit(prev) == (lo is not prev's lower member)
    const int rel = (nd.lo != nodes[nd.prev_lo].lo ? 1 : 0) ^ (c < tiny ? 1 : 0);
    int pa, pb;
    const int ra = find((int)n, pa), rb = find(nd.prev_lo, pb);
    if (ra == rb) {
      if ((pa ^ pb) != rel) return false;
    } else {
      uf_par[ra] = rb;
      uf_x[ra] = pa ^ pb ^ rel;
    }
  }
  // bits, in stage order
  std::vector<int> root_bit(nodes.size(), -1), bit(nodes.size(), 0);
  auto stays = [&](int n, int ch) { return bit[n] ^ (ch != nodes[n].lo ? 1 : 0); };
  for (size_t n = 0; n < nodes.size(); ++n) {
    int parity;
    const int root = find((int)n, parity);
    if (root_bit[root] < 0) {
      int b = 1;
      const Node& nd = nodes[n];
      if (nd.stage > 0) {
        const int x = stays(nd.prev_lo, nd.lo) ? nd.lo : nd.hi;  // in the register that stays
        const bool keep = std::fabs(S.c[nd.stage][nd.lo]) >= std::fabs(S.s[nd.stage][nd.lo]);
        b = ((x == nd.lo) == keep) ? 1 : 0;
      }
      root_bit[root] = b ^ parity;
    }
    bit[n] = root_bit[root] ^ parity;
  }
  // standings per exchange
  kset.assign(KA + 1, std::vector<uint8_t>(C, 0));
  for (int ch = 0; ch < C; ++ch) node_of[ch] = node_at[0][ch];
  for (int tau = 0; tau <= KA; ++tau) {
    for (int ch = 0; ch < C; ++ch) {
      if (node_at[tau][ch] >= 0) node_of[ch] = node_at[tau][ch];
      kset[tau][ch] = (uint8_t)stays(node_of[ch], ch);
    }
  }
  // identity pairs: a free channel that stays with a free one that does not,
  // the previous stage's partner first
  for (int tt = 1; tt <= KA; ++tt) {
    auto pair_id = [&](int a, int b) {
      S.partner[tt][a] = b;
      S.partner[tt][b] = a;
      S.first[tt][std::min(a, b)] = 1;
    };
    std::vector<int> A, B;
    for (int ch = 0; ch < C; ++ch) {
      if (S.partner[tt][ch] >= 0) continue;
      const int q = S.partner[tt - 1][ch];
      if (kset[tt - 1][ch] && S.partner[tt][q] < 0 && !kset[tt - 1][q]) {
        pair_id(ch, q);
        continue;
      }
      (kset[tt - 1][ch] ? A : B).push_back(ch);
    }
    std::vector<int> A2, B2;
    for (int ch : A) if (S.partner[tt][ch] < 0) A2.push_back(ch);
    for (int ch : B) if (S.partner[tt][ch] < 0) B2.push_back(ch);
    if (A2.size() != B2.size()) return false;
    for (size_t i = 0; i < A2.size(); ++i) pair_id(A2[i], B2[i]);
  }
  return true;
}

// Kuhn augmenting path on a bipartite multigraph given as edge lists.
bool augment(int u, const std::vector<std::vector<std::pair<int, int>>>& adj,
             std::vector<int>& match_r, std::vector<int>& match_edge_r, std::vector<char>& seen,
             const std::vector<char>& edge_used) {
  for (auto [v, e] : adj[u]) {
    if (edge_used[e] || seen[v]) continue;
    seen[v] = 1;
    if (match_r[v] < 0 || augment(match_r[v], adj, match_r, match_edge_r, seen, edge_used)) {
      match_r[v] = u;
      match_edge_r[v] = e;
      return true;
    }
  }
  return false;
}

// LDS slots for one exchange. On gfx950 a 16-byte LDS write is conflict-free
// when every 8 consecutive lanes hit 8 distinct 16-byte positions modulo 8, and
// a 16-byte read when every 16 consecutive lanes hit positions distinct modulo
// 16. src[v] is the lane whose value v reads; the lane u is written by writer
// block u / 8 and read by reader block src_inv[u] / 16. Colour c = lo + 8 hi:
// lo is an 8-edge-colouring of the bipartite multigraph (writer block) --
// (reader block half), which is 8-regular once every reader block's 16 edges
// are split into two halves of 8, so lo is distinct inside every writer block
// and appears exactly twice inside every reader block; hi then separates the
// two. slot = c + 16 k keeps slot % 8 = lo and slot % 16 = c. Returns slot[v].
std::vector<int> plan_lds_slots(const std::vector<int>& src) {
  const int nv = (int)src.size();
  const int nw = nv / 8, nr = nv / 16;
  std::vector<int> src_inv(nv);
  for (int v = 0; v < nv; ++v) src_inv[src[v]] = v;
  // reader half-node of u: (src_inv[u] / 16) * 2 + (position of u among that block's lanes) / 8
  std::vector<int> half_of(nv), seen_in_block(nr, 0);
  for (int r = 0; r < nv; ++r) {  // iterate readers in order; each reads exactly one u
    const int u = src[r];
    const int blk = r / 16;
    half_of[u] = blk * 2 + (seen_in_block[blk]++ >= 8 ? 1 : 0);
  }
  std::vector<std::vector<std::pair<int, int>>> adj(nw);
  for (int u = 0; u < nv; ++u) adj[u / 8].push_back({half_of[u], u});
  std::vector<char> used(nv, 0);
  std::vector<int> lo(nv, -1);
  for (int col = 0; col < 8; ++col) {
    std::vector<int> match_r(2 * nr, -1), match_e(2 * nr, -1);
    for (int u = 0; u < nw; ++u) {
      std::vector<char> seen(2 * nr, 0);
      augment(u, adj, match_r, match_e, seen, used);
    }
    for (int v = 0; v < 2 * nr; ++v) {
      if (match_e[v] < 0) return {};  // cannot happen for a regular bipartite multigraph
      used[match_e[v]] = 1;
      lo[match_e[v]] = col;
    }
  }
  // hi: inside every reader block each lo value occurs twice (once per half)
  std::vector<int> colour(nv);
  for (int u = 0; u < nv; ++u) colour[u] = lo[u] + 8 * (half_of[u] & 1);
  std::vector<int> slot(nv), next(16, 0);
  for (int u = 0; u < nv; ++u) slot[u] = colour[u] + 16 * next[colour[u]]++;
  return slot;
}

struct LaneState {
  std::vector<std::vector<int>> kept, fetched, src;  // [tau][v]
};

// Lane slots of one stage for the gradient kernel, which keeps a batch in LDS
// channel-major with channel c's rows in 16-byte slot c and reads (writes) the
// rows of a slot's two channels with one 16-byte access per channel. gfx950
// serves such reads without bank conflicts when every 16 consecutive lanes hit
// slots distinct modulo 16, i.e. channels distinct modulo 16, and writes when
// every 8 consecutive lanes hit channels distinct modulo 8. The pairs of a stage are placed as follows:
//  * each pair is oriented (its first channel a, second b) so that every
//    residue modulo 16 is first as often as it is second: an Eulerian
//    orientation of the multigraph on the 16 residues whose edges are the
//    pairs (every residue has even degree, two per channel); a pair stored
//    the other way round is the same rotation with the sine negated and its
//    angle gradient negated;
//  * the oriented pairs form a regular bipartite multigraph (first residue
//    -> second residue) that splits into perfect matchings of 16 pairs, one
//    per 16-lane block and slot;
//  * inside a block, the two halves of 8 lanes take the two perfect matchings
//    of the 2-regular graph of residues modulo 8.
// pr[k] = (i, j) segment-local; returns pos[k] (the slot index lane * ppl + q)
// and flip[k]; an empty result if a step fails (it cannot for valid input).
bool plan_backward_slots(const std::vector<std::pair<int, int>>& pr, int ppl, std::vector<int>& pos,
                         std::vector<char>& flip) {
  const int np = (int)pr.size();  // 64 ppl
  // Eulerian orientation by closed trails
  std::vector<std::vector<std::pair<int, int>>> g(16);
  for (int k = 0; k < np; ++k) {
    g[pr[k].first & 15].push_back({pr[k].second & 15, k});
    g[pr[k].second & 15].push_back({pr[k].first & 15, k});
  }
  std::vector<char> used(np, 0);
  std::vector<size_t> it(16, 0);
  flip.assign(np, 0);
  std::vector<int> tail(np), head(np);
  for (int s0 = 0; s0 < 16; ++s0) {
    for (;;) {
      int u = s0;
      bool moved = false;
      for (;;) {
        while (it[u] < g[u].size() && used[g[u][it[u]].second]) ++it[u];
        if (it[u] == g[u].size()) break;
        const auto [w, k] = g[u][it[u]];
        used[k] = 1;
        // orient k as u -> w
        if ((pr[k].first & 15) == u) {
          flip[k] = 0;
        } else {
          flip[k] = 1;
        }
        tail[k] = u;
        head[k] = w;
        u = w;
        moved = true;
      }
      if (!moved) break;
    }
  }
  // perfect matchings of the bipartite multigraph tail -> head
  std::vector<std::vector<std::pair<int, int>>> adj(16);
  for (int k = 0; k < np; ++k) adj[tail[k]].push_back({head[k], k});
  std::vector<char> taken(np, 0);
  std::vector<int> match_of(np, -1);
  const int nm = np / 16;
  for (int m = 0; m < nm; ++m) {
    std::vector<int> mr(16, -1), me(16, -1);
    for (int u = 0; u < 16; ++u) {
      std::vector<char> seen(16, 0);
      augment(u, adj, mr, me, seen, taken);
    }
    for (int v = 0; v < 16; ++v) {
      if (me[v] < 0) return false;
      taken[me[v]] = 1;
      match_of[me[v]] = m;
    }
  }
  // halves of each matching, and positions
  pos.assign(np, -1);
  for (int m = 0; m < nm; ++m) {
    std::vector<int> ks;
    for (int k = 0; k < np; ++k)
      if (match_of[k] == m) ks.push_back(k);
    std::vector<std::vector<std::pair<int, int>>> a8(8);
    std::vector<char> t8(np, 0);
    for (int k : ks) a8[tail[k] & 7].push_back({head[k] & 7, k});
    int fill[2] = {0, 0};
    for (int h = 0; h < 2; ++h) {
      std::vector<int> mr(8, -1), me(8, -1);
      for (int u = 0; u < 8; ++u) {
        std::vector<char> seen(8, 0);
        augment(u, a8, mr, me, seen, t8);
      }
      for (int v = 0; v < 8; ++v) {
        if (me[v] < 0) return false;
        t8[me[v]] = 1;
        const int lane = 16 * (m % 4) + 8 * h + fill[h]++;
        pos[me[v]] = lane * ppl + m / 4;
      }
    }
  }
  return true;
}

}  // namespace

int build_rotation_plan(int64_t d, int32_t group, int32_t K, const int32_t* pairs,
                        const float* theta, const float* alpha, RotPlanHost* out) {
  if (!out || !alpha || (K > 0 && (!pairs || !theta))) {
    set_error("null pointer argument");
    return PARO_ERR_NULL;
  }
  if (d <= 0 || group <= 0 || K < 0) {
    set_error("d, group must be positive and K non-negative");
    return PARO_ERR_SHAPE;
  }
  if (group != 64 && group != 128 && group != 256) {
    set_error("group must be 64, 128 or 256");
    return PARO_ERR_UNSUPPORTED;
  }
  if (d % group) {
    set_error("d must be a multiple of group");
    return PARO_ERR_SHAPE;
  }
  if (d % 128) {
    set_error("d must be a multiple of 128");
    return PARO_ERR_UNSUPPORTED;
  }
  if (K > kMaxK) {
    set_error("K > 32 is not supported");
    return PARO_ERR_UNSUPPORTED;
  }
  if (d > (int64_t(1) << 24)) {
    set_error("d > 2^24 is not supported");
    return PARO_ERR_UNSUPPORTED;
  }
  for (int64_t k = 0; k < d; ++k) {
    if (!std::isfinite(alpha[k]) || !(alpha[k] > 0.0f)) {
      set_error("alpha must be finite and > 0 (channel " + std::to_string(k) + ")");
      return PARO_ERR_VALUE;
    }
  }
  const int64_t half = d / 2;
  for (int64_t e = 0; e < (int64_t)K * half; ++e) {
    if (!std::isfinite(theta[e])) {
      set_error("theta must be finite");
      return PARO_ERR_VALUE;
    }
  }
  // pairings: a perfect pairing inside every group, per stage
  {
    std::vector<int> seen(d);
    for (int t = 0; t < K; ++t) {
      std::fill(seen.begin(), seen.end(), 0);
      for (int64_t p = 0; p < half; ++p) {
        int64_t i = pairs[(t * half + p) * 2], j = pairs[(t * half + p) * 2 + 1];
        if (i < 0 || j < 0 || i >= d || j >= d || i == j) {
          set_error("stage " + std::to_string(t) + ": channel index out of range or i == j");
          return PARO_ERR_PAIRING;
        }
        if (i / group != j / group) {
          set_error("stage " + std::to_string(t) + ": pair crosses a group boundary");
          return PARO_ERR_PAIRING;
        }
        if (seen[i]++ || seen[j]++) {
          set_error("stage " + std::to_string(t) + ": channel appears twice");
          return PARO_ERR_PAIRING;
        }
      }
    }
  }

  RotPlanHost& P = *out;
  P.alpha.assign(alpha, alpha + d);
  const int seg_ch = group == 256 ? 256 : 128;
  const int nv = seg_ch / 2;
  const int segs = (int)(d / seg_ch);

  // ---- canonical fp32 tables for the weight transform -------------------------
  const int64_t groups = d / group;
  const int gp = group / 2;
  P.wt_pairs.assign((size_t)groups * K * gp, 0);
  P.wt_c.assign((size_t)groups * K * gp, 0.f);
  P.wt_s.assign((size_t)groups * K * gp, 0.f);
  {
    std::vector<int> fill(groups);
    for (int t = 0; t < K; ++t) {
      std::fill(fill.begin(), fill.end(), 0);
      for (int64_t p = 0; p < half; ++p) {
        int64_t i = pairs[(t * half + p) * 2], j = pairs[(t * half + p) * 2 + 1];
        int64_t g = i / group;
        size_t at = ((size_t)g * K + t) * gp + fill[g]++;
        P.wt_pairs[at] = (uint32_t)(i - g * group) | ((uint32_t)(j - g * group) << 16);
        double th = (double)theta[t * half + p];
        P.wt_c[at] = (float)std::cos(th);
        P.wt_s[at] = (float)std::sin(th);
      }
    }
  }

  // ---- table of the gradient kernel --------------------------------------------
  // Per segment, stage and lane slot k (lane k / ppl, sub-slot k % ppl): the
  // pair's segment-local channels (i | j << 16), fp32 cos and sin (the same
  // roundings as the weight transform), and the pair's flat index t * d/2 + p
  // in the caller's theta. Identities (theta = 0) are kept: their angle
  // gradient is not zero.
  // Slots are placed by plan_backward_slots; a pair stored the other way
  // round has its sine negated and bit 31 of the index set (its angle
  // gradient is negated when written out).
  {
    const int ppl = seg_ch / 128;
    P.bw.assign((size_t)segs * K * nv * 4, 0);
    std::vector<std::vector<int64_t>> members(segs);
    for (int t = 0; t < K; ++t) {
      for (auto& m : members) m.clear();
      for (int64_t p = 0; p < half; ++p) members[pairs[(t * half + p) * 2] / seg_ch].push_back(p);
      for (int sg = 0; sg < segs; ++sg) {
        std::vector<std::pair<int, int>> pr;
        for (int64_t p : members[sg])
          pr.push_back({(int)(pairs[(t * half + p) * 2] - (int64_t)sg * seg_ch),
                        (int)(pairs[(t * half + p) * 2 + 1] - (int64_t)sg * seg_ch)});
        std::vector<int> pos;
        std::vector<char> flip;
        if ((int)pr.size() != nv || !plan_backward_slots(pr, ppl, pos, flip)) {
          set_error("internal: could not place the gradient kernel's pairs");
          return PARO_ERR_HIP;
        }
        for (int k = 0; k < nv; ++k) {
          const int64_t p = members[sg][k];
          uint32_t* e = &P.bw[(((size_t)sg * K + t) * nv + (size_t)pos[k]) * 4];
          const int a = flip[k] ? pr[k].second : pr[k].first, b = flip[k] ? pr[k].first : pr[k].second;
          e[0] = (uint32_t)a | ((uint32_t)b << 16);
          const double th = (double)theta[t * half + p];
          const float sn = (float)std::sin(th);
          e[1] = fbits((float)std::cos(th));
          e[2] = fbits(flip[k] ? -sn : sn);
          e[3] = (uint32_t)(t * half + p) | (flip[k] ? 0x80000000u : 0u);
        }
      }
    }
  }

  // ---- stage compaction for partial pairings ------------------------------------
  // A pair with theta == 0 is an exact identity. When a plan has identities
  // (a partial or sparse pairing), they are dropped, and every other rotation
  // moves to the earliest activation stage after the last rotation on either
  // of its channels: rotations keep their order on every channel, and
  // rotations on disjoint pairs commute, so the product is unchanged. The
  // activation kernel then executes KA <= K stages (the longest chain of
  // rotations linked by shared channels); channels a stage leaves free get
  // identity pairs chosen below. The weight transform above keeps the K
  // stages in their canonical order.
  std::vector<int> eff((size_t)K * half, -1);  // activation stage of each pair, -1: identity
  int KA = K;
  bool has_identity = false;
  {
    std::vector<int> last(d, -1);
    int ka = 0;
    bool identity = false;
    for (int t = 0; t < K; ++t)
      for (int64_t p = 0; p < half; ++p) {
        const int64_t i = pairs[(t * half + p) * 2], j = pairs[(t * half + p) * 2 + 1];
        if (theta[t * half + p] == 0.0f) {
          identity = true;
          continue;
        }
        const int e = std::max(last[i], last[j]) + 1;
        eff[(size_t)t * half + p] = e;
        last[i] = last[j] = e;
        ka = std::max(ka, e + 1);
      }
    has_identity = identity;
    if (identity) {
      KA = ka;
    } else {
      for (int t = 0; t < K; ++t)
        for (int64_t p = 0; p < half; ++p) eff[(size_t)t * half + p] = t;
    }
  }

  // ---- activation schedule ------------------------------------------------------
  for (int attempt = 0; attempt < 2; ++attempt) {
    const bool fast = attempt == 0;
    RotPlanLayout lay;
    lay.seg_ch = seg_ch;
    lay.ppl = seg_ch / 128;
    lay.nv = nv;
    lay.fast = fast;
    lay.coef = fast ? 2 : 4;
    lay.words = rot_words(KA, lay.coef);
    lay.stages = KA;
    std::vector<uint32_t> table(rot_table_words(segs, lay), 0);
    bool ok = true;

    for (int sg = 0; sg < segs && ok; ++sg) {
      const int64_t base = (int64_t)sg * seg_ch;
      SegPairings S;
      S.C = seg_ch;
      S.partner.assign(KA + 2, std::vector<int>(seg_ch, -1));
      S.first.assign(KA + 2, std::vector<uint8_t>(seg_ch, 0));
      S.c.assign(KA + 2, std::vector<double>(seg_ch, 1.0));
      S.s.assign(KA + 2, std::vector<double>(seg_ch, 0.0));
      for (int ch = 0; ch < seg_ch; ++ch) {
        S.partner[0][ch] = S.partner[KA + 1][ch] = ch ^ 1;
        S.first[0][ch] = S.first[KA + 1][ch] = (ch & 1) == 0;
      }
      for (int t = 0; t < K; ++t) {
        for (int64_t p = 0; p < half; ++p) {
          const int e = eff[(size_t)t * half + p];
          if (e < 0) continue;  // identity
          int64_t i = pairs[(t * half + p) * 2], j = pairs[(t * half + p) * 2 + 1];
          if (i < base || i >= base + seg_ch) continue;
          int li = (int)(i - base), lj = (int)(j - base);
          double th = (double)theta[t * half + p];
          S.partner[e + 1][li] = lj;
          S.partner[e + 1][lj] = li;
          S.first[e + 1][li] = 1;
          S.first[e + 1][lj] = 0;
          S.c[e + 1][li] = S.c[e + 1][lj] = std::cos(th);
          S.s[e + 1][li] = S.s[e + 1][lj] = std::sin(th);
        }
      }
      // Channels no rotation of a stage touches get identity pairs (c = 1,
      // s = 0). The factored form cannot swap the two members of an identity
      // pair (one of its coefficients would be zero), so the lane that holds
      // one must keep the channel already in its register. fill_kept() picks
      // the identity pairs so that this always holds: see there. The general
      // form takes any identity pairs: a free channel is paired with its
      // partner of the previous stage where both are free, the rest in
      // channel order.
      // Coefficient bounds. A factored stage computes c*a + s*b as
      // c*(a + (s/c)*b): one fp32 fma whose rounding error is relative to the
      // result, so a small leading coefficient costs no accuracy (a quarter
      // turn, |cos| ~ 4e-8 for a float angle, is fine). Only a leading
      // coefficient below `tiny` (in practice an exact zero) is refused, and the
      // deferred scales and ratios stay within [lo, hi] so that the registers
      // keep far from the fp32 range limits.
      const double lo = std::ldexp(1.0, -60), hi = std::ldexp(1.0, 60), tiny = std::ldexp(1.0, -40);
      std::vector<std::vector<uint8_t>> kset;  // kset[tau][ch]: ch stays in its lane at exchange tau
      if (fast && has_identity) {
        if (!fill_kept(S, KA, tiny, kset)) { ok = false; break; }
      } else {
      for (int tt = 1; tt <= KA; ++tt) {
        auto pair_id = [&](int a2, int b2) {
          S.partner[tt][a2] = b2;
          S.partner[tt][b2] = a2;
          S.first[tt][std::min(a2, b2)] = 1;
        };
        for (int ch = 0; ch < seg_ch; ++ch) {
          const int q = S.partner[tt - 1][ch];
          if (S.partner[tt][ch] < 0 && q >= 0 && q != ch && S.partner[tt][q] < 0) pair_id(ch, q);
        }
        int pending = -1;
        for (int ch = 0; ch < seg_ch; ++ch) {
          if (S.partner[tt][ch] >= 0) continue;
          if (pending < 0) pending = ch;
          else { pair_id(pending, ch); pending = -1; }
        }
      }
      }

      // mu(out <- in) of the pairing tt's 2x2 update, for two members of one pair
      auto mu = [&](int tt, int out_ch, int in_ch) -> double {
        bool oi = S.first[tt][out_ch], ii = S.first[tt][in_ch];
        double c = S.c[tt][out_ch], s = S.s[tt][out_ch];
        if (oi) return ii ? c : -s;
        return ii ? s : c;
      };


      LaneState L;
      L.kept.assign(KA + 1, std::vector<int>(nv));
      L.fetched.assign(KA + 1, std::vector<int>(nv));
      L.src.assign(KA + 1, std::vector<int>(nv));
      std::vector<int> ch_a(nv), ch_b(nv), lane_of(seg_ch);
      for (int v = 0; v < nv; ++v) {
        ch_a[v] = 2 * v;
        ch_b[v] = 2 * v + 1;
      }

      for (int tau = 0; tau <= KA; ++tau) {
        for (int v = 0; v < nv; ++v) lane_of[ch_a[v]] = lane_of[ch_b[v]] = v;
        const std::vector<int>& nxt = S.partner[tau + 1];
        std::vector<char> done(nv, 0);
        for (int L0 = 0; L0 < nv; ++L0) {
          if (done[L0]) continue;
          struct Rec { int lane, keep, fetch, from; };
          std::vector<Rec> orient[2];
          double score[2] = {1.0, 1.0};
          for (int o = 0; o < 2; ++o) {
            int lane = L0;
            int keep = o == 0 ? ch_a[L0] : ch_b[L0];
            for (int guard = 0; guard <= nv; ++guard) {
              int fetch = nxt[keep];
              int from = lane_of[fetch];
              orient[o].push_back({lane, keep, fetch, from});
              if (fast && tau >= 1) {
                // stage tau-1 at `lane` had inputs kept[tau-1] (A) and fetched[tau-1] (B)
                int a = L.kept[tau - 1][lane];
                int b = L.fetched[tau - 1][lane];
                double m = (keep == a) ? std::fabs(mu(tau, a, a)) : std::fabs(mu(tau, b, a));
                (void)b;
                score[o] = std::min(score[o], m);
              }
              if (from == L0) break;
              lane = from;
              keep = (ch_a[from] == fetch) ? ch_b[from] : ch_a[from];
            }
          }
          int o = score[1] > score[0] ? 1 : 0;
          if (!kset.empty()) o = kset[tau][ch_a[L0]] ? 0 : 1;
          for (const auto& rc : orient[o]) {
            if (!kset.empty() && !kset[tau][rc.keep]) ok = false;
            L.kept[tau][rc.lane] = rc.keep;
            L.fetched[tau][rc.lane] = rc.fetch;
            L.src[tau][rc.lane] = rc.from;
            done[rc.lane] = 1;
          }
        }
        for (int v = 0; v < nv; ++v) {
          ch_a[v] = L.kept[tau][v];
          ch_b[v] = L.fetched[tau][v];
        }
      }

      // ---- coefficients with deferred per-channel scales -------------------
      std::vector<double> lam(seg_ch);
      for (int ch = 0; ch < seg_ch; ++ch) lam[ch] = 1.0 / (double)alpha[base + ch];
      uint32_t* T = &table[(size_t)sg * lay.words * nv];
      auto put = [&](int field, int v, uint32_t w) { T[((size_t)(field >> 2) * nv + v) * 4 + (field & 3)] = w; };
      auto in_range = [&](double x) { double a = std::fabs(x); return a >= lo && a <= hi; };
      for (int t = 0; t < KA && ok; ++t) {
        const int tt = t + 1;
        std::vector<double> new_lam = lam;
        for (int v = 0; v < nv; ++v) {
          int a = L.kept[t][v], b = L.fetched[t][v];
          int p = L.kept[t + 1][v];
          int q = (p == a) ? b : a;
          double mpa = mu(tt, p, a), mpb = mu(tt, p, b), mqa = mu(tt, q, a), mqb = mu(tt, q, b);
          const int f0 = 3 + 2 * KA + lay.coef * t;
          if (fast) {
            if (std::fabs(mpa) < tiny || std::fabs(mqb) < tiny) { ok = false; break; }
            double lp = mpa * lam[a], lq = mqb * lam[b];
            double k1 = mpb * lam[b] / lp, k2 = mqa * lam[a] / lq;
            if (!in_range(lp) || !in_range(lq) || std::fabs(k1) > hi || std::fabs(k2) > hi) {
              ok = false;
              break;
            }
            new_lam[p] = lp;
            new_lam[q] = lq;
            put(f0 + 0, v, fbits((float)k1));
            put(f0 + 1, v, fbits((float)k2));
          } else {
            put(f0 + 0, v, fbits((float)(mpa * lam[a])));
            put(f0 + 1, v, fbits((float)(mpb * lam[b])));
            put(f0 + 2, v, fbits((float)(mqa * lam[a])));
            put(f0 + 3, v, fbits((float)(mqb * lam[b])));
            new_lam[p] = 1.0;
            new_lam[q] = 1.0;
          }
        }
        lam.swap(new_lam);
      }
      if (!ok) break;

      // ---- load / store / LDS fields -----------------------------------------
      for (int v = 0; v < nv; ++v) {
        put(0, v, L.kept[0][v] == 2 * v ? kSelLoadKeep : kSelLoadSwap);
      }
      for (int tau = 0; tau <= KA; ++tau) {
        std::vector<int> slot = plan_lds_slots(L.src[tau]);
        if (slot.empty()) { ok = false; break; }
        for (int v = 0; v < nv; ++v) {
          put(1 + 2 * tau, v, (uint32_t)slot[v] * 16u);
          put(2 + 2 * tau, v, (uint32_t)slot[L.src[tau][v]] * 16u);
        }
      }
      if (!ok) break;
      const int ff = 3 + 2 * KA + lay.coef * KA;
      for (int v = 0; v < nv; ++v) {
        int kx = L.kept[KA][v], kb = L.fetched[KA][v];
        int q = kx / 2;  // natural pair index the lane stores
        put(ff + 0, v, fbits((float)lam[kx]));
        put(ff + 1, v, fbits((float)lam[kb]));
        put(ff + 2, v, (uint32_t)q * 4u);
        put(ff + 3, v, (kx & 1) == 0 ? kSelStoreX : kSelStoreB);
      }
      // store permutation: virtual lane v ends with the natural pair q(v) =
      // kept / 2; one more exchange of the packed output words moves natural
      // pair w to virtual lane w, so that each store instruction of the
      // activation kernel writes one contiguous 256-byte piece of the row
      // (the kernel takes it for 256-channel segments)
      std::vector<int> src_perm(nv);
      for (int v = 0; v < nv; ++v) src_perm[L.kept[KA][v] / 2] = v;
      std::vector<int> pslot = plan_lds_slots(src_perm);
      if (pslot.empty()) { ok = false; break; }
      uint32_t* Pm = &table[rot_perm_base(segs, lay) + (size_t)sg * nv * 2];
      for (int v = 0; v < nv; ++v) {
        Pm[2 * v] = (uint32_t)pslot[v] * 16u;
        Pm[2 * v + 1] = (uint32_t)pslot[src_perm[v]] * 16u;
      }
    }
    if (ok) {
      P.lay = lay;
      P.table.swap(table);
      return PARO_OK;
    }
  }
  set_error("internal: could not build the rotation schedule");
  return PARO_ERR_HIP;
}

}  // namespace paro

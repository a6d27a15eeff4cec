// schedule.cpp -- lowering of the all-reduce schedules to transfer lists and
// the Check()-style symbolic verifier.
//
// Ring ("Inside NCCL all-reduce", section "The ring, exactly as the kernel
// runs it"): the buffer is cut into p chunks; in the reduce-scatter half
// each rank receives a chunk from its predecessor, adds its own
// contribution and passes the running total on, p-1 times; the all-gather
// half forwards the finished chunks p-1 more times.  The send rule
// "at reduce-scatter step s rank r sends chunk (r-1-s) mod p to rank r+1;
// at all-gather step s it forwards chunk (r-s) mod p" reproduces the page's
// 3-GPU table cell by cell and leaves rank r owning chunk r.
//
// All-pairs ("MSCCL, in depth ...", section "Writing an algorithm in
// MSCCLang"; "MSCCL++ ...", section "The Collective Algorithm Library",
// 2PA): every rank sends slice j to rank j, which reduces what arrived;
// then each owner sends its reduced slice to every peer.  One-shot (1PA)
// fuses both phases into one transfer per chunk.
//
// Double binary tree ("Inside NCCL all-reduce", section "The double binary
// tree"): the buffer is cut in two halves, each reduced up one of two
// complementary trees and broadcast back down it; the trees link nodes and
// the ranks of a node hang below the node's first rank as a chain.
//
// k-ary recursive exchange ("Demystifying NVSHMEM", Fig. 7, the P2P branch
// of the all-reduce dispatch): log_k(p) rounds; in round j each rank
// combines its value with the k-1 ranks that differ from it only in base-k
// digit j.
//
// 2PH ("MSCCL++ ...", section "The Collective Algorithm Library", item 4):
// a reduce-scatter inside each node, all-pairs across nodes, and an
// all-gather inside each node.  The small-message variant cuts the buffer
// into as many chunks as a node has ranks and all-reduces each chunk
// across nodes; the large-message variant cuts it into p chunks and runs
// reduce-scatter and all-gather across nodes.
//
// The verifier follows the role of Check() in the MSCCL compiler ("MSCCL,
// in depth ...", section "Architecture: language, compiler, IR, runtime"):
// it runs the schedule symbolically, carrying each slot's contributor set
// and its fold expression, and proves that the declared collective comes
// out in the algorithm's fold order.
#include "schedule.h"

#include <algorithm>
#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>
#include <utility>

#include "simar.h"

namespace simar {

static int mod(int a, int p) { return ((a % p) + p) % p; }
static int lowbit(int x) { return x & -x; }
static uint32_t bit(int r) { return 1u << r; }

static bool uses_group(int algo) {
  return algo == SIM_ALGO_TREE || algo == SIM_ALGO_HIER || algo == SIM_ALGO_HIER_LARGE;
}

// ---------------------------------------------------------------------------
// Trees.
// ---------------------------------------------------------------------------
static int bt_parent(int n, int x) {
  if (x <= 0 || x >= n) return -1;
  const int b = lowbit(x);
  const int up = (x & ~b) | (b << 1);
  return up < n ? up : (x & ~b);
}

static int bt_children(int n, int x, int out[2]) {
  int k = 0;
  if (x < 0 || x >= n) return 0;
  if (x == 0) {
    if (n > 1) {
      int c = 1;
      while (2 * c < n) c *= 2;
      out[k++] = c;
    }
    return k;
  }
  const int h = lowbit(x) >> 1;
  if (h == 0) return 0;  // odd node: a leaf
  out[k++] = x - h;
  for (int d = h; d > 0; d >>= 1)
    if (x + d < n) {
      out[k++] = x + d;
      break;
    }
  return k;
}

int tree_parent(int which, int n, int x) {
  if (n < 1 || x < 0 || x >= n) return -1;
  if (which == 0) return bt_parent(n, x);
  if (n % 2 == 0) {
    const int q = bt_parent(n, n - 1 - x);
    return q < 0 ? -1 : n - 1 - q;
  }
  const int q = bt_parent(n, mod(x - 1, n));
  return q < 0 ? -1 : mod(q + 1, n);
}

int tree_children(int which, int n, int x, int out[2]) {
  if (n < 1 || x < 0 || x >= n) return 0;
  if (which == 0) return bt_children(n, x, out);
  int c[2];
  int k;
  if (n % 2 == 0) {
    k = bt_children(n, n - 1 - x, c);
    for (int i = 0; i < k; i++) c[i] = n - 1 - c[i];
  } else {
    k = bt_children(n, mod(x - 1, n), c);
    for (int i = 0; i < k; i++) c[i] = mod(c[i] + 1, n);
  }
  if (k == 2 && c[1] < c[0]) std::swap(c[0], c[1]);
  for (int i = 0; i < k; i++) out[i] = c[i];
  return k;
}

int rank_tree_parent(int which, int p, int G, int r) {
  if (G < 1 || p % G != 0 || r < 0 || r >= p) return -1;
  if (r % G != 0) return r - 1;
  const int up = tree_parent(which, p / G, r / G);
  return up < 0 ? -1 : up * G;
}

int rank_tree_children(int which, int p, int G, int r, int out[3]) {
  if (G < 1 || p % G != 0 || r < 0 || r >= p) return 0;
  int k = 0;
  if (r % G + 1 < G) out[k++] = r + 1;  // next rank of the chain
  if (r % G == 0) {
    int c[2];
    const int m = tree_children(which, p / G, r / G, c);
    for (int i = 0; i < m; i++) out[k++] = c[i] * G;
  }
  for (int i = 1; i < k; i++)  // ascending
    for (int j = i; j > 0 && out[j] < out[j - 1]; j--) std::swap(out[j], out[j - 1]);
  return k;
}

static int rank_tree_root(int which, int p, int G) {
  for (int r = 0; r < p; r++)
    if (rank_tree_parent(which, p, G, r) < 0) return r;
  return -1;
}

// Height of r in the rank tree: 0 for a leaf, else 1 + its children's maximum.
static int rank_tree_height(int which, int p, int G, int r, int depth = 0) {
  if (depth > p) return -1;  // not a tree
  int c[3];
  const int k = rank_tree_children(which, p, G, r, c);
  int h = 0;
  for (int i = 0; i < k; i++) {
    const int hc = rank_tree_height(which, p, G, c[i], depth + 1);
    if (hc < 0) return -1;
    h = std::max(h, hc + 1);
  }
  return h;
}

static uint32_t children_mask(int which, int p, int G, int r) {
  int c[3];
  const int k = rank_tree_children(which, p, G, r, c);
  uint32_t m = 0;
  for (int i = 0; i < k; i++) m |= bit(c[i]);
  return m;
}

static bool is_power_of(int p, int k) {
  if (k < 2) return false;
  int v = 1;
  while (v < p) v *= k;
  return v == p;
}

// ---------------------------------------------------------------------------
// Lowering.
// ---------------------------------------------------------------------------
static void ring_rs_steps(int p, Schedule* s) {
  for (int st = 0; st <= p - 2; st++) {
    std::vector<Xfer> v;
    for (int r = 0; r < p; r++)
      v.push_back({st == p - 2 ? XK_REDUCE_POST : XK_REDUCE, r, mod(r + 1, p), mod(r - 1 - st, p)});
    s->steps.push_back(v);
  }
}

static bool lower_tree(int p, int G, Schedule* s) {
  s->nchunks = 2;  // chunk t travels up and down tree t
  int H = -1;
  std::vector<int> h[2];
  for (int t = 0; t < 2; t++) {
    h[t].resize(p);
    for (int r = 0; r < p; r++) h[t][r] = rank_tree_height(t, p, G, r);
    const int root = rank_tree_root(t, p, G);
    if (root < 0 || h[t][root] < 1) return false;
    if (H >= 0 && h[t][root] != H) return false;
    H = h[t][root];
  }
  for (int lvl = 1; lvl <= H; lvl++) {  // up: a rank folds its children once all are complete
    std::vector<Xfer> v;
    for (int t = 0; t < 2; t++)
      for (int r = 0; r < p; r++)
        if (h[t][r] == lvl) {
          const bool root = rank_tree_parent(t, p, G, r) < 0;
          v.push_back({root ? XK_GATHER_POST : XK_GATHER, -1, r, t, children_mask(t, p, G, r)});
        }
    s->steps.push_back(v);
  }
  for (int lvl = H; lvl >= 1; lvl--) {  // down: the finished half goes to the children
    std::vector<Xfer> v;
    for (int t = 0; t < 2; t++)
      for (int r = 0; r < p; r++)
        if (h[t][r] == lvl) v.push_back({XK_MCAST, r, -1, t, children_mask(t, p, G, r)});
    s->steps.push_back(v);
  }
  s->rounds = 2 * H;
  return true;
}

static bool lower_rexch(int p, int k, Schedule* s) {
  if (!is_power_of(p, k)) return false;
  s->nchunks = 1;
  int m = 0;
  for (int stride = 1; stride < p; stride *= k) m++;
  int stride = 1;
  for (int j = 0; j < m; j++, stride *= k) {
    std::vector<Xfer> v;
    for (int r = 0; r < p; r++) {
      const int base = r - ((r / stride) % k) * stride;
      uint32_t mask = 0;
      for (int t = 0; t < k; t++) mask |= bit(base + t * stride);
      v.push_back({j == m - 1 ? XK_EXCH_POST : XK_EXCH, -1, r, 0, mask});
    }
    s->steps.push_back(v);
  }
  s->rounds = m;
  return true;
}

static uint32_t node_mask(int G, int node) { return (G == 32 ? 0xffffffffu : (bit(G) - 1u)) << (node * G); }

static bool lower_hier(int p, int G, bool large, Schedule* s) {
  const int nN = p / G;
  s->nchunks = large ? p : G;
  // chunks rank r = (k, i) is responsible for in the node-local phases
  auto local_chunks = [&](int r) {
    std::vector<int> cs;
    if (!large) {
      cs.push_back(r % G);
    } else {
      for (int k2 = 0; k2 < nN; k2++) cs.push_back(k2 * G + r % G);
    }
    return cs;
  };
  auto peers = [&](int r) {  // same position in every other node
    uint32_t m = 0;
    for (int k2 = 0; k2 < nN; k2++)
      if (k2 != r / G) m |= bit(k2 * G + r % G);
    return m;
  };
  if (G > 1) {  // node-local reduce-scatter
    std::vector<Xfer> v;
    for (int r = 0; r < p; r++)
      for (int c : local_chunks(r))
        v.push_back({nN == 1 ? XK_GATHER_POST : XK_GATHER, -1, r, c, node_mask(G, r / G) & ~bit(r)});
    s->steps.push_back(v);
  }
  if (nN > 1) {
    std::vector<Xfer> v;
    if (!large) {  // all-pairs all-reduce of chunk i across the nodes
      for (int r = 0; r < p; r++) v.push_back({XK_EXCH_POST, -1, r, r % G, peers(r) | bit(r)});
      s->steps.push_back(v);
    } else {  // all-pairs reduce-scatter, then all-gather, across the nodes
      for (int r = 0; r < p; r++) v.push_back({XK_GATHER_POST, -1, r, r, peers(r)});
      s->steps.push_back(v);
      v.clear();
      for (int r = 0; r < p; r++) v.push_back({XK_MCAST, r, -1, r, peers(r)});
      s->steps.push_back(v);
    }
  }
  if (G > 1) {  // node-local all-gather
    std::vector<Xfer> v;
    for (int r = 0; r < p; r++)
      for (int c : local_chunks(r)) v.push_back({XK_MCAST, r, -1, c, node_mask(G, r / G) & ~bit(r)});
    s->steps.push_back(v);
  }
  s->rounds = (int)s->steps.size();
  return true;
}

bool lower(int coll, int algo, int p, const Topology& topo, Schedule* out) {
  if (p < 2 || p > SIM_MAX_RANKS || !out) return false;
  Schedule s;
  s.algo = algo;
  s.p = p;
  s.coll = coll;
  s.nchunks = p;
  if (uses_group(algo)) {
    if (topo.ranks_per_node < 1 || p % topo.ranks_per_node != 0) return false;
    s.topo.ranks_per_node = topo.ranks_per_node;
  }
  if (algo == SIM_ALGO_REXCH) {
    if (topo.radix < 2 || topo.radix > p) return false;
    s.topo.radix = topo.radix;
  }
  const int G = s.topo.ranks_per_node;
  // the single-launch ring executes the same schedule as the ring
  const bool ring = (algo == SIM_ALGO_RING || algo == SIM_ALGO_RING_FIFO);
  // the single-launch all-pairs executes the same two steps as the all-pairs
  const bool allpairs = (algo == SIM_ALGO_ALLPAIRS || algo == SIM_ALGO_ALLPAIRS_PERSISTENT);
  const bool fused = (algo == SIM_ALGO_ONESHOT || algo == SIM_ALGO_ONESHOT_LL);
  if (coll == COLL_ALLREDUCE) {
    if (ring) {
      ring_rs_steps(p, &s);
      for (int st = 0; st <= p - 2; st++) {
        std::vector<Xfer> v;
        for (int r = 0; r < p; r++) v.push_back({XK_COPY, r, mod(r + 1, p), mod(r - st, p)});
        s.steps.push_back(v);
      }
      s.rounds = 2 * (p - 1);
    } else if (allpairs) {
      std::vector<Xfer> a, b;
      for (int j = 0; j < p; j++) a.push_back({XK_GATHER_REDUCE, -1, j, j});
      for (int j = 0; j < p; j++) b.push_back({XK_FANOUT, j, -1, j});
      s.steps.push_back(a);
      s.steps.push_back(b);
      s.rounds = 2;
    } else if (fused) {
      std::vector<Xfer> a;
      for (int j = 0; j < p; j++) a.push_back({XK_ONESHOT, -1, -1, j});
      s.steps.push_back(a);
      s.rounds = 2;
    } else if (algo == SIM_ALGO_TREE) {
      if (!lower_tree(p, G, &s)) return false;
    } else if (algo == SIM_ALGO_REXCH) {
      if (!lower_rexch(p, s.topo.radix, &s)) return false;
    } else if (algo == SIM_ALGO_HIER || algo == SIM_ALGO_HIER_LARGE) {
      if (!lower_hier(p, G, algo == SIM_ALGO_HIER_LARGE, &s)) return false;
    } else {
      return false;
    }
  } else if (coll == COLL_REDUCE_SCATTER) {
    if (ring) {
      ring_rs_steps(p, &s);
      s.rounds = p - 1;
    } else if (algo == SIM_ALGO_ALLPAIRS) {
      std::vector<Xfer> a;
      for (int j = 0; j < p; j++) a.push_back({XK_GATHER_REDUCE, -1, j, j});
      s.steps.push_back(a);
      s.rounds = 1;
    } else {
      return false;
    }
  } else if (coll == COLL_ALL_GATHER) {
    if (ring) {
      // step 0 also places each rank's own block (src == dst)
      for (int st = 0; st <= p - 2; st++) {
        std::vector<Xfer> v;
        if (st == 0)
          for (int r = 0; r < p; r++) v.push_back({XK_COPY, r, r, r});
        for (int r = 0; r < p; r++) v.push_back({XK_COPY, r, mod(r + 1, p), mod(r - st, p)});
        s.steps.push_back(v);
      }
      s.rounds = p - 1;
    } else if (algo == SIM_ALGO_ALLPAIRS) {
      std::vector<Xfer> a;
      for (int j = 0; j < p; j++) a.push_back({XK_FANOUT, j, -1, j});
      s.steps.push_back(a);
      s.rounds = 1;
    } else {
      return false;
    }
  } else {
    return false;
  }
  *out = s;
  return true;
}

// ---------------------------------------------------------------------------
// Expected fold expressions, from each algorithm's definition.
// ---------------------------------------------------------------------------
static std::string fold_exprs(const std::vector<std::string>& xs) {
  if (xs.empty()) return "";
  std::string acc = xs[0];
  for (size_t i = 1; i < xs.size(); i++) acc = "(" + acc + "+" + xs[i] + ")";
  return acc;
}

static std::string rank_str(int r) { return std::to_string(r); }

static std::string tree_expr(int which, int p, int G, int r, int depth) {
  std::vector<std::string> xs{rank_str(r)};
  if (depth > p) return "?";
  int c[3];
  const int k = rank_tree_children(which, p, G, r, c);
  for (int i = 0; i < k; i++) xs.push_back(tree_expr(which, p, G, c[i], depth + 1));
  return fold_exprs(xs);
}

// node k's partial of a chunk handled by local position i: that rank's own
// element first, then the node's other ranks ascending
static std::string node_partial(int G, int k, int i) {
  std::vector<std::string> xs{rank_str(k * G + i)};
  for (int j = 0; j < G; j++)
    if (j != i) xs.push_back(rank_str(k * G + j));
  return fold_exprs(xs);
}

std::string expected_expr(const Schedule& s, int c) {
  const int p = s.p;
  const int G = s.topo.ranks_per_node;
  std::vector<std::string> xs;
  switch (s.algo) {
    case SIM_ALGO_RING:
    case SIM_ALGO_RING_FIFO:  // chunk c folds ranks c+1, ..., c+p
      for (int k = 1; k <= p; k++) xs.push_back(rank_str(mod(c + k, p)));
      return fold_exprs(xs);
    case SIM_ALGO_ALLPAIRS:
    case SIM_ALGO_ALLPAIRS_PERSISTENT:
    case SIM_ALGO_ONESHOT:
    case SIM_ALGO_ONESHOT_LL:  // owner first, then the others ascending
      xs.push_back(rank_str(c));
      for (int q = 0; q < p; q++)
        if (q != c) xs.push_back(rank_str(q));
      return fold_exprs(xs);
    case SIM_ALGO_TREE: {  // the root's subtree total: own value, then children ascending
      const int root = rank_tree_root(c, p, G);
      return root < 0 ? "?" : tree_expr(c, p, G, root, 0);
    }
    case SIM_ALGO_REXCH: {  // round j: fold of the group that differs in digit j
      const int k = s.topo.radix;
      std::vector<std::string> v(p);
      for (int r = 0; r < p; r++) v[r] = rank_str(r);
      for (int stride = 1; stride < p; stride *= k) {
        std::vector<std::string> nv(p);
        for (int r = 0; r < p; r++) {
          const int base = r - ((r / stride) % k) * stride;
          std::vector<std::string> g;
          for (int t = 0; t < k; t++) g.push_back(v[base + t * stride]);
          nv[r] = fold_exprs(g);
        }
        v = nv;
      }
      return v[0];
    }
    case SIM_ALGO_HIER: {  // node partials of chunk c, nodes ascending
      for (int k = 0; k < p / G; k++) xs.push_back(node_partial(G, k, c));
      return fold_exprs(xs);
    }
    case SIM_ALGO_HIER_LARGE: {  // the owner's node partial first, then the other nodes ascending
      const int k0 = c / G, i = c % G;
      xs.push_back(node_partial(G, k0, i));
      for (int k = 0; k < p / G; k++)
        if (k != k0) xs.push_back(node_partial(G, k, i));
      return fold_exprs(xs);
    }
  }
  return "?";
}

// ---------------------------------------------------------------------------
// Symbolic execution.
// ---------------------------------------------------------------------------
namespace {

struct Held {
  uint32_t mask = 0;  // contributors
  std::string expr;   // fold expression
  bool set = false;   // slot holds a value at all
  bool fin = false;   // value was completed by a post-processing step
};

struct Sym {
  int nchunks;
  std::vector<Held> h;  // [r * nchunks + c]
  Held& at(int r, int c) { return h[(size_t)r * nchunks + c]; }
  const Held& at(int r, int c) const { return h[(size_t)r * nchunks + c]; }
};

std::string fmt(const char* f, int a = 0, int b = 0, int c = 0, int d = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

Sym initial(const Schedule& s) {
  Sym y;
  y.nchunks = s.nchunks;
  y.h.resize((size_t)s.p * s.nchunks);
  for (int r = 0; r < s.p; r++)
    for (int c = 0; c < s.nchunks; c++) {
      Held& x = y.at(r, c);
      if (s.coll == COLL_ALL_GATHER && c != r) continue;  // only the own block exists
      x.mask = bit(r);
      x.expr = rank_str(r);
      x.set = true;
    }
  return y;
}

bool combine(const Held& acc, const Held& in, Held* out, std::string* err) {
  if (!acc.set || !in.set) {
    *err = "reads an empty slot";
    return false;
  }
  if (acc.fin || in.fin) {
    *err = "folds a value that was already post-processed";
    return false;
  }
  if (acc.mask & in.mask) {
    *err = "a contribution would be counted twice";
    return false;
  }
  out->mask = acc.mask | in.mask;
  out->expr = "(" + acc.expr + "+" + in.expr + ")";
  out->set = true;
  out->fin = false;
  return true;
}

typedef std::pair<int, int> Slot;

void rw_sets(const Xfer& x, int p, std::vector<Slot>* rd, std::vector<Slot>* wr) {
  switch (x.kind) {
    case XK_REDUCE:
    case XK_REDUCE_POST:
      rd->push_back({x.src, x.chunk});
      rd->push_back({x.dst, x.chunk});
      wr->push_back({x.dst, x.chunk});
      break;
    case XK_COPY:
      rd->push_back({x.src, x.chunk});
      if (x.src != x.dst) wr->push_back({x.dst, x.chunk});
      break;
    case XK_GATHER_REDUCE:
      for (int q = 0; q < p; q++) rd->push_back({q, x.chunk});
      wr->push_back({x.dst, x.chunk});
      break;
    case XK_FANOUT:
      rd->push_back({x.src, x.chunk});
      for (int r = 0; r < p; r++)
        if (r != x.src) wr->push_back({r, x.chunk});
      break;
    case XK_ONESHOT:
      for (int q = 0; q < p; q++) {
        rd->push_back({q, x.chunk});
        wr->push_back({q, x.chunk});
      }
      break;
    case XK_GATHER:
    case XK_GATHER_POST:
      rd->push_back({x.dst, x.chunk});
      for (int q = 0; q < p; q++)
        if (x.mask & bit(q)) rd->push_back({q, x.chunk});
      wr->push_back({x.dst, x.chunk});
      break;
    case XK_EXCH:
    case XK_EXCH_POST:
      for (int q = 0; q < p; q++)
        if (x.mask & bit(q)) rd->push_back({q, x.chunk});
      wr->push_back({x.dst, x.chunk});
      break;
    case XK_MCAST:
      rd->push_back({x.src, x.chunk});
      for (int q = 0; q < p; q++)
        if (x.mask & bit(q)) wr->push_back({q, x.chunk});
      break;
  }
}

bool valid_xfer(const Xfer& x, int p, int nchunks) {
  if (x.chunk < 0 || x.chunk >= nchunks) return false;
  auto rank_ok = [p](int r) { return r >= 0 && r < p; };
  const uint32_t full = (p == 32) ? 0xffffffffu : (bit(p) - 1u);
  if (x.mask & ~full) return false;
  switch (x.kind) {
    case XK_REDUCE: case XK_REDUCE_POST: return rank_ok(x.src) && rank_ok(x.dst) && x.src != x.dst;
    case XK_COPY: return rank_ok(x.src) && rank_ok(x.dst);
    case XK_GATHER_REDUCE: return rank_ok(x.dst);
    case XK_FANOUT: return rank_ok(x.src);
    case XK_ONESHOT: return true;
    case XK_GATHER: case XK_GATHER_POST:
      return rank_ok(x.dst) && x.mask != 0 && !(x.mask & bit(x.dst));
    case XK_EXCH: case XK_EXCH_POST: return rank_ok(x.dst) && (x.mask & bit(x.dst));
    case XK_MCAST: return rank_ok(x.src) && x.mask != 0 && !(x.mask & bit(x.src));
  }
  return false;
}

bool is_exch(int kind) { return kind == XK_EXCH || kind == XK_EXCH_POST; }

// Applies one step.
bool apply_step(const Schedule& s, int st, Sym* y, std::string* err) {
  const int p = s.p;
  const auto& xs = s.steps[st];
  // hazard check: no transfer may touch a slot another transfer writes --
  // except the members of one exchange group (same kind, chunk and set),
  // which read each other's pre-step values and all end with the one value
  // they fold (an executor computes that value once for the whole group)
  std::map<Slot, int> writer;
  for (size_t k = 0; k < xs.size(); k++) {
    if (!valid_xfer(xs[k], p, s.nchunks)) {
      *err = fmt("step %d: transfer %d has an out-of-range rank, chunk or rank set", st, (int)k);
      return false;
    }
    std::vector<Slot> rd, wr;
    rw_sets(xs[k], p, &rd, &wr);
    for (auto& w : wr) {
      if (writer.count(w)) {
        *err = fmt("step %d: rank %d chunk %d is written by two transfers", st, w.first, w.second);
        return false;
      }
      writer[w] = (int)k;
    }
  }
  for (size_t k = 0; k < xs.size(); k++) {
    std::vector<Slot> rd, wr;
    rw_sets(xs[k], p, &rd, &wr);
    for (auto& r : rd) {
      auto it = writer.find(r);
      if (it == writer.end() || it->second == (int)k) continue;
      const Xfer& a = xs[k];
      const Xfer& b = xs[it->second];
      if (is_exch(a.kind) && a.kind == b.kind && a.chunk == b.chunk && a.mask == b.mask) continue;
      *err = fmt("step %d: rank %d chunk %d is read by one transfer and written by another", st,
                 r.first, r.second);
      return false;
    }
  }
  // hazard-free, so evaluating against the pre-step snapshot is exact
  const Sym before = *y;
  auto B = [&](int r, int c) -> const Held& { return before.at(r, c); };
  for (const Xfer& x : xs) {
    std::string e;
    switch (x.kind) {
      case XK_REDUCE:
      case XK_REDUCE_POST: {
        Held out;
        if (!combine(B(x.src, x.chunk), B(x.dst, x.chunk), &out, &e)) {
          *err = fmt("step %d: reduce of chunk %d from rank %d into rank %d: ", st, x.chunk, x.src, x.dst) + e;
          return false;
        }
        out.fin = (x.kind == XK_REDUCE_POST);
        y->at(x.dst, x.chunk) = out;
        break;
      }
      case XK_COPY:
        if (!B(x.src, x.chunk).set) {
          *err = fmt("step %d: copy of chunk %d from rank %d reads an empty slot", st, x.chunk, x.src);
          return false;
        }
        y->at(x.dst, x.chunk) = B(x.src, x.chunk);
        break;
      case XK_GATHER_REDUCE:
      case XK_ONESHOT: {
        const int j = x.chunk;  // owner folds its own element first
        Held acc = B(j, x.chunk);
        for (int q = 0; q < p; q++) {
          if (q == j) continue;
          Held nx;
          if (!combine(acc, B(q, x.chunk), &nx, &e)) {
            *err = fmt("step %d: gather-reduce of chunk %d at rank %d: ", st, x.chunk, q) + e;
            return false;
          }
          acc = nx;
        }
        acc.fin = true;
        if (x.kind == XK_GATHER_REDUCE) {
          y->at(x.dst, x.chunk) = acc;
        } else {
          for (int r = 0; r < p; r++) y->at(r, x.chunk) = acc;
        }
        break;
      }
      case XK_FANOUT:
        if (!B(x.src, x.chunk).set) {
          *err = fmt("step %d: fan-out of chunk %d from rank %d reads an empty slot", st, x.chunk, x.src);
          return false;
        }
        for (int r = 0; r < p; r++)
          if (r != x.src) y->at(r, x.chunk) = B(x.src, x.chunk);
        break;
      case XK_GATHER:
      case XK_GATHER_POST:
      case XK_EXCH:
      case XK_EXCH_POST: {
        const bool gather = (x.kind == XK_GATHER || x.kind == XK_GATHER_POST);
        Held acc;
        bool first = true;
        if (gather) {
          acc = B(x.dst, x.chunk);
          first = false;
          if (!acc.set || acc.fin) {
            *err = fmt("step %d: rank %d's own value of chunk %d is missing or already finished", st,
                       x.dst, x.chunk);
            return false;
          }
        }
        for (int q = 0; q < p; q++) {
          if (!(x.mask & bit(q))) continue;
          if (first) {
            acc = B(q, x.chunk);
            first = false;
            if (!acc.set || acc.fin) {
              *err = fmt("step %d: exchange of chunk %d reads rank %d's missing or finished value", st,
                         x.chunk, q);
              return false;
            }
            continue;
          }
          Held nx;
          if (!combine(acc, B(q, x.chunk), &nx, &e)) {
            *err = fmt("step %d: fold of chunk %d into rank %d, from rank %d: ", st, x.chunk, x.dst, q) + e;
            return false;
          }
          acc = nx;
        }
        acc.fin = (x.kind == XK_GATHER_POST || x.kind == XK_EXCH_POST);
        y->at(x.dst, x.chunk) = acc;
        break;
      }
      case XK_MCAST: {
        const Held& v = B(x.src, x.chunk);
        if (!v.set || !v.fin) {
          *err = fmt("step %d: broadcast of chunk %d from rank %d sends an unfinished value", st, x.chunk,
                     x.src);
          return false;
        }
        for (int q = 0; q < p; q++)
          if (x.mask & bit(q)) y->at(q, x.chunk) = v;
        break;
      }
    }
  }
  return true;
}

int ceil_log2(int v) {
  int l = 0;
  while ((1 << l) < v) l++;
  return l;
}

// Communication rounds in closed form (independent of the lowering).
int closed_form_rounds(const Schedule& s) {
  const int p = s.p;
  const int G = s.topo.ranks_per_node;
  switch (s.algo) {
    case SIM_ALGO_RING:
    case SIM_ALGO_RING_FIFO:
      return s.coll == COLL_ALLREDUCE ? 2 * (p - 1) : p - 1;
    case SIM_ALGO_ALLPAIRS:
    case SIM_ALGO_ALLPAIRS_PERSISTENT:
    case SIM_ALGO_ONESHOT:
    case SIM_ALGO_ONESHOT_LL:
      return s.coll == COLL_ALLREDUCE ? 2 : 1;
    case SIM_ALGO_TREE:  // up and down: the chain inside a node, then log2 of the node count
      return 2 * ((G - 1) + ceil_log2(p / G));
    case SIM_ALGO_REXCH: {
      int m = 0;
      for (int v = 1; v < p; v *= s.topo.radix) m++;
      return m;
    }
    case SIM_ALGO_HIER:
      return 2 * (G > 1 ? 1 : 0) + (p / G > 1 ? 1 : 0);
    case SIM_ALGO_HIER_LARGE:
      return 2 * (G > 1 ? 1 : 0) + 2 * (p / G > 1 ? 1 : 0);
  }
  return -1;
}

}  // namespace

bool symbolic_state(const Schedule& s, int after_steps, uint32_t* masks, std::string* diag) {
  if (after_steps < 0 || after_steps > (int)s.steps.size()) {
    if (diag) *diag = "step index out of range";
    return false;
  }
  Sym y = initial(s);
  std::string err;
  for (int st = 0; st < after_steps; st++)
    if (!apply_step(s, st, &y, &err)) {
      if (diag) *diag = err;
      return false;
    }
  for (int r = 0; r < s.p; r++)
    for (int c = 0; c < s.nchunks; c++) masks[(size_t)r * s.nchunks + c] = y.at(r, c).mask;
  return true;
}

bool verify(const Schedule& s, std::string* diag) {
  std::string err;
  const int p = s.p;
  if (p < 2 || p > SIM_MAX_RANKS) {
    if (diag) *diag = "p out of range";
    return false;
  }
  if (s.nchunks < 1 || s.nchunks > p || (s.coll != COLL_ALLREDUCE && s.nchunks != p)) {
    if (diag) *diag = "chunk count out of range";
    return false;
  }
  Sym y = initial(s);
  for (int st = 0; st < (int)s.steps.size(); st++)
    if (!apply_step(s, st, &y, &err)) {
      if (diag) *diag = err;
      return false;
    }
  const uint32_t full = (p == 32) ? 0xffffffffu : (bit(p) - 1u);
  for (int c = 0; c < s.nchunks; c++) {
    const std::string want = (s.coll == COLL_ALL_GATHER) ? "" : expected_expr(s, c);
    for (int r = 0; r < p; r++) {
      const Held& h = y.at(r, c);
      if (s.coll == COLL_ALL_GATHER) {
        if (h.mask != bit(c)) {
          if (diag) *diag = fmt("rank %d block %d does not hold exactly rank %d's block", r, c, c);
          return false;
        }
        continue;
      }
      if (s.coll == COLL_REDUCE_SCATTER && c != r) continue;  // only the owned chunk is output
      if (h.mask != full) {
        if (diag) *diag = fmt("rank %d chunk %d misses contributions (mask 0x%x)", r, c, (int)h.mask);
        return false;
      }
      if (!h.fin) {
        if (diag) *diag = fmt("rank %d chunk %d was never finished by a post-op step", r, c);
        return false;
      }
      if (h.expr != want) {
        if (diag)
          *diag = fmt("rank %d chunk %d folds its contributions in another order: ", r, c) + h.expr +
                  " instead of " + want;
        return false;
      }
    }
  }
  const int want = closed_form_rounds(s);
  if (s.rounds != want) {
    if (diag) *diag = fmt("schedule claims %d rounds, closed form is %d", s.rounds, want);
    return false;
  }
  const bool one_step_per_round = !(s.algo == SIM_ALGO_ONESHOT || s.algo == SIM_ALGO_ONESHOT_LL ||
                                    s.algo == SIM_ALGO_ALLPAIRS || s.algo == SIM_ALGO_ALLPAIRS_PERSISTENT);
  if (one_step_per_round && (int)s.steps.size() != want) {
    if (diag) *diag = fmt("schedule has %d steps, closed form is %d", (int)s.steps.size(), want);
    return false;
  }
  if (diag) diag->clear();
  return true;
}

const Schedule* cached_schedule(int coll, int algo, int p, const Topology& topo, std::string* diag) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int, int, int>, Schedule> cache;
  const int G = uses_group(algo) ? topo.ranks_per_node : 1;
  const int k = (algo == SIM_ALGO_REXCH) ? topo.radix : 2;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(coll, algo, p, G, k);
  auto it = cache.find(key);
  if (it != cache.end()) return &it->second;
  Schedule s;
  if (!lower(coll, algo, p, topo, &s)) {
    if (diag) *diag = "no lowering for this (collective, algo, p, topology)";
    return nullptr;
  }
  if (!verify(s, diag)) return nullptr;
  return &(cache[key] = s);
}

}  // namespace simar

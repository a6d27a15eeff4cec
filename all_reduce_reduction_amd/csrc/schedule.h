// schedule.h -- lowering of collective algorithms to per-step transfer lists,
// and the symbolic verifier that proves a lowered schedule computes its
// collective.  Host-only C++17; no device code.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

namespace simar {

enum Coll { COLL_ALLREDUCE = 0, COLL_REDUCE_SCATTER = 1, COLL_ALL_GATHER = 2 };

// Step vocabulary, after the fused primitives of NCCL's runRing
// ("Inside NCCL all-reduce", section "The ring, exactly as the kernel runs
// it") and the step kinds of the MSCCL XML IR ("MSCCL, in depth ...",
// section "The XML IR"):
//   REDUCE        dst's slot for `chunk` = src's running value (+) dst's own
//                 element (recvReduceSend)
//   REDUCE_POST   the same, on the step where the chunk completes: the
//                 result is post-processed into dst's output
//                 (recvReduceCopySend with postOp)
//   COPY          dst's slot for `chunk` = src's slot (recvCopySend)
//   GATHER_REDUCE owner `dst` folds `chunk` over every rank: own element
//                 first, then the others ascending (all-pairs step 1)
//   FANOUT        owner `src` sends its finished `chunk` to every other
//                 rank (all-pairs step 2)
//   ONESHOT       GATHER_REDUCE + FANOUT of `chunk` fused in one transfer
// Tree, recursive-exchange and hierarchical steps carry a rank set `mask`
// (bit q = rank q); sets are always folded in ascending rank order:
//   GATHER        dst's running value for `chunk` folds in the values of
//                 the ranks in `mask`, ascending (a tree parent taking its
//                 children's subtotals; a node-local reduce-scatter owner
//                 taking its node's elements); values as before the step
//   GATHER_POST   the same, completing the value (post-processed output)
//   EXCH          dst's value becomes the fold of the values of the ranks
//                 in `mask` (which contains dst), ascending, all as they
//                 were before the step: every member of one group ends
//                 with the same value (recursive exchange, cross-node
//                 all-pairs); _POST completes the value
//   MCAST         src's value for `chunk` is copied to every rank in
//                 `mask` (tree broadcast, node-local all-gather)
enum XferKind {
  XK_REDUCE = 0,
  XK_REDUCE_POST = 1,
  XK_COPY = 2,
  XK_GATHER_REDUCE = 3,
  XK_FANOUT = 4,
  XK_ONESHOT = 5,
  XK_GATHER = 6,
  XK_GATHER_POST = 7,
  XK_EXCH = 8,
  XK_EXCH_POST = 9,
  XK_MCAST = 10,
};
constexpr int kNumXferKinds = 11;

struct Xfer {
  int kind;
  int src;    // -1: every rank (GATHER_REDUCE, ONESHOT) / unused (GATHER, EXCH)
  int dst;    // -1: every other rank (FANOUT) / every rank (ONESHOT) / unused (MCAST)
  int chunk;
  uint32_t mask = 0;  // rank set of GATHER, EXCH, MCAST
};

struct Topology {
  int ranks_per_node = 1;  // G: consecutive ranks kG .. kG+G-1 form node k
  int radix = 2;           // k of the k-ary recursive exchange
};

struct Schedule {
  int algo = 0;
  int p = 0;
  int coll = COLL_ALLREDUCE;
  int nchunks = 0;  // the buffer is cut into nchunks chunks, floor(c*n/nchunks)
  Topology topo;
  int rounds = 0;   // communication rounds (closed form of the algorithm)
  std::vector<std::vector<Xfer>> steps;  // one entry per lowered step
  int nxfers() const {
    int n = 0;
    for (auto& s : steps) n += (int)s.size();
    return n;
  }
};

// NCCL's binary tree over n nodes ("Inside NCCL all-reduce", section "The
// double binary tree"): a node's lowest set bit b fixes its height; its
// parent clears b and sets the next bit up, or only clears b when that
// leaves the node range; its children are the node minus and plus b/2,
// the plus side halving again until it falls inside the range.  Node 0 is
// the root and its one child is the largest power of two below n.
// which = 0: that tree; which = 1: the second tree of the double tree --
// node x plays node n-1-x of the first tree (mirror) for even n, node x-1
// (shifted by one) for odd n.  Parent -1 for the root; children ascending.
int tree_parent(int which, int n, int x);
int tree_children(int which, int n, int x, int out[2]);

// The tree actually run over p ranks with G ranks per node: node k's first
// rank kG takes the node's place in the tree over the p/G nodes; the other
// ranks of the node hang below it as a chain (kG+i is the parent of
// kG+i+1).  Children (at most three) are returned ascending.
int rank_tree_parent(int which, int p, int G, int r);
int rank_tree_children(int which, int p, int G, int r, int out[3]);

// Lowering.  Returns false for an unknown (coll, algo) pair, p < 2, or a
// topology the algo cannot use (G must divide p; the recursive exchange
// needs p to be a power of the radix).
bool lower(int coll, int algo, int p, const Topology& t, Schedule* out);

// The fold chunk c must end with, as an expression over rank numbers:
// "(a+b)" combines a then b.  Derived from each algorithm's definition,
// independently of its lowering.
std::string expected_expr(const Schedule& s, int c);

// Check(): symbolic run with contributor masks and fold expressions.
// Returns true when the schedule is proven; otherwise false with a message.
bool verify(const Schedule& s, std::string* diag);

// Contributor masks after `after_steps` steps, masks[r*nchunks + c].
bool symbolic_state(const Schedule& s, int after_steps, uint32_t* masks, std::string* diag);

// Cached, verified schedules (lowered and checked once per key).
const Schedule* cached_schedule(int coll, int algo, int p, const Topology& t, std::string* diag);

}  // namespace simar

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
enum XferKind {
  XK_REDUCE = 0,
  XK_REDUCE_POST = 1,
  XK_COPY = 2,
  XK_GATHER_REDUCE = 3,
  XK_FANOUT = 4,
  XK_ONESHOT = 5,
};

struct Xfer {
  int kind;
  int src;    // -1: every rank (GATHER_REDUCE, ONESHOT)
  int dst;    // -1: every other rank (FANOUT) / every rank (ONESHOT)
  int chunk;
};

struct Schedule {
  int algo = 0;
  int p = 0;
  int coll = COLL_ALLREDUCE;
  int rounds = 0;  // communication rounds: every rank sends once per round
  std::vector<std::vector<Xfer>> steps;  // one entry per lowered step (launch)
  int nxfers() const {
    int n = 0;
    for (auto& s : steps) n += (int)s.size();
    return n;
  }
};

// Lowering.  Returns false for an unknown (coll, algo) pair or p < 2.
bool lower(int coll, int algo, int p, Schedule* out);

// The fold order chunk c must follow under `algo`.
std::vector<int> expected_order(int algo, int p, int c);

// Check(): symbolic run with contributor masks and fold-order traces.
// Returns true when the schedule is proven; otherwise false with a message.
bool verify(const Schedule& s, std::string* diag);

// Contributor masks after `after_steps` steps, masks[r*p + c].
bool symbolic_state(const Schedule& s, int after_steps, uint32_t* masks, std::string* diag);

// Cached, verified schedules (lowered and checked once per (coll, algo, p)).
const Schedule* cached_schedule(int coll, int algo, int p, std::string* diag);

}  // namespace simar

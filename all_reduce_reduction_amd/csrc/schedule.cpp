// schedule.cpp -- lowering ring / all-pairs / one-shot to transfer lists and
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
// The verifier follows the role of Check() in the MSCCL compiler (same
// page, section "Architecture: language, compiler, IR, runtime"): it runs
// the schedule symbolically and proves that the declared collective comes
// out.
#include "schedule.h"

#include <cstdio>
#include <map>
#include <mutex>
#include <tuple>

#include "simar.h"

namespace simar {

static int mod(int a, int p) { return ((a % p) + p) % p; }

bool lower(int coll, int algo, int p, Schedule* out) {
  if (p < 2 || p > SIM_MAX_RANKS || !out) return false;
  Schedule s;
  s.algo = algo;
  s.p = p;
  s.coll = coll;
  // the single-launch ring executes the same schedule as the ring
  const bool ring = (algo == SIM_ALGO_RING || algo == SIM_ALGO_RING_FIFO);
  const bool allpairs = (algo == SIM_ALGO_ALLPAIRS);
  const bool fused = (algo == SIM_ALGO_ONESHOT || algo == SIM_ALGO_ONESHOT_LL);
  if (coll == COLL_ALLREDUCE) {
    if (ring) {
      for (int st = 0; st <= p - 2; st++) {
        std::vector<Xfer> v;
        for (int r = 0; r < p; r++)
          v.push_back({st == p - 2 ? XK_REDUCE_POST : XK_REDUCE, r, mod(r + 1, p), mod(r - 1 - st, p)});
        s.steps.push_back(v);
      }
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
    } else {
      return false;
    }
  } else if (coll == COLL_REDUCE_SCATTER) {
    if (ring) {
      for (int st = 0; st <= p - 2; st++) {
        std::vector<Xfer> v;
        for (int r = 0; r < p; r++)
          v.push_back({st == p - 2 ? XK_REDUCE_POST : XK_REDUCE, r, mod(r + 1, p), mod(r - 1 - st, p)});
        s.steps.push_back(v);
      }
      s.rounds = p - 1;
    } else if (allpairs) {
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
    } else if (allpairs) {
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

std::vector<int> expected_order(int algo, int p, int c) {
  std::vector<int> o;
  if (algo == SIM_ALGO_RING || algo == SIM_ALGO_RING_FIFO) {
    for (int k = 1; k <= p; k++) o.push_back(mod(c + k, p));
  } else {
    o.push_back(c);
    for (int q = 0; q < p; q++)
      if (q != c) o.push_back(q);
  }
  return o;
}

// ---------------------------------------------------------------------------
// Symbolic execution.
// ---------------------------------------------------------------------------
namespace {

struct Held {
  uint32_t mask = 0;        // contributors
  std::vector<int> trace;   // fold order (accumulator first)
  bool set = false;         // slot holds a value at all
};

struct Sym {
  int p;
  std::vector<Held> h;  // [r * p + c]
  Held& at(int r, int c) { return h[(size_t)r * p + c]; }
};

std::string fmt(const char* f, int a = 0, int b = 0, int c = 0, int d = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

Sym initial(const Schedule& s) {
  Sym y;
  y.p = s.p;
  y.h.resize((size_t)s.p * s.p);
  for (int r = 0; r < s.p; r++)
    for (int c = 0; c < s.p; c++) {
      Held& x = y.at(r, c);
      if (s.coll == COLL_ALL_GATHER && c != r) continue;  // only the own block exists
      x.mask = 1u << r;
      x.trace = {r};
      x.set = true;
    }
  return y;
}

bool combine(const Held& acc, const Held& in, Held* out, std::string* err) {
  if (!acc.set || !in.set) {
    *err = "reads an empty slot";
    return false;
  }
  if (acc.mask & in.mask) {
    *err = "a contribution would be counted twice";
    return false;
  }
  out->mask = acc.mask | in.mask;
  out->trace = acc.trace;
  out->trace.insert(out->trace.end(), in.trace.begin(), in.trace.end());
  out->set = true;
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
  }
}

bool valid_xfer(const Xfer& x, int p) {
  if (x.chunk < 0 || x.chunk >= p) return false;
  auto rank_ok = [p](int r) { return r >= 0 && r < p; };
  switch (x.kind) {
    case XK_REDUCE: case XK_REDUCE_POST: return rank_ok(x.src) && rank_ok(x.dst) && x.src != x.dst;
    case XK_COPY: return rank_ok(x.src) && rank_ok(x.dst);
    case XK_GATHER_REDUCE: return rank_ok(x.dst);
    case XK_FANOUT: return rank_ok(x.src);
    case XK_ONESHOT: return true;
  }
  return false;
}

// Applies one step; `post` records which slots were finished by a postOp.
bool apply_step(const Schedule& s, int st, Sym* y, std::vector<char>* post, std::string* err) {
  const int p = s.p;
  const auto& xs = s.steps[st];
  // hazard check: no transfer may touch a slot another transfer writes
  std::map<Slot, int> writer;
  for (size_t k = 0; k < xs.size(); k++) {
    if (!valid_xfer(xs[k], p)) {
      *err = fmt("step %d: transfer %d has an out-of-range rank or chunk", st, (int)k);
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
      if (it != writer.end() && it->second != (int)k) {
        *err = fmt("step %d: rank %d chunk %d is read by one transfer and written by another",
                   st, r.first, r.second);
        return false;
      }
    }
  }
  // hazard-free, so evaluating against the pre-step snapshot is exact
  const Sym before = *y;
  auto B = [&](int r, int c) -> const Held& { return before.h[(size_t)r * p + c]; };
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
        y->at(x.dst, x.chunk) = out;
        if (x.kind == XK_REDUCE_POST) (*post)[(size_t)x.dst * p + x.chunk] = 1;
        break;
      }
      case XK_COPY:
        if (!B(x.src, x.chunk).set) {
          *err = fmt("step %d: copy of chunk %d from rank %d reads an empty slot", st, x.chunk, x.src);
          return false;
        }
        y->at(x.dst, x.chunk) = B(x.src, x.chunk);
        if ((*post)[(size_t)x.src * p + x.chunk]) (*post)[(size_t)x.dst * p + x.chunk] = 1;
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
        if (x.kind == XK_GATHER_REDUCE) {
          y->at(x.dst, x.chunk) = acc;
          (*post)[(size_t)x.dst * p + x.chunk] = 1;
        } else {
          for (int r = 0; r < p; r++) {
            y->at(r, x.chunk) = acc;
            (*post)[(size_t)r * p + x.chunk] = 1;
          }
        }
        break;
      }
      case XK_FANOUT:
        if (!B(x.src, x.chunk).set) {
          *err = fmt("step %d: fan-out of chunk %d from rank %d reads an empty slot", st, x.chunk, x.src);
          return false;
        }
        for (int r = 0; r < p; r++)
          if (r != x.src) {
            y->at(r, x.chunk) = B(x.src, x.chunk);
            (*post)[(size_t)r * p + x.chunk] = (*post)[(size_t)x.src * p + x.chunk];
          }
        break;
    }
  }
  return true;
}

int closed_form_rounds(int coll, int algo, int p) {
  const bool ring = algo == SIM_ALGO_RING || algo == SIM_ALGO_RING_FIFO;
  if (coll == COLL_ALLREDUCE) return ring ? 2 * (p - 1) : 2;
  return ring ? p - 1 : 1;
}

}  // namespace

bool symbolic_state(const Schedule& s, int after_steps, uint32_t* masks, std::string* diag) {
  if (after_steps < 0 || after_steps > (int)s.steps.size()) {
    if (diag) *diag = "step index out of range";
    return false;
  }
  Sym y = initial(s);
  std::vector<char> post((size_t)s.p * s.p, 0);
  std::string err;
  for (int st = 0; st < after_steps; st++)
    if (!apply_step(s, st, &y, &post, &err)) {
      if (diag) *diag = err;
      return false;
    }
  for (int r = 0; r < s.p; r++)
    for (int c = 0; c < s.p; c++) masks[(size_t)r * s.p + c] = y.at(r, c).mask;
  return true;
}

bool verify(const Schedule& s, std::string* diag) {
  std::string err;
  const int p = s.p;
  if (p < 2 || p > SIM_MAX_RANKS) {
    if (diag) *diag = "p out of range";
    return false;
  }
  Sym y = initial(s);
  std::vector<char> post((size_t)p * p, 0);
  for (int st = 0; st < (int)s.steps.size(); st++)
    if (!apply_step(s, st, &y, &post, &err)) {
      if (diag) *diag = err;
      return false;
    }
  const uint32_t full = (p == 32) ? 0xffffffffu : ((1u << p) - 1u);
  for (int r = 0; r < p; r++) {
    for (int c = 0; c < p; c++) {
      const Held& h = y.at(r, c);
      if (s.coll == COLL_ALL_GATHER) {
        if (h.mask != (1u << c)) {
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
      if (!post[(size_t)r * p + c]) {
        if (diag) *diag = fmt("rank %d chunk %d was never finished by a post-op step", r, c);
        return false;
      }
      if (h.trace != expected_order(s.algo, p, c)) {
        if (diag) *diag = fmt("rank %d chunk %d folds its contributions in another order", r, c);
        return false;
      }
    }
  }
  const int want = closed_form_rounds(s.coll, s.algo, p);
  if (s.rounds != want) {
    if (diag) *diag = fmt("schedule claims %d rounds, closed form is %d", s.rounds, want);
    return false;
  }
  if ((s.algo == SIM_ALGO_RING || s.algo == SIM_ALGO_RING_FIFO) && (int)s.steps.size() != want) {
    if (diag) *diag = fmt("ring has %d steps, closed form is %d", (int)s.steps.size(), want);
    return false;
  }
  if (diag) diag->clear();
  return true;
}

const Schedule* cached_schedule(int coll, int algo, int p, std::string* diag) {
  static std::mutex mu;
  static std::map<std::tuple<int, int, int>, Schedule> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto key = std::make_tuple(coll, algo, p);
  auto it = cache.find(key);
  if (it != cache.end()) return &it->second;
  Schedule s;
  if (!lower(coll, algo, p, &s)) {
    if (diag) *diag = "no lowering for this (collective, algo, p)";
    return nullptr;
  }
  if (!verify(s, diag)) return nullptr;
  return &(cache[key] = s);
}

}  // namespace simar

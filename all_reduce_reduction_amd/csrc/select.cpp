// select.cpp -- alpha-beta model and its calibration file.
//
// The model is the one the pages price schedules with: time = latency x
// number of synchronised steps + bytes / bandwidth ("MSCCL, in depth ...",
// section "Why generic collectives leave time on the table"; "Inside NCCL
// all-reduce", section "How NCCL picks: a cost model, not a threshold":
// one line of cost per candidate, argmin per call, no stored threshold).
// On one GPU a "step" is a kernel launch and the bytes are the schedule's
// HBM traffic over all simulated ranks, so alpha and B are fitted to this
// GPU by the calibration sweep and stored as JSON.
#include "select.h"

#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <map>
#include <memory>
#include <utility>
#include <vector>

#include "schedule.h"
#include "simar.h"

namespace simar {

// Built-in defaults: the fit of the calibration sweep on MI355X (p = 8,
// bf16, 1.5 KiB .. 192 MiB per rank, rotating buffer sets; host enqueue
// costs where the pipelined form fits better; per-workgroup rates from
// budgets of 16 .. 128 workgroups at 48 MiB per rank, LL at 768 KiB; the
// topology schedules at the topologies the calibration file states),
// rounded.  A calibration file loaded with sim_model_load() or
// SIM_CALIB replaces them.
Model default_model() {
  Model m;
  // {alpha_us, gbps, steps, bytes_factor, wg_gbps, host_us}, from the MI355X
  // calibration (p = 8, bf16)
  m.a[SIM_ALGO_AUTO] = {0.0, 1.0, -1.0, -1.0, 0.0, 0.0};
  m.a[SIM_ALGO_RING] = {2.5, 6350.0, -1.0, -1.0, 24.4, 2.8};
  m.a[SIM_ALGO_ALLPAIRS] = {2.15, 6100.0, -1.0, -1.0, 47.2, 3.0};
  m.a[SIM_ALGO_ONESHOT] = {1.8, 6250.0, -1.0, -1.0, 53.3, 3.2};
  m.a[SIM_ALGO_ONESHOT_LL] = {8.9, 13500.0, -1.0, -1.0, 8.9, 0.0};
  m.a[SIM_ALGO_RING_FIFO] = {13.5, 660.0, -1.0, -1.0, 16.25, 0.0};
  m.a[SIM_ALGO_TREE] = {3.15, 6200.0, -1.0, -1.0, 0.0, 4.15};
  m.a[SIM_ALGO_REXCH] = {2.25, 6000.0, -1.0, -1.0, 0.0, 4.1};
  m.a[SIM_ALGO_HIER] = {3.35, 6200.0, -1.0, -1.0, 0.0, 4.25};
  m.a[SIM_ALGO_HIER_LARGE] = {3.2, 6000.0, -1.0, -1.0, 0.0, 4.45};
  m.a[SIM_ALGO_ALLPAIRS_PERSISTENT] = {6.95, 8000.0, -1.0, -1.0, 32.0, 0.0};
  // second regimes: the phased one-shot, the single-launch ring's FIFO protocol
  m.hi[SIM_ALGO_ONESHOT] = {8.8, 6600.0, -1.0, -1.0, 53.3, 0.0};
  m.has_hi[SIM_ALGO_ONESHOT] = true;
  m.hi[SIM_ALGO_RING_FIFO] = {24.2, 6450.0, -1.0, -1.0, 16.25, 50.6};
  m.has_hi[SIM_ALGO_RING_FIFO] = true;
  return m;
}

static bool is_topology_algo(int algo) { return algo >= SIM_ALGO_TREE && algo <= SIM_ALGO_HIER_LARGE; }

int model_launches(int coll, int algo, int p, const Topology& t) {
  switch (algo) {
    case SIM_ALGO_RING: return coll == COLL_ALLREDUCE ? 2 * (p - 1) : p - 1;
    case SIM_ALGO_ALLPAIRS: return coll == COLL_ALLREDUCE ? 2 : 1;
    case SIM_ALGO_ONESHOT: return 1;
    case SIM_ALGO_ONESHOT_LL: return 1;
    case SIM_ALGO_ALLPAIRS_PERSISTENT: return coll == COLL_ALLREDUCE ? 1 : -1;
    case SIM_ALGO_RING_FIFO: return 1;
  }
  if (is_topology_algo(algo) && coll == COLL_ALLREDUCE) {
    const Schedule* s = cached_schedule(coll, algo, p, t, nullptr);
    return s ? (int)s->steps.size() : -1;  // one launch per step
  }
  return 0;
}

double schedule_traffic(const Schedule& s, double n, int esize) {
  const double e = esize;
  const int p = s.p;
  std::vector<char> part((size_t)p * s.nchunks, 0);  // value held as a 4-byte partial
  double bytes = 0;
  for (const auto& step : s.steps) {
    std::vector<char> next = part;
    std::vector<std::pair<int, uint32_t>> groups;  // (chunk, set) of the step's exchanges
    for (const Xfer& x : step) {
      const double len = n / s.nchunks;
      auto operand = [&](int q) { return len * (part[(size_t)q * s.nchunks + x.chunk] ? 4.0 : e); };
      const bool post = (x.kind == XK_GATHER_POST || x.kind == XK_EXCH_POST);
      const double out = len * (post ? e : 4.0);
      if (x.kind == XK_GATHER || x.kind == XK_GATHER_POST) {
        bytes += operand(x.dst) + out;
        for (int q = 0; q < p; q++)
          if (x.mask & (1u << q)) bytes += operand(q);
        next[(size_t)x.dst * s.nchunks + x.chunk] = !post;
      } else if (x.kind == XK_EXCH || x.kind == XK_EXCH_POST) {
        const std::pair<int, uint32_t> key(x.chunk, x.mask);
        bool seen = false;
        for (auto& k : groups) seen = seen || (k == key);
        if (!seen) {
          groups.push_back(key);
          for (int q = 0; q < p; q++)
            if (x.mask & (1u << q)) bytes += operand(q);
        }
        bytes += out;
        next[(size_t)x.dst * s.nchunks + x.chunk] = !post;
      } else if (x.kind == XK_MCAST) {
        int k = 0;
        for (int q = 0; q < p; q++)
          if (x.mask & (1u << q)) k++;
        bytes += len * e * (1 + k);
      }
    }
    part = next;
  }
  return bytes;
}

double model_traffic(int coll, int algo, int p, double n, int esize, const Topology& t) {
  const double e = esize, S = n * e;
  if (is_topology_algo(algo)) {
    const Schedule* s = (coll == COLL_ALLREDUCE) ? cached_schedule(coll, algo, p, t, nullptr) : nullptr;
    return s ? schedule_traffic(*s, n, esize) : 0.0;
  }
  if (coll == COLL_ALLREDUCE) {
    switch (algo) {
      case SIM_ALGO_ONESHOT: return 2.0 * p * S;          // p inputs read, p outputs written
      case SIM_ALGO_ALLPAIRS: return (2.0 * p + 1.0) * S;  // step 1: pS + S; step 2: S + (p-1)S
      case SIM_ALGO_ONESHOT_LL: return 6.0 * p * S;        // pack 3pS, consume 3pS
      case SIM_ALGO_ALLPAIRS_PERSISTENT:  // step 1: pS + S; step 2: every rank pulls (p-1) chunks: 2(p-1)S
        return (3.0 * p - 1.0) * S;
      case SIM_ALGO_RING_FIFO:  // inputs and outputs once; fp32 partials through FIFOs; peer reads
        return 2.0 * p * S + (p - 1) * n * 8.0 + (p - 1) * n * e;
      case SIM_ALGO_RING: {
        // reduce-scatter: first step in,in->part; middle part,in->part;
        // last part,in->out; partials are 4-byte accumulators.  Each step
        // touches n elements in total (p transfers of n/p).
        double rs;
        if (p == 2) rs = n * (e + e + e);
        else rs = n * (e + e + 4) + (p - 3) * n * (4 + e + 4) + n * (4 + e + e);
        const double ag = (p - 1) * n * (e + e);
        return rs + ag;
      }
    }
  } else if (coll == COLL_REDUCE_SCATTER) {
    switch (algo) {
      case SIM_ALGO_ALLPAIRS: return (p + 1.0) * S;       // all inputs read, p chunk outputs
      case SIM_ALGO_RING:
        if (p == 2) return n * (e + e + e);
        return n * (e + e + 4) + (p - 3) * n * (4 + e + 4) + n * (4 + e + e);
    }
  } else if (coll == COLL_ALL_GATHER) {
    switch (algo) {
      case SIM_ALGO_ALLPAIRS: return (p + 1.0) * S;       // S/p read per block, S written per rank
      case SIM_ALGO_RING: return (2.0 * p - 1.0) * S;     // step 0 reads once, writes twice
    }
  }
  return 0.0;
}

LaunchEntry model_launch(const Model& m, int algo, int p, double bytes_per_rank) {
  LaunchEntry best;
  if (algo <= 0 || algo >= kNumAlgos || m.wg[algo].empty() || !(bytes_per_rank > 0)) return best;
  if (m.wg_p > 0 && p != m.wg_p) return best;
  const double lb = std::log2(bytes_per_rank);
  double bd = 0;
  bool found = false;
  for (const auto& e : m.wg[algo]) {
    const double d = std::fabs(e.lb - lb);
    if (!found || d < bd) {
      best = e;
      bd = d;
      found = true;
    }
  }
  return best;
}

int model_workgroups(const Model& m, int algo, int p, double bytes_per_rank) {
  return model_launch(m, algo, p, bytes_per_rank).total;
}

// A workgroup budget (T-CCL's restricted mode, "T-CCL ...", sections III-C3
// and IV-B: communication confined to a fixed number of thread blocks) caps
// how many workgroups each launch of a schedule runs.  Few workgroups
// cannot keep enough memory requests in flight, so the bandwidth term
// falls: each workgroup sustains about b GB/s, and W of them about W b,
// until they saturate HBM at B.  A hard min(B, W b) over-predicts at
// budgets near the knee, where the workgroups already contend; the cube
// smooth minimum follows the knee (one-shot, p = 8, bf16, 64 MiB per rank
// on MI355X: 32 workgroups 1.55 TB/s, 128 workgroups 4.5 TB/s, no budget
// 5.6 TB/s).
double model_bandwidth(const AlgoModel& am, int algo, int p, int budget) {
  if (budget <= 0 || !(am.wg_gbps > 0)) return am.gbps;
  const bool persistent = algo == SIM_ALGO_RING_FIFO || algo == SIM_ALGO_ALLPAIRS_PERSISTENT;
  const double w = persistent ? std::max(budget, p) : budget;
  const double bw = w * am.wg_gbps;
  return std::pow(std::pow(am.gbps, -3.0) + std::pow(bw, -3.0), -1.0 / 3.0);
}

double model_predict(const Model& m, int coll, int algo, int p, double n, int esize, const Topology& t,
                     int budget, double hi_from) {
  if (algo <= 0 || algo >= kNumAlgos) return 1e30;
  const bool hi = hi_from > 0 && m.has_hi[algo] && n * esize >= hi_from;
  const AlgoModel& am = hi ? m.hi[algo] : m.a[algo];
  const int launches = model_launches(coll, algo, p, t);
  if (launches < 0) return 1e30;  // no schedule for this topology
  const double steps = am.steps >= 0 ? am.steps : (double)launches;
  const double bytes = am.bytes_factor >= 0 ? am.bytes_factor * n * esize
                                            : model_traffic(coll, algo, p, n, esize, t);
  const double gpu = am.alpha_us * steps + bytes / (model_bandwidth(am, algo, p, budget) * 1e3);  // GB/s -> B/us
  return std::max(am.host_us * launches, gpu);
}

// ---------------------------------------------------------------------------
// A small JSON reader for the calibration file: objects, arrays, strings,
// numbers, true/false/null.
// ---------------------------------------------------------------------------
namespace {

struct JVal {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
  double num = 0;
  std::string str;
  std::vector<JVal> arr;
  std::map<std::string, JVal> obj;
};

struct Parser {
  const char* s;
  const char* end;
  std::string err;
  void ws() {
    while (s < end && std::isspace((unsigned char)*s)) s++;
  }
  bool lit(const char* w) {
    size_t k = std::strlen(w);
    if ((size_t)(end - s) >= k && std::strncmp(s, w, k) == 0) {
      s += k;
      return true;
    }
    return false;
  }
  bool str(std::string* out) {
    if (s >= end || *s != '"') return fail("expected a string");
    s++;
    while (s < end && *s != '"') {
      if (*s == '\\') {
        s++;
        if (s >= end) return fail("bad escape");
        char c = *s;
        out->push_back(c == 'n' ? '\n' : c == 't' ? '\t' : c);
      } else {
        out->push_back(*s);
      }
      s++;
    }
    if (s >= end) return fail("unterminated string");
    s++;
    return true;
  }
  bool fail(const char* m) {
    if (err.empty()) err = m;
    return false;
  }
  bool value(JVal* v, int depth) {
    if (depth > 32) return fail("nesting too deep");
    ws();
    if (s >= end) return fail("unexpected end");
    if (*s == '{') {
      v->kind = JVal::OBJ;
      s++;
      ws();
      if (s < end && *s == '}') {
        s++;
        return true;
      }
      for (;;) {
        ws();
        std::string k;
        if (!str(&k)) return false;
        ws();
        if (s >= end || *s != ':') return fail("expected ':'");
        s++;
        if (!value(&v->obj[k], depth + 1)) return false;
        ws();
        if (s < end && *s == ',') {
          s++;
          continue;
        }
        if (s < end && *s == '}') {
          s++;
          return true;
        }
        return fail("expected ',' or '}'");
      }
    }
    if (*s == '[') {
      v->kind = JVal::ARR;
      s++;
      ws();
      if (s < end && *s == ']') {
        s++;
        return true;
      }
      for (;;) {
        v->arr.emplace_back();
        if (!value(&v->arr.back(), depth + 1)) return false;
        ws();
        if (s < end && *s == ',') {
          s++;
          continue;
        }
        if (s < end && *s == ']') {
          s++;
          return true;
        }
        return fail("expected ',' or ']'");
      }
    }
    if (*s == '"') {
      v->kind = JVal::STR;
      return str(&v->str);
    }
    if (lit("true")) {
      v->kind = JVal::BOOL;
      v->num = 1;
      return true;
    }
    if (lit("false")) {
      v->kind = JVal::BOOL;
      return true;
    }
    if (lit("null")) return true;
    // JSON numbers only: strtod alone would also take inf, nan and hex forms
    if (*s != '-' && !(*s >= '0' && *s <= '9')) return fail("bad value");
    char* e2 = nullptr;
    std::string tmp(s, (size_t)std::min<ptrdiff_t>(end - s, 64));
    double d = std::strtod(tmp.c_str(), &e2);
    if (e2 == tmp.c_str() || !std::isfinite(d) || tmp.find_first_of("xX") < (size_t)(e2 - tmp.c_str()))
      return fail("bad number");
    s += (e2 - tmp.c_str());
    v->kind = JVal::NUM;
    v->num = d;
    return true;
  }
};

const char* kAlgoNames[kNumAlgos] = {"auto",      "ring",  "allpairs", "oneshot",    "oneshot_ll",         "ring_fifo",
                                     "tree",      "rexch", "hier",     "hier_large", "allpairs_persistent"};

}  // namespace

bool model_load_json(const char* path, Model* m, std::string* err) {
  FILE* f = std::fopen(path, "rb");
  if (!f) {
    if (err) *err = "cannot open file";
    return false;
  }
  std::string text;
  char buf[4096];
  size_t k;
  while ((k = std::fread(buf, 1, sizeof buf, f)) > 0) text.append(buf, k);
  std::fclose(f);
  Parser ps{text.data(), text.data() + text.size(), ""};
  JVal root;
  if (!ps.value(&root, 0) || root.kind != JVal::OBJ) {
    if (err) *err = ps.err.empty() ? "top level is not an object" : ps.err;
    return false;
  }
  ps.ws();
  if (ps.s != ps.end) {
    if (err) *err = "trailing content after the top-level object";
    return false;
  }
  auto it = root.obj.find("algos");
  if (it == root.obj.end() || it->second.kind != JVal::OBJ) {
    if (err) *err = "missing object 'algos'";
    return false;
  }
  Model out = *m;
  // one algo entry: alpha_us and gbps, optional host_us and wg_gbps
  auto entry = [&](const JVal& o, AlgoModel* am) {
    if (o.kind != JVal::OBJ) {
      if (err) *err = "algo entry is not an object";
      return false;
    }
    auto al = o.obj.find("alpha_us");
    auto bw = o.obj.find("gbps");
    if (al == o.obj.end() || bw == o.obj.end() || al->second.kind != JVal::NUM ||
        bw->second.kind != JVal::NUM || !(bw->second.num > 0) || !(al->second.num >= 0)) {
      if (err) *err = "algo entry needs numeric alpha_us >= 0 and gbps > 0";
      return false;
    }
    am->alpha_us = al->second.num;
    am->gbps = bw->second.num;
    am->steps = -1;
    am->bytes_factor = -1;
    am->wg_gbps = 0;
    am->host_us = 0;
    auto hu = o.obj.find("host_us");  // optional: host enqueue cost per launch
    if (hu != o.obj.end()) {
      if (hu->second.kind != JVal::NUM || !(hu->second.num >= 0)) {
        if (err) *err = "host_us must be a number >= 0";
        return false;
      }
      am->host_us = hu->second.num;
    }
    auto wr = o.obj.find("wg_gbps");  // optional: rate of one workgroup under a budget
    if (wr != o.obj.end()) {
      if (wr->second.kind != JVal::NUM || !(wr->second.num >= 0)) {
        if (err) *err = "wg_gbps must be a number >= 0";
        return false;
      }
      am->wg_gbps = wr->second.num;
    }
    return true;
  };
  for (int a = 1; a < kNumAlgos; a++) {
    auto ai = it->second.obj.find(kAlgoNames[a]);
    if (ai == it->second.obj.end()) continue;
    if (!entry(ai->second, &out.a[a])) return false;
    out.has_hi[a] = false;  // a file's algo entry replaces both regimes; "algos_hi" adds the second
  }
  // optional: second regimes, "algos_hi": {algo: entry} (Model::hi)
  auto hit = root.obj.find("algos_hi");
  if (hit != root.obj.end()) {
    if (hit->second.kind != JVal::OBJ) {
      if (err) *err = "'algos_hi' is not an object";
      return false;
    }
    for (int a = 1; a < kNumAlgos; a++) {
      auto ai = hit->second.obj.find(kAlgoNames[a]);
      if (ai == hit->second.obj.end()) continue;
      if (!entry(ai->second, &out.hi[a])) return false;
      out.has_hi[a] = true;
    }
  }
  // optional: the rank count the launch table was measured at
  out.wg_p = 0;
  auto pt = root.obj.find("p");
  if (pt != root.obj.end()) {
    if (pt->second.kind != JVal::NUM || !(pt->second.num >= 2 && pt->second.num <= SIM_MAX_RANKS) ||
        pt->second.num != std::floor(pt->second.num)) {
      if (err) *err = "p must be an integer rank count in 2..16";
      return false;
    }
    out.wg_p = (int)pt->second.num;
  }
  // optional launch-configuration table: "workgroups": {algo: [[bytes, total], ...]}
  auto wt = root.obj.find("workgroups");
  if (wt != root.obj.end()) {
    if (wt->second.kind != JVal::OBJ) {
      if (err) *err = "'workgroups' is not an object";
      return false;
    }
    for (int a = 1; a < kNumAlgos; a++) {
      auto ai = wt->second.obj.find(kAlgoNames[a]);
      if (ai == wt->second.obj.end()) continue;
      if (ai->second.kind != JVal::ARR) {
        if (err) *err = "workgroup entry is not an array";
        return false;
      }
      std::vector<LaunchEntry> v;
      for (const JVal& e : ai->second.arr) {
        const bool shape = e.kind == JVal::ARR && (e.arr.size() == 2 || e.arr.size() == 3);
        bool ok = shape && e.arr[0].kind == JVal::NUM && e.arr[1].kind == JVal::NUM && e.arr[0].num > 0 &&
                  e.arr[1].num >= 0 && e.arr[1].num <= (double)(1 << 24);
        if (ok && e.arr.size() == 3)
          ok = e.arr[2].kind == JVal::NUM && (e.arr[2].num == 1 || e.arr[2].num == 2 || e.arr[2].num == 4);
        if (!ok) {
          if (err) *err = "workgroup entries are [bytes > 0, total in 0..2^24(, vectors per lane 1, 2 or 4)]";
          return false;
        }
        LaunchEntry le;
        le.bytes = e.arr[0].num;
        le.total = (int)e.arr[1].num;
        le.unroll = e.arr.size() == 3 ? (int)e.arr[2].num : 0;
        le.lb = std::log2(le.bytes);
        v.push_back(le);
      }
      std::sort(v.begin(), v.end());
      out.wg[a] = v;
    }
  }
  out.source = path;
  *m = out;
  return true;
}

}  // namespace simar

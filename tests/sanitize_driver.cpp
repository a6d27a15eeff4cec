// sanitize_driver.cpp -- host-only exercise of the library's schedule layer,
// verifier, cost model and calibration-file parser, built with g++ under
// AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py.  Exits non-zero on a logic failure; the
// sanitizers abort on any memory or undefined-behaviour error.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "schedule.h"
#include "select.h"
#include "simar.h"

using namespace simar;

static int fail(const char* what) {
  std::fprintf(stderr, "FAIL: %s\n", what);
  return 1;
}

int main(int argc, char** argv) {
  const char* tmp = argc > 1 ? argv[1] : "sanitize_model.json";
  std::mt19937 rng(12345);
  long lowered = 0, mutants = 0, rejected = 0;
  // 1. every collective, algo, p and topology the lowering accepts: lowered, proven
  for (int coll = COLL_ALLREDUCE; coll <= COLL_ALL_GATHER; coll++)
    for (int algo = SIM_ALGO_RING; algo < SIM_NUM_ALGOS; algo++)
      for (int p = 2; p <= SIM_MAX_RANKS; p++)
        for (int G = 1; G <= p; G++)
          for (int k = 2; k <= 4; k++) {
            Topology t;
            t.ranks_per_node = G;
            t.radix = k;
            Schedule s;
            if (!lower(coll, algo, p, t, &s)) continue;
            std::string d;
            if (!verify(s, &d)) return fail(d.c_str());
            lowered++;
            std::vector<uint32_t> masks((size_t)p * s.nchunks);
            for (int st = 0; st <= (int)s.steps.size(); st++)
              if (!symbolic_state(s, st, masks.data(), &d)) return fail(d.c_str());
            // 2. random mutations: the verifier must never crash, and a
            // dropped transfer must be rejected
            for (int m = 0; m < 4 && !s.steps.empty(); m++) {
              Schedule mu = s;
              auto& step = mu.steps[rng() % mu.steps.size()];
              if (step.empty()) continue;
              Xfer& x = step[rng() % step.size()];
              const int what = (int)(rng() % 5);
              bool must_reject = false;
              if (what == 0) {
                step.erase(step.begin() + (long)(rng() % step.size()));
                must_reject = true;
              } else if (what == 1) {
                x.chunk = (int)(rng() % (unsigned)(mu.nchunks + 2)) - 1;  // may be out of range
              } else if (what == 2) {
                x.src = (int)(rng() % (unsigned)(p + 2)) - 1;
              } else if (what == 3) {
                x.dst = (int)(rng() % (unsigned)(p + 2)) - 1;
              } else {
                x.kind = (int)(rng() % (kNumXferKinds + 2)) - 1;
              }
              mutants++;
              const bool ok = verify(mu, &d);
              if (!ok) rejected++;
              if (must_reject && ok && coll == COLL_ALLREDUCE) return fail("a dropped transfer was accepted");
            }
          }
  // 3. the cost model on every algo and collective, with and without a budget
  //    (and with the host term, which only ever raises a prediction)
  Model m = default_model();
  for (int coll = COLL_ALLREDUCE; coll <= COLL_ALL_GATHER; coll++)
    for (int algo = 0; algo <= SIM_NUM_ALGOS; algo++)
      for (int p = 2; p <= SIM_MAX_RANKS; p++)
        for (int budget : {0, 1, 32, 4096}) {
          // combinations the library never prices (a reduce-scatter on a
          // topology schedule, AUTO) come back as 0 or 1e30; none may be NaN or negative
          const double t = model_predict(m, coll, algo, p, 1 << 20, 2, Topology(), budget);
          if (!(t >= 0)) return fail("negative or NaN prediction");
        }
  // 4. the calibration-file parser on valid, truncated and randomly corrupted files
  const std::string good =
      "{\"algos\": {\"oneshot\": {\"alpha_us\": 1.25, \"gbps\": 5650, \"wg_gbps\": 49, \"host_us\": 3.2},"
      " \"ring\": {\"alpha_us\": 2.5, \"gbps\": 6350}},"
      " \"workgroups\": {\"oneshot\": [[1048576, 0], [67108864, 4096, 2]]}}";
  long parsed = 0, refused = 0;
  for (int it = 0; it < 4000; it++) {
    std::string text = good;
    if (it > 0) {
      const int edits = 1 + (int)(rng() % 4);
      for (int e = 0; e < edits && !text.empty(); e++) {
        const size_t pos = rng() % text.size();
        switch (rng() % 4) {
          case 0: text.erase(pos, 1 + rng() % 8); break;
          case 1: text.insert(pos, 1, "{}[],:\"-0e9xn"[rng() % 13]); break;
          case 2: text[pos] = (char)(32 + rng() % 95); break;
          default: text.resize(pos); break;
        }
      }
    }
    FILE* f = std::fopen(tmp, "wb");
    if (!f) return fail("cannot write the temporary model file");
    std::fwrite(text.data(), 1, text.size(), f);
    std::fclose(f);
    Model mm = default_model();
    std::string err;
    if (model_load_json(tmp, &mm, &err)) parsed++;
    else refused++;
    if (it == 0 && parsed != 1) return fail(err.c_str());
  }
  std::remove(tmp);
  std::printf("lowered %ld schedules, %ld mutants (%ld rejected), parser %ld accepted / %ld refused\n", lowered,
              mutants, rejected, parsed, refused);
  return 0;
}

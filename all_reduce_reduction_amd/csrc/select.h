// select.h -- the alpha-beta cost model and the argmin selector (host only).
#pragma once

#include <cstddef>
#include <string>
#include <utility>
#include <vector>

#include "schedule.h"

namespace simar {

constexpr int kNumAlgos = 11;  // indices are the SIM_ALGO_* codes (0 = AUTO unused)

struct AlgoModel {
  double alpha_us = 4.0;       // fixed cost per launch (sync step)
  double gbps = 4000.0;        // effective rate for the schedule's bytes
  double steps = -1.0;         // override of the launch count law when >= 0
  double bytes_factor = -1.0;  // override of the traffic law (bytes per message byte) when >= 0
  double wg_gbps = 0.0;        // rate one workgroup sustains, for calls under a workgroup budget (0: no term)
  double host_us = 0.0;        // host enqueue cost per launch, overlapping the GPU's work (0: no term)
};

// One measured launch configuration.
struct LaunchEntry {
  double bytes = 0;  // bytes per rank it was measured at
  int total = 0;     // total workgroups (0: cover every transfer exactly)
  int unroll = 0;    // 16-byte vectors per lane per pass, 1 or 2 (0: the default, 1)
  double lb = 0;     // log2(bytes), kept for the nearest-size lookup
  bool operator<(const LaunchEntry& o) const { return bytes < o.bytes; }
};

struct Model {
  AlgoModel a[kNumAlgos];
  // A second regime of an algo whose kernels change with the size: the
  // single-launch ring's FIFO protocol above its LL limit, the phased
  // one-shot from its threshold.  Used from the size the caller names
  // (model_predict's hi_from); absent unless has_hi.
  AlgoModel hi[kNumAlgos];
  bool has_hi[kNumAlgos] = {};
  // Measured launch configurations (after T-CCL's ranked CTA-config table):
  // per algo, entries from the calibration sweep, ascending in bytes; empty
  // = cover every transfer exactly with one vector per lane.
  std::vector<LaunchEntry> wg[kNumAlgos];
  // the rank count the table was measured at: a call with another count
  // ignores it (0: the table applies to every count)
  int wg_p = 0;
  std::string source = "built-in defaults";
};

// The table's entry for (algo, p ranks, bytes per rank): the one of the
// nearest size on a log scale; a default entry (total 0, unroll 0) when the
// table has none or was measured at another rank count (a total tuned for
// p = 8 ranks' 2p streams per workgroup starves a launch at p = 2).
LaunchEntry model_launch(const Model& m, int algo, int p, double bytes_per_rank);
// Its total workgroups (0: cover the transfer).
int model_workgroups(const Model& m, int algo, int p, double bytes_per_rank);

Model default_model();

// Launches (latency units) of a schedule; `coll` is a simar::Coll.  The
// tree, recursive exchange and 2PH schedules depend on the topology (-1
// when it does not fit p).
int model_launches(int coll, int algo, int p, const Topology& t = Topology());

// Algorithmic HBM bytes of one call, summed over all simulated ranks.
// n = elements per rank of the all-reduce input (reduce-scatter: the full
// input; all-gather: the full output), esize = bytes per element.
double model_traffic(int coll, int algo, int p, double n, int esize, const Topology& t = Topology());

// The same for a lowered tree / recursive-exchange / 2PH schedule as the
// step executor runs it: each fold reads its operands once (inputs at
// storage width, partials as 4-byte accumulators) and writes every
// receiving rank once (finished values at storage width, partials at 4
// bytes); the members of an exchange group share one fold; a broadcast
// reads once and writes each receiver.
double schedule_traffic(const Schedule& s, double n, int esize);

// The bandwidth a call of `algo` can use under a workgroup budget of
// `budget` workgroups per launch (0: none): B itself without a budget or
// without a per-workgroup rate, else the smooth minimum
//   (B^-3 + (W b)^-3)^(-1/3)
// of B and the budget's aggregate rate W b, W being the budget (at least one
// workgroup per rank for the single-launch schedules, which keep that many).
double model_bandwidth(const AlgoModel& am, int algo, int p, int budget);

// T = alpha * launches + traffic / B_eff, in microseconds, B_eff being
// model_bandwidth() at `budget`; with a host enqueue cost H per launch,
// T = max(H * launches, that): calls issued back to back overlap the host's
// enqueue of one call with the GPU's execution of the previous one, so a
// call costs whichever side is slower.  From hi_from bytes per rank on
// (when > 0) the algo's second regime prices the call, when the model has
// one (Model::hi).
double model_predict(const Model& m, int coll, int algo, int p, double n, int esize,
                     const Topology& t = Topology(), int budget = 0, double hi_from = 0.0);

// Parse a calibration file; returns false (and leaves *m alone) on error.
bool model_load_json(const char* path, Model* m, std::string* err);

}  // namespace simar

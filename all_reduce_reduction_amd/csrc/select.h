// select.h -- the alpha-beta cost model and the argmin selector (host only).
#pragma once

#include <cstddef>
#include <string>

namespace simar {

constexpr int kNumAlgos = 6;  // indices are the SIM_ALGO_* codes (0 = AUTO unused)

struct AlgoModel {
  double alpha_us = 4.0;       // fixed cost per launch (sync step)
  double gbps = 4000.0;        // effective rate for the schedule's bytes
  double steps = -1.0;         // override of the launch count law when >= 0
  double bytes_factor = -1.0;  // override of the traffic law (bytes per message byte) when >= 0
};

struct Model {
  AlgoModel a[kNumAlgos];
  std::string source = "built-in defaults";
};

Model default_model();

// Launches (latency units) of a schedule; `coll` is a simar::Coll.
int model_launches(int coll, int algo, int p);

// Algorithmic HBM bytes of one call, summed over all simulated ranks.
// n = elements per rank of the all-reduce input (reduce-scatter: the full
// input; all-gather: the full output), esize = bytes per element.
double model_traffic(int coll, int algo, int p, double n, int esize);

// T = alpha * launches + traffic / B, in microseconds.
double model_predict(const Model& m, int coll, int algo, int p, double n, int esize);

// Parse a calibration file; returns false (and leaves *m alone) on error.
bool model_load_json(const char* path, Model* m, std::string* err);

}  // namespace simar

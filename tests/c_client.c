/* A plain C99 client of the library's C ABI: it includes only the public
 * header, links against the shared library and calls the host-only entry
 * points (no device needed).  Each line it prints is checked by
 * test_c_client.py. */
#include <stdio.h>
#include <stdint.h>

#include "simar.h"

int main(void) {
  int algo, nsteps, nxfers, nchunks, parent, children[3], nchildren, st, v;
  char diag[256];
  int counts[2];
  int xfers[2 * 5 * 8];
  int i;

  printf("version %d\n", sim_version());
  printf("status %s\n", sim_status_string(SIM_OK));

  for (algo = SIM_ALGO_RING; algo < SIM_NUM_ALGOS; algo++) {
    st = sim_schedule_info(algo, 8, &nsteps, &nxfers, &nchunks);
    if (st != SIM_OK) {
      printf("info %d status %d\n", algo, st);
      continue;
    }
    printf("info %d %d %d %d\n", algo, nsteps, nxfers, nchunks);
    printf("verify %d %d\n", algo, sim_verify_schedule(algo, 8, diag, sizeof diag));
  }

  /* the all-pairs schedule over 4 ranks, handed back as a custom schedule */
  st = sim_schedule_xfers(SIM_ALGO_ALLPAIRS, 4, 0, xfers, 8, &counts[0]);
  if (st == SIM_OK) st = sim_schedule_xfers(SIM_ALGO_ALLPAIRS, 4, 1, xfers + 5 * counts[0], 8, &counts[1]);
  if (st == SIM_OK)
    st = sim_verify_custom(SIM_ALGO_ALLPAIRS, 4, 4, 2, 2, counts, xfers, diag, sizeof diag);
  printf("custom %d\n", st);
  /* the same with its two steps swapped must be refused (both steps hold
   * one transfer per rank) */
  if (counts[0] != counts[1]) return 1;
  for (i = 0; i < 5 * counts[0]; i++) {
    int t = xfers[i];
    xfers[i] = xfers[5 * counts[0] + i];
    xfers[5 * counts[0] + i] = t;
  }
  printf("swapped %d\n", sim_verify_custom(SIM_ALGO_ALLPAIRS, 4, 4, 2, 2, counts, xfers, diag, sizeof diag));

  st = sim_tree_info(0, 8, 1, 4, &parent, children, &nchildren);
  printf("tree %d %d %d", st, parent, nchildren);
  for (i = 0; i < nchildren; i++) printf(" %d", children[i]);
  printf("\n");

  st = sim_config_get(SIM_CONFIG_RANKS_PER_NODE, &v);
  printf("config %d %d\n", st, v);
  printf("config_bad %d\n", sim_config_set(-1, 0));

  {
    const void* in[2] = {0, 0};
    void* out[2] = {0, 0};
    printf("before_init %d\n", sim_allreduce(in, out, 2, 4, SIM_INT32, SIM_SUM, SIM_ALGO_ONESHOT, (void*)0));
  }
  return 0;
}

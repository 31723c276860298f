/* Plain C99 use of the library's C ABI: host-only plan calls, no GPU.
 * Plans the TransformerBlock of hidden 512 as one FSDP1 FlatParameter of
 * its six linear weights at R = 4 and prints T, S, the rank offsets, the
 * all-gather elements one rank sends and the resident bytes per rank. */
#include <stdio.h>
#include <stdint.h>

#include "fsdp_mi355x.h"

int main(void) {
  const int32_t ndims[6] = {2, 2, 2, 2, 2, 2};
  const int64_t dims[12] = {512, 512, 512, 512, 512, 512, 512, 512, 512, 2048, 2048, 512};
  fsdp_plan* plan = NULL;
  fsdp_status st = fsdp_plan_layout(6, ndims, dims, 4, FSDP_LAYOUT_FLAT, &plan);
  if (st != FSDP_OK) {
    printf("error %s\n", fsdp_status_string(st));
    return 1;
  }
  fsdp_plan_info info;
  fsdp_plan_get_info(plan, &info);
  printf("T %lld S %lld R %d segments %d\n", (long long)info.numel_full,
         (long long)info.shard_numel, info.world, info.n_segments);
  int64_t seg[4 * 8];
  fsdp_plan_segments(plan, seg, 8);
  for (int i = 0; i < info.n_segments; ++i) printf("offset %lld\n", (long long)seg[4 * i + 2]);
  int64_t ledger[4];
  fsdp_plan_comm_ledger(plan, 0, ledger);
  printf("all_gather %lld\n", (long long)ledger[0]);
  printf("state_bytes %lld\n", (long long)fsdp_plan_state_bytes_per_rank(plan));
  fsdp_plan* bad = (fsdp_plan*)1;
  st = fsdp_plan_layout(6, ndims, dims, 0, FSDP_LAYOUT_FLAT, &bad);
  printf("R=0 -> %s, out %s\n", fsdp_status_string(st), bad == NULL ? "NULL" : "set");
  fsdp_plan_destroy(plan);
  return 0;
}

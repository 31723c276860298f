/* One training step of one FSDP unit driven from plain C99 through the
 * library's C ABI: device memory comes from the HIP runtime, no Python or
 * PyTorch is involved.
 *
 * Usage: step_from_c DIR.  Reads
 *   DIR/shape.txt       "R layout n_params" then the n_params ndims, then
 *                       all dims (whitespace separated);
 *   DIR/in_master.f32   the unit's full fp32 master [T];
 *   DIR/in_grads.bf16   R full-unit gradients, bf16 bits [R][T];
 * runs, on the null stream: pack of the fp32 master and of the bf16
 * parameter, the all-gather + unflatten into R receivers, the
 * reduce-scatter-average, and one fused AdamW step (t = 1, lr 1e-3, betas
 * 0.9 / 0.999, eps 1e-8, weight decay 0.01) over the R gradient replicas;
 * and writes DIR/out_gather.bf16 [R][T], out_rs.f32, out_master.f32,
 * out_m.f32, out_v.f32 [R][S] and out_param.bf16 [R][S].  Exit status 0 on
 * success; otherwise a message names the failing call. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "fsdp_mi355x.h"

static int fail(const char* what, const char* why) {
  fprintf(stderr, "step_from_c: %s: %s\n", what, why);
  return 1;
}

#define HIP_OK(call)                                                   \
  do {                                                                 \
    hipError_t e_ = (call);                                            \
    if (e_ != hipSuccess) return fail(#call, hipGetErrorString(e_)); \
  } while (0)

#define FSDP_OK_(call)                                                       \
  do {                                                                       \
    fsdp_status s_ = (call);                                                 \
    if (s_ != FSDP_OK) return fail(#call, fsdp_status_string(s_));         \
  } while (0)

static int read_file(const char* dir, const char* name, void* dst, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return fail(path, "cannot open");
  const size_t got = fread(dst, 1, bytes, f);
  fclose(f);
  return got == bytes ? 0 : fail(path, "short read");
}

static int write_file(const char* dir, const char* name, const void* src, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return fail(path, "cannot create");
  const size_t put = fwrite(src, 1, bytes, f);
  fclose(f);
  return put == bytes ? 0 : fail(path, "short write");
}

/* Device buffer -> file. */
static int save(const char* dir, const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) return fail(name, "out of host memory");
  hipError_t e = hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost);
  int rc = e == hipSuccess ? write_file(dir, name, host, bytes) : fail(name, "copy back");
  free(host);
  return rc;
}

int main(int argc, char** argv) {
  if (argc != 2) return fail("usage", "step_from_c DIR");
  const char* dir = argv[1];

  /* the unit's shapes */
  char path[4096];
  snprintf(path, sizeof path, "%s/shape.txt", dir);
  FILE* f = fopen(path, "r");
  if (!f) return fail(path, "cannot open");
  int R = 0, layout = 0, n = 0;
  if (fscanf(f, "%d %d %d", &R, &layout, &n) != 3 || n < 1 || n > 64) {
    fclose(f);
    return fail(path, "bad header");
  }
  int32_t ndims[64];
  int64_t dims[64 * 8];
  int total = 0;
  for (int p = 0; p < n; ++p) {
    if (fscanf(f, "%d", &ndims[p]) != 1 || ndims[p] < 1 || ndims[p] > 8) {
      fclose(f);
      return fail(path, "bad ndims");
    }
    total += ndims[p];
  }
  for (int i = 0; i < total; ++i) {
    long long d = 0;
    if (fscanf(f, "%lld", &d) != 1) {
      fclose(f);
      return fail(path, "bad dims");
    }
    dims[i] = (int64_t)d;
  }
  fclose(f);

  fsdp_plan* plan = NULL;
  FSDP_OK_(fsdp_plan_layout(n, ndims, dims, R, layout, &plan));
  fsdp_plan_info info;
  FSDP_OK_(fsdp_plan_get_info(plan, &info));
  const int64_t T = info.numel_full, S = info.shard_numel, RS = (int64_t)R * S;

  /* inputs */
  float* h_master = (float*)malloc((size_t)T * 4);
  uint16_t* h_grads = (uint16_t*)malloc((size_t)R * T * 2);
  if (!h_master || !h_grads) return fail("inputs", "out of host memory");
  if (read_file(dir, "in_master.f32", h_master, (size_t)T * 4)) return 1;
  if (read_file(dir, "in_grads.bf16", h_grads, (size_t)R * T * 2)) return 1;

  /* device buffers, all owned here */
  float *full, *master, *m, *v, *rs;
  uint16_t *param, *grads, *recv;
  HIP_OK(hipMalloc((void**)&full, (size_t)T * 4));
  HIP_OK(hipMalloc((void**)&master, (size_t)RS * 4));
  HIP_OK(hipMalloc((void**)&m, (size_t)RS * 4));
  HIP_OK(hipMalloc((void**)&v, (size_t)RS * 4));
  HIP_OK(hipMalloc((void**)&rs, (size_t)RS * 4));
  HIP_OK(hipMalloc((void**)&param, (size_t)RS * 2));
  HIP_OK(hipMalloc((void**)&grads, (size_t)R * T * 2));
  HIP_OK(hipMalloc((void**)&recv, (size_t)R * T * 2));
  HIP_OK(hipMemcpy(full, h_master, (size_t)T * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(grads, h_grads, (size_t)R * T * 2, hipMemcpyHostToDevice));
  HIP_OK(hipMemset(m, 0, (size_t)RS * 4));
  HIP_OK(hipMemset(v, 0, (size_t)RS * 4));

  const void* g[FSDP_MAX_RANKS];
  void* r_out[FSDP_MAX_RANKS];
  for (int r = 0; r < R; ++r) {
    g[r] = grads + (size_t)r * T;
    r_out[r] = recv + (size_t)r * T;
  }
  const fsdp_adamw_hparams hp = {1e-3, 0.9, 0.999, 1e-8, 0.01};

  FSDP_OK_(fsdp_shard_pack(plan, full, FSDP_F32, master, FSDP_F32, NULL));
  FSDP_OK_(fsdp_shard_pack(plan, full, FSDP_F32, param, FSDP_BF16, NULL));
  FSDP_OK_(fsdp_gather_unflatten(plan, param, FSDP_BF16, r_out, NULL));
  FSDP_OK_(fsdp_reduce_scatter_avg(plan, g, FSDP_BF16, rs, NULL));
  FSDP_OK_(fsdp_adamw_shard_step(plan, &hp, 1, g, FSDP_BF16, 1, master, m, v, param, FSDP_BF16,
                                 NULL));
  HIP_OK(hipDeviceSynchronize());

  if (save(dir, "out_gather.bf16", recv, (size_t)R * T * 2) ||
      save(dir, "out_rs.f32", rs, (size_t)RS * 4) ||
      save(dir, "out_master.f32", master, (size_t)RS * 4) ||
      save(dir, "out_m.f32", m, (size_t)RS * 4) || save(dir, "out_v.f32", v, (size_t)RS * 4) ||
      save(dir, "out_param.bf16", param, (size_t)RS * 2))
    return 1;

  hipFree(full);
  hipFree(master);
  hipFree(m);
  hipFree(v);
  hipFree(rs);
  hipFree(param);
  hipFree(grads);
  hipFree(recv);
  fsdp_plan_destroy(plan);
  free(h_master);
  free(h_grads);
  printf("step_from_c ok: R=%d T=%lld S=%lld\n", R, (long long)T, (long long)S);
  return 0;
}

/*
 * sgemv_c_driver.c - the SparseGemv library driven from plain C99 through
 * include/sgemv.h alone: no Python, no torch, device memory from the HIP
 * runtime's C API. The tests use it to check that the boundary needs nothing
 * beyond the header, libsgemv.so and (for "run") libamdhip64.so.
 *
 *   sgemv_c_driver pack DIR   host only: DIR/meta.txt ("N K nk B"), DIR/w.bin
 *                             (uint16 FP16 bits [N][K]) and DIR/gs.bin (int32
 *                             group sizes [N]) -> sgemv_describe, sgemv_pack,
 *                             sgemv_layout; writes DIR/desc.txt and DIR/vals.bin,
 *                             offs.bin, scale.bin, zero.bin, gptr.bin,
 *                             rowptr.bin, blob.bin; checks the host error paths.
 *   sgemv_c_driver run DIR    pack as above, then DIR/x.bin (uint16 [B][K]) ->
 *                             hipMalloc / hipMemcpy -> sgemv_run on a stream of
 *                             its own, twice -> DIR/y.bin (uint16 [B][N]); exits
 *                             non-zero if the two calls' bits differ.
 *
 * Exit status 0 on success; otherwise a message on stderr names the step.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "sgemv.h"

static int fail(const char* what, int code) {
  fprintf(stderr, "sgemv_c_driver: %s failed: %d (%s)\n", what, code, sgemv_strerror(code));
  return 1;
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) return NULL;
  void* p = malloc(bytes ? bytes : 1);
  size_t got = p ? fread(p, 1, bytes, f) : 0;
  fclose(f);
  if (got != bytes) {
    free(p);
    return NULL;
  }
  return p;
}

static int write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) return 1;
  size_t put = bytes ? fwrite(p, 1, bytes, f) : 0;
  fclose(f);
  return put != bytes;
}

/* Host error paths: every check runs before any HIP call, so these are safe
 * without a GPU. */
static int check_errors(const sgemv_desc* d) {
  int32_t gs_bad[1] = {48};   /* not a multiple of 32 */
  sgemv_desc tmp;
  sgemv_plan_t pl;
  if (sgemv_describe(1, 256, 3, gs_bad, &tmp) != SGEMV_EINVAL) return fail("describe(nk = 3) error", -100);
  if (sgemv_describe(1, 256, 2, gs_bad, &tmp) != SGEMV_EINVAL) return fail("describe(group 48) error", -100);
  if (sgemv_describe(1, 200, 2, NULL, &tmp) != SGEMV_EINVAL) return fail("describe(K = 200) error", -100);
  if (sgemv_run(NULL, NULL, NULL, NULL, 1, NULL) != SGEMV_EINVAL) return fail("run(NULL) error", -100);
  if (sgemv_plan(d, 0, &pl) != SGEMV_EINVAL) return fail("plan(B = 0) error", -100);
  if (sgemv_plan(d, 17, &pl) != SGEMV_EINVAL) return fail("plan(B = 17) error", -100);
  tmp = *d;
  tmp.blob_bytes += 256;      /* a descriptor sgemv_describe cannot produce */
  if (sgemv_plan(&tmp, 1, &pl) != SGEMV_ESIZE) return fail("plan(inconsistent descriptor) error", -100);
  /* a misaligned device pointer is refused on the host, before any launch */
  if (sgemv_run(d, (const void*)(uintptr_t)0x1000, (const void*)(uintptr_t)0x2002, (void*)(uintptr_t)0x3000, 1, NULL)
      != SGEMV_EALIGN)
    return fail("run(misaligned x) error", -100);
  for (int c = 0; c >= -4; --c)
    if (!sgemv_strerror(c) || !sgemv_strerror(c)[0]) return fail("strerror", c);
  return 0;
}

int main(int argc, char** argv) {
  if (argc != 3 || (strcmp(argv[1], "pack") && strcmp(argv[1], "run"))) {
    fprintf(stderr, "usage: sgemv_c_driver pack|run DIR\n");
    return 2;
  }
  const int run = !strcmp(argv[1], "run");
  const char* dir = argv[2];
  int N = 0, K = 0, nk = 0, B = 0;
  {
    char path[4096];
    snprintf(path, sizeof path, "%s/meta.txt", dir);
    FILE* f = fopen(path, "r");
    if (!f || fscanf(f, "%d %d %d %d", &N, &K, &nk, &B) != 4) {
      if (f) fclose(f);
      fprintf(stderr, "sgemv_c_driver: cannot read %s\n", path);
      return 1;
    }
    fclose(f);
  }
  if (N < 1 || K < 1 || B < 1 || (int64_t)N * K > ((int64_t)1 << 28)) {
    fprintf(stderr, "sgemv_c_driver: unreasonable sizes N=%d K=%d B=%d\n", N, K, B);
    return 1;
  }
  uint16_t* w = (uint16_t*)read_file(dir, "w.bin", (size_t)N * K * 2);
  int32_t* gs = (int32_t*)read_file(dir, "gs.bin", (size_t)N * 4);
  if (!w || !gs) {
    fprintf(stderr, "sgemv_c_driver: cannot read w.bin / gs.bin\n");
    return 1;
  }

  sgemv_desc d;
  int rc = sgemv_describe(N, K, nk, gs, &d);
  if (rc) return fail("sgemv_describe", rc);
  uint8_t* vals = (uint8_t*)malloc((size_t)d.vals_bytes + 1);
  uint8_t* offs = (uint8_t*)malloc((size_t)d.offs_bytes + 1);
  uint16_t* scale = (uint16_t*)malloc((size_t)d.n_groups * 2);
  uint16_t* zero = (uint16_t*)malloc((size_t)d.n_groups * 2);
  int32_t* gptr = (int32_t*)malloc((size_t)(N + 1) * 4);
  int32_t* rowptr = (int32_t*)malloc((size_t)(N + 1) * 4);
  void* blob = malloc((size_t)d.blob_bytes);
  if (!vals || !offs || !scale || !zero || !gptr || !rowptr || !blob) {
    fprintf(stderr, "sgemv_c_driver: out of host memory\n");
    return 1;
  }
  rc = sgemv_pack(w, N, K, nk, gs, vals, nk == 4 ? NULL : offs, scale, zero, gptr, rowptr);
  if (rc) return fail("sgemv_pack", rc);
  rc = sgemv_layout(&d, vals, nk == 4 ? NULL : offs, scale, zero, gptr, blob);
  if (rc) return fail("sgemv_layout", rc);
  if (check_errors(&d)) return 1;

  {
    char path[4096];
    snprintf(path, sizeof path, "%s/desc.txt", dir);
    FILE* f = fopen(path, "w");
    if (!f) return fail("writing desc.txt", -100);
    fprintf(f, "N %d\nK %d\nnk %d\nn_blocks %d\nchunks %d\nkept %lld\nvals_bytes %lld\noffs_bytes %lld\n"
               "n_groups %lld\nblob_bytes %lld\n",
            d.N, d.K, d.nk, d.n_blocks, d.chunks, (long long)d.kept, (long long)d.vals_bytes,
            (long long)d.offs_bytes, (long long)d.n_groups, (long long)d.blob_bytes);
    fclose(f);
  }
  if (write_file(dir, "vals.bin", vals, (size_t)d.vals_bytes) || write_file(dir, "offs.bin", offs, (size_t)d.offs_bytes) ||
      write_file(dir, "scale.bin", scale, (size_t)d.n_groups * 2) || write_file(dir, "zero.bin", zero, (size_t)d.n_groups * 2) ||
      write_file(dir, "gptr.bin", gptr, (size_t)(N + 1) * 4) || write_file(dir, "rowptr.bin", rowptr, (size_t)(N + 1) * 4) ||
      write_file(dir, "blob.bin", blob, (size_t)d.blob_bytes))
    return fail("writing the packed arrays", -100);
  if (!run) return 0;

  /* device path: the caller owns every buffer; the library allocates nothing */
  sgemv_plan_t pl;
  rc = sgemv_plan(&d, B, &pl);
  if (rc) return fail("sgemv_plan", rc);
  uint16_t* x = (uint16_t*)read_file(dir, "x.bin", (size_t)B * K * 2);
  uint16_t* y0 = (uint16_t*)malloc((size_t)B * N * 2);
  uint16_t* y1 = (uint16_t*)malloc((size_t)B * N * 2);
  if (!x || !y0 || !y1) return fail("reading x.bin", -100);
  void *blob_d = NULL, *x_d = NULL, *y_d = NULL;
  hipStream_t s = NULL;
  if (hipMalloc(&blob_d, (size_t)d.blob_bytes) != hipSuccess || hipMalloc(&x_d, (size_t)B * K * 2) != hipSuccess ||
      hipMalloc(&y_d, (size_t)B * N * 2) != hipSuccess || hipStreamCreate(&s) != hipSuccess)
    return fail("hipMalloc / hipStreamCreate", SGEMV_EHIP);
  if (hipMemcpy(blob_d, blob, (size_t)d.blob_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(x_d, x, (size_t)B * K * 2, hipMemcpyHostToDevice) != hipSuccess)
    return fail("hipMemcpy to the device", SGEMV_EHIP);
  uint16_t* outs[2] = {y0, y1};
  for (int it = 0; it < 2; ++it) {
    /* a poisoned y first: every element must be written by the call */
    if (hipMemsetAsync(y_d, 0x5A, (size_t)B * N * 2, s) != hipSuccess) return fail("hipMemsetAsync", SGEMV_EHIP);
    rc = sgemv_run(&d, blob_d, x_d, y_d, B, (void*)s);
    if (rc) return fail("sgemv_run", rc);
    if (hipStreamSynchronize(s) != hipSuccess) return fail("hipStreamSynchronize", SGEMV_EHIP);
    if (hipMemcpy(outs[it], y_d, (size_t)B * N * 2, hipMemcpyDeviceToHost) != hipSuccess)
      return fail("hipMemcpy to the host", SGEMV_EHIP);
  }
  if (memcmp(y0, y1, (size_t)B * N * 2) != 0) {
    fprintf(stderr, "sgemv_c_driver: two calls on the same inputs gave different bits\n");
    return 1;
  }
  if (write_file(dir, "y.bin", y0, (size_t)B * N * 2)) return fail("writing y.bin", -100);
  hipStreamDestroy(s);
  hipFree(blob_d);
  hipFree(x_d);
  hipFree(y_d);
  printf("sgemv_c_driver: N=%d K=%d nk=%d B=%d grid=%lld waves=%d\n", N, K, nk, B, (long long)pl.grid, pl.waves);
  return 0;
}

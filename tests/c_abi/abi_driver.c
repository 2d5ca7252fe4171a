/* A plain C program that drives libplr.so through include/plr.h alone (no Python, no
 * torch): it reads its inputs from files, allocates device memory with the HIP
 * runtime, calls the library and writes the outputs back to a file. The GPU test
 * tests/test_gpu_c_abi.py writes the inputs, runs this program as a child process and
 * compares what it wrote with the oracle.
 *
 *   abi_driver reduce <dtype> <W> <bytes_per_src> <notify> <in_prefix> <out_file>
 *       packed -> packed reduce of the W files <in_prefix>.<w>; dtype 0 bf16, 1 f16, 2 f32
 *   abi_driver copy <ag|a2a> <W> <bytes_per_src> <notify> <in_prefix> <out_file>
 *       AllGather (packed -> packed) or AllToAll (scattered -> transposed)
 *   abi_driver copy_v <W> <row_bytes> <in_prefix> <out_file>
 *       rows from <in_prefix>.<w>, destinations (int32) from <in_prefix>.dest.<w>; the
 *       output file holds the packed rows, then counts[W][W] and offsets[W][W] (int64)
 * With notify = 1 the call is notified: the program stores every source's flags with
 * plr_notify first and reads the sticky error word with plr_check afterwards.
 * Exit status 0 on success; otherwise a message on stderr naming the failing call. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "plr.h"

static void die(const char* what, int code) {
  fprintf(stderr, "abi_driver: %s failed: %d (%s)\n", what, code, plr_strerror(code));
  exit(1);
}
#define HIP(call)                                                              \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) {                                                    \
      fprintf(stderr, "abi_driver: %s: %s\n", #call, hipGetErrorString(e_));   \
      exit(1);                                                                 \
    }                                                                          \
  } while (0)
#define PLR(call)                  \
  do {                             \
    int rc_ = (call);              \
    if (rc_ != PLR_OK) die(#call, rc_); \
  } while (0)

static void* read_file(const char* path, size_t* bytes) {
  FILE* f = fopen(path, "rb");
  if (!f) {
    fprintf(stderr, "abi_driver: cannot open %s\n", path);
    exit(1);
  }
  fseek(f, 0, SEEK_END);
  long n = ftell(f);
  fseek(f, 0, SEEK_SET);
  void* p = malloc(n > 0 ? (size_t)n : 1);
  if (n > 0 && fread(p, 1, (size_t)n, f) != (size_t)n) {
    fprintf(stderr, "abi_driver: short read of %s\n", path);
    exit(1);
  }
  fclose(f);
  *bytes = (size_t)n;
  return p;
}

static void* to_device(const void* host, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes ? bytes : 16));
  if (bytes) HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void write_out(FILE* f, const void* dev, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (bytes) HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  if (bytes && fwrite(h, 1, bytes, f) != bytes) {
    fprintf(stderr, "abi_driver: short write\n");
    exit(1);
  }
  free(h);
}

static int layout_call(int is_reduce, int dtype, int kind_a2a, int W, size_t bytes, int notify,
                       const char* prefix, const char* out_path) {
  plr_layout_desc d;
  memset(&d, 0, sizeof d);
  d.op = is_reduce ? PLR_OP_REDUCE : PLR_OP_COPY;
  d.dtype = (plr_dtype)dtype;
  d.world = W;
  d.bytes_per_src = bytes;
  d.in_kind = kind_a2a ? PLR_SCATTERED : PLR_PACKED;
  d.out_kind = kind_a2a ? PLR_TRANSPOSED : PLR_PACKED;
  plr_layout* L = NULL;
  PLR(plr_layout_create(&d, &L));

  const void* srcs[PLR_MAX_WORLD];
  char path[4096];
  for (int w = 0; w < W; ++w) {
    size_t n = 0;
    snprintf(path, sizeof path, "%s.%d", prefix, w);
    void* h = read_file(path, &n);
    if (n != bytes) {
      fprintf(stderr, "abi_driver: %s holds %zu bytes, not %zu\n", path, n, bytes);
      return 1;
    }
    srcs[w] = to_device(h, n);
    free(h);
  }
  const size_t out_bytes = plr_layout_dst_bytes(L);
  void* dst = NULL;
  HIP(hipMalloc(&dst, out_bytes ? out_bytes : 16));
  void* ws = NULL;
  if (notify) {
    const size_t wb = plr_layout_workspace_bytes(L);
    HIP(hipMalloc(&ws, wb));
    HIP(hipMemset(ws, 0, wb));  /* zeroed once, as the header asks */
    PLR(plr_notify(L, -1, ws, NULL));
  }
  if (is_reduce)
    PLR(plr_reduce(L, srcs, dst, ws, NULL));
  else
    PLR(plr_copy(L, srcs, dst, ws, NULL));
  if (notify) PLR(plr_check(L, ws, NULL));
  HIP(hipDeviceSynchronize());

  FILE* f = fopen(out_path, "wb");
  if (!f) return 1;
  write_out(f, dst, out_bytes);
  fclose(f);
  for (int w = 0; w < W; ++w) HIP(hipFree((void*)srcs[w]));
  HIP(hipFree(dst));
  if (ws) HIP(hipFree(ws));
  plr_layout_destroy(L);
  return 0;
}

static int copy_v_call(int W, size_t row_bytes, const char* prefix, const char* out_path) {
  const void* srcs[PLR_MAX_WORLD];
  const int32_t* dests[PLR_MAX_WORLD];
  int64_t rows[PLR_MAX_WORLD], total = 0;
  char path[4096];
  for (int w = 0; w < W; ++w) {
    size_t nb = 0, nd = 0;
    snprintf(path, sizeof path, "%s.%d", prefix, w);
    void* h = read_file(path, &nb);
    snprintf(path, sizeof path, "%s.dest.%d", prefix, w);
    void* hd = read_file(path, &nd);
    rows[w] = (int64_t)(nd / 4);
    if (nb != (size_t)rows[w] * row_bytes) {
      fprintf(stderr, "abi_driver: source %d holds %zu bytes for %lld rows\n", w, nb, (long long)rows[w]);
      return 1;
    }
    srcs[w] = to_device(h, nb);
    dests[w] = (const int32_t*)to_device(hd, nd);
    total += rows[w];
    free(h);
    free(hd);
  }
  const size_t sb = plr_copy_v_scratch_bytes(W, rows);
  if (!sb) die("plr_copy_v_scratch_bytes", PLR_EINVAL);
  void *scratch = NULL, *dst = NULL, *counts = NULL, *offsets = NULL;
  HIP(hipMalloc(&scratch, sb));
  HIP(hipMemset(scratch, 0, sb));
  HIP(hipMalloc(&dst, total ? (size_t)total * row_bytes : 16));
  HIP(hipMalloc(&counts, sizeof(int64_t) * W * W));
  HIP(hipMalloc(&offsets, sizeof(int64_t) * W * W));
  PLR(plr_copy_v(W, srcs, rows, dests, row_bytes, dst, (int64_t*)counts, (int64_t*)offsets, scratch, NULL));
  HIP(hipDeviceSynchronize());
  FILE* f = fopen(out_path, "wb");
  if (!f) return 1;
  write_out(f, dst, (size_t)total * row_bytes);
  write_out(f, counts, sizeof(int64_t) * W * W);
  write_out(f, offsets, sizeof(int64_t) * W * W);
  fclose(f);
  for (int w = 0; w < W; ++w) {
    HIP(hipFree((void*)srcs[w]));
    HIP(hipFree((void*)dests[w]));
  }
  HIP(hipFree(scratch));
  HIP(hipFree(dst));
  HIP(hipFree(counts));
  HIP(hipFree(offsets));
  return 0;
}

int main(int argc, char** argv) {
  fprintf(stderr, "abi_driver: %s\n", plr_version());
  if (argc == 8 && !strcmp(argv[1], "reduce"))
    return layout_call(1, atoi(argv[2]), 0, atoi(argv[3]), strtoull(argv[4], NULL, 10), atoi(argv[5]), argv[6],
                       argv[7]);
  if (argc == 8 && !strcmp(argv[1], "copy"))
    return layout_call(0, 0, !strcmp(argv[2], "a2a"), atoi(argv[3]), strtoull(argv[4], NULL, 10), atoi(argv[5]),
                       argv[6], argv[7]);
  if (argc == 6 && !strcmp(argv[1], "copy_v"))
    return copy_v_call(atoi(argv[2]), strtoull(argv[3], NULL, 10), argv[4], argv[5]);
  fprintf(stderr, "usage: see the header of tests/c_abi/abi_driver.c\n");
  return 2;
}

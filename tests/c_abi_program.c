/* A plain C99 client of libswiglu_bwd.so (test infrastructure): the SwiGLU backward
 * (b -> w -> x, bf16) and the Swish gradient run on device memory this program allocates
 * itself with the HIP runtime's C API, no Python and no torch involved.
 *
 * usage: c_abi_program DIR M K N L
 *   reads  DIR/{x,dy,g,fc,w_g,w_fc,grad,sx}.bin   (raw bf16, row-major)
 *   writes DIR/{dg,dfc,db_g,db_fc,dw_g,dw_fc,dx,gx}.bin
 * Exit status 0 on success; any failing call prints its status string and exits 1. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "swiglu_bwd.h"

static char dir_path[4096];

static void fail(const char* what, const char* why) {
  fprintf(stderr, "c_abi_program: %s: %s\n", what, why);
  exit(1);
}

static void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) fail(what, hipGetErrorString(e));
}

static void check_swg(swg_status s, const char* what) {
  if (s != SWG_OK) fail(what, swg_status_string(s));
}

static void* read_file(const char* name, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s.bin", dir_path, name);
  FILE* f = fopen(path, "rb");
  if (!f) fail(path, "cannot open");
  void* buf = malloc(bytes ? bytes : 1);
  if (!buf) fail(path, "out of host memory");
  if (fread(buf, 1, bytes, f) != bytes) fail(path, "short read");
  fclose(f);
  return buf;
}

static void write_file(const char* name, const void* buf, size_t bytes) {
  char path[4200];
  snprintf(path, sizeof path, "%s/%s.bin", dir_path, name);
  FILE* f = fopen(path, "wb");
  if (!f) fail(path, "cannot create");
  if (fwrite(buf, 1, bytes, f) != bytes) fail(path, "short write");
  fclose(f);
}

/* device copy of DIR/name.bin */
static void* upload(const char* name, size_t bytes) {
  void* host = read_file(name, bytes);
  void* dev = NULL;
  check_hip(hipMalloc(&dev, bytes ? bytes : 1), name);
  check_hip(hipMemcpy(dev, host, bytes, hipMemcpyHostToDevice), name);
  free(host);
  return dev;
}

static void* zeros(size_t bytes) {
  void* dev = NULL;
  check_hip(hipMalloc(&dev, bytes ? bytes : 1), "hipMalloc");
  check_hip(hipMemset(dev, 0, bytes), "hipMemset");
  return dev;
}

static void download(const char* name, const void* dev, size_t bytes) {
  void* host = malloc(bytes ? bytes : 1);
  if (!host) fail(name, "out of host memory");
  check_hip(hipMemcpy(host, dev, bytes, hipMemcpyDeviceToHost), name);
  write_file(name, host, bytes);
  free(host);
}

int main(int argc, char** argv) {
  if (argc != 6) fail("usage", "c_abi_program DIR M K N L");
  snprintf(dir_path, sizeof dir_path, "%s", argv[1]);
  const int64_t M = atoll(argv[2]), K = atoll(argv[3]), N = atoll(argv[4]), L = atoll(argv[5]);
  const size_t es = 2; /* bf16 */
  const size_t mk = (size_t)(M * K) * es, mn = (size_t)(M * N) * es, kn = (size_t)(K * N) * es;

  void* x = upload("x", mk);
  void* dy = upload("dy", mn);
  void* g = upload("g", mn);
  void* fc = upload("fc", mn);
  void* w_g = upload("w_g", kn);
  void* w_fc = upload("w_fc", kn);
  void* grad = upload("grad", (size_t)L * es);
  void* sx = upload("sx", (size_t)L * es);

  void* dg = zeros(mn);
  void* dfc = zeros(mn);
  void* db_g = zeros((size_t)N * es);   /* db and dW accumulate: start from zero */
  void* db_fc = zeros((size_t)N * es);
  void* dw_g = zeros(kn);
  void* dw_fc = zeros(kn);
  void* dx = zeros(mk);
  void* gx = zeros((size_t)L * es);

  const size_t ws_b_bytes = swiglu_bwd_b_workspace_size(M, N, SWG_BF16);
  const size_t ws_w_bytes = swiglu_bwd_w_workspace_size(M, K, N, SWG_BF16);
  void* ws_b = zeros(ws_b_bytes);
  void* ws_w = zeros(ws_w_bytes);

  check_swg(swiglu_bwd_b(dy, g, fc, dg, dfc, db_g, db_fc, M, N, SWG_BF16, ws_b, ws_b_bytes,
                         NULL),
            "swiglu_bwd_b");
  check_swg(swiglu_bwd_w(x, dg, dfc, dw_g, dw_fc, M, K, N, SWG_BF16, ws_w, ws_w_bytes, NULL),
            "swiglu_bwd_w");
  check_swg(swiglu_bwd_x(dg, dfc, w_g, w_fc, dx, M, K, N, SWG_BF16, NULL), "swiglu_bwd_x");
  const float beta = 1.702f;
  check_swg(swish_grad(grad, sx, gx, L, SWG_BF16, &beta, NULL), "swish_grad");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");

  download("dg", dg, mn);
  download("dfc", dfc, mn);
  download("db_g", db_g, (size_t)N * es);
  download("db_fc", db_fc, (size_t)N * es);
  download("dw_g", dw_g, kn);
  download("dw_fc", dw_fc, kn);
  download("dx", dx, mk);
  download("gx", gx, (size_t)L * es);

  void* bufs[] = {x, dy, g, fc, w_g, w_fc, grad, sx, dg, dfc, db_g, db_fc,
                  dw_g, dw_fc, dx, gx, ws_b, ws_w};
  for (size_t i = 0; i < sizeof bufs / sizeof bufs[0]; ++i) check_hip(hipFree(bufs[i]), "hipFree");
  printf("c_abi_program ok: %s\n", swg_version());
  return 0;
}

/* One MoE layer forward through the C ABI alone (include/moe.h), from a C
 * program with no Python in the process: device buffers from hipMalloc,
 * plain pointers and sizes, every call's status checked.
 *
 *   c_abi_layer DIR T d E G M k f route_scale
 *
 * Reads, as raw little-endian arrays in DIR:
 *   x.bin    [T, d] BF16        wg.bin  [E, d] BF16        bias.bin [E] FP32
 *   w13.bin  [E+1, 2f, d] BF16 (gate rows, then up rows)  w2.bin [E+1, d, f] BF16
 * and writes idx.bin [T, k] int32, w.bin [T, k] FP32, out.bin [T, d] BF16.
 *
 * The steps are the layer's: the 128x128 weight quantisation (offline in a
 * deployed layer), routing, the 1x128 activation quantisation, the
 * permutation with the FP8 rows copied into grouped order, both expert GEMMs
 * in one call, and the combine with the shared expert. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "moe.h"

static void die(const char* what) {
  fprintf(stderr, "c_abi_layer: %s\n", what);
  exit(1);
}

static void check_hip(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "c_abi_layer: %s: %s\n", what, hipGetErrorString(e));
    exit(1);
  }
}

static void check(moe_status s, const char* what) {
  if (s != MOE_OK) {
    fprintf(stderr, "c_abi_layer: %s: %s (%s)\n", what, moe_status_string(s), moe_last_error());
    exit(1);
  }
}

static void* read_file(const char* dir, const char* name, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "rb");
  if (!f) die(path);
  void* p = malloc(bytes ? bytes : 1);
  if (!p) die("host allocation");
  if (fread(p, 1, bytes, f) != bytes) die(path);
  fclose(f);
  return p;
}

static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
  char path[4096];
  snprintf(path, sizeof path, "%s/%s", dir, name);
  FILE* f = fopen(path, "wb");
  if (!f) die(path);
  if (fwrite(p, 1, bytes, f) != bytes) die(path);
  fclose(f);
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  check_hip(hipMalloc(&p, bytes ? bytes : 16), "hipMalloc");
  return p;
}

static void* dev_from_file(const char* dir, const char* name, size_t bytes) {
  void* h = read_file(dir, name, bytes);
  void* d = dev_alloc(bytes);
  check_hip(hipMemcpy(d, h, bytes, hipMemcpyHostToDevice), name);
  free(h);
  return d;
}

static void to_file(const char* dir, const char* name, const void* d, size_t bytes) {
  void* h = malloc(bytes ? bytes : 1);
  if (!h) die("host allocation");
  check_hip(hipMemcpy(h, d, bytes, hipMemcpyDeviceToHost), name);
  write_file(dir, name, h, bytes);
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 10) die("usage: c_abi_layer DIR T d E G M k f route_scale");
  const char* dir = argv[1];
  const int T = atoi(argv[2]), d = atoi(argv[3]), E = atoi(argv[4]), G = atoi(argv[5]);
  const int M = atoi(argv[6]), k = atoi(argv[7]), f = atoi(argv[8]);
  const float rho = (float)atof(argv[9]);
  if (T < 1 || d < 128 || E < 1 || G < 1 || M < 1 || k < 1 || f < 128) die("bad shape");
  const size_t rows = (size_t)T * k + T, ng = (size_t)E + 1;

  uint16_t* x = dev_from_file(dir, "x.bin", (size_t)T * d * 2);
  uint16_t* wg = dev_from_file(dir, "wg.bin", (size_t)E * d * 2);
  float* bias = dev_from_file(dir, "bias.bin", (size_t)E * 4);
  uint16_t* w13 = dev_from_file(dir, "w13.bin", ng * 2 * f * d * 2);
  uint16_t* w2 = dev_from_file(dir, "w2.bin", ng * d * f * 2);

  /* 128x128 weight quantisation: the stacked matrices in one call each */
  uint8_t* w13q = dev_alloc(ng * 2 * f * d);
  float* w13s = dev_alloc(ng * (2 * f / 128) * (d / 128) * 4);
  uint8_t* w2q = dev_alloc(ng * d * f);
  float* w2s = dev_alloc(ng * (d / 128) * (f / 128) * 4);
  check(fp8_quant_128x128(w13, (int)(ng * 2 * f), d, w13q, w13s, NULL), "fp8_quant_128x128 (w13)");
  check(fp8_quant_128x128(w2, (int)(ng * d), f, w2q, w2s, NULL), "fp8_quant_128x128 (w2)");

  /* routing */
  int32_t* idx = dev_alloc((size_t)T * k * 4);
  float* w = dev_alloc((size_t)T * k * 4);
  moe_route_params p = {E, G, M, k, rho};
  check(moe_route(x, wg, bias, T, d, p, idx, w, NULL), "moe_route");

  /* 1x128 activation quantisation */
  uint8_t* xq = dev_alloc((size_t)T * d);
  float* xs = dev_alloc((size_t)T * (d / 128) * 4);
  check(fp8_quant_1x128(x, T, d, xq, xs, NULL), "fp8_quant_1x128");

  /* permutation, with the FP8 rows copied into grouped order */
  int32_t* offsets = dev_alloc((ng + 1) * 4);
  int32_t* pos = dev_alloc((size_t)T * k * 4);
  int32_t* row_token = dev_alloc(rows * 4);
  uint8_t* xq_perm = dev_alloc(rows * d);
  float* xs_perm = dev_alloc(rows * (d / 128) * 4);
  const size_t ws_bytes = moe_permute_workspace_bytes(T, k, E);
  void* ws = dev_alloc(ws_bytes);
  check(moe_permute(idx, T, k, E, xq, xs, d, offsets, pos, row_token, xq_perm, xs_perm, ws, ws_bytes, NULL),
        "moe_permute");

  /* both expert GEMMs (routed experts, then the shared one over all tokens) */
  uint8_t* h = dev_alloc(rows * f);
  float* hs = dev_alloc(rows * (f / 128) * 4);
  uint16_t* y = dev_alloc(rows * d * 2);
  check(grouped_gemm_fp8_swiglu(xq_perm, xs_perm, (int)rows, NULL, offsets, (int)ng, (int)rows, d, f, w13q,
                                w13s, w2q, w2s, h, hs, y, NULL),
        "grouped_gemm_fp8_swiglu");

  /* combine: gate-weighted routed rows plus the shared expert's row */
  uint16_t* out = dev_alloc((size_t)T * d * 2);
  check(moe_combine(y, pos, w, T, k, d, (int32_t)(T * k), NULL, out, NULL), "moe_combine");
  check_hip(hipDeviceSynchronize(), "hipDeviceSynchronize");

  to_file(dir, "idx.bin", idx, (size_t)T * k * 4);
  to_file(dir, "w.bin", w, (size_t)T * k * 4);
  to_file(dir, "out.bin", out, (size_t)T * d * 2);
  printf("c_abi_layer: T=%d d=%d E=%d G=%d M=%d k=%d f=%d done\n", T, d, E, G, M, k, f);
  return 0;
}

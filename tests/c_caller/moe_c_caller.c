/*
 * A plain C caller of libmoe_mi355x.so: it reads one BF16 problem's inputs from a file,
 * allocates its own device buffers with hipMalloc, runs moe_forward and moe_backward
 * through the C ABI (include/moe.h) on the null stream, and writes the outputs to a
 * second file.  It does no arithmetic of its own: the test that runs it writes the
 * inputs (from the seeded generator) and checks the outputs.
 *
 *   moe_c_caller INPUTS OUTPUTS
 *
 * INPUTS:  int64 T, H, E, K, I; then x bf16 [T][H]; probs f32 [T][E]; routing_map u8
 *          [T][E]; shared gate, up bf16 [I][H], shared down [H][I]; routed gate, up bf16
 *          [E][I][H], routed down [E][H][I]; grad_out bf16 [T][H]; and the six FP32
 *          main_grad start values in the same order and shapes as the weights.
 * OUTPUTS: int32 forward status, backward status, device status word; out bf16 [T][H];
 *          grad_hidden bf16 [T][H]; grad_probs f32 [T][E]; the six FP32 main_grads.
 * Exit status 0 when both calls return MOE_OK, 1 on a library error, 2 on an I/O or HIP
 * error.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

#define NBUF 16

static void* g_host[NBUF];
static void* g_dev[NBUF];

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "moe_c_caller: %s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

/* Buffer i: n bytes on the host, read from f when f is not NULL, and copied to a fresh
   device allocation (at least 256 bytes, so a zero-sized request still gets a pointer). */
static int load(int i, FILE* f, size_t n) {
  g_host[i] = malloc(n ? n : 1);
  if (!g_host[i]) return 0;
  memset(g_host[i], 0, n ? n : 1);
  if (f && n && fread(g_host[i], 1, n, f) != n) {
    fprintf(stderr, "moe_c_caller: short read (buffer %d, %zu bytes)\n", i, n);
    return 0;
  }
  if (!hip_ok(hipMalloc(&g_dev[i], n > 256 ? n : 256), "hipMalloc")) return 0;
  return hip_ok(hipMemcpy(g_dev[i], g_host[i], n, hipMemcpyHostToDevice), "hipMemcpy to device");
}

static int store(int i, FILE* f, size_t n) {
  if (!hip_ok(hipMemcpy(g_host[i], g_dev[i], n, hipMemcpyDeviceToHost), "hipMemcpy to host")) return 0;
  return fwrite(g_host[i], 1, n, f) == n;
}

static moe_weight bf16_weight(void* base, int64_t rows, int64_t cols, int64_t experts) {
  moe_weight w;
  memset(&w, 0, sizeof w);
  w.dtype = MOE_BF16;
  w.rows = rows;
  w.cols = cols;
  w.data.base = base;
  w.data.expert_stride = experts > 1 ? rows * cols : 0;
  w.data.ld = cols;
  return w;
}

static moe_grad fp32_grad(void* base, int64_t rows, int64_t cols) {
  moe_grad g;
  memset(&g, 0, sizeof g);
  g.base = base;
  g.expert_stride = rows * cols;
  g.ld = cols;
  g.dtype = MOE_FP32;
  return g;
}

enum { X, PROBS, MAP, SG, SU, SD, RG, RU, RD, DY, OUT, DX, DPROBS, SAVED, WSF, WSB };

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s INPUTS OUTPUTS\n", argv[0]);
    return 2;
  }
  FILE* fi = fopen(argv[1], "rb");
  if (!fi) {
    perror("moe_c_caller: inputs");
    return 2;
  }
  int64_t hdr[5];
  if (fread(hdr, sizeof hdr, 1, fi) != 1) {
    fprintf(stderr, "moe_c_caller: no header\n");
    return 2;
  }
  const int64_t T = hdr[0], H = hdr[1], E = hdr[2], K = hdr[3], I = hdr[4];
  if (T < 0 || H <= 0 || E <= 0 || K <= 0 || I <= 0 || T > (1 << 20) || H > (1 << 16) || I > (1 << 16) ||
      E > 255) {
    fprintf(stderr, "moe_c_caller: header out of range\n");
    return 2;
  }
  const size_t bf = 2, f4 = 4;
  const size_t wsz[6] = {(size_t)(I * H), (size_t)(I * H), (size_t)(H * I),
                         (size_t)(E * I * H), (size_t)(E * I * H), (size_t)(E * H * I)};
  void* mg_dev[6] = {0};
  void* mg_host[6] = {0};
  int ok = load(X, fi, T * H * bf) && load(PROBS, fi, T * E * f4) && load(MAP, fi, (size_t)(T * E));
  for (int i = 0; ok && i < 6; ++i) ok = load(SG + i, fi, wsz[i] * bf);
  ok = ok && load(DY, fi, T * H * bf);
  for (int i = 0; ok && i < 6; ++i) {
    mg_host[i] = malloc(wsz[i] * f4);
    ok = mg_host[i] && fread(mg_host[i], f4, wsz[i], fi) == wsz[i] &&
         hip_ok(hipMalloc(&mg_dev[i], wsz[i] * f4), "hipMalloc") &&
         hip_ok(hipMemcpy(mg_dev[i], mg_host[i], wsz[i] * f4, hipMemcpyHostToDevice), "hipMemcpy to device");
  }
  fclose(fi);
  if (!ok) return 2;

  moe_problem p;
  memset(&p, 0, sizeof p);
  p.tokens = T;
  p.hidden = H;
  p.intermediate = I;
  p.experts = (int32_t)E;
  p.topk = (int32_t)K;
  p.routed_dtype = MOE_BF16;
  p.flags = MOE_FLAG_HAS_SHARED;
  p.swiglu_limit = 0.0f;

  moe_weights w;
  memset(&w, 0, sizeof w);
  w.shared_gate = bf16_weight(g_dev[SG], I, H, 1);
  w.shared_up = bf16_weight(g_dev[SU], I, H, 1);
  w.shared_down = bf16_weight(g_dev[SD], H, I, 1);
  w.routed_gate = bf16_weight(g_dev[RG], I, H, E);
  w.routed_up = bf16_weight(g_dev[RU], I, H, E);
  w.routed_down = bf16_weight(g_dev[RD], H, I, E);

  moe_main_grads mg;
  memset(&mg, 0, sizeof mg);
  mg.shared_gate = fp32_grad(mg_dev[0], I, H);
  mg.shared_up = fp32_grad(mg_dev[1], I, H);
  mg.shared_down = fp32_grad(mg_dev[2], H, I);
  mg.routed_gate = fp32_grad(mg_dev[3], I, H);
  mg.routed_up = fp32_grad(mg_dev[4], I, H);
  mg.routed_down = fp32_grad(mg_dev[5], H, I);

  const size_t saved_b = moe_saved_bytes(&p);
  const size_t wsf_b = moe_workspace_bytes(&p, 0), wsb_b = moe_workspace_bytes(&p, 1);
  if (saved_b == 0) {
    fprintf(stderr, "moe_c_caller: moe_saved_bytes rejected the problem\n");
    return 1;
  }
  ok = load(OUT, NULL, T * H * bf) && load(DX, NULL, T * H * bf) && load(DPROBS, NULL, T * E * f4) &&
       load(SAVED, NULL, saved_b) && load(WSF, NULL, wsf_b) && load(WSB, NULL, wsb_b);
  if (!ok) return 2;

  const moe_status sf = moe_forward(&p, g_dev[X], (const float*)g_dev[PROBS], (const uint8_t*)g_dev[MAP], &w,
                                    g_dev[OUT], g_dev[SAVED], g_dev[WSF], wsf_b > 256 ? wsf_b : 256, NULL);
  moe_status sb = MOE_ERR_UNSUPPORTED;
  if (sf == MOE_OK)
    sb = moe_backward(&p, g_dev[DY], g_dev[X], &w, g_dev[SAVED], g_dev[DX], (float*)g_dev[DPROBS], &mg,
                      g_dev[WSB], wsb_b > 256 ? wsb_b : 256, NULL);
  if (!hip_ok(hipDeviceSynchronize(), "hipDeviceSynchronize")) return 2;
  if (sf != MOE_OK || sb != MOE_OK)
    fprintf(stderr, "moe_c_caller: forward %s, backward %s\n", moe_status_str(sf), moe_status_str(sb));

  moe_saved_layout lay;
  int32_t word = -1;
  if (moe_saved_view(&p, &lay) == MOE_OK &&
      !hip_ok(hipMemcpy(&word, (const char*)g_dev[SAVED] + lay.status_word, sizeof word, hipMemcpyDeviceToHost),
              "hipMemcpy status word"))
    return 2;

  FILE* fo = fopen(argv[2], "wb");
  if (!fo) {
    perror("moe_c_caller: outputs");
    return 2;
  }
  const int32_t st[3] = {(int32_t)sf, (int32_t)sb, word};
  ok = fwrite(st, sizeof st, 1, fo) == 1 && store(OUT, fo, T * H * bf) && store(DX, fo, T * H * bf) &&
       store(DPROBS, fo, T * E * f4);
  for (int i = 0; ok && i < 6; ++i)
    ok = hip_ok(hipMemcpy(mg_host[i], mg_dev[i], wsz[i] * f4, hipMemcpyDeviceToHost), "hipMemcpy to host") &&
         fwrite(mg_host[i], f4, wsz[i], fo) == wsz[i];
  fclose(fo);

  for (int i = 0; i < NBUF; ++i) {
    if (g_dev[i]) hipFree(g_dev[i]);
    free(g_host[i]);
  }
  for (int i = 0; i < 6; ++i) {
    if (mg_dev[i]) hipFree(mg_dev[i]);
    free(mg_host[i]);
  }
  if (!ok) return 2;
  return (sf == MOE_OK && sb == MOE_OK) ? 0 : 1;
}

/* A plain C client of libdcn4.so: no PyTorch, only the C ABI and the HIP
 * runtime for device memory.  Runs one forward pass of a small bf16 problem
 * whose exact result is known (integer offsets and one-hot weights make the
 * output a shifted copy of the input, zero where the shift leaves the image),
 * then the backward pass of the same problem, whose grad_x is grad_y shifted
 * back (one term per element, exact), through dcn4_backward (which allocates
 * its workspace) and dcn4_backward_ws (a workspace from hipMalloc); prints
 * "OK" or the first mismatch.  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "dcn4.h"

static uint16_t bf16(float f) { /* exact for the small integers used here */
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

int main(void) {
  const int N = 2, H = 9, W = 11, C = 32, G = 2, K = 9, D = C / G;
  dcn4_desc d = {N, H, W, C, G, 3, 3, 1, 1, 1, 1, 1, 1, 1.0f, 0, DCN4_BF16};
  dcn4_plan* plan = NULL;
  dcn4_status st = dcn4_create(&d, &plan);
  if (st != DCN4_OK) { printf("create: %s\n", dcn4_last_error()); return 1; }
  int32_t Ho, Wo;
  uint64_t ideal;
  dcn4_query(plan, &Ho, &Wo, &ideal);
  const size_t nx = (size_t)N * H * W * C, ny = (size_t)N * Ho * Wo * C;
  const size_t nom = (size_t)N * Ho * Wo * G * 3 * K;
  uint16_t* hx = malloc(nx * 2);
  uint16_t* hom = malloc(nom * 2);
  uint16_t* hy = malloc(ny * 2);
  for (size_t i = 0; i < nx; ++i) hx[i] = bf16((float)((int)(i % 97) - 48));
  /* group g: point k = 4 + g (i = 1, j = 1 + g... ) with offset (dx, dy) */
  for (size_t p = 0; p < (size_t)N * Ho * Wo; ++p)
    for (int g = 0; g < G; ++g) {
      uint16_t* row = hom + (p * G + g) * 3 * K;
      for (int k = 0; k < 3 * K; ++k) row[k] = 0;
      const int kk = g == 0 ? 4 : 2;                  /* centre tap / (0,2) */
      row[2 * kk] = bf16(g == 0 ? 1.0f : -2.0f);      /* dx */
      row[2 * kk + 1] = bf16(g == 0 ? 2.0f : 1.0f);   /* dy */
      row[2 * K + kk] = bf16(1.0f);                   /* m  */
    }
  void *dx, *dom, *dy;
  if (hipMalloc(&dx, nx * 2) || hipMalloc(&dom, nom * 2) || hipMalloc(&dy, ny * 2)) {
    printf("hipMalloc failed\n");
    return 1;
  }
  hipMemcpy(dx, hx, nx * 2, hipMemcpyHostToDevice);
  hipMemcpy(dom, hom, nom * 2, hipMemcpyHostToDevice);
  st = dcn4_forward(plan, dx, dom, NULL, dy, NULL);
  if (st != DCN4_OK) { printf("forward: %s\n", dcn4_last_error()); return 1; }
  if (hipDeviceSynchronize() != hipSuccess) { printf("sync failed\n"); return 1; }
  hipMemcpy(hy, dy, ny * 2, hipMemcpyDeviceToHost);
  for (int n = 0; n < N; ++n)
    for (int yo = 0; yo < Ho; ++yo)
      for (int xo = 0; xo < Wo; ++xo)
        for (int c = 0; c < C; ++c) {
          const int g = c / D;
          /* tap (1,1) + (1,2) for group 0; tap (0,2) + (-2,1) for group 1 */
          const int r = g == 0 ? yo - 1 + 1 + 2 : yo - 1 + 0 + 1;
          const int q = g == 0 ? xo - 1 + 1 + 1 : xo - 1 + 2 - 2;
          uint16_t want = 0;
          if (r >= 0 && r < H && q >= 0 && q < W)
            want = hx[(((size_t)n * H + r) * W + q) * C + c];
          const uint16_t got = hy[(((size_t)n * Ho + yo) * Wo + xo) * C + c];
          if (got != want && !((got & 0x7fff) == 0 && (want & 0x7fff) == 0)) {
            printf("mismatch n=%d y=%d x=%d c=%d got %04x want %04x\n", n, yo, xo, c, got, want);
            return 1;
          }
        }
  /* backward: grad_x[n, r, q, c] = grad_y at the output pixel whose sample
   * of weight 1 lands on (r, q), 0 where no output pixel does */
  uint16_t* hg = malloc(ny * 2);
  float* hgx = malloc(nx * 4);
  for (size_t i = 0; i < ny; ++i) hg[i] = bf16((float)((int)(i % 13) - 6));
  void *dg, *dgx, *ws;
  uint64_t wsb = 0;
  if (dcn4_backward_workspace_size(plan, &wsb) != DCN4_OK || wsb == 0) {
    printf("workspace size: %s\n", dcn4_last_error());
    return 1;
  }
  if (hipMalloc(&dg, ny * 2) || hipMalloc(&dgx, nx * 4) || hipMalloc(&ws, wsb)) {
    printf("hipMalloc failed\n");
    return 1;
  }
  hipMemcpy(dg, hg, ny * 2, hipMemcpyHostToDevice);
  for (int pass = 0; pass < 2; ++pass) {
    hipMemset(dgx, 0xff, nx * 4); /* NaN: every element must be written */
    st = pass == 0 ? dcn4_backward(plan, dx, dom, NULL, NULL, dg, (float*)dgx, NULL, NULL)
                   : dcn4_backward_ws(plan, dx, dom, NULL, NULL, dg, (float*)dgx, NULL, ws, wsb,
                                      NULL);
    if (st != DCN4_OK) { printf("backward pass %d: %s\n", pass, dcn4_last_error()); return 1; }
    if (hipDeviceSynchronize() != hipSuccess) { printf("sync failed\n"); return 1; }
    hipMemcpy(hgx, dgx, nx * 4, hipMemcpyDeviceToHost);
    for (int n = 0; n < N; ++n)
      for (int r = 0; r < H; ++r)
        for (int q = 0; q < W; ++q)
          for (int c = 0; c < C; ++c) {
            const int g = c / D;
            const int yo = g == 0 ? r - 2 : r, xo = g == 0 ? q - 1 : q + 1;
            float want = 0.0f;
            if (yo >= 0 && yo < Ho && xo >= 0 && xo < Wo) {
              const uint32_t u = (uint32_t)hg[(((size_t)n * Ho + yo) * Wo + xo) * C + c] << 16;
              memcpy(&want, &u, 4);
            }
            const float got = hgx[(((size_t)n * H + r) * W + q) * C + c];
            if (got != want) {
              printf("backward pass %d mismatch n=%d y=%d x=%d c=%d got %g want %g\n", pass, n, r,
                     q, c, got, want);
              return 1;
            }
          }
  }
  dcn4_destroy(plan);
  hipFree(dx);
  hipFree(dom);
  hipFree(dy);
  hipFree(dg);
  hipFree(dgx);
  hipFree(ws);
  free(hx);
  free(hom);
  free(hy);
  free(hg);
  free(hgx);
  printf("OK\n");
  return 0;
}

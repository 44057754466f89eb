/* validate_timing.c: time the library's host-side argument checks alone.
 *
 * [Qiaomu] 基础设施优化 (TileLang内核开发) and [kwkr] §4.2 report that moving a kernel call's host
 * checks into generated code cut them from tens or hundreds of microseconds to
 * under one. Here the checks are plain compiled C in liblca.so. This program
 * calls each hot-path entry point many times with arguments that pass every
 * check except the last one (a workspace one byte too small, or a static
 * scratch request beyond its size), so the whole validation and the split-plan
 * arithmetic run and nothing is launched: no GPU is touched. It prints one
 * line per entry point with the mean nanoseconds per call.
 *
 * Build: gcc -O2 validate_timing.c -I../../include -L.. -llca -o validate_timing
 * Run:   LD_LIBRARY_PATH=.. ./validate_timing [iterations]
 */
#define _POSIX_C_SOURCE 199309L
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <time.h>

#include "lca.h"

static double now_ns(void) {
  struct timespec ts;
  clock_gettime(CLOCK_MONOTONIC, &ts);
  return (double)ts.tv_sec * 1e9 + (double)ts.tv_nsec;
}

int main(int argc, char** argv) {
  const long n = argc > 1 ? atol(argv[1]) : 200000;
  /* aligned addresses that the checks accept and nothing ever dereferences */
  void* p = (void*)(uintptr_t)0x10000;
  float* f = (float*)p;
  int32_t* ix = (int32_t*)p;
  /* the CSA decode step: B = 16 at 131072 tokens, H = 64, D = 512, k = 512 */
  const int B = 16, H = 64, D = 512, m = 4, k = 512, W = 128, HI = 4, dI = 128;
  const int64_t pos = 131072, N = 32768;
  const size_t ws_i = csa_index_topk_workspace(LCA_BF16, B, 1, HI, dI, N, m, k, pos, 0);
  const size_t ws_a = csa_attend_workspace(LCA_BF16, LCA_BF16, B, 1, H, D, N, m, k, W, pos);
  const size_t ws_h = hca_attend_workspace(LCA_BF16, LCA_BF16, 8, 1, 128, D, 8192, 128, W, 1048576);
  int st = 0;
  double t0 = now_ns();
  for (long i = 0; i < n; ++i)
    st |= csa_index_topk(NULL, LCA_BF16, B, 1, HI, dI, N, m, k, pos, p, NULL, f, p, NULL, 0, ix, NULL, p, ws_i - 1);
  double t1 = now_ns();
  for (long i = 0; i < n; ++i)
    st |= csa_attend(NULL, LCA_BF16, LCA_BF16, B, 1, H, D, N, m, k, W, pos, p, p, NULL, ix, p, NULL, f, 0.04f,
                     LCA_INV_ROPE, 10000.f, 64, p, f, p, ws_a - 1);
  double t2 = now_ns();
  for (long i = 0; i < n; ++i)
    st |= hca_attend(NULL, LCA_BF16, LCA_BF16, 8, 1, 128, D, 8192, 128, W, 1048576, p, p, NULL, p, NULL, f, 0.04f,
                     LCA_INV_ROPE, 10000.f, 64, p, f, p, ws_h - 1);
  double t3 = now_ns();
  /* 64 sequences: beyond the static scratch of csa_attend_noalloc */
  for (long i = 0; i < n; ++i)
    st |= csa_attend_noalloc(NULL, LCA_BF16, LCA_BF16, 64, 1, H, D, N, m, k, W, pos, p, p, NULL, ix, p, NULL, f,
                             0.04f, LCA_INV_ROPE, 10000.f, 64, p, f);
  double t4 = now_ns();
  if (st != LCA_ERR_WORKSPACE) {
    fprintf(stderr, "unexpected status %d: %s\n", st, lca_last_error());
    return 1;
  }
  printf("csa_index_topk %.1f ns\n", (t1 - t0) / n);
  printf("csa_attend %.1f ns\n", (t2 - t1) / n);
  printf("hca_attend %.1f ns\n", (t3 - t2) / n);
  printf("csa_attend_noalloc %.1f ns\n", (t4 - t3) / n);
  return 0;
}

// Host-side driver for the ASan/UBSan build of the library: sweeps the
// workspace planners over many shapes (ragged, tiny, at and past every
// limit) and calls every entry point with invalid arguments.  Each call must
// return its documented error before any HIP call is made, so the whole
// driver runs without a GPU.  Exit status 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "lmce.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main() {
  // aligned, non-null addresses that are never dereferenced
  void* F = reinterpret_cast<void*>(uintptr_t(1) << 20);
  char* Fc = static_cast<char*>(F);
  const int64_t* Fl = reinterpret_cast<const int64_t*>(F);
  float* Ff = static_cast<float*>(F);
  size_t n = 0;

  // planners over a sweep of shapes
  const int64_t Ls[] = {1, 2, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000, 8192, 131072, 163840, (1 << 21) - 1,
                        1 << 21, (1 << 21) + 1, 0, -1};
  const int64_t Hs[] = {64, 128, 256, 384, 1024, 2560, 3072, 4096, 5120, 16384, 16512, 100, 0};
  const int64_t Vs[] = {1, 2, 255, 256, 257, 4096, 151936, (1 << 21), (1 << 21) + 1, 0};
  const int64_t Cs[] = {1, 31, 32, 96, 256, 1024, 1056, 4096, 4097, 0};
  int ok = 0;
  for (int64_t L : Ls)
    for (int64_t H : Hs)
      for (int64_t V : Vs)
        for (int64_t c : Cs) {
          int st = lmce_workspace_size(L, H, V, c, &n);
          if (st == LMCE_OK) {
            ++ok;
            CHECK(n > 0);
            CHECK(n % 256 == 0);
          }
          st = lmce_chunked_workspace_size(L, H, V, c, &n);
          if (st == LMCE_OK) CHECK(n > 0);
        }
  CHECK(ok > 100);
  const int64_t Is[] = {64, 768, 9728, 25600, 65536, 65600, 32, 0};
  for (int64_t L : Ls)
    for (int64_t H : Hs)
      for (int64_t I : Is)
        for (int64_t c : {int64_t(1), int64_t(256), int64_t(16384), int64_t(65536), int64_t(65537)}) {
          const int st = lmce_mlp_workspace_size(L, H, I, c, &n);
          if (st == LMCE_OK) CHECK(n > 0);
        }
  CHECK(lmce_workspace_size(512, 256, 4096, 256, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_chunked_workspace_size(512, 256, 4096, 256, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_mlp_workspace_size(512, 256, 768, 256, nullptr) == LMCE_ERR_NULL);

  // every entry point: null, misaligned, out-of-range shapes, short workspace
  CHECK(lmce_fwd(nullptr, F, Fl, 512, 256, 4096, -100, 256, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_fwd(Fc + 2, F, Fl, 512, 256, 4096, -100, 256, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_fwd(F, F, Fl, 0, 256, 4096, -100, 256, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_SHAPE);
  CHECK(lmce_fwd(F, F, Fl, 512, 200, 4096, -100, 256, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_UNSUPPORTED);
  CHECK(lmce_fwd(F, F, Fl, 512, 256, 4096, -100, 256, Ff, Ff, F, 16, nullptr) == LMCE_ERR_WORKSPACE);
  CHECK(lmce_fwd_noalloc(F, F, Fl, (1 << 20) + 1, 256, 4096, -100, 256, Ff, Ff, nullptr) == LMCE_ERR_SCRATCH);
  CHECK(lmce_fwd_noalloc(F, nullptr, Fl, 512, 256, 4096, -100, 256, Ff, Ff, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_bwd(F, F, Fl, Ff, 512, 256, 4096, -100, 256, Ff, Ff, nullptr, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_bwd(F, F, Fl, Ff, 512, 256, 4096, -100, 2048, Ff, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_UNSUPPORTED);
  CHECK(lmce_bwd_dh(F, F, Fl, Ff, 512, 256, 4096, -100, 256, Ff, nullptr, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_bwd_dW(F, F, Fl, Ff, 512, 256, 4096, -100, 256, Ff, Ff, F, 16, nullptr) == LMCE_ERR_WORKSPACE);
  CHECK(lmce_fwd_train(F, F, Fl, 512, 256, 4096, -100, 256, Ff, Ff, nullptr, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_bwd_train(F, F, Fl, Ff, -3, 256, 4096, -100, 256, Ff, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_SHAPE);
  CHECK(lmce_chunked_fwd(F, F, Fl, 512, 256, 4096, -100, 0, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_UNSUPPORTED);
  CHECK(lmce_chunked_bwd(F, F, Fl, 512, 256, 4096, -100, 256, Ff, Ff, Ff, F, 16, nullptr) == LMCE_ERR_WORKSPACE);
  CHECK(lmce_mlp_fwd(F, F, F, F, 512, 256, 768, 256, nullptr, F, 1 << 30, nullptr) == LMCE_ERR_NULL);
  CHECK(lmce_mlp_fwd(F, F, F, F, 512, 256, 700, 256, Ff, F, 1 << 30, nullptr) == LMCE_ERR_UNSUPPORTED);
  CHECK(lmce_mlp_bwd(F, F, F, F, F, 512, 256, 768, 256, Ff, Ff, Ff, Ff, F, 16, nullptr) == LMCE_ERR_WORKSPACE);
  CHECK(lmce_mlp_bwd(F, F, F, F, F, 512, 16384, 65536, 256, Ff, Ff, Ff, Ff, F, 1 << 30, nullptr) == LMCE_ERR_UNSUPPORTED);
  CHECK(lmce_read_status(Fc + 4, nullptr) == LMCE_ERR_NULL);
  for (int s = -9; s <= 1; ++s) CHECK(lmce_strerror(s) != nullptr && strlen(lmce_strerror(s)) > 0);
  CHECK(lmce_version() >= 100);

  if (failures) {
    fprintf(stderr, "%d checks failed\n", failures);
    return 1;
  }
  printf("validation driver: all checks passed (%d planned shapes)\n", ok);
  return 0;
}

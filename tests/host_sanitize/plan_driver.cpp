// Host-only driver for the plan code (lm_plan.cpp) under AddressSanitizer
// and UndefinedBehaviorSanitizer: builds plans over every supported
// transform size and option, sets and reads back filterbanks (random, with
// empty and negative rows), feeds invalid arguments, and frees every plan.
// It makes no HIP call; the one HIP symbol the plan code names (the error
// text of a HIP status) is stubbed here.  Exit status 0 when every check
// holds; the sanitizers abort on the first error they find.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "lm_internal.h"

extern "C" const char *hipGetErrorString(hipError_t) { return "(no HIP in this build)"; }

static int g_fail = 0;
#define CHECK(c)                                                   \
  do {                                                             \
    if (!(c)) {                                                    \
      std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++g_fail;                                                    \
    }                                                              \
  } while (0)

static void free_plan(lm_plan *p) { delete p; }   // no device memory was taken

int main() {
  const int sizes[] = {400, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384};
  const int mels[] = {1, 40, 128, 256};
  std::mt19937 rng(12345);
  std::uniform_real_distribution<float> uni(-1.0f, 1.0f);
  int plans = 0;
  for (int n_fft : sizes)
    for (int NM : mels)
      for (int pad_mode = 0; pad_mode < 4; ++pad_mode) {
        const int hop = n_fft == 400 ? (pad_mode & 1 ? 161 : 160) : n_fft / 4;
        lm_plan *p = nullptr;
        const int rc = lm_plan_create(&p, n_fft, hop, NM, pad_mode != 2, pad_mode, pad_mode == 3 ? 1.0f : 2.0f,
                                      pad_mode & 1);
        CHECK(rc == LM_OK && p);
        if (!p) continue;
        ++plans;
        const double sr = n_fft >= 8192 ? 44100.0 : 16000.0;
        CHECK(lm_plan_set_mel(p, sr, 0.0, sr / 2, pad_mode & 1, (pad_mode >> 1) & 1) == LM_OK);
        CHECK(lm_plan_set_mel(p, sr, 300.0, 0.25 * sr, 0, 1) == LM_OK);
        CHECK(lm_plan_set_mel(p, sr, 0.5 * sr, 0.25 * sr, 0, 1) != LM_OK);   // f_min above f_max
        const int NB = n_fft / 2 + 1;
        std::vector<float> dense((size_t)NM * NB), back((size_t)NM * NB);
        for (int m = 0; m < NM; ++m)
          for (int k = 0; k < NB; ++k) {
            float v = 0.0f;
            if (m % 7 == 3) v = 0.0f;                                  // empty rows
            else if ((k + 3 * m) % 11 < 4) v = m % 5 == 1 ? -uni(rng) : std::fabs(uni(rng));
            dense[(size_t)m * NB + k] = v;
          }
        CHECK(lm_plan_set_filters(p, dense.data(), NM, NB) == LM_OK);
        CHECK(lm_plan_get_filters(p, back.data(), NM, NB) == LM_OK);
        for (size_t i = 0; i < dense.size(); ++i) CHECK(back[i] == dense[i]);
        CHECK(lm_plan_set_filters(p, dense.data(), NM, NB + 1) != LM_OK);   // wrong shape
        CHECK(lm_plan_get_filters(p, back.data(), NM + 1, NB) != LM_OK);
        CHECK(lm_plan_set_output(p, LM_OUTPUT_MEL, LM_NORMALIZED_WINDOW) == LM_OK);
        CHECK(lm_plan_set_output(p, 7, 0) != LM_OK);
        CHECK(lm_plan_set_window(p, n_fft / 2) == LM_OK);
        CHECK(lm_plan_set_window(p, n_fft + 1) != LM_OK);
        CHECK(lm_plan_set_pad(p, 17) == LM_OK);
        CHECK(lm_plan_set_pad(p, -1) != LM_OK);
        CHECK(lm_plan_num_frames(p, 100000) > 0);
        CHECK(lm_plan_num_frames(p, -3) < 0);
        CHECK(lm_plan_set_mel(p, sr, 0.0, sr / 2, 1, 0) == LM_OK);   // back to a computed bank
        free_plan(p);
      }
  lm_plan *p = nullptr;
  CHECK(lm_plan_create(&p, 300, 100, 40, 1, 1, 2.0f, 0) != LM_OK && !p);   // unsupported size
  CHECK(lm_plan_create(&p, 512, 0, 40, 1, 1, 2.0f, 0) != LM_OK);           // hop 0
  CHECK(lm_plan_create(&p, 512, 128, 0, 1, 1, 2.0f, 0) != LM_OK);          // no bands
  CHECK(lm_plan_create(nullptr, 512, 128, 40, 1, 1, 2.0f, 0) != LM_OK);
  CHECK(lm_status_string(LM_OK) && lm_status_string(-99));
  std::printf("%d plans, %d failed checks\n", plans, g_fail);
  return g_fail ? 1 : 0;
}

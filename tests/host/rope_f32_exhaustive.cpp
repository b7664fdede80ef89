// The library's single-precision rotary cos/sin (qsa_rope_math.h) on every
// f32 angle it is used for: all non-negative floats below 2^18 (the kernels
// take the double path from 2^18 on, and angles are position * frequency with
// both non-negative).  For each angle: the absolute error of cos and sin
// against double cos/sin of the same angle stays below half the allowance the
// bf16 certificate assumes, and every certified pair rounds to the bf16 of the
// f32 rounding of the double values.  Prints the worst error, the share left
// to the double path and the count of wrong certified values (must be 0).
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <algorithm>
#include <thread>
#include <vector>

#include "../../sparse_attention_token_qsa_amd/csrc/qsa_rope_math.h"

static uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

struct Tally {
  double worst = 0.0;
  long angles = 0, left = 0, wrong = 0;
};

static void sweep(uint32_t lo, uint32_t hi, Tally* t) {
  for (uint32_t bits = lo; bits < hi; ++bits) {
    float a;
    std::memcpy(&a, &bits, 4);
    float c, s;
    qsa::cos_sin_f32(a, c, s);
    const double ce = std::cos(static_cast<double>(a)), se = std::sin(static_cast<double>(a));
    const double e = std::fmax(std::fabs(c - ce), std::fabs(s - se));
    if (e > t->worst) t->worst = e;
    ++t->angles;
    if (!(qsa::bf16_rounding_settled(c, qsa::kTrigSettle) && qsa::bf16_rounding_settled(s, qsa::kTrigSettle))) {
      ++t->left;
      continue;
    }
    if (bf16_rne(c) != bf16_rne(static_cast<float>(ce)) || bf16_rne(s) != bf16_rne(static_cast<float>(se))) ++t->wrong;
  }
}

int main(int argc, char** argv) {
  const float top = 262144.0f;  // 2^18
  uint32_t end;
  std::memcpy(&end, &top, 4);
  const unsigned nt = argc > 1 ? static_cast<unsigned>(std::atoi(argv[1])) : 8u;
  std::vector<Tally> tallies(nt);
  std::vector<std::thread> threads;
  const uint32_t per = (end + nt - 1) / nt;
  for (unsigned i = 0; i < nt; ++i) {
    const uint32_t lo = i * per, hi = std::min<uint32_t>(end, lo + per);
    threads.emplace_back(sweep, lo, hi, &tallies[i]);
  }
  Tally all;
  for (unsigned i = 0; i < nt; ++i) {
    threads[i].join();
    all.worst = std::fmax(all.worst, tallies[i].worst);
    all.angles += tallies[i].angles;
    all.left += tallies[i].left;
    all.wrong += tallies[i].wrong;
  }
  std::printf("angles %ld worst %.3e (2^%.2f) allowance 2^%.2f left-to-double %.4f%% wrong %ld\n", all.angles,
              all.worst, std::log2(all.worst), std::log2(qsa::kTrigSettle), 100.0 * all.left / all.angles, all.wrong);
  return (all.wrong == 0 && all.worst < 0.5 * qsa::kTrigSettle) ? 0 : 1;
}

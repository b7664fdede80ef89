// The f32 rotary cos/sin of the library (qsa_rope_math.h) on every position
// the library accepts, at several rotary tables: its absolute error against
// double cos/sin of the same f32 angle stays below the allowance its bf16
// certificate assumes, and every certified bf16 value equals the bf16
// rounding of the f32 rounding of the double result.  Prints the worst error
// and the share of (cos, sin) pairs left to the double path.
#include <cmath>
#include <cstdio>
#include <cstring>

#include "../../sparse_attention_token_qsa_amd/csrc/qsa_rope_math.h"

static uint16_t bf16_rne(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

int main() {
  const double thetas[] = {1e4, 1e7, 5e5, 123.5};
  const int rds[] = {64, 128, 2, 36};
  double worst = 0.0;
  long pairs = 0, left = 0, wrong = 0;
  for (int t = 0; t < 4; ++t) {
    for (int i = 0; i < rds[t] / 2; ++i) {
      // the library's table: theta^(-2i/rd) in double, rounded once to f32
      const float f = static_cast<float>(std::pow(thetas[t], -(2.0 * i) / rds[t]));
      for (long p = 0; p < 262147; ++p) {
        const float a = static_cast<float>(p) * f;
        if (std::fabs(a) >= 262144.0f) continue;
        float c, s;
        qsa::cos_sin_f32(a, c, s);
        const double ce = std::cos(static_cast<double>(a)), se = std::sin(static_cast<double>(a));
        worst = std::fmax(worst, std::fmax(std::fabs(c - ce), std::fabs(s - se)));
        ++pairs;
        if (!(qsa::bf16_rounding_settled(c, qsa::kTrigSettle) && qsa::bf16_rounding_settled(s, qsa::kTrigSettle))) {
          ++left;
          continue;
        }
        if (bf16_rne(c) != bf16_rne(static_cast<float>(ce)) || bf16_rne(s) != bf16_rne(static_cast<float>(se))) ++wrong;
      }
    }
  }
  std::printf("pairs %ld worst %.3e (2^%.2f) allowance 2^%.2f left-to-double %.4f%% wrong %ld\n", pairs, worst,
              std::log2(worst), std::log2(qsa::kTrigSettle), 100.0 * left / pairs, wrong);
  return (wrong == 0 && worst < 0.5 * qsa::kTrigSettle) ? 0 : 1;
}

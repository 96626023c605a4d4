// Host Adam building blocks (used by sf_adam_host and the sliding engine).
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

namespace sf {

struct AdamCoef {
  float b1, b2, one_b1, one_b2, inv_bc1, inv_bc2, lr, eps;
};

// Bias-correction factors 1/(1 - b^step) evaluated in double.
AdamCoef adam_coef(int64_t step, float lr, float b1, float b2, float eps);

// One Adam step over n elements; pb (may be null) receives bf16(p) (RNE).
void adam_range(float* p, float* m, float* v, const float* g, uint16_t* pb, size_t n, const AdamCoef& c);

int default_threads();

}  // namespace sf

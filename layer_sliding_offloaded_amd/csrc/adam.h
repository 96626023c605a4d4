// Host Adam building blocks (used by sf_adam_host and the sliding engine).
#pragma once

#include <cstddef>
#include <cstdint>
#include <cstring>

namespace sf {

struct AdamCoef {
  float b1, b2, one_b1, one_b2, inv_bc1, inv_bc2, lr, eps;
  float gscale;  // the gradient enters as g * gscale (the inverse loss scale; 1: as is)
};

// Bias-correction factors 1/(1 - b^step) evaluated in double; gscale 1.
AdamCoef adam_coef(int64_t step, float lr, float b1, float b2, float eps);

// One Adam step over n elements; pb (may be null) receives the 16-bit copy of
// p rounded to nearest even: bf16 when out16 == 1, IEEE fp16 when out16 == 2.
void adam_range(float* p, float* m, float* v, const float* g, uint16_t* pb, size_t n, const AdamCoef& c,
                int out16 = 1);

int default_threads();

}  // namespace sf

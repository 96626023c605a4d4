// Deterministic stand-ins for the device work the sliding engine enqueues
// (test infrastructure for tests/engine_cpu).  Each stand-in reads and
// writes exactly the buffers the real operation does, with cheap mixing
// arithmetic in place of the layer mathematics, so that ThreadSanitizer sees
// the real access pattern and any stale or early read changes the result.
// The *_now functions run synchronously; the sequential reference of
// engine_check.cpp calls them directly, the library entry points enqueue
// them on their stream.
#pragma once

#include <cstddef>
#include <cstdint>

#include "internal.h"
#include "rowops.h"

namespace fake {

struct Shape {
  int H, V, T, S, dtype;  // dtype: SF_F32 / SF_BF16 / SF_F16
  size_t e;               // storage bytes per element
  const sf_layout* L;
};

uint32_t hash_bytes(const void* p, size_t bytes, uint32_t seed);
float to_f(int dtype, const void* x, size_t i);
void from_f(int dtype, void* x, size_t i, float v);

void layer_fwd_now(const Shape& s, const void* w, const void* x, void* y, void* saved);
// part 0: Wd's gradient, 1: Wg and Wu's, 2: the rest and dx (in this order)
void layer_bwd_now(const Shape& s, const void* w, const void* x, const void* saved, const void* dy, void* dx,
                   float* dw, int part);
// head: loss, dx, dgf, dW_lm; with defer the last part of dW_lm is left in
// `scratch` (16 floats) for head_last_dw_now to add
void head_now(const Shape& s, const void* gf, const void* wlm, const void* x, const int32_t* ids, float* loss,
              void* dx, float* dgf, float* dwlm, float grad_scale, bool defer, float* scratch);
void head_last_dw_now(const Shape& s, float* dwlm, const float* scratch);
void embed_fwd_now(const Shape& s, const void* E, const int32_t* ids, void* x0);

}  // namespace fake

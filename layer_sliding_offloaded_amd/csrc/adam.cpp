// Host-side Adam over flat fp32 arrays with a fused fp32 -> bf16 / fp16 copy.
//
// The pages put the optimizer on the CPU: while the device runs the backward
// of L_{i-1}, host threads update L_i with optimizer states that live in
// host memory as flattened tensors, and shared buffers carry the FP32 ->
// BF16 conversion (es §2A "Actualizacion Asincrona", es §2B, de §2B, fr §2B).
// One pass reads g, p, m, v and writes p, m, v and the 16-bit copy (about 30
// bytes per parameter of host DRAM traffic), so the loop is written to
// vectorise (AVX2/FMA) and is split across threads in cache-sized chunks.
#include "adam.h"

#include <immintrin.h>
#include <sched.h>

#include <algorithm>
#include <cmath>
#include <thread>
#include <vector>

#include "internal.h"

namespace sf {

namespace {

inline uint16_t f32_to_bf16(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return static_cast<uint16_t>(b >> 16);
}

}  // namespace

AdamCoef adam_coef(int64_t step, float lr, float b1, float b2, float eps) {
  AdamCoef c;
  c.b1 = b1;
  c.b2 = b2;
  c.one_b1 = 1.0f - b1;
  c.one_b2 = 1.0f - b2;
  c.inv_bc1 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(b1), static_cast<double>(step))));
  c.inv_bc2 = static_cast<float>(1.0 / (1.0 - std::pow(static_cast<double>(b2), static_cast<double>(step))));
  c.lr = lr;
  c.eps = eps;
  c.gscale = 1.0f;
  return c;
}

namespace {

// 16 elements with the bf16 copy streamed out (non-temporal: the copy is not
// read again on the host, so it skips the read-for-ownership of its lines).
// Same operations in the same order as the scalar loop (no contraction), so
// the results are bitwise identical.
template <int OUT16>
inline void adam16_stream(float* p, float* m, float* v, const float* g, uint16_t* pb, const AdamCoef& c) {
  const __m256 b1 = _mm256_set1_ps(c.b1), b2 = _mm256_set1_ps(c.b2);
  const __m256 o1 = _mm256_set1_ps(c.one_b1), o2 = _mm256_set1_ps(c.one_b2);
  const __m256 ib1 = _mm256_set1_ps(c.inv_bc1), ib2 = _mm256_set1_ps(c.inv_bc2);
  const __m256 lr = _mm256_set1_ps(c.lr), eps = _mm256_set1_ps(c.eps);
  const __m256 gs = _mm256_set1_ps(c.gscale);
  __m256i bits[2];
  __m128i halves[2];
  for (int h = 0; h < 2; ++h) {
    const __m256 gi = _mm256_mul_ps(_mm256_loadu_ps(g + 8 * h), gs);
    const __m256 mi = _mm256_add_ps(_mm256_mul_ps(b1, _mm256_loadu_ps(m + 8 * h)), _mm256_mul_ps(o1, gi));
    const __m256 vi =
        _mm256_add_ps(_mm256_mul_ps(b2, _mm256_loadu_ps(v + 8 * h)), _mm256_mul_ps(_mm256_mul_ps(o2, gi), gi));
    _mm256_storeu_ps(m + 8 * h, mi);
    _mm256_storeu_ps(v + 8 * h, vi);
    const __m256 num = _mm256_mul_ps(lr, _mm256_mul_ps(mi, ib1));
    const __m256 den = _mm256_add_ps(_mm256_sqrt_ps(_mm256_mul_ps(vi, ib2)), eps);
    const __m256 pi = _mm256_sub_ps(_mm256_loadu_ps(p + 8 * h), _mm256_div_ps(num, den));
    _mm256_storeu_ps(p + 8 * h, pi);
    if constexpr (OUT16 == 1) {
      // bf16, round to nearest even: b + 0x7FFF + ((b >> 16) & 1), keep the high half
      const __m256i b = _mm256_castps_si256(pi);
      const __m256i odd = _mm256_and_si256(_mm256_srli_epi32(b, 16), _mm256_set1_epi32(1));
      bits[h] = _mm256_srli_epi32(_mm256_add_epi32(_mm256_add_epi32(b, _mm256_set1_epi32(0x7FFF)), odd), 16);
    } else {
      // IEEE fp16, round to nearest even (F16C)
      halves[h] = _mm256_cvtps_ph(pi, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    }
  }
  __m256i packed;
  if constexpr (OUT16 == 1) {
    // packus interleaves 128-bit lanes: [a0-3 b0-3 a4-7 b4-7] -> restore element order
    packed = _mm256_permute4x64_epi64(_mm256_packus_epi32(bits[0], bits[1]), 0xD8);
  } else {
    packed = _mm256_set_m128i(halves[1], halves[0]);
  }
  _mm256_stream_si256(reinterpret_cast<__m256i*>(pb), packed);
}

inline uint16_t f32_to_f16(float f) {
  return static_cast<uint16_t>(_cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC));
}

}  // namespace

void adam_range(float* __restrict p, float* __restrict m, float* __restrict v, const float* __restrict g,
                uint16_t* __restrict pb, size_t n, const AdamCoef& c, int out16) {
  const float b1 = c.b1, b2 = c.b2, o1 = c.one_b1, o2 = c.one_b2;
  const float ib1 = c.inv_bc1, ib2 = c.inv_bc2, lr = c.lr, eps = c.eps, gs = c.gscale;
  if (pb) {
    // scalar head up to a 32-byte aligned 16-bit address, 16-element blocks, scalar tail
    size_t i0 = 0;
    while (i0 < n && (reinterpret_cast<uintptr_t>(pb + i0) & 31u)) ++i0;
    size_t i1 = i0 + (n - i0) / 16 * 16;
    if (i1 <= i0) i0 = i1 = n;
    if (out16 == 2) {
      for (size_t i = i0; i < i1; i += 16) adam16_stream<2>(p + i, m + i, v + i, g + i, pb + i, c);
    } else {
      for (size_t i = i0; i < i1; i += 16) adam16_stream<1>(p + i, m + i, v + i, g + i, pb + i, c);
    }
    _mm_sfence();
    auto scalar = [&](size_t a, size_t b) {
      for (size_t i = a; i < b; ++i) {
        const float gi = g[i] * gs;
        const float mi = b1 * m[i] + o1 * gi;
        const float vi = b2 * v[i] + o2 * gi * gi;
        m[i] = mi;
        v[i] = vi;
        const float pi = p[i] - lr * (mi * ib1) / (std::sqrt(vi * ib2) + eps);
        p[i] = pi;
        pb[i] = out16 == 2 ? f32_to_f16(pi) : f32_to_bf16(pi);
      }
    };
    scalar(0, i0);
    scalar(i1, n);
    return;
  }
#pragma GCC ivdep
  for (size_t i = 0; i < n; ++i) {
    const float gi = g[i] * gs;
    const float mi = b1 * m[i] + o1 * gi;
    const float vi = b2 * v[i] + o2 * gi * gi;
    m[i] = mi;
    v[i] = vi;
    p[i] = p[i] - lr * (mi * ib1) / (std::sqrt(vi * ib2) + eps);
  }
}

int default_threads() {
  // the cores this process may run on (a container's share), not the machine's
  cpu_set_t set;
  CPU_ZERO(&set);
  int n = 0;
  if (sched_getaffinity(0, sizeof set, &set) == 0) n = CPU_COUNT(&set);
  if (n <= 0) n = static_cast<int>(std::thread::hardware_concurrency());
  return std::max(1, std::min(n, 64));
}

}  // namespace sf

using namespace sf;

namespace {

sf_status adam_host_impl(float* p, float* m, float* v, const float* g, int out16, uint16_t* p16, size_t n,
                         int64_t step, float lr, float b1, float b2, float eps, float gscale, int32_t n_threads) {
  if (n == 0) return SF_OK;
  if (!p || !m || !v || !g) return fail(SF_ERR_ARG, "NULL array");
  if (step < 1) return fail(SF_ERR_ARG, "step must be >= 1");
  AdamCoef c = adam_coef(step, lr, b1, b2, eps);
  c.gscale = gscale;
  int nt = n_threads > 0 ? n_threads : default_threads();
  const size_t min_chunk = 1 << 16;
  nt = static_cast<int>(std::max<size_t>(1, std::min<size_t>(nt, (n + min_chunk - 1) / min_chunk)));
  if (nt == 1) {
    adam_range(p, m, v, g, p16, n, c, out16);
    return SF_OK;
  }
  std::vector<std::thread> th;
  const size_t per = (n + nt - 1) / nt;
  for (int t = 0; t < nt; ++t) {
    const size_t b = t * per, e = std::min(n, b + per);
    if (b >= e) break;
    th.emplace_back([=, &c] { adam_range(p + b, m + b, v + b, g + b, p16 ? p16 + b : nullptr, e - b, c, out16); });
  }
  for (auto& x : th) x.join();
  return SF_OK;
}

}  // namespace

extern "C" sf_status sf_adam_host(float* p, float* m, float* v, const float* g, uint16_t* p_bf16, size_t n,
                                  int64_t step, float lr, float b1, float b2, float eps, int32_t n_threads) {
  return adam_host_impl(p, m, v, g, 1, p_bf16, n, step, lr, b1, b2, eps, 1.0f, n_threads);
}

extern "C" sf_status sf_adam_host_ex(int32_t dtype, float* p, float* m, float* v, const float* g, void* p_out,
                                     size_t n, int64_t step, float lr, float b1, float b2, float eps,
                                     float grad_scale, int32_t n_threads) {
  if (dtype != SF_F32 && dtype != SF_BF16 && dtype != SF_F16) return fail(SF_ERR_ARG, "bad dtype %d", dtype);
  if (!(grad_scale > 0.f) || !std::isfinite(grad_scale)) return fail(SF_ERR_ARG, "grad_scale must be finite and > 0");
  if (dtype == SF_F32) {
    if (p_out && p_out != static_cast<void*>(p)) return fail(SF_ERR_ARG, "SF_F32: p_out must be NULL or p");
    return adam_host_impl(p, m, v, g, 0, nullptr, n, step, lr, b1, b2, eps, grad_scale, n_threads);
  }
  return adam_host_impl(p, m, v, g, dtype == SF_F16 ? 2 : 1, static_cast<uint16_t*>(p_out), n, step, lr, b1, b2, eps,
                        grad_scale, n_threads);
}

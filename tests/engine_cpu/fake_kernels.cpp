// Stand-ins for the library's device entry points that the sliding engine
// calls (see fake_kernels.h).  Adam-type operations run the library's own
// host Adam (adam_range), so their results are the real ones; the layer and
// head stand-ins mix their inputs into finite outputs of the right types and
// sizes.
#include "fake_kernels.h"

#include <immintrin.h>

#include <cmath>
#include <cstring>
#include <functional>
#include <vector>

#include "adam.h"
#include "gemm.h"

namespace fake {

namespace {

inline uint32_t mix(uint32_t h, uint32_t x) {
  h ^= x + 0x9E3779B9u + (h << 6) + (h >> 2);
  h *= 0x85EBCA6Bu;
  return h ^ (h >> 13);
}
// a value in [-1, 1) from (h, i)
inline float unit(uint32_t h, uint64_t i) {
  const uint32_t m = mix(mix(h, static_cast<uint32_t>(i)), static_cast<uint32_t>(i >> 32));
  return static_cast<float>(m >> 8) * (1.0f / 8388608.0f) - 1.0f;
}
inline uint16_t f2bf(float f) {
  uint32_t u;
  std::memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}
inline float bf2f(uint16_t b) {
  const uint32_t u = static_cast<uint32_t>(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

uint32_t hash_bytes(const void* p, size_t bytes, uint32_t seed) {
  const unsigned char* c = static_cast<const unsigned char*>(p);
  uint32_t h = seed;
  size_t i = 0;
  for (; i + 4 <= bytes; i += 4) {
    uint32_t w;
    std::memcpy(&w, c + i, 4);
    h = mix(h, w);
  }
  for (; i < bytes; ++i) h = mix(h, c[i]);
  return h;
}

float to_f(int dtype, const void* x, size_t i) {
  if (dtype == SF_F32) return static_cast<const float*>(x)[i];
  const uint16_t u = static_cast<const uint16_t*>(x)[i];
  if (dtype == SF_BF16) return bf2f(u);
  return _cvtsh_ss(u);
}
void from_f(int dtype, void* x, size_t i, float v) {
  if (dtype == SF_F32) static_cast<float*>(x)[i] = v;
  else if (dtype == SF_BF16) static_cast<uint16_t*>(x)[i] = f2bf(v);
  else static_cast<uint16_t*>(x)[i] = _cvtss_sh(v, 0);
}

void layer_fwd_now(const Shape& s, const void* w, const void* x, void* y, void* saved) {
  const size_t n = static_cast<size_t>(s.T) * s.H;
  const uint32_t hw = hash_bytes(w, s.L->param_bytes, 1u);
  const uint32_t hx = hash_bytes(x, n * s.e, 2u);
  for (size_t i = 0; i < n; ++i) from_f(s.dtype, y, i, 0.5f * to_f(s.dtype, x, i) + 0.25f * unit(hw, i));
  uint32_t* sv = static_cast<uint32_t*>(saved);
  for (size_t k = 0; k < s.L->saved_bytes / 4; ++k) sv[k] = mix(hw ^ hx, static_cast<uint32_t>(k));
}

void layer_bwd_now(const Shape& s, const void* w, const void* x, const void* saved, const void* dy, void* dx,
                   float* dw, int part) {
  const size_t n = static_cast<size_t>(s.T) * s.H;
  uint32_t h = hash_bytes(w, s.L->param_bytes, 3u);
  h = mix(h, hash_bytes(x, n * s.e, 4u));
  h = mix(h, hash_bytes(saved, s.L->saved_bytes, 5u));
  h = mix(h, hash_bytes(dy, n * s.e, 6u));
  auto grad = [&](int t) {
    float* g = dw + s.L->grad_off[t] / 4;
    for (size_t k = 0; k < s.L->grad_bytes_t[t] / 4; ++k) g[k] = 0.01f * unit(mix(h, static_cast<uint32_t>(t)), k);
  };
  if (part == 0) {
    grad(SF_WD);
  } else if (part == 1) {
    grad(SF_WG);
    grad(SF_WU);
  } else {
    for (int t : {SF_WQ, SF_WK, SF_WV, SF_WO, SF_G1, SF_G2}) grad(t);
    // dx may alias dy: element i is read before it is written
    for (size_t i = 0; i < n; ++i) from_f(s.dtype, dx, i, 0.5f * to_f(s.dtype, dy, i) + 0.25f * unit(h, i));
  }
}

void head_now(const Shape& s, const void* gf, const void* wlm, const void* x, const int32_t* ids, float* loss,
              void* dx, float* dgf, float* dwlm, float grad_scale, bool defer, float* scratch) {
  const size_t n = static_cast<size_t>(s.T) * s.H, VH = static_cast<size_t>(s.V) * s.H;
  uint32_t h = hash_bytes(gf, s.H * s.e, 7u);
  h = mix(h, hash_bytes(wlm, VH * s.e, 8u));
  h = mix(h, hash_bytes(x, n * s.e, 9u));
  h = mix(h, hash_bytes(ids, static_cast<size_t>(s.T) * 4, 10u));
  *loss = 5.0f + unit(h, 0);
  for (size_t i = 0; i < n; ++i) from_f(s.dtype, dx, i, grad_scale * 0.01f * unit(mix(h, 1), i));
  for (int j = 0; j < s.H; ++j) dgf[j] = grad_scale * 0.01f * unit(mix(h, 2), j);
  // dW_lm: a first part, plus the part of the "last row chunk" (16 values
  // added to the first 16 rows' first element), now or after head_last_dw
  for (size_t k = 0; k < VH; ++k) dwlm[k] = grad_scale * 0.01f * unit(mix(h, 3), k);
  float last[16];
  for (int r = 0; r < 16; ++r) last[r] = grad_scale * 0.001f * unit(mix(h, 4), r);
  if (defer) {
    std::memcpy(scratch, last, sizeof last);
  } else {
    for (int r = 0; r < 16 && r < s.V; ++r) dwlm[static_cast<size_t>(r) * s.H] += last[r];
  }
}

void head_last_dw_now(const Shape& s, float* dwlm, const float* scratch) {
  for (int r = 0; r < 16 && r < s.V; ++r) dwlm[static_cast<size_t>(r) * s.H] += scratch[r];
}

void embed_fwd_now(const Shape& s, const void* E, const int32_t* ids, void* x0) {
  for (int t = 0; t < s.T; ++t)
    std::memcpy(static_cast<char*>(x0) + static_cast<size_t>(t) * s.H * s.e,
                static_cast<const char*>(E) + static_cast<size_t>(ids[t]) * s.H * s.e, s.H * s.e);
}

}  // namespace fake

// ------------------------------------------------ the library's entry points
namespace {

fake::Shape shape_of(const sf_ctx* c) {
  fake::Shape s;
  s.H = c->dims.H;
  s.V = c->dims.V;
  s.T = static_cast<int>(c->dims.T);
  s.S = c->dims.S;
  s.dtype = c->dims.dtype;
  s.e = c->dims.e;
  s.L = &c->layout;
  return s;
}
void enqueue(hipStream_t s, std::function<void()> f);

sf::AdamCoef coef(float b1, float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, float gscale) {
  sf::AdamCoef c;
  c.b1 = b1; c.b2 = b2; c.one_b1 = o1; c.one_b2 = o2; c.inv_bc1 = ib1; c.inv_bc2 = ib2; c.lr = lr; c.eps = eps;
  c.gscale = gscale;
  return c;
}
int out16_of(int dtype) { return dtype == SF_BF16 ? 1 : dtype == SF_F16 ? 2 : 0; }

}  // namespace

// FakeStream is opaque here; ops go through the runtime's own queueing.
struct FakeStream;
void fake_enqueue(hipStream_t s, std::function<void()> f);
namespace {
void enqueue(hipStream_t s, std::function<void()> f) { fake_enqueue(s, std::move(f)); }
}  // namespace

sf_ctx::~sf_ctx() {}

size_t sf::gemm_splitk_bytes(int, int, int) { return 0; }

extern "C" {

sf_status sf_ctx_create(const sf_shape* shape, int32_t head_chunk_rows, void* d_workspace, size_t workspace_bytes,
                        sf_ctx** out) {
  sf::Dims d;
  if (sf_status st = sf::check_shape(shape, &d)) return st;
  if (!out || !d_workspace) return sf::fail(SF_ERR_ARG, "bad argument");
  sf_ctx* c = new sf_ctx();
  c->dims = d;
  if (sf_status st = sf_layer_layout(shape, head_chunk_rows, &c->layout)) {
    delete c;
    return st;
  }
  c->saved = sf::saved_layout(d);
  c->work = sf::work_layout(d, head_chunk_rows);
  c->head_chunk_rows = head_chunk_rows;
  c->ws = static_cast<char*>(d_workspace);
  c->ws_bytes = workspace_bytes;
  if (workspace_bytes < 64) {
    delete c;
    return sf::fail(SF_ERR_POOL, "workspace too small");
  }
  *out = c;
  return SF_OK;
}

sf_status sf_ctx_destroy(sf_ctx* c) {
  delete c;
  return SF_OK;
}

sf_status sf_layer_fwd(sf_ctx* c, const void* w, const void* x, void* y, void* saved, sf_stream stream) {
  const fake::Shape s = shape_of(c);
  enqueue(static_cast<hipStream_t>(stream), [=] { fake::layer_fwd_now(s, w, x, y, saved); });
  return SF_OK;
}

sf_status sf_embed_fwd(sf_ctx* c, const void* E, const int32_t* ids, void* x0, sf_stream stream) {
  const fake::Shape s = shape_of(c);
  enqueue(static_cast<hipStream_t>(stream), [=] { fake::embed_fwd_now(s, E, ids, x0); });
  return SF_OK;
}

sf_status sf_embed_bwd(sf_ctx* c, const void* dx0, const int32_t* ids, float* dE, sf_stream stream) {
  const fake::Shape s = shape_of(c);
  enqueue(static_cast<hipStream_t>(stream), [=] {
    std::memset(dE, 0, static_cast<size_t>(s.V) * s.H * 4);
    for (int t = 0; t < s.T; ++t)
      for (int j = 0; j < s.H; ++j)
        dE[static_cast<size_t>(ids[t]) * s.H + j] += fake::to_f(s.dtype, dx0, static_cast<size_t>(t) * s.H + j);
  });
  return SF_OK;
}

}  // extern "C"

namespace sf {

sf_status layer_bwd(sf_ctx* c, const void* w, const void* x, const void* saved, const void* dy, void* dx, float* dw,
                    sf_stream stream, hipEvent_t ffn_done, hipEvent_t wd_done) {
  const fake::Shape s = shape_of(c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  enqueue(st, [=] { fake::layer_bwd_now(s, w, x, saved, dy, dx, dw, 0); });
  if (wd_done) SF_HIP(hipEventRecord(wd_done, st));
  enqueue(st, [=] { fake::layer_bwd_now(s, w, x, saved, dy, dx, dw, 1); });
  if (ffn_done) SF_HIP(hipEventRecord(ffn_done, st));
  enqueue(st, [=] { fake::layer_bwd_now(s, w, x, saved, dy, dx, dw, 2); });
  return SF_OK;
}

sf_status head_fwd_bwd(sf_ctx* c, const void* gf, const void* wlm, const void* x, const int32_t* ids, float* loss,
                       void* dx, float* dgf, float* dwlm, sf_stream stream, bool defer, float grad_scale) {
  const fake::Shape s = shape_of(c);
  float* scratch = reinterpret_cast<float*>(c->ws);  // the head pass's workspace
  enqueue(static_cast<hipStream_t>(stream),
          [=] { fake::head_now(s, gf, wlm, x, ids, loss, dx, dgf, dwlm, grad_scale, defer, scratch); });
  return SF_OK;
}

sf_status head_last_dw(sf_ctx* c, float* dwlm, sf_stream stream) {
  const fake::Shape s = shape_of(c);
  const float* scratch = reinterpret_cast<const float*>(c->ws);
  enqueue(static_cast<hipStream_t>(stream), [=] { fake::head_last_dw_now(s, dwlm, scratch); });
  return SF_OK;
}

hipError_t embed_bwd_sparse(int dtype, const void* dx0, const int32_t* ids, int32_t* out_ids, float* out_rows,
                            int32_t* count, int32_t* scratch, int rows, int H, int V, hipStream_t s) {
  enqueue(s, [=] {
    // scratch: first-occurrence slot per token (2 rows int32 of room)
    int n = 0;
    for (int t = 0; t < rows; ++t) {
      int slot = -1;
      for (int q = 0; q < n; ++q)
        if (out_ids[q] == ids[t]) slot = q;
      if (slot < 0) {
        slot = n++;
        out_ids[slot] = ids[t];
        std::memset(out_rows + static_cast<size_t>(slot) * H, 0, static_cast<size_t>(H) * 4);
      }
      scratch[t] = slot;
    }
    for (int t = 0; t < rows; ++t)
      for (int j = 0; j < H; ++j)
        out_rows[static_cast<size_t>(scratch[t]) * H + j] += fake::to_f(dtype, dx0, static_cast<size_t>(t) * H + j);
    *count = n;
    (void)V;
  });
  return hipSuccess;
}

hipError_t embed_adam_sparse(int dtype, float* p, float* m, float* v, const float* rows, const int32_t* out_ids,
                             const int32_t* count, int32_t* map, int max_rows, void* out, int V, int H, float b1,
                             float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                             float gscale, const int32_t* skip) {
  enqueue(s, [=] {
    if (skip && *skip) return;
    for (int r = 0; r < V; ++r) map[r] = -1;
    for (int q = 0; q < *count && q < max_rows; ++q) map[out_ids[q]] = q;
    const sf::AdamCoef c = coef(b1, b2, o1, o2, ib1, ib2, lr, eps, gscale);
    std::vector<float> zero(static_cast<size_t>(H), 0.0f);
    const int o16 = out16_of(dtype);
    for (int r = 0; r < V; ++r) {
      const size_t off = static_cast<size_t>(r) * H;
      const float* g = map[r] >= 0 ? rows + static_cast<size_t>(map[r]) * H : zero.data();
      uint16_t* pb = o16 ? static_cast<uint16_t*>(out) + off : nullptr;
      sf::adam_range(p + off, m + off, v + off, g, pb, static_cast<size_t>(H), c, o16);
      if (!o16 && out) std::memcpy(static_cast<float*>(out) + off, p + off, static_cast<size_t>(H) * 4);
    }
  });
  return hipSuccess;
}

hipError_t adam_device(int dtype, float* p, float* m, float* v, const float* g, void* out, int64_t n, float b1,
                       float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                       float gscale, const int32_t* skip) {
  enqueue(s, [=] {
    if (skip && *skip) return;
    const sf::AdamCoef c = coef(b1, b2, o1, o2, ib1, ib2, lr, eps, gscale);
    const int o16 = out16_of(dtype);
    sf::adam_range(p, m, v, g, o16 ? static_cast<uint16_t*>(out) : nullptr, static_cast<size_t>(n), c, o16);
    if (!o16 && out) std::memcpy(out, p, static_cast<size_t>(n) * 4);
  });
  return hipSuccess;
}

hipError_t nonfinite_flag(const float* g, int64_t n, int32_t* flag, hipStream_t s) {
  enqueue(s, [=] {
    for (int64_t i = 0; i < n; ++i)
      if (!std::isfinite(g[i])) *flag = 1;
  });
  return hipSuccess;
}

hipError_t nonfinite_flag_segs(const float* base, const FloatSegs& segs, int32_t* flag, hipStream_t s) {
  const FloatSegs sg = segs;
  enqueue(s, [=] {
    for (int k = 0; k < sg.count; ++k)
      for (int64_t i = 0; i < sg.n[k]; ++i)
        if (!std::isfinite(base[sg.off[k] + i])) *flag = 1;
  });
  return hipSuccess;
}

hipError_t nonfinite_storage(int dtype, const void* x, int64_t n, int32_t* flag, hipStream_t s) {
  enqueue(s, [=] {
    for (int64_t i = 0; i < n; ++i)
      if (!std::isfinite(fake::to_f(dtype, x, static_cast<size_t>(i)))) *flag = 1;
  });
  return hipSuccess;
}

hipError_t scale_storage(int dtype, const void* x, void* y, int64_t n, float sc, hipStream_t s) {
  enqueue(s, [=] {
    for (int64_t i = 0; i < n; ++i)
      fake::from_f(dtype, y, static_cast<size_t>(i), fake::to_f(dtype, x, static_cast<size_t>(i)) * sc);
  });
  return hipSuccess;
}

hipError_t copy_words(uint32_t* dst, const uint32_t* src, int n, hipStream_t s) {
  enqueue(s, [=] { std::memcpy(dst, src, static_cast<size_t>(n) * 4); });
  return hipSuccess;
}

hipError_t set_word(int32_t* p, int32_t v, hipStream_t s) {
  enqueue(s, [=] { *p = v; });
  return hipSuccess;
}

hipError_t copy_f32(float* dst, const float* src, int n, hipStream_t s) {
  enqueue(s, [=] { std::memcpy(dst, src, static_cast<size_t>(n) * 4); });
  return hipSuccess;
}

}  // namespace sf

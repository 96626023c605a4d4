// CPU check of the sliding engine's host logic (test infrastructure).
//
// engine.cpp, adam.cpp and layout.cpp are built unchanged against the fake
// HIP runtime (fake_hip.cpp: a worker thread per stream, events with the
// runtime's ordering rules) and the stand-in kernels (fake_kernels.cpp:
// the real buffers, mixing arithmetic, the library's own host Adam).  Each
// scenario runs a few steps of the engine and, separately, a plain
// sequential model of what one step computes (forward through every layer,
// head, backward, the Adam updates and loss-scaling decisions of the step,
// in program order, with the same stand-ins); the losses, the host masters,
// moments and parameters, the head state and the resident tensors must be
// equal bit for bit.  A missing wait in the engine either makes a stand-in
// read a buffer before its producer wrote it (a different result; the
// random stream delays of FAKE_HIP_JITTER_US vary the interleavings) or is
// reported by ThreadSanitizer in the TSan build, which sees every access
// of the stand-ins and copies and only the ordering edges the runtime
// guarantees.
//
// Usage: engine_check [scenario ...]   (no argument: every scenario)
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/sf.h"
#include "adam.h"
#include "fake_kernels.h"
#include "internal.h"

void fake_hip_drain_default();

namespace {

struct Scenario {
  const char* name;
  int flags;
  int window, slots, n_layers, dtype, steps;
  bool head;
  int fault_layer;  // SF_FAULT_NONFINITE_LAYER, -1: none
};

const Scenario kScenarios[] = {
    {"adam-sync", SF_ENGINE_ADAM | SF_ENGINE_HEAD, 2, 2, 4, SF_BF16, 3, true, -1},
    {"adam-pipe", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_PIPELINE, 2, 2, 4, SF_BF16, 4, true, -1},
    {"adam-ckpt", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_CKPT, 2, 2, 4, SF_BF16, 3, true, -1},
    {"adam-pipe-ckpt", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_PIPELINE | SF_ENGINE_CKPT, 2, 3, 5, SF_BF16, 4, true,
     -1},
    {"adam-hosthead", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_HEAD_HOST_ADAM, 2, 2, 4, SF_BF16, 3, true, -1},
    {"adam-w3", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_PIPELINE, 3, 3, 7, SF_BF16, 3, true, -1},
    {"noadam-keep", SF_ENGINE_HEAD | SF_ENGINE_KEEP_TURNAROUND, 2, 4, 4, SF_BF16, 3, true, -1},
    {"noadam-keep-pipe", SF_ENGINE_HEAD | SF_ENGINE_KEEP_TURNAROUND | SF_ENGINE_PIPELINE, 2, 4, 4, SF_BF16, 3, true,
     -1},
    {"nohead-adam", SF_ENGINE_ADAM, 2, 2, 3, SF_BF16, 3, false, -1},
    {"f32-adam", SF_ENGINE_ADAM | SF_ENGINE_HEAD, 2, 2, 3, SF_F32, 3, true, -1},
    {"f16-scale", SF_ENGINE_ADAM | SF_ENGINE_HEAD | SF_ENGINE_PIPELINE, 2, 2, 4, SF_F16, 3, true, -1},
    {"f16-fault", SF_ENGINE_ADAM | SF_ENGINE_HEAD, 2, 2, 4, SF_F16, 3, true, 1},
    {"f16-fault-pipe-nohead", SF_ENGINE_ADAM | SF_ENGINE_PIPELINE, 2, 2, 4, SF_F16, 3, false, 2},
    // keep-turnaround without Adam past two windows: gradient-region pages in
    // the forward (a slot per layer, so the last step's gradients all stay)
    {"noadam-keep-pipe-l8", SF_ENGINE_KEEP_TURNAROUND | SF_ENGINE_PIPELINE, 2, 8, 8, SF_BF16, 4, false, -1},
    {"noadam-keep-l7", SF_ENGINE_HEAD | SF_ENGINE_KEEP_TURNAROUND, 2, 7, 7, SF_BF16, 3, true, -1},
    {"noadam-keep-pipe-l5", SF_ENGINE_KEEP_TURNAROUND | SF_ENGINE_PIPELINE, 2, 5, 5, SF_BF16, 4, false, -1},
    {"noadam-keep-pipe-ckpt-l8", SF_ENGINE_HEAD | SF_ENGINE_KEEP_TURNAROUND | SF_ENGINE_PIPELINE | SF_ENGINE_CKPT, 2, 8,
     8, SF_BF16, 3, true, -1},
    {"noadam-keep-pipe-w3-l10", SF_ENGINE_HEAD | SF_ENGINE_KEEP_TURNAROUND | SF_ENGINE_PIPELINE, 3, 10, 10, SF_BF16, 3,
     true, -1},
};

constexpr float kLr = 1e-3f, kB1 = 0.9f, kB2 = 0.999f, kEps = 1e-8f;

int g_fail = 0;
#define CHECK(c, ...)                   \
  do {                                  \
    if (!(c)) {                         \
      std::printf("FAIL: " __VA_ARGS__); \
      std::printf("\n");                \
      ++g_fail;                         \
    }                                   \
  } while (0)

// "Device" memory starts as all-ones bytes: NaN in fp32, bf16 and fp16, so a
// stand-in that reads a device buffer before anything wrote it spreads NaN
// into a result that must equal the sequential model's (FAKE_HIP_POISON=0
// starts from zeros instead).
void* dev_alloc(size_t bytes) {
  const size_t n = (bytes + 255) / 256 * 256 + 256;
  void* p = std::aligned_alloc(256, n);
  const char* pz = std::getenv("FAKE_HIP_POISON");
  std::memset(p, (pz && pz[0] == '0') ? 0 : 0xFF, n);
  return p;
}
void* pinned(size_t bytes) {
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes, 0) != hipSuccess) std::abort();
  std::memset(p, 0, bytes);
  return p;
}

sf_shape make_shape(const Scenario& sc) {
  sf_shape s;
  s.hidden = 64; s.n_heads = 1; s.n_kv_heads = 1; s.head_dim = 64; s.ffn = 128;
  s.vocab = sc.head ? 64 : 0;
  s.batch = 2; s.seq = 8; s.rms_eps = 1e-6f; s.rope_base = 10000.f; s.dtype = sc.dtype;
  return s;
}

// Deterministic initial storage values (finite, |v| < 0.05).
void init_storage(int dtype, void* p, size_t n, uint32_t seed) {
  for (size_t i = 0; i < n; ++i) {
    const uint32_t h = fake::hash_bytes(&i, sizeof i, seed);
    fake::from_f(dtype, p, i, 0.05f * (static_cast<float>(h >> 8) / 8388608.0f - 1.0f));
  }
}

// What the comparison covers.
struct State {
  std::vector<float> losses;
  std::vector<std::vector<char>> params;        // per layer, storage layout
  std::vector<std::vector<float>> master, m, v; // per layer, fp32 gradient layout
  std::vector<char> E, gf, wlm;                 // resident head tensors (storage)
  std::vector<float> head_master, head_m, head_v;
  std::vector<std::vector<float>> last_grads;   // per layer, last step (no Adam)
};

// ---------------------------------------------------------------- reference
struct Ref {
  const Scenario& sc;
  sf_shape shape;
  sf_layout L;
  fake::Shape fs;
  int nl, T, H, V;
  size_t e, xn;
  float S = 1.f;
  int good = 0;
  bool lscale;
  std::vector<int64_t> adam_t;
  int64_t head_t = 0, embed_t = 0;

  Ref(const Scenario& s) : sc(s) {
    shape = make_shape(sc);
    sf_layer_layout(&shape, 2048, &L);
    nl = sc.n_layers; T = shape.batch * shape.seq; H = shape.hidden; V = shape.vocab;
    e = sc.dtype == SF_F32 ? 4 : 2;
    xn = static_cast<size_t>(T) * H;
    fs = fake::Shape{H, V, T, shape.seq, sc.dtype, e, &L};
    lscale = sc.dtype == SF_F16;
    S = lscale ? 65536.f : 1.f;
    adam_t.assign(nl, 0);
  }

  void run(State* st, const std::vector<int32_t>& ids, const std::vector<char>& xin, const std::vector<char>& dyin) {
    const bool adam = sc.flags & SF_ENGINE_ADAM;
    const size_t NH = 2 * static_cast<size_t>(V) * H + H, VH = static_cast<size_t>(V) * H;
    for (int step = 0; step < sc.steps; ++step) {
      std::vector<std::vector<char>> x(nl + 1, std::vector<char>(xn * e)), saved(nl, std::vector<char>(L.saved_bytes));
      if (sc.head) fake::embed_fwd_now(fs, st->E.data(), ids.data(), x[0].data());
      else x[0] = xin;
      for (int l = 0; l < nl; ++l) fake::layer_fwd_now(fs, st->params[l].data(), x[l].data(), x[l + 1].data(), saved[l].data());
      std::vector<char> dx(xn * e);
      std::vector<float> dgf(H), dwlm(VH);
      bool bad = false;
      bool head_ok = true;
      if (sc.head) {
        float loss;
        fake::head_now(fs, st->gf.data(), st->wlm.data(), x[nl].data(), ids.data(), &loss, dx.data(), dgf.data(),
                       dwlm.data(), S, false, nullptr);
        st->losses.push_back(loss);
        if (lscale) {
          for (float v : dgf) bad = bad || !std::isfinite(v);
          for (float v : dwlm) bad = bad || !std::isfinite(v);
        }
        head_ok = !bad;
      } else {
        for (size_t i = 0; i < xn; ++i) fake::from_f(sc.dtype, dx.data(), i, fake::to_f(sc.dtype, dyin.data(), i) * (lscale ? S : 1.f));
      }
      std::vector<std::vector<float>> g(nl, std::vector<float>(L.grad_bytes / 4, 0.f));
      std::vector<bool> apply(nl, true);
      for (int l = nl - 1; l >= 0; --l) {
        for (int part = 0; part < 3; ++part)
          fake::layer_bwd_now(fs, st->params[l].data(), x[l].data(), saved[l].data(), dx.data(), dx.data(), g[l].data(), part);
        if (lscale) {
          for (int t = 0; t < SF_NTENSORS; ++t)
            for (size_t k = 0; k < L.grad_bytes_t[t] / 4; ++k) bad = bad || !std::isfinite(g[l][L.grad_off[t] / 4 + k]);
          if (l == sc.fault_layer) bad = true;
        }
        apply[l] = !bad;
      }
      if (lscale && sc.head)
        for (size_t i = 0; i < xn; ++i) bad = bad || !std::isfinite(fake::to_f(sc.dtype, dx.data(), i));
      const bool embed_ok = !bad;
      if (!adam) {
        st->last_grads = g;
      } else {
        const float gscale = 1.0f / S;
        const int out16 = sc.dtype == SF_BF16 ? 1 : sc.dtype == SF_F16 ? 2 : 0;
        for (int l = 0; l < nl; ++l) {
          if (!apply[l]) continue;
          sf::AdamCoef c = sf::adam_coef(adam_t[l] + 1, kLr, kB1, kB2, kEps);
          c.gscale = gscale;
          for (int t = 0; t < SF_NTENSORS; ++t) {
            const size_t o = L.grad_off[t] / 4, n = L.grad_bytes_t[t] / 4, po = L.off[t] / e;
            uint16_t* pb = out16 ? reinterpret_cast<uint16_t*>(st->params[l].data()) + po : nullptr;
            sf::adam_range(st->master[l].data() + o, st->m[l].data() + o, st->v[l].data() + o, g[l].data() + o, pb, n, c,
                           out16 ? out16 : 1);
            if (!out16) std::memcpy(reinterpret_cast<float*>(st->params[l].data()) + po, st->master[l].data() + o, n * 4);
          }
          ++adam_t[l];
        }
        if (sc.head) {
          float* p = st->head_master.data();
          float* mm = st->head_m.data();
          float* vv = st->head_v.data();
          auto upd = [&](size_t off, size_t n, const float* gg, char* out, const sf::AdamCoef& c) {
            uint16_t* pb = out16 ? reinterpret_cast<uint16_t*>(out) : nullptr;
            sf::adam_range(p + off, mm + off, vv + off, gg, pb, n, c, out16 ? out16 : 1);
            if (!out16) std::memcpy(out, p + off, n * 4);
          };
          if (head_ok) {
            sf::AdamCoef c = sf::adam_coef(head_t + 1, kLr, kB1, kB2, kEps);
            c.gscale = gscale;
            upd(VH, H, dgf.data(), st->gf.data(), c);
            upd(VH + H, VH, dwlm.data(), st->wlm.data(), c);
            ++head_t;
          }
          if (embed_ok) {
            // dense Adam over the embedding with the summed rows of dx_0
            std::vector<float> dE(VH, 0.f);
            for (int t = 0; t < T; ++t)
              for (int j = 0; j < H; ++j) dE[static_cast<size_t>(ids[t]) * H + j] += fake::to_f(sc.dtype, dx.data(), static_cast<size_t>(t) * H + j);
            // rows accumulate in token order, like the sparse gradient
            sf::AdamCoef c = sf::adam_coef(embed_t + 1, kLr, kB1, kB2, kEps);
            c.gscale = gscale;
            for (int r = 0; r < V; ++r) upd(static_cast<size_t>(r) * H, H, dE.data() + static_cast<size_t>(r) * H, st->E.data() + static_cast<size_t>(r) * H * e, c);
            ++embed_t;
          }
          (void)NH;
        }
      }
      if (lscale) {
        if (bad) {
          S = std::max(1.0f, S * 0.5f);
          good = 0;
        } else if (++good >= 2000) {
          if (std::isfinite(S * 2.0f)) S *= 2.0f;
          good = 0;
        }
      }
    }
  }
};

// ------------------------------------------------------------------ engine
struct Run {
  const Scenario& sc;
  sf_shape shape;
  sf_layout L;
  int nl, T, H, V;
  size_t e, xn;
  sf_ctx* ctx = nullptr;
  sf_engine* eng = nullptr;
  hipStream_t comp = nullptr;
  std::vector<void*> h_params, h_slots;
  std::vector<float*> h_master, h_m, h_v;
  void *pool = nullptr, *act = nullptr, *ws = nullptr, *h_ckpt = nullptr;
  void *d_E = nullptr, *d_gf = nullptr, *d_wlm = nullptr;
  float *d_head_grads = nullptr, *d_head_state = nullptr;
  void* h_head_params = nullptr;
  float *h_head_master = nullptr, *h_head_m = nullptr, *h_head_v = nullptr, *h_head_grads = nullptr;
  int32_t* d_ids = nullptr;
  void *d_in = nullptr, *d_dy = nullptr;

  explicit Run(const Scenario& s) : sc(s) {
    shape = make_shape(sc);
    sf_layer_layout(&shape, 2048, &L);
    nl = sc.n_layers; T = shape.batch * shape.seq; H = shape.hidden; V = shape.vocab;
    e = sc.dtype == SF_F32 ? 4 : 2;
    xn = static_cast<size_t>(T) * H;
  }

  // initial state shared with the reference
  void init(State* st, std::vector<int32_t>* ids, std::vector<char>* xin, std::vector<char>* dyin) {
    st->params.assign(nl, std::vector<char>(L.param_bytes, 0));
    st->master.assign(nl, std::vector<float>(L.grad_bytes / 4, 0.f));
    st->m.assign(nl, std::vector<float>(L.grad_bytes / 4, 0.f));
    st->v.assign(nl, std::vector<float>(L.grad_bytes / 4, 0.f));
    for (int l = 0; l < nl; ++l) {
      for (int t = 0; t < SF_NTENSORS; ++t) {
        const size_t n = L.bytes[t] / e;
        init_storage(sc.dtype, st->params[l].data() + L.off[t], n, 100u + 10u * l + t);
        for (size_t k = 0; k < n; ++k)
          st->master[l][L.grad_off[t] / 4 + k] = fake::to_f(sc.dtype, st->params[l].data() + L.off[t], k);
      }
    }
    ids->resize(T);
    for (int t = 0; t < T; ++t) (*ids)[t] = sc.head ? (t * 7 + 3) % V : 0;
    xin->assign(xn * e, 0);
    dyin->assign(xn * e, 0);
    init_storage(sc.dtype, xin->data(), xn, 7u);
    init_storage(sc.dtype, dyin->data(), xn, 9u);
    if (sc.head) {
      const size_t VH = static_cast<size_t>(V) * H, NH = 2 * VH + H;
      st->E.assign(VH * e, 0); st->gf.assign(H * e, 0); st->wlm.assign(VH * e, 0);
      init_storage(sc.dtype, st->E.data(), VH, 11u);
      init_storage(sc.dtype, st->gf.data(), H, 12u);
      init_storage(sc.dtype, st->wlm.data(), VH, 13u);
      st->head_master.assign(NH, 0.f); st->head_m.assign(NH, 0.f); st->head_v.assign(NH, 0.f);
      for (size_t k = 0; k < VH; ++k) st->head_master[k] = fake::to_f(sc.dtype, st->E.data(), k);
      for (int k = 0; k < H; ++k) st->head_master[VH + k] = fake::to_f(sc.dtype, st->gf.data(), k);
      for (size_t k = 0; k < VH; ++k) st->head_master[VH + H + k] = fake::to_f(sc.dtype, st->wlm.data(), k);
    }
  }

  bool create(const State& st0, const std::vector<int32_t>& ids, const std::vector<char>& xin,
              const std::vector<char>& dyin) {
    ws = dev_alloc(L.workspace_bytes + L.head_workspace_bytes + 256);
    if (sf_ctx_create(&shape, 2048, ws, L.workspace_bytes + L.head_workspace_bytes + 256, &ctx)) return false;
    const size_t unit = (L.param_bytes + 255) / 256 * 256 + (L.grad_bytes + 255) / 256 * 256;
    const int W = std::min(sc.window, nl);
    pool = dev_alloc(W * unit);
    size_t act_bytes = 0;
    if (sf_engine_act_bytes_flags(&shape, nl, sc.flags, &act_bytes)) return false;
    act = dev_alloc(act_bytes);
    const bool adam = sc.flags & SF_ENGINE_ADAM;
    for (int l = 0; l < nl; ++l) {
      h_params.push_back(pinned(L.param_bytes));
      std::memcpy(h_params.back(), st0.params[l].data(), L.param_bytes);
      if (adam) {
        h_master.push_back(static_cast<float*>(std::calloc(L.grad_bytes / 4, 4)));
        std::memcpy(h_master.back(), st0.master[l].data(), L.grad_bytes);
        h_m.push_back(static_cast<float*>(std::calloc(L.grad_bytes / 4, 4)));
        h_v.push_back(static_cast<float*>(std::calloc(L.grad_bytes / 4, 4)));
      }
    }
    for (int k = 0; k < sc.slots; ++k) h_slots.push_back(pinned(L.grad_bytes));
    if (hipStreamCreateWithFlags(&comp, hipStreamNonBlocking)) return false;
    sf_engine_cfg c;
    std::memset(&c, 0, sizeof c);
    c.n_layers = nl; c.window = sc.window; c.n_grad_slots = sc.slots; c.flags = sc.flags; c.adam_threads = 3;
    c.lr = kLr; c.b1 = kB1; c.b2 = kB2; c.eps = kEps;
    c.d_pool = pool; c.pool_bytes = W * unit;
    c.d_act = act; c.act_bytes = act_bytes;
    c.h_params = h_params.data();
    c.h_master = adam ? h_master.data() : nullptr;
    c.h_m = adam ? h_m.data() : nullptr;
    c.h_v = adam ? h_v.data() : nullptr;
    c.h_grad_slots = reinterpret_cast<float**>(h_slots.data());
    c.compute_stream = comp;
    if (sc.flags & SF_ENGINE_CKPT) {
      const size_t x = (xn * e + 255) / 256 * 256;
      h_ckpt = pinned((nl - 1) * x);
      c.h_ckpt = h_ckpt;
    }
    if (sc.head) {
      const size_t VH = static_cast<size_t>(V) * H, NH = 2 * VH + H;
      d_E = dev_alloc(VH * e); d_gf = dev_alloc(H * e); d_wlm = dev_alloc(VH * e);
      std::memcpy(d_E, st0.E.data(), VH * e);
      std::memcpy(d_gf, st0.gf.data(), H * e);
      std::memcpy(d_wlm, st0.wlm.data(), VH * e);
      d_head_grads = static_cast<float*>(dev_alloc(NH * 4));
      c.d_E = d_E; c.d_gf = d_gf; c.d_wlm = d_wlm; c.d_head_grads = d_head_grads;
      if (sc.flags & SF_ENGINE_HEAD_HOST_ADAM) {
        h_head_params = pinned(NH * e);
        std::memcpy(h_head_params, st0.E.data(), VH * e);
        std::memcpy(static_cast<char*>(h_head_params) + VH * e, st0.gf.data(), H * e);
        std::memcpy(static_cast<char*>(h_head_params) + (VH + H) * e, st0.wlm.data(), VH * e);
        h_head_master = static_cast<float*>(std::calloc(NH, 4));
        std::memcpy(h_head_master, st0.head_master.data(), NH * 4);
        h_head_m = static_cast<float*>(std::calloc(NH, 4));
        h_head_v = static_cast<float*>(std::calloc(NH, 4));
        h_head_grads = static_cast<float*>(pinned(NH * 4));
        c.h_head_params = h_head_params; c.h_head_master = h_head_master; c.h_head_m = h_head_m;
        c.h_head_v = h_head_v; c.h_head_grads = h_head_grads;
      } else if (adam) {
        d_head_state = static_cast<float*>(dev_alloc(3 * NH * 4));
        std::memcpy(d_head_state, st0.head_master.data(), NH * 4);
        std::memset(d_head_state + NH, 0, 2 * NH * 4);  // moments start at zero
        c.d_head_state = d_head_state;
      }
      d_ids = static_cast<int32_t*>(dev_alloc(T * 4));
      std::memcpy(d_ids, ids.data(), T * 4);
    } else {
      d_in = dev_alloc(xn * e);
      d_dy = dev_alloc(xn * e);
      std::memcpy(d_in, xin.data(), xn * e);
      std::memcpy(d_dy, dyin.data(), xn * e);
    }
    if (sc.fault_layer >= 0) setenv("SF_FAULT_NONFINITE_LAYER", std::to_string(sc.fault_layer).c_str(), 1);
    const sf_status rc = sf_engine_create(ctx, &c, &eng);
    unsetenv("SF_FAULT_NONFINITE_LAYER");
    if (rc) std::printf("sf_engine_create: %d %s\n", rc, sf_last_error());
    return rc == SF_OK;
  }

  bool steps(State* st) {
    for (int s = 0; s < sc.steps; ++s) {
      float loss = 0.f;
      sf_step_stats stats;
      const sf_status rc = sf_slide_step(eng, sc.head ? static_cast<const void*>(d_ids) : d_in, sc.head ? nullptr : d_dy,
                                         &loss, &stats);
      if (rc) {
        std::printf("sf_slide_step: %d %s\n", rc, sf_last_error());
        return false;
      }
      if (sc.head) st->losses.push_back(loss);
    }
    sf_step_stats stats;
    if (sf_engine_sync(eng, &stats)) return false;
    return true;
  }

  void collect(State* st) {
    const bool adam = sc.flags & SF_ENGINE_ADAM;
    st->params.assign(nl, std::vector<char>(L.param_bytes));
    for (int l = 0; l < nl; ++l) std::memcpy(st->params[l].data(), h_params[l], L.param_bytes);
    if (adam) {
      st->master.assign(nl, std::vector<float>(L.grad_bytes / 4));
      st->m = st->v = st->master;
      for (int l = 0; l < nl; ++l) {
        std::memcpy(st->master[l].data(), h_master[l], L.grad_bytes);
        std::memcpy(st->m[l].data(), h_m[l], L.grad_bytes);
        std::memcpy(st->v[l].data(), h_v[l], L.grad_bytes);
      }
    } else {
      st->last_grads.clear();
      for (int k = 0; k < sc.slots; ++k) {
        std::vector<float> g(L.grad_bytes / 4);
        std::memcpy(g.data(), h_slots[k], L.grad_bytes);
        st->last_grads.push_back(g);
      }
    }
    if (sc.head) {
      const size_t VH = static_cast<size_t>(V) * H, NH = 2 * VH + H;
      st->E.assign(static_cast<char*>(d_E), static_cast<char*>(d_E) + VH * e);
      st->gf.assign(static_cast<char*>(d_gf), static_cast<char*>(d_gf) + H * e);
      st->wlm.assign(static_cast<char*>(d_wlm), static_cast<char*>(d_wlm) + VH * e);
      if (h_head_master) {
        st->head_master.assign(h_head_master, h_head_master + NH);
        st->head_m.assign(h_head_m, h_head_m + NH);
        st->head_v.assign(h_head_v, h_head_v + NH);
      } else if (d_head_state) {
        st->head_master.assign(d_head_state, d_head_state + NH);
        st->head_m.assign(d_head_state + NH, d_head_state + 2 * NH);
        st->head_v.assign(d_head_state + 2 * NH, d_head_state + 3 * NH);
      }
    }
  }

  ~Run() {
    if (eng) sf_engine_destroy(eng);
    if (ctx) sf_ctx_destroy(ctx);
    if (comp) hipStreamDestroy(comp);
    for (void* p : h_params) hipHostFree(p);
    for (void* p : h_slots) hipHostFree(p);
    for (float* p : h_master) std::free(p);
    for (float* p : h_m) std::free(p);
    for (float* p : h_v) std::free(p);
    for (void* p : {pool, act, ws, d_E, d_gf, d_wlm, static_cast<void*>(d_head_grads), static_cast<void*>(d_head_state),
                    static_cast<void*>(d_ids), d_in, d_dy})
      std::free(p);
    hipHostFree(h_ckpt);
    hipHostFree(h_head_params);
    hipHostFree(h_head_grads);
    std::free(h_head_master); std::free(h_head_m); std::free(h_head_v);
  }
};

template <typename V>
bool same(const V& a, const V& b) {
  return a.size() == b.size() && (a.empty() || std::memcmp(a.data(), b.data(), a.size() * sizeof(a[0])) == 0);
}

void run_scenario(const Scenario& sc) {
  std::printf("[engine_check] %s\n", sc.name);
  std::fflush(stdout);
  Run run(sc);
  State init, eng_st, ref_st;
  std::vector<int32_t> ids;
  std::vector<char> xin, dyin;
  run.init(&init, &ids, &xin, &dyin);
  if (!run.create(init, ids, xin, dyin) || !run.steps(&eng_st)) {
    CHECK(false, "%s: engine failed", sc.name);
    return;
  }
  run.collect(&eng_st);
  ref_st = init;
  Ref ref(sc);
  ref.run(&ref_st, ids, xin, dyin);
  CHECK(same(eng_st.losses, ref_st.losses), "%s: losses differ", sc.name);
  for (int l = 0; l < sc.n_layers; ++l) {
    CHECK(same(eng_st.params[l], ref_st.params[l]), "%s: layer %d parameters differ", sc.name, l);
    if (sc.flags & SF_ENGINE_ADAM) {
      CHECK(same(eng_st.master[l], ref_st.master[l]), "%s: layer %d master differs", sc.name, l);
      CHECK(same(eng_st.m[l], ref_st.m[l]) && same(eng_st.v[l], ref_st.v[l]), "%s: layer %d moments differ", sc.name, l);
    }
  }
  if (!(sc.flags & SF_ENGINE_ADAM)) {
    // every slot holds one layer's gradients of the last step, each layer once
    // (slots beyond the layer count hold an earlier step's)
    const sf_layout& L = run.L;
    for (int l = 0; l < sc.n_layers; ++l) {
      int hits = 0;
      for (const auto& g : eng_st.last_grads) {
        bool eq = true;
        for (int t = 0; t < SF_NTENSORS && eq; ++t)
          eq = std::memcmp(g.data() + L.grad_off[t] / 4, ref_st.last_grads[l].data() + L.grad_off[t] / 4,
                           L.grad_bytes_t[t]) == 0;
        hits += eq;
      }
      CHECK(hits == 1, "%s: layer %d's last gradients found in %d slots", sc.name, l, hits);
    }
  }
  if (sc.head) {
    CHECK(same(eng_st.E, ref_st.E), "%s: embedding differs", sc.name);
    CHECK(same(eng_st.gf, ref_st.gf), "%s: final gain differs", sc.name);
    CHECK(same(eng_st.wlm, ref_st.wlm), "%s: LM head differs", sc.name);
    if (sc.flags & SF_ENGINE_ADAM) {
      CHECK(same(eng_st.head_master, ref_st.head_master), "%s: head masters differ", sc.name);
      CHECK(same(eng_st.head_m, ref_st.head_m) && same(eng_st.head_v, ref_st.head_v), "%s: head moments differ",
            sc.name);
    }
  }
}

}  // namespace

int main(int argc, char** argv) {
  int ran = 0;
  for (const Scenario& sc : kScenarios) {
    bool want = argc < 2;
    for (int i = 1; i < argc; ++i) want = want || std::strcmp(argv[i], sc.name) == 0;
    if (!want) continue;
    run_scenario(sc);
    ++ran;
  }
  fake_hip_drain_default();
  std::printf("[engine_check] %d scenarios, %d failures\n", ran, g_fail);
  return g_fail ? 1 : (ran ? 0 : 2);
}

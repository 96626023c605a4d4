// Internal host-side definitions shared by the C-ABI implementation files.
#pragma once

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstddef>
#include <cstdint>
#include <string>

#include "../../include/sf.h"

namespace sf {

// Thread-local last-error message behind sf_last_error().
void set_error(const char* fmt, ...);
sf_status fail(sf_status code, const char* fmt, ...);

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Dims {
  int H = 0, nh = 0, nkv = 0, d = 0, F = 0, V = 0, B = 0, S = 0;
  int64_t T = 0;
  int Nq = 0, Nkv = 0, Nqkv = 0;
  int dtype = 0;
  size_t e = 4;  // storage element bytes
  float eps = 0, rope_base = 0;
};

// Offsets of the activations a layer's forward keeps for its backward.
struct SavedLayout {
  size_t xn, r1, qkv, O, lse, h, hn, r2, G, U, a, total;
};
// Offsets of the per-context workspace.
struct WorkLayout {
  size_t rope_cos, rope_sin, dGU, dhn, dh, dA, dsum, dqkv, dxn, gain_partial, splitk, splitk_bytes;
  size_t splitk_w, splitk_w_bytes;  // split-K scratch of the weight-gradient GEMMs (side stream)
  size_t dkv_partial;               // fp32 partial dK/dV sums of the attention head shares (16-bit storage)
  int kv_split;
  size_t total;
  // head (appended when vocab > 0)
  size_t hf, rf, dhf, logits, dlogits, loss_rows, head_total;
};

sf_status check_shape(const sf_shape* s, Dims* out);
void param_layout(const Dims& d, size_t elem, size_t* off, size_t* bytes, size_t* total);
SavedLayout saved_layout(const Dims& d);
// head_dw_rows: rows of dlogits kept for one LM-head weight-gradient product
// (head_dw_rows_eff); 0 = the chunk rows.
int head_dw_rows_eff(int64_t T, int head_chunk_rows, int head_dw_rows);
WorkLayout work_layout(const Dims& d, int head_chunk_rows, int head_dw_rows = 0);

}  // namespace sf

struct sf_ctx;
namespace sf {
// sf_layer_bwd with optional events recorded once the MLP weight gradients
// (Wg, Wu, Wd) are complete, before the attention half (ffn_done), and once
// the Wd gradient alone is (wd_done: the first weight-gradient GEMM).
sf_status layer_bwd(sf_ctx* c, const void* d_w, const void* d_x, const void* d_saved, const void* d_dy, void* d_dx,
                    float* d_dw, sf_stream stream, hipEvent_t ffn_done, hipEvent_t wd_done);
// sf_head_fwd_bwd; with defer_last_dw the LM-head weight gradient of the last
// row chunk is left to head_last_dw, which reads the head workspace (dlogits,
// hf) and must run before the context's next head pass.
// grad_scale multiplies dlogits (and so every gradient of the head), not the loss.
sf_status head_fwd_bwd(sf_ctx* c, const void* d_gf, const void* d_wlm, const void* d_x, const int32_t* d_ids,
                       float* d_loss, void* d_dx, float* d_dgf, float* d_dwlm, sf_stream stream, bool defer_last_dw,
                       float grad_scale = 1.0f);
sf_status head_last_dw(sf_ctx* c, float* d_dwlm, sf_stream stream);
}  // namespace sf

struct sf_ctx {
  sf::Dims dims;
  sf_layout layout;
  sf::SavedLayout saved;
  sf::WorkLayout work;
  int head_chunk_rows = 0;
  int head_dw_rows = 0;  // effective (a multiple of the chunk rows)
  char* ws = nullptr;  // caller-provided device workspace
  size_t ws_bytes = 0;
  int device = 0;
  // Weight-gradient GEMMs of the backward run on `side` (null: on the
  // caller's stream), forked and joined with the events below.
  hipStream_t side = nullptr;
  hipEvent_t ev_fork[4] = {nullptr, nullptr, nullptr, nullptr};
  hipEvent_t ev_mlp_dw = nullptr, ev_join = nullptr;
  ~sf_ctx();
};

#define SF_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return sf::fail(SF_ERR_HIP, "%s failed: %s (%s:%d)", #call, hipGetErrorString(e_), \
                      __FILE__, __LINE__);                                            \
  } while (0)

// C ABI: shape validation, buffer layouts, contexts, and the kernel
// sequences of one decoder block's forward and backward and of the fused
// LinearCrossEntropy head.
//
// The block (a Llama-family decoder layer; the pages name Llama, Qwen and
// Mistral -- de §5, es §3 -- and the fused RoPE / RMSNorm / SwiGLU /
// LinearCrossEntropy kernels -- de §2C, es §2C, fr §2C):
//   xn = RMSNorm(x; g1); [q|k|v] = xn Wqkv^T, RoPE on q and k;
//   A = causal attention; h = x + A Wo^T; hn = RMSNorm(h; g2);
//   G, U = hn Wg^T, hn Wu^T; a = silu(G) U; y = h + a Wd^T.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "adam.h"
#include "attention.h"
#include "gemm.h"
#include "internal.h"
#include "rowops.h"

namespace sf {

namespace {

sf_status check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    if (!p) return fail(SF_ERR_ARG, "NULL buffer pointer");
    if (!aligned16(p)) return fail(SF_ERR_ALIGN, "buffer %p is not 16-byte aligned", p);
  }
  return SF_OK;
}

sf_status check_ctx(const sf_ctx* c) {
  if (!c) return fail(SF_ERR_ARG, "ctx is NULL");
  return SF_OK;
}

inline char* at(void* base, size_t off) { return static_cast<char*>(base) + off; }
inline const char* at(const void* base, size_t off) { return static_cast<const char*>(base) + off; }

}  // namespace

}  // namespace sf

using namespace sf;

sf_ctx::~sf_ctx() {
  if (side) (void)hipStreamSynchronize(side);
  for (hipEvent_t ev : {ev_fork[0], ev_fork[1], ev_fork[2], ev_fork[3], ev_mlp_dw, ev_join})
    if (ev) (void)hipEventDestroy(ev);
  if (side) (void)hipStreamDestroy(side);
}

extern "C" {


sf_status sf_ctx_create(const sf_shape* shape, int32_t head_chunk_rows, void* d_workspace, size_t workspace_bytes,
                        sf_ctx** out) {
  return sf_ctx_create_ex(shape, head_chunk_rows, 0, d_workspace, workspace_bytes, out);
}

sf_status sf_ctx_create_ex(const sf_shape* shape, int32_t head_chunk_rows, int32_t head_dw_rows, void* d_workspace,
                           size_t workspace_bytes, sf_ctx** out) {
  Dims d;
  sf_status st = check_shape(shape, &d);
  if (st) return st;
  if (!out) return fail(SF_ERR_ARG, "out is NULL");
  *out = nullptr;
  sf_layout L;
  st = sf_layer_layout_ex(shape, head_chunk_rows, head_dw_rows, &L);
  if (st) return st;
  int ndev = 0;
  if (hipGetDeviceCount(&ndev) != hipSuccess || ndev <= 0) return fail(SF_ERR_NO_DEVICE, "no HIP device");
  int dev = 0;
  SF_HIP(hipGetDevice(&dev));
  hipDeviceProp_t prop;
  SF_HIP(hipGetDeviceProperties(&prop, dev));
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(SF_ERR_NO_DEVICE, "device %d is %s, not gfx950", dev, prop.gcnArchName);
  const size_t need = L.workspace_bytes + (d.V > 0 ? L.head_workspace_bytes : 0);
  if (!d_workspace) return fail(SF_ERR_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_workspace) & 255u) return fail(SF_ERR_ALIGN, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(SF_ERR_POOL, "workspace has %zu bytes, needs %zu", workspace_bytes, need);
  sf_ctx* c = new sf_ctx();
  c->dims = d;
  c->layout = L;
  c->saved = saved_layout(d);
  c->work = work_layout(d, head_chunk_rows, head_dw_rows);
  c->head_chunk_rows = head_chunk_rows;
  c->head_dw_rows = head_dw_rows_eff(d.T, head_chunk_rows, head_dw_rows);
  c->ws = static_cast<char*>(d_workspace);
  c->ws_bytes = workspace_bytes;
  c->device = dev;
  // RoPE tables: phi[s, i] = s * base^(-2i/d), evaluated in double, stored fp32.
  const int half = d.d / 2;
  std::vector<float> cs(static_cast<size_t>(d.S) * half), sn(cs.size());
  for (int s = 0; s < d.S; ++s)
    for (int i = 0; i < half; ++i) {
      const double w = std::pow(static_cast<double>(d.rope_base), -2.0 * i / d.d);
      const double phi = s * w;
      cs[static_cast<size_t>(s) * half + i] = static_cast<float>(std::cos(phi));
      sn[static_cast<size_t>(s) * half + i] = static_cast<float>(std::sin(phi));
    }
  hipError_t e1 = hipMemcpy(c->ws + c->work.rope_cos, cs.data(), cs.size() * 4, hipMemcpyHostToDevice);
  hipError_t e2 = hipMemcpy(c->ws + c->work.rope_sin, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
  if (e1 != hipSuccess || e2 != hipSuccess) {
    delete c;
    return fail(SF_ERR_HIP, "uploading RoPE tables failed: %s", hipGetErrorString(e1 != hipSuccess ? e1 : e2));
  }
  // side stream for the weight-gradient GEMMs (default priority); the
  // environment variable SF_SERIAL_WGRAD=1 keeps them on the caller's stream
  const char* serial = std::getenv("SF_SERIAL_WGRAD");
  if (!(serial && serial[0] == '1')) {
    bool ok = hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) == hipSuccess;
    // The fork events hand data from the caller's stream to kernels on the
    // side stream of the same device only: no system-scope fence (which
    // writes caches back for the host) on the compute chain.  The join keeps
    // it, since the caller may copy the results out by DMA after it.
    for (hipEvent_t* ev : {&c->ev_fork[0], &c->ev_fork[1], &c->ev_fork[2], &c->ev_fork[3]})
      ok = ok && hipEventCreateWithFlags(ev, hipEventDisableTiming | hipEventDisableSystemFence) == hipSuccess;
    for (hipEvent_t* ev : {&c->ev_mlp_dw, &c->ev_join})
      ok = ok && hipEventCreateWithFlags(ev, hipEventDisableTiming) == hipSuccess;
    if (!ok) {
      delete c;
      return fail(SF_ERR_HIP, "creating the weight-gradient stream failed");
    }
  }
  *out = c;
  return SF_OK;
}

sf_status sf_ctx_destroy(sf_ctx* ctx) {
  delete ctx;
  return SF_OK;
}

sf_status sf_layer_fwd(sf_ctx* c, const void* d_w, const void* d_x, void* d_y, void* d_saved, sf_stream stream) {
  if (sf_status st = check_ctx(c)) return st;
  if (sf_status st = check_ptrs({d_w, d_x, d_y, d_saved})) return st;
  if (d_x == d_y) return fail(SF_ERR_ARG, "d_y may not alias d_x");
  const Dims& d = c->dims;
  const sf_layout& L = c->layout;
  const SavedLayout& sv = c->saved;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(d.T);
  char* ws = c->ws;
  float* const skw = reinterpret_cast<float*>(c->ws + c->work.splitk);
  const size_t skb = c->work.splitk_bytes;

  void* xn = at(d_saved, sv.xn);
  float* r1 = reinterpret_cast<float*>(at(d_saved, sv.r1));
  void* qkv = at(d_saved, sv.qkv);
  void* O = at(d_saved, sv.O);
  float* lse = reinterpret_cast<float*>(at(d_saved, sv.lse));
  void* h = at(d_saved, sv.h);
  void* hn = at(d_saved, sv.hn);
  float* r2 = reinterpret_cast<float*>(at(d_saved, sv.r2));
  void* G = at(d_saved, sv.G);
  void* U = at(d_saved, sv.U);
  void* a = at(d_saved, sv.a);

  SF_HIP(rmsnorm_fwd(d.dtype, d_x, at(d_w, L.off[SF_G1]), xn, r1, T, d.H, d.eps, s));

  GemmArgs g;
  g.A = xn; g.lda = d.H;
  g.B = at(d_w, L.off[SF_WQ]); g.ldb = d.H;
  g.C = qkv; g.ldc = d.Nqkv;
  g.M = T; g.N = d.Nqkv; g.K = d.H;
  g.rope_cos = reinterpret_cast<const float*>(ws + c->work.rope_cos);
  g.rope_sin = reinterpret_cast<const float*>(ws + c->work.rope_sin);
  g.seq = d.S; g.head_dim = d.d; g.rope_cols = d.Nq + d.Nkv;
  SF_HIP(gemm(d.dtype, GemmLayout::NT, Epi::Rope, g, s, skw, skb));

  AttnArgs at_;
  at_.qkv = qkv; at_.ld_qkv = d.Nqkv;
  at_.out = O; at_.ld_out = d.Nq;
  at_.lse = lse;
  at_.batch = d.B; at_.seq = d.S; at_.n_heads = d.nh; at_.n_kv = d.nkv; at_.head_dim = d.d;
  at_.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d.d)));
  SF_HIP(attention_fwd(d.dtype, at_, s));

  g = GemmArgs();
  g.A = O; g.lda = d.Nq;
  g.B = at(d_w, L.off[SF_WO]); g.ldb = d.Nq;
  g.C = h; g.ldc = d.H; g.R = d_x; g.ldr = d.H;
  g.M = T; g.N = d.H; g.K = d.Nq;
  SF_HIP(gemm(d.dtype, GemmLayout::NT, Epi::Resid, g, s, skw, skb));

  SF_HIP(rmsnorm_fwd(d.dtype, h, at(d_w, L.off[SF_G2]), hn, r2, T, d.H, d.eps, s));

  g = GemmArgs();
  g.A = hn; g.lda = d.H;
  g.B = at(d_w, L.off[SF_WG]); g.ldb = d.H;
  g.C = G; g.C2 = U; g.C3 = a; g.ldc = d.F;
  g.M = T; g.N = 2 * d.F; g.K = d.H; g.ffn = d.F;
  SF_HIP(gemm(d.dtype, GemmLayout::NT, Epi::SwigluFwd, g, s, skw, skb));

  g = GemmArgs();
  g.A = a; g.lda = d.F;
  g.B = at(d_w, L.off[SF_WD]); g.ldb = d.F;
  g.C = d_y; g.ldc = d.H; g.R = h; g.ldr = d.H;
  g.M = T; g.N = d.H; g.K = d.F;
  SF_HIP(gemm(d.dtype, GemmLayout::NT, Epi::Resid, g, s, skw, skb));
  return SF_OK;
}

sf_status sf_layer_bwd(sf_ctx* c, const void* d_w, const void* d_x, const void* d_saved, const void* d_dy,
                       void* d_dx, float* d_dw, sf_stream stream) {
  return sf::layer_bwd(c, d_w, d_x, d_saved, d_dy, d_dx, d_dw, stream, nullptr, nullptr);
}

}  // extern "C"

namespace sf {

sf_status layer_bwd(sf_ctx* c, const void* d_w, const void* d_x, const void* d_saved, const void* d_dy, void* d_dx,
                    float* d_dw, sf_stream stream, hipEvent_t ffn_done, hipEvent_t wd_done) {
  if (sf_status st = check_ctx(c)) return st;
  if (sf_status st = check_ptrs({d_w, d_x, d_saved, d_dy, d_dx, d_dw})) return st;
  const Dims& d = c->dims;
  const sf_layout& L = c->layout;
  const SavedLayout& sv = c->saved;
  const WorkLayout& wl = c->work;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(d.T);
  char* ws = c->ws;
  float* const skw = reinterpret_cast<float*>(c->ws + c->work.splitk);
  const size_t skb = c->work.splitk_bytes;
  char* dw = reinterpret_cast<char*>(d_dw);
  // The weight-gradient GEMMs depend on nothing the data-gradient chain
  // computes after them, so they run on the side stream `sw`, each started
  // once its operands exist (fork) and overlapping the rest of the chain;
  // their inputs (dy, saved activations, dGU, dh, dqkv) stay untouched until
  // the join at the end.  d_dx may alias d_dy, which the Wd gradient reads:
  // the chain waits for the MLP weight gradients before writing d_dx.
  // Where the largest of them ([2F, H]) covers two waves of 256 x 256 tiles
  // on its own, running them beside the chain gains nothing: all stay on s.
  const long dw_tiles = static_cast<long>((2 * d.F + 255) / 256) * ((d.H + 255) / 256);
  const bool side = c->side != nullptr && dw_tiles < 512;
  hipStream_t sw = side ? c->side : s;
  float* const skw_w = side ? reinterpret_cast<float*>(c->ws + wl.splitk_w) : skw;
  const size_t skb_w = side ? wl.splitk_w_bytes : skb;
  auto fork = [&](int k) -> sf_status {
    if (!side) return SF_OK;
    SF_HIP(hipEventRecord(c->ev_fork[k], s));
    SF_HIP(hipStreamWaitEvent(sw, c->ev_fork[k], 0));
    return SF_OK;
  };

  const void* xn = at(d_saved, sv.xn);
  const float* r1 = reinterpret_cast<const float*>(at(d_saved, sv.r1));
  const void* qkv = at(d_saved, sv.qkv);
  const void* O = at(d_saved, sv.O);
  const float* lse = reinterpret_cast<const float*>(at(d_saved, sv.lse));
  const void* h = at(d_saved, sv.h);
  const void* hn = at(d_saved, sv.hn);
  const float* r2 = reinterpret_cast<const float*>(at(d_saved, sv.r2));
  const void* G = at(d_saved, sv.G);
  const void* U = at(d_saved, sv.U);
  const void* a = at(d_saved, sv.a);
  char* dGU = ws + wl.dGU;
  void* dhn = ws + wl.dhn;
  void* dh = ws + wl.dh;
  void* dA = ws + wl.dA;
  float* dsum = reinterpret_cast<float*>(ws + wl.dsum);
  void* dqkv = ws + wl.dqkv;
  void* dxn = ws + wl.dxn;
  float* partial = reinterpret_cast<float*>(ws + wl.gain_partial);

  // down projection: da = dy Wd fused with SwiGLU backward -> [dG | dU]
  GemmArgs g;
  g.A = d_dy; g.lda = d.H;
  g.B = at(d_w, L.off[SF_WD]); g.ldb = d.F;
  g.C = dGU; g.C2 = dGU + static_cast<size_t>(d.F) * d.e; g.ldc = 2 * d.F;
  g.R = G; g.R2 = U; g.ldr = d.F;
  g.M = T; g.N = d.F; g.K = d.H;
  // dWd = dy^T a needs only dy and the saved a: it starts with the chain
  if (sf_status st = fork(0)) return st;
  SF_HIP(gemm(d.dtype, GemmLayout::NN, Epi::SwigluBwd, g, s, skw, skb));
  {
    GemmArgs gw;
    gw.A = d_dy; gw.lda = d.H;
    gw.B = a; gw.ldb = d.F;
    gw.C = dw + L.grad_off[SF_WD]; gw.ldc = d.F;
    gw.M = d.H; gw.N = d.F; gw.K = T;
    SF_HIP(gemm(d.dtype, GemmLayout::TN, Epi::StoreF32, gw, sw, skw_w, skb_w));
    if (wd_done) SF_HIP(hipEventRecord(wd_done, sw));
  }
  if (sf_status st = fork(1)) return st;  // dGU exists
  // dhn = [dG | dU] [Wg; Wu]
  g = GemmArgs();
  g.A = dGU; g.lda = 2 * d.F;
  g.B = at(d_w, L.off[SF_WG]); g.ldb = d.H;
  g.C = dhn; g.ldc = d.H;
  g.M = T; g.N = d.H; g.K = 2 * d.F;
  SF_HIP(gemm(d.dtype, GemmLayout::NN, Epi::Store, g, s, skw, skb));
  // [dWg; dWu] = [dG | dU]^T hn
  g = GemmArgs();
  g.A = dGU; g.lda = 2 * d.F;
  g.B = hn; g.ldb = d.H;
  g.C = dw + L.grad_off[SF_WG]; g.ldc = d.H;
  g.M = 2 * d.F; g.N = d.H; g.K = T;
  SF_HIP(gemm(d.dtype, GemmLayout::TN, Epi::StoreF32, g, sw, skw_w, skb_w));
  // the MLP weight gradients (Wg, Wu, Wd) are final from here on
  if (ffn_done) SF_HIP(hipEventRecord(ffn_done, sw));
  if (side) SF_HIP(hipEventRecord(c->ev_mlp_dw, sw));
  // RMSNorm-2 backward (+ residual dy) -> dh, dg2
  SF_HIP(rmsnorm_bwd(d.dtype, dhn, h, r2, at(d_w, L.off[SF_G2]), d_dy, dh, partial, kGainChunks,
                     reinterpret_cast<float*>(dw + L.grad_off[SF_G2]), T, d.H, s));
  if (sf_status st = fork(2)) return st;  // dh exists
  // dA = dh Wo
  g = GemmArgs();
  g.A = dh; g.lda = d.H;
  g.B = at(d_w, L.off[SF_WO]); g.ldb = d.Nq;
  g.C = dA; g.ldc = d.Nq;
  g.M = T; g.N = d.Nq; g.K = d.H;
  SF_HIP(gemm(d.dtype, GemmLayout::NN, Epi::Store, g, s, skw, skb));
  // dWo = dh^T A
  g = GemmArgs();
  g.A = dh; g.lda = d.H;
  g.B = O; g.ldb = d.Nq;
  g.C = dw + L.grad_off[SF_WO]; g.ldc = d.Nq;
  g.M = d.H; g.N = d.Nq; g.K = T;
  SF_HIP(gemm(d.dtype, GemmLayout::TN, Epi::StoreF32, g, sw, skw_w, skb_w));
  // attention backward (+ inverse RoPE) -> [dq | dk | dv]
  AttnArgs at_;
  at_.qkv = qkv; at_.ld_qkv = d.Nqkv;
  at_.out = const_cast<void*>(O); at_.ld_out = d.Nq;
  at_.dout = dA; at_.ld_dout = d.Nq;
  at_.dqkv = dqkv; at_.ld_dqkv = d.Nqkv;
  at_.lse = const_cast<float*>(lse); at_.dsum = dsum;
  at_.rope_cos = reinterpret_cast<const float*>(ws + wl.rope_cos);
  at_.rope_sin = reinterpret_cast<const float*>(ws + wl.rope_sin);
  at_.batch = d.B; at_.seq = d.S; at_.n_heads = d.nh; at_.n_kv = d.nkv; at_.head_dim = d.d;
  at_.scale = static_cast<float>(1.0 / std::sqrt(static_cast<double>(d.d)));
  at_.kv_split = wl.kv_split;
  at_.dkv_partial = reinterpret_cast<float*>(ws + wl.dkv_partial);
  SF_HIP(attention_bwd(d.dtype, at_, s));
  if (sf_status st = fork(3)) return st;  // dqkv exists
  // dxn = [dq | dk | dv] Wqkv
  g = GemmArgs();
  g.A = dqkv; g.lda = d.Nqkv;
  g.B = at(d_w, L.off[SF_WQ]); g.ldb = d.H;
  g.C = dxn; g.ldc = d.H;
  g.M = T; g.N = d.H; g.K = d.Nqkv;
  SF_HIP(gemm(d.dtype, GemmLayout::NN, Epi::Store, g, s, skw, skb));
  // dWqkv = [dq | dk | dv]^T xn
  g = GemmArgs();
  g.A = dqkv; g.lda = d.Nqkv;
  g.B = xn; g.ldb = d.H;
  g.C = dw + L.grad_off[SF_WQ]; g.ldc = d.H;
  g.M = d.Nqkv; g.N = d.H; g.K = T;
  SF_HIP(gemm(d.dtype, GemmLayout::TN, Epi::StoreF32, g, sw, skw_w, skb_w));
  // RMSNorm-1 backward (+ residual dh) -> dx, dg1; d_dx may alias d_dy
  if (side) SF_HIP(hipStreamWaitEvent(s, c->ev_mlp_dw, 0));
  SF_HIP(rmsnorm_bwd(d.dtype, dxn, d_x, r1, at(d_w, L.off[SF_G1]), dh, d_dx, partial, kGainChunks,
                     reinterpret_cast<float*>(dw + L.grad_off[SF_G1]), T, d.H, s));
  if (side) {
    SF_HIP(hipEventRecord(c->ev_join, sw));
    SF_HIP(hipStreamWaitEvent(s, c->ev_join, 0));
  }
  return SF_OK;
}

}  // namespace sf

namespace sf {

// The LM-head weight gradient of the last (or only) row chunk: dW_lm (=, or
// += after earlier chunks) dlogits^T hf, from the head workspace the head
// pass left.  No split-K workspace: it may run beside the layer backward.
sf_status head_last_dw(sf_ctx* c, float* d_dwlm, sf_stream stream) {
  const Dims& d = c->dims;
  const WorkLayout& wl = c->work;
  const int T = static_cast<int>(d.T);
  const int D = c->head_dw_rows;  // the last group of dlogits rows
  const int r0 = ((T - 1) / D) * D;
  GemmArgs g;
  g.A = c->ws + wl.dlogits; g.lda = d.V;
  g.B = c->ws + wl.hf + static_cast<size_t>(r0) * d.H * d.e; g.ldb = d.H;
  g.C = d_dwlm; g.ldc = d.H;
  g.M = d.V; g.N = d.H; g.K = T - r0;
  SF_HIP(gemm(d.dtype, GemmLayout::TN, r0 == 0 ? Epi::StoreF32 : Epi::AccF32, g, static_cast<hipStream_t>(stream),
              nullptr, 0));
  return SF_OK;
}

sf_status head_fwd_bwd(sf_ctx* c, const void* d_gf, const void* d_wlm, const void* d_x, const int32_t* d_ids,
                       float* d_loss, void* d_dx, float* d_dgf, float* d_dwlm, sf_stream stream, bool defer_last_dw,
                       float grad_scale) {
  if (sf_status st = check_ctx(c)) return st;
  if (!(grad_scale > 0.f) || !std::isfinite(grad_scale)) return fail(SF_ERR_ARG, "grad_scale must be finite and > 0");
  if (sf_status st = check_ptrs({d_gf, d_wlm, d_x, d_ids, d_dx, d_dgf, d_dwlm})) return st;
  if (!d_loss) return fail(SF_ERR_ARG, "d_loss is NULL");
  const Dims& d = c->dims;
  if (d.V <= 0) return fail(SF_ERR_ARG, "context was created with vocab = 0");
  if (d.S < 2) return fail(SF_ERR_ARG, "next-token loss needs seq >= 2");
  const WorkLayout& wl = c->work;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int T = static_cast<int>(d.T);
  char* ws = c->ws;
  float* const skw = reinterpret_cast<float*>(c->ws + c->work.splitk);
  const size_t skb = c->work.splitk_bytes;
  void* hf = ws + wl.hf;
  float* rf = reinterpret_cast<float*>(ws + wl.rf);
  char* dhf = ws + wl.dhf;
  float* logits = reinterpret_cast<float*>(ws + wl.logits);
  void* dlogits = ws + wl.dlogits;
  float* loss_rows = reinterpret_cast<float*>(ws + wl.loss_rows);
  float* partial = reinterpret_cast<float*>(ws + wl.gain_partial);
  const float inv_n = 1.0f / (static_cast<float>(d.B) * static_cast<float>(d.S - 1));

  SF_HIP(rmsnorm_fwd(d.dtype, d_x, d_gf, hf, rf, T, d.H, d.eps, s));
  // Row chunks of R: logits, cross entropy and dlogits, dx.  dlogits of a
  // group of D rows (D a multiple of R) stay in the workspace, and each
  // group adds its dW_lm = dlogits^T hf in one product: the fp32 dW_lm is
  // read and written once per group rather than once per chunk.
  const int R = c->head_chunk_rows, D = c->head_dw_rows;
  for (int r0 = 0; r0 < T; r0 += R) {
    const int rows = std::min(R, T - r0);
    const int g0 = r0 / D * D;  // first row of this chunk's group
    char* dlc = static_cast<char*>(dlogits) + static_cast<size_t>(r0 - g0) * d.V * d.e;
    const char* hfc = static_cast<const char*>(hf) + static_cast<size_t>(r0) * d.H * d.e;
    GemmArgs g;
    g.A = hfc; g.lda = d.H;
    g.B = d_wlm; g.ldb = d.H;
    g.C = logits; g.ldc = d.V;
    g.M = rows; g.N = d.V; g.K = d.H;
    SF_HIP(gemm(d.dtype, GemmLayout::NT, Epi::StoreF32, g, s, skw, skb));
    SF_HIP(ce_rows(d.dtype, logits, d_ids, dlc, loss_rows, r0, rows, d.V, d.S, inv_n * grad_scale, s));
    g = GemmArgs();
    g.A = dlc; g.lda = d.V;
    g.B = d_wlm; g.ldb = d.H;
    g.C = dhf + static_cast<size_t>(r0) * d.H * d.e; g.ldc = d.H;
    g.M = rows; g.N = d.H; g.K = d.V;
    SF_HIP(gemm(d.dtype, GemmLayout::NN, Epi::Store, g, s, skw, skb));
    const int end = r0 + rows;
    if (end % D != 0 && end < T) continue;  // the group goes on
    if (defer_last_dw && end >= T) break;   // the caller runs head_last_dw later
    g = GemmArgs();
    g.A = dlogits; g.lda = d.V;
    g.B = static_cast<const char*>(hf) + static_cast<size_t>(g0) * d.H * d.e; g.ldb = d.H;
    g.C = d_dwlm; g.ldc = d.H;
    g.M = d.V; g.N = d.H; g.K = end - g0;
    SF_HIP(gemm(d.dtype, GemmLayout::TN, g0 == 0 ? Epi::StoreF32 : Epi::AccF32, g, s, skw, skb));
  }
  SF_HIP(loss_reduce(loss_rows, d_loss, T, inv_n, s));
  SF_HIP(rmsnorm_bwd(d.dtype, dhf, d_x, rf, d_gf, nullptr, d_dx, partial, kGainChunks, d_dgf, T, d.H, s));
  return SF_OK;
}

}  // namespace sf

extern "C" {

sf_status sf_head_fwd_bwd(sf_ctx* c, const void* d_gf, const void* d_wlm, const void* d_x, const int32_t* d_ids,
                          float* d_loss, void* d_dx, float* d_dgf, float* d_dwlm, sf_stream stream) {
  return sf::head_fwd_bwd(c, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, stream, false);
}

sf_status sf_head_fwd_bwd_scaled(sf_ctx* c, const void* d_gf, const void* d_wlm, const void* d_x,
                                 const int32_t* d_ids, float* d_loss, void* d_dx, float* d_dgf, float* d_dwlm,
                                 float grad_scale, sf_stream stream) {
  return sf::head_fwd_bwd(c, d_gf, d_wlm, d_x, d_ids, d_loss, d_dx, d_dgf, d_dwlm, stream, false, grad_scale);
}

size_t sf_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return gemm_splitk_bytes(M, N, K);
}

}  // extern "C"

namespace {

// Checks shared by sf_gemm and sf_gemm_noalloc; fills *g.  *empty: nothing
// to compute (M or N is 0).
sf_status gemm_args(int32_t dtype, int32_t layout, int32_t M, int32_t N, int32_t K, const void* d_A, int64_t lda,
                    const void* d_B, int64_t ldb, void* d_C, int64_t ldc, GemmArgs* g, bool* empty) {
  *empty = false;
  if (dtype != SF_F32 && dtype != SF_BF16 && dtype != SF_F16) return fail(SF_ERR_ARG, "bad dtype %d", dtype);
  if (layout < 0 || layout > 2) return fail(SF_ERR_ARG, "bad layout %d", layout);
  if (M < 0 || N < 0 || K < 0) return fail(SF_ERR_ARG, "negative size");
  if (M == 0 || N == 0) {
    *empty = true;
    return SF_OK;
  }
  if (sf_status st = check_ptrs({d_A, d_B, d_C})) return st;
  // contiguous dimensions of A, B, C and N itself in multiples of 8 elements
  const int64_t a_contig = layout == 2 ? M : K;
  const int64_t b_contig = layout == 0 ? K : N;
  if (a_contig % 8 || b_contig % 8 || N % 8 || lda % 8 || ldb % 8 || ldc % 8)
    return fail(SF_ERR_UNSUPPORTED, "contiguous dimensions and leading dimensions must be multiples of 8");
  if (lda < a_contig || ldb < b_contig || ldc < N) return fail(SF_ERR_ARG, "leading dimension too small");
  g->A = d_A; g->lda = lda;
  g->B = d_B; g->ldb = ldb;
  g->C = d_C; g->ldc = ldc;
  g->M = M; g->N = N; g->K = K;
  return SF_OK;
}

}  // namespace

extern "C" {

sf_status sf_gemm(int32_t dtype, int32_t layout, int32_t out_f32, int32_t M, int32_t N, int32_t K, const void* d_A,
                  int64_t lda, const void* d_B, int64_t ldb, void* d_C, int64_t ldc, void* d_workspace,
                  size_t workspace_bytes, sf_stream stream) {
  GemmArgs g;
  bool empty = false;
  if (sf_status st = gemm_args(dtype, layout, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, &g, &empty)) return st;
  if (empty) return SF_OK;
  if (d_workspace && !aligned16(d_workspace)) return fail(SF_ERR_ALIGN, "workspace is not 16-byte aligned");
  SF_HIP(gemm(dtype, static_cast<GemmLayout>(layout), out_f32 ? Epi::StoreF32 : Epi::Store, g,
              static_cast<hipStream_t>(stream), static_cast<float*>(d_workspace),
              d_workspace ? workspace_bytes : 0));
  return SF_OK;
}

sf_status sf_gemm_noalloc(int32_t dtype, int32_t layout, int32_t out_f32, int32_t M, int32_t N, int32_t K,
                          const void* d_A, int64_t lda, const void* d_B, int64_t ldb, void* d_C, int64_t ldc,
                          sf_stream stream) {
  GemmArgs g;
  bool empty = false;
  if (sf_status st = gemm_args(dtype, layout, M, N, K, d_A, lda, d_B, ldb, d_C, ldc, &g, &empty)) return st;
  if (empty) return SF_OK;
  const size_t need = K > 0 ? gemm_splitk_bytes(M, N, K) : 0;
  if (need > kGemmStaticScratchBytes)
    return fail(SF_ERR_POOL, "this product splits K into partial sums of %zu bytes; the static scratch holds %zu",
                need, kGemmStaticScratchBytes);
  float* ws = nullptr;
  SF_HIP(gemm_static_scratch(&ws));
  SF_HIP(gemm(dtype, static_cast<GemmLayout>(layout), out_f32 ? Epi::StoreF32 : Epi::Store, g,
              static_cast<hipStream_t>(stream), ws, kGemmStaticScratchBytes));
  return SF_OK;
}

sf_status sf_adam_device_ex(int32_t dtype, float* d_p, float* d_m, float* d_v, const float* d_g, void* d_out,
                            size_t n, int64_t step, float lr, float b1, float b2, float eps, float grad_scale,
                            sf_stream stream) {
  if (dtype != SF_F32 && dtype != SF_BF16 && dtype != SF_F16) return fail(SF_ERR_ARG, "bad dtype %d", dtype);
  if (!(grad_scale > 0.f) || !std::isfinite(grad_scale)) return fail(SF_ERR_ARG, "grad_scale must be finite and > 0");
  if (n == 0) return SF_OK;
  if (!d_p || !d_m || !d_v || !d_g) return fail(SF_ERR_ARG, "NULL array");
  if (step < 1) return fail(SF_ERR_ARG, "step must be >= 1");
  const AdamCoef c = adam_coef(step, lr, b1, b2, eps);
  // without a storage copy the kernel writes the copy over the master (same value)
  void* out = d_out ? d_out : (dtype == SF_F32 ? static_cast<void*>(d_p) : nullptr);
  if (!out) return fail(SF_ERR_ARG, "16-bit storage copy needs d_out");
  SF_HIP(adam_device(dtype, d_p, d_m, d_v, d_g, out, static_cast<int64_t>(n), c.b1, c.b2, c.one_b1, c.one_b2,
                     c.inv_bc1, c.inv_bc2, c.lr, c.eps, static_cast<hipStream_t>(stream), grad_scale));
  return SF_OK;
}

sf_status sf_adam_device(int32_t dtype, float* d_p, float* d_m, float* d_v, const float* d_g, void* d_out, size_t n,
                         int64_t step, float lr, float b1, float b2, float eps, sf_stream stream) {
  return sf_adam_device_ex(dtype, d_p, d_m, d_v, d_g, d_out, n, step, lr, b1, b2, eps, 1.0f, stream);
}

sf_status sf_embed_fwd(sf_ctx* c, const void* d_E, const int32_t* d_ids, void* d_x0, sf_stream stream) {
  if (sf_status st = check_ctx(c)) return st;
  if (sf_status st = check_ptrs({d_E, d_ids, d_x0})) return st;
  const Dims& d = c->dims;
  if (d.V <= 0) return fail(SF_ERR_ARG, "context was created with vocab = 0");
  SF_HIP(embed_fwd(d.dtype, d_E, d_ids, d_x0, static_cast<int>(d.T), d.H, d.V, static_cast<hipStream_t>(stream)));
  return SF_OK;
}

sf_status sf_embed_bwd(sf_ctx* c, const void* d_dx0, const int32_t* d_ids, float* d_dE, sf_stream stream) {
  if (sf_status st = check_ctx(c)) return st;
  if (sf_status st = check_ptrs({d_dx0, d_ids, d_dE})) return st;
  const Dims& d = c->dims;
  if (d.V <= 0) return fail(SF_ERR_ARG, "context was created with vocab = 0");
  SF_HIP(embed_bwd(d.dtype, d_dx0, d_ids, d_dE, static_cast<int>(d.T), d.H, d.V, static_cast<hipStream_t>(stream)));
  return SF_OK;
}

}  // extern "C"

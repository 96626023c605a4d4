// Shape validation, buffer layouts and the thread-local error text of the C
// ABI: host code only (no device calls), shared by the library and the CPU
// build of the sliding engine's host logic.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "attention.h"
#include "gemm.h"
#include "internal.h"
#include "rowops.h"

namespace sf {

namespace {
thread_local std::string g_last_error;
}

void set_error(const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
}

sf_status fail(sf_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

sf_status check_shape(const sf_shape* s, Dims* out) {
  if (!s) return fail(SF_ERR_ARG, "shape is NULL");
  if (s->dtype != SF_F32 && s->dtype != SF_BF16 && s->dtype != SF_F16)
    return fail(SF_ERR_ARG, "dtype %d is not SF_F32/SF_BF16/SF_F16", s->dtype);
  if (s->hidden <= 0 || s->n_heads <= 0 || s->n_kv_heads <= 0 || s->head_dim <= 0 || s->ffn <= 0 ||
      s->batch <= 0 || s->seq <= 0 || s->vocab < 0)
    return fail(SF_ERR_ARG, "non-positive size in shape");
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(SF_ERR_UNSUPPORTED, "head_dim %d not in {64, 128}", s->head_dim);
  if (s->n_heads % s->n_kv_heads != 0)
    return fail(SF_ERR_UNSUPPORTED, "n_heads %d not a multiple of n_kv_heads %d", s->n_heads, s->n_kv_heads);
  if (s->hidden % 8 || s->ffn % 8 || s->vocab % 8)
    return fail(SF_ERR_UNSUPPORTED, "hidden, ffn and vocab must be multiples of 8");
  if (!(s->rms_eps >= 0.f) || !(s->rope_base > 0.f)) return fail(SF_ERR_ARG, "rms_eps must be >= 0, rope_base > 0");
  const int64_t T = static_cast<int64_t>(s->batch) * s->seq;
  if (T > (1 << 30) || static_cast<int64_t>(s->hidden) * 4 > (1 << 30))
    return fail(SF_ERR_UNSUPPORTED, "sizes exceed 32-bit row indexing");
  Dims d;
  d.H = s->hidden; d.nh = s->n_heads; d.nkv = s->n_kv_heads; d.d = s->head_dim; d.F = s->ffn;
  d.V = s->vocab; d.B = s->batch; d.S = s->seq; d.T = T;
  d.Nq = d.nh * d.d; d.Nkv = d.nkv * d.d; d.Nqkv = d.Nq + 2 * d.Nkv;
  d.dtype = s->dtype; d.e = s->dtype == SF_F32 ? 4 : 2;
  d.eps = s->rms_eps; d.rope_base = s->rope_base;
  if (out) *out = d;
  return SF_OK;
}

// Tensor order Wq Wk Wv | Wo | Wg Wu | Wd | g1 | g2; '|' = 256-B boundary.
void param_layout(const Dims& d, size_t elem, size_t* off, size_t* bytes, size_t* total) {
  const size_t H = d.H, F = d.F;
  bytes[SF_WQ] = d.Nq * H * elem;
  bytes[SF_WK] = d.Nkv * H * elem;
  bytes[SF_WV] = d.Nkv * H * elem;
  bytes[SF_WO] = H * d.Nq * elem;
  bytes[SF_WG] = F * H * elem;
  bytes[SF_WU] = F * H * elem;
  bytes[SF_WD] = H * F * elem;
  bytes[SF_G1] = H * elem;
  bytes[SF_G2] = H * elem;
  off[SF_WQ] = 0;
  off[SF_WK] = off[SF_WQ] + bytes[SF_WQ];
  off[SF_WV] = off[SF_WK] + bytes[SF_WK];
  off[SF_WO] = align256(off[SF_WV] + bytes[SF_WV]);
  off[SF_WG] = align256(off[SF_WO] + bytes[SF_WO]);
  off[SF_WU] = off[SF_WG] + bytes[SF_WG];
  off[SF_WD] = align256(off[SF_WU] + bytes[SF_WU]);
  off[SF_G1] = align256(off[SF_WD] + bytes[SF_WD]);
  off[SF_G2] = align256(off[SF_G1] + bytes[SF_G1]);
  *total = align256(off[SF_G2] + bytes[SF_G2]);
}

SavedLayout saved_layout(const Dims& d) {
  SavedLayout s;
  const size_t T = d.T, e = d.e;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o = align256(o + bytes); return r; };
  s.xn = take(T * d.H * e);
  s.r1 = take(T * 4);
  s.qkv = take(T * d.Nqkv * e);
  s.O = take(T * d.Nq * e);
  s.lse = take(static_cast<size_t>(d.B) * d.nh * d.S * 4);
  s.h = take(T * d.H * e);
  s.hn = take(T * d.H * e);
  s.r2 = take(T * 4);
  s.G = take(T * d.F * e);
  s.U = take(T * d.F * e);
  s.a = take(T * d.F * e);
  s.total = o;
  return s;
}

int head_dw_rows_eff(int64_t T, int head_chunk_rows, int head_dw_rows) {
  const int64_t R = head_chunk_rows > 0 ? head_chunk_rows : 1;
  if (head_dw_rows <= R) return static_cast<int>(R);
  const int64_t all = (T + R - 1) / R * R;
  return static_cast<int>(std::min<int64_t>(all, (head_dw_rows + R - 1) / R * R));
}

WorkLayout work_layout(const Dims& d, int head_chunk_rows, int head_dw_rows) {
  WorkLayout w;
  const size_t T = d.T, e = d.e;
  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t r = o; o = align256(o + bytes); return r; };
  w.rope_cos = take(static_cast<size_t>(d.S) * (d.d / 2) * 4);
  w.rope_sin = take(static_cast<size_t>(d.S) * (d.d / 2) * 4);
  w.dGU = take(T * 2 * d.F * e);
  w.dhn = take(T * d.H * e);
  w.dh = take(T * d.H * e);
  w.dA = take(T * d.Nq * e);
  w.dsum = take(static_cast<size_t>(d.B) * d.nh * d.S * 4);
  w.dqkv = take(T * d.Nqkv * e);
  w.dxn = take(T * d.H * e);
  w.gain_partial = take(static_cast<size_t>(kGainChunks) * d.H * 4);
  // the 16-bit attention backward may split a GQA group's query heads
  w.kv_split = d.dtype != SF_F32 ? attn_kv_split(d.B, d.S, d.nh, d.nkv) : 1;
  w.dkv_partial = take(static_cast<size_t>(attn_kv_partial_bytes(w.kv_split, d.B, d.S, d.nkv, d.d)));
  // split-K scratch: the largest any projection of the layer or head asks for
  {
    const int Ti = static_cast<int>(d.T);
    size_t sk = 0;
    auto upd = [&](int M, int N, int K) { sk = std::max(sk, gemm_splitk_bytes(M, N, K)); };
    upd(Ti, d.Nqkv, d.H); upd(Ti, d.H, d.Nq); upd(Ti, 2 * d.F, d.H); upd(Ti, d.H, d.F);
    upd(Ti, d.F, d.H); upd(d.H, d.F, Ti); upd(Ti, d.H, 2 * d.F); upd(2 * d.F, d.H, Ti);
    upd(Ti, d.Nq, d.H); upd(d.H, d.Nq, Ti); upd(Ti, d.H, d.Nqkv); upd(d.Nqkv, d.H, Ti);
    if (d.V > 0) {
      const int R = std::min(Ti, head_chunk_rows > 0 ? head_chunk_rows : 1);
      upd(R, d.V, d.H); upd(R, d.H, d.V); upd(d.V, d.H, R);
      upd(d.V, d.H, head_dw_rows_eff(d.T, head_chunk_rows, head_dw_rows));
    }
    w.splitk = take(sk);
    w.splitk_bytes = sk;
    // the weight-gradient GEMMs run beside the data-gradient chain: own scratch
    sk = 0;
    upd(d.H, d.F, Ti); upd(2 * d.F, d.H, Ti); upd(d.H, d.Nq, Ti); upd(d.Nqkv, d.H, Ti);
    w.splitk_w = take(sk);
    w.splitk_w_bytes = sk;
  }
  w.total = o;
  if (d.V > 0) {
    const size_t R = static_cast<size_t>(head_chunk_rows > 0 ? head_chunk_rows : 1);
    w.hf = take(T * d.H * e);
    w.rf = take(T * 4);
    w.dhf = take(T * d.H * e);
    w.logits = take(R * d.V * 4);
    w.dlogits = take(static_cast<size_t>(head_dw_rows_eff(d.T, head_chunk_rows, head_dw_rows)) * d.V * e);
    w.loss_rows = take(T * 4);
  } else {
    w.hf = w.rf = w.dhf = w.logits = w.dlogits = w.loss_rows = 0;
  }
  w.head_total = o - w.total;
  return w;
}

}  // namespace sf

using namespace sf;

extern "C" {

const char* sf_last_error(void) { return sf::g_last_error.c_str(); }

sf_status sf_layer_layout_ex(const sf_shape* shape, int32_t head_chunk_rows, int32_t head_dw_rows,
                             sf_layout* out) {
  Dims d;
  sf_status st = check_shape(shape, &d);
  if (st) return st;
  if (!out) return fail(SF_ERR_ARG, "out is NULL");
  if (d.V > 0 && head_chunk_rows <= 0) return fail(SF_ERR_ARG, "head_chunk_rows must be >= 1");
  if (head_dw_rows < 0) return fail(SF_ERR_ARG, "head_dw_rows must be >= 0");
  sf_layout L;
  std::memset(&L, 0, sizeof L);
  param_layout(d, d.e, L.off, L.bytes, &L.param_bytes);
  param_layout(d, 4, L.grad_off, L.grad_bytes_t, &L.grad_bytes);
  L.n_params = static_cast<size_t>(d.Nqkv) * d.H + static_cast<size_t>(d.H) * d.Nq +
               3 * static_cast<size_t>(d.F) * d.H + 2 * static_cast<size_t>(d.H);
  L.saved_bytes = saved_layout(d).total;
  const WorkLayout w = work_layout(d, head_chunk_rows, head_dw_rows);
  L.workspace_bytes = w.total;
  L.head_workspace_bytes = w.head_total;
  *out = L;
  return SF_OK;
}

sf_status sf_layer_layout(const sf_shape* shape, int32_t head_chunk_rows, sf_layout* out) {
  return sf_layer_layout_ex(shape, head_chunk_rows, 0, out);
}

}  // extern "C"

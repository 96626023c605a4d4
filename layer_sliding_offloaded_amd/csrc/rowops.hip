// Row-wise kernels: RMSNorm forward/backward, gain-gradient reduction,
// embedding gather/scatter, cross-entropy rows and the loss reduction.
//
// All are HBM-bound.  A wavefront owns one row and walks it in 16-byte
// vectors (64 lanes x 16 B = 1 KiB per step, fully coalesced); row
// statistics are reduced with cross-lane shuffles.  Column reductions over
// tokens (gain gradients, the loss) go through fixed-order partial sums, never
// floating-point atomics, so results are bitwise reproducible.
#include <math.h>

#include <algorithm>

#include "common.h"
#include "rowops.h"

namespace sf {

namespace {

template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float* f) {
  Elem<T>::unpack(*reinterpret_cast<const uint4*>(p), f);
}
template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float* f) {
  *reinterpret_cast<uint4*>(p) = Elem<T>::pack(f);
}

// RMSNorm forward: r = (mean x^2 + eps)^-1/2, y = x r g.
template <typename T>
__global__ void __launch_bounds__(256)
rmsnorm_fwd_kernel(const T* __restrict__ x, const T* __restrict__ g, T* __restrict__ y,
                   float* __restrict__ r, int rows, int H, float eps) {
  constexpr int VE = 16 / sizeof(T);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* xr = x + static_cast<int64_t>(row) * H;
  float ss = 0.f;
  for (int c = lane * VE; c < H; c += 64 * VE) {
    float f[VE];
    load_vec<T>(xr + c, f);
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  const float rr = 1.0f / sqrtf(ss / H + eps);
  if (lane == 0) r[row] = rr;
  T* yr = y + static_cast<int64_t>(row) * H;
  for (int c = lane * VE; c < H; c += 64 * VE) {
    float f[VE], gg[VE];
    load_vec<T>(xr + c, f);
    load_vec<T>(g + c, gg);
#pragma unroll
    for (int e = 0; e < VE; ++e) f[e] = f[e] * rr * gg[e];
    store_vec<T>(yr + c, f);
  }
}

// Wide rows, H = NC x 256 x VE (NC = 2 .. 8): a block of four waves owns a
// row and each thread holds NC 16-byte vectors of it in registers, so the
// row crosses HBM once (the wave-per-row kernels read it twice: once for the
// row statistic, once for the output).  The statistic is the sum of the four
// waves' sums, added in wave order.
template <typename T, int NC>
__global__ void __launch_bounds__(256)
rmsnorm_fwd_rows_kernel(const T* __restrict__ x, const T* __restrict__ g, T* __restrict__ y,
                        float* __restrict__ r, int H, float eps) {
  constexpr int VE = 16 / sizeof(T);
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * H;
  uint4 xq[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) xq[k] = *reinterpret_cast<const uint4*>(x + base + (k * 256 + tid) * VE);
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    float f[VE];
    Elem<T>::unpack(xq[k], f);
#pragma unroll
    for (int e = 0; e < VE; ++e) ss += f[e] * f[e];
  }
  ss = wave_sum(ss);
  if (lane == 0) part[w] = ss;
  __syncthreads();
  const float rr = 1.0f / sqrtf((((part[0] + part[1]) + part[2]) + part[3]) / H + eps);
  if (tid == 0) r[blockIdx.x] = rr;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    float f[VE], gg[VE];
    Elem<T>::unpack(xq[k], f);
    load_vec<T>(g + (k * 256 + tid) * VE, gg);
#pragma unroll
    for (int e = 0; e < VE; ++e) f[e] = f[e] * rr * gg[e];
    store_vec<T>(y + base + (k * 256 + tid) * VE, f);
  }
}

// RMSNorm backward (input part) for wide rows, one HBM pass: as
// rmsnorm_bwd_kernel below, with the row in registers (layout as above).
template <typename T, int NC>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_rows_kernel(const T* __restrict__ dout, const T* __restrict__ xin, const float* __restrict__ r,
                        const T* __restrict__ g, const T* __restrict__ resid, T* __restrict__ dx, int H) {
  constexpr int VE = 16 / sizeof(T);
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t base = static_cast<int64_t>(blockIdx.x) * H;
  const float rr = r[blockIdx.x];
  uint4 dq[NC], xq[NC], gq[NC], rq[NC];
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int c = (k * 256 + tid) * VE;
    dq[k] = *reinterpret_cast<const uint4*>(dout + base + c);
    xq[k] = *reinterpret_cast<const uint4*>(xin + base + c);
    gq[k] = *reinterpret_cast<const uint4*>(g + c);
    rq[k] = resid ? *reinterpret_cast<const uint4*>(resid + base + c) : make_uint4(0, 0, 0, 0);
  }
  float dot = 0.f;
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    float d[VE], xv[VE], gg[VE];
    Elem<T>::unpack(dq[k], d);
    Elem<T>::unpack(xq[k], xv);
    Elem<T>::unpack(gq[k], gg);
#pragma unroll
    for (int e = 0; e < VE; ++e) dot += d[e] * gg[e] * xv[e];
  }
  dot = wave_sum(dot);
  if (lane == 0) part[w] = dot;
  __syncthreads();
  const float proj = (((part[0] + part[1]) + part[2]) + part[3]) * rr / H;  // mean(dn * n)
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    float d[VE], xv[VE], gg[VE], o[VE];
    Elem<T>::unpack(dq[k], d);
    Elem<T>::unpack(xq[k], xv);
    Elem<T>::unpack(gq[k], gg);
    Elem<T>::unpack(rq[k], o);  // zeros (all bits clear) without a residual
#pragma unroll
    for (int e = 0; e < VE; ++e) o[e] += rr * (d[e] * gg[e] - xv[e] * rr * proj);
    store_vec<T>(dx + base + (k * 256 + tid) * VE, o);
  }
}

// RMSNorm backward (input part): n = xin r, dn = dout g,
// dx = resid + r (dn - n mean(dn n)).  resid may be null (treated as 0).
template <typename T>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_kernel(const T* __restrict__ dout, const T* __restrict__ xin, const float* __restrict__ r,
                   const T* __restrict__ g, const T* __restrict__ resid, T* __restrict__ dx, int rows,
                   int H) {
  constexpr int VE = 16 / sizeof(T);
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int64_t base = static_cast<int64_t>(row) * H;
  const float rr = r[row];
  float dot = 0.f;
  for (int c = lane * VE; c < H; c += 64 * VE) {
    float d[VE], xv[VE], gg[VE];
    load_vec<T>(dout + base + c, d);
    load_vec<T>(xin + base + c, xv);
    load_vec<T>(g + c, gg);
#pragma unroll
    for (int e = 0; e < VE; ++e) dot += d[e] * gg[e] * xv[e];
  }
  dot = wave_sum(dot);
  const float proj = dot * rr / H;  // mean(dn * n)
  for (int c = lane * VE; c < H; c += 64 * VE) {
    float d[VE], xv[VE], gg[VE], o[VE];
    load_vec<T>(dout + base + c, d);
    load_vec<T>(xin + base + c, xv);
    load_vec<T>(g + c, gg);
    if (resid) load_vec<T>(resid + base + c, o);
    else
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) o[e] += rr * (d[e] * gg[e] - xv[e] * rr * proj);
    store_vec<T>(dx + base + c, o);
  }
}

// Gain gradient, stage 1: partial[chunk][j] = sum over the chunk's rows of
// dout[t, j] * xin[t, j] * r[t].  One wave per (column slice, chunk); a lane
// owns VE adjacent columns.
template <typename T>
__global__ void __launch_bounds__(64)
gain_partial_kernel(const T* __restrict__ dout, const T* __restrict__ xin, const float* __restrict__ r,
                    float* __restrict__ partial, int rows, int H, int rows_per_chunk) {
  constexpr int VE = 16 / sizeof(T);
  const int col = (blockIdx.x * 64 + threadIdx.x) * VE;
  const int chunk = blockIdx.y;
  if (col >= H) return;
  float acc[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) acc[e] = 0.f;
  const int t0 = chunk * rows_per_chunk, t1 = min(rows, t0 + rows_per_chunk);
  for (int t = t0; t < t1; ++t) {
    float d[VE], xv[VE];
    const int64_t base = static_cast<int64_t>(t) * H + col;
    load_vec<T>(dout + base, d);
    load_vec<T>(xin + base, xv);
    const float rr = r[t];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] += d[e] * xv[e] * rr;
  }
  float* p = partial + static_cast<int64_t>(chunk) * H + col;
#pragma unroll
  for (int e = 0; e < VE; e += 4) *reinterpret_cast<float4*>(p + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
}

// RMSNorm backward and gain-gradient partial sums in one pass over dout and
// x: a block owns one chunk of rows (waves take every 4th row); a lane holds
// NV 16-byte vectors of its row (columns (v * 64 + lane) * VE, so each wave
// load is 1 KB contiguous) of dout and x in registers for both the row dot
// and dx, and accumulates dout * x * r for its columns over the wave's rows.
// The 4 waves' column sums are then added in wave order through LDS and
// written as the chunk's partial row.  For H = NV * 64 * VE.
template <typename T, int NV>
__global__ void __launch_bounds__(256)
rmsnorm_bwd_gain_kernel(const T* __restrict__ dout, const T* __restrict__ xin, const float* __restrict__ r,
                        const T* __restrict__ g, const T* __restrict__ resid, T* __restrict__ dx,
                        float* __restrict__ partial, int rows, int H, int rows_per_chunk) {
  constexpr int VE = 16 / sizeof(T);
  __shared__ float colsum[NV * 64 * VE];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int t0 = blockIdx.x * rows_per_chunk, t1 = min(rows, t0 + rows_per_chunk);
  // row data stays packed in the storage dtype (unpacked where used)
  uint4 gq[NV];
  float acc[NV][VE];
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    gq[v] = *reinterpret_cast<const uint4*>(g + (v * 64 + lane) * VE);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[v][e] = 0.f;
  }
  for (int t = t0 + w; t < t1; t += 4) {
    const int64_t base = static_cast<int64_t>(t) * H;
    const float rr = r[t];
    // the residual is requested with dout and x: one memory round trip per row
    uint4 dq[NV], xq[NV], rq[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      dq[v] = *reinterpret_cast<const uint4*>(dout + base + (v * 64 + lane) * VE);
      xq[v] = *reinterpret_cast<const uint4*>(xin + base + (v * 64 + lane) * VE);
      rq[v] = resid ? *reinterpret_cast<const uint4*>(resid + base + (v * 64 + lane) * VE) : make_uint4(0, 0, 0, 0);
    }
    float dot = 0.f;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float d[VE], xv[VE], gg[VE];
      Elem<T>::unpack(dq[v], d);
      Elem<T>::unpack(xq[v], xv);
      Elem<T>::unpack(gq[v], gg);
#pragma unroll
      for (int e = 0; e < VE; ++e) dot += d[e] * gg[e] * xv[e];
    }
    dot = wave_sum(dot);
    const float proj = dot * rr / H;  // mean(dn * n)
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      float d[VE], xv[VE], gg[VE], o[VE];
      Elem<T>::unpack(dq[v], d);
      Elem<T>::unpack(xq[v], xv);
      Elem<T>::unpack(gq[v], gg);
      Elem<T>::unpack(rq[v], o);  // zeros (all bits clear) without a residual
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        o[e] += rr * (d[e] * gg[e] - xv[e] * rr * proj);
        acc[v][e] += d[e] * xv[e] * rr;
      }
      store_vec<T>(dx + base + (v * 64 + lane) * VE, o);
    }
  }
  // column sums of the chunk: waves 0, 1, 2, 3 in turn
  for (int ww = 0; ww < 4; ++ww) {
    if (w == ww) {
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int e = 0; e < VE; ++e) {
          float& c = colsum[(v * 64 + lane) * VE + e];
          c = ww == 0 ? acc[v][e] : c + acc[v][e];
        }
    }
    __syncthreads();
  }
  float* p = partial + static_cast<int64_t>(blockIdx.x) * H;
  for (int j = threadIdx.x * 4; j < H; j += 256 * 4)
    *reinterpret_cast<float4*>(p + j) = *reinterpret_cast<const float4*>(colsum + j);
}

// Gain gradient, stage 2: dg[j] = sum over the chunks of partial, in a fixed
// order: 32 groups of consecutive chunks, each summed in order (loads issued
// sixteen at a time), then the group sums in order.  Block = 32 columns (one
// 128-byte line of a partial row) x 32 groups: the sum of a column is
// latency-bound, not bandwidth-bound (2 MB at hidden 1024), so every thread
// waits for as few rounds of loads as possible and the blocks are many.
constexpr int kReduceCols = 32, kReduceGroups = 32;
__global__ void __launch_bounds__(kReduceCols * kReduceGroups)
gain_reduce_kernel(const float* __restrict__ partial, float* __restrict__ dg, int nchunks, int H) {
  __shared__ float part[kReduceGroups][kReduceCols];
  const int col = threadIdx.x % kReduceCols, grp = threadIdx.x / kReduceCols;
  const int j = blockIdx.x * kReduceCols + col;
  const int per = (nchunks + kReduceGroups - 1) / kReduceGroups;
  const int c0 = grp * per, c1 = min(nchunks, c0 + per);
  float s = 0.f;
  if (j < H) {
    int c = c0;
    for (; c + 16 <= c1; c += 16) {
      float v[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) v[u] = partial[static_cast<int64_t>(c + u) * H + j];
#pragma unroll
      for (int u = 0; u < 16; ++u) s += v[u];
    }
    for (; c < c1; ++c) s += partial[static_cast<int64_t>(c) * H + j];
  }
  part[grp][col] = s;
  __syncthreads();
  if (grp == 0 && j < H) {
    float t = part[0][col];
#pragma unroll
    for (int k = 1; k < kReduceGroups; ++k) t += part[k][col];
    dg[j] = t;
  }
}

// x0[t] = E[ids[t]]; an id outside [0, V) yields a NaN row.
template <typename T>
__global__ void __launch_bounds__(256)
embed_fwd_kernel(const T* __restrict__ E, const int32_t* __restrict__ ids, T* __restrict__ x0, int rows,
                 int H, int V) {
  constexpr int VE = 16 / sizeof(T);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= rows) return;
  const int id = ids[t];
  T* out = x0 + static_cast<int64_t>(t) * H;
  if (id < 0 || id >= V) {
    float f[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) f[e] = __builtin_nanf("");
    for (int c = lane * VE; c < H; c += 64 * VE) store_vec<T>(out + c, f);
    return;
  }
  const T* src = E + static_cast<int64_t>(id) * H;
  for (int c = lane * VE; c < H; c += 64 * VE)
    *reinterpret_cast<uint4*>(out + c) = *reinterpret_cast<const uint4*>(src + c);
}

__global__ void __launch_bounds__(256)
fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  if (i + 3 < n) {
    *reinterpret_cast<float4*>(p + i) = make_float4(v, v, v, v);
  } else {
    for (int64_t k = i; k < n; ++k) p[k] = v;
  }
}

__global__ void __launch_bounds__(64) copy_f32_kernel(float* __restrict__ dst, const float* __restrict__ src, int n) {
  for (int i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

__global__ void __launch_bounds__(64) copy_words_kernel(uint32_t* __restrict__ dst, const uint32_t* __restrict__ src,
                                                       int n) {
  for (int i = threadIdx.x; i < n; i += 64) dst[i] = src[i];
}

__global__ void __launch_bounds__(64) set_word_kernel(int32_t* __restrict__ p, int32_t v) {
  if (threadIdx.x == 0) *p = v;
}

// *flag = 1 when any of g[0 .. n) is an infinity or a NaN (an fp32 whose
// exponent bits are all ones); it is never cleared here.  Only the value 1
// is ever written, so the blocks' racing writes leave the same word.
__global__ void __launch_bounds__(256)
nonfinite_kernel(const float* __restrict__ g, int64_t n, int32_t* __restrict__ flag) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  bool bad = false;
  const int64_t n4 = n / 4;
  const uint4* g4 = reinterpret_cast<const uint4*>(g);
  for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < n4; q += stride) {
    const uint4 w = g4[q];
    const uint32_t e = 0x7F800000u;
    bad |= ((w.x & e) == e) | ((w.y & e) == e) | ((w.z & e) == e) | ((w.w & e) == e);
  }
  for (int64_t i = n4 * 4 + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    bad |= (__float_as_uint(g[i]) & 0x7F800000u) == 0x7F800000u;
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) *flag = 1;
}

// The same over up to kMaxSegs fp32 ranges of one buffer (blockIdx.y = range).
__global__ void __launch_bounds__(256)
nonfinite_segs_kernel(const float* __restrict__ base, FloatSegs segs, int32_t* __restrict__ flag) {
  const int k = blockIdx.y;
  const float* g = base + segs.off[k];
  const int64_t n = segs.n[k];
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    bad |= (__float_as_uint(g[i]) & 0x7F800000u) == 0x7F800000u;
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) *flag = 1;
}

// *flag = 1 when any of n values of a 16-bit storage type is non-finite
// (bf16: exponent bits 0x7F80 all ones; fp16: 0x7C00).
template <typename T>
__global__ void __launch_bounds__(256)
nonfinite16_kernel(const uint16_t* __restrict__ x, int64_t n, int32_t* __restrict__ flag) {
  constexpr uint32_t e = sizeof(T) == 2 && One16<T>::kBits == 0x3C00u ? 0x7C00u : 0x7F80u;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  bool bad = false;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride)
    bad |= (static_cast<uint32_t>(x[i]) & e) == e;
  if (__ballot(bad) != 0 && (threadIdx.x & 63) == 0) *flag = 1;
}

// y = s x in the storage dtype (rounded once), n a multiple of 8.
template <typename T>
__global__ void __launch_bounds__(256)
scale_kernel(const T* __restrict__ x, T* __restrict__ y, int64_t n, float sc) {
  constexpr int VE = 16 / sizeof(T);
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256 * VE;
  for (int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * VE; i < n; i += stride) {
    float f[VE];
    load_vec<T>(x + i, f);
#pragma unroll
    for (int e = 0; e < VE; ++e) f[e] *= sc;
    store_vec<T>(y + i, f);
  }
}

// dE[id] = sum over t with ids[t] == id of dx0[t], in increasing t.  The
// wave of token t does the work only if t is the first occurrence of its id;
// it then walks the later tokens with a ballot per 64 ids.
template <typename T>
__global__ void __launch_bounds__(256)
embed_bwd_kernel(const T* __restrict__ dx0, const int32_t* __restrict__ ids, float* __restrict__ dE,
                 int rows, int H, int V) {
  constexpr int VE = 16 / sizeof(T);
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= rows) return;
  const int id = ids[t];
  if (id < 0 || id >= V) return;
  // first occurrence?
  bool earlier = false;
  for (int base = 0; base < t && !earlier; base += 64) {
    const int u = base + lane;
    const bool hit = (u < t) && ids[u] == id;
    earlier = __ballot(hit) != 0;
  }
  if (earlier) return;
  float* out = dE + static_cast<int64_t>(id) * H;
  for (int c0 = 0; c0 < H; c0 += 64 * VE) {
    const int c = c0 + lane * VE;
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;
    for (int base = t; base < rows; base += 64) {
      const int u = base + lane;
      unsigned long long m = __ballot(u < rows && ids[u] == id);
      while (m) {
        const int k = __ffsll(static_cast<long long>(m)) - 1;
        m &= m - 1;
        if (c < H) {
          float f[VE];
          load_vec<T>(dx0 + static_cast<int64_t>(base + k) * H + c, f);
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[e] += f[e];
        }
      }
    }
    if (c < H)
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(out + c + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
}

// Sparse embedding gradient, stage 1: first[t] = 1 if token t is the first
// occurrence of its (valid) id.  The block stages all ids in LDS when they
// fit (rows <= kIdsInLds), so the scan over earlier tokens reads LDS.
constexpr int kIdsInLds = 16384;

__global__ void __launch_bounds__(256)
embed_first_kernel(const int32_t* __restrict__ ids, int32_t* __restrict__ first, int rows, int V) {
  __shared__ int32_t s_ids[kIdsInLds];
  const bool staged = rows <= kIdsInLds;
  const int t0 = blockIdx.x * 4;
  if (staged) {
    const int lim = min(rows, t0 + 4);  // only ids before the block's last token are read
    for (int i = threadIdx.x; i < lim; i += 256) s_ids[i] = ids[i];
    __syncthreads();
  }
  const int t = t0 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= rows) return;
  const int id = ids[t];
  bool earlier = false;
  for (int base = 0; base < t && !earlier; base += 64) {
    const int u = base + lane;
    const bool hit = (u < t) && (staged ? s_ids[u] : ids[u]) == id;
    earlier = __ballot(hit) != 0;
  }
  if (lane == 0) first[t] = (!earlier && id >= 0 && id < V) ? 1 : 0;
}

// Stage 2: exclusive prefix sum of first[] -> slot[], and the count.  One
// block of 1024 threads; thread j owns a contiguous run of ceil(rows/1024).
__global__ void __launch_bounds__(1024)
embed_scan_kernel(const int32_t* __restrict__ first, int32_t* __restrict__ slot, int32_t* __restrict__ count,
                  int rows) {
  __shared__ int32_t part[1024];
  const int per = (rows + 1023) / 1024;
  const int b = threadIdx.x * per, e = min(rows, b + per);
  int s = 0;
  for (int i = b; i < e; ++i) s += first[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // Hillis-Steele inclusive scan
    const int v = threadIdx.x >= off ? part[threadIdx.x - off] : 0;
    __syncthreads();
    part[threadIdx.x] += v;
    __syncthreads();
  }
  int run = part[threadIdx.x] - s;  // exclusive prefix of this thread's run
  for (int i = b; i < e; ++i) {
    slot[i] = run;
    run += first[i];
  }
  if (threadIdx.x == 1023) *count = part[1023];
}

// Stage 3: the wave of a first-occurrence token t sums dx0 over every token
// with the same id in increasing t and writes it to out_rows[slot[t]].
template <typename T>
__global__ void __launch_bounds__(256)
embed_rows_kernel(const T* __restrict__ dx0, const int32_t* __restrict__ ids, const int32_t* __restrict__ first,
                  const int32_t* __restrict__ slot, int32_t* __restrict__ out_ids, float* __restrict__ out_rows,
                  int rows, int H) {
  constexpr int VE = 16 / sizeof(T);
  __shared__ int32_t s_ids[kIdsInLds];
  const bool staged = rows <= kIdsInLds;
  if (staged) {
    for (int i = threadIdx.x; i < rows; i += 256) s_ids[i] = ids[i];
    __syncthreads();
  }
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= rows || !first[t]) return;
  const int id = ids[t];
  const int s = slot[t];
  if (lane == 0) out_ids[s] = id;
  float* out = out_rows + static_cast<int64_t>(s) * H;
  for (int c0 = 0; c0 < H; c0 += 64 * VE) {
    const int c = c0 + lane * VE;
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = 0.f;
    for (int base = t; base < rows; base += 64) {
      const int u = base + lane;
      unsigned long long m = __ballot(u < rows && (staged ? s_ids[u] : ids[u]) == id);
      while (m) {
        const int k = __ffsll(static_cast<long long>(m)) - 1;
        m &= m - 1;
        if (c < H) {
          float f[VE];
          load_vec<T>(dx0 + static_cast<int64_t>(base + k) * H + c, f);
#pragma unroll
          for (int e = 0; e < VE; ++e) acc[e] += f[e];
        }
      }
    }
    if (c < H)
#pragma unroll
      for (int e = 0; e < VE; e += 4)
        *reinterpret_cast<float4*>(out + c + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
  }
}

// Adam on the device over n fp32 elements (the same arithmetic, operation
// for operation, as the host loop): m = b1 m + (1-b1) g; v = b2 v + (1-b2) g^2;
// p -= lr (m / bc1) / (sqrt(v / bc2) + eps); out = storage copy of p.
template <typename TO>
__global__ void __launch_bounds__(256)
adam_device_kernel(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v, const float* __restrict__ g,
                   TO* __restrict__ out, int64_t n, float b1, float b2, float o1, float o2, float ib1, float ib2,
                   float lr, float eps, float gs, const int32_t* __restrict__ skip) {
  // no fused multiply-add; sqrtf and '/' are correctly rounded (HIP's default
  // for fp32), so every operation rounds exactly as the host loop's
#pragma clang fp contract(off)
  if (skip && *skip) return;  // loss scaling found a non-finite gradient: no update
  const int64_t stride = static_cast<int64_t>(gridDim.x) * 256;
  // 4 elements a thread when every operand is 16-byte aligned (8 for a bf16
  // copy) while whole vectors remain, then one a thread for the tail (and for
  // unaligned operands)
  constexpr bool kOut4 = sizeof(TO) == 2;
  const bool vec = ((reinterpret_cast<uintptr_t>(p) | reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(v) |
                     reinterpret_cast<uintptr_t>(g)) & 15u) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & (kOut4 ? 7u : 15u)) == 0;
  int64_t done = 0;
  if (vec) {
    const int64_t n4 = n / 4;
    for (int64_t q = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; q < n4; q += stride) {
      const int64_t i = q * 4;
      const float4 g4 = *reinterpret_cast<const float4*>(g + i);
      const float4 p4 = *reinterpret_cast<const float4*>(p + i);
      const float4 m4 = *reinterpret_cast<const float4*>(m + i);
      const float4 v4 = *reinterpret_cast<const float4*>(v + i);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w}, pp[4] = {p4.x, p4.y, p4.z, p4.w};
      const float mm[4] = {m4.x, m4.y, m4.z, m4.w}, vv[4] = {v4.x, v4.y, v4.z, v4.w};
      float po[4], mo[4], vo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float gi = gg[k] * gs;
        const float mi = b1 * mm[k] + o1 * gi;
        const float vi = b2 * vv[k] + o2 * gi * gi;
        mo[k] = mi;
        vo[k] = vi;
        const float den = sqrtf(vi * ib2) + eps;
        po[k] = pp[k] - lr * (mi * ib1) / den;
      }
      *reinterpret_cast<float4*>(p + i) = make_float4(po[0], po[1], po[2], po[3]);
      *reinterpret_cast<float4*>(m + i) = make_float4(mo[0], mo[1], mo[2], mo[3]);
      *reinterpret_cast<float4*>(v + i) = make_float4(vo[0], vo[1], vo[2], vo[3]);
      store4<TO>(out + i, po);
    }
    done = n4 * 4;
  }
  for (int64_t i = done + static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; i < n; i += stride) {
    const float gi = g[i] * gs;
    const float mi = b1 * m[i] + o1 * gi;
    const float vi = b2 * v[i] + o2 * gi * gi;
    m[i] = mi;
    v[i] = vi;
    const float den = sqrtf(vi * ib2) + eps;
    const float pi = p[i] - lr * (mi * ib1) / den;
    p[i] = pi;
    Elem<TO>::store(out, i, pi);
  }
}

// Row map of a sparse embedding gradient: map[r] = the slot of row r among
// the n distinct rows (out_ids), -1 for rows no token uses.
__global__ void __launch_bounds__(256) row_map_clear_kernel(int32_t* __restrict__ map, int V) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r < V) map[r] = -1;
}
__global__ void __launch_bounds__(256)
row_map_set_kernel(const int32_t* __restrict__ out_ids, const int32_t* __restrict__ count, int32_t* __restrict__ map,
                   int max_rows, int V) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s < max_rows && s < *count) {
    const int r = out_ids[s];
    if (r >= 0 && r < V) map[r] = s;
  }
}

// Device Adam over a [V, H] tensor whose gradient is sparse: row r's
// gradient is rows[map[r]] when map[r] >= 0 and zero otherwise (rows no token
// touched still decay their moments).  The same operations per element as
// adam_device_kernel, so the bits equal those of Adam on the dense gradient.
// Block = one row at a time, 4 consecutive elements a thread (H % 4 == 0).
template <typename TO>
__global__ void __launch_bounds__(256)
adam_rows_kernel(float* __restrict__ p, float* __restrict__ m, float* __restrict__ v,
                 const float* __restrict__ rows, const int32_t* __restrict__ map, TO* __restrict__ out, int V, int H,
                 float b1, float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, float gs,
                 const int32_t* __restrict__ skip) {
#pragma clang fp contract(off)
  if (skip && *skip) return;
  for (int r = blockIdx.x; r < V; r += gridDim.x) {
    const int sl = map[r];
    const int64_t base = static_cast<int64_t>(r) * H;
    for (int c = threadIdx.x * 4; c < H; c += 256 * 4) {
      const int64_t i = base + c;
      const float4 g4 = sl >= 0 ? *reinterpret_cast<const float4*>(rows + static_cast<int64_t>(sl) * H + c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
      const float4 p4 = *reinterpret_cast<const float4*>(p + i);
      const float4 m4 = *reinterpret_cast<const float4*>(m + i);
      const float4 v4 = *reinterpret_cast<const float4*>(v + i);
      const float gg[4] = {g4.x, g4.y, g4.z, g4.w}, pp[4] = {p4.x, p4.y, p4.z, p4.w};
      const float mm[4] = {m4.x, m4.y, m4.z, m4.w}, vv[4] = {v4.x, v4.y, v4.z, v4.w};
      float po[4], mo[4], vo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float gi = gg[k] * gs;
        const float mi = b1 * mm[k] + o1 * gi;
        const float vi = b2 * vv[k] + o2 * gi * gi;
        mo[k] = mi;
        vo[k] = vi;
        const float den = sqrtf(vi * ib2) + eps;
        po[k] = pp[k] - lr * (mi * ib1) / den;
      }
      *reinterpret_cast<float4*>(p + i) = make_float4(po[0], po[1], po[2], po[3]);
      *reinterpret_cast<float4*>(m + i) = make_float4(mo[0], mo[1], mo[2], mo[3]);
      *reinterpret_cast<float4*>(v + i) = make_float4(vo[0], vo[1], vo[2], vo[3]);
      store4<TO>(out + i, po);
    }
  }
}

// Cross-entropy rows of one LCE chunk.  logits [R, V] fp32 for tokens
// t0 .. t0+R-1.  Token t (position s = t mod S) targets ids[t + 1] unless
// s = S - 1.  Writes dlogits = (softmax - onehot) / N (storage dtype) and the
// per-token loss lse - logit[target] (0 when there is no target).
template <typename T>
__global__ void __launch_bounds__(256)
ce_rows_kernel(const float* __restrict__ logits, const int32_t* __restrict__ ids, T* __restrict__ dlogits,
               float* __restrict__ loss_rows, int t0, int R, int V, int S, float inv_n) {
  __shared__ float red[8];
  const int r = blockIdx.x;
  const int t = t0 + r;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* lr = logits + static_cast<int64_t>(r) * V;
  T* dr = dlogits + static_cast<int64_t>(r) * V;
  const bool has_target = (t % S) != S - 1;
  if (!has_target) {
    for (int v = tid; v < V; v += 256) Elem<T>::store(dr, v, 0.f);
    if (tid == 0) loss_rows[t] = 0.f;
    return;
  }
  const int tgt = ids[t + 1];
  // pass 1: max and sum of exp (online)
  float m = -INFINITY, s = 0.f;
  for (int v = tid; v < V; v += 256) {
    const float x = lr[v];
    if (x > m) { s = s * __expf(m - x) + 1.f; m = x; }
    else s += __expf(x - m);
  }
  float mw = wave_max(m);
  s = s * __expf(m - mw);
  s = wave_sum(s);
  if (lane == 0) { red[w] = mw; red[4 + w] = s; }
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int i = 1; i < 4; ++i) M = fmaxf(M, red[i]);
  float Ssum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) Ssum += red[4 + i] * __expf(red[i] - M);
  const float lse = M + __logf(Ssum);
  const bool ok = tgt >= 0 && tgt < V;
  if (tid == 0) loss_rows[t] = ok ? (lse - lr[tgt]) : __builtin_nanf("");
  for (int v = tid; v < V; v += 256) {
    float p = __expf(lr[v] - lse);
    if (v == tgt) p -= 1.f;
    Elem<T>::store(dr, v, ok ? p * inv_n : __builtin_nanf(""));
  }
}

// The same row computation with the whole row held in registers: 1024
// threads, NV 16-byte vectors each (V <= 4096 NV, V % 4 == 0; NV <= 16, as
// more would spill), so the logits make one trip through HBM (the two-pass
// kernel above reads them twice).
// The maximum is reduced first, then the sum of exp(x - max).
template <typename T, int NV>
__global__ void __launch_bounds__(1024)
ce_rows_reg_kernel(const float* __restrict__ logits, const int32_t* __restrict__ ids, T* __restrict__ dlogits,
                   float* __restrict__ loss_rows, int t0, int V, int S, float inv_n) {
  __shared__ float red[16];
  __shared__ float bc;
  const int r = blockIdx.x;
  const int t = t0 + r;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float4* lr = reinterpret_cast<const float4*>(logits + static_cast<int64_t>(r) * V);
  T* dr = dlogits + static_cast<int64_t>(r) * V;
  const int V4 = V / 4;
  const bool has_target = (t % S) != S - 1;
  if (!has_target) {
    const float z[4] = {0.f, 0.f, 0.f, 0.f};
    for (int v = tid; v < V4; v += 1024) store4<T>(dr + 4 * v, z);
    if (tid == 0) loss_rows[t] = 0.f;
    return;
  }
  const int tgt = ids[t + 1];
  float4 x[NV];
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = tid + k * 1024;
    x[k] = v < V4 ? lr[v] : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    m = fmaxf(m, fmaxf(fmaxf(x[k].x, x[k].y), fmaxf(x[k].z, x[k].w)));
  }
  m = wave_max(m);
  if (lane == 0) red[w] = m;
  __syncthreads();
  if (w == 0) {
    float v = lane < 16 ? red[lane] : -INFINITY;
    v = wave_max(v);
    if (lane == 0) bc = v;
  }
  __syncthreads();
  const float M = bc;
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < NV; ++k)
    sum += (__expf(x[k].x - M) + __expf(x[k].y - M)) + (__expf(x[k].z - M) + __expf(x[k].w - M));
  sum = wave_sum(sum);
  __syncthreads();  // every wave has read bc
  if (lane == 0) red[w] = sum;
  __syncthreads();
  if (w == 0) {
    float v = lane < 16 ? red[lane] : 0.f;
    v = wave_sum(v);
    if (lane == 0) bc = v;
  }
  __syncthreads();
  const float lse = M + __logf(bc);
  const bool ok = tgt >= 0 && tgt < V;
  if (tid == 0) loss_rows[t] = ok ? (lse - logits[static_cast<int64_t>(r) * V + tgt]) : __builtin_nanf("");
#pragma unroll
  for (int k = 0; k < NV; ++k) {
    const int v = tid + k * 1024;
    if (v < V4) {
      float p[4] = {__expf(x[k].x - lse), __expf(x[k].y - lse), __expf(x[k].z - lse), __expf(x[k].w - lse)};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (4 * v + q == tgt) p[q] -= 1.f;
        p[q] = ok ? p[q] * inv_n : __builtin_nanf("");
      }
      store4<T>(dr + 4 * v, p);
    }
  }
}

// loss = (sum over t of loss_rows[t]) * inv_n, one block, fixed order.
__global__ void __launch_bounds__(256)
loss_reduce_kernel(const float* __restrict__ loss_rows, float* __restrict__ loss, int rows, float inv_n) {
  __shared__ float part[256];
  float s = 0.f;
  for (int i = threadIdx.x; i < rows; i += 256) s += loss_rows[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) part[threadIdx.x] += part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) *loss = part[0] * inv_n;
}

}  // namespace

// Host dispatch: every row kernel exists for fp32, bf16 and fp16 storage.
#define SF_T typename decltype(tag)::type

// Wide-row kernels' vectors per thread: H / (256 VE) when that is a whole
// number from 2 to 8 (H = 4096 .. 16384 in steps of 2048 for 16-bit storage),
// else 0 (the wave-per-row kernels).
template <typename T>
int wide_chunks(int H) {
  constexpr int VE = 16 / sizeof(T);
  if (H % (256 * VE)) return 0;
  const int nc = H / (256 * VE);
  return nc >= 2 && nc <= 8 ? nc : 0;
}

hipError_t rmsnorm_fwd(int dtype, const void* x, const void* g, void* y, float* r, int rows, int H,
                       float eps, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    const T* xi = static_cast<const T*>(x);
    const T* gg = static_cast<const T*>(g);
    T* yo = static_cast<T*>(y);
    switch (wide_chunks<T>(H)) {
#define SF_FWD_ROWS(NC)                                                                                        \
  case NC:                                                                                                     \
    hipLaunchKernelGGL((rmsnorm_fwd_rows_kernel<T, NC>), dim3(rows), dim3(256), 0, s, xi, gg, yo, r, H, eps); \
    break;
      SF_FWD_ROWS(2) SF_FWD_ROWS(3) SF_FWD_ROWS(4) SF_FWD_ROWS(5) SF_FWD_ROWS(6) SF_FWD_ROWS(7) SF_FWD_ROWS(8)
#undef SF_FWD_ROWS
      default:
        hipLaunchKernelGGL(rmsnorm_fwd_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, xi, gg, yo, r, rows, H, eps);
    }
    return hipGetLastError();
  });
}

hipError_t rmsnorm_bwd(int dtype, const void* dout, const void* xin, const float* r, const void* g,
                       const void* resid, void* dx, float* partial, int nchunks, float* dg, int rows, int H,
                       hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    constexpr int VE = 16 / sizeof(T);
    const int rpc = (rows + nchunks - 1) / nchunks;
    const T* d = static_cast<const T*>(dout);
    const T* xi = static_cast<const T*>(xin);
    const T* gg = static_cast<const T*>(g);
    const T* rs = static_cast<const T*>(resid);
    T* o = static_cast<T*>(dx);
    // one pass (rows held in registers) when H is 64 lanes x VE x NV with NV
    // <= 4 (more would leave one wave per SIMD: the two-kernel path is then
    // faster)
    const int nv = H % (64 * VE) ? 0 : H / (64 * VE);
    if (nv >= 1 && nv <= 4) {
      switch (nv) {
        case 1: hipLaunchKernelGGL((rmsnorm_bwd_gain_kernel<T, 1>), dim3(nchunks), dim3(256), 0, s, d, xi, r, gg, rs, o,
                                   partial, rows, H, rpc); break;
        case 2: hipLaunchKernelGGL((rmsnorm_bwd_gain_kernel<T, 2>), dim3(nchunks), dim3(256), 0, s, d, xi, r, gg, rs, o,
                                   partial, rows, H, rpc); break;
        case 3: hipLaunchKernelGGL((rmsnorm_bwd_gain_kernel<T, 3>), dim3(nchunks), dim3(256), 0, s, d, xi, r, gg, rs, o,
                                   partial, rows, H, rpc); break;
        default: hipLaunchKernelGGL((rmsnorm_bwd_gain_kernel<T, 4>), dim3(nchunks), dim3(256), 0, s, d, xi, r, gg, rs,
                                    o, partial, rows, H, rpc); break;
      }
    } else {
      const dim3 pg((H / VE + 63) / 64, nchunks);
      switch (wide_chunks<T>(H)) {
#define SF_BWD_ROWS(NC)                                                                                          \
  case NC:                                                                                                       \
    hipLaunchKernelGGL((rmsnorm_bwd_rows_kernel<T, NC>), dim3(rows), dim3(256), 0, s, d, xi, r, gg, rs, o, H); \
    break;
        SF_BWD_ROWS(2) SF_BWD_ROWS(3) SF_BWD_ROWS(4) SF_BWD_ROWS(5) SF_BWD_ROWS(6) SF_BWD_ROWS(7) SF_BWD_ROWS(8)
#undef SF_BWD_ROWS
        default:
          hipLaunchKernelGGL(rmsnorm_bwd_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, d, xi, r, gg, rs, o, rows,
                             H);
      }
      hipLaunchKernelGGL(gain_partial_kernel<T>, pg, dim3(64), 0, s, d, xi, r, partial, rows, H, rpc);
    }
    hipLaunchKernelGGL(gain_reduce_kernel, dim3((H + kReduceCols - 1) / kReduceCols),
                       dim3(kReduceCols * kReduceGroups), 0, s, partial, dg, nchunks, H);
    return hipGetLastError();
  });
}

hipError_t embed_fwd(int dtype, const void* E, const int32_t* ids, void* x0, int rows, int H, int V,
                     hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    hipLaunchKernelGGL(embed_fwd_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, static_cast<const T*>(E), ids,
                       static_cast<T*>(x0), rows, H, V);
    return hipGetLastError();
  });
}

hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n / 4 + 255) / 256 + 1;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t copy_f32(float* dst, const float* src, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(1), dim3(64), 0, s, dst, src, n);
  return hipGetLastError();
}

hipError_t embed_bwd(int dtype, const void* dx0, const int32_t* ids, float* dE, int rows, int H, int V,
                     hipStream_t s) {
  hipError_t e = fill_f32(dE, static_cast<int64_t>(V) * H, 0.f, s);
  if (e != hipSuccess || rows <= 0) return e;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    hipLaunchKernelGGL(embed_bwd_kernel<T>, dim3((rows + 3) / 4), dim3(256), 0, s, static_cast<const T*>(dx0), ids,
                       dE, rows, H, V);
    return hipGetLastError();
  });
}

hipError_t embed_bwd_sparse(int dtype, const void* dx0, const int32_t* ids, int32_t* out_ids, float* out_rows,
                            int32_t* count, int32_t* scratch, int rows, int H, int V, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  int32_t* first = scratch;
  int32_t* slot = scratch + rows;
  const dim3 g((rows + 3) / 4);
  hipLaunchKernelGGL(embed_first_kernel, g, dim3(256), 0, s, ids, first, rows, V);
  hipLaunchKernelGGL(embed_scan_kernel, dim3(1), dim3(1024), 0, s, first, slot, count, rows);
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    hipLaunchKernelGGL(embed_rows_kernel<T>, g, dim3(256), 0, s, static_cast<const T*>(dx0), ids, first, slot,
                       out_ids, out_rows, rows, H);
    return hipGetLastError();
  });
}

hipError_t adam_device(int dtype, float* p, float* m, float* v, const float* g, void* out, int64_t n, float b1,
                       float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                       float gscale, const int32_t* skip) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 32);
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    hipLaunchKernelGGL(adam_device_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, p, m, v, g,
                       static_cast<T*>(out), n, b1, b2, o1, o2, ib1, ib2, lr, eps, gscale, skip);
    return hipGetLastError();
  });
}

hipError_t embed_adam_sparse(int dtype, float* p, float* m, float* v, const float* rows, const int32_t* out_ids,
                             const int32_t* count, int32_t* map, int max_rows, void* out, int V, int H, float b1,
                             float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                             float gscale, const int32_t* skip) {
  if (V <= 0 || H <= 0) return hipSuccess;
  if (H % 4) return hipErrorInvalidValue;
  hipLaunchKernelGGL(row_map_clear_kernel, dim3((V + 255) / 256), dim3(256), 0, s, map, V);
  if (max_rows > 0)
    hipLaunchKernelGGL(row_map_set_kernel, dim3((max_rows + 255) / 256), dim3(256), 0, s, out_ids, count, map,
                       max_rows, V);
  const dim3 grid(static_cast<unsigned>(std::min(V, 8192)));
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    hipLaunchKernelGGL(adam_rows_kernel<T>, grid, dim3(256), 0, s, p, m, v, rows, map, static_cast<T*>(out), V, H, b1,
                       b2, o1, o2, ib1, ib2, lr, eps, gscale, skip);
    return hipGetLastError();
  });
}

hipError_t ce_rows(int dtype, const float* logits, const int32_t* ids, void* dlogits, float* loss_rows, int t0,
                   int R, int V, int S, float inv_n, hipStream_t s) {
  if (R <= 0) return hipSuccess;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    T* dl = static_cast<T*>(dlogits);
    // whole row in registers when V fits 1024 threads x NV 16-byte vectors
    const int nv = V % 4 ? 0 : (V + 4095) / 4096;
    if (nv > 0 && nv <= 8)
      hipLaunchKernelGGL((ce_rows_reg_kernel<T, 8>), dim3(R), dim3(1024), 0, s, logits, ids, dl, loss_rows, t0, V, S,
                         inv_n);
    else if (nv > 0 && nv <= 16)
      hipLaunchKernelGGL((ce_rows_reg_kernel<T, 16>), dim3(R), dim3(1024), 0, s, logits, ids, dl, loss_rows, t0, V,
                         S, inv_n);
    else
      hipLaunchKernelGGL(ce_rows_kernel<T>, dim3(R), dim3(256), 0, s, logits, ids, dl, loss_rows, t0, R, V, S, inv_n);
    return hipGetLastError();
  });
}

hipError_t copy_words(uint32_t* dst, const uint32_t* src, int n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(copy_words_kernel, dim3(1), dim3(64), 0, s, dst, src, n);
  return hipGetLastError();
}

hipError_t set_word(int32_t* p, int32_t v, hipStream_t s) {
  hipLaunchKernelGGL(set_word_kernel, dim3(1), dim3(64), 0, s, p, v);
  return hipGetLastError();
}

hipError_t nonfinite_flag(const float* g, int64_t n, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (reinterpret_cast<uintptr_t>(g) & 15u) return hipErrorInvalidValue;
  const int64_t blocks = std::min<int64_t>((n / 4 + 255) / 256 + 1, 256 * 8);
  hipLaunchKernelGGL(nonfinite_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, g, n, flag);
  return hipGetLastError();
}

hipError_t nonfinite_flag_segs(const float* base, const FloatSegs& segs, int32_t* flag, hipStream_t s) {
  if (segs.count <= 0 || segs.count > kMaxSegs) return segs.count == 0 ? hipSuccess : hipErrorInvalidValue;
  int64_t nmax = 0;
  for (int k = 0; k < segs.count; ++k) nmax = std::max(nmax, segs.n[k]);
  if (nmax <= 0) return hipSuccess;
  const int64_t bx = std::min<int64_t>((nmax + 255) / 256, 512);
  hipLaunchKernelGGL(nonfinite_segs_kernel, dim3(static_cast<unsigned>(bx), segs.count), dim3(256), 0, s, base, segs,
                     flag);
  return hipGetLastError();
}

hipError_t nonfinite_storage(int dtype, const void* x, int64_t n, int32_t* flag, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 0) return nonfinite_flag(static_cast<const float*>(x), n, flag, s);
  const int64_t blocks = std::min<int64_t>((n + 255) / 256, 256 * 8);
  if (dtype == 2)
    hipLaunchKernelGGL(nonfinite16_kernel<f16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), n, flag);
  else
    hipLaunchKernelGGL(nonfinite16_kernel<bf16>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), n, flag);
  return hipGetLastError();
}

hipError_t scale_storage(int dtype, const void* x, void* y, int64_t n, float sc, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (n % 8) return hipErrorInvalidValue;
  return with_storage(dtype, [&](auto tag) {
    using T = SF_T;
    constexpr int VE = 16 / sizeof(T);
    const int64_t blocks = std::min<int64_t>((n / VE + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(scale_kernel<T>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, static_cast<const T*>(x),
                       static_cast<T*>(y), n, sc);
    return hipGetLastError();
  });
}

hipError_t loss_reduce(const float* loss_rows, float* loss, int rows, float inv_n, hipStream_t s) {
  hipLaunchKernelGGL(loss_reduce_kernel, dim3(1), dim3(256), 0, s, loss_rows, loss, rows, inv_n);
  return hipGetLastError();
}

#undef SF_T

}  // namespace sf

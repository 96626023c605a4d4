// Causal flash attention for gfx950 (MFMA 16x16 tiles, LDS-staged K/V).
//
// Layout.  q', k', v of a layer live in one [T, (n_h + 2 n_kv) d] row-major
// buffer (the QKV projection's output): query head h at column h d, KV head
// c at (n_h + c) d for k' and (n_h + n_kv + c) d for v.  Token t = b S + s.
// The output A is [T, n_h d]; the softmax log-sum-exp is kept per (b, h, s)
// in fp32 (base-2 units of the scaled scores) for the backward.  Query head
// h reads KV head floor(h n_kv / n_h).
//
// Forward: a block owns 128 query rows of one (b, h) (4 waves x 32 rows) and
// walks the key tiles (64 keys) up to the diagonal with an online softmax.
// Scores are computed transposed (MFMA A-operand = K tile) so a lane holds 4
// consecutive keys of one query row; the probabilities then feed the P V
// product straight from registers, with V staged transposed in LDS.
//
// Backward (deterministic, no atomics): D = rowsum(dA * A) first; then one
// kernel owns 64 keys of one (b, KV head) and accumulates dK, dV over every
// query head of its group and every query tile at or below the diagonal, and
// a second kernel owns 64 queries of one (b, h) and accumulates dQ over the
// key tiles.  Both recompute P from the saved log-sum-exp.  The inverse RoPE
// rotation of dQ and dK is applied in their store epilogues.
#include <math.h>

#include "attention.h"
#include "common.h"

namespace sf {

namespace {

constexpr float kLog2e = 1.4426950408889634f;


// Pack 8 fp32 into a 16-bit type (bf16 or fp16) or take 4 fp32 as the
// 16-byte B-operand chunk.
template <typename T>
__device__ __forceinline__ uint4 pack_chunk16(const f32x4& a, const f32x4& b) {
  return make_uint4(pack_pair<T>(a[0], a[1]), pack_pair<T>(a[2], a[3]), pack_pair<T>(b[0], b[1]),
                    pack_pair<T>(b[2], b[3]));
}
__device__ __forceinline__ uint4 pack_chunk_f32(const f32x4& a) {
  return make_uint4(__float_as_uint(a[0]), __float_as_uint(a[1]), __float_as_uint(a[2]),
                    __float_as_uint(a[3]));
}

// Copy ROWS rows x D columns (row stride ld) into LDS [ROWS][LROW]; rows at
// or beyond nvalid are zero-filled.
template <typename T, int ROWS, int D, int NT>
__device__ __forceinline__ void tile_rows(T* lds, int lrow, const T* __restrict__ src, int64_t ld,
                                          int nvalid, int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int VPR = D / VE;
  constexpr int NV = ROWS * VPR;
#pragma unroll
  for (int j = 0; j < (NV + NT - 1) / NT; ++j) {
    const int i = tid + j * NT;
    if (NV % NT == 0 || i < NV) {
      const int r = i / VPR, c = i % VPR;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (r < nvalid) v = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(r) * ld + c * VE);
      *reinterpret_cast<uint4*>(lds + r * lrow + c * VE) = v;
    }
  }
}

// Copy ROWS rows x D columns transposed into LDS [D][LROW] (row index =
// column of src).  Blocks of 4 source rows x VE columns per thread.
template <typename T, int ROWS, int D, int NT>
__device__ __forceinline__ void tile_rows_t(T* lds, int lrow, const T* __restrict__ src, int64_t ld,
                                            int nvalid, int tid) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int RG = ROWS / 4;
  constexpr int NB = RG * (D / VE);
#pragma unroll
  for (int j = 0; j < (NB + NT - 1) / NT; ++j) {
    const int i = tid + j * NT;
    if (NB % NT == 0 || i < NB) {
      const int rg = i % RG, cg = i / RG;
      uint4 v[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = rg * 4 + r;
        v[r] = (row < nvalid) ? *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(row) * ld + cg * VE)
                              : make_uint4(0, 0, 0, 0);
      }
      if constexpr (sizeof(T) == 2) {
        const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w}, {v[1].x, v[1].y, v[1].z, v[1].w},
                                  {v[2].x, v[2].y, v[2].z, v[2].w}, {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const int d = c >> 1;
          const uint32_t lo = (c & 1) ? ((w[0][d] >> 16) | (w[1][d] & 0xFFFF0000u))
                                      : ((w[0][d] & 0xFFFFu) | (w[1][d] << 16));
          const uint32_t hi = (c & 1) ? ((w[2][d] >> 16) | (w[3][d] & 0xFFFF0000u))
                                      : ((w[2][d] & 0xFFFFu) | (w[3][d] << 16));
          *reinterpret_cast<uint2*>(lds + (cg * VE + c) * lrow + rg * 4) = make_uint2(lo, hi);
        }
      } else {
        uint4 t[4];
        transpose4x4_b32(v, t);
#pragma unroll
        for (int c = 0; c < 4; ++c) *reinterpret_cast<uint4*>(lds + (cg * VE + c) * lrow + rg * 4) = t[c];
      }
    }
  }
}

// A-operand chunk from a transposed LDS tile [rows][LROW] for the product
// with register-resident probabilities: 16-bit types take keys {32j + 4g .. +3} and
// {32j + 16 + 4g .. +3} (matching pack_chunk16 of fragments 2j, 2j+1);
// fp32 takes keys {16j + 4g .. +3}.
template <typename T>
__device__ __forceinline__ uint4 tchunk(const T* lds, int lrow, int row, int j, int g) {
  if constexpr (sizeof(T) == 2) {
    const uint2 lo = *reinterpret_cast<const uint2*>(lds + row * lrow + 32 * j + 4 * g);
    const uint2 hi = *reinterpret_cast<const uint2*>(lds + row * lrow + 32 * j + 16 + 4 * g);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
  } else {
    return *reinterpret_cast<const uint4*>(lds + row * lrow + 16 * j + 4 * g);
  }
}

// ------------------------------------------------------------------ forward
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_fwd_kernel(const AttnArgs a) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int BQ = 128, BKV = 64, NT = 256;
  constexpr int KROW = D + VE;     // K tile [BKV][KROW]
  constexpr int VROW = BKV + VE;   // Vt tile [D][VROW]
  constexpr int DC = D / (4 * VE); // MFMA steps along d
  constexpr int FD = D / 16;
  constexpr int PJ = (sizeof(T) == 2) ? 2 : 4;  // P.V MFMA steps per 64 keys
  __shared__ __attribute__((aligned(16))) T Ks[2][BKV * KROW];
  __shared__ __attribute__((aligned(16))) T Vt[2][D * VROW];

  const int S = a.seq;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt = nqt - 1 - blockIdx.x;  // longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = (h * a.n_kv) / a.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const T* qbase = static_cast<const T*>(a.qkv) + static_cast<int64_t>(b) * S * ld + h * D;
  const T* kbase = static_cast<const T*>(a.qkv) + static_cast<int64_t>(b) * S * ld + (a.n_heads + kvh) * D;
  const T* vbase = static_cast<const T*>(a.qkv) + static_cast<int64_t>(b) * S * ld +
                   (a.n_heads + a.n_kv + kvh) * D;
  const int q0 = qt * BQ;
  const int qw = q0 + w * 32;  // first row of this wave

  // Q fragments in registers (B operand: lane supplies row lr, chunk lg).
  uint4 qf[2][DC];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int q = qw + f * 16 + lr;
      qf[f][c] = (q < S) ? *reinterpret_cast<const uint4*>(qbase + static_cast<int64_t>(q) * ld + c * 4 * VE + lg * VE)
                         : make_uint4(0, 0, 0, 0);
    }

  f32x4 oacc[2][FD];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int d = 0; d < FD; ++d) oacc[f][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};
  const float sc = a.scale * kLog2e;

  const int last_q = min(q0 + BQ, S) - 1;
  const int nkv = last_q / BKV + 1;

  tile_rows<T, BKV, D, NT>(Ks[0], KROW, kbase, ld, S, tid);
  tile_rows_t<T, BKV, D, NT>(Vt[0], VROW, vbase, ld, S, tid);
  __syncthreads();

  for (int kt = 0; kt < nkv; ++kt) {
    const int buf = kt & 1;
    const int kv0 = kt * BKV;
    if (kt + 1 < nkv) {
      const int64_t off = static_cast<int64_t>(kv0 + BKV) * ld;
      tile_rows<T, BKV, D, NT>(Ks[buf ^ 1], KROW, kbase + off, ld, S - kv0 - BKV, tid);
      tile_rows_t<T, BKV, D, NT>(Vt[buf ^ 1], VROW, vbase + off, ld, S - kv0 - BKV, tid);
    }
    if (kv0 <= qw + 31) {  // some row of this wave sees a key of this tile
      // S^T fragments: lane holds S[q = row lr][kv = 16 fk + 4 lg + v]
      f32x4 s[2][4];
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk) s[f][fk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < DC; ++c) {
        uint4 kf[4];
#pragma unroll
        for (int fk = 0; fk < 4; ++fk)
          kf[fk] = *reinterpret_cast<const uint4*>(&Ks[buf][(fk * 16 + lr) * KROW + c * 4 * VE + lg * VE]);
#pragma unroll
        for (int f = 0; f < 2; ++f)
#pragma unroll
          for (int fk = 0; fk < 4; ++fk) Mfma<T>::run(s[f][fk], kf[fk], qf[f][c]);
      }
      const bool diag = (kv0 + BKV - 1 > qw);
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        const int q = qw + f * 16 + lr;
        float mx = -INFINITY;
#pragma unroll
        for (int fk = 0; fk < 4; ++fk)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            float x = s[f][fk][v] * sc;
            if (diag && kv0 + fk * 16 + lg * 4 + v > q) x = -INFINITY;
            s[f][fk][v] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        const float mnew = fmaxf(mrow[f], mx);
        const float alpha = exp2f(mrow[f] - mnew);
        mrow[f] = mnew;
        float ps = 0.f;
#pragma unroll
        for (int fk = 0; fk < 4; ++fk)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float p = exp2f(s[f][fk][v] - mnew);
            s[f][fk][v] = p;
            ps += p;
          }
        lsum[f] = lsum[f] * alpha + ps;
#pragma unroll
        for (int d = 0; d < FD; ++d)
#pragma unroll
          for (int v = 0; v < 4; ++v) oacc[f][d][v] *= alpha;
      }
      // O^T += Vt P^T: lane holds O[q = row lr][d = 16 fd + 4 lg + v]
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        uint4 pf[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          if constexpr (sizeof(T) == 2) pf[f] = pack_chunk16<T>(s[f][2 * j], s[f][2 * j + 1]);
          else pf[f] = pack_chunk_f32(s[f][j]);
        }
#pragma unroll
        for (int d = 0; d < FD; ++d) {
          const uint4 vf = tchunk<T>(Vt[buf], VROW, d * 16 + lr, j, lg);
#pragma unroll
          for (int f = 0; f < 2; ++f) Mfma<T>::run(oacc[f][d], vf, pf[f]);
        }
      }
    }
    __syncthreads();
  }

  // epilogue
  T* obase = static_cast<T*>(a.out) + static_cast<int64_t>(b) * S * a.ld_out + h * D;
#pragma unroll
  for (int f = 0; f < 2; ++f) {
    float l = lsum[f];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int q = qw + f * 16 + lr;
    if (q < S) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int d = 0; d < FD; ++d) {
        float o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = oacc[f][d][v] * inv;
        store4<T>(obase + static_cast<int64_t>(q) * a.ld_out + d * 16 + lg * 4, o);
      }
      if (lg == 0) a.lse[(static_cast<int64_t>(b) * a.n_heads + h) * S + q] = mrow[f] + log2f(l);
    }
  }
}

// ---------------------------------------------------------- D = rowsum(dO*O)
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_dot_kernel(const AttnArgs a) {
  constexpr int VE = 16 / sizeof(T);
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;  // (t, h)
  const int64_t T_ = static_cast<int64_t>(a.batch) * a.seq;
  if (idx >= T_ * a.n_heads) return;
  const int64_t t = idx / a.n_heads;
  const int h = static_cast<int>(idx % a.n_heads);
  const T* o = static_cast<const T*>(a.out) + t * a.ld_out + h * D;
  const T* d = static_cast<const T*>(a.dout) + t * a.ld_dout + h * D;
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / VE; ++c) {
    float fo[VE], fd[VE];
    Elem<T>::unpack(*reinterpret_cast<const uint4*>(o + c * VE), fo);
    Elem<T>::unpack(*reinterpret_cast<const uint4*>(d + c * VE), fd);
#pragma unroll
    for (int e = 0; e < VE; ++e) acc += fo[e] * fd[e];
  }
  const int b = static_cast<int>(t / a.seq), s = static_cast<int>(t % a.seq);
  a.dsum[(static_cast<int64_t>(b) * a.n_heads + h) * a.seq + s] = acc;
}

// Inverse RoPE on a lane's fragments: x[fd] (first half) pairs with
// x[fd + FD/2]; column = 16 fd + 4 lg + v; position pos.
template <int D>
__device__ __forceinline__ void rope_inverse(f32x4 (&x)[D / 16], const AttnArgs& a, int pos, int lg) {
  constexpr int FD = D / 16;
#pragma unroll
  for (int fd = 0; fd < FD / 2; ++fd)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = fd * 16 + lg * 4 + v;
      const float c = a.rope_cos[static_cast<int64_t>(pos) * (D / 2) + i];
      const float s = a.rope_sin[static_cast<int64_t>(pos) * (D / 2) + i];
      const float u1 = x[fd][v], u2 = x[fd + FD / 2][v];
      x[fd][v] = u1 * c + u2 * s;
      x[fd + FD / 2][v] = u2 * c - u1 * s;
    }
}

// ---------------------------------------------------------------- dK, dV
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_bwd_dkdv_kernel(const AttnArgs a) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int BQ = 64, BKV = 64, NT = 256;
  constexpr int RROW = D + VE;    // [BQ][RROW]
  constexpr int TROW = BQ + VE;   // [D][TROW]
  constexpr int DC = D / (4 * VE);
  constexpr int FD = D / 16;
  constexpr int PJ = (sizeof(T) == 2) ? 2 : 4;
  __shared__ __attribute__((aligned(16))) T Qs[BQ * RROW];
  __shared__ __attribute__((aligned(16))) T Qt[D * TROW];
  __shared__ __attribute__((aligned(16))) T dOs[BQ * RROW];
  __shared__ __attribute__((aligned(16))) T dOt[D * TROW];
  __shared__ float lse_s[BQ], dsum_s[BQ];

  const int S = a.seq;
  const int kt = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int kv0 = kt * BKV;
  const int kvw = kv0 + w * 16;      // this wave's 16 keys
  const int kv = kvw + lr;           // key of this lane's B-operand row
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* kbase = qkv + bs * ld + (a.n_heads + kvh) * D;
  const T* vbase = qkv + bs * ld + (a.n_heads + a.n_kv + kvh) * D;

  uint4 kf[DC], vf[DC];
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    const bool ok = kv < S;
    kf[c] = ok ? *reinterpret_cast<const uint4*>(kbase + kv * ld + c * 4 * VE + lg * VE) : make_uint4(0, 0, 0, 0);
    vf[c] = ok ? *reinterpret_cast<const uint4*>(vbase + kv * ld + c * 4 * VE + lg * VE) : make_uint4(0, 0, 0, 0);
  }
  f32x4 dk[FD], dv[FD];
#pragma unroll
  for (int d = 0; d < FD; ++d) { dk[d] = f32x4{0.f, 0.f, 0.f, 0.f}; dv[d] = f32x4{0.f, 0.f, 0.f, 0.f}; }
  const float sc = a.scale * kLog2e;
  const int group = a.n_heads / a.n_kv;
  const int nqt = (S + BQ - 1) / BQ;

  for (int hh = 0; hh < group; ++hh) {
    const int h = kvh * group + hh;
    const T* qbase = qkv + bs * ld + h * D;
    const T* dobase = static_cast<const T*>(a.dout) + bs * a.ld_dout + h * D;
    const float* lse = a.lse + (static_cast<int64_t>(b) * a.n_heads + h) * S;
    const float* dsum = a.dsum + (static_cast<int64_t>(b) * a.n_heads + h) * S;
    for (int qt = kv0 / BQ; qt < nqt; ++qt) {
      const int q0 = qt * BQ;
      __syncthreads();
      tile_rows<T, BQ, D, NT>(Qs, RROW, qbase + static_cast<int64_t>(q0) * ld, ld, S - q0, tid);
      tile_rows_t<T, BQ, D, NT>(Qt, TROW, qbase + static_cast<int64_t>(q0) * ld, ld, S - q0, tid);
      tile_rows<T, BQ, D, NT>(dOs, RROW, dobase + static_cast<int64_t>(q0) * a.ld_dout, a.ld_dout, S - q0, tid);
      tile_rows_t<T, BQ, D, NT>(dOt, TROW, dobase + static_cast<int64_t>(q0) * a.ld_dout, a.ld_dout, S - q0, tid);
      if (tid < BQ) {
        const bool ok = q0 + tid < S;
        lse_s[tid] = ok ? lse[q0 + tid] : 0.f;
        dsum_s[tid] = ok ? dsum[q0 + tid] : 0.f;
      }
      __syncthreads();
      if (q0 + BQ - 1 < kvw) continue;  // every query of the tile precedes this wave's keys
      // P^T, dP^T: lane holds X[q = 16 fq + 4 lg + v][kv = kvw + lr]
      f32x4 p[4], dp[4];
#pragma unroll
      for (int f = 0; f < 4; ++f) { p[f] = f32x4{0.f, 0.f, 0.f, 0.f}; dp[f] = f32x4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int f = 0; f < 4; ++f) {
          const uint4 qa = *reinterpret_cast<const uint4*>(&Qs[(f * 16 + lr) * RROW + c * 4 * VE + lg * VE]);
          const uint4 da = *reinterpret_cast<const uint4*>(&dOs[(f * 16 + lr) * RROW + c * 4 * VE + lg * VE]);
          Mfma<T>::run(p[f], qa, kf[c]);
          Mfma<T>::run(dp[f], da, vf[c]);
        }
      f32x4 ds[4];
#pragma unroll
      for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int ql = f * 16 + lg * 4 + v;
          const int q = q0 + ql;
          float pv = exp2f(p[f][v] * sc - lse_s[ql]);
          if (kv > q || q >= S) pv = 0.f;
          p[f][v] = pv;
          ds[f][v] = pv * (dp[f][v] - dsum_s[ql]);
        }
      // dV^T += dO^T P, dK^T += Q^T dS: lane holds X[kv = kvw + lr][d = 16 fd + 4 lg + v]
#pragma unroll
      for (int j = 0; j < PJ; ++j) {
        uint4 pb, sb;
        if constexpr (sizeof(T) == 2) {
          pb = pack_chunk16<T>(p[2 * j], p[2 * j + 1]);
          sb = pack_chunk16<T>(ds[2 * j], ds[2 * j + 1]);
        } else {
          pb = pack_chunk_f32(p[j]);
          sb = pack_chunk_f32(ds[j]);
        }
#pragma unroll
        for (int d = 0; d < FD; ++d) {
          Mfma<T>::run(dv[d], tchunk<T>(dOt, TROW, d * 16 + lr, j, lg), pb);
          Mfma<T>::run(dk[d], tchunk<T>(Qt, TROW, d * 16 + lr, j, lg), sb);
        }
      }
    }
  }

  // epilogue: the lane owns key kvw + lr, columns 16 fd + 4 lg + v.
  if (kv < S) {
#pragma unroll
    for (int d = 0; d < FD; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dk[d][v] *= a.scale;
    rope_inverse<D>(dk, a, kv, lg);
    T* dkp = static_cast<T*>(a.dqkv) + (bs + kv) * a.ld_dqkv + (a.n_heads + kvh) * D;
    T* dvp = static_cast<T*>(a.dqkv) + (bs + kv) * a.ld_dqkv + (a.n_heads + a.n_kv + kvh) * D;
#pragma unroll
    for (int d = 0; d < FD; ++d) {
      float o[4] = {dk[d][0], dk[d][1], dk[d][2], dk[d][3]};
      store4<T>(dkp + d * 16 + lg * 4, o);
      float o2[4] = {dv[d][0], dv[d][1], dv[d][2], dv[d][3]};
      store4<T>(dvp + d * 16 + lg * 4, o2);
    }
  }
}

// -------------------------------------------------------------------- dQ
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_bwd_dq_kernel(const AttnArgs a) {
  constexpr int VE = 16 / sizeof(T);
  constexpr int BQ = 64, BKV = 64, NT = 256;
  constexpr int RROW = D + VE;
  constexpr int TROW = BKV + VE;
  constexpr int DC = D / (4 * VE);
  constexpr int FD = D / 16;
  constexpr int PJ = (sizeof(T) == 2) ? 2 : 4;
  __shared__ __attribute__((aligned(16))) T Ks[BKV * RROW];
  __shared__ __attribute__((aligned(16))) T Kt[D * TROW];
  __shared__ __attribute__((aligned(16))) T Vs[BKV * RROW];

  const int S = a.seq;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt = nqt - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = (h * a.n_kv) / a.n_heads;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int q0 = qt * BQ;
  const int qw = q0 + w * 16;
  const int q = qw + lr;  // this lane's query row
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* kbase = qkv + bs * ld + (a.n_heads + kvh) * D;
  const T* vbase = qkv + bs * ld + (a.n_heads + a.n_kv + kvh) * D;

  uint4 qf[DC], df[DC];
  const T* qrow = qkv + (bs + q) * ld + h * D;
  const T* drow = static_cast<const T*>(a.dout) + (bs + q) * a.ld_dout + h * D;
#pragma unroll
  for (int c = 0; c < DC; ++c) {
    qf[c] = (q < S) ? *reinterpret_cast<const uint4*>(qrow + c * 4 * VE + lg * VE) : make_uint4(0, 0, 0, 0);
    df[c] = (q < S) ? *reinterpret_cast<const uint4*>(drow + c * 4 * VE + lg * VE) : make_uint4(0, 0, 0, 0);
  }
  const int64_t row = (static_cast<int64_t>(b) * a.n_heads + h) * S;
  const float lse = (q < S) ? a.lse[row + q] : 0.f;
  const float dsum = (q < S) ? a.dsum[row + q] : 0.f;
  const float sc = a.scale * kLog2e;

  f32x4 dq[FD];
#pragma unroll
  for (int d = 0; d < FD; ++d) dq[d] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int last_q = min(q0 + BQ, S) - 1;
  const int nkv = last_q / BKV + 1;
  for (int kt = 0; kt < nkv; ++kt) {
    const int kv0 = kt * BKV;
    __syncthreads();
    tile_rows<T, BKV, D, NT>(Ks, RROW, kbase + static_cast<int64_t>(kv0) * ld, ld, S - kv0, tid);
    tile_rows_t<T, BKV, D, NT>(Kt, TROW, kbase + static_cast<int64_t>(kv0) * ld, ld, S - kv0, tid);
    tile_rows<T, BKV, D, NT>(Vs, RROW, vbase + static_cast<int64_t>(kv0) * ld, ld, S - kv0, tid);
    __syncthreads();
    if (kv0 > qw + 15) continue;
    // S, dP: lane holds X[q = qw + lr][kv = kv0 + 16 fk + 4 lg + v]
    f32x4 s[4], dp[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) { s[f] = f32x4{0.f, 0.f, 0.f, 0.f}; dp[f] = f32x4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
    for (int c = 0; c < DC; ++c)
#pragma unroll
      for (int f = 0; f < 4; ++f) {
        const uint4 ka = *reinterpret_cast<const uint4*>(&Ks[(f * 16 + lr) * RROW + c * 4 * VE + lg * VE]);
        const uint4 va = *reinterpret_cast<const uint4*>(&Vs[(f * 16 + lr) * RROW + c * 4 * VE + lg * VE]);
        Mfma<T>::run(s[f], ka, qf[c]);
        Mfma<T>::run(dp[f], va, df[c]);
      }
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int kv = kv0 + f * 16 + lg * 4 + v;
        float pv = exp2f(s[f][v] * sc - lse);
        if (kv > q || kv >= S) pv = 0.f;
        s[f][v] = pv * (dp[f][v] - dsum);  // dS
      }
    // dQ^T += Kt dS^T: lane holds dQ[q = qw + lr][d = 16 fd + 4 lg + v]
#pragma unroll
    for (int j = 0; j < PJ; ++j) {
      uint4 sb;
      if constexpr (sizeof(T) == 2) sb = pack_chunk16<T>(s[2 * j], s[2 * j + 1]);
      else sb = pack_chunk_f32(s[j]);
#pragma unroll
      for (int d = 0; d < FD; ++d) Mfma<T>::run(dq[d], tchunk<T>(Kt, TROW, d * 16 + lr, j, lg), sb);
    }
  }

  if (q < S) {
#pragma unroll
    for (int d = 0; d < FD; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dq[d][v] *= a.scale;
    rope_inverse<D>(dq, a, q % S, lg);
    T* dqp = static_cast<T*>(a.dqkv) + (bs + q) * a.ld_dqkv + h * D;
#pragma unroll
    for (int d = 0; d < FD; ++d) {
      float o[4] = {dq[d][0], dq[d][1], dq[d][2], dq[d][3]};
      store4<T>(dqp + d * 16 + lg * 4, o);
    }
  }
}

template <typename T, int D>
hipError_t run_fwd(const AttnArgs& a, hipStream_t s) {
  dim3 grid((a.seq + 127) / 128, a.n_heads, a.batch);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_bwd(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.batch) * a.seq * a.n_heads;
  hipLaunchKernelGGL((attn_dot_kernel<T, D>), dim3((rows + 255) / 256), dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkdv_kernel<T, D>), dim3((a.seq + 63) / 64, a.n_kv, a.batch), dim3(256), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_kernel<T, D>), dim3((a.seq + 63) / 64, a.n_heads, a.batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t attention_fwd(int dtype, const AttnArgs& a, hipStream_t s) {
  int64_t qkv_bytes = 0;
  if (dtype != 0 && attention_direct_ok(a, &qkv_bytes)) return attention_fwd_direct(dtype, a, qkv_bytes, s);
  return with_storage(dtype, [&](auto tag) {
    using T = typename decltype(tag)::type;
    return a.head_dim == 64 ? run_fwd<T, 64>(a, s) : run_fwd<T, 128>(a, s);
  });
}

hipError_t attention_bwd(int dtype, const AttnArgs& a, hipStream_t s) {
  int64_t qkv_bytes = 0;
  if (dtype != 0 && attention_direct_ok(a, &qkv_bytes) && a.ld_dout % 8 == 0 &&
      !(reinterpret_cast<uintptr_t>(a.dout) & 15u)) {
    const int64_t rows = static_cast<int64_t>(a.batch) * a.seq * a.n_heads;
    const hipError_t e = with_storage(dtype, [&](auto tag) {
      using T = typename decltype(tag)::type;
      if (a.head_dim == 64)
        hipLaunchKernelGGL((attn_dot_kernel<T, 64>), dim3((rows + 255) / 256), dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((attn_dot_kernel<T, 128>), dim3((rows + 255) / 256), dim3(256), 0, s, a);
      return hipGetLastError();
    });
    if (e != hipSuccess) return e;
    return attention_bwd_direct(dtype, a, qkv_bytes, s);
  }
  return with_storage(dtype, [&](auto tag) {
    using T = typename decltype(tag)::type;
    return a.head_dim == 64 ? run_bwd<T, 64>(a, s) : run_bwd<T, 128>(a, s);
  });
}

}  // namespace sf

// Causal flash-attention forward with direct global -> LDS loads (gfx950),
// parametrised by the query rows each wave owns (16 F).
//
// Block: 4 waves, each owning F groups of 16 query rows of one (b, h); key
// tiles of 64 rows.  Every wave reads each key tile's K (along d, 16-byte
// LDS reads) and V (transposed reads) in full: at d = 128 a 4-wave block
// reads 128 KB of LDS per key tile, against 4.2 MFLOP of MFMA work at F = 2
// and 8.4 MFLOP at F = 4.  gfx950's LDS delivers ~155 B/clk per CU to
// 16-byte reads and ~108 B/clk to the 8-byte transposed reads (measured),
// the CU's matrix units ~4070 bf16 FLOP/clk: at F = 2 a tile's LDS reads
// take about as long as its MFMAs.  F = 4 halves that but needs more than
// 256 VGPRs a wave (one wave per SIMD, accumulators spilled to AGPRs); it
// gives the same bits, and measured per launch it was 207 against 266 us at
// the 6.7B shape but 829 against 521 us at the 123B shape, where its
// exponentials and AGPR copies have no second wave to overlap with.  F = 2
// at two blocks per CU is what runs.
//
// Blocks of NW = 8 waves (256 query rows, one block per CU) gave the same
// bits and times within the launch-to-launch spread of 4-wave blocks at the
// 1.3B, 6.7B and 123B shapes; 4 waves run.
//
// The arithmetic of a query row does not depend on F: the same key tiles in
// the same order, the same MFMA accumulation orders, the same lazy shift of
// the exponent, so every F gives the same bits.
#pragma once

#include "attn_tiles.h"

namespace sf {
namespace {

// Grid: (n_heads, query tiles, batch); the query tile index runs backwards
// so that the blocks with the most key tiles are dispatched first across all
// heads.
template <typename T, int D, int F, int MINB, int NW = 4>
__global__ void __launch_bounds__(NW * 64, MINB)
attn_fwd_kernel(const AttnArgs a, int qkv_bytes) {
  constexpr int BQ = NW * F * 16, BKV = 64;
  constexpr int DC = D / 32;  // MFMA k-steps along d
  constexpr int FD = D / 16;
  constexpr int TB = BKV * D * 2;
  __shared__ __attribute__((aligned(1024))) char K0[TB];
  __shared__ __attribute__((aligned(1024))) char K1[TB];
  __shared__ __attribute__((aligned(1024))) char V0[TB];
  __shared__ __attribute__((aligned(1024))) char V1[TB];

  const int S = a.seq;
  const int h = xcd_head(blockIdx.x, a.n_heads);
  const int qt = gridDim.y - 1 - blockIdx.y;
  const int b = blockIdx.z;
  const int kvh = (h * a.n_kv) / a.n_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int q0 = qt * BQ;
  const int qw = q0 + w * F * 16;

  const __amdgpu_buffer_rsrc_t rs = rsrc(a.qkv, qkv_bytes);
  TileLoad<D, NW, 0> lk;
  TileLoad<D, NW, 1> lv;
  lk.init(w, lane, (bs * ld + (a.n_heads + kvh) * D) * 2, ld);
  lv.init(w, lane, (bs * ld + (a.n_heads + a.n_kv + kvh) * D) * 2, ld);

  // Q fragments (B operand): lane supplies row lr, d-chunk lg of each 32
  const T* qbase = static_cast<const T*>(a.qkv) + bs * ld + h * D;
  uint4 qf[F][DC];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int q = qw + f * 16 + lr;
      qf[f][c] = (q < S) ? *reinterpret_cast<const uint4*>(qbase + static_cast<int64_t>(q) * ld + c * 32 + lg * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  f32x4 oacc[F][FD];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int d = 0; d < FD; ++d) oacc[f][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[F];
  // row sums of the (16-bit) probabilities, accumulated by MFMA against a
  // fragment of ones: every element of lacc[f] holds the sum for row lr
  f32x4 lacc[F];
#pragma unroll
  for (int f = 0; f < F; ++f) {
    mrow[f] = -INFINITY;
    lacc[f] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  constexpr uint32_t kOnes = One16<T>::kBits | (One16<T>::kBits << 16);
  const uint4 ones = make_uint4(kOnes, kOnes, kOnes, kOnes);
  const float sc = a.scale * kLog2e;
  const int nkv = (min(q0 + BQ, S) - 1) / BKV + 1;
  int ko[DC], vo[FD];
#pragma unroll
  for (int c = 0; c < DC; ++c) ko[c] = ofs_d0(c, lr, lg);
#pragma unroll
  for (int d = 0; d < FD; ++d) vo[d] = ofs_t<D>(d * 16, lr, lg);

  // Software pipeline over key tiles: iteration kt computes the scores of
  // tile kt + 1 (MFMA) while the softmax of tile kt runs (VALU), then P.V of
  // tile kt.  K(kt + 1) and V(kt) were loaded during iteration kt - 1; the
  // loads of K(kt + 2) and V(kt + 1) go into the buffers that tiles kt and
  // kt - 1 used, which every wave has finished reading at the barrier that
  // opens the iteration.
  auto scores = [&](const char* Kc, f32x4 (&sv)[F][4]) {
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int fk = 0; fk < 4; ++fk) sv[f][fk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      uint4 kf[4];
#pragma unroll
      for (int fk = 0; fk < 4; ++fk) kf[fk] = lds16(Kc, ko[c] + fk * 16 * 128);
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk) Mfma<T>::run(sv[f][fk], kf[fk], qf[f][c]);
    }
  };
  // rows past the sequence end (a ragged last tile) need no work
  auto active = [&](int kt) { return kt < nkv && kt * BKV <= qw + F * 16 - 1 && qw < S; };

  lk.issue(rs, K0, w, S, 0);
  lv.issue(rs, V0, w, S, 0);
  if (nkv > 1) lk.issue(rs, K1, w, S - BKV, static_cast<uint32_t>(BKV * ld * 2));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x4 s[F][4];
  if (active(0)) scores(K0, s);

  auto tile = [&](int kt, const char* Vc, char* Vn, const char* Knext, char* Kfree) {
    // this wave's loads of K(kt + 1) and V(kt) have landed; the barrier
    // covers the other waves' loads and their reads of iteration kt - 1 (for
    // kt = 0: of K0 by the scores computed before the loop)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int kv0 = kt * BKV;
    if (kt + 2 < nkv) lk.issue(rs, Kfree, w, S - kv0 - 2 * BKV, static_cast<uint32_t>((kv0 + 2 * BKV) * ld * 2));
    if (kt + 1 < nkv) lv.issue(rs, Vn, w, S - kv0 - BKV, static_cast<uint32_t>((kv0 + BKV) * ld * 2));
    if (!active(kt)) return;
    f32x4 sn[F][4];
    if (active(kt + 1)) scores(Knext, sn);
    // raw scores are scaled inside the exponent: p = 2^(s sc - m), with the
    // running maximum m kept in scaled units (sc > 0)
    if (kv0 + BKV - 1 > qw) {  // a tile reaching past a row of this wave: mask keys after the row
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk)
#pragma unroll
          for (int v = 0; v < 4; ++v)
            if (kv0 + fk * 16 + lg * 4 + v > qw + f * 16 + lr) s[f][fk][v] = -INFINITY;
    }
    // The shift m of a row moves only when the tile's maximum exceeds it
    // by more than kLazy (log2 units): probabilities stay <= 2^kLazy, and
    // the output and row sum, which carry the same shift, are rescaled
    // only then (softmax is invariant to a common shift of the exponents).
    float alpha[F];
    bool keep = true;
#pragma unroll
    for (int f = 0; f < F; ++f) {
      float mx = -INFINITY;
#pragma unroll
      for (int fk = 0; fk < 4; ++fk)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, s[f][fk][v]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float ms = mx * sc;
      const float mnew = ms > mrow[f] + kLazy ? ms : mrow[f];
      alpha[f] = __builtin_amdgcn_exp2f(mrow[f] - mnew);
      keep = keep && alpha[f] == 1.0f;
      mrow[f] = mnew;
#pragma unroll
      for (int fk = 0; fk < 4; ++fk)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[f][fk][v] = __builtin_amdgcn_exp2f(fmaf(s[f][fk][v], sc, -mnew));
    }
    if (!__all(keep)) {
#pragma unroll
      for (int f = 0; f < F; ++f) {
#pragma unroll
        for (int d = 0; d < FD; ++d)
#pragma unroll
          for (int v = 0; v < 4; ++v) oacc[f][d][v] *= alpha[f];
#pragma unroll
        for (int v = 0; v < 4; ++v) lacc[f][v] *= alpha[f];
      }
    }
    // O^T += V^T P^T: lane holds O[q = qw + 16 f + lr][d = 16 fd + 4 lg + v]
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      uint4 pf[F];
#pragma unroll
      for (int f = 0; f < F; ++f) {
        pf[f] = pack8<T>(s[f][2 * j], s[f][2 * j + 1]);
        Mfma<T>::run(lacc[f], ones, pf[f]);
      }
#pragma unroll
      for (int d = 0; d < FD; ++d) {
        const uint4 vf = frag_t<D>(Vc, vo[d], j);
#pragma unroll
        for (int f = 0; f < F; ++f) Mfma<T>::run(oacc[f][d], vf, pf[f]);
      }
    }
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int fk = 0; fk < 4; ++fk) s[f][fk] = sn[f][fk];
  };
  for (int kt = 0; kt < nkv; kt += 2) {
    tile(kt, V0, V1, K1, K0);
    if (kt + 1 < nkv) tile(kt + 1, V1, V0, K0, K1);
  }
  __builtin_amdgcn_s_waitcnt(0);  // no load into LDS outlives the block

  T* obase = static_cast<T*>(a.out) + bs * a.ld_out + h * D;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const float l = lacc[f][0];
    const int q = qw + f * 16 + lr;
    if (q < S) {
      const float inv = 1.0f / l;
#pragma unroll
      for (int d = 0; d < FD; ++d) {
        const f32x4 o = oacc[f][d];
        *reinterpret_cast<uint2*>(obase + static_cast<int64_t>(q) * a.ld_out + d * 16 + lg * 4) =
            make_uint2(pack_pair<T>(o[0] * inv, o[1] * inv), pack_pair<T>(o[2] * inv, o[3] * inv));
      }
      if (lg == 0) a.lse[(static_cast<int64_t>(b) * a.n_heads + h) * S + q] = mrow[f] + log2f(l);
    }
  }
}

template <typename T, int D, int F, int MINB, int NW = 4>
hipError_t launch_fwd(const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  constexpr int BQ = NW * F * 16;
  dim3 grid(a.n_heads, (a.seq + BQ - 1) / BQ, a.batch);
  hipLaunchKernelGGL((attn_fwd_kernel<T, D, F, MINB, NW>), grid, dim3(NW * 64), 0, s, a, static_cast<int>(qkv_bytes));
  return hipGetLastError();
}

}  // namespace
}  // namespace sf

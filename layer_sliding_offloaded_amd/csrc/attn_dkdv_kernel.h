// dK / dV kernel of the direct-load causal attention backward (gfx950),
// parametrised by the keys each wave owns (16 KF).
//
// Every wave reads each 64-query tile's Q and dO from LDS twice (along d for
// the score and dP recompute, transposed for the dK and dV products): 64 KB
// a wave per tile at d = 128, whatever the keys it owns.  With 16 keys (KF =
// 1) those bytes feed 64 MFMAs, with 32 keys (KF = 2) 128.  KF = 2 at d =
// 128 needs the dK / dV accumulators in AGPRs and runs one block per CU; it
// gives the same bits and was measured slower than KF = 1 at two blocks per
// CU at the 1.3B, 6.7B and 123B-shaped layers (402 vs 443 us at the 6.7B
// shape), so KF = 1 is what runs.
//
// What did pay is the order of the work: a unit's length is the number of
// query tiles at or after its keys, from S / 64 down to 1, and with few KV
// heads (the 123B-shaped GQA layer: 8 KV heads, batch 1) the whole-group
// units were only two per CU, the longest ones sharing CUs.  Units are now
// numbered longest first across all KV heads and batches, and a GQA group
// is split into head shares (attn_kv_split) when the units would be few:
// 1594 -> 875 us at the 123B shape (the reduction of the shares included),
// 606 -> 364 us at the 6.7B shape.  The arithmetic of a key does not depend
// on KF or on the unit order; the split changes only the order in which the
// shares' fp32 sums are added.
#pragma once

#include <type_traits>

#include "attn_tiles.h"

namespace sf {
namespace {

// ---------------------------------------------------------------- dK, dV
// Block: NWV waves x 16 KF keys of one (b, KV head); loops over the query
// heads of its share of the group and every 64-query tile at or after its
// first key.  Q and dO tiles (kind 1) serve both the score recompute (along
// d) and the dK / dV products (transposed, along the queries); log-sum-exp
// and D of the tile's queries are staged next to them.
//
// Work units: (key block, head share g of a.kv_split, KV head, batch), one
// block each, numbered so that the earliest key blocks (the most query tiles)
// come first.  With a.kv_split = 1 a unit covers the whole group and stores
// dK (scaled, inverse RoPE) and dV; otherwise it stores its fp32 partial sums
// to a.dkv_partial[g] ([B S, n_kv D] for dK, then the same for dV), which
// attn_dkv_reduce adds in order of g.
template <typename T, int D, int KF, int NWV>
__global__ void __launch_bounds__(NWV * 64)
attn_dkdv_direct(const AttnArgs a, int qkv_bytes, int dout_bytes, int stat_bytes) {
  constexpr int KW = 16 * KF, BKV = NWV * KW, BQ = 64, NW = NWV;
  constexpr int DC = D / 32;
  constexpr int FD = D / 16;
  constexpr int TB = BQ * D * 2;
  __shared__ __attribute__((aligned(1024))) char Q0[TB];
  __shared__ __attribute__((aligned(1024))) char Q1[TB];
  __shared__ __attribute__((aligned(1024))) char O0[TB];
  __shared__ __attribute__((aligned(1024))) char O1[TB];
  __shared__ __attribute__((aligned(256))) float L0[2 * BQ];  // lse | D
  __shared__ __attribute__((aligned(256))) float L1[2 * BQ];

  const int S = a.seq;
  const int split = a.kv_split;
  // unit -> (key block, head share, KV head, batch); key block 0 holds the
  // earliest keys, which see the most queries
  int u = blockIdx.x;
  const int per_kb = split * a.n_kv * a.batch;
  const int kb = u / per_kb;
  u -= kb * per_kb;
  const int g = u / (a.n_kv * a.batch);
  u -= g * (a.n_kv * a.batch);
  const int kvh = u % a.n_kv, b = u / a.n_kv;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int kv0 = kb * BKV;
  const int kvw = kv0 + w * KW;
  const int share = a.n_heads / a.n_kv / split;  // query heads of this unit
  const int h0 = kvh * (a.n_heads / a.n_kv) + g * share;

  const __amdgpu_buffer_rsrc_t rq = rsrc(a.qkv, qkv_bytes);
  const __amdgpu_buffer_rsrc_t ro = rsrc(a.dout, dout_bytes);
  const __amdgpu_buffer_rsrc_t rl = rsrc(a.lse, stat_bytes);
  const __amdgpu_buffer_rsrc_t rd = rsrc(a.dsum, stat_bytes);

  // K, V fragments (B operand): lane supplies row kvw + 16 fk + lr, d-chunk lg
  const T* qkv = static_cast<const T*>(a.qkv);
  uint4 kf[KF][DC], vf[KF][DC];
#pragma unroll
  for (int fk = 0; fk < KF; ++fk) {
    const int kv = kvw + fk * 16 + lr;
    const T* kr = qkv + (bs + kv) * ld + (a.n_heads + kvh) * D;
    const T* vr = qkv + (bs + kv) * ld + (a.n_heads + a.n_kv + kvh) * D;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      kf[fk][c] = kv < S ? *reinterpret_cast<const uint4*>(kr + c * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
      vf[fk][c] = kv < S ? *reinterpret_cast<const uint4*>(vr + c * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  f32x4 dk[KF][FD], dv[KF][FD];
#pragma unroll
  for (int fk = 0; fk < KF; ++fk)
#pragma unroll
    for (int d = 0; d < FD; ++d) { dk[fk][d] = f32x4{0.f, 0.f, 0.f, 0.f}; dv[fk][d] = f32x4{0.f, 0.f, 0.f, 0.f}; }

  const float sc = a.scale * kLog2e;
  const int qt0 = kv0 / BQ;
  const int nqt = (S + BQ - 1) / BQ;
  const int per_head = nqt - qt0;
  const int nit = share * per_head;

  // tile loaders: Q rows of head h at column h D, dO rows of head h
  TileLoad<D, NW, 1> lq, lo;
  lq.init(w, lane, (bs * ld) * 2, ld);
  lo.init(w, lane, (bs * a.ld_dout) * 2, a.ld_dout);
  auto issue = [&](int it, char* Qn, char* On, float* Ln) {
    const int h = h0 + it / per_head;
    const int q0 = (qt0 + it % per_head) * BQ;
    lq.issue(rq, Qn, w, S - q0, static_cast<uint32_t>((q0 * ld + h * D) * 2));
    lo.issue(ro, On, w, S - q0, static_cast<uint32_t>((q0 * a.ld_dout + h * D) * 2));
    if (w < 2) {
      // wave 0: log-sum-exp, wave 1: D, one float per lane
      const int64_t st = ((static_cast<int64_t>(b) * a.n_heads + h) * S + q0 + lane) * 4;
      const uint32_t o = q0 + lane < S ? static_cast<uint32_t>(st) : kOOB;
      lds_dma4(w == 0 ? rl : rd, Ln + w * BQ, o);
    }
  };

  int dof[DC], tof[FD];
#pragma unroll
  for (int c = 0; c < DC; ++c) dof[c] = ofs_d1<D>(c, lr, lg);
#pragma unroll
  for (int d = 0; d < FD; ++d) tof[d] = ofs_t<D>(d * 16, lr, lg);

  auto step = [&](int it, const char* Qc, const char* Oc, const float* Lc, char* Qn, char* On, float* Ln) {
    if (it + 1 < nit) issue(it + 1, Qn, On, Ln);
    const int q0 = (qt0 + it % per_head) * BQ;
    if (q0 + BQ - 1 >= kvw) {
      // P^T, dP^T: lane holds X[q = q0 + 16 fq + 4 lg + v][kv = kvw + 16 fk + lr]
      f32x4 p[KF][4], dp[KF][4];
#pragma unroll
      for (int fk = 0; fk < KF; ++fk)
#pragma unroll
        for (int fq = 0; fq < 4; ++fq) { p[fk][fq] = f32x4{0.f, 0.f, 0.f, 0.f}; dp[fk][fq] = f32x4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int fq = 0; fq < 4; ++fq) {
          const uint4 qa = lds16(Qc, dof[c] + fq * 16 * (D * 2));
          const uint4 da = lds16(Oc, dof[c] + fq * 16 * (D * 2));
#pragma unroll
          for (int fk = 0; fk < KF; ++fk) {
            Mfma<T>::run(p[fk][fq], qa, kf[fk][c]);
            Mfma<T>::run(dp[fk][fq], da, vf[fk][c]);
          }
        }
      // P and dS; keys after a query, or queries past the end, exist only
      // near the diagonal / tail, where the masked variant runs
      auto probs = [&](auto mask) {
#pragma unroll
        for (int fq = 0; fq < 4; ++fq) {
          const float4 lse4 = *reinterpret_cast<const float4*>(Lc + fq * 16 + lg * 4);
          const float4 dsm4 = *reinterpret_cast<const float4*>(Lc + BQ + fq * 16 + lg * 4);
          const float lse[4] = {lse4.x, lse4.y, lse4.z, lse4.w};
          const float dsm[4] = {dsm4.x, dsm4.y, dsm4.z, dsm4.w};
#pragma unroll
          for (int fk = 0; fk < KF; ++fk) {
            const int kv = kvw + fk * 16 + lr;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int q = q0 + fq * 16 + lg * 4 + v;
              float pv = __builtin_amdgcn_exp2f(fmaf(p[fk][fq][v], sc, -lse[v]));
              if constexpr (decltype(mask)::value)
                if (kv > q || q >= S) pv = 0.f;
              p[fk][fq][v] = pv;
              dp[fk][fq][v] = pv * (dp[fk][fq][v] - dsm[v]);  // dS
            }
          }
        }
      };
      if ((kvw + KW - 1 > q0) || (q0 + BQ > S)) probs(std::true_type{});
      else probs(std::false_type{});
      // dV^T += dO^T P, dK^T += Q^T dS: lane holds X[kv][d = 16 fd + 4 lg + v]
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 pb[KF], sb[KF];
#pragma unroll
        for (int fk = 0; fk < KF; ++fk) {
          pb[fk] = pack8<T>(p[fk][2 * j], p[fk][2 * j + 1]);
          sb[fk] = pack8<T>(dp[fk][2 * j], dp[fk][2 * j + 1]);
        }
#pragma unroll
        for (int d = 0; d < FD; ++d) {
          const uint4 oa = frag_t<D>(Oc, tof[d], j);
          const uint4 qa = frag_t<D>(Qc, tof[d], j);
#pragma unroll
          for (int fk = 0; fk < KF; ++fk) {
            Mfma<T>::run(dv[fk][d], oa, pb[fk]);
            Mfma<T>::run(dk[fk][d], qa, sb[fk]);
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };

  if (nit > 0) issue(0, Q0, O0, L0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < nit; it += 2) {
    step(it, Q0, O0, L0, Q1, O1, L1);
    if (it + 1 < nit) step(it + 1, Q1, O1, L1, Q0, O0, L0);
  }

  if (split > 1) {
    // fp32 partial sums of this head share, unscaled, before inverse RoPE
    const int64_t ldp = static_cast<int64_t>(a.n_kv) * D;
    float* pk = a.dkv_partial + static_cast<int64_t>(g) * 2 * (static_cast<int64_t>(a.batch) * S) * ldp;
    float* pv = pk + static_cast<int64_t>(a.batch) * S * ldp;
#pragma unroll
    for (int fk = 0; fk < KF; ++fk) {
      const int kv = kvw + fk * 16 + lr;
      if (kv >= S) continue;
      const int64_t row = (bs + kv) * ldp + kvh * D;
#pragma unroll
      for (int d = 0; d < FD; ++d) {
        *reinterpret_cast<f32x4*>(pk + row + d * 16 + lg * 4) = dk[fk][d];
        *reinterpret_cast<f32x4*>(pv + row + d * 16 + lg * 4) = dv[fk][d];
      }
    }
    return;
  }
#pragma unroll
  for (int fk = 0; fk < KF; ++fk) {
    const int kv = kvw + fk * 16 + lr;
    if (kv >= S) continue;
#pragma unroll
    for (int d = 0; d < FD; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dk[fk][d][v] *= a.scale;
    rope_inv<D>(dk[fk], a, kv, lg);
    T* dkp = static_cast<T*>(a.dqkv) + (bs + kv) * a.ld_dqkv + (a.n_heads + kvh) * D;
    T* dvp = static_cast<T*>(a.dqkv) + (bs + kv) * a.ld_dqkv + (a.n_heads + a.n_kv + kvh) * D;
#pragma unroll
    for (int d = 0; d < FD; ++d) {
      store4v<T>(dkp + d * 16 + lg * 4, dk[fk][d]);
      store4v<T>(dvp + d * 16 + lg * 4, dv[fk][d]);
    }
  }
}

template <typename T, int D, int KF>
hipError_t launch_dkdv(const AttnArgs& a, int64_t qkv_bytes, int64_t dout_bytes, int64_t stat_bytes, hipStream_t s) {
  constexpr int BKV = 4 * 16 * KF;
  const int64_t units = static_cast<int64_t>((a.seq + BKV - 1) / BKV) * a.kv_split * a.n_kv * a.batch;
  hipLaunchKernelGGL((attn_dkdv_direct<T, D, KF, 4>), dim3(static_cast<unsigned>(units)), dim3(256), 0, s, a,
                     static_cast<int>(qkv_bytes), static_cast<int>(dout_bytes), static_cast<int>(stat_bytes));
  return hipGetLastError();
}

}  // namespace
}  // namespace sf

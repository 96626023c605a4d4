// Causal flash attention, bf16 or fp16 storage, with global -> LDS direct loads (gfx950).
//
// Same mathematics and data layout as the register-staged kernels (online
// softmax in base 2 over key tiles, log-sum-exp saved per (b, h, s),
// deterministic backward split into a dK/dV kernel and a dQ kernel, GQA by
// contiguous head groups, inverse RoPE in the gradient epilogues), arranged
// for the CDNA4 memory path:
//  - key/value (forward, dQ) and query/dO (dK/dV) tiles are copied from HBM
//    straight into LDS by buffer loads, 16 bytes a lane, 1 KB a wave
//    instruction; rows past the sequence end read as zeros through an
//    out-of-range offset;
//  - tiles whose rows feed the MFMA A operand along d ([row][d], k = d) are
//    held as 64-column blocks of 128-byte rows, slots XOR-swizzled by row;
//  - tiles that feed it along the sequence (V and dO for the P.V-type
//    products, Q and K for the dK / dQ products) are read with the LDS
//    transpose load straight from their [row][d] layout -- no register
//    transposes -- with a slot swizzle by row that keeps 32 lanes on
//    distinct banks;
//  - each pipeline stage lives in its own LDS array and the key loop is
//    unrolled by two, so the compiler can see that a stage's reads never
//    alias the next stage's loads and does not serialise them; the next
//    tile's loads are issued before the current tile's MFMAs.
#include <algorithm>
#include <type_traits>

#include "attn_dkdv_kernel.h"
#include "attn_fwd_kernel.h"
#include "attn_tiles.h"

namespace sf {

namespace {

// -------------------------------------------------------------------- dQ
// Block: NWV waves x 16 F queries of one (b, h); key tiles of 64 (kind 1: the
// score recompute reads K and V along d, the dQ product reads K transposed).
template <typename T, int D, int F, int NWV>
__global__ void __launch_bounds__(NWV * 64)
attn_dq_direct(const AttnArgs a, int qkv_bytes) {
  constexpr int QW = 16 * F, BQ = NWV * QW, BKV = 64, NW = NWV;
  constexpr int DC = D / 32;
  constexpr int FD = D / 16;
  constexpr int TB = BKV * D * 2;
  __shared__ __attribute__((aligned(1024))) char K0[TB];
  __shared__ __attribute__((aligned(1024))) char K1[TB];
  __shared__ __attribute__((aligned(1024))) char V0[TB];
  __shared__ __attribute__((aligned(1024))) char V1[TB];

  const int S = a.seq;
  // grid (n_heads, query tiles, batch), query tiles backwards: the blocks
  // with the most key tiles are dispatched first across all heads
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
  const int qw = q0 + w * QW;

  const __amdgpu_buffer_rsrc_t rs = rsrc(a.qkv, qkv_bytes);
  TileLoad<D, NW, 1> lk, lv;
  lk.init(w, lane, (bs * ld + (a.n_heads + kvh) * D) * 2, ld);
  lv.init(w, lane, (bs * ld + (a.n_heads + a.n_kv + kvh) * D) * 2, ld);

  // Q, dO fragments (B operand) and the rows' statistics
  const T* qbase = static_cast<const T*>(a.qkv) + bs * ld + h * D;
  const T* dbase = static_cast<const T*>(a.dout) + bs * a.ld_dout + h * D;
  uint4 qf[F][DC], df[F][DC];
  float lse[F], dsm[F];
  const int64_t srow = (static_cast<int64_t>(b) * a.n_heads + h) * S;
#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int q = qw + f * 16 + lr;
    const bool ok = q < S;
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      qf[f][c] = ok ? *reinterpret_cast<const uint4*>(qbase + static_cast<int64_t>(q) * ld + c * 32 + lg * 8)
                    : make_uint4(0, 0, 0, 0);
      df[f][c] = ok ? *reinterpret_cast<const uint4*>(dbase + static_cast<int64_t>(q) * a.ld_dout + c * 32 + lg * 8)
                    : make_uint4(0, 0, 0, 0);
    }
    lse[f] = ok ? a.lse[srow + q] : 0.f;
    dsm[f] = ok ? a.dsum[srow + q] : 0.f;
  }
  f32x4 dq[F][FD];
#pragma unroll
  for (int f = 0; f < F; ++f)
#pragma unroll
    for (int d = 0; d < FD; ++d) dq[f][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = a.scale * kLog2e;
  const int nkv = (min(q0 + BQ, S) - 1) / BKV + 1;
  int dof[DC], tof[FD];
#pragma unroll
  for (int c = 0; c < DC; ++c) dof[c] = ofs_d1<D>(c, lr, lg);
#pragma unroll
  for (int d = 0; d < FD; ++d) tof[d] = ofs_t<D>(d * 16, lr, lg);

  lk.issue(rs, K0, w, S, 0);
  lv.issue(rs, V0, w, S, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto tile = [&](int kt, const char* Kc, const char* Vc, char* Kn, char* Vn) {
    const int kv0 = kt * BKV;
    if (kt + 1 < nkv) {
      const uint32_t adv = static_cast<uint32_t>((kv0 + BKV) * ld * 2);
      lk.issue(rs, Kn, w, S - kv0 - BKV, adv);
      lv.issue(rs, Vn, w, S - kv0 - BKV, adv);
    }
    if (kv0 <= qw + QW - 1) {
      // S, dP: lane holds X[q = qw + 16 f + lr][kv = kv0 + 16 fk + 4 lg + v]
      f32x4 s[F][4], dp[F][4];
#pragma unroll
      for (int f = 0; f < F; ++f)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk) { s[f][fk] = f32x4{0.f, 0.f, 0.f, 0.f}; dp[f][fk] = f32x4{0.f, 0.f, 0.f, 0.f}; }
#pragma unroll
      for (int c = 0; c < DC; ++c)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk) {
          const uint4 ka = lds16(Kc, dof[c] + fk * 16 * (D * 2));
          const uint4 va = lds16(Vc, dof[c] + fk * 16 * (D * 2));
#pragma unroll
          for (int f = 0; f < F; ++f) {
            Mfma<T>::run(s[f][fk], ka, qf[f][c]);
            Mfma<T>::run(dp[f][fk], va, df[f][c]);
          }
        }
      // (one predicated path: a separate unmasked copy of this loop pushes
      // the 4-wave d = 128 kernel past 256 registers)
      const bool masked = (kv0 + BKV - 1 > qw) || (kv0 + BKV > S);
#pragma unroll
      for (int f = 0; f < F; ++f) {
        const int q = qw + f * 16 + lr;
#pragma unroll
        for (int fk = 0; fk < 4; ++fk)
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int kv = kv0 + fk * 16 + lg * 4 + v;
            float pv = __builtin_amdgcn_exp2f(fmaf(s[f][fk][v], sc, -lse[f]));
            if (masked && (kv > q || kv >= S)) pv = 0.f;
            s[f][fk][v] = pv * (dp[f][fk][v] - dsm[f]);  // dS
          }
      }
      // dQ^T += K^T dS^T: lane holds dQ[q = qw + 16 f + lr][d = 16 fd + 4 lg + v]
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        uint4 sb[F];
#pragma unroll
        for (int f = 0; f < F; ++f) sb[f] = pack8<T>(s[f][2 * j], s[f][2 * j + 1]);
#pragma unroll
        for (int d = 0; d < FD; ++d) {
          const uint4 ka = frag_t<D>(Kc, tof[d], j);
#pragma unroll
          for (int f = 0; f < F; ++f) Mfma<T>::run(dq[f][d], ka, sb[f]);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  for (int kt = 0; kt < nkv; kt += 2) {
    tile(kt, K0, V0, K1, V1);
    if (kt + 1 < nkv) tile(kt + 1, K1, V1, K0, V0);
  }

#pragma unroll
  for (int f = 0; f < F; ++f) {
    const int q = qw + f * 16 + lr;
    if (q >= S) continue;
#pragma unroll
    for (int d = 0; d < FD; ++d)
#pragma unroll
      for (int v = 0; v < 4; ++v) dq[f][d][v] *= a.scale;
    rope_inv<D>(dq[f], a, q, lg);
    T* dqp = static_cast<T*>(a.dqkv) + (bs + q) * a.ld_dqkv + h * D;
#pragma unroll
    for (int d = 0; d < FD; ++d) store4v<T>(dqp + d * 16 + lg * 4, dq[f][d]);
  }
}

// dK (scaled, inverse RoPE) and dV from the fp32 partial sums of the
// kv_split head shares, added in order of the share.  Thread: 4 columns of
// the first half of d of one (token, KV head) and their RoPE partners.
template <typename T, int D>
__global__ void __launch_bounds__(256)
attn_dkv_reduce(const AttnArgs a) {
  constexpr int Q4 = D / 8;  // 4-column groups in half of d
  const int64_t T_ = static_cast<int64_t>(a.batch) * a.seq;
  const int64_t items = T_ * a.n_kv * Q4;
  const int64_t ldp = static_cast<int64_t>(a.n_kv) * D;
  const int64_t gstride = 2 * T_ * ldp;
  for (int64_t it = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; it < items;
       it += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int i4 = static_cast<int>(it % Q4);
    const int64_t rest = it / Q4;
    const int kvh = static_cast<int>(rest % a.n_kv);
    const int64_t t = rest / a.n_kv;
    const int pos = static_cast<int>(t % a.seq);
    const int64_t base = t * ldp + kvh * D + i4 * 4;
    f32x4 k1 = f32x4{0.f, 0.f, 0.f, 0.f}, k2 = k1, v1 = k1, v2 = k1;
    for (int g = 0; g < a.kv_split; ++g) {
      const float* pk = a.dkv_partial + g * gstride + base;
      const float* pv = pk + T_ * ldp;
      k1 += *reinterpret_cast<const f32x4*>(pk);
      k2 += *reinterpret_cast<const f32x4*>(pk + D / 2);
      v1 += *reinterpret_cast<const f32x4*>(pv);
      v2 += *reinterpret_cast<const f32x4*>(pv + D / 2);
    }
    f32x4 o1, o2;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i4 * 4 + v;
      const float c = a.rope_cos[static_cast<int64_t>(pos) * (D / 2) + i];
      const float sn = a.rope_sin[static_cast<int64_t>(pos) * (D / 2) + i];
      const float u1 = k1[v] * a.scale, u2 = k2[v] * a.scale;
      o1[v] = u1 * c + u2 * sn;
      o2[v] = u2 * c - u1 * sn;
    }
    T* dk = static_cast<T*>(a.dqkv) + t * a.ld_dqkv + (a.n_heads + kvh) * D + i4 * 4;
    T* dv = static_cast<T*>(a.dqkv) + t * a.ld_dqkv + (a.n_heads + a.n_kv + kvh) * D + i4 * 4;
    store4v<T>(dk, o1);
    store4v<T>(dk + D / 2, o2);
    store4v<T>(dv, v1);
    store4v<T>(dv + D / 2, v2);
  }
}

template <typename T, int D>
hipError_t run_bwd_direct(const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  const int64_t nt = static_cast<int64_t>(a.batch) * a.seq;
  const int64_t dout_bytes = ((nt - 1) * a.ld_dout + static_cast<int64_t>(a.n_heads) * D) * 2;
  const int64_t stat_bytes = static_cast<int64_t>(a.batch) * a.n_heads * a.seq * 4;
  // Block shapes (measured; every shape gives the same bits for one
  // kv_split): dK/dV with 4 waves of 16 keys; dQ with 4 waves of 32 queries
  // when that still makes two blocks per CU, else 8 waves of 16.  (This file
  // is compiled with the MFMA accumulators held in VGPRs, which made the
  // 4-wave dQ the fastest: no AGPR-to-VGPR copies before the softmax
  // arithmetic.)
  if (a.kv_split < 1 || (a.n_heads / a.n_kv) % a.kv_split || (a.kv_split > 1 && !a.dkv_partial))
    return hipErrorInvalidValue;
  hipError_t e = launch_dkdv<T, D, 1>(a, qkv_bytes, dout_bytes, stat_bytes, s);
  if (e != hipSuccess) return e;
  if (a.kv_split > 1) {
    const int64_t items = nt * a.n_kv * (D / 8);
    const int blocks = static_cast<int>(std::min<int64_t>((items + 255) / 256, 8192));
    hipLaunchKernelGGL((attn_dkv_reduce<T, D>), dim3(blocks), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (static_cast<int64_t>((a.seq + 127) / 128) * a.n_heads * a.batch >= 512)
    hipLaunchKernelGGL((attn_dq_direct<T, D, 2, 4>), dim3(a.n_heads, (a.seq + 127) / 128, a.batch), dim3(256), 0, s,
                       a, static_cast<int>(qkv_bytes));
  else
    hipLaunchKernelGGL((attn_dq_direct<T, D, 1, 8>), dim3(a.n_heads, (a.seq + 127) / 128, a.batch), dim3(512), 0, s,
                       a, static_cast<int>(qkv_bytes));
  return hipGetLastError();
}

}  // namespace

bool attention_direct_ok(const AttnArgs& a, int64_t* qkv_bytes) {
  if ((a.head_dim != 64 && a.head_dim != 128) || a.ld_qkv % 8 || a.seq < 1 || a.batch < 1) return false;
  if (reinterpret_cast<uintptr_t>(a.qkv) & 15u) return false;
  const int64_t T = static_cast<int64_t>(a.batch) * a.seq;
  *qkv_bytes = ((T - 1) * a.ld_qkv + static_cast<int64_t>(a.n_heads + 2 * a.n_kv) * a.head_dim) * 2;
  return *qkv_bytes < (int64_t{1} << 31) - 1024;
}

hipError_t attention_fwd_direct(int dtype, const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  if (dtype == 2)
    return a.head_dim == 64 ? launch_fwd<f16, 64, 2, 2>(a, qkv_bytes, s) : launch_fwd<f16, 128, 2, 2>(a, qkv_bytes, s);
  return a.head_dim == 64 ? launch_fwd<bf16, 64, 2, 2>(a, qkv_bytes, s) : launch_fwd<bf16, 128, 2, 2>(a, qkv_bytes, s);
}

hipError_t attention_bwd_direct(int dtype, const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  if (dtype == 2)
    return a.head_dim == 64 ? run_bwd_direct<f16, 64>(a, qkv_bytes, s) : run_bwd_direct<f16, 128>(a, qkv_bytes, s);
  return a.head_dim == 64 ? run_bwd_direct<bf16, 64>(a, qkv_bytes, s) : run_bwd_direct<bf16, 128>(a, qkv_bytes, s);
}

}  // namespace sf

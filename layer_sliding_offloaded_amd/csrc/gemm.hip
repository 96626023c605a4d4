// MFMA GEMM for gfx950.
//
// Every dense projection of the decoder block and of the LM head goes
// through these kernels: the forward products y = x W^T (NT), the input
// gradients dX = dY W (NN) and the weight gradients dW = dY^T X (TN).  Fused
// epilogues carry the elementwise steps that follow a product (RoPE on q/k,
// SwiGLU forward and backward, the residual add, fp32 gradient stores), so
// those tensors make one trip through HBM instead of three.
//
// Tile scheme.  A block computes a BM x BN output tile with NW = (BM/WM) *
// (BN/WN) waves, each owning a WM x WN sub-tile built from 16x16x32 MFMA
// fragments.  bf16 operands (the production path) are copied global -> LDS
// by the buffer unit itself (buffer_load ... lds, no VGPR round trip) into
// XOR-swizzled stage buffers: k-contiguous operands as [row][k], the
// transposed side of NN / TN as [k][row] read back with the LDS transpose
// load.  Four kernels share those helpers:
//  - gemm_direct_kernel: 2 stages of 64 k (grids that fill the chip with
//    128 x 128 tiles);
//  - gemm_pipe_kernel: NS stages of BK k, the loads of stage kt + NS - 1
//    issued while stage kt is multiplied (small grids);
//  - gemm_pp_kernel: 256 x 256 tiles whose 8 waves split into two groups
//    that alternate between a memory phase and an MFMA phase (large grids);
//  - gemm_pl_kernel: the same for NT with B staged in whole 128-byte lines
//    (64 k per stage): one L2 request per line of B instead of two.
// The register-staged gemm_kernel (loads through VGPRs, in-register 8x8 /
// 4x4 transposes of row-contiguous operands, 144-byte padded LDS rows)
// serves fp32 and operands the direct loads cannot take.
//
// Output fragments are computed transposed (MFMA A-operand = B tile) so each
// lane ends with 4 consecutive output columns of one row: 8-byte (bf16) or
// 16-byte (fp32) stores, and the partner columns that RoPE (i, i + d/2) and
// SwiGLU (gate j, up j) need sit in the same lane.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "common.h"
#include "gemm.h"

namespace sf {

namespace {

constexpr int kStageBytes = 128;  // k-bytes per LDS stage row

// Map a tile-local B row (= output column slot) to the global B row, or -1.
// Pair epilogues permute the slots so that slot q and q + WN/2 of a wave are
// partners; otherwise the map is the identity.
template <Epi E, int WN>
struct ColMap {
  __device__ __forceinline__ static int brow(int r, int n0, const GemmArgs& g, int BN) {
    if constexpr (E == Epi::Rope) {
      const int wn = r / WN, q = r % WN, half = WN / 2;
      const int p = wn * half + (q % half);
      const int hd2 = g.head_dim / 2;
      const int col = n0 + (p / hd2) * g.head_dim + (p % hd2) + (q >= half ? hd2 : 0);
      return col < g.N ? col : -1;
    } else if constexpr (E == Epi::SwigluFwd) {
      const int wn = r / WN, q = r % WN, half = WN / 2;
      const int f = n0 / 2 + wn * half + (q % half);
      if (f >= g.ffn) return -1;
      return q >= half ? g.ffn + f : f;
    } else {
      const int col = n0 + r;
      return col < g.N ? col : -1;
    }
  }
};

template <typename T, int ROWS, int NT, bool KC>
struct Loader {
  static constexpr int VE = 16 / sizeof(T);
  static constexpr int KG = kStageBytes / 16;  // 16-byte k-groups per row = 8
  static constexpr int BKE = kStageBytes / sizeof(T);
  static constexpr int ROW = BKE + VE;
  // k-contiguous: one 16-byte vector per (row, k-group)
  static constexpr int NVEC_K = (ROWS * KG + NT - 1) / NT;
  // row-contiguous: blocks of 4 k-rows x VE columns, transposed on the way
  // into LDS (4 k-values per LDS row segment: 8 B bf16, 16 B fp32)
  static constexpr int KB = 4;
  static constexpr int KGT = BKE / KB;
  static constexpr int NBLK = (ROWS / VE) * KGT;
  static constexpr int NB_T = (NBLK + NT - 1) / NT;
  static constexpr int NREG = KC ? NVEC_K : NB_T * KB;
  uint4 reg[NREG];

  // src: element (row, k) at src[row * ld + k] (KC) or src[k * ld + row] (!KC).
  // rowmap(r) gives the global row of tile row r, or -1.
  template <typename RowMap>
  __device__ __forceinline__ void load(const T* __restrict__ src, int64_t ld, int k0, int K,
                                       int tid, RowMap rowmap) {
    if constexpr (KC) {
#pragma unroll
      for (int j = 0; j < NVEC_K; ++j) {
        const int i = tid + j * NT;
        const int r = i / KG, c = i % KG;
        const int kk = k0 + c * VE;
        const int gr = (i < ROWS * KG) ? rowmap(r) : -1;
        if (gr >= 0 && kk < K)
          reg[j] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(gr) * ld + kk);
        else
          reg[j] = make_uint4(0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB_T; ++j) {
        const int i = tid + j * NT;
        const int kg = i % KGT, mg = i / KGT;
        const int gc = (i < NBLK) ? rowmap(mg * VE) : -1;
#pragma unroll
        for (int r = 0; r < KB; ++r) {
          const int kk = k0 + kg * KB + r;
          if (gc >= 0 && kk < K)
            reg[j * KB + r] = *reinterpret_cast<const uint4*>(src + static_cast<int64_t>(kk) * ld + gc);
          else
            reg[j * KB + r] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store(T* lds, int tid) {
    if constexpr (KC) {
#pragma unroll
      for (int j = 0; j < NVEC_K; ++j) {
        const int i = tid + j * NT;
        if (ROWS * KG % NT == 0 || i < ROWS * KG) {
          const int r = i / KG, c = i % KG;
          *reinterpret_cast<uint4*>(lds + r * ROW + c * VE) = reg[j];
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < NB_T; ++j) {
        const int i = tid + j * NT;
        if (NBLK % NT == 0 || i < NBLK) {
          const int kg = i % KGT, mg = i / KGT;
          const uint4* v = &reg[j * KB];
          if constexpr (sizeof(T) == 2) {
            // 4 rows x 8 bf16 -> 8 columns x 4 bf16
            const uint32_t w[4][4] = {{v[0].x, v[0].y, v[0].z, v[0].w}, {v[1].x, v[1].y, v[1].z, v[1].w},
                                      {v[2].x, v[2].y, v[2].z, v[2].w}, {v[3].x, v[3].y, v[3].z, v[3].w}};
#pragma unroll
            for (int c = 0; c < 8; ++c) {
              const int d = c >> 1;
              const uint32_t lo = (c & 1) ? ((w[0][d] >> 16) | (w[1][d] & 0xFFFF0000u))
                                          : ((w[0][d] & 0xFFFFu) | (w[1][d] << 16));
              const uint32_t hi = (c & 1) ? ((w[2][d] >> 16) | (w[3][d] & 0xFFFF0000u))
                                          : ((w[2][d] & 0xFFFFu) | (w[3][d] << 16));
              *reinterpret_cast<uint2*>(lds + (mg * VE + c) * ROW + kg * KB) = make_uint2(lo, hi);
            }
          } else {
            uint4 t[4];
            transpose4x4_b32(v, t);
#pragma unroll
            for (int c = 0; c < 4; ++c)
              *reinterpret_cast<uint4*>(lds + (mg * VE + c) * ROW + kg * KB) = t[c];
          }
        }
      }
    }
  }
};

// Split-K factor for a grid of `tiles` output tiles: grids of at least half
// the CUs' worth of tiles run unsplit; smaller ones double the split while
// the blocks still fit one pass over the 256 CUs and every k-range stays at
// least 1024 deep (measured: a split of short k-ranges, or of a grid that
// already fills half the chip, costs more in partial-sum traffic and the
// reduction than it gains).
int splitk_factor(int tiles, int K) {
  if (tiles >= 128) return 1;
  int S = 1;
  while (S < 8 && tiles * S * 2 <= 256 && K / (S * 2) >= 1024) S *= 2;
  return S;
}

// Long-K products with few output tiles (the LM head's input gradient:
// [T, H] from K = vocab): 256 x 256 ping-pong tiles, K split so that the
// grid covers the CUs about once (2 to 8 ranges of >= 2048), then the
// fixed-order reduction.  1: not such a product.
int longk_split(int M, int N, int K) {
  const long t256 = static_cast<long>((M + 255) / 256) * ((N + 255) / 256);
  if (t256 >= 160 || K < 8192 || K < 4L * std::max(M, N)) return 1;
  int S = static_cast<int>(std::min<long>(8, (256 + t256 - 1) / t256));
  while (S > 1 && K / S < 2048) --S;
  return S;
}

// Logistic sigmoid with the hardware reciprocal (v_rcp_f32, 1 ulp) instead
// of an IEEE division, which costs about ten instructions per element in
// the SwiGLU epilogues; large |z| still give exactly 0 and 1.
__device__ __forceinline__ float sigmoid_f(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
__device__ __forceinline__ float silu_f(float z) { return z * sigmoid_f(z); }

template <typename T>
__device__ __forceinline__ void load4(const T* p, float* v) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    const uint4 w = make_uint4(u.x, u.y, 0u, 0u);
    float f[8];
    Elem<T>::unpack(w, f);
    v[0] = f[0]; v[1] = f[1]; v[2] = f[2]; v[3] = f[3];
  } else {
    const float4 f = *reinterpret_cast<const float4*>(p);
    v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
  }
}

// Tile order: blocks are dealt to the 8 XCDs round-robin; give each XCD a
// contiguous range of tiles, then walk that range in groups of GM tile-rows
// so the A rows and B columns a group shares stay in that XCD's L2.  GM = 4
// measured best over the layer GEMMs from hidden 1024 to 12288 (against 2,
// 8, 16, 32; 16 and 32 lose up to 30 %): at T = 8192, hidden 4096 the ten
// layer GEMMs take 1.3 % less time than with GM = 8, at hidden 1024 and
// 2048 the same within noise; with the whole-line NT kernel the 24 layer
// GEMMs of the 6.7B and 123B shapes take 0.6 % less than with GM = 8 and
// 1.5 % less than with GM = 2.
__device__ __forceinline__ void tile_coords(int ntm, int ntn, int* tm, int* tn) {
  const int ntiles = ntm * ntn;
  int t = blockIdx.x;
  if (ntiles % 8 == 0) t = (t % 8) * (ntiles / 8) + t / 8;
  constexpr int GM = 4;
  const int group = t / (GM * ntn);
  const int first_m = group * GM;
  const int gsize = min(ntm - first_m, GM);
  *tm = first_m + (t % (GM * ntn)) % gsize;
  *tn = (t % (GM * ntn)) / gsize;
}

// Epilogues that take the row-contiguous path below (bf16 storage).
// (pair epilogues need 64-column wave tiles: 32 output columns per plane)
template <Epi E, int WN>
constexpr bool kRowsEpi = E == Epi::Store || E == Epi::StoreF32 || E == Epi::Resid || E == Epi::SwigluBwd ||
                          ((E == Epi::SwigluFwd || E == Epi::Rope) && WN >= 64);

// LDS bytes of one wave's staging patch in the row epilogue: 16 rows of the
// wave's output columns in fp32 (pair epilogues: gate and up planes of WN/2
// columns each), rows padded by 4 floats.
template <int WN, Epi E>
constexpr int kPatchBytes = (E == Epi::SwigluFwd || E == Epi::Rope ? 2 * 16 * (WN / 2 + 4) : 16 * (WN + 4)) * 4;

// Row-contiguous epilogue.  A wave's accumulators hold, per lane, 4 columns
// of one row, so direct stores and operand loads touch 16 rows x 32 bytes
// per instruction.  Here each 16-row slice of the wave tile goes through a
// private LDS patch and comes back as 8 consecutive columns of one row per
// lane: the residual, gate and up operands are read and the outputs written
// as whole 16-byte vectors (one 64- or 128-byte row segment per 4 or 8
// lanes), and the operands of the next slice are requested before the
// current one is finished.  Same arithmetic as the fragment epilogue, so the
// same bits.  Caller: every wave done with the main loop's LDS (barrier),
// g.rows_epi set (16-byte aligned outputs and operands, ldc, ldr and the
// column count multiples of 8, no split-K partials).
template <typename T, int WM, int WN, int FM, int FN, Epi E>
__device__ __forceinline__ void epilogue_rows(const GemmArgs& g, const f32x4 (&acc)[FM][FN], int m0, int n0,
                                              int wm, int wn, int lane, float* patch) {
  constexpr bool PAIR = E == Epi::SwigluFwd || E == Epi::Rope;
  constexpr int WR = PAIR ? WN / 2 : WN;  // output columns of the wave (pairs: first members)
  constexpr int LDW = WR + 4;
  constexpr int LPR = WR / 8;   // lanes per row
  constexpr int RPI = 64 / LPR;  // rows per pass
  constexpr int NIT = 16 / RPI;  // passes per 16-row slice
  constexpr int NOP = E == Epi::SwigluBwd ? 2 : (E == Epi::Resid ? 1 : 0);
  static_assert(WR % 8 == 0 && 16 % RPI == 0, "wave tile width");
  const int lr = lane % 16, lg = lane / 16;
  const int rr = lane / LPR, cc = (lane % LPR) * 8;
  // output column of this lane's 8 (gate/up index f for SwiGLU; for RoPE the
  // first column of the 8 pairs (c, c + head_dim/2), whose 8 first members
  // share one head since head_dim/2 is a multiple of 8)
  int n;
  if constexpr (E == Epi::Rope) {
    const int pp = wn * WR + cc, hd2 = g.head_dim / 2;
    n = n0 + (pp / hd2) * g.head_dim + (pp % hd2);
  } else {
    n = PAIR ? n0 / 2 + wn * WR + cc : n0 + wn * WN + cc;
  }
  const bool n_ok = n < (E == Epi::SwigluFwd ? g.ffn : g.N);
  const int mb = m0 + wm * WM + rr;
  uint4 op[2][NIT][NOP > 0 ? NOP : 1];
  auto fetch = [&](int i, uint4 (&dst)[NIT][NOP > 0 ? NOP : 1]) {
    if constexpr (NOP > 0) {
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const int m = mb + i * 16 + it * RPI;
        const int64_t ro = static_cast<int64_t>(m) * g.ldr + n;
        if (m < g.M && n_ok) {
          dst[it][0] = *reinterpret_cast<const uint4*>(static_cast<const T*>(g.R) + ro);
          if constexpr (NOP > 1) dst[it][1] = *reinterpret_cast<const uint4*>(static_cast<const T*>(g.R2) + ro);
        }
      }
    }
  };
  fetch(0, op[0]);
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    if (i + 1 < FM) fetch(i + 1, op[(i + 1) & 1]);
    // lane (lr, lg) holds row lr, slots j*16 + 4*lg .. +3
#pragma unroll
    for (int j = 0; j < (PAIR ? FN / 2 : FN); ++j) {
      *reinterpret_cast<f32x4*>(patch + lr * LDW + j * 16 + lg * 4) = acc[i][j];
      if constexpr (PAIR)
        *reinterpret_cast<f32x4*>(patch + 16 * LDW + lr * LDW + j * 16 + lg * 4) = acc[i][j + FN / 2];
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int r = it * RPI + rr;
      const int m = mb + i * 16 + it * RPI;
      float o[8];
      {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(patch + r * LDW + cc);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(patch + r * LDW + cc + 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) { o[v] = lo[v]; o[4 + v] = hi[v]; }
      }
      if (m >= g.M || !n_ok) continue;
      const int64_t off = static_cast<int64_t>(m) * g.ldc + n;
      if constexpr (E == Epi::Store) {
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C) + off) = Elem<T>::pack(o);
      } else if constexpr (E == Epi::StoreF32) {
        float* c = static_cast<float*>(g.C) + off;
        *reinterpret_cast<float4*>(c) = make_float4(o[0], o[1], o[2], o[3]);
        *reinterpret_cast<float4*>(c + 4) = make_float4(o[4], o[5], o[6], o[7]);
      } else if constexpr (E == Epi::Resid) {
        float rv[8];
        Elem<T>::unpack(op[i & 1][it][0], rv);
#pragma unroll
        for (int v = 0; v < 8; ++v) o[v] += rv[v];
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C) + off) = Elem<T>::pack(o);
      } else if constexpr (E == Epi::SwigluBwd) {
        float G[8], U[8], dG[8], dU[8];
        Elem<T>::unpack(op[i & 1][it][0], G);
        Elem<T>::unpack(op[i & 1][it][1], U);
#pragma unroll
        for (int v = 0; v < 8; ++v) {
          const float sg = sigmoid_f(G[v]);
          dG[v] = o[v] * U[v] * sg * (1.0f + G[v] * (1.0f - sg));
          dU[v] = o[v] * G[v] * sg;
        }
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C) + off) = Elem<T>::pack(dG);
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C2) + off) = Elem<T>::pack(dU);
      } else if constexpr (E == Epi::Rope) {
        // o: first members (columns n ..), u: partners (columns n + head_dim/2 ..)
        float u[8];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(patch + 16 * LDW + r * LDW + cc);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(patch + 16 * LDW + r * LDW + cc + 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) { u[v] = lo[v]; u[4 + v] = hi[v]; }
        float o1[8], o2[8];
        if (n < g.rope_cols) {
          const int hd2 = g.head_dim / 2;
          const int64_t t = static_cast<int64_t>(m % g.seq) * hd2 + n % g.head_dim;
          const float4 c0 = *reinterpret_cast<const float4*>(g.rope_cos + t);
          const float4 c1 = *reinterpret_cast<const float4*>(g.rope_cos + t + 4);
          const float4 s0 = *reinterpret_cast<const float4*>(g.rope_sin + t);
          const float4 s1 = *reinterpret_cast<const float4*>(g.rope_sin + t + 4);
          const float cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          const float sn[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
          for (int v = 0; v < 8; ++v) {
            o1[v] = o[v] * cs[v] - u[v] * sn[v];
            o2[v] = u[v] * cs[v] + o[v] * sn[v];
          }
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) { o1[v] = o[v]; o2[v] = u[v]; }
        }
        T* c = static_cast<T*>(g.C) + off;
        *reinterpret_cast<uint4*>(c) = Elem<T>::pack(o1);
        *reinterpret_cast<uint4*>(c + g.head_dim / 2) = Elem<T>::pack(o2);
      } else {  // SwigluFwd: o = gate; up from the second plane
        float u[8], a[8];
        const f32x4 lo = *reinterpret_cast<const f32x4*>(patch + 16 * LDW + r * LDW + cc);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(patch + 16 * LDW + r * LDW + cc + 4);
#pragma unroll
        for (int v = 0; v < 4; ++v) { u[v] = lo[v]; u[4 + v] = hi[v]; }
#pragma unroll
        for (int v = 0; v < 8; ++v) a[v] = silu_f(o[v]) * u[v];
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C) + off) = Elem<T>::pack(o);
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C2) + off) = Elem<T>::pack(u);
        *reinterpret_cast<uint4*>(static_cast<T*>(g.C3) + off) = Elem<T>::pack(a);
      }
    }
  }
}

// Fused epilogue of one wave's WM x WN accumulator tile.
template <typename T, int WM, int WN, int FM, int FN, Epi E>
__device__ __forceinline__ void epilogue(const GemmArgs& g, const f32x4 (&acc)[FM][FN], int m0, int n0, int wm,
                                         int wn, int lr, int lg, int BN) {
  // lane holds C[m][c .. c+3] with m = row lr of fragment i, c = 4*lg of
  // fragment j (tile-local slot numbering, mapped through ColMap).
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int m = m0 + wm * WM + i * 16 + lr;
    if (m >= g.M) continue;
    if constexpr (E == Epi::Rope || E == Epi::SwigluFwd) {
#pragma unroll
      for (int j = 0; j < FN / 2; ++j) {
        const int slot = wn * WN + j * 16 + lg * 4;
        const int c1 = ColMap<E, WN>::brow(slot, n0, g, BN);
        if (c1 < 0) continue;
        const f32x4 a1 = acc[i][j], a2 = acc[i][j + FN / 2];
        float o1[4], o2[4];
        if constexpr (E == Epi::Rope) {
          const int c2 = c1 + g.head_dim / 2;
          T* C = static_cast<T*>(g.C);
          if (c1 < g.rope_cols) {
            const int pos = m % g.seq;
            const int fi = c1 % g.head_dim;  // < head_dim / 2
            const float* cs = g.rope_cos + static_cast<int64_t>(pos) * (g.head_dim / 2) + fi;
            const float* sn = g.rope_sin + static_cast<int64_t>(pos) * (g.head_dim / 2) + fi;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              o1[v] = a1[v] * cs[v] - a2[v] * sn[v];
              o2[v] = a2[v] * cs[v] + a1[v] * sn[v];
            }
          } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) { o1[v] = a1[v]; o2[v] = a2[v]; }
          }
          store4<T>(C + static_cast<int64_t>(m) * g.ldc + c1, o1);
          store4<T>(C + static_cast<int64_t>(m) * g.ldc + c2, o2);
        } else {
          const int f = c1;  // gate row index == output column
          float o3[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            o1[v] = a1[v];
            o2[v] = a2[v];
            o3[v] = silu_f(a1[v]) * a2[v];
          }
          const int64_t off = static_cast<int64_t>(m) * g.ldc + f;
          store4<T>(static_cast<T*>(g.C) + off, o1);
          store4<T>(static_cast<T*>(g.C2) + off, o2);
          store4<T>(static_cast<T*>(g.C3) + off, o3);
        }
      }
    } else {
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int n = n0 + wn * WN + j * 16 + lg * 4;
        if (n >= g.N) continue;
        const f32x4 a = acc[i][j];
        float o[4] = {a[0], a[1], a[2], a[3]};
        const int64_t off = static_cast<int64_t>(m) * g.ldc + n;
        if constexpr (E == Epi::Store || E == Epi::StoreF32) {
          if (g.partial) {  // split-K: fp32 partial sums of this k-range
            float* p = g.partial + (static_cast<int64_t>(blockIdx.y) * g.M + m) * g.N + n;
            *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
            continue;
          }
        }
        if constexpr (E == Epi::Store) {
          store4<T>(static_cast<T*>(g.C) + off, o);
        } else if constexpr (E == Epi::StoreF32) {
          *reinterpret_cast<float4*>(static_cast<float*>(g.C) + off) = make_float4(o[0], o[1], o[2], o[3]);
        } else if constexpr (E == Epi::AccF32) {
          float4* p = reinterpret_cast<float4*>(static_cast<float*>(g.C) + off);
          float4 c = *p;
          *p = make_float4(c.x + o[0], c.y + o[1], c.z + o[2], c.w + o[3]);
        } else if constexpr (E == Epi::Resid) {
          float r[4];
          load4<T>(static_cast<const T*>(g.R) + static_cast<int64_t>(m) * g.ldr + n, r);
#pragma unroll
          for (int v = 0; v < 4; ++v) o[v] += r[v];
          store4<T>(static_cast<T*>(g.C) + off, o);
        } else if constexpr (E == Epi::SwigluBwd) {
          float G[4], U[4], dG[4], dU[4];
          const int64_t roff = static_cast<int64_t>(m) * g.ldr + n;
          load4<T>(static_cast<const T*>(g.R) + roff, G);
          load4<T>(static_cast<const T*>(g.R2) + roff, U);
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float sg = sigmoid_f(G[v]);
            dG[v] = o[v] * U[v] * sg * (1.0f + G[v] * (1.0f - sg));
            dU[v] = o[v] * G[v] * sg;
          }
          store4<T>(static_cast<T*>(g.C) + off, dG);
          store4<T>(static_cast<T*>(g.C2) + off, dU);
        }
      }
    }
    // one fragment row at a time: keeps the scheduler from pulling every
    // accumulator out of the AGPRs at once
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <typename T, int BM, int BN, int WM, int WN, GemmLayout LAY, Epi E>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const GemmArgs g, int ntm, int ntn) {
  constexpr bool AKC = (LAY != GemmLayout::TN);
  constexpr bool BKC = (LAY == GemmLayout::NT);
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int NT = NW * 64;
  constexpr int VE = 16 / sizeof(T);
  constexpr int BKE = kStageBytes / sizeof(T);
  constexpr int ROW = BKE + VE;
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int WGM = BM / WM;
  static_assert(!(E == Epi::Rope || E == Epi::SwigluFwd) || FN % 2 == 0, "pair epilogue needs even FN");

  __shared__ __attribute__((aligned(16))) T smem[2][(BM + BN) * ROW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wm = w % WGM, wn = w / WGM;

  int tm, tn;
  tile_coords(ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const T* __restrict__ A = static_cast<const T*>(g.A);
  const T* __restrict__ B = static_cast<const T*>(g.B);

  Loader<T, BM, NT, AKC> la;
  Loader<T, BN, NT, BKC> lb;
  auto amap = [&](int r) { const int m = m0 + r; return m < g.M ? m : -1; };
  auto bmap = [&](int r) { return ColMap<E, WN>::brow(r, n0, g, BN); };

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // split-K: blockIdx.y owns k in [kbeg, kend)
  const int kbeg = blockIdx.y * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + BKE - 1) / BKE : 0;
  la.load(A, g.lda, kbeg, kend, tid, amap);
  lb.load(B, g.ldb, kbeg, kend, tid, bmap);
  la.store(smem[0], tid);
  lb.store(smem[0] + BM * ROW, tid);
  __syncthreads();

  const int lr = lane % 16, lg = lane / 16;
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) {
      la.load(A, g.lda, kbeg + (kt + 1) * BKE, kend, tid, amap);
      lb.load(B, g.ldb, kbeg + (kt + 1) * BKE, kend, tid, bmap);
    }
    const T* As = smem[buf];
    const T* Bs = smem[buf] + BM * ROW;
#pragma unroll
    for (int s = 0; s < BKE / (4 * VE); ++s) {
      const int koff = s * 4 * VE + lg * VE;
      uint4 af[FM], bfr[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i)
        af[i] = *reinterpret_cast<const uint4*>(As + (wm * WM + i * 16 + lr) * ROW + koff);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[j] = *reinterpret_cast<const uint4*>(Bs + (wn * WN + j * 16 + lr) * ROW + koff);
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::run(acc[i][j], bfr[j], af[i]);
    }
    if (kt + 1 < nk) {
      la.store(smem[buf ^ 1], tid);
      lb.store(smem[buf ^ 1] + BM * ROW, tid);
    }
    __syncthreads();
  }

  if constexpr (sizeof(T) == 2 && kRowsEpi<E, WN>) {
    static_assert(NW * kPatchBytes<WN, E> <= sizeof(smem), "row epilogue patches");
    if (g.rows_epi) {  // the loop ended with a barrier: the stages are free
      epilogue_rows<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lane,
                                       reinterpret_cast<float*>(&smem[0][0]) + w * (kPatchBytes<WN, E> / 4));
      return;
    }
  }
  epilogue<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lr, lg, BN);
}

// ----------------------------------------------------------------------------
// bf16 kernel with global -> LDS direct loads (gfx950).
//
// Operands are copied from HBM straight into LDS by buffer loads (no
// staging registers, no VALU transposes): each wave instruction moves 1 KB,
// 16 B per lane, and lanes past a matrix edge (or past the k-range) read
// through an out-of-range buffer offset, which the hardware turns into
// zeros.  Per stage (64 k) the block holds, for each operand, either
//  - [row][k] (k-contiguous operands): 128-byte rows whose 16-byte slots are
//    XOR-swizzled by row, so 16 lanes reading one k-chunk of 16 consecutive
//    rows hit 16 distinct bank groups, or
//  - [k][row] (row-contiguous operands: the transposed side of NN / TN):
//    the tile exactly as it lies in HBM, slots swizzled by k, read with the
//    LDS transpose load (ds_read_b64_tr_b16), which hands each lane four
//    consecutive k of one row -- the MFMA operand layout -- directly.
// The 2-stage kernel below uses 64-k stages; the multi-stage and ping-pong
// kernels use the k-depth-generic variants further down.
namespace direct {

constexpr int kBK = 64;              // k per stage
constexpr uint32_t kOOB = 0x80000000u;  // an offset past every operand's extent

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// [k][row] slot swizzle: 16 lanes of one transpose read cover 4 consecutive k
// (the same two slots each); lanes 16 apart cover k 8 apart, and the 32 lanes
// of a pass must hit distinct banks.  256-byte k-rows (ROWS = 128) all start
// at bank 0: the map sends those 8 k-rows to 8 distinct slot pairs.  128-byte
// k-rows (ROWS = 64) alternate bank halves by k's parity: the 4 k-rows of
// each parity need distinct pairs among the 4 of a half, from k bits 1 and 3
// (the low bits of the 256-byte map, k & 3, repeat for k and k + 8: a two-way
// conflict on every transpose read, measured at 0.5 per access).
template <int ROWS>
__device__ __forceinline__ int kswz(int k) {
  static_assert(ROWS == 64 || ROWS >= 128, "8 or at least 16 slots per k-row");
  if constexpr (ROWS >= 128) return 2 * ((k & 3) | (((k >> 3) & 1) << 2));
  else return 2 * (((k >> 1) & 1) | (((k >> 3) & 1) << 1));
}
// [row][k] slot swizzle
__device__ __forceinline__ int rswz(int row) { return (row >> 1) & 7; }

// Loads of one operand tile (ROWS x 64 k) for one wave: JW instructions of
// 1 KB each.  KC: k-contiguous in HBM.
template <int ROWS, int NW, bool KC>
struct Direct {
  static constexpr int NI = ROWS / 8;  // 1-KB instructions per stage
  static_assert(NI % NW == 0, "tile rows must split evenly over the waves");
  static constexpr int JW = NI / NW;
  static constexpr int ROWB = ROWS * 2;  // [k][row]: bytes per k-row
  static constexpr int KPI = 1024 / ROWB;  // [k][row]: k-rows per instruction
  uint32_t base[JW];  // byte offset at k = 0, or kOOB
  int kl[JW];         // k of this lane's 16 bytes within the stage

  // KC: rowmap(r) = global row of tile row r or -1.  !KC: rows r0.. of `rows`.
  template <typename RowMap>
  __device__ __forceinline__ void init(int w, int lane, int64_t ld, int r0, int rows, RowMap rowmap) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int idx = j * NW + w;
      if constexpr (KC) {
        const int row = idx * 8 + lane / 8;
        const int ls = (lane % 8) ^ rswz(row);
        const int gr = rowmap(row);
        base[j] = gr >= 0 ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + ls * 8) * 2) : kOOB;
        kl[j] = ls * 8;
      } else {
        const int b = lane * 16;
        const int k = idx * KPI + b / ROWB;
        const int ls = ((b % ROWB) / 16) ^ kswz<ROWS>(k);
        const int r = r0 + ls * 8;
        base[j] = r < rows ? static_cast<uint32_t>((static_cast<int64_t>(k) * ld + r) * 2) : kOOB;
        kl[j] = k;
      }
    }
  }
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* region, int w, int k0, int kend,
                                        int64_t ld) {
    const uint32_t adv = KC ? static_cast<uint32_t>(k0) * 2u : static_cast<uint32_t>(k0 * ld * 2);
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const uint32_t off = (base[j] != kOOB && k0 + kl[j] < kend) ? base[j] + adv : kOOB;
      lds_dma16(rs, region + (j * NW + w) * 1024, off);
    }
  }
};

// One 16-row x 32-k MFMA operand fragment (rows rb.., k-chunk ks) for lane
// (lr = lane % 16, lg = lane / 16): 8 consecutive k of row rb + lr.
template <int ROWS, bool KC>
__device__ __forceinline__ uint4 frag(const char* region, int rb, int ks, int lr, int lg) {
  if constexpr (KC) {
    const int row = rb + lr;
    const int slot = (ks * 4 + lg) ^ rswz(row);
    return *reinterpret_cast<const uint4*>(region + row * 128 + slot * 16);
  } else {
    // lane s of a 16-lane group addresses 4 rows at one k; the transpose read
    // returns to lane i the 4 k (k0 .. k0+3) of row i
    const int row = rb + 4 * (lr & 3);
    const int slot = row >> 3, half = (row >> 2) & 1;
    uint32_t w[4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int k = ks * 32 + 8 * lg + 4 * t + (lr >> 2);
      const char* p = region + k * (ROWS * 2) + ((slot ^ kswz<ROWS>(k)) * 16) + half * 8;
      const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_v4i16*)(const_cast<char*>(p)));
      w[2 * t] = static_cast<uint16_t>(v[0]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[1])) << 16);
      w[2 * t + 1] = static_cast<uint16_t>(v[2]) | (static_cast<uint32_t>(static_cast<uint16_t>(v[3])) << 16);
    }
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
}

// ---- k-depth-generic variants for the multi-stage pipeline ----------------
// [row][k] tiles with BK*2-byte rows: 16-byte slots XOR-swizzled by row so
// that the 16 rows x one k-chunk of a fragment read cause no LDS bank
// conflict.  The choice is measured (SQ_LDS_BANK_CONFLICT on gfx950): XOR with
// (row >> 1) is conflict-free for 128- and 64-byte rows alike, while XOR with
// (row >> 2) on 64-byte rows, or no swizzle, costs 4-12 extra cycles a read.
template <int BK>
__device__ __forceinline__ int rswzk(int row) {
  if constexpr (BK == 64) return (row >> 1) & 7;
  else return (row >> 1) & 3;
}

// Loads of one operand tile (ROWS x BK) for one wave, 1-KB instructions.
template <int ROWS, int NW, bool KC, int BK>
struct DirectK {
  static constexpr int RB = BK * 2;                  // [row][k]: bytes per row
  static constexpr int RPI = 1024 / RB;              // [row][k]: rows per instruction
  static constexpr int ROWB = ROWS * 2;              // [k][row]: bytes per k-row
  static constexpr int KPI = 1024 / ROWB;            // [k][row]: k-rows per instruction
  static constexpr int NI = ROWS * BK * 2 / 1024;    // instructions per stage
  static_assert(NI % NW == 0, "tile must split evenly over the waves");
  static constexpr int JW = NI / NW;
  uint32_t base[JW];
  int kl[JW];

  template <typename RowMap>
  __device__ __forceinline__ void init(int w, int lane, int64_t ld, int r0, int rows, RowMap rowmap) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int idx = j * NW + w;
      if constexpr (KC) {
        const int row = idx * RPI + lane / (BK / 8);
        const int ls = (lane % (BK / 8)) ^ rswzk<BK>(row);
        const int gr = rowmap(row);
        base[j] = gr >= 0 ? static_cast<uint32_t>((static_cast<int64_t>(gr) * ld + ls * 8) * 2) : kOOB;
        kl[j] = ls * 8;
      } else {
        const int b = lane * 16;
        const int k = idx * KPI + b / ROWB;
        const int ls = ((b % ROWB) / 16) ^ kswz<ROWS>(k);
        const int r = r0 + ls * 8;
        base[j] = r < rows ? static_cast<uint32_t>((static_cast<int64_t>(k) * ld + r) * 2) : kOOB;
        kl[j] = k;
      }
    }
  }
  // k0 at or past kend: every lane out of range (the load still counts)
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* region, int w, int k0, int kend,
                                        int64_t ld) {
    const uint32_t adv = KC ? static_cast<uint32_t>(k0) * 2u : static_cast<uint32_t>(static_cast<int64_t>(k0) * ld * 2);
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const uint32_t off = (base[j] != kOOB && k0 + kl[j] < kend) ? base[j] + adv : kOOB;
      lds_dma16(rs, region + (j * NW + w) * 1024, off);
    }
  }
};

template <int ROWS, bool KC, int BK>
__device__ __forceinline__ uint4 fragk(const char* region, int rb, int ks, int lr, int lg) {
  if constexpr (KC) {
    const int row = rb + lr;
    const int slot = (ks * 4 + lg) ^ rswzk<BK>(row);
    return *reinterpret_cast<const uint4*>(region + row * (BK * 2) + slot * 16);
  } else {
    return frag<ROWS, false>(region, rb, ks, lr, lg);
  }
}

// s_waitcnt for vector memory only (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt and lgkmcnt left at their no-wait maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Workgroup barrier without a memory fence: the waits before it are explicit
// (a fenced barrier would also wait for the loads still in flight into the
// other stages).  The empty asm statements keep the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void bar() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Byte extent of a row-major operand with `rows` rows of `cols` used
// elements at stride ld.
inline int64_t extent(int64_t rows, int64_t cols, int64_t ld) { return ((rows - 1) * ld + cols) * 2; }

}  // namespace direct

template <typename T, int BM, int BN, int WM, int WN, GemmLayout LAY, Epi E>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_direct_kernel(const GemmArgs g, int ntm, int ntn, int a_bytes, int b_bytes) {
  static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
  constexpr bool AKC = (LAY != GemmLayout::TN);
  constexpr bool BKC = (LAY == GemmLayout::NT);
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int WGM = BM / WM;
  constexpr int STAGE = (BM + BN) * 128;
  static_assert(!(E == Epi::Rope || E == Epi::SwigluFwd) || FN % 2 == 0, "pair epilogue needs even FN");
  __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WGM, wn = w / WGM;
  int tm, tn;
  tile_coords(ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.B), 0, b_bytes, 0x00020000);
  direct::Direct<BM, NW, AKC> la;
  direct::Direct<BN, NW, BKC> lb;
  la.init(w, lane, g.lda, m0, g.M, [&](int r) { const int m = m0 + r; return m < g.M ? m : -1; });
  lb.init(w, lane, g.ldb, n0, g.N, [&](int r) { return ColMap<E, WN>::brow(r, n0, g, BN); });

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = blockIdx.y * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + direct::kBK - 1) / direct::kBK : 0;
  if (nk > 0) {
    la.issue(ra, smem, w, kbeg, kend, g.lda);
    lb.issue(rb, smem + BM * 128, w, kbeg, kend, g.ldb);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  const int lr = lane % 16, lg = lane / 16;
  for (int kt = 0; kt < nk; ++kt) {
    const char* As = smem + (kt & 1) * STAGE;
    const char* Bs = As + BM * 128;
    // All of this stage's fragment reads are issued before the next stage's
    // loads: the compiler orders a read of LDS after a load into LDS with a
    // full wait on that load, which would expose its latency here.
    uint4 af[2][FM], bfr[2][FN];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) af[ks][i] = direct::frag<BM, AKC>(As, wm * WM + i * 16, ks, lr, lg);
#pragma unroll
      for (int j = 0; j < FN; ++j) bfr[ks][j] = direct::frag<BN, BKC>(Bs, wn * WN + j * 16, ks, lr, lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (kt + 1 < nk) {
      char* nxt = smem + ((kt + 1) & 1) * STAGE;
      la.issue(ra, nxt, w, kbeg + (kt + 1) * direct::kBK, kend, g.lda);
      lb.issue(rb, nxt + BM * 128, w, kbeg + (kt + 1) * direct::kBK, kend, g.ldb);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::run(acc[i][j], bfr[ks][j], af[ks][i]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  if constexpr (kRowsEpi<E, WN>) {
    static_assert(NW * kPatchBytes<WN, E> <= sizeof(smem), "row epilogue patches");
    if (g.rows_epi) {  // the loop ended with a barrier: the stages are free
      epilogue_rows<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lane,
                                       reinterpret_cast<float*>(smem) + w * (kPatchBytes<WN, E> / 4));
      return;
    }
  }
  epilogue<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lr, lg, BN);
}

// Multi-stage variant: NS stages of BK k each (3 to 6; 4 in use), every
// stage in its own LDS array and the loop unrolled by NS so that each stage's
// address is a constant.  The loads of stage kt + NS - 1 are issued after the
// fragment reads of stage kt; the wait at the end of a stage lets the NS - 2
// newer stages stay in flight.
template <typename T, int BM, int BN, int WM, int WN, int BK, GemmLayout LAY, Epi E, int NS>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_pipe_kernel(const GemmArgs g, int ntm, int ntn, int a_bytes, int b_bytes) {
  static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
  static_assert(NS >= 3 && NS <= 6, "3 to 6 stages");
  constexpr bool AKC = (LAY != GemmLayout::TN);
  constexpr bool BKC = (LAY == GemmLayout::NT);
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int WGM = BM / WM;
  constexpr int KS = BK / 32;
  constexpr int ABYTES = BM * BK * 2;
  constexpr int STAGE = (BM + BN) * BK * 2;
  static_assert(!(E == Epi::Rope || E == Epi::SwigluFwd) || FN % 2 == 0, "pair epilogue needs even FN");
  __shared__ __attribute__((aligned(1024))) char S0[STAGE];
  __shared__ __attribute__((aligned(1024))) char S1[STAGE];
  __shared__ __attribute__((aligned(1024))) char S2[STAGE];
  __shared__ __attribute__((aligned(1024))) char S3[NS > 3 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char S4[NS > 4 ? STAGE : 16];
  __shared__ __attribute__((aligned(1024))) char S5[NS > 5 ? STAGE : 16];
  char* const stage[6] = {S0, S1, S2, S3, S4, S5};

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WGM, wn = w / WGM;
  int tm, tn;
  tile_coords(ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.B), 0, b_bytes, 0x00020000);
  direct::DirectK<BM, NW, AKC, BK> la;
  direct::DirectK<BN, NW, BKC, BK> lb;
  constexpr int JPS = direct::DirectK<BM, NW, AKC, BK>::JW + direct::DirectK<BN, NW, BKC, BK>::JW;
  la.init(w, lane, g.lda, m0, g.M, [&](int r) { const int m = m0 + r; return m < g.M ? m : -1; });
  lb.init(w, lane, g.ldb, n0, g.N, [&](int r) { return ColMap<E, WN>::brow(r, n0, g, BN); });

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = blockIdx.y * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  auto issue = [&](char* st, int kt) {
    la.issue(ra, st, w, kbeg + kt * BK, kend, g.lda);
    lb.issue(rb, st + ABYTES, w, kbeg + kt * BK, kend, g.ldb);
  };
  const int lr = lane % 16, lg = lane / 16;
  auto body = [&](int kt, const char* cur, char* nxt) {
    uint4 af[KS][FM], bfr[KS][FN];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int i = 0; i < FM; ++i) af[ks][i] = direct::fragk<BM, AKC, BK>(cur, wm * WM + i * 16, ks, lr, lg);
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[ks][j] = direct::fragk<BN, BKC, BK>(cur + ABYTES, wn * WN + j * 16, ks, lr, lg);
    }
    __builtin_amdgcn_sched_barrier(0);
    issue(nxt, kt + NS - 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::run(acc[i][j], bfr[ks][j], af[ks][i]);
    // stage kt + 1 complete; stages kt + 2 .. kt + NS - 1 may still be loading
    direct::wait_vm<(NS - 2) * JPS>();
    direct::bar();
  };

  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(stage[u], u);
    direct::wait_vm<(NS - 2) * JPS>();
    direct::bar();
    for (int kt = 0; kt < nk; kt += NS) {
      // fully unrolled: each stage is its own LDS array, so the compiler sees
      // that the fragment reads of one stage do not alias the loads of another
#pragma unroll
      for (int u = 0; u < NS; ++u)
        if (u == 0 || kt + u < nk) body(kt + u, stage[u], stage[(u + NS - 1) % NS]);
    }
    direct::wait_vm<0>();  // no load into LDS outlives the block
  }

  if constexpr (kRowsEpi<E, WN>) {
    // patches fill stage arrays one after another, none straddling two
    constexpr int PB = kPatchBytes<WN, E>, PER = STAGE / PB;
    static_assert(PER >= 1 && NS * PER >= NW, "row epilogue patches");
    if (g.rows_epi) {
      __syncthreads();  // every wave is done with the stages
      // (only the stage arrays that hold a patch are named)
      constexpr int KMAX = (NW - 1) / PER;
      const int k = w / PER;
      char* base = S0;
      if constexpr (KMAX >= 1) base = k == 1 ? S1 : base;
      if constexpr (KMAX >= 2) base = k == 2 ? S2 : base;
      if constexpr (KMAX >= 3) base = k == 3 ? S3 : base;
      if constexpr (KMAX >= 4) base = k == 4 ? S4 : base;
      if constexpr (KMAX >= 5) base = k == 5 ? S5 : base;
      epilogue_rows<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lane,
                                       reinterpret_cast<float*>(base + (w % PER) * PB));
      return;
    }
  }
  epilogue<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lr, lg, BN);
}

template <int STAGE, int NS>
struct PPStages {
  __attribute__((aligned(1024))) char s[NS][STAGE];
};

// Ping-pong variant: the 8 waves form two groups of four (one wave per SIMD
// in each), and the groups alternate between a memory phase (fragment reads
// of the next stage from LDS, loads of a later stage into LDS) and a compute
// phase (the MFMAs of that stage), so that each SIMD's matrix unit always has
// one wave feeding it while the other waits on memory.  A barrier separates
// the phases; group 1 runs one phase behind group 0.  One fragment set per
// wave suffices because a wave's own phases alternate.
template <typename T, int BM, int BN, int WM, int WN, int BK, GemmLayout LAY, Epi E, int NS>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_pp_kernel(const GemmArgs g, int ntm, int ntn, int a_bytes, int b_bytes) {
  static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
  static_assert(NS >= 3 && NS <= 6, "3 to 6 stages");
  constexpr bool AKC = (LAY != GemmLayout::TN);
  constexpr bool BKC = (LAY == GemmLayout::NT);
  constexpr int NW = (BM / WM) * (BN / WN);
  static_assert(NW == 8, "two groups of four waves");
  static_assert(NS * (BM + BN) * BK * 2 <= 160 * 1024, "stages within the 160 KB of LDS");
  constexpr int FM = WM / 16, FN = WN / 16;
  constexpr int WGM = BM / WM;
  constexpr int KS = BK / 32;
  constexpr int ABYTES = BM * BK * 2;
  constexpr int STAGE = (BM + BN) * BK * 2;
  static_assert(!(E == Epi::Rope || E == Epi::SwigluFwd) || FN % 2 == 0, "pair epilogue needs even FN");
  // exactly NS stages (at 256 x 256 x 32, five fill the 160 KB of LDS)
  __shared__ PPStages<STAGE, NS> smem;
  char* const stage[6] = {smem.s[0], smem.s[1], smem.s[2 % NS], smem.s[3 % NS], smem.s[4 % NS], smem.s[5 % NS]};

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WGM, wn = w / WGM;
  const bool late = w >= 4;  // group 1: one phase behind
  int tm, tn;
  tile_coords(ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.B), 0, b_bytes, 0x00020000);
  direct::DirectK<BM, NW, AKC, BK> la;
  direct::DirectK<BN, NW, BKC, BK> lb;
  constexpr int JPS = direct::DirectK<BM, NW, AKC, BK>::JW + direct::DirectK<BN, NW, BKC, BK>::JW;
  la.init(w, lane, g.lda, m0, g.M, [&](int r) { const int m = m0 + r; return m < g.M ? m : -1; });
  lb.init(w, lane, g.ldb, n0, g.N, [&](int r) { return ColMap<E, WN>::brow(r, n0, g, BN); });

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = blockIdx.y * g.kchunk;
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;
  auto issue = [&](char* st, int kt) {
    la.issue(ra, st, w, kbeg + kt * BK, kend, g.lda);
    lb.issue(rb, st + ABYTES, w, kbeg + kt * BK, kend, g.ldb);
  };
  const int lr = lane % 16, lg = lane / 16;
  uint4 af[KS][FM], bfr[KS][FN];
  // phase boundary: this wave's loads of the next stage anyone reads have
  // landed, its fragment reads are in registers; then the barrier
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    direct::wait_vm<(NS - 2) * JPS>();
    direct::bar();
    __builtin_amdgcn_sched_barrier(0);
  };
  // memory phase of stage kt: its fragments into registers, stage kt + NS - 1
  // into the buffer stage kt - 1 used (both groups have read it by now)
  auto mem = [&](int kt, const char* cur, char* nxt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int j = 0; j < FN; ++j)
        bfr[ks][j] = direct::fragk<BN, BKC, BK>(cur + ABYTES, wn * WN + j * 16, ks, lr, lg);
#pragma unroll
      for (int i = 0; i < FM; ++i) af[ks][i] = direct::fragk<BM, AKC, BK>(cur, wm * WM + i * 16, ks, lr, lg);
    }
    issue(nxt, kt + NS - 1);
  };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) Mfma<T>::run(acc[i][j], bfr[ks][j], af[ks][i]);
    __builtin_amdgcn_s_setprio(0);
  };

  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) issue(stage[u], u);
    sync();
    if (late) sync();
    for (int kt = 0; kt < nk; kt += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        if (u == 0 || kt + u < nk) {
          mem(kt + u, stage[u], stage[(u + NS - 1) % NS]);
          sync();
          compute();
          sync();
        }
      }
    }
    if (!late) sync();
    direct::wait_vm<0>();  // no load into LDS outlives the block
  }

  if constexpr (kRowsEpi<E, WN>) {
    // patches fill stage arrays one after another, none straddling two
    constexpr int PB = kPatchBytes<WN, E>, PER = STAGE / PB;
    static_assert(PER >= 1 && NS * PER >= NW, "row epilogue patches");
    if (g.rows_epi) {
      __syncthreads();  // every wave is done with the stages
      // (only the stage arrays that hold a patch are named)
      constexpr int KMAX = (NW - 1) / PER;
      const int k = w / PER;
      static_assert(KMAX < NS, "patches inside the stages");
      char* base = smem.s[0] + k * STAGE;
      epilogue_rows<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lane,
                                       reinterpret_cast<float*>(base + (w % PER) * PB));
      return;
    }
  }
  epilogue<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lr, lg, BN);
}

// Ping-pong variant for NT that reads B in whole lines.  A [row][k] operand
// staged 32 k at a time contributes 64 bytes per row and stage, half a
// 128-byte line, so every line reaches L2 as two requests (the transposed
// operand of NN and TN, 512 bytes per k-row, is read in whole lines anyway).
// Here B is staged 64 k at a time, one whole line per row, in NL = 3 buffers
// of 32 KB, and A keeps 32-k stages in NO = 4 buffers of 16 KB (160 KB in
// all).  Step kt (32 k) multiplies A stage kt with half kt % 2 of B line
// kt / 2: the same 32-k steps in the same order with the same fragments and
// MFMAs as gemm_pp_kernel, so the same bits.  Loads run ahead: step kt
// issues A stage kt + 3 (into the buffer of step kt - 1) and, on even steps,
// B line kt / 2 + 2 (into the buffer of line kt / 2 - 1, whose second half
// step kt - 1 read).  What step kt + 1 needs was issued at step kt - 2 or
// earlier, so after step kt's issues a wave may leave the loads of steps
// kt - 1 and kt in flight: two A stages and one B line.  The loop body covers
// 12 steps (the periods 4 and 2 x 3 of the two rings) so that every buffer
// index is a constant.  (The same ring for NN, with A in lines, needs more
// than 256 VGPRs and spills in its loop.)
template <typename T, GemmLayout LAY, Epi E>
__global__ void __launch_bounds__(512)
gemm_pl_kernel(const GemmArgs g, int ntm, int ntn, int a_bytes, int b_bytes) {
  static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
  static_assert(LAY == GemmLayout::NT, "B read in whole lines: both operands k-contiguous");
  constexpr int BM = 256, BN = 256, WM = 128, WN = 64, NW = 8;
  constexpr int FM = WM / 16, FN = WN / 16, WGM = BM / WM;
  constexpr int NO = 4, NL = 3;
  constexpr int OSZ = BM * 32 * 2, LSZ = BN * 64 * 2;
  static_assert(NO * OSZ + NL * LSZ <= 160 * 1024, "stages within the 160 KB of LDS");
  static_assert(!(E == Epi::Rope || E == Epi::SwigluFwd) || FN % 2 == 0, "pair epilogue needs even FN");
  struct Smem {
    __attribute__((aligned(1024))) char a[NO][OSZ];
    __attribute__((aligned(1024))) char b[NL][LSZ];
  };
  __shared__ Smem smem;

  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = w % WGM, wn = w / WGM;
  const bool late = w >= 4;  // group 1: one phase behind
  int tm, tn;
  tile_coords(ntm, ntn, &tm, &tn);
  const int m0 = tm * BM, n0 = tn * BN;

  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.A), 0, a_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(g.B), 0, b_bytes, 0x00020000);
  using LA = direct::DirectK<BM, NW, true, 32>;
  using LB = direct::DirectK<BN, NW, true, 64>;
  LA la;
  LB lb;
  constexpr int WAITN = 2 * LA::JW + LB::JW;
  la.init(w, lane, g.lda, m0, g.M, [&](int r) { const int m = m0 + r; return m < g.M ? m : -1; });
  lb.init(w, lane, g.ldb, n0, g.N, [&](int r) { return ColMap<E, WN>::brow(r, n0, g, BN); });

  f32x4 acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int kbeg = blockIdx.y * g.kchunk;  // a multiple of 64
  const int kend = min(g.K, kbeg + g.kchunk);
  const int nk = kend > kbeg ? (kend - kbeg + 31) / 32 : 0;
  auto issue_a = [&](char* st, int kt) { la.issue(ra, st, w, kbeg + kt * 32, kend, g.lda); };
  auto issue_b = [&](char* st, int line) { lb.issue(rb, st, w, kbeg + line * 64, kend, g.ldb); };
  const int lr = lane % 16, lg = lane / 16;
  uint4 af[FM], bfr[FN];
  auto sync = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    direct::wait_vm<WAITN>();
    direct::bar();
    __builtin_amdgcn_sched_barrier(0);
  };
  // memory phase of step kt = kt0 + u (kt0 a multiple of 12): fragments of A
  // stage u % NO and of half u % 2 of B line (u / 2) % NL, then the loads
  auto mem = [&](int kt, auto uc) {
    constexpr int u = decltype(uc)::value;
    const char* as = smem.a[u % NO];
    const char* bs = smem.b[(u / 2) % NL];
#pragma unroll
    for (int j = 0; j < FN; ++j) bfr[j] = direct::fragk<BN, true, 64>(bs, wn * WN + j * 16, u % 2, lr, lg);
#pragma unroll
    for (int i = 0; i < FM; ++i) af[i] = direct::fragk<BM, true, 32>(as, wm * WM + i * 16, 0, lr, lg);
    issue_a(smem.a[(u + 3) % NO], kt + 3);
    if constexpr (u % 2 == 0) issue_b(smem.b[(u / 2 + 2) % NL], kt / 2 + 2);
  };
  auto compute = [&]() {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) Mfma<T>::run(acc[i][j], bfr[j], af[i]);
    __builtin_amdgcn_s_setprio(0);
  };

  if (nk > 0) {
    // the issues of steps -4 .. -1
    issue_b(smem.b[0], 0);
    issue_a(smem.a[0], 0);
    issue_a(smem.a[1], 1);
    issue_b(smem.b[1], 1);
    issue_a(smem.a[2], 2);
    sync();
    if (late) sync();
    for (int kt = 0; kt < nk; kt += 12) {
      auto step = [&](auto uc) {
        constexpr int u = decltype(uc)::value;
        if (u == 0 || kt + u < nk) {
          mem(kt + u, uc);
          sync();
          compute();
          sync();
        }
      };
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
      step(std::integral_constant<int, 3>{});
      step(std::integral_constant<int, 4>{});
      step(std::integral_constant<int, 5>{});
      step(std::integral_constant<int, 6>{});
      step(std::integral_constant<int, 7>{});
      step(std::integral_constant<int, 8>{});
      step(std::integral_constant<int, 9>{});
      step(std::integral_constant<int, 10>{});
      step(std::integral_constant<int, 11>{});
    }
    if (!late) sync();
    direct::wait_vm<0>();  // no load into LDS outlives the block
  }

  if constexpr (kRowsEpi<E, WN>) {
    static_assert(NW * kPatchBytes<WN, E> <= sizeof(Smem), "row epilogue patches");
    if (g.rows_epi) {
      __syncthreads();  // every wave is done with the stages
      epilogue_rows<T, WM, WN, FM, FN, E>(
          g, acc, m0, n0, wm, wn, lane,
          reinterpret_cast<float*>(reinterpret_cast<char*>(&smem) + w * kPatchBytes<WN, E>));
      return;
    }
  }
  epilogue<T, WM, WN, FM, FN, E>(g, acc, m0, n0, wm, wn, lr, lg, BN);
}

// out[m, n] = sum over s (in order) of partial[s][m][n]; 4 columns per thread.
template <typename TO>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ partial, TO* __restrict__ out, int M, int N, int64_t ldo, int S) {
  const int64_t i = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t MN = static_cast<int64_t>(M) * N;
  if (i >= MN) return;
  float4 acc = *reinterpret_cast<const float4*>(partial + i);
  for (int s = 1; s < S; ++s) {
    const float4 p = *reinterpret_cast<const float4*>(partial + s * MN + i);
    acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w;
  }
  const int64_t m = i / N, n = i % N;
  const float o[4] = {acc.x, acc.y, acc.z, acc.w};
  if constexpr (sizeof(TO) == 2) store4<TO>(out + m * ldo + n, o);
  else *reinterpret_cast<float4*>(out + m * ldo + n) = acc;
}

// Whether the direct-load kernel can take this product: 16-byte aligned
// operands and rows, k in whole 8-element chunks, row-contiguous operands in
// whole 8-row chunks, and byte offsets that fit the 31-bit buffer range.
template <GemmLayout LAY, Epi E>
bool direct_ok(const GemmArgs& g, int64_t* a_bytes, int64_t* b_bytes) {
  constexpr bool AKC = (LAY != GemmLayout::TN);
  constexpr bool BKC = (LAY == GemmLayout::NT);
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.K % 8 || g.lda % 8 || g.ldb % 8) return false;
  if ((reinterpret_cast<uintptr_t>(g.A) | reinterpret_cast<uintptr_t>(g.B)) & 15u) return false;
  if ((!AKC && g.M % 8) || (!BKC && g.N % 8)) return false;
  const int ncols = (E == Epi::SwigluFwd) ? 2 * g.ffn : g.N;
  *a_bytes = AKC ? direct::extent(g.M, g.K, g.lda) : direct::extent(g.K, g.M, g.lda);
  *b_bytes = BKC ? direct::extent(ncols, g.K, g.ldb) : direct::extent(g.K, g.N, g.ldb);
  constexpr int64_t lim = (int64_t{1} << 31) - 1024;
  return *a_bytes > 0 && *b_bytes > 0 && *a_bytes < lim && *b_bytes < lim;
}

// KIND 0: register-staged kernel; 1: direct loads, 2 stages of 64 k; 2: direct
// loads, NS stages of BK k; 3: the same with two wave groups in ping-pong;
// 4: ping-pong with B in whole-line stages (NT, 256 x 256).
// S_req > 0: split K into S_req ranges (Store / StoreF32, with enough scratch)
// instead of the small-grid rule.
template <typename T, int BM, int BN, int WM, int WN, GemmLayout LAY, Epi E, int KIND = 0, int BK = 64, int NS = 4>
hipError_t launch(const GemmArgs& g_in, hipStream_t s, float* ws, size_t ws_bytes, int64_t a_bytes = 0,
                  int64_t b_bytes = 0, int S_req = 0) {
  // the RoPE column map pairs columns i and i + head_dim/2 inside one tile
  if constexpr (E == Epi::Rope)
    if (g_in.head_dim <= 0 || BN % g_in.head_dim != 0) return hipErrorInvalidValue;
  const int ntm = (g_in.M + BM - 1) / BM;
  const int ncols = (E == Epi::SwigluFwd) ? 2 * g_in.ffn : g_in.N;
  const int ntn = (ncols + BN - 1) / BN;
  if (ntm == 0 || ntn == 0) return hipSuccess;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  GemmArgs g = g_in;
  int S = 1;
  if constexpr (E == Epi::Store || E == Epi::StoreF32) {
    S = S_req > 0 ? S_req : splitk_factor(ntm * ntn, g.K);
    if (S > 1 && (!ws || static_cast<size_t>(S) * g.M * g.N * 4 > ws_bytes)) S = 1;
  }
  g.kchunk = S > 1 ? ((g.K + S - 1) / S + 63) / 64 * 64 : g.K;
  if (S > 1) {
    S = (g.K + g.kchunk - 1) / g.kchunk;
    g.partial = ws;
  }
  if constexpr (sizeof(T) == 2 && kRowsEpi<E, WN>) {
    // 16-byte row epilogue: every vector it touches must be whole and aligned
    auto a16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
    bool ok = S == 1 && g.ldc % 8 == 0 && a16(g.C) && ((E == Epi::SwigluFwd ? g.ffn : g.N) % 8 == 0);
    if constexpr (E == Epi::Resid || E == Epi::SwigluBwd) ok = ok && g.ldr % 8 == 0 && a16(g.R);
    if constexpr (E == Epi::SwigluBwd) ok = ok && a16(g.R2) && a16(g.C2);
    if constexpr (E == Epi::SwigluFwd) ok = ok && a16(g.C2) && a16(g.C3);
    // RoPE: 8 pair members inside one head half, whole rotated heads, float4 table reads
    if constexpr (E == Epi::Rope)
      ok = ok && g.head_dim % 16 == 0 && g.rope_cols % g.head_dim == 0 && a16(g.rope_cos) && a16(g.rope_sin);
    g.rows_epi = ok ? 1 : 0;
  }
  if constexpr (KIND == 4) {
    static_assert(BM == 256 && BN == 256 && WM == 128 && WN == 64, "whole-line ping-pong tile");
    hipLaunchKernelGGL((gemm_pl_kernel<T, LAY, E>), dim3(ntm * ntn, S), dim3(NT), 0, s, g, ntm, ntn,
                       static_cast<int>(a_bytes), static_cast<int>(b_bytes));
  } else if constexpr (KIND == 3) {
    static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
    hipLaunchKernelGGL((gemm_pp_kernel<T, BM, BN, WM, WN, BK, LAY, E, NS>), dim3(ntm * ntn, S), dim3(NT), 0, s, g,
                       ntm, ntn, static_cast<int>(a_bytes), static_cast<int>(b_bytes));
  } else if constexpr (KIND == 2) {
    static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
    hipLaunchKernelGGL((gemm_pipe_kernel<T, BM, BN, WM, WN, BK, LAY, E, NS>), dim3(ntm * ntn, S), dim3(NT), 0, s, g,
                       ntm, ntn, static_cast<int>(a_bytes), static_cast<int>(b_bytes));
  } else if constexpr (KIND == 1) {
    static_assert(sizeof(T) == 2, "direct loads take 16-bit operands");
    hipLaunchKernelGGL((gemm_direct_kernel<T, BM, BN, WM, WN, LAY, E>), dim3(ntm * ntn, S), dim3(NT), 0, s, g, ntm,
                       ntn, static_cast<int>(a_bytes), static_cast<int>(b_bytes));
  } else {
    hipLaunchKernelGGL((gemm_kernel<T, BM, BN, WM, WN, LAY, E>), dim3(ntm * ntn, S), dim3(NT), 0, s, g, ntm, ntn);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int64_t n4 = (static_cast<int64_t>(g.M) * g.N + 3) / 4;
  const dim3 rg(static_cast<unsigned>((n4 + 255) / 256));
  if constexpr (E == Epi::Store)
    hipLaunchKernelGGL(splitk_reduce_kernel<T>, rg, dim3(256), 0, s, ws, static_cast<T*>(g.C), g.M, g.N, g.ldc, S);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<float>, rg, dim3(256), 0, s, ws, static_cast<float*>(g.C), g.M, g.N,
                       g.ldc, S);
  return hipGetLastError();
}

// Tile configurations: 0 = 256x256 (8 waves of 128x64), 1 = 128x128 (register-staged kernel: 4 waves of
// 64x64; direct-load kernel: 8 waves of 32x64).
template <typename T, GemmLayout LAY, Epi E>
hipError_t dispatch_tiles(const GemmArgs& g, hipStream_t s, float* ws, size_t wsb) {
  const int cfg = gemm_tile_config(g.M, (E == Epi::SwigluFwd) ? 2 * g.ffn : g.N);
  if constexpr (sizeof(T) == 2) {
    int64_t ab = 0, bb = 0;
    if (direct_ok<LAY, E>(g, &ab, &bb)) {
      // Measured choices: grids of at least 160 256x256 tiles take the
      // ping-pong kernel (8 waves of 128x64, 4 stages of 32 k); smaller grids
      // take 128x128 tiles, 4 stages of 64 k with 8 waves of 32x64, or 2
      // stages when there are enough tiles to keep every CU busy without a
      // deep pipeline, or 128x64 tiles when even 128x128 ones would leave
      // half the CUs idle.
      // Five stages (the whole 160 KB of LDS) give the loads a fifth more
      // lead: 7-9 % on the forward products with 3-3.5 rounds of tiles over
      // the CUs at the 123B-shaped layer, 0-5 % on the input-gradient ones.
      // The weight-gradient kernel (both operands read transposed) already
      // needs 256 VGPRs at four stages and spills in its loop at five
      // (3.5x slower): four there.  256 x 128 tiles (8 waves of 64 x 64),
      // which would turn the 3.5 rounds of qkv_fwd's 896 tiles into 7, are
      // slower on every layer GEMM (0.35-0.44 of the peak against
      // 0.45-0.58): a 64 x 64 wave tile reads 8 fragments per 16 MFMAs.
      // NT takes the whole-line variant: same bits, 5-18 % faster on the
      // forward products at the 6.7B and 123B shapes (half the L2 read
      // requests; L2 misses unchanged).
      if (cfg == 0) {
        if constexpr (LAY == GemmLayout::TN) return launch<T, 256, 256, 128, 64, LAY, E, 3, 32>(g, s, ws, wsb, ab, bb);
        if constexpr (LAY == GemmLayout::NT) return launch<T, 256, 256, 128, 64, LAY, E, 4, 32>(g, s, ws, wsb, ab, bb);
        return launch<T, 256, 256, 128, 64, LAY, E, 3, 32, 5>(g, s, ws, wsb, ab, bb);
      }
      if constexpr (E == Epi::Store || E == Epi::StoreF32) {
        const int S = longk_split(g.M, g.N, g.K);
        if (S > 1 && ws && static_cast<size_t>(S) * g.M * g.N * 4 <= wsb)
          return launch<T, 256, 256, 128, 64, LAY, E, 3, 32>(g, s, ws, wsb, ab, bb, S);
      }
      const int ncols = (E == Epi::SwigluFwd) ? 2 * g.ffn : g.N;
      const long t128 = static_cast<long>((g.M + 127) / 128) * ((ncols + 127) / 128);
      // at most half the CUs' worth of 128x128 tiles: 128x64 tiles (8 waves
      // of 32x32) double the blocks instead of splitting K (the RoPE
      // epilogue needs whole heads in a tile: head_dim <= 64 there)
      if (t128 <= 128 && (E != Epi::Rope || 64 % g.head_dim == 0))
        return launch<T, 128, 64, 32, 32, LAY, E, 2, 64>(g, s, ws, wsb, ab, bb);
      if (t128 >= 320) {
        if constexpr (LAY == GemmLayout::TN) return launch<T, 128, 128, 64, 64, LAY, E, 2, 32>(g, s, ws, wsb, ab, bb);
        return launch<T, 128, 128, 32, 64, LAY, E, 1>(g, s, ws, wsb, ab, bb);
      }
      return launch<T, 128, 128, 32, 64, LAY, E, 2, 64>(g, s, ws, wsb, ab, bb);
    }
  }
  if (cfg == 0)
    return launch<T, 256, 256, 128, 64, LAY, E>(g, s, ws, wsb);
  return launch<T, 128, 128, 64, 64, LAY, E>(g, s, ws, wsb);
}

template <typename T>
hipError_t dispatch(GemmLayout lay, Epi epi, const GemmArgs& g, hipStream_t s, float* ws, size_t wsb) {
#define SF_CASE(L, E) \
  case Epi::E: return dispatch_tiles<T, GemmLayout::L, Epi::E>(g, s, ws, wsb);
  switch (lay) {
    case GemmLayout::NT:
      switch (epi) {
        SF_CASE(NT, Store) SF_CASE(NT, StoreF32) SF_CASE(NT, Resid) SF_CASE(NT, Rope) SF_CASE(NT, SwigluFwd)
        default: break;
      }
      break;
    case GemmLayout::NN:
      switch (epi) {
        SF_CASE(NN, Store) SF_CASE(NN, StoreF32) SF_CASE(NN, SwigluBwd)
        default: break;
      }
      break;
    case GemmLayout::TN:
      switch (epi) {
        SF_CASE(TN, Store) SF_CASE(TN, StoreF32) SF_CASE(TN, AccF32)
        default: break;
      }
      break;
  }
#undef SF_CASE
  return hipErrorInvalidValue;
}

}  // namespace

// Split-K scratch of sf_gemm_noalloc: a file-scope device array, so callers
// that cannot allocate (graph capture, serving loops) need no workspace.
// Each device holds its own copy from the library's load until the process
// ends.  Host code never uses the name itself (on the host it is only a
// stand-in): the device address comes from hipGetSymbolAddress, once per
// device, with that device current.
static __device__ __align__(256) unsigned char scratch[kGemmStaticScratchBytes];

hipError_t gemm_static_scratch(float** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = static_cast<float*>(addr[dev]);
  return hipSuccess;
}

int gemm_tile_config(int M, int N) {
  const long big = static_cast<long>((M + 255) / 256) * ((N + 255) / 256);
  return big >= 160 ? 0 : 1;
}

size_t gemm_splitk_bytes(int M, int N, int K) {
  const int SL = longk_split(M, N, K);
  if (SL > 1) return static_cast<size_t>(SL) * M * N * 4;
  const int bm = gemm_tile_config(M, N) == 0 ? 256 : 128;
  const int tiles = ((M + bm - 1) / bm) * ((N + bm - 1) / bm);
  const int S = splitk_factor(tiles, K);
  return S > 1 ? static_cast<size_t>(S) * M * N * 4 : 0;
}

hipError_t gemm(int dtype, GemmLayout layout, Epi epi, const GemmArgs& g, hipStream_t stream, float* ws,
                size_t ws_bytes) {
  return with_storage(dtype, [&](auto tag) {
    return dispatch<typename decltype(tag)::type>(layout, epi, g, stream, ws, ws_bytes);
  });
}

}  // namespace sf

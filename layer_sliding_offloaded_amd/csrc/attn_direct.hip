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
#include <math.h>

#include <type_traits>

#include "attention.h"
#include "common.h"

namespace sf {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// forward softmax: largest growth (log2 units) of a row's running maximum
// over its current shift before the shift is moved
constexpr float kLazy = 8.0f;
constexpr uint32_t kOOB = 0x80000000u;  // past every operand's extent

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// [row][64 d] blocks (128-byte rows): 16 lanes reading one 16-byte chunk of
// 16 consecutive rows hit 16 distinct bank groups.
__device__ __forceinline__ int rswz(int row) { return (row >> 1) & 7; }

// [row][d] tiles with whole D*2-byte rows, read two ways: 16-byte chunks of
// 16 consecutive rows (A operand along d), and transposed, where a 16-lane
// group reads 32 bytes of each of 4 consecutive rows and two groups cover 8
// consecutive rows.  The 16-byte slot XOR below is the one, among a dozen
// row masks measured with the LDS bank-conflict counter, under which both
// patterns run conflict-free on gfx950: XOR the slot with row mod 8 (d = 64)
// or twice that (d = 128).  An earlier mask that also folded in row bit 3
// gave every along-d read a two-way conflict (8 LDS cycles per 16-byte read
// instead of 4), although 16 consecutive lanes then hit 16 distinct slots.
template <int D>
__device__ __forceinline__ int tswz(int r) {
  if constexpr (D == 128) return (r & 7) << 1;
  else return r & 7;
}

template <typename T>
__device__ __forceinline__ uint4 pack8(const f32x4& a, const f32x4& b) {
  return make_uint4(pack_pair<T>(a[0], a[1]), pack_pair<T>(a[2], a[3]), pack_pair<T>(b[0], b[1]),
                    pack_pair<T>(b[2], b[3]));
}

// ---- loads of one 64-row x D tile into LDS --------------------------------
// kind 0: [row][d] as D/64 blocks of [64][128 B] (rswz);  kind 1: [row][d]
// with D*2-byte rows (tswz).  NW waves share the D/8 wave instructions.
template <int D, int NW, int KIND>
struct TileLoad {
  static constexpr int NI = D / 8;  // 64 rows * D * 2 B / 1 KB
  static_assert(NI % NW == 0, "");
  static constexpr int JW = NI / NW;
  uint32_t off[JW];  // byte offset of this lane's 16 B for the tile at row 0, or kOOB
  int row[JW];       // tile row this lane's 16 B belong to

  // base: byte offset of (row 0, column 0) of the operand; ld in elements
  __device__ __forceinline__ void init(int w, int lane, int64_t base, int64_t ld) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const int i = j * NW + w;
      int r, col;
      if constexpr (KIND == 0) {
        const int blk = i / 8;
        r = (i % 8) * 8 + lane / 8;
        col = blk * 64 + ((lane % 8) ^ rswz(r)) * 8;
      } else {
        constexpr int RB = D * 2;       // bytes per row
        constexpr int RPI = 1024 / RB;  // rows per instruction
        const int b = lane * 16;
        r = i * RPI + b / RB;
        col = (((b % RB) / 16) ^ tswz<D>(r)) * 8;
      }
      row[j] = r;
      off[j] = static_cast<uint32_t>(base + (static_cast<int64_t>(r) * ld + col) * 2);
    }
  }
  // rows r0 + row valid while < nrows; adv = byte advance for tile row r0
  __device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rs, char* lds, int w, int rows_left,
                                        uint32_t adv) {
#pragma unroll
    for (int j = 0; j < JW; ++j) {
      const uint32_t o = row[j] < rows_left ? off[j] + adv : kOOB;
      lds_dma16(rs, lds + (j * NW + w) * 1024, o);
    }
  }
};

// Fragment reads.  Every address splits into a lane part, fixed for the
// whole kernel and computed once (the ofs_* helpers), and a part that is a
// compile-time constant of the unrolled loops (16-row group, k-chunk), which
// the LDS instructions take as an immediate offset.  The swizzles depend on a
// row's low four bits only, and every fragment starts on a 16-row boundary,
// so the lane part is the same for every fragment of a tile.

// kind-0 tile ([row][64-d blocks]), A operand along d: rows rb + lr, d-chunk c
// (32 wide, lane gets d 32c + 8 lg ..).  Full offset = ofs + rb * 128.
__device__ __forceinline__ int ofs_d0(int c, int lr, int lg) {
  return (c >> 1) * 8192 + lr * 128 + ((((c & 1) * 4 + lg) ^ rswz(lr)) * 16);
}
// kind-1 tile ([row][D]), A operand along d.  Full offset = ofs + rb * D * 2.
template <int D>
__device__ __forceinline__ int ofs_d1(int c, int lr, int lg) {
  return lr * (D * 2) + (((c * 4 + lg) ^ tswz<D>(lr)) * 16);
}
// kind-1 tile read transposed: output rows d = db + (0..15), k = tile rows
// {32 j + 4 lg .. +3} (h = 0) and {32 j + 16 + 4 lg .. +3} (h = 1) -- the
// order in which a lane holds its probabilities (pack8 of fragments 2j,
// 2j+1).  Full offset = ofs + (32 j + 16 h) * D * 2.
template <int D>
__device__ __forceinline__ int ofs_t(int db, int lr, int lg) {
  const int rl = 4 * lg + (lr >> 2);  // row within the 16-row group this lane addresses
  const int d = db + 4 * (lr & 3);
  return rl * (D * 2) + (((d >> 3) ^ tswz<D>(rl)) * 16) + ((d >> 2) & 1) * 8;
}

__device__ __forceinline__ uint4 lds16(const char* t, int off) {
  return *reinterpret_cast<const uint4*>(t + off);
}
__device__ __forceinline__ uint4 lds_tr(const char* t, int off0, int off1) {
  const v4i16 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<char*>(t) + off0));
  const v4i16 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const_cast<char*>(t) + off1));
  const uint2 x = __builtin_bit_cast(uint2, a), y = __builtin_bit_cast(uint2, b);
  return make_uint4(x.x, x.y, y.x, y.y);
}
// transposed fragment j of a kind-1 tile for the lane offset o (from ofs_t)
template <int D>
__device__ __forceinline__ uint4 frag_t(const char* t, int o, int j) {
  return lds_tr(t, o + 32 * j * (D * 2), o + (32 * j + 16) * (D * 2));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
}

// ------------------------------------------------------------------ forward
// Block: 4 waves x 32 query rows of one (b, h); key tiles of 64.
template <typename T, int D>
__global__ void __launch_bounds__(256, 2)
attn_fwd_direct(const AttnArgs a, int qkv_bytes) {
  constexpr int BQ = 128, BKV = 64, NW = 4;
  constexpr int DC = D / 32;  // MFMA k-steps along d
  constexpr int FD = D / 16;
  constexpr int TB = BKV * D * 2;
  __shared__ __attribute__((aligned(1024))) char K0[TB];
  __shared__ __attribute__((aligned(1024))) char K1[TB];
  __shared__ __attribute__((aligned(1024))) char V0[TB];
  __shared__ __attribute__((aligned(1024))) char V1[TB];

  const int S = a.seq;
  const int nqt = (S + BQ - 1) / BQ;
  const int qt = nqt - 1 - blockIdx.x;  // longest rows first
  const int h = blockIdx.y, b = blockIdx.z;
  const int kvh = (h * a.n_kv) / a.n_heads;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int q0 = qt * BQ;
  const int qw = q0 + w * 32;

  const __amdgpu_buffer_rsrc_t rs = rsrc(a.qkv, qkv_bytes);
  TileLoad<D, NW, 0> lk;
  TileLoad<D, NW, 1> lv;
  lk.init(w, lane, (bs * ld + (a.n_heads + kvh) * D) * 2, ld);
  lv.init(w, lane, (bs * ld + (a.n_heads + a.n_kv + kvh) * D) * 2, ld);

  // Q fragments (B operand): lane supplies row lr, d-chunk lg of each 32
  const T* qbase = static_cast<const T*>(a.qkv) + bs * ld + h * D;
  uint4 qf[2][DC];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      const int q = qw + f * 16 + lr;
      qf[f][c] = (q < S) ? *reinterpret_cast<const uint4*>(qbase + static_cast<int64_t>(q) * ld + c * 32 + lg * 8)
                         : make_uint4(0, 0, 0, 0);
    }
  f32x4 oacc[2][FD];
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int d = 0; d < FD; ++d) oacc[f][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  // row sums of the (16-bit) probabilities, accumulated by MFMA against a
  // fragment of ones: every element of lacc[f] holds the sum for row lr
  f32x4 lacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
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
  auto scores = [&](const char* Kc, f32x4 (&sv)[2][4]) {
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int fk = 0; fk < 4; ++fk) sv[f][fk] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < DC; ++c) {
      uint4 kf[4];
#pragma unroll
      for (int fk = 0; fk < 4; ++fk) kf[fk] = lds16(Kc, ko[c] + fk * 16 * 128);
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int fk = 0; fk < 4; ++fk) Mfma<T>::run(sv[f][fk], kf[fk], qf[f][c]);
    }
  };
  auto active = [&](int kt) { return kt < nkv && kt * BKV <= qw + 31; };

  lk.issue(rs, K0, w, S, 0);
  lv.issue(rs, V0, w, S, 0);
  if (nkv > 1) lk.issue(rs, K1, w, S - BKV, static_cast<uint32_t>(BKV * ld * 2));
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x4 s[2][4];
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
    f32x4 sn[2][4];
    if (active(kt + 1)) scores(Knext, sn);
    // raw scores are scaled inside the exponent: p = 2^(s sc - m), with the
    // running maximum m kept in scaled units (sc > 0)
    if (kv0 + BKV - 1 > qw) {  // diagonal tile: mask keys after the row
#pragma unroll
      for (int f = 0; f < 2; ++f)
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
    float alpha[2];
#pragma unroll
    for (int f = 0; f < 2; ++f) {
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
      mrow[f] = mnew;
#pragma unroll
      for (int fk = 0; fk < 4; ++fk)
#pragma unroll
        for (int v = 0; v < 4; ++v) s[f][fk][v] = __builtin_amdgcn_exp2f(fmaf(s[f][fk][v], sc, -mnew));
    }
    if (!__all(alpha[0] == 1.0f && alpha[1] == 1.0f)) {
#pragma unroll
      for (int f = 0; f < 2; ++f) {
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
      const uint4 pf0 = pack8<T>(s[0][2 * j], s[0][2 * j + 1]);
      const uint4 pf1 = pack8<T>(s[1][2 * j], s[1][2 * j + 1]);
      Mfma<T>::run(lacc[0], ones, pf0);
      Mfma<T>::run(lacc[1], ones, pf1);
#pragma unroll
      for (int d = 0; d < FD; ++d) {
        const uint4 vf = frag_t<D>(Vc, vo[d], j);
        Mfma<T>::run(oacc[0][d], vf, pf0);
        Mfma<T>::run(oacc[1][d], vf, pf1);
      }
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
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
  for (int f = 0; f < 2; ++f) {
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

// Inverse RoPE on a lane's fragments: x[fd] (first half) pairs with
// x[fd + FD/2]; column = 16 fd + 4 lg + v; position pos.
template <int D>
__device__ __forceinline__ void rope_inv(f32x4 (&x)[D / 16], const AttnArgs& a, int pos, int lg) {
  constexpr int FD = D / 16;
#pragma unroll
  for (int fd = 0; fd < FD / 2; ++fd)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = fd * 16 + lg * 4 + v;
      const float c = a.rope_cos[static_cast<int64_t>(pos) * (D / 2) + i];
      const float sn = a.rope_sin[static_cast<int64_t>(pos) * (D / 2) + i];
      const float u1 = x[fd][v], u2 = x[fd + FD / 2][v];
      x[fd][v] = u1 * c + u2 * sn;
      x[fd + FD / 2][v] = u2 * c - u1 * sn;
    }
}

template <typename T>
__device__ __forceinline__ void store4v(T* p, const f32x4& v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_pair<T>(v[0], v[1]), pack_pair<T>(v[2], v[3]));
}

// ---------------------------------------------------------------- dK, dV
// Block: NWV waves x 16 KF keys of one (b, KV head); loops over every query head
// of the group and every 64-query tile at or after its first key.  Q and dO
// tiles (kind 1) serve both the score recompute (along d) and the dK / dV
// products (transposed, along the queries); log-sum-exp and D of the tile's
// queries are staged next to them.
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
  const int kvh = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lr = lane % 16, lg = lane / 16;
  const int64_t ld = a.ld_qkv;
  const int64_t bs = static_cast<int64_t>(b) * S;
  const int kv0 = blockIdx.x * BKV;  // block 0 holds the earliest keys, which see the most queries
  const int kvw = kv0 + w * KW;
  const int group = a.n_heads / a.n_kv;

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
  const int nit = group * per_head;

  // tile loaders: Q rows of head h at column h D, dO rows of head h
  TileLoad<D, NW, 1> lq, lo;
  lq.init(w, lane, (bs * ld) * 2, ld);
  lo.init(w, lane, (bs * a.ld_dout) * 2, a.ld_dout);
  auto issue = [&](int it, char* Qn, char* On, float* Ln) {
    const int h = kvh * group + it / per_head;
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
  const int nqt = (S + BQ - 1) / BQ;
  const int qt = nqt - 1 - blockIdx.x;
  const int h = blockIdx.y, b = blockIdx.z;
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

template <typename T, int D>
hipError_t run_bwd_direct(const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  const int64_t nt = static_cast<int64_t>(a.batch) * a.seq;
  const int64_t dout_bytes = ((nt - 1) * a.ld_dout + static_cast<int64_t>(a.n_heads) * D) * 2;
  const int64_t stat_bytes = static_cast<int64_t>(a.batch) * a.n_heads * a.seq * 4;
  // Block shapes (measured; every shape gives the same bits): dK/dV with 4
  // waves of 16 keys; dQ with 4 waves of 32 queries when that still makes
  // two blocks per CU, else 8 waves of 16.  (This file is compiled with the
  // MFMA accumulators held in VGPRs, which made the 4-wave dQ the fastest:
  // no AGPR-to-VGPR copies before the softmax arithmetic.)
  hipLaunchKernelGGL((attn_dkdv_direct<T, D, 1, 4>), dim3((a.seq + 63) / 64, a.n_kv, a.batch), dim3(256), 0, s, a,
                     static_cast<int>(qkv_bytes), static_cast<int>(dout_bytes), static_cast<int>(stat_bytes));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (static_cast<int64_t>((a.seq + 127) / 128) * a.n_heads * a.batch >= 512)
    hipLaunchKernelGGL((attn_dq_direct<T, D, 2, 4>), dim3((a.seq + 127) / 128, a.n_heads, a.batch), dim3(256), 0, s,
                       a, static_cast<int>(qkv_bytes));
  else
    hipLaunchKernelGGL((attn_dq_direct<T, D, 1, 8>), dim3((a.seq + 127) / 128, a.n_heads, a.batch), dim3(512), 0, s,
                       a, static_cast<int>(qkv_bytes));
  return hipGetLastError();
}

template <typename T, int D>
hipError_t run_fwd_direct(const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  dim3 grid((a.seq + 127) / 128, a.n_heads, a.batch);
  hipLaunchKernelGGL((attn_fwd_direct<T, D>), grid, dim3(256), 0, s, a, static_cast<int>(qkv_bytes));
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
    return a.head_dim == 64 ? run_fwd_direct<f16, 64>(a, qkv_bytes, s) : run_fwd_direct<f16, 128>(a, qkv_bytes, s);
  return a.head_dim == 64 ? run_fwd_direct<bf16, 64>(a, qkv_bytes, s) : run_fwd_direct<bf16, 128>(a, qkv_bytes, s);
}

hipError_t attention_bwd_direct(int dtype, const AttnArgs& a, int64_t qkv_bytes, hipStream_t s) {
  if (dtype == 2)
    return a.head_dim == 64 ? run_bwd_direct<f16, 64>(a, qkv_bytes, s) : run_bwd_direct<f16, 128>(a, qkv_bytes, s);
  return a.head_dim == 64 ? run_bwd_direct<bf16, 64>(a, qkv_bytes, s) : run_bwd_direct<bf16, 128>(a, qkv_bytes, s);
}

}  // namespace sf

// Device helpers shared by the direct-load attention kernels (gfx950): LDS
// tile layouts, global -> LDS tile loads, and MFMA fragment reads.
//
//  - tiles whose rows feed the MFMA A operand along d ([row][d], k = d) are
//    held as 64-column blocks of 128-byte rows, slots XOR-swizzled by row
//    (kind 0), or as whole D*2-byte rows with the swizzle tswz (kind 1);
//  - tiles that feed it along the sequence are read with the LDS transpose
//    load straight from their [row][d] layout (kind 1), with a slot swizzle
//    by row that keeps 32 lanes on distinct banks.
#pragma once

#include <math.h>

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

// Query head of grid column bx.  Workgroups go to the GPU's 8 XCDs (each
// with its own L2) round-robin by linear id, and grid rows are n_heads wide:
// when n_heads is a multiple of 8, XCD x gets the heads x * n_heads / 8 ..
// (x + 1) * n_heads / 8 - 1, consecutive heads that share KV heads (a whole
// GQA group at 96 query / 8 KV heads), so their K / V tiles stay in one L2.
__device__ __forceinline__ int xcd_head(int bx, int n_heads) {
  return n_heads % 8 ? bx : (bx % 8) * (n_heads / 8) + bx / 8;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, static_cast<int>(bytes), 0x00020000);
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

}  // namespace
}  // namespace sf

// Device helpers shared by the HIP kernels: bf16 and fp16 storage, 16-byte vectors,
// wavefront reductions and the gfx950 MFMA wrappers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sf {

// ----------------------------------------------------------------- bf16
// bf16 is stored as raw uint16_t.  Conversion to fp32 is exact; conversion
// from fp32 rounds to nearest, ties to even -- gfx950 does it in hardware
// (v_cvt_pk_bf16_f32, two values per instruction).
struct bf16 { uint16_t u; };

typedef __attribute__((ext_vector_type(2))) __bf16 hw_bf16x2;

__device__ __forceinline__ float bf2f(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  const hw_bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2bf(float f) { return static_cast<uint16_t>(pack2(f, 0.0f)); }

// ----------------------------------------------------------------- fp16
// IEEE binary16 storage (SF_F16), also raw uint16_t.  Conversion to fp32 is
// exact; from fp32 it rounds to nearest even (v_cvt_f16_f32 in the default
// round mode), and magnitudes past 65504 become infinities, which the
// engine's loss scaling detects in the weight gradients.
struct f16 { uint16_t u; };

typedef __attribute__((ext_vector_type(2))) _Float16 hw_f16x2;

__device__ __forceinline__ float h2f(uint16_t u) { return static_cast<float>(__builtin_bit_cast(_Float16, u)); }
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  const hw_f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f2h(float f) { return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f)); }

// Two values of a 16-bit storage type packed into one word (low = first).
template <typename T> __device__ __forceinline__ uint32_t pack_pair(float lo, float hi);
template <> __device__ __forceinline__ uint32_t pack_pair<bf16>(float lo, float hi) { return pack2(lo, hi); }
template <> __device__ __forceinline__ uint32_t pack_pair<f16>(float lo, float hi) { return pack2h(lo, hi); }

// Element traits: the storage type of activations and weights.
template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPerVec = 4;  // elements per 16-byte vector
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
  static __device__ __forceinline__ void store(float* p, size_t i, float v) { p[i] = v; }
  // unpack / pack one 16-byte vector
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <> struct Elem<bf16> {
  static constexpr int kPerVec = 8;
  static __device__ __forceinline__ float load(const bf16* p, size_t i) { return bf2f(p[i].u); }
  static __device__ __forceinline__ void store(bf16* p, size_t i, float v) { p[i].u = f2bf(v); }
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(pack2(f[0], f[1]), pack2(f[2], f[3]), pack2(f[4], f[5]), pack2(f[6], f[7]));
  }
};

template <> struct Elem<f16> {
  static constexpr int kPerVec = 8;
  static __device__ __forceinline__ float load(const f16* p, size_t i) { return h2f(p[i].u); }
  static __device__ __forceinline__ void store(f16* p, size_t i, float v) { p[i].u = f2h(v); }
  static __device__ __forceinline__ void unpack(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = h2f(static_cast<uint16_t>(w[i] & 0xFFFFu));
      f[2 * i + 1] = h2f(static_cast<uint16_t>(w[i] >> 16));
    }
  }
  static __device__ __forceinline__ uint4 pack(const float* f) {
    return make_uint4(pack2h(f[0], f[1]), pack2h(f[2], f[3]), pack2h(f[4], f[5]), pack2h(f[6], f[7]));
  }
};

// The bit pattern of 1.0 in a 16-bit storage type.
template <typename T> struct One16;
template <> struct One16<bf16> { static constexpr uint32_t kBits = 0x3F80u; };
template <> struct One16<f16> { static constexpr uint32_t kBits = 0x3C00u; };

// Storage dtype code (0 fp32, 1 bf16, 2 fp16) -> type, for host dispatch:
// f(Tag<T>{}) with T = float, bf16 or f16.
template <typename T> struct Tag { using type = T; };
template <typename F>
hipError_t with_storage(int dtype, F&& f) {
  if (dtype == 1) return f(Tag<bf16>{});
  if (dtype == 2) return f(Tag<f16>{});
  if (dtype == 0) return f(Tag<float>{});
  return hipErrorInvalidValue;
}

// ----------------------------------------------------------------- reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// ----------------------------------------------------------------- MFMA
// 16x16 output tiles.  For D = mfma(A, B): lane l supplies row (l % 16) of
// A and column (l % 16) of B, each as its k-chunk (l / 16); lane l receives
// D[4*(l/16) + i][l % 16], i = 0..3.  A "k-chunk" is 16 bytes of one row:
// 8 bf16 (one 16x16x32 MFMA) or 4 fp32 (four 16x16x4 MFMAs, one per
// element, so that 16 consecutive k are covered either way per 4 chunks).
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4;

template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int kChunkK = 8;   // k per lane-chunk
  static __device__ __forceinline__ void run(f32x4& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                  __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
};
template <> struct Mfma<f16> {
  static constexpr int kChunkK = 8;
  static __device__ __forceinline__ void run(f32x4& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b),
                                                 acc, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int kChunkK = 4;
  static __device__ __forceinline__ void run(f32x4& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
  }
};

// Transpose an 8x8 block of 16-bit values held as 8 row vectors (v[r] = row
// r, 8 columns) into 8 column vectors (out[c] = column c, 8 rows).
__device__ __forceinline__ void transpose8x8_b16(const uint4* v, uint4* out) {
  uint32_t w[8][4];
#pragma unroll
  for (int r = 0; r < 8; ++r) { w[r][0] = v[r].x; w[r][1] = v[r].y; w[r][2] = v[r].z; w[r][3] = v[r].w; }
  uint32_t o[8][4];
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      // output column c, rows 2p and 2p+1
      const uint32_t lo = (c & 1) ? (w[2 * p][c >> 1] >> 16) : (w[2 * p][c >> 1] & 0xFFFFu);
      const uint32_t hi = (c & 1) ? (w[2 * p + 1][c >> 1] & 0xFFFF0000u) : (w[2 * p + 1][c >> 1] << 16);
      o[c][p] = lo | hi;
    }
  }
#pragma unroll
  for (int c = 0; c < 8; ++c) out[c] = make_uint4(o[c][0], o[c][1], o[c][2], o[c][3]);
}

// Transpose a 4x4 block of 32-bit values (rows -> columns).
__device__ __forceinline__ void transpose4x4_b32(const uint4* v, uint4* out) {
  out[0] = make_uint4(v[0].x, v[1].x, v[2].x, v[3].x);
  out[1] = make_uint4(v[0].y, v[1].y, v[2].y, v[3].y);
  out[2] = make_uint4(v[0].z, v[1].z, v[2].z, v[3].z);
  out[3] = make_uint4(v[0].w, v[1].w, v[2].w, v[3].w);
}

template <typename T> struct Transpose;
template <> struct Transpose<bf16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void run(const uint4* v, uint4* o) { transpose8x8_b16(v, o); }
};
template <> struct Transpose<f16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void run(const uint4* v, uint4* o) { transpose8x8_b16(v, o); }
};
template <> struct Transpose<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void run(const uint4* v, uint4* o) { transpose4x4_b32(v, o); }
};

// Store 4 consecutive values in the storage dtype (8 or 16 bytes).
template <typename T>
__device__ __forceinline__ void store4(T* p, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_pair<T>(v[0], v[1]), pack_pair<T>(v[2], v[3]));
  } else {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

// Wave-wide global -> LDS copies by the buffer unit (buffer_load ... with the
// lds flag): lane l's 16 (or 4) bytes at buffer offset voff land at LDS byte
// address lds + 16 l (+ 4 l).  Issued as inline assembly so that the
// compiler does not track them as LDS writes: its wait-count pass cannot tell
// the stages of a multi-stage pipeline apart across loop iterations and makes
// LDS reads wait for every load in flight (vmcnt(0)), draining the pipeline.
// Callers order their LDS reads after these loads themselves (s_waitcnt on
// vmcnt, then a barrier).  M0 carries the LDS address; the kernels that use
// these helpers use M0 for nothing else.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, const void* lds, uint32_t voff) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(const_cast<void*>(lds))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %2, 0 offen lds"
               :: "v"(voff), "s"(m0), "s"(rs) : "memory");
}
__device__ __forceinline__ void lds_dma4(__amdgpu_buffer_rsrc_t rs, const void* lds, uint32_t voff) {
  const uint32_t m0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) void*)(const_cast<void*>(lds))));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dword %0, %2, 0 offen lds"
               :: "v"(voff), "s"(m0), "s"(rs) : "memory");
}

}  // namespace sf

// Host interface of the MFMA GEMM: C[M, N] = sum_k A[m, k] B[n, k] with a
// fused epilogue.  Operand layouts (row-major storage):
//   NT : A is [M, K] (lda), B is [N, K] (ldb)   -- forward  y = x W^T
//   NN : A is [M, K] (lda), B is [K, N] (ldb)   -- dX       dX = dY W
//   TN : A is [K, M] (lda), B is [K, N] (ldb)   -- dW       dW = dY^T X
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sf {

enum class GemmLayout : int { NT = 0, NN = 1, TN = 2 };

enum class Epi : int {
  Store = 0,     // C (storage dtype) = acc
  StoreF32 = 1,  // C (fp32) = acc
  AccF32 = 2,    // C (fp32) += acc
  Resid = 3,     // C (storage) = R + acc
  Rope = 4,      // C (storage) = acc with RoPE on columns < rope_cols
  SwigluFwd = 5, // B = [Wg; Wu] ([2F, K]); C = G, C2 = U, C3 = silu(G) * U, all [M, F]
  SwigluBwd = 6  // acc = da; R = G, R2 = U; C = dG, C2 = dU (ldc for both)
};

struct GemmArgs {
  const void* A = nullptr;
  int64_t lda = 0;
  const void* B = nullptr;
  int64_t ldb = 0;
  void* C = nullptr;
  int64_t ldc = 0;
  int M = 0, N = 0, K = 0;
  const void* R = nullptr;   // residual / G
  const void* R2 = nullptr;  // U
  int64_t ldr = 0;           // row stride of R and R2
  void* C2 = nullptr;
  void* C3 = nullptr;
  const float* rope_cos = nullptr;  // [seq, head_dim/2]
  const float* rope_sin = nullptr;
  int seq = 1, head_dim = 64, rope_cols = 0;
  int ffn = 0;                      // SwigluFwd: F (B rows F.. are Wu)
  // set by gemm(): k-range per grid row and split-K partial buffer
  int kchunk = 0;
  float* partial = nullptr;
  int rows_epi = 0;  // set by gemm(): outputs take the 16-byte row epilogue
};

// dtype: 0 = fp32 storage, 1 = bf16 storage (inputs A, B and storage outputs).
// ws/ws_bytes: optional scratch for split-K (Store / StoreF32 epilogues with
// few output tiles): fp32 partial sums per k-range, then a fixed-order
// reduction -- deterministic.  Without enough scratch the GEMM runs unsplit.
hipError_t gemm(int dtype, GemmLayout layout, Epi epi, const GemmArgs& g, hipStream_t stream,
                float* ws = nullptr, size_t ws_bytes = 0);

// Scratch bytes gemm() uses for split-K at these sizes (0: no split).
size_t gemm_splitk_bytes(int M, int N, int K);

// Which tile configuration gemm() picks for (M, N); for measurement.
int gemm_tile_config(int M, int N);

// Bytes of the static split-K scratch (64 MiB) and its device address on the
// current device (looked up once per device).  Shared by every call on that
// device: calls that overlap in time race on it.
constexpr size_t kGemmStaticScratchBytes = size_t{64} << 20;
hipError_t gemm_static_scratch(float** ptr);

}  // namespace sf

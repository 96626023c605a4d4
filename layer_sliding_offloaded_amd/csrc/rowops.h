// Host interface of the row-wise kernels (dtype: 0 = fp32, 1 = bf16 storage).
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sf {

// y = RMSNorm(x; g) over rows of H; r[row] = (mean x^2 + eps)^-1/2.
hipError_t rmsnorm_fwd(int dtype, const void* x, const void* g, void* y, float* r, int rows, int H, float eps,
                       hipStream_t s);

// dx = resid + r (dn - n mean(dn n)) with n = xin r, dn = dout g (resid may be
// null); dg[j] = sum_t dout[t, j] n[t, j] via partial[nchunks][H] (fp32).
hipError_t rmsnorm_bwd(int dtype, const void* dout, const void* xin, const float* r, const void* g,
                       const void* resid, void* dx, float* partial, int nchunks, float* dg, int rows, int H,
                       hipStream_t s);

hipError_t embed_fwd(int dtype, const void* E, const int32_t* ids, void* x0, int rows, int H, int V,
                     hipStream_t s);
hipError_t embed_bwd(int dtype, const void* dx0, const int32_t* ids, float* dE, int rows, int H, int V,
                     hipStream_t s);
hipError_t fill_f32(float* p, int64_t n, float v, hipStream_t s);

hipError_t ce_rows(int dtype, const float* logits, const int32_t* ids, void* dlogits, float* loss_rows, int t0,
                   int R, int V, int S, float inv_n, hipStream_t s);
hipError_t loss_reduce(const float* loss_rows, float* loss, int rows, float inv_n, hipStream_t s);

// Number of row chunks used for the gain-gradient partial sums.
constexpr int kGainChunks = 64;

}  // namespace sf

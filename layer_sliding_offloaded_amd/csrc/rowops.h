// Host interface of the row-wise kernels (dtype: 0 = fp32, 1 = bf16, 2 = fp16 storage).
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
// dst[i] = src[i] for n fp32 words by plain vector stores (dst may be pinned
// host memory: the words cross the host link without a copy engine).
hipError_t copy_f32(float* dst, const float* src, int n, hipStream_t s);

// Device Adam over n fp32 elements with precomputed coefficients
// (o = 1 - b, ib = 1 / bias correction); out receives the storage-dtype copy.
// The gradient enters as g * gscale (the inverse loss scale; 1 leaves it
// exact); with skip non-null and *skip != 0 at run time nothing is updated.
hipError_t adam_device(int dtype, float* p, float* m, float* v, const float* g, void* out, int64_t n, float b1,
                       float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                       float gscale = 1.0f, const int32_t* skip = nullptr);

// Sparse embedding gradient: for the n distinct valid ids (n -> *count, in
// order of first occurrence), out_ids[s] is the id and out_rows[s] ([H] fp32)
// the sum of dx0 over its tokens in increasing t -- the nonzero rows of
// embed_bwd, bit for bit.  scratch: 2 * rows int32.  out_ids and out_rows
// need room for `rows` entries.
hipError_t embed_bwd_sparse(int dtype, const void* dx0, const int32_t* ids, int32_t* out_ids, float* out_rows,
                            int32_t* count, int32_t* scratch, int rows, int H, int V, hipStream_t s);

// Device Adam of an embedding [V, H] from its sparse gradient (as produced by
// embed_bwd_sparse: out_ids / rows for the first *count slots, at most
// max_rows): map (V int32 of scratch) is rebuilt, rows no token touched take
// a zero gradient.  Bitwise equal to adam_device over the dense gradient.
hipError_t embed_adam_sparse(int dtype, float* p, float* m, float* v, const float* rows, const int32_t* out_ids,
                             const int32_t* count, int32_t* map, int max_rows, void* out, int V, int H, float b1,
                             float b2, float o1, float o2, float ib1, float ib2, float lr, float eps, hipStream_t s,
                             float gscale = 1.0f, const int32_t* skip = nullptr);

hipError_t ce_rows(int dtype, const float* logits, const int32_t* ids, void* dlogits, float* loss_rows, int t0,
                   int R, int V, int S, float inv_n, hipStream_t s);
hipError_t loss_reduce(const float* loss_rows, float* loss, int rows, float inv_n, hipStream_t s);

// Loss scaling (fp16 storage): *flag = 1 when any of the n fp32 values at g
// (16-byte aligned) is infinite or NaN (never cleared here); y = sc x in the
// storage dtype (n % 8 == 0); n 32-bit words copied by plain stores (dst may
// be pinned host memory); *p = v.
hipError_t nonfinite_flag(const float* g, int64_t n, int32_t* flag, hipStream_t s);
// The same over several fp32 ranges of one buffer (element offsets and
// counts), and over n values of the storage dtype.
constexpr int kMaxSegs = 9;
struct FloatSegs {
  int64_t off[kMaxSegs], n[kMaxSegs];
  int count;
};
hipError_t nonfinite_flag_segs(const float* base, const FloatSegs& segs, int32_t* flag, hipStream_t s);
hipError_t nonfinite_storage(int dtype, const void* x, int64_t n, int32_t* flag, hipStream_t s);
hipError_t scale_storage(int dtype, const void* x, void* y, int64_t n, float sc, hipStream_t s);
hipError_t copy_words(uint32_t* dst, const uint32_t* src, int n, hipStream_t s);
hipError_t set_word(int32_t* p, int32_t v, hipStream_t s);

// Number of row chunks used for the gain-gradient partial sums.
constexpr int kGainChunks = 512;

}  // namespace sf

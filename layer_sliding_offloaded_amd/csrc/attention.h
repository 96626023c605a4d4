// Host interface of the causal flash-attention kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace sf {

struct AttnArgs {
  const void* qkv = nullptr;  // [T, ld_qkv]: q' | k' | v  (storage dtype)
  int64_t ld_qkv = 0;
  void* out = nullptr;        // A = [T, ld_out], head h at column h d
  int64_t ld_out = 0;
  const void* dout = nullptr; // dA, same layout as out (backward)
  int64_t ld_dout = 0;
  void* dqkv = nullptr;       // [T, ld_dqkv]: dq | dk | dv (backward output)
  int64_t ld_dqkv = 0;
  float* lse = nullptr;       // [B, n_heads, S] base-2 log-sum-exp of scaled scores
  float* dsum = nullptr;      // [B, n_heads, S] rowsum(dA * A)   (backward scratch)
  const float* rope_cos = nullptr;  // [S, d/2] (backward: inverse rotation)
  const float* rope_sin = nullptr;
  int batch = 0, seq = 0, n_heads = 0, n_kv = 0, head_dim = 0;
  float scale = 0.f;          // 1 / sqrt(d)
  // dK/dV of the 16-bit kernels: query-head shares per KV head (attn_kv_split)
  // and, when > 1, the fp32 partial sums' buffer (attn_kv_partial_bytes)
  int kv_split = 1;
  float* dkv_partial = nullptr;
};

// Query-head shares of the dK/dV work units.  A unit is (64-key block, share
// of the GQA group, KV head, batch); with few KV heads and batches (the
// 123B-shaped GQA layer: 8 KV heads, batch 1) the whole-group units are few
// for the GPU and their lengths differ by the sequence length over 64 (the
// earliest keys see every query): the group is then split into the smallest
// share count, dividing the group, that gives at least 2048 units (about
// four per block slot of a 256-CU GPU at two blocks per CU).
inline int attn_kv_split(int batch, int seq, int n_heads, int n_kv) {
  if (n_kv <= 0 || n_heads % n_kv) return 1;
  const int group = n_heads / n_kv;
  const int64_t units = static_cast<int64_t>((seq + 63) / 64) * n_kv * batch;
  for (int c = 1; c <= group; ++c)
    if (group % c == 0 && units * c >= 2048) return c;
  return group;
}
// Bytes of the fp32 partial dK/dV sums for `split` shares (0 when 1).
inline int64_t attn_kv_partial_bytes(int split, int batch, int seq, int n_kv, int head_dim) {
  return split > 1 ? static_cast<int64_t>(split) * 2 * batch * seq * n_kv * head_dim * 4 : 0;
}

hipError_t attention_fwd(int dtype, const AttnArgs& a, hipStream_t s);
hipError_t attention_bwd(int dtype, const AttnArgs& a, hipStream_t s);

// 16-bit (bf16 or fp16, dtype 1 or 2) kernels with direct global -> LDS
// loads (attn_direct.hip).  ok(): d in {64, 128}, 16-byte aligned rows, q'k'v
// buffer under 2 GiB (its byte extent is returned for the buffer-load bounds).
bool attention_direct_ok(const AttnArgs& a, int64_t* qkv_bytes);
hipError_t attention_fwd_direct(int dtype, const AttnArgs& a, int64_t qkv_bytes, hipStream_t s);
// dK/dV and dQ; needs dsum (rowsum(dA * A)) already computed
hipError_t attention_bwd_direct(int dtype, const AttnArgs& a, int64_t qkv_bytes, hipStream_t s);

}  // namespace sf

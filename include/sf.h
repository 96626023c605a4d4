/*
 * sf.h -- C ABI of the layer-sliding fine-tuning step for MI355X (gfx950).
 *
 * The method: "An Efficient Heterogeneous Co-Design for Fine-Tuning on a
 * Single GPU" (SlideFormer), as summarised on gist.science (de/es/fr).  The
 * device holds only a small window of decoder layers; each layer's weights
 * stream in from pinned host memory, its gradients stream out to host memory
 * and a host-side Adam updates it while the device moves on to the next layer
 * (de §2A "Leichtgewichtige asynchrone Engine", es §2A "Arquitectura de
 * Deslizamiento de Capas", fr §2A).  Device memory is a fixed queue of
 * pre-allocated cache units, each sized for exactly one layer's parameters and
 * gradients (de §2B, es §2B "Cola de Cache GPU Pre-asignada", fr §2B).
 *
 * Conventions for every entry point:
 *   - Return value: sf_status; 0 = SF_OK, negative = error.  No C++
 *     exception crosses the ABI.  sf_last_error() returns a thread-local
 *     message describing the last failure on the calling thread.
 *   - Ownership: the caller owns every device buffer and every pinned host
 *     buffer passed in; the library borrows raw pointers and never frees
 *     them.  The library owns only the objects its *_create calls make
 *     (contexts, engines, their side streams, events and host threads) and
 *     releases them in the matching *_destroy.
 *   - No entry point allocates device memory.  Buffers are carved out of
 *     caller-provided regions whose sizes come from sf_layer_layout().
 *   - Arguments are validated before any device work is enqueued; a
 *     validation failure leaves every buffer untouched.
 *   - Streams are passed as sf_stream (a hipStream_t); NULL is the default
 *     stream.  Device work is enqueued asynchronously on that stream unless
 *     the entry point says otherwise.
 *   - Device pointers must be 16-byte aligned.  Row-major layouts throughout.
 *   - Storage dtype: SF_F32 (everything fp32), SF_BF16 (parameters and
 *     activations bf16, accumulation and statistics fp32) or SF_F16 (the same
 *     with IEEE fp16, whose narrow range the sliding engine covers with
 *     dynamic loss scaling; de/es/fr §2B name the FP32 -> BF16/FP16
 *     conversion).  Weight gradients are always fp32.
 */
#ifndef SF_H
#define SF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sf_status;
enum {
  SF_OK = 0,
  SF_ERR_ARG = -1,          /* bad argument (NULL, size, inconsistent shape) */
  SF_ERR_UNSUPPORTED = -2,  /* shape outside what the kernels implement     */
  SF_ERR_ALIGN = -3,        /* pointer not 16-byte aligned                   */
  SF_ERR_NOT_PINNED = -4,   /* host pointer is not page-locked host memory   */
  SF_ERR_POOL = -5,         /* caller-provided region too small              */
  SF_ERR_HIP = -6,          /* a HIP runtime call failed                     */
  SF_ERR_STATE = -7,        /* object is in a sticky error state             */
  SF_ERR_NO_DEVICE = -8     /* no usable gfx950 device                       */
};

typedef enum { SF_F32 = 0, SF_BF16 = 1, SF_F16 = 2 } sf_dtype;

typedef void* sf_stream; /* hipStream_t */

/*
 * Shape of one Llama-style decoder block and its batch.  The pages name the
 * Llama, Qwen and Mistral families (de §5, es §3) and the fused RoPE,
 * RMSNorm and SwiGLU ops (de §2C, es §2C, fr §2C); the block is:
 *   xn = RMSNorm(x; g1); q,k,v = xn Wq^T, xn Wk^T, xn Wv^T; q',k' = RoPE;
 *   A = causal softmax(q'k'^T/sqrt(d)) v (GQA: query head h reads KV head
 *   floor(h*n_kv/n_h)); h = x + A Wo^T; hn = RMSNorm(h; g2);
 *   a = silu(hn Wg^T) * (hn Wu^T); y = h + a Wd^T.
 * Supported: head_dim in {64, 128}; n_heads % n_kv_heads == 0; hidden, ffn
 * and vocab multiples of 8; batch, seq >= 1.  rope_base > 0, rms_eps >= 0.
 */
typedef struct {
  int32_t hidden, n_heads, n_kv_heads, head_dim, ffn;
  int32_t vocab;      /* 0 = no embedding / LM head                        */
  int32_t batch, seq; /* tokens T = batch * seq                             */
  float rms_eps;      /* 1e-6 for the Llama family                          */
  float rope_base;    /* 10000                                              */
  int32_t dtype;      /* sf_dtype                                           */
} sf_shape;

/* Tensor order inside one layer's flat parameter (and gradient) buffer. */
enum { SF_WQ = 0, SF_WK, SF_WV, SF_WO, SF_WG, SF_WU, SF_WD, SF_G1, SF_G2, SF_NTENSORS };

/*
 * Byte layout of one layer.  Parameters use the storage dtype; gradients are
 * fp32 with the same tensor order.  W tensors are [out, in] row-major.
 * Wq, Wk, Wv are adjacent with no padding (one [(n_h+2 n_kv) d, H] matrix);
 * Wg, Wu likewise (one [2F, H] matrix); other tensors start 256-B aligned.
 */
typedef struct {
  size_t off[SF_NTENSORS], bytes[SF_NTENSORS];           /* parameters */
  size_t grad_off[SF_NTENSORS], grad_bytes_t[SF_NTENSORS]; /* fp32 grads */
  size_t n_params;        /* parameter count of one layer                      */
  size_t param_bytes;     /* size of the flat parameter buffer                 */
  size_t grad_bytes;      /* size of the flat fp32 gradient buffer             */
  size_t saved_bytes;     /* per-layer activations kept from fwd for bwd       */
  size_t workspace_bytes; /* per-context device workspace                      */
  size_t head_workspace_bytes; /* extra workspace of sf_head_fwd_bwd for the
                                  chunk size given to sf_layer_layout           */
} sf_layout;

/*
 * Sizes of every region for `shape`.  head_chunk_rows is the LCE chunk
 * (rows of logits per block, >= 1; ignored when vocab == 0).  Host-only:
 * touches no device.
 */
sf_status sf_layer_layout(const sf_shape* shape, int32_t head_chunk_rows, sf_layout* out);

/*
 * sf_layer_layout with the rows of dlogits the head keeps for one LM-head
 * weight-gradient product.  The fused head (de §2C "Fused
 * LinearCrossEntropy") computes logits, loss and dlogits in chunks of
 * head_chunk_rows rows; each chunk's dW_lm contribution, added to the fp32
 * dW_lm, reads and writes all of V x H fp32 (4.2 GB at V 128256, H 4096),
 * so small chunks pay that once per chunk.  With head_dw_rows > head_chunk_rows
 * (rounded up to a multiple of it, at most all rows) the bf16 dlogits of
 * that many rows stay in the workspace and dW_lm takes one product per
 * group: head_workspace_bytes grows by (head_dw_rows - head_chunk_rows) V e,
 * the fp32 logits stay chunked.  0 (or <= head_chunk_rows): one product per
 * chunk, as sf_layer_layout.  The sums of dW_lm then run in another order
 * (same values up to fp32 rounding).
 */
sf_status sf_layer_layout_ex(const sf_shape* shape, int32_t head_chunk_rows, int32_t head_dw_rows,
                             sf_layout* out);

typedef struct sf_ctx sf_ctx;

/*
 * Create a context for `shape` on the current HIP device.  d_workspace must
 * hold layout.workspace_bytes (+ head_workspace_bytes when the head is used);
 * the context keeps the pointer and carves bwd temporaries and the RoPE
 * tables out of it (the tables are uploaded here, synchronously).  The
 * region must stay alive and untouched by the caller until sf_ctx_destroy.
 * The context also owns a non-blocking HIP stream (default priority) on
 * which sf_layer_bwd runs its weight-gradient GEMMs; with the environment
 * variable SF_SERIAL_WGRAD=1 at creation they stay on the caller's stream.
 * Returns SF_ERR_NO_DEVICE when no gfx950 device is current.
 */
sf_status sf_ctx_create(const sf_shape* shape, int32_t head_chunk_rows, void* d_workspace,
                        size_t workspace_bytes, sf_ctx** out);
/* sf_ctx_create with the head's dW_lm grouping of sf_layer_layout_ex. */
sf_status sf_ctx_create_ex(const sf_shape* shape, int32_t head_chunk_rows, int32_t head_dw_rows,
                           void* d_workspace, size_t workspace_bytes, sf_ctx** out);
sf_status sf_ctx_destroy(sf_ctx* ctx);

/*
 * Forward of one decoder block (the steps above).
 *   d_w     : flat parameters, sf_layout.param_bytes, storage dtype.
 *   d_x     : [T, H] layer input, storage dtype.
 *   d_y     : [T, H] layer output, storage dtype (may not alias d_x).
 *   d_saved : sf_layout.saved_bytes; receives the activations bwd needs.
 * Enqueued on `stream`; no host synchronisation.
 */
sf_status sf_layer_fwd(sf_ctx* ctx, const void* d_w, const void* d_x, void* d_y, void* d_saved,
                       sf_stream stream);

/*
 * Backward of one decoder block.
 *   d_x     : the same layer input given to sf_layer_fwd (RMSNorm-1 bwd).
 *   d_saved : as filled by sf_layer_fwd with the same d_w and d_x.
 *   d_dy    : [T, H] upstream gradient, storage dtype.
 *   d_dx    : [T, H] input gradient, storage dtype (may alias d_dy).
 *   d_dw    : fp32 gradients in layout order (sf_layout.grad_off), overwritten
 *             (not accumulated).  Deterministic: no floating-point atomics.
 * Uses the context workspace for temporaries; calls on one context must be
 * serialised on one stream.  When the weight-gradient GEMMs are too small
 * to fill the device (the [2F, H] one under 512 tiles of 256 x 256), they
 * run on the context's side stream, forked from `stream` once their operands
 * exist and joined back before the call's last operation: work queued on
 * `stream` afterwards sees every output, and the results are the same bits
 * as with all work on `stream`.
 */
sf_status sf_layer_bwd(sf_ctx* ctx, const void* d_w, const void* d_x, const void* d_saved,
                       const void* d_dy, void* d_dx, float* d_dw, sf_stream stream);

/*
 * Fused LinearCrossEntropy head (de §2C "Fused LinearCrossEntropy",
 * es §2C, fr §2C): final RMSNorm with gain d_gf [H], logits = hf W_lm^T in
 * blocks of head_chunk_rows rows (the full [T, V] logits never exist),
 * next-token cross-entropy averaged over batch*(seq-1) positions (target of
 * position s is ids[b, s+1]), and its backward.
 *   d_wlm  : [V, H] storage dtype;  d_x : [T, H] last block output;
 *   d_ids  : [T] int32 token ids in [0, V) (checked on the device: an id
 *            outside the range makes the loss NaN);
 *   d_loss : one fp32 (device);  d_dx : [T, H] storage dtype;
 *   d_dgf  : [H] fp32;  d_dwlm : [V, H] fp32.  All outputs overwritten.
 */
sf_status sf_head_fwd_bwd(sf_ctx* ctx, const void* d_gf, const void* d_wlm, const void* d_x,
                          const int32_t* d_ids, float* d_loss, void* d_dx, float* d_dgf,
                          float* d_dwlm, sf_stream stream);

/*
 * sf_head_fwd_bwd with the gradients multiplied by grad_scale (> 0, finite;
 * a power of two keeps the scaling exact): dlogits, and through them d_dx,
 * d_dgf and d_dwlm, carry the factor; the loss does not.  This is how loss
 * scaling enters the backward: with SF_F16 storage the unscaled dlogits of
 * a large vocabulary (about 1/N per entry) would mostly be fp16 subnormals.
 */
sf_status sf_head_fwd_bwd_scaled(sf_ctx* ctx, const void* d_gf, const void* d_wlm, const void* d_x,
                                 const int32_t* d_ids, float* d_loss, void* d_dx, float* d_dgf,
                                 float* d_dwlm, float grad_scale, sf_stream stream);

/*
 * One dense projection with the block's MFMA GEMM -- the primitive behind
 * every projection above (exposed for measurement and testing):
 *   layout 0 (NT): C[M, N] = A[M, K] B[N, K]^T   (forward  y = x W^T)
 *   layout 1 (NN): C[M, N] = A[M, K] B[K, N]     (input gradient dX = dY W)
 *   layout 2 (TN): C[M, N] = A[K, M]^T B[K, N]   (weight gradient dW = dY^T X)
 * A, B: storage dtype `dtype`, row-major with leading dimensions lda, ldb
 * (elements).  C: fp32 when out_f32 != 0, else the storage dtype, leading
 * dimension ldc; overwritten.  The contiguous dimension of every operand
 * (and N) must be a multiple of 8; M, N, K >= 0 otherwise arbitrary.
 * d_workspace (may be NULL) lets a GEMM with few output tiles split K into
 * fp32 partial sums reduced in a fixed order (deterministic); it is used
 * only when workspace_bytes >= sf_gemm_workspace_bytes(M, N, K).
 */
sf_status sf_gemm(int32_t dtype, int32_t layout, int32_t out_f32, int32_t M, int32_t N, int32_t K,
                  const void* d_A, int64_t lda, const void* d_B, int64_t ldb, void* d_C, int64_t ldc,
                  void* d_workspace, size_t workspace_bytes, sf_stream stream);

/* Workspace bytes sf_gemm can use for split-K at these sizes (0 = none). */
size_t sf_gemm_workspace_bytes(int32_t M, int32_t N, int32_t K);

/*
 * sf_gemm for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same product, kernels and bits as sf_gemm given a workspace of at least
 * sf_gemm_workspace_bytes(M, N, K), but with no workspace argument.  The
 * split-K partial sums go to a static device buffer of
 * SF_GEMM_STATIC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends; no call allocates or frees anything.
 * Every partial sum is written before it is read, so the buffer needs no
 * clearing and keeps the last call's contents.  All calls on one device
 * share the buffer: calls that overlap in time (other streams, other host
 * threads) race and must be serialised by the caller.
 * Errors: those of sf_gemm, and SF_ERR_POOL (before any device work) when
 * sf_gemm_workspace_bytes(M, N, K) > SF_GEMM_STATIC_SCRATCH_BYTES.
 */
#define SF_GEMM_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
sf_status sf_gemm_noalloc(int32_t dtype, int32_t layout, int32_t out_f32, int32_t M, int32_t N, int32_t K,
                          const void* d_A, int64_t lda, const void* d_B, int64_t ldb, void* d_C, int64_t ldc,
                          sf_stream stream);

/* x0[t] = E[ids[t]] for t < T.  E [V, H] storage dtype, x0 [T, H]. */
sf_status sf_embed_fwd(sf_ctx* ctx, const void* d_E, const int32_t* d_ids, void* d_x0, sf_stream stream);

/* dE[v] = sum over t with ids[t] == v of dx0[t], fp32 [V, H], overwritten,
 * summed in increasing t (deterministic). */
sf_status sf_embed_bwd(sf_ctx* ctx, const void* d_dx0, const int32_t* d_ids, float* d_dE,
                       sf_stream stream);

/*
 * Host Adam over n fp32 elements (es §2A: the CPU updates layer L_i with
 * host-resident optimizer states; es §2B: states are flattened host
 * tensors; de/es/fr §2B: shared buffers do the FP32 -> BF16 conversion).
 *   m <- b1 m + (1-b1) g ; v <- b2 v + (1-b2) g^2 ;
 *   p <- p - lr (m/(1-b1^step)) / (sqrt(v/(1-b2^step)) + eps)
 * p_bf16 (optional, may be NULL) receives round-to-nearest-even bf16 of the
 * new p.  step >= 1.  Runs synchronously on n_threads host threads
 * (n_threads <= 0: one per available core).  Host pointers, any memory.
 */
sf_status sf_adam_host(float* p, float* m, float* v, const float* g, uint16_t* p_bf16, size_t n,
                       int64_t step, float lr, float b1, float b2, float eps, int32_t n_threads);

/*
 * The same Adam step on the device for tensors that stay resident in HBM
 * (the embedding and LM head): d_p (fp32 master), d_m, d_v updated in place
 * from d_g, n elements; d_out receives the storage-dtype copy of the new
 * parameters (dtype SF_BF16: round to nearest even; SF_F32: a copy; may be
 * NULL).  Every operation is rounded exactly as in sf_adam_host, so the two
 * agree bit for bit.  Enqueued on `stream`.
 */
sf_status sf_adam_device(int32_t dtype, float* d_p, float* d_m, float* d_v, const float* d_g, void* d_out, size_t n,
                         int64_t step, float lr, float b1, float b2, float eps, sf_stream stream);

/*
 * The host and device Adam steps for any storage dtype, with the gradient
 * taken as g * grad_scale (the inverse of a loss scale; 1 leaves it exact,
 * and a power of two keeps it exact): the same operations, rounded the same
 * way, on both sides.  p_out / d_out receive the storage copy (SF_BF16 or
 * SF_F16: round to nearest even; SF_F32: NULL or p itself).
 */
sf_status sf_adam_host_ex(int32_t dtype, float* p, float* m, float* v, const float* g, void* p_out, size_t n,
                          int64_t step, float lr, float b1, float b2, float eps, float grad_scale,
                          int32_t n_threads);
sf_status sf_adam_device_ex(int32_t dtype, float* d_p, float* d_m, float* d_v, const float* d_g, void* d_out,
                            size_t n, int64_t step, float lr, float b1, float b2, float eps, float grad_scale,
                            sf_stream stream);

/* ------------------------------------------------------------------ engine */

typedef struct sf_engine sf_engine;

enum {
  SF_ENGINE_ADAM = 1,           /* run host Adam on every streamed-out gradient  */
  SF_ENGINE_HEAD = 2,           /* ids in; embedding + fused LinearCrossEntropy */
  SF_ENGINE_HEAD_HOST_ADAM = 4, /* update the resident embedding / LM head on the
                                   host too (gradients out, parameters back in)
                                   instead of with sf_adam_device in HBM        */
  SF_ENGINE_CKPT = 8            /* sliding activation checkpointing (de/es/fr
                                   §2B): each layer's input leaves for h_ckpt
                                   after it is produced and comes back before
                                   the layer's backward, which first recomputes
                                   the layer's forward; the device keeps a
                                   fixed six [T, H] buffers and two saved sets
                                   whatever n_layers is.  Same bits as without */,
  SF_ENGINE_PIPELINE = 16       /* host Adam across the iteration boundary:
                                   sf_slide_step returns once the device work
                                   and the loss are done while Adam jobs still
                                   run; the next step's forward waits, layer by
                                   layer, only for the update of the layer it
                                   is about to read, and the host applies
                                   updates in ascending layer order (the order
                                   the forward needs them).  Same bits as
                                   without.  Not with SF_ENGINE_HEAD_HOST_ADAM
                                   (SF_ERR_UNSUPPORTED).  Call sf_engine_sync
                                   before reading host parameters or moments.
                                   Without SF_ENGINE_ADAM the step returns
                                   once its kernels are done while the last
                                   gradient copies still run (the next step's
                                   uploads overlap them); sf_engine_sync
                                   before reading h_grad_slots */,
  SF_ENGINE_KEEP_TURNAROUND = 32 /* without SF_ENGINE_ADAM: the caller keeps
                                   h_params unchanged between steps, so layers
                                   0 .. window-1, which end the backward in
                                   their units, open the next forward without
                                   being uploaded again (with SF_ENGINE_ADAM
                                   they always are: Adam re-uploads them).
                                   Same bits as without */
};

/*
 * Engine configuration.  All pointers are borrowed and must outlive the
 * engine.
 *   d_pool/pool_bytes : device region (256-B aligned) for min(window,
 *       n_layers) cache units; unit u holds one layer's parameters (storage
 *       dtype, param_bytes rounded up to 256) followed by its fp32 gradients
 *       (grad_bytes rounded up to 256).  In the backward layer l uses unit
 *       l % window; in the forward the engine also runs layers from the
 *       gradient regions, which are idle there once the previous backward's
 *       gradients have left.
 *   d_act/act_bytes   : device region (256-B aligned) of at least
 *       sf_engine_act_bytes_flags(): the n_layers + 1 layer inputs/outputs
 *       [T, H], the n_layers saved activation sets, one [T, H] gradient
 *       buffer and the device loss (with SF_ENGINE_CKPT: six [T, H] buffers,
 *       two saved sets, the gradient buffer and the loss).
 *   h_ckpt            : SF_ENGINE_CKPT with n_layers >= 2: pinned host,
 *       n_layers - 1 layer inputs of act x bytes each (x = [T, H] in the
 *       storage dtype rounded up to 256 bytes; layer l at l * x).
 *   h_params[l]       : pinned host, layer l flat parameters in the
 *       parameter layout (storage dtype).  Streamed to the device twice per
 *       step (forward and backward) except for the last `window` layers,
 *       which stay resident across the forward/backward turnaround.  With
 *       SF_ENGINE_ADAM the updated parameters are written back here, and
 *       those of layers 0 .. window-1 are also uploaded to their units
 *       before sf_slide_step returns (the next step starts from them): do
 *       not change h_params between steps of an engine with Adam.
 *   h_master/h_m/h_v[l]: host fp32 master weights and Adam moments of
 *       layer l in the fp32 gradient layout (grad_off / grad_bytes_t); any
 *       host memory.  Required with SF_ENGINE_ADAM.  For SF_F32 storage
 *       h_master[l] may equal h_params[l].
 *   h_grad_slots[k]   : n_grad_slots pinned fp32 buffers of grad_bytes,
 *       shared by every layer in turn (de/es/fr §2B shared CPU buffers).
 *   compute_stream    : the stream kernels run on (NULL = default stream).
 *   SF_ENGINE_HEAD: d_E [V, H], d_gf [H], d_wlm [V, H] device, storage
 *       dtype, resident; d_head_grads device fp32 [dE | dgf | dWlm] of
 *       2 V H + H floats (the engine's scratch: with SF_ENGINE_ADAM and the
 *       device update, the dE part holds the embedding gradient's distinct
 *       rows and a row map rather than the dense [V, H] gradient).  With
 *       SF_ENGINE_ADAM the resident tensors are updated in place by default
 *       on the device from d_head_state (device fp32 [master | m | v], each
 *       2 V H + H floats in [E | gf | Wlm] order; the caller sets the
 *       masters and zeroes both moments before the first step).  With SF_ENGINE_HEAD_HOST_ADAM instead: h_head_grads (pinned
 *       fp32, 2 V H + H), h_head_params (pinned, storage dtype [E | gf |
 *       Wlm]) and fp32 host h_head_master/m/v; the LM-head gradients leave
 *       after the head, the embedding gradient leaves as its nonzero rows,
 *       and the updated parameters are uploaded back before the step
 *       returns.
 */
typedef struct {
  int32_t n_layers;
  int32_t window;          /* >= 2 */
  int32_t n_grad_slots;    /* >= 2 */
  int32_t flags;
  int32_t adam_threads;    /* <= 0: one per available core, less two */
  float lr, b1, b2, eps;
  void* d_pool;
  size_t pool_bytes;
  void* d_act;
  size_t act_bytes;
  void** h_params;
  float** h_master;
  float** h_m;
  float** h_v;
  float** h_grad_slots;
  sf_stream compute_stream;
  void* d_E;
  void* d_gf;
  void* d_wlm;
  float* d_head_grads;
  void* h_head_params;
  float* h_head_master;
  float* h_head_m;
  float* h_head_v;
  float* h_head_grads;
  float* d_head_state;
  void* h_ckpt;
  /* Dynamic loss scaling (SF_F16 storage only; ignored otherwise).  The
   * backward starts from the loss gradient times S (dlogits, or the given
   * d_dy without a head); weight gradients leave scaled and Adam takes them
   * times 1/S.  After each layer's backward the device checks its fp32
   * gradients for infinities and NaNs: a layer is updated only if its
   * gradients and all computed before it in the backward (the head's, the
   * layers above) are finite, the embedding only if the whole step is; a
   * skipped update leaves the tensor, its moments and its Adam step count
   * as they were.  Then S halves (not below 1) after a step with a
   * non-finite gradient and doubles after scale_window consecutive finite
   * steps.  Host Adam of a layer starts once that layer's check is done. */
  float loss_scale;        /* initial S; 0 = 65536                              */
  int32_t scale_window;    /* 0 = 2000                                           */
} sf_engine_cfg;

/* Per-step measurements (host wall clock and device events). */
typedef struct {
  double wall_ms;          /* sf_slide_step entry to return                   */
  double compute_ms;       /* union of compute-stream busy intervals          */
  double copy_ms;          /* union of H2D and D2H busy intervals             */
  double h2d_ms, d2h_ms;   /* per-direction busy time                          */
  double overlap_pct;      /* 100 |compute n copy| / min(compute, copy): the
                              share of the shorter activity hidden under the
                              other (|compute n copy| = compute + copy - busy) */
  double busy_ms;          /* union of compute and copy intervals              */
  double span_ms;          /* first device event to last; span - busy = idle   */
  double adam_ms;          /* sum of host Adam job durations                   */
  double h2d_bytes, d2h_bytes;
  double h2d_gbps, d2h_gbps;
  float loss;
  float loss_scale;        /* S this step used (1 without loss scaling)            */
  int32_t skipped;         /* updates this step skipped for non-finite gradients:
                              layers, plus one for the LM head and final gain and
                              one for the embedding (SF_F16; pipelined: the last
                              step's)                                               */
} sf_step_stats;

/* Device bytes the engine needs in d_act for `shape`, n_layers and the
 * engine flags (SF_ENGINE_CKPT changes the layout); sf_engine_act_bytes is
 * the same with flags 0. */
sf_status sf_engine_act_bytes_flags(const sf_shape* shape, int32_t n_layers, int32_t flags, size_t* out);
sf_status sf_engine_act_bytes(const sf_shape* shape, int32_t n_layers, size_t* out);

sf_status sf_engine_create(sf_ctx* ctx, const sf_engine_cfg* cfg, sf_engine** out);

/*
 * One training iteration (de §2A, es §2A, fr §2A): forward through every
 * layer with the next layer's parameters prefetched into a free cache unit,
 * the head (with SF_ENGINE_HEAD), then backward in reverse order; each
 * layer's fp32 gradients stream to a shared host slot and, with
 * SF_ENGINE_ADAM, are applied by host Adam threads while the device runs the
 * next layer's backward.  Adam of layer i uses this iteration's gradients
 * (no staleness), so the step equals plain synchronous training.
 *   d_in  : [T] int32 ids (SF_ENGINE_HEAD) or [T, H] layer-0 input.
 *   d_dy  : [T, H] upstream gradient of the last layer (no head), else NULL.
 *   h_loss: receives the loss (SF_ENGINE_HEAD), may be NULL.
 * Returns after the iteration's device work and Adam jobs are complete
 * (with SF_ENGINE_PIPELINE: after its device work; *stats then holds only
 * wall_ms and loss, and sf_engine_sync measures the steps as a whole).
 * Host Adam takes the ranges whose copies have landed lowest layer first.
 * A HIP failure moves the engine to a sticky error state (SF_ERR_STATE on
 * later calls).
 */
sf_status sf_slide_step(sf_engine* eng, const void* d_in, const void* d_dy, float* h_loss,
                        sf_step_stats* stats);

/*
 * Wait until every copy, kernel and host Adam job of the steps issued so far
 * is complete (host parameters, masters and moments final, units 0 ..
 * window-1 loaded for the next step).  stats (may be NULL) receives the
 * measurements of all steps since the previous sync (pipelined), or of the
 * last step (synchronous engine, where this only returns them again); the
 * step trace then covers the same window.  An Adam failure surfaces here or
 * at the next step and leaves the engine in the error state.
 */
sf_status sf_engine_sync(sf_engine* eng, sf_step_stats* stats);

/* Device pointer of layer l's input activation from the last step (l = 0..
 * n_layers; l = n_layers is the last layer's output), and of the input
 * gradient of layer 0 after the last step.  For tests and inspection.
 * With SF_ENGINE_CKPT only l = n_layers - 1 and n_layers stay on the device
 * (SF_ERR_UNSUPPORTED below that: the others are in h_ckpt). */
sf_status sf_engine_layer_input(sf_engine* eng, int32_t layer, void** d_x);
sf_status sf_engine_dx0(sf_engine* eng, void** d_dx0);

/*
 * Timeline of the last completed step, for inspecting the overlap the
 * engine's design rests on (de/es/fr §2A: copies and host updates hidden
 * under device compute).  Writes min(capacity, rows) rows of 4 doubles to
 * out (host memory owned by the caller) and the total row count to *n_rows;
 * capacity 0 with out NULL just returns the count.  Row = {kind, start_ms,
 * end_ms, info}: kind 0 = compute interval (a kernel sequence on the
 * compute stream), 1 = H2D copy, 2 = D2H copy (info = bytes), 3 = host Adam
 * job on a layer's gradient range, 4 = host Adam of the LM head, 5 = host
 * Adam of the embedding (info = layer index or -1).  Times are ms after the
 * step's first device event; device rows come from HIP events, Adam rows
 * from the host clock aligned to that event (error: the latency of one
 * event record, microseconds).  Rows are grouped by source, not sorted.
 */
sf_status sf_engine_trace(sf_engine* eng, double* out, int32_t capacity, int32_t* n_rows);

/*
 * Bookkeeping of the engine's timing, for tests and inspection.  Writes
 * min(n, 5) values to out (host): [0] timing events the engine owns (all
 * created by sf_engine_create; steps never create more), [1] of them free,
 * [2] timed intervals still in flight, [3] completed intervals of the
 * current measurement window held on the host (32 bytes each, until the
 * window closes: every synchronous step, or sf_engine_sync when pipelined),
 * [4] times the host waited for an interval to complete because every
 * timing event was in use.
 *
 * Failure injection for tests of the error path: with the environment
 * variable SF_FAULT_ADAM_JOB=k set at sf_engine_create, the engine's k-th
 * host Adam job (counted from 0 over the engine's life) reports a failure
 * instead of running; the step or sync that observes it returns SF_ERR_HIP
 * and the engine is then in the sticky error state.  With
 * SF_FAULT_NONFINITE_LAYER=i (fp16 engines), layer i's non-finite flag is
 * raised in every step as if its gradients had overflowed, which exercises
 * the layer-wise skip rule of sf_engine_cfg.loss_scale without an overflow.
 */
sf_status sf_engine_counters(sf_engine* eng, int64_t* out, int32_t n);

sf_status sf_engine_destroy(sf_engine* eng);

const char* sf_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SF_H */

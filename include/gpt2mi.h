/* gpt2mi.h - C ABI of libgpt2mi.so: the GPT-2 pre-norm decoder forward and its
 * cached single-token decode step on one AMD Instinct MI355X (gfx950).
 *
 * What is computed (web pages, cited by title and section):
 *   "Decoder Block" (GPT-2, AI Engineer Exhaustive), How it works: one pre-norm
 *     block, x <- x + Attn(LN1 x); x <- x + MLP(LN2 x), LayerNorm eps 1e-5,
 *     causal multi-head attention with a fused QKV projection (c_attn) and an
 *     output projection (c_proj), a 4d-wide GELU MLP (c_fc, c_proj).
 *   "Full Forward Pass" (GPT-2, AI Engineer Exhaustive), How it works: the
 *     embedding sum wte[id] + wpe[l_past + t], L blocks, the final ln_f, the tied
 *     head logits = LN_f(H) wte^T, and the per-layer present (new K, V) stacked
 *     as [B, L, 2, h, T, d_h]; a cached step feeds only the newest token.
 *   "GPT-2 Transformer block" (Open Model Atlas), norm() excerpt: mean, biased
 *     variance of deviations, rsqrt(s + eps), gain, bias.
 *   "GPT-2 Block - TorchCode", Reference Solution: scores scaled by 1/sqrt(d_h),
 *     future positions masked.
 * GELU is the tanh approximation 0.5x(1 + tanh(sqrt(2/pi)(x + 0.044715x^3))).
 *
 * Conventions for every entry point:
 *   - Pointers named as device pointers must be device memory (hipMalloc or a
 *     torch CUDA tensor) on the current device; host structs (gpt2_hparams,
 *     gpt2_weights, gpt2_block_weights, gpt2_kv) are read only during the call.
 *   - The caller owns every buffer.  The library never allocates, frees or
 *     synchronises on the compute path; work is enqueued on `stream` (a
 *     hipStream_t; NULL is the default stream) and runs asynchronously.
 *   - All tensors are dense row-major.  Linear weights are stored [out, in]
 *     (y = x W^T + b); wte is [n_vocab, n_embd], wpe is [n_ctx, n_embd].
 *   - GPT2_BF16: weights, LayerNorm gains/biases, linear biases, block-mode x and y
 *     and the K/V cache are bfloat16; matrix products accumulate in fp32; the
 *     residual stream inside gpt2_forward / gpt2_prefill / gpt2_decode_step is fp32; logits are
 *     fp32.  GPT2_FP32: every tensor is fp32 and all arithmetic is fp32.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     are returned as a status; nothing is launched then.  A launch failure is
 *     GPT2_E_HIP.  An out-of-range token id cannot be seen without a sync: the
 *     embedding kernel zero-fills that row and raises a sticky device flag in
 *     the workspace that gpt2_read_device_flags reports and clears.
 *   - Concurrent calls must use distinct workspaces.
 *   - Reproducibility: every call is deterministic, bit for bit, for given
 *     inputs and sizes.  (With B*T <= 64 rows in GPT2_BF16 the residual
 *     products split their K range over workgroups; the parts are added in a
 *     fixed order by the LayerNorm that follows.)
 *   - Device pointers to weights, activations and the K/V cache must be
 *     16-byte aligned; token ids, targets, outputs of ids and fp32 logits /
 *     losses 4-byte aligned; the workspace 256-byte aligned (any hipMalloc or
 *     torch allocation is).  A misaligned pointer gives GPT2_E_ALIGN
 *     (GPT2_E_WORKSPACE for the workspace).
 */
#ifndef GPT2MI_H
#define GPT2MI_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPT2_OK = 0,
  GPT2_E_NULL = 1,      /* a required pointer is NULL */
  GPT2_E_SHAPE = 2,     /* unsupported or inconsistent sizes */
  GPT2_E_DTYPE = 3,     /* unknown mode */
  GPT2_E_POSITION = 4,  /* l_past + T exceeds n_ctx or the cache capacity */
  GPT2_E_WORKSPACE = 5, /* ws_bytes smaller than gpt2_workspace_size(), or ws misaligned */
  GPT2_E_TOKEN = 6,     /* a token id was outside [0, n_vocab) (device flag) */
  GPT2_E_HIP = 7,       /* the HIP runtime reported an error */
  GPT2_E_ALIGN = 8      /* a device pointer is not aligned as the conventions require */
} gpt2_status;

typedef enum { GPT2_FP32 = 0, GPT2_BF16 = 1 } gpt2_mode;

/* Model sizes ("Full Forward Pass", Overview: n_vocab, n_ctx, n_embd, n_head,
 * n_layer) and the LayerNorm epsilon (1e-5 on the pages).
 * Supported: n_embd % n_head == 0, n_embd <= 2048, n_embd % 8 == 0; head
 * width d_h = n_embd / n_head a multiple of 4 no larger than 128.  GPT2_BF16
 * with d_h = 64 runs the MFMA attention kernels; GPT2_FP32, and GPT2_BF16
 * with another d_h, run a row-wise attention kernel for which a call's
 * l_past + T must stay within 8192 keys (else GPT2_E_SHAPE). */
typedef struct {
  int32_t n_vocab, n_ctx, n_embd, n_head, n_layer;
  float eps;
} gpt2_hparams;

/* One block's parameters (device pointers, mode dtype; d = n_embd):
 * ln1_g, ln1_b [d]; attn_w [3d, d], attn_b [3d] (rows: q | k | v, head j owns
 * rows j*d_h .. of each third); proj_w [d, d], proj_b [d]; ln2_g, ln2_b [d];
 * fc_w [4d, d], fc_b [4d]; fc2_w [d, 4d], fc2_b [d]. */
typedef struct {
  const void *ln1_g, *ln1_b, *attn_w, *attn_b, *proj_w, *proj_b;
  const void *ln2_g, *ln2_b, *fc_w, *fc_b, *fc2_w, *fc2_b;
} gpt2_block_weights;

/* Whole-model parameters: wte [n_vocab, d] (also the tied head), wpe [n_ctx, d],
 * lnf_g, lnf_b [d] (device pointers), blocks: host array of n_layer entries. */
typedef struct {
  const void *wte, *wpe, *lnf_g, *lnf_b;
  const gpt2_block_weights *blocks;
} gpt2_weights;

/* K/V cache (device memory, mode dtype), layout [B, n_layer, 2, n_head,
 * capacity, d_h]; index 0 of the third axis is K, 1 is V; slot s holds the
 * key/value of absolute position s. */
typedef struct {
  void *data;
  int32_t capacity;
} gpt2_kv;

/* Bytes of workspace any of the compute calls needs for batch B and T new
 * tokens per sequence (T = 1 for gpt2_decode_step).  0 on bad arguments.
 * A new workspace must be zero-filled once before its first use (the first
 * 256 bytes hold the sticky device flags).  Every call takes the workspace
 * start 256-byte aligned (as any hipMalloc or torch allocation is); a
 * misaligned one gives GPT2_E_WORKSPACE. */
size_t gpt2_workspace_size(const gpt2_hparams *hp, gpt2_mode mode, int32_t B, int32_t T);

/* One pre-norm block ("Decoder Block", How it works) on x [B, T, d] -> y [B, T, d]
 * (device, mode dtype; x and y must not overlap).  Positions are 0..T-1 (no past).
 * present (device, may be NULL): receives the block's new K, V as
 * [B, 2, n_head, T, d_h].  Requires 1 <= T <= n_ctx.  n_vocab and n_layer are
 * not used. */
gpt2_status gpt2_block_forward(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_block_weights *w,
                               const void *x, void *y, int32_t B, int32_t T, void *present,
                               void *ws, size_t ws_bytes, void *stream);

/* Uncached full forward ("Full Forward Pass", How it works): ids [B, T] int32
 * (device) at positions 0..T-1 -> logits [B, T, n_vocab] fp32 (device).
 * present (may be NULL): a cache with capacity >= T whose slots 0..T-1 of every
 * layer receive the new K, V (the stacked present).  Requires 1 <= T <= n_ctx. */
gpt2_status gpt2_forward(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                         const int32_t *ids, int32_t B, int32_t T, float *logits,
                         const gpt2_kv *present, void *ws, size_t ws_bytes, void *stream);

/* One cached decode step ("Full Forward Pass", How it works, last paragraph):
 * ids [B] int32 (device) are the newest tokens at position l_past; the cache
 * holds slots 0..l_past-1 of every layer and receives the new K, V at slot
 * l_past; each layer attends over slots 0..l_past.  logits [B, 1, n_vocab] fp32.
 * Requires 0 <= l_past < min(n_ctx, cache->capacity). */
gpt2_status gpt2_decode_step(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                             const int32_t *ids, int32_t B, int32_t l_past, const gpt2_kv *cache,
                             float *logits, void *ws, size_t ws_bytes, void *stream);

/* gpt2_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The step's intermediate buffers live in a
 * fixed 16 MiB device array inside the library, one per GPU, held until the
 * process ends; nothing is allocated or freed by the call.  A call whose
 * workspace (gpt2_workspace_size(hp, mode, B, 1)) exceeds 16 MiB returns
 * GPT2_E_WORKSPACE before anything is enqueued (in bf16 that admits every
 * B <= 64 up to n_embd 2048 and, at n_embd 768, B up to 992; in fp32 about
 * 40 * B * n_embd bytes are needed).  Every call on a GPU shares that GPU's array: calls
 * that overlap in time on one GPU (other streams, other host threads) race
 * and must be serialised by the caller.  An out-of-range token id zero-fills
 * its row as in gpt2_decode_step, but its sticky flag lives in the library's
 * array and is not reported (gpt2_read_device_flags reads a caller's
 * workspace).  Other arguments, results and errors as gpt2_decode_step. */
gpt2_status gpt2_decode_step_noalloc(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                                     const int32_t *ids, int32_t B, int32_t l_past, const gpt2_kv *cache,
                                     float *logits, void *stream);

/* Forward over T new tokens per sequence against a cached past ("Full Forward
 * Pass", How it works: the model takes the past keys/values and new tokens, and
 * query t at position l_past + t attends to every key at positions
 * 0..l_past + t): ids [B, T] int32 (device) at positions l_past..l_past+T-1;
 * the cache holds slots 0..l_past-1 of every layer and receives the new K, V at
 * slots l_past..l_past+T-1; logits [B, T, n_vocab] fp32 (device).  Calling it
 * on consecutive chunks of a sequence fills the cache like one call on the
 * whole sequence (chunked prefill); l_past = 0 is gpt2_forward with a cache,
 * T = 1 is gpt2_decode_step.  Requires T >= 1, l_past >= 0 and
 * l_past + T <= min(n_ctx, cache->capacity), else GPT2_E_POSITION; the
 * workspace is sized by gpt2_workspace_size(hp, mode, B, T). */
gpt2_status gpt2_prefill(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                         const int32_t *ids, int32_t B, int32_t T, int32_t l_past, const gpt2_kv *cache,
                         float *logits, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace gpt2_generate_greedy needs for batch B (0 on bad
 * arguments); zero-filled once before first use, like the others. */
size_t gpt2_generate_workspace_size(const gpt2_hparams *hp, gpt2_mode mode, int32_t B);

/* Greedy generation loop ("Full Forward Pass", How it works: each step feeds
 * only the newest token with the cached keys/values, and the chosen token is
 * fed back).  ids [B] int32 (device): the token at position l_past of each
 * sequence, whose cache already holds slots 0..l_past-1.  Runs n_new decode
 * steps entirely on the device: step i feeds token i at position l_past + i
 * (appending its K, V at that slot) and picks token i + 1 as the argmax of its
 * logits (lowest index among equal maxima), written to out[b * n_new + i]
 * (out: [B, n_new] int32, device).  Nothing is synchronised and no logits are
 * returned; in GPT2_BF16 with B <= 64 none are written either (the head's
 * tiles reduce to per-row maxima in the product itself).  Requires n_new >= 1 and l_past + n_new <= min(n_ctx,
 * cache->capacity), else GPT2_E_POSITION; ws_bytes >=
 * gpt2_generate_workspace_size(hp, mode, B). */
gpt2_status gpt2_generate_greedy(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                                 const int32_t *ids, int32_t B, int32_t l_past, int32_t n_new,
                                 const gpt2_kv *cache, int32_t *out, void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace gpt2_forward_loss needs (0 on bad arguments); zero-filled
 * once before first use, like the others. */
size_t gpt2_loss_workspace_size(const gpt2_hparams *hp, gpt2_mode mode, int32_t B, int32_t T);

/* The uncached forward followed by the next-token cross-entropy that callers
 * take of the logits ("Full Forward Pass", How it works): for ids [B, T] and
 * targets [B, T] int32 (device; the token each position should predict, e.g.
 * ids shifted by one), loss [B, T] fp32 (device) receives
 * log(sum_n exp(logit_n)) - logit_target for every position.  The logits are
 * not returned: in bf16 mode the head's epilogue keeps only per-row
 * log-sum-exp partials (the 4 B x n_vocab per token logits never reach
 * memory).  present as in gpt2_forward.  A target outside [0, n_vocab) gives a
 * NaN loss and raises the same sticky flag as a bad token id
 * (gpt2_read_device_flags).  Requires 1 <= T <= n_ctx and ws_bytes >=
 * gpt2_loss_workspace_size(hp, mode, B, T). */
gpt2_status gpt2_forward_loss(const gpt2_hparams *hp, gpt2_mode mode, const gpt2_weights *W,
                              const int32_t *ids, const int32_t *targets, int32_t B, int32_t T, float *loss,
                              const gpt2_kv *present, void *ws, size_t ws_bytes, void *stream);

/* Synchronises `stream`, then reads and clears the workspace's sticky device
 * flags: GPT2_E_TOKEN if any earlier call on this workspace saw a token id
 * outside [0, n_vocab), else GPT2_OK (or GPT2_E_HIP). */
gpt2_status gpt2_read_device_flags(void *ws, void *stream);

/* Per-kernel timing, for measurement only (the compute path never needs it).
 * After gpt2_timing_begin(), every kernel that the compute calls enqueue is
 * bracketed by a HIP event pair recorded on the call's stream; the events
 * are host-side objects the library creates once and reuses (no device
 * memory).  gpt2_timing_end() waits for the last event, sums the elapsed time
 * per kernel kind, writes at most max_entries records to `out` (name: static
 * string such as "gemm_c_fc" or "attn_decode") and returns the number
 * of kinds seen, or -1 if timing was not on or a HIP call failed.  Not
 * thread-safe: one timing session per process at a time. */
typedef struct {
  const char *name;
  int32_t launches;
  double total_ms;
} gpt2_kernel_time;

gpt2_status gpt2_timing_begin(void);
int32_t gpt2_timing_end(gpt2_kernel_time *out, int32_t max_entries);

/* Static, human-readable name of a status code. */
const char *gpt2_status_str(gpt2_status s);

#ifdef __cplusplus
}
#endif

#endif /* GPT2MI_H */

// Internal launchers (host side) for the gfx950 kernels of libgpt2mi.so.
// Every launcher enqueues on `s` and returns without synchronising; shapes
// have been validated by the C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace gpt2 {

// ---------------------------------------------------------------- per-device host facts
// Device properties and function attributes belong to the device that is
// current when they are read or set; both helpers act on the current device
// and cache per device (thread-safe).
// Compute units of the current device (256 if the query fails).
int device_cu_count();
// Raises fn's dynamic-LDS limit to `bytes` on the current device, once per
// (device, kernel).
void set_dynamic_lds_limit(const void* fn, int bytes);

// ---------------------------------------------------------------- embedding
// Embedding plus the first LayerNorm: x[m, :] (fp32) = wte[ids[m], :] +
// wpe[l_past + m % T, :] and a = LN(x; g, b) in the act dtype, one pass per
// row; a bad id zero-fills the row and ORs 1 into *flags.
void launch_embed_ln(bool bf16, const int32_t* ids, const void* wte, const void* wpe, float* x,
                     const void* g, const void* b, void* a, int M, int T, int l_past, int d, int n_vocab,
                     float eps, uint32_t* flags, hipStream_t s);

// ---------------------------------------------------------------- LayerNorm
// y = LN(x) * g + b over rows of width d; one row per wave.
// x_f32: x is fp32 (else mode dtype); act_bf16: g, b, y are bf16 (else fp32).
void launch_layernorm(bool x_f32, bool act_bf16, const void* x, const void* g, const void* b,
                      void* y, int M, int d, float eps, hipStream_t s);

// Residual update and LayerNorm for products kept as K-range partials
// (bf16 activations, fp32 stream): x[m] <- x[m] + ((bias + part[0][m]) +
// part[1][m] + ... + part[S-1][m]), a fixed order; then a = LN(x) as
// launch_layernorm.  part is [S][M][d] fp32.
void launch_layernorm_reduce(float* x, const float* part, int S, const void* bias, const void* g, const void* b,
                             void* a, int M, int d, float eps, hipStream_t s);

// ---------------------------------------------------------------- GEMM
enum EpiKind {
  EPI_STORE_F32 = 0,   // out fp32 [M, N] = acc                    (tied head)
  EPI_BIAS_GELU = 1,   // out act [M, N] = gelu(acc + bias)        (c_fc)
  EPI_BIAS_RESID = 2,  // out = resid + acc + bias                 (c_proj, mlp.c_proj)
  EPI_QKV = 3          // acc + bias split to q [B,h,T,d_h] and the K/V view (c_attn)
};

struct Epilogue {
  EpiKind kind;
  const void* bias;   // [N], act dtype
  void* out;          // EPI_STORE_F32 / EPI_BIAS_GELU / EPI_BIAS_RESID
  const void* resid;  // EPI_BIAS_RESID, [M, N]
  bool resid_f32;     // residual input is fp32 (else act dtype)
  bool out_f32;       // EPI_BIAS_RESID output is fp32 (else act dtype)
  // EPI_QKV
  void* q;            // [B, h, T, d_h]
  KvView kv;          // K/V destination for positions l_past .. l_past + T - 1
  int T, l_past, n_head, d_head, d;
};


// Y = X W^T with the epilogue; X [M, K], W [N, K] row-major.
// bf16: MFMA paths (K % 8 == 0; M <= 64 uses the weight-streaming skinny
// kernel when K allows); else fp32 FMA path (K % 4 == 0).
void launch_gemm(bool bf16, const void* X, const void* W, int M, int N, int K, const Epilogue& e,
                 hipStream_t s);

// Decode-sized in-place residual products (bf16, M <= 64) stream their
// weights faster over more workgroups when K is split into ranges: the
// number of ranges S for X [M, K] x W [N, K]^T, or 1 when the product is not
// split.  launch_gemm_partials then writes the S range products to part
// [S][M][N] fp32 (no bias); launch_layernorm_reduce adds them up.
int residual_splits(bool bf16, int M, int N, int K);
void launch_gemm_partials(const void* X, const void* W, int M, int N, int K, int S, float* part, hipStream_t s);

// ---------------------------------------------------------------- head + cross-entropy
// Fused tied head for the loss (bf16, M > 64, K % 64 == 0): logits of X [M, K]
// against W [N, K] are reduced in the product's epilogue to per-row partial
// log-sum-exp states part [M][head_lse_parts(N)] (float2: max, sum of
// exp(logit - max)) and the target logit tgt[m]; no logits are stored.
bool head_lse_fused(bool bf16, int M, int K);
int head_lse_parts(int N);
void launch_head_lse(const void* X, const void* W, int M, int N, int K, const int32_t* targets, void* part,
                     float* tgt, hipStream_t s);
// loss[m] = logsumexp - target logit, from the partial states (fused head) or
// from full fp32 logits rows [M, N] (otherwise).  A target outside [0, N)
// gives NaN and ORs 1 into *flags.
void launch_loss_from_parts(const void* part, int nparts, const float* tgt, const int32_t* targets, int M,
                            int N, float* loss, uint32_t* flags, hipStream_t s);
void launch_loss_from_logits(const float* logits, const int32_t* targets, int M, int N, float* loss,
                             uint32_t* flags, hipStream_t s);

// ---------------------------------------------------------------- attention
// Causal attention for T new queries per sequence at positions l_past .. l_past+T-1
// against keys 0 .. l_past+T-1 from the K/V view; q [B, h, T, d_h];
// o [B, T, h*d_h] (act dtype).
// Prefill (bf16, d_h == 64, no past): flash kernel with MFMA.
void launch_attn_prefill_bf16(const bf16_t* q, KvView kv, bf16_t* o, int B, int H, int T, int l_past,
                              hipStream_t s);
// Row-wise kernel (any T up to 8192 keys, d_h % 4 == 0, d_h <= 128): the
// fp32 mode, and bf16 head widths other than 64 (bf16 storage, fp32 math).
void launch_attn_rows(bool bf16, const void* q, KvView kv, void* o, int B, int H, int T, int d_head, int l_past,
                      hipStream_t s);
// Single-token decode (bf16, d_h == 64): one workgroup per (sequence, head).
void launch_attn_decode_bf16(const bf16_t* q, KvView kv, bf16_t* o, int B, int H, int l_past,
                             hipStream_t s);

// ---------------------------------------------------------------- generation
// next_ids[b] = out[b * out_stride + step] = argmax_n logits[b, n] (lowest
// index among equal maxima), for b < B.
void launch_argmax_rows(const float* logits, int B, int V, int32_t* next_ids, int32_t* out, int out_stride,
                        int step, hipStream_t s);
// The same choice without the logits (bf16, M <= 64, K % 64 == 0): the head
// product X [M, K] against W [N, K] reduces each tile to per-row (value,
// column) partials part [M][head_argmax_parts(N)] (float2, column as bits),
// then launch_argmax_parts picks each row's best.
bool head_argmax_fused(bool bf16, int M, int K);
int head_argmax_parts(int N);
void launch_head_argmax(const void* X, const void* W, int M, int N, int K, void* part, hipStream_t s);
void launch_argmax_parts(const void* part, int nparts, int B, int V, int32_t* next_ids, int32_t* out,
                         int out_stride, int step, hipStream_t s);

}  // namespace gpt2

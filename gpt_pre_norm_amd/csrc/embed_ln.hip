// Embedding gather + position add fused with the first LayerNorm, the
// wave-per-row LayerNorm, and the LayerNorm that first adds a residual
// product kept as K-range partials (decode-sized calls).
//
// Embedding: H0 = wte[id] + wpe[l_past + t] ("Full Forward Pass", How it works).
// LayerNorm: mean, biased variance of the deviations, (x - u) / sqrt(s + eps),
// then gain and bias (Open Model Atlas, norm() excerpt; "Decoder Block", How it works).
//
// Both are HBM-bound streaming kernels: 4 elements per lane per access
// (16 B fp32 / 8 B bf16), rows held in registers, no LDS.  The first block's
// LN1 runs inside the embedding kernel; every other LayerNorm (LN2, the
// later LN1s, ln_f) is a launch of the row kernel.
#include "kernels.h"

namespace gpt2 {

// One row per wave; each lane holds NV groups of 4 elements (d <= 256 * NV).
// One-wave workgroups: the measured fastest launch shape for 8192 rows of 768.
template <typename Tin, typename Tact, int NV>
__global__ __launch_bounds__(64) void layernorm_kernel(const Tin* __restrict__ x,
                                                       const Tact* __restrict__ g,
                                                       const Tact* __restrict__ b,
                                                       Tact* __restrict__ y, int M, int d,
                                                       float eps) {
  const int row = blockIdx.x;
  if (row >= M) return;
  ln_row_wave<NV>(x + (long long)row * d, g, b, y + (long long)row * d, d, eps, threadIdx.x);
}

// Embedding and the first block's LayerNorm in one pass, one row per wave:
// x = wte[id] + wpe[l_past + t] (fp32, kept for the residual stream), then
// a = LN(x).  A bad id gives a zero row and raises the device flag.
template <typename Tw, int NV>
__global__ __launch_bounds__(64) void embed_ln_kernel(const int32_t* __restrict__ ids,
                                                      const Tw* __restrict__ wte,
                                                      const Tw* __restrict__ wpe, float* __restrict__ x,
                                                      const Tw* __restrict__ g, const Tw* __restrict__ bb,
                                                      Tw* __restrict__ a, int M, int T, int l_past, int d,
                                                      int n_vocab, float eps, uint32_t* flags) {
  const int m = blockIdx.x, lane = threadIdx.x;
  if (m >= M) return;
  const int id = ids[m];
  const bool ok = id >= 0 && id < n_vocab;
  if (!ok && lane == 0) atomicOr(flags, 1u);
  const int pos = l_past + m % T;
  float* xr = x + (long long)m * d;
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (lane + 64 * i) * 4;
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < d) {
      if (ok) {
        const float4 e = load4(wte + (long long)id * d + c), p = load4(wpe + (long long)pos * d + c);
        v[i] = make_float4(e.x + p.x, e.y + p.y, e.z + p.z, e.w + p.w);
      }
      store4(xr + c, v[i]);
    }
  }
  ln_row_regs<NV>(v, g, bb, a + (long long)m * d, d, eps, lane);
}

void launch_embed_ln(bool bf16, const int32_t* ids, const void* wte, const void* wpe, float* x,
                     const void* g, const void* b, void* a, int M, int T, int l_past, int d, int n_vocab,
                     float eps, uint32_t* flags, hipStream_t s) {
  const int nv = (d + 255) / 256;
#define GPT2_ELN_CASE(N)                                                                               \
  case N:                                                                                              \
    if (bf16)                                                                                          \
      embed_ln_kernel<bf16_t, N><<<M, 64, 0, s>>>(ids, (const bf16_t*)wte, (const bf16_t*)wpe, x,      \
                                                   (const bf16_t*)g, (const bf16_t*)b, (bf16_t*)a, M, T, \
                                                   l_past, d, n_vocab, eps, flags);                     \
    else                                                                                               \
      embed_ln_kernel<float, N><<<M, 64, 0, s>>>(ids, (const float*)wte, (const float*)wpe, x,         \
                                                  (const float*)g, (const float*)b, (float*)a, M, T,     \
                                                  l_past, d, n_vocab, eps, flags);                      \
    break;
  switch (nv) {
    GPT2_ELN_CASE(1) GPT2_ELN_CASE(2) GPT2_ELN_CASE(3) GPT2_ELN_CASE(4)
    GPT2_ELN_CASE(5) GPT2_ELN_CASE(6) GPT2_ELN_CASE(7) GPT2_ELN_CASE(8)
    default: break;  // d <= 2048 is enforced by the caller
  }
#undef GPT2_ELN_CASE
}

// The residual update of a product kept as K-range partials, then the
// LayerNorm of the updated row: x = x + ((bias + p_0) + p_1 + ...) in range
// order (the same order on every run), stored back, then a = LN(x).
template <int NV>
__global__ __launch_bounds__(64) void layernorm_reduce_kernel(float* __restrict__ x, const float* __restrict__ part,
                                                              int S, long long sstride,
                                                              const bf16_t* __restrict__ bias,
                                                              const bf16_t* __restrict__ g,
                                                              const bf16_t* __restrict__ b, bf16_t* __restrict__ a,
                                                              int M, int d, float eps) {
  const int row = blockIdx.x, lane = threadIdx.x;
  if (row >= M) return;
  float* xr = x + (long long)row * d;
  const float* pr = part + (long long)row * d;
  float4 v[NV];
  // t = bias, then the partials added four ranges at a time: the four loads
  // of a group are issued together (one memory round trip per group)
  float4 t[NV], r[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min((lane + 64 * i) * 4, d - 4);
    t[i] = load4(bias + c);
    r[i] = load4(xr + c);
  }
  for (int s0 = 0; s0 < S; s0 += 4) {
    float4 u[4][NV];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int c = min((lane + 64 * i) * 4, d - 4);
        u[j][i] = s0 + j < S ? load4(pr + (s0 + j) * sstride + c) : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < NV; ++i)
        if (s0 + j < S)
          t[i] = make_float4(t[i].x + u[j][i].x, t[i].y + u[j][i].y, t[i].z + u[j][i].z, t[i].w + u[j][i].w);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (lane + 64 * i) * 4;
    v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (c < d) {
      v[i] = make_float4(r[i].x + t[i].x, r[i].y + t[i].y, r[i].z + t[i].z, r[i].w + t[i].w);
      store4(xr + c, v[i]);
    }
  }
  ln_row_regs<NV>(v, g, b, a + (long long)row * d, d, eps, lane);
}

void launch_layernorm_reduce(float* x, const float* part, int S, const void* bias, const void* g, const void* b,
                             void* a, int M, int d, float eps, hipStream_t s) {
  const int nv = (d + 255) / 256;
  const long long ss = (long long)M * d;
#define GPT2_LNR_CASE(N)                                                                                 \
  case N:                                                                                                \
    layernorm_reduce_kernel<N><<<M, 64, 0, s>>>(x, part, S, ss, (const bf16_t*)bias, (const bf16_t*)g,   \
                                                (const bf16_t*)b, (bf16_t*)a, M, d, eps);                \
    break;
  switch (nv) {
    GPT2_LNR_CASE(1) GPT2_LNR_CASE(2) GPT2_LNR_CASE(3) GPT2_LNR_CASE(4)
    GPT2_LNR_CASE(5) GPT2_LNR_CASE(6) GPT2_LNR_CASE(7) GPT2_LNR_CASE(8)
    default: break;  // d <= 2048 is enforced by the caller
  }
#undef GPT2_LNR_CASE
}

template <typename Tin, typename Tact>
static void ln_dispatch(const void* x, const void* g, const void* b, void* y, int M, int d, float eps,
                        hipStream_t s) {
  const int nv = (d + 255) / 256;
#define GPT2_LN_CASE(N)                                                                  \
  case N:                                                                                \
    layernorm_kernel<Tin, Tact, N><<<M, 64, 0, s>>>((const Tin*)x, (const Tact*)g,       \
                                                     (const Tact*)b, (Tact*)y, M, d, eps); \
    break;
  switch (nv) {
    GPT2_LN_CASE(1) GPT2_LN_CASE(2) GPT2_LN_CASE(3) GPT2_LN_CASE(4)
    GPT2_LN_CASE(5) GPT2_LN_CASE(6) GPT2_LN_CASE(7) GPT2_LN_CASE(8)
    default: break;  // d <= 2048 is enforced by the caller
  }
#undef GPT2_LN_CASE
}

void launch_layernorm(bool x_f32, bool act_bf16, const void* x, const void* g, const void* b,
                      void* y, int M, int d, float eps, hipStream_t s) {
  if (act_bf16) {
    if (x_f32) ln_dispatch<float, bf16_t>(x, g, b, y, M, d, eps, s);
    else ln_dispatch<bf16_t, bf16_t>(x, g, b, y, M, d, eps, s);
  } else {
    ln_dispatch<float, float>(x, g, b, y, M, d, eps, s);
  }
}

}  // namespace gpt2

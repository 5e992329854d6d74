// Shared device helpers for the gfx950 kernels: bf16 conversions, vector
// types for the MFMA builtins, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bfloat16 storage (bit pattern)

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// f32x4 at 4-byte alignment (gfx9 vector memory accepts dword-aligned dwordx4)
typedef __attribute__((__vector_size__(4 * sizeof(float)), __aligned__(4))) float f32x4u_t;

#define GPT2_DEV __device__ __forceinline__
// for lambdas whose reference-captured register arrays must not go to memory
#define GPT2_INLINE __attribute__((always_inline))

GPT2_DEV float bf2f(bf16_t b) { return __uint_as_float((uint32_t)b << 16); }

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;

// Two fp32 -> packed bf16 (a in the low half), round to nearest even, with the
// gfx950 conversion instruction v_cvt_pk_bf16_f32.
GPT2_DEV uint32_t pack_bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// fp32 -> bf16, round to nearest even.
GPT2_DEV bf16_t f2bf(float f) { return (bf16_t)(pack_bf2(f, 0.f) & 0xFFFFu); }

// Low/high bf16 of a packed pair, as fp32.
GPT2_DEV float bf_lo(uint32_t u) { return __uint_as_float(u << 16); }
GPT2_DEV float bf_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

template <typename T> struct ActT;
template <> struct ActT<float> {
  static GPT2_DEV float load(const float* p) { return *p; }
  static GPT2_DEV void store(float* p, float v) { *p = v; }
};
template <> struct ActT<bf16_t> {
  static GPT2_DEV float load(const bf16_t* p) { return bf2f(*p); }
  static GPT2_DEV void store(bf16_t* p, float v) { *p = f2bf(v); }
};

// 16 bytes read with the non-temporal (streaming) cache policy: for data
// that is read once per call, so that it does not push data that later
// kernels re-read out of the caches.
GPT2_DEV uint4 load16_nt(const void* p) {
  return __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p)));
}

// Four consecutive elements <-> float4 (16 B for fp32, 8 B for bf16).
GPT2_DEV float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
GPT2_DEV float4 load4(const bf16_t* p) {
  uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y));
}

// Four elements as they come from memory, widened to fp32 only where they are
// used: a load whose result is not touched right away does not stall the wave.
template <typename T>
struct Raw4;
template <>
struct Raw4<float> {
  using type = float4;
};
template <>
struct Raw4<bf16_t> {
  using type = uint2;
};
GPT2_DEV float4 load4_raw(const float* p) { return *reinterpret_cast<const float4*>(p); }
GPT2_DEV uint2 load4_raw(const bf16_t* p) { return *reinterpret_cast<const uint2*>(p); }
GPT2_DEV float4 widen4(float4 v) { return v; }
GPT2_DEV float4 widen4(uint2 u) { return make_float4(bf_lo(u.x), bf_hi(u.x), bf_lo(u.y), bf_hi(u.y)); }
GPT2_DEV void store4(float* p, float4 v) { *reinterpret_cast<float4*>(p) = v; }
GPT2_DEV void store4(bf16_t* p, float4 v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf2(v.x, v.y), pack_bf2(v.z, v.w));
}

// Cross-lane data movement without LDS. DPP (a VALU operand modifier) moves
// values inside each row of 16 lanes; v_permlane16_swap / v_permlane32_swap
// exchange whole rows / halves of the wave. A ds_bpermute-based shuffle
// costs an LDS round trip per step instead.
template <int CTRL>
GPT2_DEV float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]: lane i <- i ^ 1
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]: lane i <- i ^ 2
constexpr int kDppHalfMirror = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int kDppRor8 = 0x128;        // lane i <- i ^ 8 within each 16 lanes

// Both orders of (lane's own row, partner row), for rows 16 apart (R = 16)
// or halves 32 apart (R = 32): every lane receives {value of the even
// row/half, value of the odd row/half}, so op(first, second) takes the same
// operands in the same order in both partners.
template <int R>
GPT2_DEV void row_pair(float v, float& first, float& second) {
  static_assert(R == 16 || R == 32, "row distance");
  const unsigned u = __float_as_uint(v);
  if constexpr (R == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    first = __uint_as_float(p[0]);
    second = __uint_as_float(p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    first = __uint_as_float(p[0]);
    second = __uint_as_float(p[1]);
  }
}

// op of a lane's value and the value 32 lanes away (the same in both lanes)
template <typename Op>
GPT2_DEV float halves(float v, Op op) {
  float a, b;
  row_pair<32>(v, a, b);
  return op(a, b);
}
GPT2_DEV float halves_sum(float v) {
  return halves(v, [](float x, float y) { return x + y; });
}
GPT2_DEV float halves_max(float v) {
  return halves(v, [](float x, float y) { return fmaxf(x, y); });
}

// Sum of v over each group of 8 lanes, returned to all 8: two exact xor
// steps, then the mirror within 8 lanes (exact here because all four lanes
// of each quad already hold the same value).
GPT2_DEV float sum8(float v) {
  v += dpp<kDppXor1>(v);
  v += dpp<kDppXor2>(v);
  return v + dpp<kDppHalfMirror>(v);
}

// Reduction over the 64 lanes with a commutative op, returned to every lane.
template <typename Op>
GPT2_DEV float wave_reduce(float v, Op op) {
  v = op(v, dpp<kDppXor1>(v));
  v = op(v, dpp<kDppXor2>(v));
  v = op(v, dpp<kDppHalfMirror>(v));
  v = op(v, dpp<kDppRor8>(v));
  float a, b;
  row_pair<16>(v, a, b);
  v = op(a, b);
  row_pair<32>(v, a, b);
  return op(a, b);
}
// The same over a pair of values: op(x, y, x2, y2) folds state (x2, y2) into
// (x, y). Integers travel as their bit patterns.
template <typename Op>
GPT2_DEV void wave_reduce2(float& x, float& y, Op op) {
  op(x, y, dpp<kDppXor1>(x), dpp<kDppXor1>(y));
  op(x, y, dpp<kDppXor2>(x), dpp<kDppXor2>(y));
  op(x, y, dpp<kDppHalfMirror>(x), dpp<kDppHalfMirror>(y));
  op(x, y, dpp<kDppRor8>(x), dpp<kDppRor8>(y));
  float xb, yb;
  row_pair<16>(x, x, xb);
  row_pair<16>(y, y, yb);
  op(x, y, xb, yb);
  row_pair<32>(x, x, xb);
  row_pair<32>(y, y, yb);
  op(x, y, xb, yb);
}
GPT2_DEV float wave_sum(float v) {
  return wave_reduce(v, [](float x, float y) { return x + y; });
}
GPT2_DEV float wave_max(float v) {
  return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

// LayerNorm of one row by one wave ("GPT-2 Transformer block", norm()
// excerpt): mean, biased variance of the deviations (two passes over the row
// held in registers), (x - mean) / sqrt(var + eps), then gain and bias.
// Lane l holds elements 4(l + 64 i) .. +3, i < NV (zeros past d); requires
// d <= 256 NV, d % 4 == 0.
template <int NV, typename Tact>
GPT2_DEV void ln_row_regs(const float4 (&v)[NV], const Tact* __restrict__ g, const Tact* __restrict__ b,
                          Tact* __restrict__ yr, int d, float eps, int lane) {
  // gain and bias first: their loads overlap the row's reductions
  typename Raw4<Tact>::type graw[NV], braw[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = min((lane + 64 * i) * 4, d - 4);
    graw[i] = load4_raw(g + c);
    braw[i] = load4_raw(b + c);
  }
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) sum += (v[i].x + v[i].y) + (v[i].z + v[i].w);
  const float inv_d = 1.0f / (float)d;
  const float mean = wave_sum(sum) * inv_d;
  float sq = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (lane + 64 * i) * 4;
    if (c < d) {
      const float a0 = v[i].x - mean, a1 = v[i].y - mean, a2 = v[i].z - mean, a3 = v[i].w - mean;
      sq += (a0 * a0 + a1 * a1) + (a2 * a2 + a3 * a3);
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(sq) * inv_d + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (lane + 64 * i) * 4;
    if (c < d) {
      const float4 gg = widen4(graw[i]), bb = widen4(braw[i]);
      store4(yr + c, make_float4((v[i].x - mean) * rstd * gg.x + bb.x, (v[i].y - mean) * rstd * gg.y + bb.y,
                                 (v[i].z - mean) * rstd * gg.z + bb.z, (v[i].w - mean) * rstd * gg.w + bb.w));
    }
  }
}

template <int NV, typename Tin, typename Tact>
GPT2_DEV void ln_row_wave(const Tin* __restrict__ xr, const Tact* __restrict__ g, const Tact* __restrict__ b,
                          Tact* __restrict__ yr, int d, float eps, int lane) {
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = (lane + 64 * i) * 4;
    v[i] = c < d ? load4(xr + c) : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  ln_row_regs<NV>(v, g, b, yr, d, eps, lane);
}

// GELU, tanh approximation: 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated through the identity 1 + tanh(u) = 2 / (1 + exp(-2u)), i.e.
// x / (1 + 2^(-2u log2 e)), with the hardware exp2 and reciprocal (about 1 ulp
// each).  Large |u| saturates correctly: exp2 -> inf gives 0, exp2 -> 0 gives x.
GPT2_DEV float gelu_tanh(float x) {
  // -2 u log2(e) = x (c1 + c2 x^2), c1 = -2 log2(e) sqrt(2/pi), c2 = 0.044715 c1
  const float c1 = -2.0f * 1.4426950408889634f * 0.7978845608028654f;
  const float c2 = 0.044715f * c1;
  return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(x * fmaf(c2, x * x, c1)));
}

// Unsigned division by a run-time constant d >= 1 with a precomputed
// multiplier (round-up method): n / d = (umulhi(n, mul) + n) >> shift for
// every 31-bit n.
struct FastDiv {
  uint32_t mul, shift, d;
  static FastDiv make(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << s) - d)) / d + 1);
    return f;
  }
  GPT2_DEV uint32_t div(uint32_t n) const { return (__umulhi(n, mul) + n) >> shift; }
};

// Strided view of a K/V store: element (b, kv, h, pos, j) lives at
//   base + b*sb + kv*skv + h*sh + pos*d_h + j
// Covers the cache [B, L, 2, h, cap, d_h] (base offset by the layer) and the
// block-mode present [B, 2, h, T, d_h].
struct KvView {
  void* base;
  long long sb, skv, sh;
};

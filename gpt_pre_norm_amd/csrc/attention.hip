// Causal multi-head scaled dot-product attention.
//
// Query i of a sequence sits at absolute position l_past + i and sees keys
// 0 .. l_past + i; scores are scaled by 1/sqrt(d_h) and normalised with a
// softmax ("GPT-2 Block - TorchCode", Reference Solution; "Full Forward Pass",
// How it works, for the cache offset).
//
// Three kernels:
//  * attn_prefill_bf16: flash-style, 128 queries per workgroup (32 per wave),
//    64-key K/V tiles staged through LDS (double buffered), online softmax in
//    fp32 with exp2, MFMA 32x32x16 bf16 for Q K^T and P V.  Key tiles past the
//    causal frontier are never loaded; tiles entirely above a wave's queries
//    are skipped by that wave; only diagonal tiles apply the mask.
//  * attn_rows_f32: one wave per query row with a full (max-subtracted)
//    softmax, for the fp32 mode.
//  * attn_decode_bf16: one new query per (sequence, head) streaming the cache
//    with one 16-wave workgroup per (sequence, head); the waves' online
//    softmax states merge in LDS.
#include "kernels.h"

namespace gpt2 {

static constexpr float kLog2e = 1.4426950408889634f;

// ================================================================ prefill (bf16, d_h = 64)
// MFMA v_mfma_f32_32x32x16_bf16 throughout.  A wave owns 32 queries; per 64-key
// tile it computes S^T = K Q^T (keys on the MFMA rows, queries on the columns,
// so each lane holds 32 scores of one query), runs the online softmax in fp32
// with exp2, and accumulates O^T += V^T P^T.  The P fragment is the S fragment
// converted to bf16 in place: within a 16-key MFMA step, lane half kh supplies
// keys {4kh..4kh+3, 8+4kh..8+4kh+3}, and the V^T operand is read with the same
// key order, so P never leaves registers.
//
// LDS: K tile [64 keys][64 d] with 16-byte chunks XOR-swizzled by (row>>1)&7;
// V^T tile [64 d][64 keys] with 8-byte key quads XOR-swizzled by (d>>1)&15.
// Both swizzles make the fragment reads conflict-free.  Double buffered.
GPT2_DEV int vt_swz(int d) { return (d >> 1) & 15; }

__global__ __launch_bounds__(256) void attn_prefill_bf16_kernel(const bf16_t* __restrict__ q,
                                                                KvView kv, bf16_t* __restrict__ o,
                                                                int H, int T, int l_past, int nqb) {
  constexpr int D = 64;
  __shared__ uint4 ks[2][64 * 8];      // K tile, 16-byte chunks
  __shared__ uint2 vt[2][64 * 16];     // V^T tile, 8-byte key quads

  const int qb = nqb - 1 - (int)blockIdx.y;  // longest rows first
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5;

  const int q0 = qb * 128;
  const int qw0 = q0 + wave * 32;                       // this wave's first query (relative)
  const int kend = l_past + min(q0 + 128, T);           // keys needed by the workgroup
  const int nkb = (kend + 63) / 64;
  const int wave_last = l_past + min(qw0 + 31, T - 1);  // last position this wave needs
  const int qpos = l_past + qw0 + l32;                  // this lane's query position

  const bf16_t* kbase = (const bf16_t*)kv.base + b * kv.sb + h * kv.sh;
  const bf16_t* vbase = kbase + kv.skv;
  const bf16_t* qbase = q + (long long)bh * T * D;

  // Q^T fragments (MFMA B operand): query qw0 + l32, dims 16*ds + 8*kh .. +7
  bf16x8_t qf[4];
  {
    const int t = min(qw0 + l32, T - 1);
#pragma unroll
    for (int ds = 0; ds < 4; ++ds)
      qf[ds] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(qbase + (long long)t * D + 16 * ds + 8 * kh));
  }

  // loader mapping: K rows tid>>3 (+32), chunk tid&7; V key pair tid>>3, dims 8*(tid&7)
  const int lr = tid >> 3, lc = tid & 7;
  uint4 rk[2], rv[2];
  auto gload = [&](int kb) {
    const int key0 = kb * 64;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int key = min(key0 + lr + 32 * i, kend - 1);
      rk[i] = *reinterpret_cast<const uint4*>(kbase + (long long)key * D + lc * 8);
      const int vkey = min(key0 + 2 * lr + i, kend - 1);
      rv[i] = *reinterpret_cast<const uint4*>(vbase + (long long)vkey * D + lc * 8);
    }
  };
  auto lstore = [&](int st) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = lr + 32 * i;
      ks[st][r * 8 + (lc ^ ((r >> 1) & 7))] = rk[i];
    }
    // transpose keys (2*lr, 2*lr+1) x dims 8*lc..8*lc+7 into V^T
    const uint32_t a[4] = {rv[0].x, rv[0].y, rv[0].z, rv[0].w};
    const uint32_t c[4] = {rv[1].x, rv[1].y, rv[1].z, rv[1].w};
    const int kq = lr >> 1, half = lr & 1;
    uint32_t* vt32 = reinterpret_cast<uint32_t*>(vt[st]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = lc * 8 + e;
      const uint32_t lo = (e & 1) ? (a[e >> 1] >> 16) : (a[e >> 1] & 0xFFFFu);
      const uint32_t hi = (e & 1) ? (c[e >> 1] >> 16) : (c[e >> 1] & 0xFFFFu);
      vt32[(d * 16 + (kq ^ vt_swz(d))) * 2 + half] = lo | (hi << 16);
    }
  };

  f32x16_t oacc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float sc = 0.125f * kLog2e;  // 1/sqrt(64), in the log2 domain

  gload(0);
  lstore(0);
  __syncthreads();
  for (int kb = 0; kb < nkb; ++kb) {
    const bool more = kb + 1 < nkb;
    if (more) gload(kb + 1);
    const int st = kb & 1;
    const int key0 = kb * 64;
    if (key0 <= wave_last) {
      // ---- S^T for 2 x 32 keys
      f32x16_t s[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kk][r] = 0.f;
        const int row = kk * 32 + l32;
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          const int chunk = 2 * ds + kh;
          const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, ks[st][row * 8 + (chunk ^ ((row >> 1) & 7))]);
          s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[kk], 0, 0, 0);
        }
      }
      // ---- mask (diagonal tiles only) and online softmax; lane's keys:
      // key0 + 32*kk + 8*(r/4) + 4*kh + r%4
      const bool need_mask = key0 + 63 > l_past + qw0;
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[kk][r] * sc;
          if (need_mask && key0 + 32 * kk + 8 * (r >> 2) + 4 * kh + (r & 3) > qpos) v = -INFINITY;
          s[kk][r] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mnew = fmaxf(mrun, mx);
      const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
      mrun = mnew;
      float ls = 0.f;
      bf16x8_t pf[4];  // 16-key MFMA steps
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(s[kk][r] - mnew);
          ls += p[r];
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const float* pp = p + 8 * hs;
          pf[2 * kk + hs] = __builtin_bit_cast(
              bf16x8_t, make_uint4(pack_bf2(pp[0], pp[1]), pack_bf2(pp[2], pp[3]), pack_bf2(pp[4], pp[5]),
                                   pack_bf2(pp[6], pp[7])));
        }
      }
      lrun = lrun * alpha + ls;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      // ---- O^T += V^T P^T over 4 steps of 16 keys
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const int d = db * 32 + l32;
        const uint2* vrow = &vt[st][d * 16];
#pragma unroll
        for (int ksx = 0; ksx < 4; ++ksx) {
          const uint2 x1 = vrow[(4 * ksx + kh) ^ vt_swz(d)];
          const uint2 x2 = vrow[(4 * ksx + 2 + kh) ^ vt_swz(d)];
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(x1.x, x1.y, x2.x, x2.y));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ksx], oacc[db], 0, 0, 0);
        }
      }
    }
    if (more) lstore((kb + 1) & 1);
    __syncthreads();
  }

  // ---- normalise and store O [B, T, H*64]; lane holds query qw0 + l32 and
  // dims 32*db + 8*(r/4) + 4*kh + r%4
  float l = lrun + __shfl_xor(lrun, 32, 64);
  const float inv = 1.0f / l;
  const int t = qw0 + l32;
  if (t < T) {
    bf16_t* orow = o + ((long long)b * T + t) * (H * D) + h * D;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const f32x16_t& v = oacc[db];
        store4(orow + db * 32 + 8 * g4 + 4 * kh,
               make_float4(v[4 * g4] * inv, v[4 * g4 + 1] * inv, v[4 * g4 + 2] * inv, v[4 * g4 + 3] * inv));
      }
  }
}

void launch_attn_prefill_bf16(const bf16_t* q, KvView kv, bf16_t* o, int B, int H, int T, int l_past,
                              hipStream_t s) {
  const int nqb = (T + 127) / 128;
  dim3 grid(B * H, nqb);
  attn_prefill_bf16_kernel<<<grid, 256, 0, s>>>(q, kv, o, H, T, l_past, nqb);
}

// ================================================================ row-wise (fp32)
// One wave per query row: scores into LDS, row max, exp, sum, then lanes over
// the head dimension accumulate p_j v_j and divide by the sum.
__global__ __launch_bounds__(256) void attn_rows_f32_kernel(const float* __restrict__ q, KvView kv,
                                                            float* __restrict__ o, int B, int H, int T,
                                                            int dh, int l_past, int maxk) {
  extern __shared__ float sbuf[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wave;
  const bool active = row < (long long)B * H * T;
  float* s = sbuf + wave * maxk;
  int t = 0, b = 0, h = 0, nk = 0;
  const float *qv = nullptr, *kb = nullptr, *vb = nullptr;
  float m = -INFINITY, l = 0.f;
  if (active) {
    t = (int)(row % T);
    const int bh = (int)(row / T);
    b = bh / H;
    h = bh - b * H;
    nk = l_past + t + 1;
    qv = q + row * dh;
    kb = (const float*)kv.base + b * kv.sb + h * kv.sh;
    vb = kb + kv.skv;
    const float scale = 1.0f / sqrtf((float)dh);
    for (int j = lane; j < nk; j += 64) {
      const float* kr = kb + (long long)j * dh;
      float acc = 0.f;
      for (int c = 0; c < dh; c += 4) {
        const float4 a = *reinterpret_cast<const float4*>(qv + c);
        const float4 k4 = *reinterpret_cast<const float4*>(kr + c);
        acc = fmaf(a.x, k4.x, acc);
        acc = fmaf(a.y, k4.y, acc);
        acc = fmaf(a.z, k4.z, acc);
        acc = fmaf(a.w, k4.w, acc);
      }
      const float v = acc * scale;
      s[j] = v;
      m = fmaxf(m, v);
    }
  }
  m = wave_max(m);
  if (active) {
    for (int j = lane; j < nk; j += 64) {
      const float p = expf(s[j] - m);
      s[j] = p;
      l += p;
    }
  }
  l = wave_sum(l);
  __syncthreads();
  if (active) {
    const float inv = 1.0f / l;
    float* orow = o + ((long long)b * T + t) * (H * dh) + h * dh;
    for (int c = lane; c < dh; c += 64) {
      float acc = 0.f;
      for (int j = 0; j < nk; ++j) acc = fmaf(s[j], vb[(long long)j * dh + c], acc);
      orow[c] = acc * inv;
    }
  }
}

void launch_attn_rows_f32(const float* q, KvView kv, float* o, int B, int H, int T, int d_head,
                          int l_past, hipStream_t s) {
  const long long rows = (long long)B * H * T;
  const int maxk = l_past + T;
  const int blocks = (int)((rows + 3) / 4);
  attn_rows_f32_kernel<<<blocks, 256, 4 * maxk * sizeof(float), s>>>(q, kv, o, B, H, T, d_head,
                                                                     l_past, maxk);
}

// ================================================================ decode (bf16, d_h = 64)
// One workgroup of 16 waves per (sequence, head) streams the whole cache row
// range 0 .. l_past: wave w takes keys w*64 + 1024*j.  Inside a wave, 8 lanes
// share a key row (8 dims each) and 8 rows are in flight per pass; a lane
// issues its 8 K and 8 V row loads together (256 KB in flight per workgroup).
// Each wave keeps an online softmax (running max, partial sums per lane);
// the 16 waves then merge through LDS, so no second kernel is needed.
static constexpr int kDecWaves = 16;

__global__ __launch_bounds__(1024) void attn_decode_bf16_kernel(const bf16_t* __restrict__ q, KvView kv,
                                                                bf16_t* __restrict__ o, int H, int nk) {
  constexpr int D = 64;
  __shared__ float wm[kDecWaves];
  __shared__ float wl[kDecWaves];
  __shared__ float wo[kDecWaves][D];
  const int bh = blockIdx.x;
  const int b = bh / H, h = bh - (bh / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int c8 = lane & 7, rg = lane >> 3;

  const bf16_t* kbase = (const bf16_t*)kv.base + b * kv.sb + h * kv.sh;
  const bf16_t* vbase = kbase + kv.skv;
  const uint4 qu = *reinterpret_cast<const uint4*>(q + (long long)bh * D + c8 * 8);
  const float qv[8] = {bf_lo(qu.x), bf_hi(qu.x), bf_lo(qu.y), bf_hi(qu.y),
                       bf_lo(qu.z), bf_hi(qu.z), bf_lo(qu.w), bf_hi(qu.w)};
  const float sc = 0.125f * kLog2e;  // 1/sqrt(64), in the log2 domain

  float m = -INFINITY, l = 0.f;
  float ov[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int key0 = wave * 64; key0 < nk; key0 += 64 * kDecWaves) {
    uint4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int key = min(key0 + rg + 8 * i, nk - 1);
      kr[i] = *reinterpret_cast<const uint4*>(kbase + (long long)key * D + c8 * 8);
      vr[i] = *reinterpret_cast<const uint4*>(vbase + (long long)key * D + c8 * 8);
    }
    float sv[8];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint4 u = kr[i];
      float acc = qv[0] * bf_lo(u.x);
      acc = fmaf(qv[1], bf_hi(u.x), acc);
      acc = fmaf(qv[2], bf_lo(u.y), acc);
      acc = fmaf(qv[3], bf_hi(u.y), acc);
      acc = fmaf(qv[4], bf_lo(u.z), acc);
      acc = fmaf(qv[5], bf_hi(u.z), acc);
      acc = fmaf(qv[6], bf_lo(u.w), acc);
      acc = fmaf(qv[7], bf_hi(u.w), acc);
      acc += __shfl_xor(acc, 1, 64);
      acc += __shfl_xor(acc, 2, 64);
      acc += __shfl_xor(acc, 4, 64);
      sv[i] = key0 + rg + 8 * i < nk ? acc * sc : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 8, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mnew = fmaxf(m, mx);  // finite: key0 < nk, so row rg=0, i=0 is a real key
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] *= alpha;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(sv[i] - mnew);  // 0 for masked keys
      l += p;
      const uint4 u = vr[i];
      ov[0] = fmaf(p, bf_lo(u.x), ov[0]);
      ov[1] = fmaf(p, bf_hi(u.x), ov[1]);
      ov[2] = fmaf(p, bf_lo(u.y), ov[2]);
      ov[3] = fmaf(p, bf_hi(u.y), ov[3]);
      ov[4] = fmaf(p, bf_lo(u.z), ov[4]);
      ov[5] = fmaf(p, bf_hi(u.z), ov[5]);
      ov[6] = fmaf(p, bf_lo(u.w), ov[6]);
      ov[7] = fmaf(p, bf_hi(u.w), ov[7]);
    }
  }
  // sum the 8 row groups (each key's p is replicated over the 8 lanes of its row)
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
    l += __shfl_xor(l, off, 64);
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] += __shfl_xor(ov[e], off, 64);
  }
  if (lane < 8) {
#pragma unroll
    for (int e = 0; e < 8; ++e) wo[wave][lane * 8 + e] = ov[e];
  }
  if (lane == 0) {
    wm[wave] = m;  // -inf for a wave that had no keys
    wl[wave] = l;
  }
  __syncthreads();
  if (tid < D) {
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) M = fmaxf(M, wm[w]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w] - M);
      L = fmaf(wl[w], f, L);
      acc = fmaf(wo[w][tid], f, acc);
    }
    o[(long long)b * H * D + h * D + tid] = f2bf(acc / L);
  }
}

void launch_attn_decode_bf16(const bf16_t* q, KvView kv, bf16_t* o, int B, int H, int l_past,
                             hipStream_t s) {
  attn_decode_bf16_kernel<<<B * H, 64 * kDecWaves, 0, s>>>(q, kv, o, H, l_past + 1);
}

}  // namespace gpt2

// Causal multi-head scaled dot-product attention.
//
// Query i of a sequence sits at absolute position l_past + i and sees keys
// 0 .. l_past + i; scores are scaled by 1/sqrt(d_h) and normalised with a
// softmax ("GPT-2 Block - TorchCode", Reference Solution; "Full Forward Pass",
// How it works, for the cache offset).
//
// Three kernels:
//  * attn_prefill_bf16: flash-style, 128 queries per workgroup (32 per wave),
//    64-key K and V^T tiles moved to LDS by DMA through a 2-stage ring, online
//    softmax in fp32 with exp2, MFMA 32x32x16 bf16 for Q K^T and P V.  Key tiles past the
//    causal frontier are never loaded; tiles entirely above a wave's queries
//    are skipped by that wave; only diagonal tiles apply the mask.
//  * attn_rows: one wave per query row with a full (max-subtracted)
//    softmax, for the fp32 mode and for bf16 head widths other than 64.
//  * attn_decode_bf16: one new query per (sequence, head) streaming the cache
//    with one 8-wave workgroup per (sequence, head); the waves' online
//    softmax states merge in LDS.
#include "kernels.h"

namespace gpt2 {

static constexpr float kLog2e = 1.4426950408889634f;

// ================================================================ prefill (bf16, d_h = 64)
// MFMA v_mfma_f32_32x32x16_bf16 throughout.  A wave owns 32 queries; per 64-key
// tile it computes S^T = K Q^T (keys on the MFMA rows, queries on the columns,
// so each lane holds 32 scores of one query), runs the online softmax in fp32
// with exp2, and accumulates O^T += V^T P^T.
//
// Key order: the S MFMA reads K row pi(i) for its row i, pi swapping bits 2 and
// 3 of i.  A lane's score registers r = 0..15 then hold keys 16*(r/8) + 8*kh +
// r%8 of the 32-key block, so the bf16 P fragment of each 16-key P*V step is
// 8 consecutive keys per lane half: the matching V^T operand is one 16-byte
// chunk of a V^T row, and P never leaves registers.
//
// K and V tiles [64 keys][64 d] are copied from the cache rows global -> LDS
// with global_load_lds_dwordx4 through a ring of STAGES buffers, STAGES-1 tiles
// ahead.  The V^T operand is read with the gfx950 transposing LDS read
// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4k+q supplies the address
// of dims 4q..4q+3 of key k and lane i receives key 0..3 of dim i, so two such
// reads give a lane its 8 consecutive keys of one dim.  16-byte chunks are
// XOR-swizzled per row: K by (key>>1)&7 (conflict-free 16-row fragment reads),
// V by 4*((key>>1)&1) (conflict-free 4-row x 32-dim transposing reads).
// Two stages (32 KB) rather than four: three workgroups share a CU instead of
// two, which measured faster (26.5 against 28.5 us per layer at B8 T1024).
constexpr int kAttnStages = 2;
constexpr int kAttnStageU4 = 2 * 64 * 8;  // K tile + V^T tile, uint4 units

GPT2_DEV int key_perm(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int N>
GPT2_DEV void attn_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4_t;

GPT2_DEV int v_swz(int key) { return ((key >> 1) & 1) << 2; }

// Work items (head, query block) in order of decreasing length are dealt in
// rounds of one per CU slot, every other round reversed, so that the CUs
// that took the longest blocks of one round take the shortest of the next.
GPT2_DEV void attn_item(int i, int nbh, int nqb, int round, int& bh, int& qb) {
  const int total = nbh * nqb;
  const int r = i / round, p = i - r * round;
  const int chunk = min(round, total - r * round);
  const int j = r * round + ((r & 1) ? chunk - 1 - p : p);
  qb = nqb - 1 - j / nbh;
  bh = j - (j / nbh) * nbh;
}

__global__ __launch_bounds__(256) void attn_prefill_bf16_kernel(const bf16_t* __restrict__ q,
                                                                KvView kv, bf16_t* __restrict__ o,
                                                                int H, int T, int l_past, int nbh, int nqb,
                                                                int round) {
  constexpr int D = 64;
  __shared__ uint4 lds[kAttnStages * kAttnStageU4];  // 16 KB per stage

  int qb, bh;
  attn_item(blockIdx.x, nbh, nqb, round, bh, qb);
  const int b = bh / H, h = bh - (bh / H) * H;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, kh = lane >> 5;

  // queries are rows t of this call; query t sits at position l_past + t and
  // keys are cache slots (absolute positions)
  const int q0 = qb * 128;
  const int qw0 = q0 + wave * 32;                   // this wave's first query row
  const int kend = l_past + min(q0 + 128, T);       // keys needed by the workgroup
  const int nkb = (kend + 63) / 64;
  const int wave_last = l_past + min(qw0 + 31, T - 1);  // its last query's position
  const int qpos = l_past + qw0 + l32;              // this lane's query position

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

  // loads: this wave fills K and V rows 8*wave.. and 8*(wave+4).. of each
  // tile through buffer loads into LDS: the lane's byte offset within a tile
  // is fixed, the tile's offset is a scalar, and rows at or past kend read as
  // zeros (the resource ends there), which the mask then drops.
  const int lrow = lane >> 3, lpc = lane & 7;
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const __amdgpu_buffer_rsrc_t krsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)kbase, (short)0, kend * D * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)vbase, (short)0, kend * D * 2, 0x00020000);
  int koff[2], voff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int row = 8 * (wave + 4 * i) + lrow;
    koff[i] = (row * D + (lpc ^ ((row >> 1) & 7)) * 8) * 2;
    voff[i] = (row * D + (lpc ^ v_swz(row)) * 8) * 2;
  }
  auto issue = [&](int kb, int st) {
    const int tile = kb * 64 * D * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int g = wave_s + 4 * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          krsrc, (__attribute__((address_space(3))) void*)(lds + st * kAttnStageU4 + g * 64), 16, koff[i], tile, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          vrsrc, (__attribute__((address_space(3))) void*)(lds + st * kAttnStageU4 + 512 + g * 64), 16, voff[i], tile,
          0, 0);
    }
  };
  // transposing-read addresses (bytes within a V tile): lane group G = lane/16
  // holds dims 16*(G&1) (+32*db) and keys 8*(G>>1) (+16*ksx, +4 for the second read)
  const int tq = (lane & 15) & 3, tk = (lane & 15) >> 2;
  const int tdim0 = 16 * ((lane >> 4) & 1) + 4 * tq;  // + 32*db
  const int tkey0 = 8 * (lane >> 5) + tk;             // + 16*ksx (+4)
  auto tr_addr = [&](int key, int dim) {  // byte offset of (key, dims dim..dim+3)
    const int c = dim >> 3;
    return key * 128 + ((c ^ v_swz(key)) << 4) + ((dim & 4) << 1);
  };

  f32x16_t oacc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[i][r] = 0.f;
  float mrun = -INFINITY, lrun = 0.f;
  const float sc = 0.125f * kLog2e;  // 1/sqrt(64), in the log2 domain

#pragma unroll
  for (int s = 0; s < kAttnStages - 1; ++s)
    if (s < nkb) issue(s, s);

  for (int kb = 0; kb < nkb; ++kb) {
    const int ahead = min(kAttnStages - 2, nkb - 1 - kb);
    if (ahead >= 2) attn_wait_vmcnt<8>();
    else if (ahead == 1) attn_wait_vmcnt<4>();
    else attn_wait_vmcnt<0>();
    // (own loads of tile kb done; a barrier that waits only for LDS
    // instructions, as __syncthreads() would also drain the tiles in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (kb + kAttnStages - 1 < nkb) issue(kb + kAttnStages - 1, (kb + kAttnStages - 1) % kAttnStages);
    const uint4* ks = lds + (kb % kAttnStages) * kAttnStageU4;
    const uint4* vs = ks + 512;
    const int key0 = kb * 64;
    if (key0 <= wave_last) {
      // ---- S^T for 2 x 32 keys: all eight K fragments read first, then the
      // two independent accumulation chains interleaved
      f32x16_t s[2];
      bf16x8_t kfr[2][4];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int row = kk * 32 + key_perm(l32);
#pragma unroll
        for (int ds = 0; ds < 4; ++ds) {
          const int chunk = 2 * ds + kh;
          kfr[kk][ds] = __builtin_bit_cast(bf16x8_t, ks[row * 8 + (chunk ^ ((row >> 1) & 7))]);
        }
      }
      const f32x16_t zero = {};
      __builtin_amdgcn_sched_barrier(0);  // keep the eight reads ahead of the MFMAs
#pragma unroll
      for (int ds = 0; ds < 4; ++ds)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
          s[kk] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[kk][ds], qf[ds], ds == 0 ? zero : s[kk], 0, 0, 0);
      // ---- mask (diagonal tiles only) and online softmax; register r of block
      // kk holds key key0 + 32*kk + 16*(r/8) + 8*kh + r%8.  The reference max
      // mref only moves when the tile max exceeds it by more than 8 (log2
      // units): weights are then at most 2^8, exact in fp32 and in bf16's range,
      // and the O / sum rescale is skipped for most tiles.  Both use the same
      // mref, so the final O / sum is the softmax.
      if (key0 + 63 > l_past + qw0) {
        const int lim = qpos - key0 - 8 * kh;  // key offsets above lim are masked
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kk + 16 * (r >> 3) + (r & 7) > lim) s[kk][r] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kk][r]);
      mx = halves_max(mx) * sc;
      if (mx > mrun + 8.0f) {
        const float alpha = __builtin_amdgcn_exp2f(mrun - mx);  // 0 on the first tile
        mrun = mx;
        lrun *= alpha;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
      }
      float ls4[4] = {0.f, 0.f, 0.f, 0.f};  // four independent partial sums
      bf16x8_t pf[4];  // 16-key P*V steps
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(s[kk][r], sc, -mrun));
          ls4[r & 3] += p[r];
        }
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const float* pp = p + 8 * hs;
          pf[2 * kk + hs] = __builtin_bit_cast(
              bf16x8_t, make_uint4(pack_bf2(pp[0], pp[1]), pack_bf2(pp[2], pp[3]), pack_bf2(pp[4], pp[5]),
                                   pack_bf2(pp[6], pp[7])));
        }
      }
      lrun += (ls4[0] + ls4[1]) + (ls4[2] + ls4[3]);
      // ---- O^T += V^T P^T over 4 steps of 16 keys (transposing reads of V)
      const char* vbytes = reinterpret_cast<const char*>(vs);
#pragma unroll
      for (int db = 0; db < 2; ++db) {
#pragma unroll
        for (int ksx = 0; ksx < 4; ++ksx) {
          const int key = 16 * ksx + tkey0;
          const int dim = 32 * db + tdim0;
          const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vbytes + tr_addr(key, dim)));
          const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) s16x4_t*)(vbytes + tr_addr(key + 4, dim)));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ksx], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalise and store O [B, T, H*64]; lane holds query qw0 + l32 and
  // dims 32*db + 8*(r/4) + 4*kh + r%4
  const float l = halves_sum(lrun);
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
  const int n_cu = device_cu_count();
  attn_prefill_bf16_kernel<<<B * H * nqb, 256, 0, s>>>(q, kv, o, H, T, l_past, B * H, nqb, n_cu);
}

// ================================================================ row-wise (any head width)
// One wave per query row: scores into LDS, row max, exp, sum, then lanes over
// the head dimension accumulate p_j v_j and divide by the sum.  Arithmetic in
// fp32; q, K, V and o in the mode's storage type (fp32, or bf16 for head
// widths other than 64).
template <typename Tio>
__global__ __launch_bounds__(256) void attn_rows_kernel(const Tio* __restrict__ q, KvView kv, Tio* __restrict__ o,
                                                        int B, int H, int T, int dh, int l_past, int maxk) {
  extern __shared__ float sbuf[];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long row = (long long)blockIdx.x * 4 + wave;
  const bool active = row < (long long)B * H * T;
  float* s = sbuf + wave * maxk;
  int t = 0, b = 0, h = 0, nk = 0;
  const Tio *qv = nullptr, *kb = nullptr, *vb = nullptr;
  float m = -INFINITY, l = 0.f;
  if (active) {
    t = (int)(row % T);
    const int bh = (int)(row / T);
    b = bh / H;
    h = bh - b * H;
    nk = l_past + t + 1;
    qv = q + row * dh;
    kb = (const Tio*)kv.base + b * kv.sb + h * kv.sh;
    vb = kb + kv.skv;
    const float scale = 1.0f / sqrtf((float)dh);
    for (int j = lane; j < nk; j += 64) {
      const Tio* kr = kb + (long long)j * dh;
      float acc = 0.f;
      for (int c = 0; c < dh; c += 4) {
        const float4 a = load4(qv + c);
        const float4 k4 = load4(kr + c);
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
    Tio* orow = o + ((long long)b * T + t) * (H * dh) + h * dh;
    for (int c = lane; c < dh; c += 64) {
      float acc = 0.f;
      for (int j = 0; j < nk; ++j) acc = fmaf(s[j], ActT<Tio>::load(vb + (long long)j * dh + c), acc);
      ActT<Tio>::store(orow + c, acc * inv);
    }
  }
}

template <typename Tio>
static void rows_launch(const Tio* q, KvView kv, Tio* o, int B, int H, int T, int d_head, int l_past,
                        hipStream_t s) {
  const long long rows = (long long)B * H * T;
  const int maxk = l_past + T;
  const int blocks = (int)((rows + 3) / 4);
  // a row of scores per wave: 4 waves x maxk x 4 B, up to 128 KB at the
  // 8192-key limit the entry points enforce, beyond the 64 KB default
  set_dynamic_lds_limit((const void*)attn_rows_kernel<Tio>, 4 * 8192 * (int)sizeof(float));
  attn_rows_kernel<Tio><<<blocks, 256, 4 * maxk * sizeof(float), s>>>(q, kv, o, B, H, T, d_head, l_past, maxk);
}

void launch_attn_rows(bool bf16, const void* q, KvView kv, void* o, int B, int H, int T, int d_head, int l_past,
                      hipStream_t s) {
  if (bf16)
    rows_launch((const bf16_t*)q, kv, (bf16_t*)o, B, H, T, d_head, l_past, s);
  else
    rows_launch((const float*)q, kv, (float*)o, B, H, T, d_head, l_past, s);
}

// ================================================================ decode (bf16, d_h = 64)
// One workgroup of NW waves per (sequence, head) streams the whole cache row
// range 0 .. l_past: wave w takes keys [8 RP (w + NW j), +8 RP).  Inside a
// wave, 8 lanes share a key row (8 dims each); a lane issues its RP K and RP V
// row loads together (RP = 8: 16 KB in flight per wave, 100 VGPRs, so four
// waves per SIMD and every workgroup of a 768-workgroup launch resident).
// The cache rows are read once per step, with the non-temporal cache policy:
// the 2.4 GB stream then leaves the weights, which every step re-reads, in
// the last-level cache (decode step 0.825 -> 0.764 ms, attention 37.9 ->
// 34.6 us per layer, head 23.0 -> 21.0 us).
// Each wave keeps an online softmax (running max, partial sums per lane);
// the waves then merge through LDS, so no second kernel is needed.
constexpr int kDecWaves = 8, kDecRows = 8;  // measured best at 1024 keys, d_h 64

// NW waves; RP key rows per lane per pass (RP/8 passes of 8 rows); PF: the
// next pass's rows are loaded before the current pass is reduced.
template <int NW, int RP, bool PF>
__global__ __launch_bounds__(64 * NW) void attn_decode_bf16_kernel(const bf16_t* __restrict__ q, KvView kv,
                                                                   bf16_t* __restrict__ o, int H, int nk) {
  constexpr int D = 64;
  __shared__ float wm[NW];
  __shared__ float wl[NW];
  __shared__ float wo[NW][D];
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
  constexpr int KP = 8 * RP;  // keys per wave per pass
  uint4 kr[RP], vr[RP];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const int key = min(k0 + rg + 8 * i, nk - 1);
      kr[i] = load16_nt(kbase + (long long)key * D + c8 * 8);
      vr[i] = load16_nt(vbase + (long long)key * D + c8 * 8);
    }
  };
  int key0 = wave * KP;
  if (PF && key0 < nk) load(key0);
  for (; key0 < nk; key0 += KP * NW) {
    uint4 kc[RP], vc[RP];
    if constexpr (PF) {
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        kc[i] = kr[i];
        vc[i] = vr[i];
      }
      if (key0 + KP * NW < nk) load(key0 + KP * NW);
    } else {
      load(key0);
#pragma unroll
      for (int i = 0; i < RP; ++i) {
        kc[i] = kr[i];
        vc[i] = vr[i];
      }
    }
    float sv[RP];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const uint4 u = kc[i];
      float acc = qv[0] * bf_lo(u.x);
      acc = fmaf(qv[1], bf_hi(u.x), acc);
      acc = fmaf(qv[2], bf_lo(u.y), acc);
      acc = fmaf(qv[3], bf_hi(u.y), acc);
      acc = fmaf(qv[4], bf_lo(u.z), acc);
      acc = fmaf(qv[5], bf_hi(u.z), acc);
      acc = fmaf(qv[6], bf_lo(u.w), acc);
      acc = fmaf(qv[7], bf_hi(u.w), acc);
      acc = sum8(acc);
      sv[i] = key0 + rg + 8 * i < nk ? acc * sc : -INFINITY;
      mx = fmaxf(mx, sv[i]);
    }
    {  // max over the 8 row groups
      float a, b;
      mx = fmaxf(mx, dpp<kDppRor8>(mx));
      row_pair<16>(mx, a, b);
      row_pair<32>(fmaxf(a, b), a, b);
      mx = fmaxf(a, b);
    }
    const float mnew = fmaxf(m, mx);  // finite: key0 < nk, so row rg=0, i=0 is a real key
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    m = mnew;
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) ov[e] *= alpha;
#pragma unroll
    for (int i = 0; i < RP; ++i) {
      const float p = __builtin_amdgcn_exp2f(sv[i] - mnew);  // 0 for masked keys
      l += p;
      const uint4 u = vc[i];
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
  auto sum_groups = [](float v) {
    float a, b;
    v += dpp<kDppRor8>(v);
    row_pair<16>(v, a, b);
    row_pair<32>(a + b, a, b);
    return a + b;
  };
  l = sum_groups(l);
#pragma unroll
  for (int e = 0; e < 8; ++e) ov[e] = sum_groups(ov[e]);
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
    for (int w = 0; w < NW; ++w) M = fmaxf(M, wm[w]);
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(wm[w] - M);
      L = fmaf(wl[w], f, L);
      acc = fmaf(wo[w][tid], f, acc);
    }
    o[(long long)b * H * D + h * D + tid] = f2bf(acc / L);
  }
}

void launch_attn_decode_bf16(const bf16_t* q, KvView kv, bf16_t* o, int B, int H, int l_past,
                             hipStream_t s) {
  attn_decode_bf16_kernel<kDecWaves, kDecRows, false><<<B * H, 64 * kDecWaves, 0, s>>>(q, kv, o, H, l_past + 1);
}

}  // namespace gpt2

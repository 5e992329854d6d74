// Y = X W^T with fused epilogues, for the five matrix products of the decoder:
// c_attn (+bias, split into q and the K/V store), attn c_proj and mlp c_proj
// (+bias +residual), c_fc (+bias, GELU) and the tied head (wte^T, fp32 logits).
// ("Decoder Block", How it works; "Full Forward Pass", How it works.)
//
// Both operands are K-contiguous ([rows, K] row-major), the layout the MFMA
// fragments want; the W tile is the MFMA A operand and the X tile the B
// operand, so each lane's accumulators hold consecutive output columns of one
// row.  bf16 kernels, by shape:
//   * M > 64, K % 64 == 0: 128x192 tiles (the head: 256x256 when M / 32 is a
//     multiple of 256), 8 waves of
//     v_mfma_f32_32x32x16_bf16, tiles DMA'd global -> LDS with
//     global_load_lds_dwordx4 through a two-stage ring, epilogue through a
//     per-wave LDS patch so stores cover whole rows of 128 bytes;
//   * M <= 64 (decode): a weight-streaming kernel (split K into fixed-order
//     partials for the in-place residual products);
//   * otherwise: a register-staged 16x16x32 kernel.
// fp32 path: a plain LDS-tiled FMA kernel (correctness mode).
#include "kernels.h"

#include <type_traits>
#include <utility>

namespace gpt2 {

// ================================================================ epilogues
struct EpiStoreF32 {
  // Rows of the fp32 head output are only 4-byte aligned (N = n_vocab is odd),
  // so the MFMA kernel hands this epilogue one value per lane with 32
  // consecutive lanes on one row (row_store), which coalesces dword stores.
  static constexpr bool kRowStore = true;
  float* out;
  int N;
  struct Ctx {};
  GPT2_DEV Ctx load(int, int) const { return {}; }
  GPT2_DEV void store(int m, int n, f32x4_t v, Ctx) const { (*this)(m, n, v); }
  GPT2_DEV void store1(int m, int n, float v) const { out[(long long)m * N + n] = v; }
  GPT2_DEV void operator()(int m, int n, f32x4_t v) const {
    float* p = out + (long long)m * N + n;
    if (n + 3 < N) {
      *reinterpret_cast<f32x4u_t*>(p) = v;  // one dwordx4 store, 4-byte aligned
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (n + r < N) p[r] = v[r];
    }
  }
};

// The head's fp32 logits through the DMA-ring MFMA kernel, written in whole
// 128-byte lines.  Rows of [M, N] start at arbitrary 4-byte phases (N is odd),
// so plain column tiles share a partial line with their neighbours in every
// row, and partial-line writes run at well under half the write bandwidth.
// Instead the kernel's tile rows are positions in an order that groups rows by
// phase (row m = r + 32 j, r = class, in class-major order), all rows of a
// tile share one phase, and the tile's column window starts on a line boundary
// of those rows (window origin = that phase's offset + BN * (tn - 1), so one
// extra window per row block covers the leading columns).  Results are the
// same; only which tile writes which element changes.
struct EpiStoreF32Lines {
  float* out;
  int N, M;
  int q, s;  // M = 32 q + s: classes r < s hold q + 1 rows, the others q
  static EpiStoreF32Lines make(float* out, int N, int M) { return {out, N, M, M >> 5, M & 31}; }
  // row of position i in the class-major order
  GPT2_DEV int row_of(int i) const {
    const int big = s * (q + 1);
    int r, j;
    if (i < big) {
      r = i / (q + 1);
      j = i - r * (q + 1);
    } else {
      const int i2 = i - big;
      r = s + i2 / q;
      j = i2 - (r - s) * q;
    }
    return r + 32 * j;
  }
  // columns from the start of row_of(i) to its first 128-byte line boundary
  GPT2_DEV int line_offset(int i) const {
    const long long w = (long long)((uintptr_t)out >> 2) + (long long)row_of(i) * N;
    return (int)(-w & 31);
  }
  struct Ctx {};
  GPT2_DEV Ctx load(int, int) const { return {}; }
  GPT2_DEV void store(int i, int n, f32x4_t v, Ctx) const { (*this)(i, n, v); }
  GPT2_DEV void operator()(int i, int n, f32x4_t v) const { store(row(i), n, v, Ctx{}); }
  // The row of position i is found once per row a lane stores, not per
  // store (kColRow): it takes integer divisions.
  static constexpr bool kColRow = true;
  using Col = int;
  using Row = long long;  // row_of(i) * N
  GPT2_DEV Col col(int n) const { return n; }
  GPT2_DEV Row row(int i) const { return (long long)row_of(i) * N; }
  // Non-temporal stores: the logits are not read back by this kernel, and
  // kept out of the way in L2 they leave it to the X and W tiles that every
  // workgroup re-reads.
  GPT2_DEV void store(Row r, Col n, f32x4_t v, Ctx) const {
    float* p = out + r + n;
    if (n >= 0 && n + 3 < N) {
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4u_t*>(p));
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (n + k >= 0 && n + k < N) __builtin_nontemporal_store(v[k], p + k);
    }
  }
};

// The tied head without its logits: per row m and per (column tile, wave
// column) the partial log-sum-exp state (max, sum of exp(logit - max)) goes to
// part[m][slot] and the logit of the row's target column to tgt[m]; a row
// kernel combines them into the next-token cross-entropy (loss_rows_kernel).
struct EpiLoss {
  static constexpr bool kRowLse = true;
  const int32_t* targets;  // [M]
  float2* part;            // [M][nparts]
  float* tgt;              // [M]
  int N, nparts;
  struct Ctx {};
  GPT2_DEV Ctx load(int, int) const { return {}; }
  GPT2_DEV void store(int, int, f32x4_t, Ctx) const {}
  GPT2_DEV void operator()(int, int, f32x4_t) const {}
};

// The head for greedy generation without its logits: per row m and per
// (column tile, wave column) the largest logit and its column go to
// part[m][slot] (the lowest column among equal values; NaN is never chosen
// over a number); argmax_parts_kernel picks the best of a row's partials.
struct EpiArgmax {
  static constexpr bool kRowArgmax = true;
  float2* part;  // [M][nparts]: value, column (as bits)
  int N, nparts;
  struct Ctx {};
  GPT2_DEV Ctx load(int, int) const { return {}; }
  GPT2_DEV void store(int, int, f32x4_t, Ctx) const {}
  GPT2_DEV void operator()(int, int, f32x4_t) const {}
};

template <typename Tact>
struct EpiBiasGelu {
  const Tact* bias;
  Tact* out;
  int N;
  using Ctx = typename Raw4<Tact>::type;  // bias
  GPT2_DEV Ctx load(int, int n) const { return load4_raw(bias + n); }
  GPT2_DEV void store(int m, int n, f32x4_t v, const Ctx& braw) const {
    const float4 b = widen4(braw);
    store4(out + (long long)m * N + n,
           make_float4(gelu_tanh(v[0] + b.x), gelu_tanh(v[1] + b.y), gelu_tanh(v[2] + b.z),
                       gelu_tanh(v[3] + b.w)));
  }
  GPT2_DEV void operator()(int m, int n, f32x4_t v) const { store(m, n, v, load(m, n)); }
};

template <typename Tact, typename Tres, typename Tout>
struct EpiBiasResid {
  const Tact* bias;
  const Tres* res;
  Tout* out;
  int N;
  struct Ctx {
    typename Raw4<Tact>::type b;  // bias
    typename Raw4<Tres>::type r;  // residual
  };
  GPT2_DEV Ctx load(int m, int n) const { return {load4_raw(bias + n), load4_raw(res + (long long)m * N + n)}; }
  GPT2_DEV void store(int m, int n, f32x4_t v, const Ctx& c) const {
    const float4 b = widen4(c.b), r = widen4(c.r);
    store4(out + (long long)m * N + n,
           make_float4(r.x + (v[0] + b.x), r.y + (v[1] + b.y), r.z + (v[2] + b.z), r.w + (v[3] + b.w)));
  }
  GPT2_DEV void operator()(int m, int n, f32x4_t v) const { store(m, n, v, load(m, n)); }
};

// In-place fp32 residual update x += acc + bias.
template <typename Tact>
struct EpiResidInPlace {
  const Tact* bias;
  float* x;
  int N;
  struct Ctx {
    typename Raw4<Tact>::type b;  // bias
    float4 r;                     // residual
  };
  GPT2_DEV Ctx load(int m, int n) const {
    return {load4_raw(bias + n), *reinterpret_cast<const float4*>(x + (long long)m * N + n)};
  }
  GPT2_DEV void store(int m, int n, f32x4_t v, const Ctx& c) const {
    const float4 b = widen4(c.b);
    *reinterpret_cast<float4*>(x + (long long)m * N + n) =
        make_float4(c.r.x + (v[0] + b.x), c.r.y + (v[1] + b.y), c.r.z + (v[2] + b.z), c.r.w + (v[3] + b.w));
  }
  GPT2_DEV void operator()(int m, int n, f32x4_t v) const { store(m, n, v, load(m, n)); }
};

// The products of S ranges of K, kept apart for a fixed-order sum later:
// part[split][m][n] (fp32, [S][M][N]).  The skinny decode kernel writes
// them when an in-place residual product splits K over workgroups; the
// LayerNorm that follows adds them to the residual stream in range order
// (launch_layernorm_reduce), so results do not depend on timing.
struct EpiPartial {
  static constexpr bool kPartial = true;
  float* part;
  int N;
  long long split_stride;  // M * N
  struct Ctx {};
  GPT2_DEV Ctx load(int, int) const { return {}; }
  GPT2_DEV void store(int, int, f32x4_t, Ctx) const {}
  GPT2_DEV void operator()(int, int, f32x4_t) const {}
  GPT2_DEV void put(int split, int m, int n, f32x4_t v) const {
    *reinterpret_cast<f32x4_t*>(part + split * split_stride + (long long)m * N + n) = v;
  }
};

template <typename Tact>
struct EpiQKV {
  const Tact* bias;
  Tact* q;
  KvView kv;
  int T, l_past, H, dh, d;
  FastDiv divT, divDh;
  using Ctx = typename Raw4<Tact>::type;  // bias
  GPT2_DEV Ctx load(int, int n) const { return load4_raw(bias + n); }
  GPT2_DEV void operator()(int m, int n, f32x4_t v) const { store(m, n, v, load(m, n)); }
  // The destination splits into a part that depends on the column only (q,
  // k or v; head; element) and one that depends on the row only (sequence,
  // position), so the tile epilogue computes each once per column block
  // and per row rather than per store (kColRow).
  static constexpr bool kColRow = true;
  struct Col {
    bool is_q;
    long long off;  // elements from q (is_q) or from the K/V view base
  };
  struct Row {
    long long q_off, kv_off;
  };
  GPT2_DEV Col col(int n) const {
    const int sec = (n >= d) + (n >= 2 * d);
    const int c = n - sec * d;
    const int h = (int)divDh.div((uint32_t)c);
    const int j = c - h * dh;
    if (sec == 0) return {true, (long long)h * T * dh + j};
    return {false, (sec - 1) * kv.skv + h * kv.sh + (long long)l_past * dh + j};
  }
  GPT2_DEV Row row(int m) const {
    const int bi = (int)divT.div((uint32_t)m);
    const int t = m - bi * T;
    return {((long long)bi * H * T + t) * dh, bi * kv.sb + (long long)t * dh};
  }
  GPT2_DEV void store(const Row& r, const Col& c, f32x4_t v, const Ctx& braw) const {
    const float4 b = widen4(braw);
    const float4 y = make_float4(v[0] + b.x, v[1] + b.y, v[2] + b.z, v[3] + b.w);
    Tact* dst = c.is_q ? q + (c.off + r.q_off) : (Tact*)kv.base + (c.off + r.kv_off);
    store4(dst, y);
  }
  GPT2_DEV void store(int m, int n, f32x4_t v, const Ctx& braw) const { store(row(m), col(n), v, braw); }
};

// ================================================================ tile order
// Maps the hardware block id to an output tile.  Workgroups are dealt to the
// 8 XCDs round-robin; when the grid divides evenly the ids are regrouped so
// each XCD walks a contiguous run of logical tiles, then logical tiles are
// ordered in groups of GM tile-rows so neighbours share X rows and W rows in
// that XCD's L2.
GPT2_DEV void tile_coords(int bid, int nb, int tiles_m, int tiles_n, int& tm, int& tn) {
  int L = bid;
  if ((nb & 7) == 0) L = (bid & 7) * (nb >> 3) + (bid >> 3);
  constexpr int GM = 8;
  const int per_group = GM * tiles_n;
  const int group = L / per_group;
  const int first_m = group * GM;
  const int gsize = min(tiles_m - first_m, GM);
  const int r = L - group * per_group;
  tm = first_m + r % gsize;
  tn = r / gsize;
}

// ================================================================ bf16 MFMA kernel
template <int BM, int BN, class Epi>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(const bf16_t* __restrict__ X,
                                                        const bf16_t* __restrict__ W, int M, int N,
                                                        int K, Epi epi, int tiles_m, int tiles_n) {
  constexpr int BK = 64;             // K per stage: 8 chunks of 16 B per row
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int TM = WM / 16, TN = WN / 16;
  constexpr int PA = BM / 32, PB = BN / 32;  // 16-byte loads per thread per stage
  constexpr int STAGE = (BM + BN) * 8;       // uint4 per stage
  __shared__ uint4 lds[2 * STAGE];

  int tm_idx, tn_idx;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm_idx, tn_idx);
  const int m0 = tm_idx * BM, n0 = tn_idx * BN;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int lrow = tid >> 3, lchunk = tid & 7;

  const bf16_t* xrow[PA];
  const bf16_t* wrow[PB];
#pragma unroll
  for (int i = 0; i < PA; ++i) xrow[i] = X + (long long)min(m0 + lrow + 32 * i, M - 1) * K;
#pragma unroll
  for (int i = 0; i < PB; ++i) wrow[i] = W + (long long)min(n0 + lrow + 32 * i, N - 1) * K;

  uint4 ra[PA], rb[PB];
  auto gload = [&](int k0) {
    const int kc = k0 + lchunk * 8;
    const bool ok = kc < K;
#pragma unroll
    for (int i = 0; i < PA; ++i)
      ra[i] = ok ? *reinterpret_cast<const uint4*>(xrow[i] + kc) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int i = 0; i < PB; ++i)
      rb[i] = ok ? *reinterpret_cast<const uint4*>(wrow[i] + kc) : make_uint4(0, 0, 0, 0);
  };
  auto lstore = [&](int stage) {
    uint4* sa = lds + stage * STAGE;
    uint4* sb = sa + BM * 8;
#pragma unroll
    for (int i = 0; i < PA; ++i) {
      const int r = lrow + 32 * i;
      sa[r * 8 + (lchunk ^ ((r >> 1) & 7))] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < PB; ++i) {
      const int r = lrow + 32 * i;
      sb[r * 8 + (lchunk ^ ((r >> 1) & 7))] = rb[i];
    }
  };

  f32x4_t acc[TN][TM];
#pragma unroll
  for (int a = 0; a < TN; ++a)
#pragma unroll
    for (int b = 0; b < TM; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const bool more = kt + 1 < nk;
    if (more) gload((kt + 1) * BK);
    const uint4* sa = lds + (kt & 1) * STAGE;
    const uint4* sb = sa + BM * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int chunk = ks * 4 + (lane >> 4);
      bf16x8_t xa[TM], wb[TN];
#pragma unroll
      for (int t = 0; t < TM; ++t) {
        const int r = wm * WM + t * 16 + (lane & 15);
        uint4 u = sa[r * 8 + (chunk ^ ((r >> 1) & 7))];
        xa[t] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const int r = wn * WN + t * 16 + (lane & 15);
        uint4 u = sb[r * 8 + (chunk ^ ((r >> 1) & 7))];
        wb[t] = __builtin_bit_cast(bf16x8_t, u);
      }
#pragma unroll
      for (int a = 0; a < TN; ++a)
#pragma unroll
        for (int b = 0; b < TM; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wb[a], xa[b], acc[a][b], 0, 0, 0);
    }
    if (more) lstore((kt + 1) & 1);
    __syncthreads();
  }

#pragma unroll
  for (int a = 0; a < TN; ++a) {
    const int n = n0 + wn * WN + a * 16 + 4 * (lane >> 4);
    if (n >= N) continue;
#pragma unroll
    for (int b = 0; b < TM; ++b) {
      const int m = m0 + wm * WM + b * 16 + (lane & 15);
      if (m < M) epi(m, n, acc[a][b]);
    }
  }
}

template <int BM, int BN, class Epi>
static void run_bf16(const bf16_t* X, const bf16_t* W, int M, int N, int K, const Epi& epi,
                     hipStream_t s) {
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN;
  gemm_bf16_kernel<BM, BN, Epi><<<tiles_m * tiles_n, 256, 0, s>>>(X, W, M, N, K, epi, tiles_m, tiles_n);
}


// ================================================================ bf16 MFMA kernel, DMA ring
// 32x32x16 MFMA (twice the throughput of 16x16x32 on gfx950), WGM x WGN waves
// of (BM/WGM)x(BN/WGN), K step BK (32 or 64).  Tiles move global -> LDS with
// global_load_lds_dwordx4 (no register staging) through a ring of STAGES
// buffers.  A wave's 64-lane load fills 1 KB of LDS (1024/(2*BK) tile rows),
// and each lane picks the global 16-byte chunk that the XOR swizzle puts in
// its slot, so the fragment reads (16 lanes = 16 rows of one chunk) touch all
// 64 banks once.  Requires K % BK == 0.
template <int BM, int BN, int BK, int STAGES, int NW = 4>
struct V2Cfg {
  static constexpr int CH = BK / 8;                  // 16-byte chunks per row
  static constexpr int RPL = 64 / CH;                // rows per wave load (1 KB)
  static constexpr int SWZ_SHIFT = BK == 64 ? 1 : 2; // rows sharing a bank phase
  static constexpr int ROWS = BM + BN;               // X rows then W rows
  static constexpr int GROUPS = ROWS / RPL;          // wave loads per stage
  static constexpr int LOADS = (GROUPS + NW - 1) / NW;  // per wave per stage
  // When the groups do not split evenly, the waves short of LOADS issue a
  // dummy load (one 16-byte line, all lanes) into a spare 1 KB of LDS that is
  // never read, so every wave has the same count of loads in flight.
  static constexpr bool DUMMY = LOADS * NW != GROUPS;
  static constexpr int STAGE_U4 = ROWS * CH;         // uint4 per stage
  static constexpr size_t LDS_BYTES = (size_t)STAGES * STAGE_U4 * 16 + (DUMMY ? 1024 : 0);
  static_assert(BK == 32 || BK == 64, "BK");
  static_assert(ROWS % RPL == 0, "tile rows fill whole wave loads");
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tiles are multiples of 32");
  static_assert((size_t)NW * 32 * 36 * 4 <= LDS_BYTES, "epilogue patches fit in the stage ring");
  static GPT2_DEV int swz(int row, int c) { return c ^ ((row >> SWZ_SHIFT) & (CH - 1)); }
};

template <class Epi>
constexpr bool line_aligned() {
  return std::is_base_of_v<EpiStoreF32Lines, Epi>;
}

template <class Epi>
constexpr bool row_lse() {
  if constexpr (requires { Epi::kRowLse; }) return Epi::kRowLse;
  else return false;
}

// EpiLoss at the end of a tile, straight from the MFMA layout: lane l holds,
// for token m = mw0 + 32 b + l%32, the 16 x FN logits of columns
// nw0 + 32 a + 8 (r/4) + 4 (l/32) + r%4; the two lanes l and l + 32 cover the
// wave's WN columns of that token.
template <int FM, int FN, int WN>
GPT2_DEV void lse_epilogue(const f32x16_t (&acc)[FN][FM], const EpiLoss& epi, int M, int mw0, int nw0,
                           int slot, int lane) {
  constexpr float kLog2e = 1.4426950408889634f;
  const int r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int m = mw0 + b * 32 + r32;
    float mx = -INFINITY;
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = nw0 + a * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (n < epi.N) mx = fmaxf(mx, acc[a][b][r]);
      }
    mx = halves_max(mx);
    float sm = 0.f;
    const int t = m < M ? epi.targets[m] : -1;
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = nw0 + a * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        if (n < epi.N) {
          sm += __builtin_amdgcn_exp2f((acc[a][b][r] - mx) * kLog2e);
          if (n == t) epi.tgt[m] = acc[a][b][r];
        }
      }
    sm = halves_sum(sm);
    if (kh == 0 && m < M) epi.part[(long long)m * epi.nparts + slot] = make_float2(mx, sm);
  }
  (void)WN;
}

template <class Epi>
constexpr bool row_argmax() {
  if constexpr (requires { Epi::kRowArgmax; }) return Epi::kRowArgmax;
  else return false;
}

// Epilogues that reduce rows straight from the accumulators (no stores of
// the product, no epilogue reads).
template <class Epi>
constexpr bool row_reduce() {
  return row_lse<Epi>() || row_argmax<Epi>();
}

// EpiArgmax at the end of a tile, from the MFMA layout described for
// lse_epilogue.  A lane scans its columns in increasing order, so a strict
// "greater" keeps the lowest column among equal values; the two lanes of a
// token then combine with the same tie rule.
template <int FM, int FN>
GPT2_DEV void argmax_epilogue(const f32x16_t (&acc)[FN][FM], const EpiArgmax& epi, int M, int mw0, int nw0,
                              int slot, int lane) {
  const int r32 = lane & 31, kh = lane >> 5;
#pragma unroll
  for (int b = 0; b < FM; ++b) {
    const int m = mw0 + b * 32 + r32;
    float best = -INFINITY;
    int bi = 0x7fffffff;  // no column yet: loses every tie
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = nw0 + a * 32 + 8 * (r >> 2) + 4 * kh + (r & 3);
        const float v = acc[a][b][r];
        if (n < epi.N && (v > best || (v == best && n < bi))) {
          best = v;
          bi = n;
        }
      }
    float v0, v1, i0, i1;
    row_pair<32>(best, v0, v1);
    row_pair<32>(__int_as_float(bi), i0, i1);
    const int j0 = __float_as_int(i0), j1 = __float_as_int(i1);
    const bool take1 = v1 > v0 || (v1 == v0 && j1 < j0);
    if (kh == 0 && m < M) epi.part[(long long)m * epi.nparts + slot] = make_float2(take1 ? v1 : v0, take1 ? i1 : i0);
  }
}

template <class Epi>
constexpr bool row_store() {
  if constexpr (requires { Epi::kRowStore; }) return Epi::kRowStore;
  else return false;
}

// Whether the epilogue's global reads are issued ahead of the last K stage
// (all at once) or fragment by fragment inside the epilogue.
template <class Epi>
constexpr bool hoist_ctx() {
  if constexpr (requires { Epi::kHoistCtx; }) return Epi::kHoistCtx;
  else return true;
}

template <int N>
GPT2_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 s_waitcnt: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt_hi[15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier for the LDS ring.  __syncthreads() also drains every
// outstanding global access (vmcnt 0), which would wait for the loads of the
// stages still being prefetched; this waits only for the wave's LDS
// instructions.  Each wave has already waited (wait_stage) for its own loads of
// the stage about to be read, so after the barrier that stage is complete.
GPT2_DEV void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Waits until at most `ahead` later stages of this wave's loads are in flight.
template <int LOADS, int MAXAHEAD>
GPT2_DEV void wait_stage(int ahead) {
  if constexpr (MAXAHEAD > 0) {
    if (ahead >= MAXAHEAD) {
      wait_vmcnt<MAXAHEAD * LOADS>();
      return;
    }
    wait_stage<LOADS, MAXAHEAD - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

// Epilogue through LDS (the patch is wave-private and LDS executes a wave's
// accesses in order, so no wait is needed between its write and read-back).
// A C[n][m] fragment holds, per lane, column m = lane%32
// and rows n = 8*(r/4) + 4*(lane/32) + r%4: stored directly that is 32 rows x 16 B
// per instruction.  Each wave instead writes one 32x32 fragment at a time to
// its own LDS patch as [m][n] (row pitch 36 floats) and reads it back with 8
// lanes per row, so every epilogue access covers 8 rows x 32 consecutive columns.
// (mw0, nw0) is the wave tile's first output row and column.
// The epilogue's own global reads (bias, residual) for every element the lane
// will store, issued in one batch before the last K stage's MFMAs so that
// their latency is paid once and overlaps the tail of the main loop.
template <int FM, int FN, class Epi>
GPT2_DEV void tile_epilogue_loads(typename Epi::Ctx (&cx)[FN][FM][4], const Epi& epi, int M, int N, int mw0,
                                  int nw0, int lane) {
  if constexpr (!row_store<Epi>()) {
    const int er = lane >> 3, ec = (lane & 7) * 4;
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < FM; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // unconditional, so the loads issue back to back; lanes outside
          // the output read element (0, 0) and never use it
          const int m = mw0 + b * 32 + 8 * i + er, n = nw0 + a * 32 + ec;
          const bool in = m < M && n < N;
          cx[a][b][i] = epi.load(in ? m : 0, in ? n : 0);
        }
  }
}

template <class Epi>
constexpr bool col_row() {
  if constexpr (requires { Epi::kColRow; }) return Epi::kColRow;
  else return false;
}

// Per-row part of a kColRow epilogue's destinations, one per row a lane
// stores (or an empty placeholder for other epilogues).
template <class Epi, bool = col_row<Epi>()>
struct RowParts {
  template <int FM>
  GPT2_DEV void init(const Epi&, int, int, int) {}
};
template <class Epi>
struct RowParts<Epi, true> {
  typename Epi::Row r[4 * 4];  // up to FM = 4 fragments x 4 rows
  template <int FM>
  GPT2_DEV void init(const Epi& epi, int M, int mw0, int er) {
    static_assert(FM <= 4, "row parts");
#pragma unroll
    for (int b = 0; b < FM; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i) r[b * 4 + i] = epi.row(min(mw0 + b * 32 + 8 * i + er, M - 1));
  }
};

template <int FM, int FN, class Epi>
GPT2_DEV void tile_epilogue(const f32x16_t (&acc)[FN][FM], const typename Epi::Ctx (&cx)[FN][FM][4], uint4* lds,
                            const Epi& epi, int M, int N, int mw0, int nw0, int wave, int lane) {
  const int r32 = lane & 31, khalf = lane >> 5;
  float* patch = reinterpret_cast<float*>(lds) + wave * (32 * 36);
  const int er = lane >> 3;        // row within an 8-row group
  const int ec = (lane & 7) * 4;   // first of 4 columns
  RowParts<Epi> rows;
  if constexpr (col_row<Epi>()) rows.template init<FM>(epi, M, mw0, er);
#pragma unroll
  for (int a = 0; a < FN; ++a) {
#pragma unroll
    for (int b = 0; b < FM; ++b) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(patch + r32 * 36 + 8 * q + 4 * khalf) =
            make_float4(acc[a][b][4 * q], acc[a][b][4 * q + 1], acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
      if constexpr (row_store<Epi>()) {
        const int n = nw0 + a * 32 + r32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int row = 2 * i + khalf;
          const float v = patch[row * 36 + r32];
          const int m = mw0 + b * 32 + row;
          if (m < M && n < N) epi.store1(m, n, v);
        }
      } else {
        f32x4_t v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 t = *reinterpret_cast<const float4*>(patch + (8 * i + er) * 36 + ec);
          v[i] = f32x4_t{t.x, t.y, t.z, t.w};
        }
        const int n = nw0 + a * 32 + ec;
        if constexpr (col_row<Epi>()) {
          const auto c = epi.col(n);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = mw0 + b * 32 + 8 * i + er;
            if (m < M && n < N) epi.store(rows.r[b * 4 + i], c, v[i], cx[a][b][i]);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int m = mw0 + b * 32 + 8 * i + er;
            if (m < M && n < N) epi.store(m, n, v[i], cx[a][b][i]);
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------- the kernel
// Tiles, loads and fragments as described for V2Cfg.  Schedule per K step: the
// step's MFMAs with the next step's fragment reads between them; a K step's
// last MFMAs are issued after the barrier that publishes the next stage, so
// the first fragment reads of stage kt+1 (and the barrier's own skew) overlap
// them instead of leaving the matrix cores idle at every stage boundary.  The
// ring is refilled right after that barrier: stage kt+STAGES goes into the
// buffer that stage kt has just released.
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, class Epi>
__global__ __launch_bounds__(64 * WGM * WGN) void gemm_bf16_v3_kernel(const bf16_t* __restrict__ X,
                                                                      const bf16_t* __restrict__ W, int M,
                                                                      int N, int K, Epi epi, int tiles_m,
                                                                      int tiles_n) {
  constexpr int NW = WGM * WGN;
  using C = V2Cfg<BM, BN, BK, STAGES, NW>;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int KS = BK / 16;  // MFMA steps per stage
  static_assert(WM % 32 == 0 && WN % 32 == 0, "wave tiles are multiples of 32");
  static_assert(KS % 2 == 0, "fragment double buffer assumes an even step count");
  extern __shared__ uint4 lds[];

  int tm_idx, tn_idx;
  tile_coords(blockIdx.x, gridDim.x, tiles_m, tiles_n, tm_idx, tn_idx);
  const int m0 = tm_idx * BM;
  int n0 = tn_idx * BN;
  if constexpr (line_aligned<Epi>()) {
    n0 = epi.line_offset(m0) + BN * (tn_idx - 1);
    if (n0 >= N || n0 + BN <= 0) return;  // whole workgroup: window outside the row
  }
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave % WGM, wn = wave / WGM;

  const bf16_t* src[C::LOADS];
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) {
    const int g = wave + NW * i;
    if (g >= C::GROUPS) {  // dummy load: one line of this tile's first X row
      src[i] = X + (long long)m0 * K;
      continue;
    }
    const int row = C::RPL * g + lane / C::CH;
    const int c = C::swz(row, lane % C::CH);
    int xr = min(m0 + row, M - 1);
    if constexpr (line_aligned<Epi>()) xr = epi.row_of(xr);
    const bf16_t* base = row < BM ? X + (long long)xr * K
                                  : W + (long long)min(max(n0 + row - BM, 0), N - 1) * K;
    src[i] = base + c * 8;
  }
  auto issue = [&](int kt, int stage) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int g = wave + NW * i;
      uint4* dst = g < C::GROUPS ? lds + stage * C::STAGE_U4 + g * 64 : lds + STAGES * C::STAGE_U4;
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + k0),
                                       (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
    }
  };

  f32x16_t acc[FN][FM];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < FM; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  const int r32 = lane & 31, khalf = lane >> 5;
  bf16x8_t xf[2][FM], wf[2][FN];
  // fragment f of K step ks: X rows for f < FM, W rows after
  auto ldone = [&](int buf, const uint4* st, int ks, int f) {
    const int chunk = 2 * ks + khalf;
    if (f < FM) {
      const int row = wm * WM + f * 32 + r32;
      xf[buf][f] = __builtin_bit_cast(bf16x8_t, st[row * C::CH + C::swz(row, chunk)]);
    } else {
      const int row = BM + wn * WN + (f - FM) * 32 + r32;
      wf[buf][f - FM] = __builtin_bit_cast(bf16x8_t, st[row * C::CH + C::swz(row, chunk)]);
    }
  };
  // The MFMAs of one K step (fragments in `buf`) with the fragment reads of
  // the next step (into the other buffer) between them: issued after the
  // step's first MFMAs (so the compiler's wait before those covers only reads
  // that have had a whole step to land) and early enough that the rest of
  // the step's MFMAs hide their latency.
  auto step = [&](int buf, const uint4* nst, int nks) {
    constexpr int NM = FN * FM, NL = FM + FN;
    constexpr int SPREAD = NM > 2 ? NM / 2 : NM;  // MFMAs that the reads follow
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      acc[i / FM][i % FM] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[buf][i / FM], xf[buf][i % FM],
                                                                    acc[i / FM][i % FM], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (i < SPREAD) {
#pragma unroll
        for (int l = i * NL / SPREAD; l < (i + 1) * NL / SPREAD; ++l) ldone(buf ^ 1, nst, nks, l);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = K / BK;
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nk) issue(s, s);
  wait_stage<C::LOADS, STAGES - 1>(min(STAGES - 1, nk - 1));
  lds_barrier();
#pragma unroll
  for (int f = 0; f < FM + FN; ++f) ldone(0, lds, 0, f);

  for (int kt = 0; kt + 1 < nk; ++kt) {
    const uint4* st = lds + (kt % STAGES) * C::STAGE_U4;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) step(ks & 1, st, ks + 1);
    // own loads of stage kt+1 done (later stages may stay in flight), this
    // wave's reads of stage kt done; after the barrier both hold for all waves
    wait_stage<C::LOADS, STAGES - 2>(min(STAGES - 2, nk - 2 - kt));
    lds_barrier();
    if (kt + STAGES < nk) issue(kt + STAGES, kt % STAGES);
    __builtin_amdgcn_sched_barrier(0);
    step(1, lds + ((kt + 1) % STAGES) * C::STAGE_U4, 0);
  }
  // the last K stage: no main-loop loads are waited for from here on
  typename Epi::Ctx cx[FN][FM][4];
  if constexpr (!row_reduce<Epi>() && hoist_ctx<Epi>())
    tile_epilogue_loads<FM, FN>(cx, epi, M, N, m0 + wm * WM, n0 + wn * WN, lane);
  if (nk > 0) {
    const int kt = nk - 1;
    const uint4* st = lds + (kt % STAGES) * C::STAGE_U4;
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks) step(ks & 1, st, ks + 1);
    __builtin_amdgcn_sched_barrier(0);
    // its reads of the following stage fetch unused data from the ring (in
    // bounds, never consumed)
    step(1, lds + ((kt + 1) % STAGES) * C::STAGE_U4, 0);
  }
  if constexpr (!row_reduce<Epi>() && !hoist_ctx<Epi>())
    tile_epilogue_loads<FM, FN>(cx, epi, M, N, m0 + wm * WM, n0 + wn * WN, lane);

  if constexpr (row_lse<Epi>()) {
    lse_epilogue<FM, FN, WN>(acc, epi, M, m0 + wm * WM, n0 + wn * WN, tn_idx * WGN + wn, lane);
  } else if constexpr (row_argmax<Epi>()) {
    argmax_epilogue<FM, FN>(acc, epi, M, m0 + wm * WM, n0 + wn * WN, tn_idx * WGN + wn, lane);
  } else {
    __syncthreads();  // all waves are done reading the K stages
    tile_epilogue<FM, FN>(acc, cx, lds, epi, M, N, m0 + wm * WM, n0 + wn * WN, wave, lane);
  }
}

template <int BM, int BN, int BK, int STAGES, class Epi, int WGM, int WGN>
static void run_bf16_v3(const bf16_t* X, const bf16_t* W, int M, int N, int K, const Epi& epi,
                        hipStream_t s) {
  using C = V2Cfg<BM, BN, BK, STAGES, WGM * WGN>;
  set_dynamic_lds_limit((const void*)gemm_bf16_v3_kernel<BM, BN, BK, STAGES, WGM, WGN, Epi>, (int)C::LDS_BYTES);
  const int tiles_m = (M + BM - 1) / BM, tiles_n = (N + BN - 1) / BN + (line_aligned<Epi>() ? 1 : 0);
  gemm_bf16_v3_kernel<BM, BN, BK, STAGES, WGM, WGN, Epi>
      <<<tiles_m * tiles_n, 64 * WGM * WGN, C::LDS_BYTES, s>>>(X, W, M, N, K, epi, tiles_m, tiles_n);
}

// ================================================================ skinny bf16 kernel (M <= 64)
// Decode-sized products: each weight byte is used once, so the job is to
// stream W from HBM with every CU busy and many bytes in flight.  A workgroup
// owns NT output columns (NT rows of W) and one of S ranges of K (kc = K/S
// <= 768): it issues every load of its X tile [64 x kc] and W tile [NT x kc]
// at once with global_load_lds_dwordx4 (coalesced rows, XOR-swizzled 16-byte
// chunks in LDS), waits once, and its 4 waves split kc for the MFMA
// v_mfma_f32_16x16x32_bf16 (W rows as the A operand).  The waves' partial sums
// meet in LDS.  S > 1 is used only with EpiPartial, which keeps each K
// range's product apart for a fixed-order sum; every other epilogue runs
// with S = 1.
constexpr int kSkinnyMaxKc = 768;

template <class Epi>
constexpr bool partial_out() {
  if constexpr (requires { Epi::kPartial; }) return Epi::kPartial;
  else return false;
}

template <int NT, class Epi>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(const bf16_t* __restrict__ X,
                                                          const bf16_t* __restrict__ W, int M, int N,
                                                          int K, int S, Epi epi, FastDiv cdiv) {
  extern __shared__ uint4 lds[];
  constexpr int ROWS = 64 + NT;  // X rows then W rows
  constexpr int FN = NT / 16;    // A fragments (W) per step
  const int ns = blockIdx.x / S, split = blockIdx.x - (blockIdx.x / S) * S;
  const int n0 = ns * NT;
  const int kc = K / S, k0 = split * kc;
  const int cpr = kc / 8;  // 16-byte chunks per row
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

  // ---- issue the whole tile: slot p of LDS holds (row p / cpr, chunk (p % cpr) ^ (row & 15)).
  // total is a multiple of 256 (ROWS is 80 or 96, cpr a multiple of 16), so
  // every 64-slot wave load lies inside the tile.
  const int total = ROWS * cpr;
  for (int base = wave * 64; base < total; base += 256) {
    const int p = base + lane;
    const int row = (int)cdiv.div((uint32_t)p);
    const int c = (p - row * cpr) ^ (row & 15);
    const bf16_t* src = row < 64 ? X + (long long)min(row, M - 1) * K
                                 : W + (long long)min(n0 + row - 64, N - 1) * K;
    __builtin_amdgcn_global_load_lds((const void*)(src + k0 + c * 8),
                                     (__attribute__((address_space(3))) void*)(lds + base), 16, 0, 0);
  }
  wait_vmcnt<0>();
  __syncthreads();

  // ---- MFMA over this wave's quarter of kc
  f32x4_t acc[FN][4];
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int l16 = lane & 15, kg = lane >> 4;
  const int steps = kc / 32 / 4;  // 32-wide k steps per wave
  for (int st = 0; st < steps; ++st) {
    const int c = (wave * steps + st) * 4 + kg;
    bf16x8_t wf[FN], xf[4];
#pragma unroll
    for (int a = 0; a < FN; ++a) {
      const int row = 64 + a * 16 + l16;
      wf[a] = __builtin_bit_cast(bf16x8_t, lds[row * cpr + (c ^ (row & 15))]);
    }
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int row = b * 16 + l16;
      xf[b] = __builtin_bit_cast(bf16x8_t, lds[row * cpr + (c ^ (row & 15))]);
    }
#pragma unroll
    for (int a = 0; a < FN; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[a], xf[b], acc[a][b], 0, 0, 0);
  }
  // ---- the 4 waves' partial sums meet in LDS: [wave][FN*4 fragments][64 lanes] float4
  __syncthreads();
  float4* red = reinterpret_cast<float4*>(lds);
#pragma unroll
  for (int a = 0; a < FN; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
      red[(wave * FN * 4 + a * 4 + b) * 64 + lane] =
          make_float4(acc[a][b][0], acc[a][b][1], acc[a][b][2], acc[a][b][3]);
  __syncthreads();
  // fragment f = tid / 64 (+4): C[n][m] with m = 16*(f%4) + lane%16, n = 16*(f/4) + 4*(lane/16)
  for (int f = wave; f < FN * 4; f += 4) {
    float4 v = red[f * 64 + lane];
#pragma unroll
    for (int w = 1; w < 4; ++w) {
      const float4 u = red[(w * FN * 4 + f) * 64 + lane];
      v = make_float4(v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w);
    }
    const int m = 16 * (f & 3) + l16;
    const int n = n0 + 16 * (f >> 2) + 4 * kg;
    if (m < M && n < N) {
      if constexpr (partial_out<Epi>())
        epi.put(split, m, n, f32x4_t{v.x, v.y, v.z, v.w});
      else
        epi(m, n, f32x4_t{v.x, v.y, v.z, v.w});
    }
  }
}

// K ranges for the skinny kernel: the fewest that keep kc = K/S <= 768 with
// K/S a multiple of 128 (16 chunks per LDS row) and, where the products may
// be kept per range (min_wg > 0), give at least min_wg workgroups over the
// nslices column slices.  Each range adds an M x N fp32 partial to write
// and sum, so no more than that: at M = 64, N = K = 768 (48 slices) two
// ranges took 4.5 us against 5.3 us for one and 6.7 us for six.  0 if none
// exists.
static int skinny_splits(int K, int nslices = 0, int min_wg = 0) {
  int first = 0;
  for (int s = 1; s <= K / 128; ++s)
    if (K % s == 0 && (K / s) % 128 == 0 && K / s <= kSkinnyMaxKc) {
      if (!first) first = s;
      if (nslices * s >= min_wg) return s;
    }
  return first;
}

template <int NT, class Epi>
static void run_skinny(const bf16_t* X, const bf16_t* W, int M, int N, int K, int S, const Epi& epi,
                       hipStream_t s) {
  // the tile, and after the MFMAs the four waves' partial sums
  // (4 waves x NT/16 x 4 fragments x 64 lanes x 16 B = NT KB) in the same space
  const size_t lds = std::max((size_t)(64 + NT) * (K / S) * 2, (size_t)NT * 1024);
  set_dynamic_lds_limit((const void*)gemm_skinny_kernel<NT, Epi>, 160 * 1024);
  const int nslices = (N + NT - 1) / NT;
  gemm_skinny_kernel<NT, Epi><<<nslices * S, 256, lds, s>>>(X, W, M, N, K, S, epi,
                                                             FastDiv::make((uint32_t)(K / S / 8)));
}

// Chooses the skinny kernel when it applies; returns false otherwise.
template <class Epi>
static bool try_skinny(const bf16_t* X, const bf16_t* W, int M, int N, int K, const Epi& epi,
                       hipStream_t s) {
  if (M > 64) return false;
  const int S = skinny_splits(K);
  if (S != 1) return false;
  if (N >= 8192)
    run_skinny<32>(X, W, M, N, K, S, epi, s);
  else
    run_skinny<16>(X, W, M, N, K, S, epi, s);
  return true;
}

// Tile shape for the block products (M > 64), chosen by an estimate of the
// busiest CU's time.  Each shape has a measured throughput per CU when its
// workgroups fill the CU (fraction of the bf16 MFMA peak, random data,
// M = 4096 and 8192 products of the GPT-2 depths); a CU left with one
// workgroup of a two-per-CU shape in its last round runs at 0.8 of that.  The
// estimate is the busiest CU's tile count in whole rounds of `per_cu`
// workgroups, times the tile's area, over that throughput; K is common to
// every shape.  On the 20 measured products it picks the fastest shape or one
// within 6% of it (M = 4096, N = 1024: mlp c_proj 53.6 -> 47.1 us with
// 128x128; N = 4096: c_fc 44.6 -> 40.3 us with 256x256), and keeps 128x192
// for every GPT-2-small product at M = 8192.  128x256 and 256x192 tiles beat
// these on a few products by 2-5% at most, within run-to-run variation, and
// are left out.  256-row tiles are left out for the
// residual epilogues, whose prefetched fp32 residual would not fit in
// registers beside a 64-row wave tile.
enum class Tiles { k128x192, k128x96, k128x128, k256x256 };

struct TileShape {
  Tiles id;
  int bm, bn, per_cu;
  double rate;
};
constexpr TileShape kTileShapes[] = {
    {Tiles::k128x192, 128, 192, 2, 0.31},
    {Tiles::k128x96, 128, 96, 2, 0.24},
    {Tiles::k128x128, 128, 128, 2, 0.28},
    {Tiles::k256x256, 256, 256, 1, 0.32},
};

static Tiles block_tiles(int M, int N, bool tall_ok) {
  const long long ncu = device_cu_count();
  Tiles best = Tiles::k128x192;
  double best_t = 0.0;
  for (const TileShape& t : kTileShapes) {
    if (t.bm == 256 && !tall_ok) continue;
    const long long tiles = (long long)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn);
    const long long k = (tiles + ncu - 1) / ncu;  // tiles on the busiest CU
    const long long rounds = k / t.per_cu, rem = k % t.per_cu;
    const double area = (double)t.bm * t.bn;
    double est = rounds * t.per_cu * area / t.rate;
    if (rem) est += rem * area / (t.rate * (t.per_cu == 2 && rem == 1 ? 0.8 : 1.0));
    if (best_t == 0.0 || est < best_t) {
      best = t.id;
      best_t = est;
    }
  }
  return best;
}

// Epilogues that may take 256-row tiles: those without a prefetched residual.
template <class Epi>
constexpr bool tall_tiles_ok() {
  return std::is_same_v<Epi, EpiBiasGelu<bf16_t>> || std::is_same_v<Epi, EpiQKV<bf16_t>>;
}

template <class Epi>
static void dispatch_bf16(const bf16_t* X, const bf16_t* W, int M, int N, int K, const Epi& epi,
                          hipStream_t s) {
  if (M <= 64) {
    // the head (fp32 logits) and other wide outputs: enough 64x128 tiles to
    // stream W over every CU, X read once per tile instead of once per 32
    // columns.  The head always takes this kernel, the one that the fused
    // greedy choice (EpiArgmax) runs, so both see the same logits.
    if ((N >= 8192 || std::is_same_v<Epi, EpiStoreF32>) && K % 64 == 0) {
      run_bf16_v3<64, 128, 64, 2, Epi, 2, 4>(X, W, M, N, K, epi, s);
      return;
    }
    if (try_skinny(X, W, M, N, K, epi, s)) return;
    run_bf16<64, 64>(X, W, M, N, K, epi, s);
  } else if (K % 64 == 0) {
    if constexpr (std::is_same_v<Epi, EpiStoreF32>) {
      // a tile's rows share one line phase only when it lies inside one
      // phase class (M / 32 rows): 256-row tiles when the classes hold a
      // multiple of 256 rows, 128-row tiles otherwise
      const auto lines = EpiStoreF32Lines::make(epi.out, N, M);
      if (M % 32 == 0 && (M / 32) % 256 == 0)
        run_bf16_v3<256, 256, 64, 2, EpiStoreF32Lines, 4, 2>(X, W, M, N, K, lines, s);
      else
        run_bf16_v3<128, 192, 64, 2, EpiStoreF32Lines, 4, 2>(X, W, M, N, K, lines, s);
    } else {
      constexpr bool tall_ok = tall_tiles_ok<Epi>();
      switch (block_tiles(M, N, tall_ok)) {
        case Tiles::k128x96: run_bf16_v3<128, 96, 64, 2, Epi, 4, 1>(X, W, M, N, K, epi, s); break;
        case Tiles::k128x128: run_bf16_v3<128, 128, 64, 2, Epi, 4, 2>(X, W, M, N, K, epi, s); break;
        case Tiles::k256x256:
          if constexpr (tall_ok) run_bf16_v3<256, 256, 64, 2, Epi, 4, 2>(X, W, M, N, K, epi, s);
          break;
        default: run_bf16_v3<128, 192, 64, 2, Epi, 4, 2>(X, W, M, N, K, epi, s); break;
      }
    }
  } else {
    run_bf16<128, 128>(X, W, M, N, K, epi, s);
  }
}

// ================================================================ fp32 FMA kernel
// 64x64 output tile, K step 16, 256 threads, 4x4 outputs per thread
// (four consecutive columns per row, as the epilogues expect).
template <class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ X,
                                                       const float* __restrict__ W, int M, int N,
                                                       int K, Epi epi) {
  constexpr int BT = 64, BK = 16;
  __shared__ float xs[BK][BT + 4];
  __shared__ float ws[BK][BT + 4];
  const int m0 = blockIdx.y * BT, n0 = blockIdx.x * BT;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int lr = tid >> 2, lk = (tid & 3) * 4;  // loader: row, k offset
  const float* xr = X + (long long)min(m0 + lr, M - 1) * K;
  const float* wr = W + (long long)min(n0 + lr, N - 1) * K;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BK) {
    const int k = k0 + lk;
    float4 a = k < K ? *reinterpret_cast<const float4*>(xr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    float4 b = k < K ? *reinterpret_cast<const float4*>(wr + k) : make_float4(0.f, 0.f, 0.f, 0.f);
    xs[lk + 0][lr] = a.x; xs[lk + 1][lr] = a.y; xs[lk + 2][lr] = a.z; xs[lk + 3][lr] = a.w;
    ws[lk + 0][lr] = b.x; ws[lk + 1][lr] = b.y; ws[lk + 2][lr] = b.z; ws[lk + 3][lr] = b.w;
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = xs[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bv[j] = ws[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
  const int n = n0 + tx * 4;
  if (n >= N) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m < M) epi(m, n, f32x4_t{acc[i][0], acc[i][1], acc[i][2], acc[i][3]});
  }
}

template <class Epi>
static void dispatch_f32(const float* X, const float* W, int M, int N, int K, const Epi& epi,
                         hipStream_t s) {
  dim3 grid((N + 63) / 64, (M + 63) / 64);
  gemm_f32_kernel<Epi><<<grid, 256, 0, s>>>(X, W, M, N, K, epi);
}

// ================================================================ dispatch
template <typename Tact>
static void launch_typed(const Tact* X, const Tact* W, int M, int N, int K, const Epilogue& e,
                         hipStream_t s) {
  auto go = [&](const auto& epi) {
    if constexpr (sizeof(Tact) == 2)
      dispatch_bf16(X, W, M, N, K, epi, s);
    else
      dispatch_f32(X, W, M, N, K, epi, s);
  };
  switch (e.kind) {
    case EPI_STORE_F32:
      go(EpiStoreF32{(float*)e.out, N});
      break;
    case EPI_BIAS_GELU:
      go(EpiBiasGelu<Tact>{(const Tact*)e.bias, (Tact*)e.out, N});
      break;
    case EPI_BIAS_RESID:
      if (e.resid_f32 && e.out_f32 && e.resid == e.out)
        go(EpiResidInPlace<Tact>{(const Tact*)e.bias, (float*)e.out, N});
      else if (e.resid_f32 && e.out_f32)
        go(EpiBiasResid<Tact, float, float>{(const Tact*)e.bias, (const float*)e.resid, (float*)e.out, N});
      else if (e.resid_f32)
        go(EpiBiasResid<Tact, float, Tact>{(const Tact*)e.bias, (const float*)e.resid, (Tact*)e.out, N});
      else if (e.out_f32)
        go(EpiBiasResid<Tact, Tact, float>{(const Tact*)e.bias, (const Tact*)e.resid, (float*)e.out, N});
      else
        go(EpiBiasResid<Tact, Tact, Tact>{(const Tact*)e.bias, (const Tact*)e.resid, (Tact*)e.out, N});
      break;
    case EPI_QKV:
      go(EpiQKV<Tact>{(const Tact*)e.bias, (Tact*)e.q, e.kv, e.T, e.l_past, e.n_head, e.d_head, e.d,
                      FastDiv::make(e.T), FastDiv::make(e.d_head)});
      break;
  }
}

int residual_splits(bool bf16, int M, int N, int K) {
  if (!bf16 || M > 64 || N >= 8192 || N % 8 != 0) return 1;
  const int S = skinny_splits(K, (N + 15) / 16, 96);
  return S > 1 ? S : 1;
}

void launch_gemm_partials(const void* X, const void* W, int M, int N, int K, int S, float* part, hipStream_t s) {
  run_skinny<16>((const bf16_t*)X, (const bf16_t*)W, M, N, K, S, EpiPartial{part, N, (long long)M * N}, s);
}

bool head_lse_fused(bool bf16, int M, int K) { return bf16 && M > 64 && K % 64 == 0; }

int head_lse_parts(int N) { return 2 * ((N + 255) / 256); }

void launch_head_lse(const void* X, const void* W, int M, int N, int K, const int32_t* targets, void* part,
                     float* tgt, hipStream_t s) {
  const EpiLoss epi{targets, (float2*)part, tgt, N, head_lse_parts(N)};
  run_bf16_v3<256, 256, 64, 2, EpiLoss, 4, 2>((const bf16_t*)X, (const bf16_t*)W, M, N, K, epi, s);
}

bool head_argmax_fused(bool bf16, int M, int K) { return bf16 && M <= 64 && K % 64 == 0; }

int head_argmax_parts(int N) { return 4 * ((N + 127) / 128); }

void launch_head_argmax(const void* X, const void* W, int M, int N, int K, void* part, hipStream_t s) {
  const EpiArgmax epi{(float2*)part, N, head_argmax_parts(N)};
  run_bf16_v3<64, 128, 64, 2, EpiArgmax, 2, 4>((const bf16_t*)X, (const bf16_t*)W, M, N, K, epi, s);
}

void launch_gemm(bool bf16, const void* X, const void* W, int M, int N, int K, const Epilogue& e,
                 hipStream_t s) {
  if (bf16)
    launch_typed<bf16_t>((const bf16_t*)X, (const bf16_t*)W, M, N, K, e, s);
  else
    launch_typed<float>((const float*)X, (const float*)W, M, N, K, e, s);
}



}  // namespace gpt2

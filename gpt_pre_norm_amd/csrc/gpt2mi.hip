// C ABI of libgpt2mi.so (declared in include/gpt2mi.h): argument checks,
// workspace carving and the launch sequence of the decoder.
//
// Sequence per block ("Decoder Block", How it works; "Full Forward Pass", How
// it works):
//   LN1 -> c_attn GEMM (+bias, q and K/V written in place) -> causal attention
//   -> c_proj GEMM (+bias +residual, fp32 stream) -> LN2 -> c_fc GEMM (+bias,
//   GELU) -> mlp.c_proj GEMM (+bias +residual).
// Full forward: embedding -> L blocks -> ln_f -> tied head GEMM (fp32 logits).
// Decode: the same with T = 1 at position l_past, K/V appended into the cache by
// the c_attn epilogue and a split-key attention over slots 0 .. l_past.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <algorithm>
#include <cstdint>
#include <atomic>
#include <mutex>
#include <set>
#include <utility>
#include <vector>

#include "../../include/gpt2mi.h"
#include "kernels.h"

// Workspace of gpt2_decode_step_noalloc: a file-scope device array that every
// GPU the library runs on holds until the process ends (16 MiB).
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

namespace gpt2 {

namespace {
constexpr int kMaxDeviceIds = 64;
int current_device_id() {
  int dev = 0;
  return hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDeviceIds ? dev : -1;
}
}  // namespace

int device_cu_count() {
  static std::atomic<int> n[kMaxDeviceIds];
  const int dev = current_device_id();
  if (dev < 0) return 256;
  int v = n[dev].load(std::memory_order_relaxed);
  if (v <= 0) {
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0) v = 256;
    n[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

void set_dynamic_lds_limit(const void* fn, int bytes) {
  static std::mutex mu;
  static std::set<std::pair<int, const void*>> done;
  const int dev = current_device_id();
  std::lock_guard<std::mutex> lock(mu);
  if (dev < 0 || done.emplace(dev, fn).second)
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

}  // namespace gpt2

namespace {

using namespace gpt2;

constexpr size_t kAlign = 256;
constexpr size_t kHeader = 256;  // sticky device flags at offset 0
constexpr long long kMaxTokens = 1LL << 24;
constexpr int kMaxRowKeys = 8192;  // the row-wise attention keeps a row of scores in LDS

// The MFMA attention kernels take bf16 with head width 64; fp32 and other
// bf16 head widths run the row-wise kernel.
bool rows_attention(const gpt2_hparams& hp, gpt2_mode mode) {
  return mode == GPT2_FP32 || hp.n_embd / hp.n_head != 64;
}

size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// Workspace regions are carved at kAlign offsets from its start, so the start
// itself must be kAlign-aligned (every hipMalloc / torch allocation is).
bool ws_aligned(const void* ws) { return (uintptr_t)ws % kAlign == 0; }

// Weights, activations and the cache are read with 16-byte vector and DMA
// loads; ids, targets and fp32 outputs with 4-byte accesses.  NULL passes
// (NULL checks are separate).
bool al16(const void* p) { return (uintptr_t)p % 16 == 0; }
bool al4(const void* p) { return (uintptr_t)p % 4 == 0; }

struct Layout {
  size_t x, a, q, o, u, kv, part, total;
};

// K ranges of the block's two residual products (attention c_proj, mlp
// c_proj) when they are split for a decode-sized call (1: not split).
int proj_splits(const gpt2_hparams& hp, gpt2_mode mode, int M) {
  const int d = hp.n_embd;
  return residual_splits(mode == GPT2_BF16, M, d, d);
}
int fc2_splits(const gpt2_hparams& hp, gpt2_mode mode, int M) {
  const int d = hp.n_embd;
  return residual_splits(mode == GPT2_BF16, M, d, 4 * d);
}

// Workspace regions for M = B*T rows: fp32 residual x, LN output a, q, attention
// output o, MLP hidden u, K/V scratch (when no present/cache is given) and,
// for decode-sized calls, the K-range partials of the residual products.
Layout layout(const gpt2_hparams& hp, gpt2_mode mode, int B, int T) {
  const size_t act = mode == GPT2_BF16 ? 2 : 4;
  const size_t M = (size_t)B * T, d = (size_t)hp.n_embd;
  const int m = (int)std::min(M, (size_t)kMaxTokens);
  const size_t S = (size_t)std::max(proj_splits(hp, mode, m), fc2_splits(hp, mode, m));
  Layout L;
  size_t off = kHeader;
  L.x = off;  off += up(M * d * 4);
  L.a = off;  off += up(M * d * act);
  L.q = off;  off += up(M * d * act);
  L.o = off;  off += up(M * d * act);
  L.u = off;  off += up(M * 4 * d * act);
  L.kv = off; off += up(2 * M * d * act);
  L.part = off; off += S > 1 ? up(S * M * d * 4) : 0;
  L.total = off;
  return L;
}

// Generation: the decode step's regions, then the step's logits [B, V] fp32
// and the next tokens [B] int32.
struct GenLayout {
  Layout step;
  bool fused;  // the head reduces to (value, column) partials; no logits
  size_t logits, ids, total;
};

GenLayout gen_layout(const gpt2_hparams& hp, gpt2_mode mode, int B) {
  GenLayout G;
  G.step = layout(hp, mode, B, 1);
  G.fused = head_argmax_fused(mode == GPT2_BF16, B, hp.n_embd);
  size_t off = G.step.total;
  G.logits = off;  // full logits rows, or the head's partials
  off += up(G.fused ? (size_t)B * head_argmax_parts(hp.n_vocab) * 8 : (size_t)B * hp.n_vocab * 4);
  G.ids = off;     off += up((size_t)B * 4);
  G.total = off;
  return G;
}

// Loss: the forward's regions, then either the fused head's partial
// log-sum-exp states and target logits, or full fp32 logits rows.
struct LossLayout {
  Layout fwd;
  bool fused;
  size_t part, tgt, logits, total;
};

LossLayout loss_layout(const gpt2_hparams& hp, gpt2_mode mode, int B, int T) {
  LossLayout G;
  G.fwd = layout(hp, mode, B, T);
  const size_t M = (size_t)B * T;
  G.fused = head_lse_fused(mode == GPT2_BF16, (int)M, hp.n_embd);
  size_t off = G.fwd.total;
  G.part = G.tgt = G.logits = 0;
  if (G.fused) {
    G.part = off;  off += up(M * head_lse_parts(hp.n_vocab) * 8);
    G.tgt = off;   off += up(M * 4);
  } else {
    G.logits = off;  off += up(M * (size_t)hp.n_vocab * 4);
  }
  G.total = off;
  return G;
}

gpt2_status check_hparams(const gpt2_hparams* hp, gpt2_mode mode, bool need_model) {
  if (!hp) return GPT2_E_NULL;
  if (mode != GPT2_FP32 && mode != GPT2_BF16) return GPT2_E_DTYPE;
  const int d = hp->n_embd, h = hp->n_head;
  if (d <= 0 || h <= 0 || d % h != 0 || d > 2048 || d % 8 != 0) return GPT2_E_SHAPE;
  const int dh = d / h;
  if (dh % 4 != 0 || dh > 128) return GPT2_E_SHAPE;
  if (hp->n_ctx <= 0) return GPT2_E_SHAPE;
  if (!(hp->eps >= 0.f) || !std::isfinite(hp->eps)) return GPT2_E_SHAPE;
  if (need_model && (hp->n_vocab <= 0 || hp->n_layer <= 0)) return GPT2_E_SHAPE;
  return GPT2_OK;
}

bool any_null(const gpt2_block_weights& w) {
  return !w.ln1_g || !w.ln1_b || !w.attn_w || !w.attn_b || !w.proj_w || !w.proj_b || !w.ln2_g ||
         !w.ln2_b || !w.fc_w || !w.fc_b || !w.fc2_w || !w.fc2_b;
}

bool all_al16(const gpt2_block_weights& w) {
  return al16(w.ln1_g) && al16(w.ln1_b) && al16(w.attn_w) && al16(w.attn_b) && al16(w.proj_w) &&
         al16(w.proj_b) && al16(w.ln2_g) && al16(w.ln2_b) && al16(w.fc_w) && al16(w.fc_b) && al16(w.fc2_w) &&
         al16(w.fc2_b);
}

gpt2_status check_weights(const gpt2_hparams& hp, const gpt2_weights* W) {
  if (!W || !W->wte || !W->wpe || !W->lnf_g || !W->lnf_b || !W->blocks) return GPT2_E_NULL;
  for (int l = 0; l < hp.n_layer; ++l)
    if (any_null(W->blocks[l])) return GPT2_E_NULL;
  if (!al16(W->wte) || !al16(W->wpe) || !al16(W->lnf_g) || !al16(W->lnf_b)) return GPT2_E_ALIGN;
  for (int l = 0; l < hp.n_layer; ++l)
    if (!all_al16(W->blocks[l])) return GPT2_E_ALIGN;
  return GPT2_OK;
}

gpt2_status check_common(const gpt2_hparams& hp, gpt2_mode mode, int B, int T, int l_past, void* ws,
                         size_t ws_bytes) {
  if (B < 1 || T < 1 || (long long)B * T > kMaxTokens) return GPT2_E_SHAPE;
  if (l_past < 0 || (long long)l_past + T > hp.n_ctx) return GPT2_E_POSITION;
  if (rows_attention(hp, mode) && l_past + T > kMaxRowKeys) return GPT2_E_SHAPE;
  if (!ws) return GPT2_E_NULL;
  if (!ws_aligned(ws) || ws_bytes < layout(hp, mode, B, T).total) return GPT2_E_WORKSPACE;
  return GPT2_OK;
}

gpt2_status hip_status() { return hipGetLastError() == hipSuccess ? GPT2_OK : GPT2_E_HIP; }

// ---------------------------------------------------------------- static scratch
// The workspace of gpt2_decode_step_noalloc lives in `scratch` (defined above
// the namespace).  In host code its name is only a stand-in for the symbol;
// the device address, which differs per GPU, is looked up once per device and
// kept, and only that address is ever passed to kernels.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the scratch array on the current device (NULL on failure).
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

// ---------------------------------------------------------------- kernel timing
// Between gpt2_timing_begin and gpt2_timing_end every launch is bracketed by
// a HIP event pair on its stream; events are created once and reused.
enum Kern {
  K_EMBED, K_LAYERNORM, K_GEMM_C_ATTN, K_GEMM_ATTN_PROJ, K_GEMM_C_FC, K_GEMM_MLP_PROJ, K_GEMM_HEAD,
  K_ATTN_PREFILL, K_ATTN_ROWS, K_ATTN_DECODE, K_ARGMAX, K_LOSS, K_COUNT
};
const char* const kKernNames[K_COUNT] = {
    "embed", "layernorm", "gemm_c_attn", "gemm_attn_c_proj", "gemm_c_fc", "gemm_mlp_c_proj",
    "gemm_lm_head", "attn_prefill", "attn_rows", "attn_decode", "argmax", "loss"};

struct Timing {
  bool on = false;
  bool failed = false;
  std::vector<hipEvent_t> pool;
  std::vector<int> kinds;  // one per recorded pair
  size_t used = 0;         // events taken from the pool in this session

  hipEvent_t take() {
    if (used == pool.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) {
        failed = true;
        return nullptr;
      }
      pool.push_back(e);
    }
    return pool[used++];
  }
};
Timing g_timing;

// Runs launch() on stream s, bracketed by an event pair when timing is on.
template <class F>
void timed(int kind, hipStream_t s, F&& launch) {
  if (!g_timing.on) {
    launch();
    return;
  }
  hipEvent_t a = g_timing.take(), b = g_timing.take();
  if (a && hipEventRecord(a, s) != hipSuccess) g_timing.failed = true;
  launch();
  if (b && hipEventRecord(b, s) != hipSuccess) g_timing.failed = true;
  g_timing.kinds.push_back(kind);
}

struct Run {
  const gpt2_hparams& hp;
  gpt2_mode mode;
  int B, T, l_past;
  bool decode;  // single new token per sequence against the cache
  char* ws;
  Layout L;
  hipStream_t s;

  bool bf16() const { return mode == GPT2_BF16; }
  size_t act() const { return bf16() ? 2 : 4; }
  int M() const { return B * T; }
  void* at(size_t off) const { return ws + off; }

  // One pre-norm block.  x_in: block input (fp32 if x_in_f32, else act dtype);
  // x1: fp32 stream after the attention residual; y: block output.
  // ln1_done: a already holds LN1(x_in).  pend_S > 0: x_in (the fp32 stream,
  // updated in place) still lacks the previous block's mlp c_proj, held as
  // pend_S K-range partials whose bias is pend_bias; LN1 adds them first.
  // Returns the count of K-range partials this block's own mlp c_proj left
  // pending in the same way (0: its output is complete).
  int block(const gpt2_block_weights& w, const void* x_in, bool x_in_f32, float* x1, void* y, bool y_f32,
            KvView kv, bool ln1_done = false, const void* pend_bias = nullptr, int pend_S = 0) const {
    const int d = hp.n_embd, H = hp.n_head, dh = d / H, m = M();
    const bool b16 = bf16();
    void* a = at(L.a);
    void* q = at(L.q);
    void* o = at(L.o);
    void* u = at(L.u);
    float* part = (float*)at(L.part);
    // the residual products update the fp32 stream in place: decode-sized
    // ones may be split into K-range partials
    const bool in_place = x_in_f32 && x_in == (const void*)x1 && (void*)x1 == y && y_f32;
    const int s_proj = in_place ? proj_splits(hp, mode, m) : 1;
    const int s_fc2 = in_place ? fc2_splits(hp, mode, m) : 1;
    // LN1
    if (pend_S > 0)
      timed(K_LAYERNORM, s, [&] {
        launch_layernorm_reduce(x1, part, pend_S, pend_bias, w.ln1_g, w.ln1_b, a, m, d, hp.eps, s);
      });
    else if (!ln1_done)
      timed(K_LAYERNORM, s, [&] { launch_layernorm(x_in_f32 || !b16, b16, x_in, w.ln1_g, w.ln1_b, a, m, d, hp.eps, s); });
    // c_attn: q to [B,H,T,dh], k/v into the view at positions l_past..
    Epilogue e{};
    e.kind = EPI_QKV;
    e.bias = w.attn_b;
    e.q = q;
    e.kv = kv;
    e.T = T;
    e.l_past = l_past;
    e.n_head = H;
    e.d_head = dh;
    e.d = d;

    timed(K_GEMM_C_ATTN, s, [&] { launch_gemm(b16, a, w.attn_w, m, 3 * d, d, e, s); });
    // causal attention -> o [B, T, d]
    if (rows_attention(hp, mode)) {
      timed(K_ATTN_ROWS, s, [&] { launch_attn_rows(b16, q, kv, o, B, H, T, dh, l_past, s); });
    } else if (decode) {
      timed(K_ATTN_DECODE, s, [&] { launch_attn_decode_bf16((const bf16_t*)q, kv, (bf16_t*)o, B, H, l_past, s); });
    } else {
      timed(K_ATTN_PREFILL, s, [&] { launch_attn_prefill_bf16((const bf16_t*)q, kv, (bf16_t*)o, B, H, T, l_past, s); });
    }
    // c_proj + bias + residual -> x1 (fp32), then LN2
    if (s_proj > 1) {
      timed(K_GEMM_ATTN_PROJ, s, [&] { launch_gemm_partials(o, w.proj_w, m, d, d, s_proj, part, s); });
      timed(K_LAYERNORM, s, [&] {
        launch_layernorm_reduce(x1, part, s_proj, w.proj_b, w.ln2_g, w.ln2_b, a, m, d, hp.eps, s);
      });
    } else {
      Epilogue p{};
      p.kind = EPI_BIAS_RESID;
      p.bias = w.proj_b;
      p.resid = x_in;
      p.resid_f32 = x_in_f32 || !b16;
      p.out = x1;
      p.out_f32 = true;
      timed(K_GEMM_ATTN_PROJ, s, [&] { launch_gemm(b16, o, w.proj_w, m, d, d, p, s); });
      timed(K_LAYERNORM, s, [&] { launch_layernorm(true, b16, x1, w.ln2_g, w.ln2_b, a, m, d, hp.eps, s); });
    }
    // c_fc + GELU
    Epilogue f{};
    f.kind = EPI_BIAS_GELU;
    f.bias = w.fc_b;
    f.out = u;
    timed(K_GEMM_C_FC, s, [&] { launch_gemm(b16, a, w.fc_w, m, 4 * d, d, f, s); });
    // mlp.c_proj + bias + residual -> y (left as partials for the next LayerNorm when split)
    if (s_fc2 > 1) {
      timed(K_GEMM_MLP_PROJ, s, [&] { launch_gemm_partials(u, w.fc2_w, m, d, 4 * d, s_fc2, part, s); });
      return s_fc2;
    }
    Epilogue f2{};
    f2.kind = EPI_BIAS_RESID;
    f2.bias = w.fc2_b;
    f2.resid = x1;
    f2.resid_f32 = true;
    f2.out = y;
    f2.out_f32 = y_f32 || !b16;
    timed(K_GEMM_MLP_PROJ, s, [&] { launch_gemm(b16, u, w.fc2_w, m, d, 4 * d, f2, s); });
    return 0;
  }

  // Cache [B, n_layer, 2, H, cap, dh] viewed at one layer.
  KvView cache_view(void* data, int cap, int layer) const {
    const long long H = hp.n_head, dh = hp.n_embd / hp.n_head;
    const long long per_layer = 2 * H * cap * dh;
    KvView v;
    v.base = (char*)data + (size_t)layer * per_layer * act();
    v.sb = hp.n_layer * per_layer;
    v.skv = H * cap * dh;
    v.sh = (long long)cap * dh;
    return v;
  }
  // Present / scratch [B, 2, H, T, dh].
  KvView present_view(void* data) const {
    const long long H = hp.n_head, dh = hp.n_embd / hp.n_head;
    KvView v;
    v.base = data;
    v.sb = 2 * H * T * dh;
    v.skv = H * T * dh;
    v.sh = (long long)T * dh;
    return v;
  }

  // Embedding, L blocks, ln_f, head.
  void model(const gpt2_weights& W, const int32_t* ids, float* logits, const gpt2_kv* cache) const {
    trunk(W, ids, cache);
    Epilogue e{};
    e.kind = EPI_STORE_F32;
    e.out = logits;
    timed(K_GEMM_HEAD, s, [&] { launch_gemm(bf16(), at(L.a), W.wte, M(), hp.n_vocab, hp.n_embd, e, s); });
  }

  // Embedding, L blocks and ln_f: a holds LN_f(H) afterwards.
  void trunk(const gpt2_weights& W, const int32_t* ids, const gpt2_kv* cache) const {
    const int d = hp.n_embd, m = M();
    const bool b16 = bf16();
    float* x = (float*)at(L.x);
    void* a = at(L.a);
    // embedding and the first block's LN1 in one pass
    timed(K_EMBED, s, [&] {
      launch_embed_ln(b16, ids, W.wte, W.wpe, x, W.blocks[0].ln1_g, W.blocks[0].ln1_b, a, m, T, l_past, d,
                      hp.n_vocab, hp.eps, (uint32_t*)ws, s);
    });
    int pend = 0;  // K-range partials of the previous block's mlp c_proj not yet added
    for (int l = 0; l < hp.n_layer; ++l) {
      const KvView kv = cache ? cache_view(cache->data, cache->capacity, l) : present_view(at(L.kv));
      pend = block(W.blocks[l], x, true, x, x, true, kv, l == 0, l > 0 ? W.blocks[l - 1].fc2_b : nullptr, pend);
    }
    if (pend > 0) {
      const void* bias = W.blocks[hp.n_layer - 1].fc2_b;
      timed(K_LAYERNORM, s, [&] {
        launch_layernorm_reduce(x, (const float*)at(L.part), pend, bias, W.lnf_g, W.lnf_b, a, m, d, hp.eps, s);
      });
    } else {
      timed(K_LAYERNORM, s, [&] { launch_layernorm(true, b16, x, W.lnf_g, W.lnf_b, a, m, d, hp.eps, s); });
    }
  }
};

}  // namespace

extern "C" {

const char* gpt2_status_str(gpt2_status st) {
  switch (st) {
    case GPT2_OK: return "ok";
    case GPT2_E_NULL: return "a required pointer is NULL";
    case GPT2_E_SHAPE: return "unsupported or inconsistent sizes";
    case GPT2_E_DTYPE: return "unknown mode";
    case GPT2_E_POSITION: return "positions exceed n_ctx or the cache capacity";
    case GPT2_E_WORKSPACE: return "workspace too small or misaligned";
    case GPT2_E_TOKEN: return "token id outside [0, n_vocab)";
    case GPT2_E_HIP: return "HIP runtime error";
    case GPT2_E_ALIGN: return "a device pointer is misaligned";
  }
  return "unknown status";
}

size_t gpt2_workspace_size(const gpt2_hparams* hp, gpt2_mode mode, int32_t B, int32_t T) {
  if (check_hparams(hp, mode, false) != GPT2_OK) return 0;
  if (B < 1 || T < 1 || (long long)B * T > kMaxTokens) return 0;
  return layout(*hp, mode, B, T).total;
}

gpt2_status gpt2_block_forward(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_block_weights* w,
                               const void* x, void* y, int32_t B, int32_t T, void* present, void* ws,
                               size_t ws_bytes, void* stream) {
  gpt2_status st = check_hparams(hp, mode, false);
  if (st != GPT2_OK) return st;
  if (!w || !x || !y) return GPT2_E_NULL;
  if (any_null(*w)) return GPT2_E_NULL;
  if (!all_al16(*w) || !al16(x) || !al16(y) || !al16(present)) return GPT2_E_ALIGN;
  st = check_common(*hp, mode, B, T, 0, ws, ws_bytes);
  if (st != GPT2_OK) return st;
  (void)hipGetLastError();
  Run r{*hp, mode, B, T, 0, false, (char*)ws, layout(*hp, mode, B, T), (hipStream_t)stream};
  const KvView kv = r.present_view(present ? present : r.at(r.L.kv));
  r.block(*w, x, mode == GPT2_FP32, (float*)r.at(r.L.x), y, mode == GPT2_FP32, kv);
  return hip_status();
}

gpt2_status gpt2_forward(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                         const int32_t* ids, int32_t B, int32_t T, float* logits,
                         const gpt2_kv* present, void* ws, size_t ws_bytes, void* stream) {
  gpt2_status st = check_hparams(hp, mode, true);
  if (st != GPT2_OK) return st;
  if (!ids || !logits) return GPT2_E_NULL;
  if ((st = check_weights(*hp, W)) != GPT2_OK) return st;
  if (present && !present->data) return GPT2_E_NULL;
  if (!al4(ids) || !al4(logits) || (present && !al16(present->data))) return GPT2_E_ALIGN;
  st = check_common(*hp, mode, B, T, 0, ws, ws_bytes);
  if (st != GPT2_OK) return st;
  if (present && present->capacity < T) return GPT2_E_POSITION;
  (void)hipGetLastError();
  Run r{*hp, mode, B, T, 0, false, (char*)ws, layout(*hp, mode, B, T), (hipStream_t)stream};
  r.model(*W, ids, logits, present);
  return hip_status();
}

// Argument checks of the decode step, up to the workspace.
gpt2_status decode_checks(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W, const int32_t* ids,
                          int32_t B, int32_t l_past, const gpt2_kv* cache, float* logits) {
  gpt2_status st = check_hparams(hp, mode, true);
  if (st != GPT2_OK) return st;
  if (!ids || !logits || !cache) return GPT2_E_NULL;
  if (!cache->data) return GPT2_E_NULL;
  if ((st = check_weights(*hp, W)) != GPT2_OK) return st;
  if (!al4(ids) || !al4(logits) || !al16(cache->data)) return GPT2_E_ALIGN;
  if (B < 1 || B > kMaxTokens) return GPT2_E_SHAPE;
  if (l_past < 0 || (long long)l_past + 1 > hp->n_ctx || l_past >= cache->capacity) return GPT2_E_POSITION;
  if (rows_attention(*hp, mode) && l_past + 1 > kMaxRowKeys) return GPT2_E_SHAPE;
  return GPT2_OK;
}

gpt2_status gpt2_decode_step(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                             const int32_t* ids, int32_t B, int32_t l_past, const gpt2_kv* cache,
                             float* logits, void* ws, size_t ws_bytes, void* stream) {
  gpt2_status st = decode_checks(hp, mode, W, ids, B, l_past, cache, logits);
  if (st != GPT2_OK) return st;
  st = check_common(*hp, mode, B, 1, l_past, ws, ws_bytes);
  if (st != GPT2_OK) return st;
  (void)hipGetLastError();
  Run r{*hp, mode, B, 1, l_past, true, (char*)ws, layout(*hp, mode, B, 1), (hipStream_t)stream};
  r.model(*W, ids, logits, cache);
  return hip_status();
}

gpt2_status gpt2_decode_step_noalloc(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                                     const int32_t* ids, int32_t B, int32_t l_past, const gpt2_kv* cache,
                                     float* logits, void* stream) {
  gpt2_status st = decode_checks(hp, mode, W, ids, B, l_past, cache, logits);
  if (st != GPT2_OK) return st;
  const Layout L = layout(*hp, mode, B, 1);
  if (L.total > kScratchBytes) return GPT2_E_WORKSPACE;
  (void)hipGetLastError();
  char* ws = (char*)scratch_on_current_device();
  if (!ws) return GPT2_E_HIP;
  Run r{*hp, mode, B, 1, l_past, true, ws, L, (hipStream_t)stream};
  r.model(*W, ids, logits, cache);
  return hip_status();
}

gpt2_status gpt2_prefill(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                         const int32_t* ids, int32_t B, int32_t T, int32_t l_past, const gpt2_kv* cache,
                         float* logits, void* ws, size_t ws_bytes, void* stream) {
  gpt2_status st = check_hparams(hp, mode, true);
  if (st != GPT2_OK) return st;
  if (!ids || !logits || !cache) return GPT2_E_NULL;
  if (!cache->data) return GPT2_E_NULL;
  if ((st = check_weights(*hp, W)) != GPT2_OK) return st;
  if (!al4(ids) || !al4(logits) || !al16(cache->data)) return GPT2_E_ALIGN;
  st = check_common(*hp, mode, B, T, l_past, ws, ws_bytes);
  if (st != GPT2_OK) return st;
  if ((long long)l_past + T > cache->capacity) return GPT2_E_POSITION;
  (void)hipGetLastError();
  // one new token per sequence is the decode step (its attention kernel)
  Run r{*hp, mode, B, T, l_past, T == 1, (char*)ws, layout(*hp, mode, B, T), (hipStream_t)stream};
  r.model(*W, ids, logits, cache);
  return hip_status();
}

size_t gpt2_generate_workspace_size(const gpt2_hparams* hp, gpt2_mode mode, int32_t B) {
  if (check_hparams(hp, mode, true) != GPT2_OK) return 0;
  if (B < 1 || B > kMaxTokens) return 0;
  return gen_layout(*hp, mode, B).total;
}

gpt2_status gpt2_generate_greedy(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                                 const int32_t* ids, int32_t B, int32_t l_past, int32_t n_new,
                                 const gpt2_kv* cache, int32_t* out, void* ws, size_t ws_bytes, void* stream) {
  gpt2_status st = check_hparams(hp, mode, true);
  if (st != GPT2_OK) return st;
  if (!ids || !out || !cache || !ws) return GPT2_E_NULL;
  if (!cache->data) return GPT2_E_NULL;
  if ((st = check_weights(*hp, W)) != GPT2_OK) return st;
  if (!al4(ids) || !al4(out) || !al16(cache->data)) return GPT2_E_ALIGN;
  if (B < 1 || n_new < 1 || B > kMaxTokens) return GPT2_E_SHAPE;
  if (l_past < 0 || (long long)l_past + n_new > hp->n_ctx || (long long)l_past + n_new > cache->capacity)
    return GPT2_E_POSITION;
  if (rows_attention(*hp, mode) && l_past + n_new > kMaxRowKeys) return GPT2_E_SHAPE;
  const GenLayout G = gen_layout(*hp, mode, B);
  if (!ws_aligned(ws) || ws_bytes < G.total) return GPT2_E_WORKSPACE;
  (void)hipGetLastError();
  char* w = (char*)ws;
  float* logits = (float*)(w + G.logits);
  int32_t* next = (int32_t*)(w + G.ids);
  for (int i = 0; i < n_new; ++i) {
    // token i sits at position l_past + i; its logits choose token i + 1
    Run r{*hp, mode, B, 1, l_past + i, true, w, G.step, (hipStream_t)stream};
    if (G.fused) {
      const int parts = head_argmax_parts(hp->n_vocab);
      r.trunk(*W, i == 0 ? ids : next, cache);
      timed(K_GEMM_HEAD, r.s, [&] { launch_head_argmax(r.at(r.L.a), W->wte, B, hp->n_vocab, hp->n_embd, logits, r.s); });
      timed(K_ARGMAX, r.s, [&] { launch_argmax_parts(logits, parts, B, hp->n_vocab, next, out, n_new, i, r.s); });
    } else {
      r.model(*W, i == 0 ? ids : next, logits, cache);
      timed(K_ARGMAX, r.s, [&] { launch_argmax_rows(logits, B, hp->n_vocab, next, out, n_new, i, r.s); });
    }
  }
  return hip_status();
}

size_t gpt2_loss_workspace_size(const gpt2_hparams* hp, gpt2_mode mode, int32_t B, int32_t T) {
  if (check_hparams(hp, mode, true) != GPT2_OK) return 0;
  if (B < 1 || T < 1 || (long long)B * T > kMaxTokens) return 0;
  return loss_layout(*hp, mode, B, T).total;
}

gpt2_status gpt2_forward_loss(const gpt2_hparams* hp, gpt2_mode mode, const gpt2_weights* W,
                              const int32_t* ids, const int32_t* targets, int32_t B, int32_t T, float* loss,
                              const gpt2_kv* present, void* ws, size_t ws_bytes, void* stream) {
  gpt2_status st = check_hparams(hp, mode, true);
  if (st != GPT2_OK) return st;
  if (!ids || !targets || !loss) return GPT2_E_NULL;
  if ((st = check_weights(*hp, W)) != GPT2_OK) return st;
  if (present && !present->data) return GPT2_E_NULL;
  if (!al4(ids) || !al4(targets) || !al4(loss) || (present && !al16(present->data))) return GPT2_E_ALIGN;
  st = check_common(*hp, mode, B, T, 0, ws, 0);
  if (st != GPT2_OK && st != GPT2_E_WORKSPACE) return st;
  const LossLayout G = loss_layout(*hp, mode, B, T);
  if (!ws_aligned(ws) || ws_bytes < G.total) return GPT2_E_WORKSPACE;
  if (present && present->capacity < T) return GPT2_E_POSITION;
  (void)hipGetLastError();
  Run r{*hp, mode, B, T, 0, false, (char*)ws, G.fwd, (hipStream_t)stream};
  r.trunk(*W, ids, present);
  char* w = (char*)ws;
  const int m = B * T, V = hp->n_vocab, d = hp->n_embd;
  uint32_t* flags = (uint32_t*)ws;
  if (G.fused) {
    timed(K_GEMM_HEAD, r.s, [&] {
      launch_head_lse(r.at(G.fwd.a), W->wte, m, V, d, targets, w + G.part, (float*)(w + G.tgt), r.s);
    });
    timed(K_LOSS, r.s, [&] {
      launch_loss_from_parts(w + G.part, head_lse_parts(V), (const float*)(w + G.tgt), targets, m, V, loss, flags,
                             r.s);
    });
  } else {
    Epilogue e{};
    e.kind = EPI_STORE_F32;
    e.out = w + G.logits;
    timed(K_GEMM_HEAD, r.s, [&] { launch_gemm(mode == GPT2_BF16, r.at(G.fwd.a), W->wte, m, V, d, e, r.s); });
    timed(K_LOSS, r.s, [&] {
      launch_loss_from_logits((const float*)(w + G.logits), targets, m, V, loss, flags, r.s);
    });
  }
  return hip_status();
}

gpt2_status gpt2_read_device_flags(void* ws, void* stream) {
  if (!ws) return GPT2_E_NULL;
  if (hipStreamSynchronize((hipStream_t)stream) != hipSuccess) return GPT2_E_HIP;
  uint32_t flags = 0;
  if (hipMemcpy(&flags, ws, sizeof(flags), hipMemcpyDeviceToHost) != hipSuccess) return GPT2_E_HIP;
  if (flags == 0) return GPT2_OK;
  if (hipMemset(ws, 0, sizeof(flags)) != hipSuccess) return GPT2_E_HIP;
  if (hipDeviceSynchronize() != hipSuccess) return GPT2_E_HIP;
  return GPT2_E_TOKEN;
}

gpt2_status gpt2_timing_begin(void) {
  g_timing.on = true;
  g_timing.failed = false;
  g_timing.used = 0;
  g_timing.kinds.clear();
  return GPT2_OK;
}

int32_t gpt2_timing_end(gpt2_kernel_time* out, int32_t max_entries) {
  if (!g_timing.on) return -1;
  g_timing.on = false;
  if (g_timing.failed) return -1;
  double total[K_COUNT] = {};
  int count[K_COUNT] = {};
  for (size_t i = 0; i < g_timing.kinds.size(); ++i) {
    hipEvent_t a = g_timing.pool[2 * i], b = g_timing.pool[2 * i + 1];
    if (hipEventSynchronize(b) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return -1;
    total[g_timing.kinds[i]] += ms;
    count[g_timing.kinds[i]] += 1;
  }
  int32_t n = 0;
  for (int k = 0; k < K_COUNT; ++k) {
    if (count[k] == 0) continue;
    if (out && n < max_entries) {
      out[n].name = kKernNames[k];
      out[n].launches = count[k];
      out[n].total_ms = total[k];
    }
    ++n;
  }
  return n;
}

}  // extern "C"

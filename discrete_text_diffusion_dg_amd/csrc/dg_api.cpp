// C ABI of the denoise-step library: handles, argument checks, the state
// buffer layout, and the launch sequences of the four calls of include/dg.h.
#include "../../include/dg.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <thread>
#include <type_traits>
#include <vector>

#include "dg_kernels.h"

using namespace dg;

// ------------------------------------------------------------------ errors
static thread_local std::string g_err;

static dg_status fail(dg_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define DG_HIP(call)                                                                  \
  do {                                                                                \
    hipError_t e_ = (call);                                                           \
    if (e_ != hipSuccess)                                                             \
      return fail(DG_ERR_HIP, "%s failed: %s", #call, hipGetErrorString(e_));         \
  } while (0)

extern "C" const char* dg_last_error(void) { return g_err.c_str(); }

// ------------------------------------------------------------------ handles
struct LayerW {
  const float* attn_norm;
  const void* wq;
  const void* wk;
  const void* wv;
  const void* wo;
  const float* ffn_norm;
  const void* w_router;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  void* wqkv;   // owned slice of dg_model::qkv_buf: [(Hq + 2 Hkv) hd, d]
  void* pgu;    // owned slice of dg_model::pack_buf: fragment-packed gate/up (or null)
  void* pd;     // owned slice of dg_model::pack_buf: fragment-packed down (or null)
  float* sgu;   // FP8 experts: gate/up channel scales [E][2][F] (slice of pack_buf)
  float* sd;    // FP8 experts: down channel scales [E][d]
};

struct dg_model {
  dg_config cfg;
  bool fp8;              // expert weights in FP8 E4M3 (packed codes and scales only)
  size_t esz;            // bytes per weight element
  const void* emb;
  fp8e4m3* head8 = nullptr;     // owned (FP8 LM head): E4M3 codes of the embedding rows, P8 order
  float* head_scale = nullptr;  // owned (FP8 LM head): one scale per vocabulary id
  const void* w_sc;
  const float* final_norm;
  std::vector<LayerW> layers;
  void* emb_t = nullptr;     // owned: [d, V] transposed embedding (self-conditioning)
  void* qkv_buf = nullptr;   // owned: fused QKV matrices of every layer
  void* pack_buf = nullptr;  // owned: fragment-packed expert weights of every layer
};

// One captured denoise + commit step of the device-driven canvas loop and what
// it was captured for (buffers, sampler parameters, seeds, attention plan).
struct StepGraph {
  hipGraphExec_t exec = nullptr;
  std::vector<const void*> bufs;
  dg_sampler_params params{};
  std::vector<uint64_t> seeds;
  int attn_splits = -1, attn_keys_class = -1;
};

struct dg_state {
  const dg_model* m;
  int B, max_ctx, n, R;  // R = B * n rows per pass
  // per-request context lengths and canvas indices live in the state buffer
  // (ctx_dev, cidx_dev); the host keeps their largest values (capacity
  // checks, launch plans) and whether all requests still agree
  int ctx = 0, canvas_index = 0;
  bool uniform = true;
  int32_t* ctx_dev; int32_t* cidx_dev; float* inv_tab; float* lse;
  TopkPart* topk; int topk_seg;   // top-k truncated sampler: per (row, vocabulary segment) records
  int32_t* step_dev;     // [0] step of the canvas, [1] every request done, [2] loop steps completed
  volatile int32_t* progress = nullptr;      // mapped host memory: (steps completed, all done)
  int32_t* progress_dev = nullptr;           // its device address
  int64_t steps_launched = 0;                // loop steps enqueued since init (progress[0] counts them done)
  int loop_step = 0;                         // next step of the loop's current canvas
  hipStream_t cap_stream = nullptr;          // graphs are captured here (never on the null stream), launched on the caller's
  float* inv_tab_host = nullptr;             // pinned: 1 / T per step of the loop's budget
  dg_sampler_params tab_params{};
  bool tab_valid = false;
  StepGraph graph;
  int chunks, attn_splits_max, cap_tiles;   // chunks: 128-id vocabulary chunks of the head statistics
  int ctx_pad;            // max_ctx rounded up to the 64-key attention tile: K/V row stride
  size_t kv_layer_elems;  // B * Hkv * ctx_pad * hd
  // persistent
  void* kc; void* vc; float2* rope; float* s; int32_t* prev_am;
  // workspace
  float* h; void* xn; float* part; size_t part_floats; void* q; void* attn; float* attn_po; float* attn_pml;
  float* rlog; int* ridx; float* rw; int* perm; int* pos; int4* tiles; int* rcnt;
  int* n_tiles; void* act; void* y; HeadPart* hp; float* chunk_scale;
  void* ptilde; float* sc_part; int sc_splits, sc_kchunk; int32_t* tok;
  size_t total_bytes;
  // stage timing (dg_profile_enable): event pairs from a fixed pool
  uint32_t prof_mask = 0;
  std::vector<hipEvent_t> prof_ev;   // 2 * kProfPairs
  std::vector<int> prof_stage;       // stage of each used pair
  int prof_used = 0;
};

static constexpr int kProfPairs = 4096;

// Records an event pair around one stage launch when that stage is profiled.
struct StageTimer {
  dg_state* st;
  hipStream_t s;
  int pair = -1;
  StageTimer(dg_state* st_, int stage, hipStream_t s_) : st(st_), s(s_) {
    if (!(st->prof_mask & (1u << stage)) || st->prof_used >= kProfPairs) return;
    pair = st->prof_used++;
    st->prof_stage[pair] = stage;
    hipEventRecord(st->prof_ev[2 * pair], s);
  }
  ~StageTimer() {
    if (pair >= 0) hipEventRecord(st->prof_ev[2 * pair + 1], s);
  }
};

// ------------------------------------------------------------------ config checks
static dg_status check_config(const dg_config* c) {
  if (!c) return fail(DG_ERR_ARG, "config is null");
  if (c->n_layers < 1) return fail(DG_ERR_ARG, "n_layers must be >= 1");
  // the row kernels give each thread whole 4-element chunks of a row: 256..1024
  // in steps of 256 (one chunk, d / 4 threads), then multiples of 1024 (256 threads)
  if (c->d_model < 256 || c->d_model % 256 || c->d_model > kMaxModel || (c->d_model > 1024 && c->d_model % 1024))
    return fail(DG_ERR_UNSUPPORTED, "d_model must be 256, 512, 768, 1024 or a multiple of 1024 up to %d", kMaxModel);
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DG_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(DG_ERR_ARG, "n_kv_heads must divide n_q_heads");
  if (c->n_experts < 1 || c->n_experts > 128) return fail(DG_ERR_UNSUPPORTED, "n_experts must be in 1..128");
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
    return fail(DG_ERR_UNSUPPORTED, "top_k must be in 1..min(8, n_experts)");
  if (c->ffn_hidden < 64 || c->ffn_hidden % 64) return fail(DG_ERR_UNSUPPORTED, "ffn_hidden must be a multiple of 64");
  if (c->vocab < 64 || c->vocab % 64 || c->vocab > 262144)
    return fail(DG_ERR_UNSUPPORTED, "vocab must be a multiple of 64 in 64..262144");
  if (c->canvas_len < 1 || c->canvas_len > 256) return fail(DG_ERR_UNSUPPORTED, "canvas_len must be in 1..256");
  if (c->dtype != DG_DTYPE_F32 && c->dtype != DG_DTYPE_BF16) return fail(DG_ERR_ARG, "dtype must be F32 or BF16");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(DG_ERR_ARG, "rope_theta > 0 and rms_eps >= 0 required");
  if (c->expert_dtype != 0 && c->expert_dtype != DG_DTYPE_FP8_E4M3)
    return fail(DG_ERR_ARG, "expert_dtype must be 0 or DG_DTYPE_FP8_E4M3");
  if (c->expert_dtype == DG_DTYPE_FP8_E4M3 && (c->dtype != DG_DTYPE_BF16 || !expert_stream_fp8_ok(c->d_model, c->ffn_hidden)))
    return fail(DG_ERR_UNSUPPORTED, "FP8 experts need a bf16 model with d_model %% 512 == 0 and ffn_hidden %% 256 == 0");
  if (c->head_dtype != 0 && c->head_dtype != DG_DTYPE_FP8_E4M3)
    return fail(DG_ERR_ARG, "head_dtype must be 0 or DG_DTYPE_FP8_E4M3");
  if (c->head_dtype == DG_DTYPE_FP8_E4M3 && c->dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_UNSUPPORTED, "an FP8 LM head needs a bf16 model");
  return DG_OK;
}

extern "C" int32_t dg_weight_count(const dg_config* cfg) {
  if (!cfg) return -1;
  return 2 + (cfg->self_cond ? 1 : 0) + 10 * cfg->n_layers;
}

extern "C" dg_status dg_model_create(const dg_config* cfg, const void* const* w, int32_t n_weights,
                                     dg_model** out) {
  if (!out) return fail(DG_ERR_ARG, "out is null");
  *out = nullptr;
  dg_status st = check_config(cfg);
  if (st) return st;
  if (!w) return fail(DG_ERR_ARG, "weights pointer array is null");
  if (n_weights != dg_weight_count(cfg))
    return fail(DG_ERR_ARG, "expected %d weight pointers, got %d", dg_weight_count(cfg), n_weights);
  for (int i = 0; i < n_weights; ++i)
    if (!w[i]) return fail(DG_ERR_ARG, "weight pointer %d is null", i);

  dg_model* m = new dg_model();
  m->cfg = *cfg;
  m->esz = cfg->dtype == DG_DTYPE_BF16 ? 2 : 4;
  int i = 0;
  m->emb = w[i++];
  m->w_sc = cfg->self_cond ? w[i++] : nullptr;
  m->final_norm = static_cast<const float*>(w[i++]);
  const int d = cfg->d_model, hd = cfg->head_dim;
  const int nqkv = (cfg->n_q_heads + 2 * cfg->n_kv_heads) * hd;
  const size_t qkv_bytes = (size_t)nqkv * d * m->esz;
  hipError_t e = hipMalloc(&m->qkv_buf, qkv_bytes * cfg->n_layers);
  if (e != hipSuccess) { delete m; return fail(DG_ERR_HIP, "hipMalloc(qkv): %s", hipGetErrorString(e)); }
  for (int l = 0; l < cfg->n_layers; ++l) {
    LayerW L;
    L.pgu = nullptr;
    L.pd = nullptr;
    L.sgu = nullptr;
    L.sd = nullptr;
    L.attn_norm = static_cast<const float*>(w[i++]);
    L.wq = w[i++]; L.wk = w[i++]; L.wv = w[i++]; L.wo = w[i++];
    L.ffn_norm = static_cast<const float*>(w[i++]);
    L.w_router = w[i++]; L.w_gate = w[i++]; L.w_up = w[i++]; L.w_down = w[i++];
    L.wqkv = static_cast<char*>(m->qkv_buf) + qkv_bytes * l;
    char* dst = static_cast<char*>(L.wqkv);
    const size_t qb = (size_t)cfg->n_q_heads * hd * d * m->esz, kb = (size_t)cfg->n_kv_heads * hd * d * m->esz;
    if ((e = hipMemcpy(dst, L.wq, qb, hipMemcpyDeviceToDevice)) != hipSuccess ||
        (e = hipMemcpy(dst + qb, L.wk, kb, hipMemcpyDeviceToDevice)) != hipSuccess ||
        (e = hipMemcpy(dst + qb + kb, L.wv, kb, hipMemcpyDeviceToDevice)) != hipSuccess) {
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "building fused QKV: %s", hipGetErrorString(e));
    }
    m->layers.push_back(L);
  }
  m->fp8 = cfg->expert_dtype == DG_DTYPE_FP8_E4M3;
  if (m->fp8) {
    // FP8 E4M3 codes (one byte per weight) and fp32 channel scales, packed per layer
    const int E = cfg->n_experts, F = cfg->ffn_hidden;
    const size_t codes = (size_t)3 * E * F * d, scales = (size_t)E * (2 * F + d) * 4;
    const size_t per_layer = (codes + scales + 255) / 256 * 256;
    e = hipMalloc(&m->pack_buf, per_layer * cfg->n_layers);
    for (int l = 0; e == hipSuccess && l < cfg->n_layers; ++l) {
      LayerW& L = m->layers[l];
      char* base = static_cast<char*>(m->pack_buf) + per_layer * l;
      L.pgu = base;
      L.pd = base + (size_t)2 * E * F * d;
      L.sgu = reinterpret_cast<float*>(base + codes);
      L.sd = L.sgu + (size_t)2 * E * F;
      e = pack_expert_weights_fp8(static_cast<const bf16*>(L.w_gate), static_cast<const bf16*>(L.w_up),
                                  static_cast<const bf16*>(L.w_down), static_cast<fp8e4m3*>(L.pgu),
                                  static_cast<fp8e4m3*>(L.pd), L.sgu, L.sd, E, d, F, 0);
    }
    if (e != hipSuccess) {
      if (m->pack_buf) hipFree(m->pack_buf);
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "quantising expert weights: %s", hipGetErrorString(e));
    }
  } else if (expert_stream_ok(d, cfg->ffn_hidden, (int)m->esz)) {
    // expert weights repacked in MFMA-fragment order for the weight-streaming path
    const size_t per_layer = (size_t)3 * cfg->n_experts * cfg->ffn_hidden * d * m->esz;
    e = hipMalloc(&m->pack_buf, per_layer * cfg->n_layers);
    for (int l = 0; e == hipSuccess && l < cfg->n_layers; ++l) {
      LayerW& L = m->layers[l];
      char* base = static_cast<char*>(m->pack_buf) + per_layer * l;
      L.pgu = base;
      L.pd = base + per_layer / 3 * 2;
      e = cfg->dtype == DG_DTYPE_BF16
              ? pack_expert_weights<bf16>(static_cast<const bf16*>(L.w_gate), static_cast<const bf16*>(L.w_up),
                                          static_cast<const bf16*>(L.w_down), static_cast<bf16*>(L.pgu),
                                          static_cast<bf16*>(L.pd), cfg->n_experts, d, cfg->ffn_hidden, 0)
              : pack_expert_weights<float>(static_cast<const float*>(L.w_gate), static_cast<const float*>(L.w_up),
                                           static_cast<const float*>(L.w_down), static_cast<float*>(L.pgu),
                                           static_cast<float*>(L.pd), cfg->n_experts, d, cfg->ffn_hidden, 0);
    }
    if (e != hipSuccess) {
      if (m->pack_buf) hipFree(m->pack_buf);
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "packing expert weights: %s", hipGetErrorString(e));
    }
  }
  if (cfg->head_dtype == DG_DTYPE_FP8_E4M3) {
    // the LM head's copy of the embedding in E4M3 with one scale per vocabulary id
    const size_t codes = ((size_t)cfg->vocab * d + 255) / 256 * 256;
    void* buf = nullptr;
    e = hipMalloc(&buf, codes + (size_t)cfg->vocab * 4);
    if (e == hipSuccess) {
      m->head8 = static_cast<fp8e4m3*>(buf);
      m->head_scale = reinterpret_cast<float*>(static_cast<char*>(buf) + codes);
      e = pack_head_fp8(static_cast<const bf16*>(m->emb), m->head8, m->head_scale, cfg->vocab, d, 0);
    }
    if (e != hipSuccess) {
      if (buf) hipFree(buf);
      if (m->pack_buf) hipFree(m->pack_buf);
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "quantising the LM head: %s", hipGetErrorString(e));
    }
  }
  if (cfg->self_cond) {
    e = hipMalloc(&m->emb_t, (size_t)cfg->vocab * d * m->esz);
    if (e == hipSuccess) {
      e = cfg->dtype == DG_DTYPE_BF16
              ? transpose<bf16>(static_cast<const bf16*>(m->emb), static_cast<bf16*>(m->emb_t), cfg->vocab, d, 0)
              : transpose<float>(static_cast<const float*>(m->emb), static_cast<float*>(m->emb_t), cfg->vocab, d, 0);
    }
    if (e != hipSuccess) {
      if (m->emb_t) hipFree(m->emb_t);
      if (m->head8) hipFree(m->head8);
      if (m->pack_buf) hipFree(m->pack_buf);
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "building transposed embedding: %s", hipGetErrorString(e));
    }
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (m->emb_t) hipFree(m->emb_t);
    if (m->head8) hipFree(m->head8);
    if (m->pack_buf) hipFree(m->pack_buf);
    hipFree(m->qkv_buf); delete m;
    return fail(DG_ERR_HIP, "model create: %s", hipGetErrorString(e));
  }
  *out = m;
  return DG_OK;
}

extern "C" dg_status dg_model_view(const dg_model* m, int32_t which, int32_t layer, void** ptr, size_t* bytes) {
  if (!m || !ptr || !bytes) return fail(DG_ERR_ARG, "null argument");
  const dg_config& c = m->cfg;
  if (which == DG_MODEL_VIEW_HEAD_CODES || which == DG_MODEL_VIEW_HEAD_SCALES) {
    if (!m->head8) return fail(DG_ERR_ARG, "the model holds no such copy");
    *ptr = which == DG_MODEL_VIEW_HEAD_CODES ? static_cast<void*>(m->head8) : static_cast<void*>(m->head_scale);
    *bytes = which == DG_MODEL_VIEW_HEAD_CODES ? (size_t)c.vocab * c.d_model : (size_t)c.vocab * 4;
    return DG_OK;
  }
  if (layer < 0 || layer >= c.n_layers) return fail(DG_ERR_ARG, "layer %d outside 0..%d", layer, c.n_layers - 1);
  const LayerW& L = m->layers[layer];
  const size_t E = c.n_experts, F = c.ffn_hidden, d = c.d_model, es = m->fp8 ? 1 : m->esz;
  switch (which) {
    case DG_MODEL_VIEW_EXPERT_GATEUP: *ptr = L.pgu; *bytes = 2 * E * F * d * es; break;
    case DG_MODEL_VIEW_EXPERT_DOWN: *ptr = L.pd; *bytes = E * F * d * es; break;
    case DG_MODEL_VIEW_EXPERT_SCALES_GATEUP: *ptr = L.sgu; *bytes = 2 * E * F * 4; break;
    case DG_MODEL_VIEW_EXPERT_SCALES_DOWN: *ptr = L.sd; *bytes = E * d * 4; break;
    default: return fail(DG_ERR_ARG, "unknown model view %d", which);
  }
  if (*ptr == nullptr) return fail(DG_ERR_ARG, "the model holds no such copy");
  return DG_OK;
}

extern "C" void dg_model_destroy(dg_model* m) {
  if (!m) return;
  if (m->emb_t) hipFree(m->emb_t);
  if (m->head8) hipFree(m->head8);
  if (m->pack_buf) hipFree(m->pack_buf);
  if (m->qkv_buf) hipFree(m->qkv_buf);
  delete m;
}

// ------------------------------------------------------------------ state layout
namespace {
struct Layout {
  size_t off = 0;
  size_t take(size_t bytes) {
    const size_t o = off;
    off += (bytes + 255) / 256 * 256;
    return o;
  }
};

constexpr int kMaxLoopSteps = 4096;   // longest step budget of the device-driven loop

struct Offsets {
  size_t kc, vc, rope, s, prev_am, h, xn, part, q, attn, attn_po, attn_pml, rlog, ridx, rw, perm, pos, rcnt,
      tiles, n_tiles, act, y, hp, chunk_scale, ptilde, sc_part, tok, ctxv, cidx, stepv, inv_tab, lse, topk, total;
  size_t part_floats;
  int chunks, splits, cap_tiles, sc_splits, sc_kchunk;
};

// K splits of the softmax @ E contraction (K = vocabulary): enough workgroups
// to fill the chip (~512), each split at least four 128-byte K steps.  The
// chunk scales are applied in the operand loader, so splits need not follow
// the 128-id chunks.
constexpr int kHeadChunkIds = 128;   // vocabulary ids per head chunk (the sampler's unit)
void selfcond_plan(int R, int d, int V, int esz, int* splits, int* kchunk) {
  const int bm = (R >= 128 && d >= 128) ? 128 : 64;
  const int tiles = ((R + bm - 1) / bm) * ((d + bm - 1) / bm);
  const int bk = 128 / esz;
  int sp = (512 + tiles - 1) / tiles;
  const int max_sp = V / (4 * bk);
  if (sp > max_sp) sp = max_sp;
  if (sp < 1) sp = 1;
  // whole 128-id chunks per split: each split applies its chunks' probability scales
  const int kc = ((V + sp - 1) / sp + kHeadChunkIds - 1) / kHeadChunkIds * kHeadChunkIds;
  *kchunk = kc;
  *splits = (V + kc - 1) / kc;
}

Offsets layout(const dg_model* m, int B, int max_ctx) {
  const dg_config& c = m->cfg;
  const size_t es = m->esz;
  const int n = c.canvas_len, R = B * n, d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int nqkv = (Hq + 2 * Hkv) * hd, k = c.top_k, E = c.n_experts, F = c.ffn_hidden, V = c.vocab;
  Offsets o;
  o.chunks = head_chunks(V);
  selfcond_plan(R, d, V, (int)es, &o.sc_splits, &o.sc_kchunk);
  o.splits = 16;
  o.cap_tiles = expert_tile_capacity(R, k, E);
  Layout L;
  const int ctx_pad = (max_ctx + 63) / 64 * 64;
  const size_t kv = (size_t)c.n_layers * B * Hkv * ctx_pad * hd * es;
  o.kc = L.take(kv);
  o.vc = L.take(kv);
  o.rope = L.take((size_t)max_ctx * (hd / 2) * sizeof(float2));
  o.s = L.take((size_t)R * d * 4);
  o.prev_am = L.take((size_t)R * 4);
  o.h = L.take((size_t)R * d * 4);
  o.xn = L.take((size_t)R * d * es);
  const int maxN = nqkv > d ? (nqkv > E ? nqkv : E) : (d > E ? d : E);
  o.part_floats = std::max((size_t)R * maxN * 8, (size_t)1 << 22);
  o.part = L.take(o.part_floats * 4);
  o.q = L.take((size_t)R * Hq * hd * es);
  o.attn = L.take((size_t)R * Hq * hd * es);
  o.attn_po = L.take((size_t)o.splits * R * Hq * hd * 4);
  o.attn_pml = L.take((size_t)o.splits * R * Hq * 2 * 4);
  o.rlog = L.take((size_t)c.n_layers * R * E * 4);      // per layer, kept for inspection
  o.ridx = L.take((size_t)c.n_layers * R * k * 4);
  o.rw = L.take((size_t)R * k * 4);
  o.perm = L.take((size_t)R * k * 4);
  o.pos = L.take((size_t)R * k * 4);
  o.tiles = L.take((size_t)o.cap_tiles * sizeof(int4));
  o.n_tiles = L.take(4);
  o.rcnt = L.take((size_t)E * ((R + router_rows_per_block(E) - 1) / router_rows_per_block(E)) * 4);  // router counts
  o.act = L.take((size_t)R * k * F * es);
  o.y = L.take((size_t)R * k * d * 4);
  o.hp = L.take((size_t)R * o.chunks * sizeof(HeadPart));
  o.chunk_scale = L.take((size_t)R * o.chunks * 4);
  o.ptilde = c.self_cond ? L.take((size_t)R * V * es) : 0;
  o.sc_part = c.self_cond ? L.take((size_t)o.sc_splits * R * d * 4) : 0;
  o.tok = L.take((size_t)R * 4);
  o.ctxv = L.take((size_t)B * 4);
  o.cidx = L.take((size_t)B * 4);
  o.stepv = L.take(4 * 4);                          // step counter, all-done flag, steps completed
  o.inv_tab = L.take((size_t)kMaxLoopSteps * 4);
  o.lse = L.take((size_t)R * 4);
  o.topk = L.take((size_t)R * topk_segments(R, V) * sizeof(TopkPart));
  o.total = L.off;
  return o;
}
}  // namespace

extern "C" dg_status dg_state_bytes(const dg_model* m, int32_t batch, int32_t max_ctx, size_t* bytes) {
  if (!m || !bytes) return fail(DG_ERR_ARG, "null argument");
  if (batch < 1 || batch > kMaxBatch) return fail(DG_ERR_UNSUPPORTED, "batch must be in 1..%d", kMaxBatch);
  if (max_ctx < m->cfg.canvas_len) return fail(DG_ERR_ARG, "max_ctx must be >= canvas_len");
  *bytes = layout(m, batch, max_ctx).total;
  return DG_OK;
}

extern "C" dg_status dg_state_init(const dg_model* m, void* buf, size_t bytes, int32_t batch, int32_t max_ctx,
                                   dg_state** out) {
  if (!out) return fail(DG_ERR_ARG, "out is null");
  *out = nullptr;
  if (!m || !buf) return fail(DG_ERR_ARG, "null argument");
  if (batch < 1 || batch > kMaxBatch) return fail(DG_ERR_UNSUPPORTED, "batch must be in 1..%d", kMaxBatch);
  if (max_ctx < m->cfg.canvas_len) return fail(DG_ERR_ARG, "max_ctx must be >= canvas_len");
  if (reinterpret_cast<uintptr_t>(buf) % 256) return fail(DG_ERR_ARG, "state buffer must be 256-byte aligned");
  const Offsets o = layout(m, batch, max_ctx);
  if (bytes < o.total) return fail(DG_ERR_CAPACITY, "state buffer has %zu bytes, needs %zu", bytes, o.total);
  dg_state* s = new dg_state();
  char* b = static_cast<char*>(buf);
  s->m = m; s->B = batch; s->max_ctx = max_ctx; s->n = m->cfg.canvas_len; s->R = batch * s->n;
  s->chunks = o.chunks; s->attn_splits_max = o.splits; s->cap_tiles = o.cap_tiles;
  s->ctx_pad = (max_ctx + 63) / 64 * 64;
  s->kv_layer_elems = (size_t)batch * m->cfg.n_kv_heads * s->ctx_pad * m->cfg.head_dim;
  s->kc = b + o.kc; s->vc = b + o.vc; s->rope = reinterpret_cast<float2*>(b + o.rope);
  s->s = reinterpret_cast<float*>(b + o.s); s->prev_am = reinterpret_cast<int32_t*>(b + o.prev_am);
  s->h = reinterpret_cast<float*>(b + o.h); s->xn = b + o.xn;
  s->part = reinterpret_cast<float*>(b + o.part); s->part_floats = o.part_floats;
  s->sc_splits = o.sc_splits; s->sc_kchunk = o.sc_kchunk;
  s->q = b + o.q; s->attn = b + o.attn;
  s->attn_po = reinterpret_cast<float*>(b + o.attn_po); s->attn_pml = reinterpret_cast<float*>(b + o.attn_pml);
  s->rlog = reinterpret_cast<float*>(b + o.rlog); s->ridx = reinterpret_cast<int*>(b + o.ridx);
  s->rw = reinterpret_cast<float*>(b + o.rw);
  s->perm = reinterpret_cast<int*>(b + o.perm); s->pos = reinterpret_cast<int*>(b + o.pos);
  s->tiles = reinterpret_cast<int4*>(b + o.tiles); s->n_tiles = reinterpret_cast<int*>(b + o.n_tiles);
  s->rcnt = reinterpret_cast<int*>(b + o.rcnt);
  s->act = b + o.act; s->y = b + o.y;
  s->hp = reinterpret_cast<HeadPart*>(b + o.hp); s->chunk_scale = reinterpret_cast<float*>(b + o.chunk_scale);
  s->ptilde = m->cfg.self_cond ? b + o.ptilde : nullptr;
  s->sc_part = m->cfg.self_cond ? reinterpret_cast<float*>(b + o.sc_part) : nullptr;
  s->tok = reinterpret_cast<int32_t*>(b + o.tok);
  s->ctx_dev = reinterpret_cast<int32_t*>(b + o.ctxv);
  s->cidx_dev = reinterpret_cast<int32_t*>(b + o.cidx);
  s->step_dev = reinterpret_cast<int32_t*>(b + o.stepv);
  s->inv_tab = reinterpret_cast<float*>(b + o.inv_tab);
  s->lse = reinterpret_cast<float*>(b + o.lse);
  s->topk = reinterpret_cast<TopkPart*>(b + o.topk);
  s->topk_seg = topk_segments(s->R, m->cfg.vocab);
  s->total_bytes = o.total;
  // progress record of the device-driven loop in mapped host memory
  void* hp = nullptr;
  void* tabp = nullptr;
  hipError_t e = hipHostMalloc(&tabp, (size_t)kMaxLoopSteps * 4, hipHostMallocDefault);
  if (e == hipSuccess) s->inv_tab_host = static_cast<float*>(tabp);
  if (e == hipSuccess) e = hipHostMalloc(&hp, 16, hipHostMallocMapped);
  if (e == hipSuccess) {
    s->progress = static_cast<volatile int32_t*>(hp);
    s->progress[0] = 0; s->progress[1] = 0;
    void* dp = nullptr;
    e = hipHostGetDevicePointer(&dp, hp, 0);
    s->progress_dev = static_cast<int32_t*>(dp);
  }
  if (e == hipSuccess) e = hipStreamCreateWithFlags(&s->cap_stream, hipStreamNonBlocking);
  if (e == hipSuccess) e = rope_table(s->rope, max_ctx, m->cfg.head_dim, m->cfg.rope_theta, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->s, 0, (size_t)s->R * m->cfg.d_model * 4, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->prev_am, 0, (size_t)s->R * 4, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->ctx_dev, 0, (size_t)batch * 4, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->cidx_dev, 0, (size_t)batch * 4, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->step_dev, 0, 16, 0);
  // attention tiles read whole 64-key rows of V^T past the context: keep them finite
  if (e == hipSuccess) e = hipMemsetAsync(s->kc, 0, s->kv_layer_elems * m->cfg.n_layers * m->esz, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->vc, 0, s->kv_layer_elems * m->cfg.n_layers * m->esz, 0);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (s->progress) hipHostFree(const_cast<int32_t*>(s->progress));
    if (s->inv_tab_host) hipHostFree(s->inv_tab_host);
    if (s->cap_stream) hipStreamDestroy(s->cap_stream);
    delete s;
    return fail(DG_ERR_HIP, "state init: %s", hipGetErrorString(e));
  }
  *out = s;
  return DG_OK;
}

extern "C" void dg_state_destroy(dg_state* s) {
  if (!s) return;
  for (hipEvent_t e : s->prof_ev) hipEventDestroy(e);
  if (s->graph.exec) hipGraphExecDestroy(s->graph.exec);
  if (s->progress || s->inv_tab_host) hipDeviceSynchronize();   // queued loop steps use both
  if (s->progress) hipHostFree(const_cast<int32_t*>(s->progress));
  if (s->inv_tab_host) hipHostFree(s->inv_tab_host);
  if (s->cap_stream) hipStreamDestroy(s->cap_stream);
  delete s;
}

extern "C" dg_status dg_profile_enable(dg_state* st, uint32_t mask) {
  if (!st) return fail(DG_ERR_ARG, "state is null");
  if (mask && st->prof_ev.empty()) {
    st->prof_ev.resize(2 * kProfPairs);
    st->prof_stage.resize(kProfPairs);
    for (auto& e : st->prof_ev) DG_HIP(hipEventCreate(&e));
  }
  st->prof_mask = mask & ((1u << DG_NUM_STAGES) - 1);
  st->prof_used = 0;
  return DG_OK;
}

extern "C" dg_status dg_profile_read(dg_state* st, double* ms, int64_t* launches) {
  if (!st || !ms || !launches) return fail(DG_ERR_ARG, "null argument");
  for (int i = 0; i < DG_NUM_STAGES; ++i) { ms[i] = 0.0; launches[i] = 0; }
  for (int p = 0; p < st->prof_used; ++p) {
    DG_HIP(hipEventSynchronize(st->prof_ev[2 * p + 1]));
    float t = 0.f;
    DG_HIP(hipEventElapsedTime(&t, st->prof_ev[2 * p], st->prof_ev[2 * p + 1]));
    ms[st->prof_stage[p]] += (double)t;
    launches[st->prof_stage[p]] += 1;
  }
  st->prof_used = 0;
  return DG_OK;
}
extern "C" int32_t dg_state_ctx_len(const dg_state* s) { return s ? s->ctx : -1; }
extern "C" int32_t dg_state_canvas_index(const dg_state* s) { return s ? s->canvas_index : -1; }

extern "C" dg_status dg_state_view(dg_state* s, int32_t which, void** ptr, size_t* bytes) {
  if (!s || !ptr || !bytes) return fail(DG_ERR_ARG, "null argument");
  const dg_config& c = s->m->cfg;
  switch (which) {
    case DG_VIEW_K_CACHE: *ptr = s->kc; *bytes = s->kv_layer_elems * c.n_layers * s->m->esz; break;
    case DG_VIEW_V_CACHE: *ptr = s->vc; *bytes = s->kv_layer_elems * c.n_layers * s->m->esz; break;
    case DG_VIEW_SELF_COND: *ptr = s->s; *bytes = (size_t)s->R * c.d_model * 4; break;
    case DG_VIEW_PREV_ARGMAX: *ptr = s->prev_am; *bytes = (size_t)s->R * 4; break;
    case DG_VIEW_ROUTE: *ptr = s->ridx; *bytes = (size_t)c.n_layers * s->R * c.top_k * 4; break;
    case DG_VIEW_HIDDEN: *ptr = s->h; *bytes = (size_t)s->R * c.d_model * 4; break;
    case DG_VIEW_ROUTER_LOGITS: *ptr = s->rlog; *bytes = (size_t)c.n_layers * s->R * c.n_experts * 4; break;
    case DG_VIEW_ATTN_OUT: *ptr = s->attn; *bytes = (size_t)s->R * c.n_q_heads * c.head_dim * s->m->esz; break;
    case DG_VIEW_CTX_LENS: *ptr = s->ctx_dev; *bytes = (size_t)s->B * 4; break;
    case DG_VIEW_CANVAS_INDEX: *ptr = s->cidx_dev; *bytes = (size_t)s->B * 4; break;
    default: return fail(DG_ERR_ARG, "unknown view %d", which);
  }
  return DG_OK;
}

// ------------------------------------------------------------------ forward passes
namespace {

SeedArg make_seeds(const uint64_t* h, int B) {
  SeedArg a;
  memset(&a, 0, sizeof(a));
  for (int b = 0; b < B; ++b) a.v[b] = h[b];
  return a;
}

// Split plan of a small-M product, reduced if the partial buffer is too small.
// bf16 products with whole 64-element slices take the DMA loop's two K groups
// per workgroup: half as many workgroups (and split partials) as the register loop.
SplitPlan plan(const dg_state* st, int M, int N, int K, bool dma_groups = false) {
  SplitPlan p = plan_splits(M, N, K, 64, 64, (int)st->m->esz, dma_groups && st->m->esz == 2 && K % 64 == 0 ? 256 : 512);
  const int bk = 128 / (int)st->m->esz;
  while (p.splits > 1 && (size_t)p.splits * M * N > st->part_floats) {
    const int s = p.splits - 1;
    p.kchunk = ((K + s - 1) / s + bk - 1) / bk * bk;
    p.splits = (K + p.kchunk - 1) / p.kchunk;
  }
  return p;
}

int attn_splits_for(const dg_state* st, int nq, int keys) {
  const dg_config& c = st->m->cfg;
  int splits = attention_splits(st->B, nq, c.n_q_heads, c.n_kv_heads, c.head_dim, keys, (int)st->m->esz);
  return splits > st->attn_splits_max ? st->attn_splits_max : splits;
}

// Layer stack over B x nq new rows whose tokens are `tok`: request b's rows
// sit at positions ctx[b] + pos_off + i and write their K/V to the cache there.
// Requests the gate leaves out compute and write nothing.  Leaves the residual
// stream in st->h and rnd(final RMSNorm(h)) in st->xn.
template <typename T>
dg_status run_stack(dg_state* st, const int32_t* tok, int nq, bool causal, bool self_cond, Gate gate, int pos_off,
                    hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, E = c.n_experts;
  const int k = c.top_k, F = c.ffn_hidden, M = st->B * nq;
  const int nqkv = (Hq + 2 * Hkv) * hd;
  T* xn = static_cast<T*>(st->xn);
  if ((size_t)M * std::max(nqkv, std::max(d, E)) > st->part_floats ||
      (size_t)router_ksplits(M, d, E) * M * E > st->part_floats)
    return fail(DG_ERR_CAPACITY, "partial buffer too small for %d rows", M);
  const PosArg pa{st->ctx_dev, pos_off};
  {
    StageTimer tm(st, DG_STAGE_EMBED, s);
    int S = 0;
    if (self_cond) {
      const SplitPlan sp = plan(st, M, d, d);
      DG_HIP(gemm_partials_f32a<T>(st->s, d, static_cast<const T*>(m->w_sc), d, st->part, M, d, d, sp, gate, nq, s));
      S = sp.splits;
    }
    DG_HIP(embed_norm<T>(static_cast<const T*>(m->emb), tok, st->part, S, M, d, c.vocab, m->layers[0].attn_norm,
                         c.rms_eps, st->h, xn, gate, nq, s));
  }
  const int keys = st->ctx + pos_off + nq;    // the largest key count over the requests
  const int splits = attn_splits_for(st, nq, keys);
  const int cap = expert_tile_capacity(M, k, E);
  const SplitPlan p_qkv = plan(st, M, nqkv, d, true), p_o = plan(st, M, d, Hq * hd, true);
  const bool stream_ok = m->pack_buf != nullptr && !m->fp8;
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = m->layers[l];
    T* kc = static_cast<T*>(st->kc) + st->kv_layer_elems * l;
    T* vc = static_cast<T*>(st->vc) + st->kv_layer_elems * l;
    {
      StageTimer tm(st, DG_STAGE_QKV, s);
      if (qkv_rope_ok(d, hd, (int)m->esz)) {
        // one head per tile, RoPE and the cache scatter in the product's epilogue
        DG_HIP(gemm_qkv_rope<T>(xn, static_cast<const T*>(L.wqkv), M, d, hd, st->rope, static_cast<T*>(st->q), kc, vc,
                                nq, Hq, Hkv, st->ctx_pad, pa, gate, s));
      } else {
        DG_HIP(gemm_partials<T>(xn, d, static_cast<const T*>(L.wqkv), d, st->part, M, nqkv, d, p_qkv, gate, nq, s));
        DG_HIP(rope_scatter<T>(st->part, p_qkv.splits, st->rope, static_cast<T*>(st->q), kc, vc, st->B, nq, Hq, Hkv,
                               hd, st->ctx_pad, pa, gate, s));
      }
    }
    {
      StageTimer tm(st, DG_STAGE_ATTN, s);
      AttnArgs a;
      a.q = st->q; a.kc = kc; a.vc = vc; a.out = st->attn; a.part_o = st->attn_po; a.part_ml = st->attn_pml;
      a.B = st->B; a.nq = nq; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.kv_stride = st->ctx_pad;
      a.pos = pa; a.keys_max = keys; a.gate = gate;
      a.causal = causal ? 1 : 0; a.splits = splits; a.scale = (float)(1.0 / std::sqrt((double)hd));
      DG_HIP(attention<T>(a, s));
    }
    {
      StageTimer tm(st, DG_STAGE_OPROJ, s);
      DG_HIP(gemm_partials<T>(static_cast<const T*>(st->attn), Hq * hd, static_cast<const T*>(L.wo), Hq * hd,
                              st->part, M, d, Hq * hd, p_o, gate, nq, s));
    }
    float* rlog = st->rlog + (size_t)l * st->R * E;
    int* ridx = st->ridx + (size_t)l * st->R * k;
    // weight streaming while experts see at most ~64 routed rows on average
    // (the batch-1 shapes); the LDS-tiled engine once they see many; FP8
    // experts always stream (their codes feed the bf16 MFMA from registers)
    const bool stream = m->fp8 || (stream_ok && (size_t)M * k <= (size_t)64 * E);
    const int tile_rows = stream ? 64 : expert_group_tile_rows(d, F, m->esz);
    if (router_fused_ok(M, d, E, k)) {
      // few routed entries: the norm's workgroups form the router logits, top-k
      // and weights; one workgroup sorts the entries by expert
      {
        StageTimer tm(st, DG_STAGE_NORM, s);
        DG_HIP(add_norm_router<T>(st->part, p_o.splits, M, d, L.ffn_norm, c.rms_eps, st->h, xn,
                                  static_cast<const T*>(L.w_router), E, k, rlog, ridx, st->rw, gate, nq, s));
      }
      {
        StageTimer tm(st, DG_STAGE_ROUTER, s);
        DG_HIP(route_sort(ridx, M, k, E, tile_rows, st->perm, st->pos, st->tiles, st->n_tiles, s));
      }
    } else {
      {
        StageTimer tm(st, DG_STAGE_NORM, s);
        DG_HIP(add_norm<T>(st->part, p_o.splits, M, d, L.ffn_norm, c.rms_eps, st->h, xn, gate, nq, s));
      }
      {
        StageTimer tm(st, DG_STAGE_ROUTER, s);
        // the split-K partial buffer is free here (the output projection's
        // partials were consumed by add_norm); it holds the router's partial logits
        DG_HIP(router<T>(xn, static_cast<const T*>(L.w_router), M, d, E, k, rlog, ridx, st->rw, st->perm, st->pos,
                         st->tiles, st->n_tiles, tile_rows, st->rcnt, st->part, gate, nq, s));
      }
    }
    {
      StageTimer tm(st, DG_STAGE_EXPERT_UP, s);
      if (m->fp8) {
        if constexpr (std::is_same<T, bf16>::value)
          DG_HIP((expert_stream_gateup<T, fp8e4m3>(xn, st->perm, static_cast<const fp8e4m3*>(L.pgu), L.sgu,
                                                  static_cast<T*>(st->act), st->tiles, st->n_tiles, cap, d, F, s)));
      } else if (stream)
        DG_HIP((expert_stream_gateup<T, T>(xn, st->perm, static_cast<const T*>(L.pgu), nullptr,
                                          static_cast<T*>(st->act), st->tiles, st->n_tiles, cap, d, F, s)));
      else
        DG_HIP(gemm_expert_gateup<T>(xn, st->perm, static_cast<const T*>(L.w_gate), static_cast<const T*>(L.w_up),
                                     static_cast<T*>(st->act), st->tiles, st->n_tiles, cap, d, F, s,
                                     static_cast<const T*>(L.pgu)));
    }
    {
      StageTimer tm(st, DG_STAGE_EXPERT_DOWN, s);
      if (m->fp8) {
        if constexpr (std::is_same<T, bf16>::value)
          DG_HIP((expert_stream_down<T, fp8e4m3>(static_cast<const T*>(st->act), static_cast<const fp8e4m3*>(L.pd),
                                                L.sd, static_cast<T*>(st->y), st->tiles, st->n_tiles, cap, d, F,
                                                s)));
      } else if (stream)
        DG_HIP((expert_stream_down<T, T>(static_cast<const T*>(st->act), static_cast<const T*>(L.pd), nullptr,
                                        static_cast<T*>(st->y), st->tiles, st->n_tiles, cap, d, F, s)));
      else
        DG_HIP(gemm_expert_down<T>(static_cast<const T*>(st->act), static_cast<const T*>(L.w_down), static_cast<T*>(st->y),
                                   st->tiles, st->n_tiles, cap, d, F, s, static_cast<const T*>(L.pd)));
    }
    {
      StageTimer tm(st, DG_STAGE_COMBINE, s);
      const float* g_next = l + 1 < c.n_layers ? m->layers[l + 1].attn_norm : m->final_norm;
      DG_HIP(combine_norm<T>(static_cast<const T*>(st->y), st->pos, st->rw, k, M, d, g_next, c.rms_eps, st->h, xn,
                             gate, nq, s));
    }
  }
  return DG_OK;
}

template <typename T>
dg_status run_encode(dg_state* st, const int32_t* ids, int P, hipStream_t s) {
  const int n = st->n;
  const Gate all{nullptr, 0};
  for (int p0 = 0; p0 < P; p0 += n) {
    const int len = P - p0 < n ? P - p0 : n;
    // gather the chunk's tokens of every request into [B, len]
    DG_HIP(hipMemcpy2DAsync(st->tok, (size_t)len * 4, ids + p0, (size_t)P * 4, (size_t)len * 4, st->B,
                            hipMemcpyDeviceToDevice, s));
    dg_status r = run_stack<T>(st, st->tok, len, true, false, all, p0, s);
    if (r) return r;
  }
  DG_HIP(advance_context(st->ctx_dev, st->cidx_dev, st->B, P, 0, all, s));
  st->ctx += P;
  return DG_OK;
}

float step_temperature(const dg_sampler_params* p, int step) {
  const double t0 = (double)p->t_start, t1 = (double)p->t_end;
  if (p->max_steps <= 1) return (float)t0;
  return (float)(t0 + (t1 - t0) * (double)step / (double)(p->max_steps - 1));
}

float step_inv_temperature(const dg_sampler_params* p, int step) {
  return (float)(1.0 / (double)step_temperature(p, step));
}

// Step and temperature given by value (the explicit step calls).
StepInfo explicit_step(const dg_state* st, const dg_sampler_params* p, int step) {
  return StepInfo{step, step_inv_temperature(p, step), nullptr, nullptr, st->cidx_dev};
}
// Step and temperature read from the state (the device-driven loop).
StepInfo loop_step(const dg_state* st) {
  return StepInfo{0, 0.f, st->step_dev, st->inv_tab, st->cidx_dev};
}

// Sampler stage after the head statistics: the per-row merge (entropy, sample,
// arg-max, margin) and, for self-conditioning models, the next step's
// self-conditioning vector softmax(z) @ E.
template <typename T>
dg_status run_merge(dg_state* st, Gate gate, float* H, int32_t* y, int32_t* am, float* margin, hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, V = c.vocab, R = st->R;
  {
    StageTimer tm(st, DG_STAGE_SAMPLER, s);
    DG_HIP(sampler_merge(st->hp, R, st->chunks, st->n, gate, H, y, am, margin,
                         c.self_cond ? st->chunk_scale : nullptr, s));
  }
  if (c.self_cond) {
    StageTimer tm(st, DG_STAGE_SELFCOND, s);
    DG_HIP(gemm_selfcond<T>(static_cast<const T*>(st->ptilde), st->chunk_scale, st->chunks,
                            static_cast<const T*>(m->emb_t), st->sc_part, R, d, V, st->sc_splits, st->sc_kchunk,
                            gate, st->n, s));
    DG_HIP(selfcond_reduce(st->sc_part, R, d, st->sc_splits, st->s, gate, st->n, s));
  }
  return DG_OK;
}

// Sampler stage on supplied logits [R][V].
template <typename T>
dg_status run_topk_merge(dg_state* st, int top_k, const StepInfo& si, const uint64_t* seeds, Gate gate, float* H,
                         int32_t* y, int32_t* am, float* margin, hipStream_t s) {
  const dg_config& c = st->m->cfg;
  StageTimer tm(st, DG_STAGE_SAMPLER, s);
  DG_HIP(topk_merge<T>(st->topk, st->R, st->topk_seg, top_k, si, make_seeds(seeds, st->B), st->n, gate, H, y, am,
                       margin, static_cast<const T*>(st->m->emb), c.d_model, c.self_cond ? st->s : nullptr, s));
  return DG_OK;
}

template <typename T>
dg_status run_head(dg_state* st, const float* logits, const StepInfo& si, int top_k, const uint64_t* seeds,
                   Gate gate, float* H, int32_t* y, int32_t* am, float* margin, hipStream_t s) {
  const dg_config& c = st->m->cfg;
  if (top_k > 0) {
    {
      StageTimer tm(st, DG_STAGE_LM_HEAD, s);
      DG_HIP(topk_from_logits(logits, st->R, c.vocab, st->topk_seg, st->topk, gate, st->n, s));
    }
    return run_topk_merge<T>(st, top_k, si, seeds, gate, H, y, am, margin, s);
  }
  {
    StageTimer tm(st, DG_STAGE_SAMPLER, s);
    DG_HIP(head_from_logits<T>(logits, st->R, c.vocab, si, make_seeds(seeds, st->B), st->n, st->hp,
                               c.self_cond ? static_cast<T*>(st->ptilde) : nullptr, gate, s));
  }
  return run_merge<T>(st, gate, H, y, am, margin, s);
}

// One denoising round.  sc_mode: 0 no self-conditioning term, 1 the term
// (s of the previous step), as the explicit calls decide from the step; the
// loop always adds it, with s cleared at the start of each canvas.
// The LM head with the statistics epilogue over the model's head weights: the
// embedding, or its E4M3 copy with per-id scales (FP8 head).
template <typename T>
hipError_t lm_head(const dg_model* m, const T* xn, int R, const HeadArgs<T>& h, hipStream_t s) {
  const int d = m->cfg.d_model, V = m->cfg.vocab;
  if constexpr (std::is_same<T, bf16>::value) {
    if (m->head8 != nullptr) return gemm_lm_head_fp8(xn, d, m->head8, m->head_scale, R, V, d, h, s);
  }
  return gemm_lm_head<T>(xn, d, static_cast<const T*>(m->emb), d, R, V, d, h, s);
}

template <typename T>
dg_status run_denoise(dg_state* st, const int32_t* canvas, const StepInfo& si, bool sc, int top_k,
                      const uint64_t* seeds, Gate gate, float* H, int32_t* y, int32_t* am, float* margin,
                      float* logits_out, hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, V = c.vocab, R = st->R;
  dg_status r = run_stack<T>(st, canvas, st->n, false, sc, gate, 0, s);
  if (r) return r;
  T* xn = static_cast<T*>(st->xn);   // rnd(final RMSNorm(h)), written by the last combine
  if (top_k > 0) {
    {
      // the LM head keeping each row's top logits per vocabulary segment
      StageTimer tm(st, DG_STAGE_LM_HEAD, s);
      if constexpr (std::is_same<T, bf16>::value) {
        if (m->head8 != nullptr)
          DG_HIP(gemm_lm_head_topk_fp8(xn, d, m->head8, m->head_scale, R, V, d, st->topk_seg, st->topk, gate, st->n, s));
        else
          DG_HIP(gemm_lm_head_topk<T>(xn, d, static_cast<const T*>(m->emb), d, R, V, d, st->topk_seg, st->topk, gate,
                                      st->n, s));
      } else {
        DG_HIP(gemm_lm_head_topk<T>(xn, d, static_cast<const T*>(m->emb), d, R, V, d, st->topk_seg, st->topk, gate,
                                    st->n, s));
      }
    }
    if (logits_out != nullptr) {
      // the raw logits, only when a caller asks for them (the plain head writes them)
      const HeadArgs<T> h{si, make_seeds(seeds, st->B), st->n, st->hp, nullptr, logits_out, gate};
      DG_HIP(lm_head<T>(m, xn, R, h, s));
    }
    return run_topk_merge<T>(st, top_k, si, seeds, gate, H, y, am, margin, s);
  }
  {
    // the LM head with the head statistics in its epilogue (logits stored only when asked for)
    StageTimer tm(st, DG_STAGE_LM_HEAD, s);
    const HeadArgs<T> h{si, make_seeds(seeds, st->B), st->n, st->hp,
                        c.self_cond ? static_cast<T*>(st->ptilde) : nullptr, logits_out, gate};
    DG_HIP(lm_head<T>(m, xn, R, h, s));
  }
  return run_merge<T>(st, gate, H, y, am, margin, s);
}

dg_status check_params(const dg_sampler_params* p) {
  if (!p) return fail(DG_ERR_ARG, "sampler params are null");
  if (p->top_k < 0 || p->top_k > kTopkList) return fail(DG_ERR_UNSUPPORTED, "top_k must be in 0..%d", kTopkList);
  if (p->max_steps < 1) return fail(DG_ERR_ARG, "max_steps must be >= 1");
  if (p->stop_mode < 0 || p->stop_mode > 2) return fail(DG_ERR_ARG, "stop_mode must be 0, 1 or 2");
  if (!(p->t_start > 0.f) || !(p->t_end > 0.f)) return fail(DG_ERR_ARG, "temperatures must be > 0");
  if (!(p->entropy_bound >= 0.f)) return fail(DG_ERR_ARG, "entropy_bound must be >= 0");
  return DG_OK;
}

dg_status check_capacity(const dg_state* st) {
  if (st->ctx + st->n > st->max_ctx)
    return fail(DG_ERR_CAPACITY, "context %d + canvas %d exceeds max_ctx %d", st->ctx, st->n, st->max_ctx);
  return DG_OK;
}

}  // namespace

// ------------------------------------------------------------------ the calls
extern "C" dg_status dg_init_canvas(dg_state* st, int32_t* d_canvas, const uint64_t* h_seeds, dg_stream stream) {
  if (!st || !d_canvas || !h_seeds) return fail(DG_ERR_ARG, "null argument");
  const SeedArg sa = make_seeds(h_seeds, st->B);
  DG_HIP(init_canvas(d_canvas, sa, st->B, st->n, st->m->cfg.vocab, st->cidx_dev, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

extern "C" dg_status dg_encode_prompt(dg_state* st, const int32_t* d_ids, int32_t P, dg_stream stream) {
  if (!st) return fail(DG_ERR_ARG, "state is null");
  if (P < 0) return fail(DG_ERR_ARG, "P must be >= 0");
  if (P == 0) return DG_OK;
  if (!d_ids) return fail(DG_ERR_ARG, "ids are null");
  if ((long long)st->ctx + P > st->max_ctx)
    return fail(DG_ERR_CAPACITY, "context %d + prompt %d exceeds max_ctx %d", st->ctx, P, st->max_ctx);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return st->m->cfg.dtype == DG_DTYPE_BF16 ? run_encode<bf16>(st, d_ids, P, s) : run_encode<float>(st, d_ids, P, s);
}

extern "C" dg_status dg_denoise_step(dg_state* st, const int32_t* d_canvas, int32_t step,
                                     const dg_sampler_params* params, const uint64_t* h_seeds,
                                     const uint8_t* d_active, float* d_H, int32_t* d_y, int32_t* d_argmax,
                                     float* d_margin, float* d_logits, dg_stream stream) {
  if (!st || !d_canvas || !h_seeds || !d_H || !d_y || !d_argmax || !d_margin) return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_params(params);
  if (r) return r;
  if (step < 0 || step >= params->max_steps) return fail(DG_ERR_ARG, "step %d outside 0..max_steps-1", step);
  if ((r = check_capacity(st))) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const StepInfo si = explicit_step(st, params, step);
  const bool sc = st->m->cfg.self_cond && step > 0;
  const Gate g{d_active, 0};
  if (params->top_k > 0 && st->m->cfg.dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_UNSUPPORTED, "top-k truncation in the denoising step needs a bf16 model");
  return st->m->cfg.dtype == DG_DTYPE_BF16
             ? run_denoise<bf16>(st, d_canvas, si, sc, params->top_k, h_seeds, g, d_H, d_y, d_argmax, d_margin,
                                 d_logits, s)
             : run_denoise<float>(st, d_canvas, si, sc, 0, h_seeds, g, d_H, d_y, d_argmax, d_margin, d_logits, s);
}

extern "C" dg_status dg_sample_logits(dg_state* st, const float* d_logits, int32_t step,
                                      const dg_sampler_params* params, const uint64_t* h_seeds,
                                      const uint8_t* d_active, float* d_H, int32_t* d_y, int32_t* d_argmax,
                                      float* d_margin, dg_stream stream) {
  if (!st || !d_logits || !h_seeds || !d_H || !d_y || !d_argmax || !d_margin) return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_params(params);
  if (r) return r;
  if (step < 0 || step >= params->max_steps) return fail(DG_ERR_ARG, "step %d outside 0..max_steps-1", step);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const StepInfo si = explicit_step(st, params, step);
  const Gate g{d_active, 0};
  return st->m->cfg.dtype == DG_DTYPE_BF16
             ? run_head<bf16>(st, d_logits, si, params->top_k, h_seeds, g, d_H, d_y, d_argmax, d_margin, s)
             : run_head<float>(st, d_logits, si, params->top_k, h_seeds, g, d_H, d_y, d_argmax, d_margin, s);
}

extern "C" dg_status dg_sample_logits_static(const float* d_logits, int32_t rows, int32_t vocab, int32_t canvas_len,
                                             int32_t canvas_index, int32_t step, const dg_sampler_params* params,
                                             const uint64_t* h_seeds, float* d_H, int32_t* d_y, int32_t* d_argmax,
                                             float* d_margin, dg_stream stream) {
  if (!d_logits || !h_seeds || !d_H || !d_y || !d_argmax || !d_margin) return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_params(params);
  if (r) return r;
  if (step < 0 || step >= params->max_steps) return fail(DG_ERR_ARG, "step %d outside 0..max_steps-1", step);
  if (canvas_len < 1 || canvas_len > 256) return fail(DG_ERR_UNSUPPORTED, "canvas_len must be in 1..256");
  if (rows < 1 || rows % canvas_len) return fail(DG_ERR_ARG, "rows must be a positive multiple of canvas_len");
  if (rows / canvas_len > kMaxBatch) return fail(DG_ERR_UNSUPPORTED, "at most %d requests", kMaxBatch);
  if (vocab < 64 || vocab % 64 || vocab > 262144)
    return fail(DG_ERR_UNSUPPORTED, "vocab must be a multiple of 64 in 64..262144");
  if (canvas_index < 0) return fail(DG_ERR_ARG, "canvas_index must be >= 0");
  if (params->top_k != 0)
    return fail(DG_ERR_UNSUPPORTED, "the static sampler takes the full vocabulary (top_k 0), not top_k %d", params->top_k);
  const size_t need = kStaticHeadOffset + (size_t)rows * head_chunks(vocab) * sizeof(HeadPart);
  if (need > kStaticScratchBytes)
    return fail(DG_ERR_CAPACITY, "rows x 128-id chunks need %zu scratch bytes, the fixed scratch holds %zu", need,
                kStaticScratchBytes);
  void* base = nullptr;
  DG_HIP(static_scratch(&base));
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int B = rows / canvas_len;
  int32_t* cidx = static_cast<int32_t*>(base);
  HeadPart* hp = reinterpret_cast<HeadPart*>(static_cast<char*>(base) + kStaticHeadOffset);
  DG_HIP(fill_u32(cidx, (uint32_t)canvas_index, (size_t)B, s));     // every request: this canvas index
  const StepInfo si{step, step_inv_temperature(params, step), nullptr, nullptr, cidx};
  const Gate all{nullptr, 0};
  DG_HIP(head_from_logits<float>(d_logits, rows, vocab, si, make_seeds(h_seeds, B), canvas_len, hp, nullptr, all, s));
  DG_HIP(sampler_merge(hp, rows, head_chunks(vocab), canvas_len, all, d_H, d_y, d_argmax, d_margin, nullptr, s));
  return DG_OK;
}

extern "C" dg_status dg_sample_commit(dg_state* st, const float* d_H, const int32_t* d_y, const int32_t* d_argmax,
                                      int32_t* d_canvas, int32_t step, const dg_sampler_params* params,
                                      const uint64_t* h_seeds, uint8_t* d_commit_mask, int32_t* d_n_committed,
                                      uint8_t* d_done, dg_stream stream) {
  if (!st || !d_H || !d_y || !d_argmax || !d_canvas || !h_seeds || !d_commit_mask || !d_n_committed || !d_done)
    return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_params(params);
  if (r) return r;
  if (step < 0 || step >= params->max_steps) return fail(DG_ERR_ARG, "step %d outside 0..max_steps-1", step);
  const SeedArg sa = make_seeds(h_seeds, st->B);
  StageTimer tm(st, DG_STAGE_COMMIT, reinterpret_cast<hipStream_t>(stream));
  DG_HIP(commit_kernel(d_H, d_y, d_argmax, d_canvas, st->prev_am, d_commit_mask, d_n_committed, d_done, sa, st->B,
                       st->n, st->m->cfg.vocab, explicit_step(st, params, step), params->max_steps,
                       params->entropy_bound, params->stop_mode, params->stop_tau,
                       reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

// ------------------------------------------------------------------ training-side forward pass
namespace {
template <typename T>
dg_status run_corrupt_loss(dg_state* st, const int32_t* clean, const RateArg& rates, const uint64_t* seeds,
                           int32_t* corrupted, float* ce, float* loss, hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, V = c.vocab, R = st->R;
  const SeedArg sa = make_seeds(seeds, st->B);
  const Gate all{nullptr, 0};
  DG_HIP(corrupt_canvas(clean, corrupted, sa, rates, st->B, st->n, V, st->cidx_dev, s));
  dg_status r = run_stack<T>(st, corrupted, st->n, false, false, all, 0, s);
  if (r) return r;
  T* xn = static_cast<T*>(st->xn);
  {
    // the LM head at temperature 1: the chunk statistics give each row's log-sum-exp
    StageTimer tm(st, DG_STAGE_LM_HEAD, s);
    const HeadArgs<T> h{StepInfo{0, 1.0f, nullptr, nullptr, st->cidx_dev}, sa, st->n, st->hp, nullptr, nullptr, all};
    DG_HIP(lm_head<T>(m, xn, R, h, s));
  }
  {
    StageTimer tm(st, DG_STAGE_SAMPLER, s);
    DG_HIP(sampler_merge(st->hp, R, st->chunks, st->n, all, nullptr, nullptr, nullptr, nullptr, nullptr, s, st->lse));
    if constexpr (std::is_same<T, bf16>::value) {
      if (m->head8 != nullptr)
        DG_HIP(clean_token_loss_fp8(xn, m->head8, m->head_scale, clean, st->lse, st->B, st->n, d, V, ce, loss, s));
      else
        DG_HIP(clean_token_loss<T>(xn, static_cast<const T*>(m->emb), clean, st->lse, st->B, st->n, d, V, ce, loss, s));
    } else {
      DG_HIP(clean_token_loss<T>(xn, static_cast<const T*>(m->emb), clean, st->lse, st->B, st->n, d, V, ce, loss, s));
    }
  }
  return DG_OK;
}
}  // namespace

extern "C" dg_status dg_corrupt_forward_loss(dg_state* st, const int32_t* d_clean, const float* h_rates,
                                             const uint64_t* h_seeds, int32_t* d_corrupted, float* d_ce,
                                             float* d_loss, dg_stream stream) {
  if (!st || !d_clean || !h_rates || !h_seeds || !d_corrupted || !d_ce || !d_loss)
    return fail(DG_ERR_ARG, "null argument");
  RateArg ra;
  memset(&ra, 0, sizeof(ra));
  for (int b = 0; b < st->B; ++b) {
    if (!(h_rates[b] >= 0.f && h_rates[b] <= 1.f)) return fail(DG_ERR_ARG, "rate of request %d outside [0, 1]", b);
    ra.v[b] = h_rates[b];
  }
  dg_status r = check_capacity(st);
  if (r) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return st->m->cfg.dtype == DG_DTYPE_BF16
             ? run_corrupt_loss<bf16>(st, d_clean, ra, h_seeds, d_corrupted, d_ce, d_loss, s)
             : run_corrupt_loss<float>(st, d_clean, ra, h_seeds, d_corrupted, d_ce, d_loss, s);
}

extern "C" dg_status dg_commit_canvas_to_kv(dg_state* st, const int32_t* d_canvas, const uint8_t* d_which,
                                            dg_stream stream) {
  if (!st || !d_canvas) return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_capacity(st);
  if (r) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const Gate g{d_which, 0};
  r = st->m->cfg.dtype == DG_DTYPE_BF16 ? run_stack<bf16>(st, d_canvas, st->n, true, false, g, 0, s)
                                        : run_stack<float>(st, d_canvas, st->n, true, false, g, 0, s);
  if (r) return r;
  DG_HIP(advance_context(st->ctx_dev, st->cidx_dev, st->B, st->n, 1, g, s));
  st->ctx += st->n;            // largest context over the requests (those left out stay behind)
  st->canvas_index += 1;
  if (d_which != nullptr) st->uniform = false;
  return DG_OK;
}

// ------------------------------------------------------------------ the device-driven canvas loop
namespace {

// Enqueue one loop step: the denoise round of the requests not yet done, the
// commit, and the step end (step counter, all-done flag, progress record).
template <typename T>
dg_status enqueue_loop_step(dg_state* st, int32_t* canvas, const dg_sampler_params* p, const uint64_t* seeds,
                            float* H, int32_t* y, int32_t* am, float* margin, uint8_t* mask, int32_t* ncom,
                            uint8_t* done, hipStream_t s) {
  const Gate g{done, 1};
  const StepInfo si = loop_step(st);
  dg_status r = run_denoise<T>(st, canvas, si, st->m->cfg.self_cond != 0, p->top_k, seeds, g, H, y, am, margin,
                               nullptr, s);
  if (r) return r;
  {
    StageTimer tm(st, DG_STAGE_COMMIT, s);
    DG_HIP(commit_kernel(H, y, am, canvas, st->prev_am, mask, ncom, done, make_seeds(seeds, st->B), st->B, st->n,
                         st->m->cfg.vocab, si, p->max_steps, p->entropy_bound, p->stop_mode, p->stop_tau, s));
  }
  DG_HIP(step_end(done, st->B, st->step_dev, st->progress_dev, s));
  return DG_OK;
}

bool same_params(const dg_sampler_params& a, const dg_sampler_params& b) {
  return a.t_start == b.t_start && a.t_end == b.t_end && a.entropy_bound == b.entropy_bound &&
         a.stop_tau == b.stop_tau && a.max_steps == b.max_steps && a.stop_mode == b.stop_mode && a.top_k == b.top_k;
}

}  // namespace

extern "C" dg_status dg_run_canvas(dg_state* st, int32_t* d_canvas, const dg_sampler_params* params,
                                   const uint64_t* h_seeds, float* d_H, int32_t* d_y, int32_t* d_argmax,
                                   float* d_margin, uint8_t* d_commit_mask, int32_t* d_n_committed, uint8_t* d_done,
                                   int32_t first_step, int32_t n_steps, uint32_t flags, int32_t* h_result,
                                   dg_stream stream) {
  if (!st || !d_canvas || !h_seeds || !d_H || !d_y || !d_argmax || !d_margin || !d_commit_mask || !d_n_committed ||
      !d_done)
    return fail(DG_ERR_ARG, "null argument");
  dg_status r = check_params(params);
  if (r) return r;
  if (params->max_steps > kMaxLoopSteps) return fail(DG_ERR_UNSUPPORTED, "max_steps above %d", kMaxLoopSteps);
  if (params->top_k > 0 && st->m->cfg.dtype != DG_DTYPE_BF16)
    return fail(DG_ERR_UNSUPPORTED, "top-k truncation in the denoising step needs a bf16 model");
  if (first_step < 0 || first_step >= params->max_steps)
    return fail(DG_ERR_ARG, "first_step %d outside 0..max_steps-1", first_step);
  if (n_steps < 1 || n_steps > params->max_steps - first_step)
    return fail(DG_ERR_ARG, "n_steps %d outside 1..%d", n_steps, params->max_steps - first_step);
  if (first_step > 0 && first_step != st->loop_step)
    return fail(DG_ERR_ARG, "first_step %d does not continue the canvas (next step %d)", first_step, st->loop_step);
  if (flags & ~(uint32_t)(DG_RUN_GRAPH | DG_RUN_EARLY_EXIT | DG_RUN_COMMIT_KV))
    return fail(DG_ERR_ARG, "unknown flags 0x%x", flags);
  if ((r = check_capacity(st))) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool bf = st->m->cfg.dtype == DG_DTYPE_BF16;
  const int S = params->max_steps;
  // the temperature table of this budget: copied from pinned host memory,
  // rewritten only when the parameters change (after the copies still queued
  // from it have run)
  if (!st->tab_valid || !same_params(st->tab_params, *params)) {
    if (st->tab_valid) DG_HIP(hipStreamSynchronize(s));
    for (int t = 0; t < S; ++t) st->inv_tab_host[t] = step_inv_temperature(params, t);
    st->tab_params = *params;
    st->tab_valid = true;
  }
  if (first_step == 0) {
    DG_HIP(hipMemcpyAsync(st->inv_tab, st->inv_tab_host, (size_t)S * 4, hipMemcpyHostToDevice, s));
    // canvas set-up: tokens, cleared done flags, self-conditioning vector and step counter
    DG_HIP(init_canvas(d_canvas, make_seeds(h_seeds, st->B), st->B, st->n, st->m->cfg.vocab, st->cidx_dev, s));
    DG_HIP(fill_u8(d_done, 0, (size_t)st->B, s));
    if (st->m->cfg.self_cond) DG_HIP(fill_u32(st->s, 0u, (size_t)st->R * st->m->cfg.d_model, s));
    DG_HIP(fill_u32(st->step_dev, 0u, 2, s));      // step counter and all-done flag (not the completed count)
    st->loop_step = 0;
  }

  const int keys = st->ctx + st->n;
  const int splits = attn_splits_for(st, st->n, keys);
  const int keys_class = attention_launch_class(st->B, st->n, st->m->cfg.n_q_heads, st->m->cfg.n_kv_heads,
                                                st->m->cfg.head_dim, keys);
  const uint32_t saved_prof = st->prof_mask;
  if (flags & DG_RUN_GRAPH) {
    std::vector<const void*> bufs{d_canvas, d_H, d_y, d_argmax, d_margin, d_commit_mask, d_n_committed, d_done};
    std::vector<uint64_t> seeds(h_seeds, h_seeds + st->B);
    StepGraph& G = st->graph;
    const bool reuse = G.exec && G.bufs == bufs && same_params(G.params, *params) && G.seeds == seeds &&
                       G.attn_splits == splits && G.attn_keys_class == keys_class;
    if (!reuse) {
      if (G.exec) { hipGraphExecDestroy(G.exec); G.exec = nullptr; }
      st->prof_mask = 0;      // no event records inside the graph
      hipGraph_t graph = nullptr;
      hipStream_t cs = st->cap_stream;
      DG_HIP(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal));
      r = bf ? enqueue_loop_step<bf16>(st, d_canvas, params, h_seeds, d_H, d_y, d_argmax, d_margin, d_commit_mask,
                                       d_n_committed, d_done, cs)
             : enqueue_loop_step<float>(st, d_canvas, params, h_seeds, d_H, d_y, d_argmax, d_margin, d_commit_mask,
                                        d_n_committed, d_done, cs);
      const hipError_t ec = hipStreamEndCapture(cs, &graph);
      st->prof_mask = saved_prof;
      if (r) { if (graph) hipGraphDestroy(graph); return r; }
      if (ec != hipSuccess) return fail(DG_ERR_HIP, "graph capture: %s", hipGetErrorString(ec));
      const hipError_t ei = hipGraphInstantiate(&G.exec, graph, nullptr, nullptr, 0);
      hipGraphDestroy(graph);
      if (ei != hipSuccess) { G.exec = nullptr; return fail(DG_ERR_HIP, "graph instantiate: %s", hipGetErrorString(ei)); }
      G.bufs = bufs; G.params = *params; G.seeds = seeds; G.attn_splits = splits; G.attn_keys_class = keys_class;
    }
  }
  // the steps: at most S; with DG_RUN_EARLY_EXIT the host stays at most two
  // steps ahead of the device (reading the progress record in mapped host
  // memory, no synchronisation) and stops issuing once every request is done
  const int64_t base = st->steps_launched;
  int issued = 0;
  bool seen_done = false;
  for (int t = first_step; t < first_step + n_steps; ++t) {
    if (flags & DG_RUN_GRAPH) {
      DG_HIP(hipGraphLaunch(st->graph.exec, s));
    } else {
      r = bf ? enqueue_loop_step<bf16>(st, d_canvas, params, h_seeds, d_H, d_y, d_argmax, d_margin, d_commit_mask,
                                       d_n_committed, d_done, s)
             : enqueue_loop_step<float>(st, d_canvas, params, h_seeds, d_H, d_y, d_argmax, d_margin, d_commit_mask,
                                        d_n_committed, d_done, s);
      if (r) return r;
    }
    ++issued;
    ++st->steps_launched;
    if (flags & DG_RUN_EARLY_EXIT) {
      const int64_t need = st->steps_launched - 2;
      bool all_done = false;
      for (;;) {
        const int64_t got = (int64_t)__atomic_load_n(const_cast<int32_t*>(&st->progress[0]), __ATOMIC_ACQUIRE);
        if (got > base) all_done = __atomic_load_n(const_cast<int32_t*>(&st->progress[1]), __ATOMIC_RELAXED) != 0;
        if (all_done || got >= need) break;
        std::this_thread::yield();
      }
      if (all_done) { seen_done = true; break; }
    }
  }
  st->loop_step = first_step + issued;
  const bool finished = seen_done || st->loop_step == S;
  if (h_result) { h_result[0] = issued; h_result[1] = finished ? 1 : 0; }
  if ((flags & DG_RUN_COMMIT_KV) && finished) {
    r = dg_commit_canvas_to_kv(st, d_canvas, nullptr, stream);
    if (r) return r;
  }
  return DG_OK;
}

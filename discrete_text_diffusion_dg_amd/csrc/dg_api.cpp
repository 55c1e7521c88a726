// C ABI of the denoise-step library: handles, argument checks, the state
// buffer layout, and the launch sequences of the four calls of include/dg.h.
#include "../../include/dg.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
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
};

struct dg_model {
  dg_config cfg;
  size_t esz;            // bytes per weight element
  const void* emb;
  const void* w_sc;
  const float* final_norm;
  std::vector<LayerW> layers;
  void* emb_t = nullptr;     // owned: [d, V] transposed embedding (self-conditioning)
  void* qkv_buf = nullptr;   // owned: fused QKV matrices of every layer
};

struct dg_state {
  const dg_model* m;
  int B, max_ctx, n, R;  // R = B * n rows per pass
  int ctx = 0, canvas_index = 0;
  int chunks, clen, attn_splits_max, cap_tiles;
  size_t kv_layer_elems;  // B * Hkv * max_ctx * hd
  // persistent
  void* kc; void* vc; float2* rope; float* s; int32_t* prev_am;
  // workspace
  float* h; void* xn; float* qkv; void* q; void* attn; float* attn_po; float* attn_pml;
  float* rlog; int* ridx; float* rw; int* chunk_counts; int* perm; int* pos; int4* tiles;
  int* n_tiles; void* act; float* y; float* logits; HeadPart* hp; float* chunk_scale;
  void* ptilde; float* sc_part; int32_t* tok;
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
  if (c->d_model < 64 || c->d_model % 64) return fail(DG_ERR_UNSUPPORTED, "d_model must be a positive multiple of 64");
  if (c->head_dim != 64 && c->head_dim != 128) return fail(DG_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(DG_ERR_ARG, "n_kv_heads must divide n_q_heads");
  if (c->n_experts < 1 || c->n_experts > 128) return fail(DG_ERR_UNSUPPORTED, "n_experts must be in 1..128");
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_experts)
    return fail(DG_ERR_UNSUPPORTED, "top_k must be in 1..min(8, n_experts)");
  if (c->ffn_hidden < 64 || c->ffn_hidden % 64) return fail(DG_ERR_UNSUPPORTED, "ffn_hidden must be a multiple of 64");
  if (c->vocab < 64 || c->vocab % 64) return fail(DG_ERR_UNSUPPORTED, "vocab must be a positive multiple of 64");
  if (c->canvas_len < 1 || c->canvas_len > 256) return fail(DG_ERR_UNSUPPORTED, "canvas_len must be in 1..256");
  if (c->dtype != DG_DTYPE_F32 && c->dtype != DG_DTYPE_BF16) return fail(DG_ERR_ARG, "dtype must be F32 or BF16");
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return fail(DG_ERR_ARG, "rope_theta > 0 and rms_eps >= 0 required");
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
  if (cfg->self_cond) {
    e = hipMalloc(&m->emb_t, (size_t)cfg->vocab * d * m->esz);
    if (e == hipSuccess) {
      e = cfg->dtype == DG_DTYPE_BF16
              ? transpose<bf16>(static_cast<const bf16*>(m->emb), static_cast<bf16*>(m->emb_t), cfg->vocab, d, 0)
              : transpose<float>(static_cast<const float*>(m->emb), static_cast<float*>(m->emb_t), cfg->vocab, d, 0);
    }
    if (e != hipSuccess) {
      if (m->emb_t) hipFree(m->emb_t);
      hipFree(m->qkv_buf); delete m;
      return fail(DG_ERR_HIP, "building transposed embedding: %s", hipGetErrorString(e));
    }
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    if (m->emb_t) hipFree(m->emb_t);
    hipFree(m->qkv_buf); delete m;
    return fail(DG_ERR_HIP, "model create: %s", hipGetErrorString(e));
  }
  *out = m;
  return DG_OK;
}

extern "C" void dg_model_destroy(dg_model* m) {
  if (!m) return;
  if (m->emb_t) hipFree(m->emb_t);
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

struct Offsets {
  size_t kc, vc, rope, s, prev_am, h, xn, qkv, q, attn, attn_po, attn_pml, rlog, ridx, rw, chunk_counts, perm, pos,
      tiles, n_tiles, act, y, logits, hp, chunk_scale, ptilde, sc_part, tok, total;
  int chunks, clen, splits, cap_tiles;
};

Offsets layout(const dg_model* m, int B, int max_ctx) {
  const dg_config& c = m->cfg;
  const size_t es = m->esz;
  const int n = c.canvas_len, R = B * n, d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int nqkv = (Hq + 2 * Hkv) * hd, k = c.top_k, E = c.n_experts, F = c.ffn_hidden, V = c.vocab;
  Offsets o;
  o.chunks = sampler_chunks(V);
  o.clen = sampler_chunk_len(V, o.chunks);
  o.splits = 16;
  o.cap_tiles = expert_tile_capacity(R, k, E);
  Layout L;
  const size_t kv = (size_t)c.n_layers * B * Hkv * max_ctx * hd * es;
  o.kc = L.take(kv);
  o.vc = L.take(kv);
  o.rope = L.take((size_t)max_ctx * (hd / 2) * sizeof(float2));
  o.s = L.take((size_t)R * d * 4);
  o.prev_am = L.take((size_t)R * 4);
  o.h = L.take((size_t)R * d * 4);
  o.xn = L.take((size_t)R * d * es);
  o.qkv = L.take((size_t)R * nqkv * 4);
  o.q = L.take((size_t)R * Hq * hd * es);
  o.attn = L.take((size_t)R * Hq * hd * es);
  o.attn_po = L.take((size_t)o.splits * R * Hq * hd * 4);
  o.attn_pml = L.take((size_t)o.splits * R * Hq * 2 * 4);
  o.rlog = L.take((size_t)c.n_layers * R * E * 4);      // per layer, kept for inspection
  o.ridx = L.take((size_t)c.n_layers * R * k * 4);
  o.rw = L.take((size_t)R * k * 4);
  o.chunk_counts = L.take((size_t)((R + 255) / 256) * E * 4);
  o.perm = L.take((size_t)R * k * 4);
  o.pos = L.take((size_t)R * k * 4);
  o.tiles = L.take((size_t)o.cap_tiles * sizeof(int4));
  o.n_tiles = L.take(4);
  o.act = L.take((size_t)R * k * F * es);
  o.y = L.take((size_t)R * k * d * 4);
  o.logits = L.take((size_t)R * V * 4);
  o.hp = L.take((size_t)R * o.chunks * sizeof(HeadPart));
  o.chunk_scale = L.take((size_t)R * o.chunks * 4);
  o.ptilde = c.self_cond ? L.take((size_t)R * V * es) : 0;
  o.sc_part = c.self_cond ? L.take((size_t)o.chunks * R * d * 4) : 0;
  o.tok = L.take((size_t)R * 4);
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
  s->chunks = o.chunks; s->clen = o.clen; s->attn_splits_max = o.splits; s->cap_tiles = o.cap_tiles;
  s->kv_layer_elems = (size_t)batch * m->cfg.n_kv_heads * max_ctx * m->cfg.head_dim;
  s->kc = b + o.kc; s->vc = b + o.vc; s->rope = reinterpret_cast<float2*>(b + o.rope);
  s->s = reinterpret_cast<float*>(b + o.s); s->prev_am = reinterpret_cast<int32_t*>(b + o.prev_am);
  s->h = reinterpret_cast<float*>(b + o.h); s->xn = b + o.xn; s->qkv = reinterpret_cast<float*>(b + o.qkv);
  s->q = b + o.q; s->attn = b + o.attn;
  s->attn_po = reinterpret_cast<float*>(b + o.attn_po); s->attn_pml = reinterpret_cast<float*>(b + o.attn_pml);
  s->rlog = reinterpret_cast<float*>(b + o.rlog); s->ridx = reinterpret_cast<int*>(b + o.ridx);
  s->rw = reinterpret_cast<float*>(b + o.rw); s->chunk_counts = reinterpret_cast<int*>(b + o.chunk_counts);
  s->perm = reinterpret_cast<int*>(b + o.perm); s->pos = reinterpret_cast<int*>(b + o.pos);
  s->tiles = reinterpret_cast<int4*>(b + o.tiles); s->n_tiles = reinterpret_cast<int*>(b + o.n_tiles);
  s->act = b + o.act; s->y = reinterpret_cast<float*>(b + o.y); s->logits = reinterpret_cast<float*>(b + o.logits);
  s->hp = reinterpret_cast<HeadPart*>(b + o.hp); s->chunk_scale = reinterpret_cast<float*>(b + o.chunk_scale);
  s->ptilde = m->cfg.self_cond ? b + o.ptilde : nullptr;
  s->sc_part = m->cfg.self_cond ? reinterpret_cast<float*>(b + o.sc_part) : nullptr;
  s->tok = reinterpret_cast<int32_t*>(b + o.tok);
  s->total_bytes = o.total;
  hipError_t e = rope_table(s->rope, max_ctx, m->cfg.head_dim, m->cfg.rope_theta, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->s, 0, (size_t)s->R * m->cfg.d_model * 4, 0);
  if (e == hipSuccess) e = hipMemsetAsync(s->prev_am, 0, (size_t)s->R * 4, 0);
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) { delete s; return fail(DG_ERR_HIP, "state init: %s", hipGetErrorString(e)); }
  *out = s;
  return DG_OK;
}

extern "C" void dg_state_destroy(dg_state* s) {
  if (!s) return;
  for (hipEvent_t e : s->prof_ev) hipEventDestroy(e);
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

// Layer stack over B x nq new rows at positions ctx..ctx+nq-1 whose tokens are
// st->tok (or `tok`), writing their K/V to the cache.  Leaves the residual
// stream in st->h.
template <typename T>
dg_status run_stack(dg_state* st, const int32_t* tok, int nq, bool causal, bool self_cond, hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, hd = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads, E = c.n_experts;
  const int k = c.top_k, F = c.ffn_hidden, M = st->B * nq;
  const int nqkv = (Hq + 2 * Hkv) * hd;
  T* xn = static_cast<T*>(st->xn);
  {
    StageTimer tm(st, DG_STAGE_EMBED, s);
    if (self_cond)
      DG_HIP(gemm_embed_selfcond<T>(st->s, static_cast<const T*>(m->w_sc), static_cast<const T*>(m->emb), tok,
                                    st->h, M, d, c.vocab, s));
    else
      DG_HIP(embed_rows<T>(static_cast<const T*>(m->emb), tok, st->h, M, d, c.vocab, s));
  }
  const int keys = st->ctx + nq;
  int splits = attention_splits(st->B, nq, Hq, Hkv, keys);
  if (splits > st->attn_splits_max) splits = st->attn_splits_max;
  const int cap = expert_tile_capacity(M, k, E);
  for (int l = 0; l < c.n_layers; ++l) {
    const LayerW& L = m->layers[l];
    T* kc = static_cast<T*>(st->kc) + st->kv_layer_elems * l;
    T* vc = static_cast<T*>(st->vc) + st->kv_layer_elems * l;
    {
      StageTimer tm(st, DG_STAGE_NORM, s);
      DG_HIP(rmsnorm_rows<T>(st->h, L.attn_norm, xn, M, d, c.rms_eps, s));
    }
    {
      StageTimer tm(st, DG_STAGE_QKV, s);
      DG_HIP(gemm_store_f32<T>(xn, d, static_cast<const T*>(L.wqkv), d, st->qkv, nqkv, M, nqkv, d, s));
      DG_HIP(rope_scatter<T>(st->qkv, st->rope, static_cast<T*>(st->q), kc, vc, st->B, nq, Hq, Hkv, hd,
                             st->max_ctx, st->ctx, s));
    }
    {
      StageTimer tm(st, DG_STAGE_ATTN, s);
      AttnArgs a;
      a.q = st->q; a.kc = kc; a.vc = vc; a.out = st->attn; a.part_o = st->attn_po; a.part_ml = st->attn_pml;
      a.B = st->B; a.nq = nq; a.Hq = Hq; a.Hkv = Hkv; a.hd = hd; a.max_ctx = st->max_ctx; a.ctx = st->ctx;
      a.causal = causal ? 1 : 0; a.splits = splits; a.scale = (float)(1.0 / std::sqrt((double)hd));
      DG_HIP(attention<T>(a, s));
    }
    {
      StageTimer tm(st, DG_STAGE_OPROJ, s);
      DG_HIP(gemm_resid_add<T>(static_cast<const T*>(st->attn), Hq * hd, static_cast<const T*>(L.wo), Hq * hd,
                               st->h, d, M, d, Hq * hd, s));
    }
    {
      StageTimer tm(st, DG_STAGE_NORM, s);
      DG_HIP(rmsnorm_rows<T>(st->h, L.ffn_norm, xn, M, d, c.rms_eps, s));
    }
    {
      StageTimer tm(st, DG_STAGE_ROUTER, s);
      float* rlog = st->rlog + (size_t)l * st->R * E;
      int* ridx = st->ridx + (size_t)l * st->R * k;
      DG_HIP(gemm_store_f32<T>(xn, d, static_cast<const T*>(L.w_router), d, rlog, E, M, E, d, s));
      DG_HIP(router_topk(rlog, M, E, k, ridx, st->rw, s));
      DG_HIP(route_bucket(ridx, M, k, E, st->chunk_counts, st->perm, st->pos, st->tiles, st->n_tiles, s));
    }
    {
      StageTimer tm(st, DG_STAGE_EXPERT_UP, s);
      DG_HIP(gemm_expert_gateup<T>(xn, st->perm, static_cast<const T*>(L.w_gate), static_cast<const T*>(L.w_up),
                                   static_cast<T*>(st->act), st->tiles, st->n_tiles, cap, d, F, s));
    }
    {
      StageTimer tm(st, DG_STAGE_EXPERT_DOWN, s);
      DG_HIP(gemm_expert_down<T>(static_cast<const T*>(st->act), static_cast<const T*>(L.w_down), st->y,
                                 st->tiles, st->n_tiles, cap, d, F, s));
    }
    {
      StageTimer tm(st, DG_STAGE_COMBINE, s);
      DG_HIP(moe_combine(st->y, st->pos, st->rw, st->h, M, k, d, s));
    }
  }
  return DG_OK;
}

template <typename T>
dg_status run_encode(dg_state* st, const int32_t* ids, int P, hipStream_t s) {
  const int n = st->n;
  for (int p0 = 0; p0 < P; p0 += n) {
    const int len = P - p0 < n ? P - p0 : n;
    // gather the chunk's tokens of every request into [B, len]
    DG_HIP(hipMemcpy2DAsync(st->tok, (size_t)len * 4, ids + p0, (size_t)P * 4, (size_t)len * 4, st->B,
                            hipMemcpyDeviceToDevice, s));
    dg_status r = run_stack<T>(st, st->tok, len, true, false, s);
    if (r) return r;
    st->ctx += len;
  }
  return DG_OK;
}

float step_temperature(const dg_sampler_params* p, int step) {
  const double t0 = (double)p->t_start, t1 = (double)p->t_end;
  if (p->max_steps <= 1) return (float)t0;
  return (float)(t0 + (t1 - t0) * (double)step / (double)(p->max_steps - 1));
}

template <typename T>
dg_status run_denoise(dg_state* st, const int32_t* canvas, int step, const dg_sampler_params* p,
                      const uint64_t* seeds, const uint8_t* active, float* H, int32_t* y, int32_t* am,
                      float* margin, float* logits_out, hipStream_t s) {
  const dg_model* m = st->m;
  const dg_config& c = m->cfg;
  const int d = c.d_model, V = c.vocab, R = st->R;
  const bool sc = c.self_cond && step > 0;
  dg_status r = run_stack<T>(st, canvas, st->n, false, sc, s);
  if (r) return r;
  T* xn = static_cast<T*>(st->xn);
  {
    StageTimer tm(st, DG_STAGE_NORM, s);
    DG_HIP(rmsnorm_rows<T>(st->h, m->final_norm, xn, R, d, c.rms_eps, s));
  }
  float* logits = logits_out ? logits_out : st->logits;
  {
    StageTimer tm(st, DG_STAGE_LM_HEAD, s);
    DG_HIP(gemm_store_f32<T>(xn, d, static_cast<const T*>(m->emb), d, logits, V, R, V, d, s));
  }
  const float T_t = step_temperature(p, step);
  const float inv_t = (float)(1.0 / (double)T_t);
  const SeedArg sa = make_seeds(seeds, st->B);
  T* pt = c.self_cond ? static_cast<T*>(st->ptilde) : nullptr;
  {
    StageTimer tm(st, DG_STAGE_SAMPLER, s);
    DG_HIP(sampler_partial<T>(logits, R, V, st->chunks, inv_t, sa, st->n, st->canvas_index, step, st->hp, pt, s));
    DG_HIP(sampler_merge(st->hp, R, st->chunks, st->n, active, H, y, am, margin,
                         c.self_cond ? st->chunk_scale : nullptr, s));
  }
  if (c.self_cond) {
    StageTimer tm(st, DG_STAGE_SELFCOND, s);
    DG_HIP(gemm_splitk<T>(pt, V, static_cast<const T*>(m->emb_t), V, st->sc_part, R, d, V, st->chunks, st->clen,
                          s));
    DG_HIP(selfcond_reduce(st->sc_part, st->chunk_scale, R, d, st->chunks, st->s, s));
  }
  return DG_OK;
}

dg_status check_params(const dg_sampler_params* p) {
  if (!p) return fail(DG_ERR_ARG, "sampler params are null");
  if (p->max_steps < 1) return fail(DG_ERR_ARG, "max_steps must be >= 1");
  if (p->stop_mode < 0 || p->stop_mode > 2) return fail(DG_ERR_ARG, "stop_mode must be 0, 1 or 2");
  if (!(p->t_start > 0.f) || !(p->t_end > 0.f)) return fail(DG_ERR_ARG, "temperatures must be > 0");
  if (!(p->entropy_bound >= 0.f)) return fail(DG_ERR_ARG, "entropy_bound must be >= 0");
  return DG_OK;
}

}  // namespace

// ------------------------------------------------------------------ the calls
extern "C" dg_status dg_init_canvas(dg_state* st, int32_t* d_canvas, const uint64_t* h_seeds, dg_stream stream) {
  if (!st || !d_canvas || !h_seeds) return fail(DG_ERR_ARG, "null argument");
  const SeedArg sa = make_seeds(h_seeds, st->B);
  DG_HIP(init_canvas(d_canvas, sa, st->B, st->n, st->m->cfg.vocab, st->canvas_index,
                     reinterpret_cast<hipStream_t>(stream)));
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
  if (st->ctx + st->n > st->max_ctx)
    return fail(DG_ERR_CAPACITY, "context %d + canvas %d exceeds max_ctx %d", st->ctx, st->n, st->max_ctx);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  return st->m->cfg.dtype == DG_DTYPE_BF16
             ? run_denoise<bf16>(st, d_canvas, step, params, h_seeds, d_active, d_H, d_y, d_argmax, d_margin, d_logits, s)
             : run_denoise<float>(st, d_canvas, step, params, h_seeds, d_active, d_H, d_y, d_argmax, d_margin, d_logits,
                                  s);
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
                       st->n, st->m->cfg.vocab, step, params->max_steps, params->entropy_bound, params->stop_mode,
                       params->stop_tau, st->canvas_index, reinterpret_cast<hipStream_t>(stream)));
  return DG_OK;
}

extern "C" dg_status dg_commit_canvas_to_kv(dg_state* st, const int32_t* d_canvas, dg_stream stream) {
  if (!st || !d_canvas) return fail(DG_ERR_ARG, "null argument");
  if (st->ctx + st->n > st->max_ctx)
    return fail(DG_ERR_CAPACITY, "context %d + canvas %d exceeds max_ctx %d", st->ctx, st->n, st->max_ctx);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  dg_status r = st->m->cfg.dtype == DG_DTYPE_BF16 ? run_stack<bf16>(st, d_canvas, st->n, true, false, s)
                                                  : run_stack<float>(st, d_canvas, st->n, true, false, s);
  if (r) return r;
  st->ctx += st->n;
  st->canvas_index += 1;
  return DG_OK;
}

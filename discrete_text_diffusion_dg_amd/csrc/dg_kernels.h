// Host-side launchers of the gfx950 kernels (internal to the library).
// Each returns the launch status (hipGetLastError after the launch).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "dg_common.h"

namespace dg {

// Per-request Philox seeds travel by value in the kernel arguments, so a step
// needs no host-to-device copy.
constexpr int kMaxBatch = 128;
struct SeedArg {
  uint64_t v[kMaxBatch];
};

// Requests taking part in a pass.  Request b computes iff active(b): every
// kernel of the pass skips the rows, tiles and blocks of the others, whose
// outputs and state are left as they were.  p == nullptr: every request.
struct Gate {
  const uint8_t* p;
  int invert;          // 0: p[b] != 0 marks an active request; 1: p[b] != 0 marks a finished one
  __device__ __forceinline__ bool active(int b) const { return p == nullptr || ((p[b] != 0) != (invert != 0)); }
  // any request among rows r0 .. r0 + rows - 1 (n rows per request) active
  __device__ __forceinline__ bool any_active(int r0, int rows, int n) const {
    if (p == nullptr) return true;
    for (int b = r0 / n; b <= (r0 + rows - 1) / n; ++b)
      if (active(b)) return true;
    return false;
  }
};

// Positions of a pass: request b's new rows sit at ctx[b] + off + i (ctx: the
// per-request context lengths held in the state).
struct PosArg {
  const int32_t* ctx;
  int off;
  __device__ __forceinline__ int base(int b) const { return ctx[b] + off; }
};

// Step of the canvas, its temperature and the canvas index of each request.
// The explicit step calls give the step and 1 / T by value; the device-driven
// canvas loop reads them from the state (the step counter and a per-step
// table of 1 / T computed on the host), so one captured step serves them all.
struct StepInfo {
  int step;
  float inv_t;
  const int32_t* pstep;     // non-null: the step counter of the loop
  const float* inv_tab;     // 1 / T of each step (loop mode)
  const int32_t* cidx;      // canvas index of each request
  __device__ __forceinline__ int get_step() const { return pstep != nullptr ? *pstep : step; }
  __device__ __forceinline__ float get_inv_t(int st) const { return pstep != nullptr ? inv_tab[st] : inv_t; }
};

// Statistics of one (row, 128-id vocabulary chunk), written by the LM-head
// epilogue (or by head_from_logits) and combined per row by sampler_merge.
struct HeadPart {       // statistics of one (row, vocab chunk)
  float m;              // max of z = logit / T
  float s;              // sum exp(z - m)
  float w;              // sum exp(z - m) * (z - m)
  float lmax;           // max logit
  int lidx;             // its index (lowest on ties)
  float g1;             // best Gumbel-perturbed score
  int gidx;             // its index
  float g2;             // second-best score
};

// Sampler inputs of the LM-head epilogue; ptilde (exp(z - chunk max), operand
// type) and logits (fp32) are written when non-null.
template <typename T>
struct HeadArgs {
  StepInfo si; SeedArg seeds; int n;
  HeadPart* part; T* ptilde; float* logits;
  Gate gate;
};

// One expert-routed tile: (expert, first gathered row, rows, unused).
// Capacity of the tile list for R rows routed to k experts each, tiles of at
// least 64 rows.
inline int expert_tile_capacity(int rows, int top_k, int n_experts) {
  return (rows * top_k + 63) / 64 + n_experts;
}

// ---- matrix products (k_gemm.hip); B operands are [N, K] K-contiguous
constexpr int kMaxSplits = 16;
constexpr int kMaxModel = 4096;           // largest d_model of the row-wise kernels
struct SplitPlan {
  int splits, kchunk;
};
SplitPlan plan_splits(int M, int N, int K, int bm, int bn, int elem_bytes, int target);
// part[s][r][c] = sum over k in split s of A[r][k] * B[c][k]   (fp32, [splits][M][N])
// Tiles whose rows (n per request) all belong to requests the gate leaves
// out are skipped.
template <typename T>
hipError_t gemm_partials(const T* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                         SplitPlan sp, Gate g, int n, hipStream_t s);
// same with an fp32 A rounded to the operand type on load
template <typename T>
hipError_t gemm_partials_f32a(const float* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                              SplitPlan sp, Gate g, int n, hipStream_t s);
// The tied LM head, logits[r][v] = A[r] . B[v], in 128 x 128 tiles whose epilogue
// writes the head statistics of each (row, 128-id chunk) -- part[r][v / 128] --
// and, as asked, exp(z - chunk max) and the logits.  V must be a multiple of 64.
template <typename T>
hipError_t gemm_lm_head(const T* A, int lda, const T* B, int ldb, int M, int V, int K, const HeadArgs<T>& h,
                        hipStream_t s);
// The same over FP8 (E4M3) rows: B8 holds the codes of B [V, K] in the P8
// fragment order (pack_head_fp8), bscale[v] the scale of row v; logits[r][v] =
// bscale[v] * (A[r] . codes of row v).  V and K multiples of 64.
hipError_t gemm_lm_head_fp8(const bf16* A, int lda, const fp8e4m3* B8, const float* bscale, int M, int V, int K,
                            const HeadArgs<bf16>& h, hipStream_t s);
// Quantise the rows of a bf16 [V, K] matrix to E4M3 with one fp32 scale per
// row (scale = fl32(fl64(max |row|) / 448), 1 for a zero row; code =
// E4M3(fl32(w / scale)), nearest even, saturating) into the P8 order above.
hipError_t pack_head_fp8(const bf16* w, fp8e4m3* codes, float* scales, int V, int K, hipStream_t s);
// The fused QKV projection of rows r = b * n + i with RoPE at position
// pos.base(b) + i applied to q and k in its epilogue: q -> q [M][Hq * hd],
// k -> K cache rows, v -> V^T cache columns (the layouts rope_scatter writes).
// One head per tile; requests the gate leaves out write nothing.
bool qkv_rope_ok(int d, int hd, int elem_bytes);
template <typename T>
hipError_t gemm_qkv_rope(const T* xn, const T* wqkv, int M, int d, int hd, const float2* rope, T* q, T* kc, T* vc,
                         int n, int Hq, int Hkv, int stride, PosArg pos, Gate g, hipStream_t s);
// Rows per tile of the expert-grouped products (the router writes its tile
// list with this many rows per tile for them): 128 on the bf16 LDS-DMA tile
// loop, else 64.
int expert_group_tile_rows(int d, int F, size_t elem_bytes);
// act[g][f] = silu(x[perm[g]] . gate_e[f]) * (x[perm[g]] . up_e[f]), rounded to T.
// pgu (optional): the fragment-packed gate/up weights (pack_expert_weights),
// read instead of gate / up by the bf16 DMA tile loop.
template <typename T>
hipError_t gemm_expert_gateup(const T* X, const int* perm, const T* gate, const T* up, T* act,
                              const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F,
                              hipStream_t s, const T* pgu = nullptr);
// Y[g][c] = act[g] . down_e[c]; pd (optional): the packed down weights
template <typename T>
hipError_t gemm_expert_down(const T* act, const T* down, T* Y, const int4* tiles,
                            const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s, const T* pd = nullptr);
// Weight-streaming expert products for thin routed tiles (k_expert.hip) over
// fragment-packed weights: PGU[e][F/16][d/32][2][64][8] (gate/up) and
// PD[e][d/16][F/32][64][8] (down), built by pack_expert_weights.
bool expert_stream_ok(int d, int F, int elem_bytes);
template <typename T>
hipError_t pack_expert_weights(const T* gate, const T* up, const T* down, T* pgu, T* pd, int E, int d, int F,
                               hipStream_t s);
// FP8 (OCP E4M3) experts: per output channel scales sgu [E][2][F] (gate, up)
// and sd [E][d], fl32(fl64(max |w|) / 448); codes E4M3(w / scale) packed as
// P8GU[E][F/16][d/64][2][64][16 B] and P8D[E][d/16][F/64][64][16 B] (two
// 32-wide K steps per lane piece).  WT = fp8e4m3 selects them in the streaming
// products (the scales multiply the sums); WT = T the plain packed weights
// (scale unused).
bool expert_stream_fp8_ok(int d, int F);
hipError_t pack_expert_weights_fp8(const bf16* gate, const bf16* up, const bf16* down, fp8e4m3* pgu, fp8e4m3* pd,
                                   float* sgu, float* sd, int E, int d, int F, hipStream_t s);
template <typename T, typename WT>
hipError_t expert_stream_gateup(const T* X, const int* perm, const WT* pgu, const float* scale, T* act,
                                const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s);
template <typename T, typename WT>
hipError_t expert_stream_down(const T* act, const WT* pd, const float* scale, T* Y, const int4* tiles,
                              const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s);
// part[split][r][c] = sum over k in [split*kchunk, (split+1)*kchunk) of
// rnd(P[r][k] * scale[r][k / 128]) * Bt[c][k]   (P: [M][K], scale: [M][nchunk], Bt: [N][K])
template <typename T>
hipError_t gemm_selfcond(const T* P, const float* scale, int nchunk, const T* Bt, float* part, int M, int N, int K,
                         int splits, int kchunk, Gate g, int n, hipStream_t s);

// ---- attention (k_attn.hip)
struct AttnArgs {
  const void* q;        // [B*nq, Hq*hd] operand type, RoPE applied
  const void* kc;       // K cache of this layer: [B][Hkv][kv_stride][hd]
  const void* vc;       // V cache of this layer, transposed: [B][Hkv][hd][kv_stride]
  void* out;            // [B*nq, Hq*hd] operand type
  void* part_o;         // split partials [splits][B*nq*Hq][hd] (operand type, unnormalised)
  float* part_ml;       // split partials [splits][B*nq*Hq][2] (running max, sum)
  int B, nq, Hq, Hkv, hd, kv_stride;   // kv_stride: context capacity rounded up to 64
  PosArg pos;           // request b: keys 0..pos.base(b)+nq-1 (the new rows sit at pos.base(b)..+nq-1)
  int keys_max;         // largest key count over the requests (launch shape only)
  Gate gate;            // requests left out compute and write nothing
  int causal;
  int splits;
  float scale;
};
template <typename T>
hipError_t attention(const AttnArgs& a, hipStream_t s);
int attention_splits(int B, int nq, int Hq, int Hkv, int hd, int keys, int elem_bytes);
// Which attention kernel a launch takes for this many keys (0 spread, 1 wide).
int attention_launch_class(int B, int nq, int Hq, int Hkv, int hd, int keys);

// ---- row-wise kernels (k_misc.hip); S = number of split partials to reduce
// Row kernels: one workgroup per row; rows of requests the gate leaves out
// (n rows per request) return at once.
template <typename T>
hipError_t embed_norm(const T* emb, const int32_t* tok, const float* part, int S, int M, int d, int vocab,
                      const float* g, float eps, float* H, T* xn, Gate gt, int n, hipStream_t s);
template <typename T>
hipError_t add_norm(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                    Gate gt, int n, hipStream_t s);
template <typename T>
hipError_t combine_norm(const T* Y, const int* pos, const float* w, int k, int M, int d, const float* g,
                        float eps, float* H, T* xn, Gate gt, int n, hipStream_t s);
// RoPE on q and k of the fused projection (sum of S partials), q -> Q buffer, k and v -> cache at
// pos.base(b) + i (K rows [B][Hkv][stride][hd], V transposed [B][Hkv][hd][stride])
template <typename T>
hipError_t rope_scatter(const float* part, int S, const float2* rope, T* q, T* kc, T* vc, int B, int n, int Hq,
                        int Hkv, int hd, int stride, PosArg pos, Gate gt, hipStream_t s);
hipError_t rope_table(float2* tab, int max_ctx, int hd, float theta, hipStream_t s);
// Router of one layer: logits, top-k + softmax weights, and the expert-sorted
// order (perm, pos, 64-row tiles).  cnt: scratch of E * ceil(M / router_rows_per_block(E)) ints;
// part: scratch of router_ksplits(M, d, E) * M * E floats (K-split partial logits).
// Requires d % (32 * kRouterWaves) == 0, E <= 128, k <= 8.
constexpr int kRouterWaves = 4, kRouterMaxSplits = 8;
int router_rows_per_block(int E);
int router_ksplits(int M, int d, int E);
// Rows of requests the gate leaves out get expert id -1 in every slot and take
// no place in the expert-sorted order (their pos entries are not written).
template <typename T>
hipError_t router(const T* xn, const T* wr, int M, int d, int E, int k, float* rlog, int* idx, float* w, int* perm,
                  int* pos, int4* tiles, int* n_tiles, int tile_rows, int* cnt, float* part, Gate gt, int n,
                  hipStream_t s);
// Few routed entries (M * k <= 4096, E a power of two <= 128): add_norm plus
// the router logits, top-k and softmax of each row (rlog, idx, w), then the
// expert-sorted order (perm, pos, tiles) in one workgroup.
bool router_fused_ok(int M, int d, int E, int k);
template <typename T>
hipError_t add_norm_router(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                           const T* wr, int E, int k, float* rlog, int* idx, float* w, Gate gt, int n,
                           hipStream_t s);
hipError_t route_sort(const int* idx, int M, int k, int E, int tile_rows, int* perm, int* pos, int4* tiles,
                      int* n_tiles, hipStream_t s);
template <typename T>
hipError_t transpose(const T* src, T* dst, int rows, int cols, hipStream_t s);
// canvas_len uniform tokens per request b, Philox canvas index cidx[b]
hipError_t init_canvas(int32_t* canvas, const SeedArg& seeds, int B, int n, int vocab, const int32_t* cidx,
                       hipStream_t s);
// Per-request context bookkeeping: ctx[b] += add and cidx[b] += add_canvas for
// the requests the gate selects.
hipError_t advance_context(int32_t* ctx, int32_t* cidx, int B, int add, int add_canvas, Gate g, hipStream_t s);
// Fills of a device buffer (kernels, so that captured graphs hold no memset nodes).
hipError_t fill_u32(void* p, uint32_t v, size_t count, hipStream_t s);
hipError_t fill_u8(void* p, uint8_t v, size_t count, hipStream_t s);
// End of a step of the device-driven loop.  step[0] (the canvas step)
// advances, step[1] = every request done, step[2] counts the loop steps
// completed; progress (mapped host memory, may be null) receives
// (step[2], step[1]).
hipError_t step_end(const uint8_t* done, int B, int32_t* step, volatile int32_t* progress, hipStream_t s);

// ---- top-k truncated sampler ([mlqm] 九: top-k truncation of the vocabulary)
// A vocabulary segment's top kTopkList logits of one row, descending (ties:
// lower id first); written per (row, segment) by the LM head's top-k variant
// (or from supplied logits) and combined per row by topk_merge.
constexpr int kTopkList = 8;
struct TopkPart {
  float v[kTopkList];
  int id[kTopkList];
};
// Segments of the vocabulary for M rows (one workgroup per 128-row block and
// segment, about 256 workgroups).
int topk_segments(int M, int vocab);
// logits = A . B^T tile by tile over each (row block, segment); per row and
// segment its top kTopkList logits.  Rows of requests the gate leaves out are
// skipped (whole row blocks).
// (gemm_lm_head_topk_fp8: the same over the E4M3 rows and per-id scales of an FP8 head)
hipError_t gemm_lm_head_topk_fp8(const bf16* A, int lda, const fp8e4m3* B8, const float* bscale, int M, int V, int K,
                                 int nseg, TopkPart* out, Gate g, int n, hipStream_t s);
template <typename T>
hipError_t gemm_lm_head_topk(const T* A, int lda, const T* B, int ldb, int M, int V, int K, int nseg, TopkPart* out,
                             Gate g, int n, hipStream_t s);
// the same records from supplied fp32 logits [M][V]
hipError_t topk_from_logits(const float* logits, int M, int V, int nseg, TopkPart* out, Gate g, int n, hipStream_t s);
// Per row: the top_k (1..kTopkList) largest logits of all segments; the
// truncated tempered distribution's entropy, its Gumbel-max sample and top-2
// margin, the logit argmax, and (emb non-null) the self-conditioning vector
// s = sum p_v E_v over the k ids.
template <typename T>
hipError_t topk_merge(const TopkPart* part, int M, int nseg, int top_k, const StepInfo& si, const SeedArg& seeds, int n,
                      Gate g, float* H, int32_t* y, int32_t* am, float* margin, const T* emb, int d, float* s_out,
                      hipStream_t s);

// ---- sampler (k_sampler.hip)
// Fixed device scratch of the allocation-free sampler entry point
// (dg_sample_logits_static): its device address on the current device, looked
// up on the first call there.  Layout: kMaxBatch canvas indices (int32), then
// from kStaticHeadOffset the per-(row, chunk) head statistics.
constexpr size_t kStaticScratchBytes = (size_t)16 << 20;
constexpr size_t kStaticHeadOffset = 4096;
constexpr int kMaxDevices = 64;
hipError_t static_scratch(void** ptr);
int head_chunks(int vocab);     // 128-id chunks of the vocabulary
// head statistics of supplied fp32 logits [M][V] (V a multiple of 64)
template <typename T>
hipError_t head_from_logits(const float* logits, int M, int V, const StepInfo& si, const SeedArg& seeds, int n,
                            HeadPart* part, T* ptilde, Gate g, hipStream_t s);
// H, y, am, margin may be null (not written); lse (may be null) receives each
// row's log sum exp(z).
hipError_t sampler_merge(const HeadPart* part, int M, int chunks, int n, Gate g,
                         float* H, int32_t* y, int32_t* am, float* margin, float* chunk_scale,
                         hipStream_t s, float* lse = nullptr);
// Training-side forward pass: corruption of clean canvases (per-request
// rates), then the cross-entropy of the clean tokens (ce [B*n]) and its mean
// per request (loss [B]) from the final normed rows, the embedding and the
// rows' log-sum-exp.
struct RateArg {
  float v[kMaxBatch];
};
hipError_t corrupt_canvas(const int32_t* clean, int32_t* out, const SeedArg& seeds, const RateArg& rates, int B,
                          int n, int vocab, const int32_t* cidx, hipStream_t s);
template <typename T>
hipError_t clean_token_loss(const T* xn, const T* emb, const int32_t* clean, const float* lse, int B, int n, int d,
                            int vocab, float* ce, float* loss, hipStream_t s);
// The same with the clean token's logit from an FP8 head (E4M3 codes in the P8
// order of gemm_lm_head_fp8 and per-id scales).
hipError_t clean_token_loss_fp8(const bf16* xn, const fp8e4m3* codes, const float* scale, const int32_t* clean,
                                const float* lse, int B, int n, int d, int vocab, float* ce, float* loss,
                                hipStream_t s);
// S[r][c] = sum over splits (in order) of part[split][r][c], rows of active requests
hipError_t selfcond_reduce(const float* part, int M, int d, int splits, float* S, Gate g, int n, hipStream_t s);
hipError_t commit_kernel(const float* H, const int32_t* y, const int32_t* am, int32_t* canvas,
                         int32_t* prev_am, uint8_t* mask, int32_t* n_committed, uint8_t* done,
                         const SeedArg& seeds, int B, int n, int vocab, const StepInfo& si, int max_steps,
                         float bound, int stop_mode, float tau, hipStream_t s);

}  // namespace dg

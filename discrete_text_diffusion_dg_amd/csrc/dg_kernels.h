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
  float inv_t; SeedArg seeds; int n, canvas_index, step;
  HeadPart* part; T* ptilde; float* logits;
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
template <typename T>
hipError_t gemm_partials(const T* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                         SplitPlan sp, hipStream_t s);
// same with an fp32 A rounded to the operand type on load
template <typename T>
hipError_t gemm_partials_f32a(const float* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                              SplitPlan sp, hipStream_t s);
// The tied LM head, logits[r][v] = A[r] . B[v], in 128 x 128 tiles whose epilogue
// writes the head statistics of each (row, 128-id chunk) -- part[r][v / 128] --
// and, as asked, exp(z - chunk max) and the logits.  V must be a multiple of 64.
template <typename T>
hipError_t gemm_lm_head(const T* A, int lda, const T* B, int ldb, int M, int V, int K, const HeadArgs<T>& h,
                        hipStream_t s);
// The fused QKV projection of rows r = b * n + i with RoPE at position ctx + i
// applied to q and k in its epilogue: q -> q [M][Hq * hd], k -> K cache rows,
// v -> V^T cache columns (the layouts rope_scatter writes).  One head per tile.
bool qkv_rope_ok(int d, int hd, int elem_bytes);
template <typename T>
hipError_t gemm_qkv_rope(const T* xn, const T* wqkv, int M, int d, int hd, const float2* rope, T* q, T* kc, T* vc,
                         int n, int Hq, int Hkv, int stride, int ctx, hipStream_t s);
// Rows per tile of the expert-grouped products (the router writes its tile
// list with this many rows per tile for them): 128 on the bf16 LDS-DMA tile
// loop, else 64.
int expert_group_tile_rows(int d, int F, size_t elem_bytes);
// act[g][f] = silu(x[perm[g]] . gate_e[f]) * (x[perm[g]] . up_e[f]), rounded to T
template <typename T>
hipError_t gemm_expert_gateup(const T* X, const int* perm, const T* gate, const T* up, T* act,
                              const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F,
                              hipStream_t s);
// Y[g][c] = act[g] . down_e[c]
template <typename T>
hipError_t gemm_expert_down(const T* act, const T* down, float* Y, const int4* tiles,
                            const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s);
// Weight-streaming expert products for thin routed tiles (k_expert.hip) over
// fragment-packed weights: PGU[e][F/16][d/32][2][64][8] (gate/up) and
// PD[e][d/16][F/32][64][8] (down), built by pack_expert_weights.
bool expert_stream_ok(int d, int F, int elem_bytes);
template <typename T>
hipError_t pack_expert_weights(const T* gate, const T* up, const T* down, T* pgu, T* pd, int E, int d, int F,
                               hipStream_t s);
template <typename T>
hipError_t expert_stream_gateup(const T* X, const int* perm, const T* pgu, T* act, const int4* tiles,
                                const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s);
template <typename T>
hipError_t expert_stream_down(const T* act, const T* pd, float* Y, const int4* tiles, const int* n_tiles,
                              int cap_tiles, int d, int F, hipStream_t s);
// part[split][r][c] = sum over k in [split*kchunk, (split+1)*kchunk) of
// rnd(P[r][k] * scale[r][k / 128]) * Bt[c][k]   (P: [M][K], scale: [M][nchunk], Bt: [N][K])
template <typename T>
hipError_t gemm_selfcond(const T* P, const float* scale, int nchunk, const T* Bt, float* part, int M, int N, int K,
                         int splits, int kchunk, hipStream_t s);

// ---- attention (k_attn.hip)
struct AttnArgs {
  const void* q;        // [B*nq, Hq*hd] operand type, RoPE applied
  const void* kc;       // K cache of this layer: [B][Hkv][kv_stride][hd]
  const void* vc;       // V cache of this layer, transposed: [B][Hkv][hd][kv_stride]
  void* out;            // [B*nq, Hq*hd] operand type
  float* part_o;        // split partials [splits][B*nq*Hq][hd] (fp32, unnormalised)
  float* part_ml;       // split partials [splits][B*nq*Hq][2] (running max, sum)
  int B, nq, Hq, Hkv, hd, kv_stride;   // kv_stride: context capacity rounded up to 64
  int ctx;              // keys 0..ctx+nq-1 (the new rows sit at ctx..ctx+nq-1)
  int causal;
  int splits;
  float scale;
};
template <typename T>
hipError_t attention(const AttnArgs& a, hipStream_t s);
int attention_splits(int B, int nq, int Hq, int Hkv, int hd, int keys, int elem_bytes);

// ---- row-wise kernels (k_misc.hip); S = number of split partials to reduce
template <typename T>
hipError_t embed_norm(const T* emb, const int32_t* tok, const float* part, int S, int M, int d, int vocab,
                      const float* g, float eps, float* H, T* xn, hipStream_t s);
template <typename T>
hipError_t add_norm(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                    hipStream_t s);
template <typename T>
hipError_t combine_norm(const float* Y, const int* pos, const float* w, int k, int M, int d, const float* g,
                        float eps, float* H, T* xn, hipStream_t s);
// RoPE on q and k of the fused projection (sum of S partials), q -> Q buffer, k and v -> cache at ctx + i
// (K rows [B][Hkv][stride][hd], V transposed [B][Hkv][hd][stride])
template <typename T>
hipError_t rope_scatter(const float* part, int S, const float2* rope, T* q, T* kc, T* vc, int B, int n, int Hq,
                        int Hkv, int hd, int stride, int ctx, hipStream_t s);
hipError_t rope_table(float2* tab, int max_ctx, int hd, float theta, hipStream_t s);
// Router of one layer: logits, top-k + softmax weights, and the expert-sorted
// order (perm, pos, 64-row tiles).  cnt: scratch of E * ceil(M / router_rows_per_block(E)) ints;
// part: scratch of router_ksplits(M, d, E) * M * E floats (K-split partial logits).
// Requires d % (32 * kRouterWaves) == 0, E <= 128, k <= 8.
constexpr int kRouterWaves = 4, kRouterMaxSplits = 8;
int router_rows_per_block(int E);
int router_ksplits(int M, int d, int E);
template <typename T>
hipError_t router(const T* xn, const T* wr, int M, int d, int E, int k, float* rlog, int* idx, float* w, int* perm,
                  int* pos, int4* tiles, int* n_tiles, int tile_rows, int* cnt, float* part, hipStream_t s);
// Few routed entries (M * k <= 4096, E a power of two <= 128): add_norm plus
// the router logits, top-k and softmax of each row (rlog, idx, w), then the
// expert-sorted order (perm, pos, tiles) in one workgroup.
bool router_fused_ok(int M, int d, int E, int k);
template <typename T>
hipError_t add_norm_router(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                           const T* wr, int E, int k, float* rlog, int* idx, float* w, hipStream_t s);
hipError_t route_sort(const int* idx, int M, int k, int E, int tile_rows, int* perm, int* pos, int4* tiles,
                      int* n_tiles, hipStream_t s);
template <typename T>
hipError_t transpose(const T* src, T* dst, int rows, int cols, hipStream_t s);
hipError_t init_canvas(int32_t* canvas, const SeedArg& seeds, int B, int n, int vocab, int canvas_index,
                       hipStream_t s);

// ---- sampler (k_sampler.hip)
int head_chunks(int vocab);     // 128-id chunks of the vocabulary
// head statistics of supplied fp32 logits [M][V] (V a multiple of 64)
template <typename T>
hipError_t head_from_logits(const float* logits, int M, int V, float inv_t, const SeedArg& seeds, int n,
                            int canvas_index, int step, HeadPart* part, T* ptilde, hipStream_t s);
hipError_t sampler_merge(const HeadPart* part, int M, int chunks, int n, const uint8_t* active,
                         float* H, int32_t* y, int32_t* am, float* margin, float* chunk_scale,
                         hipStream_t s);
// S[r][c] = sum over splits (in order) of part[split][r][c]
hipError_t selfcond_reduce(const float* part, int M, int d, int splits, float* S, hipStream_t s);
hipError_t commit_kernel(const float* H, const int32_t* y, const int32_t* am, int32_t* canvas,
                         int32_t* prev_am, uint8_t* mask, int32_t* n_committed, uint8_t* done,
                         const SeedArg& seeds, int B, int n, int vocab, int step, int max_steps,
                         float bound, int stop_mode, float tau, int canvas_index, hipStream_t s);

}  // namespace dg

// Matrix products of the denoise step on the MFMA tile engine:
// fused QKV / O-projection / router / LM head (dense), the self-conditioning
// input projection fused with the embedding gather, the expert SwiGLU pair and
// down projection (grouped by expert), and the split-K contraction of the
// sampled distribution with the embedding (self-conditioning vector).
#include "dg_kernels.h"
#include "gemm_engine.h"

namespace dg {

// ------------------------------------------------------------------ epilogues
struct EpStoreF32 {        // C[row_base + r][n0 + c] = v
  float* out; int ldo;
  __device__ void operator()(const TileCtx& t, const f32x4_t (&acc)[2][2], char*) const {
    for_each_acc(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) out[(size_t)(t.row_base + r) * ldo + t.n0 + c] = v;
    });
  }
};

struct EpResidAdd {        // H[r][c] += v   (residual stream, fp32)
  float* h; int ldh;
  __device__ void operator()(const TileCtx& t, const f32x4_t (&acc)[2][2], char*) const {
    for_each_acc(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) {
        float* p = h + (size_t)(t.m0 + r) * ldh + t.n0 + c;
        *p = *p + v;
      }
    });
  }
};

template <typename T>
struct EpEmbedAdd {        // H[r][c] = emb[tok[r]][c] + v  (ids clamped to [0, vocab))
  const T* emb; const int32_t* tok; float* h; int d; int vocab;
  __device__ void operator()(const TileCtx& t, const f32x4_t (&acc)[2][2], char*) const {
    for_each_acc(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) {
        const int row = t.m0 + r, col = t.n0 + c;
        const int id = min(max(tok[row], 0), vocab - 1);
        h[(size_t)row * d + col] = Num<T>::load(emb + (size_t)id * d + col) + v;
      }
    });
  }
};

template <typename T>
struct EpSwiGLU {          // waves with wn = 1 hold the up projection; exchange through LDS
  T* act; int F;
  __device__ void operator()(const TileCtx& t, const f32x4_t (&acc)[2][2], char* smem) const {
    float* x = reinterpret_cast<float*>(smem);   // [64][33]
    const int wn = (threadIdx.x >> 6) & 1;
    if (wn == 1) for_each_acc(acc, [&](int r, int c, float v) { x[r * 33 + (c - 32)] = v; });
    __syncthreads();
    if (wn == 0)
      for_each_acc(acc, [&](int r, int c, float g) {
        if (r < t.rows && c < t.cols) {
          const float u = x[r * 33 + c];
          const float a = g / (1.0f + expf(-g)) * u;
          Num<T>::store(act + (size_t)(t.row_base + r) * F + t.n0 + c, a);
        }
      });
  }
};

struct EpSplitK {          // part[split][row][col] = v
  float* part; int ldo; size_t split_stride;
  __device__ void operator()(const TileCtx& t, const f32x4_t (&acc)[2][2], char*) const {
    float* base = part + (size_t)t.group * split_stride;
    for_each_acc(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) base[(size_t)(t.m0 + r) * ldo + t.n0 + c] = v;
    });
  }
};

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

template <typename T, class SCHED, class AL, class BL, class EP>
static hipError_t launch(int grid, const SCHED& sc, const AL& al, const BL& bl, const EP& ep,
                         hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<T, SCHED, AL, BL, EP>), dim3(grid), dim3(256), 0, s, sc, al, bl, ep);
  return hipGetLastError();
}

template <typename T>
hipError_t gemm_store_f32(const T* A, int lda, const T* B, int ldb, float* C, int ldc, int M, int N,
                          int K, hipStream_t s) {
  SchedDense sc{M, N, K, cdiv(M, 64), cdiv(N, 64)};
  return launch<T>(sc.mt * sc.nt, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb}, EpStoreF32{C, ldc}, s);
}

template <typename T>
hipError_t gemm_resid_add(const T* A, int lda, const T* B, int ldb, float* H, int ldh, int M, int N,
                          int K, hipStream_t s) {
  SchedDense sc{M, N, K, cdiv(M, 64), cdiv(N, 64)};
  return launch<T>(sc.mt * sc.nt, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb}, EpResidAdd{H, ldh}, s);
}

template <typename T>
hipError_t gemm_embed_selfcond(const float* S, const T* W, const T* emb, const int32_t* tok,
                               float* H, int M, int d, int vocab, hipStream_t s) {
  SchedDense sc{M, d, d, cdiv(M, 64), cdiv(d, 64)};
  return launch<T>(sc.mt * sc.nt, sc, ALF32<T>{S, d}, BLPlain<T>{W, d},
                   EpEmbedAdd<T>{emb, tok, H, d, vocab}, s);
}

template <typename T>
hipError_t gemm_expert_gateup(const T* X, const int* perm, const T* gate, const T* up, T* act,
                              const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F,
                              hipStream_t s) {
  SchedGroup sc{tiles, n_tiles, cdiv(F, 32), F, d, 32};
  return launch<T>(cap_tiles * sc.nt, sc, ALGather<T>{X, d, perm},
                   BLGateUp<T>{gate, up, (size_t)F * d, d}, EpSwiGLU<T>{act, F}, s);
}

template <typename T>
hipError_t gemm_expert_down(const T* act, const T* down, float* Y, const int4* tiles,
                            const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s) {
  SchedGroup sc{tiles, n_tiles, cdiv(d, 64), d, F, 64};
  return launch<T>(cap_tiles * sc.nt, sc, ALRows<T>{act, F}, BLExpert<T>{down, (size_t)d * F, F},
                   EpStoreF32{Y, d}, s);
}

template <typename T>
hipError_t gemm_splitk(const T* P, int ldp, const T* Bt, int ldb, float* part, int M, int N, int K,
                       int splits, int kchunk, hipStream_t s) {
  SchedSplitK sc{M, N, K, cdiv(M, 64), cdiv(N, 64), splits, kchunk};
  return launch<T>(sc.mt * sc.nt * splits, sc, ALPlain<T>{P, ldp}, BLPlain<T>{Bt, ldb},
                   EpSplitK{part, N, (size_t)M * N}, s);
}

#define DG_INST(T)                                                                                 \
  template hipError_t gemm_store_f32<T>(const T*, int, const T*, int, float*, int, int, int, int,  \
                                        hipStream_t);                                             \
  template hipError_t gemm_resid_add<T>(const T*, int, const T*, int, float*, int, int, int, int,  \
                                        hipStream_t);                                             \
  template hipError_t gemm_embed_selfcond<T>(const float*, const T*, const T*, const int32_t*,     \
                                             float*, int, int, int, hipStream_t);                 \
  template hipError_t gemm_expert_gateup<T>(const T*, const int*, const T*, const T*, T*,          \
                                            const int4*, const int*, int, int, int, hipStream_t);  \
  template hipError_t gemm_expert_down<T>(const T*, const T*, float*, const int4*, const int*, int, \
                                          int, int, hipStream_t);                                 \
  template hipError_t gemm_splitk<T>(const T*, int, const T*, int, float*, int, int, int, int, int, \
                                     hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

// Matrix products of the denoise step on the MFMA tile engine:
// the fused QKV / output / self-conditioning projections (dense, split along
// K; the fp32 partials are reduced in a fixed order by the row-wise kernel
// that consumes them), the tied LM head with the head statistics in its
// epilogue, the expert SwiGLU pair and down projection (grouped by expert),
// and the split-K contraction of the sampled distribution with the embedding
// (self-conditioning vector).
#include "dg_head.h"
#include "gemm_engine.h"

namespace dg {

// ------------------------------------------------------------------ epilogues
struct EpStoreF32 {        // out[group * split_stride + (row_base + r) * ldo + n0 + c] = v
  static constexpr int kSmemBytes = 0;
  float* out; int ldo; size_t split_stride;
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc)[C::FM][C::FN], char*) const {
    float* base = out + (size_t)t.group * split_stride;
    for_each_acc<C>(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) base[(size_t)(t.row_base + r) * ldo + t.n0 + c] = v;
    });
  }
};

template <typename T>
struct EpStore {           // out[(row_base + r) * ldo + n0 + c] = v in the operand type
  static constexpr int kSmemBytes = 0;
  T* out; int ldo;
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc)[C::FM][C::FN], char*) const {
    for_each_acc<C>(acc, [&](int r, int c, float v) {
      if (r < t.rows && c < t.cols) Num<T>::store(out + (size_t)(t.row_base + r) * ldo + t.n0 + c, v);
    });
  }
};

template <typename T>
struct EpSwiGLU {          // blocks 2j / 2j+1 of a wave hold gate / up of the same 16 features
  static constexpr int kSmemBytes = 0;
  T* act; int F;
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc)[C::FM][C::FN], char*) const {
    static_assert(C::KG == 1, "one wave group");
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, wm = w >> 1, wn = w & 1;
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int j = 0; j < C::FN / 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = wm * C::WM + a * 16 + (lane >> 4) * 4 + i;
          const int f = (wn * C::WN / 32 + j) * 16 + (lane & 15);
          if (r < t.rows && f < t.cols) {
            const float g = acc[a][2 * j][i], u = acc[a][2 * j + 1][i];
            Num<T>::store(act + (size_t)(t.row_base + r) * F + t.n0 + f, swiglu(g, u));
          }
        }
  }
};

// LM-head tile -> head statistics of its 128 rows x 128 vocabulary ids (and,
// when asked for, the fp32 logits).  The accumulators go through the tile's
// shared memory, free once the K loop has ended.
// kScaled (FP8 head rows): logit = bscale[v] * (the product with the E4M3
// codes of row v), the scale applied in fp32 before anything reads the tile.
template <typename T, bool kScaled = false>
struct EpHead {
  static constexpr int kSmemBytes = kHeadTileBytes;
  StepInfo si; SeedArg seeds; int n, V, nchunk;
  HeadPart* part; T* ptilde; float* logits;
  Gate gate;      // a tile may hold rows of a request left out: their logits are not stored
  const float* bscale;   // kScaled: one fp32 scale per vocabulary id
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc_in)[C::FM][C::FN], char* smem) const {
    static_assert(C::BM == kHeadChunk && C::BN == kHeadChunk, "head tiles");
    static_assert(C::KG == 1, "the head statistics map 256 threads onto the tile");
    f32x4_t acc[C::FM][C::FN];
    {
      const int lane = threadIdx.x & 63, wn = (threadIdx.x >> 6) & 1;
#pragma unroll
      for (int b = 0; b < C::FN; ++b) {
        float sc = 1.f;
        if constexpr (kScaled) {
          const int c = wn * C::WN + b * 16 + (lane & 15);
          sc = bscale[t.n0 + (c < t.cols ? c : 0)];
        }
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][b][i] = kScaled ? acc_in[a][b][i] * sc : acc_in[a][b][i];
      }
    }
    float* tile = reinterpret_cast<float*>(smem);
    for_each_acc<C>(acc, [&](int r, int c, float v) { tile[r * kHeadLd + c] = v; });
    if (logits != nullptr)
      for_each_acc<C>(acc, [&](int r, int c, float v) {
        if (r < t.rows && c < t.cols && gate.active((t.m0 + r) / n)) logits[(size_t)(t.m0 + r) * V + t.n0 + c] = v;
      });
    __syncthreads();
    head_tile_stats<T>(tile, t.m0, t.rows, t.n0, t.cols, V, si, seeds, n, part, nchunk, ptilde);
  }
};

// Fused QKV projection tile -> RoPE and scatter: the tile covers BM rows x one
// head (BN == hd columns of the [q heads | k heads | v heads] projection).  q
// and k are rotated (rotate-half, table rope[pos][j] = (cos, sin)) and stored
// to the query buffer / the K cache row pos; v goes to the transposed V cache
// column pos.  Row r of the product is (request b = r / n, position
// pos.base(b) + r % n); rows of requests the gate leaves out are not stored.
template <typename T, int HD>
struct EpQKV {
  static constexpr int kLd = HD + 4;
  static constexpr int kSmemBytes = 128 * kLd * 4;         // at most 128 rows staged
  const float2* rope; T* q; T* kc; T* vc;
  int n, Hq, Hkv, stride;
  PosArg pa; Gate gate;
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc)[C::FM][C::FN], char* smem) const {
    static_assert(C::BN == HD && C::BM <= 128, "one head per tile");
    float* tile = reinterpret_cast<float*>(smem);
    for_each_acc<C>(acc, [&](int r, int c, float v) { tile[r * kLd + c] = v; });
    __syncthreads();
    constexpr int half = HD / 2;
    const int head = t.n0 / HD;
    // request and position of a row: shifts when the canvas length is a power
    // of two (the usual 256), else a division
    const bool pow2 = (n & (n - 1)) == 0;
    const int nsh = __ffs(n) - 1;
    auto split_row = [&](int row, int& b, int& pos) __attribute__((always_inline)) {
      if (pow2) { b = row >> nsh; pos = pa.base(b) + (row & (n - 1)); }
      else { b = row / n; pos = pa.base(b) + row % n; }
    };
    if (head < Hq + Hkv) {
      for (int u = threadIdx.x; u < C::BM * half; u += blockDim.x) {
        const int r = u / half, j = u % half;
        if (r >= t.rows) continue;
        const int row = t.m0 + r;
        int b, pos;
        split_row(row, b, pos);
        if (!gate.active(b)) continue;
        const float a = tile[r * kLd + j], bb = tile[r * kLd + j + half];
        const float2 cs = rope[(size_t)pos * half + j];
        const float o1 = a * cs.x - bb * cs.y, o2 = bb * cs.x + a * cs.y;
        T* dst = head < Hq ? q + (size_t)row * Hq * HD + head * HD
                           : kc + (((size_t)b * Hkv + (head - Hq)) * stride + pos) * HD;
        Num<T>::store(dst + j, o1);
        Num<T>::store(dst + j + half, o2);
      }
    } else {
      const int kh = head - Hq - Hkv;
      for (int u = threadIdx.x; u < C::BM * HD; u += blockDim.x) {
        const int c = u / C::BM, r = u % C::BM;           // consecutive threads: consecutive positions
        if (r >= t.rows) continue;
        const int row = t.m0 + r;
        int b, pos;
        split_row(row, b, pos);
        if (!gate.active(b)) continue;
        Num<T>::store(vc + (((size_t)b * Hkv + kh) * HD + c) * stride + pos, tile[r * kLd + c]);
      }
    }
  }
};

// Half-head QKV tiles (128-dim heads, few rows): a 64-column tile of head h
// holds features [j0, j0 + hd/4) and [hd/2 + j0, hd/2 + j0 + hd/4), j0 = 0 or
// hd/4, so both halves of every rotate-half pair meet in the tile.  The B
// loader fetches those weight rows; the epilogue is EpQKV's on half the
// columns.
template <int HD>
__device__ __forceinline__ int pair_feature(int n0, int c) {
  const int j0 = (n0 % HD) / 2;
  return c < HD / 4 ? j0 + c : HD / 2 + j0 + (c - HD / 4);
}
template <typename T, int HD>
struct BLHeadPairs {
  using Row = const void*;
  const T* p; int ldb;
  __device__ const void* row(const TileCtx& t, int n, bool& valid) const {
    valid = n < t.cols;
    const int head = t.n0 / HD;
    return p + (size_t)(head * HD + pair_feature<HD>(t.n0, valid ? n : 0)) * ldb;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};
template <typename T, int HD>
struct EpQKVPairs {
  static constexpr int BN = HD / 2, Q = HD / 4;
  static constexpr int kLd = BN + 4;
  static constexpr int kSmemBytes = 128 * kLd * 4;
  const float2* rope; T* q; T* kc; T* vc;
  int n, Hq, Hkv, stride;
  PosArg pa; Gate gate;
  template <class C>
  __device__ void apply(const TileCtx& t, const f32x4_t (&acc)[C::FM][C::FN], char* smem) const {
    static_assert(C::BN == BN && C::BM <= 128, "half a head per tile");
    float* tile = reinterpret_cast<float*>(smem);
    for_each_acc<C>(acc, [&](int r, int c, float v) { tile[r * kLd + c] = v; });
    __syncthreads();
    constexpr int half = HD / 2;
    const int head = t.n0 / HD, j0 = (t.n0 % HD) / 2;
    const bool pow2 = (n & (n - 1)) == 0;
    const int nsh = __ffs(n) - 1;
    auto split_row = [&](int row, int& b, int& pos) __attribute__((always_inline)) {
      if (pow2) { b = row >> nsh; pos = pa.base(b) + (row & (n - 1)); }
      else { b = row / n; pos = pa.base(b) + row % n; }
    };
    if (head < Hq + Hkv) {
      for (int u = threadIdx.x; u < C::BM * Q; u += blockDim.x) {
        const int r = u / Q, j = u % Q;
        if (r >= t.rows) continue;
        const int row = t.m0 + r;
        int b, pos;
        split_row(row, b, pos);
        if (!gate.active(b)) continue;
        const int f = j0 + j;
        const float a = tile[r * kLd + j], bb = tile[r * kLd + j + Q];
        const float2 cs = rope[(size_t)pos * half + f];
        const float o1 = a * cs.x - bb * cs.y, o2 = bb * cs.x + a * cs.y;
        T* dst = head < Hq ? q + (size_t)row * Hq * HD + head * HD
                           : kc + (((size_t)b * Hkv + (head - Hq)) * stride + pos) * HD;
        Num<T>::store(dst + f, o1);
        Num<T>::store(dst + f + half, o2);
      }
    } else {
      const int kh = head - Hq - Hkv;
      for (int u = threadIdx.x; u < C::BM * BN; u += blockDim.x) {
        const int c = u / C::BM, r = u % C::BM;
        if (r >= t.rows) continue;
        const int row = t.m0 + r;
        int b, pos;
        split_row(row, b, pos);
        if (!gate.active(b)) continue;
        Num<T>::store(vc + (((size_t)b * Hkv + kh) * HD + pair_feature<HD>(t.n0, c)) * stride + pos, tile[r * kLd + c]);
      }
    }
  }
};

// A rows of exp(z - m_c) (128-id chunks c) times the chunk's probability scale
// scale[row][c], in fp32, rounded to the operand type: the softmax @ E operand.
template <typename T>
struct ALScaled {
  const T* p; int lda; const float* scale; int nchunk;
  struct Row {
    const T* p; const float* sc;
  };
  __device__ Row row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    const size_t rr = (size_t)t.m0 + (valid ? r : 0);
    return Row{p + rr * lda, scale + rr * nchunk};
  }
  __device__ uint4 ld(const Row& rp, int k) const {
    const uint4 raw = *reinterpret_cast<const uint4*>(rp.p + k);
    const float sc = rp.sc[k / kHeadChunk];           // the 16 bytes lie in one chunk
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
      float v[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w[j] << 16) * sc;
        v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u) * sc;
      }
      return pack8_bf16(v);
    } else {
      return make_uint4(__float_as_uint(__uint_as_float(raw.x) * sc), __float_as_uint(__uint_as_float(raw.y) * sc),
                        __float_as_uint(__uint_as_float(raw.z) * sc), __float_as_uint(__uint_as_float(raw.w) * sc));
    }
  }
};

static inline int cdiv(int a, int b) { return (a + b - 1) / b; }

template <class C, typename T, class SCHED, class AL, class BL, class EP>
static hipError_t launch(int grid, const SCHED& sc, const AL& al, const BL& bl, const EP& ep, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm<C, T, SCHED, AL, BL, EP>), dim3(grid), dim3(256), 0, s, sc, al, bl, ep);
  return hipGetLastError();
}

template <class C, class SCHED, class AL, class BL, class EP>
static hipError_t launch_dma(int grid, const SCHED& sc, const AL& al, const BL& bl, const EP& ep, hipStream_t s) {
  if (grid <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gemm_dma<C, SCHED, AL, BL, EP>), dim3(grid), dim3(256 * C::KG), 0, s, sc, al, bl, ep);
  return hipGetLastError();
}

// Split count for a small-M product: enough workgroups to fill the chip, at
// least four 128-byte K slices per workgroup.
SplitPlan plan_splits(int M, int N, int K, int bm, int bn, int elem_bytes, int target) {
  const int bk = 128 / elem_bytes;
  const int tiles = cdiv(M, bm) * cdiv(N, bn);
  int s = cdiv(target, tiles);
  const int max_s = K / (4 * bk);
  if (s > max_s) s = max_s;
  if (s > kMaxSplits) s = kMaxSplits;
  if (s < 1) s = 1;
  const int kchunk = cdiv(cdiv(K, s), bk) * bk;
  s = cdiv(K, kchunk);
  return SplitPlan{s, kchunk};
}

// Split-K slices hold at least four 128-byte K steps; the prefetch depth of the
// small-M products (4 slices in registers) puts a whole slice's loads in flight
// at once instead of walking it in two round trips.
constexpr int kSplitStages = 5;
// rows from which an unsplit product takes 128 x 128 DMA tiles
constexpr int kDmaMinRows = 512;
// LDS ring depth of the expert-grouped 128 x 128 tiles
constexpr int kGroupStages = 2;

// exp(z - m_c) rows (row-locating) with the probability scale of each 128-id
// chunk: scale[row][c] multiplies the chunk's fp32 partial products.
template <typename T>
struct ALChunkScaled {
  static constexpr bool kChunkScale = true;
  using Row = const void*;
  const T* p; int lda; const float* scale; int nchunk;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)(t.m0 + (valid ? r : 0)) * lda;
  }
  __device__ const void* scale_ptr(const TileCtx& t, int r, int chunk, bool& valid) const {
    valid = r < t.rows;
    return scale + (size_t)(t.m0 + (valid ? r : 0)) * nchunk + chunk;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

template <typename T>
hipError_t gemm_partials(const T* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                         SplitPlan sp, Gate g, int n, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    // many rows, no split: 128 x 128 tiles through the DMA loop
    if (sp.splits == 1 && M >= kDmaMinRows && K % 64 == 0) {
      using C = TileCfgD<128, 128, 2>;
      SchedDense<128, 128> sc{M, N, K, cdiv(M, 128), cdiv(N, 128), 1, K, g, n};
      return launch_dma<C>(sc.mt * sc.nt, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb}, EpStoreF32{part, N, 0}, s);
    }
    // few rows, split along K: 64 x 64 tiles, two K groups of 4 waves per
    // workgroup (the split plan targets half as many workgroups as for the
    // register loop), each group's slices in flight at once
    if (sp.kchunk % 64 == 0 && K % 64 == 0) {
      using C = TileCfgD<64, 64, kSplitStages - 1, 2>;
      SchedDense<64, 64> sc{M, N, K, cdiv(M, 64), cdiv(N, 64), sp.splits, sp.kchunk, g, n};
      return launch_dma<C>(sc.mt * sc.nt * sp.splits, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb},
                           EpStoreF32{part, N, (size_t)M * N}, s);
    }
  }
  using C = TileCfg<T, 64, 64, kSplitStages>;
  SchedDense<64, 64> sc{M, N, K, cdiv(M, 64), cdiv(N, 64), sp.splits, sp.kchunk, g, n};
  return launch<C, T>(sc.mt * sc.nt * sp.splits, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb},
                      EpStoreF32{part, N, (size_t)M * N}, s);
}

template <typename T>
hipError_t gemm_partials_f32a(const float* A, int lda, const T* B, int ldb, float* part, int M, int N, int K,
                              SplitPlan sp, Gate g, int n, hipStream_t s) {
  using C = TileCfg<T, 64, 64, kSplitStages>;
  SchedDense<64, 64> sc{M, N, K, cdiv(M, 64), cdiv(N, 64), sp.splits, sp.kchunk, g, n};
  return launch<C, T>(sc.mt * sc.nt * sp.splits, sc, ALF32<T>{A, lda}, BLPlain<T>{B, ldb},
                      EpStoreF32{part, N, (size_t)M * N}, s);
}

// few rows: one workgroup per CU, two K groups of 4 waves each with its own
// slice ring (the 30-layer proxy's QKV, 256 x 4096 x 2048: 18.5 -> 13.8 us
// against one group of four slices; eight slices of one group measured no
// faster on the small shape: 8.55 against 8.45 us).  64-dim heads take
// 32-row tiles of a whole head; 128-dim heads take 64 x 64 half-head tiles
// with four slices per group: at 256 rows each workgroup reads (64 + 64)
// instead of (32 + 128) operand rows per slice, and the QKV stage of the
// proxy step went 19.7 -> 17.7 us per layer (two or three slices, or 32 x 64
// tiles at two workgroups per CU, were slower).
constexpr int kQkvGroups = 2;

template <typename T, int HD>
static hipError_t qkv_rope_hd(const T* xn, const T* wqkv, int M, int K, const float2* rope, T* q, T* kc, T* vc, int n,
                              int Hq, int Hkv, int stride, PosArg pa, Gate g, hipStream_t s) {
  const int N = (Hq + 2 * Hkv) * HD;
  const EpQKV<T, HD> ep{rope, q, kc, vc, n, Hq, Hkv, stride, pa, g};
  if constexpr (sizeof(T) == 2) {
    if (M <= 512) {
      if constexpr (HD == 128) {
        const EpQKVPairs<T, HD> eph{rope, q, kc, vc, n, Hq, Hkv, stride, pa, g};
        SchedDense<64, 64> sc{M, N, K, cdiv(M, 64), N / 64, 1, K, g, n};
        return launch_dma<TileCfgD<64, 64, 4, kQkvGroups>>(sc.mt * sc.nt, sc, ALPlain<T>{xn, K},
                                                           BLHeadPairs<T, HD>{wqkv, K}, eph, s);
      } else {
        SchedDense<32, HD> sc{M, N, K, cdiv(M, 32), N / HD, 1, K, g, n};
        return launch_dma<TileCfgD<32, HD, 4, kQkvGroups>>(sc.mt * sc.nt, sc, ALPlain<T>{xn, K},
                                                           BLPlain<T>{wqkv, K}, ep, s);
      }
    }
    SchedDense<128, HD> sc{M, N, K, cdiv(M, 128), N / HD, 1, K, g, n};
    return launch_dma<TileCfgD<128, HD, 2>>(sc.mt * sc.nt, sc, ALPlain<T>{xn, K}, BLPlain<T>{wqkv, K}, ep, s);
  } else {
    using C = TileCfg<T, 64, HD>;
    SchedDense<64, HD> sc{M, N, K, cdiv(M, 64), N / HD, 1, K, g, n};
    return launch<C, T>(sc.mt * sc.nt, sc, ALPlain<T>{xn, K}, BLPlain<T>{wqkv, K}, ep, s);
  }
}

bool qkv_rope_ok(int d, int hd, int elem_bytes) {
  if (elem_bytes == 2) return (hd == 64 || hd == 128) && d % 64 == 0;
  return hd == 64 && d % 32 == 0;
}

template <typename T>
hipError_t gemm_qkv_rope(const T* xn, const T* wqkv, int M, int d, int hd, const float2* rope, T* q, T* kc, T* vc,
                         int n, int Hq, int Hkv, int stride, PosArg pa, Gate g, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!qkv_rope_ok(d, hd, (int)sizeof(T))) return hipErrorInvalidValue;
  if (hd == 64) return qkv_rope_hd<T, 64>(xn, wqkv, M, d, rope, q, kc, vc, n, Hq, Hkv, stride, pa, g, s);
  if constexpr (sizeof(T) == 2) {
    return qkv_rope_hd<T, 128>(xn, wqkv, M, d, rope, q, kc, vc, n, Hq, Hkv, stride, pa, g, s);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t gemm_lm_head(const T* A, int lda, const T* B, int ldb, int M, int V, int K, const HeadArgs<T>& h,
                        hipStream_t s) {
  if (V % 64) return hipErrorInvalidValue;
  SchedDense<kHeadChunk, kHeadChunk> sc{M, V, K, cdiv(M, kHeadChunk), cdiv(V, kHeadChunk), 1, K, h.gate, h.n};
  EpHead<T> ep{h.si, h.seeds, h.n, V, cdiv(V, kHeadChunk), h.part, h.ptilde, h.logits, h.gate};
  if constexpr (sizeof(T) == 2) {
    if (K % 64 == 0)
      return launch_dma<TileCfgD<kHeadChunk, kHeadChunk, 2>>(sc.mt * sc.nt, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb},
                                                              ep, s);
  }
  using C = TileCfg<T, kHeadChunk, kHeadChunk>;
  return launch<C, T>(sc.mt * sc.nt, sc, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb}, ep, s);
}

// The LM head over FP8 (E4M3) rows of the embedding in the P8 fragment order,
// one fp32 scale per vocabulary id: the same 128 x 128 tiles and statistics
// epilogue, B slices at half the bytes.
hipError_t gemm_lm_head_fp8(const bf16* A, int lda, const fp8e4m3* B8, const float* bscale, int M, int V, int K,
                            const HeadArgs<bf16>& h, hipStream_t s) {
  if (V % 64 || K % 64) return hipErrorInvalidValue;
  SchedDense<kHeadChunk, kHeadChunk> sc{M, V, K, cdiv(M, kHeadChunk), cdiv(V, kHeadChunk), 1, K, h.gate, h.n};
  EpHead<bf16, true> ep{h.si, h.seeds, h.n, V, cdiv(V, kHeadChunk), h.part, h.ptilde, h.logits, h.gate, bscale};
  return launch_dma<TileCfgD<kHeadChunk, kHeadChunk, 2, 1, true>>(sc.mt * sc.nt, sc, ALPlain<bf16>{A, lda},
                                                                  BLPackedFp8Rows{B8, V, K}, ep, s);
}

// ------------------------------------------------------------------ top-k LM head
// Tied LM head for the top-k truncated sampler: a workgroup owns a 128-row
// block and a vocabulary segment and walks the segment's 128-id tiles in
// order.  Each tile's logits go through LDS as for the head statistics; lane
// (row, half) of the four waves keeps the 8 largest logits of its 64-id halves
// (a branch-free insertion, ids arriving in increasing order so an equal
// value never displaces the held one), and at the end the two halves of a row
// are merged and written: 64 bytes per (row, segment) instead of the logits or
// exp(z - m).
__device__ __forceinline__ void topk_insert(float (&tv)[kTopkList], int (&ti)[kTopkList], float v, int id, bool ties) {
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) {
    const bool c = v > tv[j] || (ties && v == tv[j] && id < ti[j]);
    const float nv = c ? v : tv[j];
    const int ni = c ? id : ti[j];
    v = c ? tv[j] : v;
    id = c ? ti[j] : id;
    tv[j] = nv;
    ti[j] = ni;
  }
}

// C: the tile configuration for the B loader (bf16 rows of E, or their E4M3
// codes); bscale (FP8 rows): each id's scale, applied as the tile is staged.
template <typename T, class C, class BL>
__global__ __launch_bounds__(256, 2) void k_lm_head_topk(ALPlain<T> al, BL bl, const float* bscale, int M, int V,
                                                         int K, int nseg, int cps, TopkPart* out, Gate gate, int n) {
  constexpr int kBytes = C::kSmemBytes > kHeadTileBytes ? C::kSmemBytes : kHeadTileBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kBytes];
  const int nmb = (M + kHeadChunk - 1) / kHeadChunk, nchunk = (V + kHeadChunk - 1) / kHeadChunk;
  const int total = nmb * nseg;
  if ((int)blockIdx.x >= total) return;
  // the row blocks of a segment are adjacent on one XCD: they share the segment's rows of E
  const int idx = xcd_run(blockIdx.x, total), mb = idx % nmb, sg = idx / nmb;
  const int m0 = mb * kHeadChunk, rows = min(kHeadChunk, M - m0);
  if (!gate.any_active(m0, rows, n)) return;
  const int c_begin = sg * cps, c_end = min(nchunk, c_begin + cps);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rl = w * 32 + (lane & 31), half = lane >> 5, c0 = half * 64;
  float tv[kTopkList];
  int ti[kTopkList];
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) { tv[j] = -INFINITY; ti[j] = 0x7fffffff; }
  float* tile = reinterpret_cast<float*>(smem);
  for (int c = c_begin; c < c_end; ++c) {
    TileCtx t;
    t.m0 = m0; t.n0 = c * kHeadChunk; t.rows = rows; t.cols = min(kHeadChunk, V - t.n0);
    t.k0 = 0; t.k1 = K; t.group = 0; t.row_base = m0;
    f32x4_t acc[C::FM][C::FN];
    tile_mma_dma<C>(t, al, bl, smem, acc);
    for_each_acc<C>(acc, [&](int r, int cc, float v) {
      if constexpr (C::B8) v *= bscale[t.n0 + (cc < t.cols ? cc : 0)];
      tile[r * kHeadLd + cc] = v;
    });
    __syncthreads();
    if (rl < rows && c0 < t.cols) {
      const float* tr = tile + rl * kHeadLd + c0;
#pragma unroll 4
      for (int q = 0; q < 16; ++q) {
        const float4 x = reinterpret_cast<const float4*>(tr)[q];
        const int id = t.n0 + c0 + 4 * q;
        topk_insert(tv, ti, x.x, id, false);
        topk_insert(tv, ti, x.y, id + 1, false);
        topk_insert(tv, ti, x.z, id + 2, false);
        topk_insert(tv, ti, x.w, id + 3, false);
      }
    }
    __syncthreads();          // the next tile's K loop reuses the LDS
  }
  // the row's two halves (lanes l and l ^ 32): ids interleave, so ties compare ids
  float pv[kTopkList];
  int pi[kTopkList];
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) { pv[j] = lane_partner<5>(tv[j]); pi[j] = lane_partner<5>(ti[j]); }
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) topk_insert(tv, ti, pv[j], pi[j], true);
  if (half == 0 && rl < rows) {
    TopkPart rec;
#pragma unroll
    for (int j = 0; j < kTopkList; ++j) { rec.v[j] = tv[j]; rec.id[j] = ti[j]; }
    out[(size_t)(m0 + rl) * nseg + sg] = rec;
  }
}

int topk_segments(int M, int vocab) {
  const int nmb = cdiv(M, kHeadChunk), nchunk = cdiv(vocab, kHeadChunk);
  int nseg = cdiv(256, nmb);
  return nseg < 1 ? 1 : (nseg > nchunk ? nchunk : nseg);
}

template <typename T>
hipError_t gemm_lm_head_topk(const T* A, int lda, const T* B, int ldb, int M, int V, int K, int nseg, TopkPart* out,
                             Gate g, int n, hipStream_t s) {
  if constexpr (sizeof(T) != 2) {
    return hipErrorInvalidValue;
  } else {
    if (V % 64 || K % 64 || M <= 0) return hipErrorInvalidValue;
    const int nmb = cdiv(M, kHeadChunk), nchunk = cdiv(V, kHeadChunk);
    const int cps = cdiv(nchunk, nseg);
    hipLaunchKernelGGL((k_lm_head_topk<T, TileCfgD<kHeadChunk, kHeadChunk, 2>, BLPlain<T>>), dim3(nmb * nseg),
                       dim3(256), 0, s, ALPlain<T>{A, lda}, BLPlain<T>{B, ldb}, (const float*)nullptr, M, V, K, nseg,
                       cps, out, g, n);
    return hipGetLastError();
  }
}

hipError_t gemm_lm_head_topk_fp8(const bf16* A, int lda, const fp8e4m3* B8, const float* bscale, int M, int V, int K,
                                 int nseg, TopkPart* out, Gate g, int n, hipStream_t s) {
  if (V % 64 || K % 64 || M <= 0) return hipErrorInvalidValue;
  const int nmb = cdiv(M, kHeadChunk), nchunk = cdiv(V, kHeadChunk);
  const int cps = cdiv(nchunk, nseg);
  hipLaunchKernelGGL((k_lm_head_topk<bf16, TileCfgD<kHeadChunk, kHeadChunk, 2, 1, true>, BLPackedFp8Rows>),
                     dim3(nmb * nseg), dim3(256), 0, s, ALPlain<bf16>{A, lda}, BLPackedFp8Rows{B8, V, K}, bscale, M, V,
                     K, nseg, cps, out, g, n);
  return hipGetLastError();
}
template hipError_t gemm_lm_head_topk<float>(const float*, int, const float*, int, int, int, int, int, TopkPart*, Gate,
                                             int, hipStream_t);
template hipError_t gemm_lm_head_topk<bf16>(const bf16*, int, const bf16*, int, int, int, int, int, TopkPart*, Gate,
                                            int, hipStream_t);

// Grouped products on the DMA tile loop take 128-row tiles: each 128 x 128
// tile reads 32 KB of operands per 64-wide K step for 2 MFLOP, against 24 KB
// for 1 MFLOP with 64-row tiles.
static bool expert_group_dma(int d, int F, size_t es) { return es == 2 && d % 64 == 0 && F % 64 == 0; }
int expert_group_tile_rows(int d, int F, size_t es) { return expert_group_dma(d, F, es) ? 128 : 64; }

template <typename T>
hipError_t gemm_expert_gateup(const T* X, const int* perm, const T* gate, const T* up, T* act,
                              const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F,
                              hipStream_t s, const T* pgu) {
  if constexpr (sizeof(T) == 2) {
    if (expert_group_dma(d, F, sizeof(T))) {
      // 128 rows x 64 features (gate and up interleaved) per tile; the
      // fragment-packed weights when the model holds them, else the caller's rows
      SchedGroup<128, 128> sc{tiles, n_tiles, cdiv(F, 64), F, d, 64};
      if (pgu != nullptr)
        return launch_dma<TileCfgD<128, 128, kGroupStages>>(cap_tiles * sc.nt, sc, ALGather<T>{X, d, perm},
                                                            BLPackedGateUp<T>{pgu, F, d}, EpSwiGLU<T>{act, F}, s);
      return launch_dma<TileCfgD<128, 128, kGroupStages>>(cap_tiles * sc.nt, sc, ALGather<T>{X, d, perm},
                                                          BLGateUp<T>{gate, up, (size_t)F * d, d},
                                                          EpSwiGLU<T>{act, F}, s);
    }
  }
  using C = TileCfg<T, 64, 64>;
  SchedGroup<64, 64> sc{tiles, n_tiles, cdiv(F, 32), F, d, 32};
  return launch<C, T>(cap_tiles * sc.nt, sc, ALGather<T>{X, d, perm}, BLGateUp<T>{gate, up, (size_t)F * d, d},
                      EpSwiGLU<T>{act, F}, s);
}

template <typename T>
hipError_t gemm_expert_down(const T* act, const T* down, T* Y, const int4* tiles,
                            const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s, const T* pd) {
  if constexpr (sizeof(T) == 2) {
    if (expert_group_dma(d, F, sizeof(T))) {
      SchedGroup<128, 128> sc{tiles, n_tiles, cdiv(d, 128), d, F, 128};
      if (pd != nullptr)
        return launch_dma<TileCfgD<128, 128, kGroupStages>>(cap_tiles * sc.nt, sc, ALRows<T>{act, F},
                                                            BLPackedRows<T>{pd, d, F}, EpStore<T>{Y, d}, s);
      return launch_dma<TileCfgD<128, 128, kGroupStages>>(cap_tiles * sc.nt, sc, ALRows<T>{act, F},
                                                          BLExpert<T>{down, (size_t)d * F, F}, EpStore<T>{Y, d}, s);
    }
  }
  using C = TileCfg<T, 64, 64>;
  SchedGroup<64, 64> sc{tiles, n_tiles, cdiv(d, 64), d, F, 64};
  return launch<C, T>(cap_tiles * sc.nt, sc, ALRows<T>{act, F}, BLExpert<T>{down, (size_t)d * F, F},
                      EpStore<T>{Y, d}, s);
}

template <typename T>
hipError_t gemm_selfcond(const T* P, const float* scale, int nchunk, const T* Bt, float* part, int M, int N, int K,
                         int splits, int kchunk, Gate g, int n, hipStream_t s) {
  if constexpr (sizeof(T) == 2) {
    if (M >= 128 && N >= 128 && kchunk % 128 == 0 && K % 64 == 0) {
      SchedDense<128, 128> sc{M, N, K, cdiv(M, 128), cdiv(N, 128), splits, kchunk, g, n};
      return launch_dma<TileCfgD<128, 128, 2>>(sc.mt * sc.nt * splits, sc, ALChunkScaled<T>{P, K, scale, nchunk},
                                               BLPlain<T>{Bt, K}, EpStoreF32{part, N, (size_t)M * N}, s);
    }
  }
  const ALScaled<T> al{P, K, scale, nchunk};
  if (M >= 128 && N >= 128) {
    using C = TileCfg<T, 128, 128>;
    SchedDense<128, 128> sc{M, N, K, cdiv(M, 128), cdiv(N, 128), splits, kchunk, g, n};
    return launch<C, T>(sc.mt * sc.nt * splits, sc, al, BLPlain<T>{Bt, K}, EpStoreF32{part, N, (size_t)M * N}, s);
  }
  using C = TileCfg<T, 64, 64>;
  SchedDense<64, 64> sc{M, N, K, cdiv(M, 64), cdiv(N, 64), splits, kchunk, g, n};
  return launch<C, T>(sc.mt * sc.nt * splits, sc, al, BLPlain<T>{Bt, K}, EpStoreF32{part, N, (size_t)M * N}, s);
}

#define DG_INST(T)                                                                                       \
  template hipError_t gemm_partials<T>(const T*, int, const T*, int, float*, int, int, int, SplitPlan,    \
                                       Gate, int, hipStream_t);                                         \
  template hipError_t gemm_partials_f32a<T>(const float*, int, const T*, int, float*, int, int, int,      \
                                            SplitPlan, Gate, int, hipStream_t);                         \
  template hipError_t gemm_lm_head<T>(const T*, int, const T*, int, int, int, int, const HeadArgs<T>&,      \
                                      hipStream_t);                                                     \
  template hipError_t gemm_qkv_rope<T>(const T*, const T*, int, int, int, const float2*, T*, T*, T*, int, int, \
                                       int, int, PosArg, Gate, hipStream_t);                            \
  template hipError_t gemm_expert_gateup<T>(const T*, const int*, const T*, const T*, T*, const int4*,    \
                                            const int*, int, int, int, hipStream_t, const T*);          \
  template hipError_t gemm_expert_down<T>(const T*, const T*, T*, const int4*, const int*, int, int,      \
                                          int, hipStream_t, const T*);                                  \
  template hipError_t gemm_selfcond<T>(const T*, const float*, int, const T*, float*, int, int, int, int, \
                                       int, Gate, int, hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

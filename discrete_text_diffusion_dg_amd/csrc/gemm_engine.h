// MFMA tile engine for the matrix products of the denoise step (gfx950).
//
// One workgroup = 4 wave64s computes a 64 x 64 fp32 tile of C = A * B^T with
// A [rows, K] and B [cols, K] both K-contiguous.  K is walked in 128-byte
// slices (64 bf16 or 32 fp32 elements) staged through LDS with two buffers:
// the next slice is fetched into registers while the current one feeds the
// matrix cores, then written to the other buffer, one barrier per slice.
// Waves are arranged 2 x 2; each owns a 32 x 32 sub-tile = 2 x 2 MFMA blocks
// of 16 x 16 (v_mfma_f32_16x16x32_bf16, or 8 x v_mfma_f32_16x16x4_f32).
//
// Schedulers map a workgroup id to a tile (dense, grouped by expert, or split
// along K); loaders produce 16 bytes of operand data for (tile row, k); an
// epilogue consumes the accumulators.
#pragma once
#include "dg_common.h"

namespace dg {

struct TileCtx {
  int m0, n0;        // first row / column of the tile in C
  int rows, cols;    // valid rows / columns (<= 64)
  int k0, k1;        // K range handled by this workgroup
  int group;         // expert id (grouped GEMMs), split index (split-K)
  int row_base;      // first gathered row of the tile (grouped GEMMs)
};

template <typename T>
struct TileShape {
  static constexpr int BM = 64, BN = 64;
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(T);      // K elements per slice
  static constexpr int LDK = BK + EPC;                 // padded LDS row stride (elements)
  static constexpr int KSTEPS = BK / 32;
  static constexpr int kSmemBytes = 2 * 2 * BM * LDK * (int)sizeof(T);
};

// ------------------------------------------------------------------ schedulers
// Dense tiles, column-tile major so that the row tiles sharing a weight tile are
// consecutive; when the tile count is a multiple of 8, consecutive logical tiles
// are placed on the same XCD (workgroups are dealt round-robin over 8 XCDs).
struct SchedDense {
  int M, N, K, mt, nt;
  __device__ bool get(int bid, TileCtx& t) const {
    const int total = mt * nt;
    if (bid >= total) return false;
    int idx = bid;
    if ((total & 7) == 0) idx = (bid & 7) * (total >> 3) + (bid >> 3);
    const int tm = idx % mt, tn = idx / mt;
    t.m0 = tm * 64; t.n0 = tn * 64;
    t.rows = min(64, M - t.m0); t.cols = min(64, N - t.n0);
    t.k0 = 0; t.k1 = K; t.group = 0; t.row_base = t.m0;
    return true;
  }
};

// Expert-grouped tiles: a device list of (expert, first gathered row, rows).
struct SchedGroup {
  const int4* tiles;
  const int* n_tiles;
  int nt, N, K, bn;      // bn: output columns per tile (64, or 32 for gate/up)
  __device__ bool get(int bid, TileCtx& t) const {
    const int ti = bid / nt, tn = bid % nt;
    if (ti >= *n_tiles) return false;
    const int4 d = tiles[ti];
    t.group = d.x; t.row_base = d.y; t.rows = d.z;
    t.m0 = 0; t.n0 = tn * bn; t.cols = min(bn, N - t.n0);
    t.k0 = 0; t.k1 = K;
    return true;
  }
};

// Split-K over equal K chunks; the split index goes to t.group.
struct SchedSplitK {
  int M, N, K, mt, nt, splits, kchunk;
  __device__ bool get(int bid, TileCtx& t) const {
    const int per = mt * nt;
    if (bid >= per * splits) return false;
    const int s = bid / per, r = bid % per;
    const int tn = r / mt, tm = r % mt;
    t.m0 = tm * 64; t.n0 = tn * 64;
    t.rows = min(64, M - t.m0); t.cols = min(64, N - t.n0);
    t.k0 = s * kchunk; t.k1 = min(K, t.k0 + kchunk);
    t.group = s; t.row_base = t.m0;
    return true;
  }
};

// ------------------------------------------------------------------ loaders
__device__ __forceinline__ uint4 zero16() { return make_uint4(0, 0, 0, 0); }

template <typename T>
struct ALPlain {            // A rows m0 + r of a K-contiguous matrix
  const T* p; int lda;
  __device__ uint4 load(const TileCtx& t, int r, int k) const {
    if (r >= t.rows) return zero16();
    return *reinterpret_cast<const uint4*>(p + (size_t)(t.m0 + r) * lda + k);
  }
};

template <typename T>
struct ALRows {             // A rows row_base + r (grouped, contiguous per tile)
  const T* p; int lda;
  __device__ uint4 load(const TileCtx& t, int r, int k) const {
    if (r >= t.rows) return zero16();
    return *reinterpret_cast<const uint4*>(p + (size_t)(t.row_base + r) * lda + k);
  }
};

template <typename T>
struct ALGather {           // A rows perm[row_base + r] (tokens routed to one expert)
  const T* p; int lda; const int* perm;
  __device__ uint4 load(const TileCtx& t, int r, int k) const {
    if (r >= t.rows) return zero16();
    const int src = perm[t.row_base + r];
    return *reinterpret_cast<const uint4*>(p + (size_t)src * lda + k);
  }
};

template <typename T> struct ALF32;   // fp32 source converted to the operand type
template <>
struct ALF32<float> {
  const float* p; int lda;
  __device__ uint4 load(const TileCtx& t, int r, int k) const {
    if (r >= t.rows) return zero16();
    return *reinterpret_cast<const uint4*>(p + (size_t)(t.m0 + r) * lda + k);
  }
};
template <>
struct ALF32<bf16> {
  const float* p; int lda;
  __device__ uint4 load(const TileCtx& t, int r, int k) const {
    if (r >= t.rows) return zero16();
    const float4* s = reinterpret_cast<const float4*>(p + (size_t)(t.m0 + r) * lda + k);
    const float4 a = s[0], b = s[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return pack8_bf16(v);
  }
};

template <typename T>
struct BLPlain {            // B rows n0 + n of a [N, K] matrix
  const T* p; int ldb;
  __device__ uint4 load(const TileCtx& t, int n, int k) const {
    if (n >= t.cols) return zero16();
    return *reinterpret_cast<const uint4*>(p + (size_t)(t.n0 + n) * ldb + k);
  }
};

template <typename T>
struct BLExpert {           // B rows of expert `group`: base + group * stride
  const T* p; size_t stride; int ldb;
  __device__ uint4 load(const TileCtx& t, int n, int k) const {
    if (n >= t.cols) return zero16();
    return *reinterpret_cast<const uint4*>(p + (size_t)t.group * stride + (size_t)(t.n0 + n) * ldb + k);
  }
};

template <typename T>
struct BLGateUp {           // tile rows 0..31: gate rows n0.., rows 32..63: up rows n0..
  const T* gate; const T* up; size_t stride; int ldb;
  __device__ uint4 load(const TileCtx& t, int n, int k) const {
    const int nn = n & 31;
    if (nn >= t.cols) return zero16();
    const T* base = (n < 32 ? gate : up) + (size_t)t.group * stride;
    return *reinterpret_cast<const uint4*>(base + (size_t)(t.n0 + nn) * ldb + k);
  }
};

// ------------------------------------------------------------------ the tile loop
// acc[tm][tn][i] holds C[wm*32 + tm*16 + (lane>>4)*4 + i][wn*32 + tn*16 + (lane&15)].
template <typename T, class AL, class BL>
__device__ __forceinline__ void tile_mma(const TileCtx& t, const AL& al, const BL& bl, char* smem,
                                         f32x4_t (&acc)[2][2]) {
  using S = TileShape<T>;
  T* sA = reinterpret_cast<T*>(smem);
  T* sB = sA + 2 * S::BM * S::LDK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (t.k1 - t.k0) / S::BK;
  if (nk <= 0) return;
  uint4 ra[2], rb[2];
  int rr[2], cc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    rr[i] = c >> 3;
    cc[i] = (c & 7) * S::EPC;
  }
  auto gload = [&](int k) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      ra[i] = al.load(t, rr[i], k + cc[i]);
      rb[i] = bl.load(t, rr[i], k + cc[i]);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<uint4*>(sA + buf * S::BM * S::LDK + rr[i] * S::LDK + cc[i]) = ra[i];
      *reinterpret_cast<uint4*>(sB + buf * S::BM * S::LDK + rr[i] * S::LDK + cc[i]) = rb[i];
    }
  };
  gload(t.k0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload(t.k0 + (kt + 1) * S::BK);
    const T* a0 = sA + cur * S::BM * S::LDK;
    const T* b0 = sB + cur * S::BM * S::LDK;
#pragma unroll
    for (int s = 0; s < S::KSTEPS; ++s) {
      Frag<T> fa[2], fb[2];
      const int kk = s * 32 + (lane >> 4) * 8;
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        lds_frag(fa[q], a0 + (wm * 32 + q * 16 + (lane & 15)) * S::LDK + kk);
        lds_frag(fb[q], b0 + (wn * 32 + q * 16 + (lane & 15)) * S::LDK + kk);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) mma16x16x32(acc[a][b], fa[a], fb[b]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }
}

// Visit every accumulator element with its tile-relative (row, col).
template <class F>
__device__ __forceinline__ void for_each_acc(const f32x4_t (&acc)[2][2], F&& f) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f(wm * 32 + a * 16 + (lane >> 4) * 4 + i, wn * 32 + b * 16 + (lane & 15), acc[a][b][i]);
}

template <typename T, class SCHED, class AL, class BL, class EP>
__global__ __launch_bounds__(256) void k_gemm(SCHED sc, AL al, BL bl, EP ep) {
  __shared__ __attribute__((aligned(16))) char smem[TileShape<T>::kSmemBytes];
  TileCtx t;
  if (!sc.get(blockIdx.x, t)) return;
  f32x4_t acc[2][2];
  tile_mma<T>(t, al, bl, smem, acc);
  ep(t, acc, smem);
}

}  // namespace dg

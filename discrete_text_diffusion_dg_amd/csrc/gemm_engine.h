// MFMA tile engine for the matrix products of the denoise step (gfx950).
//
// One workgroup = 4 wave64s computes a BM x BN fp32 tile of C = A * B^T with
// A [rows, K] and B [cols, K] both K-contiguous (BM, BN in {64, 128}).  Waves
// are arranged 2 x 2; each owns a (BM/2) x (BN/2) sub-tile made of 16 x 16
// MFMA blocks (v_mfma_f32_16x16x32_bf16, or 8 x v_mfma_f32_16x16x4_f32).
//
// K is walked in 128-byte slices (64 bf16 / 32 fp32 per row).  Global loads
// run STAGES-1 slices ahead of the matrix cores: each thread keeps STAGES-1
// slices in registers, and the slice about to be used is written to one of two
// LDS buffers, one barrier per slice.  With little arithmetic per slice (the
// batch-1 products stream weights), the number of slices in flight is what
// sets the achieved bandwidth.
//
// Schedulers map a workgroup id to a tile (dense, grouped by expert, split
// along K); loaders produce 16 bytes of operand data for (tile row, k); an
// epilogue consumes the accumulators (and may reuse the tile's shared memory,
// free once the K loop has ended).
//
// bf16 products whose loaders only locate rows (plain, grouped, gathered) use
// a second tile loop, tile_mma_dma: operand rows go from global memory
// straight into LDS (16 bytes per lane, no register staging) through an
// S-stage ring, S-1 slices ahead of the matrix cores.  A slice row (128 bytes)
// keeps its eight 16-byte pieces in a rotated order, piece q of tile row r at
// position q ^ ((r >> 1) & 7), so every row is still fetched as one whole
// cache line and each 16-lane phase of a fragment read touches 16 distinct
// bank groups.  Each wave waits for its own slice loads with an explicit
// memory-counter wait and the slice is handed over with an LDS-only barrier,
// so the later slices' loads stay in flight.
#pragma once
#include "dg_kernels.h"

#include <type_traits>

namespace dg {

struct TileCtx {
  int m0, n0;        // first row / column of the tile in C
  int rows, cols;    // valid rows / columns of the tile
  int k0, k1;        // K range handled by this workgroup
  int group;         // expert id (grouped products), split index (split-K)
  int row_base;      // first output row of the tile (gathered rows for grouped products)
};

template <typename T, int BM_, int BN_, int STAGES_ = 3>
struct TileCfg {
  static constexpr int BM = BM_, BN = BN_, STAGES = STAGES_, KG = 1;
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per 16-byte chunk
  static constexpr int BK = 128 / (int)sizeof(T);      // K elements per slice
  static constexpr int LDK = BK + EPC;                 // padded LDS row stride (elements)
  static constexpr int KSTEPS = BK / 32;
  static constexpr int WM = BM / 2, WN = BN / 2;       // per-wave sub-tile
  static constexpr int FM = WM / 16, FN = WN / 16;     // MFMA blocks per wave
  static constexpr int ACH = BM * 8 / 256, BCH = BN * 8 / 256;   // 16 B chunks per thread per slice
  static constexpr int kSmemBytes = 2 * (BM + BN) * LDK * (int)sizeof(T);
};

// ------------------------------------------------------------------ schedulers
// (xcd_run, in dg_common.h, gives each XCD a contiguous run of logical tiles)

// Dense tiles in bands of kBandRows row tiles: within a band the row tiles
// vary fastest, then the column tiles, so the workgroups resident on one XCD
// at a time cover about 8 row tiles x 8 column tiles and both operands are
// re-read from that XCD's L2 (column-major over all row tiles would stream
// the whole A operand through every L2 once per column tile).  Optional
// split-K: the split index varies slowest.
constexpr int kBandRows = 8;
template <int BM, int BN>
struct SchedDense {
  int M, N, K, mt, nt, splits, kchunk;
  Gate gate;       // tiles whose rows all belong to requests left out are skipped
  int n;           // rows per request (with a gate)
  __device__ bool get(int bid, TileCtx& t) const {
    const int per = mt * nt, total = per * splits;
    if (bid >= total) return false;
    const int idx = xcd_run(bid, total);
    const int s = idx / per, r = idx % per;
    const int band = r / (kBandRows * nt), first = band * kBandRows;
    const int bh = min(kBandRows, mt - first), rb = r - band * kBandRows * nt;
    const int tm = first + rb % bh, tn = rb / bh;
    t.m0 = tm * BM; t.n0 = tn * BN;
    t.rows = min(BM, M - t.m0); t.cols = min(BN, N - t.n0);
    t.k0 = s * kchunk; t.k1 = min(K, t.k0 + kchunk);
    t.group = s; t.row_base = t.m0;
    return gate.p == nullptr || gate.any_active(t.m0, t.rows, n);
  }
};

// Expert-grouped tiles: a device list of (expert, first gathered row, rows).
template <int BM, int BN>
struct SchedGroup {
  const int4* tiles;
  const int* n_tiles;
  int nt, N, K, bn;      // bn: output columns per tile
  __device__ bool get(int bid, TileCtx& t) const {
    // The grid is sized for the list's capacity; the first n_tiles * nt
    // workgroups take a tile each.  Workgroup bid runs on XCD bid % 8: XCD x
    // takes a contiguous run of (row tile, column tile) pairs, column tiles
    // fastest, so the workgroups sharing a row tile (and the tiles of one
    // expert) meet in one L2.
    const int total = *n_tiles * nt;
    if (bid >= total) return false;
    const int idx = xcd_run(bid, total);
    const int ti = idx / nt, tn = idx % nt;
    const int4 d = tiles[ti];
    t.group = d.x; t.row_base = d.y; t.rows = d.z;
    t.m0 = 0; t.n0 = tn * bn; t.cols = min(bn, N - t.n0);
    t.k0 = 0; t.k1 = K;
    return true;
  }
};

// ------------------------------------------------------------------ loaders
// A loader resolves, once per tile, the row a thread copies (row(), returning
// the loader's Row: a row pointer, or more per-row state); every K-slice then
// reads 16 bytes at an offset of that row (ld()).  Rows past the
// tile's valid range are clamped to a valid row and their data zeroed after the
// load, so every thread issues the same loads and the memory-wait counts stay
// exact for the pipeline.
__device__ __forceinline__ uint4 zero16() { return make_uint4(0, 0, 0, 0); }

template <typename T>
__device__ __forceinline__ uint4 ld16(const void* rowp, int k) {
  return *reinterpret_cast<const uint4*>(static_cast<const T*>(rowp) + k);
}

template <typename T>
struct ALPlain {            // A rows m0 + r of a K-contiguous matrix
  using Row = const void*;
  const T* p; int lda;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)(t.m0 + (valid ? r : 0)) * lda;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

template <typename T>
struct ALRows {             // A rows row_base + r (grouped, contiguous per tile)
  using Row = const void*;
  const T* p; int lda;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)(t.row_base + (valid ? r : 0)) * lda;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

template <typename T>
struct ALGather {           // A rows perm[row_base + r] (tokens routed to one expert)
  using Row = const void*;
  const T* p; int lda; const int* perm;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)perm[t.row_base + (valid ? r : 0)] * lda;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

template <typename T> struct ALF32;   // fp32 source converted to the operand type
template <>
struct ALF32<float> {
  using Row = const void*;
  const float* p; int lda;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)(t.m0 + (valid ? r : 0)) * lda;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<float>(rp, k); }
};
template <>
struct ALF32<bf16> {
  using Row = const void*;
  const float* p; int lda;
  __device__ const void* row(const TileCtx& t, int r, bool& valid) const {
    valid = r < t.rows;
    return p + (size_t)(t.m0 + (valid ? r : 0)) * lda;
  }
  __device__ uint4 ld(const void* rp, int k) const {
    const float4* s = reinterpret_cast<const float4*>(static_cast<const float*>(rp) + k);
    const float4 a = s[0], b = s[1];
    const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    return pack8_bf16(v);
  }
};

template <typename T>
struct BLPlain {            // B rows n0 + n of a [N, K] matrix
  using Row = const void*;
  const T* p; int ldb;
  __device__ const void* row(const TileCtx& t, int n, bool& valid) const {
    valid = n < t.cols;
    return p + (size_t)(t.n0 + (valid ? n : 0)) * ldb;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

template <typename T>
struct BLExpert {           // B rows of expert `group`: base + group * stride
  using Row = const void*;
  const T* p; size_t stride; int ldb;
  __device__ const void* row(const TileCtx& t, int n, bool& valid) const {
    valid = n < t.cols;
    return p + (size_t)t.group * stride + (size_t)(t.n0 + (valid ? n : 0)) * ldb;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

// Gate and up rows interleaved in blocks of 16: tile rows [32j, 32j+16) are
// gate rows n0 + 16j.., rows [32j+16, 32j+32) the up rows of the same features,
// so each wave's accumulator holds gate and up of the same 16 features side by side.
template <typename T>
struct BLGateUp {
  using Row = const void*;
  const T* gate; const T* up; size_t stride; int ldb;
  __device__ const void* row(const TileCtx& t, int n, bool& valid) const {
    const int f = (n >> 5) * 16 + (n & 15);     // feature within the tile
    valid = f < t.cols;
    const T* base = ((n & 16) ? up : gate) + (size_t)t.group * stride;
    return base + (size_t)(t.n0 + (valid ? f : 0)) * ldb;
  }
  __device__ uint4 ld(const void* rp, int k) const { return ld16<T>(rp, k); }
};

// B operands already in MFMA fragment order (the fragment-packed expert
// weights the streaming products read): for 16 B rows and a 32-wide K step,
// 64 lanes x 16 bytes, lane l holding row (l & 15), K elements (l >> 4) * 8.. .
// The DMA tile loop copies each such kilobyte as is into LDS and reads it back
// one 16-byte piece per lane.
//   BLPackedGateUp: PGU[e][F/16][K/32][gate, up][1 KB]; tile rows [32j, 32j+16)
//     are the gate rows of features n0 + 16j.., [32j+16, 32j+32) their up rows.
//   BLPackedRows:   PD[e][N/16][K/32][1 KB]; tile rows n0 + ...
template <typename T>
struct BLPackedGateUp {
  using Row = const void*;
  static constexpr bool kPacked = true;
  const T* p; int F, K;
  // the kilobyte of 16-row block rb (of the tile) at K step ks; blocks past the
  // matrix repeat its last one (their products are never stored)
  __device__ const char* frag(const TileCtx& t, int rb, int ks) const {
    int fb = t.n0 / 16 + (rb >> 1);
    if (fb >= F / 16) fb = F / 16 - 1;
    const size_t ksn = (size_t)K / 32;
    return reinterpret_cast<const char*>(p) +
           ((((size_t)t.group * (F / 16) + fb) * ksn + ks) * 2 + (rb & 1)) * 1024;
  }
  static constexpr int kStepBytes = 2048;     // from one K step to the next
};
template <typename T>
struct BLPackedRows {
  using Row = const void*;
  static constexpr bool kPacked = true;
  const T* p; int N, K;
  __device__ const char* frag(const TileCtx& t, int rb, int ks) const {
    int fb = t.n0 / 16 + rb;
    if (fb >= N / 16) fb = N / 16 - 1;
    const size_t ksn = (size_t)K / 32;
    return reinterpret_cast<const char*>(p) + (((size_t)t.group * (N / 16) + fb) * ksn + ks) * 1024;
  }
  static constexpr int kStepBytes = 1024;
};
// FP8 (OCP E4M3) B rows in the order the FP8 expert products stream:
// P8[N/16][K/64][64 lanes][16 B], lane (c, g) of block (n/16, k/64) holding
// row n0 + c, K elements g*8 .. +8 then 32 + g*8 .. +8 -- one kilobyte per 16
// rows and 64-wide K step, copied as is into LDS by the DMA tile loop, whose
// fragment reads widen a lane's 8 codes of a 32-wide K step to bf16.  The
// per-row scales are left to the epilogue.
struct BLPackedFp8Rows {
  using Row = const void*;
  static constexpr bool kPacked = true;
  static constexpr bool kFp8 = true;
  const fp8e4m3* p; int N, K;
  // the kilobyte of 16-row block rb (of the tile) at 64-wide K step ks; blocks
  // past the matrix repeat its last one (their products are never stored)
  __device__ const char* frag(const TileCtx& t, int rb, int ks) const {
    int fb = t.n0 / 16 + rb;
    if (fb >= N / 16) fb = N / 16 - 1;
    return reinterpret_cast<const char*>(p) + ((size_t)fb * (size_t)(K / 64) + ks) * 1024;
  }
  static constexpr int kStepBytes = 1024;
};
template <class BL, class = void>
struct b_packed : std::false_type {};
template <class BL>
struct b_packed<BL, std::void_t<decltype(BL::kPacked)>> : std::integral_constant<bool, BL::kPacked> {};
template <class BL, class = void>
struct b_fp8 : std::false_type {};
template <class BL>
struct b_fp8<BL, std::void_t<decltype(BL::kFp8)>> : std::integral_constant<bool, BL::kFp8> {};

// ------------------------------------------------------------------ the tile loop
// acc[a][b][i] holds C[wm*WM + a*16 + (lane>>4)*4 + i][wn*WN + b*16 + (lane&15)].
template <class C, typename T, class AL, class BL>
__device__ __forceinline__ void tile_mma(const TileCtx& t, const AL& al, const BL& bl, char* smem,
                                         f32x4_t (&acc)[C::FM][C::FN]) {
  T* sA = reinterpret_cast<T*>(smem);
  T* sB = sA + 2 * C::BM * C::LDK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int nk = (t.k1 - t.k0) / C::BK;
  if (nk <= 0) return;
  constexpr int P = C::STAGES - 1;       // slices held in registers
  uint4 ra[P][C::ACH], rb[P][C::BCH];
  typename AL::Row arow[C::ACH];
  typename BL::Row brow[C::BCH];
  bool aval[C::ACH], bval[C::BCH];
#pragma unroll
  for (int i = 0; i < C::ACH; ++i) arow[i] = al.row(t, (tid + 256 * i) >> 3, aval[i]);
#pragma unroll
  for (int i = 0; i < C::BCH; ++i) brow[i] = bl.row(t, (tid + 256 * i) >> 3, bval[i]);
  const int kc = (tid & 7) * C::EPC;     // this thread's 16-byte column within a slice
  auto gload = [&](int slot, int kt) {
    if (kt >= nk) return;
    const int k = t.k0 + kt * C::BK + kc;
#pragma unroll
    for (int i = 0; i < C::ACH; ++i) {
      const uint4 v = al.ld(arow[i], k);
      ra[slot][i] = aval[i] ? v : zero16();
    }
#pragma unroll
    for (int i = 0; i < C::BCH; ++i) {
      const uint4 v = bl.ld(brow[i], k);
      rb[slot][i] = bval[i] ? v : zero16();
    }
  };
  auto sstore = [&](int slot, int buf) {
    T* a0 = sA + buf * C::BM * C::LDK;
    T* b0 = sB + buf * C::BN * C::LDK;
#pragma unroll
    for (int i = 0; i < C::ACH; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(a0 + (c >> 3) * C::LDK + (c & 7) * C::EPC) = ra[slot][i];
    }
#pragma unroll
    for (int i = 0; i < C::BCH; ++i) {
      const int c = tid + 256 * i;
      *reinterpret_cast<uint4*>(b0 + (c >> 3) * C::LDK + (c & 7) * C::EPC) = rb[slot][i];
    }
  };
  auto compute = [&](int buf) {
    const T* a0 = sA + buf * C::BM * C::LDK;
    const T* b0 = sB + buf * C::BN * C::LDK;
#pragma unroll
    for (int s = 0; s < C::KSTEPS; ++s) {
      const int kk = s * 32 + (lane >> 4) * 8;
      Frag<T> fa[C::FM], fb[C::FN];
#pragma unroll
      for (int a = 0; a < C::FM; ++a) lds_frag(fa[a], a0 + (wm * C::WM + a * 16 + (lane & 15)) * C::LDK + kk);
#pragma unroll
      for (int b = 0; b < C::FN; ++b) lds_frag(fb[b], b0 + (wn * C::WN + b * 16 + (lane & 15)) * C::LDK + kk);
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int b = 0; b < C::FN; ++b) mma16x16x32(acc[a][b], fa[a], fb[b]);
    }
  };

#pragma unroll
  for (int p = 0; p < P; ++p) gload(p, p);
  // slice kt sits in register slot kt % P; unrolled by P so every slot index is static
  for (int kt0 = 0; kt0 < nk; kt0 += P) {
#pragma unroll
    for (int u = 0; u < P; ++u) {
      const int kt = kt0 + u;
      if (kt < nk) {
        sstore(u, kt & 1);
        gload(u, kt + P);
        __syncthreads();
        compute(kt & 1);
      }
    }
  }
  __syncthreads();   // the epilogue may reuse the shared memory
}

// ------------------------------------------------------------------ the DMA tile loop (bf16)
// Same tile and accumulator layout as TileCfg<bf16, BM, BN> (4 waves, 2 x 2),
// S slices of 64 K-elements in LDS.  KG > 1: KG groups of 4 waves split the
// tile's K range (each with its own slice ring) and add their sums in LDS in
// group order before the epilogue -- more loads in flight per workgroup
// without split-K partials in global memory.
template <int BM_, int BN_, int S_, int KG_ = 1, bool B8_ = false>
struct TileCfgD {
  static constexpr int BM = BM_, BN = BN_, STAGES = S_, KG = KG_;
  static constexpr bool B8 = B8_;                           // B rows in FP8 (BLPackedFp8Rows)
  static constexpr int WM = BM / 2, WN = BN / 2;
  static constexpr int FM = WM / 16, FN = WN / 16;
  static constexpr int ROWB = 128;                          // bytes of a slice row (64 bf16)
  static constexpr int BROWB = B8_ ? 64 : ROWB;             // bytes of a B slice row
  static constexpr int STAGE = BM * ROWB + BN * BROWB;      // bytes of one slice of the tile
  static constexpr int NI = STAGE / 1024 / 4;               // 1 KB load groups per wave per slice
  static_assert(STAGE % 4096 == 0 && FM >= 1 && FN >= 1, "tile shape");
  static constexpr int RING = S_ * STAGE + S_ * BM * 4;   // a group's slices, then per-slice row scales (scaled loaders)
  static constexpr int RED = (KG_ - 1) * BM * BN * 4;       // groups 1..KG-1's sums for the reduction
  static constexpr int kSmemBytes = KG_ * RING > RED ? KG_ * RING : RED;
};

// Wait until at most N of this wave's vector-memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

// 16 bytes per lane from global memory straight into LDS: lane i writes
// lds_addr + 16 * i (lds_addr wave-uniform).  Issued from asm so that the
// compiler's wait insertion, which cannot tell these LDS writes from the
// fragment reads of other slices, does not drain them before every LDS read;
// the tile loop waits for them itself.  M0 is saved and restored around it.
__device__ __forceinline__ void lds_dma16(const void* g, uint32_t lds_addr) {
  uint32_t m0save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(m0save)
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(g)
               : "memory");
}

// 4 bytes per lane: lane i writes lds_addr + 4 * i.
__device__ __forceinline__ void lds_dma4(const void* g, uint32_t lds_addr) {
  uint32_t m0save;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
               : "=&s"(m0save)
               : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(g)
               : "memory");
}

// Loader traits: a loader that defines kChunkScale = true also supplies a
// per-row scale for every 128-element K chunk (scale_ptr(t, r, chunk)); the
// loop then sums each chunk's products apart and adds them in times the row's
// scale, in fp32.
template <class AL, class = void>
struct chunk_scaled : std::false_type {};
template <class AL>
struct chunk_scaled<AL, std::void_t<decltype(AL::kChunkScale)>> : std::integral_constant<bool, AL::kChunkScale> {};

template <class C, class AL, class BL>
__device__ __forceinline__ void tile_mma_dma(const TileCtx& t, const AL& al, const BL& bl, char* smem,
                                             f32x4_t (&acc)[C::FM][C::FN]) {
  constexpr bool BPACK = b_packed<BL>::value;
  constexpr bool B8 = b_fp8<BL>::value;
  static_assert(B8 == C::B8, "FP8 B rows need a tile configuration laid out for them");
  static_assert(std::is_same<typename AL::Row, const void*>::value &&
                    (BPACK || std::is_same<typename BL::Row, const void*>::value),
                "row-locating loaders only");
  // K group kg (4 waves) takes slices [kg * per, kg * per + nk) of the tile's
  // K range and its own slice ring; every group runs `per` slice steps so the
  // workgroup's barriers pair up
  const int tid = threadIdx.x & 255, kg = threadIdx.x >> 8, lane = tid & 63, w = tid >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b) acc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nk_all = (t.k1 - t.k0) / 64;
  if (nk_all <= 0) return;      // uniform over the workgroup
  const int per = (nk_all + C::KG - 1) / C::KG;
  const int nk = max(0, min(per, nk_all - kg * per));
  smem += kg * C::RING;
  // load group j of this wave: tile rows 8 * (w + 4 j) .. + 7 (A rows, then B
  // rows); lane (row rr = lane >> 3, position p = lane & 7) fetches piece
  // p ^ ((r >> 1) & 7) of its row.  Rows past the tile repeat a valid row;
  // their products are never stored.
  // packed B: its kilobytes follow the A rows in LDS, (16-row block, K step of
  // the slice) in order -- load group gi >= BM / 8 copies kilobyte gi - BM / 8
  // (FP8 rows: one kilobyte per 16-row block covers the slice's 64 K elements)
  const char* src[C::NI];
  uint32_t dst[C::NI];
  size_t adv[C::NI];          // bytes from one slice to the next
  const size_t kbase = (size_t)t.k0 + (size_t)kg * per * 64;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int gi = w + 4 * j;
    const int row = gi * 8 + (lane >> 3);
    const bool isA = row < C::BM;
    dst[j] = (uint32_t)(gi * 8 * C::ROWB);
    if constexpr (BPACK) {
      if (!isA) {
        const int gb = gi - C::BM / 8;
        if constexpr (B8) {
          src[j] = bl.frag(t, gb, (int)(kbase / 64)) + lane * 16;
          adv[j] = (size_t)BL::kStepBytes;
        } else {
          src[j] = bl.frag(t, gb >> 1, (int)(kbase / 32) + (gb & 1)) + lane * 16;
          adv[j] = 2 * (size_t)BL::kStepBytes;
        }
        continue;
      }
    }
    const int r = isA ? row : row - C::BM;
    bool valid;
    const void* rp;
    if constexpr (BPACK) rp = al.row(t, r, valid);
    else rp = isA ? al.row(t, r, valid) : bl.row(t, r, valid);
    const int q = (lane & 7) ^ ((r >> 1) & 7);
    src[j] = static_cast<const char*>(rp) + kbase * 2 + q * 16;
    adv[j] = 128;
  }
  const uint32_t lbase = (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)smem);
  constexpr bool SCALED = chunk_scaled<AL>::value;
  static_assert(!SCALED || (C::STAGES == 2 && C::BM == 128 && C::KG == 1), "chunk scales: two stages, 128 rows");
  // chunk scales: wave 0 brings the 128 rows' scales of a slice's chunk with the slice
  const char* ssrc[2] = {nullptr, nullptr};
  if constexpr (SCALED) {
    if (w == 0) {
      bool valid;
      ssrc[0] = static_cast<const char*>(al.scale_ptr(t, lane, t.k0 / 128, valid));
      ssrc[1] = static_cast<const char*>(al.scale_ptr(t, 64 + lane, t.k0 / 128, valid));
    }
  }
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const uint32_t sb = lbase + (uint32_t)((kt % C::STAGES) * C::STAGE);
#pragma unroll
    for (int j = 0; j < C::NI; ++j) lds_dma16(src[j] + (size_t)kt * adv[j], sb + dst[j]);
    if constexpr (SCALED) {
      if (w == 0) {
        const uint32_t slot = lbase + (uint32_t)(C::STAGES * C::STAGE + (kt % C::STAGES) * C::BM * 4);
        lds_dma4(ssrc[0] + (size_t)(kt >> 1) * 4, slot);
        lds_dma4(ssrc[1] + (size_t)(kt >> 1) * 4, slot + 256);
      }
    }
  };
  const int c16 = lane & 15, g4 = lane >> 4, sw = (c16 >> 1) & 7;
  const int aoff = (wm * C::WM + c16) * C::ROWB, boff = (C::BM + wn * C::WN + c16) * C::ROWB;
  f32x4_t accc[SCALED ? C::FM : 1][SCALED ? C::FN : 1];   // the current chunk's products (scaled loaders)
  // fresh: the first step of a 128-element chunk (scaled loaders) starts the
  // chunk products from zero in the matrix instruction itself
  auto kstep = [&](const char* sb, int kk, auto fresh) __attribute__((always_inline)) {
    constexpr bool FRESH = decltype(fresh)::value;
    const int ch = ((kk * 4 + g4) ^ sw) * 16;
    Frag<bf16> fa[C::FM], fb[C::FN];
#pragma unroll
    for (int a = 0; a < C::FM; ++a) fa[a].v = *reinterpret_cast<const uint4*>(sb + aoff + a * 16 * C::ROWB + ch);
#pragma unroll
    for (int b = 0; b < C::FN; ++b) {
      if constexpr (B8) {
        const uint4 u = *reinterpret_cast<const uint4*>(sb + C::BM * C::ROWB + (wn * C::WN / 16 + b) * 1024 + lane * 16);
        fb[b].v = kk == 0 ? fp8x8_to_bf16x8(u.x, u.y) : fp8x8_to_bf16x8(u.z, u.w);
      } else if constexpr (BPACK)
        fb[b].v = *reinterpret_cast<const uint4*>(sb + C::BM * C::ROWB + ((wn * C::WN / 16 + b) * 2 + kk) * 1024 +
                                                  lane * 16);
      else
        fb[b].v = *reinterpret_cast<const uint4*>(sb + boff + b * 16 * C::ROWB + ch);
    }
#pragma unroll
    for (int a = 0; a < C::FM; ++a)
#pragma unroll
      for (int b = 0; b < C::FN; ++b) {
        if constexpr (SCALED && FRESH) {
          accc[a][b] = f32x4_t{0.f, 0.f, 0.f, 0.f};
          mma16x16x32(accc[a][b], fa[a], fb[b]);
        } else if constexpr (SCALED) {
          mma16x16x32(accc[a][b], fa[a], fb[b]);
        } else {
          mma16x16x32(acc[a][b], fa[a], fb[b]);
        }
      }
  };
  using Fresh = std::true_type;
  using Cont = std::false_type;
#pragma unroll
  for (int p = 0; p < C::STAGES - 1; ++p)
    if (p < nk) issue(p);
  // one K slice: wait for this wave's loads of it, hand it over, issue the
  // slice S-1 ahead, two K steps
  auto slice = [&](int kt, auto fresh) __attribute__((always_inline)) {
    // this wave's loads of slice kt are done once at most the next S-2 slices' are outstanding
    if (kt + C::STAGES - 2 < nk) wait_vmcnt<(C::STAGES - 2) * C::NI>();
    else wait_vmcnt<0>();
    lds_barrier();            // slice kt is in LDS for every wave; slice kt-1 is no longer read
    if (kt + C::STAGES - 1 < nk) issue(kt + C::STAGES - 1);
    const char* sb = smem + (kt % C::STAGES) * C::STAGE;
    kstep(sb, 0, fresh);
    kstep(sb, 1, Cont{});
  };
  if constexpr (SCALED) {
    // a 128-element chunk is two slices (chunks start at even slices); its
    // products start from zero and end as acc += scale(row) * chunk products
    for (int kt = 0; kt < nk; kt += 2) {
      slice(kt, Fresh{});
      if (kt + 1 < nk) slice(kt + 1, Cont{});
      const int kl = kt + 1 < nk ? kt + 1 : kt;
      const float* sc = reinterpret_cast<const float*>(smem + C::STAGES * C::STAGE + (kl % C::STAGES) * C::BM * 4);
#pragma unroll
      for (int a = 0; a < C::FM; ++a) {
        const float4 s4 = *reinterpret_cast<const float4*>(sc + wm * C::WM + a * 16 + g4 * 4);
        const float sv[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[a][b][i] = __builtin_fmaf(sv[i], accc[a][b][i], acc[a][b][i]);
      }
    }
  } else {
    for (int kt = 0; kt < nk; ++kt) slice(kt, Cont{});
    if constexpr (C::KG > 1)
      for (int kt = nk; kt < per; ++kt) lds_barrier();   // a short (or empty) group keeps the barriers paired
  }
  __syncthreads();   // the epilogue may reuse the shared memory
  if constexpr (C::KG > 1) {
    // groups 1..KG-1 hand their sums to group 0, which adds them in group order
    float* red = reinterpret_cast<float*>(smem - kg * C::RING);
    constexpr int PT = C::FM * C::FN * 4;          // accumulator elements per thread
    if (kg > 0) {
#pragma unroll
      for (int a = 0; a < C::FM; ++a)
#pragma unroll
        for (int b = 0; b < C::FN; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((size_t)(kg - 1) * PT + (a * C::FN + b) * 4 + i) * 256 + tid] = acc[a][b][i];
    }
    __syncthreads();
    if (kg == 0) {
      for (int g = 1; g < C::KG; ++g)
#pragma unroll
        for (int a = 0; a < C::FM; ++a)
#pragma unroll
          for (int b = 0; b < C::FN; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[a][b][i] += red[((size_t)(g - 1) * PT + (a * C::FN + b) * 4 + i) * 256 + tid];
    }
    __syncthreads();
  }
}

// Visit every accumulator element with its tile-relative (row, col) and block
// indices (the first 4 waves: with K groups, group 0 holds the sums).
template <class C, class F>
__device__ __forceinline__ void for_each_acc(const f32x4_t (&acc)[C::FM][C::FN], F&& f) {
  if (threadIdx.x >= 256) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wm = w >> 1, wn = w & 1;
#pragma unroll
  for (int a = 0; a < C::FM; ++a)
#pragma unroll
    for (int b = 0; b < C::FN; ++b)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        f(wm * C::WM + a * 16 + (lane >> 4) * 4 + i, wn * C::WN + b * 16 + (lane & 15), acc[a][b][i]);
}

template <class C, typename T, class SCHED, class AL, class BL, class EP>
__global__ __launch_bounds__(256, 2) void k_gemm(SCHED sc, AL al, BL bl, EP ep) {
  constexpr int kBytes = C::kSmemBytes > EP::kSmemBytes ? C::kSmemBytes : EP::kSmemBytes;
  __shared__ __attribute__((aligned(16))) char smem[kBytes];
  TileCtx t;
  if (!sc.get(blockIdx.x, t)) return;
  f32x4_t acc[C::FM][C::FN];
  tile_mma<C, T>(t, al, bl, smem, acc);
  ep.template apply<C>(t, acc, smem);
}

// LDS: the slice ring, or what the epilogue needs if that is more
template <class C, class SCHED, class AL, class BL, class EP>
__global__ __launch_bounds__(256 * C::KG, C::KG == 1 ? 2 : 1) void k_gemm_dma(SCHED sc, AL al, BL bl, EP ep) {
  constexpr int kBytes = C::kSmemBytes > EP::kSmemBytes ? C::kSmemBytes : EP::kSmemBytes;
  __shared__ __attribute__((aligned(1024))) char smem[kBytes];
  TileCtx t;
  if (!sc.get(blockIdx.x, t)) return;
  f32x4_t acc[C::FM][C::FN];
  tile_mma_dma<C>(t, al, bl, smem, acc);
  ep.template apply<C>(t, acc, smem);
}

}  // namespace dg

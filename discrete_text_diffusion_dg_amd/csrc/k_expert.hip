// Expert SwiGLU products for thin routed tiles (at most 64 rows, the batch-1
// shapes): weights streamed from a fragment-packed layout, the tile's
// activation rows staged through LDS.
//
// Packed layout (built once by dg_model_create): a weight matrix W[N][K] of
// one expert is stored as blocks P[N/16][K/32][64 lanes][8 elements], where
// lane (c, g) of block (nb, ks) holds W[nb*16 + c][ks*32 + g*8 .. +8] -- exactly
// the MFMA B-operand fragment of that lane.  A wave's fragment load is then one
// contiguous 1 KB (bf16) read, so the weights stream at plain-copy efficiency.
// Gate and up of the same 16 features are interleaved per K step
// (PGU[F/16][d/32][2][64][8]) so silu(g) * u is formed lane-locally.
//
// A workgroup of NW waves owns NW feature blocks (of 16 outputs) of one tile;
// each wave streams the weights of its block over the whole K range.  The
// tile's activation rows are read once per workgroup, as whole cache lines,
// in chunks of KC K steps that are double-buffered in LDS (padded rows: the
// fragment reads of 8 lanes cover distinct banks), so the weight stream keeps
// the CU's memory requests to itself; the activations in registers would be
// re-read by every wave, in half-line pieces.  Chunks are handed over with an
// LDS-only barrier, so the weight loads in flight are not drained at the
// hand-over.  The number of row blocks (1..4) is a template parameter chosen
// per tile at run time, so every load of a path is unconditional and the
// memory-wait counts stay exact.
#include "dg_kernels.h"

#include <type_traits>

namespace dg {

namespace {

template <typename T>
__device__ __forceinline__ void frag_ld(Frag<T>& f, const T* p);
template <>
__device__ __forceinline__ void frag_ld(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
template <>
__device__ __forceinline__ void frag_ld(Frag<float>& f, const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p);
  const float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// K steps per group (the weight loads of the next group are issued before the
// MFMAs of the current one) and per staged activation chunk, per element type.
// Measured on the batch-1 tile lists (9..32 active experts of 32, d = F = 1024):
// one feature block per wave and four waves per workgroup (two workgroups per
// CU) beat wider blocks, eight or sixteen waves, and 128-row tiles.
template <typename T> struct StreamCfg;
template <> struct StreamCfg<bf16> { static constexpr int U = 2, KC = 4; };
template <> struct StreamCfg<float> { static constexpr int U = 1, KC = 2; };
constexpr int kStreamWaves = 4;

// ---- packing
// Gate/up of expert e: PGU[e][F/16][d/32][2][64][8] from gate/up [e][F][d].
template <typename T>
__global__ void k_pack_gateup(const T* gate, const T* up, T* out, int F, int d) {
  const size_t per_e = (size_t)F * d;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;    // one 8-element fragment per thread
  const size_t total = (size_t)gridDim.y * 2 * per_e / 8;
  (void)total;
  const int e = blockIdx.y;
  if (i >= 2 * per_e / 8) return;
  const int lane = (int)(i % 64);
  size_t rest = i / 64;
  const int which = (int)(rest % 2); rest /= 2;
  const int ks = (int)(rest % (d / 32));
  const int fb = (int)(rest / (d / 32));
  const int f = fb * 16 + (lane & 15), k = ks * 32 + (lane >> 4) * 8;
  const T* src = (which ? up : gate) + (size_t)e * per_e + (size_t)f * d + k;
  T* dst = out + (size_t)e * 2 * per_e + i * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = src[j];
}

// Down of expert e: PD[e][d/16][F/32][64][8] from down [e][d][F].
template <typename T>
__global__ void k_pack_down(const T* down, T* out, int d, int F) {
  const size_t per_e = (size_t)d * F;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int e = blockIdx.y;
  if (i >= per_e / 8) return;
  const int lane = (int)(i % 64);
  const size_t rest = i / 64;
  const int ks = (int)(rest % (F / 32));
  const int nb = (int)(rest / (F / 32));
  const int n = nb * 16 + (lane & 15), k = ks * 32 + (lane >> 4) * 8;
  const T* src = down + (size_t)e * per_e + (size_t)n * F + k;
  T* dst = out + (size_t)e * per_e + i * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) dst[j] = src[j];
}

// ---- streaming products
// GATEUP: out = act [rows][F] (T), B = PGU, A rows gathered through perm.
// else:   out = Y   [rows][d] (fp32), B = PD, A rows row_base + r of act.
// LDS: two stages of [64 rows][KC*32 + pad] elements; a stage holds K steps
// [c*KC, (c+1)*KC) of the tile's rows.
template <typename T, bool GATEUP, int RB, int NW, int U, int KC>
__device__ __forceinline__ void stream_body(const T* X, const int* perm, const T* Wp, void* out, int e,
                                            int row_base, int rows, int K, int N, int nb, T* lds) {
  constexpr int EPR = KC * 32;              // elements of a row per chunk
  constexpr int VEC = 16 / (int)sizeof(T);  // elements per 16-byte piece
  constexpr int LROW = EPR + VEC;           // padded LDS row (elements)
  constexpr int SEGS = EPR / VEC;           // pieces per row per chunk
  constexpr int NT = 64 * NW;
  constexpr int PIECES = RB * 16 * SEGS;
  static_assert(NT % SEGS == 0, "a thread's pieces share one column");
  constexpr int PPT = (PIECES + NT - 1) / NT;
  constexpr int RSTEP = NT / SEGS;          // rows between a thread's pieces
  constexpr int STAGE = 64 * LROW;          // elements per LDS stage
  constexpr int NF = GATEUP ? 2 : 1;        // B fragments per K step
  constexpr int GPC = KC / U;               // groups per chunk
  static_assert(GPC % 2 == 0, "the double buffer alternates within a chunk");

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
  const int KS = K / 32, NC = KS / KC;
  // staging: this thread moves pieces (row r0 + j * RSTEP, column seg) of every chunk
  const int seg = tid % SEGS, r0 = tid / SEGS;
  const T* aptr[PPT];
  bool pok[PPT];
#pragma unroll
  for (int j = 0; j < PPT; ++j) {
    const int r = r0 + j * RSTEP;
    pok[j] = PIECES % NT == 0 || r < RB * 16;
    // rows past the tile repeat a real row (their outputs are not stored), so
    // every staging load is issued
    const int rr = r < rows ? r : rows - 1;
    const int src = GATEUP ? perm[row_base + rr] : row_base + rr;
    aptr[j] = X + (size_t)src * K + seg * VEC;
  }
  uint4 st[PPT];
  auto stage_load = [&](int c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) st[j] = *reinterpret_cast<const uint4*>(aptr[j] + (size_t)c * EPR);
  };
  auto stage_store = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      if (pok[j]) *reinterpret_cast<uint4*>(lds + buf * STAGE + (r0 + j * RSTEP) * LROW + seg * VEC) = st[j];
  };

  constexpr int blk = NF * 512;             // elements per (block, K step)
  const T* bp = Wp + (size_t)e * NF * N * K + (size_t)nb * KS * blk + lane * 8;
  f32x4_t acc[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Frag<T> b[2][U][NF];
  auto load_b = [&](int buf, int ks0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int j = 0; j < NF; ++j) frag_ld(b[buf][u][j], bp + (size_t)(ks0 + u) * blk + j * 512);
  };
  // K steps kk .. kk+U-1 of the chunk in LDS stage abuf
  auto comp = [&](int buf, int abuf, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      Frag<T> a[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        lds_frag(a[rb], lds + abuf * STAGE + (rb * 16 + c16) * LROW + (kk + u) * 32 + g4 * 8);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NF; ++j) mma16x16x32(acc[rb][j], a[rb], b[buf][u][j]);
    }
  };
  // one chunk: stage the next one while its K steps stream; the last chunk
  // stages nothing and prefetches no weights past the end
  auto chunk = [&](int c, auto last) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last)::value;
    if (!LAST) stage_load(c + 1);
#pragma unroll
    for (int g = 0; g < GPC; ++g) {
      if (!LAST || g + 1 < GPC) load_b((g + 1) & 1, c * KC + (g + 1) * U);
      comp(g & 1, c & 1, g * U);
    }
    if (!LAST) stage_store((c + 1) & 1);
    lds_barrier();
  };
  stage_load(0);
  load_b(0, 0);
  stage_store(0);
  lds_barrier();
  int c = 0;
  for (; c + 1 < NC; ++c) chunk(c, std::false_type{});
  chunk(c, std::true_type{});

  // epilogue: the lane holds rows rb*16 + g4*4 + i, column c16 of the block
  const int col = nb * 16 + c16;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + g4 * 4 + i;
      if (r >= rows) continue;
      if (GATEUP) {
        const float g = acc[rb][0][i], u = acc[rb][1][i];
        Num<T>::store(static_cast<T*>(out) + (size_t)(row_base + r) * N + col, g / (1.0f + expf(-g)) * u);
      } else {
        static_cast<float*>(out)[(size_t)(row_base + r) * N + col] = acc[rb][0][i];
      }
    }
}

// Grid: x = N / (16 * NW) feature-block groups (exact), y = tile capacity
// (tiles past n_tiles exit; the exit is uniform over the workgroup, so every
// wave reaches the same barriers).
template <typename T, bool GATEUP, int NW, int U, int KC>
__global__ __launch_bounds__(64 * NW, 2) void k_expert_stream(const T* X, const int* perm, const T* Wp, void* out,
                                                              const int4* tiles, const int* n_tiles, int K, int N) {
  __shared__ __attribute__((aligned(16))) T lds[2 * 64 * (KC * 32 + 16 / sizeof(T))];
  const int ti = blockIdx.y;
  if (ti >= *n_tiles) return;
  const int4 td = tiles[ti];
  const int nb = blockIdx.x * NW + (int)(threadIdx.x >> 6);
  switch ((td.z + 15) >> 4) {
    case 1: stream_body<T, GATEUP, 1, NW, U, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 2: stream_body<T, GATEUP, 2, NW, U, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 3: stream_body<T, GATEUP, 3, NW, U, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    default: stream_body<T, GATEUP, 4, NW, U, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
  }
}

}  // namespace

bool expert_stream_ok(int d, int F, int elem_bytes) {
  const int KC = elem_bytes == 2 ? StreamCfg<bf16>::KC : StreamCfg<float>::KC;
  // whole staged chunks along K, whole workgroups of feature blocks along N
  return d % (32 * KC) == 0 && F % (32 * KC) == 0 && F % (16 * kStreamWaves) == 0 && d % (16 * kStreamWaves) == 0;
}

template <typename T>
hipError_t pack_expert_weights(const T* gate, const T* up, const T* down, T* pgu, T* pd, int E, int d, int F,
                               hipStream_t s) {
  const size_t frags_gu = 2 * (size_t)F * d / 8, frags_d = (size_t)d * F / 8;
  hipLaunchKernelGGL((k_pack_gateup<T>), dim3((unsigned)((frags_gu + 255) / 256), E), dim3(256), 0, s, gate, up, pgu,
                     F, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_pack_down<T>), dim3((unsigned)((frags_d + 255) / 256), E), dim3(256), 0, s, down, pd, d, F);
  return hipGetLastError();
}

template <typename T>
hipError_t expert_stream_gateup(const T* X, const int* perm, const T* pgu, T* act, const int4* tiles,
                                const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s) {
  constexpr int NW = kStreamWaves;
  hipLaunchKernelGGL((k_expert_stream<T, true, NW, StreamCfg<T>::U, StreamCfg<T>::KC>), dim3(F / (16 * NW), cap_tiles),
                     dim3(64 * NW), 0, s, X, perm, pgu, (void*)act, tiles, n_tiles, d, F);
  return hipGetLastError();
}

template <typename T>
hipError_t expert_stream_down(const T* act, const T* pd, float* Y, const int4* tiles, const int* n_tiles,
                              int cap_tiles, int d, int F, hipStream_t s) {
  constexpr int NW = kStreamWaves;
  hipLaunchKernelGGL((k_expert_stream<T, false, NW, StreamCfg<T>::U, StreamCfg<T>::KC>), dim3(d / (16 * NW), cap_tiles),
                     dim3(64 * NW), 0, s, act, (const int*)nullptr, pd, (void*)Y, tiles, n_tiles, F, d);
  return hipGetLastError();
}

#define DG_INST(T)                                                                                              \
  template hipError_t pack_expert_weights<T>(const T*, const T*, const T*, T*, T*, int, int, int, hipStream_t); \
  template hipError_t expert_stream_gateup<T>(const T*, const int*, const T*, T*, const int4*, const int*, int, \
                                              int, int, hipStream_t);                                         \
  template hipError_t expert_stream_down<T>(const T*, const T*, float*, const int4*, const int*, int, int, int, \
                                            hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

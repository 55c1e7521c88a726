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
// each wave streams the weights of its block over the whole K range through a
// ring of PD K steps of fragments: the load of step s + PD is issued as soon as
// step s has been multiplied, so PD steps of weights stay in flight.  The
// tile's activation rows are read once per workgroup, as whole cache lines, in
// chunks of KC K steps that are double-buffered in LDS (padded rows: the
// fragment reads of 8 lanes cover distinct banks), and the staging registers
// are double-buffered too: the rows of chunk c + 2 are requested when chunk c
// starts and written to LDS when chunk c + 1 ends, so a staging load is never
// waited on in the chunk that issued it (the memory counter completes in
// order: waiting on it would also drain the weight ring).  Chunks are handed
// over with an LDS-only barrier.  The number of row blocks (1..4) is a
// template parameter chosen per tile at run time, so every load of a path is
// unconditional and the memory-wait counts stay exact.
#include "dg_kernels.h"

#include <type_traits>
#include <utility>

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

// Weight ring depth PD and activation chunk KC (K steps), per element type and
// product.  Measured on batch-1 tile lists (11..32 active experts of 32,
// d = F = 1024, bf16): gate/up gains 10-25% from an 8-step ring on the skewed
// lists; the down product, with half the bytes per step, is flat from 2 to 8.
template <typename T, bool GATEUP> struct StreamCfg;
template <> struct StreamCfg<bf16, true> { static constexpr int PD = 8, KC = 4; };
template <> struct StreamCfg<bf16, false> { static constexpr int PD = 4, KC = 4; };
template <bool G> struct StreamCfg<float, G> { static constexpr int PD = 2, KC = 2; };
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
template <int... U, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}

// GATEUP: out = act [rows][F] (T), B = PGU, A rows gathered through perm.
// else:   out = Y   [rows][d] (fp32), B = PD, A rows row_base + r of act.
// LDS: two stages of [64 rows][KC*32 + pad] elements; a stage holds K steps
// [c*KC, (c+1)*KC) of the tile's rows.  The K loop runs in super steps of SS
// K steps (an even number of chunks, a multiple of the ring depth), unrolled so
// that every ring slot and staging set is a compile-time index.
template <typename T, bool GATEUP, int RB, int NW, int PD, int KC>
__device__ __forceinline__ void stream_body(const T* X, const int* perm, const T* Wp, void* out, int e,
                                            int row_base, int rows, int K, int N, int nb, T* lds) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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
  constexpr int SS = PD > 2 * KC ? PD : 2 * KC;
  constexpr int CPS = SS / KC;              // chunks per super step (even)
  static_assert(SS % PD == 0 && SS % KC == 0 && CPS % 2 == 0, "ring and chunk sizes are powers of two");
  constexpr bool PIN = KC > 2;              // keep the issue order of the loads as written

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
  const int KS = K / 32, NSS = KS / SS;
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
  u32x4 st[2][PPT];
  auto stage_load = [&](int set, int c) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PPT; ++j) st[set][j] = *reinterpret_cast<const u32x4*>(aptr[j] + (size_t)c * EPR);
  };
  auto stage_store = [&](int set, int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < PPT; ++j)
      if (pok[j]) *reinterpret_cast<u32x4*>(lds + buf * STAGE + (r0 + j * RSTEP) * LROW + seg * VEC) = st[set][j];
  };

  constexpr int blk = NF * 512;             // elements per (block, K step)
  const T* bp = Wp + (size_t)e * NF * N * K + (size_t)nb * KS * blk + lane * 8;
  f32x4_t acc[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  Frag<T> b[PD][NF];
  auto load_b = [&](int slot, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NF; ++j) frag_ld(b[slot][j], bp + (size_t)ks * blk + j * 512);
  };
  // K step kk of the chunk in LDS stage abuf, weights from ring slot `slot`
  auto comp = [&](int slot, int abuf, int kk) __attribute__((always_inline)) {
    Frag<T> a[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      lds_frag(a[rb], lds + abuf * STAGE + (rb * 16 + c16) * LROW + kk * 32 + g4 * 8);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int j = 0; j < NF; ++j) mma16x16x32(acc[rb][j], a[rb], b[slot][j]);
  };
  // K step u of super step g; the last super step stages and prefetches
  // nothing past the end
  auto kstep = [&](int g, auto last, auto uc) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(last)::value;
    constexpr int u = decltype(uc)::value;
    constexpr int cl = u / KC;                // chunk within the super step; its parity is the chunk's
    if constexpr (u % KC == 0 && (!LAST || cl + 2 < CPS)) stage_load(cl & 1, g * CPS + cl + 2);
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
    comp(u % PD, cl & 1, u % KC);
    if constexpr (!LAST || u + PD < SS) load_b(u % PD, g * SS + u + PD);
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
    if constexpr (u % KC == KC - 1) {
      if constexpr (!LAST || cl + 1 < CPS) stage_store((cl + 1) & 1, (cl + 1) & 1);
      lds_barrier();
    }
  };
  auto superstep = [&](int g, auto last) __attribute__((always_inline)) {
    static_for(std::make_integer_sequence<int, SS>{}, [&](auto uc) __attribute__((always_inline)) { kstep(g, last, uc); });
  };
#pragma unroll
  for (int s = 0; s < PD; ++s) load_b(s, s);
  stage_load(0, 0);
  stage_load(1, 1);
  stage_store(0, 0);
  lds_barrier();
  int g = 0;
  for (; g + 1 < NSS; ++g) superstep(g, std::false_type{});
  superstep(g, std::true_type{});

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
        Num<T>::store(static_cast<T*>(out) + (size_t)(row_base + r) * N + col, swiglu(g, u));
      } else {
        static_cast<float*>(out)[(size_t)(row_base + r) * N + col] = acc[rb][0][i];
      }
    }
}

// Grid: x = N / (16 * NW) feature-block groups (exact), y = tile capacity
// (tiles past n_tiles exit; the exit is uniform over the workgroup, so every
// wave reaches the same barriers).
template <typename T, bool GATEUP, int NW, int PD, int KC>
__global__ __launch_bounds__(64 * NW, 2) void k_expert_stream(const T* X, const int* perm, const T* Wp, void* out,
                                                              const int4* tiles, const int* n_tiles, int K, int N) {
  __shared__ __attribute__((aligned(16))) T lds[2 * 64 * (KC * 32 + 16 / sizeof(T))];
  const int ti = blockIdx.y;
  if (ti >= *n_tiles) return;
  const int4 td = tiles[ti];
  const int nb = blockIdx.x * NW + (int)(threadIdx.x >> 6);
  switch ((td.z + 15) >> 4) {
    case 1: stream_body<T, GATEUP, 1, NW, PD, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 2: stream_body<T, GATEUP, 2, NW, PD, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 3: stream_body<T, GATEUP, 3, NW, PD, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
    default: stream_body<T, GATEUP, 4, NW, PD, KC>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb, lds); break;
  }
}

}  // namespace

// K steps per super step of a configuration
template <typename C>
constexpr int stream_ss() {
  return C::PD > 2 * C::KC ? C::PD : 2 * C::KC;
}

bool expert_stream_ok(int d, int F, int elem_bytes) {
  const int ssg = elem_bytes == 2 ? stream_ss<StreamCfg<bf16, true>>() : stream_ss<StreamCfg<float, true>>();
  const int ssd = elem_bytes == 2 ? stream_ss<StreamCfg<bf16, false>>() : stream_ss<StreamCfg<float, false>>();
  // whole super steps along K, whole workgroups of feature blocks along N
  return d % (32 * ssg) == 0 && F % (32 * ssd) == 0 && F % (16 * kStreamWaves) == 0 && d % (16 * kStreamWaves) == 0;
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
  using C = StreamCfg<T, true>;
  hipLaunchKernelGGL((k_expert_stream<T, true, NW, C::PD, C::KC>), dim3(F / (16 * NW), cap_tiles),
                     dim3(64 * NW), 0, s, X, perm, pgu, (void*)act, tiles, n_tiles, d, F);
  return hipGetLastError();
}

template <typename T>
hipError_t expert_stream_down(const T* act, const T* pd, float* Y, const int4* tiles, const int* n_tiles,
                              int cap_tiles, int d, int F, hipStream_t s) {
  constexpr int NW = kStreamWaves;
  using C = StreamCfg<T, false>;
  hipLaunchKernelGGL((k_expert_stream<T, false, NW, C::PD, C::KC>), dim3(d / (16 * NW), cap_tiles),
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

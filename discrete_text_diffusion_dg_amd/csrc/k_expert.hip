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
//
// FP8 experts (OCP E4M3, one fp32 scale per output channel): the packed
// blocks hold two 32-wide K steps per lane in the same 16 bytes
// (P8[N/16][K/64][64 lanes][8 + 8 codes]), so a weight step streams the same
// 1 KB per fragment set as bf16 for twice the K range; each half is widened to
// a bf16 fragment in registers (exact) and multiplied on the bf16 MFMA, and the
// channel scale multiplies the fp32 sum in the epilogue.  At these row counts
// the products are weight reads, so halving the bytes is what counts; the
// activations stay bf16.
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
// FP8: a weight step covers two 32-wide K steps; 8 steps (16 KB per wave) in
// flight for gate/up, 4 for down; chunks of two weight steps keep the LDS
// stage at 128 activation columns
template <> struct StreamCfg<fp8e4m3, true> { static constexpr int PD = 8, KC = 2; };
template <> struct StreamCfg<fp8e4m3, false> { static constexpr int PD = 4, KC = 2; };
// Waves (16-feature blocks) per workgroup: 4 for gate/up; 8 for the bf16 and
// fp32 down products, whose short K range (F) leaves a 4-wave workgroup too
// little streaming to cover its fixed cost (proxy: 0.80 -> 0.78 ms per
// step); FP8 down weights stream half the bytes per step and keep 4 (8 was
// 0.72 -> 0.73 ms).
constexpr int kStreamWaves = 4;
template <typename WT> constexpr int kStreamDownWaves = std::is_same<WT, fp8e4m3>::value ? 4 : 8;

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

// ---- FP8 quantisation (OCP E4M3, per output channel)
// Scales of rows r of a [rows][K] source: fl32(fl64(max |w_row|) / 448), 1 for
// a zero row; written to dst[(r / rpg) * gstride + goff + r % rpg].  One wave per row.
__global__ __launch_bounds__(256) void k_row_scales(const bf16* w, int K, size_t rows, int rpg, int gstride, int goff,
                                                    float* dst) {
  const size_t r = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (r >= rows) return;
  const bf16* row = w + r * K;
  float m = 0.f;
  for (int k = lane * 8; k < K; k += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(x[j] << 16)), fabsf(__uint_as_float(x[j] & 0xFFFF0000u))));
  }
  m = wave_max(m);
  if (lane == 0) {
    const float sc = m > 0.f ? (float)((double)m / 448.0) : 1.f;
    dst[(r / rpg) * gstride + goff + r % rpg] = sc;
  }
}

// 16 codes of one lane: W[n][k0 .. k0 + 8) then W[n][k0 + 32 .. k0 + 40), each w / scale (fp32) -> E4M3
__device__ __forceinline__ uint4 quant16(const bf16* src, int k0, float sc) {
  uint32_t out[4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const uint4 v = *reinterpret_cast<const uint4*>(src + k0 + h * 32);
    const uint32_t x[4] = {v.x, v.y, v.z, v.w};
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t c0 = f32_to_e4m3(__fdiv_rn(__uint_as_float(x[j] << 16), sc));
      const uint32_t c1 = f32_to_e4m3(__fdiv_rn(__uint_as_float(x[j] & 0xFFFF0000u), sc));
      const uint32_t pair = c0 | (c1 << 8);
      if (j < 2) lo |= pair << (16 * j); else hi |= pair << (16 * (j - 2));
    }
    out[2 * h] = lo;
    out[2 * h + 1] = hi;
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Gate/up of expert e: P8GU[e][F/16][d/64][2][64][16 B] from gate/up [e][F][d]; scales [e][2][F].
__global__ void k_pack_gateup_fp8(const bf16* gate, const bf16* up, const float* sgu, uint4* out, int F, int d) {
  const size_t per_e = (size_t)F * d;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;    // one 16-byte lane piece per thread
  const int e = blockIdx.y;
  if (i >= 2 * per_e / 16) return;
  const int lane = (int)(i % 64);
  size_t rest = i / 64;
  const int which = (int)(rest % 2); rest /= 2;
  const int ks = (int)(rest % (d / 64));
  const int fb = (int)(rest / (d / 64));
  const int f = fb * 16 + (lane & 15), k0 = ks * 64 + (lane >> 4) * 8;
  const bf16* src = (which ? up : gate) + (size_t)e * per_e + (size_t)f * d;
  out[(size_t)e * (2 * per_e / 16) + i] = quant16(src, k0, sgu[((size_t)e * 2 + which) * F + f]);
}

// Down of expert e: P8D[e][d/16][F/64][64][16 B] from down [e][d][F]; scales [e][d].
__global__ void k_pack_down_fp8(const bf16* down, const float* sd, uint4* out, int d, int F) {
  const size_t per_e = (size_t)d * F;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int e = blockIdx.y;
  if (i >= per_e / 16) return;
  const int lane = (int)(i % 64);
  const size_t rest = i / 64;
  const int ks = (int)(rest % (F / 64));
  const int nb = (int)(rest / (F / 64));
  const int n = nb * 16 + (lane & 15), k0 = ks * 64 + (lane >> 4) * 8;
  out[(size_t)e * (per_e / 16) + i] = quant16(down + (size_t)e * per_e + (size_t)n * F, k0, sd[(size_t)e * d + n]);
}

// ---- streaming products
template <int... U, class F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, U...>, F&& f) {
  (f(std::integral_constant<int, U>{}), ...);
}

// Weight fragment of one weight step as loaded (16 bytes per lane for bf16 and
// FP8, 32 for fp32) and its bf16 / fp32 MFMA fragments.
template <typename WT> struct WFrag { Frag<WT> f; };
template <> struct WFrag<fp8e4m3> { uint4 v; };
template <typename WT> struct SubSteps { static constexpr int value = 1; };
template <> struct SubSteps<fp8e4m3> { static constexpr int value = 2; };
template <typename WT> struct Operand { using type = WT; };
template <> struct Operand<fp8e4m3> { using type = bf16; };

template <typename WT>
__device__ __forceinline__ void wfrag_ld(WFrag<WT>& f, const char* p) {
  if constexpr (std::is_same<WT, fp8e4m3>::value) f.v = *reinterpret_cast<const uint4*>(p);
  else frag_ld(f.f, reinterpret_cast<const WT*>(p));
}
// sub-step h of the fragment as an MFMA B operand
template <typename WT>
__device__ __forceinline__ Frag<typename Operand<WT>::type> wfrag_sub(const WFrag<WT>& f, int h) {
  if constexpr (std::is_same<WT, fp8e4m3>::value) {
    Frag<bf16> o;
    o.v = h == 0 ? fp8x8_to_bf16x8(f.v.x, f.v.y) : fp8x8_to_bf16x8(f.v.z, f.v.w);
    return o;
  } else {
    return f.f;
  }
}

// GATEUP: out = act [rows][F] (T), B = PGU, A rows gathered through perm.
// else:   out = Y   [rows][d] (fp32), B = PD, A rows row_base + r of act.
// WT: weight storage (T, or FP8 with per-channel scales: scale[e][NF][N]).
// LDS: two stages of [64 rows][KC*SUB*32 + pad] elements; a stage holds weight
// steps [c*KC, (c+1)*KC) of the tile's rows (SUB 32-wide K steps each).  The K
// loop runs in super steps of SS weight steps (an even number of chunks, a
// multiple of the ring depth), unrolled so that every ring slot and staging
// set is a compile-time index.
template <typename T, typename WT, bool GATEUP, int RB, int NW, int PD, int KC>
__device__ __forceinline__ void stream_body(const T* X, const int* perm, const WT* Wp, const float* scale, void* out,
                                            int e, int row_base, int rows, int K, int N, int nb, T* lds) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  constexpr int SUB = SubSteps<WT>::value;  // 32-wide K steps per weight step
  constexpr int EPR = KC * SUB * 32;        // elements of a row per chunk
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
  constexpr bool PIN = KC > 2 || SUB > 1;   // keep the issue order of the loads as written
  constexpr int LANE_BYTES = 8 * SUB * (int)sizeof(WT);   // one lane's share of a fragment set
  constexpr int BLK = NF * 64 * LANE_BYTES;               // bytes per (block, weight step)

  const int tid = threadIdx.x, lane = tid & 63, g4 = lane >> 4, c16 = lane & 15;
  const int KS = K / (32 * SUB), NSS = KS / SS;
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

  const char* bp = reinterpret_cast<const char*>(Wp) + (size_t)e * NF * N * K * sizeof(WT) +
                   (size_t)nb * KS * BLK + lane * LANE_BYTES;
  f32x4_t acc[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  WFrag<WT> b[PD][NF];
  auto load_b = [&](int slot, int ks) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NF; ++j) wfrag_ld(b[slot][j], bp + (size_t)ks * BLK + j * 64 * LANE_BYTES);
  };
  // weight step kk of the chunk in LDS stage abuf, weights from ring slot `slot`
  auto comp = [&](int slot, int abuf, int kk) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < SUB; ++h) {
      Frag<T> a[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
        lds_frag(a[rb], lds + abuf * STAGE + (rb * 16 + c16) * LROW + (kk * SUB + h) * 32 + g4 * 8);
#pragma unroll
      for (int j = 0; j < NF; ++j) {
        const auto bf = wfrag_sub(b[slot][j], h);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) mma16x16x32(acc[rb][j], a[rb], bf);
      }
    }
  };
  // weight step u of super step g; the last super step stages and prefetches
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

  // epilogue: the lane holds rows rb*16 + g4*4 + i, column c16 of the block;
  // FP8 weights: the channel scales multiply the sums
  const int col = nb * 16 + c16;
  float sc[NF];
#pragma unroll
  for (int j = 0; j < NF; ++j)
    sc[j] = std::is_same<WT, fp8e4m3>::value ? scale[((size_t)e * NF + j) * N + col] : 1.f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + g4 * 4 + i;
      if (r >= rows) continue;
      if (GATEUP) {
        float g = acc[rb][0][i], u = acc[rb][1][i];
        if constexpr (std::is_same<WT, fp8e4m3>::value) { g *= sc[0]; u *= sc[NF - 1]; }
        Num<T>::store(static_cast<T*>(out) + (size_t)(row_base + r) * N + col, swiglu(g, u));
      } else {
        float y = acc[rb][0][i];
        if constexpr (std::is_same<WT, fp8e4m3>::value) y *= sc[0];
        Num<T>::store(static_cast<T*>(out) + (size_t)(row_base + r) * N + col, y);
      }
    }
}

// Grid: groups = N / (16 * NW) feature-block groups (exact) times the tile
// capacity, one dimension.  The first groups * n_tiles workgroups take
// (tile, group) pairs, tile-major, in contiguous runs per XCD: the groups of a
// tile and the neighbouring tiles (an expert's row tiles are adjacent in the
// list) run together on one XCD, so an expert's weight slices streamed for
// several row tiles are fetched from HBM once into that XCD's L2.  The rest
// exit (uniformly over the workgroup, so every wave reaches the same barriers).
template <typename T, typename WT, bool GATEUP, int NW, int PD, int KC>
__global__ __launch_bounds__(64 * NW, 2) void k_expert_stream(const T* X, const int* perm, const WT* Wp,
                                                              const float* scale, void* out, const int4* tiles,
                                                              const int* n_tiles, int K, int N) {
  __shared__ __attribute__((aligned(16))) T lds[2 * 64 * (KC * SubSteps<WT>::value * 32 + 16 / sizeof(T))];
  const int groups = N / (16 * NW), total = groups * *n_tiles;
  if ((int)blockIdx.x >= total) return;
  const int lg = xcd_run(blockIdx.x, total), ti = lg / groups;
  const int4 td = tiles[ti];
  const int nb = (lg % groups) * NW + (int)(threadIdx.x >> 6);
  switch ((td.z + 15) >> 4) {
    case 1: stream_body<T, WT, GATEUP, 1, NW, PD, KC>(X, perm, Wp, scale, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 2: stream_body<T, WT, GATEUP, 2, NW, PD, KC>(X, perm, Wp, scale, out, td.x, td.y, td.z, K, N, nb, lds); break;
    case 3: stream_body<T, WT, GATEUP, 3, NW, PD, KC>(X, perm, Wp, scale, out, td.x, td.y, td.z, K, N, nb, lds); break;
    default: stream_body<T, WT, GATEUP, 4, NW, PD, KC>(X, perm, Wp, scale, out, td.x, td.y, td.z, K, N, nb, lds); break;
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
  return d % (32 * ssg) == 0 && F % (32 * ssd) == 0 && F % (16 * kStreamWaves) == 0 && d % (16 * kStreamDownWaves<bf16>) == 0;
}

bool expert_stream_fp8_ok(int d, int F) {
  const int ssg = stream_ss<StreamCfg<fp8e4m3, true>>(), ssd = stream_ss<StreamCfg<fp8e4m3, false>>();
  return d % (64 * ssg) == 0 && F % (64 * ssd) == 0 && F % (16 * kStreamWaves) == 0 && d % (16 * kStreamDownWaves<fp8e4m3>) == 0;
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

hipError_t pack_expert_weights_fp8(const bf16* gate, const bf16* up, const bf16* down, fp8e4m3* pgu, fp8e4m3* pd,
                                   float* sgu, float* sd, int E, int d, int F, hipStream_t s) {
  const size_t rows_gu = (size_t)E * F, rows_d = (size_t)E * d;
  hipLaunchKernelGGL(k_row_scales, dim3((unsigned)((rows_gu + 3) / 4)), dim3(256), 0, s, gate, d, rows_gu, F, 2 * F, 0,
                     sgu);
  hipLaunchKernelGGL(k_row_scales, dim3((unsigned)((rows_gu + 3) / 4)), dim3(256), 0, s, up, d, rows_gu, F, 2 * F, F,
                     sgu);
  hipLaunchKernelGGL(k_row_scales, dim3((unsigned)((rows_d + 3) / 4)), dim3(256), 0, s, down, F, rows_d, d, d, 0, sd);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t pieces_gu = 2 * (size_t)F * d / 16, pieces_d = (size_t)d * F / 16;
  hipLaunchKernelGGL(k_pack_gateup_fp8, dim3((unsigned)((pieces_gu + 255) / 256), E), dim3(256), 0, s, gate, up, sgu,
                     reinterpret_cast<uint4*>(pgu), F, d);
  hipLaunchKernelGGL(k_pack_down_fp8, dim3((unsigned)((pieces_d + 255) / 256), E), dim3(256), 0, s, down, sd,
                     reinterpret_cast<uint4*>(pd), d, F);
  return hipGetLastError();
}

hipError_t pack_head_fp8(const bf16* w, fp8e4m3* codes, float* scales, int V, int K, hipStream_t s) {
  if (V % 16 || K % 64) return hipErrorInvalidValue;
  // the down projection's P8 order with one "expert": rows V, K elements per row K
  hipLaunchKernelGGL(k_row_scales, dim3((unsigned)((V + 3) / 4)), dim3(256), 0, s, w, K, (size_t)V, V, 0, 0, scales);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t pieces = (size_t)V * K / 16;
  hipLaunchKernelGGL(k_pack_down_fp8, dim3((unsigned)((pieces + 255) / 256), 1), dim3(256), 0, s, w, scales,
                     reinterpret_cast<uint4*>(codes), V, K);
  return hipGetLastError();
}

template <typename T, typename WT>
hipError_t expert_stream_gateup(const T* X, const int* perm, const WT* pgu, const float* scale, T* act,
                                const int4* tiles, const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s) {
  constexpr int NW = kStreamWaves;
  using C = StreamCfg<WT, true>;
  hipLaunchKernelGGL((k_expert_stream<T, WT, true, NW, C::PD, C::KC>), dim3(F / (16 * NW) * cap_tiles),
                     dim3(64 * NW), 0, s, X, perm, pgu, scale, (void*)act, tiles, n_tiles, d, F);
  return hipGetLastError();
}

template <typename T, typename WT>
hipError_t expert_stream_down(const T* act, const WT* pd, const float* scale, T* Y, const int4* tiles,
                              const int* n_tiles, int cap_tiles, int d, int F, hipStream_t s) {
  constexpr int NW = kStreamDownWaves<WT>;
  using C = StreamCfg<WT, false>;
  hipLaunchKernelGGL((k_expert_stream<T, WT, false, NW, C::PD, C::KC>), dim3(d / (16 * NW) * cap_tiles),
                     dim3(64 * NW), 0, s, act, (const int*)nullptr, pd, scale, (void*)Y, tiles, n_tiles, F, d);
  return hipGetLastError();
}

#define DG_INST(T, WT)                                                                                            \
  template hipError_t expert_stream_gateup<T, WT>(const T*, const int*, const WT*, const float*, T*, const int4*,  \
                                                  const int*, int, int, int, hipStream_t);                      \
  template hipError_t expert_stream_down<T, WT>(const T*, const WT*, const float*, T*, const int4*, const int*,     \
                                                int, int, int, hipStream_t);
DG_INST(float, float)
DG_INST(bf16, bf16)
DG_INST(bf16, fp8e4m3)
#undef DG_INST
template hipError_t pack_expert_weights<float>(const float*, const float*, const float*, float*, float*, int, int,
                                               int, hipStream_t);
template hipError_t pack_expert_weights<bf16>(const bf16*, const bf16*, const bf16*, bf16*, bf16*, int, int, int,
                                              hipStream_t);

}  // namespace dg

// Expert SwiGLU products for thin routed tiles (at most 64 rows, the batch-1
// shapes): weight streaming from a fragment-packed layout, no LDS tiles.
//
// Packed layout (built once by dg_model_create): a weight matrix W[N][K] of
// one expert is stored as blocks P[N/16][K/32][64 lanes][8 elements], where
// lane (c, g) of block (nb, ks) holds W[nb*16 + c][ks*32 + g*8 .. +8] -- exactly
// the MFMA B-operand fragment of that lane.  A wave's fragment load is then one
// contiguous 1 KB (bf16) read, so the weights stream at plain-copy efficiency.
// Gate and up of the same 16 features are interleaved per K step
// (PGU[F/16][d/32][2][64][8]) so silu(g) * u is formed lane-locally.
//
// A wave owns FB feature blocks (of 16 outputs), all row blocks of the tile and
// 1/KW of the K range (KW > 1: the waves of a block group add their partial
// sums through LDS once, at the end); the tile's activation rows are read with
// plain row loads (small, shared through the caches).  K steps are processed in groups of U; the loads of the
// next group are issued before the MFMAs of the current one.  The number of
// row blocks (1..4) is a template parameter chosen per tile at run time, so
// every load of a path is unconditional and the memory-wait counts stay exact.
#include "dg_kernels.h"

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
template <typename T>
__device__ __forceinline__ void frag_keep(Frag<T>& f, bool keep);
template <>
__device__ __forceinline__ void frag_keep(Frag<bf16>& f, bool keep) {
  if (!keep) f.v = make_uint4(0, 0, 0, 0);
}
template <>
__device__ __forceinline__ void frag_keep(Frag<float>& f, bool keep) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = keep ? f.v[j] : 0.f;
}

template <typename T> struct StreamCfg;
template <> struct StreamCfg<bf16> { static constexpr int U = 2; };
template <> struct StreamCfg<float> { static constexpr int U = 1; };
// Blocking of the two products: FB output blocks (of 16) per wave, and KW waves
// of a workgroup splitting the K range of the same blocks (4 / KW block groups
// per 4-wave workgroup).  These products are bound by the weight loads each CU
// keeps in flight; every wave also re-reads its tile's activation rows, so the
// split pays only where it adds streaming waves without multiplying those
// re-reads: measured on skewed routings (9..31 of 32 experts active), the
// down product gains 20-28% from a 4-way split, gate/up gains nothing.
constexpr int kFbUp = 2, kKwUp = 1;
constexpr int kFbDown = 2, kKwDown = 4;

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
// The wave covers K steps [kb, kb + KSw); with KW > 1 the KW waves of a block
// group add their accumulators through `red` (LDS) and the first one stores.
template <typename T, bool GATEUP, int RB, int FB, int U, int KW>
__device__ __forceinline__ void stream_body(const T* X, const int* perm, const T* Wp, void* out, int e,
                                            int row_base, int rows, int K, int N, int nb0, int wk, float* red) {
  const int lane = threadIdx.x & 63, g4 = lane >> 4, c16 = lane & 15;
  constexpr int NF = GATEUP ? 2 * FB : FB;           // fragments of B per K step
  const int KS = K / 32, KSw = KS / KW, kb = wk * KSw;
  const T* arow[RB];
  bool aval[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * 16 + c16;
    aval[rb] = r < rows;
    const int rr = aval[rb] ? r : 0;
    const int src = GATEUP ? perm[row_base + rr] : row_base + rr;
    arow[rb] = X + (size_t)src * K + kb * 32 + g4 * 8;
  }
  // per block: base pointer of its packed column of K steps
  constexpr int blk = (GATEUP ? 2 : 1) * 512;   // elements per (block, K step)
  const T* bp[FB];
  bool bval[FB];
#pragma unroll
  for (int f = 0; f < FB; ++f) {
    const int nb = nb0 + f;
    bval[f] = nb * 16 < N;
    const int nbc = bval[f] ? nb : 0;
    bp[f] = Wp + (size_t)e * (GATEUP ? 2 : 1) * N * K + ((size_t)nbc * KS + kb) * blk + lane * 8;
  }
  f32x4_t acc[RB][NF];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int j = 0; j < NF; ++j) acc[rb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  Frag<T> a[2][U][RB], b[2][U][NF];
  auto load = [&](int buf, int ks0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = ks0 + u;
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        if (GATEUP) {
          frag_ld(b[buf][u][2 * f], bp[f] + (size_t)ks * blk);
          frag_ld(b[buf][u][2 * f + 1], bp[f] + (size_t)ks * blk + 512);
        } else {
          frag_ld(b[buf][u][f], bp[f] + (size_t)ks * blk);
        }
      }
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) frag_ld(a[buf][u][rb], arow[rb] + ks * 32);
    }
  };
  auto comp = [&](int buf) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) frag_keep(a[buf][u][rb], aval[rb]);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NF; ++j) mma16x16x32(acc[rb][j], a[buf][u][rb], b[buf][u][j]);
    }
  };
  // KSw is a multiple of U; groups of U steps, double-buffered
  load(0, 0);
  int ks0 = 0;
  for (; ks0 + U < KSw; ks0 += 2 * U) {
    load(1, ks0 + U);
    comp(0);
    if (ks0 + 2 * U < KSw) load(0, ks0 + 2 * U);
    comp(1);
  }
  if (ks0 < KSw) comp(0);

  if constexpr (KW > 1) {
    // lane-major slots: entry j of wave wk lives at red[((wk - 1) * NA + j) * 64 + lane]
    constexpr int NA = RB * NF * 4;
    if (wk > 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) red[((wk - 1) * NA + (rb * NF + j) * 4 + i) * 64 + lane] = acc[rb][j][i];
    }
    __syncthreads();
    if (wk > 0) return;
#pragma unroll
    for (int v = 1; v < KW; ++v)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int j = 0; j < NF; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[rb][j][i] += red[((v - 1) * NA + (rb * NF + j) * 4 + i) * 64 + lane];
  }

  // epilogue: the lane holds rows rb*16 + g4*4 + i, column c16 of each block
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = rb * 16 + g4 * 4 + i;
      if (r >= rows) continue;
#pragma unroll
      for (int f = 0; f < FB; ++f) {
        if (!bval[f]) continue;
        const int col = (nb0 + f) * 16 + c16;
        if (GATEUP) {
          const float g = acc[rb][2 * f][i], u = acc[rb][2 * f + 1][i];
          Num<T>::store(static_cast<T*>(out) + (size_t)(row_base + r) * N + col, g / (1.0f + expf(-g)) * u);
        } else {
          static_cast<float*>(out)[(size_t)(row_base + r) * N + col] = acc[rb][f][i];
        }
      }
    }
}

// Grid: x = N / (16 * FB * 4 / KW) block groups (exact, so every exit below is
// uniform over the workgroup and all of its waves reach the reduction barrier),
// y = tile capacity (tiles past n_tiles exit).
template <typename T, bool GATEUP, int FB, int KW, int U>
__global__ __launch_bounds__(256) void k_expert_stream(const T* X, const int* perm, const T* Wp, void* out,
                                                       const int4* tiles, const int* n_tiles, int K, int N) {
  constexpr int NF = GATEUP ? 2 * FB : FB;
  constexpr int GW = 4 / KW;                          // block groups per workgroup
  __shared__ float red[KW > 1 ? GW * (KW - 1) * 4 * NF * 4 * 64 : 1];
  const int ti = blockIdx.y;
  if (ti >= *n_tiles) return;
  const int4 td = tiles[ti];
  const int w = threadIdx.x >> 6, wf = w / KW, wk = w % KW;
  const int nb0 = (blockIdx.x * GW + wf) * FB;
  float* r = red + (KW > 1 ? wf * (KW - 1) * 4 * NF * 4 * 64 : 0);
  switch ((td.z + 15) >> 4) {
    case 1: stream_body<T, GATEUP, 1, FB, U, KW>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb0, wk, r); break;
    case 2: stream_body<T, GATEUP, 2, FB, U, KW>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb0, wk, r); break;
    case 3: stream_body<T, GATEUP, 3, FB, U, KW>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb0, wk, r); break;
    default: stream_body<T, GATEUP, 4, FB, U, KW>(X, perm, Wp, out, td.x, td.y, td.z, K, N, nb0, wk, r); break;
  }
}

}  // namespace

bool expert_stream_ok(int d, int F, int elem_bytes) {
  const int U = elem_bytes == 2 ? StreamCfg<bf16>::U : StreamCfg<float>::U;
  // K steps split evenly over the waves in groups of U; whole block groups along N
  return d % (32 * U * kKwUp) == 0 && F % (32 * U * kKwDown) == 0 && F % (16 * kFbUp * 4 / kKwUp) == 0 &&
         d % (16 * kFbDown * 4 / kKwDown) == 0;
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
  const int per_wg = 16 * kFbUp * 4 / kKwUp;
  dim3 grid(F / per_wg, cap_tiles);
  hipLaunchKernelGGL((k_expert_stream<T, true, kFbUp, kKwUp, StreamCfg<T>::U>), grid, dim3(256), 0, s, X, perm, pgu, (void*)act, tiles,
                     n_tiles, d, F);
  return hipGetLastError();
}

template <typename T>
hipError_t expert_stream_down(const T* act, const T* pd, float* Y, const int4* tiles, const int* n_tiles,
                              int cap_tiles, int d, int F, hipStream_t s) {
  const int per_wg = 16 * kFbDown * 4 / kKwDown;
  dim3 grid(d / per_wg, cap_tiles);
  hipLaunchKernelGGL((k_expert_stream<T, false, kFbDown, kKwDown, StreamCfg<T>::U>), grid, dim3(256), 0, s, act, (const int*)nullptr, pd,
                     (void*)Y, tiles, n_tiles, F, d);
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

// Row-wise kernels of the denoise step.  Each reduces, in a fixed split order,
// the fp32 partials of the split-K product before it and fuses the next
// element-wise step: embedding gather (+ self-conditioning projection) with
// the first RMSNorm, the attention output residual with the MoE RMSNorm, the
// expert combine with the next layer's (or the final) RMSNorm, RoPE with the
// KV-cache write, and the router logits with top-k (lowest expert id on
// ties) and the softmax over the k selected logits.  Routed rows are bucketed
// per expert by a stable counting sort; canvas initialisation draws Philox.
#include "dg_kernels.h"

namespace dg {

namespace {
// One workgroup per row, TPR = min(256, d / 4) threads, each owning up to
// kRowChunks float4 chunks of the row (d <= kMaxModel).
constexpr int kRowChunks = kMaxModel / 1024;

inline int row_threads(int d) { return d / 4 < 256 ? d / 4 : 256; }

__device__ __forceinline__ void add4(float4& a, const float4 b) {
  a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
}

// Four consecutive values of an fp32 or bf16 array (4-element aligned) as fp32.
__device__ __forceinline__ float4 load4f(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4f(const bf16* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                     __uint_as_float(u.y & 0xFFFF0000u));
}

// Sum over the S split partials of one float4 (part + s * stride + off), in
// split order; the loads of up to 8 splits are issued together (indices past S
// re-read the last split and are not added).
__device__ __forceinline__ float4 sum_splits4(const float* part, int S, size_t stride, size_t off) {
  float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const float4*>(part + (size_t)min(s0 + u, S - 1) * stride + off);
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) add4(p, v[u]);
  }
  return p;
}
__device__ __forceinline__ float sum_splits1(const float* part, int S, size_t stride, size_t off) {
  float p = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = part[(size_t)min(s0 + u, S - 1) * stride + off];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < S) p += v[u];
  }
  return p;
}

// Four consecutive values in one store (8 bytes bf16, 16 bytes fp32).
__device__ __forceinline__ void store_row4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(f32x2_to_bf16x2(a, b), f32x2_to_bf16x2(c, d));
}
__device__ __forceinline__ void store_row4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
// Stores the updated residual row v and y = rnd(v * g / sqrt(mean(v^2) + eps)).
template <typename T>
__device__ __forceinline__ void norm_store(float4 (&v)[kRowChunks], int nj, int d, const float* g, float eps,
                                           float* hrow, T* xrow, float* xs = nullptr) {
  __shared__ float red[8];             // up to 512 threads
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, nw = (blockDim.x + 63) >> 6;
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
  ss = wave_sum(ss);
  if (lane == 0) red[w] = ss;
  __syncthreads();
  ss = red[0];
  for (int q = 1; q < nw; ++q) ss += red[q];
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + tid) * 4;
      *reinterpret_cast<float4*>(hrow + c) = v[j];
      const float4 gg = *reinterpret_cast<const float4*>(g + c);
      store_row4(xrow + c, v[j].x * inv * gg.x, v[j].y * inv * gg.y, v[j].z * inv * gg.z, v[j].w * inv * gg.w);
      if (xs != nullptr)   // the rounded row, as the products downstream see it
        *reinterpret_cast<float4*>(xs + c) =
            make_float4(Num<T>::round(v[j].x * inv * gg.x), Num<T>::round(v[j].y * inv * gg.y),
                        Num<T>::round(v[j].z * inv * gg.z), Num<T>::round(v[j].w * inv * gg.w));
    }
}


}  // namespace

// h = emb[tok] (+ sum_s part[s]); xn = rnd(rmsnorm(h) * g)
template <typename T>
__global__ __launch_bounds__(256) void k_embed_norm(const T* emb, const int32_t* tok, const float* part, int S,
                                                    int M, int d, int vocab, const float* g, float eps, float* H,
                                                    T* xn, Gate gt, int n) {
  const int r = blockIdx.x, nj = d / (4 * blockDim.x);
  if (!gt.active(r / n)) return;
  const int id = min(max(tok[r], 0), vocab - 1);   // out-of-range ids are clamped, never read past E
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + threadIdx.x) * 4;
      const T* e = emb + (size_t)id * d + c;
      float4 x;
      if constexpr (sizeof(T) == 2) {           // four bf16 in one 8-byte load
        const uint2 u = *reinterpret_cast<const uint2*>(e);
        x = make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                        __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
      } else {
        x = *reinterpret_cast<const float4*>(e);
      }
      add4(x, S > 0 ? sum_splits4(part, S, (size_t)M * d, (size_t)r * d + c) : make_float4(0.f, 0.f, 0.f, 0.f));
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

// h += sum_s part[s]; xn = rnd(rmsnorm(h) * g).  NJ = d / (4 * threads)
// chunks per thread; every chunk's partials (up to 8 splits at a time) and h
// are loaded before the first sum, so the row costs one load round trip.
template <typename T, int NJ>
__global__ __launch_bounds__(256) void k_add_norm(const float* part, int S, int M, int d, const float* g, float eps,
                                                  float* H, T* xn, Gate gt, int n) {
  const int r = blockIdx.x;
  if (!gt.active(r / n)) return;
  const size_t stride = (size_t)M * d;
  float4 v[kRowChunks];
  float4 p[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) p[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += 8) {
    float4 pv[NJ][8];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        pv[j][u] = *reinterpret_cast<const float4*>(part + (size_t)min(s0 + u, S - 1) * stride + (size_t)r * d +
                                                    (j * blockDim.x + threadIdx.x) * 4);
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (s0 + u < S) add4(p[j], pv[j][u]);
  }
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float4 x = *reinterpret_cast<const float4*>(H + (size_t)r * d + (j * blockDim.x + threadIdx.x) * 4);
    add4(x, p[j]);
    v[j] = x;
  }
  norm_store<T>(v, NJ, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

// h += sum_j w[j] * Y[pos[j]] (slots in selection order, expert outputs in the
// operand type); xn = rnd(rmsnorm(h) * g).
// Every slot's expert output (slot indices clamped to the k selected, so the
// loads are unconditional) and h are loaded before the first sum: one load
// round trip after the slot indices, where conditional loads went one by one.
template <typename T, int NJ>
__global__ __launch_bounds__(256) void k_combine_norm(const T* Y, const int* pos, const float* w, int k, int M,
                                                      int d, const float* g, float eps, float* H, T* xn, Gate gt,
                                                      int n) {
  const int r = blockIdx.x;
  if (!gt.active(r / n)) return;
  int ps[8];
  float ws[8];
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int sc = min(s, k - 1);
    ps[s] = pos[(size_t)r * k + sc];
    ws[s] = w[(size_t)r * k + sc];
  }
  float4 y[NJ][8], hx[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int c = (j * blockDim.x + threadIdx.x) * 4;
#pragma unroll
    for (int s = 0; s < 8; ++s) y[j][s] = load4f(Y + (size_t)ps[s] * d + c);
    hx[j] = *reinterpret_cast<const float4*>(H + (size_t)r * d + c);
  }
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int s = 0; s < 8; ++s)
      if (s < k) {
        acc.x += ws[s] * y[j][s].x; acc.y += ws[s] * y[j][s].y; acc.z += ws[s] * y[j][s].z; acc.w += ws[s] * y[j][s].w;
      }
    float4 x = hx[j];
    add4(x, acc);
    v[j] = x;
  }
  norm_store<T>(v, NJ, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

// Chunks per thread of a row kernel: d / (4 * row_threads(d)), exactly 1..4
// for the widths the model accepts (256..1024 in steps of 256, then 2048,
// 3072, 4096).
#define DG_ROW_NJ(d, LAUNCH)                    \
  switch ((d) / (4 * row_threads(d))) {         \
    case 1: LAUNCH(1); break;                    \
    case 2: LAUNCH(2); break;                    \
    case 3: LAUNCH(3); break;                    \
    default: LAUNCH(4); break;                   \
  }

template <typename T>
hipError_t embed_norm(const T* emb, const int32_t* tok, const float* part, int S, int M, int d, int vocab,
                      const float* g, float eps, float* H, T* xn, Gate gt, int n, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_embed_norm<T>), dim3(M), dim3(row_threads(d)), 0, s, emb, tok, part, S, M, d, vocab, g, eps,
                     H, xn, gt, n);
  return hipGetLastError();
}
template <typename T>
hipError_t add_norm(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                    Gate gt, int n, hipStream_t s) {
  if (M <= 0) return hipSuccess;
#define DG_L(NJ) \
  hipLaunchKernelGGL((k_add_norm<T, NJ>), dim3(M), dim3(row_threads(d)), 0, s, part, S, M, d, g, eps, H, xn, gt, n)
  DG_ROW_NJ(d, DG_L)
#undef DG_L
  return hipGetLastError();
}
template <typename T>
hipError_t combine_norm(const T* Y, const int* pos, const float* w, int k, int M, int d, const float* g,
                        float eps, float* H, T* xn, Gate gt, int n, hipStream_t s) {
  if (M <= 0) return hipSuccess;
#define DG_L(NJ)                                                                                              \
  hipLaunchKernelGGL((k_combine_norm<T, NJ>), dim3(M), dim3(row_threads(d)), 0, s, Y, pos, w, k, M, d, g, eps, H, \
                     xn, gt, n)
  DG_ROW_NJ(d, DG_L)
#undef DG_L
  return hipGetLastError();
}

// ------------------------------------------------------------------ RoPE
// Table of (cos, sin) of pos * theta^(-2j/hd), evaluated in fp64.
__global__ void k_rope_table(float2* tab, int max_ctx, int hd, double theta) {
  const int half = hd / 2;
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (size_t)max_ctx * half) return;
  const int pos = (int)(i / half), j = (int)(i % half);
  const double freq = pow(theta, -2.0 * (double)j / (double)hd);
  const double ang = (double)pos * freq;
  tab[i] = make_float2((float)cos(ang), (float)sin(ang));
}
hipError_t rope_table(float2* tab, int max_ctx, int hd, float theta, hipStream_t s) {
  const size_t n = (size_t)max_ctx * (hd / 2);
  hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, tab, max_ctx, hd,
                     (double)theta);
  return hipGetLastError();
}

// Sum the split partials of the fused projection, apply rotate-half RoPE to q
// and k (fp32), then round: q to the query buffer, k and v to the cache at
// position ctx + i.
template <typename T>
__global__ void k_rope_scatter(const float* part, int S, const float2* rope, T* q, T* kc, T* vc, int M, int n,
                               int Hq, int Hkv, int hd, int stride, PosArg pa, Gate gt) {
  const int r = blockIdx.x, b = r / n, i = r % n, half = hd / 2;
  if (!gt.active(b)) return;
  const int pos = pa.base(b) + i;
  const int ncol = (Hq + 2 * Hkv) * hd;
  const size_t sstride = (size_t)M * ncol;
  const float* x = part + (size_t)r * ncol;
  const float2* cs = rope + (size_t)pos * half;
  for (int u = threadIdx.x; u < (Hq + Hkv) * half; u += blockDim.x) {
    const int head = u / half, j = u % half;
    const float a = sum_splits1(x, S, sstride, head * hd + j);
    const float bb = sum_splits1(x, S, sstride, head * hd + j + half);
    const float2 t = cs[j];
    const float o1 = a * t.x - bb * t.y, o2 = bb * t.x + a * t.y;
    if (head < Hq) {
      T* dst = q + (size_t)r * Hq * hd + head * hd;
      Num<T>::store(dst + j, o1);
      Num<T>::store(dst + j + half, o2);
    } else {
      const int kh = head - Hq;
      T* dst = kc + (((size_t)b * Hkv + kh) * stride + pos) * hd;
      Num<T>::store(dst + j, o1);
      Num<T>::store(dst + j + half, o2);
    }
  }
  for (int u = threadIdx.x; u < Hkv * hd; u += blockDim.x) {
    const int kh = u / hd, c = u % hd;
    const float v = sum_splits1(x, S, sstride, (Hq + Hkv) * hd + u);
    Num<T>::store(vc + (((size_t)b * Hkv + kh) * hd + c) * stride + pos, v);   // V^T
  }
}
template <typename T>
hipError_t rope_scatter(const float* part, int S, const float2* rope, T* q, T* kc, T* vc, int B, int n, int Hq,
                        int Hkv, int hd, int stride, PosArg pa, Gate gt, hipStream_t s) {
  if (B * n <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_rope_scatter<T>), dim3(B * n), dim3(256), 0, s, part, S, rope, q, kc, vc, B * n, n, Hq,
                     Hkv, hd, stride, pa, gt);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router
// Three launches per layer, no atomics.
//  k_router_logits: a workgroup owns 16 rows x 16 experts x one K split; its
//    waves split that K range, add their MFMA partial sums through LDS in wave
//    order and store fp32 partial logits.  Spreading the router matrix over
//    rows x expert blocks x K splits keeps every workgroup's reads small (one
//    workgroup per 16 rows would stream the whole matrix per CU).
//  k_router_select: a workgroup owns RPB rows --
//    1. their logits, the K-split partials added in split order;
//    2. per row, the top k logits -- ties going to the lower expert id -- by
//       rank counting (E <= 32) or by bisection on unique keys (larger E),
//       then softmax over the selected;
//    3. per expert, the count of the block's (row, slot) entries -> cnt[e][blk],
//       and per entry its rank among the block's entries of that expert, in
//       (row, slot) order -> pos.
//  k_route_finish turns the count table into per-block exclusive prefixes
//    (per expert, in place), the expert totals into offsets, writes the tile
//    list (runs of at most tile_rows rows of one expert), and the final
//    position of every
//    entry in the expert-sorted order, offset + block prefix + rank, into pos
//    and perm: rows of an expert stay in ascending row order.
template <typename T>
__device__ __forceinline__ void router_frag(Frag<T>& f, const T* p);
template <>
__device__ __forceinline__ void router_frag(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
template <>
__device__ __forceinline__ void router_frag(Frag<float>& f, const float* p) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// Top k of one row (E <= 128 logits in LDS) by one wave: keys (order-preserving
// bits of the logit, then 127 - expert) are unique, so k rounds of a wave-wide
// maximum pick the slots in order -- largest logit first, ties to the lower
// expert id.  A lane holds experts lane and lane + 64.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 7) | (uint64_t)(127 - e);
}
// Wave-wide maximum of a 64-bit key, in every lane: DPP lane moves within
// rows of 16 (pairs, quads, half rows, rows) and the gfx950 row swaps across
// rows and halves -- plain VALU moves, where shuffles go through the LDS
// crossbar.
template <int CTRL>
__device__ __forceinline__ uint64_t max_dpp_u64(uint64_t m) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)m, CTRL, 0xF, 0xF, false);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(m >> 32), CTRL, 0xF, 0xF, false);
  const uint64_t x = ((uint64_t)hi << 32) | lo;
  return x > m ? x : m;
}
__device__ __forceinline__ uint64_t max_swap_u64(uint64_t m, bool rows32) {
  const uint32_t lo = (uint32_t)m, hi = (uint32_t)(m >> 32);
  if (rows32) {
    const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
    const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
    const uint64_t x = ((uint64_t)b[0] << 32) | a[0], y = ((uint64_t)b[1] << 32) | a[1];
    return x > y ? x : y;
  }
  const auto a = __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const uint64_t x = ((uint64_t)b[0] << 32) | a[0], y = ((uint64_t)b[1] << 32) | a[1];
  return x > y ? x : y;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t m) {
  m = max_dpp_u64<0xB1>(m);     // quad_perm 1,0,3,2: lane pairs
  m = max_dpp_u64<0x4E>(m);     // quad_perm 2,3,0,1: quads
  m = max_dpp_u64<0x141>(m);    // row_half_mirror: eight lanes
  m = max_dpp_u64<0x140>(m);    // row_mirror: rows of 16
  m = max_swap_u64(m, false);   // rows 0/1 and 2/3
  return max_swap_u64(m, true); // halves
}

__device__ __forceinline__ void topk_rounds(const float* row, int E, int k, int lane, int* sel_e, float* sel_v) {
  bool a0 = lane < E, a1 = lane + 64 < E;
  const uint64_t k0 = a0 ? route_key(row[lane], lane) : 0ull, k1 = a1 ? route_key(row[lane + 64], lane + 64) : 0ull;
  for (int slot = 0; slot < k; ++slot) {
    // remaining keys only; an exhausted lane offers 0, below every remaining key
    // of another lane unless that key is 0 too, and then the winner check below
    // still finds the one remaining owner
    uint64_t m = a0 ? k0 : 0ull;
    if (a1 && (!a0 || k1 > k0)) m = k1;
    m = wave_max_u64(m);
    const int e = 127 - (int)(m & 127u);
    if (a0 && k0 == m) a0 = false;
    if (a1 && k1 == m) a1 = false;
    if (lane == 0) {
      sel_e[slot] = e;
      sel_v[slot] = row[e];
    }
  }
}

template <typename T, int NW>
__global__ __launch_bounds__(64 * NW) void k_router_logits(const T* xn, const T* wr, int M, int d, int E, float* part) {
  __shared__ float red[NW - 1][4][64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6, g4 = lane >> 4, c16 = lane & 15;
  const int r0 = blockIdx.x * 16, e0 = blockIdx.y * 16, z = blockIdx.z, ksp = gridDim.z;
  const int KS = d / 32, KSW = KS / (ksp * NW), ks0 = (z * NW + wv) * KSW, ks1 = ks0 + KSW;
  // rows past M and experts past E repeat a valid one; their results are not stored
  const T* ap = xn + (size_t)min(r0 + c16, M - 1) * d + g4 * 8;
  const T* bp = wr + (size_t)min(e0 + c16, E - 1) * d + g4 * 8;
  f32x4_t acc = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int ks = ks0; ks < ks1; ks += 4) {
    Frag<T> a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ks + u < ks1) {
        router_frag(a[u], ap + (ks + u) * 32);
        router_frag(b[u], bp + (ks + u) * 32);
      }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (ks + u < ks1) mma16x16x32(acc, a[u], b[u]);
  }
  if (wv > 0)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv - 1][i][lane] = acc[i];
  __syncthreads();
  if (wv != 0) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float v = acc[i];
#pragma unroll
    for (int q = 0; q < NW - 1; ++q) v += red[q][i][lane];
    const int r = r0 + g4 * 4 + i, e = e0 + c16;
    if (r < M && e < E) part[((size_t)z * M + r) * E + e] = v;
  }
}

template <int RPB, int NW>
__global__ __launch_bounds__(64 * NW) void k_router_select(const float* part, int ksp, int M, int E, int k, float* rlog,
                                                          int* idx, float* w, int* pos, int* cnt, Gate gt, int n) {
  __shared__ float lg[RPB][129];
  __shared__ int sel_e[RPB][8];
  __shared__ float sel_v[RPB][8];
  __shared__ int ent_e[RPB * 8];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int r0 = blockIdx.x * RPB;
  const int nrow = min(RPB, M - r0);
  // every partial of this thread's (row, expert) entries is loaded before any
  // is added (one round trip), then the splits are summed in order
  constexpr int EPT = RPB * 128 / (64 * NW);       // entries per thread, at most
  float pv[EPT][kRouterMaxSplits];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int pr = t + j * 64 * NW;
    const int rl = pr / E, e = pr - rl * E;
    const size_t o = (size_t)(r0 + rl) * E + e;
#pragma unroll
    for (int z = 0; z < kRouterMaxSplits; ++z)
      if (pr < nrow * E && z < ksp) pv[j][z] = part[(size_t)z * M * E + o];
  }
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int pr = t + j * 64 * NW;
    if (pr < nrow * E) {
      const int rl = pr / E, e = pr - rl * E;
      float v = pv[j][0];
#pragma unroll
      for (int z = 1; z < kRouterMaxSplits; ++z)
        if (z < ksp) v += pv[j][z];
      lg[rl][e] = v;
      rlog[(size_t)(r0 + rl) * E + e] = v;
    }
  }
  __syncthreads();
  if (E > 32) {
    // top-k by rounds of a wave maximum, one row per wave
    for (int rl = wv; rl < nrow; rl += NW) topk_rounds(lg[rl], E, k, lane, sel_e[rl], sel_v[rl]);
  } else {
    // top-k by rank: the rank of expert e in its row is the number of logits
    // that beat it (greater, or equal with a lower id); ranks 0..k-1 are slots
    for (int pr = t; pr < nrow * E; pr += 64 * NW) {
      const int rl = pr / E, e = pr - rl * E;
      const float v = lg[rl][e];
      int rank = 0;
      for (int x = 0; x < E; ++x) {
        const float o = lg[rl][x];
        rank += (o > v) || (o == v && x < e);
      }
      if (rank < k) {
        sel_e[rl][rank] = e;
        sel_v[rl][rank] = v;
      }
    }
  }
  __syncthreads();
  // softmax over the selected logits, slots summed in order; entry q = (row q / k, slot q % k)
  const int nent = nrow * k;
  int* se = &ent_e[0];
  if (t < nent) {
    const int rl = t / k, j = t - rl * k;
    const float mx = sel_v[rl][0];
    float sum = 0.f;
    for (int u = 0; u < k; ++u) sum += expf(sel_v[rl][u] - mx);
    // rows of requests left out: expert -1, no place in the sorted order
    const bool live = gt.active((r0 + rl) / n);
    const int e = live ? sel_e[rl][j] : -1;
    idx[(size_t)r0 * k + t] = e;
    w[(size_t)r0 * k + t] = live ? expf(sel_v[rl][j] - mx) / sum : 0.f;
    se[t] = e;
  }
  __syncthreads();
  // rank of each entry among the block's entries of its expert, in entry order,
  // and the block's count per expert: eight consecutive lanes share an entry
  // (an expert), each scanning one sixteenth of the entries, added by shuffles
  static_assert(64 * NW >= 8 * RPB * 8 && 64 * NW >= 8 * 128, "eight lanes per entry and per expert");
  const int q = t >> 3, sl = t & 7, u0 = sl * (RPB * 8 / 8), u1 = u0 + RPB * 8 / 8;
  {
    const int e = q < nent ? se[q] : -1;
    int r = 0;
    for (int u = u0; u < u1 && u < q; ++u) r += se[u] == e;
    r += lane_partner<0>(r);      // the eight lanes of the entry: pairs, quads, half rows
    r += lane_partner<1>(r);
    r += lane_partner<2>(r);
    if (q < nent && sl == 0) pos[(size_t)r0 * k + q] = r;
  }
  {
    int c = 0;
    for (int u = u0; u < u1 && u < nent; ++u) c += se[u] == q;
    c += lane_partner<0>(c);
    c += lane_partner<1>(c);
    c += lane_partner<2>(c);
    if (q < E && sl == 0) cnt[(size_t)q * gridDim.x + blockIdx.x] = c;
  }
}

constexpr int kFinishLds = 16384;     // count-table entries kept in LDS by the finish kernel
constexpr int kFinishThreads = 1024;

__global__ __launch_bounds__(kFinishThreads) void k_route_finish(const int* idx, int M, int k, int E, int nblk,
                                                                 int rpb, int tr, int* cnt, int* perm, int* pos,
                                                                 int4* tiles, int* n_tiles) {
  constexpr int NT = kFinishThreads;
  __shared__ int seg[NT];
  __shared__ int offs[128], toff[129], routed;
  __shared__ int tab[kFinishLds];
  const int t = threadIdx.x;
  // the count table [E][nblk]: in LDS when it fits (one coalesced read), else
  // in place in memory.  With the table in LDS several workgroups may run:
  // each forms the (identical) prefixes and offsets and places its own slice
  // of the entries; workgroup 0 writes the tile list.
  const bool in_lds = E * nblk <= kFinishLds;
  int* ct = in_lds ? tab : cnt;
  if (in_lds) {
#pragma unroll 4
    for (int i = t; i < E * nblk; i += NT) tab[i] = cnt[i];
    __syncthreads();
  }
  // per expert: tpe threads each sum a run of blocks, then turn their run into
  // exclusive per-block prefixes
  int ep = 1;
  while (ep < E) ep <<= 1;
  const int tpe = NT / ep;                        // threads per expert (>= 8)
  const int e = t / tpe, sg = t % tpe;
  const int per = (nblk + tpe - 1) / tpe, b0 = min(nblk, sg * per), b1 = min(nblk, b0 + per);
  int* row = ct + (size_t)(e < E ? e : 0) * nblk;
  int ssum = 0;
  if (e < E)
    for (int b = b0; b < b1; ++b) ssum += row[b];
  seg[t] = ssum;
  __syncthreads();
  if (e < E) {
    int run = 0;
    for (int j = 0; j < sg; ++j) run += seg[e * tpe + j];
    for (int b = b0; b < b1; ++b) {
      const int c = row[b];
      row[b] = run;
      run += c;
    }
    if (sg == tpe - 1) offs[e] = run;             // the expert's total
  }
  __syncthreads();
  // exclusive prefixes over experts of the row counts and of the tr-row tile
  // counts: one wave, two experts per lane, a shuffle scan
  if (t < 64) {
    const int x0 = 2 * t, x1 = 2 * t + 1;
    const int c0 = x0 < E ? offs[x0] : 0, c1 = x1 < E ? offs[x1] : 0;
    const int n0 = (c0 + tr - 1) / tr, n1 = (c1 + tr - 1) / tr;
    int rs = c0 + c1, ts = n0 + n1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int ro = __shfl_up(rs, o, 64), to = __shfl_up(ts, o, 64);
      if (t >= o) { rs += ro; ts += to; }
    }
    const int rx = rs - c0 - c1, tx = ts - n0 - n1;   // exclusive
    if (x0 < E) { offs[x0] = rx; toff[x0] = tx; }
    if (x1 < E) { offs[x1] = rx + c0; toff[x1] = tx + n0; }
    if (t == 63) {
      toff[E] = ts;
      routed = rs;          // entries with an expert (rows left out have none)
      if (blockIdx.x == 0) *n_tiles = ts;
    }
  }
  __syncthreads();
  for (int x = t; x < E && blockIdx.x == 0; x += NT) {
    const int c = (x + 1 < E ? offs[x + 1] : routed) - offs[x];
    for (int q = 0; q < toff[x + 1] - toff[x]; ++q)
      tiles[toff[x] + q] = make_int4(x, offs[x] + q * tr, min(tr, c - q * tr), 0);
  }
  const int MK = M * k, slice = (MK + gridDim.x - 1) / gridDim.x;
  const int lo = blockIdx.x * slice, hi = min(MK, lo + slice);
  for (int i0 = lo + t; i0 < hi; i0 += 4 * NT) {   // four independent entries in flight per thread
    int ex[4], rk[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT;
      ex[u] = i < hi ? idx[i] : 0;
      rk[u] = i < hi ? pos[i] : 0;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u * NT;
      if (i < hi && ex[u] >= 0) {
        const int p = offs[ex[u]] + ct[(size_t)ex[u] * nblk + i / (rpb * k)] + rk[u];
        pos[i] = p;
        perm[p] = i / k;
      }
    }
  }
}

int router_rows_per_block(int) { return 16; }

// K splits of the logits: enough workgroups to spread the router matrix over
// the chip (~256), each wave keeping at least one whole K step.
int router_ksplits(int M, int d, int E) {
  const int blocks = ((M + 15) / 16) * ((E + 15) / 16);
  int ksp = 1;
  while (blocks * ksp < 256 && 2 * ksp <= kRouterMaxSplits && d % (32 * 2 * ksp * kRouterWaves) == 0) ksp *= 2;
  return ksp;
}

template <typename T>
hipError_t router(const T* xn, const T* wr, int M, int d, int E, int k, float* rlog, int* idx, float* w, int* perm,
                  int* pos, int4* tiles, int* n_tiles, int tile_rows, int* cnt, float* part, Gate gt, int n,
                  hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (d % (32 * kRouterWaves) != 0 || E > 128 || k > 8 || tile_rows < 1) return hipErrorInvalidValue;
  constexpr int RPB = 16;
  const int nblk = (M + RPB - 1) / RPB, ksp = router_ksplits(M, d, E);
  hipLaunchKernelGGL((k_router_logits<T, kRouterWaves>), dim3(nblk, (E + 15) / 16, ksp), dim3(64 * kRouterWaves), 0, s,
                     xn, wr, M, d, E, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((k_router_select<RPB, 16>), dim3(nblk), dim3(1024), 0, s, part, ksp, M, E, k, rlog, idx, w, pos,
                     cnt, gt, n);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // one workgroup per 1024 entries (up to 64) when the count table fits LDS
  const int fin_ent = (M * k + kFinishThreads - 1) / kFinishThreads;
  const int fin_wg = E * nblk <= kFinishLds ? (fin_ent < 64 ? fin_ent : 64) : 1;
  hipLaunchKernelGGL(k_route_finish, dim3(fin_wg), dim3(kFinishThreads), 0, s, idx, M, k, E, nblk, RPB, tile_rows,
                     cnt, perm, pos, tiles, n_tiles);
  return hipGetLastError();
}
template hipError_t router<float>(const float*, const float*, int, int, int, int, float*, int*, float*, int*, int*,
                                  int4*, int*, int, int*, float*, Gate, int, hipStream_t);
template hipError_t router<bf16>(const bf16*, const bf16*, int, int, int, int, float*, int*, float*, int*, int*,
                                 int4*, int*, int, int*, float*, Gate, int, hipStream_t);

// ------------------------------------------------------------------ router for few entries
// When the routed entries of a launch fit one workgroup (M * k <= 4096), the
// router is two launches instead of three plus the norm:
//  k_add_norm_router: the add-norm workgroup of a row also forms the row's E
//    router logits from the rounded normed row (E groups of threads, each
//    thread a fixed interleave of 8-element pieces so a group reads whole
//    cache lines of W_r; pieces in order, then a fixed shuffle tree), its top
//    k -- ties to the lower expert id -- and the softmax over the selected;
//  k_route_sort (one workgroup): the expert-sorted order of all M * k
//    entries, rows of an expert in row order: per (entry block, wave) counts
//    and in-wave ranks by ballots, exclusive prefixes per expert, expert
//    offsets, the tile list, pos and perm.
constexpr int kSortThreads = 1024, kSortMaxEntries = 4096, kSortBlocks = kSortMaxEntries / kSortThreads;
constexpr int kRouterPieces = 16;

// at most kRouterPieces 8-element pieces of W_r per thread, all loaded at once
static bool router_pieces_ok(int d, int E) {
  const int nt = row_threads(d);
  return (E & (E - 1)) == 0 && nt >= 64 && E <= nt && nt / E <= 64 && d % (8 * (nt / E)) == 0 &&
         d / (8 * (nt / E)) <= kRouterPieces;
}
// W_r streamed by whole waves in kilobyte pieces
static bool router_stream_ok(int d) {
  const int it = d / 512;
  return d % 512 == 0 && (it == 1 || it == 2 || it == 4 || it == 6 || it == 8);
}

bool router_fused_ok(int M, int d, int E, int k) {
  return M * k <= kSortMaxEntries && E <= 128 && k >= 1 && k <= 8 && k <= E && d <= kMaxModel &&
         (router_pieces_ok(d, E) || router_stream_ok(d));
}

// One 8-element piece of a router-matrix row, held as loaded (load) and
// widened to fp32 where it is used (get).
template <typename T> struct WrPiece;
template <>
struct WrPiece<bf16> {
  uint4 u;
  __device__ __forceinline__ void load(const bf16* p) { u = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void get(float (&w)[8]) const {
    const uint32_t x[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) { w[2 * j] = __uint_as_float(x[j] << 16); w[2 * j + 1] = __uint_as_float(x[j] & 0xFFFF0000u); }
  }
};
template <>
struct WrPiece<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void get(float (&w)[8]) const {
    w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w; w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
  }
};

// Top k of one row's E logits (lg, in LDS) by one wave -- ties to the lower
// expert id -- and the softmax over the selected, slots summed in order.
__device__ __forceinline__ void row_topk_softmax(const float* lg, int E, int k, int r, int* idx, float* w, int* sel_e,
                                                 float* sel_v) {
  const int lane = threadIdx.x & 63;
  if (E > 32) {
    topk_rounds(lg, E, k, lane, sel_e, sel_v);
  } else if (lane < E) {
    // rank of expert lane: the logits that beat it (greater, or equal with a lower id)
    const float x = lg[lane];
    int rank = 0;
    for (int q = 0; q < E; ++q) {
      const float o = lg[q];
      rank += (o > x) || (o == x && q < lane);
    }
    if (rank < k) { sel_e[rank] = lane; sel_v[rank] = x; }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");   // one wave: LDS writes before reads
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
  if (lane < k) {
    const float mx = sel_v[0];
    float sum = 0.f;
    for (int u = 0; u < k; ++u) sum += expf(sel_v[u] - mx);
    idx[(size_t)r * k + lane] = sel_e[lane];
    w[(size_t)r * k + lane] = expf(sel_v[lane] - mx) / sum;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_add_norm_router(const float* part, int S, int M, int d, const float* g,
                                                         float eps, float* H, T* xn, const T* wr, int E, int k,
                                                         float* rlog, int* idx, float* w, Gate gt, int n) {
  __shared__ float xs[kMaxModel];
  __shared__ float lg[128];
  __shared__ int sel_e[8];
  __shared__ float sel_v[8];
  const int r = blockIdx.x, nj = d / (4 * blockDim.x), tid = threadIdx.x, lane = tid & 63;
  if (!gt.active(r / n)) {            // a row of a request left out: no expert, no place in the order
    if (tid < k) { idx[(size_t)r * k + tid] = -1; w[(size_t)r * k + tid] = 0.f; }
    return;
  }
  // this thread's pieces of the router matrix (expert e, pieces sl, sl + tpe,
  // ...), requested first so that they arrive while the row is added and
  // normalised; pieces past ppt repeat the last one and are not added
  const int tpe = blockDim.x / E, e = tid / tpe, sl = tid % tpe;
  const T* wrow = wr + (size_t)e * d;
  const int ppt = d / (8 * tpe);                  // pieces of this thread (<= kRouterPieces)
  WrPiece<T> wp[kRouterPieces];
#pragma unroll
  for (int u = 0; u < kRouterPieces; ++u) wp[u].load(wrow + (sl + min(u, ppt - 1) * tpe) * 8);
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + tid) * 4;
      const float4 p = sum_splits4(part, S, (size_t)M * d, (size_t)r * d + c);
      float4 x = *reinterpret_cast<const float4*>(H + (size_t)r * d + c);
      add4(x, p);
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d, xs);
  __syncthreads();
  // logit of expert e: tpe threads, thread sl taking pieces sl, sl + tpe, ...
  float acc = 0.f;
#pragma unroll
  for (int u = 0; u < kRouterPieces; ++u)
    if (u < ppt) {
      const int c = sl + u * tpe;
      float wv[8];
      wp[u].get(wv);
      const float4 x0 = *reinterpret_cast<const float4*>(xs + c * 8), x1 = *reinterpret_cast<const float4*>(xs + c * 8 + 4);
      acc += x0.x * wv[0]; acc += x0.y * wv[1]; acc += x0.z * wv[2]; acc += x0.w * wv[3];
      acc += x1.x * wv[4]; acc += x1.y * wv[5]; acc += x1.z * wv[6]; acc += x1.w * wv[7];
    }
  // the expert's tpe (aligned, a power of two <= 64) lanes: butterfly steps up to tpe
  butterfly_steps([&](auto st) {
    if ((2 << decltype(st)::value) <= tpe) acc += lane_partner<decltype(st)::value>(acc);
  });
  if (sl == 0) {
    lg[e] = acc;
    rlog[(size_t)r * E + e] = acc;
  }
  __syncthreads();
  if (tid < 64) row_topk_softmax(lg, E, k, r, idx, w, sel_e, sel_v);
}

// Sums over a wave's 64 lanes of C values at once: each step over lane bit S
// (high bits first) pairs every lane with its partner across that bit; while
// more than one value is left, a lane keeps one half of its values (the upper
// half where the bit is set), adds the partner's copy of that half and sends
// the other half.  After log2 C halving steps lane l holds value
// idx = (the top log2 C bits of l), and the remaining steps sum it over the
// lanes that share idx, in a fixed order.
template <int S, int C>
__device__ __forceinline__ void halving_sum(float* v, int& idx) {
  if constexpr (C > 1) {
    const bool hi = (threadIdx.x >> S) & 1;
#pragma unroll
    for (int u = 0; u < C / 2; ++u) {
      const float send = hi ? v[u] : v[u + C / 2];
      const float keep = hi ? v[u + C / 2] : v[u];
      v[u] = keep + lane_partner<S>(send);
    }
    if (hi) idx += C / 2;
  } else {
    v[0] += lane_partner<S>(v[0]);
  }
  if constexpr (S > 0) halving_sum<S - 1, (C > 1 ? C / 2 : 1)>(v, idx);
}

// Dot product of a kilobyte-piece run of a router-matrix row with the row's
// matching pieces: bf16 pairs on the packed dot instruction (fp32 sums, the
// pairs in element order), fp32 by fused multiply-adds.
template <typename T, int IT> struct RouterDot;
template <int IT>
struct RouterDot<bf16, IT> {
  uint32_t x[IT][4];                  // the normalised row, bf16 pairs
  __device__ __forceinline__ void set(const float* xs, int lane) {
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float* p = xs + (lane + 64 * i) * 8 + 2 * q;   // bf16 values: their upper halves are exact
        x[i][q] = (__float_as_uint(p[0]) >> 16) | (__float_as_uint(p[1]) & 0xFFFF0000u);
      }
  }
  __device__ __forceinline__ float dot(const WrPiece<bf16> (&w)[IT]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      const uint32_t wq[4] = {w[i].u.x, w[i].u.y, w[i].u.z, w[i].u.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, x[i][q]),
                                              __builtin_bit_cast(bf16x2_t, wq[q]), acc, false);
    }
    return acc;
  }
};
template <int IT>
struct RouterDot<float, IT> {
  float x[IT][8];
  __device__ __forceinline__ void set(const float* xs, int lane) {
#pragma unroll
    for (int i = 0; i < IT; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) x[i][q] = xs[(lane + 64 * i) * 8 + q];
  }
  __device__ __forceinline__ float dot(const WrPiece<float> (&w)[IT]) const {
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < IT; ++i) {
      float wq[8];
      w[i].get(wq);
#pragma unroll
      for (int q = 0; q < 8; ++q) acc += x[i][q] * wq[q];
    }
    return acc;
  }
};

// Large router matrices (d a multiple of 512): the row's workgroup streams
// W_r in batches of EB rows, each row read by a whole wave as IT = d / 512
// contiguous kilobyte pieces (lane l takes 8-element pieces l, l + 64, ...);
// a lane's products go through its pieces in order, and the batch's EB sums
// over the wave are formed together (halving_sum).  Waves take expert batches
// round-robin, two batches in flight; the first is requested before the row
// is added and normalised.  Row r visits the experts from expert r mod E on,
// so that the rows' workgroups, which all read the same matrix at once,
// spread their requests over the L2 channels.
template <typename T, int IT>
__global__ __launch_bounds__(512) void k_add_norm_router_stream(const float* part, int S, int M, int d,
                                                                const float* g, float eps, float* H, T* xn,
                                                                const T* wr, int E, int k, float* rlog, int* idx,
                                                                float* w, Gate gt, int n) {
  // router rows per batch: 16 bf16 (8 fp32) pieces in flight per lane
  constexpr int PIF = sizeof(T) == 2 ? 16 : 8, EB = IT >= PIF ? 1 : PIF / IT;
  static_assert((EB & (EB - 1)) == 0 && EB <= 64, "a power-of-two batch");
  __shared__ float xs[kMaxModel];
  __shared__ float lg[128];
  __shared__ int sel_e[8];
  __shared__ float sel_v[8];
  const int r = blockIdx.x, nj = d / (4 * blockDim.x), tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave: scalar loop control
  const int step = (blockDim.x >> 6) * EB;
  if (!gt.active(r / n)) {            // a row of a request left out: no expert, no place in the order
    if (tid < k) { idx[(size_t)r * k + tid] = -1; w[(size_t)r * k + tid] = 0.f; }
    return;
  }
  const int rot = r % E;
  WrPiece<T> wa[EB][IT], wb[EB][IT];
  auto load = [&](WrPiece<T>(&buf)[EB][IT], int e0) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < EB; ++j) {
      // visit index past E: a repeat of the last one, not stored
      const int e = min(e0 + j, E - 1) + rot;
      const T* row = wr + (size_t)(e < E ? e : e - E) * d;
#pragma unroll
      for (int i = 0; i < IT; ++i) buf[j][i].load(row + (lane + 64 * i) * 8);
    }
  };
  int e0 = wv * EB;
  load(wa, e0);
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + tid) * 4;
      const float4 p = sum_splits4(part, S, (size_t)M * d, (size_t)r * d + c);
      float4 x = *reinterpret_cast<const float4*>(H + (size_t)r * d + c);
      add4(x, p);
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d, xs);
  __syncthreads();
  RouterDot<T, IT> xd;
  xd.set(xs, lane);
  auto consume = [&](const WrPiece<T>(&buf)[EB][IT], int b0) __attribute__((always_inline)) {
    float acc[EB];
#pragma unroll
    for (int j = 0; j < EB; ++j) acc[j] = xd.dot(buf[j]);
    int q = 0;
    halving_sum<5, EB>(acc, q);
    const int e = b0 + q + rot < E ? b0 + q + rot : b0 + q + rot - E;
    if ((lane & (64 / EB - 1)) == 0 && b0 + q < E) {
      lg[e] = acc[0];
      rlog[(size_t)r * E + e] = acc[0];
    }
  };
  // the next batch is requested unconditionally (visit indices past E repeat
  // the last row): a load under a branch would make the wait before the
  // batch in hand cover the loads just issued
  for (; e0 < E; e0 += 2 * step) {
    load(wb, e0 + step);
    consume(wa, e0);
    if (e0 + step >= E) break;
    load(wa, e0 + 2 * step);
    consume(wb, e0 + step);
  }
  __syncthreads();
  if (tid < 64) row_topk_softmax(lg, E, k, r, idx, w, sel_e, sel_v);
}

__global__ __launch_bounds__(kSortThreads) void k_route_sort(const int* idx, int MK, int k, int E, int tr, int* perm,
                                                            int* pos, int4* tiles, int* n_tiles) {
  constexpr int NW = kSortThreads / 64;
  __shared__ int cnt[kSortBlocks][NW][128];
  __shared__ int offs[128], toff[129], routed;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int nb = (MK + kSortThreads - 1) / kSortThreads;
  int ex[kSortBlocks], rk[kSortBlocks];
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));   // lanes below this one
#pragma unroll
  for (int j = 0; j < kSortBlocks; ++j) {
    ex[j] = -1; rk[j] = 0;
    if (j < nb) {
      const int i = j * kSortThreads + t;
      ex[j] = i < MK ? idx[i] : -1;
      cnt[j][wv][lane] = 0;
      cnt[j][wv][lane + 64] = 0;
      // entries of this wave in entry order: one ballot per distinct expert
      uint64_t left = __ballot(ex[j] >= 0);
      while (left) {
        const int leader = __ffsll((unsigned long long)left) - 1;
        const int e = __builtin_amdgcn_readlane(ex[j], leader);
        const uint64_t m = __ballot(ex[j] == e);
        if (ex[j] == e) rk[j] = __popcll(m & lt);
        if (lane == 0) cnt[j][wv][e] = __popcll(m);
        left &= ~m;
      }
    }
  }
  __syncthreads();
  // per expert: exclusive prefix over (block, wave) in entry order; the total
  if (t < E) {
    int run = 0;
    for (int j = 0; j < nb; ++j)
      for (int q = 0; q < NW; ++q) {
        const int c = cnt[j][q][t];
        cnt[j][q][t] = run;
        run += c;
      }
    offs[t] = run;
  }
  __syncthreads();
  // exclusive prefixes over experts of the row counts and of the tr-row tile
  // counts: one wave, two experts per lane, a shuffle scan
  if (t < 64) {
    const int x0 = 2 * t, x1 = 2 * t + 1;
    const int c0 = x0 < E ? offs[x0] : 0, c1 = x1 < E ? offs[x1] : 0;
    const int n0 = (c0 + tr - 1) / tr, n1 = (c1 + tr - 1) / tr;
    int rs = c0 + c1, ts = n0 + n1;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int ro = __shfl_up(rs, o, 64), to = __shfl_up(ts, o, 64);
      if (t >= o) { rs += ro; ts += to; }
    }
    const int rx = rs - c0 - c1, tx = ts - n0 - n1;   // exclusive
    if (x0 < E) { offs[x0] = rx; toff[x0] = tx; }
    if (x1 < E) { offs[x1] = rx + c0; toff[x1] = tx + n0; }
    if (t == 63) { toff[E] = ts; routed = rs; *n_tiles = ts; }
  }
  __syncthreads();
  for (int x = t; x < E; x += kSortThreads) {
    const int c = (x + 1 < E ? offs[x + 1] : routed) - offs[x];
    for (int q = 0; q < toff[x + 1] - toff[x]; ++q)
      tiles[toff[x] + q] = make_int4(x, offs[x] + q * tr, min(tr, c - q * tr), 0);
  }
#pragma unroll
  for (int j = 0; j < kSortBlocks; ++j) {
    if (ex[j] < 0) continue;
    const int i = j * kSortThreads + t;
    const int p = offs[ex[j]] + cnt[j][wv][ex[j]] + rk[j];
    pos[i] = p;
    perm[p] = i / k;
  }
}

template <typename T>
hipError_t add_norm_router(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                           const T* wr, int E, int k, float* rlog, int* idx, float* w, Gate gt, int n,
                           hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (!router_fused_ok(M, d, E, k)) return hipErrorInvalidValue;
  if (router_pieces_ok(d, E)) {
    hipLaunchKernelGGL((k_add_norm_router<T>), dim3(M), dim3(row_threads(d)), 0, s, part, S, M, d, g, eps, H, xn, wr, E,
                       k, rlog, idx, w, gt, n);
    return hipGetLastError();
  }
  // up to eight waves, each thread the same whole number of float4 chunks of the row
  int nt = d / 4, nj = 1;
  while (nt > 512 || 4 * nt * nj != d) nt = d / (4 * ++nj);
  const dim3 block(nt);
  switch (d / 512) {
#define DG_ROUTER_IT(IT)                                                                                         \
  case IT:                                                                                                       \
    hipLaunchKernelGGL((k_add_norm_router_stream<T, IT>), dim3(M), block, 0, s, part, S, M, d, g, eps, H, xn, wr, E, \
                       k, rlog, idx, w, gt, n);                                                                  \
    break;
    DG_ROUTER_IT(1)
    DG_ROUTER_IT(2)
    DG_ROUTER_IT(4)
    DG_ROUTER_IT(6)
    DG_ROUTER_IT(8)
#undef DG_ROUTER_IT
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t route_sort(const int* idx, int M, int k, int E, int tile_rows, int* perm, int* pos, int4* tiles,
                      int* n_tiles, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (M * k > kSortMaxEntries || E > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_route_sort, dim3(1), dim3(kSortThreads), 0, s, idx, M * k, k, E, tile_rows, perm, pos, tiles,
                     n_tiles);
  return hipGetLastError();
}

// ------------------------------------------------------------------ transpose
template <typename T>
__global__ void k_transpose(const T* src, T* dst, int rows, int cols) {
  __shared__ T tile[32][33];
  const int c0 = blockIdx.x * 32, r0 = blockIdx.y * 32;
  for (int y = threadIdx.y; y < 32; y += 8) {
    const int r = r0 + y, c = c0 + threadIdx.x;
    if (r < rows && c < cols) tile[y][threadIdx.x] = src[(size_t)r * cols + c];
  }
  __syncthreads();
  for (int y = threadIdx.y; y < 32; y += 8) {
    const int c = c0 + y, r = r0 + threadIdx.x;
    if (r < rows && c < cols) dst[(size_t)c * rows + r] = tile[threadIdx.x][y];
  }
}
template <typename T>
hipError_t transpose(const T* src, T* dst, int rows, int cols, hipStream_t s) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  hipLaunchKernelGGL((k_transpose<T>), grid, dim3(32, 8), 0, s, src, dst, rows, cols);
  return hipGetLastError();
}

// ------------------------------------------------------------------ canvas init
__global__ void k_init_canvas(int32_t* canvas, SeedArg seeds, int n, int vocab, const int32_t* cidx) {
  const int b = blockIdx.x;
  const uint32_t c = (uint32_t)cidx[b];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint4 x = philox_block(seeds.v[b], kTagInit, c, 0u, (uint32_t)i, 0u);
    canvas[(size_t)b * n + i] = token_of(x.x, vocab);
  }
}
hipError_t init_canvas(int32_t* canvas, const SeedArg& seeds, int B, int n, int vocab, const int32_t* cidx,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_init_canvas, dim3(B), dim3(256), 0, s, canvas, seeds, n, vocab, cidx);
  return hipGetLastError();
}

__global__ void k_advance_context(int32_t* ctx, int32_t* cidx, int B, int add, int add_canvas, Gate g) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < B && g.active(b)) {
    ctx[b] += add;
    cidx[b] += add_canvas;
  }
}
hipError_t advance_context(int32_t* ctx, int32_t* cidx, int B, int add, int add_canvas, Gate g, hipStream_t s) {
  hipLaunchKernelGGL(k_advance_context, dim3((B + 63) / 64), dim3(64), 0, s, ctx, cidx, B, add, add_canvas, g);
  return hipGetLastError();
}

__global__ void k_fill_u32(uint32_t* p, uint32_t v, size_t count) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}
__global__ void k_fill_u8(uint8_t* p, uint8_t v, size_t count) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) p[i] = v;
}
hipError_t fill_u8(void* p, uint8_t v, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u8, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, static_cast<uint8_t*>(p), v,
                     count);
  return hipGetLastError();
}
hipError_t fill_u32(void* p, uint32_t v, size_t count, hipStream_t s) {
  if (count == 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3((unsigned)((count + 255) / 256)), dim3(256), 0, s, static_cast<uint32_t*>(p), v,
                     count);
  return hipGetLastError();
}

#define DG_INST(T)                                                                                               \
  template hipError_t add_norm_router<T>(const float*, int, int, int, const float*, float, float*, T*, const T*,  \
                                         int, int, float*, int*, float*, Gate, int, hipStream_t);               \
  template hipError_t embed_norm<T>(const T*, const int32_t*, const float*, int, int, int, int, const float*,  \
                                    float, float*, T*, Gate, int, hipStream_t);                                 \
  template hipError_t add_norm<T>(const float*, int, int, int, const float*, float, float*, T*, Gate, int,      \
                                  hipStream_t);                                                                 \
  template hipError_t combine_norm<T>(const T*, const int*, const float*, int, int, int, const float*, float,     \
                                      float*, T*, Gate, int, hipStream_t);                                      \
  template hipError_t rope_scatter<T>(const float*, int, const float2*, T*, T*, T*, int, int, int, int, int, int, \
                                      PosArg, Gate, hipStream_t);                                               \
  template hipError_t transpose<T>(const T*, T*, int, int, hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

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

// Stores the updated residual row v and y = rnd(v * g / sqrt(mean(v^2) + eps)).
template <typename T>
__device__ __forceinline__ void norm_store(float4 (&v)[kRowChunks], int nj, int d, const float* g, float eps,
                                           float* hrow, T* xrow) {
  __shared__ float red[4];
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
      Num<T>::store(xrow + c + 0, v[j].x * inv * gg.x);
      Num<T>::store(xrow + c + 1, v[j].y * inv * gg.y);
      Num<T>::store(xrow + c + 2, v[j].z * inv * gg.z);
      Num<T>::store(xrow + c + 3, v[j].w * inv * gg.w);
    }
}

__device__ __forceinline__ void add4(float4& a, const float4 b) {
  a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
}
}  // namespace

// h = emb[tok] (+ sum_s part[s]); xn = rnd(rmsnorm(h) * g)
template <typename T>
__global__ __launch_bounds__(256) void k_embed_norm(const T* emb, const int32_t* tok, const float* part, int S,
                                                    int M, int d, int vocab, const float* g, float eps, float* H,
                                                    T* xn) {
  const int r = blockIdx.x, nj = d / (4 * blockDim.x);
  const int id = min(max(tok[r], 0), vocab - 1);   // out-of-range ids are clamped, never read past E
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + threadIdx.x) * 4;
      const T* e = emb + (size_t)id * d + c;
      float4 x = make_float4(Num<T>::load(e), Num<T>::load(e + 1), Num<T>::load(e + 2), Num<T>::load(e + 3));
      float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < S; ++s) add4(p, *reinterpret_cast<const float4*>(part + ((size_t)s * M + r) * d + c));
      add4(x, p);
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

// h += sum_s part[s]; xn = rnd(rmsnorm(h) * g)
template <typename T>
__global__ __launch_bounds__(256) void k_add_norm(const float* part, int S, int M, int d, const float* g, float eps,
                                                  float* H, T* xn) {
  const int r = blockIdx.x, nj = d / (4 * blockDim.x);
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + threadIdx.x) * 4;
      float4 p = make_float4(0.f, 0.f, 0.f, 0.f);
      for (int s = 0; s < S; ++s) add4(p, *reinterpret_cast<const float4*>(part + ((size_t)s * M + r) * d + c));
      float4 x = *reinterpret_cast<const float4*>(H + (size_t)r * d + c);
      add4(x, p);
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

// h += sum_j w[j] * Y[pos[j]] (slots in selection order); xn = rnd(rmsnorm(h) * g)
template <typename T>
__global__ __launch_bounds__(256) void k_combine_norm(const float* Y, const int* pos, const float* w, int k, int M,
                                                      int d, const float* g, float eps, float* H, T* xn) {
  const int r = blockIdx.x, nj = d / (4 * blockDim.x);
  int ps[8];
  float ws[8];
#pragma unroll
  for (int s = 0; s < 8; ++s)
    if (s < k) { ps[s] = pos[(size_t)r * k + s]; ws[s] = w[(size_t)r * k + s]; }
  float4 v[kRowChunks];
#pragma unroll
  for (int j = 0; j < kRowChunks; ++j)
    if (j < nj) {
      const int c = (j * blockDim.x + threadIdx.x) * 4;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int s = 0; s < 8; ++s)
        if (s < k) {
          const float4 y = *reinterpret_cast<const float4*>(Y + (size_t)ps[s] * d + c);
          acc.x += ws[s] * y.x; acc.y += ws[s] * y.y; acc.z += ws[s] * y.z; acc.w += ws[s] * y.w;
        }
      float4 x = *reinterpret_cast<const float4*>(H + (size_t)r * d + c);
      add4(x, acc);
      v[j] = x;
    }
  norm_store<T>(v, nj, d, g, eps, H + (size_t)r * d, xn + (size_t)r * d);
}

template <typename T>
hipError_t embed_norm(const T* emb, const int32_t* tok, const float* part, int S, int M, int d, int vocab,
                      const float* g, float eps, float* H, T* xn, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_embed_norm<T>), dim3(M), dim3(row_threads(d)), 0, s, emb, tok, part, S, M, d, vocab, g, eps,
                     H, xn);
  return hipGetLastError();
}
template <typename T>
hipError_t add_norm(const float* part, int S, int M, int d, const float* g, float eps, float* H, T* xn,
                    hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_add_norm<T>), dim3(M), dim3(row_threads(d)), 0, s, part, S, M, d, g, eps, H, xn);
  return hipGetLastError();
}
template <typename T>
hipError_t combine_norm(const float* Y, const int* pos, const float* w, int k, int M, int d, const float* g,
                        float eps, float* H, T* xn, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_combine_norm<T>), dim3(M), dim3(row_threads(d)), 0, s, Y, pos, w, k, M, d, g, eps, H, xn);
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
                               int Hq, int Hkv, int hd, int max_ctx, int ctx) {
  const int r = blockIdx.x, b = r / n, i = r % n, pos = ctx + i, half = hd / 2;
  const int ncol = (Hq + 2 * Hkv) * hd;
  const size_t sstride = (size_t)M * ncol;
  const float* x = part + (size_t)r * ncol;
  const float2* cs = rope + (size_t)pos * half;
  for (int u = threadIdx.x; u < (Hq + Hkv) * half; u += blockDim.x) {
    const int head = u / half, j = u % half;
    float a = 0.f, bb = 0.f;
    for (int s = 0; s < S; ++s) {
      a += x[s * sstride + head * hd + j];
      bb += x[s * sstride + head * hd + j + half];
    }
    const float2 t = cs[j];
    const float o1 = a * t.x - bb * t.y, o2 = bb * t.x + a * t.y;
    if (head < Hq) {
      T* dst = q + (size_t)r * Hq * hd + head * hd;
      Num<T>::store(dst + j, o1);
      Num<T>::store(dst + j + half, o2);
    } else {
      const int kh = head - Hq;
      T* dst = kc + (((size_t)b * Hkv + kh) * max_ctx + pos) * hd;
      Num<T>::store(dst + j, o1);
      Num<T>::store(dst + j + half, o2);
    }
  }
  for (int u = threadIdx.x; u < Hkv * hd; u += blockDim.x) {
    const int kh = u / hd, c = u % hd;
    float v = 0.f;
    for (int s = 0; s < S; ++s) v += x[s * sstride + (Hq + Hkv) * hd + u];
    Num<T>::store(vc + (((size_t)b * Hkv + kh) * max_ctx + pos) * hd + c, v);
  }
}
template <typename T>
hipError_t rope_scatter(const float* part, int S, const float2* rope, T* q, T* kc, T* vc, int B, int n, int Hq,
                        int Hkv, int hd, int max_ctx, int ctx, hipStream_t s) {
  if (B * n <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_rope_scatter<T>), dim3(B * n), dim3(256), 0, s, part, S, rope, q, kc, vc, B * n, n, Hq,
                     Hkv, hd, max_ctx, ctx);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router
// One wave per row: the router logits (sum of split partials) sit two per
// lane; k rounds of a wave arg-max (ties to the lower expert id) pick the
// experts in descending order, then softmax over the selected logits.
__global__ __launch_bounds__(256) void k_router_topk(const float* part, int S, int M, int E, int k, float* rlog,
                                                     int* idx, float* w) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  float v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = lane + 64 * h;
    float x = -INFINITY;
    if (e < E) {
      x = 0.f;
      for (int s = 0; s < S; ++s) x += part[((size_t)s * M + r) * E + e];
      rlog[(size_t)r * E + e] = x;
    }
    v[h] = x;
  }
  bool used0 = lane >= E, used1 = lane + 64 >= E;
  float sel[8];
  int sid[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= k) break;
    float bv;
    int bi;
    if (!used0 && (used1 || v[0] >= v[1])) { bv = v[0]; bi = lane; }
    else if (!used1) { bv = v[1]; bi = lane + 64; }
    else { bv = -INFINITY; bi = 0x7fffffff; }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > bv || (ov == bv && oi < bi)) { bv = ov; bi = oi; }
    }
    if (bi == lane) used0 = true;
    if (bi == lane + 64) used1 = true;
    sel[j] = bv;
    sid[j] = bi;
  }
  if (lane == 0) {
    const float mx = sel[0];   // selection order is descending, so slot 0 holds the max
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) if (j < k) { sel[j] = expf(sel[j] - mx); sum += sel[j]; }
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (j < k) {
        idx[(size_t)r * k + j] = sid[j];
        w[(size_t)r * k + j] = sel[j] / sum;
      }
  }
}
hipError_t router_topk(const float* part, int S, int M, int E, int k, float* rlog, int* idx, float* w,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_topk, dim3((M + 3) / 4), dim3(256), 0, s, part, S, M, E, k, rlog, idx, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bucketing
// One workgroup: per-expert counts, the 64-row tile list, then a stable
// scatter of (row, slot) entries by expert, rows in chunks of 256 whose ranks
// within an expert come from an LDS bitmask.
__global__ __launch_bounds__(256) void k_route_bucket(const int* idx, int M, int k, int E, int* perm, int* pos,
                                                      int4* tiles, int* n_tiles) {
  __shared__ int cnt[128], base[128];
  __shared__ uint32_t bits[128][8];
  const int t = threadIdx.x;
  if (t < 128) cnt[t] = 0;
  __syncthreads();
  for (int r = t; r < M; r += 256)
    for (int j = 0; j < k; ++j) atomicAdd(&cnt[idx[(size_t)r * k + j]], 1);
  __syncthreads();
  if (t == 0) {
    int acc = 0, nt = 0;
    for (int e = 0; e < E; ++e) {
      base[e] = acc;
      for (int r0 = 0; r0 < cnt[e]; r0 += 64) tiles[nt++] = make_int4(e, acc + r0, min(64, cnt[e] - r0), 0);
      acc += cnt[e];
    }
    *n_tiles = nt;
  }
  for (int c0 = 0; c0 < M; c0 += 256) {
    for (int i = t; i < E * 8; i += 256) bits[i >> 3][i & 7] = 0u;
    __syncthreads();
    const int r = c0 + t;
    if (r < M)
      for (int j = 0; j < k; ++j) atomicOr(&bits[idx[(size_t)r * k + j]][t >> 5], 1u << (t & 31));
    __syncthreads();
    if (r < M)
      for (int j = 0; j < k; ++j) {
        const int e = idx[(size_t)r * k + j];
        int rank = 0;
        for (int wd = 0; wd < (t >> 5); ++wd) rank += __popc(bits[e][wd]);
        rank += __popc(bits[e][t >> 5] & ((1u << (t & 31)) - 1u));
        const int g = base[e] + rank;
        perm[g] = r;
        pos[(size_t)r * k + j] = g;
      }
    __syncthreads();
    if (t < E) {
      int c = 0;
      for (int wd = 0; wd < 8; ++wd) c += __popc(bits[t][wd]);
      base[t] += c;
    }
  }
}
hipError_t route_bucket(const int* idx, int M, int k, int E, int* perm, int* pos, int4* tiles, int* n_tiles,
                        hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_route_bucket, dim3(1), dim3(256), 0, s, idx, M, k, E, perm, pos, tiles, n_tiles);
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
__global__ void k_init_canvas(int32_t* canvas, SeedArg seeds, int n, int vocab, int canvas_index) {
  const int b = blockIdx.x;
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint4 x = philox_block(seeds.v[b], kTagInit, (uint32_t)canvas_index, 0u, (uint32_t)i, 0u);
    canvas[(size_t)b * n + i] = token_of(x.x, vocab);
  }
}
hipError_t init_canvas(int32_t* canvas, const SeedArg& seeds, int B, int n, int vocab, int canvas_index,
                       hipStream_t s) {
  hipLaunchKernelGGL(k_init_canvas, dim3(B), dim3(256), 0, s, canvas, seeds, n, vocab, canvas_index);
  return hipGetLastError();
}

#define DG_INST(T)                                                                                               \
  template hipError_t embed_norm<T>(const T*, const int32_t*, const float*, int, int, int, int, const float*,  \
                                    float, float*, T*, hipStream_t);                                            \
  template hipError_t add_norm<T>(const float*, int, int, int, const float*, float, float*, T*, hipStream_t);   \
  template hipError_t combine_norm<T>(const float*, const int*, const float*, int, int, int, const float*, float, \
                                      float*, T*, hipStream_t);                                                 \
  template hipError_t rope_scatter<T>(const float*, int, const float2*, T*, T*, T*, int, int, int, int, int, int, \
                                      int, hipStream_t);                                                        \
  template hipError_t transpose<T>(const T*, T*, int, int, hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

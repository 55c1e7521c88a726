// Row-wise kernels of the denoise step: embedding gather, RMSNorm, RoPE with
// the KV-cache write, the MoE router (top-k, lowest expert id on ties, softmax
// over the k selected logits), a stable counting sort of the routed rows by
// expert, the fixed-order combine of expert outputs, and canvas initialisation.
#include "dg_kernels.h"

namespace dg {

// ------------------------------------------------------------------ embedding
template <typename T>
__global__ void k_embed(const T* emb, const int32_t* tok, float* H, int d, int vocab) {
  const int r = blockIdx.x;
  const int id = min(max(tok[r], 0), vocab - 1);   // out-of-range ids are clamped, never read past E
  const T* src = emb + (size_t)id * d;
  for (int c = threadIdx.x; c < d; c += blockDim.x) H[(size_t)r * d + c] = Num<T>::load(src + c);
}
template <typename T>
hipError_t embed_rows(const T* emb, const int32_t* tok, float* H, int M, int d, int vocab, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_embed<T>), dim3(M), dim3(256), 0, s, emb, tok, H, d, vocab);
  return hipGetLastError();
}

// ------------------------------------------------------------------ RMSNorm
// y = x * g / sqrt(mean(x^2) + eps), rounded to the operand type; one wave per row.
template <typename T>
__global__ __launch_bounds__(256) void k_rmsnorm(const float* H, const float* g, T* out, int M, int d,
                                                 float eps) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  const float* x = H + (size_t)r * d;
  float ss = 0.f;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
  }
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)d + eps);
  T* o = out + (size_t)r * d;
  for (int c = lane * 4; c < d; c += 256) {
    const float4 v = *reinterpret_cast<const float4*>(x + c);
    const float4 gg = *reinterpret_cast<const float4*>(g + c);
    Num<T>::store(o + c + 0, v.x * inv * gg.x);
    Num<T>::store(o + c + 1, v.y * inv * gg.y);
    Num<T>::store(o + c + 2, v.z * inv * gg.z);
    Num<T>::store(o + c + 3, v.w * inv * gg.w);
  }
}
template <typename T>
hipError_t rmsnorm_rows(const float* H, const float* g, T* out, int M, int d, float eps, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_rmsnorm<T>), dim3((M + 3) / 4), dim3(256), 0, s, H, g, out, M, d, eps);
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

// Rotate-half RoPE on the fused projection output (fp32), then round: q to the
// query buffer, k and v to the cache at position ctx + i.
template <typename T>
__global__ void k_rope_scatter(const float* qkv, const float2* rope, T* q, T* kc, T* vc, int n, int Hq,
                               int Hkv, int hd, int max_ctx, int ctx) {
  const int r = blockIdx.x, b = r / n, i = r % n, pos = ctx + i, half = hd / 2;
  const int ncol = (Hq + 2 * Hkv) * hd;
  const float* x = qkv + (size_t)r * ncol;
  const float2* cs = rope + (size_t)pos * half;
  for (int u = threadIdx.x; u < (Hq + Hkv) * half; u += blockDim.x) {
    const int head = u / half, j = u % half;
    const float a = x[head * hd + j], bb = x[head * hd + j + half];
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
    Num<T>::store(vc + (((size_t)b * Hkv + kh) * max_ctx + pos) * hd + c, x[(Hq + Hkv) * hd + u]);
  }
}
template <typename T>
hipError_t rope_scatter(const float* qkv, const float2* rope, T* q, T* kc, T* vc, int B, int n, int Hq,
                        int Hkv, int hd, int max_ctx, int ctx, hipStream_t s) {
  if (B * n <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_rope_scatter<T>), dim3(B * n), dim3(256), 0, s, qkv, rope, q, kc, vc, n, Hq, Hkv,
                     hd, max_ctx, ctx);
  return hipGetLastError();
}

// ------------------------------------------------------------------ router
// One thread per row: k passes of an arg-max over the E logits (strict > keeps
// the lowest id among equal values), then softmax over the selected logits.
__global__ void k_router_topk(const float* logits, int M, int E, int k, int* idx, float* w) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= M) return;
  const float* x = logits + (size_t)r * E;
  uint32_t used[4] = {0u, 0u, 0u, 0u};
  float sel[8];
  int sid[8];
  for (int j = 0; j < k; ++j) {
    float best = -INFINITY;
    int bi = -1;
    for (int e = 0; e < E; ++e) {
      if ((used[e >> 5] >> (e & 31)) & 1u) continue;
      const float v = x[e];
      if (bi < 0 || v > best) { best = v; bi = e; }
    }
    used[bi >> 5] |= 1u << (bi & 31);
    sel[j] = best;
    sid[j] = bi;
  }
  const float mx = sel[0];   // selection order is descending, so slot 0 holds the max
  float sum = 0.f;
  for (int j = 0; j < k; ++j) { sel[j] = expf(sel[j] - mx); sum += sel[j]; }
  for (int j = 0; j < k; ++j) {
    idx[(size_t)r * k + j] = sid[j];
    w[(size_t)r * k + j] = sel[j] / sum;
  }
}
hipError_t router_topk(const float* logits, int M, int E, int k, int* idx, float* w, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_router_topk, dim3((M + 127) / 128), dim3(128), 0, s, logits, M, E, k, idx, w);
  return hipGetLastError();
}

// ------------------------------------------------------------------ bucketing
// Stable counting sort of (row, slot) entries by expert, rows in chunks of 256:
// (1) per-chunk expert counts, (2) one workgroup scans them into per-chunk
// bases and writes the 64-row tile list, (3) each entry's rank among the
// chunk's earlier rows for the same expert comes from an LDS bitmask.
__global__ __launch_bounds__(256) void k_route_count(const int* idx, int M, int k, int E, int* cc) {
  __shared__ int cnt[128];
  const int chunk = blockIdx.x, r = chunk * 256 + threadIdx.x;
  if (threadIdx.x < E) cnt[threadIdx.x] = 0;
  __syncthreads();
  if (r < M)
    for (int j = 0; j < k; ++j) atomicAdd(&cnt[idx[(size_t)r * k + j]], 1);
  __syncthreads();
  if (threadIdx.x < E) cc[chunk * E + threadIdx.x] = cnt[threadIdx.x];
}

__global__ __launch_bounds__(128) void k_route_scan(int* cc, int nchunks, int E, int4* tiles, int* n_tiles) {
  __shared__ int tot[128], off[129];
  const int e = threadIdx.x;
  if (e < E) {
    int t = 0;
    for (int c = 0; c < nchunks; ++c) t += cc[c * E + e];
    tot[e] = t;
  }
  __syncthreads();
  if (e == 0) {
    int acc = 0, nt = 0;
    for (int x = 0; x < E; ++x) {
      off[x] = acc;
      for (int r0 = 0; r0 < tot[x]; r0 += 64) tiles[nt++] = make_int4(x, acc + r0, min(64, tot[x] - r0), 0);
      acc += tot[x];
    }
    off[E] = acc;
    *n_tiles = nt;
  }
  __syncthreads();
  if (e < E) {
    int base = off[e];
    for (int c = 0; c < nchunks; ++c) {
      const int v = cc[c * E + e];
      cc[c * E + e] = base;
      base += v;
    }
  }
}

__global__ __launch_bounds__(256) void k_route_scatter(const int* idx, int M, int k, int E, const int* base,
                                                       int* perm, int* pos) {
  __shared__ uint32_t bits[128][8];
  const int chunk = blockIdx.x, t = threadIdx.x, r = chunk * 256 + t;
  for (int i = t; i < E * 8; i += 256) bits[i >> 3][i & 7] = 0u;
  __syncthreads();
  if (r < M)
    for (int j = 0; j < k; ++j) atomicOr(&bits[idx[(size_t)r * k + j]][t >> 5], 1u << (t & 31));
  __syncthreads();
  if (r >= M) return;
  for (int j = 0; j < k; ++j) {
    const int e = idx[(size_t)r * k + j];
    int rank = 0;
    for (int wd = 0; wd < (t >> 5); ++wd) rank += __popc(bits[e][wd]);
    rank += __popc(bits[e][t >> 5] & ((1u << (t & 31)) - 1u));
    const int g = base[chunk * E + e] + rank;
    perm[g] = r;
    pos[(size_t)r * k + j] = g;
  }
}

hipError_t route_bucket(const int* idx, int M, int k, int E, int* chunk_counts, int* perm, int* pos,
                        int4* tiles, int* n_tiles, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int nchunks = (M + 255) / 256;
  hipLaunchKernelGGL(k_route_count, dim3(nchunks), dim3(256), 0, s, idx, M, k, E, chunk_counts);
  hipLaunchKernelGGL(k_route_scan, dim3(1), dim3(128), 0, s, chunk_counts, nchunks, E, tiles, n_tiles);
  hipLaunchKernelGGL(k_route_scatter, dim3(nchunks), dim3(256), 0, s, idx, M, k, E, chunk_counts, perm, pos);
  return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// H[r] += sum_j w[r][j] * Y[pos[r][j]], slots in selection order.
__global__ void k_moe_combine(const float* Y, const int* pos, const float* w, float* H, int k, int d) {
  const int r = blockIdx.x;
  for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; ++j) {
      const float wj = w[(size_t)r * k + j];
      const float4 y = *reinterpret_cast<const float4*>(Y + (size_t)pos[(size_t)r * k + j] * d + c);
      acc.x += wj * y.x; acc.y += wj * y.y; acc.z += wj * y.z; acc.w += wj * y.w;
    }
    float4* h = reinterpret_cast<float4*>(H + (size_t)r * d + c);
    float4 hv = *h;
    hv.x += acc.x; hv.y += acc.y; hv.z += acc.z; hv.w += acc.w;
    *h = hv;
  }
}
hipError_t moe_combine(const float* Y, const int* pos, const float* w, float* H, int M, int k, int d,
                       hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_moe_combine, dim3(M), dim3(256), 0, s, Y, pos, w, H, k, d);
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

#define DG_INST(T)                                                                                   \
  template hipError_t embed_rows<T>(const T*, const int32_t*, float*, int, int, int, hipStream_t);  \
  template hipError_t rmsnorm_rows<T>(const float*, const float*, T*, int, int, float, hipStream_t); \
  template hipError_t rope_scatter<T>(const float*, const float2*, T*, T*, T*, int, int, int, int,  \
                                      int, int, int, hipStream_t);                                  \
  template hipError_t transpose<T>(const T*, T*, int, int, hipStream_t);
DG_INST(float)
DG_INST(bf16)
#undef DG_INST

}  // namespace dg

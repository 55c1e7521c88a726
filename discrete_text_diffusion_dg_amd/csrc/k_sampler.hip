// Sampler of the denoise step ([mlqm] 四: entropy-ordered commit with a 0.1 nat
// running bound, uniform re-randomisation of the rest, temperature 0.8 -> 0.4,
// adaptive stop; [mlqm] 一: multinomial diffusion replaces an uncertain
// position by any vocabulary token).
//
// Head statistics are computed in one read of the logits: each workgroup owns
// one (row, vocab chunk); it keeps its z = logit / T values in registers, takes
// the chunk max, the logit argmax and the Gumbel-max top two (Philox draws,
// four vocabulary ids per call), then sums exp(z - m) and exp(z - m)(z - m),
// and writes exp(z - m) rounded to the operand type for the self-conditioning
// contraction.  A merge pass combines the chunks of a row in order.
#include "dg_kernels.h"

namespace dg {

namespace {
constexpr int kChunkMax = 4096;         // vocabulary ids per workgroup (16 per thread)
constexpr int kPerThread = kChunkMax / 256;
}

int sampler_chunks(int vocab) {
  int c = (vocab + kChunkMax - 1) / kChunkMax;
  return c < 1 ? 1 : c;
}
// chunk length: a multiple of 64 so that split-K slices of the contraction align
static __host__ __device__ inline int chunk_len(int vocab, int chunks) {
  const int per = (vocab + chunks - 1) / chunks;
  return (per + 63) / 64 * 64;
}

struct Top2 {
  float b1; int i1; float b2;
};
__device__ __forceinline__ void top2_merge(Top2& a, const Top2& o) {
  if (o.b1 > a.b1 || (o.b1 == a.b1 && o.i1 < a.i1)) {
    a.b2 = fmaxf(a.b1, o.b2);
    a.b1 = o.b1; a.i1 = o.i1;
  } else {
    a.b2 = fmaxf(a.b2, o.b1);
  }
}
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) { v = ov; i = oi; }
}

// Four consecutive values in one store (8 bytes bf16, 16 bytes fp32).
__device__ __forceinline__ void store4(bf16* p, const float* e) {
  uint2 u;
  u.x = f32x2_to_bf16x2(e[0], e[1]);
  u.y = f32x2_to_bf16x2(e[2], e[3]);
  *reinterpret_cast<uint2*>(p) = u;
}
__device__ __forceinline__ void store4(float* p, const float* e) {
  *reinterpret_cast<float4*>(p) = make_float4(e[0], e[1], e[2], e[3]);
}

template <typename T>
__global__ __launch_bounds__(256) void k_sampler_partial(const float* logits, int V, int chunks, int clen,
                                                         float inv_t, SeedArg seeds, int n,
                                                         int canvas_index, int step, HeadPart* part,
                                                         T* ptilde) {
  __shared__ float red_f[3][4];
  __shared__ int red_i[2][4];
  __shared__ float red_b2[4];
  const int chunk = blockIdx.x, row = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int b = row / n, pos = row % n;
  const int v0 = chunk * clen, v1 = min(V, v0 + clen);
  const float* L = logits + (size_t)row * V;
  const uint64_t seed = seeds.v[b];

  float z[kPerThread];
  float zmax = -INFINITY, lmax = -INFINITY;
  int lidx = 0x7fffffff;
  Top2 t2{-INFINITY, 0x7fffffff, -INFINITY};
  // every load is issued unconditionally (addresses clamped into the chunk, the
  // values past its end masked) so that all of them are in flight together
  float4 l4[kPerThread / 4];
#pragma unroll
  for (int it = 0; it < kPerThread / 4; ++it) {
    const int v = min(v0 + (it * 256 + tid) * 4, v1 - 4);
    l4[it] = *reinterpret_cast<const float4*>(L + v);
  }
  // logit arg-max and the max of z over all of the thread's values
#pragma unroll
  for (int it = 0; it < kPerThread / 4; ++it) {
    const int v = v0 + (it * 256 + tid) * 4;
    const bool ok = v < v1;
    const float lv[4] = {l4[it].x, l4[it].y, l4[it].z, l4[it].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float zz = ok ? lv[j] * inv_t : -INFINITY;
      z[it * 4 + j] = zz;
      zmax = fmaxf(zmax, zz);
      if (ok) argmax_merge(lmax, lidx, lv[j], v + j);
    }
  }
  // Gumbel-max top two.  The first four values of every lane are scored
  // exactly; the wave's second-best score b2 and largest z then bound the rest:
  // a value can enter the chunk's top two only if its Gumbel noise exceeds
  // b2 - max z, i.e. only if its uniform exceeds exp(-exp(-(b2 - max z))) -- a
  // threshold on the raw Philox word (lowered by a 1e-3 margin on the score,
  // far above fp32 rounding).  Values under it cannot change the top two, so
  // they skip the two logarithms.
  auto score = [&](int it, const uint4& x, uint32_t qmin) {
    const int v = v0 + (it * 256 + tid) * 4;
    if (v >= v1) return;
    const uint32_t xv[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if ((xv[j] >> 9) >= qmin) top2_merge(t2, Top2{z[it * 4 + j] + gumbel_of(xv[j]), v + j, -INFINITY});
  };
  score(0, philox_block(seed, kTagGumbel, (uint32_t)canvas_index, (uint32_t)step, (uint32_t)pos,
                        (uint32_t)((v0 + tid * 4) >> 2)), 0u);
  uint32_t qmin = 0;
  {
    Top2 tw = t2;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      top2_merge(tw, Top2{__shfl_xor(tw.b1, o, 64), __shfl_xor(tw.i1, o, 64), __shfl_xor(tw.b2, o, 64)});
    const float delta = tw.b2 - wave_max(zmax) - 1e-3f;
    if (delta > -INFINITY) {
      const float uthr = expf(-expf(-delta));                 // prune when u < uthr
      const float q = floorf(uthr * 8388608.f - 0.5f) - 1.f;  // u = (2q + 1) 2^-24 < uthr for q < qmin
      qmin = q > 0.f ? (uint32_t)q : 0u;
    }
  }
#pragma unroll
  for (int it = 1; it < kPerThread / 4; ++it) {
    const int v = v0 + (it * 256 + tid) * 4;
    score(it, philox_block(seed, kTagGumbel, (uint32_t)canvas_index, (uint32_t)step, (uint32_t)pos,
                           (uint32_t)(v >> 2)), qmin);
  }
  // workgroup reductions (fixed order)
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    zmax = fmaxf(zmax, __shfl_xor(zmax, o, 64));
    const float ol = __shfl_xor(lmax, o, 64);
    const int oi = __shfl_xor(lidx, o, 64);
    argmax_merge(lmax, lidx, ol, oi);
    Top2 ot{__shfl_xor(t2.b1, o, 64), __shfl_xor(t2.i1, o, 64), __shfl_xor(t2.b2, o, 64)};
    top2_merge(t2, ot);
  }
  if (lane == 0) {
    red_f[0][w] = zmax; red_f[1][w] = lmax; red_f[2][w] = t2.b1;
    red_i[0][w] = lidx; red_i[1][w] = t2.i1; red_b2[w] = t2.b2;
  }
  __syncthreads();
  zmax = red_f[0][0];
  lmax = red_f[1][0]; lidx = red_i[0][0];
  t2 = Top2{red_f[2][0], red_i[1][0], red_b2[0]};
  for (int q = 1; q < 4; ++q) {
    zmax = fmaxf(zmax, red_f[0][q]);
    argmax_merge(lmax, lidx, red_f[1][q], red_i[0][q]);
    top2_merge(t2, Top2{red_f[2][q], red_i[1][q], red_b2[q]});
  }
  __syncthreads();

  float s = 0.f, ws = 0.f;
#pragma unroll
  for (int it = 0; it < kPerThread / 4; ++it) {
    const int v = v0 + (it * 256 + tid) * 4;
    if (v < v1) {
      float e4[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float dz = z[it * 4 + j] - zmax;
        const float e = expf(dz);
        e4[j] = e;
        s += e;
        ws += e * dz;
      }
      if (ptilde != nullptr) store4(ptilde + (size_t)row * V + v, e4);
    }
  }
  s = wave_sum(s);
  ws = wave_sum(ws);
  if (lane == 0) { red_f[0][w] = s; red_f[1][w] = ws; }
  __syncthreads();
  if (tid == 0) {
    s = red_f[0][0] + red_f[0][1] + red_f[0][2] + red_f[0][3];
    ws = red_f[1][0] + red_f[1][1] + red_f[1][2] + red_f[1][3];
    HeadPart hp;
    hp.m = zmax; hp.s = s; hp.w = ws; hp.lmax = lmax; hp.lidx = lidx;
    hp.g1 = t2.b1; hp.gidx = t2.i1; hp.g2 = t2.b2;
    part[(size_t)row * chunks + chunk] = hp;
  }
}

// One wave per row, lane c holding chunk c (chunks <= 64): the chunk statistics
// combine in fp64 through a fixed butterfly, so the result does not depend on
// scheduling; arg-max and Gumbel top-two merges are order-free.
__global__ __launch_bounds__(256) void k_sampler_merge(const HeadPart* part, int M, int chunks, int n,
                                                       const uint8_t* active, float* H, int32_t* y, int32_t* am,
                                                       float* margin, float* chunk_scale) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  const bool has = lane < chunks;
  HeadPart p;
  if (has) p = part[(size_t)r * chunks + lane];
  else { p.m = -INFINITY; p.s = 0.f; p.w = 0.f; p.lmax = -INFINITY; p.lidx = 0x7fffffff;
         p.g1 = -INFINITY; p.gidx = 0x7fffffff; p.g2 = -INFINITY; }
  const float mf = wave_max(p.m);
  const double m = (double)mf;
  const double f = has ? exp((double)p.m - m) : 0.0;
  double S = (double)p.s * f;
  double W = has ? f * ((double)p.w + ((double)p.m - m) * (double)p.s) : 0.0;
  float lmax = p.lmax;
  int lidx = p.lidx;
  Top2 t2{p.g1, p.gidx, p.g2};
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    S += __shfl_xor(S, o, 64);
    W += __shfl_xor(W, o, 64);
    argmax_merge(lmax, lidx, __shfl_xor(lmax, o, 64), __shfl_xor(lidx, o, 64));
    top2_merge(t2, Top2{__shfl_xor(t2.b1, o, 64), __shfl_xor(t2.i1, o, 64), __shfl_xor(t2.b2, o, 64)});
  }
  if (chunk_scale != nullptr && has) chunk_scale[(size_t)r * chunks + lane] = (float)(f / S);
  if (lane != 0 || (active != nullptr && active[r / n] == 0)) return;
  H[r] = (float)(log(S) - W / S);
  y[r] = t2.i1;
  am[r] = lidx;
  margin[r] = t2.b1 - t2.b2;
}

// s[r][c] = sum over chunks of scale[r][chunk] * (sum of the chunk's `sub` K-slice
// partials, slice order).  Four columns per thread; the partial loads of up to
// four chunks are issued together.
__global__ __launch_bounds__(256) void k_selfcond_reduce(const float* part, const float* chunk_scale, int M, int d,
                                                         int chunks, int sub, float* S) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;      // float4 index
  const size_t nq = (size_t)M * d / 4;
  if (q >= nq) return;
  const size_t r = q * 4 / d;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int c0 = 0; c0 < chunks; c0 += 4) {
    float4 pc[4];
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      pc[cc] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (c0 + cc < chunks)
        for (int u = 0; u < sub; ++u) {
          const float4 v = p4[(size_t)((c0 + cc) * sub + u) * nq + q];
          pc[cc].x += v.x; pc[cc].y += v.y; pc[cc].z += v.z; pc[cc].w += v.w;
        }
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
      if (c0 + cc < chunks) {
        const float sc = chunk_scale[r * chunks + c0 + cc];
        acc.x += sc * pc[cc].x; acc.y += sc * pc[cc].y; acc.z += sc * pc[cc].z; acc.w += sc * pc[cc].w;
      }
  }
  reinterpret_cast<float4*>(S)[q] = acc;
}

// ------------------------------------------------------------------ commit
// One workgroup per request: bitonic sort of (H, position), fp64 running total
// in sorted order (thread 0, sequential, so the rounding is fixed), then every
// position takes y or a fresh uniform token.
__global__ __launch_bounds__(256) void k_commit(const float* H, const int32_t* y, const int32_t* am,
                                                int32_t* canvas, int32_t* prev_am, uint8_t* mask,
                                                int32_t* n_committed, uint8_t* done, SeedArg seeds, int n,
                                                int vocab, int step, int max_steps, float bound,
                                                int stop_mode, float tau, int canvas_index) {
  __shared__ float sh[256];
  __shared__ float hpos[256];
  __shared__ int sp[256];
  __shared__ int rank[256];
  __shared__ int s_cnt, s_final, s_diff;
  const int b = blockIdx.x, t = threadIdx.x;
  if (done[b]) return;
  const size_t base = (size_t)b * n;
  sh[t] = t < n ? H[base + t] : INFINITY;
  hpos[t] = sh[t];
  sp[t] = t;
  if (t == 0) s_diff = 0;
  __syncthreads();
  if (t < n && stop_mode == 2 && am[base + t] != prev_am[base + t]) s_diff = 1;
  for (int k = 2; k <= 256; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      const int o = t ^ j;
      if (o > t) {
        const bool asc = (t & k) == 0;
        const float ha = sh[t], hb = sh[o];
        const int pa = sp[t], pb = sp[o];
        const bool gt = ha > hb || (ha == hb && pa > pb);
        if (gt == asc) { sh[t] = hb; sh[o] = ha; sp[t] = pb; sp[o] = pa; }
      }
      __syncthreads();
    }
  }
  rank[sp[t]] = t;
  if (t == 0) {
    const double bnd = (double)bound;
    double c = 0.0;
    int cnt = 0;
    for (int j = 0; j < n; ++j) {
      c += (double)sh[j];
      if (c <= bnd) ++cnt; else break;
    }
    double mean = 0.0;
    for (int i = 0; i < n; ++i) mean += (double)hpos[i];
    mean /= (double)n;
    bool stop = false;
    if (stop_mode == 1) stop = mean < (double)tau;
    else if (stop_mode == 2) stop = mean < (double)tau && step > 0 && s_diff == 0;
    const bool fin = stop || step >= max_steps - 1;
    s_cnt = cnt;
    s_final = fin ? 1 : 0;
  }
  __syncthreads();
  if (t < n) {
    const bool fin = s_final != 0;
    const bool keep = fin || rank[t] < s_cnt;
    int32_t tok = y[base + t];
    if (!keep) {
      const uint4 x = philox_block(seeds.v[b], kTagRenoise, (uint32_t)canvas_index, (uint32_t)step,
                                   (uint32_t)t, 0u);
      tok = token_of(x.x, vocab);
    }
    canvas[base + t] = tok;
    mask[base + t] = keep ? 1 : 0;
    prev_am[base + t] = am[base + t];
  }
  if (t == 0) {
    n_committed[b] = s_final ? n : s_cnt;
    done[b] = (uint8_t)s_final;
  }
}

}  // namespace dg

namespace dg {

template <typename T>
hipError_t sampler_partial(const float* logits, int M, int V, int chunks, float inv_t, const SeedArg& seeds,
                           int n, int canvas_index, int step, HeadPart* part, T* ptilde, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const int clen = chunk_len(V, chunks);
  if (clen > kChunkMax) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_sampler_partial<T>), dim3(chunks, M), dim3(256), 0, s, logits, V, chunks, clen, inv_t,
                     seeds, n, canvas_index, step, part, ptilde);
  return hipGetLastError();
}

hipError_t sampler_merge(const HeadPart* part, int M, int chunks, int n, const uint8_t* active, float* H,
                         int32_t* y, int32_t* am, float* margin, float* chunk_scale, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_sampler_merge, dim3((M + 3) / 4), dim3(256), 0, s, part, M, chunks, n, active, H, y,
                     am, margin, chunk_scale);
  return hipGetLastError();
}

hipError_t selfcond_reduce(const float* part, const float* chunk_scale, int M, int d, int chunks, int sub, float* S,
                           hipStream_t s) {
  const size_t nq = (size_t)M * d / 4;      // d is a multiple of 256
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_selfcond_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, part, chunk_scale,
                     M, d, chunks, sub, S);
  return hipGetLastError();
}

hipError_t commit_kernel(const float* H, const int32_t* y, const int32_t* am, int32_t* canvas, int32_t* prev_am,
                         uint8_t* mask, int32_t* n_committed, uint8_t* done, const SeedArg& seeds, int B, int n,
                         int vocab, int step, int max_steps, float bound, int stop_mode, float tau,
                         int canvas_index, hipStream_t s) {
  hipLaunchKernelGGL(k_commit, dim3(B), dim3(256), 0, s, H, y, am, canvas, prev_am, mask, n_committed, done, seeds,
                     n, vocab, step, max_steps, bound, stop_mode, tau, canvas_index);
  return hipGetLastError();
}

int sampler_chunk_len(int vocab, int chunks) { return chunk_len(vocab, chunks); }

template hipError_t sampler_partial<float>(const float*, int, int, int, float, const SeedArg&, int, int, int,
                                           HeadPart*, float*, hipStream_t);
template hipError_t sampler_partial<bf16>(const float*, int, int, int, float, const SeedArg&, int, int, int,
                                          HeadPart*, bf16*, hipStream_t);

}  // namespace dg

// Sampler of the denoise step ([mlqm] 四: entropy-ordered commit with a 0.1 nat
// running bound, uniform re-randomisation of the rest, temperature 0.8 -> 0.4,
// adaptive stop; [mlqm] 一: multinomial diffusion replaces an uncertain
// position by any vocabulary token).
//
// Head statistics per (row, 128-id chunk) come from the LM-head epilogue; for
// supplied logits, k_head_logits stages the same 128 x 128 tiles through LDS
// and runs the same code (dg_head.h).  A merge pass combines the chunks of a
// row in order; the self-conditioning contraction scales each chunk's
// exp(z - m) in its operand loader, so its split partials add plainly.
#include "dg_head.h"

namespace dg {

int head_chunks(int vocab) { return (vocab + kHeadChunk - 1) / kHeadChunk; }

// One workgroup per 128 x 128 tile of supplied fp32 logits [M][V].
template <typename T>
__global__ __launch_bounds__(256) void k_head_logits(const float* logits, int M, int V, float inv_t, SeedArg seeds,
                                                     int n, int canvas_index, int step, HeadPart* part, int nchunk,
                                                     T* ptilde) {
  __shared__ __attribute__((aligned(16))) float tile[kHeadChunk * kHeadLd];
  const int n0 = blockIdx.x * kHeadChunk, m0 = blockIdx.y * kHeadChunk;
  const int rows = min(kHeadChunk, M - m0), cols = min(kHeadChunk, V - n0);
  // 32 float4 per tile row: all loads issued together, rows / ids past the end read as 0
  float4 v[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q = threadIdx.x + 256 * i, r = q >> 5, c = (q & 31) * 4;
    v[i] = r < rows && c < cols ? *reinterpret_cast<const float4*>(logits + (size_t)(m0 + r) * V + n0 + c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int q = threadIdx.x + 256 * i, r = q >> 5, c = (q & 31) * 4;
    *reinterpret_cast<float4*>(tile + r * kHeadLd + c) = v[i];
  }
  __syncthreads();
  head_tile_stats<T>(tile, m0, rows, n0, cols, V, inv_t, seeds, n, canvas_index, step, part, nchunk, ptilde);
}

// One workgroup per row; thread t holds chunks t, t + 256, ... (CPT of them) in
// registers: first the row max of the chunk maxima (and the order-free arg-max
// and Gumbel top-two merges), then its chunks' sums in fp64 in chunk order,
// combined by a fixed butterfly per wave and the four waves in wave order -- the
// result does not depend on scheduling -- and last the per-chunk scales
// exp(m_c - M) / S that turn each chunk's exp(z - m_c) into probabilities.
template <int CPT>
__global__ __launch_bounds__(256) void k_sampler_merge(const HeadPart* part, int chunks, int n, const uint8_t* active,
                                                       float* H, int32_t* y, int32_t* am, float* margin,
                                                       float* chunk_scale) {
  __shared__ float sm_m[4], sm_l[4], sm_g1[4], sm_g2[4];
  __shared__ int sm_li[4], sm_gi[4];
  __shared__ double sm_S[4], sm_W[4];
  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const HeadPart* pr = part + (size_t)r * chunks;
  HeadPart p[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int c = t + 256 * j;
    if (c < chunks) p[j] = pr[c];
    else { p[j].m = -INFINITY; p[j].s = 0.f; p[j].w = 0.f; p[j].lmax = -INFINITY; p[j].lidx = 0x7fffffff;
           p[j].g1 = -INFINITY; p[j].gidx = 0x7fffffff; p[j].g2 = -INFINITY; }
  }
  float mloc = -INFINITY, lmax = -INFINITY;
  int lidx = 0x7fffffff;
  Top2 t2{-INFINITY, 0x7fffffff, -INFINITY};
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    mloc = fmaxf(mloc, p[j].m);
    argmax_merge(lmax, lidx, p[j].lmax, p[j].lidx);
    top2_merge(t2, Top2{p[j].g1, p[j].gidx, p[j].g2});
  }
  mloc = wave_max(mloc);
  butterfly_steps([&](auto st) {
    constexpr int S = decltype(st)::value;
    argmax_merge(lmax, lidx, lane_partner<S>(lmax), lane_partner<S>(lidx));
    top2_merge(t2, Top2{lane_partner<S>(t2.b1), lane_partner<S>(t2.i1), lane_partner<S>(t2.b2)});
  });
  if (lane == 0) {
    sm_m[wv] = mloc; sm_l[wv] = lmax; sm_li[wv] = lidx; sm_g1[wv] = t2.b1; sm_gi[wv] = t2.i1; sm_g2[wv] = t2.b2;
  }
  __syncthreads();
  const double m = (double)fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
  double S = 0.0, W = 0.0;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    if (p[j].m == -INFINITY) continue;
    const double f = exp((double)p[j].m - m);
    S += (double)p[j].s * f;
    W += f * ((double)p[j].w + ((double)p[j].m - m) * (double)p[j].s);
  }
  butterfly_steps([&](auto st) {
    S += lane_partner<decltype(st)::value>(S);
    W += lane_partner<decltype(st)::value>(W);
  });
  if (lane == 0) { sm_S[wv] = S; sm_W[wv] = W; }
  __syncthreads();
  S = ((sm_S[0] + sm_S[1]) + sm_S[2]) + sm_S[3];
  W = ((sm_W[0] + sm_W[1]) + sm_W[2]) + sm_W[3];
  if (chunk_scale != nullptr) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int c = t + 256 * j;
      if (c < chunks)
        chunk_scale[(size_t)r * chunks + c] = p[j].m == -INFINITY ? 0.f : (float)(exp((double)p[j].m - m) / S);
    }
  }
  if (t != 0 || (active != nullptr && active[r / n] == 0)) return;
  lmax = sm_l[0]; lidx = sm_li[0];
  t2 = Top2{sm_g1[0], sm_gi[0], sm_g2[0]};
  for (int q = 1; q < 4; ++q) {
    argmax_merge(lmax, lidx, sm_l[q], sm_li[q]);
    top2_merge(t2, Top2{sm_g1[q], sm_gi[q], sm_g2[q]});
  }
  H[r] = (float)(log(S) - W / S);
  y[r] = t2.i1;
  am[r] = lidx;
  margin[r] = t2.b1 - t2.b2;
}

// s[r][c] = sum of the split partials in split order, four columns per thread,
// the loads of up to eight splits issued together.
__global__ __launch_bounds__(256) void k_selfcond_reduce(const float* part, int M, int d, int splits, float* S) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;      // float4 index
  const size_t nq = (size_t)M * d / 4;
  if (q >= nq) return;
  const float4* p4 = reinterpret_cast<const float4*>(part);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = 0; s0 < splits; s0 += 8) {
    float4 pc[8];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < splits) pc[u] = p4[(size_t)(s0 + u) * nq + q];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (s0 + u < splits) { acc.x += pc[u].x; acc.y += pc[u].y; acc.z += pc[u].z; acc.w += pc[u].w; }
  }
  reinterpret_cast<float4*>(S)[q] = acc;
}

// ------------------------------------------------------------------ commit
// Value of lane (lane ^ J) for J < 64: quad permutes for 1 and 2, row shifts
// for 4 and 8 (the partner lies J lanes up or down inside the row of 16), the
// gfx950 row swaps for 16 and 32.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int lane = threadIdx.x & 63;
  if constexpr (J == 1 || J == 2 || J == 16 || J == 32) {
    return lane_partner<J == 1 ? 0 : J == 2 ? 1 : J == 16 ? 4 : 5>(v);
  } else {
    static_assert(J == 4 || J == 8, "lane distance");
    const uint32_t up = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x100 + J, 0xF, 0xF, false);   // row_shl: lane + J
    const uint32_t dn = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x110 + J, 0xF, 0xF, false);   // row_shr: lane - J
    return (lane & J) ? dn : up;
  }
}

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
  const size_t base = (size_t)b * n;
  // every input of this position is requested at once (a finished request
  // returns after its loads, before any barrier)
  const uint8_t fin_before = done[b];
  const float h_in = t < n ? H[base + t] : INFINITY;
  const int32_t y_t = t < n ? y[base + t] : 0, am_t = t < n ? am[base + t] : 0;
  const int32_t pam_t = t < n ? prev_am[base + t] : 0;
  if (fin_before) return;
  sh[t] = h_in;
  hpos[t] = h_in;
  if (t == 0) s_diff = 0;
  __syncthreads();
  if (t < n && stop_mode == 2 && am_t != pam_t) s_diff = 1;
  // bitonic sort of (H, position) over the 256 threads, ascending; thread i
  // holds element i.  Partners within a wave (distance < 64) are exchanged by
  // lane moves, the others through LDS.
  float kh = sh[t];
  int kp = t;
  auto cmpx = [&](int k, int j, float ph, int pp) __attribute__((always_inline)) {
    const bool asc = (t & k) == 0, lower = (t & j) == 0;
    const bool gt = kh > ph || (kh == ph && kp > pp);      // this element orders after its partner
    if ((lower == asc) == gt) { kh = ph; kp = pp; }        // keep the smaller (or larger) of the pair
  };
  auto step_lds = [&](int k, int j) __attribute__((always_inline)) {
    sh[t] = kh; sp[t] = kp;
    __syncthreads();
    const float ph = sh[t ^ j];
    const int pp = sp[t ^ j];
    __syncthreads();
    cmpx(k, j, ph, pp);
  };
  auto step_lane = [&](int k, auto jc) __attribute__((always_inline)) {
    constexpr int J = decltype(jc)::value;
    const float ph = __uint_as_float(xor_lane<J>(__float_as_uint(kh)));
    const int pp = (int)xor_lane<J>((uint32_t)kp);
    cmpx(k, J, ph, pp);
  };
  auto lanes_from = [&](int k, int jtop) __attribute__((always_inline)) {   // steps j = jtop .. 1 (jtop < 64)
    if (jtop >= 32) step_lane(k, std::integral_constant<int, 32>{});
    if (jtop >= 16) step_lane(k, std::integral_constant<int, 16>{});
    if (jtop >= 8) step_lane(k, std::integral_constant<int, 8>{});
    if (jtop >= 4) step_lane(k, std::integral_constant<int, 4>{});
    if (jtop >= 2) step_lane(k, std::integral_constant<int, 2>{});
    step_lane(k, std::integral_constant<int, 1>{});
  };
  for (int k = 2; k <= 64; k <<= 1) lanes_from(k, k >> 1);
  step_lds(128, 64);
  lanes_from(128, 32);
  step_lds(256, 128);
  step_lds(256, 64);
  lanes_from(256, 32);
  sh[t] = kh; sp[t] = kp;
  __syncthreads();
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
    int32_t tok = y_t;
    if (!keep) {
      const uint4 x = philox_block(seeds.v[b], kTagRenoise, (uint32_t)canvas_index, (uint32_t)step,
                                   (uint32_t)t, 0u);
      tok = token_of(x.x, vocab);
    }
    canvas[base + t] = tok;
    mask[base + t] = keep ? 1 : 0;
    prev_am[base + t] = am_t;
  }
  if (t == 0) {
    n_committed[b] = s_final ? n : s_cnt;
    done[b] = (uint8_t)s_final;
  }
}

}  // namespace dg

namespace dg {

template <typename T>
hipError_t head_from_logits(const float* logits, int M, int V, float inv_t, const SeedArg& seeds, int n,
                            int canvas_index, int step, HeadPart* part, T* ptilde, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (V % 64) return hipErrorInvalidValue;
  const dim3 grid(head_chunks(V), (M + kHeadChunk - 1) / kHeadChunk);
  hipLaunchKernelGGL((k_head_logits<T>), grid, dim3(256), 0, s, logits, M, V, inv_t, seeds, n, canvas_index, step,
                     part, head_chunks(V), ptilde);
  return hipGetLastError();
}

hipError_t sampler_merge(const HeadPart* part, int M, int chunks, int n, const uint8_t* active, float* H,
                         int32_t* y, int32_t* am, float* margin, float* chunk_scale, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(M), block(256);
  if (chunks <= 256)
    hipLaunchKernelGGL((k_sampler_merge<1>), grid, block, 0, s, part, chunks, n, active, H, y, am, margin, chunk_scale);
  else if (chunks <= 512)
    hipLaunchKernelGGL((k_sampler_merge<2>), grid, block, 0, s, part, chunks, n, active, H, y, am, margin, chunk_scale);
  else if (chunks <= 1024)
    hipLaunchKernelGGL((k_sampler_merge<4>), grid, block, 0, s, part, chunks, n, active, H, y, am, margin, chunk_scale);
  else if (chunks <= 2048)
    hipLaunchKernelGGL((k_sampler_merge<8>), grid, block, 0, s, part, chunks, n, active, H, y, am, margin, chunk_scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t selfcond_reduce(const float* part, int M, int d, int splits, float* S, hipStream_t s) {
  const size_t nq = (size_t)M * d / 4;      // d is a multiple of 256
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_selfcond_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, part, M, d, splits, S);
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

template hipError_t head_from_logits<float>(const float*, int, int, float, const SeedArg&, int, int, int,
                                            HeadPart*, float*, hipStream_t);
template hipError_t head_from_logits<bf16>(const float*, int, int, float, const SeedArg&, int, int, int,
                                           HeadPart*, bf16*, hipStream_t);

}  // namespace dg

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

#include <mutex>

namespace dg {

int head_chunks(int vocab) { return (vocab + kHeadChunk - 1) / kHeadChunk; }

// One workgroup per 128 x 128 tile of supplied fp32 logits [M][V].
template <typename T>
__global__ __launch_bounds__(256) void k_head_logits(const float* logits, int M, int V, StepInfo si, SeedArg seeds,
                                                     int n, HeadPart* part, int nchunk, T* ptilde, Gate g) {
  __shared__ __attribute__((aligned(16))) float tile[kHeadChunk * kHeadLd];
  const int n0 = blockIdx.x * kHeadChunk, m0 = blockIdx.y * kHeadChunk;
  const int rows = min(kHeadChunk, M - m0), cols = min(kHeadChunk, V - n0);
  if (!g.any_active(m0, rows, n)) return;
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
  head_tile_stats<T>(tile, m0, rows, n0, cols, V, si, seeds, n, part, nchunk, ptilde);
}

// One workgroup per row; thread t holds chunks t, t + 256, ... (CPT of them) in
// registers: first the row max of the chunk maxima (and the order-free arg-max
// and Gumbel top-two merges), then its chunks' sums in fp64 in chunk order,
// combined by a fixed butterfly per wave and the four waves in wave order -- the
// result does not depend on scheduling -- and last the per-chunk scales
// exp(m_c - M) / S that turn each chunk's exp(z - m_c) into probabilities.
template <int CPT>
__global__ __launch_bounds__(256) void k_sampler_merge(const HeadPart* part, int chunks, int n, Gate g,
                                                       float* H, int32_t* y, int32_t* am, float* margin,
                                                       float* chunk_scale, float* lse) {
  __shared__ float sm_m[4], sm_l[4], sm_g1[4], sm_g2[4];
  __shared__ int sm_li[4], sm_gi[4];
  __shared__ double sm_S[4], sm_W[4];
  const int r = blockIdx.x, t = threadIdx.x, lane = t & 63, wv = t >> 6;
  if (!g.active(r / n)) return;          // the whole workgroup: no barrier is reached
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
  if (t != 0) return;
  lmax = sm_l[0]; lidx = sm_li[0];
  t2 = Top2{sm_g1[0], sm_gi[0], sm_g2[0]};
  for (int q = 1; q < 4; ++q) {
    argmax_merge(lmax, lidx, sm_l[q], sm_li[q]);
    top2_merge(t2, Top2{sm_g1[q], sm_gi[q], sm_g2[q]});
  }
  if (lse != nullptr) lse[r] = (float)(m + log(S));     // log sum exp(z) of the row
  if (H == nullptr) return;
  H[r] = (float)(log(S) - W / S);
  y[r] = t2.i1;
  am[r] = lidx;
  margin[r] = t2.b1 - t2.b2;
}

// s[r][c] = sum of the split partials in split order, four columns per thread,
// the loads of up to eight splits issued together.
__global__ __launch_bounds__(256) void k_selfcond_reduce(const float* part, int M, int d, int splits, float* S,
                                                         Gate g, int n) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;      // float4 index
  const size_t nq = (size_t)M * d / 4;
  if (q >= nq || !g.active((int)(q / (d / 4)) / n)) return;
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
                                                int vocab, StepInfo si, int max_steps, float bound,
                                                int stop_mode, float tau) {
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
  const int step = si.get_step(), canvas_index = si.cidx[b];
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
hipError_t head_from_logits(const float* logits, int M, int V, const StepInfo& si, const SeedArg& seeds, int n,
                            HeadPart* part, T* ptilde, Gate g, hipStream_t s) {
  if (M <= 0) return hipSuccess;
  if (V % 64) return hipErrorInvalidValue;
  const dim3 grid(head_chunks(V), (M + kHeadChunk - 1) / kHeadChunk);
  hipLaunchKernelGGL((k_head_logits<T>), grid, dim3(256), 0, s, logits, M, V, si, seeds, n, part, head_chunks(V),
                     ptilde, g);
  return hipGetLastError();
}

hipError_t sampler_merge(const HeadPart* part, int M, int chunks, int n, Gate g, float* H,
                         int32_t* y, int32_t* am, float* margin, float* chunk_scale, hipStream_t s, float* lse) {
  if (M <= 0) return hipSuccess;
  const dim3 grid(M), block(256);
  if (chunks <= 256)
    hipLaunchKernelGGL((k_sampler_merge<1>), grid, block, 0, s, part, chunks, n, g, H, y, am, margin, chunk_scale, lse);
  else if (chunks <= 512)
    hipLaunchKernelGGL((k_sampler_merge<2>), grid, block, 0, s, part, chunks, n, g, H, y, am, margin, chunk_scale, lse);
  else if (chunks <= 1024)
    hipLaunchKernelGGL((k_sampler_merge<4>), grid, block, 0, s, part, chunks, n, g, H, y, am, margin, chunk_scale, lse);
  else if (chunks <= 2048)
    hipLaunchKernelGGL((k_sampler_merge<8>), grid, block, 0, s, part, chunks, n, g, H, y, am, margin, chunk_scale, lse);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ------------------------------------------------------------------ top-k truncated sampler
// Branch-free insertion into a descending list of (value, id); `ties`: an
// equal value with a lower id goes first (else ids arrive in increasing order
// and an equal value never displaces the held one).
__device__ __forceinline__ void topk_push(float (&tv)[kTopkList], int (&ti)[kTopkList], float v, int id, bool ties) {
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) {
    const bool c = v > tv[j] || (ties && v == tv[j] && id < ti[j]);
    const float nv = c ? v : tv[j];
    const int ni = c ? id : ti[j];
    v = c ? tv[j] : v;
    id = c ? ti[j] : id;
    tv[j] = nv;
    ti[j] = ni;
  }
}
// Order-preserving 64-bit key of (value descending, id ascending).
__device__ __forceinline__ uint64_t topk_key(float v, int id) {
  const uint32_t u = __float_as_uint(v);
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)id);
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t k) {
  butterfly_steps([&](auto st) {
    constexpr int S = decltype(st)::value;
    const uint64_t o = ((uint64_t)lane_partner<S>((uint32_t)(k >> 32)) << 32) | lane_partner<S>((uint32_t)k);
    k = o > k ? o : k;
  });
  return k;
}
// k rounds: every lane offers the head of its sorted list, the wave's largest
// key wins and its lane moves on; out lists the winners in order (every lane).
__device__ __forceinline__ void topk_wave_select(float (&tv)[kTopkList], int (&ti)[kTopkList], int k,
                                                 float (&ov)[kTopkList], int (&oi)[kTopkList]) {
#pragma unroll
  for (int r = 0; r < kTopkList; ++r) {
    if (r >= k) { ov[r] = -INFINITY; oi[r] = 0x7fffffff; continue; }
    const uint64_t mine = topk_key(tv[0], ti[0]);
    const uint64_t best = wave_max_u64(mine);
    const uint32_t id = 0xFFFFFFFFu - (uint32_t)best;
    const uint32_t o = (uint32_t)(best >> 32);
    ov[r] = __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
    oi[r] = (int)id;
    if (mine == best) {                 // this lane's head was taken: shift its list
#pragma unroll
      for (int j = 0; j + 1 < kTopkList; ++j) { tv[j] = tv[j + 1]; ti[j] = ti[j + 1]; }
      tv[kTopkList - 1] = -INFINITY;
      ti[kTopkList - 1] = 0x7fffffff;
    }
  }
}

// Supplied logits: one wave per (row, segment); lane l scans ids l, l + 64, ...
__global__ __launch_bounds__(256) void k_topk_logits(const float* logits, int M, int V, int nseg, int cps,
                                                     TopkPart* out, Gate g, int n) {
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (item >= M * nseg) return;
  const int r = item / nseg, sg = item % nseg;
  if (!g.active(r / n)) return;
  const int v0 = sg * cps * kHeadChunk, v1 = min(V, v0 + cps * kHeadChunk);
  float tv[kTopkList];
  int ti[kTopkList];
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) { tv[j] = -INFINITY; ti[j] = 0x7fffffff; }
  const float* row = logits + (size_t)r * V;
  for (int v = v0 + lane; v < v1; v += 64) topk_push(tv, ti, row[v], v, false);
  float ov[kTopkList];
  int oi[kTopkList];
  topk_wave_select(tv, ti, kTopkList, ov, oi);
  if (lane == 0) {
    TopkPart rec;
#pragma unroll
    for (int j = 0; j < kTopkList; ++j) { rec.v[j] = ov[j]; rec.id[j] = oi[j]; }
    out[(size_t)r * nseg + sg] = rec;
  }
}

// One wave per row: the row's top k over its segments' lists, then the
// truncated tempered distribution (fp64 sums), the Gumbel-max sample over the
// k ids (each its own word of the GUMBEL stream), the top-2 margin, the
// argmax, and s = sum_j p_j E[id_j] (fp32, j in order; lanes over columns).
template <typename T>
__global__ __launch_bounds__(256) void k_topk_merge(const TopkPart* part, int M, int nseg, int k, StepInfo si,
                                                    SeedArg seeds, int n, Gate g, float* H, int32_t* y, int32_t* am,
                                                    float* margin, const T* emb, int d, float* s_out) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  const int b = r / n, pos = r % n;
  if (!g.active(b)) return;
  float tv[kTopkList];
  int ti[kTopkList];
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) { tv[j] = -INFINITY; ti[j] = 0x7fffffff; }
  const TopkPart* pr = part + (size_t)r * nseg;
  for (int sg = lane; sg < nseg; sg += 64) {
    const TopkPart rec = pr[sg];
#pragma unroll
    for (int j = 0; j < kTopkList; ++j) topk_push(tv, ti, rec.v[j], rec.id[j], true);
  }
  float lv[kTopkList];
  int li[kTopkList];
  topk_wave_select(tv, ti, k, lv, li);
  // the distribution over the k (every lane the same values)
  const int step = si.get_step();
  const float inv_t = si.get_inv_t(step);
  const double m = (double)(lv[0] * inv_t);
  double S = 0.0, W = 0.0;
  double e[kTopkList];
#pragma unroll
  for (int j = 0; j < kTopkList; ++j) {
    const double z = (double)(lv[j] * inv_t);
    e[j] = j < k ? exp(z - m) : 0.0;
    S += e[j];
    W += j < k ? e[j] * (z - m) : 0.0;
  }
  // Gumbel scores: lane j draws for the j-th id
  float score = -INFINITY;
  int sid = 0x7fffffff;
  if (lane < k) {
    float lvj = lv[0];
    int lij = li[0];
#pragma unroll
    for (int j = 1; j < kTopkList; ++j) if (lane == j) { lvj = lv[j]; lij = li[j]; }
    const uint4 x = philox_block(seeds.v[b], kTagGumbel, (uint32_t)si.cidx[b], (uint32_t)step, (uint32_t)pos,
                                 ((uint32_t)(lij >> 6) << 4) | (uint32_t)(lij & 15));
    const int word = (lij >> 4) & 3;
    const uint32_t xw = word == 0 ? x.x : word == 1 ? x.y : word == 2 ? x.z : x.w;
    score = lvj * inv_t + gumbel_of(xw);
    sid = lij;
  }
  const uint64_t k1 = wave_max_u64(topk_key(score, sid));
  const uint64_t mine = topk_key(score, sid);
  const uint64_t k2 = wave_max_u64(mine == k1 ? topk_key(-INFINITY, 0x7fffffff) : mine);
  auto val = [](uint64_t key) {
    const uint32_t o = (uint32_t)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
  };
  if (lane == 0) {
    H[r] = (float)(log(S) - W / S);
    y[r] = (int)(0xFFFFFFFFu - (uint32_t)k1);
    am[r] = li[0];
    margin[r] = k > 1 ? val(k1) - val(k2) : INFINITY;
  }
  if (s_out != nullptr) {
    float p[kTopkList];
#pragma unroll
    for (int j = 0; j < kTopkList; ++j) p[j] = (float)(e[j] / S);
    for (int c = lane; c < d; c += 64) {
      float acc = 0.f;
#pragma unroll
      for (int j = 0; j < kTopkList; ++j)
        if (j < k) acc += p[j] * Num<T>::load(emb + (size_t)li[j] * d + c);
      s_out[(size_t)r * d + c] = acc;
    }
  }
}

hipError_t topk_from_logits(const float* logits, int M, int V, int nseg, TopkPart* out, Gate g, int n, hipStream_t s) {
  const int nchunk = (V + kHeadChunk - 1) / kHeadChunk, cps = (nchunk + nseg - 1) / nseg;
  const int items = M * nseg;
  hipLaunchKernelGGL(k_topk_logits, dim3((items + 3) / 4), dim3(256), 0, s, logits, M, V, nseg, cps, out, g, n);
  return hipGetLastError();
}

template <typename T>
hipError_t topk_merge(const TopkPart* part, int M, int nseg, int top_k, const StepInfo& si, const SeedArg& seeds,
                      int n, Gate g, float* H, int32_t* y, int32_t* am, float* margin, const T* emb, int d,
                      float* s_out, hipStream_t s) {
  if (top_k < 1 || top_k > kTopkList) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_topk_merge<T>), dim3((M + 3) / 4), dim3(256), 0, s, part, M, nseg, top_k, si, seeds, n, g, H,
                     y, am, margin, emb, d, s_out);
  return hipGetLastError();
}
template hipError_t topk_merge<float>(const TopkPart*, int, int, int, const StepInfo&, const SeedArg&, int, Gate,
                                      float*, int32_t*, int32_t*, float*, const float*, int, float*, hipStream_t);
template hipError_t topk_merge<bf16>(const TopkPart*, int, int, int, const StepInfo&, const SeedArg&, int, Gate,
                                     float*, int32_t*, int32_t*, float*, const bf16*, int, float*, hipStream_t);

// ------------------------------------------------------------------ training-side corruption and loss
// Corruption of a clean canvas ([mlqm] 一: a share of the tokens, 0 to 100%,
// replaced by random vocabulary tokens): one Philox call per position (tag
// CORRUPT, counter (0, position, 0, CORRUPT << 24 | canvas index)); word 0
// decides (u < rate of the request, fp32), word 1 is the replacement.
__global__ void k_corrupt(const int32_t* clean, int32_t* out, SeedArg seeds, RateArg rates, int n, int vocab,
                          const int32_t* cidx) {
  const int b = blockIdx.x;
  const uint32_t c = (uint32_t)cidx[b];
  const float rate = rates.v[b];
  for (int i = threadIdx.x; i < n; i += blockDim.x) {
    const uint4 x = philox_block(seeds.v[b], kTagCorrupt, c, 0u, (uint32_t)i, 0u);
    const int32_t t = clean[(size_t)b * n + i];
    out[(size_t)b * n + i] = u01(x.x) < rate ? token_of(x.y, vocab) : t;
  }
}

// Cross-entropy of the clean token per row (one wave per row): the clean
// token's logit rnd(final norm(h)) . E[x0] (operands as the LM head takes
// them, fp32 sums in a fixed order), subtracted from the row's log-sum-exp.
template <typename T>
__global__ __launch_bounds__(256) void k_clean_ce(const T* xn, const T* emb, const int32_t* clean, const float* lse,
                                                  int M, int d, int vocab, float* ce) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  const T* a = xn + (size_t)r * d;
  const T* e = emb + (size_t)min(max(clean[r], 0), vocab - 1) * d;   // ids outside [0, V) are clamped
  float acc = 0.f;
  for (int k = lane; k < d; k += 64) acc += Num<T>::load(a + k) * Num<T>::load(e + k);
  acc = wave_sum(acc);
  if (lane == 0) ce[r] = lse[r] - acc;
}

// The same for an FP8 head: the clean token's logit is scale[x0] times the
// product with the E4M3 codes of row x0, read from the P8 fragment order
// (block (x0/16, k/64), lane (k%32)/8 * 16 + x0%16, byte (k%64)/32 * 8 + k%8).
__global__ __launch_bounds__(256) void k_clean_ce_fp8(const bf16* xn, const fp8e4m3* codes, const float* scale,
                                                      const int32_t* clean, const float* lse, int M, int d,
                                                      int vocab, float* ce) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (r >= M) return;
  const bf16* a = xn + (size_t)r * d;
  const int v = min(max(clean[r], 0), vocab - 1);
  const uint8_t* rowblk = reinterpret_cast<const uint8_t*>(codes) + (size_t)(v / 16) * (d / 64) * 1024;
  float acc = 0.f;
  for (int k = lane; k < d; k += 64) {
    const uint8_t c = rowblk[(size_t)(k / 64) * 1024 + (((k % 32) / 8) * 16 + v % 16) * 16 + ((k % 64) / 32) * 8 + k % 8];
    acc += Num<bf16>::load(a + k) * __builtin_amdgcn_cvt_pk_f32_fp8((int)c, false)[0];
  }
  acc = wave_sum(acc);
  if (lane == 0) ce[r] = lse[r] - scale[v] * acc;
}

// Mean cross-entropy per request: fp64, positions in order.
__global__ void k_loss_mean(const float* ce, int B, int n, float* loss) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  double s = 0.0;
  for (int i = 0; i < n; ++i) s += (double)ce[(size_t)b * n + i];
  loss[b] = (float)(s / (double)n);
}

hipError_t corrupt_canvas(const int32_t* clean, int32_t* out, const SeedArg& seeds, const RateArg& rates, int B,
                          int n, int vocab, const int32_t* cidx, hipStream_t s) {
  hipLaunchKernelGGL(k_corrupt, dim3(B), dim3(256), 0, s, clean, out, seeds, rates, n, vocab, cidx);
  return hipGetLastError();
}

template <typename T>
hipError_t clean_token_loss(const T* xn, const T* emb, const int32_t* clean, const float* lse, int B, int n, int d,
                            int vocab, float* ce, float* loss, hipStream_t s) {
  const int M = B * n;
  hipLaunchKernelGGL((k_clean_ce<T>), dim3((M + 3) / 4), dim3(256), 0, s, xn, emb, clean, lse, M, d, vocab, ce);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_loss_mean, dim3((B + 63) / 64), dim3(64), 0, s, ce, B, n, loss);
  return hipGetLastError();
}
hipError_t clean_token_loss_fp8(const bf16* xn, const fp8e4m3* codes, const float* scale, const int32_t* clean,
                                const float* lse, int B, int n, int d, int vocab, float* ce, float* loss,
                                hipStream_t s) {
  const int M = B * n;
  if (d % 64 || vocab % 16) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_clean_ce_fp8, dim3((M + 3) / 4), dim3(256), 0, s, xn, codes, scale, clean, lse, M, d, vocab,
                     ce);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_loss_mean, dim3((B + 63) / 64), dim3(64), 0, s, ce, B, n, loss);
  return hipGetLastError();
}
template hipError_t clean_token_loss<float>(const float*, const float*, const int32_t*, const float*, int, int, int,
                                            int, float*, float*, hipStream_t);
template hipError_t clean_token_loss<bf16>(const bf16*, const bf16*, const int32_t*, const float*, int, int, int,
                                           int, float*, float*, hipStream_t);

hipError_t selfcond_reduce(const float* part, int M, int d, int splits, float* S, Gate g, int n, hipStream_t s) {
  const size_t nq = (size_t)M * d / 4;      // d is a multiple of 256
  if (nq == 0) return hipSuccess;
  hipLaunchKernelGGL(k_selfcond_reduce, dim3((unsigned)((nq + 255) / 256)), dim3(256), 0, s, part, M, d, splits, S,
                     g, n);
  return hipGetLastError();
}

hipError_t commit_kernel(const float* H, const int32_t* y, const int32_t* am, int32_t* canvas, int32_t* prev_am,
                         uint8_t* mask, int32_t* n_committed, uint8_t* done, const SeedArg& seeds, int B, int n,
                         int vocab, const StepInfo& si, int max_steps, float bound, int stop_mode, float tau,
                         hipStream_t s) {
  hipLaunchKernelGGL(k_commit, dim3(B), dim3(256), 0, s, H, y, am, canvas, prev_am, mask, n_committed, done, seeds,
                     n, vocab, si, max_steps, bound, stop_mode, tau);
  return hipGetLastError();
}

// End of a step of the device-driven loop (one wave): every request done?
// The canvas step moves on, the completed-step count too, and the progress
// record in mapped host memory (steps completed, all done) is written with
// system-scope stores so the host sees it without a synchronisation.
__global__ __launch_bounds__(64) void k_step_end(const uint8_t* done, int B, int32_t* step,
                                                 volatile int32_t* progress) {
  const int lane = threadIdx.x;
  int fin = 1;
  for (int b = lane; b < B; b += 64) fin &= done[b] != 0 ? 1 : 0;
  fin = __all(fin) ? 1 : 0;
  if (lane == 0) {
    step[0] = step[0] + 1;
    step[1] = fin;
    const int32_t count = step[2] + 1;
    step[2] = count;
    if (progress != nullptr) {
      __hip_atomic_store(const_cast<int32_t*>(progress + 1), fin, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
      __hip_atomic_store(const_cast<int32_t*>(progress), count, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
  }
}

hipError_t step_end(const uint8_t* done, int B, int32_t* step, volatile int32_t* progress, hipStream_t s) {
  hipLaunchKernelGGL(k_step_end, dim3(1), dim3(64), 0, s, done, B, step, progress);
  return hipGetLastError();
}

// ------------------------------------------------------------------ fixed scratch
// Device memory of the allocation-free sampler entry point: a file-scope
// array each GPU holds until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the
// symbol); its device address is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  static std::mutex mu;
  static void* per_device[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    per_device[dev] = p;
  }
  *ptr = per_device[dev];
  return hipSuccess;
}

template hipError_t head_from_logits<float>(const float*, int, int, const StepInfo&, const SeedArg&, int,
                                            HeadPart*, float*, Gate, hipStream_t);
template hipError_t head_from_logits<bf16>(const float*, int, int, const StepInfo&, const SeedArg&, int,
                                           HeadPart*, bf16*, Gate, hipStream_t);

}  // namespace dg

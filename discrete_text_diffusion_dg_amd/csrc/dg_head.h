// Head statistics of the denoise step ([mlqm] 四: entropy of the tempered
// distribution, Gumbel-max sample and top-2 margin; [mlqm] 一: the sampled
// distribution feeds the next step's self-conditioning vector).
//
// The vocabulary is cut into chunks of 128 ids -- one LM-head tile.  A tile of
// 128 rows x 128 logits sits in LDS (fp32, padded rows); lane (row, half) of
// the four waves owns 64 consecutive ids of one row, which is exactly the set
// served by 16 Philox calls of the Gumbel stream (ids c, c + 16, c + 32, c + 48
// of an aligned 64-id group share a call), so every statistic of a half is
// formed in registers and the two halves of a row meet in one lane exchange.
// Per (row, chunk) the lane pair writes: the chunk max m of z = logit / T,
// sum exp(z - m), sum exp(z - m)(z - m), the logit arg-max, and the best two
// Gumbel-perturbed scores; and (self-conditioning models) exp(z - m) rounded to
// the operand type.  The merge kernel combines the chunks of a row.
#pragma once
#include "dg_kernels.h"

namespace dg {

constexpr int kHeadChunk = 128;     // vocabulary ids per head chunk
constexpr int kHeadLd = 132;        // LDS row stride of a staged 128 x 128 tile (floats, 16-byte rows)
constexpr int kHeadTileBytes = kHeadChunk * kHeadLd * 4;

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
// Branch-free insertion of one new value (selects, no divergent control flow)
// for values visited in increasing id order: an equal value never replaces
// the held one (its id is larger), so one comparison decides.
__device__ __forceinline__ void top2_insert_ordered(Top2& a, float v, int i) {
  const bool better = v > a.b1;
  a.b2 = __builtin_amdgcn_fmed3f(a.b1, v, a.b2);   // b2 <= b1: the middle value is the new second best
  a.b1 = fmaxf(a.b1, v);
  a.i1 = better ? i : a.i1;
}
__device__ __forceinline__ void argmax_insert_ordered(float& v, int& i, float ov, int oi) {
  const bool better = ov > v;
  v = better ? ov : v;
  i = better ? oi : i;
}

// Gumbel stream: counter word 0 of the call serving vocabulary id v is
// 16 * (v >> 6) + (v & 15); v takes its output word (v >> 4) & 3.
__device__ __forceinline__ uint32_t gumbel_call(int v) { return ((uint32_t)(v >> 6) << 4) | (uint32_t)(v & 15); }

// Statistics of the tile rows m0 .. m0 + rows - 1 (of R), vocabulary ids
// n0 .. n0 + cols - 1 (cols 64 or 128).  tile: LDS [128][kHeadLd] raw logits.
// Called by all 256 threads of the workgroup.
template <typename T>
__device__ __forceinline__ void head_tile_stats(const float* tile, int m0, int rows, int n0, int cols, int V,
                                                const StepInfo& si, const SeedArg& seeds, int n, HeadPart* part,
                                                int nchunk, T* ptilde) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rl = w * 32 + (lane & 31), half = lane >> 5, c0 = half * 64;
  const bool have = rl < rows && c0 < cols;
  const int row = m0 + rl, v0 = n0 + c0;
  const int b = have ? row / n : 0, pos = have ? row % n : 0;
  const int step = si.get_step();
  const float inv_t = si.get_inv_t(step);
  const int canvas_index = si.cidx[b];
  const float* tr = tile + rl * kHeadLd + c0;
  float x[64];
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const float4 t4 = reinterpret_cast<const float4*>(tr)[q];
    x[4 * q] = t4.x; x[4 * q + 1] = t4.y; x[4 * q + 2] = t4.z; x[4 * q + 3] = t4.w;
  }
  // logit arg-max (lowest id on ties); rounding is monotone and 1 / T > 0, so
  // the largest z = logit * (1 / T) is the largest logit times 1 / T
  float lmax = -INFINITY;
  int lidx = 0x7fffffff;
  if (have) {
    // ids local to the half (constants of the unrolled scan), made global once
#pragma unroll
    for (int k = 0; k < 64; ++k) argmax_insert_ordered(lmax, lidx, x[k], k);
    lidx += v0;
  }
  const float zmax = lmax * inv_t;
  // Gumbel-max top two: every value is scored (a lane owns a row of its own,
  // so pruning by a per-row threshold would leave the wave executing the
  // scoring of almost every value anyway)
  Top2 t2{-INFINITY, 0x7fffffff, -INFINITY};
  const uint64_t seed = seeds.v[b];
  const uint32_t call0 = gumbel_call(v0);
  if (have) {
    // all 16 calls first, then the 64 scores in id order (id v0 + k takes
    // word k >> 4 of call k & 15)
    uint32_t xs[16][4];
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      const uint4 xw = philox_block(seed, kTagGumbel, (uint32_t)canvas_index, (uint32_t)step, (uint32_t)pos, call0 | c);
      xs[c][0] = xw.x; xs[c][1] = xw.y; xs[c][2] = xw.z; xs[c][3] = xw.w;
    }
#pragma unroll
    for (int k = 0; k < 64; ++k) top2_insert_ordered(t2, x[k] * inv_t + gumbel_of(xs[k & 15][k >> 4]), k);
    t2.i1 += v0;
  }
  // the chunk's row max, then exp(z - m) and its sums (ids in order)
  const float m = fmaxf(zmax, lane_partner<5>(zmax));     // lane ^ 32: the row's other half
  float s = 0.f, ws = 0.f;
  if (have) {
#pragma unroll
    for (int k = 0; k < 64; ++k) {
      const float dz = x[k] * inv_t - m;
      const float e = exp_fast(dz);
      x[k] = e;
      s += e;
      ws += e * dz;
    }
    if (ptilde != nullptr) {
      T* dst = ptilde + (size_t)row * V + v0;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int q = 0; q < 8; ++q) reinterpret_cast<uint4*>(dst)[q] = pack8_bf16(x + 8 * q);
      } else {
#pragma unroll
        for (int q = 0; q < 16; ++q)
          reinterpret_cast<float4*>(dst)[q] = make_float4(x[4 * q], x[4 * q + 1], x[4 * q + 2], x[4 * q + 3]);
      }
    }
  }
  // the two halves of the row (lanes l and l ^ 32): sums in half order
  const float so = lane_partner<5>(s), wo = lane_partner<5>(ws);
  const float lo = lane_partner<5>(lmax);
  const int lio = lane_partner<5>(lidx);
  const Top2 to{lane_partner<5>(t2.b1), lane_partner<5>(t2.i1), lane_partner<5>(t2.b2)};
  if (half == 0 && rl < rows) {
    argmax_merge(lmax, lidx, lo, lio);
    top2_merge(t2, to);
    HeadPart hp;
    hp.m = m; hp.s = s + so; hp.w = ws + wo; hp.lmax = lmax; hp.lidx = lidx;
    hp.g1 = t2.b1; hp.gidx = t2.i1; hp.g2 = t2.b2;
    part[(size_t)row * nchunk + n0 / kHeadChunk] = hp;
  }
}

}  // namespace dg

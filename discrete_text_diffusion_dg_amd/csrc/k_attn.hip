// Attention of the denoise step and of the causal encoder (gfx950).
//
// Canvas rows attend bidirectionally to every cached key and every canvas key;
// the encoder (prompt chunks, committed canvases) attends causally
// ([mlqm] 二: causal attention when encoding the prompt, bidirectional
// attention over the 256-token canvas).  New rows' keys and values are already
// in the cache at ctx..ctx+nq-1, so one loop covers keys 0..ctx+nq-1.
//
// Layout: a workgroup owns 64 query rows of one (request, kv head); the rows
// are the (query head in the group, position) pairs, head-major, so all query
// heads sharing a kv head reuse one K/V tile in LDS.  Each wave owns 16 rows.
// Per 64-key tile: S^T = K Q^T on MFMA (keys on the M side, so each lane holds
// 16 scores of a single query), online softmax in registers, then
// O^T += V^T P on MFMA with V staged transposed in LDS; the accumulator layout
// again gives each lane one query, so rescaling needs no lane exchange.
// Long key ranges are split across workgroups; partial (O, max, sum) are merged
// in a fixed order by a second kernel.
#include "dg_kernels.h"

namespace dg {

namespace {

template <typename T, int HD>
struct AttnShape {
  static constexpr int KT = 64;                         // keys per tile
  static constexpr int LDK = HD + 16 / (int)sizeof(T);  // sK row stride
  static constexpr int LDV = KT + 16 / (int)sizeof(T);  // sVt row stride
  static constexpr int kSmem = (KT * LDK + HD * LDV) * (int)sizeof(T);
};

// Four consecutive operand elements from LDS into fragment slots [off, off+4).
__device__ __forceinline__ void lds4(Frag<bf16>& f, int half, const bf16* p) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  if (half == 0) { f.v.x = v.x; f.v.y = v.y; } else { f.v.z = v.x; f.v.w = v.y; }
}
__device__ __forceinline__ void lds4(Frag<float>& f, int half, const float* p) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  f.v[half * 4 + 0] = v.x; f.v[half * 4 + 1] = v.y; f.v[half * 4 + 2] = v.z; f.v[half * 4 + 3] = v.w;
}
__device__ __forceinline__ void set_p(Frag<bf16>& f, const float* p) {
  f.v = pack8_bf16(p);
}
__device__ __forceinline__ void set_p(Frag<float>& f, const float* p) {
#pragma unroll
  for (int j = 0; j < 8; ++j) f.v[j] = p[j];
}
template <typename T>
__device__ __forceinline__ void store4(T* dst, const float* v) {
#pragma unroll
  for (int j = 0; j < 4; ++j) Num<T>::store(dst + j, v[j]);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attention(AttnArgs a) {
  using S = AttnShape<T, HD>;
  __shared__ __attribute__((aligned(16))) char smem[S::kSmem];
  T* sK = reinterpret_cast<T*>(smem);
  T* sVt = sK + S::KT * S::LDK;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, q16 = lane & 15;
  const int G = a.Hq / a.Hkv;
  const int rows_total = G * a.nq;
  const int bk = blockIdx.y;                  // request * Hkv + kv head
  const int b = bk / a.Hkv, kvh = bk % a.Hkv;
  const int split = blockIdx.z;
  const int rho0 = blockIdx.x * 64;
  if (rho0 >= rows_total) return;

  // this lane's query row
  const int rho = rho0 + w * 16 + q16;
  const bool qvalid = rho < rows_total;
  const int hh = qvalid ? rho / a.nq : 0, qi = qvalid ? rho % a.nq : 0;
  const int head = kvh * G + hh;
  const int qpos = a.ctx + qi;

  // key range of this workgroup
  const int total = a.ctx + a.nq;
  int klimit = total;
  if (a.causal) {
    const int last = min(rho0 + 63, rows_total - 1);
    const int imax = (rho0 / a.nq == last / a.nq) ? last % a.nq : a.nq - 1;
    klimit = a.ctx + imax + 1;
  }
  const int per = ((total + a.splits - 1) / a.splits + S::KT - 1) / S::KT * S::KT;
  const int kbeg = split * per;
  const int kend = min(klimit, kbeg + per);

  const T* Q = reinterpret_cast<const T*>(a.q);
  const size_t qstride = (size_t)a.Hq * HD;
  const size_t qrow = (size_t)(b * a.nq + qi) * qstride + (size_t)head * HD;
  Frag<T> qf[HD / 32];
#pragma unroll
  for (int s = 0; s < HD / 32; ++s) {
    if (qvalid) {
      lds_frag(qf[s], Q + qrow + s * 32 + g4 * 8);   // global read, same shape as an LDS fragment
    } else {
      float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      set_p(qf[s], z);
    }
  }

  const T* Kc = reinterpret_cast<const T*>(a.kc) + ((size_t)b * a.Hkv + kvh) * a.max_ctx * HD;
  const T* Vc = reinterpret_cast<const T*>(a.vc) + ((size_t)b * a.Hkv + kvh) * a.max_ctx * HD;

  f32x4_t o[HD / 16];
#pragma unroll
  for (int j = 0; j < HD / 16; ++j) o[j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;

  constexpr int EPC = 16 / (int)sizeof(T);
  constexpr int CH_PER_KEY = HD / EPC;                  // 16-byte chunks per key row
  constexpr int CHUNKS = S::KT * CH_PER_KEY;

  for (int k0 = kbeg; k0 < kend; k0 += S::KT) {
    // stage K [key][d] and V^T [d][key]; keys past kend are zero
    for (int c = tid; c < CHUNKS; c += 256) {
      const int key = c / CH_PER_KEY, dc = (c % CH_PER_KEY) * EPC;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (k0 + key < kend) {
        kv = *reinterpret_cast<const uint4*>(Kc + (size_t)(k0 + key) * HD + dc);
        vv = *reinterpret_cast<const uint4*>(Vc + (size_t)(k0 + key) * HD + dc);
      }
      *reinterpret_cast<uint4*>(sK + key * S::LDK + dc) = kv;
      const T* ve = reinterpret_cast<const T*>(&vv);
#pragma unroll
      for (int j = 0; j < EPC; ++j) sVt[(dc + j) * S::LDV + key] = ve[j];
    }
    __syncthreads();

    // scores S^T[key][query] for the 64 keys of the tile
    f32x4_t sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < HD / 32; ++s) {
        Frag<T> kf;
        lds_frag(kf, sK + (kb * 16 + q16) * S::LDK + s * 32 + g4 * 8);
        mma16x16x32(sc[kb], kf, qf[s]);
      }
    }
    float p[16];
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kpos = k0 + kb * 16 + g4 * 4 + i;
        float v = sc[kb][i] * a.scale;
        if (kpos >= kend || (a.causal && kpos > qpos)) v = -INFINITY;
        p[kb * 4 + i] = v;
        tmax = fmaxf(tmax, v);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(m_run, tmax);
    const float alpha = (m_new == -INFINITY) ? 1.f : expf(m_run - m_new);
    float lsum = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float e = (p[j] == -INFINITY) ? 0.f : expf(p[j] - m_new);
      p[j] = e;
      lsum += e;
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int j = 0; j < HD / 16; ++j) o[j] *= alpha;

    // O^T[d][q] += V^T[d][keys] P[keys][q], two 32-key steps.  With bf16
    // operands the fp32 probabilities are split into a bf16 head and a bf16
    // remainder (two MFMAs, ~16 significant bits): a single bf16 rounding of P
    // would dominate the output error, while beyond 16 bits the fp32 summation
    // over the keys does (a third term was measured to change nothing).
    constexpr int NT = sizeof(T) == 2 ? 2 : 1;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      Frag<T> pf[NT];
      float rest[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rest[i] = p[(2 * ks) * 4 + i];
        rest[4 + i] = p[(2 * ks + 1) * 4 + i];
      }
#pragma unroll
      for (int term = 0; term < NT; ++term) {
        float part[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          part[j] = Num<T>::round(rest[j]);
          rest[j] -= part[j];
        }
        set_p(pf[term], part);
      }
#pragma unroll
      for (int db = 0; db < HD / 16; ++db) {
        Frag<T> vf;
        const T* row = sVt + (db * 16 + q16) * S::LDV + ks * 32 + g4 * 4;
        lds4(vf, 0, row);
        lds4(vf, 1, row + 16);
#pragma unroll
        for (int term = 0; term < NT; ++term) mma16x16x32(o[db], vf, pf[term]);
      }
    }
    __syncthreads();
  }

  // full row sum across the four lane groups holding the same query
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  if (!qvalid) return;
  const size_t rowid = (size_t)(b * a.nq + qi) * a.Hq + head;
  if (a.splits == 1) {
    T* out = reinterpret_cast<T*>(a.out) + qrow;
    const float inv = 1.f / l_run;
#pragma unroll
    for (int db = 0; db < HD / 16; ++db) {
      float v[4] = {o[db][0] * inv, o[db][1] * inv, o[db][2] * inv, o[db][3] * inv};
      store4(out + db * 16 + g4 * 4, v);
    }
  } else {
    float* po = a.part_o + ((size_t)split * a.B * a.nq * a.Hq + rowid) * HD;
#pragma unroll
    for (int db = 0; db < HD / 16; ++db)
      *reinterpret_cast<float4*>(po + db * 16 + g4 * 4) = make_float4(o[db][0], o[db][1], o[db][2], o[db][3]);
    if (g4 == 0) {
      float* pm = a.part_ml + ((size_t)split * a.B * a.nq * a.Hq + rowid) * 2;
      pm[0] = m_run;
      pm[1] = l_run;
    }
  }
}

// One thread per (row, 4 dims): combine the split partials in split order.
template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  const size_t nrows = (size_t)a.B * a.nq * a.Hq;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rowid = gid / (HD / 4);
  const int d0 = (int)(gid % (HD / 4)) * 4;
  if (rowid >= nrows) return;
  float m = -INFINITY;
  for (int s = 0; s < a.splits; ++s) m = fmaxf(m, a.part_ml[(s * nrows + rowid) * 2]);
  float l = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < a.splits; ++s) {
    const float ms = a.part_ml[(s * nrows + rowid) * 2];
    if (ms == -INFINITY) continue;
    const float f = expf(ms - m);
    l += a.part_ml[(s * nrows + rowid) * 2 + 1] * f;
    const float4 v = *reinterpret_cast<const float4*>(a.part_o + (s * nrows + rowid) * HD + d0);
    acc[0] += v.x * f; acc[1] += v.y * f; acc[2] += v.z * f; acc[3] += v.w * f;
  }
  const float inv = 1.f / l;
  const int head = (int)(rowid % a.Hq);
  const size_t tok = rowid / a.Hq;
  T* out = reinterpret_cast<T*>(a.out) + tok * (size_t)a.Hq * HD + (size_t)head * HD + d0;
  float v[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  store4(out, v);
}

template <typename T, int HD>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  dim3 grid((G * a.nq + 63) / 64, a.B * a.Hkv, a.splits);
  hipLaunchKernelGGL((k_attention<T, HD>), grid, dim3(256), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const size_t threads = (size_t)a.B * a.nq * a.Hq * (HD / 4);
  hipLaunchKernelGGL((k_attn_merge<T, HD>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

int attention_splits(int B, int nq, int Hq, int Hkv, int keys) {
  const int wg = ((Hq / Hkv) * nq + 63) / 64 * B * Hkv;
  int splits = (512 + wg - 1) / wg;
  const int max_by_keys = (keys + 255) / 256;
  if (splits > max_by_keys) splits = max_by_keys;
  if (splits > 16) splits = 16;
  if (splits < 1) splits = 1;
  return splits;
}

template <typename T>
hipError_t attention(const AttnArgs& a, hipStream_t s) {
  if (a.nq <= 0) return hipSuccess;
  if (a.hd == 64) return launch_attn<T, 64>(a, s);
  if (a.hd == 128) return launch_attn<T, 128>(a, s);
  return hipErrorInvalidValue;
}

template hipError_t attention<float>(const AttnArgs&, hipStream_t);
template hipError_t attention<bf16>(const AttnArgs&, hipStream_t);

}  // namespace dg

// Attention of the denoise step and of the causal encoder (gfx950).
//
// Canvas rows attend bidirectionally to every cached key and every canvas key;
// the encoder (prompt chunks, committed canvases) attends causally
// ([mlqm] 二: causal attention when encoding the prompt, bidirectional
// attention over the 256-token canvas).  New rows' keys and values are already
// in the cache at ctx..ctx+nq-1, so one loop covers keys 0..ctx+nq-1.
//
// Cache layout: K rows [key][d], V transposed [d][key] (row stride: the context
// capacity rounded up to the 64-key tile).  Query rows of a (request, kv head)
// are the (query head in the group, position) pairs, head-major, so every
// query head sharing a kv head reads the same K/V.  Per 64-key tile:
// S^T = K Q^T on MFMA (keys on the M side, each lane holding 16 scores of one
// query), online softmax in registers, O^T += V^T P on MFMA (again one query
// per lane, so rescaling needs no lane exchange).  Both MFMA operands come as
// fragments: K rows give the A operand of S^T directly, V^T rows that of O^T.
//
// Two launch shapes:
//  * spread (few query rows per kv head and short contexts, the small batch-1
//    shape): a workgroup owns 16 * QB query rows; its NW waves take the key
//    tiles round-robin, streaming K and V^T fragments straight from memory one
//    tile ahead, and merge their partial (O, max, sum) through LDS in wave
//    order at the end -- many short chains instead of a few long ones;
//  * wide (everything else): a workgroup owns 16 * NWQ query rows, one wave
//    per 16, and the waves share each K / V^T tile staged in LDS (two stages,
//    the global loads of a tile issued two tiles ahead, one LDS-only barrier
//    per tile).  Every workgroup of a kv head reads the head's whole key range
//    (or its split of it), so the K/V bytes a launch moves scale with the
//    number of query blocks per kv head: 16-row blocks re-read a long context
//    too often, which is what decides between the two shapes.
// Long key ranges are further split across workgroups; partial (O, max, sum)
// are merged in a fixed order by a second kernel.
#include "dg_kernels.h"

#include <type_traits>

namespace dg {

namespace {

// Key order inside a 64-key tile.  Row r of score block kb (S^T = K Q^T, 16
// keys on the M side) holds key (kb / 2) * 32 + (r / 4) * 8 + (kb % 2) * 4 + r % 4,
// so the accumulator rows a lane group g owns (g*4 .. g*4+3 of blocks 2s and
// 2s+1) are the 8 consecutive keys s*32 + g*8 .. +7 -- exactly the k-elements
// that group supplies to O^T += V^T P for that 32-key step.  The V^T fragment
// is then one contiguous 16-byte read; the sum over keys does not depend on
// their order.
__device__ __forceinline__ int tile_key(int kb, int r) { return (kb >> 1) * 32 + (r >> 2) * 8 + (kb & 1) * 4 + (r & 3); }

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
// P operand of O^T += V^T P.  bf16: head = rnd(p), remainder = rnd(p - head)
// (two MFMAs, ~16 significant bits); a pair of values per conversion.
__device__ __forceinline__ void split_p(Frag<bf16> (&f)[2], float* r) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w[j] = f32x2_to_bf16x2(r[2 * j], r[2 * j + 1]);
    r[2 * j] -= __uint_as_float(w[j] << 16);
    r[2 * j + 1] -= __uint_as_float(w[j] & 0xFFFF0000u);
  }
  f[0].v = make_uint4(w[0], w[1], w[2], w[3]);
  f[1].v = make_uint4(f32x2_to_bf16x2(r[0], r[1]), f32x2_to_bf16x2(r[2], r[3]), f32x2_to_bf16x2(r[4], r[5]),
                      f32x2_to_bf16x2(r[6], r[7]));
}
__device__ __forceinline__ void split_p(Frag<float> (&f)[1], float* r) { set_p(f[0], r); }
// Four consecutive output values (dst 4-element aligned): one 8-byte store of
// bf16 pairs, or one 16-byte store.
template <typename T>
__device__ __forceinline__ void store4(T* dst, const float* v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(f32x2_to_bf16x2(v[0], v[1]), f32x2_to_bf16x2(v[2], v[3]));
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}
template <typename T>
__device__ __forceinline__ float4 load4(const T* src) {
  if constexpr (sizeof(T) == 2) {
    const uint2 u = *reinterpret_cast<const uint2*>(src);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                       __uint_as_float(u.y & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4*>(src);
  }
}

// ---- wide: 16 * NWQ query rows per workgroup sharing LDS-staged K / V^T tiles
// bf16 V^T pieces are staged as fp16 so that the probabilities enter
// O^T += V^T P as one fp16 operand (11 significant bits) instead of a two-term
// bf16 split.  The conversion is exact for bf16 values with 2^-17 <= |v| <
// 2^16 (fp16's largest finite value is 65504; every bf16 value below 2^16 is
// at most 65280); smaller ones are rounded to fp16's 2^-24 grid.  A tile whose
// largest |v| is 2^16 or more, or below 2^-14, is staged instead as
// fp16(v * 2^-s), s chosen so that its largest |v| lands in [2^14, 2^15), and
// its products are taken as O = 2^s (2^-s O + V'^T P): exact power-of-two
// scalings around the same fp16 products.  Either way each staged value is
// within 2^-11 of its tile's largest |v| of the exact one.
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
}
__device__ __forceinline__ uint4 bf16x8_to_f16x8(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = f32x2_to_f16x2(__uint_as_float(w[j] << 16), __uint_as_float(w[j] & 0xFFFF0000u));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
// Largest biased exponent (the 8-bit field) among eight bf16 values.
__device__ __forceinline__ uint32_t bf16x8_max_exp(uint4 x) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t m = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7F80u, (w[j] >> 16) & 0x7F80u));
  return m >> 7;
}
// fp16(v * 2^-s) of eight bf16 values (the scaling is exact in fp32).
__device__ __forceinline__ uint4 bf16x8_to_f16x8_scaled(uint4 x, int s) {
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t r[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    r[j] = f32x2_to_f16x2(__builtin_amdgcn_ldexpf(__uint_as_float(w[j] << 16), -s),
                          __builtin_amdgcn_ldexpf(__uint_as_float(w[j] & 0xFFFF0000u), -s));
  return make_uint4(r[0], r[1], r[2], r[3]);
}
constexpr uint32_t kF16ExpHi = 127 + 16;   // |v| >= 2^16: beyond fp16
constexpr uint32_t kF16ExpLo = 127 - 14;   // |v| >= 2^-14: fp16 normal
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  butterfly_steps([&](auto st) { v = max(v, lane_partner<decltype(st)::value>(v)); });
  return v;
}
__device__ __forceinline__ void mma16x16x32_f16(f32x4_t& acc, uint4 a, uint4 b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), acc, 0,
                                               0, 0);
}
// Maximum over the four lanes q16 + 16 g4 that hold one query's scores: the
// gfx950 row swaps (16-lane rows, then 32-lane halves) are plain VALU moves,
// where a shuffle goes through the LDS crossbar.
__device__ __forceinline__ float max_over_g4(float v) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

template <typename T, int HD, int NWQ, int QBW>
__global__ __launch_bounds__(64 * NWQ) void k_attn_wide(AttnArgs a) {
  constexpr int KT = 64, NS = HD / 32, NDB = HD / 16;
  constexpr int NT = sizeof(T) == 2 ? 2 : 1;
  constexpr int EPC = 16 / (int)sizeof(T);
  // bf16 128-dim K rows are unpadded, their 16-byte pieces XOR-swizzled by
  // kswz(key): the 16 keys a fragment read takes (tile_key over 16 lanes) then
  // fall on 16 distinct piece slots, where a padded row put rows r and r + 16
  // on the same banks (proxy shape, no key splits: 63.7 -> 61.7 us).  64-dim
  // rows keep one piece of padding (the swizzle measured 1-2% slower at the
  // batched shape), as do fp32 rows.
  constexpr bool KSWZ = sizeof(T) == 2 && HD == 128;
  constexpr int LDK = KSWZ ? HD : HD + EPC, LDV = KT + EPC;
  constexpr int KBUF = KT * LDK, VBUF = HD * LDV;     // elements per stage
  constexpr int NTH = 64 * NWQ;
  constexpr int CH_PER_KEY = HD / EPC;
  auto kswz = [](int key) { return KSWZ ? ((key & 3) | (((key >> 3) & 3) << 2)) & (CH_PER_KEY - 1) : 0; };
  constexpr int KCH = KT * CH_PER_KEY / NTH, VCH = HD * (KT / EPC) / NTH;
  constexpr int RPW = 16 * NWQ;                        // query rows per query block of the workgroup
  static_assert(KCH >= 1 && VCH >= 1 && KT * CH_PER_KEY % NTH == 0 && HD * (KT / EPC) % NTH == 0, "tile shape");
  static_assert(QBW == 1 || sizeof(T) == 2, "several query blocks per wave: bf16 path only");
  __shared__ __attribute__((aligned(16))) T smem[2 * (KBUF + VBUF)];
  // per stage and wave: bit 0 some |v| >= 2^16, bit 1 some |v| >= 2^-14 (bf16)
  __shared__ uint32_t s_vflag[2][NWQ];
  __shared__ uint32_t s_vexp[NWQ];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g4 = lane >> 4, q16 = lane & 15;
  const int G = a.Hq / a.Hkv, rows_total = G * a.nq;
  const int bk = blockIdx.y, b = bk / a.Hkv, kvh = bk % a.Hkv, split = blockIdx.z;
  const int rho0 = blockIdx.x * RPW * QBW;
  if (!a.gate.active(b)) return;                 // the whole workgroup, before any barrier
  const int ctx = a.pos.base(b);
  // query block qb of this wave: rows rho0 + qb * RPW + 16 w + (0..15)
  bool qvalid[QBW];
  int qi[QBW], head[QBW], qpos[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const int rho = rho0 + qb * RPW + w * 16 + q16;
    qvalid[qb] = rho < rows_total;
    const int hh = qvalid[qb] ? rho / a.nq : 0;
    qi[qb] = qvalid[qb] ? rho % a.nq : 0;
    head[qb] = kvh * G + hh;
    qpos[qb] = ctx + qi[qb];
  }
  const int total = ctx + a.nq;
  int klimit = total;
  if (a.causal) {
    const int last = min(rho0 + RPW * QBW - 1, rows_total - 1);
    const int imax = (rho0 / a.nq == last / a.nq) ? last % a.nq : a.nq - 1;
    klimit = ctx + imax + 1;
  }
  const int per = ((total + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kbeg = split * per, kend = min(klimit, kbeg + per);
  const int ntiles = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;

  const T* Q = reinterpret_cast<const T*>(a.q);
  Frag<T> qf[QBW][NS];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    const size_t qrow = (size_t)(b * a.nq + qi[qb]) * a.Hq * HD + (size_t)head[qb] * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qvalid[qb]) {
        lds_frag(qf[qb][s], Q + qrow + s * 32 + g4 * 8);
      } else {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        set_p(qf[qb][s], z);
      }
    }
  }
  const T* Kc = reinterpret_cast<const T*>(a.kc) + ((size_t)b * a.Hkv + kvh) * a.kv_stride * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vc) + ((size_t)b * a.Hkv + kvh) * HD * a.kv_stride;
  f32x4_t o[QBW][NDB];
  float m_run[QBW], l_run[QBW];            // bf16 path: m_run in base-2 units (score * cs)
  // bf16 path: the row sums come from the matrix cores, as a 16-row block of
  // ones times P (every element of osum is the query's running sum of the
  // fp16 P it multiplied into O)
  f32x4_t osum[QBW];
#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[qb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    osum[qb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
  }
  const float cs = a.scale * 1.4426950408889634f;
  const uint4 ones16 = make_uint4(0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u);

  uint4 kr0[KCH], vr0[VCH], kr1[KCH], vr1[VCH];
  // K rows past the range are clamped to its last key; V^T rows are padded to
  // whole tiles (finite past the context), so every load is in bounds
  auto gload = [&](auto slot, int t) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    const int k0 = kbeg + t * KT;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NTH * i, key = min(k0 + c / CH_PER_KEY, kend - 1);
      const uint4 v = *reinterpret_cast<const uint4*>(Kc + (size_t)key * HD + (c % CH_PER_KEY) * EPC);
      if constexpr (SL == 0) kr0[i] = v; else kr1[i] = v;
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + NTH * i, d = c / (KT / EPC), kc = (c % (KT / EPC)) * EPC;
      const uint4 v = *reinterpret_cast<const uint4*>(Vt + (size_t)d * a.kv_stride + k0 + kc);
      if constexpr (SL == 0) vr0[i] = v; else vr1[i] = v;
    }
  };
  auto sstore = [&](auto slot, int buf) __attribute__((always_inline)) {
    constexpr int SL = decltype(slot)::value;
    T* sK = smem + buf * (KBUF + VBUF);
    T* sV = sK + KBUF;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + NTH * i;
      const int kr = c / CH_PER_KEY;
      *reinterpret_cast<uint4*>(sK + kr * LDK + ((c % CH_PER_KEY) ^ kswz(kr)) * EPC) = SL == 0 ? kr0[i] : kr1[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + NTH * i;
      uint4 v = SL == 0 ? vr0[i] : vr1[i];
      if constexpr (sizeof(T) == 2) v = bf16x8_to_f16x8(v);
      *reinterpret_cast<uint4*>(sV + (c / (KT / EPC)) * LDV + (c % (KT / EPC)) * EPC) = v;
    }
    if constexpr (sizeof(T) == 2) {
      uint32_t em = 0;
#pragma unroll
      for (int i = 0; i < VCH; ++i) em = max(em, bf16x8_max_exp(SL == 0 ? vr0[i] : vr1[i]));
      const bool hi = __ballot(em >= kF16ExpHi) != 0, nrm = __ballot(em >= kF16ExpLo) != 0;
      if (lane == 0) s_vflag[buf][w] = (hi ? 1u : 0u) | (nrm ? 2u : 0u);
    }
  };
  // After the barrier that publishes stage `buf`: a tile outside fp16's range
  // is staged again, scaled by 2^-s (workgroup-uniform branch), and s kept for
  // its products; 0 for a tile staged as is.
  int vsc0 = 0, vsc1 = 0;
  auto vrange = [&](auto slot, int buf) __attribute__((always_inline)) {
    if constexpr (sizeof(T) == 2) {
      constexpr int SL = decltype(slot)::value;
      uint32_t f = 0;
#pragma unroll
      for (int j = 0; j < NWQ; ++j) f |= s_vflag[buf][j];
      f = __builtin_amdgcn_readfirstlane(f);
      int sc = 0;
      if ((f & 1u) || !(f & 2u)) {
        uint32_t em = 0;
#pragma unroll
        for (int i = 0; i < VCH; ++i) em = max(em, bf16x8_max_exp(SL == 0 ? vr0[i] : vr1[i]));
        em = wave_max_u32(em);
        if (lane == 0) s_vexp[w] = em;
        lds_barrier();
        uint32_t e = 0;
#pragma unroll
        for (int j = 0; j < NWQ; ++j) e = max(e, s_vexp[j]);
        e = __builtin_amdgcn_readfirstlane(e);
        sc = min(max((int)e - 127 - 14, -100), 113);   // never 0 here: e >= 143 or e < 113
        T* sV = smem + buf * (KBUF + VBUF) + KBUF;
#pragma unroll
        for (int i = 0; i < VCH; ++i) {
          const int c = tid + NTH * i;
          *reinterpret_cast<uint4*>(sV + (c / (KT / EPC)) * LDV + (c % (KT / EPC)) * EPC) =
              bf16x8_to_f16x8_scaled(SL == 0 ? vr0[i] : vr1[i], sc);
        }
        lds_barrier();
      }
      if (buf == 0) vsc0 = sc; else vsc1 = sc;
    }
  };
  auto compute = [&](int buf, int t) __attribute__((always_inline)) {
    const T* sK = smem + buf * (KBUF + VBUF);
    const T* sV = sK + KBUF;
    const int k0 = kbeg + t * KT;
    // scores S^T[key][query] for the 64 keys of the tile; each K fragment
    // serves every query block of the wave
    f32x4_t sc[QBW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) sc[qb][kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        Frag<T> kf;
        const int key = tile_key(kb, q16);
        if constexpr (KSWZ)
          lds_frag(kf, sK + key * LDK + ((s * 4 + g4) ^ kswz(key)) * EPC);
        else
          lds_frag(kf, sK + key * LDK + s * 32 + g4 * 8);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) mma16x16x32(sc[qb][kb], kf, qf[qb][s]);
      }
    }
    if constexpr (sizeof(T) == 2) {
      uint4 pf[QBW][2];                                    // fp16 exp2(z - m), two 32-key steps per block
#pragma unroll
      for (int qb = 0; qb < QBW; ++qb) {
        // masks only where a tile crosses the end of the range or the causal diagonal
        if (k0 + KT > kend || a.causal) {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int kpos = k0 + tile_key(kb, g4 * 4 + i);
              if (kpos >= kend || (a.causal && kpos > qpos[qb])) sc[qb][kb][i] = -INFINITY;
            }
        }
        // online softmax in base-2 units: z = score * scale * log2(e)
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[qb][kb][i]);
        tmax = max_over_g4(tmax);
        const float m_new = fmaxf(m_run[qb], tmax * cs);
        const float mo = m_new == -INFINITY ? 0.f : m_new;   // a row with no key yet: every term is 0
        if (__ballot(m_new != m_run[qb]) != 0) {             // rescale only when some running max moved
          const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mo);
          osum[qb] *= alpha;
#pragma unroll
          for (int j = 0; j < NDB; ++j) o[qb][j] *= alpha;
        }
        m_run[qb] = m_new;
        uint32_t ph[8];                                      // fp16 pairs, keys in tile order
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          float e[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) e[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][kb][i], cs, -mo));
          ph[kb * 2] = f32x2_to_f16x2(e[0], e[1]);
          ph[kb * 2 + 1] = f32x2_to_f16x2(e[2], e[3]);
        }
        pf[qb][0] = make_uint4(ph[0], ph[1], ph[2], ph[3]);
        pf[qb][1] = make_uint4(ph[4], ph[5], ph[6], ph[7]);
      }
      // O^T[d][q] += V^T[d][keys] P[keys][q]; each V^T fragment serves every query block
      const int vs = buf == 0 ? vsc0 : vsc1;
      if (vs != 0) {                       // the tile was staged as V * 2^-vs
        const float f = __builtin_amdgcn_ldexpf(1.f, -vs);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= f;
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const uint4 vf = *reinterpret_cast<const uint4*>(sV + (db * 16 + q16) * LDV + ks * 32 + g4 * 8);
#pragma unroll
          for (int qb = 0; qb < QBW; ++qb) mma16x16x32_f16(o[qb][db], vf, pf[qb][ks]);
        }
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb) mma16x16x32_f16(osum[qb], ones16, pf[qb][ks]);
      }
      if (vs != 0) {
        const float f = __builtin_amdgcn_ldexpf(1.f, vs);
#pragma unroll
        for (int qb = 0; qb < QBW; ++qb)
#pragma unroll
          for (int db = 0; db < NDB; ++db) o[qb][db] *= f;
      }
    } else {
      float p[16];
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kpos = k0 + tile_key(kb, g4 * 4 + i);
          float v = sc[0][kb][i] * a.scale;
          if (kpos >= kend || (a.causal && kpos > qpos[0])) v = -INFINITY;
          p[kb * 4 + i] = v;
          tmax = fmaxf(tmax, v);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float m_new = fmaxf(m_run[0], tmax);
      const float alpha = (m_new == -INFINITY) ? 1.f : exp_fast(m_run[0] - m_new);
      float lsum = 0.f;
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = (p[j] == -INFINITY) ? 0.f : exp_fast(p[j] - m_new);
        p[j] = e;
        lsum += e;
      }
      l_run[0] = l_run[0] * alpha + lsum;
      m_run[0] = m_new;
#pragma unroll
      for (int j = 0; j < NDB; ++j) o[0][j] *= alpha;
      // O^T[d][q] += V^T[d][keys] P[keys][q], two 32-key steps (fp32 operands)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag<T> pfr[NT];
        float rest[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rest[i] = p[(2 * ks) * 4 + i];
          rest[4 + i] = p[(2 * ks + 1) * 4 + i];
        }
        split_p(pfr, rest);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          Frag<T> vf;
          lds_frag(vf, sV + (db * 16 + q16) * LDV + ks * 32 + g4 * 8);
#pragma unroll
          for (int term = 0; term < NT; ++term) mma16x16x32(o[0][db], vf, pfr[term]);
        }
      }
    }
  };

  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  // tile t: its data came through register slot t % 2 into LDS stage t % 2.
  // Tile t + 2 is loaded into slot t % 2 while tile t is computed; tile t + 1
  // (slot (t + 1) % 2, loaded during tile t - 1) is staged at the end.
  // vrange(slot, stage) follows each barrier that publishes a staged tile,
  // while its register slot still holds the tile.
  if (ntiles > 0) {
    gload(S0{}, 0);
    gload(S1{}, min(1, ntiles - 1));
    sstore(S0{}, 0);
    lds_barrier();
    vrange(S0{}, 0);
  }
  int t = 0;
  for (; t + 3 < ntiles; t += 2) {          // every load here exists
    gload(S0{}, t + 2);
    compute(0, t);
    sstore(S1{}, 1);
    lds_barrier();
    vrange(S1{}, 1);
    gload(S1{}, t + 3);
    compute(1, t + 1);
    sstore(S0{}, 0);
    lds_barrier();
    vrange(S0{}, 0);
  }
  // at most three tiles left (t even): loads only for tiles that exist
  if (t < ntiles) {
    if (t + 2 < ntiles) gload(S0{}, t + 2);
    compute(0, t);
    if (t + 1 < ntiles) sstore(S1{}, 1);
    lds_barrier();
    if (t + 1 < ntiles) vrange(S1{}, 1);
  }
  if (t + 1 < ntiles) {
    compute(1, t + 1);
    if (t + 2 < ntiles) sstore(S0{}, 0);
    lds_barrier();
    if (t + 2 < ntiles) vrange(S0{}, 0);
  }
  if (t + 2 < ntiles) compute(0, t + 2);

#pragma unroll
  for (int qb = 0; qb < QBW; ++qb) {
    // full row sum: the matrix-core sums (bf16), else across the four lane
    // groups holding the same query
    if constexpr (sizeof(T) == 2) {
      l_run[qb] = osum[qb][0];
    } else {
      l_run[qb] += __shfl_xor(l_run[qb], 16, 64);
      l_run[qb] += __shfl_xor(l_run[qb], 32, 64);
    }
    if (!qvalid[qb]) continue;
    const size_t qrow = (size_t)(b * a.nq + qi[qb]) * a.Hq * HD + (size_t)head[qb] * HD;
    const size_t rowid = (size_t)(b * a.nq + qi[qb]) * a.Hq + head[qb];
    if (a.splits == 1) {
      T* out = reinterpret_cast<T*>(a.out) + qrow;
      const float inv = 1.f / l_run[qb];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        float v[4] = {o[qb][db][0] * inv, o[qb][db][1] * inv, o[qb][db][2] * inv, o[qb][db][3] * inv};
        store4(out + db * 16 + g4 * 4, v);
      }
    } else {
      // unnormalised partial output in the operand type (rounded once more
      // before the merge, which rounds its result to the operand type too)
      T* po = reinterpret_cast<T*>(a.part_o) + ((size_t)split * a.B * a.nq * a.Hq + rowid) * HD;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const float v[4] = {o[qb][db][0], o[qb][db][1], o[qb][db][2], o[qb][db][3]};
        store4(po + db * 16 + g4 * 4, v);
      }
      if (g4 == 0) {
        float* pm = a.part_ml + ((size_t)split * a.B * a.nq * a.Hq + rowid) * 2;
        pm[0] = sizeof(T) == 2 ? m_run[qb] * 0.6931471805599453f : m_run[qb];   // the merge takes natural units
        pm[1] = l_run[qb];
      }
    }
  }
}

// ---- spread: 16 * QB query rows per workgroup, NW waves taking key tiles round-robin
template <typename T, int HD, int NW, int QB>
__global__ __launch_bounds__(64 * NW) void k_attn_spread(AttnArgs a) {
  constexpr int KT = 64, NS = HD / 32, NDB = HD / 16;
  constexpr int NT = sizeof(T) == 2 ? 2 : 1;
  __shared__ float sm_o[NW][QB][HD][16];
  __shared__ float sm_m[NW][QB][16], sm_l[NW][QB][16], sm_tot[2][QB][16];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g4 = lane >> 4, q16 = lane & 15;
  const int G = a.Hq / a.Hkv, rows_total = G * a.nq;
  const int bk = blockIdx.y, b = bk / a.Hkv, kvh = bk % a.Hkv, split = blockIdx.z;
  const int rho0 = blockIdx.x * 16 * QB;           // < rows_total (grid.x is exact)
  if (!a.gate.active(b)) return;                   // the whole workgroup, before any barrier
  const int ctx = a.pos.base(b);

  bool qv[QB];
  int qpos[QB];
  Frag<T> qf[QB][NS];
  const T* Q = reinterpret_cast<const T*>(a.q);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int rho = rho0 + qb * 16 + q16;
    qv[qb] = rho < rows_total;
    const int hh = qv[qb] ? rho / a.nq : 0, qi = qv[qb] ? rho % a.nq : 0;
    qpos[qb] = ctx + qi;
    const size_t qrow = ((size_t)(b * a.nq + qi) * a.Hq + kvh * G + hh) * HD;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (qv[qb]) {
        lds_frag(qf[qb][s], Q + qrow + s * 32 + g4 * 8);
      } else {
        float z[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        set_p(qf[qb][s], z);
      }
    }
  }

  // key range of this workgroup (one split)
  const int total = ctx + a.nq;
  int klimit = total;
  if (a.causal) {
    const int last = min(rho0 + 16 * QB - 1, rows_total - 1);
    const int imax = (rho0 / a.nq == last / a.nq) ? last % a.nq : a.nq - 1;
    klimit = ctx + imax + 1;
  }
  const int per = ((total + a.splits - 1) / a.splits + KT - 1) / KT * KT;
  const int kbeg = split * per, kend = min(klimit, kbeg + per);
  const int ntiles = kend > kbeg ? (kend - kbeg + KT - 1) / KT : 0;

  const T* Kc = reinterpret_cast<const T*>(a.kc) + ((size_t)b * a.Hkv + kvh) * a.kv_stride * HD;
  const T* Vt = reinterpret_cast<const T*>(a.vc) + ((size_t)b * a.Hkv + kvh) * HD * a.kv_stride;

  f32x4_t o[QB][NDB];
  float m_run[QB], l_run[QB];              // m_run in base-2 units (score * cs)
  const float cs = a.scale * 1.4426950408889634f;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -INFINITY;
    l_run[qb] = 0.f;
#pragma unroll
    for (int j = 0; j < NDB; ++j) o[qb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // fragments of one tile: K rows (A of S^T, rows in tile_key order) and V^T
  // rows (A of O^T: keys ks*32 + g4*8 .. +7, matching P's layout)
  Frag<T> kf[2][4][NS], vf[2][2][NDB];
  auto load = [&](int buf, int t) {
    const int k0 = kbeg + t * KT;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = min(k0 + tile_key(kb, q16), kend - 1);
#pragma unroll
      for (int s = 0; s < NS; ++s) lds_frag(kf[buf][kb][s], Kc + (size_t)key * HD + s * 32 + g4 * 8);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        lds_frag(vf[buf][ks][db], Vt + (size_t)(db * 16 + q16) * a.kv_stride + k0 + ks * 32 + g4 * 8);
  };
  auto compute = [&](int buf, int t) {
    const int k0 = kbeg + t * KT;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      f32x4_t sc[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        sc[kb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NS; ++s) mma16x16x32(sc[kb], kf[buf][kb][s], qf[qb][s]);
      }
      // masks only where a tile crosses the end of the range or the causal diagonal
      if (k0 + KT > kend || a.causal) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kpos = k0 + tile_key(kb, g4 * 4 + i);
            if (kpos >= kend || (a.causal && kpos > qpos[qb])) sc[kb][i] = -INFINITY;
          }
      }
      // online softmax in base-2 units: z = score * scale * log2(e)
      float tmax = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[kb][i]);
      tmax = max_over_g4(tmax);
      const float m_new = fmaxf(m_run[qb], tmax * cs);
      const float mo = m_new == -INFINITY ? 0.f : m_new;   // a row with no key yet: every term is 0
      if (__ballot(m_new != m_run[qb]) != 0) {             // rescale only when some running max moved
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - mo);
        l_run[qb] *= alpha;
#pragma unroll
        for (int j = 0; j < NDB; ++j) o[qb][j] *= alpha;
      }
      m_run[qb] = m_new;
      float p[16];
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][i], cs, -mo));
          p[kb * 4 + i] = e;
          lsum += e;
        }
      l_run[qb] += lsum;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        Frag<T> pf[NT];
        float rest[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          rest[i] = p[(2 * ks) * 4 + i];
          rest[4 + i] = p[(2 * ks + 1) * 4 + i];
        }
        split_p(pf, rest);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int term = 0; term < NT; ++term) mma16x16x32(o[qb][db], vf[buf][ks][db], pf[term]);
      }
    }
  };
  // the wave's tiles w, w + NW, ...: the next one is loaded (unconditionally,
  // clamped to the last tile) while the current one is computed (a three-tile
  // ring was measured slower on the small canvas shape: 12.7 against 11.0 us)
  if (w < ntiles) load(0, w);
  for (int t0 = w; t0 < ntiles; t0 += 2 * NW) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int t = t0 + u * NW;
      if (t >= ntiles) break;
      load(u ^ 1, min(t + NW, ntiles - 1));
      compute(u, t);
    }
  }

  // merge the waves' partials in wave order
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    l_run[qb] += __shfl_xor(l_run[qb], 16, 64);
    l_run[qb] += __shfl_xor(l_run[qb], 32, 64);
    if (g4 == 0) {
      sm_m[w][qb][q16] = m_run[qb];
      sm_l[w][qb][q16] = l_run[qb];
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) sm_o[w][qb][db * 16 + g4 * 4 + i][q16] = o[qb][db][i];
  }
  __syncthreads();
  // per (query, wave): rescale factor exp(m_w - M) and the total 1 / sum (or M, sum for a split)
  if (threadIdx.x < QB * 16) {
    const int qb = threadIdx.x / 16, q = threadIdx.x % 16;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, sm_m[v][qb][q]);
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
      const float mv = sm_m[v][qb][q];
      const float f = mv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mv - M);
      L += f * sm_l[v][qb][q];
      sm_m[v][qb][q] = f;                       // the slot now holds the wave's factor
    }
    sm_tot[0][qb][q] = M * 0.6931471805599453f;   // natural units for the split merge
    sm_tot[1][qb][q] = L;
  }
  __syncthreads();
  const size_t nrows = (size_t)a.B * a.nq * a.Hq;
  for (int e = threadIdx.x; e < QB * 16 * HD; e += 64 * NW) {
    const int d = e % HD, q = (e / HD) % 16, qb = e / (16 * HD);
    const int rho = rho0 + qb * 16 + q;
    if (rho >= rows_total) continue;
    float O = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) O += sm_m[v][qb][q] * sm_o[v][qb][d][q];
    const float M = sm_tot[0][qb][q], L = sm_tot[1][qb][q];
    const int hh = rho / a.nq, qi = rho % a.nq;
    const size_t rowid = (size_t)(b * a.nq + qi) * a.Hq + kvh * G + hh;
    if (a.splits == 1) {
      Num<T>::store(reinterpret_cast<T*>(a.out) + rowid * HD + d, O / L);
    } else {
      Num<T>::store(reinterpret_cast<T*>(a.part_o) + ((size_t)split * nrows + rowid) * HD + d, O);
      if (d == 0) {
        a.part_ml[((size_t)split * nrows + rowid) * 2] = M;
        a.part_ml[((size_t)split * nrows + rowid) * 2 + 1] = L;
      }
    }
  }
}

// One thread per (row, kMergeDims<T> dims -- 16 bytes of partial output per
// split): combine the split partials in split order.
constexpr int kMaxAttnSplits = 16;   // key splits of one launch (the merge unrolls over them)
template <typename T> constexpr int kMergeDims = 16 / (int)sizeof(T);

template <typename T, int HD>
__global__ __launch_bounds__(256) void k_attn_merge(AttnArgs a) {
  constexpr int V = kMergeDims<T>;
  const size_t nrows = (size_t)a.B * a.nq * a.Hq;
  const size_t gid = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t rowid = gid / (HD / V);
  const int d0 = (int)(gid % (HD / V)) * V;
  if (rowid >= nrows || !a.gate.active((int)(rowid / a.Hq / a.nq))) return;
  // every split's (max, sum) and output piece are loaded before the first
  // use (at most kMaxAttnSplits), so the loads are one round trip, not one per split
  float2 ml[kMaxAttnSplits];
  float4 po[kMaxAttnSplits][V / 4];
  const T* part = reinterpret_cast<const T*>(a.part_o);
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s) {
    if (s < a.splits) {
      ml[s] = *reinterpret_cast<const float2*>(a.part_ml + (s * nrows + rowid) * 2);
#pragma unroll
      for (int h = 0; h < V / 4; ++h) po[s][h] = load4(part + (s * nrows + rowid) * HD + d0 + 4 * h);
    }
  }
  float m = -INFINITY;
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s)
    if (s < a.splits) m = fmaxf(m, ml[s].x);
  float l = 0.f, acc[V];
#pragma unroll
  for (int i = 0; i < V; ++i) acc[i] = 0.f;
#pragma unroll
  for (int s = 0; s < kMaxAttnSplits; ++s) {
    if (s >= a.splits || ml[s].x == -INFINITY) continue;
    const float f = expf(ml[s].x - m);
    l += ml[s].y * f;
#pragma unroll
    for (int h = 0; h < V / 4; ++h) {
      acc[4 * h] += po[s][h].x * f; acc[4 * h + 1] += po[s][h].y * f;
      acc[4 * h + 2] += po[s][h].z * f; acc[4 * h + 3] += po[s][h].w * f;
    }
  }
  const float inv = 1.f / l;
  const int head = (int)(rowid % a.Hq);
  const size_t tok = rowid / a.Hq;
  T* out = reinterpret_cast<T*>(a.out) + tok * (size_t)a.Hq * HD + (size_t)head * HD + d0;
#pragma unroll
  for (int h = 0; h < V / 4; ++h) {
    float v[4] = {acc[4 * h] * inv, acc[4 * h + 1] * inv, acc[4 * h + 2] * inv, acc[4 * h + 3] * inv};
    store4(out + 4 * h, v);
  }
}

// Launch shape.  Spread while the K/V bytes its 16-row query blocks re-read
// stay small (measured on MI355X: 768 keys, 16/4 heads x 64, 50 MB: spread
// 10.4 us against 13.1 us wide); wide otherwise (2304 keys, 16/8 x 128:
// 51.8 -> 29.1 us; 9216 keys, 16/4 x 64: 80.8 -> 44.5 us; 32 requests x 4352
// keys: 842 -> 414 us).
constexpr int kSpreadNW = 4, kSpreadQB = 1, kWideNWQ = 8;
// Query blocks per wave of the wide kernel.  Two (256 query rows per
// workgroup share each staged K/V tile, halving the K/V bytes re-read through
// L2 per query) for bf16 with 64-dim heads when that still leaves ~256
// workgroups without key splits (many requests; measured 250 -> 230 us per
// layer at 32 x 256 rows and 4352 keys).  Else one: at batch 1 the halved
// workgroup count asks for twice the key splits (multi-canvas, 8448 keys:
// 34 -> 39 us), and 128-dim heads would spill.
inline int wide_qbw(int elem_bytes, int hd, int B, int nq, int Hq, int Hkv) {
  if (elem_bytes != 2 || hd != 64) return 1;
  const int rows = 16 * kWideNWQ * 2;
  return ((Hq / Hkv) * nq + rows - 1) / rows * B * Hkv >= 256 ? 2 : 1;
}
constexpr double kSpreadMaxBytes = 128.0 * (1 << 20);
inline bool use_spread(int B, int nq, int Hq, int Hkv, int hd, int keys) {
  const double blocks = (double)(((Hq / Hkv) * nq + 15) / 16) * B * Hkv;
  return blocks * keys * hd * 4.0 <= kSpreadMaxBytes && ((Hq / Hkv) * nq + 63) / 64 * B * Hkv < 128;
}

template <typename T, int HD>
hipError_t launch_attn(const AttnArgs& a, hipStream_t s) {
  const int G = a.Hq / a.Hkv;
  if (use_spread(a.B, a.nq, a.Hq, a.Hkv, HD, a.keys_max)) {
    constexpr int NW = kSpreadNW, QB = kSpreadQB;
    dim3 grid((G * a.nq + 16 * QB - 1) / (16 * QB), a.B * a.Hkv, a.splits);
    hipLaunchKernelGGL((k_attn_spread<T, HD, NW, QB>), grid, dim3(64 * NW), 0, s, a);
  } else {
    constexpr int NWQ = kWideNWQ;
    if (wide_qbw((int)sizeof(T), HD, a.B, a.nq, a.Hq, a.Hkv) == 2) {
      if constexpr (sizeof(T) == 2 && HD == 64) {
        dim3 grid((G * a.nq + 32 * NWQ - 1) / (32 * NWQ), a.B * a.Hkv, a.splits);
        hipLaunchKernelGGL((k_attn_wide<T, HD, NWQ, 2>), grid, dim3(64 * NWQ), 0, s, a);
      }
    } else {
      dim3 grid((G * a.nq + 16 * NWQ - 1) / (16 * NWQ), a.B * a.Hkv, a.splits);
      hipLaunchKernelGGL((k_attn_wide<T, HD, NWQ, 1>), grid, dim3(64 * NWQ), 0, s, a);
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const size_t threads = (size_t)a.B * a.nq * a.Hq * (HD / kMergeDims<T>);
  hipLaunchKernelGGL((k_attn_merge<T, HD>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

// Key splits (and the merge launch they need): spread -- at most 8 tiles per
// wave; wide -- only as many as filling the chip (~256 workgroups) asks, with
// at least four tiles per split.
int attention_splits(int B, int nq, int Hq, int Hkv, int hd, int keys, int elem_bytes) {
  const int tiles = (keys + 63) / 64;
  int splits;
  if (use_spread(B, nq, Hq, Hkv, hd, keys)) {
    splits = (tiles + 8 * kSpreadNW - 1) / (8 * kSpreadNW);
  } else {
    const int rows = 16 * kWideNWQ * wide_qbw(elem_bytes, hd, B, nq, Hq, Hkv);
    const int wg = ((Hq / Hkv) * nq + rows - 1) / rows * B * Hkv;
    splits = (256 + wg - 1) / wg;
    const int max_by_keys = tiles / 4;
    if (splits > max_by_keys) splits = max_by_keys;
  }
  if (splits > kMaxAttnSplits) splits = kMaxAttnSplits;
  if (splits < 1) splits = 1;
  return splits;
}

int attention_launch_class(int B, int nq, int Hq, int Hkv, int hd, int keys) {
  return use_spread(B, nq, Hq, Hkv, hd, keys) ? 0 : 1;
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

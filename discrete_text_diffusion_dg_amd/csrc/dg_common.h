// Device-side building blocks shared by the gfx950 kernels of the denoise step.
#pragma once
#include <type_traits>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dg {

// ------------------------------------------------------------------ types
// bfloat16 is kept as raw bits in memory; arithmetic is always fp32.
struct bf16 {
  uint16_t bits;
};

// OCP FP8 E4M3 storage (1 sign, 4 exponent bits with bias 7, 3 mantissa bits,
// no infinities, largest finite 448): expert weights of FP8 models.
struct fp8e4m3 {
  uint8_t bits;
};

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Round to nearest, ties to even: the gfx950 packed converter (v_cvt_pk_bf16_f32,
// rounding per the default mode, nearest-even), two values per instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float a, float b) {
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return (uint16_t)f32x2_to_bf16x2(f, 0.f); }

// Eight E4M3 values (bytes of w0, then w1) -> eight bf16 (an MFMA fragment):
// the gfx950 converter takes two bytes to two fp32 values, which bf16 holds
// exactly (every E4M3 value has at most 4 significant bits).
__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint32_t w0, uint32_t w1) {
  const f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, false), b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w0, true);
  const f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, false), d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w1, true);
  return make_uint4(f32x2_to_bf16x2(a[0], a[1]), f32x2_to_bf16x2(b[0], b[1]), f32x2_to_bf16x2(c[0], c[1]),
                    f32x2_to_bf16x2(d[0], d[1]));
}

// fp32 -> E4M3 code, round to nearest even, saturating at +-448 (the OCP
// specification's saturating conversion; inputs are finite).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (!(a <= 448.f)) {
    code = 0x7Eu;
  } else if (a < 0.015625f) {                     // below 2^-6: subnormal steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.f);  // exact scaling, ties to even; 8 is the smallest normal
  } else {
    const uint32_t au = __float_as_uint(a);
    int e = (int)(au >> 23) - 127;                // -6 .. 8
    uint32_t m3 = (au >> 20) & 7u;
    const uint32_t rest = au & 0xFFFFFu;          // the 20 bits rounded away
    if (rest > 0x80000u || (rest == 0x80000u && (m3 & 1u))) ++m3;
    if (m3 == 8u) { m3 = 0; ++e; }
    code = e > 8 ? 0x7Eu : ((uint32_t)(e + 7) << 3) | m3;
  }
  return sign | code;
}

template <typename T> struct Num;
template <> struct Num<float> {
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static float round(float v) { return v; }
};
template <> struct Num<bf16> {
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load(const bf16* p) { return bf16_to_f32(p->bits); }
  __device__ __forceinline__ static void store(bf16* p, float v) { p->bits = f32_to_bf16_bits(v); }
  __device__ __forceinline__ static float round(float v) { return bf16_to_f32(f32_to_bf16_bits(v)); }
};

// Pack 8 fp32 values into 16 bytes (bf16) or 32 bytes (fp32) of operand data.
__device__ __forceinline__ uint4 pack8_bf16(const float* v) {
  uint4 r;
  r.x = f32x2_to_bf16x2(v[0], v[1]);
  r.y = f32x2_to_bf16x2(v[2], v[3]);
  r.z = f32x2_to_bf16x2(v[4], v[5]);
  r.w = f32x2_to_bf16x2(v[6], v[7]);
  return r;
}

// ------------------------------------------------------------------ MFMA
// Fragment: 8 consecutive k-elements of one row (A) or one column (B) per lane.
// Lane l supplies row/column (l & 15); its lane group g = l >> 4 supplies the
// k-elements g*8 .. g*8+7 of a 32-wide k step.  A and B use the same mapping,
// so the products pair up whatever order the unit sums them in.
// Accumulator: lane l holds C[(l>>4)*4 + i][l & 15], i = 0..3.
template <typename T> struct Frag;
template <> struct Frag<bf16> {
  uint4 v;  // 8 bf16
};
template <> struct Frag<float> {
  float v[8];
};

__device__ __forceinline__ void mma16x16x32(f32x4_t& acc, const Frag<bf16>& a, const Frag<bf16>& b) {
  bf16x8_t av = __builtin_bit_cast(bf16x8_t, a.v);
  bf16x8_t bv = __builtin_bit_cast(bf16x8_t, b.v);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma16x16x32(f32x4_t& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// Load a fragment from shared memory: 8 consecutive elements starting at p.
__device__ __forceinline__ void lds_frag(Frag<bf16>& f, const bf16* p) {
  f.v = *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void lds_frag(Frag<float>& f, const float* p) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
  f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
}

// e^x through the hardware base-2 exponential (about 1 ulp; x <= 0 here).
__device__ __forceinline__ float exp_fast(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
// SwiGLU of one (gate, up) pair: silu(g) * u = g * u / (1 + exp(-g)), with the
// hardware exp2 and reciprocal (about 1 ulp each, far below the operand
// rounding the product then gets).  For g below about -88, exp(-g) is +inf and
// the value is -0 (the limit); above, 1 + exp(-g) rounds to 1.
__device__ __forceinline__ float swiglu(float g, float u) {
  const float den = 1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * u * __builtin_amdgcn_rcpf(den);
}

// ------------------------------------------------------------------ reductions
// Wave-wide butterflies in six lane-exchange steps, all plain VALU moves (the
// shuffles they replace go through the LDS crossbar): DPP moves inside rows
// of 16 lanes -- pairs, quads, mirrored half rows, mirrored rows -- then the
// gfx950 row swaps (rows 0/1 and 2/3, then the two halves).  Each step pairs
// every lane with one partner (an involution), so after step s every lane
// holds the combination of its 2^(s+1) lanes; with a commutative merge the
// two lanes of a pair compute the same value.
template <int S>
__device__ __forceinline__ uint32_t lane_partner(uint32_t v) {
  if constexpr (S == 0) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);    // quad_perm 1,0,3,2
  } else if constexpr (S == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);    // quad_perm 2,3,0,1
  } else if constexpr (S == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false);   // row_half_mirror
  } else if constexpr (S == 3) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false);   // row_mirror
  } else if constexpr (S == 4) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);         // rows 0/1, 2/3
    return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);         // halves
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}
template <int S>
__device__ __forceinline__ float lane_partner(float v) { return __uint_as_float(lane_partner<S>(__float_as_uint(v))); }
template <int S>
__device__ __forceinline__ int lane_partner(int v) { return (int)lane_partner<S>((uint32_t)v); }
template <int S>
__device__ __forceinline__ double lane_partner(double v) {
  const uint64_t u = __double_as_longlong(v);
  const uint64_t p = ((uint64_t)lane_partner<S>((uint32_t)(u >> 32)) << 32) | lane_partner<S>((uint32_t)u);
  return __longlong_as_double((long long)p);
}
// f(step) for the six steps, each with its step as a compile-time constant
template <class F>
__device__ __forceinline__ void butterfly_steps(F&& f) {
  f(std::integral_constant<int, 0>{}); f(std::integral_constant<int, 1>{}); f(std::integral_constant<int, 2>{});
  f(std::integral_constant<int, 3>{}); f(std::integral_constant<int, 4>{}); f(std::integral_constant<int, 5>{});
}
__device__ __forceinline__ float wave_sum(float v) {
  butterfly_steps([&](auto st) { v += lane_partner<decltype(st)::value>(v); });
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  butterfly_steps([&](auto st) { v = fmaxf(v, lane_partner<decltype(st)::value>(v)); });
  return v;
}

// Workgroups are dealt round-robin over the 8 XCDs (workgroup bid runs on XCD
// bid % 8), each with its own L2; xcd_run gives XCD x a contiguous run of the
// `total` logical tiles (bid < total), so neighbouring tiles meet in one L2.
__device__ __forceinline__ int xcd_run(int bid, int total) {
  const int q = total >> 3, r = total & 7, x = bid & 7;
  return x * q + min(x, r) + (bid >> 3);
}

// Workgroup barrier for LDS hand-overs: orders this wave's LDS writes before
// the barrier and the other waves' LDS reads after it (s_waitcnt lgkmcnt(0);
// s_barrier), without waiting for the wave's outstanding global loads, which
// __syncthreads() would drain.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// ------------------------------------------------------------------ Philox4x32-10
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds of two 32x32->64 multiplies, xor with the key and the
// odd counter words, key advanced by the Weyl constants between rounds.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    // each 32x32 -> 64-bit product is one multiply-add on the vector unit
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    // three-way xors in one instruction each (gfx950 v_bitop3_b32, truth table 0x96 = odd parity)
    c = make_uint4(__builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96), (uint32_t)p1,
                   __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96), (uint32_t)p0);
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c;
}

enum : uint32_t { kTagInit = 2, kTagGumbel = 3, kTagRenoise = 4, kTagCorrupt = 5 };

// Counter layout: (j >> 2, position, step, tag << 24 | canvas), output word j & 3.
__device__ __forceinline__ uint4 philox_block(uint64_t seed, uint32_t tag, uint32_t canvas,
                                              uint32_t step, uint32_t pos, uint32_t jblock) {
  uint4 c = make_uint4(jblock, pos, step, (tag << 24) | (canvas & 0xFFFFFFu));
  return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// Uniform in (0, 1): (2 * (x >> 9) + 1) * 2^-24, exact in fp32.
__device__ __forceinline__ float u01(uint32_t x) {
  return (float)(2u * (x >> 9) + 1u) * 5.9604644775390625e-08f;
}
// Gumbel draw -log(-log u) through the hardware base-2 logarithm: over every
// uniform of the (2q + 1) 2^-24 grid it stays within 1.6e-6 of the value
// evaluated in fp64 (measured exhaustively on MI355X; the accurate logf path
// is within 1.9e-6), so no per-draw library calls are needed.
__device__ __forceinline__ float gumbel_of(uint32_t x) {
  const float e = -__builtin_amdgcn_logf(u01(x)) * 0.6931471805599453f;    // -ln u
  return -__builtin_amdgcn_logf(e) * 0.6931471805599453f;
}
__device__ __forceinline__ int32_t token_of(uint32_t x, int32_t vocab) {
  return (int32_t)(((uint64_t)x * (uint64_t)(uint32_t)vocab) >> 32);
}

}  // namespace dg

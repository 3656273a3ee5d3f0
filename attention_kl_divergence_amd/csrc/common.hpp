// Device helpers shared by the StreamKL kernels: MFMA operand fragments for
// CDNA4 (gfx950) 32x32 matrix instructions, base-2 exponentials, the
// five-scalar running state and its merge rule.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace streamkl {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// One wave64 computes a 32x32 fp32 tile C += A (32 x K) * B (K x 32).
// Operand layout per lane l (col = l % 32, grp = l / 32):
//   A: row `col`, k values [step*KSTEP + grp*KPL, +KPL)
//   B: column `col`, the same k values
//   C: column `col`, rows 8*(e/4) + 4*grp + (e%4) for element e = 0..15
// Any permutation of k works as long as A and B use the same one.
template <typename T> struct Mfma;

template <> struct Mfma<bf16> {
  static constexpr int KSTEP = 16;
  static constexpr int KPL = 8;
  using frag = bf16x8;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mfma<float> {
  static constexpr int KSTEP = 2;
  static constexpr int KPL = 1;
  using frag = float;
  __device__ static inline f32x16 run(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int e = 0; e < 16; ++e) z[e] = 0.f;
  return z;
}

// Row (within a 32-row block) held by accumulator element e of lane group grp.
__device__ __forceinline__ int acc_row(int e, int grp) { return 8 * (e >> 2) + 4 * grp + (e & 3); }

// A-operand fragment built from a 32x32 accumulator whose lane column is the
// operand's row; contraction runs over the accumulator's rows in the order
// acc_row(h*KPL + e', grp).
__device__ __forceinline__ bf16x8 frag_from_acc(const f32x16& c, int h, bf16) {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (bf16)c[8 * h + e];
  return f;
}
__device__ __forceinline__ float frag_from_acc(const f32x16& c, int h, float) { return c[h]; }

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }


// The five running scalars of one (partial) row, in base-2 units:
// M_t = running max of y_t = S_t * log2(e), l_t = sum 2^(y_t - M_t),
// A = sum 2^(y1 - M1) (y1 - y2).  Empty state: (-inf, 0, 0, -inf, 0).
struct RowState {
  float M1, l1, A, M2, l2;
};

__device__ __forceinline__ RowState empty_state() { return {kNegInf, 0.f, 0.f, kNegInf, 0.f}; }

__device__ __forceinline__ float finite_or_zero(float m) { return m == kNegInf ? 0.f : m; }

// Associative merge of two partial states over disjoint key sets.
__device__ __forceinline__ RowState merge_state(const RowState& a, const RowState& b) {
  RowState r;
  r.M1 = fmaxf(a.M1, b.M1);
  r.M2 = fmaxf(a.M2, b.M2);
  const float m1 = finite_or_zero(r.M1), m2 = finite_or_zero(r.M2);
  const float wa1 = exp2_fast(a.M1 - m1), wb1 = exp2_fast(b.M1 - m1);
  const float wa2 = exp2_fast(a.M2 - m2), wb2 = exp2_fast(b.M2 - m2);
  r.l1 = wa1 * a.l1 + wb1 * b.l1;
  r.A = wa1 * a.A + wb1 * b.A;
  r.l2 = wa2 * a.l2 + wb2 * b.l2;
  return r;
}

// KL, LSE1, LSE2 (natural units) from a complete row state:
// KL = ln2 * (A / l1 + LSE2_2 - LSE1_2), LSE_t = ln2 * (M_t + log2 l_t).
// Returns the KL it stored.
__device__ __forceinline__ float finish_state(const RowState& s, float* kl, float* lse1, float* lse2) {
  const float L1 = s.M1 + log2f(s.l1);
  const float L2 = s.M2 + log2f(s.l2);
  const float k = kLn2 * (s.A / s.l1 + (L2 - L1));
  *kl = k;
  *lse1 = kLn2 * L1;
  *lse2 = kLn2 * L2;
  return k;
}

__device__ __forceinline__ RowState shfl_xor_state(const RowState& s, int mask) {
  RowState o;
  o.M1 = __shfl_xor(s.M1, mask);
  o.l1 = __shfl_xor(s.l1, mask);
  o.A = __shfl_xor(s.A, mask);
  o.M2 = __shfl_xor(s.M2, mask);
  o.l2 = __shfl_xor(s.l2, mask);
  return o;
}

}  // namespace streamkl

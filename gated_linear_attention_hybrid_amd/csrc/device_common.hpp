// device_common.hpp -- small gfx950 device helpers shared by the HIP kernels of
// the hybrid gated-linear + window attention library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace glah {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 2^x and log2(x) on the transcendental unit (v_exp_f32 / v_log_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float exp_fast(float x) { return exp2_fast(x * kLog2e); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// Element loads/stores with conversion to/from fp32 (bf16 stores round to
// nearest even through v_cvt_pk_bf16_f32).
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <class T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

template <class T> __device__ __forceinline__ float ld(const T *p) { return to_f32(*p); }

// Element offset of the gate of head bh (of H), token t (of L), feature r (of f)
// for gate layout `mode`: 0 = one per feature [BH][L][f], 1 = one per token
// [BH][L], 2 = one per head [H].  The decode step uses L = 1, t = 0.
__device__ __forceinline__ size_t gate_index(int mode, size_t bh, int H, int L, int f, int t, int r) {
  if (mode == 1) return bh * (size_t)L + t;
  if (mode == 2) return bh % (size_t)H;
  return (bh * (size_t)L + t) * f + r;
}

// Gate value Gamma in [0,1] from a logit (sigmoid) or from a log-gate (exp).
__device__ __forceinline__ float gate_from(float g, bool gate_is_log) {
  if (gate_is_log) return exp_fast(g);
  return rcp_fast(1.0f + exp_fast(-g));
}

// log Gamma <= 0 from a logit (log-sigmoid = -softplus(-g)) or a log-gate.
__device__ __forceinline__ float log_gate_from(float g, bool gate_is_log) {
  if (gate_is_log) return g;
  // -softplus(-g) = min(g, 0) - log(1 + e^{-|g|})
  const float e = exp_fast(-fabsf(g));
  return fminf(g, 0.0f) - kLn2 * log2_fast(1.0f + e);
}

// Cross-lane all-reductions without LDS: DPP quad permutes and row rotations
// within each 16-lane row, then the gfx950 row swaps (v_permlane16_swap with
// both operands x gives rows (x0, x0, x2, x2) and (x1, x1, x3, x3);
// v_permlane32_swap gives (x0, x1, x0, x1) and (x2, x3, x2, x3)).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
template <class Op>
__device__ __forceinline__ float rows_reduce(float x, Op op) {  // over the 4 rows
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = op(__builtin_bit_cast(float, (unsigned)p[0]), __builtin_bit_cast(float, (unsigned)p[1]));
  const unsigned w = __builtin_bit_cast(unsigned, x);
  const auto q = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return op(__builtin_bit_cast(float, (unsigned)q[0]), __builtin_bit_cast(float, (unsigned)q[1]));
}
template <class Op>
__device__ __forceinline__ float row16_reduce(float x, Op op) {  // within each 16-lane row
  x = op(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]: lane ^ 1
  x = op(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]: lane ^ 2
  x = op(x, dpp_f<0x124>(x));  // row_ror:4
  return op(x, dpp_f<0x128>(x));  // row_ror:8
}
struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };
struct OpMin { __device__ float operator()(float a, float b) const { return fminf(a, b); } };

__device__ __forceinline__ float wave_sum(float x) { return rows_reduce(row16_reduce(x, OpAdd()), OpAdd()); }
__device__ __forceinline__ float wave_max(float x) { return rows_reduce(row16_reduce(x, OpMax()), OpMax()); }
__device__ __forceinline__ float wave_min(float x) { return rows_reduce(row16_reduce(x, OpMin()), OpMin()); }

}  // namespace glah

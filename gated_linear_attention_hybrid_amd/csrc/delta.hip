// delta.hip -- the gated delta rule (Gated DeltaNet token mixer): a
// token-recurrent prefill and a bandwidth-bound decode step, bf16 or fp32 I/O,
// fp32 state.
//
// The pages recommend Gated DeltaNet for hybrids ("systematic analysis of
// hybrid linear attention", 2507.06457, findings and recommendations; "LT2"
// technical summary, 2605.20670, hybrid designs) and describe its update as an
// error-correcting write with gated forgetting.  Per (b, h), with the state M
// kept as d_v rows of d_k:
//     k^ = k / sqrt(|k|^2 + 1e-6),  q^ likewise
//     M_t = alpha_t M_{t-1} (I - beta_t k^ k^T) + beta_t v_t k^T,  alpha_t = e^{a_t}
//     o_t = M_t q^
// Row i of M only ever meets v_t[i]: m_i <- alpha (m_i - beta (m_i . k^) k^)
// + beta v_i k^ = alpha m_i + beta (v_i - alpha (m_i . k^)) k^, and o_t[i] =
// m_i . q^.  So the d_v rows are independent recurrences and the kernels give
// each row to one 16-lane DPP row of a wave (d_k / 16 elements per lane, d_k
// in {32, 64, 128}): the dot products reduce inside the lane row with DPP, no
// LDS and no barrier.
#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kLPR = 16;                 // lanes per state row
constexpr int kThreads = 256;            // 4 waves x 4 rows = 16 rows per block
constexpr int kRowsPerBlock = kThreads / kLPR;
constexpr float kNormEps = 1e-6f;        // added to |x|^2 under the root
constexpr int kAhead = 8;                // prefill: tokens of operands in flight

struct DeltaParams {
  const void *q, *k, *v, *a, *beta;
  const float *state_in;
  float *state_out;  // prefill: final state (nullable); decode: the state, in place
  void *o;
  int L, dv;
};

template <class T, int N>
struct VecOf {
  typedef T type __attribute__((ext_vector_type(N)));
};

// Operands of one token for one lane, as loaded (widened to fp32 only where
// they are used, so a load in flight never stalls the lane).
template <class T, int EPL>
struct TokenOps {
  typename VecOf<T, EPL>::type k, q;  // this lane's d_k / 16 elements of k_t and q_t
  T v, a, beta;                       // v_t[row], a_t, beta_t
};

template <class T, int EPL>
__device__ __forceinline__ void load_token(const DeltaParams &p, size_t bh, int row, int l16, int t,
                                           TokenOps<T, EPL> &x) {
  typedef typename VecOf<T, EPL>::type vec;
  constexpr int DK = EPL * kLPR;
  const size_t tok = bh * (size_t)p.L + t;
  x.k = *(const vec *)((const T *)p.k + tok * DK + l16 * EPL);
  x.q = *(const vec *)((const T *)p.q + tok * DK + l16 * EPL);
  x.v = ((const T *)p.v)[tok * p.dv + row];
  x.a = ((const T *)p.a)[tok];
  x.beta = ((const T *)p.beta)[tok];
}

// One token of one row: updates m in place and returns o_t[row] (every lane
// of the row holds it).
template <class T, int EPL>
__device__ __forceinline__ float delta_token(float (&m)[EPL], const TokenOps<T, EPL> &x) {
  float k[EPL], q[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    k[e] = to_f32(x.k[e]);
    q[e] = to_f32(x.q[e]);
  }
  float kk = 0.0f, qq = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    kk += k[e] * k[e];
    qq += q[e] * q[e];
  }
  kk = row16_reduce(kk, OpAdd());
  qq = row16_reduce(qq, OpAdd());
  const float rk = __builtin_amdgcn_rsqf(kk + kNormEps);
  const float rq = __builtin_amdgcn_rsqf(qq + kNormEps);
  // recall of the normalised key: (m . k) / |k|
  float mk = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) mk += m[e] * k[e];
  mk = row16_reduce(mk, OpAdd()) * rk;
  const float alpha = exp2_fast(to_f32(x.a) * kLog2e);  // a = -inf gives 0
  const float c = to_f32(x.beta) * (to_f32(x.v) - alpha * mk) * rk;  // coefficient of the raw key
  float mq = 0.0f;
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    m[e] = alpha * m[e] + c * k[e];
    mq += m[e] * q[e];
  }
  return row16_reduce(mq, OpAdd()) * rq;
}

// Prefill: one 16-lane row per state row, the whole sequence in registers.
// Operands are loaded kAhead tokens ahead into a register ring so the serial
// chain of each row never waits on memory.
template <class T, int EPL>
__global__ __launch_bounds__(kThreads) void gdn_prefill_kernel(DeltaParams p) {
  constexpr int DK = EPL * kLPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
  const int nrb = (p.dv + kRowsPerBlock - 1) / kRowsPerBlock;
  const size_t bh = blockIdx.x / nrb;
  const int row0 = (blockIdx.x % nrb) * kRowsPerBlock + wave * 4 + (lane >> 4);
  const bool live = row0 < p.dv;
  const int row = live ? row0 : p.dv - 1;  // rows past d_v compute a copy, store nothing

  float m[EPL];
  if (p.state_in) {
    const float *s = p.state_in + (bh * p.dv + row) * DK + l16 * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = s[e];
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = 0.0f;
  }
  T *o = (T *)p.o + bh * (size_t)p.L * p.dv + row;

  TokenOps<T, EPL> ring[kAhead];
#pragma unroll
  for (int j = 0; j < kAhead; ++j) load_token<T, EPL>(p, bh, row, l16, min(j, p.L - 1), ring[j]);
  for (int t0 = 0; t0 < p.L; t0 += kAhead) {
#pragma unroll
    for (int j = 0; j < kAhead; ++j) {
      const int t = t0 + j;
      if (t < p.L) {
        const float ot = delta_token<T, EPL>(m, ring[j]);
        if (live && l16 == 0) o[(size_t)t * p.dv] = from_f32<T>(ot);
        // refill the slot with token t + kAhead (clamped: the last token is
        // re-read past the end and never used)
        load_token<T, EPL>(p, bh, row, l16, min(t + kAhead, p.L - 1), ring[j]);
      }
    }
  }
  if (p.state_out && live) {
    float *s = p.state_out + (bh * p.dv + row) * DK + l16 * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) s[e] = m[e];
  }
}

// Decode: one token; the state streams from HBM once and back once
// (non-temporal), everything else is a few hundred bytes per head.
template <class T, int EPL>
__global__ __launch_bounds__(kThreads) void gdn_decode_kernel(DeltaParams p) {
  constexpr int DK = EPL * kLPR;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, l16 = lane & 15;
  const int nrb = (p.dv + kRowsPerBlock - 1) / kRowsPerBlock;
  const size_t bh = blockIdx.x / nrb;
  const int row0 = (blockIdx.x % nrb) * kRowsPerBlock + wave * 4 + (lane >> 4);
  const bool live = row0 < p.dv;
  const int row = live ? row0 : p.dv - 1;

  float *s = p.state_out + (bh * p.dv + row) * DK + l16 * EPL;
  float m[EPL];
  if constexpr (EPL % 4 == 0) {
#pragma unroll
    for (int c = 0; c < EPL / 4; ++c) {
      const f32x4 w = __builtin_nontemporal_load((const f32x4 *)(s + 4 * c));
#pragma unroll
      for (int j = 0; j < 4; ++j) m[4 * c + j] = w[j];
    }
  } else {
#pragma unroll
    for (int e = 0; e < EPL; ++e) m[e] = s[e];
  }
  TokenOps<T, EPL> x;
  {
    DeltaParams one = p;
    one.L = 1;
    load_token<T, EPL>(one, bh, row, l16, 0, x);
  }
  const float ot = delta_token<T, EPL>(m, x);
  if (live) {
    if constexpr (EPL % 4 == 0) {
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c)
        __builtin_nontemporal_store((f32x4){m[4 * c], m[4 * c + 1], m[4 * c + 2], m[4 * c + 3]},
                                    (f32x4 *)(s + 4 * c));
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s[e] = m[e];
    }
    if (l16 == 0) ((T *)p.o)[bh * p.dv + row] = from_f32<T>(ot);
  }
}

template <class T, int EPL>
hipError_t launch(const LayerArgs &a, bool decode) {
  DeltaParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.a = a.gate; p.beta = a.beta;
  p.state_in = a.state_in;
  p.state_out = decode ? a.state : a.state_out;
  p.o = a.o;
  p.L = a.L; p.dv = a.dv;
  const size_t nrb = (size_t)(a.dv + kRowsPerBlock - 1) / kRowsPerBlock;
  const dim3 grid((unsigned)((size_t)a.B * a.H * nrb)), block(kThreads);
  if (decode)
    hipLaunchKernelGGL((gdn_decode_kernel<T, EPL>), grid, block, 0, a.stream, p);
  else
    hipLaunchKernelGGL((gdn_prefill_kernel<T, EPL>), grid, block, 0, a.stream, p);
  return hipGetLastError();
}

template <class T>
hipError_t dispatch(const LayerArgs &a, bool decode) {
  switch (a.d) {
    case 32: return launch<T, 2>(a, decode);
    case 64: return launch<T, 4>(a, decode);
    case 128: return launch<T, 8>(a, decode);
  }
  return hipErrorInvalidValue;
}

}  // namespace

bool delta_supported(const LayerArgs &a) {
  return (a.d == 32 || a.d == 64 || a.d == 128) && a.dv >= 1;
}

hipError_t launch_delta(const LayerArgs &a, bool decode) {
  if ((size_t)a.B * a.H == 0 || (!decode && a.L == 0)) return hipSuccess;
  return a.bf16 ? dispatch<bf16>(a, decode) : dispatch<float>(a, decode);
}

}  // namespace glah

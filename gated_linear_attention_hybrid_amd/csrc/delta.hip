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
constexpr int kDecRows = 2 * kRowsPerBlock;  // decode: two state rows per 16-lane group
constexpr float kNormEps = 1e-6f;        // added to |x|^2 under the root

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

// Operands of one decode token for one lane, as loaded.
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

// Sum over groups of G consecutive lanes (G in {4, 8, 16, 32}), every lane
// of a group receiving its group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<0xB1>(x);  // lane ^ 1
  x += dpp_f<0x4E>(x);  // lane ^ 2
  if constexpr (G >= 8) x += dpp_f<0x141>(x);  // row_half_mirror: the other quad of the 8
  if constexpr (G >= 16) x += dpp_f<0x140>(x);  // row_mirror: the other 8 of the 16
  if constexpr (G >= 32) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // rows 0<->1, 2<->3
    x = __builtin_bit_cast(float, (unsigned)p[0]) + __builtin_bit_cast(float, (unsigned)p[1]);
  }
  return x;
}

// Dot product of a lane's EPL elements with two partial sums (a shorter
// dependent chain than one running sum).
template <int EPL>
__device__ __forceinline__ float dot2(const float (&x)[EPL], const float (&y)[EPL]) {
  float s0 = x[0] * y[0], s1 = EPL > 1 ? x[1] * y[1] : 0.0f;
#pragma unroll
  for (int e = 2; e < EPL; e += 2) {
    s0 += x[e] * y[e];
    if (e + 1 < EPL) s1 += x[e + 1] * y[e + 1];
  }
  return s0 + s1;
}

// One token of one row from the normalised key and query slices: updates m in
// place and returns o_t[row] (every lane of the 16-lane row holds it).
//   m <- alpha m + (beta v - alpha beta (m . k^)) k^,   o = m . q^
template <int EPL>
__device__ __forceinline__ float delta_row(float (&m)[EPL], const float (&kh)[EPL], const float (&qh)[EPL],
                                           float alpha, float alpha_beta, float beta_v) {
  const float mk = row16_reduce(dot2<EPL>(m, kh), OpAdd());
  const float c = beta_v - alpha_beta * mk;
#pragma unroll
  for (int e = 0; e < EPL; ++e) m[e] = alpha * m[e] + c * kh[e];
  return row16_reduce(dot2<EPL>(m, qh), OpAdd());
}

// 1 / sqrt(|x|^2 + eps) of the row a 16-lane group holds (EPL elements per lane)
template <int EPL>
__device__ __forceinline__ float row_rnorm(const float (&x)[EPL]) {
  return __builtin_amdgcn_rsqf(row16_reduce(dot2<EPL>(x, x), OpAdd()) + kNormEps);
}

// Prefill: one 16-lane row per state row, the whole sequence in registers.
// The block's 16 rows belong to one head and share every token's k, q, a and
// beta, so the block stages tiles of kTile tokens in LDS, already prepared:
// k^ and q^ normalised in fp32, alpha = e^a and beta widened.  While the waves
// run the recurrence of one tile from LDS, the next tile's global loads are in
// flight in registers (issued at the start of the tile, prepared and written to
// the other LDS buffer at its end, one barrier per tile), so the serial chain
// of a row waits only on LDS and holds only the state-dependent work.  Outputs
// go to LDS and leave once per tile.
constexpr int kTile = 32;

template <class T, int EPL>
struct DeltaTile {
  static constexpr int DK = EPL * kLPR;
  static constexpr int kCE = 16 / (int)sizeof(T);                    // elements per 16-byte chunk
  static constexpr int kCPT = DK / kCE;                               // chunks per token row
  static constexpr int kChunks = kTile * kCPT;                        // chunks of k (or q) per tile
  static constexpr int kPer = (kChunks + kThreads - 1) / kThreads;   // per thread
  static constexpr int kVPer = kTile * kRowsPerBlock / kThreads;     // v (and o) elements per thread
  alignas(16) float kh[2][kTile][DK];
  alignas(16) float qh[2][kTile][DK];
  // per token and row: alpha, alpha beta, beta v_t[row] (one 16-byte read)
  alignas(16) f32x4 rec[2][kTile][kRowsPerBlock];
  float alpha[kTile], beta[kTile];  // of the tile being prepared
  T o[2][kTile][kRowsPerBlock];
};

template <class T, int EPL>
struct TileRegs {
  u32x4 k[DeltaTile<T, EPL>::kPer], q[DeltaTile<T, EPL>::kPer];
  T v[DeltaTile<T, EPL>::kVPer];
  T ab;  // a (threads 0 .. kTile-1) or beta (kTile .. 2 kTile-1)
};

template <class T, int EPL>
__device__ __forceinline__ void tile_load(const DeltaParams &p, size_t bh, int rb, int t0, TileRegs<T, EPL> &r) {
  using Tl = DeltaTile<T, EPL>;
  const int tid = threadIdx.x;
  // k and q rows of tokens t0 .. t0 + kTile - 1 are contiguous; past the end
  // the chunk index is clamped to the last token's chunks (never used)
  const size_t base = bh * (size_t)p.L * Tl::kCPT;
  const size_t last = (size_t)p.L * Tl::kCPT - 1;
#pragma unroll
  for (int c = 0; c < Tl::kPer; ++c) {
    const int ch = tid + c * kThreads;
    if (ch < Tl::kChunks) {
      const size_t g = base + min((size_t)t0 * Tl::kCPT + ch, last);
      r.k[c] = ((const u32x4 *)p.k)[g];
      r.q[c] = ((const u32x4 *)p.q)[g];
    }
  }
#pragma unroll
  for (int e = 0; e < Tl::kVPer; ++e) {
    const int idx = tid + e * kThreads, tt = idx / kRowsPerBlock, rr = rb * kRowsPerBlock + idx % kRowsPerBlock;
    const size_t tok = bh * (size_t)p.L + min(t0 + tt, p.L - 1);
    r.v[e] = ((const T *)p.v)[tok * p.dv + min(rr, p.dv - 1)];
  }
  if (tid < 2 * kTile) {
    const size_t tok = bh * (size_t)p.L + min(t0 + (tid % kTile), p.L - 1);
    r.ab = tid < kTile ? ((const T *)p.a)[tok] : ((const T *)p.beta)[tok];
  }
}

// Normalises the tile's keys and queries (the kCPT chunks of a token row sit in
// kCPT consecutive lanes, so |k|^2 is a group sum) and writes the prepared tile.
template <class T, int EPL>
__device__ __forceinline__ void tile_store(DeltaTile<T, EPL> &lds, int buf, const TileRegs<T, EPL> &r) {
  using Tl = DeltaTile<T, EPL>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int c = 0; c < Tl::kPer; ++c) {
    const int ch = tid + c * kThreads;
    if (Tl::kChunks % kThreads == 0 || ch < Tl::kChunks) {  // whole lane groups either way
      float kx[Tl::kCE], qx[Tl::kCE];
      const T *ke = (const T *)&r.k[c], *qe = (const T *)&r.q[c];
#pragma unroll
      for (int j = 0; j < Tl::kCE; ++j) {
        kx[j] = to_f32(ke[j]);
        qx[j] = to_f32(qe[j]);
      }
      const float rk = __builtin_amdgcn_rsqf(group_sum<Tl::kCPT>(dot2<Tl::kCE>(kx, kx)) + kNormEps);
      const float rq = __builtin_amdgcn_rsqf(group_sum<Tl::kCPT>(dot2<Tl::kCE>(qx, qx)) + kNormEps);
      float *kd = &lds.kh[buf][0][0] + ch * Tl::kCE, *qd = &lds.qh[buf][0][0] + ch * Tl::kCE;
#pragma unroll
      for (int j = 0; j < Tl::kCE; j += 4) {
        *(f32x4 *)(kd + j) = (f32x4){kx[j] * rk, kx[j + 1] * rk, kx[j + 2] * rk, kx[j + 3] * rk};
        *(f32x4 *)(qd + j) = (f32x4){qx[j] * rq, qx[j + 1] * rq, qx[j + 2] * rq, qx[j + 3] * rq};
      }
    }
  }
  if (tid < kTile)
    lds.alpha[tid] = exp2_fast(to_f32(r.ab) * kLog2e);  // a = -inf gives 0
  else if (tid < 2 * kTile)
    lds.beta[tid - kTile] = to_f32(r.ab);
  __syncthreads();  // alpha, beta of the tile visible to the record writers
#pragma unroll
  for (int e = 0; e < Tl::kVPer; ++e) {
    const int idx = tid + e * kThreads, tt = idx / kRowsPerBlock;
    const float al = lds.alpha[tt], be = lds.beta[tt];
    lds.rec[buf][tt][idx % kRowsPerBlock] = (f32x4){al, al * be, be * to_f32(r.v[e]), 0.0f};
  }
}

template <class T, int EPL>
__global__ __launch_bounds__(kThreads) void gdn_prefill_kernel(DeltaParams p) {
  using Tl = DeltaTile<T, EPL>;
  constexpr int DK = EPL * kLPR;
  __shared__ Tl lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, l16 = lane & 15;
  const int nrb = (p.dv + kRowsPerBlock - 1) / kRowsPerBlock;
  const size_t bh = blockIdx.x / nrb;
  const int rb = blockIdx.x % nrb;
  const int rloc = wave * 4 + (lane >> 4);  // row within the block
  const int row0 = rb * kRowsPerBlock + rloc;
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

  TileRegs<T, EPL> regs;
  tile_load<T, EPL>(p, bh, rb, 0, regs);
  tile_store<T, EPL>(lds, 0, regs);
  __syncthreads();
  const int ntiles = (p.L + kTile - 1) / kTile;
  for (int i = 0; i < ntiles; ++i) {
    const int buf = i & 1, t0 = i * kTile;
    const bool more = i + 1 < ntiles;
    if (more) tile_load<T, EPL>(p, bh, rb, t0 + kTile, regs);
    const int n = min(kTile, p.L - t0);
    // o_t of the row for token j is kept by lane j % 16 of the row (ob[j / 16]),
    // so the token loop has no branch and no LDS write: the next token's LDS
    // reads can be issued while this token's chain runs
    float ob0 = 0.0f, ob1 = 0.0f;
    auto token = [&](int j) {
      float kh[EPL], qh[EPL];
      if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPL; e += 4) {
          const f32x4 a = *(const f32x4 *)__builtin_assume_aligned(&lds.kh[buf][j][l16 * EPL + e], 16);
          const f32x4 b = *(const f32x4 *)__builtin_assume_aligned(&lds.qh[buf][j][l16 * EPL + e], 16);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            kh[e + u] = a[u];
            qh[e + u] = b[u];
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          kh[e] = lds.kh[buf][j][l16 * EPL + e];
          qh[e] = lds.qh[buf][j][l16 * EPL + e];
        }
      }
      const f32x4 rc = lds.rec[buf][j][rloc];
      const float ot = delta_row<EPL>(m, kh, qh, rc[0], rc[1], rc[2]);
      ob0 = (j == l16) ? ot : ob0;
      ob1 = (j == l16 + 16) ? ot : ob1;
    };
    if (n == kTile) {
#pragma unroll 4
      for (int j = 0; j < kTile; ++j) token(j);
    } else {
      for (int j = 0; j < n; ++j) token(j);
    }
    lds.o[buf][l16][rloc] = from_f32<T>(ob0);
    lds.o[buf][l16 + 16][rloc] = from_f32<T>(ob1);
    if (more) tile_store<T, EPL>(lds, buf ^ 1, regs);
    __syncthreads();
    // the tile's outputs: kRowsPerBlock consecutive values of each token row
    // (double-buffered: the next tile writes the other half while slower waves
    // may still read this one)
#pragma unroll
    for (int e = 0; e < Tl::kVPer; ++e) {
      const int idx = tid + e * kThreads, tt = idx / kRowsPerBlock, rr = rb * kRowsPerBlock + idx % kRowsPerBlock;
      if (tt < n && rr < p.dv)
        ((T *)p.o)[(bh * (size_t)p.L + t0 + tt) * p.dv + rr] = lds.o[buf][tt][idx % kRowsPerBlock];
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
  const int nrb = (p.dv + kDecRows - 1) / kDecRows;
  const size_t bh = blockIdx.x / nrb;
  // each 16-lane group holds rows g and g + 16 of the block's 32: twice the
  // state bytes in flight per lane, and the token's k, q, a and beta (with the
  // key and query norms) are loaded and formed once for both rows
  const int g = wave * 4 + (lane >> 4);
  int rows[2];
  bool live[2];
  float *sp[2];
  float m[2][EPL];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row0 = (blockIdx.x % nrb) * kDecRows + 16 * r + g;
    live[r] = row0 < p.dv;
    rows[r] = live[r] ? row0 : p.dv - 1;  // rows past d_v compute a copy, store nothing
    sp[r] = p.state_out + (bh * p.dv + rows[r]) * DK + l16 * EPL;
    if constexpr (EPL % 4 == 0) {
#pragma unroll
      for (int c = 0; c < EPL / 4; ++c) {
        const f32x4 w = __builtin_nontemporal_load((const f32x4 *)(sp[r] + 4 * c));
#pragma unroll
        for (int j = 0; j < 4; ++j) m[r][4 * c + j] = w[j];
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPL; ++e) m[r][e] = sp[r][e];
    }
  }
  TokenOps<T, EPL> x;
  {
    DeltaParams one = p;
    one.L = 1;
    load_token<T, EPL>(one, bh, rows[0], l16, 0, x);
  }
  const float v1 = to_f32(((const T *)p.v)[bh * p.dv + rows[1]]);
  float kh[EPL], qh[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    kh[e] = to_f32(x.k[e]);
    qh[e] = to_f32(x.q[e]);
  }
  const float rk = row_rnorm<EPL>(kh), rq = row_rnorm<EPL>(qh);
#pragma unroll
  for (int e = 0; e < EPL; ++e) {
    kh[e] *= rk;
    qh[e] *= rq;
  }
  const float alpha = exp2_fast(to_f32(x.a) * kLog2e), beta = to_f32(x.beta);
  float ot[2];
  ot[0] = delta_row<EPL>(m[0], kh, qh, alpha, alpha * beta, beta * to_f32(x.v));
  ot[1] = delta_row<EPL>(m[1], kh, qh, alpha, alpha * beta, beta * v1);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (live[r]) {
      if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int c = 0; c < EPL / 4; ++c)
          __builtin_nontemporal_store((f32x4){m[r][4 * c], m[r][4 * c + 1], m[r][4 * c + 2], m[r][4 * c + 3]},
                                      (f32x4 *)(sp[r] + 4 * c));
      } else {
#pragma unroll
        for (int e = 0; e < EPL; ++e) sp[r][e] = m[r][e];
      }
      if (l16 == 0) ((T *)p.o)[bh * p.dv + rows[r]] = from_f32<T>(ot[r]);
    }
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
  const int rows = decode ? kDecRows : kRowsPerBlock;
  const size_t nrb = (size_t)(a.dv + rows - 1) / rows;
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
  if (!decode && delta_chunk_supported(a)) return launch_delta_chunk(a);
  return a.bf16 ? dispatch<bf16>(a, decode) : dispatch<float>(a, decode);
}

}  // namespace glah

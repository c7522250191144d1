// delta_chunk.hip -- chunkwise gated delta rule prefill on the gfx950 matrix
// cores (bf16 inputs, fp32 state, d_k = 128, d_v a multiple of 16).
//
// The mixer is Gated DeltaNet ("systematic analysis of hybrid linear
// attention", 2507.06457, findings and recommendations; "LT2" technical
// summary, 2605.20670, hybrid designs): per (b, h), with M the d_v x d_k state,
//     M_t = alpha_t M_{t-1} (I - beta_t k^_t k^_t^T) + beta_t v_t k^_t^T,
//     o_t = M_t q^_t,   k^ = k / sqrt(|k|^2 + 1e-6), q^ likewise.
// Rewritten with the error-correcting write d_t = beta_t (v_t - alpha_t
// M_{t-1} k^_t), the state is M_t = alpha_t M_{t-1} + d_t k^_t^T, so over a
// chunk that starts from M0, with g_t the in-chunk cumulative log-decay and
// gamma_t = e^{g_t} (all ratios gamma_t / gamma_s <= 1 for s <= t):
//     M_t = gamma_t M0 + sum_{s<=t} (gamma_t/gamma_s) d_s k^_s^T
//     (I + L) D = Y,   L_ts = beta_t (gamma_t/gamma_s) k^_t . k^_s (s < t),
//                      Y_t  = beta_t (v_t - gamma_t M0 k^_t)
//     o_t = gamma_t M0 q^_t + sum_{s<=t} (gamma_t/gamma_s) (q^_t . k^_s) d_s
//     M_C = gamma_C M0 + sum_s (gamma_C/gamma_s) d_s k^_s^T.
// Everything but Y, D, o and M_C is independent of the state, so the work
// splits in two kernels:
//   gdn_prep_kernel   one block per (b, h, 64-token chunk), all chunks at
//                     once: the cumulative log-decays, the norms, L and P_ts =
//                     (gamma_t/gamma_s) q^_t . k^_s (s <= t) from the raw score
//                     products, and T = (I + L)^-1 -- each diagonal 16 x 16
//                     block X_i by forward substitution in fp32 (a lane per
//                     column), the blocks below it by block substitution down
//                     each block column, T_ij = -X_i sum_{j<=k<i} L_ik T_kj, on
//                     the matrix cores.  (A power series for X_i, such as
//                     Neumann doubling, is exact in exact arithmetic but not
//                     with bf16 operands: for a key repeated over a block with
//                     full write strength the powers of L_ii grow like binomial
//                     coefficients, into the thousands, and must cancel.)
//                     T and P go to the workspace as matrix-core operands, with
//                     the per-token scalars gamma/|k|, beta, gamma_C/(gamma |k|),
//                     gamma/|q| and gamma_C.
//   gdn_recur_kernel  one block per (b, h, 16-row d_v tile), the chunks in
//                     order: R = K M0^T, Y = beta (v - (gamma/|k|) R), D = T Y,
//                     o = (gamma/|q|) Q M0^T + P D and
//                     M^T <- gamma_C M^T + K^T diag(gamma_C/(gamma |k|)) D.
//                     Its four waves split d_k (32 columns of M each): the
//                     partial products of R and Q M0^T over each wave's slice
//                     meet in LDS, the wave of token block i forms Y_i, every
//                     wave forms all of D (T is small) and updates its own
//                     slice of the state.  Two barriers per chunk.
// The products with keys and queries take the raw bf16 k and q (exact
// operands) and apply the fp32 norms to the fp32 results, so nearly orthogonal
// q^ . k^ keep their relative accuracy; the fp32 state enters its products as
// a hi + lo pair of bf16 operands.
//
// Lane layouts (n = lane & 15, g = lane >> 4).  16x16x16 MFMA: operand A holds
// row n, K-slots 4g..4g+3; operand B column n, K-slots 4g..4g+3; the
// accumulator column n, rows 4g..4g+3, so a matrix kept in accumulator form is
// the B operand of itself and the A operand of its transpose.  16x16x32 MFMA:
// the same with K-slots 8g..8g+7.  Two 16x16x16 operands over token blocks 2p
// and 2p + 1 joined lane by lane are one 16x16x32 operand over the 32 tokens
// of pair p (K-slot 8g + j <-> token 32p + 16 (j / 4) + 4g + j % 4); every
// operand over tokens below uses that order.
#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;

constexpr int kCT = 64;         // tokens per chunk
constexpr int kDK = 128;        // key / query dim
constexpr int kThreads = 256;   // four waves, both kernels
constexpr int kOp16 = 512;      // bytes of one 16x16x16 operand (64 lanes x 4 bf16)
constexpr float kEps = 1e-6f;   // added to |x|^2 under the root
// floor of the per-token log-decay: alpha >= e^-30 keeps every in-chunk decay
// difference finite; a state term that passes through such a gate is already
// below 1e-13 of its size
constexpr float kLogDecayFloor = -30.0f;

// Workspace record of one (b, h, chunk), written by the prep kernel.
struct Rec {
  static constexpr int T = 0;              // T, 16x16x32 A operands (row block i, token pair p) [6]
  static constexpr int P = T + 6 * kFrag;  // P likewise [6]
  static constexpr int S = P + 6 * kFrag;  // fp32 per token [5][64]: gamma/|k|, beta,
                                           // gamma_C/(gamma |k|), gamma/|q|, gamma_C
  static constexpr int BYTES = S + 5 * 64 * 4;
};
static_assert(Rec::BYTES % 256 == 0, "record alignment");

// operand index of row block i, token pair p (p <= i / 2): the blocks above
// the diagonal pair are never stored
__device__ __forceinline__ int opidx(int i, int p) { return i < 2 ? i : 2 * i - 2 + p; }

__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ s16x4 pk(f32x4 x) {
  s16x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_bit_cast(short, (bf16)x[j]);
  return r;
}
__device__ __forceinline__ f32x4 unpk(s16x4 h) {
  f32x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = __builtin_bit_cast(float, (unsigned)(unsigned short)h[j] << 16);
  return r;
}
__device__ __forceinline__ f32x4 z4() { return (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ bf16x8 join(s16x4 lo, s16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ s16x4 half_of(bf16x8 x, int u) {
  const s16x8 s = __builtin_bit_cast(s16x8, x);
  return u == 0 ? __builtin_shufflevector(s, s, 0, 1, 2, 3) : __builtin_shufflevector(s, s, 4, 5, 6, 7);
}

__device__ __forceinline__ void st4(char *base, s16x4 x) { *(s16x4 *)(base + (threadIdx.x & 63) * 8) = x; }
__device__ __forceinline__ s16x4 ld4(const char *base) { return *(const s16x4 *)(base + (threadIdx.x & 63) * 8); }
__device__ __forceinline__ void stacc(char *base, f32x4 x) { *(f32x4 *)(base + (threadIdx.x & 63) * 16) = x; }
__device__ __forceinline__ f32x4 ldacc(const char *base) { return *(const f32x4 *)(base + (threadIdx.x & 63) * 16); }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)base, (short)0, (int)bytes, 0x00020000);
}
// one bf16 element, kept raw: the conversion happens where the value is used,
// so nothing waits for a prefetched load where it is issued
__device__ __forceinline__ unsigned bf_at(__amdgpu_buffer_rsrc_t r, unsigned byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, 0);
}
__device__ __forceinline__ float bf2f(unsigned raw) { return __builtin_bit_cast(float, (raw & 0xFFFFu) << 16); }

// Inclusive scan over the 64 lanes of a wave: DPP row_shr steps inside each
// 16-lane row, then the totals of the earlier rows.
__device__ __forceinline__ float wave_scan(float x) {
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  x += dpp_f<0x118>(x);
  const float t0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float t1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float t2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = (threadIdx.x & 63) >> 4;
  return x + (row >= 1 ? t0 : 0.0f) + (row >= 2 ? t1 : 0.0f) + (row >= 3 ? t2 : 0.0f);
}

// ================================ prep kernel ================================

struct PrepParams {
  const bf16 *q, *k, *a, *beta;
  char *ws;
  int L, nchunks;
};

struct LdsPrep {
  static constexpr int KF = 0;                   // k rows, 16x16x32 operands [4 blocks][4 d_k steps]
  static constexpr int QF = KF + 16 * kFrag;     // q rows likewise
  static constexpr int NL = QF + 16 * kFrag;     // -L_ij in A form [4][4] (j < i)
  static constexpr int XA = NL + 16 * kOp16;     // X_i = (I + L_ii)^-1 in A form [4]
  static constexpr int XB = XA + 4 * kOp16;      // X_i in B form [4]
  static constexpr int SC = XB + 4 * kOp16;      // g, beta, 1/|k|, 1/|q| [4][64] fp32
  static constexpr int NF = SC + 4 * 64 * 4;     // -L_ii, fp32 row-major [4][16][16]
  static constexpr int XF = NF + 4 * 256 * 4;    // X_i, fp32 row-major [4][16][16]
  static constexpr int BYTES = XF + 4 * 256 * 4;
};

// the score pairs (i, j <= i) of a chunk's 16-token blocks, spread over the
// four waves; each wave also owns the diagonal block of its own index
__device__ __forceinline__ int pair_count(int w) { return (w == 0 || w == 3) ? 3 : 2; }
__device__ __forceinline__ void pair_of(int w, int u, int &i, int &j) {
  // w0: (0,0) (1,0) (3,2)   w1: (1,1) (2,0)   w2: (2,2) (3,0)   w3: (3,3) (2,1) (3,1)
  constexpr int tab[4][3][2] = {{{0, 0}, {1, 0}, {3, 2}}, {{1, 1}, {2, 0}, {0, 0}},
                                {{2, 2}, {3, 0}, {0, 0}}, {{3, 3}, {2, 1}, {3, 1}}};
  i = tab[w][u][0];
  j = tab[w][u][1];
}

__global__ __launch_bounds__(kThreads) void gdn_prep_kernel(PrepParams p) {
  using LD = LdsPrep;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int blk = __builtin_amdgcn_readfirstlane(tid >> 6);  // token block of this wave
  const size_t bh = blockIdx.x / p.nchunks;
  const int c = blockIdx.x % p.nchunks;
  const unsigned Lu = (unsigned)p.L;
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k + bh * (size_t)p.L * kDK, Lu * kDK * 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q + bh * (size_t)p.L * kDK, Lu * kDK * 2);
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a + bh * (size_t)p.L, Lu * 2);
  const __amdgpu_buffer_rsrc_t rb = rsrc(p.beta + bh * (size_t)p.L, Lu * 2);
  char *const rec = p.ws + (bh * p.nchunks + c) * (size_t)Rec::BYTES;
  float *const sc = (float *)(smem + LD::SC);  // [g | beta | 1/|k| | 1/|q|][64]

  // ---- rows of token block blk (lane (n, g): d_k 32 m + 8 g + j of token
  // 16 blk + n; past the end: zeros), norms from the diagonals of K K^T and
  // Q Q^T, cumulative log-decays (lane = token; past the end: 0, no decay)
  {
    const unsigned row = (unsigned)(c * kCT + 16 * blk + n) * (kDK * 2);
    bf16x8 kf[4], qf[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      kf[m] = bload(rk, row + 64 * m + 16 * g);
      qf[m] = bload(rq, row + 64 * m + 16 * g);
    }
    const float la = bf2f(bf_at(ra, (unsigned)(c * kCT + lane) * 2));
    const float bl = bf2f(bf_at(rb, (unsigned)(c * kCT + lane) * 2));
    f32x4 kk = z4(), qq = z4();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      sts8(smem + LD::KF + (blk * 4 + m) * kFrag + lane * 16, kf[m]);
      sts8(smem + LD::QF + (blk * 4 + m) * kFrag + lane * 16, qf[m]);
      kk = mfma(kf[m], kf[m], kk);
      qq = mfma(qf[m], qf[m], qq);
    }
    // diagonal element (token n) sits in lane (n, g = n / 4), slot n % 4
    if (g == (n >> 2)) {
      sc[128 + 16 * blk + n] = __builtin_amdgcn_rsqf(kk[n & 3] + kEps);
      sc[192 + 16 * blk + n] = __builtin_amdgcn_rsqf(qq[n & 3] + kEps);
    }
    if (blk == 0) {
      sc[lane] = wave_scan(fmaxf(la, kLogDecayFloor));
      sc[64 + lane] = bl;
    }
  }
  __syncthreads();

  // ---- score pairs: L and P with decay ratios and norms
  const int np = pair_count(blk);
  for (int u = 0; u < 3; ++u) {
    if (u >= np) break;
    int i, j;
    pair_of(blk, u, i, j);
    f32x4 S = z4(), P = z4();
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const bf16x8 kj = lds8(smem + LD::KF + (j * 4 + m) * kFrag + lane * 16);
      const bf16x8 ki = lds8(smem + LD::KF + (i * 4 + m) * kFrag + lane * 16);
      const bf16x8 qi = lds8(smem + LD::QF + (i * 4 + m) * kFrag + lane * 16);
      S = mfma(kj, ki, S);
      P = mfma(kj, qi, P);
    }
    // lane (tau = 16 i + n, g), slot r: sigma = 16 j + 4 g + r
    const int tau = 16 * i + n;
    const float g_t = sc[tau], b_t = sc[64 + tau], nk_t = sc[128 + tau], nq_t = sc[192 + tau];
    const f32x4 g_s = *(const f32x4 *)(sc + 16 * j + 4 * g);
    const f32x4 nk_s = *(const f32x4 *)(sc + 128 + 16 * j + 4 * g);
    f32x4 NLv, PLv;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int sig = 4 * g + r;
      const float ratio = exp2_fast((g_t - g_s[r]) * kLog2e) * nk_s[r];
      const bool lower = j < i || sig < n, lower_eq = j < i || sig <= n;
      PLv[r] = lower_eq ? P[r] * ratio * nq_t : 0.0f;
      NLv[r] = lower ? -b_t * ratio * nk_t * S[r] : 0.0f;  // -L_tau,sigma
    }
    // P_ij (A form: PLv is P_ij^T in accumulator form) into half j & 1 of
    // operand (i, j / 2); the even diagonal blocks also clear the other half
    char *const pop = rec + Rec::P + opidx(i, j >> 1) * kFrag + lane * 16;
    *(s16x4 *)(pop + (j & 1) * 8) = pk(PLv);
    if (j < i) {
      st4(smem + LD::NL + (i * 4 + j) * kOp16, pk(NLv));
    } else {
      // N = -L_ii for the forward substitution: row tau, columns 4 g .. 4 g + 3
      *(f32x4 *)(smem + LD::NF + ((i * 16 + n) * 16 + 4 * g) * 4) = NLv;
      if ((i & 1) == 0) *(s16x4 *)(pop + 8) = (s16x4){0, 0, 0, 0};
    }
  }
  __syncthreads();

  // ---- X_blk = (I + L_blk,blk)^-1 = (I - N)^-1 by forward substitution in
  // fp32: lane (n, g) computes column n (the four lane groups alike), x_t =
  // [t == n] + sum_{s<t} N_ts x_s
  {
    const float *const nf = (const float *)(smem + LD::NF) + blk * 256;
    float x[16];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      float acc = t == n ? 1.0f : 0.0f;
#pragma unroll
      for (int s4 = 0; s4 < t; s4 += 4) {
        const f32x4 row = *(const f32x4 *)(nf + t * 16 + s4);
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          if (s4 + jj < t) acc += row[jj] * x[s4 + jj];
      }
      x[t] = acc;
    }
    float *const xf = (float *)(smem + LD::XF) + blk * 256;
    if (g == 0) {
#pragma unroll
      for (int t = 0; t < 16; ++t) xf[t * 16 + n] = x[t];
    }
    // the same wave reads them back (its LDS operations complete in order):
    // A form, lane (n, g) row n, columns 4 g + r; B form, column n, rows 4 g + r
    const s16x4 xa = pk(*(const f32x4 *)(xf + n * 16 + 4 * g));
    f32x4 xbv;
#pragma unroll
    for (int r = 0; r < 4; ++r) xbv[r] = xf[(4 * g + r) * 16 + n];
    st4(smem + LD::XA + blk * kOp16, xa);
    st4(smem + LD::XB + blk * kOp16, pk(xbv));
    char *const top = rec + Rec::T + opidx(blk, blk >> 1) * kFrag + lane * 16;
    *(s16x4 *)(top + (blk & 1) * 8) = xa;
    if ((blk & 1) == 0) *(s16x4 *)(top + 8) = (s16x4){0, 0, 0, 0};
  }
  __syncthreads();

  // ---- T below the diagonal, one block column per wave: Z = -sum_k L_ik T_kj
  // (A form of -L_ik, B form of T_kj), T_ij = X_i Z in both forms
  if (blk < 3) {
    const int j = blk;
    s16x4 TB[3];  // B forms of T_kj, k = j .. 2
#pragma unroll
    for (int k = 0; k < 3; ++k) TB[k] = (s16x4){0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < j) continue;
      if (i == j) {
        if (i < 3) TB[i] = ld4(smem + LD::XB + i * kOp16);
        continue;
      }
      f32x4 Z = z4();
#pragma unroll
      for (int k = 0; k < 3; ++k)
        if (k >= j && k < i) Z = mma16(ld4(smem + LD::NL + (i * 4 + k) * kOp16), TB[k], Z);
      const s16x4 xa = ld4(smem + LD::XA + i * kOp16), zb = pk(Z);
      if (i < 3) TB[i] = pk(mma16(xa, zb, z4()));  // T_ij (accumulator form = B form)
      *(s16x4 *)(rec + Rec::T + opidx(i, j >> 1) * kFrag + lane * 16 + (j & 1) * 8) =
          pk(mma16(zb, xa, z4()));  // T_ij^T in accumulator form = T_ij in A form
    }
  } else {
    // per-token scalars of the recurrence (lane = token)
    const float gt = sc[lane], gC = sc[63];
    const float et = exp2_fast(gt * kLog2e);
    float *const out = (float *)(rec + Rec::S);
    out[lane] = et * sc[128 + lane];
    out[64 + lane] = sc[64 + lane];
    out[128 + lane] = exp2_fast((gC - gt) * kLog2e) * sc[128 + lane];
    out[192 + lane] = et * sc[192 + lane];
    out[256 + lane] = exp2_fast(gC * kLog2e);
  }
}

// ============================= recurrence kernel =============================

struct RecParams {
  const bf16 *q, *k, *v;
  const char *ws;
  const float *state_in;
  float *state_out;
  bf16 *o;
  int L, nchunks, dv;
};

struct LdsRec {
  static constexpr int RP = 0;                // partial R = K M0^T [4 token blocks][4 waves], accumulators
  static constexpr int QP = RP + 16 * kFrag;  // partial Q M0^T likewise
  static constexpr int YF = QP + 16 * kFrag;  // Y_i in B form [4]
  static constexpr int TF = YF + 4 * kOp16;   // T operands [2 chunk parity][6]
  static constexpr int SF = TF + 2 * 6 * kFrag;  // per-token scalars of the record [2 chunk parity]
  static constexpr int SB = 5 * 64 * 4;          // bytes of the scalars
  static constexpr int BYTES = SF + 2 * SB;
};

// Operands of one chunk for one wave of the recurrence, loaded three chunks
// ahead: key and query rows of the wave's d_k slice (token 16 i + n, d_k
// 32 w + 8 g + j), v of token block w as a 16x16x16 A operand (token 16 w + n,
// d_v 16 rt + 4 g + r), the wave's share of T (operands w and w + 4), P of row
// block w, and the wave's share of the per-token scalars (16 bytes a lane,
// waves 0 and 1).  All stay as loaded until used: a conversion next to a load
// would make the wave wait for it there.  At most 14 loads a set, so three
// sets in flight stay within the 63 the wait counter tracks.
struct ChunkOps {
  bf16x8 kf[4], qf[4];
  s16x4 v;
  u32x4 t[2], p[2], s;
};

__global__ __launch_bounds__(kThreads) void gdn_recur_kernel(RecParams p) {
  using LD = LdsRec;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // d_k slice 32 w .. 32 w + 31
  const int nrt = p.dv / 16;
  // blocks are dealt to the 8 XCDs in turn: keep the d_v tiles of a head, which
  // read the same rows and records, on one XCD (its L2)
  unsigned x = blockIdx.x;
  if (gridDim.x % 8 == 0) x = (x % 8) * (gridDim.x / 8) + x / 8;
  const size_t bh = x / nrt;
  const int rt = x % nrt;
  const int col = 16 * rt + n;  // this lane's d_v row of M
  const unsigned Lu = (unsigned)p.L, dvu = (unsigned)p.dv;
  const __amdgpu_buffer_rsrc_t rk = rsrc(p.k + bh * (size_t)p.L * kDK, Lu * kDK * 2);
  const __amdgpu_buffer_rsrc_t rq = rsrc(p.q + bh * (size_t)p.L * kDK, Lu * kDK * 2);
  const __amdgpu_buffer_rsrc_t rv = rsrc(p.v + bh * (size_t)p.L * p.dv, Lu * dvu * 2);
  const __amdgpu_buffer_rsrc_t ro = rsrc(p.o + bh * (size_t)p.L * p.dv, Lu * dvu * 2);
  const char *const recs = p.ws + bh * (size_t)p.nchunks * Rec::BYTES;
  // identity as a 16x16x16 B operand: column n, K-slots 4g + r
  s16x4 eye;
#pragma unroll
  for (int r = 0; r < 4; ++r) eye[r] = __builtin_bit_cast(short, (bf16)(4 * g + r == n ? 1.0f : 0.0f));

  // fp32 state, two accumulator tiles of M^T: lane (n, g) of tile u holds
  // M[col][32 w + 8 g + 4 u + r], so the pair joined is the 16x16x32 B operand
  // with K-slot 8 g + j <-> d_k 32 w + 8 g + j, the order of the key rows below
  f32x4 M[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    M[u] = z4();
    if (p.state_in) M[u] = *(const f32x4 *)(p.state_in + (bh * p.dv + col) * (size_t)kDK + 32 * w + 8 * g + 4 * u);
  }

  // chunk c's operands, key rows, query rows and the rest apart (c past the last chunk
  // loads the last one again: every load is unconditional, so the wait counts
  // before each use stay exact)
  auto load_rows = [&](int c, ChunkOps &s) {
    c = min(c, p.nchunks - 1);
    const unsigned tok0 = (unsigned)(c * kCT);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned off = (tok0 + 16 * i + n) * (kDK * 2) + 64 * w + 16 * g;
      s.kf[i] = bload(rk, off);
    }
  };
  auto load_qrows = [&](int c, ChunkOps &s) {
    c = min(c, p.nchunks - 1);
    const unsigned tok0 = (unsigned)(c * kCT);
#pragma unroll
    for (int i = 0; i < 4; ++i) s.qf[i] = bload(rq, (tok0 + 16 * i + n) * (kDK * 2) + 64 * w + 16 * g);
  };
  auto load_rest = [&](int c, ChunkOps &s) {
    c = min(c, p.nchunks - 1);
    const unsigned tok0 = (unsigned)(c * kCT);
    s.v = __builtin_bit_cast(
        s16x4, __builtin_amdgcn_raw_buffer_load_b64(rv, (int)(((tok0 + 16 * w + n) * dvu + 16 * rt + 4 * g) * 2), 0, 0));
    // the loads a wave does not use read other bytes of the same record
    const char *const rc = recs + (size_t)c * Rec::BYTES;
    s.t[0] = *(const u32x4 *)(rc + Rec::T + w * kFrag + lane * 16);
    s.t[1] = *(const u32x4 *)(rc + Rec::T + (w + 4) * kFrag + lane * 16);  // used by waves 0, 1
    s.p[0] = *(const u32x4 *)(rc + Rec::P + opidx(w, 0) * kFrag + lane * 16);
    s.p[1] = *(const u32x4 *)(rc + Rec::P + opidx(w, 1) * kFrag + lane * 16);  // used by waves 2, 3
    s.s = *(const u32x4 *)(rc + Rec::S + min(w * kFrag + lane * 16, LD::SB - 16));
  };

  // one chunk; s holds its operands (loaded three chunks before) and, after
  // their last use, receives those of chunk c + 3
  auto step = [&](int c, ChunkOps &s) {
    const int par = c & 1;
    const ChunkOps &cur = s;
    // this wave's shares of T and the scalars into the buffers of this parity
    // (their readers, chunk c - 2, passed the first barrier of chunk c - 1)
    *(u32x4 *)(smem + LD::TF + (par * 6 + w) * kFrag + lane * 16) = cur.t[0];
    if (w < 2) *(u32x4 *)(smem + LD::TF + (par * 6 + w + 4) * kFrag + lane * 16) = cur.t[1];
    if (w * kFrag + lane * 16 < LD::SB) *(u32x4 *)(smem + LD::SF + par * LD::SB + w * kFrag + lane * 16) = cur.s;
    // [gamma/|k| | beta | gamma_C/(gamma |k|) | gamma/|q| | gamma_C][64], read after B1
    const float *const sf = (const float *)(smem + LD::SF + par * LD::SB);
    // ---- partial products over this wave's d_k slice with M0 = hi + lo
    const s16x4 h0 = pk(M[0]), h1 = pk(M[1]);
    const bf16x8 mh = join(h0, h1), ml = join(pk(M[0] - unpk(h0)), pk(M[1] - unpk(h1)));
#pragma unroll
    for (int i = 0; i < 4; ++i) stacc(smem + LD::RP + (i * 4 + w) * kFrag, mfma(cur.kf[i], ml, mfma(cur.kf[i], mh, z4())));
#pragma unroll
    for (int i = 0; i < 4; ++i) stacc(smem + LD::QP + (i * 4 + w) * kFrag, mfma(cur.qf[i], ml, mfma(cur.qf[i], mh, z4())));
    // K^T of the slice for the update (row 4 g' + r' <-> d_k 32 w + 8 g' + 4 u
    // + r', K-slots over tokens in pair order), transposed on the matrix core
    bf16x8 KT[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
        KT[u][pp] = join(pk(mma16(half_of(cur.kf[2 * pp], u), eye, z4())),
                         pk(mma16(half_of(cur.kf[2 * pp + 1], u), eye, z4())));
    load_rows(c + 3, s);  // the key rows are used up: the next ones
    __syncthreads();  // B1: partials, T and scalars in LDS
    load_qrows(c + 3, s);  // the query rows likewise, spread from the key rows
    // ---- Y of token block w from the partials, summed in slice order
    f32x4 Rs = ldacc(smem + LD::RP + (w * 4) * kFrag), Qs = ldacc(smem + LD::QP + (w * 4) * kFrag);
#pragma unroll
    for (int v2 = 1; v2 < 4; ++v2) {
      Rs += ldacc(smem + LD::RP + (w * 4 + v2) * kFrag);
      Qs += ldacc(smem + LD::QP + (w * 4 + v2) * kFrag);
    }
    const f32x4 vt = mma16(cur.v, eye, z4());  // v in accumulator form (exact)
    f32x4 Y;
    {
      const f32x4 ca = *(const f32x4 *)(sf + 16 * w + 4 * g), cb = *(const f32x4 *)(sf + 64 + 16 * w + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) Y[r] = cb[r] * (vt[r] - ca[r] * Rs[r]);
    }
    st4(smem + LD::YF + w * kOp16, pk(Y));
    __syncthreads();  // B2: Y in LDS
    // ---- D = T Y, every block (the pair operands of Y from the four waves)
    const bf16x8 Yb0 = join(ld4(smem + LD::YF + 0 * kOp16), ld4(smem + LD::YF + 1 * kOp16));
    const bf16x8 Yb1 = join(ld4(smem + LD::YF + 2 * kOp16), ld4(smem + LD::YF + 3 * kOp16));
    const char *const tf = smem + LD::TF + par * 6 * kFrag + lane * 16;
    f32x4 D[4];
    D[0] = mfma(lds8(tf + 0 * kFrag), Yb0, z4());
    D[1] = mfma(lds8(tf + 1 * kFrag), Yb0, z4());
    D[2] = mfma(lds8(tf + 3 * kFrag), Yb1, mfma(lds8(tf + 2 * kFrag), Yb0, z4()));
    D[3] = mfma(lds8(tf + 5 * kFrag), Yb1, mfma(lds8(tf + 4 * kFrag), Yb0, z4()));
    // ---- o of token block w: (gamma/|q|) Q M0^T + P D
    // D enters as hi + lo: over a run of similar keys D holds differences whose
    // sum telescopes, and separately rounded terms would not cancel
    f32x4 O = *(const f32x4 *)(sf + 192 + 16 * w + 4 * g) * Qs;
    {
      s16x4 dh[4], dl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        dh[i] = pk(D[i]);
        dl[i] = pk(D[i] - unpk(dh[i]));
      }
      const bf16x8 p0 = __builtin_bit_cast(bf16x8, cur.p[0]), p1 = __builtin_bit_cast(bf16x8, cur.p[1]);
      O = mfma(p0, join(dl[0], dl[1]), mfma(p0, join(dh[0], dh[1]), O));
      if (w >= 2) O = mfma(p1, join(dl[2], dl[3]), mfma(p1, join(dh[2], dh[3]), O));
    }
    {
      // transposed on the matrix core (exact: bf16 values times the identity)
      // so lane (n, g) holds d_v 16 rt + 4 g .. 4 g + 3 of token 16 w + n: one
      // 8-byte store a lane
      const s16x4 ot = pk(mma16(pk(O), eye, z4()));
      const unsigned tok = (unsigned)(c * kCT + 16 * w + n);
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ot), ro, (int)((tok * dvu + 16 * rt + 4 * g) * 2),
                                            0, 0);
    }
    // ---- state: M^T <- gamma_C M^T + K^T diag(gamma_C / (gamma |k|)) D
    f32x4 cc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cc[i] = *(const f32x4 *)(sf + 128 + 16 * i + 4 * g);
    const float gC = sf[256];
    const bf16x8 DS0 = join(pk(D[0] * cc[0]), pk(D[1] * cc[1]));
    const bf16x8 DS1 = join(pk(D[2] * cc[2]), pk(D[3] * cc[3]));
#pragma unroll
    for (int u = 0; u < 2; ++u) M[u] = mfma(KT[u][1], DS1, mfma(KT[u][0], DS0, M[u] * gC));
    load_rest(c + 3, s);
  };

  // three operand sets in turn (the loop unrolled by three keeps each in its
  // own registers, so no copy makes the wave wait for a load in flight; the
  // loop is left by breaks, so every path back to its head issued the same
  // loads)
  ChunkOps s0, s1, s2;
  load_rows(0, s0);
  load_qrows(0, s0);
  load_rest(0, s0);
  issue_fence();  // the sets in order, as in the loop
  load_rows(1, s1);
  load_qrows(1, s1);
  load_rest(1, s1);
  issue_fence();
  load_rows(2, s2);
  load_qrows(2, s2);
  load_rest(2, s2);
  for (int c = 0;; c += 3) {
    step(c, s0);
    if (c + 1 >= p.nchunks) break;
    step(c + 1, s1);
    if (c + 2 >= p.nchunks) break;
    step(c + 2, s2);
    if (c + 3 >= p.nchunks) break;
  }
  if (p.state_out) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
      *(f32x4 *)(p.state_out + (bh * p.dv + col) * (size_t)kDK + 32 * w + 8 * g + 4 * u) = M[u];
  }
}

}  // namespace

bool delta_chunk_supported(const LayerArgs &a) {
  if (!(a.bf16 && a.d == kDK && a.dv >= 16 && a.dv % 16 == 0 && a.L >= kCT)) return false;
  // byte offsets within a head's rows (one chunk past the end included) are
  // 32-bit, and so is the block index of the prep grid
  const size_t row = (size_t)(a.L + kCT) * (size_t)(a.dv > kDK ? a.dv : kDK) * 2;
  const size_t blocks = (size_t)a.B * a.H * (size_t)((a.L + kCT - 1) / kCT);
  return row <= 0xFFFFFFFFull && blocks <= 0x7FFFFFFFull;
}

size_t delta_chunk_ws_bytes(const LayerArgs &a) {
  if (!delta_chunk_supported(a)) return 0;
  return (size_t)a.B * a.H * (size_t)((a.L + kCT - 1) / kCT) * Rec::BYTES;
}

hipError_t launch_delta_chunk(const LayerArgs &a) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  if (!a.ws || a.ws_bytes < delta_chunk_ws_bytes(a)) return hipErrorInvalidValue;
  const int nchunks = (a.L + kCT - 1) / kCT;
  PrepParams pp;
  pp.q = (const bf16 *)a.q; pp.k = (const bf16 *)a.k; pp.a = (const bf16 *)a.gate; pp.beta = (const bf16 *)a.beta;
  pp.ws = (char *)a.ws; pp.L = a.L; pp.nchunks = nchunks;
  hipError_t e = hipFuncSetAttribute((const void *)gdn_prep_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     LdsPrep::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_prep_kernel, dim3((unsigned)((size_t)a.B * a.H * nchunks)), dim3(kThreads), LdsPrep::BYTES,
                     a.stream, pp);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  RecParams rp;
  rp.q = (const bf16 *)a.q; rp.k = (const bf16 *)a.k; rp.v = (const bf16 *)a.v; rp.ws = (const char *)a.ws;
  rp.state_in = a.state_in; rp.state_out = a.state_out; rp.o = (bf16 *)a.o;
  rp.L = a.L; rp.nchunks = nchunks; rp.dv = a.dv;
  e = hipFuncSetAttribute((const void *)gdn_recur_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LdsRec::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gdn_recur_kernel, dim3((unsigned)((size_t)a.B * a.H * (a.dv / 16))), dim3(kThreads),
                     LdsRec::BYTES, a.stream, rp);
  return hipGetLastError();
}

}  // namespace glah

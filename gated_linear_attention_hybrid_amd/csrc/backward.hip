// backward.hip -- gradient of the hybrid layer in its token-recurrent form.
//
// Gradients of L = <o, dO> + <S_final, dS_final> with respect to q, k, v, the
// gate input (every layout), both Hedgehog projections, the meta-memory
// scalars and the initial state: the parameters the two-stage training of
// Lizard fits ("Lizard" technical summary, gist.science 2507.09025,
// Methodology B; the layer itself is Methodology A.1 / A.2 / C).
//
// Gated part.  With b_t = sum_{r<=t} log Gamma_r (per feature), the output
// o_t = sum_{s<=t} (phiq_t e^{b_t}) . (phik_s e^{-b_s}) v_s + phiq_t e^{b_t} S_0,
// so with dS_t = phiq_t dO_t^T + diag(Gamma_{t+1}) dS_{t+1} (dS_{L-1} starting
// from dS_final):
//   dphiq_t = S_t dO_t,  dphik_t = dS_t v_t,  dv_t += dS_t^T phik_t,
//   d b_t   = phiq_t . dphiq_t - phik_t . dphik_t  (+ S_{L-1} . dS_final at t = L-1),
//   d log Gamma_t = sum_{s>=t} d b_s,  dS_0 = Gamma_0 dS_0^(t=0).
// Kernels: a prologue (phi and Gamma of every token), the forward state sweep
// (dphiq, per-tile sums of phiq . dphiq) and the reverse sweep (dphik, dv,
// per-tile sums of phik . dphik, d log Gamma_0) in one launch, a scan over
// 64-token tiles giving
// d log Gamma at each tile's first token, and a per-token kernel that finishes
// d log Gamma inside the tile, takes phi's softmax Jacobian back to dq and dk,
// accumulates the projection gradients and writes the gate gradient in its
// layout.
//
// Window part.  P_tj = e^{s_tj - lse_t}, with the sinks' e^{t_m} inside the
// normaliser; D_t = dO_t . o_swa,t; ds_tj = P_tj (dO_t . v_j - D_t); a query
// kernel gives dq, lse, D and the sink gradient -sum_t P_tm D_t; a key kernel
// gives dk_j = scale sum_t ds_tj q_t and dv_j = sum_t P_tj dO_t.  On the
// matrix-core path (bf16, one gate per feature, window <= 64) the window
// kernels run after the state walks, which write the gated part's dv to the
// output rows: the key kernel adds its dv there and writes dq and dk there, and
// the per-token kernel adds the gated part's dq and dk in place.  Otherwise
// they run on a side stream beside the prologue and the sweeps, into the
// workspace, and the per-token kernel, which adds their dq, dk and dv, waits
// for them.
//
// Every reduction is done in a fixed order into per-block partials (no atomics),
// so the gradients are bitwise repeatable.  All arithmetic is fp32.
#include <algorithm>
#include <mutex>
#include <type_traits>

#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kBT = 256;         // threads of every backward block
constexpr int kSliceCols = 32;   // d_v columns of one sweep block
constexpr int kPrepTok = 16;     // tokens of one prologue block
constexpr int kFeatTok = 64;     // tokens of one feature-gradient block
constexpr int kFeatPF = 2;       // tokens the feature-gradient block loads ahead
constexpr int kSwaTok = 16;      // query (key) tokens of one window block
constexpr int kMaxF2 = kBwdMaxF / 2;
constexpr int kMaxSlices = kBwdMaxD / kSliceCols;  // d_v slices of the sweeps
constexpr int kMaxRowWaves = kBwdMaxF / 32;       // row waves of the reverse sweep

template <class T> __device__ __forceinline__ f32x4 ld4(const T *p);
template <> __device__ __forceinline__ f32x4 ld4<float>(const float *p) { return *(const f32x4 *)p; }
template <> __device__ __forceinline__ f32x4 ld4<bf16>(const bf16 *p) {
  const bf16x4 x = *(const bf16x4 *)p;
  return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

__device__ __forceinline__ float dot4(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// Sum over the 8 lanes of an aligned group (the column groups of one row
// group): quad permutes l ^ 1, l ^ 2, then the half-row mirror 7 - l, which
// pairs each quad with the other quad of its group.  DPP only, no LDS trip.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  return x + dpp_f<0x141>(x);
}
// Sum over lanes l, l ^ 8, ..., l ^ 56 (the 8 row groups of one wave): a row
// rotate by 8 pairs the halves of each 16-lane row, then the row swaps.
__device__ __forceinline__ float sum_rows8(float x) {
  x += dpp_f<0x128>(x);
  return rows_reduce(x, OpAdd());
}

struct BwdParams {
  const void *q, *k, *v, *gate, *wq, *wk, *dout;
  const float *meta, *state_in, *dstate_out;
  void *gq, *gk, *gv, *gg;  // dq, dk, dv, dgate
  float *dwq, *dwk, *dmeta, *dstate_in;
  // workspace (fp32)
  float *pq, *pk, *gam;       // [N][f]
  float *dpq, *dpk;           // [nsl][N][f]
  float *dvg;                 // [nw][N][dv]
  float *xs;                  // [2][BH][nsl][f]: S_{L-1}.dS_final, d log Gamma_0
  float *tq, *tk;             // [nsl][BH][nft][f]: tile sums of phiq.dphiq, phik.dphik
  float *ta;                  // [BH][nft][f]: d log Gamma at each tile's first token
  float *lse, *del;           // [N]
  float *dqs, *dks;           // [N][d]
  float *dvs;                 // [N][dv]
  float *wqp, *wkp;           // [BH][nft][d][f2]
  float *gp;                  // [BH][nft]
  float *mp;                  // [BH][nmp][n_meta]
  int B, H, L, d, dv, f, f2, lf2, window, n_meta;
  int nsl, nw, nft, nsb, npt;
  float scale;
  int gate_is_log, gate_mode, gla, swa;
  // gam holds the in-tile cumsum of the floored log-gate over 16-token tiles
  // (the tile walks) instead of Gamma (the token sweeps)
  int gam_cum;
  int nwp;  // dW partials per head (wqp, wkp)
  int nmp;  // sink-gradient partials per head (mp)
  int win_bf16;  // dqs, dks, dvs hold bf16 (the matrix-core window kernels)
  // a call run as sub-problems: add this sub-problem's sums over batch rows to
  // the per-head outputs instead of writing them; gacc [H] holds the per-head
  // gate's gradient in fp32 across the rows
  int accum;
  float *gacc;
};

// ---------------------------------------------------------------------------
// Prologue: phi(q_t), phi(k_t) and Gamma_t of every token.  Block = (b, h,
// kPrepTok tokens); the two projections are staged in LDS as fp32.
template <class T>
__global__ __launch_bounds__(kBT) void bwd_prep_kernel(BwdParams p) {
  __shared__ float W[2][kBwdMaxD * kMaxF2];
  __shared__ float X[2][kPrepTok][kBwdMaxD];
  __shared__ float U[2][kPrepTok][kMaxF2];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / p.npt, tile = blockIdx.x % p.npt;
  const int h = bh % p.H, d = p.d, f = p.f, f2 = p.f2, L = p.L;
  const int t0 = tile * kPrepTok, nt = min(kPrepTok, L - t0);
  const size_t row0 = (size_t)bh * L + t0;
  const T *wq = (const T *)p.wq + (size_t)h * d * f2;
  const T *wk = (const T *)p.wk + (size_t)h * d * f2;
  for (int i = tid; i < d * f2; i += kBT) {
    W[0][i] = ld(wq + i);
    W[1][i] = ld(wk + i);
  }
  for (int i = tid; i < nt * d; i += kBT) {
    const int tt = i / d, e = i - tt * d;
    X[0][tt][e] = ld((const T *)p.q + (row0 + tt) * d + e);
    X[1][tt][e] = ld((const T *)p.k + (row0 + tt) * d + e);
  }
  __syncthreads();
  for (int o = tid; o < 2 * nt * f2; o += kBT) {
    const int m = o / (nt * f2), r = o - m * nt * f2;
    const int tt = r / f2, j = r - tt * f2;
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc += X[m][tt][e] * W[m][e * f2 + j];
    U[m][tt][j] = acc;
  }
  __syncthreads();
  const int wave = tid >> 6, lane = tid & 63;
  for (int row = wave; row < 2 * nt; row += kBT / 64) {
    const int m = row / nt, tt = row - m * nt;
    const bool ok = lane < f2;
    const float u = ok ? U[m][tt][lane] : 0.0f;
    const float mx = wave_max(ok ? u : -INFINITY), mn = wave_min(ok ? u : INFINITY);
    const float ep = ok ? exp_fast(u - mx) : 0.0f, en = ok ? exp_fast(mn - u) : 0.0f;
    const float zp = wave_sum(ep), zn = wave_sum(en);
    float *dst = (m ? p.pk : p.pq) + (row0 + tt) * f;
    if (ok) {
      dst[lane] = ep / zp;
      dst[f2 + lane] = en / zn;
    }
  }
  const T *g = (const T *)p.gate;
  for (int i = tid; i < nt * f; i += kBT) {
    const int tt = i / f, r = i - tt * f;
    p.gam[(row0 + tt) * f + r] =
        gate_from(ld(g + gate_index(p.gate_mode, bh, p.H, L, f, t0 + tt, r)), p.gate_is_log);
  }
}

// Raw quads of the I/O dtype, widened when used: a prefetched bf16 quad costs
// two registers.
template <class T> struct Quad;
template <> struct Quad<float> { typedef f32x4 type; };
template <> struct Quad<bf16> { typedef bf16x4 type; };
__device__ __forceinline__ f32x4 widen(f32x4 x) { return x; }
__device__ __forceinline__ f32x4 widen(bf16x4 x) { return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]}; }
template <class Q> __device__ __forceinline__ Q zero_quad() {
  Q z;
#pragma unroll
  for (int i = 0; i < 4; ++i) z[i] = 0.0f;
  return z;
}

// Prologue in 64-token tiles (d a multiple of 4 up to 128, f/2 a multiple of 4
// up to 64): the projections as a register-tiled product, thread (tg, fg) =
// (tid / 16, tid % 16) computing tokens 4tg .. 4tg+3 by features 4fg .. 4fg+3
// from the tile's inputs transposed in LDS (16-byte reads of four tokens and
// of four features per step), the two maps one after the other.  The
// projection is staged once per 64 tokens instead of once per 16; u reuses the
// input tile's LDS (65 KiB a block, two blocks per CU).
constexpr int kPrepTile = 64;

template <class T>
__global__ __launch_bounds__(kBT) void bwd_prep_tile_kernel(BwdParams p) {
  __shared__ __align__(16) float W[kBwdMaxD * kMaxF2];   // [d][f/2]
  __shared__ __align__(16) float XT[kBwdMaxD][kPrepTile];  // [d][token]; then u [token][f/2 + 1]
  float (*U)[kMaxF2 + 1] = (float (*)[kMaxF2 + 1])&XT[0][0];
  static_assert(kPrepTile * (kMaxF2 + 1) <= kBwdMaxD * kPrepTile, "u fits in the input tile");
  const int tid = threadIdx.x, tg = tid >> 4, fg = tid & 15;
  const int ntl = (p.L + kPrepTile - 1) / kPrepTile;
  const int bh = blockIdx.x / ntl, tile = blockIdx.x % ntl;
  const int h = bh % p.H, d = p.d, f = p.f, f2 = p.f2, L = p.L;
  const int t0 = tile * kPrepTile, nt = min(kPrepTile, L - t0);
  const size_t row0 = (size_t)bh * L + t0;
  const int wave = tid >> 6, lane = tid & 63;
  typedef typename Quad<T>::type Q;
  // quads (4 elements) each thread stages: of W (d x f/2) and of the input tile
  // (64 tokens x d); all of a thread's loads are issued before its LDS stores
  constexpr int kNQ = kBwdMaxD * kMaxF2 / 4 / kBT;
  constexpr int kXQ = kPrepTile * kBwdMaxD / 4 / kBT;
  static_assert(kNQ * 4 * kBT == kBwdMaxD * kMaxF2 && kXQ * 4 * kBT == kPrepTile * kBwdMaxD, "whole quads");
  const int d4 = d >> 2, nwq = d * f2 / 4, nxq = kPrepTile * d4;
  for (int m = 0; m < 2; ++m) {
    const T *w = (const T *)(m ? p.wk : p.wq) + (size_t)h * d * f2;
    const T *x = (const T *)(m ? p.k : p.q) + row0 * d;
    Q wv[kNQ], xv[kXQ];
#pragma unroll
    for (int k = 0; k < kNQ; ++k) wv[k] = *(const Q *)(w + 4 * min(tid + kBT * k, nwq - 1));
#pragma unroll
    for (int k = 0; k < kXQ; ++k) {
      const int q = min(tid + kBT * k, nxq - 1), tt = q / d4;
      xv[k] = *(const Q *)(x + (size_t)min(tt, nt - 1) * d + 4 * (q - tt * d4));
    }
#pragma unroll
    for (int k = 0; k < kNQ; ++k)
      if (tid + kBT * k < nwq) *(f32x4 *)&W[4 * (tid + kBT * k)] = widen(wv[k]);
#pragma unroll
    for (int k = 0; k < kXQ; ++k) {
      const int q = tid + kBT * k, tt = q / d4, e = 4 * (q - tt * d4);
      if (q < nxq) {
        const f32x4 v4 = widen(xv[k]);
#pragma unroll
        for (int j = 0; j < 4; ++j) XT[e + j][tt] = tt < nt ? v4[j] : 0.0f;
      }
    }
    __syncthreads();
    f32x4 acc[4] = {};
    if (4 * fg < f2) {
      for (int e = 0; e < d; ++e) {
        const f32x4 x4 = *(const f32x4 *)&XT[e][4 * tg];
        const f32x4 w4 = *(const f32x4 *)&W[e * f2 + 4 * fg];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] += x4[i] * w4;
      }
    }
    __syncthreads();  // every read of the input tile done: u takes its place
    if (4 * fg < f2) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) U[4 * tg + i][4 * fg + j] = acc[i][j];
    }
    __syncthreads();
    // phi = [softmax(u), softmax(-u)] of each token: one wave per token row
    for (int tt = wave; tt < nt; tt += kBT / 64) {
      const bool ok = lane < f2;
      const float u = ok ? U[tt][lane] : 0.0f;
      const float mx = wave_max(ok ? u : -INFINITY), mn = wave_min(ok ? u : INFINITY);
      const float ep = ok ? exp_fast(u - mx) : 0.0f, en = ok ? exp_fast(mn - u) : 0.0f;
      const float zp = wave_sum(ep), zn = wave_sum(en);
      float *dst = (m ? p.pk : p.pq) + (row0 + tt) * f;
      if (ok) {
        dst[lane] = ep / zp;
        dst[f2 + lane] = en / zn;
      }
    }
    __syncthreads();  // W, XT and U are reused by the next map
  }
  const T *g = (const T *)p.gate;
  if (p.gam_cum) {
    // b_t = sum of max(log Gamma, -10) over the 16-token tile up to t: thread
    // (feature, tile), the tile's 16 gates loaded before the sum
    for (int i = tid; i < f * (kPrepTile / 16); i += kBT) {
      const int r = i % f, j = i / f, tt0 = 16 * j;
      if (tt0 >= nt) continue;
      float a[16];
#pragma unroll
      for (int u = 0; u < 16; ++u)
        a[u] = ld(g + gate_index(p.gate_mode, bh, p.H, L, f, t0 + min(tt0 + u, nt - 1), r));
      float acc = 0.0f;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        acc += fmaxf(log_gate_from(a[u], p.gate_is_log), -10.0f);
        if (tt0 + u < nt) p.gam[(row0 + tt0 + u) * f + r] = acc;
      }
    }
  } else if (p.gate_mode == 0) {
    // per-feature gates: quads of the tile's [nt][f] rows, loads first
    constexpr int kGQ = kPrepTile * kBwdMaxF / 4 / kBT;
    const int f4 = f >> 2, ngq = nt * f4;
    const T *gb = g + row0 * f;
    Q gv[kGQ];
#pragma unroll
    for (int k = 0; k < kGQ; ++k) gv[k] = *(const Q *)(gb + 4 * (size_t)min(tid + kBT * k, ngq - 1));
#pragma unroll
    for (int k = 0; k < kGQ; ++k) {
      const int q = tid + kBT * k;
      if (q < ngq) {
        const f32x4 v4 = widen(gv[k]);
        f32x4 r4;
#pragma unroll
        for (int j = 0; j < 4; ++j) r4[j] = gate_from(v4[j], p.gate_is_log);
        *(f32x4 *)(p.gam + row0 * f + 4 * (size_t)q) = r4;
      }
    }
  } else {
    for (int i = tid; i < nt * f; i += kBT) {
      const int tt = i / f, r = i - tt * f;
      p.gam[(row0 + tt) * f + r] =
          gate_from(ld(g + gate_index(p.gate_mode, bh, p.H, L, f, t0 + tt, r)), p.gate_is_log);
    }
  }
}

// ---------------------------------------------------------------------------
// State sweeps.  Block = (b, h, 32-column slice of d_v); lane l of wave w owns
// rows 4 (8 w + l / 8) .. +3 and columns 4 (l % 8) .. +3 of the slice, so a
// row sum over the slice is a sum over 8 adjacent lanes and a column sum over
// the wave's 32 rows is a sum over lanes l ^ 8, l ^ 16, l ^ 32.  No barriers:
// every wave is independent; waves whose rows lie beyond f leave at once.
struct SweepLane {
  int r0, c0;
  bool rok, cok;
};

__device__ __forceinline__ SweepLane sweep_lane(const BwdParams &p, int slice) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  SweepLane s;
  s.r0 = 4 * (8 * w + (l >> 3));
  s.c0 = slice * kSliceCols + 4 * (l & 7);
  s.rok = s.r0 < p.f;
  s.cok = s.c0 < p.dv;
  return s;
}

constexpr int kPF = 8;  // tokens a sweep loads ahead of the one it computes

// Forward sweep: S_t = diag(Gamma_t) S_{t-1} + phik_t v_t^T, then the slice's
// part of dphiq_t = S_t dO_t, and per 64-token tile the slice's part of
// sum_t phiq_t . dphiq_t; at the end the slice's part of S_{L-1} . dS_final.
// Each step's operands are loaded kPF tokens ahead (the step is a chain of
// dependent arithmetic on the state; its loads must not wait on it).
template <class T>
__device__ __forceinline__ void fwd_sweep(const BwdParams &p, int blk) {
  typedef typename Quad<T>::type Q;
  const int bh = blk / p.nsl, slice = blk % p.nsl;
  if (32 * (int)(threadIdx.x >> 6) >= p.f) return;
  const SweepLane s = sweep_lane(p, slice);
  const int L = p.L, f = p.f, dv = p.dv;
  const size_t BH = (size_t)p.B * p.H, N = BH * L;
  const size_t rowf = (size_t)bh * L * f + s.r0;
  float *dpq = p.dpq + (size_t)slice * N * f + rowf;
  float *tq = p.tq + ((size_t)slice * BH + bh) * p.nft * f + s.r0;
  const bool lead = (threadIdx.x & 7) == 0;
  const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};

  f32x4 S[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    S[i] = z4;
    if (p.state_in && s.rok && s.cok) S[i] = *(const f32x4 *)(p.state_in + ((size_t)bh * f + s.r0 + i) * dv + s.c0);
  }
  f32x4 bg[kPF], bk[kPF], bq[kPF];
  Q bv[kPF], bo[kPF];
  // Loads are unconditional, from clamped rows, columns and tokens (lanes past f
  // or d_v are masked where the values are used): a predicated load made the
  // compiler wait for every load in flight before each token.
  const size_t rowf_ld = (size_t)bh * L * f + min(s.r0, f - 4);
  const size_t rowv_ld = (size_t)bh * L * dv + min(s.c0, dv - 4);
  auto fetch = [&](int u, int t) {
    const size_t tc = (size_t)min(t, L - 1);
    bg[u] = *(const f32x4 *)(p.gam + rowf_ld + tc * f);
    bk[u] = *(const f32x4 *)(p.pk + rowf_ld + tc * f);
    bq[u] = *(const f32x4 *)(p.pq + rowf_ld + tc * f);
    bv[u] = *(const Q *)((const T *)p.v + rowv_ld + tc * dv);
    bo[u] = *(const Q *)((const T *)p.dout + rowv_ld + tc * dv);
  };
  // L = 0 (the sweeps still pass the state gradient through): no token to load
  if (L > 0) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) fetch(u, u);
  }
  f32x4 tile = z4;
  auto step = [&](int u, int t) {
    const f32x4 g4 = s.rok ? bg[u] : z4, k4 = s.rok ? bk[u] : z4, q4 = s.rok ? bq[u] : z4;
    const f32x4 v4 = s.cok ? widen(bv[u]) : z4, o4 = s.cok ? widen(bo[u]) : z4;
    fetch(u, t + kPF);
    f32x4 part;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) S[i][j] = g4[i] * S[i][j] + k4[i] * v4[j];
      part[i] = sum8(dot4(S[i], o4));
      tile[i] += q4[i] * part[i];
    }
    if (lead && s.rok) *(f32x4 *)(dpq + (size_t)t * f) = part;
    if ((t & (kFeatTok - 1)) == kFeatTok - 1 || t == L - 1) {
      if (lead && s.rok) *(f32x4 *)(tq + (size_t)(t / kFeatTok) * f) = tile;
      tile = z4;
    }
  };
  // whole groups without a per-token branch, then the last L % kPF tokens
  int t0 = 0;
  for (; t0 + kPF <= L; t0 += kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      step(u, t0 + u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < kPF - 1; ++u)
    if (t0 + u < L) step(u, t0 + u);
  if (p.dstate_out) {
    f32x4 part;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 d4 = (s.rok && s.cok) ? *(const f32x4 *)(p.dstate_out + ((size_t)bh * f + s.r0 + i) * dv + s.c0) : z4;
      part[i] = sum8(dot4(S[i], d4));
    }
    if (lead && s.rok) *(f32x4 *)(p.xs + ((size_t)bh * p.nsl + slice) * f + s.r0) = part;
  }
}

// Reverse sweep: dS_t = phiq_t dO_t^T + diag(Gamma_{t+1}) dS_{t+1} from dS_final;
// the slice's part of dphik_t = dS_t v_t (and per tile of sum_t phik_t .
// dphik_t), the wave's part of dS_t^T phik_t, dS_0-gradient = diag(Gamma_0)
// dS_0, and the slice's part of d log Gamma_0 = Gamma_0 (S_in . dS_0).
template <class T>
__device__ __forceinline__ void rev_sweep(const BwdParams &p, int blk) {
  typedef typename Quad<T>::type Q;
  const int bh = blk / p.nsl, slice = blk % p.nsl;
  const int wave = threadIdx.x >> 6;
  if (32 * wave >= p.f) return;
  const SweepLane s = sweep_lane(p, slice);
  const int L = p.L, f = p.f, dv = p.dv;
  const size_t BH = (size_t)p.B * p.H, N = BH * L;
  const size_t rowf = (size_t)bh * L * f + s.r0;
  const size_t rowv = (size_t)bh * L * dv + s.c0;
  float *dpk = p.dpk + (size_t)slice * N * f + rowf;
  float *dvg = p.dvg + (size_t)wave * N * dv + rowv;
  float *tk = p.tk + ((size_t)slice * BH + bh) * p.nft * f + s.r0;
  const int l = threadIdx.x & 63;
  const bool lead = (l & 7) == 0;

  const f32x4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  f32x4 dS[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    dS[i] = z4;
    if (p.dstate_out && s.rok && s.cok)
      dS[i] = *(const f32x4 *)(p.dstate_out + ((size_t)bh * f + s.r0 + i) * dv + s.c0);
  }
  f32x4 bq[kPF], bk[kPF], bg[kPF];
  Q bv[kPF], bo[kPF];
  // unconditional loads from clamped rows, columns and tokens, masked where used
  // (as in the forward sweep)
  const size_t rowf_ld = (size_t)bh * L * f + min(s.r0, f - 4);
  const size_t rowv_ld = (size_t)bh * L * dv + min(s.c0, dv - 4);
  auto fetch = [&](int u, int t) {
    const size_t tc = (size_t)max(t, 0);
    bq[u] = *(const f32x4 *)(p.pq + rowf_ld + tc * f);
    bk[u] = *(const f32x4 *)(p.pk + rowf_ld + tc * f);
    bg[u] = *(const f32x4 *)(p.gam + rowf_ld + tc * f);
    bv[u] = *(const Q *)((const T *)p.v + rowv_ld + tc * dv);
    bo[u] = *(const Q *)((const T *)p.dout + rowv_ld + tc * dv);
  };
  // L = 0 (the sweeps still pass the state gradient through): no token to load
  if (L > 0) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) fetch(u, L - 1 - u);
  }
  f32x4 gn = {1.0f, 1.0f, 1.0f, 1.0f};
  f32x4 tile = z4;
  auto step = [&](int u, int t) {
    const f32x4 q4 = s.rok ? bq[u] : z4, k4 = s.rok ? bk[u] : z4, g4 = s.rok ? bg[u] : z4;
    const f32x4 v4 = s.cok ? widen(bv[u]) : z4, o4 = s.cok ? widen(bo[u]) : z4;
    fetch(u, t - kPF);
    f32x4 a, c = z4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int j = 0; j < 4; ++j) dS[i][j] = gn[i] * dS[i][j] + q4[i] * o4[j];
      a[i] = sum8(dot4(dS[i], v4));
      tile[i] += k4[i] * a[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] += dS[i][j] * k4[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) c[j] = sum_rows8(c[j]);
    if (lead && s.rok) *(f32x4 *)(dpk + (size_t)t * f) = a;
    if (l < 8 && s.cok) *(f32x4 *)(dvg + (size_t)t * dv) = c;
    if ((t & (kFeatTok - 1)) == 0) {
      if (lead && s.rok) *(f32x4 *)(tk + (size_t)(t / kFeatTok) * f) = tile;
      tile = z4;
    }
    gn = g4;
  };
  // whole groups without a per-token branch, then the first L % kPF tokens
  int t0 = L - 1;
  for (; t0 - kPF + 1 >= 0; t0 -= kPF) {
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      step(u, t0 - u);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int u = 0; u < kPF - 1; ++u)
    if (t0 - u >= 0) step(u, t0 - u);
  if (p.dstate_in && s.rok && s.cok) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 r;
#pragma unroll
      for (int j = 0; j < 4; ++j) r[j] = gn[i] * dS[i][j];
      *(f32x4 *)(p.dstate_in + ((size_t)bh * f + s.r0 + i) * dv + s.c0) = r;
    }
  }
  // taken directly: without an initial state it is exactly zero, which a sum
  // of the d b_t reaches only up to rounding
  f32x4 x0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x4 s4 = (p.state_in && s.rok && s.cok)
                         ? *(const f32x4 *)(p.state_in + ((size_t)bh * f + s.r0 + i) * dv + s.c0) : z4;
    x0[i] = gn[i] * sum8(dot4(s4, dS[i]));
  }
  if (lead && s.rok) *(f32x4 *)(p.xs + ((BH + bh) * p.nsl + slice) * f + s.r0) = x0;
}

// Both sweeps in one launch: they share only inputs, and each has B H nsl
// blocks of one wave per SIMD (128 at 32 heads of 128 columns), so apart they
// leave half of the compute units idle.  The longer reverse sweep takes the
// first blocks.
template <class T>
__global__ __launch_bounds__(kBT) void bwd_sweeps_kernel(BwdParams p) {
  const int n = p.B * p.H * p.nsl;
  if ((int)blockIdx.x < n)
    rev_sweep<T>(p, (int)blockIdx.x);
  else
    fwd_sweep<T>(p, (int)blockIdx.x - n);
}

// d log Gamma at the first token of every 64-token tile.  With d b_t =
// phiq_t . dphiq_t - phik_t . dphik_t and tile totals T_i (from the sweeps),
// d log Gamma_t = sum_{s>=t} d b_s is known exactly at both ends (d log Gamma_0
// from the reverse sweep, the sum past the end = S_{L-1} . dS_final), so the
// first half of the tiles is summed forward from the start and the second half
// backward from the end: the exact zero of Gamma_0 without an initial state
// stays exact, and no running sum spans more than half the sequence.  A block
// per (b, h, 16 features), each half of the tiles cut into runs, one a thread.
constexpr int kTsFeat = 16;             // features of a tile-scan block
constexpr int kTsParts = kBT / kTsFeat;  // threads (runs of tiles) per feature

__global__ __launch_bounds__(kBT) void bwd_tile_scan_kernel(BwdParams p) {
  // block = (bh, kTsFeat features); the kTsParts threads of a feature take
  // consecutive runs of tiles of each half: sums of their runs, the runs before
  // (after) them combined through LDS, then the run scanned again from there
  const int f = p.f, nft = p.nft, nsl = p.nsl;
  const size_t BH = (size_t)p.B * p.H;
  const int ngr = (f + kTsFeat - 1) / kTsFeat;
  const size_t bh = blockIdx.x / ngr;
  const int rl = threadIdx.x % kTsFeat, part = threadIdx.x / kTsFeat;
  const int r = (int)(blockIdx.x % ngr) * kTsFeat + rl;
  const bool rok = r < f;
  const int rc = rok ? r : f - 1;  // clamped: loads stay in range, results unused
  const int half = (nft + 1) / 2;
  const int cf = (half + kTsParts - 1) / kTsParts, cb = (nft - half + kTsParts - 1) / kTsParts;
  const int f0 = min(part * cf, half), f1 = min(f0 + cf, half);
  const int b0 = min(half + part * cb, nft), b1 = min(b0 + cb, nft);
  // tile totals kTS at a time, every load of a group issued before they are used
  constexpr int kTS = 8;
  auto totals = [&](int i0, int dir, int lo, int hi, float (&tot)[kTS]) {
    float a[kTS][kMaxSlices], b[kTS][kMaxSlices];
#pragma unroll
    for (int u = 0; u < kTS; ++u)
#pragma unroll
      for (int sl = 0; sl < kMaxSlices; ++sl) {
        const int i = min(max(i0 + dir * u, 0), nft - 1);
        const size_t o = (((size_t)min(sl, nsl - 1) * BH + bh) * nft + i) * f + rc;
        a[u][sl] = p.tq[o];
        b[u][sl] = p.tk[o];
      }
#pragma unroll
    for (int u = 0; u < kTS; ++u) {
      const int i = i0 + dir * u;
      float s = 0.0f;
#pragma unroll
      for (int sl = 0; sl < kMaxSlices; ++sl)
        if (sl < nsl) s += a[u][sl] - b[u][sl];
      tot[u] = (i >= lo && i < hi) ? s : 0.0f;
    }
  };
  float sf = 0.0f, sb = 0.0f;
  for (int i0 = f0; i0 < f1; i0 += kTS) {
    float tot[kTS];
    totals(i0, 1, f0, f1, tot);
#pragma unroll
    for (int u = 0; u < kTS; ++u) sf += tot[u];
  }
  for (int i0 = b1 - 1; i0 >= b0; i0 -= kTS) {
    float tot[kTS];
    totals(i0, -1, b0, b1, tot);
#pragma unroll
    for (int u = 0; u < kTS; ++u) sb += tot[u];
  }
  __shared__ float runf[kTsParts][kTsFeat], runb[kTsParts][kTsFeat];
  runf[part][rl] = sf;
  runb[part][rl] = sb;
  __syncthreads();
  // forward half: ta = d log Gamma_0 term minus the totals of the tiles before;
  // backward half: the dS_final term plus the totals from the tile on
  float accf = 0.0f, accb = 0.0f;
  for (int sl = 0; sl < nsl; ++sl) accf += p.xs[((BH + bh) * nsl + sl) * f + rc];
  if (p.dstate_out)
    for (int sl = 0; sl < nsl; ++sl) accb += p.xs[(bh * nsl + sl) * f + rc];
  for (int q = 0; q < part; ++q) accf -= runf[q][rl];
  for (int q = kTsParts - 1; q > part; --q) accb += runb[q][rl];
  if (!rok) return;
  for (int i0 = f0; i0 < f1; i0 += kTS) {
    float tot[kTS];
    totals(i0, 1, f0, f1, tot);
#pragma unroll
    for (int u = 0; u < kTS; ++u)
      if (i0 + u < f1) {
        p.ta[(bh * nft + i0 + u) * f + r] = accf;
        accf -= tot[u];
      }
  }
  for (int i0 = b1 - 1; i0 >= b0; i0 -= kTS) {
    float tot[kTS];
    totals(i0, -1, b0, b1, tot);
#pragma unroll
    for (int u = 0; u < kTS; ++u)
      if (i0 - u >= b0) {
        accb += tot[u];
        p.ta[(bh * nft + i0 - u) * f + r] = accb;
      }
  }
}

// ---------------------------------------------------------------------------
// Per-token gradients.  Block = (b, h, kFeatTok tokens).  For each token: the
// slice sums of dphiq and dphik, the softmax Jacobian of both halves of phi,
// dq and dk (plus the window part), dv (both parts), d log Gamma_t (the tile's
// start value minus the d b of the tile's earlier tokens) turned into the gate
// gradient of its layout, and this block's share of dWphi_q = sum_t q_t^T
// du_q,t and of dWphi_k.  The projections sit in LDS as padded [d][f/2] rows,
// so a lane of dq = du Wphi^T reads its row 16 bytes at a time.
template <class T, bool GLA, bool SWA>
__global__ __launch_bounds__(kBT) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_feature_kernel(BwdParams p) {
  // W_phi rows [d][f/2], padded to kWR floats (16-byte reads of consecutive
  // rows by consecutive lanes fall on different banks)
  constexpr int kWR = kMaxF2 + 4;
  __shared__ __align__(16) float WT[2][kBwdMaxD * kWR];
  __shared__ __align__(16) float X[2][kBwdMaxD];
  __shared__ __align__(16) float DU[2][kMaxF2];
  __shared__ float E[2][kBwdMaxF];
  constexpr int NP = kBwdMaxD * kMaxF2 / kBT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int bh = blockIdx.x / p.nft, tile = blockIdx.x % p.nft;
  const int h = bh % p.H, d = p.d, dv = p.dv, f = p.f, f2 = p.f2, L = p.L;
  const int t0 = tile * kFeatTok, nt = min(kFeatTok, L - t0);
  const size_t N = (size_t)p.B * p.H * L, NF = N * f;
  constexpr bool gla = GLA;
  if (gla) {
    const T *wq = (const T *)p.wq + (size_t)h * d * f2;
    const T *wk = (const T *)p.wk + (size_t)h * d * f2;
    for (int i = tid; i < d * f2; i += kBT) {
      const int e = i >> p.lf2, j = i & (f2 - 1);
      WT[0][e * kWR + j] = ld(wq + i);
      WT[1][e * kWR + j] = ld(wk + i);
    }
  }
  const int jj = tid & (f2 - 1);
  // thread (i0, jj) accumulates dW rows i0 NP .. i0 NP + NP - 1 of feature jj:
  // contiguous rows, so the X reads are 16-byte (broadcast) reads
  const int i0 = tid >> p.lf2, ib = min(i0 * NP, kBwdMaxD - NP);
  float aq[NP], ak[NP];
#pragma unroll
  for (int n = 0; n < NP; ++n) aq[n] = ak[n] = 0.0f;
  // wave 2 carries d log Gamma of features lane and lane + 64 through the tile
  float run[2] = {0.0f, 0.0f};
  if (gla && wave == 2)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int r = lane + 64 * u;
      if (r < f) run[u] = p.ta[((size_t)bh * p.nft + tile) * f + r];
    }
  float gsum = 0.0f;
  const T *g = (const T *)p.gate;
  T *dg = (T *)p.gg;

  // every global operand of one token (loaded kFeatPF tokens ahead)
  struct Pre {
    float x, pp, pn, dp[kMaxSlices], dn[kMaxSlices], gr[2], ds, dvw[kMaxRowWaves], dvs;
  };
  const int m = wave >> 1, mi = tid & 127;  // m = tid >> 7
  // Every lane loads every operand from clamped indices (tokens past the tile,
  // features past f/2, slices past nsl, row waves past nw, columns past d or
  // d_v read valid memory and are masked where used): loads under a lane or
  // wave condition made the compiler wait for every load in flight, the next
  // token's included, before each token.
  const int mic = min(mi, d - 1), lanec = min(lane, f2 - 1), tidv = min(tid, dv - 1);
  // Wave-uniform base pointers at the tile's first token (m and wave & 1 are
  // wave-uniform), formed once; a token adds a 32-bit offset of a fixed stride,
  // so the token loop carries no 64-bit index arithmetic.
  const size_t row0 = (size_t)bh * L + t0;
  const T *bx = (const T *)(m ? p.k : p.q) + row0 * d;
  const float *bph = ((wave & 1) ? p.pk : p.pq) + row0 * f;
  const float *bdp[kMaxSlices];
#pragma unroll
  for (int sl = 0; sl < kMaxSlices; ++sl)
    bdp[sl] = ((wave & 1) ? p.dpk : p.dpq) + (size_t)min(sl, p.nsl - 1) * NF + row0 * f;
  const float *bdvw[kMaxRowWaves];
#pragma unroll
  for (int w = 0; w < kMaxRowWaves; ++w) bdvw[w] = p.dvg + ((size_t)min(w, p.nw - 1) * N + row0) * dv;
  const float *bds = (m ? p.dks : p.dqs) + row0 * d;
  const float *bdvs = p.dvs + row0 * dv;
  // the same rows when the window part left bf16
  const bf16 *bds0 = (const bf16 *)(m ? p.dks : p.dqs) + row0 * d;
  const bf16 *bdvs0 = (const bf16 *)p.dvs + row0 * dv;
  // gates: per feature (stride f), per token (stride 1) or one per head
  const T *bg = g + gate_index(p.gate_mode, bh, p.H, L, f, t0, 0);
  const unsigned gstep = p.gate_mode == 0 ? (unsigned)f : p.gate_mode == 1 ? 1u : 0u;
  const unsigned glane0 = p.gate_mode == 0 ? (unsigned)min(lane, f - 1) : 0u;
  const unsigned glane1 = p.gate_mode == 0 ? (unsigned)min(lane + 64, f - 1) : 0u;
  // outputs of the tile's first token: dq or dk (per wave), dv, the gate gradient
  T *bgx = (T *)(m ? p.gk : p.gq) + row0 * d;
  T *bgv = (T *)p.gv + row0 * dv;
  T *bdg = dg + row0 * (p.gate_mode == 0 ? (size_t)f : (size_t)1);
  // a load at a 32-bit byte offset from a wave-uniform base (scalar base plus
  // vector offset addressing)
  auto at = [](const auto *base, unsigned elems) {
    typedef typename std::remove_cv<typename std::remove_reference<decltype(*base)>::type>::type E;
    return *(const E *)((const char *)base + elems * (unsigned)sizeof(E));
  };
  auto fetch = [&](int tt) {
    Pre r;
    const unsigned tl = (unsigned)min(tt, nt - 1);  // token within the tile
    if constexpr (GLA) {
      r.x = to_f32(at(bx, tl * d + mic));
      r.pp = at(bph, tl * f + lanec);
      r.pn = at(bph, tl * f + f2 + lanec);
#pragma unroll
      for (int sl = 0; sl < kMaxSlices; ++sl) {
        r.dp[sl] = at(bdp[sl], tl * f + lanec);
        r.dn[sl] = at(bdp[sl], tl * f + f2 + lanec);
      }
      r.gr[0] = to_f32(at(bg, tl * gstep + glane0));
      r.gr[1] = to_f32(at(bg, tl * gstep + glane1));
#pragma unroll
      for (int w = 0; w < kMaxRowWaves; ++w) r.dvw[w] = at(bdvw[w], tl * dv + tidv);
    } else {
      r.x = r.pp = r.pn = r.gr[0] = r.gr[1] = 0.0f;
#pragma unroll
      for (int sl = 0; sl < kMaxSlices; ++sl) r.dp[sl] = r.dn[sl] = 0.0f;
#pragma unroll
      for (int w = 0; w < kMaxRowWaves; ++w) r.dvw[w] = 0.0f;
    }
    if constexpr (SWA) {
      if (p.win_bf16) {
        r.ds = to_f32(at((const bf16 *)bds0, tl * d + mic));
        r.dvs = to_f32(at((const bf16 *)bdvs0, tl * dv + tidv));
      } else {
        r.ds = at(bds, tl * d + mic);
        r.dvs = at(bdvs, tl * dv + tidv);
      }
    } else {
      r.ds = r.dvs = 0.0f;
    }
    return r;
  };

  // One token's work.  Tokens past the tile (the last group of a short tile)
  // run with zero feature gradients and store nothing, so every group runs whole
  // with no per-token branch.
  auto token = [&](const Pre &cur, int tt) {
    const bool live = tt < nt;
    const unsigned ut = (unsigned)tt;
    __syncthreads();
    if (gla) {
      if (mi < d) X[m][mi] = cur.x;
      if (wave < 2) {
        const bool ok = lane < f2;
        float dp = 0.0f, dn = 0.0f;
#pragma unroll
        for (int sl = 0; sl < kMaxSlices; ++sl) {
          dp += sl < p.nsl ? cur.dp[sl] : 0.0f;
          dn += sl < p.nsl ? cur.dn[sl] : 0.0f;
        }
        const float pp = (ok && live) ? cur.pp : 0.0f, pn = (ok && live) ? cur.pn : 0.0f;
        const float sp = wave_sum(pp * dp), sn = wave_sum(pn * dn);
        if (ok) {
          DU[wave][lane] = pp * (dp - sp) - pn * (dn - sn);
          E[wave][lane] = pp * dp;
          E[wave][f2 + lane] = pn * dn;
        }
      }
    }
    __syncthreads();
    if (gla && wave == 2) {
      float tsum = 0.0f;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = lane + 64 * u;
        if (r < f) {
          const float da = run[u];
          run[u] = da - (E[0][r] - E[1][r]);
          if (p.gate_mode == 0) {
            if (live)
              *(T *)((char *)bdg + (ut * f + r) * (unsigned)sizeof(T)) = from_f32<T>(p.gate_is_log ? da : da * rcp_fast(1.0f + exp_fast(cur.gr[u])));
          } else {
            tsum += da;
          }
        }
      }
      if (p.gate_mode == 1) {
        tsum = wave_sum(tsum);
        if (lane == 0 && live) *(T *)((char *)bdg + ut * (unsigned)sizeof(T)) = from_f32<T>(tsum);
      } else if (p.gate_mode == 2) {
        gsum += live ? tsum : 0.0f;
      }
    }
    if (mi < d && live) {
      float acc = cur.ds;
      if (gla) {
        // du . Wphi^T column mi: LDS reads requested 8 at a time into separate
        // sums (one dependent LDS round trip per feature otherwise)
        const float *du = DU[m], *wt = &WT[m][mi * kWR];
        if (f2 % 8 == 0) {
          float a8[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
          for (int j = 0; j < f2; j += 8) {
            float x8[8], w8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              x8[e] = du[j + e];
              w8[e] = wt[j + e];
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) a8[e] += x8[e] * w8[e];
          }
          acc += ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
        } else {
          for (int j = 0; j < f2; ++j) acc += du[j] * wt[j];
        }
      }
      *(T *)((char *)bgx + (ut * d + mi) * (unsigned)sizeof(T)) = from_f32<T>(acc);
    }
    if (tid < dv && live) {
      float acc = cur.dvs;
#pragma unroll
      for (int w = 0; w < kMaxRowWaves; ++w) acc += w < p.nw ? cur.dvw[w] : 0.0f;
      *(T *)((char *)bgv + (ut * dv + tid) * (unsigned)sizeof(T)) = from_f32<T>(acc);
    }
    if (gla) {
      // rows i >= d (and groups past the last row) accumulate into sums that
      // are never stored (clamped reads, no per-row branch)
      const float duq = DU[0][jj], duk = DU[1][jj];
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        aq[n] += X[0][ib + n] * duq;
        ak[n] += X[1][ib + n] * duk;
      }
    }
  };
  // Operands kFeatPF tokens ahead in a ring whose slots are fixed registers (a
  // loop-carried copy of the next token's operands made every token wait for
  // its loads, one memory round trip per token).
  Pre ring[kFeatPF];
#pragma unroll
  for (int u = 0; u < kFeatPF; ++u) ring[u] = fetch(u);
  for (int g0 = 0; g0 < nt; g0 += kFeatPF) {
#pragma unroll
    for (int u = 0; u < kFeatPF; ++u) {
      const Pre cur = ring[u];
      ring[u] = fetch(g0 + u + kFeatPF);
      token(cur, g0 + u);
    }
  }
  if (!gla) return;
  const size_t base = ((size_t)bh * p.nft + tile) * d * f2;
#pragma unroll
  for (int n = 0; n < NP; ++n) {
    const int i = i0 * NP + n;
    if (i < d) {
      p.wqp[base + (size_t)i * f2 + jj] = aq[n];
      p.wkp[base + (size_t)i * f2 + jj] = ak[n];
    }
  }
  if (p.gate_mode == 2 && wave == 2) {
    const float s2 = wave_sum(gsum);
    if (lane == 0) p.gp[(size_t)bh * p.nft + tile] = s2;
  }
}

// ---------------------------------------------------------------------------
// Window part, query side.  One wave per query token, kSwaTok tokens a block.
template <class T>
__global__ __launch_bounds__(kBT) void bwd_swa_q_kernel(BwdParams p) {
  __shared__ __align__(16) float QS[kBT / 64][kBwdMaxD];
  __shared__ __align__(16) float DO[kBT / 64][kBwdMaxD];
  __shared__ float SC[kBT / 64][kBwdMaxWindow];
  __shared__ float MR[kBT / 64][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.x / p.nsb, blk = blockIdx.x % p.nsb;
  const int h = bh % p.H, d = p.d, dv = p.dv, L = p.L;
  const T *q = (const T *)p.q, *k = (const T *)p.k, *v = (const T *)p.v, *dO = (const T *)p.dout;
  const bool sink = lane < p.n_meta;
  const float mt = sink ? p.meta[(size_t)h * p.n_meta + lane] : -INFINITY;
  const float mmax = wave_max(mt);
  float macc = 0.0f;
  float *sc = SC[wave];
  for (int tt = wave; tt < kSwaTok; tt += kBT / 64) {
    const int t = blk * kSwaTok + tt;
    if (t >= L) break;
    const size_t row = (size_t)bh * L + t;
    for (int e = lane; e < d; e += 64) QS[wave][e] = ld(q + row * d + e);
    for (int c = lane; c < dv; c += 64) DO[wave][c] = ld(dO + row * dv + c);
    __builtin_amdgcn_wave_barrier();
    const int n = min(t + 1, p.window);
    float lmax = -INFINITY;
    for (int i = lane; i < n; i += 64) {
      const T *kr = k + (row - i) * d;
      float acc = 0.0f;
      for (int e = 0; e < d; e += 4) acc += dot4(ld4(kr + e), *(const f32x4 *)&QS[wave][e]);
      const float sv = p.scale * acc;
      sc[i] = sv;
      lmax = fmaxf(lmax, sv);
    }
    const float m = fmaxf(wave_max(lmax), mmax);
    float z = 0.0f;
    for (int i = lane; i < n; i += 64) z += exp_fast(sc[i] - m);
    z = wave_sum(z) + wave_sum(sink ? exp_fast(mt - m) : 0.0f);
    const float iz = 1.0f / z;
    for (int i = lane; i < n; i += 64) sc[i] = exp_fast(sc[i] - m) * iz;
    __builtin_amdgcn_wave_barrier();
    float dsum = 0.0f;
    for (int c = lane; c < dv; c += 64) {
      float o = 0.0f;
      for (int i = 0; i < n; ++i) o += sc[i] * ld(v + (row - i) * dv + c);
      dsum += o * DO[wave][c];
    }
    const float D = wave_sum(dsum);
    for (int i = lane; i < n; i += 64) {
      const T *vr = v + (row - i) * dv;
      float dp = 0.0f;
      for (int c = 0; c < dv; c += 4) dp += dot4(ld4(vr + c), *(const f32x4 *)&DO[wave][c]);
      sc[i] = sc[i] * (dp - D);
    }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < d; e += 64) {
      float acc = 0.0f;
      for (int i = 0; i < n; ++i) acc += sc[i] * ld(k + (row - i) * d + e);
      p.dqs[row * d + e] = p.scale * acc;
    }
    if (sink) macc -= exp_fast(mt - m) * iz * D;
    if (lane == 0) {
      p.lse[row] = m + logf(z);
      p.del[row] = D;
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (p.n_meta) {
    MR[wave][lane] = macc;
    __syncthreads();
    if (tid < p.n_meta) {
      float s = 0.0f;
      for (int w = 0; w < kBT / 64; ++w) s += MR[w][tid];
      p.mp[((size_t)bh * p.nmp + blk) * p.n_meta + tid] = s;
    }
  }
}

// Window part, key side.  One wave per key token j: the queries t in
// [j, j + w - 1] that see it.
template <class T>
__global__ __launch_bounds__(kBT) void bwd_swa_kv_kernel(BwdParams p) {
  __shared__ __align__(16) float KS[kBT / 64][kBwdMaxD];
  __shared__ __align__(16) float VS[kBT / 64][kBwdMaxD];
  __shared__ float PS[kBT / 64][kBwdMaxWindow];
  __shared__ float DS[kBT / 64][kBwdMaxWindow];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int bh = blockIdx.x / p.nsb, blk = blockIdx.x % p.nsb;
  const int d = p.d, dv = p.dv, L = p.L;
  const T *q = (const T *)p.q, *k = (const T *)p.k, *v = (const T *)p.v, *dO = (const T *)p.dout;
  for (int jt = wave; jt < kSwaTok; jt += kBT / 64) {
    const int j = blk * kSwaTok + jt;
    if (j >= L) break;
    const size_t row = (size_t)bh * L + j;
    for (int e = lane; e < d; e += 64) KS[wave][e] = ld(k + row * d + e);
    for (int c = lane; c < dv; c += 64) VS[wave][c] = ld(v + row * dv + c);
    __builtin_amdgcn_wave_barrier();
    const int n = min(p.window, L - j);
    for (int i = lane; i < n; i += 64) {
      const size_t tr = row + i;
      const T *qr = q + tr * d;
      float s = 0.0f;
      for (int e = 0; e < d; e += 4) s += dot4(ld4(qr + e), *(const f32x4 *)&KS[wave][e]);
      const float P = exp_fast(p.scale * s - p.lse[tr]);
      const T *orow = dO + tr * dv;
      float dp = 0.0f;
      for (int c = 0; c < dv; c += 4) dp += dot4(ld4(orow + c), *(const f32x4 *)&VS[wave][c]);
      PS[wave][i] = P;
      DS[wave][i] = P * (dp - p.del[tr]);
    }
    __builtin_amdgcn_wave_barrier();
    for (int e = lane; e < d; e += 64) {
      float acc = 0.0f;
      for (int i = 0; i < n; ++i) acc += DS[wave][i] * ld(q + (row + i) * d + e);
      p.dks[row * d + e] = p.scale * acc;
    }
    for (int c = lane; c < dv; c += 64) {
      float acc = 0.0f;
      for (int i = 0; i < n; ++i) acc += PS[wave][i] * ld(dO + (row + i) * dv + c);
      p.dvs[row * dv + c] = acc;
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// ---------------------------------------------------------------------------
// Window part in 64-token tiles (bf16, d = d_v = 128, window <= 64, n_meta <=
// 16): the same quantities as the two per-token kernels above, computed as
// LDS-tiled fp32 products.  A query tile (64 queries of chunk c) meets the 128
// keys of chunks c-1 and c; a key tile (64 keys of chunk c) meets the 128
// queries of chunks c and c+1.  512 threads: thread (rg, cg) = (tid / 16,
// tid % 16) holds score rows 2rg, 2rg+1 and columns cg + 16j (j < 8), so each
// row's 16 threads are one 16-lane DPP row; the products with the scores hold
// rows 2rg, 2rg+1 and output columns 8cg .. 8cg+7.
constexpr int kWT = 512;          // threads of a window tile block
constexpr int kWC = 64;           // tokens of a tile
constexpr int kWD = 128;          // d = d_v of the tiled path
constexpr int kWS = kWD + 8;      // LDS row stride (bf16): consecutive rows 4 banks apart
constexpr int kWP = 2 * kWC + 1;  // score row stride (fp32)

struct WinTileLds {
  bf16 a[kWC][kWS];          // query tile: Q; key tile: K
  bf16 b[kWC][kWS];          // query tile: dO; key tile: V
  bf16 c[2 * kWC][kWS];      // query tile: K; key tile: Q
  bf16 e[2 * kWC][kWS];      // query tile: V; key tile: dO
  float sc[kWC][kWP];        // scores / weights of the tile
  float lse[2 * kWC], del[2 * kWC];
  float mp[kWT / 16][16];
};

// The four operand matrices of a tile: rows [ra, ra + kWC) of sa and sb, rows
// [rc, rc + 2 kWC) of sc and se (zeros outside [0, L), L >= 1).  Every load
// is issued (from clamped rows) before the first LDS store: a load per store
// made each block wait one memory round trip per step.
__device__ __forceinline__ void win_stage_all(WinTileLds &S, const bf16 *sa, const bf16 *sb, int ra, const bf16 *sc,
                                              const bf16 *se, int rc, size_t bh, int L) {
  constexpr int kQ = kWD / 8;             // 16-byte quads per row
  constexpr int kA = kWC * kQ / kWT;      // quads per thread of a kWC-row matrix
  constexpr int kC = 2 * kWC * kQ / kWT;  // of a 2 kWC-row matrix
  static_assert(kA * kWT == kWC * kQ && kC * kWT == 2 * kWC * kQ, "whole quads per thread");
  const int tid = threadIdx.x;
  auto at = [&](const bf16 *src, int r0, int idx) {
    const int pos = min(max(r0 + idx / kQ, 0), L - 1);
    return *(const u32x4 *)(src + ((size_t)bh * L + pos) * kWD + (idx % kQ) * 8);
  };
  u32x4 xa[kA], xb[kA], xc[kC], xe[kC];
#pragma unroll
  for (int k = 0; k < kA; ++k) {
    xa[k] = at(sa, ra, tid + kWT * k);
    xb[k] = at(sb, ra, tid + kWT * k);
  }
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    xc[k] = at(sc, rc, tid + kWT * k);
    xe[k] = at(se, rc, tid + kWT * k);
  }
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k = 0; k < kA; ++k) {
    const int idx = tid + kWT * k, r = idx / kQ, c8 = (idx % kQ) * 8;
    const bool ok = ra + r >= 0 && ra + r < L;
    *(u32x4 *)&S.a[r][c8] = ok ? xa[k] : z;
    *(u32x4 *)&S.b[r][c8] = ok ? xb[k] : z;
  }
#pragma unroll
  for (int k = 0; k < kC; ++k) {
    const int idx = tid + kWT * k, r = idx / kQ, c8 = (idx % kQ) * 8;
    const bool ok = rc + r >= 0 && rc + r < L;
    *(u32x4 *)&S.c[r][c8] = ok ? xc[k] : z;
    *(u32x4 *)&S.e[r][c8] = ok ? xe[k] : z;
  }
}

__device__ __forceinline__ void bf8(const bf16 *p, float (&x)[8]) {
  const u32x4 w = *(const u32x4 *)p;
  const bf16 *e = (const bf16 *)&w;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)e[j];
}

// acc[i][j] = sum_e A[2rg+i][e] B[cg+16j][e] over e < 128 (A rows broadcast
// in the 16-lane row, B rows 16 apart)
__device__ __forceinline__ void win_scores(const bf16 (*A)[kWS], const bf16 (*Bm)[kWS], int rg, int cg,
                                           float (&acc)[2][8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0f;
  for (int e = 0; e < kWD; e += 8) {
    float a0[8], a1[8];
    bf8(&A[2 * rg][e], a0);
    bf8(&A[2 * rg + 1][e], a1);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float b[8];
      bf8(&Bm[cg + 16 * j][e], b);
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        acc[0][j] += a0[u] * b[u];
        acc[1][j] += a1[u] * b[u];
      }
    }
  }
}

// out[i][u] = sum_x W[2rg+i][x] M[x][8cg+u] over x < 2 kWC (W the fp32 score
// tile, M a bf16 LDS matrix)
__device__ __forceinline__ void win_apply(const float (*W)[kWP], const bf16 (*M)[kWS], int rg, int cg,
                                          float (&out)[2][8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int u = 0; u < 8; ++u) out[i][u] = 0.0f;
  for (int x = 0; x < 2 * kWC; ++x) {
    float m[8];
    bf8(&M[x][8 * cg], m);
    const float w0 = W[2 * rg][x], w1 = W[2 * rg + 1][x];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      out[0][u] += w0 * m[u];
      out[1][u] += w1 * m[u];
    }
  }
}

// Query tile: dq (window part), lse, D and the sinks' gradient partial.
__global__ __launch_bounds__(kWT) void bwd_swa_tile_q_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  WinTileLds &S = *(WinTileLds *)smem;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int nch = (p.L + kWC - 1) / kWC;
  const size_t bh = blockIdx.x / nch;
  const int c = blockIdx.x % nch, t0 = c * kWC, h = (int)(bh % p.H);
  const bf16 *q = (const bf16 *)p.q, *k = (const bf16 *)p.k, *v = (const bf16 *)p.v, *dO = (const bf16 *)p.dout;
  win_stage_all(S, q, dO, t0, k, v, t0 - kWC, bh, p.L);
  __syncthreads();

  float sc[2][8], dp[2][8];
  win_scores(S.a, S.c, rg, cg, sc);
  win_scores(S.b, S.e, rg, cg, dp);
  const float tm = cg < p.n_meta ? p.meta[(size_t)h * p.n_meta + cg] : -INFINITY;
  float mm = tm;  // max of the sinks over the 16 lanes
  mm = fmaxf(mm, dpp_f<0xB1>(mm));
  mm = fmaxf(mm, dpp_f<0x4E>(mm));
  mm = fmaxf(mm, dpp_f<0x141>(mm));
  mm = fmaxf(mm, dpp_f<0x140>(mm));
  float mpart = 0.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 2 * rg + i;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int kp = t0 - kWC + cg + 16 * j;  // key position
      const bool ok = t < p.L && kp >= 0 && kp <= t && t - kp < p.window;
      sc[i][j] = ok ? sc[i][j] * p.scale : -INFINITY;
      mx = fmaxf(mx, sc[i][j]);
    }
    const float m = fmaxf(row16_reduce(mx, OpMax()), mm);
    float z = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sc[i][j] = exp_fast(sc[i][j] - m);  // 0 outside the window
      z += sc[i][j];
    }
    const float es = cg < p.n_meta ? exp_fast(tm - m) : 0.0f;
    z = row16_reduce(z + es, OpAdd());
    const float iz = 1.0f / z;
    float dsum = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sc[i][j] *= iz;
      dsum += sc[i][j] * dp[i][j];
    }
    const float D = row16_reduce(dsum, OpAdd());
#pragma unroll
    for (int j = 0; j < 8; ++j) S.sc[2 * rg + i][cg + 16 * j] = sc[i][j] * (dp[i][j] - D);
    if (t < p.L) {
      mpart -= es * iz * D;
      if (cg == 0) {
        p.lse[bh * p.L + t] = m + logf(z);
        p.del[bh * p.L + t] = D;
      }
    }
  }
  S.mp[rg][cg] = mpart;
  __syncthreads();
  float dq[2][8];
  win_apply(S.sc, S.c, rg, cg, dq);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int t = t0 + 2 * rg + i;
    if (t < p.L) {
      float *dst = p.dqs + (bh * p.L + t) * kWD + 8 * cg;
      *(f32x4 *)dst = (f32x4){dq[i][0], dq[i][1], dq[i][2], dq[i][3]} * p.scale;
      *(f32x4 *)(dst + 4) = (f32x4){dq[i][4], dq[i][5], dq[i][6], dq[i][7]} * p.scale;
    }
  }
  // the sinks' gradient of this tile goes to its first 16-token block, zeros
  // to the others (the reduction sums all blocks in a fixed order)
  if (tid < p.n_meta * (kWC / kSwaTok)) {
    const int m = tid % p.n_meta, sub = tid / p.n_meta, blk = c * (kWC / kSwaTok) + sub;
    float acc = 0.0f;
    if (sub == 0)
      for (int r = 0; r < kWT / 16; ++r) acc += S.mp[r][m];
    if (blk < p.nmp) p.mp[(bh * p.nmp + blk) * p.n_meta + m] = acc;
  }
}

// Key tile: dk and dv (window parts) of the 64 keys of chunk c from the 128
// queries of chunks c and c+1, with the query kernel's lse and D.
__global__ __launch_bounds__(kWT) void bwd_swa_tile_kv_kernel(BwdParams p) {
  extern __shared__ __align__(16) unsigned char smem[];
  WinTileLds &S = *(WinTileLds *)smem;
  const int tid = threadIdx.x, rg = tid >> 4, cg = tid & 15;
  const int nch = (p.L + kWC - 1) / kWC;
  const size_t bh = blockIdx.x / nch;
  const int c = blockIdx.x % nch, j0 = c * kWC;
  const bf16 *q = (const bf16 *)p.q, *k = (const bf16 *)p.k, *v = (const bf16 *)p.v, *dO = (const bf16 *)p.dout;
  win_stage_all(S, k, v, j0, q, dO, j0, bh, p.L);
  if (tid < 2 * kWC) {
    const int t = j0 + tid;
    const float ls = p.lse[bh * p.L + min(t, p.L - 1)], de = p.del[bh * p.L + min(t, p.L - 1)];
    S.lse[tid] = t < p.L ? ls : 0.0f;
    S.del[tid] = t < p.L ? de : 0.0f;
  }
  __syncthreads();

  float sc[2][8], dp[2][8];
  win_scores(S.a, S.c, rg, cg, sc);
  win_scores(S.b, S.e, rg, cg, dp);
  float pw[2][8];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kp = j0 + 2 * rg + i;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int x = cg + 16 * j, t = j0 + x;  // query position
      const bool ok = kp < p.L && t < p.L && t >= kp && t - kp < p.window;
      pw[i][j] = ok ? exp_fast(sc[i][j] * p.scale - S.lse[x]) : 0.0f;
      S.sc[2 * rg + i][x] = pw[i][j];
    }
  }
  __syncthreads();
  float dvv[2][8];
  win_apply(S.sc, S.e, rg, cg, dvv);  // dv_j = sum_t P_tj dO_t
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int x = cg + 16 * j;
      S.sc[2 * rg + i][x] = pw[i][j] * (dp[i][j] - S.del[x]);
    }
  __syncthreads();
  float dkk[2][8];
  win_apply(S.sc, S.c, rg, cg, dkk);  // dk_j = scale sum_t ds_tj q_t
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int kp = j0 + 2 * rg + i;
    if (kp < p.L) {
      float *dk = p.dks + (bh * p.L + kp) * kWD + 8 * cg, *dvp = p.dvs + (bh * p.L + kp) * kWD + 8 * cg;
      *(f32x4 *)dk = (f32x4){dkk[i][0], dkk[i][1], dkk[i][2], dkk[i][3]} * p.scale;
      *(f32x4 *)(dk + 4) = (f32x4){dkk[i][4], dkk[i][5], dkk[i][6], dkk[i][7]} * p.scale;
      *(f32x4 *)dvp = (f32x4){dvv[i][0], dvv[i][1], dvv[i][2], dvv[i][3]};
      *(f32x4 *)(dvp + 4) = (f32x4){dvv[i][4], dvv[i][5], dvv[i][6], dvv[i][7]};
    }
  }
}

// ---------------------------------------------------------------------------
// Sums of the per-block partials over batch rows and token blocks: dWphi_q,
// dWphi_k [H][d][f/2], the sink gradients [H][n_meta] and, for a per-head
// gate, its gradient [H].  Fixed order, one output per thread.
// Sums of the per-block partials, each in a fixed order: blocks [0, nwb) take
// 64 quads of dWphi_q / dWphi_k, four waves a quad (a quarter of the partials
// each, added in LDS); then one block per
// head sums its sink-gradient partials (thread (part, sink) over every fourth
// partial, the four parts added in LDS); a last block sums the per-head gate
// gradient (one gate per head).
constexpr int kRedQuads = 64;  // dW quads (4 elements) a block of the partial sums

template <class T>
__global__ __launch_bounds__(kBT) void bwd_reduce_kernel(BwdParams p) {
  const size_t per = (size_t)p.d * p.f2;  // a multiple of 4 (d is)
  const size_t nw4 = p.gla ? 2 * (size_t)p.H * per / 4 : 0;
  const size_t nwb = (nw4 + kRedQuads - 1) / kRedQuads;
  const size_t nmb = (p.swa && p.n_meta > 0) ? (size_t)p.H : 0;
  constexpr int kRG = 16;  // partials loaded (clamped, masked) before they are added
  if (blockIdx.x < nwb) {
    // 64 quads a block; wave wv sums its quarter of every batch row's
    // partials, and the four quarters are added in LDS in a fixed order
    constexpr int kRQ = kBT / kRedQuads;
    __shared__ f32x4 wpart[kRQ][kRedQuads];
    const int l = threadIdx.x % kRedQuads, wv = threadIdx.x / kRedQuads;
    const size_t idx = (size_t)blockIdx.x * kRedQuads + l;
    const bool ok = idx < nw4;
    const size_t nwt = (size_t)p.H * per, e4 = 4 * (ok ? idx : nw4 - 1);
    const int m = e4 >= nwt;
    const size_t e = e4 - m * nwt, h = e / per, r = e - h * per;
    const float *src = m ? p.wkp : p.wqp;
    const int qn = (p.nwp + kRQ - 1) / kRQ, t_lo = min(wv * qn, p.nwp), t_hi = min(t_lo + qn, p.nwp);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int b = 0; b < p.B; ++b) {
      const float *row = src + ((size_t)b * p.H + h) * p.nwp * per + r;
      for (int t0 = t_lo; t0 < t_hi; t0 += kRG) {
        f32x4 x[kRG];
#pragma unroll
        for (int u = 0; u < kRG; ++u) x[u] = *(const f32x4 *)(row + (size_t)min(t0 + u, t_hi - 1) * per);
#pragma unroll
        for (int u = 0; u < kRG; ++u)
          if (t0 + u < t_hi) acc += x[u];
      }
    }
    wpart[wv][l] = acc;
    __syncthreads();
    if (wv == 0 && ok) {
      acc = wpart[0][l];
#pragma unroll
      for (int q = 1; q < kRQ; ++q) acc += wpart[q][l];
      float *dst = (m ? p.dwk : p.dwq) + e;
      if (p.accum) acc += *(const f32x4 *)dst;
      *(f32x4 *)dst = acc;
    }
  } else if (blockIdx.x < nwb + nmb) {
    __shared__ float part[kBT / 64][64];
    const int h = (int)(blockIdx.x - nwb), mm = threadIdx.x & 63, pt = threadIdx.x >> 6;
    const int mmc = min(mm, max(p.n_meta - 1, 0));
    float acc = 0.0f;
    for (int b = 0; b < p.B; ++b) {
      const float *col = p.mp + ((size_t)b * p.H + h) * p.nmp * p.n_meta + mmc;
      for (int t0 = pt; t0 < p.nmp; t0 += 4 * kRG) {
        float x[kRG];
#pragma unroll
        for (int u = 0; u < kRG; ++u) x[u] = col[(size_t)min(t0 + 4 * u, p.nmp - 1) * p.n_meta];
#pragma unroll
        for (int u = 0; u < kRG; ++u)
          if (t0 + 4 * u < p.nmp) acc += x[u];
      }
    }
    part[pt][mm] = acc;
    __syncthreads();
    if (pt == 0 && mm < p.n_meta) {
      float *dst = p.dmeta + (size_t)h * p.n_meta + mm;
      const float sum = ((part[0][mm] + part[1][mm]) + part[2][mm]) + part[3][mm];
      *dst = p.accum ? *dst + sum : sum;
    }
  } else {
    for (int h = threadIdx.x; h < p.H; h += kBT) {
      float acc = 0.0f;
      for (int b = 0; b < p.B; ++b)
        for (int tl = 0; tl < p.nft; ++tl) acc += p.gp[((size_t)b * p.H + h) * p.nft + tl];
      if (p.accum) acc += p.gacc[h];
      p.gacc[h] = acc;
      ((T *)p.gg)[h] = from_f32<T>(acc);
    }
  }
}

// Workspace layout, in floats; every region starts on a 256-byte boundary.
struct BwdLayout {
  size_t pq, pk, gam, tq, tk, ta, dpq, dpk, dvg, xs, lse, del, dqs, dks, dvs, wqp, wkp, gp, mp, wst, gacc, total;
};

size_t up64(size_t n) { return (n + 63) & ~(size_t)63; }

// The state walks write complete feature sums (one d_v slice); the token
// sweeps one partial sum per 32-column slice of d_v.
bool use_walk(const LayerArgs &a, int parts) {
  return (parts & PART_GLA) && bwd_walk_supported(a.f, a.dv, a.L, a.bf16);
}
size_t sweep_slices(const LayerArgs &a, int parts) {
  return use_walk(a, parts) ? 1 : (size_t)(a.dv + kSliceCols - 1) / kSliceCols;
}
// dv parts of the gated part: the walks sum theirs; the sweeps leave one per
// 32 features
size_t row_parts(const LayerArgs &a, int parts) { return use_walk(a, parts) ? 1 : (size_t)(a.f + 31) / 32; }

// The matrix-core window kernels, and the per-token kernel on the matrix cores
// (per-feature gates, bf16, d = f = d_v = 128, after the walks).  With the
// latter the window part, when it runs, is the matrix-core one and goes first:
// it writes its dq, dk, dv into the output rows, the reverse walk adds the
// gated part's dv to them and the per-token kernel its dq and dk, so neither
// part's gradients pass through the workspace.
bool use_win_mfma(const LayerArgs &a, int parts) {
  return (parts & PART_SWA) && bwd_window_mfma_supported(a.d, a.dv, a.window, a.n_meta, a.bf16);
}
bool use_feat_mfma(const LayerArgs &a, int parts) {
  return use_walk(a, parts) && bwd_feat_mfma_supported(a.d, a.f, a.dv, a.L, a.gate_mode, a.bf16) &&
         (!(parts & PART_SWA) || use_win_mfma(a, parts));
}
// dW partials per head: one a block of the matrix-core per-token kernel, else
// one a 64-token tile
size_t dw_partials(const LayerArgs &a, int parts) {
  const size_t nft = (a.L + kFeatTok - 1) / kFeatTok;
  if (!use_feat_mfma(a, parts)) return nft;
  const size_t span = (size_t)bwd_feat_span(a.B * a.H, a.L);
  return ((a.L + 15) / 16 + span - 1) / span;
}

BwdLayout bwd_layout(const LayerArgs &a, int parts) {
  const size_t BH = (size_t)a.B * a.H, N = BH * a.L;
  const size_t nsl = sweep_slices(a, parts), nw = row_parts(a, parts);
  const size_t nft = (a.L + kFeatTok - 1) / kFeatTok, nsb = (a.L + kSwaTok - 1) / kSwaTok;
  // the window part's dq, dk, dv: bf16 from the matrix-core kernels, none when
  // they go straight to the output rows
  const size_t wsz = use_win_mfma(a, parts) ? 2 : 1;
  const bool gla = parts & PART_GLA, swa = parts & PART_SWA, feat_mfma = use_feat_mfma(a, parts);
  const size_t nws = swa && !feat_mfma ? N : 0;
  BwdLayout o;
  size_t at = 0;
  auto take = [&](size_t n) { const size_t r = at; at += up64(n); return r; };
  const size_t nf = gla ? N * a.f : 0;
  o.pq = take(nf); o.pk = take(nf); o.gam = take(nf);
  const size_t nt = gla ? BH * nft * a.f : 0;
  o.tq = take(nsl * nt); o.tk = take(nsl * nt); o.ta = take(nt);
  o.dpq = take(nsl * nf); o.dpk = take(nsl * nf);
  // the gated part's dv (none when the reverse walk writes the finished dv)
  o.dvg = take(gla && !feat_mfma ? nw * N * a.dv : 0);
  o.xs = take(gla ? 2 * BH * nsl * a.f : 0);
  // lse and D of the window part (the matrix-core kernel keeps them in LDS)
  const size_t nld = swa && !use_win_mfma(a, parts) ? N : 0;
  o.lse = take(nld); o.del = take(nld);
  o.dqs = take(nws * a.d / wsz); o.dks = take(nws * a.d / wsz);
  o.dvs = take(nws * a.dv / wsz);
  const size_t wp = gla ? BH * dw_partials(a, parts) * a.d * (a.f / 2) : 0;
  o.wqp = take(wp); o.wkp = take(wp);
  o.gp = take(gla ? BH * nft : 0);
  o.mp = take(swa ? BH * nsb * a.n_meta : 0);
  o.wst = take(use_walk(a, parts) ? bwd_walk_ws_floats((int)BH, a.L) : 0);
  o.gacc = take(gla && a.gate_mode == 2 ? a.H : 0);
  o.total = at;
  return o;
}

// A side stream and two events per device, created on first use and kept
// until the process ends: the window part of the backward runs on it beside
// the prologue and the state sweeps (the two share only inputs, and a window
// tile block fits on a compute unit next to a sweep block).  The lock is held
// while a call enqueues, so concurrent calls do not interleave their event
// records.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool tried = false;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxDevices];

// The current device's side stream, or nullptr: no device id, creation failed,
// or the caller's stream is being captured into a graph before the side stream
// exists (creating one then is not allowed); the caller then runs everything
// on its own stream.  Call with g_side_mu held.
SideStream *side_stream(hipStream_t main) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  SideStream &ss = g_side[dev];
  if (!ss.tried) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(main, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return nullptr;
    ss.tried = true;
    if (hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&ss.join, hipEventDisableTiming) != hipSuccess) {
      ss.s = nullptr;
      (void)hipGetLastError();
    }
  }
  return ss.s ? &ss : nullptr;
}

template <class T>
hipError_t bwd_dispatch(const LayerArgs &a, const BwdArgs &g, int parts, bool accum) {
  BwdParams p = {};
  p.accum = accum ? 1 : 0;
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.wq = a.wq; p.wk = a.wk; p.dout = g.dout;
  p.meta = a.meta; p.state_in = a.state_in; p.dstate_out = g.dstate_out;
  p.gq = g.dq; p.gk = g.dk; p.gv = g.dv; p.gg = g.dgate;
  p.dwq = g.dwq; p.dwk = g.dwk; p.dmeta = g.dmeta; p.dstate_in = g.dstate_in;
  const BwdLayout lay = bwd_layout(a, parts);
  float *ws = (float *)a.ws;
  p.pq = ws + lay.pq; p.pk = ws + lay.pk; p.gam = ws + lay.gam;
  p.tq = ws + lay.tq; p.tk = ws + lay.tk; p.ta = ws + lay.ta;
  p.dpq = ws + lay.dpq; p.dpk = ws + lay.dpk; p.dvg = ws + lay.dvg; p.xs = ws + lay.xs;
  p.lse = ws + lay.lse; p.del = ws + lay.del; p.dqs = ws + lay.dqs; p.dks = ws + lay.dks;
  p.dvs = ws + lay.dvs; p.wqp = ws + lay.wqp; p.wkp = ws + lay.wkp; p.gp = ws + lay.gp; p.mp = ws + lay.mp;
  p.gacc = ws + lay.gacc;
  p.B = a.B; p.H = a.H; p.L = a.L; p.d = a.d; p.dv = a.dv; p.f = a.f; p.f2 = a.f / 2;
  p.lf2 = 0;
  while ((1 << p.lf2) < p.f2) ++p.lf2;
  p.window = a.window; p.n_meta = a.n_meta;
  p.nsl = (int)sweep_slices(a, parts); p.nw = (int)row_parts(a, parts);
  p.gam_cum = use_walk(a, parts) ? 1 : 0;
  const bool feat_mfma = use_feat_mfma(a, parts);
  p.nft = (a.L + kFeatTok - 1) / kFeatTok; p.nsb = (a.L + kSwaTok - 1) / kSwaTok;
  p.nwp = (int)dw_partials(a, parts);
  // the matrix-core window kernels leave one sink partial a 64-token chunk,
  // the others one a 16-token block
  const bool win_mfma = use_win_mfma(a, parts);
  p.nmp = win_mfma ? (a.L + 63) / 64 : p.nsb;
  p.win_bf16 = win_mfma ? 1 : 0;
  p.npt = (a.L + kPrepTok - 1) / kPrepTok;
  p.scale = a.scale; p.gate_is_log = a.gate_is_log ? 1 : 0; p.gate_mode = a.gate_mode;
  p.gla = (parts & PART_GLA) != 0; p.swa = (parts & PART_SWA) != 0;
  if (!p.gla) p.dstate_out = nullptr;

  const unsigned BH = (unsigned)(a.B * a.H);
  const dim3 block(kBT);
  hipError_t e = hipSuccess;
  auto launched = [&]() { if (e == hipSuccess) e = hipGetLastError(); return e == hipSuccess; };
  // the window part on the side stream when both parts run and meet only in
  // the per-token kernel (forked from and joined back to the caller's stream),
  // else on the caller's stream: with the matrix-core per-token kernel it goes
  // first and the reverse walk adds to its dv
  std::unique_lock<std::mutex> lock(g_side_mu, std::defer_lock);
  SideStream *ss = nullptr;
  if (p.gla && p.swa && !feat_mfma && a.L > 0 && BH > 0) {
    lock.lock();
    ss = side_stream(a.stream);
    if (!ss) lock.unlock();
  }
  const hipStream_t wstream = ss ? ss->s : a.stream;
  if (ss) {
    if ((e = hipEventRecord(ss->fork, a.stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
  }
  // the window part: on the side stream, or (matrix-core per-token kernel)
  // after the walks, adding its dv to theirs in the output rows
  auto launch_window = [&]() -> hipError_t {
    if (!p.swa || a.L <= 0) return hipSuccess;
    if (win_mfma) {
      WinBwdArgs wa;
      wa.q = a.q; wa.k = a.k; wa.v = a.v; wa.dout = g.dout; wa.meta = a.meta;
      wa.mp = p.mp;
      if (feat_mfma) {
        wa.dq = g.dq; wa.dk = g.dk; wa.dv = g.dv; wa.add_dv = p.gla;
      } else {
        wa.dq = p.dqs; wa.dk = p.dks; wa.dv = p.dvs;
      }
      wa.B = a.B; wa.H = a.H; wa.L = a.L; wa.window = a.window; wa.n_meta = a.n_meta;
      wa.scale = a.scale;
      return launch_bwd_window_mfma(wa, wstream);
    }
    if (std::is_same<T, bf16>::value && a.d == kWD && a.dv == kWD && a.window <= kWC && a.n_meta <= 16) {
      const unsigned nch = (unsigned)((a.L + kWC - 1) / kWC);
      const size_t lds = sizeof(WinTileLds);
      // dynamic LDS above 64 KiB has to be allowed for each kernel
      hipError_t we = hipFuncSetAttribute((const void *)bwd_swa_tile_q_kernel,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
      if (we == hipSuccess)
        we = hipFuncSetAttribute((const void *)bwd_swa_tile_kv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                 (int)lds);
      if (we != hipSuccess) return we;
      hipLaunchKernelGGL(bwd_swa_tile_q_kernel, dim3(BH * nch), dim3(kWT), lds, wstream, p);
      if ((we = hipGetLastError()) != hipSuccess) return we;
      hipLaunchKernelGGL(bwd_swa_tile_kv_kernel, dim3(BH * nch), dim3(kWT), lds, wstream, p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL(bwd_swa_q_kernel<T>, dim3(BH * p.nsb), block, 0, wstream, p);
    hipError_t we = hipGetLastError();
    if (we != hipSuccess) return we;
    hipLaunchKernelGGL(bwd_swa_kv_kernel<T>, dim3(BH * p.nsb), block, 0, wstream, p);
    return hipGetLastError();
  };
  if (!feat_mfma && (e = launch_window()) != hipSuccess) return e;
  if (p.gla && a.L > 0 && use_walk(a, parts) && bwd_prep_mfma_supported(a.d, a.f, a.L, a.bf16)) {
    PrepArgs pa;
    pa.q = a.q; pa.k = a.k; pa.gate = a.gate; pa.wq = a.wq; pa.wk = a.wk;
    pa.pq = p.pq; pa.pk = p.pk; pa.gb = p.gam;
    pa.BH = (int)BH; pa.H = a.H; pa.L = a.L; pa.gate_mode = a.gate_mode; pa.gate_is_log = a.gate_is_log;
    if ((e = launch_bwd_prep_mfma(pa, a.stream)) != hipSuccess) return e;
  } else if (p.gla && a.L > 0) {
    if (a.f / 2 % 4 == 0) {
      const unsigned ntl = (unsigned)((a.L + kPrepTile - 1) / kPrepTile);
      hipLaunchKernelGGL(bwd_prep_tile_kernel<T>, dim3(BH * ntl), block, 0, a.stream, p);
    } else {
      hipLaunchKernelGGL(bwd_prep_kernel<T>, dim3(BH * p.npt), block, 0, a.stream, p);
    }
    if (!launched()) return e;
  }
  if (p.gla && BH > 0) {
    // with no tokens the sweeps still pass dS_final through to dS_0
    if (use_walk(a, parts)) {
      WalkArgs wa;
      wa.pq = p.pq; wa.pk = p.pk; wa.gb = p.gam; wa.v = a.v; wa.dout = g.dout; wa.ws = ws + lay.wst;
      wa.state_in = a.state_in; wa.dstate_out = p.dstate_out;
      wa.dpq = p.dpq; wa.dpk = p.dpk; wa.dvg = p.dvg; wa.tq = p.tq; wa.tk = p.tk; wa.xs = p.xs;
      wa.dstate_in = g.dstate_in;
      wa.dv = g.dv; wa.dv_mode = feat_mfma ? (p.swa ? 2 : 1) : 0;
      wa.BH = (int)BH; wa.L = a.L; wa.nft = p.nft;
      if ((e = launch_bwd_walk(wa, a.stream)) != hipSuccess) return e;
    } else {
      hipLaunchKernelGGL(bwd_sweeps_kernel<T>, dim3(2 * BH * p.nsl), block, 0, a.stream, p);
      if (!launched()) return e;
    }
    if (a.L > 0) {
      hipLaunchKernelGGL(bwd_tile_scan_kernel, dim3((unsigned)(BH * (size_t)((a.f + kTsFeat - 1) / kTsFeat))), block,
                         0, a.stream, p);
      if (!launched()) return e;
    }
  }
  if (feat_mfma && (e = launch_window()) != hipSuccess) return e;
  if (ss) {  // the per-token kernel reads the window part's outputs
    if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(a.stream, ss->join, 0)) != hipSuccess) return e;
    lock.unlock();
  }
  if (a.L > 0 && BH > 0 && feat_mfma) {
    FeatArgs fa;
    fa.q = a.q; fa.k = a.k; fa.gate = a.gate; fa.wq = a.wq; fa.wk = a.wk;
    fa.pq = p.pq; fa.pk = p.pk; fa.dpq = p.dpq; fa.dpk = p.dpk; fa.ta = p.ta;
    fa.swa = p.swa;
    fa.dq = g.dq; fa.dk = g.dk; fa.dg = g.dgate; fa.wqp = p.wqp; fa.wkp = p.wkp;
    fa.BH = (int)BH; fa.H = a.H; fa.L = a.L; fa.nft = p.nft; fa.gate_is_log = a.gate_is_log;
    if ((e = launch_bwd_feat_mfma(fa, a.stream)) != hipSuccess) return e;
  } else if (a.L > 0 && BH > 0) {
    if (p.gla && p.swa)
      hipLaunchKernelGGL((bwd_feature_kernel<T, true, true>), dim3(BH * p.nft), block, 0, a.stream, p);
    else if (p.gla)
      hipLaunchKernelGGL((bwd_feature_kernel<T, true, false>), dim3(BH * p.nft), block, 0, a.stream, p);
    else
      hipLaunchKernelGGL((bwd_feature_kernel<T, false, true>), dim3(BH * p.nft), block, 0, a.stream, p);
    if (!launched()) return e;
  }
  const size_t nwb = p.gla ? (2 * (size_t)a.H * a.d * p.f2 / 4 + kRedQuads - 1) / kRedQuads : 0;
  const size_t nred = nwb + ((p.swa && a.n_meta > 0) ? (size_t)a.H : 0) + ((p.gla && a.gate_mode == 2) ? 1 : 0);
  if (nred) {
    hipLaunchKernelGGL(bwd_reduce_kernel<T>, dim3((unsigned)nred), block, 0, a.stream, p);
    if (!launched()) return e;
  }
  return e;
}

}  // namespace

bool bwd_supported(const LayerArgs &a, int parts) {
  if (a.d > kBwdMaxD || a.dv > kBwdMaxD || (a.d & 3) || (a.dv & 3)) return false;
  if (parts & PART_GLA) {
    const int f2 = a.f / 2;
    if (a.f > kBwdMaxF || (a.f & 3) || (f2 & (f2 - 1))) return false;
  }
  if ((parts & PART_SWA) && (a.window > kBwdMaxWindow || a.n_meta > 64)) return false;
  return true;
}

// The backward of every (batch row, head) is independent of the others, so a
// call can run as a sequence of sub-problems, each with its own share of the
// workspace: blocks of whole batch rows (every head), or one batch row and a
// block of heads.  They run head block by head block, batch rows innermost, so
// the per-head sums over the batch (dWphi, the sink gradients, a per-head
// gate's gradient) are written by a block's first row and added to by the
// others.  The plan is the fewest sub-problems whose workspace fits.
namespace {

struct BwdPlan {
  bool ok = false;
  int rows = 0, heads = 0;  // sub-problem shape
};

LayerArgs bwd_sub_shape(const LayerArgs &a, int rows, int heads) {
  LayerArgs s = a;
  s.B = rows;
  s.H = heads;
  return s;
}

size_t bwd_sub_bytes(const LayerArgs &a, int parts, int rows, int heads) {
  return bwd_layout(bwd_sub_shape(a, rows, heads), parts).total * sizeof(float);
}

// candidates, fewest sub-problems first: the whole call, blocks of rows, then
// one row and blocks of heads; the first whose workspace is at most `cap`
BwdPlan bwd_plan(const LayerArgs &a, int parts, size_t cap) {
  if (bwd_sub_bytes(a, parts, a.B, a.H) <= cap) return {true, a.B, a.H};
  if (a.B <= 0 || a.H <= 0) return {};
  for (int r = a.B - 1; r >= 1; --r)
    if (a.B % r == 0 && bwd_sub_bytes(a, parts, r, a.H) <= cap) return {true, r, a.H};
  for (int h = a.H - 1; h >= 1; --h)
    if (a.H % h == 0 && bwd_sub_bytes(a, parts, 1, h) <= cap) return {true, 1, h};
  return {};
}

// the workspace the sizing query reports: the whole call's when it is at most
// this, else the largest sub-problem's that is
constexpr size_t kBwdDefaultBytes = 1500000000;

}  // namespace

size_t bwd_workspace_min_bytes(const LayerArgs &a, int parts) {
  if (a.B <= 0 || a.H <= 0) return bwd_sub_bytes(a, parts, a.B, a.H);
  return bwd_sub_bytes(a, parts, 1, 1);
}

size_t bwd_workspace_whole_bytes(const LayerArgs &a, int parts) { return bwd_sub_bytes(a, parts, a.B, a.H); }

size_t bwd_workspace_bytes(const LayerArgs &a, int parts) {
  const BwdPlan pl = bwd_plan(a, parts, kBwdDefaultBytes);
  return pl.ok ? bwd_sub_bytes(a, parts, pl.rows, pl.heads) : bwd_workspace_min_bytes(a, parts);
}

hipError_t launch_layer_bwd(const LayerArgs &a, const BwdArgs &g, int parts) {
  const BwdPlan pl = bwd_plan(a, parts, a.ws_bytes);
  if (!pl.ok) return hipErrorInvalidValue;  // the caller checks the minimum
  auto run = [&](const LayerArgs &s, const BwdArgs &sg, bool accum) {
    return s.bf16 ? bwd_dispatch<bf16>(s, sg, parts, accum) : bwd_dispatch<float>(s, sg, parts, accum);
  };
  if (pl.rows == a.B && pl.heads == a.H) return run(a, g, false);
  const size_t es = a.bf16 ? 2 : 4, L = (size_t)a.L;
  const size_t gtok = a.gate_mode == 0 ? (size_t)a.f : 1;  // gate elements per token (modes 0, 1)
  for (int h0 = 0; h0 < a.H; h0 += pl.heads) {
    for (int b0 = 0; b0 < a.B; b0 += pl.rows) {
      const size_t bh0 = (size_t)b0 * a.H + h0;  // first (row, head) of the sub-problem
      auto at = [&](const void *x, size_t elems, size_t bytes) -> const void * {
        return x ? (const char *)x + elems * bytes : nullptr;
      };
      auto atw = [&](void *x, size_t elems, size_t bytes) -> void * {
        return x ? (char *)x + elems * bytes : nullptr;
      };
      LayerArgs s = bwd_sub_shape(a, pl.rows, pl.heads);
      s.q = at(a.q, bh0 * L * a.d, es); s.k = at(a.k, bh0 * L * a.d, es); s.v = at(a.v, bh0 * L * a.dv, es);
      s.gate = a.gate_mode == 2 ? at(a.gate, h0, es) : at(a.gate, bh0 * L * gtok, es);
      s.wq = at(a.wq, (size_t)h0 * a.d * (a.f / 2), es); s.wk = at(a.wk, (size_t)h0 * a.d * (a.f / 2), es);
      s.meta = (const float *)at(a.meta, (size_t)h0 * a.n_meta, 4);
      s.state_in = (const float *)at(a.state_in, bh0 * a.f * a.dv, 4);
      BwdArgs sg;
      sg.dout = at(g.dout, bh0 * L * a.dv, es);
      sg.dstate_out = (const float *)at(g.dstate_out, bh0 * a.f * a.dv, 4);
      sg.dq = atw(g.dq, bh0 * L * a.d, es); sg.dk = atw(g.dk, bh0 * L * a.d, es);
      sg.dv = atw(g.dv, bh0 * L * a.dv, es);
      sg.dgate = a.gate_mode == 2 ? atw(g.dgate, h0, es) : atw(g.dgate, bh0 * L * gtok, es);
      sg.dwq = (float *)atw(g.dwq, (size_t)h0 * a.d * (a.f / 2), 4);
      sg.dwk = (float *)atw(g.dwk, (size_t)h0 * a.d * (a.f / 2), 4);
      sg.dmeta = (float *)atw(g.dmeta, (size_t)h0 * a.n_meta, 4);
      sg.dstate_in = (float *)atw(g.dstate_in, bh0 * a.f * a.dv, 4);
      const hipError_t e = run(s, sg, b0 > 0);
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace glah

// bwd_walk.hip -- the state sweeps of the gated part's backward in tile form on
// the gfx950 matrix cores (bf16 values, fp32 feature maps and gates from the
// backward prologue, d_v = f = 128).
//
// The gated part ("Lizard" technical summary, gist.science 2507.09025,
// Methodology A.1): S_t = diag(Gamma_t) S_{t-1} + phik_t v_t^T, o_t = S_t^T
// phiq_t.  Its backward needs, per token, dphiq_t = S_t dO_t and, with dS_t the
// gradient reaching S_t (dS_t = phiq_t dO_t^T + diag(Gamma_{t+1}) dS_{t+1}, from
// dS_final), dphik_t = dS_t v_t and dv_t = dS_t^T phik_t.  Over a 16-token tile
// with b_t the inclusive cumsum of a = log Gamma inside the tile and B its
// total, from the state S before the tile and the gradient G reaching the
// state after it (diag(Gamma) dS of the next token, or dS_final):
//   dphiq_t = e^{b_t} (S dO_t) + sum_{s<=t} e^{b_t - b_s} (dO_t . v_s) phik_s
//   dphik_t = e^{B - b_t} (G v_t) + sum_{t'>=t} e^{b_t' - b_t} (dO_t' . v_t) phiq_t'
//   dv_t    = G^T (e^{B - b_t} phik_t) + sum_{t'>=t} A_t't dO_t',
//             A_t't = sum_f phiq_t'[f] phik_t[f] e^{b_t'[f] - b_t[f]}
//   S <- e^{B} S + sum_s (e^{B - b_s} phik_s) v_s^T
//   G <- e^{B} G + sum_t (e^{b_t} phiq_t) dO_t^T.
// Inside a tile the decay between two tokens is split at the tile's middle
// (e^{b_t - b_s} = e^{b_t - m} e^{m - b_s}, m = B / 2), so with the per-token
// log-gate floored at -10 no factor leaves e^{+-80}; every other factor is <= 1.
// Two walks, one wave per block, in one launch:
//   forward walk  (b, h, 16 features): S^T of its features, dphiq and the
//                 64-token tile sums of phiq . dphiq, S_{L-1} . dS_final
//   reverse walk  (b, h, 32 features): G^T of its features, dphik and its tile
//                 sums, the part of dv from these features, dS_in = the state
//                 gradient before the sequence, and Gamma_0 (S_in . dS_0)
// Lane layouts (n = lane & 15, g = lane >> 4) of the 16x16x16 MFMA as in the
// other kernels: A row n, K-slots 4g..4g+3; B column n, K-slots 4g..4g+3;
// accumulator column n, rows 4g..4g+3.  "Layout F" holds element (token 4g + r,
// feature n) of a tile in lane (n, g), slot r (a B operand over tokens);
// "layout T" holds (token n, features 4g + j and 16 + 4g + j) (an operand over
// features, K-slots in the order of two joined 16x16x16 operands).
#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr float kMinLogGate = -10.0f;  // natural log-gate floor (see above)

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ f32x4 zf4() { return (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ float ex(float x) { return exp2_fast(x * kLog2e); }
__device__ __forceinline__ float dot4f(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// In-tile inclusive cumsum over the tokens of layout F (lane (n, g) holds
// tokens 4g .. 4g+3 of feature n): b, the tile total B (in every lane).
__device__ __forceinline__ void cumsum_f(const float *a, float *b, float &B) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  float c0 = a[0], c1 = c0 + a[1], c2 = c1 + a[2], c3 = c2 + a[3];
  const float t0 = __shfl(c3, n), t1 = __shfl(c3, n + 16), t2 = __shfl(c3, n + 32);
  const float pre = (g >= 1 ? t0 : 0.0f) + (g >= 2 ? t1 : 0.0f) + (g >= 3 ? t2 : 0.0f);
  b[0] = pre + c0;
  b[1] = pre + c1;
  b[2] = pre + c2;
  b[3] = pre + c3;
  B = __shfl(b[3], n + 48);
}

// x = hi + lo to about 2^-17 of |x|: two bf16 operands whose products with an
// exact bf16 operand sum (in fp32) to nearly the fp32 product.  The gate
// gradient is a running sum of phiq . dphiq - phik . dphik, differences of
// nearly equal terms, so the products behind dphiq and dphik take the state
// and the decayed maps in this split form.
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
  hi = pack4(x);
  f32x4 h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = (float)hi[r];
  lo = pack4(x - h);
}

// identity as a 16x16x16 B operand
__device__ __forceinline__ bf16x4 eye16() {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  bf16x4 e;
#pragma unroll
  for (int r = 0; r < 4; ++r) e[r] = (bf16)(4 * g + r == n ? 1.0f : 0.0f);
  return e;
}

struct WalkParams {
  const float *pq, *pk, *gam;          // [B H L][128] fp32 (prologue)
  const bf16 *v, *dout;                // [B H][L][128]
  const float *state_in, *dstate_out;  // [B H][128][128] or null
  float *dpq, *dpk, *dvg;              // [N][128], [N][128], [4][N][128]
  float *tq, *tk, *xs, *dstate_in;     // [BH][nft][128] x 2, [2][BH][128], [BH][128][128]
  int BH, L, nft;
};

// ============================== forward walk ================================
__device__ __forceinline__ void fwd_walk(const WalkParams &p, int blk) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int bh = blk >> 3, ft = blk & 7;
  const int f = 16 * ft + n;
  const int L = p.L, ntiles = (L + 15) / 16;
  const size_t rowN = (size_t)bh * L;
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v, bh, L), ro = head_rsrc(p.dout, bh, L);
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  // S^T tiles (s, dt): rows d_v 32 s + 8 g + 4 dt + r, column f
  f32x4 ST[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
      ST[s][dt] = p.state_in ? *(const f32x4 *)(p.state_in + ((size_t)bh * 128 + f) * 128 + 32 * s + 8 * g + 4 * dt)
                             : zf4();
  // operands of a tile (rows of v and dO in the value layout, layout F of the
  // maps and gates), loaded a tile ahead
  bf16x8 xv[4], xo[4];
  float lq[4], lk[4], lg[4];
  auto load = [&](int tau) {
    tau = min(tau, ntiles - 1);
    const unsigned base = (unsigned)(16 * tau + n) * 256;
    load_vals(rv, base, xv);
    load_vals(ro, base, xo);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const size_t i = (rowN + min(16 * tau + 4 * g + r, L - 1)) * 128 + f;
      lq[r] = p.pq[i];
      lk[r] = p.pk[i];
      lg[r] = p.gam[i];
    }
  };
  if (L > 0) load(0);
  float tqa = 0.0f;
  for (int tau = 0; tau < ntiles; ++tau) {
    // this tile's operands, then the next tile's loads
    bf16x8 cv[4], co[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cv[s] = xv[s];
      co[s] = xo[s];
    }
    float a[4], fq[4], fk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool ok = 16 * tau + 4 * g + r < L;  // past the end: no decay, no map
      a[r] = ok ? fmaxf(log2_fast(lg[r]) * kLn2, kMinLogGate) : 0.0f;
      fq[r] = ok ? lq[r] : 0.0f;
      fk[r] = ok ? lk[r] : 0.0f;
    }
    load(tau + 1);
    float b[4], B;
    cumsum_f(a, b, B);
    const float mid = 0.5f * B, eB = ex(B);
    f32x4 eo, kb, ein, kh;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      eo[r] = ex(b[r] - mid);
      kb[r] = fk[r] * ex(mid - b[r]);
      ein[r] = ex(b[r]);
      kh[r] = fk[r] * ex(B - b[r]);
    }
    // M^T (column t, rows s): v_s . dO_t; kept for s <= t it is M in A form
    f32x4 mt = zf4();
#pragma unroll
    for (int s = 0; s < 4; ++s) mt = mfma(cv[s], co[s], mt);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r > n) mt[r] = 0.0f;
    // dphiq: the tile itself and the state before it (split operands)
    bf16x4 mh, ml, kbh, kbl;
    split4(mt, mh, ml);
    split4(kb, kbh, kbl);
    f32x4 dq = mma16(mh, kbh, zf4());
    dq = mma16(mh, kbl, dq);
    dq = mma16(ml, kbh, dq) * eo;
    f32x4 inter = zf4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x4 h0, l0, h1, l1;
      split4(ST[s][0], h0, l0);
      split4(ST[s][1], h1, l1);
      inter = mfma(co[s], join44(h0, h1), inter);
      inter = mfma(co[s], join44(l0, l1), inter);
    }
    dq += inter * ein;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * tau + 4 * g + r;
      if (t < L) p.dpq[(rowN + t) * 128 + f] = dq[r];
      tqa += fq[r] * dq[r];
    }
    if ((tau & 3) == 3 || tau == ntiles - 1) {
      const float ssum = grp_sum(tqa);
      if (g == 0) p.tq[((size_t)bh * p.nft + (tau >> 2)) * 128 + f] = ssum;
      tqa = 0.0f;
    }
    // S^T <- e^{B} S^T + V^T k-hat
    bf16x4 khh, khl;
    split4(kh, khh, khl);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x4 vt = pack4(mfma(cv[s], sel[dt], zf4()));
        ST[s][dt] = mma16(vt, khl, mma16(vt, khh, ST[s][dt] * eB));
      }
  }
  if (p.dstate_out) {
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        acc += dot4f(ST[s][dt], *(const f32x4 *)(p.dstate_out + ((size_t)bh * 128 + f) * 128 + 32 * s + 8 * g + 4 * dt));
    acc = grp_sum(acc);
    if (g == 0) p.xs[(size_t)bh * 128 + f] = acc;
  }
}

// ============================== reverse walk ================================
__device__ __forceinline__ void rev_walk(const WalkParams &p, int blk) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int bh = blk >> 2, fs = blk & 3;
  const int L = p.L, ntiles = (L + 15) / 16;
  const size_t rowN = (size_t)bh * L, N = (size_t)p.BH * L;
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v, bh, L), ro = head_rsrc(p.dout, bh, L);
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  const bf16x4 eye = eye16();
  // features of layout F (fa = 0, 1) and of layout T (two quads)
  const int fF[2] = {32 * fs + n, 32 * fs + 16 + n};
  const int fT[2] = {32 * fs + 4 * g, 32 * fs + 16 + 4 * g};
  // G^T tiles [fa][s][dt]: rows d_v 32 s + 8 g + 4 dt + r, column fF[fa]
  f32x4 GT[2][4][2];
#pragma unroll
  for (int fa = 0; fa < 2; ++fa)
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        GT[fa][s][dt] = p.dstate_out ? *(const f32x4 *)(p.dstate_out + ((size_t)bh * 128 + fF[fa]) * 128 + 32 * s +
                                                        8 * g + 4 * dt)
                                     : zf4();
  bf16x8 xv[4], xo[4];
  float lq[2][4], lk[2][4], lg[2][4];
  f32x4 tq4[2], tk4[2], tg4[2];  // layout T: token 16 tau + n, features fT[h] .. + 3
  auto load = [&](int tau) {
    tau = max(tau, 0);
    const unsigned base = (unsigned)(16 * tau + n) * 256;
    load_vals(rv, base, xv);
    load_vals(ro, base, xo);
#pragma unroll
    for (int fa = 0; fa < 2; ++fa)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const size_t i = (rowN + min(16 * tau + 4 * g + r, L - 1)) * 128 + fF[fa];
        lq[fa][r] = p.pq[i];
        lk[fa][r] = p.pk[i];
        lg[fa][r] = p.gam[i];
      }
    const size_t it = (rowN + min(16 * tau + n, L - 1)) * 128;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      tq4[h] = *(const f32x4 *)(p.pq + it + fT[h]);
      tk4[h] = *(const f32x4 *)(p.pk + it + fT[h]);
      tg4[h] = *(const f32x4 *)(p.gam + it + fT[h]);
    }
  };
  if (L > 0) load(ntiles - 1);
  float tka[2] = {0.0f, 0.0f};
  for (int tau = ntiles - 1; tau >= 0; --tau) {
    bf16x8 cv[4], co[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cv[s] = xv[s];
      co[s] = xo[s];
    }
    // layout F per feature half: log-gates, cumsum, maps
    float bF[2][4], BF[2], fqF[2][4], fkF[2][4];
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      float a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool ok = 16 * tau + 4 * g + r < L;
        a[r] = ok ? fmaxf(log2_fast(lg[fa][r]) * kLn2, kMinLogGate) : 0.0f;
        fqF[fa][r] = ok ? lq[fa][r] : 0.0f;
        fkF[fa][r] = ok ? lk[fa][r] : 0.0f;
      }
      cumsum_f(a, bF[fa], BF[fa]);
    }
    // layout T: cumsum over the tokens of the 16-lane row
    f32x4 qT[2], kT[2], bT[2], BT[2];
    {
      const bool ok = 16 * tau + n < L;
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float a = ok ? fmaxf(log2_fast(tg4[h][j]) * kLn2, kMinLogGate) : 0.0f;
          bT[h][j] = row_scan(a);
          BT[h][j] = row_bcast15(bT[h][j]);
          qT[h][j] = ok ? tq4[h][j] : 0.0f;
          kT[h][j] = ok ? tk4[h][j] : 0.0f;
        }
    }
    load(tau - 1);
    // M (column t, rows t'): dO_t' . v_t; kept for t' >= t it is M^T in A form
    f32x4 mm = zf4();
#pragma unroll
    for (int s = 0; s < 4; ++s) mm = mfma(co[s], cv[s], mm);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < n) mm[r] = 0.0f;
    bf16x4 mmh, mml;
    split4(mm, mmh, mml);
    // dphik per feature half
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      const float mid = 0.5f * BF[fa];
      f32x4 qp, eo, egk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        qp[r] = fqF[fa][r] * ex(bF[fa][r] - mid);
        eo[r] = ex(mid - bF[fa][r]);
        egk[r] = ex(BF[fa] - bF[fa][r]);
      }
      bf16x4 qph, qpl;
      split4(qp, qph, qpl);
      f32x4 dk = mma16(mmh, qph, zf4());
      dk = mma16(mmh, qpl, dk);
      dk = mma16(mml, qph, dk) * eo;
      f32x4 inter = zf4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x4 h0, l0, h1, l1;
        split4(GT[fa][s][0], h0, l0);
        split4(GT[fa][s][1], h1, l1);
        inter = mfma(cv[s], join44(h0, h1), inter);
        inter = mfma(cv[s], join44(l0, l1), inter);
      }
      dk += inter * egk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tau + 4 * g + r;
        if (t < L) p.dpk[(rowN + t) * 128 + fF[fa]] = dk[r];
        tka[fa] += fkF[fa][r] * dk[r];
      }
    }
    if ((tau & 3) == 0) {
#pragma unroll
      for (int fa = 0; fa < 2; ++fa) {
        const float ssum = grp_sum(tka[fa]);
        if (g == 0) p.tk[((size_t)bh * p.nft + (tau >> 2)) * 128 + fF[fa]] = ssum;
        tka[fa] = 0.0f;
      }
    }
    // A (column t, rows t') over this wave's features, kept for t' >= t; and
    // k-hat^T, both over features in layout T
    bf16x4 ab;
    bf16x8 khT;
    {
      f32x4 qp[2], kp[2], kh[2];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float mid = 0.5f * BT[h][j];
          qp[h][j] = qT[h][j] * ex(bT[h][j] - mid);
          kp[h][j] = kT[h][j] * ex(mid - bT[h][j]);
          kh[h][j] = kT[h][j] * ex(BT[h][j] - bT[h][j]);
        }
      f32x4 am = mfma(pack44(qp[0], qp[1]), pack44(kp[0], kp[1]), zf4());
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r < n) am[r] = 0.0f;
      ab = pack4(am);
      khT = pack44(kh[0], kh[1]);
    }
    // dv^T (rows d_v, column t) and the G update, per d_v tile (s, dt)
    f32x4 qb[2];  // e^{b} phiq, layout F
#pragma unroll
    for (int fa = 0; fa < 2; ++fa)
#pragma unroll
      for (int r = 0; r < 4; ++r) qb[fa][r] = fqF[fa][r] * ex(bF[fa][r]);
    bf16x4 qbh[2], qbl[2];
    split4(qb[0], qbh[0], qbl[0]);
    split4(qb[1], qbh[1], qbl[1]);
    const float eB[2] = {ex(BF[0]), ex(BF[1])};
    const int tv = 16 * tau + n;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        // G^T of this d_v tile as an A operand over features (transposed twice
        // on the matrix core: the bf16 values pass unchanged)
        const bf16x4 g0 = pack4(mma16(pack4(GT[0][s][dt]), eye, zf4()));
        const bf16x4 g1 = pack4(mma16(pack4(GT[1][s][dt]), eye, zf4()));
        const bf16x4 ot = pack4(mfma(co[s], sel[dt], zf4()));  // dO^T half: rows d_v, K tokens
        // the two parts in separate accumulators, added on the VALU: a
        // 16x16x16 product accumulating straight onto a 16x16x32 result read
        // stale accumulator rows (the compiler spaces such a mixed pair as if
        // both had one shape)
        const f32x4 dvt = mfma(join44(g0, g1), khT, zf4()) + mma16(ot, ab, zf4());
        if (tv < L) *(f32x4 *)(p.dvg + fs * N * 128 + (rowN + tv) * 128 + 32 * s + 8 * g + 4 * dt) = dvt;
#pragma unroll
        for (int fa = 0; fa < 2; ++fa) GT[fa][s][dt] = mma16(ot, qbl[fa], mma16(ot, qbh[fa], GT[fa][s][dt] * eB[fa]));
      }
  }
  // G after the first tile = Gamma_0 dS_0: the gradient of the initial state,
  // and Gamma_0 (S_in . dS_0) for the gate gradient at token 0
#pragma unroll
  for (int fa = 0; fa < 2; ++fa) {
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const size_t off = ((size_t)bh * 128 + fF[fa]) * 128 + 32 * s + 8 * g + 4 * dt;
        if (p.dstate_in) *(f32x4 *)(p.dstate_in + off) = GT[fa][s][dt];
        if (p.state_in) acc += dot4f(GT[fa][s][dt], *(const f32x4 *)(p.state_in + off));
      }
    acc = grp_sum(acc);
    if (g == 0) p.xs[((size_t)p.BH + bh) * 128 + fF[fa]] = acc;
  }
}

// Both walks in one launch: the reverse walks (4 a head) first, then the
// forward walks (8 a head); one wave each.
__global__ __launch_bounds__(64) void bwd_walk_kernel(WalkParams p) {
  const int nrev = 4 * p.BH;
  if ((int)blockIdx.x < nrev)
    rev_walk(p, (int)blockIdx.x);
  else
    fwd_walk(p, (int)blockIdx.x - nrev);
}

}  // namespace

bool bwd_walk_supported(int f, int dv, bool bf16) { return bf16 && f == 128 && dv == 128; }

hipError_t launch_bwd_walk(const WalkArgs &a, hipStream_t stream) {
  WalkParams p;
  p.pq = a.pq; p.pk = a.pk; p.gam = a.gam; p.v = (const bf16 *)a.v; p.dout = (const bf16 *)a.dout;
  p.state_in = a.state_in; p.dstate_out = a.dstate_out;
  p.dpq = a.dpq; p.dpk = a.dpk; p.dvg = a.dvg; p.tq = a.tq; p.tk = a.tk; p.xs = a.xs; p.dstate_in = a.dstate_in;
  p.BH = a.BH; p.L = a.L; p.nft = a.nft;
  if (p.BH == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_walk_kernel, dim3((unsigned)(12 * p.BH)), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace glah

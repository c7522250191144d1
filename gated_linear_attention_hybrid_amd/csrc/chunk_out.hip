// chunk_out.hip -- output pass of the chunkwise MFMA prefill for gfx950 with
// two waves per 16-token tile (bf16 inputs, fp32 accumulation,
// d = f = d_v = 128, 64-token chunks).
//
// Same method as the kernels in chunked.hip ("Lizard" technical summary,
// gist.science 2507.09025, Methodology C, hardware-aware algorithm; window part
// Methodology A.2): with b the in-chunk inclusive cumsum of the base-2 log-gates,
// a fold reference r per feature (chunk mode: r = B/2; tile mode: r = P_w + T_w/2)
// and q~ = phi_q 2^{b-r}, k~ = phi_k 2^{r-b}:
//   intra  A^T = k~ q~^T (masked causally; cross-tile factors in tile mode)
//   inter  o  += q-bar S,               q-bar = phi_q 2^{b}
//   state  S  <- diag(2^{B}) S + k-hat^T V,  k-hat = phi_k 2^{B-b}
// and the window probabilities are added to A^T so one GEMM with V gives both.
//
// A block of 512 threads runs 8 waves, two per SIMD, so that the dependency and
// issue stalls of one wave are filled by the other's work (a lone wave issues
// vector instructions at about half the rate of two).  Row phase, tile t = w & 3:
//   key wave   (w = 0..3): V^T fragments, u_k = k Wphi_k, log-gates and in-tile
//                          cumsums of the phi+ half, phi(k), k~ and k-hat^T
//   query wave (w = 4..7): raw-k fragments, u_q, log-gates and cumsums of the
//                          phi- half, phi(q), q-bar, window scores and softmax,
//                          intra-chunk scores, weight fragments
// The two halves of the cumsums are swapped through LDS (over the q-bar and
// k-hat^T buffers, which are free at that point of the chunk).  Column phase:
// wave w owns d_v columns [16w, 16w + 16) and the matching 128 x 16 slice of the
// fp32 state, which stays in MFMA accumulators for the whole segment.
//
// Per chunk: B3 (column phase of the previous chunk done) -> phase A -> B1a
// (cumsum halves, tile totals, raw k visible) -> phase B -> B1 (k~ visible) ->
// phase C -> B2 (q-bar, k-hat^T, weights visible).
#include "chunk_common.hpp"

namespace glah {

namespace {

constexpr int kNT8 = 512;

template <bool SWA>
struct Lds8 {
  static constexpr int NKS = SWA ? 3 : 2;                 // k-steps of the (weights x V) GEMM
  static constexpr int WQ = 0;                            // Wphi_q^T frags [4 mt][4 s]
  static constexpr int WK = WQ + 16 * kFrag;              // Wphi_k^T frags [4 mt][4 s]
  static constexpr int RK = WK + 16 * kFrag;              // raw k frags [2 slot][4 tile][4 s]
  static constexpr int VT = RK + (SWA ? 32 * kFrag : 0);  // V^T half frags [slot][4 tile][8 dv tile]
  static constexpr int KT = VT + (SWA ? 2 : 1) * 32 * kHalf;  // k~ frags [4 tile][4 s]
  static constexpr int QB = KT + 16 * kFrag;              // q-bar frags [4 tile][4 s]
  static constexpr int KH = QB + 16 * kFrag;              // k-hat^T frags [8 mt][2 sp]
  static constexpr int W = KH + 16 * kFrag;               // weight frags [4 qt][NKS]
  static constexpr int T = W + 4 * NKS * kFrag;           // tile log-gate totals [4 tile][128]
  static constexpr int BYTES = T + 4 * kF * 4;
  // in-tile cumsums [4 tile][8 slot group][64 lanes][4] (32 KiB) over QB and KH:
  // written after B3, read before B1, while QB and KH hold nothing live
  static constexpr int DD = QB;
};
static_assert(Lds8<true>::DD + 4 * 8 * 64 * 16 <= Lds8<true>::W, "cumsum exchange overlaps the weights");
static_assert(Lds8<true>::BYTES <= 160 * 1024, "LDS budget");

// One chunk's inputs of one wave, prefetched one chunk ahead.
struct Regs8 {
  bf16x8 xa[4];  // key wave: k, query wave: q   [token 16t + n][32g + 8s + j]
  bf16x8 xb[4];  // key wave: v [token][32s + 8g + j]; query wave: raw k [token][32g + 8s + j]
  bf16x8 xg[2];  // gate[token][feat(g, 16h + 8s + j)], h = 0 key wave, 1 query wave
};
enum { L8_A = 1, L8_B = 2, L8_G = 4, L8_ALL = 7 };

template <bool SWA, int PARTS>
__device__ __forceinline__ void load8(const ChunkParams &p, size_t bh, int c, int tile, bool kw, Regs8 &r) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  // rows outside [0, L) come from a clamped valid row; every consumer masks them
  const int t = min(max(c * kC + 16 * tile + n, 0), p.L - 1);
  const size_t row = bh * p.L + t;
  if (PARTS & L8_A) {
    const bf16 *src = (kw ? p.k : p.q) + row * kD + 32 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s) r.xa[s] = *(const bf16x8 *)(src + 8 * s);
  }
  if (PARTS & L8_B) {
    if (kw) {
#pragma unroll
      for (int s = 0; s < 4; ++s) r.xb[s] = *(const bf16x8 *)(p.v + row * kDV + 32 * s + 8 * g);
    } else if (SWA) {
#pragma unroll
      for (int s = 0; s < 4; ++s) r.xb[s] = *(const bf16x8 *)(p.k + row * kD + 32 * g + 8 * s);
    }
  }
  if (PARTS & L8_G) {
    const bf16 *src = p.gate + row * kF + feat(g, kw ? 0 : 16);
#pragma unroll
    for (int s = 0; s < 2; ++s) r.xg[s] = *(const bf16x8 *)(src + 8 * s);
  }
}

// 0/1 selection operand: output column n picks K-slot 16 dt + n, so for a
// token-row operand A (lane = token, K = 32 value dims 32s + k),
// A x select16(dt) is the accumulator tile (row = token 4g + j, column n) of
// value dims 32s + 16dt + n: an exact transpose on the matrix core.
__device__ __forceinline__ bf16x8 select16(int dt) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (bf16)((g == ((16 * dt + n) >> 3) && j == (n & 7)) ? 1.0f : 0.0f);
  return b;
}

// Unnormalised Hedgehog exponentials of the lane's token: e[4mt + j] =
// 2^{(u - max u) log2e} (phi+ feature 16g + 4mt + j) and e[16 + 4mt + j] =
// 2^{(min u - u) log2e} (phi- feature 64 + 16g + 4mt + j), and the reciprocal
// normalisers of the two halves.
__device__ __forceinline__ void hedgehog_exp(const f32x4 *u, float *e, float &izp, float &izn) {
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mx = fmaxf(mx, u[mt][j]);
      mn = fminf(mn, u[mt][j]);
    }
  mx = grp_max(mx) * kLog2e;
  mn = grp_min(mn) * kLog2e;
  float zp = 0.0f, zn = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * mt + j;
      e[i] = exp2_fast(u[mt][j] * kLog2e - mx);
      e[16 + i] = exp2_fast(mn - u[mt][j] * kLog2e);
      zp += e[i];
      zn += e[16 + i];
    }
  izp = rcp_fast(grp_sum(zp));
  izn = rcp_fast(grp_sum(zn));
}

// ---------------------------------------------------------------- the kernel
template <bool SWA>
__global__ __launch_bounds__(kNT8) void chunk_out_kernel(ChunkParams p) {
  using LD = Lds8<SWA>;
  constexpr int NKS = LD::NKS;
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int tile = wave & 3;
  const bool kw = wave < 4;  // key wave (uniform)
  const size_t bh = blockIdx.x / p.P;
  const int seg = blockIdx.x % p.P;
  const int h = (int)(bh % p.H);
  const int c_begin = seg * p.seg_chunks;
  const int c_end = min(c_begin + p.seg_chunks, p.nchunks);

  // ---- Hedgehog projections as MFMA A fragments: frag (mt, s), lane (r, g)
  // holds W[32g + 8s + j][m] with m = 16(r/4) + 4mt + (r%4), so that the
  // accumulator of tile mt gives lane (n, g) the u-values m = 16g + 4mt + j.
  for (int idx = tid; idx < 2 * 16 * 64; idx += kNT8) {
    const int which = idx >> 10, fi = (idx >> 6) & 15, l = idx & 63, rr = l & 15, gg = l >> 4;
    const int mt = fi >> 2, s = fi & 3;
    const int m = 16 * (rr >> 2) + 4 * mt + (rr & 3);
    const bf16 *w = (which ? p.wk : p.wq) + (size_t)h * kD * kF2;
    bf16x8 f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = w[(32 * gg + 8 * s + j) * kF2 + m];
    sts8(smem + (which ? LD::WK : LD::WQ) + fi * kFrag + l * 16, f);
  }

  // ---- state slice: S[mt][j] = S[feat(g, 4mt + j)][16 wave + n]
  f32x4 S[8];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) S[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  {
    const float *src = nullptr;
    if (seg == 0)
      src = p.state_in ? p.state_in + bh * kF * kDV : nullptr;
    else
      src = p.seg_state + (bh * ((p.P - 1) * p.R) + (seg * p.R - 1)) * (size_t)(kF * kDV);
    if (src) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int j = 0; j < 4; ++j) S[mt][j] = src[feat(g, 4 * mt + j) * kDV + 16 * wave + n];
    }
  }
  const bf16x8 selv[2] = {select16(0), select16(1)};
  const bf16x8 selk[2] = {select_operand(0), select_operand(1)};
  // meta-memory sinks of this head, base 2 (query waves)
  float meta_max = -INFINITY, meta_sum = 0.0f;
  if (SWA && !kw) {
    const float *meta = p.meta + (size_t)h * p.n_meta;
    for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, meta[m] * kLog2e);
    for (int m = 0; m < p.n_meta; ++m) meta_sum += exp2_fast(meta[m] * kLog2e - meta_max);
    if (p.n_meta == 0) meta_max = 0.0f;  // meta_sum = 0: no sink mass
  }

  // V^T half fragments (key waves) or raw-k fragments (query waves) of this
  // wave's tile of chunk c into ring slot `slot`
  auto stage = [&](const Regs8 &r, int slot) {
    if (kw) {
      char *base = smem + LD::VT + (slot * 4 + tile) * 8 * kHalf + lane * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const f32x4 t = mfma(r.xb[s], selv[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
          *(bf16x4 *)(base + (2 * s + dt) * kHalf) = pack4(t);
        }
    } else if (SWA) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sts8(smem + LD::RK + ((slot * 4 + tile) * 4 + s) * kFrag + lane * 16, r.xb[s]);
    }
  };

  // ---- window part: keys and values of the chunk before the segment
  if (SWA) {
    Regs8 pr;
    load8<SWA, L8_B>(p, bh, c_begin - 1, tile, kw, pr);
    stage(pr, (c_begin - 1) & 1);
  }

  // ================= column phase of chunk cc: outputs and state =================
  float fdec[2] = {1.0f, 1.0f};  // 2^{B} of the chunk whose column phase is pending
  auto column = [&](int cc) {
    const int c0 = cc * kC;
    const int slot = SWA ? (cc & 1) : 0;
    const int pslot = slot ^ 1;
    f32x4 O[4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) O[qt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    // inter-chunk readout O^T += S^T q-bar^T; the state is decayed right after
    // it is read (S <- diag(2^{B}) S).  The q-bar fragments of k-step s+1 are
    // requested before the MFMAs of step s.
    bf16x8 qf[2][4];
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) qf[0][qt] = lds8(smem + LD::QB + (qt * 4) * kFrag + lane * 16);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (s + 1 < 4) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          qf[(s + 1) & 1][qt] = lds8(smem + LD::QB + (qt * 4 + s + 1) * kFrag + lane * 16);
      }
      issue_fence();
      const bf16x8 a = pack44(S[2 * s], S[2 * s + 1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        S[2 * s][j] *= row_bcast(fdec[j & 1], (8 * s + j) >> 1);
        S[2 * s + 1][j] *= row_bcast(fdec[j & 1], (8 * s + 4 + j) >> 1);
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) O[qt] = mfma(a, qf[s & 1][qt], O[qt]);
    }
    // weights x V over the key tiles of each query tile; the operands of query
    // tile qt+1 are requested before the MFMAs of qt
    auto vt_half = [&](int kt) -> bf16x4 {
      const int sl = kt >= 0 ? slot : pslot;
      const int tl = kt >= 0 ? kt : kt + 4;
      return *(const bf16x4 *)(smem + LD::VT + ((sl * 4 + tl) * 8 + wave) * kHalf + lane * 8);
    };
    bf16x8 wf[2][NKS], vf[2][NKS];
    auto wv_load = [&](int qt, int buf) {
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        wf[buf][ks] = lds8(smem + LD::W + (qt * NKS + ks) * kFrag + lane * 16);
        bf16x4 lo, hi;
        if (SWA) {
          const int ka = qt - 4 + 2 * ks;
          lo = vt_half(ka);
          if (ks < 2) {
            hi = vt_half(ka + 1);
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) hi[j] = (bf16)0.0f;
          }
        } else {
          lo = vt_half(2 * ks);
          hi = vt_half(2 * ks + 1);
        }
        vf[buf][ks] = join44(lo, hi);
      }
    };
    wv_load(0, 0);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      if (qt + 1 < 4) wv_load(qt + 1, (qt + 1) & 1);
      issue_fence();
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) O[qt] = mfma(vf[qt & 1][ks], wf[qt & 1][ks], O[qt]);
    }
    // store o: lane (n, g) of query tile qt holds o[16qt + n][16 wave + 4g + j]
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      const int t = c0 + 16 * qt + n;
      if (t < p.L) *(bf16x4 *)(p.o + (bh * p.L + t) * kDV + 16 * wave + 4 * g) = pack4(O[qt]);
    }
    // S += k-hat^T V, in groups of 4 state tiles; group i+1 requested before the
    // MFMAs of group i
    const char *vb = smem + LD::VT + (slot * 32 + wave) * kHalf + lane * 8;
    const bf16x8 bv[2] = {join44(*(const bf16x4 *)vb, *(const bf16x4 *)(vb + 8 * kHalf)),
                          join44(*(const bf16x4 *)(vb + 16 * kHalf), *(const bf16x4 *)(vb + 24 * kHalf))};
    bf16x8 kf[2][4];
#pragma unroll
    for (int m4 = 0; m4 < 4; ++m4) kf[0][m4] = lds8(smem + LD::KH + (m4 * 2) * kFrag + lane * 16);
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {  // grp = 2 sp + (mt / 4)
      if (grp + 1 < 4) {
        const int sp1 = (grp + 1) >> 1, mb1 = 4 * ((grp + 1) & 1);
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4)
          kf[(grp + 1) & 1][m4] = lds8(smem + LD::KH + ((mb1 + m4) * 2 + sp1) * kFrag + lane * 16);
      }
      issue_fence();
      const int sp = grp >> 1, mb = 4 * (grp & 1);
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) S[mb + m4] = mfma(kf[grp & 1][m4], bv[sp], S[mb + m4]);
    }
  };

  Regs8 cur;
  load8<SWA, L8_ALL>(p, bh, c_begin, tile, kw, cur);
  __syncthreads();

  const float sl2 = p.scale * kLog2e;
  for (int c = c_begin; c <= c_end; ++c) {
    if (c > c_begin) column(c - 1);
    __syncthreads();  // B3: LDS fragments of chunk c-1 consumed
    if (c == c_end) break;
    const int c0 = c * kC;
    const int slot = SWA ? (c & 1) : 0;
    const int pslot = slot ^ 1;
    const int tq = c0 + 16 * tile + n;  // this lane's token in the row phase
    const bool tok_ok = tq < p.L;
    const bool full = c0 + kC <= p.L;  // every token of the chunk exists (uniform)
    const bool more = c + 1 < c_end;
    const int hh = kw ? 0 : 16;  // first fold slot of this wave's log-gate half

    // ================= phase A =================
    stage(cur, slot);
    if (more && kw) load8<SWA, L8_B>(p, bh, c + 1, tile, kw, cur);

    // band scores (query waves): sc[i] for key tile tile-4+i; tiles of the
    // previous chunk and the diagonal now, the others after B1a
    f32x4 sc[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) sc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    auto band = [&](int i) {
      const int kt = tile - 4 + i;
      bf16x8 a[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (i == 4)
          a[s] = cur.xb[s];
        else if (kt >= 0)
          a[s] = lds8(smem + LD::RK + ((slot * 4 + kt) * 4 + s) * kFrag + lane * 16);
        else
          a[s] = lds8(smem + LD::RK + ((pslot * 4 + kt + 4) * 4 + s) * kFrag + lane * 16);
      }
      issue_fence();
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma(a[s], cur.xa[s], acc);
      sc[i] = acc;
    };
    if (SWA && !kw) {
#pragma unroll
      for (int i = 0; i < 5; ++i)
        if (i == 4 || tile - 4 + i < 0) band(i);
      if (more) load8<SWA, L8_B>(p, bh, c + 1, tile, kw, cur);
    }

    // u = x Wphi (16 x 64 per tile)
    f32x4 u[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) u[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    {  // the 4 fragments of tile mt+1 are requested before the MFMAs of tile mt
      const char *wb = smem + (kw ? LD::WK : LD::WQ) + lane * 16;
      bf16x8 wfr[2][4];
#pragma unroll
      for (int s = 0; s < 4; ++s) wfr[0][s] = lds8(wb + s * kFrag);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt + 1 < 4) {
#pragma unroll
          for (int s = 0; s < 4; ++s) wfr[(mt + 1) & 1][s] = lds8(wb + ((mt + 1) * 4 + s) * kFrag);
        }
        issue_fence();
#pragma unroll
        for (int s = 0; s < 4; ++s) u[mt] = mfma(wfr[mt & 1][s], cur.xa[s], u[mt]);
      }
    }
    if (more && kw) load8<SWA, L8_A>(p, bh, c + 1, tile, kw, cur);

    // log-gates of this wave's half (fold slots hh .. hh+15), base 2, floored,
    // zero for tokens past the end; in-tile inclusive cumsum over the 16 tokens
    float dh[16];
    if (p.gate_is_log) {  // one uniform branch around the whole loop
#pragma unroll
      for (int i = 0; i < 16; ++i) dh[i] = (float)cur.xg[i >> 3][i & 7] * kLog2e;
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) dh[i] = log2_sigmoid((float)cur.xg[i >> 3][i & 7]);
    }
    if (more) load8<SWA, L8_G>(p, bh, c + 1, tile, kw, cur);
    if (full) {
#pragma unroll
      for (int i = 0; i < 16; ++i) dh[i] = fmaxf(dh[i], kMinLog2Gate);
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) dh[i] = tok_ok ? fmaxf(dh[i], kMinLog2Gate) : 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dh[i] += row_shr<1>(dh[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) dh[i] += row_shr<2>(dh[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) dh[i] += row_shr<4>(dh[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) dh[i] += row_shr<8>(dh[i]);
    {
      char *xd = smem + LD::DD + tile * 8 * 1024 + lane * 16;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4 *)(xd + ((hh >> 2) + q4) * 1024) =
            (f32x4){dh[4 * q4], dh[4 * q4 + 1], dh[4 * q4 + 2], dh[4 * q4 + 3]};
      if (n == 15) {
        float *T = (float *)(smem + LD::T) + tile * kF;
#pragma unroll
        for (int i = 0; i < 16; ++i) T[feat(g, hh + i)] = dh[i];
      }
    }
    // unnormalised Hedgehog exponentials
    float e[32], izp, izn;
    hedgehog_exp(u, e, izp, izn);
    __syncthreads();  // B1a: cumsum halves, tile totals, raw-k fragments visible

    // ================= phase B =================
    // Fold reference r (base 2, per feature).  Chunk mode: r = B/2 for the whole
    // chunk, so cross-tile factors are 1; used when every feature's chunk total
    // has |B| <= kChunkRefLimit.  Tile mode otherwise: r_w = P_w + T_w/2.
    // Per-tile quantities are computed for features 2n, 2n+1 of the lane's group
    // and broadcast to the row (DPP) where needed.
    float tt[4][2], pre[2], btot[2], tw[2], rr2[2], dd[32];
    bool chunk_mode = true;
    {
      const float *T = (const float *)(smem + LD::T);
      const int f0 = feat(g, 2 * n);
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float2 v2 = *(const float2 *)(T + w2 * kF + f0);
        tt[w2][0] = v2.x;
        tt[w2][1] = v2.y;
      }
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        pre[e2] = 0.0f;
        btot[e2] = 0.0f;
        tw[e2] = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          btot[e2] += tt[w2][e2];
          if (w2 < tile) pre[e2] += tt[w2][e2];
          if (w2 == tile) tw[e2] = tt[w2][e2];
        }
      }
      // every wave sees all 128 features, so the vote is the same in all waves
      chunk_mode = __all(fabsf(btot[0]) <= kChunkRefLimit && fabsf(btot[1]) <= kChunkRefLimit);
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        rr2[e2] = chunk_mode ? 0.5f * btot[e2] : pre[e2] + 0.5f * tw[e2];
        fdec[e2] = exp2_fast(btot[e2]);
      }
      // the other wave's cumsum half
      const char *xd = smem + LD::DD + tile * 8 * 1024 + lane * 16;
      float oth[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v4 = *(const f32x4 *)(xd + ((4 - (hh >> 2)) + q4) * 1024);
#pragma unroll
        for (int j = 0; j < 4; ++j) oth[4 * q4 + j] = v4[j];
      }
      if (kw) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dd[i] = dh[i];
          dd[16 + i] = oth[i];
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          dd[i] = oth[i];
          dd[16 + i] = dh[i];
        }
      }
      float off[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) off[e2] = pre[e2] - rr2[e2];  // b_chunk - r = b_loc + off
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_bcast(off[i & 1], i >> 1);
    }

    bf16x8 xr[4];  // key wave: k~; query wave: q~ (MFMA operands, token rows)
    bf16x8 xs[4];  // key wave: k-hat; query wave: q-bar
    {
      // key: k~ = phi_k 2^{-(b - r)}, k-hat = k~ 2^{B - r}
      // query: q~ = phi_q 2^{b - r}, q-bar = q~ 2^{r}
      float fs[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) fs[e2] = exp2_fast(kw ? btot[e2] - rr2[e2] : rr2[e2]);
      const float sgn = kw ? -1.0f : 1.0f;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        float a8[8], b8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * s + j;
          a8[j] = e[i] * (i < 16 ? izp : izn) * exp2_fast(sgn * dd[i]);
          b8[j] = a8[j] * row_bcast(fs[j & 1], i >> 1);
        }
        xr[s] = pack8(a8);
        xs[s] = pack8(b8);
      }
    }
    if (kw) {
      if (!full && !tok_ok) {  // keys past the end contribute nothing
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          xr[s] = zero8();
          xs[s] = zero8();
        }
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::KT + (tile * 4 + s) * kFrag + lane * 16, xr[s]);
    }

    // window: remaining band scores, masks, one-shot softmax with the sinks
    f32x4 Wt[5];  // weights^T for key tiles tile-4+i (i = 4: the diagonal tile)
#pragma unroll
    for (int i = 0; i < 5; ++i) Wt[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
    if (SWA && !kw) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tile - 4 + i >= 0) band(i);
      // key position minus query position: 16(i-4) + 4g + j - n; valid when in
      // (-window, 0] and the key exists (position >= 0)
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rel = 16 * (i - 4) + 4 * g + j - n;
          const bool ok = rel <= 0 && rel > -p.window && tq + rel >= 0;
          sc[i][j] = ok ? sc[i][j] * sl2 : -INFINITY;
          mx = fmaxf(mx, sc[i][j]);
        }
      mx = grp_max(mx);
      mx = fmaxf(mx, meta_max);
      float sum = 0.0f;
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float ex = exp2_fast(sc[i][j] - mx);  // 2^{-inf} = 0
          sc[i][j] = ex;
          sum += ex;
        }
      sum = grp_sum(sum);
      sum += meta_sum * exp2_fast(meta_max - mx);  // sum_m 2^{t_m log2e - mx}
      const float inv = rcp_fast(sum);
#pragma unroll
      for (int i = 0; i < 5; ++i) Wt[i] = sc[i] * inv;
    }
    if (more && !kw) load8<SWA, L8_A>(p, bh, c + 1, tile, kw, cur);
    __syncthreads();  // B1: k~ fragments visible, cumsum exchange consumed

    // ================= phase C =================
    if (kw) {
      // k-hat^T fragments: state tile mt takes its 16 features from K-step
      // s(mt) = 2(mt/4) + (mt%4)/2 of the token-row operand, transposed on the
      // matrix core
      const int sp = tile >> 1, hf = tile & 1;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const int s2 = 2 * (mt >> 2) + ((mt & 3) >> 1);
        const f32x4 t = mfma(xs[s2], selk[mt & 1], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
        *(bf16x4 *)(smem + LD::KH + (mt * 2 + sp) * kFrag + lane * 16 + hf * 8) = pack4(t);
      }
    } else {
      // intra-chunk scores A^T for key tiles kt = tile-4+i, i = 1..4, kt >= 0
      {  // diagonal tile: both sides share the reference
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
          acc = mfma(lds8(smem + LD::KT + (tile * 4 + s) * kFrag + lane * 16), xr[s], acc);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (4 * g + j > n) acc[j] = 0.0f;  // causal: key after query
        Wt[4] += acc;
      }
      // earlier tiles: in chunk mode both sides share the reference; in tile mode
      // q~ is scaled by 2^{r_w - r_kt} <= 1 with r_x = P_x + T_x/2
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        const int kt = tile - 4 + i;
        if (kt >= 0 && chunk_mode) {
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s)
            acc = mfma(lds8(smem + LD::KT + (kt * 4 + s) * kFrag + lane * 16), xr[s], acc);
          Wt[i] += acc;
        } else if (kt >= 0) {
          float fo[2];
#pragma unroll
          for (int e2 = 0; e2 < 2; ++e2) {
            float run = 0.0f, tk = 0.0f;  // log-gate sum of tiles kt .. tile-1
#pragma unroll
            for (int w2 = 0; w2 < 4; ++w2) {
              if (w2 >= kt && w2 < tile) run += tt[w2][e2];
              if (w2 == kt) tk = tt[w2][e2];
            }
            fo[e2] = exp2_fast(run + 0.5f * (tw[e2] - tk));
          }
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            float tmp[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) tmp[j] = (float)xr[s][j] * row_bcast(fo[j & 1], (8 * s + j) >> 1);
            acc = mfma(lds8(smem + LD::KT + (kt * 4 + s) * kFrag + lane * 16), pack8(tmp), acc);
          }
          Wt[i] += acc;
        }
      }
      // weight fragments for the (weights x V) GEMM
      if (SWA) {
        sts8(smem + LD::W + (tile * NKS + 0) * kFrag + lane * 16, pack44(Wt[0], Wt[1]));
        sts8(smem + LD::W + (tile * NKS + 1) * kFrag + lane * 16, pack44(Wt[2], Wt[3]));
        sts8(smem + LD::W + (tile * NKS + 2) * kFrag + lane * 16,
             pack44(Wt[4], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}));
      } else {
        // absolute key tiles 0..3 of the chunk: tile kt is Wt[kt - tile + 4]
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 w0 = z, w1 = z, w2 = z, w3 = z;
        switch (tile) {
          case 0: w0 = Wt[4]; break;
          case 1: w0 = Wt[3]; w1 = Wt[4]; break;
          case 2: w0 = Wt[2]; w1 = Wt[3]; w2 = Wt[4]; break;
          default: w0 = Wt[1]; w1 = Wt[2]; w2 = Wt[3]; w3 = Wt[4]; break;
        }
        sts8(smem + LD::W + (tile * NKS + 0) * kFrag + lane * 16, pack44(w0, w1));
        sts8(smem + LD::W + (tile * NKS + 1) * kFrag + lane * 16, pack44(w2, w3));
      }
      // q-bar fragments (inter-chunk readout)
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::QB + (tile * 4 + s) * kFrag + lane * 16, xs[s]);
    }
    __syncthreads();  // B2: q-bar, k-hat^T, weight fragments visible
  }

  // ---- epilogue
  if (p.state_out && seg == p.P - 1) {
    float *dst = p.state_out + bh * kF * kDV;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + 16 * wave + n] = S[mt][j];
  }
}

template <bool SWA>
hipError_t launch8(const ChunkParams &p, int blocks, hipStream_t stream) {
  const int bytes = Lds8<SWA>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void *)chunk_out_kernel<SWA>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_out_kernel<SWA>, dim3((unsigned)blocks), dim3(kNT8), bytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_out(const ChunkParams &p, bool swa, int blocks, hipStream_t stream) {
  return swa ? launch8<true>(p, blocks, stream) : launch8<false>(p, blocks, stream);
}

}  // namespace glah

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
// A block of 512 threads runs 8 waves, two per SIMD, so that the stalls of one
// wave are filled by the other's work (a lone wave issues vector instructions at
// about half the rate of two).  Tile t = w & 3:
//   key wave   (w = 0..3): holds d_v columns [32t, 32t + 32) of the fp32 state in
//                          MFMA accumulators and runs the column phase (readout,
//                          weights x V, state update) of the previous chunk; then
//                          u_k = k Wphi_k, the log-gates of its tile, phi(k), k~,
//                          k-hat^T and V^T fragments
//   query wave (w = 4..7): raw-k fragments, window scores and softmax, u_q,
//                          phi(q), q~, q-bar, intra-chunk scores, weight
//                          fragments; and the log-gates of the NEXT chunk, whose
//                          tile totals it publishes one chunk ahead, so every
//                          wave knows the chunk-wide fold reference when a chunk
//                          starts
// Per chunk there are two barriers: B1 (raw-k and k~ fragments visible, column
// phase of the previous chunk done) and B2 (q-bar, k-hat^T, V^T and weights
// visible).
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
  // per query tile: window part 2 full fragments + the diagonal tile as a half
  // fragment (its upper K half is zero); no window: 2 full fragments
  static constexpr int WQT = SWA ? 2 * kFrag + kHalf : 2 * kFrag;
  static constexpr int T = W + 4 * WQT;                   // tile decay totals (-log2-gate sums) [2 slot][4 tile][128]
  static constexpr int BYTES = T + 2 * 4 * kF * 4;
};
static_assert(Lds8<true>::BYTES <= 160 * 1024, "LDS budget");

// Per-feature chunk quantities for features 2n, 2n+1 of the lane's group from
// the tile totals of the chunk (base 2): fold reference rr2, offset off = P_w - r
// of this wave's tile, total B, and the per-tile totals tt (tile mode).
struct FoldRef {
  float tt[4][2], tw[2], btot[2], rr2[2], off[2];
  bool chunk_mode;
};
__device__ __forceinline__ FoldRef fold_ref(const float *T, int tile) {
  FoldRef r;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int f0 = feat(g, 2 * n);
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const float2 v2 = *(const float2 *)(T + w2 * kF + f0);  // decay exponents: totals are -T
    r.tt[w2][0] = -v2.x;
    r.tt[w2][1] = -v2.y;
  }
  float pre[2];
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    pre[e2] = 0.0f;
    r.btot[e2] = 0.0f;
    r.tw[e2] = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < 4; ++w2) {
      r.btot[e2] += r.tt[w2][e2];
      if (w2 < tile) pre[e2] += r.tt[w2][e2];
      if (w2 == tile) r.tw[e2] = r.tt[w2][e2];
    }
  }
  // Chunk mode: r = B/2 for the whole chunk, so cross-tile factors are 1; used
  // when every feature's chunk total has |B| <= kChunkRefLimit.  Tile mode
  // otherwise: r_w = P_w + T_w/2.  Every wave sees all 128 features, so the vote
  // is the same in all waves.
  r.chunk_mode = __all(fabsf(r.btot[0]) <= kChunkRefLimit && fabsf(r.btot[1]) <= kChunkRefLimit);
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) {
    r.rr2[e2] = r.chunk_mode ? 0.5f * r.btot[e2] : pre[e2] + 0.5f * r.tw[e2];
    r.off[e2] = pre[e2] - r.rr2[e2];  // b_chunk - r = b_loc + off
  }
  return r;
}

// Folded feature operands: xr = phi 2^{sgn (b - r)} (k~ with sgn = -1, q~ with
// sgn = +1) and xs = xr 2^{fs} (per feature: k-hat with fs = B - r, q-bar with
// fs = r), as MFMA token-row operands (slot i = 8s + j).
__device__ __forceinline__ void fold(const float *e, float izp, float izn, const float *dn, const FoldRef &r,
                                     float sgn, const float *fs, bf16x8 *xr, bf16x8 *xs) {
  float fsx[2];
#pragma unroll
  for (int e2 = 0; e2 < 2; ++e2) fsx[e2] = exp2_fast(fs[e2]);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    float a8[8], b8[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = 8 * s + j;
      const float d = row_bcast(r.off[i & 1], i >> 1) - dn[i];  // b - r
      a8[j] = e[i] * (i < 16 ? izp : izn) * exp2_fast(sgn * d);
      b8[j] = a8[j] * row_bcast(fsx[i & 1], i >> 1);
    }
    xr[s] = pack8(a8);
    xs[s] = pack8(b8);
  }
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
  const bool gate_is_log = p.gate_is_log != 0;

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
  // The column phase of the chunk before the segment runs on zero operands (its
  // outputs are not stored), so the loop needs no first-iteration branch.  The
  // window part's V^T slot of that chunk is staged below.
  for (int off = LD::KT + tid * 16; off < LD::T; off += kNT8 * 16) sts8(smem + off, zero8());
  for (int off = LD::VT + tid * 16; off < LD::KT; off += kNT8 * 16) sts8(smem + off, zero8());
  __syncthreads();  // zero fill before the staged fragments below

  if (kw) {
    // =============================== key waves ===============================
    const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
    // state slice: S[mt][dt][j] = S[feat(g, 4mt + j)][dvcol(tile, dt, n)]
    f32x4 S[8][2];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) S[mt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
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
          for (int dt = 0; dt < 2; ++dt)
#pragma unroll
            for (int j = 0; j < 4; ++j) S[mt][dt][j] = src[feat(g, 4 * mt + j) * kDV + dvcol(tile, dt, n)];
      }
    }
    // V^T half fragments of token tile `tile` into ring slot `slot`: for d_v tile
    // (2w' + dt), lane 16g + r holds v[16 tile + 4g + j][dvcol(w', dt, r)]
    auto stage_vt = [&](const bf16x8 *xv, int slot) {
      char *base = smem + LD::VT + (slot * 4 + tile) * 8 * kHalf + lane * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f32x4 t2[2];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) t2[dt] = mfma(xv[s], sel[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) *(bf16x4 *)(base + (2 * s + dt) * kHalf) = pack4(t2[dt]);
      }
    };
    const HeadBufs hb = head_bufs(p, bh);
    const unsigned ro = row_off(tile);
    bf16x8 xk[4], xv[4], xg[4];  // this chunk's keys, values, gates
    if (SWA) {  // values of the chunk before the segment (window part)
      load_vals(hb.v, ro + chunk_off(c_begin - 1), xv);
      stage_vt(xv, (c_begin - 1) & 1);
    }
    load_rows(hb.k, ro + chunk_off(c_begin), xk);
    load_vals(hb.v, ro + chunk_off(c_begin), xv);
    load_gates(hb.g, ro + chunk_off(c_begin), xg);
    float fdec[2] = {1.0f, 1.0f};  // 2^{B} of the chunk whose column phase is pending
    __syncthreads();               // staged fragments and the first chunk's totals

    // column phase of chunk cc: outputs and state
    auto column = [&](int cc) {
      const int c0 = cc * kC;
      const int slot = SWA ? (cc & 1) : 0;
      const int pslot = slot ^ 1;
      f32x4 O[4][2];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) O[qt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      // inter-chunk readout O^T += S^T q-bar^T; the state is decayed right after
      // it is read (S <- diag(2^{B}) S).  The 4 q-bar fragments of a k-step are
      // requested together.
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 qf[4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) qf[qt] = lds8(smem + LD::QB + (qt * 4 + s) * kFrag + lane * 16);
        issue_fence();
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const bf16x8 a = pack44(S[2 * s][dt], S[2 * s + 1][dt]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            S[2 * s][dt][j] *= row_bcast(fdec[j & 1], (8 * s + j) >> 1);
            S[2 * s + 1][dt][j] *= row_bcast(fdec[j & 1], (8 * s + 4 + j) >> 1);
          }
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) O[qt][dt] = mfma(a, qf[qt], O[qt][dt]);
        }
      }
      // weights x V over the key tiles of each query tile
      auto vt_half = [&](int kt, int dt) -> bf16x4 {
        const int sl = kt >= 0 ? slot : pslot;
        const int tl = kt >= 0 ? kt : kt + 4;
        return *(const bf16x4 *)(smem + LD::VT + ((sl * 4 + tl) * 8 + 2 * tile + dt) * kHalf + lane * 8);
      };
      const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        bf16x8 wf[NKS], vf[NKS][2];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const char *wb = smem + LD::W + qt * LD::WQT + ks * kFrag;
          if (SWA && ks == 2)
            wf[ks] = join44(*(const bf16x4 *)(wb + lane * 8), z4);
          else
            wf[ks] = lds8(wb + lane * 16);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            bf16x4 lo, hi;
            if (SWA) {
              const int ka = qt - 4 + 2 * ks;
              lo = vt_half(ka, dt);
              hi = ks < 2 ? vt_half(ka + 1, dt) : z4;
            } else {
              lo = vt_half(2 * ks, dt);
              hi = vt_half(2 * ks + 1, dt);
            }
            vf[ks][dt] = join44(lo, hi);
          }
        }
        issue_fence();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) O[qt][dt] = mfma(vf[ks][dt], wf[ks], O[qt][dt]);
      }
      // store o: lane (n, g) of query tile qt holds d_v 32 tile + 8g + (4dt + j);
      // rows past the end are dropped by the range check
      if (cc >= c_begin) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, pack44(O[qt][0], O[qt][1])), hb.o,
              (int)(chunk_off(cc) + (unsigned)(16 * qt + n) * (kDV * 2) + 64 * tile + 16 * g), 0, 0);
      }
      // S += k-hat^T V in groups of 4 state tiles (fragments of a group requested
      // together)
      bf16x8 bv[2][2];
#pragma unroll
      for (int sp = 0; sp < 2; ++sp)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const char *vb = smem + LD::VT + ((slot * 4 + 2 * sp) * 8 + 2 * tile + dt) * kHalf + lane * 8;
          bv[sp][dt] = join44(*(const bf16x4 *)vb, *(const bf16x4 *)(vb + 8 * kHalf));
        }
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {  // grp = 2 sp + (mt / 4)
        const int sp = grp >> 1, mb = 4 * (grp & 1);
        bf16x8 kf[4];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) kf[m4] = lds8(smem + LD::KH + ((mb + m4) * 2 + sp) * kFrag + lane * 16);
        issue_fence();
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) S[mb + m4][dt] = mfma(kf[m4], bv[sp][dt], S[mb + m4][dt]);
      }
    };

    for (int c = c_begin; c < c_end; ++c) {
      const int slot = SWA ? (c & 1) : 0;
      const int tq = c * kC + 16 * tile + n;
      const bool tok_ok = tq < p.L;
      const unsigned ro1 = ro + chunk_off(c + 1);
      // ---- phase A: previous chunk's column phase, then this tile's keys
      column(c - 1);
      f32x4 u[4];
      project(smem + LD::WK + lane * 16, xk, u);
      load_rows(hb.k, ro1, xk);  // next chunk's keys
      float dd[32];
      tile_decay(xg, gate_is_log, tok_ok, dd);
      load_gates(hb.g, ro1, xg);
      float e[32], izp, izn;
      hedgehog_exp(u, e, izp, izn);
      const FoldRef r = fold_ref((const float *)(smem + LD::T) + (c & 1) * 4 * kF, tile);
      bf16x8 xr[4], xs[4];  // k~ (intra scores), k-hat (state update)
      float fs[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        fs[e2] = r.btot[e2] - r.rr2[e2];
        fdec[e2] = exp2_fast(r.btot[e2]);
      }
      // Keys past the end need no masking: their k~ meets only queries past the
      // end (causal mask), whose outputs are not stored, and their k-hat meets
      // value rows that read as zero (range check).
      fold(e, izp, izn, dd, r, -1.0f, fs, xr, xs);
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::KT + (tile * 4 + s) * kFrag + lane * 16, xr[s]);
      __syncthreads();  // B1: raw-k and k~ fragments visible; column phase done

      // ---- phase C: V^T and k-hat^T fragments of this tile
      stage_vt(xv, slot);
      load_vals(hb.v, ro1, xv);  // next chunk's values
      {  // state tile mt takes its 16 features from K-step s(mt) = 2(mt/4) + (mt%4)/2
         // of the token-row operand, transposed on the matrix core
        const int sp = tile >> 1, hf = tile & 1;
#pragma unroll
        for (int m2 = 0; m2 < 4; ++m2) {
          f32x4 t2[2];
#pragma unroll
          for (int d2 = 0; d2 < 2; ++d2) {
            const int mt = 2 * m2 + d2;
            const int s2 = 2 * (mt >> 2) + ((mt & 3) >> 1);
            t2[d2] = mfma(xs[s2], sel[mt & 1], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
          }
#pragma unroll
          for (int d2 = 0; d2 < 2; ++d2)
            *(bf16x4 *)(smem + LD::KH + ((2 * m2 + d2) * 2 + sp) * kFrag + lane * 16 + hf * 8) = pack4(t2[d2]);
        }
      }
      __syncthreads();  // B2: q-bar, k-hat^T, V^T, weight fragments visible
    }
    column(c_end - 1);
    if (p.state_out && seg == p.P - 1) {
      float *dst = p.state_out + bh * kF * kDV;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvcol(tile, dt, n)] = S[mt][dt][j];
    }
  } else {
    // ============================== query waves ==============================
    // meta-memory sinks of this head, base 2
    float meta_max = -INFINITY, meta_sum = 0.0f;
    if (SWA) {
      const float *meta = p.meta + (size_t)h * p.n_meta;
      for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, meta[m] * kLog2e);
      for (int m = 0; m < p.n_meta; ++m) meta_sum += exp2_fast(meta[m] * kLog2e - meta_max);
      if (p.n_meta == 0) meta_max = 0.0f;  // meta_sum = 0: no sink mass
      // wave-uniform: keep them in scalar registers
      meta_max = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, meta_max)));
      meta_sum = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, meta_sum)));
    }
    auto stage_rk = [&](const bf16x8 *xk, int slot) {
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::RK + ((slot * 4 + tile) * 4 + s) * kFrag + lane * 16, xk[s]);
    };
    // q and raw keys of this chunk, gates of the next
    bf16x8 xq[4], xb[4], xg[4];
    const HeadBufs hb = head_bufs(p, bh);
    const unsigned ro = row_off(tile);
    if (SWA) {  // keys of the chunk before the segment (window part)
      load_rows(hb.k, ro + chunk_off(c_begin - 1), xb);
      stage_rk(xb, (c_begin - 1) & 1);
    }
    float dd[32];  // decay exponents (-cumsums, tile_decay) of the chunk being processed
    {
      load_rows(hb.q, ro + chunk_off(c_begin), xq);
      if (SWA) load_rows(hb.k, ro + chunk_off(c_begin), xb);
      load_gates(hb.g, ro + chunk_off(c_begin), xg);
      tile_decay(xg, gate_is_log, c_begin * kC + 16 * tile + n < p.L, dd);
      if (n == 15) {  // tile totals of the first chunk
        float *T = (float *)(smem + LD::T) + ((c_begin & 1) * 4 + tile) * kF;
#pragma unroll
        for (int i = 0; i < 32; ++i) T[feat(g, i)] = dd[i];
      }
      load_gates(hb.g, ro + chunk_off(c_begin + 1), xg);
    }
    const float sl2 =
        __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.scale * kLog2e)));
    __syncthreads();  // staged fragments and the first chunk's totals

    for (int c = c_begin; c < c_end; ++c) {
      const int slot = SWA ? (c & 1) : 0;
      const int pslot = slot ^ 1;
      const int tq = c * kC + 16 * tile + n;
      const unsigned ro1 = ro + chunk_off(c + 1);
      // ---- phase A
      // band scores sc[i] for key tile tile-4+i: tiles of the previous chunk and
      // the diagonal at the end of this phase (their keys are in LDS: the own
      // tile's were staged by this wave), the others after B1
      f32x4 sc[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) sc[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      auto band = [&](int i) {
        const int kt = tile - 4 + i;
        bf16x8 a[4];
        issue_fence();  // keep the loads next to their MFMAs
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          if (kt >= 0)
            a[s] = lds8(smem + LD::RK + ((slot * 4 + kt) * 4 + s) * kFrag + lane * 16);
          else
            a[s] = lds8(smem + LD::RK + ((pslot * 4 + kt + 4) * 4 + s) * kFrag + lane * 16);
        }
        issue_fence();
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma(a[s], xq[s], acc);
        sc[i] = acc;
      };
      if (SWA) stage_rk(xb, slot);
      f32x4 u[4];
      project(smem + LD::WQ + lane * 16, xq, u);
      float e[32], izp, izn;
      hedgehog_exp(u, e, izp, izn);
      bf16x8 xr[4], xs[4];  // q~ (intra scores), q-bar (readout)
      bool chunk_mode;
      {
        const FoldRef r = fold_ref((const float *)(smem + LD::T) + (c & 1) * 4 * kF, tile);
        fold(e, izp, izn, dd, r, 1.0f, r.rr2, xr, xs);
        chunk_mode = r.chunk_mode;
      }
      // cumsums and tile totals of the next chunk, published one chunk ahead
      tile_decay(xg, gate_is_log, tq + kC < p.L, dd);
      load_gates(hb.g, ro + chunk_off(c + 2), xg);
      if (n == 15) {
        float *T = (float *)(smem + LD::T) + (((c + 1) & 1) * 4 + tile) * kF;
#pragma unroll
        for (int i = 0; i < 32; ++i) T[feat(g, i)] = dd[i];
      }
      if (SWA) {
#pragma unroll
        for (int i = 0; i < 5; ++i)
          if (i == 4 || tile - 4 + i < 0) band(i);
      }
      __syncthreads();  // B1: raw-k and k~ fragments visible; column phase done

      // ---- phase C
      f32x4 Wt[5];  // weights^T for key tiles tile-4+i (i = 4: the diagonal tile)
#pragma unroll
      for (int i = 0; i < 5; ++i) Wt[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      if (SWA) {
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
      // intra-chunk scores A^T for key tiles kt = tile-4+i, i = 1..4, kt >= 0
      {
        auto kt_frags = [&](int kt, bf16x8 *kf) {
          issue_fence();  // keep the loads next to their MFMAs
#pragma unroll
          for (int s = 0; s < 4; ++s) kf[s] = lds8(smem + LD::KT + (kt * 4 + s) * kFrag + lane * 16);
          issue_fence();
        };
        {  // diagonal tile: both sides share the reference
          bf16x8 kf[4];
          kt_frags(tile, kf);
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma(kf[s], xr[s], acc);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * g + j > n) acc[j] = 0.0f;  // causal: key after query
          Wt[4] += acc;
        }
        // earlier tiles: in chunk mode both sides share the reference; in tile
        // mode q~ is scaled by 2^{r_w - r_kt} <= 1 with r_x = P_x + T_x/2
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          const int kt = tile - 4 + i;
          if (kt >= 0 && chunk_mode) {
            bf16x8 kf[4];
            kt_frags(kt, kf);
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = mfma(kf[s], xr[s], acc);
            Wt[i] += acc;
          } else if (kt >= 0) {
            bf16x8 kf[4];
            kt_frags(kt, kf);
            // tile totals of this chunk again (the slot is rewritten only in the
            // next chunk's phase A)
            const float *T = (const float *)(smem + LD::T) + (c & 1) * 4 * kF + feat(g, 2 * n);
            float fo[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              float run = 0.0f, tk = 0.0f, tw = 0.0f;  // log-gate sum of tiles kt .. tile-1
#pragma unroll
              for (int w2 = 0; w2 < 4; ++w2) {
                const float tv = -T[w2 * kF + e2];
                if (w2 >= kt && w2 < tile) run += tv;
                if (w2 == kt) tk = tv;
                if (w2 == tile) tw = tv;
              }
              fo[e2] = exp2_fast(run + 0.5f * (tw - tk));
            }
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              float tmp[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) tmp[j] = (float)xr[s][j] * row_bcast(fo[j & 1], (8 * s + j) >> 1);
              acc = mfma(kf[s], pack8(tmp), acc);
            }
            Wt[i] += acc;
          }
        }
      }
      // weight fragments for the (weights x V) GEMM
      char *wq = smem + LD::W + tile * LD::WQT;
      if (SWA) {
        sts8(wq + lane * 16, pack44(Wt[0], Wt[1]));
        sts8(wq + kFrag + lane * 16, pack44(Wt[2], Wt[3]));
        *(bf16x4 *)(wq + 2 * kFrag + lane * 8) = pack4(Wt[4]);
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
        sts8(wq + lane * 16, pack44(w0, w1));
        sts8(wq + kFrag + lane * 16, pack44(w2, w3));
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::QB + (tile * 4 + s) * kFrag + lane * 16, xs[s]);
      // next chunk's queries and raw keys; their first use waits out the key
      // waves' longer phase A
      load_rows(hb.q, ro1, xq);
      if (SWA) load_rows(hb.k, ro1, xb);
      __syncthreads();  // B2: q-bar, k-hat^T, V^T, weight fragments visible
    }
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

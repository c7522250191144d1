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
// A block of 512 threads runs 8 waves, two per SIMD (waves w and w + 4 share
// one), so that the stalls of one wave are filled by the other's work (a lone
// wave issues vector instructions at about half the rate of two).  Tile t = w & 3:
//   key wave   (w = 0..3): holds d_v columns dvpair(t, 0..1, 0..15) of the fp32
//                          state in MFMA accumulators and runs the column phase
//                          (readout, weights x V, state update) of the previous
//                          chunk, with the value operands read straight from
//                          memory; then u_k = k Wphi_k, phi(k), k~ and the
//                          k-hat^T fragments; and, in the second phase, the gate
//                          decay exponents of every feature of its tile of the
//                          NEXT chunk
//   query wave (w = 4..7): first phase: u_q, phi(q), q~, q-bar, the scores of
//                          all five window bands and the softmax with the sinks
//                          (the raw keys of a chunk are staged one chunk ahead);
//                          second phase: the next chunk's raw keys, the
//                          intra-chunk scores and the weight fragments
// The decay exponents are shared through LDS, so each is computed once and
// every wave knows the chunk-wide fold reference when a chunk starts.
// Per chunk there are two barriers: B1 (k~ fragments visible, column phase of
// the previous chunk and every read of the decay exponents and of the previous
// chunk's raw keys done) and B2 (q-bar, k-hat^T, weights, the next chunk's raw
// keys and decay exponents visible).
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
  static constexpr int DD = RK + (SWA ? 32 * kFrag : 0);  // decay exponents (fp32) [4 tile][8 q][64 lane][4]
  static constexpr int KT = DD + 32 * kFrag;              // k~ frags [4 tile][4 s]
  static constexpr int QB = KT + 16 * kFrag;              // q-bar frags [4 tile][4 s]
  static constexpr int KH = QB + 16 * kFrag;              // k-hat^T frags [8 mt][2 sp]
  static constexpr int W = KH + 16 * kFrag;               // weight frags [4 qt][NKS]
  // per query tile: window part 2 full fragments + the diagonal tile as a half
  // fragment (its upper K half is zero); no window: 2 full fragments
  static constexpr int WQT = SWA ? 2 * kFrag + kHalf : 2 * kFrag;
  static constexpr int BYTES = W + 4 * WQT;
};
static_assert(Lds8<true>::BYTES <= 160 * 1024, "LDS budget");

// An empty use of x: the value is computed before this point (the scheduler may
// otherwise sink pure arithmetic past a barrier).  Emits no instruction.
template <typename T>
__device__ __forceinline__ void pin(const T &x) { asm volatile("" ::"v"(x)); }

// Decay exponents (tile_decay) of the chunk, exchanged through LDS: tile t,
// lane l, fold slots 4q .. 4q+3 at ((t * 8 + q) * 64 + l) * 16 bytes.
__device__ __forceinline__ void store_dd(char *dd, int tile, const float *dn) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int q = 0; q < 8; ++q)
    *(f32x4 *)(dd + ((tile * 8 + q) * 64 + lane) * 16) =
        (f32x4){dn[4 * q], dn[4 * q + 1], dn[4 * q + 2], dn[4 * q + 3]};
}
__device__ __forceinline__ void load_dd(const char *dd, int tile, float *dn) {
  const int lane = threadIdx.x & 63;
  f32x4 v[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) v[q] = *(const f32x4 *)(dd + ((tile * 8 + q) * 64 + lane) * 16);
#pragma unroll
  for (int q = 0; q < 8; ++q)
#pragma unroll
    for (int j = 0; j < 4; ++j) dn[4 * q + j] = v[q][j];
}

// Per-feature chunk quantities for features 2n, 2n+1 of the lane's group from
// the tile totals of the chunk (base 2): fold reference rr2, offset off = P_w - r
// of this wave's tile, total B, and the per-tile totals tt (tile mode).  A
// tile's totals are the decay exponents of its last token (lane 16g + 15).
struct FoldRef {
  float tt[4][2], tw[2], btot[2], rr2[2], off[2];
  bool chunk_mode;
};
__device__ __forceinline__ FoldRef fold_ref(const char *dd, int tile) {
  FoldRef r;
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
#pragma unroll
  for (int w2 = 0; w2 < 4; ++w2) {
    const float2 v2 = *(const float2 *)(dd + ((w2 * 8 + (n >> 1)) * 64 + 16 * g + 15) * 16 + (n & 1) * 8);
    r.tt[w2][0] = -v2.x;  // log2-gate totals are minus the decay totals
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
template <bool SWA, bool SG>
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
  for (int off = LD::KT + tid * 16; off < LD::BYTES; off += kNT8 * 16) sts8(smem + off, zero8());
  __syncthreads();  // zero fill before the staged fragments below

  if (kw) {
    // =============================== key waves ===============================
    const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
    // state slice: S[mt][dt][j] = S[feat(g, 4mt + j)][dvpair(tile, dt, n)]
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
            for (int j = 0; j < 4; ++j) S[mt][dt][j] = src[feat(g, 4 * mt + j) * kDV + dvpair(tile, dt, n)];
      }
    }
    const HeadBufs hb = head_bufs(p, bh);
    const unsigned ro = row_off(tile);
    // Values as MFMA operands, read straight from memory: for the 16 d_v columns
    // of column tile dt (dvpair(tile, dt, n)) and K-steps over two token tiles
    // (a, b), lane (n, g) needs v[16a + 4g + j][.] and v[16b + 4g + j][.],
    // j = 0..3.  One dword per token row holds both column tiles (adjacent
    // columns 32 tile + 2n, + 1); vt[T][2 dt + h] packs tokens 4g + 2h, 4g + 2h + 1
    // of tile T for column tile dt.
    uint32_t vraw[4][4];                 // dwords of the chunk being loaded
    uint32_t vcur[4][4], vprev[4][4];    // packed: the column phase's chunk and the one before
    auto load_v = [&](int cc) {
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          vraw[T][j] = __builtin_amdgcn_raw_buffer_load_b32(
              hb.v, (int)(chunk_off(cc) + (unsigned)(16 * T + 4 * g + j) * (kDV * 2) + 64 * tile + 4 * n), 0, 0);
    };
    auto pack_v = [&]() {
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          vcur[T][h] = __builtin_amdgcn_perm(vraw[T][2 * h + 1], vraw[T][2 * h], 0x05040100u);      // low halves
          vcur[T][2 + h] = __builtin_amdgcn_perm(vraw[T][2 * h + 1], vraw[T][2 * h], 0x07060302u);  // high halves
        }
    };
    // operand of column tile dt over token tiles (a, b) of the current (a, b >= 0)
    // or previous (a, b < 0) chunk; b > 3 gives zeros
    auto vop = [&](int a, int b, int dt) -> bf16x8 {
      const uint32_t *ta = a >= 0 ? vcur[a] : vprev[a + 4];
      u32x4 r;
      r[0] = ta[2 * dt];
      r[1] = ta[2 * dt + 1];
      if (b > 3) {
        r[2] = 0u;
        r[3] = 0u;
      } else {
        const uint32_t *tb = b >= 0 ? vcur[b] : vprev[b + 4];
        r[2] = tb[2 * dt];
        r[3] = tb[2 * dt + 1];
      }
      return __builtin_bit_cast(bf16x8, r);
    };
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) vcur[T][j] = 0u;
    load_v(c_begin - 1);  // the chunk before the segment (window part); zeros before token 0
    // The decay exponents of a chunk are computed one chunk ahead, in phase C
    // (the key waves wait for the query waves there)
    bf16x8 xk[4], xg[4];  // this chunk's keys, the next chunk's gates
    load_rows(hb.k, ro + chunk_off(c_begin), xk);
    load_gates<SG>(hb, ro + chunk_off(c_begin), xg);
    {
      float dn[32];
      tile_decay<32>(xg, gate_is_log, c_begin * kC + 16 * tile + n < p.L, dn);
      store_dd(smem + LD::DD, tile, dn);
    }
    float fdec[2] = {1.0f, 1.0f};  // 2^{B} of the chunk whose column phase is pending
    __syncthreads();               // staged fragments and the first chunk's decay exponents

    // column phase of chunk cc: outputs and state
    auto column = [&](int cc) {
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
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        bf16x8 wf[NKS];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const char *wb = smem + LD::W + qt * LD::WQT + ks * kFrag;
          if (SWA && ks == 2)
            wf[ks] = join44(*(const bf16x4 *)(wb + lane * 8), (bf16x4){(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f});
          else
            wf[ks] = lds8(wb + lane * 16);
        }
        issue_fence();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            // key tiles (qt - 4 + 2ks, qt - 3 + 2ks) with the window, (2ks, 2ks + 1)
            // without; the diagonal tile's step has no second tile
            const int a = SWA ? qt - 4 + 2 * ks : 2 * ks;
            const int b = SWA && ks == 2 ? 4 : a + 1;
            O[qt][dt] = mfma(vop(a, b, dt), wf[ks], O[qt][dt]);
          }
      }
      // store o: lane (n, g) of query tile qt holds d_v 32 tile + 8g + 2j + dt;
      // rows past the end are dropped by the range check
      if (cc >= c_begin) {
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          bf16x8 ov;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            ov[2 * j] = (bf16)O[qt][0][j];
            ov[2 * j + 1] = (bf16)O[qt][1][j];
          }
          __builtin_amdgcn_raw_buffer_store_b128(
              __builtin_bit_cast(u32x4, ov), hb.o,
              (int)(chunk_off(cc) + (unsigned)(16 * qt + n) * (kDV * 2) + 64 * tile + 16 * g), 0, 0);
        }
      }
      // S += k-hat^T V in groups of 4 state tiles (fragments of a group requested
      // together)
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
          for (int dt = 0; dt < 2; ++dt) S[mb + m4][dt] = mfma(kf[m4], vop(2 * sp, 2 * sp + 1, dt), S[mb + m4][dt]);
      }
    };

    for (int c = c_begin; c < c_end; ++c) {
      const int tq = c * kC + 16 * tile + n;
      const unsigned ro1 = ro + chunk_off(c + 1);
      // ---- phase A: previous chunk's column phase, then this tile's keys
#pragma unroll
      for (int T = 0; T < 4; ++T)
#pragma unroll
        for (int j = 0; j < 4; ++j) vprev[T][j] = vcur[T][j];
      pack_v();  // values of chunk c - 1
      column(c - 1);
      load_gates<SG>(hb, ro1, xg);  // next chunk's gates (decay exponents in phase C)
      f32x4 u[4];
      project(smem + LD::WK + lane * 16, xk, u);
      load_rows(hb.k, ro1, xk);  // next chunk's keys
      float e[32], izp, izn;
      hedgehog_exp(u, e, izp, izn);
      const FoldRef r = fold_ref(smem + LD::DD, tile);
      bf16x8 xr[4], xs[4];  // k~ (intra scores), k-hat (state update)
      float fs[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        fs[e2] = r.btot[e2] - r.rr2[e2];
        fdec[e2] = exp2_fast(r.btot[e2]);
      }
      {
        float dn[32];
        load_dd(smem + LD::DD, tile, dn);
        // Keys past the end need no masking: their k~ meets only queries past the
        // end (causal mask), whose outputs are not stored, and their k-hat meets
        // value rows that read as zero (range check).
        fold(e, izp, izn, dn, r, -1.0f, fs, xr, xs);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) sts8(smem + LD::KT + (tile * 4 + s) * kFrag + lane * 16, xr[s]);
      __syncthreads();  // B1: k~ fragments visible; column phase, decay and raw-key reads done

      // ---- phase C: k-hat^T fragments of this tile, values of this chunk for
      // the next column phase, decay exponents of the next chunk
      load_v(c);
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
      {
        float dn[32];
        tile_decay<32>(xg, gate_is_log, tq + kC < p.L, dn);
        store_dd(smem + LD::DD, tile, dn);
      }
      __syncthreads();  // B2: q-bar, k-hat^T, weights, raw keys and decay exponents visible
    }
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j) vprev[T][j] = vcur[T][j];
    pack_v();
    column(c_end - 1);
    if (p.state_out && seg == p.P - 1) {
      float *dst = p.state_out + bh * kF * kDV;
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvpair(tile, dt, n)] = S[mt][dt][j];
    }
    if (p.kc && seg == p.P - 1) {
      // the ring of the last `window` keys and values for decoding: slot
      // t % window holds token t of [L - window, L), zeros for tokens before 0
      // (16-byte pieces, 16 a row; the key waves are threads 0..255)
      const int w = p.window, L = p.L;
      const bf16x8 z8 = {};
      for (int i = threadIdx.x; i < w * 32; i += 256) {
        const int slot = i >> 5, part = i & 31, piece = part & 15;
        const int t = L - w + ((slot - (L - w)) % w + w) % w;
        const bf16 *src = (part < 16 ? p.k : p.v) + (bh * (size_t)L + (size_t)max(t, 0)) * kD + 8 * piece;
        bf16 *dst = (part < 16 ? p.kc : p.vc) + (bh * (size_t)w + slot) * kD + 8 * piece;
        *(bf16x8 *)dst = t >= 0 ? *(const bf16x8 *)src : z8;
      }
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
    // q and raw keys: the raw keys of a chunk are staged one chunk ahead (in the
    // previous chunk's phase C), so every band of a chunk is scored in its
    // phase A; the key waves compute the gate decay exponents, one chunk ahead
    bf16x8 xq[4], xb[4];
    const HeadBufs hb = head_bufs(p, bh);
    const unsigned ro = row_off(tile);
    if (SWA) {  // keys of the chunk before the segment and of its first chunk
      load_rows(hb.k, ro + chunk_off(c_begin - 1), xb);
      stage_rk(xb, (c_begin - 1) & 1);
      load_rows(hb.k, ro + chunk_off(c_begin), xb);
      stage_rk(xb, c_begin & 1);
    }
    load_rows(hb.q, ro + chunk_off(c_begin), xq);
    const float sl2 =
        __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, p.scale * kLog2e)));
    __syncthreads();  // staged fragments and the first chunk's decay exponents

    for (int c = c_begin; c < c_end; ++c) {
      const int slot = SWA ? (c & 1) : 0;
      const int pslot = slot ^ 1;
      const unsigned ro1 = ro + chunk_off(c + 1);
      // ---- phase A
      if (SWA) load_rows(hb.k, ro1, xb);  // next chunk's raw keys, staged in phase C
      f32x4 u[4];
      project(smem + LD::WQ + lane * 16, xq, u);
      float e[32], izp, izn;
      hedgehog_exp(u, e, izp, izn);
      bf16x8 xr[4], xs[4];  // q~ (intra scores), q-bar (readout)
      const FoldRef r = fold_ref(smem + LD::DD, tile);
      {
        float dn[32];
        load_dd(smem + LD::DD, tile, dn);
        fold(e, izp, izn, dn, r, 1.0f, r.rr2, xr, xs);
      }
      const bool chunk_mode = r.chunk_mode;
      f32x4 Wt[5];  // weights^T for key tiles tile-4+i (i = 4: the diagonal tile)
#pragma unroll
      for (int i = 0; i < 5; ++i) Wt[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      if (SWA) {
        // band scores sc[i] for key tile tile-4+i: tiles of the previous chunk
        // (slot pslot) and of this one (slot slot), all staged before this chunk
        f32x4 sc[5];
#pragma unroll
        for (int i = 0; i < 5; ++i) {
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
        }
        // query position minus key position: 16(4-i) - j - (4g - n); valid when in
        // [0, window) (one unsigned compare) and the key exists: its position
        // 64c + 16(tile + i - 4) + 4g + j is >= 0 exactly when c > 0 or
        // tile + i >= 4 (uniform per key tile)
        const unsigned uw = (unsigned)p.window;
#pragma unroll
        for (int i = 0; i < 5; ++i) {
          const bool exists = c > 0 || tile + i >= 4;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const unsigned back = (unsigned)(16 * (4 - i) - j - (4 * g - n));
            sc[i][j] = (back < uw && exists) ? sc[i][j] : -INFINITY;
          }
        }
        // softmax with the sinks, base 2: the scale is positive, so the row
        // maximum is taken on the raw scores and scaled once
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 5; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) mx = fmaxf(mx, sc[i][j]);
        mx = fmaxf(grp_max(mx) * sl2, meta_max);
        float sum = 0.0f;
#pragma unroll
        for (int i = 0; i < 5; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float ex = exp2_fast(fmaf(sc[i][j], sl2, -mx));  // 2^{-inf} = 0
            sc[i][j] = ex;
            sum += ex;
          }
        sum = grp_sum(sum);
        sum += meta_sum * exp2_fast(meta_max - mx);  // sum_m 2^{t_m log2e - mx}
        const float inv = rcp_fast(sum);
#pragma unroll
        for (int i = 0; i < 5; ++i) Wt[i] = sc[i] * inv;
      }
      // the folds and the window softmax belong to this phase: without these
      // uses the scheduler sinks them past the barrier, into the longer phase
#pragma unroll
      for (int i = 0; i < 5; ++i) pin(Wt[i]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        pin(xr[s]);
        pin(xs[s]);
      }
      __syncthreads();  // B1: k~ fragments visible; column phase, decay and raw-key reads done

      // ---- phase C
      // the next chunk's raw keys go to the slot of the previous chunk, whose
      // bands were all scored before B1
      if (SWA) stage_rk(xb, pslot);
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
            float fo[2];
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
              float run = 0.0f, tk = 0.0f, tw = 0.0f;  // log2-gate sum of tiles kt .. tile-1
#pragma unroll
              for (int w2 = 0; w2 < 4; ++w2) {  // unrolled: no dynamic register indexing
                const float tv = r.tt[w2][e2];
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
      load_rows(hb.q, ro1, xq);  // next chunk's queries
      __syncthreads();  // B2: q-bar, k-hat^T, weights, raw keys and decay exponents visible
    }
  }
}

template <bool SWA, bool SG>
hipError_t launch8(const ChunkParams &p, int blocks, hipStream_t stream) {
  const int bytes = Lds8<SWA>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void *)chunk_out_kernel<SWA, SG>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_out_kernel<SWA, SG>), dim3((unsigned)blocks), dim3(kNT8), bytes, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_out(const ChunkParams &p, bool swa, int blocks, hipStream_t stream) {
  if (p.gate_mode != 0)
    return swa ? launch8<true, true>(p, blocks, stream) : launch8<false, true>(p, blocks, stream);
  return swa ? launch8<true, false>(p, blocks, stream) : launch8<false, false>(p, blocks, stream);
}

}  // namespace glah

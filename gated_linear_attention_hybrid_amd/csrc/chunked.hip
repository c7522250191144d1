// chunked.hip -- chunkwise-parallel MFMA prefill of the hybrid layer for gfx950
// (bf16 inputs, fp32 accumulation, d = f = d_v = 128, 64-token chunks).
//
// Method ("Lizard" technical summary, gist.science 2507.09025, Methodology C,
// hardware-aware algorithm): the Hedgehog features are non-negative, so the
// cumulative log-gates can be moved into phi(q) and phi(k) and every product
// inside a chunk becomes a plain low-precision GEMM instead of a cumulative
// product that underflows.  With b_t the in-chunk inclusive cumsum of
// a = log Gamma (per feature):
//   intra:  A[t][s] = sum_f phi_q[t,f] e^{b_t,f - r_f} * phi_k[s,f] e^{r_f - b_s,f}
//   inter:  o_t    += (phi_q[t] e^{b_t}) S_c
//   state:  S_{c+1} = diag(e^{B_c}) S_c + sum_s (phi_k[s] e^{B_c - b_s})^T v_s
// The reference r is taken per 16-token tile, in the middle of the tile's decay
// (r_w = P_w + T_w/2 with P_w the log-gate sum of the earlier tiles and T_w the
// tile's own), so every exponent stays inside the fp32/bf16 range even when the
// gate product over a whole chunk underflows; cross-tile factors
// e^{r_qt - r_kt} <= 1, and q-bar / k-hat are formed from summed exponents that
// are never positive.
// The window part (Methodology A.2) reuses the same tiles: band scores over the
// 5 key tiles that can reach a 16-query tile, a one-shot softmax whose
// denominator starts from the meta-memory sinks, and the probabilities are added
// to the intra-chunk weights so one GEMM with V yields both parts.
//
// Parallel structure over one head: the sequence is cut into P segments.
//   chunk_kernel<MODE_STATE>   each segment's end state from a zero state and its
//                              total log-decay (segments 0..P-2)
//   segment_scan_kernel        start state of every segment (fp32, sequential in p)
//   chunk_kernel<MODE_HYBRID>  (or MODE_GLA) the outputs, one block per segment,
//                              starting from that segment's state
//   chunk_kernel<MODE_SWA>     window attention alone, one block per chunk
//
// Block = 256 threads = 4 waves.  Row phase: wave w owns query/key tile w (16
// tokens).  Column phase: wave w owns d_v columns [32w, 32w+32) for all 64
// tokens and the matching 128 x 32 slice of the fp32 state, which stays in
// MFMA accumulators for the whole segment.  Operands are exchanged through LDS
// as ready-made MFMA fragments (1 KiB: 64 lanes x 16 B).
#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kNT = 256;    // threads per block

// ---------------------------------------------------------------- LDS layout
template <int MODE>
struct Lds {
  static constexpr bool Q = MODE != MODE_STATE;
  static constexpr bool GLA = MODE != MODE_SWA;
  static constexpr bool SWA = MODE == MODE_HYBRID || MODE == MODE_SWA;
  static constexpr int VSLOTS = SWA ? 2 : 1;
  static constexpr int NKS = SWA ? 3 : 2;  // k-steps of the (weights x V) GEMM
  static constexpr int WQ = 0;                                   // Wphi_q^T frags [4][4]
  static constexpr int WK = WQ + ((Q && GLA) ? 16 * kFrag : 0);  // Wphi_k^T frags [4][4]
  static constexpr int RK = WK + (GLA ? 16 * kFrag : 0);         // raw k frags [2][4][4]
  static constexpr int VT = RK + (SWA ? 32 * kFrag : 0);         // V^T half frags [slot][4][8]
  static constexpr int KT = VT + VSLOTS * 32 * kHalf;            // k-tilde frags [4][4]
  static constexpr int QB = KT + ((Q && GLA) ? 16 * kFrag : 0);  // q-bar frags [4][4]
  static constexpr int KH = QB + ((Q && GLA) ? 16 * kFrag : 0);  // k-hat^T frags [8][2]
  static constexpr int W = KH + (GLA ? 16 * kFrag : 0);          // weight frags [4][NKS]
  static constexpr int T = W + (Q ? 4 * NKS * kFrag : 0);        // tile log-gate totals [4][128]
  static constexpr int BYTES = T + (GLA ? 4 * kF * 4 : 0);
};

// One chunk's inputs held in registers (prefetched one chunk ahead).
struct ChunkRegs {
  bf16x8 xq[4];  // q[token 16w+n][32g + 8s + j]
  bf16x8 xk[4];  // k, same layout
  bf16x8 xg[4];  // gate[token][feat(g, 8s + j)]
  bf16x8 xv[4];  // v[token 16w+n][32s + 8g + j]
};

// Parts of a chunk's inputs, loaded separately so that each part of the next
// chunk can be requested as soon as this chunk's copy has been consumed.
enum { LOAD_V = 1, LOAD_QK = 2, LOAD_G = 4, LOAD_ALL = 7 };

template <int MODE, int PARTS>
__device__ __forceinline__ void load_chunk(const ChunkParams &p, size_t bh, int c, ChunkRegs &r) {
  constexpr bool Q = Lds<MODE>::Q, GLA = Lds<MODE>::GLA, SWA = Lds<MODE>::SWA;
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  // Rows outside [0, L) are read from a clamped, valid row instead of being
  // zero-filled: every consumer masks such tokens (gates and keys of tokens >= L,
  // window keys before 0, outputs not stored), and unconditional loads let the
  // prefetch stay in flight (a conditional zero-fill would have to wait for it).
  const int t = min(max(c * kC + 16 * wave + n, 0), p.L - 1);
  const size_t row = bh * p.L + t;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (Q && (PARTS & LOAD_QK)) r.xq[s] = *(const bf16x8 *)(p.q + row * kD + 32 * g + 8 * s);
    if ((GLA || SWA) && (PARTS & LOAD_QK)) r.xk[s] = *(const bf16x8 *)(p.k + row * kD + 32 * g + 8 * s);
    if (GLA && (PARTS & LOAD_G)) r.xg[s] = *(const bf16x8 *)(p.gate + row * kF + feat(g, 8 * s));
    if (PARTS & LOAD_V) r.xv[s] = *(const bf16x8 *)(p.v + row * kDV + 32 * s + 8 * g);
  }
}

// V^T half fragments of this wave's 16 tokens into ring slot `slot`: for d_v
// tile (2w' + dt), lane 16g + r holds v[16*wave + 4g + j][dvcol(w', dt, r)].
// K-step s of xv covers d_v [32s, 32s+32), i.e. the two d_v tiles of w' = s.
template <int MODE>
__device__ __forceinline__ void store_vt(char *smem, int slot, const ChunkRegs &r, const bf16x8 *sel) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  char *base = smem + Lds<MODE>::VT + (slot * 4 + wave) * 8 * kHalf + lane * 8;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(r.xv[s], sel[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f},
                                                            0, 0, 0);
      *(bf16x4 *)(base + (2 * s + dt) * kHalf) = pack4(t);
    }
}

// ---------------------------------------------------------------- the kernel
template <int MODE>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(MODE == MODE_STATE ? 2 : 1, MODE == MODE_STATE ? 2 : 1)))
void chunk_kernel(ChunkParams p) {
  using LD = Lds<MODE>;
  constexpr bool Q = LD::Q, GLA = LD::GLA, SWA = LD::SWA;
  constexpr bool INTRA = Q && GLA;
  constexpr int NKS = LD::NKS;
  extern __shared__ __align__(16) char smem[];

  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int NS = (p.P - 1) * p.R;
  const int nseg = MODE == MODE_STATE ? NS : p.P;
  const size_t bh = blockIdx.x / nseg;
  const int seg = blockIdx.x % nseg;  // state slice (state pass) or segment
  const int h = (int)(bh % p.H);
  int c_begin, c_end;
  if (MODE == MODE_STATE) {
    const int ps = seg / p.R, r = seg % p.R;
    const int seg_end = min((ps + 1) * p.seg_chunks, p.nchunks);
    c_begin = min(ps * p.seg_chunks + r * p.sub_chunks, seg_end);
    c_end = min(c_begin + p.sub_chunks, seg_end);  // may be empty: zero state, zero decay
  } else {
    c_begin = seg * p.seg_chunks;
    c_end = min(c_begin + p.seg_chunks, p.nchunks);
  }

  // ---- Hedgehog projections as MFMA A fragments: frag (mt, s), lane (r, g)
  // holds W[32g + 8s + j][m] with m = 16(r/4) + 4mt + (r%4), so that the
  // accumulator of tile mt gives lane (n, g) the u-values m = 16g + 4mt + j.
  if (GLA) {
    for (int idx = tid; idx < 16 * 64; idx += kNT) {
      const int fi = idx >> 6, l = idx & 63, rr = l & 15, gg = l >> 4;
      const int mt = fi >> 2, s = fi & 3;
      const int m = 16 * (rr >> 2) + 4 * mt + (rr & 3);
      const bf16 *wk = p.wk + (size_t)h * kD * kF2;
      bf16x8 fk;
#pragma unroll
      for (int j = 0; j < 8; ++j) fk[j] = wk[(32 * gg + 8 * s + j) * kF2 + m];
      sts8(smem + LD::WK + fi * kFrag + l * 16, fk);
      if (Q) {
        const bf16 *wq = p.wq + (size_t)h * kD * kF2;
        bf16x8 fq;
#pragma unroll
        for (int j = 0; j < 8; ++j) fq[j] = wq[(32 * gg + 8 * s + j) * kF2 + m];
        sts8(smem + LD::WQ + fi * kFrag + l * 16, fq);
      }
    }
  }

  // ---- state slice: S[mt][dt][j] = S[feat(g, 4mt + j)][dvcol(wave, dt, n)]
  f32x4 S[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) S[mt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  if (GLA && MODE != MODE_STATE) {
    const float *src = nullptr;
    if (seg == 0)
      src = p.state_in ? p.state_in + bh * kF * kDV : nullptr;
    else
      src = p.seg_state + (bh * NS + (seg * p.R - 1)) * (size_t)(kF * kDV);
    if (src) {
#pragma unroll
      for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            S[mt][dt][j] = src[feat(g, 4 * mt + j) * kDV + dvcol(wave, dt, n)];
    }
  }
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  // meta-memory sinks of this head, base 2: max_m t_m log2e and
  // sum_m 2^{t_m log2e - max}, so a query's denominator needs one power of two
  float meta_max = -INFINITY, meta_sum = 0.0f;
  if (SWA) {
    const float *meta = p.meta + (size_t)h * p.n_meta;
    for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, meta[m] * kLog2e);
    for (int m = 0; m < p.n_meta; ++m) meta_sum += exp2_fast(meta[m] * kLog2e - meta_max);
    if (p.n_meta == 0) meta_max = 0.0f;  // meta_sum = 0: no sink mass
  }
  // total base-2 log-decay of the segment (state pass): features 2n and 2n+1
  float dsum2[2] = {0.0f, 0.0f};

  // ---- window part: keys and values of the chunk before the segment
  if (SWA) {
    ChunkRegs pr;
    load_chunk<MODE, LOAD_ALL>(p, bh, c_begin - 1, pr);
    const int slot = (c_begin - 1) & 1;
    store_vt<MODE>(smem, slot, pr, sel);
#pragma unroll
    for (int s = 0; s < 4; ++s)
      sts8(smem + LD::RK + ((slot * 4 + wave) * 4 + s) * kFrag + lane * 16, pr.xk[s]);
  }

  // ================= column phase of chunk cc: outputs and state =================
  // Runs while the next chunk's inputs are in flight (software pipelining).
  float fdec[2] = {1.0f, 1.0f};  // 2^{B} of the chunk whose column phase is pending
  auto column = [&](int cc) {
    const int c0 = cc * kC;
    const int slot = LD::VSLOTS == 2 ? (cc & 1) : 0;
    const int pslot = slot ^ 1;
    if (Q) {
      f32x4 O[4][2];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) O[qt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      if (GLA) {  // inter-chunk readout: O^T += S^T q-bar^T; the state is decayed
                  // (S <- diag(2^{B}) S) right after it is read for the readout
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const bf16x8 a = pack44(S[2 * s][dt], S[2 * s + 1][dt]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              S[2 * s][dt][j] *= row_bcast(fdec[j & 1], (8 * s + j) >> 1);
              S[2 * s + 1][dt][j] *= row_bcast(fdec[j & 1], (8 * s + 4 + j) >> 1);
            }
#pragma unroll
            for (int qt = 0; qt < 4; ++qt)
              O[qt][dt] = mfma(a, lds8(smem + LD::QB + (qt * 4 + s) * kFrag + lane * 16), O[qt][dt]);
          }
      }
      // weights x V over the key tiles of each query tile
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
          const bf16x8 b = lds8(smem + LD::W + (qt * NKS + ks) * kFrag + lane * 16);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            bf16x4 lo, hi;
            auto vt_half = [&](int kt) -> bf16x4 {
              const int sl = kt >= 0 ? slot : pslot;
              const int tile = kt >= 0 ? kt : kt + 4;
              return *(const bf16x4 *)(smem + LD::VT + (sl * 4 + tile) * 8 * kHalf +
                                       (2 * wave + dt) * kHalf + lane * 8);
            };
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
            O[qt][dt] = mfma(join44(lo, hi), b, O[qt][dt]);
          }
        }
      // store o: lane (n, g) of query tile qt holds d_v 32w + 8g + (4dt + j)
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int t = c0 + 16 * qt + n;
        if (t < p.L)
          *(bf16x8 *)(p.o + (bh * p.L + t) * kDV + 32 * wave + 8 * g) = pack44(O[qt][0], O[qt][1]);
      }
    }

    if (GLA) {  // S <- diag(2^{B}) S + k-hat^T V (the decay is already applied in the
                // readout when there are queries)
      if (!Q) {
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int i = 4 * mt + j;
            const float eb = row_bcast(fdec[i & 1], i >> 1);
            S[mt][0][j] *= eb;
            S[mt][1][j] *= eb;
          }
      }
#pragma unroll
      for (int sp = 0; sp < 2; ++sp) {
        bf16x8 bv[2];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const char *vb = smem + LD::VT + slot * 32 * kHalf + (2 * wave + dt) * kHalf + lane * 8;
          bv[dt] = join44(*(const bf16x4 *)(vb + (2 * sp) * 8 * kHalf),
                          *(const bf16x4 *)(vb + (2 * sp + 1) * 8 * kHalf));
        }
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const bf16x8 a = lds8(smem + LD::KH + (mt * 2 + sp) * kFrag + lane * 16);
          S[mt][0] = mfma(a, bv[0], S[mt][0]);
          S[mt][1] = mfma(a, bv[1], S[mt][1]);
        }
      }
    }
  };

  ChunkRegs cur;
  load_chunk<MODE, LOAD_ALL>(p, bh, c_begin, cur);
  __syncthreads();

  for (int c = c_begin; c <= c_end; ++c) {
    if (c > c_begin) column(c - 1);
    __syncthreads();  // B3: LDS fragments of chunk c-1 consumed
    if (c == c_end) break;
    const int c0 = c * kC;
    const int slot = LD::VSLOTS == 2 ? (c & 1) : 0;
    const int pslot = slot ^ 1;
    const int tq = c0 + 16 * wave + n;  // this lane's token in the row phase
    const bool tok_ok = tq < p.L;
    const bool full = c0 + kC <= p.L;  // every token of the chunk exists (uniform)

    const bool more = c + 1 < c_end;
    store_vt<MODE>(smem, slot, cur, sel);
    if (more) load_chunk<MODE, LOAD_V>(p, bh, c + 1, cur);
    f32x4 Wt[5];  // weights^T for key tiles wave-4+i, i = 0..4 (i = 4: the diagonal tile)
#pragma unroll
    for (int i = 0; i < 5; ++i) Wt[i] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

    if (SWA) {
#pragma unroll
      for (int s = 0; s < 4; ++s)
        sts8(smem + LD::RK + ((slot * 4 + wave) * 4 + s) * kFrag + lane * 16, cur.xk[s]);
      __syncthreads();  // B0: raw-k fragments of this chunk visible
      // band scores for key tiles wave-4 .. wave, one-shot softmax with sinks
      f32x4 sc[5];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int kt = wave - 4 + i;
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          bf16x8 a;
          if (i == 4)
            a = cur.xk[s];
          else if (kt >= 0)
            a = lds8(smem + LD::RK + ((slot * 4 + kt) * 4 + s) * kFrag + lane * 16);
          else
            a = lds8(smem + LD::RK + ((pslot * 4 + kt + 4) * 4 + s) * kFrag + lane * 16);
          acc = mfma(a, cur.xq[s], acc);
        }
        sc[i] = acc;
      }
      // key position minus query position: 16(i-4) + 4g + j - n; valid when in
      // (-window, 0] and the key exists (position >= 0)
      const float sl2 = p.scale * kLog2e;
      const int qpos = c0 + 16 * wave + n;
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rel = 16 * (i - 4) + 4 * g + j - n;
          const bool ok = rel <= 0 && rel > -p.window && qpos + rel >= 0;
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
          const float e = exp2_fast(sc[i][j] - mx);  // 2^{-inf} = 0
          sc[i][j] = e;
          sum += e;
        }
      sum = grp_sum(sum);
      sum += meta_sum * exp2_fast(meta_max - mx);  // sum_m 2^{t_m log2e - mx}
      const float inv = rcp_fast(sum);
#pragma unroll
      for (int i = 0; i < 5; ++i) Wt[i] = sc[i] * inv;
      if (!GLA && more) load_chunk<MODE, LOAD_QK>(p, bh, c + 1, cur);
    }

    // ================= row phase 1: features, gates, folds =================
    // For the 32 features F_g of this lane's token (fold slot i):
    //   d_i = b_i - T_i/2  (base 2; b: in-tile inclusive log-gate cumsum, T: tile total)
    //   q~ = phi_q 2^{d},  k~ = phi_k 2^{-d},  |d| <= 10 log2(e) * 16 / 2
    bf16x8 qb[4];  // q~ as MFMA operands
    bf16x8 kb[4];  // k~ as MFMA operands
    f32x4 uk[4], uq[4];
    float dd[32];
    if (GLA) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        uk[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
        uq[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          uk[mt] = mfma(lds8(smem + LD::WK + (mt * 4 + s) * kFrag + lane * 16), cur.xk[s], uk[mt]);
          if (Q) uq[mt] = mfma(lds8(smem + LD::WQ + (mt * 4 + s) * kFrag + lane * 16), cur.xq[s], uq[mt]);
        }
      if (more) load_chunk<MODE, LOAD_QK>(p, bh, c + 1, cur);
      if (p.gate_is_log) {  // one uniform branch around the whole loop
#pragma unroll
        for (int i = 0; i < 32; ++i) dd[i] = (float)cur.xg[i >> 3][i & 7] * kLog2e;
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) dd[i] = log2_sigmoid((float)cur.xg[i >> 3][i & 7]);
      }
      if (more) load_chunk<MODE, LOAD_G>(p, bh, c + 1, cur);
      if (full) {
#pragma unroll
        for (int i = 0; i < 32; ++i) dd[i] = fmaxf(dd[i], kMinLog2Gate);
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) dd[i] = tok_ok ? fmaxf(dd[i], kMinLog2Gate) : 0.0f;
      }
      // in-tile inclusive cumsum over the 16 tokens: one scan step across all 32
      // features at a time, so consecutive DPP reads never wait on each other
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_shr<1>(dd[i]);
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_shr<2>(dd[i]);
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_shr<4>(dd[i]);
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_shr<8>(dd[i]);
      if (n == 15) {
        float *T = (float *)(smem + LD::T) + wave * kF;
#pragma unroll
        for (int i = 0; i < 32; ++i) T[feat(g, i)] = dd[i];
      }
    }
    __syncthreads();  // B1a: tile log-gate totals visible

    // Fold reference r (base 2, per feature).  Chunk mode: r = B/2, one
    // reference for the whole chunk, so cross-tile factors are 1; used when every
    // feature's chunk total satisfies |B| <= kChunkRefLimit, which keeps
    // |b - r| <= |B|/2 in range.  Tile mode otherwise: r_w = P_w + T_w/2.
    // Per-tile quantities are computed for features 2n, 2n+1 of the lane's group
    // and broadcast to the row (DPP) where needed.
    float tt[4][2], pre[2], btot[2], tw[2], rr2[2];
    bool chunk_mode = true;
    if (GLA) {
      const float *T = (const float *)(smem + LD::T);
      const int f0 = feat(g, 2 * n);
#pragma unroll
      for (int w2 = 0; w2 < 4; ++w2) {
        const float2 v2 = *(const float2 *)(T + w2 * kF + f0);
        tt[w2][0] = v2.x;
        tt[w2][1] = v2.y;
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        pre[e] = 0.0f;
        btot[e] = 0.0f;
        tw[e] = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          btot[e] += tt[w2][e];
          if (w2 < wave) pre[e] += tt[w2][e];
          if (w2 == wave) tw[e] = tt[w2][e];
        }
      }
      // every wave sees all 128 features, so the vote is the same in all waves
      chunk_mode = __all(fabsf(btot[0]) <= kChunkRefLimit && fabsf(btot[1]) <= kChunkRefLimit);
      float off[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        rr2[e] = chunk_mode ? 0.5f * btot[e] : pre[e] + 0.5f * tw[e];
        off[e] = pre[e] - rr2[e];  // b_chunk - r = b_loc + off
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) dd[i] += row_bcast(off[i & 1], i >> 1);

      // Hedgehog softmaxes of +u and -u, scaled by the fold factors
      auto features = [&](const f32x4 *u, bf16x8 *outb, float sgn) {
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
        float out[32];
        float zp = 0.0f, zn = 0.0f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int e = 4 * mt + j;
            out[e] = exp2_fast(u[mt][j] * kLog2e - mx);
            out[16 + e] = exp2_fast(mn - u[mt][j] * kLog2e);
            zp += out[e];
            zn += out[16 + e];
          }
        const float izp = rcp_fast(grp_sum(zp)), izn = rcp_fast(grp_sum(zn));
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          out[e] *= izp * exp2_fast(sgn * dd[e]);
          out[16 + e] *= izn * exp2_fast(sgn * dd[16 + e]);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) outb[s] = pack8(out + 8 * s);
      };
      features(uk, kb, -1.0f);
      if (!full && !tok_ok) {
#pragma unroll
        for (int s = 0; s < 4; ++s) kb[s] = zero8();
      }
      if (INTRA) {
#pragma unroll
        for (int s = 0; s < 4; ++s) sts8(smem + LD::KT + (wave * 4 + s) * kFrag + lane * 16, kb[s]);
      }
      if (Q) features(uq, qb, 1.0f);
    }
    __syncthreads();  // B1: k~ fragments visible

    // ================= row phase 2: cross-tile factors, intra scores =================
    // Per-tile factors depend on the feature only; lane n computes them for
    // features 2n, 2n+1 of its group and the others broadcast them (DPP).
    if (GLA) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        fdec[e] = exp2_fast(btot[e]);
        dsum2[e] += btot[e];
      }
      // q-bar = phi_q 2^{b_chunk} = q~ 2^{r} (inter-chunk readout), r <= 0
      if (Q) {
        float fq[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) fq[e] = exp2_fast(rr2[e]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          float tmp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) tmp[j] = (float)qb[s][j] * row_bcast(fq[j & 1], (8 * s + j) >> 1);
          sts8(smem + LD::QB + (wave * 4 + s) * kFrag + lane * 16, pack8(tmp));
        }
      }
      {  // k-hat = phi_k 2^{B - b_chunk} = k~ 2^{B - r} (state update) -> k-hat^T fragments: state
         // tile mt takes its 16 features from K-step s(mt) = 2(mt/4) + (mt%4)/2 of
         // the token-row operand, transposed on the matrix core
        float fk[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) fk[e] = exp2_fast(btot[e] - rr2[e]);
        bf16x8 kh[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
          float tmp[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) tmp[j] = (float)kb[s2][j] * row_bcast(fk[j & 1], (8 * s2 + j) >> 1);
          kh[s2] = pack8(tmp);
        }
        const int sp = wave >> 1, hh = wave & 1;
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
          const int s2 = 2 * (mt >> 2) + ((mt & 3) >> 1);
          const f32x4 t = mfma(kh[s2], sel[mt & 1], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
          *(bf16x4 *)(smem + LD::KH + (mt * 2 + sp) * kFrag + lane * 16 + hh * 8) = pack4(t);
        }
      }
      // intra-chunk scores A^T for key tiles kt = wave-4+i, i = 1..4, kt >= 0
      if (INTRA) {
        {  // diagonal tile: q~ k~^T with the tile's own reference
          f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < 4; ++s) acc = mfma(kb[s], qb[s], acc);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (4 * g + j > n) acc[j] = 0.0f;  // causal: key after query
          Wt[4] += acc;
        }
        // earlier tiles: in chunk mode both sides share the reference; in tile mode
        // q~ is scaled by 2^{r_w - r_kt} <= 1 with r_x = P_x + T_x/2
#pragma unroll
        for (int i = 1; i < 4; ++i) {
          const int kt = wave - 4 + i;
          if (kt >= 0 && chunk_mode) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s)
              acc = mfma(lds8(smem + LD::KT + (kt * 4 + s) * kFrag + lane * 16), qb[s], acc);
            Wt[i] += acc;
          } else if (kt >= 0) {
            float fo[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
              float run = 0.0f, tk = 0.0f;  // log-gate sum of tiles kt .. wave-1
#pragma unroll
              for (int w2 = 0; w2 < 4; ++w2) {
                if (w2 >= kt && w2 < wave) run += tt[w2][e];
                if (w2 == kt) tk = tt[w2][e];
              }
              fo[e] = exp2_fast(run + 0.5f * (tw[e] - tk));
            }
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              float tmp[8];
#pragma unroll
              for (int j = 0; j < 8; ++j) tmp[j] = (float)qb[s][j] * row_bcast(fo[j & 1], (8 * s + j) >> 1);
              acc = mfma(lds8(smem + LD::KT + (kt * 4 + s) * kFrag + lane * 16), pack8(tmp), acc);
            }
            Wt[i] += acc;
          }
        }
      }
    }

    if (Q) {
      // weight fragments for the (weights x V) GEMM
      if (SWA) {
        sts8(smem + LD::W + (wave * NKS + 0) * kFrag + lane * 16, pack44(Wt[0], Wt[1]));
        sts8(smem + LD::W + (wave * NKS + 1) * kFrag + lane * 16, pack44(Wt[2], Wt[3]));
        sts8(smem + LD::W + (wave * NKS + 2) * kFrag + lane * 16,
             pack44(Wt[4], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}));
      } else {
        // absolute key tiles 0..3 of the chunk: tile kt is Wt[kt - wave + 4]
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        f32x4 w0 = z, w1 = z, w2 = z, w3 = z;
        switch (wave) {
          case 0: w0 = Wt[4]; break;
          case 1: w0 = Wt[3]; w1 = Wt[4]; break;
          case 2: w0 = Wt[2]; w1 = Wt[3]; w2 = Wt[4]; break;
          default: w0 = Wt[1]; w1 = Wt[2]; w2 = Wt[3]; w3 = Wt[4]; break;
        }
        sts8(smem + LD::W + (wave * NKS + 0) * kFrag + lane * 16, pack44(w0, w1));
        sts8(smem + LD::W + (wave * NKS + 1) * kFrag + lane * 16, pack44(w2, w3));
      }
    }
    __syncthreads();  // B2: q-bar, k-hat^T, weight fragments visible

  }

  // ---- epilogue
  if (MODE == MODE_STATE) {
    float *dst = p.seg_state + (bh * NS + seg) * (size_t)(kF * kDV);
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvcol(wave, dt, n)] = S[mt][dt][j];
    if (wave == 0) {
      float *dd = p.seg_decay + (bh * NS + seg) * (size_t)kF;
      *(float2 *)(dd + feat(g, 2 * n)) = make_float2(dsum2[0], dsum2[1]);
    }
  } else if (GLA && p.state_out && seg == p.P - 1) {
    float *dst = p.state_out + bh * kF * kDV;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvcol(wave, dt, n)] = S[mt][dt][j];
  }
}

// ---------------------------------------------------------------- state pass
// End state, from a zero state, of one slice of a segment and the slice's total
// base-2 log-decay: S <- diag(2^{B}) S + k-hat^T V per chunk with
// k-hat = phi_k 2^{B - b} (exponent <= 0, so no fold reference is needed).
// Block = 4 waves, two blocks per CU.  Wave w: token tile w for the row work
// (u_k, the log-gate cumsums, phi(k), k-hat^T fragments transposed on the matrix
// core, V^T fragments) and d_v columns [32w, 32w + 32) of the state.  Two
// barriers per chunk: B1a (tile totals visible, previous update done) and B1
// (k-hat^T and V^T fragments visible).
struct LdsState {
  static constexpr int WK = 0;                   // Wphi_k^T frags [4 mt][4 s]
  static constexpr int VT = WK + 16 * kFrag;     // V^T half frags [4 tile][8 dv tile]
  static constexpr int KH = VT + 32 * kHalf;     // k-hat^T frags [8 mt][2 sp]
  static constexpr int T = KH + 16 * kFrag;      // tile log-gate totals [4 tile][128]
  static constexpr int BYTES = T + 4 * kF * 4;
};

__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(2, 2)))
void state_kernel(ChunkParams p) {
  using LD = LdsState;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int NS = (p.P - 1) * p.R;
  const size_t bh = blockIdx.x / NS;
  const int seg = blockIdx.x % NS;  // state slice
  const int h = (int)(bh % p.H);
  const int ps = seg / p.R, r = seg % p.R;
  const int seg_end = min((ps + 1) * p.seg_chunks, p.nchunks);
  const int c_begin = min(ps * p.seg_chunks + r * p.sub_chunks, seg_end);
  const int c_end = min(c_begin + p.sub_chunks, seg_end);  // may be empty: zero state, zero decay
  const bool gate_is_log = p.gate_is_log != 0;

  // Wphi_k^T fragments (see the output pass for the layout)
  for (int idx = tid; idx < 16 * 64; idx += kNT) {
    const int fi = idx >> 6, l = idx & 63, rr = l & 15, gg = l >> 4;
    const int mt = fi >> 2, s = fi & 3;
    const int m = 16 * (rr >> 2) + 4 * mt + (rr & 3);
    const bf16 *w = p.wk + (size_t)h * kD * kF2;
    bf16x8 f;
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = w[(32 * gg + 8 * s + j) * kF2 + m];
    sts8(smem + LD::WK + fi * kFrag + l * 16, f);
  }
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  const HeadBufs hb = head_bufs(p, bh);
  const unsigned ro = row_off(wave);
  // state slice: S[mt][dt][j] = S[feat(g, 4mt + j)][dvcol(wave, dt, n)]
  f32x4 S[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) S[mt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  float dsum2[2] = {0.0f, 0.0f};  // total base-2 log-decay (features 2n, 2n+1 of the group)
  bf16x8 xk[4], xv[4], xg[4];
  load_rows(hb.k, ro + chunk_off(c_begin), xk);
  load_vals(hb.v, ro + chunk_off(c_begin), xv);
  load_gates(hb.g, ro + chunk_off(c_begin), xg);
  __syncthreads();

  for (int c = c_begin; c < c_end; ++c) {
    const unsigned ro1 = ro + chunk_off(c + 1);
    const bool tok_ok = c * kC + 16 * wave + n < p.L;
    // ---- row work of tile `wave` up to the tile totals
    f32x4 u[4];
    project(smem + LD::WK + lane * 16, xk, u);
    load_rows(hb.k, ro1, xk);  // next chunk's keys
    float dd[32];
    tile_cumsum(xg, gate_is_log, tok_ok, dd);
    load_gates(hb.g, ro1, xg);
    if (n == 15) {
      float *T = (float *)(smem + LD::T) + wave * kF;
#pragma unroll
      for (int i = 0; i < 32; ++i) T[feat(g, i)] = dd[i];
    }
    float e[32], izp, izn;
    hedgehog_exp(u, e, izp, izn);
    __syncthreads();  // B1a: tile totals visible; the previous chunk's update done

    // ---- V^T fragments of this tile
    {
      char *base = smem + LD::VT + wave * 8 * kHalf + lane * 8;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        f32x4 t2[2];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) t2[dt] = mfma(xv[s], sel[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) *(bf16x4 *)(base + (2 * s + dt) * kHalf) = pack4(t2[dt]);
      }
    }
    load_vals(hb.v, ro1, xv);  // next chunk's values
    // ---- k-hat = phi_k 2^{B - b} with B - b = (B - P_w) - b_loc <= 0
    float fdec[2], rest[2];  // 2^{B}; B - P_w
    {
      const float *T = (const float *)(smem + LD::T);
      const int f0 = feat(g, 2 * n);
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        float btot = 0.0f, pre = 0.0f;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float tv = T[w2 * kF + f0 + e2];
          btot += tv;
          if (w2 < wave) pre += tv;
        }
        fdec[e2] = exp2_fast(btot);
        dsum2[e2] += btot;
        rest[e2] = btot - pre;
      }
    }
    bf16x8 kh[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float a8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * s + j;
        a8[j] = e[i] * (i < 16 ? izp : izn) * exp2_fast(row_bcast(rest[i & 1], i >> 1) - dd[i]);
      }
      kh[s] = tok_ok ? pack8(a8) : zero8();  // keys past the end contribute nothing
    }
    {  // k-hat^T fragments: state tile mt takes its 16 features from K-step
       // s(mt) = 2(mt/4) + (mt%4)/2 of the token-row operand
      const int sp = wave >> 1, hf = wave & 1;
#pragma unroll
      for (int m2 = 0; m2 < 4; ++m2) {
        f32x4 t2[2];
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2) {
          const int mt = 2 * m2 + d2;
          const int s2 = 2 * (mt >> 2) + ((mt & 3) >> 1);
          t2[d2] = mfma(kh[s2], sel[mt & 1], (f32x4){0.0f, 0.0f, 0.0f, 0.0f});
        }
#pragma unroll
        for (int d2 = 0; d2 < 2; ++d2)
          *(bf16x4 *)(smem + LD::KH + ((2 * m2 + d2) * 2 + sp) * kFrag + lane * 16 + hf * 8) = pack4(t2[d2]);
      }
    }
    __syncthreads();  // B1: k-hat^T and V^T fragments visible

    // ---- S <- diag(2^{B}) S + k-hat^T V (columns of this wave), fragments of a
    // group of 4 state tiles requested together
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float eb = row_bcast(fdec[j & 1], (4 * mt + j) >> 1);
        S[mt][0][j] *= eb;
        S[mt][1][j] *= eb;
      }
    bf16x8 bv[2][2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const char *vb = smem + LD::VT + ((2 * sp) * 8 + 2 * wave + dt) * kHalf + lane * 8;
        bv[sp][dt] = join44(*(const bf16x4 *)vb, *(const bf16x4 *)(vb + 8 * kHalf));
      }
#pragma unroll
    for (int grp = 0; grp < 4; ++grp) {  // grp = 2 sp + (mt / 4)
      const int sp = grp >> 1, mb = 4 * (grp & 1);
      bf16x8 kf[4];
      issue_fence();
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) kf[m4] = lds8(smem + LD::KH + ((mb + m4) * 2 + sp) * kFrag + lane * 16);
      issue_fence();
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) S[mb + m4][dt] = mfma(kf[m4], bv[sp][dt], S[mb + m4][dt]);
    }
  }

  float *dst = p.seg_state + (bh * NS + seg) * (size_t)(kF * kDV);
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvcol(wave, dt, n)] = S[mt][dt][j];
  if (wave == 0) {
    float *dd = p.seg_decay + (bh * NS + seg) * (size_t)kF;
    *(float2 *)(dd + feat(g, 2 * n)) = make_float2(dsum2[0], dsum2[1]);
  }
}

// State after every state slice: S_(0) = e^{D_0} S_in + dS_0,
// S_(q) = e^{D_q} S_(q-1) + dS_q.  Thread = one state element of one head; the
// slots are overwritten in place (slot q receives S_(q)).
__global__ __launch_bounds__(kNT) void segment_scan_kernel(float *seg_state, const float *seg_decay,
                                                           const float *state_in, int BH, int NS) {
  const size_t idx = (size_t)blockIdx.x * kNT + threadIdx.x;
  const size_t per = (size_t)kF * kDV;
  if (idx >= (size_t)BH * per) return;
  const size_t bh = idx / per, e = idx % per;
  const int f = (int)(e / kDV);
  float s = state_in ? state_in[idx] : 0.0f;
  for (int q = 0; q < NS; ++q) {
    float *slot = seg_state + (bh * NS + q) * per;
    const float dec = exp2_fast(seg_decay[(bh * NS + q) * kF + f]);  // base-2 log-decay
    s = dec * s + slot[e];
    slot[e] = s;
  }
}

// How one call is cut: P output segments of seg_chunks chunks; the state pass
// cuts segments 0..P-2 into R slices of sub_chunks chunks.
struct SegPlan {
  int nchunks = 0, P = 1, seg_chunks = 0, R = 1, sub_chunks = 0;
  int slices() const { return (P - 1) * R; }
};

SegPlan plan_segments(const LayerArgs &a) {
  SegPlan s;
  s.nchunks = (a.L + kC - 1) / kC;
  const int bh = a.B * a.H;
  const int cus = device_cu_count();
  // output pass: about one block per compute unit (its LDS allows one), at least
  // 4 chunks per segment, and every segment owns at least one chunk
  int P = (cus + bh - 1) / bh;
  P = max(1, min(P, s.nchunks / 4));
  s.seg_chunks = (s.nchunks + P - 1) / P;
  s.P = (s.nchunks + s.seg_chunks - 1) / s.seg_chunks;
  // state pass: two blocks fit on a compute unit, so aim at two per unit, with
  // at least 2 chunks per slice
  if (s.P > 1) {
    int R = (2 * cus) / (bh * (s.P - 1));
    s.R = max(1, min(R, s.seg_chunks / 2));
  }
  s.sub_chunks = (s.seg_chunks + s.R - 1) / s.R;
  return s;
}

ChunkParams make_params(const LayerArgs &a, int P, int seg_chunks, int nchunks) {
  ChunkParams p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.v = (const bf16 *)a.v;
  p.gate = (const bf16 *)a.gate; p.wq = (const bf16 *)a.wq; p.wk = (const bf16 *)a.wk;
  p.meta = a.meta; p.state_in = a.state_in; p.state_out = a.state_out; p.o = (bf16 *)a.o;
  p.seg_state = nullptr; p.seg_decay = nullptr;
  p.B = a.B; p.H = a.H; p.L = a.L; p.window = a.window; p.n_meta = a.n_meta;
  p.nchunks = nchunks; p.P = P; p.seg_chunks = seg_chunks;
  p.R = 1; p.sub_chunks = seg_chunks;
  p.scale = a.scale; p.gate_is_log = a.gate_is_log ? 1 : 0;
  return p;
}

template <int MODE>
hipError_t launch_mode(const ChunkParams &p, int blocks, hipStream_t stream) {
  const int bytes = Lds<MODE>::BYTES;
  hipError_t e = hipFuncSetAttribute((const void *)chunk_kernel<MODE>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(chunk_kernel<MODE>, dim3((unsigned)blocks), dim3(kNT), bytes, stream, p);
  return hipGetLastError();
}

}  // namespace

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n;
}

bool chunked_supported(const LayerArgs &a, int parts) {
  if (!a.bf16 || a.d != kD || a.dv != kDV) return false;
  if ((parts & PART_GLA) && (a.f != kF || a.chunk != kC)) return false;
  if ((parts & PART_SWA) && (a.window < 1 || a.window > kC)) return false;
  return true;
}

size_t chunked_workspace_bytes(const LayerArgs &a, int parts) {
  if (!(parts & PART_GLA) || a.L <= 0) return 0;
  const SegPlan s = plan_segments(a);
  const size_t bh = (size_t)a.B * a.H;
  return bh * s.slices() * ((size_t)kF * kDV + kF) * sizeof(float);
}

hipError_t launch_chunked_prefill(const LayerArgs &a, int parts) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  const int bh = a.B * a.H;
  const SegPlan s = plan_segments(a);
  ChunkParams p = make_params(a, s.P, s.seg_chunks, s.nchunks);
  p.R = s.R;
  p.sub_chunks = s.sub_chunks;
  if (s.P > 1) {
    const int NS = s.slices();
    p.seg_state = (float *)a.ws;
    p.seg_decay = p.seg_state + (size_t)bh * NS * kF * kDV;
    hipError_t e = hipFuncSetAttribute((const void *)state_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       LdsState::BYTES);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(state_kernel, dim3((unsigned)(bh * NS)), dim3(kNT), LdsState::BYTES, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t elems = (size_t)bh * kF * kDV;
    hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)((elems + kNT - 1) / kNT)), dim3(kNT), 0,
                       a.stream, p.seg_state, (const float *)p.seg_decay, a.state_in, bh, NS);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_chunk_out(p, parts != PART_GLA, bh * s.P, a.stream);
}

bool swa_mfma_supported(const LayerArgs &a) {
  return a.bf16 && a.d == kD && a.dv == kDV && a.window >= 1 && a.window <= kC;
}

hipError_t launch_swa_mfma(const LayerArgs &a) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  const int nchunks = (a.L + kC - 1) / kC;
  ChunkParams p = make_params(a, nchunks, 1, nchunks);
  return launch_mode<MODE_SWA>(p, a.B * a.H * nchunks, a.stream);
}

}  // namespace glah

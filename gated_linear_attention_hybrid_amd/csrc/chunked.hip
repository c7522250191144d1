// chunked.hip -- chunkwise-parallel MFMA prefill of the hybrid layer for gfx950
// (bf16 inputs, fp32 accumulation, d = f = d_v = 128, 64-token chunks): the
// state pass, the segment scan and the window-only kernel, and the host-side
// plan of one call.  The output pass is in chunk_out.hip.
//
// Method ("Lizard" technical summary, gist.science 2507.09025, Methodology C,
// hardware-aware algorithm): the Hedgehog features are non-negative, so the
// cumulative log-gates can be moved into phi(q) and phi(k) and every product
// inside a chunk becomes a plain low-precision GEMM instead of a cumulative
// product that underflows.  With b_t the in-chunk inclusive cumsum of
// a = log Gamma (per feature) and B the chunk total:
//   state:  S_{c+1} = diag(e^{B}) S_c + sum_s (phi_k[s] e^{B - b_s})^T v_s
// The window part (Methodology A.2) is a banded softmax over the 5 key tiles that
// can reach a 16-query tile, with a denominator that starts from the meta-memory
// sinks.
//
// Parallel structure over one head: the sequence is cut into P segments.
//   state_kernel         end state of every slice of the segments 0..P-2 from a
//                        zero state, and its total log-decay
//   segment_scan_kernel  the state after every segment's last slice (fp32,
//                        sequential over the slices)
//   chunk_out_kernel     the outputs, one block per segment, starting from the
//                        state after the segment's preceding slice
//   swa_kernel           window attention alone, one block per chunk
//
// Operands are exchanged through LDS as ready-made MFMA fragments (1 KiB: 64
// lanes x 16 B).
#include <mutex>

#include "chunk_common.hpp"
#include "launch.hpp"

// Device scratch of the no-allocation entry point: the segment states of the
// state pass live here instead of in a caller workspace.  One copy per device,
// held until the process ends; every call on a device shares it.  Host code
// uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[glah::kNoAllocScratchBytes];

namespace glah {

namespace {

constexpr int kNT = 256;    // threads per block

// ---------------------------------------------------------------- window only
// swa_meta_attn: one block of 4 waves per 64-token chunk.  Wave w stages the raw
// keys and V^T fragments of token tile w of this chunk and the one before, scores
// query tile w against the 5 key tiles w-4 .. w, takes the one-shot softmax with
// the sinks and writes the weight fragments; after a barrier it multiplies them
// with V^T for d_v columns [32w, 32w + 32).
struct LdsSwa {
  static constexpr int RK = 0;                 // raw k frags [2 chunk][4 tile][4 s]
  static constexpr int VT = RK + 32 * kFrag;   // V^T half frags [2 chunk][4 tile][8 dv tile]
  static constexpr int W = VT + 64 * kHalf;    // weight frags [4 qt][3]
  static constexpr int BYTES = W + 12 * kFrag;
};

__global__ __launch_bounds__(kNT) void swa_kernel(ChunkParams p) {
  using LD = LdsSwa;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const size_t bh = blockIdx.x / p.nchunks;
  const int c = blockIdx.x % p.nchunks;
  const int h = (int)(bh % p.H);
  const HeadBufs hb = head_bufs(p, bh);
  const unsigned ro = row_off(wave);
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};

  // keys and values of tile `wave` of the previous chunk (ci = 0) and this one
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    bf16x8 xk[4], xv[4];
    load_rows(hb.k, ro + chunk_off(c - 1 + ci), xk);
    load_vals(hb.v, ro + chunk_off(c - 1 + ci), xv);
#pragma unroll
    for (int s = 0; s < 4; ++s) sts8(smem + LD::RK + ((ci * 4 + wave) * 4 + s) * kFrag + lane * 16, xk[s]);
    char *base = smem + LD::VT + (ci * 4 + wave) * 8 * kHalf + lane * 8;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        *(bf16x4 *)(base + (2 * s + dt) * kHalf) =
            pack4(mfma(xv[s], sel[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}));
  }
  bf16x8 xq[4];
  load_rows(hb.q, ro + chunk_off(c), xq);
  // meta-memory sinks of this head, base 2
  float meta_max = -INFINITY, meta_sum = 0.0f;
  {
    const float *meta = p.meta + (size_t)h * p.n_meta;
    for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, meta[m] * kLog2e);
    for (int m = 0; m < p.n_meta; ++m) meta_sum += exp2_fast(meta[m] * kLog2e - meta_max);
    if (p.n_meta == 0) meta_max = 0.0f;  // meta_sum = 0: no sink mass
  }
  __syncthreads();

  // band scores for key tiles wave-4+i; key position minus query position is
  // 16(i-4) + 4g + j - n, valid when in (-window, 0] and at a position >= 0
  const int tq = c * kC + 16 * wave + n;
  const float sl2 = p.scale * kLog2e;
  f32x4 sc[5];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int kt = wave - 4 + i;
    const int ci = kt >= 0 ? 1 : 0, tl = kt >= 0 ? kt : kt + 4;
    bf16x8 a[4];
    issue_fence();
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = lds8(smem + LD::RK + ((ci * 4 + tl) * 4 + s) * kFrag + lane * 16);
    issue_fence();
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma(a[s], xq[s], acc);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rel = 16 * (i - 4) + 4 * g + j - n;
      const bool ok = rel <= 0 && rel > -p.window && tq + rel >= 0;
      acc[j] = ok ? acc[j] * sl2 : -INFINITY;
      mx = fmaxf(mx, acc[j]);
    }
    sc[i] = acc;
  }
  mx = fmaxf(grp_max(mx), meta_max);
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < 5; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sc[i][j] = exp2_fast(sc[i][j] - mx);  // 2^{-inf} = 0
      sum += sc[i][j];
    }
  sum = grp_sum(sum) + meta_sum * exp2_fast(meta_max - mx);
  const float inv = rcp_fast(sum);
  sts8(smem + LD::W + (wave * 3 + 0) * kFrag + lane * 16, pack44(sc[0] * inv, sc[1] * inv));
  sts8(smem + LD::W + (wave * 3 + 1) * kFrag + lane * 16, pack44(sc[2] * inv, sc[3] * inv));
  sts8(smem + LD::W + (wave * 3 + 2) * kFrag + lane * 16, pack44(sc[4] * inv, (f32x4){0.0f, 0.0f, 0.0f, 0.0f}));
  __syncthreads();

  // O^T = V^T W^T for d_v columns [32 wave, 32 wave + 32); lane (n, g) of query
  // tile qt holds d_v 32 wave + 8g + (4dt + j)
  const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
  auto vt_half = [&](int kt, int dt) -> bf16x4 {
    const int ci = kt >= 0 ? 1 : 0, tl = kt >= 0 ? kt : kt + 4;
    return *(const bf16x4 *)(smem + LD::VT + ((ci * 4 + tl) * 8 + 2 * wave + dt) * kHalf + lane * 8);
  };
#pragma unroll
  for (int qt = 0; qt < 4; ++qt) {
    f32x4 O[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < 3; ++ks) {
      const bf16x8 b = lds8(smem + LD::W + (qt * 3 + ks) * kFrag + lane * 16);
      const int ka = qt - 4 + 2 * ks;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        O[dt] = mfma(join44(vt_half(ka, dt), ks < 2 ? vt_half(ka + 1, dt) : z4), b, O[dt]);
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack44(O[0], O[1])), hb.o,
                                           (int)(chunk_off(c) + (unsigned)(16 * qt + n) * (kDV * 2) +
                                                 64 * wave + 16 * g),
                                           0, 0);
  }
}

// ---------------------------------------------------------------- state pass
// End state, from a zero state, of one slice of a segment and the slice's total
// base-2 log-decay.  Unrolled over the slice's chunks the recurrence
// S <- diag(2^{B_c}) S + k-hat_c^T V_c gives S = sum_c (k-hat_c 2^{R_c})^T V_c with
// k-hat_c = phi_k 2^{B_c - b} and R_c the log-decay of the chunks after c; taking
// the chunks last to first builds R_c as a running sum, so every exponent is
// <= 0 (no fold reference) and the state is never rescaled.
// Block = 4 waves, two blocks per CU.  Wave w: token tile w for the row work
// (u_k, the gate decay exponents, phi(k), k-hat^T fragments transposed on the
// matrix core) and d_v columns dvpair(w, 0..1, 0..15) of the state, whose value
// operands it reads straight from memory (one dword per token row holds both
// of a lane's columns).  Two barriers per chunk: B1a (tile totals visible,
// previous update done) and B1 (k-hat^T fragments visible).
struct LdsState {
  static constexpr int WK = 0;                   // Wphi_k^T frags [4 mt][4 s]
  static constexpr int KH = WK + 16 * kFrag;     // k-hat^T frags [8 mt][2 sp]
  static constexpr int T = KH + 16 * kFrag;      // tile decay totals (-log2-gate sums) [4 tile][128]
  static constexpr int BYTES = T + 4 * kF * 4;
};

template <bool SG>
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
  // state slice: S[mt][dt][j] = S[feat(g, 4mt + j)][dvpair(wave, dt, n)]
  f32x4 S[8][2];
#pragma unroll
  for (int mt = 0; mt < 8; ++mt)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) S[mt][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
  // base-2 log-decay of the chunks after the current one (features 2n, 2n+1 of
  // the group); the slice total at the end
  float rsum2[2] = {0.0f, 0.0f};
  // value operands of d_v columns dvpair(wave, dt, n) over token tiles (2sp,
  // 2sp + 1): dwords of tokens 16T + 4g + j (vraw), packed per column tile
  uint32_t vraw[4][4];
  auto load_v = [&](int cc) {
#pragma unroll
    for (int T = 0; T < 4; ++T)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vraw[T][j] = __builtin_amdgcn_raw_buffer_load_b32(
            hb.v, (int)(chunk_off(cc) + (unsigned)(16 * T + 4 * g + j) * (kDV * 2) + 64 * wave + 4 * n), 0, 0);
  };
  bf16x8 xk[4], xg[4];
  load_rows(hb.k, ro + chunk_off(c_end - 1), xk);
  load_v(c_end - 1);
  load_gates<SG>(hb, ro + chunk_off(c_end - 1), xg);
  __syncthreads();

  // The chunks are taken last to first, so the state is never decayed: chunk c
  // adds (phi_k 2^{B_c - b + R_c})^T V with R_c the log-decay of the later chunks
  // of the slice, an exponent <= 0.  Rows past the end have V = 0 (range check)
  // and add nothing.
  for (int c = c_end - 1; c >= c_begin; --c) {
    const unsigned ro1 = ro + chunk_off(c - 1);  // c - 1 < 0 wraps past the range: reads 0
    // ---- row work of tile `wave` up to the tile totals
    f32x4 u[4];
    project(smem + LD::WK + lane * 16, xk, u);
    load_rows(hb.k, ro1, xk);  // preceding chunk's keys
    float dn[32];
    tile_decay(xg, gate_is_log, c * kC + 16 * wave + n < p.L, dn);
    load_gates<SG>(hb, ro1, xg);
    if (n == 15) {
      float *T = (float *)(smem + LD::T) + wave * kF;
#pragma unroll
      for (int i = 0; i < 32; ++i) T[feat(g, i)] = dn[i];
    }
    float e[32], izp, izn;
    hedgehog_exp(u, e, izp, izn);
    __syncthreads();  // B1a: tile totals visible; the previous update done

    // ---- value operands of this chunk, then the preceding chunk's dwords requested
    bf16x8 bv[2][2];
#pragma unroll
    for (int sp = 0; sp < 2; ++sp)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const uint32_t halves = dt ? 0x07060302u : 0x05040100u;  // high or low halves
        u32x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int T = 2 * sp + (e >> 1), hh = e & 1;
          r[e] = __builtin_amdgcn_perm(vraw[T][2 * hh + 1], vraw[T][2 * hh], halves);
        }
        bv[sp][dt] = __builtin_bit_cast(bf16x8, r);
      }
    load_v(c - 1);  // preceding chunk's values
    // ---- k-hat = phi_k 2^{B - b + R} with B - b = (B - P_w) - b_loc <= 0
    float base[2];  // B - P_w + R, then R += B
    {
      const float *T = (const float *)(smem + LD::T);
      const int f0 = feat(g, 2 * n);
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        float btot = 0.0f, rest = 0.0f;  // decay exponents of the chunk and of tiles >= wave
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2) {
          const float tv = T[w2 * kF + f0 + e2];
          btot += tv;
          if (w2 >= wave) rest += tv;
        }
        base[e2] = rsum2[e2] - rest;
        rsum2[e2] -= btot;
      }
    }
    bf16x8 kh[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      float a8[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int i = 8 * s + j;
        a8[j] = e[i] * (i < 16 ? izp : izn) * exp2_fast(row_bcast(base[i & 1], i >> 1) + dn[i]);
      }
      kh[s] = pack8(a8);
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
    __syncthreads();  // B1: k-hat^T fragments visible

    // ---- S += k-hat^T V (columns of this wave), fragments of a group of 4 state
    // tiles requested together
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
      for (int j = 0; j < 4; ++j) dst[feat(g, 4 * mt + j) * kDV + dvpair(wave, dt, n)] = S[mt][dt][j];
  if (wave == 0) {
    float *dd = p.seg_decay + (bh * NS + seg) * (size_t)kF;
    *(float2 *)(dd + feat(g, 2 * n)) = make_float2(rsum2[0], rsum2[1]);
  }
}

// State after every state slice: S_(0) = e^{D_0} S_in + dS_0,
// S_(q) = e^{D_q} S_(q-1) + dS_q.  Thread = one state element of one head; the
// slots are overwritten in place, but only the last slice of each segment (q =
// R - 1, 2R - 1, ...) receives S_(q): the output pass reads no other (the
// kernel is bound by HBM, so the other stores are skipped).
__global__ __launch_bounds__(kNT) void segment_scan_kernel(float *seg_state, const float *seg_decay,
                                                           const float *state_in, int BH, int NS, int R) {
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
    if ((q + 1) % R == 0) slot[e] = s;
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
  p.kc = nullptr; p.vc = nullptr;
  p.B = a.B; p.H = a.H; p.L = a.L; p.window = a.window; p.n_meta = a.n_meta;
  p.nchunks = nchunks; p.P = P; p.seg_chunks = seg_chunks;
  p.R = 1; p.sub_chunks = seg_chunks;
  p.scale = a.scale; p.gate_is_log = a.gate_is_log ? 1 : 0; p.gate_mode = a.gate_mode;
  return p;
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
  // every accepted chunk request (16, 32, 64, 128) is served with 64-token
  // chunks: the blocking changes only the rounding, not the result
  if ((parts & PART_GLA) && a.f != kF) return false;
  if ((parts & PART_SWA) && (a.window < 1 || a.window > kC)) return false;
  return true;
}

size_t chunked_workspace_bytes(const LayerArgs &a, int parts) {
  if (!(parts & PART_GLA) || a.L <= 0) return 0;
  const SegPlan s = plan_segments(a);
  const size_t bh = (size_t)a.B * a.H;
  return bh * s.slices() * ((size_t)kF * kDV + kF) * sizeof(float);
}

hipError_t noalloc_scratch(void **ptr) {
  static std::mutex mu;
  static void *addr[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // the current device's copy
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_chunked_prefill(const LayerArgs &a, int parts, bool ring) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  const int bh = a.B * a.H;
  const SegPlan s = plan_segments(a);
  ChunkParams p = make_params(a, s.P, s.seg_chunks, s.nchunks);
  if (ring) {
    p.kc = (bf16 *)a.kcache;
    p.vc = (bf16 *)a.vcache;
  }
  p.R = s.R;
  p.sub_chunks = s.sub_chunks;
  if (s.P > 1) {
    const int NS = s.slices();
    p.seg_state = (float *)a.ws;
    p.seg_decay = p.seg_state + (size_t)bh * NS * kF * kDV;
    const void *fn = p.gate_mode != 0 ? (const void *)state_kernel<true> : (const void *)state_kernel<false>;
    hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LdsState::BYTES);
    if (e != hipSuccess) return e;
    if (p.gate_mode != 0)
      hipLaunchKernelGGL(state_kernel<true>, dim3((unsigned)(bh * NS)), dim3(kNT), LdsState::BYTES, a.stream, p);
    else
      hipLaunchKernelGGL(state_kernel<false>, dim3((unsigned)(bh * NS)), dim3(kNT), LdsState::BYTES, a.stream, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t elems = (size_t)bh * kF * kDV;
    hipLaunchKernelGGL(segment_scan_kernel, dim3((unsigned)((elems + kNT - 1) / kNT)), dim3(kNT), 0,
                       a.stream, p.seg_state, (const float *)p.seg_decay, a.state_in, bh, NS, s.R);
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
  hipError_t e = hipFuncSetAttribute((const void *)swa_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     LdsSwa::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(swa_kernel, dim3((unsigned)(a.B * a.H * nchunks)), dim3(kNT), LdsSwa::BYTES, a.stream, p);
  return hipGetLastError();
}

}  // namespace glah

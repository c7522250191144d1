// bwd_walk.hip -- the state walks of the gated part's backward in tile form on
// the gfx950 matrix cores (bf16 values, fp32 feature maps from the backward
// prologue, f = d_v = 128).
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
// (e^{b_t - b_s} = e^{b_t - m} e^{m - b_s}, m = B / 2); the prologue floors the
// per-token log-gate at -10 and stores b, so no factor leaves e^{+-80}.
//
// Each head's tokens are cut into P segments of whole 64-token tiles so that
// the walks run P-fold in parallel:
//   pass 1  each segment's own state from zero, S_loc (forward, segments
//           0 .. P-2) and G_loc (reverse, segments 1 .. P-1), and its total
//           log-decay D per feature;
//   pass 2  the walks, each segment starting from the state combined from the
//           earlier segments (S_start[p] = e^{D[p-1]} S_start[p-1] + S_loc[p-1])
//           or the later ones (G_end[p] = e^{D[p+1]} G_end[p+1] + G_loc[p+1]):
//     forward walk   (b, h, segment, 16 features; one wave): S^T of its
//                    features, dphiq and the 64-token tile sums of phiq .
//                    dphiq; the last segment S_{L-1} . dS_final
//     reverse walk   (b, h, segment; four waves of 32 features): G^T, dphik
//                    and its tile sums, dv (the four waves' parts summed in
//                    LDS every tile); the first segment dS_in and Gamma_0
//                    (S_in . dS_0).
// The state, the decayed maps and the tile's dO . v products enter the
// products behind dphiq and dphik as bf16 hi + lo pairs: the gate gradient is a
// running sum of phiq . dphiq - phik . dphik, differences of nearly equal
// terms.  dv takes bf16 operands.
// Lane layouts (n = lane & 15, g = lane >> 4) of the 16x16x16 MFMA as in the
// other kernels: A row n, K-slots 4g..4g+3; B column n, K-slots 4g..4g+3;
// accumulator column n, rows 4g..4g+3.  "Layout F" holds element (token 4g + r,
// feature n) of a tile in lane (n, g), slot r (a B operand over tokens, or an A
// operand with the feature as row); the reverse walk turns its layout-F
// operands into token rows over features with an identity product.
#include <algorithm>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;

// Pass-2 waves the segment count aims at: 768 blocks of four waves, half again
// as many as fit at once at two waves per SIMD.  Measured at 32K tokens, 16 and
// 32 heads (segments of 2048 and 4096 tokens), this beats 2048, 2304, 2688,
// 3456, 4096 and 4608 waves by 1-10%: shorter segments shorten the serial tile
// chains, and the forward-walk blocks, which finish first, leave their places
// to the rest.
constexpr int kWalkWaves = 3072;
// Each state is kept as e^{c} X with c the log-decay gathered since it was last
// written out in full, per feature: the tile's decay then scales the update's
// four map values instead of the state's 64 per lane.  Once c would fall
// below -kReref the state is rescaled and c restarts at 0, so the map factors
// e^{-c} stay below e^{kReref}.
constexpr float kReref = 40.0f;

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ f32x4 zf4() { return (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ float ex(float x) { return exp2_fast(x * kLog2e); }
__device__ __forceinline__ float dot4f(f32x4 a, f32x4 b) { return a[0] * b[0] + a[1] * b[1] + a[2] * b[2] + a[3] * b[3]; }

// x = hi + lo to about 2^-17 of |x|: two bf16 operands whose products with an
// exact bf16 operand sum (in fp32) to nearly the fp32 product.
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
// a layout-F operand (row = feature, K = token) as token rows over features
__device__ __forceinline__ bf16x4 to_rows(f32x4 x, bf16x4 eye) { return pack4(mma16(pack4(x), eye, zf4())); }

// One head's fp32 [L][128] rows as a buffer: reads past the last row return 0
// and writes there are dropped (offsets are 32-bit: L < 2^22).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t frows(const float *base, int bh, int L) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)(base + (size_t)bh * L * 128), (short)0, L * 512, 0x00020000);
}
__device__ __forceinline__ float fld(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
}
__device__ __forceinline__ void fst(__amdgpu_buffer_rsrc_t r, unsigned off, float x) {
  __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, (int)off, 0, 0);
}
__device__ __forceinline__ void fst4(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}
// byte offset of (token 16 tau + 4 g + r, column c) in [L][128] fp32 rows
__device__ __forceinline__ unsigned foff(int tau, int r, int c) {
  const unsigned g = (threadIdx.x & 63) >> 4;
  return ((unsigned)(16 * tau + r) + 4u * g) * 512u + (unsigned)c * 4u;
}

struct WalkParams {
  const float *pq, *pk, *gb;           // [B H L][128] fp32: maps, in-tile cumsum of the log-gate
  const bf16 *v, *dout;                // [B H][L][128]
  const float *state_in, *dstate_out;  // [B H][128][128] or null
  float *dpq, *dpk, *dvg;              // [B H L][128]
  bf16 *dvo;                           // [B H L][128] bf16: the gated part's dv (dv_mode 1)
  float *tq, *tk, *xs, *dstate_in;     // [BH][nft][128] x 2, [2][BH][128], [BH][128][128]
  float *sloc, *gloc, *dseg;           // [BH][P][128][128] x 2, [BH][P][128]
  int BH, L, nft, P, seg;              // seg: 16-token tiles per segment (a multiple of 4)
  int dv_mode;                         // 0: fp32 to dvg; 1: bf16 to dvo
};

// layout-F values of one tile: tokens 16 tau + 4 g + r, column c (0 past the end)
__device__ __forceinline__ void load_f(__amdgpu_buffer_rsrc_t r, int tau, int c, float *x) {
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = fld(r, foff(tau, i, c));
}
// b at the tile's last token (its total B; the last valid token for a ragged tile)
__device__ __forceinline__ float load_total(__amdgpu_buffer_rsrc_t r, int tau, int c, int L) {
  return fld(r, (unsigned)min(16 * tau + 15, L - 1) * 512u + (unsigned)c * 4u);
}

// ================================ pass 1 ====================================
// The four waves of a pass-1 block walk the same 16-token tiles, so a tile of
// value (or dO) rows is read once a block and shared through LDS: wave w loads
// rows 4w .. 4w + 3 (16 bytes a lane) into a buffer in the row-operand
// fragment layout (fragment (c & 3), lane (row + 16 (c >> 2)) holding row
// `row`, columns 8c .. 8c + 7), and every wave reads its transposed half
// fragments from it with gfx950's transposing LDS read.  Two buffers: one
// barrier a tile.
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_ptr;
constexpr int kRowTileBytes = 16 * 128 * 2;
__device__ __forceinline__ u32x4 tile_piece_load(__amdgpu_buffer_rsrc_t r, int tau) {
  const int lane = threadIdx.x & 63, row = 4 * (int)(threadIdx.x >> 6) + (lane >> 4), c = lane & 15;
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)((unsigned)(16 * tau + row) * 256u + (unsigned)c * 16u), 0, 0);
}
__device__ __forceinline__ void tile_piece_store(char *buf, u32x4 x) {
  const int lane = threadIdx.x & 63, row = 4 * (int)(threadIdx.x >> 6) + (lane >> 4), c = lane & 15;
  *(u32x4 *)(buf + (c & 3) * 1024 + (row + 16 * (c >> 2)) * 16) = x;
}
// Transposed half fragment (s, dt) of a staged tile: lane (n, g) gets
// x[token 4 g + r][32 s + 8 (n / 4) + 4 dt + n % 4], r = 0..3 (the A operand of a
// 16x16x16 product over tokens, as a selection product of the value-layout
// rows gives it).  ds_read_b64_tr_b16 hands lane i of each 16-lane row element
// i % 4 of the 8-byte chunks addressed by lanes 4 r + i / 4 of that row.
__device__ __forceinline__ bf16x4 tile_tr_half(const char *buf, int s, int dt) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const char *p = buf + (m & 3) * 1024 + (4 * g + (m >> 2) + 16 * s) * 16 + 8 * dt;
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(char *)p));
}

// forward: S_loc of segment seg from zero, 16 features (ft); D of the segment
__device__ __forceinline__ void fwd_state(const WalkParams &p, int bh, int seg, int ft, char *lds) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int f = 16 * ft + n, L = p.L, nt = (L + 15) / 16;
  const int t0 = seg * p.seg, t1 = min(t0 + p.seg, nt);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v, bh, L), rk = frows(p.pk, bh, L), rb = frows(p.gb, bh, L);
  f32x4 S[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) S[s][0] = S[s][1] = zf4();
  float lk[4], lb[4], lB;
  auto load = [&](int tau) {
    load_f(rk, tau, f, lk);
    load_f(rb, tau, f, lb);
    lB = load_total(rb, tau, f, L);
  };
  u32x4 vraw = tile_piece_load(rv, t0);
  load(t0);
  tile_piece_store(lds + (t0 & 1) * kRowTileBytes, vraw);
  if (t0 + 1 < t1) vraw = tile_piece_load(rv, t0 + 1);
  float dsum = 0.0f, c = 0.0f;  // the state is e^{c} S
  for (int tau = t0; tau < t1; ++tau) {
    __syncthreads();  // value rows of tile tau staged; the other buffer free
    if (tau + 1 < t1) tile_piece_store(lds + ((tau + 1) & 1) * kRowTileBytes, vraw);
    if (tau + 2 < t1) vraw = tile_piece_load(rv, tau + 2);
    const char *vb = lds + (tau & 1) * kRowTileBytes;
    const float B = lB, cn = c + B;
    const bool full = __any(cn < -kReref);
    const float ks = full ? 0.0f : -cn;
    f32x4 kh;
#pragma unroll
    for (int r = 0; r < 4; ++r) kh[r] = lk[r] * ex(B - lb[r] + ks);
    load(min(tau + 1, t1 - 1));
    dsum += B;
    bf16x4 khh, khl;
    split4(kh, khh, khl);
    if (full) {
      const float e = ex(cn);
#pragma unroll
      for (int s = 0; s < 4; ++s) S[s][0] *= e, S[s][1] *= e;
    }
    c = full ? 0.0f : cn;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x4 vt = tile_tr_half(vb, s, dt);
        S[s][dt] = mma16(vt, khl, mma16(vt, khh, S[s][dt]));
      }
  }
  const size_t base = ((size_t)bh * p.P + seg) * 128 + f;
  const float e = ex(c);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) *(f32x4 *)(p.sloc + base * 128 + 32 * s + 8 * g + 4 * dt) = S[s][dt] * e;
  if (g == 0) p.dseg[base] = dsum;
}

// reverse: G_loc of segment seg from zero, 16 features (ft); D of the last segment
__device__ __forceinline__ void rev_state(const WalkParams &p, int bh, int seg, int ft, char *lds) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int f = 16 * ft + n, L = p.L, nt = (L + 15) / 16;
  const int t0 = seg * p.seg, t1 = min(t0 + p.seg, nt);
  const __amdgpu_buffer_rsrc_t ro = head_rsrc(p.dout, bh, L), rq = frows(p.pq, bh, L), rb = frows(p.gb, bh, L);
  f32x4 G[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s) G[s][0] = G[s][1] = zf4();
  float lq[4], lb[4], lB;
  auto load = [&](int tau) {
    load_f(rq, tau, f, lq);
    load_f(rb, tau, f, lb);
    lB = load_total(rb, tau, f, L);
  };
  u32x4 oraw = tile_piece_load(ro, t1 - 1);
  load(t1 - 1);
  tile_piece_store(lds + ((t1 - 1) & 1) * kRowTileBytes, oraw);
  if (t1 - 2 >= t0) oraw = tile_piece_load(ro, t1 - 2);
  float dsum = 0.0f, c = 0.0f;  // the gradient is e^{c} G
  for (int tau = t1 - 1; tau >= t0; --tau) {
    __syncthreads();  // dO rows of tile tau staged; the other buffer free
    if (tau - 1 >= t0) tile_piece_store(lds + ((tau - 1) & 1) * kRowTileBytes, oraw);
    if (tau - 2 >= t0) oraw = tile_piece_load(ro, tau - 2);
    const char *ob = lds + (tau & 1) * kRowTileBytes;
    const float B = lB, cn = c + B;
    const bool full = __any(cn < -kReref);
    const float qs = full ? 0.0f : -cn;
    f32x4 qb;
#pragma unroll
    for (int r = 0; r < 4; ++r) qb[r] = lq[r] * ex(lb[r] + qs);
    load(max(tau - 1, t0));
    dsum += B;
    bf16x4 qh, ql;
    split4(qb, qh, ql);
    if (full) {
      const float e = ex(cn);
#pragma unroll
      for (int s = 0; s < 4; ++s) G[s][0] *= e, G[s][1] *= e;
    }
    c = full ? 0.0f : cn;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x4 ot = tile_tr_half(ob, s, dt);
        G[s][dt] = mma16(ot, ql, mma16(ot, qh, G[s][dt]));
      }
  }
  const size_t base = ((size_t)bh * p.P + seg) * 128 + f;
  const float e = ex(c);
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) *(f32x4 *)(p.gloc + base * 128 + 32 * s + 8 * g + 4 * dt) = G[s][dt] * e;
  if (g == 0 && seg == p.P - 1) p.dseg[base] = dsum;
}

// Blocks of four waves: the forward states of segments 0 .. P-2 (two blocks a
// segment), then the reverse states of segments 1 .. P-1.
// Blocks are dealt to the 8 XCDs in turn; when the counts allow, the two
// blocks of a segment and direction (which read the same value or dO rows) are
// numbered onto one XCD, each XCD taking a contiguous run of segments.
__global__ __launch_bounds__(256) void bwd_walk_state_kernel(WalkParams p) {
  const int wave = threadIdx.x >> 6, per = 2 * (p.P - 1);
  const int nf = p.BH * per;
  int blk = blockIdx.x;
  const bool rev = blk >= nf;
  if (rev) blk -= nf;
  if (nf % 16 == 0) {
    const int x = blk & 7, l = blk >> 3;
    blk = 2 * (x * (nf / 16) + (l >> 1)) + (l & 1);
  }
  const int bh = blk / per, r = blk - bh * per, seg = r >> 1, ft = 4 * (r & 1) + wave;
  __shared__ __align__(16) char lds[2 * kRowTileBytes];
  if (rev)
    rev_state(p, bh, seg + 1, ft, lds);
  else
    fwd_state(p, bh, seg, ft, lds);
}

// ================================ pass 2 ====================================
// a value-layout operand (lane (n, g): token n, columns 32 s + 8 g .. + 7) read
// from a staged tile
__device__ __forceinline__ bf16x8 tile_val(const char *buf, int s) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  return *(const bf16x8 *)(buf + g * 1024 + (n + 16 * s) * 16);
}

// The forward walks of a segment's block (four waves, 16 features each) share
// the value and dO rows of each tile through LDS as pass 1 does (two buffers of
// both tiles, one barrier a tile).
__device__ __forceinline__ void fwd_walk(const WalkParams &p, int bh, int seg, int ft, char *lds) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int f = 16 * ft + n, L = p.L, nt = (L + 15) / 16;
  const int t0 = seg * p.seg, t1 = min(t0 + p.seg, nt);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v, bh, L), ro = head_rsrc(p.dout, bh, L);
  const __amdgpu_buffer_rsrc_t rq = frows(p.pq, bh, L), rk = frows(p.pk, bh, L), rb = frows(p.gb, bh, L);
  const __amdgpu_buffer_rsrc_t rd = frows(p.dpq, bh, L);
  // S^T tiles (s, dt): rows d_v 32 s + 8 g + 4 dt + r, column f; the state
  // before the segment
  f32x4 ST[4][2];
  const size_t srow = ((size_t)bh * 128 + f) * 128 + 8 * g;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) ST[s][dt] = p.state_in ? *(const f32x4 *)(p.state_in + srow + 32 * s + 4 * dt) : zf4();
  for (int q = 0; q < seg; ++q) {
    const size_t base = ((size_t)bh * p.P + q) * 128 + f;
    const float e = ex(p.dseg[base]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        ST[s][dt] = ST[s][dt] * e + *(const f32x4 *)(p.sloc + base * 128 + 32 * s + 8 * g + 4 * dt);
  }
  // layout-F operands two tiles ahead in a ring of two fixed register sets; the
  // value and dO rows through LDS (buffer tau & 1: value tile, then dO tile)
  float lq[2][4], lk[2][4], lb[2][4], lB[2];
  auto load = [&](int u, int tau) {
    tau = min(tau, t1 - 1);
    load_f(rq, tau, f, lq[u]);
    load_f(rk, tau, f, lk[u]);
    load_f(rb, tau, f, lb[u]);
    lB[u] = load_total(rb, tau, f, L);
  };
  u32x4 vraw = {0u, 0u, 0u, 0u}, oraw = {0u, 0u, 0u, 0u};
  if (t1 > t0) {
    vraw = tile_piece_load(rv, t0);
    oraw = tile_piece_load(ro, t0);
    load(0, t0);
    load(1, t0 + 1);
    tile_piece_store(lds + (t0 & 1) * 2 * kRowTileBytes, vraw);
    tile_piece_store(lds + (t0 & 1) * 2 * kRowTileBytes + kRowTileBytes, oraw);
    if (t0 + 1 < t1) {
      vraw = tile_piece_load(rv, t0 + 1);
      oraw = tile_piece_load(ro, t0 + 1);
    }
  }
  float tqa = 0.0f, c = 0.0f;  // the state is e^{c} ST
  auto step = [&](int u, int tau) {
    __syncthreads();  // rows of tile tau staged; the other buffer free
    if (tau + 1 < t1) {
      char *nb = lds + ((tau + 1) & 1) * 2 * kRowTileBytes;
      tile_piece_store(nb, vraw);
      tile_piece_store(nb + kRowTileBytes, oraw);
    }
    if (tau + 2 < t1) {
      vraw = tile_piece_load(rv, tau + 2);
      oraw = tile_piece_load(ro, tau + 2);
    }
    const char *vb = lds + (tau & 1) * 2 * kRowTileBytes, *ob = vb + kRowTileBytes;
    bf16x8 cv[4], co[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cv[s] = tile_val(vb, s);
      co[s] = tile_val(ob, s);
    }
    const float B = lB[u], mid = 0.5f * B, cn = c + B;
    const bool full = __any(cn < -kReref);
    const float ks = full ? 0.0f : -cn;
    f32x4 fq, eo, kb, ein, kh;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      fq[r] = lq[u][r];
      eo[r] = ex(lb[u][r] - mid);
      kb[r] = lk[u][r] * ex(mid - lb[u][r]);
      ein[r] = ex(lb[u][r] + c);
      kh[r] = lk[u][r] * ex(B - lb[u][r] + ks);
    }
    load(u, tau + 2);
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
    f32x4 ih = zf4(), il = zf4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x4 h0, l0, h1, l1;
      split4(ST[s][0], h0, l0);
      split4(ST[s][1], h1, l1);
      ih = mfma(co[s], join44(h0, h1), ih);
      il = mfma(co[s], join44(l0, l1), il);
    }
    dq += (ih + il) * ein;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      fst(rd, foff(tau, r, f), dq[r]);
      tqa += fq[r] * dq[r];
    }
    if ((tau & 3) == 3 || tau == nt - 1) {
      const float ssum = grp_sum(tqa);
      if (g == 0) p.tq[((size_t)bh * p.nft + (tau >> 2)) * 128 + f] = ssum;
      tqa = 0.0f;
    }
    // S^T <- e^{B} S^T + V^T k-hat (the e^{B} in c, or in a full rescale)
    bf16x4 khh, khl;
    split4(kh, khh, khl);
    if (full) {
      const float e = ex(cn);
#pragma unroll
      for (int s = 0; s < 4; ++s) ST[s][0] *= e, ST[s][1] *= e;
    }
    c = full ? 0.0f : cn;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x4 vt = tile_tr_half(vb, s, dt);
        ST[s][dt] = mma16(vt, khl, mma16(vt, khh, ST[s][dt]));
      }
  };
  for (int tau = t0; tau < t1;) {
    step(0, tau);
    if (++tau >= t1) break;
    step(1, tau);
    ++tau;
  }
  if (seg == p.P - 1 && p.dstate_out) {
    float acc = 0.0f;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) acc += dot4f(ST[s][dt], *(const f32x4 *)(p.dstate_out + srow + 32 * s + 4 * dt));
    acc = grp_sum(acc * ex(c));
    if (g == 0) p.xs[(size_t)bh * 128 + f] = acc;
  }
}

// LDS of a reverse-walk block: each wave's dv part of a tile, double-buffered
// (part[buf][wave][s][dt][lane] as f32x4)
constexpr int kPartBytes = 4 * 4 * 2 * 64 * 16;  // one buffer: 32 KiB
__device__ __forceinline__ unsigned part_off(int buf, int wave, int s, int dt) {
  return (unsigned)(buf * kPartBytes + (((wave * 4 + s) * 2 + dt) * 64 + (int)(threadIdx.x & 63)) * 16);
}

__device__ __forceinline__ void rev_walk(const WalkParams &p, int bh, int seg, char *lds) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4, fs = threadIdx.x >> 6;
  const int L = p.L, nt = (L + 15) / 16;
  const int t0 = seg * p.seg, t1 = min(t0 + p.seg, nt);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(p.v, bh, L), ro = head_rsrc(p.dout, bh, L);
  const __amdgpu_buffer_rsrc_t rq = frows(p.pq, bh, L), rk = frows(p.pk, bh, L), rb = frows(p.gb, bh, L);
  const __amdgpu_buffer_rsrc_t rd = frows(p.dpk, bh, L);
  // the gated part's dv rows: fp32 [L][128] (workspace) or bf16 [L][128]
  const __amdgpu_buffer_rsrc_t rdv =
      p.dv_mode ? __builtin_amdgcn_make_buffer_rsrc((void *)(p.dvo + (size_t)bh * L * 128), (short)0, L * 256, 0x00020000)
                : frows(p.dvg, bh, L);
  // this lane's eight dv columns of a bf16 token row
  const unsigned dvcol = (unsigned)(32 * fs + 8 * g) * 2u;
  const bf16x4 eye = eye16();
  const int fF[2] = {32 * fs + n, 32 * fs + 16 + n};
  // G^T tiles [fa][s][dt]: rows d_v 32 s + 8 g + 4 dt + r, column fF[fa]; the
  // gradient reaching the state after the segment
  f32x4 GT[2][4][2];
#pragma unroll
  for (int fa = 0; fa < 2; ++fa) {
    const size_t srow = ((size_t)bh * 128 + fF[fa]) * 128 + 8 * g;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        GT[fa][s][dt] = p.dstate_out ? *(const f32x4 *)(p.dstate_out + srow + 32 * s + 4 * dt) : zf4();
  }
  for (int q = p.P - 1; q > seg; --q) {
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      const size_t base = ((size_t)bh * p.P + q) * 128 + fF[fa];
      const float e = ex(p.dseg[base]);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          GT[fa][s][dt] = GT[fa][s][dt] * e + *(const f32x4 *)(p.gloc + base * 128 + 32 * s + 8 * g + 4 * dt);
    }
  }
  float lq[2][4], lk[2][4], lb[2][4], lB[2];
  auto load = [&](int tau) {
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      load_f(rq, tau, fF[fa], lq[fa]);
      load_f(rk, tau, fF[fa], lk[fa]);
      load_f(rb, tau, fF[fa], lb[fa]);
      lB[fa] = load_total(rb, tau, fF[fa], L);
    }
  };
  // the value and dO rows of a tile through LDS, after the dv parts (buffer
  // tau & 1: value tile, then dO tile): tile tau - 1 is stored during tile tau,
  // before the tile's barrier, and read after it
  char *const rows = lds + 2 * kPartBytes;
  u32x4 vraw = {0u, 0u, 0u, 0u}, oraw = {0u, 0u, 0u, 0u};
  if (t1 > t0) {
    vraw = tile_piece_load(rv, t1 - 1);
    oraw = tile_piece_load(ro, t1 - 1);
    load(t1 - 1);
    tile_piece_store(rows + ((t1 - 1) & 1) * 2 * kRowTileBytes, vraw);
    tile_piece_store(rows + ((t1 - 1) & 1) * 2 * kRowTileBytes + kRowTileBytes, oraw);
    if (t1 - 2 >= t0) {
      vraw = tile_piece_load(rv, t1 - 2);
      oraw = tile_piece_load(ro, t1 - 2);
    }
  }
  __syncthreads();
  float tka[2] = {0.0f, 0.0f}, c[2] = {0.0f, 0.0f};  // the gradient is e^{c} G^T
  for (int tau = t1 - 1; tau >= t0; --tau) {
    const char *vb = rows + (tau & 1) * 2 * kRowTileBytes, *ob = vb + kRowTileBytes;
    bf16x8 cv[4], co[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      cv[s] = tile_val(vb, s);
      co[s] = tile_val(ob, s);
    }
    if (tau - 1 >= t0) {
      char *nb = rows + ((tau - 1) & 1) * 2 * kRowTileBytes;
      tile_piece_store(nb, vraw);
      tile_piece_store(nb + kRowTileBytes, oraw);
    }
    if (tau - 2 >= t0) {
      vraw = tile_piece_load(rv, tau - 2);
      oraw = tile_piece_load(ro, tau - 2);
    }
    const float cn[2] = {c[0] + lB[0], c[1] + lB[1]};
    const bool full = __any(cn[0] < -kReref || cn[1] < -kReref);
    // this tile's layout-F values (the next tile's loads go into the buffers)
    float cq[2][4], ck[2][4], cb[2][4], cB[2];
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      cB[fa] = lB[fa];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        cq[fa][r] = lq[fa][r];
        ck[fa][r] = lk[fa][r];
        cb[fa][r] = lb[fa][r];
      }
    }
    load(max(tau - 1, t0));
    // M (column t, rows t'): dO_t' . v_t; kept for t' >= t it is M^T in A form
    f32x4 mm = zf4();
#pragma unroll
    for (int s = 0; s < 4; ++s) mm = mfma(co[s], cv[s], mm);
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < n) mm[r] = 0.0f;
    bf16x4 mmh, mml;
    split4(mm, mmh, mml);
    // per feature half: dphik (split operands), then the decayed maps in the
    // forms the rest of the tile takes (token rows over features for A and
    // k-hat, split feature rows for the update); maps meeting G carry its
    // e^{c}, the update's the e^{-c} of the new c
    bf16x4 qrw[2], krw[2], khw[2], qbh[2], qbl[2];
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      const float B = cB[fa], mid = 0.5f * B, qs = full ? 0.0f : -cn[fa];
      f32x4 qp, kp, kh, qb, eo, egk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float b = cb[fa][r], up = ex(b - mid), dn = ex(mid - b), tail = ex(B - b + c[fa]);
        qp[r] = cq[fa][r] * up;
        kp[r] = ck[fa][r] * dn;
        eo[r] = dn;
        egk[r] = tail;
        kh[r] = ck[fa][r] * tail;
        qb[r] = cq[fa][r] * ex(b + qs);
      }
      bf16x4 qph, qpl;
      split4(qp, qph, qpl);
      f32x4 dk = mma16(mmh, qph, zf4());
      dk = mma16(mmh, qpl, dk);
      dk = mma16(mml, qph, dk) * eo;
      f32x4 ih = zf4(), il = zf4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x4 h0, l0, h1, l1;
        split4(GT[fa][s][0], h0, l0);
        split4(GT[fa][s][1], h1, l1);
        ih = mfma(cv[s], join44(h0, h1), ih);
        il = mfma(cv[s], join44(l0, l1), il);
      }
      dk += (ih + il) * egk;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        fst(rd, foff(tau, r, fF[fa]), dk[r]);
        tka[fa] += ck[fa][r] * dk[r];
      }
      qrw[fa] = pack4(mma16(qph, eye, zf4()));
      krw[fa] = to_rows(kp, eye);
      khw[fa] = to_rows(kh, eye);
      split4(qb, qbh[fa], qbl[fa]);
    }
    if ((tau & 3) == 0) {
#pragma unroll
      for (int fa = 0; fa < 2; ++fa) {
        const float ssum = grp_sum(tka[fa]);
        if (g == 0) p.tk[((size_t)bh * p.nft + (tau >> 2)) * 128 + fF[fa]] = ssum;
        tka[fa] = 0.0f;
      }
    }
    const bf16x8 qr = join44(qrw[0], qrw[1]), kr = join44(krw[0], krw[1]), khr = join44(khw[0], khw[1]);
    // A (column t, rows t') over the wave's features, kept for t' >= t
    f32x4 am = mfma(qr, kr, zf4());
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * g + r < n) am[r] = 0.0f;
    const bf16x4 ab = pack4(am);
    const float er[2] = {full ? ex(cn[0]) : 1.0f, full ? ex(cn[1]) : 1.0f};
    const int buf = tau & 1;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        // G^T of this d_v tile as an A operand over features (transposed twice
        // on the matrix core: the bf16 values pass unchanged)
        const bf16x4 g0 = to_rows(GT[0][s][dt], eye);
        const bf16x4 g1 = to_rows(GT[1][s][dt], eye);
        const bf16x4 ot = tile_tr_half(ob, s, dt);  // dO^T half: rows d_v, K tokens
        // the two parts in separate accumulators, added on the VALU: a
        // 16x16x16 product accumulating straight onto a 16x16x32 result read
        // stale accumulator rows (the compiler spaces such a mixed pair as if
        // both had one shape)
        const f32x4 dvt = mfma(join44(g0, g1), khr, zf4()) + mma16(ot, ab, zf4());
        *(f32x4 *)(lds + part_off(buf, fs, s, dt)) = dvt;
#pragma unroll
        for (int fa = 0; fa < 2; ++fa) {
          if (full) GT[fa][s][dt] *= er[fa];
          GT[fa][s][dt] = mma16(ot, qbl[fa], mma16(ot, qbh[fa], GT[fa][s][dt]));
        }
      }
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) c[fa] = full ? 0.0f : cn[fa];
    __syncthreads();
    // this wave's quarter of d_v (s = fs), summed over the four waves' parts
    f32x4 acc[2];
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      acc[dt] = *(const f32x4 *)(lds + part_off(buf, 0, fs, dt));
#pragma unroll
      for (int w = 1; w < 4; ++w) acc[dt] += *(const f32x4 *)(lds + part_off(buf, w, fs, dt));
    }
    if (p.dv_mode == 0) {
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        fst4(rdv, (unsigned)(16 * tau + n) * 512u + (unsigned)(32 * fs + 8 * g + 4 * dt) * 4u, acc[dt]);
    } else {
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack44(acc[0], acc[1])), rdv,
                                             (int)((unsigned)(16 * tau + n) * 256u + dvcol), 0, 0);
    }
  }
  // G after the first tile = Gamma_0 dS_0: the gradient of the initial state,
  // and Gamma_0 (S_in . dS_0) for the gate gradient at token 0
  if (seg == 0) {
#pragma unroll
    for (int fa = 0; fa < 2; ++fa) {
      float acc = 0.0f;
      const float e = ex(c[fa]);
      const size_t srow = ((size_t)bh * 128 + fF[fa]) * 128 + 8 * g;
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const size_t off = srow + 32 * s + 4 * dt;
          const f32x4 gt = GT[fa][s][dt] * e;
          if (p.dstate_in) *(f32x4 *)(p.dstate_in + off) = gt;
          if (p.state_in) acc += dot4f(gt, *(const f32x4 *)(p.state_in + off));
        }
      acc = grp_sum(acc);
      if (g == 0) p.xs[((size_t)p.BH + bh) * 128 + fF[fa]] = acc;
    }
  }
}

// Blocks of four waves: the reverse walks (one block a head and segment) first,
// then the forward walks (two blocks a head and segment).  Two waves a SIMD (a
// few loop-invariant values spill to scratch) and 80 KiB of LDS a block (the
// reverse walks' dv parts, both roles' staged value and dO rows).  When
// the counts allow, the two forward blocks of a segment, which walk the same
// value and dO rows in step, are numbered onto one XCD (blocks are dealt to the
// 8 XCDs in turn; each XCD takes a contiguous run of segments).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_walk_kernel(WalkParams p) {
  __shared__ __align__(16) char lds[2 * kPartBytes + 4 * kRowTileBytes];
  const int nrev = p.BH * p.P;
  int blk = blockIdx.x;
  if (blk < nrev) {
    rev_walk(p, blk / p.P, blk % p.P, lds);
  } else {
    blk -= nrev;
    if (nrev % 8 == 0) {
      const int x = blk & 7, l = blk >> 3;
      blk = 2 * (x * (nrev / 8) + (l >> 1)) + (l & 1);
    }
    const int bh = blk / (2 * p.P), r = blk - bh * 2 * p.P;
    fwd_walk(p, bh, r >> 1, 4 * (r & 1) + (int)(threadIdx.x >> 6), lds);
  }
}

// segments of whole 64-token tiles, at most about kWalkWaves pass-2 waves in all
int walk_segments(int BH, int L, int *seg16) {
  const int nt64 = (L + 63) / 64;
  if (nt64 == 0 || BH <= 0) {
    *seg16 = 4;
    return 1;
  }
  const int want = std::max(1, std::min(nt64, kWalkWaves / (12 * BH)));
  const int seg64 = (nt64 + want - 1) / want;
  *seg16 = 4 * seg64;
  return (nt64 + seg64 - 1) / seg64;
}

}  // namespace

bool bwd_walk_supported(int f, int dv, int L, bool bf16) { return bf16 && f == 128 && dv == 128 && L < (1 << 22); }

size_t bwd_walk_ws_floats(int BH, int L) {
  int seg16 = 0;
  const size_t P = (size_t)walk_segments(BH, L, &seg16);
  return (size_t)BH * P * (2 * 128 * 128 + 128);
}

hipError_t launch_bwd_walk(const WalkArgs &a, hipStream_t stream) {
  WalkParams p;
  p.pq = a.pq; p.pk = a.pk; p.gb = a.gb; p.v = (const bf16 *)a.v; p.dout = (const bf16 *)a.dout;
  p.state_in = a.state_in; p.dstate_out = a.dstate_out;
  p.dpq = a.dpq; p.dpk = a.dpk; p.dvg = a.dvg; p.tq = a.tq; p.tk = a.tk; p.xs = a.xs; p.dstate_in = a.dstate_in;
  p.dvo = (bf16 *)a.dv; p.dv_mode = a.dv_mode;
  p.BH = a.BH; p.L = a.L; p.nft = a.nft;
  if (p.BH == 0) return hipSuccess;
  p.P = walk_segments(p.BH, p.L, &p.seg);
  const size_t nst = (size_t)p.BH * p.P * 128 * 128;
  p.sloc = a.ws;
  p.gloc = a.ws + nst;
  p.dseg = a.ws + 2 * nst;
  if (p.P > 1) {
    hipLaunchKernelGGL(bwd_walk_state_kernel, dim3((unsigned)(4 * p.BH * (p.P - 1))), dim3(256), 0, stream, p);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(bwd_walk_kernel, dim3((unsigned)(3 * p.BH * p.P)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace glah

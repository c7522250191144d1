// bwd_feat.hip -- the per-token part of the layer's backward on the gfx950
// matrix cores: bf16, d = f = d_v = 128, one gate per feature.
//
// From the feature maps phi (the prologue's fp32 [B H L][128]), their gradients
// dphi (the state walks) and, when the window part runs, its dq and dk already
// in the output rows (bf16; each is read and then overwritten by the same lane):
//   Hedgehog map ("Lizard" technical summary, gist.science 2507.09025,
//   Methodology A.1): phi = [softmax(u), softmax(-u)], u = x W (W [d][f/2]).
//   The gradient of u is du = phi+ (dphi+ - phi+ . dphi+) - phi- (dphi- -
//   phi- . dphi-) (the softmax Jacobian of each half), so
//     dx = du W^T (+ the window part),  dW += x^T du,
//   and the gate gradient from
//   d log Gamma_t = d log Gamma at the 64-token tile's first token minus the sum
//   over the tile's earlier tokens of phiq . dphiq - phik . dphik (per
//   feature), times d log Gamma / d gate.
// Block = (b, h, span of 16-token sub-tiles), four waves; wave w = (map m =
// w / 2, half = w % 2).  Per sub-tile:
//   phase 1  wave (m, half) forms du and phi . dphi for its half of map m's
//            features (rows over tokens: lane (n, g) holds token n, features
//            16 i + 4 g + r) and leaves them in LDS;
//   phase 2  wave (m, half) adds the two halves' du of map m, then on the
//            matrix cores dx^T for d in [64 half, 64 half + 64) (A = W rows, B
//            = du as hi + lo) and dW rows [64 half, +64) (A = x^T from the
//            value-layout rows transposed by a selection product, B = du
//            turned to feature rows by an identity product, hi + lo); the gate
//            gradient of features [32 w, 32 w + 32) (a scan over the tokens of
//            the sub-tile).
// dv is not touched here: the reverse state walk writes the finished dv.
// The LDS halves are double-buffered: one barrier a sub-tile.  dW leaves as one
// fp32 partial a block ([B H][blocks][d][f/2]).
#include <algorithm>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

typedef __attribute__((ext_vector_type(4))) short s16x4;

constexpr int kFeatBlocks = 512;  // blocks the span aims at (fewer dW partials to sum)

__device__ __forceinline__ f32x4 mma16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c, 0,
                                                   0, 0);
}
__device__ __forceinline__ f32x4 zf4() { return (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ void split4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
  hi = pack4(x);
  f32x4 h;
#pragma unroll
  for (int r = 0; r < 4; ++r) h[r] = (float)hi[r];
  lo = pack4(x - h);
}
__device__ __forceinline__ bf16x4 eye16() {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  bf16x4 e;
#pragma unroll
  for (int r = 0; r < 4; ++r) e[r] = (bf16)(4 * g + r == n ? 1.0f : 0.0f);
  return e;
}
// rows of one head as a buffer (base + byte_off, bytes long): reads past the
// end return 0 and writes there are dropped
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *base, size_t byte_off, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + byte_off), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ f32x4 ld4f(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
__device__ __forceinline__ bf16x4 ld4h(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st4h(__amdgpu_buffer_rsrc_t r, unsigned off, bf16x4 x) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, (int)off, 0, 0);
}

struct FeatParams {
  const bf16 *q, *k, *gate, *wq, *wk;
  const float *pq, *pk, *dpq, *dpk, *ta;        // [B H L][128] x 4, [B H][tiles][128]
  bf16 *dq, *dk, *dg;                           // dq, dk hold the window part on entry (SWA)
  float *wqp, *wkp;                             // [B H][blocks][128][64]
  int H, L, nft, span, nblk, gate_is_log;       // span: 16-token sub-tiles a block (a multiple of 4)
};

// LDS slots, lane-major f32x4 (slot * 64 + lane): du and phi . dphi of
// [buf][map][half][i]
constexpr int kSlots = 2 * 2 * 2 * 4;
__device__ __forceinline__ unsigned slot_off(int buf, int m, int hf, int i) {
  return (unsigned)((((buf * 2 + m) * 2 + hf) * 4 + i) * 64 + (int)(threadIdx.x & 63)) * 16u;
}

template <bool SWA>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_feat_mfma_kernel(FeatParams p) {
  __shared__ __align__(16) char sdu[kSlots * 1024];
  __shared__ __align__(16) char sep[kSlots * 1024];
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  // wave-uniform (SGPR) so the per-map buffer resources are scalar
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), m = wave >> 1, hf = wave & 1;
  const int bh = blockIdx.x / p.nblk, kb = blockIdx.x - bh * p.nblk, h = bh % p.H, L = p.L;
  const int nt16 = (L + 15) / 16, tau0 = kb * p.span, tau1 = min(tau0 + p.span, nt16);
  const size_t row0 = (size_t)bh * L;
  const unsigned rowbytes = (unsigned)L * 512u, hrowbytes = (unsigned)L * 256u;
  // fp32 [L][128] rows of this head, bf16 [L][128] rows
  const __amdgpu_buffer_rsrc_t rph = rows_rsrc(m ? p.pk : p.pq, row0 * 512, rowbytes);
  const __amdgpu_buffer_rsrc_t rdp = rows_rsrc(m ? p.dpk : p.dpq, row0 * 512, rowbytes);
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(m ? p.k : p.q, row0 * 256, hrowbytes);
  // dx rows: the window part's on entry (SWA), the whole gradient on exit
  const __amdgpu_buffer_rsrc_t rdx = rows_rsrc(m ? p.dk : p.dq, row0 * 256, hrowbytes);
  const __amdgpu_buffer_rsrc_t rg = rows_rsrc(p.gate, row0 * 256, hrowbytes);
  const __amdgpu_buffer_rsrc_t rdg = rows_rsrc(p.dg, row0 * 256, hrowbytes);
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  const bf16x4 eye = eye16();
  // W rows d = 64 hf + 16 et + n, features 16 i + 4 g .. + 3: the A operands of
  // dx^T (held for the block)
  bf16x4 wop[4][4];
  {
    const bf16 *w = (m ? p.wk : p.wq) + (size_t)h * 128 * 64;
#pragma unroll
    for (int et = 0; et < 4; ++et)
#pragma unroll
      for (int i = 0; i < 4; ++i) wop[et][i] = *(const bf16x4 *)(w + (64 * hf + 16 * et + n) * 64 + 16 * i + 4 * g);
  }
  // dW tiles [s'][dt][i]: rows d = 32 (2 hf + s') + 8 g + 4 dt + r, column
  // feature 16 i + n
  f32x4 dw[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) dw[a][dt][i] = zf4();
  // gate features of this wave: 32 wave + 16 i' + 4 g + r
  float run[2][4];
  // phase-1 operands of a sub-tile: phi, dphi of token 16 tau + n, features
  // 64 hf + 16 i + 4 g .. + 3
  f32x4 xph[4], xdp[4];
  auto load1 = [&](int tau) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const unsigned off = (unsigned)(16 * tau + n) * 512u + (unsigned)(64 * hf + 16 * i + 4 * g) * 4u;
      xph[i] = ld4f(rph, off);
      xdp[i] = ld4f(rdp, off);
    }
  };
  if (tau1 > tau0) load1(tau0);
  for (int tau = tau0; tau < tau1; ++tau) {
    const int buf = tau & 1;
    const unsigned tok = (unsigned)(16 * tau + n);
    // ---- phase 1: du and phi . dphi of this half
    f32x4 ph[4], dp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ph[i] = xph[i];
      dp[i] = xdp[i];
    }
    // the phase-2 operands, loaded now: x rows (value layout, columns
    // 32 s + 8 g .. + 7 for s = 2 hf, 2 hf + 1), the gates
    bf16x8 xv[2];
#pragma unroll
    for (int a = 0; a < 2; ++a) xv[a] = bload(rx, tok * 256u + 16u * g + 64u * (2 * hf + a));
    bf16x4 gr[2];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) gr[i2] = ld4h(rg, tok * 256u + (unsigned)(32 * wave + 16 * i2 + 4 * g) * 2u);
    if ((tau & 3) == 0) {
      const float *ta = p.ta + ((size_t)bh * p.nft + (tau >> 2)) * 128 + 32 * wave + 4 * g;
#pragma unroll
      for (int i2 = 0; i2 < 2; ++i2) {
        const f32x4 t4 = *(const f32x4 *)(ta + 16 * i2);
#pragma unroll
        for (int r = 0; r < 4; ++r) run[i2][r] = t4[r];
      }
    }
    if (tau + 1 < tau1) load1(tau + 1);
    float sum = 0.0f;
    f32x4 e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[i] = ph[i] * dp[i];
      sum += (e[i][0] + e[i][1]) + (e[i][2] + e[i][3]);
    }
    sum = grp_sum(sum);
    const float sg = hf ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      *(f32x4 *)(sdu + slot_off(buf, m, hf, i)) = ph[i] * (dp[i] - sum) * sg;
      *(f32x4 *)(sep + slot_off(buf, m, hf, i)) = e[i];
    }
    __syncthreads();
    // ---- phase 2: the window part's dx first (added after dW)
    f32x4 sx[4];
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      if (SWA) {
        const bf16x4 h = ld4h(rdx, tok * 256u + (unsigned)(64 * hf + 16 * et + 4 * g) * 2u);
        sx[et] = (f32x4){(float)h[0], (float)h[1], (float)h[2], (float)h[3]};
      } else {
        sx[et] = zf4();
      }
    }
    // du of map m (rows over tokens), hi + lo
    bf16x4 duh[4], dul[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 du = *(const f32x4 *)(sdu + slot_off(buf, m, 0, i)) + *(const f32x4 *)(sdu + slot_off(buf, m, 1, i));
      split4(du, duh[i], dul[i]);
    }
    // dW += x^T du (du turned to feature rows block by block)
    bf16x4 xt[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) xt[a][dt] = pack4(mfma(xv[a], sel[dt], zf4()));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x4 dfh = pack4(mma16(duh[i], eye, zf4())), dfl = pack4(mma16(dul[i], eye, zf4()));
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) dw[a][dt][i] = mma16(xt[a][dt], dfl, mma16(xt[a][dt], dfh, dw[a][dt][i]));
    }
    // dx^T rows d = 64 hf + 16 et + 4 g + r, column token n
#pragma unroll
    for (int et = 0; et < 4; ++et) {
      f32x4 acc = zf4();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc = mma16(wop[et][i], duh[i], acc);
        acc = mma16(wop[et][i], dul[i], acc);
      }
      acc += sx[et];
      st4h(rdx, tok * 256u + (unsigned)(64 * hf + 16 * et + 4 * g) * 2u, pack4(acc));
    }
    // gate gradient of features 32 wave + 16 i2 + 4 g + r
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int hs = wave >> 1, is = 2 * (wave & 1) + i2;
      const f32x4 db = *(const f32x4 *)(sep + slot_off(buf, 0, hs, is)) - *(const f32x4 *)(sep + slot_off(buf, 1, hs, is));
      bf16x4 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float inc = row_scan(db[r]);
        const float dl = run[i2][r] - (inc - db[r]);
        run[i2][r] -= row_bcast15(inc);
        const float gv = (float)gr[i2][r];
        o[r] = (bf16)(p.gate_is_log ? dl : dl * rcp_fast(1.0f + exp_fast(gv)));
      }
      st4h(rdg, tok * 256u + (unsigned)(32 * wave + 16 * i2 + 4 * g) * 2u, o);
    }
  }
  // this block's dW rows
  float *wp = (m ? p.wkp : p.wqp) + ((size_t)bh * p.nblk + kb) * 128 * 64;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) wp[(32 * (2 * hf + a) + 8 * g + 4 * dt + r) * 64 + 16 * i + n] = dw[a][dt][i][r];
}

}  // namespace

bool bwd_feat_mfma_supported(int d, int f, int dv, int L, int gate_mode, bool bf16) {
  return bf16 && d == 128 && f == 128 && dv == 128 && gate_mode == 0 && L < (1 << 22);
}

// sub-tiles a block (a multiple of 4: whole 64-token tiles), about kFeatBlocks blocks
int bwd_feat_span(int BH, int L) {
  const long nt16 = (L + 15) / 16;
  if (BH <= 0 || nt16 == 0) return 4;
  const long per = (BH * nt16 + kFeatBlocks - 1) / kFeatBlocks;
  return (int)std::max(4L, (per + 3) / 4 * 4);
}

hipError_t launch_bwd_feat_mfma(const FeatArgs &a, hipStream_t stream) {
  FeatParams p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.gate = (const bf16 *)a.gate;
  p.wq = (const bf16 *)a.wq; p.wk = (const bf16 *)a.wk;
  p.pq = a.pq; p.pk = a.pk; p.dpq = a.dpq; p.dpk = a.dpk; p.ta = a.ta;
  p.dq = (bf16 *)a.dq; p.dk = (bf16 *)a.dk; p.dg = (bf16 *)a.dg;
  p.wqp = a.wqp; p.wkp = a.wkp;
  p.H = a.H; p.L = a.L; p.nft = a.nft; p.gate_is_log = a.gate_is_log ? 1 : 0;
  p.span = bwd_feat_span(a.BH, a.L);
  p.nblk = (int)(((a.L + 15) / 16 + p.span - 1) / p.span);
  if (a.BH == 0 || a.L == 0) return hipSuccess;
  const dim3 grid((unsigned)(a.BH * p.nblk)), block(256);
  if (a.swa)
    hipLaunchKernelGGL(bwd_feat_mfma_kernel<true>, grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL(bwd_feat_mfma_kernel<false>, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace glah

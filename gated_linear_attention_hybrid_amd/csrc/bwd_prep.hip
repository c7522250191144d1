// bwd_prep.hip -- the backward prologue on the gfx950 matrix cores (bf16,
// d = f = 128): the Hedgehog feature maps of q and k and the in-tile cumsum of
// the floored log-gate that the tile walks of the state read.
//
// Hedgehog map ("Lizard" technical summary, gist.science 2507.09025,
// Methodology A.1): phi(x) = [softmax(x W), softmax(-x W)] with W [d][f/2]
// per head.  Outputs, fp32 [B H L][128]: phi(q), phi(k) and b_t = the sum over
// the 16-token tile up to t of max(log Gamma, -10) (Gamma from a logit or a
// log-gate, one per feature, per token or per head).
// Block = (b, h, span of 16-token sub-tiles), four waves: wave (m, par) =
// (map, parity) takes the map's sub-tiles of its parity.  u^T = W^T x^T comes
// out with the token as the lane (lane (n, g): token n, features 4 g .. + 3 of
// each tile), so the softmax over the 64 features of a half is an in-lane sum
// and a sum over the four lane groups, and phi leaves in 16-byte rows.  W^T's
// operands are built once per block: W rows in the value layout turned by a
// selection product (exact for bf16), two 16-feature halves joined.
#include <algorithm>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kPrepBlocks = 1024;  // blocks the span aims at

__device__ __forceinline__ f32x4 zf4() { return (f32x4){0.0f, 0.0f, 0.0f, 0.0f}; }
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void *base, size_t byte_off, unsigned bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)((const char *)base + byte_off), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x4 ld4h(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}
__device__ __forceinline__ void st4f(__amdgpu_buffer_rsrc_t r, unsigned off, f32x4 x) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, 0);
}

struct PrepParams {
  const bf16 *q, *k, *gate, *wq, *wk;
  float *pq, *pk, *gb;
  int H, L, span, nblk, gate_mode, gate_is_log;
};

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_prep_mfma_kernel(PrepParams p) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), m = wave >> 1, par = wave & 1;
  const int bh = blockIdx.x / p.nblk, kb = blockIdx.x - bh * p.nblk, h = bh % p.H, L = p.L;
  const int nt16 = (L + 15) / 16, tau0 = kb * p.span, tau1 = min(tau0 + p.span, nt16);
  const size_t row0 = (size_t)bh * L;
  const __amdgpu_buffer_rsrc_t rx = rows_rsrc(m ? p.k : p.q, row0 * 256, (unsigned)L * 256u);
  const __amdgpu_buffer_rsrc_t rph = rows_rsrc(m ? p.pk : p.pq, row0 * 512, (unsigned)L * 512u);
  const __amdgpu_buffer_rsrc_t rgb = rows_rsrc(p.gb, row0 * 512, (unsigned)L * 512u);
  // W^T operands a[k][s][dt] (16x16x32 A, K = 32 features of x): row n is u's
  // column j = 32 s + 8 (n / 4) + 4 dt + n % 4, K-slot 8 g + i is x's feature
  // 32 k + 16 (i / 4) + 4 g + i % 4
  bf16x8 a[4][2][2];
  {
    const __amdgpu_buffer_rsrc_t rw = rows_rsrc(m ? p.wk : p.wq, (size_t)h * 128 * 128, 128u * 128u);
    const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // W rows 32 k + n and 32 k + 16 + n, columns 32 s + 8 g .. + 7
        const bf16x8 w0 = bload(rw, (unsigned)(32 * k + n) * 128u + 16u * g + 64u * s);
        const bf16x8 w1 = bload(rw, (unsigned)(32 * k + 16 + n) * 128u + 16u * g + 64u * s);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
          a[k][s][dt] = join44(pack4(mfma(w0, sel[dt], zf4())), pack4(mfma(w1, sel[dt], zf4())));
      }
  }
  // gates of this wave: features 64 m + 16 i + 4 g .. + 3
  __amdgpu_buffer_rsrc_t rg;
  if (p.gate_mode == 1)
    rg = rows_rsrc(p.gate, row0 * 2, (unsigned)L * 2u);
  else if (p.gate_mode == 2)
    rg = rows_rsrc(p.gate, (size_t)h * 2, 2u);
  else
    rg = rows_rsrc(p.gate, row0 * 256, (unsigned)L * 256u);
  for (int tau = tau0 + par; tau < tau1; tau += 2) {
    const unsigned tok = (unsigned)(16 * tau + n);
    // x^T operands: token n, features 32 k + 4 g .. + 3 and 32 k + 16 + 4 g .. + 3
    bf16x8 xb[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      xb[k] = join44(ld4h(rx, tok * 256u + (unsigned)(32 * k + 4 * g) * 2u),
                     ld4h(rx, tok * 256u + (unsigned)(32 * k + 16 + 4 * g) * 2u));
    float gv[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (p.gate_mode == 0) {
        const bf16x4 g4 = ld4h(rg, tok * 256u + (unsigned)(64 * m + 16 * i + 4 * g) * 2u);
#pragma unroll
        for (int r = 0; r < 4; ++r) gv[i][r] = (float)g4[r];
      } else {
        const unsigned off = p.gate_mode == 1 ? tok * 2u : 0u;
        const float x = __builtin_bit_cast(float, (unsigned)__builtin_amdgcn_raw_buffer_load_b16(rg, (int)off, 0, 0)
                                                      << 16);
#pragma unroll
        for (int r = 0; r < 4; ++r) gv[i][r] = x;
      }
    }
    // u^T tiles (s, dt): rows j = 32 s + 8 g + 4 dt + r, column token n
    f32x4 u[2][2];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        f32x4 acc = zf4();
#pragma unroll
        for (int k = 0; k < 4; ++k) acc = mfma(a[k][s][dt], xb[k], acc);
        u[s][dt] = acc;
      }
    float mx = -INFINITY, mn = INFINITY;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mx = fmaxf(mx, u[s][dt][r]);
          mn = fminf(mn, u[s][dt][r]);
        }
    mx = grp_max(mx);
    mn = grp_min(mn);
    f32x4 ep[2][2], en[2][2];
    float zp = 0.0f, zn = 0.0f;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ep[s][dt][r] = exp_fast(u[s][dt][r] - mx);
          en[s][dt][r] = exp_fast(mn - u[s][dt][r]);
          zp += ep[s][dt][r];
          zn += en[s][dt][r];
        }
    zp = grp_sum(zp);
    zn = grp_sum(zn);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const unsigned col = (unsigned)(32 * s + 8 * g + 4 * dt);
        st4f(rph, tok * 512u + col * 4u, ep[s][dt] / zp);
        st4f(rph, tok * 512u + (64u + col) * 4u, en[s][dt] / zn);
      }
    // b: the floored log-gates summed over the sub-tile's tokens up to this one
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f32x4 b4;
#pragma unroll
      for (int r = 0; r < 4; ++r) b4[r] = row_scan(fmaxf(log_gate_from(gv[i][r], p.gate_is_log), -10.0f));
      st4f(rgb, tok * 512u + (unsigned)(64 * m + 16 * i + 4 * g) * 4u, b4);
    }
  }
}

}  // namespace

bool bwd_prep_mfma_supported(int d, int f, int L, bool bf16) { return bf16 && d == 128 && f == 128 && L < (1 << 22); }

hipError_t launch_bwd_prep_mfma(const PrepArgs &a, hipStream_t stream) {
  PrepParams p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.gate = (const bf16 *)a.gate;
  p.wq = (const bf16 *)a.wq; p.wk = (const bf16 *)a.wk;
  p.pq = a.pq; p.pk = a.pk; p.gb = a.gb;
  p.H = a.H; p.L = a.L; p.gate_mode = a.gate_mode; p.gate_is_log = a.gate_is_log ? 1 : 0;
  const long nt16 = (a.L + 15) / 16;
  if (a.BH == 0 || nt16 == 0) return hipSuccess;
  const long per = (a.BH * nt16 + kPrepBlocks - 1) / kPrepBlocks;
  p.span = (int)std::max(2L, (per + 1) / 2 * 2);
  p.nblk = (int)((nt16 + p.span - 1) / p.span);
  hipLaunchKernelGGL(bwd_prep_mfma_kernel, dim3((unsigned)(a.BH * p.nblk)), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace glah

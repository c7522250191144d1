// bwd_window.hip -- gradient of the window part of the hybrid layer on the
// gfx950 matrix cores (bf16 inputs, d = d_v = 128, window <= 64, 64-token
// chunks).
//
// The window part ("Lizard" technical summary, gist.science 2507.09025,
// Methodology A.2) is a softmax over the keys [t - w + 1, t] whose denominator
// also holds e^{t_m} of the meta-memory scalars (sinks with a zero value):
//   P_tj = e^{scale q_t.k_j - lse_t},  o_t = sum_j P_tj v_j.
// Its gradient for the loss sum o . dO, with D_t = dO_t . o_t and
// ds_tj = P_tj (dO_t . v_j - D_t):
//   dq_t = scale sum_j ds_tj k_j,  dk_j = scale sum_t ds_tj q_t,
//   dv_j = sum_t P_tj dO_t,        d t_m = -sum_t e^{t_m - lse_t} D_t.
// One kernel; a block of eight waves walks a run of chunks of one (b, h) with
// the token rows (K, V, Q, dO) of two chunks c, c + 1 in an LDS ring.  Step c:
//   query side of chunk c + 1   wave w scores query tile w % 4 of chunk c + 1
//                               against the five key tiles that reach it (in
//                               chunks c and c + 1), takes the softmax with the
//                               sinks, leaves lse and D in LDS and forms
//                               dq^T = K^T ds^T for half the d rows (w / 4)
//   key side of chunk c         wave w recomputes P for key tile w % 4 of chunk
//                               c against the five query tiles that reach it
//                               (chunks c and c + 1, with their lse and D) and
//                               forms dv^T = dO^T P and dk^T = Q^T ds for half
//                               the d rows; dv is either written or added to
//                               the bf16 dv already in its rows (the gated
//                               part's)
// while the rows of chunk c + 2 are loaded into registers, to replace chunk c
// in the ring at the end of the step.  Each run starts one step early (the
// query side of its first chunk) and ends with the query side of the next
// run's first chunk (for its lse and D only), so every input row is read once
// plus one chunk a run.
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation; P and ds enter
// as bf16 operands.  The transposed operands (K^T, Q^T, dO^T: four tokens of
// one feature per lane) are read from the staged rows with gfx950's
// transposing LDS read.
#include <algorithm>

#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kWNT = 512;         // eight waves
// One block a compute unit (the ring takes 130 KiB of LDS); blocks of as many
// chunks as fill the chip once run fastest: at 32K tokens, 32 heads, runs of
// 64 chunks (256 blocks) take 8% less time than runs of 16 (1024 blocks).
constexpr int kRunMax = 64;      // chunks a block at most
constexpr int kWinBlocks = 256;  // blocks the run length aims at

// LDS: the token rows of two chunks (ring slot = chunk % 2) of each tensor, a
// chunk as 4 tiles x 4 fragments (fragment (tile, s), lane (n, g) holding
// x[token 16 tile + n][32 g + 8 s + j]); lse and D of two chunks; the sink
// partials of a chunk's four query tiles.
struct LdsWin {
  static constexpr int kChunk = 16 * kFrag;
  static constexpr int KR = 0;
  static constexpr int VR = KR + 2 * kChunk;
  static constexpr int QR = VR + 2 * kChunk;
  static constexpr int OR = QR + 2 * kChunk;
  static constexpr int LS = OR + 2 * kChunk;      // [slot][lse, D][64] fp32
  static constexpr int MP = LS + 2 * 2 * 64 * 4;  // [query tile][64] fp32
  static constexpr int BYTES = MP + 4 * 64 * 4;
};

// Blocks are dealt to the 8 XCDs in turn (block b to XCD b % 8).  Number the
// runs so that each XCD takes a contiguous run of them: a block reads one chunk
// of each neighbouring run, which its neighbour then finds in the same L2.
__device__ __forceinline__ unsigned xcd_run(unsigned b, unsigned grid) {
  const unsigned x = b & 7, per = grid >> 3, rem = grid & 7;
  return x * per + min(x, rem) + (b >> 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_ptr;

// Transposed half fragment of d tile (s, dt) of row tile tl of a staged chunk
// (`rows`): lane (n, g) gets x[token 16 tl + 4 g + r][32 s + 8 (n / 4) + 4 dt +
// n % 4], r = 0..3, the A operand of a 16x16x16 product over tokens whose row n
// is that feature.  ds_read_b64_tr_b16 hands lane i of each 16-lane row element
// i % 4 of the 8-byte chunks addressed by lanes 4 r + i / 4 of that row (r =
// 0..3), so lane (m, g) addresses token 4 g + m / 4, features 32 s + 8 (m % 4) +
// 4 dt + 0..3.
__device__ __forceinline__ bf16x4 tr_half(const char *rows, int tl, int s, int dt) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const char *p = rows + (tl * 4 + (m & 3)) * kFrag + (4 * g + (m >> 2) + 16 * s) * 16 + 8 * dt;
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(char *)p));
}

// Output row of d tile (s, dt) held by lane (n, g) in slot r of an accumulator
// whose A operand came from tr_half: 32 s + 8 g + 4 dt + r.
__device__ __forceinline__ unsigned dcol(int s, int dt) {
  const unsigned g = (threadIdx.x & 63) >> 4;
  return 32 * s + 8 * g + 4 * dt;
}

struct WinBwd {
  const bf16 *q, *k, *v, *dout;
  const float *meta;
  float *mp;  // [B H][chunks][n_meta]: the sink gradient, one partial a chunk
  bf16 *dq, *dk, *dv;
  int H, L, nchunks, run, nruns, window, n_meta, add_dv;
  float scale;
};

__global__ __launch_bounds__(kWNT) void bwd_win_kernel(WinBwd p) {
  using LD = LdsWin;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tw = w & 3, hd = w >> 2;  // the wave's tile in a chunk, its half of d
  const unsigned blk = xcd_run(blockIdx.x, gridDim.x);
  const size_t bh = blk / (unsigned)p.nruns;
  const int run = (int)(blk % (unsigned)p.nruns), h = (int)(bh % p.H);
  const int c0 = run * p.run, c1 = min(c0 + p.run, p.nchunks);
  const unsigned Lu = (unsigned)p.L;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(p.q, bh, p.L), rk = head_rsrc(p.k, bh, p.L),
                               rv = head_rsrc(p.v, bh, p.L), ro = head_rsrc(p.dout, bh, p.L);
  const unsigned rw = row_off(tw);
  auto slot = [&](int cc) { return (cc & 1) * LD::kChunk; };

  // staging: waves 0-3 carry the key and value rows of tile tw of a chunk,
  // waves 4-7 its query and dO rows; rows outside [0, L) read zeros (offsets of
  // chunks before 0 wrap past the range)
  bf16x8 st0[4], st1[4];
  auto fetch = [&](int cc) {
    if (hd == 0) {
      load_rows(rk, rw + chunk_off(cc), st0);
      load_rows(rv, rw + chunk_off(cc), st1);
    } else {
      load_rows(rq, rw + chunk_off(cc), st0);
      load_rows(ro, rw + chunk_off(cc), st1);
    }
  };
  auto stash = [&](int cc) {
    char *b0 = smem + (hd == 0 ? LD::KR : LD::QR) + slot(cc) + tw * 4 * kFrag + lane * 16;
    char *b1 = smem + (hd == 0 ? LD::VR : LD::OR) + slot(cc) + tw * 4 * kFrag + lane * 16;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sts8(b0 + s * kFrag, st0[s]);
      sts8(b1 + s * kFrag, st1[s]);
    }
  };
  fetch(c0 - 1);
  stash(c0 - 1);
  fetch(c0);
  stash(c0);

  // sinks of this head, base 2
  float meta_max = -INFINITY;
  for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, p.meta[(size_t)h * p.n_meta + m] * kLog2e);
  const float sl2 = p.scale * kLog2e;
  const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
  float *lsd = (float *)(smem + LD::LS);
  __syncthreads();

  for (int c = c0 - 1; c < c1; ++c) {
    if (c + 2 <= c1) fetch(c + 2);
    // the dv already in the key side's output rows (loaded early)
    const int jk = c * kC + 16 * tw + n;  // the key side's key
    const bool klive = c >= c0 && jk < p.L;
    const size_t korow = (bh * Lu + (unsigned)min(max(jk, 0), p.L - 1)) * kD;
    bf16x4 dvo[2][2];
    if (p.add_dv && c >= c0) {
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) dvo[si][dt] = *(const bf16x4 *)(p.dv + korow + dcol(2 * hd + si, dt));
    }

    // ---- query side of chunk cq = c + 1: query tile tw, key tiles tw .. tw + 4
    // of chunks c (0-3) and cq (4-7); lane (n, g) holds query n and keys
    // 16 kt + 4 g + r
    {
      const int cq = c + 1, tq = cq * kC + 16 * tw + n;
      bf16x8 xq[4], xo[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xq[s] = lds8(smem + LD::QR + slot(cq) + (tw * 4 + s) * kFrag + lane * 16);
        xo[s] = lds8(smem + LD::OR + slot(cq) + (tw * 4 + s) * kFrag + lane * 16);
      }
      f32x4 sc[5], dp[5];
      float mx = -INFINITY;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int kt = tw + i, kb = slot(c + (kt >> 2)) + (kt & 3) * 4 * kFrag + lane * 16;
        bf16x8 a[4], b[4];
        issue_fence();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a[s] = lds8(smem + LD::KR + kb + s * kFrag);
          b[s] = lds8(smem + LD::VR + kb + s * kFrag);
        }
        issue_fence();
        f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f}, d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          s4 = mfma(a[s], xq[s], s4);
          d4 = mfma(b[s], xo[s], d4);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int j = c * kC + 16 * kt + 4 * g + r;  // key position
          const bool ok = tq < p.L && j >= 0 && j <= tq && tq - j < p.window;
          s4[r] = ok ? s4[r] * sl2 : -INFINITY;
          mx = fmaxf(mx, s4[r]);
        }
        sc[i] = s4;
        dp[i] = d4;
      }
      mx = fmaxf(grp_max(mx), meta_max);
      if (mx == -INFINITY) mx = 0.0f;  // a query past the end: nothing to normalise
      float z = 0.0f;
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[i][r] = exp2_fast(sc[i][r] - mx);  // 2^{-inf} = 0
          z += sc[i][r];
        }
      float meta_sum = 0.0f;
      for (int m = 0; m < p.n_meta; ++m) meta_sum += exp2_fast(p.meta[(size_t)h * p.n_meta + m] * kLog2e - mx);
      z = grp_sum(z) + meta_sum;
      const float iz = z > 0.0f ? rcp_fast(z) : 0.0f;
      float dsum = 0.0f;
#pragma unroll
      for (int i = 0; i < 5; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          sc[i][r] *= iz;  // P
          dsum += sc[i][r] * dp[i][r];
        }
      const float D = grp_sum(dsum);
      const bool live = tq < p.L;
      if (hd == 0) {
        // lse and D for the key side (zeros past the end), the sink gradient
        // -sum_t P_tm D_t over the tile's queries
        if (g == 0) {
          lsd[(cq & 1) * 128 + 16 * tw + n] = live ? (mx + log2_fast(z)) * kLn2 : 0.0f;
          lsd[(cq & 1) * 128 + 64 + 16 * tw + n] = live ? D : 0.0f;
        }
        float *mp = (float *)(smem + LD::MP) + tw * 64;
        for (int m = 0; m < p.n_meta; ++m) {
          float x = (g == 0 && live) ? -exp2_fast(p.meta[(size_t)h * p.n_meta + m] * kLog2e - mx) * iz * D : 0.0f;
          x = grp_sum(x);  // lanes n, n+16, ...: only g = 0 non-zero
          x += dpp_f<0xB1>(x);
          x += dpp_f<0x4E>(x);
          x += dpp_f<0x124>(x);
          x += dpp_f<0x128>(x);  // sum over the 16 queries of the row
          if (lane == 0) mp[m] = x;
        }
      }
      if (cq < c1) {
        // ds as bf16 B operands over key tile pairs (tw, tw+1), (tw+2, tw+3),
        // (tw+4, -); dq^T = K^T ds^T for d tiles (s, dt), s = 2 hd, 2 hd + 1
        bf16x8 dsb[3];
        {
          f32x4 ds[6];
#pragma unroll
          for (int i = 0; i < 5; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) ds[i][r] = sc[i][r] * (dp[i][r] - D);
          ds[5] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int pp = 0; pp < 3; ++pp) dsb[pp] = pack44(ds[2 * pp], ds[2 * pp + 1]);
        }
        const size_t orow = (bh * Lu + (unsigned)min(tq, p.L - 1)) * kD;
#pragma unroll
        for (int si = 0; si < 2; ++si)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) {
            const int s = 2 * hd + si;
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int pp = 0; pp < 3; ++pp) {
              const int k0 = tw + 2 * pp, k1 = k0 + 1;
              const bf16x4 lo = tr_half(smem + LD::KR + slot(c + (k0 >> 2)), k0 & 3, s, dt);
              const bf16x4 hi =
                  k1 < 8 && pp < 2 ? tr_half(smem + LD::KR + slot(c + (k1 >> 2)), k1 & 3, s, dt) : z4;
              acc = mfma(join44(lo, hi), dsb[pp], acc);
            }
            if (live) *(bf16x4 *)(p.dq + orow + dcol(s, dt)) = pack4(acc * p.scale);
          }
      }
    }
    __syncthreads();

    // the chunk's sink gradient (the four tiles' parts in a fixed order)
    if (c + 1 < c1 && tid < p.n_meta) {
      const float *mp = (const float *)(smem + LD::MP);
      const float acc = ((mp[tid] + mp[64 + tid]) + mp[128 + tid]) + mp[192 + tid];
      p.mp[(bh * p.nchunks + (c + 1)) * p.n_meta + tid] = acc;
    }
    // ---- key side of chunk c: key tile tw, query tiles tw .. tw + 4 of chunks
    // c (0-3) and c + 1 (4-7); lane (n, g) holds key n and queries 16 qt + 4 g + r
    if (c >= c0) {
      bf16x8 xk[4], xv[4];
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        xk[s] = lds8(smem + LD::KR + slot(c) + (tw * 4 + s) * kFrag + lane * 16);
        xv[s] = lds8(smem + LD::VR + slot(c) + (tw * 4 + s) * kFrag + lane * 16);
      }
      f32x4 pw[6], ds[6];
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int qt = tw + i, cc = c + (qt >> 2), qb = slot(cc) + (qt & 3) * 4 * kFrag + lane * 16;
        bf16x8 a[4], b[4];
        issue_fence();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a[s] = lds8(smem + LD::QR + qb + s * kFrag);
          b[s] = lds8(smem + LD::OR + qb + s * kFrag);
        }
        issue_fence();
        f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f}, d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          s4 = mfma(a[s], xk[s], s4);
          d4 = mfma(b[s], xv[s], d4);
        }
        const float *ls = lsd + (cc & 1) * 128 + 16 * (qt & 3) + 4 * g;
        const f32x4 l4 = *(const f32x4 *)ls, e4 = *(const f32x4 *)(ls + 64);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = c * kC + 16 * qt + 4 * g + r;  // query position
          const bool ok = jk < p.L && t < p.L && t >= jk && t - jk < p.window;
          const float pr = ok ? exp_fast(s4[r] * p.scale - l4[r]) : 0.0f;
          pw[i][r] = pr;
          ds[i][r] = pr * (d4[r] - e4[r]);
        }
      }
      pw[5] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
      ds[5] = pw[5];
      bf16x8 pb[3], db[3];
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
        pb[pp] = pack44(pw[2 * pp], pw[2 * pp + 1]);
        db[pp] = pack44(ds[2 * pp], ds[2 * pp + 1]);
      }
      // dv^T = dO^T P, dk^T = Q^T ds: d tile (s, dt), lane (n, g) holds key n
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) {
          const int s = 2 * hd + si;
          f32x4 av = {0.0f, 0.0f, 0.0f, 0.0f}, ak = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int pp = 0; pp < 3; ++pp) {
            const int q0 = tw + 2 * pp, q1 = q0 + 1;
            const bool h1 = q1 < 8 && pp < 2;
            const int o0 = slot(c + (q0 >> 2)), o1 = slot(c + (q1 >> 2));
            const bf16x4 olo = tr_half(smem + LD::OR + o0, q0 & 3, s, dt);
            const bf16x4 ohi = h1 ? tr_half(smem + LD::OR + o1, q1 & 3, s, dt) : z4;
            const bf16x4 qlo = tr_half(smem + LD::QR + o0, q0 & 3, s, dt);
            const bf16x4 qhi = h1 ? tr_half(smem + LD::QR + o1, q1 & 3, s, dt) : z4;
            av = mfma(join44(olo, ohi), pb[pp], av);
            ak = mfma(join44(qlo, qhi), db[pp], ak);
          }
          if (klive) {
            if (p.add_dv) {
#pragma unroll
              for (int r = 0; r < 4; ++r) av[r] += (float)dvo[si][dt][r];
            }
            *(bf16x4 *)(p.dv + korow + dcol(s, dt)) = pack4(av);
            *(bf16x4 *)(p.dk + korow + dcol(s, dt)) = pack4(ak * p.scale);
          }
        }
    }
    __syncthreads();
    // chunk c + 2 takes chunk c's place in the ring
    if (c + 2 <= c1) stash(c + 2);
    __syncthreads();
  }
}

}  // namespace

bool bwd_window_mfma_supported(int d, int dv, int window, int n_meta, bool bf16) {
  return bf16 && d == kD && dv == kDV && window >= 1 && window <= kC && n_meta <= 64;
}

hipError_t launch_bwd_window_mfma(const WinBwdArgs &a, hipStream_t stream) {
  const size_t BH = (size_t)a.B * a.H;
  if (BH * a.L == 0) return hipSuccess;
  WinBwd p;
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.v = (const bf16 *)a.v; p.dout = (const bf16 *)a.dout;
  p.meta = a.meta; p.mp = a.mp;
  p.dq = (bf16 *)a.dq; p.dk = (bf16 *)a.dk; p.dv = (bf16 *)a.dv; p.add_dv = a.add_dv ? 1 : 0;
  p.H = a.H; p.L = a.L; p.window = a.window; p.n_meta = a.n_meta; p.scale = a.scale;
  p.nchunks = (a.L + kC - 1) / kC;
  // chunks a block: about kWinBlocks blocks (each walks its run one chunk at a
  // time and reads one extra chunk a run)
  const size_t want = (BH * (size_t)p.nchunks + kWinBlocks - 1) / kWinBlocks;
  p.run = (int)std::min<size_t>(std::max<size_t>(want, 1), kRunMax);
  p.nruns = (p.nchunks + p.run - 1) / p.run;
  const size_t grid = BH * (size_t)p.nruns;
  if (grid > 0x7fffffffu) return hipErrorInvalidValue;
  hipError_t e = hipFuncSetAttribute((const void *)bwd_win_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     LdsWin::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_win_kernel, dim3((unsigned)grid), dim3(kWNT), LdsWin::BYTES, stream, p);
  return hipGetLastError();
}

}  // namespace glah

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
// Two kernels, one block of four waves per (b, h, 64-token chunk):
//   query kernel  wave w owns query tile w (16 queries); it scores the five
//                 key tiles that reach it (tiles w .. w + 4 of the previous and
//                 this chunk), takes the softmax with the sinks, writes lse and
//                 D, and forms dq^T = K^T ds^T
//   key kernel    wave w owns key tile w; with the query kernel's lse and D it
//                 recomputes P for the five query tiles that reach it (this and
//                 the next chunk), and forms dv^T = dO^T P and dk^T = Q^T ds;
//                 dv is either written or added to the bf16 dv already in its
//                 rows (the gated part's)
// Every product is a 16x16x32 bf16 MFMA with fp32 accumulation; P and ds enter
// as bf16 operands.  The token rows are staged in LDS once; the transposed
// operands (K^T, Q^T, dO^T: four tokens of one feature per lane) are read from
// those rows with gfx950's transposing LDS read, so a block needs 65 KiB and
// two blocks share a compute unit.
#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kWNT = 256;  // four waves

struct LdsWinQ {
  static constexpr int KR = 0;                // key rows [8 tiles][4 s] (previous chunk tiles 0-3, this chunk 0-3)
  static constexpr int VR = KR + 32 * kFrag;  // value rows, same
  static constexpr int MP = VR + 32 * kFrag;  // sink gradient partials [4 waves][64]
  static constexpr int BYTES = MP + 4 * 64 * 4;
};

struct LdsWinK {
  static constexpr int QR = 0;                // query rows [8 tiles][4 s] (this chunk tiles 0-3, next chunk 0-3)
  static constexpr int OR = QR + 32 * kFrag;  // dO rows, same
  static constexpr int LS = OR + 32 * kFrag;  // lse and D of the 128 queries [2][128] fp32
  static constexpr int BYTES = LS + 2 * 128 * 4;
};

// Blocks are dealt to the 8 XCDs in turn (block b to XCD b % 8).  Number the
// chunks so that each XCD takes a contiguous run of them: a block reads the rows
// of its neighbouring chunk too, which its neighbour then finds in the same L2.
__device__ __forceinline__ unsigned xcd_run(unsigned b, unsigned grid) {
  const unsigned x = b & 7, per = grid >> 3, rem = grid & 7;
  return x * per + min(x, rem) + (b >> 3);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 *lds_s16x4_ptr;

// Transposed half fragment of d tile (s, dt) of row tile tl, from token rows
// staged as load_rows lays them (fragment (tl, s'), lane (n, g) holding
// x[token 16 tl + n][32 g + 8 s' + j]): lane (n, g) gets
// x[token 16 tl + 4 g + r][32 s + 8 (n / 4) + 4 dt + n % 4], r = 0..3, the A
// operand of a 16x16x16 product over tokens whose row n is that feature.
// ds_read_b64_tr_b16 hands lane i of each 16-lane row element i % 4 of the
// 8-byte chunks addressed by lanes 4 r + i / 4 of that row (r = 0..3), so lane
// (m, g) addresses token 4 g + m / 4, features 32 s + 8 (m % 4) + 4 dt + 0..3.
__device__ __forceinline__ bf16x4 tr_half(const char *rows, int tl, int s, int dt) {
  const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
  const char *p = rows + (tl * 4 + (m & 3)) * kFrag + (4 * g + (m >> 2) + 16 * s) * 16 + 8 * dt;
  return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_ptr)(char *)p));
}

// Output row of d tile (s, dt) held by lane (n, g) in slot r of an accumulator
// whose A operand came from stage_transposed: 32 s + 8 g + 4 dt + r.
__device__ __forceinline__ unsigned dcol(int s, int dt) {
  const unsigned g = (threadIdx.x & 63) >> 4;
  return 32 * s + 8 * g + 4 * dt;
}

struct WinBwdQ {
  const bf16 *q, *k, *v, *dout;
  const float *meta;
  float *lse, *del, *mp;
  bf16 *dq;
  int H, L, nchunks, window, n_meta, nsb;
  float scale;
};

// ============================== query kernel ================================
__global__ __launch_bounds__(kWNT) void bwd_win_q_kernel(WinBwdQ p) {
  using LD = LdsWinQ;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned blk = xcd_run(blockIdx.x, gridDim.x);
  const size_t bh = blk / p.nchunks;
  const int c = blk % p.nchunks;
  const int h = (int)(bh % p.H);
  const unsigned Lu = (unsigned)p.L;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(p.q, bh, p.L), rk = head_rsrc(p.k, bh, p.L),
                               rv = head_rsrc(p.v, bh, p.L), ro = head_rsrc(p.dout, bh, p.L);
  const unsigned rw = row_off(w);

  // stage key and value rows of tile w of the previous chunk (ci = 0) and of
  // this chunk (ci = 1); rows before 0 read zeros (offsets wrap past the range)
  // and are masked below
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    bf16x8 xk[4], xv[4];
    load_rows(rk, rw + chunk_off(c - 1 + ci), xk);
    load_rows(rv, rw + chunk_off(c - 1 + ci), xv);
    const int tl = 4 * ci + w;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sts8(smem + LD::KR + (tl * 4 + s) * kFrag + lane * 16, xk[s]);
      sts8(smem + LD::VR + (tl * 4 + s) * kFrag + lane * 16, xv[s]);
    }
  }
  bf16x8 xq[4], xo[4];
  load_rows(rq, rw + chunk_off(c), xq);
  load_rows(ro, rw + chunk_off(c), xo);
  // sinks of this head, base 2
  float meta_max = -INFINITY, meta_sum = 0.0f;
  for (int m = 0; m < p.n_meta; ++m) meta_max = fmaxf(meta_max, p.meta[(size_t)h * p.n_meta + m] * kLog2e);
  __syncthreads();

  // scores S^T and dP^T for key tiles w .. w + 4 (index in [0, 8)): lane (n, g)
  // holds query n of tile w and keys 16 kt + 4 g + r
  const int tq = c * kC + 16 * w + n;  // this lane's query
  const float sl2 = p.scale * kLog2e;
  f32x4 sc[5], dp[5];
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int kt = w + i;
    bf16x8 a[4], b[4];
    issue_fence();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = lds8(smem + LD::KR + (kt * 4 + s) * kFrag + lane * 16);
      b[s] = lds8(smem + LD::VR + (kt * 4 + s) * kFrag + lane * 16);
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
      const int j = c * kC - kC + 16 * kt + 4 * g + r;  // key position
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
  if (g == 0 && live) {
    p.lse[bh * Lu + tq] = (mx + log2_fast(z)) * kLn2;
    p.del[bh * Lu + tq] = D;
  }
  // sink gradient: -sum_t P_tm D_t over this wave's queries (lanes g = 0)
  {
    float *mp = (float *)(smem + LD::MP) + w * 64;
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
  // ds as bf16 B operands over key tile pairs (w, w+1), (w+2, w+3), (w+4, -)
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
  // dq^T = K^T ds^T: d tile (s, dt), lane (n, g) holds query n, d rows dcol + r
  const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
  const unsigned orow = (bh * Lu + (unsigned)min(tq, p.L - 1)) * kD;
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
        const int k0 = w + 2 * pp, k1 = k0 + 1;
        const bf16x4 lo = tr_half(smem + LD::KR, k0, s, dt);
        const bf16x4 hi = k1 < 8 && pp < 2 ? tr_half(smem + LD::KR, k1, s, dt) : z4;
        acc = mfma(join44(lo, hi), dsb[pp], acc);
      }
      if (live) *(bf16x4 *)(p.dq + orow + dcol(s, dt)) = pack4(acc * p.scale);
    }
  __syncthreads();
  // the chunk's sink gradient (the four waves' parts in a fixed order): one
  // partial a chunk (nsb = chunks)
  if (tid < p.n_meta) {
    float acc = 0.0f;
    for (int ww = 0; ww < 4; ++ww) acc += ((const float *)(smem + LD::MP))[ww * 64 + tid];
    p.mp[(bh * p.nsb + c) * p.n_meta + tid] = acc;
  }
}

struct WinBwdK {
  const bf16 *q, *k, *v, *dout;
  const float *lse, *del;
  bf16 *dk, *dv;
  int L, nchunks, window, add_dv;  // add_dv: dv += this part (else dv = it)
  float scale;
};

// =============================== key kernel =================================
__global__ __launch_bounds__(kWNT) void bwd_win_k_kernel(WinBwdK p) {
  using LD = LdsWinK;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const unsigned blk = xcd_run(blockIdx.x, gridDim.x);
  const size_t bh = blk / p.nchunks;
  const int c = blk % p.nchunks;
  const unsigned Lu = (unsigned)p.L;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc(p.q, bh, p.L), rk = head_rsrc(p.k, bh, p.L),
                               rv = head_rsrc(p.v, bh, p.L), ro = head_rsrc(p.dout, bh, p.L);
  const unsigned rw = row_off(w);

  // stage query and dO rows of tile w of this chunk (ci = 0) and of the next
  // one (ci = 1); rows past the end read zeros
#pragma unroll
  for (int ci = 0; ci < 2; ++ci) {
    bf16x8 xq[4], xo[4];
    load_rows(rq, rw + chunk_off(c + ci), xq);
    load_rows(ro, rw + chunk_off(c + ci), xo);
    const int tl = 4 * ci + w;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      sts8(smem + LD::QR + (tl * 4 + s) * kFrag + lane * 16, xq[s]);
      sts8(smem + LD::OR + (tl * 4 + s) * kFrag + lane * 16, xo[s]);
    }
  }
  if (tid < 128) {
    const int t = c * kC + tid;
    const unsigned tc = (unsigned)min(t, p.L - 1);
    const float ls = p.lse[bh * Lu + tc], de = p.del[bh * Lu + tc];
    float *ld = (float *)(smem + LD::LS);
    ld[tid] = t < p.L ? ls : 0.0f;
    ld[128 + tid] = t < p.L ? de : 0.0f;
  }
  bf16x8 xk[4], xv[4];
  load_rows(rk, rw + chunk_off(c), xk);
  load_rows(rv, rw + chunk_off(c), xv);
  const int jk = c * kC + 16 * w + n;  // this lane's key
  const bool live = jk < p.L;
  const unsigned orow = (bh * Lu + (unsigned)min(jk, p.L - 1)) * kD;
  // the dv already in the output rows, to add to (loaded early)
  bf16x4 dvo[4][2];
  if (p.add_dv) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) dvo[s][dt] = *(const bf16x4 *)(p.dv + orow + dcol(s, dt));
  }
  __syncthreads();

  // S and dP for query tiles w .. w + 4 (index in [0, 8)): lane (n, g) holds
  // key n of tile w and queries 16 qt + 4 g + r
  const float *lse = (const float *)(smem + LD::LS), *del = lse + 128;
  f32x4 pw[6], ds[6];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int qt = w + i;
    bf16x8 a[4], b[4];
    issue_fence();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      a[s] = lds8(smem + LD::QR + (qt * 4 + s) * kFrag + lane * 16);
      b[s] = lds8(smem + LD::OR + (qt * 4 + s) * kFrag + lane * 16);
    }
    issue_fence();
    f32x4 s4 = {0.0f, 0.0f, 0.0f, 0.0f}, d4 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      s4 = mfma(a[s], xk[s], s4);
      d4 = mfma(b[s], xv[s], d4);
    }
    const f32x4 l4 = *(const f32x4 *)(lse + 16 * qt + 4 * g), e4 = *(const f32x4 *)(del + 16 * qt + 4 * g);
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
  const bf16x4 z4 = {(bf16)0.0f, (bf16)0.0f, (bf16)0.0f, (bf16)0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      f32x4 av = {0.0f, 0.0f, 0.0f, 0.0f}, ak = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int pp = 0; pp < 3; ++pp) {
        const int q0 = w + 2 * pp, q1 = q0 + 1;
        const bool h1 = q1 < 8 && pp < 2;
        const bf16x4 olo = tr_half(smem + LD::OR, q0, s, dt);
        const bf16x4 ohi = h1 ? tr_half(smem + LD::OR, q1, s, dt) : z4;
        const bf16x4 qlo = tr_half(smem + LD::QR, q0, s, dt);
        const bf16x4 qhi = h1 ? tr_half(smem + LD::QR, q1, s, dt) : z4;
        av = mfma(join44(olo, ohi), pb[pp], av);
        ak = mfma(join44(qlo, qhi), db[pp], ak);
      }
      if (live) {
        if (p.add_dv) {
#pragma unroll
          for (int r = 0; r < 4; ++r) av[r] += (float)dvo[s][dt][r];
        }
        *(bf16x4 *)(p.dv + orow + dcol(s, dt)) = pack4(av);
        *(bf16x4 *)(p.dk + orow + dcol(s, dt)) = pack4(ak * p.scale);
      }
    }
}

}  // namespace

bool bwd_window_mfma_supported(int d, int dv, int window, int n_meta, bool bf16) {
  return bf16 && d == kD && dv == kDV && window >= 1 && window <= kC && n_meta <= 64;
}

hipError_t launch_bwd_window_mfma(const WinBwdArgs &a, hipStream_t stream) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  const int nchunks = (a.L + kC - 1) / kC;
  const unsigned grid = (unsigned)((size_t)a.B * a.H * nchunks);
  WinBwdQ pq;
  pq.q = (const bf16 *)a.q; pq.k = (const bf16 *)a.k; pq.v = (const bf16 *)a.v; pq.dout = (const bf16 *)a.dout;
  pq.meta = a.meta; pq.lse = a.lse; pq.del = a.del; pq.dq = (bf16 *)a.dq; pq.mp = a.mp;
  pq.H = a.H; pq.L = a.L; pq.nchunks = nchunks; pq.window = a.window; pq.n_meta = a.n_meta; pq.nsb = a.nsb;
  pq.scale = a.scale;
  hipError_t e = hipFuncSetAttribute((const void *)bwd_win_q_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     LdsWinQ::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_win_q_kernel, dim3(grid), dim3(kWNT), LdsWinQ::BYTES, stream, pq);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  WinBwdK pk;
  pk.q = pq.q; pk.k = pq.k; pk.v = pq.v; pk.dout = pq.dout; pk.lse = a.lse; pk.del = a.del;
  pk.dk = (bf16 *)a.dk; pk.dv = (bf16 *)a.dv; pk.add_dv = a.add_dv ? 1 : 0; pk.L = a.L; pk.nchunks = nchunks; pk.window = a.window; pk.scale = a.scale;
  e = hipFuncSetAttribute((const void *)bwd_win_k_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, LdsWinK::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_win_k_kernel, dim3(grid), dim3(kWNT), LdsWinK::BYTES, stream, pk);
  return hipGetLastError();
}

}  // namespace glah

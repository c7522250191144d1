// swa_wide.hip -- sliding-window softmax attention with meta-memory sinks for
// any window (bf16 inputs, fp32 accumulation, d = d_v = 128) on the gfx950
// matrix cores, with an online softmax over 64-key chunks.
//
// Method ("Lizard" technical summary, gist.science 2507.09025, Methodology
// A.2): the query at position t attends to the keys [t - w + 1, t], and the
// meta-memory scalars t_m add e^{t_m} to the softmax denominator (sinks with a
// zero value).  The window kernels inside the chunked prefill take the whole
// band of a 64-query chunk at once (w <= 64: two key chunks); this kernel
// serves wider windows.  The running maximum and denominator start from the
// sinks (m = max_m t_m, l = sum_m e^{t_m - m}), so the sinks are counted once,
// whatever the number of key chunks; every later chunk rescales the
// accumulator by 2^{m_old - m_new} (base-2 scores).
//
// Block = one 64-query chunk of one (b, h), 4 waves; wave w owns query tile w
// (16 queries) and all 128 value columns.  Per key chunk each wave stages key
// tile w (raw key fragments, and V^T half fragments transposed on the matrix
// core) into one of two LDS buffers, then every wave scores its queries
// against the chunk's 64 keys (S^T = K Q^T: lane = query, 4 keys per lane and
// tile), updates its softmax statistics and accumulates O^T += V^T P^T.  The
// next chunk's key and value rows are loaded into registers while the current
// chunk is computed; one barrier per chunk.
#include "chunk_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kNTW = 256;

struct LdsWide {
  static constexpr int RK = 0;                  // raw k frags [4 tile][4 s]
  static constexpr int VT = RK + 16 * kFrag;    // V^T half frags [4 tile][8 (s, dt)]
  static constexpr int BUF = VT + 32 * kHalf;   // one key chunk
  static constexpr int BYTES = 2 * BUF;
};

// ACC: o += o_swa (the hybrid layer after the gated part), else o = o_swa.
template <bool ACC>
__global__ __launch_bounds__(kNTW) void swa_wide_kernel(ChunkParams p) {
  using LD = LdsWide;
  extern __shared__ __align__(16) char smem[];
  const int tid = threadIdx.x, lane = tid & 63, n = lane & 15, g = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const size_t bh = blockIdx.x / p.nchunks;
  const int c = blockIdx.x % p.nchunks;
  const int h = (int)(bh % p.H);
  const HeadBufs hb = head_bufs(p, bh);
  const unsigned ro = row_off(wave);
  const bf16x8 sel[2] = {select_operand(0), select_operand(1)};
  const int w = p.window;
  // key chunks that reach this query chunk: keys from 64c - w + 1 (or 0) up to
  // the chunk's last query
  const int first_key = max(0, c * kC - w + 1);
  const int kc_lo = first_key / kC;
  const int tq = c * kC + 16 * wave + n;  // this lane's query position

  // stage key tile `wave` of key chunk kc (rows from registers) into buffer b
  auto stage = [&](const bf16x8 *xk, const bf16x8 *xv, int b) {
    char *base = smem + b * LD::BUF;
#pragma unroll
    for (int s = 0; s < 4; ++s) sts8(base + LD::RK + (wave * 4 + s) * kFrag + lane * 16, xk[s]);
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        *(bf16x4 *)(base + LD::VT + (wave * 8 + 2 * s + dt) * kHalf + lane * 8) =
            pack4(mfma(xv[s], sel[dt], (f32x4){0.0f, 0.0f, 0.0f, 0.0f}));
  };

  bf16x8 xq[4], xk[4], xv[4];
  load_rows(hb.q, ro + chunk_off(c), xq);
  load_rows(hb.k, ro + chunk_off(kc_lo), xk);
  load_vals(hb.v, ro + chunk_off(kc_lo), xv);
  // softmax statistics of this lane's query, base 2, seeded by the sinks; a
  // finite start without sinks so 2^{m_old - m_new} is never (-inf) - (-inf)
  float m_run = -1.0e30f, l_run = 0.0f;
  if (p.n_meta > 0) {
    const float *meta = p.meta + (size_t)h * p.n_meta;
    float mm = -INFINITY;
    for (int m = 0; m < p.n_meta; ++m) mm = fmaxf(mm, meta[m] * kLog2e);
    float ss = 0.0f;
    for (int m = 0; m < p.n_meta; ++m) ss += exp2_fast(meta[m] * kLog2e - mm);
    m_run = mm;
    l_run = ss;
  }
  const float sl2 = p.scale * kLog2e;
  // O^T accumulators: O[s][dt] holds columns 32 s + 8 g + 4 dt + r (r = 0..3)
  // of query n of this wave's tile
  f32x4 O[4][2];
#pragma unroll
  for (int s = 0; s < 4; ++s)
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) O[s][dt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};

  stage(xk, xv, 0);
  for (int kc = kc_lo; kc <= c; ++kc) {
    const int b = (kc - kc_lo) & 1;
    if (kc < c) {  // the next chunk's rows, in flight during this chunk
      load_rows(hb.k, ro + chunk_off(kc + 1), xk);
      load_vals(hb.v, ro + chunk_off(kc + 1), xv);
    }
    __syncthreads();  // buffer b staged by every wave; buffer b ^ 1 free
    const char *base = smem + b * LD::BUF;
    // scores S^T for key tiles 0..3: lane (n, g) holds keys 16 kt + 4 g + r
    f32x4 sc[4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      bf16x8 a[4];
      issue_fence();
#pragma unroll
      for (int s = 0; s < 4; ++s) a[s] = lds8(base + LD::RK + (kt * 4 + s) * kFrag + lane * 16);
      issue_fence();
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s) acc = mfma(a[s], xq[s], acc);
      sc[kt] = acc;
    }
    // window mask: query minus key position in [0, w) (one unsigned compare);
    // keys before 0 do not occur (kc >= 0), keys past the end only meet
    // queries before them
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const unsigned back = (unsigned)(tq - (kc * kC + 16 * kt + 4 * g + r));
        sc[kt][r] = back < (unsigned)w ? sc[kt][r] * sl2 : -INFINITY;
        mx = fmaxf(mx, sc[kt][r]);
      }
    const float m_new = fmaxf(m_run, grp_max(mx));
    const float alpha = exp2_fast(m_run - m_new);
    float sum = 0.0f;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sc[kt][r] = exp2_fast(sc[kt][r] - m_new);  // 2^{-inf} = 0
        sum += sc[kt][r];
      }
    l_run = l_run * alpha + grp_sum(sum);
    m_run = m_new;
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) O[s][dt] *= alpha;
    // O^T += V^T P^T over the two 32-key steps (tiles 0,1 and 2,3)
    const bf16x8 pf[2] = {pack44(sc[0], sc[1]), pack44(sc[2], sc[3])};
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const char *vb = base + LD::VT + ((2 * ks) * 8 + 2 * s + dt) * kHalf + lane * 8;
          const bf16x8 a = join44(*(const bf16x4 *)vb, *(const bf16x4 *)(vb + 8 * kHalf));
          O[s][dt] = mfma(a, pf[ks], O[s][dt]);
        }
    if (kc < c) stage(xk, xv, b ^ 1);
  }
  // o = O / l (plus the gated part already in o); rows past the end are
  // dropped by the range check of the buffer stores
  const float inv = rcp_fast(l_run);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const unsigned off = chunk_off(c) + (unsigned)(16 * wave + n) * (kDV * 2) + 64 * s + 16 * g;
    f32x4 lo = O[s][0] * inv, hi = O[s][1] * inv;
    if (ACC) {
      const bf16x8 prev = bload(hb.o, off);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        lo[r] += (float)prev[r];
        hi[r] += (float)prev[4 + r];
      }
    }
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, pack44(lo, hi)), hb.o, (int)off, 0, 0);
  }
}

}  // namespace

bool swa_wide_supported(const LayerArgs &a) {
  return a.bf16 && a.d == kD && a.dv == kDV && a.window >= 1;
}

hipError_t launch_swa_wide(const LayerArgs &a, bool accumulate) {
  if ((size_t)a.B * a.H * a.L == 0) return hipSuccess;
  const int nchunks = (a.L + kC - 1) / kC;
  ChunkParams p = {};
  p.q = (const bf16 *)a.q; p.k = (const bf16 *)a.k; p.v = (const bf16 *)a.v;
  p.gate = (const bf16 *)a.q;  // unused (the buffer resources need a valid base)
  p.meta = a.meta; p.o = (bf16 *)a.o;
  p.B = a.B; p.H = a.H; p.L = a.L; p.window = a.window; p.n_meta = a.n_meta;
  p.nchunks = nchunks; p.P = 1; p.seg_chunks = nchunks; p.R = 1; p.sub_chunks = nchunks;
  p.scale = a.scale; p.gate_mode = 0;
  const void *fn = accumulate ? (const void *)swa_wide_kernel<true> : (const void *)swa_wide_kernel<false>;
  hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, LdsWide::BYTES);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((size_t)a.B * a.H * nchunks)), block(kNTW);
  if (accumulate)
    hipLaunchKernelGGL(swa_wide_kernel<true>, grid, block, LdsWide::BYTES, a.stream, p);
  else
    hipLaunchKernelGGL(swa_wide_kernel<false>, grid, block, LdsWide::BYTES, a.stream, p);
  return hipGetLastError();
}

}  // namespace glah

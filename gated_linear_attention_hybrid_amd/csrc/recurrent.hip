// recurrent.hip -- token-recurrent VALU kernels of the hybrid layer.
//
// These evaluate the layer in its recurrent (constant-memory) form: the state
// S = diag(Gamma_t) S + phi(k_t)^T v_t is advanced one token at a time and read
// out with phi(q_t) ("Lizard" technical summary, gist.science 2507.09025,
// Methodology A.1), plus the window softmax with meta-memory sinks (A.2).
//   * recurrent_prefill_kernel: whole sequences, the state slice stays in
//     registers for the entire sequence.  It serves the fp32 mode and any size
//     the chunkwise MFMA kernels do not cover.  All arithmetic is fp32.
//   * decode_step_kernel: one token for every (b, h), the state is read from and
//     written back to HBM in place; window keys come from the ring cache.  This
//     step is bound by HBM bandwidth: the fp32 state is streamed once with
//     16-byte loads issued before any other work.
#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;

struct RecParams {
  const void *q, *k, *v, *gate, *wq, *wk;
  const float *meta;
  const float *state_in;
  float *state_out;
  float *state;
  void *o;
  void *kcache, *vcache;
  const int32_t *pos;
  int B, H, L, d, dv, f, window, n_meta, nslices;
  float scale;
  int gate_is_log, gate_mode;
};

struct RecShared {
  float xq[kRecMaxD];
  float xk[kRecMaxD];
  float ubuf[kRecMaxF];
  float phq[kRecMaxF];
  float phk[kRecMaxF];
  float gam[kRecMaxF];
  float sc[kRecMaxWindow];
  float wred[2 * kWaves];
};

__device__ __forceinline__ float block_max(float x, float *wred) {
  x = wave_max(x);
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) wred[wave] = x;
  __syncthreads();
  float r = wred[0];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) r = fmaxf(r, wred[w]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ float block_sum(float x, float *wred) {
  x = wave_sum(x);
  const int wave = threadIdx.x / 64;
  if ((threadIdx.x & 63) == 0) wred[kWaves + wave] = x;
  __syncthreads();
  float r = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) r += wred[kWaves + w];
  return r;
}

// Hedgehog map of the staged q and k rows: phi = [softmax(u), softmax(-u)],
// u = x Wphi ("Lizard" summary, Methodology C: non-negative Hedgehog features).
// Ends with a barrier.
template <class T>
__device__ void hedgehog_block(RecShared &sh, const T *Wq, const T *Wk, int d, int f2) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < 2 * f2; idx += kThreads) {
    const int m = idx >= f2;
    const int j = idx - m * f2;
    const float *x = m ? sh.xk : sh.xq;
    const T *W = m ? Wk : Wq;
    float acc = 0.0f;
    for (int i = 0; i < d; ++i) acc += x[i] * ld(W + (size_t)i * f2 + j);
    sh.ubuf[idx] = acc;
  }
  __syncthreads();
  const int wave = tid / 64, lane = tid & 63;
  if (wave < 2) {
    const float *u = sh.ubuf + wave * f2;
    float *ph = wave ? sh.phk : sh.phq;
    float mx = -INFINITY, mn = INFINITY;
    for (int j = lane; j < f2; j += 64) {
      mx = fmaxf(mx, u[j]);
      mn = fminf(mn, u[j]);
    }
    mx = wave_max(mx);
    mn = wave_min(mn);
    float zp = 0.0f, zn = 0.0f;
    for (int j = lane; j < f2; j += 64) {
      zp += exp_fast(u[j] - mx);
      zn += exp_fast(mn - u[j]);
    }
    zp = wave_sum(zp);
    zn = wave_sum(zn);
    const float ip = 1.0f / zp, in = 1.0f / zn;
    for (int j = lane; j < f2; j += 64) {
      ph[j] = exp_fast(u[j] - mx) * ip;
      ph[f2 + j] = exp_fast(mn - u[j]) * in;
    }
  }
  __syncthreads();
}

// Window softmax weights for n keys: on return sh.sc[i] = e^{s_i - m} and the
// function returns 1 / (sum_i e^{s_i - m} + sum_m e^{t_m - m}).  key(i) gives
// the d-vector of the i-th window key.  Ends with a barrier.
template <class T, class KeyFn>
__device__ float window_weights(RecShared &sh, KeyFn key, int n, int d, float scale,
                                const float *meta, int n_meta) {
  const int tid = threadIdx.x;
  for (int i = tid; i < n; i += kThreads) {
    const T *kr = key(i);
    float acc = 0.0f;
    for (int e = 0; e < d; ++e) acc += sh.xq[e] * ld(kr + e);
    sh.sc[i] = scale * acc;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int i = tid; i < n; i += kThreads) m = fmaxf(m, sh.sc[i]);
  if (tid < n_meta) m = fmaxf(m, meta[tid]);
  m = block_max(m, sh.wred);
  float s = 0.0f;
  for (int i = tid; i < n; i += kThreads) {
    const float e = exp_fast(sh.sc[i] - m);
    sh.sc[i] = e;
    s += e;
  }
  if (tid < n_meta) s += exp_fast(meta[tid] - m);
  s = block_sum(s, sh.wred);
  __syncthreads();
  return 1.0f / s;
}

// ---------------------------------------------------------------------------
// Whole-sequence recurrent prefill.  Block = (b, h, 64-column slice of d_v).
template <class T, int PARTS>
__global__ __launch_bounds__(kThreads) void recurrent_prefill_kernel(RecParams p) {
  constexpr bool GLA = PARTS & PART_GLA;
  constexpr bool SWA = PARTS & PART_SWA;
  constexpr int DVS = 64;
  constexpr int NRG = kThreads / DVS;
  constexpr int MAXR = kRecMaxF / NRG;
  __shared__ RecShared sh;
  __shared__ float vt[DVS];
  __shared__ float red[NRG][DVS];

  const int tid = threadIdx.x;
  const int bh = blockIdx.x / p.nslices;
  const int slice = blockIdx.x % p.nslices;
  const int h = bh % p.H;
  const int d = p.d, dv = p.dv, f = p.f, f2 = p.f / 2, L = p.L;
  const int dv0 = slice * DVS;
  const int c = tid % DVS, rg = tid / DVS;
  const int col = dv0 + c;
  const bool colok = col < dv;

  const T *q = (const T *)p.q + (size_t)bh * L * d;
  const T *k = (const T *)p.k + (size_t)bh * L * d;
  const T *v = (const T *)p.v + (size_t)bh * L * dv;
  const T *g = (const T *)p.gate;
  const T *Wq = GLA ? (const T *)p.wq + (size_t)h * d * f2 : nullptr;
  const T *Wk = GLA ? (const T *)p.wk + (size_t)h * d * f2 : nullptr;
  const float *meta = p.n_meta ? p.meta + (size_t)h * p.n_meta : nullptr;
  T *o = (T *)p.o + (size_t)bh * L * dv;

  float S[MAXR];
#pragma unroll
  for (int ii = 0; ii < MAXR; ++ii) {
    const int r = rg + NRG * ii;
    S[ii] = (GLA && p.state_in && r < f && colok) ? p.state_in[((size_t)bh * f + r) * dv + col] : 0.0f;
  }

  for (int t = 0; t < L; ++t) {
    for (int i = tid; i < d; i += kThreads) {
      sh.xq[i] = ld(q + (size_t)t * d + i);
      if (GLA) sh.xk[i] = ld(k + (size_t)t * d + i);
    }
    if (GLA)
      for (int r = tid; r < f; r += kThreads)
        sh.gam[r] = gate_from(ld(g + gate_index(p.gate_mode, bh, p.H, L, f, t, r)), p.gate_is_log);
    if (tid < DVS) vt[tid] = (dv0 + tid < dv) ? ld(v + (size_t)t * dv + dv0 + tid) : 0.0f;
    __syncthreads();
    if (GLA) hedgehog_block<T>(sh, Wq, Wk, d, f2);

    float acc = 0.0f;
    if (GLA) {
#pragma unroll
      for (int ii = 0; ii < MAXR; ++ii) {
        const int r = rg + NRG * ii;
        if (r < f) {
          S[ii] = sh.gam[r] * S[ii] + sh.phk[r] * vt[c];
          acc += sh.phq[r] * S[ii];
        }
      }
    }
    if (SWA) {
      const int n = min(t + 1, p.window);
      auto key = [&](int i) { return k + (size_t)(t - i) * d; };
      const float inv = window_weights<T>(sh, key, n, d, p.scale, meta, p.n_meta);
      float accs = 0.0f;
      if (colok)
        for (int i = rg; i < n; i += NRG) accs += sh.sc[i] * ld(v + (size_t)(t - i) * dv + col);
      acc += accs * inv;
    }
    red[rg][c] = acc;
    __syncthreads();
    if (tid < DVS && dv0 + tid < dv) {
      float s = 0.0f;
#pragma unroll
      for (int r2 = 0; r2 < NRG; ++r2) s += red[r2][tid];
      o[(size_t)t * dv + dv0 + tid] = from_f32<T>(s);
    }
    __syncthreads();
  }

  if (GLA && p.state_out) {
#pragma unroll
    for (int ii = 0; ii < MAXR; ++ii) {
      const int r = rg + NRG * ii;
      if (r < f && colok) p.state_out[((size_t)bh * f + r) * dv + col] = S[ii];
    }
  }
}

// ---------------------------------------------------------------------------
// One decode step.  Block = (b, h, DVS-column slice); each thread owns four
// adjacent state columns (one 16-byte load per state row it covers).
template <class T, int PARTS, int DVS>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(RecParams p) {
  constexpr bool GLA = PARTS & PART_GLA;
  constexpr bool SWA = PARTS & PART_SWA;
  constexpr int C4 = DVS / 4;
  constexpr int NRG = kThreads / C4;
  constexpr int MAXR = (kRecMaxF + NRG - 1) / NRG;
  __shared__ RecShared sh;
  __shared__ float vt[DVS];
  __shared__ f32x4 red[NRG][C4];

  const int tid = threadIdx.x;
  // Blocks are dealt round-robin to the 8 XCDs; keep every slice of one head
  // (and the same head of every batch row) on one XCD so the ring keys and the
  // Hedgehog weights are fetched into one L2.
  int bh, slice;
  {
    const int bid = blockIdx.x;
    const int nbh = p.B * p.H;
    if ((nbh & 7) == 0) {
      const int xcd = bid & 7, local = bid >> 3;
      slice = local % p.nslices;
      bh = (local / p.nslices) * 8 + xcd;
    } else {
      bh = bid / p.nslices;
      slice = bid % p.nslices;
    }
  }
  const int b = bh / p.H, h = bh % p.H;
  const int d = p.d, dv = p.dv, f = p.f, f2 = p.f / 2, w = p.window;
  const int dv0 = slice * DVS;
  const int c4 = tid % C4, rg = tid / C4;
  const int col = dv0 + 4 * c4;
  const bool colok = col < dv;  // dv is a multiple of 4
  const int pos = max(p.pos[b], 0);  // a negative position is treated as 0

  float *Sg = GLA ? p.state + (size_t)bh * f * dv : nullptr;
  f32x4 S[MAXR];
  if (GLA) {
#pragma unroll
    for (int ii = 0; ii < MAXR; ++ii) {
      const int r = rg + NRG * ii;
      if (r < f && colok) S[ii] = *(const f32x4 *)(Sg + (size_t)r * dv + col);
    }
  }

  const T *qt = (const T *)p.q + (size_t)bh * d;
  const T *kt = (const T *)p.k + (size_t)bh * d;
  const T *vtg = (const T *)p.v + (size_t)bh * dv;
  const float *meta = p.n_meta ? p.meta + (size_t)h * p.n_meta : nullptr;
  T *kc = SWA ? (T *)p.kcache + (size_t)bh * w * d : nullptr;
  T *vc = SWA ? (T *)p.vcache + (size_t)bh * w * dv : nullptr;

  for (int i = tid; i < d; i += kThreads) {
    sh.xq[i] = ld(qt + i);
    sh.xk[i] = ld(kt + i);
  }
  if (GLA) {
    const T *gt = (const T *)p.gate;
    for (int r = tid; r < f; r += kThreads)
      sh.gam[r] = gate_from(ld(gt + gate_index(p.gate_mode, bh, p.H, 1, f, 0, r)), p.gate_is_log);
  }
  if (tid < DVS) vt[tid] = (dv0 + tid < dv) ? ld(vtg + dv0 + tid) : 0.0f;
  __syncthreads();

  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
  if (GLA) {
    hedgehog_block<T>(sh, (const T *)p.wq + (size_t)h * d * f2, (const T *)p.wk + (size_t)h * d * f2, d, f2);
    const f32x4 v4 = {vt[4 * c4], vt[4 * c4 + 1], vt[4 * c4 + 2], vt[4 * c4 + 3]};
#pragma unroll
    for (int ii = 0; ii < MAXR; ++ii) {
      const int r = rg + NRG * ii;
      if (r < f && colok) {
        S[ii] = sh.gam[r] * S[ii] + sh.phk[r] * v4;
        acc += sh.phq[r] * S[ii];
        *(f32x4 *)(Sg + (size_t)r * dv + col) = S[ii];
      }
    }
  }
  if (SWA) {
    // window: the new token (i = 0, from the inputs) and tokens pos-1 .. pos-n+1
    // from ring slots (pos-i) % w
    const int n = min(pos + 1, w);
    auto key = [&](int i) -> const T * {
      return i == 0 ? kt : kc + (size_t)((pos - i) % w) * d;
    };
    const float inv = window_weights<T>(sh, key, n, d, p.scale, meta, p.n_meta);
    f32x4 accs = {0.0f, 0.0f, 0.0f, 0.0f};
    if (colok) {
      for (int i = rg; i < n; i += NRG) {
        f32x4 vv;
        if (i == 0) {
          vv = (f32x4){vt[4 * c4], vt[4 * c4 + 1], vt[4 * c4 + 2], vt[4 * c4 + 3]};
        } else {
          const T *vr = vc + (size_t)((pos - i) % w) * dv + col;
          vv = (f32x4){ld(vr), ld(vr + 1), ld(vr + 2), ld(vr + 3)};
        }
        accs += sh.sc[i] * vv;
      }
    }
    acc += accs * inv;
  }
  red[rg][c4] = acc;
  __syncthreads();
  if (tid < DVS && dv0 + tid < dv) {
    const int cc = tid >> 2, e = tid & 3;
    float s = 0.0f;
    for (int r2 = 0; r2 < NRG; ++r2) s += red[r2][cc][e];
    ((T *)p.o)[(size_t)bh * dv + dv0 + tid] = from_f32<T>(s);
  }
  if (SWA) {
    // append the token to the ring: slot pos % w holds token pos - w, which no
    // block reads in this step
    const int slot = pos % w;
    if (slice == 0)
      for (int i = tid; i < d; i += kThreads) kc[(size_t)slot * d + i] = kt[i];
    if (tid < DVS && dv0 + tid < dv) vc[(size_t)slot * dv + dv0 + tid] = vtg[dv0 + tid];
  }
}

// Ring of the last `window` keys/values after a prefill (zeros for slots of
// tokens before position 0).  Block = (b, h, slot).
template <class T>
__global__ __launch_bounds__(kThreads) void window_cache_kernel(const T *k, const T *v, T *kc, T *vc,
                                                                int L, int d, int dv, int w) {
  const int bh = blockIdx.x / w, slot = blockIdx.x % w;
  // the token p in [L - w, L - 1] with p % w == slot
  int p = L - w + ((slot - (L - w)) % w + w) % w;
  const bool ok = p >= 0 && p < L;
  for (int i = threadIdx.x; i < d; i += kThreads)
    kc[((size_t)bh * w + slot) * d + i] = ok ? k[((size_t)bh * L + p) * d + i] : from_f32<T>(0.0f);
  for (int i = threadIdx.x; i < dv; i += kThreads)
    vc[((size_t)bh * w + slot) * dv + i] = ok ? v[((size_t)bh * L + p) * dv + i] : from_f32<T>(0.0f);
}

RecParams make_params(const LayerArgs &a) {
  RecParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.wq = a.wq; p.wk = a.wk;
  p.meta = a.meta; p.state_in = a.state_in; p.state_out = a.state_out; p.state = a.state;
  p.o = a.o; p.kcache = a.kcache; p.vcache = a.vcache; p.pos = a.pos;
  p.B = a.B; p.H = a.H; p.L = a.L; p.d = a.d; p.dv = a.dv; p.f = a.f;
  p.window = a.window; p.n_meta = a.n_meta; p.nslices = 1;
  p.scale = a.scale; p.gate_is_log = a.gate_is_log ? 1 : 0; p.gate_mode = a.gate_mode;
  return p;
}

template <class T>
hipError_t prefill_dispatch(const LayerArgs &a, int parts) {
  RecParams p = make_params(a);
  p.nslices = (a.dv + 63) / 64;
  const dim3 grid((unsigned)(a.B * a.H * p.nslices)), block(kThreads);
  switch (parts) {
    case PART_GLA: hipLaunchKernelGGL((recurrent_prefill_kernel<T, PART_GLA>), grid, block, 0, a.stream, p); break;
    case PART_SWA: hipLaunchKernelGGL((recurrent_prefill_kernel<T, PART_SWA>), grid, block, 0, a.stream, p); break;
    default: hipLaunchKernelGGL((recurrent_prefill_kernel<T, PART_BOTH>), grid, block, 0, a.stream, p); break;
  }
  return hipGetLastError();
}

template <class T, int DVS>
hipError_t decode_dispatch(const LayerArgs &a, int parts) {
  RecParams p = make_params(a);
  p.nslices = (a.dv + DVS - 1) / DVS;
  const dim3 grid((unsigned)(a.B * a.H * p.nslices)), block(kThreads);
  switch (parts) {
    case PART_GLA: hipLaunchKernelGGL((decode_step_kernel<T, PART_GLA, DVS>), grid, block, 0, a.stream, p); break;
    case PART_SWA: hipLaunchKernelGGL((decode_step_kernel<T, PART_SWA, DVS>), grid, block, 0, a.stream, p); break;
    default: hipLaunchKernelGGL((decode_step_kernel<T, PART_BOTH, DVS>), grid, block, 0, a.stream, p); break;
  }
  return hipGetLastError();
}

// state_out of an empty sequence: a plain copy of state_in, or zeros (a kernel,
// not a memset, so the call may be captured in a graph)
__global__ __launch_bounds__(kThreads) void state_passthrough_kernel(const float *in, float *out, size_t n) {
  const size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (i < n) out[i] = in ? in[i] : 0.0f;
}

}  // namespace

bool recurrent_supported(const LayerArgs &a, int parts) {
  if (a.d > kRecMaxD || a.n_meta > kRecMaxMeta) return false;
  if ((parts & PART_GLA) && a.f > kRecMaxF) return false;
  if ((parts & PART_SWA) && a.window > kRecMaxWindow) return false;
  return true;
}

hipError_t launch_recurrent_prefill(const LayerArgs &a, int parts) {
  if (a.B * a.H == 0 || a.L == 0) return hipSuccess;
  return a.bf16 ? prefill_dispatch<bf16>(a, parts) : prefill_dispatch<float>(a, parts);
}

hipError_t launch_decode_step(const LayerArgs &a, int parts) {
  if (a.B * a.H == 0) return hipSuccess;
  if (decode128_supported(a, parts)) return launch_decode128(a, parts);
  // 32 state columns per block: 4 blocks per head at d_v = 128, so a batch of
  // 8 x 32 heads spreads over 1024 blocks.
  return a.bf16 ? decode_dispatch<bf16, 32>(a, parts) : decode_dispatch<float, 32>(a, parts);
}

hipError_t launch_state_passthrough(const LayerArgs &a) {
  if (!a.state_out || a.state_out == a.state_in) return hipSuccess;
  const size_t n = (size_t)a.B * a.H * a.f * a.dv;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(state_passthrough_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0,
                     a.stream, a.state_in, a.state_out, n);
  return hipGetLastError();
}

hipError_t launch_window_cache(const LayerArgs &a) {
  if (a.B * a.H == 0 || a.window == 0 || !a.kcache || !a.vcache) return hipSuccess;
  const dim3 grid((unsigned)(a.B * a.H * a.window)), block(kThreads);
  if (a.bf16)
    hipLaunchKernelGGL(window_cache_kernel<bf16>, grid, block, 0, a.stream, (const bf16 *)a.k,
                       (const bf16 *)a.v, (bf16 *)a.kcache, (bf16 *)a.vcache, a.L, a.d, a.dv, a.window);
  else
    hipLaunchKernelGGL(window_cache_kernel<float>, grid, block, 0, a.stream, (const float *)a.k,
                       (const float *)a.v, (float *)a.kcache, (float *)a.vcache, a.L, a.d, a.dv, a.window);
  return hipGetLastError();
}

}  // namespace glah

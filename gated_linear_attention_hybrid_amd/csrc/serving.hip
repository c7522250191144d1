// serving.hip -- pieces a serving loop needs around the layer: a prefill that
// continues a sequence (the window part reaches back into the previous call's
// ring of keys and values), and the output-gate epilogue.
//
// Continuation.  A prefill of tokens at positions start .. start+L-1 computes
// the gated part from state_in (the state after token start-1) and the window
// part over keys [P-w+1, P] for the query at position P ("Lizard" technical
// summary, 2507.09025, Methodology A.2: anchor window attention with
// meta-memory sinks).  The layer kernels compute every window from the keys of
// their own call; for the first w-1 queries the keys at positions before
// `start` live in the ring (slot p % w holds token p).  `halo_fix_kernel` adds
// to those queries' outputs the difference between the window softmax over
// the ring and call keys and the one over the call keys alone, both in fp32.
// `ring_cont_kernel` writes the ring after the call with global positions.
//
// Output gate.  o <- o * sigmoid(g) per element, the output gate the "LT2"
// technical summary (2605.20670, contributions) puts on attention outputs to
// keep activations from growing across loop iterations.
#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kThreads = 256;
constexpr int kQPerBlock = kThreads / 64;  // one query per wave

struct HaloParams {
  const void *q, *k, *v, *kc, *vc;
  const float *meta;
  void *o;
  int L, d, dv, window, n_meta, H;
  long start;
  float scale;
};

template <class T>
__device__ __forceinline__ float dot_row(const T *a, const T *b, int d) {
  float s = 0.0f;
  constexpr int per = 16 / (int)sizeof(T);
  if (d % per == 0) {
#pragma unroll 4
    for (int c = 0; c < d; c += per) {
      const u32x4 x = *(const u32x4 *)(a + c), y = *(const u32x4 *)(b + c);
      const T *xe = (const T *)&x, *ye = (const T *)&y;
#pragma unroll
      for (int j = 0; j < per; ++j) s += to_f32(xe[j]) * to_f32(ye[j]);
    }
  } else {
    for (int c = 0; c < d; ++c) s += to_f32(a[c]) * to_f32(b[c]);
  }
  return s;
}

// Block = (b, h, group of 4 queries); wave = one query t < min(w - 1, L); lane i
// = the key at position P - i (P = start + t).  Keys i <= t are this call's,
// keys i > t with P - i >= 0 come from the ring.
template <class T>
__global__ __launch_bounds__(kThreads) void halo_fix_kernel(HaloParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nq = min(p.window - 1, p.L);
  const int ngrp = (nq + kQPerBlock - 1) / kQPerBlock;
  const size_t bh = blockIdx.x / ngrp;
  const int t = (blockIdx.x % ngrp) * kQPerBlock + wave;
  if (t >= nq) return;  // whole wave: no barrier below
  const int h = (int)(bh % p.H);
  const T *q = (const T *)p.q + (bh * p.L + t) * p.d;
  const T *kl = (const T *)p.k + bh * p.L * p.d;
  const T *vl = (const T *)p.v + bh * p.L * p.dv;
  const T *kc = (const T *)p.kc + bh * p.window * p.d;
  const T *vc = (const T *)p.vc + bh * p.window * p.dv;
  const long P = p.start + t;

  const int i = lane;
  const bool loc = i <= t;
  const long pos = P - i;
  const bool valid = i < p.window && pos >= 0;
  // ring slot of position P - i = start + t - i (one 64-bit modulo per wave;
  // -1 for this call's keys and for keys outside the window)
  const int base = (int)(p.start % p.window);
  int slot = (base + t - i) % p.window;
  slot = (!loc && valid) ? (slot < 0 ? slot + p.window : slot) : -1;
  const T *key = loc ? kl + (size_t)(t - i) * p.d : slot >= 0 ? kc + (size_t)slot * p.d : kl;
  const float tm = lane < p.n_meta ? p.meta[(size_t)h * p.n_meta + lane] : -INFINITY;
  const float s = dot_row<T>(q, key, p.d) * p.scale;
  const float mm = wave_max(tm);
  // full window (ring and call keys) and the call keys alone, each with the sinks
  const float sf = valid ? s : -INFINITY, sl = (valid && loc) ? s : -INFINITY;
  const float mf = fmaxf(wave_max(sf), mm), ml = fmaxf(wave_max(sl), mm);
  const float ef = valid ? exp_fast(sf - mf) : 0.0f, el = (valid && loc) ? exp_fast(sl - ml) : 0.0f;
  const float zf = wave_sum(ef) + wave_sum(lane < p.n_meta ? exp_fast(tm - mf) : 0.0f);
  const float zl = wave_sum(el) + wave_sum(lane < p.n_meta ? exp_fast(tm - ml) : 0.0f);
  const float pd = ef / zf - el / zl;  // weight change of key i

  // each key's weight change and value row go to LDS once; the column loop
  // reads them as wave-wide broadcasts
  __shared__ float s_pd[kQPerBlock][64];
  __shared__ const T *s_row[kQPerBlock][64];
  s_pd[wave][lane] = pd;
  s_row[wave][lane] = loc ? vl + (size_t)(t - i) * p.dv : slot >= 0 ? vc + (size_t)slot * p.dv : vl;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  T *o = (T *)p.o + (bh * p.L + t) * p.dv;
  const int nk = min(p.window, 64);
  for (int c0 = 0; c0 < p.dv; c0 += 64) {
    const int c = min(c0 + lane, p.dv - 1);  // lanes past d_v read a valid column, store nothing
    float acc = 0.0f;
#pragma unroll 16
    for (int j = 0; j < nk; ++j) acc += s_pd[wave][j] * to_f32(s_row[wave][j][c]);
    if (c0 + lane < p.dv) o[c] = from_f32<T>(to_f32(o[c]) + acc);
  }
}

// Ring after the call: slot s holds the newest token p <= start + L - 1 with
// p % w == s; from this call when p >= start, from the input ring when
// 0 <= p < start, zeros before the sequence.  Block = (b, h, slot).
template <class T>
__global__ __launch_bounds__(kThreads) void ring_cont_kernel(const T *k, const T *v, const T *kci, const T *vci,
                                                             T *kco, T *vco, long start, int L, int d, int dv,
                                                             int w) {
  const size_t bh = blockIdx.x / w;
  const int slot = blockIdx.x % w;
  const long end = start + L;
  const long p = end - w + (((slot - (end - w)) % w) + w) % w;
  const bool cur = p >= start, old = !cur && p >= 0;
  for (int e = threadIdx.x; e < d; e += kThreads) {
    const size_t dst = (bh * w + slot) * d + e;
    kco[dst] = cur ? k[(bh * L + (p - start)) * d + e] : old ? kci[dst] : from_f32<T>(0.0f);
  }
  for (int e = threadIdx.x; e < dv; e += kThreads) {
    const size_t dst = (bh * w + slot) * dv + e;
    vco[dst] = cur ? v[(bh * L + (p - start)) * dv + e] : old ? vci[dst] : from_f32<T>(0.0f);
  }
}

// o <- o * sigmoid(g), 16 bytes per thread per step (grid-stride).
template <class T>
__global__ __launch_bounds__(kThreads) void output_gate_kernel(T *o, const T *g, size_t n) {
  constexpr int per = 16 / (int)sizeof(T);
  const size_t nvec = n / per;
  const size_t stride = (size_t)gridDim.x * kThreads;
  for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < nvec; i += stride) {
    u32x4 x = ((const u32x4 *)o)[i];
    const u32x4 y = __builtin_nontemporal_load((const u32x4 *)g + i);
    T *xe = (T *)&x;
    const T *ye = (const T *)&y;
#pragma unroll
    for (int j = 0; j < per; ++j) xe[j] = from_f32<T>(to_f32(xe[j]) * rcp_fast(1.0f + exp_fast(-to_f32(ye[j]))));
    ((u32x4 *)o)[i] = x;
  }
  // the last n % per elements
  const size_t tail = nvec * per + (size_t)blockIdx.x * kThreads + threadIdx.x;
  if (tail < n && blockIdx.x * (size_t)kThreads + threadIdx.x < (size_t)per)
    o[tail] = from_f32<T>(to_f32(o[tail]) * rcp_fast(1.0f + exp_fast(-to_f32(g[tail]))));
}

}  // namespace

bool halo_supported(const LayerArgs &a) { return a.window >= 1 && a.window <= 64 && a.n_meta <= 64 && a.d <= 4096; }

hipError_t launch_halo_fix(const LayerArgs &a, long start, const void *kcache_in, const void *vcache_in) {
  const int nq = a.window - 1 < a.L ? a.window - 1 : a.L;
  if (start <= 0 || nq <= 0 || (size_t)a.B * a.H == 0) return hipSuccess;
  HaloParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.kc = kcache_in; p.vc = vcache_in; p.meta = a.meta; p.o = a.o;
  p.L = a.L; p.d = a.d; p.dv = a.dv; p.window = a.window; p.n_meta = a.n_meta; p.H = a.H;
  p.start = start; p.scale = a.scale;
  const size_t ngrp = (size_t)(nq + kQPerBlock - 1) / kQPerBlock;
  const dim3 grid((unsigned)((size_t)a.B * a.H * ngrp)), block(kThreads);
  if (a.bf16)
    hipLaunchKernelGGL(halo_fix_kernel<bf16>, grid, block, 0, a.stream, p);
  else
    hipLaunchKernelGGL(halo_fix_kernel<float>, grid, block, 0, a.stream, p);
  return hipGetLastError();
}

hipError_t launch_ring_cont(const LayerArgs &a, long start, const void *kcache_in, const void *vcache_in) {
  if ((size_t)a.B * a.H == 0 || a.window == 0 || !a.kcache || !a.vcache) return hipSuccess;
  const dim3 grid((unsigned)((size_t)a.B * a.H * a.window)), block(kThreads);
  if (a.bf16)
    hipLaunchKernelGGL(ring_cont_kernel<bf16>, grid, block, 0, a.stream, (const bf16 *)a.k, (const bf16 *)a.v,
                       (const bf16 *)kcache_in, (const bf16 *)vcache_in, (bf16 *)a.kcache, (bf16 *)a.vcache, start,
                       a.L, a.d, a.dv, a.window);
  else
    hipLaunchKernelGGL(ring_cont_kernel<float>, grid, block, 0, a.stream, (const float *)a.k, (const float *)a.v,
                       (const float *)kcache_in, (const float *)vcache_in, (float *)a.kcache, (float *)a.vcache,
                       start, a.L, a.d, a.dv, a.window);
  return hipGetLastError();
}

hipError_t launch_output_gate(void *o, const void *g, size_t n, bool is_bf16, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const size_t per = is_bf16 ? 8 : 4;
  size_t blocks = (n / per + kThreads - 1) / kThreads;
  if (blocks < 1) blocks = 1;
  if (blocks > 8192) blocks = 8192;
  if (is_bf16)
    hipLaunchKernelGGL(output_gate_kernel<bf16>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (bf16 *)o,
                       (const bf16 *)g, n);
  else
    hipLaunchKernelGGL(output_gate_kernel<float>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, (float *)o,
                       (const float *)g, n);
  return hipGetLastError();
}

}  // namespace glah

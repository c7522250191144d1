// decode.hip -- one recurrent decode step of the hybrid layer at d = f = d_v = 128
// (window <= 64), bf16 or fp32 tokens, fp32 state updated in place.
//
// Constant-memory inference ("Lizard" technical summary, gist.science
// 2507.09025, Methodology A.1): per (b, h) the step reads the f x d_v fp32 state
// once and writes it once; everything else is small.  The step is bound by HBM
// bandwidth, so the block issues every load before any arithmetic (16-byte
// vector loads, the whole 64 KiB state of a head in flight per block), the
// state last, and does the Hedgehog GEMVs and the window scores while the
// state streams in; each state row is written back as soon as it arrives:
//   * Hedgehog GEMV: each thread loads 1 row x 8 columns of each projection
//     with 16-byte loads, partial sums are reduced across lanes (DPP and row
//     swaps) and waves (LDS).
//   * window scores: 16 threads per ring slot, 8 dimensions each, 16-byte loads.
//   * window values: loaded up front, 16 bytes per lane (two lanes share
//     eight columns of two ring slots and swap halves by DPP).
//   * the sinks and the new key for the ring append are loaded up front too,
//     so no load sits in the softmax chain or in the kernel's tail.
// Block = (b, h), 1024 threads: the projections, the window keys and the new
// token are read once per head instead of once per column slice.
#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

namespace {

constexpr int kNT = 1024;
constexpr int kD = 128, kF = 128, kF2 = 64, kDV = 128, kMaxW = 64;
constexpr int kDVS = 128;                // state columns per block
constexpr int kC4 = kDVS / 4;            // float4 column groups per block
constexpr int kNRG = kNT / kC4;          // row groups
constexpr int kRPT = kF / kNRG;          // state rows per thread
constexpr int kNSL = kDV / kDVS;         // blocks per head
static_assert(2 * kNRG == kMaxW, "two ring slots per row group (the value loads)");
static_assert(kNRG == 2 * (kNT / 64), "two row groups per wave, in lanes l and l + 32");

struct DecParams {
  const void *q, *k, *v, *gate, *wq, *wk;
  const float *meta;
  float *state;
  void *kcache, *vcache;
  const int32_t *pos;
  void *o;
  int B, H, window, n_meta;
  float scale;
  int gate_is_log, gate_mode;
};

template <class T> struct Vec;
template <> struct Vec<bf16> {
  static __device__ __forceinline__ f32x4 ld4(const bf16 *p) {
    const bf16x4 x = *(const bf16x4 *)p;
    return (f32x4){(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  }
  static __device__ __forceinline__ void ld8(const bf16 *p, float *o) {
    const bf16x8 x = *(const bf16x8 *)p;
#pragma unroll
    for (int j = 0; j < 8; ++j) o[j] = (float)x[j];
  }
  static __device__ __forceinline__ void st4(bf16 *p, f32x4 v) {
    bf16x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j) x[j] = (bf16)v[j];
    *(bf16x4 *)p = x;
  }
};
template <> struct Vec<float> {
  static __device__ __forceinline__ f32x4 ld4(const float *p) { return *(const f32x4 *)p; }
  static __device__ __forceinline__ void ld8(const float *p, float *o) {
    const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      o[j] = a[j];
      o[4 + j] = b[j];
    }
  }
  static __device__ __forceinline__ void st4(float *p, f32x4 v) { *(f32x4 *)p = v; }
};

template <class T, int PARTS>
__global__ __launch_bounds__(kNT) void decode128_kernel(DecParams p) {
  constexpr bool SWA = PARTS & PART_SWA;
  using V = Vec<T>;
  constexpr int kWaves = kNT / 64;
  constexpr int kGR = kD / (kNT / 8);  // GEMV rows per thread
  __shared__ float s_uw[kWaves][2][kF2];  // per-wave Hedgehog partial sums
  __shared__ float s_ph[2][kF];      // phi(q), phi(k)
  __shared__ float s_gam[kF];
  __shared__ float s_p[kMaxW + 1];   // window weights: ring slots, then the new token
  __shared__ float s_qk[2];          // q . k of the new token, per wave of waves 0-1
  __shared__ f32x4 s_red[kNT / 64][kC4];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int bh, slice;
  {
    const int bid = blockIdx.x, nbh = p.B * p.H;
    if ((nbh & 7) == 0) {
      const int xcd = bid & 7, local = bid >> 3;
      slice = local % kNSL;
      bh = (local / kNSL) * 8 + xcd;
    } else {
      bh = bid / kNSL;
      slice = bid % kNSL;
    }
  }
  const int b = bh / p.H, h = bh % p.H;
  const int w = p.window;
  const int pos = max(p.pos[b], 0);
  const int c4 = tid % kC4, rg = tid / kC4;
  const int col = slice * kDVS + 4 * c4;

  const T *qt = (const T *)p.q + (size_t)bh * kD;
  const T *kt = (const T *)p.k + (size_t)bh * kD;
  const T *vt = (const T *)p.v + (size_t)bh * kDV;
  T *kc = SWA ? (T *)p.kcache + (size_t)bh * w * kD : nullptr;
  T *vc = SWA ? (T *)p.vcache + (size_t)bh * w * kDV : nullptr;
  // Window keys: the new token pos and the ring tokens pos-1 .. pos-n+1, n =
  // min(pos+1, w).  The ring is read by slot (slot s holds token pos - ((pos - s)
  // mod w)), so no load waits for pos; masks are applied after the scores.
  const int n = SWA ? min(pos + 1, w) : 0;
  auto ring_ok = [&](int s) {  // slot s holds a token of the window
    const int j = (pos - s) % w;  // pos >= 0, s < w
    return s < w && j >= 1 && j < n;
  };

  // All loads are issued before any arithmetic, the operands of the longest
  // dependent chain (window scores -> softmax -> weighted values) first.  Every
  // load is unconditional, from a clamped index (slots past the window, lanes
  // past a row), and masked where it is used: a load under a lane condition
  // made the compiler wait for it, and for everything issued before it, right
  // where it was issued.
  // (1) window score operands: 16 threads per ring slot, 8 dimensions each
  const int ks_slot = tid >> 4, ks_seg = tid & 15;
  float ka[8], qa[8];
  if (SWA) {
    V::ld8(kc + (size_t)min(ks_slot, w - 1) * kD + 8 * ks_seg, ka);  // slots past w: masked by ring_ok
    V::ld8(qt + 8 * ks_seg, qa);
  }
  // (2) Hedgehog GEMV operands: rows kGR*rgw .. kGR*rgw+kGR-1, columns 8*cb .. 8*cb+7
  const int cb = tid & 7, rgw = tid >> 3;
  float xq[kGR], xk[kGR], wqv[kGR][8], wkv[kGR][8];
  {
    const T *Wq = (const T *)p.wq + (size_t)h * kD * kF2;
    const T *Wk = (const T *)p.wk + (size_t)h * kD * kF2;
#pragma unroll
    for (int i = 0; i < kGR; ++i) {
      const int row = kGR * rgw + i;
      xq[i] = to_f32(qt[row]);
      xk[i] = to_f32(kt[row]);
      V::ld8(Wq + (size_t)row * kF2 + 8 * cb, wqv[i]);
      V::ld8(Wk + (size_t)row * kF2 + 8 * cb, wkv[i]);
    }
  }
  // (3) window values, 16 bytes per lane: ring slot rg + kNRG (c4 & 1), columns
  // 8 (c4 >> 1) .. +7, i.e. this thread's four columns and those of lane ^ 1;
  // after weighting, the two lanes swap the halves they do not own
  float vw[8];
  const int vslot = rg + kNRG * (c4 & 1);
  if (SWA) V::ld8(vc + (size_t)min(vslot, w - 1) * kDV + slice * kDVS + 8 * (c4 >> 1), vw);  // weight 0 past w
  const f32x4 v4 = V::ld4(vt + col);
  // (4) gates
  const float graw = to_f32(((const T *)p.gate)[gate_index(p.gate_mode, bh, p.H, 1, kF, 0, min(tid, kF - 1))]);
  const float qn = to_f32(qt[min(tid, kD - 1)]), kn = to_f32(kt[min(tid, kD - 1)]);  // used by waves 0-1 only
  // (5) operands of the ring append and of the sink softmax, so that no load
  // sits in the dependent chain after the first barrier or in the kernel's tail
  const f32x4 kt4 = V::ld4(kt + 4 * min(tid, kD / 4 - 1));  // stored by threads tid < kD / 4
  // p.meta is a valid address even without sinks (the host passes another
  // buffer then); lanes past n_meta are masked
  const float tmraw = p.meta[(size_t)h * max(p.n_meta, 1) * (p.n_meta > 0) + min(lane, max(p.n_meta - 1, 0))];
  const float tmeta = lane < p.n_meta ? tmraw : -INFINITY;
  // (6) state slice, LAST: rows rg + kNRG * ii, four columns per thread
  // (streamed: read and written once per step, non-temporal).  Loads complete
  // in order for the wait counter, so everything the two barriers wait for
  // (projections, gates, window operands) was issued before; each state row
  // is then updated and stored as soon as its own load lands, and the state
  // writes overlap the state reads still in flight.
  float *Sg = p.state + (size_t)bh * kF * kDV;
  f32x4 S[kRPT];
#pragma unroll
  for (int ii = 0; ii < kRPT; ++ii)
    S[ii] = __builtin_nontemporal_load((const f32x4 *)(Sg + (size_t)(rg + kNRG * ii) * kDV + col));

  // window scores (ring slots) and q . k of the new token (waves 0-1)
  if (SWA) {
    float acc = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += qa[e] * ka[e];
    acc = row16_reduce(acc, OpAdd());
    if (ks_seg == 0 && ks_slot < kMaxW) s_p[ks_slot] = acc * p.scale;
    if (wave < 2) {
      const float pq = wave_sum(qn * kn);
      if (lane == 0) s_qk[wave] = pq;
    }
  }
  // Hedgehog GEMV partials, reduced over the 8 row groups of the wave (lane bits
  // 3..5: row_ror:8 pairs lanes i and i ^ 8 inside a 16-lane row, then the row
  // swaps) and written per wave
  {
    float pq[8], pk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pq[e] = 0.0f;
      pk[e] = 0.0f;
#pragma unroll
      for (int i = 0; i < kGR; ++i) {
        pq[e] += xq[i] * wqv[i][e];
        pk[e] += xk[i] * wkv[i][e];
      }
      pq[e] = rows_reduce(pq[e] + dpp_f<0x128>(pq[e]), OpAdd());
      pk[e] = rows_reduce(pk[e] + dpp_f<0x128>(pk[e]), OpAdd());
    }
    if ((lane >> 3) == 0) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s_uw[wave][0][8 * cb + e] = pq[e];
        s_uw[wave][1][8 * cb + e] = pk[e];
      }
    }
  }
  if (tid < kF) s_gam[tid] = gate_from(graw, p.gate_is_log);
  __syncthreads();

  // (7) wave 0 / 1: log-softmax of +u and -u for q / k; wave 2: window softmax
  if (wave < 2) {
    float u = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) u += s_uw[w2][wave][lane];
    const float mx = wave_max(u), mn = wave_min(u);
    const float ep = exp_fast(u - mx), en = exp_fast(mn - u);
    const float zp = wave_sum(ep), zn = wave_sum(en);
    s_ph[wave][lane] = ep / zp;
    s_ph[wave][kF2 + lane] = en / zn;
  } else if (SWA && wave == 2) {
    // one-shot softmax over the ring slots in the window, the new token and the
    // meta-memory sinks
    const bool ok = ring_ok(lane);
    const float s = ok ? s_p[lane] : -INFINITY;
    const float snew = (s_qk[0] + s_qk[1]) * p.scale;
    float m = fmaxf(wave_max(s), snew);
    const float tm = tmeta;
    m = fmaxf(m, wave_max(tm));
    const float e = ok ? exp_fast(s - m) : 0.0f;
    const float es = lane < p.n_meta ? exp_fast(tm - m) : 0.0f;
    const float enew = exp_fast(snew - m);
    const float den = wave_sum(e) + wave_sum(es) + enew;
    s_p[lane] = e / den;
    if (lane == 0) s_p[kMaxW] = enew / den;
  }
  __syncthreads();

  // (8) ring append, before the state update so these stores are not the
  // kernel's tail: slot pos % w holds token pos - w, outside this step's window
  // (its score is masked and its weight is 0, so the loads of that slot at
  // the start may see the old or the new token)
  if (SWA) {
    const int slot = pos % w;
    if (slice == 0 && tid < kD / 4) V::st4(kc + (size_t)slot * kD + 4 * tid, kt4);
    if (tid < kC4) V::st4(vc + (size_t)slot * kDV + col, v4);  // rg == 0: col = slice * kDVS + 4 tid
  }
  // (9) state update, readout, window weights x values
  f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ii = 0; ii < kRPT; ++ii) {
    const int r = rg + kNRG * ii;
    S[ii] = s_gam[r] * S[ii] + s_ph[1][r] * v4;
    acc += s_ph[0][r] * S[ii];
    __builtin_nontemporal_store(S[ii], (f32x4 *)(Sg + (size_t)r * kDV + col));
  }
  if (SWA) {
    {
      // weight 0 outside the window; even c4 owns columns 0..3 of the eight
      // loaded, odd c4 columns 4..7 (lane ^ 1 is quad_perm [1,0,3,2])
      const float pw = s_p[vslot];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = pw * vw[e], hi = pw * vw[4 + e];
        const float own = (c4 & 1) ? hi : lo, other = (c4 & 1) ? lo : hi;
        acc[e] += own + dpp_f<0xB1>(other);
      }
    }
    if (rg == 0) acc += s_p[kMaxW] * v4;
  }
  // column sums over the row groups: lanes l and l + 32 hold row groups
  // 2 wave and 2 wave + 1 of the same columns, then one partial per wave
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] += __shfl_xor(acc[e], 32);
  if (lane < 32) s_red[wave][c4] = acc;
  __syncthreads();
  if (tid < kC4) {
    f32x4 s = s_red[0][tid];
#pragma unroll
    for (int r2 = 1; r2 < kWaves; ++r2) s += s_red[r2][tid];
    V::st4((T *)p.o + (size_t)bh * kDV + slice * kDVS + 4 * tid, s);
  }
}

template <class T>
hipError_t dispatch(const LayerArgs &a, int parts) {
  DecParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.wq = a.wq; p.wk = a.wk;
  p.meta = a.meta && a.n_meta > 0 ? a.meta : a.state;  // the kernel loads it unconditionally
  p.state = a.state; p.kcache = a.kcache; p.vcache = a.vcache; p.pos = a.pos; p.o = a.o;
  p.B = a.B; p.H = a.H; p.window = a.window; p.n_meta = a.n_meta; p.scale = a.scale;
  p.gate_is_log = a.gate_is_log ? 1 : 0;
  p.gate_mode = a.gate_mode;
  const dim3 grid((unsigned)(a.B * a.H * kNSL)), block(kNT);
  if (parts & PART_SWA)
    hipLaunchKernelGGL((decode128_kernel<T, PART_BOTH>), grid, block, 0, a.stream, p);
  else
    hipLaunchKernelGGL((decode128_kernel<T, PART_GLA>), grid, block, 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode128_supported(const LayerArgs &a, int parts) {
  return a.d == kD && a.f == kF && a.dv == kDV && (parts & PART_GLA) &&
         (!(parts & PART_SWA) || (a.window >= 1 && a.window <= kMaxW && a.n_meta <= 64));
}

hipError_t launch_decode128(const LayerArgs &a, int parts) {
  if (a.B * a.H == 0) return hipSuccess;
  return a.bf16 ? dispatch<bf16>(a, parts) : dispatch<float>(a, parts);
}

}  // namespace glah

// chunk_common.hpp -- shared pieces of the chunkwise MFMA prefill kernels for
// gfx950 (bf16 inputs, fp32 accumulation, d = f = d_v = 128, 64-token chunks):
// call parameters, sizes and the small device helpers (MFMA operand packing,
// lane-group reductions, DPP scans and broadcasts, the log-gate).
#pragma once
#include "device_common.hpp"

namespace glah {

struct ChunkParams {
  const bf16 *q, *k, *v, *gate, *wq, *wk;
  const float *meta;
  const float *state_in;  // [BH][F][DV] state before token 0 (segment 0), or null
  float *state_out;       // [BH][F][DV] written by the last segment, or null
  bf16 *o;
  bf16 *kc, *vc;          // [BH][window][128]: the ring of the last `window` keys and
                          // values, written by each head's last segment, or null
  float *seg_state;       // [BH][NS][F][DV]: end state of state slice q from zero (state
                          // pass), overwritten by the scan with the state after slice q
  float *seg_decay;       // [BH][NS][F]: total base-2 log-decay of state slice q
  int B, H, L, window, n_meta;
  int nchunks, P, seg_chunks;
  // The state pass cuts each of the segments 0..P-2 into R slices of sub_chunks
  // chunks (NS = (P-1) R slices per head) so that it runs more blocks than the
  // output pass; segment p >= 1 starts from the state after slice pR - 1.
  int R, sub_chunks;
  float scale;
  int gate_is_log;
  int gate_mode;  // 0: one gate per feature [BH][L][f]; 1: per token [BH][L]; 2: per head [H]
};

// Output pass with two waves per 16-token tile (chunk_out.hip); `swa` adds the
// window part.  blocks = heads x segments.
hipError_t launch_chunk_out(const ChunkParams &p, bool swa, int blocks, hipStream_t stream);

namespace {

constexpr int kC = 64;      // chunk (tokens)
constexpr int kD = 128;     // q/k head dim
constexpr int kF = 128;     // feature dim
constexpr int kF2 = 64;     // Hedgehog half
constexpr int kDV = 128;    // value dim
constexpr int kFrag = 1024; // bytes of one MFMA operand fragment
constexpr int kHalf = 512;  // bytes of a half fragment (4 bf16 per lane)


// ---------------------------------------------------------------- helpers
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int j = 0; j < 8; ++j) z[j] = (bf16)0.0f;
  return z;
}

__device__ __forceinline__ bf16x8 pack8(const float *x) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (bf16)x[j];
  return r;
}

__device__ __forceinline__ bf16x8 pack44(f32x4 lo, f32x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = (bf16)lo[j];
    r[4 + j] = (bf16)hi[j];
  }
  return r;
}

__device__ __forceinline__ bf16x8 lds8(const char *base) { return *(const bf16x8 *)base; }

// Compiler-only ordering point for memory operations: loads written before it are
// issued before it, so a group of LDS operand loads is in flight together rather
// than one load per MFMA.  Emits no instruction.
__device__ __forceinline__ void issue_fence() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void sts8(char *base, bf16x8 x) { *(bf16x8 *)base = x; }

__device__ __forceinline__ bf16x8 join44(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    r[j] = lo[j];
    r[4 + j] = hi[j];
  }
  return r;
}

// reductions over the 4 lane groups (lanes n, n+16, n+32, n+48): the gfx950 row
// swaps of rows_reduce (device_common.hpp), no LDS
__device__ __forceinline__ float grp_max(float x) { return rows_reduce(x, OpMax()); }
__device__ __forceinline__ float grp_min(float x) { return rows_reduce(x, OpMin()); }
__device__ __forceinline__ float grp_sum(float x) { return rows_reduce(x, OpAdd()); }

// inclusive scan over the 16 lanes of a row (the 16 tokens of a tile)
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float row_scan(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}

// broadcast lane 15 of each 16-lane row (the tile's last token) to the row
__device__ __forceinline__ float row_bcast15(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x15F,
                                                               0xF, 0xF, false));
}

// Largest per-token base-2 decay exponent (-log2 of the gate) used by the
// chunkwise path.  A 16-token tile then spans at most 2^{+-231}, so with the
// mid-tile reference every fold factor stays within 2^{+-116}.  Gates below e^{-10}
// (~4.5e-5) act as 4.5e-5: any term they touch is already below 4.5e-5 of its
// undecayed size, so the change is bounded by that factor.
constexpr float kMaxLog2Decay = 10.0f * kLog2e;

// Largest |chunk log2-decay| for which one chunk-wide fold reference is used:
// the fold exponents then stay within 2^{+-100}.
constexpr float kChunkRefLimit = 200.0f;

// value of x in lane SRC (0..15) of this lane's 16-lane row (DPP row_newbcast)
template <int SRC>
__device__ __forceinline__ float row_bcast_c(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               0x150 + SRC, 0xF, 0xF, true));
}
// the same for an index that is a constant after unrolling (the switch folds)
__device__ __forceinline__ float row_bcast(float x, int src) {
  switch (src & 15) {
    case 0: return row_bcast_c<0>(x);
    case 1: return row_bcast_c<1>(x);
    case 2: return row_bcast_c<2>(x);
    case 3: return row_bcast_c<3>(x);
    case 4: return row_bcast_c<4>(x);
    case 5: return row_bcast_c<5>(x);
    case 6: return row_bcast_c<6>(x);
    case 7: return row_bcast_c<7>(x);
    case 8: return row_bcast_c<8>(x);
    case 9: return row_bcast_c<9>(x);
    case 10: return row_bcast_c<10>(x);
    case 11: return row_bcast_c<11>(x);
    case 12: return row_bcast_c<12>(x);
    case 13: return row_bcast_c<13>(x);
    case 14: return row_bcast_c<14>(x);
    default: return row_bcast_c<15>(x);
  }
}

// feature index of fold slot i (0..31) of lane group g: phi+ half then phi- half
__device__ __forceinline__ int feat(int g, int i) { return 64 * (i >> 4) + 16 * g + (i & 15); }

// d_v column held by lane n, column-tile dt, of wave w (state pass and output
// pass): the two column tiles of a lane are adjacent columns, so one dword of a
// value row feeds both
__device__ __forceinline__ int dvpair(int w, int dt, int n) { return 32 * w + 2 * n + dt; }

// 0/1 selection operand: as the B operand of a 16x16x32 MFMA, output column n
// picks K-slot (group n/4, element 4*dt + n%4).  A x sel(dt) re-lays a
// row-per-lane operand (lane = row, 8 K-values) into accumulator form
// (lane = column, 4 consecutive rows): a transpose on the matrix core, exact
// for bf16 inputs since every output is one input times 1.
__device__ __forceinline__ bf16x8 select_operand(int dt) {
  const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
  bf16x8 b;
#pragma unroll
  for (int j = 0; j < 8; ++j) b[j] = (bf16)((g == (n >> 2) && j == 4 * dt + (n & 3)) ? 1.0f : 0.0f);
  return b;
}

__device__ __forceinline__ bf16x4 pack4(f32x4 x) {
  bf16x4 r;
#pragma unroll
  for (int j = 0; j < 4; ++j) r[j] = (bf16)x[j];
  return r;
}

// Per-head buffer resources over the [L][128] bf16 rows of q, k, v, gate and o.
// Loads past the last row return zeros and stores there are dropped by the range
// check of the buffer instructions (offsets are unsigned, so rows before 0 are
// past the end too); every consumer masks such tokens anyway.
struct HeadBufs {
  __amdgpu_buffer_rsrc_t q, k, v, g, o;
  int gmode;   // gate layout (ChunkParams::gate_mode)
  unsigned L;  // tokens
};
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const bf16 *base, size_t bh, int L) {
  return __builtin_amdgcn_make_buffer_rsrc((void *)(base + bh * (size_t)L * kD), (short)0, L * kD * 2,
                                           0x00020000);
}
__device__ __forceinline__ HeadBufs head_bufs(const ChunkParams &p, size_t bh) {
  // the gates: [L][128] rows (per feature), [L] (per token) or the head's one value
  __amdgpu_buffer_rsrc_t g;
  if (p.gate_mode == 1)
    g = __builtin_amdgcn_make_buffer_rsrc((void *)(p.gate + bh * (size_t)p.L), (short)0, p.L * 2, 0x00020000);
  else if (p.gate_mode == 2)
    g = __builtin_amdgcn_make_buffer_rsrc((void *)(p.gate + bh % (size_t)p.H), (short)0, 2, 0x00020000);
  else
    g = head_rsrc(p.gate, bh, p.L);
  return {head_rsrc(p.q, bh, p.L), head_rsrc(p.k, bh, p.L), head_rsrc(p.v, bh, p.L), g,
          head_rsrc(p.o, bh, p.L), p.gate_mode, (unsigned)p.L};
}
__device__ __forceinline__ bf16x8 bload(__amdgpu_buffer_rsrc_t r, unsigned off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}
// byte offset of chunk c's rows (wraps for c < 0, which reads zeros)
__device__ __forceinline__ unsigned chunk_off(int c) { return (unsigned)c * (unsigned)(kC * kD * 2); }
// Per-lane byte offsets within a chunk, lane (n, g) of tile t on token 16t + n:
// token-row operand x[token][32g + 8s + j], values v[token][32s + 8g + j] and
// gates gate[token][feat(g, 8s + j)]
__device__ __forceinline__ unsigned row_off(int tile) { return (unsigned)(16 * tile + (threadIdx.x & 15)) * (kD * 2); }
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t r, unsigned base, bf16x8 *x) {
  const unsigned g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) x[s] = bload(r, base + 64 * g + 16 * s);
}
__device__ __forceinline__ void load_vals(__amdgpu_buffer_rsrc_t r, unsigned base, bf16x8 *x) {
  const unsigned g = (threadIdx.x & 63) >> 4;
#pragma unroll
  for (int s = 0; s < 4; ++s) x[s] = bload(r, base + 16 * g + 64 * s);
}
// A scalar log-gate of the lane's token (base = byte offset of its [128] row, as
// for the per-feature layout) for every fold slot: per-token gates read element
// base / 256, the per-head gate its one value (0 for tokens past the end, so
// they add no decay; past-end per-token gates read 0 through the range check).
__device__ __forceinline__ bf16x8 scalar_gate(const HeadBufs &hb, unsigned base) {
  const unsigned tok = base >> 8;
  unsigned raw;
  if (hb.gmode == 1)
    raw = __builtin_amdgcn_raw_buffer_load_b16(hb.g, (int)(2 * tok), 0, 0);
  else
    raw = tok < hb.L ? __builtin_amdgcn_raw_buffer_load_b16(hb.g, 0, 0, 0) : 0u;
  const unsigned w = (raw & 0xFFFFu) * 0x10001u;
  return __builtin_bit_cast(bf16x8, (u32x4){w, w, w, w});
}
// SG: the scalar layouts (per token or per head), a compile-time choice so the
// per-feature kernels carry no branch for them
template <bool SG>
__device__ __forceinline__ void load_gates(const HeadBufs &hb, unsigned base, bf16x8 *x) {
  const unsigned g = (threadIdx.x & 63) >> 4;
  if constexpr (SG) {
    const bf16x8 s1 = scalar_gate(hb, base);
#pragma unroll
    for (int s = 0; s < 4; ++s) x[s] = s1;
    return;
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) x[s] = bload(hb.g, base + 2 * feat(g, 8 * s));
}
// Unnormalised Hedgehog exponentials of the lane's token: e[4mt + j] =
// 2^{(u - max u) log2e} (phi+ feature 16g + 4mt + j) and e[16 + 4mt + j] =
// 2^{(min u - u) log2e} (phi- feature 64 + 16g + 4mt + j), and the reciprocal
// normalisers of the two halves.
__device__ __forceinline__ void hedgehog_exp(const f32x4 *u, float *e, float &izp, float &izn) {
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      mx = fmaxf(mx, u[mt][j]);
      mn = fminf(mn, u[mt][j]);
    }
  mx = grp_max(mx) * kLog2e;
  mn = grp_min(mn) * kLog2e;
  float zp = 0.0f, zn = 0.0f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = 4 * mt + j;
      e[i] = exp2_fast(u[mt][j] * kLog2e - mx);
      e[16 + i] = exp2_fast(mn - u[mt][j] * kLog2e);
      zp += e[i];
      zn += e[16 + i];
    }
  izp = rcp_fast(grp_sum(zp));
  izn = rcp_fast(grp_sum(zn));
}

// u = x Wphi for a 16-token tile (A = Wphi^T fragments in LDS, B = the tile's
// token rows); the 4 fragments of tile mt+1 are requested before the MFMAs of mt
__device__ __forceinline__ void project(const char *wb, const bf16x8 *x, f32x4 *u) {
  bf16x8 wf[2][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) u[mt] = (f32x4){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) wf[0][s] = lds8(wb + s * kFrag);
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    if (mt + 1 < 4) {
#pragma unroll
      for (int s = 0; s < 4; ++s) wf[(mt + 1) & 1][s] = lds8(wb + ((mt + 1) * 4 + s) * kFrag);
    }
    issue_fence();
#pragma unroll
    for (int s = 0; s < 4; ++s) u[mt] = mfma(wf[mt & 1][s], x[s], u[mt]);
  }
}

// Running decay exponents of the lane's token in a 16-token tile: dn[i] is the
// sum over tokens s <= n of -log2 Gamma_s for fold slot i (feature feat(g, i)),
// so the in-tile inclusive cumsum of the base-2 log-gates is b = -dn.  The gate
// input is the logit g (Gamma = sigmoid(g), -log2 Gamma = log2(1 + 2^{-g log2e}))
// or, with gate_is_log, log Gamma itself.  The power's exponent is capped at
// kMaxLog2Decay, which caps each term at kMaxLog2Decay + 2^{-kMaxLog2Decay}/ln 2.
// Tokens past the end (!tok_ok) contribute 0: their gates read as 0 (range
// check), which gives 0 in the log form, and a cap of -inf gives log2(1 + 0) = 0
// in the logit form.  NV slots starting at the first of xg (NV/8 fragments).
template <int NV = 32>
__device__ __forceinline__ void tile_decay(const bf16x8 *xg, bool gate_is_log, bool tok_ok, float *dn) {
  if (gate_is_log) {  // one uniform branch around the whole loop
#pragma unroll
    for (int i = 0; i < NV; ++i) dn[i] = fminf((float)xg[i >> 3][i & 7] * -kLog2e, kMaxLog2Decay);
  } else {
    float cap = tok_ok ? kMaxLog2Decay : -INFINITY;
    asm volatile("" : "+v"(cap));  // opaque: one min per value, no select after it
#pragma unroll
    for (int i = 0; i < NV; ++i)
      dn[i] = log2_fast(1.0f + exp2_fast(fminf((float)xg[i >> 3][i & 7] * -kLog2e, cap)));
  }
  // one scan step across all slots at a time, so consecutive DPP reads never
  // wait on each other
#pragma unroll
  for (int i = 0; i < NV; ++i) dn[i] += row_shr<1>(dn[i]);
#pragma unroll
  for (int i = 0; i < NV; ++i) dn[i] += row_shr<2>(dn[i]);
#pragma unroll
  for (int i = 0; i < NV; ++i) dn[i] += row_shr<4>(dn[i]);
#pragma unroll
  for (int i = 0; i < NV; ++i) dn[i] += row_shr<8>(dn[i]);
}

}  // namespace

}  // namespace glah

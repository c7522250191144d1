// launch.hpp -- host-side launchers of the HIP kernels (internal to the library;
// the public interface is include/glahybrid.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace glah {

enum { PART_GLA = 1, PART_SWA = 2, PART_BOTH = 3 };

// One call's arguments after validation (sizes checked, scale resolved).
struct LayerArgs {
  int B = 0, H = 0, L = 0, d = 0, dv = 0, f = 0;
  int window = 0, n_meta = 0, chunk = 64;
  float scale = 1.0f;
  bool bf16 = true;
  bool gate_is_log = false;
  // gate layout: 0 = one per feature [BH][L][f], 1 = one per token [BH][L],
  // 2 = one per head [H] (1 and 2 are log-gates)
  int gate_mode = 0;
  const void *q = nullptr, *k = nullptr, *v = nullptr, *gate = nullptr;
  const void *wq = nullptr, *wk = nullptr;
  const void *beta = nullptr;        // gated delta rule: write strength per token
  const float *meta = nullptr;
  const float *state_in = nullptr;
  float *state_out = nullptr;
  float *state = nullptr;            // decode: in/out
  void *o = nullptr;
  void *kcache = nullptr, *vcache = nullptr;
  const int32_t *pos = nullptr;      // decode
  void *ws = nullptr;
  size_t ws_bytes = 0;
  hipStream_t stream = nullptr;
};

// Limits of the token-recurrent VALU kernels (any dtype, general sizes).
constexpr int kRecMaxD = 256;
constexpr int kRecMaxF = 256;
constexpr int kRecMaxWindow = 4096;
constexpr int kRecMaxMeta = 64;

bool recurrent_supported(const LayerArgs &a, int parts);
hipError_t launch_recurrent_prefill(const LayerArgs &a, int parts);
hipError_t launch_decode_step(const LayerArgs &a, int parts);
hipError_t launch_window_cache(const LayerArgs &a);
// state_out of an empty sequence (L = 0): the state before it, state_in or zeros
hipError_t launch_state_passthrough(const LayerArgs &a);

// Bandwidth-oriented decode step at d = f = d_v = 128, window <= 64.
bool decode128_supported(const LayerArgs &a, int parts);
hipError_t launch_decode128(const LayerArgs &a, int parts);

// Chunkwise MFMA path (bf16, d = f = d_v = 128).
bool chunked_supported(const LayerArgs &a, int parts);
size_t chunked_workspace_bytes(const LayerArgs &a, int parts);
// ring: also write the decode ring (a.kcache, a.vcache) of the last `window` keys
// and values (the bf16 matrix-core path, from each head's last segment)
hipError_t launch_chunked_prefill(const LayerArgs &a, int parts, bool ring = false);

// Device scratch of hybrid_layer_fwd_noalloc (chunked.hip): a static device
// array of kNoAllocScratchBytes per device; *ptr receives the current device's
// copy (looked up once per device).
constexpr size_t kNoAllocScratchBytes = (size_t)40 << 20;
constexpr int kMaxDevices = 64;
hipError_t noalloc_scratch(void **ptr);

// Banded MFMA window attention (bf16, d = d_v = 128).
bool swa_mfma_supported(const LayerArgs &a);
hipError_t launch_swa_mfma(const LayerArgs &a);

// Window attention for any window (bf16, d = d_v = 128): online softmax over
// 64-key chunks on the matrix cores (swa_wide.hip); accumulate: o += o_swa.
bool swa_wide_supported(const LayerArgs &a);
hipError_t launch_swa_wide(const LayerArgs &a, bool accumulate);

// Backward of the layer (token-recurrent VALU kernels, any dtype).
constexpr int kBwdMaxD = 128;        // d_qk and d_v
constexpr int kBwdMaxF = 128;        // f (f/2 a power of two)
constexpr int kBwdMaxWindow = 1024;

struct BwdArgs {
  const void *dout = nullptr;        // dO, the layout of o
  const float *dstate_out = nullptr; // gradient of the final state (nullable)
  void *dq = nullptr, *dk = nullptr, *dv = nullptr, *dgate = nullptr;  // input dtype
  float *dwq = nullptr, *dwk = nullptr, *dmeta = nullptr, *dstate_in = nullptr;
};
bool bwd_supported(const LayerArgs &a, int parts);
// workspace the sizing query reports (the whole call's, or a sub-problem's when
// that exceeds 1.5e9 bytes) and the least any call accepts (one row and one head
// at a time); launch_layer_bwd runs the fewest sub-problems that fit a.ws_bytes
size_t bwd_workspace_bytes(const LayerArgs &a, int parts);
size_t bwd_workspace_min_bytes(const LayerArgs &a, int parts);
size_t bwd_workspace_whole_bytes(const LayerArgs &a, int parts);  // no sub-problems
hipError_t launch_layer_bwd(const LayerArgs &a, const BwdArgs &g, int parts);

// Window part of the backward on the matrix cores (bwd_window.hip): bf16,
// d = d_v = 128, window <= 64, n_meta <= 64.  Writes the window part's dq, dk,
// dv (bf16 [B][H][L][128]; dv optionally added to the values already there)
// and the sink-gradient partial of every 64-token chunk ([B H][chunks][n_meta]).
struct WinBwdArgs {
  const void *q = nullptr, *k = nullptr, *v = nullptr, *dout = nullptr;
  const float *meta = nullptr;
  float *mp = nullptr;
  void *dq = nullptr, *dk = nullptr, *dv = nullptr;  // bf16
  bool add_dv = false;  // add dv to the bf16 values already there
  int B = 0, H = 0, L = 0, window = 0, n_meta = 0;
  float scale = 1.0f;
};
bool bwd_window_mfma_supported(int d, int dv, int window, int n_meta, bool bf16);
hipError_t launch_bwd_window_mfma(const WinBwdArgs &a, hipStream_t stream);

// State walks of the gated part's backward on the matrix cores (bwd_walk.hip):
// bf16 values, f = d_v = 128.  From the prologue's fp32 feature maps and the
// in-tile cumsum b of the floored log-gate ([B H L][128], 16-token tiles) it
// writes dphiq, dphik and dv of the gated part ([B H L][128], complete sums),
// the 64-token tile sums of phiq . dphiq and phik . dphik ([B H][tiles][128]),
// S_{L-1} . dS_final and Gamma_0 (S_in . dS_0) ([2][B H][128]) and dS_in.  ws
// holds bwd_walk_ws_floats(B H, L) floats of segment states.
struct WalkArgs {
  const float *pq = nullptr, *pk = nullptr, *gb = nullptr;
  const void *v = nullptr, *dout = nullptr;
  const float *state_in = nullptr, *dstate_out = nullptr;
  float *dpq = nullptr, *dpk = nullptr, *dvg = nullptr, *tq = nullptr, *tk = nullptr, *xs = nullptr;
  float *dstate_in = nullptr, *ws = nullptr;
  void *dv = nullptr;  // bf16 [B H L][128] (dv_mode 1)
  int BH = 0, L = 0, nft = 0;
  int dv_mode = 0;  // the gated part's dv: 0 to dvg (fp32), 1 to dv (bf16)
};
bool bwd_walk_supported(int f, int dv, int L, bool bf16);
size_t bwd_walk_ws_floats(int BH, int L);
hipError_t launch_bwd_walk(const WalkArgs &a, hipStream_t stream);

// Per-token part of the backward on the matrix cores (bwd_feat.hip): bf16,
// d = f = d_v = 128, one gate per feature.  From the feature maps and their
// gradients (fp32 [B H L][128]), the gated part's dv, d log Gamma at every
// 64-token tile's first token and the window part's dq, dk, dv (bf16 when
// win_bf16, else fp32; or null), it
// writes dq, dk, dv, the gate gradient and one dW partial per block
// ([B H][blocks][128][64], blocks = ceil(ceil(L / 16) / bwd_feat_span)).
struct FeatArgs {
  const void *q = nullptr, *k = nullptr, *gate = nullptr, *wq = nullptr, *wk = nullptr;
  const float *pq = nullptr, *pk = nullptr, *dpq = nullptr, *dpk = nullptr, *ta = nullptr;
  bool swa = false;  // dq and dk hold the window part's gradient (bf16) on entry
  void *dq = nullptr, *dk = nullptr, *dg = nullptr;
  float *wqp = nullptr, *wkp = nullptr;
  int BH = 0, H = 0, L = 0, nft = 0;
  bool gate_is_log = false;
};
bool bwd_feat_mfma_supported(int d, int f, int dv, int L, int gate_mode, bool bf16);
int bwd_feat_span(int BH, int L);
hipError_t launch_bwd_feat_mfma(const FeatArgs &a, hipStream_t stream);

// Backward prologue on the matrix cores (bwd_prep.hip): bf16, d = f = 128.
// Writes phi(q), phi(k) and the in-tile cumsum of the floored log-gate (fp32
// [B H L][128], 16-token tiles) for the tile walks.
struct PrepArgs {
  const void *q = nullptr, *k = nullptr, *gate = nullptr, *wq = nullptr, *wk = nullptr;
  float *pq = nullptr, *pk = nullptr, *gb = nullptr;
  int BH = 0, H = 0, L = 0, gate_mode = 0;
  bool gate_is_log = false;
};
bool bwd_prep_mfma_supported(int d, int f, int L, bool bf16);
hipError_t launch_bwd_prep_mfma(const PrepArgs &a, hipStream_t stream);

// Gated delta rule (token-recurrent prefill, bandwidth-bound decode step):
// q, k [B][H][L][d], v and o [B][H][L][dv], log-decay (gate) and beta [B][H][L],
// state [B][H][dv][d] fp32.
bool delta_supported(const LayerArgs &a);
hipError_t launch_delta(const LayerArgs &a, bool decode);
// Chunkwise prefill on the matrix cores (delta_chunk.hip): bf16, d = 128,
// d_v a multiple of 16, at least one 64-token chunk.  Its per-chunk records
// (T, P, per-token scalars) go to the workspace a.ws of delta_chunk_ws_bytes(a)
// bytes (0 where the chunkwise path does not apply).
bool delta_chunk_supported(const LayerArgs &a);
size_t delta_chunk_ws_bytes(const LayerArgs &a);
hipError_t launch_delta_chunk(const LayerArgs &a);

// Continuation prefill (serving.hip): window part of the first w - 1 queries
// reaching into the input ring, and the ring after the call (global positions).
bool halo_supported(const LayerArgs &a);
hipError_t launch_halo_fix(const LayerArgs &a, long start, const void *kcache_in, const void *vcache_in);
hipError_t launch_ring_cont(const LayerArgs &a, long start, const void *kcache_in, const void *vcache_in);
// o <- o * sigmoid(g) over n elements
hipError_t launch_output_gate(void *o, const void *g, size_t n, bool is_bf16, hipStream_t stream);

int device_cu_count();

}  // namespace glah

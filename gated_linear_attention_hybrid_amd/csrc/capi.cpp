// capi.cpp -- the C ABI of the library (include/glahybrid.h): argument checks,
// choice of kernel path, launches on the caller's stream.  No entry point
// allocates memory, synchronises, or lets an exception cross the boundary.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "glahybrid.h"
#include "launch.hpp"

using namespace glah;

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

// Entry-point kinds: which parts of the layer they compute.
enum class Op { kGlaPrefill, kSwa, kHybrid, kDecode };

int parts_of(Op op, const glah_desc *d) {
  switch (op) {
    case Op::kGlaPrefill: return PART_GLA;
    case Op::kSwa: return PART_SWA;
    case Op::kHybrid: return PART_BOTH;
    case Op::kDecode: return PART_GLA | (d->window > 0 ? PART_SWA : 0);
  }
  return 0;
}

// Size and enum checks shared by every entry point.
glah_status check_desc(const glah_desc *d, Op op, LayerArgs &a) {
  if (!d) return GLAH_EINVAL;
  const int parts = parts_of(op, d);
  if (d->B < 0 || d->H < 0 || d->d_qk <= 0 || d->d_v <= 0 || d->n_meta < 0) return GLAH_EINVAL;
  if (op != Op::kDecode && d->L < 0) return GLAH_EINVAL;
  if ((parts & PART_GLA) && (d->f <= 0 || (d->f & 1))) return GLAH_EINVAL;
  if ((parts & PART_SWA) && d->window < 1) return GLAH_EINVAL;
  if (op == Op::kDecode && d->window < 0) return GLAH_EINVAL;
  if (d->dtype != GLAH_BF16 && d->dtype != GLAH_F32) return GLAH_EINVAL;
  if (d->gate_kind != GLAH_GATE_LOGITS && d->gate_kind != GLAH_GATE_LOG && d->gate_kind != GLAH_GATE_LOG_TOKEN &&
      d->gate_kind != GLAH_GATE_LOG_HEAD)
    return GLAH_EINVAL;
  if (d->chunk != 0 && d->chunk != 16 && d->chunk != 32 && d->chunk != 64 && d->chunk != 128)
    return GLAH_EINVAL;
  // element counts must stay far from overflow of 64-bit offsets and of the
  // 32-bit grid sizes used by the kernels
  const double L = op == Op::kDecode ? 1.0 : (double)d->L;
  const double rows = (double)d->B * d->H * L;
  const double widest = fmax(fmax((double)d->d_qk, (double)d->d_v), (double)d->f);
  if (rows * widest > 9.0e15 || (double)d->B * d->H * (d->window + 1.0) > 1.0e9) return GLAH_EINVAL;
  if ((double)d->f * d->d_v > 1.0e8) return GLAH_EINVAL;

  a.B = d->B; a.H = d->H; a.L = op == Op::kDecode ? 1 : d->L;
  a.d = d->d_qk; a.dv = d->d_v; a.f = (parts & PART_GLA) ? d->f : 2;
  a.window = (parts & PART_SWA) ? d->window : 0;
  a.n_meta = (parts & PART_SWA) ? d->n_meta : 0;
  a.chunk = d->chunk == 0 ? 64 : d->chunk;
  a.scale = d->scale > 0.0f ? d->scale : 1.0f / sqrtf((float)d->d_qk);
  a.bf16 = d->dtype == GLAH_BF16;
  a.gate_is_log = d->gate_kind != GLAH_GATE_LOGITS;
  a.gate_mode = d->gate_kind == GLAH_GATE_LOG_TOKEN ? 1 : d->gate_kind == GLAH_GATE_LOG_HEAD ? 2 : 0;
  return GLAH_OK;
}

// A required pointer must be non-null (unless the call has no work) and
// 16-byte aligned; an optional one must be aligned when given.
bool req(const void *p, bool has_work) { return has_work ? (p && aligned16(p)) : aligned16(p); }
bool opt(const void *p) { return aligned16(p); }

glah_status finish(hipError_t e) { return e == hipSuccess ? GLAH_OK : GLAH_EHIP; }

// Descriptor of the gated delta rule: B, H, L (prefill), d_qk, d_v, dtype.
glah_status check_delta_desc(const glah_desc *d, bool decode, LayerArgs &a) {
  if (!d) return GLAH_EINVAL;
  if (d->B < 0 || d->H < 0 || d->d_qk <= 0 || d->d_v <= 0 || (!decode && d->L < 0)) return GLAH_EINVAL;
  if (d->dtype != GLAH_BF16 && d->dtype != GLAH_F32) return GLAH_EINVAL;
  const double L = decode ? 1.0 : (double)d->L;
  if ((double)d->B * d->H * L * fmax((double)d->d_qk, (double)d->d_v) > 9.0e15 ||
      (double)d->B * d->H * ((double)d->d_v + 15.0) / 16.0 > 2.0e9)
    return GLAH_EINVAL;
  a.B = d->B; a.H = d->H; a.L = decode ? 1 : d->L;
  a.d = d->d_qk; a.dv = d->d_v; a.f = d->d_qk;  // the state is d_v x d_qk
  a.bf16 = d->dtype == GLAH_BF16;
  return delta_supported(a) ? GLAH_OK : GLAH_ENOTSUP;
}

// hybrid_layer_fwd with the workspace given: checks, then the chunked MFMA path
// (or the token-recurrent one), then the ring copy.
glah_status hybrid_fwd(const glah_desc *desc, const void *q, const void *k, const void *v, const void *gate,
                       const void *wphi_q, const void *wphi_k, const float *meta, const float *state_in,
                       float *state_out, void *kcache_out, void *vcache_out, void *o, void *ws, size_t ws_bytes,
                       hipStream_t stream) {
  LayerArgs a;
  glah_status st = check_desc(desc, Op::kHybrid, a);
  if (st != GLAH_OK) return st;
  const bool work = (size_t)a.B * a.H * a.L > 0;
  const bool heads = (size_t)a.B * a.H > 0;
  if (!req(q, work) || !req(k, work) || !req(v, work) || !req(gate, work) || !req(o, work) ||
      !req(wphi_q, heads) || !req(wphi_k, heads) || !req(meta, a.n_meta > 0 && a.H > 0) ||
      !opt(state_in) || !opt(state_out) || !opt(ws) || !opt(kcache_out) || !opt(vcache_out))
    return GLAH_EINVAL;
  if ((kcache_out == nullptr) != (vcache_out == nullptr)) return GLAH_EINVAL;
  a.q = q; a.k = k; a.v = v; a.gate = gate; a.wq = wphi_q; a.wk = wphi_k; a.meta = meta;
  a.state_in = state_in; a.state_out = state_out; a.o = o;
  a.kcache = kcache_out; a.vcache = vcache_out;
  a.ws = ws; a.ws_bytes = ws_bytes; a.stream = stream;
  hipError_t e;
  if (a.L == 0) {  // no tokens: the state passes through, the ring is all zeros
    e = launch_state_passthrough(a);
    if (e == hipSuccess && kcache_out) e = launch_window_cache(a);
    return finish(e);
  }
  if (chunked_supported(a, PART_BOTH)) {
    if (ws_bytes < chunked_workspace_bytes(a, PART_BOTH) || (!ws && chunked_workspace_bytes(a, PART_BOTH)))
      return GLAH_EWORKSPACE;
    e = launch_chunked_prefill(a, PART_BOTH, kcache_out != nullptr);  // the ring from the output pass
    if (e == hipSuccess) return finish(e);
  } else if (chunked_supported(a, PART_GLA) && swa_wide_supported(a)) {
    // windows wider than one chunk: the gated part in the chunked kernels, then
    // the window part with an online softmax over key chunks, added to o
    if (ws_bytes < chunked_workspace_bytes(a, PART_GLA) || (!ws && chunked_workspace_bytes(a, PART_GLA)))
      return GLAH_EWORKSPACE;
    e = launch_chunked_prefill(a, PART_GLA);
    if (e == hipSuccess) e = launch_swa_wide(a, true);
  } else {
    if (!recurrent_supported(a, PART_BOTH)) return GLAH_ENOTSUP;
    e = launch_recurrent_prefill(a, PART_BOTH);
  }
  if (e == hipSuccess && kcache_out) e = launch_window_cache(a);
  return finish(e);
}

}  // namespace

extern "C" {

const char *glah_status_str(int status) {
  switch (status) {
    case GLAH_OK: return "ok";
    case GLAH_EINVAL: return "invalid argument";
    case GLAH_ENOTSUP: return "unsupported size or dtype combination";
    case GLAH_EWORKSPACE: return "workspace missing or too small";
    case GLAH_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

int glah_version(void) { return (0 << 16) | 1; }

size_t glah_workspace_bytes(const glah_desc *desc) {
  LayerArgs a;
  if (!desc) return (size_t)-1;
  // the hybrid call needs the most: the state pass of the gated part
  if (check_desc(desc, Op::kHybrid, a) != GLAH_OK && check_desc(desc, Op::kGlaPrefill, a) != GLAH_OK)
    return (size_t)-1;
  if (!chunked_supported(a, PART_GLA)) return 0;
  return chunked_workspace_bytes(a, PART_GLA);
}

glah_status gla_prefill(const glah_desc *desc, const void *q, const void *k, const void *v,
                        const void *gate, const void *wphi_q, const void *wphi_k,
                        const float *state_in, float *state_out, void *o, void *ws,
                        size_t ws_bytes, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_desc(desc, Op::kGlaPrefill, a);
    if (st != GLAH_OK) return st;
    const bool work = (size_t)a.B * a.H * a.L > 0;
    const bool heads = (size_t)a.B * a.H > 0;
    if (!req(q, work) || !req(k, work) || !req(v, work) || !req(gate, work) || !req(o, work) ||
        !req(wphi_q, heads) || !req(wphi_k, heads) || !opt(state_in) || !opt(state_out) || !opt(ws))
      return GLAH_EINVAL;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.wq = wphi_q; a.wk = wphi_k;
    a.state_in = state_in; a.state_out = state_out; a.o = o;
    a.ws = ws; a.ws_bytes = ws_bytes; a.stream = (hipStream_t)stream;
    if (a.L == 0) return finish(launch_state_passthrough(a));
    if (chunked_supported(a, PART_GLA)) {
      if (ws_bytes < chunked_workspace_bytes(a, PART_GLA) || (!ws && chunked_workspace_bytes(a, PART_GLA)))
        return GLAH_EWORKSPACE;
      return finish(launch_chunked_prefill(a, PART_GLA));
    }
    if (!recurrent_supported(a, PART_GLA)) return GLAH_ENOTSUP;
    return finish(launch_recurrent_prefill(a, PART_GLA));
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status swa_meta_attn(const glah_desc *desc, const void *q, const void *k, const void *v,
                          const float *meta, void *o, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_desc(desc, Op::kSwa, a);
    if (st != GLAH_OK) return st;
    const bool work = (size_t)a.B * a.H * a.L > 0;
    if (!req(q, work) || !req(k, work) || !req(v, work) || !req(o, work) ||
        !req(meta, a.n_meta > 0 && a.H > 0))
      return GLAH_EINVAL;
    a.q = q; a.k = k; a.v = v; a.meta = meta; a.o = o; a.stream = (hipStream_t)stream;
    if (swa_mfma_supported(a)) return finish(launch_swa_mfma(a));
    if (swa_wide_supported(a)) return finish(launch_swa_wide(a, false));
    if (!recurrent_supported(a, PART_SWA)) return GLAH_ENOTSUP;
    return finish(launch_recurrent_prefill(a, PART_SWA));
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status hybrid_layer_fwd(const glah_desc *desc, const void *q, const void *k, const void *v,
                             const void *gate, const void *wphi_q, const void *wphi_k,
                             const float *meta, const float *state_in, float *state_out,
                             void *kcache_out, void *vcache_out, void *o, void *ws,
                             size_t ws_bytes, glah_stream_t stream) {
  try {
    return hybrid_fwd(desc, q, k, v, gate, wphi_q, wphi_k, meta, state_in, state_out, kcache_out, vcache_out, o,
                      ws, ws_bytes, (hipStream_t)stream);
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status hybrid_layer_fwd_noalloc(const glah_desc *desc, const void *q, const void *k, const void *v,
                                     const void *gate, const void *wphi_q, const void *wphi_k,
                                     const float *meta, const float *state_in, float *state_out,
                                     void *kcache_out, void *vcache_out, void *o, glah_stream_t stream) {
  try {
    void *scratch = nullptr;
    if (noalloc_scratch(&scratch) != hipSuccess) return GLAH_EHIP;
    // a call whose segment states would not fit the scratch array is rejected
    // with GLAH_EWORKSPACE before anything is launched
    return hybrid_fwd(desc, q, k, v, gate, wphi_q, wphi_k, meta, state_in, state_out, kcache_out, vcache_out, o,
                      scratch, kNoAllocScratchBytes, (hipStream_t)stream);
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status gla_decode_step(const glah_desc *desc, const void *q_t, const void *k_t,
                            const void *v_t, const void *gate_t, const void *wphi_q,
                            const void *wphi_k, const float *meta, float *state, void *kcache,
                            void *vcache, const int32_t *pos, void *o_t, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_desc(desc, Op::kDecode, a);
    if (st != GLAH_OK) return st;
    const int parts = parts_of(Op::kDecode, desc);
    const bool work = (size_t)a.B * a.H > 0;
    if (!req(q_t, work) || !req(k_t, work) || !req(v_t, work) || !req(gate_t, work) ||
        !req(wphi_q, work) || !req(wphi_k, work) || !req(state, work) || !req(pos, work) ||
        !req(o_t, work))
      return GLAH_EINVAL;
    if ((parts & PART_SWA) && (!req(kcache, work) || !req(vcache, work) ||
                               !req(meta, a.n_meta > 0 && work)))
      return GLAH_EINVAL;
    if (a.dv % 4 != 0 || !recurrent_supported(a, parts)) return GLAH_ENOTSUP;
    a.q = q_t; a.k = k_t; a.v = v_t; a.gate = gate_t; a.wq = wphi_q; a.wk = wphi_k;
    a.meta = meta; a.state = state; a.kcache = kcache; a.vcache = vcache; a.pos = pos;
    a.o = o_t; a.stream = (hipStream_t)stream;
    return finish(launch_decode_step(a, parts));
  } catch (...) {
    return GLAH_EHIP;
  }
}

size_t glah_bwd_workspace_bytes(const glah_desc *desc) {
  LayerArgs a;
  if (!desc || check_desc(desc, Op::kHybrid, a) != GLAH_OK) return (size_t)-1;
  if (!bwd_supported(a, PART_BOTH)) return 0;
  return bwd_workspace_bytes(a, PART_BOTH);
}

size_t glah_bwd_workspace_bytes_whole(const glah_desc *desc) {
  LayerArgs a;
  if (!desc || check_desc(desc, Op::kHybrid, a) != GLAH_OK) return (size_t)-1;
  if (!bwd_supported(a, PART_BOTH)) return 0;
  return bwd_workspace_whole_bytes(a, PART_BOTH);
}

glah_status hybrid_layer_bwd(const glah_desc *desc, const void *q, const void *k, const void *v,
                             const void *gate, const void *wphi_q, const void *wphi_k,
                             const float *meta, const float *state_in, const void *d_o,
                             const float *dstate_out, void *dq, void *dk, void *dv, void *dgate,
                             float *dwphi_q, float *dwphi_k, float *dmeta, float *dstate_in, void *ws,
                             size_t ws_bytes, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_desc(desc, Op::kHybrid, a);
    if (st != GLAH_OK) return st;
    const bool work = (size_t)a.B * a.H * a.L > 0;
    const bool heads = a.H > 0;
    const bool head_gate = a.gate_mode == 2 && heads;
    if (!req(q, work) || !req(k, work) || !req(v, work) || !req(gate, work || head_gate) ||
        !req(d_o, work) || !req(dq, work) || !req(dk, work) || !req(dv, work) ||
        !req(dgate, work || head_gate) || !req(wphi_q, heads) || !req(wphi_k, heads) ||
        !req(dwphi_q, heads) || !req(dwphi_k, heads) || !req(meta, a.n_meta > 0 && heads) ||
        !req(dmeta, a.n_meta > 0 && heads) || !opt(state_in) || !opt(dstate_out) || !opt(dstate_in) ||
        !opt(ws))
      return GLAH_EINVAL;
    if (!bwd_supported(a, PART_BOTH)) return GLAH_ENOTSUP;
    const size_t need = bwd_workspace_min_bytes(a, PART_BOTH);
    if (ws_bytes < need || (!ws && need)) return GLAH_EWORKSPACE;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.wq = wphi_q; a.wk = wphi_k; a.meta = meta;
    a.state_in = state_in; a.ws = ws; a.ws_bytes = ws_bytes; a.stream = (hipStream_t)stream;
    BwdArgs g;
    g.dout = d_o; g.dstate_out = dstate_out;
    g.dq = dq; g.dk = dk; g.dv = dv; g.dgate = dgate;
    g.dwq = dwphi_q; g.dwk = dwphi_k; g.dmeta = dmeta; g.dstate_in = dstate_in;
    return finish(launch_layer_bwd(a, g, PART_BOTH));
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status hybrid_layer_fwd_cont(const glah_desc *desc, int32_t start, const void *q, const void *k,
                                  const void *v, const void *gate, const void *wphi_q, const void *wphi_k,
                                  const float *meta, const float *state_in, const void *kcache_in,
                                  const void *vcache_in, float *state_out, void *kcache_out, void *vcache_out,
                                  void *o, void *ws, size_t ws_bytes, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_desc(desc, Op::kHybrid, a);
    if (st != GLAH_OK) return st;
    if (start < 0) return GLAH_EINVAL;
    const bool work = (size_t)a.B * a.H * a.L > 0;
    const bool heads = (size_t)a.B * a.H > 0;
    if (!req(q, work) || !req(k, work) || !req(v, work) || !req(gate, work) || !req(o, work) ||
        !req(wphi_q, heads) || !req(wphi_k, heads) || !req(meta, a.n_meta > 0 && a.H > 0) ||
        !req(kcache_in, start > 0 && heads) || !req(vcache_in, start > 0 && heads) || !opt(state_in) ||
        !opt(state_out) || !opt(ws) || !opt(kcache_out) || !opt(vcache_out))
      return GLAH_EINVAL;
    if ((kcache_out == nullptr) != (vcache_out == nullptr) || (kcache_in == nullptr) != (vcache_in == nullptr))
      return GLAH_EINVAL;
    if (!halo_supported(a)) return GLAH_ENOTSUP;
    a.q = q; a.k = k; a.v = v; a.gate = gate; a.wq = wphi_q; a.wk = wphi_k; a.meta = meta;
    a.state_in = state_in; a.state_out = state_out; a.o = o;
    a.ws = ws; a.ws_bytes = ws_bytes; a.stream = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (a.L == 0) {
      e = launch_state_passthrough(a);
    } else if (chunked_supported(a, PART_BOTH)) {
      if (ws_bytes < chunked_workspace_bytes(a, PART_BOTH) || (!ws && chunked_workspace_bytes(a, PART_BOTH)))
        return GLAH_EWORKSPACE;
      e = launch_chunked_prefill(a, PART_BOTH);
    } else {
      if (!recurrent_supported(a, PART_BOTH)) return GLAH_ENOTSUP;
      e = launch_recurrent_prefill(a, PART_BOTH);
    }
    // the first window - 1 queries also see the ring's keys (read before the
    // ring is rewritten, which may be in place)
    if (e == hipSuccess && a.L > 0) e = launch_halo_fix(a, start, kcache_in, vcache_in);
    if (e == hipSuccess && kcache_out) {
      a.kcache = kcache_out; a.vcache = vcache_out;
      e = launch_ring_cont(a, start, kcache_in, vcache_in);
    }
    return finish(e);
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status glah_output_gate(const glah_desc *desc, void *o, const void *g, glah_stream_t stream) {
  try {
    if (!desc || desc->B < 0 || desc->H < 0 || desc->L < 0 || desc->d_v <= 0) return GLAH_EINVAL;
    if (desc->dtype != GLAH_BF16 && desc->dtype != GLAH_F32) return GLAH_EINVAL;
    const double n = (double)desc->B * desc->H * desc->L * desc->d_v;
    if (n > 9.0e15) return GLAH_EINVAL;
    if (!req(o, n > 0) || !req(g, n > 0)) return GLAH_EINVAL;
    return finish(launch_output_gate(o, g, (size_t)n, desc->dtype == GLAH_BF16, (hipStream_t)stream));
  } catch (...) {
    return GLAH_EHIP;
  }
}

size_t gdn_workspace_bytes(const glah_desc *desc) {
  LayerArgs a;
  const glah_status st = check_delta_desc(desc, false, a);
  if (st == GLAH_ENOTSUP) return 0;
  if (st != GLAH_OK) return (size_t)-1;
  return delta_chunk_ws_bytes(a);
}

glah_status gdn_prefill(const glah_desc *desc, const void *q, const void *k, const void *v,
                        const void *log_alpha, const void *beta, const float *state_in,
                        float *state_out, void *o, void *ws, size_t ws_bytes, glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_delta_desc(desc, false, a);
    if (st != GLAH_OK) return st;
    const bool work = (size_t)a.B * a.H * a.L > 0;
    if (!req(q, work) || !req(k, work) || !req(v, work) || !req(log_alpha, work) || !req(beta, work) ||
        !req(o, work) || !opt(state_in) || !opt(state_out))
      return GLAH_EINVAL;
    a.q = q; a.k = k; a.v = v; a.gate = log_alpha; a.beta = beta;
    a.state_in = state_in; a.state_out = state_out; a.o = o; a.stream = (hipStream_t)stream;
    if (a.L == 0) return finish(launch_state_passthrough(a));  // f = d_qk: d_v x d_qk floats
    const size_t need = delta_chunk_ws_bytes(a);
    if (need && (!ws || ws_bytes < need)) return GLAH_EWORKSPACE;
    if (!opt(ws)) return GLAH_EINVAL;
    a.ws = ws; a.ws_bytes = ws_bytes;
    return finish(launch_delta(a, false));
  } catch (...) {
    return GLAH_EHIP;
  }
}

glah_status gdn_decode_step(const glah_desc *desc, const void *q_t, const void *k_t, const void *v_t,
                            const void *log_alpha_t, const void *beta_t, float *state, void *o_t,
                            glah_stream_t stream) {
  try {
    LayerArgs a;
    glah_status st = check_delta_desc(desc, true, a);
    if (st != GLAH_OK) return st;
    const bool work = (size_t)a.B * a.H > 0;
    if (!req(q_t, work) || !req(k_t, work) || !req(v_t, work) || !req(log_alpha_t, work) ||
        !req(beta_t, work) || !req(state, work) || !req(o_t, work))
      return GLAH_EINVAL;
    a.q = q_t; a.k = k_t; a.v = v_t; a.gate = log_alpha_t; a.beta = beta_t;
    a.state = state; a.o = o_t; a.stream = (hipStream_t)stream;
    return finish(launch_delta(a, true));
  } catch (...) {
    return GLAH_EHIP;
  }
}

}  // extern "C"

"""The Python binding rejects tensor arguments that the C boundary could not
detect (it sees only addresses): wrong shapes, mixed element types,
non-contiguous views and host tensors.  Every check runs before any pointer is
passed, so these tests run on the CPU."""
import pytest
import torch

from gated_linear_attention_hybrid_amd import binding as G


def layer(B=1, H=2, L=8, d=16, dv=8, f=8, M=3, dtype=torch.bfloat16):
    """CPU tensors of a valid call (they fail only the device check)."""
    return dict(q=torch.zeros(B, H, L, d, dtype=dtype), k=torch.zeros(B, H, L, d, dtype=dtype),
                v=torch.zeros(B, H, L, dv, dtype=dtype), gate=torch.zeros(B, H, L, f, dtype=dtype),
                wq=torch.zeros(H, d, f // 2, dtype=dtype), wk=torch.zeros(H, d, f // 2, dtype=dtype),
                meta=torch.zeros(H, M))


def hybrid(x, **kw):
    return G.hybrid_layer_fwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], window=4, **kw)


def test_host_tensors_are_rejected():
    with pytest.raises(ValueError, match="GPU tensor"):
        hybrid(layer())


@pytest.mark.parametrize("name,bad", [
    ("k", lambda x: x["k"][:, :, :-1]),
    ("v", lambda x: x["v"][:, :1]),
    ("gate", lambda x: x["gate"][..., :-2]),
    ("wk", lambda x: x["wk"][:1]),
    ("wq", lambda x: torch.zeros(2, 16, 3, dtype=torch.bfloat16)),
    ("meta", lambda x: x["meta"][:1]),
])
def test_shape_mismatch(name, bad):
    x = layer()
    x[name] = bad(x)
    with pytest.raises(ValueError, match="shape"):
        hybrid(x)


@pytest.mark.parametrize("name", ["k", "v", "gate", "wq", "wk"])
def test_dtype_mismatch(name):
    x = layer()
    x[name] = x[name].float()
    with pytest.raises(TypeError, match="dtype"):
        hybrid(x)


def test_meta_must_be_fp32():
    x = layer()
    x["meta"] = x["meta"].double()
    with pytest.raises(TypeError, match="dtype"):
        hybrid(x)


def test_unsupported_input_dtype():
    x = layer(dtype=torch.float16)
    with pytest.raises(TypeError):
        hybrid(x)


@pytest.mark.parametrize("name", ["q", "k", "v", "gate", "wq"])
def test_non_contiguous_view(name):
    x = layer()
    t = x[name]
    wide = torch.zeros(t.shape[:-1] + (2 * t.shape[-1],), dtype=t.dtype)
    x[name] = wide[..., ::2]  # the right shape and dtype, every other element
    assert x[name].shape == t.shape and not x[name].is_contiguous()
    with pytest.raises(ValueError, match="contiguous"):
        hybrid(x)


def test_state_and_ring_checks():
    x = layer()
    with pytest.raises(ValueError, match="shape"):
        hybrid(x, state_out=torch.zeros(1, 2, 8, 9))
    with pytest.raises(TypeError, match="dtype"):
        hybrid(x, state_in=torch.zeros(1, 2, 8, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        hybrid(x, kcache_out=torch.zeros(1, 2, 5, 16, dtype=torch.bfloat16),
               vcache_out=torch.zeros(1, 2, 4, 8, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="shape"):
        hybrid(x, o=torch.zeros(1, 2, 8, 16, dtype=torch.bfloat16))


def test_scalar_gate_layouts():
    x = layer()
    x["gate"] = torch.zeros(1, 2, 8, dtype=torch.bfloat16)   # one log-gate per token
    with pytest.raises(ValueError, match="GPU tensor"):     # shape accepted
        hybrid(x, gate_kind=G.GLAH_GATE_LOG_TOKEN)
    with pytest.raises(ValueError, match="shape"):          # not a per-feature gate
        hybrid(x)
    x["gate"] = torch.zeros(2, dtype=torch.bfloat16)         # one log-gate per head
    with pytest.raises(ValueError, match="GPU tensor"):
        hybrid(x, gate_kind=G.GLAH_GATE_LOG_HEAD)


def test_decode_checks():
    B, H, d, dv, f, w = 2, 3, 16, 8, 8, 4
    bf = torch.bfloat16
    q, k, v = torch.zeros(B, H, d, dtype=bf), torch.zeros(B, H, d, dtype=bf), torch.zeros(B, H, dv, dtype=bf)
    g = torch.zeros(B, H, f, dtype=bf)
    wq = wk = torch.zeros(H, d, f // 2, dtype=bf)
    meta = torch.zeros(H, 2)
    st = torch.zeros(B, H, f, dv)
    kc, vc = torch.zeros(B, H, w, d, dtype=bf), torch.zeros(B, H, w, dv, dtype=bf)
    pos = torch.zeros(B, dtype=torch.int32)
    with pytest.raises(ValueError, match="GPU tensor"):
        G.gla_decode_step(q, k, v, g, wq, wk, meta, st, kc, vc, pos, window=w)
    with pytest.raises(TypeError, match="dtype"):
        G.gla_decode_step(q, k, v, g, wq, wk, meta, st, kc, vc, pos.long(), window=w)
    with pytest.raises(ValueError, match="shape"):
        G.gla_decode_step(q, k, v, g, wq, wk, meta, st[:, :2], kc, vc, pos, window=w)
    with pytest.raises(ValueError, match="shape"):
        G.gla_decode_step(q, k, v, g, wq, wk, meta, st, kc, vc, pos, window=w + 1)


def test_delta_checks():
    B, H, L, d, dv = 1, 2, 5, 32, 8
    bf = torch.bfloat16
    q, k, v = torch.zeros(B, H, L, d, dtype=bf), torch.zeros(B, H, L, d, dtype=bf), torch.zeros(B, H, L, dv, dtype=bf)
    la, be = torch.zeros(B, H, L, dtype=bf), torch.zeros(B, H, L, dtype=bf)
    with pytest.raises(ValueError, match="GPU tensor"):
        G.gdn_prefill(q, k, v, la, be)
    with pytest.raises(TypeError, match="dtype"):
        G.gdn_prefill(q, k, v, la.float(), be)
    with pytest.raises(ValueError, match="shape"):
        G.gdn_prefill(q, k, v, la, be, state_in=torch.zeros(B, H, d, dv))


def test_backward_checks():
    x = layer()
    d_o = torch.zeros(1, 2, 8, 8, dtype=torch.float32)
    with pytest.raises(TypeError, match="dtype"):
        G.hybrid_layer_bwd(x["q"], x["k"], x["v"], x["gate"], x["wq"], x["wk"], x["meta"], d_o, window=4)

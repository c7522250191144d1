"""C-ABI checks that need no GPU: the library loads, exports every function that
include/glahybrid.h declares, and rejects bad arguments before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

from gated_linear_attention_hybrid_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "glahybrid.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIBRARY):
        from gated_linear_attention_hybrid_amd import build_lib
        build_lib.build()
    return binding.load()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while", "return")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gla_prefill", "swa_meta_attn", "hybrid_layer_fwd", "gla_decode_step",
              "glah_workspace_bytes", "glah_status_str", "glah_version"):
        assert n in names


def test_library_exports_every_declared_function(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIBRARY], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in declared_functions():
        assert n in exported, n
        assert getattr(lib, n) is not None
    assert set(binding.EXPORTS) <= set(declared_functions())


def test_status_strings(lib):
    for code in range(5):
        assert lib.glah_status_str(code)
    assert lib.glah_status_str(99) == b"unknown status"
    assert lib.glah_version() >= 1


FAKE = 0x10000  # an aligned, non-null address: never dereferenced by these calls


def _desc(**kw):
    base = dict(B=1, H=2, L=16, d=64, dv=64, f=64, window=8, n_meta=4, chunk=0, scale=0.0,
                dtype=binding.GLAH_F32, gate_is_log=False)
    base.update(kw)
    return binding.make_desc(base["B"], base["H"], base["L"], base["d"], base["dv"], base["f"],
                             window=base["window"], n_meta=base["n_meta"], chunk=base["chunk"],
                             scale=base["scale"], dtype=base["dtype"],
                             gate_is_log=base["gate_is_log"])


def _hybrid(lib, desc, **ptrs):
    names = ["q", "k", "v", "gate", "wq", "wk", "meta", "state_in", "state_out", "kc", "vc", "o", "ws"]
    p = {n: FAKE for n in ("q", "k", "v", "gate", "wq", "wk", "meta", "o")}
    p.update(ptrs)
    args = [ctypes.c_void_p(p.get(n)) if p.get(n) else None for n in names]
    return lib.hybrid_layer_fwd(ctypes.byref(desc) if desc is not None else None, *args[:12],
                                args[12], ptrs.get("ws_bytes", 0), None)


@pytest.mark.parametrize("bad", [
    dict(f=63), dict(f=0), dict(B=-1), dict(H=-2), dict(L=-1), dict(d=0), dict(dv=0),
    dict(window=0), dict(n_meta=-1), dict(chunk=48), dict(dtype=7),
])
def test_bad_descriptor_is_einval(lib, bad):
    d = _desc(**bad)
    if "gate_is_log" not in bad and bad.get("dtype") is None:
        pass
    assert _hybrid(lib, d) == binding.GLAH_EINVAL


def test_bad_gate_kind_is_einval(lib):
    for kind in (4, 5, -1):
        d = _desc()
        d.gate_kind = kind
        assert _hybrid(lib, d) == binding.GLAH_EINVAL


def test_scalar_gate_kinds_are_valid_descriptors(lib):
    for kind in (binding.GLAH_GATE_LOG_TOKEN, binding.GLAH_GATE_LOG_HEAD):
        d = _desc()
        d.gate_kind = kind
        assert lib.glah_workspace_bytes(ctypes.byref(d)) != ctypes.c_size_t(-1).value


def test_null_descriptor_is_einval(lib):
    assert _hybrid(lib, None) == binding.GLAH_EINVAL
    assert lib.glah_workspace_bytes(None) == ctypes.c_size_t(-1).value


@pytest.mark.parametrize("missing", ["q", "k", "v", "gate", "wq", "wk", "meta", "o"])
def test_missing_required_pointer_is_einval(lib, missing):
    assert _hybrid(lib, _desc(), **{missing: 0}) == binding.GLAH_EINVAL


@pytest.mark.parametrize("which", ["q", "o", "state_in", "kc"])
def test_misaligned_pointer_is_einval(lib, which):
    extra = {"vc": FAKE} if which == "kc" else {}
    assert _hybrid(lib, _desc(), **{which: FAKE + 4}, **extra) == binding.GLAH_EINVAL


def test_one_sided_window_cache_is_einval(lib):
    assert _hybrid(lib, _desc(), kc=FAKE) == binding.GLAH_EINVAL


def test_meta_may_be_null_only_without_sinks(lib):
    assert _hybrid(lib, _desc(n_meta=4), meta=0) == binding.GLAH_EINVAL


def _decode(lib, desc, **ptrs):
    names = ["q", "k", "v", "gate", "wq", "wk", "meta", "state", "kc", "vc", "pos", "o"]
    p = {n: FAKE for n in names}
    p.update(ptrs)
    args = [ctypes.c_void_p(p[n]) if p[n] else None for n in names]
    return lib.gla_decode_step(ctypes.byref(desc), *args, None)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, _desc(dv=66)) == binding.GLAH_ENOTSUP
    assert _decode(lib, _desc(), pos=0) == binding.GLAH_EINVAL
    assert _decode(lib, _desc(), state=0) == binding.GLAH_EINVAL
    assert _decode(lib, _desc(), kc=0) == binding.GLAH_EINVAL
    assert _decode(lib, _desc(window=-1)) == binding.GLAH_EINVAL
    assert _decode(lib, _desc(d=1024)) == binding.GLAH_ENOTSUP


def test_prefill_rejects_unsupported_sizes(lib):
    # a head dim beyond every kernel's limit is a valid but unsupported request
    assert _hybrid(lib, _desc(d=1024)) == binding.GLAH_ENOTSUP
    assert _hybrid(lib, _desc(window=100000)) == binding.GLAH_ENOTSUP


def test_swa_and_gla_prefill_argument_checks(lib):
    d = _desc()
    f = ctypes.c_void_p(FAKE)
    assert lib.swa_meta_attn(ctypes.byref(d), f, f, None, f, f, None) == binding.GLAH_EINVAL
    assert lib.gla_prefill(ctypes.byref(_desc(f=7)), f, f, f, f, f, f, None, None, f, None, 0,
                           None) == binding.GLAH_EINVAL
    assert lib.gla_prefill(ctypes.byref(d), f, f, f, None, f, f, None, None, f, None, 0,
                           None) == binding.GLAH_EINVAL


def _bwd(lib, desc, ws_bytes=0, **ptrs):
    names = ["q", "k", "v", "gate", "wq", "wk", "meta", "state_in", "do", "dstate_out", "dq", "dk", "dv",
             "dgate", "dwq", "dwk", "dmeta", "dstate_in", "ws"]
    p = {n: FAKE for n in ("q", "k", "v", "gate", "wq", "wk", "meta", "do", "dq", "dk", "dv", "dgate",
                           "dwq", "dwk", "dmeta", "ws")}
    p.update(ptrs)
    args = [ctypes.c_void_p(p.get(n)) if p.get(n) else None for n in names]
    return lib.hybrid_layer_bwd(ctypes.byref(desc), *args, ws_bytes, None)


def test_backward_argument_checks(lib):
    d = _desc()
    need = lib.glah_bwd_workspace_bytes(ctypes.byref(d))
    assert 0 < need < ctypes.c_size_t(-1).value
    for missing in ("q", "do", "dq", "dgate", "dwq", "dmeta"):
        assert _bwd(lib, d, need, **{missing: 0}) == binding.GLAH_EINVAL, missing
    assert _bwd(lib, d, need, dq=FAKE + 8) == binding.GLAH_EINVAL
    # the least workspace any call takes: one batch row and one head at a time
    least = lib.glah_bwd_workspace_bytes(ctypes.byref(_desc(H=1)))
    assert 0 < least < need
    assert _bwd(lib, d, least - 1) == binding.GLAH_EWORKSPACE
    assert _bwd(lib, d, need, ws=0) == binding.GLAH_EWORKSPACE
    # sizes beyond the backward kernels: valid but unsupported
    for bad in (dict(d=256), dict(dv=66), dict(f=96), dict(f=256), dict(window=2048)):
        assert _bwd(lib, _desc(**bad), 1 << 40) == binding.GLAH_ENOTSUP, bad
    assert lib.glah_bwd_workspace_bytes(ctypes.byref(_desc(f=7))) == ctypes.c_size_t(-1).value


def test_backward_workspace_sizing(lib):
    """The sizing query reports the whole call's workspace up to 1.5e9 bytes, else
    the largest sub-problem's within that (blocks of heads, or of batch rows)."""
    gib = 1500000000
    def ws(B, H, L):
        d = binding.make_desc(B, H, L, 128, 128, 128, window=64, n_meta=4, dtype=binding.GLAH_BF16)
        return lib.glah_bwd_workspace_bytes(ctypes.byref(d))
    def whole(B, H, L):
        d = binding.make_desc(B, H, L, 128, 128, 128, window=64, n_meta=4, dtype=binding.GLAH_BF16)
        return lib.glah_bwd_workspace_bytes_whole(ctypes.byref(d))
    assert ws(1, 32, 2048) < ws(2, 32, 2048) <= gib               # small calls run whole
    assert whole(1, 32, 2048) == ws(1, 32, 2048) and whole(1, 32, 32768) > gib
    big = ws(1, 32, 32768)
    assert big <= gib and big == ws(1, 16, 32768) > ws(1, 8, 32768)  # 32K: blocks of 16 heads
    assert ws(8, 32, 8192) == ws(2, 32, 8192) <= gib < whole(4, 32, 8192)  # batch 8: two rows at a time
    assert ws(1, 1, 1 << 22) > gib                                 # nothing fits: the least


def _gdn_desc(**kw):
    base = dict(B=1, H=2, L=16, d=64, dv=64)
    base.update(kw)
    return binding.make_desc(base["B"], base["H"], base["L"], base["d"], base["dv"], base["d"],
                             dtype=kw.get("dtype", binding.GLAH_F32))


def _gdn_prefill(lib, desc, ptrs=None):
    p = [FAKE] * 9 if ptrs is None else ptrs  # q k v a beta state_in state_out o
    return lib.gdn_prefill(ctypes.byref(desc), *[ctypes.c_void_p(x) for x in p[:8]], None, 0, None)


@pytest.mark.parametrize("bad", [dict(d=0), dict(dv=0), dict(B=-1), dict(H=-1), dict(L=-1), dict(dtype=9)])
def test_gdn_bad_descriptor_is_einval(lib, bad):
    assert _gdn_prefill(lib, _gdn_desc(**bad)) == binding.GLAH_EINVAL


@pytest.mark.parametrize("d", [16, 48, 256])
def test_gdn_unsupported_key_dim_is_enotsup(lib, d):
    assert _gdn_prefill(lib, _gdn_desc(d=d)) == binding.GLAH_ENOTSUP


@pytest.mark.parametrize("missing", range(5))
def test_gdn_missing_input_is_einval(lib, missing):
    p = [FAKE] * 8
    p[missing] = 0
    assert _gdn_prefill(lib, _gdn_desc(), p) == binding.GLAH_EINVAL


def test_gdn_misaligned_and_null_checks(lib):
    p = [FAKE] * 8
    p[4] = FAKE + 2
    assert _gdn_prefill(lib, _gdn_desc(), p) == binding.GLAH_EINVAL
    p = [FAKE] * 8
    p[7] = 0  # o
    assert _gdn_prefill(lib, _gdn_desc(), p) == binding.GLAH_EINVAL
    assert lib.gdn_prefill(None, *[ctypes.c_void_p(FAKE)] * 8, None, 0, None) == binding.GLAH_EINVAL
    d = _gdn_desc()
    args = [ctypes.c_void_p(FAKE)] * 7
    args[5] = ctypes.c_void_p(0)  # state
    assert lib.gdn_decode_step(ctypes.byref(d), *args, None) == binding.GLAH_EINVAL
    assert lib.gdn_decode_step(ctypes.byref(_gdn_desc(d=96)), *[ctypes.c_void_p(FAKE)] * 7,
                               None) == binding.GLAH_ENOTSUP


def _cont(lib, desc, start, ptrs=None):
    p = [FAKE] * 15 if ptrs is None else ptrs  # q k v gate wq wk meta s_in kc_in vc_in s_out kc_out vc_out o ws
    return lib.hybrid_layer_fwd_cont(ctypes.byref(desc), start, *[ctypes.c_void_p(x) for x in p], 1 << 40, None)


def test_continuation_argument_checks(lib):
    assert _cont(lib, _desc(), -1) == binding.GLAH_EINVAL
    p = [FAKE] * 15
    p[8] = 0  # kcache_in missing with start > 0
    assert _cont(lib, _desc(), 3, p) == binding.GLAH_EINVAL
    p = [FAKE] * 15
    p[12] = 0  # one-sided output ring
    assert _cont(lib, _desc(), 3, p) == binding.GLAH_EINVAL
    assert _cont(lib, _desc(window=65), 3) == binding.GLAH_ENOTSUP
    assert lib.hybrid_layer_fwd_cont(None, 0, *[ctypes.c_void_p(FAKE)] * 15, 0, None) == binding.GLAH_EINVAL


def test_output_gate_argument_checks(lib):
    d = _desc()
    assert lib.glah_output_gate(ctypes.byref(d), None, ctypes.c_void_p(FAKE), None) == binding.GLAH_EINVAL
    assert lib.glah_output_gate(ctypes.byref(d), ctypes.c_void_p(FAKE + 4), ctypes.c_void_p(FAKE),
                                None) == binding.GLAH_EINVAL
    assert lib.glah_output_gate(None, ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), None) == binding.GLAH_EINVAL
    bad = _desc(dtype=5)
    assert lib.glah_output_gate(ctypes.byref(bad), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE),
                                None) == binding.GLAH_EINVAL


def test_gdn_workspace_bytes(lib):
    # chunkwise path (bf16, d_qk = 128, d_v a multiple of 16, L >= 64): one
    # 13568-byte record per 64-token chunk of every (b, h); none otherwise
    def ws(**kw):
        return lib.gdn_workspace_bytes(ctypes.byref(_gdn_desc(**kw)))
    assert ws(B=2, H=3, L=130, d=128, dv=48, dtype=binding.GLAH_BF16) == 2 * 3 * 3 * 13568
    assert ws(L=64, d=128, dv=128, dtype=binding.GLAH_BF16) == 2 * 13568
    assert ws(L=63, d=128, dv=128, dtype=binding.GLAH_BF16) == 0
    assert ws(L=640, d=128, dv=40, dtype=binding.GLAH_BF16) == 0
    assert ws(L=640, d=64, dv=64, dtype=binding.GLAH_BF16) == 0
    assert ws(L=640, d=128, dv=128) == 0  # fp32: token-recurrent
    assert ws(d=256) == 0  # unsupported
    assert ws(B=-1) == ctypes.c_size_t(-1).value
    assert lib.gdn_workspace_bytes(None) == ctypes.c_size_t(-1).value


def test_gdn_missing_workspace_is_eworkspace(lib):
    d = _gdn_desc(L=128, d=128, dv=128, dtype=binding.GLAH_BF16)
    need = lib.gdn_workspace_bytes(ctypes.byref(d))
    ptrs = [ctypes.c_void_p(FAKE)] * 8
    assert lib.gdn_prefill(ctypes.byref(d), *ptrs, None, 0, None) == binding.GLAH_EWORKSPACE
    assert lib.gdn_prefill(ctypes.byref(d), *ptrs, ctypes.c_void_p(FAKE), need - 1, None) == binding.GLAH_EWORKSPACE
    assert lib.gdn_prefill(ctypes.byref(d), *ptrs, ctypes.c_void_p(FAKE + 8), need, None) == binding.GLAH_EINVAL

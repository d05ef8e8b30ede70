"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every symbol include/ttt.h declares, and rejects bad arguments before any HIP
call is made."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ttt.h")

ttt = pytest.importorskip("linear_complexity_attention_amd.ttt",
                          reason="libttt.so not built (run __graft_entry__.build())")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(ttt_\w+)\s*\(", src, flags=re.M)))


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(ttt.LIB_PATH)
    names = _declared_functions()
    assert len(names) >= 8, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/ttt.h but not exported"
    assert set(names) == set(ttt.EXPORTED)


def test_version_and_status_strings():
    assert ttt.ttt_version() == 1
    assert ttt.ttt_status_string(0) == "ok"
    assert "workspace" in ttt.ttt_status_string(5)


def _cfg(**kw):
    base = dict(B=2, H=3, N=100, d=64, hidden=256, dtype=ttt.TTT_BF16, key_norm=1, eps=1e-5, renorm=0, flags=0)
    base.update(kw)
    return ttt.ttt_config(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(B=0), ttt.TTT_ERR_INVALID),
    (dict(N=0), ttt.TTT_ERR_INVALID),
    (dict(d=129), ttt.TTT_ERR_UNSUPPORTED),
    (dict(d=0), ttt.TTT_ERR_UNSUPPORTED),
    (dict(dtype=7), ttt.TTT_ERR_INVALID),
    (dict(eps=-1.0), ttt.TTT_ERR_INVALID),
    (dict(eps=float("nan")), ttt.TTT_ERR_INVALID),
    (dict(flags=0x100), ttt.TTT_ERR_INVALID),
])
def test_create_rejects_bad_config(kw, code):
    with pytest.raises(ttt.TTTError) as ei:
        ttt.ttt_create(_cfg(**kw))
    assert ei.value.status == code
    assert ttt.ttt_last_error(None) != ""


def test_workspace_and_request_validation():
    h = ttt.ttt_create(_cfg())
    try:
        n = ttt.ttt_workspace_bytes(h, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0)
        assert n > 0 and n % 256 == 0
        with pytest.raises(ttt.TTTError) as ei:
            ttt.ttt_workspace_bytes(h, 9, ttt.TTT_INNER_MLP_GELU, 0)
        assert ei.value.status == ttt.TTT_ERR_INVALID
        with pytest.raises(ttt.TTTError) as ei:     # causal chunks + key norm would leak the future
            ttt.ttt_workspace_bytes(h, ttt.TTT_LOSS_DOT, ttt.TTT_INNER_SWIGLU, 16)
        assert ei.value.status == ttt.TTT_ERR_UNSUPPORTED
        with pytest.raises(ttt.TTTError):
            ttt.ttt_workspace_bytes(h, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, -1)
        assert ttt.ttt_path_name(h, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0) is not None
        assert ttt.ttt_path_name(h, 9, ttt.TTT_INNER_MLP_GELU, 0) is None
    finally:
        ttt.ttt_destroy(h)


def test_forward_rejects_before_enqueue():
    """Argument errors are reported before any HIP call, so these run without a GPU."""
    h = ttt.ttt_create(_cfg())
    try:
        W = ttt.ttt_weights()
        e = ttt.ttt_eta(1.0, None)
        fake = 1 << 20   # never dereferenced: validation fails first
        rc = ttt.ttt_forward(h, None, fake, fake, W, e, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0, fake,
                             None, fake, 1 << 30, None)
        assert rc == ttt.TTT_ERR_INVALID and "non-NULL" in ttt.ttt_last_error(h)
        rc = ttt.ttt_forward(h, fake, fake, fake, W, e, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0, fake,
                             None, fake, 1 << 30, None)
        assert rc == ttt.TTT_ERR_INVALID and "W0" in ttt.ttt_last_error(h)
        W.w[0] = fake
        W.w[1] = fake
        rc = ttt.ttt_forward(h, fake, fake, fake, W, e, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0, fake,
                             None, None, 0, None)
        assert rc == ttt.TTT_ERR_WORKSPACE
        rc = ttt.ttt_forward(h, fake, fake, fake, W, e, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0, fake,
                             None, fake, 16, None)
        assert rc == ttt.TTT_ERR_WORKSPACE and "too small" in ttt.ttt_last_error(h)
        rc = ttt.ttt_forward(h, fake, fake, fake, W, ttt.ttt_eta(float("inf"), None), ttt.TTT_LOSS_MSE,
                             ttt.TTT_INNER_MLP_GELU, 0, fake, None, fake, 1 << 30, None)
        assert rc == ttt.TTT_ERR_INVALID
        W.batch_stride = 5
        rc = ttt.ttt_forward(h, fake, fake, fake, W, e, ttt.TTT_LOSS_MSE, ttt.TTT_INNER_MLP_GELU, 0, fake,
                             None, fake, 1 << 30, None)
        assert rc == ttt.TTT_ERR_INVALID and "batch_stride" in ttt.ttt_last_error(h)
    finally:
        ttt.ttt_destroy(h)

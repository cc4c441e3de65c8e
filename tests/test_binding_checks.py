"""The Python binding's own argument checks, without a GPU.

The C ABI receives raw pointers and cannot see sizes, so a tensor of the wrong shape or element
type would reach a kernel as a pointer and be read or written past its end.  The binding must
reject it before any library call.  Here the library is replaced by a recorder that notes every
call, the device-placement check is bypassed (host tensors stand in for device ones), and every
wrapper is driven once with valid arguments (exactly one library call) and once per mismatch
(ValueError, no library call).
"""
import pytest
import torch

import exact_io_aware_66_amd as fa

B, H, N, D = 2, 3, 40, 64


class _Recorder:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def call(*args):
            self.calls.append(name)
            return 0
        return call


@pytest.fixture
def rec(monkeypatch):
    r = _Recorder()
    monkeypatch.setattr(fa, "_lib", r)
    monkeypatch.setattr(fa, "_same", lambda *a, **k: None)
    monkeypatch.setattr(fa, "_stream", lambda s: None)
    monkeypatch.setattr(fa, "_seqlens", lambda s, b, dev: s)
    monkeypatch.setattr(fa, "_block_mask", lambda m, *a: m)
    return r


def _t(shape=(B, H, N, D), dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def _lse(shape=(B, H, N), dtype=torch.float32):
    return torch.zeros(shape, dtype=dtype)


def _ws(n=1024, dtype=torch.uint8):
    return torch.zeros(n, dtype=dtype)


def _args(kind):
    """Valid arguments of each wrapper, as a dict of named tensors plus the call."""
    q = _t()
    base = dict(q=q, k=_t(), v=_t())
    if kind == "fa_forward":
        a = dict(base, o=_t(), lse=_lse())
        return a, lambda a: fa.fa_forward(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1)
    if kind == "fa_forward_block_sparse":
        a = dict(base, o=_t(), lse=_lse())
        return a, lambda a: fa.fa_forward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, False, None,
                                                       torch.zeros(1, dtype=torch.uint8))
    if kind == "fa_forward_dropout":
        a = dict(base, o=_t(), lse=_lse())
        return a, lambda a: fa.fa_forward_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, False, None, 0.1, 1, 0)
    if kind == "fa_forward_kv_outer":
        a = dict(base, o=_t(), lse=_lse(), workspace=_ws())
        return a, lambda a: fa.fa_forward_kv_outer(a["q"], a["k"], a["v"], a["o"], a["lse"], 0.1, 32768, a["workspace"])
    if kind in ("fa_backward", "fa_backward_block_sparse", "fa_backward_dropout"):
        a = dict(base, o=_t(), do=_t(), lse=_lse(), dq=_t(), dk=_t(), dv=_t(), workspace=_ws())
        if kind == "fa_backward":
            return a, lambda a: fa.fa_backward(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                               a["dv"], 0.1, True, None, a["workspace"])
        if kind == "fa_backward_block_sparse":
            return a, lambda a: fa.fa_backward_block_sparse(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"],
                                                            a["dk"], a["dv"], 0.1, True, None,
                                                            torch.zeros(1, dtype=torch.uint8), a["workspace"])
        return a, lambda a: fa.fa_backward_dropout(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                                                   a["dv"], 0.1, True, None, 0.1, 1, 0, a["workspace"])
    if kind == "fa_backward_prepare":
        a = dict(o=_t(), do=_t(), lse=_lse(), workspace=_ws())
        return a, lambda a: fa.fa_backward_prepare(a["o"], a["do"], a["lse"], a["workspace"])
    if kind == "fa_backward_dkdv":
        a = dict(base, do=_t(), lse=_lse(), dk=_t(), dv=_t(), workspace=_ws())
        return a, lambda a: fa.fa_backward_dkdv(a["q"], a["k"], a["v"], a["do"], a["lse"], a["dk"], a["dv"], 0.1, True,
                                                None, a["workspace"])
    if kind == "fa_backward_dq_prepare":
        a = dict(base, o=_t(), do=_t(), lse=_lse(), dq=_t(), workspace=_ws())
        return a, lambda a: fa.fa_backward_dq_prepare(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], 0.1,
                                                      True, None, a["workspace"])
    if kind == "fa_backward_dq":
        a = dict(base, do=_t(), lse=_lse(), dq=_t(), workspace=_ws())
        return a, lambda a: fa.fa_backward_dq(a["q"], a["k"], a["v"], a["do"], a["lse"], a["dq"], 0.1, True, None,
                                              a["workspace"])
    if kind == "fa_forward_fp8":
        f8 = torch.float8_e4m3fn
        a = dict(q=_t(dtype=f8), k=_t(dtype=f8), v=_t(dtype=f8), o=_t(), lse=_lse())
        return a, lambda a: fa.fa_forward_fp8(a["q"], a["k"], a["v"], 1.0, 1.0, 1.0, a["o"], a["lse"], 0.1)
    raise KeyError(kind)


WRAPPERS = ["fa_forward", "fa_forward_block_sparse", "fa_forward_dropout", "fa_forward_kv_outer", "fa_backward",
            "fa_backward_block_sparse", "fa_backward_dropout", "fa_backward_prepare", "fa_backward_dkdv",
            "fa_backward_dq_prepare", "fa_backward_dq", "fa_forward_fp8"]


def _mismatches(a):
    """(description, replacement dict) for every tensor argument: wrong N, wrong d, wrong dtype."""
    out = []
    for name, t in a.items():
        if name == "q":
            continue  # the reference every other tensor is compared with
        if name == "lse":
            out += [("lse short", {name: _lse((B, H, N - 1))}), ("lse bf16", {name: _lse(dtype=torch.bfloat16)}),
                    ("lse 4-D", {name: _lse((B, H, N, 1))})]
        elif name == "workspace":
            out += [("workspace float32", {name: _ws(256, torch.float32)}),
                    ("workspace 2-D", {name: torch.zeros(4, 256, dtype=torch.uint8)})]
        else:
            other = torch.float32 if t.dtype != torch.float32 else torch.bfloat16
            out += [(f"{name} short N", {name: _t((B, H, N - 8, D), t.dtype)}),
                    (f"{name} small d", {name: _t((B, H, N, D // 2), t.dtype)}),
                    (f"{name} dtype", {name: _t(dtype=other)})]
    return out


@pytest.mark.parametrize("kind", WRAPPERS)
def test_valid_arguments_reach_the_library_once(rec, kind):
    a, call = _args(kind)
    call(a)
    assert rec.calls == [kind]


@pytest.mark.parametrize("kind", WRAPPERS)
def test_mismatched_tensors_raise_before_any_call(rec, kind):
    a, call = _args(kind)
    cases = _mismatches(a)
    assert cases
    for what, repl in cases:
        bad = dict(a, **repl)
        with pytest.raises((ValueError, fa.FAError)):  # FAError: an unsupported FP8 input type
            call(bad)
        assert rec.calls == [], (kind, what)


def test_none_output_is_rejected(rec):
    a, call = _args("fa_backward")
    with pytest.raises(ValueError):
        call(dict(a, dk=None))
    assert rec.calls == []

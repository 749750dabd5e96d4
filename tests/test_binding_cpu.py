"""The Python binding's argument checks (CPU only): tensors the library
cannot check through raw pointers are refused with ValueError before any
library call."""
import pytest
import torch

from linear_attention_rnn_amd import wkv7 as W

H = 2


class NoLibrary:
    """Stands in for the loaded library: any use of it fails the test."""
    def __getattr__(self, name):
        raise AssertionError(f"library call {name} made before the checks")


@pytest.fixture
def no_lib(monkeypatch):
    monkeypatch.setattr(W, "lib", NoLibrary())


def _io(T=3, dtype=torch.bfloat16):
    x = [torch.zeros((T, H, 64), dtype=dtype) for _ in range(6)]
    return x, torch.zeros((T, H, 64), dtype=torch.float32)


CALLS = {
    "forward": lambda x, o, **kw: W.wkv7_forward(1, [0], [0, 3], *x, o, **kw),
    "forward_noalloc": lambda x, o, **kw: W.wkv7_forward_noalloc(
        1, [0], [0, 3], *x, o, **kw),
    "forward_plan": lambda x, o, **kw: W.wkv7_forward_plan(1, 1, *x, o, **kw),
}


@pytest.mark.parametrize("call", sorted(CALLS))
def test_rejections_before_any_library_call(call, no_lib):
    f = CALLS[call]
    x, o = _io()
    bad = list(x)
    bad[3] = x[3].to(torch.float32)                       # mixed dtypes
    with pytest.raises(ValueError, match="share one dtype"):
        f(bad, o)
    bad = list(x)
    bad[0] = torch.zeros((H, 3, 64), dtype=torch.bfloat16).transpose(0, 1)
    with pytest.raises(ValueError, match="contiguous"):
        f(bad, o)
    with pytest.raises(ValueError, match="contiguous"):
        f(x, torch.zeros((3, 64, H)).transpose(1, 2))
    with pytest.raises(ValueError, match="float32"):
        f(x, o.to(torch.float16))
    with pytest.raises(ValueError, match="does not match"):
        f(x, o, dtype=W.WKV7_F32)                         # bf16 read as fp32
    with pytest.raises(ValueError, match="torch.Tensor"):
        f([[0.0]] + x[1:], o)
    with pytest.raises(ValueError, match="not on a GPU"):
        f(x, o)                                           # CPU tensors


def test_short_tensors_are_refused():
    x, o = _io(T=3)
    short = list(x)
    short[2] = torch.zeros((2, H, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="elements"):
        W._check_io(3, H, None, short, o)
    with pytest.raises(ValueError, match="elements"):
        W._check_io(3, H, None, x, torch.zeros((3, H, 63)))
    # a larger buffer passes the size check (the call reads the first rows
    # only; these CPU tensors then fail the device check), and unsupported
    # dtypes or NULL tensors are left to the library
    with pytest.raises(ValueError, match="not on a GPU"):
        W._check_io(2, H, None, x, o)
    W._check_io(None, None, 7, [None] * 6, None)
    half = [t.to(torch.float16) for t in x]
    with pytest.raises(ValueError, match="not on a GPU"):
        W._check_io(3, H, None, half, o)     # fp16 passes to the library

"""INT8 projections on the GPU against the oracle: codes and scales bit for
bit, products to float32 rounding of the exact integer sums (GPU)."""
import numpy as np
import pytest
import torch

from linear_attention_rnn_amd import wkv7 as W
from oracle import quantize_rows, q8_matmul
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu
TOL = 1e-6      # fp32 conversion of the int32 sums and of the scale product


def _rel(got, ref):
    ref = np.asarray(ref, np.float64)
    return float(np.max(np.abs(np.asarray(got, np.float64) - ref))
                 / np.sqrt(np.mean(ref ** 2)))


def _quantize_dev(x):
    q = torch.empty(x.shape, dtype=torch.int8, device=DEV)
    s = torch.empty(x.shape[0], dtype=torch.float32, device=DEV)
    W.wkv7_q8_quantize(x, q, s)
    torch.cuda.synchronize()
    return q, s


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_bitexact(dtype):
    rng = np.random.default_rng(61)
    x = (rng.standard_normal((37, 193)) *
         10.0 ** rng.integers(-4, 4, (37, 1))).astype(np.float32)
    x[3] = 0.0                                   # zero row
    x[5] = 0.0
    x[5, 7] = -2.0                               # single entry
    x[6, :5] = [127.0, 2.5, -2.5, 0.5, -0.5]     # exact halves at scale 1
    x[6, 5:] = 0.0
    xt = torch.from_numpy(x).to(dtype)
    x_in = xt.float().numpy()                    # the values the GPU sees
    q, s = _quantize_dev(xt.to(DEV))
    q_ref, s_ref = quantize_rows(x_in)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert list(q_ref[6, :5]) == [127, 3, -3, 1, -1]


# Rows of whole 16-byte groups: up to 1023 rows take the row-split kernel
# (four wavefronts per row), more rows the one-wavefront kernel; rows longer
# than 4096 values the two-pass form.
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("rows,cols", [(37, 2048), (300, 1088), (5, 4096),
                                       (2, 8), (1100, 512), (3, 4104)])
def test_quantize_bitexact_vector_rows(dtype, rows, cols):
    rng = np.random.default_rng(rows * 7 + cols)
    x = (rng.standard_normal((rows, cols)) *
         10.0 ** rng.integers(-4, 4, (rows, 1))).astype(np.float32)
    x[1] = 0.0                                   # zero row
    x[0, :5] = [127.0, 2.5, -2.5, 0.5, -0.5]     # exact halves at scale 1
    x[0, 5:] = 0.0
    x[0, cols - 1] = -127.0                      # the maximum in the last chunk
    xt = torch.from_numpy(x).to(dtype)
    x_in = xt.float().numpy()
    q, s = _quantize_dev(xt.to(DEV))
    q_ref, s_ref = quantize_rows(x_in)
    say(f"quantize rows={rows} cols={cols} {dtype}")
    assert np.array_equal(s.cpu().numpy().view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert list(q_ref[0, :5]) == [127, 3, -3, 1, -1]


@pytest.mark.parametrize("O,I,B", [(48, 128, 1), (64, 256, 17), (208, 640, 130),
                                   (16, 64, 300), (64, 1088, 2), (32, 2112, 3),
                                   (16, 64, 4), (1040, 2048, 1),
                                   # rows a multiple of the workgroup's 96 or
                                   # not, I a multiple of the 128-wide k step
                                   # or not, partial token blocks
                                   (9600, 128, 200), (13440, 192, 200),
                                   (16000, 128, 200), (112, 4160, 129)])
def test_matmul_matches_oracle(O, I, B):
    rng = np.random.default_rng(O + I + B)
    w = rng.standard_normal((O, I)).astype(np.float32)
    x = rng.standard_normal((B, I)).astype(np.float32)
    wq, ws = _quantize_dev(torch.from_numpy(w).to(DEV))
    xq, xs = _quantize_dev(torch.from_numpy(x).to(DEV))
    y = torch.full((B, O), float("nan"), dtype=torch.float32, device=DEV)
    W.wkv7_q8_matmul(wq, ws, xq, xs, y)
    torch.cuda.synchronize()
    ref = q8_matmul(wq.cpu().numpy(), ws.cpu().numpy(), xq.cpu().numpy(),
                    xs.cpu().numpy())
    e = _rel(y.cpu().numpy(), ref)
    say(f"q8 matmul O={O} I={I} B={B}: rel err {e:.2e}")
    assert np.all(np.isfinite(y.cpu().numpy()))
    assert e < TOL


@pytest.mark.parametrize("B", [1, 2, 3, 4])
def test_few_tokens_equal_tiled_product_bitwise(B):
    """Up to four tokens take a matrix-vector kernel; the same tokens with a
    fifth added take the tiled MFMA kernel. Integer sums are exact and the
    rescale is the same, so their rows agree bit for bit."""
    O, I = 96, 2112
    rng = np.random.default_rng(40 + B)
    w = torch.from_numpy(rng.standard_normal((O, I)).astype(np.float32)).to(DEV)
    x = torch.from_numpy(rng.standard_normal((B + 1, I)).astype(np.float32)).to(DEV)
    wq, ws = _quantize_dev(w)
    xq, xs = _quantize_dev(x)
    y_few = torch.empty((B, O), dtype=torch.float32, device=DEV)
    y_all = torch.empty((B + 1, O), dtype=torch.float32, device=DEV)
    W.wkv7_q8_matmul(wq, ws, xq[:B].contiguous(), xs[:B].contiguous(), y_few)
    W.wkv7_q8_matmul(wq, ws, xq, xs, y_all)
    torch.cuda.synchronize()
    say(f"q8 few-token path, B={B}")
    assert torch.equal(y_few.view(torch.int32), y_all[:B].view(torch.int32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("O,I,B", [(48, 64, 1), (96, 1088, 2), (32, 2048, 3),
                                   (16, 2048, 4), (48, 2112, 2), (32, 256, 5)])
def test_linear_equals_quantize_then_matmul(dtype, O, I, B):
    """wkv7_q8_linear (one launch for up to four tokens with in <= 2048, two
    otherwise) gives the same codes, scales and outputs, bit for bit, as
    wkv7_q8_quantize followed by wkv7_q8_matmul."""
    rng = np.random.default_rng(O * 7 + I + B)
    w = torch.from_numpy(rng.standard_normal((O, I)).astype(np.float32)).to(DEV)
    x = torch.from_numpy(rng.standard_normal((B, I)).astype(np.float32))
    x = x.to(DEV).to(dtype)
    x[0, 5] = 0.0
    wq, ws = _quantize_dev(w)
    xq1, xs1 = _quantize_dev(x)
    y1 = torch.empty((B, O), dtype=torch.float32, device=DEV)
    W.wkv7_q8_matmul(wq, ws, xq1, xs1, y1)
    xq2 = torch.zeros((B, I), dtype=torch.int8, device=DEV)
    xs2 = torch.full((B,), float("nan"), dtype=torch.float32, device=DEV)
    y2 = torch.full((B, O), float("nan"), dtype=torch.float32, device=DEV)
    W.wkv7_q8_linear(wq, ws, x, xq2, xs2, y2)
    torch.cuda.synchronize()
    say(f"q8 linear O={O} I={I} B={B} {dtype}")
    assert torch.equal(xq1, xq2)
    assert torch.equal(xs1.view(torch.int32), xs2.view(torch.int32))
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_full_size_stacked_projection_sampled():
    """r,w,k,v,a,b weights of a C=2048 layer stacked into [12288, 2048],
    bf16, 256 decode tokens: 512 sampled outputs against exact integer dot
    products; the quantized result stays within 5% rms of the float64
    product of the unquantized operands."""
    C, B = 2048, 256
    gen = torch.Generator(device=DEV)
    gen.manual_seed(62)
    w = (torch.randn((6 * C, C), device=DEV, generator=gen) / C ** 0.5
         ).to(torch.bfloat16)
    x = torch.randn((B, C), device=DEV, generator=gen).to(torch.bfloat16)
    wq, ws = _quantize_dev(w)
    xq, xs = _quantize_dev(x)
    y = torch.empty((B, 6 * C), dtype=torch.float32, device=DEV)
    W.wkv7_q8_matmul(wq, ws, xq, xs, y)
    torch.cuda.synchronize()
    rng = np.random.default_rng(63)
    bs, os_ = rng.integers(0, B, 512), rng.integers(0, 6 * C, 512)
    wqn, xqn = wq.cpu().numpy(), xq.cpu().numpy()
    wsn, xsn = ws.cpu().numpy(), xs.cpu().numpy()
    yn = y.cpu().numpy()
    ref = np.array([int(np.dot(wqn[o].astype(np.int64), xqn[b].astype(np.int64)))
                    * float(wsn[o]) * float(xsn[b]) for b, o in zip(bs, os_)])
    got = yn[bs, os_]
    e = float(np.max(np.abs(got - ref)) / np.sqrt(np.mean(ref ** 2)))
    say(f"full-size q8 projection, sampled: rel err {e:.2e}")
    assert e < TOL
    wf = w.float().cpu().numpy().astype(np.float64)
    xf = x.float().cpu().numpy().astype(np.float64)
    exact = np.array([np.dot(wf[o], xf[b]) for b, o in zip(bs, os_)])
    qe = float(np.max(np.abs(got - exact)) / np.sqrt(np.mean(exact ** 2)))
    say(f"  quantization error against the float64 product: {qe:.2e}")
    assert qe < 0.05


def test_q8_errors():
    q = torch.zeros((16, 64), dtype=torch.int8, device=DEV)
    s = torch.ones(16, dtype=torch.float32, device=DEV)
    y = torch.zeros((4, 16), dtype=torch.float32, device=DEV)
    xq = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    xs = torch.ones(4, dtype=torch.float32, device=DEV)
    L = W.lib
    assert L.wkv7_q8_matmul(q.data_ptr(), s.data_ptr(), 16, 96, xq.data_ptr(),
                            xs.data_ptr(), 4, y.data_ptr(), None) == \
        W.WKV7_ERR_UNSUPPORTED                       # in % 64 != 0
    assert L.wkv7_q8_matmul(q.data_ptr(), s.data_ptr(), 8, 64, xq.data_ptr(),
                            xs.data_ptr(), 4, y.data_ptr(), None) == \
        W.WKV7_ERR_UNSUPPORTED                       # out % 16 != 0
    assert L.wkv7_q8_matmul(q.data_ptr() + 1, s.data_ptr(), 16, 64,
                            xq.data_ptr(), xs.data_ptr(), 4, y.data_ptr(),
                            None) == W.WKV7_ERR_INVALID_ARG   # misaligned
    assert L.wkv7_q8_matmul(None, s.data_ptr(), 16, 64, xq.data_ptr(),
                            xs.data_ptr(), 4, y.data_ptr(), None) == \
        W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_q8_matmul(None, None, 16, 64, None, None, 0, None, None) == \
        W.WKV7_OK                                    # B = 0: nothing to do
    assert L.wkv7_q8_quantize(q.data_ptr(), 5, 1, 1, q.data_ptr(), s.data_ptr(),
                              None) == W.WKV7_ERR_UNSUPPORTED
    assert L.wkv7_q8_quantize(None, 0, 0, 4, None, None, None) == W.WKV7_OK

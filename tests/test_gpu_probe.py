"""The hardware-ceiling probes move and count what they claim (GPU): the
copy is bit-exact in place and source to destination, for sizes that end
inside a workgroup's last unrolled pass, and the matrix-core loop runs."""
import pytest
import torch

from linear_attention_rnn_amd import hw_probe as P
from tests.gpu_util import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16 * 7, (1 << 20) + 16 * 513,
                                    64 << 20])
@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("blocks", [0, 3])
def test_copy_is_exact(nbytes, nt, blocks):
    say(f"probe copy {nbytes} B nt={nt} blocks={blocks}")
    n = nbytes // 4
    src = torch.randint(-2**31, 2**31 - 1, (n + 64,), dtype=torch.int32,
                        device=DEV)
    dst = torch.zeros_like(src)
    P.hwprobe_copy(src, dst, nbytes, nt, blocks)
    keep = src.clone()
    P.hwprobe_copy(src, src, nbytes, nt, blocks)        # in place
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src[:n])
    assert torch.equal(src, keep)
    assert int(dst[n:].abs().sum()) == 0                # nothing past the end


@pytest.mark.parametrize("kind", [P.MFMA_BF16, P.MFMA_I8, P.MFMA_I8_32])
def test_mfma_loop_runs(kind):
    say(f"probe mfma kind {kind}")
    blocks = 8
    out = torch.full((blocks * P.WAVES_PER_BLOCK,), float("nan"),
                     device=DEV)
    ops = P.hwprobe_mfma(kind, blocks, 100, out)
    torch.cuda.synchronize()
    assert ops == blocks * 4 * 100 * 8 * P.OPS_PER_MFMA[kind]
    assert bool(torch.isfinite(out).all())
    assert float(out.abs().sum()) > 0


def test_probe_rejects_short_buffers():
    a = torch.empty(16, dtype=torch.float32, device=DEV)
    with pytest.raises(P.ProbeError):
        P.hwprobe_copy(a, a, 128)
    with pytest.raises(P.ProbeError):
        P.hwprobe_mfma(P.MFMA_BF16, 8, 1, a)

"""The hardware-ceiling probe library: it loads, exports what its binding
names, and rejects bad arguments before touching a device (no GPU)."""
import ctypes
import subprocess

from linear_attention_rnn_amd import hw_probe as P


def test_probe_exports():
    out = subprocess.run(["nm", "-D", "--defined-only", P.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    names = sorted(line.split()[-1] for line in out.splitlines()
                   if line.split()[-1].startswith("hwprobe_"))
    assert names == sorted(P.EXPORTS)
    assert P.lib.hwprobe_mfma_per_iter() == 8


def test_probe_rejects_before_device():
    buf = ctypes.create_string_buffer(64)
    addr = ctypes.addressof(buf)
    addr16 = addr + (-addr) % 16
    inval = 1                                   # hipErrorInvalidValue
    assert P.lib.hwprobe_copy(None, addr16, 32, 0, 0, None) == inval
    assert P.lib.hwprobe_copy(addr16, addr16, 24, 0, 0, None) == inval
    assert P.lib.hwprobe_copy(addr16 + 4, addr16, 16, 0, 0, None) == inval
    assert P.lib.hwprobe_copy(addr16, addr16, 16, 0, -1, None) == inval
    assert P.lib.hwprobe_copy(addr16, addr16, 0, 0, 0, None) == 0
    assert P.lib.hwprobe_mfma(0, 4, 1, addr16, 15, None) == inval   # < 4 x 4
    assert P.lib.hwprobe_mfma(3, 1, 1, addr16, 16, None) == inval
    assert P.lib.hwprobe_mfma(-1, 1, 1, addr16, 16, None) == inval
    assert P.lib.hwprobe_mfma(0, 0, 1, addr16, 16, None) == inval
    assert P.lib.hwprobe_mfma(0, 1, -1, addr16, 16, None) == inval

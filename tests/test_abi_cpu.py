"""libwkv7 on the CPU: it loads, exports every declared symbol, and rejects
bad arguments before touching a device (no compute calls without a GPU)."""
import ctypes
import os
import re

import pytest

from linear_attention_rnn_amd import wkv7 as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_symbols():
    names = set()
    inc = os.path.join(ROOT, "include")
    for fn in sorted(os.listdir(inc)):
        if not fn.endswith(".h"):
            continue
        with open(os.path.join(inc, fn)) as f:
            src = f.read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(wkv7_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) >= 16
    lib = ctypes.CDLL(W.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/wkv7.h but not exported"
    assert sorted(W.EXPORTS) == names


def test_version():
    assert W.wkv7_version() == 100


@pytest.mark.parametrize("args,code", [
    ((4, 2, 32), W.WKV7_ERR_UNSUPPORTED),
    ((4, 2, 128), W.WKV7_ERR_UNSUPPORTED),
    ((0, 2, 64), W.WKV7_ERR_INVALID_ARG),
    ((4, 0, 64), W.WKV7_ERR_INVALID_ARG),
    ((-1, 2, 64), W.WKV7_ERR_INVALID_ARG),
])
def test_pool_create_rejects_before_device(args, code):
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_pool_create(*args)
    assert e.value.status == code
    assert e.value.message


def test_null_pool_everywhere():
    L = W.lib
    assert L.wkv7_pool_create(4, 2, 64, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_forward(None, None, None, 0, 0, *([None] * 8)) == \
        W.WKV7_ERR_INVALID_ARG
    assert b"NULL" in L.wkv7_last_error()
    assert L.wkv7_snapshot(None, 0, None, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_fork(None, None, None, 0, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_reset(None, None, 0, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_hibernate(None, None, 0, None, 0, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_resume(None, None, 0, None, 0, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_slot_alloc(None, 1, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_slot_free(None, None, 0) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_pool_set_option(None, 1, 64) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_pool_shape(None, None, None, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_pool_device(None, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_slot_bytes(None) == 0
    assert L.wkv7_pool_state_ptr(None) is None
    assert L.wkv7_pool_destroy(None) == W.WKV7_OK
    out = ctypes.c_void_p(123)
    assert L.wkv7_plan_create(None, None, None, 0, ctypes.byref(out)) == \
        W.WKV7_ERR_INVALID_ARG
    assert out.value is None
    assert L.wkv7_plan_create(None, None, None, 0, None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_forward_plan(None, None, 0, *([None] * 8)) == \
        W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_plan_tokens(None) == 0
    assert L.wkv7_plan_destroy(None) == W.WKV7_OK


def test_last_error_is_per_thread():
    import threading
    W.lib.wkv7_forward(None, None, None, 0, 0, *([None] * 8))
    seen = {}

    def other():
        seen["msg"] = W.wkv7_last_error()
    t = threading.Thread(target=other)
    t.start()
    t.join()
    assert seen["msg"] == ""
    assert "NULL" in W.wkv7_last_error()


def test_image_header_roundtrip_and_rejections():
    assert ctypes.sizeof(W.wkv7_image_header) == 64
    hdr = W.wkv7_image_header_init(32, 64, 5)
    assert bytes(hdr.magic) == W.WKV7_IMAGE_MAGIC
    assert hdr.version == W.WKV7_IMAGE_VERSION and hdr.header_bytes == 64
    assert (hdr.H, hdr.N, hdr.n_slots) == (32, 64, 5)
    assert hdr.slot_bytes == 32 * 64 * 64 * 4
    W.wkv7_image_header_check(hdr, 32, 64)

    def rejected(h, H, N, code):
        with pytest.raises(W.Wkv7Error) as e:
            W.wkv7_image_header_check(h, H, N)
        assert e.value.status == code

    rejected(hdr, 12, 64, W.WKV7_ERR_UNSUPPORTED)          # other shape
    bad = W.wkv7_image_header.from_buffer_copy(hdr)
    bad.version = 2
    rejected(bad, 32, 64, W.WKV7_ERR_UNSUPPORTED)          # other version
    bad = W.wkv7_image_header.from_buffer_copy(hdr)
    bad.magic = b"WKV7SLOX"
    rejected(bad, 32, 64, W.WKV7_ERR_INVALID_ARG)
    bad = W.wkv7_image_header.from_buffer_copy(hdr)
    bad.reserved[1] = 7
    rejected(bad, 32, 64, W.WKV7_ERR_INVALID_ARG)
    bad = W.wkv7_image_header.from_buffer_copy(hdr)
    bad.slot_bytes += 4
    rejected(bad, 32, 64, W.WKV7_ERR_INVALID_ARG)
    with pytest.raises(W.Wkv7Error) as e:
        W.wkv7_image_header_init(32, 128, 1)
    assert e.value.status == W.WKV7_ERR_UNSUPPORTED
    assert W.lib.wkv7_image_header_check(None, 1, 64) == W.WKV7_ERR_INVALID_ARG
    assert W.lib.wkv7_migrate(None, None, None, None, 0, None) == \
        W.WKV7_ERR_INVALID_ARG


def test_q8_rejects_before_device():
    L = W.lib
    assert L.wkv7_q8_quantize(None, 0, 2, 4, None, None, None) == \
        W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_q8_quantize(None, 9, 2, 4, None, None, None) == \
        W.WKV7_ERR_UNSUPPORTED
    assert L.wkv7_q8_quantize(None, 0, -1, 4, None, None, None) == \
        W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_q8_matmul(None, None, 16, 100, None, None, 1, None, None) == \
        W.WKV7_ERR_UNSUPPORTED
    assert L.wkv7_q8_matmul(None, None, 16, 64, None, None, 1, None, None) == \
        W.WKV7_ERR_INVALID_ARG
    # linear: dtype, shape and pointer checks, in that order
    assert L.wkv7_q8_linear(None, None, 16, 64, None, 7, 1, None, None, None,
                            None) == W.WKV7_ERR_UNSUPPORTED
    assert L.wkv7_q8_linear(None, None, 16, 100, None, 0, 1, None, None, None,
                            None) == W.WKV7_ERR_UNSUPPORTED
    assert L.wkv7_q8_linear(None, None, 16, 64, None, 1, -1, None, None, None,
                            None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_q8_linear(None, None, 16, 64, None, 1, 1, None, None, None,
                            None) == W.WKV7_ERR_INVALID_ARG
    assert L.wkv7_q8_linear(None, None, 16, 64, None, 1, 0, None, None, None,
                            None) == W.WKV7_OK            # nothing to do

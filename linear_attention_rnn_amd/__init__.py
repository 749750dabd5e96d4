"""libwkv7: the RWKV-7 WKV state-slot hot path for MI355X (gfx950).

The C ABI is declared in include/wkv7.h and built into libwkv7.so by
`python -m linear_attention_rnn_amd.build`; `linear_attention_rnn_amd.wkv7`
is its ctypes binding.
"""

"""The oracle's operators against their pins (closed forms, invariants, brute force)."""
import oracle
from tests import pins


def test_bf16_round():
    pins.check_bf16_round(oracle.bf16_round)


def test_widen_bf16():
    pins.check_widen(oracle.widen_bf16)


def test_embedding():
    pins.check_embedding(oracle.embedding)


def test_rms_norm():
    pins.check_rms_norm(oracle.rms_norm)


def test_rope():
    pins.check_rope(oracle.rope, oracle.rope_cos_sin)


def test_linear():
    pins.check_linear(oracle.linear)


def test_attention():
    pins.check_attention(oracle.attention)


def test_silu_swiglu():
    pins.check_silu_swiglu(oracle.silu, oracle.swiglu)


def test_argmax():
    pins.check_argmax(oracle.argmax)


def test_rearrange():
    import numpy as np
    x = np.arange(60, dtype=np.float32).reshape(3, 4, 5).transpose(2, 0, 1)
    y = oracle.rearrange(x)
    assert y.flags.c_contiguous and y.shape == x.shape
    for idx in np.ndindex(*x.shape):
        assert y[idx] == x[idx]


def test_e4m3_codec():
    pins.check_e4m3(oracle.e4m3_values, oracle.e4m3_encode, oracle.e4m3_decode)


def test_kv_block_quantization():
    pins.check_kv_quant(oracle.kv_quantize, oracle.kv_dequantize)

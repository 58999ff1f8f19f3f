"""Oracle pins: attention over fp8 (OCP E4M3, finite form) KV caches.

The decode of every byte equals torch's float8_e4m3fn conversion; hand values
of the format (1.0, the largest finite 448, the smallest subnormal 2^-9, the
smallest normal 2^-6, -0, NaN); and attention over fp8 caches with scales
equals, bit for bit, the fp32 oracle on the dequantized caches (power-of-two
scales keep the dequantized values exact in fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import to_fp8_e4m3


def test_decode_matches_torch_and_hand_values():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.fp8_e4m3(i) for i in range(256)])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan) and nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])
    assert oracle.fp8_e4m3(0x38) == 1.0 and oracle.fp8_e4m3(0x7E) == 448.0
    assert oracle.fp8_e4m3(0x01) == 2.0 ** -9 and oracle.fp8_e4m3(0x08) == 2.0 ** -6
    assert oracle.fp8_e4m3(0x80) == 0.0 and math.copysign(1.0, oracle.fp8_e4m3(0x80)) < 0
    assert oracle.fp8_e4m3(0xB8) == -1.0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp8_attention_equals_dequantized(dtype):
    rng = np.random.default_rng(1201)
    B, Hq, Hkv, D, L, T_list = 2, 4, 2, 64, 150, (5, 3)
    Lcap = L + 5
    N = sum(T_list)
    q = rng.standard_normal((N, Hq, D)).astype(np.float32)
    k8 = to_fp8_e4m3(rng.standard_normal((B, Hkv, Lcap, D)) * 3, 0.5).numpy()
    v8 = to_fp8_e4m3(rng.standard_normal((B, Hkv, Lcap, D)), 0.25).numpy()
    cu = np.array([0, 5, 8], np.int32)
    ctx = np.array([L, L - 20], np.int32)
    parent = np.array([-1, 0, 0, 1, -1, -1, 0, 1], np.int32)
    kd = (np.vectorize(oracle.fp8_e4m3)(k8) * 0.5).astype(np.float32)
    vd = (np.vectorize(oracle.fp8_e4m3)(v8) * 0.25).astype(np.float32)
    if dtype == "bf16":
        q = (q.view(np.uint32) >> 16).astype(np.uint16)
        qf = (q.astype(np.uint32) << 16).view(np.float32)
    else:
        qf = q
    got = oracle.attention(q, k8, v8, ctx, cu, parent, Hq=Hq, Hkv=Hkv, dtype=dtype, kv_fp8_scales=(0.5, 0.25))
    ref = oracle.attention(qf, kd, vd, ctx, cu, parent, Hq=Hq, Hkv=Hkv, dtype="f32")
    assert np.array_equal(got, ref)

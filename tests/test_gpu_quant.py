"""GPU parity of the offline weight preparation and of the activation
quantizer: bytes must equal the oracle's exactly (Q8_0 blocks of 32 codes
and an fp16 scale; emit_qwen38_generate, "Where the speed comes from")."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty_u8, host, split_act_q8, unpack_device_layout

pytestmark = pytest.mark.gpu


def _special_activation(k: int) -> np.ndarray:
    x = synth.activation(0x5EED0000, 77, k, outlier_frac=0.01)
    if k >= 256:
        x[32:64] = 0.0                      # zero block
        x[64:96] = 1e-12                    # scale underflows fp16
        s = np.float32(2.0 ** -7)           # planted half quotients, d = 2^-7 exactly
        x[96:128] = 0.0
        x[96] = 127 * s
        x[97:103] = np.array([2.5, -2.5, 0.5, -0.5, 126.5, 3.5], np.float32) * s
        x[128:160] = -0.0
        x[160:192] = 3e-4                    # subnormal fp16 scale
        x[160] = 2.5e-3
    return x


@pytest.mark.parametrize("k", [32, 96, 1024, 2080, 4096, 5120, 17408])
def test_quantize_act_bitexact(gpu_lib, k):
    wsg = gpu_lib
    x = _special_activation(k)
    xq = empty_u8(wsg.act_q8_0_bytes(k))
    wsg.quantize_act_q8_0(dev(x), k, xq)
    d_gpu, q_gpu = split_act_q8(host(xq), k)
    d_ref, q_ref = oracle.quantize_q8_0(x)
    assert np.array_equal(d_gpu, d_ref)
    assert np.array_equal(q_gpu, q_ref)


@pytest.mark.parametrize("n,k", [(1, 32), (3, 96), (17, 2080), (64, 4128), (33, 5120), (5, 17408)])
def test_quantize_weights_bitexact(gpu_lib, n, k):
    wsg = gpu_lib
    w = synth.normal_f32(0x5EED0001, 5, n * k, 0.02).reshape(n, k)
    w[0, :32] = 0.0
    if k >= 64:
        w[-1, 32:64] = 1e-12
    packed = empty_u8(wsg.q8_0_packed_bytes(n, k))
    wsg.quantize_q8_0_weights(dev(w), n, k, packed)
    d_gpu, q_gpu, pad = unpack_device_layout(host(packed), n, k)
    d_ref, q_ref = oracle.quantize_q8_0(w)
    assert np.array_equal(d_gpu, d_ref)
    assert np.array_equal(q_gpu, q_ref)
    assert not pad.any()


@pytest.mark.parametrize("n,k", [(2, 32), (7, 2048), (9, 2112), (3, 8224)])
def test_pack_q8_0_from_canonical_blocks(gpu_lib, n, k):
    wsg = gpu_lib
    d, q = synth.q8_blocks(0x5EED0002, 10, n, k)
    aos = synth.blocks_to_aos(d, q)
    packed = empty_u8(wsg.q8_0_packed_bytes(n, k))
    wsg.pack_q8_0(dev(aos.reshape(-1)), n, k, packed)
    d_gpu, q_gpu, pad = unpack_device_layout(host(packed), n, k)
    assert np.array_equal(d_gpu, d)
    assert np.array_equal(q_gpu, q)
    assert not pad.any()


def test_pack_into_row_ranges_concatenates(gpu_lib):
    """Projections that share an activation are stacked by rows: packing each
    part at its row offset gives the concatenated matrix."""
    wsg = gpu_lib
    k = 1024
    parts = [synth.q8_blocks(0x5EED0002, 20 + 2 * i, r, k) for i, r in enumerate((5, 3, 2))]
    n = 10
    rb = wsg.q8_0_row_bytes(k)
    packed = empty_u8(n * rb)
    r0 = 0
    for d, q in parts:
        aos = synth.blocks_to_aos(d, q)
        wsg.pack_q8_0(dev(aos.reshape(-1)), d.shape[0], k, packed.data_ptr() + r0 * rb)
        r0 += d.shape[0]
    d_gpu, q_gpu, _ = unpack_device_layout(host(packed), n, k)
    assert np.array_equal(d_gpu, np.concatenate([p[0] for p in parts]))
    assert np.array_equal(q_gpu, np.concatenate([p[1] for p in parts]))


def test_convert_bf16_bitexact(gpu_lib):
    import torch
    wsg = gpu_lib
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=1_000_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    x = x[np.isfinite(x)]
    extra = np.array([0.0, -0.0, np.inf, -np.inf, 3.3895314e38, 1 + 2 ** -8, 1 + 3 * 2 ** -8,
                      1e-40, -1e-45], np.float32)
    x = np.concatenate([x, extra, (rng.standard_normal(100_000) * 0.02).astype(np.float32)])
    out = torch.empty(x.size, dtype=torch.int16, device="cuda")
    wsg.convert_bf16(dev(x), x.size, out)
    got = host(out).view(np.uint16)
    assert np.array_equal(got, oracle.f32_to_bf16_bits(x))

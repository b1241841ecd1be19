"""GPU parity of the fused residual add + RMSNorm + Q8_0 re-quantization
(emit_qwen38_generate, "Where the speed comes from", item 3; GPU Kernel
Lab, "Decode integration").

Against the oracle on the same inputs:
* h' = h + r is one IEEE fp32 add, so h_out is bit-exact;
* y within 2^-16 |y_ref|.  Derivation: the kernel sums the k squares in fp32
  along chains of at most 8*7 (per thread) + 6 (wave butterfly) + 16 (wave
  partials) = 78 additions, relative error <= 78 * 2^-24 ~ 4.6e-6; the square
  root halves it and the divide, root, reciprocal and two products add
  about 5 * 2^-24, so |y - y_ref| <= ~2.7e-6 |y_ref| < 2^-16 |y_ref|;
* the codes and scales are bit-exact against the oracle's Q8_0 quantizer
  applied to the y the kernel computed (the integer decision is taken on the
  same fp32 values on both sides).
"""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import dev, empty_u8, host, split_act_q8

pytestmark = pytest.mark.gpu

SEED = 0x5EED0009
Y_REL_TOL = 2.0 ** -16

# every units-per-thread path (1..7 eight-value units per thread of 1024),
# small and ragged thread counts, and the largest k
KS = [32, 96, 1056, 4096, 5120, 8224, 17408, 32768, 40960, 49152, 57344]


def _inputs(k, scale=1.0, tensor=0):
    h = synth.normal_f32(SEED, 3 * tensor, k, 1.0) * np.float32(scale)
    r = synth.normal_f32(SEED, 3 * tensor + 1, k, 0.5) * np.float32(scale)
    g = (np.float32(1.0) + synth.normal_f32(SEED, 3 * tensor + 2, k, 0.1)).astype(np.float32)
    return h.astype(np.float32), r.astype(np.float32), g


def _run(wsg, h, r, g, eps, want=("h_out", "y", "y_q8"), inplace=False):
    import torch
    k = h.size
    dh = dev(h)
    dr = dev(r) if r is not None else None
    dg = dev(g) if g is not None else None
    h_out = (dh if inplace else torch.empty(k, dtype=torch.float32, device="cuda")) if "h_out" in want else None
    y = torch.empty(k, dtype=torch.float32, device="cuda") if "y" in want else None
    yq = empty_u8(wsg.act_q8_0_bytes(k)) if "y_q8" in want else None
    wsg.residual_rmsnorm_q8_0(dh, dr, dg, k, eps, h_out, y, yq)
    out = {}
    if h_out is not None:
        out["h_out"] = host(h_out)
    if y is not None:
        out["y"] = host(y)
    if yq is not None:
        out["y_q8"] = host(yq)
    return out


def _check(out, h, r, g, eps):
    k = h.size
    g_ref = g if g is not None else np.ones(k, np.float32)
    h_ref, y_ref = oracle.residual_rmsnorm(h, r, g_ref, eps)
    if "h_out" in out:
        assert np.array_equal(out["h_out"].view(np.uint32), h_ref.view(np.uint32)), "h_out not bit-exact"
    y = out["y"]
    err = np.abs(y.astype(np.float64) - y_ref)
    bad = np.nonzero(err > Y_REL_TOL * np.abs(y_ref))[0]
    assert bad.size == 0, (bad[:5].tolist(), y[bad[:5]].tolist(), y_ref[bad[:5]].tolist())
    if "y_q8" in out:
        d_gpu, q_gpu = split_act_q8(out["y_q8"], k)
        d_ref, q_ref = oracle.quantize_q8_0(y)
        assert np.array_equal(d_gpu, d_ref), "scales differ"
        assert np.array_equal(q_gpu, q_ref), "codes differ"


@pytest.mark.parametrize("k", KS)
def test_residual_rmsnorm_matches_oracle(gpu_lib, k):
    h, r, g = _inputs(k)
    _check(_run(gpu_lib, h, r, g, 1e-6), h, r, g, 1e-6)


@pytest.mark.parametrize("k", [96, 5120, 40960])
def test_without_residual_or_weight(gpu_lib, k):
    h, r, g = _inputs(k, tensor=1)
    _check(_run(gpu_lib, h, None, g, 1e-6), h, None, g, 1e-6)
    _check(_run(gpu_lib, h, r, None, 1e-6), h, r, None, 1e-6)
    _check(_run(gpu_lib, h, None, None, 1e-5), h, None, None, 1e-5)


@pytest.mark.parametrize("k", [1056, 17408])
def test_in_place_residual_update(gpu_lib, k):
    h, r, g = _inputs(k, tensor=2)
    _check(_run(gpu_lib, h, r, g, 1e-6, inplace=True), h, r, g, 1e-6)


@pytest.mark.parametrize("k", [5120, 57344])
def test_outputs_are_independent_of_which_are_requested(gpu_lib, k):
    wsg = gpu_lib
    h, r, g = _inputs(k, tensor=3)
    full = _run(wsg, h, r, g, 1e-6)
    assert np.array_equal(_run(wsg, h, r, g, 1e-6, want=("y_q8",))["y_q8"], full["y_q8"])
    assert np.array_equal(_run(wsg, h, r, g, 1e-6, want=("y",))["y"].view(np.uint32), full["y"].view(np.uint32))
    assert np.array_equal(_run(wsg, h, r, g, 1e-6, want=("h_out",))["h_out"].view(np.uint32),
                          full["h_out"].view(np.uint32))
    again = _run(wsg, h, r, g, 1e-6)
    for name in full:
        assert np.array_equal(again[name].view(np.uint8), full[name].view(np.uint8)), name


@pytest.mark.parametrize("scale", [2.0 ** -40, 2.0 ** -10, 2.0 ** 20, 2.0 ** 50])
def test_adversarial_scales(gpu_lib, scale):
    # tiny vectors are dominated by eps; large ones must not lose the mean
    h, r, g = _inputs(5120, scale=scale, tensor=4)
    _check(_run(gpu_lib, h, r, g, 1e-6), h, r, g, 1e-6)


def test_zero_and_cancelling_input(gpu_lib):
    k = 2048
    h, r, g = _inputs(k, tensor=5)
    out = _run(gpu_lib, h, -h, g, 1e-6)  # h + r == 0 exactly
    assert not out["h_out"].any() and not out["y"].any()
    assert not out["y_q8"].any()  # zero codes and +0 scales
    _check(out, h, -h, g, 1e-6)
    # one block cancels, the rest does not
    r2 = r.copy()
    r2[64:96] = -h[64:96]
    _check(_run(gpu_lib, h, r2, g, 1e-6), h, r2, g, 1e-6)

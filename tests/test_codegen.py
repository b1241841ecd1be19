"""The row loops' weight loads stay pipelined in the code hipcc generates for
gfx950 (host-only check: device assembly of the library's own sources).

Every step of a row loop issues the same loads, so the compiler can wait for
one ring set at a time.  If a load or a store were issued on some paths of
the loop only, the compiler would instead wait for every outstanding load
before each item (the ring would hold one item in flight instead of two),
which costs ~10% of the weight stream's bandwidth without changing any
result -- so no numeric test would notice.  Checked here:

* no kernel uses scratch memory (no register spills);
* in the int8 kernels, some dot-product block waits with at least 6 vector
  memory operations still outstanding (two one-chunk items of 3 loads)."""
import os
import re
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from weight_streaming_gemv_q8_amd import build as libbuild

SOURCES = ["stream.hip", "gemv.hip", "norm.hip", "decode.hip"]


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    out = tmp_path_factory.mktemp("asm")

    def compile_one(src):
        path = str(out / (src + ".s"))
        cmd = ["hipcc", *libbuild.HIP_FLAGS, "-x", "hip", "-S", "--cuda-device-only",
               os.path.join(libbuild.CSRC, src), "-o", path]
        subprocess.run(cmd, check=True, capture_output=True)
        return src, open(path).read()

    with ThreadPoolExecutor(len(SOURCES)) as ex:
        return dict(ex.map(compile_one, SOURCES))


def _kernels(text):
    """name -> assembly of each kernel function (to its end label: a kernel
    may have more than one s_endpgm)."""
    out = {}
    for m in re.finditer(r"^(_Z\S+):[^\n]*\n(.*?)^\.Lfunc_end", text, re.S | re.M):
        out[m.group(1)] = m.group(2)
    return out


def _max_wait_before_dot(body):
    """Largest vmcnt of the waits that directly precede a v_dot4 block."""
    best, last = -1, None
    for line in body.splitlines():
        m = re.search(r"s_waitcnt\s+vmcnt\((\d+)\)", line)
        if m:
            last = int(m.group(1))
        elif "v_dot4" in line and last is not None:
            best = max(best, last)
            last = None
        elif re.match(r"\.LBB|\s*s_cbranch|\s*s_branch", line):
            last = None
    return best


@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch(asm, src):
    sizes = re.findall(r"\.private_segment_fixed_size:\s*(\d+)", asm[src])
    assert sizes and all(int(s) == 0 for s in sizes), f"{src}: a kernel spills to scratch"


def test_stream_ring_keeps_two_items_in_flight(asm):
    ks = {n: b for n, b in _kernels(asm["stream.hip"]).items() if "stream_kernel" in n and "Lb0E" in n}
    assert ks
    for name, body in ks.items():
        assert _max_wait_before_dot(body) >= 6, name


def test_fused_norm_and_swiglu_gemvs_keep_two_items_in_flight(asm):
    # the GEMVs that compute the residual add + RMSNorm in their prologue,
    # and the gate+up GEMV with the SwiGLU epilogue (int8 activations: the
    # block dot; f32 activations, the W8A16 form: the dequantizing FMAs)
    ks = {n: b for n, b in _kernels(asm["gemv.hip"]).items()
          if "q8_i8_norm_kernel" in n or "q8_i8_swiglu_kernel" in n or "q8_f32_norm_kernel" in n}
    f32 = {n for n in ks if "q8_f32_norm_kernel" in n or re.search(r"q8_i8_swiglu_kernelILi\d+ELi1EE", n)}
    assert ks and f32 and len(f32) < len(ks)
    for name, body in ks.items():
        if name in f32:
            assert _max_wait_before_fma(body) >= 6, name
        else:
            assert _max_wait_before_dot(body) >= 6, name


def test_w4_ring_keeps_two_items_in_flight(asm):
    # 4-bit items are two loads (codes and scale): two in flight = 4
    ks = {n: b for n, b in _kernels(asm["gemv.hip"]).items() if "q4_i8_" in n}
    assert len(ks) == 18 + 9 + 6  # plain, fused-norm and SwiGLU instantiations
    for name, body in ks.items():
        assert _max_wait_before_dot(body) >= 4, name


def _max_wait_before_fma(body):
    """Largest vmcnt of the waits that directly precede an f32 FMA."""
    best, last = -1, None
    for line in body.splitlines():
        m = re.search(r"s_waitcnt\s+vmcnt\((\d+)\)", line)
        if m:
            last = int(m.group(1))
        elif re.search(r"v_fmac?_f32", line) and last is not None:
            best = max(best, last)
            last = None
        elif re.match(r"\.LBB|\s*s_cbranch|\s*s_branch", line):
            last = None
    return best


def test_w4_f32_ring_keeps_two_items_in_flight(asm):
    ks = {n: b for n, b in _kernels(asm["gemv.hip"]).items() if "q4_f32_kernel" in n}
    assert len(ks) == 9
    for name, body in ks.items():
        assert _max_wait_before_fma(body) >= 4, name


def test_eager_int8_ring_keeps_two_items_in_flight(asm):
    # one-chunk items (U = 1), int8 activations and the requantizing staging
    ks = {n: b for n, b in _kernels(asm["gemv.hip"]).items()
          if re.search(r"q8_i8_kernelILi\d+ELi\dELi1ELi[02]ELb1ELb0ELb0E", n)}
    assert ks
    for name, body in ks.items():
        assert _max_wait_before_dot(body) >= 6, name

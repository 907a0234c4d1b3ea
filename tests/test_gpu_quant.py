"""GPU quantisers vs the oracle: codes, scales and Kbar must be bit-exact."""
import numpy as np
import pytest
import torch

import bit_quantized_attention_qk4pv8_amd as qfa
import oracle
from bit_quantized_attention_qk4pv8_amd.workloads import WORKLOADS, bf16_bits, make_inputs
from gpu_util import say, to_np

pytestmark = pytest.mark.gpu


def _check_qk4(x: torch.Tensor, smooth: bool, label: str, prescale: float = 1.0):
    say("quantize_qk4", label, tuple(x.shape), "smooth", smooth, "prescale", prescale)
    codes, scales, kbar = qfa.quantize_qk4(x, smooth=smooth, prescale=prescale)
    torch.cuda.synchronize()
    oc, os_, ok = oracle.quantize_qk4(bf16_bits(x), smooth=smooth, prescale=prescale)
    assert np.array_equal(to_np(codes), oc), label + ": codes differ"
    assert np.array_equal(to_np(scales), os_), label + ": scales differ"
    if smooth:
        assert np.array_equal(to_np(kbar.view(torch.int16)).view(np.uint16), ok), label + ": kbar differs"


def _check_v8(v: torch.Tensor, label: str):
    say("quantize_v8", label, tuple(v.shape))
    codes, scales = qfa.quantize_v8(v)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_v8(bf16_bits(v))
    assert np.array_equal(to_np(codes), oc), label + ": codes differ"
    assert np.array_equal(to_np(scales), os_), label + ": scales differ"


@pytest.mark.parametrize("shape,smooth", [((1, 2, 300, 64), False), ((1, 3, 1000, 128), False),
                                          ((2, 2, 300, 128), True), ((1, 1, 77, 256), True),
                                          ((1, 1, 5, 32), False)])
def test_qk4_bitexact_shapes(shape, smooth):
    g = torch.Generator(device="cuda").manual_seed(sum(shape))
    x = torch.randn(shape, generator=g, device="cuda")
    x[..., 3] *= 40.0                                             # outlier channel
    x[..., 0, :] = 0.0                                            # all-zero row
    x += torch.randn((1, shape[1], 1, shape[3]), generator=g, device="cuda") * 3.0 * smooth
    _check_qk4(x.to(torch.bfloat16), smooth, "shape%s" % (shape,))
    # Q side: the softmax factor applied in binary32 before the block scale is chosen
    _check_qk4(x.to(torch.bfloat16), False, "shape%s.prescaled" % (shape,), prescale=oracle.exp2_scale(0.0883883))


@pytest.mark.parametrize("shape", [(1, 2, 75, 64), (2, 3, 1000, 128), (1, 1, 31, 128), (1, 1, 64, 256)])
def test_v8_bitexact_shapes(shape):
    g = torch.Generator(device="cuda").manual_seed(sum(shape) + 1)
    v = torch.randn(shape, generator=g, device="cuda")
    v[..., 5, :] *= 100.0
    v[..., :, 7] *= 1e-3
    _check_v8(v.to(torch.bfloat16), "shape%s" % (shape,))


def _check_v4(v: torch.Tensor, label: str):
    say("quantize_v4", label, tuple(v.shape))
    codes, scales = qfa.quantize_v4(v)
    torch.cuda.synchronize()
    oc, os_ = oracle.quantize_v4(bf16_bits(v))
    assert np.array_equal(to_np(codes), oc), label + ": codes differ"
    assert np.array_equal(to_np(scales), os_), label + ": scales differ"


@pytest.mark.parametrize("shape", [(1, 2, 75, 64), (2, 3, 1000, 128), (1, 1, 31, 128), (1, 1, 64, 256)])
def test_v4_bitexact_shapes(shape):
    g = torch.Generator(device="cuda").manual_seed(sum(shape) + 2)
    v = torch.randn(shape, generator=g, device="cuda")
    v[..., 5, :] *= 100.0
    v[..., :, 7] *= 1e-3
    _check_v4(v.to(torch.bfloat16), "shape%s" % (shape,))


def _check_nvfp4(x: torch.Tensor, smooth: bool, label: str, prescale: float = 1.0):
    xs = x.float() * prescale if prescale != 1.0 else x.float()
    g = qfa.nvfp4_tensor_scale(float(xs.abs().nan_to_num(0.0, 0.0, 0.0).max()))
    say("quantize_nvfp4", label, tuple(x.shape), "smooth", smooth, "prescale", prescale, "g", g)
    codes, scales, kbar = qfa.quantize_nvfp4(x, g, smooth=smooth, prescale=prescale)
    torch.cuda.synchronize()
    oc, os_, ok = oracle.quantize_nvfp4(bf16_bits(x), g, smooth=smooth, prescale=prescale)
    assert np.array_equal(to_np(codes), oc), label + ": codes differ"
    assert np.array_equal(to_np(scales), os_), label + ": scales differ"
    if smooth:
        assert np.array_equal(to_np(kbar.view(torch.int16)).view(np.uint16), ok), label + ": kbar differs"


@pytest.mark.parametrize("shape,smooth", [((1, 2, 300, 64), False), ((1, 3, 1000, 128), False),
                                          ((2, 2, 300, 128), True), ((1, 1, 77, 256), False)])
def test_nvfp4_bitexact_shapes(shape, smooth):
    g = torch.Generator(device="cuda").manual_seed(sum(shape) + 3)
    x = torch.randn(shape, generator=g, device="cuda")
    x[..., 3] *= 40.0
    x[..., 0, :] = 0.0
    x[..., 5, 16:32] *= 1e-4
    x += torch.randn((1, shape[1], 1, shape[3]), generator=g, device="cuda") * 3.0 * smooth
    xb = x.to(torch.bfloat16)
    _check_nvfp4(xb, smooth, "shape%s" % (shape,))
    _check_nvfp4(xb, False, "shape%s.prescaled" % (shape,), prescale=oracle.exp2_scale(0.0883883))


def test_quantizers_nonfinite_and_tiny():
    x = torch.randn((1, 1, 64, 128), device="cuda")
    x[0, 0, 1, 5] = float("nan")
    x[0, 0, 2, 100] = float("inf")
    x[0, 0, 3, :32] = 1e-39                 # bf16 subnormals
    x[0, 0, 4, 32:64] = -0.0
    xb = x.to(torch.bfloat16)
    _check_qk4(xb, False, "nonfinite")
    _check_qk4(xb, False, "nonfinite.prescaled", prescale=oracle.exp2_scale(0.125))
    _check_v8(xb, "nonfinite")
    _check_v4(xb, "nonfinite")
    _check_nvfp4(xb, False, "nonfinite")
    _check_qk4(xb, True, "nonfinite.smooth")
    _check_nvfp4(xb, True, "nonfinite.smooth")


def _row_order_vs_grouped(col: np.ndarray, groups: int):
    """Binary64 sums of one channel of one tile: in row order, and as `groups`
    strided partial sums added up afterwards."""
    seq = 0.0
    for v in col:
        seq += float(v)
    parts = [0.0] * groups
    for j, v in enumerate(col):
        parts[j % groups] += float(v)
    tot = 0.0
    for p in parts:
        tot += p
    return seq, tot


@pytest.mark.parametrize("D", [64, 96, 128, 256])
def test_kbar_order_sensitive_tiles(D):
    """K-bar is the row-order binary64 sum also where the order changes the
    result (a tile whose values span more exponents than binary64 adds
    exactly), next to tiles that sum exactly (wide but bounded range), hold
    an infinity or a NaN, or mix subnormals with normal values."""
    rng = np.random.default_rng(D)
    x = rng.standard_normal((1, 2, 300, D)).astype(np.float32)
    col = np.ones(128, np.float32)
    col[0], col[64] = 2.0 ** 60, -(2.0 ** 60)
    x[0, 0, :128, 0] = col
    seq, grouped = _row_order_vs_grouped(col, 256 // (D // 8))
    assert seq != grouped  # the case is order sensitive
    x[0, 0, :128, 1] = -col
    # exponents within 38 of each other: exact in any order
    e = rng.integers(-19, 20, size=(128, D))
    x[0, 0, 128:256] = (np.ldexp(1.0, e) * rng.uniform(1.0, 2.0, (128, D)) * rng.choice([-1.0, 1.0], (128, D))
                        ).astype(np.float32)
    x[0, 0, 260, 3] = np.inf
    x[0, 0, 270, 4] = np.nan
    x[0, 0, 280:290, 5] = -np.inf
    x[0, 0, 281, 6], x[0, 0, 282, 6] = np.inf, -np.inf
    x[0, 1, :128, :8] = 1e-39                    # bf16 subnormals beside normal values
    x[0, 1, 3, :8] = 3.0
    x[0, 1, 128:256, 9] = 3.0e38                 # sums past the bf16 range
    xb = torch.from_numpy(x).to(torch.bfloat16).cuda()
    _check_qk4(xb, True, "kbar-order D%d" % D)
    _check_nvfp4(xb, True, "kbar-order D%d" % D)


@pytest.mark.parametrize("name", ["tiny", "llama16k", "qwen32k"])
def test_workload_tensors_bitexact(name):
    w = WORKLOADS[name]
    inp = make_inputs(w, seed=0)
    _check_qk4(inp["q"], False, name + ".q", prescale=oracle.exp2_scale(w.scale))
    _check_qk4(inp["k"], w.smooth, name + ".k")
    _check_v8(inp["v"], name + ".v")


def test_long128k_and_decode_slices_bitexact():
    w = WORKLOADS["long128k"]
    inp = make_inputs(w, seed=0)
    _check_qk4(inp["k"][:, :2].contiguous(), False, "long128k.k[:2]")
    _check_v8(inp["v"][:, 6:].contiguous(), "long128k.v[6:]")
    _check_qk4(inp["q"][:, 5:7].contiguous(), False, "long128k.q[5:7]", prescale=oracle.exp2_scale(w.scale))
    del inp
    wd = WORKLOADS["decode"]
    inp = make_inputs(wd, seed=0, B_override=3)
    _check_qk4(inp["k"], False, "decode.k")
    _check_v8(inp["v"], "decode.v")

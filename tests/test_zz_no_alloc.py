"""qfa_fwd_decode_noalloc (the decode entry point that allocates nothing) against
qfa_fwd_decode with a caller workspace, through the C ABI: two calls in a row,
the second with a smaller input, must give the same O and LSE as the
workspace entry point on the same inputs.  An oversized shape is rejected on
the host with QFA_ERR_WORKSPACE.
"""
import math

import numpy as np
import pytest
import torch

import bit_quantized_attention_qk4pv8_amd as qfa
import oracle
from bit_quantized_attention_qk4pv8_amd.workloads import bf16_bits
from gpu_util import compare_o, say, to_np

pytestmark = pytest.mark.gpu


def _case(B, Hq, Hkv, L, D, seed, lens=None):
    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev).manual_seed(seed)
    q = torch.randn((B, Hq, 1, D), generator=g, device=dev).to(torch.bfloat16)
    k = torch.randn((B, Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((B, Hkv, L, D), generator=g, device=dev).to(torch.bfloat16)
    k4, k4s, _ = qfa.quantize_qk4(k)
    v8, v8s = qfa.quantize_v8(v)
    kv_lens = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=dev)
    return q, k, v, k4, k4s, v8, v8s, kv_lens


def _noalloc(q, k4, k4s, v8, v8s, L, kv_lens, scale, splits):
    B, Hq, _, D = q.shape
    Hkv = k4.shape[1]
    O = torch.full((B, Hq, D), float("nan"), dtype=torch.float32, device=q.device)
    lse = torch.full((B, Hq), float("nan"), dtype=torch.float32, device=q.device)
    used = qfa.qfa_fwd_decode_noalloc(None, None, k4, k4s, None, q, v8, v8s, B, Hq, Hkv, L, kv_lens, D, scale, 32,
                                      splits, O, lse)
    return O, lse, used


@pytest.mark.parametrize("order", ["large_then_small"])
def test_noalloc_decode_matches_workspace_decode(order):
    cases = [dict(B=8, Hq=32, Hkv=8, L=4000, D=128, seed=5, lens=None, splits=0),
             dict(B=3, Hq=8, Hkv=2, L=700, D=64, seed=6, lens=[700, 129, 0], splits=3)]
    for c in cases:
        q, k, v, k4, k4s, v8, v8s, kv_lens = _case(c["B"], c["Hq"], c["Hkv"], c["L"], c["D"], c["seed"], c["lens"])
        scale = 1.0 / math.sqrt(c["D"])
        say("noalloc decode B%d Hq%d L%d D%d splits %d" % (c["B"], c["Hq"], c["L"], c["D"], c["splits"]))
        O1, l1, u1 = _noalloc(q, k4, k4s, v8, v8s, c["L"], kv_lens, scale, c["splits"])
        O2, l2, u2 = qfa.fwd_decode(None, None, k4, k4s, v8, v8s, c["L"], scale, num_splits=c["splits"],
                                    kv_lens=kv_lens, q_bf16=q)
        torch.cuda.synchronize()
        assert u1 == u2
        # the same kernels on the same inputs: identical results
        assert torch.equal(O1, O2)
        assert torch.equal(torch.nan_to_num(l1, neginf=-1e30), torch.nan_to_num(l2, neginf=-1e30))
        # and within the parity bar of the oracle
        rows = np.array([(b, h, 0) for b in range(c["B"]) for h in range(c["Hq"])], dtype=np.int64)
        res = oracle.decode_rows(bf16_bits(q), bf16_bits(k), bf16_bits(v), rows, scale, u1, kv_lens=c["lens"],
                                 exact=False)
        compare_o(to_np(O1)[rows[:, 0], rows[:, 1]], res["O_q"], to_np(l1)[rows[:, 0], rows[:, 1]],
                  res["lse_q"], label="noalloc-B%d-L%d-D%d" % (c["B"], c["L"], c["D"]))


def test_noalloc_rejects_oversized_shape_on_host():
    dev = torch.device("cuda:0")
    B, Hq, Hkv, L, D, splits = 64, 64, 8, 65536, 128, 64  # 64*64*64*128*4 B of partials > 32 MiB
    need = qfa.qfa_decode_workspace_bytes(B, Hq, D, splits)
    assert need > qfa.QFA_DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((B, Hq, 1, D), dtype=torch.bfloat16, device=dev)
    k4 = torch.zeros((16,), dtype=torch.uint8, device=dev)  # never touched: the call is rejected first
    O = torch.zeros((B, Hq, D), dtype=torch.float32, device=dev)
    lse = torch.zeros((B, Hq), dtype=torch.float32, device=dev)
    with pytest.raises(qfa.QfaError) as e:
        qfa.qfa_fwd_decode_noalloc(None, None, k4, k4, None, q, k4, k4, B, Hq, Hkv, L, None, D, 0.1, 32, splits,
                                   O, lse)
    assert e.value.status == qfa.QFA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert float(O.abs().sum()) == 0.0  # nothing was written

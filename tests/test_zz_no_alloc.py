"""attnfuse_decode_noalloc (partials in the library's static per-GPU buffer)
against attnfuse_decode (caller workspace), both through the C ABI: identical
outputs and lse on two calls in a row, the second with a smaller input (the
buffer still holds the first call's partials), each also within the oracle's
tolerance; an oversized request is refused."""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import oracle
import workloads
from gpu_helpers import check_close, check_lse, host, log, to_dev

pytestmark = pytest.mark.gpu

CASES = [  # B, Hq, Hkv, Nk, D, splits, rope_theta
    (1, 64, 8, 8192, 128, 64, 5e5),   # Llama-3-70B heads, 8k cache: 2.1 MB of partials
    (2, 8, 2, 1000, 64, 7, 1e4),      # smaller: 29 KB of partials
]


def test_decode_noalloc_matches_decode_on_two_calls():
    rng = np.random.default_rng(31)
    for B, Hq, Hkv, Nk, D, splits, theta in CASES:
        (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                     ((B, Hq, 1, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D)))
        qd, kd, vd = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
        kw = dict(rope_theta=theta, q_pos0=Nk)
        log(f"case decode_noalloc B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} D={D} splits={splits}")
        ref_out, ref_lse = af.decode(qd, kd, vd, num_splits=splits, return_lse=True, **kw)
        out = torch.empty_like(qd)
        lse = torch.empty((B, Hq, 1), dtype=torch.float32, device="cuda")
        af.decode_noalloc(qd, kd, vd, out, num_splits=splits, lse=lse, **kw)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(out), host(ref_out))
        np.testing.assert_array_equal(host(lse), host(ref_lse))
        oref, olse = oracle.attention(q, k, v, **kw)
        check_close(host(out), oref, "bf16", f"decode_noalloc {B, Hq, Hkv, Nk, D, splits}")
        check_lse(host(lse), olse, 2e-2, f"decode_noalloc {B, Hq, Hkv, Nk, D, splits}")


def test_decode_noalloc_refuses_more_partials_than_its_buffer():
    q = torch.zeros(1, 64, 1, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 8, 256, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(q)
    splits = 8 * 1024 * 1024 // (64 * 130 * 4) + 1
    with pytest.raises(af.AttnfuseError) as e:
        af.decode_noalloc(q, k, k, out, num_splits=splits)
    assert e.value.status == -3

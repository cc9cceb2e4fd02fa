"""GPU parity of the fp8 prefill (Q, K, V as OCP E4M3 codes with per-tensor
scales, "9.1 Limitations and Future Directions"): the oracle runs on the
dequantised values (code * scale) and the output must meet the bf16 bar
(max |err| <= 2e-2, mean |err| <= 2e-3)."""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import oracle
import workloads
from gpu_helpers import check_close, check_lse, host, log, oracle_all_heads

pytestmark = pytest.mark.gpu


def _fp8_inputs(B, Hq, Hkv, Nq, Nk, D, seed):
    rng = np.random.default_rng(seed)
    return [workloads.normal_e4m3(s, rng) for s in ((B, Hq, Nq, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D))]


def _dev8(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).cuda().view(torch.float8_e4m3fn)


def _run(qkv, **kw):
    (qc, _, qs), (kc, _, ks), (vc, _, vs) = qkv
    out, lse = af.fwd(_dev8(qc), _dev8(kc), _dev8(vc), q_scale=qs, k_scale=ks, v_scale=vs, return_lse=True,
                      **kw)
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    return host(out), host(lse)


CASES = {
    # name: (B, Hq, Hkv, Nq, Nk, D, keywords)
    "gqa_causal_ragged_d128": (2, 4, 2, 300, 300, 128, dict(causal=True)),
    "gqa4_causal_d128": (1, 16, 4, 1024, 1024, 128, dict(causal=True)),
    "dense_more_keys_d128": (2, 4, 4, 256, 320, 128, dict()),
    "window_alibi_d64": (1, 8, 8, 777, 777, 64, dict(causal=True, window=100, alibi=True)),
    "two_sided_window_d64": (2, 2, 1, 400, 400, 64, dict(window=70)),
    "queries_after_keys_d128": (1, 8, 2, 200, 64, 128, dict(causal=True, q_pos0=64)),
    "single_query_d128": (1, 8, 2, 1, 500, 128, dict(q_pos0=499, causal=True)),
}


# Paired workgroups (block n_qblk - 1 - j, then block j, in one stream):
# shapes with at least 256 pairs.
PAIRED = {
    # GQA 4:1, 15 blocks of 64 rows (odd: the middle block alone), ragged tail
    "paired_gqa_causal_odd_ragged_d128": (2, 64, 16, 950, 950, 128, dict(causal=True)),
    # ALiBi + window, MHA, 15 blocks of 256 rows, ragged tail
    "paired_alibi_window_d128": (2, 32, 32, 3600, 3600, 128, dict(causal=True, window=300, alibi=True)),
    # d = 64, queries after the keys
    "paired_after_keys_d64": (4, 32, 32, 1000, 1100, 64, dict(causal=True, q_pos0=100)),
}


def _kw_pair(kw, Hq):
    kw = dict(kw)
    okw = {k: v for k, v in kw.items() if k != "alibi"}
    if kw.pop("alibi", False):
        sl = workloads.alibi_slopes(Hq)
        kw["alibi_slopes"] = torch.from_numpy(sl).cuda()
        okw["alibi_slopes"] = sl.astype(np.float64)
    return kw, okw


@pytest.mark.parametrize("name", sorted(PAIRED))
def test_fp8_prefill_paired(name):
    B, Hq, Hkv, Nq, Nk, D, kw = PAIRED[name]
    qkv = _fp8_inputs(B, Hq, Hkv, Nq, Nk, D, seed=len(name))
    kw, okw = _kw_pair(kw, Hq)
    plan = af.fwd_plan(_dev8(qkv[0][0]), _dev8(qkv[1][0]), _dev8(qkv[2][0]), **kw)
    log(f"case fp8 prefill {name}: plan {plan}")
    assert plan["kernel"] == "fp8" and plan["paired"] == 1, plan
    out, lse = _run(qkv, **kw)
    ref, rlse = oracle_all_heads(qkv[0][1], qkv[1][1], qkv[2][1], B, Hq, **okw)
    check_close(out, ref, "bf16", f"fp8 prefill {name} (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, f"fp8 prefill {name}")


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp8_prefill_small(name):
    B, Hq, Hkv, Nq, Nk, D, kw = CASES[name]
    qkv = _fp8_inputs(B, Hq, Hkv, Nq, Nk, D, seed=len(name))
    kw = dict(kw)
    okw = {k: v for k, v in kw.items() if k != "alibi"}
    if kw.pop("alibi", False):
        sl = workloads.alibi_slopes(Hq)
        kw["alibi_slopes"] = torch.from_numpy(sl).cuda()
        okw["alibi_slopes"] = sl.astype(np.float64)
    log(f"case fp8 prefill {name}")
    out, lse = _run(qkv, **kw)
    ref, rlse = oracle.attention(qkv[0][1], qkv[1][1], qkv[2][1], **okw)
    check_close(out, ref, "bf16", f"fp8 prefill {name}")
    check_lse(lse, rlse, 2e-2, f"fp8 prefill {name}")


def test_fp8_prefill_block_mask():
    """A shared 256x64 block mask (rows of the eight-wave workgroup) and a
    per-head one with empty rows."""
    B, H, N, D = 1, 2, 512, 64
    qkv = _fp8_inputs(B, H, H, N, N, D, seed=41)
    for per_head in (False, True):
        rp, ci = workloads.random_csr(N // 256, N // 64, 0.5, seed=5, n_heads=H if per_head else 0)
        if per_head:
            rows = [[list(ci[rp[h, r]:rp[h, r + 1]]) for r in range(N // 256)] for h in range(H)]
            rows[1][0] = []  # an empty block row
            flat, rps = [], []
            for h in range(H):
                r = [len(flat)]
                for rr in rows[h]:
                    flat.extend(rr)
                    r.append(len(flat))
                rps.append(r)
            rp, ci = np.asarray(rps, dtype=np.int32), np.asarray(flat, dtype=np.int32)
        mask = af.block_mask_from_csr(rp, ci, 256, 64, "cuda")
        log(f"case fp8 prefill block mask per_head={per_head} nnz={ci.size}")
        out, lse = _run(qkv, block_mask=mask)
        ref, rlse = oracle.attention(qkv[0][1], qkv[1][1], qkv[2][1], block_mask=(rp, ci, 256, 64))
        check_close(out, ref, "bf16", f"fp8 block mask per_head={per_head}")
        check_lse(lse, rlse, 2e-2, f"fp8 block mask per_head={per_head}")


def test_fp8_prefill_full_size_alibi_window():
    """The ALiBi + causal + sliding-window workload (B=2, H=16, N=8192, D=128,
    W=1024) with Q, K, V quantised to E4M3: every output element against the
    oracle on the dequantised values."""
    w = workloads.WORKLOADS["alibi_causal_window1024_n8192"]
    qkv = _fp8_inputs(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.D, seed=w.seed)
    sl = workloads.alibi_slopes(w.Hq)
    log("case fp8 prefill ALiBi+window full size")
    out, lse = _run(qkv, causal=True, window=w.window, alibi_slopes=torch.from_numpy(sl).cuda())
    ref, rlse = oracle_all_heads(qkv[0][1], qkv[1][1], qkv[2][1], w.B, w.Hq, causal=True, window=w.window,
                                 alibi_slopes=sl.astype(np.float64))
    check_close(out, ref, "bf16", f"fp8 ALiBi+window full (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, "fp8 ALiBi+window full")


def test_fp8_prefill_no_keys_and_rejections():
    q = torch.zeros(1, 2, 40, 128, dtype=torch.float8_e4m3fn, device="cuda")
    k = torch.zeros(1, 2, 0, 128, dtype=torch.float8_e4m3fn, device="cuda")
    out, lse = af.fwd(q, k, k, return_lse=True)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    kk = torch.zeros(1, 2, 64, 128, dtype=torch.float8_e4m3fn, device="cuda")
    with pytest.raises(af.AttnfuseError):
        af.fwd(q, kk, kk, rope_theta=1e4)  # rotated values are not fp8 codes

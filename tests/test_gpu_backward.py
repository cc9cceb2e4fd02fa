"""GPU parity of the attention backward ("4.4 Backward Pass") against the fp64
oracle backward, through the C ABI, at shapes that span several tiles (128-row
query blocks, 64-key and 128-key tiles) with ragged tails, for each supported
mask / score combinator, GQA, position offsets and both head dims.

Tolerance (derived from the arithmetic): every gradient element is a sum of
products whose MFMA operands are bf16-rounded (Q', K', P, dS: relative error
2^-9 each) with fp32 accumulation, and the result is rounded to bf16.  The
errors are relative to the size of the gradients, so the bar is relative to
the largest reference magnitude: max|err| <= 2e-2 * max|ref| and
mean|err| <= 2e-3 * max|ref| (the forward's bar, scaled)."""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import oracle
import workloads
from gpu_helpers import host, log, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    "rope_causal_d128_gqa": dict(B=1, Hq=4, Hkv=2, Nq=200, Nk=200, D=128, rope_theta=1e4, causal=True),
    "plain_d128_mha": dict(B=2, Hq=2, Hkv=2, Nq=150, Nk=170, D=128),
    "window_alibi_d64": dict(B=1, Hq=4, Hkv=4, Nq=260, Nk=260, D=64, causal=True, window=70, alibi=True),
    "rope_offsets_prefix_d64_gqa8": dict(B=1, Hq=8, Hkv=1, Nq=90, Nk=300, D=64, rope_theta=5e5,
                                         causal=True, q_pos0=210, k_pos0=0),
    "noncausal_window_d128": dict(B=1, Hq=2, Hkv=1, Nq=130, Nk=190, D=128, window=40, rope_theta=500.0),
    "bias_d64_gqa": dict(B=2, Hq=4, Hkv=2, Nq=140, Nk=170, D=64, bias="full"),
    "bias_broadcast_rope_causal_alibi_d128": dict(B=1, Hq=2, Hkv=2, Nq=200, Nk=200, D=128, bias="rows",
                                                  rope_theta=1e4, causal=True, alibi=True),
    # block masks ("4.3 Block-Sparse Attention": the backward visits only listed blocks)
    "bigbird_rope_d64": dict(B=2, Hq=4, Hkv=4, Nq=512, Nk=512, D=64, rope_theta=1e4,
                             mask=("bigbird", 64, 64)),
    "blocks_128x64_causal_gqa_d128": dict(B=1, Hq=4, Hkv=2, Nq=300, Nk=330, D=128, causal=True,
                                          mask=("random", 128, 64)),
    "blocks_64x128_per_head_d64": dict(B=1, Hq=2, Hkv=1, Nq=256, Nk=384, D=64, rope_theta=500.0,
                                       mask=("per_head", 64, 128)),
}


def _mask(kind, bm, bn, Hq, Nq, Nk, rng):
    """CSR block mask (row_ptr, col_idx): BigBird, random with an empty row,
    or one random mask per q-head (row_ptr [Hq, nqb + 1])."""
    nqb, nkb = -(-Nq // bm), -(-Nk // bn)
    if kind == "bigbird":
        return workloads.bigbird_csr(nqb, nkb, seed=4)

    def rows():
        rp, ci = [0], []
        for qb in range(nqb):
            cols = [] if qb == 1 else sorted(rng.choice(nkb, size=int(rng.integers(1, nkb + 1)), replace=False))
            ci.extend(int(c) for c in cols)
            rp.append(len(ci))
        return rp, ci
    if kind == "random":
        rp, ci = rows()
        return np.asarray(rp, np.int32), np.asarray(ci, np.int32)
    rps, cis = [], []
    for _ in range(Hq):
        rp, ci = rows()
        rps.append([r + len(cis) for r in rp])
        cis.extend(ci)
    return np.asarray(rps, np.int32), np.asarray(cis, np.int32)


def _run(c, seed):
    rng = np.random.default_rng(seed)
    B, Hq, Hkv, Nq, Nk, D = c["B"], c["Hq"], c["Hkv"], c["Nq"], c["Nk"], c["D"]
    (qb, q), (kb, k), (vb, v), (gb, g) = (workloads.normal_bf16(s, rng) for s in
                                          ((B, Hq, Nq, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D), (B, Hq, Nq, D)))
    kw = dict(causal=c.get("causal", False), window=c.get("window", 0), rope_theta=c.get("rope_theta"),
              q_pos0=c.get("q_pos0", 0), k_pos0=c.get("k_pos0", 0))
    okw = dict(kw)
    if c.get("alibi"):
        sl = workloads.alibi_slopes(Hq)
        kw["alibi_slopes"] = torch.from_numpy(sl).cuda()
        okw["alibi_slopes"] = sl.astype(np.float64)
    if c.get("bias") == "full":  # one bias plane per (b, h)
        bias = rng.standard_normal((B, Hq, Nq, Nk)).astype(np.float32)
        kw["bias"] = torch.from_numpy(bias).cuda()
        okw["bias"] = bias.astype(np.float64)
    elif c.get("bias") == "rows":  # one [Nq, Nk] plane broadcast over b and h (zero strides)
        bias = rng.standard_normal((Nq, Nk)).astype(np.float32)
        kw["bias"] = torch.from_numpy(bias).cuda().expand(B, Hq, Nq, Nk)
        okw["bias"] = np.broadcast_to(bias.astype(np.float64), (B, Hq, Nq, Nk))
    if "mask" in c:
        kind, bm, bn = c["mask"]
        rp, ci = _mask(kind, bm, bn, Hq, Nq, Nk, rng)
        kw["block_mask"] = af.block_mask_from_csr(rp, ci, bm, bn, "cuda")
        okw["block_mask"] = (rp, ci, bm, bn)
    qd, kd, vd, gd = (to_dev(x, "bf16") for x in (qb, kb, vb, gb))
    out, lse = af.fwd(qd, kd, vd, return_lse=True, decode_fast_path=False, **kw)
    bkw = {key: val for key, val in kw.items() if key != "block_mask"}
    dq, dk, dv = af.bwd(qd, kd, vd, out, gd, lse, block_mask=kw.get("block_mask"), **bkw)
    torch.cuda.synchronize()
    ref = oracle.attention_backward(q, k, v, g, **okw)
    return (host(dq), host(dk), host(dv)), ref


def _check(name, got, ref):
    for nm, a, r in zip(("dq", "dk", "dv"), got, ref):
        assert np.all(np.isfinite(a)), f"{name} {nm}: non-finite"
        err = np.abs(a - r)
        # relative to the gradient's largest magnitude, with a floor for gradients
        # that vanish exactly (one visible key: dS = P (dP - delta) = 0)
        scale = max(float(np.abs(r).max()), 1e-2)
        where = np.unravel_index(int(err.argmax()), err.shape)
        log(f"{name} {nm}: max {err.max():.3e} mean {err.mean():.3e} (max|ref| {scale:.3e}) at {where}")
        assert err.max() <= 2e-2 * scale, (name, nm, float(err.max()), scale)
        assert err.mean() <= 2e-3 * scale, (name, nm, float(err.mean()), scale)


@pytest.mark.parametrize("name", sorted(CASES))
def test_backward_matches_oracle(name):
    log(f"case bwd {name}")
    got, ref = _run(CASES[name], seed=hash(name) % 1000)
    _check(name, got, ref)


def test_backward_rows_without_keys_get_zero_dq():
    # causal with the keys placed after the queries: rows 0..2 see no key
    c = dict(B=1, Hq=2, Hkv=1, Nq=70, Nk=70, D=64, causal=True, q_pos0=0, k_pos0=3)
    log("case bwd rows without keys")
    got, ref = _run(c, seed=3)
    assert np.all(got[0][:, :, :3] == 0.0)
    _check("rows_without_keys", got, ref)


def test_backward_full_size_bench_config():
    """Llama-3-8B shape (B=1, Hq=32, Hkv=8, N=4096, D=128, RoPE theta=5e5,
    causal) in the launch configuration the benchmark times (workspace from
    bwd_workspace_size, so the split key blocks and their reduction run):
    full gradients of two kv-head groups (q-heads 0-3 / kv-head 0 and
    q-heads 28-31 / kv-head 7) against the oracle."""
    w = workloads.WORKLOADS["llama3_8b_rope_causal_n4096"]
    inp = workloads.make_inputs(w)
    log("case bwd full size llama3_8b_rope_causal_n4096")
    q, k, v = (to_dev(x, "bf16") for x in (inp.q_dev, inp.k_dev, inp.v_dev))
    rng = np.random.default_rng(3)
    dout = torch.from_numpy(rng.standard_normal(q.shape, dtype=np.float32)).cuda().to(torch.bfloat16)
    kw = dict(causal=w.causal, window=w.window, rope_theta=w.rope_theta)
    out, lse = af.fwd(q, k, v, return_lse=True, **kw)
    ws = torch.empty(af.bwd_workspace_size(q, k, v, **kw) // 4 + 4, dtype=torch.float32, device="cuda")
    dq, dk, dv = af.bwd(q, k, v, out, dout, lse, workspace=ws, **kw)
    torch.cuda.synchronize()
    qh, kh, vh, gh = host(q), host(k), host(v), host(dout)
    G = w.Hq // w.Hkv
    for kvh in (0, w.Hkv - 1):
        hs = slice(kvh * G, (kvh + 1) * G)
        ref = oracle.attention_backward(qh[:, hs], kh[:, kvh:kvh + 1], vh[:, kvh:kvh + 1], gh[:, hs],
                                        rope_theta=w.rope_theta, causal=True)
        got = (host(dq[:, hs]), host(dk[:, kvh:kvh + 1]), host(dv[:, kvh:kvh + 1]))
        _check(f"full_size_kvh{kvh}", got, ref)


@pytest.mark.parametrize("Nq,Nk", [(0, 50), (40, 0), (1, 1), (65, 3)], ids=["no_queries", "no_keys", "one_one", "few_keys"])
def test_backward_degenerate_shapes(Nq, Nk):
    """Empty query or key sets and tiny ones: gradients of an empty side are
    empty, those of the other side are zero; tiny shapes match the oracle."""
    rng = np.random.default_rng(Nq * 100 + Nk)
    B, Hq, Hkv, D = 1, 4, 2, 64
    (qb, q), (kb, k), (vb, v), (gb, g) = (workloads.normal_bf16(s, rng) for s in
                                          ((B, Hq, Nq, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D), (B, Hq, Nq, D)))
    kw = dict(causal=True, rope_theta=1e4, q_pos0=max(Nk - Nq, 0))
    log(f"case bwd degenerate Nq={Nq} Nk={Nk}")
    qd, kd, vd, gd = (to_dev(x, "bf16") for x in (qb, kb, vb, gb))
    out, lse = af.fwd(qd, kd, vd, return_lse=True, decode_fast_path=False, **kw)
    dq, dk, dv = af.bwd(qd, kd, vd, out, gd, lse, **kw)
    torch.cuda.synchronize()
    assert dq.shape == qd.shape and dk.shape == kd.shape and dv.shape == vd.shape
    if Nq == 0:
        assert float(host(dk).__abs__().sum() if dk.numel() else 0.0) == 0.0 and float(np.abs(host(dv)).sum()) == 0.0
    elif Nk == 0:
        assert float(np.abs(host(dq)).sum()) == 0.0
    else:
        ref = oracle.attention_backward(q, k, v, g, **kw)
        _check(f"degenerate {Nq}x{Nk}", (host(dq), host(dk), host(dv)), ref)

"""GPU parity of the second workload grid (GPT-2-small geometry, B=4 H=12
D=64, the variants of the pages' "6.1 Forward Head-to-Head on Ampere" and
"6.2 RoPE on Ampere" tables) and of every tile choice of the bf16 prefill
kernel ("3.2 From DSL to Kernel", the Tile pass), against the fp64 oracle."""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import oracle
import workloads
from gpu_helpers import check_close, check_lse, dev_inputs, host, log

pytestmark = pytest.mark.gpu


def _kw(w, inp, gpu):
    kw = dict(rope_theta=w.rope_theta, causal=w.causal, window=w.window)
    if w.alibi:
        kw["alibi_slopes"] = (torch.from_numpy(inp.alibi_slopes).cuda() if gpu
                              else inp.alibi_slopes.astype(np.float64))
    return kw


@pytest.mark.parametrize("variant", sorted(workloads.GPT2_VARIANTS))
def test_gpt2_small_grid_n512_elementwise(variant):
    w = workloads.gpt2_small(variant, 512)
    inp = workloads.make_inputs(w)
    log(f"case {w.name} (library tiles)")
    q, k, v = dev_inputs(inp)
    out, lse = af.fwd(q, k, v, return_lse=True, **_kw(w, inp, True))
    ref, rlse = oracle.attention(inp.q, inp.k, inp.v, **_kw(w, inp, False))
    check_close(host(out), ref, "bf16", w.name)
    check_lse(host(lse), rlse, 2e-2, w.name)


@pytest.mark.parametrize("variant", ["rope_causal", "causal_alibi", "rope_sw256"])
def test_gpt2_small_grid_n4096_sampled_rows(variant):
    w = workloads.gpt2_small(variant, 4096)
    inp = workloads.make_inputs(w)
    log(f"case {w.name} sampled rows")
    q, k, v = dev_inputs(inp)
    out = host(af.fwd(q, k, v, **_kw(w, inp, True)))
    rng = np.random.default_rng(7)
    rows = sorted(set([0, 1, 63, 64, 255, 256, 257, 2047, 4095]) | set(int(x) for x in rng.integers(0, 4096, 10)))
    heads = [(0, 0), (3, 11), (1, 6)]
    ref, _ = oracle.attention(inp.q, inp.k, inp.v, rows=rows, heads=heads, **_kw(w, inp, False))
    for b, h in heads:
        check_close(out[b, h, rows], ref[b, h], "bf16", f"{w.name} b{b} h{h}")


TILES_GQA = [(8, 1), (8, 2), (8, 4), (4, 1), (4, 2), (4, 4), (2, 1), (2, 2)]


@pytest.mark.parametrize("tile", TILES_GQA, ids=[f"{t[0]}w{t[1]}h" for t in TILES_GQA])
def test_every_tile_choice_gqa_rope_causal(tile):
    w = workloads.WORKLOADS["llama3_8b_rope_causal_n4096"].with_(Nq=300, Nk=300, Hq=8, Hkv=2)
    inp = workloads.make_inputs(w)
    log(f"case tile {tile} on {w}")
    q, k, v = dev_inputs(inp)
    out, lse = af.fwd(q, k, v, return_lse=True, tile=tile, **_kw(w, inp, True))
    ref, rlse = oracle.attention(inp.q, inp.k, inp.v, **_kw(w, inp, False))
    check_close(host(out), ref, "bf16", f"tile {tile}")
    check_lse(host(lse), rlse, 2e-2, f"tile {tile}")


@pytest.mark.parametrize("tile", [(2, 1), (4, 1), (8, 1)], ids=["2w", "4w", "8w"])
@pytest.mark.parametrize("variant", ["rope_sw256", "causal_alibi"])
def test_every_tile_choice_gpt2(variant, tile):
    w = workloads.gpt2_small(variant, 512).with_(B=1, Hq=3, Hkv=3, Nq=600, Nk=600)
    inp = workloads.make_inputs(w)
    log(f"case tile {tile} on {w.name} (B1 H3 N600)")
    q, k, v = dev_inputs(inp)
    out = host(af.fwd(q, k, v, tile=tile, **_kw(w, inp, True)))
    ref, _ = oracle.attention(inp.q, inp.k, inp.v, **_kw(w, inp, False))
    check_close(out, ref, "bf16", f"{w.name} tile {tile}")


def test_unsupported_tile_choice_raises():
    w = workloads.gpt2_small("dense", 512).with_(B=1, Hq=2, Hkv=2, Nq=64, Nk=64)
    inp = workloads.make_inputs(w)
    q, k, v = dev_inputs(inp)
    with pytest.raises(af.AttnfuseError):
        af.fwd(q, k, v, tile=(8, 2))  # G = 1: two heads per workgroup do not divide it

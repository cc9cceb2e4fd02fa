"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Small shapes and the full-size workloads (in the launch configuration the
benchmark times) are compared element by element, plus properties that hold
at any size.
"""
import numpy as np
import pytest
import torch

import attention_attnfuse_fwd_amd as af
import oracle
import workloads
from gpu_helpers import check_close, check_lse, dev_inputs, host, log, oracle_all_heads, to_dev

pytestmark = pytest.mark.gpu

W = workloads.WORKLOADS


def _oracle_kw(w: workloads.Workload, inp: workloads.Inputs):
    kw = dict(rope_theta=w.rope_theta, causal=w.causal, window=w.window, q_pos0=w.q_pos0,
              k_pos0=w.k_pos0)
    if inp.alibi_slopes is not None:
        kw["alibi_slopes"] = inp.alibi_slopes.astype(np.float64)
    if inp.bs_row_ptr is not None:
        kw["block_mask"] = (inp.bs_row_ptr, inp.bs_col_idx, w.bigbird_block, w.bigbird_block)
    if inp.bias is not None:
        kw["bias"] = np.broadcast_to(inp.bias.astype(np.float64), (w.B, w.Hq, w.Nq, w.Nk))
    return kw


def _gpu_kw(w: workloads.Workload, inp: workloads.Inputs):
    kw = dict(rope_theta=w.rope_theta, causal=w.causal, window=w.window, q_pos0=w.q_pos0,
              k_pos0=w.k_pos0)
    if inp.alibi_slopes is not None:
        kw["alibi_slopes"] = torch.from_numpy(inp.alibi_slopes).cuda()
    if inp.bs_row_ptr is not None:
        kw["block_mask"] = af.block_mask_from_csr(inp.bs_row_ptr, inp.bs_col_idx, w.bigbird_block,
                                                  w.bigbird_block, "cuda")
    if inp.bias is not None:
        kw["bias"] = torch.from_numpy(inp.bias).cuda().expand(w.B, w.Hq, w.Nq, w.Nk)
    return kw


def _run(w, inp, **extra):
    q, k, v = dev_inputs(inp)
    kw = _gpu_kw(w, inp)
    kw.update(extra)
    out, lse = af.fwd(q, k, v, return_lse=True, **kw)
    torch.cuda.synchronize()
    return host(out), host(lse)


# ----------------------------------------------------------------------------
# Element-by-element parity at oracle-sized shapes (several tiles + ragged tails)
# ----------------------------------------------------------------------------

def test_fp32_rope_causal_full_config():
    w = W["rope_causal_fp32_n256"]
    inp = workloads.make_inputs(w)
    log(f"case {w.name} seed {w.seed}")
    out, lse = _run(w, inp)
    ref, rlse = oracle.attention(inp.q, inp.k, inp.v, **_oracle_kw(w, inp))
    check_close(out, ref, "fp32", w.name)
    check_lse(lse, rlse, 1e-4, w.name)


SMALL = [
    # (name, base workload, overrides)
    ("llama8b_rope_causal_ragged", "llama3_8b_rope_causal_n4096", dict(Nq=300, Nk=300)),
    ("llama8b_rope_causal_n1024", "llama3_8b_rope_causal_n4096", dict(Nq=1024, Nk=1024, B=1, Hq=8, Hkv=2)),
    ("alibi_window_small", "alibi_causal_window1024_n8192", dict(B=1, Hq=4, Hkv=4, Nq=777, Nk=777, window=100)),
    ("bigbird_small", "bigbird_rope_n4096", dict(B=1, Hq=4, Hkv=4, Nq=1024, Nk=1024)),
    ("bigbird_ragged", "bigbird_rope_n4096", dict(B=1, Hq=2, Hkv=2, Nq=1000, Nk=1000)),
    # the shallow two-slot schedule at its smallest: one ragged query block and
    # two key blocks; and more keys than queries (a ragged last key tile)
    ("bigbird_tiny_ragged", "bigbird_rope_n4096", dict(B=1, Hq=2, Hkv=2, Nq=50, Nk=70)),
    ("bigbird_keys_past_queries", "bigbird_rope_n4096", dict(B=2, Hq=3, Hkv=3, Nq=333, Nk=777)),
]


@pytest.mark.parametrize("name,base,over", SMALL, ids=[s[0] for s in SMALL])
def test_small_shapes_elementwise(name, base, over):
    w = W[base].with_(**over)
    inp = workloads.make_inputs(w)
    log(f"case {name}: {w}")
    out, lse = _run(w, inp)
    ref, rlse = oracle.attention(inp.q, inp.k, inp.v, **_oracle_kw(w, inp))
    check_close(out, ref, w.dtype, name)
    check_lse(lse, rlse, 2e-2, name)


VARIANTS = [
    dict(),
    dict(causal=True),
    dict(window=37),
    dict(causal=True, window=1),
    dict(causal=True, window=65),
    dict(rope_theta=1e4, causal=True, q_pos0=1000, k_pos0=1000),
    dict(rope_theta=1e4, q_pos0=64, k_pos0=0),
    dict(rope_theta=1e4, causal=True, q_pos0=200, k_pos0=0),   # queries after the keys
]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("vi", range(len(VARIANTS)))
def test_variant_grid(D, dtype, vi):
    kw = VARIANTS[vi]
    rng = np.random.default_rng(100 + vi + D)
    B, Hq, Hkv, Nq, Nk = 2, 4, 2, 150, 200
    shape_q, shape_k = (B, Hq, Nq, D), (B, Hkv, Nk, D)
    if dtype == "bf16":
        (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in (shape_q, shape_k, shape_k))
    else:
        q, k, v = (rng.standard_normal(s).astype(np.float32) for s in (shape_q, shape_k, shape_k))
        qb, kb, vb = q, k, v
        q, k, v = (x.astype(np.float64) for x in (q, k, v))
    log(f"case variant {kw} D={D} {dtype}")
    out, lse = af.fwd(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), return_lse=True,
                      decode_fast_path=False, **kw)
    ref, rlse = oracle.attention(q, k, v, **kw)
    check_close(host(out), ref, dtype, f"variant {kw}")
    check_lse(host(lse), rlse, 2e-2 if dtype == "bf16" else 1e-4, f"variant {kw}")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_alibi_and_additive_bias(dtype):
    rng = np.random.default_rng(7)
    B, Hq, Hkv, N, D = 2, 4, 4, 130, 64
    if dtype == "bf16":
        (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16((B, h, N, D), rng) for h in (Hq, Hkv, Hkv))
    else:
        q, k, v = (rng.standard_normal((B, h, N, D)).astype(np.float32) for h in (Hq, Hkv, Hkv))
        qb, kb, vb = q, k, v
        q, k, v = (x.astype(np.float64) for x in (q, k, v))
    slopes = workloads.alibi_slopes(Hq)
    bias = rng.standard_normal((1, Hq, N, N)).astype(np.float32)  # broadcast over batch
    for kw_dev, kw_ref in [
        (dict(alibi_slopes=torch.from_numpy(slopes).cuda(), causal=True),
         dict(alibi_slopes=slopes.astype(np.float64), causal=True)),
        (dict(bias=torch.from_numpy(bias).cuda()), dict(bias=bias.astype(np.float64))),
        (dict(bias=torch.from_numpy(bias).cuda(), alibi_slopes=torch.from_numpy(slopes).cuda(),
              rope_theta=1e4, window=50),
         dict(bias=bias.astype(np.float64), alibi_slopes=slopes.astype(np.float64),
              rope_theta=1e4, window=50)),
    ]:
        log(f"case bias/alibi {dtype} {sorted(kw_ref)}")
        out, lse = af.fwd(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), return_lse=True,
                          **kw_dev)
        ref, rlse = oracle.attention(q, k, v, **kw_ref)
        check_close(host(out), ref, dtype, f"bias {sorted(kw_ref)}")
        check_lse(host(lse), rlse, 2e-2 if dtype == "bf16" else 1e-4, "bias")


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_block_sparse_per_head_with_empty_rows(dtype):
    rng = np.random.default_rng(8)
    B, H, N, D, bs = 1, 4, 320, 64, 64
    if dtype == "bf16":
        (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16((B, H, N, D), rng) for _ in range(3))
    else:
        q, k, v = (rng.standard_normal((B, H, N, D)).astype(np.float32) for _ in range(3))
        qb, kb, vb = q, k, v
        q, k, v = (x.astype(np.float64) for x in (q, k, v))
    nb = N // bs
    rp, ci = workloads.random_csr(nb, nb, 0.4, seed=3, n_heads=H)
    # head 0, block row 1: make it empty by rebuilding its CSR rows
    rows = [[list(ci[rp[h, r]:rp[h, r + 1]]) for r in range(nb)] for h in range(H)]
    rows[0][1] = []
    rows[2][nb - 1] = []
    flat, rps = [], []
    for h in range(H):
        r = [len(flat)]
        for rr in rows[h]:
            flat.extend(rr)
            r.append(len(flat))
        rps.append(r)
    rp = np.asarray(rps, dtype=np.int32)
    ci = np.asarray(flat, dtype=np.int32)
    mask = af.block_mask_from_csr(rp, ci, bs, bs, "cuda")
    log(f"case block sparse per head {dtype} nnz={ci.size}")
    out, lse = af.fwd(to_dev(qb, dtype), to_dev(kb, dtype), to_dev(vb, dtype), return_lse=True,
                      block_mask=mask, rope_theta=1e4)
    ref, rlse = oracle.attention(q, k, v, rope_theta=1e4, block_mask=(rp, ci, bs, bs))
    check_close(host(out), ref, dtype, "block sparse per head")
    check_lse(host(lse), rlse, 2e-2 if dtype == "bf16" else 1e-4, "block sparse per head")
    assert np.all(host(out)[0, 0, 64:128] == 0.0)
    assert np.all(np.isneginf(host(lse)[0, 0, 64:128]))


def test_create_block_mask_predicate_matches_csr():
    nb = 6
    m = af.create_block_mask(lambda qb, kb: kb <= qb or kb == 0, nb, nb, 64, 64, "cuda")
    rp = m.row_ptr.cpu().numpy()
    ci = m.col_idx.cpu().numpy()
    for qb in range(nb):
        assert list(ci[rp[qb]:rp[qb + 1]]) == [kb for kb in range(nb) if kb <= qb or kb == 0]


# ----------------------------------------------------------------------------
# Full-size workloads: every output element against the oracle
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["llama3_8b_rope_causal_n4096", "alibi_causal_window1024_n8192",
                                  "bigbird_rope_n4096", "bias_heads_causal_n2048"])
def test_full_size_elementwise(name):
    """The prefill workloads at full size, in the launch configuration the
    benchmark times (the library's tile table), compared with the oracle on
    every (batch, head, row, d) element of the output and every lse value."""
    w = W[name]
    inp = workloads.make_inputs(w)
    log(f"case {name} full size, seed {w.seed}")
    q, k, v = dev_inputs(inp)
    log(f"plan {af.fwd_plan(q, k, v, **_gpu_kw(w, inp))}")
    del q, k, v
    out, lse = _run(w, inp)
    ref, rlse = oracle_all_heads(inp.q, inp.k, inp.v, w.B, w.Hq, **_oracle_kw(w, inp))
    check_close(out, ref, w.dtype, f"{name} (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, f"{name} (all {lse.size} rows)")
    if w.causal:
        # row 0 sees only key 0: output equals V[0] exactly (all heads)
        G = w.Hq // w.Hkv
        v0 = inp.v[:, np.arange(w.Hq) // G, 0, :]
        np.testing.assert_array_equal(out[:, :, 0, :], v0)


# Paired workgroups: causal dense launches with enough query blocks run block
# n_qblk - 1 - j and block j in one workgroup, as one stream of key tiles.
PAIRED = [
    # odd block count (15: the middle block runs alone) and a ragged last block
    ("paired_odd_ragged_rope", "llama3_8b_rope_causal_n4096", dict(B=2, Hq=64, Hkv=16, Nq=950, Nk=950)),
    # one q-head per workgroup (no GQA), 256-row blocks, d = 64, no RoPE
    ("paired_mha_d64", "llama3_8b_rope_causal_n4096",
     dict(B=4, Hq=32, Hkv=32, Nq=1024, Nk=1024, D=64, rope_theta=None)),
    # queries after the keys: every block sees 200 keys beyond its diagonal
    ("paired_queries_after_keys", "llama3_8b_rope_causal_n4096",
     dict(B=2, Hq=64, Hkv=16, Nq=1000, Nk=1200, q_pos0=200, rope_theta=1e4)),
    # causal window with RoPE: each block streams its own window's tiles; 15 blocks, ragged tail
    ("paired_rope_window", "llama3_8b_rope_causal_n4096",
     dict(B=2, Hq=64, Hkv=16, Nq=915, Nk=915, window=200)),
    # ALiBi (tiles visited from the diagonal down) + window, 15 blocks of 256 rows, ragged tail
    ("paired_alibi_window_odd_ragged", "alibi_causal_window1024_n8192",
     dict(B=2, Hq=32, Hkv=32, Nq=3600, Nk=3600, window=300)),
    # ALiBi causal, no window, queries after the keys
    ("paired_alibi_after_keys", "alibi_causal_window1024_n8192",
     dict(B=4, Hq=32, Hkv=32, Nq=1000, Nk=1100, window=0, q_pos0=100)),
]


@pytest.mark.parametrize("name,base,over", PAIRED, ids=[c[0] for c in PAIRED])
def test_paired_workgroups_elementwise(name, base, over):
    w = W[base].with_(**over)
    inp = workloads.make_inputs(w)
    log(f"case {name}: {w}")
    q, k, v = dev_inputs(inp)
    plan = af.fwd_plan(q, k, v, **_gpu_kw(w, inp))
    log(f"plan {plan}")
    assert plan["kernel"] == "bf16" and plan["paired"] == 1, plan
    out, lse = _run(w, inp)
    ref, rlse = oracle_all_heads(inp.q, inp.k, inp.v, w.B, w.Hq, **_oracle_kw(w, inp))
    check_close(out, ref, w.dtype, f"{name} (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, f"{name} (all {lse.size} rows)")


# The eight-wave kernel without RoPE skips the masks and exponentials of the
# key tiles a wave's 32 rows cannot see (a window's start, keys past a
# block's diagonal or past the end of the keys): every element against the
# oracle, the eight-wave tile forced.
DEAD_TILES = [
    # plain causal window, GQA, ragged tail
    ("dead_plain_window_gqa", "llama3_8b_rope_causal_n4096",
     dict(B=2, Hq=16, Hkv=4, Nq=915, Nk=915, window=200, rope_theta=None)),
    # queries after the keys, a window shorter than a key tile
    ("dead_plain_window_after_keys", "llama3_8b_rope_causal_n4096",
     dict(B=1, Hq=8, Hkv=2, Nq=700, Nk=900, q_pos0=200, window=50, rope_theta=None)),
    # per-head additive bias under a causal window
    ("dead_bias_window", "bias_heads_causal_n2048", dict(B=1, Hq=4, Hkv=4, Nq=600, Nk=600, window=120)),
]


@pytest.mark.parametrize("name,base,over", DEAD_TILES, ids=[c[0] for c in DEAD_TILES])
def test_eight_wave_tiles_a_wave_cannot_see(name, base, over):
    w = W[base].with_(**over)
    inp = workloads.make_inputs(w)
    log(f"case {name}: {w}")
    q, k, v = dev_inputs(inp)
    plan = af.fwd_plan(q, k, v, tile=(8, 0), **_gpu_kw(w, inp))
    log(f"plan {plan}")
    assert plan["kernel"] == "bf16" and plan["waves"] == 8, plan
    out, lse = _run(w, inp, tile=(8, 0))
    ref, rlse = oracle_all_heads(inp.q, inp.k, inp.v, w.B, w.Hq, **_oracle_kw(w, inp))
    check_close(out, ref, w.dtype, f"{name} (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, f"{name} (all {lse.size} rows)")


# Chained workgroups: block-sparse launches on two or four waves run `chain`
# consecutive query blocks of one head as one stream of key tiles (the
# full-size BigBird workload above runs the library's chains of 4).  Besides
# the oracle, the same launch with single blocks must give the same bits:
# chaining changes the grid, not the arithmetic of a block.
CHAINED = [
    # (name, base workload, overrides, tile = (waves, heads, chain))
    # 16 blocks in chains of 3 (the last holds one), ragged tail
    ("chain3_bigbird_ragged", "bigbird_rope_n4096", dict(B=1, Hq=2, Hkv=2, Nq=1000, Nk=1000), (0, 0, 3)),
    # causal band inside the chains, D = 128, ALiBi, queries after the keys
    ("chain4_causal_alibi_d128", "bigbird_rope_n4096",
     dict(B=1, Hq=4, Hkv=4, Nq=900, Nk=1000, D=128, causal=True, alibi=True, q_pos0=100), (0, 0, 4)),
    # four waves on 128-row blocks, GQA (one q-head per workgroup)
    ("chain2_four_waves_gqa", "bigbird_rope_n4096",
     dict(B=1, Hq=4, Hkv=2, Nq=1100, Nk=1100, bigbird_block=128), (4, 1, 2)),
    # window, no RoPE, two batches
    ("chain5_window_norope", "bigbird_rope_n4096",
     dict(B=2, Hq=2, Hkv=2, Nq=640, Nk=640, window=100, rope_theta=None), (0, 0, 5)),
    # the shallow two-slot schedule (D = 64, two waves) with ALiBi, causal,
    # queries after the keys, ragged tails
    ("chain2_shallow_alibi_causal", "bigbird_rope_n4096",
     dict(B=1, Hq=4, Hkv=4, Nq=700, Nk=800, causal=True, alibi=True, q_pos0=100), (0, 0, 2)),
]


@pytest.mark.parametrize("name,base,over,tile", CHAINED, ids=[c[0] for c in CHAINED])
def test_chained_workgroups_elementwise(name, base, over, tile):
    w = W[base].with_(**over)
    inp = workloads.make_inputs(w)
    log(f"case {name}: {w}, tile {tile}")
    q, k, v = dev_inputs(inp)
    plan = af.fwd_plan(q, k, v, tile=tile, **_gpu_kw(w, inp))
    log(f"plan {plan}")
    assert plan["kernel"] == "bf16" and plan["waves"] < 8, plan
    assert plan["chain"] == min(tile[2], plan["query_blocks"]) > 1, plan
    out, lse = _run(w, inp, tile=tile)
    ref, rlse = oracle_all_heads(inp.q, inp.k, inp.v, w.B, w.Hq, **_oracle_kw(w, inp))
    check_close(out, ref, w.dtype, f"{name} (all {out.size} elements)")
    check_lse(lse, rlse, 2e-2, f"{name} (all {lse.size} rows)")
    out1, lse1 = _run(w, inp, tile=(tile[0], tile[1], 1))
    np.testing.assert_array_equal(out, out1)
    np.testing.assert_array_equal(lse, lse1)


@pytest.mark.parametrize("chain", [2, 3, 6])
def test_chained_per_head_masks_with_empty_blocks(chain):
    # Per-head masks (one q-head per workgroup) with empty query blocks at the
    # start of a chain, inside it, at its end, and a head with no blocks at all.
    rng = np.random.default_rng(21)
    B, H, N, D, bs = 1, 4, 384, 64, 64
    (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16((B, H, N, D), rng) for _ in range(3))
    nb = N // bs
    rp, ci = workloads.random_csr(nb, nb, 0.5, seed=5, n_heads=H)
    rows = [[list(ci[rp[h, r]:rp[h, r + 1]]) or [r] for r in range(nb)] for h in range(H)]
    rows[0][0] = []
    rows[1][2] = rows[1][3] = []
    rows[2][nb - 1] = []
    rows[3] = [[] for _ in range(nb)]
    flat, rps = [], []
    for h in range(H):
        r = [len(flat)]
        for rr in rows[h]:
            flat.extend(rr)
            r.append(len(flat))
        rps.append(r)
    rp = np.asarray(rps, dtype=np.int32)
    ci = np.asarray(flat, dtype=np.int32)
    mask = af.block_mask_from_csr(rp, ci, bs, bs, "cuda")
    qd, kd, vd = (to_dev(x, "bf16") for x in (qb, kb, vb))
    plan = af.fwd_plan(qd, kd, vd, block_mask=mask, rope_theta=1e4, tile=(0, 0, chain))
    log(f"case chained per-head masks, chain {chain}, nnz={ci.size}, plan {plan}")
    assert plan["chain"] == chain and plan["waves"] == 2, plan
    out, lse = af.fwd(qd, kd, vd, return_lse=True, block_mask=mask, rope_theta=1e4, tile=(0, 0, chain))
    ref, rlse = oracle.attention(q, k, v, rope_theta=1e4, block_mask=(rp, ci, bs, bs))
    out, lse = host(out), host(lse)
    check_close(out, ref, "bf16", f"chained per-head masks, chain {chain}")
    check_lse(lse, rlse, 2e-2, f"chained per-head masks, chain {chain}")
    for h, r in ((0, 0), (1, 2), (1, 3), (2, nb - 1)):
        assert np.all(out[0, h, r * bs:(r + 1) * bs] == 0.0)
        assert np.all(np.isneginf(lse[0, h, r * bs:(r + 1) * bs]))
    assert np.all(out[0, 3] == 0.0) and np.all(np.isneginf(lse[0, 3]))


# ----------------------------------------------------------------------------
# Decode (split-KV + LSE combine)
# ----------------------------------------------------------------------------

def test_decode_full_config_and_split_invariance():
    w = W["llama3_70b_decode_32k"]
    inp = workloads.make_inputs(w)
    q, k, v = dev_inputs(inp)
    ref, rlse = oracle.attention(inp.q, inp.k, inp.v, **_oracle_kw(w, inp))
    outs = {}
    for splits in (64, 1, 7, 100):
        log(f"case decode 70b splits={splits}")
        out, lse = af.decode(q, k, v, num_splits=splits, rope_theta=w.rope_theta, q_pos0=w.q_pos0,
                             k_pos0=w.k_pos0, return_lse=True)
        torch.cuda.synchronize()
        outs[splits] = host(out)
        check_close(outs[splits], ref, "bf16", f"decode splits={splits}")
        check_lse(host(lse), rlse, 2e-2, f"decode splits={splits}")
    for s in (1, 7, 100):
        assert np.max(np.abs(outs[s] - outs[64])) <= 2e-2


@pytest.mark.parametrize("kw", [dict(window=1000, causal=True), dict(alibi=True),
                                dict(rope_theta=1e4, k_pos0=5)], ids=str)
def test_decode_variants_small(kw):
    rng = np.random.default_rng(5)
    B, Hq, Hkv, Nk, D = 2, 8, 2, 3000, 128
    (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                 ((B, Hq, 1, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D)))
    kw = dict(kw)
    okw = dict(q_pos0=Nk + kw.get("k_pos0", 0), k_pos0=kw.get("k_pos0", 0),
               rope_theta=kw.get("rope_theta"), causal=kw.get("causal", False),
               window=kw.get("window", 0))
    dkw = dict(okw)
    if kw.get("alibi"):
        sl = workloads.alibi_slopes(Hq)
        okw["alibi_slopes"] = sl.astype(np.float64)
        dkw["alibi_slopes"] = torch.from_numpy(sl).cuda()
    log(f"case decode variant {kw}")
    out = af.decode(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), num_splits=13, **dkw)
    ref, _ = oracle.attention(q, k, v, **okw)
    check_close(host(out), ref, "bf16", f"decode {kw}")


def test_decode_shared_workspace_and_head_groups():
    """One workspace, filled with garbage first, reused by calls of different
    shapes and split counts; GQA groups wider than 32 q-heads (two head
    groups per kv-head, the second one partial) and D = 64.  Every call must
    match the oracle."""
    rng = np.random.default_rng(11)
    cases = [  # B, Hq, Hkv, Nk, D, splits
        (2, 40, 1, 2000, 128, 64),
        (1, 16, 2, 777, 64, 7),
        (2, 40, 1, 2000, 128, 100),
        (1, 48, 1, 300, 64, 33),
        (1, 16, 2, 777, 64, 7),
    ]
    need = max(B * Hq * sp * (D + 2) * 4 for B, Hq, Hkv, Nk, D, sp in cases)
    ws = torch.from_numpy(rng.integers(0, 2**31, need // 4, dtype=np.int32)).cuda().view(torch.float32)
    for B, Hq, Hkv, Nk, D, sp in cases:
        (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                     ((B, Hq, 1, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D)))
        kw = dict(rope_theta=1e4, q_pos0=Nk)
        qd, kd, vd = to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16")
        assert af.decode_workspace_size(qd, kd, sp) <= need
        log(f"case decode shared workspace B={B} Hq={Hq} Hkv={Hkv} Nk={Nk} D={D} splits={sp}")
        out, lse = af.decode(qd, kd, vd, num_splits=sp, return_lse=True, workspace=ws, **kw)
        torch.cuda.synchronize()
        ref, rlse = oracle.attention(q, k, v, **kw)
        check_close(host(out), ref, "bf16", f"decode shared ws {B, Hq, Hkv, Nk, D, sp}")
        check_lse(host(lse), rlse, 2e-2, f"decode shared ws {B, Hq, Hkv, Nk, D, sp}")


def test_fwd_single_query_uses_decode_and_matches_prefill_kernel():
    rng = np.random.default_rng(6)
    (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                 ((1, 8, 1, 128), (1, 2, 777, 128), (1, 2, 777, 128)))
    kw = dict(rope_theta=5e5, q_pos0=777)
    a = host(af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), **kw))
    b = host(af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"),
                    decode_fast_path=False, **kw))
    ref, _ = oracle.attention(q, k, v, **kw)
    check_close(a, ref, "bf16", "fwd Nq=1 (decode)")
    check_close(b, ref, "bf16", "fwd Nq=1 (prefill kernel)")


# ----------------------------------------------------------------------------
# Edge cases and properties
# ----------------------------------------------------------------------------

def test_empty_keys_give_zero_rows():
    q = torch.randn(1, 2, 40, 128, device="cuda").bfloat16()
    k = torch.randn(1, 2, 0, 128, device="cuda").bfloat16()
    out, lse = af.fwd(q, k, k, return_lse=True)
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


def test_window_one_is_identity_exactly():
    rng = np.random.default_rng(9)
    (qb, _), (kb, _), (vb, v) = (workloads.normal_bf16((1, 4, 257, 128), rng) for _ in range(3))
    out = af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), causal=True, window=1,
                 rope_theta=1e4)
    np.testing.assert_array_equal(host(out), v)


def test_rope_shift_invariance_on_gpu():
    rng = np.random.default_rng(10)
    (qb, _), (kb, _), (vb, _) = (workloads.normal_bf16((1, 4, 200, 128), rng) for _ in range(3))
    a = host(af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), causal=True, rope_theta=1e4))
    b = host(af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), causal=True, rope_theta=1e4,
                    q_pos0=1000, k_pos0=1000))
    assert np.max(np.abs(a - b)) <= 2e-2 and np.mean(np.abs(a - b)) <= 2e-3


def test_deterministic_bitwise():
    w = W["llama3_8b_rope_causal_n4096"].with_(Nq=512, Nk=512)
    inp = workloads.make_inputs(w)
    a, _ = _run(w, inp)
    b, _ = _run(w, inp)
    np.testing.assert_array_equal(a, b)


def test_rope_table_matches_fp64():
    D, L, theta = 128, 40000, 5e5
    cos, sin, cs16 = af.rope_tables(theta, D, L, "cuda")
    torch.cuda.synchronize()
    pos = np.array([0, 1, 4095, 32768, 39999])
    r = np.arange(D // 2)
    ang = pos[:, None] * np.power(theta, -2.0 * r / D)[None, :]
    np.testing.assert_allclose(cos.cpu().numpy()[pos], np.cos(ang), rtol=0, atol=1.2e-7)
    np.testing.assert_allclose(sin.cpu().numpy()[pos], np.sin(ang), rtol=0, atol=1.2e-7)
    # fp16 pairs: cos in the low half, sin in the high half, each within half an fp16 ulp
    h = cs16.cpu().numpy()[pos].view(np.uint32)
    c16 = (h & 0xFFFF).astype(np.uint16).view(np.float16).astype(np.float64)
    s16 = (h >> 16).astype(np.uint16).view(np.float16).astype(np.float64)
    np.testing.assert_allclose(c16, np.cos(ang), rtol=0, atol=2.5e-4)
    np.testing.assert_allclose(s16, np.sin(ang), rtol=0, atol=2.5e-4)
    assert np.max(np.abs(c16 - np.cos(ang))) > 0  # really fp16-rounded
    # bf16 pairs (written on request only): the fp32 values rounded to nearest
    # even bf16, bit for bit
    import ctypes
    csb16 = torch.empty((L, D // 2), dtype=torch.int32, device="cuda")
    st = af.load_library().attnfuse_rope_table(theta, D, L, None, None, None,
                                               ctypes.c_void_p(csb16.data_ptr()), None)
    assert st == 0
    torch.cuda.synchronize()
    hb = csb16.cpu().numpy()[pos].view(np.uint32)

    def bf16_rne(x):
        u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
        return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint32)
    np.testing.assert_array_equal(hb & 0xFFFF, bf16_rne(cos.cpu().numpy()[pos]))
    np.testing.assert_array_equal(hb >> 16, bf16_rne(sin.cpu().numpy()[pos]))


def test_prerotated_path_matches_oracle():
    w = W["llama3_8b_rope_causal_n4096"].with_(Nq=640, Nk=640)
    inp = workloads.make_inputs(w)
    q, k, v = dev_inputs(inp)
    qr = af.prerotate(q, rope_theta=w.rope_theta)
    kr = af.prerotate(k, rope_theta=w.rope_theta)
    out = host(af.fwd(qr, kr, v, causal=True))
    fused = host(af.fwd(q, k, v, causal=True, rope_theta=w.rope_theta))
    ref, _ = oracle.attention(inp.q, inp.k, inp.v, rope_theta=w.rope_theta, causal=True)
    check_close(out, ref, "bf16", "pre-rotated path")
    check_close(fused, ref, "bf16", "fused path")
    # both paths round Q' and K' to bf16 the same way: they agree closely
    assert np.max(np.abs(out - fused)) <= 2e-2


def test_gqa_matches_repeated_heads():
    rng = np.random.default_rng(12)
    (qb, _), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                 ((1, 8, 130, 128), (1, 2, 130, 128), (1, 2, 130, 128)))
    kr = np.repeat(kb.reshape(1, 2, 130, 128), 4, axis=1)
    vr = np.repeat(vb.reshape(1, 2, 130, 128), 4, axis=1)
    a = host(af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), causal=True, rope_theta=1e4))
    b = host(af.fwd(to_dev(qb, "bf16"), to_dev(kr, "bf16"), to_dev(vr, "bf16"), causal=True, rope_theta=1e4))
    assert np.max(np.abs(a - b)) <= 2e-2


# ----------------------------------------------------------------------------
# Decode from an FP8 E4M3 KV cache (per-tensor scales)
# ----------------------------------------------------------------------------

def _fp8_cache(shape, rng, scale_to=448.0):
    """float32 N(0,1) draws quantised to E4M3 with a per-tensor scale:
    (codes uint8, dequantised float64 values, scale)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    scale = float(np.abs(x).max()) / scale_to
    codes = workloads.round_to_e4m3(x / scale)
    return codes, workloads.e4m3_to_f64(codes) * scale, scale


def _fp8_dev(codes, as_uint8=False):
    t = torch.from_numpy(codes).cuda()
    return t if as_uint8 else t.view(torch.float8_e4m3fn)


@pytest.mark.parametrize("case", [
    dict(B=2, Hq=8, Hkv=2, Nk=3000, D=128, rope_theta=1e4, splits=13),
    dict(B=1, Hq=40, Hkv=1, Nk=2000, D=128, splits=64, alibi=True, window=700, causal=True),
    dict(B=2, Hq=16, Hkv=2, Nk=777, D=64, rope_theta=5e5, splits=7, k_pos0=9, uint8=True),
], ids=["rope_gqa_d128", "alibi_window_gqa40", "rope_offset_d64_uint8"])
def test_decode_fp8_cache_small(case):
    c = dict(case)
    rng = np.random.default_rng(21)
    B, Hq, Hkv, Nk, D = c["B"], c["Hq"], c["Hkv"], c["Nk"], c["D"]
    qb, q = workloads.normal_bf16((B, Hq, 1, D), rng)
    kc, k, ks = _fp8_cache((B, Hkv, Nk, D), rng)
    vc, v, vs = _fp8_cache((B, Hkv, Nk, D), rng)
    k0 = c.get("k_pos0", 0)
    okw = dict(q_pos0=Nk + k0, k_pos0=k0, rope_theta=c.get("rope_theta"), causal=c.get("causal", False),
               window=c.get("window", 0))
    dkw = dict(okw)
    if c.get("alibi"):
        sl = workloads.alibi_slopes(Hq)
        okw["alibi_slopes"] = sl.astype(np.float64)
        dkw["alibi_slopes"] = torch.from_numpy(sl).cuda()
    log(f"case decode fp8 {case}")
    out, lse = af.decode(to_dev(qb, "bf16"), _fp8_dev(kc, c.get("uint8")), _fp8_dev(vc, c.get("uint8")),
                         num_splits=c["splits"], k_scale=ks, v_scale=vs, return_lse=True, **dkw)
    ref, rlse = oracle.attention(q, k, v, **okw)
    check_close(host(out), ref, "bf16", f"decode fp8 {case}")
    check_lse(host(lse), rlse, 2e-2, f"decode fp8 {case}")


def test_decode_fp8_cache_full_config():
    """Llama-3-70B decode geometry (B=1, Hq=64, Hkv=8, D=128, 32768 cached keys,
    RoPE theta=5e5, 64 splits) with the cache in E4M3: every head against the
    oracle on the dequantised values."""
    w = W["llama3_70b_decode_32k"]
    rng = np.random.default_rng(w.seed)
    qb, q = workloads.normal_bf16((w.B, w.Hq, 1, w.D), rng)
    kc, k, ks = _fp8_cache((w.B, w.Hkv, w.Nk, w.D), rng)
    vc, v, vs = _fp8_cache((w.B, w.Hkv, w.Nk, w.D), rng)
    log("case decode fp8 70b full size")
    out = af.decode(to_dev(qb, "bf16"), _fp8_dev(kc), _fp8_dev(vc), num_splits=w.decode_splits,
                    rope_theta=w.rope_theta, q_pos0=w.q_pos0, k_scale=ks, v_scale=vs)
    ref, _ = oracle.attention(q, k, v, rope_theta=w.rope_theta, q_pos0=w.q_pos0)
    check_close(host(out), ref, "bf16", "decode fp8 70b")


def test_fp8_cache_is_rejected_outside_decode():
    rng = np.random.default_rng(3)
    kc, _, _ = _fp8_cache((1, 2, 64, 64), rng)
    d = af.VariantDesc.new()
    d.dtype, d.B, d.Hq, d.Hkv, d.Nq, d.Nk, d.D = 0, 1, 2, 2, 64, 64, 64
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = 2 * 64 * 64, 64 * 64, 64
    d.kv_fp8, d.k_scale, d.v_scale = 1, 1.0, 1.0
    lib = af.load_library()
    kd = _fp8_dev(kc)
    q = torch.zeros(1, 2, 64, 64, dtype=torch.bfloat16, device="cuda")
    import ctypes
    st = lib.attnfuse_fwd(ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kd.data_ptr()),
                          ctypes.c_void_p(kd.data_ptr()), ctypes.c_void_p(q.data_ptr()), ctypes.byref(d), None)
    assert st == -2  # ATTNFUSE_ERR_UNSUPPORTED


@pytest.mark.parametrize("Nk,splits", [(1, 1), (31, 4), (33, 64), (100, 7)])
def test_decode_fp8_cache_short(Nk, splits):
    """Short fp8 caches: fewer keys than one 32-key step, more splits than keys."""
    rng = np.random.default_rng(Nk)
    B, Hq, Hkv, D = 1, 8, 2, 128
    qb, q = workloads.normal_bf16((B, Hq, 1, D), rng)
    kc, k, ks = _fp8_cache((B, Hkv, Nk, D), rng)
    vc, v, vs = _fp8_cache((B, Hkv, Nk, D), rng)
    log(f"case decode fp8 short Nk={Nk} splits={splits}")
    out = af.decode(to_dev(qb, "bf16"), _fp8_dev(kc), _fp8_dev(vc), num_splits=splits, rope_theta=1e4,
                    q_pos0=Nk, k_scale=ks, v_scale=vs)
    ref, _ = oracle.attention(q, k, v, rope_theta=1e4, q_pos0=Nk)
    check_close(host(out), ref, "bf16", f"decode fp8 Nk={Nk}")


BIAS_LAYOUTS = {
    # name: (B, Hq, Hkv, Nq, Nk, D, layout, extra variant keywords)
    "aligned_gqa_causal_d128": (2, 4, 2, 300, 332, 128, "full", dict(causal=True)),
    "ragged_keys_d128": (1, 2, 2, 200, 330, 128, "full", dict()),
    "broadcast_rows_window_rope_d64": (2, 4, 4, 260, 260, 64, "rows",
                                       dict(window=90, causal=True, rope_theta=1e4)),
    "key_major_view_d128": (1, 2, 1, 180, 200, 128, "transposed", dict(alibi=True)),
    "misaligned_rows_d64": (1, 2, 2, 140, 192, 64, "offset", dict(causal=True)),
}


@pytest.mark.parametrize("name", sorted(BIAS_LAYOUTS))
def test_additive_bias_layouts_eight_wave_tiles(name):
    """The 8-wave prefill tile reads the bias of a key tile one step ahead as
    16-byte runs when the key stride is 1, Nk is a multiple of 4 and every row
    is 16-byte aligned, else element by element: both routes, with broadcast
    (zero) strides, a key-major view and rows shifted by one element."""
    B, Hq, Hkv, Nq, Nk, D, layout, extra = BIAS_LAYOUTS[name]
    rng = np.random.default_rng(len(name))
    (qb, q), (kb, k), (vb, v) = (workloads.normal_bf16(s, rng) for s in
                                 ((B, Hq, Nq, D), (B, Hkv, Nk, D), (B, Hkv, Nk, D)))
    if layout == "full":
        host_bias = rng.standard_normal((B, Hq, Nq, Nk)).astype(np.float32)
        dev_bias = torch.from_numpy(host_bias).cuda()
    elif layout == "rows":  # one plane for every (b, h)
        plane = rng.standard_normal((Nq, Nk)).astype(np.float32)
        host_bias = np.broadcast_to(plane, (B, Hq, Nq, Nk))
        dev_bias = torch.from_numpy(plane).cuda().expand(B, Hq, Nq, Nk)
    elif layout == "transposed":  # stored [B, Hq, Nk, Nq]: unit stride along queries
        stored = rng.standard_normal((B, Hq, Nk, Nq)).astype(np.float32)
        host_bias = np.swapaxes(stored, 2, 3)
        dev_bias = torch.from_numpy(stored).cuda().transpose(2, 3)
    else:  # rows of Nk + 1 floats, starting one element in
        stored = rng.standard_normal((B, Hq, Nq, Nk + 1)).astype(np.float32)
        host_bias = stored[..., 1:]
        dev_bias = torch.from_numpy(stored).cuda()[..., 1:]
    kw = {key: val for key, val in extra.items() if key != "alibi"}
    okw = dict(kw)
    if extra.get("alibi"):
        sl = workloads.alibi_slopes(Hq)
        kw["alibi_slopes"] = torch.from_numpy(sl).cuda()
        okw["alibi_slopes"] = sl.astype(np.float64)
    log(f"case bias layout {name} tile (8, 1)")
    out, lse = af.fwd(to_dev(qb, "bf16"), to_dev(kb, "bf16"), to_dev(vb, "bf16"), bias=dev_bias,
                      return_lse=True, tile=(8, 1), **kw)
    torch.cuda.synchronize()
    ref, rlse = oracle.attention(q, k, v, bias=host_bias.astype(np.float64), **okw)
    check_close(host(out), ref, "bf16", f"bias layout {name}")
    check_lse(host(lse), rlse, 2e-2, f"bias layout {name}")

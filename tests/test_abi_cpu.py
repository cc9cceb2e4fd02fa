"""C-ABI checks that need no GPU: exports, struct layout, host-side validation.

Every call here returns from argument validation before any HIP call or
launch (validation is pure host code), so nothing touches a device.
"""
import ctypes
import os
import re
import subprocess

import pytest

from attention_attnfuse_fwd_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attnfuse.h")
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))
FAKE = ctypes.c_void_p(0x100000)  # aligned, never dereferenced (validation fails first)


@pytest.fixture(scope="module")
def lib():
    return _abi.load()


def _declared_functions():
    names = set()
    for path in HEADERS:
        src = open(path).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        names |= set(re.findall(r"\b(attnfuse_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_header_declares_exactly_the_binding_exports():
    assert _declared_functions() == sorted(_abi.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    res = subprocess.run(["nm", "-D", "--defined-only", _abi.LIB_PATH], capture_output=True,
                         text=True, check=True)
    exported = set(re.findall(r"\bT (attnfuse_\w+)", res.stdout))
    for name in _declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in _abi.VariantDesc._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){",
            'printf("size %zu\\n", sizeof(attnfuse_variant_desc));']
    for f in fields:
        prog.append(f'printf("{f} %zu\\n", offsetof(attnfuse_variant_desc, {f}));')
    prog.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", str(c), "-o", str(exe)], check=True)
    out = dict(line.split() for line in subprocess.run([str(exe)], capture_output=True, text=True,
                                                       check=True).stdout.splitlines())
    assert int(out["size"]) == ctypes.sizeof(_abi.VariantDesc)
    for f in fields:
        assert int(out[f]) == getattr(_abi.VariantDesc, f).offset, f


def test_status_strings(lib):
    for s in (0, -1, -2, -3, -4, 7):
        assert isinstance(_abi.status_string(s), str) and _abi.status_string(s)


def _good_desc(**kw):
    d = _abi.VariantDesc.new()
    d.dtype = _abi.BF16
    d.B, d.Hq, d.Hkv, d.Nq, d.Nk, d.D = 1, 4, 2, 64, 64, 128
    for f, H, N in (("q_stride", 4, 64), ("k_stride", 2, 64), ("v_stride", 2, 64), ("o_stride", 4, 64)):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = H * N * 128, N * 128, 128
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _fwd(lib, d):
    return lib.attnfuse_fwd(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), None)


def test_fp8_cache_fields_are_validated(lib):
    # only attnfuse_decode reads an fp8 cache; bad scales are invalid everywhere
    assert _fwd(lib, _good_desc(kv_fp8=1, k_scale=1.0, v_scale=1.0)) == _abi.ERR_UNSUPPORTED
    assert _fwd(lib, _good_desc(kv_fp8=2)) == _abi.ERR_INVALID
    assert _fwd(lib, _good_desc(kv_fp8=1, k_scale=0.0, v_scale=1.0)) == _abi.ERR_INVALID
    assert _fwd(lib, _good_desc(kv_fp8=1, k_scale=1.0, v_scale=float("inf"))) == _abi.ERR_INVALID


@pytest.mark.parametrize("tile", [(3, 1), (8, 3), (2, 4), (16, 1), (4, 4)])
def test_unsupported_tile_choices_are_rejected_before_launch(lib, tile):
    # the default descriptor has G = Hq / Hkv = 2: tile_heads 4 does not divide it
    d = _good_desc(tile_waves=tile[0], tile_heads=tile[1])
    assert _fwd(lib, d) == _abi.ERR_UNSUPPORTED


def test_empty_query_is_ok_without_work(lib):
    assert _fwd(lib, _good_desc(Nq=0)) == _abi.OK


@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), _abi.ERR_INVALID),
    (dict(dtype=5), _abi.ERR_INVALID),
    (dict(norm=_abi.NORM_RELU, Nq=0), _abi.ERR_UNSUPPORTED),
    (dict(norm=9), _abi.ERR_INVALID),
    (dict(Hq=3), _abi.ERR_INVALID),
    (dict(D=96), _abi.ERR_UNSUPPORTED),
    (dict(D=63), _abi.ERR_INVALID),
    (dict(B=0), _abi.ERR_INVALID),
    (dict(Nq=-1), _abi.ERR_INVALID),
    (dict(scale=-1.0), _abi.ERR_INVALID),
    (dict(scale=float("nan")), _abi.ERR_INVALID),
    (dict(causal=2), _abi.ERR_INVALID),
    (dict(window=-3), _abi.ERR_INVALID),
    (dict(q_pos0=-1), _abi.ERR_INVALID),
    (dict(rope=1), _abi.ERR_INVALID),                        # no tables
    (dict(rope=1, rope_theta=1e4, rope_cos=0x1000, rope_sin=0x2000, rope_table_len=10),
     _abi.ERR_INVALID),                                      # table shorter than the positions
    (dict(rope=1, rope_theta=1e4, rope_cos=0x1004, rope_sin=0x2000, rope_table_len=100,
          dtype=_abi.FP32), _abi.ERR_INVALID),               # misaligned fp32 table
    (dict(rope=1, rope_theta=1e4, rope_cos=0x1000, rope_table_len=100, dtype=_abi.FP32),
     _abi.ERR_INVALID),                                      # sin table missing
    (dict(rope=1, rope_theta=1e4, rope_cos=0x1000, rope_sin=0x2000, rope_table_len=100),
     _abi.ERR_INVALID),                                      # bf16 prefill reads the packed pairs, not fp32
    (dict(rope=1, rope_theta=1e4, rope_cs_bf16=0x3000, rope_table_len=100),
     _abi.ERR_INVALID),                                      # fp16 pair table missing (bf16 one is not read)
    (dict(rope=1, rope_theta=1e4, rope_cs_f16=0x1004, rope_cs_bf16=0x3000,
          rope_table_len=100), _abi.ERR_INVALID),            # misaligned fp16 pair table
    (dict(bs_row_ptr=0x1000, bs_block_m=0, bs_block_n=64), _abi.ERR_INVALID),
    (dict(bs_row_ptr=0x1000, bs_block_m=64, bs_block_n=64, bs_nnz=3), _abi.ERR_INVALID),  # no col_idx
    (dict(bs_row_ptr=0x1000, bs_col_idx=0x2000, bs_block_m=48, bs_block_n=64, bs_nnz=3),
     _abi.ERR_UNSUPPORTED),
    (dict(bs_row_ptr=0x1000, bs_col_idx=0x2000, bs_block_m=64, bs_block_n=32, bs_nnz=3),
     _abi.ERR_UNSUPPORTED),
    (dict(bs_row_ptr=0x1000, bs_col_idx=0x2000, bs_block_m=64, bs_block_n=64, bs_nnz=3,
          bs_head_stride=1), _abi.ERR_INVALID),             # head stride shorter than a row_ptr
])
def test_fwd_rejects(lib, kw, status):
    assert _fwd(lib, _good_desc(**kw)) == status


def test_fwd_rejects_bad_strides_and_pointers(lib):
    d = _good_desc()
    d.q_stride[2] = 100  # not a multiple of 8 bf16 elements
    assert _fwd(lib, d) == _abi.ERR_UNSUPPORTED
    d = _good_desc()
    d.k_stride[1] = -8
    assert _fwd(lib, d) == _abi.ERR_INVALID
    d = _good_desc()
    assert lib.attnfuse_fwd(None, FAKE, FAKE, FAKE, ctypes.byref(d), None) == _abi.ERR_INVALID
    assert lib.attnfuse_fwd(ctypes.c_void_p(0x100002), FAKE, FAKE, FAKE, ctypes.byref(d), None) \
        == _abi.ERR_UNSUPPORTED
    assert lib.attnfuse_fwd(FAKE, FAKE, FAKE, FAKE, None, None) == _abi.ERR_INVALID


def test_decode_validation(lib):
    d = _good_desc(Nq=1)
    ws_need = lib.attnfuse_decode_workspace_size(ctypes.byref(d), 16)
    assert ws_need == 1 * 4 * 16 * (128 + 2) * 4
    assert lib.attnfuse_decode_workspace_size(ctypes.byref(d), 0) == 0
    assert lib.attnfuse_decode_workspace_size(ctypes.byref(_good_desc(D=96)), 4) == 0
    call = lambda d, s, ws, nb: lib.attnfuse_decode(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), s, ws, nb, None)
    assert call(_good_desc(Nq=2), 16, FAKE, ws_need) == _abi.ERR_INVALID
    assert call(d, 0, FAKE, ws_need) == _abi.ERR_INVALID
    assert call(d, 5000, FAKE, ws_need) == _abi.ERR_INVALID
    assert call(d, 16, FAKE, ws_need - 4) == _abi.ERR_WORKSPACE
    assert call(d, 16, None, ws_need) == _abi.ERR_WORKSPACE
    assert call(_good_desc(Nq=1, bias=0x1000), 16, FAKE, ws_need) == _abi.ERR_UNSUPPORTED
    assert call(_good_desc(Nq=1, dtype=_abi.FP32), 16, FAKE, 10**9) == _abi.ERR_UNSUPPORTED
    # decode reads the fp16 pair table
    assert call(_good_desc(Nq=1, rope=1, rope_theta=1e4, rope_cos=0x1000, rope_sin=0x2000,
                           rope_table_len=100), 16, FAKE, ws_need) == _abi.ERR_INVALID


def test_bwd_validation(lib):
    d = _good_desc()
    need = lib.attnfuse_bwd_workspace_size(ctypes.byref(d))
    r256 = lambda x: (x + 255) // 256 * 256
    assert need == r256(d.B * d.Hq * d.Nq * 4)
    # a causal band on a small grid splits each key block over two workgroups (fp32 partials)
    dc = _good_desc(causal=1)
    assert lib.attnfuse_bwd_workspace_size(ctypes.byref(dc)) == need + r256(2 * 2 * dc.B * dc.Hkv * dc.Nk * dc.D * 4)
    call = lambda d, ws, nb, lse=FAKE: lib.attnfuse_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, lse, FAKE, FAKE,
                                                      FAKE, ctypes.byref(d), ws, nb, None)
    assert call(d, FAKE, need - 4) == _abi.ERR_WORKSPACE
    assert call(d, None, need) == _abi.ERR_WORKSPACE
    assert call(d, FAKE, need, lse=None) == _abi.ERR_INVALID
    # block masks need 64-aligned blocks
    assert call(_good_desc(bs_row_ptr=0x1000, bs_col_idx=0x2000, bs_block_m=64, bs_block_n=32,
                           bs_nnz=1), FAKE, need) == _abi.ERR_UNSUPPORTED
    assert call(_good_desc(dtype=_abi.FP32), FAKE, 10**9) == _abi.ERR_UNSUPPORTED
    # the gradient kernels address a tile's rows by 32-bit offsets: row strides below 2^24
    for field in ("q_stride", "k_stride", "v_stride", "o_stride"):
        dw = _good_desc()
        getattr(dw, field)[2] = 1 << 24
        assert call(dw, FAKE, need) == _abi.ERR_UNSUPPORTED, field
    # the backward reads the fp32 cos / sin tables
    assert call(_good_desc(rope=1, rope_theta=1e4, rope_cs_f16=0x1000, rope_cs_bf16=0x2000,
                           rope_table_len=10**5), FAKE, need) == _abi.ERR_INVALID
    # with RoPE the workspace also holds the rotated Q and K (bf16)
    dr = _good_desc(rope=1, rope_theta=1e4, rope_cos=0x1000, rope_sin=0x2000, rope_table_len=10**5)
    assert lib.attnfuse_bwd_workspace_size(ctypes.byref(dr)) == (
        need + r256(dr.B * dr.Hq * dr.Nq * dr.D * 2) + r256(dr.B * dr.Hkv * dr.Nk * dr.D * 2))
    assert call(dr, FAKE, need) == _abi.ERR_WORKSPACE
    assert lib.attnfuse_bwd(ctypes.c_void_p(0x100002), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                            ctypes.byref(d), FAKE, need, None) == _abi.ERR_UNSUPPORTED


def test_rope_table_and_prerotate_validation(lib):
    assert lib.attnfuse_rope_table(0.0, 64, 10, FAKE, FAKE, FAKE, FAKE, None) == _abi.ERR_INVALID
    assert lib.attnfuse_rope_table(1e4, 63, 10, FAKE, FAKE, FAKE, FAKE, None) == _abi.ERR_INVALID
    assert lib.attnfuse_rope_table(1e4, 64, 0, FAKE, FAKE, FAKE, FAKE, None) == _abi.ERR_INVALID
    assert lib.attnfuse_rope_table(1e4, 64, 10, None, None, None, None, None) == _abi.ERR_INVALID
    d = _good_desc()
    assert lib.attnfuse_prerotate(FAKE, FAKE, ctypes.byref(d), 1, None) == _abi.ERR_INVALID  # rope off
    d = _good_desc(rope=1, rope_theta=1e4, rope_cos=0x1000, rope_sin=0x2000, rope_table_len=100)
    assert lib.attnfuse_prerotate(FAKE, FAKE, ctypes.byref(d), 2, None) == _abi.ERR_INVALID
    d = _good_desc(rope=1, rope_theta=1e4, rope_cs_f16=0x1000, rope_table_len=100)
    assert lib.attnfuse_prerotate(FAKE, FAKE, ctypes.byref(d), 0, None) == _abi.ERR_INVALID


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(_abi, "_lib", None)
    monkeypatch.setattr(_abi, "LIB_PATH", str(tmp_path / "nope.so"))
    with pytest.raises(_abi.LibraryNotBuilt):
        _abi.load()


def test_product_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "attention_attnfuse_fwd_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", txt, flags=re.M), f
                assert "oracle/" not in txt, f


def test_microbench_entry_points_reject_bad_arguments(lib):
    """The machine-peak probes validate on the host and launch nothing on error."""
    P = ctypes.c_void_p
    sink, stamps = P(0x100000), P(0x200000)
    assert lib.attnfuse_mb_mfma_bf16(0, 10, sink, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16(1, 0, sink, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16(1, 10, None, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16_ops(1, 10, None, sink, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16_ops(1, 10, P(0x300008), sink, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16_ops(0, 10, P(0x300000), sink, stamps, None) == -1
    assert lib.attnfuse_mb_mfma_bf16_ops(1, 0, P(0x300000), sink, stamps, None) == -1
    assert lib.attnfuse_mb_hbm_read(P(0x100000), 15, 1, sink, stamps, None) == -1
    assert lib.attnfuse_mb_hbm_read(P(0x100008), 1024, 1, sink, stamps, None) == -1
    assert lib.attnfuse_mb_hbm_read(None, 1024, 1, sink, stamps, None) == -1
    ns = ctypes.c_double(0)
    assert lib.attnfuse_mb_host_cost(4, None, None, None, None, None, 0, None, 0, 10, ctypes.byref(ns),
                                     None) == -1
    assert lib.attnfuse_mb_host_cost(3, None, None, None, None, None, 0, None, 0, 10, ctypes.byref(ns),
                                     None) == -1
    assert lib.attnfuse_mb_host_cost(0, None, None, None, None, None, 0, None, 0, 10, ctypes.byref(ns),
                                     None) == -1
    assert lib.attnfuse_mb_host_cost(2, None, None, None, None, None, 0, None, 0, 0, ctypes.byref(ns),
                                     None) == -1


def test_decode_noalloc_rejects_oversized_partials_before_any_hip_call(lib):
    """attnfuse_decode_noalloc checks the partials size against its static
    buffer on the host: too many (batch, head, split) records -> WORKSPACE."""
    d = _abi.VariantDesc.new()
    d.dtype, d.B, d.Hq, d.Hkv, d.Nq, d.Nk, d.D = _abi.BF16, 1, 64, 8, 1, 32768, 128
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = 64 * 128, 128, 128
    splits_max = _abi.DECODE_NOALLOC_MAX_BYTES // (d.B * d.Hq * (d.D + 2) * 4)
    assert lib.attnfuse_decode_workspace_size(ctypes.byref(d), splits_max + 1) > _abi.DECODE_NOALLOC_MAX_BYTES
    assert lib.attnfuse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), splits_max + 1,
                                       None) == _abi.ERR_WORKSPACE
    assert lib.attnfuse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 0, None) == _abi.ERR_INVALID
    assert lib.attnfuse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, None, 4, None) == _abi.ERR_INVALID
    d.Hq = 7  # not a multiple of Hkv
    assert lib.attnfuse_decode_noalloc(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 4, None) == _abi.ERR_INVALID


def test_decode_noalloc_limit_matches_header():
    src = open(HEADER).read()
    assert "#define ATTNFUSE_DECODE_NOALLOC_MAX_BYTES ((size_t)8 << 20)" in src
    assert _abi.DECODE_NOALLOC_MAX_BYTES == 8 << 20


def _fp8_desc(**kw):
    """A valid all-fp8 prefill descriptor (byte strides, multiples of 16)."""
    base = dict(kv_fp8=1, q_fp8=1, q_scale=0.5, k_scale=0.25, v_scale=2.0)
    base.update(kw)
    return _good_desc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(q_fp8=0), _abi.ERR_UNSUPPORTED),                   # fp8 K / V with a bf16 Q
    (dict(kv_fp8=0, k_scale=0.0, v_scale=0.0), _abi.ERR_UNSUPPORTED),  # fp8 Q alone
    (dict(q_fp8=3), _abi.ERR_INVALID),
    (dict(q_scale=0.0), _abi.ERR_INVALID),
    (dict(q_scale=float("nan")), _abi.ERR_INVALID),
    (dict(dtype=_abi.FP32), _abi.ERR_UNSUPPORTED),
    (dict(rope=1, rope_theta=1e4, rope_cs_f16=0x1000, rope_table_len=100), _abi.ERR_UNSUPPORTED),
    (dict(bias=0x1000), _abi.ERR_UNSUPPORTED),
    (dict(tile_waves=4), _abi.ERR_UNSUPPORTED),
    (dict(tile_heads=4), _abi.ERR_UNSUPPORTED),              # does not divide G = 2
    (dict(Nq=0), _abi.OK),                                   # nothing to do, validated
])
def test_fp8_prefill_descriptor_rules(lib, kw, status):
    assert _fwd(lib, _fp8_desc(**kw)) == status


def test_fp8_prefill_byte_strides_must_be_16_aligned(lib):
    d = _fp8_desc(Nq=0)
    d.k_stride[2] = 136  # bytes: a multiple of 8 (bf16 rule) but not of 16
    assert _fwd(lib, d) == _abi.ERR_UNSUPPORTED


def test_fp8_query_is_rejected_by_the_other_entry_points(lib):
    d = _fp8_desc(Nq=1)
    assert lib.attnfuse_decode(FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), 4, FAKE, 1 << 20,
                               None) == _abi.ERR_UNSUPPORTED
    assert lib.attnfuse_bwd(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(d), FAKE,
                            1 << 20, None) == _abi.ERR_UNSUPPORTED


def _shape_desc(B, Hq, Hkv, N, D, rope=True, dtype=_abi.BF16, **kw):
    d = _abi.VariantDesc.new()
    d.dtype = dtype
    d.B, d.Hq, d.Hkv, d.Nq, d.Nk, d.D = B, Hq, Hkv, N, N, D
    for f, H in (("q_stride", Hq), ("k_stride", Hkv), ("v_stride", Hkv), ("o_stride", Hq)):
        arr = getattr(d, f)
        arr[0], arr[1], arr[2] = H * N * D, N * D, D
    if rope:
        d.rope, d.rope_theta, d.rope_table_len = 1, 5e5, 2 * N + 1
        d.rope_cs_f16 = d.rope_cos = d.rope_sin = FAKE.value
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _plan(lib, d):
    info = _abi.FwdPlanInfo()
    st = lib.attnfuse_fwd_plan(ctypes.byref(d), ctypes.byref(info))
    return st, {f: getattr(info, f) for f, _ in _abi.FwdPlanInfo._fields_}


def test_plan_struct_layout_matches_c(tmp_path):
    fields = [f for f, _ in _abi.FwdPlanInfo._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){",
            'printf("size %zu\\n", sizeof(attnfuse_fwd_plan_info));']
    prog += [f'printf("{f} %zu\\n", offsetof(attnfuse_fwd_plan_info, {f}));' for f in fields]
    prog += ['printf("kinds %d %d %d %d\\n", ATTNFUSE_PLAN_NONE, ATTNFUSE_PLAN_FP32, ATTNFUSE_PLAN_BF16,'
             ' ATTNFUSE_PLAN_FP8);', "return 0;}"]
    c = tmp_path / "plan.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "plan"
    subprocess.run(["gcc", "-std=c99", str(c), "-o", str(exe)], check=True)
    lines = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines()
    out = {ln.split()[0]: ln.split()[1:] for ln in lines}
    assert int(out["size"][0]) == ctypes.sizeof(_abi.FwdPlanInfo)
    for f in fields:
        assert int(out[f][0]) == getattr(_abi.FwdPlanInfo, f).offset, f
    assert {int(x): _abi.PLAN_KERNELS[int(x)] for x in out["kinds"]} == _abi.PLAN_KERNELS


# (desc kwargs, expected plan fields).  The Llama-3-8B prefill (B=1, Hq=32,
# Hkv=8, N=4096, d=128): four q-heads of a group per eight-wave workgroup,
# 64-row blocks, 8 units x 64 blocks; causal without a window pairs block
# 63 - j with block j in 256 workgroups.
_BS64 = dict(bs_row_ptr=FAKE.value, bs_col_idx=FAKE.value, bs_block_m=64, bs_block_n=64, bs_nnz=1)

PLAN_CASES = [
    ("llama8b_causal", dict(B=1, Hq=32, Hkv=8, N=4096, D=128, causal=1),
     dict(kernel=2, waves=8, heads=4, rows=64, query_blocks=64, paired=1, workgroups=256)),
    ("llama8b_full", dict(B=1, Hq=32, Hkv=8, N=4096, D=128),
     dict(kernel=2, waves=8, heads=4, rows=64, query_blocks=64, paired=0, workgroups=512)),
    # a causal window of 1024: one round of 256 pairs of 34 tiles does not beat
    # 512 single blocks (952 tiles per unit) spread over the CUs
    ("llama8b_causal_window", dict(B=1, Hq=32, Hkv=8, N=4096, D=128, causal=1, window=1024),
     dict(paired=0, workgroups=512)),
    # GPT-2-small, N=4096: 384 pairs would be one and a half rounds, so the
    # causal band takes four waves (128-row blocks)
    ("gpt2_small_causal", dict(B=4, Hq=12, Hkv=12, N=4096, D=64, causal=1),
     dict(waves=4, rows=128, query_blocks=32, paired=0, workgroups=1536)),
    # a two-sided window at D = 64: four waves
    ("gpt2_small_window", dict(B=4, Hq=12, Hkv=12, N=4096, D=64, window=256),
     dict(waves=4, rows=128, paired=0, workgroups=1536)),
    # dense at D = 64 keeps eight waves in whole rounds (768 = 3 x 256) ...
    ("gpt2_small_dense", dict(B=4, Hq=12, Hkv=12, N=4096, D=64), dict(waves=8, workgroups=768)),
    ("gpt2_small_dense_1k", dict(B=4, Hq=12, Hkv=12, N=1024, D=64), dict(waves=8, workgroups=192)),
    # ... and takes four waves when eight would make one and a half rounds (384)
    ("gpt2_small_dense_2k", dict(B=4, Hq=12, Hkv=12, N=2048, D=64), dict(waves=4, workgroups=768)),
    # N=8192: 768 pairs, three full rounds (eight waves, paired)
    ("gpt2_small_causal_8k", dict(B=4, Hq=12, Hkv=12, N=8192, D=64, causal=1),
     dict(waves=8, paired=1, workgroups=768)),
    # the ALiBi + causal + window workload (B=2, H=16, N=8192, W=1024): 32 units x 16 pairs
    ("alibi_window", dict(B=2, Hq=16, Hkv=16, N=8192, D=128, rope=False, causal=1, window=1024,
                          alibi_slopes=FAKE.value),
     dict(kernel=2, waves=8, heads=1, rows=256, query_blocks=32, paired=1, workgroups=512)),
    # non-causal: no pairing
    ("two_sided_window", dict(B=2, Hq=16, Hkv=16, N=8192, D=128, rope=False, window=1024),
     dict(paired=0, workgroups=1024)),
    # odd block count: the middle block runs alone (32 units x 8 = 256 workgroups)
    ("odd_blocks", dict(B=2, Hq=64, Hkv=16, N=950, D=128, causal=1),
     dict(kernel=2, waves=8, heads=4, rows=64, query_blocks=15, paired=1, workgroups=256)),
    # 19 blocks: 320 pairs are one and a quarter rounds, so no pairing
    ("odd_blocks_partial_round", dict(B=2, Hq=64, Hkv=16, N=1200, D=128, causal=1),
     dict(query_blocks=19, paired=0, workgroups=32 * 19)),
    # too few pairs to fill the chip
    ("small_grid", dict(B=1, Hq=8, Hkv=2, N=1024, D=128, causal=1), dict(paired=0)),
    # an additive bias keeps one block per workgroup (ALiBi slopes alone pair)
    ("bias", dict(B=1, Hq=32, Hkv=32, N=4096, D=128, rope=False, causal=1, bias=FAKE.value,
                  bias_stride=(0, 4096 * 4096, 4096, 1)),
     dict(paired=0)),
    ("alibi", dict(B=1, Hq=32, Hkv=32, N=4096, D=128, rope=False, causal=1, alibi_slopes=FAKE.value),
     dict(paired=1, workgroups=256)),
    # queries before the keys: early rows have no keys, no pairing
    ("rows_without_keys", dict(B=1, Hq=32, Hkv=8, N=4096, D=128, causal=1, k_pos0=64), dict(paired=0)),
    ("fp32", dict(B=1, Hq=4, Hkv=4, N=256, D=64, dtype=_abi.FP32, causal=1),
     dict(kernel=1, waves=1, heads=1, rows=64, query_blocks=4, paired=0, workgroups=16)),
    # fp8 inputs pair the same way (GQA 4:1, 15 blocks of 64 rows)
    ("fp8_causal", dict(B=2, Hq=64, Hkv=16, N=950, D=128, rope=False, causal=1, kv_fp8=1, q_fp8=1,
                        q_scale=1.0, k_scale=1.0, v_scale=1.0),
     dict(kernel=3, waves=8, heads=4, rows=64, query_blocks=15, paired=1, workgroups=256)),
    ("no_queries", dict(B=1, Hq=4, Hkv=4, N=256, D=64, Nq=0),
     dict(kernel=0, waves=0, workgroups=0)),
    # BigBird (B2 H16 N4096 D64, 64x64 blocks): two waves on the shallow
    # schedule (40 KB, four workgroups per CU), 2048 blocks on 1024 workgroup
    # slots -> chains of 2
    ("bigbird_chain", dict(B=2, Hq=16, Hkv=16, N=4096, D=64, **_BS64),
     dict(kernel=2, waves=2, heads=1, rows=64, query_blocks=64, paired=0, chain=2, workgroups=1024)),
    # at D = 128 (four-slot rings, 144 KB: one workgroup per CU): chains of 8
    ("bigbird_d128_chain", dict(B=2, Hq=16, Hkv=16, N=4096, D=128, **_BS64),
     dict(waves=2, chain=8, workgroups=256)),
    # one round of single blocks: no chain
    ("bigbird_one_round", dict(B=1, Hq=16, Hkv=16, N=4096, D=64, **_BS64), dict(chain=1, workgroups=1024)),
    ("bigbird_small", dict(B=1, Hq=4, Hkv=4, N=1024, D=64, **_BS64), dict(chain=1, workgroups=64)),
    # the caller's chain length; 16 blocks, chains of 3 (the last holds one)
    ("bigbird_chain_3", dict(B=1, Hq=4, Hkv=4, N=1000, D=64, tile_chain=3, **_BS64),
     dict(chain=3, query_blocks=16, workgroups=4 * 6)),
    # longer than the blocks: one chain per unit
    ("bigbird_chain_long", dict(B=1, Hq=2, Hkv=2, N=300, D=64, tile_chain=50, **_BS64),
     dict(chain=5, workgroups=2)),
    # dense launches and eight-wave block-sparse ones run single blocks
    ("dense_chain_1", dict(B=1, Hq=32, Hkv=8, N=4096, D=128, tile_chain=1), dict(chain=1, workgroups=512)),
    ("gqa_bigbird_eight_waves", dict(B=1, Hq=16, Hkv=4, N=4096, D=64, **_BS64),
     dict(waves=8, heads=4, chain=1)),
]


@pytest.mark.parametrize("name,kw,want", PLAN_CASES, ids=[c[0] for c in PLAN_CASES])
def test_fwd_plan(lib, name, kw, want):
    kw = dict(kw)
    d = _shape_desc(kw.pop("B"), kw.pop("Hq"), kw.pop("Hkv"), kw.pop("N"), kw.pop("D"), **kw)
    st, info = _plan(lib, d)
    assert st == _abi.OK
    for f, v in want.items():
        assert info[f] == v, (f, info)


@pytest.mark.parametrize("kw,status", [
    (dict(tile_chain=-1, **_BS64), _abi.ERR_INVALID),
    # chains need a block mask, two or four waves, one CSR block row per workgroup, no bias
    (dict(tile_chain=2), _abi.ERR_UNSUPPORTED),
    (dict(tile_chain=2, tile_waves=8, tile_heads=4, **_BS64), _abi.ERR_UNSUPPORTED),
    (dict(tile_chain=2, tile_waves=2, tile_heads=1, **dict(_BS64, bs_block_m=128)), _abi.ERR_UNSUPPORTED),
    (dict(tile_chain=2, **dict(_BS64, bs_block_m=128)), _abi.OK),  # four waves: 128 rows
    (dict(tile_chain=2, bias=FAKE.value, bias_stride=(0, 0, 64, 1), **_BS64), _abi.ERR_UNSUPPORTED),
    (dict(tile_chain=2, dtype=_abi.FP32, **_BS64), _abi.ERR_UNSUPPORTED),
    (dict(tile_chain=1, dtype=_abi.FP32, **_BS64), _abi.OK),
    (dict(tile_chain=2, **_BS64), _abi.OK),
])
def test_fwd_plan_chain_choices(lib, kw, status):
    d = _shape_desc(1, 4, 4, 256, 64, rope=False, **kw)
    st, info = _plan(lib, d)
    assert st == status, (kw, st)
    if st != _abi.OK:
        assert _fwd(lib, d) == st  # rejected before any HIP call (never launched here)
    elif kw.get("dtype") != _abi.FP32:
        assert info["chain"] == kw["tile_chain"]


def test_fwd_plan_status_matches_fwd(lib):
    for kw in (dict(tile_waves=3), dict(struct_size=8), dict(window=-1), dict(kv_fp8=2)):
        d = _good_desc(**kw)
        st, _ = _plan(lib, d)
        assert st == _fwd(lib, d) != _abi.OK, kw
    info = _abi.FwdPlanInfo(kernel=7)
    assert lib.attnfuse_fwd_plan(ctypes.byref(_good_desc(tile_waves=3)), ctypes.byref(info)) != _abi.OK
    assert info.kernel == 7  # left unchanged on an error
    assert lib.attnfuse_fwd_plan(ctypes.byref(_good_desc()), None) == _abi.ERR_INVALID

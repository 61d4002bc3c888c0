"""The C-ABI library on the host: loads, exports every declared symbol, plans and
validates without a GPU (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import attention_forward_attn_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    src = open(os.path.join(ROOT, "include", "attn_fwd.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = A.load_library()
    names = _declared_functions()
    assert len(names) >= 10, names
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/attn_fwd.h but not exported"
    assert set(names) == set(A.EXPORTS)


def test_ceiling_library_exports():
    """The benchmark's ceiling diagnostics live in their own library."""
    from attention_forward_attn_amd import build as B

    assert os.path.exists(B.CEILING_LIB), "build with python -m attention_forward_attn_amd.build"
    lib = ctypes.CDLL(B.CEILING_LIB)
    for n in ("attn_ceiling_device_info", "attn_ceiling_mfma", "attn_ceiling_copy", "attn_ceiling_spin"):
        assert hasattr(lib, n), n
    # the attention library does not carry them
    assert not hasattr(A.load_library(), "attn_ceiling_mfma")


def test_abi_version_and_struct_sizes():
    assert A.abi_version() == A.ABI_VERSION
    # the library checks struct_size; a plan call with the binding's structs must succeed
    A.plan_dense(1, 4, 1, 128, 128, 64, 64)


def test_abi_mismatch_is_reported():
    lib = A.load_library()
    a = A.AttnDenseArgs()
    a.struct_size = ctypes.sizeof(A.AttnDenseArgs) + 8
    p = A.AttnPlan()
    p.struct_size = ctypes.sizeof(A.AttnPlan)
    st = lib.attn_plan_dense(ctypes.byref(a), ctypes.byref(p))
    assert st == A.ATTN_ABI_MISMATCH
    assert b"struct_size" in lib.attn_last_error()


@pytest.mark.parametrize("kw,exc", [
    (dict(B=1, H=3, Hkv=2, Tq=16, Tk=16, d_qk=128, d_v=128), A.AttnInvalidArgument),   # H % Hkv
    (dict(B=1, H=4, Hkv=1, Tq=16, Tk=16, d_qk=96, d_v=96), A.AttnUnsupported),         # head dim
    (dict(B=1, H=4, Hkv=1, Tq=16, Tk=16, d_qk=128, d_v=64), A.AttnUnsupported),        # pair
    (dict(B=0, H=4, Hkv=1, Tq=16, Tk=16, d_qk=128, d_v=128), A.AttnInvalidArgument),   # B
    (dict(B=1, H=4, Hkv=1, Tq=-1, Tk=16, d_qk=128, d_v=128), A.AttnInvalidArgument),   # Tq
])
def test_dense_validation_errors(kw, exc):
    with pytest.raises(exc):
        A.plan_dense(**kw)


def test_dense_scale_and_dtype_errors():
    with pytest.raises(A.AttnInvalidArgument):
        A.plan_dense(1, 4, 1, 16, 16, 128, 128, scale=float("nan"))
    with pytest.raises(A.AttnInvalidArgument):
        A.plan_dense(1, 4, 1, 16, 16, 128, 128, scale=-1.0)
    with pytest.raises(A.AttnUnsupported):
        A.plan_dense(1, 4, 1, 16, 16, 512, 512, dtype="f32")


def test_null_and_misaligned_pointers_rejected():
    lib = A.load_library()
    a = A.AttnDenseArgs()
    a.struct_size = ctypes.sizeof(A.AttnDenseArgs)
    a.dtype = A.ATTN_BF16
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = 1, 4, 1, 8, 8, 128, 128
    a.scale = 0.1
    a.q_sb, a.q_sh, a.q_st = 4 * 8 * 128, 8 * 128, 128
    a.k_sb, a.k_sh, a.k_st = 8 * 128, 8 * 128, 128
    a.v_sb, a.v_sh, a.v_st = 8 * 128, 8 * 128, 128
    a.o_sb, a.o_sh, a.o_st = 4 * 8 * 128, 8 * 128, 128
    # NULL q
    a.k = a.v = a.out = a.lse = 4096
    assert lib.attn_fwd_dense(ctypes.byref(a), None) == A.ATTN_INVALID_ARGUMENT
    assert b"non-NULL" in lib.attn_last_error()
    # NULL k/v are fine when there are no keys (nothing is read) -- plan only, no launch
    a.q = 4096
    a.k = a.v = None
    a.Tk = 0
    p = A.AttnPlan()
    p.struct_size = ctypes.sizeof(A.AttnPlan)
    assert lib.attn_plan_dense(ctypes.byref(a), ctypes.byref(p)) == A.ATTN_OK
    a.k = a.v = 4096
    a.Tk = 8
    a.q = None
    # misaligned q (8-byte aligned only)
    a.q = 4096 + 8
    assert lib.attn_fwd_dense(ctypes.byref(a), None) == A.ATTN_INVALID_ARGUMENT
    assert b"aligned" in lib.attn_last_error()
    # a stride that breaks row alignment
    a.q = 4096
    a.q_st = 130
    assert lib.attn_fwd_dense(ctypes.byref(a), None) == A.ATTN_INVALID_ARGUMENT


def test_oversized_grids_rejected_before_narrowing():
    """Tile counts are formed in 64 bits and checked before they are narrowed to a
    32-bit launch size, also for the dropout kernels' smaller row tiles."""
    lib = A.load_library()

    def args(H, Tq, d, keep=False):
        a = A.AttnDenseArgs()
        a.struct_size = ctypes.sizeof(A.AttnDenseArgs)
        a.dtype = A.ATTN_BF16
        a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = 1, H, 1, Tq, 64, d, d
        a.scale, a.causal = 0.1, 1
        a.q = a.k = a.v = a.out = a.lse = 4096
        a.q_sb, a.q_sh, a.q_st = H * Tq * d, Tq * d, d
        a.k_sb, a.k_sh, a.k_st = 64 * d, 64 * d, d
        a.v_sb, a.v_sh, a.v_st = 64 * d, 64 * d, d
        a.o_sb, a.o_sh, a.o_st = H * Tq * d, Tq * d, d
        if keep:
            a.keep, a.p_drop = 4096, 0.1
            a.m_sb, a.m_sh, a.m_st = H * Tq * 2, Tq * 2, 2
        return a

    def plan(a):
        p = A.AttnPlan()
        p.struct_size = ctypes.sizeof(A.AttnPlan)
        return lib.attn_plan_dense(ctypes.byref(a), ctypes.byref(p))

    # 2^16 heads x 2^26 tokens: 2^34 row tiles of one group, past a 32-bit count
    assert plan(args(1 << 16, 1 << 26, 128)) == A.ATTN_INVALID_ARGUMENT
    assert b"too large" in lib.attn_last_error()
    # 128-wide: 3 * 2^29 tiles of 256 rows fit, the separate dropout kernel's
    # 128-row tiles do not
    assert plan(args(1 << 16, 3 << 21, 128)) == A.ATTN_OK
    assert plan(args(1 << 16, 3 << 21, 128, keep=True)) == A.ATTN_INVALID_ARGUMENT
    assert b"too large" in lib.attn_last_error()
    # 512-wide heads take the mask inside the fused kernel, on its own tiles
    assert plan(args(1 << 16, 3 << 20, 512, keep=True)) == A.ATTN_OK


def test_dropout_plans():
    """A keep mask with 512-wide heads plans the fused kernel's dropout instance (the
    mask applied inside, on the plain kernel's tiles); narrower heads run the separate
    dropout kernel, which plans do not describe."""
    lib = A.load_library()

    def args(d, keep):
        a = A.AttnDenseArgs()
        a.struct_size = ctypes.sizeof(A.AttnDenseArgs)
        a.dtype = A.ATTN_BF16
        a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = 1, 64, 1, 1400, 1400, d, d
        a.scale, a.causal = 0.05, 1
        a.q = a.k = a.v = a.out = a.lse = 4096
        a.q_sb, a.q_sh, a.q_st = 64 * 1400 * d, 1400 * d, d
        a.k_sb, a.k_sh, a.k_st = 1400 * d, 1400 * d, d
        a.v_sb, a.v_sh, a.v_st = 1400 * d, 1400 * d, d
        a.o_sb, a.o_sh, a.o_st = 64 * 1400 * d, 1400 * d, d
        if keep:
            a.keep, a.p_drop = 4096, 0.1
            a.m_sb, a.m_sh, a.m_st = 64 * 1400 * 44, 1400 * 44, 44
        return a

    def plan(a):
        p = A.AttnPlan()
        p.struct_size = ctypes.sizeof(A.AttnPlan)
        st = lib.attn_plan_dense(ctypes.byref(a), ctypes.byref(p))
        return st, p

    st, plain = plan(args(512, False))
    assert st == A.ATTN_OK and plain.path == b"dense_bf16_d512"
    st, drop = plan(args(512, True))
    assert st == A.ATTN_OK and drop.path == b"dense_bf16_d512_dropout"
    assert (drop.block_rows, drop.grid, drop.waves) == (plain.block_rows, plain.grid, plain.waves)
    st, _ = plan(args(128, True))
    assert st == A.ATTN_UNSUPPORTED and b"separate kernel" in lib.attn_last_error()


def test_sparse_validation_errors():
    with pytest.raises(A.AttnInvalidArgument):
        A.plan_sparse_topk(4, 64, 100, 512, 513, 16)           # d_v > d_qk
    with pytest.raises(A.AttnUnsupported):
        A.plan_sparse_topk(4, 128, 100, 512, 512, 16)          # too many heads per query
    with pytest.raises(A.AttnUnsupported):
        A.plan_sparse_topk(4, 64, 100, 256, 256, 16)           # head dim


def test_plans_for_the_five_workloads():
    p1 = A.plan_dense(1, 4, 1, 128, 128, 64, 64, dtype="f32")
    assert p1["path"] == "dense_f32split_d64" and p1["fold_g"] == 4 and p1["folded_rows"] == 512
    p2 = A.plan_dense(2, 32, 8, 4096, 4096, 128, 128)
    assert p2["path"] == "dense_bf16_d128" and p2["folded_rows"] == 4 * 4096
    assert p2["grid"] == 2 * 8 * 4 * (4096 // p2["block_rows"])
    p3 = A.plan_dense(4, 16, 16, 4096, 4096, 192, 128)
    assert p3["path"] == "dense_bf16_d192_v128" and p3["fold_g"] == 1
    p4 = A.plan_dense(1, 64, 1, 1400, 1400, 512, 512, sinks=True)
    assert p4["path"] == "dense_bf16_d512" and p4["fold_g"] == 64 and p4["folded_rows"] == 89600
    p5 = A.plan_sparse_topk(13312, 64, 65536, 512, 512, 2176)
    assert p5["path"] == "sparse_bf16_d512" and p5["grid"] == 13312
    for p in (p1, p2, p3, p4, p5):
        assert p["hbm_score_bytes"] == 0            # scores never leave the chip
        assert p["lds_bytes"] <= 160 * 1024


def test_budget_tiling_reproduces_arcflash_arithmetic():
    """The planner's byte-budget tiling at the DeepSeek-V4 prefill shape of the
    ArcFlash page (B=1 H=64 D=512 T=1400 bf16, 32 MiB): 11,983 folded rows per
    tile, 8 tiles, tile boundaries straddling heads."""
    p4 = A.plan_dense(1, 64, 1, 1400, 1400, 512, 512, sinks=True)
    assert p4["budget_bytes"] == 32 << 20
    assert p4["budget_tile_rows"] == 11983 and p4["budget_tiles"] == 8
    assert p4["budget_tile_rows"] % 1400 != 0
    assert A.budget_tile_rows(32 << 20, 1400, 8) == 2995
    assert A.budget_tile_rows(0, 1400, 2) == 0


def test_tile_budget_env(monkeypatch):
    monkeypatch.setenv("ATTN_TILE_BYTES", str(16 << 20))
    p = A.plan_dense(1, 64, 1, 1400, 1400, 512, 512)
    assert p["budget_tile_rows"] == (16 << 20) // (1400 * 2)


def test_dispatch_counts_start_at_zero():
    A.reset_dispatch_counts()
    assert A.dispatch_count("dense_bf16_d128") == 0
    assert A.dispatch_count("no_such_path") == 0


# ------------------------------------------------------------------ split-KV (host side)
def test_splitkv_planning():
    # prefill that already fills the device: one range, no workspace
    assert A.splitkv_choose(2, 32, 8, 4096, 4096, 128, 128) == 1
    assert A.splitkv_workspace_bytes(2, 32, 8, 4096, 4096, 128, 128) == 0
    # decode: ranges of whole 128-key blocks, never more than there are blocks
    assert A.splitkv_workspace_bytes(1, 8, 2, 1, 1000, 128, 128, n_splits=3) == 3 * 8 * 129 * 4
    assert A.splitkv_workspace_bytes(1, 8, 2, 1, 1000, 128, 128, n_splits=100) == 8 * 8 * 129 * 4
    n = A.splitkv_choose(8, 64, 1, 1, 32768, 512, 512, sinks=True)
    # 8 row blocks; without a device: 256 CUs, one 160 KB workgroup per CU
    assert n == 32
    assert A.splitkv_workspace_bytes(8, 64, 1, 1, 32768, 512, 512, sinks=True) == n * 8 * 64 * 513 * 4
    # no keys: one range
    assert A.splitkv_choose(1, 8, 2, 1, 0, 128, 128) == 1
    with pytest.raises(A.AttnInvalidArgument):
        A.splitkv_workspace_bytes(1, 8, 2, 1, 1000, 128, 128, n_splits=-1)
    with pytest.raises(A.AttnInvalidArgument):
        A.splitkv_workspace_bytes(1, 8, 2, 1, 1000, 128, 128, n_splits=5000)


def _fake_dense(dtype=0):
    a = A._shape_args(1, 8, 2, 1, 1000, 128, 128, "bf16" if dtype == 0 else "f32", True, False, None)
    return a


def test_splitkv_rejects_bad_workspace_before_launch():
    lib = A.load_library()
    a = _fake_dense()
    need = lib.attn_splitkv_workspace_bytes(ctypes.byref(a), 4)
    assert need > 0
    st = lib.attn_fwd_dense_splitkv(ctypes.byref(a), 4, None, 0, None)
    assert st == A.ATTN_INVALID_ARGUMENT and b"workspace" in lib.attn_last_error()
    st = lib.attn_fwd_dense_splitkv(ctypes.byref(a), 4, ctypes.c_void_p(4096), need - 16, None)
    assert st == A.ATTN_INVALID_ARGUMENT
    st = lib.attn_fwd_dense_splitkv(ctypes.byref(a), 4, ctypes.c_void_p(4096 + 8), need, None)
    assert st == A.ATTN_INVALID_ARGUMENT and b"aligned" in lib.attn_last_error()
    st = lib.attn_fwd_dense_splitkv(ctypes.byref(a), 2000, ctypes.c_void_p(4096), need, None)
    assert st == A.ATTN_INVALID_ARGUMENT
    f = _fake_dense(dtype=1)
    st = lib.attn_fwd_dense_splitkv(ctypes.byref(f), 4, ctypes.c_void_p(4096), 1 << 30, None)
    assert st == A.ATTN_UNSUPPORTED



# ------------------------------------------------------------------ dense backward (host side)
def _fake_bwd(**over):
    a = A.AttnDenseBwdArgs()
    a.struct_size = ctypes.sizeof(A.AttnDenseBwdArgs)
    a.dtype = A.ATTN_BF16
    a.B, a.H, a.Hkv, a.Tq, a.Tk, a.d_qk, a.d_v = 1, 8, 2, 16, 16, 128, 128
    a.causal, a.scale = 1, 0.1
    a.window_left = a.window_right = -1
    fake = 0x10000  # aligned, never dereferenced: validation fails first
    for n in ("q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"):
        setattr(a, n, fake)
    for n in ("q", "dq", "k", "dk"):
        setattr(a, n + "_st", 128)
    for n in ("v", "o", "do", "dv"):
        setattr(a, n + "_st", 128)
    for k, v in over.items():
        setattr(a, k, v)
    return a


def test_bwd_workspace_and_validation():
    lib = A.load_library()
    assert A.bwd_workspace_bytes(2, 32, 8, 4096, 4096, 128, 128) == 2 * 32 * 4096 * 4
    assert A.bwd_workspace_bytes(1, 8, 2, 3, 5, 64, 64) == 256          # rounded up to 256
    with pytest.raises(A.AttnInvalidArgument):
        A.bwd_workspace_bytes(1, 8, 3, 3, 5, 64, 64)                    # H % Hkv != 0
    assert lib.attn_bwd_dense_workspace_bytes(ctypes.byref(_fake_bwd(d_qk=384, d_v=384))) == -1
    assert lib.attn_bwd_dense_workspace_bytes(ctypes.byref(_fake_bwd(d_qk=256, d_v=128))) == -1
    assert lib.attn_bwd_dense_workspace_bytes(ctypes.byref(_fake_bwd(d_qk=512, d_v=512))) > 0
    # 512-wide MQA, 1400 keys: 44 key blocks of 32, so the 64 query heads are split
    # 16 ways and the workspace adds 16 fp32 [dK | dV] partials of the kv head
    assert A.bwd_workspace_bytes(1, 64, 1, 1400, 1400, 512, 512) == 64 * 1400 * 4 + 16 * 1400 * 1024 * 4
    # many key blocks (8 groups x 64 blocks of 64 keys): no split
    assert A.bwd_workspace_bytes(2, 32, 8, 4096, 4096, 256, 256) == 2 * 32 * 4096 * 4
    # the split never exceeds the heads of a group: 2 heads, 1 key block
    assert A.bwd_workspace_bytes(1, 2, 1, 16, 16, 256, 256) == 256 + 2 * 16 * 512 * 4
    ws = ctypes.c_void_p(0x20000)
    st = lib.attn_bwd_dense(ctypes.byref(_fake_bwd(d_qk=384, d_v=384)), ws, 1 << 20, None)
    assert st == A.ATTN_UNSUPPORTED
    st = lib.attn_bwd_dense(ctypes.byref(_fake_bwd(dsinks=0x30000)), ws, 1 << 20, None)
    assert st == A.ATTN_INVALID_ARGUMENT and b"dsinks" in lib.attn_last_error()
    st = lib.attn_bwd_dense(ctypes.byref(_fake_bwd()), ws, 16, None)
    assert st == A.ATTN_INVALID_ARGUMENT and b"workspace" in lib.attn_last_error()
    st = lib.attn_bwd_dense(ctypes.byref(_fake_bwd(dq=None)), ws, 1 << 20, None)
    assert st == A.ATTN_INVALID_ARGUMENT
    st = lib.attn_bwd_dense(ctypes.byref(_fake_bwd(q_st=100)), ws, 1 << 20, None)
    assert st == A.ATTN_INVALID_ARGUMENT
    bad = _fake_bwd()
    bad.struct_size = 8
    assert lib.attn_bwd_dense(ctypes.byref(bad), ws, 1 << 20, None) == A.ATTN_ABI_MISMATCH
    assert lib.attn_bwd_dense(ctypes.byref(_fake_bwd(dtype=A.ATTN_F32)), ws, 1 << 20, None) == A.ATTN_UNSUPPORTED


@pytest.mark.parametrize("d_v", [128, 256, 384])
def test_sparse_value_prefix_widths_plan(d_v):
    """V = the first d_v columns of each 512-wide pool row: d_v in {128, 256, 384} (and 512)
    are compiled, one kernel path each; other prefixes are UNSUPPORTED."""
    p = A.plan_sparse_topk(100, 64, 1000, 512, d_v, 300)
    assert p["path"] == f"sparse_bf16_d512_v{d_v}" and p["grid"] == 100 and p["block_rows"] == 64


@pytest.mark.parametrize("d_v", [64, 200, 448])
def test_sparse_value_prefix_unsupported(d_v):
    with pytest.raises(A.AttnUnsupported):
        A.plan_sparse_topk(10, 64, 1000, 512, d_v, 30)


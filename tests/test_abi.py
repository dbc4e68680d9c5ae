"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects invalid calls with the documented status before any HIP
call (only failing calls are made here, so nothing is ever launched)."""
import ctypes
import os
import re
import subprocess

import pytest

import precision_decode_amd as pd
from precision_decode_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", n) for n in sorted(os.listdir(os.path.join(ROOT, "include")))
           if n.endswith(".h")]

# Fake, never dereferenced device addresses (validation fails before any use).
# Tests that pass them to launch calls run only where no GPU is visible: there
# a validation regression ends in NVFP4_GEMV_ERR_DEVICE or a failed launch, and
# can never enqueue a kernel on unmapped addresses.
GPU_VISIBLE = os.path.exists("/dev/kfd")
fake_pointers = pytest.mark.skipif(GPU_VISIBLE, reason="fake device addresses are passed to "
                                   "launch calls only on machines without a GPU")
A, SA, X, SX, AL, C = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(nvfp4_\w+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_binding.LIB_PATH):
        from precision_decode_amd import build
        build.build()
    return pd.load()


def test_header_declares_the_exported_list():
    assert header_functions() == sorted(_binding.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _binding.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (nvfp4_\w+)", out))
    assert set(header_functions()) <= exported


def test_status_strings(lib):
    for st in range(0, -10, -1):
        s = pd.nvfp4_gemv_status_string(st)
        assert s and s != "unknown status"
    assert pd.nvfp4_gemv_status_string(-99) == "unknown status"


def call(l=1, m=8, k=64, a=A, sa=SA, x=X, sx=SX, al=AL, c=C):
    return pd.load().nvfp4_gemv_launch(a, sa, x, sx, al, c, l, m, k, None)


@fake_pointers
def test_null_pointers(lib):
    for kw in ("a", "sa", "x", "sx", "c"):
        assert call(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER


@fake_pointers
@pytest.mark.parametrize("l,m,k", [(0, 8, 64), (1, 0, 64), (1, 8, 0), (1, 8, 8), (1, 8, 40),
                                   (-1, 8, 64), (1, 8, 1 << 31), (1 << 20, 1 << 12, 64)])
def test_bad_shapes(lib, l, m, k):
    assert call(l=l, m=m, k=k) == pd.NVFP4_GEMV_ERR_BAD_SHAPE


@fake_pointers
def test_alias_detected(lib):
    # c overlapping A's (l*m*k/2)-byte range
    assert call(c=A + 100) == pd.NVFP4_GEMV_ERR_ALIAS
    assert call(c=SX) == pd.NVFP4_GEMV_ERR_ALIAS
    assert call(c=AL - 2) == pd.NVFP4_GEMV_ERR_ALIAS


@fake_pointers
def test_output_and_alpha_alignment(lib):
    assert call(c=C + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert call(al=AL + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT


@fake_pointers
def test_workspace_required_before_launch(lib):
    l, m, k = 1, 64, 16384
    need = pd.nvfp4_gemv_workspace_size(l, m, k)
    assert need > 0
    st = lib.nvfp4_gemv_launch_ws(A, SA, X, SX, AL, C, l, m, k, None, 0, None)
    assert st == pd.NVFP4_GEMV_ERR_WORKSPACE
    st = lib.nvfp4_gemv_launch_ws(A, SA, X, SX, AL, C, l, m, k, 0x70000000, need - 4, None)
    assert st == pd.NVFP4_GEMV_ERR_WORKSPACE
    st = lib.nvfp4_gemv_launch_ws(A, SA, X, SX, AL, C, l, m, k, 0x70000002, need, None)
    assert st == pd.NVFP4_GEMV_ERR_ALIGNMENT


def test_plan_defaults(lib):
    t, ws = pd.nvfp4_gemv_plan(1, 7168, 16384)
    assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.ksplit == 1 and ws == 0
    t, ws = pd.nvfp4_gemv_plan(1, 896, 16384)            # one eighth of the rows: split K
    assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.ksplit > 1 and ws == t.ksplit * 896 * 4
    t, ws = pd.nvfp4_gemv_plan(1, 64, 65536)             # K longer than one LDS stage
    assert t.ksplit >= 4
    t, _ = pd.nvfp4_gemv_plan(2, 100, 48)                # k % 32 != 0
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC
    t, _ = pd.nvfp4_gemv_plan(2, 100, 64, aligned=False)
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC
    assert pd.nvfp4_gemv_workspace_size(1, 896, 16384) >= pd.nvfp4_gemv_plan(1, 896, 16384)[1]


def test_plan_rejects_bad_tuning(lib):
    with pytest.raises(pd.Nvfp4GemvError) as e:
        pd.nvfp4_gemv_plan(1, 64, 48, tuning={"path": pd.NVFP4_GEMV_PATH_FAST})
    assert e.value.status == pd.NVFP4_GEMV_ERR_BAD_TUNING
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 64, tuning={"variant": pd.nvfp4_gemv_num_variants() + 1})
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 64, tuning={"ksplit": 3})   # 64/3 < one 32-element chunk each
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 65536, tuning={"ksplit": 1})  # exceeds one LDS stage
    t = _binding.Tuning(0, 0, 0, 1)
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 64, tuning=t)


def test_plan_explicit_choices(lib):
    n = pd.nvfp4_gemv_num_variants()
    assert n >= 1
    forms = set()
    for v in range(1, n + 1):
        r, u, w, px = pd.nvfp4_gemv_variant_info(v)
        assert r >= 1 and u >= 1 and 1 <= w <= 16 and px in (0, 1, 2, 3)
        forms.add(px)
        t, _ = pd.nvfp4_gemv_plan(3, 100, 4096, tuning={"variant": v, "ksplit": 2})
        assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.variant == v and t.ksplit == 2
    assert forms == {0, 1, 2, 3}   # every x staging form is available
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_variant_info(n + 1)
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 64, tuning={"path": pd.NVFP4_GEMV_PATH_GENERIC, "variant": 1})
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemv_plan(1, 64, 64, tuning={"path": 3})
    t, ws = pd.nvfp4_gemv_plan(3, 100, 4096, tuning={"path": pd.NVFP4_GEMV_PATH_GENERIC, "ksplit": 5})
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC and t.ksplit == 5 and ws == 5 * 300 * 4



def test_tile_variants_plan(lib):
    """Row-tile variants (16, 8 or 4 rows): K bound, no K split while waves cover the slices."""
    tiles = [v for v in range(1, pd.nvfp4_gemv_num_variants() + 1)
             if pd.nvfp4_gemv_variant_info(v)[3] == 3]
    assert tiles
    for v in tiles:
        r, u, w, _ = pd.nvfp4_gemv_variant_info(v)
        assert r in (16, 8, 4) and u == 1
        with pytest.raises(pd.Nvfp4GemvError):
            pd.nvfp4_gemv_plan(1, 64, 2 ** 26 + 32, tuning={"variant": v})
        t, ws = pd.nvfp4_gemv_plan(1, 64, 2 ** 26, tuning={"variant": v, "ksplit": 1})
        assert t.ksplit == 1 and ws == 0
        # 448 to 1792 tiles fill the 256 compute units: no split
        t, _ = pd.nvfp4_gemv_plan(1, 7168, 16384, tuning={"variant": v})
        assert t.ksplit == 1
        # 8 to 32 tiles: split while each split keeps a slice for every wave
        t, _ = pd.nvfp4_gemv_plan(1, 128, 16384, tuning={"variant": v})
        assert t.ksplit == max(1, 8 // w)

@fake_pointers
def test_probe_validation(lib):
    assert lib.nvfp4_hbm_read_probe(None, 1024, C, None) == pd.NVFP4_GEMV_ERR_NULL_POINTER
    assert lib.nvfp4_hbm_read_probe(A, 1000, C, None) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert lib.nvfp4_hbm_read_probe(A + 8, 1024, C, None) == pd.NVFP4_GEMV_ERR_ALIGNMENT


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(_binding, "LIB_PATH", "/nonexistent/libnvfp4_gemv.so")
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _binding.load()


def test_binding_refuses_host_tensors():
    import torch
    with pytest.raises(ValueError):
        _binding._ptr(torch.zeros(4, dtype=torch.uint8))


def test_binding_exports_same_names():
    for name in _binding.EXPORTED:
        assert callable(getattr(pd, name))


def test_header_constants_match_binding():
    for h in HEADERS:
        for name, val in re.findall(r"#define\s+(NVFP4_\w+)\s+\(?(-?\d+)\)?", open(h).read()):
            assert getattr(_binding, name) == int(val), name


# ---- activation quantiser and the bf16-activation GEMV (validation only)

XB, GS, Q, SF = 0x11000000, 0x12000000, 0x13000000, 0x14000000


def qcall(rows=2, d=64, x=XB, gs=GS, per_row=1, q=Q, sf=SF, rule=0):
    return pd.load().nvfp4_quantize_activation(x, gs, per_row, q, sf, rows, d, rule, None)


@fake_pointers
def test_quantize_validation(lib):
    for kw in ("x", "gs", "q", "sf"):
        assert qcall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER
    for rule in (-1, 3):
        assert qcall(rule=rule) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    assert qcall(per_row=2) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    for rows, d in ((0, 64), (2, 0), (2, 8), (2, 40), (-1, 64), (1 << 20, 1 << 16)):
        assert qcall(rows=rows, d=d) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert qcall(x=XB + 8) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert qcall(q=Q + 4) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert qcall(gs=GS + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert qcall(q=XB + 64) == pd.NVFP4_GEMV_ERR_ALIAS         # inside x's 256 bytes
    assert qcall(sf=XB + 255) == pd.NVFP4_GEMV_ERR_ALIAS
    assert qcall(sf=GS + 4) == pd.NVFP4_GEMV_ERR_ALIAS          # per-row scales: 8 bytes
    assert qcall(sf=Q + 63) == pd.NVFP4_GEMV_ERR_ALIAS          # q holds 64 bytes



def wcall(groups=2, rows=2, d=64, x=XB, rule=2, q=Q, sf=SF, g=GS):
    return pd.load().nvfp4_quantize_weight(x, groups, rows, d, rule, q, sf, g, None)


@fake_pointers
def test_weight_quantize_validation(lib):
    """Every rejection happens before any HIP call (this machine has no GPU)."""
    for kw in ("x", "q", "sf", "g"):
        assert wcall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER, kw
    for rule in (-1, 3):
        assert wcall(rule=rule) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    for groups, rows, d in ((0, 2, 64), (2, 0, 64), (2, 2, 8), (2, 2, 40), (-3, 2, 64),
                            (1 << 20, 1 << 12, 1 << 8)):
        assert wcall(groups=groups, rows=rows, d=d) == pd.NVFP4_GEMV_ERR_BAD_SHAPE, (groups, rows, d)
    assert wcall(x=XB + 8) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert wcall(q=Q + 4) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert wcall(g=GS + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert wcall(q=XB + 64) == pd.NVFP4_GEMV_ERR_ALIAS          # inside the 2*2*64 bf16 values
    assert wcall(g=Q + 60) == pd.NVFP4_GEMV_ERR_ALIAS           # the packed output holds 128 bytes
    assert wcall(g=SF + 12) == pd.NVFP4_GEMV_ERR_ALIAS          # sf holds 16 bytes
    assert wcall(g=XB + 508) == pd.NVFP4_GEMV_ERR_ALIAS         # the scales overlap x's last bytes

def bcall(l=2, m=8, k=64, a=A, sa=SA, asc=AL, x=XB, xs=GS, rule=0, q=Q, sf=SF, al=C + 4096, c=C):
    return pd.load().nvfp4_gemv_bf16x_launch(a, sa, asc, x, xs, rule, q, sf, al, c, l, m, k, None)


@fake_pointers
def test_bf16x_gemv_validation(lib):
    for kw in ("a", "sa", "x", "xs", "q", "sf", "al", "c"):
        assert bcall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER, kw
    assert bcall(rule=5) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    for l, m, k in ((0, 8, 64), (2, 0, 64), (2, 8, 40)):
        assert bcall(l=l, m=m, k=k) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert bcall(c=C + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert bcall(al=C + 4098) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert bcall(asc=AL + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert bcall(c=A + 10) == pd.NVFP4_GEMV_ERR_ALIAS           # c inside A
    assert bcall(al=Q + 8) == pd.NVFP4_GEMV_ERR_ALIAS           # alpha inside x_packed
    assert bcall(c=SF) == pd.NVFP4_GEMV_ERR_ALIAS               # c on sfx
    assert bcall(q=AL) == pd.NVFP4_GEMV_ERR_ALIAS               # x_packed on A_scale
    assert bcall(al=GS + 4) == pd.NVFP4_GEMV_ERR_ALIAS          # alpha on x_scale


# ---- small-N GEMM and grouped GEMV (validation and plans only)

B_, SB_, OF, GX, GW = 0x15000000, 0x16000000, 0x17000000, 0x18000000, 0x19000000


def scall(l=2, m=24, n=4, k=64, a=A, sa=SA, b=B_, sb=SB_, al=AL, c=C, out=0):
    return pd.load().nvfp4_gemm_smalln_launch(a, sa, b, sb, al, c, l, m, n, k, out, None)


@fake_pointers
def test_smalln_validation(lib):
    for kw in ("a", "sa", "b", "sb", "c"):
        assert scall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER, kw
    for out in (-1, 2):
        assert scall(out=out) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    for l, m, n, k in ((0, 8, 2, 64), (1, 0, 2, 64), (1, 8, 0, 64), (1, 8, 2, 40), (1, 8, 2, 8),
                       (1 << 12, 1 << 12, 1 << 8, 64)):
        assert scall(l=l, m=m, n=n, k=k) == pd.NVFP4_GEMV_ERR_BAD_SHAPE, (l, m, n, k)
    assert scall(c=C + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert scall(al=AL + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert scall(c=A + 10) == pd.NVFP4_GEMV_ERR_ALIAS
    assert scall(c=B_ + 8) == pd.NVFP4_GEMV_ERR_ALIAS
    assert scall(c=SB_ - 2) == pd.NVFP4_GEMV_ERR_ALIAS          # c's 192 bytes reach sfB


def test_smalln_plans(lib):
    t, ws = pd.nvfp4_gemm_smalln_plan(1, 7168, 16, 16384)
    assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.variant >= 1
    assert ws == (t.ksplit * 7168 * 16 * 4 if t.ksplit > 1 else 0)
    # few workgroups: rows per workgroup chosen so every one of the 256 CUs gets the same number
    blocks = -(-7168 // t.rows_per_block) * t.ksplit
    assert blocks % 256 == 0 and 1 <= t.rows_per_block <= 32
    t, _ = pd.nvfp4_gemm_smalln_plan(1, 7168, 16, 16384, tuning={"variant": 1, "rows_per_block": 9})
    assert t.rows_per_block == 9 and t.ksplit >= 1
    t, _ = pd.nvfp4_gemm_smalln_plan(64, 4096, 4, 4096)      # plenty of tiles: full 16-row tiles
    r, _, _ = pd.nvfp4_mma_variant_info(t.variant)
    assert t.rows_per_block == 16 * r and t.ksplit == 1
    t, ws = pd.nvfp4_gemm_smalln_plan(2, 100, 3, 48)           # k % 32 != 0
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC and t.ksplit == 1 and ws == 0
    t, _ = pd.nvfp4_gemm_smalln_plan(2, 100, 3, 64, aligned=False)
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC
    # the launches' shape rules: outputs below 2^31 elements
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemm_smalln_plan(1, 1 << 16, 1 << 15, 64)
    t, _ = pd.nvfp4_gemm_smalln_plan(1, 1 << 16, (1 << 15) - 1, 64)
    n = pd.nvfp4_mma_num_variants()
    forms = set()
    for v in range(1, n + 1):
        r, u, w = pd.nvfp4_mma_variant_info(v)
        form = pd.nvfp4_mma_variant_form(v)
        forms.add(form)
        if form in (pd.NVFP4_MMA_FORM_MATRIX_CORES, pd.NVFP4_MMA_FORM_LDS_STAGED,
                    pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS):
            assert r in (1, 2) and u >= 1 and 1 <= w <= 16
            t, ws = pd.nvfp4_gemm_smalln_plan(3, 100, 5, 4096, tuning={"variant": v, "ksplit": 3})
            assert t.variant == v and t.ksplit == 3 and ws == 3 * 3 * 100 * 5 * 4
        else:
            # VALU row tiles: r rows per workgroup, u vectors per pass, never a K split
            assert form == pd.NVFP4_MMA_FORM_VALU_TILES
            assert r in (4, 8) and u in (1, 2, 4) and 1 <= w <= 16
            t, ws = pd.nvfp4_gemm_smalln_plan(3, 100, 5, 4096, tuning={"variant": v})
            assert t.variant == v and t.ksplit == 1 and ws == 0 and t.rows_per_block == r
            t, _ = pd.nvfp4_gemm_smalln_plan(3, 100, 5, 4096, tuning={"variant": v, "rows_per_block": 3})
            assert t.rows_per_block == 3
            for bad in ({"variant": v, "ksplit": 3}, {"variant": v, "rows_per_block": r + 1}):
                with pytest.raises(pd.Nvfp4GemvError):
                    pd.nvfp4_gemm_smalln_plan(3, 100, 5, 4096, tuning=bad)
    assert forms == {pd.NVFP4_MMA_FORM_MATRIX_CORES, pd.NVFP4_MMA_FORM_VALU_TILES,
                     pd.NVFP4_MMA_FORM_LDS_STAGED, pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS}
    for bad_v in (0, n + 1):
        with pytest.raises(pd.Nvfp4GemvError):
            pd.nvfp4_mma_variant_form(bad_v)
    for bad in ({"variant": n + 1}, {"ksplit": 3, "path": pd.NVFP4_GEMV_PATH_GENERIC},
                {"path": pd.NVFP4_GEMV_PATH_GENERIC, "variant": 1}, {"path": 3},
                {"rows_per_block": -1}, {"variant": 1, "rows_per_block": 33},
                {"path": pd.NVFP4_GEMV_PATH_GENERIC, "rows_per_block": 8}):
        with pytest.raises(pd.Nvfp4GemvError):
            pd.nvfp4_gemm_smalln_plan(1, 64, 4, 4096, tuning=bad)
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemm_smalln_plan(1, 64, 4, 64, tuning={"ksplit": 3})   # under 32 elements a split
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_gemm_smalln_plan(1, 64, 4, 48, tuning={"path": pd.NVFP4_GEMV_PATH_FAST})
    with pytest.raises(pd.Nvfp4GemvError):
        pd.nvfp4_mma_variant_info(0)


@fake_pointers
def test_smalln_tuned_needs_workspace(lib):
    l, m, n, k = 1, 64, 4, 4096
    t = _binding.MmaTuning(0, 0, 4, 0)
    _, need = pd.nvfp4_gemm_smalln_plan(l, m, n, k, tuning=t)
    assert need == 4 * m * n * 4
    f = lib.nvfp4_gemm_smalln_launch_tuned
    assert f(A, SA, B_, SB_, AL, C, l, m, n, k, 0, ctypes.byref(t), None, 0, None) == \
        pd.NVFP4_GEMV_ERR_WORKSPACE
    assert f(A, SA, B_, SB_, AL, C, l, m, n, k, 0, ctypes.byref(t), 0x70000000, need - 4, None) == \
        pd.NVFP4_GEMV_ERR_WORKSPACE
    assert f(A, SA, B_, SB_, AL, C, l, m, n, k, 0, ctypes.byref(t), 0x70000002, need, None) == \
        pd.NVFP4_GEMV_ERR_ALIGNMENT


def gcall(tokens=8, experts=3, n=32, k=64, x=X, sx=SX, w=A, sw=SA, of=OF, gx=GX, gw=GW, c=C, out=1,
          tuning=None):
    if tuning is None:
        return pd.load().nvfp4_grouped_gemv_launch(x, sx, w, sw, of, gx, gw, c, tokens, experts, n,
                                                   k, out, None)
    return pd.load().nvfp4_grouped_gemv_launch_tuned(x, sx, w, sw, of, gx, gw, c, tokens, experts,
                                                     n, k, out, ctypes.byref(tuning), None)


@fake_pointers
def test_grouped_validation(lib):
    for kw in ("x", "sx", "w", "sw", "of", "c"):
        assert gcall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER, kw
    assert gcall(out=3) == pd.NVFP4_GEMV_ERR_BAD_ARGUMENT
    for tokens, experts, n, k in ((-1, 3, 32, 64), (8, 0, 32, 64), (8, 3, 0, 64), (8, 3, 32, 40),
                                  (1 << 20, 3, 1 << 12, 64)):
        assert gcall(tokens=tokens, experts=experts, n=n, k=k) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert gcall(c=C + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert gcall(of=OF + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert gcall(gx=GX + 1) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert gcall(c=A + 64) == pd.NVFP4_GEMV_ERR_ALIAS               # c inside the weights
    assert gcall(c=OF - 4) == pd.NVFP4_GEMV_ERR_ALIAS               # c's 512 bytes reach offsets
    assert gcall(c=GW) == pd.NVFP4_GEMV_ERR_ALIAS
    assert gcall(tuning=_binding.MmaTuning(0, 0, 2, 0)) == pd.NVFP4_GEMV_ERR_BAD_TUNING  # no K split
    assert gcall(tuning=_binding.MmaTuning(1, 0, 0, 0), k=48) == pd.NVFP4_GEMV_ERR_BAD_TUNING
    assert gcall(tuning=_binding.MmaTuning(0, 1, 0, 17)) == pd.NVFP4_GEMV_ERR_BAD_TUNING  # > 16 rows


@pytest.mark.parametrize("l,m,k,variant", [(1, 7168, 16384, 31), (8, 4096, 7168, 20),
                                           (4, 7168, 2048, 29), (16, 2048, 4096, 25),
                                           (1, 7168, 32768, 1)])
def test_default_plans_of_the_benchmark_workloads(lib, l, m, k, variant):
    """The measured defaults: the 8-wave 4-row tile for 6-8 slices, (2, 4, 7)
    staged for longer rows, x read next to A for 3-5 slices, the 2-wave 16-row
    tile for 2 slices, the 1-wave 4-row tile for 1 slice; none of the
    benchmark workloads splits K (the staged kernel splits 32768 in two LDS
    stages)."""
    t, ws = pd.nvfp4_gemv_plan(l, m, k)
    assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.variant == variant
    assert (t.ksplit, ws) == ((2, 2 * l * m * 4) if k > 16384 else (1, 0))


def test_smalln_default_form_by_vector_count(lib):
    """One or two vectors against a weight that fills the GPU with 4-row tiles
    go to the VALU tiles; 3 to 13 vectors (or one or two with too few tiles)
    to the matrix cores with LDS-staged weights and the vectors in registers;
    more vectors to the all-LDS form (row-major weights)."""
    for n in (1, 2):
        t, ws = pd.nvfp4_gemm_smalln_plan(1, 7168, n, 16384)
        assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_VALU_TILES
        assert pd.nvfp4_mma_variant_info(t.variant) == (4, n, 4)   # one vector slot per vector
        assert t.ksplit == 1 and ws == 0 and t.rows_per_block == 4
    for l, m, n, k in ((1, 7168, 3, 16384), (1, 7168, 8, 16384), (1, 7168, 13, 16384),
                       (1, 256, 2, 16384)):
        t, _ = pd.nvfp4_gemm_smalln_plan(l, m, n, k)
        assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS, (l, m, n, k)
        assert pd.nvfp4_mma_variant_info(t.variant) == (2, 2, 4)
    for l, m, n, k in ((1, 7168, 14, 16384), (1, 7168, 16, 16384)):
        t, _ = pd.nvfp4_gemm_smalln_plan(l, m, n, k)
        assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_LDS_STAGED, (l, m, n, k)
        assert pd.nvfp4_mma_variant_info(t.variant) == (2, 2, 4)


def test_grouped_plan(lib):
    """The grouped plan: LDS-staged matrix cores on row-major weights (with the
    tokens in registers while the experts average at most 4 tokens), the
    register-fed ones on packed weights, the generic kernel off the fast
    shapes; never a K split."""
    for tokens in (0, 128, 256):
        t = pd.nvfp4_grouped_gemv_plan(64, 2048, 7168, tokens)
        assert t.path == pd.NVFP4_GEMV_PATH_FAST and t.ksplit == 1
        assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS
        assert pd.nvfp4_mma_variant_info(t.variant) == (2, 2, 2)
    t = pd.nvfp4_grouped_gemv_plan(64, 2048, 7168, 257)
    assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_LDS_STAGED
    assert pd.nvfp4_mma_variant_info(t.variant) == (2, 2, 2)
    t = pd.nvfp4_grouped_gemv_plan(64, 2048, 7168, 128, packed=True)
    assert pd.nvfp4_mma_variant_form(t.variant) == pd.NVFP4_MMA_FORM_MATRIX_CORES
    assert pd.nvfp4_mma_variant_info(t.variant) == (2, 1, 8)
    t = pd.nvfp4_grouped_gemv_plan(4, 96, 96, 20)               # k % 64 != 0
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC and t.variant == 0
    t = pd.nvfp4_grouped_gemv_plan(4, 96, 128, 20, aligned=False)
    assert t.path == pd.NVFP4_GEMV_PATH_GENERIC
    staged = [v for v in range(1, pd.nvfp4_mma_num_variants() + 1)
              if pd.nvfp4_mma_variant_form(v) in (pd.NVFP4_MMA_FORM_LDS_STAGED,
                                                  pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS)]
    t = pd.nvfp4_grouped_gemv_plan(4, 96, 128, 20, tuning={"variant": staged[-1], "rows_per_block": 20})
    assert t.variant == staged[-1] and t.rows_per_block == 20
    for kw in ({"packed": True, "k": 96}, {"k": 0}, {"experts": 0}, {"tokens": -1},
               {"tokens": 1 << 21, "n": 1 << 10}):
        args = {"experts": 4, "n": 96, "k": 128, "tokens": 20}
        args.update(kw)
        packed = args.pop("packed", False)
        with pytest.raises(pd.Nvfp4GemvError):
            pd.nvfp4_grouped_gemv_plan(args["experts"], args["n"], args["k"], args["tokens"],
                                       packed=packed)
    for v in (staged[0], staged[-1]):
        for kw in ({"tuning": {"ksplit": 2}}, {"packed": True, "tuning": {"variant": v}}):
            with pytest.raises(pd.Nvfp4GemvError):
                pd.nvfp4_grouped_gemv_plan(4, 96, 128, 20, **kw)
    assert lib.nvfp4_grouped_gemv_plan(4, 96, 128, 20, 1, 0, None, None) == \
        pd.NVFP4_GEMV_ERR_NULL_POINTER


# ---------------------------------------------------------------- packed weights
WP, SWP = 0x80000000, 0x90000000


def test_packed_sizes(lib):
    cb, sb = pd.nvfp4_mma_packed_sizes(1, 7168, 16384)        # 448 tiles x 64 windows
    assert (cb, sb) == (448 * 64 * 2048, 448 * 64 * 256)
    assert cb == 7168 * 16384 // 2 and sb == 7168 * 16384 // 16   # whole tiles and windows: no padding
    cb, sb = pd.nvfp4_mma_packed_sizes(3, 33, 320)             # 3 tiles (33 rows), 2 windows (320)
    assert (cb, sb) == (3 * 3 * 2 * 2048, 3 * 3 * 2 * 256)
    for bad in ((1, 16, 48), (1, 16, 96), (1, 16, 2 ** 26 + 64), (0, 16, 64), (1, 0, 64), (1, 16, 0)):
        with pytest.raises(pd.Nvfp4GemvError):
            pd.nvfp4_mma_packed_sizes(*bad)
    assert lib.nvfp4_mma_packed_sizes(1, 16, 64, None, None) == pd.NVFP4_GEMV_ERR_NULL_POINTER


def pcall(W=A, sW=SA, groups=2, rows=20, k=128, Wp=WP, sWp=SWP):
    return pd.load().nvfp4_mma_pack_weight(W, sW, groups, rows, k, Wp, sWp, None)


@fake_pointers
def test_pack_weight_validation(lib):
    for kw in ("W", "sW", "Wp", "sWp"):
        assert pcall(**{kw: None}) == pd.NVFP4_GEMV_ERR_NULL_POINTER, kw
    for groups, rows, k in ((0, 20, 128), (2, 0, 128), (2, 20, 96), (2, 20, 40)):
        assert pcall(groups=groups, rows=rows, k=k) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert pcall(W=A + 8) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert pcall(Wp=WP + 8) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert pcall(sW=SA + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert pcall(sWp=SWP + 2) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert pcall(Wp=A + 16) == pd.NVFP4_GEMV_ERR_ALIAS             # output over the input codes
    assert pcall(sWp=SA) == pd.NVFP4_GEMV_ERR_ALIAS
    assert pcall(sWp=WP + 1024) == pd.NVFP4_GEMV_ERR_ALIAS          # the two outputs overlap


@fake_pointers
def test_packed_launch_validation(lib):
    f = pd.load().nvfp4_gemm_smalln_launch_packed
    g = pd.load().nvfp4_grouped_gemv_launch_packed

    def s(k=128, A_=A, tuning=None, **kw):
        t = ctypes.byref(_binding.MmaTuning(*tuning)) if tuning else None
        return f(A_, SA, B_, SB_, AL, C, 1, 64, 4, k, 0, t, None)

    def gr(k=128, tuning=None):
        t = ctypes.byref(_binding.MmaTuning(*tuning)) if tuning else None
        return g(X, SX, A, SA, OF, GX, GW, C, 8, 3, 32, k, 1, t, None)

    assert s(k=96) == pd.NVFP4_GEMV_ERR_BAD_SHAPE                  # packed: k % 64 == 0, no generic path
    assert gr(k=96) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert s(A_=A + 8) == pd.NVFP4_GEMV_ERR_ALIGNMENT
    assert f(None, SA, B_, SB_, AL, C, 1, 64, 4, 128, 0, None, None) == pd.NVFP4_GEMV_ERR_NULL_POINTER
    assert f(C, SA, B_, SB_, AL, C, 1, 64, 4, 128, 0, None, None) == pd.NVFP4_GEMV_ERR_ALIAS
    valu = [v for v in range(1, pd.nvfp4_mma_num_variants() + 1)
            if pd.nvfp4_mma_variant_form(v) == pd.NVFP4_MMA_FORM_VALU_TILES]
    staged = [v for v in range(1, pd.nvfp4_mma_num_variants() + 1)
              if pd.nvfp4_mma_variant_form(v) == pd.NVFP4_MMA_FORM_LDS_STAGED]
    vregs = [v for v in range(1, pd.nvfp4_mma_num_variants() + 1)
             if pd.nvfp4_mma_variant_form(v) == pd.NVFP4_MMA_FORM_LDS_VECTOR_REGS]
    for bad in ((0, valu[0], 0, 0), (0, staged[0], 0, 0), (0, vregs[0], 0, 0), (2, 0, 0, 0),
                (0, 1, 0, 8), (0, 3, 0, 24), (0, 1, 0, 48)):
        # VALU or LDS-staged variants, generic path, partial tiles
        assert s(tuning=bad) == pd.NVFP4_GEMV_ERR_BAD_TUNING, bad
        assert gr(tuning=bad) == pd.NVFP4_GEMV_ERR_BAD_TUNING, bad
    assert gr(tuning=(0, 1, 2, 0)) == pd.NVFP4_GEMV_ERR_BAD_TUNING   # the grouped call never splits K


@fake_pointers
def test_workspace_reserve_without_a_device(lib):
    assert lib.nvfp4_workspace_reserve(0, None) == pd.NVFP4_GEMV_OK          # nothing to do
    assert lib.nvfp4_workspace_reserve(4096, None) == pd.NVFP4_GEMV_ERR_DEVICE


@fake_pointers
def test_split_k_launch_without_a_device(lib):
    """A valid split-K call reaches the workspace step, which needs a device."""
    need = lib.nvfp4_gemv_workspace_size(1, 896, 16384)
    assert need > 0
    assert call(l=1, m=896, k=16384) == pd.NVFP4_GEMV_ERR_DEVICE


@fake_pointers
def test_noalloc_validation_and_size_limit(lib):
    f = lib.nvfp4_gemv_launch_noalloc
    assert f(None, SA, X, SX, AL, C, 1, 8, 64, None) == pd.NVFP4_GEMV_ERR_NULL_POINTER
    assert f(A, SA, X, SX, AL, C, 1, 8, 40, None) == pd.NVFP4_GEMV_ERR_BAD_SHAPE
    assert f(A, SA, X, SX, AL, A + 2, 1, 8, 64, None) == pd.NVFP4_GEMV_ERR_ALIAS
    # partial sums above the fixed array: refused before any device query
    l, m, k = 1, 524352, 32768
    assert pd.nvfp4_gemv_workspace_size(l, m, k) > pd.NVFP4_GEMV_NOALLOC_SCRATCH_BYTES
    big = (1 << 44, 2 << 44, 3 << 44, 4 << 44, 5 << 44, 6 << 44)
    assert f(*big, l, m, k, None) == pd.NVFP4_GEMV_ERR_WORKSPACE
    # a split that fits reaches the device query (none here)
    assert f(A, SA, X, SX, AL, C, 1, 896, 16384, None) == pd.NVFP4_GEMV_ERR_DEVICE


def test_noalloc_limit_matches_header():
    text = open(os.path.join(ROOT, "include", "nvfp4_gemv.h")).read()
    assert "#define NVFP4_GEMV_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)" in text
    assert pd.NVFP4_GEMV_NOALLOC_SCRATCH_BYTES == 4 << 20

"""GPU parity of the activation quantiser and of the bf16-activation GEMV
against the CPU oracle (called through the C ABI).

Quantised bytes (codes and block scales) and alpha must match bit for bit
under every rounding rule: both sides take every decision from the same fp32
operations.  The GEMV output fed by a quantised Gaussian activation is
compared within max(2 fp16 ulp, 1e-3 relative), as for the Gaussian workload.
"""
import numpy as np
import pytest
import torch

import precision_decode_amd as pd
import workloads
from golden_io import quant_examples
from gpu_util import assert_within_tolerance, to_device
from oracle import quantize as oq

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]

RULES = [pd.NVFP4_ROUND_HALF_STEP, pd.NVFP4_ROUND_NEAREST_EVEN, pd.NVFP4_ROUND_NEAREST_LOWER]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    pd.load()


def bf16_bits(vals):
    """float32 values that are bf16-exact -> uint16 bit patterns (numpy)."""
    v = np.ascontiguousarray(np.asarray(vals, dtype=np.float32))
    bits = v.view(np.uint32)
    assert np.all((bits & 0xFFFF) == 0) or np.isnan(v).any(), "values must be bf16-exact"
    return (bits >> 16).astype(np.uint16)


def bits_to_f32(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def run_quant(bits, gs, rule, per_row=None):
    """bits: (rows, d) uint16 bf16 patterns; gs: scalar or (rows,) float32."""
    rows, d = bits.shape
    x = torch.from_numpy(bits.view(np.int16).copy()).cuda()
    g = torch.from_numpy(np.atleast_1d(np.asarray(gs, dtype=np.float32)).copy()).cuda()
    if per_row is None:
        per_row = 1 if g.numel() == rows and rows > 1 else 0
    q = torch.full((rows, d // 2), 0xA5, dtype=torch.uint8, device="cuda")
    sf = torch.full((rows, d // 16), 0xA5, dtype=torch.uint8, device="cuda")
    pd.nvfp4_quantize_activation(x, g, per_row, q, sf, rows, d, rule)
    torch.cuda.synchronize()
    return q.cpu().numpy(), sf.cpu().numpy()


def check_quant(bits, gs, rule, what=""):
    want_q, want_sf = oq.quantize_with_scale(bits_to_f32(bits), gs, rule)
    got_q, got_sf = run_quant(bits, gs, rule)
    bad_sf = np.argwhere(got_sf != want_sf)
    assert bad_sf.size == 0, f"{what}: {len(bad_sf)} scale bytes differ, first {bad_sf[:3].tolist()}"
    bad_q = np.argwhere(got_q != want_q)
    assert bad_q.size == 0, f"{what}: {len(bad_q)} code bytes differ, first {bad_q[:3].tolist()}"


@pytest.mark.parametrize("ex", quant_examples(), ids=lambda e: f"{e['name']}-{e['rule']}")
def test_hand_derived_examples(ex):
    q, sf = run_quant(bf16_bits(ex["values"])[None, :], ex["gs"], oq.RULE_NAMES[ex["rule"]])
    assert int(sf[0, 0]) == ex["sf"]
    assert q[0].tobytes().hex() == ex["packed"].tobytes().hex()


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("rows,d", [(1, 16), (1, 16384), (3, 4144), (8, 7168), (64, 2048),
                                    (1000, 48), (5, 16), (9, 1008), (7, 1024), (11, 1040)])
def test_gaussian_rows_per_row_scale(rule, rows, d):
    raw = workloads.gaussian_bf16(1, rows, d, seed=rows * 31 + d)["A"][0]
    amax = np.abs(raw).max(axis=1).astype(np.float32)
    gs = (amax / np.float32(2688.0)).astype(np.float32)
    check_quant(bf16_bits(raw), gs, rule, f"{rows}x{d}")


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("gs", [1e-4, 2.0 ** -9, 0.0037, 1.0, 300.0])
def test_scalar_scale_across_ranges(rule, gs):
    """Small scales push blocks past E4M3's range (NaN scales), large ones into
    its subnormals and to zero scales."""
    raw = workloads.gaussian_bf16(1, 16, 1024, seed=17)["A"][0]
    check_quant(bf16_bits(raw), np.float32(gs), rule, f"gs={gs}")


@pytest.mark.parametrize("rule", RULES)
def test_every_bf16_pattern(rule):
    """All 65536 bf16 bit patterns (zeros, subnormals, normals, infinities, NaNs)
    as 4096 blocks, at three global scales."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(16, 4096)
    for gs in (1.0, 3.5e-3, 2.0 ** 40):
        check_quant(bits, np.float32(gs), rule, f"all patterns, gs={gs}")
    rng = np.random.default_rng(3)
    check_quant(bits[:, rng.permutation(4096)], np.float32(0.75), rule, "all patterns, shuffled")



# Every E2M1 cut point of the three rules (grid midpoints and the half-step
# table's cuts).
CUTS = [0.25, 0.75, 1.25, 1.75, 2.25, 2.5, 2.75, 3.25, 3.5, 3.75, 4.25, 4.5, 4.75, 5.0, 5.25,
        5.75, 6.0]


def near_cut_blocks(g, den):
    """Blocks whose largest element makes the block scale `den` (6 * den * g),
    the other 15 the bf16 neighbours (below, nearest, above, negated) of
    cut * den * g, so x/g/den lands on or next to the cut points."""
    cand = []
    for t in CUTS:
        v = np.float32(t * den * g)
        b = int(np.array([v], dtype=np.float32).view(np.uint32)[0] >> 16)
        for nb in (b - 1, b, b + 1):
            cand += [nb, nb | 0x8000]
    top = int(np.array([np.float32(6.0 * den * g)], dtype=np.float32).view(np.uint32)[0] >> 16)
    blocks = []
    for i in range(0, len(cand), 15):
        chunk = cand[i:i + 15]
        chunk += [0] * (15 - len(chunk))
        blocks.append([top] + chunk)
    return np.array(blocks, dtype=np.uint32).astype(np.uint16).reshape(1, -1)


@pytest.mark.parametrize("rule", RULES)
def test_values_on_and_next_to_every_cut(rule):
    """Ties and their neighbours after both divisions, for global scales that
    are and are not powers of two and block scales across E4M3's range
    (normal, subnormal), so each rounding rule's tie handling is exercised."""
    for g in (1.0, 0.0037, 1.3, 7.77e-3, 2.0 ** -20, 123.0):
        for den in (1.0, 0.875, 1.25, 0.0625, 3.0 * 2.0 ** -9, 448.0, 0.6875):
            check_quant(near_cut_blocks(g, den), np.float32(g), rule, f"g={g} den={den}")

def test_negative_subnormals_keep_their_sign():
    """bf16 subnormals stay subnormal in fp32; a flush to zero would turn
    their negative codes (8 + index) into code 0."""
    vals = np.zeros(16, dtype=np.uint16)
    vals[:8] = [0x8001, 0x0001, 0x807F, 0x007F, 0x8040, 0x0010, 0x8000, 0x0000]
    for rule in RULES:
        check_quant(vals[None, :], np.float32(1.0), rule, "subnormals")
        q, _ = run_quant(vals[None, :], np.float32(1.0), rule)
        assert q[0, 0] & 0x8 == 0x8


def test_scalar_and_per_row_scale_agree():
    raw = workloads.gaussian_bf16(1, 6, 256, seed=23)["A"][0]
    bits = bf16_bits(raw)
    q1, s1 = run_quant(bits, np.float32(0.002), pd.NVFP4_ROUND_HALF_STEP, per_row=0)
    q2, s2 = run_quant(bits, np.full(6, 0.002, dtype=np.float32), pd.NVFP4_ROUND_HALF_STEP, per_row=1)
    assert np.array_equal(q1, q2) and np.array_equal(s1, s2)


def test_misaligned_input_rejected_before_launch():
    x = torch.zeros(2, 64 + 8, dtype=torch.int16, device="cuda")
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    q = torch.empty(2, 32, dtype=torch.uint8, device="cuda")
    sf = torch.empty(2, 4, dtype=torch.uint8, device="cuda")
    with pytest.raises(pd.Nvfp4GemvError) as e:
        pd.nvfp4_quantize_activation(x.view(-1)[4:].data_ptr(), g, 0, q, sf, 2, 64, 0)
    assert e.value.status == pd.NVFP4_GEMV_ERR_ALIGNMENT


# ------------------------------------------------------------ GEMV fed by a bf16 activation
def run_bf16x(dA, sfA, A_scale, xbits, x_scale, rule, l, m, k):
    x = torch.from_numpy(xbits.view(np.int16).copy()).cuda()
    xs = torch.from_numpy(np.asarray(x_scale, dtype=np.float32)).cuda()
    a_s = None if A_scale is None else torch.from_numpy(np.asarray(A_scale, dtype=np.float32)).cuda()
    xq = torch.empty((l, k // 2), dtype=torch.uint8, device="cuda")
    sfx = torch.empty((l, k // 16), dtype=torch.uint8, device="cuda")
    alpha = torch.empty(l, dtype=torch.float32, device="cuda")
    c = torch.full((l, m), -1, dtype=torch.int16, device="cuda")
    pd.nvfp4_gemv_bf16x_launch(dA, sfA, a_s, x, xs, rule, xq, sfx, alpha, c, l, m, k)
    torch.cuda.synchronize()
    return (c.cpu().numpy().view(np.uint16), xq.cpu().numpy(), sfx.cpu().numpy(),
            alpha.cpu().numpy())


@pytest.mark.parametrize("name,rule", [("gaussian", pd.NVFP4_ROUND_HALF_STEP),
                                       ("decode", pd.NVFP4_ROUND_NEAREST_EVEN),
                                       ("tiny", pd.NVFP4_ROUND_NEAREST_LOWER),
                                       ("shortk", pd.NVFP4_ROUND_HALF_STEP)])
def test_bf16x_gemv_against_oracle(name, rule):
    cfg = workloads.CONFIGS[name]
    l, m, k = cfg.l, cfg.m, cfg.k
    if cfg.kind == "gaussian":
        raw = workloads.gaussian_bf16(l, m, k, seed=cfg.seed)
        ops = oq.gaussian_operands(raw, l, m, k)
        # the weights' global scales, as the amax quantiser computes them
        amax = np.maximum(np.abs(raw["A"]).max(axis=(1, 2)), np.float32(1e-8)).astype(np.float32)
        A_scale = (amax / np.float32(6.0 * 448.0)).astype(np.float32)
        xv = raw["x"]
    else:
        ops = workloads.for_config(cfg)
        A_scale = None
        xv = workloads.gaussian_bf16(l, 1, k, seed=cfg.seed + 1)["x"]
    x_scale = (np.abs(xv).max(axis=1) / np.float32(2688.0)).astype(np.float32)
    want_c, want_q, want_sf, want_alpha = oq.activation_gemv(ops["A"], ops["sfA"], A_scale, xv,
                                                             x_scale, rule, l, m, k)
    d = to_device({"A": ops["A"], "sfA": ops["sfA"]})
    c, xq, sfx, alpha = run_bf16x(d["A"], d["sfA"], A_scale, bf16_bits(xv), x_scale, rule, l, m, k)
    assert np.array_equal(sfx, want_sf) and np.array_equal(xq, want_q)
    assert np.array_equal(alpha.view(np.uint32), want_alpha.view(np.uint32))
    assert_within_tolerance(c, want_c, what=name)
    print(f"{name}: {float(np.mean(c == want_c)):.6f} of outputs bit-identical to the oracle")


@pytest.mark.parametrize("l,m,k", [(2, 300, 20480), (3, 77, 2080), (1, 9, 64), (5, 130, 16384)])
@pytest.mark.parametrize("rule", RULES)
def test_bf16x_fused_shapes(l, m, k, rule):
    """The one-kernel path (activation quantised inside the GEMV): ragged rows,
    K split across workgroups (k > 16384), K shorter than one iteration; every
    workgroup quantises the activation itself and row block 0 writes it out."""
    ops = workloads.integer_coded(l, m, k, seed=l * 1000 + m + k + rule)
    xv = workloads.gaussian_bf16(l, 1, k, seed=k + rule)["x"]
    x_scale = (np.abs(xv).max(axis=1) / np.float32(2688.0)).astype(np.float32)
    A_scale = np.linspace(0.5, 2.0, l).astype(np.float32)
    want_c, want_q, want_sf, want_alpha = oq.activation_gemv(ops["A"], ops["sfA"], A_scale, xv,
                                                             x_scale, rule, l, m, k)
    d = to_device({"A": ops["A"], "sfA": ops["sfA"]})
    c, xq, sfx, alpha = run_bf16x(d["A"], d["sfA"], A_scale, bf16_bits(xv), x_scale, rule, l, m, k)
    assert np.array_equal(sfx, want_sf) and np.array_equal(xq, want_q)
    assert np.array_equal(alpha.view(np.uint32), want_alpha.view(np.uint32))
    assert_within_tolerance(c, want_c, what=f"{(l, m, k)} rule {rule}")


def test_bf16x_misaligned_weights_take_two_kernels():
    """A weight pointer off the fast kernel's alignment: the quantiser and the
    generic GEMV run instead, with the same results."""
    l, m, k = 2, 40, 512
    ops = workloads.integer_coded(l, m, k, seed=77)
    xv = workloads.gaussian_bf16(l, 1, k, seed=78)["x"]
    x_scale = (np.abs(xv).max(axis=1) / np.float32(2688.0)).astype(np.float32)
    rule = pd.NVFP4_ROUND_NEAREST_EVEN
    want_c, want_q, want_sf, want_alpha = oq.activation_gemv(ops["A"], ops["sfA"], None, xv,
                                                             x_scale, rule, l, m, k)
    buf = torch.zeros(ops["A"].size + 8, dtype=torch.uint8, device="cuda")
    dA = buf[8:]                                   # 8-byte aligned, not 16
    dA.copy_(torch.from_numpy(ops["A"].reshape(-1)).cuda())
    dsf = torch.from_numpy(ops["sfA"].reshape(-1).copy()).cuda()
    c, xq, sfx, alpha = run_bf16x(dA, dsf, None, bf16_bits(xv), x_scale, rule, l, m, k)
    assert np.array_equal(sfx, want_sf) and np.array_equal(xq, want_q)
    assert np.array_equal(alpha.view(np.uint32), want_alpha.view(np.uint32))
    assert_within_tolerance(c, want_c, what="misaligned weights")


def run_weight(bits, groups, rows, d, rule):
    x = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).reshape(-1).copy()).cuda()
    q = torch.full((groups * rows, d // 2), 0xA5, dtype=torch.uint8, device="cuda")
    sf = torch.full((groups * rows, d // 16), 0xA5, dtype=torch.uint8, device="cuda")
    g = torch.full((groups,), -1.0, dtype=torch.float32, device="cuda")
    pd.nvfp4_quantize_weight(x, groups, rows, d, rule, q, sf, g)
    torch.cuda.synchronize()
    return (q.cpu().numpy().reshape(groups, rows, d // 2), sf.cpu().numpy().reshape(groups, rows, d // 16),
            g.cpu().numpy())


def to_bf16_bits(vals):
    """float32 -> bf16 bit patterns, round to nearest even (torch's cast)."""
    t = torch.from_numpy(np.ascontiguousarray(vals, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("rule", RULES)
@pytest.mark.parametrize("groups,rows,d", [(5, 37, 272), (8, 256, 2048), (1, 3, 16)])
def test_weight_quantizer_against_oracle(rule, groups, rows, d):
    """Per-tensor amax global scales computed on the device, then the codes:
    bytes and scales bit-identical to the oracle's amax quantiser, tensor by
    tensor; a tensor of zeros (amax floor 1e-8) and one holding a NaN (NaN
    scale, every code 0) among them."""
    rng = np.random.default_rng(groups * 100 + rows + d + rule)
    mags = np.float32(10.0) ** rng.uniform(-3, 3, size=groups).astype(np.float32)
    vals = (rng.standard_normal((groups, rows, d)).astype(np.float32) * mags[:, None, None])
    if groups > 2:
        vals[1] = 0.0
        vals[2, rows // 2, d // 3] = np.nan
    bits = to_bf16_bits(vals)
    got_q, got_sf, got_g = run_weight(bits, groups, rows, d, rule)
    for e in range(groups):
        want_q, want_sf, want_g = oq.quantize_nvfp4(bits_to_f32(bits[e]), rule)
        if np.isnan(want_g):
            assert np.isnan(got_g[e]), e
        else:
            assert got_g[e].view(np.uint32) == np.float32(want_g).view(np.uint32), (e, got_g[e], want_g)
        assert np.array_equal(got_sf[e], want_sf), f"tensor {e}: scale bytes differ"
        assert np.array_equal(got_q[e], want_q), f"tensor {e}: code bytes differ"

"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these tests needs a GPU.  Each one checks the oracle against
something other than its own formulas: values printed on the pages (the
golden files), library routines (the normal quantile function, torch's
AdamW in float64), closed forms (Adafactor's rank-1 case), invariants and
brute force on tiny inputs.
"""
import math
import os
import struct
from statistics import NormalDist

import numpy as np
import pytest

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


# ---------------------------------------------------------------------------
# Codebooks
# ---------------------------------------------------------------------------

def test_nf4_equals_normal_quantile_construction():
    """NF4 (paper abstract, Table 2) equals the QLoRA construction evaluated
    with Python's own inverse normal CDF, bit for bit after rounding."""
    nd = NormalDist()
    d = 1 - 0.5 * (1 / 30 + 1 / 32)
    pos = [nd.inv_cdf(0.5 + j * (d - 0.5) / 8) for j in range(1, 9)]
    neg = [-nd.inv_cdf(0.5 + j * (d - 0.5) / 7) for j in range(1, 8)]
    top = nd.inv_cdf(d)
    ref = np.array(sorted(neg + [0.0] + pos), np.float64) / top
    got = O.codebook(O.CB_NF4)
    assert [f32_bits(x) for x in got] == [f32_bits(np.float32(x)) for x in ref]


def test_codebook_membership():
    """Zero is in the v map of ZIP-SR and absent from the v map of ZE-EDEN
    and of the factored vectors; NF4 has 7 negative and 8 positive levels."""
    nf4 = O.codebook(O.CB_NF4)
    assert (np.diff(nf4) > 0).all()
    assert nf4[0] == -1.0 and nf4[-1] == 1.0 and nf4[7] == 0.0
    assert (nf4 < 0).sum() == 7 and (nf4 > 0).sum() == 8
    dyn4 = O.codebook(O.CB_DYN4)
    assert (np.diff(dyn4) > 0).all() and dyn4[0] == 0.0 and dyn4[-1] == 1.0
    nz = O.codebook(O.CB_DYN4_NZ)
    assert (np.diff(nz) > 0).all() and nz.min() > 0.0 and nz[-1] == 1.0 and 0.0 not in nz
    assert (nz[1:] == dyn4[1:]).all()
    lin = O.codebook(O.CB_LIN4_NZ)
    assert lin.min() > 0.0 and lin[-1] == 1.0 and (np.diff(lin) > 0).all()
    sd = O.codebook(O.CB_SDYN4)
    L, code, mid = O.sorted_levels(O.CB_SDYN4)
    assert len(L) == 15 and (np.diff(L) > 0).all() and L[0] == -1 and L[-1] == 1 and 0.0 in L
    assert np.array_equal(L, -L[::-1])                  # sign-magnitude map is symmetric
    assert set(code.tolist()) == set(range(16)) - {8}   # code "-0" never emitted
    assert sd[8] == 0.0


def test_dynamic_exponent_structure():
    """Dyn4 is a dynamic-exponent map: the number of leading zero bits of a
    code selects its decade, so each decade (0.001, 0.01], (0.01, 0.1],
    (0.1, 1] holds 1, 2, 4, 8 codes; the signed map's magnitudes are the
    3-bit version of the same map and hence a subset."""
    dyn4 = O.codebook(O.CB_DYN4)
    for c in range(1, 16):
        E = 4 - c.bit_length()
        assert 10.0 ** (-E - 1) < dyn4[c] <= 10.0 ** (-E) * (1 + 1e-6)
    counts = [sum(1 for c in range(1, 16) if 4 - c.bit_length() == E) for E in range(4)]
    assert counts == [8, 4, 2, 1]
    mags = set(np.abs(O.codebook(O.CB_SDYN4)).tolist())
    assert mags <= set(dyn4.tolist())


def test_midpoints_lie_strictly_between_levels():
    for cb in range(5):
        L, _, mid = O.sorted_levels(cb)
        assert (L[:-1] < mid).all() and (mid < L[1:]).all()


# ---------------------------------------------------------------------------
# Philox
# ---------------------------------------------------------------------------

def test_philox_known_answers():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) if l.strip()
            and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        vals = [int(x, 16) for x in r]
        out = O.philox(vals[0:4], vals[4:6])
        assert out.tolist() == vals[6:10]


def test_uniform_grid_and_sanity():
    u = np.array([O.uniform(7, 3, 11, 1, i) for i in range(40000)], np.float64)
    assert (u >= 0).all() and (u <= 1 - 2 ** -24).all()
    assert np.all(u * 2 ** 24 == np.floor(u * 2 ** 24))          # exact 24-bit grid
    assert abs(u.mean() - 0.5) < 5 * math.sqrt(1 / 12 / u.size)
    hist = np.histogram(u, bins=32, range=(0, 1))[0]
    chi2 = ((hist - u.size / 32) ** 2 / (u.size / 32)).sum()
    assert chi2 < 70  # 31 dof, p ~ 1e-4
    # element i uses word i mod 4 of the block i / 4
    w = O.philox([5, 3, 11, 1], [7, 0])
    for k in range(4):
        assert O.uniform(7, 3, 11, 1, 20 + k) == (int(w[k]) >> 8) * 2.0 ** -24


# ---------------------------------------------------------------------------
# Host scalars
# ---------------------------------------------------------------------------

def test_host_scalars_closed_form():
    hp = O.HParams(lr=1e-3, beta1=0.9, beta2=0.999, weight_decay=0.1, step=1)
    decay, step_size, rsbc2, omb1, omb2 = O.host_scalars(hp).tolist()
    assert decay == np.float32(1 - 1e-4)
    b1, b2, lr = float(np.float32(0.9)), float(np.float32(0.999)), float(np.float32(1e-3))
    assert step_size == pytest.approx(lr / (1 - b1), rel=1e-7)
    assert rsbc2 == pytest.approx(1 / math.sqrt(1 - b2), rel=1e-7)
    assert omb1 == np.float32(1) - np.float32(0.9) and omb2 == np.float32(1) - np.float32(0.999)
    big = O.host_scalars(O.HParams(step=10 ** 7)).tolist()
    assert big[1] == pytest.approx(1e-3, rel=1e-6) and big[2] == pytest.approx(1.0, rel=1e-6)


# ---------------------------------------------------------------------------
# Table 1: the four rules on the cell next to zero
# ---------------------------------------------------------------------------

def _table1_quantities(rule, eps, b=1e-3, vt=0.3e-3, beta2=0.999):
    p_up = O.cell_prob_up(rule, 0.0, b, vt, eps)
    g2 = eps * eps

    def r_next(q):
        return 1.0 / (math.sqrt(beta2 * q + (1 - beta2) * g2) + eps)

    p0 = 1.0 - p_up
    dv = p_up * b - vt
    dr = p0 * r_next(0.0) + p_up * r_next(b) - r_next(vt)
    return p0, dv, dr


def test_table1_rounding_rules_limits():
    rows = {l.split()[0]: l.split()[1:] for l in open(os.path.join(GOLDEN, "table1_rounding_rules.txt"))
            if l.strip() and not l.startswith("#")}
    b, vt = 1e-3, 0.3e-3
    rules = {"State-RTN": O.STATE_RTN, "State-SR": O.STATE_SR, "Update-RTN": O.UPDATE_RTN,
             "Update-SR": O.UPDATE_SR}
    epss = [1e-8, 1e-9, 1e-10]
    for name, rule in rules.items():
        p0_c, dv_c, dr_c = rows[name]
        q = [_table1_quantities(rule, e, b, vt) for e in epss]
        p0 = [x[0] for x in q]
        dv = [x[1] for x in q]
        dr = [x[2] for x in q]
        # P(Q = 0)
        if p0_c == "one":
            assert all(x == 1.0 for x in p0)
        elif p0_c == "zero":
            assert all(x == 0.0 for x in p0)
        elif p0_c == "1-v/b":
            assert all(abs(x - (1 - vt / b)) < 1e-12 for x in p0)
        elif p0_c == "theta_eps":
            ratio = [x / e for x, e in zip(p0, epss)]
            assert ratio[-1] > 0 and abs(ratio[-1] / ratio[-2] - 1) < 1e-3
        # state error
        if dv_c == "-v":
            assert all(x == pytest.approx(-vt, rel=1e-12) for x in dv)
        elif dv_c == "zero":
            assert all(abs(x) < 1e-15 for x in dv)
        elif dv_c == "b-v":
            assert all(x == pytest.approx(b - vt, rel=1e-12) for x in dv)
        elif dv_c == "b-v-theta_eps":
            gap = [(b - vt - x) / e for x, e in zip(dv, epss)]
            assert gap[-1] > 0 and abs(gap[-1] / gap[-2] - 1) < 1e-3
        # preconditioner error
        if dr_c == "+inv_eps":
            scaled = [x * e for x, e in zip(dr, epss)]
            assert scaled[-1] > 0.1 and abs(scaled[-1] / scaled[-2] - 1) < 1e-2
        elif dr_c == "-one":
            assert dr[-1] < 0 and abs(dr[-1] / dr[-2] - 1) < 1e-2 and abs(dr[-1]) < 1e3


def test_cell_decision_matches_probability():
    """The division-free FP32 decision of each SR rule rounds up on the
    fraction of the 2^24 uniform grid that the rule's probability says."""
    for rule, (lo, hi, s, v, eps) in [(O.UPDATE_SR, (0.2125, 0.325, 1.0, 0.25, 1e-8)),
                                      (O.UPDATE_SR, (0.0, 0.001, 1.0, 1e-9, 1e-8)),
                                      (O.STATE_SR, (0.2125, 0.325, 1.0, 0.25, 1e-8))]:
        x = np.float32(v / s)
        sv = np.float32(math.sqrt(np.float32(v)))
        # monotone in u: binary search for the first grid point that rounds down
        a, z = 0, 2 ** 24
        while a < z:
            k = (a + z) // 2
            if O.cell_round(rule, x, lo, hi, s, sv, eps, k * 2.0 ** -24):
                a = k + 1
            else:
                z = k
        frac = a / 2 ** 24
        p = O.cell_prob_up(rule, lo * s, hi * s, float(np.float32(v)), eps)
        assert abs(frac - p) < 1e-5


# ---------------------------------------------------------------------------
# Unbiasedness of preconditioner-space SR (10^6 draws on one cell)
# ---------------------------------------------------------------------------

def _draws(rule, vt, eps_sr, n_draws=10 ** 6):
    """Crafted blocks: element 0 holds 1.0 (the block max, so s = 1 and the
    element sits on the top level) and the other 127 hold the test value."""
    cb = O.CB_DYN4
    L = O.codebook(cb)
    per = O.BLOCK - 1
    nblk = -(-n_draws // per)
    v1 = np.full(O.BLOCK, vt, np.float32)
    v1[0] = 1.0
    got = []
    for b in range(nblk):
        codes, s = O.requant_v_block(cb, rule, 0, v1, eps_sr=eps_sr, seed=1, step=1, tensor_id=3,
                                     elem0=b * O.BLOCK)
        assert s == 1.0
        c = O.unpack(codes, O.BLOCK)
        assert c[0] == 15
        got.append(L[c[1:]])
    q = np.concatenate(got)[:n_draws].astype(np.float64)
    return q


@pytest.mark.parametrize("vt", [1e-9, 0.25])
def test_update_sr_unbiased_in_preconditioner_space(vt):
    eps = 1e-8
    q = _draws(O.UPDATE_SR, vt, eps)
    r = 1.0 / (np.sqrt(q) + eps)
    vt32 = float(np.float32(vt))
    r_true = 1.0 / (math.sqrt(vt32) + eps)
    L = O.codebook(O.CB_DYN4).astype(np.float64)
    lo = L[L <= vt32].max()
    hi = L[L > vt32].min()
    rlo, rhi = 1 / (math.sqrt(lo) + eps), 1 / (math.sqrt(hi) + eps)
    p = (rlo - r_true) / (rlo - rhi)
    se = (rlo - rhi) * math.sqrt(p * (1 - p) / q.size)
    assert abs(r.mean() - r_true) <= 5 * se
    # the same draws are biased in state space (towards the upper level)
    se_v = (hi - lo) * math.sqrt(p * (1 - p) / q.size)
    assert q.mean() - vt32 > 5 * se_v


def test_state_sr_unbiased_in_state_not_in_preconditioner():
    eps, vt = 1e-8, 0.25
    q = _draws(O.STATE_SR, vt, eps)
    vt32 = float(np.float32(vt))
    lo, hi = 0.2125, 0.325
    p = (vt32 - lo) / (hi - lo)
    se_v = (hi - lo) * math.sqrt(p * (1 - p) / q.size)
    assert abs(q.mean() - vt32) <= 5 * se_v
    r = 1.0 / (np.sqrt(q) + eps)
    rlo, rhi = 1 / math.sqrt(lo), 1 / math.sqrt(hi)
    se_r = (rlo - rhi) * math.sqrt(p * (1 - p) / q.size)
    assert r.mean() - 1 / math.sqrt(vt32) > 5 * se_r  # Jensen: biased upwards in r


def test_zero_cell_update_sr_rarely_stores_zero():
    """The news article and the abstract: preconditioner-space SR makes a tiny
    positive v less likely to be stored as zero than state-space rounding."""
    eps, vt = 1e-8, 1e-7
    z_upd = (_draws(O.UPDATE_SR, vt, eps, 127 * 400) == 0).mean()
    z_ssr = (_draws(O.STATE_SR, vt, eps, 127 * 400) == 0).mean()
    z_rtn = (_draws(O.STATE_RTN, vt, eps, 127 * 40) == 0).mean()
    assert z_upd < z_ssr < z_rtn == 1.0


# ---------------------------------------------------------------------------
# RTN, state-space SR, EDEN, packing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("cb,moment", [(O.CB_NF4, "m"), (O.CB_SDYN4, "m"), (O.CB_DYN4, "v"),
                                       (O.CB_DYN4_NZ, "v"), (O.CB_LIN4_NZ, "v")])
def test_rtn_ties_go_to_the_lower_level(cb, moment):
    """Reading of round-to-nearest ties (the pages fix none): a normalized
    value equal to the FP32 midpoint (L_k + L_k+1) * 0.5 stores level k, and
    the next float above it stores level k + 1."""
    L, code, mid = O.sorted_levels(cb)
    for k, md in enumerate(mid):
        above = np.nextafter(md, np.float32(2))
        vals = np.array([1.0, md, above], np.float32)   # the block max is 1, so x = value
        if moment == "m":
            codes, s = O.requant_m_block(cb, O.STATE_RTN, vals)
        else:
            codes, s = O.requant_v_block(cb, O.STATE_RTN, 0, vals)
        assert s == 1.0
        got = O.unpack(codes, 3)
        assert got[1] == code[k] and got[2] == code[k + 1], (k, md)


@pytest.mark.parametrize("cb", [O.CB_NF4, O.CB_SDYN4])
def test_m_rtn_is_nearest_level(cb):
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.uniform(-1, 1, 20000), O.sorted_levels(cb)[2],
                         np.nextafter(O.sorted_levels(cb)[2], 2), np.nextafter(O.sorted_levels(cb)[2], -2)])
    xs = xs.astype(np.float32)
    dec = O.codebook(cb)
    L = O.sorted_levels(cb)[0].astype(np.float64)
    for i in range(0, xs.size, 127):
        chunk = xs[i:i + 127]
        m1 = np.concatenate([[1.0], chunk]).astype(np.float32)
        codes, s = O.requant_m_block(cb, O.STATE_RTN, m1)
        assert s == 1.0
        got = dec[O.unpack(codes, m1.size)[1:]].astype(np.float64)
        x = chunk.astype(np.float64)
        best = np.abs(x[:, None] - L[None, :]).min(axis=1)
        err = np.abs(x - got)
        assert (err <= best + 1e-7).all()


def test_m_state_sr_unbiased_and_rtn_error_smaller():
    """NF4-SR (LM-head rule, paper Table 2) is unbiased in state space and its
    per-element error is never below RTN's (direction of Table 11)."""
    cb = O.CB_NF4
    dec = O.codebook(cb)
    x = np.float32(0.3)
    tot, n = 0.0, 0
    for b in range(2000):
        m1 = np.full(O.BLOCK, x, np.float32)
        m1[0] = -1.0
        codes, s = O.requant_m_block(cb, O.STATE_SR, m1, seed=5, step=2, tensor_id=1, elem0=b * 128)
        q = dec[O.unpack(codes, O.BLOCK)[1:]].astype(np.float64)
        tot += q.sum()
        n += q.size
    lo, hi = 0.24611226, 0.33791512
    p = (0.3 - lo) / (hi - lo)
    se = (hi - lo) * math.sqrt(p * (1 - p) / n)
    assert abs(tot / n - 0.3) < 5 * se
    rng = np.random.default_rng(1)
    m1 = rng.uniform(-1, 1, O.BLOCK).astype(np.float32)
    m1[0] = 1.0
    c_rtn, _ = O.requant_m_block(cb, O.STATE_RTN, m1)
    c_sr, _ = O.requant_m_block(cb, O.STATE_SR, m1, seed=9)
    e_rtn = np.abs(m1 - dec[O.unpack(c_rtn, O.BLOCK)])
    e_sr = np.abs(m1 - dec[O.unpack(c_sr, O.BLOCK)])
    assert (e_rtn <= e_sr).all() and (e_rtn < e_sr).any()


def test_eden_rescale_invariant():
    rng = np.random.default_rng(2)
    L = O.codebook(O.CB_DYN4_NZ)
    for trial in range(50):
        n = int(rng.integers(1, 129))
        v1 = (rng.standard_t(3, n) * 1e-3).astype(np.float32) ** 2
        codes, sc = O.requant_v_block(O.CB_DYN4_NZ, O.STATE_RTN, 1, v1)
        codes0, s = O.requant_v_block(O.CB_DYN4_NZ, O.STATE_RTN, 0, v1)
        assert np.array_equal(codes, codes0)           # EDEN leaves the RTN codes alone
        q = L[O.unpack(codes, n)].astype(np.float64)
        x = np.minimum(v1.astype(np.float64) / float(s), 1.0)
        S = float(sc) / float(s)
        assert np.dot(x, S * q) == pytest.approx(np.dot(x, x), rel=2e-5)
    # a block already on the levels needs no rescale
    v1 = L[[15, 3, 7, 0, 9]].copy()
    codes, sc = O.requant_v_block(O.CB_DYN4_NZ, O.STATE_RTN, 1, v1)
    assert sc == 1.0


def test_nibble_order_and_zero_blocks():
    L = O.codebook(O.CB_NF4)
    codes, s = O.requant_m_block(O.CB_NF4, O.STATE_RTN, L.copy())
    assert s == 1.0 and codes.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    codes, s = O.requant_m_block(O.CB_NF4, O.STATE_RTN, L[:3].copy())   # odd length: high nibble 0
    assert codes.tolist() == [0x10, 0x02] or codes[-1] >> 4 == 0
    z = np.zeros(128, np.float32)
    codes, s = O.requant_m_block(O.CB_NF4, O.STATE_RTN, z)
    assert s == 0.0 and (codes == 0x77).all()
    for cb, rule, eden in [(O.CB_DYN4, O.UPDATE_SR, 0), (O.CB_DYN4_NZ, O.STATE_RTN, 1)]:
        codes, s = O.requant_v_block(cb, rule, eden, z)
        assert s == 0.0 and (codes == 0).all()


# ---------------------------------------------------------------------------
# Factored second moment: Adafactor's rank-1 case
# ---------------------------------------------------------------------------

def _bf16_bits(x: np.ndarray) -> np.ndarray:
    b = x.astype(np.float32).view(np.uint32)
    assert ((b & 0xFFFF) == 0).all()
    return (b >> 16).astype(np.uint16)


def test_factored_rank_one_exact():
    rows, cols = 6, 10
    a = np.array([1, -2, 3, 0.5, -1.5, 4], np.float64) * 2.0 ** -12
    bb = np.array([1, 2, -3, 0.25, 5, -6, 7, 1.5, -0.75, 3], np.float64) * 2.0 ** -8
    g = np.outer(a, bb)
    gb = _bf16_bits(g)
    cfg = O.Config.of(O.FACTORED)
    st = O.TensorState(cfg, (rows, cols), tensor_id=0)
    p = np.zeros(rows * cols, np.float32)
    b2 = float(np.float32(0.999))
    for t, expect in [(1, 1 - b2), (2, 1 - b2 ** 2)]:
        st.step(O.HParams(step=t), p, gb.reshape(-1))
        _, v = st.dequant()
        ref = expect * (g ** 2).reshape(-1)
        assert np.allclose(v, ref, rtol=1e-5, atol=0)


# ---------------------------------------------------------------------------
# Quantization off: dense FP32 AdamW
# ---------------------------------------------------------------------------

def _workload_host(w, steps):
    import torch
    params = [p.numpy().reshape(-1).copy() for p in w.init_params("cpu")]
    consts = w._tensor_consts("cpu")
    grads = [[g.view(torch.uint16).numpy().reshape(-1).copy() for g in w.grads(t, "cpu", consts)]
             for t in range(1, steps + 1)]
    return params, grads


def test_fp32_recipe_matches_torch_adamw_float64():
    import torch
    from bit_adamw_update_amd import inputs
    w = inputs.custom([(1000,), (37, 29)], grad_kind="masked", seed=3)
    steps = 10
    params, grads = _workload_host(w, steps)
    cfg = O.Config.of(O.FP32)
    hpk = w.hp
    states = [O.TensorState(cfg, t.shape, t.tensor_id) for t in w.tensors]
    p_or = [p.copy() for p in params]
    tp = [torch.nn.Parameter(torch.from_numpy(p.astype(np.float64))) for p in params]
    f = {k: float(np.float32(v)) for k, v in hpk.items()}   # the FP32 values the oracle computes with
    opt = torch.optim.AdamW(tp, lr=f["lr"], betas=(f["beta1"], f["beta2"]), eps=f["eps"],
                            weight_decay=f["weight_decay"], foreach=False)
    for t in range(1, steps + 1):
        hp = O.HParams(step=t, **hpk)
        for i, st in enumerate(states):
            st.step(hp, p_or[i], grads[t - 1][i])
            g64 = (grads[t - 1][i].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
            tp[i].grad = torch.from_numpy(g64)
        opt.step()
    for i in range(len(states)):
        ref = tp[i].detach().numpy()
        scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
        assert (np.abs(p_or[i] - ref) / scale).max() < 2e-6
        s = opt.state[tp[i]]
        for mine, ref in ((states[i].m32, s["exp_avg"].numpy()), (states[i].v32, s["exp_avg_sq"].numpy())):
            sc = np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
            assert (np.abs(mine - ref) / sc).max() < 2e-6


@pytest.mark.parametrize("recipe", [O.ZIP_SR, O.ZE_EDEN, O.FACTORED])
def test_quantized_first_step_equals_fp32_step(recipe):
    """From the zero state the decoded moments are exactly 0, so the first
    quantized step updates the weights exactly as FP32 AdamW does (for a
    factored matrix only the vectors keep an elementwise v, so only they do)."""
    from bit_adamw_update_amd import inputs
    w = inputs.custom([(1000,), (24, 40)], grad_kind="masked", seed=4)
    params, grads = _workload_host(w, 1)
    hp = O.HParams(step=1, **w.hp)
    for i, t in enumerate(w.tensors):
        if recipe == O.FACTORED and len(t.shape) > 1:
            continue
        a, b = params[i].copy(), params[i].copy()
        O.TensorState(O.Config.of(recipe), t.shape, t.tensor_id).step(hp, a, grads[0][i])
        O.TensorState(O.Config.of(O.FP32), t.shape, t.tensor_id).step(hp, b, grads[0][i])
        assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ---------------------------------------------------------------------------
# Storage, windows, LM-head phase
# ---------------------------------------------------------------------------

def test_state_bytes_match_pages():
    fig = dict(l.split() for l in open(os.path.join(GOLDEN, "storage_figures.txt")) if l.strip()
               and not l.startswith("#"))
    n = 128 * 1000
    for recipe in (O.ZIP_SR, O.ZE_EDEN):
        q, meta, tot = O.state_bytes(recipe, n, n, False)
        assert q == n and tot / n == float(fig["bytes_per_param_4bit"])
    _, _, tot32 = O.state_bytes(O.FP32, n, n, False)
    assert tot32 / n == float(fig["bytes_per_param_fp32_two_buffers"])
    assert round(tot32 / tot, 2) == float(fig["reduction"])


def test_windows_equal_whole_tensor():
    """Blocks are parameter-local and the uniforms are keyed on the element
    index, so stepping a tensor in block-aligned pieces changes nothing."""
    from bit_adamw_update_amd import inputs
    w = inputs.custom([(1000,)], grad_kind="masked", seed=5)
    params, grads = _workload_host(w, 3)
    for recipe in (O.ZIP_SR, O.ZE_EDEN):
        cfg = O.Config.of(recipe)
        whole = O.TensorState(cfg, (1000,), 0)
        pw = params[0].copy()
        parts = O.TensorState(cfg, (1000,), 0)
        pp = params[0].copy()
        for t in range(1, 4):
            hp = O.HParams(step=t, **w.hp)
            whole.step(hp, pw, grads[t - 1][0])
            for lo, hi in [(0, 512), (512, 1000)]:
                O.step_window(cfg, hp, tensor_id=0, flags=0, numel=1000, base=lo, param=pp[lo:hi],
                              grad=grads[t - 1][0][lo:hi], m_codes=parts.m_codes[lo // 2:(hi + 1) // 2],
                              m_scales=parts.m_scales[lo // 128:], v_codes=parts.v_codes[lo // 2:(hi + 1) // 2],
                              v_scales=parts.v_scales[lo // 128:])
        assert np.array_equal(pw, pp)
        assert np.array_equal(whole.m_codes, parts.m_codes) and np.array_equal(whole.v_codes, parts.v_codes)


def test_lm_head_sr_only_in_final_phase():
    from bit_adamw_update_amd import inputs
    w = inputs.custom([(4096,)], grad_kind="masked", seed=6)
    params, grads = _workload_host(w, 2)
    cfg = O.Config.of(O.ZIP_SR)
    out = {}
    for flags, phase in [(0, 0), (0, 1), (O.TF_LM_HEAD, 0), (O.TF_LM_HEAD, 1)]:
        st = O.TensorState(cfg, (4096,), 0, flags)
        p = params[0].copy()
        for t in (1, 2):
            st.step(O.HParams(step=t, lm_head_sr=phase, **w.hp), p, grads[t - 1][0])
        out[(flags, phase)] = st.m_codes.copy()
    assert np.array_equal(out[(0, 0)], out[(0, 1)]) and np.array_equal(out[(0, 0)], out[(O.TF_LM_HEAD, 0)])
    assert not np.array_equal(out[(0, 0)], out[(O.TF_LM_HEAD, 1)])
    assert inputs.lm_head_sr_on(10, 10) == 1 and inputs.lm_head_sr_on(9, 10) == 0


# ---------------------------------------------------------------------------
# The step before: BF16 accumulation, gradient norm, clipping
# ---------------------------------------------------------------------------

def _torch_bf16_bits(x):
    import torch
    return x.to(torch.bfloat16).view(torch.uint16).numpy().copy()


def test_accumulate_bf16_matches_torch_round_to_nearest_even():
    """acc <- bf16(f32(acc) + f32(micro)) over four microbatches equals
    torch's own FP32 addition and BF16 conversion (round to nearest even),
    on random gradients and on crafted halfway cases."""
    import torch
    g = torch.Generator().manual_seed(11)
    n = 200_000
    micro = [torch.randn(n, generator=g) * torch.exp(torch.randn(n, generator=g) * 3) for _ in range(4)]
    acc = np.zeros(n, np.uint16)
    ref = None
    for k, m in enumerate(micro):
        mb = _torch_bf16_bits(m)
        O.accumulate_bf16(acc, mb, first=(k == 0))
        mt = torch.from_numpy(mb.view(np.int16)).view(torch.bfloat16)
        ref = mt.clone() if k == 0 else (ref.float() + mt.float()).to(torch.bfloat16)
        assert np.array_equal(acc, ref.view(torch.uint16).numpy())
    # halfway cases: 1 + 2^-8 rounds to 1, (1 + 2^-7) + 2^-8 rounds up to 1 + 2^-6
    a = np.array([0x3F80, 0x3F81, 0xBF80, 0x3F80], np.uint16)
    b = np.array([0x3B80, 0x3B80, 0xBB80, 0x0000], np.uint16)   # 2^-8, 2^-8, -2^-8, +0
    O.accumulate_bf16(a, b, first=False)
    ta = torch.tensor([1.0, 1.0078125, -1.0, 1.0]).to(torch.bfloat16)
    tb = torch.tensor([2 ** -8, 2 ** -8, -2 ** -8, 0.0]).to(torch.bfloat16)
    assert np.array_equal(a, (ta.float() + tb.float()).to(torch.bfloat16).view(torch.uint16).numpy())
    assert a[0] == 0x3F80 and a[1] == 0x3F82


@pytest.mark.parametrize("max_norm", [0.05, 1e9])
def test_grad_norm_and_clip_factor_match_torch(max_norm):
    """The global norm (binary64 sum of squares) and the clip factor equal
    torch.nn.utils.clip_grad_norm_ on float64 copies of the same BF16
    gradients: the norm to 1e-12, the factor to the FP32 rounding of
    torch's."""
    import torch
    g = torch.Generator().manual_seed(12)
    shapes = [(1000,), (64, 37), (5,)]
    grads = [_torch_bf16_bits(torch.randn(*s, generator=g) * 1e-3) .reshape(-1) for s in shapes]
    sq = sum(O.grad_sumsq(x) for x in grads)
    ps = []
    for x in grads:
        p = torch.nn.Parameter(torch.zeros(x.size, dtype=torch.float64))
        p.grad = torch.from_numpy((x.astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        ps.append(p)
    before = [p.grad.clone() for p in ps]
    total = float(torch.nn.utils.clip_grad_norm_(ps, max_norm))
    assert abs(np.sqrt(sq) - total) <= 1e-12 * total
    coef = float((ps[0].grad[before[0] != 0] / before[0][before[0] != 0]).mean())
    c = O.clip_factor(sq, max_norm)
    assert c == float(np.float32(coef)) or abs(c - coef) <= 2 ** -23 * coef
    if max_norm > total:
        assert c == 1.0
    else:
        assert c < 1.0
    assert O.clip_factor(sq, 0.0) == 1.0


def test_power_of_two_clip_scales_moments_exactly():
    """A clip factor of 1/2 halves g exactly, so from the zero state the
    first ZE-EDEN step writes the same codes, m scales exactly halved and v
    scales exactly quartered, and the factored row/column statistics come
    out exactly a quarter of the unclipped ones."""
    import torch
    g = torch.Generator().manual_seed(13)
    n = 4096
    grad = _torch_bf16_bits(torch.randn(n, generator=g) * 1e-3)
    outs = []
    for s in (1.0, 0.5):
        st = O.TensorState(O.Config.of(O.ZE_EDEN), (n,), 5)
        p = np.zeros(n, np.float32)
        st.step(O.HParams(step=1, grad_scale=s), p, grad)
        outs.append(st)
    a, b = outs
    assert np.array_equal(a.m_codes, b.m_codes) and np.array_equal(a.v_codes, b.v_codes)
    assert np.array_equal(a.m_scales * np.float32(0.5), b.m_scales)
    assert np.array_equal(a.v_scales * np.float32(0.25), b.v_scales)
    rows, cols = 32, 128
    gm = grad[: rows * cols]
    res = []
    for s in (1.0, 0.5):
        R = np.zeros(rows, np.float32)
        Cc = np.zeros(cols, np.float32)
        O.factored_update(O.HParams(step=1, grad_scale=s), rows, cols, gm, R, Cc)
        res.append((R, Cc))
    assert np.array_equal(res[0][0] * np.float32(0.25), res[1][0])
    assert np.array_equal(res[0][1] * np.float32(0.25), res[1][1])


def test_fp32_recipe_with_clipping_matches_torch():
    """FP32 recipe with clipping against torch: clip_grad_norm_ on float64
    gradients, then AdamW, 5 steps."""
    import torch
    from bit_adamw_update_amd import inputs
    w = inputs.custom([(1000,), (37, 29)], grad_kind="masked", seed=14)
    steps, max_norm = 5, 1e-3
    params, grads = _workload_host(w, steps)
    cfg = O.Config.of(O.FP32)
    states = [O.TensorState(cfg, t.shape, t.tensor_id) for t in w.tensors]
    p_or = [p.copy() for p in params]
    tp = [torch.nn.Parameter(torch.from_numpy(p.astype(np.float64))) for p in params]
    f = {k: float(np.float32(v)) for k, v in w.hp.items()}
    opt = torch.optim.AdamW(tp, lr=f["lr"], betas=(f["beta1"], f["beta2"]), eps=f["eps"],
                            weight_decay=f["weight_decay"], foreach=False)
    clipped = 0
    for t in range(1, steps + 1):
        sq = sum(O.grad_sumsq(x) for x in grads[t - 1])
        c = O.clip_factor(sq, max_norm)
        clipped += c < 1.0
        hp = O.HParams(step=t, grad_scale=c, **w.hp)
        for i, st in enumerate(states):
            st.step(hp, p_or[i], grads[t - 1][i])
            tp[i].grad = torch.from_numpy((grads[t - 1][i].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
        torch.nn.utils.clip_grad_norm_(tp, max_norm)
        opt.step()
    assert clipped == steps
    for i in range(len(states)):
        ref = tp[i].detach().numpy()
        scale = np.maximum(np.abs(ref), np.sqrt(np.mean(ref ** 2)))
        assert (np.abs(p_or[i] - ref) / scale).max() < 2e-6


# ---------------------------------------------------------------------------
# 8-bit blockwise AdamW
# ---------------------------------------------------------------------------

def _dyn_exact(code, bits):
    from fractions import Fraction
    if code == 0:
        return Fraction(0)
    E = bits - code.bit_length()
    F = bits - 1 - E
    f = code & ((1 << F) - 1)
    return Fraction(1, 10 ** E) * (Fraction(1, 10) + Fraction(9, 10) * Fraction(f + 1, 1 << F))


def test_8bit_maps_follow_the_dynamic_exponent_construction():
    """Dyn8 and SDyn8 equal the construction evaluated in exact rational
    arithmetic and rounded to FP32, code by code; Dyn8 is sorted by code with
    2^(7-E) levels in decade E; SDyn8 is the sign-magnitude mirror of the
    7-bit map with -0 decoding to +0."""
    d8 = O.codebook8(O.CB8_DYN8)
    s8 = O.codebook8(O.CB8_SDYN8)
    for c in range(256):
        assert d8[c] == np.float32(float(_dyn_exact(c, 8)))
        mag = np.float32(float(_dyn_exact(c & 127, 7)))
        assert s8[c] == (-mag if c & 128 and c != 128 else mag)
    assert np.all(np.diff(d8) > 0) and d8[0] == 0 and d8[255] == 1
    for E in range(8):
        lo, hi = 10.0 ** (-E - 1), 10.0 ** (-E)
        assert int(((d8 > lo * (1 + 1e-6)) & (d8 <= hi * (1 + 1e-6))).sum()) == 2 ** (7 - E)
    L, code, mid = O.sorted_levels8(O.CB8_SDYN8)
    assert len(L) == 255 and 128 not in code and np.array_equal(L, -L[::-1])
    assert np.all(L[:-1] < mid) and np.all(mid < L[1:])


def test_8bit_first_step_rounds_to_the_nearest_level_and_matches_fp32():
    """From the zero state the decoded moments are 0, so the weights equal
    the FP32 recipe's bit for bit; the stored m and v codes are the nearest
    levels (ties to the lower one) of m1 / s_m and v1 / s_v, by brute force."""
    import torch
    g = torch.Generator().manual_seed(15)
    n = 3 * 128 + 57
    grad = (torch.randn(n, generator=g) * 1e-3).to(torch.bfloat16).view(torch.uint16).numpy().copy()
    param = (torch.randn(n, generator=g) * 0.02).numpy()
    hp = O.HParams(step=1)
    st8 = O.TensorState8((n,), 3)
    p8 = param.copy()
    st8.step(hp, p8, grad)
    st32 = O.TensorState(O.Config.of(O.FP32), (n,), 3)
    p32 = param.copy()
    st32.step(hp, p32, grad)
    assert np.array_equal(p8.view(np.uint32), p32.view(np.uint32))
    for vals, codes, scales, cb, signed in ((st32.m32, st8.m_codes, st8.m_scales, O.CB8_SDYN8, True),
                                            (st32.v32, st8.v_codes, st8.v_scales, O.CB8_DYN8, False)):
        table = O.codebook8(cb)
        L, lcode, _ = O.sorted_levels8(cb)
        for b in range(len(scales)):
            blk = vals[b * 128: (b + 1) * 128]
            s = np.float32(np.abs(blk).max())
            assert scales[b] == s
            inv = np.float32(1) / s
            x = np.clip(blk * inv, -1, 1) if signed else np.minimum(blk * inv, 1)
            d = np.abs(x[:, None].astype(np.float64) - L[None, :].astype(np.float64))
            best = lcode[np.argmin(d, axis=1)]     # argmin takes the first (lower) level on a tie
            assert np.array_equal(codes[b * 128: b * 128 + blk.size], best)
            assert np.all(np.abs(table[codes[b * 128: b * 128 + blk.size]] - x) <= np.diff(L).max() / 2 + 1e-7)


def _rtn_codes(x, cb8=None, cb=None):
    """Round to nearest by brute force: the count of FP32 midpoints strictly
    below x (an exact midpoint goes to the lower level), as a code."""
    if cb8 is not None:
        L, code, mid = O.sorted_levels8(cb8)
    else:
        L, code, mid = O.sorted_levels(cb)
    idx = (x[:, None] > mid[None, :]).sum(axis=1)
    return np.asarray(code)[idx]


def test_subnormal_block_scales_follow_the_reciprocal():
    """Normalization divides a block by its scale through x = m1 * (1/s).
    A subnormal scale whose IEEE reciprocal is finite (s > 2^-128) normalizes
    exactly like any other: the codes are the nearest levels of
    x = m1 * fl(1/s), spread over the map.  A scale whose reciprocal
    overflows (s <= 2^-128) has no usable normalization (m1 * inf is
    infinite, 0 * inf is NaN), so its block stores the code of zero in every
    slot, as a zero block does.  The scale is stored as computed either way.
    4-bit and 8-bit states; the third block, of normal values, is plain."""
    import torch
    g = torch.Generator().manual_seed(61)
    x = torch.randn(384, generator=g)
    x = x / x.abs().max()
    # m1 = fl((1 - b1) g) at step 1 from the zero state: block 0 peaks near
    # 6e-39 (reciprocal finite), block 1 near 1.5e-39 (reciprocal overflows)
    grad = torch.cat([x[:128] * 6e-38, x[128:256] * 1.5e-38, x[256:] * 1e-3])
    grad = grad.to(torch.bfloat16).view(torch.uint16).numpy().copy()
    g32 = (grad.astype(np.uint32) << 16).view(np.float32)
    hp = O.HParams(step=1)
    omb1 = np.float32(1) - np.float32(hp.beta1)
    m1 = omb1 * g32                         # FP32 products, subnormals kept
    s = [np.float32(np.abs(m1[b * 128:(b + 1) * 128]).max()) for b in range(3)]
    with np.errstate(over="ignore"):
        inv = [np.float32(1) / v for v in s]
    assert 2.0 ** -128 < s[0] < 2.0 ** -126 and np.isfinite(inv[0])
    assert 0 < s[1] <= 2.0 ** -128 and np.isinf(inv[1])
    for recipe in (O.ZIP_SR, O.ZE_EDEN):
        cfg = O.Config.of(recipe)
        st = O.TensorState(cfg, (384,), 3)
        st.step(hp, np.zeros(384, np.float32), grad)
        c = O.unpack(st.m_codes, 384)
        assert [f32_bits(v) for v in st.m_scales] == [f32_bits(v) for v in s]
        x0 = np.clip(m1[:128] * inv[0], -1, 1)
        assert np.array_equal(c[:128], _rtn_codes(x0, cb=cfg.m_cb))
        assert len(set(c[:128].tolist())) > 4
        assert np.all(c[128:256] == O.zero_code(cfg.m_cb))
        assert len(set(c[256:].tolist())) > 4
    st8 = O.TensorState8((384,), 3)
    st8.step(hp, np.zeros(384, np.float32), grad)
    assert [f32_bits(v) for v in st8.m_scales] == [f32_bits(v) for v in s]
    x0 = np.clip(m1[:128] * inv[0], -1, 1)
    assert np.array_equal(st8.m_codes[:128], _rtn_codes(x0, cb8=O.CB8_SDYN8))
    assert np.all(st8.m_codes[128:256] == 0)
    assert len(set(st8.m_codes[256:].tolist())) > 4

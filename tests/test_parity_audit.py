"""The parity harness's tie audit, on the CPU: a differing code is accepted
only when it is a stochastic-rounding tie (|u den - num| within 2 FP32 ulp
of num, recomputed in binary64, and the two codes bracket the value);
round-to-nearest codes, codes outside the bracket and SR decisions far from
their threshold are rejected."""
import numpy as np

from oracle import oracle as O
from tests import parity


class _Spec:
    def __init__(self, tensor_id, flags=0):
        self.tensor_id, self.flags = tensor_id, flags


def _audit(cfg, **hp):
    return parity.Audit(cfg, O.HParams(**hp), [_Spec(5), _Spec(6, O.TF_LM_HEAD)])


def _zip_tie_block(seed, step, tid, elem, eps):
    """A block of v values (max 1.0, so x = v) whose element `elem % 128`
    lies in the zero cell [0, L_1] where the Update-SR probability of
    rounding up equals its uniform: sqrt(v) (r_hi + eps) = u r_hi (sqrt(v) +
    eps) with r_hi = sqrt(L_1); of the nearby floats the one closest to the
    threshold is taken."""
    u = O.uniform(seed, step, tid, 1, elem)
    L, _, _ = O.sorted_levels(O.CB_DYN4)
    rhi = np.sqrt(float(np.float32(L[1])))
    sv = u * rhi * eps / (rhi * (1 - u) + eps)
    v0 = np.float32(sv * sv)

    def gap(v):
        s = np.sqrt(float(v))
        return abs(u * rhi * (s + eps) - s * (rhi + eps))

    cands = [v0]
    for _ in range(4):
        cands += [np.nextafter(cands[-1], np.float32(1)), np.nextafter(cands[0], np.float32(0))]
    v = min(cands, key=gap)
    vals = np.full(128, 0.25, np.float32)
    vals[0] = 1.0
    vals[elem % 128] = v
    return vals, 0


def test_accepts_a_preconditioner_space_tie():
    cfg = O.Config.of(O.ZIP_SR)
    a = _audit(cfg, step=7, seed=3)
    elem = 128 * 4 + 77
    vals, lo = _zip_tie_block(3, 7, 5, elem, 1e-8)
    _, code, _ = O.sorted_levels(O.CB_DYN4)
    j = elem % 128
    assert a.is_tie("v", 0, elem, vals, j, int(code[lo]), int(code[lo + 1]))
    assert a.is_tie("v", 0, elem, vals, j, int(code[lo + 1]), int(code[lo]))
    # the same value with another element's uniform is far from its threshold
    assert not a.is_tie("v", 0, elem + 1, vals, j, int(code[lo]), int(code[lo + 1]))
    # codes that do not bracket the value
    assert not a.is_tie("v", 0, elem, vals, j, int(code[lo]), int(code[lo + 2]))


def test_rejects_round_to_nearest_codes():
    cfg = O.Config.of(O.ZE_EDEN)
    a = _audit(cfg, step=2)
    vals = np.linspace(0.01, 1.0, 128).astype(np.float32)
    assert not a.is_tie("v", 0, 40, vals, 40, 3, 4)
    assert not a.is_tie("m", 0, 40, vals, 40, 9, 10)


def test_state_sr_tie_on_the_lm_head_only():
    cfg = O.Config.of(O.ZIP_SR)
    step, seed, elem = 10, 0, 300
    u = O.uniform(seed, step, 6, 0, elem)
    L, code, _ = O.sorted_levels(O.CB_NF4)
    lo = 7                                            # the cell [0, L_8]: x - L_lo = x is exact
    x = np.float32(u * L[lo + 1])                     # P(up) = (x - L_lo) / (L_hi - L_lo) = u
    vals = np.zeros(128, np.float32)
    vals[0] = -1.0
    vals[elem % 128] = x
    a = _audit(cfg, step=step, seed=seed, lm_head_sr=1)
    j = elem % 128
    assert a.is_tie("m", 1, elem, vals, j, int(code[lo]), int(code[lo + 1]))
    assert not a.is_tie("m", 0, elem, vals, j, int(code[lo]), int(code[lo + 1]))   # not the LM head: RTN
    b = _audit(cfg, step=step, seed=seed, lm_head_sr=0)
    assert not b.is_tie("m", 1, elem, vals, j, int(code[lo]), int(code[lo + 1]))   # before the final phase

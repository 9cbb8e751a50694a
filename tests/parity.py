"""Parity harness: the HIP path (through the C ABI) against the CPU oracle.

Both sides consume the same seeded bytes.  After every step the harness
compares, per tensor window:
  * packed m and v codes nibble by nibble (bit-exact; an element whose code
    ever differed is remembered and excluded from the weight check),
  * block scales bit for bit,
  * master weights: |w_gpu - w_ora| / max(|w_ora|, rms(w_ora)) <= 1e-6,
  * factored row/column vectors within 1e-6 relative (binary64 sums in a
    different order on the two sides, rounded to FP32).
The fraction of differing codes must stay <= 1e-6 of all codes compared,
and every differing code must be an audited stochastic-rounding tie: from
the oracle's unquantized moment of that step, the harness recomputes the
rule's two sides in binary64 and accepts the difference only if
|u * den - num| <= 2 ulp(num) in FP32 and both codes bracket the value
(round-to-nearest and EDEN codes involve no square root and must match).
The weight tolerance is relative to max(|w|, rms of the tensor's window):
near a weight that crosses zero FP32 is accurate relative to the terms of
the update, not to the tiny result.  A non-finite value (NaN, an infinity)
must be matched exactly, by NaN or by the same infinity.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import inputs
from oracle import oracle as O

# The codebook/rule variants run on the GPU: (m codebook, v codebook, m rule,
# v rule, eden).  The first eight are the component grid of [P] Tables 1, 3
# and 8; the last two reach branches no recipe takes.
VARIANTS = [
    (q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 0),
    (q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_STATE_SR, 0),
    (q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_UPDATE_RTN, 0),
    (q4.CB_NF4, q4.CB_DYN4_NZ, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 0),
    (q4.CB_SDYN4, q4.CB_LIN4_NZ, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 0),
    (q4.CB_SDYN4, q4.CB_DYN4_NZ, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 1),
    (q4.CB_SDYN4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_UPDATE_SR, 0),
    (q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_SR, q4.RULE_UPDATE_SR, 0),
    # EDEN on the ZIP-SR kernel: its generic v branch (compact tables, EDEN
    # sums) instead of the flat-table one
    (q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_UPDATE_SR, 1),
    # m by state-space SR on every tensor in a kernel with compact tables
    (q4.CB_NF4, q4.CB_DYN4_NZ, q4.RULE_STATE_SR, q4.RULE_STATE_RTN, 1),
]

ORACLE_RECIPE = {"zip_sr": O.ZIP_SR, "ze_eden": O.ZE_EDEN, "factored": O.FACTORED, "fp32": O.FP32}
W_TOL = 1e-6
RC_TOL = 1e-6
CODE_FRAC = 1e-6


def oracle_config(recipe: str, cfg: q4.Q4Config | None = None) -> O.Config:
    if cfg is None:
        return O.Config.of(ORACLE_RECIPE[recipe])
    return O.Config(O.CUSTOM if cfg.recipe == q4.RECIPE_CUSTOM else cfg.recipe, cfg.m_codebook, cfg.v_codebook,
                    cfg.m_rule, cfg.v_rule, cfg.eden)


def unpack(codes: np.ndarray) -> np.ndarray:
    out = np.empty(2 * codes.size, np.uint8)
    out[0::2] = codes & 0x0F
    out[1::2] = codes >> 4
    return out


@dataclass
class Window:
    """Whole blocks [b0, b1) of tensor i, stepped by the oracle on the host."""
    i: int
    b0: int
    b1: int
    lo: int = 0
    hi: int = 0
    param: np.ndarray = None
    m_codes: np.ndarray = None
    m_scales: np.ndarray = None
    v_codes: np.ndarray = None
    v_scales: np.ndarray = None
    m32: np.ndarray = None
    v32: np.ndarray = None
    m_bad: np.ndarray = None
    v_bad: np.ndarray = None
    m1: np.ndarray = None       # the oracle's unquantized moments of the last step
    v1: np.ndarray = None


@dataclass
class Report:
    codes_compared: int = 0
    codes_differ: int = 0
    scales_compared: int = 0
    scales_differ: int = 0
    weights_compared: int = 0
    weights_excluded: int = 0
    max_w_err: float = 0.0
    max_rc_err: float = 0.0
    padding_nonzero: int = 0
    ties_audited: int = 0
    untied_differ: int = 0
    nonfinite_weights: int = 0   # oracle weights that are NaN or infinite (matched exactly)
    notes: list = field(default_factory=list)

    def check(self):
        assert self.padding_nonzero == 0, "a nibble past the end of an odd-length tensor is not 0"
        assert self.untied_differ == 0, \
            f"{self.untied_differ} differing codes are not stochastic-rounding ties: {self.notes[:5]}"
        assert self.scales_differ == 0, f"{self.scales_differ} of {self.scales_compared} scales differ"
        assert self.codes_differ <= CODE_FRAC * max(self.codes_compared, 1), \
            f"{self.codes_differ} of {self.codes_compared} codes differ"
        assert self.weights_excluded <= CODE_FRAC * max(self.weights_compared, 1) + self.codes_differ
        assert self.max_w_err <= W_TOL, f"max weight error {self.max_w_err:.3e}"
        assert self.max_rc_err <= RC_TOL, f"max factored R/C error {self.max_rc_err:.3e}"


def _rms(x):
    x = x[np.isfinite(x)]
    return float(np.sqrt(np.mean(x.astype(np.float64) ** 2))) if x.size else 0.0


def _rel_err(mine: np.ndarray, ref: np.ndarray, floor: float | None = None) -> np.ndarray:
    """|mine - ref| / max(|ref|, floor) per element (floor: the rms of ref's
    finite values unless given).  A non-finite ref must be matched exactly
    (NaN by NaN, an infinity by the same infinity) and a finite ref by a
    finite value: otherwise the error is inf."""
    x, r = mine.astype(np.float64), ref.astype(np.float64)
    fin_r, fin_x = np.isfinite(r), np.isfinite(x)
    same = (np.isnan(x) & np.isnan(r)) | (np.isinf(r) & (x == r))
    sc = np.maximum(np.abs(r), _rms(ref) if floor is None else floor)
    sc[~(sc > 0)] = 1.0
    with np.errstate(invalid="ignore", over="ignore"):
        err = np.where(fin_r & fin_x, np.abs(x - r) / sc, 0.0)
    err[~same & ~(fin_r & fin_x)] = np.inf
    return err


def run(workload: inputs.Workload, recipe: str, steps: int, *, windows=None, device="cuda",
        cfg: q4.Q4Config | None = None, grads_on: str = "cpu", lm_head_phase: bool = False,
        hp: dict | None = None, check_every_step: bool = True, step_offset: int = 0) -> Report:
    """Run `steps` steps on both sides and compare.  windows=None compares
    every element of every tensor; otherwise a list of (i, b0, b1).  The
    step counts are step_offset + 1 .. step_offset + steps (the gradients
    are those of steps 1 .. steps)."""
    dev = torch.device(device)
    hpk = dict(workload.hp)
    if hp:
        hpk.update(hp)
    specs = workload.tensors
    params = workload.init_params(grads_on)
    consts = workload._tensor_consts(grads_on)
    gp = [p.to(dev).reshape(-1).contiguous() for p in params]
    st = q4.Q4State(recipe, specs, device=dev, cfg=cfg)
    ocfg = oracle_config(recipe, cfg)
    fp32 = recipe == "fp32"
    full = windows is None
    if full:
        windows = [(i, 0, (t.numel + 127) // 128) for i, t in enumerate(specs)]
    wins = []
    for (i, b0, b1) in windows:
        t = specs[i]
        w = Window(i, b0, b1)
        w.lo, w.hi = 128 * b0, min(128 * b1, t.numel)
        w.param = params[i].reshape(-1)[w.lo:w.hi].cpu().numpy().copy()
        n = w.hi - w.lo
        nb = b1 - b0
        if fp32:
            w.m32 = np.zeros(n, np.float32)
            w.v32 = np.zeros(n, np.float32)
        else:
            zm = O.zero_code(ocfg.m_cb)
            w.m_codes = np.full((n + 1) // 2, zm | (zm << 4), np.uint8)
            if n % 2:
                w.m_codes[-1] = zm
            w.m_scales = np.zeros(nb, np.float32)
            if not (recipe == "factored" and len(t.shape) >= 2):
                zv = O.zero_code(ocfg.v_cb)
                w.v_codes = np.full((n + 1) // 2, zv | (zv << 4), np.uint8)
                if n % 2:
                    w.v_codes[-1] = zv
                w.v_scales = np.zeros(nb, np.float32)
        w.m_bad = np.zeros(n, bool)
        w.v_bad = np.zeros(n, bool)
        w.m1 = np.zeros(n, np.float32)
        w.v1 = np.zeros(n, np.float32)
        wins.append(w)
    # factored matrices: the oracle keeps full R and C
    fact = {}
    if recipe == "factored":
        for i, t in enumerate(specs):
            if len(t.shape) >= 2 and t.numel > 0:
                fact[i] = (np.zeros(t.shape[0], np.float32), np.zeros(t.numel // t.shape[0], np.float32))
    rep = Report()
    for k in range(1, steps + 1):
        step = step_offset + k
        phase = inputs.lm_head_sr_on(k, steps) if lm_head_phase else 0
        grads = workload.grads(k, grads_on, consts)
        gg = [g.to(dev).reshape(-1).contiguous() for g in grads]
        st.step(gp, gg, step, lm_head_sr=phase, **hpk)
        ohp = O.HParams(step=step, lm_head_sr=phase, **hpk)
        inv = {}
        for i, (R, Cc) in fact.items():
            t = specs[i]
            gfull = grads[i].reshape(-1).view(torch.uint16).cpu().numpy()
            inv[i] = O.factored_update(ohp, t.shape[0], t.numel // t.shape[0], gfull, R, Cc)
        for w in wins:
            t = specs[w.i]
            gw = grads[w.i].reshape(-1)[w.lo:w.hi].view(torch.uint16).cpu().numpy().copy()
            kw = dict(tensor_id=t.tensor_id, flags=t.flags, numel=t.numel, base=w.lo, param=w.param, grad=gw,
                      m_codes=w.m_codes, m_scales=w.m_scales, v_codes=w.v_codes, v_scales=w.v_scales,
                      m32=w.m32, v32=w.v32, m1_out=w.m1, v1_out=w.v1)
            if w.i in fact:
                R, Cc = fact[w.i]
                kw.update(cols=t.numel // t.shape[0], R=R, Cc=Cc, inv_meanR=inv[w.i])
            O.step_window(ocfg, ohp, **kw)
        if check_every_step or k == steps:
            torch.cuda.synchronize()
            _compare(st, gp, wins, fact, rep, fp32, Audit(ocfg, ohp, specs))
    return rep


def _ulp32(x: float) -> float:
    return float(np.spacing(np.float32(abs(x))))


class Audit:
    """Decides whether a code that differs between the GPU and the oracle is
    a stochastic-rounding tie, from the oracle's unquantized moment m1 or v1
    of the step just compared (recomputed in binary64 here)."""

    def __init__(self, ocfg: O.Config, ohp: O.HParams, specs):
        self.cfg, self.hp, self.specs = ocfg, ohp, specs
        self.eps_sr = ohp.eps if ohp.eps_sr is None else ohp.eps_sr

    def _rule(self, moment: str, ti: int) -> int:
        if moment == "v":
            return self.cfg.v_rule
        lm_sr = (self.specs[ti].flags & O.TF_LM_HEAD) and self.hp.lm_head_sr
        return O.STATE_SR if (lm_sr or self.cfg.m_rule == O.STATE_SR) else O.STATE_RTN

    def is_tie(self, moment: str, ti: int, elem: int, vals: np.ndarray, j: int, code_gpu: int,
               code_ora: int) -> bool:
        """vals: the window's unquantized moments (FP32), j the element's
        index in the window, elem its index in the tensor."""
        rule = self._rule(moment, ti)
        if rule in (O.STATE_RTN, O.UPDATE_RTN):
            return False
        b0 = (j // 128) * 128
        blk = vals[b0:b0 + 128].astype(np.float32)
        blk = blk[~np.isnan(blk)]   # the block maximum skips NaN
        if blk.size == 0 or not np.isfinite(vals[j]):
            return False
        s = np.float32(np.abs(blk).max()) if moment == "m" else np.float32(blk.max())
        with np.errstate(over="ignore", divide="ignore"):
            inv = np.float32(1) / s if s > 0 else np.float32(0)
        if not np.isfinite(inv):
            return False
        x = np.float32(vals[j]) * inv
        x = np.float32(min(max(x, -1.0), 1.0)) if moment == "m" else np.float32(min(x, 1.0))
        L, code, _ = O.sorted_levels(self.cfg.m_cb if moment == "m" else self.cfg.v_cb)
        lo = int(np.max(np.nonzero(L <= x)[0])) if np.any(L <= x) else 0
        if lo + 1 >= L.size or L[lo] == x:
            return False
        if {code_gpu, code_ora} != {int(code[lo]), int(code[lo + 1])}:
            return False   # not the two levels that bracket the value
        u = O.uniform(self.hp.seed, self.hp.step, self.specs[ti].tensor_id, 0 if moment == "m" else 1, elem)
        if rule == O.STATE_SR:
            num, den = float(x) - float(L[lo]), float(L[lo + 1]) - float(L[lo])
        else:   # preconditioner-space SR, in binary64 from the FP32 inputs
            a_lo, a_hi = np.float32(L[lo]) * s, np.float32(L[lo + 1]) * s
            rlo, rhi, sv = np.sqrt(float(a_lo)), np.sqrt(float(a_hi)), np.sqrt(float(vals[j]))
            num = (sv - rlo) * (rhi + self.eps_sr)
            den = (rhi - rlo) * (sv + self.eps_sr)
        return abs(u * den - num) <= 2 * _ulp32(num)


def _audit(rep: Report, audit: Audit, moment: str, w: "Window", gcodes, ocodes, diff):
    vals = w.m1 if moment == "m" else w.v1
    for j in np.nonzero(diff)[0]:
        if audit.is_tie(moment, w.i, w.lo + int(j), vals, int(j), int(gcodes[j]), int(ocodes[j])):
            rep.ties_audited += 1
        else:
            rep.untied_differ += 1
            rep.notes.append((moment, w.i, w.lo + int(j), int(gcodes[j]), int(ocodes[j])))


def _compare(st, gp, wins, fact, rep: Report, fp32: bool, audit: Audit):
    for w in wins:
        b = st.bufs[w.i]
        n = w.hi - w.lo
        if fp32:
            for mine, ref in ((b.m32[w.lo:w.hi], w.m32), (b.v32[w.lo:w.hi], w.v32)):
                x = mine.cpu().numpy()
                rep.max_w_err = max(rep.max_w_err, float(_rel_err(x, ref).max()) if n else 0.0)
        else:
            cl, ch = w.lo // 2, (w.hi + 1) // 2
            if w.hi == b.numel and b.numel % 2 == 1:
                # the header fixes the high nibble of the last byte to 0
                for codes in (b.m_codes, b.v_codes):
                    if codes is not None:
                        rep.padding_nonzero += int(codes[-1].item() >> 4 != 0)
            gm = unpack(b.m_codes[cl:ch].cpu().numpy())[:n]
            om = unpack(w.m_codes)[:n]
            dm = gm != om
            w.m_bad |= dm
            rep.codes_compared += n
            rep.codes_differ += int(dm.sum())
            if dm.any():
                _audit(rep, audit, "m", w, gm, om, dm)
            gs = b.m_scales[w.b0:w.b1].cpu().numpy()
            rep.scales_compared += gs.size
            rep.scales_differ += int((gs.view(np.uint32) != w.m_scales.view(np.uint32)).sum())
            if w.v_codes is not None:
                gv = unpack(b.v_codes[cl:ch].cpu().numpy())[:n]
                ov = unpack(w.v_codes)[:n]
                dv = gv != ov
                w.v_bad |= dv
                rep.codes_compared += n
                rep.codes_differ += int(dv.sum())
                if dv.any():
                    _audit(rep, audit, "v", w, gv, ov, dv)
                gs = b.v_scales[w.b0:w.b1].cpu().numpy()
                rep.scales_compared += gs.size
                rep.scales_differ += int((gs.view(np.uint32) != w.v_scales.view(np.uint32)).sum())
        pw = gp[w.i][w.lo:w.hi].cpu().numpy()
        rep.nonfinite_weights += int((~np.isfinite(w.param)).sum())
        ok = ~(w.m_bad | w.v_bad)
        rep.weights_compared += n
        rep.weights_excluded += int((~ok).sum())
        if ok.any():
            err = _rel_err(pw, w.param)[ok]
            rep.max_w_err = max(rep.max_w_err, float(err.max()))
    for i, (R, Cc) in fact.items():
        b = st.bufs[i]
        for mine, ref in ((b.v_row, R), (b.v_col, Cc)):
            x = mine.cpu().numpy()
            rep.max_rc_err = max(rep.max_rc_err, float(_rel_err(x, ref, floor=1e-30).max()))


def sample_windows(workload: inputs.Workload, n_random: int = 48, seed: int = 0, blocks_per_window: int = 8):
    """Block windows for a full-size workload: the first and last blocks of
    every tensor, plus random interior windows."""
    rng = np.random.default_rng(seed)
    out = []
    for i, t in enumerate(workload.tensors):
        nb = (t.numel + 127) // 128
        out.append((i, 0, min(nb, 4)))
        if nb > 4:
            out.append((i, max(4, nb - 4), nb))
    big = [i for i, t in enumerate(workload.tensors) if (t.numel + 127) // 128 > 64]
    for _ in range(n_random):
        i = int(rng.choice(big))
        nb = (workload.tensors[i].numel + 127) // 128
        b0 = int(rng.integers(4, nb - 4 - blocks_per_window))
        out.append((i, b0, b0 + blocks_per_window))
    # merge overlaps per tensor
    merged = {}
    for i, b0, b1 in out:
        merged.setdefault(i, []).append((b0, b1))
    res = []
    for i, segs in merged.items():
        segs.sort()
        cur = list(segs[0])
        for b0, b1 in segs[1:]:
            if b0 <= cur[1]:
                cur[1] = max(cur[1], b1)
            else:
                res.append((i, cur[0], cur[1]))
                cur = [b0, b1]
        res.append((i, cur[0], cur[1]))
    return res

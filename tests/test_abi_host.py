"""Host-only checks of the C ABI library: it loads, exports every symbol the
header declares, and its host logic (validation, workspace and state-byte
arithmetic, headers, host scalars, codebook tables) behaves as documented.
No call here launches GPU work."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import bit_adamw_update_amd as q4
from bit_adamw_update_amd import api, build
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module", autouse=True)
def lib():
    if not os.path.exists(build.LIB_PATH):
        build.build(force=False)
    return api.load_library()


def header_functions():
    src = open(os.path.join(ROOT, "include", "q4adamw.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(q4adamw_[a-z_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    # and the shared object really exports them (dynamic symbol table)
    out = os.popen(f"nm -D --defined-only {build.LIB_PATH}").read()
    for n in names:
        assert re.search(rf"\bT {n}\b", out), n


def test_every_header_is_served_by_a_library():
    """Each header under include/ names the functions of one library, which
    loads on this host and exports all of them."""
    import ctypes
    libs = {"q4adamw.h": build.LIB_PATH, "q4probe.h": build.PROBE_PATH}
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == sorted(libs), headers
    for h in headers:
        if not os.path.exists(libs[h]):
            build.build(force=False)
        src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", h)).read(), flags=re.S)
        names = sorted(set(re.findall(r"\b(q4[a-z]+_[a-z0-9_]+)\s*\(", src)))
        assert names, h
        so = ctypes.CDLL(libs[h])
        out = os.popen(f"nm -D --defined-only {libs[h]}").read()
        for n in names:
            assert hasattr(so, n) and re.search(rf"\bT {n}\b", out), (h, n)


def test_abi_version_and_status_strings():
    assert q4.q4adamw_abi_version() == 3 == q4.api.ABI_VERSION
    assert q4.q4adamw_status_string(0) == "ok"
    assert "workspace" in q4.q4adamw_status_string(7)


@pytest.mark.parametrize("cb", range(5))
def test_library_codebooks_equal_oracle_construction(cb):
    got = np.array(q4.q4adamw_codebook(cb), np.float32)
    assert np.array_equal(got.view(np.uint32), O.codebook(cb).view(np.uint32))


@pytest.mark.parametrize("cb,cb8", [(5, O.CB8_SDYN8), (6, O.CB8_DYN8)])
def test_library_8bit_codebooks_equal_oracle_construction(cb, cb8):
    got = np.array(q4.q4adamw_codebook(cb), np.float32)
    assert got.size == 256
    assert np.array_equal(got.view(np.uint32), O.codebook8(cb8).view(np.uint32))


_CB_INC = os.path.join(os.path.dirname(build.__file__), "csrc", "q4_codebooks.inc")


@pytest.mark.parametrize("cb8,name", [(O.CB8_SDYN8, "M"), (O.CB8_DYN8, "V")])
def test_8bit_nearest_level_buckets(cb8, name):
    """The 8-bit step counts midpoints below x with a bucket table (key >> SHIFT
    from LO, NB buckets, two candidate midpoints per bucket).  The compiled-in
    bucket parameters must leave at most two of the oracle's positive
    midpoints in any bucket, and the bucketed count must equal the plain count
    at every midpoint, its FP32 neighbours, and a dense sample of [0, 1]."""
    d = {k: int(v) for k, v in re.findall(r"#define Q4_RTN8_%s_(\w+) (\d+)" % name, open(_CB_INC).read())}
    shift, lo, nb = d["SHIFT"], d["LO"], d["NB"]
    mid = np.asarray(O.sorted_levels8(cb8)[2], np.float32)
    mid = mid[np.isfinite(mid)]
    pos = mid[mid > 0]
    keys = pos.view(np.uint32)
    assert keys[0] >> shift == lo
    assert np.bincount((keys >> shift) - lo).max() <= 2
    assert (np.uint32(0x3F800001) >> shift) - lo == nb - 1
    pad = np.append(pos, np.full(256 - len(pos), np.inf, np.float32)).astype(np.float32)
    lower = ((np.arange(nb, dtype=np.uint64) + lo) << shift).astype(np.uint32).view(np.float32)
    floor = np.searchsorted(pad, lower, side="left")
    x = np.concatenate([pos, np.nextafter(pos, np.float32(0)), np.nextafter(pos, np.float32(2)),
                        np.linspace(0, 1, 1 << 20, dtype=np.float32), np.float32([0, 1, 1e-30])])
    key = x.view(np.uint32)
    b = np.clip((key >> shift).astype(np.int64) - lo, 0, nb - 1)
    f = floor[b]
    got = f + (pad[f] < x) + (pad[np.minimum(f + 1, 255)] < x)
    assert np.array_equal(got, np.searchsorted(pos, x, side="left"))


def test_8bit_recipe_is_one_configuration():
    """[A] "Requirements and errors": 4-bit and 8-bit options do not mix."""
    b = q4.q4adamw_default_config(q4.RECIPE_BLOCK8)
    assert (b.m_codebook, b.v_codebook, b.m_rule, b.v_rule, b.eden) == (
        q4.CB_SDYN8, q4.CB_DYN8, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 0)
    t = [fake_tensor((64, 32))]
    q4.q4adamw_validate(b, hp(), t)
    b.v_codebook = q4.CB_DYN4
    assert status_of(q4.q4adamw_validate, b, hp(), t) == 4
    c = q4.q4adamw_default_config(q4.RECIPE_CUSTOM)
    c.v_codebook = q4.CB_DYN8
    assert status_of(q4.q4adamw_validate, c, hp(), t) == 4
    # an 8-bit state never resumes as 4-bit, nor the reverse
    h8 = q4.q4adamw_make_header(q4.q4adamw_default_config(q4.RECIPE_BLOCK8))
    assert status_of(q4.q4adamw_check_header, q4.q4adamw_default_config(q4.RECIPE_ZIP_SR), h8) == 5
    sb = q4.q4adamw_state_bytes(q4.q4adamw_default_config(q4.RECIPE_BLOCK8), [fake_tensor((1024,))])
    assert sb["adam4_quantized_state_bytes"] == 2048 and sb["adam4_scale_metadata_bytes"] == 64


def test_default_configs_follow_table2():
    z = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    assert (z.m_codebook, z.v_codebook, z.m_rule, z.v_rule, z.eden) == (
        q4.CB_NF4, q4.CB_DYN4, q4.RULE_STATE_RTN, q4.RULE_UPDATE_SR, 0)
    e = q4.q4adamw_default_config(q4.RECIPE_ZE_EDEN)
    assert (e.m_codebook, e.v_codebook, e.m_rule, e.v_rule, e.eden) == (
        q4.CB_NF4, q4.CB_DYN4_NZ, q4.RULE_STATE_RTN, q4.RULE_STATE_RTN, 1)
    f = q4.q4adamw_default_config(q4.RECIPE_FACTORED)
    assert (f.v_codebook, f.v_rule, f.eden) == (q4.CB_DYN4_NZ, q4.RULE_STATE_RTN, 0)
    assert f.block == 128 and f.abi_version == 3


@pytest.mark.parametrize("step", [1, 2, 10, 1000, 123456789])
def test_host_scalars_equal_oracle_bits(step):
    for lr, b1, b2, wd in [(1e-3, 0.9, 0.999, 0.1), (6e-4, 0.95, 0.98, 0.0), (2e-4, 0.5, 0.0, 0.01)]:
        hp = q4.Q4HParams(lr, b1, b2, 1e-8, wd, 0.0, step, 0, 0, 0)
        got = np.array(q4.q4adamw_host_scalars(hp), np.float32)
        ref = O.host_scalars(O.HParams(lr=lr, beta1=b1, beta2=b2, weight_decay=wd, step=step))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def fake_tensor(shape, tid=0, base=0x10000, fp32=False, factored=False):
    """Tensor descriptor with fake (never dereferenced) aligned pointers."""
    t = q4.Q4Tensor()
    t.tensor_id = tid
    t.ndim = len(shape)
    n = 1
    for d, x in enumerate(shape):
        t.shape[d] = x
        n *= x
    t.numel = n
    names = ["param", "grad", "m_codes", "m_scales"]
    if fp32:
        names += ["m_fp32", "v_fp32"]
    elif factored:
        names += ["v_row", "v_col"]
    else:
        names += ["v_codes", "v_scales"]
    for k, nm in enumerate(names):
        setattr(t, nm, base + 0x1000 * k)
    return t


def hp(**kw):
    d = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.1, eps_sr=0.0, step=1, seed=0,
             lm_head_sr=0, flags=0, max_grad_norm=0.0, reserved=0)
    d.update(kw)
    return q4.Q4HParams(*[d[k] for k, _ in q4.Q4HParams._fields_])


def status_of(fn, *a):
    with pytest.raises(q4.Q4Error) as ei:
        fn(*a)
    return ei.value.status


def test_validation_accepts_good_input():
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    q4.q4adamw_validate(cfg, hp(), [fake_tensor((256, 512)), fake_tensor((65536,), 1)])


def test_validation_errors():
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    good = fake_tensor((100, 7))
    V = q4.q4adamw_validate
    assert status_of(V, cfg, hp(step=0), [good]) == 1
    assert status_of(V, cfg, hp(beta1=1.0), [good]) == 1
    assert status_of(V, cfg, hp(beta2=-0.1), [good]) == 1
    assert status_of(V, cfg, hp(eps=0.0), [good]) == 1
    assert status_of(V, cfg, hp(lr=float("nan")), [good]) == 1
    assert status_of(V, cfg, hp(max_grad_norm=-1.0), [good]) == 1
    assert status_of(V, cfg, hp(max_grad_norm=float("inf")), [good]) == 1
    q4.q4adamw_validate(cfg, hp(max_grad_norm=1.0), [good])
    bad = fake_tensor((100, 7)); bad.numel = 701
    assert status_of(V, cfg, hp(), [bad]) == 2
    bad = fake_tensor((100, 7)); bad.ndim = 9
    assert status_of(V, cfg, hp(), [bad]) == 2
    bad = fake_tensor((1 << 17, 1 << 17))
    assert status_of(V, cfg, hp(), [bad]) == 2
    bad = fake_tensor((100, 7)); bad.m_codes = 0x10008
    assert status_of(V, cfg, hp(), [bad]) == 3
    bad = fake_tensor((100, 7)); bad.v_scales = None
    assert status_of(V, cfg, hp(), [bad]) == 1
    c2 = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR); c2.block = 64
    assert status_of(V, c2, hp(), [good]) == 1
    c3 = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR); c3.v_codebook = q4.CB_DYN4_NZ
    assert status_of(V, c3, hp(), [good]) == 4   # a recipe fixes its codebooks
    c4 = q4.q4adamw_default_config(q4.RECIPE_CUSTOM); c4.v_codebook = q4.CB_NF4
    assert status_of(V, c4, hp(), [good]) == 4   # signed map for v
    c5 = q4.q4adamw_default_config(q4.RECIPE_CUSTOM); c5.m_rule = q4.RULE_UPDATE_SR
    assert status_of(V, c5, hp(), [good]) == 4
    assert status_of(V, cfg, hp(), []) == 2
    # factored matrices need their row/column vectors
    cf = q4.q4adamw_default_config(q4.RECIPE_FACTORED)
    q4.q4adamw_validate(cf, hp(), [fake_tensor((64, 32), factored=True), fake_tensor((64,))])
    assert status_of(V, cf, hp(), [fake_tensor((64, 32))]) == 1


def test_shard_offsets_are_validated():
    """A shard starts on a 512-element boundary (its pointers stay 16-byte
    aligned) inside the 2^34-element range of the Philox counter; a
    factored matrix cannot be a shard."""
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    V = q4.q4adamw_validate
    ok = fake_tensor((1000,)); ok.elem_offset = 512 * 37
    V(cfg, hp(), [ok])
    for off in (-512, 128, 64, 1, (1 << 34) - 512):
        bad = fake_tensor((1000,)); bad.elem_offset = off
        assert status_of(V, cfg, hp(), [bad]) == 2, off
    cf = q4.q4adamw_default_config(q4.RECIPE_FACTORED)
    mat = fake_tensor((64, 32), factored=True); mat.elem_offset = 512
    assert status_of(V, cf, hp(), [mat]) == 2
    vec = fake_tensor((2048,)); vec.elem_offset = 512
    V(cf, hp(), [vec])


def test_step_refuses_before_any_device_work_on_bad_input():
    """Invalid calls return their status before touching a device."""
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZE_EDEN)
    assert status_of(q4.q4adamw_step, cfg, hp(step=0), [fake_tensor((10,))], 0x20000, 4096, 0) == 1
    bad = fake_tensor((10,)); bad.numel = 11
    assert status_of(q4.q4adamw_step, cfg, hp(), [bad], 0x20000, 4096, 0) == 2


def test_state_bytes_1_0625_per_param():
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    ts = [fake_tensor((50304, 768)), fake_tensor((768,), 1)]
    sb = q4.q4adamw_state_bytes(cfg, ts)
    n = 50304 * 768 + 768
    assert sb["adam4_total_bytes"] == 1.0625 * n
    assert sb["adam4_quantized_state_bytes"] == n
    f32 = q4.q4adamw_state_bytes(q4.q4adamw_default_config(q4.RECIPE_FP32),
                                 [fake_tensor((50304, 768), fp32=True), fake_tensor((768,), 1, fp32=True)])
    assert f32["adam4_total_bytes"] == 8 * n
    assert round(8 / 1.0625, 2) == 7.53
    # the oracle's count agrees
    assert O.state_bytes(O.ZIP_SR, n - 768, 50304, True)[2] + O.state_bytes(O.ZIP_SR, 768, 768, False)[2] == \
        sb["adam4_total_bytes"]


def test_state_bytes_factored():
    cfg = q4.q4adamw_default_config(q4.RECIPE_FACTORED)
    sb = q4.q4adamw_state_bytes(cfg, [fake_tensor((1024, 2048), factored=True), fake_tensor((1024,), 1)])
    assert sb["adam4_quantized_state_bytes"] == 1024 * 2048 // 2 + 1024
    assert sb["adam4_scale_metadata_bytes"] == 4 * (1024 * 2048 // 128) + 4 * (1024 + 2048) + 8 * 8


def test_workspace_bytes_monotone():
    cfg = q4.q4adamw_default_config(q4.RECIPE_FACTORED)
    a = q4.q4adamw_workspace_bytes(cfg, [fake_tensor((64,))])
    b = q4.q4adamw_workspace_bytes(cfg, [fake_tensor((1024, 2048), factored=True), fake_tensor((64,), 1)])
    assert 256 <= a < b and a % 256 == 0 and b % 256 == 0


def test_state_header_roundtrip():
    cfg = q4.q4adamw_default_config(q4.RECIPE_ZIP_SR)
    h = q4.q4adamw_make_header(cfg)
    q4.q4adamw_check_header(cfg, h)
    other = q4.q4adamw_default_config(q4.RECIPE_ZE_EDEN)
    assert status_of(q4.q4adamw_check_header, other, h) == 5
    h.layout_version = 0
    assert status_of(q4.q4adamw_check_header, cfg, h) == 5
    h2 = q4.q4adamw_make_header(cfg); h2.magic = 0
    assert status_of(q4.q4adamw_check_header, cfg, h2) == 5


def test_product_path_has_no_oracle_dependency():
    """The package never imports or links the oracle, and fails loudly without
    its library."""
    pkg = os.path.join(ROOT, "bit_adamw_update_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h", ".inc")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"(from|import)\s+oracle|q4_oracle|q4oracle|or_step", src), f
    with pytest.raises(RuntimeError):
        api._lib_saved = api._lib
        try:
            api._lib = None
            api.load_library(os.path.join(ROOT, "does_not_exist.so"))
        finally:
            api._lib = api._lib_saved


def test_flat_offsets_of_the_microbatch_layout():
    """Tensor i starts at 512 * sum_{j<i} ceil(numel_j / 512)."""
    ts = [fake_tensor((1000,)), fake_tensor((3, 5)), fake_tensor((512,)), fake_tensor((7, 129))]
    offs, total = q4.q4adamw_flat_offsets(ts)
    assert offs == [0, 1024, 1536, 2048]
    assert total == 2048 + 1024

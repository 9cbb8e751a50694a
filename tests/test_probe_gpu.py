"""The bandwidth probes (libq4probe.so) do the memory work they claim: the
byte-mix probes (4-bit and 8-bit codes), in both their walks, read and
rewrite every byte of their mix (masters, codes and
scales changed as its arithmetic says, nothing outside touched), the copy
copies, the in-place update rewrites every element and the read probe reads
everything."""
import numpy as np
import pytest
import torch

from bit_adamw_update_amd import probe

pytestmark = pytest.mark.gpu


# 37 chunks: one slab-run and a ragged slab; 512 * 4 * 8 * 3000 + 512 * 5:
# more runs of 8 slabs than resident groups, so the queue hands out runs
# again, and a ragged last run
@pytest.mark.parametrize("n", [512 * 37, 512 * (4 * 8 * 3000 + 5)], ids=["small", "queue_laps"])
@pytest.mark.parametrize("form", ["step_walk", "queue"])
@pytest.mark.parametrize("bits", [4, 8])
def test_byte_mix_touches_exactly_its_bytes(bits, form, n):
    bm = probe.ByteMix(n, bits=bits)
    before = {f: getattr(bm, f).clone() for f in ("param", "grad", "m_codes", "v_codes", "m_scales", "v_scales")}
    guard = torch.full((4096,), 7, dtype=torch.uint8, device="cuda")
    print("byte mix probe", bits, form, n, flush=True)
    bm.run() if form == "step_walk" else bm.run_queue()
    torch.cuda.synchronize()
    assert bm.bytes() == 12 * n + n // 8 + (2 * n if bits == 8 else 0)
    a = np.float32(0.999)
    # element c*512 + 128r + 64h + 4s + e is value e of half h of lane s of
    # row r in chunk c
    shape = (-1, 4, 2, 16, 4)
    p0 = before["param"].cpu().numpy().reshape(shape)
    g16 = before["grad"].view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).reshape(shape)
    # the lane's gradient term: its first half's first value plus its
    # second half's last value
    gq = ((g16[:, :, 0, :, 0] << 16).view(np.float32) + (g16[:, :, 1, :, 3] << 16).view(np.float32)).astype(np.float32)
    expect = (p0 * a + gq[:, :, None, :, None]).reshape(-1)
    assert np.array_equal(bm.param.cpu().numpy().view(np.uint32), expect.view(np.uint32))
    # each half's codes of the lane (16 bits of 4-bit codes, 32 bits of
    # 8-bit ones) take the first half's second gradient word (m) or the
    # second half's first (v), cut to the codes' width
    g32 = before["grad"].view(torch.int16).cpu().numpy().view(np.uint32).reshape(-1, 4, 2, 16, 2)
    key = {"m_codes": g32[:, :, 0, :, 1], "v_codes": g32[:, :, 1, :, 0]}
    cdt = {4: np.uint16, 8: np.uint32}[bits]
    for codes in ("m_codes", "v_codes"):
        c0 = before[codes].cpu().numpy().view(cdt).reshape(-1, 4, 2, 16)
        got = getattr(bm, codes).cpu().numpy().view(cdt).reshape(-1, 4, 2, 16)
        assert np.array_equal(got, c0 ^ key[codes].astype(cdt)[:, :, None, :])
    for sc in ("m_scales", "v_scales"):
        assert np.array_equal(getattr(bm, sc).cpu().numpy(), before[sc].cpu().numpy() * a)
    assert torch.equal(bm.grad.view(torch.int16), before["grad"].view(torch.int16))
    assert int((guard != 7).sum()) == 0


def test_copy_and_read():
    n = (1 << 20) + 16
    src = torch.randint(1, 1 << 30, (n,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    sink = torch.zeros(probe.load_library().q4probe_read_sink_words(), dtype=torch.int32, device="cuda")
    print("copy and read probes", flush=True)
    probe.copy(dst, src)
    probe.read(src, sink)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    # the XOR over all threads' partial XORs is the XOR of every word read
    ref = np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32))
    assert np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32)) == ref


def test_update_in_place():
    """Every element scaled by 0.999f once, in the segment part and the tail."""
    n = (1 << 20) + 12
    x = torch.randn(n, device="cuda")
    ref = x * torch.tensor(0.999, dtype=torch.float32, device="cuda")
    print("in-place probe", flush=True)
    probe.update_in_place(x)
    torch.cuda.synchronize()
    assert torch.equal(x.view(torch.int32), ref.view(torch.int32))

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
    p0 = before["param"].cpu().numpy()
    q = before["grad"].view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32).reshape(-1, 8)
    # lane l's gradient term: low half of its first word plus high half of its fourth
    gq = ((q[:, 0] << 16).view(np.float32) + ((q[:, 7] << 16) & 0xFFFF0000).view(np.float32)).astype(np.float32)
    expect = (p0.reshape(-1, 8) * a + gq[:, None]).reshape(-1)
    assert np.array_equal(bm.param.cpu().numpy().view(np.uint32), expect.view(np.uint32))
    # lane l's 4-bit codes (one word) take its gradient word 1 (m) or 2 (v);
    # its 8-bit codes (two words) take words 0-1 (m) or 2-3 (v)
    words = {4: ((1,), (2,)), 8: ((0, 1), (2, 3))}[bits]
    g32 = before["grad"].view(torch.int16).cpu().numpy().view(np.uint32).reshape(-1, 4)
    for codes, w in zip(("m_codes", "v_codes"), words):
        c0 = before[codes].cpu().numpy().view(np.uint32).reshape(-1, len(w))
        got = getattr(bm, codes).cpu().numpy().view(np.uint32).reshape(-1, len(w))
        assert np.array_equal(got, c0 ^ g32[:, list(w)])
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

"""GPU tests of the fused calls' safety contract: a grid barrier that gives
up leaves its workspace consistent (the next call on it is bit-exact), the
binding's default workspaces and status words are per (device, stream), and
the checked mode raises on a barrier timeout.

The timeout is forced from the host with fos_set_barrier_poll_limit(0):
every workgroup that is not the barrier's last arrival then gives up at
once and returns, so each kernel still exits normally.
"""
import numpy as np
import pytest
import torch

import nvfp4_adaptive_block_amd as fos
import synthdata
from synthdata import raw_bits

pytestmark = pytest.mark.gpu


def dev(t):
    return t.to("cuda")


class poll_limit:
    """Set the fused calls' poll limit for the duration of a block."""

    def __init__(self, polls):
        self.polls = polls

    def __enter__(self):
        self.prev = fos.set_barrier_poll_limit(self.polls)

    def __exit__(self, *exc):
        fos.set_barrier_poll_limit(self.prev)


def _group_amaxes(orc, b, dtype, offs):
    starts = np.concatenate([[0], offs[:-1]])
    return np.array([orc.amax(b[s:e], dtype, "tensor")[0] if e > s else 0.0 for s, e in zip(starts, offs)],
                    np.float32)


def test_per_tensor_fused_after_a_timeout(orc):
    """A fused quantize whose barrier gave up (status bit set) is followed,
    on the same workspace, by a call on other data that matches the oracle
    and leaves the counters zero."""
    M, K = 2048, 4096
    big = synthdata.normal(M, K, 71, "bf16").to(torch.float32).mul_(1000.0).to(torch.bfloat16)
    x = synthdata.normal(M, K, 72, "bf16")
    b = raw_bits(x)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with poll_limit(0):
        fos.fos_quantize_fused(dev(big), workspace=ws, status=status, recipe="4over6")
        torch.cuda.synchronize()
    assert int(status.item()) & fos.STATUS_BARRIER_TIMEOUT, "the forced timeout did not show"
    assert not ws[256:].any(), "the counters must be zero once the barrier completed"
    status.zero_()
    for kw in (dict(recipe="4over6", err_metric="mse"), dict(recipe="4over6", err_metric="mae", err_prec="fp16")):
        codes, scales, amax, _ = fos.fos_quantize_fused(dev(x), workspace=ws, status=status, **kw)
        y, qa = fos.fos_qdq_fused(dev(x), workspace=ws, status=status, **kw)
        torch.cuda.synchronize()
        a = orc.amax(b, "bf16", "tensor")
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), a.view(np.uint32))
        np.testing.assert_array_equal(qa.cpu().numpy().view(np.uint32), a.view(np.uint32))
        want = orc.quantize(b, "bf16", a, **kw)
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"], err_msg=f"{kw}")
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"], err_msg=f"{kw}")
        np.testing.assert_array_equal(raw_bits(y.cpu()), orc.qdq(b, "bf16", a, **kw), err_msg=f"{kw}")
    assert int(status.item()) == 0
    assert not ws[256:].any()


def test_grouped_fused_after_a_timeout(orc):
    """The grouped form keeps per-group maxima in banked slots. After a call
    whose barrier gave up (workgroup 0 included, most likely), the next
    grouped call must still start from a cleared bank: its group amaxes are
    far smaller than the first call's, so a stale maximum would show."""
    M, pad, K, G = 4096, 64, 2048, 16
    xa, offs_a, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=(81, 82, 83, 84), dtype="bf16")
    xa = (xa.to(torch.float32) * 1000.0).to(torch.bfloat16)
    xb, offs_b, _ = synthdata.grouped_tokens(M, pad, K, G, seeds=(85, 86, 87, 88), dtype="bf16")
    bb = raw_bits(xb)
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with poll_limit(0):
        fos.fos_quantize_grouped_fused(dev(xa), dev(torch.from_numpy(offs_a)), workspace=ws, status=status,
                                       recipe="4over6")
        torch.cuda.synchronize()
    assert int(status.item()) & fos.STATUS_BARRIER_TIMEOUT, "the forced timeout did not show"
    status.zero_()
    gam = _group_amaxes(orc, bb, "bf16", offs_b)
    for _ in range(2):  # both banks
        codes, scales, amax, gsdec = fos.fos_quantize_grouped_fused(dev(xb), dev(torch.from_numpy(offs_b)),
                                                                    workspace=ws, status=status, recipe="4over6")
        torch.cuda.synchronize()
        np.testing.assert_array_equal(amax.cpu().numpy().view(np.uint32), gam.view(np.uint32))
        want = orc.quantize_grouped(bb, "bf16", offs_b, gam, recipe="4over6")
        np.testing.assert_array_equal(gsdec.cpu().numpy().view(np.uint32), want["group_sdec"].view(np.uint32))
        np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])
    assert int(status.item()) == 0


def test_list_fused_after_a_timeout(orc):
    """The fused amaxes + QDQ list shares the grouped call's banked slots: a
    list call whose barrier gave up is followed by list calls on smaller
    data that match the oracle (both banks)."""
    big = [(synthdata.weight(512, 1024, 90 + i, "bf16").to(torch.float32) * 1000.0).to(torch.bfloat16)
           for i in range(4)]
    xs = [synthdata.weight(512, 1024, 95 + i, "bf16") for i in range(4)]
    bits = [raw_bits(x) for x in xs]
    want_a = [orc.amax(b, "bf16", "tensor") for b in bits]
    ws = torch.zeros(fos.FUSED_WORKSPACE_BYTES, dtype=torch.uint8, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    with poll_limit(0):
        fos.fos_qdq_list_fused([dev(t) for t in big], workspace=ws, status=status, recipe="4over6")
        torch.cuda.synchronize()
    assert int(status.item()) & fos.STATUS_BARRIER_TIMEOUT, "the forced timeout did not show"
    status.zero_()
    for _ in range(2):
        ys, amax = fos.fos_qdq_list_fused([dev(t) for t in xs], workspace=ws, status=status, recipe="4over6")
        torch.cuda.synchronize()
        for i in range(4):
            assert amax.cpu().numpy().view(np.uint32)[i] == want_a[i].view(np.uint32)[0]
            np.testing.assert_array_equal(raw_bits(ys[i].cpu()), orc.qdq(bits[i], "bf16", want_a[i], recipe="4over6"))
    assert int(status.item()) == 0


def test_checked_mode_raises_on_timeout(orc):
    """check=True synchronizes and raises when the barrier gave up; the
    binding's own status word is cleared by the check, and a checked call
    afterwards passes."""
    x = synthdata.normal(2048, 4096, 73, "bf16")
    xd = dev(x)
    with poll_limit(0):
        with pytest.raises(fos.FosError, match="timed out"):
            fos.fos_quantize_fused(xd, recipe="4over6", check=True)
        with pytest.raises(fos.FosError, match="timed out"):
            fos.fos_qdq_fused(xd, recipe="4over6", err_prec="fp16", check=True)
    assert fos.fused_status("cuda") == 0
    codes, scales, amax, _ = fos.fos_quantize_fused(xd, recipe="4over6", check=True)
    a = orc.amax(raw_bits(x), "bf16", "tensor")
    want = orc.quantize(raw_bits(x), "bf16", a, recipe="4over6")
    np.testing.assert_array_equal(codes.cpu().numpy(), want["codes"])
    np.testing.assert_array_equal(scales.cpu().numpy(), want["scales"])


def test_default_workspace_and_status_per_stream(orc):
    """Fused calls issued on two streams, one after the other (the streams
    are synchronized between the calls; nothing overlaps on purpose), take
    distinct default workspaces and status words, and both match the
    oracle with a clean status."""
    x = synthdata.normal(1024, 2048, 74, "bf16")
    b = raw_bits(x)
    xd = dev(x)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            outs.append(fos.fos_quantize_fused(xd, recipe="4over6"))
            g = fos.fos_quantize_grouped_fused(xd, dev(torch.tensor([512, 1024], dtype=torch.int32)),
                                               recipe="4over6")
            outs.append(g)
        s.synchronize()
    assert fos.fused_workspace("cuda", s1) is not fos.fused_workspace("cuda", s2)
    assert fos.fused_status_word("cuda", s1) is not fos.fused_status_word("cuda", s2)
    assert fos.fused_workspace("cuda", s1).data_ptr() != fos.fused_workspace("cuda", s2).data_ptr()
    assert fos.fused_status("cuda", s1) == 0 and fos.fused_status("cuda", s2) == 0
    a = orc.amax(b, "bf16", "tensor")
    want = orc.quantize(b, "bf16", a, recipe="4over6")
    offs = np.array([512, 1024], np.int32)
    gam = _group_amaxes(orc, b, "bf16", offs)
    gwant = orc.quantize_grouped(b, "bf16", offs, gam, recipe="4over6")
    for i in (0, 2):
        np.testing.assert_array_equal(outs[i][0].cpu().numpy(), want["codes"])
        np.testing.assert_array_equal(outs[i][1].cpu().numpy(), want["scales"])
        np.testing.assert_array_equal(outs[i + 1][0].cpu().numpy(), gwant["codes"])
        np.testing.assert_array_equal(outs[i + 1][2].cpu().numpy().view(np.uint32), gam.view(np.uint32))

"""The attainable-rate probes: each launch does the work it reports.

The read probe must touch every 16-byte piece of its buffer exactly as
described in include/moe.h (lane t of the grid reads the pieces j with
j mod (blocks * 256) == t): its per-lane XOR is checked bit for bit against
numpy, for all four load forms, on a buffer with a ragged tail.  The MFMA
probes must report the FLOPs of the launch and leave finite sums.
"""
import numpy as np
import pytest
import torch

import routing_expert_ffn_amd as moe

pytestmark = pytest.mark.gpu

BLOCKS = 4
LANES = BLOCKS * 256
N16 = 8 * LANES * 3 + LANES * 2 + 517  # three full rounds of eight, two more strides, a partial one


def _buffer():
    g = torch.Generator().manual_seed(1234)
    host = torch.randint(0, 256, (N16 * 16,), dtype=torch.uint8, generator=g)
    return host, host.cuda()


def _expected(host, mode):
    words = host.numpy().view(np.uint32).reshape(N16, 4)
    out = np.zeros(LANES, dtype=np.uint32)
    for t in range(LANES):
        js = np.arange(t, N16, LANES)
        if mode <= 1:
            v = np.bitwise_xor.reduce(words[js], axis=0)
        else:
            # global->LDS forms: the lane reports its LDS slot of piece 0 of a
            # round, which the tail pieces overwrite last: the lane's last piece
            v = words[js[-1]]
        out[t] = (v[0] ^ v[1] ^ v[2] ^ v[3]) & 0x007FFFFF
    return out


@pytest.mark.parametrize("mode", [0, 1, 2, 3])
def test_read_probe_reads_every_piece(mode):
    host, buf = _buffer()
    sink = torch.full((LANES,), -1.0, dtype=torch.float32, device="cuda")
    n = moe.probe_read(buf, mode, BLOCKS, sink)
    torch.cuda.synchronize()
    assert n == N16 * 16
    got = sink.cpu().view(torch.int32).numpy().view(np.uint32)
    assert np.array_equal(got, _expected(host, mode))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("vary", [True, False])
def test_mfma_probe_reports_its_flops(fp8, vary):
    blocks, iters = 8, 37
    sink = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    probe = moe.probe_mfma_fp8 if fp8 else moe.probe_mfma_bf16
    flops = probe(blocks, iters, sink, vary=vary)
    torch.cuda.synchronize()
    # four wavefronts per block, eight MFMAs per round, 32 x 32 x K MACs each
    assert flops == blocks * iters * 4 * 8 * 2 * 32 * 32 * (64 if fp8 else 16)
    assert torch.isfinite(sink).all()


def test_probe_arguments_are_checked():
    sink = torch.empty(256, dtype=torch.float32, device="cuda")
    with pytest.raises(moe.MoeError):
        moe.probe_mfma_fp8(0, 1, sink)
    with pytest.raises(moe.MoeError):
        moe.probe_mfma_bf16(1, 0, sink)
    buf = torch.empty(100, dtype=torch.uint8, device="cuda")  # not a multiple of 16 bytes
    with pytest.raises(moe.MoeError):
        moe.probe_read(buf, 0, 1, sink)

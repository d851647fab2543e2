"""The asynchronous calls in a captured graph. Encode, decode, a second
encode and the fused reduce launch kernels only (no allocation, no memset
node, no host synchronisation), so a caller can capture them once and
replay them. Every replay is checked against the oracle, with the outputs
overwritten by eager work between replays."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def test_encode_decode_reduce_replayed_from_a_graph():
    w = workloads.config(2, small=True)
    x = w.x
    n, C = x.size, 1024
    xb = np.roll(x, n // 2)
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    want = oracle.encode(x, C, ocb.dec)
    want_b = oracle.encode(xb, C, ocb.dec)
    want_r = oracle.reduce_add(want, want_b, n, C, ocb.dec)
    xd = torch.from_numpy(x.view(np.int16)).to(DEV)
    xbd = torch.from_numpy(xb.view(np.int16)).to(DEV)
    cap = uzip.max_bytes(n, C)
    out = torch.empty(cap, dtype=torch.uint8, device=DEV)
    outb = torch.empty_like(out)
    outr = torch.empty_like(out)
    ws = torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=DEV)
    y = torch.empty(n, dtype=torch.int16, device=DEV)

    def calls():
        uzip.encode(xd, cb, C, out=out, ws=ws)
        uzip.decode(out, cb, n, C, out=y)
        uzip.encode(xbd, cb, C, out=outb, ws=ws)
        uzip.reduce_add(out, outb, cb, n, C, out=outr, ws=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()                              # eager run on the capture stream first
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(3):
        out.fill_(0xEE)
        outb.fill_(0xEE)
        outr.fill_(0xEE)
        y.fill_(0x1234)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out[:want.size].cpu().numpy(), want), f"replay {rep}: stream"
        assert np.array_equal(y.cpu().numpy().view(np.uint16), x), f"replay {rep}: decode"
        assert np.array_equal(outr[:want_r.size].cpu().numpy(), want_r), f"replay {rep}: reduce"

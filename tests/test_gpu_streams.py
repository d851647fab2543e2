"""Calls on two streams at once. Each stream has its own outputs and
workspace, and the calls of the two streams are launched back to back with
no synchronisation between them, so their kernels may overlap on the GPU.
Every result must still equal the oracle's: the library keeps no device
state of its own between or across calls."""
import numpy as np
import pytest
import torch

import oracle
import workloads
from lossless_bf16_tensor_amd import uzip

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(x_np):
    return torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV)


def test_encode_decode_reduce_on_two_streams():
    w = workloads.config(2, small=True)          # 1.5 Mi values: 192 tiles per call
    C = 1024
    xs = [w.x, np.roll(w.x, w.x.size // 3)]
    n = xs[0].size
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    want = [oracle.encode(x, C, ocb.dec) for x in xs]
    # stream i adds the streams of input i and of the other input, in that order
    want_r = [oracle.reduce_add(want[0], want[1], n, C, ocb.dec),
              oracle.reduce_add(want[1], want[0], n, C, ocb.dec)]
    xd = [to_dev(x) for x in xs]
    cap = uzip.max_bytes(n, C)
    outs = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(2)]
    reds = [torch.empty(cap, dtype=torch.uint8, device=DEV) for _ in range(2)]
    wss = [torch.empty(uzip.workspace_bytes(n, C), dtype=torch.uint8, device=DEV) for _ in range(2)]
    ys = [torch.empty(n, dtype=torch.int16, device=DEV) for _ in range(2)]
    # the streams the reduces read, encoded once before the concurrent calls
    ins = [uzip.encode(xd[i], cb, C) for i in range(2)]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for rep in range(3):
        for t in outs + reds:
            t.fill_(0xEE)
        for y in ys:
            y.fill_(0x1234)
        torch.cuda.synchronize()
        for i in range(2):
            with torch.cuda.stream(streams[i]):
                uzip.encode(xd[i], cb, C, out=outs[i], ws=wss[i])
                uzip.decode(outs[i], cb, n, C, out=ys[i])
                uzip.reduce_add(ins[i], ins[1 - i], cb, n, C, out=reds[i], ws=wss[i])
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(outs[i][:want[i].size].cpu().numpy(), want[i]), f"rep {rep} stream {i}: encode"
            assert np.array_equal(ys[i].cpu().numpy().view(np.uint16), xs[i]), f"rep {rep} stream {i}: decode"
            assert np.array_equal(reds[i][:want_r[i].size].cpu().numpy(), want_r[i]), f"rep {rep} stream {i}: reduce"


def test_stream_argument_without_buffers():
    """Calls given stream= and no out/ws: the binding's temporaries belong
    to that stream, so allocations made meanwhile on the current stream (and
    filled there) cannot take their memory while the call's kernels run."""
    w = workloads.config(2, small=True)
    C = 1024
    xs = [w.x, np.roll(w.x, w.x.size // 5)]
    n = xs[0].size
    ocb = oracle.calibrate(w.calib)
    cb = uzip.codebook_from_hist(ocb.hist)
    want = [oracle.encode(x, C, ocb.dec) for x in xs]
    want_r = oracle.reduce_add(want[0], want[1], n, C, ocb.dec)
    xd = [to_dev(x) for x in xs]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    cap = uzip.max_bytes(n, C)
    wsb = uzip.workspace_bytes(n, C)
    for rep in range(3):
        outs = [uzip.encode(xd[i], cb, C, stream=streams[i]) for i in range(2)]
        # same-sized allocations on the current stream, overwritten at once
        junk = [torch.full((sz,), 0x5A, dtype=torch.uint8, device=DEV) for sz in (wsb, cap, wsb, cap)]
        ys = [uzip.decode(outs[i], cb, n, C, stream=streams[i]) for i in range(2)]
        streams[1].wait_stream(streams[0])
        red = uzip.reduce_add(outs[0], outs[1], cb, n, C, stream=streams[1])
        junk += [torch.full((sz,), 0xA5, dtype=torch.uint8, device=DEV) for sz in (wsb, cap)]
        torch.cuda.synchronize()
        for i in range(2):
            assert np.array_equal(outs[i][:want[i].size].cpu().numpy(), want[i]), f"rep {rep} stream {i}: encode"
            assert np.array_equal(ys[i].cpu().numpy().view(np.uint16), xs[i]), f"rep {rep} stream {i}: decode"
        assert np.array_equal(red[:want_r.size].cpu().numpy(), want_r), f"rep {rep}: reduce"
        del junk, outs, ys, red

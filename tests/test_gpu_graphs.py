"""The codec's calls captured into HIP graphs and replayed, through the C ABI.

Callers under graph capture are one reason for sh_encode_noalloc (its workspace is a fixed
device array), and sh_encode_batch with a placement stream forks and joins a second stream
with events.  Each graph is replayed several times; between replays the program's own eager
work rewrites the inputs (a different permutation of the same values, so that the tables
still hold every value), and every replay's containers and decoded tensors are compared with
the eager calls' on the same inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

from entropy_coding_quantized_amd import codec
from entropy_coding_quantized_amd import datagen as D

pytestmark = pytest.mark.gpu

REPLAYS = 3


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    codec.lib()
    return torch


def _perm(x, k):
    return np.random.default_rng(100 + k).permutation(x)


def test_noalloc_encode_and_decode_replayed(torch_cuda):
    torch = torch_cuda
    p = codec.Params(K=16, log2_L=7, chunk_symbols=4096, streams=32)
    print("case: graph of sh_encode_noalloc + sh_decode, weight 4096x1024", flush=True)
    x0 = D.weight().reshape(-1)
    n = x0.size
    t = codec.sh_table_from_histogram(np.bincount(x0.astype(np.int16) + 128, minlength=256)
                                      .astype(np.uint64), p)
    cap = codec.sh_encode_bound(n, p)
    xd = torch.from_numpy(x0).cuda()
    out = torch.zeros(cap, dtype=torch.uint8, device="cuda")
    y = torch.zeros(n, dtype=torch.int8, device="cuda")
    info = torch.zeros(2, dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    # the first call on the device (outside the capture) sets up the scratch array
    codec.sh_encode_noalloc(t, p, xd, n, out, cap, info, status)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        codec.sh_encode_noalloc(t, p, xd, n, out, cap, info, status)
        codec.sh_decode(t, p, out, cap, y, n, status)
    for k in range(REPLAYS):
        xk = _perm(x0, k)
        xd.copy_(torch.from_numpy(xk))
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, k
        nbytes = int(info[0].item())
        ref, ref_info, ref_st = torch.empty_like(out), torch.zeros_like(info), torch.zeros_like(status)
        wsb = codec.sh_encode_workspace(n, p)
        ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
        codec.sh_encode(t, p, xd, n, ref, cap, ws, wsb, ref_info, ref_st)
        torch.cuda.synchronize()
        assert int(ref_st.item()) == 0
        assert torch.equal(info, ref_info), k
        assert torch.equal(out[:nbytes], ref[:nbytes]), k
        assert torch.equal(y, xd), k


def test_batch_encode_with_placement_stream_replayed(torch_cuda):
    torch = torch_cuda
    p = codec.Params(chunk_symbols=4096, streams=32)
    print("case: graph of sh_encode_batch with a placement stream + sh_decode_batch, "
          "61 tensors", flush=True)
    rng = np.random.default_rng(7)
    xs0 = [D.quantize(rng.laplace(0, float(rng.uniform(3, 30)), size=int(rng.integers(1, 90000))))
           for _ in range(61)]
    ns = [x.size for x in xs0]
    dx = [torch.from_numpy(x).cuda() for x in xs0]
    tables, _ = codec.build_tables_tensors(dx, p)
    caps = [codec.sh_encode_bound(n, p) for n in ns]
    offs = [sum((c + 255) // 256 * 256 for c in caps[:i]) for i in range(len(caps))]
    buf = torch.zeros(offs[-1] + caps[-1], dtype=torch.uint8, device="cuda")
    outs = [buf.data_ptr() + o for o in offs]
    y = torch.zeros(sum((n + 255) // 256 * 256 for n in ns), dtype=torch.int8, device="cuda")
    y_offs = [sum((m + 255) // 256 * 256 for m in ns[:i]) for i in range(len(ns))]
    ys = [y.data_ptr() + o for o in y_offs]
    wsb = codec.sh_encode_batch_workspace(ns, p)
    ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
    info = torch.zeros((len(ns), 2), dtype=torch.int64, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        codec.sh_encode_batch(tables, dx, ns, p, outs, caps, ws, wsb, info, status,
                              place_stream=side)
        codec.sh_decode_batch(tables, outs, caps, ys, ns, p, status)
    for k in range(REPLAYS):
        for x, d in zip(xs0, dx):
            d.copy_(torch.from_numpy(_perm(x, k)))
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert int(status.item()) == 0, k
        rbuf, roffs, _, rinfo, rst = codec.encode_tensors(tables, dx, p)
        torch.cuda.synchronize()
        assert int(rst.item()) == 0
        assert torch.equal(info, rinfo), k
        for i in range(len(ns)):
            nb = int(info[i, 0].item())
            assert torch.equal(buf[offs[i]: offs[i] + nb], rbuf[roffs[i]: roffs[i] + nb]), (k, i)
            assert torch.equal(y[y_offs[i]: y_offs[i] + ns[i]], dx[i]), (k, i)

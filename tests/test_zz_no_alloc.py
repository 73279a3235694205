"""sh_encode_noalloc, the encode entry point for callers that cannot allocate device memory,
against sh_encode (the same encode with a caller-owned workspace), through the C ABI.

Two calls in a row on one GPU, the second on a smaller tensor, each byte-identical to
sh_encode's container with the same encoder totals and status; then a tensor whose
workspace exceeds the fixed scratch array is refused on the host before any GPU work.
"""
from __future__ import annotations

import ctypes as C

import numpy as np
import pytest

from entropy_coding_quantized_amd import codec
from entropy_coding_quantized_amd import datagen as D

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    codec.lib()
    return torch


def _both(torch, x, p):
    x = np.ascontiguousarray(x, dtype=np.int8).reshape(-1)
    t = codec.sh_table_from_histogram(np.bincount(x.astype(np.int16) + 128, minlength=256)
                                      .astype(np.uint64), p)
    xd = torch.from_numpy(x).cuda()
    cap = codec.sh_encode_bound(x.size, p)
    outs = []
    for noalloc in (False, True):
        out = torch.full((cap,), 0xAB, dtype=torch.uint8, device="cuda")
        info = torch.zeros(2, dtype=torch.int64, device="cuda")
        status = torch.zeros(1, dtype=torch.int32, device="cuda")
        if noalloc:
            codec.sh_encode_noalloc(t, p, xd, x.size, out, cap, info, status)
        else:
            wsb = codec.sh_encode_workspace(x.size, p)
            ws = torch.empty(wsb, dtype=torch.uint8, device="cuda")
            codec.sh_encode(t, p, xd, x.size, out, cap, ws, wsb, info, status)
        torch.cuda.synchronize()
        nbytes = int(info[0].item())
        outs.append((out[:nbytes].cpu().numpy(), info.cpu().numpy(), int(status.item())))
    (a, ia, sa), (b, ib, sb) = outs
    assert sa == 0 and sb == 0
    assert np.array_equal(ia, ib)
    assert a.size == b.size and np.array_equal(a, b)
    return a


@pytest.mark.parametrize("S", [32, 64, 128])
def test_noalloc_matches_sh_encode_twice_the_second_smaller(torch_cuda, S):
    p = codec.Params(K=16, log2_L=7, chunk_symbols=4096, streams=S)
    print(f"case: no-alloc encode S={S}, weight 4096x1024 then tiny 65536", flush=True)
    big = _both(torch_cuda, D.weight(), p)
    small = _both(torch_cuda, D.tiny(), p)
    assert small.size < big.size


def test_noalloc_refuses_tensors_beyond_its_scratch(torch_cuda):
    p = codec.Params(K=16, log2_L=7, chunk_symbols=4096, streams=32)
    limit = codec.sh_encode_noalloc_scratch_bytes()
    n = 1 << 26   # 64 Mi values at 4,096 a chunk: a workspace of 128 MiB
    assert codec.sh_encode_workspace(n, p) > limit
    x = np.zeros(4096, dtype=np.int8)
    t = codec.sh_table_from_histogram(np.bincount(x.astype(np.int16) + 128, minlength=256)
                                      .astype(np.uint64), p)
    xd = torch_cuda.zeros(16, dtype=torch_cuda.int8, device="cuda")
    out = torch_cuda.zeros(16, dtype=torch_cuda.uint8, device="cuda")
    st = codec.lib().sh_encode_noalloc(C.byref(t), C.byref(p.c()), xd.data_ptr(), n,
                                       out.data_ptr(), codec.sh_encode_bound(n, p), None, None, None)
    assert st == -5  # SH_ERR_BUFFER_TOO_SMALL, before any GPU work

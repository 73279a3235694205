"""GPU parity: the HIP codec against the CPU oracle, through the C ABI.

The bar is bit-exactness -- the compressed containers and the decoded tensors -- on the
same seeded inputs.  Small cases are compared whole; full-size workloads are compared
whole on the GPU (round trip) and, against the oracle, on sampled chunks that the
oracle encodes one by one (a chunk's bytes depend only on its values and the table).
"""
from __future__ import annotations

import numpy as np
import pytest

from entropy_coding_quantized_amd import codec
from entropy_coding_quantized_amd import datagen as D
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    codec.lib()  # the HIP library must load; there is no fallback
    return torch


def _table(x, K, log2_L):
    h = O.histogram(x)
    lo, f = O.build_table(h, K, log2_L)
    t = codec.sh_table_from_histogram(h, codec.Params(K=K, log2_L=log2_L))
    assert (t.lo_array == lo).all() and (t.freq_array == f).all()
    return t, lo, f


def _gpu_encode(torch, x, t, p):
    xd = torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda()
    out, info, status = codec.encode_tensor(xd, t, p)
    torch.cuda.synchronize()
    cont, bits = codec.finish_encode(out, info, status)
    return xd, cont, bits


def _gpu_decode(torch, cont, n, t, p):
    y, status = codec.decode_tensor(cont, n, t, p)
    torch.cuda.synchronize()
    return y, int(status.item())


def _case(torch, x, K=16, log2_L=7, C_=4096):
    x = np.ascontiguousarray(x, dtype=np.int8).reshape(-1)
    p = codec.Params(K=K, log2_L=log2_L, chunk_symbols=C_)
    t, lo, f = _table(x, K, log2_L)
    ref, ref_bits = O.encode(x, lo, f, log2_L, C_, 32)
    # GPU decode of the oracle's stream
    y, st = _gpu_decode(torch, torch.from_numpy(ref).cuda(), x.size, t, p)
    assert st == 0
    assert np.array_equal(y.cpu().numpy(), x)
    # GPU encode: byte-identical to the oracle
    _, cont, bits = _gpu_encode(torch, x, t, p)
    got = cont.cpu().numpy()
    assert got.size == ref.size
    if not np.array_equal(got, ref):
        bad = np.nonzero(got != ref)[0]
        raise AssertionError(f"containers differ at {bad.size} bytes, first {bad[:8]}")
    assert bits == ref_bits
    return ref


def test_tiny_workload(torch_cuda):
    print("case: tiny N(0,20) n=65536 K=16 L=128 C=4096", flush=True)
    _case(torch_cuda, D.tiny())


def test_weight_workload(torch_cuda):
    print("case: weight 4096x1024 K=16 L=128 C=4096", flush=True)
    _case(torch_cuda, D.weight())


@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 63, 64, 65, 4095, 4096, 4097, 8191, 12345])
def test_ragged_sizes(torch_cuda, n):
    print(f"case: ragged n={n}", flush=True)
    x = D.quantize(np.random.default_rng(n).normal(0, 15, size=n))
    _case(torch_cuda, x)


@pytest.mark.parametrize("n,C_", [(16384 * 64, 64), (16384 * 64 + 64, 64), (20000 * 32 + 5, 32)])
def test_chunk_counts_around_the_one_kernel_placement(torch_cuda, n, C_):
    """Up to 16384 chunks a tensor the encoder indexes and compacts in one kernel, beyond it
    the index comes first from its own kernel: both give the oracle's container."""
    print(f"case: chunks n={n} C={C_} ({(n + C_ - 1) // C_} chunks)", flush=True)
    x = D.quantize(np.random.default_rng(n).laplace(0, 10, size=n))
    _case(torch_cuda, x, C_=C_)


@pytest.mark.parametrize("K,log2_L,C_", [(1, 7, 4096), (2, 1, 32), (3, 2, 64), (16, 8, 4096),
                                         (64, 8, 1024), (256, 8, 4096), (16, 5, 8192),
                                         (16, 7, 65536), (8, 4, 96), (16, 7, 16384)])
def test_parameter_grid(torch_cuda, K, log2_L, C_):
    print(f"case: grid K={K} R={log2_L} C={C_}", flush=True)
    rng = np.random.default_rng(K * 1000 + log2_L * 10 + C_)
    n = int(rng.integers(3 * C_ // 2, 3 * C_ + 1000)) if C_ <= 16384 else 2 * C_ + 77
    sigma = 60.0 if K >= 64 else 12.0
    x = D.quantize(rng.laplace(0, sigma, size=n))
    h = O.histogram(x)
    if (h > 0).sum() > (1 << log2_L) and K >= (1 << log2_L):
        x = np.clip(x, -(1 << (log2_L - 1)), (1 << (log2_L - 1)) - 1).astype(np.int8)
    _case(torch_cuda, x, K, log2_L, C_)


def test_all_zero_and_uniform(torch_cuda):
    print("case: all-zero and exactly uniform", flush=True)
    ref = _case(torch_cuda, np.zeros(70001, dtype=np.int8))
    assert ref.size > 0
    _case(torch_cuda, D.uniform_exact(300))


def test_histogram_and_device_table_build(torch_cuda):
    torch = torch_cuda
    print("case: device histogram", flush=True)
    for x in [D.weight().reshape(-1), np.zeros(17, np.int8), D.tiny(n=1000003)]:
        xd = torch.from_numpy(x).cuda()
        hd = torch.empty(256, dtype=torch.int64, device="cuda")
        codec.sh_histogram(xd, x.size, hd)
        torch.cuda.synchronize()
        assert np.array_equal(hd.cpu().numpy().astype(np.uint64), O.histogram(x))
        ws = torch.empty(codec.sh_build_tables_workspace(), dtype=torch.uint8, device="cuda")
        t = codec.sh_build_tables(xd, x.size, True, codec.Params(), ws, ws.numel())
        lo, f = O.build_table(O.histogram(x), 16, 7)
        assert (t.lo_array == lo).all() and (t.freq_array == f).all()


def test_symbol_outside_table(torch_cuda):
    torch = torch_cuda
    x = np.zeros(5000, np.int8)
    t, _, _ = _table(x, 16, 7)
    x[4321] = 77
    xd = torch.from_numpy(x).cuda()
    out, info, status = codec.encode_tensor(xd, t, codec.Params())
    torch.cuda.synchronize()
    assert int(status.item()) == codec.SH_ERR_SYMBOL_NOT_IN_TABLE


def test_corruption_matches_oracle(torch_cuda):
    """Damaged containers: the GPU reports exactly what the oracle reports."""
    torch = torch_cuda
    x = D.tiny(n=40000)
    p = codec.Params()
    t, lo, f = _table(x, 16, 7)
    ref, _ = O.encode(x, lo, f, 7, 4096, 32)
    rng = np.random.default_rng(3)
    cases = [ref[:-4], ref[:-1]]
    for _ in range(40):
        bad = ref.copy()
        pos = int(rng.integers(0, bad.size * 8))
        bad[pos // 8] ^= np.uint8(1 << (pos % 8))
        cases.append(bad)
    hb = (32 + 3 * 16 - 1 + 3) // 4 * 4
    bad = ref.copy()
    bad[hb + 8: hb + 12] = np.frombuffer(np.uint32(7).tobytes(), np.uint8)  # misaligned offset
    cases.append(bad)
    agree = 0
    for c in cases:
        st_o, y_o = O.decode(c, x.size, raise_on_error=False)
        cd = torch.from_numpy(np.ascontiguousarray(c)).cuda()
        if c.size < hb + 4 * 11:
            continue
        y, st = _gpu_decode(torch, cd, x.size, t, p)
        assert st in (0, codec.SH_ERR_CORRUPT_STREAM)
        assert (st == 0) == (st_o == 0), (st, st_o)
        if st == 0:
            assert np.array_equal(y.cpu().numpy(), y_o)
        agree += 1
    assert agree > 30


def _sampled_chunk_parity(torch, x, t, lo, f, cont, p, samples=64, seed=0):
    """Compare sampled chunks of a GPU container with the oracle's encoding of them."""
    C_ = p.chunk_symbols
    n = x.size
    nch = (n + C_ - 1) // C_
    K = p.K
    hb = (32 + 3 * K - 1 + 3) // 4 * 4
    head = cont[: hb + 4 * (nch + 1)].cpu().numpy()
    idx = np.frombuffer(head[hb:].tobytes(), dtype="<u4")
    pay0 = hb + 4 * (nch + 1)
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(nch, size=min(samples, nch), replace=False).tolist()) | {0, nch - 1}
    for c in sorted(pick):
        part = x[c * C_: min(n, (c + 1) * C_)]
        one, _ = O.encode(part, lo, f, p.log2_L, C_, 32)
        one_pay = one[hb + 8:]
        got = cont[pay0 + int(idx[c]): pay0 + int(idx[c + 1])].cpu().numpy()
        assert np.array_equal(got, one_pay), f"chunk {c}"


def test_kv_cache_workload(torch_cuda):
    torch = torch_cuda
    cfg = D.CONFIGS["kv_cache"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"])
    kv = D.kv_cache()
    for a in range(2):
        for h in range(8):
            print(f"case: kv_cache kv={a} head={h}", flush=True)
            x = kv[a, h].reshape(-1)
            t, lo, f = _table(x, p.K, p.log2_L)
            xd, cont, bits = _gpu_encode(torch, x, t, p)
            y, st = _gpu_decode(torch, cont, x.size, t, p)
            assert st == 0 and torch.equal(y, xd)
            if h in (0, 5):   # one K head and one V head compared whole with the oracle
                ref, ref_bits = O.encode(x, lo, f, p.log2_L, p.chunk_symbols, 32)
                assert np.array_equal(cont.cpu().numpy(), ref) and bits == ref_bits
            else:
                _sampled_chunk_parity(torch, x, t, lo, f, cont, p, samples=16, seed=h)


def test_activation_workload(torch_cuda):
    torch = torch_cuda
    cfg = D.CONFIGS["activations"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"])
    print("case: activations [16,2048,4096] C=16384", flush=True)
    x = D.activations().reshape(-1)
    t, lo, f = _table(x, p.K, p.log2_L)
    xd, cont, bits = _gpu_encode(torch, x, t, p)
    y, st = _gpu_decode(torch, cont, x.size, t, p)
    assert st == 0 and torch.equal(y, xd)
    _sampled_chunk_parity(torch, x, t, lo, f, cont, p, samples=64)
    s = codec.sh_stats(t, x.size, bits, cont.numel())
    assert s["pct_payload_over_H"] < 1.0


@pytest.mark.parametrize("idx", [0, 3, 1, 4, 6, 117])
def test_model_tensors(torch_cuda, idx):
    torch = torch_cuda
    cfg = D.CONFIGS["model"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"])
    name, shape = D.model_layout()[idx]
    print(f"case: model tensor {idx} {name} {shape}", flush=True)
    x = D.model_tensor(idx).reshape(-1)
    t, lo, f = _table(x, p.K, p.log2_L)
    xd, cont, bits = _gpu_encode(torch, x, t, p)
    y, st = _gpu_decode(torch, cont, x.size, t, p)
    assert st == 0 and torch.equal(y, xd)
    _sampled_chunk_parity(torch, x, t, lo, f, cont, p, samples=32, seed=idx)
    if name == "layers.0.q_proj":
        assert bits == 0

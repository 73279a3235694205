"""GPU parity of the batched calls: tables built on the GPU and many tensors per launch.

Tables built on the GPU must equal the oracle's (lo and freq) and, byte for byte, the
device form of the host-built table; batched encodes must write the oracle's containers
and batched decodes must give back the tensors, on the same seeded inputs.
"""
from __future__ import annotations

import numpy as np
import pytest

from entropy_coding_quantized_amd import codec
from entropy_coding_quantized_amd import datagen as D
import container_layout as CL
from oracle import oracle as O

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_cuda():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    codec.lib()
    return torch


def _mixed_tensors(seed: int, count: int, max_n: int = 120000):
    """Ragged tensors of varied shape, with the degenerate cases among them."""
    rng = np.random.default_rng(seed)
    xs = [np.zeros(0, np.int8), np.zeros(1000, np.int8), np.full(77, -128, np.int8),
          D.uniform_exact(40, seed=seed), D.quantize(rng.normal(0, 0.3, size=5000))]
    while len(xs) < count:
        n = int(rng.integers(1, max_n))
        kind = int(rng.integers(0, 4))
        if kind == 0:
            x = D.quantize(rng.laplace(0, rng.choice([1.0, 4.0, 12.0, 40.0]), size=n))
        elif kind == 1:
            x = D.quantize(rng.normal(rng.integers(-50, 50), rng.choice([2.0, 9.0, 30.0]), size=n))
        elif kind == 2:
            x = D.quantize(rng.standard_t(3, size=n) * 20)
        else:
            x = rng.integers(-128, 128, size=n).astype(np.int8)
        xs.append(x)
    return xs[:count]


def _to_dev(torch, xs):
    return [torch.from_numpy(np.ascontiguousarray(x)).cuda() if x.size else
            torch.empty(16, dtype=torch.int8, device="cuda")[:0] for x in xs]


@pytest.mark.parametrize("K,log2_L", [(16, 7), (1, 7), (2, 1), (3, 2), (8, 8), (64, 8),
                                      (256, 8), (16, 5), (32, 3)])
def test_gpu_table_build_matches_oracle(torch_cuda, K, log2_L):
    torch = torch_cuda
    print(f"case: GPU table build K={K} R={log2_L}", flush=True)
    xs = _mixed_tensors(K * 31 + log2_L, 24)
    p = codec.Params(K=K, log2_L=log2_L)
    dx = _to_dev(torch, xs)
    tables, _ = codec.build_tables_tensors(dx, p)
    torch.cuda.synchronize()
    tb = codec.sh_device_table_bytes()
    host = tables.cpu().numpy()
    # parsing a host copy gives what the device read-back gives
    t_dev, st_dev = codec.sh_tables_from_device(tables, len(xs))
    t_host, st_host = codec.sh_tables_from_bytes(host, len(xs))
    assert st_dev == st_host
    for a_, b_ in zip(t_dev, t_host):
        assert bytes(a_) == bytes(b_)
    for i, x in enumerate(xs):
        h = O.histogram(x)
        part = tables[i * tb:(i + 1) * tb]
        try:
            lo, f = O.build_table(h, K, log2_L)
        except O.OracleError as e:
            with pytest.raises(codec.ShannonicError) as ei:
                codec.table_from_device(part)
            assert ei.value.status == e.status == codec.SH_ERR_UNSUPPORTED
            continue
        t = codec.table_from_device(part)
        assert (t.lo_array == lo).all(), i
        assert (t.freq_array == f).all(), i
        assert (t.hist_array == h).all() and t.n == x.size
        # every derived entry equals the device form of the host-built table
        ht = codec.sh_table_from_histogram(h, p)
        up = codec.tables_to_device([ht], p, "cuda")
        torch.cuda.synchronize()
        assert np.array_equal(up.cpu().numpy(), host[i * tb:(i + 1) * tb]), i


def _check_containers(buf, offs, info, xs, tabs, p, whole=None):
    """Every container against the oracle: whole for the indexes in `whole` (all if None),
    else its header, index and first and last chunks."""
    info = info.cpu().numpy()
    b = buf.cpu().numpy()
    for i, x in enumerate(xs):
        lo, f = tabs[i]
        nbytes, bits = int(info[i, 0]), int(info[i, 1])
        got = b[offs[i]: offs[i] + nbytes]
        if whole is None or i in whole:
            ref, ref_bits = O.encode(x, lo, f, p.log2_L, p.chunk_symbols, p.streams)
            assert got.size == ref.size and np.array_equal(got, ref), f"container {i}"
            assert bits == ref_bits, f"container {i}"
        else:
            C_ = p.chunk_symbols
            nch = (x.size + C_ - 1) // C_
            spans, pay0 = CL.chunk_spans(got, x.size, p.K, C_, p.log2_L, p.streams)
            assert pay0 + (spans[-1][1] + 3) // 4 * 4 == nbytes
            for c in {0, nch // 2, nch - 1}:
                part = x[c * C_: (c + 1) * C_]
                one, _ = O.encode(part, lo, f, p.log2_L, C_, p.streams)
                assert np.array_equal(CL.chunk_bytes(got, x.size, p.K, C_, p.log2_L, c, p.streams),
                                      CL.chunk_bytes(one, part.size, p.K, C_, p.log2_L, 0,
                                                     p.streams)), \
                    f"container {i} chunk {c}"


def _roundtrip_batch(torch, xs, p, whole=None):
    dx = _to_dev(torch, xs)
    tables, _ = codec.build_tables_tensors(dx, p)
    buf, offs, caps, info, st = codec.encode_tensors(tables, dx, p)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, codec.status_string(int(st.item()))
    tabs = [O.build_table(O.histogram(x), p.K, p.log2_L) for x in xs]
    _check_containers(buf, offs, info, xs, tabs, p, whole)
    # decode with the capacity as the readable size (no host round trip needed)
    y, starts, st = codec.decode_tensors(tables, buf, offs, caps, [x.size for x in xs], p)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, codec.status_string(int(st.item()))
    yh = y.cpu().numpy()
    for i, x in enumerate(xs):
        assert np.array_equal(yh[starts[i]: starts[i] + x.size], x), f"tensor {i}"
    return tables, buf, offs, caps, info


@pytest.mark.parametrize("C_,S,n_max", [(4096, 32, 0), (32, 32, 0), (96, 32, 0), (16384, 32, 0),
                                        (4096, 64, 0), (64, 64, 0), (192, 64, 0), (16384, 64, 0),
                                        (64, 64, 50000), (4096, 128, 0), (128, 128, 0)])
def test_batch_mixed_tensors(torch_cuda, C_, S, n_max):
    """More tensors than one launch carries (48), ragged sizes and degenerate tensors.  With
    n_max = 50000 at C = 64 the first launch holds more than 16,384 chunks and the second
    fewer, so chunks of 64 streams go through both decode mappings (16-lane rows with four
    streams a lane, half wavefronts with two)."""
    print(f"case: batch of 61 mixed tensors C={C_} S={S} n_max={n_max}", flush=True)
    if n_max == 0:
        n_max = 120000 if C_ >= 4096 else 9000
    xs = _mixed_tensors(C_, 61, n_max)
    _roundtrip_batch(torch_cuda, xs, codec.Params(chunk_symbols=C_, streams=S))


def test_batch_kv_cache(torch_cuda):
    """The KV-cache layer: one table per (K/V, head), all 16 slabs in one launch each."""
    torch = torch_cuda
    cfg = D.CONFIGS["kv_cache"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"],
                     streams=cfg["streams"])
    print("case: kv_cache batch of 16 slabs", flush=True)
    kv = D.kv_cache()
    xs = [kv[a, h].reshape(-1) for a in range(2) for h in range(8)]
    _roundtrip_batch(torch, xs, p, whole={0, 13})


def test_batch_model_tensors(torch_cuda):
    """Layer 0 of the model-scale layout (with the all-zero and uniform edge tensors) and
    layer 1's k and v projections, full size, in one batch."""
    torch = torch_cuda
    cfg = D.CONFIGS["model"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"],
                     streams=cfg["streams"])
    print("case: model tensors 0..6, 8, 9 batch", flush=True)
    xs = [D.model_tensor(i).reshape(-1) for i in list(range(7)) + [8, 9]]
    _, _, _, _, info = _roundtrip_batch(torch, xs, p, whole={0, 1, 3})
    assert int(info[0, 1].item()) == 0  # all-zero tensor: no field bits


@pytest.mark.parametrize("count,C_,S,n_max", [(61, 4096, 32, 120000), (150, 16384, 64, 400000)])
def test_batch_placement_on_a_second_stream(torch_cuda, count, C_, S, n_max):
    """Batches of two and four launches with a placement stream: every launch's placement
    runs there beside the next launch's chunk kernel, the launches take the workspace's two
    regions in turn, and a decode queued on the main stream after the call reads finished
    containers.  The containers and totals equal the one-stream encode's, byte for byte, and
    the oracle's."""
    torch = torch_cuda
    p = codec.Params(chunk_symbols=C_, streams=S)
    print(f"case: {count} tensors C={C_} S={S} with a placement stream", flush=True)
    xs = _mixed_tensors(1000 + count, count, n_max)
    ns = [x.size for x in xs]
    dx = _to_dev(torch, xs)
    tables, _ = codec.build_tables_tensors(dx, p)
    side = torch.cuda.Stream()
    buf, offs, caps, info, st = codec.encode_tensors(tables, dx, p, place_stream=side)
    y, starts, st2 = codec.decode_tensors(tables, buf, offs, caps, ns, p)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    for i, x in enumerate(dx):
        assert torch.equal(y[starts[i]: starts[i] + ns[i]], x[:ns[i]]), f"tensor {i}"
    buf1, offs1, _, info1, st1 = codec.encode_tensors(tables, dx, p)
    torch.cuda.synchronize()
    assert int(st1.item()) == 0
    assert torch.equal(info, info1)
    b, b1 = buf.cpu().numpy(), buf1.cpu().numpy()
    for i in range(count):
        nb = int(info[i, 0].item())
        assert np.array_equal(b[offs[i]: offs[i] + nb], b1[offs1[i]: offs1[i] + nb]), i
    tabs = [O.build_table(O.histogram(x), p.K, p.log2_L) for x in xs]
    _check_containers(buf, offs, info, xs, tabs, p, whole=set(range(0, count, 10)))


def test_model_first_launch_as_the_bench_runs_it(torch_cuda):
    """The model workload's first launch in the form the bench times it: the first 48
    tensors (the decode and encode batches' launch size), drawn on the GPU by the same
    generator, at C = 16,384 and 64 streams a chunk.  The launch holds about 91,000 chunks,
    so it goes through the 16-lane rows with four streams a lane.  Every GPU-built table
    equals the oracle's, three chunks of every container equal the oracle's encoding of
    them, and every tensor decodes back whole."""
    torch = torch_cuda
    cfg = D.CONFIGS["model"]
    p = codec.Params(K=cfg["K"], log2_L=cfg["log2_L"], chunk_symbols=cfg["chunk"],
                     streams=cfg["streams"])
    print("case: model tensors 0..47 drawn on the GPU, one launch", flush=True)
    dx = [D.model_tensor_torch(i, "cuda").view(-1) for i in range(48)]
    ns = [x.numel() for x in dx]
    assert sum((n + p.chunk_symbols - 1) // p.chunk_symbols for n in ns) >= 16384
    tables, _ = codec.build_tables_tensors(dx, p)
    buf, offs, caps, info, st = codec.encode_tensors(tables, dx, p)
    y, starts, st2 = codec.decode_tensors(tables, buf, offs, caps, ns, p)
    torch.cuda.synchronize()
    assert int(st.item()) == 0 and int(st2.item()) == 0
    for i, x in enumerate(dx):
        assert torch.equal(y[starts[i]: starts[i] + ns[i]], x), f"tensor {i}"
    del y
    xs = [x.cpu().numpy() for x in dx]
    tb = codec.sh_device_table_bytes()
    tabs = []
    for i, x in enumerate(xs):
        lo, f = O.build_table(O.histogram(x), p.K, p.log2_L)
        t = codec.table_from_device(tables[i * tb:(i + 1) * tb])
        assert (t.lo_array == lo).all() and (t.freq_array == f).all(), i
        tabs.append((lo, f))
    _check_containers(buf, offs, info, xs, tabs, p, whole=set())


def test_batch_errors(torch_cuda):
    torch = torch_cuda
    p = codec.Params()
    print("case: batch error reporting", flush=True)
    xs = _mixed_tensors(7, 6)[3:]
    dx = _to_dev(torch, xs)
    tables, _ = codec.build_tables_tensors(dx, p)
    buf, offs, caps, info, st = codec.encode_tensors(tables, dx, p)
    torch.cuda.synchronize()
    assert int(st.item()) == 0
    ns = [x.size for x in xs]
    # one corrupt container among good ones: reported, and the oracle agrees
    b2 = buf.clone()
    i = 1
    nbytes = int(info[i, 0].item())
    pos = offs[i] + CL.payload_at(ns[i], p.K, p.chunk_symbols)  # initial states of lane 0..
    b2[pos] ^= 0x01
    bad = b2[offs[i]: offs[i] + nbytes].cpu().numpy()
    st_o, _ = O.decode(bad, ns[i], raise_on_error=False)
    y, starts, st = codec.decode_tensors(tables, b2, offs, caps, ns, p)
    torch.cuda.synchronize()
    assert (int(st.item()) == codec.SH_ERR_CORRUPT_STREAM) == (st_o != 0)
    # a value outside its table
    x = np.zeros(5000, np.int8)
    t0, _ = codec.build_tables_tensors(_to_dev(torch, [x]), p)
    x[1234] = 55
    _, _, _, _, st = codec.encode_tensors(t0, _to_dev(torch, [x]), p)
    torch.cuda.synchronize()
    assert int(st.item()) == codec.SH_ERR_SYMBOL_NOT_IN_TABLE
    # a table that could not be built: more occupied ranges than states
    q = codec.Params(K=256, log2_L=2)
    xu = D.uniform_exact(10)
    tu, _ = codec.build_tables_tensors(_to_dev(torch, [xu]), q)
    _, _, _, _, st = codec.encode_tensors(tu, _to_dev(torch, [xu]), q)
    torch.cuda.synchronize()
    assert int(st.item()) == codec.SH_ERR_UNSUPPORTED
    with pytest.raises(codec.ShannonicError):
        codec.table_from_device(tu)
    # an empty table decodes nothing
    te, _ = codec.build_tables_tensors(_to_dev(torch, [np.zeros(0, np.int8)]), p)
    y, _, st = codec.decode_tensors(te, buf, [offs[0]], [caps[0]], [ns[0]], p)
    torch.cuda.synchronize()
    assert int(st.item()) == codec.SH_ERR_CORRUPT_STREAM

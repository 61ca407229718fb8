"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle.

Compress: block scales bit-exact; micro-scales and codes bit-exact except within
1e-6 of a rounding boundary (tests/parity.py).  Decompress, fed the oracle's
payload: bit-exact fp32 (and the 1e-6 row rule).  Receiver-side reduce: within
1e-6 of the row maximum of the fp64 oracle sum."""
import os
import sys

import numpy as np
import pytest

import oracle
from fp4_communication_compression_amd import inputs
from tests import bruteforce as bfm
from tests import parity

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def fp4q():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_communication_compression_amd as m
    m.lib()  # raises if the HIP library is missing: no fallback
    oracle.set_threads(16)
    return m


DEV = "cuda:0"


def to_dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(DEV)


def gpu_compress(fp4q, xb, flags=0):
    c, m, b = fp4q.fp4q_compress(to_dev(xb), flags=flags)
    torch.cuda.synchronize()
    return c.cpu().numpy(), m.cpu().numpy(), b.cpu().numpy()


def run_compress_decompress(fp4q, xb, fwht=True, name=""):
    _say("case %s shape %s fwht %s" % (name, xb.shape, fwht))
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    ref = oracle.compress(xb, fwht=fwht, debug=True)
    got = gpu_compress(fp4q, xb, flags)
    stats = parity.check_compress_exact(got, ref)
    # decompress the ORACLE payload on the GPU: equal codes -> bit-exact output
    dp = [to_dev(ref[k]) for k in ("codes", "micro", "block")]
    out = fp4q.fp4q_decompress(*dp, flags=flags)
    out_bf = fp4q.fp4q_decompress(*dp, out_dtype=torch.bfloat16, flags=flags)
    torch.cuda.synchronize()
    want = oracle.decompress(ref["codes"], ref["micro"], ref["block"], fwht=fwht)
    o = out.cpu().numpy()
    np.testing.assert_array_equal(o.view(np.uint32), want.view(np.uint32))
    parity.check_rowwise(o, want)
    ob = out_bf.cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ob, oracle.round_bf16(want))
    return stats


SMALL = [("tiny", lambda: inputs.make_config("tiny")),
         ("one_block", lambda: inputs.make_normal(1, 256, seed=3)),
         ("ragged_37x4096", lambda: inputs.make_normal(37, 4096, seed=4, scale=2.0)),
         ("mlp_5x11008", lambda: inputs.make_normal(5, 11008, seed=5)),
         ("act_rows_100", lambda: inputs.make_config("act2048", rows=100)),
         ("outlier_rows_100", lambda: inputs.make_config("outlier8192", rows=100))]
EDGE = ["zeros", "ones", "spike", "tiny", "huge", "sparse", "ties", "mixed_blocks"]


@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("name,make", SMALL, ids=[s[0] for s in SMALL])
def test_small_cases(fp4q, name, make, fwht):
    st = run_compress_decompress(fp4q, make(), fwht, name)
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0


@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("kind", EDGE)
def test_edge_cases(fp4q, kind, fwht):
    xb = inputs.make_edge_case(kind, 24, 1024, seed=9)
    run_compress_decompress(fp4q, xb, fwht, "edge-" + kind)


def test_empty_tensor(fp4q):
    x = torch.empty((0, 4096), dtype=torch.bfloat16, device=DEV)
    c, m, b = fp4q.fp4q_compress(x)
    out = fp4q.fp4q_decompress(c, m, b)
    torch.cuda.synchronize()
    assert out.shape == (0, 4096)


@pytest.mark.parametrize("name", ["act2048", "outlier8192", "large32768"])
def test_full_size_configs(fp4q, name):
    xb = inputs.make_config(name)
    st = run_compress_decompress(fp4q, xb, True, name)
    _say("  %s: %s" % (name, st))
    if name in ("act2048", "outlier8192"):
        run_compress_decompress(fp4q, xb, False, name + "-nofwht")


def test_determinism(fp4q):
    xb = inputs.make_config("act2048", rows=512)
    x = to_dev(xb)
    first = [t.clone() for t in fp4q.fp4q_compress(x)]
    for _ in range(4):
        again = fp4q.fp4q_compress(x)
        for a, b in zip(first, again):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))
    out0 = fp4q.fp4q_decompress(*first)
    for _ in range(3):
        assert torch.equal(out0, fp4q.fp4q_decompress(*first))


def _reduce_case(fp4q, peers_b, out_dtype=torch.float32, fwht=True):
    ref = [oracle.compress(p, fwht=fwht) for p in peers_b]
    trip = [(r["codes"], r["micro"], r["block"]) for r in ref]
    want = oracle.accumulate_f64(trip, fwht=fwht)
    dev = [tuple(to_dev(a) for a in t) for t in trip]
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    out = fp4q.fp4q_decompress_accumulate(dev, out_dtype=out_dtype, flags=flags)
    torch.cuda.synchronize()
    return out, want


@pytest.mark.parametrize("k", [1, 2, 3, 8, 16])
def test_reduce_small(fp4q, k):
    _say("reduce small k=%d" % k)
    peers = [inputs.make_normal(9, 2048, seed=50 + p, scale=1e-3) for p in range(k)]
    out, want = _reduce_case(fp4q, peers)
    parity.check_rowwise(out.cpu().numpy(), want)


def test_reduce_nofwht_and_bf16(fp4q):
    peers = [inputs.make_normal(7, 1280, seed=70 + p) for p in range(4)]
    out, want = _reduce_case(fp4q, peers, fwht=False)
    parity.check_rowwise(out.cpu().numpy(), want)
    out, want = _reduce_case(fp4q, peers, out_dtype=torch.bfloat16)
    o = out.float().cpu().numpy()
    # bf16 output: within half a bf16 ulp (2^-9 relative) plus the fp32 sum error
    err = np.abs(o - want).max(axis=1)
    assert np.all(err <= (2.0 ** -8) * np.abs(want).max(axis=1))
    # and bit for bit the bf16 rounding (oracle's) of the same sum in fp32
    out32, _ = _reduce_case(fp4q, peers)
    np.testing.assert_array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16),
                                  oracle.round_bf16(out32.cpu().numpy()))


@pytest.fixture(scope="module")
def reduce_peers():
    """The 8 peers of the reduce workload (4096 x 11008, N(0, 1e-3), seeds 4..11)
    and their oracle payloads, made once for the full-size receiver tests."""
    peers = [inputs.make_reduce_peer(p) for p in range(8)]
    trip = [(r["codes"], r["micro"], r["block"]) for r in (oracle.compress(p) for p in peers)]
    return peers, trip


def test_reduce_full_size(fp4q, reduce_peers):
    """k = 8 payloads of 4096 x 11008, N(0, 1e-3), seeds 4..11 -> fp32."""
    _say("reduce full k=8 4096x11008")
    _, trip = reduce_peers
    out = fp4q.fp4q_decompress_accumulate([tuple(to_dev(a) for a in t) for t in trip])
    torch.cuda.synchronize()
    worst = parity.check_rowwise(out.cpu().numpy(), oracle.accumulate_f64(trip))
    _say("  worst row error / row max = %.3e" % worst)


def test_roundtrip_rmse_matches_oracle(fp4q):
    xb = inputs.make_config("act2048", rows=256)
    x = to_dev(xb)
    out = fp4q.fp4q_decompress(*fp4q.fp4q_compress(x))
    torch.cuda.synchronize()
    p = oracle.compress(xb)
    ref = oracle.decompress(p["codes"], p["micro"], p["block"])
    assert oracle.rel_rmse(xb, out.cpu().numpy()) == oracle.rel_rmse(xb, ref)


@pytest.mark.parametrize("k,rows,L", [(1, 4, 256), (2, 37, 4096), (3, 5, 11008), (8, 64, 4096),
                                      (16, 9, 2048)])
def test_requantize_parity(fp4q, k, rows, L):
    _say("requantize k=%d %dx%d" % (k, rows, L))
    peers = [inputs.make_normal(rows, L, seed=200 + p, scale=1e-3) for p in range(k)]
    trip = [(r["codes"], r["micro"], r["block"]) for r in (oracle.compress(p) for p in peers)]
    ref = oracle.requantize(trip, debug=True)
    out = fp4q.fp4q_reduce_requantize([tuple(to_dev(a) for a in t) for t in trip])
    torch.cuda.synchronize()
    st = parity.check_compress([o.cpu().numpy() for o in out], ref)
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0


@pytest.mark.parametrize("kind", ["tiny", "huge", "mixed_blocks", "zeros"])
def test_requantize_edge_cases(fp4q, kind):
    peers = [inputs.make_edge_case(kind, 12, 1024, seed=300 + p) for p in range(3)]
    trip = [(r["codes"], r["micro"], r["block"]) for r in (oracle.compress(p) for p in peers)]
    ref = oracle.requantize(trip, debug=True)
    out = fp4q.fp4q_reduce_requantize([tuple(to_dev(a) for a in t) for t in trip])
    torch.cuda.synchronize()
    parity.check_compress_exact([o.cpu().numpy() for o in out], ref)


def test_requantize_full_size(fp4q, reduce_peers):
    """k = 8 slices of 4096 x 11008 (the reduce workload)."""
    _say("requantize full k=8 4096x11008")
    _, trip = reduce_peers
    ref = oracle.requantize(trip, debug=True)
    out = fp4q.fp4q_reduce_requantize([tuple(to_dev(a) for a in t) for t in trip])
    torch.cuda.synchronize()
    st = parity.check_compress_exact([o.cpu().numpy() for o in out], ref)
    _say("  %s" % st)


def test_max_peers_full_size(fp4q, reduce_peers):
    """The largest peer count, k = 16, at the receiver's real shape (4096 x
    11008).  Peers 8..15 are peers 0..7 doubled: their payloads are the oracle's
    with every block scale doubled, exactly the compress of 2x (scaling by a
    power of two only moves the block scale), and the local slice of the
    re-quantisation (15 peers + the 16th peer's tensor) is 2x peer 7 in bf16.
    The accumulate (fp32 and bf16), the re-quantisation and the re-quantisation
    with the local slice run over the whole tensors, in the launch configuration
    the bench times; sampled rows on both sides of every 1024-row boundary, plus
    random rows, are checked against the oracle on those rows' payload slices
    (blocks never straddle rows), the bf16 output over the whole tensor."""
    _say("max peers k=16 4096x11008")
    peers, trip = reduce_peers
    trip16 = list(trip) + [(c, m, 2.0 * b) for c, m, b in trip]
    local = ((peers[7].astype(np.uint32) << 16).view(np.float32) * 2.0).view(np.uint32) >> 16
    local = local.astype(np.uint16)
    dev = [tuple(to_dev(a) for a in t) for t in trip16]
    acc = fp4q.fp4q_decompress_accumulate(dev)
    accb = fp4q.fp4q_decompress_accumulate(dev, out_dtype=torch.bfloat16)
    req = fp4q.fp4q_reduce_requantize(dev)
    reql = fp4q.fp4q_reduce_requantize(dev[:15], local=to_dev(local))
    torch.cuda.synchronize()
    acc_h = acc.cpu().numpy()
    np.testing.assert_array_equal(accb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  oracle.round_bf16(acc_h))
    rng = np.random.default_rng(16)
    rows = sorted(set([0, 1, 4095] + [b + d for b in (1024, 2048, 3072) for d in (-1, 0)] +
                      rng.integers(0, 4096, 48).tolist()))
    sl = [tuple(a[rows] for a in t) for t in trip16]
    parity.check_rowwise(acc_h[rows], oracle.accumulate_f64(sl))
    parity.check_compress_exact([o.cpu().numpy()[rows] for o in req], oracle.requantize(sl, debug=True))
    parity.check_compress_exact([o.cpu().numpy()[rows] for o in reql],
                                oracle.requantize(sl[:15], debug=True, local=local[rows]))


def run_mx(fp4q, xb, fwht, name):
    _say("mx case %s shape %s fwht %s" % (name, xb.shape, fwht))
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    ref = oracle.compress_mx(xb, fwht=fwht, debug=True)
    c, sc = fp4q.fp4q_compress_mx(to_dev(xb), flags=flags)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(sc.cpu().numpy(), ref["scales"])
    np.testing.assert_array_equal(c.cpu().numpy(), ref["codes"])
    out = fp4q.fp4q_decompress_mx(to_dev(ref["codes"]), to_dev(ref["scales"]), flags=flags)
    outb = fp4q.fp4q_decompress_mx(to_dev(ref["codes"]), to_dev(ref["scales"]),
                                   out_dtype=torch.bfloat16, flags=flags)
    torch.cuda.synchronize()
    want = oracle.decompress_mx(ref["codes"], ref["scales"], fwht=fwht)
    np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
    np.testing.assert_array_equal(outb.cpu().view(torch.int16).numpy().view(np.uint16),
                                  oracle.round_bf16(want))


@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("name,make", SMALL[:4] + [("edge-mixed", lambda: inputs.make_edge_case("mixed_blocks", 24, 1024, seed=9)),
                                               ("edge-tiny", lambda: inputs.make_edge_case("tiny", 24, 1024, seed=9)),
                                               ("edge-zeros", lambda: inputs.make_edge_case("zeros", 8, 1024))],
                         ids=[n for n, _ in SMALL[:4]] + ["edge-mixed", "edge-tiny", "edge-zeros"])
def test_mx_parity(fp4q, name, make, fwht):
    run_mx(fp4q, make(), fwht, name)


def test_mx_full_size(fp4q):
    run_mx(fp4q, inputs.make_config("large32768"), True, "large32768")


def test_graph_capture_replay(fp4q):
    """The entry points allocate nothing and never synchronise, so every one of
    them can be captured in a HIP graph; every replay (with eager work in
    between) must equal the eager result."""
    xb = inputs.make_config("act2048", rows=256)
    x = to_dev(xb)
    codes, micro, block = fp4q.fp4q_compress(x)
    out = fp4q.fp4q_decompress(codes, micro, block)
    peers = [fp4q.fp4q_compress(to_dev(inputs.make_normal(256, 4096, seed=500 + p))) for p in range(3)]
    acc = fp4q.fp4q_decompress_accumulate(peers)
    req = fp4q.fp4q_reduce_requantize(peers, local=x)
    mx = fp4q.fp4q_compress_mx(x)
    mout = fp4q.fp4q_decompress_mx(*mx)
    torch.cuda.synchronize()
    bufs = (codes, micro, block, out, acc, *req, *mx, mout)
    want = [t.clone() for t in bufs]
    for t in bufs:
        t.zero_()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fp4q.fp4q_compress(x, codes, micro, block)
            fp4q.fp4q_decompress(codes, micro, block, out=out)
            fp4q.fp4q_decompress_accumulate(peers, out=acc)
            fp4q.fp4q_reduce_requantize(peers, *req, local=x)
            fp4q.fp4q_compress_mx(x, *mx)
            fp4q.fp4q_decompress_mx(*mx, out=mout)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        for t in bufs:
            t.zero_()                      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(bufs, want):
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), "replay %d differs" % rep


def test_concurrent_streams(fp4q):
    """The library keeps no state: launches on two streams at once give the same
    results as one at a time."""
    xs = [to_dev(inputs.make_normal(512, 4096, seed=600 + i)) for i in range(2)]
    ref = [[t.clone() for t in fp4q.fp4q_compress(x)] for x in xs]
    ref_out = [fp4q.fp4q_decompress(*r) for r in ref]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in range(2)]
    res = [None, None]
    for _ in range(3):
        for i, s in enumerate(streams):
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                p = fp4q.fp4q_compress(xs[i])
                res[i] = (p, fp4q.fp4q_decompress(*p))
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(res[i][0], ref[i]):
                assert torch.equal(a, b)
            assert torch.equal(res[i][1], ref_out[i])
    # the same with the stream passed explicitly (outputs allocated for it)
    for _ in range(3):
        for i, s in enumerate(streams):
            s.wait_stream(torch.cuda.current_stream())
            p = fp4q.fp4q_compress(xs[i], stream=s)
            res[i] = (p, fp4q.fp4q_decompress(*p, stream=s))
        for s in streams:
            torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(2):
            for a, b in zip(res[i][0], ref[i]):
                assert torch.equal(a, b)
            assert torch.equal(res[i][1], ref_out[i])


def test_stacked_tensors_give_stacked_payloads(fp4q):
    """Tensors of one row length stacked into one call: the payload of the stack
    is the payloads of its parts end to end (blocks never straddle rows and every
    payload array is flat in block order), and so is the decompressed output."""
    parts = [inputs.make_normal(r, 4096, seed=40 + i) for i, r in enumerate((37, 2048, 5))]
    pd = [to_dev(p) for p in parts]
    stack = torch.cat(pd, 0)
    whole = fp4q.fp4q_compress(stack)
    each = [fp4q.fp4q_compress(p) for p in pd]
    out_whole = fp4q.fp4q_decompress(*whole)
    out_each = [fp4q.fp4q_decompress(*e) for e in each]
    torch.cuda.synchronize()
    for k in range(3):
        assert torch.equal(whole[k].view(torch.uint8), torch.cat([e[k] for e in each], 0).view(torch.uint8))
    assert torch.equal(out_whole.view(torch.int32), torch.cat(out_each, 0).view(torch.int32))


def test_offsets_beyond_32_bits(fp4q):
    """N = 2^32 + 2^20 elements (rows of 4096): input, code, micro-scale and output
    offsets all pass 2^31 and 2^32 bytes in the tail.  The tensor is a seeded
    1024-row source gathered in a scrambled row order, so a block written to the
    wrong place changes a sampled row.  Sampled rows on both sides of every
    boundary are checked against the oracle; accumulate([P, P]) must equal
    2 x decompress(P) bit for bit over the whole tensor (the sum of two equal
    exact products is exact), and the re-quantisation of [P, P] matches the
    oracle on the sampled rows."""
    L, src_rows = 4096, 1024
    rows = (1 << 20) + 256
    n = rows * L
    free, _ = torch.cuda.mem_get_info()
    if free < 64 << 30:
        pytest.skip("needs about 50 GiB of free device memory")
    _say("offsets beyond 32 bits: %d x %d" % (rows, L))
    xs = inputs.make_normal(src_rows, L, seed=900)
    src_of = (np.arange(rows, dtype=np.int64) * 613 + 11) % src_rows
    x = to_dev(xs).index_select(0, torch.from_numpy(src_of).to(DEV))
    c, m, b = fp4q.fp4q_compress(x)
    mc, ms = fp4q.fp4q_compress_mx(x)
    del x
    out = fp4q.fp4q_decompress(c, m, b)
    torch.cuda.synchronize()

    # rows holding element 2^29, 2^30, 2^31, 2^32 (fp32 output at 2^31 and 2^32
    # bytes, bf16 input at 2^32 bytes, codes at 2^31 bytes) and their neighbours
    edge = [e // L for e in (1 << 29, 1 << 30, 1 << 31, 1 << 32)]
    rng = np.random.default_rng(901)
    pick = sorted(set([0, 1, rows - 2, rows - 1] + [r + d for r in edge for d in (-1, 0)] +
                      list(rng.integers(0, rows, 48))))
    pick_d = torch.tensor(pick, device=DEV)
    src = src_of[pick]
    ref = oracle.compress(xs, debug=True)
    ref_rows = {key: ref[key][src] for key in ref}
    got = [t.index_select(0, pick_d).cpu().numpy() for t in (c, m, b)]
    st = parity.check_compress(got, ref_rows)
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0
    want = oracle.decompress(*got)
    o = out.index_select(0, pick_d).cpu().numpy()
    np.testing.assert_array_equal(o.view(np.uint32), want.view(np.uint32))

    refmx = oracle.compress_mx(xs)
    np.testing.assert_array_equal(ms.index_select(0, pick_d).cpu().numpy(), refmx["scales"][src])
    np.testing.assert_array_equal(mc.index_select(0, pick_d).cpu().numpy(), refmx["codes"][src])
    del mc, ms

    acc = fp4q.fp4q_decompress_accumulate([(c, m, b), (c, m, b)])
    acc_bf = fp4q.fp4q_decompress_accumulate([(c, m, b), (c, m, b)], out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    out.mul_(2.0)
    assert torch.equal(acc, out)
    ob = acc_bf.index_select(0, pick_d).cpu().view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ob, oracle.round_bf16(2.0 * want))
    del acc, acc_bf, out
    # the re-quantisation of two copies of the payload (peer codes read past 2^31
    # bytes, by the multi-peer kernels' contiguous loads): sampled rows
    rq = fp4q.fp4q_reduce_requantize([(c, m, b), (c, m, b)])
    torch.cuda.synchronize()
    got_rq = [t.index_select(0, pick_d).cpu().numpy() for t in rq]
    st = parity.check_compress(got_rq, oracle.requantize([tuple(got)] * 2, debug=True))
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0
    assert n > (1 << 32)
    del rq, c, m, b
    torch.cuda.empty_cache()


def _requantize_local_case(fp4q, peers_b, local_b, fwht, name):
    _say("requantize+local %s k=%d shape %s fwht %s" % (name, len(peers_b), local_b.shape, fwht))
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    trip = [(r["codes"], r["micro"], r["block"])
            for r in (oracle.compress(p, fwht=fwht) for p in peers_b)]
    ref = oracle.requantize(trip, debug=True, local=local_b, fwht=fwht)
    out = fp4q.fp4q_reduce_requantize([tuple(to_dev(a) for a in t) for t in trip],
                                      local=to_dev(local_b), flags=flags)
    torch.cuda.synchronize()
    return parity.check_compress_exact([o.cpu().numpy() for o in out], ref)


@pytest.mark.parametrize("fwht", [True, False])
@pytest.mark.parametrize("k,rows,L", [(0, 37, 4096), (1, 4, 256), (3, 5, 11008), (8, 64, 4096),
                                      (16, 9, 2048)])
def test_requantize_local_parity(fp4q, k, rows, L, fwht):
    """The rank's own bf16 slice added uncompressed, then k peers' payloads."""
    peers = [inputs.make_normal(rows, L, seed=400 + p, scale=1e-3) for p in range(k)]
    local = inputs.make_normal(rows, L, seed=450, scale=1e-3)
    st = _requantize_local_case(fp4q, peers, local, fwht, "%dx%d" % (rows, L))
    assert st["code_mismatch"] == 0 and st["micro_mismatch"] == 0


def test_requantize_local_edge_cases(fp4q):
    peers = [inputs.make_edge_case("tiny", 12, 1024, seed=500 + p) for p in range(2)]
    for kind in ("mixed_blocks", "huge", "zeros", "spike"):
        local = inputs.make_edge_case(kind, 12, 1024, seed=510)
        _requantize_local_case(fp4q, peers, local, True, "edge-" + kind)


@pytest.mark.parametrize("fwht", [True, False])
def test_requantize_local_alone_is_compress(fp4q, fwht):
    """With no peers the re-quantised local slice is exactly its compressed payload."""
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    x = to_dev(inputs.make_config("outlier8192", rows=300))
    a = fp4q.fp4q_reduce_requantize([], local=x, flags=flags)
    b = fp4q.fp4q_compress(x, flags=flags)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8), v.view(torch.uint8))


def test_requantize_local_full_size(fp4q, reduce_peers):
    """An 8-rank slice: 7 received payloads of 4096 x 11008 plus the rank's own
    uncompressed part (the eighth tensor of the reduce workload)."""
    _say("requantize+local full k=7 4096x11008")
    peers, trip = reduce_peers
    ref = oracle.requantize(trip[:7], debug=True, local=peers[7])
    out = fp4q.fp4q_reduce_requantize([tuple(to_dev(a) for a in t) for t in trip[:7]],
                                      local=to_dev(peers[7]))
    torch.cuda.synchronize()
    _say("  %s" % parity.check_compress_exact([o.cpu().numpy() for o in out], ref))


def test_two_exchange_allreduce_emulated(fp4q):
    """The compressed AllReduce of tensor parallelism, as the library's calls compose
    it, for 8 ranks emulated on one GPU: every rank compresses its partial tensor;
    rank j receives row-slice j of the 7 other payloads (payload arrays are
    row-major, so a row-slice is a contiguous view) and re-quantises their sum
    plus its own uncompressed slice; every rank then decompresses the 8 reduced
    slices.  The GPU result equals the same composition through the oracle bit for
    bit, and stays within FP4 error of the exact sum."""
    ranks, rows, L = 8, 64, 4096
    per = rows // ranks
    xs = [inputs.make_normal(rows, L, seed=700 + r, scale=1e-3) for r in range(ranks)]
    # GPU
    xd = [to_dev(x) for x in xs]
    pays = [fp4q.fp4q_compress(x) for x in xd]
    sl = lambda t, j: t[j * per:(j + 1) * per]
    reduced = [fp4q.fp4q_reduce_requantize(
        [tuple(sl(t, j) for t in pays[r]) for r in range(ranks) if r != j], local=sl(xd[j], j))
        for j in range(ranks)]
    out = torch.cat([fp4q.fp4q_decompress(*p) for p in reduced])
    torch.cuda.synchronize()
    # oracle, same composition
    opay = [oracle.compress(x) for x in xs]
    osl = lambda d, j: tuple(d[k][j * per:(j + 1) * per] for k in ("codes", "micro", "block"))
    ored = [oracle.requantize([osl(opay[r], j) for r in range(ranks) if r != j],
                              local=xs[j][j * per:(j + 1) * per]) for j in range(ranks)]
    want = np.concatenate([oracle.decompress(p["codes"], p["micro"], p["block"]) for p in ored])
    for j in range(ranks):
        for got, key in zip(reduced[j], ("codes", "micro", "block")):
            assert np.array_equal(got.cpu().numpy().view(np.uint8), ored[j][key].view(np.uint8)), (j, key)
    o = out.cpu().numpy()
    np.testing.assert_array_equal(o.view(np.uint32), want.view(np.uint32))
    exact = sum(inputs.bf16_bits_to_f32(x).astype(np.float64) for x in xs)
    rel = np.linalg.norm(o - exact) / np.linalg.norm(exact)
    _say("  emulated 8-rank compressed AllReduce: relative error %.4f" % rel)
    assert rel < 0.25


def test_nonfinite_input_stays_in_its_block(fp4q):
    """Non-finite input is outside the method's domain (the result is unspecified),
    but every call completes, and blocks without a NaN or an infinity come out
    exactly as the oracle computes them: the damage stays inside its block."""
    rows, L = 16, 1024
    xb = inputs.make_normal(rows, L, seed=950)
    bad = np.zeros(rows * L // 256, bool)
    flat = xb.reshape(-1)
    for blk, val in ((1, 0x7FC0), (6, 0x7F80), (11, 0xFF80), (20, 0x7FC0), (63, 0xFF80)):
        flat[256 * blk + 37] = val          # bf16 NaN, +Inf, -Inf
        bad[blk] = True
    good = np.repeat(~bad, 256).reshape(rows, L)
    x = to_dev(xb)
    c, m, b = fp4q.fp4q_compress(x)
    out = fp4q.fp4q_decompress(c, m, b)
    acc = fp4q.fp4q_decompress_accumulate([(c, m, b), (c, m, b)])
    req = fp4q.fp4q_reduce_requantize([(c, m, b)], local=x)
    mc, ms = fp4q.fp4q_compress_mx(x)
    mout = fp4q.fp4q_decompress_mx(mc, ms)
    torch.cuda.synchronize()
    ref = oracle.compress(xb)
    g = good.reshape(-1, 256)[:, 0]
    np.testing.assert_array_equal(c.cpu().numpy().reshape(-1, 128)[g], ref["codes"].reshape(-1, 128)[g])
    np.testing.assert_array_equal(m.cpu().numpy().reshape(-1, 16)[g], ref["micro"].reshape(-1, 16)[g])
    np.testing.assert_array_equal(b.cpu().numpy().reshape(-1)[g].view(np.uint32),
                                  ref["block"].reshape(-1)[g].view(np.uint32))
    want = oracle.decompress(ref["codes"], ref["micro"], ref["block"])
    np.testing.assert_array_equal(out.cpu().numpy()[good].view(np.uint32), want[good].view(np.uint32))
    np.testing.assert_array_equal(acc.cpu().numpy()[good], 2 * want[good])
    rq = oracle.requantize([(ref["codes"], ref["micro"], ref["block"])], local=xb)
    np.testing.assert_array_equal(req[0].cpu().numpy().reshape(-1, 128)[g], rq["codes"].reshape(-1, 128)[g])
    rmx = oracle.compress_mx(xb)
    np.testing.assert_array_equal(mc.cpu().numpy().reshape(-1, 128)[g], rmx["codes"].reshape(-1, 128)[g])
    wmx = oracle.decompress_mx(rmx["codes"], rmx["scales"])
    np.testing.assert_array_equal(mout.cpu().numpy()[good].view(np.uint32), wmx[good].view(np.uint32))


@pytest.mark.parametrize("fwht", [True, False])
def test_full_size_invariances(fp4q, fwht):
    """On the 32768 x 4096 tensor, on the GPU alone: negating the input leaves
    every scale and every code magnitude unchanged, and scaling it by 2^-7
    leaves codes and micro-scales unchanged and scales each block scale by
    exactly 2^-7 (both follow from the method's definition)."""
    flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
    x = to_dev(inputs.make_config("large32768")).view(torch.bfloat16)
    c, m, b = fp4q.fp4q_compress(x, flags=flags)
    cn, mn, bn = fp4q.fp4q_compress(-x, flags=flags)
    cs, ms, bs = fp4q.fp4q_compress(x * 2.0 ** -7, flags=flags)    # exact in bf16 here
    torch.cuda.synchronize()
    assert torch.equal(b.view(torch.int32), bn.view(torch.int32))
    assert torch.equal(m, mn)
    assert torch.equal(c & 0x77, cn & 0x77)                        # magnitudes of both nibbles
    assert torch.equal(c, cs) and torch.equal(m, ms)
    assert torch.equal(b * 2.0 ** -7, bs)


SWEEP_CHUNKS = int(os.environ.get("FP4Q_SWEEP_CHUNKS", "10"))   # 40 cases each


@pytest.mark.parametrize("chunk", range(SWEEP_CHUNKS))
def test_random_sweep(fp4q, chunk):
    """Seeded random shapes (1-40 rows, 256-6144 columns) and random per-row
    scales and per-block kinds (make_random_mixture), 400 cases in all (set
    FP4Q_SWEEP_CHUNKS for more), through every entry point, against the oracle
    under the parity rule."""
    rng = np.random.default_rng(4000 + chunk)
    for case in range(40):
        rows, L = int(rng.integers(1, 41)), 256 * int(rng.integers(1, 25))
        seed = int(rng.integers(1 << 30))
        fwht = bool(rng.integers(2))
        flags = 0 if fwht else fp4q.FP4Q_FLAG_NO_FWHT
        _say("sweep %d.%d: %dx%d seed %d fwht %s" % (chunk, case, rows, L, seed, fwht))
        xb = inputs.make_random_mixture(rows, L, seed)
        ref = oracle.compress(xb, fwht=fwht, debug=True)
        parity.check_compress_exact(gpu_compress(fp4q, xb, flags), ref)
        dp = [to_dev(ref[k]) for k in ("codes", "micro", "block")]
        out = fp4q.fp4q_decompress(*dp, flags=flags)
        outb = fp4q.fp4q_decompress(*dp, out_dtype=torch.bfloat16, flags=flags)
        torch.cuda.synchronize()
        want = oracle.decompress(ref["codes"], ref["micro"], ref["block"], fwht=fwht)
        np.testing.assert_array_equal(out.cpu().numpy().view(np.uint32), want.view(np.uint32))
        np.testing.assert_array_equal(outb.cpu().view(torch.int16).numpy().view(np.uint16),
                                      oracle.round_bf16(want))
        # MX round trip
        rmx = oracle.compress_mx(xb, fwht=fwht, debug=True)
        mc, ms = fp4q.fp4q_compress_mx(to_dev(xb), flags=flags)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(ms.cpu().numpy(), rmx["scales"])
        np.testing.assert_array_equal(mc.cpu().numpy(), rmx["codes"])
        mo = fp4q.fp4q_decompress_mx(to_dev(rmx["codes"]), to_dev(rmx["scales"]), flags=flags)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(
            mo.cpu().numpy().view(np.uint32),
            oracle.decompress_mx(rmx["codes"], rmx["scales"], fwht=fwht).view(np.uint32))
        if case % 4 == 0:   # receivers: k peers (plus a local slice for the re-quantisation)
            k = int(rng.integers(1, 17))
            peers = [inputs.make_random_mixture(rows, L, seed + 1 + p) for p in range(k)]
            trip = [(r["codes"], r["micro"], r["block"])
                    for r in (oracle.compress(p, fwht=fwht) for p in peers)]
            dev_trip = [tuple(to_dev(a) for a in t) for t in trip]
            acc = fp4q.fp4q_decompress_accumulate(dev_trip, flags=flags)
            accb = fp4q.fp4q_decompress_accumulate(dev_trip, out_dtype=torch.bfloat16, flags=flags)
            req = fp4q.fp4q_reduce_requantize(dev_trip, local=to_dev(xb), flags=flags)
            req0 = fp4q.fp4q_reduce_requantize(dev_trip, flags=flags)
            torch.cuda.synchronize()
            # the peers' rows carry unrelated scales (2^-30 .. 2^30), so their terms can
            # cancel: the reduce is held to 1e-6 of the summed term magnitudes
            mag = sum(np.abs(oracle.decompress_f64(*t, fwht=fwht)) for t in trip)
            parity.check_rowwise(acc.cpu().numpy(), oracle.accumulate_f64(trip, fwht=fwht),
                                 magnitude=mag)
            # the bf16 output is the bf16 rounding of the same fp32 sum, bit for bit
            np.testing.assert_array_equal(accb.cpu().view(torch.int16).numpy().view(np.uint16),
                                          oracle.round_bf16(acc.cpu().numpy()))
            parity.check_compress_exact([o.cpu().numpy() for o in req],
                                        oracle.requantize(trip, debug=True, local=xb, fwht=fwht))
            parity.check_compress_exact([o.cpu().numpy() for o in req0],
                                        oracle.requantize(trip, debug=True, fwht=fwht))
    _say("  sweep chunk %d: every payload byte exact" % chunk)

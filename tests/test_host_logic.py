"""Host-side arithmetic of the library, checked on the CPU.

The scan-direction remap divides a scan step t < 2^31 by W or H with the
multiply-shift constants of Granlund & Montgomery (PLDI 1994): with
s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1, t // d equals
(umulhi(t, m) + t) >> s.  This restates that formula (as the library computes
it) and checks it against exact integer division, exhaustively for small
divisors and on edge values for large ones.
"""

import random

import pytest


def constants(d):
    s = 0
    while (1 << s) < d:
        s += 1
    m = ((((1 << s) - d) << 32) // d + 1) & 0xFFFFFFFF
    return m, s


def fast_div(t, m, s):
    return (((t * m) >> 32) + t) >> s


def edge_values(d):
    vals = {0, 1, d - 1, d, d + 1, 2 * d - 1, 2 * d, (1 << 31) - 1, (1 << 30), (1 << 30) - 1}
    q = ((1 << 31) - 1) // d
    vals |= {q * d - 1, q * d, q * d + d - 1}
    return [v for v in vals if 0 <= v < (1 << 31)]


@pytest.mark.parametrize("d", list(range(1, 300)) + [1023, 1024, 1025, 4096, 65535, 65536, 1 << 20,
                                                     (1 << 30) - 1, 1 << 30])
def test_fast_division(d):
    m, s = constants(d)
    assert 0 < m < (1 << 32) or d == 1
    rng = random.Random(d)
    for t in edge_values(d) + [rng.randrange(1 << 31) for _ in range(2000)]:
        assert fast_div(t, m, s) == t // d, (t, d)
    if d <= 300:
        for t in range(0, 70 * d):
            assert fast_div(t, m, s) == t // d


# The Spatial SwiGLU kernel numbers its tiles so that each of the 8 XCDs,
# which receive launch slots round robin (slot i on XCD i % 8), gets one
# contiguous run of tiles: slot i -> x * (n // 8) + min(x, n % 8) + i // 8
# with x = i % 8.  Restated here and checked to be a permutation whose runs
# are contiguous per XCD.
def xcd_tile(i, n):
    per, rem = n // 8, n % 8
    x = i % 8
    return x * per + min(x, rem) + i // 8


@pytest.mark.parametrize("n", list(range(1, 70)) + [255, 256, 257, 1023, 1024, 2048, 4099])
def test_xcd_contiguous_tile_order_is_a_permutation(n):
    tiles = [xcd_tile(i, n) for i in range(n)]
    assert sorted(tiles) == list(range(n))
    for x in range(8):
        run = sorted(t for i, t in enumerate(tiles) if i % 8 == x)
        assert run == list(range(run[0], run[0] + len(run))) if run else True


def test_bench_refuses_more_than_one_gpu():
    import subprocess
    import sys
    root = __import__("os").path.dirname(__import__("os").path.dirname(__file__))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root,
                       stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def test_all_cores_oracle_pool_matches_the_oracle():
    # the bench's all-cores CPU figure runs the oracle per (batch, head) slice in
    # spawned worker processes; the slices must reproduce the whole-tensor call
    import numpy as np
    import bench
    from oracle import gla_forward
    from recurrent_vision_token_amd.workloads import Workload, make_inputs
    wl = Workload("pool", 2, 3, 5, 7, 8, 4, 64, "fp32", 1.0, [0, 0], [1, 2])
    host = {0: make_inputs(2, 3, 5, 7, 8, 4, "fp32", 1.0, seed=0)}
    pool, workers = bench.start_oracle_pool(max_workers=2)
    try:
        line = bench.cpu_baseline_pool(wl, host, pool, workers)
        q, k, v, la = host[0]
        slices = [(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1], v[b:b + 1, h:h + 1],
                   la[b:b + 1, h:h + 1], 2) for b in range(2) for h in range(3)]
        got = list(pool.map(bench._oracle_slice, slices))
    finally:
        pool.shutdown()
    ref_o, ref_f = gla_forward(q, k, v, la, 2)
    for (b, h), (o, f) in zip([(b, h) for b in range(2) for h in range(3)], got):
        np.testing.assert_array_equal(o[0, 0], ref_o[b, h])
        np.testing.assert_array_equal(f[0, 0], ref_f[b, h])
    assert line["kind"] == "oracle" and line["cores"] == workers and line["value"] > 0


def test_kernel_bytes_of_both_forward_paths():
    # the two-pass output kernel reads every earlier span's summary (float32
    # state and gate); on the three-pass path the summaries are float16, the
    # scan turns them into float16 entry states in place, and the output
    # kernel reads one entry state per span
    import bench
    from recurrent_vision_token_amd.workloads import WORKLOADS
    wl = WORKLOADS["gtr1.6k"]
    bh, st, gate = wl.B * wl.heads, 64 * 64 * 4, 64 * 4
    st16 = 64 * 64 * 2      # float16 summaries and entry states of the three-pass path
    kv = wl.B * wl.heads * wl.T * 2 * (2 * 64 + 64)       # k, log-alpha, v
    io = wl.B * wl.heads * wl.T * 2 * (3 * 64 + 2 * 64)
    three = bench.kernel_bytes(wl, 13, 3)
    two = bench.kernel_bytes(wl, 13, 2)
    assert three["chunk_output"] == io + bh * st + bh * 13 * st16
    assert three["span_summary"] == kv + bh * 13 * (st16 + gate)
    assert three["span_scan"] == bh * 13 * (st16 + gate + st16)
    assert two["chunk_output"] == io + bh * st + bh * (13 * 12 // 2) * (st + gate)
    assert two["span_summary"] == kv + bh * 13 * (st + gate)
    assert "span_scan" in three and "span_scan" not in two
    assert bench.kernel_bytes(wl, 1, 1) == {"chunk_output": io + bh * st}

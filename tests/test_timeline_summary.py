"""The timeline tool's per-matrix summary (host logic, no GPU): synthetic
records with known stamps give the expected period, staging, tail, gap,
wave spread and per-CU workgroup split (graph plan), and the expected
producer tail, readiness latency, body and store times (persistent plan).
Ticks are the 100 MHz clock's: 100 ticks = 1 us."""
import numpy as np

from weight_streaming_gemv_q8_amd import timeline as tl

NM, LAYERS = 4, 3  # matrices per layer, layers: GEMVs 4..7 are summarized


def _graph_records(grid):
    """GEMV j starts at 2000 j; workgroup b enters at +b and stages 300
    ticks later; its first wave ends 1000 ticks after entry and its last
    one at the same time (b < 8) or 100 ticks later (b >= 8); it exits 10
    ticks after its last wave."""
    by = {}
    for j in range(NM * LAYERS):
        e = np.zeros((grid, tl.NF), dtype=np.int64)
        b = np.arange(grid)
        t0 = 2000 * j
        e[:, 2] = t0 + b
        e[:, 3] = e[:, 2] + 300
        e[:, 4] = e[:, 2] + 1000
        late = np.where(b >= 8, 100, 0)
        e[:, 5] = e[:, 2] + 1000 + late
        e[:, 6] = e[:, 5] + 10
        by[(0, j)] = (grid, e)
    return by


def test_graph_summary_columns():
    grid = 16
    per, keys, heads, sums = tl._graph_summary(np, _graph_records(grid), 1, NM, NM * LAYERS, 8)
    assert len(keys) == len(heads) and "gap" in sums
    for q in range(NM):
        d = per[q]
        assert len(d["period"]) == 1  # only layer 1 is inside layers 1 .. L-2
        assert d["period"][0] == 20.0
        assert d["entry"][0] == (grid - 1) * 0.01
        assert d["staging"][0] == 3.0
        ends = np.arange(grid) + 1010 + np.where(np.arange(grid) >= 8, 100, 0)
        assert np.isclose(d["body"][0], float(np.median(ends)) * 0.01)
        assert np.isclose(d["tail"][0], (ends.max() - np.median(ends)) * 0.01)
        assert np.isclose(d["gap"][0], (2000 - ends.max()) * 0.01)
        assert np.isclose(d["waves"][0], 0.5 * (0.0 + 1.0))  # median of 0 (b < 8) and 100 ticks (b >= 8)
        # workgroups b < 8 and 8 <= b < 16 share CUs: their median ends
        assert np.isclose(d["first_wg"][0], float(np.median(ends[:8])) * 0.01)
        assert np.isclose(d["second_wg"][0], float(np.median(ends[8:16])) * 0.01)


def test_graph_summary_single_round_has_no_cu_split():
    per, *_ = tl._graph_summary(np, _graph_records(8), 1, NM, NM * LAYERS, 8)
    assert all(per[q]["first_wg"] == [] and per[q]["second_wg"] == [] for q in range(NM))


def test_persistent_summary_columns():
    """Op j: workgroup b stores its results at 5000 j + 10 b (the last
    producer 10 (grid - 1) ticks after the first), 50 ticks after its row
    loop ends; every workgroup of op j has its input staged 400 ticks after
    op j - 1's last store, and 700 ticks after it requested its first
    weights."""
    grid = 9
    by = {}
    b = np.arange(grid)
    for j in range(NM * LAYERS):
        e = np.zeros((grid, tl.NF), dtype=np.int64)
        e[:, 0] = j
        e[:, 5] = 5000 * j + 10 * b
        e[:, 4] = e[:, 5] - 50
        e[:, 3] = 5000 * (j - 1) + 10 * (grid - 1) + 400 if j else 0
        e[:, 2] = e[:, 3] - 700
        by[(0, j)] = (grid, e)
    per, keys, heads, sums = tl._persistent_summary(np, by, 1, NM, NM * LAYERS)
    assert keys == heads and sums[0] == "period"
    for q in range(NM):
        d = per[q]
        assert d["period"] == [50.0]
        assert np.isclose(d["prod_tail"][0], (10 * (grid - 1) - float(np.median(10 * b))) * 0.01)
        # ready: the median consumer staged minus the last producer's store
        assert np.isclose(d["ready"][0], 4.0)
        assert np.isclose(d["stage"][0], 7.0)
        assert np.isclose(d["store"][0], 0.5)
        body = by[(0, NM + q)][1][:, 4] - by[(0, NM + q)][1][:, 3]
        assert np.isclose(d["body"][0], float(np.median(body)) * 0.01)
        ends = by[(0, NM + q)][1][:, 4]
        assert np.isclose(d["tail"][0], (ends.max() - float(np.median(ends))) * 0.01)


def test_record_readers_reject_missing_records():
    import pytest
    nwg, nf = tl.NWG, tl.NF
    h = np.zeros(2 * nwg * nf, dtype=np.int64)
    with pytest.raises(RuntimeError):
        tl._persistent_records(h, 2, 0)
    outs = [1 << 12, 2 << 12]
    mod = 7
    h = np.zeros(mod * nwg * nf, dtype=np.int64)
    with pytest.raises(RuntimeError):
        tl._graph_records(h, outs, mod, 0)
    # a complete record set for the persistent layout is accepted
    h = np.zeros(2 * nwg * nf, dtype=np.int64).reshape(2, nwg, nf)
    for j in range(2):
        h[j, :4, 0] = j
        h[j, :4, 1] = np.arange(4) | (4 << 32)
        h[j, :4, 5] = 1
    recs = tl._persistent_records(h.reshape(-1), 2, 0)
    assert set(recs) == {(0, 0), (0, 1)} and recs[(0, 1)][0] == 4

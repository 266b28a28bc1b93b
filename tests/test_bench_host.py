"""Host logic of bench.py that decides which HBM counter figures it reports
(no GPU): an op's traffic is the sum of its kernels' per-launch bytes, and
only where every kernel's counters were taken on the current sources and
their dispatches moved nearly the same bytes."""
import bench

ROWS = "quant_rows_kernel<unsigned short, true, 1, false, false, false>"
AMAX = "amax_kernel<unsigned short, 0>"
FIN = "amax_finalize_kernel"


def entry(label, nbytes, spread=0):
    return {"bytes_per_launch": nbytes, "fetch_spread_bytes": spread, "source_digest": bench.source_digest(label)}


def table(**ents):
    return {"workloads": {"w": dict(ents)}}


def test_own_kernels_are_digested():
    assert bench.own_kernel(ROWS) and bench.own_kernel(FIN) and bench.own_kernel("gemm_fp4_kernel<true, 256, 4, 1, false>")
    assert not bench.own_kernel("vectorized_elementwise_kernel<4, at::native::AbsFunctor<float>>")


def test_single_kernel():
    t = table(**{ROWS: entry(ROWS, 1000, 10)})
    assert bench.traffic_for(ROWS, "w", t) == 1000
    assert bench.traffic_for(ROWS, "other", t) is None


def test_composite_sums_its_kernels():
    t = table(**{AMAX: entry(AMAX, 800, 1), FIN: entry(FIN, 7, 3), ROWS: entry(ROWS, 1000, 2)})
    assert bench.traffic_for(f"{AMAX}+{FIN}+{ROWS}", "w", t) == 1807
    # one kernel missing: no figure
    t2 = table(**{AMAX: entry(AMAX, 800), ROWS: entry(ROWS, 1000)})
    assert bench.traffic_for(f"{AMAX}+{FIN}+{ROWS}", "w", t2) is None


def test_stale_digest_is_not_reported():
    e = entry(ROWS, 1000)
    e["source_digest"] = "0" * 16
    assert bench.traffic_for(ROWS, "w", table(**{ROWS: e})) is None


def test_mixed_sizes_are_not_reported():
    # dispatches of one instantiation on two tensor sizes: the average is neither op's figure
    t = table(**{ROWS: entry(ROWS, 1000, 600)})
    assert bench.traffic_for(ROWS, "w", t) is None
    # a tiny kernel's relative spread does not veto the op it belongs to
    t = table(**{AMAX: entry(AMAX, 800), FIN: entry(FIN, 7, 5), ROWS: entry(ROWS, 1000)})
    assert bench.traffic_for(f"{AMAX}+{FIN}+{ROWS}", "w", t) == 1807


def test_quant_call_label_names_prepass():
    import block_scaled_fp4_amax_amd as F

    q = bench.QuantCall.__new__(bench.QuantCall)
    q.F, q.nv, q.amax, q.dt = F, True, None, F.FP4_BF16
    q.flags = F.FP4_FOUR_OVER_SIX | F.FP4_HADAMARD | F.FP4_TRANSPOSE
    assert q.kernel() == ("amax_kernel<unsigned short, 2>+amax_finalize_kernel+"
                          "quant_cols_kernel<unsigned short, true, 1, false, false, true>")
    q.flags = F.FP4_FOUR_OVER_SIX | F.FP4_HADAMARD
    assert q.kernel().startswith("amax_kernel<unsigned short, 1>+amax_finalize_kernel+quant_rows_kernel<")
    q.flags = F.FP4_FOUR_OVER_SIX
    assert q.kernel() == f"{AMAX}+{FIN}+{ROWS}"
    q.amax = object()  # amax supplied: the quantizer alone
    assert q.kernel() == ROWS

"""Host-side checks of bench.py's live clock reading (no GPU: the samples are planted)."""
import bench


def test_live_clock_summary_leaves_out_the_first_second():
    lc = bench.LiveClock()
    lc.t0 = 100.0
    # (time, mean XCD clock in MHz, socket power in W): the first second still shows the ramp
    lc.samples = [(100.2, 300.0, 250.0), (100.8, 1200.0, 900.0),
                  (101.1, 2000.0, 1350.0), (101.5, 1900.0, None), (102.0, 2100.0, 1370.0)]
    ghz, watts = lc.summary()
    assert ghz == 2.0
    assert watts == 1360.0


def test_live_clock_without_samples_reports_nothing():
    lc = bench.LiveClock()
    lc._h = None   # as where the metrics library is missing or refuses
    with lc:
        pass
    assert lc.summary() == (None, None)
    lc.samples = [(lc.t0 + 0.5, 1900.0, 1300.0)]   # only inside the left-out first second
    assert lc.summary() == (None, None)

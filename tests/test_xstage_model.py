"""The store-path model (X-Stage paper, section 3.2, Eq. 1-7; section 4.2,
Eq. 14-15) as restated in moe_expert_ffn_persistent_amd.xstage, pinned
against an independent discrete simulation of the fluid process the paper
describes (producers inject into a finite buffer that drains at rate R),
and the fits against data drawn from known parameters. CPU only."""
import numpy as np
import pytest

from moe_expert_ffn_persistent_amd import xstage as xs


def simulate(V, t0, R, Q, G, bursts=40, dt=0.001):
    """Periodic bursts of volume V: injection at V/t0 while the outstanding
    volume is below Q (at the drain rate once it is full), drain at R, then a
    gap G. Returns per-burst issue times and start-to-start periods."""
    q = 0.0
    t = 0.0
    starts, issues = [], []
    for _ in range(bursts):
        starts.append(t)
        left = V
        t_issue = 0.0
        while left > 1e-9:
            q = max(0.0, q - R * dt)
            room = max(0.0, Q - q)
            inj = min(left, V / t0 * dt, room)
            q += inj
            left -= inj
            t += dt
            t_issue += dt
        issues.append(t_issue)
        q = max(0.0, q - R * G)
        t += G
    return np.array(issues), np.diff(np.array(starts))


@pytest.mark.parametrize("G", [0.0, 1.0, 3.0, 6.0, 12.0])
def test_periodic_issue_and_period_follow_eq3_and_the_max_law(G):
    # V/R = 8, G* = 6; Q above the isolated peak V - R t0 = 30, so a
    # recovered burst issues at t0
    V, t0, R, Q = 40.0, 2.0, 5.0, 35.0
    iss, per = simulate(V, t0, R, Q, G)
    ss_iss, ss_per = np.median(iss[10:]), np.median(per[10:])
    assert ss_iss == pytest.approx(float(xs.t_iss(G, V, t0, R)), abs=0.02)
    assert ss_per == pytest.approx(float(xs.t_period(G, V, t0, R)), abs=0.02)
    assert ss_iss - t0 == pytest.approx(float(xs.delta_t_iss(G, V, t0, R)), abs=0.02)
    # the period is a max, not the completion-coupled sum G + V/R
    if G > 0:
        assert ss_per < G + V / R - 0.5


def test_recovery_gap_is_the_knee_of_the_sweep():
    V, t0, R, Q = 40.0, 2.0, 5.0, 35.0
    gs = float(xs.g_star(V, t0, R))
    assert gs == pytest.approx(6.0)
    below, _ = simulate(V, t0, R, Q, gs - 1.0)
    above, _ = simulate(V, t0, R, Q, gs + 1.0)
    assert np.median(below[10:]) > t0 + 0.5
    assert np.median(above[10:]) == pytest.approx(t0, abs=0.02)


@pytest.mark.parametrize("V", [4.0, 10.0, 14.0, 30.0, 60.0])
def test_isolated_burst_follows_eq6_and_eq7(V):
    t0_rate = 10.0       # injection at 10 units/us: t0 = V / 10
    t0, R, Q = V / t0_rate, 2.0, 8.0
    iss, _ = simulate(V, t0, R, Q, G=1e6, bursts=1)
    assert iss[0] == pytest.approx(float(xs.t_iss_isolated(V, t0, R, Q)), abs=0.02)
    # below the knee the unconstrained peak stays within the capacity
    if xs.q_peak0(V, t0, R) <= Q:
        assert iss[0] == pytest.approx(t0, abs=0.02)


def test_fits_recover_drain_rate_and_capacity():
    rng = np.random.default_rng(3)
    R, Q = 4.7e6, 3.0e6                               # bytes/us, bytes
    V = np.array([8, 16, 32, 64, 128]) * 2.0 ** 20
    T = V / R * (1 + 0.01 * rng.standard_normal(len(V)))
    assert xs.fit_drain_rate(V, T) == pytest.approx(R, rel=0.02)
    Vi = np.array([0.5, 1, 2, 4, 8, 16, 32, 64]) * 2.0 ** 20
    t0 = Vi / 30e6 + 0.5                              # issue-rate floor per volume
    Ti = np.array([float(xs.t_iss_isolated(v, a, R, Q)) for v, a in zip(Vi, t0)])
    assert xs.fit_capacity(Vi, Ti, t0, R) == pytest.approx(Q, rel=1e-6)
    assert xs.fit_capacity(Vi[:2], Ti[:2], t0[:2], R) is None


def test_eq14_is_the_interleaved_gap_reaching_g_star():
    rng = np.random.default_rng(5)
    for _ in range(200):
        n1, n2 = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        V, t0, R = rng.uniform(1e5, 1e8), rng.uniform(0.1, 10), rng.uniform(1e5, 1e7)
        tl1, tl2 = rng.uniform(1, 200), rng.uniform(1, 100)
        g_int = tl2 + n1 / n2 * tl1                     # Eq. 12
        assert xs.interleave_sufficient(n1, n2, V, t0, R, tl1, tl2) == (g_int >= xs.g_star(V, t0, R))
    assert xs.critical_stall([3.0, 1.0], [2.0, 2.0]).tolist() == [1.0, 0.0]


def test_tile_spans_from_a_hand_made_trace():
    khz = 100_000                                      # 100 MHz: 100 ticks per us
    tr = np.full((2, 4, 10), -1, dtype=np.int64)
    # instance 0: Linear-1 then Linear-2; instance 1: one Linear-2
    tr[0, 0] = [1 | 0 << 2, 0, 1000, 1000, 5000, 5600, 0, 0, 5600, 0]
    tr[0, 1] = [2 | 3 << 2, 0, 5600, 5700, 8700, 9200, 0, 0, 9900, 0]
    tr[1, 0] = [2 | 1 << 2, 0, 5000, 5100, 8800, 9000, 0, 0, 9400, 8]
    s = xs.tile_spans(tr.astype(np.int32), khz)
    assert s["l2_tiles"] == 2
    assert s["t_rs_us"]["median"] == pytest.approx((5.0 + 2.0) / 2)     # 500 and 200 ticks
    assert s["drain_lag_us"]["median"] == pytest.approx((7.0 + 4.0) / 2)
    # span [8700, 9200) shares 200 of its 500 ticks; [8800, 9000) all of its 200
    assert s["k_act"]["median"] == pytest.approx((1.4 + 2.0) / 2)
    assert s["mainloop_us"]["l1"] == pytest.approx(40.0)


def test_burst_concurrency_counts_open_intervals():
    # three producers: 0 and 1 overlap for half of 0's burst, 2 stands alone
    start = np.array([[0, 100], [50, 200], [400, 500]])
    end = np.array([[100, 150], [150, 260], [450, 500]])
    c = xs.burst_concurrency(start, end)
    assert c[0, 0] == pytest.approx(1.5)          # 50 ticks alone, 50 with producer 1
    assert c[1, 0] == pytest.approx(2.0)          # [50,150): producer 0 issues throughout
    assert c[0, 1] == pytest.approx(2.0)          # [100,150) inside producer 1's burst
    assert c[1, 1] == pytest.approx(1.0)
    assert c[2, 0] == pytest.approx(1.0)
    assert c[2, 1] == pytest.approx(1.0)          # zero-length burst counts itself
    # K producers issuing the same interval
    K = 7
    assert (xs.burst_concurrency(np.zeros((K, 1)), np.full((K, 1), 10)) == K).all()

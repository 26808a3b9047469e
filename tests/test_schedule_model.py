"""Pins of the CPU schedule model (X-Stage paper, section 4.2, Algorithm 1,
and the Expert-Wave order of section 2.2): a hand-traced fixture, exactly-once
coverage, dependency safety by simulation, and the special cases."""
import itertools
import os
import random

import pytest

from oracle import schedule as sc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _parse_task(t):
    kind = 1 if t.startswith("L1") else 2
    p, n = t[3:-1].split(",")
    return (kind, int(p), int(n))


def test_alg1_hand_trace():
    streams = {}
    prm = {}
    for line in open(os.path.join(GOLDEN, "alg1_small.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("params"):
            prm = dict(kv.split("=") for kv in line.split()[1:])
            continue
        g, rest = line.split(":")
        streams[int(g)] = [_parse_task(t) for t in rest.split()]
    P, N1, N2, G, D = (int(prm[x]) for x in ("P", "N1", "N2", "G", "D"))
    for g in range(G):
        assert sc.interleaved_stream(g, G, P, N1, N2, D) == streams[g]


def _read_wave_fixture():
    cases = []
    for line in open(os.path.join(GOLDEN, "expert_wave_small.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("params"):
            prm = dict(kv.split("=") for kv in line.split()[1:])
            cases.append({"tile_offset": [int(v) for v in prm["tile_offset"].split(",")],
                          "N1": int(prm["N1"]), "N2": int(prm["N2"]), "G": int(prm["G"]),
                          "epw": int(prm["experts_per_wave"]), "streams": {}})
        elif line.startswith("waves"):
            cases[-1]["waves"] = [tuple(int(v) for v in w.split("-")) for w in line.split()[1:]]
        else:
            g, rest = line.split(":")
            cases[-1]["streams"][int(g)] = [_parse_task(t) for t in rest.split()]
    return cases


def test_expert_wave_multi_wave_hand_trace():
    # three waves, an expert without rows, a partial last wave; greedy and
    # fixed-size grouping (X-Stage paper, section 2.2, Figure 4(a))
    cases = _read_wave_fixture()
    assert len(cases) == 2
    for c in cases:
        waves = sc.waves_greedy(c["tile_offset"], c["N1"], c["G"], c["epw"])
        assert waves == c["waves"]
        streams = sc.all_streams("expert_wave", c["G"], c["tile_offset"], c["N1"], c["N2"],
                                 experts_per_wave=c["epw"])
        assert streams == [c["streams"][g] for g in range(c["G"])]


def test_dknee_fixture():
    for line in open(os.path.join(GOLDEN, "dknee.txt")):
        if line.startswith("#") or not line.strip():
            continue
        bn, K, h, want = map(int, line.split())
        assert sc.d_knee(bn, K, h) == want


def _all_tasks(P, N1, N2):
    return ({(1, p, n) for p in range(P) for n in range(N1)}
            | {(2, p, n) for p in range(P) for n in range(N2)})


def _simulate(streams, N1, max_steps=10 ** 6):
    """Run every instance's stream in order; a Linear-2 tile of row p may run
    only once all N1 Linear-1 tiles of row p have run. Returns True when all
    streams drain, False on deadlock."""
    pos = [0] * len(streams)
    done_l1 = {}
    remaining = sum(len(s) for s in streams)
    while remaining:
        progressed = False
        for g, s in enumerate(streams):
            if pos[g] == len(s):
                continue
            kind, p, n = s[pos[g]]
            if kind == 2 and done_l1.get(p, 0) < N1:
                continue
            if kind == 1:
                done_l1[p] = done_l1.get(p, 0) + 1
            pos[g] += 1
            remaining -= 1
            progressed = True
        if not progressed:
            return False
    return True


@pytest.mark.parametrize("seed", range(40))
def test_streams_cover_every_task_once_and_never_deadlock(seed):
    rnd = random.Random(seed)
    L = rnd.randint(1, 6)
    counts = [rnd.choice([0, 1, 2, 3, 5]) for _ in range(L)]
    tile_offset = [0]
    for c in counts:
        tile_offset.append(tile_offset[-1] + c)
    P = tile_offset[-1]
    N1, N2 = rnd.randint(1, 5), rnd.randint(1, 7)
    G = rnd.randint(1, 9)
    for schedule in ("interleaved", "expert_wave"):
        for D in (1, 2, 5, P + 1):
            streams = sc.all_streams(schedule, G, tile_offset, N1, N2, D,
                                     experts_per_wave=rnd.choice([0, 1, 2]))
            got = [t for s in streams for t in s]
            assert len(got) == len(set(got))
            assert set(got) == _all_tasks(P, N1, N2)
            assert _simulate(streams, N1)


def test_lead_zero_can_deadlock():
    # with D = 0 an instance can wait on a Linear-1 tile it has not issued yet
    streams = [sc.interleaved_stream(g, 1, 2, 2, 1, 0) for g in range(1)]
    assert streams[0][0] == (2, 0, 0)
    assert not _simulate(streams, 2)


def test_large_lead_is_all_l1_then_all_l2_and_equals_one_wave():
    tile_offset = [0, 2, 3, 7]
    P, N1, N2, G = 7, 3, 4, 5
    for g in range(G):
        s = sc.interleaved_stream(g, G, P, N1, N2, D=P)
        kinds = [t[0] for t in s]
        assert kinds == sorted(kinds)
    inter = sc.all_streams("interleaved", G, tile_offset, N1, N2, D=P)
    wave = sc.all_streams("expert_wave", G, tile_offset, N1, N2, experts_per_wave=3)
    assert inter == wave


def test_greedy_waves_close_at_instance_count():
    # expert rows 1,1,2,0,3 with N1=4, G=8: waves close at >= 8 L1 tiles
    tile_offset = [0, 1, 2, 4, 4, 7]
    assert sc.waves_greedy(tile_offset, 4, 8) == [(0, 2), (2, 4), (4, 7)]
    assert sc.waves_greedy(tile_offset, 4, 8, experts_per_wave=2) == [(0, 2), (2, 4), (4, 7)]
    assert sc.waves_greedy(tile_offset, 4, 100) == [(0, 7)]


def test_expert_of_row():
    tile_offset = [0, 2, 2, 5]
    assert [sc.expert_of_row(tile_offset, p) for p in range(5)] == [0, 0, 2, 2, 2]

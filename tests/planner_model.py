"""Timing model of the persistent task streams, written independently of the
library's schedule planner (moe_predict_schedule) to test it.

The streams come from the CPU schedule model (oracle/schedule.py, pinned by
its own tests to hand-traced fixtures of Algorithm 1 and the Expert-Wave
order); the planner instead runs the kernel's stream code on the host. The
costs are the planner's documented model: a Linear-1 task costs H/128 + 2
units, a Linear-2 task I/128 + 2, and a Linear-2 task of row p starts once
every Linear-1 task of p has ended, its instance waiting in place until then.
"""
from __future__ import annotations

import heapq

from oracle import schedule as sc


def tile_offsets(counts, block_m):
    off = [0]
    for c in counts:
        off.append(off[-1] + -(-int(c) // block_m))
    return off


def simulate(streams, off, N1, c1, c2, w1_bytes, w2_bytes):
    """Returns (makespan, time-averaged weight bytes in use). Instances take
    their next task in the order of the time they become free."""
    P = off[-1]
    expert = [sc.expert_of_row(off, p) for p in range(P)]
    G = len(streams)
    pos = [0] * G
    done = [0] * P
    ready = [0.0] * P
    waiting = {}
    busy = {}   # (expert, linear) -> intervals during which a task reads that matrix
    heap = [(0.0, g) for g in range(G)]
    end_all = 0.0
    while heap:
        t, g = heapq.heappop(heap)
        if pos[g] == len(streams[g]):
            end_all = max(end_all, t)
            continue
        kind, p, _ = streams[g][pos[g]]
        if kind == 2 and done[p] < N1:
            waiting.setdefault(p, []).append((t, g))
            continue
        pos[g] += 1
        if kind == 1:
            end = t + c1
            busy.setdefault((expert[p], 1), []).append((t, end))
            ready[p] = max(ready[p], end)
            done[p] += 1
            if done[p] == N1:
                for tw, gw in waiting.pop(p, []):
                    heapq.heappush(heap, (max(tw, ready[p]), gw))
        else:
            start = max(t, ready[p])
            end = start + c2
            busy.setdefault((expert[p], 2), []).append((start, end))
        heapq.heappush(heap, (end, g))
    assert not waiting, "streams deadlocked"
    area = 0.0
    for (e, lin), iv in busy.items():
        iv.sort()
        cs, ce = iv[0]
        length = 0.0
        for s, t in iv[1:]:
            if s > ce:
                length += ce - cs
                cs, ce = s, t
            else:
                ce = max(ce, t)
        length += ce - cs
        area += length * (w1_bytes if lin == 1 else w2_bytes)
    return end_all, (area / end_all if end_all > 0 else 0.0)


def predict(counts, block_m, N1, N2, G, H, I, weight_bytes, schedule, lead_d=1, experts_per_wave=0):
    off = tile_offsets(counts, block_m)
    if off[-1] == 0:
        return 0.0, 0.0
    streams = sc.all_streams(schedule, G, off, N1, N2, D=lead_d, experts_per_wave=experts_per_wave)
    return simulate(streams, off, N1, H / 128 + 2, I / 128 + 2, 2 * I * H * weight_bytes,
                    H * I * weight_bytes)

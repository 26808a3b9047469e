"""Timing model of the persistent task streams, written independently of the
library's schedule planner (moe_predict_schedule) to test it.

The streams come from the CPU schedule model (oracle/schedule.py, pinned by
its own tests to hand-traced fixtures of Algorithm 1 and the Expert-Wave
order); the planner instead runs the kernel's stream code on the host. The
costs are the planner's documented model: a Linear-1 task costs H/128 + 2
units, a Linear-2 task I/128 + 2, and a Linear-2 task of row p starts once
every Linear-1 task of p has ended, its instance waiting in place until then.
The reads of each task (its weight tile, then its activation block) go, in
start order, through an LRU cache of the Infinity Cache's size.
"""
from __future__ import annotations

import collections
import heapq

from oracle import schedule as sc

CACHE_BYTES = 256.0 * 1024 * 1024   # the Infinity Cache


def tile_offsets(counts, block_m):
    off = [0]
    for c in counts:
        off.append(off[-1] + -(-int(c) // block_m))
    return off


def lru_misses(reads, capacity=CACHE_BYTES):
    """Bytes of an access sequence [(key, bytes), ...] that miss an LRU cache
    of `capacity` bytes (an entry that does not fit is dropped at once), and
    the bytes of the distinct keys."""
    cache = collections.OrderedDict()
    used = miss = 0.0
    distinct = {}
    for key, nbytes in reads:
        distinct[key] = nbytes
        if key in cache:
            cache.move_to_end(key)
            continue
        miss += nbytes
        cache[key] = nbytes
        used += nbytes
        while used > capacity and cache:
            used -= cache.popitem(last=False)[1]
    return miss, sum(distinct.values())


def simulate(streams, off, N1, c1, c2, w1_bytes, w2_bytes, tiles=None):
    """Returns (makespan, time-averaged weight bytes in use) and, with
    tiles = (W1 tile, token block, W2 tile, h block) bytes, the LRU misses
    and distinct bytes of every task's reads (weight tile, then activation
    block) in start order (time, then instance). Instances take their next
    task in the order of the time they become free."""
    P = off[-1]
    expert = [sc.expert_of_row(off, p) for p in range(P)]
    G = len(streams)
    pos = [0] * G
    done = [0] * P
    ready = [0.0] * P
    waiting = {}
    busy = {}   # (expert, linear) -> intervals during which a task reads that matrix
    starts = []   # (start, instance, kind, row, N-tile)
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
        n = streams[g][pos[g] - 1][2]
        if kind == 1:
            end = t + c1
            starts.append((t, g, 1, p, n))
            busy.setdefault((expert[p], 1), []).append((t, end))
            ready[p] = max(ready[p], end)
            done[p] += 1
            if done[p] == N1:
                for tw, gw in waiting.pop(p, []):
                    heapq.heappush(heap, (max(tw, ready[p]), gw))
        else:
            start = max(t, ready[p])
            end = start + c2
            starts.append((start, g, 2, p, n))
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
    ws = area / end_all if end_all > 0 else 0.0
    if tiles is None:
        return end_all, ws
    w1t, xb, w2t, hb = tiles
    reads = []
    for t, g, kind, p, n in sorted(starts, key=lambda a: (a[0], a[1])):
        if kind == 1:
            reads += [(("W1", expert[p], n), w1t), (("x", p), xb)]
        else:
            reads += [(("W2", expert[p], n), w2t), (("h", p), hb)]
    miss, distinct = lru_misses(reads)
    return end_all, ws, miss, distinct


def predict(counts, block_m, N1, N2, G, H, I, weight_bytes, schedule, lead_d=1, experts_per_wave=0,
            block_n1=None, block_n2=None, act_bytes=None):
    """(makespan, working set), or with block_n1, block_n2 and act_bytes (bytes
    per token or h element) also (HBM bytes, distinct bytes) of the reads."""
    off = tile_offsets(counts, block_m)
    tiles = None
    if block_n1 is not None:
        tiles = (block_n1 * H * weight_bytes, block_m * H * act_bytes, block_n2 * I * weight_bytes,
                 block_m * I * act_bytes)
    if off[-1] == 0:
        return (0.0, 0.0) if tiles is None else (0.0, 0.0, 0.0, 0.0)
    streams = sc.all_streams(schedule, G, off, N1, N2, D=lead_d, experts_per_wave=experts_per_wave)
    return simulate(streams, off, N1, H / 128 + 2, I / 128 + 2, 2 * I * H * weight_bytes,
                    H * I * weight_bytes, tiles)

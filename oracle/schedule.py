"""CPU model of the persistent kernel's two tile schedules.

TEST INFRASTRUCTURE ONLY (see ``oracle/moe_oracle.py``): nothing on the
product path imports it, and it imports nothing from there.

Tasks are (kind, p, n): kind 1 is a Linear-1 tile (scheduler row p, N-tile n
of the gate/up output, N1 tiles per row), kind 2 a Linear-2 tile (row p,
N-tile n of the hidden output, N2 tiles per row). Scheduler rows p are the
M-blocks of all local experts laid end to end, expert e owning rows
O_e .. O_{e+1}-1 (X-Stage paper, Algorithm 1 legend).

Interleaved order (X-Stage paper, section 4.2, Algorithm 1): instance g keeps
two cursors k1 and k2, both starting at g and advancing by the instance count
G. Row p_i = floor(k_i / N_i). It emits the Linear-2 tile at k2 when that
stream is not finished and p2 + D <= p1, where p1 is taken as +infinity once
the Linear-1 stream is finished; otherwise it emits the Linear-1 tile at k1.
The paired-CTA role r of the paper is dropped (one instance per tile), so the
N-tile index is simply k mod N_i.

Expert-Wave order (section 2.2; Figure 4(a)): local experts are grouped into
waves; the wave's Linear-1 tiles run, then its Linear-2 tiles, then the next
wave. Within each wave, each of the two tile streams is walked the way
Algorithm 1 walks its streams (cursor starts at g and advances by G; the
persistent tile visitor of the resource-management paper, section C, takes
tiles b, b+G, b+2G, ... the same way). With one wave holding every row this
is exactly Algorithm 1 with a lead D >= P. The wave size is not given on the
pages; the reading taken here closes a wave, in local-expert order, as soon
as it holds at least G Linear-1 tiles (one tile for every instance).
"""
from __future__ import annotations

import math

L1, L2 = 1, 2

__all__ = ["L1", "L2", "expert_of_row", "waves_greedy", "expert_wave_stream",
           "interleaved_stream", "d_knee", "all_streams"]


def expert_of_row(tile_offset, p: int) -> int:
    """e(p): the expert whose scheduler rows contain p."""
    for e in range(len(tile_offset) - 1):
        if tile_offset[e] <= p < tile_offset[e + 1]:
            return e
    raise ValueError(p)


def waves_greedy(tile_offset, N1: int, G: int, experts_per_wave: int = 0):
    """Wave boundaries as scheduler-row ranges [(r0, r1), ...]. With
    experts_per_wave > 0, waves take that many experts each; otherwise a wave
    closes once it holds >= G Linear-1 tiles. Experts with no rows are skipped
    over (they add no rows). The last wave takes whatever is left."""
    L = len(tile_offset) - 1
    waves = []
    start = tile_offset[0]
    n_exp = 0
    for e in range(L):
        n_exp += 1
        r1 = tile_offset[e + 1]
        full = (n_exp >= experts_per_wave) if experts_per_wave > 0 else ((r1 - start) * N1 >= G)
        if full or e == L - 1:
            if r1 > start:
                waves.append((start, r1))
            start = r1
            n_exp = 0
    return waves


def expert_wave_stream(g: int, G: int, waves, N1: int, N2: int):
    """Tasks of instance g under the Expert-Wave order."""
    seq = []
    for (r0, r1) in waves:
        rows = r1 - r0
        seq += [(L1, r0 + t // N1, t % N1) for t in range(g, rows * N1, G)]
        seq += [(L2, r0 + t // N2, t % N2) for t in range(g, rows * N2, G)]
    return seq


def interleaved_stream(g: int, G: int, P: int, N1: int, N2: int, D: int):
    """Tasks of instance g under Algorithm 1."""
    out = []
    k1 = k2 = g
    while k1 < P * N1 or k2 < P * N2:
        p1 = k1 // N1 if k1 < P * N1 else math.inf
        p2 = k2 // N2
        if k2 < P * N2 and p2 + D <= p1:
            out.append((L2, p2, k2 % N2))
            k2 += G
        else:
            out.append((L1, p1, k1 % N1))
            k1 += G
    return out


def d_knee(block_n: int, instances: int, inter: int) -> int:
    """Anti-starvation lead (X-Stage paper, Eq. 16): ceil(b_n * K / (2 h)),
    with b_n the Linear-1 N-tile width, K the number of concurrently
    advancing instances and h the expert intermediate size."""
    return -(-block_n * instances // (2 * inter))


def all_streams(schedule: str, G: int, tile_offset, N1: int, N2: int, D: int = 1,
                experts_per_wave: int = 0):
    P = int(tile_offset[-1])
    if schedule == "interleaved":
        return [interleaved_stream(g, G, P, N1, N2, D) for g in range(G)]
    waves = waves_greedy(list(tile_offset), N1, G, experts_per_wave)
    return [expert_wave_stream(g, G, waves, N1, N2) for g in range(G)]

"""CPU model of the persistent kernel's two tile schedules.

TEST INFRASTRUCTURE ONLY (see ``oracle/moe_oracle.py``): nothing on the
product path imports it, and it imports nothing from there.

Tasks are (kind, p, n): kind 1 is a Linear-1 tile (scheduler row p, N-tile n
of the gate/up output, N1 tiles per row), kind 2 a Linear-2 tile (row p,
N-tile n of the hidden output, N2 tiles per row). Scheduler rows p are the
M-blocks of all local experts laid end to end, expert e owning rows
O_e .. O_{e+1}-1 (X-Stage paper, Algorithm 1 legend).

Both orders are written here from the properties the pages state, not as a
cursor machine, so that they check the kernel's stream code (which is one)
from another direction:

Interleaved order (X-Stage paper, section 4.2, Algorithm 1): instance g owns
the Linear-1 tiles whose global index k = p*N1 + n is g modulo G and the
Linear-2 tiles whose index k = p*N2 + n is g modulo G, and runs each kind in
ascending index. The two kinds are merged by the lead rule: a Linear-2 tile
of row p goes ahead of the instance's next Linear-1 tile exactly when that
tile's row is at least p + D (or no Linear-1 tile is left). The paired-CTA
role of the paper is dropped (one instance per tile), so n = k mod N_i.

Expert-Wave order (section 2.2; Figure 4(a)): local experts are grouped into
waves; all Linear-1 tiles of a wave run, then its Linear-2 tiles, then the
next wave. The tiles of one wave and kind are enumerated row by row, N-tile by
N-tile, and instance g takes every G-th of them starting at the g-th (the
persistent tile visitor of the resource-management paper, section C, takes
tiles b, b+G, b+2G, ... the same way). With one wave holding every row this
is exactly Algorithm 1 with a lead D >= P. The wave size is not given on the
pages; the reading taken here closes a wave, in local-expert order, as soon
as it holds at least G Linear-1 tiles (one tile for every instance); the
last wave takes the rest.
"""
from __future__ import annotations

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
    """Wave boundaries as scheduler-row ranges [(r0, r1), ...]. The local
    experts are cut into consecutive groups: groups of experts_per_wave
    experts when that is positive (the last group takes what is left);
    otherwise each group runs from its first expert to the first expert at
    which the group's Linear-1 tile count, N1 times its rows, reaches G, or
    to the last expert. Groups without rows are dropped."""
    L = len(tile_offset) - 1
    groups = []                        # [first expert, one past the last expert)
    a = 0
    while a < L:
        if experts_per_wave > 0:
            b = min(L, a + experts_per_wave)
        else:
            full = [e + 1 for e in range(a, L) if (tile_offset[e + 1] - tile_offset[a]) * N1 >= G]
            b = full[0] if full else L
        groups.append((a, b))
        a = b
    return [(tile_offset[a], tile_offset[b]) for a, b in groups if tile_offset[b] > tile_offset[a]]


def _phase_tiles(kind: int, r0: int, r1: int, N: int):
    """The tiles of one kind over rows r0..r1-1, row by row, N-tile by N-tile."""
    return [(kind, p, n) for p in range(r0, r1) for n in range(N)]


def expert_wave_stream(g: int, G: int, waves, N1: int, N2: int):
    """Tasks of instance g under the Expert-Wave order: per wave, every G-th
    Linear-1 tile from the g-th, then every G-th Linear-2 tile from the g-th."""
    seq = []
    for (r0, r1) in waves:
        seq += _phase_tiles(L1, r0, r1, N1)[g::G]
        seq += _phase_tiles(L2, r0, r1, N2)[g::G]
    return seq


def interleaved_stream(g: int, G: int, P: int, N1: int, N2: int, D: int):
    """Tasks of instance g under Algorithm 1: the instance's own Linear-1 and
    Linear-2 tiles (every G-th from the g-th, ascending), merged so that each
    Linear-2 tile of row p follows exactly the own Linear-1 tiles of rows
    below p + D that precede it in ascending order."""
    own1 = _phase_tiles(L1, 0, P, N1)[g::G]
    own2 = _phase_tiles(L2, 0, P, N2)[g::G]
    out = []
    i = 0
    for t2 in own2:
        while i < len(own1) and own1[i][1] < t2[1] + D:
            out.append(own1[i])
            i += 1
        out.append(t2)
    return out + own1[i:]


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

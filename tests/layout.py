"""Byte layout of the library's workspace (the sections documented beside
cgtp_workspace_size), for tests that read the prepared graph view back.

Sections, each starting on a 256-byte boundary: srow[N+1], perm[E], sdst[E],
uperm[E], usdst[E] (int32); the per-node counters cnt, 32 int32 apart;
key1[N] (uint64); center, crank, ccnt, coff [N] (int32); the block schedules
rorder and sorder, 8*ceil(N/8) int32 each; the degree-bin counts and cursors
of the schedules (4 x 1024 int32) and the out-degree sums of every 1024 nodes
(ceil(N/1024) int32).
"""


def _a(v):
    return (v + 255) // 256 * 256


def ws_sections(N, E):
    n1, e1 = max(N, 1), max(E, 1)
    grid = 8 * ((N + 7) // 8)
    sizes = [("srow", 4 * (n1 + 1)), ("perm", 4 * e1), ("sdst", 4 * e1), ("uperm", 4 * e1), ("usdst", 4 * e1),
             ("cnt", 4 * 32 * n1), ("key1", 8 * n1), ("center", 4 * n1), ("crank", 4 * n1),
             ("ccnt", 4 * n1), ("coff", 4 * n1), ("rorder", 4 * max(grid, 1)), ("sorder", 4 * max(grid, 1)),
             ("bins", 4 * 4 * 1024), ("bsum", 4 * ((n1 + 1023) // 1024))]
    out, o = {}, 0
    for name, b in sizes:
        out[name] = o
        o += _a(b)
    out["total"] = o
    out["grid"] = grid
    return out

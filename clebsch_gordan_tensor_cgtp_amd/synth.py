"""Seeded synthetic workloads for the CGTP convolution.

This module only draws inputs: atom positions, the receiver-sorted neighbour
graph, edge vectors and the random tensors x, W and dL/dout.  It holds none of
the method's arithmetic (no spherical harmonics, no CG coefficients), so the
GPU path and the CPU oracle can both be fed from it.

The workloads follow the message-passing layers that the LunaTP abstract
("LunaTP: Enabling Efficient and Scalable Tensor Product for Equivariant
MLIPs") calls the cost centre of equivariant interatomic potentials: periodic
atomic systems at MACE/NequIP-like widths.  No dataset is used; these seeded
systems stand in for one layer on one structure.

Graph recipe:
  * positions uniform in a periodic cube (fp64), atom ids in generation order;
  * cutoff graphs: all ordered pairs (i, j), i != j, with minimum-image distance
    strictly below the cutoff; edges sorted by (receiver i, sender j);
  * the skewed dense graph: receiver i takes its k_i nearest atoms (minimum
    image), k_i = clip(round(LogNormal(ln 135.7 - 0.18, 0.6)), 20, 400);
  * the edge vector of edge j -> i is r = minimum_image(pos_j - pos_i).
Tensor recipe: x ~ N(0,1) [N][D_in][C], W ~ N(0,1)/sqrt(P) [E][P][C],
G = dL/dout ~ N(0,1) [N][D_out][C], all fp32.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    key: str
    name: str
    n_atoms: int
    box: float          # periodic cube edge, Angstrom
    cutoff: float       # Angstrom (nominal for the kNN graph)
    l_max: int          # degrees of features, SH and outputs
    channels: int
    knn_lognormal: bool = False

    @property
    def dim(self) -> int:
        return (self.l_max + 1) ** 2

    @property
    def num_paths(self) -> int:
        L = self.l_max
        return sum(1 for a in range(L + 1) for b in range(L + 1) for c in range(L + 1)
                   if abs(a - b) <= c <= a + b)


def _box(n, density):
    return (n / density) ** (1.0 / 3.0)


WORKLOADS = {
    "tiny": Workload("tiny", "32 atoms, 6 A cube, rc 3 A, L=1, C=8", 32, 6.0, 3.0, 1, 8),
    "layer": Workload("layer", "2000 atoms, 0.1 /A^3, rc 5 A, L=2, C=128",
                      2000, _box(2000, 0.1), 5.0, 2, 128),
    "large": Workload("large", "50000 atoms, 0.1 /A^3, rc 5 A, L=2, C=128",
                      50000, _box(50000, 0.1), 5.0, 2, 128),
    "high_l": Workload("high_l", "10000 atoms, 0.1 /A^3, rc 5 A, L=3, C=64",
                       10000, _box(10000, 0.1), 5.0, 3, 64),
    "dense": Workload("dense", "4000 atoms, 0.15 /A^3, kNN 20-400 log-normal, L=2, C=128",
                      4000, _box(4000, 0.15), 6.0, 2, 128, knn_lognormal=True),
}


@dataclasses.dataclass
class Graph:
    n_nodes: int
    row_ptr: np.ndarray   # int32 [N+1]
    src: np.ndarray       # int32 [E]
    r: np.ndarray         # float32 [E][3], minimum_image(pos_src - pos_dst)
    pos: np.ndarray       # float64 [N][3]

    @property
    def n_edges(self) -> int:
        return int(self.src.shape[0])


def _rng(seed: int, *stream: int) -> np.random.Generator:
    return np.random.default_rng([seed, *stream])


def _min_image(d, box):
    return d - box * np.round(d / box)


def make_graph(w: Workload, seed: int = 0) -> Graph:
    """Receiver-sorted CSR of the workload's atomic system."""
    from scipy.spatial import cKDTree

    rng = _rng(seed, 1)
    pos = rng.uniform(0.0, w.box, size=(w.n_atoms, 3))
    tree = cKDTree(pos, boxsize=w.box)
    N = w.n_atoms
    if w.knn_lognormal:
        krng = _rng(seed, 2)
        k = np.rint(krng.lognormal(math.log(135.7) - 0.18, 0.6, size=N))
        k = np.clip(k, 20, 400).astype(np.int64)
        _, nbr = tree.query(pos, k=int(k.max()) + 1)
        recv, send = [], []
        for i in range(N):
            cand = nbr[i][nbr[i] != i][: k[i]]
            recv.append(np.full(cand.shape[0], i, dtype=np.int64))
            send.append(np.sort(cand))
        recv = np.concatenate(recv)
        send = np.concatenate(send)
    else:
        pairs = tree.query_pairs(w.cutoff, output_type="ndarray").astype(np.int64)
        a, b = pairs[:, 0], pairs[:, 1]
        d = _min_image(pos[b] - pos[a], w.box)
        keep = np.einsum("ij,ij->i", d, d) < w.cutoff * w.cutoff
        a, b = a[keep], b[keep]
        recv = np.concatenate([a, b])
        send = np.concatenate([b, a])
        order = np.lexsort((send, recv))
        recv, send = recv[order], send[order]
    counts = np.bincount(recv, minlength=N)
    row_ptr = np.zeros(N + 1, dtype=np.int64)
    np.cumsum(counts, out=row_ptr[1:])
    r = _min_image(pos[send] - pos[recv], w.box).astype(np.float32)
    return Graph(N, row_ptr.astype(np.int32), send.astype(np.int32), r, pos)


def random_graph(n_nodes: int, degrees, seed: int = 0) -> Graph:
    """Small receiver-sorted CSR with the given in-degree per receiver (senders
    distinct, never the receiver itself), random edge vectors.  For edge cases."""
    rng = _rng(seed, 7)
    degrees = np.asarray(degrees, dtype=np.int64)
    recv, send = [], []
    for i in range(n_nodes):
        d = int(degrees[i])
        cand = np.array([j for j in range(n_nodes) if j != i], dtype=np.int64)
        pick = np.sort(rng.choice(cand, size=d, replace=False)) if d else cand[:0]
        recv.append(np.full(d, i, dtype=np.int64))
        send.append(pick)
    recv = np.concatenate(recv) if recv else np.zeros(0, np.int64)
    send = np.concatenate(send) if send else np.zeros(0, np.int64)
    row_ptr = np.zeros(n_nodes + 1, dtype=np.int64)
    np.cumsum(degrees, out=row_ptr[1:])
    r = rng.normal(size=(send.shape[0], 3)).astype(np.float32)
    # keep edge vectors away from zero length
    r += np.sign(r) * 0.05
    pos = np.zeros((n_nodes, 3))
    return Graph(n_nodes, row_ptr.astype(np.int32), send.astype(np.int32), r, pos)


def make_tensors_numpy(n_nodes: int, n_edges: int, l_max: int, channels: int, seed: int = 0,
                       l_in: int | None = None, l_sh: int | None = None, l_out: int | None = None):
    """x, W, G as fp32 numpy arrays (host generation; for small problems)."""
    l_in = l_max if l_in is None else l_in
    l_sh = l_max if l_sh is None else l_sh
    l_out = l_max if l_out is None else l_out
    P = sum(1 for a in range(l_in + 1) for b in range(l_sh + 1) for c in range(l_out + 1)
            if abs(a - b) <= c <= a + b)
    x = _rng(seed, 3).standard_normal((n_nodes, (l_in + 1) ** 2, channels), dtype=np.float32)
    W = _rng(seed, 4).standard_normal((n_edges, P, channels), dtype=np.float32)
    W *= np.float32(1.0 / math.sqrt(P))
    G = _rng(seed, 5).standard_normal((n_nodes, (l_out + 1) ** 2, channels), dtype=np.float32)
    return x, W, G


def make_tensors_torch(n_nodes: int, n_edges: int, l_max: int, channels: int, device,
                       seed: int = 0):
    """x, W, G as fp32 torch tensors drawn directly on ``device`` by a seeded
    torch generator (used for the large workloads, whose W is tens of GB)."""
    import torch

    P = sum(1 for a in range(l_max + 1) for b in range(l_max + 1) for c in range(l_max + 1)
            if abs(a - b) <= c <= a + b)
    D = (l_max + 1) ** 2
    g = torch.Generator(device=device)
    g.manual_seed(1000 + seed)
    x = torch.randn((n_nodes, D, channels), generator=g, device=device, dtype=torch.float32)
    W = torch.randn((n_edges, P, channels), generator=g, device=device, dtype=torch.float32)
    W.mul_(1.0 / math.sqrt(P))
    G = torch.randn((n_nodes, D, channels), generator=g, device=device, dtype=torch.float32)
    return x, W, G


def random_rotation(seed: int) -> np.ndarray:
    """Haar-random 3x3 rotation matrix (QR of a Gaussian matrix, det +1)."""
    rng = _rng(seed, 11)
    q, r = np.linalg.qr(rng.normal(size=(3, 3)))
    q = q * np.sign(np.diag(r))
    if np.linalg.det(q) < 0:
        q[:, 0] = -q[:, 0]
    return q

"""Seeded synthetic inputs for the edge tensor-product convolution.

This module is shared by the oracle side (tests) and the GPU side (tests,
bench, smoke). It holds only input generation -- graphs, bond vectors and
random feature / weight / cotangent arrays -- and none of the convolution's
arithmetic.

Workloads (the shapes the pages measure, with synthetic data standing in for
their datasets):
  tiny      32 nodes x 8 distinct random neighbours, C=8, l_max=1, |r| in [0.8, 5.0]
  micro     1024 nodes x 128 distinct random neighbours, C=128, l_max=2, |r| in
            [0.8, 6.0] -- the edge-convolution microbenchmark shape of "How does
            FlashCart make equivariant interatomic potentials faster and more
            accurate?" (section "Generated kernels beat SH baselines at high order")
  micro3 / micro4   the same graph and vectors at l_max=3 / 4
  water     1728 rigid H2O at 1.0 g/cm^3 in a periodic box, 6.0 A cutoff, C=64,
            l_max=2 (the ~5k-atom water boxes per GPU of "High-performance
            training and inference for deep equivariant interatomic
            potentials", section "Main results")
  diamond   16^3 conventional diamond cells (32768 atoms), 6.0 A cutoff
            (158 neighbours on the perfect lattice, the diamond benchmark of the
            FlashCart page), C=128, l_max=3, x stored bf16

Random streams: numpy PCG64. Each named array has its own child stream of
SeedSequence(seed), so arrays can be drawn lazily and independently:
graph, dirs, lens, x, w, G, ggx, ggw, ggvec (and pos / jitter / orient for
the lattice systems).
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np

STREAMS = ("graph", "dirs", "lens", "x", "w", "G", "ggx", "ggw", "ggvec",
           "pos", "orient", "h", "wr")


def _n_paths(L: int) -> int:
    # number of (l1, l2, l3) triples with l1, l2, l3 <= L and |l1-l2| <= l3 <= l1+l2;
    # a count of index triples, used only to set the weight variance 1/P
    return sum(1 for a in range(L + 1) for b in range(L + 1)
               for c in range(abs(a - b), min(a + b, L) + 1))


def _dout(L: int) -> int:
    return sum(2 * c + 1 for a in range(L + 1) for b in range(L + 1)
               for c in range(abs(a - b), min(a + b, L) + 1))


def rng(seed: int, name: str) -> np.random.Generator:
    child = np.random.SeedSequence(seed).spawn(len(STREAMS))[STREAMS.index(name)]
    return np.random.Generator(np.random.PCG64(child))


def random_csr(n: int, k: int, g: np.random.Generator):
    """n destinations, each with k distinct random sources != itself, rows sorted by src."""
    src = np.empty((n, k), np.int32)
    for i in range(n):
        cand = g.choice(n - 1, size=k, replace=False)
        cand = cand + (cand >= i)        # skip self
        src[i] = np.sort(cand)
    row_ptr = (np.arange(n + 1, dtype=np.int64) * k).astype(np.int32)
    return row_ptr, src.reshape(-1)


def cutoff_csr(pos: np.ndarray, box: float, rc: float):
    """Periodic neighbour list with strict |d| < rc under the minimum image,
    both directions, sorted by (dst, src); returns row_ptr, src, vec (src - dst)."""
    from scipy.spatial import cKDTree
    n = pos.shape[0]
    p = np.mod(pos, box)
    tree = cKDTree(p, boxsize=box)
    pairs = tree.query_pairs(r=rc, output_type="ndarray")
    a = np.concatenate([pairs[:, 0], pairs[:, 1]])
    b = np.concatenate([pairs[:, 1], pairs[:, 0]])
    d = p[b] - p[a]
    d -= box * np.round(d / box)
    keep = np.einsum("ij,ij->i", d, d) < rc * rc
    a, b, d = a[keep], b[keep], d[keep]
    order = np.lexsort((b, a))            # by dst = a, then src = b
    a, b, d = a[order], b[order], d[order]
    counts = np.bincount(a, minlength=n)
    row_ptr = np.zeros(n + 1, np.int64)
    row_ptr[1:] = np.cumsum(counts)
    return row_ptr.astype(np.int32), b.astype(np.int32), d.astype(np.float32)


def water_positions(seed: int, n_side: int = 12):
    """1728 rigid waters (O-H 0.96 A, HOH 104.5 deg), Haar-random orientation,
    O jittered N(0, 0.10 A) around a cubic lattice site; box from 1.0 g/cm^3."""
    from scipy.spatial.transform import Rotation
    n_mol = n_side ** 3
    avogadro = 6.02214076e23
    vol_a3 = n_mol * 18.015 / avogadro * 1e24          # cm^3 -> A^3 at 1.0 g/cm^3
    box = vol_a3 ** (1.0 / 3.0)
    spacing = box / n_side
    idx = np.stack(np.meshgrid(np.arange(n_side), np.arange(n_side), np.arange(n_side),
                               indexing="ij"), -1).reshape(-1, 3)
    o = (idx + 0.5) * spacing + rng(seed, "pos").normal(0.0, 0.10, size=(n_mol, 3))
    half = np.deg2rad(104.5) / 2
    h_local = 0.96 * np.array([[np.sin(half), 0.0, np.cos(half)],
                               [-np.sin(half), 0.0, np.cos(half)]])
    rot = Rotation.random(n_mol, random_state=rng(seed, "orient")).as_matrix()
    h = o[:, None, :] + np.einsum("mij,kj->mki", rot, h_local)
    pos = np.concatenate([o[:, None, :], h], axis=1).reshape(-1, 3)
    return pos, box


def node_features(n: int, L: int, C: int, nu: int, seed: int = 0):
    """Inputs of the node-local product: A[n, (L+1)^2, C] ~ N(0, 0.5^2) and
    W[nu-1, P, C] ~ N(0, 1/P) (float32)."""
    A = (0.5 * rng(seed, "x").standard_normal((n, (L + 1) ** 2, C))).astype(np.float32)
    P = _n_paths(L)
    W = (rng(seed, "w").standard_normal((max(nu - 1, 0), P, C)) / np.sqrt(P)).astype(np.float32)
    return A, W


def radial_inputs(E: int, K: int, L: int, C: int, seed: int = 0):
    """Inputs of the forward with radial weights: per-edge features
    h[E, K] ~ N(0, 1) (what a radial network's hidden layers hand on) and the
    shared last-layer matrix Wr[K, P, C] ~ N(0, 1/(K P)), so that the formed
    weights have the spread of the plain forward's w (float32)."""
    P = _n_paths(L)
    h = rng(seed, "h").standard_normal((E, K), np.float32)
    Wr = (rng(seed, "wr").standard_normal((K, P, C), np.float32) * np.float32(1.0 / np.sqrt(K * P)))
    return h, Wr


def gas_positions(n: int, box, seed: int, images: int = 1):
    """n atoms uniform over [-images L, (1 + images) L) per axis (so most sit
    outside the primary box), float32; box: one side or three."""
    L = np.broadcast_to(np.asarray(box, np.float64), (3,))
    u = rng(seed, "pos").random((n, 3))
    return ((u * (2 * images + 1) - images) * L).astype(np.float32)


def lattice_positions(n: int, box_units: int, seed: int, dup: int = 0):
    """n atoms on a grid of spacing 1/8 (exact in float32) over three boxes of
    box_units / 8 per axis, the last dup of them copies of earlier atoms
    (coincident pairs)."""
    g = rng(seed, "pos")
    ip = g.integers(-box_units, 2 * box_units, size=(n, 3))
    if dup:
        ip[n - dup:] = ip[g.integers(0, n - dup, size=dup)]
    return ip.astype(np.float32) / 8.0


def diamond_positions(seed: int, n_side: int = 16, a: float = 3.567, sigma: float = 0.05):
    basis = np.array([[0, 0, 0], [0, .5, .5], [.5, 0, .5], [.5, .5, 0],
                      [.25, .25, .25], [.25, .75, .75], [.75, .25, .75], [.75, .75, .25]])
    idx = np.stack(np.meshgrid(np.arange(n_side), np.arange(n_side), np.arange(n_side),
                               indexing="ij"), -1).reshape(-1, 1, 3)
    pos = ((idx + basis[None]) * a).reshape(-1, 3)
    pos = pos + rng(seed, "pos").normal(0.0, sigma, size=pos.shape)
    return pos, n_side * a


@dataclasses.dataclass
class Workload:
    """A graph plus lazily drawn arrays. Shapes: x[n, (L+1)^2, C] (n source
    nodes), w[E, P, C], G[n_dst, Dout, C], vec[E, 3]; all float32. n_dst
    defaults to n."""
    name: str
    L: int
    C: int
    n: int
    row_ptr: np.ndarray
    src: np.ndarray
    vec: np.ndarray
    seed: int = 0
    x_bf16: bool = False
    n_dst: int = -1

    def __post_init__(self):
        if self.n_dst < 0:
            self.n_dst = self.n

    @property
    def E(self) -> int:
        return int(self.row_ptr[-1])

    @property
    def P(self) -> int:
        return _n_paths(self.L)

    @property
    def Din(self) -> int:
        return (self.L + 1) ** 2

    @property
    def Dout(self) -> int:
        return _dout(self.L)

    @functools.cached_property
    def x(self) -> np.ndarray:
        return rng(self.seed, "x").standard_normal((self.n, self.Din, self.C), np.float32)

    @functools.cached_property
    def w(self) -> np.ndarray:
        g = rng(self.seed, "w")
        return (g.standard_normal((self.E, self.P, self.C), np.float32)
                * np.float32(1.0 / np.sqrt(self.P)))

    @functools.cached_property
    def G(self) -> np.ndarray:
        return rng(self.seed, "G").standard_normal((self.n_dst, self.Dout, self.C), np.float32)

    @functools.cached_property
    def ggx(self) -> np.ndarray:
        return rng(self.seed, "ggx").standard_normal((self.n, self.Din, self.C), np.float32)

    @functools.cached_property
    def ggw(self) -> np.ndarray:
        g = rng(self.seed, "ggw")
        return g.standard_normal((self.E, self.P, self.C), np.float32)

    @functools.cached_property
    def ggvec(self) -> np.ndarray:
        return rng(self.seed, "ggvec").standard_normal((self.E, 3), np.float32)


def device_normal(shape, seed: int, name: str, chunk: int, scale: float = 1.0):
    """N(0, scale^2) float32 tensor drawn on the GPU by torch's generator,
    seeded from (seed, name, chunk): for arrays too large to draw on the
    host (the diamond workload's per-edge weights, drawn per chunk of
    destination rows). Same inputs for every caller with the same key."""
    import torch
    key = np.random.SeedSequence([seed, STREAMS.index(name), chunk]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(int(key) & ((1 << 63) - 1))
    t = torch.randn(*shape, generator=g, device="cuda", dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t


def device_normal_(t, seed: int, name: str, chunk: int, scale: float = 1.0):
    """Fill the float32 device tensor t in place with N(0, scale^2) values from
    torch's generator seeded as in device_normal (no new allocation: for
    per-chunk arrays redrawn inside a timing loop)."""
    import torch
    key = np.random.SeedSequence([seed, STREAMS.index(name), chunk]).generate_state(1, np.uint64)[0]
    g = torch.Generator(device="cuda")
    g.manual_seed(int(key) & ((1 << 63) - 1))
    t.normal_(0.0, scale, generator=g)
    return t


def random_vectors(E: int, lo: float, hi: float, seed: int) -> np.ndarray:
    d = rng(seed, "dirs").standard_normal((E, 3))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    length = rng(seed, "lens").uniform(lo, hi, size=(E, 1))
    return (d * length).astype(np.float32)


def random_graph_workload(name: str, n: int, k: int, L: int, C: int, lo: float, hi: float,
                          seed: int = 0) -> Workload:
    row_ptr, src = random_csr(n, k, rng(seed, "graph"))
    vec = random_vectors(n * k, lo, hi, seed)
    return Workload(name, L, C, n, row_ptr, src, vec, seed)


@functools.lru_cache(maxsize=None)
def _micro_graph(seed: int):
    row_ptr, src = random_csr(1024, 128, rng(seed, "graph"))
    vec = random_vectors(1024 * 128, 0.8, 6.0, seed)
    return row_ptr, src, vec


def get(name: str, seed: int = 0) -> Workload:
    """One of: tiny, micro, micro3, micro4, water, diamond."""
    if name == "tiny":
        return random_graph_workload("tiny", 32, 8, 1, 8, 0.8, 5.0, seed)
    if name in ("micro", "micro3", "micro4"):
        L = {"micro": 2, "micro3": 3, "micro4": 4}[name]
        row_ptr, src, vec = _micro_graph(seed)
        return Workload(name, L, 128, 1024, row_ptr, src, vec, seed)
    if name == "water":
        pos, box = water_positions(seed)
        row_ptr, src, vec = cutoff_csr(pos, box, 6.0)
        return Workload("water", 2, 64, pos.shape[0], row_ptr, src, vec, seed)
    if name == "diamond":
        pos, box = diamond_positions(seed)
        row_ptr, src, vec = cutoff_csr(pos, box, 6.0)
        return Workload("diamond", 3, 128, pos.shape[0], row_ptr, src, vec, seed, x_bf16=True)
    raise KeyError(name)


def bipartite(L: int, C: int, n_dst: int, n_src: int, k_min: int, k_max: int, seed: int = 0,
              lo: float = 0.8, hi: float = 5.0) -> "Workload":
    """n_dst destinations drawing k in [k_min, k_max] distinct sources each
    from n_src nodes (rows sorted by src). Few destinations with many sources
    exercise long destination segments; few sources, long source segments."""
    g = rng(seed, "graph")
    deg = g.integers(k_min, k_max + 1, size=n_dst)
    deg = np.minimum(deg, n_src)
    rows = [np.sort(g.choice(n_src, size=int(d), replace=False)) for d in deg]
    row_ptr = np.zeros(n_dst + 1, np.int64)
    row_ptr[1:] = np.cumsum(deg)
    src = np.concatenate(rows).astype(np.int32) if n_dst else np.zeros(0, np.int32)
    vec = random_vectors(int(row_ptr[-1]), lo, hi, seed)
    w = Workload(f"bip_L{L}_C{C}_{n_dst}x{n_src}", L, C, n_src, row_ptr.astype(np.int32), src, vec, seed)
    w.n_dst = n_dst
    return w


def small(L: int, C: int, n: int, k_max: int, seed: int = 0, lo: float = 0.8, hi: float = 5.0,
          empty_rows: bool = True) -> Workload:
    """A small ragged graph for parity tests: in-degrees drawn from 0..k_max
    (some rows empty if empty_rows), distinct sources (self allowed to be
    excluded), rows sorted by src."""
    g = rng(seed, "graph")
    deg = g.integers(0 if empty_rows else 1, k_max + 1, size=n)
    deg = np.minimum(deg, n - 1)
    rows = []
    for i in range(n):
        cand = g.choice(n - 1, size=int(deg[i]), replace=False)
        cand = cand + (cand >= i)
        rows.append(np.sort(cand))
    row_ptr = np.zeros(n + 1, np.int64)
    row_ptr[1:] = np.cumsum(deg)
    src = np.concatenate(rows).astype(np.int32) if n else np.zeros(0, np.int32)
    vec = random_vectors(int(row_ptr[-1]), lo, hi, seed)
    return Workload(f"small_L{L}_C{C}_n{n}", L, C, n, row_ptr.astype(np.int32), src, vec, seed)

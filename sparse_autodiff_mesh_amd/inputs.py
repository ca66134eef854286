"""Seeded synthetic inputs for the triangulated-grid workloads.

This module only *produces data*: grid topology, seeded perturbations,
per-element rest constants, Hessian-vector directions and contact pairs.  It
holds none of the differentiation or assembly arithmetic, and it is the one
module that both the CPU oracle tests and the GPU path consume.

Workloads (the mesh-energy families named on the page "Locality-Aware
Automatic Differentiation on the GPU for Mesh-Based Computations", Results
section: mass-spring cloth, per-face distortion energies, contact):

* n x n vertex grid on the unit square, z = 0, spacing h = 1/(n-1).
  Vertex v = j*n + i sits at (i*h, j*h, 0).
* every quad (i, j) with corners v00, v10 = v00+1, v01 = v00+n, v11 = v00+n+1
  is split along its +x+y diagonal into (v00, v10, v11) and (v00, v11, v01),
  both counter-clockwise in the xy plane.
* springs are the unique undirected triangle edges (min, max), sorted.
* rest lengths and per-face rest data come from the *unperturbed* grid.
* positions are x = X + a*h*u with u ~ U(-1, 1)^3, drawn vertex-major, x/y/z.

Random numbers come from SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014): state advances by the golden
gamma 0x9E3779B97F4A7C15 and each output is the published 64-bit finaliser of
the new state.  u = (r >> 11) * 2^-53 gives a uniform double in [0, 1).
Gaussians are Box-Muller pairs from the same stream.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

_GAMMA = 0x9E3779B97F4A7C15
_M1 = 0xBF58476D1CE4E5B9
_M2 = 0x94D049BB133111EB
_MASK = (1 << 64) - 1

SEED_POSITIONS = 1
SEED_HVP_DIRECTION = 2
SEED_CONTACT_BASE = 1000
SEED_VF_BASE = 2000


# ----------------------------------------------------------------------------
# SplitMix64, scalar (Python ints) and vectorised (numpy uint64)
# ----------------------------------------------------------------------------
class SplitMix64:
    """Sequential SplitMix64 stream; `next_u64` returns the next output."""

    def __init__(self, seed: int):
        self.state = seed & _MASK

    def next_u64(self) -> int:
        self.state = (self.state + _GAMMA) & _MASK
        z = self.state
        z = ((z ^ (z >> 30)) * _M1) & _MASK
        z = ((z ^ (z >> 27)) * _M2) & _MASK
        return z ^ (z >> 31)

    def uniform(self) -> float:
        return (self.next_u64() >> 11) * (1.0 / 9007199254740992.0)

    def gaussian_pair(self) -> tuple[float, float]:
        u1 = 1.0 - self.uniform()  # (0, 1]
        u2 = self.uniform()
        r = math.sqrt(-2.0 * math.log(u1))
        return r * math.cos(2.0 * math.pi * u2), r * math.sin(2.0 * math.pi * u2)


def splitmix64_block(seed: int, count: int, start: int = 0) -> np.ndarray:
    """Outputs start+1 .. start+count of the SplitMix64 stream seeded `seed`.

    The k-th output is the finaliser applied to seed + k*gamma (mod 2^64), so a
    block can be produced without stepping through the earlier outputs.
    """
    k = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed & _MASK) + k * np.uint64(_GAMMA)
        z = (z ^ (z >> np.uint64(30))) * np.uint64(_M1)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(_M2)
        z = z ^ (z >> np.uint64(31))
    return z


def uniform_block(seed: int, count: int, start: int = 0) -> np.ndarray:
    r = splitmix64_block(seed, count, start)
    return (r >> np.uint64(11)).astype(np.float64) * (1.0 / 9007199254740992.0)


def gaussian_block(seed: int, count: int) -> np.ndarray:
    """`count` standard normals: Box-Muller on consecutive uniform pairs."""
    npairs = (count + 1) // 2
    u = uniform_block(seed, 2 * npairs)
    u1 = 1.0 - u[0::2]
    u2 = u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    out = np.empty(2 * npairs)
    out[0::2] = r * np.cos(2.0 * np.pi * u2)
    out[1::2] = r * np.sin(2.0 * np.pi * u2)
    return out[:count]


# ----------------------------------------------------------------------------
# Grid topology
# ----------------------------------------------------------------------------
def grid_counts(n: int) -> dict:
    """Closed-form sizes of the n x n triangulated grid."""
    V = n * n
    F = 2 * (n - 1) ** 2
    S = (n - 1) * (3 * n - 1)
    return {"V": V, "F": F, "S": S}


def grid_rest_positions(n: int) -> np.ndarray:
    h = 1.0 / (n - 1)
    j, i = np.meshgrid(np.arange(n), np.arange(n), indexing="ij")
    X = np.zeros((n * n, 3))
    X[:, 0] = (i.reshape(-1) * h)
    X[:, 1] = (j.reshape(-1) * h)
    return X


def grid_faces(n: int) -> np.ndarray:
    j, i = np.meshgrid(np.arange(n - 1), np.arange(n - 1), indexing="ij")
    v00 = (j * n + i).reshape(-1)
    v10 = v00 + 1
    v01 = v00 + n
    v11 = v00 + n + 1
    F = np.empty((2 * v00.size, 3), dtype=np.int32)
    F[0::2] = np.stack([v00, v10, v11], axis=1)
    F[1::2] = np.stack([v00, v11, v01], axis=1)
    return F


def grid_quads(n: int) -> np.ndarray:
    """The (n-1)^2 cells of the grid as four-vertex elements (v00, v10, v11,
    v01), cells in row-major order; int32 (Q, 4)."""
    j, i = np.meshgrid(np.arange(n - 1), np.arange(n - 1), indexing="ij")
    v00 = (j * n + i).reshape(-1)
    return np.stack([v00, v00 + 1, v00 + n + 1, v00 + n], axis=1).astype(np.int32)


def unique_edges(faces: np.ndarray) -> np.ndarray:
    """Unique undirected edges (min, max) of a triangle list, sorted."""
    e = np.concatenate([faces[:, [0, 1]], faces[:, [1, 2]], faces[:, [2, 0]]])
    e = np.sort(e, axis=1).astype(np.int64)
    nv = int(faces.max()) + 1 if faces.size else 0
    key = np.unique(e[:, 0] * nv + e[:, 1])
    return np.stack([key // nv, key % nv], axis=1).astype(np.int32)


def grid_adjacent(n: int, a: int, b: int) -> bool:
    """True if grid vertices a, b share a triangle edge (grid-specific)."""
    ia, ja = a % n, a // n
    ib, jb = b % n, b // n
    di, dj = ib - ia, jb - ja
    return (di, dj) in ((1, 0), (-1, 0), (0, 1), (0, -1), (1, 1), (-1, -1))


# ----------------------------------------------------------------------------
# Workload bundles
# ----------------------------------------------------------------------------
@dataclass
class Mesh:
    n: int
    h: float
    X: np.ndarray            # (V, 3) rest positions, fp64
    faces: np.ndarray        # (F, 3) int32
    springs: np.ndarray      # (S, 2) int32, sorted unique edges
    rest_len: np.ndarray     # (S,) fp64
    dm_inv: np.ndarray       # (F, 4) fp64, row-major 2x2 inverse of rest edge matrix
    area: np.ndarray         # (F,) fp64, rest area
    x: np.ndarray            # (V, 3) perturbed positions, fp64
    params: dict = field(default_factory=dict)

    @property
    def nv(self) -> int:
        return self.X.shape[0]


def face_rest_data(X: np.ndarray, faces: np.ndarray):
    """Per-face rest data from rest positions (xy plane).

    Dm = [X1 - X0, X2 - X0] restricted to (x, y), stored as its 2x2 inverse in
    row-major order, and A = |det Dm| / 2.
    """
    X0 = X[faces[:, 0], :2]
    X1 = X[faces[:, 1], :2]
    X2 = X[faces[:, 2], :2]
    e1 = X1 - X0
    e2 = X2 - X0
    # Dm columns are e1, e2:  Dm = [[e1x, e2x], [e1y, e2y]]
    det = e1[:, 0] * e2[:, 1] - e2[:, 0] * e1[:, 1]
    inv = np.empty((faces.shape[0], 4))
    inv[:, 0] = e2[:, 1] / det
    inv[:, 1] = -e2[:, 0] / det
    inv[:, 2] = -e1[:, 1] / det
    inv[:, 3] = e1[:, 0] / det
    return inv, 0.5 * np.abs(det)


def make_grid(n: int, amp: float = 0.1, seed: int = SEED_POSITIONS) -> Mesh:
    """n x n triangulated grid with seeded uniform perturbation of +-amp*h."""
    if n < 2:
        raise ValueError("grid needs n >= 2")
    h = 1.0 / (n - 1)
    X = grid_rest_positions(n)
    faces = grid_faces(n)
    springs = unique_edges(faces)
    rest_len = np.linalg.norm(X[springs[:, 0]] - X[springs[:, 1]], axis=1)
    dm_inv, area = face_rest_data(X, faces)
    u = 2.0 * uniform_block(seed, 3 * n * n) - 1.0
    x = X + amp * h * u.reshape(-1, 3)
    return Mesh(n=n, h=h, X=X, faces=faces, springs=springs, rest_len=rest_len,
                dm_inv=dm_inv, area=area, x=x, params={"amp": amp, "seed": seed})


def hvp_direction(nv: int, seed: int = SEED_HVP_DIRECTION) -> np.ndarray:
    """Unit-norm Gaussian direction over the 3*nv DOFs (fp64)."""
    g = gaussian_block(seed, 3 * nv)
    return (g / np.linalg.norm(g)).reshape(nv, 3)


def contact_pairs(mesh: Mesh, x: np.ndarray, step: int, frac: float = 0.02,
                  dhat: float | None = None):
    """Seeded vertex-vertex contact pairs for one step on a grid mesh.

    P = round(frac * V) source vertices are drawn without replacement (partial
    Fisher-Yates).  Each source gets a partner drawn uniformly among vertices
    that are neither itself, nor grid-adjacent to it, nor already used, so all
    2P vertices are distinct.  The partner is then placed at distance
    d ~ U(0.1*dhat, dhat) from its source along a normalised Gaussian
    direction.  Returns (pairs int32 (P, 2), positions (V, 3) fp64).
    """
    n = mesh.n
    V = n * n
    if dhat is None:
        dhat = 0.5 * mesh.h
    P = int(round(frac * V))
    if 2 * P > V:
        raise ValueError("too many pairs for this grid")
    rng = SplitMix64(SEED_CONTACT_BASE + step)
    perm = list(range(V))
    used = bytearray(V)
    src = []
    for k in range(P):
        r = k + int(rng.uniform() * (V - k))
        perm[k], perm[r] = perm[r], perm[k]
        src.append(perm[k])
        used[perm[k]] = 1
    pairs = np.empty((P, 2), dtype=np.int32)
    for k, a in enumerate(src):
        while True:
            b = int(rng.uniform() * V)
            if b != a and not used[b] and not grid_adjacent(n, a, b):
                break
        used[b] = 1
        pairs[k] = (a, b)
    xn = x.copy()
    for k in range(P):
        a, b = int(pairs[k, 0]), int(pairs[k, 1])
        d = dhat * (0.1 + 0.9 * rng.uniform())
        g0, g1 = rng.gaussian_pair()
        g2, _ = rng.gaussian_pair()
        nrm = math.sqrt(g0 * g0 + g1 * g1 + g2 * g2)
        xn[b] = x[a] + (d / nrm) * np.array([g0, g1, g2])
    return pairs, xn


def vf_contacts(mesh: Mesh, x: np.ndarray, step: int, frac: float = 0.02,
                dhat: float | None = None):
    """Seeded vertex-face contacts for one step on a grid mesh.

    Q = round(frac * V) faces are drawn without replacement; each gets a
    contact vertex drawn uniformly among the vertices that belong to no
    drawn face and are not already used.  The vertex is then moved to
    distance d ~ U(0.2*dhat, 0.9*dhat) from its face, cycling through three
    placements so that every closest-point region occurs, each well inside
    its region:
      k % 3 == 0  above the face interior (barycentric weights >= 0.2),
      k % 3 == 1  beside an edge (edge parameter in [0.3, 0.7], elevation
                  20..70 degrees out of the face plane),
      k % 3 == 2  beyond a vertex (along the outward bisector of its two
                  edges, same elevation range).
    The side of the face plane is random.  Returns (vf int32 (Q, 2) of
    (vertex, face id), positions (V, 3) fp64).
    """
    V = mesh.nv
    F = mesh.faces.shape[0]
    if dhat is None:
        dhat = 0.5 * mesh.h
    Q = int(round(frac * V))
    if 4 * Q > V or Q > F:
        raise ValueError("too many vertex-face contacts for this grid")
    rng = SplitMix64(SEED_VF_BASE + step)
    fperm = list(range(F))
    in_face = bytearray(V)
    faces = []
    for k in range(Q):
        r = k + int(rng.uniform() * (F - k))
        fperm[k], fperm[r] = fperm[r], fperm[k]
        faces.append(fperm[k])
        for t in mesh.faces[fperm[k]]:
            in_face[int(t)] = 1
    used = bytearray(V)
    vf = np.empty((Q, 2), dtype=np.int32)
    for k, f in enumerate(faces):
        while True:
            v = int(rng.uniform() * V)
            if not in_face[v] and not used[v]:
                break
        used[v] = 1
        vf[k] = (v, f)
    xn = x.copy()
    for k in range(Q):
        v, f = int(vf[k, 0]), int(vf[k, 1])
        t = [x[int(i)] for i in mesh.faces[f]]
        nrm = np.cross(t[1] - t[0], t[2] - t[0])
        nrm /= np.linalg.norm(nrm)
        d = dhat * (0.2 + 0.7 * rng.uniform())
        side = 1.0 if rng.uniform() < 0.5 else -1.0
        theta = math.radians(20.0 + 50.0 * rng.uniform())
        kind = k % 3
        if kind == 0:
            w = np.array([1.0 + rng.uniform(), 1.0 + rng.uniform(), 1.0 + rng.uniform()])
            w /= w.sum()
            xn[v] = w[0] * t[0] + w[1] * t[1] + w[2] * t[2] + side * d * nrm
        elif kind == 1:
            i = min(int(3 * rng.uniform()), 2)
            j, o = (i + 1) % 3, (i + 2) % 3
            lam = 0.3 + 0.4 * rng.uniform()
            m = t[i] + lam * (t[j] - t[i])
            a = (t[j] - t[i]) / np.linalg.norm(t[j] - t[i])
            out = np.cross(a, nrm)
            if np.dot(t[o] - m, out) > 0.0:
                out = -out
            xn[v] = m + d * (math.cos(theta) * out + side * math.sin(theta) * nrm)
        else:
            i = min(int(3 * rng.uniform()), 2)
            a1 = (t[(i + 1) % 3] - t[i]) / np.linalg.norm(t[(i + 1) % 3] - t[i])
            a2 = (t[(i + 2) % 3] - t[i]) / np.linalg.norm(t[(i + 2) % 3] - t[i])
            w = -(a1 + a2)
            w /= np.linalg.norm(w)
            xn[v] = t[i] + d * (math.cos(theta) * w + side * math.sin(theta) * nrm)
    return vf, xn


# ----------------------------------------------------------------------------
# Named workloads (sizes and constants of the synthetic benchmark families)
# ----------------------------------------------------------------------------
CLOTH_K = 1.0e3          # spring stiffness
CLOTH_MASS = 1.0 / 100   # per-vertex mass
CLOTH_DT = 1.0e-2        # time step; inertia weight c = m / dt^2
FACE_AMP = 0.2           # face-energy grid perturbation, in units of h
CLOTH_AMP = 0.1
BARRIER_KAPPA = 1.0e2


def cloth(n: int) -> Mesh:
    """Mass-spring cloth: springs with k = 1e3 plus inertia m/dt^2 = 100."""
    m = make_grid(n, amp=CLOTH_AMP)
    m.params.update(k=CLOTH_K, c=CLOTH_MASS / CLOTH_DT ** 2, x_tilde=m.X)
    return m


def face_grid(n: int) -> Mesh:
    """Per-face symmetric-Dirichlet grid (no springs, no inertia)."""
    m = make_grid(n, amp=FACE_AMP)
    return m


def round_f32(a):
    """Round an fp64 array or scalar to fp32 and widen back to fp64."""
    return np.asarray(a, dtype=np.float32).astype(np.float64)

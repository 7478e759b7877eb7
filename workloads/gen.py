"""Seeded synthetic inputs shaped like the pages' verify workloads.

The pages describe the method (a drafter proposes a block or tree of tokens; the target
scores every node in one pass and keeps the matching ones) but ship no data, so every
input here is synthetic:

* values: N(0, 1) float32 drawn from PCG64, rounded once to bfloat16 (round to nearest
  even) on the CPU;
* trees: ``parent[]`` arrays in breadth-first order (``parent[i] < i``; ``-1`` marks a
  child of the committed prefix);
* logits and draft tokens: N(0, 1) rows with a planted accepted path. A node that should
  match gets ``+16`` at its draft token (so that token is the row's unique maximum); a
  node that should not match gets ``-16`` at its draft token (so the draft can never be
  the row's maximum). The accepted length is therefore known by construction.

Seeds follow ``SeedSequence([42, config_id, trial])`` (42 is the seed the DFlash
contributor guide fixes for its benchmark, "coding conventions" section), spawned into
independent streams per part so that a test can ask for the tree without the KV cache.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

SEED_ROOT = 42
HEAD_DIM = 128
VOCAB = 152064
PLANT_HIGH = 16.0  # exact in bf16 and fp32; far above any N(0,1) draw
PLANT_LOW = -16.0

# Five workloads plus the two extra trees the tests use. ``tree`` names the generator,
# ``plant`` the default draft construction.
CONFIGS: dict[str, dict] = {
    # 16-node chain over a 512-token context, 8 q heads / 2 KV heads, fp32 logits [16, 4096]
    "tiny_chain": dict(cid=0, L=512, N=16, Hq=8, Hkv=2, V=4096, logits="f32",
                       tree="chain", plant="prefix", peaky=False),
    # 64-node random tree (depth <= 16, branching <= 4) over an 8K context, 32/8 heads
    "branch_8k": dict(cid=1, L=8192, N=64, Hq=32, Hkv=8, V=VOCAB, logits="bf16",
                      tree="random16", plant="path", peaky=False),
    # same tree shape over a 128K context
    "long_128k": dict(cid=2, L=131072, N=64, Hq=32, Hkv=8, V=VOCAB, logits="bf16",
                      tree="random16", plant="path", peaky=False),
    # one drafted block of 16 as a chain over a 256K context, 24/4 heads, 1% of keys x8
    "max_256k": dict(cid=3, L=262144, N=16, Hq=24, Hkv=4, V=VOCAB, logits="bf16",
                     tree="chain", plant="prefix", peaky=True),
    # 256-node breadth-first 4-ary tree (depth 4) over a 32K context, 64/8 heads
    "wide_tree": dict(cid=4, L=32768, N=256, Hq=64, Hkv=8, V=VOCAB, logits="bf16",
                      tree="kary4", plant="path", peaky=False),
    # single-token decode on the wide tree's KV cache (its first L+1 rows)
    "decode_1node": dict(cid=5, L=32768, N=1, Hq=64, Hkv=8, V=VOCAB, logits="bf16",
                         tree="chain", plant="path", peaky=False, qkv_from="wide_tree"),
    # a 22-node random tree (the DDTree node budget) over a ragged context
    "budget22": dict(cid=6, L=1000, N=22, Hq=32, Hkv=8, V=VOCAB, logits="bf16",
                     tree="random16", plant="path", peaky=False),
}


def rng_for(config_id: int, trial: int, stream: int = 0) -> np.random.Generator:
    """PCG64 generator for ``(config_id, trial)``; ``stream`` picks an independent child."""
    ss = np.random.SeedSequence([SEED_ROOT, int(config_id), int(trial)])
    child = ss.spawn(4)[stream]
    return np.random.Generator(np.random.PCG64(child))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Inputs here are finite; NaN and overflow handling is not needed by the generators.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def _normal_bf16(rng: np.random.Generator, shape, chunk: int = 1 << 24) -> np.ndarray:
    """N(0, 1) float32 draws rounded to bf16 bits, generated in chunks to bound memory."""
    total = int(np.prod(shape))
    out = np.empty(total, dtype=np.uint16)
    for lo in range(0, total, chunk):
        hi = min(total, lo + chunk)
        out[lo:hi] = bf16_bits_from_f32(rng.standard_normal(hi - lo, dtype=np.float32))
    return out.reshape(shape)


# --------------------------------------------------------------------------- trees


def chain_parent(n: int) -> np.ndarray:
    """A chain: node i hangs under node i-1; node 0 under the committed prefix."""
    return np.arange(-1, n - 1, dtype=np.int32)


def kary_bfs_parent(n: int, branch: int = 4) -> np.ndarray:
    """First ``n`` nodes of a complete ``branch``-ary tree numbered breadth first.

    For n=256, branch=4 the level sizes are 4, 16, 64 and 172.
    """
    i = np.arange(n, dtype=np.int64)
    p = np.where(i < branch, -1, (i - branch) // branch)
    return p.astype(np.int32)


def random_tree_parent(rng: np.random.Generator, n: int, max_depth: int = 16,
                       max_branch: int = 4) -> np.ndarray:
    """Random tree of exactly ``n`` nodes, depth <= max_depth, <= max_branch children each.

    Built level by level. The level size at depth d is uniform on [lo, hi] with
    ``hi = min(max_branch * previous_level_size, remaining)`` and
    ``lo = min(ceil(remaining / (max_depth - d + 1)), hi)`` (so the remaining nodes still
    fit in the levels left; the clamp only binds for trees too wide for the first levels).
    Each new node picks its parent uniformly among the previous level's nodes that still
    have fewer than ``max_branch`` children. Nodes are then renumbered breadth first,
    siblings grouped under ascending parent index.
    """
    if n < 1:
        raise ValueError("n must be >= 1")
    creation_parent: list[int] = []
    levels: list[list[int]] = []
    prev = [-1]
    children = {-1: 0}
    remaining = n
    depth = 1
    while remaining > 0:
        if depth > max_depth:
            raise AssertionError("level sizing failed to place all nodes")
        hi = min(max_branch * len(prev), remaining)
        lo = min(-(-remaining // (max_depth - depth + 1)), hi)
        size = int(rng.integers(lo, hi + 1))
        cur = []
        for _ in range(size):
            open_parents = [p for p in prev if children[p] < max_branch]
            p = open_parents[int(rng.integers(len(open_parents)))]
            children[p] += 1
            c = len(creation_parent)
            creation_parent.append(p)
            children[c] = 0
            cur.append(c)
        levels.append(cur)
        remaining -= size
        prev = cur
        depth += 1
    new_id = {-1: -1}
    order: list[int] = []
    for level in levels:
        for c in sorted(level, key=lambda c: (new_id[creation_parent[c]], c)):
            new_id[c] = len(order)
            order.append(c)
    return np.array([new_id[creation_parent[c]] for c in order], dtype=np.int32)


def _root_to_node(parent: np.ndarray, node: int) -> list[int]:
    path = []
    while node >= 0:
        path.append(int(node))
        node = int(parent[node])
    return path[::-1]


def _leaves(parent: np.ndarray) -> np.ndarray:
    has_child = np.zeros(len(parent), dtype=bool)
    has_child[parent[parent >= 0]] = True
    return np.nonzero(~has_child)[0]


# ----------------------------------------------------------------------- workloads


@dataclass
class Workload:
    name: str
    config_id: int
    trial: int
    L: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    scale: float
    parent: np.ndarray                    # int32 [N]
    draft: np.ndarray                     # int32 [N]
    matched: np.ndarray                   # bool [N]: nodes planted to match
    planted_len: int                      # accepted length implied by the planting
    planted_end: int                      # last node of the planted path, -1 if none
    logits_dtype: str = "bf16"
    q: np.ndarray | None = None           # uint16 bf16 bits [N, Hq, D]
    k: np.ndarray | None = None           # uint16 bf16 bits [L+N, Hkv, D]
    v: np.ndarray | None = None           # uint16 bf16 bits [L+N, Hkv, D]
    logits: np.ndarray | None = None      # uint16 bf16 bits or float32 [N, V]
    meta: dict = field(default_factory=dict)


def _plant(rng: np.random.Generator, parent: np.ndarray, mode: str):
    """Choose which nodes match. Returns (matched mask, planted length, end node)."""
    n = len(parent)
    matched = np.zeros(n, dtype=bool)
    if mode == "prefix":           # chain: the first k nodes match, k ~ U{0..n}
        k = int(rng.integers(0, n + 1))
        matched[:k] = True
        return matched, k, k - 1
    if mode == "path":             # a random leaf's path, first m nodes, m ~ U{0..depth}
        leaves = _leaves(parent)
        leaf = int(leaves[int(rng.integers(len(leaves)))])
        path = _root_to_node(parent, leaf)
        m = int(rng.integers(0, len(path) + 1))
        matched[path[:m]] = True
        return matched, m, (path[m - 1] if m else -1)
    if mode == "all":              # every draft equals its row's maximum
        matched[:] = True
        depth = np.array([len(_root_to_node(parent, i)) for i in range(n)])
        end = int(np.nonzero(depth == depth.max())[0][0])
        return matched, int(depth.max()), end
    if mode == "none":             # every draft misses
        return matched, 0, -1
    raise ValueError(f"unknown plant mode {mode!r}")


def make(name: str, trial: int = 0, parts=("tree", "qkv", "logits"),
         plant: str | None = None, **override) -> Workload:
    """Build workload ``name`` for ``trial``. ``parts`` limits what is generated.

    ``override`` may replace L, N, Hq, Hkv, V, logits ("bf16"/"f32"), tree
    ("chain"/"random16"/"kary4") or peaky for edge-case tests; the seed streams stay
    tied to the named configuration.
    """
    cfg = dict(CONFIGS[name])
    cfg.update(override)
    cid, L, N, Hq, Hkv, V = cfg["cid"], cfg["L"], cfg["N"], cfg["Hq"], cfg["Hkv"], cfg["V"]
    D = HEAD_DIM
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")

    rng_tree = rng_for(cid, trial, 0)
    if cfg["tree"] == "chain":
        parent = chain_parent(N)
    elif cfg["tree"] == "kary4":
        parent = kary_bfs_parent(N, 4)
    elif cfg["tree"] == "random16":
        parent = random_tree_parent(rng_tree, N, 16, 4)
    else:
        raise ValueError(cfg["tree"])

    rng_plant = rng_for(cid, trial, 3)
    matched, plen, pend = _plant(rng_plant, parent, plant or cfg["plant"])
    draft = rng_plant.integers(0, V, size=N).astype(np.int32)

    w = Workload(name=name, config_id=cid, trial=trial, L=L, N=N, Hq=Hq, Hkv=Hkv, D=D,
                 V=V, scale=1.0 / math.sqrt(D), parent=parent, draft=draft,
                 matched=matched, planted_len=plen, planted_end=pend,
                 logits_dtype=cfg["logits"])

    if "qkv" in parts:
        src = cfg.get("qkv_from")
        if src is not None:
            base = make(src, trial, parts=("qkv",))
            w.q = np.ascontiguousarray(base.q[:N])
            w.k = np.ascontiguousarray(base.k[:L + N])
            w.v = np.ascontiguousarray(base.v[:L + N])
        else:
            rng_qkv = rng_for(cid, trial, 1)
            w.q = _normal_bf16(rng_qkv, (N, Hq, D))
            w.k = _normal_bf16(rng_qkv, (L + N, Hkv, D))
            w.v = _normal_bf16(rng_qkv, (L + N, Hkv, D))
            if cfg.get("peaky"):
                _scale_some_keys(rng_qkv, w.k, L, Hkv, 0.01, 8.0)
                w.meta["peaky_keys_per_head"] = -(-L // 100)

    if "logits" in parts:
        rng_log = rng_for(cid, trial, 2)
        raw = rng_log.standard_normal((N, V), dtype=np.float32)
        rows = np.arange(N)
        raw[rows, draft] = np.where(matched, PLANT_HIGH, PLANT_LOW).astype(np.float32)
        w.logits = raw if cfg["logits"] == "f32" else bf16_bits_from_f32(raw)
    return w


def _scale_some_keys(rng, k_bits: np.ndarray, L: int, Hkv: int, frac: float, factor: float):
    """Multiply ceil(frac * L) distinct context key rows per KV head by ``factor``.

    ``factor`` is a power of two, so the scaled bf16 values are exact.
    """
    count = -(-L // int(round(1 / frac)))
    for h in range(Hkv):
        rows = rng.choice(L, size=count, replace=False)
        vals = (k_bits[rows, h, :].astype(np.uint32) << np.uint32(16)).view(np.float32)
        k_bits[rows, h, :] = bf16_bits_from_f32(vals * np.float32(factor))


def accept_trial(name: str, trial: int):
    """Small inputs for acceptance alone: (parent, draft, tok, planted_len, planted_end).

    ``tok`` stands in for the row maxima: equal to the draft on matched nodes and a
    different token elsewhere.
    """
    w = make(name, trial, parts=("tree",))
    rng = rng_for(w.config_id, trial, 2)  # the logits stream, unused without logits
    shift = rng.integers(1, w.V, size=w.N)
    tok = np.where(w.matched, w.draft, (w.draft.astype(np.int64) + shift) % w.V).astype(np.int32)
    return w.parent, w.draft, tok, w.planted_len, w.planted_end


def tie_rows(rng: np.random.Generator, V: int, dtype: str = "bf16") -> np.ndarray:
    """Rows that stress the tie rule of an argmax (first index wins).

    Row kinds: all equal; maximum repeated at scattered positions; maximum only at the
    last index; +0.0 and -0.0 as the tied maximum; all -inf but one finite value;
    a plain N(0, 1) row; max repeated at both ends.
    """
    rows = []
    rows.append(np.full(V, 0.5, dtype=np.float32))
    r = rng.standard_normal(V, dtype=np.float32)
    pos = np.sort(rng.choice(V, size=5, replace=False))
    r[pos] = 7.0
    rows.append(r)
    r = rng.standard_normal(V, dtype=np.float32)
    r[-1] = 9.0
    rows.append(r)
    r = -np.abs(rng.standard_normal(V, dtype=np.float32)) - 1.0
    r[V // 3] = -0.0
    r[V // 2] = 0.0
    rows.append(r)
    r = np.full(V, -np.inf, dtype=np.float32)
    r[V - 2] = -3.0
    rows.append(r)
    rows.append(rng.standard_normal(V, dtype=np.float32))
    r = rng.standard_normal(V, dtype=np.float32)
    r[0] = r[-1] = 8.0
    rows.append(r)
    out = np.stack(rows)
    return out if dtype == "f32" else bf16_bits_from_f32(out)

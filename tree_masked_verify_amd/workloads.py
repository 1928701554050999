"""Seeded synthetic inputs for the tree-verify step.

This module only draws random inputs with the shapes and structure of the
workloads on the pages; it performs none of the verify step's own arithmetic
(no masks, attention, argmax search, acceptance or commit).  Both the GPU tests
and the oracle tests take their inputs from here, and so does the benchmark.

Randomness:
  * small structure (trees, prefix lengths, draft decisions, block tables) comes
    from numpy ``Generator(PCG64(seed))`` on the host, so it is identical on
    every machine;
  * bulk tensors (Q, K, V, cache pools, logits) come from a ``torch.Generator``
    seeded with the same seed on the device the tensors are made on.

Logits are drawn so that each row's maximum position is known without
searching for it: the maximum of V i.i.d. N(0, s^2) values is sampled from its
own law (CDF Phi(x/s)^V), its position uniformly, and the other V-1 entries from
N(0, s^2) truncated below it.  That is exactly the i.i.d. law, and it lets a
draft token be "set equal to its parent row's argmax" with a chosen probability.
"""
from __future__ import annotations

import heapq
import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str                 # "f32" or "bf16"
    prefix: tuple[int, int]    # inclusive range of prefix lengths (equal ends = fixed)
    T: int
    tree: str                  # "fixed", "random", "chain", "eagle2"
    V: int
    logit_std: float
    draft_p: float
    block_size: int            # 0 = contiguous cache (one block per sequence)
    shuffled: bool = False
    parents: tuple[int, ...] = ()          # for tree == "fixed"
    max_levels: int = 0                    # random / eagle2 trees (root = level 1)
    max_children: int = 0                  # random trees
    topk: int = 0                          # eagle2 trees
    capacity: int = 0                      # contiguous caches: rows per sequence
    qkv_std: float = 1.0
    temperature: float = 0.3               # sampled acceptance: target softmax temperature
    notes: str = field(default="", compare=False)


# The five workload shapes (sizes, trees, vocabularies, draft-match rates).
WORKLOADS: dict[str, Workload] = {
    "tiny": Workload(
        name="tiny", B=1, Hq=1, Hkv=1, D=256, dtype="f32", prefix=(56, 56), T=8,
        tree="fixed", parents=(-1, 0, 0, 1, 1, 2, 3, 5), V=1024, logit_std=1.0, draft_p=0.7,
        block_size=0, capacity=64,
        notes="prefix 56 + 8-node asymmetric tree (4 levels) = kv 64, fp32"),
    "parity512": Workload(
        name="parity512", B=1, Hq=16, Hkv=2, D=256, dtype="bf16", prefix=(504, 504), T=8,
        tree="random", max_levels=4, max_children=3, V=32000, logit_std=2.0, draft_p=0.7,
        block_size=0, capacity=512,
        notes="prefix 504 + 8-node random asymmetric tree (4 levels, 1-3 children) = kv 512"),
    "chain2k": Workload(
        name="chain2k", B=1, Hq=8, Hkv=1, D=512, dtype="bf16", prefix=(2040, 2040), T=8,
        tree="chain", V=262144, logit_std=2.0, draft_p=0.5, block_size=0, capacity=2048,
        notes="prefix 2040 + 8-node chain = kv 2048, head_dim 512"),
    "batched8k": Workload(
        name="batched8k", B=32, Hq=32, Hkv=4, D=256, dtype="bf16", prefix=(4096, 8192), T=64,
        tree="eagle2", max_levels=6, topk=8, V=151936, logit_std=2.0, draft_p=0.75,
        block_size=16, shuffled=True,
        notes="32 sequences, prefix U[4096,8192], 64-node best-first tree, paged cache"),
    "long32k": Workload(
        name="long32k", B=16, Hq=32, Hkv=8, D=256, dtype="bf16", prefix=(32768, 32768), T=60,
        tree="random", max_levels=8, max_children=4, V=151936, logit_std=2.0, draft_p=0.6,
        block_size=16, shuffled=True,
        notes="16 sequences, prefix 32768, 60-node random tree (8 levels, 1-4 children), "
              "paged cache with shuffled block table"),
    # head_dim 128 (the head size of the Qwen target the pages retrofit the tree attention
    # for), otherwise the 32K shape
    "long32k_d128": Workload(
        name="long32k_d128", B=16, Hq=32, Hkv=8, D=128, dtype="bf16", prefix=(32768, 32768),
        T=60, tree="random", max_levels=8, max_children=4, V=151936, logit_std=2.0,
        draft_p=0.6, block_size=16, shuffled=True,
        notes="long32k with head_dim 128"),
}


# --------------------------------------------------------------------------- trees
def chain_tree(T: int) -> list[int]:
    return [-1] + list(range(T - 1))


def random_tree(rng: np.random.Generator, T: int, max_levels: int, max_children: int,
                max_tries: int = 10000) -> list[int]:
    """Each new node picks its parent uniformly among earlier nodes that are above
    the last level and have fewer than max_children children; draws are repeated
    until the tree reaches exactly max_levels levels."""
    for _ in range(max_tries):
        parents, level, nchild = [-1], [1], [0]
        ok = True
        for _i in range(1, T):
            cands = [j for j in range(len(parents))
                     if level[j] < max_levels and nchild[j] < max_children]
            if not cands:
                ok = False
                break
            p = cands[int(rng.integers(len(cands)))]
            parents.append(p)
            level.append(level[p] + 1)
            nchild.append(0)
            nchild[p] += 1
        if ok and max(level) == max_levels:
            return parents
    raise RuntimeError("random_tree: no tree with the requested number of levels")


def eagle2_tree(rng: np.random.Generator, T: int, max_levels: int, topk: int) -> list[int]:
    """Global best-first expansion: every admitted node above the last level offers
    topk children whose confidence c ~ U(0, 1]; the pending candidate with the
    highest cumulative log-confidence is admitted next, until T nodes."""
    parents, level, cum = [-1], [1], [0.0]
    heap: list[tuple[float, int, int]] = []
    order = 0

    def offer(n: int) -> None:
        nonlocal order
        if level[n] >= max_levels:
            return
        for _ in range(topk):
            c = 1.0 - float(rng.random())          # (0, 1]
            heapq.heappush(heap, (-(cum[n] + math.log(c)), order, n))
            order += 1

    offer(0)
    while len(parents) < T:
        negc, _, p = heapq.heappop(heap)
        parents.append(p)
        level.append(level[p] + 1)
        cum.append(-negc)
        offer(len(parents) - 1)
    return parents


def make_trees(w: Workload, rng: np.random.Generator) -> np.ndarray:
    out = []
    for _ in range(w.B):
        if w.tree == "fixed":
            out.append(list(w.parents))
        elif w.tree == "chain":
            out.append(chain_tree(w.T))
        elif w.tree == "random":
            out.append(random_tree(rng, w.T, w.max_levels, w.max_children))
        elif w.tree == "eagle2":
            out.append(eagle2_tree(rng, w.T, w.max_levels, w.topk))
        else:
            raise ValueError(w.tree)
    return np.asarray(out, dtype=np.int32)


# --------------------------------------------------------------------------- logits
def planted_max_logits(R: int, V: int, std: float, gen: torch.Generator,
                       device: torch.device) -> tuple[torch.Tensor, torch.Tensor]:
    """[R, V] float32 rows with the law of i.i.d. N(0, std^2), plus each row's
    maximum position (drawn first, uniformly)."""
    pos = torch.randint(0, V, (R,), generator=gen, device=device)
    u = torch.rand(R, generator=gen, device=device, dtype=torch.float64)
    u = u.clamp_min(1e-300)
    # max of V standard normals: Phi(m)^V = u  ->  m = -Phi^-1(1 - u^(1/V))
    tail = -torch.expm1(torch.log(u) / V)
    m = -torch.special.ndtri(tail)
    x = torch.empty((R, V), dtype=torch.float32, device=device)
    x.normal_(generator=gen)
    over = x.to(torch.float64) >= m[:, None]
    idx = over.nonzero(as_tuple=False)
    if idx.numel():
        # redraw from N(0,1) truncated to (-inf, m):  Phi^-1(u' * Phi(m))
        u2 = torch.rand(idx.shape[0], generator=gen, device=device, dtype=torch.float64)
        lim = torch.special.ndtr(m[idx[:, 0]])
        x[idx[:, 0], idx[:, 1]] = torch.special.ndtri(u2 * lim).to(torch.float32)
    x.mul_(std)
    top = (m * std).to(torch.float32)
    below = torch.nextafter(top, torch.full_like(top, -math.inf))
    x = torch.minimum(x, below[:, None])
    x[torch.arange(R, device=device), pos] = top
    return x, pos.to(torch.int32)


# --------------------------------------------------------------------------- inputs
def _randn(shape, dtype: str, std: float, gen, device) -> torch.Tensor:
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(generator=gen)
    if std != 1.0:
        x.mul_(std)
    return x.to(torch.bfloat16) if dtype == "bf16" else x


def _randn_chunked(shape, dtype: str, std: float, gen, device, chunk_rows: int = 1 << 12):
    """Like _randn but fills the leading dimension chunk by chunk (bounded temp)."""
    out = torch.empty(shape, dtype=torch.bfloat16 if dtype == "bf16" else torch.float32,
                      device=device)
    for s in range(0, shape[0], chunk_rows):
        e = min(shape[0], s + chunk_rows)
        out[s:e] = _randn((e - s, *shape[1:]), dtype, std, gen, device)
    return out


@dataclass
class Inputs:
    w: Workload
    seed: int
    parents: torch.Tensor        # int32 [B, T]
    q: torch.Tensor              # [B, Hq, T, D]
    k_tree: torch.Tensor         # [B, Hkv, T, D]
    v_tree: torch.Tensor
    k_pool: torch.Tensor         # [num_blocks, Hkv, block_size, D]
    v_pool: torch.Tensor
    block_table: torch.Tensor    # int32 [B, max_blocks]
    block_size: int
    prefix_len: torch.Tensor     # int32 [B]
    max_prefix_len: int
    logits: torch.Tensor         # float32 [B, T, V]
    planted_argmax: torch.Tensor  # int32 [B, T]
    draft: torch.Tensor          # int32 [B, T]
    scale: float

    @property
    def num_blocks(self) -> int:
        return int(self.k_pool.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def strides(self) -> tuple[int, int, int]:
        """(block_stride, head_stride, row_stride) in elements."""
        _, Hkv, bs, D = self.k_pool.shape
        return Hkv * bs * D, bs * D, D


def make_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu",
                prefix_override: list[int] | None = None, with_logits: bool = True,
                capacity_override: int | None = None) -> Inputs:
    device = torch.device(device)
    rng = np.random.Generator(np.random.PCG64(seed))
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)

    parents = make_trees(w, rng)
    if prefix_override is not None:
        prefix = np.asarray(prefix_override, dtype=np.int32)
        assert prefix.shape == (w.B,)
    else:
        lo, hi = w.prefix
        prefix = rng.integers(lo, hi + 1, size=w.B).astype(np.int32)
    max_p = int(prefix.max()) if w.B else 0

    # cache geometry: every sequence owns ceil((P_b + T) / block_size) blocks
    if w.block_size == 0:
        # one block per sequence; block sizes are multiples of 16 rows
        cap = capacity_override or -(-max(w.capacity, max_p + w.T) // 16) * 16
        bs = cap
        nblk = np.ones(w.B, dtype=np.int64)
    else:
        bs = w.block_size
        nblk = (prefix.astype(np.int64) + w.T + bs - 1) // bs
    max_blocks = int(nblk.max()) if w.B else 1
    num_blocks = int(nblk.sum())
    ids = rng.permutation(num_blocks) if w.shuffled else np.arange(num_blocks)
    table = np.full((w.B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(w.B):
        table[b, : nblk[b]] = ids[off: off + nblk[b]]
        off += int(nblk[b])

    q = _randn((w.B, w.Hq, w.T, w.D), w.dtype, w.qkv_std, gen, device)
    k_tree = _randn((w.B, w.Hkv, w.T, w.D), w.dtype, w.qkv_std, gen, device)
    v_tree = _randn((w.B, w.Hkv, w.T, w.D), w.dtype, 1.0, gen, device)
    k_pool = _randn_chunked((num_blocks, w.Hkv, bs, w.D), w.dtype, w.qkv_std, gen, device)
    v_pool = _randn_chunked((num_blocks, w.Hkv, bs, w.D), w.dtype, 1.0, gen, device)

    R = w.B * w.T
    if with_logits:
        logits, top = planted_max_logits(R, w.V, w.logit_std, gen, device)
        logits = logits.view(w.B, w.T, w.V)
        top_np = top.cpu().numpy().reshape(w.B, w.T)
    else:
        logits = torch.empty((w.B, w.T, 0), dtype=torch.float32, device=device)
        top_np = rng.integers(0, w.V, size=(w.B, w.T)).astype(np.int32)

    # draft tokens: node i >= 1 copies its parent row's maximum position with
    # probability draft_p, else a token drawn uniformly from the vocabulary
    draft = rng.integers(0, w.V, size=(w.B, w.T)).astype(np.int32)
    hit = rng.random(size=(w.B, w.T)) < w.draft_p
    for b in range(w.B):
        for i in range(1, w.T):
            if hit[b, i]:
                draft[b, i] = top_np[b, parents[b, i]]

    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return Inputs(
        w=w, seed=seed, parents=t(parents), q=q, k_tree=k_tree, v_tree=v_tree,
        k_pool=k_pool, v_pool=v_pool, block_table=t(table), block_size=bs,
        prefix_len=t(prefix), max_prefix_len=max_p, logits=logits,
        planted_argmax=t(top_np), draft=t(draft), scale=1.0 / math.sqrt(w.D))


def make_uniforms(B: int, T: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """The random numbers sampled acceptance consumes, drawn up front: float32 in
    [0, 1), u_accept[b][c] for trying node c as a proposal and u_sample[b][v] for
    drawing the emitted token at node v (numpy PCG64, its own stream per seed)."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x5A3D]))
    u = rng.random((2, B, T), dtype=np.float32)
    return np.ascontiguousarray(u[0]), np.ascontiguousarray(u[1])


def make_drafter_inputs(w: Workload, seed: int = 0, device: str | torch.device = "cpu",
                        T: int | None = None) -> tuple[torch.Tensor, torch.Tensor]:
    """Synthetic drafter output for building a tree of T (default w.T) nodes: float32
    logits [B, T, V] ~ N(0, logit_std^2), row i standing for the drafter's output at the
    node admitted i-th, and the root tokens int32 [B] uniform over the vocabulary."""
    device = torch.device(device)
    T = w.T if T is None else T
    gen = torch.Generator(device=device)
    gen.manual_seed(seed * 7919 + 0xD2A)
    logits = _randn((w.B, T, w.V), "f32", w.logit_std, gen, device)
    roots = torch.randint(0, w.V, (w.B,), generator=gen, device=device, dtype=torch.int64)
    return logits, roots.to(torch.int32)


def scaled(w: Workload, **kw) -> Workload:
    """A copy of a workload with some fields replaced (smaller parity variants)."""
    d = {f: getattr(w, f) for f in w.__dataclass_fields__}
    d.update(kw)
    return Workload(**d)

"""Seeded synthetic inputs for tree-masked verify attention.

This module only draws inputs: draft trees, visibility masks, lengths, slot
placement and bf16 values.  It holds none of the attention arithmetic, and it is
the one module that both the oracle tests and the HIP path's tests and bench
import.

What the inputs look like follows the pages:

* queries ``q[N, H, 576]`` bf16 in the absorbed MLA form (512 latent dims plus
  64 RoPE dims, page 3 "The Pivot to Live Cutover", section "Input Knowledge
  Required");
* one latent KV row of 576 bf16 per pool slot, ``kv_buf[num_slots, 576]``, with
  page size 1 (same page, sections "The Technical Investigation" and "Input
  Knowledge Required");
* ``kv_indices`` of a request = its prefix slots followed by the slots that its
  draft tokens were written to, and a per-request visibility mask with row
  stride ``prefix_len + n_draft`` (page 2 "Flipping the Switch", section "The
  Long Road to Parity", whose live shapes q=(9, 8, 576), mask=(270,) = 9 x 30
  fix that stride);
* the mask of request b is the flat block that ``mask_indptr[b]`` points at
  (page 3, section "The Technical Investigation").

Tree shape, value distributions, pool sizes and the lengths of the five
workloads are those of the benchmark configurations; where they leave a detail
open the reading is stated next to the code.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

QK_DIM = 576          # 512 latent + 64 RoPE dims per key and query row
V_DIM = 512           # V is the first 512 latent dims of the same row
SM_SCALE = np.float32(1.0 / math.sqrt(192.0))  # 1/sqrt(128 + 64), fp32
BF16_NAN = np.uint16(0x7FC0)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round-to-nearest-even.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


# --------------------------------------------------------------------------- trees

def gen_tree(rng: np.random.Generator, n: int, max_depth: Optional[int] = None,
             max_branch: Optional[int] = None) -> np.ndarray:
    """Parent array of a draft tree with ``n`` nodes; parent[0] = -1 (the root).

    Parents always precede children.  With ``max_depth`` set, nodes 0..max_depth-1
    first form a spine so the tree reaches that depth; every further node takes a
    parent uniformly among the earlier nodes whose depth is below ``max_depth``
    and whose child count is below ``max_branch``.
    """
    if n <= 0:
        return np.zeros(0, dtype=np.int32)
    parent = np.full(n, -1, dtype=np.int32)
    depth = np.zeros(n, dtype=np.int32)
    children = np.zeros(n, dtype=np.int32)
    depth[0] = 1
    start = 1
    if max_depth is not None:
        spine = min(n, max_depth)
        for i in range(1, spine):
            parent[i] = i - 1
            depth[i] = depth[i - 1] + 1
            children[i - 1] += 1
        start = spine
    for i in range(start, n):
        ok = np.ones(i, dtype=bool)
        if max_depth is not None:
            ok &= depth[:i] < max_depth
        if max_branch is not None:
            ok &= children[:i] < max_branch
        cand = np.flatnonzero(ok)
        if cand.size == 0:
            raise ValueError("tree constraints leave no parent for node %d" % i)
        p = int(cand[rng.integers(cand.size)])
        parent[i] = p
        depth[i] = depth[p] + 1
        children[p] += 1
    return parent


def ancestors_and_self(parent: np.ndarray, i: int) -> list:
    out = []
    while i >= 0:
        out.append(i)
        i = int(parent[i])
    return out[::-1]


def tree_mask(parent: np.ndarray, prefix_len: int) -> np.ndarray:
    """uint8 [n, prefix_len + n]: prefix all visible, draft k visible to row i
    iff k is an ancestor of i or i itself (a draft sees its own tree path)."""
    n = len(parent)
    m = np.zeros((n, prefix_len + n), dtype=np.uint8)
    m[:, :prefix_len] = 1
    for i in range(n):
        for k in ancestors_and_self(parent, i):
            m[i, prefix_len + k] = 1
    return m


# ----------------------------------------------------------------------- workloads

@dataclasses.dataclass
class Workload:
    q: np.ndarray            # uint16 bf16 bits [N, H, 576]
    kv: np.ndarray           # uint16 bf16 bits [num_slots, 576]
    kv_indices: np.ndarray   # int32 [kv_indptr[B]]
    kv_indptr: np.ndarray    # int32 [B+1]
    qo_indptr: np.ndarray    # int32 [B+1]
    mask: np.ndarray         # uint8 [mask_indptr[B]]
    mask_indptr: np.ndarray  # int32 [B+1]
    sm_scale: np.float32
    num_heads: int
    prefix_lens: list = dataclasses.field(default_factory=list)
    parents: list = dataclasses.field(default_factory=list)
    name: str = ""
    # mask in the prefix-visible form: n_b x n_b bytes per request (draft keys
    # only), every prefix key visible
    prefix_visible: bool = False
    # contiguous-prefix form: the P_b prefix keys of request b are the pool run
    # starting at kv_indices[kv_indptr[b]]; the other prefix entries are not
    # part of the input (filled with -1 here)
    contiguous_prefix: bool = False

    @property
    def batch(self) -> int:
        return len(self.qo_indptr) - 1

    @property
    def total_q(self) -> int:
        return int(self.q.shape[0])

    @property
    def num_slots(self) -> int:
        return int(self.kv.shape[0])

    @property
    def q_lens(self) -> np.ndarray:
        return np.diff(self.qo_indptr.astype(np.int64))

    @property
    def kv_lens(self) -> np.ndarray:
        return np.diff(self.kv_indptr.astype(np.int64))

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.batch else 0

    @property
    def max_kv_len(self) -> int:
        return int(self.kv_lens.max()) if self.batch else 0

    def gathered_kv_bytes(self) -> int:
        """Bytes of latent KV rows the call gathers: sum over requests of L_b * 1152."""
        return int(self.kv_lens.sum()) * QK_DIM * 2

    def visible_pairs(self) -> int:
        """Visible (draft row, key) pairs, summed over requests."""
        nz = int(np.count_nonzero(self.mask[self.mask_indptr[0]:self.mask_indptr[-1]]))
        if self.prefix_visible:
            nz += int((self.q_lens * (self.kv_lens - self.q_lens)).sum())
        return nz


def _spawn(seed: int):
    ss = np.random.SeedSequence(seed)
    # streams: lengths+trees, slots, q, kv, outliers, spare
    return [np.random.default_rng(s) for s in ss.spawn(6)]


def _values(rng: np.random.Generator, shape, out_rng: Optional[np.random.Generator],
            outlier_p: float) -> np.ndarray:
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_p > 0.0:
        hit = out_rng.random(shape, dtype=np.float32) < outlier_p
        x[hit] *= np.float32(30.0)
    return bf16_round(x)


def contiguous_slots(rng: np.random.Generator, pool: int, prefix_lens: Sequence[int],
                     n_drafts: Sequence[int]) -> np.ndarray:
    """Slot list of a batch whose prefixes each sit in one contiguous run of
    the pool (a defragmented cache): the runs go into the pool in a seeded
    request order, separated by seeded gaps; the draft tokens take seeded
    random slots among those left.  Returned in key order: per request its run,
    then its draft slots."""
    B = len(prefix_lens)
    P = np.array(prefix_lens, dtype=np.int64)
    n = np.array(n_drafts, dtype=np.int64)
    slack = pool - int(P.sum()) - int(n.sum())
    if slack < 0:
        raise ValueError("pool too small")
    order = rng.permutation(B)
    gap_max = max(1, slack // (2 * (B + 1)))
    start = np.zeros(B, dtype=np.int64)
    pos = int(rng.integers(0, gap_max))
    for b in order:
        start[b] = pos
        pos += int(P[b]) + int(rng.integers(0, gap_max))
    used = np.zeros(pool, dtype=bool)
    for b in range(B):
        used[start[b]:start[b] + P[b]] = True
    free = np.flatnonzero(~used)
    drafts = free[rng.permutation(free.size)[:int(n.sum())]]
    out, d = [], 0
    for b in range(B):
        out.append(np.arange(start[b], start[b] + P[b], dtype=np.int64))
        out.append(drafts[d:d + n[b]])
        d += int(n[b])
    return np.concatenate(out).astype(np.int32) if B else np.zeros(0, np.int32)


def build(seed: int, prefix_lens: Sequence[int], parents: Sequence[np.ndarray], num_heads: int,
          pool: int, outlier_p: float = 0.0, poison: bool = True, name: str = "",
          sm_scale: np.float32 = SM_SCALE, placement: str = "random") -> Workload:
    """Assemble a segmented batch from per-request prefix lengths and draft trees.

    Slots (placement="random"): one seeded permutation of the pool, consumed in
    order; each request takes its prefix slots, then one slot per draft token
    (random 1-slot placement, disjoint across requests).  placement=
    "contiguous": each prefix is one run of consecutive slots
    (contiguous_slots).  The values drawn for the keys, in key order, do not
    depend on the placement.  Only referenced rows get values; the rest are
    bf16 NaN when ``poison`` (a stray gather then shows up), else 0.
    """
    rngs = _spawn(seed)
    r_slot, r_q, r_kv, r_out = rngs[1], rngs[2], rngs[3], rngs[4]
    B = len(prefix_lens)
    n = np.array([len(p) for p in parents], dtype=np.int64)
    L = np.array(prefix_lens, dtype=np.int64) + n
    need = int(L.sum())
    while pool < need:
        pool *= 2
    if placement == "random":
        perm = r_slot.permutation(pool).astype(np.int32)
        kv_indices = perm[:need].copy()
    elif placement == "contiguous":
        kv_indices = contiguous_slots(r_slot, pool, prefix_lens, n)
    else:
        raise ValueError("placement %r" % placement)
    kv_indptr = np.zeros(B + 1, dtype=np.int64)
    kv_indptr[1:] = np.cumsum(L)
    qo_indptr = np.zeros(B + 1, dtype=np.int64)
    qo_indptr[1:] = np.cumsum(n)
    masks = [tree_mask(np.asarray(parents[b]), int(prefix_lens[b])) for b in range(B)]
    mask_indptr = np.zeros(B + 1, dtype=np.int64)
    mask_indptr[1:] = np.cumsum([m.size for m in masks])
    if mask_indptr[-1] >= 2 ** 31 or kv_indptr[-1] >= 2 ** 31:
        raise ValueError("index ranges exceed int32")
    mask = np.concatenate([m.reshape(-1) for m in masks]) if B else np.zeros(0, np.uint8)
    N = int(qo_indptr[-1])
    q = _values(r_q, (N, num_heads, QK_DIM), r_out, outlier_p)
    kv = np.full((pool, QK_DIM), BF16_NAN if poison else np.uint16(0), dtype=np.uint16)
    kv[kv_indices] = _values(r_kv, (need, QK_DIM), r_out, outlier_p)
    return Workload(q=q, kv=kv, kv_indices=kv_indices, kv_indptr=kv_indptr.astype(np.int32),
                    qo_indptr=qo_indptr.astype(np.int32), mask=mask.astype(np.uint8),
                    mask_indptr=mask_indptr.astype(np.int32), sm_scale=np.float32(sm_scale),
                    num_heads=num_heads, prefix_lens=[int(p) for p in prefix_lens],
                    parents=[np.asarray(p) for p in parents], name=name)


# The five benchmark workloads.  Open details and the readings taken:
#  C2 tree: "random tree, branching <= 4" -> max_branch=4, no depth limit.
#  C3 tree: "depth-8 tree, branching 4" with 32 nodes cannot be a full tree;
#           read as a depth-8 spine plus nodes of depth <= 8, <= 4 children each.
#  C5 trees: "mixed depths 3-10" -> per-request max_depth ~ U{3..10}, spine to it.
#  C5 prefix: log-uniform in [256, 65536], rounded to an integer.
#  C5 outliers: each q/kv element independently, p = 0.01, scaled x30 before
#           bf16 rounding.
#  Seeds: config k uses seed k; the long-prefix sweep uses 100 + k.
CONFIG_DESC = {
    1: "C1: 1 request, n_draft=9, prefix 21, H=8, pool 4096",
    2: "C2: 8 requests, n_draft=16, prefix U[512,4096], H=8, pool 65536",
    3: "C3: 1 request, n_draft=32 (depth-8, branching 4), prefix 32768, H=16, pool 200000",
    4: "C4: 1 request, n_draft=64, prefix 200000, H=8, pool 262144",
    5: "C5: 32 requests, n_draft=24 (depths 3-10), prefix log-U[256,65536], H=64, 1% x30 outliers",
}

# Split count that a configuration names for itself (C3 states split-K = 32).
CONFIG_SPLITS = {3: 32}


def config(k: int, poison: bool = True, placement: str = "random") -> Workload:
    rngs = _spawn(k)
    rt = rngs[0]
    if k == 1:
        prefix = [21]
        parents = [gen_tree(rt, 9)]
        return build(k, prefix, parents, 8, 4096, poison=poison, name="C1",
                     placement=placement)
    if k == 2:
        prefix = [int(x) for x in rt.integers(512, 4097, size=8)]
        parents = [gen_tree(rt, 16, max_branch=4) for _ in range(8)]
        return build(k, prefix, parents, 8, 65536, poison=poison, name="C2",
                     placement=placement)
    if k == 3:
        parents = [gen_tree(rt, 32, max_depth=8, max_branch=4)]
        return build(k, [32768], parents, 16, 200000, poison=poison, name="C3",
                     placement=placement)
    if k == 4:
        parents = [gen_tree(rt, 64)]
        return build(k, [200000], parents, 8, 262144, poison=poison, name="C4",
                     placement=placement)
    if k == 5:
        prefix = [int(round(math.exp(x))) for x in rt.uniform(math.log(256), math.log(65536), size=32)]
        parents = []
        for _ in range(32):
            d = int(rt.integers(3, 11))
            parents.append(gen_tree(rt, 24, max_depth=d))
        return build(k, prefix, parents, 64, 524288, outlier_p=0.01, poison=poison, name="C5",
                     placement=placement)
    raise ValueError("unknown config %r" % k)


SWEEP_PREFIX = {1: 32768, 2: 131072, 3: 200000}


def sweep(k: int, poison: bool = True, placement: str = "random") -> Workload:
    """The live shape (n_draft=9, H=8) at long prefixes: 32768 / 131072 / 200000."""
    rngs = _spawn(100 + k)
    parents = [gen_tree(rngs[0], 9)]
    return build(100 + k, [SWEEP_PREFIX[k]], parents, 8, 262144, poison=poison, name="S%d" % k,
                 placement=placement)


def small(seed: int, prefix_lens: Sequence[int], n_drafts: Sequence[int], num_heads: int,
          pool: Optional[int] = None, outlier_p: float = 0.0, poison: bool = True,
          max_branch: Optional[int] = None, placement: str = "random") -> Workload:
    """Ad-hoc seeded workload (tests): random trees with the given draft counts."""
    rngs = _spawn(seed)
    parents = [gen_tree(rngs[0], int(n), max_branch=max_branch) for n in n_drafts]
    need = int(sum(prefix_lens) + sum(n_drafts))
    pool = pool if pool is not None else max(64, 2 * need)
    return build(seed, prefix_lens, parents, num_heads, pool, outlier_p=outlier_p, poison=poison,
                 name="small%d" % seed, placement=placement)


def contiguous_prefix_form(w: Workload) -> Workload:
    """The same workload in the contiguous-prefix form: every prefix must be
    one run of consecutive slots (placement="contiguous"); kv_indices keeps its
    layout, but of each prefix only the first entry (the run's first slot)
    stays part of the input; the other prefix entries become -1, which a
    reader that used them would turn into a slot outside the pool."""
    ki = w.kv_indices.astype(np.int64).copy()
    for b in range(w.batch):
        k0 = int(w.kv_indptr[b])
        P = int(w.kv_lens[b] - w.q_lens[b])
        run = ki[k0:k0 + P]
        if P and not np.array_equal(run, run[0] + np.arange(P)):
            raise ValueError("request %d: prefix slots are not one contiguous run" % b)
        ki[k0 + 1:k0 + P] = -1
    return dataclasses.replace(w, kv_indices=ki.astype(np.int32), contiguous_prefix=True,
                               name=w.name + "/contiguous-prefix")


def prefix_visible_form(w: Workload) -> Workload:
    """The same workload with its mask in the prefix-visible form: per request
    only the draft-key columns (the last n_b of each row), n_b x n_b bytes,
    row stride n_b.  The prefix columns must all be visible (true of tree
    masks); the visible sets are unchanged."""
    blocks = []
    for b in range(w.batch):
        n, L = int(w.q_lens[b]), int(w.kv_lens[b])
        m = w.mask[w.mask_indptr[b]:w.mask_indptr[b + 1]].reshape(n, L)
        if not np.all(m[:, :L - n] != 0):
            raise ValueError("request %d: a prefix key is masked; no prefix-visible form" % b)
        blocks.append(np.ascontiguousarray(m[:, L - n:]).reshape(-1))
    mask_indptr = np.zeros(w.batch + 1, dtype=np.int64)
    mask_indptr[1:] = np.cumsum([x.size for x in blocks])
    mask = np.concatenate(blocks) if blocks else np.zeros(0, np.uint8)
    return dataclasses.replace(w, mask=mask.astype(np.uint8),
                               mask_indptr=mask_indptr.astype(np.int32), prefix_visible=True,
                               name=w.name + "/prefix-visible")


def chain(seed: int, prefix_lens: Sequence[int], n: int, num_heads: int,
          pool: Optional[int] = None, poison: bool = True, name: str = "",
          placement: str = "random") -> Workload:
    """Requests whose n draft tokens form one chain (draft i's parent is i - 1):
    a causal mask over the drafts.  n = 1 is plain decode: one query token per
    request seeing its prefix and itself."""
    parents = [np.arange(-1, n - 1, dtype=np.int32) for _ in prefix_lens]
    need = int(sum(prefix_lens)) + n * len(prefix_lens)
    pool = pool if pool is not None else max(64, 2 * need)
    return build(seed, prefix_lens, parents, num_heads, pool, poison=poison,
                 name=name or "chain%d" % seed, placement=placement)


# Workloads of the same kernels beyond tree verification (not part of the five
# configurations): plain MLA decode with all 128 heads of a model on one GPU,
# and a causal chain of drafts.
EXTRA_DESC = {
    "D": "D: plain decode, 8 requests x 1 token, prefix 32768, H=128, pool 524288",
    "K": "K: chain verify, 1 request, 16 drafts in a chain, prefix 32768, H=16, pool 200000",
}


def extra(key: str, poison: bool = True, placement: str = "random") -> Workload:
    if key == "D":
        return chain(301, [32768] * 8, 1, 128, pool=524288, poison=poison, name="D",
                     placement=placement)
    if key == "K":
        return chain(302, [32768], 16, 16, pool=200000, poison=poison, name="K",
                     placement=placement)
    raise ValueError("unknown workload %r" % key)


def marshal_inputs(w: Workload) -> dict:
    """A generated workload taken apart into the inputs of the marshaling step
    (draft rows into the pool, key lists, tree mask): the pool without the draft
    rows (bf16 NaN there), the draft rows, their slots, the prefix slot lists,
    the prefix indptr, qo_indptr and the parents.  The workload's own kv_indices,
    indptrs and mask are what the step must rebuild from them."""
    B = w.batch
    qo = w.qo_indptr.astype(np.int64)
    kvp = w.kv_indptr.astype(np.int64)
    n = np.diff(qo)
    P = np.diff(kvp) - n
    prefix_indptr = np.zeros(B + 1, dtype=np.int64)
    prefix_indptr[1:] = np.cumsum(P)
    prefix = [w.kv_indices[kvp[b]:kvp[b] + P[b]] for b in range(B)]
    draft = [w.kv_indices[kvp[b] + P[b]:kvp[b + 1]] for b in range(B)]
    prefix_indices = np.concatenate(prefix) if B else np.zeros(0, np.int32)
    out_cache_loc = np.concatenate(draft) if B else np.zeros(0, np.int32)
    draft_kv = w.kv[out_cache_loc].copy()
    pool = w.kv.copy()
    pool[out_cache_loc] = BF16_NAN
    parents = np.concatenate([np.asarray(p, dtype=np.int32) for p in w.parents]) if B else \
        np.zeros(0, np.int32)
    return dict(kv_buf=pool, draft_kv=draft_kv, out_cache_loc=out_cache_loc.astype(np.int32),
                prefix_indices=prefix_indices.astype(np.int32),
                prefix_indptr=prefix_indptr.astype(np.int32), qo_indptr=w.qo_indptr.copy(),
                parents=parents)

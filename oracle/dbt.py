"""AllReduce over two binary trees (the double binary tree), executed on N host
arrays — TEST INFRASTRUCTURE ONLY.

Sources.  The pages name the double binary tree and give its cost and use,
but no construction:

* tirogla.com "Ring all-reduce", section "How it works" (cost model): about
  2 log2 N latency terms and 2 S/B of bandwidth, bandwidth-optimal up to a
  constant; sections "Avoid when", "Efficiency" (levers) and "Variants and
  alternatives": the choice for small and medium messages at large N, in
  NCCL since 2.4;
* "2.1 Collective communication primitives in detail", section 4.4: NCCL's
  tree algorithm for large multi-node AllReduce.

The construction is the two-tree scheme of P. Sanders, J. Speck and J. L.
Träff, "Two-tree algorithms for full bandwidth broadcast, reduction and
scan", Parallel Computing 35(12), 2009: two binary trees over the same ranks,
each carrying half of the data, arranged so that no rank is an inner node of
both (a leaf sends and receives only its half once each way, so every rank
moves about 2 S in all).

Readings (where neither the pages nor that construction fix a detail):

* the halves are the ring's floor chunk plan with two chunks:
  [0, len/2) goes up and down tree 0, [len/2, len) tree 1;
* tree 0 is the in-order binary tree over positions 1..N, position p holding
  rank p - 1.  The height of position p is the number of trailing zero bits
  of p; the root is the largest power of two not above N; a node p of height
  h > 0 has the left child p - 2^(h-1) and the right child p + 2^j for the
  largest j < h with p + 2^j <= N (none when p = N);
* tree 1 has the same shape with every rank moved on by one: position p
  holds rank p mod N.  Inner positions are even, so the inner ranks of tree 0
  are odd and those of tree 1 even (rank 0 too when N is even): no rank is
  inner in both, for any N;
* an inner node combines ((left partial (op) own value) (op) right partial),
  rounded to the working type after each operation; the root finishes its
  value once (avg's division by N, bf16acc32's rounding to bf16);
* both trees run at once, in stages: before reduction stage 1 every leaf
  sends its half to its parent; in reduction stage j (j = 1..H, with
  H = floor(log2 N) the height of the root) every node of height j combines
  its children's partials and, unless it is the root, sends the result to
  its parent; in distribution stage j (j = H..1) every node of height j sends
  the finished half to its children.  2H stages in all.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .ring import _ITEMSIZE, _STORAGE, _WORK, _check_inputs, _same_bits, chunk, finish, reduce_op, to_work
from .orders import tree_order_fold

TREES = 2


@dataclass
class DbtStats:
    """What the schedule did: per-rank bytes sent and received, and its stage count."""

    sent: list = field(default_factory=list)
    received: list = field(default_factory=list)
    stages: int = 0


def height(p: int) -> int:
    """Height of position p (p >= 1) in the in-order tree: its trailing zero bits."""
    h = 0
    while p % 2 == 0:
        p //= 2
        h += 1
    return h


def root(n: int) -> int:
    """Root position of the in-order tree over positions 1..n: the largest power of two <= n."""
    r = 1
    while 2 * r <= n:
        r *= 2
    return r


def children(p: int, n: int) -> tuple:
    """(left, right) child positions of position p in the tree over 1..n (None when absent)."""
    h = height(p)
    if h == 0:
        return None, None
    left = p - 2 ** (h - 1)
    right = None
    for j in range(h - 1, -1, -1):
        if p + 2 ** j <= n:
            right = p + 2 ** j
            break
    return left, right


def parents(n: int) -> dict:
    """Parent position of every non-root position, from the children rule."""
    par = {}
    for p in range(1, n + 1):
        for c in children(p, n):
            if c is not None:
                if c in par:
                    raise AssertionError(f"position {c} has two parents")
                par[c] = p
    return par


def rank_of(p: int, tree: int, n: int) -> int:
    """Rank at position p of tree 0 (rank p - 1) or tree 1 (rank p mod n)."""
    return (p - 1 + tree) % n


def inner_ranks(tree: int, n: int) -> set:
    """Ranks that are inner nodes (have a child) of the given tree."""
    return {rank_of(p, tree, n) for p in range(1, n + 1) if children(p, n)[0] is not None}


def bracketing(tree: int, n: int):
    """The bracketing tree ``tree`` computes (nested 2-tuples of ranks)."""
    if n < 1:
        raise ValueError("need at least one rank")

    def node(p):
        left, right = children(p, n)
        if left is None:
            return rank_of(p, tree, n)
        v = (node(left), rank_of(p, tree, n))
        return (v, node(right)) if right is not None else v

    return node(root(n))


def double_binary_trees(n: int) -> tuple:
    """The bracketings of the two trees: (half 0's, half 1's)."""
    return bracketing(0, n), bracketing(1, n)


def halves(length: int) -> tuple:
    """Element bounds of the two halves (the floor chunk plan with two chunks)."""
    return chunk(0, 2, length), chunk(1, 2, length)


# --------------------------------------------------------------------------
# the schedule, executed
# --------------------------------------------------------------------------

class _Mail:
    """Per-rank mailboxes; a message is taken by naming its sender, as a rank
    that waits for a given child does."""

    def __init__(self, n, stats):
        self.box = [[] for _ in range(n)]
        self.stats = stats

    def send(self, src, dst, tag, payload, esz):
        self.box[dst].append((src, tag, payload))
        self.stats.sent[src] += payload.size * esz

    def take(self, dst, src, tag, esz):
        hits = [k for k, (s, t, _) in enumerate(self.box[dst]) if s == src and t == tag]
        if len(hits) != 1:
            raise AssertionError(f"rank {dst} expected one message {tag} from rank {src}, found {len(hits)}")
        _, _, payload = self.box[dst].pop(hits[0])
        self.stats.received[dst] += payload.size * esz
        return payload

    def empty(self):
        return not any(self.box)


def double_binary_tree_allreduce(xs, op: str = "sum", dtype: str = "f32", check: bool = True):
    """Reduce each half up its tree, then send it back down; returns (outputs, stats)."""
    n, length = _check_inputs(xs, dtype)
    wd = _WORK[dtype]
    stats = DbtStats(sent=[0] * n, received=[0] * n)
    mail = _Mail(n, stats)
    spans = halves(length)
    par = parents(n)
    top = root(n)
    levels = height(top)
    # the value each position holds of its tree's half, in working precision while reducing
    val = [{p: to_work(xs[rank_of(p, t, n)][slice(*spans[t])], dtype) for p in range(1, n + 1)}
           for t in range(TREES)]

    def up(t, p, v):
        if p in par:
            mail.send(rank_of(p, t, n), rank_of(par[p], t, n), (t, "up", p), v.copy(), _ITEMSIZE[wd])

    for t in range(TREES):                                   # leaves start the reduction
        for p in range(1, n + 1):
            if height(p) == 0:
                up(t, p, val[t][p])
    for j in range(1, levels + 1):                           # reduction stages
        for t in range(TREES):
            for p in range(1, n + 1):
                if height(p) != j:
                    continue
                me = rank_of(p, t, n)
                left, right = children(p, n)
                v = reduce_op(op, wd, mail.take(me, rank_of(left, t, n), (t, "up", left), _ITEMSIZE[wd]),
                              val[t][p])
                if right is not None:
                    v = reduce_op(op, wd, v, mail.take(me, rank_of(right, t, n), (t, "up", right),
                                                      _ITEMSIZE[wd]))
                val[t][p] = v
                up(t, p, v)
        stats.stages += 1
    final = [{} for _ in range(TREES)]
    for t in range(TREES):
        final[t][top] = finish(op, dtype, val[t][top], n)
    for j in range(levels, 0, -1):                           # distribution stages
        for t in range(TREES):
            for p in range(1, n + 1):
                if height(p) == j:
                    for c in children(p, n):
                        if c is not None:
                            mail.send(rank_of(p, t, n), rank_of(c, t, n), (t, "down", c), final[t][p].copy(),
                                      _ITEMSIZE[dtype])
            for p in range(1, n + 1):
                if p in par and height(par[p]) == j:
                    final[t][p] = mail.take(rank_of(p, t, n), rank_of(par[p], t, n), (t, "down", p),
                                            _ITEMSIZE[dtype])
        stats.stages += 1
    if not mail.empty():
        raise AssertionError("messages left undelivered")
    out = []
    for r in range(n):
        o = np.empty(length, dtype=_STORAGE[dtype])
        for t in range(TREES):
            o[slice(*spans[t])] = final[t][(r - t) % n + 1]   # rank r sits at position (r - t) mod n + 1
        out.append(o)
    if check:
        for r in range(1, n):
            if not _same_bits(out[r], out[0], dtype):
                raise AssertionError("ranks disagree at the end of the schedule")
    return out, stats


# --------------------------------------------------------------------------
# the result as a definition
# --------------------------------------------------------------------------

def double_binary_tree_fold(xs, op: str = "sum", dtype: str = "f32") -> np.ndarray:
    """Each half evaluated directly in its tree's bracketing (no schedule)."""
    n, length = _check_inputs(xs, dtype)
    out = np.empty(length, dtype=_STORAGE[dtype])
    for t, span in enumerate(halves(length)):
        out[slice(*span)] = tree_order_fold([x[slice(*span)] for x in xs], bracketing(t, n), op, dtype)
    return out

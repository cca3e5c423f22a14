"""CPU oracle for the ring AllReduce — TEST INFRASTRUCTURE ONLY.

Nothing in the product imports this package.  It is used by the tests,
by the entry point's smoke check and by the benchmark's CPU-baseline leg,
and it shares no code with the HIP library (no kernels, headers, helpers,
tables or constants).

What it holds, each piece written from the pages on ring AllReduce:

* ``ring``      the literal ring schedule executed on N host arrays with
                FIFO mailboxes and byte counters (reduce-scatter then
                all-gather, as stated on tirogla.com "Ring all-reduce",
                section "How it works"), the standalone reduce-scatter and
                all-gather, the element operators, bf16 round-to-nearest-even,
                and the closed definition of the result (the ring's
                association order), which the full-size checks compare
                every output element with;
* ``threaded``  one thread per rank, each a state machine that answers
                arrivals and forwards the chunk it just completed, with a
                receive time-out that turns a stuck ring into an error;
* ``orders``    the tree-shaped schedules (binomial tree reduce and
                distribution, recursive doubling, and Rabenseifner's recursive
                halving and doubling), executed the same way, and the
                bracketings they compute written from their definitions;
* ``dbt``       the double binary tree: each half of the buffer reduced up
                one of two in-order binary trees and sent back down it, no
                rank an inner node of both (the two-tree construction of
                Sanders, Speck and Träff, 2009), executed stage by stage,
                and each half's bracketing evaluated directly;
* ``explore``   brute force for tiny rings: every interleaving of the ranks'
                send/receive events, and every bracketing of an N-term sum;
* ``staged``    AllReduce as a reduce onto a root followed by a broadcast
                (bitfern.com "AllReduce Explained", section "Reduce Followed
                by Broadcast"), the root folding in the ring's order.

Pins (what each part is checked against) are in ``tests/test_oracle_*.py``.
Every function has a pin; none is "parity unpinned".
"""

from .ring import (  # noqa: F401
    DTYPES,
    OPS,
    RingStats,
    all_gather,
    bf16_bits_to_f32,
    chunk,
    chunk_owner,
    f16_bits_to_f32,
    f32_to_bf16_bits,
    f32_to_f16_bits,
    finish,
    reduce_op,
    reduce_scatter,
    ring_allreduce,
    ring_order_fold,
    ring_order_fold_columns,
)
from .orders import (  # noqa: F401,E402
    ORDERS,
    OrderStats,
    binomial_tree,
    halving_doubling_allreduce,
    halving_tree,
    order_allreduce,
    order_bracketing,
    recursive_doubling_allreduce,
    tree_allreduce,
    tree_order_fold,
    tree_order_fold_columns,
)
from .staged import reduce_then_broadcast, reduce_to_root  # noqa: F401,E402
from .dbt import double_binary_tree_allreduce, double_binary_tree_fold, double_binary_trees  # noqa: F401,E402

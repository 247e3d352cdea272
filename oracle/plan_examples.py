"""Host-side formulas the pages state, for checking the library's planner.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Each function is the pages' statement, written out; the worked examples the
pages print are stored under tests/golden/ and pin these functions.
"""

from __future__ import annotations

import math


def decode_task_mapping(task: int, num_kv_heads: int, group: int) -> tuple[int, int, int]:
    """One decode task = one batch row + one KV head + the group of query
    heads that share it; tasks run batch-major over KV heads, and the KV
    head's first query head is kv_head * group ("Writing Page Attention with
    PyPTO", section 1.3). Returns (batch, kv_head, first_q_head)."""
    batch = task // num_kv_heads
    kv_head = task % num_kv_heads
    return batch, kv_head, kv_head * group


def page_stack_counts(seq_len: int, page_size: int, pages_per_stack: int) -> tuple[int, int, int]:
    """Pages and stacks one request walks, and the valid tokens in its last
    stack ("Writing Page Attention with PyPTO", sections 1.4 and 5.1: page
    count is the ceiling of seq_len over the page size, stack count the
    ceiling over the stack size). Returns (pages, stacks, last_stack_tokens)."""
    pages = -(-seq_len // page_size)
    stack_tokens = page_size * pages_per_stack
    stacks = -(-seq_len // stack_tokens)
    last = seq_len - (stacks - 1) * stack_tokens if stacks else 0
    return pages, stacks, last


def fold_factor(num_heads: int, q_len: int, m_capacity: int = 128) -> int:
    """Largest F with q_len % F == 0 and num_heads * F <= m_capacity; 1 when
    nothing larger divides ("TokenSpeed-MLA", section "Key Optimization of
    TokenSpeed MLA decode kernel": query tokens folded into the MMA M
    dimension). The folded shape is H_eff = H * F, q_eff = q_len / F."""
    best = 1
    for f in range(1, q_len + 1):
        if q_len % f == 0 and num_heads * f <= m_capacity:
            best = f
    return best


def packed_query_tiles(num_heads: int, q_len: int, m_tile: int = 128) -> int:
    """Query tiles under continuous (token * H + head) row packing: the rows
    are packed into consecutive tiles of m_tile, only the last one padded
    ("TokenSpeed-MLA", packed-query paragraph)."""
    return -(-(num_heads * q_len) // m_tile)


def mla_packed_workspace_bytes(batch: int, num_heads: int, q_len: int, split_kv: int) -> int:
    """Split-KV workspace for 512-wide V with FP32 partials under packed
    queries: batch * 128 * tiles * split_kv * 513 * 4 bytes, or zero when
    there is a single split ("TokenSpeed-MLA", packed-query paragraph)."""
    if split_kv <= 1:
        return 0
    return batch * 128 * packed_query_tiles(num_heads, q_len) * split_kv * 513 * 4


def static_anchor_tau(n_keys: int, v_max: float, delta: float = 2.0) -> float:
    """Largest safe score excess over a fixed anchor, in nats:
    tau = 88.7 - ln N - ln Vmax - delta ("Flywheel Attention", Appendix A,
    the definition of tau before Claim 1)."""
    return 88.7 - math.log(n_keys) - math.log(v_max) - delta

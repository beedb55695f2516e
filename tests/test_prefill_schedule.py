"""The persistent prefill's fixed schedule, restated on the host (no GPU).

kb_attn.hip runs a dense or partitioned prefill launch of n_items position
blocks either one workgroup per block, or, when `use_persistent_prefill`
admits it, with 8 U workgroups (one per CU) that walk a fixed list: the
workgroup p on XCD k = p % 8, local index u = p / 8, takes XCD k's items
x = 8 i + k, i = n U + u in even rounds n and n U + U - 1 - u in odd ones.
This test restates those formulas and the admission rule, and checks, for
the launches admitted on a 256-CU device, that every block runs exactly
once and every workgroup gets the same number of tiles (the balance the
rule is there to guarantee); and that the rule refuses the launches that
would not balance.
"""
import numpy as np
import pytest

HKV = 8


def admitted(batch, n_kv_heads, n_pb, resident):
    n_items = batch * n_kv_heads * n_pb
    U = resident // 8
    if resident <= 0 or resident % 8 or (batch * n_kv_heads) % 8:
        return False
    if n_items < 2 * resident or n_items > 16 * resident:
        return False
    if (n_items // 8) % (2 * U):
        return False
    return n_pb % (2 * U) == 0 or U % n_pb == 0


def item_tiles(x, batch, n_kv_heads, n_pb, pb_first):
    """Tiles of work item x (its block's diagonal tile + 1), as prefill_item maps x."""
    nbg = batch * n_kv_heads
    pbr = (x >> 3) % n_pb if nbg % 8 == 0 else x // nbg
    return pb_first + n_pb - 1 - pbr + 1


def schedule(n_items, resident):
    U = resident // 8
    lists = []
    for p in range(resident):
        k, u = p & 7, p >> 3
        n_k = (n_items - k + 7) >> 3
        items, n = [], 0
        while True:
            i = n * U + ((U - 1 - u) if n & 1 else u)
            if i >= n_k:
                break
            items.append(8 * i + k)
            n += 1
        lists.append(items)
    return lists


# (batch, q_len, kv_len): the pages' B=1 set, B=4 S=4096, 1024- and
# 2048-row partitioned calls, the test shapes of test_gpu_persistent.py
ADMITTED = [(1, 4096, 4096), (1, 8192, 8192), (1, 16384, 16384), (4, 4096, 4096), (2, 8192, 8192),
            (8, 1024, 2048), (8, 1024, 8192), (16, 1024, 16384), (4, 2048, 8192), (8, 1000, 16384)]
REFUSED = [(1, 1024, 1024), (8, 8192, 8192), (16, 16384, 16384), (3, 5000, 5000), (1, 4000, 4000),
           (2, 100, 9000), (1, 1000, 4096)]


def blocks(q_len, kv_len):
    first, last = (kv_len - q_len) // 64, (kv_len - 1) // 64
    return first, last - first + 1


@pytest.mark.parametrize("batch,q_len,kv_len", ADMITTED)
def test_admitted_launches_cover_every_block_once_and_balance(batch, q_len, kv_len):
    first, n_pb = blocks(q_len, kv_len)
    assert admitted(batch, HKV, n_pb, 256)
    n_items = batch * HKV * n_pb
    lists = schedule(n_items, 256)
    seen = np.zeros(n_items, dtype=int)
    for items in lists:
        for x in items:
            seen[x] += 1
    assert (seen == 1).all()
    tiles = [sum(item_tiles(x, batch, HKV, n_pb, first) for x in items) for items in lists]
    assert min(tiles) == max(tiles), f"tiles per workgroup {min(tiles)}..{max(tiles)}"


@pytest.mark.parametrize("batch,q_len,kv_len", REFUSED)
def test_refused_launches(batch, q_len, kv_len):
    first, n_pb = blocks(q_len, kv_len)
    assert not admitted(batch, HKV, n_pb, 256)


def test_rule_is_what_keeps_the_balance():
    """A launch the rule refuses for its block count (79 blocks per pair)
    would leave the workgroups 36% apart under this schedule."""
    batch, n_pb = 3, 79
    n_items = batch * HKV * n_pb
    tiles = [sum(item_tiles(x, batch, HKV, n_pb, 0) for x in items) for items in schedule(n_items, 256)]
    assert max(tiles) > 1.3 * np.mean(tiles)
    assert not admitted(batch, HKV, n_pb, 256)

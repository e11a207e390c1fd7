"""CPU model of the persistent grid's scheduler words (no GPU).

The decode kernel's persistent walk keeps two words at the head of a split
workspace: a 64-bit (tag, counter) word at offset 0 and a 32-bit finish
count at offset 128. This model replays the protocol under random
interleavings of the work-groups and checks what the kernels rely on:
every item is taken exactly once under both schedules, and the words end
at (tag, 0) and 0 after a counted walk even when the combine kernel does
not run. It also checks the head layout the library's sources and header
state against the workspace sizes the library reports.
"""
import os
import re

import numpy as np
import pytest

from paged_kv_cache_331_amd import pa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


class Words:
    def __init__(self, tag, counter, done):
        self.tag, self.counter, self.done = tag, counter, done


def walk(words, tag, total, grid, rng):
    """One partition-kernel launch; returns how often each item was taken."""
    counted = words.tag == tag
    taken = np.zeros(total, np.int64)
    item = list(range(grid))                 # each work-group starts with item blockIdx.x
    alive = list(range(grid))
    while alive:
        w = alive[rng.integers(len(alive))]  # any work-group may move next
        taken[item[w]] += 1
        if not counted:
            item[w] += grid
        else:
            t = words.counter                 # atomicAdd on the counter half
            words.counter = (words.counter + 1) & 0xFFFFFFFF
            item[w] = grid + t if t < total - grid else total
        if item[w] >= total:
            alive.remove(w)
            if counted:
                d = words.done                # atomicAdd on the finish count
                words.done += 1
                if d == grid - 1:
                    words.tag, words.counter, words.done = tag, 0, 0
    return taken


def combine(words, tag):
    words.tag, words.counter, words.done = tag, 0, 0


@pytest.mark.parametrize("total,grid", [(1, 1), (7, 3), (64, 64), (300, 17), (1024, 512)])
def test_every_item_once_and_words_reset(total, grid):
    rng = np.random.default_rng(total * 31 + grid)
    tag = 0x1234ABCD
    w = Words(tag=0xDEADBEEF, counter=0x55555555, done=0x777)   # a fresh, random head
    for call in range(6):
        taken = walk(w, tag, total, grid, rng)
        assert np.all(taken == 1), call
        if call % 2 == 0:
            combine(w, tag)                    # the usual case
        # after a counted walk the words are reset even without the combine
        if call >= 1:
            assert (w.tag, w.counter, w.done) == (tag, 0, 0)


def test_stale_counter_under_intact_tag_skips_items():
    """Why the header forbids changing bytes 4-7 alone: a counter that does
    not start at 0 under a valid tag skips items."""
    rng = np.random.default_rng(5)
    tag = 0x42
    w = Words(tag=tag, counter=3, done=0)
    taken = walk(w, tag, 40, 8, rng)
    assert taken.sum() == 37 and np.all(taken[8:11] == 0)


def _const(src, name):
    m = re.search(r"constexpr int " + name + r" = (\d+);", src)
    return int(m.group(1))


def test_head_layout_matches_sources_and_sizes():
    launch = open(os.path.join(ROOT, "paged_kv_cache_331_amd", "csrc", "pa_launch.h")).read()
    head, done_off = _const(launch, "kSchedBytes"), _const(launch, "kSchedDoneOffset")
    assert head == 256 and done_off == 128 and done_off % 128 == 0 and done_off + 4 <= head
    header = open(os.path.join(ROOT, "include", "pa.h")).read()
    assert "32-bit finish count at offset 128" in header
    if not os.path.exists(pa.LIB_PATH):
        pytest.skip("library not built")
    # head + three 256-byte-aligned arrays: maxima, exp-sums, weighted V sums
    for B, H, D, L, P in [(64, 32, 128, 2048, 1024), (4, 32, 128, 100000, 512), (3, 4, 64, 100, 32)]:
        n = B * H * -(-L // P)
        a256 = lambda x: -(-x // 256) * 256
        want = head + 2 * a256(4 * n) + a256(4 * n * D)
        assert pa.decode_workspace_size(B, H, D, L, P) == want

"""Host logic of the benchmark (CPU only): the state pools it cycles must
together be several times the 256 MB Infinity Cache, or a step's rewind
reads find slots written a few steps earlier still cached."""
import pytest

import bench
from speculative_decode_amd import workloads

INFINITY_CACHE = 256 << 20


@pytest.mark.parametrize("name", ["mtp_b32", "decode_b128", "mixed_b128"])
def test_small_pools_are_cycled_past_the_cache(name):
    b = workloads.make(name)
    pool_bytes = b.pool.numel() * b.pool.element_size()
    n = bench.pools_to_cycle(pool_bytes)
    assert n >= 4 and n * pool_bytes >= 8 * INFINITY_CACHE, (name, n, pool_bytes)


def test_pools_to_cycle_rule():
    gib = 1 << 30
    assert bench.pools_to_cycle(gib) == 4                 # 4 GiB of 1 GiB pools
    assert bench.pools_to_cycle(128 << 20) == 16          # 2 GiB of 128 MiB pools
    assert bench.pools_to_cycle(320 << 20) == 7           # ceil(2048 / 320)
    assert bench.pools_to_cycle(4 * gib) == 4
    assert bench.pools_to_cycle(128 << 20, 3) == 3        # an explicit --layers wins

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


@pytest.mark.parametrize("threads", [1, 3])
def test_cpu_baseline_covers_both_parts_of_a_batch(threads):
    """The oracle baseline times only the C calls, on the spec sequences and
    the single-token entries of the sample, and records the host."""
    b = workloads.mixed_batch(n_non_spec=5, n_spec=4, T=3, HK=1, HV=2, act="bf16",
                              state="bf16", seed=7)
    b.state_indices[1] = -1
    r = bench.cpu_baseline(b, 8, threads)
    assert r["value"] > 0 and r["cores"] == threads and r["kind"] == "oracle"
    assert r["nproc"] >= 1 and r["cpu_model"]
    assert "4 of 4 spec sequences" in r["sample"] and "5 of 5 single-token" in r["sample"]
    assert "(16 draft tokens" in r["sample"]            # 4 x 3 rows + 4 live singles


def test_cpu_baseline_of_a_pure_spec_workload():
    r = bench.cpu_baseline(workloads.make("tiny"), 128)
    assert r["value"] > 0 and "2 of 2 spec sequences" in r["sample"]

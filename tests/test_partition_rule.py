"""The library's partition-size rule (pkv_decode_partition_size), host-only: the values the
crossover sweep on MI355X chose (bench.py --crossover; the committed summary lists the
timings), and the rule's edges."""

import pytest

from libpkv_util import ensure_built


@pytest.fixture(scope="module")
def rule():
    ensure_built()
    from paged_kv_cache_200_amd import ops
    return ops.decode_partition_size


# (batch, context) of uniform-length bf16 workloads, 8 KV heads x 128 dims -> the partition
# size that measured fastest (within 1%), as the rule gives it
SWEEP = {(1, 512): 0, (1, 2048): 256, (1, 8192): 256, (1, 32768): 1024, (4, 2048): 256,
         (4, 8192): 1024, (4, 32768): 4096, (16, 512): 0, (16, 2048): 1024,
         (16, 8192): 4096, (16, 32768): 8192, (64, 512): 0, (64, 2048): 0, (64, 8192): 0,
         (64, 32768): 0, (256, 512): 0, (256, 2048): 0, (256, 8192): 0}


@pytest.mark.parametrize("shape,want", sorted(SWEEP.items()))
def test_sweep_choices(rule, shape, want):
    B, n = shape
    assert rule(B, 8, 128, n, B * n) == want


def test_rule_edges(rule):
    # short contexts are never split; an unknown total takes batch x max
    assert rule(1, 8, 128, 512, 0) == 0
    assert rule(4, 8, 128, 32768, 0) == rule(4, 8, 128, 32768, 4 * 32768)
    # raised to at most 8 partitions when that only doubles it: a 64-dim, 2-head batch
    # (the Qwen-shaped workload, sum 44774, max 2297) takes 512 rather than 256
    assert rule(64, 2, 64, 2297, 44774) == 512
    # the 256-sequence long-tailed workload is not split (seed 0: max 5831, sum 340004)
    assert rule(256, 8, 128, 5831, 340004) == 0
    # results are powers of two in [256, 8192], or 0
    for B in (1, 3, 17, 100):
        for n in (600, 1000, 5000, 20000, 100000):
            P = rule(B, 8, 128, n, B * n)
            assert P == 0 or (256 <= P <= 8192 and P & (P - 1) == 0 and P < n)
    assert rule(0, 8, 128, 4096, 0) == 0 and rule(4, 0, 128, 4096, 0) == 0


def test_engine_choice():
    """pkv_decode_engine: the bf16 matrix-core tile for groups of 7 and 8, the VALU pass
    otherwise; shapes the decode calls refuse are refused here too."""
    import paged_kv_cache_200_amd as pkv
    for d in (64, 128):
        for g in range(1, 9):
            want = "matrix" if g >= 7 else "valu"
            assert pkv.decode_engine("bf16", d, 2 * g, 2) == want, (d, g)
            assert pkv.decode_engine("f32", d, 2 * g, 2) == "valu", (d, g)
    for bad in (("bf16", 96, 8, 8), ("bf16", 128, 18, 2), ("bf16", 128, 9, 2)):
        with pytest.raises(Exception):
            pkv.decode_engine(*bad)

"""The CPU oracle against closed forms, brute force, a library routine,
invariants and the pages' worked copy-on-write example (no GPU needed)."""

import pytest

import oracle.block_pool as bp
import oracle.paged_attention as pa
import oracle_checks as oc


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_gather_roundtrip(kv_dtype):
    oc.check_gather_roundtrip(pa, kv_dtype)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_paged_equals_contiguous(kv_dtype):
    oc.check_paged_vs_contiguous(pa, kv_dtype)


def test_closed_forms():
    oc.check_closed_forms(pa)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_library_sdpa(kv_dtype):
    oc.check_library_sdpa(pa, kv_dtype)


def test_permutation_invariance():
    oc.check_permutation_invariance(pa)


def test_batched_equals_alone():
    oc.check_batched_equals_alone(pa)


def test_forks_identical():
    oc.check_forks_identical(pa)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_append(kv_dtype):
    oc.check_append(pa, kv_dtype)


def test_copy_blocks():
    oc.check_copy_blocks(pa)


@pytest.mark.parametrize("q_scale", [1.0, 30.0, 400.0])
def test_split_identity(q_scale):
    oc.check_split_identity(pa, "f32", q_scale=q_scale)


def test_brute_force():
    oc.check_brute_force(pa)


def test_all_pool_permutations():
    oc.check_all_pool_permutations(pa)


def test_cow_golden_example():
    oc.check_cow_golden(bp)


def test_cow_write_rules():
    oc.check_cow_write(bp)


def test_waste_bound():
    oc.check_waste_bound(bp)


def test_fifo_free_list():
    oc.check_fifo_free_list(bp)

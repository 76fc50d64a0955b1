"""Pins of oracle.accounting against the numbers the pages print and against
closed forms (eqs. (1)-(3) of the memory-budget page, core eqs. (1)-(3) of the
PagedAttention page, the OPT-13B cache figures of the NetLeverage article)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import accounting as A
from tests.conftest import load_golden

GIB = 1 << 30


def test_kv_bytes_per_token_memory_budget_example():
    g = load_golden("memory_budget_witness.json")["kv_example"]
    per_tok = A.kv_bytes_per_token(g["L"], g["H_kv"], g["d"], g["b"])
    assert per_tok == g["bytes_per_token"] == 128 * 1024
    assert A.kv_bytes(g["L"], g["H_kv"], g["d"], g["b"], [g["request_tokens"]]) == g["request_gib"] * GIB
    assert A.kv_bytes(g["L"], 32, g["d"], g["b"], [g["request_tokens"]]) == g["request_gib_at_hkv_32"] * GIB


def test_kv_bytes_sums_lengths_linearly():
    # eq. (1) is linear in the retained lengths and in each factor
    lens = [3, 5, 11]
    assert A.kv_bytes(2, 3, 4, 2, lens) == A.kv_bytes(2, 3, 4, 2, [sum(lens)])
    assert A.kv_bytes(2, 3, 4, 2, lens) == 2 * 2 * 3 * 4 * 2 * 19
    assert A.kv_bytes(1, 1, 1, 1, []) == 0


def test_opt13b_per_token_and_slots():
    g = load_golden("opt13b_cache.json")
    # the article's hidden size 5120 = 40 heads x 128 dims
    per_tok = A.kv_bytes_per_token(g["layers"], 40, 128, g["bytes_per_scalar"])
    assert per_tok == 2 * g["hidden"] * g["layers"] * g["bytes_per_scalar"]
    assert per_tok == g["bytes_per_token_kib"] * 1024
    req = A.kv_bytes(g["layers"], 40, 128, 2, [g["max_sequence_tokens"]])
    # the article counts 800 "KB" per token (KiB), so 2048 tokens are
    # 1,638,400 KiB, printed as "1.6 GB"
    assert req // 1024 == 800 * g["max_sequence_tokens"]
    assert round(req / 1024 / 1e6, 1) == g["max_request_gb_rounded"]
    slots = A.slots_in_budget(g["cache_gib"] * GIB, per_tok)
    assert slots == 15728
    assert round(slots / 1000, 1) == g["slots_thousands_rounded"]
    k = g["kernel_page_example"]
    assert k["block_size"] * k["head_size"] == k["elements_per_head_per_block"]


def test_worked_example_five_lengths():
    g = load_golden("worked_example_five_lengths.json")
    lens = g["lengths"]
    assert sum(lens) == g["useful_positions"]
    fr = g["fixed_reservation"]
    assert A.reservation_slots(lens, fr["M"]) == fr["allocated"]
    assert round(float(A.reservation_utilization(lens, fr["M"])) * 100, 2) == fr["utilization_percent"]
    for row in g["paged"]:
        B = row["B"]
        assert sum(A.allocated_slots(n, B) for n in lens) == row["allocated"]
        assert round(float(A.utilization(lens, B)) * 100, 2) == row["utilization_percent"]


def test_worked_example_blocks_per_length():
    # follows from the printed totals: 992 = 16 * 62 and 1024 = 32 * 32
    lens = [37, 91, 128, 201, 511]
    assert [A.blocks_needed(n, 16) for n in lens] == [3, 6, 8, 13, 32]
    assert [A.blocks_needed(n, 32) for n in lens] == [2, 3, 4, 7, 16]
    assert A.total_tail_waste(lens, 16) == 992 - 968
    assert A.total_tail_waste(lens, 32) == 1024 - 968


def test_tail_waste_bound_eq2():
    rng = np.random.default_rng(7)
    for B in (1, 2, 3, 4, 16, 32, 64):
        lens = rng.integers(1, 5000, size=200)
        w = A.total_tail_waste(lens, B)
        assert 0 <= w <= len(lens) * (B - 1)
        for n in lens[:20]:
            assert 0 <= A.tail_waste(int(n), B) <= B - 1
            assert A.allocated_slots(int(n), B) % B == 0
            assert A.allocated_slots(int(n), B) >= n
    # exact multiples waste nothing; one past a multiple wastes B-1
    assert A.tail_waste(64, 16) == 0
    assert A.tail_waste(65, 16) == 15
    assert A.blocks_needed(0, 16) == 0


def test_mean_tail_waste_uniform_eq3():
    g = load_golden("memory_budget_witness.json")
    T = g["uniform_lengths_max"]
    for B in (1, 2, 4, 8, 16, 32, 64, 128, 256, 512):
        assert A.mean_tail_waste_uniform(B, T) == Fraction(B - 1, 2)
    M = g["fixed_reservation_slots"]
    assert A.mean_reservation_waste_uniform(M, T) == Fraction(g["fixed_reservation_mean_waste"])
    # eq. (3) needs max_len to be a multiple of B: a non-divisor breaks it
    assert A.mean_tail_waste_uniform(3, 512) != Fraction(3 - 1, 2)


def test_six_request_example_bound_only():
    # parity unpinned: the six lengths are not printed; the printed total is
    # consistent with the eq. (2) bound for any page size of at least 7 slots
    g = load_golden("memory_budget_witness.json")["six_request_example"]
    assert g["page_tail_slots"] <= g["requests"] * (16 - 1)

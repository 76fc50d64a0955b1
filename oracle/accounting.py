"""Key/value byte budget and page-allocation accounting (exact integers).

Sources:
  * "Serving Language Models Within a Memory Budget", section 3 and eq. (1):
    uncompressed K/V state is 2 * L * H_kv * d * b bytes per retained token,
    times the sum of retained lengths.
  * same page, section 5 and eq. (2): a request of length T in pages of B
    slots is allocated B * ceil(T / B) slots; the tail waste summed over N
    nonempty requests is at most N * (B - 1).
  * same page, eq. (3): under uniform integer lengths 1..kB the expected tail
    waste of one request is (B - 1) / 2.
  * "PagedAttention and Online Inference", core eqs. (1)-(3): A_B(n),
    W_B(n) = A_B(n) - n, and position utilisation U = sum n / sum A_B(n).
"""

from __future__ import annotations

from fractions import Fraction
from typing import Iterable, Sequence


def kv_bytes_per_token(L: int, H_kv: int, d: int, b: int) -> int:
    """eq. (1) without the length sum: keys and values, every layer and head."""
    return 2 * L * H_kv * d * b


def kv_bytes(L: int, H_kv: int, d: int, b: int, lengths: Iterable[int]) -> int:
    """eq. (1): bytes of K/V state for the given retained lengths."""
    return kv_bytes_per_token(L, H_kv, d, b) * sum(int(t) for t in lengths)


def blocks_needed(n: int, B: int) -> int:
    """ceil(n / B) blocks for a sequence of n tokens (n >= 0)."""
    if n < 0 or B <= 0:
        raise ValueError("need n >= 0 and B > 0")
    return (n + B - 1) // B


def allocated_slots(n: int, B: int) -> int:
    """A_B(n) = B * ceil(n / B)."""
    return B * blocks_needed(n, B)


def tail_waste(n: int, B: int) -> int:
    """W_B(n) = A_B(n) - n."""
    return allocated_slots(n, B) - n


def total_tail_waste(lengths: Sequence[int], B: int) -> int:
    """W_tail of eq. (2), summed over the requests."""
    return sum(tail_waste(int(n), B) for n in lengths)


def reservation_slots(lengths: Sequence[int], M: int) -> int:
    """Slots held when every request reserves a fixed M positions."""
    return M * len(lengths)


def utilization(lengths: Sequence[int], B: int) -> Fraction:
    """U = sum n / sum A_B(n) (paging), as an exact fraction."""
    return Fraction(sum(int(n) for n in lengths),
                    sum(allocated_slots(int(n), B) for n in lengths))


def reservation_utilization(lengths: Sequence[int], M: int) -> Fraction:
    """Useful positions over fixed-reservation positions."""
    return Fraction(sum(int(n) for n in lengths), reservation_slots(lengths, M))


def mean_tail_waste_uniform(B: int, max_len: int) -> Fraction:
    """Expected W_B(T) for T uniform on the integers 1..max_len, by brute force."""
    total = sum(tail_waste(t, B) for t in range(1, max_len + 1))
    return Fraction(total, max_len)


def mean_reservation_waste_uniform(M: int, max_len: int) -> Fraction:
    """Expected M - T for T uniform on 1..max_len, by brute force."""
    return Fraction(sum(M - t for t in range(1, max_len + 1)), max_len)


def slots_in_budget(cache_bytes: int, bytes_per_token: int) -> int:
    """Whole token slots that fit in a cache budget."""
    return cache_bytes // bytes_per_token

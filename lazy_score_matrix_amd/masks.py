"""Pair masks for lazy scores (guide, Task Map, Attention row: causal, band
and same_group). Each helper returns op entries for ``lazy(..., ops=...)``,
``LazyScores.masked`` or a consumer's ``mask=`` argument; a masked pair takes
no part in any consumer's reduction.

    e = pw.lazy(Q, K, "linear", ops=[("mul", 0.125)])
    out = e.softmax_matmul(V, mask=pw.masks.causal())
"""
from __future__ import annotations


def causal(diagonal: int = 0):
    """Keep pairs with j - i <= diagonal (j <= i for the default)."""
    return [("band_upper", int(diagonal))]


def band(lower: int, upper: int):
    """Keep pairs with i - lower <= j <= i + upper."""
    return [("band_lower", int(lower)), ("band_upper", int(upper))]


def same_group(row_groups, column_groups):
    """Keep pairs whose int64 group ids match: row_groups[i] == column_groups[j]."""
    return [("group_rows", row_groups), ("group_columns", column_groups)]


def rows(keep):
    """Keep the rows i with keep[i] true (bool or uint8 [N])."""
    return [("mask_rows", keep)]


def columns(keep):
    """Keep the columns j with keep[j] true (bool or uint8 [M])."""
    return [("mask_columns", keep)]

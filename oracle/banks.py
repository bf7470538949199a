"""Shared-memory bank model and XOR swizzle (test infrastructure only).

Source: "Tensor Core 数据布局的演进", section "先记住两项访存要求" (two memory
requirements): shared-memory addresses of one access should spread over the
banks; and section "写回结果与对 shared memory 做 swizzle": in an (8, 64) fp16
tile each row is 128 bytes, so with 4-byte banks the 8 elements of one column
fall into one bank (an 8-way conflict); hand-written XOR addressing keeps rows
contiguous for writes and spreads column reads over the banks.

The model: banks are ``bank_bytes`` wide and there are ``n_banks`` of them; the
lanes of one access are served in groups of ``lanes_per_cycle``; within a
group, a bank that must deliver k distinct words takes k cycles (the same
word to several lanes is a broadcast).  The conflict degree of an access is
the largest k over groups and banks.
"""
from __future__ import annotations

from collections import defaultdict


def conflict_ways(byte_addrs, access_bytes=4, n_banks=32, bank_bytes=4, lanes_per_cycle=None):
    addrs = list(byte_addrs)
    if lanes_per_cycle is None:
        lanes_per_cycle = len(addrs)
    worst = 0
    for g in range(0, len(addrs), lanes_per_cycle):
        words = defaultdict(set)
        for a in addrs[g:g + lanes_per_cycle]:
            for w in range(a // bank_bytes, (a + access_bytes - 1) // bank_bytes + 1):
                words[w % n_banks].add(w)
        worst = max(worst, max(len(v) for v in words.values()))
    return worst


def xor_swizzle_chunk(row, chunk, chunks_per_row):
    """The textbook XOR layout: 16-byte chunk c of row r is stored at c ^ (r mod chunks)."""
    return chunk ^ (row % chunks_per_row)

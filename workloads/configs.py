"""Workload definitions: the five seeded synthetic configurations and their
small parity variants.

Each workload names the shapes, sizes and structure of one case the method is
run on.  Nothing here computes any part of the method; these are plain
records consumed by ``workloads.gen`` (input synthesis), the tests and the
benchmark.

The full-size configurations follow the workload descriptions used for this
library's headline measurements:

* ``tiny_decode``             batch 1, 4 q heads / 1 KV head, d 64, fp32,
                              1024 tokens in 64 pages of 16, sink page 0 +
                              last 4 pages + top-8.
* ``llama3_8b_decode_32k``    batch 32, 32/8 heads, d 128, bf16, 32768 tokens,
                              pages of 64; 5% planted heavy-hitter pages;
                              sink 64 tokens + window 512 tokens + top-41.
* ``token_head_decode_128k``  batch 8, 32/8 heads, d 128, bf16, 131072 tokens,
                              pages of 16; per-query-head lists from Gumbel
                              draft scores, 10% of pages kept, 16 splits.
* ``chunked_prefill_128k``    1 sequence, 32/8 heads, d 128, bf16, a 2048-token
                              query chunk at 126976..129023 over 129024 KV
                              tokens, 64x64 blocks, diagonal + first block +
                              8% random blocks per row.
* ``mla_tiered_decode_64k``   batch 16, 2 query tokens (MTP), 128 heads over one
                              512+64 latent, bf16, 65536 tokens, pages of 64,
                              Critical 8 pages (all heads) + Ambient 32 pages
                              (32 seeded heads each).

The token-to-page conversions (sink 64 tokens = 1 page of 64, window 512 tokens
= 8 pages) are stated here so that the C interface can speak in pages only.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    q_tokens: int
    n_q_heads: int
    n_kv_heads: int
    d_qk: int
    d_v: int
    dtype: str                 # "bf16" | "fp32" | "fp8" (E4M3 K/V pages with per-page scales, bf16 q)
    context: int               # tokens per sequence (unless seq_lens given)
    page_size: int
    mode: str                  # "per_kv_head" | "per_q_head"
    sink_pages: int
    window_pages: int
    top_k: int
    critical_k: Optional[int] = None   # None: untiered lists
    ambient_heads: int = 0             # heads per Ambient page (tiered only)
    scores: str = "summary"            # "summary": q . mean(K_page); "gumbel": given draft scores
    plant_fraction: float = 0.0        # fraction of pages given +offset along the query direction
    plant_offset: float = 0.0
    num_splits: int = 0                # 0: library chooses
    latent: bool = False               # MLA: V is the first d_v dims of the K row (no V pool)
    seq_lens: Optional[Tuple[int, ...]] = None  # ragged lengths (overrides context)
    extra_pool_pages: int = 0          # unreferenced physical pages in the pool

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_sel(self) -> int:
        return self.n_kv_heads if self.mode == "per_kv_head" else self.n_q_heads

    def lengths(self) -> Tuple[int, ...]:
        return tuple(self.seq_lens) if self.seq_lens is not None else (self.context,) * self.batch

    @property
    def max_pages(self) -> int:
        return max(math.ceil(L / self.page_size) for L in self.lengths())

    @property
    def n_phys_pages(self) -> int:
        return sum(math.ceil(L / self.page_size) for L in self.lengths()) + self.extra_pool_pages

    @property
    def list_stride(self) -> int:
        # forced pages + top-k, never more than the pages a sequence has
        return min(self.max_pages, self.sink_pages + self.window_pages + self.top_k)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def tiered(self) -> bool:
        return self.critical_k is not None

    def replace(self, **kw) -> "DecodeWorkload":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    d: int
    dtype: str
    q_len: int
    q_start: int
    page_size: int
    block_q: int
    random_fraction: float     # fraction of eligible off-diagonal blocks kept per mask row
    extra_pool_pages: int = 0
    mask_kind: str = "random"  # "random" | "ones" | "shared_columns"

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_len(self) -> int:
        return self.q_start + self.q_len

    @property
    def n_kv_blocks(self) -> int:
        return math.ceil(self.kv_len / self.page_size)

    @property
    def n_q_blocks(self) -> int:
        return math.ceil(self.q_len / self.block_q)

    @property
    def n_phys_pages(self) -> int:
        return self.n_kv_blocks + self.extra_pool_pages

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def replace(self, **kw) -> "PrefillWorkload":
        return dataclasses.replace(self, **kw)


# ---------------------------------------------------------------- full size
TINY_DECODE = DecodeWorkload(
    name="tiny_decode", batch=1, q_tokens=1, n_q_heads=4, n_kv_heads=1, d_qk=64, d_v=64,
    dtype="fp32", context=1024, page_size=16, mode="per_kv_head",
    sink_pages=1, window_pages=4, top_k=8)

LLAMA3_DECODE_32K = DecodeWorkload(
    name="llama3_8b_decode_32k", batch=32, q_tokens=1, n_q_heads=32, n_kv_heads=8, d_qk=128,
    d_v=128, dtype="bf16", context=32768, page_size=64, mode="per_kv_head",
    sink_pages=1, window_pages=8, top_k=41, plant_fraction=0.05, plant_offset=2.0)

TOKEN_HEAD_DECODE_128K = DecodeWorkload(
    name="token_head_decode_128k", batch=8, q_tokens=1, n_q_heads=32, n_kv_heads=8, d_qk=128,
    d_v=128, dtype="bf16", context=131072, page_size=16, mode="per_q_head",
    sink_pages=0, window_pages=0, top_k=819, scores="gumbel", num_splits=16)

CHUNKED_PREFILL_128K = PrefillWorkload(
    name="chunked_prefill_128k", n_q_heads=32, n_kv_heads=8, d=128, dtype="bf16",
    q_len=2048, q_start=126976, page_size=64, block_q=64, random_fraction=0.08)

MLA_TIERED_DECODE_64K = DecodeWorkload(
    name="mla_tiered_decode_64k", batch=16, q_tokens=2, n_q_heads=128, n_kv_heads=1, d_qk=576,
    d_v=512, dtype="bf16", context=65536, page_size=64, mode="per_kv_head",
    sink_pages=0, window_pages=0, top_k=40, critical_k=8, ambient_heads=32, latent=True)

# the Llama-3-8B decode layer over FP8 K/V pages (one scale per page and KV head)
LLAMA3_DECODE_32K_FP8 = LLAMA3_DECODE_32K.replace(name="llama3_8b_decode_32k_fp8", dtype="fp8")

FULL = {w.name: w for w in (TINY_DECODE, LLAMA3_DECODE_32K, TOKEN_HEAD_DECODE_128K,
                             CHUNKED_PREFILL_128K, MLA_TIERED_DECODE_64K, LLAMA3_DECODE_32K_FP8)}

# ---------------------------------------------------------- parity variants
# Same structure as the full-size cases, sized so the oracle finishes in
# seconds, spanning several tiles/splits and a ragged tail.
SMALL = {
    "tiny_decode": TINY_DECODE,
    "llama3_decode_small": LLAMA3_DECODE_32K.replace(
        name="llama3_decode_small", batch=3, n_q_heads=8, n_kv_heads=2, context=0,
        seq_lens=(64 * 37 + 13, 64 * 20, 64 * 9 + 1), top_k=7, sink_pages=1, window_pages=2,
        extra_pool_pages=5),
    "token_head_decode_small": TOKEN_HEAD_DECODE_128K.replace(
        name="token_head_decode_small", batch=2, n_q_heads=8, n_kv_heads=2, context=16 * 301,
        top_k=30, num_splits=4),
    "mla_tiered_decode_small": MLA_TIERED_DECODE_64K.replace(
        name="mla_tiered_decode_small", batch=2, n_q_heads=32, context=64 * 30 + 5,
        top_k=10, critical_k=3, ambient_heads=8),
    # every other shape the decode side dispatches: head dim 64 in bf16 at both
    # page sizes and both selection modes, the staged per-KV-head path on pages
    # of 16, per-query-head lists on pages of 64, and fp32 caches at d 128
    "bf16_d64_p16_kv_small": LLAMA3_DECODE_32K.replace(
        name="bf16_d64_p16_kv_small", batch=2, n_q_heads=8, n_kv_heads=2, d_qk=64, d_v=64, page_size=16,
        context=0, seq_lens=(16 * 70 + 5, 16 * 33), top_k=9, sink_pages=1, window_pages=3, plant_fraction=0.0,
        extra_pool_pages=3),
    "bf16_d64_p64_q_small": LLAMA3_DECODE_32K.replace(
        name="bf16_d64_p64_q_small", batch=2, n_q_heads=4, n_kv_heads=2, d_qk=64, d_v=64, mode="per_q_head",
        context=0, seq_lens=(64 * 25 + 7, 64 * 12), top_k=6, sink_pages=1, window_pages=2, plant_fraction=0.0),
    "bf16_d128_p16_kv_small": LLAMA3_DECODE_32K.replace(
        name="bf16_d128_p16_kv_small", batch=2, n_q_heads=8, n_kv_heads=2, page_size=16, context=0,
        seq_lens=(16 * 150 + 9, 16 * 77), top_k=20, sink_pages=1, window_pages=4, plant_fraction=0.0),
    "bf16_d128_p64_q_small": LLAMA3_DECODE_32K.replace(
        name="bf16_d128_p64_q_small", batch=2, n_q_heads=4, n_kv_heads=2, mode="per_q_head", context=0,
        seq_lens=(64 * 30 + 3, 64 * 17), top_k=8, sink_pages=1, window_pages=2, plant_fraction=0.0),
    "fp32_d128_p64_kv_small": TINY_DECODE.replace(
        name="fp32_d128_p64_kv_small", batch=2, d_qk=128, d_v=128, page_size=64, context=0,
        seq_lens=(64 * 20 + 1, 64 * 11), top_k=5, sink_pages=1, window_pages=2),
    "fp32_d64_p16_q_small": TINY_DECODE.replace(
        name="fp32_d64_p16_q_small", batch=2, n_q_heads=4, n_kv_heads=2, mode="per_q_head", context=0,
        seq_lens=(16 * 50 + 3, 16 * 31), top_k=7, sink_pages=1, window_pages=3),
    # FP8 K/V pages: per-KV-head lists on pages of 64, per-query-head lists on pages of 16
    "fp8_d128_p64_kv_small": LLAMA3_DECODE_32K.replace(
        name="fp8_d128_p64_kv_small", dtype="fp8", batch=3, n_q_heads=8, n_kv_heads=2, context=0,
        seq_lens=(64 * 37 + 13, 64 * 20, 64 * 9 + 1), top_k=7, sink_pages=1, window_pages=2, extra_pool_pages=5),
    "fp8_d128_p16_q_small": TOKEN_HEAD_DECODE_128K.replace(
        name="fp8_d128_p16_q_small", dtype="fp8", batch=2, n_q_heads=8, n_kv_heads=2, context=16 * 301,
        top_k=30, num_splits=4),
    "chunked_prefill_small": CHUNKED_PREFILL_128K.replace(
        name="chunked_prefill_small", n_q_heads=8, n_kv_heads=2, q_len=200, q_start=1000,
        random_fraction=0.3, extra_pool_pages=3),
}

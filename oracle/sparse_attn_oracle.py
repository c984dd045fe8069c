"""CPU oracle for dynamic page/block-sparse attention over a paged KV cache.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
library's product path never does, and shares no code with it.

Plain, slow and direct: numpy float64 throughout (inputs arrive as exact
upcasts of the bf16/fp32 bits), explicit loops over sequences, heads and
pages, library primitives (sum, matmul, a stable sort) as steps, no blocking,
fusion or reordering.  The quantities that decide an integer outcome (the page
scores that top-k ranks) are rounded to fp32 exactly as the library hands them
between its calls; both sides accumulate in float64 before that rounding.

Sources (pages as titled on the web; sections named):
  [UAE]   "Universal Attention Engine - Declarative Sparse Attention for
          Production": section "The Product" (sink_tokens, local_window,
          cache_budget), "Content-Dependent Dynamic Routing (Novel)" (router
          top_k_blocks(q @ mean(k_blocks), k); selected blocks get full
          fine-grained attention; only selected blocks are loaded),
          "Milestones / Phase 1" (sink+local+sparse pattern),
          "Architecture / Layer 3" (PagedAttention-compatible layout).
  [TS]    "TileSparse: Arithmetic-Intensity-Aware Sparse Attention for
          Compute-Bound LLM Decoding" (README): "Motivation" (QK 2D sparsity,
          Tiered QK 2D sparsity: Critical tier of alpha pages with all query
          heads, Ambient tier of beta pages with h heads), "Two
          implementations, by design" (mask-based path == per-head page-list
          Flash-decode), "Configuration" (critical_top_count, ambient_head_count,
          key_top_count), TILESPARSE_MODE=streaming (sinks + window only).
  [STS]   STS abstract (page titled "Vortex: Efficient and Programmable Sparse
          Attention Serving for AI Agents"): draft-model scores build a
          token-and-head-wise sparsity mask.
  [CA]    CompactAttention abstract (page titled "Causal Attention on CPU: A
          Cache-Aware and Load-Balanced Scheduling Kernel for Prefill"): 2D
          block masks become GQA-aware per-group KV block tables by Q-block
          union then intra-group union; tables keep every selected block and KV
          is read in place from the paged cache under chunked prefill.

Readings where the pages are silent (each is listed with its reason in the
design notes): the router score is the unscaled dot product of the query summed
over the selection head's query heads and query tokens with the page's mean key
over its valid tokens; sink/window/top-k are counted in pages, forced pages are
not top-k candidates, ranking is (score descending, logical index ascending)
with NaN last; lists are ascending logical ids (tiered: Critical segment then
Ambient segment); each query row softmaxes over exactly its own token set;
an empty token set gives output 0 and lse -inf; the prefill union is taken over
all Q-blocks of the chunk and every query of a group attends causally to the
whole group table; a skipped block, and a page in the AutoTuner's mass
estimate, stands in for its n tokens by its mean key (log-weight
sm_scale q.mu + ln n); the AutoTuner's budget counts (page, query head)
entries beyond the forced pages, its coverage is the estimated mass on the
(head, page) pairs the tiered decode computes, and an Ambient page takes the
heads of largest estimated mass.

Pins (tests/test_oracle_pins.py): brute force in pure Python on tiny inputs,
torch's scaled_dot_product_attention (float64, CPU) for select-all and
all-ones-mask cases, closed forms (constant V, single token, constant pages),
invariants (pool permutation, linearity of the score, union contains the
mask, split/merge), hand-derived golden lists under tests/golden/.
"""
from __future__ import annotations

import math
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

PER_KV_HEAD = "per_kv_head"
PER_Q_HEAD = "per_q_head"


def n_pages_of(seq_len: int, page_size: int) -> int:
    return (int(seq_len) + page_size - 1) // page_size


def valid_tokens(seq_len: int, logical_page: int, page_size: int) -> int:
    """Tokens of logical page ``logical_page`` that lie below ``seq_len``."""
    return max(0, min(page_size, int(seq_len) - logical_page * page_size))


# --------------------------------------------------------------------- a0
def page_summary(k_pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                 page_size: int, last_pages: int = 0) -> np.ndarray:
    """Mean key of each referenced physical page, per KV head  [UAE routing: mean(k_blocks)].

    mu[p, g, :] = (sum over the page's valid tokens j of K[p, g, j, :]) / n_valid,
    accumulated in float64 and rounded to fp32.  ``last_pages`` > 0 restricts the
    update to the last ``last_pages`` logical pages of each sequence.  Entries
    of pages not updated are NaN.
    """
    n_phys, n_kv, P, d = k_pool.shape
    mu = np.full((n_phys, n_kv, d), np.nan, dtype=np.float32)
    for b in range(block_table.shape[0]):
        n = n_pages_of(seq_lens[b], P)
        first = 0 if last_pages <= 0 else max(0, n - last_pages)
        for lp in range(first, n):
            nv = valid_tokens(seq_lens[b], lp, P)
            phys = int(block_table[b, lp])
            rows = np.asarray(k_pool[phys, :, :nv, :], dtype=np.float64)   # [n_kv][nv][d]
            mu[phys] = (rows.sum(axis=1) / nv).astype(np.float32)
    return mu


# --------------------------------------------------------------------- a1
def selection_heads(s: int, mode: str, group: int) -> Tuple[List[int], int]:
    """Query heads pooled by selection head ``s`` and the KV head it reads."""
    if mode == PER_KV_HEAD:
        return list(range(s * group, (s + 1) * group)), s
    return [s], s // group


def page_scores(q: np.ndarray, mu: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                page_size: int, n_kv_heads: int, mode: str) -> np.ndarray:
    """Router score of every page  [UAE routing: q @ mean(k_blocks); STS/TS per-head selection].

    s[b, sel, p] = fp32( sum_d Qbar[d] * mu[phys(b, p), g(sel), d] ),
    Qbar = sum over query tokens t and the selection head's query heads h of
    q[b, t, h, :] (float64).  Pages past the sequence's end get NaN.
    """
    B, T, Hq, d = q.shape
    G = Hq // n_kv_heads
    n_sel = n_kv_heads if mode == PER_KV_HEAD else Hq
    max_pages = block_table.shape[1]
    out = np.full((B, n_sel, max_pages), np.nan, dtype=np.float32)
    for b in range(B):
        n = n_pages_of(seq_lens[b], page_size)
        for s in range(n_sel):
            heads, g = selection_heads(s, mode, G)
            qbar = np.zeros(d, dtype=np.float64)
            for t in range(T):
                for h in heads:
                    qbar += q[b, t, h].astype(np.float64)
            for lp in range(n):
                m = mu[int(block_table[b, lp]), g].astype(np.float64)
                out[b, s, lp] = np.float32(np.dot(qbar, m))
    return out


# --------------------------------------------------------------------- a2
def forced_pages(n: int, sink_pages: int, window_pages: int) -> List[int]:
    """Sink pages [0, sink) and window pages [n - window, n), clipped  [UAE: sink_tokens, local_window]."""
    f = set(range(0, min(sink_pages, n))) | set(range(max(0, n - window_pages), n))
    return sorted(f)


def rank_candidates(scores_row: np.ndarray, candidates: Sequence[int]) -> List[int]:
    """Candidates ordered by (score descending, logical index ascending), NaN last."""
    cand = np.asarray(candidates, dtype=np.int64)
    if cand.size == 0:
        return []
    sc = scores_row[cand].astype(np.float64)
    nan = np.isnan(sc)
    neg = np.where(nan, np.inf, -sc)          # -0.0 and +0.0 compare equal
    order = np.lexsort((cand, neg, nan))      # primary: NaN flag, then -score, then index
    return [int(x) for x in cand[order]]


def select_pages(scores: np.ndarray, n_pages: Sequence[int], sink_pages: int, window_pages: int,
                 top_k: int, critical_k: Optional[int] = None):
    """Per-selection-head page lists  [UAE sink+local+sparse; TS tiers; STS top-k masks].

    F = forced pages; C = the other pages; the first min(top_k, |C|) of C in
    rank order are selected.  Untiered: list = ascending(F u selected).
    Tiered: Critical = ascending(F u first critical_k selected), Ambient =
    ascending(remaining selected); list = Critical then Ambient.
    Returns (lists [B][S][stride] int32 padded with -1, counts [B][S],
    critical counts [B][S] or None).
    """
    B, S, max_pages = scores.shape
    stride = max_pages
    lists = np.full((B, S, stride), -1, dtype=np.int32)
    counts = np.zeros((B, S), dtype=np.int32)
    ccounts = np.zeros((B, S), dtype=np.int32) if critical_k is not None else None
    for b in range(B):
        n = int(n_pages[b])
        forced = forced_pages(n, sink_pages, window_pages)
        fset = set(forced)
        cand = [i for i in range(n) if i not in fset]
        for s in range(S):
            order = rank_candidates(scores[b, s], cand)
            k_eff = min(max(top_k, 0), len(order))
            chosen = order[:k_eff]
            if critical_k is None:
                lst = sorted(fset | set(chosen))
            else:
                ck = min(max(critical_k, 0), k_eff)
                crit = sorted(fset | set(chosen[:ck]))
                amb = sorted(chosen[ck:])
                lst = crit + amb
                ccounts[b, s] = len(crit)
            counts[b, s] = len(lst)
            lists[b, s, :len(lst)] = lst
    return lists, counts, ccounts


# ----------------------------------------------------------------- a3-a5
def head_bit(mask_words: np.ndarray, h: int) -> bool:
    return bool((int(mask_words[h // 32]) >> (h % 32)) & 1)


def row_pages(b: int, s: int, h: int, page_lists, page_counts, critical_counts, ambient_mask) -> List[int]:
    """Logical pages query head h of selection head s attends  [TS Tiered QK 2D sparsity].

    Untiered: the whole list.  Tiered: the Critical segment plus each Ambient
    page whose head mask has bit h.
    """
    cnt = int(page_counts[b, s])
    pages = [int(x) for x in page_lists[b, s, :cnt]]
    if critical_counts is None:
        return pages
    cc = int(critical_counts[b, s])
    amb = [p for p in pages[cc:] if head_bit(ambient_mask[b, p], h)]
    return pages[:cc] + amb


def gather_tokens(k_pool, v_pool, block_table, b, g, pages, seq_len, page_size, d_v):
    """Keys/values of the given logical pages (valid tokens only), in ascending token order.

    K pool is [phys][g][token][d]; V pool is page-transposed [phys][g][d_v][token];
    with no V pool, V is the first d_v dims of the K row (MLA latent).
    """
    ks, vs = [], []
    for lp in sorted(pages):
        nv = valid_tokens(seq_len, lp, page_size)
        if nv == 0:
            continue
        phys = int(block_table[b, lp])
        k = np.asarray(k_pool[phys, g, :nv, :], dtype=np.float64)
        if v_pool is None:
            v = k[:, :d_v]
        else:
            v = np.asarray(v_pool[phys, g, :, :nv], dtype=np.float64).T
        ks.append(k)
        vs.append(v)
    if not ks:
        return None, None
    return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)


def softmax_attend(qrow: np.ndarray, K: Optional[np.ndarray], V: Optional[np.ndarray], sm_scale: float,
                   d_v: int):
    """Softmax attention of one query over exactly the given tokens  [UAE: selected blocks get full attention].

    z_j = sm_scale * q . K_j; o = sum_j softmax(z)_j V_j; lse = log sum_j exp(z_j).
    Empty token set: o = 0, lse = -inf.
    """
    if K is None or K.shape[0] == 0:
        return np.zeros(d_v, dtype=np.float64), -np.inf
    z = sm_scale * (K @ qrow.astype(np.float64))
    m = z.max()
    e = np.exp(z - m)
    l = e.sum()
    return (e @ V) / l, m + math.log(l)


def sparse_decode(q, k_pool, v_pool, block_table, seq_lens, page_size, page_lists, page_counts,
                  n_kv_heads, mode, sm_scale, critical_counts=None, ambient_mask=None, d_v=None,
                  rows: Optional[Iterable[Tuple[int, int, int]]] = None):
    """Decode attention of every query row over its selected pages  [TS page-list Flash-decode; UAE gather decode].

    Returns (out [B][T][Hq][d_v] float64, lse [B][T][Hq] float64).  With
    ``rows`` only those (b, t, h) entries are computed (others stay 0 / NaN).
    """
    B, T, Hq, _ = q.shape
    G = Hq // n_kv_heads
    P = page_size
    if d_v is None:
        d_v = v_pool.shape[2]
    out = np.zeros((B, T, Hq, d_v), dtype=np.float64)
    lse = np.full((B, T, Hq), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(b, t, h) for b in range(B) for t in range(T) for h in range(Hq)]
    for (b, t, h) in rows:
        s = h // G if mode == PER_KV_HEAD else h
        g = h // G
        pages = row_pages(b, s, h, page_lists, page_counts, critical_counts, ambient_mask)
        K, V = gather_tokens(k_pool, v_pool, block_table, b, g, pages, seq_lens[b], P, d_v)
        out[b, t, h], lse[b, t, h] = softmax_attend(q[b, t, h], K, V, sm_scale, d_v)
    return out, lse


def split_ranges(count: int, num_splits: int) -> List[Tuple[int, int]]:
    """Contiguous chunks of a list of ``count`` entries whose sizes differ by at most one."""
    base, extra = divmod(count, num_splits)
    out, start = [], 0
    for i in range(num_splits):
        n = base + (1 if i < extra else 0)
        out.append((start, start + n))
        start += n
    return out


def lse_merge(o_parts: np.ndarray, lse_parts: np.ndarray):
    """Combine per-split partial outputs: o = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max).

    o_parts [S][d_v] (each normalised over its own tokens), lse_parts [S].
    All-empty gives o = 0, lse = -inf.
    """
    M = np.max(lse_parts)
    if not np.isfinite(M):
        return np.zeros(o_parts.shape[1]), -np.inf
    w = np.exp(lse_parts - M)
    L = w.sum()
    return (w[:, None] * o_parts).sum(axis=0) / L, M + math.log(L)


# ------------------------------------------------------------------- a6-a7
def gqa_union_block_table(block_mask: np.ndarray, n_kv_heads: int):
    """GQA-aware per-group KV block tables  [CA: Q-block union then intra-group union].

    U[h, kb] = OR over Q-blocks of mask[h, qb, kb]; T[g, kb] = OR over the
    group's heads of U[h, kb]; table_g = ascending {kb : T[g, kb]}.
    Returns (tables [n_kv_heads][n_kv_blocks] int32 padded with -1, counts).
    """
    Hq, nqb, nkb = block_mask.shape
    G = Hq // n_kv_heads
    tables = np.full((n_kv_heads, nkb), -1, dtype=np.int32)
    counts = np.zeros(n_kv_heads, dtype=np.int32)
    for g in range(n_kv_heads):
        union = np.zeros(nkb, dtype=bool)
        for h in range(g * G, (g + 1) * G):
            for qb in range(nqb):
                union |= block_mask[h, qb] != 0
        ids = np.flatnonzero(union)
        tables[g, :ids.size] = ids
        counts[g] = ids.size
    return tables, counts


def block_sparse_prefill(q, k_pool, v_pool, block_table_row, seq_len, page_size, q_start,
                         tables, counts, n_kv_heads, sm_scale,
                         rows: Optional[Iterable[Tuple[int, int]]] = None):
    """Chunked-prefill attention in place over the group block tables  [CA].

    Query i sits at position q_start + i; head h attends the tokens j of the
    blocks in table_{g(h)} with j <= q_start + i and j < seq_len.
    q [q_len][Hq][d]; returns (out [q_len][Hq][d] float64, lse [q_len][Hq]).
    ``rows`` restricts to the given (i, h) pairs.
    """
    q_len, Hq, d = q.shape
    G = Hq // n_kv_heads
    P = page_size
    out = np.zeros((q_len, Hq, d), dtype=np.float64)
    lse = np.full((q_len, Hq), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(i, h) for i in range(q_len) for h in range(Hq)]
    by_group = {}
    for (i, h) in rows:
        by_group.setdefault(h // G, []).append((i, h))
    for g, grp_rows in by_group.items():
        pos, ks, vs = [], [], []
        for kb in [int(x) for x in tables[g, :int(counts[g])]]:
            nv = valid_tokens(seq_len, kb, P)
            if nv == 0:
                continue
            phys = int(block_table_row[kb])
            ks.append(np.asarray(k_pool[phys, g, :nv, :], dtype=np.float64))
            vs.append(np.asarray(v_pool[phys, g, :, :nv], dtype=np.float64).T)
            pos.append(kb * P + np.arange(nv))
        if not ks:
            for (i, h) in grp_rows:
                out[i, h], lse[i, h] = np.zeros(d), -np.inf
            continue
        K, V, J = np.concatenate(ks), np.concatenate(vs), np.concatenate(pos)
        heads = sorted({h for (_, h) in grp_rows})
        for h in heads:
            qi = np.array([i for (i, hh) in grp_rows if hh == h], dtype=np.int64)
            Qh = np.asarray(q[qi, h, :], dtype=np.float64)              # [rows][d]
            Z = sm_scale * (Qh @ K.T)                                   # [rows][tokens]
            visible = J[None, :] <= (q_start + qi)[:, None]             # causal: j <= position
            Z = np.where(visible, Z, -np.inf)
            m = Z.max(axis=1)
            empty = ~np.isfinite(m)
            m_safe = np.where(empty, 0.0, m)
            E = np.exp(Z - m_safe[:, None])                             # exp(-inf) = 0
            L = E.sum(axis=1)
            L_safe = np.where(empty, 1.0, L)
            O = (E @ V) / L_safe[:, None]
            out[qi, h] = np.where(empty[:, None], 0.0, O)
            with np.errstate(divide="ignore"):
                lse[qi, h] = np.where(empty, -np.inf, m_safe + np.log(L_safe))
    return out, lse


# ------------------------------------------------------------- prefill mask
def prefill_block_mask(q, mu, block_table_row, seq_len, page_size, q_start, block_q, n_kv_blocks,
                       n_kv_heads, sm_scale, top_k=None, max_gap=None):
    """2D block mask for a prefill chunk by block-level pattern discovery.

    Sources: the block-sparse prefill brief on the Paperraft page ("instantaneous
    pattern discovery, max-based dynamic thresholding"), the router score form of
    [UAE] "Content-Dependent Dynamic Routing" (pooled query against the block's
    mean key) and the mask structure the CompactAttention abstract feeds to its
    Q-block / intra-group union ([CA]).

    For query head h and Q-block qb (queries i in [qb*block_q, min((qb+1)*block_q, q_len))):
      qbar = mean over the Q-block's queries of q[i, h, :]   (float64)
      n    = number of KV blocks holding a token at or before the block's last
             position q_start + i_last (and below seq_len): the causal blocks
      s[kb] = fp32( sm_scale * sum_d qbar[d] * mu[phys(kb), g(h), d] ),  kb < n
      forced = {0} u [kb_lo, n), kb_lo = block of the first query's position
               (the sink block and the diagonal blocks)
      chosen (top-k mode)     = the first min(top_k, |C|) candidates C = causal
                                minus forced, by (score desc, index asc)
      chosen (threshold mode) = {c in C : s[c] >= max_{kb < n} s[kb] - max_gap}
      mask[h, qb, kb] = 1 for kb in forced u chosen, else 0.
    Exactly one of top_k / max_gap is given.  Returns (mask uint8
    [Hq][nqb][n_kv_blocks], scores fp32 [Hq][nqb][n_kv_blocks] with NaN past
    the causal blocks).
    """
    assert (top_k is None) != (max_gap is None)
    q_len, Hq, d = q.shape
    G = Hq // n_kv_heads
    P = page_size
    nqb = (q_len + block_q - 1) // block_q
    n_seq_pages = n_pages_of(seq_len, P)
    mask = np.zeros((Hq, nqb, n_kv_blocks), dtype=np.uint8)
    scores = np.full((Hq, nqb, n_kv_blocks), np.nan, dtype=np.float32)
    for h in range(Hq):
        g = h // G
        for qb in range(nqb):
            i0, i1 = qb * block_q, min((qb + 1) * block_q, q_len)
            qbar = np.asarray(q[i0:i1, h, :], dtype=np.float64).sum(axis=0) / (i1 - i0)
            n = min((q_start + i1 - 1) // P + 1, n_seq_pages, n_kv_blocks)
            if n <= 0:
                continue
            kb_lo = min((q_start + i0) // P, n - 1)
            for kb in range(n):
                m = np.asarray(mu[int(block_table_row[kb]), g], dtype=np.float64)
                scores[h, qb, kb] = np.float32(sm_scale * np.dot(qbar, m))
            forced = {0} | set(range(kb_lo, n))
            cand = [kb for kb in range(n) if kb not in forced]
            if top_k is not None:
                chosen = rank_candidates(scores[h, qb], cand)[:max(0, min(top_k, len(cand)))]
            else:
                row = scores[h, qb, :n]
                top = np.float32(np.max(row))
                thr = np.float32(top - np.float32(max_gap))
                chosen = [kb for kb in cand if row[kb] >= thr]
            for kb in forced | set(chosen):
                mask[h, qb, kb] = 1
    return mask, scores


# -------------------------------------------------------------- FP8 pages
def fp8_e4m3_to_float(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP FP8 E4M3 byte (1 sign bit, 4 exponent bits with bias 7,
    3 mantissa bits; exponent 0 is subnormal, m * 2^-9; S.1111.111 is NaN; no
    infinities), as float64.

    Source: the quantized KV cache named in "Universal Attention Engine", "Key
    Design Decisions" 2 (cache format paged, block-sparse, quantized) and
    "Milestones" (Phase 3: quantized KV cache support), and the FP8 regime of
    the block-sparse prefill brief; the byte encoding is the OCP 8-bit floating
    point E4M3 format.
    """
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = sign * (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = sign * m * 2.0 ** -9
    out = np.where(e == 0, sub, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, out)


def dequantize_pages(pool_u8: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """Dequantised pool: every element of page (phys, g) is its FP8 value times
    the page's scale scale[phys, g] (one scale per page and KV head for K and
    one for V, applied when the page is loaded).  pool_u8 [n_phys][Hkv][...]."""
    vals = fp8_e4m3_to_float(pool_u8)
    s = np.asarray(scale, dtype=np.float64).reshape(scale.shape + (1,) * (pool_u8.ndim - 2))
    return vals * s


# -------------------------------------------------------- mean correction
def page_value_summary(v_pool: np.ndarray, block_table: np.ndarray, seq_lens: np.ndarray,
                       page_size: int) -> np.ndarray:
    """Mean value row of each referenced physical page, per KV head (the value
    counterpart of page_summary): nu[p, g, :] = mean over the page's valid
    tokens j of V[p, g, :, j] (page-transposed pool), float64 rounded to fp32;
    NaN for pages no sequence references."""
    n_phys, n_kv, d_v, P = v_pool.shape
    nu = np.full((n_phys, n_kv, d_v), np.nan, dtype=np.float32)
    for b in range(block_table.shape[0]):
        for lp in range(n_pages_of(seq_lens[b], P)):
            nv = valid_tokens(seq_lens[b], lp, P)
            phys = int(block_table[b, lp])
            cols = np.asarray(v_pool[phys, :, :, :nv], dtype=np.float64)      # [n_kv][d_v][nv]
            nu[phys] = (cols.sum(axis=2) / nv).astype(np.float32)
    return nu


def mean_corrected_prefill(q, k_pool, v_pool, block_table_row, seq_len, page_size, q_start, tables, counts,
                           n_kv_heads, sm_scale, rows: Optional[Iterable[Tuple[int, int]]] = None):
    """Block-sparse chunked prefill with a mean correction for the skipped blocks.

    Source: the block-sparse prefill brief on the Paperraft page ("a mean
    correction term" beside pattern discovery and thresholding; the term bounds
    the error of the blocks left out).  The formula is not on the pages; the
    reading taken is the plainest one: every causal block of the sequence that
    the query's group table leaves out and that lies wholly at or before the
    query's position stands in for its n_b tokens by their mean key mu_b and
    mean value nu_b, so it adds n_b * exp(z_b) to the softmax normaliser and
    n_b * exp(z_b) * nu_b to the numerator, z_b = sm_scale * q . mu_b:
      o = (sum_{j in table, j <= p} e^{z_j} v_j + sum_b n_b e^{z_b} nu_b)
          / (sum_{j in table, j <= p} e^{z_j} + sum_b n_b e^{z_b})
      lse = log of the denominator.
    The means are taken in float64 over the block's valid tokens (no rounding
    to fp32).  With no skipped block this is block_sparse_prefill; when every
    skipped block's tokens share one key and one value it is exact dense
    causal attention.
    """
    q_len, Hq, d = q.shape
    G = Hq // n_kv_heads
    P = page_size
    d_v = v_pool.shape[2]
    n_seq = n_pages_of(seq_len, P)
    out = np.zeros((q_len, Hq, d_v), dtype=np.float64)
    lse = np.full((q_len, Hq), np.nan, dtype=np.float64)
    if rows is None:
        rows = [(i, h) for i in range(q_len) for h in range(Hq)]
    for (i, h) in rows:
        g = h // G
        pos = q_start + i
        table = set(int(x) for x in tables[g, :int(counts[g])])
        zs, vs = [], []
        for kb in range(n_seq):
            nv = valid_tokens(seq_len, kb, P)
            phys = int(block_table_row[kb])
            K = np.asarray(k_pool[phys, g, :nv, :], dtype=np.float64)
            V = np.asarray(v_pool[phys, g, :, :nv], dtype=np.float64).T
            if kb in table:
                for r in range(nv):
                    if kb * P + r <= pos:
                        zs.append(sm_scale * float(q[i, h] @ K[r]))
                        vs.append(V[r])
            elif kb * P + nv - 1 <= pos:
                zs.append(sm_scale * float(q[i, h] @ K.mean(axis=0)) + math.log(nv))
                vs.append(V.mean(axis=0))
        if not zs:
            out[i, h], lse[i, h] = np.zeros(d_v), -np.inf
            continue
        z = np.array(zs)
        m = z.max()
        e = np.exp(z - m)
        out[i, h] = (e @ np.stack(vs)) / e.sum()
        lse[i, h] = m + math.log(e.sum())
    return out, lse


# ---------------------------------------------------------------- autotuner
def head_page_mass(q, mu, block_table, seq_lens, page_size, n_kv_heads, sm_scale):
    """Estimated attention mass of every (query head, page)  [TS "Motivation":
    the AutoTuner maximises an estimated attention-mass coverage; the estimate
    itself is not given on the pages].

    Reading: a page stands in for its n_p valid tokens by its mean key mu_p,
    so query row (t, h) of sequence b gives page p the log-weight
        est = sm_scale * q[b, t, h] . mu[phys(b, p), g(h)] + ln n_p
    and the row's estimated mass on p is the softmax of est over the
    sequence's pages.  M[b, h, p] = sum over the query tokens t of that mass
    (so sum_p M[b, h, p] = q_tokens).  float64; NaN for pages past the end.
    """
    B, T, Hq, d = q.shape
    G = Hq // n_kv_heads
    max_pages = block_table.shape[1]
    M = np.full((B, Hq, max_pages), np.nan, dtype=np.float64)
    for b in range(B):
        n = n_pages_of(seq_lens[b], page_size)
        if n == 0:
            continue
        counts = np.array([valid_tokens(seq_lens[b], p, page_size) for p in range(n)], dtype=np.float64)
        M[b, :, :n] = 0.0
        for h in range(Hq):
            g = h // G
            mus = np.stack([np.asarray(mu[int(block_table[b, p]), g], dtype=np.float64) for p in range(n)])
            for t in range(T):
                est = sm_scale * (mus @ np.asarray(q[b, t, h], dtype=np.float64)) + np.log(counts)
                e = np.exp(est - est.max())
                M[b, h, :n] += e / e.sum()
    return M


def tier_beta(alpha: int, h: int, budget: int, group: int) -> Optional[int]:
    """Ambient pages a configuration affords  [TS "Configuration": token_budget
    is the total compute-entry budget B, critical_top_count is alpha,
    ambient_head_count is h].  Reading: B counts (page, query head) entries of
    one selection head beyond its forced pages; alpha Critical pages take all
    `group` heads, each Ambient page h of them:  beta = floor((B - alpha*group)/h),
    None (infeasible) when alpha*group > B."""
    rest = budget - alpha * group
    if rest < 0 or h <= 0:
        return None
    return rest // h


def top_heads(masses: np.ndarray, heads: Sequence[int], h: int) -> List[int]:
    """The h heads of `heads` with the largest mass (mass descending, head
    index ascending)."""
    order = sorted(heads, key=lambda x: (-float(masses[x]), x))
    return sorted(order[:max(0, min(h, len(order)))])


def tier_coverage(M, scores, seq_lens, page_size, n_kv_heads, q_tokens, sink_pages, window_pages,
                  budget, alphas, head_counts):
    """Estimated attention-mass coverage of each tier configuration, and the
    configuration the AutoTuner picks  [TS "Motivation": AutoTuner picks the
    tier/head configuration per layer that maximises the estimated coverage].

    For selection head g (a KV head; its query heads are g*G .. g*G+G-1) of
    sequence b, configuration (alpha, h) selects, as the tiered selection does
    with top_k = alpha + beta and critical_k = alpha: the forced pages and the
    first alpha ranked candidates (Critical, all G heads) and the next beta
    (Ambient, the h heads of largest M on that page).  Its coverage is the
    mass M on those (head, page) pairs over q_tokens * G; the layer's coverage
    is the mean over sequences and KV heads.  Returns (cov [n_alpha][n_h],
    NaN where infeasible; beta [n_alpha][n_h], -1 where infeasible; best
    (ia, ih) = the first maximum in row-major grid order, None if none)."""
    B, Hq, _ = M.shape
    G = Hq // n_kv_heads
    na, nh = len(alphas), len(head_counts)
    cov = np.full((na, nh), np.nan, dtype=np.float64)
    beta = np.full((na, nh), -1, dtype=np.int64)
    for ia, a in enumerate(alphas):
        for ih, h in enumerate(head_counts):
            bt = tier_beta(int(a), int(h), budget, G)
            if bt is None:
                continue
            beta[ia, ih] = bt
            total = 0.0
            for b in range(B):
                n = n_pages_of(seq_lens[b], page_size)
                forced = forced_pages(n, sink_pages, window_pages)
                fset = set(forced)
                cand = [p for p in range(n) if p not in fset]
                for g in range(n_kv_heads):
                    heads = list(range(g * G, (g + 1) * G))
                    order = rank_candidates(scores[b, g], cand)
                    a_eff = min(int(a), len(order))
                    b_eff = min(bt, len(order) - a_eff)
                    covered = 0.0
                    for p in forced + order[:a_eff]:
                        covered += sum(M[b, x, p] for x in heads)
                    for p in order[a_eff:a_eff + b_eff]:
                        covered += sum(M[b, x, p] for x in top_heads(M[b, :, p], heads, int(h)))
                    total += covered / (q_tokens * G)
            cov[ia, ih] = total / (B * n_kv_heads)
    best = None
    for ia in range(na):
        for ih in range(nh):
            if np.isnan(cov[ia, ih]):
                continue
            if best is None or cov[ia, ih] > cov[best]:
                best = (ia, ih)
    return cov, beta, best


def ambient_head_mask(M, page_lists, page_counts, critical_counts, n_kv_heads, ambient_heads):
    """Head mask of the Ambient tier  [TS "Motivation": Ambient pages are
    computed with only h heads].  Reading: for every Ambient page p of
    selection head g (list entries past the Critical count), the h heads of g
    with the largest M[b, :, p] (mass descending, index ascending) get their
    bit; other bits are 0.  Returns [B][max_pages][ceil(Hq/32)] uint32 words."""
    B, Hq, max_pages = M.shape
    G = Hq // n_kv_heads
    words = (Hq + 31) // 32
    mask = np.zeros((B, max_pages, words), dtype=np.uint32)
    for b in range(B):
        for g in range(n_kv_heads):
            heads = list(range(g * G, (g + 1) * G))
            cc, c = int(critical_counts[b, g]), int(page_counts[b, g])
            for e in range(cc, c):
                p = int(page_lists[b, g, e])
                for x in top_heads(M[b, :, p], heads, ambient_heads):
                    mask[b, p, x // 32] |= np.uint32(1 << (x % 32))
    return mask

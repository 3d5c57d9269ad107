"""Plain float64 CPU oracle for retrieval-sparse paged decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module:
only the tests, the smoke check in ``__graft_entry__`` and the ``cpu_baseline``
leg of ``bench.py`` may use it.  It shares no code with the HIP library.

What it computes follows these passages (cited by page title and section):

* openGauss DataVec docs, "KV Cache Query-Based Computation Inference
  Acceleration", section *Overall Solution*: each sequence's KV cache is cut
  into initial tokens, a sliding window and offload tokens; the offload part is
  represented block by block by a key representation vector; at each decode
  step the current query is scored against every representation by inner
  product, the top-K "closest" blocks are selected and attention runs over the
  selected blocks joined with the initial and window blocks.
* same page, section *Configuration Parameters*: defaults init 1024, local
  7192, ratio 0.2, block size 128, dense boundary 32K (prompt shorter than the
  boundary: no sparsity).
* rkmt.cn article on ATB KV-cache reuse, section 1.1 (attention as
  softmax(QK^T / sqrt(d_k)) V with one query per autoregressive step) and
  section 2.2 (PageAttention reads K/V through a page table).
* CSDN "KV cache" survey, section *Share--KV cache共享*: query heads of one
  group share one K/V head (MQA/GQA).

Readings where the pages are silent:

* the representation vector of a block is the mean of its 128 keys per KV
  head, and only complete blocks get one;
* "closest" by inner product means the largest inner product;
* the query heads of one KV group are summed into one score per (sequence,
  KV head), and the top-k runs per (sequence, KV head); the page keeps one
  (representation, block index) record per block and leaves open whether
  retrieval runs per KV head or once per sequence, so the other reading is
  offered too (``per_sequence``): the scores of all KV heads are summed, one
  top-k runs per sequence, and every KV head attends the same blocks;
* query head h' belongs to KV head h' // G (contiguous groups);
* init is ceil(init_tokens / 128) blocks; local is every block that meets the
  last ``local_tokens`` positions, and the last (possibly partial) block is
  always local; offload is the complete blocks strictly in between;
* k = ceil(n_off * ppm / 10**6) in exact integers (ppm = ratio * 10**6);
* a prompt with ``prompt_len < dense_boundary`` (or ppm = 10**6) attends to
  every block; ``dense_boundary = 0`` disables the dense switch;
* ties in the score order go to the smaller logical block index; the selected
  blocks are reported in ascending order;
* an empty sequence (L = 0) attends to nothing and its output is zero.

All arithmetic is float64 on the exact values of the bf16 inputs.
Every function here is pinned by a test in ``tests/test_oracle_pins.py``.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK = 128
HEAD_DIM = 128
PPM_ONE = 1_000_000


@dataclass(frozen=True)
class Params:
    """Method parameters, named after the page's environment variables."""

    n_q_heads: int
    n_kv_heads: int
    init_tokens: int = 1024      # VLLM_RETRIEVAL_INIT_TOKENS_NUM
    local_tokens: int = 7192     # VLLM_RETRIEVAL_LOCAL_TOKENS_NUM
    topk_ppm: int = 200_000      # VLLM_RETRIEVAL_TOPK_PERCENT = 0.2
    dense_boundary: int = 32768  # VLLM_RETRIEVAL_DENSE_BOUNDARY = 32K
    block: int = BLOCK
    scale: float = field(default=1.0 / np.sqrt(HEAD_DIM))
    per_sequence: bool = False   # one selection per sequence (all KV heads)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


# ----------------------------------------------------------------------------
# Input decoding and the page layout (the layout is part of the library ABI:
# K page slice [token][dim], V page slice [dim][token], each per (page, head)).
# ----------------------------------------------------------------------------

def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.ascontiguousarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def logical_kv(k_pages: np.ndarray, v_pages: np.ndarray, table_row: np.ndarray,
               L: int, block: int = BLOCK):
    """Gather one sequence's logical K and V from the paged pools.

    k_pages: uint16 [P, Hkv, block, d]   (token-major inside a page slice)
    v_pages: uint16 [P, Hkv, d, block]   (dim-major inside a page slice)
    Returns float64 K, V of shape [Hkv, L, d].  The block table maps logical
    block j to a physical page (ATB page, section 2.2: a page table).
    """
    nb = -(-L // block)
    pages = np.asarray(table_row[:nb], dtype=np.int64)
    hkv, d = k_pages.shape[1], k_pages.shape[3]
    K = k_pages[pages]                        # [nb, Hkv, block, d]
    V = v_pages[pages].transpose(0, 1, 3, 2)  # [nb, Hkv, block, d]
    K = K.transpose(1, 0, 2, 3).reshape(hkv, nb * block, d)[:, :L]
    V = V.transpose(1, 0, 2, 3).reshape(hkv, nb * block, d)[:, :L]
    return bf16_to_f64(K), bf16_to_f64(V)


# ----------------------------------------------------------------------------
# Regions, k and the dense switch (openGauss page, Overall Solution and
# Configuration Parameters).
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Regions:
    nb: int           # blocks holding the L tokens (last one may be partial)
    n_init: int       # init blocks are [0, n_init)
    local_start: int  # local blocks are [max(local_start, n_init), nb)
    n_off: int        # offload blocks are [n_init, n_init + n_off)


def block_regions(L: int, init_tokens: int, local_tokens: int,
                  block: int = BLOCK) -> Regions:
    """Split a sequence of L tokens into init / offload / local blocks."""
    if L <= 0:
        return Regions(0, 0, 0, 0)
    nb = -(-L // block)
    n_init = min(-(-init_tokens // block), nb)
    local_start = min(max(L - local_tokens, 0) // block, nb - 1)
    n_off = max(local_start - n_init, 0)
    return Regions(nb, n_init, local_start, n_off)


def topk_count(n_off: int, ppm: int) -> int:
    """k = ceil(n_off * ppm / 10**6) with exact integer arithmetic."""
    return (n_off * ppm + PPM_ONE - 1) // PPM_ONE


def is_dense(prompt_len: int, dense_boundary: int, ppm: int) -> bool:
    """Dense switch: prompt shorter than the boundary, or ratio 1.0."""
    return prompt_len < dense_boundary or ppm >= PPM_ONE


# ----------------------------------------------------------------------------
# Representations, scores and top-k (Overall Solution).
# ----------------------------------------------------------------------------

def block_reps(K_h: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """Mean key of every complete block of one KV head: [L, d] -> [n, d]."""
    n = K_h.shape[0] // block
    return K_h[: n * block].reshape(n, block, K_h.shape[1]).mean(axis=1)


def ip_scores(q_group: np.ndarray, reps: np.ndarray) -> np.ndarray:
    """Inner-product score of each representation against the group's
    queries, summed over the G query heads: s_j = sum_g q_g . rep_j."""
    return (reps @ q_group.T).sum(axis=1)


def top_k(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the smaller index, returned
    in ascending index order."""
    order = np.lexsort((np.arange(scores.shape[0]), -scores))
    return np.sort(order[:k])


def selection_gap(scores: np.ndarray, k: int) -> float:
    """Relative gap between the k-th and (k+1)-th largest scores; +inf when
    k is 0 or covers every block (the selection cannot be ambiguous)."""
    n = scores.shape[0]
    if k <= 0 or k >= n:
        return float("inf")
    s = np.sort(scores)[::-1]
    a, b = s[k - 1], s[k]
    den = max(abs(a), abs(b))
    return 0.0 if den == 0.0 else float((a - b) / den)


def merged_blocks(reg: Regions, selected_offload: np.ndarray) -> np.ndarray:
    """Logical blocks attended: init, then the selected offload blocks, then
    the local blocks, in ascending order without repeats."""
    init = np.arange(0, reg.n_init)
    local = np.arange(max(reg.local_start, reg.n_init), reg.nb)
    sel = np.asarray(selected_offload, dtype=np.int64)
    return np.concatenate([init, sel, local]).astype(np.int64)


# ----------------------------------------------------------------------------
# Attention (ATB article, section 1.1).
# ----------------------------------------------------------------------------

def attend(q_rows: np.ndarray, K: np.ndarray, V: np.ndarray,
           scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for each query row; max-subtracted softmax.
    q_rows [G, d], K [T, d], V [T, d] -> [G, d].  T = 0 gives zeros."""
    if K.shape[0] == 0:
        return np.zeros((q_rows.shape[0], V.shape[1]))
    z = scale * (q_rows @ K.T)
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ V


# ----------------------------------------------------------------------------
# One decode step for one sequence.
# ----------------------------------------------------------------------------

@dataclass
class HeadResult:
    selected: np.ndarray      # selected offload blocks (logical, ascending)
    merged: np.ndarray        # attended logical blocks (ascending)
    scores: np.ndarray        # scores of offload blocks n_init .. n_init+n_off-1
    k: int
    gap_rel: float
    dense: bool


@dataclass
class StepResult:
    out: np.ndarray           # [Hq, d]
    regions: Regions
    heads: list               # HeadResult per KV head


def decode_step(q: np.ndarray, K: np.ndarray, V: np.ndarray, L: int,
                prompt_len: int, prm: Params,
                reps: np.ndarray | None = None,
                merged_override: list | None = None) -> StepResult:
    """One decode step of one sequence.

    q: [Hq, d] float64 (the current token's queries); K, V: [Hkv, >=L, d]
    float64 logical keys / values (the current token already appended, so L
    counts it).  ``reps`` [Hkv, >= n_complete, d] may be passed in precomputed
    (they are a pure function of K).  ``merged_override`` (list of logical
    block arrays per KV head) replaces the selection, for checking attention
    over a given block set.
    """
    G = prm.group
    reg = block_regions(L, prm.init_tokens, prm.local_tokens, prm.block)
    dense = is_dense(prompt_len, prm.dense_boundary, prm.topk_ppm)
    out = np.zeros((prm.n_q_heads, q.shape[1]))
    heads = []
    lo, hi = reg.n_init, reg.n_init + reg.n_off
    k = reg.n_off if dense else topk_count(reg.n_off, prm.topk_ppm)
    # scores of the offload blocks per KV head (group queries summed)
    scores = []
    for h in range(prm.n_kv_heads):
        qg = q[h * G:(h + 1) * G]
        if reg.n_off > 0:
            r = reps[h, lo:hi] if reps is not None else \
                block_reps(K[h, :L], prm.block)[lo:hi]
            scores.append(ip_scores(qg, r))
        else:
            scores.append(np.zeros(0))
    if prm.per_sequence:  # one score per block: the sum over the KV heads
        total = np.sum(scores, axis=0)
        scores = [total] * prm.n_kv_heads
    for h in range(prm.n_kv_heads):
        qg = q[h * G:(h + 1) * G]
        s = scores[h]
        sel = top_k(s, k) + lo
        merged = merged_blocks(reg, sel)
        if merged_override is not None:
            merged = np.asarray(merged_override[h], dtype=np.int64)
        tok = (merged[:, None] * prm.block + np.arange(prm.block)[None, :])
        tok = tok.reshape(-1)
        tok = tok[tok < L]
        out[h * G:(h + 1) * G] = attend(qg, K[h, tok], V[h, tok], prm.scale)
        heads.append(HeadResult(sel, merged, s, k, selection_gap(s, k), dense))
    return StepResult(out, reg, heads)

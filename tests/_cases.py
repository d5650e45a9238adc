"""Shared small mask cases for the CPU tests (test helper)."""
import numpy as np

from mad_inputs import doc_lengths
from oracle.masks import MaskSpec, topk_keep, uniform_edges


def small_specs(T, seed=0):
    """Every pattern at scaled-down parameters so each shows its structure at size T."""
    docs = tuple(int(x) for x in doc_lengths(seed, T, lo=max(2, T // 16), hi=max(3, T // 2)))
    w = max(2, T // 5)
    out = [
        MaskSpec("FULL", T, T),
        MaskSpec("CAUSAL", T, T),
        MaskSpec("SLIDING_WINDOW", T, T, window=w),
        MaskSpec("FULL_DOCUMENT", T, T, doc_lens=docs),
        MaskSpec("CAUSAL_DOCUMENT", T, T, doc_lens=docs),
        MaskSpec("SLIDING_WINDOW_CAUSAL_DOCUMENT", T, T, window=w, doc_lens=docs),
        MaskSpec("PREFIX_LM", T, T),
        MaskSpec("SHARED_QUESTION", T, T, question=max(1, T // 4), n_answers=3),
        MaskSpec("GLOBAL_SLIDING", T, T, global_len=max(1, T // 8), window=w),
        MaskSpec("CAUSAL_BLOCKWISE", T, T, block=max(1, T // 3)),
        MaskSpec("BLOCK_CAUSAL_DOCUMENT", T, T, block=max(1, T // 7), doc_lens=docs),
        MaskSpec("PREFIX_LM_DOCUMENT", T, T, doc_lens=docs),
        MaskSpec("CAUSAL_BLOCKWISE_LAST", T, T, block=max(1, T // 3)),
        MaskSpec("BLOCK_CAUSAL_DOCUMENT_GLOBAL", T, T, block=max(1, T // 7), doc_lens=docs),
    ]
    return out


def sparse_spec(T, b, n_groups, pct, seed=0, variable_sizes=None):
    from mad_inputs import block_scores
    if variable_sizes is not None:
        edges = np.concatenate([[0], np.cumsum(variable_sizes)]).astype(np.int64)
        pat = "VARIABLE_BLOCK_SPARSE"
    else:
        edges = uniform_edges(T, b)
        pat = "BLOCK_SPARSE"
    n = len(edges) - 1
    keep = topk_keep(block_scores(seed, n_groups, n, n), pct)
    return MaskSpec(pat, T, T, q_edges=edges, k_edges=edges, keep=keep)

"""Oracle part 5: brute-force attention with Python's ``math`` module.

TEST INFRASTRUCTURE (see ``oracle/__init__.py``).

The direct definition, one scalar at a time, for tiny inputs (a handful of
requests, keys and dims).  It walks the page table token by token, decides
visibility key by key and sums exponentials in a plain loop; it exists to pin
``oracle.attention`` with code that shares nothing with it but the
definitions on the pages.
"""

from __future__ import annotations

import math


def attention(q, k_pages, v_pages, *, qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
              page_size: int, group: int, causal: bool, sm_scale: float):
    """Nested-list attention.

    q[row][head][d]; k_pages[page][slot][kv_head][d] (NHD tuple form) and the
    same for v_pages.  Returns (o[row][head][d], lse[row][head]) with lse in
    base 2 (log2 of the sum of exp of the scaled logits).

    Row i of request b (local index) sees key j when j < K_b and, if causal,
    j <= K_b - Q_b + i: Deep Dive - FlashInfer, "Causality uses logical
    positions, not page numbers".  Key j of request b is slot j % P of page
    kv_indices[kv_indptr[b] + j // P].  Query head h reads kv head h // group.
    """
    out_o = [[None for _ in row] for row in q]
    out_l = [[None for _ in row] for row in q]
    n_req = len(kv_last_page_len)
    for b in range(n_req):
        n_pages = kv_indptr[b + 1] - kv_indptr[b]
        k_len = page_size * (n_pages - 1) + kv_last_page_len[b]
        q_len = qo_indptr[b + 1] - qo_indptr[b]
        for i in range(q_len):
            row = qo_indptr[b] + i
            for h in range(len(q[row])):
                kvh = h // group
                scores = []
                vals = []
                for j in range(k_len):
                    if causal and j > k_len - q_len + i:
                        continue
                    page = kv_indices[kv_indptr[b] + j // page_size]
                    slot = j % page_size
                    kvec = k_pages[page][slot][kvh]
                    dot = 0.0
                    for d in range(len(kvec)):
                        dot += q[row][h][d] * kvec[d]
                    scores.append(sm_scale * dot)
                    vals.append(v_pages[page][slot][kvh])
                dim_v = len(v_pages[0][0][0])
                if not scores:
                    out_o[row][h] = [0.0] * dim_v
                    out_l[row][h] = -math.inf
                    continue
                top = max(scores)
                weights = [math.exp(s - top) for s in scores]
                total = 0.0
                for w in weights:
                    total += w
                vec = []
                for d in range(dim_v):
                    acc = 0.0
                    for w, v in zip(weights, vals):
                        acc += w * v[d]
                    vec.append(acc / total)
                out_o[row][h] = vec
                out_l[row][h] = (top + math.log(total)) / math.log(2.0)
    return out_o, out_l

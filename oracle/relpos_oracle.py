"""Plain float64 CPU oracle for attention with a decomposed relative-position bias.

TEST INFRASTRUCTURE ONLY.  This module is the checker, not the product: only the
test suite, the package's smoke check and the CPU-baseline leg of the benchmark
may import it.  It shares no code, tables or helpers with the HIP library, and it
imports nothing from that package.

What it computes (source: the prhub summary page of vllm-project/vllm PR #55629,
"DeepEncoder relative-position attention fused into a Triton kernel", section
关键源码片段 (key source snippet), the ``RelPosAttention.forward`` branch):

* q, k, v come from ``qkv.reshape(3, B*heads, H*W, -1)``, so token ``i`` of an
  ``H x W`` grid is the row-major position ``i = qh*W + qw``.
* ``rel_h, rel_w = add_decomposed_rel_pos(q, rel_pos_h, rel_pos_w, (H, W), (H, W))``
  is called on the *unscaled* q.  The page shows only the call, not its body.
  The reading taken here (the formula the task states):
  ``rel_h[i, kh] = sum_c q[i, c] * rel_pos_h[qh - kh + H - 1, c]`` and
  ``rel_w[i, kw] = sum_c q[i, c] * rel_pos_w[qw - kw + W - 1, c]``.
* The unfused fallback adds the two into one dense ``[B, heads, HW, HW]`` bias,
  ``bias[i, j] = rel_h[i, j // W] + rel_w[i, j % W]``, and calls scaled
  dot-product attention with it as an additive mask:
  ``out = softmax_j(scale * q . k_j + bias[i, j]) @ v``.

Everything is float64, written from that definition; nothing is blocked, fused or
reordered beyond it.  The row softmax subtracts the row maximum first, which does
not change its value.
"""

import numpy as np

__all__ = [
    "token_coords",
    "rel_tables",
    "dense_bias",
    "softmax_rows",
    "attention_dense",
    "relpos_attention",
    "relpos_attention_rows",
]


def token_coords(H, W):
    """Grid coordinates of the row-major tokens: ``(i // W, i % W)`` for i < H*W.

    Source: PR #55629 page, key source snippet: q/k/v are reshaped from a
    ``[B, H, W, C]`` activation to ``H*W`` tokens.
    """
    idx = np.arange(H * W)
    return idx // W, idx % W


def rel_tables(q, rel_pos_h, rel_pos_w, H, W):
    """Per-query relative-position logits along each grid axis.

    q: ``[..., H*W, D]``; rel_pos_h: ``[2H-1, D]``; rel_pos_w: ``[2W-1, D]``.
    Returns ``rel_h [..., H*W, H]`` and ``rel_w [..., H*W, W]``, float64.

    Source: PR #55629 page, key source snippet, the ``add_decomposed_rel_pos``
    call on the unscaled q; table index ``qh - kh + H - 1`` (resp. ``qw - kw + W - 1``).
    Step 1: dot each query with every table row (a matmul).
    Step 2: for each (query, key row/column) pick the row at the relative offset.
    """
    q = np.asarray(q, dtype=np.float64)
    th = np.asarray(rel_pos_h, dtype=np.float64)
    tw = np.asarray(rel_pos_w, dtype=np.float64)
    if th.shape[0] != 2 * H - 1 or tw.shape[0] != 2 * W - 1:
        raise ValueError("table lengths must be 2H-1 and 2W-1")
    qh, qw = token_coords(H, W)
    dots_h = q @ th.T  # [..., N, 2H-1]
    dots_w = q @ tw.T  # [..., N, 2W-1]
    kh = np.arange(H)
    kw = np.arange(W)
    idx_h = qh[:, None] - kh[None, :] + (H - 1)  # [N, H]
    idx_w = qw[:, None] - kw[None, :] + (W - 1)  # [N, W]
    rows = np.arange(H * W)[:, None]
    rel_h = dots_h[..., rows, idx_h]
    rel_w = dots_w[..., rows, idx_w]
    return rel_h, rel_w


def dense_bias(rel_h_rows, rel_w_rows, H, W):
    """The dense additive bias for the given query rows.

    rel_h_rows: ``[R, H]``, rel_w_rows: ``[R, W]`` -> ``[R, H*W]`` with
    ``bias[r, j] = rel_h_rows[r, j // W] + rel_w_rows[r, j % W]``.

    Source: PR #55629 page, key source snippet, the SDPA fallback that forms
    ``(rel_h + rel_w).view(B, heads, HW, HW)`` from the broadcast shapes
    ``[.., HW, H, 1]`` and ``[.., HW, 1, W]``.
    """
    kh, kw = token_coords(H, W)
    return rel_h_rows[:, kh] + rel_w_rows[:, kw]


def softmax_rows(S):
    """Row softmax of a float64 matrix (subtracting the row max first)."""
    S = np.asarray(S, dtype=np.float64)
    m = S.max(axis=-1, keepdims=True)
    e = np.exp(S - m)
    return e / e.sum(axis=-1, keepdims=True)


def attention_dense(q, k, v, bias, scale):
    """``softmax(scale * q @ k.T + bias) @ v`` for one head; returns (out, P).

    Source: PR #55629 page, key source snippet: ``scaled_dot_product_attention(q,
    k, v, attn_mask=attn_bias)`` with an additive float mask.  All keys take part:
    no causal mask, no dropout.
    """
    S = scale * (q @ k.T) + bias
    P = softmax_rows(S)
    return P @ v, P


def relpos_attention_rows(q, k, v, rel_pos_h, rel_pos_w, H, W, scale, rows):
    """Oracle output for selected query rows of ONE (batch, head).

    q, k, v: ``[H*W, D]``.  rows: 1-D integer array of query indices.
    Returns ``out [len(rows), D]`` float64.  Rows are independent under the
    definition, so this is the full definition restricted to those rows.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.int64)
    rel_h, rel_w = rel_tables(q, rel_pos_h, rel_pos_w, H, W)
    bias = dense_bias(rel_h[rows], rel_w[rows], H, W)
    out, _ = attention_dense(q[rows], k, v, bias, scale)
    return out


def relpos_attention(q, k, v, rel_pos_h, rel_pos_w, H, W, scale,
                     return_probs=False, row_chunk=1024):
    """Full oracle over ``[B, heads, H*W, D]`` inputs.

    Returns ``(out, rel_h, rel_w)`` (and ``P [B, heads, N, N]`` when
    ``return_probs``; only for tiny shapes).  The dense bias is formed per
    (batch, head) in chunks of query rows to bound host memory.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, nh, N, D = q.shape
    if N != H * W:
        raise ValueError("token count must equal H*W")
    rel_h, rel_w = rel_tables(q, rel_pos_h, rel_pos_w, H, W)
    out = np.empty((B, nh, N, v.shape[-1]), dtype=np.float64)
    probs = np.empty((B, nh, N, N), dtype=np.float64) if return_probs else None
    for b in range(B):
        for h in range(nh):
            for r0 in range(0, N, row_chunk):
                r1 = min(N, r0 + row_chunk)
                bias = dense_bias(rel_h[b, h, r0:r1], rel_w[b, h, r0:r1], H, W)
                o, P = attention_dense(q[b, h, r0:r1], k[b, h], v[b, h], bias, scale)
                out[b, h, r0:r1] = o
                if return_probs:
                    probs[b, h, r0:r1] = P
    if return_probs:
        return out, rel_h, rel_w, probs
    return out, rel_h, rel_w

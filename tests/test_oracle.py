"""Pins of the float64 oracle against facts it cannot produce about itself.

Each pin is something other than the oracle's own formula: hand-derived closed
forms (tests/golden), a library routine (torch's scaled_dot_product_attention in
float64 on the CPU), an explicit loop over grid coordinates written independently
of the vectorised gather, invariants of softmax, and degenerate cases with known
results.  A mutation test shows that plausible slips (flipped index, swapped axes,
column-major tokens, scaled q in the bias, missing scale) fail the pins.
"""

import glob
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import relpos_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cases():
    return [json.load(open(p)) for p in sorted(glob.glob(os.path.join(GOLDEN, "*.json")))]


def _as_bhnd(x):
    return np.asarray(x, dtype=np.float64)[None, None]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    H, W = case["H"], case["W"]
    out, rel_h, rel_w = O.relpos_attention(
        _as_bhnd(case["q"]), _as_bhnd(case["k"]), _as_bhnd(case["v"]),
        np.asarray(case["rel_pos_h"]), np.asarray(case["rel_pos_w"]), H, W, case["scale"])
    np.testing.assert_allclose(rel_h[0, 0], case["expected_rel_h"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(rel_w[0, 0], case["expected_rel_w"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[0, 0], case["expected_out"], rtol=0, atol=1e-13)


def _brute_rel(q, th, tw, H, W):
    """Explicit loops over (qh, qw, kh, kw): an independent statement of the tables."""
    N, D = q.shape
    rel_h = np.zeros((N, H))
    rel_w = np.zeros((N, W))
    for qh in range(H):
        for qw in range(W):
            i = qh * W + qw
            for kh in range(H):
                acc = 0.0
                for c in range(D):
                    acc += q[i, c] * th[qh - kh + H - 1, c]
                rel_h[i, kh] = acc
            for kw in range(W):
                acc = 0.0
                for c in range(D):
                    acc += q[i, c] * tw[qw - kw + W - 1, c]
                rel_w[i, kw] = acc
    return rel_h, rel_w


def _brute_attention(q, k, v, rel_h, rel_w, H, W, scale):
    """Loop form: per query, scores over keys (kh, kw), softmax via math.exp."""
    N, Dv = v.shape
    out = np.zeros((N, Dv))
    for i in range(N):
        s = []
        for kh in range(H):
            for kw in range(W):
                j = kh * W + kw
                s.append(scale * float(np.dot(q[i], k[j])) + rel_h[i, kh] + rel_w[i, kw])
        mx = max(s)
        e = [math.exp(x - mx) for x in s]
        tot = sum(e)
        for j in range(N):
            out[i] += (e[j] / tot) * v[j]
    return out


@pytest.mark.parametrize("H,W,D", [(1, 1, 1), (1, 3, 4), (2, 3, 4), (3, 2, 1), (5, 2, 4), (3, 5, 64), (2, 2, 64)])
def test_vectorised_matches_loops(H, W, D):
    rng = np.random.default_rng(1000 + 31 * H + 7 * W + D)
    N = H * W
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    th = rng.standard_normal((2 * H - 1, D)) * 0.3
    tw = rng.standard_normal((2 * W - 1, D)) * 0.3
    rh_ref, rw_ref = _brute_rel(q, th, tw, H, W)
    out, rh, rw = O.relpos_attention(q[None, None], k[None, None], v[None, None], th, tw, H, W, 0.37)
    np.testing.assert_allclose(rh[0, 0], rh_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(rw[0, 0], rw_ref, rtol=0, atol=1e-12)
    ref = _brute_attention(q, k, v, rh_ref, rw_ref, H, W, 0.37)
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-12)


def test_matches_torch_sdpa_with_dense_mask():
    """Library routine: torch SDPA (float64, CPU) with the loop-built dense bias."""
    H, W, D = 3, 4, 8
    rng = np.random.default_rng(7)
    N = H * W
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    th = rng.standard_normal((2 * H - 1, D)) * 0.5
    tw = rng.standard_normal((2 * W - 1, D)) * 0.5
    rh, rw = _brute_rel(q, th, tw, H, W)
    bias = np.zeros((N, N))
    for i in range(N):
        for j in range(N):
            bias[i, j] = rh[i, j // W] + rw[i, j % W]
    t = lambda a: torch.from_numpy(a)[None, None]
    # SDPA's default scale is 1/sqrt(D); pass it explicitly to match the oracle's scale.
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(q), t(k), t(v), attn_mask=t(bias), scale=1.0 / math.sqrt(D))[0, 0].numpy()
    out, _, _ = O.relpos_attention(q[None, None], k[None, None], v[None, None], th, tw, H, W,
                                   1.0 / math.sqrt(D))
    np.testing.assert_allclose(out[0, 0], ref, rtol=0, atol=1e-12)


def test_zero_tables_is_plain_attention():
    H, W, D = 4, 5, 16
    rng = np.random.default_rng(3)
    N = H * W
    q, k, v = (rng.standard_normal((2, 3, N, D)) for _ in range(3))
    out, rh, rw = O.relpos_attention(q, k, v, np.zeros((2 * H - 1, D)), np.zeros((2 * W - 1, D)), H, W, 0.125)
    assert not rh.any() and not rw.any()
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=0.125).numpy()
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_per_query_constant_shift_invariance():
    H, W, D = 4, 6, 8
    rng = np.random.default_rng(11)
    N = H * W
    q, k, v = (rng.standard_normal((N, D)) for _ in range(3))
    th = rng.standard_normal((2 * H - 1, D))
    tw = rng.standard_normal((2 * W - 1, D))
    rh, rw = O.rel_tables(q, th, tw, H, W)
    c = rng.standard_normal((N, 1)) * 5.0
    base, _ = O.attention_dense(q, k, v, O.dense_bias(rh, rw, H, W), 0.3)
    sh_h, _ = O.attention_dense(q, k, v, O.dense_bias(rh + c, rw, H, W), 0.3)
    sh_w, _ = O.attention_dense(q, k, v, O.dense_bias(rh, rw - c, H, W), 0.3)
    np.testing.assert_allclose(sh_h, base, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sh_w, base, rtol=0, atol=1e-12)


def test_ones_v_gives_ones_and_rows_sum_to_one():
    H, W, D = 3, 7, 16
    rng = np.random.default_rng(5)
    N = H * W
    q = rng.standard_normal((1, 2, N, D)) * 3
    k = rng.standard_normal((1, 2, N, D)) * 3
    v = np.ones((1, 2, N, D))
    th = rng.standard_normal((2 * H - 1, D))
    tw = rng.standard_normal((2 * W - 1, D))
    out, _, _, P = O.relpos_attention(q, k, v, th, tw, H, W, 0.125, return_probs=True)
    np.testing.assert_allclose(out, 1.0, rtol=0, atol=1e-14)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-14)
    assert (P > 0).all()


def test_zero_q_gives_mean_of_v():
    H, W, D = 3, 5, 8
    rng = np.random.default_rng(9)
    N = H * W
    q = np.zeros((1, 1, N, D))
    k = rng.standard_normal((1, 1, N, D))
    v = rng.standard_normal((1, 1, N, D))
    th = rng.standard_normal((2 * H - 1, D))
    tw = rng.standard_normal((2 * W - 1, D))
    out, rh, rw = O.relpos_attention(q, k, v, th, tw, H, W, 0.125)
    assert not rh.any() and not rw.any()
    np.testing.assert_allclose(out[0, 0], np.broadcast_to(v[0, 0].mean(0), (N, D)), rtol=0, atol=1e-14)


def test_single_token_returns_v():
    rng = np.random.default_rng(2)
    q, k, v = (rng.standard_normal((2, 3, 1, 64)) for _ in range(3))
    th = rng.standard_normal((1, 64))
    tw = rng.standard_normal((1, 64))
    out, _, _ = O.relpos_attention(q, k, v, th, tw, 1, 1, 0.125)
    np.testing.assert_allclose(out, v, rtol=0, atol=1e-15)


def test_rows_variant_matches_full():
    H, W, D = 5, 6, 16
    rng = np.random.default_rng(4)
    N = H * W
    q, k, v = (rng.standard_normal((1, 1, N, D)) for _ in range(3))
    th = rng.standard_normal((2 * H - 1, D)) * 0.2
    tw = rng.standard_normal((2 * W - 1, D)) * 0.2
    full, _, _ = O.relpos_attention(q, k, v, th, tw, H, W, 0.125, row_chunk=7)
    rows = np.array([0, 3, 17, 29, 11])
    part = O.relpos_attention_rows(q[0, 0], k[0, 0], v[0, 0], th, tw, H, W, 0.125, rows)
    np.testing.assert_allclose(part, full[0, 0, rows], rtol=0, atol=1e-14)


def test_large_logits_stay_finite():
    """Online-softmax stress (q, k ~ 4 N(0,1)): the row-max shift keeps exp finite."""
    H, W, D = 4, 4, 64
    rng = np.random.default_rng(6)
    N = H * W
    q = rng.standard_normal((1, 1, N, D)) * 40
    k = rng.standard_normal((1, 1, N, D)) * 40
    v = rng.uniform(-1, 1, (1, 1, N, D))
    out, _, _ = O.relpos_attention(q, k, v, np.zeros((2 * H - 1, D)), np.zeros((2 * W - 1, D)), H, W, 0.125)
    assert np.isfinite(out).all()
    # Logits this large make each row's softmax one-hot at its argmax.
    S = 0.125 * q[0, 0] @ k[0, 0].T
    np.testing.assert_allclose(out[0, 0], v[0, 0][S.argmax(1)], rtol=0, atol=1e-5)


# --- mutation check: plausible slips in the tables must fail a pin ------------

def _mut_flipped(q, th, tw, H, W):
    qh, qw = O.token_coords(H, W)
    rh = (q @ th.T)[..., np.arange(H * W)[:, None], (np.arange(H)[None, :] - qh[:, None] + H - 1)]
    rw = (q @ tw.T)[..., np.arange(H * W)[:, None], (np.arange(W)[None, :] - qw[:, None] + W - 1)]
    return rh, rw


_REL_TABLES = O.rel_tables  # the unmutated function, captured before any patching


def _mut_scaled_q(q, th, tw, H, W):
    return _REL_TABLES(q * 0.125, th, tw, H, W)


def _mut_colmajor(q, th, tw, H, W):
    idx = np.arange(H * W)
    qh, qw = idx % H, idx // H
    rh = (q @ th.T)[..., idx[:, None], qh[:, None] - np.arange(H)[None, :] + H - 1]
    rw = (q @ tw.T)[..., idx[:, None], qw[:, None] - np.arange(W)[None, :] + W - 1]
    return rh, rw


def _mut_swapped_axes(q, th, tw, H, W):
    qh, qw = O.token_coords(H, W)
    # uses the height table for the width axis when it is long enough, else clips
    th2 = np.concatenate([th, np.zeros((max(0, 2 * W - 1 - th.shape[0]), th.shape[1]))])[: 2 * W - 1]
    tw2 = np.concatenate([tw, np.zeros((max(0, 2 * H - 1 - tw.shape[0]), tw.shape[1]))])[: 2 * H - 1]
    return _REL_TABLES(q, tw2, th2, H, W)


@pytest.mark.parametrize("mut", [_mut_flipped, _mut_scaled_q, _mut_colmajor, _mut_swapped_axes])
def test_pins_catch_plausible_mistakes(mut, monkeypatch):
    """Planting a slip in the oracle (on the CPU) must break at least one hand case."""
    monkeypatch.setattr(O, "rel_tables", mut)
    failed = 0
    for case in _cases():
        out, _, _ = O.relpos_attention(
            _as_bhnd(case["q"]), _as_bhnd(case["k"]), _as_bhnd(case["v"]),
            np.asarray(case["rel_pos_h"]), np.asarray(case["rel_pos_w"]), case["H"], case["W"], case["scale"])
        if not np.allclose(out[0, 0], case["expected_out"], rtol=0, atol=1e-9):
            failed += 1
    assert failed >= 1


def test_pins_catch_missing_scale(monkeypatch):
    orig = O.attention_dense
    monkeypatch.setattr(O, "attention_dense", lambda q, k, v, b, s: orig(q, k, v, b, 1.0))
    case = json.load(open(os.path.join(GOLDEN, "scale_on_qk_1x2.json")))
    out, _, _ = O.relpos_attention(_as_bhnd(case["q"]), _as_bhnd(case["k"]), _as_bhnd(case["v"]),
                                   np.asarray(case["rel_pos_h"]), np.asarray(case["rel_pos_w"]),
                                   case["H"], case["W"], case["scale"])
    assert not np.allclose(out[0, 0], case["expected_out"], atol=1e-6)

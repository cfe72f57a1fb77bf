"""GPU parity of the router on exact ties: moe_topk against the oracle's
routing on rows built to tie.

The rule (vLLM docs page "vllm.model_executor.layers.fused_moe.layer",
FusedMoE.select_experts, read plainly): the selected ids come in descending
key order and equal keys go to the lower expert index, at every level (the
experts, and the groups of grouped top-k).  -0 and +0 are equal values, so
they tie too.

Rows: all-zero rows with random zero signs, -0/+0 pairs, values drawn from a
small set (many equal keys), the top key repeated across the K boundary,
groups with identical contents (every group tied), and two groups tied
across the topk_group boundary.  Softmax keys are the fp32 logits
themselves, equal on both sides.  Sigmoid keys sigmoid(l) + b are fp32 on
the GPU and fp64 in the oracle, so those rows use logits and biases from
small sets and keep only rows where every comparison of distinct
(logit, bias) pairs (and of distinct group contents) has a margin of at
least 1e-5: then both precisions decide alike, and every tie is exact by
construction.

Bars: ids bit-exact; weights within 2e-6 relative (fp32 against fp64).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from mixture_experts_layer_14_amd import binding as B
from oracle import oracle as O

WEIGHT_RTOL = 2e-6
MARGIN = 1e-5

# name: E, K, scoring, G, TG, bias ("none" | "zero" | "lattice"), renormalize, rsf
CASES = {
    "softmax_e8": (8, 2, O.SOFTMAX, 0, 0, "none", True, 1.0),
    "softmax_e8_no_renorm": (8, 2, O.SOFTMAX, 0, 0, "none", False, 1.0),
    "softmax_e128": (128, 8, O.SOFTMAX, 0, 0, "none", True, 1.0),
    "softmax_e256_grouped": (256, 8, O.SOFTMAX, 8, 4, "none", True, 1.0),
    "sigmoid_e256_grouped_bias": (256, 8, O.SIGMOID, 8, 4, "lattice", True, 2.5),
    "sigmoid_e256_grouped_zero_bias": (256, 8, O.SIGMOID, 8, 4, "zero", True, 2.5),
    "sigmoid_e16_bias": (16, 4, O.SIGMOID, 0, 0, "lattice", False, 1.0),
    "sigmoid_e8_grouped_no_bias": (8, 2, O.SIGMOID, 4, 2, "none", True, 1.0),
    # group sizes 64 (a whole wave), 8 over two lanes' slots, 16 with a part
    # filled second slot, and 24 (not a power of two: one reduction a group)
    "sigmoid_e256_g4_bias": (256, 8, O.SIGMOID, 4, 2, "lattice", True, 2.5),
    "softmax_e128_g16": (128, 8, O.SOFTMAX, 16, 4, "none", True, 1.0),
    "softmax_e96_g6": (96, 4, O.SOFTMAX, 6, 2, "none", True, 1.0),
    "sigmoid_e72_g3_bias": (72, 4, O.SIGMOID, 3, 2, "lattice", True, 1.0),
    # the largest routing shapes: 8 experts a lane (E > 256), K = 32, 64
    # groups (of 8, and of 5: one reduction per group), and E = 130 (runs
    # of 4 that end inside a lane's run: element loads)
    "softmax_e512_k32": (512, 32, O.SOFTMAX, 0, 0, "none", True, 1.0),
    "sigmoid_e384_g12_bias": (384, 8, O.SIGMOID, 12, 4, "lattice", True, 2.5),
    "softmax_e512_g64": (512, 8, O.SOFTMAX, 64, 4, "none", True, 1.0),
    "sigmoid_e320_g64_bias": (320, 16, O.SIGMOID, 64, 8, "lattice", False, 1.0),
    "softmax_e130_k6": (130, 6, O.SOFTMAX, 0, 0, "none", False, 1.0),
}

ROWS_PER_KIND = 48


def _bias(kind, E, G, rng):
    if kind == "none":
        return None
    if kind == "zero":
        return np.zeros(E, np.float32)
    # multiples of 1/64 in [-3/64, 3/64], periodic over the groups so that
    # groups with the same logits have the same keys
    per = E // G if G > 1 else E
    pat = rng.integers(-3, 4, per).astype(np.float32) / 64.0
    return np.tile(pat, E // per).astype(np.float32)


def _signed_zeros(rng, n):
    return np.where(rng.random(n) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)


def _candidate_rows(rng, E, K, G, TG, scoring):
    """Rows of each tie kind (more than needed; the sigmoid rows are
    filtered afterwards)."""
    small = np.array([-1.5, -0.5, 0.25, 1.0, 2.0], np.float32)
    rows = []
    for _ in range(ROWS_PER_KIND):
        # all zero, random signs
        rows.append(_signed_zeros(rng, E))
        # -0 / +0 pair above a negative floor, in either order
        r = (-1.0 - rng.integers(0, 16, E) / 16.0).astype(np.float32)
        i, j = rng.choice(E, 2, replace=False)
        r[i], r[j] = np.float32(-0.0), np.float32(0.0)
        rows.append(r.astype(np.float32))
        # values from a small set (softmax: zeros of either sign among them)
        r = rng.choice(small, E).astype(np.float32)
        if scoring == O.SOFTMAX:
            z = rng.random(E) < 0.3
            r[z] = _signed_zeros(rng, int(z.sum()))
        rows.append(r)
        # the largest value repeated K+1 times: the K-th and (K+1)-th keys tie
        r = (-2.0 + rng.integers(0, 16, E) / 16.0).astype(np.float32)
        top = rng.choice(E, min(K + 1, E), replace=False)
        r[top] = np.float32(1.0)
        rows.append(r)
        if G > 1:
            per = E // G
            # every group holds the same values: all groups tie
            pat = rng.choice(small, per).astype(np.float32)
            rows.append(np.tile(pat, G).astype(np.float32))
            # TG-1 clear winners, then two groups tied for the last place
            base = rng.choice(np.array([-1.5, -0.5], np.float32), E).astype(np.float32)
            order = rng.permutation(G)
            for g in order[: TG - 1]:
                base[g * per:(g + 1) * per] = np.float32(2.0)
            tie_pat = rng.choice(small[:3], per).astype(np.float32)
            for g in order[TG - 1: TG + 1]:
                base[g * per:(g + 1) * per] = tie_pat
            rows.append(base)
    return np.stack(rows).astype(np.float32)


def _robust_sigmoid(row, bias, K, G, TG):
    """Every comparison of distinct (logit, bias) pairs, and of groups with
    distinct top contents, differs by at least MARGIN in float64."""
    E = row.size
    b = np.zeros(E) if bias is None else bias.astype(np.float64)
    key = 1.0 / (1.0 + np.exp(-row.astype(np.float64))) + b
    pair = np.stack([row.astype(np.float64), b], 1)
    same = (pair[:, None, 0] == pair[None, :, 0]) & (pair[:, None, 1] == pair[None, :, 1])
    d = np.abs(key[:, None] - key[None, :])
    if np.any((~same) & (d < MARGIN)):
        return False
    if G > 1:
        per = E // G
        top = 2 if (bias is not None and per >= 2) else 1
        gs, content = [], []
        for g in range(G):
            idx = np.arange(g * per, (g + 1) * per)
            o = idx[np.argsort(-key[idx], kind="stable")][:top]
            gs.append(key[o].sum())
            content.append(tuple(sorted(map(tuple, pair[o]))))
        for i in range(G):
            for j in range(i + 1, G):
                if content[i] != content[j] and abs(gs[i] - gs[j]) < MARGIN:
                    return False
    return True


@pytest.mark.gpu
@pytest.mark.parametrize("name", sorted(CASES))
def test_topk_exact_ties_match_oracle(name):
    E, K, scoring, G, TG, bias_kind, renorm, rsf = CASES[name]
    print("case", name, flush=True)
    rng = np.random.default_rng(sum(map(ord, name)))
    bias = _bias(bias_kind, E, G, rng)
    logits = _candidate_rows(rng, E, K, G, TG, scoring)
    if scoring == O.SIGMOID:
        keep = [i for i in range(logits.shape[0]) if _robust_sigmoid(logits[i], bias, K, G, TG)]
        logits = np.ascontiguousarray(logits[keep])
    T = logits.shape[0]
    assert T >= 2 * ROWS_PER_KIND, "too few usable tie rows (%d)" % T
    ref_ids, ref_w = O.route(logits, K, bias=bias, scoring=scoring, renormalize=renorm,
                             n_group=G, topk_group=TG, routed_scaling_factor=rsf)
    p = B.make_params(num_tokens=T, num_experts=E, top_k=K, hidden_size=64,
                      intermediate_size=64, scoring_func=scoring, renormalize=renorm,
                      num_expert_group=G, topk_group=TG, routed_scaling_factor=rsf)
    dl = torch.from_numpy(logits).cuda()
    db = None if bias is None else torch.from_numpy(bias).cuda()
    ids = torch.full((T, K), -1, dtype=torch.int32, device="cuda")
    w = torch.empty(T, K, dtype=torch.float32, device="cuda")
    B.moe_topk(p, dl, db, ids, w)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    bad = np.nonzero(~np.all(got == ref_ids, axis=1))[0]
    assert bad.size == 0, "ids differ on %d rows, first row %d: gpu %s oracle %s (logits %s)" % (
        bad.size, bad[0], got[bad[0]].tolist(), ref_ids[bad[0]].tolist(), logits[bad[0]].tolist())
    gw = w.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(gw - ref_w) / np.maximum(np.abs(ref_w), 1e-30)) <= WEIGHT_RTOL


def test_tie_rows_really_tie():
    """The generated rows hold exact ties among the selected keys (a check of
    the inputs, on the CPU side of the test module)."""
    for name, (E, K, scoring, G, TG, bias_kind, renorm, rsf) in CASES.items():
        rng = np.random.default_rng(sum(map(ord, name)))
        bias = _bias(bias_kind, E, G, rng)
        logits = _candidate_rows(rng, E, K, G, TG, scoring)
        key = logits.astype(np.float64)
        if scoring == O.SIGMOID:
            key = 1.0 / (1.0 + np.exp(-key)) + (0 if bias is None else bias.astype(np.float64))
        top = -np.sort(-key, axis=1)[:, : K + 1]
        tied = np.any(top[:, 1:] == top[:, :-1], axis=1)
        assert tied.mean() >= 0.25, (name, tied.mean())
        if scoring == O.SOFTMAX:
            assert np.any(np.signbit(logits) & (logits == 0)), name

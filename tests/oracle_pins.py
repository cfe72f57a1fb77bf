"""Pins of the CPU oracle: checks against what the pages and the mathematics fix.

Each ``check_*`` takes an optional oracle library (``lib_``) so the planted-
mistake tests can run the same checks against deliberately broken builds of
the oracle and show that every planted mistake fails at least one check.

What pins what (no check re-types the oracle's own code; each compares with
a brute force, a closed form, an invariant, or a library routine):

* number formats  -> torch's bfloat16 / float8_e4m3fn conversions;
* fp8 group quantisation -> torch float32 arithmetic + torch's e4m3 encoder,
  plus the round-trip error bound of a 3-bit mantissa;
* routing -> brute-force search over all expert (and group) subsets, torch
  softmax/sigmoid/topk, the tie rule;
* permutation -> numpy's stable argsort;
* the layer -> the dense SwiGLU MLP (one expert, top-1) written with torch
  library routines, identical-experts and linearity invariants, token-order
  invariance, a brute-force combine of per-expert dense MLPs, the shared-
  expert difference, and an fp8 layer rebuilt from torch's e4m3 encoder;
* router gate logits -> torch's float64 matmul and one-hot gate rows;
* activation variants -> closed forms of the clipped SwiGLU on single
  values, an inactive clamp (bitwise no-op), torch's dense MLP with the
  alpha slope, the clamp or the non-gated form, and for the routing weight
  on the input a brute force plus the w^2 law of the bilinear regime.

Sources: vLLM docs page "vllm.model_executor.layers.fused_moe.layer"
(FusedMoE.select_experts; w13 = [w1 (gate); w3 (up)] per _load_w13); SGLang
page "srt/models/deepseek_v2.py" (DeepseekV2MLP gate_up -> SiluAndMul ->
down; DeepseekV2MoE shared-expert add; per-token-group-128 fp8 quantisation).
"""
from __future__ import annotations

import itertools

import numpy as np
import torch
import torch.nn.functional as F

from oracle import oracle as O

# ---------------------------------------------------------------------------
# helpers (torch/numpy library routines only)
# ---------------------------------------------------------------------------


def _bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _bits_to_f64(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).to(torch.float64)


def _e4m3_torch_decode(codes: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).to(torch.float64)


def _e4m3_torch_encode(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def dense_swiglu(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor) -> torch.Tensor:
    """Textbook gated MLP down(silu(gate x) * up x), gate = first half of w13."""
    I = w2.shape[1]
    return (F.silu(x @ w13[:I].T) * (x @ w13[I:].T)) @ w2.T


def brute_route(row, K, *, bias=None, scoring=O.SOFTMAX, renormalize=True,
                n_group=0, topk_group=0, rsf=1.0):
    """Routing of one row by exhaustive search over subsets."""
    l = torch.tensor(np.asarray(row, np.float64))
    E = l.numel()
    if scoring == O.SOFTMAX:
        score = torch.softmax(l, 0)
        key = l
    else:
        score = torch.sigmoid(l)
        key = score + (0 if bias is None else torch.tensor(np.asarray(bias, np.float64)))
    eligible = list(range(E))
    if n_group > 1:
        per = E // n_group
        groups = key.reshape(n_group, per)
        if bias is not None and per >= 2:
            gscore = torch.topk(groups, 2, dim=1).values.sum(1)
        else:
            gscore = groups.max(1).values
        best = max(itertools.combinations(range(n_group), topk_group),
                   key=lambda c: float(sum(gscore[j] for j in c)))
        eligible = [e for e in range(E) if e // per in best]
    subset = max(itertools.combinations(eligible, K), key=lambda c: float(sum(key[e] for e in c)))
    ids = sorted(subset, key=lambda e: -float(key[e]))
    w = score[ids]
    if renormalize:
        w = w / w.sum()
    return np.array(ids, np.int32), (w * rsf).numpy()


def make_layer(E, K, H, I, T, *, w_dtype=O.F32, x_dtype=O.F32, seed=0, scoring=O.SOFTMAX,
               renormalize=True, n_group=0, topk_group=0, rsf=1.0, bias=False,
               shared=False, identical=False, act_fp8=False, w_std=0.05, shared_I=0):
    """A small random layer as oracle arrays plus torch float64 copies of what
    it encodes; the shared expert has intermediate size shared_I (0: I)."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(T, H, generator=g)
    logits = torch.randn(T, E, generator=g).numpy().astype(np.float32)
    w13 = torch.randn(E, 2 * I, H, generator=g) * w_std
    w2 = torch.randn(E, H, I, generator=g) * w_std
    if identical:
        w13[:] = w13[0]
        w2[:] = w2[0]
    Is = shared_I or I
    sw13 = torch.randn(2 * Is, H, generator=g) * w_std
    sw2 = torch.randn(H, Is, generator=g) * w_std
    b = (torch.randn(E, generator=g) * 0.01).numpy().astype(np.float32) if bias else None
    L = dict(T=T, E=E, K=K, H=H, I=I, scoring=scoring, renormalize=renormalize,
             n_group=n_group, topk_group=topk_group, routed_scaling_factor=rsf,
             x_dtype=x_dtype, w_dtype=w_dtype, act_fp8=act_fp8, logits=logits, bias=b,
             shared_I=shared_I)
    ref = {}
    if x_dtype == O.F32:
        L["hidden"] = x.numpy().astype(np.float32)
        ref["x"] = x.double()
    else:
        L["hidden"] = _bf16_bits(x)
        ref["x"] = _bits_to_f64(L["hidden"])

    def enc(w):
        if w_dtype == O.F32:
            return w.numpy().astype(np.float32), None, w.double()
        if w_dtype == O.BF16:
            bits = _bf16_bits(w)
            return bits, None, _bits_to_f64(bits)
        # e4m3 with 128x128 block scales, quantised by torch
        N, Kd = w.shape[-2:]
        lead = w.shape[:-2]
        blk = w.reshape(*lead, N // 128, 128, Kd // 128, 128)
        s = (blk.abs().amax(dim=(-3, -1)).clamp(min=1e-10) / 448.0).float()
        q = (blk / s[..., :, None, :, None]).clamp(-448, 448).reshape(w.shape)
        codes = _e4m3_torch_encode(q)
        dq = _e4m3_torch_decode(codes).reshape(*lead, N // 128, 128, Kd // 128, 128)
        dq = (dq * s.double()[..., :, None, :, None]).reshape(w.shape)
        return codes, s.numpy(), dq

    L["w13"], L["w13_scale"], ref["w13"] = enc(w13)
    L["w2"], L["w2_scale"], ref["w2"] = enc(w2)
    if shared:
        L["shared_w13"], L["shared_w13_scale"], ref["sw13"] = enc(sw13)
        L["shared_w2"], L["shared_w2_scale"], ref["sw2"] = enc(sw2)
    return L, ref


def _close(a, b, rtol, what):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    err = np.max(np.abs(a - b)) if a.size else 0.0
    scale = max(np.max(np.abs(b)) if b.size else 0.0, 1e-300)
    assert err <= rtol * scale, "%s: max|err|/max|ref| = %.3e > %.1e" % (what, err / scale, rtol)


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def check_bf16_decode(lib_=None):
    codes = np.arange(65536, dtype=np.uint16)
    mine = O.bf16_to_f64(codes, lib_=lib_)
    ref = _bits_to_f64(codes).numpy()
    both_nan = np.isnan(mine) & np.isnan(ref)
    assert np.array_equal(mine[~both_nan], ref[~both_nan]), "bf16 decode differs from torch"
    assert np.array_equal(np.isnan(mine), np.isnan(ref))


def check_e4m3_decode(lib_=None):
    codes = np.arange(256, dtype=np.uint8)
    mine = O.e4m3_to_f64(codes, lib_=lib_)
    ref = _e4m3_torch_decode(codes).numpy()
    assert np.array_equal(np.isnan(mine), np.isnan(ref)), "e4m3 NaN codes differ"
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok]), "e4m3 decode differs from torch"
    assert np.nanmax(mine) == 448.0 and np.nanmin(mine) == -448.0


def check_e4m3_encode(lib_=None):
    grid = _e4m3_torch_decode(np.arange(256, dtype=np.uint8)).numpy()
    grid = np.unique(grid[~np.isnan(grid)])
    mids = 0.5 * (grid[:-1] + grid[1:])
    rng = np.random.default_rng(7)
    xs = np.concatenate([
        grid, mids, np.nextafter(mids, 0), np.nextafter(mids, 1000),
        rng.uniform(-448, 448, 3000), rng.uniform(-1, 1, 2000) * 2.0 ** -6,
        rng.standard_normal(2000) * 20,
    ]).astype(np.float32)
    xs = xs[np.abs(xs) <= 448]
    mine = O.e4m3_from_f32(xs, lib_=lib_)
    ref = _e4m3_torch_encode(torch.from_numpy(xs))
    bad = np.nonzero(mine != ref)[0]
    assert bad.size == 0, "e4m3 encode differs from torch at %r" % (xs[bad[:5]].tolist(),)
    # reading: saturate out-of-range magnitudes to +-448
    sat = O.e4m3_from_f32(np.array([448.5, 470.0, 1e6, -1e6, -500.0], np.float32), lib_=lib_)
    assert sat.tolist() == [0x7E, 0x7E, 0x7E, 0xFE, 0xFE], sat


def check_quant_rule(lib_=None):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((9, 512)) * rng.uniform(0.01, 30, (9, 1))).astype(np.float32)
    x[3, 128:256] = 0.0                      # an all-zero group
    x[4, :128] *= 1e-8                       # a tiny group
    q, s = O.quant_fp8_groups(x, 128, lib_=lib_)
    xt = torch.from_numpy(x).reshape(9, 4, 128)
    st = torch.clamp(xt.abs().amax(-1), min=1e-10) / 448.0          # float32 torch
    qt = _e4m3_torch_encode((xt / st[..., None]).clamp(-448, 448)).reshape(9, 512)
    assert np.array_equal(s, st.numpy()), "group scales differ from the float32 rule"
    assert np.array_equal(q, qt), "group codes differ from torch's encoder"
    deq = _e4m3_torch_decode(q).numpy().reshape(9, 4, 128) * s[..., None].astype(np.float64)
    err = np.abs(deq - x.reshape(9, 4, 128).astype(np.float64))
    bound = np.maximum(2.0 ** -4 * np.abs(x.reshape(9, 4, 128)), 2.0 ** -10 * s[..., None]) * (1 + 1e-6)
    assert np.all(err <= bound), "round-trip error above half an e4m3 ulp"
    # the largest magnitude of every non-zero group lands on +-448
    amax_code = np.take_along_axis(q.reshape(9, 4, 128), np.abs(x.reshape(9, 4, 128)).argmax(-1)[..., None], -1)
    nz = np.abs(x.reshape(9, 4, 128)).max(-1) > 0
    assert np.all((amax_code[..., 0][nz] & 0x7F) == 0x7E)


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------


def check_route_softmax_bruteforce(lib_=None):
    rng = np.random.default_rng(3)
    for E, K in [(4, 1), (4, 2), (6, 3), (8, 2), (12, 4), (16, 3), (16, 1), (5, 5)]:
        logits = rng.standard_normal((20, E)).astype(np.float32)
        for renorm in (True, False):
            ids, w = O.route(logits, K, renormalize=renorm, routed_scaling_factor=1.7, lib_=lib_)
            for t in range(20):
                bi, bw = brute_route(logits[t], K, renormalize=renorm, rsf=1.7)
                assert np.array_equal(ids[t], bi), (E, K, t, ids[t], bi)
                _close(w[t], bw, 1e-13, "softmax weights")


def check_route_softmax_weights(lib_=None):
    rng = np.random.default_rng(5)
    logits = (rng.standard_normal((64, 32)) * 3).astype(np.float32)
    ids, w = O.route(logits, 6, renormalize=True, lib_=lib_)
    sel = torch.tensor(np.take_along_axis(logits, ids, 1), dtype=torch.float64)
    _close(w, torch.softmax(sel, 1).numpy(), 1e-13, "renormalised weights = softmax of the selected logits")
    _close(w.sum(1), np.ones(64), 1e-14, "renormalised weights sum to 1")
    ids2, w2 = O.route(logits, 6, renormalize=False, routed_scaling_factor=2.5, lib_=lib_)
    assert np.array_equal(ids, ids2)
    full = torch.softmax(torch.tensor(logits, dtype=torch.float64), 1).numpy()
    _close(w2, 2.5 * np.take_along_axis(full, ids, 1), 1e-13, "plain softmax weights")
    # descending selection order
    assert np.all(np.diff(np.take_along_axis(logits, ids, 1), axis=1) < 0)


def check_route_ties(lib_=None):
    # exact ties break to the lower expert index, at every level
    logits = np.zeros((1, 8), np.float32)
    ids, _ = O.route(logits, 3, lib_=lib_)
    assert ids[0].tolist() == [0, 1, 2], ids
    logits = np.array([[1, 3, 3, 0, 3, 1, 2, 2]], np.float32)
    ids, _ = O.route(logits, 5, lib_=lib_)
    assert ids[0].tolist() == [1, 2, 4, 6, 7], ids
    # tied groups: group 1 and 2 tie on score, the lower group wins
    logits = np.array([[0.0, 0.1, 2.0, 1.0, 2.0, 1.0, -1.0, -2.0]], np.float32)
    ids, _ = O.route(logits, 2, scoring=O.SIGMOID, n_group=4, topk_group=1,
                     bias=np.zeros(8, np.float32), lib_=lib_)
    assert ids[0].tolist() == [2, 3], ids
    # -0 and +0 are the same value (IEEE 754 equality), so they tie and the
    # lower index wins whichever sign it carries
    logits = np.array([[-1.0, -0.0, 0.0, -2.0, -0.0, 0.0]], np.float32)
    assert np.signbit(logits[0, 1]) and not np.signbit(logits[0, 2])
    ids, w = O.route(logits, 4, lib_=lib_)
    assert ids[0].tolist() == [1, 2, 4, 5], ids
    assert np.all(w[0] == 0.25), w  # four equal probabilities, renormalised
    ids, _ = O.route(logits, 1, renormalize=False, lib_=lib_)
    assert ids[0].tolist() == [1], ids
    # groups scored by their largest key (no bias): group 0's best is -0,
    # group 1's +0; the tie keeps the lower group
    logits = np.array([[-0.0, -3.0, 0.0, -1.0, -5.0, -4.0]], np.float32)
    ids, _ = O.route(logits, 2, n_group=3, topk_group=1, lib_=lib_)
    assert ids[0].tolist() == [0, 1], ids


def check_route_grouped_bruteforce(lib_=None):
    rng = np.random.default_rng(9)
    cases = [(8, 4, 2, 2), (8, 4, 2, 3), (12, 3, 2, 4), (16, 4, 3, 5), (16, 8, 4, 4), (16, 2, 1, 3)]
    for E, G, TG, K in cases:
        logits = rng.standard_normal((25, E)).astype(np.float32)
        for use_bias in (True, False):
            b = (rng.standard_normal(E) * 0.3).astype(np.float32) if use_bias else None
            for scoring in (O.SIGMOID, O.SOFTMAX):
                if scoring == O.SOFTMAX and use_bias:
                    continue
                ids, w = O.route(logits, K, bias=b, scoring=scoring, n_group=G, topk_group=TG,
                                 routed_scaling_factor=2.5, lib_=lib_)
                for t in range(25):
                    bi, bw = brute_route(logits[t], K, bias=b, scoring=scoring, n_group=G,
                                         topk_group=TG, rsf=2.5)
                    assert np.array_equal(ids[t], bi), (E, G, TG, K, use_bias, t, ids[t], bi)
                    _close(w[t], bw, 1e-13, "grouped weights")


def check_route_grouped_reductions(lib_=None):
    rng = np.random.default_rng(13)
    E, K = 32, 6
    logits = rng.standard_normal((40, E)).astype(np.float32)
    b = (rng.standard_normal(E) * 0.05).astype(np.float32)
    key = torch.sigmoid(torch.tensor(logits, dtype=torch.float64)) + torch.tensor(b, dtype=torch.float64)
    ref = torch.topk(key, K, dim=1).indices.numpy()
    for G, TG in [(1, 1), (4, 4), (8, 8), (0, 0)]:
        ids, w = O.route(logits, K, bias=b, scoring=O.SIGMOID, n_group=G, topk_group=TG, lib_=lib_)
        assert np.array_equal(ids, ref), (G, TG)
        s = torch.sigmoid(torch.tensor(np.take_along_axis(logits, ids, 1), dtype=torch.float64))
        _close(w, (s / s.sum(1, keepdim=True)).numpy(), 1e-13, "bias never enters the weights")
    ids, w = O.route(logits, K, bias=b, scoring=O.SIGMOID, renormalize=False,
                     routed_scaling_factor=2.5, lib_=lib_)
    s = torch.sigmoid(torch.tensor(np.take_along_axis(logits, ids, 1), dtype=torch.float64))
    _close(w, 2.5 * s.numpy(), 1e-13, "sigmoid weights without renormalisation")


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------


def check_permute(lib_=None):
    rng = np.random.default_rng(21)
    for T, K, E in [(0, 2, 8), (1, 1, 1), (37, 2, 8), (200, 8, 128), (64, 8, 256), (50, 3, 5)]:
        if E <= 8:
            ids = rng.integers(0, E, (T, K)).astype(np.int32)
        else:  # skewed, with empty experts
            ids = np.minimum(rng.zipf(1.5, (T, K)) - 1, E - 1).astype(np.int32)
        off, srt, inv = O.permute(ids, E, lib_=lib_)
        flat = ids.reshape(-1)
        ref = np.argsort(flat, kind="stable")
        assert np.array_equal(srt, ref.astype(np.int32))
        cnt = np.bincount(flat, minlength=E)
        assert np.array_equal(off, np.concatenate([[0], np.cumsum(cnt)]).astype(np.int32))
        assert np.array_equal(inv[srt], np.arange(flat.size))


# ---------------------------------------------------------------------------
# the layer
# ---------------------------------------------------------------------------


def _forward(L, tokens=None, lib_=None, nthreads=1):
    tokens = range(L["T"]) if tokens is None else tokens
    return O.moe_forward_tokens(L, list(tokens), nthreads=nthreads, lib_=lib_)


def check_layer_dense(lib_=None):
    for w_dtype, x_dtype in [(O.F32, O.F32), (O.BF16, O.BF16)]:
        L, ref = make_layer(1, 1, 64, 96, 7, w_dtype=w_dtype, x_dtype=x_dtype, seed=1)
        out = _forward(L, lib_=lib_)
        exp = dense_swiglu(ref["x"], ref["w13"][0], ref["w2"][0]).numpy()
        _close(out, exp, 1e-12, "top-1 single expert = dense SwiGLU")


def check_layer_identical_experts(lib_=None):
    L, ref = make_layer(6, 2, 48, 80, 9, seed=2, identical=True)
    _close(_forward(L, lib_=lib_), dense_swiglu(ref["x"], ref["w13"][0], ref["w2"][0]).numpy(),
           1e-12, "identical experts, renormalised = dense")
    L, ref = make_layer(8, 3, 32, 40, 9, seed=3, identical=True, scoring=O.SIGMOID,
                        n_group=4, topk_group=2, rsf=2.5, bias=True)
    _close(_forward(L, lib_=lib_), 2.5 * dense_swiglu(ref["x"], ref["w13"][0], ref["w2"][0]).numpy(),
           1e-12, "identical experts, grouped sigmoid = rsf * dense")


def check_layer_bruteforce_combine(lib_=None):
    for kw in [dict(E=6, K=2), dict(E=8, K=3, scoring=O.SIGMOID, n_group=4, topk_group=2,
                                    rsf=2.5, bias=True),
               dict(E=5, K=2, renormalize=False)]:
        E, K = kw.pop("E"), kw.pop("K")
        L, ref = make_layer(E, K, 40, 56, 11, seed=4, **kw)
        out = _forward(L, lib_=lib_)
        exp = np.zeros_like(out)
        for t in range(L["T"]):
            ids, w = brute_route(L["logits"][t], K, bias=L["bias"], scoring=L["scoring"],
                                 renormalize=L["renormalize"], n_group=L["n_group"],
                                 topk_group=L["topk_group"], rsf=L["routed_scaling_factor"])
            for e, wk in zip(ids, w):
                exp[t] += wk * dense_swiglu(ref["x"][t:t + 1], ref["w13"][e], ref["w2"][e]).numpy()[0]
        _close(out, exp, 1e-12, "weighted combine of per-expert dense MLPs")


def check_layer_linearity(lib_=None):
    L, _ = make_layer(8, 2, 32, 48, 6, seed=5, scoring=O.SIGMOID, n_group=2, topk_group=1,
                      bias=True, rsf=1.0)
    base = _forward(L, lib_=lib_)
    L["routed_scaling_factor"] = 2.5
    _close(_forward(L, lib_=lib_), 2.5 * base, 1e-14, "output linear in routed_scaling_factor")


def check_layer_token_permutation(lib_=None):
    L, _ = make_layer(8, 2, 32, 40, 13, seed=6, w_dtype=O.BF16, x_dtype=O.BF16)
    out = _forward(L, lib_=lib_)
    perm = np.random.default_rng(1).permutation(13)
    L2 = dict(L)
    L2["hidden"] = L["hidden"][perm]
    L2["logits"] = L["logits"][perm]
    out2 = _forward(L2, lib_=lib_, nthreads=3)
    assert np.array_equal(out2, out[perm]), "output rows do not follow the token permutation"


def check_layer_shared(lib_=None):
    # the shared expert is a dense gated MLP of its own intermediate size Is
    # (the SGLang DeepseekV2MoE builds it with moe_intermediate_size *
    # n_shared_experts), added with weight 1
    for Is in (0, 384):
        L, ref = make_layer(8, 2, 128, 128, 5, seed=7, shared=True, scoring=O.SIGMOID,
                            n_group=4, topk_group=2, bias=True, rsf=2.5, shared_I=Is)
        with_shared = _forward(L, lib_=lib_)
        L2 = {k: v for k, v in L.items() if not k.startswith("shared")}
        without = _forward(L2, lib_=lib_)
        _close(with_shared - without, dense_swiglu(ref["x"], ref["sw13"], ref["sw2"]).numpy(), 1e-11,
               "shared expert (Is=%d) adds its dense MLP with weight 1 (not rsf)" % Is)


def check_layer_fp8(lib_=None):
    """fp8 layer rebuilt with torch's e4m3 encoder and float32 scale arithmetic."""
    L, ref = make_layer(4, 2, 256, 256, 6, seed=8, w_dtype=O.E4M3, x_dtype=O.BF16, act_fp8=True,
                        shared=True, scoring=O.SIGMOID, n_group=2, topk_group=1, bias=True,
                        rsf=2.5, shared_I=512)
    out = _forward(L, lib_=lib_)

    def q128(v64):  # per-row group-128 quantise-dequantise in float32 with torch's encoder
        v = v64.float().reshape(v64.shape[0], -1, 128)
        s = torch.clamp(v.abs().amax(-1), min=1e-10) / 448.0
        c = _e4m3_torch_encode((v / s[..., None]).clamp(-448, 448))
        return (_e4m3_torch_decode(c).reshape(v.shape) * s.double()[..., None]).reshape(v64.shape)

    x = q128(ref["x"])

    def mlp(xr, w13, w2):
        I = w2.shape[1]
        act = F.silu(xr @ w13[:I].T) * (xr @ w13[I:].T)
        return q128(act) @ w2.T

    exp = np.zeros_like(out)
    for t in range(L["T"]):
        ids, w = brute_route(L["logits"][t], 2, bias=L["bias"], scoring=O.SIGMOID, n_group=2,
                             topk_group=1, rsf=2.5)
        for e, wk in zip(ids, w):
            exp[t] += wk * mlp(x[t:t + 1], ref["w13"][e], ref["w2"][e]).numpy()[0]
        exp[t] += mlp(x[t:t + 1], ref["sw13"], ref["sw2"]).numpy()[0]
    # act codes may round differently when the two float64 sums straddle a
    # float32 boundary; that moves an output by far less than this bound
    _close(out, exp, 1e-4, "fp8 layer vs torch-encoded rebuild")
    # and the fp8 layer stays near the unquantised layer (a few percent)
    Lf = dict(L, w_dtype=O.F32, act_fp8=False, x_dtype=O.F32,
              hidden=ref["x"].numpy().astype(np.float32),
              w13=ref["w13"].numpy().astype(np.float32), w2=ref["w2"].numpy().astype(np.float32),
              w13_scale=None, w2_scale=None,
              shared_w13=ref["sw13"].numpy().astype(np.float32),
              shared_w2=ref["sw2"].numpy().astype(np.float32),
              shared_w13_scale=None, shared_w2_scale=None)
    _close(out, _forward(Lf, lib_=lib_), 0.1, "fp8 layer near the unquantised layer")


# ---------------------------------------------------------------------------
# router gate logits and activation variants
# ---------------------------------------------------------------------------


def check_router_logits(lib_=None):
    """x W_g^T against torch's float64 matmul of the decoded values, and a
    gate of one-hot rows, which must copy hidden columns exactly."""
    g = torch.Generator().manual_seed(11)
    T, E, H = 9, 12, 96
    x = torch.randn(T, H, generator=g)
    w = torch.randn(E, H, generator=g) * 0.05
    for x_dtype, g_dtype in [(O.BF16, O.BF16), (O.BF16, O.F32), (O.F32, O.F32)]:
        xa = _bf16_bits(x) if x_dtype == O.BF16 else x.numpy().astype(np.float32)
        wa = _bf16_bits(w) if g_dtype == O.BF16 else w.numpy().astype(np.float32)
        x64 = _bits_to_f64(xa) if x_dtype == O.BF16 else torch.from_numpy(xa).double()
        w64 = _bits_to_f64(wa) if g_dtype == O.BF16 else torch.from_numpy(wa).double()
        out = O.router_logits(xa, x_dtype, wa, g_dtype, lib_=lib_)
        _close(out, (x64 @ w64.T).numpy(), 1e-13, "router logits vs torch matmul")
    cols = np.random.default_rng(3).permutation(H)[:E]
    onehot = np.zeros((E, H), np.float32)
    onehot[np.arange(E), cols] = 1.0
    xa = x.numpy().astype(np.float32)
    out = O.router_logits(xa, O.F32, onehot, O.F32, lib_=lib_)
    assert np.array_equal(out, xa[:, cols].astype(np.float64)), "one-hot gate rows must copy columns"


def _one_unit_layer(g, u_scale, limit=0.0, alpha=1.0):
    """E=1, K=1, H=1, I=1: gate = 2*g, up = 2*u_scale, down = 1, so the
    output is the activation of one (gate, up) pair."""
    return dict(T=1, E=1, K=1, H=1, I=1, x_dtype=O.F32, w_dtype=O.F32,
                hidden=np.array([[2.0]], np.float32), logits=np.zeros((1, 1), np.float32),
                w13=np.array([[[g], [u_scale]]], np.float32), w2=np.array([[[1.0]]], np.float32),
                clamp_limit=limit, act_alpha=alpha)


def check_layer_clamp_closed_form(lib_=None):
    """Clipped SwiGLU on single values: gate 10 -> 7, up -8 -> -7 (limit 7);
    gate -10 stays (only capped above), up 9 -> 7; alpha in the sigmoid."""
    import math
    cases = [((5.0, -4.0, 7.0, 1.0), 7.0 / (1.0 + math.exp(-7.0)) * -7.0),
             ((-5.0, 4.5, 7.0, 1.0), -10.0 / (1.0 + math.exp(10.0)) * 7.0),
             ((1.5, 2.0, 7.0, 1.0), 3.0 / (1.0 + math.exp(-3.0)) * 4.0),
             ((5.0, -4.0, 7.0, 1.702), 7.0 / (1.0 + math.exp(-1.702 * 7.0)) * -7.0),
             ((1.5, 2.0, 0.0, 1.702), 3.0 / (1.0 + math.exp(-1.702 * 3.0)) * 4.0)]
    for (gs, us, lim, a), exp in cases:
        out = _forward(_one_unit_layer(gs, us, lim, a), lib_=lib_)[0, 0]
        assert abs(out - exp) <= 1e-14 * abs(exp), "clipped SwiGLU %r: %r != %r" % ((gs, us, lim, a), out, exp)


def check_layer_activation_variants(lib_=None):
    """A limit above every |gate| and |up| changes nothing (bitwise); alpha
    and the non-gated form against torch's dense MLP for one expert."""
    L, ref = make_layer(4, 2, 48, 64, 7, seed=12)
    base = _forward(L, lib_=lib_)
    assert np.array_equal(_forward(dict(L, clamp_limit=1e6), lib_=lib_), base), "inactive clamp changed the output"
    assert np.array_equal(_forward(dict(L, act_alpha=1.0), lib_=lib_), base), "alpha = 1 changed the output"
    L, ref = make_layer(1, 1, 64, 96, 5, seed=13, w_dtype=O.BF16, x_dtype=O.BF16)
    I = 96
    x, w13, w2 = ref["x"], ref["w13"][0], ref["w2"][0]
    gate, up = x @ w13[:I].T, x @ w13[I:].T
    exp = ((gate * torch.sigmoid(1.702 * gate)) * up) @ w2.T
    _close(_forward(dict(L, act_alpha=1.702), lib_=lib_), exp.numpy(), 1e-12, "silu alpha, dense")
    gc, uc = gate.clamp(max=0.3), up.clamp(-0.3, 0.3)
    exp = (F.silu(gc) * uc) @ w2.T
    _close(_forward(dict(L, clamp_limit=0.3), lib_=lib_), exp.numpy(), 1e-12, "clipped SwiGLU, dense")
    # non-gated: w13 holds I rows only
    Ln = dict(L, gated=False, w13=L["w13"][:, :I])
    exp = F.silu(x @ w13[:I].T) @ w2.T
    _close(_forward(Ln, lib_=lib_), exp.numpy(), 1e-12, "non-gated SiLU MLP, dense")


def check_layer_weight_on_input(lib_=None):
    """Routing weight on the input: top-1 with renormalisation is unchanged;
    otherwise a brute force over per-expert dense MLPs of w_k x; and with
    every gate deep in SiLU's linear range the MLP is bilinear, so scaling
    the input by w scales the output by w^2."""
    L, _ = make_layer(6, 1, 32, 48, 5, seed=14)
    assert np.array_equal(_forward(dict(L, weight_on_input=True), lib_=lib_), _forward(L, lib_=lib_)), \
        "top-1 renormalised weight 1 must not change the output"
    L, ref = make_layer(6, 2, 40, 56, 8, seed=15, scoring=O.SIGMOID, n_group=2, topk_group=1,
                        bias=True, rsf=2.5, shared=True)
    out = _forward(dict(L, weight_on_input=True), lib_=lib_)
    exp = np.zeros_like(out)
    for t in range(L["T"]):
        ids, w = brute_route(L["logits"][t], 2, bias=L["bias"], scoring=O.SIGMOID, n_group=2,
                             topk_group=1, rsf=2.5)
        for e, wk in zip(ids, w):
            exp[t] += dense_swiglu(wk * ref["x"][t:t + 1], ref["w13"][e], ref["w2"][e]).numpy()[0]
        exp[t] += dense_swiglu(ref["x"][t:t + 1], ref["sw13"], ref["sw2"]).numpy()[0]
    _close(out, exp, 1e-12, "weight on input, brute force")
    # bilinear regime: positive x and gate rows make every gate >= ~1e3 * w
    g = torch.Generator().manual_seed(16)
    E, K, H, I, T = 4, 2, 16, 8, 5
    x = torch.rand(T, H, generator=g) + 1.0
    w13 = torch.randn(E, 2 * I, H, generator=g)
    w13[:, :I] = torch.rand(E, I, H, generator=g) * 200.0 + 100.0
    w2 = torch.randn(E, H, I, generator=g)
    Lb = dict(T=T, E=E, K=K, H=H, I=I, x_dtype=O.F32, w_dtype=O.F32, renormalize=True,
              hidden=x.numpy().astype(np.float32),
              logits=torch.randn(T, E, generator=g).numpy().astype(np.float32),
              w13=w13.numpy().astype(np.float32), w2=w2.numpy().astype(np.float32))
    per_w = _forward(Lb, lib_=lib_)
    on_in = _forward(dict(Lb, weight_on_input=True), lib_=lib_)
    exp_def = np.zeros_like(per_w)
    exp_sq = np.zeros_like(per_w)
    for t in range(T):
        ids, w = brute_route(Lb["logits"][t], K)
        for e, wk in zip(ids, w):
            y = O.moe_forward_tokens(dict(Lb, E=1, K=1, logits=np.zeros((T, 1), np.float32),
                                          w13=Lb["w13"][e:e + 1], w2=Lb["w2"][e:e + 1]), [t],
                                     lib_=lib_)[0]
            exp_def[t] += wk * y
            exp_sq[t] += wk * wk * y
    _close(per_w, exp_def, 1e-12, "bilinear regime, weight on output")
    _close(on_in, exp_sq, 1e-12, "bilinear regime, weight on input scales by w^2")


ALL_CHECKS = [
    check_bf16_decode, check_e4m3_decode, check_e4m3_encode, check_quant_rule,
    check_route_softmax_bruteforce, check_route_softmax_weights, check_route_ties,
    check_route_grouped_bruteforce, check_route_grouped_reductions, check_permute,
    check_layer_dense, check_layer_identical_experts, check_layer_bruteforce_combine,
    check_layer_linearity, check_layer_token_permutation, check_layer_shared, check_layer_fp8,
    check_router_logits, check_layer_clamp_closed_form, check_layer_activation_variants,
    check_layer_weight_on_input,
]

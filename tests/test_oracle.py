"""Pins for the oracle's routing and expert computation (CPU only).

Each test checks the oracle against something other than itself: brute-force
enumeration, closed forms, per-token textbook loops, invariants.  A plausible
mistake (missing bias, softmax over all experts, dropped bf16 rounding of the
intermediate, a transposed projection, a gate applied to the wrong slot)
fails at least one of them."""
import itertools
import math
import os

import numpy as np
import torch

from oracle import codecs
from oracle import moe as om
from sparse_moe_routed_amd import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)


def _x(T, H, seed=0, scale=1.0):
    return codecs.bf16_rne(np.random.default_rng(seed).standard_normal((T, H)) * scale)


# ---------------------------------------------------------------- routing
def test_route_matches_brute_force_subsets():
    rng = np.random.default_rng(7)
    E, k, H, T = 10, 3, 24, 50
    x = _x(T, H, 1)
    w = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    b = rng.normal(0, 0.1, E).astype(np.float32)
    ids, gates, gap, logits = om.route(x, w, b, k)
    for t in range(T):
        lt = [sum(float(x[t, h]) * float(w[e, h]) for h in range(H)) + float(b[e]) for e in range(E)]
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(lt[e] for e in s))
        assert set(ids[t].tolist()) == set(best)
        # ordered by logit, descending
        assert all(lt[ids[t, j]] >= lt[ids[t, j + 1]] for j in range(k - 1))
        z = [math.exp(lt[e]) for e in ids[t]]
        assert np.allclose(gates[t], [v / sum(z) for v in z], rtol=1e-12, atol=0)


def test_route_zero_router_closed_form():
    w = np.zeros((128, 2688), np.float32)
    _, b = synth.make_router(0)
    b = b.numpy()
    x = _x(3, 2688, 2)
    ids, gates, gap, _ = om.route(x, w, b, 6)
    rank = np.rint(np.exp(-2.0 * b.astype(np.float64))).astype(int)  # b_e = -0.5 ln(rank_e)
    want_ids = [int(np.nonzero(rank == r)[0][0]) for r in range(1, 7)]
    gold = []
    with open(os.path.join(GOLD, "route_zero_router.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                gold.append(float(line.split()[1]))
    for t in range(3):
        assert ids[t].tolist() == want_ids
        assert np.allclose(gates[t], gold, rtol=0, atol=2e-6)
    assert np.allclose(gap, -0.5 * math.log(6) + 0.5 * math.log(7))


def test_gates_sum_to_one_and_shift_invariant():
    w, b = synth.make_router(0)
    x = synth.make_tokens(16).float().numpy()
    ids, g, _, _ = om.route(x, w.numpy(), b.numpy(), 6)
    assert np.allclose(g.sum(1), 1.0, atol=1e-12)
    assert (g > 0).all()
    ids2, g2, _, _ = om.route(x, w.numpy(), b.numpy().astype(np.float64) + 3.25, 6)
    assert np.array_equal(ids, ids2)
    assert np.allclose(g, g2, rtol=1e-12, atol=0)
    # six distinct experts in [0, 128) per token
    assert all(len(set(r)) == 6 for r in ids.tolist())
    assert ids.min() >= 0 and ids.max() < 128


def test_route_ties_go_to_lower_index():
    x = np.ones((1, 4))
    w = np.zeros((5, 4), np.float32)
    b = np.array([1.0, 2.0, 2.0, 0.5, 2.0], np.float32)
    ids, g, gap, _ = om.route(x, w, b, 3)
    assert ids[0].tolist() == [1, 2, 4]
    assert np.allclose(g[0], 1 / 3)
    ids, g, gap, _ = om.route(x, w, b, 2)
    assert ids[0].tolist() == [1, 2] and gap[0] == 0.0


def test_route_k_equals_e_is_dense_softmax():
    rng = np.random.default_rng(5)
    x = _x(4, 8, 3)
    w = rng.normal(0, 1, (6, 8)).astype(np.float32)
    ids, g, _, logits = om.route(x, w, None, 6)
    sm = np.exp(logits - logits.max(1, keepdims=True))
    sm /= sm.sum(1, keepdims=True)
    dense = np.zeros_like(sm)
    np.put_along_axis(dense, ids.astype(np.int64), g, axis=1)
    assert np.allclose(dense, sm, rtol=1e-12, atol=1e-15)


# ---------------------------------------------------------------- experts
def _identity_bank(E, H, F, scales=None):
    up = np.zeros((E, F, H), np.float32)
    down = np.zeros((E, H, F), np.float32)
    for e in range(E):
        c = 1.0 if scales is None else scales[e]
        up[e, :, :F] = np.eye(F) * c
        down[e, :F, :] = np.eye(F)
    return _bf16(up), _bf16(down)


def test_identity_experts_bit_exact():
    # W_up = [I | 0], W_down = [I ; 0], k = 1 (gate exactly 1):
    # y[:F] = bf16(relu(x[:F])^2) and y[F:] = 0, every step exact.
    H, F, E, T = 48, 32, 3, 20
    up, down = _identity_bank(E, H, F)
    x = _x(T, H, 4, scale=3.0)
    ids = np.random.default_rng(0).integers(0, E, (T, 1)).astype(np.int32)
    y = om.forward(x, ids, np.ones((T, 1)), om.ExpertBank(up, down))
    want = codecs.bf16_rne(np.maximum(x[:, :F], 0) ** 2)
    assert np.array_equal(y[:, :F], want)
    assert not y[:, F:].any()
    # the intermediate is rounded to bf16: the unrounded square differs somewhere
    assert not np.array_equal(want, np.maximum(x[:, :F], 0) ** 2)


def test_scaled_identity_places_gates_per_slot():
    # expert e scales the identity by c_e, so each slot's contribution is
    # distinguishable: y_t[:F] = sum_j g_tj * bf16(relu(c_{e_tj} x_t[:F])^2)
    H, F, E, T, k = 40, 24, 7, 12, 3
    c = [0.5, 1.0, 1.5, 2.0, 2.5, 3.0, 0.25]
    up, down = _identity_bank(E, H, F, c)
    x = _x(T, H, 6)
    rng = np.random.default_rng(9)
    ids = np.stack([rng.choice(E, k, replace=False) for _ in range(T)]).astype(np.int32)
    g = rng.random((T, k))
    g /= g.sum(1, keepdims=True)
    y = om.forward(x, ids, g, om.ExpertBank(up, down))
    for t in range(T):
        want = np.zeros(F)
        for j in range(k):
            cb = float(_bf16(np.array([c[ids[t, j]]])).float()[0])
            want += g[t, j] * codecs.bf16_rne(np.maximum(cb * x[t, :F], 0) ** 2)
        assert np.allclose(y[t, :F], want, rtol=1e-13, atol=1e-13)
        assert not y[t, F:].any()


def test_single_expert_is_textbook_ffn():
    # E = 1, k = 1: y = W_down relu(W_up x)^2 with a bf16 intermediate, by loops
    H, F, T = 20, 12, 5
    rng = np.random.default_rng(11)
    up = _bf16(rng.normal(0, 1 / math.sqrt(H), (1, F, H)))
    down = _bf16(rng.normal(0, 1 / math.sqrt(F), (1, H, F)))
    x = _x(T, H, 12)
    y = om.forward(x, np.zeros((T, 1), np.int32), np.ones((T, 1)), om.ExpertBank(up, down))
    U = up.float().numpy()[0].astype(np.float64)
    D = down.float().numpy()[0].astype(np.float64)
    for t in range(T):
        a = []
        for f in range(F):
            h = 0.0
            for i in range(H):
                h += U[f, i] * x[t, i]
            a.append(float(codecs.bf16_rne(np.array([max(h, 0.0) ** 2]))[0]))
        for o in range(H):
            acc = 0.0
            for f in range(F):
                acc += D[o, f] * a[f]
            assert abs(y[t, o] - acc) <= 1e-12 * (1 + abs(acc))


def _small_layer(seed=0, E=9, H=32, F=16, T=11, k=3):
    rng = np.random.default_rng(seed)
    up = _bf16(rng.normal(0, 1 / math.sqrt(H), (E, F, H)))
    down = _bf16(rng.normal(0, 1 / math.sqrt(F), (E, H, F)))
    w = rng.normal(0, 0.3, (E, H)).astype(np.float32)
    b = rng.normal(0, 0.2, E).astype(np.float32)
    x = _x(T, H, seed + 100)
    return x, w, b, up, down, k


def test_layer_equals_dense_masked_sum_over_all_experts():
    x, w, b, up, down, k = _small_layer()
    ids, g, _, _ = om.route(x, w, b, k)
    y = om.forward(x, ids, g, om.ExpertBank(up, down))
    E = w.shape[0]
    G = np.zeros((x.shape[0], E))
    np.put_along_axis(G, ids.astype(np.int64), g, axis=1)
    U = up.float().numpy().astype(np.float64)
    D = down.float().numpy().astype(np.float64)
    dense = np.zeros_like(y)
    for e in range(E):
        a = codecs.bf16_rne(np.maximum(x @ U[e].T, 0) ** 2)
        dense += G[:, e:e + 1] * (a @ D[e].T)
    assert np.allclose(y, dense, rtol=1e-12, atol=1e-12)


def test_linear_in_gates_and_relabelling_equivariant():
    x, w, b, up, down, k = _small_layer(1)
    ids, g, _, _ = om.route(x, w, b, k)
    bank = om.ExpertBank(up, down)
    y = om.forward(x, ids, g, bank)
    assert np.allclose(om.forward(x, ids, 2.5 * g, bank), 2.5 * y, rtol=1e-12, atol=1e-13)
    perm = np.random.default_rng(2).permutation(w.shape[0])  # new index of old expert e
    inv = np.argsort(perm)
    bank_p = om.ExpertBank(up[torch.from_numpy(inv)], down[torch.from_numpy(inv)])
    y_p = om.forward(x, perm[ids].astype(np.int32), g, bank_p)
    assert np.allclose(y_p, y, rtol=1e-13, atol=1e-13)
    ids_p, g_p, _, _ = om.route(x, w[inv], b[inv], k)
    assert np.array_equal(np.sort(ids_p, 1), np.sort(perm[ids], 1))


def test_quantised_forward_matches_hand_dequantised():
    # fp8 / nvfp4 forward = bf16 math on fake-quantised activations and weights
    x, w, b, up, down, k = _small_layer(3, H=64, F=32)
    ids, g, _, _ = om.route(x, w, b, k)
    for fmt in ("fp8", "nvfp4"):
        y, a = om.forward(x, ids, g, om.ExpertBank(up, down, fmt), return_a=True)
        if fmt == "fp8":
            qx, sx = codecs.fp8_quantize(x)
            xq = codecs.e4m3_decode(qx) * np.float64(sx)
        else:
            qx, sbx, Sx = codecs.nvfp4_quantize(x)
            xq = codecs.nvfp4_dequantize(qx, sbx, Sx)
        U = up.float().numpy().astype(np.float64)
        D = down.float().numpy().astype(np.float64)
        T = x.shape[0]
        a2 = np.zeros((T * k, U.shape[1]))
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                if fmt == "fp8":
                    qu, su = codecs.fp8_quantize(U[e])
                    Ue = codecs.e4m3_decode(qu) * np.float64(su)
                else:
                    Ue = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(U[e]))
                a2[t * k + j] = codecs.bf16_rne(np.maximum(Ue @ xq[t], 0) ** 2)
        assert np.array_equal(a, a2)
        # the down half by hand: the stacked intermediate [T*k, F] is quantised
        # once as one tensor (one scale for all rows of all experts), each
        # W_down per expert, then a per-token, per-slot loop in float64
        if fmt == "fp8":
            qa, sa = codecs.fp8_quantize(a2)
            a2q = codecs.e4m3_decode(qa) * np.float64(sa)
        else:
            a2q = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(a2))
        y2 = np.zeros_like(y)
        for t in range(T):
            for j in range(k):
                e = ids[t, j]
                if fmt == "fp8":
                    qd, sd = codecs.fp8_quantize(D[e])
                    De = codecs.e4m3_decode(qd) * np.float64(sd)
                else:
                    De = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(D[e]))
                for o in range(De.shape[0]):
                    y2[t, o] += g[t, j] * float(np.dot(De[o], a2q[t * k + j]))
        assert np.allclose(y, y2, rtol=1e-12, atol=1e-12 * np.abs(y2).max())
        # different from the bf16 path (the quantisation is really applied)
        yb = om.forward(x, ids, g, om.ExpertBank(up, down, "bf16"))
        assert not np.allclose(y, yb, rtol=1e-3, atol=1e-3)
        rel = np.abs(y - yb).max() / np.sqrt(np.mean(yb ** 2))
        assert rel < (0.5 if fmt == "fp8" else 1.5)


def test_quantised_intermediate_is_one_tensor():
    # the intermediate scale is taken over all routed rows together: with one
    # expert's rows made much larger than the others', quantising each
    # expert's rows on their own would give the small rows finer codes
    x, w, b, up, down, k = _small_layer(4, H=64, F=32)
    T = x.shape[0]
    ids = np.stack([np.arange(k) + (t % 2) * k for t in range(T)]).astype(np.int32)
    g = np.full((T, k), 1.0 / k)
    big = up.clone()
    big[0] = big[0] * 8  # expert 0 (even tokens, slot 0): rows 64x larger after ReLU^2
    for fmt in ("fp8", "nvfp4"):
        bank = om.ExpertBank(big, down, fmt)
        y, a = om.forward(x, ids, g, bank, return_a=True)
        aq_tensor = om.quantise_activation(a, fmt)
        per_expert = np.zeros_like(a)
        for e in np.unique(ids):
            rows = np.nonzero(ids.reshape(-1) == e)[0]
            per_expert[rows] = om.quantise_activation(a[rows], fmt)
        assert not np.array_equal(aq_tensor, per_expert)

        def down_half(aq):
            out = np.zeros_like(y)
            for t in range(T):
                for j in range(k):
                    De = bank.down(int(ids[t, j]))
                    out[t] += g[t, j] * (De @ aq[t * k + j])
            return out

        assert np.allclose(y, down_half(aq_tensor), rtol=1e-12, atol=1e-12 * np.abs(y).max())
        assert not np.allclose(y, down_half(per_expert), rtol=1e-6, atol=0)
        assert not np.allclose(y, down_half(a), rtol=1e-6, atol=0)


def test_shared_expert_textbook_and_quantised_loops():
    # the shared expert is an FFN on every token with weight 1; in the
    # quantised formats x is quantised as one tensor and the shared
    # intermediate [T, F_s] as a tensor of its own
    H, Fs, T = 48, 32, 7
    rng = np.random.default_rng(21)
    up = _bf16(rng.normal(0, 1 / math.sqrt(H), (Fs, H)))
    down = _bf16(rng.normal(0, 1 / math.sqrt(Fs), (H, Fs)))
    x = _x(T, H, 22)
    U = up.float().numpy().astype(np.float64)
    D = down.float().numpy().astype(np.float64)
    for fmt in ("bf16", "fp8", "nvfp4"):
        y = om.shared_expert(x, up, down, fmt)
        if fmt == "bf16":
            xq, Uq, Dq = x, U, D
        elif fmt == "fp8":
            qx, sx = codecs.fp8_quantize(x)
            xq = codecs.e4m3_decode(qx) * np.float64(sx)
            qu, su = codecs.fp8_quantize(U)
            Uq = codecs.e4m3_decode(qu) * np.float64(su)
            qd, sd = codecs.fp8_quantize(D)
            Dq = codecs.e4m3_decode(qd) * np.float64(sd)
        else:
            xq = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(x))
            Uq = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(U))
            Dq = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(D))
        a = np.zeros((T, Fs))
        for t in range(T):
            for f in range(Fs):
                h = 0.0
                for i in range(H):
                    h += Uq[f, i] * xq[t, i]
                a[t, f] = float(codecs.bf16_rne(np.array([max(h, 0.0) ** 2]))[0])
        if fmt == "fp8":
            qa, sa = codecs.fp8_quantize(a)
            aq = codecs.e4m3_decode(qa) * np.float64(sa)
        elif fmt == "nvfp4":
            aq = codecs.nvfp4_dequantize(*codecs.nvfp4_quantize(a))
        else:
            aq = a
        for t in range(T):
            for o in range(H):
                acc = 0.0
                for f in range(Fs):
                    acc += Dq[o, f] * aq[t, f]
                assert abs(y[t, o] - acc) <= 1e-12 * (1 + abs(acc)), (fmt, t, o)


def test_shared_expert_identity_and_block_sum():
    # identity weights: y_s = bf16(relu(x)^2) on the first F_s dims, exactly
    H, Fs, T = 48, 32, 9
    up, down = _identity_bank(1, H, Fs)
    x = _x(T, H, 23, scale=2.0)
    y = om.shared_expert(x, up[0], down[0])
    assert np.array_equal(y[:, :Fs], codecs.bf16_rne(np.maximum(x[:, :Fs], 0) ** 2))
    assert not y[:, Fs:].any()
    # the block is the routed layer plus the shared expert
    x, w, b, upr, downr, k = _small_layer(5, H=48, F=32)
    bank = om.ExpertBank(upr, downr)
    yb, ids, g, _ = om.block(x, w, b, bank, up[0], down[0], k)
    yr, ids2, g2, _ = om.layer(x, w, b, bank, k)
    assert np.array_equal(ids, ids2)
    assert np.allclose(yb - yr, om.shared_expert(x, up[0], down[0]), rtol=1e-12, atol=1e-12)


def test_empty_batch():
    x, w, b, up, down, k = _small_layer()
    y = om.forward(x[:0], np.zeros((0, k), np.int32), np.zeros((0, k)), om.ExpertBank(up, down))
    assert y.shape == (0, x.shape[1])


# ---------------------------------------------------------------- stacked path helpers
def test_prenorm_closed_form():
    x = np.array([[2.0] * 8, [-0.5] * 8, [0.0] * 8, [3.0, -3.0] * 4])
    y = om.prenorm(x)
    assert np.array_equal(y[0], np.ones(8))
    assert np.array_equal(y[1], -np.ones(8))
    assert not y[2].any()
    assert np.array_equal(y[3], np.array([1.0, -1.0] * 4))


def test_residual_add_rounds_to_bf16():
    assert om.residual_add(np.array([1.0]), np.array([2.0 ** -8 + 2.0 ** -30]))[0] == 1.0 + 2.0 ** -7


def test_full_size_routing_statistics():
    # the synthetic router gives skewed expert use at the real shape
    w, b = synth.make_router(0)
    x = synth.make_tokens(512).float().numpy()
    ids, g, gap, _ = om.route(x, w.numpy(), b.numpy(), 6)
    counts = np.bincount(ids.reshape(-1), minlength=128)
    assert counts.sum() == 512 * 6
    assert counts.max() > 4 * counts.mean()  # heavy head from the rank bias

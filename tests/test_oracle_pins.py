"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test names the passage it checks.  None of them re-types the oracle's own
formula: they compare it with worked examples from the pages, closed forms
derived by hand, brute force, an independent least-squares solve, explicit
sub-matrix inverses, or invariances.
"""
import json
import os

import numpy as np
import pytest

from oracle import gptq_ref as ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _correlated_x(rng, n, d, mix=0.6):
    """Token-major inputs with strongly correlated features."""
    base = rng.standard_normal((n, d))
    common = rng.standard_normal((n, 1))
    return base * (1 - mix) + common * mix * rng.uniform(0.5, 1.5, size=(1, d))


# --- P1: the ruler example ("What quantization is, and why anyone bothers") ---
def test_grid_example_from_page():
    g = _golden("grid_example.json")
    scale, zero, _ = ref.fit_ruler(np.array([[g["row_min"], g["row_max"]]]), g["bits"])
    # fp32 decision arithmetic: 0.08 to within one fp32 ulp.
    assert abs(float(scale[0]) - g["scale"]) <= np.spacing(np.float32(g["scale"]))
    assert zero[0] == g["zero_tick"]
    ticks = ref.dequantize(np.arange(16), scale[0], zero[0])
    np.testing.assert_allclose(ticks, g["ticks"], atol=1e-6)
    # 0.0 is exactly one of the ticks.
    assert ref.dequantize(g["zero_tick"], scale[0], zero[0]) == 0.0
    q, _ = ref.round_to_grid(np.array(g["ticks"]), scale[0], zero[0], g["bits"])
    np.testing.assert_array_equal(q, np.arange(16))


def test_grid_range_includes_zero_and_clamps():
    # All-positive row: the range is stretched down to 0, so the zero tick is 0.
    scale, zero, _ = ref.fit_ruler(np.array([[0.3, 0.6, 0.9]]), 4)
    assert zero[0] == 0 and np.isclose(scale[0], 0.9 / 15, rtol=1e-6)
    # All-negative row: zero sits on the top tick.
    scale, zero, _ = ref.fit_ruler(np.array([[-0.3, -0.9]]), 3)
    assert zero[0] == 7
    # A value past the end of the ruler clamps to the end tick.
    q, _ = ref.round_to_grid(np.array([5.0, -5.0]), np.float32(0.1), 3.0, 3)
    np.testing.assert_array_equal(q, [7, 0])
    # Exact midpoints round half to even.
    q, _ = ref.round_to_grid(np.array([0.25, 0.75]), np.float32(0.5), 0.0, 4)
    np.testing.assert_array_equal(q, [0, 2])


# --- P2: H = 2 X X^T is the Hessian of the output damage ("Measuring damage") ---
def test_hessian_matches_finite_differences():
    rng = np.random.default_rng(2)
    n, d = 50, 5
    X = rng.standard_normal((n, d))
    w0 = rng.standard_normal(d)

    def damage(w):
        y = X @ (w - w0)
        return float(y @ y)

    h = 1e-2
    fd = np.zeros((d, d))
    w = w0 + rng.standard_normal(d) * 0.1
    I = np.eye(d)
    for i in range(d):
        for j in range(d):
            fd[i, j] = (damage(w + h * I[i] + h * I[j]) - damage(w + h * I[i] - h * I[j])
                        - damage(w - h * I[i] + h * I[j]) + damage(w - h * I[i] - h * I[j])) / (4 * h * h)
    H = ref.hessian(X)
    assert np.linalg.norm(H - fd) / np.linalg.norm(H) <= 1e-6


def test_hessian_chunking_and_loss_forms_agree():
    rng = np.random.default_rng(3)
    X = rng.standard_normal((1000, 7)).astype(np.float32)
    H1 = ref.hessian(X, chunk=1 << 20)
    H2 = ref.hessian(X, chunk=37)
    np.testing.assert_allclose(H1, H2, rtol=1e-12, atol=1e-9)
    W0 = rng.standard_normal((3, 7))
    Wh = W0 + 0.01 * rng.standard_normal((3, 7))
    a = ref.layer_loss(W0, Wh, H1)
    b = ref.layer_loss_from_x(W0, Wh, X)
    assert abs(a - b) <= 1e-10 * b


# --- P3: the two-weight example ("Measuring damage where it matters") ---
def test_two_weight_example_undamped_repair_is_exact():
    g = _golden("two_weight_example.json")
    rng = np.random.default_rng(4)
    x1 = rng.standard_normal(1000)
    X = np.stack([x1, x1], axis=1)
    w = np.array([g["w1"], g["w2"]])
    unrep = np.array([g["w1_forced"], g["w2"]])
    err_unrep = ref.layer_loss_from_x(w[None], unrep[None], X)
    assert np.isclose(err_unrep, g["error"] ** 2 * np.sum(x1 * x1), rtol=1e-12)
    fixed = ref.lstsq_repair(w, X, 0, g["w1_forced"])
    assert np.isclose(fixed[1], g["w2_repaired"], atol=1e-12)
    err_fixed = ref.layer_loss_from_x(w[None], fixed[None], X)
    assert err_fixed <= 1e-25 * err_unrep


def test_two_weight_example_damped_pipeline_closed_form():
    # With x2 = x1, H = 2a[[1,1],[1,1]]; 1 % damping of the mean diagonal gives
    # H_d = 2a[[1+p, 1],[1, 1+p]], whose OBS repair moves w2 by e1/(1+p).
    # The output error left before w2's own rounding is therefore
    # (p/(1+p))^2 of the unrepaired one (derived by hand from the 2x2 inverse).
    p = _golden("damping.json")["percdamp"]
    g = _golden("two_weight_example.json")
    rng = np.random.default_rng(5)
    x1 = rng.standard_normal(1000)
    X = np.stack([x1, x1], axis=1)
    W0 = np.array([[g["w1"], g["w2"]]])
    out = ref.gptq_quantize(W0, ref.hessian(X), bits=4, percdamp=p)
    e1 = W0[0, 0] - out["w_hat"][0, 0]
    assert abs(e1) > 1e-4
    w2_turn = out["pre_round"][0, 1]
    assert np.isclose(w2_turn - W0[0, 1], e1 / (1 + p), rtol=1e-12)
    partial = np.array([[out["w_hat"][0, 0], w2_turn]])
    ratio = ref.layer_loss_from_x(W0, partial, X) / (e1 * e1 * np.sum(x1 * x1))
    assert np.isclose(ratio, (p / (1 + p)) ** 2, rtol=1e-9)
    assert np.isclose((p / (1 + p)) ** 2, 9.80296e-5, rtol=1e-5)


def test_singular_without_damping_is_an_error():
    x1 = np.random.default_rng(6).standard_normal(100)
    X = np.stack([x1, x1], axis=1)
    with pytest.raises(ref.NotPositiveDefinite):
        ref.gptq_quantize(np.array([[0.1, 0.2]]), ref.hessian(X), bits=4, percdamp=0.0)


# --- P4: OBS formula equals brute-force least squares ("The repair rule") ---
def test_obs_repair_equals_least_squares():
    rng = np.random.default_rng(7)
    for trial in range(5):
        X = _correlated_x(rng, 40, 6)
        w = rng.standard_normal(6)
        q = trial % 6
        value = np.round(w[q] * 4) / 4
        a = ref.obs_repair(w, ref.hessian(X), q, value)
        b = ref.lstsq_repair(w, X, q, value)
        assert a[q] == pytest.approx(value, abs=1e-15)
        assert np.max(np.abs(a - b)) <= 1e-13 * max(1.0, np.max(np.abs(w)))


# --- P5: correlation rho ("The repair rule", two correlated inputs) ---
@pytest.mark.parametrize("rho", [0.0, 0.3, 0.9, -0.5])
@pytest.mark.parametrize("damp", [0.0, 0.01])
def test_correlated_pair_absorption_and_damage(rho, damp):
    rng = np.random.default_rng(8)
    n = 256
    x1 = rng.standard_normal(n)
    z = rng.standard_normal(n)
    z -= (z @ x1) / (x1 @ x1) * x1            # exactly orthogonal to x1
    z *= np.linalg.norm(x1) / np.linalg.norm(z)
    x2 = rho * x1 + np.sqrt(1 - rho * rho) * z  # sample correlation exactly rho
    X = np.stack([x1, x2], axis=1)
    H = ref.hessian(X)
    H[np.arange(2), np.arange(2)] += damp * np.mean(np.diag(H))
    w = np.array([0.4, -0.2])
    e = 0.05
    rep = ref.obs_repair(w, H, 0, w[0] - e)
    assert rep[1] - w[1] == pytest.approx(rho * e / (1 + damp), abs=1e-14)
    if damp == 0.0:
        unrep = np.array([w[0] - e, w[1]])
        dmg_rep = ref.layer_loss_from_x(w[None], rep[None], X)
        dmg_unrep = ref.layer_loss_from_x(w[None], unrep[None], X)
        assert dmg_rep / dmg_unrep == pytest.approx(1 - rho * rho, abs=1e-12)


# --- P6: the Cholesky factor holds every shrinking inverse ("From one repair to a whole model") ---
def test_upper_factor_rows_are_the_shrinking_inverses():
    rng = np.random.default_rng(9)
    d = 7
    A = rng.standard_normal((d, 3 * d))
    Hd = A @ A.T + 0.1 * np.eye(d)
    U = ref.upper_cholesky_of_inverse(Hd)
    assert np.allclose(np.tril(U, -1), 0)
    np.testing.assert_allclose(U.T @ U, np.linalg.inv(Hd), rtol=1e-10, atol=1e-12)
    for q in range(d):
        Finv = np.linalg.inv(Hd[q:, q:])       # inverse restricted to the free set
        assert U[q, q] ** 2 == pytest.approx(Finv[0, 0], rel=1e-10)
        np.testing.assert_allclose(U[q, q:] / U[q, q], Finv[:, 0] / Finv[0, 0], rtol=1e-9, atol=1e-12)


def test_oracle_steps_match_repeated_obs_repairs():
    # Column-by-column GPTQ = quantize one weight, OBS-repair the rest with the
    # inverse of the still-free sub-matrix, repeat (the pre-GPTQ formulation
    # with a fixed order).  Check the pre-rounding values step by step.
    rng = np.random.default_rng(10)
    d = 6
    X = _correlated_x(rng, 60, d)
    W0 = rng.standard_normal((1, d)) * 0.1
    out = ref.gptq_quantize(W0, ref.hessian(X), bits=3, percdamp=0.01)
    Hd, _, _, _ = ref.prepare(ref.hessian(X), 0.01)
    w = W0[0].copy()
    for j in range(d):
        assert w[j] == pytest.approx(out["pre_round"][0, j], abs=1e-12)
        sub = ref.obs_repair(w[j:], Hd[j:, j:], 0, out["w_hat"][0, j])
        w[j:] = sub


# --- P7: H = c I reduces GPTQ to round-to-nearest ("The repair rule", rho = 0) ---
@pytest.mark.parametrize("groupsize", [-1, 16, 32])
@pytest.mark.parametrize("bits", [3, 4])
def test_identity_hessian_is_round_to_nearest(groupsize, bits):
    rng = np.random.default_rng(11)
    r, c = 17, 64
    W0 = rng.standard_normal((r, c)) * 0.02
    X = 3.0 * np.eye(c)                       # c tokens, one per input
    out = ref.gptq_quantize(W0, ref.hessian(X), bits=bits, groupsize=groupsize)
    codes, w_hat = ref.rtn(W0, bits, groupsize)
    np.testing.assert_array_equal(out["codes"], codes)
    np.testing.assert_array_equal(out["w_hat"], w_hat)


# --- P8: lazy blocks equal the plain column loop ("From one repair to a whole model") ---
@pytest.mark.parametrize("B,groupsize", [(128, -1), (1, -1), (7, -1), (32, 64), (128, 32), (32, 32), (64, 128)])
def test_lazy_batches_equal_plain_loop(B, groupsize):
    rng = np.random.default_rng(12)
    r, c = 9, 300 if groupsize <= 0 else 256
    X = _correlated_x(rng, 400, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    H = ref.hessian(X)
    a = ref.gptq_quantize(W0, H, bits=4, groupsize=groupsize)
    b = ref.gptq_quantize(W0, H, bits=4, groupsize=groupsize, blocksize=B)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_allclose(a["row_loss"], b["row_loss"], rtol=1e-12)
    np.testing.assert_allclose(a["pre_round"], b["pre_round"], rtol=1e-10, atol=1e-14)


# --- P9: the tracked losses add up to the damped quadratic form ---
def test_loss_bookkeeping_sums_to_quadratic_form():
    rng = np.random.default_rng(13)
    r, c = 11, 40
    X = _correlated_x(rng, 200, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    H = ref.hessian(X)
    for act_order in (False, True):
        out = ref.gptq_quantize(W0, H, bits=3, groupsize=8, act_order=act_order)
        Hd, perm, _, lam = ref.prepare(H, 0.01, act_order)
        D = (out["w_hat"] - W0)[:, perm]
        quad = 0.5 * np.einsum("ri,ij,rj->r", D, Hd, D)
        np.testing.assert_allclose(out["row_loss"], quad, rtol=1e-9)
        direct = ref.layer_loss_from_x(W0, out["w_hat"], X) + 0.5 * lam * np.sum(D * D)
        assert np.sum(out["row_loss"]) == pytest.approx(direct, rel=1e-9)


# --- P10: tiny layers against the exhaustive optimum ---
def test_tiny_layers_against_brute_force():
    rng = np.random.default_rng(14)
    ratios_gptq, ratios_rtn = [], []
    for _ in range(30):
        d = int(rng.integers(3, 6))
        X = _correlated_x(rng, 24, d, mix=0.8)
        w0 = rng.standard_normal(d) * 0.1
        out = ref.gptq_quantize(w0[None], ref.hessian(X), bits=3, percdamp=0.01)
        scale, zero = out["scales"][0, 0], out["zeros"][0, 0]
        best_codes, best = ref.brute_force_row(w0, X, scale, zero, 3)
        rtn_codes, rtn_hat = ref.rtn(w0[None], 3)
        g_obj = ref.layer_loss_from_x(w0[None], out["w_hat"], X)
        r_obj = ref.layer_loss_from_x(w0[None], rtn_hat, X)
        assert best <= g_obj * (1 + 1e-12) and best <= r_obj * (1 + 1e-12)
        ratios_gptq.append(g_obj / best)
        ratios_rtn.append(r_obj / best)
    # Compensation must help on correlated inputs; a flipped sign makes it hurt.
    assert np.mean(ratios_gptq) < np.mean(ratios_rtn)
    assert np.median(ratios_gptq) < 1.5


# --- P11: act-order is GPTQ on the explicitly permuted problem ("Paper vs. code") ---
def test_act_order_is_explicit_permutation():
    rng = np.random.default_rng(15)
    r, c = 8, 48
    X = _correlated_x(rng, 200, c) * rng.uniform(0.1, 3.0, size=(1, c))
    X[:, 5] = X[:, 9]                          # a tie in diag(H)
    W0 = rng.standard_normal((r, c)) * 0.02
    H = ref.hessian(X)
    a = ref.gptq_quantize(W0, H, bits=4, groupsize=16, act_order=True)
    perm = a["perm"]
    dg = np.diag(H)[perm]
    assert np.all(np.diff(dg) <= 0)
    ties = np.flatnonzero(np.diff(dg) == 0)
    assert all(perm[t] < perm[t + 1] for t in ties) and len(ties) >= 1
    b = ref.gptq_quantize(W0[:, perm], H[np.ix_(perm, perm)], bits=4, groupsize=16)
    np.testing.assert_array_equal(a["codes"][:, perm], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])
    np.testing.assert_array_equal(a["g_idx"][perm], np.arange(c) // 16)


# --- P12: one group spanning the row equals the per-row ruler ---
def test_single_group_equals_per_row():
    rng = np.random.default_rng(16)
    r, c = 10, 64
    X = _correlated_x(rng, 300, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    H = ref.hessian(X)
    a = ref.gptq_quantize(W0, H, bits=4, groupsize=-1)
    b = ref.gptq_quantize(W0, H, bits=4, groupsize=c)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["scales"], b["scales"])


# --- P13: invariances (H shared by every row; scale of H irrelevant) ---
def test_scaling_inputs_and_permuting_rows():
    rng = np.random.default_rng(17)
    r, c = 12, 40
    X = _correlated_x(rng, 120, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    a = ref.gptq_quantize(W0, ref.hessian(X), bits=4, groupsize=8)
    b = ref.gptq_quantize(W0, ref.hessian(2.0 * X), bits=4, groupsize=8)
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(a["w_hat"], b["w_hat"])
    rp = rng.permutation(r)
    p = ref.gptq_quantize(W0[rp], ref.hessian(X), bits=4, groupsize=8)
    np.testing.assert_array_equal(p["codes"], a["codes"][rp])
    np.testing.assert_array_equal(p["row_loss"], a["row_loss"][rp])


# --- dead inputs ("Paper vs. code": silent inputs zeroed) ---
def test_dead_inputs_zeroed_and_per_row_ruler_sees_original():
    rng = np.random.default_rng(18)
    r, c = 6, 16
    X = _correlated_x(rng, 100, c)
    X[:, 3] = 0.0
    W0 = rng.standard_normal((r, c)) * 0.02
    W0[0, 3] = 1.0                              # dominates row 0's range
    out = ref.gptq_quantize(W0, ref.hessian(X), bits=4)
    assert out["dead"][3] and out["dead"].sum() == 1
    assert np.all(out["w_hat"][:, 3] == 0.0)
    np.testing.assert_array_equal(out["codes"][:, 3], out["zeros"][:, 0])
    s_row, _, _ = ref.fit_ruler(W0[:1], 4)
    assert out["scales"][0, 0] == s_row[0]      # range still includes the 1.0
    # The dead diagonal is set to 1 before damping, so it enters the mean.
    H = ref.hessian(X)
    assert out["lam"] == pytest.approx(0.01 * (np.trace(H) + 1.0) / c, rel=1e-14)


# --- tie replay adjudication ---
# The parity procedure: at a near-tie (the pre-rounding value within 1e-3 of a
# tick midpoint) both neighbouring ticks are the nearest tick up to rounding
# order ("What quantization is, and why anyone bothers": each weight goes to
# its nearest tick), so another implementation's choice of the other
# neighbour is adopted; anything else is a hard mismatch.  These pins build
# the pre-rounding values by hand, so every branch asserts something.
def test_tie_replay_identical_codes_change_nothing():
    rng = np.random.default_rng(19)
    r, c = 6, 32
    X = _correlated_x(rng, 100, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    H = ref.hessian(X)
    base = ref.gptq_quantize(W0, H, bits=4)
    same = ref.TieReplay(base["codes_proc"], base["zeros"])
    again = ref.gptq_quantize(W0, H, bits=4, replay=same)
    assert same.hard == 0 and same.near_ties == 0
    assert same.zero_hard == 0 and same.zero_near_ties == 0
    np.testing.assert_array_equal(again["codes"], base["codes"])


def _adjudicate_codes(t, theirs, zero, maxq=15, band=1e-3):
    """One column through TieReplay.code with hand-made pre-rounding values t."""
    t = np.asarray(t, np.float32)
    theirs = np.asarray(theirs, np.int64)
    n = t.size
    zero = np.broadcast_to(np.asarray(zero, np.float64), (n,)).copy()
    rep = ref.TieReplay(theirs.reshape(n, 1), band=band)
    mine = np.clip(np.rint(t.astype(np.float64)) + zero, 0, maxq)
    out = rep.code(np.arange(n), 0, mine, t, zero, maxq)
    return mine, out, rep


def test_tie_replay_adopts_the_other_neighbour_at_a_near_tie():
    # zero 3; t = 4.5 +- 4e-4 and 6.5 + 9e-4 (inside the band of 1e-3).
    t = [4.5 + 4e-4, 4.5 - 4e-4, 6.5 + 9e-4]
    mine, _, _ = _adjudicate_codes(t, [0, 0, 0], 3)
    np.testing.assert_array_equal(mine, [8, 7, 10])          # the oracle's own picks
    theirs = [7, 8, 9]                                       # the other neighbour each time
    _, out, rep = _adjudicate_codes(t, theirs, 3)
    np.testing.assert_array_equal(out, theirs)
    assert rep.near_ties == 3 and rep.hard == 0


def test_tie_replay_rejects_a_neighbour_away_from_a_midpoint():
    # A neighbouring tick is not a valid choice when t is far from a midpoint,
    # nor just outside the band (1.5e-3 and 2e-3 away).
    t = [4.3, 4.7, 4.5 + 2e-3, 4.5 - 1.5e-3]
    mine, _, _ = _adjudicate_codes(t, [0, 0, 0, 0], 3)
    np.testing.assert_array_equal(mine, [7, 8, 8, 7])
    _, out, rep = _adjudicate_codes(t, [8, 7, 7, 8], 3)
    np.testing.assert_array_equal(out, mine)                  # the oracle keeps its own
    assert rep.hard == 4 and rep.near_ties == 0


def test_tie_replay_rejects_a_non_neighbour_at_a_near_tie():
    # t = 4.5 exactly: the neighbours are 4 and 5 (codes 7 and 8 with zero 3);
    # codes two ticks away are never valid.
    t = [4.5, 4.5, 4.5 + 1e-4, 4.5 - 1e-4]
    mine, _, _ = _adjudicate_codes(t, [0] * 4, 3)
    _, out, rep = _adjudicate_codes(t, [9, 6, 10, 5], 3)
    np.testing.assert_array_equal(out, mine)
    assert rep.hard == 4 and rep.near_ties == 0


def test_tie_replay_neighbours_are_clamped_to_the_grid():
    # zero 8, 4 bits: t = 7.5 sits between ticks 15 and 16, and 16 clamps to
    # 15, so only 15 is valid; at the bottom t = -8.5 gives -1 and 0 -> 0.
    t = [7.5 + 1e-4, -8.5 + 1e-4, 6.5 + 1e-4]
    mine, _, _ = _adjudicate_codes(t, [0] * 3, 8)
    np.testing.assert_array_equal(mine, [15, 0, 15])
    _, out, rep = _adjudicate_codes(t, [14, 1, 14], 8)
    # 14 is a neighbour of 6.5 (ticks 14 and 15) but not of 7.5; 1 is not a
    # neighbour of -8.5 once clamped.
    np.testing.assert_array_equal(out, [15, 0, 14])
    assert rep.near_ties == 1 and rep.hard == 2


def _adjudicate_zero(zt, theirs, band=1e-3):
    zt = np.asarray(zt, np.float32)
    n = zt.size
    rep = ref.TieReplay(np.zeros((n, 1), np.int64), zeros=np.asarray(theirs).reshape(n, 1), band=band)
    mine = np.rint(zt.astype(np.float64))
    return mine, rep.zero(np.arange(n), 0, mine, zt), rep


def test_tie_replay_zero_point_branch():
    # Adopted: -min/scale within the band of a half-integer, other neighbour.
    zt = [9.5 + 3e-4, 9.5 - 3e-4]
    mine, out, rep = _adjudicate_zero(zt, [9, 10])
    np.testing.assert_array_equal(mine, [10, 9])
    np.testing.assert_array_equal(out, [9, 10])
    assert rep.zero_near_ties == 2 and rep.zero_hard == 0
    # Hard: a neighbour far from the midpoint, outside the band, and a
    # non-neighbour at the midpoint.
    zt = [9.2, 9.5 + 2e-3, 9.5 + 1e-4, 9.5 - 1e-4]
    mine, out, rep = _adjudicate_zero(zt, [10, 9, 11, 8])
    np.testing.assert_array_equal(out, mine)
    assert rep.zero_hard == 4 and rep.zero_near_ties == 0
    # The code counters are untouched by the zero branch, and no zeros given
    # means nothing to adjudicate.
    assert rep.hard == 0 and rep.near_ties == 0
    none = ref.TieReplay(np.zeros((1, 1), np.int64))
    assert none.zero(np.arange(1), 0, np.array([4.0]), np.array([4.5], np.float32))[0] == 4.0


def test_tie_replay_adopted_code_flows_into_the_outputs():
    # H = 8 I: no repairs, so each pre-rounding value is the weight itself.
    # Row 0's column 5 is placed 2e-4 above a midpoint; an implementation
    # that picked the lower neighbour is adopted there and nowhere else.
    rng = np.random.default_rng(23)
    r, c = 3, 16
    W0 = rng.uniform(-0.7, 0.3, size=(r, c))
    W0[:, 0], W0[:, 1] = -0.8, 0.4                            # rulers: scale 0.08, zero 10
    scale = np.float32(0.8 + 0.4) / np.float32(15)
    W0[0, 5] = float(np.float32((2.5 + 2e-4) * float(scale)))
    H = 8.0 * np.eye(c)
    base = ref.gptq_quantize(W0, H, bits=4, percdamp=0.0)
    assert base["codes"][0, 5] == 13
    theirs = base["codes_proc"].copy()
    theirs[0, 5] = 12
    rep = ref.TieReplay(theirs, base["zeros"])
    out = ref.gptq_quantize(W0, H, bits=4, percdamp=0.0, replay=rep)
    assert rep.near_ties == 1 and rep.hard == 0
    np.testing.assert_array_equal(out["codes"], theirs)
    assert out["w_hat"][0, 5] == pytest.approx(float(scale) * 2, rel=1e-7)


# --- P14: packed layout (this project's layout; the pages fix none) ---
def test_pack_layout_closed_forms_and_round_trip():
    # 4 bits: code k of a word sits in hex digit k.
    w4 = ref.pack_codes(np.arange(8)[None], 4)
    assert int(w4[0, 0]) == 0x76543210
    # 3 bits: codes k % 8 for k = 0..31 over 96 little-endian bits; the 24-bit
    # pattern 0xFAC688 (codes 0..7) repeats four times.
    w3 = ref.pack_codes((np.arange(32) % 8)[None], 3)
    assert [int(x) for x in w3[0]] == [0x88FAC688, 0xC688FAC6, 0xFAC688FA]
    rng = np.random.default_rng(20)
    for bits, c in ((4, 64), (3, 96)):
        codes = rng.integers(0, 2 ** bits, size=(5, c))
        words = ref.pack_codes(codes, bits)
        assert words.nbytes == 5 * c * bits // 8
        np.testing.assert_array_equal(ref.unpack_codes(words, bits, c), codes)


# --- symmetric grid (the pages name the option without a formula; reading:
# range [-m, m], m = max|w|, scale = 2m/(2^b - 1), zero = the middle tick) ---
def test_symmetric_grid_closed_form():
    w = np.array([[-0.8, 0.4, 0.0, 0.05]])
    scale, zero, zt = ref.fit_ruler(w, 4, sym=True)
    s32 = np.float32(np.float32(1.6) / np.float32(15.0))     # 2m / 15 in fp32
    assert scale[0] == s32 and zero[0] == 8.0 and zt[0] == 8.0
    q, t = ref.round_to_grid(w[0], scale[0], zero[0], 4)
    # -0.8 / s = -7.5 -> rne -8 -> code 0;  0.4 / s = 3.75 -> 4 -> 12;  0 -> 8
    np.testing.assert_array_equal(q[:3], [0.0, 12.0, 8.0])
    assert ref.dequantize(np.float64(8.0), scale[0], 8.0) == 0.0      # 0 exactly on a tick
    # the asymmetric ruler of the same row differs (the page's example grid)
    a_scale, a_zero, _ = ref.fit_ruler(w, 4)
    assert a_zero[0] == 10.0 and a_scale[0] != scale[0]


def test_symmetric_grid_is_odd_up_to_the_extra_negative_tick():
    rng = np.random.default_rng(31)
    w = rng.standard_normal((6, 50)) * 0.03
    for bits in (2, 3, 4, 8):
        s1, z1, _ = ref.fit_ruler(w, bits, sym=True)
        s2, z2, _ = ref.fit_ruler(-w, bits, sym=True)
        np.testing.assert_array_equal(s1, s2)
        np.testing.assert_array_equal(z1, z2)
        assert np.all(z1 == 2 ** (bits - 1))
        for i in range(w.shape[0]):
            q1, t1 = ref.round_to_grid(w[i], s1[i], z1[i], bits)
            q2, _ = ref.round_to_grid(-w[i], s2[i], z2[i], bits)
            inner = np.abs(t1) < 2 ** (bits - 1) - 0.5 - 1e-3   # no clamp, no tie
            np.testing.assert_array_equal(q2[inner], 2 * z1[i] - q1[inner])


@pytest.mark.parametrize("groupsize", [-1, 16])
def test_symmetric_identity_hessian_is_round_to_nearest(groupsize):
    rng = np.random.default_rng(32)
    W0 = rng.standard_normal((13, 48)) * 0.02
    out = ref.gptq_quantize(W0, ref.hessian(2.0 * np.eye(48)), bits=4, groupsize=groupsize, sym=True)
    codes, w_hat = ref.rtn(W0, 4, groupsize, sym=True)
    np.testing.assert_array_equal(out["codes"], codes)
    np.testing.assert_array_equal(out["w_hat"], w_hat)
    assert np.all(out["zeros"] == 8)


def test_symmetric_tiny_layers_against_brute_force():
    rng = np.random.default_rng(33)
    for _ in range(20):
        d = int(rng.integers(3, 6))
        X = _correlated_x(rng, 24, d, mix=0.8)
        w0 = rng.standard_normal(d) * 0.1
        out = ref.gptq_quantize(w0[None], ref.hessian(X), bits=3, sym=True)
        scale, zero = out["scales"][0, 0], out["zeros"][0, 0]
        assert zero == 4
        _, best = ref.brute_force_row(w0, X, scale, zero, 3)
        assert best <= ref.layer_loss_from_x(w0[None], out["w_hat"], X) * (1 + 1e-12)


# --- dequantize-on-the-fly product over the packed layer ---
def test_dequant_gemv_closed_form():
    # one row, 8 columns, 4 bits, two groups of 4: codes 0..7, rulers (0.5, 2) and (0.25, 5)
    words = ref.pack_codes(np.arange(8)[None], 4)
    scales = np.array([[0.5, 0.25]], np.float32)
    zeros = np.array([[2, 5]])
    x = np.array([1.0, -1.0, 2.0, 0.5, 4.0, 1.0, -2.0, 3.0])
    # w_hat = 0.5*(0..3 - 2) = [-1, -0.5, 0, 0.5]; 0.25*(4..7 - 5) = [-0.25, 0, 0.25, 0.5]
    expect = (-1 * 1 + -0.5 * -1 + 0 * 2 + 0.5 * 0.5) + (-0.25 * 4 + 0 * 1 + 0.25 * -2 + 0.5 * 3)
    y = ref.dequant_gemv(words, 4, 8, scales, zeros, [0, 0, 0, 0, 1, 1, 1, 1], x)
    assert y[0] == expect == -0.25


@pytest.mark.parametrize("bits,groupsize,act_order", [(4, 16, False), (3, 32, True), (4, -1, True), (3, -1, False)])
def test_dequant_gemv_matches_the_quantizers_w_hat(bits, groupsize, act_order):
    rng = np.random.default_rng(40 + bits)
    r, c = 7, 64
    X = _correlated_x(rng, 150, c)
    W0 = rng.standard_normal((r, c)) * 0.02
    out = ref.gptq_quantize(W0, ref.hessian(X), bits=bits, groupsize=groupsize, act_order=act_order)
    words = ref.pack_codes(out["codes"], bits)
    x = rng.standard_normal(c)
    y = ref.dequant_gemv(words, bits, c, out["scales"], out["zeros"], out["g_idx"], x)
    np.testing.assert_allclose(y, out["w_hat"] @ x, rtol=1e-12, atol=1e-15)


# --- Hadamard pre-rotation ---
def test_hadamard_small_orders_written_out():
    np.testing.assert_array_equal(ref.hadamard(1), [[1]])
    np.testing.assert_array_equal(ref.hadamard(2), [[1, 1], [1, -1]])
    np.testing.assert_array_equal(ref.hadamard(4), [[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("n", [8, 64, 256])
def test_hadamard_rows_are_perpendicular_and_pm1(n):
    H = ref.hadamard(n)
    assert set(np.unique(H)) == {-1.0, 1.0}
    np.testing.assert_array_equal(H @ H.T, n * np.eye(n))
    np.testing.assert_array_equal(H, H.T)


def test_rotation_leaves_the_layer_product_unchanged():
    rng = np.random.default_rng(9)
    W = rng.standard_normal((5, 96))       # 96 = 3 * 32: block 32
    x = rng.standard_normal(96)
    Wr = ref.hadamard_rotate(W)
    xr = ref.hadamard_rotate(x[None])[0]
    np.testing.assert_allclose(Wr @ xr, W @ x, rtol=1e-12, atol=1e-12)
    # rotation preserves each row's norm and the Hessian's eigen-structure: H_r = Q H Q^T
    np.testing.assert_allclose(np.linalg.norm(Wr, axis=1), np.linalg.norm(W, axis=1), rtol=1e-13)
    X = rng.standard_normal((40, 96))
    Xr = ref.hadamard_rotate(X)
    np.testing.assert_allclose(np.linalg.eigvalsh(ref.hessian(Xr)), np.linalg.eigvalsh(ref.hessian(X)),
                               rtol=1e-10, atol=1e-9)


def test_rotation_spreads_a_lone_outlier():
    x = np.zeros((1, 64))
    x[0, 17] = 100.0
    y = ref.hadamard_rotate(x)
    np.testing.assert_allclose(np.abs(y), 100.0 / 8.0)     # every entry +-100 / sqrt(64)
    assert np.max(np.abs(y)) < np.max(np.abs(x)) / 7.9


def test_rotation_blocks_and_default_block():
    assert ref.default_hadamard_block(4096) == 4096
    assert ref.default_hadamard_block(11008) == 256
    assert ref.default_hadamard_block(12288) == 4096
    rng = np.random.default_rng(2)
    A = rng.standard_normal((3, 48))
    B = ref.hadamard_rotate(A, 16)
    for k in range(3):                    # block-diagonal: each 16-block on its own
        np.testing.assert_allclose(B[:, 16 * k:16 * (k + 1)], A[:, 16 * k:16 * (k + 1)] @ ref.hadamard(16) / 4.0,
                                   rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(ref.hadamard_rotate(B, 16), A, rtol=1e-12, atol=1e-12)   # Q^2 = I (symmetric, orthogonal)


# --- layer-by-layer pass ---
def test_round16_agrees_with_torch_single_rounding():
    import torch
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(20000) * np.exp(rng.uniform(-30, 30, 20000))).astype(np.float32)
    for dt, tdt in (("bfloat16", torch.bfloat16), ("float16", torch.float16)):
        want = torch.from_numpy(x32).to(tdt).to(torch.float64).numpy()
        got = ref.round16(x32.astype(np.float64), dt)
        np.testing.assert_array_equal(got, want)
    # ties to even, written out
    assert ref.round16(1 + 2.0 ** -8, "bfloat16") == 1.0
    assert ref.round16(1 + 3 * 2.0 ** -8, "bfloat16") == 1 + 2.0 ** -6
    assert ref.round16(2.0 ** -25, "float16") == 0.0 and ref.round16(3 * 2.0 ** -25, "float16") == 2.0 ** -23


def test_linear_forward_closed_form():
    X = np.array([[1.0, 2.0], [-1.0, 0.5]])
    W = np.array([[0.5, 0.25], [1.0, -1.0], [2.0, 0.0]])      # all exact in bf16
    np.testing.assert_array_equal(ref.linear_forward(X, W, "bfloat16"), [[1.0, -1.0, 2.0], [-0.375, -1.5, -2.0]])
    G = np.array([[0.0, 1.0, -2.0], [3.0, 0.0, 1.0]])
    s = lambda g: g / (1 + np.exp(-g))
    want = np.array([[0.0, s(1.0) * -1.0, s(-2.0) * 2.0], [s(3.0) * -0.375, 0.0, s(1.0) * -2.0]])
    np.testing.assert_allclose(ref.linear_forward(X, W, "bfloat16", gate=G), want, rtol=1e-15)
    assert ref.silu(0.0) == 0.0 and abs(ref.silu(40.0) - 40.0) < 1e-12 and abs(ref.silu(-40.0)) < 1e-15


def _stack(rng, d, h, nb):
    return [(rng.standard_normal((h, d)) * 0.05, rng.standard_normal((h, d)) * 0.05, rng.standard_normal((d, h)) * 0.05)
            for _ in range(nb)]


def test_stack_calibrates_each_layer_on_quantized_outputs():
    rng = np.random.default_rng(12)
    d, h, n = 16, 24, 300
    X0 = ref.round16(rng.standard_normal((n, d)), "bfloat16")
    blocks = _stack(rng, d, h, 2)
    recs, Xout = ref.quantize_mlp_stack(X0, blocks, bits=3)
    r0, r1 = recs
    # down's calibration input is silu(gate) * up of the QUANTIZED gate and up
    G = ref.round16(X0 @ ref.round16(r0["gate"]["w_hat"], "bfloat16").T, "bfloat16")
    U = ref.round16(X0 @ ref.round16(r0["up"]["w_hat"], "bfloat16").T, "bfloat16")
    np.testing.assert_array_equal(r0["Z"], ref.round16(ref.silu(G) * U, "bfloat16"))
    # ... and differs from what the float weights would give
    Gf = ref.round16(X0 @ ref.round16(blocks[0][0], "bfloat16").T, "bfloat16")
    assert np.abs(Gf - G).max() > 1e-3
    # block 2 reads block 1's quantized output; the next H is that input's
    np.testing.assert_array_equal(r1["X"], ref.round16(r0["Z"] @ ref.round16(r0["down"]["w_hat"], "bfloat16").T,
                                                       "bfloat16"))
    np.testing.assert_allclose(r1["H"], ref.hessian(r1["X"]), rtol=1e-12)
    # gate and up share the block's Hessian: each equals a stand-alone GPTQ on it
    np.testing.assert_array_equal(r0["up"]["codes"], ref.gptq_quantize(blocks[0][1], r0["H"], 3)["codes"])
    assert Xout.shape == (n, d)


def test_stack_with_fine_grid_tracks_the_float_stack():
    rng = np.random.default_rng(13)
    d, h, n = 16, 32, 400
    X0 = ref.round16(rng.standard_normal((n, d)), "bfloat16")
    blocks = _stack(rng, d, h, 2)
    _, Xq = ref.quantize_mlp_stack(X0, blocks, bits=8)
    X = X0
    for Wg, Wu, Wd in blocks:
        Z = ref.silu(X @ Wg.T) * (X @ Wu.T)
        X = Z @ Wd.T
    assert np.linalg.norm(Xq - X) / np.linalg.norm(X) < 0.02
    _, X3 = ref.quantize_mlp_stack(X0, blocks, bits=3)
    assert np.linalg.norm(X3 - X) > np.linalg.norm(Xq - X)          # coarser grid, larger drift


"""Pins of the oracle's query compression, output projection and the two folds.

Each pin checks the oracle against something other than its own formula: pure-Python
loops on tiny inputs, and closed forms where a weight is an identity or a selection.
"""
import numpy as np

from oracle import mla_oracle as O


def _tiny(seed=0, M=2, d_model=5, d_cq=4, n_h=3, d_h=2, d_r=2, d_c=3):
    rng = np.random.default_rng(seed)
    return dict(x=rng.normal(size=(M, d_model)), w_dq=rng.normal(size=(d_model, d_cq)),
                w_uq=rng.normal(size=(d_cq, n_h, d_h)), w_qr=rng.normal(size=(d_cq, n_h, d_r)),
                w_uk=rng.normal(size=(n_h, d_h, d_c)), w_uv=rng.normal(size=(n_h, d_c, d_h)),
                w_o=rng.normal(size=(n_h * d_h, d_model)), o_lat=rng.normal(size=(M, n_h, d_c)))


def pin_query_brute_force():
    t = _tiny()
    q_nope, q_rope = O.query_from_hidden(t["x"], t["w_dq"], t["w_uq"], t["w_qr"])
    M, d_model = t["x"].shape
    d_cq, n_h, d_h = t["w_uq"].shape
    d_r = t["w_qr"].shape[2]
    for m in range(M):
        c = [sum(t["x"][m, i] * t["w_dq"][i, k] for i in range(d_model)) for k in range(d_cq)]
        for h in range(n_h):
            for j in range(d_h):
                assert abs(q_nope[m, h, j] - sum(c[k] * t["w_uq"][k, h, j] for k in range(d_cq))) < 1e-12
            for j in range(d_r):
                assert abs(q_rope[m, h, j] - sum(c[k] * t["w_qr"][k, h, j] for k in range(d_cq))) < 1e-12


def pin_fold_query_selection():
    # d_cq = n_h * d_h and w_uq the selection c_q[h d_h + j] -> head h dim j: the fold is
    # W_UK itself, head by head.
    t = _tiny(n_h=3, d_h=2, d_cq=6)
    n_h, d_h, d_c = t["w_uk"].shape
    sel = np.zeros((n_h * d_h, n_h, d_h))
    for h in range(n_h):
        for j in range(d_h):
            sel[h * d_h + j, h, j] = 1.0
    f = O.fold_query_weights(sel, t["w_uk"])
    for h in range(n_h):
        np.testing.assert_array_equal(f[h * d_h:(h + 1) * d_h, h, :], t["w_uk"][h])
        other = np.delete(np.arange(n_h * d_h), np.arange(h * d_h, (h + 1) * d_h))
        assert np.all(f[other, h, :] == 0)


def pin_fold_query_brute_force():
    t = _tiny(1)
    f = O.fold_query_weights(t["w_uq"], t["w_uk"])
    d_cq, n_h, d_h = t["w_uq"].shape
    d_c = t["w_uk"].shape[2]
    for k in range(d_cq):
        for h in range(n_h):
            for c in range(d_c):
                want = sum(t["w_uq"][k, h, j] * t["w_uk"][h, j, c] for j in range(d_h))
                assert abs(f[k, h, c] - want) < 1e-12


def pin_output_identity_and_brute_force():
    t = _tiny(2)
    M, n_h, d_h = 2, 3, 2
    o = np.random.default_rng(5).normal(size=(M, n_h, d_h))
    # identity W_O (d_model = n_h d_h): the output is the concatenation of the heads
    np.testing.assert_array_equal(O.output_projection(o, np.eye(n_h * d_h)), o.reshape(M, -1))
    y = O.output_projection(o, t["w_o"])
    for m in range(M):
        for dd in range(t["w_o"].shape[1]):
            want = sum(o[m, h, j] * t["w_o"][h * d_h + j, dd] for h in range(n_h) for j in range(d_h))
            assert abs(y[m, dd] - want) < 1e-12


def pin_fold_output_brute_force():
    t = _tiny(3)
    f = O.fold_output_weights(t["w_uv"], t["w_o"])
    n_h, d_c, d_h = t["w_uv"].shape
    for h in range(n_h):
        for c in range(d_c):
            for dd in range(t["w_o"].shape[1]):
                want = sum(t["w_uv"][h, c, j] * t["w_o"][h * d_h + j, dd] for j in range(d_h))
                assert abs(f[h, c, dd] - want) < 1e-12


def test_query_brute_force():
    pin_query_brute_force()


def test_fold_query_selection():
    pin_fold_query_selection()


def test_fold_query_brute_force():
    pin_fold_query_brute_force()


def test_output_identity_and_brute_force():
    pin_output_identity_and_brute_force()


def test_fold_output_brute_force():
    pin_fold_output_brute_force()


def test_folds_agree_with_the_unfolded_chain():
    """Associativity: the folded and unfolded routes give the same latent query and output
    ([Dispatch] associative property), checked on independent random inputs."""
    t = _tiny(4, M=3, d_model=6, d_cq=5, n_h=2, d_h=3, d_r=2, d_c=4)
    q_nope, _ = O.query_from_hidden(t["x"], t["w_dq"], t["w_uq"], t["w_qr"])
    q_lat = O.absorb_query(q_nope[:, None], t["w_uk"])[:, 0]
    c_q = t["x"] @ t["w_dq"]
    q_lat_f = np.einsum("mk,khc->mhc", c_q, O.fold_query_weights(t["w_uq"], t["w_uk"]))
    np.testing.assert_allclose(q_lat_f, q_lat, rtol=1e-12, atol=1e-12)
    o_lat = t["o_lat"][:, None]
    y = O.output_projection(O.absorb_output(o_lat, t["w_uv"])[:, 0], t["w_o"])
    y_f = np.einsum("mhc,hcd->md", t["o_lat"], O.fold_output_weights(t["w_uv"], t["w_o"]))
    np.testing.assert_allclose(y_f, y, rtol=1e-12, atol=1e-12)

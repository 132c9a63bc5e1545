"""Pins of the oracle's Recolor fit (moment-matched affine map).

"Prefill-Free Cross-Family KV Cache Transfer ..." (Key Contributions 2,
Methodology in Plain English 3): both feature spaces whitened, aligned by a
Procrustes solution, receiver means and covariances restored.  Each pin
follows from the mathematics, not from the oracle's own formula:

* a planted exact linear relation Y = X A + c (A of full column rank) is
  recovered exactly: its whitened cross-covariance is already orthonormal;
* the translated calibration rows have the receiver's mean and covariance
  (the moment matching the method is named for);
* one feature in and out: w = sign(cov) * sd_y / sd_x;
* the result does not depend on which whitening is used (Cholesky factors
  instead of symmetric square roots give the same map);
* with both sides already white, the map is the orthogonal Procrustes
  rotation that scipy computes;
* the regulariser is relative: scaling X by a scales W by 1/a.
"""
import numpy as np
import pytest
import scipy.linalg

from oracle import kvx_oracle as O


def _rand(rng, *shape):
    return rng.standard_normal(shape)


@pytest.mark.parametrize("f_in,f_out", [(6, 6), (9, 4), (24, 8)])
def test_recolor_recovers_planted_linear_map(f_in, f_out):
    rng = np.random.default_rng(f_in * 10 + f_out)
    n = 400
    x = _rand(rng, n, f_in) @ _rand(rng, f_in, f_in) + _rand(rng, f_in)  # correlated, offset
    a = _rand(rng, f_in, f_out)
    c = _rand(rng, f_out)
    y = x @ a + c
    w, b = O.recolor_fit(x, y)
    assert np.max(np.abs(w - a)) <= 1e-9 * np.max(np.abs(a))
    assert np.max(np.abs(b - c)) <= 1e-8


@pytest.mark.parametrize("f_in,f_out", [(5, 5), (12, 3), (40, 16)])
def test_recolor_matches_receiver_moments(f_in, f_out):
    rng = np.random.default_rng(3 + f_in)
    n = 300
    x = _rand(rng, n, f_in) * rng.uniform(0.5, 3.0, f_in) + 2.0
    y = _rand(rng, n, f_out) @ _rand(rng, f_out, f_out) - 1.0  # unrelated to x
    w, b = O.recolor_fit(x, y)
    t = x @ w + b
    my = y.mean(axis=0)
    cy = (y - my).T @ (y - my) / n
    ct = (t - t.mean(axis=0)).T @ (t - t.mean(axis=0)) / n
    assert np.max(np.abs(t.mean(axis=0) - my)) <= 1e-10 * (1 + np.max(np.abs(my)))
    assert np.max(np.abs(ct - cy)) <= 1e-10 * np.max(np.abs(cy))


def test_recolor_scalar_closed_form():
    rng = np.random.default_rng(11)
    x = rng.normal(3.0, 2.0, size=(50, 1))
    for sign in (1.0, -1.0):
        y = sign * 0.7 * x + rng.normal(0.0, 1.5, size=(50, 1)) - 4.0
        w, b = O.recolor_fit(x, y)
        cov = np.mean((x - x.mean()) * (y - y.mean()))
        want = np.sign(cov) * y.std() / x.std()
        assert w.shape == (1, 1) and abs(w[0, 0] - want) <= 1e-12 * abs(want)
        assert abs(b[0] - (y.mean() - x.mean() * want)) <= 1e-12 * 10


def test_recolor_independent_of_whitening_choice():
    """Whitening by the inverse Cholesky factors (any A with A^T S A = I)
    gives the same map: W is unchanged when the whitening is rotated."""
    rng = np.random.default_rng(5)
    n, f_in, f_out = 200, 10, 4
    x = _rand(rng, n, f_in) @ _rand(rng, f_in, f_in)
    y = _rand(rng, n, f_out) @ _rand(rng, f_out, f_out) + 0.3 * x[:, :f_out]
    w, b = O.recolor_fit(x, y)
    xc, yc = x - x.mean(0), y - y.mean(0)
    lx = np.linalg.cholesky(xc.T @ xc / n)
    ly = np.linalg.cholesky(yc.T @ yc / n)
    ax = np.linalg.inv(lx).T          # A_x^T S_xx A_x = I
    ay = np.linalg.inv(ly).T
    u, _, vt = np.linalg.svd(ax.T @ (xc.T @ yc / n) @ ay, full_matrices=False)
    w2 = ax @ (u @ vt) @ ly.T         # A_y^-1 = L_y^T
    assert np.max(np.abs(w - w2)) <= 1e-10 * np.max(np.abs(w))


def test_recolor_white_sides_is_orthogonal_procrustes():
    rng = np.random.default_rng(9)
    n, f = 120, 6

    def white(m):
        m = m - m.mean(axis=0)
        q, _ = np.linalg.qr(m)
        return q * np.sqrt(n)        # zero mean, covariance exactly I

    x = white(_rand(rng, n, f))
    y = white(x @ _rand(rng, f, f) + 0.5 * _rand(rng, n, f))
    w, b = O.recolor_fit(x, y)
    r, _ = scipy.linalg.orthogonal_procrustes(x, y)
    assert np.max(np.abs(w - r)) <= 1e-10
    assert np.max(np.abs(b)) <= 1e-10


def test_recolor_regulariser_is_relative():
    """rho * trace(S)/F scales with the data: X -> a X gives W -> W / a (and
    the same b); a singular S_xx (a duplicated column) is fitted with rho > 0
    and its two copies get equal weight rows."""
    rng = np.random.default_rng(21)
    n = 80
    x = _rand(rng, n, 7)
    x = np.concatenate([x, x[:, 2:3]], axis=1)  # duplicated column: S_xx singular
    y = _rand(rng, n, 3) + 0.5 * x[:, :3]
    with pytest.raises(np.linalg.LinAlgError):
        O.recolor_fit(x, y)
    w, b = O.recolor_fit(x, y, rho_x=1e-3)
    w2, b2 = O.recolor_fit(8.0 * x, y, rho_x=1e-3)
    assert np.max(np.abs(w2 * 8.0 - w)) <= 1e-10 * np.max(np.abs(w))
    assert np.max(np.abs(b2 - b)) <= 1e-10
    assert np.max(np.abs(w[2] - w[7])) <= 1e-10 * np.max(np.abs(w))

"""Pins for the fp64 oracle: each check is an independent route to a value the
pages and the mathematics fix.  None of these re-use the oracle's loop.

Every check takes an oracle object (``.scan`` / ``.step``) and raises
AssertionError on a mismatch, so the same checks can be run against mutated
copies of the oracle to show that they catch plausible mistakes.
"""
from __future__ import annotations

import numpy as np
import scipy.signal
import scipy.special

RTOL = 1e-12


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    scale = max(np.max(np.abs(b)), 1e-300)
    return float(np.max(np.abs(a - b)) / scale)


def _softplus(x):
    return np.logaddexp(0.0, x)          # library route, independent of log1p(exp(-|x|))


def _silu(z):
    return z * scipy.special.expit(z)


def tiny_inputs(seed, Bsz=2, Dm=3, N=4, L=40, gate=True, skip=True, bias=True, h0=False):
    rng = np.random.default_rng(seed)
    inp = dict(
        u=rng.standard_normal((Bsz, Dm, L)),
        delta=0.5 * rng.standard_normal((Bsz, Dm, L)),
        A=-rng.uniform(0.2, 3.0, (Dm, N)),
        B=rng.standard_normal((Bsz, N, L)),
        C=rng.standard_normal((Bsz, N, L)),
        D=rng.standard_normal(Dm) if skip else None,
        z=rng.standard_normal((Bsz, Dm, L)) if gate else None,
        delta_bias=rng.uniform(-3.0, 0.5, Dm) if bias else None,
    )
    if h0:
        inp["h0"] = rng.standard_normal((Bsz, Dm, N))
    return inp


def brute_force(u, delta, A, B, C, D=None, z=None, delta_bias=None, h0=None, product="prod"):
    """Unrolled sums: h_t = sum_{s<=t} (prod_{r=s+1..t} Abar_r) Bbar_s u_s (+ prod_{r<=t} Abar_r h0),
    y_t = C_t . h_t + D u_t, out_t = y_t * silu(z_t).  product='prod' multiplies the Abar
    factors one by one, product='sum' uses exp(A * sum of dt)."""
    Bsz, Dm, L = u.shape
    N = A.shape[1]
    out = np.zeros((Bsz, Dm, L))
    hL = np.zeros((Bsz, Dm, N))
    for b in range(Bsz):
        for d in range(Dm):
            x = delta[b, d] + (delta_bias[d] if delta_bias is not None else 0.0)
            dt = _softplus(x)
            abar = np.exp(np.outer(dt, A[d]))            # [L, N]
            bbar = dt[:, None] * B[b].T                  # [L, N]
            cum = np.concatenate([[0.0], np.cumsum(dt)])
            for t in range(L):
                h = np.zeros(N)
                for s in range(t + 1):
                    if product == "prod":
                        w = np.prod(abar[s + 1:t + 1], axis=0)
                    else:
                        w = np.exp(A[d] * (cum[t + 1] - cum[s + 1]))
                    h += w * bbar[s] * u[b, d, s]
                if h0 is not None:
                    w0 = np.prod(abar[:t + 1], axis=0) if product == "prod" else np.exp(A[d] * cum[t + 1])
                    h += w0 * h0[b, d]
                y = float(C[b, :, t] @ h)
                if D is not None:
                    y += D[d] * u[b, d, t]
                if z is not None:
                    y *= _silu(z[b, d, t])
                out[b, d, t] = y
                if t == L - 1:
                    hL[b, d] = h
    return out, hL


# ---------------------------------------------------------------- the checks

def check_brute_force(orc):
    for seed, kw in [(1, {}), (2, dict(gate=False)), (3, dict(skip=False, bias=False)),
                     (4, dict(N=1, L=17)), (5, dict(Bsz=1, Dm=1, N=3, L=64))]:
        inp = tiny_inputs(seed, **kw)
        y, h = orc.scan(**inp)
        for prod in ("prod", "sum"):
            yb, hb = brute_force(**inp, product=prod)
            assert rel(y, yb) < 1e-11, ("brute force y", seed, prod, rel(y, yb))
            assert rel(h, hb) < 1e-11, ("brute force state", seed, prod, rel(h, hb))


def check_initial_state(orc):
    inp = tiny_inputs(11, h0=True)
    y, h = orc.scan(**inp)
    yb, hb = brute_force(**inp)
    assert rel(y, yb) < 1e-11 and rel(h, hb) < 1e-11
    # chunking over calls: scan(x[:L1]) then scan(x[L1:], h0 = its final state) == scan(x)
    inp = tiny_inputs(12, L=50)
    y, h = orc.scan(**inp)
    L1 = 23
    cut = lambda k, sl: {key: (v[..., sl] if key in ("u", "delta", "z", "B", "C") and v is not None else v)
                         for key, v in inp.items()}
    y1, h1 = orc.scan(**cut(None, slice(0, L1)))
    y2, h2 = orc.scan(**cut(None, slice(L1, None)), h0=h1)
    assert rel(np.concatenate([y1, y2], -1), y) < 1e-13 and rel(h2, h) < 1e-13


def check_lti_closed_form(orc):
    """Constant dt, B, C: y = silu(z) * (K * u + D u) with K_k = sum_n C[n] Abar[n]^k dtB[n]."""
    rng = np.random.default_rng(21)
    Dm, N, L = 3, 5, 120
    A = -rng.uniform(0.1, 2.0, (Dm, N))
    dl = rng.standard_normal(Dm) * 0.5
    bias = rng.uniform(-2, 0, Dm)
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    u = rng.standard_normal((1, Dm, L))
    z = rng.standard_normal((1, Dm, L))
    Dv = rng.standard_normal(Dm)
    inp = dict(u=u, delta=np.repeat(dl[None, :, None], L, -1), A=A,
               B=np.repeat(Bc[None, :, None], L, -1), C=np.repeat(Cc[None, :, None], L, -1),
               D=Dv, z=z, delta_bias=bias)
    y, h = orc.scan(**inp)
    for d in range(Dm):
        dt = _softplus(dl[d] + bias[d])
        abar = np.exp(dt * A[d])
        k = np.arange(L)
        K = (Cc[None, :] * abar[None, :] ** k[:, None] * (dt * Bc)[None, :]).sum(1)
        conv1 = np.convolve(u[0, d], K)[:L]
        conv2 = scipy.signal.fftconvolve(u[0, d], K)[:L]
        hs = np.stack([scipy.signal.lfilter([dt * Bc[n]], [1.0, -abar[n]], u[0, d]) for n in range(N)])
        conv3 = Cc @ hs
        for ref in (conv1, conv2, conv3):
            ref_y = (ref + Dv[d] * u[0, d]) * _silu(z[0, d])
            assert rel(y[0, d], ref_y) < 1e-10, rel(y[0, d], ref_y)
        assert rel(h[0, d], hs[:, -1]) < 1e-12
        # impulse response h_t = Abar^t dt B u_0
        imp = dict(inp)
        imp["u"] = np.zeros_like(u)
        imp["u"][0, :, 0] = 1.0
        imp["z"] = None
        imp["D"] = None
    yi, _ = orc.scan(**imp)
    for d in range(Dm):
        dt = _softplus(dl[d] + bias[d])
        abar = np.exp(dt * A[d])
        t = np.arange(L)
        expect = (Cc[None, :] * np.exp(np.outer(t, dt * A[d])) * (dt * Bc)[None, :]).sum(1)
        assert rel(yi[0, d], expect) < 1e-12


def check_zoh_library(orc):
    """Exact ZOH B_bar against scipy.signal.cont2discrete on a constant (LTI) diagonal system."""
    rng = np.random.default_rng(31)
    N, L = 4, 60
    A = -rng.uniform(0.1, 2.0, (1, N))
    Bc = rng.standard_normal(N)
    Cc = rng.standard_normal(N)
    dl, bias = 0.3, -0.7
    u = rng.standard_normal((1, 1, L))
    y, h = orc.scan(u, np.full((1, 1, L), dl), A, np.repeat(Bc[None, :, None], L, -1),
                    np.repeat(Cc[None, :, None], L, -1), D=np.array([0.5]), delta_bias=np.array([bias]),
                    zoh=True)
    dt = _softplus(dl + bias)
    Ad, Bd, Cd, Dd, _ = scipy.signal.cont2discrete((np.diag(A[0]), Bc[:, None], Cc[None, :],
                                                    np.array([[0.5]])), dt, method="zoh")
    # y_k = C x_k + D u_k with x_k = Ad x_{k-1} + Bd u_k  (state read after the update)
    x = np.zeros(N)
    ref = np.zeros(L)
    for k in range(L):
        x = Ad @ x + Bd[:, 0] * u[0, 0, k]
        ref[k] = Cd[0] @ x + Dd[0, 0] * u[0, 0, k]
    assert rel(y[0, 0], ref) < 1e-10, rel(y[0, 0], ref)
    # A -> 0 limit of ZOH is the Euler B_bar = dt * B
    inp = tiny_inputs(32)
    inp["A"] = np.zeros_like(inp["A"])
    y1, _ = orc.scan(**inp, zoh=True)
    y2, _ = orc.scan(**inp, zoh=False)
    assert rel(y1, y2) == 0.0


def check_a_zero_cumsum(orc):
    inp = tiny_inputs(41, gate=False, skip=False)
    inp["A"] = np.zeros_like(inp["A"])
    y, h = orc.scan(**inp)
    for b in range(2):
        for d in range(3):
            dt = _softplus(inp["delta"][b, d] + inp["delta_bias"][d])
            hs = np.cumsum(dt[:, None] * inp["B"][b].T * inp["u"][b, d][:, None], axis=0)  # [L, N]
            assert rel(h[b, d], hs[-1]) < 1e-13
            assert rel(y[b, d], (inp["C"][b].T * hs).sum(1)) < 1e-12


def check_small_step_skip(orc):
    """dt -> 0 (bias -40): y = D u silu(z), and y = D u without a gate."""
    inp = tiny_inputs(51)
    inp["delta_bias"] = np.full(3, -40.0)
    y, h = orc.scan(**inp)
    ref = inp["D"][None, :, None] * inp["u"] * _silu(inp["z"])
    assert rel(y, ref) < 1e-14 and np.max(np.abs(h)) < 1e-15
    inp["z"] = None
    y, _ = orc.scan(**inp)
    assert rel(y, inp["D"][None, :, None] * inp["u"]) < 1e-14


def check_single_step_closed_form(orc):
    rng = np.random.default_rng(61)
    for with_h0 in (False, True):
        inp = tiny_inputs(62 + with_h0, L=1, h0=with_h0)
        y, h = orc.scan(**inp)
        dt = _softplus(inp["delta"][..., 0] + inp["delta_bias"][None, :])        # [B, D]
        h_exp = dt[..., None] * inp["B"][:, None, :, 0] * inp["u"][..., 0][..., None]
        if with_h0:
            h_exp = h_exp + np.exp(dt[..., None] * inp["A"][None]) * inp["h0"]
        assert rel(h, h_exp) < 1e-14
        y_exp = ((h_exp * inp["C"][:, None, :, 0]).sum(-1) + inp["D"][None] * inp["u"][..., 0]) \
            * _silu(inp["z"][..., 0])
        assert rel(y[..., 0], y_exp) < 1e-14
    del rng


def check_step_matches_scan(orc):
    """scan(L) equals L single steps, in both discretisations (the scan's ZOH is pinned to
    scipy's cont2discrete and to 60-digit decimal arithmetic near A = 0, so this carries those
    pins over to the step); decays from the workload range and from next to A = 0."""
    for zoh in (False, True):
        for near_zero in (False, True):
            inp = tiny_inputs(71 + 2 * zoh + near_zero, L=20)
            if near_zero:
                inp["A"] = -np.logspace(-7, -3, inp["A"].size).reshape(inp["A"].shape)
            y, h = orc.scan(**inp, zoh=zoh)
            st = np.zeros((2, 3, 4))
            for t in range(20):
                yt, st = orc.step(st, inp["u"][..., t], inp["delta"][..., t], inp["A"], inp["B"][..., t],
                                  inp["C"][..., t], D=inp["D"], z=inp["z"][..., t],
                                  delta_bias=inp["delta_bias"], zoh=zoh)
                assert rel(yt, y[..., t]) < 1e-14, (zoh, near_zero, t)
            assert rel(st, h) < 1e-14, (zoh, near_zero)


def check_step_zoh_closed_form(orc):
    """One ZOH step by hand: delta + bias = 0 gives dt = ln 2 and A = -1 gives A_bar = 1/2, so
    B_bar = (A_bar - 1) / A * B = B / 2 (freeguideonline tutorial, section 2.2).  From h = 3 with
    B = 4, u = 1.5: h' = 3/2 + 2 * 1.5 = 4.5, and y = C h' = 9 for C = 2.  Then a general step
    against scipy's cont2discrete (zoh) of the one-state system (A, B) at that step size, and
    the step next to A = 0 against its closed form in 60-digit decimal arithmetic."""
    from decimal import Decimal, getcontext
    one = np.ones((1, 1))
    y, st = orc.step(np.full((1, 1, 1), 3.0), 1.5 * one, 0.0 * one, -one, 4.0 * one, 2.0 * one, zoh=True)
    assert abs(st[0, 0, 0] - 4.5) < 1e-15 and abs(y[0, 0] - 9.0) < 1e-14, (st, y)
    rng = np.random.default_rng(77)
    for _ in range(5):
        a, bq, x, u0, h0 = -rng.uniform(0.05, 4.0), rng.standard_normal(), rng.uniform(-2, 1), \
            rng.standard_normal(), rng.standard_normal()
        dt = float(_softplus(x))
        Ad, Bd, _, _, _ = scipy.signal.cont2discrete((np.array([[a]]), np.array([[bq]]), np.ones((1, 1)),
                                                      np.zeros((1, 1))), dt, method="zoh")
        _, st = orc.step(np.full((1, 1, 1), h0), u0 * one, x * one, a * one, bq * one, one, zoh=True)
        want = Ad[0, 0] * h0 + Bd[0, 0] * u0
        assert abs(st[0, 0, 0] - want) < 1e-12 * max(1.0, abs(want)), (a, st[0, 0, 0], want)
    getcontext().prec = 60
    x, u0, bq = 0.4, 1.3, 0.6
    dt = float(np.logaddexp(0.0, x))
    for a in (-1e-6, 3e-7, -2e-3, -0.05):
        _, st = orc.step(np.zeros((1, 1, 1)), u0 * one, x * one, a * one, bq * one, one, zoh=True)
        D_dt, D_A = Decimal(dt), Decimal(a)
        want = float(((D_dt * D_A).exp() - 1) / D_A * Decimal(bq) * Decimal(u0))
        assert abs(st[0, 0, 0] - want) <= 1e-14 * abs(want), (a, st[0, 0, 0], want)


def check_softplus_silu(orc):
    """Through the oracle: N=1, A=0, B=C=u=1, D=0, L=1 gives y = softplus(delta + bias);
    B=0, D=u=1 gives y = silu(z)."""
    x = np.concatenate([np.linspace(-50, 50, 201), [0.0, 1e-8, -1e-8, 700.0, -700.0]])
    M = x.size
    one = np.ones((1, M, 1))
    y, _ = orc.scan(one, x.reshape(1, M, 1), np.zeros((M, 1)), np.ones((1, 1, 1)), np.ones((1, 1, 1)))
    sp = y[0, :, 0]
    assert rel(sp, _softplus(x)) < 1e-15
    assert np.max(np.abs(sp[:201] - sp[:201][::-1] - x[:201])) < 1e-12   # softplus(x) - softplus(-x) = x
    assert abs(sp[201] - np.log(2.0)) < 1e-16
    y, _ = orc.scan(one, np.zeros((1, M, 1)), np.zeros((M, 1)), np.zeros((1, 1, 1)), np.ones((1, 1, 1)),
                    D=np.ones(M), z=x.reshape(1, M, 1))
    si = y[0, :, 0]
    assert rel(si[:201], x[:201] * scipy.special.expit(x[:201])) < 1e-15
    assert np.max(np.abs(si[:201] - si[:201][::-1] - x[:201])) < 1e-12    # silu(z) - silu(-z) = z
    assert si[201] == 0.0


def check_linearity_in_u(orc):
    inp = tiny_inputs(81)
    rng = np.random.default_rng(82)
    u2 = rng.standard_normal(inp["u"].shape)
    a, b = 0.7, -1.3
    y1, h1 = orc.scan(**inp)
    y2, h2 = orc.scan(**{**inp, "u": u2})
    y3, h3 = orc.scan(**{**inp, "u": a * inp["u"] + b * u2})
    assert rel(y3, a * y1 + b * y2) < 1e-12 and rel(h3, a * h1 + b * h2) < 1e-12


def check_causality(orc):
    inp = tiny_inputs(91, L=30)
    y, _ = orc.scan(**inp)
    for s in (0, 7, 29):
        pert = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in inp.items()}
        for key in ("u", "delta", "z", "B", "C"):
            pert[key][..., s] += 1.5
        yp, _ = orc.scan(**pert)
        assert np.array_equal(yp[..., :s], y[..., :s])
        assert not np.allclose(yp[..., s], y[..., s])


def check_reverse(orc):
    inp = tiny_inputs(101)
    y, h = orc.scan(**inp, reverse=True)
    flip = {k: (v[..., ::-1].copy() if k in ("u", "delta", "z", "B", "C") else v) for k, v in inp.items()}
    yf, hf = orc.scan(**flip)
    assert rel(y, yf[..., ::-1]) < 1e-15 and rel(h, hf) < 1e-15
    yb, _ = brute_force(**flip)
    assert rel(y, yb[..., ::-1]) < 1e-11


def check_permutation_equivariance(orc):
    inp = tiny_inputs(111, Bsz=3, Dm=5)
    y, h = orc.scan(**inp)
    pd = np.array([3, 0, 4, 1, 2])
    pb = np.array([2, 0, 1])
    p = dict(inp)
    for k in ("u", "delta", "z"):
        p[k] = inp[k][pb][:, pd]
    for k in ("B", "C"):
        p[k] = inp[k][pb]
    p["A"] = inp["A"][pd]
    p["D"] = inp["D"][pd]
    p["delta_bias"] = inp["delta_bias"][pd]
    yp, hp = orc.scan(**p)
    assert np.array_equal(yp, y[pb][:, pd]) and np.array_equal(hp, h[pb][:, pd])


# ---- the conv step that produces u (ai.xwebgame.com Mamba page, PyTorch block step 2) ----

def conv_inputs(seed, Bsz=2, Dm=3, L=37, K=4, bias=True, state=False):
    rng = np.random.default_rng(seed)
    inp = dict(x=rng.standard_normal((Bsz, Dm, L)), w=rng.standard_normal((Dm, K)),
               bias=rng.standard_normal(Dm) if bias else None)
    if state:
        inp["state"] = rng.standard_normal((Bsz, Dm, K - 1))
    return inp


def _torch_block_conv(x, w, bias, state=None):
    """The page's formulation with torch's own conv: a depthwise nn.Conv1d-style call with
    K-1 padding on both sides, output cut to the first L steps, then SiLU.  With a state
    the state is prepended and no padding is used."""
    import torch
    import torch.nn.functional as F
    xt = torch.from_numpy(np.ascontiguousarray(x))
    wt = torch.from_numpy(np.ascontiguousarray(w))[:, None, :]
    bt = None if bias is None else torch.from_numpy(np.ascontiguousarray(bias))
    Dm, K = w.shape
    L = x.shape[-1]
    if state is None:
        v = F.conv1d(xt, wt, bt, padding=K - 1, groups=Dm)[..., :L]
    else:
        v = F.conv1d(torch.cat([torch.from_numpy(state), xt], dim=-1), wt, bt, groups=Dm)
    return v.numpy() * scipy.special.expit(v.numpy())


def check_conv_library(orc):
    for K in (1, 2, 3, 4):
        for st in (False, True):
            for bias in (True, False):
                inp = conv_inputs(120 + K, K=K, state=st, bias=bias)
                u, _ = orc.conv1d(**inp)
                assert rel(u, _torch_block_conv(**inp)) < 1e-13, (K, st, bias)


def check_conv_impulse(orc):
    """A unit impulse at t0 yields pre-activations w[K-1-j] at t0 + j and 0 elsewhere."""
    Dm, K, L, t0 = 2, 4, 12, 5
    w = np.array([[0.5, -1.25, 2.0, 0.75], [-0.3, 0.9, 1.7, -2.2]])
    x = np.zeros((1, Dm, L))
    x[..., t0] = 1.0
    u, _ = orc.conv1d(x, w)
    v = np.zeros((Dm, L))
    for j in range(K):
        v[:, t0 + j] = w[:, K - 1 - j]
    assert rel(u[0], _silu(v)) < 1e-15


def check_conv_k1(orc):
    inp = conv_inputs(131, K=1)
    u, so = orc.conv1d(**inp)
    v = inp["w"][None, :, 0:1] * inp["x"] + inp["bias"][None, :, None]
    assert rel(u, _silu(v)) < 1e-15 and so.shape == (2, 3, 0)


def check_conv_state_out(orc):
    K = 4
    for L in (1, 2, 3, 4, 9):
        inp = conv_inputs(140 + L, L=L, K=K, state=True)
        _, so = orc.conv1d(**inp)
        ext = np.concatenate([inp["state"], inp["x"]], axis=-1)
        assert np.array_equal(so, ext[..., -(K - 1):]), L


def check_conv_chunking(orc):
    """Processing in pieces with the state carried equals one pass; so does the per-step form."""
    inp = conv_inputs(151, L=23)
    u, so = orc.conv1d(**inp)
    for cut in (1, 2, 3, 10, 22):
        u1, s1 = orc.conv1d(inp["x"][..., :cut], inp["w"], inp["bias"])
        u2, s2 = orc.conv1d(inp["x"][..., cut:], inp["w"], inp["bias"], s1)
        assert rel(np.concatenate([u1, u2], axis=-1), u) < 1e-15 and np.array_equal(s2, so)
    st = np.zeros((2, 3, 3))
    for t in range(23):
        ut, st = orc.conv_step(st, inp["x"][..., t], inp["w"], inp["bias"])
        assert rel(ut, u[..., t]) < 1e-15
    assert np.array_equal(st, so)


def check_conv_causality(orc):
    inp = conv_inputs(161, L=20)
    u, _ = orc.conv1d(**inp)
    for s in (0, 9, 19):
        x2 = inp["x"].copy()
        x2[..., s] += 2.0
        u2, _ = orc.conv1d(x2, inp["w"], inp["bias"])
        assert np.array_equal(u2[..., :s], u[..., :s])
        assert not np.allclose(u2[..., s], u[..., s])
        if s + 4 < 20:
            assert np.array_equal(u2[..., s + 4:], u[..., s + 4:])   # width 4: no reach beyond


# ---- gradients of the scan (chain rule on the forward definition; not on the pages) ----

def _torch_forward(u, delta, A, B, C, D, z, delta_bias, h0, reverse=False, zoh=False):
    """A plain fp64 torch forward, written step by step over time with tensor ops over
    (batch, channel, state); its autograd gives gradients by a route independent of the
    oracle's hand-derived adjoint."""
    import torch
    import torch.nn.functional as F
    Bsz, Dm, L = u.shape
    x = delta + (delta_bias[None, :, None] if delta_bias is not None else 0.0)
    dt = F.softplus(x, beta=1.0, threshold=60.0)
    h = h0 if h0 is not None else torch.zeros(Bsz, Dm, A.shape[1], dtype=torch.float64)
    outs = [None] * L
    for t in (range(L - 1, -1, -1) if reverse else range(L)):
        a = torch.exp(dt[:, :, t, None] * A[None])
        # zero-order hold: B_bar = (exp(dt A) - 1) / A * B  (A is nonzero in these inputs)
        e = torch.expm1(dt[:, :, t, None] * A[None]) / A[None] if zoh else dt[:, :, t, None]
        h = a * h + e * B[:, None, :, t] * u[:, :, t, None]
        y = (h * C[:, None, :, t]).sum(-1)
        if D is not None:
            y = y + D[None, :] * u[:, :, t]
        if z is not None:
            y = y * F.silu(z[:, :, t])
        outs[t] = y
    return torch.stack(outs, dim=-1), h


_GRAD_NAMES = [("u", "du"), ("delta", "ddelta"), ("A", "dA"), ("B", "dB"), ("C", "dC"), ("D", "dD"),
               ("z", "dz"), ("delta_bias", "ddelta_bias"), ("h0", "dh0")]


def check_bwd_autograd(orc):
    import torch
    for reverse, zoh in ((False, False), (True, False), (False, True), (True, True)):
        inp = tiny_inputs(171 + reverse + 2 * zoh, L=25, h0=True)
        rng = np.random.default_rng(173)
        dout = rng.standard_normal(inp["u"].shape)
        dfin = rng.standard_normal(inp["h0"].shape)
        tin = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in inp.items()}
        out, hL = _torch_forward(**tin, reverse=reverse, zoh=zoh)
        y, h = orc.scan(**inp, reverse=reverse, zoh=zoh)
        assert rel(out.detach().numpy(), y) < 1e-13 and rel(hL.detach().numpy(), h) < 1e-13
        ((out * torch.from_numpy(dout)).sum() + (hL * torch.from_numpy(dfin)).sum()).backward()
        g = orc.scan_bwd(**inp, dout=dout, dfinal=dfin, reverse=reverse, zoh=zoh)
        for k, gk in _GRAD_NAMES:
            e = rel(g[gk], tin[k].grad.numpy())
            assert e < 1e-11, (reverse, zoh, gk, e)


def check_bwd_finite_difference(orc):
    """Directional derivatives of L = <dout, out> + <dfinal, h_L> from central differences of the
    forward oracle, one input at a time, against <gradient, direction>."""
    for zoh in (False, True):
        inp = tiny_inputs(181, L=20, h0=True)
        rng = np.random.default_rng(183)
        dout = rng.standard_normal(inp["u"].shape)
        dfin = rng.standard_normal(inp["h0"].shape)
        g = orc.scan_bwd(**inp, dout=dout, dfinal=dfin, zoh=zoh)

        def loss(p):
            y, h = orc.scan(**p, zoh=zoh)
            return float(np.sum(y * dout) + np.sum(h * dfin))

        eps = 1e-5
        for k, gk in _GRAD_NAMES:
            v = rng.standard_normal(inp[k].shape)
            lp = loss({**inp, k: inp[k] + eps * v})
            lm = loss({**inp, k: inp[k] - eps * v})
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(g[gk] * v))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (zoh, gk, fd, an)


def check_bwd_scalar_closed_form(orc):
    """One channel, one state, two steps, no gate: out_t = C_t h_t with h_1 = a_1 h_0 + dt_1 B_1 u_1.
    dL/du_0 for L = out_1 is C_1 a_1 dt_0 B_0, by hand."""
    dt_x = np.array([0.3, -0.2])
    u = np.array([[[0.7, -1.1]]])
    Bm = np.array([[[0.5, 1.5]]])
    Cm = np.array([[[2.0, -0.25]]])
    A = np.array([[-0.8]])
    dtv = np.logaddexp(0.0, dt_x)
    a1 = np.exp(dtv[1] * A[0, 0])
    g = orc.scan_bwd(u, dt_x.reshape(1, 1, 2), A, Bm, Cm, dout=np.array([[[0.0, 1.0]]]))
    assert abs(g["du"][0, 0, 0] - Cm[0, 0, 1] * a1 * dtv[0] * Bm[0, 0, 0]) < 1e-15
    assert abs(g["du"][0, 0, 1] - Cm[0, 0, 1] * dtv[1] * Bm[0, 0, 1]) < 1e-15
    h0 = dtv[0] * Bm[0, 0, 0] * u[0, 0, 0]
    assert abs(g["dC"][0, 0, 1] - (a1 * h0 + dtv[1] * Bm[0, 0, 1] * u[0, 0, 1])) < 1e-15
    assert g["dC"][0, 0, 0] == 0.0


def check_bwd_zoh_at_zero_decay(orc):
    """ZOH with A = 0: B_bar = dt B and d(B_bar)/dA = dt^2 B / 2 (the series of (e^(dt A) - 1) / A).
    One step from a zero state, L = out_0 = C h_1 = C dt B u:  dL/dA = C B u dt^2 / 2 and
    dL/d(delta) = C B u * logistic(delta); a central difference over A = +-eps agrees."""
    x = np.array([[[0.4]]])
    u = np.array([[[1.3]]])
    Bm = np.array([[[0.6]]])
    Cm = np.array([[[-1.7]]])
    A0 = np.array([[0.0]])
    dt = np.logaddexp(0.0, 0.4)
    g = orc.scan_bwd(u, x, A0, Bm, Cm, dout=np.array([[[1.0]]]), zoh=True)
    want = Cm[0, 0, 0] * Bm[0, 0, 0] * u[0, 0, 0] * dt * dt / 2
    assert abs(g["dA"][0, 0] - want) < 1e-15, (g["dA"], want)
    sg = 1.0 / (1.0 + np.exp(-0.4))
    assert abs(g["ddelta"][0, 0, 0] - Cm[0, 0, 0] * Bm[0, 0, 0] * u[0, 0, 0] * sg) < 1e-15
    eps = 1e-4  # (e^(dt A) - 1) / A cancels near 0: rounding error ~1e-16 / eps, truncation ~eps^2
    yp, _ = orc.scan(u, x, A0 + eps, Bm, Cm, zoh=True)
    ym, _ = orc.scan(u, x, A0 - eps, Bm, Cm, zoh=True)
    assert abs((yp - ym)[0, 0, 0] / (2 * eps) - want) < 1e-7


def check_zoh_near_zero_decay_exact(orc):
    """ZOH close to A = 0, against its closed forms evaluated in 60-digit decimal arithmetic
    (where exp(dt A) - 1 and dt exp(dt A) - e lose nothing to cancellation).  One step from a
    zero state with no skip and no gate: out_0 = C e B u with e = (exp(dt A) - 1) / A, and
    d out_0 / dA = C B u (dt exp(dt A) - e) / A.  In fp64 the plain closed forms lose up to
    ~1e-16 / (dt A)^2 relative here; the oracle must not."""
    from decimal import Decimal, getcontext
    getcontext().prec = 60
    x = np.array([[[0.4]]])
    u = np.array([[[1.3]]])
    Bm = np.array([[[0.6]]])
    Cm = np.array([[[-1.7]]])
    dt = float(np.logaddexp(0.0, 0.4))
    cbu = Decimal(Cm[0, 0, 0]) * Decimal(Bm[0, 0, 0]) * Decimal(u[0, 0, 0])
    for a in (-1e-6, 3e-7, -2e-3, 2e-2, -0.05, -1.0):
        A = np.array([[a]])
        y, _ = orc.scan(u, x, A, Bm, Cm, zoh=True)
        g = orc.scan_bwd(u, x, A, Bm, Cm, dout=np.array([[[1.0]]]), zoh=True)
        D_dt, D_A = Decimal(dt), Decimal(a)
        ex = (D_dt * D_A).exp()
        e = (ex - 1) / D_A
        want_y = float(cbu * e)
        want_dA = float(cbu * (D_dt * ex - e) / D_A)
        assert abs(y[0, 0, 0] - want_y) <= 1e-14 * abs(want_y), (a, y[0, 0, 0], want_y)
        assert abs(g["dA"][0, 0] - want_dA) <= 1e-13 * abs(want_dA), (a, g["dA"][0, 0], want_dA)


ALL_CHECKS = [check_brute_force, check_initial_state, check_lti_closed_form, check_zoh_library,
              check_a_zero_cumsum, check_small_step_skip, check_single_step_closed_form,
              check_step_matches_scan, check_step_zoh_closed_form, check_softplus_silu, check_linearity_in_u, check_causality,
              check_reverse, check_permutation_equivariance,
              check_conv_library, check_conv_impulse, check_conv_k1, check_conv_state_out,
              check_conv_chunking, check_conv_causality,
              check_bwd_autograd, check_bwd_finite_difference, check_bwd_scalar_closed_form,
              check_bwd_zoh_at_zero_decay, check_zoh_near_zero_decay_exact]

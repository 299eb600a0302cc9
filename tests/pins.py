"""Pins of the fp64 oracle: checks that tie it to something other than itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with what the mathematics fixes: closed forms, brute-force
unrolling, textbook special cases, exact invariances and the chunked-vs-
sequential equivalence that the "From S4 to Mamba-3" case study tests
(section 04 "Chunked SSD with a sequential reference", section 09 Validation:
aligned (32) and misaligned (64) chunks; step() equals a full forward).

The same functions run against planted-mistake builds of the oracle in
``test_oracle_mutants.py``: every planted mistake must fail at least one pin.
"""
import math

import numpy as np

TIGHT = 1e-10  # fp64 vs fp64: differences are rounding-order only


def relerr(a, b):
    a, b = np.asarray(a), np.asarray(b)
    dt = np.complex128 if (np.iscomplexobj(a) or np.iscomplexobj(b)) else np.float64
    a, b = a.astype(dt), b.astype(dt)
    nb = np.linalg.norm(b.ravel())
    d = np.linalg.norm((a - b).ravel())
    return d / nb if nb > 0 else d


def close(a, b, tol=TIGHT, what=""):
    e = relerr(a, b)
    assert e <= tol, f"{what}: normwise relative error {e:.3e} > {tol:.1e}"


# ----------------------------------------------------------- random problems
def mamba1_problem(B, L, D, N, seed, h0=True, Dskip=True, z=True):
    """fp64 Mamba-1 problem with distinct A per (d, n) and positive Delta."""
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((B, L, D)),
        delta=np.logaddexp(0.0, r.normal(-2.0, 1.0, (B, L, D))),
        A=-np.exp(r.uniform(-1.0, 1.5, (D, N))),
        Bm=r.standard_normal((B, L, N)) / math.sqrt(N),
        Cm=r.standard_normal((B, L, N)) / math.sqrt(N),
        D=r.standard_normal(D) if Dskip else None,
        z=r.standard_normal((B, L, D)) if z else None,
        h0=0.5 * r.standard_normal((B, D, N)) if h0 else None,
    )


def ssd_problem(B, L, H, P, N, seed, h0=True, Dskip=True, z=True):
    r = np.random.default_rng(seed)
    return dict(
        x=r.standard_normal((B, L, H, P)),
        delta=np.logaddexp(0.0, r.normal(-2.0, 1.0, (B, L, H))),
        A=-np.exp(r.uniform(0.0, math.log(16.0), H)),
        Bm=r.standard_normal((B, L, N)) / math.sqrt(N),
        Cm=r.standard_normal((B, L, N)) / math.sqrt(N),
        D=r.standard_normal(H) if Dskip else None,
        z=r.standard_normal((B, L, H, P)) if z else None,
        h0=0.5 * r.standard_normal((B, H, N, P)) if h0 else None,
    )


def silu(z):
    return z / (1.0 + np.exp(-z))


def ssd_as_mamba1(p):
    """SSD problem -> the Mamba-1 problem with D' = H*P channels that it equals:
    channel h*P+p gets x[..,h,p], Delta[..,h], A[h] for every state index n,
    skip D[h], and the (N, P) state transposed to (P, N)."""
    x = p["x"]
    B, L, H, P = x.shape
    N = p["Bm"].shape[2]
    m = dict(
        x=x.reshape(B, L, H * P),
        delta=np.repeat(p["delta"], P, axis=2),
        A=np.repeat(p["A"], P)[:, None] * np.ones((1, N)),
        Bm=p["Bm"], Cm=p["Cm"],
        D=None if p["D"] is None else np.repeat(p["D"], P),
        z=None if p["z"] is None else p["z"].reshape(B, L, H * P),
        h0=None if p["h0"] is None else p["h0"].transpose(0, 1, 3, 2).reshape(B, H * P, N),
    )
    return m


# ----------------------------------------------------------------- P1
def pin_chunked_equals_sequential(orc):
    """SSD chunked form == sequential recurrence for aligned, misaligned, ragged,
    single-step and longer-than-L chunks."""
    for L, Q in [(96, 32), (96, 64), (100, 7), (64, 1), (100, 256), (50, 50), (33, 32)]:
        p = ssd_problem(2, L, 3, 4, 5, seed=L * 1000 + Q)
        ys, hs = orc.ssd_seq(**p)
        yc, hc = orc.ssd_chunked(**p, chunk=Q)
        close(yc, ys, what=f"chunked y L={L} Q={Q}")
        close(hc, hs, what=f"chunked h_final L={L} Q={Q}")


# ----------------------------------------------------------------- P2
def _mamba1_constant_closed_form(x0, d0, A, b0, c0, Dv, z0, h0, L):
    """Constant inputs: h_t = a^{t+1} h0 + beta (1 - a^{t+1})/(1 - a),
    a = exp(delta A), beta = delta B x; the ratio is expm1((t+1) delta A) / expm1(delta A)."""
    Dd, N = A.shape
    t1 = np.arange(1, L + 1)[:, None, None]                  # [L,1,1]
    lam = d0 * A[None]                                        # [1,D,N]
    geo = np.expm1(t1 * lam) / np.expm1(lam)                  # [L,D,N]
    h = np.exp(t1 * lam) * h0[None] + (d0 * b0[None, None, :] * x0) * geo
    v = (c0[None, None, :] * h).sum(-1) + Dv[None] * x0
    return v * silu(z0), h[-1]


def pin_constant_input_closed_form(orc):
    """Geometric-series closed form for constant inputs (all four recurrences)."""
    B, L, D, N = 1, 37, 3, 4
    r = np.random.default_rng(7)
    x0, d0, z0 = 0.7, 0.05, -0.4
    A = -np.exp(r.uniform(-1, 1.5, (D, N)))
    b0 = r.standard_normal(N)
    c0 = r.standard_normal(N)
    Dv = r.standard_normal(D)
    h0 = r.standard_normal((B, D, N))
    yref, href = _mamba1_constant_closed_form(x0, d0, A, b0, c0, Dv, z0, h0[0], L)
    args = dict(x=np.full((B, L, D), x0), delta=np.full((B, L, D), d0), A=A,
                Bm=np.broadcast_to(b0, (B, L, N)), Cm=np.broadcast_to(c0, (B, L, N)),
                D=Dv, z=np.full((B, L, D), z0), h0=h0)
    y, hf = orc.scan(**args)
    close(y[0], yref, what="scan closed form y")
    close(hf[0], href, what="scan closed form h")
    # the decode step iterated L times
    st = h0.copy()
    ys = []
    for t in range(L):
        yt, st = orc.step(st, np.full((B, D), x0), np.full((B, D), d0), A, b0[None], c0[None],
                          D=Dv, z=np.full((B, D), z0))
        ys.append(yt[0])
    close(np.stack(ys), yref, what="step closed form y")
    close(st[0], href, what="step closed form h")
    # SSD: scalar A per head; state (N, P); every p sees the same constants
    H, P = 2, 3
    Ah = -np.exp(r.uniform(0, math.log(16), H))
    Dh = r.standard_normal(H)
    hs0 = r.standard_normal((B, H, N, P))
    sargs = dict(x=np.full((B, L, H, P), x0), delta=np.full((B, L, H), d0), A=Ah,
                 Bm=np.broadcast_to(b0, (B, L, N)), Cm=np.broadcast_to(c0, (B, L, N)),
                 D=Dh, z=np.full((B, L, H, P), z0), h0=hs0)
    for name, fn in [("ssd_seq", orc.ssd_seq), ("ssd_chunked", lambda **k: orc.ssd_chunked(**k, chunk=8))]:
        y, hf = fn(**sargs)
        for h in range(H):
            for p_ in range(P):
                yr, hr = _mamba1_constant_closed_form(
                    x0, d0, np.full((1, N), Ah[h]), b0, c0, np.array([Dh[h]]), z0,
                    hs0[0, h, :, p_][None], L)
                close(y[0, :, h, p_], yr[:, 0], what=f"{name} closed form y")
                close(hf[0, h, :, p_], hr[0], what=f"{name} closed form h")
    # SSD decode step iterated
    st = hs0.copy()
    ys = []
    for t in range(L):
        yt, st = orc.ssd_step(st, np.full((B, H, P), x0), np.full((B, H), d0), Ah, b0[None],
                              c0[None], D=Dh, z=np.full((B, H, P), z0))
        ys.append(yt[0])
    ys = np.stack(ys)
    for h in range(H):
        yr, hr = _mamba1_constant_closed_form(x0, d0, np.full((1, N), Ah[h]), b0, c0,
                                              np.array([Dh[h]]), z0, hs0[0, h, :, 0][None], L)
        close(ys[:, h, 0], yr[:, 0], what="ssd_step closed form y")


# ----------------------------------------------------------------- P3, P4
def pin_prefill_one_equals_step(orc):
    """L = 1 prefill == one decode step from the same state (y and state)."""
    p = mamba1_problem(2, 1, 5, 6, seed=3)
    y, hf = orc.scan(**p)
    ys, st = orc.step(p["h0"], p["x"][:, 0], p["delta"][:, 0], p["A"], p["Bm"][:, 0],
                      p["Cm"][:, 0], D=p["D"], z=p["z"][:, 0])
    close(ys, y[:, 0], what="step vs L=1 y")
    close(st, hf, what="step vs L=1 state")
    q = ssd_problem(2, 1, 3, 4, 5, seed=4)
    y, hf = orc.ssd_seq(**q)
    ys, st = orc.ssd_step(q["h0"], q["x"][:, 0], q["delta"][:, 0], q["A"], q["Bm"][:, 0],
                          q["Cm"][:, 0], D=q["D"], z=q["z"][:, 0])
    close(ys, y[:, 0], what="ssd_step vs L=1 y")
    close(st, hf, what="ssd_step vs L=1 state")


def pin_prefill_then_step(orc):
    """prefill(L) then step(token L+1) == prefill(L+1): last y and final state."""
    L = 23
    p = mamba1_problem(2, L + 1, 4, 5, seed=5)
    yfull, hfull = orc.scan(**p)
    cut = {k: (v[:, :L] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
    _, h = orc.scan(**cut)
    ys, st = orc.step(h, p["x"][:, L], p["delta"][:, L], p["A"], p["Bm"][:, L], p["Cm"][:, L],
                      D=p["D"], z=p["z"][:, L])
    close(ys, yfull[:, L], what="prefill+step y")
    close(st, hfull, what="prefill+step state")
    q = ssd_problem(2, L + 1, 2, 3, 4, seed=6)
    yfull, hfull = orc.ssd_seq(**q)
    cut = {k: (v[:, :L] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in q.items()}
    _, h = orc.ssd_chunked(**cut, chunk=8)
    ys, st = orc.ssd_step(h, q["x"][:, L], q["delta"][:, L], q["A"], q["Bm"][:, L],
                          q["Cm"][:, L], D=q["D"], z=q["z"][:, L])
    close(ys, yfull[:, L], what="ssd prefill+step y")
    close(st, hfull, what="ssd prefill+step state")


# ----------------------------------------------------------------- P5
def pin_brute_force_unroll(orc):
    """Sequential recurrences == the state written out as explicit products."""
    for (B, L, D, N, s) in [(1, 12, 3, 4, 11), (2, 7, 2, 3, 12), (1, 1, 1, 1, 13)]:
        p = mamba1_problem(B, L, D, N, seed=s)
        y, hf = orc.scan(**p)
        yu, hu = orc.scan_unroll(**p)
        close(y, yu, what="scan vs unroll y")
        close(hf, hu, what="scan vs unroll h")
    for (B, L, H, P, N, s) in [(1, 12, 2, 3, 4, 21), (2, 6, 1, 2, 3, 22)]:
        q = ssd_problem(B, L, H, P, N, seed=s)
        y, hf = orc.ssd_seq(**q)
        yu, hu = orc.ssd_unroll(**q)
        close(y, yu, what="ssd vs unroll y")
        close(hf, hu, what="ssd vs unroll h")


# ----------------------------------------------------------------- P6
def pin_special_cases(orc):
    """A = 0: the state is h0 plus a cumulative sum; Delta = 0: the state never
    moves; C = 0 and D = 0: the output is zero; C = 0 alone: y = D x silu(z)."""
    p = mamba1_problem(2, 19, 3, 4, seed=31)
    p0 = dict(p, A=np.zeros_like(p["A"]))
    y, hf = orc.scan(**p0)
    inc = p["delta"][..., None] * p["Bm"][:, :, None, :] * p["x"][..., None]   # [B,L,D,N]
    h = p["h0"][:, None] + np.cumsum(inc, axis=1)
    v = np.einsum("bln,bldn->bld", p["Cm"], h) + p["D"] * p["x"]
    close(y, v * silu(p["z"]), what="A=0 cumsum y")
    close(hf, h[:, -1], what="A=0 cumsum h")
    pd = dict(p, delta=np.zeros_like(p["delta"]))
    y, hf = orc.scan(**pd)
    v = np.einsum("bln,bdn->bld", p["Cm"], p["h0"]) + p["D"] * p["x"]
    close(y, v * silu(p["z"]), what="Delta=0 y")
    close(hf, p["h0"], what="Delta=0 h")
    pc = dict(p, Cm=np.zeros_like(p["Cm"]), D=np.zeros_like(p["D"]))
    y, _ = orc.scan(**pc)
    assert np.all(y == 0.0), "C=0, D=0 must give y=0"
    pc = dict(p, Cm=np.zeros_like(p["Cm"]))
    y, _ = orc.scan(**pc)
    close(y, p["D"] * p["x"] * silu(p["z"]), what="C=0 y")
    # no gate, no skip: y = C . h only
    pn = dict(p, z=None, D=None)
    y, _ = orc.scan(**pn)
    yd, _ = orc.scan(**dict(pn, D=np.zeros_like(p["D"])))
    close(y, yd, what="D=None vs D=0")
    # SSD with A = 0 reduces to a cumulative sum of outer products
    q = ssd_problem(1, 11, 2, 3, 4, seed=32)
    q0 = dict(q, A=np.zeros_like(q["A"]))
    inc = (q["delta"][..., None, None] * q["Bm"][:, :, None, :, None]
           * q["x"][:, :, :, None, :])                                           # [B,L,H,N,P]
    S = q["h0"][:, None] + np.cumsum(inc, axis=1)
    v = np.einsum("bln,blhnp->blhp", q["Cm"], S) + q["D"][None, None, :, None] * q["x"]
    for name, fn in [("seq", orc.ssd_seq), ("chunk", lambda **k: orc.ssd_chunked(**k, chunk=4))]:
        y, hf = fn(**q0)
        close(y, v * silu(q["z"]), what=f"ssd {name} A=0 y")
        close(hf, S[:, -1], what=f"ssd {name} A=0 h")


# ----------------------------------------------------------------- P7
def pin_ssd_equals_mamba1_mapping(orc):
    """SSD == Mamba-1 with D = H*P channels sharing Delta and A per head."""
    q = ssd_problem(2, 17, 3, 4, 5, seed=41)
    m = ssd_as_mamba1(q)
    ym, hm = orc.scan(**m)
    B, L, H, P = q["x"].shape
    N = q["Bm"].shape[2]
    for name, fn in [("seq", orc.ssd_seq), ("chunk", lambda **k: orc.ssd_chunked(**k, chunk=6))]:
        y, hf = fn(**q)
        close(y.reshape(B, L, H * P), ym, what=f"ssd {name} vs mamba1 y")
        close(hf.transpose(0, 1, 3, 2).reshape(B, H * P, N), hm, what=f"ssd {name} vs mamba1 h")


# ----------------------------------------------------------------- P8
def pin_split_carry(orc):
    """scan(x[:m]) -> h; scan(x[m:], h0 = h) == scan(x), at several cut points."""
    p = mamba1_problem(2, 40, 3, 4, seed=51)
    y, hf = orc.scan(**p)
    for m in (1, 13, 39):
        a = {k: (v[:, :m] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
        y1, h1 = orc.scan(**a)
        b = {k: (v[:, m:] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
        b["h0"] = h1
        y2, h2 = orc.scan(**b)
        close(np.concatenate([y1, y2], axis=1), y, what=f"split y m={m}")
        close(h2, hf, what=f"split h m={m}")
    q = ssd_problem(1, 40, 2, 3, 4, seed=52)
    y, hf = orc.ssd_seq(**q)
    for m in (9, 30):
        a = {k: (v[:, :m] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in q.items()}
        y1, h1 = orc.ssd_chunked(**a, chunk=8)
        b = {k: (v[:, m:] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in q.items()}
        b["h0"] = h1
        y2, h2 = orc.ssd_chunked(**b, chunk=8)
        close(np.concatenate([y1, y2], axis=1), y, what=f"ssd split y m={m}")
        close(h2, hf, what=f"ssd split h m={m}")


# ----------------------------------------------------------------- P9
def pin_causality(orc):
    """Changing inputs at t' > t leaves y[:t+1] bit-identical."""
    p = mamba1_problem(1, 30, 3, 4, seed=61)
    y, _ = orc.scan(**p)
    t = 17
    pp = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    for k in ("x", "delta", "Bm", "Cm", "z"):
        pp[k][:, t + 1:] = pp[k][:, t + 1:] * 1.5 + 0.25
    y2, _ = orc.scan(**pp)
    assert np.array_equal(y[:, :t + 1], y2[:, :t + 1]), "scan is not causal"
    assert not np.array_equal(y[:, t + 1:], y2[:, t + 1:])
    q = ssd_problem(1, 30, 2, 3, 4, seed=62)
    for fn in (orc.ssd_seq, lambda **k: orc.ssd_chunked(**k, chunk=8)):
        y, _ = fn(**q)
        qq = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in q.items()}
        for k in ("x", "delta", "Bm", "Cm", "z"):
            qq[k][:, t + 1:] = qq[k][:, t + 1:] * 1.5 + 0.25
        y2, _ = fn(**qq)
        assert np.array_equal(y[:, :t + 1], y2[:, :t + 1]), "ssd is not causal"


# ----------------------------------------------------------------- P10
def pin_linearity(orc):
    """y(alpha x, alpha h0) = alpha y(x, h0) for fixed Delta, B, C, z (exact for alpha = 2)."""
    p = mamba1_problem(2, 21, 3, 4, seed=71)
    y, hf = orc.scan(**p)
    y2, h2 = orc.scan(**dict(p, x=2 * p["x"], h0=2 * p["h0"]))
    assert np.array_equal(y2, 2 * y) and np.array_equal(h2, 2 * hf)
    y3, h3 = orc.scan(**dict(p, x=-3 * p["x"], h0=-3 * p["h0"]))
    close(y3, -3 * y, what="linearity y")
    close(h3, -3 * hf, what="linearity h")
    q = ssd_problem(1, 21, 2, 3, 4, seed=72)
    y, hf = orc.ssd_chunked(**q, chunk=5)
    y2, h2 = orc.ssd_chunked(**dict(q, x=2 * q["x"], h0=2 * q["h0"]), chunk=5)
    assert np.array_equal(y2, 2 * y) and np.array_equal(h2, 2 * hf)


# ------------------------------------------------------------- backward (O6)
GRAD_OF = {"x": "dx", "delta": "ddelta", "A": "dA", "Bm": "dBm", "Cm": "dCm", "D": "dD", "z": "dz",
           "h0": "dh0"}


def _loss(orc, p, dy, dhf):
    """l = sum(dy * y) + sum(dh_final * h_final), through the forward oracle O1."""
    y, hf = orc.scan(**p)
    return float(np.sum(dy * y) + np.sum(dhf * hf))


def _cotangents(p, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal(p["x"].shape), r.standard_normal(p["h0"].shape if p["h0"] is not None
                                                              else (p["x"].shape[0], p["A"].shape[0],
                                                                    p["A"].shape[1]))


def pin_bwd_finite_differences(orc):
    """Every gradient element equals the central difference of the loss computed by
    the forward oracle (O(eps^2) truncation, ~1e-10 round-off at eps = 1e-6)."""
    for (B, L, D, N), opts, seed in [((2, 6, 3, 4), {}, 81),
                                     ((1, 5, 2, 3), dict(h0=False, Dskip=False, z=False), 82)]:
        p = mamba1_problem(B, L, D, N, seed=seed, **opts)
        dy, dhf = _cotangents(p, seed + 100)
        g = orc.scan_bwd(dy=dy, dh_final=dhf, **p)
        for name, gname in GRAD_OF.items():
            if p.get(name) is None:
                if gname in ("dD", "dz"):
                    assert g[gname] is None
                    continue
                # no h0 means a zero initial state, whose gradient still exists
                p = dict(p, h0=np.zeros((B, D, N)))
            base = p[name]
            fd = np.zeros_like(base)
            for idx in np.ndindex(base.shape):
                eps = 1e-6 * max(1.0, abs(base[idx]))
                q = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
                q[name][idx] = base[idx] + eps
                lp = _loss(orc, q, dy, dhf)
                q[name][idx] = base[idx] - eps
                lm = _loss(orc, q, dy, dhf)
                fd[idx] = (lp - lm) / (2 * eps)
            close(g[gname], fd, tol=1e-6, what=f"finite differences {gname} {B, L, D, N} {opts}")


def pin_bwd_directional_derivative(orc):
    """<grad, v> equals the derivative of the loss along a random direction v over
    all inputs at once, on a longer sequence with every optional part present."""
    p = mamba1_problem(2, 37, 4, 5, seed=91)
    dy, dhf = _cotangents(p, 191)
    g = orc.scan_bwd(dy=dy, dh_final=dhf, **p)
    r = np.random.default_rng(291)
    v = {k: r.standard_normal(p[k].shape) for k in GRAD_OF}
    v["delta"] *= 0.05  # keeps Delta positive along the path
    lin = sum(float(np.sum(g[GRAD_OF[k]] * v[k])) for k in GRAD_OF)
    eps = 1e-5
    lp = _loss(orc, {k: (p[k] + eps * v[k] if k in v else p[k]) for k in p}, dy, dhf)
    lm = _loss(orc, {k: (p[k] - eps * v[k] if k in v else p[k]) for k in p}, dy, dhf)
    fd = (lp - lm) / (2 * eps)
    assert abs(lin - fd) <= 1e-7 * max(1.0, abs(fd)), f"directional derivative {lin} vs {fd}"


def pin_bwd_zero_decay_cumsum(orc):
    """A = 0 and no gate: the state is h0 plus a running sum, so the adjoint is a
    reverse running sum of dy C (+ dh_final); every gradient then has a closed form
    in cumsums."""
    p = mamba1_problem(2, 13, 3, 4, seed=101, z=False)
    p["A"] = np.zeros_like(p["A"])
    dy, dhf = _cotangents(p, 201)
    g = orc.scan_bwd(dy=dy, dh_final=dhf, **p)
    x, dl, Bm, Cm, h0, Dv = p["x"], p["delta"], p["Bm"], p["Cm"], p["h0"], p["D"]
    u = dl * x                                                     # [B,L,D]
    h = h0[:, None] + np.cumsum(u[..., None] * Bm[:, :, None, :], axis=1)   # h_t [B,L,D,N]
    hprev = np.concatenate([h0[:, None], h[:, :-1]], axis=1)
    adj = dy[..., None] * Cm[:, :, None, :]                       # dy_t C_t [B,L,D,N]
    gt = np.flip(np.cumsum(np.flip(adj, 1), axis=1), 1) + dhf[:, None]      # g_t
    close(g["dx"], dy * Dv + dl * np.einsum("bldn,bln->bld", gt, Bm), what="A=0 dx")
    close(g["ddelta"], x * np.einsum("bldn,bln->bld", gt, Bm), what="A=0 ddelta")
    close(g["dA"], np.einsum("bldn,bldn,bld->dn", gt, hprev, dl), what="A=0 dA")
    close(g["dBm"], np.einsum("bldn,bld->bln", gt, u), what="A=0 dB")
    close(g["dCm"], np.einsum("bld,bldn->bln", dy, h), what="A=0 dC")
    close(g["dD"], np.einsum("bld,bld->d", dy, x), what="A=0 dD")
    close(g["dh0"], gt[:, 0], what="A=0 dh0")


def pin_bwd_linear_in_cotangents(orc):
    """The gradients are linear in (dy, dh_final); dy = 0, dh_final = 0 gives zeros."""
    p = mamba1_problem(1, 11, 3, 4, seed=111)
    d1, h1 = _cotangents(p, 1)
    d2, h2 = _cotangents(p, 2)
    g1 = orc.scan_bwd(dy=d1, dh_final=h1, **p)
    g2 = orc.scan_bwd(dy=d2, dh_final=h2, **p)
    g3 = orc.scan_bwd(dy=2 * d1 - 3 * d2, dh_final=2 * h1 - 3 * h2, **p)
    for k in g1:
        close(g3[k], 2 * g1[k] - 3 * g2[k], what=f"linearity {k}")
    g0 = orc.scan_bwd(dy=np.zeros_like(d1), dh_final=None, **p)
    assert all(not np.any(v) for v in g0.values()), "zero cotangents give a nonzero gradient"


# --------------------------------------------------- discretisation variants (O7)
def pin_disc_euler_is_scan(orc):
    """Exponential-Euler with no Delta preprocessing is O1 / O4 exactly."""
    p = mamba1_problem(2, 23, 3, 4, seed=121)
    y, hf = orc.scan(**p)
    y2, h2 = orc.scan_disc(**p, disc="euler")
    assert np.array_equal(y, y2) and np.array_equal(hf, h2)
    t = {k: (v[:, 0] if k in ("x", "delta", "z", "Bm", "Cm") else v) for k, v in p.items() if k != "h0"}
    ys, ss = orc.step(p["h0"], **t)
    ys2, ss2 = orc.step_disc(p["h0"], **t, disc="euler")
    assert np.array_equal(ys, ys2) and np.array_equal(ss, ss2)


def pin_softplus_bias_preprocessing(orc):
    """Delta = softplus(raw + bias) inside equals O1 on Delta precomputed with numpy's
    logaddexp(0, .); a bias without softplus is a plain shift."""
    p = mamba1_problem(2, 19, 3, 4, seed=122)
    r = np.random.default_rng(222)
    raw = r.normal(-2.5, 1.5, p["delta"].shape)
    bias = r.normal(0.0, 0.8, 3)
    for disc in ("euler", "zoh"):
        y, hf = orc.scan_disc(**dict(p, delta=raw), disc=disc, delta_bias=bias, delta_softplus=True)
        y2, h2 = orc.scan_disc(**dict(p, delta=np.logaddexp(0.0, raw + bias)), disc=disc)
        close(y, y2, tol=1e-13, what=f"softplus+bias {disc} y")
        close(hf, h2, tol=1e-13, what=f"softplus+bias {disc} h")
    y3, _ = orc.scan_disc(**dict(p, delta=np.abs(raw)), delta_bias=np.abs(bias))
    y4, _ = orc.scan(**dict(p, delta=np.abs(raw) + np.abs(bias)))
    close(y3, y4, tol=1e-13, what="bias shift")
    t = {k: (v[:, 0] if k in ("x", "z", "Bm", "Cm") else v) for k, v in p.items() if k not in ("h0", "delta")}
    ys, ss = orc.step_disc(p["h0"], delta=raw[:, 0], **t, delta_bias=bias, delta_softplus=True)
    ys2, ss2 = orc.step(p["h0"], delta=np.logaddexp(0.0, raw[:, 0] + bias), **t)
    close(ys, ys2, tol=1e-13, what="step softplus y")
    close(ss, ss2, tol=1e-13, what="step softplus state")


def pin_zoh_step_is_exact_ode_solution(orc):
    """One zero-order-hold step is the exact solution of dh/dt = A h + B x over Delta
    with B x held: e^{A Delta} h0 + (integral of e^{A (Delta - s)} ds over [0, Delta]) B x,
    the integral taken by adaptive quadrature; includes |z| < 1e-4 (Taylor branch),
    A = 0 and A > 0."""
    from scipy.integrate import quad
    cases = [(0.1, -3.0), (0.5, -0.2), (1e-3, -2.0), (2e-5, -1.5), (0.3, 0.0), (0.01, 1.5), (1.7, -6.0)]
    D, N = 1, len(cases)
    A = np.array([[a for _, a in cases]])
    h0 = np.linspace(-0.5, 0.7, N).reshape(1, 1, N)
    Bm = np.linspace(0.3, 1.9, N).reshape(1, 1, N)
    for j, (dt, a) in enumerate(cases):
        # one channel per case: Delta is per channel, so run them one at a time
        y, hf = orc.scan_disc(x=np.array([[[0.7]]]), delta=np.array([[[dt]]]), A=A[:, j:j + 1],
                              Bm=Bm[:, :, j:j + 1], Cm=np.ones((1, 1, 1)), h0=h0[:, :, j:j + 1], disc="zoh")
        integral = quad(lambda s_: math.exp(a * (dt - s_)), 0.0, dt, epsabs=0.0, epsrel=1e-13)[0]
        exact = math.exp(a * dt) * h0[0, 0, j] + integral * Bm[0, 0, j] * 0.7
        assert abs(hf[0, 0, 0] - exact) <= 1e-12 * max(1.0, abs(exact)), (dt, a, hf[0, 0, 0], exact)
        assert abs(y[0, 0, 0] - exact) <= 1e-12 * max(1.0, abs(exact))


def pin_zoh_constant_input_closed_form(orc):
    """Constant inputs: h_t = a^t h0 + c (1 - a^t)/(1 - a), a = e^{Delta A},
    c = expm1(Delta A)/A B x (the ZOH input), written with expm1."""
    B, L, D, N = 1, 40, 2, 3
    r = np.random.default_rng(131)
    A = -np.exp(r.uniform(-1.0, 1.5, (D, N)))
    x0, d0, b0, c0 = 0.8, 0.07, r.standard_normal(N), r.standard_normal(N)
    h0 = r.standard_normal((B, D, N))
    p = dict(x=np.full((B, L, D), x0), delta=np.full((B, L, D), d0), A=A,
             Bm=np.tile(b0, (B, L, 1)), Cm=np.tile(c0, (B, L, 1)), h0=h0)
    y, hf = orc.scan_disc(**p, disc="zoh")
    t = np.arange(1, L + 1)[:, None, None]                       # [L,1,1]
    z = d0 * A[None]                                             # [1,D,N]
    c = np.expm1(z) / A[None] * b0 * x0
    h = np.exp(t * z) * h0 + c * np.expm1(t * z) / np.expm1(z)  # [L,D,N]
    close(y[0], np.einsum("ldn,n->ld", h, c0), tol=1e-11, what="zoh constant y")
    close(hf[0], h[-1], tol=1e-11, what="zoh constant h")


def pin_zoh_phi_both_branches(orc):
    """Bbar / (Delta B) = (e^z - 1)/z on both sides of the page's 1e-4 switch,
    against numpy's expm1(z)/z."""
    zs = np.array([1e-6, -5e-5, 9.9e-5, -1e-4, 1.01e-4, -1e-3, 0.1, -2.0])
    for z_ in zs:
        y, _ = orc.scan_disc(x=np.ones((1, 1, 1)), delta=np.ones((1, 1, 1)), A=np.array([[z_]]),
                             Bm=np.ones((1, 1, 1)), Cm=np.ones((1, 1, 1)), disc="zoh")
        ref = np.expm1(z_) / z_
        assert abs(y[0, 0, 0] - ref) <= 1e-10 * abs(ref), (z_, y[0, 0, 0], ref)


def pin_disc_step_matches_scan(orc):
    """Under ZOH with softplus(Delta + bias): prefill(1) equals one step, and
    prefill(L) then a step equals prefill(L + 1)."""
    p = mamba1_problem(2, 14, 3, 4, seed=141)
    r = np.random.default_rng(241)
    p["delta"] = r.normal(-2.0, 1.0, p["delta"].shape)
    kw = dict(disc="zoh", delta_bias=r.normal(0.0, 0.5, 3), delta_softplus=True)
    y, hf = orc.scan_disc(**p, **kw)
    q = {k: (v[:, :13] if k in ("x", "delta", "z", "Bm", "Cm") else v) for k, v in p.items()}
    y13, h13 = orc.scan_disc(**q, **kw)
    t = {k: p[k][:, 13] for k in ("x", "delta", "z", "Bm", "Cm")}
    ys, ss = orc.step_disc(h13, A=p["A"], D=p["D"], **t, **kw)
    close(ys, y[:, 13], what="zoh prefill+step y")
    close(ss, hf, what="zoh prefill+step state")
    q1 = {k: (v[:, :1] if k in ("x", "delta", "z", "Bm", "Cm") else v) for k, v in p.items()}
    y1, h1 = orc.scan_disc(**q1, **kw)
    t0 = {k: p[k][:, 0] for k in ("x", "delta", "z", "Bm", "Cm")}
    ys0, ss0 = orc.step_disc(p["h0"], A=p["A"], D=p["D"], **t0, **kw)
    close(ys0, y1[:, 0], what="zoh L=1 y")
    close(ss0, h1, what="zoh L=1 state")


# --------------------------------------------------- Mamba-3 (O8)
def mamba3_problem(B, L, D, N, seed, lam=None, theta=True, h0=True, Dskip=True, z=True):
    """fp64 Mamba-3 problem: Are < 0, rotation rates theta, lam in [0, 1] per (b, t, d)."""
    r = np.random.default_rng(seed)
    p = mamba1_problem(B, L, D, N, seed, h0=False, Dskip=Dskip, z=z)
    A = p.pop("A")
    p["Are"] = A
    p["theta"] = r.uniform(-3.0, 3.0, (D, N)) if theta else np.zeros((D, N))
    p["lam"] = r.uniform(0.0, 1.0, (B, L, D)) if lam is None else np.full((B, L, D), float(lam))
    if h0:
        p["h0"] = 0.5 * (r.standard_normal((B, D, N)) + 1j * r.standard_normal((B, D, N)))
    return p


def pin_m3_reduces_to_euler(orc):
    """lam = 1, theta = 0 is exponential-Euler, i.e. O1 (the reduction the case study's
    test pins: section 04 "Complex transitions for state tracking", section 09)."""
    p = mamba3_problem(2, 37, 3, 5, seed=301, lam=1.0, theta=False, h0=False)
    y, hf = orc.scan3(**p)
    q = {k: p[k] for k in ("x", "delta", "Bm", "Cm", "D", "z")}
    y1, h1 = orc.scan(**q, A=p["Are"])
    close(y, y1, tol=1e-13, what="m3 reduction y")
    close(hf.real, h1, tol=1e-13, what="m3 reduction h")
    assert np.max(np.abs(hf.imag)) == 0.0


def pin_m3_rotation_block_form(orc):
    """lam = 1: the complex recurrence equals the real 2-dimensional system whose
    transition over one step is the matrix exponential of Delta [[Are, -theta],
    [theta, Are]] acting on (Re h, Im h) (scipy's expm), with the input entering the
    real component; the output reads the real component."""
    from scipy.linalg import expm
    B, L, D, N = 1, 9, 2, 3
    p = mamba3_problem(B, L, D, N, seed=302, lam=1.0, Dskip=False, z=False)
    y, hf = orc.scan3(**p)
    yr = np.zeros((B, L, D))
    for d in range(D):
        for n in range(N):
            v = np.array([p["h0"][0, d, n].real, p["h0"][0, d, n].imag])
            M = np.array([[p["Are"][d, n], -p["theta"][d, n]], [p["theta"][d, n], p["Are"][d, n]]])
            for t in range(L):
                dt = p["delta"][0, t, d]
                v = expm(dt * M) @ v + np.array([dt * p["Bm"][0, t, n] * p["x"][0, t, d], 0.0])
                yr[0, t, d] += p["Cm"][0, t, n] * v[0]
            assert abs(hf[0, d, n] - (v[0] + 1j * v[1])) <= 1e-12 * max(1.0, abs(v[0]) + abs(v[1]))
    close(y, yr, tol=1e-12, what="m3 rotation-block y")


def _m3_exact(a, th, b, xf, T):
    """h(T) of dh/dt = (a + i th) h + b x(t), h(0) = 0, by adaptive quadrature."""
    from scipy.integrate import quad
    re = quad(lambda s_: math.exp(a * (T - s_)) * math.cos(th * (T - s_)) * b * xf(s_), 0.0, T,
              epsabs=1e-15, epsrel=1e-13, limit=400)[0]
    im = quad(lambda s_: math.exp(a * (T - s_)) * math.sin(th * (T - s_)) * b * xf(s_), 0.0, T,
              epsabs=1e-15, epsrel=1e-13, limit=400)[0]
    return re + 1j * im


def pin_m3_trapezoid_order(orc):
    """Against the exact solution of dh/dt = A h + B x(t) for a smooth input sampled at
    the step ends: lam = 1/2 (the trapezoidal rule on the one-step integral) is second
    order -- halving Delta cuts the error about 4x -- and lam = 1 (exponential-Euler)
    first order, about 2x; for real and complex A."""
    T, b = 2.0, 0.9
    xf = lambda t: math.sin(1.3 * t) + 0.5 * math.cos(0.4 * t)  # noqa: E731
    for a, th in ((-0.7, 0.0), (-0.4, 1.7)):
        exact = _m3_exact(a, th, b, xf, T)
        for lam, lo, hi in ((0.5, 3.6, 4.4), (1.0, 1.7, 2.3)):
            errs = []
            for L in (64, 128, 256):
                dt = T / L
                xs = np.array([xf((t + 1) * dt) for t in range(L)])
                p = dict(x=xs.reshape(1, L, 1), delta=np.full((1, L, 1), dt), lam=np.full((1, L, 1), lam),
                         Are=np.array([[a]]), theta=np.array([[th]]), Bm=np.full((1, L, 1), b),
                         Cm=np.ones((1, L, 1)), x_prev=np.array([[xf(0.0)]]), B_prev=np.array([[b]]))
                _, hf = orc.scan3(**p)
                errs.append(abs(hf[0, 0, 0] - exact))
            for e1, e2 in zip(errs, errs[1:]):
                assert lo <= e1 / e2 <= hi, (a, th, lam, errs)


def pin_m3_constant_input_closed_form(orc):
    """Constant inputs (and the same token before the sequence): h_t = alpha^t h0 +
    c (1 - alpha^t)/(1 - alpha) with alpha = e^{Delta (Are + i theta)} and
    c = ((1 - lam) alpha + lam) Delta B x, in numpy complex arithmetic."""
    B, L, D, N = 1, 33, 2, 3
    r = np.random.default_rng(303)
    Are = -np.exp(r.uniform(-1.0, 1.0, (D, N)))
    th = r.uniform(-2.0, 2.0, (D, N))
    x0, d0, l0 = 0.8, 0.11, 0.3
    b0, c0 = r.standard_normal(N), r.standard_normal(N)
    h0 = r.standard_normal((B, D, N)) + 1j * r.standard_normal((B, D, N))
    p = dict(x=np.full((B, L, D), x0), delta=np.full((B, L, D), d0), lam=np.full((B, L, D), l0), Are=Are,
             theta=th, Bm=np.tile(b0, (B, L, 1)), Cm=np.tile(c0, (B, L, 1)), h0=h0,
             x_prev=np.full((B, D), x0), B_prev=np.tile(b0, (B, 1)))
    y, hf = orc.scan3(**p)
    alpha = np.exp(d0 * (Are + 1j * th))                          # [D,N]
    c = ((1 - l0) * alpha + l0) * d0 * b0 * x0                     # [D,N]
    t = np.arange(1, L + 1)[:, None, None]
    h = alpha[None] ** t * h0[0] + c * (1 - alpha[None] ** t) / (1 - alpha)   # [L,D,N]
    close(y[0], np.einsum("ldn,n->ld", h.real, c0), tol=1e-11, what="m3 constant y")
    close(hf[0], h[-1], tol=1e-11, what="m3 constant h")


def pin_m3_split_carry(orc):
    """scan3(x[:m]) then scan3(x[m:]) from its final state and its last token equals
    scan3(x)."""
    p = mamba3_problem(2, 40, 3, 4, seed=304)
    y, hf = orc.scan3(**p)
    m = 17
    cut = lambda k, s_: p[k][:, s_]  # noqa: E731
    seq = ("x", "delta", "lam", "Bm", "Cm", "z")
    y1, h1 = orc.scan3(**{k: (cut(k, slice(0, m)) if k in seq else v) for k, v in p.items()})
    q = {k: (cut(k, slice(m, None)) if k in seq else v) for k, v in p.items()}
    q.update(h0=h1, x_prev=p["x"][:, m - 1], B_prev=p["Bm"][:, m - 1])
    y2, h2 = orc.scan3(**q)
    close(np.concatenate([y1, y2], axis=1), y, what="m3 split y")
    close(h2, hf, what="m3 split h")


ALL_PINS = [
    pin_chunked_equals_sequential,
    pin_constant_input_closed_form,
    pin_prefill_one_equals_step,
    pin_prefill_then_step,
    pin_brute_force_unroll,
    pin_special_cases,
    pin_ssd_equals_mamba1_mapping,
    pin_split_carry,
    pin_causality,
    pin_linearity,
    pin_bwd_finite_differences,
    pin_bwd_directional_derivative,
    pin_bwd_zero_decay_cumsum,
    pin_bwd_linear_in_cotangents,
    pin_disc_euler_is_scan,
    pin_softplus_bias_preprocessing,
    pin_zoh_step_is_exact_ode_solution,
    pin_zoh_constant_input_closed_form,
    pin_zoh_phi_both_branches,
    pin_disc_step_matches_scan,
    pin_m3_reduces_to_euler,
    pin_m3_rotation_block_form,
    pin_m3_trapezoid_order,
    pin_m3_constant_input_closed_form,
    pin_m3_split_carry,
]

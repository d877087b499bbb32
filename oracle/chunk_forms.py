"""fp64 chunkwise forms of gated delta-rule attention (numpy).

TEST INFRASTRUCTURE (see oracle/__init__.py). These are the method's own
algebraic forms, written from the ReWY paper: they pin the token oracle (the
chunk forms must reproduce it) and pin the algebra (the reduced and the
expanded backward graphs must agree, with the FLOP counts the pages print).

Notation (paper Sec. 2.3 and Sec. 3; the symbols are the ones the onedev.kr
summary prints in "How it works" and "What is different"). For one chunk of
n tokens and one head, rows are tokens, the state S is key-major (DK x DV):
    G      chunk-local inclusive cumsum of the log decay g; gam = exp(G)
    E  = diag(beta) (gam * K)     erase factor
    Y  = K / gam                  write key, undecayed to the chunk start
    Z  = diag(beta) V
    Qg = gam * Q,   Kt = exp(G_n - G) * K
    L  = strict_lower(E Y^T),  M = I + L,  A = M^{-1}
    W  = A E,   U = A Z,   R = U - W S     (so M R = Z - E S)
    Hm = lower_incl(Qg Y^T)                inclusive output projection
    O  = Qg S + Hm R
    S' = diag(gam_n) S + Kt^T R
Backward, given the output adjoint Ob and the next-state adjoint Sbn:
    Rb = Hm^T Ob + Kt Sbn        (both paths summed before the pullback, Sec. 3.1)
  ReWY producer (three products; Sec. 3.1-3.2):
    P = A^T Rb;  Zb = P;  Eb_dir = -P S^T;  D = -strict_lower(P R^T);
    Sb_res = -E^T P
  expanded WY producer (seven products; Sec. 2.3, "conventional WY backward"):
    Wb = -Rb S^T;  Ab = Rb Z^T + Wb E^T;  Mb = -A^T Ab A^T;  D = strict_lower(Mb);
    Eb_dir = A^T Wb;  Zb = A^T Rb;  Sb_res = -W^T Rb
  shared interaction contractions:
    Eb = Eb_dir + D Y;  Yb = Hb^T Qg + D^T E  with Hb = lower_incl(Ob R^T);
    Qgb = Ob S^T + Hb Y;  Ktb = R Sbn^T;  Sb = diag(gam_n) Sbn + Qg^T Ob + Sb_res
  feature-local chain rules:
    dq = gam Qgb;  dv = beta Zb;  dbeta = <Zb, v> + <Eb, gam k>  (undivided, App. B.3)
    dk = beta gam Eb + Yb / gam + exp(G_n - G) Ktb
    Gb = Qg Qgb + E Eb - Y Yb - Kt Ktb;  Gb_n += sum_j Kt_j Ktb_j + gam_n rowsum(S Sbn)
    scalar gate: Gb summed over features (App. E.1); dg = reverse cumsum of Gb (Sec. 3.5)
Consumers of D and Hb:
  "direct"   the dense D Y, D^T E, Hb Y, Hb^T Qg above;
  "gram"     Gram elimination for a scalar gate (Sec. 3.4): Gamma = D o Lam,
             Gq = Hb o Lam (Lam_ij = exp(G_i - G_j)), A_K = Gamma K,
             B_K = Gamma^T diag(beta) K; gate and beta terms from row inner
             products, no K K^T;
  "centred"  centred matrix intra for a vector gate (Sec. 3.3): c = (max G +
             min G)/2 per feature, alpha = exp(G - c), zeta = exp(c - G),
             Q' = alpha Q, E' = beta alpha K, Y' = zeta K;
             U_q = Hb Y', U_e = D Y', U_y = Hb^T Q' + D^T E'.
  "windowed" the centred factors applied per window of the chunk (16 tokens
             by default: one token tile of the device kernels) for a vector gate with
             strong decay: a block of two tokens in the same window uses that
             window's centre; the block of a later window's rows against an
             earlier window's columns uses a boundary pivot p (G at the last
             token of the earlier window for Hb Y' and D Y', at the first token
             of the later window for Hb^T Q' and D^T E'), for which G_i <= p <=
             G_j, so both factors exp(G_i - p) and exp(p - G_j) are at most 1
             when g <= 0. The factors then span exp(+-window range / 2) instead
             of exp(+-chunk range / 2). (Paper Sec. 3.3 centres per chunk; the
             windows are this implementation's reading of the "subchunk path"
             that the repository page's "Compatibility" section gives stronger
             gates.)
GDN2 (paper Table 1: independent vector erase and write gates in place of
the shared beta; pass ers (T, DK) and wrt (T, DV) with beta None): the same
forms with E = ers o gam o K and Z = wrt o V; the chain rules then give
dv = wrt o Zb, dwrt = v o Zb, dk's erase term ers o gam o Eb and
ders = gam o k o Eb, entry by entry (no sum over channels).
Readings where the pages are silent are the ones listed with the design notes:
decay before erase, inclusive output, key-major state, undivided dbeta.
"""
from __future__ import annotations

import numpy as np


class FlopCounter:
    """Counts dense matmul FLOPs (2 m n k, the pages' convention) per tag."""

    def __init__(self):
        self.by_tag: dict[str, int] = {}
        self.calls: dict[str, int] = {}

    def mm(self, a, b, tag="other"):
        m, k = a.shape
        k2, n = b.shape
        assert k == k2
        self.by_tag[tag] = self.by_tag.get(tag, 0) + 2 * m * n * k
        self.calls[tag] = self.calls.get(tag, 0) + 1
        return a @ b

    def __getitem__(self, tag):
        return self.by_tag.get(tag, 0)


def _tril(x, k):
    return np.tril(x, k)


def _chunks(T, C):
    return [(s, min(s + C, T)) for s in range(0, T, C)]


def _gate_parts(gc, vec, DK):
    """gc: log decays of one chunk, shape (n,) or (n, DK). Returns G (n, DK)."""
    G = np.cumsum(gc, axis=0)
    if not vec:
        G = np.repeat(G[:, None], DK, axis=1)
    return G


def _erase_write(beta, ers, wrt, s, e):
    """Per-row erase and write weights of rows s..e: (n, 1) columns of the
    shared beta, or the GDN2 gates (n, DK) and (n, DV)."""
    if ers is not None:
        return ers[s:e], wrt[s:e]
    b = beta[s:e][:, None]
    return b, b


def chunk_forward(q, k, v, g, beta, h0, C, keep=False, ers=None, wrt=None):
    """Chunkwise forward of one (b, h) sequence.

    q, k: (T, DK); v: (T, DV); g: (T,) or (T, DK); beta: (T,); h0: (DK, DV).
    GDN2: beta None, ers (T, DK), wrt (T, DV).
    Returns o (T, DV), ht (DK, DV) and, if keep, the per-chunk intermediates.
    """
    T, DK = q.shape
    DV = v.shape[1]
    vec = g.ndim == 2
    S = np.array(h0, dtype=np.float64, copy=True)
    o = np.zeros((T, DV))
    cache = []
    for s, e in _chunks(T, C):
        n = e - s
        Q, K, V = q[s:e], k[s:e], v[s:e]
        be, bw = _erase_write(beta, ers, wrt, s, e)
        G = _gate_parts(g[s:e], vec, DK)
        gam = np.exp(G)
        E = be * gam * K
        Y = K / gam
        Z = bw * V
        Qg = gam * Q
        Kt = np.exp(G[-1][None, :] - G) * K
        L = _tril(E @ Y.T, -1)
        A = np.linalg.inv(np.eye(n) + L)
        W = A @ E
        U = A @ Z
        R = U - W @ S
        Hm = _tril(Qg @ Y.T, 0)
        o[s:e] = Qg @ S + Hm @ R
        if keep:
            cache.append(dict(s=s, e=e, S=S.copy(), G=G, gam=gam, E=E, Y=Y, Z=Z, Qg=Qg, Kt=Kt,
                              L=L, A=A, W=W, U=U, R=R, Hm=Hm))
        S = gam[-1][:, None] * S + Kt.T @ R
    return (o, S, cache) if keep else (o, S)


def chunk_backward(q, k, v, g, beta, h0, dO, dht, C, producer="rewy", consumer="direct",
                   flops: FlopCounter | None = None, centre=None, window=16, ers=None, wrt=None):
    """Chunkwise backward of one (b, h) sequence.

    producer: "rewy" (three products) or "wy7" (expanded graph).
    consumer: "direct", "gram" (scalar gate only), "centred" or "windowed"
              (any gate).
    centre:   optional override of the centring constants, a function
              (G (n, DK)) -> c (DK,), used to test centring invariance.
    window:   window length of the "windowed" consumer.
    GDN2: beta None, ers (T, DK), wrt (T, DV) ("direct" and "windowed").
    Returns dict dq, dk, dv, dg, dbeta (GDN2: ders, dwrt), dh0.
    """
    fc = flops if flops is not None else FlopCounter()
    mm = fc.mm
    T, DK = q.shape
    DV = v.shape[1]
    vec = g.ndim == 2
    gdn2 = ers is not None
    if consumer == "gram" and vec:
        raise ValueError("Gram elimination applies to a scalar gate")
    if gdn2 and consumer not in ("direct", "windowed"):
        raise ValueError("GDN2 takes the direct or windowed consumer")
    _, _, cache = chunk_forward(q, k, v, g, beta, h0, C, keep=True, ers=ers, wrt=wrt)
    ders = np.zeros((T, DK)) if gdn2 else None
    dwrt = np.zeros((T, DV)) if gdn2 else None
    dq = np.zeros_like(q, dtype=np.float64)
    dk = np.zeros_like(k, dtype=np.float64)
    dv = np.zeros_like(v, dtype=np.float64)
    dbeta = np.zeros(T)
    dg = np.zeros((T, DK)) if vec else np.zeros(T)
    Sbn = np.zeros((DK, DV)) if dht is None else np.array(dht, dtype=np.float64)
    for ch in reversed(cache):
        s, e = ch["s"], ch["e"]
        S, G, gam, E, Y, Z, Qg, Kt, A, W, R, Hm = (ch[x] for x in (
            "S", "G", "gam", "E", "Y", "Z", "Qg", "Kt", "A", "W", "R", "Hm"))
        Q, K, V, Ob = q[s:e], k[s:e], v[s:e], dO[s:e]
        be, bw = _erase_write(beta, ers, wrt, s, e)
        bt = None if gdn2 else beta[s:e]
        de_c = np.zeros((e - s, DK))
        gn = gam[-1]
        Rb = Hm.T @ Ob + Kt @ Sbn
        # --- local WY producer ---
        if producer == "rewy":
            P = mm(A.T, Rb, "local_wy")
            Zb = P
            Eb = -mm(P, S.T, "local_wy")
            D = -_tril(mm(P, R.T, "local_wy"), -1)
            Sb_res = -E.T @ P
        elif producer == "wy7":
            Wb = -mm(Rb, S.T, "local_wy")
            Ab = mm(Rb, Z.T, "local_wy") + mm(Wb, E.T, "local_wy")
            Mb = -mm(mm(A.T, Ab, "local_wy"), A.T, "local_wy")
            D = _tril(Mb, -1)
            Eb = mm(A.T, Wb, "local_wy")
            Zb = mm(A.T, Rb, "local_wy")
            Sb_res = -W.T @ Rb
        else:
            raise ValueError(producer)
        Hb = _tril(Ob @ R.T, 0)
        # state-direct terms
        Qgb = Ob @ S.T
        Ktb = R @ Sbn.T
        Yb = np.zeros_like(Y)
        dq_c = np.zeros_like(Q)
        dk_c = np.zeros_like(K)
        db_c = np.zeros(e - s)
        Gb = np.zeros((e - s, DK))
        # --- consumers of D and Hb ---
        if consumer == "direct":
            Eb = Eb + D @ Y
            Yb = Yb + Hb.T @ Qg + D.T @ E
            Qgb = Qgb + Hb @ Y
        elif consumer == "gram":
            Gs = G[:, 0]
            Lam = np.tril(np.exp(Gs[:, None] - Gs[None, :]), 0)
            Gam = D * Lam
            Gq = Hb * Lam
            AK = Gam @ K
            BK = Gam.T @ (bt[:, None] * K)
            GqK = Gq @ K
            GqtQ = Gq.T @ Q
            dk_c += bt[:, None] * AK + BK + GqtQ
            dq_c += GqK
            db_c += np.sum(K * AK, axis=1)
            gl = bt * np.sum(K * AK, axis=1) - np.sum(K * BK, axis=1) \
                + np.sum(Q * GqK, axis=1) - np.sum(K * GqtQ, axis=1)
            Gb[:, 0] += gl  # scalar gate: all feature columns are summed below
        elif consumer == "windowed":
            n = e - s
            wins = [(a, min(a + window, n)) for a in range(0, n, window)]
            for ia, (a0, a1) in enumerate(wins):
                for ib, (b0, b1) in enumerate(wins[:ia + 1]):
                    Gi, Gj = G[a0:a1], G[b0:b1]          # rows i (later), columns j
                    if ia == ib:
                        c = 0.5 * (Gi.max(axis=0) + Gi.min(axis=0))
                        p_lo = p_up = c
                    else:
                        p_lo = G[b1 - 1]                 # last token of window b
                        p_up = G[a0]                     # first token of window a
                    Hb_ab, D_ab = Hb[a0:a1, b0:b1], D[a0:a1, b0:b1]
                    Ki, Qi, bi = K[a0:a1], Q[a0:a1], be[a0:a1]
                    Kj = K[b0:b1]
                    # rows i: Hb Y' and D Y', scaled back by exp(G_i - p_lo)
                    al = np.exp(Gi - p_lo)
                    Yp = np.exp(p_lo - Gj) * Kj
                    uq = al * (Hb_ab @ Yp)
                    ue = al * (D_ab @ Yp)
                    dq_c[a0:a1] += uq
                    dk_c[a0:a1] += bi * ue
                    if gdn2:
                        de_c[a0:a1] += ue * Ki
                    else:
                        db_c[a0:a1] += np.sum(ue * Ki, axis=1)
                    Gb[a0:a1] += Qi * uq + bi * Ki * ue
                    # columns j: Hb^T Q' + D^T E', scaled back by exp(p_up - G_j)
                    al2 = np.exp(Gi - p_up)
                    uy = np.exp(p_up - Gj) * (Hb_ab.T @ (al2 * Qi) + D_ab.T @ (bi * al2 * Ki))
                    dk_c[b0:b1] += uy
                    Gb[b0:b1] -= Kj * uy
        elif consumer == "centred":
            c = centre(G) if centre is not None else 0.5 * (G.max(axis=0) + G.min(axis=0))
            al = np.exp(G - c[None, :])
            ze = np.exp(c[None, :] - G)
            Qp = al * Q
            Ep = bt[:, None] * al * K
            Yp = ze * K
            Uq = Hb @ Yp
            Ue = D @ Yp
            Uy = Hb.T @ Qp + D.T @ Ep
            dq_c += al * Uq
            dk_c += bt[:, None] * al * Ue + ze * Uy
            db_c += np.sum(Ue * al * K, axis=1)
            Gb += Qp * Uq + Ep * Ue - Yp * Uy
        else:
            raise ValueError(consumer)
        # --- feature-local chain rules for the remaining terms ---
        dq_c += gam * Qgb
        dv[s:e] = bw * Zb
        if gdn2:
            dwrt[s:e] = Zb * V
            de_c += Eb * gam * K
            ders[s:e] = de_c
        else:
            db_c += np.sum(Zb * V, axis=1) + np.sum(Eb * gam * K, axis=1)
        dk_c += be * gam * Eb + Yb / gam + np.exp(G[-1][None, :] - G) * Ktb
        Gb += Qg * Qgb + E * Eb - Y * Yb - Kt * Ktb
        Gb[-1] += np.sum(Kt * Ktb, axis=0) + gn * np.sum(S * Sbn, axis=1)
        Gtok = Gb if vec else Gb.sum(axis=1)
        dg[s:e] = np.flip(np.cumsum(np.flip(Gtok, 0), axis=0), 0)
        dq[s:e] = dq_c
        dk[s:e] = dk_c
        dbeta[s:e] = db_c
        # --- reverse state scan ---
        Sbn = gn[:, None] * Sbn + Qg.T @ Ob + Sb_res
    if gdn2:
        return dict(dq=dq, dk=dk, dv=dv, dg=dg, ders=ders, dwrt=dwrt, dh0=Sbn)
    return dict(dq=dq, dk=dk, dv=dv, dg=dg, dbeta=dbeta, dh0=Sbn)


def pivoted_lower(X, Y, G, incl, tile=16):
    """lower((X o exp(G)) (Y o exp(-G))^T) of one chunk -- entries
    sum_f X_if Y_jf exp(G_if - G_jf) for j < i (j <= i if incl) -- formed tile
    by tile as a product of factors that stay in range under strong decay:
    a diagonal tile uses its rows' centre c = (max G + min G)/2, a tile below
    the diagonal the pivot p = G at the last row of its column tile, so that
    exp(G_i - p) <= 1 and exp(p - G_j) <= 1 when g <= 0. The per-chunk L and
    Hm of the forward (X = beta K or Q, Y = K) are formed this way on the
    device."""
    n = X.shape[0]
    out = np.zeros((n, n))
    tiles = [(a, min(a + tile, n)) for a in range(0, n, tile)]
    for ia, (a0, a1) in enumerate(tiles):
        for (b0, b1) in tiles[:ia + 1]:
            if b0 == a0:
                Ga = G[a0:a1]
                p = 0.5 * (Ga.max(axis=0) + Ga.min(axis=0))
            else:
                p = G[b1 - 1]
            out[a0:a1, b0:b1] = (np.exp(G[a0:a1] - p) * X[a0:a1]) @ (np.exp(p - G[b0:b1]) * Y[b0:b1]).T
    return np.tril(out, 0 if incl else -1)


def local_wy_flops(n: int, dk: int, dv: int, producer: str) -> tuple[int, int]:
    """(FLOPs, number of products) of the local WY producer, counted by running
    chunk_backward once on one random chunk of n tokens."""
    rng = np.random.default_rng(0)
    q = rng.standard_normal((n, dk))
    k = rng.standard_normal((n, dk)) / np.sqrt(dk)
    v = rng.standard_normal((n, dv))
    g = -0.01 * np.ones(n)
    beta = np.full(n, 0.5)
    h0 = rng.standard_normal((dk, dv))
    dO = rng.standard_normal((n, dv))
    fc = FlopCounter()
    chunk_backward(q, k, v, g, beta, h0, dO, None, n, producer=producer, flops=fc)
    return fc["local_wy"], fc.calls.get("local_wy", 0)

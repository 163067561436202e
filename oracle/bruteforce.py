"""Brute force in 50-digit arithmetic, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see the oracle package docstring).

Written independently of lt_oracle.c to pin it: scores and weights use
mpmath at 50 significant digits, the softmax denominator is the direct sum of
e^{s_ij} with no max-subtraction, and every quantity is taken from its plain
definition:
  * attention weight P_ij = e^{s_ij} / sum_{j'<=i} e^{s_ij'}, s_ij = scale q_i.k_j;
  * LSE_i = ln sum_{j<=i} e^{s_ij}; out_i = sum_j P_ij v_j;
  * lazy ratio of a row: sum of P_ij over keys j<S or i-R<j<=i
    (press-release page, "LightTransfer method": the weights from queries to
    the initial and the recent keys); per head, the mean over the last W rows;
  * streaming attention: the same softmax over only those keys.
"""
from __future__ import annotations

import mpmath as mp

mp.mp.dps = 50


def _mp(x):
    return mp.mpf(float(x))


def attention(q, k, v, S=0, R=1, W=0, scale=None):
    """q [B][Hq][N][D], k/v [B][Hkv][N][D] nested sequences (numbers).
    Returns a dict of nested lists of mpf values."""
    B, Hq, N, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Hkv = len(k[0])
    G = Hq // Hkv
    sc = mp.mpf(1) / mp.sqrt(D) if scale is None else _mp(scale)
    out, lse, sout, slse, lrows, lratio = [], [], [], [], [], []
    for b in range(B):
        ob, lb, sob, slb, lrb, lab = [], [], [], [], [], []
        for h in range(Hq):
            hk = h // G
            oh, lh, soh, slh, lrh = [], [], [], [], []
            for i in range(N):
                e = []
                for j in range(i + 1):
                    s = sc * mp.fsum(_mp(q[b][h][i][d]) * _mp(k[b][hk][j][d]) for d in range(D))
                    e.append(mp.e ** s)
                Z = mp.fsum(e)
                lh.append(mp.log(Z))
                oh.append([mp.fsum(e[j] / Z * _mp(v[b][hk][j][d]) for j in range(i + 1))
                           for d in range(D)])
                keep = [j for j in range(i + 1) if j < S or j > i - R]
                Zs = mp.fsum(e[j] for j in keep)
                slh.append(mp.log(Zs))
                soh.append([mp.fsum(e[j] / Zs * _mp(v[b][hk][j][d]) for j in keep)
                            for d in range(D)])
                if W and i >= N - W:
                    lrh.append(Zs / Z)
            ob.append(oh); lb.append(lh); sob.append(soh); slb.append(slh)
            if W:
                lrb.append(lrh)
                lab.append(mp.fsum(lrh) / W)
        out.append(ob); lse.append(lb); sout.append(sob); slse.append(slb)
        lrows.append(lrb); lratio.append(lab)
    res = {"out": out, "lse": lse, "sout": sout, "slse": slse}
    if W:
        res["lazy_rows"], res["lazy_ratio"] = lrows, lratio
    return res


def decode(q, k, v, scale=None):
    """q [B][Hq][D]; k/v [B][Hkv][L][D]: one query sees all L rows."""
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, L = len(k[0]), len(k[0][0])
    G = Hq // Hkv
    sc = mp.mpf(1) / mp.sqrt(D) if scale is None else _mp(scale)
    out, lse = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            hk = h // G
            e = [mp.e ** (sc * mp.fsum(_mp(q[b][h][d]) * _mp(k[b][hk][j][d]) for d in range(D)))
                 for j in range(L)]
            Z = mp.fsum(e)
            lb.append(mp.log(Z))
            ob.append([mp.fsum(e[j] / Z * _mp(v[b][hk][j][d]) for j in range(L)) for d in range(D)])
        out.append(ob); lse.append(lb)
    return {"out": out, "lse": lse}

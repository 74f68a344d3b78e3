"""Write tests/golden/tiny_mixer_mpmath.json: a tiny mixer evaluated at 50 digits.

This script does not import the oracle. It evaluates the mixer core from its
definition in a different form from the oracle's loops:

* the convolution with an explicit time index (tap j of K reads token t-(K-1)+j,
  falling back to the carried state, oldest first, before token 0);
* the scan as the unrolled sum over all earlier tokens with cumulative steps,
      h_t = exp(A * S(1, t)) h_0 + sum_{s<=t} exp(A * S(s+1, t)) * Bbar_s * u_s,
  S(a, b) = dt_a + ... + dt_b, which is what the recurrence of the Jamba page's
  "The Mamba Layer" section (discrete recurrence equation, ZOH equation) unrolls
  to; Bbar_s = dt_s * B_s (first order) or (exp(dt_s A) - 1) / A * B_s (ZOH);
* y_t = (sum_n C_t[n] h_t[n] + D u_t) * SiLU(z_t); RMSNorm per the page's
  "RMSNorm definition and placement" equation on the dt_low / B / C slices.

Inputs are small rationals from a fixed integer recipe below (no random module).
Run:  python tests/golden/make_tiny_mpmath.py
"""
from __future__ import annotations

import json
import os

import mpmath as mp

mp.mp.dps = 50

B_, L, D, N, K, R = 1, 6, 3, 2, 3, 2
EPS = mp.mpf("1e-6")


def rat(k, scale):
    """Deterministic small rational in [-scale, scale]: ((k * 37 + 11) mod 97 - 48) / 48 * scale."""
    return mp.mpf((k * 37 + 11) % 97 - 48) / 48 * mp.mpf(scale)


def build_inputs():
    c = iter(range(10_000))
    x = [[rat(next(c), 2) for _ in range(D)] for _ in range(L)]
    z = [[rat(next(c), 2) for _ in range(D)] for _ in range(L)]
    conv_w = [[rat(next(c), "0.5") for _ in range(K)] for _ in range(D)]
    conv_b = [rat(next(c), "0.5") for _ in range(D)]
    x_proj_w = [[rat(next(c), "0.7") for _ in range(D)] for _ in range(R + 2 * N)]
    dt_proj_w = [[rat(next(c), "0.7") for _ in range(R)] for _ in range(D)]
    dt_proj_b = [rat(next(c), 1) - 2 for _ in range(D)]
    A = [[-mp.mpf(n + 1) * (1 + rat(next(c), "0.25")) for n in range(N)] for _ in range(D)]
    Dskip = [1 + rat(next(c), "0.5") for _ in range(D)]
    dt_norm_w = [1 + rat(next(c), "0.5") for _ in range(R)]
    B_norm_w = [1 + rat(next(c), "0.5") for _ in range(N)]
    C_norm_w = [1 + rat(next(c), "0.5") for _ in range(N)]
    conv_state0 = [[rat(next(c), 1) for _ in range(K - 1)] for _ in range(D)]
    ssm_state0 = [[rat(next(c), 1) for _ in range(N)] for _ in range(D)]
    return dict(x=x, z=z, conv_w=conv_w, conv_b=conv_b, x_proj_w=x_proj_w,
                dt_proj_w=dt_proj_w, dt_proj_b=dt_proj_b, A=A, Dskip=Dskip,
                dt_norm_w=dt_norm_w, B_norm_w=B_norm_w, C_norm_w=C_norm_w,
                conv_state0=conv_state0, ssm_state0=ssm_state0)


def sig_mul(v):
    return v / (1 + mp.exp(-v))


def rms(vec, gamma):
    ms = mp.fsum(v * v for v in vec) / len(vec)
    den = mp.sqrt(ms + EPS)
    return [v / den * g for v, g in zip(vec, gamma)]


def evaluate(inp, zoh):
    x, z = inp["x"], inp["z"]

    def x_at(tau, i):
        if tau >= 0:
            return x[tau][i]
        return inp["conv_state0"][i][K - 1 + tau]

    u = [[sig_mul(inp["conv_b"][i] + mp.fsum(inp["conv_w"][i][j] * x_at(t - (K - 1) + j, i)
                                             for j in range(K)))
          for i in range(D)] for t in range(L)]
    dt, Bm, Cm = [], [], []
    for t in range(L):
        row = [mp.fsum(inp["x_proj_w"][r][i] * u[t][i] for i in range(D)) for r in range(R + 2 * N)]
        dl = rms(row[:R], inp["dt_norm_w"])
        Bm.append(rms(row[R:R + N], inp["B_norm_w"]))
        Cm.append(rms(row[R + N:], inp["C_norm_w"]))
        dt.append([mp.log(1 + mp.exp(mp.fsum(inp["dt_proj_w"][i][r] * dl[r] for r in range(R))
                                     + inp["dt_proj_b"][i])) for i in range(D)])

    def S(a, b, i):
        return mp.fsum(dt[r][i] for r in range(a, b + 1))

    y = [[None] * D for _ in range(L)]
    hL = [[None] * N for _ in range(D)]
    for i in range(D):
        for t in range(L):
            h = []
            for n in range(N):
                a = inp["A"][i][n]
                acc = mp.exp(a * S(0, t, i)) * inp["ssm_state0"][i][n]
                for s in range(t + 1):
                    if zoh:
                        bbar = (mp.exp(dt[s][i] * a) - 1) / a * Bm[s][n]
                    else:
                        bbar = dt[s][i] * Bm[s][n]
                    acc += mp.exp(a * S(s + 1, t, i)) * bbar * u[s][i]
                h.append(acc)
            y[t][i] = (mp.fsum(Cm[t][n] * h[n] for n in range(N)) + inp["Dskip"][i] * u[t][i]) \
                * sig_mul(z[t][i])
            if t == L - 1:
                hL[i] = h
    conv_state = [[x_at(L - (K - 1) + j, i) for j in range(K - 1)] for i in range(D)]
    return y, conv_state, hL


def s(v):
    return mp.nstr(v, 40)


def main():
    inp = build_inputs()
    out = {
        "source": "mpmath 50-digit evaluation of the unrolled mixer definition; "
                  "see make_tiny_mpmath.py for the formulas and the page passages they follow",
        "shape": dict(B=B_, L=L, D=D, N=N, K=K, R=R, eps="1e-6"),
        "inputs": {k: _tree(v) for k, v in inp.items()},
    }
    for zoh in (False, True):
        y, cs, hL = evaluate(inp, zoh)
        out["zoh" if zoh else "euler"] = {"y": _tree(y), "conv_state": _tree(cs),
                                          "ssm_state": _tree(hL)}
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_mixer_mpmath.json")
    with open(path, "w") as f:
        json.dump(out, f, indent=1)
    print("wrote", path)


def _tree(v):
    if isinstance(v, list):
        return [_tree(e) for e in v]
    return s(v)


if __name__ == "__main__":
    main()

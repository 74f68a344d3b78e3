"""fp64 oracle of the mixer core's gradients -- TEST INFRASTRUCTURE (see oracle/__init__.py).

The gradients of the scalar loss  l = sum_{b,t,i} dy[b,t,i] * y[b,t,i],  with y the output of
mixer_f64.mixer_prefill, with respect to xz, every parameter and the two carried states: the
backward pass that training through the parallel scan needs ([Jamba] "Parallel training via the
parallel scan"). The forward steps are those of mixer_f64 (conv1d + SiLU, x_proj, the three
RMSNorms, dt_proj + softplus, the selective scan with D feed-through and the SiLU(z) gate); this
module takes them in reverse order and applies the chain rule to each, in the forward's notation:

  gate        y = ys * SiLU(z), ys = y_ssm + D u
  scan        h_t = Abar_t h_{t-1} + Bbar_t u_t, y_ssm_t = C_t . h_t, Abar = exp(dt A),
              Bbar = dt B (first order) or expm1(dt A) / A * B (ZOH)
              so  dh_t = C_t dys_t + Abar_{t+1} dh_{t+1}  (reverse recurrence, dh_L+1 = 0)
  softplus    dt = softplus(p)  ->  dp = ddt * sigmoid(p)
  RMSNorm     o = v / r * g, r = sqrt(mean(v^2) + eps)
              ->  dv = g do / r - v sum(g do v) / (n r^3),  dg = sum_t do v / r
  projections out = a @ W^T  ->  da = dout @ W,  dW = dout^T @ a
  conv + SiLU u = SiLU(q), q_t = b + sum_k w_k xt_{t+k}  ->  dq = du SiLU'(q),
              dxt_{t+k} += w_k dq_t,  dw_k = sum_t dq_t xt_{t+k},  db = sum_t dq_t

SiLU'(v) = s (1 + v (1 - s)) with s = sigmoid(v). The SSM states h are recomputed forward from
checkpoints kept every `ckpt` tokens (a plain memory bound, no change to any value). numpy's
matmul is the library primitive for the products. Pinned against central finite differences of
mixer_prefill (tests/test_oracle_backward.py).
"""
from __future__ import annotations

import numpy as np

from .mixer_f64 import rmsnorm, silu


def _sigmoid(v):
    v = np.asarray(v, np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-v))


def _dsilu(v):
    s = _sigmoid(v)
    return s * (1.0 + v * (1.0 - s))


def _softplus(v):
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def _rmsnorm_backward(v, gamma, eps, do):
    """v: [L, n] pre-norm values, do: [L, n] gradient of the normalised output.
    Returns (dv [L, n], dgamma [n])."""
    n = v.shape[-1]
    r = np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    gdo = do * gamma
    dv = gdo / r - v * np.sum(gdo * v, axis=-1, keepdims=True) / (n * r ** 3)
    dg = np.sum(do * v / r, axis=0)
    return dv, dg


def mixer_prefill_backward(xz, p, dy, conv_state0=None, ssm_state0=None, eps=1e-6, zoh=False,
                           ckpt=64):
    """Gradients of sum(dy * y), y = mixer_prefill(xz, p, conv_state0, ssm_state0)[0].

    xz [B, L, 2D], dy [B, L, D]; p as for mixer_prefill (float64 arrays); states or None (zeros).
    Returns a dict: xz [B, L, 2D], conv_w [D, K], conv_b [D] (None when p has no conv_b),
    x_proj_w [R+2N, D], dt_proj_w [D, R], dt_proj_b [D], A [D, N], Dskip [D], dt_norm_w [R],
    B_norm_w [N], C_norm_w [N], conv_state0 [B, D, K-1], ssm_state0 [B, D, N].
    """
    xz = np.asarray(xz, np.float64)
    dy = np.asarray(dy, np.float64)
    B_, L, D2 = xz.shape
    D = D2 // 2
    A = p["A"]
    N = A.shape[1]
    R = p["dt_proj_w"].shape[1]
    K = p["conv_w"].shape[1]
    w, Wx, Wdt = p["conv_w"], p["x_proj_w"], p["dt_proj_w"]
    has_b = p.get("conv_b") is not None
    g = {"xz": np.zeros_like(xz), "conv_w": np.zeros_like(w),
         "conv_b": np.zeros(D) if has_b else None, "x_proj_w": np.zeros_like(Wx),
         "dt_proj_w": np.zeros_like(Wdt), "dt_proj_b": np.zeros(D), "A": np.zeros_like(A),
         "Dskip": np.zeros(D), "dt_norm_w": np.zeros(R), "B_norm_w": np.zeros(N),
         "C_norm_w": np.zeros(N), "conv_state0": np.zeros((B_, D, K - 1)),
         "ssm_state0": np.zeros((B_, D, N))}
    for b in range(B_):
        # ---- forward, keeping what the backward needs
        x, z = xz[b, :, :D], xz[b, :, D:]
        pre = np.zeros((K - 1, D)) if conv_state0 is None else np.asarray(conv_state0[b]).T
        xt = np.concatenate([pre, x], axis=0)                      # [L + K - 1, D]
        q = np.zeros((L, D))
        for k in range(K):
            q += w[:, k] * xt[k:k + L]
        if has_b:
            q += p["conv_b"]
        u = silu(q)
        xd = u @ Wx.T
        va, vb, vc = xd[:, :R], xd[:, R:R + N], xd[:, R + N:]
        dtn = rmsnorm(va, p["dt_norm_w"], eps)
        Bm = rmsnorm(vb, p["B_norm_w"], eps)
        Cm = rmsnorm(vc, p["C_norm_w"], eps)
        pdt = dtn @ Wdt.T + p["dt_proj_b"]
        dt = _softplus(pdt)
        h0 = np.zeros((D, N)) if ssm_state0 is None else np.asarray(ssm_state0[b], np.float64)

        def step(t, h):
            dtA = dt[t][:, None] * A
            Ab = np.exp(dtA)
            Bb = (np.expm1(dtA) / A if zoh else dt[t][:, None]) * Bm[t][None, :]
            return Ab * h + Bb * u[t][:, None], Ab, dtA

        cks = {}
        h = h0.copy()
        ys = np.empty((L, D))
        for t in range(L):
            if t % ckpt == 0:
                cks[t] = h.copy()
            h, _, _ = step(t, h)
            ys[t] = h @ Cm[t] + p["Dskip"] * u[t]

        # ---- gate
        dz = dy[b] * ys * _dsilu(z)
        dys = dy[b] * silu(z)
        g["Dskip"] += np.sum(dys * u, axis=0)
        du = dys * p["Dskip"]
        # ---- scan, in reverse, the states of each checkpoint block recomputed forward
        ddt = np.zeros((L, D))
        dB = np.zeros((L, N))
        dC = np.zeros((L, N))
        carry = np.zeros((D, N))                                  # Abar_{t+1} dh_{t+1}
        for t0 in sorted(cks, reverse=True):
            t1 = min(L, t0 + ckpt)
            hs = [cks[t0]]
            for t in range(t0, t1):
                hs.append(step(t, hs[-1])[0])                     # hs[k] = h_{t0 + k - 1}
            for t in range(t1 - 1, t0 - 1, -1):
                hprev, hcur = hs[t - t0], hs[t - t0 + 1]
                _, Ab, dtA = step(t, hprev)
                dC[t] = dys[t] @ hcur
                dh = Cm[t][None, :] * dys[t][:, None] + carry
                dAb = dh * hprev                                  # d/dAbar
                dBb = dh * u[t][:, None]                          # d/dBbar
                du[t] += np.sum(dh * (np.expm1(dtA) / A * Bm[t][None, :] if zoh
                                      else dt[t][:, None] * Bm[t][None, :]), axis=1)
                # Abar = exp(dt A)
                ddt[t] += np.sum(dAb * Ab * A, axis=1)
                g["A"] += dAb * Ab * dt[t][:, None]
                if zoh:   # Bbar = expm1(dt A) / A * B
                    E = np.expm1(dtA)
                    ddt[t] += np.sum(dBb * Ab * Bm[t][None, :], axis=1)
                    g["A"] += dBb * Bm[t][None, :] * (dtA * Ab - E) / (A * A)
                    dB[t] = np.sum(dBb * E / A, axis=0)
                else:     # Bbar = dt B
                    ddt[t] += np.sum(dBb * Bm[t][None, :], axis=1)
                    dB[t] = np.sum(dBb * dt[t][:, None], axis=0)
                carry = Ab * dh
        g["ssm_state0"][b] = carry
        # ---- dt_proj + softplus
        dp = ddt * _sigmoid(pdt)
        g["dt_proj_b"] += np.sum(dp, axis=0)
        g["dt_proj_w"] += dp.T @ dtn
        ddtn = dp @ Wdt
        # ---- the three RMSNorms
        dva, dg = _rmsnorm_backward(va, p["dt_norm_w"], eps, ddtn)
        g["dt_norm_w"] += dg
        dvb, dg = _rmsnorm_backward(vb, p["B_norm_w"], eps, dB)
        g["B_norm_w"] += dg
        dvc, dg = _rmsnorm_backward(vc, p["C_norm_w"], eps, dC)
        g["C_norm_w"] += dg
        dxd = np.concatenate([dva, dvb, dvc], axis=1)
        # ---- x_proj
        g["x_proj_w"] += dxd.T @ u
        du += dxd @ Wx
        # ---- conv + SiLU
        dq = du * _dsilu(q)
        if has_b:
            g["conv_b"] += np.sum(dq, axis=0)
        dxt = np.zeros((L + K - 1, D))
        for k in range(K):
            g["conv_w"][:, k] += np.sum(dq * xt[k:k + L], axis=0)
            dxt[k:k + L] += w[:, k] * dq
        g["xz"][b, :, :D] = dxt[K - 1:]
        g["xz"][b, :, D:] = dz
        g["conv_state0"][b] = dxt[:K - 1].T
    return g

"""fp64 oracle of the Mamba-1 mixer core -- TEST INFRASTRUCTURE (see oracle/__init__.py).

Notation follows the Jamba analysis page's SSM section with the mixer's names:
h = SSM state, u = post-conv SSM input, x / z = the two halves of xz, dt = the step
the page calls Delta. Shapes: L tokens, D = d_inner channels, N = d_state,
K = d_conv, R = dt_rank.
"""
from __future__ import annotations

import numpy as np


def silu(v):
    """SiLU(v) = v * sigmoid(v) = v / (1 + e^-v).  [Mamba-1] gate and conv activation
    (not written out on the pages)."""
    v = np.asarray(v, dtype=np.float64)
    with np.errstate(over="ignore"):
        return v / (1.0 + np.exp(-v))


def softplus(v):
    """softplus(v) = log(1 + e^v), written as max(v, 0) + log1p(e^-|v|), an exact
    identity that never overflows.  [Mamba-1] maps dt_proj's output to a positive
    step (the pages only say Delta comes from a small learned linear layer,
    [Jamba] "The selective mechanism")."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def rmsnorm(v, gamma, eps):
    """RMSNorm(v) = v / sqrt(mean(v^2) + eps) * gamma over the last axis.
    [Jamba] "RMSNorm definition and placement", RMSNorm equation; applied to the
    mixer's internal activations per "Stabilization: RMSNorm in Mamba layers"."""
    v = np.asarray(v, dtype=np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * np.asarray(gamma, dtype=np.float64)


def causal_conv1d_silu(x, w, b=None, state0=None):
    """Causal depthwise conv1d followed by SiLU, for one sequence.  [Mamba-1]

    x: [L, D]; w: [D, K] with tap K-1 on the current token; b: [D] or None;
    state0: [D, K-1], the K-1 inputs before x, oldest first, or None for zeros.
    u[t, i] = SiLU(b_i + sum_k w[i, k] * xt[t + k, i]) with xt = concat(state0^T, x).
    Returns (u [L, D], final state [D, K-1] = last K-1 rows of xt, oldest first).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    L, D = x.shape
    K = w.shape[1]
    pre = np.zeros((K - 1, D)) if state0 is None else np.asarray(state0, np.float64).T
    xt = np.concatenate([pre, x], axis=0)
    acc = np.zeros((L, D))
    for k in range(K):
        acc += w[:, k] * xt[k:k + L]
    if b is not None:
        acc += np.asarray(b, dtype=np.float64)
    return silu(acc), xt[L:L + K - 1].T.copy()


def x_proj(u, w_x):
    """xdbl[t, :] = W_x u[t, :]: the 'small learned linear layer' that makes B, C and
    (a low-rank) Delta functions of the token.  [Jamba] "The selective mechanism"."""
    return np.asarray(u, np.float64) @ np.asarray(w_x, np.float64).T


def split_xdbl(xdbl, R, N):
    """Rows of x_proj are [dt_low (R) | B (N) | C (N)] (reading: order not given on the pages)."""
    return xdbl[..., :R], xdbl[..., R:R + N], xdbl[..., R + N:R + 2 * N]


def dt_proj_softplus(dt_low, w_dt, bias):
    """dt[t, i] = softplus(W_dt[i, :] . dt_low[t, :] + bias_i).  [Mamba-1]; Delta per
    token and channel, [Jamba] "From scalar SSM to vector processing"."""
    pre = np.asarray(dt_low, np.float64) @ np.asarray(w_dt, np.float64).T
    return softplus(pre + np.asarray(bias, np.float64))


def selective_scan(u, dt, A, Bm, Cm, Dskip, z, h0=None, zoh=False):
    """The selective SSM over one sequence, one time step after another.

    [Jamba] "The Mamba Layer": each channel i runs its own scalar SSM ("From scalar
    SSM to vector processing") with diagonal A[i, :] of N states; ZOH gives
    Abar = exp(Delta A) (ZOH equation); the discrete recurrence is
    h_t = Abar h_{t-1} + Bbar u_t, y_t = C h_t (recurrence equation), and the
    continuous model's feed-through adds D u_t (continuous SSM equation).
    Bbar = Delta * B (first-order, the default) or, with zoh=True, the page's
    ZOH form (Delta A)^-1 (exp(Delta A) - 1) Delta B = expm1(Delta A) / A * B.
    The output is gated: y_t <- y_t * SiLU(z_t)  [Mamba-1].

    u, dt, z: [L, D]; A: [D, N]; Bm, Cm: [L, N] (shared by all channels of a token);
    Dskip: [D]; h0: [D, N] or None. Returns (y [L, D], h_L [D, N]).
    """
    u = np.asarray(u, np.float64)
    dt = np.asarray(dt, np.float64)
    A = np.asarray(A, np.float64)
    Bm = np.asarray(Bm, np.float64)
    Cm = np.asarray(Cm, np.float64)
    Dskip = np.asarray(Dskip, np.float64)
    L, D = u.shape
    N = A.shape[1]
    h = np.zeros((D, N)) if h0 is None else np.array(h0, dtype=np.float64)
    y = np.empty((L, D))
    for t in range(L):
        dtA = dt[t][:, None] * A
        Abar = np.exp(dtA)
        if zoh:
            Bbar = np.expm1(dtA) / A * Bm[t][None, :]
        else:
            Bbar = dt[t][:, None] * Bm[t][None, :]
        h = Abar * h + Bbar * u[t][:, None]
        y[t] = h @ Cm[t] + Dskip * u[t]
    return y * silu(z), h


def as_f64_params(p: dict) -> dict:
    """Convert a parameter dict (torch tensors or arrays, any dtype) to float64 arrays."""
    out = {}
    for k, v in p.items():
        if v is None:
            out[k] = None
        elif hasattr(v, "detach"):
            out[k] = v.detach().to("cpu").double().numpy()
        else:
            out[k] = np.asarray(v, dtype=np.float64)
    return out


def mixer_prefill(xz, p, conv_state0=None, ssm_state0=None, eps=1e-6, zoh=False,
                  channels=None, token_block=None, workers=1):
    """The whole mixer core over a batch of sequences.

    xz: [B, L, 2D] (x = first half, z = second half); p: dict of float64 arrays
    (conv_w [D,K], conv_b [D] or None, x_proj_w [R+2N, D], dt_proj_w [D, R],
    dt_proj_b [D], A [D, N], Dskip [D], dt_norm_w [R], B_norm_w [N], C_norm_w [N]);
    conv_state0: [B, D, K-1] or None; ssm_state0: [B, D, N] or None.

    channels: optional index array; when given, y and the SSM state are computed
    only for those channels (the convolution and x_proj still cover every channel,
    since B, C and dt_low depend on all of them). token_block / workers split the
    convolution + x_proj + RMSNorm pass into independent token blocks (each takes its
    K-1 preceding inputs from x, or from the carried state before token 0) evaluated
    on a thread pool; neither changes any result. The scan itself is sequential.

    Returns (y [B, L, Dsel], conv_state [B, D, K-1], ssm_state [B, Dsel, N]).
    """
    B_, L, D2 = xz.shape
    D = D2 // 2
    N = p["A"].shape[1]
    R = p["dt_proj_w"].shape[1]
    K = p["conv_w"].shape[1]
    sel = np.arange(D) if channels is None else np.asarray(channels)
    tb = L if token_block is None else token_block
    ys, css, sss = [], [], []
    for b in range(B_):
        state0 = None if conv_state0 is None else np.asarray(conv_state0[b], np.float64)
        u_sel = np.empty((L, len(sel)))
        dtlow = np.empty((L, R))
        Bm = np.empty((L, N))
        Cm = np.empty((L, N))

        def run_block(t0, b=b, state0=state0):
            # conv + SiLU for all channels, x_proj, RMSNorm of each slice, for tokens [t0, t1)
            t1 = min(L, t0 + tb)
            if t0 == 0:
                pre = state0
            else:
                lo = max(0, t0 - (K - 1))
                rows = _f64(xz[b, lo:t0, :D])
                if rows.shape[0] < K - 1:  # the window reaches back before token 0
                    head = (np.zeros((K - 1, D)) if state0 is None else state0.T)
                    rows = np.concatenate([head[rows.shape[0]:], rows], axis=0)
                pre = rows.T
            u, _ = causal_conv1d_silu(_f64(xz[b, t0:t1, :D]), p["conv_w"], p.get("conv_b"), pre)
            xd = x_proj(u, p["x_proj_w"])
            a, bb, c = split_xdbl(xd, R, N)
            dtlow[t0:t1] = rmsnorm(a, p["dt_norm_w"], eps)
            Bm[t0:t1] = rmsnorm(bb, p["B_norm_w"], eps)
            Cm[t0:t1] = rmsnorm(c, p["C_norm_w"], eps)
            u_sel[t0:t1] = u[:, sel]

        starts = list(range(0, L, tb))
        if workers > 1 and len(starts) > 1:
            import concurrent.futures
            import threadpoolctl
            # one BLAS thread per block: the pool supplies the parallelism
            with threadpoolctl.threadpool_limits(1), \
                    concurrent.futures.ThreadPoolExecutor(max_workers=workers) as ex:
                list(ex.map(run_block, starts))
        else:
            for t0 in starts:
                run_block(t0)
        # final conv state: the last K-1 inputs of concat(state0, x), oldest first
        tail = _f64(xz[b, max(0, L - (K - 1)):L, :D])
        if tail.shape[0] < K - 1:
            head = np.zeros((K - 1, D)) if state0 is None else state0.T
            tail = np.concatenate([head[tail.shape[0]:], tail], axis=0)
        state = tail.T.copy()
        dt = dt_proj_softplus(dtlow, p["dt_proj_w"][sel], p["dt_proj_b"][sel])
        z = _f64(xz[b][:, D + sel])
        h0 = None if ssm_state0 is None else np.asarray(ssm_state0[b], np.float64)[sel]
        y, h = selective_scan(u_sel, dt, p["A"][sel], Bm, Cm, p["Dskip"][sel], z, h0, zoh)
        ys.append(y)
        css.append(state)
        sss.append(h)
    return np.stack(ys), np.stack(css), np.stack(sss)


def mixer_decode_step(xz_t, p, conv_state, ssm_state, eps=1e-6, zoh=False, channels=None):
    """One recurrent token for every sequence: the prefill with L = 1 and the carried
    states.  [Jamba] "Inference behavior (generation)": the state updates from
    h_{t-1} to h_t with the new token, with no re-scan of the past.

    xz_t: [B, 2D]. Returns (y [B, Dsel], conv_state [B, D, K-1], ssm_state [B, Dsel, N]).
    """
    xz_t = _f64(xz_t)
    y, cs, ss = mixer_prefill(xz_t[:, None, :], p, conv_state, ssm_state, eps, zoh, channels)
    return y[:, 0], cs, ss


def _f64(a):
    if hasattr(a, "detach"):
        return a.detach().to("cpu").double().numpy()
    return np.asarray(a, dtype=np.float64)

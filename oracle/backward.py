"""Backward pass of the recurrence in fp64 -- TEST INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may use this
module (see the package header). It shares nothing with the HIP library.

`forward(p)` runs the recurrence of the pages once more, plainly, on fp64 copies
of the inputs (so finite differences can perturb them): per (batch b, head h)
and token t, with alpha = e^{dt A}, gamma = lambda dt, delta = (1 - lambda) dt
(the exponential-trapezoidal rule: "复值SSM × 广义梯形离散 × MIMO，线性模型的全面重构",
§2.2; "Mamba-3架构技术解析：新一代语言建模的范式转移", §2.1), u_t = B_t x_t^T (MIMO
rank R, digest §2.3), the pair rotation Rot(dt omega) of the complex state
(digest §2.1; Rot = [[c, -s], [s, c]] on rows (2k, 2k+1)):

    g_t = h_{t-1} + delta_t u_{t-1}
    h_t = alpha_t Rot(dt_t omega) g_t + gamma_t u_t
    y_t = h_t^T C_t + D x_t

It is pinned to the C oracle (m3_oracle.c) on the same inputs.

`backward(p, dy, dh_out)` is the reverse-mode derivative of that loop, taken
step by step in reverse (the adjoint a_t of h_t):

    a_t   += C_t dy_t^T                        (y_t reads h_t)
    dC_t   = h_t dy_t,  dD += <dy_t, x_t>,  dx_t += D dy_t
    with w_t = h_t - gamma_t u_t  (= alpha_t Rot g_t):
      d alpha_t alpha_t = <w_t, a_t>            -> d dt += A <w, a>,  d A += dt <w, a>
      d theta_{t,k}     = <J w_t, a_t>_pair k   (J turns a pair by 90 degrees)
                                                -> d dt += sum_k omega_k d theta_k,  d omega_k += dt d theta_k
      d gamma_t         = <u_t, a_t>
    dg_t   = alpha_t Rot(dt omega)^T a_t
    du_t   = gamma_t a_t + delta_{t+1} dg_{t+1}
    d delta_t = <u_{t-1}, dg_t>
    a_{t-1} = dg_t
    dB_t = du_t x_t,  dx_t += du_t^T B_t
and gamma = lambda dt, delta = (1 - lambda) dt give d lambda and the rest of
d dt. dh0 = a_0, and the carry (B_0, x_0) of the token before the first gets
du_0 = delta_1 dg_1. Gradients of B, C (and of carry_B) are summed over the
heads of a group. The tests check every gradient against central finite
differences of `forward`.
"""
from __future__ import annotations

import numpy as np


def _np64(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return a.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(a, dtype=np.float64)


def _unpack(p):
    q = {k: _np64(p.get(k)) for k in ("x", "B", "C", "dt", "lam", "A", "omega", "D", "h0", "carry_B", "carry_x")}
    b, L, H, R, P = q["x"].shape
    G, N = q["B"].shape[2], q["B"].shape[4]
    return q, (b, L, H, G, R, P, N)


def _rot(v, c, s):
    """Turn the row pairs (2k, 2k+1) of v [N][P] by the angles with cosines c, sines s [N/2]."""
    out = np.empty_like(v)
    out[0::2] = c[:, None] * v[0::2] - s[:, None] * v[1::2]
    out[1::2] = s[:, None] * v[0::2] + c[:, None] * v[1::2]
    return out


def _walk(q, dims, bb, h, keep=False):
    """Forward for one (batch, head): y [L][R][P], h_L, and the states h_t (t = 1..L) when keep."""
    b, L, H, G, R, P, N = dims
    g_ = h // (H // G)
    A, D = q["A"][h], q["D"][h]
    om = q["omega"][h]
    hs = np.zeros((N, P)) if q["h0"] is None else q["h0"][bb, h].copy()
    if q["carry_B"] is not None:
        u_prev = q["carry_B"][bb, g_].T @ q["carry_x"][bb, h]  # [N][R] @ [R][P]
    else:
        u_prev = np.zeros((N, P))
    ys = np.empty((L, R, P))
    states = np.empty((L, N, P)) if keep else None
    for t in range(L):
        dt, lam = q["dt"][bb, t, h], q["lam"][bb, t, h]
        Bt, xt, Ct = q["B"][bb, t, g_], q["x"][bb, t, h], q["C"][bb, t, g_]   # [R][N], [R][P], [R][N]
        u = Bt.T @ xt
        g = hs + (1.0 - lam) * dt * u_prev
        hs = np.exp(dt * A) * _rot(g, np.cos(dt * om), np.sin(dt * om)) + lam * dt * u
        ys[t] = Ct @ hs + D * xt
        if keep:
            states[t] = hs
        u_prev = u
    return ys, hs, states


def forward(p):
    """y [b][L][H][R][P] and h_L [b][H][N][P] in fp64."""
    q, dims = _unpack(p)
    b, L, H, G, R, P, N = dims
    y = np.empty((b, L, H, R, P))
    hL = np.empty((b, H, N, P))
    for bb in range(b):
        for h in range(H):
            y[bb, :, h], hL[bb, h], _ = _walk(q, dims, bb, h)
    return y, hL


def backward(p, dy, dh_out=None):
    """Gradients of the loss <dy, y> + <dh_out, h_L> with respect to every input.

    Returns a dict with x, B, C, dt, lam, A, omega, D, h0 (always, as if h0 = 0
    when none was given), carry_B, carry_x (None without a carry), in fp64.
    """
    q, dims = _unpack(p)
    b, L, H, G, R, P, N = dims
    dy = _np64(dy)
    dhL = None if dh_out is None else _np64(dh_out)
    gr = {"x": np.zeros_like(q["x"]), "B": np.zeros_like(q["B"]), "C": np.zeros_like(q["C"]),
          "dt": np.zeros_like(q["dt"]), "lam": np.zeros_like(q["lam"]), "A": np.zeros(H),
          "omega": np.zeros_like(q["omega"]), "D": np.zeros(H), "h0": np.zeros((b, H, N, P)),
          "carry_B": None if q["carry_B"] is None else np.zeros_like(q["carry_B"]),
          "carry_x": None if q["carry_x"] is None else np.zeros_like(q["carry_x"])}
    for bb in range(b):
        for h in range(H):
            g_ = h // (H // G)
            A, D = q["A"][h], q["D"][h]
            om = q["omega"][h]
            _, _, states = _walk(q, dims, bb, h, keep=True)
            a = np.zeros((N, P)) if dhL is None else dhL[bb, h].copy()
            e = np.zeros((N, P))  # delta_{t+1} dg_{t+1}: the next step's share of du_t
            for t in range(L - 1, -1, -1):
                dt, lam = q["dt"][bb, t, h], q["lam"][bb, t, h]
                Bt, xt, Ct = q["B"][bb, t, g_], q["x"][bb, t, h], q["C"][bb, t, g_]
                dyt = dy[bb, t, h]                                # [R][P]
                ht = states[t]
                u = Bt.T @ xt
                if t > 0:
                    u_prev = q["B"][bb, t - 1, g_].T @ q["x"][bb, t - 1, h]
                elif q["carry_B"] is not None:
                    u_prev = q["carry_B"][bb, g_].T @ q["carry_x"][bb, h]
                else:
                    u_prev = np.zeros((N, P))
                # y_t = h_t^T C_t + D x_t
                a = a + Ct.T @ dyt
                gr["C"][bb, t, g_] += (ht @ dyt.T).T            # [R][N]
                gr["D"][h] += np.sum(dyt * xt)
                gr["x"][bb, t, h] += D * dyt
                # h_t = alpha Rot(theta) g_t + gamma u_t
                alpha = np.exp(dt * A)
                c, s = np.cos(dt * om), np.sin(dt * om)
                w = ht - lam * dt * u                          # alpha Rot g
                s_alpha = np.sum(w * a)                        # d alpha * alpha
                dtheta = np.sum(-w[1::2] * a[0::2] + w[0::2] * a[1::2], axis=1)  # [N/2]
                s_gamma = np.sum(u * a)
                dg = alpha * _rot(a, c, -s)                    # Rot(theta)^T a
                du = lam * dt * a + e
                s_delta = np.sum(u_prev * dg)
                # scalars
                gr["dt"][bb, t, h] += A * s_alpha + np.sum(om * dtheta) + lam * s_gamma + (1.0 - lam) * s_delta
                gr["lam"][bb, t, h] += dt * (s_gamma - s_delta)
                gr["A"][h] += dt * s_alpha
                gr["omega"][h] += dt * dtheta
                # u_t = B_t x_t^T
                gr["B"][bb, t, g_] += (du @ xt.T).T            # [R][N]
                gr["x"][bb, t, h] += Bt @ du                     # [R][P]
                a = dg
                e = (1.0 - lam) * dt * dg
            gr["h0"][bb, h] = a
            if q["carry_B"] is not None:
                gr["carry_B"][bb, g_] += (e @ q["carry_x"][bb, h].T).T
                gr["carry_x"][bb, h] += q["carry_B"][bb, g_] @ e
    return gr

"""fp64 model of the bf16 backward's rounding points (test helper).

The bf16 backward kernels round at fixed points: the forward's output O
(bf16, so D_i = dO_i . O_i uses the rounded O), the probabilities P fed to
the dV product, P again where the dk/dv kernel hands it from the wave that
computes it to the wave that forms dS for dK (fp16), the score gradients dS
fed to the dQ and dK products, and the gradients themselves.  ``rounded_backward`` evaluates the backward in
fp64 with exactly those rounding points and no other error, so its distance
from the exact oracle is the floor any correct kernel with these rounding
points reaches on the same inputs.  It is dense (masked S x S matrices), for
the small cases of the tests only.
"""
from __future__ import annotations

import numpy as np
import torch

BF16 = torch.bfloat16


def rb(x: np.ndarray) -> np.ndarray:
    """Round to bf16 (nearest-even) and back to fp64."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(BF16).double().numpy()


def rh(x: np.ndarray) -> np.ndarray:
    """Round to fp16 (nearest-even) and back to fp64."""
    return np.ascontiguousarray(x).astype(np.float16).astype(np.float64)


def rounded_backward(q, k, v, sink, dout, W, rnd=rb, rnd_out=None, rnd_pk=None):
    """fp64 backward with the bf16 kernels' rounding points (see the module
    notes); ``rnd`` is the rounding applied at each of them, ``rnd_out`` (if
    given) the one applied to the forward's O instead, ``rnd_pk`` the one of
    the P that forms dS for dK (default: fp16 when ``rnd`` is bf16, else
    ``rnd``)."""
    r_o = rnd if rnd_out is None else rnd_out
    r_pk = (rh if rnd is rb else rnd) if rnd_pk is None else rnd_pk
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D)
    i = np.arange(S)[:, None]
    j = np.arange(S)[None, :]
    vis = (j <= i) & (j > i - W)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dsink = np.zeros(Hq)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            x = scale * (q[b, :, h] @ k[b, :, g].T)
            x = np.where(vis, x, -np.inf)
            s = sink[h]
            M = np.maximum(x.max(axis=1), s)
            e = np.exp(x - M[:, None])
            es = 0.0 if np.isneginf(s) else np.exp(s - M)
            lse = M + np.log(e.sum(axis=1) + es)
            P = np.exp(x - lse[:, None])
            O = r_o(P @ v[b, :, g])                               # forward output, bf16
            Di = (dout[b, :, h] * O).sum(axis=1)
            Pb = rnd(P)
            dv[b, :, g] += Pb.T @ dout[b, :, h]
            dP = dout[b, :, h] @ v[b, :, g].T
            dS = rnd(P * (dP - Di[:, None]))
            dSk = rnd(r_pk(P) * (dP - Di[:, None]))
            dq[b, :, h] = scale * (dS @ k[b, :, g])
            dk[b, :, g] += scale * (dSk.T @ q[b, :, h])
            if not np.isneginf(s):
                dsink[h] -= (np.exp(s - lse) * Di).sum()
    return rnd(dq), rnd(dk), rnd(dv), dsink


def scaled_error(got, ref):
    rms = np.sqrt((ref ** 2).mean())
    return float((np.abs(got - ref) / (rms + np.abs(ref) + 1e-30)).max())

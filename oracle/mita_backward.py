"""CPU oracle for the gradient of the MiTA forward pass: dQ, dK, dV.

TEST INFRASTRUCTURE ONLY.  Imported by ``tests/`` (and by nothing on the
product path); it shares no code with the GPU path.

What is differentiated.  The pages train MiTA models end to end (MiTA
tutorial (iwxt.cn), ch.7: LRA training time; paper section 4) but write no
backward pass.  The forward (``mita_oracle``) has two selection steps, the
top-k keys of each landmark (step 3) and the top-s landmarks of each query
(step 5).  Both are piecewise constant in the inputs, so wherever the choice
is unique their derivative is zero and the gradient flows only through the
values they pick.  Readings (each listed in the design notes):

* the experts I [m, k] and routes e [N, s] are held fixed (passed in);
* q~ is rounded to the input dtype in the forward; the backward takes that
  rounding as the identity, so dQ receives d q~_i / |W_i| for every token of
  window W_i (pooling's adjoint; windows may overlap);
* the shared values v~_i = softmax_j(q~_i . k_j / sqrt(d)) V over all N keys
  are differentiated exactly (they depend on Q through q~ and on all of K, V);
* the joint softmax of each query over its m shared entries (q~_i, v~_i) and
  s k routed entries (k_j, v_j) is differentiated exactly, a key chosen by
  two experts counting twice, as in the forward.

How.  The forward is restated with torch float64 tensors and differentiated
by torch.autograd (a library primitive).  To bound memory it runs in two
parts: the joint softmax per chunk of queries, with q~ and v~ as leaves, then
the pooling and the shared-value softmax from those leaves' gradients back to
Q, K and V.  The restated forward is checked against ``mita_oracle.attend``
and the gradients against central differences of ``mita_oracle``'s forward
(tests/test_oracle_backward.py).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from oracle import mita_oracle as mo

__all__ = ["pool_matrix", "backward", "forward_fixed", "joint_lse", "landmark_lse",
           "ORACLE_IS_TEST_INFRASTRUCTURE"]

ORACLE_IS_TEST_INFRASTRUCTURE = True

_F64 = torch.float64


def pool_matrix(grid_h: int, grid_w: int, land_h: int, land_w: int) -> torch.Tensor:
    """[m, N] averaging matrix: row i holds 1 / |W_i| on the tokens of window W_i
    (the windows of step 1, mita_oracle.pool_windows)."""
    wins = mo.pool_windows(grid_h, grid_w, land_h, land_w)
    P = torch.zeros((len(wins), grid_h * grid_w), dtype=_F64)
    for i, w in enumerate(wins):
        P[i, w] = 1.0 / len(w)
    return P


def _landmarks(Q, grid_h, grid_w, land_h, land_w, dtype):
    """q~ with the forward's value (rounded to dtype) and pooling's gradient."""
    exact = pool_matrix(grid_h, grid_w, land_h, land_w) @ Q
    rounded = torch.from_numpy(mo.round_to_dtype(exact.detach().numpy(), dtype))
    return exact + (rounded - exact).detach()


def _shared_values(Qt, K, V):
    """v~_i = softmax_j(q~_i . k_j / sqrt(d)) V over all N keys (step 4)."""
    d = K.shape[1]
    return torch.softmax(Qt @ K.T / math.sqrt(d), dim=1) @ V


def _joint(q, K, V, Qt, Vt, I, e_rows, variant):
    """Outputs of a chunk of queries: one softmax over [shared; routed] entries
    (step 6).  e_rows [n, s] are the chunk's routes."""
    n, d = q.shape
    s = e_rows.shape[1]
    k = I.shape[1]
    sel = torch.from_numpy(np.asarray(I)[np.asarray(e_rows)].reshape(n, s * k))
    Kr, Vr = K[sel], V[sel]                                    # [n, s k, d]
    raw = torch.einsum("nd,njd->nj", q, Kr) / math.sqrt(d)
    if variant == "routed":
        w = torch.softmax(raw, dim=1)
        return torch.einsum("nj,njd->nd", w, Vr)
    sh = math.sqrt(d) if variant == "paper" else float(d)
    logits = torch.cat([q @ Qt.T / sh, raw], dim=1)
    w = torch.softmax(logits, dim=1)
    m = Qt.shape[0]
    return w[:, :m] @ Vt + torch.einsum("nj,njd->nd", w[:, m:], Vr)


def _check(variant, I, e, N, m):
    if variant not in ("paper", "official", "routed"):
        raise ValueError("variant must be 'paper', 'official' or 'routed'")
    I = np.asarray(I)
    e = np.asarray(e)
    if I.shape[0] != m or e.shape[0] != N:
        raise ValueError("I must be [m, k] and e [N, s]")
    return I, e


def forward_fixed(Q, K, V, grid_h, grid_w, land_h, land_w, I, e, dtype="bf16", variant="paper"):
    """O [N, d] of the torch restatement (no gradient), for checking it
    against mita_oracle.attend."""
    Q, K, V = (torch.tensor(np.asarray(x, dtype=np.float64)) for x in (Q, K, V))
    I, e = _check(variant, I, e, Q.shape[0], land_h * land_w)
    Qt = _landmarks(Q, grid_h, grid_w, land_h, land_w, dtype)
    Vt = _shared_values(Qt, K, V)
    return _joint(Q, K, V, Qt, Vt, I, e, variant).numpy()


def backward(Q, K, V, dO, grid_h, grid_w, land_h, land_w, I, e, dtype="bf16", variant="paper", chunk=1024):
    """(dQ, dK, dV), each [N, d] float64: the gradient of sum(O * dO) with
    respect to Q, K and V, with I and e held fixed (see the module notes)."""
    Q, K, V = (torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in (Q, K, V))
    dO = torch.tensor(np.asarray(dO, dtype=np.float64))
    N, d = Q.shape
    I, e = _check(variant, I, e, N, land_h * land_w)
    Qt = _landmarks(Q, grid_h, grid_w, land_h, land_w, dtype)
    Vt = _shared_values(Qt, K, V)
    Qt_l = Qt.detach().requires_grad_()
    Vt_l = Vt.detach().requires_grad_()
    for n0 in range(0, N, chunk):
        n1 = min(N, n0 + chunk)
        O = _joint(Q[n0:n1], K, V, Qt_l, Vt_l, I, e[n0:n1], variant)
        (O * dO[n0:n1]).sum().backward()
    pairs = [(t, g) for t, g in ((Qt, Qt_l.grad), (Vt, Vt_l.grad)) if g is not None and t.requires_grad]
    if pairs:
        torch.autograd.backward([t for t, _ in pairs], [g for _, g in pairs])
    out = []
    for x in (Q, K, V):
        out.append(x.grad.numpy() if x.grad is not None else np.zeros((N, d)))
    return tuple(out)


def joint_lse(Q, K, Qt, I, e, variant="paper"):
    """[N] natural log-sum-exp of each query's joint logits (step 6)."""
    Q, K, Qt = (np.asarray(x, dtype=np.float64) for x in (Q, K, Qt))
    N, d = Q.shape
    I, e = _check(variant, I, e, N, Qt.shape[0])
    out = np.empty(N)
    sh = math.sqrt(d) if variant == "paper" else float(d)
    for n in range(N):
        sel = np.concatenate([I[x] for x in e[n]])
        l = K[sel] @ Q[n] / math.sqrt(d)
        if variant != "routed":
            l = np.concatenate([Qt @ Q[n] / sh, l])
        mx = l.max()
        out[n] = mx + math.log(np.exp(l - mx).sum())
    return out


def landmark_lse(Qt, K):
    """[m] natural log-sum-exp of each landmark row's scores over all N keys
    (the normaliser of step 4)."""
    S = mo.landmark_scores(Qt, K)
    mx = S.max(axis=1)
    return mx + np.log(np.exp(S - mx[:, None]).sum(axis=1))

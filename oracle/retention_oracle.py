"""fp64 CPU oracle for multi-scale retention — TEST INFRASTRUCTURE ONLY.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import or call anything in this directory.  The library itself never
does: it has no CPU fallback.  Nothing here shares code with the HIP kernels.

What is computed (per batch b and head h, all in float64):

    Y_n = sum_{m <= n} gamma^(n-m) (Q_n . K_m) V_m  +  gamma^(n+1) Q_n S_in

The first term is the retention definition written out on "Retentive Networks
— Microsoft Propone l'Alternativa Architetturale ai Transformer" (aimpact
page, section "Il meccanismo: Multi-Scale Retention"); the same section gives
the recurrent form S_n = gamma S_(n-1) + K_n^T V_n, Y_n = Q_n S_n, says that
the parallel, recurrent and chunkwise forms are mathematically equivalent, and
that gamma is a hyperparameter per head.  The second term is what the
recurrence produces when it starts from a state S_in instead of zero (the
pages are silent on the initial state; zero is the default here).

Readings taken where the pages are silent (each also pinned by a test):
  * m = n is included: Y_n uses S_n after adding K_n^T V_n.
  * gamma^0 = 1 even for gamma = 0 (the diagonal of the decay mask is kept).
  * no 1/sqrt(d) scale, no normalisation and no denominator inside the
    operator (the author answer to Q3 on the paperhub page says Eq. (1) has no
    denominator, unlike RFA-Gate and linear attention), no softmax and no clamp
    (the answer to Q2 there says retention scores may be negative).
  * causal only (the closing list on the paperhub page: GPT settings, no
    bidirectional use).
  * the state has shape d_k x d_v (the answer to Q1 on inference cost there).

Functions
  recurrent(q, k, v, gamma, state_in)       -- oracle of record (recurrent form)
  recurrent_step(q, k, v, gamma, state)     -- one decode step of that form
  parallel(q, k, v, gamma, state_in)        -- brute-force parallel form
  chunkwise(q, k, v, gamma, C, state_in)    -- chunkwise form (derived, see below)
  chunk_state_contribution(...)             -- helper of the chunkwise form
  recurrent_backward(q, k, v, gamma, dy, state_in, dstate_out)
                                            -- gradients of the recurrent form
                                               (chain rule; the pages give none)
  group_norm(y, weight, bias, eps)          -- per-head GroupNorm of the output

Tensors are torch tensors (any float dtype, any device is copied to the CPU)
with layouts q, k: [B,H,T,d_k]; v: [B,H,T,d_v]; state: [B,H,d_k,d_v];
gamma: [H].  Inputs are upcast exactly to float64 before any arithmetic.

Parity status: every function above is pinned by tests/test_oracle.py against
closed forms, a pure-Python brute force of the definition, and invariants;
recurrent_backward against central finite differences of ``recurrent`` and
the exact homogeneity identities of the operator (y is linear in q; y and the
final state are linear in k, in v and in the initial state taken apart);
group_norm against torch's group_norm routine, hand values and invariants.
"""
from __future__ import annotations

import torch

__all__ = ["recurrent", "recurrent_step", "parallel", "chunkwise", "chunk_state_contribution",
           "recurrent_backward", "group_norm"]


def _f64(x: torch.Tensor) -> torch.Tensor:
    return x.detach().to(device="cpu", dtype=torch.float64)


def _gamma64(gamma, H: int) -> torch.Tensor:
    g = torch.as_tensor(gamma).detach().to(device="cpu", dtype=torch.float64).reshape(-1)
    if g.numel() != H:
        raise ValueError(f"gamma has {g.numel()} entries, expected one per head ({H})")
    return g


def _check(q, k, v):
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("expected q,k [B,H,T,dk] and v [B,H,T,dv]")


def recurrent(q, k, v, gamma, state_in=None):
    """Recurrent form, the oracle of record.

    Follows the recurrence of the aimpact page ("Il meccanismo: Multi-Scale
    Retention"): S_n = gamma S_(n-1) + K_n^T V_n, then Y_n = Q_n S_n, with
    S_(-1) = state_in (zeros when None).  K_n^T V_n is the outer product of the
    1 x d_k key row and the 1 x d_v value row.

    Returns (y [B,H,T,dv] float64, state_out [B,H,dk,dv] float64).
    """
    _check(q, k, v)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = _gamma64(gamma, H).view(1, H, 1, 1)
    S = torch.zeros(B, H, dk, dv, dtype=torch.float64) if state_in is None else _f64(state_in).clone()
    y = torch.empty(B, H, T, dv, dtype=torch.float64)
    for n in range(T):
        # S_n = gamma * S_(n-1) + K_n^T V_n
        S = g * S + k[:, :, n, :, None] * v[:, :, n, None, :]
        # Y_n = Q_n S_n  (a 1 x d_k row times the d_k x d_v state)
        y[:, :, n, :] = torch.einsum("bhk,bhkv->bhv", q[:, :, n, :], S)
    return y, S


def recurrent_step(q, k, v, gamma, state):
    """One decode step of the recurrent form (same passage as ``recurrent``).

    q, k: [B,H,dk]; v: [B,H,dv]; state: [B,H,dk,dv].  Returns
    (y [B,H,dv], new_state), both float64; the input state is not modified.
    """
    q, k, v, S = _f64(q), _f64(k), _f64(v), _f64(state)
    H = q.shape[1]
    g = _gamma64(gamma, H).view(1, H, 1, 1)
    S_new = g * S + k[:, :, :, None] * v[:, :, None, :]
    y = torch.einsum("bhk,bhkv->bhv", q, S_new)
    return y, S_new


def parallel(q, k, v, gamma, state_in=None):
    """Brute-force parallel form: Y = ((Q K^T) * D) V (+ diag(gamma^(n+1)) Q S_in).

    The aimpact page says the parallel form computes the whole retention matrix
    at once, like attention; the decay mask is read off the definition
    sum_(m<=n) gamma^(n-m): D[n,m] = gamma^(n-m) for n >= m, else 0, with
    D[n,n] = 1 also when gamma = 0.  The state term is the contribution of an
    initial state S_in carried through n+1 applications of the recurrence.

    Builds the T x T mask explicitly (O(T^2) memory): small inputs only.
    Returns y [B,H,T,dv] float64.
    """
    _check(q, k, v)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    g = _gamma64(gamma, H)
    n = torch.arange(T, dtype=torch.float64)
    diff = n[:, None] - n[None, :]                       # n - m
    causal = diff >= 0
    D = torch.zeros(H, T, T, dtype=torch.float64)
    for h in range(H):
        p = torch.where(causal, diff, torch.zeros_like(diff))
        Dh = torch.pow(g[h].expand(T, T), p)             # gamma^(n-m); pow(0, 0) == 1
        D[h] = torch.where(causal, Dh, torch.zeros_like(Dh))
    scores = torch.matmul(q, k.transpose(-1, -2))        # Q K^T, [B,H,T,T]
    y = torch.matmul(scores * D.unsqueeze(0), v)
    if state_in is not None:
        S0 = _f64(state_in)
        xi = torch.pow(g.view(H, 1), (n + 1.0).view(1, T))   # gamma^(n+1), [H,T]
        y = y + xi.view(1, H, T, 1) * torch.matmul(q, S0)
    return y


def chunk_state_contribution(k_c, v_c, g):
    """sum_{j<L} gamma^(L-1-j) K_j^T V_j for one chunk of length L (float64).

    k_c [B,H,L,dk], v_c [B,H,L,dv], g [H] -> [B,H,dk,dv].  This is the state
    the recurrence builds over the chunk when it starts from zero.
    """
    L = k_c.shape[2]
    H = k_c.shape[1]
    j = torch.arange(L, dtype=torch.float64)
    zeta = torch.pow(g.view(H, 1), (L - 1 - j).view(1, L))   # [H, L]
    return torch.matmul(k_c.transpose(-1, -2), zeta.view(1, H, L, 1) * v_c)


def chunkwise(q, k, v, gamma, C, state_in=None):
    """Chunkwise form with chunk length C (the last chunk may be shorter).

    The aimpact page describes this form only in words: the sequence is cut
    into blocks of length C, processed in parallel inside a block and
    recurrently across blocks.  Unrolling the recurrence inside chunk i
    (rows iC .. iC+L-1, R_i = state after the previous chunk) gives, for the
    row j of the chunk,

        S_(iC+j) = gamma^(j+1) R_i + sum_{t<=j} gamma^(j-t) K_t^T V_t,

    hence Y_[i] = ((Q_[i] K_[i]^T) * D_L) V_[i] + diag(gamma^(j+1)) Q_[i] R_i and
    R_(i+1) = gamma^L R_i + sum_j gamma^(L-1-j) K_j^T V_j.

    Returns (y [B,H,T,dv] float64, state_out [B,H,dk,dv] float64).
    """
    _check(q, k, v)
    if int(C) < 1:
        raise ValueError("chunk length must be >= 1")
    C = int(C)
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    g = _gamma64(gamma, H)
    R = torch.zeros(B, H, dk, dv, dtype=torch.float64) if state_in is None else _f64(state_in).clone()
    y = torch.empty(B, H, T, dv, dtype=torch.float64)
    for s in range(0, T, C):
        e = min(s + C, T)
        L = e - s
        qc, kc, vc = q[:, :, s:e], k[:, :, s:e], v[:, :, s:e]
        # intra-chunk: the parallel form on the chunk alone
        y_intra = parallel(qc, kc, vc, g)
        # cross-chunk: gamma^(j+1) Q_j R_i
        j = torch.arange(L, dtype=torch.float64)
        xi = torch.pow(g.view(H, 1), (j + 1.0).view(1, L))
        y[:, :, s:e] = y_intra + xi.view(1, H, L, 1) * torch.matmul(qc, R)
        # state carried to the next chunk
        R = torch.pow(g, float(L)).view(1, H, 1, 1) * R + chunk_state_contribution(kc, vc, g)
    return y, R


def recurrent_backward(q, k, v, gamma, dy, state_in=None, dstate_out=None):
    """Gradients of the recurrent form (the training use of the operator).

    The aimpact page says the parallel form is the one parallelised for
    training; it gives no backward pass, so this is the chain rule applied to
    the recurrence of ``recurrent`` (S_n = gamma S_(n-1) + K_n^T V_n,
    Y_n = Q_n S_n, S_(-1) = state_in, state_out = S_(T-1)) for the scalar
    L = sum_n <dY_n, Y_n> + <dS_out, state_out>:

        G_n      = dL/dS_n = Q_n^T dY_n + gamma G_(n+1)   (G_(T-1) also gets dS_out)
        dQ_n     = dY_n S_n^T
        dK_n     = G_n V_n^T,  i.e. dK_n[d] = sum_c G_n[d,c] V_n[c]
        dV_n     = K_n G_n
        dS_in    = gamma G_0                               (dS_out when T = 0)

    dy: [B,H,T,dv]; dstate_out: [B,H,dk,dv] or None (zeros).  Returns
    (dq [B,H,T,dk], dk [B,H,T,dk], dv [B,H,T,dv], dstate_in [B,H,dk,dv]), float64.
    """
    _check(q, k, v)
    q, k, v, dy = _f64(q), _f64(k), _f64(v), _f64(dy)
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    if dy.shape != v.shape:
        raise ValueError("dy must have the shape of v")
    g = _gamma64(gamma, H).view(1, H, 1, 1)
    # forward sweep: the states S_n, used at once for dQ_n
    S = torch.zeros(B, H, dk, dv, dtype=torch.float64) if state_in is None else _f64(state_in).clone()
    gq = torch.empty(B, H, T, dk, dtype=torch.float64)
    for n in range(T):
        S = g * S + k[:, :, n, :, None] * v[:, :, n, None, :]
        gq[:, :, n, :] = torch.einsum("bhv,bhkv->bhk", dy[:, :, n, :], S)
    # reverse sweep: carry = gradient reaching S_n from later steps (dS_out at n = T-1)
    carry = torch.zeros(B, H, dk, dv, dtype=torch.float64) if dstate_out is None else _f64(dstate_out).clone()
    gk = torch.empty(B, H, T, dk, dtype=torch.float64)
    gv = torch.empty(B, H, T, dv, dtype=torch.float64)
    for n in reversed(range(T)):
        G = carry + q[:, :, n, :, None] * dy[:, :, n, None, :]       # G_n
        gk[:, :, n, :] = torch.einsum("bhkv,bhv->bhk", G, v[:, :, n, :])
        gv[:, :, n, :] = torch.einsum("bhk,bhkv->bhv", k[:, :, n, :], G)
        carry = g * G                                                 # reaches S_(n-1)
    return gq, gk, gv, carry


def group_norm(y, weight=None, bias=None, eps=1e-5):
    """Per-head GroupNorm of the retention output.

    The paperhub page (author answer A4, on the GroupNorm of Eq. 8) says that
    multi-scale retention normalises with GroupNorm rather than LayerNorm
    because different heads have different statistics: each head is one
    group.  So for every (b, h, t) the d_v outputs of head h are normalised
    together:
        mu = mean_c y[c],  var = mean_c (y[c] - mu)^2   (biased, as GroupNorm)
        out[c] = (y[c] - mu) / sqrt(var + eps) * weight[h, c] + bias[h, c]
    weight, bias: per-channel affine [H, d_v] (None: 1 and 0).
    y: [B,H,T,dv].  Returns float64 [B,H,T,dv].
    """
    y = _f64(y)
    if y.dim() != 4:
        raise ValueError("expected y [B,H,T,dv]")
    H, dv = y.shape[1], y.shape[3]
    mu = y.mean(dim=-1, keepdim=True)
    var = ((y - mu) ** 2).mean(dim=-1, keepdim=True)
    out = (y - mu) / torch.sqrt(var + float(eps))
    if weight is not None:
        out = out * _f64(weight).reshape(1, H, 1, dv)
    if bias is not None:
        out = out + _f64(bias).reshape(1, H, 1, dv)
    return out

"""fp64 CPU oracle for the E2-TTT chunk-parallel fast-weight update.

TEST INFRASTRUCTURE.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import or call this module.  It shares no
code with the GPU library (no kernels, headers, helpers or tables) and never
imports it; the only module both sides use is the seeded input generator.

Source.  "Rethinking Expressivity and Efficiency in Test-Time Training"
(E2-TTT, arXiv 2608.21308).  The pages describe the method in prose only:

* abstract (arxivlens / mlsanity / searcharxiv pages): gradients of the
  fast-weight loss are taken at the chunk-start weights, and a closed-form
  state transition gives exactly the chunk-end fast weight and momentum of the
  per-token recurrence;
* atlas summary, "Approach": unrolling the recurrence with per-token learning
  rate, momentum and decay yields two scalar kernels (a momentum kernel and a
  weight kernel), evaluated with log-space cumulative sums, plus two weighted
  gradient aggregations;
* arxivlens, "Limitations" and atlas, "Surprising findings": the output of a
  chunk is computed from the chunk-start weights;
* atlas, "Key results": the fast weight is an MLP or a SwiGLU block.

The pages print no equations.  The recurrence is fixed here as

    M_t = beta_t * M_{t-1} + eta_t * g_t,      W_t = alpha_t * W_{t-1} - M_t,

with g_t the gradient of token t's loss at the chunk-start weights W0.  This
is the *definition* (``brute_force``); ``chunk_forward`` is the closed form
derived from it (method as the pages describe it), and the two are pinned
against each other in the tests.

Closed form for one chunk of tokens i = 1..C (products over an empty range
are 1):

    m_i   = prod_{s=i+1..C} beta_s                        (momentum kernel)
    w_i   = sum_{tau=i..C} prod_{s=tau+1..C} alpha_s * prod_{s=i+1..tau} beta_s
                                                          (weight kernel)
    A     = prod_s alpha_s,   Bb = prod_s beta_s,
    gamma = sum_{tau=1..C} prod_{s>tau} alpha_s * prod_{s<=tau} beta_s
    G^M   = sum_i m_i eta_i g_i,    G^W = sum_i w_i eta_i g_i
    M_C   = Bb * M0 + G^M,          W_C = A * W0 - gamma * M0 - G^W

Derivation: M_t = beta(0:t] M0 + sum_{i<=t} beta(i:t] eta_i g_i and
W_C = alpha(0:C] W0 - sum_tau alpha(tau:C] M_tau; substitute and swap sums.

Fast weights and losses (per token, k and v are D-vectors):

* linear:  y = W k, W in R^{D x D}
* mlp:     y = W2 silu(W1 k), W1 in R^{Hd x D}, W2 in R^{D x Hd}
* swiglu:  y = (silu(k W1) * (k W3)) W2 (row vectors),
           W1, W3 in R^{D x Hd}, W2 in R^{Hd x D}
* losses:  "mse" 0.5 ||y - v||^2,  "negdot" -<y, v>

Packing of the per-(b, h) parameter vector P (fp32 on the device, fp64
here): linear W; mlp W1 | W2; swiglu W1 | W3 | W2, each row-major.

Variants (flags of ``chunk_forward``):

* ``momentum=False``: the recurrence without momentum,
  W_t = alpha_t * W_{t-1} - eta_t * g_t (beta and M0 are not used).  The
  pages name no-momentum token weights among the official code's functions;
  the plainest reading is the momentum rule with M removed.  Closed form:
  w_i = prod_{s=i+1..C} alpha_s, A = prod alpha, W_C = A W0 - sum_i w_i eta_i g_i.
* a ragged tail (T % chunk != 0): the last chunk holds the remaining
  T mod chunk tokens and takes the same closed form over them (the pages
  name a tail-length helper among the official code's functions; the
  plainest reading is a shorter last chunk).
* ``chunk_avg=True``: the chunk-averaged variant the pages report as an
  ablation (atlas, "Surprising findings").  Reading: the per-token kernel values m_i and w_i are replaced by
  their mean over the chunk, the per-token learning rate eta_i is kept, and
  the chunk scalars A, Bb, gamma are unchanged.  It is defined by this closed
  form (there is no per-token recurrence behind it).

Parity status: every public function is pinned by ``tests/test_oracle_pins.py``
(brute force, limits alpha=beta=1, beta=0 and C=1 with autograd gradients,
geometric-sum closed forms, semigroup, resume, finite differences,
linearity; a ragged tail against the brute force and against a separate
call on the remainder; for the variants: the no-momentum brute force and autograd SGD,
and for the chunk average its C=1 and equal-token reductions to the
per-token form and its alpha=beta=1 closed form).  No function here is
"parity unpinned".
"""
from __future__ import annotations

import numpy as np

KINDS = ("linear", "mlp", "swiglu")
LOSSES = ("mse", "negdot")


# ----------------------------------------------------------------------------
# parameter packing
# ----------------------------------------------------------------------------

def param_count(kind: str, D: int, Hd: int) -> int:
    if kind == "linear":
        return D * D
    if kind == "mlp":
        return 2 * D * Hd
    if kind == "swiglu":
        return 3 * D * Hd
    raise ValueError(f"unknown kind {kind!r}")


def unpack(kind: str, p: np.ndarray, D: int, Hd: int) -> dict:
    """Split packed parameters p[..., P] into named matrices (views)."""
    lead = p.shape[:-1]
    if kind == "linear":
        return {"W": p.reshape(*lead, D, D)}
    if kind == "mlp":
        n = D * Hd
        return {"W1": p[..., :n].reshape(*lead, Hd, D),
                "W2": p[..., n:2 * n].reshape(*lead, D, Hd)}
    if kind == "swiglu":
        n = D * Hd
        return {"W1": p[..., :n].reshape(*lead, D, Hd),
                "W3": p[..., n:2 * n].reshape(*lead, D, Hd),
                "W2": p[..., 2 * n:3 * n].reshape(*lead, Hd, D)}
    raise ValueError(f"unknown kind {kind!r}")


def pack(kind: str, mats: dict) -> np.ndarray:
    names = {"linear": ("W",), "mlp": ("W1", "W2"), "swiglu": ("W1", "W3", "W2")}[kind]
    parts = []
    for nm in names:
        m = mats[nm]
        parts.append(m.reshape(*m.shape[:-2], -1))
    return np.concatenate(parts, axis=-1)


# ----------------------------------------------------------------------------
# fast weight forward / backward
# ----------------------------------------------------------------------------

def sigmoid(x):
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def silu(x):
    return x * sigmoid(x)


def dsilu(x):
    s = sigmoid(x)
    return s * (1.0 + x * (1.0 - s))


def fast_weight_forward(kind: str, mats: dict, X: np.ndarray) -> np.ndarray:
    """y = f_W(x) for every row of X[..., N, D] (leading dims broadcast)."""
    if kind == "linear":
        return X @ np.swapaxes(mats["W"], -1, -2)
    if kind == "mlp":
        a = silu(X @ np.swapaxes(mats["W1"], -1, -2))
        return a @ np.swapaxes(mats["W2"], -1, -2)
    if kind == "swiglu":
        u = silu(X @ mats["W1"]) * (X @ mats["W3"])
        return u @ mats["W2"]
    raise ValueError(kind)


def _dloss_dy(loss: str, Y: np.ndarray, V: np.ndarray) -> np.ndarray:
    if loss == "mse":
        return Y - V
    if loss == "negdot":
        return -V
    raise ValueError(loss)


def grad_factors(kind: str, loss: str, mats: dict, K: np.ndarray, V: np.ndarray) -> dict:
    """Per-token backward factors at weights ``mats`` for tokens K, V [..., N, D].

    Token i's gradient is a sum of outer products of these rows:
      linear: g_W  = dy_i k_i^T
      mlp:    g_W2 = dy_i a_i^T,  g_W1 = dz_i k_i^T
      swiglu: g_W1 = k_i^T dh1_i, g_W3 = k_i^T dh3_i, g_W2 = u_i^T dy_i
    """
    if kind == "linear":
        Y = K @ np.swapaxes(mats["W"], -1, -2)
        return {"dy": _dloss_dy(loss, Y, V)}
    if kind == "mlp":
        z = K @ np.swapaxes(mats["W1"], -1, -2)
        a = silu(z)
        Y = a @ np.swapaxes(mats["W2"], -1, -2)
        dy = _dloss_dy(loss, Y, V)
        dz = (dy @ mats["W2"]) * dsilu(z)
        return {"dy": dy, "a": a, "dz": dz}
    if kind == "swiglu":
        h1 = K @ mats["W1"]
        h3 = K @ mats["W3"]
        u = silu(h1) * h3
        Y = u @ mats["W2"]
        dy = _dloss_dy(loss, Y, V)
        du = dy @ np.swapaxes(mats["W2"], -1, -2)
        dh1 = du * h3 * dsilu(h1)
        dh3 = du * silu(h1)
        return {"dy": dy, "u": u, "dh1": dh1, "dh3": dh3}
    raise ValueError(kind)


def weighted_grad_sum(kind: str, fac: dict, K: np.ndarray, c: np.ndarray) -> dict:
    """sum_i c_i g_i for per-token weights c[..., N] (one gradient aggregation)."""
    cc = c[..., :, None]
    T = lambda x: np.swapaxes(x, -1, -2)
    if kind == "linear":
        return {"W": T(cc * fac["dy"]) @ K}
    if kind == "mlp":
        return {"W1": T(cc * fac["dz"]) @ K, "W2": T(cc * fac["dy"]) @ fac["a"]}
    if kind == "swiglu":
        return {"W1": T(K) @ (cc * fac["dh1"]), "W3": T(K) @ (cc * fac["dh3"]),
                "W2": T(cc * fac["u"]) @ fac["dy"]}
    raise ValueError(kind)


def token_grads(kind: str, loss: str, mats: dict, K: np.ndarray, V: np.ndarray) -> dict:
    """Explicit per-token gradients as stacked matrices [..., N, *shape]."""
    fac = grad_factors(kind, loss, mats, K, V)
    o = lambda a, b: a[..., :, :, None] * b[..., :, None, :]
    if kind == "linear":
        return {"W": o(fac["dy"], K)}
    if kind == "mlp":
        return {"W1": o(fac["dz"], K), "W2": o(fac["dy"], fac["a"])}
    return {"W1": o(K, fac["dh1"]), "W3": o(K, fac["dh3"]), "W2": o(fac["u"], fac["dy"])}


# ----------------------------------------------------------------------------
# scalar kernels (direct products, fp64)
# ----------------------------------------------------------------------------

def chunk_coefficients(alpha: np.ndarray, beta: np.ndarray):
    """Momentum kernel m, weight kernel w and chunk scalars A, Bb, gamma.

    alpha, beta: [..., C] gates of the chunk's tokens in order.  Every
    quantity is evaluated as a plain product or sum of products, in fp64.
    """
    alpha = np.asarray(alpha, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    C = alpha.shape[-1]
    # a_i = prod_{s>i} alpha_s ; m_i = prod_{s>i} beta_s
    a = np.ones_like(alpha)
    m = np.ones_like(beta)
    if C > 1:
        a[..., :-1] = np.cumprod(alpha[..., ::-1], axis=-1)[..., :-1][..., ::-1]
        m[..., :-1] = np.cumprod(beta[..., ::-1], axis=-1)[..., :-1][..., ::-1]
    w = np.empty_like(alpha)
    for i in range(C):
        # prod_{s=i+1..tau} beta_s for tau = i..C-1
        pb = np.ones(alpha.shape[:-1] + (C - i,))
        if C - i > 1:
            pb[..., 1:] = np.cumprod(beta[..., i + 1:], axis=-1)
        w[..., i] = np.sum(a[..., i:] * pb, axis=-1)
    A = np.prod(alpha, axis=-1)
    Bb = np.prod(beta, axis=-1)
    gamma = np.sum(a * np.cumprod(beta, axis=-1), axis=-1)
    return m, w, A, Bb, gamma


def chunk_coefficients_nomomentum(alpha: np.ndarray):
    """Weight kernel w and chunk decay A of the no-momentum recurrence
    W_t = alpha_t W_{t-1} - eta_t g_t: w_i = prod_{s>i} alpha_s, A = prod alpha."""
    alpha = np.asarray(alpha, dtype=np.float64)
    C = alpha.shape[-1]
    w = np.ones_like(alpha)
    for i in range(C - 1):
        w[..., i] = np.prod(alpha[..., i + 1:], axis=-1)
    return w, np.prod(alpha, axis=-1)


def chunk_mean(x: np.ndarray) -> np.ndarray:
    """Mean over the chunk (last axis), broadcast back to every token."""
    x = np.asarray(x, dtype=np.float64)
    return np.broadcast_to(np.mean(x, axis=-1, keepdims=True), x.shape).copy()


# ----------------------------------------------------------------------------
# closed-form transition and the chunk loop
# ----------------------------------------------------------------------------

def closed_form_transition(g: np.ndarray, eta, alpha, beta, W: np.ndarray, M: np.ndarray):
    """Chunk transition from explicit per-token gradients g[..., C, P]."""
    m, w, A, Bb, gamma = chunk_coefficients(alpha, beta)
    GM = np.einsum("...i,...ip->...p", m * eta, g)
    GW = np.einsum("...i,...ip->...p", w * eta, g)
    W_new = A[..., None] * W - gamma[..., None] * M - GW
    M_new = Bb[..., None] * M + GM
    return W_new, M_new


def _flatten(q, k, v, eta, alpha, beta, W0, M0):
    B, H, T, D = q.shape
    f = lambda x: np.asarray(x, dtype=np.float64).reshape(B * H, *x.shape[2:])
    return (B, H, T, D), [f(x) for x in (q, k, v, eta, alpha, beta, W0, M0)]


def chunk_forward(kind, loss, q, k, v, eta, alpha, beta, W0, M0, chunk, Hd=0, keep=False,
                  momentum=True, chunk_avg=False):
    """Closed-form chunk update over a whole sequence.

    q, k, v: [B, H, T, D]; eta, alpha, beta: [B, H, T]; W0, M0: [B, H, P].
    Returns (out [B,H,T,D], W_end [B,H,P], M_end [B,H,P]) in fp64, plus a
    per-chunk list of intermediates when ``keep``.  With ``momentum=False``
    beta and M0 may be None and M_end is None.
    """
    if not momentum:
        beta = np.zeros(np.shape(eta))
        M0 = np.zeros(np.shape(W0))
    (B, H, T, D), (q, k, v, eta, alpha, beta, W, M) = _flatten(q, k, v, eta, alpha, beta, W0, M0)
    if chunk <= 0:
        raise ValueError("the chunk size must be positive")
    W = W.copy()
    M = M.copy()
    out = np.zeros_like(q)
    inter = []
    for c0 in range(0, T, chunk):
        sl = slice(c0, min(c0 + chunk, T))  # the last chunk may be shorter
        mats = unpack(kind, W, D, Hd)
        # 1. chunk output from the chunk-start weights
        out[:, sl] = fast_weight_forward(kind, mats, q[:, sl])
        # 2. per-token backward factors at the chunk-start weights
        fac = grad_factors(kind, loss, mats, k[:, sl], v[:, sl])
        # 3. scalar kernels
        if momentum:
            m, w, A, Bb, gamma = chunk_coefficients(alpha[:, sl], beta[:, sl])
        else:
            w, A = chunk_coefficients_nomomentum(alpha[:, sl])
            m = np.zeros_like(w)
            Bb = np.zeros_like(A)
            gamma = np.zeros_like(A)
        if chunk_avg:
            m, w = chunk_mean(m), chunk_mean(w)
        cM = m * eta[:, sl]
        cW = w * eta[:, sl]
        # 4. the two weighted gradient aggregations
        GM = pack(kind, weighted_grad_sum(kind, fac, k[:, sl], cM))
        GW = pack(kind, weighted_grad_sum(kind, fac, k[:, sl], cW))
        # 5. state transition (uses the chunk-start momentum)
        W_new = A[:, None] * W - gamma[:, None] * M - GW
        M_new = Bb[:, None] * M + GM
        if keep:
            inter.append(dict(m=m, w=w, A=A, Bb=Bb, gamma=gamma, cM=cM, cW=cW, GM=GM, GW=GW))
        W, M = W_new, M_new
    P = W.shape[-1]
    res = (out.reshape(B, H, T, D), W.reshape(B, H, P), M.reshape(B, H, P) if momentum else None)
    return (res + (inter,)) if keep else res


def brute_force(kind, loss, q, k, v, eta, alpha, beta, W0, M0, chunk, Hd=0, momentum=True):
    """The definition: per-token recurrence with gradients frozen at chunk start
    (``momentum=False``: W_t = alpha_t W_{t-1} - eta_t g_t, M_end None).

    For small inputs only (materialises every per-token gradient).
    """
    if not momentum:
        beta = np.zeros(np.shape(eta))
        M0 = np.zeros(np.shape(W0))
    (B, H, T, D), (q, k, v, eta, alpha, beta, W, M) = _flatten(q, k, v, eta, alpha, beta, W0, M0)
    if chunk <= 0:
        raise ValueError("the chunk size must be positive")
    W = W.copy()
    M = M.copy()
    out = np.zeros_like(q)
    for c0 in range(0, T, chunk):
        mats = unpack(kind, W, D, Hd)
        sl = slice(c0, min(c0 + chunk, T))  # the last chunk may be shorter
        out[:, sl] = fast_weight_forward(kind, mats, q[:, sl])
        g = pack(kind, token_grads(kind, loss, mats, k[:, sl], v[:, sl]))  # [BH, C, P]
        for i in range(sl.stop - c0):
            t = c0 + i
            if momentum:
                M = beta[:, t, None] * M + eta[:, t, None] * g[:, i]
                W = alpha[:, t, None] * W - M
            else:
                W = alpha[:, t, None] * W - eta[:, t, None] * g[:, i]
    P = W.shape[-1]
    return out.reshape(B, H, T, D), W.reshape(B, H, P), M.reshape(B, H, P) if momentum else None


def rel_err(x, ref) -> float:
    """max_i |x_i - ref_i| / max_i |ref_i| (0 when both are all zero)."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.max(np.abs(ref)) if ref.size else 0.0
    num = np.max(np.abs(x - ref)) if ref.size else 0.0
    if den == 0.0:
        return float(num)
    return float(num / den)

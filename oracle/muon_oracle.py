"""Plain float64 CPU oracle of the Muon optimizer step (and the Newton-Muon
right-preconditioner).

TEST INFRASTRUCTURE ONLY.  This module is the checker that the GPU path is
compared against.  Only the test suite, the smoke entry point and the CPU
baseline leg of the benchmark may import or run it; the product path never
does, and it shares no code with the HIP library (no kernels, headers,
helpers, tables or pre/post-processing).  Inputs arrive as NumPy arrays;
bfloat16 tensors arrive as their uint16 bit patterns and are decoded exactly
here.

Every step is written for readability, not speed: one matrix at a time, the
library matmul as the only primitive, no blocking, fusion or reordering.

The module also holds AdamW, which the pages assign to the parameters Muon
does not take (embeddings, heads, gains, biases).

Sources (cited by page title and section):
  [README]  "Muon: An optimizer for the hidden layers of neural networks"
            (the KellerJordan/Muon README), sections "Usage" and
            "Hyperparameter tuning".
  [BLOG]    "Muon: when LLM optimizers treat weight matrices as matrices"
            (S. Venkatramana), sections 1-4 and 7.
  [NMUON]   "The Newton-Muon Optimizer" (Newton-Muon README), section
            "What Is Newton-Muon?".

Readings taken where the pages leave a step open are marked READING and are
listed with their justification in the design notes of the repository:
  * Nesterov form (EMA form by default, SGD form on request),
  * epsilon in the Frobenius normalisation (1e-7),
  * shape-dependent learning-rate factor (three conventions),
  * decoupled decay applied to the pre-update weight,
  * float32 momentum buffer, one round-to-nearest-even to bfloat16 for W,
  * AdamW: standard bias correction, eps 1e-8 added to sqrt(v_hat).

Pinning: every function here is pinned by tests that do not re-type it (see
tests/test_oracle_pins.py): the scalar-polynomial closed form verified by
SVD, the page's worked example, the printed coefficients, the quintic's band,
polar/transpose/scale invariants, momentum closed forms, update special
cases, Cholesky/inverse identities and brute-force tiny cases.  The
shape-scale conventions and the EMA-vs-SGD choice with nonzero initial
momentum are fixed by reading only ("parity unpinned" for those choices).
"""

from __future__ import annotations

import numpy as np

# [BLOG] section 3: the quintic Newton-Schulz coefficients as printed.
NS_A = 3.4445
NS_B = -4.7750
NS_C = 2.0315
# [README] "Hyperparameter tuning": default momentum, Nesterov and NS steps.
DEFAULT_MOMENTUM = 0.95
DEFAULT_NESTEROV = True
DEFAULT_NS_STEPS = 5
# [README] "Usage": lr and weight decay of the Muon parameter group.
DEFAULT_LR = 0.02
DEFAULT_WEIGHT_DECAY = 0.01
# READING: guard for the Frobenius normalisation of an all-zero update.
DEFAULT_EPS = 1e-7

SCALE_NONE = "none"
SCALE_ORIGINAL = "original"
SCALE_MATCH_RMS_ADAMW = "match_rms_adamw"
SCALE_SPECTRAL = "spectral"


# ----------------------------------------------------------------------------
# bfloat16 decoding / rounding (exact; the oracle's own implementation)
# ----------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) exactly to float64.

    A bfloat16 value is the top half of a float32 with the same bits, so the
    decode is a shift into the high half followed by an exact widening.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    f32 = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return f32.astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value, ties to even.

    Written from the format's definition: 8 significant bits (7 stored plus
    the implicit one).  x = f * 2**e with 0.5 <= |f| < 1, so the candidate
    grid near x is multiples of 2**(e-8); np.rint rounds half to even.
    Values beyond the largest finite bfloat16 overflow to +-inf; bfloat16
    subnormals are not produced by any workload here and are rounded on the
    float32-subnormal grid (2**-133).
    """
    x = np.asarray(x, dtype=np.float64)
    f, e = np.frexp(x)
    e = np.maximum(e, -125)              # below this the spacing is fixed at 2**-133
    scale = np.ldexp(1.0, (8 - e).astype(np.int64))
    y = np.rint(x * scale) / scale
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    y = np.where(np.abs(y) > max_bf16, np.copysign(np.inf, y), y)
    return np.where(np.isfinite(x), y, x)


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (ties to even) and return the uint16 bit patterns."""
    y = round_to_bf16(x).astype(np.float32)   # exact: y is on the bf16 grid
    return (y.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


# ----------------------------------------------------------------------------
# Momentum  ([README] "Hyperparameter tuning"; [BLOG] section 1 for the EMA
# convention of a first moment)
# ----------------------------------------------------------------------------

def momentum_update(M, G, mu=DEFAULT_MOMENTUM, nesterov=DEFAULT_NESTEROV,
                    form="ema"):
    """One momentum step; returns (M_new, U) where U is what gets
    orthogonalised.

    READING (Nesterov form).  "ema": M' = mu*M + (1-mu)*G and, with Nesterov,
    U = (1-mu)*G + mu*M'.  "sgd": M' = mu*M + G and U = G + mu*M'.  Without
    Nesterov U = M'.
    """
    M = np.asarray(M, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    if form == "ema":
        M_new = mu * M + (1.0 - mu) * G
        U = (1.0 - mu) * G + mu * M_new if nesterov else M_new
    elif form == "sgd":
        M_new = mu * M + G
        U = G + mu * M_new if nesterov else M_new
    else:
        raise ValueError(f"unknown momentum form {form!r}")
    return M_new, U


# ----------------------------------------------------------------------------
# Orthogonalisation ([BLOG] section 3)
# ----------------------------------------------------------------------------

def frobenius_normalise(X, eps=DEFAULT_EPS):
    """X / (||X||_F + eps)  ([BLOG] section 3; eps is a READING)."""
    X = np.asarray(X, dtype=np.float64)
    return X / (np.sqrt(np.sum(X * X)) + eps)


def newton_schulz(X0, steps=DEFAULT_NS_STEPS, a=NS_A, b=NS_B, c=NS_C,
                  record=False):
    """Quintic Newton-Schulz iteration ([BLOG] section 3).

    Each iteration forms A = X X^T, B = b*A + c*A*A and X <- a*X + B*X, which
    is a*X + b*(X X^T)X + c*(X X^T)^2 X.  X0 must be the normalised, short-
    side-first matrix (rows <= cols).  With record=True the list of all
    iterates X_0..X_steps is returned instead of the last one.
    """
    X = np.asarray(X0, dtype=np.float64)
    iterates = [X]
    for _ in range(steps):
        A = X @ X.T
        B = b * A + c * (A @ A)
        X = a * X + B @ X
        iterates.append(X)
    return iterates if record else X


def orthogonalise(U, steps=DEFAULT_NS_STEPS, eps=DEFAULT_EPS,
                  a=NS_A, b=NS_B, c=NS_C):
    """Approximate U V^T of the update U ([BLOG] sections 2 and 3).

    Tall inputs (rows > cols) are transposed first so the iteration's Gram
    matrix is the small min(rows, cols) square, and transposed back at the
    end.
    """
    U = np.asarray(U, dtype=np.float64)
    transposed = U.shape[0] > U.shape[1]
    X = U.T if transposed else U
    X = newton_schulz(frobenius_normalise(X, eps), steps, a, b, c)
    return X.T if transposed else X


# ----------------------------------------------------------------------------
# Update ([README] "Usage"; [BLOG] sections 2 and 4)
# ----------------------------------------------------------------------------

def shape_scale(rows, cols, mode=SCALE_ORIGINAL):
    """Shape-dependent learning-rate factor.  READING: the pages name three
    conventions without printing a formula; "original" is
    sqrt(max(1, rows/cols)), "match_rms_adamw" is 0.2*sqrt(max(rows, cols)),
    "spectral" (the theoretical rule) is sqrt(rows/cols), the factor that
    gives a semi-orthogonal update an RMS->RMS operator norm of 1 under the
    blog's section-4 definition of that norm (rows = output width), and
    "none" is 1."""
    if mode == SCALE_NONE:
        return 1.0
    if mode == SCALE_ORIGINAL:
        return float(np.sqrt(max(1.0, rows / cols)))
    if mode == SCALE_MATCH_RMS_ADAMW:
        return float(0.2 * np.sqrt(max(rows, cols)))
    if mode == SCALE_SPECTRAL:
        return float(np.sqrt(rows / cols))
    raise ValueError(f"unknown scale mode {mode!r}")


def apply_update(W, O, lr, weight_decay, scale):
    """Decoupled weight decay plus the orthogonalised step:
    W' = W - lr*wd*W - lr*scale*O (READING: decay acts on the pre-update W)."""
    W = np.asarray(W, dtype=np.float64)
    O = np.asarray(O, dtype=np.float64)
    return W - lr * weight_decay * W - lr * scale * O


# ----------------------------------------------------------------------------
# Newton-Muon right-preconditioner ([NMUON] "What Is Newton-Muon?")
# ----------------------------------------------------------------------------

def second_moment(acts, damping=1e-4):
    """S = X^T X / N + damping*I from N x d layer-input activations."""
    X = np.asarray(acts, dtype=np.float64)
    n_rows, d = X.shape
    return X.T @ X / n_rows + damping * np.eye(d)


def second_moment_accumulated(batches, beta=1.0, damping=1e-4):
    """S from activations that arrive in micro-batches X_1..X_K (the online
    form of the second moment): Sigma = sum_k beta^(K-k) X_k^T X_k and
    N = sum_k beta^(K-k) n_k, S = Sigma / N + damping*I.  beta = 1 is the plain
    sum (S equals second_moment of all rows at once); beta < 1 weights older
    micro-batches down exponentially.
    READING: the pages build S from a layer's inputs and say it is refreshed
    during training without fixing how samples are pooled; this is the
    plainest pooling (a running sum, optionally decayed)."""
    Sigma, N = None, 0.0
    for X in batches:
        X = np.asarray(X, dtype=np.float64)
        XtX = X.T @ X
        Sigma = XtX if Sigma is None else beta * Sigma + XtX
        N = beta * N + X.shape[0]
    return Sigma / N + damping * np.eye(Sigma.shape[0])


def spd_inverse(S):
    """S^-1 of a symmetric positive definite S via its Cholesky factor:
    S = L L^T, so S^-1 = L^-T L^-1."""
    S = np.asarray(S, dtype=np.float64)
    L = np.linalg.cholesky(S)
    L_inv = np.linalg.solve(L, np.eye(S.shape[0]))
    return L_inv.T @ L_inv


def precondition(G, S_invs):
    """Right-precondition G by one inverse (G S^-1) or by a block-diagonal
    set of k inverses applied to G's k column blocks of width d."""
    G = np.asarray(G, dtype=np.float64)
    if isinstance(S_invs, np.ndarray) and S_invs.ndim == 2:
        S_invs = [S_invs]
    d = S_invs[0].shape[0]
    if G.shape[1] != d * len(S_invs):
        raise ValueError("columns must equal block size times block count")
    out = np.empty_like(G)
    for k, S_inv in enumerate(S_invs):
        out[:, k * d:(k + 1) * d] = G[:, k * d:(k + 1) * d] @ S_inv
    return out


# ----------------------------------------------------------------------------
# AdamW for the parameters Muon does not take ([README] "Usage": embeddings,
# classifier heads, hidden gains and biases go to AdamW, with lr 3e-4, betas
# (0.9, 0.95) and weight decay 0.01; [BLOG] section 1 gives the two moment
# recurrences).
# ----------------------------------------------------------------------------

DEFAULT_ADAM_LR = 3e-4
DEFAULT_ADAM_BETAS = (0.9, 0.95)
DEFAULT_ADAM_WEIGHT_DECAY = 0.01
DEFAULT_ADAM_EPS = 1e-8        # READING: the README's AdamW line leaves eps at its default


def adamw_update(W, G, M, V, t, lr=DEFAULT_ADAM_LR, betas=DEFAULT_ADAM_BETAS,
                 eps=DEFAULT_ADAM_EPS, weight_decay=DEFAULT_ADAM_WEIGHT_DECAY):
    """Step t (1-based) of AdamW on one parameter tensor, all in float64.

    First and second moments follow the blog's recurrences,
        M' = b1*M + (1-b1)*G,   V' = b2*V + (1-b2)*G^2,
    and the update divides the moments' bias-corrected values,
        Mh = M'/(1-b1^t),  Vh = V'/(1-b2^t),
    W' = W - lr*wd*W - lr * Mh / (sqrt(Vh) + eps).
    READING: the bias correction and eps are the standard Adam ones (the
    blog's "roughly" form omits both); the decay is decoupled and acts on
    the pre-update W, as for the Muon update.
    Returns (W', M', V')."""
    if t < 1:
        raise ValueError("Adam steps count from 1")
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    b1, b2 = betas
    M_new = b1 * M + (1.0 - b1) * G
    V_new = b2 * V + (1.0 - b2) * G * G
    m_hat = M_new / (1.0 - b1 ** t)
    v_hat = V_new / (1.0 - b2 ** t)
    W_new = W - lr * weight_decay * W - lr * m_hat / (np.sqrt(v_hat) + eps)
    return W_new, M_new, V_new


# ----------------------------------------------------------------------------
# Whole step
# ----------------------------------------------------------------------------

def muon_step(W, G, M, *, lr=DEFAULT_LR, weight_decay=DEFAULT_WEIGHT_DECAY,
              momentum=DEFAULT_MOMENTUM, nesterov=DEFAULT_NESTEROV,
              ns_steps=DEFAULT_NS_STEPS, eps=DEFAULT_EPS,
              coeffs=(NS_A, NS_B, NS_C), scale_mode=SCALE_ORIGINAL,
              momentum_form="ema", split_rows=0, lr_mult=1.0, S_invs=None):
    """One Muon step for one hidden weight matrix, all in float64.

    W, G, M are float64 arrays (decode bfloat16 inputs first).  split_rows>0
    orthogonalises consecutive row blocks of that height separately (packed
    Q/K/V, [BLOG] section 1), each with the shape scale of its block.
    S_invs, if given, right-preconditions G first ([NMUON]).
    Returns a dict with M (new momentum), O (orthogonalised update),
    W (new weight, float64) and scale (per row block).
    """
    G = np.asarray(G, dtype=np.float64)
    if S_invs is not None:
        G = precondition(G, S_invs)
    M_new, U = momentum_update(M, G, momentum, nesterov, momentum_form)
    rows, cols = U.shape
    h = split_rows if split_rows else rows
    if rows % h:
        raise ValueError("split_rows must divide rows")
    O = np.empty_like(U)
    scales = np.empty(rows)
    a, b, c = coeffs
    for r0 in range(0, rows, h):
        O[r0:r0 + h] = orthogonalise(U[r0:r0 + h], ns_steps, eps, a, b, c)
        scales[r0:r0 + h] = shape_scale(h, cols, scale_mode) * lr_mult
    W_new = apply_update(W, O, lr, weight_decay, scales[:, None])
    return {"M": M_new, "O": O, "W": W_new, "scale": scales}

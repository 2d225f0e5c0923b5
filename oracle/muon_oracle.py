"""Plain float64 CPU oracle of the Muon / Aurora-Muon optimizer step.

TEST INFRASTRUCTURE ONLY. This module is the checker that the HIP library is
compared against. Only the test suite, the package-level smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
it shares no code, constant table or helper with the GPU path.

Everything here is written for a reader to check by eye against the pages:
one matrix at a time, numpy float64, library matmuls as the only primitive,
steps in the order the pages give them, each step its own small function.

Sources (cited below by the short names in brackets):

[Aurora page]  "modded-nanogpt Track 3 优化实录：Aurora 行均衡 polar + Contra-Muon +
               u/w-floor 将 3.28 验证损失推进到 3175 步", www.xxmr.cn/news/295280.
               Sections used: "Aurora 是什么" (what Aurora is), "Aurora 的迭代伪代码"
               (the iteration pseudocode), "要点解释" (notes), "源码实现" (source
               implementation), "组合优化栈" with its Contra-Muon and u/w-floor
               parts, "完整的超参配置表" (the locked hyper-parameter table) and
               "复现与扩展建议" (reproduction and extensions).
[Track-1 page] "Modded-NanoGPT 纪录解读：U-Net 式跳跃连接与学习率翻倍如何将 124M GPT
               训练压到 7.23 分钟", www.trdm.cn/news/788905, sections
               "核心改动二：学习率翻倍" (momentum warm-up) and "训练管线与系统实现"
               (the classic five-step Muon recipe).

Readings taken where the extracted text is silent or garbled (the extraction
dropped most ASCII operators such as '=', '+', '<', '@'):

R1  Newton-Schulz runs 12 iterations of X <- a X + (b A + c A^2) X with
    A = X X^T, (a, b, c) = (2, -1.5, 0.5), after dividing the input by its
    Frobenius norm plus 1e-7. The Gram is formed on the short side (the result
    is the same in exact arithmetic).
R2  Aurora: square inputs (and pp_iterations = 0) get plain NS; otherwise the
    long side is equilibrated (rows of a tall input, columns of a wide one).
    The diagonal starts at the inverse long-side line norms clamped at eps;
    pp_iterations polar factors are taken, and between two of them the
    diagonal moves by the damped ratio (n/m / leverage)^beta, the leverage
    clamped at eps^2.
R3  Unit-operator-norm direction (body not printed): start vector = all-ones
    over the columns divided by sqrt(cols); 5 steps of w = X^T (X v),
    v = w / ||w||; sigma = ||X v||; result X / max(sigma, 1e-7). If the first
    step gives w = 0 while X != 0, restart from e_j, j = lowest index of a
    column of largest norm. X = 0 gives sigma = 0 and a zero direction.
R4  The Nesterov update X is computed exactly (no rounding to the grad's
    storage type); the oracle keeps float64 throughout.
R5  contra = 0 skips the power iteration (its term is multiplied by zero).
R6  Momentum forms. The Aurora page's step keeps an exponential moving
    average, M' = mu M + (1 - mu) G, and blends X = (1 - mu) G + mu M'
    (Nesterov) or X = M'. The Track-1 page's classic Muon runs SGD momentum
    with Nesterov; its plainest reading is the usual heavy-ball buffer with no
    dampening, M' = mu M + G, and X = G + mu M' (Nesterov) or X = M'. The two
    differ in the buffer's scale (1 / (1 - mu) at constant mu) and, under the
    momentum warm-up, in the update's direction.
R7  Wide matrices' own rows (Aurora page, "复现与扩展建议": one result applies
    the row-balanced polar to the wide MLP output projection; no formula is
    given). Plainest reading: for a wide G (rows < cols) the preconditioner
    sits on the short side, the rows of G itself, and the target squared row
    norm of a polar factor with orthonormal rows is 1; the same damped
    fixed point as R2 is run with that target. Tall and square inputs are
    unchanged. Off by default.
"""
from __future__ import annotations

from dataclasses import dataclass
import math

import numpy as np

__all__ = [
    "OracleConfig", "ns_poly", "newton_schulz", "aurora_orthogonalize",
    "power_sigma", "momentum_step", "momentum_nesterov", "muon_update",
    "ns5_classic", "classic_config", "momentum_warmup",
]


@dataclass(frozen=True)
class OracleConfig:
    """Hyper-parameters of one optimizer step.

    Defaults are the locked values of [Aurora page] §"完整的超参配置表" and the
    signature defaults of its §"源码实现" and §"组合优化栈"; NS constants from
    §"源码实现" (12 iterations, a, b, c). `momentum` is "ema" (the Aurora
    page's form) or "sgd" (the Track-1 page's, reading R6); `wide_rows`
    selects reading R7.
    """
    ns_steps: int = 12
    ns_a: float = 2.0
    ns_b: float = -1.5
    ns_c: float = 0.5
    ns_eps: float = 1e-7
    pp_iterations: int = 2
    pp_beta: float = 0.5
    pp_eps: float = 1e-7
    mu: float = 0.95
    nesterov: bool = True
    power_steps: int = 5
    contra: float = 0.4
    target_uw: float = 0.35
    lr: float = 0.0375
    momentum: str = "ema"
    wide_rows: bool = False


# ---------------------------------------------------------------------------
# Newton-Schulz polar iteration  ([Aurora page] §"源码实现", last paragraph)
# ---------------------------------------------------------------------------

def ns_poly(sigma, a=2.0, b=-1.5, c=0.5):
    """Scalar map of one NS iteration on a singular value: a s + b s^3 + c s^5.

    One step X <- a X + (b A + c A^2) X with A = X X^T sends each singular
    value s of X to this polynomial of s (the singular vectors are unchanged).
    """
    s = np.asarray(sigma, dtype=np.float64)
    return a * s + b * s ** 3 + c * s ** 5


def newton_schulz(G, steps=12, a=2.0, b=-1.5, c=0.5, eps=1e-7):
    """Approximate polar factor of G by the quintic Newton-Schulz iteration.

    [Aurora page] §"源码实现": the shared NS primitive normalises the matrix by
    its norm plus 1e-7 and then repeats X <- a X + B X, 12 times, with
    (a, b, c) = (2, -1.5, 0.5). Reading R1 (Frobenius norm, B = b A + c A^2,
    Gram on the short side).
    """
    X = np.array(G, dtype=np.float64, copy=True)
    if X.ndim != 2:
        raise ValueError("newton_schulz expects a 2-D matrix")
    X = X / (np.linalg.norm(X) + eps)          # Frobenius norm + eps
    flip = X.shape[0] > X.shape[1]
    if flip:                                   # work on the wide orientation
        X = X.T
    for _ in range(steps):
        A = X @ X.T                            # short-side Gram
        B = b * A + c * (A @ A)
        X = a * X + B @ X
    return X.T if flip else X


# ---------------------------------------------------------------------------
# Aurora: leverage-equilibrated polar  ([Aurora page] §"Aurora 是什么",
# §"Aurora 的迭代伪代码", §"要点解释", §"源码实现", §"复现与扩展建议")
# ---------------------------------------------------------------------------

def _line_norms(T):
    """Euclidean norm of every row of T."""
    return np.sqrt(np.sum(T * T, axis=1))


def _scaled_polar(d, T, ns):
    """Polar factor of diag(d) T (each row of T scaled by its entry of d)."""
    return ns(d[:, None] * T)


def _equilibrate(d, U, target, beta, eps):
    """One damped fixed-point move of the diagonal: rows of U whose squared
    norm (leverage) is above the target get a smaller weight, rows below it a
    larger one, by the ratio target / leverage raised to beta."""
    leverage = np.maximum(np.sum(U * U, axis=1), eps * eps)
    return d * (target / leverage) ** beta


def aurora_orthogonalize(G, pp_iterations=2, pp_beta=0.5, eps=1e-7,
                         ns_steps=12, a=2.0, b=-1.5, c=0.5, ns_eps=1e-7,
                         wide_rows=False):
    """polar(D G) for tall G, polar(G D) for wide G, D evening out the
    long-side line norms of the result ([Aurora page], reading R2).

    A polar factor of a tall m x n matrix with orthonormal columns has total
    squared norm n, so the uniform leverage is n / m per row; the square case
    has no freedom left (its polar factor is orthogonal) and is plain NS. In
    the tall orientation T: d = 1 / max(||T_i||, eps), U = polar(diag(d) T),
    and pp_iterations - 1 times {d <- d (n/m / leverage(U))^beta; U = polar
    (diag(d) T)}. With wide_rows (reading R7) a wide G is equilibrated on its
    own rows with target 1 instead.
    """
    G = np.asarray(G, dtype=np.float64)
    rows, cols = G.shape

    def ns(Y):
        return newton_schulz(Y, ns_steps, a, b, c, ns_eps)

    if rows == cols or pp_iterations == 0:
        return ns(G)
    if wide_rows and rows < cols:
        T, target, flipped = G, 1.0, False        # short side: G's own rows
    elif rows < cols:
        T, target, flipped = G.T, rows / cols, True
    else:
        T, target, flipped = G, cols / rows, False
    d = 1.0 / np.maximum(_line_norms(T), eps)
    U = _scaled_polar(d, T, ns)
    for _ in range(pp_iterations - 1):
        d = _equilibrate(d, U, target, pp_beta, eps)
        U = _scaled_polar(d, T, ns)
    return U.T if flipped else U


# ---------------------------------------------------------------------------
# Unit-operator-norm direction  ([Aurora page] §"组合优化栈", Contra-Muon part)
# ---------------------------------------------------------------------------

def power_sigma(X, steps=5):
    """Operator-norm estimate of X by `steps` power iterations on X^T X.

    The page states only that 5 power iterations estimate the operator norm;
    the start vector, the estimate and the degenerate case follow reading R3.
    """
    X = np.asarray(X, dtype=np.float64)
    r, c = X.shape
    if not np.any(X):
        return 0.0
    v = np.ones(c) / math.sqrt(c)
    w = X.T @ (X @ v)
    if np.linalg.norm(w) == 0.0:
        j = int(np.argmax(np.linalg.norm(X, axis=0)))   # first max-norm column
        v = np.zeros(c)
        v[j] = 1.0
        w = X.T @ (X @ v)
    v = w / np.linalg.norm(w)
    for _ in range(steps - 1):
        w = X.T @ (X @ v)
        v = w / np.linalg.norm(w)
    return float(np.linalg.norm(X @ v))


def unit_operator_direction(X, steps=5):
    """X divided by its estimated operator norm (clamped at 1e-7)."""
    return X / max(power_sigma(X, steps), 1e-7)


# ---------------------------------------------------------------------------
# One Muon step  ([Aurora page] §"组合优化栈": the step function, Contra-Muon,
# u/w-floor, and the lr / weight-decay rows of §"完整的超参配置表";
# [Track-1 page] §"训练管线与系统实现" for the SGD-momentum form)
# ---------------------------------------------------------------------------

def momentum_step(G, M, mu=0.95, nesterov=True, form="ema"):
    """Momentum state update and the update X fed to the orthogonalisation.

    Returns (M', X), reading R6:
      form "ema" (Aurora page): M' is the exponential moving average of the
        gradients, M' = mu M + (1 - mu) G; Nesterov looks one average ahead,
        X = (1 - mu) G + mu M'.
      form "sgd" (Track-1 page): heavy-ball buffer M' = mu M + G; Nesterov
        X = G + mu M'.
    Without Nesterov X = M' in both forms.
    """
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    if form == "ema":
        M_new = mu * M + (1.0 - mu) * G
        X = (1.0 - mu) * G + mu * M_new if nesterov else M_new
    elif form == "sgd":
        M_new = mu * M + G
        X = G + mu * M_new if nesterov else M_new
    else:
        raise ValueError(f"unknown momentum form {form!r}")
    return M_new, X


def momentum_nesterov(G, M, mu=0.95, nesterov=True):
    """The Aurora page's form of `momentum_step` (form "ema")."""
    return momentum_step(G, M, mu, nesterov, "ema")


def contra_mix(U, N, contra):
    """Contra-Muon: subtract contra/2 times the unit-operator-norm direction N
    from the polar factor U, then give the result U's Frobenius norm back
    (clamp 1e-10 on the divisor)."""
    norm_U = np.linalg.norm(U)
    V = U - (contra / 2.0) * N if contra != 0.0 else U
    return V * (norm_U / max(np.linalg.norm(V), 1e-10))


def aspect_scale(V, rows, cols):
    """Scale by sqrt(max(1, rows / cols)) of the stored shape."""
    return V * math.sqrt(max(1.0, rows / cols))


def uw_floor(V, W, target):
    """Raise ||V|| to target ||W|| when it is below that (both norms clamped
    at 1e-8; strict comparison)."""
    norm_W = max(np.linalg.norm(W), 1e-8)
    norm_V = max(np.linalg.norm(V), 1e-8)
    if norm_V / norm_W < target:
        return V * (target * norm_W / norm_V)
    return V


def muon_update(G, M, W=None, cfg: OracleConfig = OracleConfig()):
    """One Aurora + Contra-Muon + u/w-floor step on one matrix.

    Returns (M_new, V, W_new): the updated momentum, the update after the
    floor (before lr), and W - lr V (None when W is None). The steps, in the
    page's order: momentum and Nesterov blend (`momentum_step`); the unit-
    operator-norm direction of X (only when contra != 0, reading R5); the
    Aurora polar factor U of X; `contra_mix`; `aspect_scale`; `uw_floor`
    (when W is given and target_uw > 0); W - lr V (no weight decay).
    """
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    if G.shape != M.shape or G.ndim != 2:
        raise ValueError("G and M must be matrices of one shape")
    rows, cols = G.shape

    M_new, X = momentum_step(G, M, cfg.mu, cfg.nesterov, cfg.momentum)
    U = aurora_orthogonalize(X, cfg.pp_iterations, cfg.pp_beta, cfg.pp_eps,
                             cfg.ns_steps, cfg.ns_a, cfg.ns_b, cfg.ns_c,
                             cfg.ns_eps, cfg.wide_rows)
    N = unit_operator_direction(X, cfg.power_steps) if cfg.contra != 0.0 else None
    V = contra_mix(U, N, cfg.contra)
    V = aspect_scale(V, rows, cols)

    W_new = None
    if W is not None:
        W = np.asarray(W, dtype=np.float64)
        if W.shape != G.shape:
            raise ValueError("W must have the shape of G")
        if cfg.target_uw > 0.0:
            V = uw_floor(V, W, cfg.target_uw)
        W_new = W - cfg.lr * V
    return M_new, V, W_new


# ---------------------------------------------------------------------------
# Classic five-step recipe  ([Track-1 page] §"训练管线与系统实现")
# ---------------------------------------------------------------------------

def ns5_classic(G, steps=5, a=3.4445, b=-4.7750, c=2.0315, eps=1e-7):
    """The earlier tuned 5-iteration NS used by the Track-1 record.

    Same iteration form as `newton_schulz` with the constants printed on the
    Track-1 page; its fixed point is deliberately not 1 (p(1) != 1).
    """
    return newton_schulz(G, steps, a, b, c, eps)


def classic_config() -> OracleConfig:
    """The classic recipe as one OracleConfig ([Track-1 page]).

    Muon on every 2-D matrix with lr 0.04, SGD momentum 0.95 with Nesterov
    (reading R6; the coefficient is warmed up, see `momentum_warmup`), five NS
    iterations with the page's (a, b, c), the sqrt(max(1, rows / cols))
    scale; none of Aurora's preconditioner, the Contra term or the u/w-floor
    (pp_iterations 0, contra 0, target_uw 0).
    """
    return OracleConfig(ns_steps=5, ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315,
                        pp_iterations=0, mu=0.95, nesterov=True, contra=0.0,
                        target_uw=0.0, lr=0.04, momentum="sgd")


def momentum_warmup(step, mu_start=0.85, mu_end=0.95, warmup_steps=500):
    """Momentum at a given step ([Track-1 page] §"核心改动二：学习率翻倍"): over
    the first 500 steps the coefficient moves linearly from 0.85 to 0.95
    (frac = min(step / 500, 1), mu = (1 - frac) 0.85 + frac 0.95), then stays
    at 0.95."""
    if warmup_steps <= 0:
        return float(mu_end)
    frac = min(max(step, 0) / warmup_steps, 1.0)
    return (1.0 - frac) * mu_start + frac * mu_end

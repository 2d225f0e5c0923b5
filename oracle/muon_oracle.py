"""Plain float64 CPU oracle of the Muon / Aurora-Muon optimizer step.

TEST INFRASTRUCTURE ONLY. This module is the checker that the HIP library is
compared against. Only the test suite, the package-level smoke check and the
benchmark's CPU-baseline leg may import it; the library itself never does, and
it shares no code, constant table or helper with the GPU path.

Everything here is written for a reader to check by eye against the pages:
one matrix at a time, numpy float64, library matmuls as the only primitive,
steps in the order the pages give them.

Sources (cited below by the short names in brackets):

[Aurora page]  "modded-nanogpt Track 3 优化实录：Aurora 行均衡 polar + Contra-Muon +
               u/w-floor 将 3.28 验证损失推进到 3175 步", www.xxmr.cn/news/295280.
               Sections used: "Aurora 是什么" (what Aurora is), "Aurora 的迭代伪代码"
               (the iteration pseudocode), "要点解释" (notes), "源码实现" (source
               implementation), "组合优化栈" with its Contra-Muon and u/w-floor
               parts, and "完整的超参配置表" (the locked hyper-parameter table).
[Track-1 page] "Modded-NanoGPT 纪录解读：U-Net 式跳跃连接与学习率翻倍如何将 124M GPT
               训练压到 7.23 分钟", www.trdm.cn/news/788905, section
               "训练管线与系统实现" (the classic five-step Muon recipe).

Readings taken where the extracted text is silent or garbled (the extraction
dropped most ASCII operators such as '=', '+', '<', '@'):

R1  Newton-Schulz runs 12 iterations of X <- a X + (b A + c A^2) X with
    A = X X^T, (a, b, c) = (2, -1.5, 0.5), after dividing the input by its
    Frobenius norm plus 1e-7. The Gram is formed on the short side (the result
    is the same in exact arithmetic).
R2  In aurora_orthogonalize the stripped comparisons are: square -> plain NS;
    transpose when rows < cols; D is updated only in non-final passes; the
    row-norm clamp is eps and the row_sq clamp is eps^2.
R3  scale_to_unit_operator_norm (body not printed): start vector = all-ones
    over the columns divided by sqrt(cols); 5 steps of w = X^T (X v),
    v = w / ||w||; sigma = ||X v||; result X / max(sigma, 1e-7). If the first
    step gives w = 0 while X != 0, restart from e_j, j = lowest index of a
    column of largest norm. X = 0 gives sigma = 0 and a zero direction.
R4  The Nesterov update X is computed exactly (no rounding to the grad's
    storage type); the oracle keeps float64 throughout.
R5  pp_iterations = 0 means plain NS without the diagonal preconditioner;
    contra = 0 skips the power iteration (its term is multiplied by zero).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

__all__ = [
    "OracleConfig", "ns_poly", "newton_schulz", "aurora_orthogonalize",
    "power_sigma", "momentum_nesterov", "muon_update", "ns5_classic",
    "classic_config", "momentum_warmup",
]


@dataclass(frozen=True)
class OracleConfig:
    """Hyper-parameters of one optimizer step.

    Defaults are the locked values of [Aurora page] §"完整的超参配置表" and the
    signature defaults of muon_update / aurora_orthogonalize in §"源码实现" and
    §"组合优化栈"; NS constants from §"源码实现" (12 iterations, a, b, c).
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
    (a, b, c) = (2, -1.5, 0.5). Readings R1 (Frobenius norm, B = b A + c A^2,
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
# §"Aurora 的迭代伪代码", §"要点解释", §"源码实现")
# ---------------------------------------------------------------------------

def aurora_orthogonalize(G, pp_iterations=2, pp_beta=0.5, eps=1e-7,
                         ns_steps=12, a=2.0, b=-1.5, c=0.5, ns_eps=1e-7):
    """polar(D G) for tall G, polar(G D) for wide G, D chosen to even out row norms.

    Follows §"源码实现" (aurora_orthogonalize) with reading R2:
      * square -> plain NS (no leverage freedom, §"Aurora 是什么");
      * wide inputs are transposed, handled as tall (m > n), and transposed back;
      * D starts as the inverse of each (clamped) row norm;
      * each pass computes U = NS(D * G); in every pass but the last, D is
        multiplied by (target / row_sq) ** beta with target = n / m and
        row_sq the clamped squared row norms of U.
    pp_iterations = 0 is plain NS (reading R5).
    """
    G = np.asarray(G, dtype=np.float64)
    ns = lambda Y: newton_schulz(Y, ns_steps, a, b, c, ns_eps)
    m, n = G.shape
    if m == n or pp_iterations == 0:
        return ns(G)
    transposed = m < n
    T = G.T if transposed else G
    m, n = T.shape                               # now m > n (tall)
    target_row_sq = n / m
    row_norm = np.maximum(np.linalg.norm(T, axis=1), eps)
    D = 1.0 / row_norm
    U = None
    for k in range(pp_iterations):
        U = ns(D[:, None] * T)                   # row scaling D * G
        if k < pp_iterations - 1:
            row_sq = np.maximum(np.sum(U * U, axis=1), eps * eps)
            D = D * (target_row_sq / row_sq) ** pp_beta
    return U.T if transposed else U


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


# ---------------------------------------------------------------------------
# One Muon step  ([Aurora page] §"组合优化栈": muon_update, Contra-Muon,
# u/w-floor, and the lr / weight-decay rows of §"完整的超参配置表")
# ---------------------------------------------------------------------------

def momentum_nesterov(G, M, mu=0.95, nesterov=True):
    """Elementwise first two steps of muon_update: returns (M', X).

    momentum.lerp_(grad, 1 - mu) gives M' = M + (1 - mu)(G - M); the Nesterov
    blend grad.lerp_(momentum, mu) gives X = G + mu (M' - G); without Nesterov
    X = M' ([Aurora page] §"组合优化栈", muon_update).
    """
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    M_new = M + (1.0 - mu) * (G - M)
    X = G + mu * (M_new - G) if nesterov else M_new
    return M_new, X


def muon_update(G, M, W=None, cfg: OracleConfig = OracleConfig()):
    """One Aurora + Contra-Muon + u/w-floor step on one matrix.

    Returns (M_new, V, W_new): the updated momentum, the update after the
    floor (before lr), and W - lr * V (None when W is None).

    Steps, in the page's order:
      1. momentum.lerp_(grad, 1 - mu): M' = M + (1 - mu) (G - M).
      2. Nesterov: X = G + mu (M' - G)  (plain momentum X = M' otherwise).
      3. N = X / sigma with sigma from `power_sigma` (reading R3).
      4. U = aurora_orthogonalize(X); f = ||U||_F.
      5. V = U - (contra / 2) N, rescaled to Frobenius norm f (clamp 1e-10).
      6. V *= sqrt(max(1, rows / cols)).
      7. u/w-floor: p = max(||W||, 1e-8), u = max(||V||, 1e-8); when
         u / p < target_uw, V *= target_uw * p / u.
      8. W' = W - lr V (weight decay is 0).
    """
    G = np.asarray(G, dtype=np.float64)
    M = np.asarray(M, dtype=np.float64)
    if G.shape != M.shape or G.ndim != 2:
        raise ValueError("G and M must be matrices of one shape")
    rows, cols = G.shape

    M_new, X = momentum_nesterov(G, M, cfg.mu, cfg.nesterov)

    U = aurora_orthogonalize(X, cfg.pp_iterations, cfg.pp_beta, cfg.pp_eps,
                             cfg.ns_steps, cfg.ns_a, cfg.ns_b, cfg.ns_c,
                             cfg.ns_eps)
    polar_fro = np.linalg.norm(U)
    if cfg.contra != 0.0:
        sigma = power_sigma(X, cfg.power_steps)
        N = X / max(sigma, 1e-7)
        V = U - (cfg.contra / 2.0) * N
    else:
        V = U
    V = V * (polar_fro / max(np.linalg.norm(V), 1e-10))
    V = V * math.sqrt(max(1.0, rows / cols))

    W_new = None
    if W is not None:
        W = np.asarray(W, dtype=np.float64)
        if W.shape != G.shape:
            raise ValueError("W must have the shape of G")
        if cfg.target_uw > 0.0:
            p_fro = max(np.linalg.norm(W), 1e-8)
            u_fro = max(np.linalg.norm(V), 1e-8)
            if u_fro / p_fro < cfg.target_uw:
                V = V * (cfg.target_uw * p_fro / u_fro)
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

    Muon on every 2-D matrix with lr 0.04, Nesterov momentum 0.95 (warmed up,
    see `momentum_warmup`), five NS iterations with the page's (a, b, c), the
    sqrt(max(1, rows / cols)) scale; none of Aurora's preconditioner, the
    Contra term or the u/w-floor (pp_iterations 0, contra 0, target_uw 0;
    reading R5).
    """
    return OracleConfig(ns_steps=5, ns_a=3.4445, ns_b=-4.7750, ns_c=2.0315,
                        pp_iterations=0, mu=0.95, nesterov=True, contra=0.0,
                        target_uw=0.0, lr=0.04)


def momentum_warmup(step, mu_start=0.85, mu_end=0.95, warmup_steps=500):
    """Momentum at a given step ([Track-1 page]): over the first 500 steps the
    coefficient moves linearly from 0.85 to 0.95 (frac = min(step / 500, 1),
    mu = (1 - frac) 0.85 + frac 0.95), then stays at 0.95."""
    if warmup_steps <= 0:
        return float(mu_end)
    frac = min(max(step, 0) / warmup_steps, 1.0)
    return (1.0 - frac) * mu_start + frac * mu_end

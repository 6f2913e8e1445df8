"""fp64 CPU oracle of the ButterflyMoE expert-layer forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import or call this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library; both sides only read the arrays made by
``compressed_mixture_experts_amd.workloads``.

Sources (web summaries of the papers; cited by page and section):
  [MoE-zh]  "ButterflyMoE: Sub-Linear Ternary Experts via Structured Butterfly
            Orbits", gist.science/zh/paper/2601.13563, technical summary:
            §2.1 (formal definition of an expert), §2.2 (ternary substrate,
            butterfly = hierarchical Givens rotations + permutations),
            §4.4 (inference cost).
  [MoE-pt]  same paper, gist.science/pt/paper/2601.13563, technical summary
            §2 "Metodologia" (expert formula, O(d log d) angles, memory
            O(d^2 + N d log d)) and §4 "Resultados" (4.70 MB at 256 experts).
  [MoE-nl]  same paper, gist.science/nl/paper/2601.13563, §2 "Methodologie",
            "Drie Fasen van de Methode" (standard top-k gating network;
            experts never materialised during inference).
  [ViT-pt]  "ButterflyViT", gist.science/pt/paper/2603.06746, §2 "Metodologia"
            (block-diagonal Givens parameterisation, rotations before and after
            the shared substrate in the FFN) and §3 (per-expert cost n_l * d).

What the pages leave open is read as follows (each choice is a convention that
every statement on the pages still satisfies):
  * stage s of a butterfly of size n = 2^L rotates the index pair (i, i + 2^s)
    (bit s of i clear) by the angle with pair number p = i with bit s deleted;
    the rotation acts as [[c, -s], [s, c]] on (v_i, v_j);
    B = S_{L-1} ... S_1 S_0, so B v applies the stride-1 stage first;
  * angles are stored [log2 n][n/2] per butterfly, fp32, and are used exactly
    (their cos/sin are taken in fp64);
  * B(theta) has the input width, B(phi) the output width; an FFN expert has an
    up substrate (d_ff x d) and a down substrate (d x d_ff), each with its own
    pair of rotations, and an exact-erf GELU between them;
  * the router is a bias-free linear map x -> logits, top-k on the logits
    (larger first, ties to the lower expert index), gate = softmax probability
    of the chosen expert over all N logits (optionally renormalised over the k);
  * the combine is y_t = sum_j gate_{t,j} * E_{e_j}(x_t), no capacity limit;
  * an optional scalar alpha multiplies each substrate (default 1).
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import numpy as np
from scipy.special import erf as _erf

__all__ = [
    "stored_to_f64", "pair_index", "stage_matrix", "butterfly_dense",
    "butterfly_apply", "butterfly_backward", "expert_matrix", "expert_apply", "gelu",
    "route", "forward", "forward_tokens", "param_counts", "ternary_product",
]


# ---------------------------------------------------------------------------
# stored values -> float64
# ---------------------------------------------------------------------------
def stored_to_f64(a: np.ndarray, act: str) -> np.ndarray:
    """Exact float64 value of stored activations (float32, or bf16 bit patterns)."""
    if act == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if act == "bf16":
        bits = np.asarray(a, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    raise ValueError(act)


# ---------------------------------------------------------------------------
# butterfly matrices  ([MoE-zh] §2.2, [ViT-pt] §2)
# ---------------------------------------------------------------------------
def pair_index(i: int, s: int) -> int:
    """Pair number of index i (bit s clear) in stage s: i with bit s deleted."""
    low = i & ((1 << s) - 1)
    return ((i >> (s + 1)) << s) | low


def stage_matrix(angles_s: np.ndarray, s: int, n: int) -> np.ndarray:
    """Dense n x n matrix of butterfly stage s (small n only)."""
    S = np.zeros((n, n))
    ang = np.asarray(angles_s, dtype=np.float64)
    for i in range(n):
        if i & (1 << s):
            continue
        j = i + (1 << s)
        t = ang[pair_index(i, s)]
        c, sn = math.cos(t), math.sin(t)
        S[i, i] = c
        S[i, j] = -sn
        S[j, i] = sn
        S[j, j] = c
    return S


def butterfly_dense(angles: np.ndarray) -> np.ndarray:
    """B = S_{L-1} ... S_0 as an explicit dense product (small n only)."""
    angles = np.asarray(angles)
    L = angles.shape[0]
    n = 1 << L
    B = np.eye(n)
    for s in range(L):
        B = stage_matrix(angles[s], s, n) @ B
    return B


def butterfly_apply(angles: np.ndarray, M: np.ndarray, transpose: bool = False) -> np.ndarray:
    """B(angles) @ M, or B(angles)^T @ M, one Givens stage at a time.

    M has shape (n, m) (or (n,)).  B @ M applies S_0 first; B^T @ M applies
    S_{L-1}^T first.  Each stage rotates the rows i and i + 2^s of M.
    """
    ang = np.asarray(angles, dtype=np.float64)
    L = ang.shape[0]
    n = 1 << L
    V = np.array(M, dtype=np.float64, copy=True)
    vec = V.ndim == 1
    if vec:
        V = V[:, None]
    if V.shape[0] != n:
        raise ValueError(f"butterfly of size {n} applied to {V.shape[0]} rows")
    order = range(L - 1, -1, -1) if transpose else range(L)
    for s in order:
        h = 1 << s
        c = np.cos(ang[s]).reshape(n // (2 * h), h, 1)
        sn = np.sin(ang[s]).reshape(n // (2 * h), h, 1)
        W = V.reshape(n // (2 * h), 2, h, V.shape[1])
        a = W[:, 0].copy()
        b = W[:, 1].copy()
        if not transpose:
            W[:, 0] = c * a - sn * b
            W[:, 1] = sn * a + c * b
        else:
            W[:, 0] = c * a + sn * b
            W[:, 1] = -sn * a + c * b
        V = W.reshape(n, -1)
    return V[:, 0] if vec else V


def butterfly_backward(angles: np.ndarray, X: np.ndarray, dY: np.ndarray, transpose: bool = False):
    """Gradients of the rotated columns Y = B(angles) X (or B^T X) for a given dY.

    The rotations are learnable parameters of every expert ([MoE-zh] §2.2: the
    butterfly angles are the experts' parameters; training them is the
    adjacent step of the method).  Plain chain rule, one Givens stage at a
    time: the forward pass keeps every stage's input; walking the stages back,
    the angle of pair (i, j) of stage s collects, summed over the columns,
        dY_i * d(out_i)/dt + dY_j * d(out_j)/dt
    with out = [[c, -s], [s, c]] (a, b) (or its transpose for B^T), and the
    gradient passes to the stage input through the transposed stage.

    X, dY [n][m] float64-convertible.  Returns (dX [n][m], dAngles [L][n/2]).
    """
    ang = np.asarray(angles, dtype=np.float64)
    L = ang.shape[0]
    n = 1 << L
    V = np.array(X, dtype=np.float64, copy=True)
    G = np.array(dY, dtype=np.float64, copy=True)
    if V.shape != G.shape or V.shape[0] != n:
        raise ValueError("X and dY must both be [n][m]")
    order = list(range(L - 1, -1, -1)) if transpose else list(range(L))
    kept = []
    for s in order:
        kept.append((s, V.copy()))
        V = _apply_stage(ang[s], s, V, transpose)
    dang = np.zeros((L, n // 2))
    for s, Vin in reversed(kept):
        # pairs of stage s: lower index i (bit s clear), upper j = i + 2^s; in
        # the [n / 2^(s+1)][2][2^s] view pair p = (block, offset) is row-major
        h = 1 << s
        c = np.cos(ang[s]).reshape(n // (2 * h), h, 1)
        sn = np.sin(ang[s]).reshape(n // (2 * h), h, 1)
        Vw = Vin.reshape(n // (2 * h), 2, h, -1)
        Gw = G.reshape(n // (2 * h), 2, h, -1)
        a, b = Vw[:, 0], Vw[:, 1]
        if not transpose:      # out_i = c a - s b, out_j = s a + c b
            da, db = -sn * a - c * b, c * a - sn * b
        else:                  # out_i = c a + s b, out_j = -s a + c b
            da, db = -sn * a + c * b, -c * a - sn * b
        dang[s] = np.sum(Gw[:, 0] * da + Gw[:, 1] * db, axis=2).reshape(n // 2)
        # gradient to the stage input: through the transposed stage
        G = _apply_stage(ang[s], s, G, not transpose)
    return G, dang


def _apply_stage(ang_s: np.ndarray, s: int, V: np.ndarray, transpose: bool) -> np.ndarray:
    """Stage s alone (or its transpose) applied to the rows of V [n][m]: rows
    i and i + 2^s rotate by the angle of their pair, as in butterfly_apply."""
    n = V.shape[0]
    h = 1 << s
    c = np.cos(np.asarray(ang_s, dtype=np.float64)).reshape(n // (2 * h), h, 1)
    sn = np.sin(np.asarray(ang_s, dtype=np.float64)).reshape(n // (2 * h), h, 1)
    W = np.array(V, dtype=np.float64).reshape(n // (2 * h), 2, h, V.shape[1])
    a, b = W[:, 0].copy(), W[:, 1].copy()
    if not transpose:
        W[:, 0] = c * a - sn * b
        W[:, 1] = sn * a + c * b
    else:
        W[:, 0] = c * a + sn * b
        W[:, 1] = -sn * a + c * b
    return W.reshape(n, -1)


# ---------------------------------------------------------------------------
# experts  ([MoE-zh] §2.1: W_i = B(phi_i) W_base B(theta_i)^T)
# ---------------------------------------------------------------------------
def expert_matrix(theta: np.ndarray, phi: np.ndarray, w_base: np.ndarray,
                  alpha: float = 1.0) -> np.ndarray:
    """Materialise W_e = B(phi) (alpha W_base) B(theta)^T as a float64 array."""
    W = alpha * np.asarray(w_base, dtype=np.float64)
    P = butterfly_apply(phi, W)                     # B(phi) @ W
    return butterfly_apply(theta, P.T).T            # (B(theta) @ P^T)^T = P B(theta)^T


def expert_apply(theta: np.ndarray, phi: np.ndarray, w_base: np.ndarray, X: np.ndarray,
                 alpha: float = 1.0) -> np.ndarray:
    """W_e @ X evaluated right to left: B(phi) (alpha W_base (B(theta)^T X)).

    Same value as ``expert_matrix(...) @ X`` by associativity; used where
    materialising every expert is too slow (sampled tokens of large layers).
    X has shape (d_in, m).
    """
    U = butterfly_apply(theta, X, transpose=True)
    Z = alpha * (np.asarray(w_base, dtype=np.float64) @ U)
    return butterfly_apply(phi, Z)


def gelu(h: np.ndarray) -> np.ndarray:
    """Exact GELU, h * Phi(h) = h * (1 + erf(h / sqrt 2)) / 2."""
    return h * 0.5 * (1.0 + _erf(h / math.sqrt(2.0)))


# ---------------------------------------------------------------------------
# routing  ([MoE-nl] §2 "Gated Routing": standard top-k gating network)
# ---------------------------------------------------------------------------
class Routing:
    def __init__(self, logits, idx, gates, probs, ambiguous, gap_eps):
        self.logits = logits          # [T][N] float64
        self.idx = idx                # [T][k] int64
        self.gates = gates            # [T][k] float64
        self.probs = probs            # [T][N] float64
        self.ambiguous = ambiguous    # [T] bool: a decisive gap is within fp64 noise
        self.gap_eps = gap_eps        # [T] float64


def route(x64: np.ndarray, wg64: np.ndarray, k: int, renorm: bool = False) -> Routing:
    """Top-k softmax gating on logits l = W_g x (no bias, no noise).

    Experts are ordered by logit, larger first, equal logits by lower index.
    gate = softmax(l)[e] for each chosen e (divided by the sum of the k chosen
    gates when ``renorm``).  A token is flagged ambiguous when one of the k
    decisive gaps (between consecutive chosen experts, and between the k-th and
    the (k+1)-th) is below 4 d 2^-53 |x| max|w| (fp64 rounding level).
    """
    T, d = x64.shape
    N = wg64.shape[0]
    logits = x64 @ wg64.T
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :k]
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    probs = ex / ex.sum(axis=1, keepdims=True)
    gates = np.take_along_axis(probs, idx, axis=1)
    if renorm:
        gates = gates / gates.sum(axis=1, keepdims=True)
    srt = np.take_along_axis(logits, order, axis=1)
    n_gaps = min(k, N - 1)
    eps = 4.0 * d * 2.0 ** -53 * np.linalg.norm(x64, axis=1) * np.linalg.norm(wg64, axis=1).max()
    if n_gaps > 0:
        gaps = srt[:, :n_gaps] - srt[:, 1:n_gaps + 1]
        ambiguous = (gaps < eps[:, None]).any(axis=1)
    else:
        ambiguous = np.zeros(T, dtype=bool)
    return Routing(logits, idx, gates, probs, ambiguous, eps)


# ---------------------------------------------------------------------------
# layer forward
# ---------------------------------------------------------------------------
def _inputs_f64(inp):
    cfg = inp.cfg
    x = stored_to_f64(inp.x, cfg.act)
    wg = stored_to_f64(inp.w_gate, cfg.act)
    return cfg, x, wg


def forward(inp, routing: Optional[Routing] = None, idx_override: Optional[np.ndarray] = None):
    """Full layer forward by materialising every used expert (the definition).

    y_t = sum_j g_{t,j} W_{e_j} x_t for square experts, and
    y_t = sum_j g_{t,j} W_dn,e GELU(W_up,e x_t) for FFN experts (GELU replaced
    by the identity when the layer's FFN activation is "none"), where each
    W_e = B(phi_e) W_base B(theta_e)^T ([MoE-zh] §2.1, [ViT-pt] §2).
    ``idx_override`` evaluates the layer at given expert choices (gates are then
    the softmax probabilities of those experts).
    Returns (y float64 [T][d], routing).
    """
    cfg, x, wg = _inputs_f64(inp)
    if routing is None:
        routing = route(x, wg, cfg.top_k, cfg.renorm_gates)
    idx, gates = routing.idx, routing.gates
    if idx_override is not None:
        idx = np.asarray(idx_override)
        gates = np.take_along_axis(routing.probs, idx, axis=1)
        if cfg.renorm_gates:
            gates = gates / gates.sum(axis=1, keepdims=True)
    T = x.shape[0]
    y = np.zeros((T, cfg.d_model))
    for e in np.unique(idx):
        tok, slot = np.nonzero(idx == e)
        Xe = x[tok]                                     # rows = tokens
        if cfg.is_ffn:
            Wup = expert_matrix(inp.theta[0][e], inp.phi[0][e], inp.w_base[0], cfg.w_scale)
            Wdn = expert_matrix(inp.theta[1][e], inp.phi[1][e], inp.w_base[1], cfg.w_scale)
            H = Xe @ Wup.T
            Ye = (gelu(H) if cfg.ffn_act == "gelu" else H) @ Wdn.T
        else:
            We = expert_matrix(inp.theta[0][e], inp.phi[0][e], inp.w_base[0], cfg.w_scale)
            Ye = Xe @ We.T
        np.add.at(y, tok, gates[tok, slot][:, None] * Ye)
    return y, routing


def forward_tokens(inp, tokens: Sequence[int], routing: Optional[Routing] = None,
                   idx_override: Optional[np.ndarray] = None):
    """Layer output for a subset of tokens without materialising experts: the
    same products as ``forward`` evaluated right to left, B(phi) (W (B(theta)^T x))
    ([MoE-zh] §2.1: the expert is applied as input rotation, substrate product and
    output rotation; the nl page, §2 "Drie Fasen", has it never formed during
    inference).  The chosen tokens of one expert are stacked as the columns of
    one matrix, which changes nothing but the rounding order of the fp64 sums.

    Used for the checks of layers too large to materialise.  Routing is
    computed for the requested tokens only unless ``routing`` is given.
    Returns (y float64 [len(tokens)][d], idx [len][k], gates [len][k]).
    """
    cfg = inp.cfg
    tokens = np.asarray(tokens, dtype=np.int64)
    x = stored_to_f64(inp.x[tokens], cfg.act)
    if routing is None:
        wg = stored_to_f64(inp.w_gate, cfg.act)
        r = route(x, wg, cfg.top_k, cfg.renorm_gates)
        idx, gates, probs = r.idx, r.gates, r.probs
    else:
        idx, gates, probs = routing.idx[tokens], routing.gates[tokens], routing.probs[tokens]
    if idx_override is not None:
        idx = np.asarray(idx_override)
        gates = np.take_along_axis(probs, idx, axis=1)
        if cfg.renorm_gates:
            gates = gates / gates.sum(axis=1, keepdims=True)
    w64 = [np.asarray(w, dtype=np.float64) for w in inp.w_base]
    y = np.zeros((len(tokens), cfg.d_model))
    for e in np.unique(idx):
        t, j = np.nonzero(idx == e)                 # the tokens that chose expert e
        V = x[t].T                                  # [d][m], one column per token
        if cfg.is_ffn:
            h = expert_apply(inp.theta[0][e], inp.phi[0][e], w64[0], V, cfg.w_scale)
            a = gelu(h) if cfg.ffn_act == "gelu" else h
            z = expert_apply(inp.theta[1][e], inp.phi[1][e], w64[1], a, cfg.w_scale)
        else:
            z = expert_apply(inp.theta[0][e], inp.phi[0][e], w64[0], V, cfg.w_scale)
        np.add.at(y, t, gates[t, j][:, None] * z.T)
    return y, idx, gates


# ---------------------------------------------------------------------------
# parameter counts  ([MoE-pt] §2 memory O(d^2 + N d log d); [ViT-pt] §3)
# ---------------------------------------------------------------------------
def param_counts(d_model: int, n_experts: int, d_ff: int = 0, angle_bytes: int = 4,
                 dense_bytes: int = 4) -> dict:
    """Storage of one layer: shared ternary substrate(s) + per-expert angles,
    against N independent dense experts of the same shapes."""
    shapes = [(d_ff, d_model), (d_model, d_ff)] if d_ff else [(d_model, d_model)]
    angles_per_expert = 0
    substrate_weights = 0
    for d_out, d_in in shapes:
        angles_per_expert += (d_in // 2) * int(math.log2(d_in)) + (d_out // 2) * int(math.log2(d_out))
        substrate_weights += d_out * d_in
    return {
        "angles_per_expert": angles_per_expert,
        "angle_bytes_total": n_experts * angles_per_expert * angle_bytes,
        "substrate_weights": substrate_weights,
        "substrate_bytes_2bit": substrate_weights * 2 // 8,
        "ternary_entropy_bits": math.log2(3.0),
        "dense_expert_bytes_total": n_experts * substrate_weights * dense_bytes,
    }


def ternary_product(U: np.ndarray, w_base: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    """Z = alpha * U @ W_base^T in fp64: the shared-substrate product every
    routed row goes through ([MoE-zh] §2.1: rotated input times the ternary
    substrate).  U [M][d_in], W_base [d_out][d_in]."""
    return alpha * (np.asarray(U, dtype=np.float64) @ np.asarray(w_base, dtype=np.float64).T)


def router_backward(x64: np.ndarray, wg64: np.ndarray, idx: np.ndarray, dgate: np.ndarray,
                    renorm: bool = False):
    """Gradients of L = sum(dgate * gates) through the gating network with the
    chosen experts held ([MoE-nl] §2 "Gated Routing": standard top-k gating).
    Logits l = W_g x_t, p = softmax(l) over all N experts, gate_j = p_{e_j}
    (divided by the sum over the k chosen when ``renorm``).  Chain rule:
      without renorm  dl_n = p_n (a_n - s), a_n = sum_j dgate_j [n = e_j],
                      s = sum_j dgate_j p_{e_j};
      with renorm     dl_{e_j} = g_j (dgate_j - sum_i dgate_i g_i), other n 0;
    then dW_g = sum_t dl_t x_t^T and dx_t = W_g^T dl_t.
    x64 [T][d], wg64 [N][d], idx [T][k], dgate [T][k].
    Returns (dx [T][d], dW_g [N][d], dlogits [T][N])."""
    x64 = np.asarray(x64, dtype=np.float64)
    wg64 = np.asarray(wg64, dtype=np.float64)
    dgate = np.asarray(dgate, dtype=np.float64)
    T, N = x64.shape[0], wg64.shape[0]
    logits = x64 @ wg64.T
    m = logits.max(axis=1, keepdims=True)
    ex = np.exp(logits - m)
    p = ex / ex.sum(axis=1, keepdims=True)
    dl = np.zeros((T, N))
    rows = np.arange(T)[:, None]
    pc = p[rows, idx]                                   # [T][k] chosen probabilities
    if renorm:
        g = pc / pc.sum(axis=1, keepdims=True)
        inner = np.sum(dgate * g, axis=1, keepdims=True)
        np.add.at(dl, (np.repeat(np.arange(T), idx.shape[1]), idx.ravel()), (g * (dgate - inner)).ravel())
    else:
        a = np.zeros((T, N))
        np.add.at(a, (np.repeat(np.arange(T), idx.shape[1]), idx.ravel()), dgate.ravel())
        s = np.sum(dgate * pc, axis=1, keepdims=True)
        dl = p * (a - s)
    return dl @ wg64, dl.T @ x64, dl


def gelu_backward(h: np.ndarray, da: np.ndarray) -> np.ndarray:
    """dh = da * GELU'(h) for the exact (erf) GELU h Phi(h):
    GELU'(h) = Phi(h) + h phi(h), Phi the standard normal distribution function
    and phi its density ([ViT-pt] §2: the FFN's activation between its two
    projections)."""
    h = np.asarray(h, dtype=np.float64)
    Phi = 0.5 * (1.0 + _erf(h / math.sqrt(2.0)))
    phi = np.exp(-0.5 * h * h) / math.sqrt(2.0 * math.pi)
    return np.asarray(da, dtype=np.float64) * (Phi + h * phi)


def layer_backward_experts(inp, dy: np.ndarray, routing: "Routing"):
    """Gradients of L = sum(dy * y) through the experts of a square layer,
    with the routing and the gates held at ``routing`` (they are piecewise
    constant in the parameters for a fixed choice; the router's own gradient
    is a separate step).  Follows the forward's definition per routed slot
    (t, j) with expert e = idx[t][j] and gate g = gates[t][j]:
        u = B(theta_e)^T x_t,  z = alpha W_base u,  o = B(phi_e) z,  y_t += g o
    so the slot receives do = g dy_t, and the chain runs back through the
    output rotation (dphi_e, dz), the substrate (dW_base through the
    straight-through estimator, du = alpha W_base^T dz) and the input rotation
    (dtheta_e, dx_t += its input gradient).  Also returns the gates'
    gradients dgate[t][j] = dy_t . o.
    Returns dict(theta, phi [N][L][n/2], w_base [d][d], x [T][d], gate [T][k],
    w_base_abs): w_base_abs = alpha sum_r |dZ_r|^T |U_r|, the same sum as dW
    over magnitudes, a scale for the error of dW computed from rounded rows.

    FFN layers (two substrates, a GELU or the identity between) go through
    ``_ffn_backward``: the same chain twice with the activation's derivative
    between; their dict holds lists (up, down) for theta, phi and w_base."""
    cfg, x, _ = _inputs_f64(inp)
    if cfg.is_ffn:
        return _ffn_backward(inp, cfg, x, np.asarray(dy, dtype=np.float64), routing)
    dy = np.asarray(dy, dtype=np.float64)
    alpha = cfg.w_scale
    W = np.asarray(inp.w_base[0], dtype=np.float64)
    th_all, ph_all = inp.theta[0], inp.phi[0]
    dth = np.zeros(np.shape(th_all))
    dph = np.zeros(np.shape(ph_all))
    dW = np.zeros(W.shape)
    dWa = np.zeros(W.shape)
    dx = np.zeros(x.shape)
    dgate = np.zeros(routing.gates.shape)
    for e in np.unique(routing.idx):
        tok, slot = np.nonzero(routing.idx == e)
        th = np.asarray(th_all[e], dtype=np.float64)
        ph = np.asarray(ph_all[e], dtype=np.float64)
        X = x[tok].T                                     # columns = routed slots
        U = butterfly_apply(th, X, transpose=True)
        Z = alpha * (W @ U)
        O = butterfly_apply(ph, Z)
        dO = dy[tok].T * routing.gates[tok, slot][None, :]
        dgate[tok, slot] = np.sum(dy[tok].T * O, axis=0)
        dZ, dph[e] = butterfly_backward(ph, Z, dO, False)
        dW += substrate_weight_grad(U.T, dZ.T, alpha)
        dWa += substrate_weight_grad(np.abs(U.T), np.abs(dZ.T), abs(alpha))
        dU = alpha * (W.T @ dZ)
        dX, dth[e] = butterfly_backward(th, X, dU, True)
        np.add.at(dx, tok, dX.T)
    return {"theta": dth, "phi": dph, "w_base": dW, "x": dx, "gate": dgate, "w_base_abs": dWa}


def _ffn_backward(inp, cfg, x, dy, routing):
    """The FFN form of ``layer_backward_experts``: per routed slot
        u = B(th_up)^T x, h1 = alpha W_up u, h = B(ph_up) h1, a = act(h),
        v = B(th_dn)^T a, z = alpha W_dn v, o = B(ph_dn) z, y_t += g o
    walked back one step at a time ([ViT-pt] §2: rotations before and after
    each shared substrate of the FFN)."""
    alpha = cfg.w_scale
    Wu = np.asarray(inp.w_base[0], dtype=np.float64)
    Wd = np.asarray(inp.w_base[1], dtype=np.float64)
    out = {"theta": [np.zeros(np.shape(inp.theta[0])), np.zeros(np.shape(inp.theta[1]))],
           "phi": [np.zeros(np.shape(inp.phi[0])), np.zeros(np.shape(inp.phi[1]))],
           "w_base": [np.zeros(Wu.shape), np.zeros(Wd.shape)],
           "w_base_abs": [np.zeros(Wu.shape), np.zeros(Wd.shape)],
           "x": np.zeros(x.shape), "gate": np.zeros(routing.gates.shape)}
    use_gelu = cfg.ffn_act == "gelu"
    for e in np.unique(routing.idx):
        tok, slot = np.nonzero(routing.idx == e)
        thu, phu = (np.asarray(a[e], dtype=np.float64) for a in (inp.theta[0], inp.phi[0]))
        thd, phd = (np.asarray(a[e], dtype=np.float64) for a in (inp.theta[1], inp.phi[1]))
        X = x[tok].T
        U = butterfly_apply(thu, X, transpose=True)
        H1 = alpha * (Wu @ U)
        H = butterfly_apply(phu, H1)
        A = gelu(H) if use_gelu else H
        V = butterfly_apply(thd, A, transpose=True)
        Z = alpha * (Wd @ V)
        O = butterfly_apply(phd, Z)
        dO = dy[tok].T * routing.gates[tok, slot][None, :]
        out["gate"][tok, slot] = np.sum(dy[tok].T * O, axis=0)
        dZ, dphd = butterfly_backward(phd, Z, dO, False)
        out["w_base"][1] += substrate_weight_grad(V.T, dZ.T, alpha)
        out["w_base_abs"][1] += substrate_weight_grad(np.abs(V.T), np.abs(dZ.T), abs(alpha))
        dA, dthd = butterfly_backward(thd, A, alpha * (Wd.T @ dZ), True)
        dH = gelu_backward(H, dA) if use_gelu else dA
        dH1, dphu = butterfly_backward(phu, H1, dH, False)
        out["w_base"][0] += substrate_weight_grad(U.T, dH1.T, alpha)
        out["w_base_abs"][0] += substrate_weight_grad(np.abs(U.T), np.abs(dH1.T), abs(alpha))
        dX, dthu = butterfly_backward(thu, X, alpha * (Wu.T @ dH1), True)
        np.add.at(out["x"], tok, dX.T)
        out["theta"][0][e], out["phi"][0][e], out["theta"][1][e], out["phi"][1][e] = dthu, dphu, dthd, dphd
    return out


def substrate_weight_grad(U: np.ndarray, dZ: np.ndarray, alpha: float = 1.0) -> np.ndarray:
    """Gradient of the latent full-precision substrate, fp64.

    The substrate is trained with a straight-through estimator ([MoE-nl] §2
    "Drie Fasen": ternary quantisation with STE; [MoE-zh] §2.2): the forward
    uses the ternary codes, and the gradient passes through the quantiser
    unchanged, so the latent weights receive the gradient of the product
    Z = alpha U W^T with respect to W.  The substrate is shared by every expert,
    so the sum runs over all routed rows of all experts:
        dW[o][i] = alpha * sum_r dZ[r][o] U[r][i]
    U [R][d_in] (rows after the input rotation), dZ [R][d_out].  Returns
    dW [d_out][d_in].  The reading takes the estimator as the plain identity
    (no clipping of the latent weights' gradient): the pages name the
    estimator and nothing more."""
    return alpha * (np.asarray(dZ, dtype=np.float64).T @ np.asarray(U, dtype=np.float64))

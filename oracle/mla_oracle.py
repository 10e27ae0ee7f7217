"""Plain float64 CPU oracle for Multi-head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY.  Nothing in the product library may import, call or
link this file: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path; both are fed the same seeded arrays, widened exactly to float64 here.

Sources (cited by page and section; the pages print the equations, not code):
  [walkthrough]  "MLA（多头潜在注意力）" walkthrough, h.sjds.net/a/578141:
                 "1. MLA 的处理步骤描述" steps 1-5, and
                 "3. ... 训练态和推理态（decode）的差异点" orders A and B.
  [wiki]         "MLA 多头潜在注意力", chenshi221.pages.dev wiki:
                 "技术细节", "与 RoPE 的兼容性", "压缩比".
  [formulas]     DeepSeek-V2 MLA formula walk-through, modelers.csdn.net:
                 equations (9)-(13), "三、为什么能大幅减少 KV Cache".
  [blog]         attention-to-MLA blog, xianlaiwan.cn/article/379067
                 (RoPE paragraph; decoupled RoPE paragraph).
  [course]       "Day 18 · 注意力变体", ai.air7.fun: §3 MLA and the
                 decoupled RoPE key note.

Notation follows the pages: h_t hidden state (d), c_t^KV latent (d_c),
k_t^R shared RoPE key (d_R), c_t^Q query latent (d_c'), q^C_i / q^R_i the
per-head content / RoPE query parts.  Weights are row-major [out][in] with
y = W x.  Head i owns rows [i*d_h, (i+1)*d_h) of W_UQ, W_UK and W_UV, rows
[i*d_R, (i+1)*d_R) of W_QR, and columns [i*d_h, (i+1)*d_h) of W_O.

Readings where the pages are silent or garbled (each one is listed with its
reason in the design notes):
  * softmax scale 1/sqrt(d_h + d_R) in both orders;
  * RoPE pairs are interleaved (x_2k, x_2k+1), theta_k = base^(-2k/d_R),
    positions are 0-based, k^R is rotated before it is cached;
  * W_KR acts on h_t, W_QR acts on c^Q (per head);
  * no norms and no biases anywhere;
  * a decode query attends to every cached token including its own row.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
(brute force, textbook special cases, closed forms, exact identities); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------------------
# cache sizes ([formulas] §三 and [walkthrough] step 1)
# ---------------------------------------------------------------------------

def mla_numbers_per_token(d_c: int, d_r: int) -> int:
    """MLA caches only c_t^KV and the shared k_t^R for each token."""
    return d_c + d_r


def mha_numbers_per_token(n_h: int, d_h: int) -> int:
    """MHA caches a key and a value for every head ([formulas] §一)."""
    return 2 * n_h * d_h


def latent_compression_ratio(d_c: int, n_h: int, d_h: int) -> float:
    """d_c / (2 n_h d_h), the ratio [formulas] §三 prints (it leaves k^R out)."""
    return d_c / (2 * n_h * d_h)


# ---------------------------------------------------------------------------
# RoPE ([blog] RoPE paragraph: rotate q and k by their positions)
# ---------------------------------------------------------------------------

def rope_frequencies(d_r: int, base: float) -> np.ndarray:
    k = np.arange(d_r // 2, dtype=F64)
    return np.power(F64(base), -2.0 * k / d_r)


def rope(x: np.ndarray, pos, base: float) -> np.ndarray:
    """Rotate each pair (x_2k, x_2k+1) of the last axis by pos * theta_k.

    ``pos`` broadcasts against the leading axes of ``x``.
    """
    x = np.asarray(x, dtype=F64)
    d_r = x.shape[-1]
    theta = rope_frequencies(d_r, base)
    ang = np.asarray(pos, dtype=F64)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * cos - xo * sin
    out[..., 1::2] = xe * sin + xo * cos
    return out


# ---------------------------------------------------------------------------
# step 1: write memory ([formulas] eq. (9); [walkthrough] step 1)
# ---------------------------------------------------------------------------

def latent_rows(h: np.ndarray, W_DKV: np.ndarray, W_KR: np.ndarray, positions, base: float):
    """c_t^KV = W_DKV h_t and k_t^R = RoPE(W_KR h_t) for each row h_t of ``h``.

    Returns (c [T][d_c], k_R [T][d_R]).  No head index appears: one latent per
    token serves every head, for both keys and values.
    """
    h = np.asarray(h, dtype=F64)
    c = h @ np.asarray(W_DKV, F64).T
    k_r = rope(h @ np.asarray(W_KR, F64).T, np.asarray(positions), base)
    return c, k_r


# ---------------------------------------------------------------------------
# step 3: query side ([formulas] eq. (12), (13); [walkthrough] step 3)
# ---------------------------------------------------------------------------

def query(h_q: np.ndarray, W_DQ, W_UQ, W_QR, pos, n_h: int, base: float):
    """c^Q = W_DQ h; q^C_i = W_UQ,i c^Q; q^R_i = RoPE(W_QR,i c^Q) per head.

    Returns (q_C [n_h][d_h], q_R [n_h][d_R]).
    """
    c_q = np.asarray(W_DQ, F64) @ np.asarray(h_q, F64)
    q_c = (np.asarray(W_UQ, F64) @ c_q).reshape(n_h, -1)
    q_r = rope((np.asarray(W_QR, F64) @ c_q).reshape(n_h, -1), pos, base)
    return q_c, q_r


# ---------------------------------------------------------------------------
# step 4: attention
# ---------------------------------------------------------------------------

def softmax(s: np.ndarray, axis: int = -1) -> np.ndarray:
    """exp(s_j) / sum_k exp(s_k); the shift by the max is exact in real arithmetic."""
    s = np.asarray(s, F64)
    e = np.exp(s - np.max(s, axis=axis, keepdims=True))
    return e / np.sum(e, axis=axis, keepdims=True)


def attend_order_a(q_c, q_r, c, k_r, W_UK, W_UV, scale: float, return_p: bool = False):
    """Order A ([walkthrough] §3 顺序 A and step 4): decompress, then dot.

    Per head i: k_ij = [W_UK,i c_j ; k^R_j] (d_h + d_R wide), v_ij = W_UV,i c_j
    ([formulas] eq. (10), (11)), q_i = [q^C_i ; q^R_i], s_ij = q_i . k_ij * scale,
    p_i = softmax_j(s_i), o_i = sum_j p_ij v_ij.  Returns o [n_h][d_h].
    """
    n_h, d_h = q_c.shape
    c = np.asarray(c, F64)
    k_r = np.asarray(k_r, F64)
    W_UK = np.asarray(W_UK, F64)
    W_UV = np.asarray(W_UV, F64)
    o = np.empty((n_h, d_h), F64)
    ps = []
    for i in range(n_h):
        rows = slice(i * d_h, (i + 1) * d_h)
        k = np.concatenate([c @ W_UK[rows].T, k_r], axis=1)     # [N][d_h + d_R]
        v = c @ W_UV[rows].T                                     # [N][d_h]
        q = np.concatenate([q_c[i], q_r[i]])
        p = softmax(k @ q * scale)
        o[i] = p @ v
        ps.append(p)
    return (o, np.stack(ps)) if return_p else o


def absorbed_query(q_c, q_r, W_UK, scale: float) -> np.ndarray:
    """Order B query side ([walkthrough] §3 顺序 B; [formulas] §三 absorption).

    q~_i = W_UK,i^T q^C_i (d_c wide) is the per-head "absorbed query"; packed
    with q^R_i and the softmax scale as Q~_i = [q~_i ; q^R_i] * scale, so that
    s_ij = Q~_i . [c_j ; k^R_j].  Returns Q~ [n_h][d_c + d_R].
    """
    n_h, d_h = q_c.shape
    W_UK = np.asarray(W_UK, F64)
    qt = np.stack([W_UK[i * d_h:(i + 1) * d_h].T @ q_c[i] for i in range(n_h)])
    return np.concatenate([qt, np.asarray(q_r, F64)], axis=1) * scale


def latent_attention(Qt: np.ndarray, rows: np.ndarray, d_c: int) -> np.ndarray:
    """Scores Q~ . row_j over the cached rows, softmax per head, and the
    weighted sum of the latents c_j in d_c-space ([walkthrough] §3 顺序 B,
    "先在 512 维潜空间加权求和").  Returns o~ [n_h][d_c]."""
    rows = np.asarray(rows, F64)
    p = softmax(np.asarray(Qt, F64) @ rows.T, axis=1)
    return p @ rows[:, :d_c]


def latent_output(o_lat: np.ndarray, W_UV, W_O) -> np.ndarray:
    """Decompress once per head, o_i = W_UV,i o~_i, then integrate, u = W_O [o_0; ...]."""
    n_h = o_lat.shape[0]
    W_UV = np.asarray(W_UV, F64)
    d_h = W_UV.shape[0] // n_h
    o = np.stack([W_UV[i * d_h:(i + 1) * d_h] @ o_lat[i] for i in range(n_h)])
    return integrate(o, W_O)


def attend_order_b(q_c, q_r, c, k_r, W_UK, W_UV, scale: float) -> np.ndarray:
    """Order B: absorb W_UK into the query, attend in latent space, apply W_UV
    once.  Returns o [n_h][d_h] (equal to order A in exact arithmetic)."""
    n_h, d_h = q_c.shape
    Qt = absorbed_query(q_c, q_r, W_UK, scale)
    rows = np.concatenate([np.asarray(c, F64), np.asarray(k_r, F64)], axis=1)
    o_lat = latent_attention(Qt, rows, c.shape[1])
    W_UV = np.asarray(W_UV, F64)
    return np.stack([W_UV[i * d_h:(i + 1) * d_h] @ o_lat[i] for i in range(n_h)])


# ---------------------------------------------------------------------------
# order B on matrices multiplied out ahead of time ([walkthrough] §3 顺序 B:
# the product is computed once at deployment and decoding runs B on it;
# [formulas] §三: W^UK goes into the query projection, W^UV into W^O)
# ---------------------------------------------------------------------------

def merged_query_matrix(W_UQ, W_UK, n_h: int) -> np.ndarray:
    """W_UQK,i = W_UK,i^T W_UQ,i ([d_c][d_c'] per head), stacked by head, so
    that q~_i = W_UQK,i c^Q.  Returns [n_h * d_c][d_c']."""
    W_UQ, W_UK = np.asarray(W_UQ, F64), np.asarray(W_UK, F64)
    d_h = W_UQ.shape[0] // n_h
    return np.concatenate([W_UK[i * d_h:(i + 1) * d_h].T @ W_UQ[i * d_h:(i + 1) * d_h]
                           for i in range(n_h)], axis=0)


def merged_output_matrix(W_O, W_UV, n_h: int) -> np.ndarray:
    """W_OUV,i = W_O,i W_UV,i ([d][d_c] per head; W_O,i = the head's d_h
    columns of W_O), side by side, so that u = sum_i W_OUV,i o~_i.  Returns
    [d][n_h * d_c]."""
    W_O, W_UV = np.asarray(W_O, F64), np.asarray(W_UV, F64)
    d_h = W_UV.shape[0] // n_h
    return np.concatenate([W_O[:, i * d_h:(i + 1) * d_h] @ W_UV[i * d_h:(i + 1) * d_h]
                           for i in range(n_h)], axis=1)


def decode_merged(h_q, pos: int, c, k_r, Wm: Dict[str, np.ndarray], n_h: int, base: float,
                  scale: float) -> np.ndarray:
    """One decode query from the merged matrices (Wm holds W_DQ, W_QR, W_UQK,
    W_OUV): c^Q = W_DQ h; Q~_i = [W_UQK,i c^Q ; RoPE(W_QR,i c^Q)] * scale;
    o~ by latent attention over the rows [c_j ; k^R_j]; u = W_OUV [o~_0; ...]."""
    c, k_r = np.asarray(c, F64), np.asarray(k_r, F64)
    d_c, d_r = c.shape[1], k_r.shape[1]
    c_q = np.asarray(Wm["W_DQ"], F64) @ np.asarray(h_q, F64)
    qt = (np.asarray(Wm["W_UQK"], F64) @ c_q).reshape(n_h, d_c)
    W_QR = np.asarray(Wm["W_QR"], F64)
    q_r = np.stack([rope(W_QR[i * d_r:(i + 1) * d_r] @ c_q, pos, base) for i in range(n_h)])
    Qt = np.concatenate([qt, q_r], axis=1) * scale
    o_lat = latent_attention(Qt, np.concatenate([c, k_r], axis=1), d_c)
    return np.asarray(Wm["W_OUV"], F64) @ o_lat.reshape(-1)


# ---------------------------------------------------------------------------
# the multi-head baseline the pages weigh MLA against ([formulas] §一 and §三;
# [walkthrough] §2): a key and a value cached per head and token
# ---------------------------------------------------------------------------

def mha_attention(q, K, V, scale: float) -> np.ndarray:
    """One query of every head over a multi-head cache: q [n_h][d_h], K and V
    [N][n_h][d_h]; head i: o_i = sum_j softmax_j(scale q_i . K[j, i]) V[j, i].
    Returns [n_h][d_h]."""
    q, K, V = (np.asarray(x, F64) for x in (q, K, V))
    n_h = q.shape[0]
    out = []
    for i in range(n_h):
        p = softmax(K[:, i] @ q[i] * scale)
        out.append(p @ V[:, i])
    return np.stack(out)


# ---------------------------------------------------------------------------
# step 5: integrate ([walkthrough] step 5)
# ---------------------------------------------------------------------------

def integrate(o: np.ndarray, W_O) -> np.ndarray:
    """Concatenate the heads' outputs (n_h * d_h) and project back to d."""
    return np.asarray(W_O, F64) @ np.asarray(o, F64).reshape(-1)


# ---------------------------------------------------------------------------
# whole layer
# ---------------------------------------------------------------------------

def default_scale(d_h: int, d_r: int) -> float:
    return 1.0 / math.sqrt(d_h + d_r)


def decode(h_q, pos: int, c, k_r, W: Dict[str, np.ndarray], n_h: int, base: float,
           scale: Optional[float] = None, order: str = "A") -> np.ndarray:
    """One decode query over the cached rows (c, k_r); returns u [d]."""
    d_h = W["W_UQ"].shape[0] // n_h
    d_r = W["W_QR"].shape[0] // n_h
    if scale is None:
        scale = default_scale(d_h, d_r)
    q_c, q_r = query(h_q, W["W_DQ"], W["W_UQ"], W["W_QR"], pos, n_h, base)
    attend = attend_order_a if order == "A" else attend_order_b
    o = attend(q_c, q_r, c, k_r, W["W_UK"], W["W_UV"], scale)
    return integrate(o, W["W_O"])


def decode_from_hidden(H: np.ndarray, W: Dict[str, np.ndarray], n_h: int, base: float,
                       scale: Optional[float] = None, order: str = "A") -> np.ndarray:
    """Tokens 0..N-1 with hidden states H; the last one is the decode query at
    position N-1 and attends to all N cached rows (its own included)."""
    N = H.shape[0]
    c, k_r = latent_rows(H, W["W_DKV"], W["W_KR"], np.arange(N), base)
    return decode(H[-1], N - 1, c, k_r, W, n_h, base, scale, order)


def prefill_order_a(H: np.ndarray, positions, c, k_r, W: Dict[str, np.ndarray], n_h: int,
                    base: float, scale: Optional[float] = None, rows=None) -> np.ndarray:
    """Causal prefill in order A: query t (position positions[t]) attends to the
    cached rows 0..positions[t].  ``rows`` selects which query rows to return
    (all by default).  Returns u [len(rows)][d]."""
    d_h = W["W_UQ"].shape[0] // n_h
    d_r = W["W_QR"].shape[0] // n_h
    if scale is None:
        scale = default_scale(d_h, d_r)
    positions = np.asarray(positions)
    rows = range(H.shape[0]) if rows is None else rows
    out = []
    for t in rows:
        p = int(positions[t])
        q_c, q_r = query(H[t], W["W_DQ"], W["W_UQ"], W["W_QR"], p, n_h, base)
        o = attend_order_a(q_c, q_r, c[:p + 1], k_r[:p + 1], W["W_UK"], W["W_UV"], scale)
        out.append(integrate(o, W["W_O"]))
    return np.stack(out)


# ---------------------------------------------------------------------------
# order A backward ([walkthrough] §3 顺序 A: training keeps W_UK and W_UV as
# two matrices, each with its own gradient path)
# ---------------------------------------------------------------------------

def attend_order_a_backward(q_c, q_r, positions, c, k_r, W_UK, W_UV, scale: float, dO):
    """Gradients of causal order-A attention.  Forward, for query t at
    position positions[t] and head i over the cached rows j <= positions[t]:
      k_ij = [W_UK,i c_j ; k^R_j],  v_ij = W_UV,i c_j,
      s_tij = scale [q^C_ti ; q^R_ti] . k_ij,  p_tij = softmax_j(s_tij),
      o_ti = sum_j p_tij v_ij.
    Given dO = dL/do [T][n_h][d_h], the chain rule through these steps gives
      dv_ij = sum_t p_tij dO_ti,   dp_tij = dO_ti . v_ij,
      ds_tij = p_tij (dp_tij - sum_j' p_tij' dp_tij'),
      dk_ij = scale sum_t ds_tij [q^C_ti ; q^R_ti],
      dq_ti = scale sum_j ds_tij k_ij,
      dW_UK,i = sum_j dk^C_ij c_j^T,  dW_UV,i = sum_j dv_ij c_j^T,
      dc_j = sum_i (W_UK,i^T dk^C_ij + W_UV,i^T dv_ij),  dk^R_j = sum_i dk^R_ij.
    q_c [T][n_h][d_h], q_r [T][n_h][d_R], c [N][d_c], k_r [N][d_R].
    Returns dict(dW_UK, dW_UV [n_h d_h][d_c], dq_c, dq_r, dc [N][d_c], dk_r [N][d_R])."""
    q_c, q_r, c, k_r, dO = (np.asarray(x, F64) for x in (q_c, q_r, c, k_r, dO))
    W_UK, W_UV = np.asarray(W_UK, F64), np.asarray(W_UV, F64)
    T, n_h, d_h = q_c.shape
    N = c.shape[0]
    mask = np.arange(N)[None, :] <= np.asarray(positions)[:, None]
    out = {k: np.zeros_like(v) for k, v in (("dW_UK", W_UK), ("dW_UV", W_UV), ("dq_c", q_c),
                                            ("dq_r", q_r), ("dc", c), ("dk_r", k_r))}
    for i in range(n_h):
        hs = slice(i * d_h, (i + 1) * d_h)
        K, V = c @ W_UK[hs].T, c @ W_UV[hs].T
        S = np.where(mask, scale * (q_c[:, i] @ K.T + q_r[:, i] @ k_r.T), -np.inf)
        P = softmax(S, axis=1)
        dP = dO[:, i] @ V.T
        dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
        dV = P.T @ dO[:, i]
        dK = scale * dS.T @ q_c[:, i]
        out["dq_c"][:, i] = scale * dS @ K
        out["dq_r"][:, i] = scale * dS @ k_r
        out["dk_r"] += scale * dS.T @ q_r[:, i]
        out["dW_UK"][hs] = dK.T @ c
        out["dW_UV"][hs] = dV.T @ c
        out["dc"] += dK @ W_UK[hs] + dV @ W_UV[hs]
    return out


# ---------------------------------------------------------------------------
# brute force (tiny shapes only): explicit loops, no matrix routines and no
# reuse of the functions above
# ---------------------------------------------------------------------------

def decode_bruteforce(H, W: Dict[str, np.ndarray], n_h: int, base: float, scale: float):
    """Same layer as ``decode_from_hidden(order='A')`` written as scalar loops."""
    H = [[float(v) for v in row] for row in np.asarray(H, F64)]
    Wl = {k: [[float(v) for v in r] for r in np.asarray(m, F64)] for k, m in W.items()}
    N, d = len(H), len(H[0])
    d_c = len(Wl["W_DKV"])
    d_r = len(Wl["W_KR"])
    d_h = len(Wl["W_UQ"]) // n_h
    d_cq = len(Wl["W_DQ"])

    def matvec(M, x, r0=0, r1=None):
        r1 = len(M) if r1 is None else r1
        out = []
        for r in range(r0, r1):
            acc = 0.0
            for k in range(len(x)):
                acc += M[r][k] * x[k]
            out.append(acc)
        return out

    def rot(x, pos):
        y = list(x)
        for k in range(len(x) // 2):
            ang = pos * (base ** (-(2.0 * k) / len(x)))
            cs, sn = math.cos(ang), math.sin(ang)
            y[2 * k] = x[2 * k] * cs - x[2 * k + 1] * sn
            y[2 * k + 1] = x[2 * k] * sn + x[2 * k + 1] * cs
        return y

    cache = [(matvec(Wl["W_DKV"], H[j]), rot(matvec(Wl["W_KR"], H[j]), j)) for j in range(N)]
    hq = H[N - 1]
    cq = matvec(Wl["W_DQ"], hq)
    assert len(cq) == d_cq
    o_all = []
    for i in range(n_h):
        qc = matvec(Wl["W_UQ"], cq, i * d_h, (i + 1) * d_h)
        qr = rot(matvec(Wl["W_QR"], cq, i * d_r, (i + 1) * d_r), N - 1)
        scores = []
        vals = []
        for j in range(N):
            cj, krj = cache[j]
            kc = matvec(Wl["W_UK"], cj, i * d_h, (i + 1) * d_h)
            v = matvec(Wl["W_UV"], cj, i * d_h, (i + 1) * d_h)
            s = 0.0
            for a in range(d_h):
                s += qc[a] * kc[a]
            for a in range(d_r):
                s += qr[a] * krj[a]
            scores.append(s * scale)
            vals.append(v)
        m = max(scores)
        e = [math.exp(s - m) for s in scores]
        z = sum(e)
        o = [0.0] * d_h
        for j in range(N):
            for a in range(d_h):
                o[a] += e[j] / z * vals[j][a]
        o_all.extend(o)
    u = matvec(Wl["W_O"], o_all)
    assert len(u) == d
    return np.array(u, F64)


# ---------------------------------------------------------------------------
# tolerance metric
# ---------------------------------------------------------------------------

def max_rel_error(y: np.ndarray, ref: np.ndarray) -> float:
    """max over output vectors of max_k |y_k - ref_k| / max_k |ref_k|.

    The last axis is the vector; leading axes index vectors."""
    y = np.asarray(y, F64)
    ref = np.asarray(ref, F64)
    ref2 = ref.reshape(-1, ref.shape[-1])
    y2 = y.reshape(-1, ref.shape[-1])
    den = np.max(np.abs(ref2), axis=1)
    num = np.max(np.abs(y2 - ref2), axis=1)
    den = np.where(den == 0, 1.0, den)
    if not np.all(np.isfinite(y2)):
        return float("inf")
    return float(np.max(num / den))

"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each pin takes an oracle handle and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix.  They are collected by
test_oracle_pins.py (against the real oracle) and by test_oracle_mutants.py
(against deliberately broken builds, each of which some pin must reject).

Sources, by page title:
  [Atlas]  "Kimi K3 - KDA layer" (OpenModelAtlas): step equations and the
           parameter table of the KDA block.
  [Baena]  "Inside Kimi K3: How KDA, AttnRes, and 896 Experts Work":
           "KDA writes corrections into a recurrent matrix", "The lower bound
           on decay is a hardware decision", "Short convolutions ...".
  [SGLang] "Kimi K3: Architecture and SGLang Day-0 Support": "Attention
           mechanisms in detail" (linear attention, DeltaNet, KDA and their
           math boxes), "KV cache memory estimation".
  [Jawad]  "Kimi K3's Architecture: Kimi Delta Attention, Attention
           Residuals, and 896 Experts": "Deriving the delta rule".
"""
from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _core(orc, q, k, v, la, b, S0=None, scale=1.0):
    """One sequence, one head, prologue and epilogue off.  q,k,la: [T,dk]; v: [T,dv]."""
    T = q.shape[0]
    o, s, _ = orc.prefill(q[:, None], k[:, None], v[:, None], la[:, None], np.asarray(b)[:, None],
                          [0, T], state_in=None if S0 is None else S0[None, None], scale=scale,
                          prologue=False, epilogue=False, threads=1)
    return o[:, 0], s[0, 0]


def _close(a, b, tol, what):
    a = np.asarray(a, np.float64); b = np.asarray(b, np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    ref = max(1.0, float(np.max(np.abs(b)))) if b.size else 1.0
    assert err <= tol * ref, f"{what}: max err {err:.3e} > {tol:.1e}"


# --------------------------------------------------------------------------- pins

def pin_no_decay_no_write_keeps_state(orc):
    """alpha = 1 (log alpha = 0) and beta = 0: the state is untouched, and every
    read is scale * S0^T q ([Atlas] update and read steps with those gates)."""
    r = _rng(1)
    T, dk, dv = 6, 8, 5
    S0 = r.standard_normal((dk, dv))
    q = r.standard_normal((T, dk)); k = _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    o, S = _core(orc, q, k, v, np.zeros((T, dk)), np.zeros(T), S0, scale=0.37)
    assert np.array_equal(S, S0), "state changed with alpha=1, beta=0"
    _close(o, 0.37 * q @ S0, 1e-13, "read of the untouched state")


def pin_beta1_exact_recall(orc):
    """beta = 1 with a unit key: right after the write the state returns v
    exactly for that key ([Jawad] "Deriving the delta rule": at beta = 1 the
    read returns v_t exactly; [SGLang] KDA math box: beta = 1 replaces fully)."""
    r = _rng(2)
    T, dk, dv = 7, 6, 4
    S0 = r.standard_normal((dk, dv))
    k = _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    la = -5.0 * r.random((T, dk))
    o, _ = _core(orc, k, k, v, la, np.ones(T), S0, scale=1.0)
    _close(o, v, 1e-12, "S_t^T k_t at beta=1")


def pin_orthonormal_keys_store_all(orc):
    """beta = 1, alpha = 1, S0 = 0 and 128 orthonormal keys: the writes do not
    interfere, so S = sum_i k_i v_i^T and every key reads back its own value
    ([SGLang] DeltaNet math box: crosstalk-free iff the keys are pairwise
    orthogonal, at most d_k of them)."""
    r = _rng(3)
    d = 128
    Q, _ = np.linalg.qr(r.standard_normal((d, d)))
    K = Q.T  # rows are orthonormal keys
    V = r.standard_normal((d, d))
    _, S = _core(orc, K, K, V, np.zeros((d, d)), np.ones(d), None, scale=1.0)
    _close(S, K.T @ V, 1e-12, "S after orthonormal writes")
    _close(K @ S, V, 1e-12, "read-back of every stored key")


def pin_retention_identity(orc):
    """For a unit key and any beta, S_t^T k_t = (1-beta) (Diag(alpha) S_{t-1})^T k_t
    + beta v_t ([SGLang] KDA math box), and the whole update equals one
    gradient step on 1/2 ||S^T k - v||^2 taken from the decayed state
    ([Jawad] "Deriving the delta rule")."""
    r = _rng(4)
    dk, dv = 8, 3
    for trial in range(5):
        S_prev = r.standard_normal((dk, dv))
        k = _unit(r.standard_normal(dk)); v = r.standard_normal(dv)
        la = -5.0 * r.random(dk); b = r.random()
        o, S = _core(orc, k[None], k[None], v[None], la[None], [b], S_prev, scale=1.0)
        St = np.exp(la)[:, None] * S_prev
        _close(o[0], (1 - b) * (St.T @ k) + b * v, 1e-12, "retention identity")
        grad = np.outer(k, St.T @ k - v)
        _close(S, St - b * grad, 1e-12, "gradient-step form")


def pin_decay_only(orc):
    """beta = 0: only the gate acts, S_T = Diag(exp(sum_t log alpha_t)) S0
    ([Atlas] S <- Diag(alpha) S, alpha acting on the key channel = row)."""
    r = _rng(5)
    T, dk, dv = 9, 6, 4
    S0 = r.standard_normal((dk, dv))
    la = -5.0 * r.random((T, dk))
    q = r.standard_normal((T, dk)); k = _unit(r.standard_normal((T, dk)))
    v = r.standard_normal((T, dv))
    _, S = _core(orc, q, k, v, la, np.zeros(T), S0)
    _close(S, np.exp(la.sum(0))[:, None] * S0, 1e-12, "decay-only state")


def pin_one_hot_keys_are_scalar_emas(orc):
    """Axis-aligned keys decouple the rows: writing along e_m turns row m into
    (1-beta) alpha_m S[m,:] + beta v and leaves every other row at alpha_i S[i,:]
    -- a per-row exponential moving average, computed here in exact rationals."""
    r = _rng(6)
    T, dk, dv = 8, 4, 3
    S0 = r.integers(-4, 5, (dk, dv)).astype(np.float64)
    m = r.integers(0, dk, T)
    k = np.eye(dk)[m]
    v = r.integers(-8, 9, (T, dv)).astype(np.float64)
    alpha = r.choice([0.5, 0.75, 0.25, 1.0], (T, dk))
    la = np.log(alpha)
    b = r.choice([0.0, 0.25, 0.5, 1.0], T)
    _, S = _core(orc, k, k, v, la, b, S0)
    E = [[Fraction(x) for x in row] for row in S0]
    for t in range(T):
        a = [Fraction(math.exp(x)) for x in la[t]]
        bt = Fraction(b[t])
        for i in range(dk):
            for j in range(dv):
                E[i][j] = a[i] * E[i][j]
        for j in range(dv):
            E[m[t]][j] = (1 - bt) * E[m[t]][j] + bt * Fraction(v[t, j])
    _close(S, np.array([[float(x) for x in row] for row in E]), 1e-13, "one-hot EMA")


def _unrolled(S0, k, v, la, b, t):
    """S_t = M_t...M_1 S0 + sum_{s<=t} M_t...M_{s+1} beta_s k_s v_s^T with
    M_u = (I - beta_u k_u k_u^T) Diag(alpha_u): the unrolled form of the KDA
    recurrence ([SGLang] KDA math box), later factors on the left, plus the
    S0 term the page leaves out."""
    dk = S0.shape[0]
    M = [(np.eye(dk) - b[u] * np.outer(k[u], k[u])) @ np.diag(np.exp(la[u])) for u in range(t)]

    def prod(lo, hi):  # M_{hi-1} ... M_{lo}
        P = np.eye(dk)
        for u in range(lo, hi):
            P = M[u] @ P
        return P

    S = prod(0, t) @ S0
    for s in range(t):
        S = S + prod(s + 1, t) @ (b[s] * np.outer(k[s], v[s]))
    return S


def pin_unrolled_product_form(orc):
    """T <= 4 tokens against the explicit product form, every prefix read,
    keys of arbitrary norm (the recurrence itself does not normalise)."""
    r = _rng(7)
    for trial in range(6):
        T = 1 + trial % 4
        dk, dv = 5, 3
        S0 = r.standard_normal((dk, dv))
        q = r.standard_normal((T, dk)); k = r.standard_normal((T, dk)) * 0.7
        v = r.standard_normal((T, dv)); la = -5.0 * r.random((T, dk)); b = r.random(T)
        o, S = _core(orc, q, k, v, la, b, S0, scale=0.8)
        for t in range(1, T + 1):
            _close(o[t - 1], 0.8 * _unrolled(S0, k, v, la, b, t).T @ q[t - 1], 1e-12,
                   f"read at t={t}")
        _close(S, _unrolled(S0, k, v, la, b, T), 1e-12, "final state")


def pin_teaching_examples_2d(orc):
    """The 2-D teaching slice printed on the SGLang page (golden fixture)."""
    with open(os.path.join(GOLDEN, "teaching_2d.json")) as f:
        gold = {c["name"]: c for c in json.load(f)["cases"]}
    ka = np.array([1.0, 1.0]) / math.sqrt(2.0)
    kb = np.array([1.0, -1.0]) / math.sqrt(2.0)
    K = np.stack([ka, ka]); V = np.array([[1.0], [4.0]])
    # beta = 1 twice: the second write replaces the first
    o, _ = _core(orc, K, K, V, np.zeros((2, 2)), [1.0, 1.0])
    _close(o[1, 0], gold["delta_beta1"]["reads"], 1e-14, "delta rule, beta=1")
    assert abs(o[1, 0] - gold["naive_sum"]["reads"]) > 0.5, "read equals plain accumulation"
    for beta in (0.0, 0.3, 0.5, 0.9):
        o, _ = _core(orc, K, K, V, np.zeros((2, 2)), [1.0, beta])
        _close(o[1, 0], (1 - beta) * 1 + 4 * beta, 1e-14, f"delta rule, beta={beta}")
    for a1, a2, beta in ((0.5, 1.0, 0.4), (0.9, 0.2, 1.0), (0.3, 0.3, 0.0)):
        la = np.log(np.array([[1.0, 1.0], [a1, a2]]))
        o, _ = _core(orc, K, K, V, la, [1.0, beta])
        _close(o[1, 0], (1 - beta) * (a1 + a2) / 2 + 4 * beta, 1e-14, "gated delta rule")
    for theta in (0.3, 1.1, 2.0):
        kb_t = np.array([math.cos(math.pi / 4 - theta), math.sin(math.pi / 4 - theta)])
        va, vb = 1.5, -0.7
        S0 = np.outer(ka, [va]) + np.outer(kb_t, [vb])
        o, _ = _core(orc, ka[None], ka[None], np.zeros((1, 1)), np.zeros((1, 2)), [0.0], S0)
        _close(o[0, 0], va + math.cos(theta) * vb, 1e-14, "crosstalk read")
    # the two page keys are orthogonal: no crosstalk at all
    S0 = np.outer(ka, [2.0]) + np.outer(kb, [3.0])
    o, _ = _core(orc, ka[None], ka[None], np.zeros((1, 1)), np.zeros((1, 2)), [0.0], S0)
    _close(o[0, 0], 2.0, 1e-14, "orthogonal keys read")


def _silu(x):
    return x / (1.0 + np.exp(-x))


def pin_prologue_conv_taps(orc):
    """Causal depthwise conv of width 4 then SiLU ([Atlas] q^c_t = SiLU(sum_j
    w_j * q^p_{t-j}); [Baena] Swish, L2 on q and k, none on v).  One-hot taps
    select x_{t-j}; with q = k, one token, beta = 1, alpha = 1 and S0 = 0 the
    read is (q^.k^) v^c = v^c and the state is k^ v^c^T."""
    r = _rng(8)
    H, d, N = 2, 4, 5
    taps = r.integers(0, 4, (H * d,))
    w1 = np.zeros((H * d, 4)); w1[np.arange(H * d), taps] = 1.0
    wscale = r.uniform(0.5, 1.5, (H * d, 1))
    w = w1 * wscale
    x = r.standard_normal((N, H, d))
    hist = r.standard_normal((N, 3, H * d))  # oldest first: x_{t-3}, x_{t-2}, x_{t-1}
    o, S, conv_out = orc.prefill(x, x, x, np.zeros((N, H, d)), np.ones((N, H)),
                                 np.arange(N + 1), conv_w=(w, w, w), conv_in=(hist, hist, hist),
                                 scale=1.0, l2_eps=0.0, epilogue=False, threads=1)
    for n in range(N):
        for h in range(H):
            sel = np.empty(d)
            for c in range(d):
                ch = h * d + c
                j = taps[ch]
                sel[c] = x[n, h, c] if j == 0 else hist[n, 3 - j, ch]
            y = _silu(sel * wscale[h * d:(h + 1) * d, 0])
            _close(o[n, h], y, 1e-13, "v stream after conv+SiLU")
            kh = y / np.linalg.norm(y)
            _close(S[n, h], np.outer(kh, y), 1e-13, "k stream after conv+SiLU+L2")
    for s in range(3):
        assert np.array_equal(conv_out[s][:, :2], hist[:, 1:]), "conv cache shift"
        assert np.array_equal(conv_out[s][:, 2], x.reshape(N, H * d)), "conv cache newest entry"


def pin_conv_cache_short_sequences(orc):
    """The cache keeps the last three pre-conv inputs, oldest first; sequences
    shorter than three keep the tail of the incoming cache; an empty sequence
    passes state and cache through unchanged."""
    r = _rng(9)
    H, d = 1, 3
    lens = [0, 1, 2, 3, 5]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1]); N = len(lens)
    x = r.standard_normal((T, H, d))
    w = r.standard_normal((H * d, 4))
    hist = r.standard_normal((N, 3, H * d))
    S0 = r.standard_normal((N, H, d, d))
    _, S, co = orc.prefill(x, x, x, -r.random((T, H, d)), r.random((T, H)), cu,
                           conv_w=(w, w, w), conv_in=(hist, hist, hist), state_in=S0,
                           epilogue=False, threads=1)
    assert np.array_equal(S[0], S0[0]), "empty sequence must pass the state through"
    for n, L in enumerate(lens):
        seq = np.concatenate([hist[n], x[cu[n]:cu[n + 1], 0]], axis=0)
        for s in range(3):
            assert np.array_equal(co[s][n], seq[-3:]), f"conv cache of a length-{L} sequence"


def pin_epilogue_gate_rmsnorm(orc):
    """o^g = sigma(g) * RMSNorm(o~) per head over d_v ([Atlas] last two steps):
    unit RMS when the gate is open and the gain is one, half of it at g = 0,
    a per-channel gain multiplies, and RMSNorm ignores the scale of o~."""
    r = _rng(10)
    T, H, d = 5, 2, 8
    q = r.standard_normal((T, H, d)); k = _unit(r.standard_normal((T, H, d)))
    v = r.standard_normal((T, H, d)); la = -5 * r.random((T, H, d)); b = r.random((T, H))
    cu = [0, T]

    def run(vv, g, rw=None):
        o, _, _ = orc.prefill(q, k, vv, la, b, cu, g=g, rms_w=rw, rms_eps=0.0,
                              prologue=False, threads=1)
        return o
    o_open = run(v, np.full((T, H, d), 40.0))
    _close(np.sqrt((o_open ** 2).mean(-1)), np.ones((T, H)), 1e-12, "unit RMS with open gate")
    _close(run(v, np.zeros((T, H, d))), 0.5 * o_open, 1e-12, "gate at g=0 halves")
    _close(run(3.7 * v, np.full((T, H, d), 40.0)), o_open, 1e-12, "scale invariance of RMSNorm")
    rw = r.uniform(0.5, 2.0, d)
    _close(run(v, np.full((T, H, d), 40.0), rw), o_open * rw, 1e-12, "per-channel gain")
    g = r.standard_normal((T, H, d))
    _close(run(v, g), o_open / (1 + np.exp(-g)), 1e-12, "sigmoid gate")


def _layer_inputs(r, T, H, d):
    return dict(q=r.standard_normal((T, H, d)), k=r.standard_normal((T, H, d)),
                v=r.standard_normal((T, H, d)), g=r.standard_normal((T, H, d)),
                log_alpha=-5 / (1 + np.exp(-r.standard_normal((T, H, d)))),
                beta=1 / (1 + np.exp(-r.standard_normal((T, H)))))


def pin_chaining(orc):
    """State and conv cache are the whole memory of a sequence: prefill(a)
    then prefill(b) from the returned state and cache equals prefill(a || b),
    and prefill(T) followed by m decode steps equals prefill(T + m)."""
    r = _rng(11)
    T, H, d = 11, 2, 16
    x = _layer_inputs(r, T, H, d)
    cw = r.standard_normal((3, H * d, 4)) * 0.5
    S0 = r.standard_normal((1, H, d, d)) * 0.1
    ci = r.standard_normal((1, 3, 3, H * d))
    kw = dict(conv_w=cw, threads=1)
    o_all, s_all, c_all = orc.prefill(**x, cu_seqlens=[0, T], state_in=S0, conv_in=ci, **kw)
    a = {n: t[:4] for n, t in x.items()}
    bpart = {n: t[4:] for n, t in x.items()}
    o1, s1, c1 = orc.prefill(**a, cu_seqlens=[0, 4], state_in=S0, conv_in=ci, **kw)
    o2, s2, c2 = orc.prefill(**bpart, cu_seqlens=[0, T - 4], state_in=s1, conv_in=c1, **kw)
    _close(np.concatenate([o1, o2]), o_all, 1e-12, "chained prefill outputs")
    _close(s2, s_all, 1e-12, "chained prefill state")
    assert np.array_equal(c2, c_all), "chained conv cache"
    # prefill(8) then 3 decode steps
    p = {n: t[:8] for n, t in x.items()}
    o_p, s, c = orc.prefill(**p, cu_seqlens=[0, 8], state_in=S0, conv_in=ci, **kw)
    outs = [o_p]
    for t in range(8, T):
        step = {n: tt[t:t + 1] for n, tt in x.items()}
        o_t, s, c = orc.decode_step(step["q"], step["k"], step["v"], step["log_alpha"],
                                    step["beta"], s, g=step["g"], conv_state=c, **kw)
        outs.append(o_t)
    _close(np.concatenate(outs), o_all, 1e-12, "prefill + decode outputs")
    _close(s, s_all, 1e-12, "prefill + decode state")


def pin_heads_and_sequences_independent(orc):
    """Heads and packed sequences never mix: a batched run equals separate runs;
    the state has the fixed size [N, H, d_k, d_v] whatever the length
    ([Baena]: the state does not grow with sequence length)."""
    r = _rng(12)
    H, d = 3, 8
    lens = [1, 16, 37]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = int(cu[-1])
    x = _layer_inputs(r, T, H, d)
    cw = r.standard_normal((3, H * d, 4)) * 0.5
    S0 = r.standard_normal((3, H, d, d)) * 0.1
    o, s, c = orc.prefill(**x, cu_seqlens=cu, conv_w=cw, state_in=S0, threads=2)
    assert s.shape == (3, H, d, d)
    for n in range(3):
        for h in range(H):
            sl = slice(cu[n], cu[n + 1])
            one = {name: t[sl, h:h + 1] for name, t in x.items()}
            cwh = cw[:, h * d:(h + 1) * d]
            o1, s1, _ = orc.prefill(**one, cu_seqlens=[0, lens[n]], conv_w=cwh,
                                    state_in=S0[n:n + 1, h:h + 1], threads=1)
            assert np.array_equal(o1[:, 0], o[sl, h]), "head/sequence mixing in o"
            assert np.array_equal(s1[0, 0], s[n, h]), "head/sequence mixing in S"


# --------------------------------------------------------------- low-rank gate
# [Atlas] step list: z = z_down W_up, alpha = exp(-5 sigmoid(e^A (z + b_alpha))); [Jawad]
# "Channel-wise decay, and the floor K3 puts under it": g = g_min sigmoid(e^{A_h} z) with
# g_min = -5, so log alpha lies in (-5, 0).


def pin_gate_zero_projection_is_half_floor(orc):
    """z_down = 0 and b = 0: sigmoid(0) = 1/2, so log alpha = -2.5 for every A."""
    rng = _rng(90)
    H, d, r = 3, 4, 5
    la = orc.lowrank_log_alpha(np.zeros((6, r)), rng.standard_normal((H * d, r)), np.zeros(H * d),
                               rng.standard_normal(H))
    _close(la, np.full((6, H, d), -2.5), 1e-15, "log alpha at zero projection")


def pin_gate_floor_and_ceiling(orc):
    """A large positive argument saturates at the floor log alpha = -5, a large negative
    one at log alpha = 0 (no decay)."""
    H, d, r = 2, 3, 4
    z = np.zeros((2, r))
    for b, want in ((1e3, -5.0), (-1e3, 0.0)):
        la = orc.lowrank_log_alpha(z, np.zeros((H * d, r)), np.full(H * d, b), np.zeros(H))
        _close(la, np.full((2, H, d), want), 1e-12, f"saturation at b = {b}")


def pin_gate_sigmoid_symmetry(orc):
    """sigmoid(-u) = 1 - sigmoid(u): negating z_down and b maps log alpha to -5 - log alpha."""
    rng = _rng(91)
    H, d, r = 2, 4, 6
    z, w, b, a = rng.standard_normal((5, r)), rng.standard_normal((H * d, r)), rng.standard_normal(H * d), \
        rng.standard_normal(H) * 0.5
    la = orc.lowrank_log_alpha(z, w, b, a)
    lb = orc.lowrank_log_alpha(-z, w, -b, a)
    _close(la + lb, np.full_like(la, -5.0), 1e-13, "gate symmetry")
    assert np.all(la < 0) and np.all(la > -5)


def pin_gate_one_hot_selects_channel_and_head(orc):
    """One-hot z_down (coordinate j) and a W_up whose only nonzero entry is output channel
    c = h d + i, coordinate j: only that channel moves.  With e^{A_h} w = ln 3 the
    sigmoid is 3/4 and log alpha = -3.75; head 1 has A = ln 2, so the same product
    needs w = ln 3 / 2 there.  Every other channel stays at -2.5."""
    H, d, r = 2, 3, 4
    for h, i, j in ((0, 2, 1), (1, 0, 3)):
        a = np.array([0.0, np.log(2.0)])
        w = np.zeros((H * d, r))
        w[h * d + i, j] = np.log(3.0) / np.exp(a[h])
        z = np.zeros((1, r))
        z[0, j] = 1.0
        la = orc.lowrank_log_alpha(z, w, np.zeros(H * d), a)
        want = np.full((1, H, d), -2.5)
        want[0, h, i] = -3.75
        _close(la, want, 1e-14, f"one-hot channel ({h}, {i}) via coordinate {j}")


def pin_gate_bias_per_channel(orc):
    """b_alpha shifts each output channel separately: with z_down = 0 and A = 0,
    b_c = ln 3 gives log alpha = -3.75 and b_c = -ln 3 gives -1.25 (sigmoid = 1/4)."""
    H, d, r = 2, 2, 3
    b = np.array([np.log(3.0), -np.log(3.0), 0.0, np.log(3.0)])
    la = orc.lowrank_log_alpha(np.zeros((1, r)), np.ones((H * d, r)), b, np.zeros(H))
    _close(la.reshape(-1), np.array([-3.75, -1.25, -2.5, -3.75]), 1e-14, "bias per channel")


# ------------------------------------------------------ Kimi Linear's unbounded gate
# [Jawad] "Channel-wise decay, and the floor K3 puts under it": Kimi Linear's log-decay
# g = -e^A softplus(z) takes any value in (-inf, 0).


def pin_softplus_gate_at_zero_is_ln2(orc):
    """z_down = 0 and b = 0: softplus(0) = ln 2, so log alpha = -e^{A_h} ln 2, per head."""
    rng = _rng(92)
    H, d, r = 3, 4, 5
    a = rng.standard_normal(H)
    la = orc.softplus_log_alpha(np.zeros((2, r)), rng.standard_normal((H * d, r)), np.zeros(H * d), a)
    want = np.broadcast_to((-np.exp(a) * np.log(2.0))[None, :, None], (2, H, d))
    _close(la, want, 1e-15, "log alpha at zero argument")


def pin_softplus_gate_closed_forms(orc):
    """softplus(ln 3) = ln 4 and softplus(-ln 3) = ln(4/3); far out, softplus(u) -> u for
    u = 800 (where e^u overflows fp64) and -> e^u for u = -50; the decay is unbounded:
    e^A = 10 at u = 800 gives log alpha = -8000."""
    H, d, r = 1, 4, 2
    b = np.array([np.log(3.0), -np.log(3.0), 800.0, -50.0])
    for a_h, ea in ((0.0, 1.0), (np.log(10.0), 10.0)):
        la = orc.softplus_log_alpha(np.zeros((1, r)), np.zeros((H * d, r)), b, np.array([a_h]))
        want = -ea * np.array([np.log(4.0), np.log(4.0 / 3.0), 800.0, np.exp(-50.0)])
        _close(la.reshape(-1), want, 1e-14, f"closed forms at e^A = {ea}")


def pin_softplus_gate_reflection(orc):
    """softplus(u) - softplus(-u) = u: negating z_down and b changes log alpha by
    -e^{A_h} (z_down W_up + b), with the projection taken as a numpy matrix product; and
    e^{-softplus(-u)} = sigmoid(u) ties the gate to the logistic function."""
    rng = _rng(93)
    H, d, r = 2, 3, 6
    z, w, b, a = rng.standard_normal((4, r)), rng.standard_normal((H * d, r)), rng.standard_normal(H * d), \
        rng.standard_normal(H) * 0.5
    la = orc.softplus_log_alpha(z, w, b, a)
    lb = orc.softplus_log_alpha(-z, w, -b, a)
    u = (z @ w.T + b).reshape(4, H, d)
    ea = np.exp(a)[None, :, None]
    _close(la - lb, -ea * u, 1e-12, "softplus reflection")
    _close(np.exp(lb / ea), 1.0 / (1.0 + np.exp(-u)), 1e-12, "exp(-softplus(-u)) = sigmoid(u)")
    assert np.all(la < 0)


def pin_softplus_gate_one_hot_channel(orc):
    """One-hot z_down and a single nonzero W_up entry move one output channel only: with
    w = ln 3 there, that channel has softplus(ln 3) = ln 4, every other ln 2 (A = 0)."""
    H, d, r = 2, 3, 4
    for h, i, j in ((1, 1, 0), (0, 2, 3)):
        w = np.zeros((H * d, r))
        w[h * d + i, j] = np.log(3.0)
        z = np.zeros((1, r))
        z[0, j] = 1.0
        la = orc.softplus_log_alpha(z, w, np.zeros(H * d), np.zeros(H))
        want = np.full((1, H, d), -np.log(2.0))
        want[0, h, i] = -np.log(4.0)
        _close(la, want, 1e-14, f"one-hot channel ({h}, {i})")


def pin_beta_logit_closed_forms(orc):
    """beta = sigma(w) ("Kimi K3 - KDA layer" step list): sigma(0) = 1/2, sigma(ln 3) = 3/4,
    sigma(-ln 3) = 1/4 exactly up to rounding; the far tails are 0 and 1 with no overflow."""
    w = np.array([0.0, np.log(3.0), -np.log(3.0), 800.0, -800.0, 40.0])
    b = orc.beta_from_logit(w)
    _close(b[:3], np.array([0.5, 0.75, 0.25]), 1e-15, "sigma closed forms")
    assert b[3] == 1.0 and b[4] == 0.0 and abs(b[5] - 1.0) < 1e-15
    assert np.all(np.isfinite(b))


def pin_beta_logit_symmetry_and_order(orc):
    """sigma(w) + sigma(-w) = 1, sigma is increasing, and e^{-w} sigma(w) = sigma(-w)
    (the odds of sigma(w) are e^w) on random pre-activations of any shape."""
    w = _rng(61).standard_normal((7, 5)) * 4.0
    b, c = orc.beta_from_logit(w), orc.beta_from_logit(-w)
    assert b.shape == w.shape
    _close(b + c, np.ones_like(w), 1e-15, "sigma(w) + sigma(-w)")
    _close(np.exp(-w) * b, c, 1e-14, "odds of sigma")
    s = np.sort(w.ravel())
    assert np.all(np.diff(orc.beta_from_logit(s)) >= 0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]

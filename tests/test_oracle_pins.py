"""Pins of the fp64 oracle against facts fixed by the mathematics (CPU only).

Each test checks the oracle against something other than itself: a closed
form, an invariant, a hand computation, or a brute-force dense product.  The
mistakes each one catches are listed in its docstring.
"""
import numpy as np
import pytest

import oracle
from oracle import mirror
from workloads import make_workload, ckpt_offsets, leveled_segments

TIGHT = 1e-11


def rnd_inputs(seed, T, H, dk, dv, gate_shift=0.0, beta_shift=0.0, N=None):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H, dk)) + gate_shift)
    beta = 1.0 / (1.0 + np.exp(-(rng.standard_normal((T, H)) + beta_shift)))
    return q, k, v, g, beta


def unit_rows(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
def test_hand_computed_two_tokens():
    """Two tokens, dk = dv = 2, worked by hand from the recurrence.

    Token 1: S0 = 0, k = (1,0), v = (2,3), beta = 1/2, g = (0,0)
        S1 = 1/2 k v^T = [[1, 1.5], [0, 0]];  q = (1,0) -> o1 = S1^T q = (1, 1.5)
    Token 2: alpha = (1/2, 1): decayed S = [[0.5, 0.75], [0, 0]]
        k = (0.6, 0.8), r = S^T k = (0.3, 0.45), v = (1, -1), beta = 1
        S2 = S + k (v - r)^T = [[0.92, -0.12], [0.56, -1.16]]
        q = (0, 1) -> o2 = S2^T q = (0.56, -1.16)
    Catches: decay after the erase, o from the pre-update state, S vs S^T,
    beta applied to the erase only.
    """
    q = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    k = np.array([[[1.0, 0.0]], [[0.6, 0.8]]])
    v = np.array([[[2.0, 3.0]], [[1.0, -1.0]]])
    g = np.array([[[0.0, 0.0]], [[np.log(0.5), 0.0]]])
    beta = np.array([[0.5], [1.0]])
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, 2], qk_l2norm=0)
    np.testing.assert_allclose(o[0, 0], [1.0, 1.5], atol=1e-14)
    np.testing.assert_allclose(o[1, 0], [0.56, -1.16], atol=1e-14)
    np.testing.assert_allclose(Sf[0, 0], [[0.92, -0.12], [0.56, -1.16]], atol=1e-14)


def test_beta_zero_is_pure_decay():
    """beta = 0: S_t = Diag(prod alpha) S0 and o_t = S0^T (exp(G_t) * q_t).
    Catches: wrong gate map (g vs exp(g)), decay on the wrong axis, missing S0."""
    T, H, dk, dv = 40, 2, 8, 6
    q, k, v, g, _ = rnd_inputs(1, T, H, dk, dv)
    q = unit_rows(q)
    beta = np.zeros((T, H))
    S0 = np.random.default_rng(2).standard_normal((1, H, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, qk_l2norm=0)
    G = np.cumsum(g, axis=0)                                   # [T,H,dk]
    exp_o = np.einsum("hij,thi->thj", S0[0], np.exp(G) * q)
    np.testing.assert_allclose(o, exp_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sf[0], np.exp(G[-1])[:, :, None] * S0[0], rtol=1e-12, atol=1e-14)


def test_alpha_one_beta_zero_constant_state():
    """alpha = 1, beta = 0: the state never changes; o_t = S0^T q_t."""
    T, H, dk, dv = 17, 1, 5, 7
    q, k, v, _, _ = rnd_inputs(3, T, H, dk, dv)
    S0 = np.random.default_rng(4).standard_normal((1, H, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, np.zeros((T, H, dk)), np.zeros((T, H)), [0, T],
                              S0=S0, qk_l2norm=0)
    np.testing.assert_allclose(Sf[0], S0[0], atol=0)
    np.testing.assert_allclose(o, np.einsum("hij,thi->thj", S0[0], q), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("dk,dv,n", [(8, 8, 8), (16, 5, 11), (6, 12, 6)])
def test_orthonormal_keys_recall_values(dk, dv, n):
    """alpha = 1, beta = 1, orthonormal keys k_1..k_n (n <= dk), any S0:
    S_n^T k_i = v_i for every i, and a query equal to the key just written
    reads back its value.  Catches: S vs S^T, a missing erase, o taken before
    the write."""
    rng = np.random.default_rng(5 + dk + dv)
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    keys = Qm[:n]                                            # orthonormal rows
    k = keys[:, None, :]
    v = rng.standard_normal((n, 1, dv))
    q = k.copy()
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, np.zeros((n, 1, dk)), np.ones((n, 1)), [0, n],
                              S0=S0, qk_l2norm=0)
    np.testing.assert_allclose(Sf[0, 0].T @ keys.T, v[:, 0].T, atol=1e-12)
    np.testing.assert_allclose(o[:, 0], v[:, 0], atol=1e-12)


def test_l2norm_definition():
    """With beta = 0, alpha = 1 and S0 = I the output is the normalised query,
    q / sqrt(|q|^2 + 1e-6): for |q| = 1e-3 that is q / sqrt(2e-6).  Large
    queries are scale-invariant.  Catches: a missing or misplaced eps, the norm
    taken over the wrong axis, the query scale dropped."""
    dk = 4
    u = unit_rows(np.array([[1.0, 2.0, -2.0, 0.5]]))
    q = np.stack([1e-3 * u, 30.0 * u, 1.0 * u])[:, :, :]      # [3,1,dk]
    T = q.shape[0]
    S0 = np.eye(dk)[None, None]
    o, _, _ = oracle.prefill(q, q, q, np.zeros((T, 1, dk)), np.zeros((T, 1)), [0, T],
                             S0=S0, qk_l2norm=1, scale=0.5)
    np.testing.assert_allclose(o[0, 0], 0.5 * 1e-3 / np.sqrt(2e-6) * u[0], rtol=1e-12)
    np.testing.assert_allclose(o[1, 0], 0.5 * u[0], rtol=1e-8)
    np.testing.assert_allclose(o[2, 0], 0.5 * u[0] / np.sqrt(1.0 + 1e-6), rtol=1e-13)


def brute_force(q, k, v, g, beta, S0):
    """Explicit dense products: A_t = (I - b k k^T) Diag(alpha_t), S_t from the
    closed form S_t = (prod_{s<=t} A_s) S0 + sum_{s<=t} (prod_{s<u<=t} A_u) b_s k_s v_s^T."""
    T, dk = k.shape
    A = [(np.eye(dk) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]
    outs, states = [], []
    for t in range(T):
        prod = np.eye(dk)
        for s in range(t + 1):
            prod = A[s] @ prod
        S = prod @ S0
        for s in range(t + 1):
            tail = np.eye(dk)
            for u in range(s + 1, t + 1):
                tail = A[u] @ tail
            S = S + tail @ (beta[s] * np.outer(k[s], v[s]))
        states.append(S)
        outs.append(S.T @ q[t])
    return np.array(outs), states


def test_brute_force_dense_product():
    """The token loop equals the explicit product of the per-token maps.
    Catches: any dropped term, sign, or index in the recurrence."""
    T, dk, dv = 24, 6, 4
    q, k, v, g, beta = rnd_inputs(7, T, 1, dk, dv)
    q, k = unit_rows(q), unit_rows(k)
    S0 = np.random.default_rng(8).standard_normal((1, 1, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, qk_l2norm=0)
    ob, states = brute_force(q[:, 0], k[:, 0], v[:, 0], g[:, 0], beta[:, 0], S0[0, 0])
    np.testing.assert_allclose(o[:, 0], ob, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sf[0, 0], states[-1], rtol=1e-11, atol=1e-12)


def test_package_equals_dense_product():
    """M is the product of the per-token maps, D the zero-start state, and
    o_local the zero-start outputs; S_out = M S_in + D for any S_in."""
    T, dk, dv = 20, 5, 3
    q, k, v, g, beta = rnd_inputs(9, T, 1, dk, dv)
    q, k = unit_rows(q), unit_rows(k)
    a, b = 4, 17
    M, D, ol = oracle.package(q, k, v, g, beta, a, b, qk_l2norm=0)
    Mb = np.eye(dk)
    for t in range(a, b):
        At = (np.eye(dk) - beta[t, 0] * np.outer(k[t, 0], k[t, 0])) @ np.diag(np.exp(g[t, 0]))
        Mb = At @ Mb
    np.testing.assert_allclose(M[0], Mb, rtol=1e-12, atol=1e-14)
    ob, states = brute_force(q[a:b, 0], k[a:b, 0], v[a:b, 0], g[a:b, 0], beta[a:b, 0],
                             np.zeros((dk, dv)))
    np.testing.assert_allclose(D[0], states[-1], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(ol[a:b, 0], ob, rtol=1e-11, atol=1e-13)
    S_in = np.random.default_rng(10).standard_normal((1, 1, dk, dv))
    _, Sf, _ = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, b - a],
                              S0=S_in, qk_l2norm=0)
    np.testing.assert_allclose(Sf[0, 0], M[0] @ S_in[0, 0] + D[0], rtol=1e-11, atol=1e-13)


def test_superposition():
    """The state map is jointly linear in (S0, V): run(S0, V) = run(S0, 0) + run(0, V)."""
    T, H, dk, dv = 50, 2, 8, 8
    q, k, v, g, beta = rnd_inputs(11, T, H, dk, dv)
    S0 = np.random.default_rng(12).standard_normal((1, H, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0)
    o1, S1, _ = oracle.prefill(q, k, np.zeros_like(v), g, beta, [0, T], S0=S0)
    o2, S2, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=None)
    np.testing.assert_allclose(o, o1 + o2, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(Sf, S1 + S2, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("C", [1, 2, 8, 16, 32, 64, 128])
def test_chunk_size_independence(C):
    """The chunkwise fp64 form equals the token loop for every chunk size,
    with a ragged last chunk (T = 150).  C = 1 is the recurrence itself."""
    T, H, dk, dv = 150, 2, 16, 8
    q, k, v, g, beta = rnd_inputs(13, T, H, dk, dv)
    S0 = 0.1 * np.random.default_rng(14).standard_normal((1, H, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0)
    om, Sm = mirror.chunked_prefill(q, k, v, g, beta, [0, T], S0, C)
    assert oracle.rel_l2(om, o) < 1e-12
    assert oracle.rel_l2(Sm, Sf) < 1e-12


def test_composition_over_random_cuts():
    """Packages of random chunk-aligned cuts, composed in order, reproduce the
    sequential state; sequential and Blelloch scans agree; each segment's
    outputs are its zero-start outputs plus the contribution of its incoming
    state.  Long-memory gates keep M far from zero."""
    T, H, dk, dv = 384, 2, 8, 8
    q, k, v, g, beta = rnd_inputs(15, T, H, dk, dv, gate_shift=-6.0, beta_shift=-3.0)
    S0 = np.random.default_rng(16).standard_normal((1, H, dk, dv))
    o, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0)
    rng = np.random.default_rng(17)
    for nseg in (1, 2, 3, 5, 6):
        cuts = np.sort(rng.choice(np.arange(1, T // 64), nseg - 1, replace=False)) * 64
        starts = np.concatenate([[0], cuts, [T]])
        Ms, Ds, oloc = [], [], np.zeros_like(o)
        for j in range(nseg):
            M, D, ol = oracle.package(q, k, v, g, beta, starts[j], starts[j + 1])
            assert np.abs(M).max() > 1e-3          # long memory: M is not negligible
            Ms.append(M)
            Ds.append(D)
            oloc[starts[j]:starts[j + 1]] = ol[starts[j]:starts[j + 1]]
        S_in, S_fin = oracle.scan_sequential(Ms, Ds, S0[0])
        np.testing.assert_allclose(S_fin, Sf[0], rtol=1e-10, atol=1e-12)
        S_in_b, S_fin_b = oracle.scan_blelloch(Ms, Ds, S0[0])
        np.testing.assert_allclose(S_in_b, S_in, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(S_fin_b, S_fin, rtol=1e-11, atol=1e-12)
        # outputs: o = o_local + correction from S_in (linearity in S_in)
        for j in range(nseg):
            a, b = starts[j], starts[j + 1]
            oc, _, _ = oracle.prefill(q[a:b], k[a:b], np.zeros_like(v[a:b]), g[a:b],
                                      beta[a:b], [0, b - a], S0=S_in[j][None])
            np.testing.assert_allclose(oloc[a:b] + oc, o[a:b], rtol=1e-9, atol=1e-11)


def test_resume_from_checkpoint():
    """Checkpoint at p = m * interval, then resume with it as S0: equals the
    continuous run (outputs and final state)."""
    T, H, dk, dv = 320, 2, 8, 8
    q, k, v, g, beta = rnd_inputs(18, T, H, dk, dv, gate_shift=-4.0)
    S0 = np.random.default_rng(19).standard_normal((1, H, dk, dv))
    off = ckpt_offsets([T], 64)
    o, Sf, ck = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, ckpt_interval=64,
                               ckpt_offsets=off)
    assert ck.shape[0] == 5
    np.testing.assert_allclose(ck[4], Sf[0], atol=0)     # rung at the prompt end
    for m in (1, 3):
        p = 64 * m
        o2, Sf2, _ = oracle.prefill(q[p:], k[p:], v[p:], g[p:], beta[p:], [0, T - p],
                                    S0=ck[m - 1][None])
        np.testing.assert_allclose(o2, o[p:], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(Sf2, Sf, rtol=1e-11, atol=1e-12)


def test_state_norm_bound():
    """||S_t||_F <= max_d alpha_{t,d} ||S_{t-1}||_F + beta_t ||v_t||, since
    ||I - b k k^T||_2 <= 1 for unit k and 0 <= b <= 1."""
    T, dk, dv = 64, 8, 8
    q, k, v, g, beta = rnd_inputs(20, T, 1, dk, dv)
    S0 = np.random.default_rng(21).standard_normal((1, 1, dk, dv))
    off = ckpt_offsets([T], 1)
    _, _, ck = oracle.prefill(q, k, v, g, beta, [0, T], S0=S0, ckpt_interval=1,
                              ckpt_offsets=off)
    prev = S0[0, 0]
    for t in range(T):
        lhs = np.linalg.norm(ck[t, 0])
        rhs = np.exp(g[t, 0]).max() * np.linalg.norm(prev) + beta[t, 0] * np.linalg.norm(v[t, 0])
        assert lhs <= rhs * (1 + 1e-12)
        prev = ck[t, 0]


def test_varlen_packing_and_permutation():
    """Packing sequences equals running each alone; permuting the sequences
    permutes outputs and states; checkpoint rows follow the offsets."""
    lens = [70, 1, 128, 200, 64]
    T, H, dk, dv = sum(lens), 2, 8, 4
    q, k, v, g, beta = rnd_inputs(22, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)])
    S0 = np.random.default_rng(23).standard_normal((len(lens), H, dk, dv))
    off = ckpt_offsets(lens, 64)
    o, Sf, ck = oracle.prefill(q, k, v, g, beta, cu, S0=S0, ckpt_interval=64, ckpt_offsets=off)
    for n, L in enumerate(lens):
        a, b = cu[n], cu[n + 1]
        o1, S1, c1 = oracle.prefill(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], [0, L],
                                    S0=S0[n:n + 1], ckpt_interval=64,
                                    ckpt_offsets=ckpt_offsets([L], 64))
        np.testing.assert_allclose(o1, o[a:b], atol=0)
        np.testing.assert_allclose(S1[0], Sf[n], atol=0)
        if L >= 64:
            np.testing.assert_allclose(c1, ck[off[n]:off[n + 1]], atol=0)
    perm = [3, 0, 4, 2, 1]
    idx = np.concatenate([np.arange(cu[p], cu[p + 1]) for p in perm])
    cu2 = np.concatenate([[0], np.cumsum([lens[p] for p in perm])])
    o2, S2, _ = oracle.prefill(q[idx], k[idx], v[idx], g[idx], beta[idx], cu2, S0=S0[perm])
    np.testing.assert_allclose(o2, o[idx], atol=0)
    np.testing.assert_allclose(S2, Sf[perm], atol=0)


def test_empty_sequences_and_zero_length():
    """A zero-length sequence keeps its S0 and writes nothing; T = 0 works."""
    H, dk, dv = 1, 4, 4
    S0 = np.random.default_rng(24).standard_normal((2, H, dk, dv))
    z = np.zeros((0, H, dk))
    o, Sf, _ = oracle.prefill(z, z, np.zeros((0, H, dv)), z, np.zeros((0, H)), [0, 0, 0], S0=S0)
    assert o.shape == (0, H, dv)
    np.testing.assert_allclose(Sf, S0, atol=0)


def test_standard_workload_recipes():
    """The generator reproduces the documented workload shapes: config 3's
    leveled segments and config 4's length draw (sum 447,540; 82 rungs)."""
    b = leveled_segments(131072, 16)
    assert list(np.diff(b))[:3] == [9536, 9344, 9088] and b[-1] == 131072
    from workloads import varlen_lengths
    L = varlen_lengths(46004, 64)
    assert int(L.sum()) == 447540 and int(L.min()) == 513 and int(L.max()) == 29856
    assert int((L // 4096).sum()) == 82
    w = make_workload("t", [100, 28], 2, 8, 8, "bf16", 1)
    assert w.q.dtype == np.uint16 and w.T == 128 and w.S0.shape == (2, 2, 8, 8)


def test_bf16_rounding_matches_torch():
    """The generator's round-to-nearest-even to bf16 agrees bit for bit with
    torch's CPU conversion, ties and NaN included."""
    import torch
    from workloads import bf16_round_bits, bf16_bits_to_f32
    rng = np.random.default_rng(25)
    x = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -0.0, 3e38, 1e-40,
                                  np.inf, -np.inf], dtype=np.float32)])
    ours = bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert np.isnan(bf16_bits_to_f32(bf16_round_bits(np.array([np.nan], np.float32))))[0]


# ---------------------------------------------------------------------------
# Decode against a state pool
# ---------------------------------------------------------------------------
def test_gate_activations_closed_forms():
    """softplus and sigmoid against values and identities fixed by their
    definitions, and against scipy's independent routines.
    Catches: softplus(-x) for softplus(x), a sign flip in sigmoid, overflow at
    large |x|."""
    from scipy.special import expit, log_expit
    assert oracle.softplus(0.0) == pytest.approx(np.log(2.0), abs=1e-16)
    assert oracle.sigmoid(0.0) == 0.5
    x = np.linspace(-60.0, 60.0, 241)
    np.testing.assert_allclose(oracle.softplus(x) - oracle.softplus(-x), x, atol=1e-12)
    np.testing.assert_allclose(oracle.sigmoid(x) + oracle.sigmoid(-x), 1.0, atol=1e-15)
    np.testing.assert_allclose(oracle.sigmoid(x), np.exp(-oracle.softplus(-x)), rtol=1e-13)
    np.testing.assert_allclose(oracle.sigmoid(x), expit(x), rtol=1e-14)
    np.testing.assert_allclose(-oracle.softplus(-x), log_expit(x), rtol=1e-13, atol=1e-300)
    assert oracle.softplus(-40.0) == pytest.approx(np.exp(-40.0), rel=1e-12)
    assert np.isfinite(oracle.softplus(1e4)) and oracle.softplus(1e4) == 1e4


def l2n(x):
    """x / sqrt(|x|^2 + 1e-6), the normalisation the recurrence applies."""
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-6)


def _decode_inputs(seed, N, H, dk, dv, n_slots):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, H, dk))
    k = rng.standard_normal((N, H, dk))
    v = rng.standard_normal((N, H, dv))
    ga = rng.standard_normal((N, H, dk))
    ba = rng.standard_normal((N, H))
    pool = 0.1 * rng.standard_normal((n_slots, H, dk, dv))
    return q, k, v, ga, ba, pool


def test_decode_from_zero_state_closed_form():
    """Read index -1: S = beta k^ v^T and o = beta (k^ . q^) v, whatever the
    decay.  Catches: a missing normalisation, S^T for S, the decay applied
    to the write, a read of slot 0 for a negative index."""
    N, H, dk, dv = 3, 2, 8, 5
    q, k, v, ga, ba, pool = _decode_inputs(7, N, H, dk, dv, 4)
    read = np.array([-1, -1, -1])
    write = np.array([0, 1, -1])
    o, out = oracle.decode(q, k, v, ga, ba, pool, read, write, gate_logits=True)
    beta = 1.0 / (1.0 + np.exp(-ba))
    qn, kn = l2n(q), l2n(k)
    for n in range(N):
        for h in range(H):
            S = beta[n, h] * np.outer(kn[n, h], v[n, h])
            np.testing.assert_allclose(o[n, h], beta[n, h] * (kn[n, h] @ qn[n, h]) * v[n, h],
                                       rtol=1e-12, atol=1e-14)
            if write[n] >= 0:
                np.testing.assert_allclose(out[write[n], h], S, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(out[2:], pool[2:])


def test_decode_pure_decay_and_recall():
    """beta = 0 gives S' = Diag(alpha) S and o = S'^T q^; alpha = 1, beta = 1
    and q = k give o = v (the written key recalls its value).  Catches:
    decay on the value axis, exp(g) vs g, the erase sign."""
    N, H, dk, dv = 2, 2, 6, 4
    q, k, v, ga, _, pool = _decode_inputs(8, N, H, dk, dv, 2)
    g = -oracle.softplus(ga)
    read = np.array([1, 0])
    write = np.array([1, 0])
    o, out = oracle.decode(q, k, v, g, np.zeros((N, H)), pool, read, write)
    for n in range(N):
        for h in range(H):
            S = np.exp(g[n, h])[:, None] * pool[read[n], h]
            np.testing.assert_allclose(out[write[n], h], S, rtol=1e-13)
            np.testing.assert_allclose(o[n, h], S.T @ l2n(q)[n, h], rtol=1e-12, atol=1e-15)
    ku = unit_rows(k)
    o, out = oracle.decode(ku, ku, v, np.zeros((N, H, dk)), np.ones((N, H)), pool, read, write,
                           qk_l2norm=0)
    np.testing.assert_allclose(o, v, rtol=1e-12, atol=1e-12)


def test_decode_slot_semantics():
    """Forks leave the read slot as it was, in-place rows replace it, rows
    with a negative write index keep nothing, untouched slots are copied
    through, and the logits path equals the activated gates computed with
    scipy.  Catches: writes into the read slot of a fork, a write for index
    -1, gates activated twice or not at all."""
    from scipy.special import expit, log_expit
    N, H, dk, dv = 4, 1, 4, 3
    q, k, v, ga, ba, pool = _decode_inputs(9, N, H, dk, dv, 8)
    read = np.array([2, 5, 0, 3])
    write = np.array([2, 6, -1, 7])
    o, out = oracle.decode(q, k, v, ga, ba, pool, read, write, gate_logits=True)
    o2, out2 = oracle.decode(q, k, v, log_expit(-ga), expit(ba), pool, read, write)
    np.testing.assert_allclose(o, o2, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out, out2, rtol=1e-13, atol=1e-15)
    for s in (0, 1, 3, 4, 5):
        np.testing.assert_array_equal(out[s], pool[s])
    assert not np.allclose(out[2], pool[2])
    # the forked and in-place states are one-token updates of their read slots
    for n, (r, w) in enumerate(zip(read, write)):
        if w < 0:
            continue
        o1, S1, _ = oracle.prefill(q[n:n + 1], k[n:n + 1], v[n:n + 1], log_expit(-ga[n:n + 1]),
                                   expit(ba[n:n + 1]), [0, 1], S0=pool[r][None])
        np.testing.assert_allclose(out[w], S1[0], rtol=1e-13, atol=1e-15)


def test_decode_chain_equals_prefill():
    """T decode steps in place on one slot equal a T-token prefill from that
    slot's state: the pool plumbing adds nothing to the recurrence."""
    T, H, dk, dv = 12, 2, 8, 8
    q, k, v, g, beta = rnd_inputs(10, T, H, dk, dv)
    pool = 0.1 * np.random.default_rng(11).standard_normal((3, H, dk, dv))
    o_ref, Sf, _ = oracle.prefill(q, k, v, g, beta, [0, T], S0=pool[1][None])
    cur = pool.copy()
    outs = []
    for t in range(T):
        o, cur = oracle.decode(q[t:t + 1], k[t:t + 1], v[t:t + 1], g[t:t + 1], beta[t:t + 1],
                               cur, [1], [1])
        outs.append(o[0])
    np.testing.assert_allclose(np.stack(outs), o_ref, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(cur[1], Sf[0], rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cur[0], pool[0])


def test_prefill_resume_matches_continuous_run():
    """Two sequences resumed from pool slots holding the continuous run's
    states at P1 = 128 (a rung) and P2 = 192 (on the chunk grid, between
    rungs) reproduce the continuous run's outputs, its later rungs (at their
    absolute positions) and its final states; the pool's other slots are
    untouched.  The reference is the oracle's own rung logic on the whole
    sequence, independent of the piecewise resume.  Catches: rungs counted
    from the resume point instead of the sequence start, a rung missed at the
    resumed prompt end, the initial state read from the wrong slot."""
    T, H, dk, dv, iv = 448, 2, 8, 8, 128
    q, k, v, g, beta = rnd_inputs(31, 2 * T, H, dk, dv, gate_shift=-3.0)
    S0 = np.random.default_rng(32).standard_normal((2, H, dk, dv))
    cu = [0, T, 2 * T]
    o, Sf, ck = oracle.prefill(q, k, v, g, beta, cu, S0=S0, ckpt_interval=iv,
                               ckpt_offsets=ckpt_offsets([T, T], iv))
    # states at 128 (sequence 0) and 192 (sequence 1)
    _, S128, _ = oracle.prefill(q[:128], k[:128], v[:128], g[:128], beta[:128], [0, 128], S0=S0[:1])
    _, S192, _ = oracle.prefill(q[T:T + 192], k[T:T + 192], v[T:T + 192], g[T:T + 192],
                                beta[T:T + 192], [0, 192], S0=S0[1:])
    np.testing.assert_allclose(S128[0], ck[0], rtol=1e-12, atol=1e-14)
    pool = np.zeros((5, H, dk, dv))
    pool[3], pool[1], pool[4] = S128[0], S192[0], 7.0
    sel = np.r_[128:T, T + 192:2 * T]
    cu2 = [0, T - 128, T - 128 + T - 192]
    o2, out, ck2 = oracle.prefill_resume(q[sel], k[sel], v[sel], g[sel], beta[sel], cu2, pool,
                                         [3, 1], [0, 2], pos0=[128, 192], ckpt_interval=iv)
    np.testing.assert_allclose(o2[:T - 128], o[128:T], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(o2[T - 128:], o[T + 192:], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out[0], Sf[0], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(out[2], Sf[1], rtol=1e-10, atol=1e-12)
    np.testing.assert_array_equal(out[[1, 3, 4]], pool[[1, 3, 4]])
    # rungs of sequence 0 at 256, 384; of sequence 1 at 256, 384 (rows 1, 2 of each)
    assert ck2.shape[0] == 4
    np.testing.assert_allclose(ck2[0:2], ck[1:3], rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(ck2[2:4], ck[4:6], rtol=1e-10, atol=1e-12)
    assert list(ckpt_offsets([T - 128, T - 192], iv, pos0=[128, 192])) == [0, 2, 4]


# ---------------------------------------------------------------------------
# Short causal convolution
# ---------------------------------------------------------------------------
def test_short_conv_identity_and_shift_taps():
    """A tap on the current token is the identity; a tap on the oldest row
    delays by W-1 rows, reading the window first.  Catches: reversed taps,
    an off-by-one in the window, windows not stored or stored from x alone."""
    rng = np.random.default_rng(41)
    T, C, W = 10, 8, 4
    x = rng.standard_normal((T, C))
    win = rng.standard_normal((3, W - 1, C))
    cu = [0, 2, 10]
    ident = np.zeros((C, W)); ident[:, -1] = 1.0
    y, new = oracle.short_conv(x, cu, ident, windows=win, read_idx=[1, -1], write_idx=[0, 2])
    np.testing.assert_array_equal(y, x)
    # sequence 0 has 2 rows: its new window is (oldest kept window row, its rows)
    np.testing.assert_array_equal(new[0], np.concatenate([win[1][-1:], x[0:2]]))
    np.testing.assert_array_equal(new[2], x[7:10])
    np.testing.assert_array_equal(new[1], win[1])
    shift = np.zeros((C, W)); shift[:, 0] = 1.0
    y, _ = oracle.short_conv(x, cu, shift, windows=win, read_idx=[1, -1])
    np.testing.assert_array_equal(y[0:2], win[1][0:2])
    np.testing.assert_array_equal(y[2:5], 0.0)
    np.testing.assert_array_equal(y[5:10], x[2:7])


def test_short_conv_against_numpy_convolve():
    """Each channel equals numpy's own 1-D convolution (kernel reversed,
    'valid' over window + rows), plus bias, then SiLU = z * expit(z) from
    scipy.  Catches: taps applied to the wrong rows, bias after the
    activation, a wrong activation."""
    from scipy.special import expit
    rng = np.random.default_rng(42)
    T, C, W = 37, 16, 5
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    bias = rng.standard_normal(C)
    win = rng.standard_normal((1, W - 1, C))
    y, _ = oracle.short_conv(x, [0, T], w, bias, windows=win, read_idx=[0], activation=1)
    xx = np.concatenate([win[0], x])
    for c in range(C):
        z = np.convolve(xx[:, c], w[c, ::-1], mode="valid") + bias[c]
        np.testing.assert_allclose(y[:, c], z * expit(z), rtol=1e-12, atol=1e-14)
    assert oracle.silu(0.0) == 0.0


def test_short_conv_window_chaining_and_halo():
    """Convolving a sequence in two calls, the first call's window feeding
    the second, equals one call; per-segment convolution with halo windows
    equals the whole-sequence convolution.  Catches: windows holding outputs
    instead of inputs, halo rows taken from the segment start."""
    rng = np.random.default_rng(43)
    T, C, W = 50, 8, 4
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, W))
    y_all, _ = oracle.short_conv(x, [0, T], w)
    win = np.zeros((2, W - 1, C))
    y1, win = oracle.short_conv(x[:21], [0, 21], w, windows=win, read_idx=[-1], write_idx=[1])
    y2, _ = oracle.short_conv(x[21:], [0, T - 21], w, windows=win, read_idx=[1])
    np.testing.assert_allclose(np.concatenate([y1, y2]), y_all, rtol=1e-13, atol=1e-14)
    bounds = [0, 16, 30, 50]
    halo = oracle.conv_halo(x, bounds, W, np.zeros((4, W - 1, C)), [1, 2, 3])
    np.testing.assert_array_equal(halo[1], x[13:16])
    y_seg, _ = oracle.short_conv(x, bounds, w, windows=halo, read_idx=[0, 1, 2])
    np.testing.assert_allclose(y_seg, y_all, rtol=1e-13, atol=1e-14)

"""Pins for the CPU oracle, against facts that do not come from the oracle.

The pages print no worked example for decode attention, so the oracle is
pinned by closed forms, a library special case, invariances that the
mathematics fixes, and brute force at 50 digits.  Each check runs on both
oracle implementations (the C one and the numpy twin).
"""
import math

import numpy as np
import pytest

import oracle
from oracle import ref_np
from decode_attention_prefix_amd import workloads as wl


def both(w):
    t = w.tree
    a = oracle.decode(t, w.q, w.k_pool, w.v_pool)
    b = ref_np.decode_np(t, w.q, w.k_pool, w.v_pool)
    return a, b


def f64(bits):
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def test_one_token_returns_v():
    rng = np.random.default_rng(1)
    w = wl.make_workload([1], [-1], [[0]], 4, 2, 16, rng)
    for out in both(w):
        ref = np.repeat(f64(w.v_tokens[0]), 2, axis=0)   # head h reads KV head h // 2
        assert np.max(np.abs(out[0] - ref)) <= 1e-15


def test_two_tokens_logistic():
    # q = a e_0, k_1 = e_0, k_2 = 0  ->  out = s(a sigma) v_1 + (1 - s(a sigma)) v_2
    D, a = 16, 3.5
    q = np.zeros((1, 1, D), np.float32); q[0, 0, 0] = a
    k = np.zeros((2, 1, D), np.float32); k[0, 0, 0] = 1.0
    v = np.random.default_rng(2).standard_normal((2, 1, D)).astype(np.float32)
    w = wl.make_workload([2], [-1], [[0]], 1, 1, D, np.random.default_rng(3),
                         q_values=q, k_values=k, v_values=v)
    sig = 1.0 / math.sqrt(D)
    s = 1.0 / (1.0 + math.exp(-a * sig))
    vv = f64(w.v_tokens)[:, 0, :]
    ref = s * vv[0] + (1 - s) * vv[1]
    for out in both(w):
        assert np.max(np.abs(out[0, 0] - ref)) <= 1e-14


@pytest.mark.parametrize("mode", ["equal_keys", "zero_query"])
def test_uniform_weights_give_mean(mode):
    rng = np.random.default_rng(4)
    Hq, Hkv, D = 4, 2, 32
    nt, par, paths = [37, 21, 5], [-1, 0, 1], [[0, 1, 2], [0, 1]]
    T = sum(nt)
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    q = rng.standard_normal((2, Hq, D)).astype(np.float32)
    if mode == "equal_keys":
        k[:] = k[0]
    else:
        q[:] = 0
    w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng, q_values=q, k_values=k)
    V = f64(w.v_tokens)
    for out in both(w):
        for r, L in enumerate([63, 58]):
            mean = V[:L].mean(axis=0)                    # [Hkv][D]
            ref = np.repeat(mean, Hq // Hkv, axis=0)
            assert np.max(np.abs(out[r] - ref)) <= 1e-14


@pytest.mark.parametrize("Hq,Hkv,D", [(8, 2, 64), (4, 4, 32), (16, 2, 128)])
def test_unshared_matches_torch_sdpa(Hq, Hkv, D):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(5)
    lens = [1, 15, 16, 17, 40]
    w = wl.make_workload(lens, [-1] * 5, [[i] for i in range(5)], Hq, Hkv, D, rng)
    outs = both(w)
    for r, L in enumerate(lens):
        o0 = int(w.token_offsets[r])
        K = torch.from_numpy(f64(w.k_tokens[o0:o0 + L])).permute(1, 0, 2)[None]   # [1][Hkv][T][D]
        V = torch.from_numpy(f64(w.v_tokens[o0:o0 + L])).permute(1, 0, 2)[None]
        Q = torch.from_numpy(f64(w.q[r]))[None, :, None, :]                     # [1][Hq][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, scale=1.0 / math.sqrt(D), enable_gqa=True)[0, :, 0, :].numpy()
        for out in outs:
            assert np.max(np.abs(out[r] - ref)) <= 1e-12


def _tree_case(seed):
    rng = np.random.default_rng(seed)
    nt, par, paths = wl.make_random_tree(rng, num_requests=6, max_depth=4, max_len=45,
                                         num_q_heads=8, num_kv_heads=2, head_dim=32,
                                         internal_end_prob=0.3)
    return nt, par, paths


@pytest.mark.parametrize("seed", [10, 11, 12])
def test_split_node_invariance(seed):
    nt, par, paths = _tree_case(seed)
    rng = np.random.default_rng(seed + 100)
    w = wl.make_workload(nt, par, paths, 8, 2, 32, rng)
    base = both(w)
    # split the longest node n at a non-page-aligned boundary: n -> (n', n'')
    n = int(np.argmax(nt))
    cut = max(1, min(nt[n] - 1, 7))
    N = len(nt)
    nt2 = list(nt) + [nt[n] - cut]
    nt2[n] = cut
    par2 = list(par) + [n]
    for i in range(N):
        if par2[i] == n:
            par2[i] = N               # children of n hang below n''
    # token order: node order with the tail of n appended at the end
    kt, vt = w.k_tokens, w.v_tokens
    o = w.token_offsets
    idx = np.concatenate([np.arange(o[i], o[i + 1]) if i != n else np.arange(o[n], o[n] + cut)
                          for i in range(N)] + [np.arange(o[n] + cut, o[n + 1])])
    paths2 = [[x for y in p for x in ([y, N] if y == n else [y])] for p in paths]
    # parent[i] < i must hold: node N is last, its children have smaller ids, so
    # renumber by building a topological order
    order = _topo(par2)
    remap = {old: new for new, old in enumerate(order)}
    nt3 = [nt2[o_] for o_ in order]
    par3 = [(-1 if par2[o_] < 0 else remap[par2[o_]]) for o_ in order]
    paths3 = [[remap[x] for x in p] for p in paths2]
    off = 0
    node_tok = []
    for i in range(N + 1):
        L = nt2[i]
        node_tok.append(idx[off:off + L]); off += L
    idx3 = np.concatenate([node_tok[o_] for o_ in order])
    w2 = wl.make_workload(nt3, par3, paths3, 8, 2, 32, np.random.default_rng(seed + 200),
                          q_values=wl.bf16_bits_to_f32(w.q),
                          k_values=wl.bf16_bits_to_f32(kt[idx3]),
                          v_values=wl.bf16_bits_to_f32(vt[idx3]))
    for a, b in zip(base, both(w2)):
        assert np.max(np.abs(a - b)) <= 1e-12


def _topo(par):
    order, seen = [], set()
    def visit(i):
        if i in seen:
            return
        if par[i] >= 0:
            visit(par[i])
        seen.add(i); order.append(i)
    for i in range(len(par)):
        visit(i)
    return order


@pytest.mark.parametrize("seed", [20, 21])
def test_flatten_control_invariance(seed):
    nt, par, paths = _tree_case(seed)
    w = wl.make_workload(nt, par, paths, 8, 2, 32, np.random.default_rng(seed))
    c = wl.control_workload(w)
    for a, b in zip(both(w), both(c)):
        assert np.max(np.abs(a - b)) <= 1e-12


def test_permutations_and_duplicates():
    rng = np.random.default_rng(30)
    Hq, Hkv, D = 8, 2, 32
    L = 50
    w = wl.make_workload([L], [-1], [[0], [0]], Hq, Hkv, D, rng)
    base = both(w)
    perm = rng.permutation(L)
    # shuffled token order, same query: same output
    w2 = wl.make_workload([L], [-1], [[0], [0]], Hq, Hkv, D, rng,
                          q_values=wl.bf16_bits_to_f32(w.q),
                          k_values=wl.bf16_bits_to_f32(w.k_tokens[perm]),
                          v_values=wl.bf16_bits_to_f32(w.v_tokens[perm]))
    # request order swapped: outputs swap
    w3 = wl.make_workload([L], [-1], [[0], [0]], Hq, Hkv, D, rng,
                          q_values=wl.bf16_bits_to_f32(w.q[::-1].copy()),
                          k_values=wl.bf16_bits_to_f32(w.k_tokens),
                          v_values=wl.bf16_bits_to_f32(w.v_tokens))
    # a request duplicated three times: identical rows
    w4 = wl.make_workload([L], [-1], [[0]] * 3, Hq, Hkv, D, rng,
                          q_values=np.repeat(wl.bf16_bits_to_f32(w.q[:1]), 3, axis=0),
                          k_values=wl.bf16_bits_to_f32(w.k_tokens),
                          v_values=wl.bf16_bits_to_f32(w.v_tokens))
    for a, b, c, d in zip(base, both(w2), both(w3), both(w4)):
        assert np.max(np.abs(a - b)) <= 1e-12
        assert np.max(np.abs(a[::-1] - c)) <= 1e-12
        assert np.max(np.abs(d - a[0])) <= 1e-12


@pytest.mark.parametrize("seed", [40, 41, 42])
def test_merge_identity(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, D, T = 8, 2, 16, 70
    q = rng.standard_normal((Hq, D)) * 2
    K = rng.standard_normal((T, Hkv, D))
    V = rng.standard_normal((T, Hkv, D))
    direct = ref_np.attend(q, K, V, 0.25)
    cuts = np.sort(rng.choice(np.arange(1, T), size=5, replace=False))
    bounds = [0, *cuts.tolist(), T]
    parts = [ref_np.partial_stats(q, K[a:b], V[a:b], 0.25) for a, b in zip(bounds[:-1], bounds[1:])]
    parts.append(ref_np.partial_stats(q, K[:0], V[:0], 0.25))      # an empty piece
    rng.shuffle(parts)
    assert np.max(np.abs(ref_np.merge_stats(parts) - direct)) <= 1e-12


def test_brute_force_mpmath():
    mp = pytest.importorskip("mpmath")
    mp.mp.dps = 50
    rng = np.random.default_rng(50)
    Hq, Hkv, D = 4, 2, 8
    nt, par, paths = [11, 9, 13, 4], [-1, 0, 0, 2], [[0, 1], [0, 2, 3], [0, 2]]
    w = wl.make_workload(nt, par, paths, Hq, Hkv, D, rng)
    # stretch the logits so that the softmax is far from uniform
    w.q = wl.f32_to_bf16_bits(wl.bf16_bits_to_f32(w.q) * 3)
    outs = both(w)
    K, V, Q = f64(w.k_tokens), f64(w.v_tokens), f64(w.q)
    o = w.token_offsets
    sig = mp.mpf(1) / mp.sqrt(D)
    for r, p in enumerate(paths):
        idx = np.concatenate([np.arange(o[n], o[n + 1]) for n in p])
        for h in range(Hq):
            g = h // (Hq // Hkv)
            s = [sig * mp.fsum(mp.mpf(Q[r, h, d]) * mp.mpf(K[t, g, d]) for d in range(D)) for t in idx]
            mx = max(s)
            e = [mp.exp(x - mx) for x in s]
            den = mp.fsum(e)
            for d in range(D):
                ref = mp.fsum(e[i] * mp.mpf(V[t, g, d]) for i, t in enumerate(idx)) / den
                for out in outs:
                    assert abs(float(out[r, h, d] - ref)) <= 1e-13


@pytest.mark.parametrize("cfg", [0, 1])
def test_two_oracles_agree_on_configs(cfg):
    w = wl.make_config(cfg)
    a, b = both(w)
    assert np.all(np.isfinite(a))
    assert np.max(np.abs(a - b)) <= 1e-12


def test_two_oracles_agree_random_trees():
    for seed in range(60, 66):
        rng = np.random.default_rng(seed)
        nt, par, paths = wl.make_random_tree(rng, num_requests=7, max_depth=4, max_len=100,
                                             num_q_heads=16, num_kv_heads=2, head_dim=64,
                                             internal_end_prob=0.3, empty_root=bool(seed % 2))
        w = wl.make_workload(nt, par, paths, 16, 2, 64, rng)
        a, b = both(w)
        assert np.max(np.abs(a - b)) <= 1e-12


def test_oracle_rejects_bad_inputs():
    rng = np.random.default_rng(70)
    w = wl.make_workload([5], [-1], [[0]], 6, 4, 16, rng)      # Hq % Hkv != 0
    with pytest.raises(ValueError):
        oracle.decode(w.tree, w.q, w.k_pool, w.v_pool)

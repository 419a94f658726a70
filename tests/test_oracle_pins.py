"""Pins of the fp64 oracle against things other than itself: closed forms,
textbook routines, invariants, the pages' stated counts, and the scalar loop
restatement in oracle.brute."""
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, csa as C, pipeline as P
import synth

FACTS = os.path.join(os.path.dirname(__file__), "golden", "pages_facts.txt")


def _facts():
    out = {}
    with open(FACTS) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            k, v = line.split()
            out[k] = float(v)
    return out


# ------------------------------------------------------------------ pooling


def test_entry_counts_match_pages():
    f = _facts()
    first, end = C.entry_range(0, 1 << 20, 128, overlap=False)
    assert end - first == f["hca_entries_1m"]
    first, end = C.entry_range(0, 1 << 20, 4, overlap=True)
    assert end - first == f["csa_entries_1m"]
    assert math.lcm(4, 128) == f["kv_block_tokens"]
    # a chunk that starts mid-stream with overlap needs the previous block as b rows
    assert C.entry_range(8, 10, 4, True) == (3, 4)
    assert C.entry_range(8, 3, 4, True) == (3, 3)


def test_kv_bytes_reproduce_two_percent():
    """576 B main entry (448 FP8 + 64 BF16) + 68 B MXFP4 indexer key give 161 B per
    token for a CSA layer and 4.5 B for an HCA layer; their mean against a BF16
    GQA-8 cache with head dim 128 (8 heads x (K+V) x 128 x 2 B) is the pages' ~2%."""
    csa = (448 + 64 * 2) / 4 + (64 + 4) / 4
    hca = (448 + 64 * 2) / 128
    frac = (csa + hca) / 2 / (8 * 2 * 128 * 2)
    assert abs(frac - _facts()["kv_fraction_vs_gqa8"]) < 0.001


def _rand(rng, *shape):
    return rng.normal(size=shape)


def test_uniform_logits_give_mean_pooling():
    rng = np.random.default_rng(0)
    m, D, T = 4, 6, 20
    ca, cb = _rand(rng, T, D), _rand(rng, T, D)
    z = np.full((T, D), 0.7)
    first, e, _ = C.pool(ca, z, np.zeros((m, D)), m, 0, cb, z, np.zeros((m, D)))
    assert first == 0
    assert np.allclose(e[0], ca[0:4].mean(0), atol=1e-15)
    for i in range(1, T // m):
        want = (ca[m * i:m * i + m].sum(0) + cb[m * (i - 1):m * i].sum(0)) / (2 * m)
        assert np.allclose(e[i], want, atol=1e-14)


def test_dominant_logit_copies_token():
    rng = np.random.default_rng(1)
    m, D, T = 4, 5, 16
    ca, cb = _rand(rng, T, D), _rand(rng, T, D)
    za, zb = np.zeros((T, D)), np.zeros((T, D))
    zb[5, :] = 1e3            # b-branch token 5 feeds entry 2 (block 1 = rows 4..7)
    za[13, 2] = 1e3           # a-branch token 13, channel 2 only, feeds entry 3
    _, e, _ = C.pool(ca, za, None, m, 0, cb, zb, None)
    assert np.allclose(e[2], cb[5])
    assert np.isclose(e[3, 2], ca[13, 2])


def test_bias_indexes_offset_in_window():
    """B^a_{j-mi}: a bias on offset r lifts token mi+r of every entry."""
    rng = np.random.default_rng(2)
    m, D, T = 4, 3, 16
    ca = _rand(rng, T, D)
    ba = np.zeros((m, D))
    ba[3] = 1e3
    _, e, _ = C.pool(ca, None, ba, m, 0)
    for i in range(T // m):
        assert np.allclose(e[i], ca[m * i + 3])


def test_m1_is_identity_and_weights_sum_to_one():
    rng = np.random.default_rng(3)
    x = _rand(rng, 9, 7)
    _, e, w = C.pool(x, _rand(rng, 9, 7), None, 1, 0)
    assert np.array_equal(e, x)
    _, _, w = C.pool(x[:8], _rand(rng, 8, 7), _rand(rng, 4, 7), 4, 0, x[:8], _rand(rng, 8, 7),
                     _rand(rng, 4, 7))
    assert w[0].shape[0] == 4 and w[1].shape[0] == 8      # entry 0 has no b candidates
    for s in w:
        assert np.allclose(s.sum(axis=0), 1.0, atol=1e-15) and np.all(s > 0)


def test_pool_matches_brute_with_offset():
    rng = np.random.default_rng(4)
    m, D = 4, 5
    pos0, rows = 8, 14       # rows 0..13 = positions 8..21 -> entries 3 and 4
    ca, za, cb, zb = (_rand(rng, rows, D) for _ in range(4))
    ba, bb = _rand(rng, m, D) * 0.1, _rand(rng, m, D) * 0.1
    first, e, _ = C.pool(ca, za, ba, m, pos0, cb, zb, bb)
    assert first == 3 and e.shape[0] == 2
    for k, i in enumerate(range(3, 5)):
        ra, rb = m * i - pos0, m * (i - 1) - pos0
        want = brute.pool_entry(i, m, ca[ra:ra + m].tolist(), za[ra:ra + m].tolist(), ba.tolist(),
                                cb[rb:rb + m].tolist(), zb[rb:rb + m].tolist(), bb.tolist())
        assert np.allclose(e[k], want, rtol=0, atol=1e-13)


# ------------------------------------------------------------------ norm / rope


def test_rmsnorm_closed_form():
    rng = np.random.default_rng(5)
    x = _rand(rng, 10, 512) * 3
    y = C.rmsnorm(x)
    ms = (x * x).mean(1)
    assert np.allclose((y * y).mean(1), ms / (ms + C.RMS_EPS), rtol=1e-14)


def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(6)
    x = _rand(rng, 64)
    for pos in (0, 1, 12345, (1 << 20) + 7, -999):
        got = C.rope(x, pos, 160000.0, 16)
        want = brute.rotate(x.tolist(), pos, 160000.0, 16)
        assert np.allclose(got, want, rtol=0, atol=1e-12)
        assert np.array_equal(got[:48], x[:48])


def test_rope_relative_position_and_inverse():
    rng = np.random.default_rng(7)
    q, k = _rand(rng, 512), _rand(rng, 512)
    a, b, shift = 1_000_003, 999_000, 4096
    s1 = C.rope(q, a, 160000.0, 64) @ C.rope(k, b, 160000.0, 64)
    s2 = C.rope(q, a + shift, 160000.0, 64) @ C.rope(k, b + shift, 160000.0, 64)
    assert abs(s1 - s2) < 1e-9
    back = C.rope(C.rope(q, a, 160000.0, 64), -a, 160000.0, 64)
    assert np.allclose(back, q, atol=1e-12)


# ------------------------------------------------------------------ indexer / top-k


def test_index_scores_match_brute_and_relu():
    rng = np.random.default_rng(8)
    q, w, keys = _rand(rng, 4, 32), np.abs(_rand(rng, 4)), _rand(rng, 50, 32)
    sc = C.index_scores(q, w, keys, 40)
    assert sc.shape == (40,)
    for i in range(40):
        assert abs(sc[i] - brute.index_score(q.tolist(), w.tolist(), keys[i].tolist())) < 1e-12
    # a head whose dot is negative contributes nothing
    sc_neg = C.index_scores(-np.abs(q), w, np.abs(keys), 40)
    assert np.all(sc_neg == 0)


def test_topk_ties_and_padding():
    s = np.array([1.0, 3.0, 3.0, 0.5, 3.0, 2.0])
    assert C.topk(s, 2).tolist() == [1, 2]            # three-way tie at 3: lower indices
    assert C.topk(s, 4).tolist() == [1, 2, 4, 5]
    assert C.topk(s, 8).tolist() == [0, 1, 2, 3, 4, 5, -1, -1]
    rng = np.random.default_rng(9)
    r = np.round(rng.normal(size=60), 1)
    assert C.topk(r, 17).tolist() == brute.select(r.tolist(), 17)


def test_visibility_excludes_own_block():
    assert C.visible_entries(2048, 4, 512) == 512
    assert C.visible_entries(2047, 4, 512) == 511
    assert C.visible_entries(3, 4, 512) == 0
    assert C.visible_entries(4096, 4, 100) == 100


# ------------------------------------------------------------------ attention


def test_attend_matches_brute():
    rng = np.random.default_rng(10)
    H, d, N = 3, 16, 9
    q, kv, sink = _rand(rng, H, d), _rand(rng, N, d), _rand(rng, H)
    o, lse = C.attend_core(q, 77, kv, sink, 160000.0, 4)
    ob, lb = brute.attend(q.tolist(), 77, kv.tolist(), sink.tolist(), 160000.0, 4, 1 / 4)
    assert np.allclose(o, ob, atol=1e-13) and np.allclose(lse, lb, atol=1e-13)


def test_sink_to_minus_infinity_is_textbook_attention():
    """With z_h -> -inf the sink vanishes: the result is softmax attention, which
    torch's scaled_dot_product_attention computes in fp64 on the CPU."""
    rng = np.random.default_rng(11)
    H, d, N = 4, 32, 23
    q, kv = _rand(rng, H, d), _rand(rng, N, d)
    o, _ = C.attend_core(q, 5, kv, np.full(H, -1e300), 160000.0, 0, norm_q=False)
    qt = torch.from_numpy(q)[None, :, None, :]
    kt = torch.from_numpy(kv)[None, None].expand(1, H, N, d)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, scale=1 / math.sqrt(d))
    assert np.allclose(o, ref[0, :, 0].numpy(), atol=1e-13)


def test_sink_mass_below_one():
    rng = np.random.default_rng(12)
    H, d, N = 6, 32, 40
    q, kv, sink = _rand(rng, H, d), _rand(rng, N, d), _rand(rng, H) * 3
    o, lse = C.attend_core(q, 0, kv, sink, 160000.0, 0, norm_q=False)
    o0, _ = C.attend_core(q, 0, kv, np.full(H, -1e300), 160000.0, 0, norm_q=False)
    mass = np.exp(lse) / (np.exp(lse) + np.exp(sink))
    assert np.all((mass > 0) & (mass < 1))
    assert np.allclose(o, o0 * mass[:, None], atol=1e-13)


def test_topk_covering_all_equals_dense():
    """k >= #visible: CSA over the selection equals dense attention over every
    visible entry plus the window."""
    rng = np.random.default_rng(13)
    H, d, m, n_e = 4, 64, 4, 30
    ent, win, q, sink = _rand(rng, n_e, d), _rand(rng, 16, d), _rand(rng, H, d), _rand(rng, H)
    t = 4 * 25 + 2
    sel = C.topk(rng.normal(size=C.visible_entries(t, m, n_e)), 64)
    a = C.csa_attend(q, t, ent, sel, win, t - 15, 16, sink, 160000.0, 16, m)
    b = C.hca_attend(q, t, ent, win, t - 15, 16, sink, 160000.0, 16, m)
    assert np.allclose(a[0], b[0], atol=1e-14) and np.allclose(a[1], b[1], atol=1e-14)


def test_window_rows():
    assert C.window_rows(200, 128, 0, 300).tolist() == list(range(73, 201))
    assert C.window_rows(5, 128, 0, 300).tolist() == list(range(0, 6))
    assert C.window_rows(200, 128, 150, 40).tolist() == list(range(0, 40))


# ------------------------------------------------------------------ whole tiny pipeline


def _brute_tiny(shape, inp):
    """Scalar loops over the whole tiny workload, written against oracle.brute only."""
    g = {k: v.numpy().astype(float) for k, v in inp["main"].items()}
    m, d_r, th = shape.m, shape.d_r, shape.theta
    T = shape.L
    ents = []
    for i in range(T // m):
        rb = (g["cb"][0][m * (i - 1):m * i].tolist(), g["zb"][0][m * (i - 1):m * i].tolist(),
              g["bb"].tolist()) if shape.overlap and i >= 1 else (None, None, None)
        e = brute.pool_entry(i, m, g["ca"][0][m * i:m * i + m].tolist(),
                             g["za"][0][m * i:m * i + m].tolist(), g["ba"].tolist(), *rb)
        ents.append(brute.rotate(brute.rms(e), m * i, th, d_r))
    t = int(inp["q_pos"][0, 0])
    raw = inp["win_raw"][0].numpy().astype(float)
    win = [brute.rotate(brute.rms(raw[j].tolist()), j, th, d_r)
           for j in range(max(0, t - shape.n_win + 1), t + 1)]
    if shape.csa:
        ix = {k: v.numpy().astype(float) for k, v in inp["idx"].items()}
        keys = []
        for i in range(t // m):
            rb = (ix["cb"][0][m * (i - 1):m * i].tolist(), ix["zb"][0][m * (i - 1):m * i].tolist(),
                  ix["bb"].tolist()) if i >= 1 else (None, None, None)
            keys.append(brute.pool_entry(i, m, ix["ca"][0][m * i:m * i + m].tolist(),
                                         ix["za"][0][m * i:m * i + m].tolist(), ix["ba"].tolist(), *rb))
        qI = inp["q_idx"][0, 0].numpy().astype(float).tolist()
        w = inp["w"][0, 0].numpy().astype(float).tolist()
        sc = [brute.index_score(qI, w, k) for k in keys]
        sel = brute.select(sc, shape.top_k)
        rows = [ents[i] for i in sel if i >= 0] + win
    else:
        sc, sel = None, None
        rows = ents[:t // m] + win
    q = inp["q"][0, 0].numpy().astype(float).tolist()
    o, lse = brute.attend(q, t, rows, inp["sink"].numpy().astype(float).tolist(), th, d_r,
                          1 / math.sqrt(shape.d))
    return ents, sc, sel, o, lse


@pytest.mark.parametrize("shape", [synth.TINY_CSA, synth.TINY_HCA], ids=lambda s: s.name)
def test_tiny_pipeline_matches_brute(shape):
    inp = synth.tiny_inputs(shape)
    res = P.tiny_step(shape, inp)
    ents, sc, sel, o, lse = _brute_tiny(shape, inp)
    assert np.allclose(res["entries"], ents, atol=1e-12)
    if shape.csa:
        assert np.allclose(res["scores"][0], sc, atol=1e-12)
        assert res["sel"][0].tolist() == sel
    assert np.allclose(res["out"][0], o, atol=1e-12)
    assert np.allclose(res["lse"][0], lse, atol=1e-12)


# ------------------------------------------------------------------ planted mistakes


def test_pins_catch_planted_mistakes(monkeypatch):
    """A few plausible slips planted in the oracle must each break a pin above."""
    rng = np.random.default_rng(14)
    x = _rand(rng, 64)
    good = C.rope(x, 321, 160000.0, 16)
    # 1. wrong rotation sign
    bad = C.rope(x, -321, 160000.0, 16)
    assert not np.allclose(bad, brute.rotate(x.tolist(), 321, 160000.0, 16), atol=1e-6)
    # 2. half-split pairs instead of interleaved pairs
    y = x.copy()
    h = y[48:56].copy(), y[56:64].copy()
    u = np.arange(8)
    ang = 321 * 160000.0 ** (-2.0 * u / 16)
    y[48:56] = h[0] * np.cos(ang) - h[1] * np.sin(ang)
    y[56:64] = h[0] * np.sin(ang) + h[1] * np.cos(ang)
    assert not np.allclose(y, good, atol=1e-6)
    # 3. dropping the b-branch changes the overlapped entries
    ca, za, cb, zb = (_rand(rng, 12, 5) for _ in range(4))
    _, e_ok, _ = C.pool(ca, za, None, 4, 0, cb, zb, None)
    _, e_nob, _ = C.pool(ca, za, None, 4, 0)
    assert np.allclose(e_ok[0], e_nob[0]) and not np.allclose(e_ok[1:], e_nob[1:])
    # 4. sink left out of the denominator breaks the mass identity
    q, kv, sink = _rand(rng, 3, 16), _rand(rng, 7, 16), _rand(rng, 3)
    o_s, lse = C.attend_core(q, 0, kv, sink, 1.0, 0, norm_q=False)
    o_n, _ = C.attend_core(q, 0, kv, np.full(3, -1e300), 1.0, 0, norm_q=False)
    assert not np.allclose(o_s, o_n, atol=1e-6)

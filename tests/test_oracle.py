"""Pins for the fp64 oracle: it is checked against things other than itself.

Map of pins (function -> what fixes it):

* oracle.attention: pure-Python brute force written from the definition
  (no max shift, math.exp); the two-key logistic closed form; V = I gives
  P with rows summing to 1; V = 1 gives 1; Q = 0 gives mean(V); one key
  gives V; scipy.special.logsumexp for lse; joint key permutation and query
  permutation equivariance; shift invariance at logits near 10^3 where a
  softmax without the max shift overflows.
* oracle.geometry / cube_layout: the numbers printed in "Anatomy of Wan2.2's
  53.6x speedup", sections "VSA selects cubes" and "Roofline analysis set
  the 3.35 ms target" (tests/golden/page4_vsa_480p.json); hand-computed
  cube ids and slots; a per-token loop on a ragged grid.
* oracle.pool / coarse_scores / select_topk / fine / vsa: a brute-force
  VSA written with Python loops and sorted() on a ragged 5x6x7 grid; top-k
  = all cubes reduces to dense attention; Q = 0 makes every score tie so the
  plan is cubes 0..k-1 and O is the mean of their real V rows; permuting
  tokens inside a key cube leaves everything unchanged; one-cube grids
  reduce to dense; a hand-made score table for the tie rule and margins.
* oracle.coarse_output / gated: a brute force with Python loops (cube
  membership from the coordinates, means, math.exp softmax, broadcast to
  every real token) on a ragged grid; scipy.special.softmax on the same
  scores; V constant gives that constant; Q = 0 gives the mean of all cube
  means; a one-cube grid gives the mean of V; gate = 0 gives the fine output
  exactly; the merge is linear in the gate.
* oracle.flops_fine / kv_stream_bytes: the page's 3.35 TFLOP and 64 GB.
* oracle.rope (3D RoPE, adopted definition): closed forms on D = 6 (angles
  are exactly t, h, w radians) and D = 12 (second pair at theta**-0.5); a
  Python loop over complex numbers on a ragged grid; position 0 is the
  identity; pair norms are kept; dot products depend only on the position
  difference; each axis part moves only with its own coordinate.
* oracle.rope, precision "fp32": every output is an fp32 value, within a few
  fp32 rounding steps of the fp64 rotation, and its bf16 rounding agrees
  with the fp64 mode's except on a sliver of near-ties (never by more than
  one bf16 step).
* oracle.tile_grid / tile_tokens / sta_plan / sta (sliding-tile attention,
  adopted definition): the 6x8x8 tile divides both grids the page accepts
  and not the default grid it refuses; tiles partition the grid row-major;
  the plan against its geometric definition tile by tile (window size, own
  tile inside, centred where it fits, pushed inward at edges); the output
  against a token-level brute force (an allowed-key mask built from token
  coordinates alone, and plain math.exp loops on some rows); a window
  covering the whole tile grid reduces to dense attention; a 1x1x1 window to
  attention within each tile.
* oracle.round_bf16: matches the float32 round-to-nearest-even of synth on
  float32-representable values, resolves exact ties to even, and rounds fp64
  values just above a tie upward (where an fp32 intermediate would not).
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp

import oracle
import synth



def rng(seed):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- dense

def brute_attention(q, k, v, scale):
    """Softmax attention with Python loops and math.exp, straight from the definition."""
    N, D = len(q), len(q[0])
    M, Dv = len(k), len(v[0])
    out, lses = [], []
    for i in range(N):
        w = []
        for j in range(M):
            s = 0.0
            for d in range(D):
                s += q[i][d] * k[j][d]
            w.append(math.exp(scale * s))
        tot = sum(w)
        out.append([sum(w[j] * v[j][e] for j in range(M)) / tot for e in range(Dv)])
        lses.append(math.log(tot))
    return np.array(out), np.array(lses)


@pytest.mark.parametrize("N,M,D,Dv", [(5, 7, 4, 3), (9, 13, 8, 8), (1, 1, 3, 2), (16, 3, 6, 5)])
def test_dense_brute_force(N, M, D, Dv):
    r = rng(N * 100 + M)
    q, k, v = r.normal(size=(N, D)), r.normal(size=(M, D)), r.normal(size=(M, Dv))
    scale = 1 / math.sqrt(D)
    o, lse = oracle.attention(q, k, v, scale)
    ob, lb = brute_attention(q.tolist(), k.tolist(), v.tolist(), scale)
    np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lb, rtol=0, atol=1e-12)


def test_dense_two_keys_is_logistic():
    r = rng(3)
    q, k, v = r.normal(size=(4, 8)), r.normal(size=(2, 8)), r.normal(size=(2, 5))
    s = 0.37
    o, _ = oracle.attention(q, k, v, s)
    for i in range(4):
        a = s * (q[i] @ k[0] - q[i] @ k[1])
        w0 = 1.0 / (1.0 + math.exp(-a))
        np.testing.assert_allclose(o[i], w0 * v[0] + (1 - w0) * v[1], atol=1e-13)


def test_dense_rows_sum_to_one_and_match_probabilities():
    r = rng(4)
    N, M, D = 11, 17, 8
    q, k = r.normal(size=(N, D)) * 2, r.normal(size=(M, D)) * 2
    P, _ = oracle.attention(q, k, np.eye(M), 0.5)          # V = I gives P itself
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    assert (P > 0).all()
    Pb, _ = brute_attention(q.tolist(), k.tolist(), np.eye(M).tolist(), 0.5)
    np.testing.assert_allclose(P, Pb, atol=1e-12)
    ones, _ = oracle.attention(q, k, np.ones((M, 3)), 0.5)
    np.testing.assert_allclose(ones, 1.0, atol=1e-12)


def test_dense_closed_forms():
    r = rng(5)
    M, D = 23, 16
    k, v = r.normal(size=(M, D)), r.normal(size=(M, 7))
    o, lse = oracle.attention(np.zeros((3, D)), k, v, 0.25)
    np.testing.assert_allclose(o, np.tile(v.mean(axis=0), (3, 1)), atol=1e-12)
    np.testing.assert_allclose(lse, math.log(M), atol=1e-12)
    o1, lse1 = oracle.attention(r.normal(size=(4, D)), k[:1], v[:1], 0.25)
    np.testing.assert_allclose(o1, np.tile(v[0], (4, 1)), atol=1e-14)


def test_dense_lse_matches_library_logsumexp():
    r = rng(6)
    q, k, v = r.normal(size=(40, 32)) * 3, r.normal(size=(300, 32)) * 3, r.normal(size=(300, 4))
    s = 1 / math.sqrt(32)
    _, lse = oracle.attention(q, k, v, s, chunk=7)
    np.testing.assert_allclose(lse, logsumexp(s * q @ k.T, axis=1), rtol=1e-13)


def test_dense_permutation_equivariance():
    r = rng(7)
    q, k, v = r.normal(size=(20, 8)), r.normal(size=(30, 8)), r.normal(size=(30, 6))
    o, lse = oracle.attention(q, k, v, 0.4)
    pk = r.permutation(30)
    o2, lse2 = oracle.attention(q, k[pk], v[pk], 0.4)
    np.testing.assert_allclose(o2, o, atol=1e-13)
    np.testing.assert_allclose(lse2, lse, atol=1e-13)
    pq = r.permutation(20)
    o3, _ = oracle.attention(q[pq], k, v, 0.4)
    np.testing.assert_allclose(o3, o[pq], atol=1e-13)
    # swapping the roles of q and k is NOT a symmetry: catches a transposed operand
    o4, _ = oracle.attention(k[:20], q, v[:20], 0.4)
    assert not np.allclose(o4, o)


def test_dense_shift_invariance_at_overflowing_logits():
    """A common shift of every logit of a row changes nothing, even near 1e3.

    Appending a column to q (value 1) and to k (value c/scale) adds c to every
    logit.  Without subtracting the row maximum exp(1000) would overflow.
    """
    r = rng(8)
    q, k, v = r.normal(size=(6, 8)), r.normal(size=(50, 8)), r.normal(size=(50, 3))
    s = 0.5
    o, lse = oracle.attention(q, k, v, s)
    c = 1000.0
    qa = np.hstack([q, np.ones((6, 1))])
    ka = np.hstack([k, np.full((50, 1), c / s)])
    oa, lsea = oracle.attention(qa, ka, v, s)
    assert np.isfinite(oa).all()
    with np.errstate(over="ignore", invalid="ignore"):
        naive = np.exp(s * qa @ ka.T)
        assert not np.isfinite((naive @ v) / naive.sum(1, keepdims=True)).all()
    np.testing.assert_allclose(oa, o, atol=1e-12)
    np.testing.assert_allclose(lsea, lse + c, rtol=1e-15)


def test_dense_row_subset_and_heads():
    r = rng(9)
    q, k, v = r.normal(size=(2, 3, 50, 8)), r.normal(size=(2, 3, 50, 8)), r.normal(size=(2, 3, 50, 8))
    rows = [0, 7, 49]
    o, lse = oracle.attention_heads(q, k, v, 0.3, rows)
    for b in range(2):
        for h in range(3):
            ob, lb = brute_attention(q[b, h, rows].tolist(), k[b, h].tolist(), v[b, h].tolist(), 0.3)
            np.testing.assert_allclose(o[b, h], ob, atol=1e-12)
            np.testing.assert_allclose(lse[b, h], lb, atol=1e-12)


# --------------------------------------------------------------------------- geometry

@pytest.fixture(scope="module")
def page4(golden_dir):
    with open(os.path.join(golden_dir, "page4_vsa_480p.json")) as f:
        return json.load(f)


def test_geometry_matches_page(page4):
    g = oracle.geometry(page4["T"], page4["H"], page4["W"])
    assert g["N"] == page4["tokens"]
    assert (g["Tp"], g["Hp"], g["Wp"]) == (page4["padded_T"], page4["padded_H"], page4["padded_W"])
    assert g["Np"] == page4["padded_tokens"]
    assert [g["nt"], g["nh"], g["nw"]] == page4["cube_grid"]
    assert g["C"] == page4["cubes"]
    assert g["C"] * page4["heads"] == page4["output_tiles"]
    assert round(g["C"] * (1 - page4["sparsity"])) == page4["kept_cubes"]


def test_cost_conventions_match_page(page4):
    fl = oracle.flops_fine(page4["tokens"], page4["kept_cubes"], page4["head_dim"], page4["heads"])
    assert round(fl / 1e12, 2) == page4["tflop_rounded"]
    kv = oracle.kv_stream_bytes(page4["cubes"], page4["kept_cubes"], page4["head_dim"], page4["heads"])
    assert round(kv / 1e9) == page4["kv_stream_gb_rounded"]


def test_cube_layout_hand_values():
    tok = oracle.cube_layout(21, 30, 52)
    assert tok.shape == (624, 64)
    # token (t,h,w) = (0,0,0): cube 0 slot 0
    assert tok[0, 0] == 0
    # (0,0,5): cube (0,0,1) = 1, slot (0*4+0)*4+1 = 1
    assert tok[1, 1] == 5
    # (20,29,51): cube (5,7,12) = (5*8+7)*13+12 = 623, slot (0*4+1)*4+3 = 7
    assert tok[623, 7] == (20 * 30 + 29) * 52 + 51
    # (5,6,7): cube (1,1,1) = (1*8+1)*13+1 = 118, slot (1*4+2)*4+3 = 27
    assert tok[118, 27] == (5 * 30 + 6) * 52 + 7
    # the last t-layer of cubes (t=20..23) holds only t=20: 16 real tokens per full (h,w) cube
    assert (tok[5 * 104] >= 0).sum() == 16
    # a corner cube (t 20-23, h 28-31, w 48-51): 1*2*4 = 8 real tokens, the minimum at 480p
    assert (tok[623] >= 0).sum() == 8
    # every real token appears exactly once
    real = tok[tok >= 0]
    assert np.array_equal(np.sort(real), np.arange(21 * 30 * 52))


def test_cube_layout_against_token_loop():
    T, H, W = 5, 6, 7
    tok = oracle.cube_layout(T, H, W)
    seen = {}
    for t in range(T):
        for h in range(H):
            for w in range(W):
                c = ((t // 4) * 2 + h // 4) * 2 + w // 4
                s = ((t % 4) * 4 + h % 4) * 4 + w % 4
                seen[(c, s)] = (t * H + h) * W + w
    for c in range(8):
        for s in range(64):
            assert tok[c, s] == seen.get((c, s), -1)


# --------------------------------------------------------------------------- VSA

def brute_vsa(q, k, v, T, H, W, topk, scale):
    """VSA with Python loops: membership by (t//4, h//4, w//4), sorted() for top-k."""
    nt, nh, nw = -(-T // 4), -(-H // 4), -(-W // 4)
    members = {}
    for t in range(T):
        for h in range(H):
            for w in range(W):
                c = ((t // 4) * nh + h // 4) * nw + w // 4
                members.setdefault(c, []).append((t * H + h) * W + w)
    C = nt * nh * nw
    D = len(q[0])

    def mean(x, rows):
        return [sum(x[r][d] for r in rows) / len(rows) for d in range(D)]

    qb = [mean(q, members[c]) for c in range(C)]
    kb = [mean(k, members[c]) for c in range(C)]
    scores = [[scale * sum(qb[c][d] * kb[c2][d] for d in range(D)) for c2 in range(C)] for c in range(C)]
    idx = []
    for c in range(C):
        ranked = sorted(range(C), key=lambda c2: (-scores[c][c2], c2))
        idx.append(sorted(ranked[:topk]))
    o = [None] * (T * H * W)
    for c in range(C):
        keys = [j for c2 in idx[c] for j in members[c2]]
        ob, _ = brute_attention([q[i] for i in members[c]], [k[j] for j in keys], [v[j] for j in keys], scale)
        for a, i in enumerate(members[c]):
            o[i] = ob[a]
    return np.array(scores), np.array(idx), np.array(o)


@pytest.mark.parametrize("topk", [1, 3, 8])
def test_vsa_brute_force_ragged_grid(topk):
    T, H, W, D = 5, 6, 7, 8
    N = T * H * W
    r = rng(10 + topk)
    # a smooth field plus noise so cube scores differ clearly
    pos = np.stack(np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij"), -1).reshape(N, 3)
    f = np.cos(pos @ r.normal(size=(3, D)) * 0.6 + r.uniform(0, 6, D))
    q, k, v = f * 2 + r.normal(size=(N, D)), f * 2 + r.normal(size=(N, D)), r.normal(size=(N, D))
    s = 1 / math.sqrt(D)
    res = oracle.vsa(q, k, v, T, H, W, topk, s)
    sb, ib, ob = brute_vsa(q.tolist(), k.tolist(), v.tolist(), T, H, W, topk, s)
    np.testing.assert_allclose(res["scores"], sb, atol=1e-12)
    assert np.array_equal(res["idx"], ib)
    np.testing.assert_allclose(res["o"], ob, atol=1e-12)


def test_vsa_all_cubes_equals_dense():
    T, H, W, D = 6, 9, 10, 16
    N = T * H * W
    r = rng(12)
    q, k, v = r.normal(size=(N, D)), r.normal(size=(N, D)), r.normal(size=(N, D))
    C = oracle.geometry(T, H, W)["C"]
    res = oracle.vsa(q, k, v, T, H, W, C, 0.25)
    od, ld = oracle.attention(q, k, v, 0.25)
    np.testing.assert_allclose(res["o"], od, atol=1e-12)
    np.testing.assert_allclose(res["lse"], ld, atol=1e-12)
    assert np.isinf(res["margin"]).all()


def test_vsa_zero_queries_tie_to_first_cubes():
    T, H, W, D, topk = 7, 5, 9, 8, 3
    N = T * H * W
    r = rng(13)
    k, v = r.normal(size=(N, D)), r.normal(size=(N, D))
    res = oracle.vsa(np.zeros((N, D)), k, v, T, H, W, topk, 0.3)
    C = oracle.geometry(T, H, W)["C"]
    assert np.array_equal(res["idx"], np.tile(np.arange(topk), (C, 1)))
    tok = oracle.cube_layout(T, H, W)
    sel = tok[:topk].ravel()
    expect = v[sel[sel >= 0]].mean(axis=0)
    np.testing.assert_allclose(res["o"], np.tile(expect, (N, 1)), atol=1e-12)


def test_vsa_within_cube_permutation_invariance():
    T, H, W, D, topk = 8, 8, 6, 8, 2
    N = T * H * W
    r = rng(14)
    f = np.cos(np.arange(N)[:, None] * r.normal(size=(1, D)) * 0.05)
    q, k, v = f * 3 + r.normal(size=(N, D)), f * 3 + r.normal(size=(N, D)), r.normal(size=(N, D))
    base = oracle.vsa(q, k, v, T, H, W, topk, 0.35)
    tok = oracle.cube_layout(T, H, W)
    c = 5
    members = tok[c][tok[c] >= 0]
    perm = np.arange(N)
    perm[members] = members[r.permutation(members.size)]
    k2, v2 = k[perm], v[perm]
    res = oracle.vsa(q, k2, v2, T, H, W, topk, 0.35)
    np.testing.assert_allclose(res["kbar"], base["kbar"], atol=1e-13)
    assert np.array_equal(res["idx"], base["idx"])
    np.testing.assert_allclose(res["o"], base["o"], atol=1e-12)


@pytest.mark.parametrize("grid", [(4, 4, 4), (3, 2, 3), (1, 1, 1)])
def test_vsa_single_cube_is_dense(grid):
    T, H, W = grid
    N, D = T * H * W, 8
    r = rng(N)
    q, k, v = r.normal(size=(N, D)), r.normal(size=(N, D)), r.normal(size=(N, D))
    res = oracle.vsa(q, k, v, T, H, W, 1, 0.5)
    od, _ = oracle.attention(q, k, v, 0.5)
    np.testing.assert_allclose(res["o"], od, atol=1e-12)
    np.testing.assert_allclose(res["qbar"][0], q.mean(axis=0), atol=1e-14)


def test_select_topk_tie_rule_and_margin():
    scores = np.array([[3.0, 1.0, 3.0, 2.0],
                       [0.0, 0.0, 0.0, 0.0],
                       [-1.0, 5.0, 4.5, 5.0]])
    idx, m = oracle.select_topk(scores, 2)
    assert idx.tolist() == [[0, 2], [0, 1], [1, 3]]
    np.testing.assert_allclose(m, [1.0, 0.0, 0.5])
    idx3, m3 = oracle.select_topk(scores, 3)
    assert idx3.tolist() == [[0, 2, 3], [0, 1, 2], [1, 2, 3]]
    np.testing.assert_allclose(m3, [1.0, 0.0, 5.5])
    with pytest.raises(ValueError):
        oracle.select_topk(scores, 5)


def test_pool_uses_real_tokens_only():
    T, H, W, D = 5, 5, 5, 3
    N = T * H * W
    x = np.arange(N * D, dtype=np.float64).reshape(N, D)
    tok = oracle.cube_layout(T, H, W)
    qb = oracle.pool(x, tok)
    # the far corner cube (t,h,w >= 4) holds only the token (4,4,4)
    last = (4 * 5 + 4) * 5 + 4
    np.testing.assert_allclose(qb[-1], x[last])
    # cube (0,0,1) holds w = 4 only, for t,h < 4: 16 tokens
    rows = [(t * 5 + h) * 5 + 4 for t in range(4) for h in range(4)]
    np.testing.assert_allclose(qb[1], x[rows].mean(axis=0))


def test_near_tie_tolerance_bounds_fp32_scores():
    """fp32 cube means and fp32 dot products (any order) stay within tau/4 of fp64."""
    T, H, W, D = 9, 10, 11, 128
    N = T * H * W
    r = rng(15)
    q, k = (r.normal(size=(N, D)) * 2).astype(np.float32), (r.normal(size=(N, D)) * 2).astype(np.float32)
    tok = oracle.cube_layout(T, H, W)
    s = 1 / math.sqrt(D)
    exact = oracle.coarse_scores(oracle.pool(q.astype(np.float64), tok), oracle.pool(k.astype(np.float64), tok), s)
    tau = oracle.near_tie_tolerance(q.astype(np.float64), k.astype(np.float64), tok, s)
    valid = tok >= 0

    def pool32(x):
        acc = np.zeros((tok.shape[0], D), np.float32)
        for slot in range(64):                      # sequential fp32 sums
            acc += np.where(valid[:, slot, None], x[np.maximum(tok[:, slot], 0)], np.float32(0))
        return acc / valid.sum(axis=1)[:, None].astype(np.float32)

    qb, kb = pool32(q), pool32(k)
    s32 = np.zeros((qb.shape[0], kb.shape[0]), np.float32)
    for d in range(D):                              # sequential fp32 dot products
        s32 += qb[:, d:d + 1] * kb[None, :, d]
    s32 *= np.float32(s)
    err = np.abs(s32.astype(np.float64) - exact).max(axis=1)
    assert (err <= tau / 4).all()



def _bf16_rne(x):
    """fp32 -> nearest bf16 (ties to even), kept as fp32 values (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def test_three_part_bf16_split_scores_within_tau():
    """Scores from an exact three-part bf16 split of fp32 cube means (hi = bf16(x),
    mid = bf16(x - hi), lo = bf16(x - hi - mid); hi + mid + lo == x) with the six
    leading partial products (mid*lo, lo*mid, lo*lo dropped) summed in fp32, in
    either of two orders, stay within tau/4 of fp64, like plain fp32 dot products."""
    T, H, W, D = 9, 10, 11, 128
    N = T * H * W
    r = rng(15)
    q, k = (r.normal(size=(N, D)) * 2).astype(np.float32), (r.normal(size=(N, D)) * 2).astype(np.float32)
    tok = oracle.cube_layout(T, H, W)
    s = 1 / math.sqrt(D)
    exact = oracle.coarse_scores(oracle.pool(q.astype(np.float64), tok), oracle.pool(k.astype(np.float64), tok), s)
    tau = oracle.near_tie_tolerance(q.astype(np.float64), k.astype(np.float64), tok, s)
    valid = tok >= 0

    def pool32(x):
        acc = np.zeros((tok.shape[0], D), np.float32)
        for slot in range(64):
            acc += np.where(valid[:, slot, None], x[np.maximum(tok[:, slot], 0)], np.float32(0))
        return acc / valid.sum(axis=1)[:, None].astype(np.float32)

    def split(x):
        hi = _bf16_rne(x)
        mid = _bf16_rne(x - hi)
        lo = _bf16_rne(x - hi - mid)
        assert np.array_equal(hi.astype(np.float64) + mid + lo, x.astype(np.float64))   # exact
        return hi, mid, lo

    qp, kp = split(pool32(q)), split(pool32(k))
    terms = [(2, 0), (1, 1), (0, 2), (1, 0), (0, 1), (0, 0)]       # smallest first
    for order in (terms, terms[::-1]):
        s32 = np.zeros((tok.shape[0], tok.shape[0]), np.float32)
        for d0 in range(0, D, 16):                                   # 16-wide steps, term by term
            for a, b in order:
                for d in range(d0, d0 + 16):
                    s32 += qp[a][:, d:d + 1] * kp[b][None, :, d]   # bf16 x bf16 is exact in fp32
        s32 *= np.float32(s)
        err = np.abs(s32.astype(np.float64) - exact).max(axis=1)
        assert (err <= tau / 4).all()

# --------------------------------------------------------------- coarse branch and gate

def brute_coarse_branch(q, k, v, T, H, W, scale):
    """Coarse-branch output broadcast to every real token, with Python loops: [N][D]."""
    nt, nh, nw = -(-T // 4), -(-H // 4), -(-W // 4)
    members = {}
    for t in range(T):
        for h in range(H):
            for w in range(W):
                members.setdefault(((t // 4) * nh + h // 4) * nw + w // 4, []).append((t * H + h) * W + w)
    C, D = nt * nh * nw, len(q[0])

    def mean(x, rows):
        return [sum(x[r][d] for r in rows) / len(rows) for d in range(D)]

    qb = [mean(q, members[c]) for c in range(C)]
    kb = [mean(k, members[c]) for c in range(C)]
    vb = [mean(v, members[c]) for c in range(C)]
    out = [None] * (T * H * W)
    for c in range(C):
        w = [math.exp(scale * sum(qb[c][d] * kb[c2][d] for d in range(D))) for c2 in range(C)]
        tot = sum(w)
        oc = [sum(w[c2] * vb[c2][d] for c2 in range(C)) / tot for d in range(D)]
        for i in members[c]:
            out[i] = oc
    return np.array(out)


def small_vsa_inputs(seed, T=5, H=6, W=7, D=8):
    N = T * H * W
    r = rng(seed)
    pos = np.stack(np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij"), -1).reshape(N, 3)
    f = np.cos(pos @ r.normal(size=(3, D)) * 0.6 + r.uniform(0, 6, D))
    return f * 2 + r.normal(size=(N, D)), f * 2 + r.normal(size=(N, D)), r.normal(size=(N, D))


def test_coarse_branch_brute_force_ragged_grid():
    T, H, W, D = 5, 6, 7, 8
    q, k, v = small_vsa_inputs(31, T, H, W, D)
    s = 1 / math.sqrt(D)
    tok = oracle.cube_layout(T, H, W)
    idx, _ = oracle.select_topk(oracle.coarse_scores(oracle.pool(q, tok), oracle.pool(k, tok), s), 3)
    gate = rng(32).uniform(-1, 1, size=q.shape)
    o, lse = oracle.gated(q, k, v, tok, idx, s, gate)
    of, lf = oracle.fine(q, k, v, tok, idx, s)
    ob = brute_coarse_branch(q.tolist(), k.tolist(), v.tolist(), T, H, W, s)
    np.testing.assert_allclose(o, of + gate * ob, atol=1e-12)
    np.testing.assert_array_equal(lse, lf)


def test_coarse_output_matches_library_softmax():
    from scipy.special import softmax
    r = rng(33)
    qb, kb, vb = r.normal(size=(11, 6)), r.normal(size=(11, 6)), r.normal(size=(11, 4))
    p = softmax(0.4 * qb @ kb.T, axis=1)
    np.testing.assert_allclose(oracle.coarse_output(qb, kb, vb, 0.4), p @ vb, atol=1e-13)


def test_coarse_output_closed_forms():
    T, H, W, D = 6, 9, 10, 16
    q, k, v = small_vsa_inputs(34, T, H, W, D)
    tok = oracle.cube_layout(T, H, W)
    s = 1 / math.sqrt(D)
    qb, kb, vb = oracle.pool(q, tok), oracle.pool(k, tok), oracle.pool(v, tok)
    const = np.full_like(vb, 0.75)
    np.testing.assert_allclose(oracle.coarse_output(qb, kb, const, s), 0.75, atol=1e-13)
    oc = oracle.coarse_output(np.zeros_like(qb), kb, vb, s)  # every score ties: uniform weights
    np.testing.assert_allclose(oc, np.broadcast_to(vb.mean(axis=0), oc.shape), atol=1e-13)
    q1, k1, v1 = small_vsa_inputs(35, 4, 4, 4, D)  # one cube: the mean of V
    t1 = oracle.cube_layout(4, 4, 4)
    o1 = oracle.coarse_output(oracle.pool(q1, t1), oracle.pool(k1, t1), oracle.pool(v1, t1), s)
    np.testing.assert_allclose(o1[0], v1.mean(axis=0), atol=1e-13)


def test_gate_zero_and_linearity():
    T, H, W, D = 5, 6, 7, 8
    q, k, v = small_vsa_inputs(36, T, H, W, D)
    tok = oracle.cube_layout(T, H, W)
    s = 1 / math.sqrt(D)
    idx, _ = oracle.select_topk(oracle.coarse_scores(oracle.pool(q, tok), oracle.pool(k, tok), s), 4)
    of, _ = oracle.fine(q, k, v, tok, idx, s)
    o0, _ = oracle.gated(q, k, v, tok, idx, s, np.zeros_like(q))
    np.testing.assert_array_equal(o0, of)
    g1, g2 = rng(37).normal(size=q.shape), rng(38).normal(size=q.shape)
    d1 = oracle.gated(q, k, v, tok, idx, s, g1)[0] - of
    d2 = oracle.gated(q, k, v, tok, idx, s, g2)[0] - of
    d12 = oracle.gated(q, k, v, tok, idx, s, g1 + g2)[0] - of
    np.testing.assert_allclose(d12, d1 + d2, atol=1e-12)


# --------------------------------------------------------------- 3D RoPE

def test_rope_closed_form_d6():
    """D = 6: one pair per axis, frequency theta**0 = 1, so the angles are t, h, w radians."""
    x = np.tile([1.0, 0.0, 1.0, 0.0, 1.0, 0.0], (2 * 3 * 4, 1))
    r = oracle.rope(x, 2, 3, 4)
    t, h, w = 1, 2, 3
    n = (t * 3 + h) * 4 + w
    expect = [math.cos(t), math.sin(t), math.cos(h), math.sin(h), math.cos(w), math.sin(w)]
    np.testing.assert_allclose(r[n], expect, atol=1e-15)
    # a pair (0, 1) turns to (-sin, cos)
    y = np.tile([0.0, 1.0, 0.0, 1.0, 0.0, 1.0], (24, 1))
    np.testing.assert_allclose(oracle.rope(y, 2, 3, 4)[n], [-math.sin(1), math.cos(1), -math.sin(2),
                                                             math.cos(2), -math.sin(3), math.cos(3)], atol=1e-15)


def test_rope_closed_form_d12_second_frequency():
    """D = 12: parts of 4 dims, two pairs each, frequencies 1 and theta**(-2/4) = 0.01."""
    assert oracle.axis_split(12) == (4, 4, 4)
    x = np.zeros((5 * 1 * 1, 12))
    x[:, 2] = 1.0                                  # pair 1 of the t part
    r = oracle.rope(x, 5, 1, 1)
    np.testing.assert_allclose(r[3, 2:4], [math.cos(0.03), math.sin(0.03)], atol=1e-15)
    assert oracle.axis_split(128) == (44, 42, 42) and oracle.axis_split(64) == (24, 20, 20)


def test_rope_loop_brute_force_ragged_grid():
    T, H, W, D, theta = 3, 5, 7, 20, 500.0
    x = rng(60).normal(size=(T * H * W, D))
    r = oracle.rope(x, T, H, W, theta)
    dt, dh, dw = D - 4 * (D // 6), 2 * (D // 6), 2 * (D // 6)
    for t in range(T):
        for h in range(H):
            for w in range(W):
                n = (t * H + h) * W + w
                start = 0
                for pos, d_a in ((t, dt), (h, dh), (w, dw)):
                    for i in range(d_a // 2):
                        z = complex(x[n, start + 2 * i], x[n, start + 2 * i + 1])
                        z *= complex(math.cos(pos * math.pow(theta, -2.0 * i / d_a)),
                                     math.sin(pos * math.pow(theta, -2.0 * i / d_a)))
                        assert abs(r[n, start + 2 * i] - z.real) < 1e-12
                        assert abs(r[n, start + 2 * i + 1] - z.imag) < 1e-12
                    start += d_a
                assert start == D


def test_rope_invariants():
    T, H, W, D = 4, 6, 5, 128
    x = rng(61).normal(size=(T * H * W, D))
    r = oracle.rope(x, T, H, W)
    np.testing.assert_array_equal(r[0], x[0])       # position (0, 0, 0): identity
    np.testing.assert_allclose(r[:, 0::2] ** 2 + r[:, 1::2] ** 2, x[:, 0::2] ** 2 + x[:, 1::2] ** 2,
                               rtol=1e-12)          # each pair keeps its length
    # the q.k product depends only on the position difference
    q, k = rng(62).normal(size=(1, D)), rng(63).normal(size=(1, D))
    def dot(p, pp):
        rq = oracle.rotate(q, oracle.angles(np.array([p]), D))
        rk = oracle.rotate(k, oracle.angles(np.array([pp]), D))
        return float((rq * rk).sum())
    for p, pp, s in (((3, 1, 4), (0, 2, 2), (5, 7, 9)), ((0, 0, 0), (1, 1, 1), (20, 3, 11))):
        shifted = tuple(a + b for a, b in zip(p, s)), tuple(a + b for a, b in zip(pp, s))
        assert abs(dot(p, pp) - dot(*shifted)) < 1e-10
    assert abs(dot((3, 1, 4), (0, 2, 2)) - dot((3, 1, 4), (0, 2, 3))) > 1e-3
    # each axis part moves with its own coordinate only
    dt, dh, dw = oracle.axis_split(D)
    a = oracle.angles(np.array([[2, 3, 4], [2, 5, 4]]), D)
    assert (a[0, :dt // 2] == a[1, :dt // 2]).all() and (a[0, (dt + dh) // 2:] == a[1, (dt + dh) // 2:]).all()
    assert (a[0, dt // 2:(dt + dh) // 2] != a[1, dt // 2:(dt + dh) // 2]).all()


def test_round_bf16():
    x32 = (rng(64).normal(size=10000) * np.exp(rng(65).uniform(-20, 20, size=10000))).astype(np.float32)
    np.testing.assert_array_equal(oracle.round_bf16(x32.astype(np.float64)),
                                  synth.bits_to_f64(synth.bf16_bits(x32)))
    one = 1.0
    assert oracle.round_bf16(np.array([one + 2.0 ** -8]))[0] == 1.0                      # tie: to even
    assert oracle.round_bf16(np.array([one + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6      # tie: to even
    assert oracle.round_bf16(np.array([-(one + 2.0 ** -8)]))[0] == -1.0
    # just above a tie only in fp64: rounds up (an fp32 intermediate would land on the tie)
    assert oracle.round_bf16(np.array([one + 2.0 ** -8 + 2.0 ** -40]))[0] == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(np.array([0.0]))[0] == 0.0


def test_rope_fp32_mode():
    T, H, W, D = 5, 7, 9, 128
    x = synth.bits_to_f64(synth.bf16_bits(rng(66).normal(size=(T * H * W, D)).astype(np.float32)))
    r64 = oracle.rope(x, T, H, W)
    r32 = oracle.rope(x, T, H, W, precision="fp32")
    np.testing.assert_array_equal(r32.astype(np.float32).astype(np.float64), r32)   # fp32 values
    # two products (each off by <= 1/2 ulp, plus the cos/sin rounding) and one sum: a few fp32 ulps
    scale = np.abs(x).max()
    assert np.abs(r32 - r64).max() <= 4 * 2.0 ** -24 * 2 * scale
    b64, b32 = oracle.round_bf16(r64), oracle.round_bf16(r32)
    differ = b64 != b32
    assert differ.mean() < 1e-3
    step = np.ldexp(1.0, np.frexp(np.abs(b64[differ]))[1] - 8)         # one bf16 step at that size
    assert (np.abs(b64[differ] - b32[differ]) <= step * 1.0000001).all()
    with pytest.raises(ValueError):
        oracle.rope(x, T, H, W, precision="fp16")


# --------------------------------------------------------------- sliding-tile attention

def test_sta_tile_reading_matches_the_pages_accept_rule():
    """The 6x8x8 tile divides both grids the page accepts and not the default grid it refuses."""
    for g in oracle.TUNED_GRIDS:
        nt, nh, nw = oracle.tile_grid(*g)
        assert (nt * 6, nh * 8, nw * 8) == g
    assert oracle.tile_grid(36, 48, 48) == (6, 6, 6) and oracle.tile_grid(18, 48, 80) == (3, 6, 10)
    with pytest.raises(ValueError):
        oracle.tile_grid(31, 22, 40)


def test_sta_tile_tokens_layout():
    T, H, W = 12, 16, 24                          # tile grid 2 x 2 x 3
    tok = oracle.tile_tokens(T, H, W)
    assert tok.shape == (12, 384)
    assert np.array_equal(np.sort(tok.ravel()), np.arange(T * H * W))      # a partition of the grid
    for tile in (0, 5, 11):
        tt, th, tw = tile // 6, (tile // 3) % 2, tile % 3
        t, h, w = tok[tile] // (H * W), (tok[tile] // W) % H, tok[tile] % W
        assert (t // 6 == tt).all() and (h // 8 == th).all() and (w // 8 == tw).all()
        assert (np.diff(tok[tile]) > 0).all()                                # row-major inside the tile


def test_sta_plan_geometry():
    T, H, W = 24, 24, 48                          # tile grid 4 x 3 x 6
    plan = oracle.sta_plan(T, H, W, (3, 3, 3))
    nt, nh, nw = 4, 3, 6
    assert plan.shape == (72, 27)
    for c in range(72):
        ct, ch, cw = c // (nh * nw), (c // nw) % nh, c % nw
        row = plan[c]
        assert (np.diff(row) > 0).all() and c in row
        coords = np.stack([row // (nh * nw), (row // nw) % nh, row % nw], 1)
        for axis, (cc, n) in enumerate(((ct, nt), (ch, nh), (cw, nw))):
            lo, hi = coords[:, axis].min(), coords[:, axis].max()
            assert hi - lo == 2 and 0 <= lo and hi < n
            if 1 <= cc <= n - 2:
                assert lo == cc - 1                 # centred where it fits
            else:
                assert lo == (0 if cc == 0 else n - 3)   # pushed inward at the edges
    assert oracle.window_start(0, 4, 10) == 0 and oracle.window_start(5, 4, 10) == 4
    assert oracle.window_start(9, 4, 10) == 6
    with pytest.raises(ValueError):
        oracle.sta_plan(T, H, W, (5, 1, 1))
    with pytest.raises(ValueError):
        oracle.sta_plan(25, H, W, (1, 1, 1))


def _sta_mask_brute(T, H, W, window):
    """allowed[i, j]: key token j lies in query token i's window, from token coordinates alone."""
    N = T * H * W
    n = np.arange(N)
    coords = np.stack([n // (H * W) // 6, (n // W) % H // 8, n % W // 8], 1)
    tiles = (T // 6, H // 8, W // 8)
    allowed = np.ones((N, N), dtype=bool)
    for axis in range(3):
        c, w, nt = coords[:, axis], window[axis], tiles[axis]
        lo = np.minimum(np.maximum(c - (w - 1) // 2, 0), nt - w)
        allowed &= (coords[None, :, axis] >= lo[:, None]) & (coords[None, :, axis] < lo[:, None] + w)
    return allowed


def test_sta_token_brute_force():
    T, H, W, D = 12, 8, 24, 8                     # tile grid 2 x 1 x 3
    N = T * H * W
    r = np.random.default_rng(95)
    q, k, v = (r.standard_normal((N, D)) for _ in range(3))
    s = 1 / math.sqrt(D)
    window = (1, 1, 2)
    o, lse = oracle.sta(q, k, v, T, H, W, window, s)
    allowed = _sta_mask_brute(T, H, W, window)
    assert (allowed.sum(axis=1) == 2 * 384).all()
    sc = np.where(allowed, (q @ k.T) * s, -np.inf)
    e = np.exp(sc - sc.max(axis=1, keepdims=True))
    np.testing.assert_allclose(o, (e @ v) / e.sum(axis=1, keepdims=True), atol=1e-12)
    np.testing.assert_allclose(lse, sc.max(axis=1) + np.log(e.sum(axis=1)), atol=1e-12)
    for i in r.choice(N, 12, replace=False):      # a few rows by plain loops
        js = [j for j in range(N) if allowed[i, j]]
        ex = [math.exp(s * float(q[i] @ k[j])) for j in js]
        ref = sum(w_ * v[j] for w_, j in zip(ex, js)) / sum(ex)
        np.testing.assert_allclose(o[i], ref, atol=1e-12)
        assert abs(lse[i] - math.log(sum(ex))) < 1e-12


def test_sta_closed_forms():
    T, H, W, D = 12, 16, 8, 16                    # tile grid 2 x 2 x 1
    r = np.random.default_rng(96)
    q, k, v = (r.standard_normal((T * H * W, D)) for _ in range(3))
    s = 1 / math.sqrt(D)
    o, lse = oracle.sta(q, k, v, T, H, W, (2, 2, 1), s)          # the whole tile grid
    od, ld = oracle.attention(q, k, v, s)
    np.testing.assert_allclose(o, od, atol=1e-12)
    np.testing.assert_allclose(lse, ld, atol=1e-12)
    o1, _ = oracle.sta(q, k, v, T, H, W, (1, 1, 1), s)           # each tile on its own
    tok = oracle.tile_tokens(T, H, W)
    for c in range(tok.shape[0]):
        ob, _ = oracle.attention(q[tok[c]], k[tok[c]], v[tok[c]], s)
        np.testing.assert_allclose(o1[tok[c]], ob, atol=1e-12)

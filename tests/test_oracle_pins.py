"""Pins of the CPU oracle to things other than itself (CPU only).

Kinds of pin used (the pages print no worked attention example, so none is a
printed value):

* library routines: torch's float64 ``scaled_dot_product_attention`` on the CPU,
  with its own grouped-query expansion and its own bottom-right causal bias, and
  with a float ``attn_mask`` for the explicit additive mask;
  numpy's ``logaddexp`` for the log-sum-exp split identity;
* closed forms: scale 0 gives the mean of the visible V rows and lse = ln(n);
  one query and two keys give the logistic weights;
* invariants: constant V rows, a one-hot dominant score, key permutation,
  causal first query, microbatch concatenation, paging and MLA sharing; for the
  additive mask: a zero mask and a 0/-inf causal matrix reproduce the unmasked
  and causal results bit for bit, a row-constant mask shifts only lse, single
  visible keys and fully hidden rows, and per-batch masks.

A wrong sign, a dropped scale, a transposed operand, a wrong head group or an
off-by-one causal offset each fails at least one of these.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from torch.nn.attention.bias import causal_lower_right

import oracle

RNG = np.random.default_rng(12345)


def _sdpa(q, k, v, causal, scale):
    """torch float64 SDPA on CPU; inputs in [B, S, H, D] layout."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    Sq, Skv = q.shape[1], k.shape[1]
    mask = causal_lower_right(Sq, Skv) if causal else None
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, scale=scale,
                                       enable_gqa=q.shape[2] != k.shape[2])
    return o.permute(0, 2, 1, 3).numpy()


def _rand(*shape):
    return RNG.standard_normal(shape)


@pytest.mark.parametrize("trial", range(40))
def test_matches_torch_sdpa(oracle_lib, trial):
    r = np.random.default_rng(trial)
    B = int(r.integers(1, 3))
    Hkv = int(r.integers(1, 3))
    G = int(r.integers(1, 4))
    Hq = Hkv * G
    Skv = int(r.integers(1, 12))
    causal = bool(trial % 2)
    # bottom-right causal with Sq <= Skv keeps every row non-empty (torch's
    # lower-right bias gives NaN rows otherwise; empty rows are pinned below)
    Sq = int(r.integers(1, Skv + 1)) if causal else int(r.integers(1, 12))
    Dqk = int(r.integers(1, 9))
    Dv = int(r.integers(1, 9))
    scale = float(r.uniform(0.1, 1.5))
    q = r.standard_normal((B, Sq, Hq, Dqk))
    k = r.standard_normal((B, Skv, Hkv, Dqk))
    v = r.standard_normal((B, Skv, Hkv, Dv))
    o, lse = oracle.attention(q, k, v, causal, scale)
    ref = _sdpa(q, k, v, causal, scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert lse.shape == (B, Hq, Sq) and np.all(np.isfinite(lse))


def test_lse_split_identity(oracle_lib):
    """Splitting the keys in two: lse = logaddexp(lse_A, lse_B) and
    o = (e^{lse_A} o_A + e^{lse_B} o_B) / e^{lse}; checks lse (natural log,
    scale included) against numpy's logaddexp."""
    B, S, H, D = 2, 7, 3, 5
    q, k, v = _rand(B, 4, H, D), _rand(B, S, H, D), _rand(B, S, H, D)
    scale = 0.7
    o, lse = oracle.attention(q, k, v, False, scale)
    oa, la = oracle.attention(q, k[:, :3], v[:, :3], False, scale)
    ob, lb = oracle.attention(q, k[:, 3:], v[:, 3:], False, scale)
    np.testing.assert_allclose(lse, np.logaddexp(la, lb), rtol=0, atol=1e-12)
    wa = np.exp(la - lse).transpose(0, 2, 1)[..., None]
    wb = np.exp(lb - lse).transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(o, wa * oa + wb * ob, rtol=0, atol=1e-12)


def test_two_keys_logistic(oracle_lib):
    """One query, two keys, D = 1: weights 1/(1+e^{-d}) and 1/(1+e^{d}) with
    d = scale * q * (k0 - k1); lse = scale*q*k0 + ln(1 + e^{-d})."""
    for qv, k0, k1, scale in [(1.0, 2.0, -1.0, 0.5), (-0.3, 0.25, 4.0, 2.0), (3.0, 1.0, 1.0, 1.0)]:
        q = np.array([[[[qv]]]])
        k = np.array([[[[k0]], [[k1]]]])
        v = np.array([[[[10.0]], [[-20.0]]]])
        o, lse = oracle.attention(q, k, v, False, scale)
        d = scale * qv * (k0 - k1)
        w0 = 1.0 / (1.0 + math.exp(-d))
        assert o[0, 0, 0, 0] == pytest.approx(10.0 * w0 - 20.0 * (1.0 - w0), abs=1e-13)
        assert lse[0, 0, 0] == pytest.approx(scale * qv * k0 + math.log1p(math.exp(-d)), abs=1e-13)


@pytest.mark.parametrize("Sq,Skv", [(5, 5), (3, 8), (8, 3), (1, 6)])
def test_scale_zero_prefix_mean(oracle_lib, Sq, Skv):
    """scale = 0: every visible key has weight 1/n, so o_i is the mean of the
    visible V rows and lse = ln(n). Causal bottom-right: query i sees keys
    0 .. i + Skv - Sq; rows with no visible key give 0 and -inf."""
    B, H, D = 1, 2, 3
    q, k, v = _rand(B, Sq, H, D), _rand(B, Skv, H, D), _rand(B, Skv, H, D)
    o, lse = oracle.attention(q, k, v, True, 0.0)
    for i in range(Sq):
        n = i + Skv - Sq + 1
        for h in range(H):
            if n <= 0:
                assert np.all(o[0, i, h] == 0.0) and lse[0, h, i] == -np.inf
            else:
                np.testing.assert_allclose(o[0, i, h], v[0, :n, h].mean(axis=0), atol=1e-14)
                assert lse[0, h, i] == pytest.approx(math.log(n), abs=1e-14)
    o2, lse2 = oracle.attention(q, k, v, False, 0.0)
    np.testing.assert_allclose(o2, np.broadcast_to(v.mean(axis=1, keepdims=True), o2.shape),
                               atol=1e-14)
    np.testing.assert_allclose(lse2, math.log(Skv), atol=1e-14)


def test_constant_v_rows(oracle_lib):
    B, Sq, Skv, H, D = 2, 6, 9, 2, 4
    q, k = _rand(B, Sq, H, D), _rand(B, Skv, H, D)
    c = _rand(B, 1, H, D)
    v = np.broadcast_to(c, (B, Skv, H, D)).copy()
    for causal in (False, True):
        o, _ = oracle.attention(q, k, v, causal, 0.9)
        np.testing.assert_allclose(o, np.broadcast_to(c, o.shape), rtol=0, atol=1e-14)


def test_one_hot_dominant_score(oracle_lib):
    """q = c*e0, k_{j*} = e0, other keys orthogonal to e0: with c*scale = 40 the
    weight of every other key is e^-40, so o = v_{j*} to ~1e-17."""
    D, Skv, jstar, scale = 4, 7, 3, 0.125
    q = np.zeros((1, 1, 1, D)); q[0, 0, 0, 0] = 320.0
    k = _rand(1, Skv, 1, D); k[..., 0] = 0.0; k[0, jstar, 0, :] = 0.0; k[0, jstar, 0, 0] = 1.0
    v = _rand(1, Skv, 1, D)
    o, _ = oracle.attention(q, k, v, False, scale)
    np.testing.assert_allclose(o[0, 0, 0], v[0, jstar, 0], rtol=0, atol=1e-15)


def test_key_permutation_invariance(oracle_lib):
    B, Sq, Skv, H, D = 1, 5, 11, 2, 6
    q, k, v = _rand(B, Sq, H, D), _rand(B, Skv, H, D), _rand(B, Skv, H, D)
    p = RNG.permutation(Skv)
    o1, l1 = oracle.attention(q, k, v, False, 0.4)
    o2, l2 = oracle.attention(q, k[:, p], v[:, p], False, 0.4)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_causal_first_query_is_v0(oracle_lib):
    B, S, H, D = 2, 8, 3, 5
    q, k, v = _rand(B, S, H, D), _rand(B, S, H, D), _rand(B, S, H, D)
    o, _ = oracle.attention(q, k, v, True, 1.3)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])


def test_microbatch_concatenation(oracle_lib):
    """A causal call over the whole sequence equals microbatch calls u with
    queries [u*ub, (u+1)*ub) against keys [0, (u+1)*ub) (bottom-right)."""
    S, ub, Hq, Hkv, D = 24, 6, 4, 2, 4
    q, k, v = _rand(1, S, Hq, D), _rand(1, S, Hkv, D), _rand(1, S, Hkv, D)
    o, lse = oracle.attention(q, k, v, True, 0.5)
    for u in range(S // ub):
        ou, lu = oracle.attention(q[:, u * ub:(u + 1) * ub], k[:, :(u + 1) * ub],
                                  v[:, :(u + 1) * ub], True, 0.5)
        np.testing.assert_allclose(ou, o[:, u * ub:(u + 1) * ub], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lu, lse[:, :, u * ub:(u + 1) * ub], rtol=0, atol=1e-14)


def test_gqa_equals_repeated_mha(oracle_lib):
    B, Sq, Skv, Hkv, G, D = 1, 4, 6, 2, 3, 5
    q, k, v = _rand(B, Sq, Hkv * G, D), _rand(B, Skv, Hkv, D), _rand(B, Skv, Hkv, D)
    o1, l1 = oracle.attention(q, k, v, True, 0.6)
    o2, l2 = oracle.attention(q, np.repeat(k, G, axis=2), np.repeat(v, G, axis=2), True, 0.6)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_rows_api_matches_full(oracle_lib):
    B, Sq, Skv, Hq, Hkv, D = 2, 5, 7, 4, 2, 3
    q, k, v = _rand(B, Sq, Hq, D), _rand(B, Skv, Hkv, D), _rand(B, Skv, Hkv, D)
    o, lse = oracle.attention(q, k, v, True, 0.8)
    rows = np.array([[1, 3, 4], [0, 0, 0], [1, 1, 2]])
    orow, lrow = oracle.attention_rows(q[rows[:, 0], rows[:, 2], rows[:, 1]], rows[:, 0],
                                       rows[:, 1], rows[:, 2], k, v, Hq, Sq, True, 0.8)
    for n, (b, h, i) in enumerate(rows):
        np.testing.assert_array_equal(orow[n], o[b, i, h])
        assert lrow[n] == lse[b, h, i]


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("masked", [False, True])
def test_prefill_rows_matches_full_and_sdpa(oracle_lib, causal, masked):
    """The row checker used for the full-size prefill workloads: on a shape where
    B, Hq, Hkv, Sq, Skv and D all differ, every (b, h, i) row in a shuffled order
    equals the full oracle's o[b, i, h] and lse[b, h, i] bit for bit, and torch's
    float64 SDPA (its own gather, GQA expansion and bottom-right causal bias)
    to 1e-12."""
    import fa_inputs as fi
    inp = fi.prefill_inputs(9, 3, 6, 2, 5, 11, 8, causal, "bf16")
    if masked:
        inp = fi.with_mask(inp, 9, "normal", batched=True, stride=16)
    o, lse = oracle.prefill(inp)
    rows = np.array([(b, h, i) for b in range(3) for h in range(6) for i in range(5)])
    rows = rows[np.random.default_rng(4).permutation(len(rows))]
    orow, lrow = oracle.prefill_rows(inp, rows)
    np.testing.assert_array_equal(orow, o[rows[:, 0], rows[:, 2], rows[:, 1]])
    np.testing.assert_array_equal(lrow, lse[rows[:, 0], rows[:, 1], rows[:, 2]])
    q, k, v = (oracle.widen(x, "bf16") for x in (inp.q, inp.k, inp.v))
    if masked:
        m = torch.from_numpy(oracle.widen(inp.mask, "bf16")[:, None, :, :11])
        if causal:
            m = m + torch.where(torch.ones(5, 11, dtype=torch.bool).tril(11 - 5), 0.0,
                                -math.inf).double()
        tq, tk, tv = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
        ref = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m, scale=float(inp.scale),
                                             enable_gqa=True).permute(0, 2, 1, 3).numpy()
    else:
        ref = _sdpa(q, k, v, causal, float(inp.scale))
    np.testing.assert_allclose(orow, ref[rows[:, 0], rows[:, 2], rows[:, 1]], rtol=0,
                               atol=1e-12)


def test_thread_count_does_not_change_result(oracle_lib):
    q, k, v = _rand(2, 9, 4, 8), _rand(2, 13, 2, 8), _rand(2, 13, 2, 8)
    o1, l1 = oracle.attention(q, k, v, True, 0.3, nthreads=1)
    o7, l7 = oracle.attention(q, k, v, True, 0.3, nthreads=7)
    np.testing.assert_array_equal(o1, o7)
    np.testing.assert_array_equal(l1, l7)


# --------------------------------------------------------------------------
# explicit additive mask
# --------------------------------------------------------------------------

def _sdpa_masked(q, k, v, mask, causal, scale):
    """torch float64 SDPA with a float attn_mask [Bm, Sq, Skv] (broadcast over
    heads); the causal rule is folded in as -inf above the bottom-right
    diagonal, built here from key and query positions."""
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3)
    Sq, Skv = q.shape[1], k.shape[1]
    m = torch.from_numpy(mask.copy())
    if causal:
        hide = torch.arange(Skv)[None, :] > torch.arange(Sq)[:, None] + (Skv - Sq)
        m = m.masked_fill(hide[None], float("-inf"))
    o = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=m[:, None], scale=scale,
                                       enable_gqa=q.shape[2] != k.shape[2])
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("trial", range(24))
def test_mask_matches_torch_sdpa(oracle_lib, trial):
    """Random finite masks with scattered -inf (never a whole visible row),
    shared by the batch or one per batch entry, with and without the causal
    rule: against torch's float64 SDPA with a float attn_mask."""
    r = np.random.default_rng(100 + trial)
    B, Hkv, G = int(r.integers(1, 3)), int(r.integers(1, 3)), int(r.integers(1, 4))
    Hq = Hkv * G
    Skv = int(r.integers(2, 12))
    causal = bool(trial % 2)
    Sq = int(r.integers(1, Skv + 1)) if causal else int(r.integers(1, 12))
    D = int(r.integers(1, 9))
    scale = float(r.uniform(0.1, 1.5))
    q, k, v = r.standard_normal((B, Sq, Hq, D)), r.standard_normal((B, Skv, Hkv, D)), \
        r.standard_normal((B, Skv, Hkv, D))
    Bm = B if trial % 3 == 0 else 1
    mask = 2.0 * r.standard_normal((Bm, Sq, Skv))
    hide = r.random((Bm, Sq, Skv)) < 0.3
    hide[..., 0] = False  # key 0 is visible to every row (also under the causal rule)
    mask[hide] = -np.inf
    o, lse = oracle.attention(q, k, v, causal, scale, mask=mask)
    ref = _sdpa_masked(q, k, v, np.broadcast_to(mask, (B, Sq, Skv)), causal, scale)
    np.testing.assert_allclose(o, ref, rtol=1e-12, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_zero_mask_is_no_mask(oracle_lib):
    """An all-zero mask changes nothing, bit for bit."""
    q, k, v = _rand(2, 5, 4, 6), _rand(2, 9, 2, 6), _rand(2, 9, 2, 6)
    for causal in (False, True):
        o0, l0 = oracle.attention(q, k, v, causal, 0.4)
        o1, l1 = oracle.attention(q, k, v, causal, 0.4, mask=np.zeros((1, 5, 9)))
        assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_causal_mask_matrix_equals_causal_rule(oracle_lib):
    """A 0 / -inf matrix of the bottom-right causal pattern, without the causal
    flag, gives exactly the causal result (with a padded row stride)."""
    Sq, Skv = 6, 10
    q, k, v = _rand(1, Sq, 2, 5), _rand(1, Skv, 1, 5), _rand(1, Skv, 1, 5)
    mask = np.full((1, Sq, Skv + 3), np.nan)
    for i in range(Sq):
        for j in range(Skv):
            mask[0, i, j] = 0.0 if j <= i + Skv - Sq else -np.inf
    o0, l0 = oracle.attention(q, k, v, True, 0.9)
    o1, l1 = oracle.attention(q, k, v, False, 0.9, mask=mask)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_row_constant_mask_shifts_lse_only(oracle_lib):
    """Adding c_i to every key of row i leaves o unchanged and adds c_i to lse."""
    Sq, Skv = 4, 7
    q, k, v = _rand(1, Sq, 3, 4), _rand(1, Skv, 3, 4), _rand(1, Skv, 3, 4)
    c = np.array([0.5, -3.0, 7.25, 0.0])
    mask = np.repeat(c[:, None], Skv, axis=1)[None]
    o0, l0 = oracle.attention(q, k, v, False, 0.6)
    o1, l1 = oracle.attention(q, k, v, False, 0.6, mask=mask)
    np.testing.assert_allclose(o1, o0, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l0 + c[None, None, :], rtol=0, atol=1e-12)


def test_single_visible_key_and_empty_rows(oracle_lib):
    """Row 0 sees only key 3 (o = v_3, lse = score_3 + mask_3); row 1 sees
    nothing (o = 0, lse = -inf); row 2 sees only key 4 (o = v_4). With the
    causal rule on top (Sq = 3 < Skv = 5: row 0 sits at position 2), row 0
    loses key 3 and becomes empty while row 2 keeps key 4."""
    Sq, Skv, D = 3, 5, 4
    q, k, v = _rand(1, Sq, 1, D), _rand(1, Skv, 1, D), _rand(1, Skv, 1, D)
    mask = np.full((1, Sq, Skv), -np.inf)
    mask[0, 0, 3] = 1.5
    mask[0, 2, 4] = 0.0
    o, lse = oracle.attention(q, k, v, False, 0.8, mask=mask)
    np.testing.assert_array_equal(o[0, 0, 0], v[0, 3, 0])
    assert lse[0, 0, 0] == pytest.approx(0.8 * float(q[0, 0, 0] @ k[0, 3, 0]) + 1.5, abs=1e-13)
    assert np.all(o[0, 1, 0] == 0) and lse[0, 0, 1] == -np.inf
    np.testing.assert_array_equal(o[0, 2, 0], v[0, 4, 0])
    o2, lse2 = oracle.attention(q, k, v, True, 0.8, mask=mask)
    assert np.all(o2[0, 0, 0] == 0) and lse2[0, 0, 0] == -np.inf
    np.testing.assert_array_equal(o2[0, 2, 0], v[0, 4, 0])


def test_batched_mask_equals_per_batch_calls(oracle_lib):
    """One mask per batch entry equals separate single-batch calls."""
    q, k, v = _rand(3, 4, 2, 5), _rand(3, 6, 2, 5), _rand(3, 6, 2, 5)
    mask = _rand(3, 4, 6)
    mask[_rand(3, 4, 6) > 1.0] = -np.inf
    mask[..., 0] = 0.0
    o, lse = oracle.attention(q, k, v, False, 0.5, mask=mask)
    for b in range(3):
        ob, lb = oracle.attention(q[b:b + 1], k[b:b + 1], v[b:b + 1], False, 0.5,
                                  mask=mask[b:b + 1])
        assert np.array_equal(o[b:b + 1], ob) and np.array_equal(lse[b:b + 1], lb)


def test_bad_arguments_raise(oracle_lib):
    q, k, v = _rand(1, 2, 3, 4), _rand(1, 2, 2, 4), _rand(1, 2, 2, 4)
    with pytest.raises(RuntimeError):
        oracle.attention(q, k, v, False, 1.0)  # Hq % Hkv != 0


# --------------------------------------------------------------------------
# paging and MLA
# --------------------------------------------------------------------------

class _Dec:
    pass


def _scatter_split_pool(K, V, page_size, r, spare=3):
    """Place contiguous K, V ([B][n_b, Hkv, D] lists) into a paged pool with a
    random page assignment (the inverse of the oracle's gather, written here
    independently), poisoning unused slots with NaN."""
    B = len(K)
    Hkv, D = K[0].shape[1], K[0].shape[2]
    pages_per = [(k.shape[0] + page_size - 1) // page_size for k in K]
    P = sum(pages_per) + spare
    perm = r.permutation(P)
    pool = np.full((P, 2, Hkv, page_size, D), np.nan)
    table = np.full((B, max(1, max(pages_per))), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        for t in range(K[b].shape[0]):
            pg = perm[at + t // page_size]
            table[b, t // page_size] = pg
            pool[pg, 0, :, t % page_size, :] = K[b][t]
            pool[pg, 1, :, t % page_size, :] = V[b][t]
        at += pages_per[b]
    return pool, table


@pytest.mark.parametrize("page_size", [1, 3, 16])
def test_paged_split_equals_contiguous(oracle_lib, page_size):
    r = np.random.default_rng(page_size)
    B, Hkv, G, D = 3, 2, 2, 4
    lens = [5, 17, 1]
    K = [r.standard_normal((n, Hkv, D)) for n in lens]
    V = [r.standard_normal((n, Hkv, D)) for n in lens]
    pool, table = _scatter_split_pool(K, V, page_size, r)
    d = _Dec()
    d.q = r.standard_normal((B, Hkv * G, D)); d.pool = pool; d.page_table = table
    d.seq_lens = np.array(lens, dtype=np.int32); d.page_size = page_size; d.layout = "split"
    d.Hkv = Hkv; d.D_qk = D; d.D_v = D; d.scale = 0.45; d.dtype = "fp64"; d.B = B
    o, lse = oracle.decode_paged(d)
    for b in range(B):
        ob, lb = oracle.attention(d.q[b][None, None], K[b][None], V[b][None], False, 0.45)
        np.testing.assert_array_equal(o[b], ob[0, 0])
        np.testing.assert_array_equal(lse[b], lb[0, :, 0])
        assert np.all(np.isfinite(o[b]))


@pytest.mark.parametrize("page_size", [1, 4])
def test_paged_multi_token_matches_torch_sdpa(oracle_lib, page_size):
    """Sq new tokens per sequence over a paged pool: against torch float64 SDPA
    with its own lower-right causal bias on the K/V scattered into the pool
    (the pool is built independently of the oracle's gather)."""
    r = np.random.default_rng(40 + page_size)
    B, Hkv, G, D, Sq = 3, 2, 3, 5, 4
    lens = [9, 4, 13]
    K = [r.standard_normal((n, Hkv, D)) for n in lens]
    V = [r.standard_normal((n, Hkv, D)) for n in lens]
    pool, table = _scatter_split_pool(K, V, page_size, r)
    d = _Dec()
    d.q = r.standard_normal((B, Sq, Hkv * G, D)); d.pool = pool; d.page_table = table
    d.seq_lens = np.array(lens, dtype=np.int32); d.page_size = page_size; d.layout = "split"
    d.Hkv = Hkv; d.D_qk = D; d.D_v = D; d.scale = 0.6; d.dtype = "fp64"; d.B = B; d.Sq = Sq
    o, lse = oracle.decode_paged(d)
    assert o.shape == (B, Sq, Hkv * G, D) and lse.shape == (B, Hkv * G, Sq)
    for b in range(B):
        ref = _sdpa(d.q[b][None], K[b][None], V[b][None], True, 0.6)
        np.testing.assert_allclose(o[b], ref[0], rtol=1e-12, atol=1e-12)


def test_paged_multi_token_is_truncated_single_token(oracle_lib):
    """New token i of Sq equals a one-token decode of the same sequence cut to
    its first seq_len - Sq + i + 1 tokens; a token whose position is negative
    (seq_len < Sq) sees nothing."""
    r = np.random.default_rng(44)
    B, Hkv, G, D, Sq = 2, 1, 2, 3, 5
    lens = [8, 3]
    K = [r.standard_normal((n, Hkv, D)) for n in lens]
    V = [r.standard_normal((n, Hkv, D)) for n in lens]
    pool, table = _scatter_split_pool(K, V, 2, r)
    d = _Dec()
    d.q = r.standard_normal((B, Sq, Hkv * G, D)); d.pool = pool; d.page_table = table
    d.seq_lens = np.array(lens, dtype=np.int32); d.page_size = 2; d.layout = "split"
    d.Hkv = Hkv; d.D_qk = D; d.D_v = D; d.scale = 1.1; d.dtype = "fp64"; d.B = B; d.Sq = Sq
    o, lse = oracle.decode_paged(d)
    for b in range(B):
        for i in range(Sq):
            n = lens[b] - Sq + i + 1
            if n <= 0:
                assert np.all(o[b, i] == 0) and np.all(np.isneginf(lse[b, :, i]))
                continue
            e = _Dec()
            e.__dict__.update(d.__dict__)
            e.Sq = 1
            e.q = d.q[:, i]
            e.seq_lens = np.array([n if bb == b else 1 for bb in range(B)], dtype=np.int32)
            o1, l1 = oracle.decode_paged(e, [b])
            np.testing.assert_array_equal(o[b, i], o1[0])
            np.testing.assert_array_equal(lse[b, :, i], l1[0])


def test_paged_zero_length_sequence(oracle_lib):
    d = _Dec()
    d.q = _rand(1, 2, 4); d.pool = np.full((2, 2, 1, 4, 4), np.nan)
    d.page_table = np.full((1, 1), -1, dtype=np.int32); d.seq_lens = np.zeros(1, np.int32)
    d.page_size = 4; d.layout = "split"; d.Hkv = 1; d.D_qk = 4; d.D_v = 4; d.scale = 1.0
    d.dtype = "fp64"; d.B = 1
    o, lse = oracle.decode_paged(d)
    assert np.all(o == 0.0) and np.all(lse == -np.inf)


@pytest.mark.parametrize("page_size", [1, 4])
def test_mla_equals_mha_with_materialised_kv(oracle_lib, page_size):
    """MLA decode with one shared [ckv | kpe] row per token equals MHA with
    Hkv = 1, K = [ckv, kpe] and V = ckv."""
    r = np.random.default_rng(7 + page_size)
    B, Hq, Dc, Dr, n = 2, 8, 6, 2, 12
    ckv = r.standard_normal((B, n, Dc))
    kpe = r.standard_normal((B, n, Dr))
    rows = np.concatenate([ckv, kpe], axis=2)
    P = B * n // page_size
    perm = r.permutation(P)
    table = perm.reshape(B, n // page_size).astype(np.int32)
    pool = np.empty((P, page_size, Dc + Dr))
    for b in range(B):
        for t in range(n):
            pool[table[b, t // page_size], t % page_size] = rows[b, t]
    d = _Dec()
    d.q = r.standard_normal((B, Hq, Dc + Dr)); d.pool = pool; d.page_table = table
    d.seq_lens = np.full(B, n, np.int32); d.page_size = page_size; d.layout = "mla"; d.Hkv = 1
    d.D_qk = Dc + Dr; d.D_v = Dc; d.scale = 0.33; d.dtype = "fp64"; d.B = B
    o, lse = oracle.decode_paged(d)
    for b in range(B):
        K = np.concatenate([ckv[b], kpe[b]], axis=1)[None, :, None, :]
        V = ckv[b][None, :, None, :]
        ob, lb = oracle.attention(d.q[b][None, None], K, V, False, 0.33)
        np.testing.assert_array_equal(o[b], ob[0, 0])
        ref = _sdpa(d.q[b][None, None], K, V, False, 0.33)
        np.testing.assert_allclose(o[b], ref[0, 0], rtol=1e-12, atol=1e-12)


def test_widen_matches_torch():
    bits = np.arange(0, 65536, 7, dtype=np.uint16)
    w = oracle.widen(bits, "bf16")
    t = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(np.isnan(w), np.isnan(t))
    ok = ~np.isnan(w)
    np.testing.assert_array_equal(w[ok], t[ok])
    w = oracle.widen(bits, "fp16")
    t = torch.from_numpy(bits.view(np.int16)).view(torch.float16).double().numpy()
    ok = ~np.isnan(w)
    np.testing.assert_array_equal(w[ok], t[ok])

"""Pins of the fp64 attention oracle against facts that do not come from itself.

Each ``pin_*`` takes the attention routine under test so the same checks can be
run against deliberately broken copies of the oracle (``test_pins_have_teeth``):
every planted mistake must trip at least one pin.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import attention as oatt
from synth import TINY_PREFILL, prefill_inputs

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

TOL = 1e-12


def rnd(seed, *shape):
    return np.random.Generator(np.random.SFC64(seed)).standard_normal(shape)


def tiny_cases():
    """Random tiny shapes: N <= 8, d <= 4, G in {1, 2}, causal on and off."""
    cases = []
    seed = 100
    for N in (1, 2, 3, 5, 8):
        for d in (1, 2, 4):
            for (Hq, Hk) in ((1, 1), (2, 1), (2, 2), (4, 2)):
                for causal in (False, True):
                    seed += 1
                    cases.append((seed, 1 + (seed % 2), Hq, Hk, N, d, causal))
    return cases


# ---------------------------------------------------------------------------
# pins, parameterised by the routine under test
# ---------------------------------------------------------------------------
def pin_brute(fn):
    for seed, B, Hq, Hk, N, d, causal in tiny_cases()[::3]:
        q, k, v = rnd(seed, B, Hq, N, d), rnd(seed + 1, B, Hk, N, d), rnd(seed + 2, B, Hk, N, d)
        scale = 0.5 + (seed % 3) * 0.25
        O, L = fn(q, k, v, scale, causal)
        Ob, Lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        assert np.max(np.abs(O - np.array(Ob))) <= TOL
        assert np.max(np.abs(L - np.array(Lb))) <= TOL


def pin_constant_v(fn):
    q, k = rnd(1, 2, 4, 7, 3), rnd(2, 2, 2, 7, 3)
    for c in (-1.5, 0.0, 3.25):
        v = np.full((2, 2, 7, 3), c)
        for causal in (False, True):
            O, _ = fn(q, k, v, 0.7, causal)
            assert np.max(np.abs(O - c)) <= TOL


def pin_zero_query(fn):
    """q = 0: every visible key gets weight 1/#visible, and lse = ln #visible."""
    N, d = 6, 4
    q = np.zeros((1, 2, N, d))
    k, v = rnd(3, 1, 1, N, d) * 5, rnd(4, 1, 1, N, d)
    for causal in (False, True):
        O, L = fn(q, k, v, 1.3, causal)
        for i in range(N):
            n_vis = i + 1 if causal else N
            expect = v[0, 0, :n_vis].mean(axis=0)
            assert np.max(np.abs(O[0, :, i] - expect)) <= TOL
            assert np.max(np.abs(L[0, :, i] - math.log(n_vis))) <= TOL


def pin_single_key(fn):
    """One key: O is that key's value row exactly, lse is its score."""
    q, k, v = rnd(5, 1, 1, 1, 5), rnd(6, 1, 1, 1, 5), rnd(7, 1, 1, 1, 5)
    O, L = fn(q, k, v, 0.9, False)
    assert np.array_equal(O[0, 0, 0], v[0, 0, 0])
    assert abs(L[0, 0, 0] - 0.9 * float(q[0, 0, 0] @ k[0, 0, 0])) <= TOL
    # causal row 0 of a longer sequence sees only key 0
    q, k, v = rnd(8, 1, 1, 4, 3), rnd(9, 1, 1, 4, 3), rnd(10, 1, 1, 4, 3)
    O, L = fn(q, k, v, 0.5, True)
    assert np.max(np.abs(O[0, 0, 0] - v[0, 0, 0])) <= TOL
    assert abs(L[0, 0, 0] - 0.5 * float(q[0, 0, 0] @ k[0, 0, 0])) <= TOL


def pin_dominant_key(fn):
    """A key scoring 1000 above every other takes all the weight."""
    N, d = 9, 4
    q = np.zeros((1, 1, N, d))
    q[..., 0] = 1.0
    k = rnd(11, 1, 1, N, d) * 0.1
    k[0, 0, 4, 0] = 1000.0
    v = rnd(12, 1, 1, N, d)
    O, _ = fn(q, k, v, 1.0, False)
    assert np.max(np.abs(O[0, 0] - v[0, 0, 4])) <= TOL


def pin_permutation(fn):
    """Without a mask, permuting K and V rows together changes nothing."""
    q, k, v = rnd(13, 2, 4, 5, 3), rnd(14, 2, 2, 7, 3), rnd(15, 2, 2, 7, 3)
    perm = np.random.Generator(np.random.SFC64(16)).permutation(7)
    O1, L1 = fn(q, k, v, 0.8, False)
    O2, L2 = fn(q, k[:, :, perm], v[:, :, perm], 0.8, False)
    assert np.max(np.abs(O1 - O2)) <= 1e-13
    assert np.max(np.abs(L1 - L2)) <= 1e-13


def pin_gqa_is_repeated_mha(fn):
    """GQA equals MHA with every KV head repeated G times in a contiguous run."""
    B, Hk, G, N, d = 2, 2, 3, 5, 4
    q, k, v = rnd(17, B, Hk * G, N, d), rnd(18, B, Hk, N, d), rnd(19, B, Hk, N, d)
    krep, vrep = np.repeat(k, G, axis=1), np.repeat(v, G, axis=1)
    for causal in (False, True):
        O1, L1 = fn(q, k, v, 0.6, causal)
        O2, L2 = fn(q, krep, vrep, 0.6, causal)
        assert np.max(np.abs(O1 - O2)) <= TOL
        assert np.max(np.abs(L1 - L2)) <= TOL


def pin_torch_sdpa(fn):
    """A third opinion: torch's CPU fp64 scaled-dot-product attention."""
    torch = pytest.importorskip("torch")
    import torch.nn.functional as F
    for causal in (False, True):
        q, k, v = rnd(20, 2, 4, 9, 8), rnd(21, 2, 4, 9, 8), rnd(22, 2, 4, 9, 8)
        O, _ = fn(q, k, v, 0.35, causal)
        ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k),
                                             torch.from_numpy(v), is_causal=causal,
                                             scale=0.35).numpy()
        assert np.max(np.abs(O - ref)) <= 1e-12


PINS = [pin_brute, pin_constant_v, pin_zero_query, pin_single_key, pin_dominant_key,
        pin_permutation, pin_gqa_is_repeated_mha, pin_torch_sdpa]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_one_shot_pins(pin):
    pin(oracle.one_shot)


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_tiled_pins(pin):
    pin(lambda q, k, v, s, c: oracle.tiled(q, k, v, s, c, tile=3))


def test_rows_sum_to_one():
    for causal in (False, True):
        q, k = rnd(30, 2, 4, 11, 5) * 3, rnd(31, 2, 2, 11, 5) * 3
        P = oracle.softmax_weights(q, k, 0.4, causal)
        assert np.max(np.abs(P.sum(axis=-1) - 1.0)) <= TOL
        if causal:
            assert np.all(np.triu(P[0, 0], 1) == 0.0)


def test_tiny_workload_matches_brute():
    """The whole tiny fp32 prefill (B=1, H=2, N=64, d=16) against pure Python."""
    case = TINY_PREFILL
    raw = prefill_inputs(case)
    q, k, v = (oracle.decode_bits(raw[n], case.dtype) for n in ("q", "k", "v"))
    O, L = oracle.one_shot(q, k, v, case.sm_scale, case.causal)
    Ob, Lb = oracle.brute_attention(q.tolist(), k.tolist(), v.tolist(), case.sm_scale, case.causal)
    assert np.max(np.abs(O - np.array(Ob))) <= TOL
    assert np.max(np.abs(L - np.array(Lb))) <= TOL


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_one_shot_every_tile(causal):
    """The pages' claim: the tiled online softmax reaches the one-shot result."""
    N = 13
    q, k, v = rnd(40, 2, 4, N, 6), rnd(41, 2, 2, N, 6), rnd(42, 2, 2, N, 6)
    O, L = oracle.one_shot(q, k, v, 0.45, causal)
    for tile in range(1, N + 2):
        Ot, Lt = oracle.tiled(q, k, v, 0.45, causal, tile=tile)
        assert np.max(np.abs(Ot - O)) <= TOL, tile
        assert np.max(np.abs(Lt - L)) <= TOL, tile


@pytest.mark.parametrize("causal", [False, True])
def test_splitk_equals_one_shot_every_split(causal):
    N = 11
    q, k, v = rnd(43, 1, 4, N, 5), rnd(44, 1, 2, N, 5), rnd(45, 1, 2, N, 5)
    O, L = oracle.one_shot(q, k, v, 0.6, causal)
    for split in range(1, N + 2):
        Os, Ls = oracle.splitk_merge(q, k, v, 0.6, split, causal)
        assert np.max(np.abs(Os - O)) <= TOL, split
        assert np.max(np.abs(Ls - L)) <= TOL, split


def test_attention_rows_match_one_shot():
    q, k, v = rnd(46, 2, 4, 9, 5), rnd(47, 2, 2, 9, 5), rnd(48, 2, 2, 9, 5)
    for causal in (False, True):
        O, L = oracle.one_shot(q, k, v, 0.7, causal)
        rows = [(b, h, i) for b in range(2) for h in range(4) for i in (0, 4, 8)]
        Or, Lr = oracle.attention_rows(q, k, v, 0.7, rows, causal)
        for r, (b, h, i) in enumerate(rows):
            assert np.max(np.abs(Or[r] - O[b, h, i])) <= TOL
            assert abs(Lr[r] - L[b, h, i]) <= TOL


def test_large_scores_stay_finite():
    """Scores of order 1e4 must not overflow: the max shift keeps exp in range."""
    q, k, v = rnd(49, 1, 1, 4, 3) * 100, rnd(50, 1, 1, 4, 3) * 100, rnd(51, 1, 1, 4, 3)
    for fn in (oracle.one_shot, lambda *a: oracle.tiled(*a, tile=2)):
        O, L = fn(q, k, v, 1.0, False)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))


# ---------------------------------------------------------------------------
# planted mistakes: each must fail at least one pin
# ---------------------------------------------------------------------------
def _mutants():
    def no_scale(q, k, v, s, c):
        return oracle.one_shot(q, k, v, 1.0, c)

    def swapped_kv(q, k, v, s, c):
        return oracle.one_shot(q, v, k, s, c)

    def transposed_mask(q, k, v, s, c):
        O, L = oracle.one_shot(q, k, v, s, False)
        if not c:
            return O, L
        # strictly-lower mask (drops the diagonal key)
        B, H, N, d = q.shape
        vis = np.tril(np.ones((N, N), bool), -1)
        O2, L2 = np.zeros_like(O), np.zeros_like(L)
        for b in range(B):
            for h in range(H):
                g = h // (H // k.shape[1])
                O2[b, h], L2[b, h], _ = oatt._softmax_attend(s * q[b, h] @ k[b, g].T, vis, v[b, g])
        return O2, L2

    def modulo_heads(q, k, v, s, c):
        H, Hk = q.shape[1], k.shape[1]
        idx = [h % Hk for h in range(H)]
        return oracle.one_shot(q, k[:, idx], v[:, idx], s, c)

    def ln2_lse(q, k, v, s, c):
        O, L = oracle.one_shot(q, k, v, s, c)
        return O, L / math.log(2)

    def no_renorm(q, k, v, s, c):
        # forgets to divide by the softmax denominator
        O, L = oracle.one_shot(q, k, v, s, c)
        return O * np.exp(L - L.max())[..., None], L

    def stale_max(q, k, v, s, c):
        # the per-tile-max mistake: rescales by sums only, never by a carried max
        B, H, N, d = q.shape
        out = np.zeros((B, H, N, v.shape[-1]))
        Ls = np.zeros((B, H, N))
        G = H // k.shape[1]
        for b in range(B):
            for h in range(H):
                g = h // G
                acc = np.zeros((N, v.shape[-1]))
                l = np.zeros(N)
                for j in range(N):
                    sc = s * q[b, h] @ k[b, g, j]
                    mask = (np.arange(N) >= j) if c else np.ones(N, bool)
                    p = np.where(mask, 1.0, 0.0)  # exp(s - per-block max) with block 1
                    newl = l + p
                    acc = np.where((newl > 0)[:, None],
                                   acc * np.where(newl > 0, l / np.where(newl > 0, newl, 1), 0)[:, None]
                                   + p[:, None] * v[b, g, j], 0)
                    l = newl
                    del sc
                out[b, h] = acc
                Ls[b, h] = np.log(np.maximum(l, 1e-300))
        return out, Ls

    return {"no_scale": no_scale, "swapped_kv": swapped_kv, "transposed_mask": transposed_mask,
            "modulo_heads": modulo_heads, "ln2_lse": ln2_lse, "no_renorm": no_renorm,
            "stale_max": stale_max}


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_pins_have_teeth(name):
    fn = _mutants()[name]
    failed = []
    for pin in PINS:
        try:
            pin(fn)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name!r} passed every pin"

"""Pins of the fp64 oracle against facts other than itself.

Each test checks the oracle against one of: an independent scalar-loop
implementation (tests/bruteforce.py), a closed form, an invariant that the
definition fixes, or a library routine in a special case. Together they are
chosen so that a dropped term, a wrong sign, a wrong index or a transposed
operand anywhere in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import FULL, SLIDING, LayerSpec
from tests import bruteforce


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _inputs(B, T, Hq, Hkv, D, seed):
    return (_rand((B, T, Hq, D), seed), _rand((B, T, Hkv, D), seed + 1),
            _rand((B, T, Hkv, D), seed + 2), _rand((B, T, Hq), seed + 3))


CASES = [
    # layer_type, W, Hq, Hkv, D, theta, fraction, scale, T
    (SLIDING, 1, 2, 1, 4, 10.0, 1.0, None, 7),
    (SLIDING, 3, 4, 2, 8, 1e4, 1.0, None, 16),
    (SLIDING, 5, 4, 1, 8, 10.0, 0.5, 0.3, 13),
    (FULL, 0, 4, 4, 4, 100.0, 1.0, None, 11),
    (FULL, 0, 4, 1, 8, 5e6, 0.5, None, 16),
    (FULL, 0, 2, 1, 8, 0.0, 1.0, None, 9),
    (SLIDING, 16, 2, 2, 4, 1e4, 1.0, 1.7, 10),
]


@pytest.mark.parametrize("idx", range(len(CASES)))
def test_bruteforce_agreement(idx):
    lt, W, Hq, Hkv, D, theta, f, scale, T = CASES[idx]
    layer = LayerSpec(lt, W, Hq, Hkv, D, theta, f, scale)
    q, k, v, g = _inputs(2, T, Hq, Hkv, D, seed=100 + 10 * idx)
    y = oracle.prefill(q, k, v, g, layer)
    yb = np.array(bruteforce.prefill(q.tolist(), k.tolist(), v.tolist(), g.tolist(),
                                     lt == SLIDING, W, Hq // Hkv, theta, f, scale))
    np.testing.assert_allclose(y, yb, rtol=0, atol=1e-12)
    # the row-sampled form of the definition agrees with the brute force too
    rows = [(b, t, h) for b in range(2) for t in (0, T // 2, T - 1) for h in range(Hq)]
    yr = oracle.prefill_rows(q, k, v, g, layer, rows)
    np.testing.assert_allclose(yr, np.array([yb[b, t, h] for b, t, h in rows]),
                               rtol=0, atol=1e-12)


def test_window_one_returns_gated_value():
    layer = LayerSpec(SLIDING, 1, 4, 2, 8, 1e4, 1.0)
    q, k, v, g = _inputs(1, 20, 4, 2, 8, 5)
    y = oracle.prefill(q, k, v, g, layer)
    sig = 1.0 / (1.0 + np.exp(-g))
    for h in range(4):
        expect = sig[:, :, h, None] * v[:, :, h // 2, :]
        np.testing.assert_allclose(y[:, :, h], expect, rtol=1e-15, atol=0)


@pytest.mark.parametrize("W", [40, 41, 100])
def test_window_at_least_T_is_full_causal(W):
    T = 40
    q, k, v, g = _inputs(1, T, 4, 1, 8, 7)
    ys = oracle.prefill(q, k, v, g, LayerSpec(SLIDING, W, 4, 1, 8, 1e4, 1.0))
    yf = oracle.prefill(q, k, v, g, LayerSpec(FULL, 0, 4, 1, 8, 1e4, 1.0))
    np.testing.assert_array_equal(ys, yf)


@pytest.mark.parametrize("lt,W", [(SLIDING, 1), (SLIDING, 6), (SLIDING, 25), (FULL, 0)])
def test_uniform_scores_average_the_window(lt, W):
    """Q = 0 makes every visible score equal, so attention is the plain mean
    of the min(i+1, W) visible values: pins the window count exactly."""
    T, Hq, Hkv, D = 30, 2, 1, 4
    q, k, v, g = _inputs(1, T, Hq, Hkv, D, 11)
    q[:] = 0.0
    y = oracle.prefill(q, k, v, g, LayerSpec(lt, W, Hq, Hkv, D, 1e4, 1.0))
    for i in range(T):
        lo = 0 if lt == FULL else max(0, i - W + 1)
        mean = v[0, lo:i + 1, 0].mean(axis=0)
        for h in range(Hq):
            sig = 1.0 / (1.0 + math.exp(-g[0, i, h]))
            np.testing.assert_allclose(y[0, i, h], sig * mean, rtol=1e-13, atol=1e-15)


def test_hidden_keys_do_not_change_a_row():
    T, W, i = 24, 5, 13
    layer = LayerSpec(SLIDING, W, 2, 1, 8, 1e4, 1.0)
    q, k, v, g = _inputs(1, T, 2, 1, 8, 13)
    base = oracle.prefill(q, k, v, g, layer)
    for j in list(range(0, i - W + 1)) + list(range(i + 1, T)):
        k2, v2 = k.copy(), v.copy()
        k2[0, j] += 3.0
        v2[0, j] -= 2.0
        y = oracle.prefill(q, k2, v2, g, layer)
        np.testing.assert_array_equal(y[0, i], base[0, i])
    # a key inside the window does change the row
    k2 = k.copy()
    k2[0, i - W + 1] += 3.0
    assert not np.array_equal(oracle.prefill(q, k2, v, g, layer)[0, i], base[0, i])


@pytest.mark.parametrize("lt,W", [(SLIDING, 7), (FULL, 0)])
def test_probabilities_and_convex_hull(lt, W):
    T = 33
    layer = LayerSpec(lt, W, 4, 2, 8, 1e4, 0.5)
    q, k, v, g = _inputs(1, T, 4, 2, 8, 17)
    y, p = oracle.prefill(q, k, v, g, layer, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=-1), 1.0, rtol=0, atol=1e-12)
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    hidden = ~oracle.visible(i, j, layer)
    assert np.all(p[:, :, hidden] == 0.0)
    sig = 1.0 / (1.0 + np.exp(-g))
    for t in range(T):
        lo = 0 if lt == FULL else max(0, t - W + 1)
        for h in range(4):
            a = y[0, t, h] / sig[0, t, h]
            vv = v[0, lo:t + 1, h // 2]
            assert np.all(a <= vv.max(axis=0) + 1e-12)
            assert np.all(a >= vv.min(axis=0) - 1e-12)


# ---------------------------------------------------------------- RoPE pins

def test_rope_closed_form_frequencies():
    """theta = 16, r = 4: omega = (16^0, 16^(-1/2)) = (1, 1/4), worked by hand.
    Dim 1 pairs with dim 3; dims 4..7 pass through."""
    D = 8
    e1 = np.zeros(D)
    e1[1] = 1.0
    y = oracle.rope(e1, 2.0, 16.0, 4)
    expect = np.zeros(D)
    expect[1] = math.cos(0.5)
    expect[3] = math.sin(0.5)
    np.testing.assert_allclose(y, expect, rtol=0, atol=1e-15)
    e0 = np.zeros(D)
    e0[0] = 1.0
    y0 = oracle.rope(e0, 3.0, 16.0, 4)
    expect0 = np.zeros(D)
    expect0[0] = math.cos(3.0)
    expect0[2] = math.sin(3.0)
    np.testing.assert_allclose(y0, expect0, rtol=0, atol=1e-15)
    x = np.arange(1.0, 9.0)
    np.testing.assert_array_equal(oracle.rope(x, 5.0, 16.0, 4)[4:], x[4:])


def test_rope_score_is_cosine_of_offset():
    """q = k = e_0 with r = D: score = scale * cos((a - b) * omega_0), omega_0 = 1."""
    D = 8
    layer = LayerSpec(FULL, 0, 1, 1, D, 1e4, 1.0)
    e0 = np.zeros(D)
    e0[0] = 1.0
    for a, b in [(5, 2), (100, 3), (131071, 65536)]:
        s = oracle.rope(e0, a, 1e4, D) @ oracle.rope(e0, b, 1e4, D) * layer.scale
        assert abs(s - layer.scale * math.cos(a - b)) < 1e-10


def test_rope_depends_only_on_relative_offset():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(128), rng.standard_normal(128)
    for theta, r in [(1e4, 128), (5e6, 64), (5e5, 128)]:
        base = oracle.rope(q, 37.0, theta, r) @ oracle.rope(k, 11.0, theta, r)
        for shift in [1, 1000, 131000]:
            s = oracle.rope(q, 37.0 + shift, theta, r) @ oracle.rope(k, 11.0 + shift, theta, r)
            assert abs(s - base) < 1e-9


def test_rope_identities_and_norms():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((5, 16))
    np.testing.assert_array_equal(oracle.rope(x, 123.0, 0.0, 16), x)      # base 0
    np.testing.assert_array_equal(oracle.rope(x, 123.0, 1e4, 0), x)       # r = 0
    np.testing.assert_allclose(oracle.rope(x, 0.0, 1e4, 16), x, rtol=0, atol=0)  # p = 0
    y = oracle.rope(x, np.arange(5.0)[:, None][:, 0], 1e4, 8)
    np.testing.assert_array_equal(y[:, 8:], x[:, 8:])
    for i in range(4):
        n_in = x[:, i] ** 2 + x[:, i + 4] ** 2
        n_out = y[:, i] ** 2 + y[:, i + 4] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=1e-14)


def test_rope_matches_complex_rotation():
    """Half-split RoPE as a complex product: (x_i + i x_{i+r/2}) * e^{i p w_i}."""
    rng = np.random.default_rng(5)
    D, r, theta = 16, 12, 5e6
    x = rng.standard_normal((9, D))
    pos = np.arange(9.0) * 4097.0
    z = torch.complex(torch.tensor(x[:, :r // 2]), torch.tensor(x[:, r // 2:r]))
    w = torch.tensor([theta ** (-2.0 * i / r) for i in range(r // 2)], dtype=torch.float64)
    rot = torch.polar(torch.ones(9, r // 2, dtype=torch.float64), torch.tensor(pos)[:, None] * w)
    zr = z * rot
    y = oracle.rope(x, pos, theta, r)
    np.testing.assert_allclose(y[:, :r // 2], zr.real.numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(y[:, r // 2:r], zr.imag.numpy(), rtol=0, atol=1e-12)


# ------------------------------------------------------------ GQA and gate

def test_gqa_equals_mha_with_repeated_kv():
    B, T, Hkv, G, D = 1, 20, 2, 3, 8
    q, k, v, g = _inputs(B, T, Hkv * G, Hkv, D, 21)
    y = oracle.prefill(q, k, v, g, LayerSpec(SLIDING, 6, Hkv * G, Hkv, D, 1e4, 1.0))
    kr = np.repeat(k, G, axis=2)
    vr = np.repeat(v, G, axis=2)
    ym = oracle.prefill(q, kr, vr, g, LayerSpec(SLIDING, 6, Hkv * G, Hkv * G, D, 1e4, 1.0))
    np.testing.assert_array_equal(y, ym)


def test_gate_half_at_zero_and_linear():
    layer = LayerSpec(FULL, 0, 2, 1, 8, 1e4, 1.0)
    q, k, v, g = _inputs(1, 12, 2, 1, 8, 23)
    y0 = oracle.prefill(q, k, v, np.zeros_like(g), layer)
    assert oracle.sigmoid(0.0) == 0.5
    y = oracle.prefill(q, k, v, g, layer)
    sig = 1.0 / (1.0 + np.exp(-g))
    np.testing.assert_allclose(y, 2.0 * y0 * sig[..., None], rtol=1e-14, atol=1e-16)


# ------------------------------------------------- library special case

def _sdpa_reference(q, k, v, g, G, mask):
    qt = torch.tensor(q[0]).permute(1, 0, 2)                 # [Hq,T,D]
    kt = torch.tensor(np.repeat(k[0], G, axis=1)).permute(1, 0, 2)
    vt = torch.tensor(np.repeat(v[0], G, axis=1)).permute(1, 0, 2)
    a = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, attn_mask=torch.tensor(mask))
    a = a.permute(1, 0, 2).numpy()
    return torch.sigmoid(torch.tensor(g[0])).numpy()[..., None] * a


@pytest.mark.parametrize("lt,W", [(FULL, 0), (SLIDING, 9)])
def test_matches_sdpa_without_rotation(lt, W):
    T, Hkv, G, D = 50, 2, 4, 16
    q, k, v, g = _inputs(1, T, Hkv * G, Hkv, D, 29)
    y = oracle.prefill(q, k, v, g, LayerSpec(lt, W, Hkv * G, Hkv, D, 0.0, 1.0))
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    mask = j <= i
    if lt == SLIDING:
        mask &= (i - j) < W
    ref = _sdpa_reference(q, k, v, g, G, mask)
    np.testing.assert_allclose(y[0], ref, rtol=0, atol=1e-12)


# ------------------------------------------------------- decode and cache

# llama3 scaling with a short original context (16 positions), so that on a
# 16-dim head with r = 8 the first pair is blended and the others divided by
# the factor (wavelengths 6.3, 298, 1.4e4, 6.6e5 against 16/4 and 16/1)
SCALED = (2.0, 1.0, 4.0, 16)


@pytest.mark.parametrize("lt,W,f,theta,sc", [(FULL, 0, 0.5, 5e6, None), (SLIDING, 8, 1.0, 1e4, None),
                                             (SLIDING, 64, 1.0, 1e4, None),
                                             (FULL, 0, 0.5, 5e6, SCALED),
                                             (FULL, 0, 1.0, 1e4, (3.0, 1.0, 8.0, 64))])
def test_decode_equals_last_prefill_row(lt, W, f, theta, sc):
    """Decode over a cache that kv_append filled equals the last prefill row:
    with frequency scaling the cache's keys, the decode query and prefill's
    queries and keys must all use the same rescaled frequencies."""
    B, L, Hq, Hkv, D = 2, 29, 4, 2, 16
    layer = LayerSpec(lt, W, Hq, Hkv, D, theta, f, rope_scaling=sc)
    q, k, v, g = _inputs(B, L, Hq, Hkv, D, 31)
    cap = W if lt == SLIDING else 40
    kc = np.zeros((B, Hkv, cap, D))
    vc = np.zeros((B, Hkv, cap, D))
    kc, vc = oracle.kv_append(kc, vc, k, v, np.zeros(B, dtype=int), layer)
    yd = oracle.decode(q[:, L - 1], g[:, L - 1], kc, vc, np.full(B, L), layer)
    yp = oracle.prefill(q, k, v, g, layer)
    np.testing.assert_allclose(yd, yp[:, L - 1], rtol=0, atol=1e-12)


def test_decode_with_appends_in_pieces():
    """Appending in several calls and decoding at every length reproduces
    every prefill row, through several wraps of a small ring."""
    B, T, Hq, Hkv, D, W = 1, 23, 2, 1, 8, 4
    layer = LayerSpec(SLIDING, W, Hq, Hkv, D, 1e4, 1.0)
    q, k, v, g = _inputs(B, T, Hq, Hkv, D, 37)
    yp = oracle.prefill(q, k, v, g, layer)
    kc = np.zeros((B, Hkv, W, D))
    vc = np.zeros((B, Hkv, W, D))
    for p in range(T):
        kc, vc = oracle.kv_append(kc, vc, k[:, p:p + 1], v[:, p:p + 1], np.array([p]), layer)
        yd = oracle.decode(q[:, p], g[:, p], kc, vc, np.array([p + 1]), layer)
        np.testing.assert_allclose(yd, yp[:, p], rtol=0, atol=1e-12)


def test_scaled_full_layer_decode_with_appends_in_pieces():
    """A full layer with llama3 scaling, appended in uneven pieces (positions
    past the original context included) and decoded at each piece's end,
    reproduces the prefill rows; the scaling changes those rows."""
    B, T, Hq, Hkv, D = 1, 40, 4, 1, 16
    layer = LayerSpec(FULL, 0, Hq, Hkv, D, 5e6, 0.5, rope_scaling=SCALED)
    plain = LayerSpec(FULL, 0, Hq, Hkv, D, 5e6, 0.5)
    q, k, v, g = _inputs(B, T, Hq, Hkv, D, 43)
    yp = oracle.prefill(q, k, v, g, layer)
    assert np.abs(yp - oracle.prefill(q, k, v, g, plain)).max() > 1e-3
    kc = np.zeros((B, Hkv, T, D))
    vc = np.zeros((B, Hkv, T, D))
    cuts = [0, 1, 7, 8, 20, 33, 40]
    for a, b in zip(cuts[:-1], cuts[1:]):
        kc, vc = oracle.kv_append(kc, vc, k[:, a:b], v[:, a:b], np.array([a]), layer)
        yd = oracle.decode(q[:, b - 1], g[:, b - 1], kc, vc, np.array([b]), layer)
        np.testing.assert_allclose(yd, yp[:, b - 1], rtol=0, atol=1e-12)
    # the cache holds keys rotated at their positions with the rescaled frequencies
    om = oracle.llama3_frequencies(np.power(5e6, -2.0 * np.arange(4) / 8), *SCALED)
    p = 37
    ang = p * om
    x = k[0, p, 0]
    want = x.copy()
    want[:4] = x[:4] * np.cos(ang) - x[4:8] * np.sin(ang)
    want[4:8] = x[4:8] * np.cos(ang) + x[:4] * np.sin(ang)
    np.testing.assert_allclose(kc[0, 0, p], want, rtol=0, atol=1e-14)


def test_ring_at_least_as_long_as_history_equals_full_cache():
    B, L, Hq, Hkv, D = 1, 12, 2, 1, 8
    q, k, v, g = _inputs(B, L, Hq, Hkv, D, 41)
    ring = LayerSpec(SLIDING, 16, Hq, Hkv, D, 1e4, 1.0)
    full = LayerSpec(FULL, 0, Hq, Hkv, D, 1e4, 1.0)
    z = np.zeros((B, Hkv, 16, D))
    kr, vr = oracle.kv_append(z, z, k, v, [0], ring)
    kf, vf = oracle.kv_append(z, z, k, v, [0], full)
    yr = oracle.decode(q[:, -1], g[:, -1], kr, vr, [L], ring)
    yf = oracle.decode(q[:, -1], g[:, -1], kf, vf, [L], full)
    np.testing.assert_array_equal(yr, yf)


def test_ring_slot_map_keeps_last_W_positions():
    """Position-tagged V rows: after appending positions s..s+n-1 with n > W,
    ring slot p mod W holds the highest such position."""
    W, Hkv, D = 8, 2, 4
    layer = LayerSpec(SLIDING, W, 2, Hkv, D, 1e4, 1.0)
    start, n = 13, 21
    vnew = np.zeros((1, n, Hkv, D))
    for t in range(n):
        vnew[0, t] = start + t
    kc, vc = oracle.kv_append(np.zeros((1, Hkv, W, D)), np.full((1, Hkv, W, D), -1.0),
                              np.zeros((1, n, Hkv, D)), vnew, [start], layer)
    for slot in range(W):
        expect = max(p for p in range(start, start + n) if p % W == slot)
        assert np.all(vc[0, :, slot] == expect)


def test_full_cache_slot_is_position():
    Hkv, D, cap = 1, 4, 30
    layer = LayerSpec(FULL, 0, 1, Hkv, D, 0.0, 1.0)
    n = 5
    knew = np.arange(2 * n * D, dtype=float).reshape(2, n, Hkv, D)
    vnew = -knew
    kc, vc = oracle.kv_append(np.zeros((2, Hkv, cap, D)), np.zeros((2, Hkv, cap, D)),
                              knew, vnew, [3, 17], layer)
    np.testing.assert_array_equal(kc[0, :, 3:8], knew[0].transpose(1, 0, 2))
    np.testing.assert_array_equal(vc[1, :, 17:22], vnew[1].transpose(1, 0, 2))
    assert np.all(kc[0, :, :3] == 0) and np.all(kc[0, :, 8:] == 0)
    with pytest.raises(ValueError):
        oracle.kv_append(kc, vc, knew, vnew, [27, 0], layer)


# ------------------------------------------------------------ rounding

def test_round_bf16_matches_library_and_ties():
    rng = np.random.default_rng(7)
    x = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    lib = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(x.astype(np.float64)), lib)
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0                  # tie to even
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6  # tie to even (up)
    assert oracle.round_bf16(-(1.0 + 2.0 ** -8 + 2.0 ** -40)) == -(1.0 + 2.0 ** -7)


# ---- "llama3" frequency scaling of the full layers ([P1] 2.3; parameters
# other than the factor are readings, see the oracle's header)

def test_llama3_frequencies_regimes_by_hand():
    N, f = 1000.0, 2.0
    w = lambda wavelength: 2.0 * np.pi / wavelength
    got = oracle.llama3_frequencies(np.array([w(200.0), w(2000.0), w(400.0)]), f, 1.0, 4.0, N)
    # wavelength N/5 < N/4 keeps w; 2N > N halves it; N/2.5 blends with s = 0.5
    np.testing.assert_allclose(got, [w(200.0), w(2000.0) / 2.0, 0.75 * w(400.0)], rtol=1e-15)


def test_llama3_frequencies_identity_and_continuity():
    w = 2.0 * np.pi / np.geomspace(10.0, 1e6, 200)
    np.testing.assert_array_equal(oracle.llama3_frequencies(w, 1.0, 1.0, 4.0, 8192.0), w)
    N = 8192.0
    for edge, expect in ((N / 4.0, 1.0), (N, 0.5)):     # blend meets both plain regimes
        we = 2.0 * np.pi / edge
        for eps in (1 - 1e-9, 1 + 1e-9):
            got = oracle.llama3_frequencies(np.array([we * eps]), 2.0, 1.0, 4.0, N)[0]
            assert abs(got / (we * eps) - expect) < 1e-6


def test_llama3_frequencies_stay_ordered():
    i = np.arange(32.0)
    w = 5e6 ** (-2.0 * i / 64.0)
    s = oracle.llama3_frequencies(w, 2.0, 1.0, 4.0, 131072.0)
    assert np.all(np.diff(s) < 0)
    assert np.all(s <= w) and np.all(s >= w / 2.0)


def test_scaled_rope_scores_depend_only_on_offset():
    rng = np.random.default_rng(7)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    sc = (2.0, 1.0, 4.0, 64.0)
    base = oracle.rope(q, 37.0, 1e4, 64, sc) @ oracle.rope(k, 11.0, 1e4, 64, sc)
    for shift in (1.0, 250.0, 1e5):
        s = oracle.rope(q, 37.0 + shift, 1e4, 64, sc) @ oracle.rope(k, 11.0 + shift, 1e4, 64, sc)
        assert abs(s - base) < 1e-9 * max(1.0, abs(base))
    plain = oracle.rope(q, 37.0, 1e4, 64) @ oracle.rope(k, 11.0, 1e4, 64)
    assert abs(plain - base) > 1e-3          # the scaling does change scores


def test_scaling_applies_to_full_layers_only():
    rng = np.random.default_rng(8)
    B, T, Hq, Hkv, D = 1, 40, 2, 1, 16
    q, k, v = (rng.standard_normal((B, T, h, D)) for h in (Hq, Hkv, Hkv))
    g = rng.standard_normal((B, T, Hq))
    sc = (2.0, 1.0, 4.0, 16.0)
    s_plain = oracle.prefill(q, k, v, g, LayerSpec(SLIDING, 8, Hq, Hkv, D, 1e4, 1.0))
    s_sc = oracle.prefill(q, k, v, g, LayerSpec(SLIDING, 8, Hq, Hkv, D, 1e4, 1.0, None, sc))
    np.testing.assert_array_equal(s_plain, s_sc)
    f_plain = oracle.prefill(q, k, v, g, LayerSpec(FULL, 0, Hq, Hkv, D, 1e4, 1.0))
    f_sc = oracle.prefill(q, k, v, g, LayerSpec(FULL, 0, Hq, Hkv, D, 1e4, 1.0, None, sc))
    assert np.abs(f_plain - f_sc).max() > 1e-3

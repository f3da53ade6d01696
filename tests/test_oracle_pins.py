"""Pins for the CPU oracle (runs without a GPU).

Each test ties a part of the oracle to something other than the oracle's own
formulas: library casts (numpy / torch), exact integer arithmetic, the exact
erf-based GeLU with the tanh approximation's known error bound, fp64
evaluation within a derived rounding bound, and algebraic invariants of the
chain (identity W2, zero X, scaling and additivity in W2, row independence).
A plausible mistake anywhere in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong constant, a wrong rounding rule) fails
at least one of them.
"""
import math

import numpy as np
import pytest
import torch
from scipy.special import erf, expit

from consumer_gemm_chain_amd import gen

U32 = 2.0 ** -24


# ----------------------------------------------------------------- helpers

def f16_bits_all():
    return np.arange(65536, dtype=np.uint32).astype(np.uint16)


def torch_bf16_to_f32(bits):
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)
    return t.to(torch.float32).numpy()


def torch_f32_to_bf16(vals):
    t = torch.from_numpy(np.ascontiguousarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def ulp(v, dtype):
    """Spacing of the storage format at |v| (fp64 array)."""
    a = np.abs(np.asarray(v, np.float64))
    if dtype == "f16":
        e = np.floor(np.log2(np.maximum(a, 2.0 ** -14)))
        return 2.0 ** (e - 10)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def widen_lib(bits, dtype):
    return gen.from_bits(bits, dtype).astype(np.float64)


def gamma(n):
    return n * U32 / (1 - n * U32)


# ------------------------------------------------------- storage formats

def test_widen_f16_exhaustive(oracle_mod):
    b = f16_bits_all()
    got = oracle_mod.widen(b, "f16")
    ref = b.view(np.float16).astype(np.float32)
    nan = np.isnan(ref)
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_widen_bf16_exhaustive(oracle_mod):
    b = f16_bits_all()
    got = oracle_mod.widen(b, "bf16")
    ref = torch_bf16_to_f32(b)
    nan = np.isnan(ref)
    assert np.isnan(got[nan]).all()
    assert np.array_equal(got[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def _rounding_probe_values(dtype):
    """Every finite value of the format, every midpoint between neighbours
    (the tie cases) and the fp32 neighbours of each midpoint, both signs,
    plus 2^22 random fp32 bit patterns."""
    b = f16_bits_all()
    if dtype == "f16":
        v = b.view(np.float16).astype(np.float64)
    else:
        v = torch_bf16_to_f32(b).astype(np.float64)
    v = np.unique(v[np.isfinite(v) & (v >= 0)])
    mids = (v[:-1] + v[1:]) / 2.0                      # exact in fp32 for both formats
    mids32 = mids.astype(np.float32)
    assert np.array_equal(mids32.astype(np.float64), mids)
    up = np.nextafter(mids32, np.float32(np.inf))
    dn = np.nextafter(mids32, np.float32(0))
    rnd = np.random.Generator(np.random.PCG64(7)).integers(0, 2 ** 32, size=1 << 22, dtype=np.uint32)
    rnd = rnd.view(np.float32)
    allv = np.concatenate([v.astype(np.float32), mids32, up, dn, rnd,
                           np.array([65504, 65519.996, 65520, 65536, 1e30, np.inf, -0.0, 0.0,
                                     2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -149],
                                    np.float32)])
    allv = np.concatenate([allv, -allv])
    return allv[~np.isnan(allv)]


def test_round_f16_against_numpy(oracle_mod):
    vals = _rounding_probe_values("f16")
    got = oracle_mod.round_to(vals, "f16")
    ref = vals.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_round_bf16_against_torch(oracle_mod):
    vals = _rounding_probe_values("bf16")
    got = oracle_mod.round_to(vals, "bf16")
    ref = torch_f32_to_bf16(vals)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, (vals[bad[:5]], got[bad[:5]], ref[bad[:5]])


def test_round_nan_stays_nan(oracle_mod):
    vals = np.array([np.nan, -np.nan], np.float32)
    for dt in ("f16", "bf16"):
        back = oracle_mod.widen(oracle_mod.round_to(vals, dt), dt)
        assert np.isnan(back).all()


# ------------------------------------------------------------ activations

GRID = np.concatenate([np.linspace(-12, 12, 400001), np.linspace(-0.01, 0.01, 20001)]).astype(np.float32)


def test_gelu_tanh_within_known_bound_of_exact_gelu(oracle_mod):
    # The tanh form approximates x*Phi(x) with a maximum absolute error of
    # about 4.73e-4 (near |x| = 2.7); a wrong constant (0.04 or 0.05 instead
    # of 0.044715, 0.8 instead of sqrt(2/pi), sqrt(pi/2)) exceeds 6e-4.
    x = GRID
    got = oracle_mod.act(x, "gelu_tanh").astype(np.float64)
    x64 = x.astype(np.float64)
    exact = 0.5 * x64 * (1.0 + erf(x64 / math.sqrt(2.0)))
    tol = 4.75e-4 + 8 * U32 * np.maximum(1.0, np.abs(x64))
    assert np.all(np.abs(got - exact) <= tol), np.max(np.abs(got - exact))
    assert np.max(np.abs(got - exact)) > 4.5e-4        # it is the tanh form, not erf


def test_gelu_odd_part_identity(oracle_mod):
    # 0.5x(1+tanh(s(x))) - 0.5(-x)(1+tanh(s(-x))) = x for odd s: a sign or
    # factor mistake breaks this.
    x = GRID
    gp = oracle_mod.act(x, "gelu_tanh").astype(np.float64)
    gm = oracle_mod.act(-x, "gelu_tanh").astype(np.float64)
    tol = 6 * U32 * np.maximum(np.abs(x), 1e-30) + 1e-37
    assert np.all(np.abs((gp - gm) - x.astype(np.float64)) <= tol)


def test_gelu_special_values(oracle_mod):
    x = np.array([0.0, -0.0, 10.0, 20.0, 1e4, -10.0, -20.0, -1e4], np.float32)
    g = oracle_mod.act(x, "gelu_tanh")
    assert g[0] == 0 and g[1] == 0
    assert np.array_equal(g[2:5], x[2:5])               # tanh saturates to 1
    assert np.all(g[5:] == 0)                           # tanh saturates to -1


def test_silu_against_library_logistic(oracle_mod):
    g = GRID
    u = np.ones_like(g)
    got = oracle_mod.act(g, "swiglu", u).astype(np.float64)
    g64 = g.astype(np.float64)
    ref = g64 * expit(g64)
    assert np.all(np.abs(got - ref) <= 6 * U32 * np.abs(ref) + 1e-38)


def test_swiglu_uses_up_as_plain_factor(oracle_mod):
    r = np.random.Generator(np.random.PCG64(3))
    g = r.standard_normal(10000).astype(np.float32) * 4
    u = r.standard_normal(10000).astype(np.float32) * 4
    got = oracle_mod.act(g, "swiglu", u).astype(np.float64)
    ref = (g.astype(np.float64) * expit(g.astype(np.float64))) * u.astype(np.float64)
    assert np.all(np.abs(got - ref) <= 8 * U32 * np.abs(ref) + 1e-38)
    # silu odd-part identity: silu(g) - silu(-g) = g
    one = np.ones_like(g)
    d = oracle_mod.act(g, "swiglu", one).astype(np.float64) - oracle_mod.act(-g, "swiglu", one).astype(np.float64)
    assert np.all(np.abs(d - g) <= 8 * U32 * np.abs(g) + 1e-38)
    assert np.all(oracle_mod.act(g, "swiglu", np.zeros_like(g)) == 0)


def test_act_none_is_identity(oracle_mod):
    x = GRID
    assert np.array_equal(oracle_mod.act(x, "none"), x)


# ------------------------------------------------------------------- chain

def _int_bits(shape, seed, lo, hi, density, dtype):
    r = np.random.Generator(np.random.PCG64(seed))
    v = r.integers(lo, hi + 1, size=shape).astype(np.float32)
    v[r.random(shape) >= density] = 0
    return gen.to_bits(v, dtype), v.astype(np.int64)


def _lib_round(vals_int64, dtype):
    """Library RNE of exact integers (numpy / torch casts)."""
    f = vals_int64.astype(np.float64)
    if dtype == "f16":
        return f.astype(np.float16).view(np.uint16)
    return torch_f32_to_bf16(f.astype(np.float32))   # |v| < 2^24: exact in fp32


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("M,H,I", [(7, 40, 24), (3, 512, 96), (16, 64, 200)])
def test_exact_integer_chain(oracle_mod, dtype, M, H, I):
    """Integer inputs whose partial sums are exact in fp32: the oracle must
    equal exact int64 matrix products followed by the library's rounding,
    bit for bit.  Non-square shapes catch transposed operands; large
    integers make both roundings (T and Y) non-trivial."""
    # integer range chosen so that |h| has a std of about 3000 (fp16) or 400
    # (bf16): well past 2048 / 256, where the formats start to round integers
    target = 9000.0 if dtype == "f16" else 1200.0
    hi = max(2, int(round(math.sqrt(target / math.sqrt(0.9 * H)))))
    x, xi = _int_bits((M, H), 11, -hi, hi, 0.9, dtype)
    w1, w1i = _int_bits((H, I), 12, -hi, hi, 0.9, dtype)
    w2, w2i = _int_bits((I, H), 13, -1, 1, 0.05 if dtype == "f16" else 0.5, dtype)
    h = xi @ w1i
    assert np.abs(np.abs(xi) @ np.abs(w1i)).max() < 2 ** 24
    t_ref = _lib_round(h, dtype)
    t_int = widen_lib(t_ref, dtype).astype(np.int64)
    assert np.array_equal(t_int.astype(np.float64), widen_lib(t_ref, dtype))   # integers
    yv = t_int @ w2i
    assert (np.abs(t_int) @ np.abs(w2i)).max() < 2 ** 24
    if dtype == "f16":
        assert np.abs(yv).max() < 65504
    y_ref = _lib_round(yv, dtype)
    y, t = oracle_mod.mlp_chain(x, w1, w2, "none", dtype, want_t=True)
    assert np.array_equal(t, t_ref)
    assert np.array_equal(y, y_ref)
    # the rounding of T was actually exercised
    assert np.any(t_int != h)


@pytest.mark.parametrize("act", ["gelu_tanh", "swiglu"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_activation_wiring_on_exact_accumulators(oracle_mod, act, dtype):
    """With integer X and W1 the first GEMM is exact, so T must equal the
    (separately pinned) activation applied to the exact int64 product, with
    gate = columns [0, I) and up = columns [I, 2I) for SwiGLU."""
    M, H, I = 5, 64, 48
    g = 2 if act == "swiglu" else 1
    x, xi = _int_bits((M, H), 21, -2, 2, 0.5, dtype)
    w1, w1i = _int_bits((H, g * I), 22, -2, 2, 0.5, dtype)
    w2 = gen.normal_bits((I, H), 23, 0.05, dtype)
    h = (xi @ w1i).astype(np.float32)
    if act == "swiglu":
        a = oracle_mod.act(h[:, :I], "swiglu", h[:, I:])
        # swapping gate and up gives a different T: the test can tell them apart
        a_swapped = oracle_mod.act(h[:, I:], "swiglu", h[:, :I])
        assert not np.array_equal(oracle_mod.round_to(a, dtype), oracle_mod.round_to(a_swapped, dtype))
    else:
        a = oracle_mod.act(h, act)
    _, t = oracle_mod.mlp_chain(x, w1, w2, act, dtype, want_t=True)
    assert np.array_equal(t, oracle_mod.round_to(a, dtype))
    # and T round-trips through the library's cast the same way
    assert np.array_equal(t, gen.to_bits(a, dtype))


ACTS = ["none", "gelu_tanh", "swiglu"]
DTS = ["f16", "bf16"]


def _act64(h, act, I):
    if act == "none":
        return h
    if act == "gelu_tanh":
        return 0.5 * h * (1.0 + erf(h / math.sqrt(2.0)))   # exact GeLU; tanh-form error added below
    g, u = h[:, :I], h[:, I:]
    return g * expit(g) * u


def _act_lipschitz(h, act, I):
    if act == "none":
        return np.ones_like(h), 0.0
    if act == "gelu_tanh":
        return np.full_like(h, 1.13), 4.75e-4
    g, u = h[:, :I], h[:, I:]
    dsilu = 1.1
    return (np.abs(u) * dsilu, np.abs(g * expit(g)) + 1.0), 0.0


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", DTS)
def test_chain_within_fp64_rounding_bound(oracle_mod, act, dtype):
    """Normal inputs: the oracle's T and Y lie within a rigorous rounding
    bound of an fp64 evaluation with library matmuls (numpy float64),
    the exact erf GeLU (plus the tanh form's 4.75e-4 approximation bound) and
    the library logistic."""
    M, H, I = 6, 320, 136
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, seed=5)
    y, t = oracle_mod.mlp_chain(x, w1, w2, act, dtype, want_t=True)
    X, W1, W2 = widen_lib(x, dtype), widen_lib(w1, dtype), widen_lib(w2, dtype)
    h = X @ W1
    dh = gamma(H) * (np.abs(X) @ np.abs(W1))
    a = _act64(h, act, I)
    lip, approx = _act_lipschitz(h, act, I)
    if act == "swiglu":
        da = lip[0] * dh[:, :I] + lip[1] * dh[:, I:] + 8 * U32 * np.abs(a)
    else:
        da = lip * dh + approx + 8 * U32 * np.abs(a)
    T = widen_lib(t, dtype)
    err_t = np.abs(T - a)
    bound_t = 0.5 * ulp(T, dtype) + da + 1e-30
    assert np.all(err_t <= bound_t), np.max(err_t / bound_t)
    # second GEMM, taking the oracle's own T as input
    y64 = T @ W2
    bound_y = 0.5 * ulp(y64, dtype) * 1.0001 + gamma(I) * (np.abs(T) @ np.abs(W2)) + 1e-30
    Y = widen_lib(y, dtype)
    assert np.all(np.abs(Y - y64) <= bound_y)
    # and the bound is tight enough to see a transposed or dropped term
    assert np.max(np.abs((T[:, ::-1] @ W2) - y64)) > 100 * np.max(bound_y)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", DTS)
def test_identity_w2_gives_intermediate(oracle_mod, act, dtype):
    M, H, I = 9, 96, 160
    x, w1, _ = gen.random_case(M, H, I, act, dtype, seed=8)
    eye = np.zeros((I, H), np.float32)
    eye[np.arange(H), np.arange(H)] = 1.0
    w2 = gen.to_bits(eye, dtype)
    y, t = oracle_mod.mlp_chain(x, w1, w2, act, dtype, want_t=True)
    yv, tv = widen_lib(y, dtype), widen_lib(t[:, :H], dtype)
    assert np.array_equal(yv, tv)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", DTS)
def test_zero_x_gives_zero(oracle_mod, act, dtype):
    M, H, I = 4, 64, 80
    _, w1, w2 = gen.random_case(M, H, I, act, dtype, seed=9)
    x = np.zeros((M, H), np.uint16)
    y = oracle_mod.mlp_chain(x, w1, w2, act, dtype)
    assert np.all(widen_lib(y, dtype) == 0)


@pytest.mark.parametrize("act", ACTS)
@pytest.mark.parametrize("dtype", DTS)
def test_linear_in_w2(oracle_mod, act, dtype):
    M, H, I = 8, 128, 72
    x, w1, w2 = gen.random_case(M, H, I, act, dtype, seed=10)
    W2 = widen_lib(w2, dtype)
    y1 = widen_lib(oracle_mod.mlp_chain(x, w1, w2, act, dtype), dtype)
    # scaling by a power of two is exact through fp32 sums and the rounding
    y2 = widen_lib(oracle_mod.mlp_chain(x, w1, gen.to_bits(W2 * 4.0, dtype), act, dtype), dtype)
    normal = np.abs(y1) >= (2.0 ** -14 if dtype == "f16" else 2.0 ** -126)
    assert np.array_equal(y2[normal], 4.0 * y1[normal])
    # additivity over a split of W2 into disjoint supports
    mask = np.random.Generator(np.random.PCG64(1)).random(W2.shape) < 0.5
    wa, wb = np.where(mask, W2, 0.0), np.where(mask, 0.0, W2)
    ya = widen_lib(oracle_mod.mlp_chain(x, w1, gen.to_bits(wa, dtype), act, dtype), dtype)
    yb = widen_lib(oracle_mod.mlp_chain(x, w1, gen.to_bits(wb, dtype), act, dtype), dtype)
    tol = (1e-2 if dtype == "f16" else 2e-2) * (1 + np.abs(y1))
    assert np.all(np.abs(ya + yb - y1) <= 2 * tol)


@pytest.mark.parametrize("act", ACTS)
def test_rows_are_independent(oracle_mod, act):
    M, H, I = 10, 64, 48
    x, w1, w2 = gen.random_case(M, H, I, act, "f16", seed=12)
    y = oracle_mod.mlp_chain(x, w1, w2, act, "f16")
    for r in (0, 3, 9):
        yr = oracle_mod.mlp_chain(x[r:r + 1], w1, w2, act, "f16")
        assert np.array_equal(yr[0], y[r])


def test_threads_do_not_change_result(oracle_mod):
    x, w1, w2 = gen.random_case(33, 96, 64, "gelu_tanh", "f16", seed=13)
    a = oracle_mod.mlp_chain(x, w1, w2, "gelu_tanh", "f16", nthreads=1)
    b = oracle_mod.mlp_chain(x, w1, w2, "gelu_tanh", "f16", nthreads=4)
    assert np.array_equal(a, b)


def test_brute_force_tiny_fractions(oracle_mod):
    """Exact rational sums (fractions.Fraction) on tiny shapes: with act
    none the oracle's T is the exact sum rounded once, except where the fp32
    summation error carries it across a rounding boundary (1 ulp)."""
    from fractions import Fraction
    for (M, H, I, dtype, seed) in [(2, 3, 5, "f16", 1), (3, 8, 4, "bf16", 2), (1, 17, 16, "f16", 3)]:
        x, w1, w2 = gen.random_case(M, H, I, "none", dtype, seed=seed, w_std=0.5)
        X, W1, W2 = (widen_lib(a, dtype) for a in (x, w1, w2))
        y, t = oracle_mod.mlp_chain(x, w1, w2, "none", dtype, want_t=True)
        T = widen_lib(t, dtype)
        for m in range(M):
            for i in range(I):
                exact = sum(Fraction(float(X[m, k])) * Fraction(float(W1[k, i])) for k in range(H))
                assert abs(T[m, i] - float(exact)) <= ulp(float(exact), dtype) + 1e-30
            for n in range(H):
                exact = sum(Fraction(float(T[m, i])) * Fraction(float(W2[i, n])) for i in range(I))
                assert abs(widen_lib(y, dtype)[m, n] - float(exact)) <= ulp(float(exact), dtype) + 1e-30


def test_empty_and_bad_arguments(oracle_mod):
    x = np.zeros((0, 8), np.uint16)
    w1 = np.zeros((8, 8), np.uint16)
    w2 = np.zeros((8, 8), np.uint16)
    y = oracle_mod.mlp_chain(x, w1, w2, "none", "f16")
    assert y.shape == (0, 8)
    with pytest.raises(ValueError):
        oracle_mod.mlp_chain(np.zeros((2, 8), np.uint16), w1, w2, "swiglu", "f16")


# ---- chains of several layers (the composition) ------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_exact_integer_layers(oracle_mod, dtype):
    """Two layers of integer weights (act none): the oracle's chain of layers
    equals exact int64 products with the library's rounding after every GEMM,
    layer by layer, bit for bit.  The layers' weights differ and do not
    commute, so a swapped layer order or a layer fed the wrong input fails."""
    M, H, I = 6, 48, 40
    x, xi = _int_bits((M, H), 21, -3, 3, 0.8, dtype)
    ws = [(_int_bits((H, I), 22 + 2 * l, -2, 2, 0.6, dtype), _int_bits((I, H), 23 + 2 * l, -1, 1, 0.3, dtype))
          for l in range(2)]
    yi = xi
    for (w1, w1i), (w2, w2i) in ws:
        h = yi @ w1i
        assert (np.abs(yi) @ np.abs(w1i)).max() < 2 ** 24
        t_int = widen_lib(_lib_round(h, dtype), dtype).astype(np.int64)
        yv = t_int @ w2i
        assert (np.abs(t_int) @ np.abs(w2i)).max() < 2 ** 24
        yi = widen_lib(_lib_round(yv, dtype), dtype).astype(np.int64)
    y = oracle_mod.mlp_layers(x, [w[0][0] for w in ws], [w[1][0] for w in ws], "none", dtype)
    assert np.array_equal(widen_lib(y, dtype), yi.astype(np.float64))
    swapped = oracle_mod.mlp_layers(x, [ws[1][0][0], ws[0][0][0]], [ws[1][1][0], ws[0][1][0]], "none", dtype)
    assert not np.array_equal(swapped, y)


@pytest.mark.parametrize("act", ["none", "gelu_tanh"])
def test_identity_layers(oracle_mod, act):
    """Identity W1 and W2 in every layer: with act none the chain returns X
    exactly after three layers; with GeLU each layer applies the separately
    pinned activation once (checked against three explicit applications)."""
    M, H = 9, 64
    x = gen.normal_bits((M, H), 31, 1.0, "f16")
    eye = gen.to_bits(np.eye(H, dtype=np.float32), "f16")
    y = oracle_mod.mlp_layers(x, [eye] * 3, [eye] * 3, act, "f16")
    if act == "none":
        assert np.array_equal(y, x)
    else:
        v = x
        for _ in range(3):
            v = oracle_mod.round_to(oracle_mod.act(oracle_mod.widen(v, "f16"), "gelu_tanh"), "f16")
        assert np.array_equal(y, v)


def test_one_layer_is_the_chain(oracle_mod):
    x, w1, w2 = gen.random_case(5, 64, 96, "swiglu", "bf16", seed=3)
    assert np.array_equal(oracle_mod.mlp_layers(x, [w1], [w2], "swiglu", "bf16"),
                          oracle_mod.mlp_chain(x, w1, w2, "swiglu", "bf16"))

"""The FP8 (MX block-scaled) oracle against its pins, and planted mistakes in
copies of it that the pins must catch (no GPU)."""
import numpy as np
import pytest

from oracle import attention
from oracle import fp8 as F


# ---------------------------------------------------------------------------
# E4M3 rounding
# ---------------------------------------------------------------------------

def pin_grid_is_the_format(round_fn):
    """127 non-negative finite codes; grid points are fixed points; extremes."""
    g = F.e4m3_grid()
    assert len(g[g >= 0]) == 127 and g.max() == 448.0 and g[g > 0].min() == 2.0 ** -9
    np.testing.assert_array_equal(round_fn(g), g)


def pin_round_half_even(round_fn):
    """Midpoints between neighbours go to the one whose last mantissa bit is 0."""
    g = F.e4m3_grid()
    pos = g[g >= 0]
    mids = (pos[:-1] + pos[1:]) / 2
    got = round_fn(mids)
    for lo, hi, m, r in zip(pos[:-1], pos[1:], mids, got):
        # the even neighbour: its code's mantissa field is even
        def mant(v):
            if v == 0:
                return 0
            if v < 2.0 ** -6:
                return int(round(v / 2.0 ** -9))
            e = int(np.floor(np.log2(v)))
            return int(round((v / 2.0 ** e - 1) * 8))
        even = lo if mant(lo) % 2 == 0 else hi
        assert r == even, (m, r, lo, hi)
    # just off the midpoint goes to the nearer neighbour
    np.testing.assert_array_equal(round_fn(mids * (1 - 1e-9)), pos[:-1])
    np.testing.assert_array_equal(round_fn(mids * (1 + 1e-9)), pos[1:])


def pin_saturation_and_sign(round_fn):
    x = np.array([448.0, 463.9, 464.0, 480.0, 1e6, 3e38])
    np.testing.assert_array_equal(round_fn(x), 448.0)
    np.testing.assert_array_equal(round_fn(-x), -448.0)
    rng = np.random.default_rng(1)
    y = rng.standard_normal(1000) * 50
    np.testing.assert_array_equal(round_fn(-y), -round_fn(y))
    assert round_fn(np.array([0.0]))[0] == 0.0


def pin_matches_torch_float8(round_fn):
    """Library cross-check: torch's float8_e4m3fn conversion (round to nearest
    even) on every bf16 value below the saturation threshold 464."""
    torch = pytest.importorskip("torch")
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    x = bits.view(np.float32).astype(np.float64)
    keep = np.isfinite(x) & (np.abs(x) < 464)
    x = x[keep]
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_fn(x), ref)


def pin_relative_error(round_fn):
    rng = np.random.default_rng(2)
    x = np.exp(rng.uniform(np.log(2.0 ** -6), np.log(448), 20000)) * rng.choice([-1, 1], 20000)
    err = np.abs(round_fn(x) - x) / np.abs(x)
    assert err.max() <= 2.0 ** -4 + 1e-15
    y = rng.uniform(0, 2.0 ** -6, 20000)
    assert np.abs(round_fn(y) - y).max() <= 2.0 ** -10 + 1e-18


ROUND_PINS = [pin_grid_is_the_format, pin_round_half_even, pin_saturation_and_sign,
              pin_matches_torch_float8, pin_relative_error]


@pytest.mark.parametrize("pin", ROUND_PINS, ids=lambda p: p.__name__)
def test_e4m3_round_pins(pin):
    pin(F.e4m3_round)


def _round_mutant(kind):
    def fn(x):
        x = np.asarray(x, dtype=np.float64)
        a = np.abs(x)
        with np.errstate(divide="ignore"):
            e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
        e = np.clip(e, -6, 8)
        mbits = 2 if kind == "two_mantissa_bits" else 3
        quantum = np.where(a < 2.0 ** -6, 2.0 ** -9, 2.0 ** (e - mbits))
        q = a / quantum
        r = (np.floor(q + 0.5) if kind == "ties_away" else np.rint(q)) * quantum
        if kind != "no_saturation":
            r = np.minimum(r, 448.0)
        if kind == "no_subnormals":
            r = np.where(a < 2.0 ** -6, 0.0, r)
        return np.copysign(r, x)
    return fn


@pytest.mark.parametrize("kind", ["two_mantissa_bits", "ties_away", "no_saturation",
                                  "no_subnormals"])
def test_e4m3_round_mutant_is_caught(kind):
    fn = _round_mutant(kind)
    failed = []
    for pin in ROUND_PINS:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001 - any failure counts as caught
            failed.append(pin.__name__)
    assert failed, f"rounding mutant {kind} passed every pin"


# ---------------------------------------------------------------------------
# MX block scaling
# ---------------------------------------------------------------------------

def pin_block_exponent(quant):
    """The block maximum's quotient lies in [256, 512) before saturation, so the
    quantised block maximum is in [256, 448]; exponents are integers in range."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((50, 64)) * np.exp(rng.uniform(-20, 20, (50, 1)))
    q, e = quant(x, -1)
    assert e.shape == (50, 2) and e.dtype.kind == "i"
    qmax = np.abs(q).reshape(50, 2, 32).max(-1)
    assert np.all((qmax >= 256) & (qmax <= 448))
    amax = np.abs(x).reshape(50, 2, 32).max(-1)
    assert np.all((amax / 2.0 ** e >= 256) & (amax / 2.0 ** e < 512))


def pin_power_of_two_exactness(quant):
    """Scaling the input by 2^k shifts every exponent by k and leaves the values."""
    rng = np.random.default_rng(4)
    x = rng.standard_normal((8, 96))
    q0, e0 = quant(x, -1)
    for k in (-30, -1, 3, 17):
        qk, ek = quant(x * 2.0 ** k, -1)
        np.testing.assert_array_equal(qk, q0)
        np.testing.assert_array_equal(ek, e0 + k)
    # a block of powers of two (within E4M3's range of the block max) is exact
    p = 2.0 ** rng.integers(-14, 3, (4, 32)).astype(np.float64)
    qp, ep = quant(p, -1)
    np.testing.assert_array_equal(F.mx_dequantize(qp, ep, -1), p)


def pin_blocks_independent_and_axis(quant):
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 128))
    q, e = quant(x, -1)
    for j in range(4):   # each block quantised alone gives the same
        qj, ej = quant(x[:, 32 * j:32 * (j + 1)], -1)
        np.testing.assert_array_equal(qj, q[:, 32 * j:32 * (j + 1)])
        np.testing.assert_array_equal(ej[:, 0], e[:, j])
    qa, ea = quant(x.T.copy(), 0)   # blocking along axis 0 of the transpose
    np.testing.assert_array_equal(qa, q.T)
    np.testing.assert_array_equal(ea, e.T)


def pin_zero_block_and_error_bound(quant):
    x = np.zeros((2, 32))
    q, e = quant(x, -1)
    assert np.all(q == 0) and np.all(e == -127)
    rng = np.random.default_rng(6)
    y = rng.standard_normal((200, 32))
    q, e = quant(y, -1)
    back = F.mx_dequantize(q, e, -1)
    X = 2.0 ** np.repeat(e, 32, axis=-1)
    normal = np.abs(y) >= 2.0 ** -6 * X
    rel = np.abs(back - y)[normal] / np.abs(y)[normal]
    # saturation of the block maximum (quotient in [448, 512)) costs at most 1 - 448/512
    assert rel.max() <= max(2.0 ** -4, 1 - 448 / 512) + 1e-15
    assert np.all(np.abs(back - y)[~normal] <= 2.0 ** -10 * X[~normal] + 1e-300)


def pin_non_finite_block(quant):
    """A block with an infinity or a NaN gets the NaN scale (exponent 128) and
    zero elements; its neighbours are untouched."""
    rng = np.random.default_rng(9)
    x = rng.standard_normal((3, 64))
    x[0, 3] = np.inf
    x[1, 40] = np.nan
    x[2, 0] = -np.inf
    q, e = quant(x, -1)
    assert e[0, 0] == 128 and e[1, 1] == 128 and e[2, 0] == 128
    assert np.all(q[0, :32] == 0) and np.all(q[1, 32:] == 0) and np.all(q[2, :32] == 0)
    qr, er = quant(x[:, 32:].copy(), -1)
    np.testing.assert_array_equal(q[[0, 2], 32:], qr[[0, 2]])
    assert np.all(np.isnan(F.mx_dequantize(q, e, -1)[0, :32]))


MX_PINS = [pin_non_finite_block, pin_block_exponent, pin_power_of_two_exactness, pin_blocks_independent_and_axis,
           pin_zero_block_and_error_bound]


@pytest.mark.parametrize("pin", MX_PINS, ids=lambda p: p.__name__)
def test_mx_quantize_pins(pin):
    pin(F.mx_quantize)


def _mx_mutant(kind):
    def fn(x, axis=-1):
        x = np.asarray(x, dtype=np.float64)
        xm = np.moveaxis(x, axis, -1)
        n = xm.shape[-1]
        bs = 16 if kind == "block_16" else 32
        blocks = xm.reshape(*xm.shape[:-1], n // bs, bs)
        amax = np.max(np.abs(blocks), axis=-1)
        with np.errstate(divide="ignore"):
            lg = np.log2(np.where(amax > 0, amax, 1.0))
        e = (np.ceil(lg) if kind == "ceil_exponent" else np.floor(lg)) - (7 if kind == "emax_7" else 8)
        e = np.clip(np.where(amax > 0, e, -127), -127, 127).astype(np.int64)
        q = F.e4m3_round(blocks / (2.0 ** e)[..., None])
        if kind == "block_16":   # report one exponent per 32 (the first half's)
            e = e[..., ::2]
        return np.moveaxis(q.reshape(xm.shape), -1, axis), np.moveaxis(e, -1, axis)
    return fn


@pytest.mark.parametrize("kind", ["emax_7", "ceil_exponent", "block_16"])
def test_mx_quantize_mutant_is_caught(kind):
    fn = _mx_mutant(kind)
    failed = []
    for pin in MX_PINS:
        try:
            pin(fn)
        except Exception:  # noqa: BLE001
            failed.append(pin.__name__)
    assert failed, f"MX mutant {kind} passed every pin"


# ---------------------------------------------------------------------------
# Attention on the quantised operands
# ---------------------------------------------------------------------------

def test_attention_mx8_is_the_definition_on_dequantised_values():
    rng = np.random.default_rng(7)
    B, N, H, d = 2, 70, 3, 64
    q, k, v = (rng.standard_normal((B, N, H, d)) for _ in range(3))
    q8, qe = F.quantize_qk(q)
    k8, ke = F.quantize_qk(k)
    vt8, vte = F.quantize_v_transposed(v)
    assert vt8.shape == (B, H, d, 128) and vte.shape == (B, H, d, 4)
    assert np.all(vt8[..., N:] == 0)
    for causal in (False, True):
        O, L = F.attention_mx8(q8, qe, k8, ke, vt8, vte, 0.125, causal)
        Q, K = F.mx_dequantize(q8, qe), F.mx_dequantize(k8, ke)
        V = F.mx_dequantize(vt8, vte)[..., :N].transpose(0, 3, 1, 2)
        for b in range(B):
            for h in range(H):
                o, l = attention(Q[b, :, h], K[b, :, h], V[b, :, h], 0.125, causal)
                np.testing.assert_array_equal(O[b, :, h], o)
                np.testing.assert_array_equal(L[b, h], l)
        # and it stays near the unquantised attention: each operand element
        # carries at most 2^-4 relative error (3 mantissa bits), so O moves by
        # at most about 2^-4 max|V| + the score perturbation's effect
        Or, Lr = (np.stack([np.stack([attention(q[b, :, h], k[b, :, h], v[b, :, h], 0.125,
                                                causal)[i] for h in range(H)], 0)
                            for b in range(B)], 0) for i in (0, 1))
        diff = np.abs(O - Or.transpose(0, 2, 1, 3))
        assert diff.max() < 2.0 ** -3 * np.abs(v).max() and diff.mean() < 0.02
        assert np.abs(L - Lr).max() < 0.1


def test_quantize_v_transposed_layout():
    rng = np.random.default_rng(8)
    v = rng.standard_normal((1, 100, 2, 32))
    vt8, vte = F.quantize_v_transposed(v)
    # token j of head h, dim c sits at vt8[0, h, c, j]; blocks run along tokens
    q, e = F.mx_quantize(np.pad(v[0, :, 1, 5], (0, 28)), axis=-1)
    np.testing.assert_array_equal(vt8[0, 1, 5], q)
    np.testing.assert_array_equal(vte[0, 1, 5], e)

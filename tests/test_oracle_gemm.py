"""Pins for oracle/gemm.py and oracle/bounds.py, independent of the oracle itself.

* brute force: a pure-Python triple loop over exact rationals (fractions) on
  tiny inputs, for fp16, int8 and the tile-wise indexed form;
* the int8 epilogue checked against exact rational rounding to float32;
* closed forms: one-hot weights select a column of A, zero weights give zero,
  2:4 with positions (0, 1) everywhere is a dense GEMM on a column subset;
* the two tile-wise formulations (masked dense vs indexed) agree;
* planted mistakes in copies of the oracle functions make these checks fail.
"""

from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads as wl

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers
def exact_product(A, W):
    """Pure-Python sum of exact rational products: the definition of A . W."""
    M, K = len(A), len(A[0])
    N = len(W[0])
    Af = [[Fraction(float(A[m][k])) for k in range(K)] for m in range(M)]
    Wf = [[Fraction(float(W[k][n])) for n in range(N)] for k in range(K)]
    return [[sum((Af[m][k] * Wf[k][n] for k in range(K)), Fraction(0)) for n in range(N)]
            for m in range(M)]


def check_gemm_bruteforce(gemm_fn, seed=0, trials=6):
    """True iff gemm_fn(A, W) matches the exact rational product to f64 accuracy."""
    rng = np.random.default_rng(seed)
    for t in range(trials):
        M, K, N = rng.integers(1, 9), 4 * rng.integers(1, 6), rng.integers(1, 9)
        case = wl.random_24_f16(rng, M, K, N, std_w=0.5)
        A, Wp = case["A"], case["Wp"]
        got = gemm_fn(A, Wp)
        ex = exact_product(A.tolist(), Wp.tolist())
        S = np.abs(A.astype(np.float64)) @ np.abs(Wp.astype(np.float64))
        for m in range(M):
            for n in range(N):
                if abs(Fraction(float(got[m, n])) - ex[m][n]) > Fraction(K * 2.0 ** -52 * S[m, n]):
                    return False
    return True


def round_to_f32(x: Fraction):
    """Nearest float32 to the rational x, ties to even (pure rational search)."""
    f = np.float32(float(x))
    best = None
    for cand in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - x)
        if best is None or d < best[0] or (d == best[0] and
                                           (int(cand.view(np.uint32)) & 1) == 0):
            best = (d, cand)
    return best[1]


# ---------------------------------------------------------------- brute force
def test_f16_gemm_matches_exact_rationals():
    assert check_gemm_bruteforce(oracle.ref_gemm_f64)


def test_f16_output_is_rne_of_exact_value():
    rng = np.random.default_rng(1)
    case = wl.random_24_f16(rng, 5, 16, 7, std_w=0.3)
    C64, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
    # the fp16 result is within half an ulp of C64 (nearest), checked by neighbours
    for c64, c16 in zip(C64.ravel(), C16.ravel()):
        lo = np.nextafter(c16, np.float16(-np.inf))
        hi = np.nextafter(c16, np.float16(np.inf))
        d = abs(float(c16) - c64)
        assert d <= abs(float(lo) - c64) and d <= abs(float(hi) - c64)


def test_i8_accumulator_matches_python_ints():
    rng = np.random.default_rng(2)
    for _ in range(5):
        M, K, N = rng.integers(1, 7), 4 * rng.integers(1, 9), rng.integers(1, 7)
        case = wl.random_24_i8(rng, M, K, N)
        acc = oracle.ref_gemm_i8(case["A"], case["Wp"])
        assert acc.dtype == np.int32
        A, W = case["A"].astype(int).tolist(), case["Wp"].astype(int).tolist()
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(A[m][k] * W[k][n] for k in range(K))


def test_i8_scaled_output_is_two_roundings():
    rng = np.random.default_rng(3)
    case = wl.random_24_i8(rng, 4, 64, 6)
    acc = oracle.ref_gemm_i8(case["A"], case["Wp"])
    C = oracle.ref_gemm_i8(case["A"], case["Wp"], case["scale"])
    assert C.dtype == np.float32
    for m in range(4):
        for n in range(6):
            a32 = round_to_f32(Fraction(int(acc[m, n])))
            want = round_to_f32(Fraction(float(a32)) * Fraction(float(case["scale"][n])))
            assert C[m, n].view(np.uint32) == want.view(np.uint32)


def test_i8_large_k_accumulator_still_exact():
    # K = 4096 with extreme values: |acc| up to 2048 * 127 * 127 > 2^24
    K, N = 4096, 3
    A = np.full((2, K), 127, dtype=np.int8)
    A[1] = -127
    W = np.zeros((K, N), dtype=np.int8)
    W[0::4] = 127
    W[1::4] = 127
    acc = oracle.ref_gemm_i8(A, W)
    assert acc[0, 0] == 2048 * 127 * 127 and acc[1, 2] == -2048 * 127 * 127


def test_tw_indexed_matches_exact_rationals():
    rng = np.random.default_rng(4)
    M, K, N, G = 3, 12, 8, 4
    case = wl.random_tw_f16(rng, M, K, N, G, [0.5, 0.3])
    packed = oracle.ref_tw_pack(case["Wp"], G)
    got = oracle.ref_tw_gemm_indexed(case["A"], packed, N, G)
    ex = exact_product(case["A"].tolist(), case["Wp"].tolist())
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(float(got[m, n])) - ex[m][n]) < Fraction(1, 2 ** 40)


# ---------------------------------------------------------------- closed forms
@pytest.mark.parametrize("dtype", [np.float16, np.int8])
def test_one_hot_selects_column(dtype):
    rng = np.random.default_rng(5)
    case = wl.one_hot_24(rng, 9, 64, 40, dtype=dtype)
    if dtype == np.int8:
        C = oracle.ref_gemm_i8(case["A"], case["Wp"])
        assert np.array_equal(C, case["A"][:, case["k_of_n"]].astype(np.int32))
    else:
        _, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
        assert np.array_equal(C16.view(np.uint16), case["A"][:, case["k_of_n"]].view(np.uint16))


def test_zero_weights_give_zero():
    A = np.ones((3, 8), np.float16)
    assert not oracle.ref_gemm_f64(A, np.zeros((8, 5), np.float16)).any()


def test_fixed_positions_reduce_to_dense_subset():
    # 2:4 with kept positions (0, 1) in every group equals a dense GEMM on the
    # columns {4g, 4g+1} of A against the compressed rows.
    rng = np.random.default_rng(6)
    M, K, N = 7, 32, 5
    A = wl.f16_normal(rng, (M, K))
    dense_half = wl.f16_normal(rng, (K // 2, N))
    Wp = np.zeros((K, N), np.float16)
    Wp[0::4] = dense_half[0::2]
    Wp[1::4] = dense_half[1::2]
    sub = np.sort(np.concatenate([np.arange(0, K, 4), np.arange(1, K, 4)]))
    want = A[:, sub].astype(np.float64) @ dense_half.astype(np.float64)
    np.testing.assert_allclose(oracle.ref_gemm_f64(A, Wp), want, rtol=0, atol=1e-12)


def test_tw_indexed_equals_masked_dense():
    rng = np.random.default_rng(7)
    case = wl.random_tw_f16(rng, 33, 96, 64, 16, [0.2, 0.9, 0.0, 0.5])
    packed = oracle.ref_tw_pack(case["Wp"], 16)
    a = oracle.ref_tw_gemm_indexed(case["A"], packed, 64, 16)
    b = oracle.ref_gemm_f64(case["A"], case["Wp"])
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-12)
    assert not a[:, 32:48].any()  # the empty tile's window is zero


def test_transpose():
    A = np.arange(12, dtype=np.float16).reshape(3, 4)
    At = oracle.ref_transpose(A)
    assert At.shape == (4, 3) and At.flags["C_CONTIGUOUS"] and At[2, 1] == A[1, 2]


# ---------------------------------------------------------------- bounds
def test_strict_bound_catches_one_dropped_term():
    rng = np.random.default_rng(8)
    case = wl.random_24_f16(rng, 64, 768, 64)
    C_ref, C16 = oracle.ref_gemm_f16(case["A"], case["Wp"])
    S = oracle.ref_abs_gemm(case["A"], case["Wp"])
    assert oracle.strict_ok_f16(C16, C_ref, S, 384)
    assert oracle.loose_ok(C16, C_ref)
    # drop a single product from one output: the loose bound misses it, the strict one does not
    Wd = case["Wp"].copy()
    k = int(np.argmax(np.abs(case["Wp"][:, 0].astype(np.float64))))
    Wd[k, 0] = 0
    _, Cd = oracle.ref_gemm_f16(case["A"], Wd)
    assert not oracle.strict_ok_f16(Cd, C_ref, S, 384)


def check_abs_gemm(fn, seed=0, trials=5):
    """True iff fn(A, W) is S = |A| . |W| (the error scale of the strict bound):
    a hand-computed 2 x 2 case whose products have mixed signs, then the
    exact rational sum of |a| |w| on tiny random inputs."""
    A = np.array([[1, -2], [3, 4]], np.float16)
    W = np.array([[-1, 0.5], [2, 0.25]], np.float16)
    # |A|.|W| by hand: [[1*1 + 2*2, 1*0.5 + 2*0.25], [3*1 + 4*2, 3*0.5 + 4*0.25]]
    if not np.array_equal(np.asarray(fn(A, W), dtype=np.float64), np.array([[5.0, 1.0], [11.0, 2.5]])):
        return False
    rng = np.random.default_rng(seed)
    for _ in range(trials):
        M, K, N = rng.integers(1, 6), 4 * rng.integers(1, 5), rng.integers(1, 6)
        case = wl.random_24_f16(rng, M, K, N, std_w=0.5)
        got = np.asarray(fn(case["A"], case["Wp"]), dtype=np.float64)
        Aa = [[abs(Fraction(float(x))) for x in row] for row in case["A"].tolist()]
        Wa = [[abs(Fraction(float(x))) for x in row] for row in case["Wp"].tolist()]
        for m in range(M):
            for n in range(N):
                ex = sum((Aa[m][k] * Wa[k][n] for k in range(K)), Fraction(0))
                if abs(Fraction(float(got[m, n])) - ex) > Fraction(K * 2.0 ** -52) * ex:
                    return False
    return True


def test_abs_gemm_pinned():
    assert check_abs_gemm(oracle.ref_abs_gemm)
    # S bounds |C_ref| everywhere and equals it when every operand is nonnegative
    rng = np.random.default_rng(3)
    case = wl.random_24_f16(rng, 16, 64, 24)
    S = oracle.ref_abs_gemm(case["A"], case["Wp"])
    C = oracle.ref_gemm_f64(case["A"], case["Wp"])
    assert (S >= np.abs(C)).all()
    Ap, Wpp = np.abs(case["A"]), np.abs(case["Wp"])
    assert np.array_equal(oracle.ref_abs_gemm(Ap, Wpp), oracle.ref_gemm_f64(Ap, Wpp))


@pytest.mark.parametrize("mutant", [
    lambda A, W: np.abs(A.astype(np.float64)) @ W.astype(np.float64),   # abs on A only
    lambda A, W: A.astype(np.float64) @ np.abs(W.astype(np.float64)),   # abs on W only
    lambda A, W: np.abs(A.astype(np.float64) @ W.astype(np.float64)),   # abs of the sum
    lambda A, W: 2.0 * oracle.ref_abs_gemm(A, W),                       # loosened by a factor
    lambda A, W: np.abs(A.astype(np.float64)) @ np.abs(W.astype(np.float64))[::-1],  # rows of W reversed
])
def test_abs_gemm_pin_catches_planted_mistakes(mutant):
    assert not check_abs_gemm(mutant)


def test_loose_rejects_nan():
    assert not oracle.loose_ok(np.array([np.nan, 1.0]), np.array([1.0, 1.0]))
    assert oracle.loose_err(np.zeros(3), np.zeros(3)) == 0.0


# ---------------------------------------------------------------- planted mistakes
def _mut_transposed(A, W):
    return oracle.ref_gemm_f64(A, np.asarray(W)[::-1])


def _mut_dropped_last_k(A, W):
    W = np.array(W, copy=True)
    W[-1] = 0
    return oracle.ref_gemm_f64(A, W)


def _mut_sign(A, W):
    C = oracle.ref_gemm_f64(A, W)
    C[0, 0] = -C[0, 0]
    return C


def _mut_f32_accumulate(A, W):
    return (np.asarray(A).astype(np.float16) @ np.asarray(W).astype(np.float16)).astype(np.float64)


@pytest.mark.parametrize("mutant", [_mut_transposed, _mut_dropped_last_k, _mut_sign,
                                    _mut_f32_accumulate])
def test_bruteforce_catches_planted_mistakes(mutant):
    assert not check_gemm_bruteforce(mutant)


# ---------------------------------------------------------------- int8 epilogues
def round_to_f16(x: Fraction):
    """Nearest fp16 to the rational x, ties to even, |x| beyond the largest
    finite value rounds to +-inf (IEEE binary16 by enumeration of the finite set)."""
    finite = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)  # +0 .. 65504
    mags = [Fraction(float(v)) for v in finite]
    ax = abs(x)
    # overflow threshold: halfway between 65504 and the next step 65536
    if ax >= Fraction(65520):
        r = np.float16(np.inf)
    else:
        lo, hi = 0, len(mags) - 1
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if mags[mid] <= ax:
                lo = mid
            else:
                hi = mid
        cands = [lo] if mags[lo] == ax else [lo, hi]
        best = min(cands, key=lambda i: (abs(mags[i] - ax), i & 1))
        r = finite[best]
    return -r if x < 0 else r


def round_to_i8(x: Fraction):
    """Nearest integer, ties to even, saturated to [-128, 127]."""
    fl = x.numerator // x.denominator
    frac = x - fl
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return max(-128, min(127, fl))


def expected_epilogue(acc, scale, bias, out):
    """Exact rationals with one round-to-float32 per step, then the output rounding."""
    M, N = acc.shape
    res = []
    for m in range(M):
        row = []
        for n in range(N):
            a32 = round_to_f32(Fraction(int(acc[m, n])))
            y = round_to_f32(Fraction(float(a32)) * Fraction(float(scale[n])))
            if bias is not None:
                y = round_to_f32(Fraction(float(y)) + Fraction(float(bias[n])))
            if out == "f32":
                row.append(y)
            elif out == "f16":
                row.append(round_to_f16(Fraction(float(y))))
            else:
                row.append(round_to_i8(Fraction(float(y))))
        res.append(row)
    return res


@pytest.mark.parametrize("out", ["f32", "f16", "i8"])
@pytest.mark.parametrize("with_bias", [False, True])
def test_i8_epilogue_matches_exact_rationals(out, with_bias):
    rng = np.random.default_rng(11)
    case = wl.random_24_i8(rng, 4, 64, 5)
    acc = oracle.ref_acc_i8(case["A"], case["Wp"])
    # scales that put y in the interesting range of each output kind
    scale = {"f32": case["scale"], "f16": case["scale"] * np.float32(40.0),
             "i8": rng.uniform(1e-4, 3e-3, size=5).astype(np.float32)}[out]
    bias = rng.normal(0, 3.0, size=5).astype(np.float32) if with_bias else None
    got = oracle.ref_i8_epilogue(acc, scale, bias, out)
    want = expected_epilogue(acc, scale, bias, out)
    assert got.dtype == {"f32": np.float32, "f16": np.float16, "i8": np.int8}[out]
    for m in range(4):
        for n in range(5):
            if out == "i8":
                assert int(got[m, n]) == want[m][n]
            else:
                bits = np.uint32 if out == "f32" else np.uint16
                assert got[m, n].view(bits) == np.asarray(want[m][n]).view(bits)


def test_i8_epilogue_hand_computed_cases():
    # fp16 spacing is 2 on [2048, 4096): 2049 and 2051 are ties, to the even mantissa
    acc = np.array([[2049, 2051, -2049, 65519, 65520, 70000]], dtype=np.int32)
    one = np.ones(6, np.float32)
    f16 = oracle.ref_i8_epilogue(acc, one, None, "f16")
    assert f16.tolist() == [[2048.0, 2052.0, -2048.0, 65504.0, np.inf, np.inf]]
    # int8: ties to even, then saturation (127.5 rounds to 128 and saturates)
    acc = np.array([[5, 7, -5, 255, 256, -257, 600, -600]], dtype=np.int32)
    half = np.full(8, 0.5, np.float32)
    i8 = oracle.ref_i8_epilogue(acc, half, None, "i8")
    assert i8.tolist() == [[2, 4, -2, 127, 127, -128, 127, -128]]
    # the bias is added to the rounded product (no fused multiply-add):
    # 3 * (1 + 2^-23) = 3 + 1.5 * 2^-22 is a tie and rounds to even, 3 + 2^-21;
    # adding 2^-22 then gives 3 + 3 * 2^-22 exactly.  One fused rounding of
    # 3 + 2.5 * 2^-22 would give 3 + 2^-21 instead.
    acc = np.array([[3]], dtype=np.int32)
    s = np.array([1 + 2.0 ** -23], np.float32)
    b = np.array([2.0 ** -22], np.float32)
    y = oracle.ref_i8_epilogue(acc, s, b, "f32")[0, 0]
    assert Fraction(float(y)) == 3 + 3 * Fraction(1, 2 ** 22)
    assert Fraction(float(y)) != 3 + Fraction(1, 2 ** 21)


def test_i8_raw_output_is_the_accumulator():
    rng = np.random.default_rng(12)
    case = wl.random_24_i8(rng, 3, 32, 4)
    acc = oracle.ref_acc_i8(case["A"], case["Wp"])
    assert np.array_equal(oracle.ref_gemm_i8_out(case["A"], case["Wp"], None, None, "i32"), acc)
    with pytest.raises(ValueError):
        oracle.ref_i8_epilogue(acc, case["scale"], None, "i32")


def _mut_fused(acc, scale, bias, out):
    y = (acc.astype(np.float64) * scale.astype(np.float64)[None, :] + bias.astype(np.float64)[None, :])
    return y.astype(np.float32)


def _mut_trunc_i8(acc, scale, bias, out):
    y = acc.astype(np.float32) * scale[None, :] + bias[None, :]
    return np.clip(np.trunc(y), -128, 127).astype(np.int8)


def _mut_sym_i8(acc, scale, bias, out):
    y = acc.astype(np.float32) * scale[None, :] + bias[None, :]
    return np.clip(np.rint(y), -127, 127).astype(np.int8)


@pytest.mark.parametrize("mutant,out", [(_mut_fused, "f32"), (_mut_trunc_i8, "i8"), (_mut_sym_i8, "i8")])
def test_epilogue_pins_catch_planted_mistakes(mutant, out):
    rng = np.random.default_rng(13)
    acc = rng.integers(-40000, 40000, size=(16, 8)).astype(np.int32)
    acc[0, :] = -400  # drives int8 outputs to the negative limit
    if out == "f32":
        scale = rng.uniform(1e-3, 1e-2, 8).astype(np.float32)
    else:
        scale = np.full(8, 0.01, np.float32)
    bias = rng.normal(0, 1.0, 8).astype(np.float32)
    want = expected_epilogue(acc, scale, bias, out)
    got = mutant(acc, scale, bias, out)
    same = all((int(got[m, n]) == want[m][n]) if out == "i8" else
               (got[m, n].view(np.uint32) == np.asarray(want[m][n]).view(np.uint32))
               for m in range(16) for n in range(8))
    assert not same

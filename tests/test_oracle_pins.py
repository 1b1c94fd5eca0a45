"""Pins for the CPU oracle: each function in oracle/ is tied to something other
than itself (exact rational arithmetic, closed forms, an independent integer
loop, hand-derived rounding cases), and planted mistakes in a copy of the
oracle must each fail at least one pin.

The product pinned is the plain definition C = A.B (with D = |A|.|B|) that the
pages' dense GEMM computes ("GPU speed, without leaving Rust's safety model",
section "Safety without a visible tax").
"""

import os
import re
import subprocess
import sys
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import bf16_to_f64, rne_bf16
from tile_partitioned_dense_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_bf16(shape, seed, dist="normal"):
    return synth.draw(shape[0], shape[1], dist, seed)


def exact_sum(A, B):
    """Exact rational C and D by brute force (bf16 values are dyadic rationals)."""
    a = bf16_to_f64(A)
    b = bf16_to_f64(B)
    M, K = a.shape
    N = b.shape[1]
    C = [[Fraction(0)] * N for _ in range(M)]
    D = [[Fraction(0)] * N for _ in range(M)]
    for i in range(M):
        for j in range(N):
            s = Fraction(0)
            sa = Fraction(0)
            for k in range(K):
                x = Fraction(a[i, k]) * Fraction(b[k, j])
                s += x
                sa += abs(x)
            C[i][j] = s
            D[i][j] = sa
    return C, D


# ---------------------------------------------------------------- pin helpers
# Each returns a list of failure strings; an empty list means the pin holds.
# They take the oracle functions as arguments so the same pins run against
# planted-mistake copies of the oracle library.

def pin_bruteforce(gemm_fn, shapes=((1, 1, 1), (2, 3, 5), (3, 2, 8), (5, 8, 17), (8, 5, 3), (17, 3, 2))):
    fails = []
    for n, (M, N, K) in enumerate(shapes):
        for dist in ("normal", "uniform"):
            A = rand_bf16((M, K), 100 + n, dist)
            B = rand_bf16((K, N), 200 + n, dist)
            C, D = gemm_fn(A, B)
            Ce, De = exact_sum(A, B)
            for i in range(M):
                for j in range(N):
                    bound = Fraction(K) * Fraction(2) ** -53 * De[i][j]
                    if abs(Fraction(C[i, j]) - Ce[i][j]) > bound:
                        fails.append(f"C[{i},{j}] {M}x{N}x{K} {dist}")
                    if abs(Fraction(D[i, j]) - De[i][j]) > bound:
                        fails.append(f"D[{i},{j}] {M}x{N}x{K} {dist}")
    return fails


def pin_identity(gemm_fn):
    fails = []
    A = rand_bf16((7, 9), 11)
    I9 = np.where(np.eye(9, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    C, _ = gemm_fn(A, I9)
    if not np.array_equal(C, bf16_to_f64(A)):
        fails.append("A.I != A")
    B = rand_bf16((7, 5), 12)
    I7 = np.where(np.eye(7, dtype=bool), np.uint16(0x3F80), np.uint16(0))
    C, _ = gemm_fn(I7, B)
    if not np.array_equal(C, bf16_to_f64(B)):
        fails.append("I.B != B")
    return fails


def pin_permutation(gemm_fn):
    """P.B permutes rows of B, A.Q permutes columns of A, exactly."""
    fails = []
    rng = np.random.default_rng(5)
    K, N = 13, 11
    # distinct bf16 values so any misplaced element is visible
    vals = rng.permutation(np.arange(1, K * N + 1, dtype=np.float64)) / 64.0
    B = synth.f64_to_bf16_bits(vals.reshape(K, N))
    perm = rng.permutation(K)
    P = np.zeros((K, K), np.uint16)
    P[np.arange(K), perm] = 0x3F80          # row i of P.B is row perm[i] of B
    C, _ = gemm_fn(P, B)
    if not np.array_equal(C, bf16_to_f64(B)[perm]):
        fails.append("P.B is not the row permutation")
    A = synth.f64_to_bf16_bits((rng.permutation(np.arange(1, 6 * K + 1)) / 32.0).reshape(6, K))
    q = rng.permutation(K)
    Q = np.zeros((K, K), np.uint16)
    Q[q, np.arange(K)] = 0x3F80             # column j of A.Q is column q[j] of A
    C, _ = gemm_fn(A, Q)
    if not np.array_equal(C, bf16_to_f64(A)[:, q]):
        fails.append("A.Q is not the column permutation")
    return fails


def pin_integer(gemm_fn, shapes=((64, 48, 300), (33, 65, 129), (1, 70, 1000))):
    """Entries in {-3..3}: an int64 loop written independently gives the exact C."""
    fails = []
    for n, (M, N, K) in enumerate(shapes):
        A = rand_bf16((M, K), 300 + n, "int3")
        Bt = rand_bf16((N, K), 400 + n, "int3")
        for B in (np.ascontiguousarray(Bt.T), Bt.T):     # row-major and column-major B
            Ai = bf16_to_f64(A).astype(np.int64)
            Bi = bf16_to_f64(B).astype(np.int64)
            want = np.zeros((M, N), np.int64)
            for k in range(K):
                want += np.outer(Ai[:, k], Bi[k, :])
            C, D = gemm_fn(A, B)
            if not np.array_equal(C, want.astype(np.float64)):
                fails.append(f"integer C {M}x{N}x{K} strides={B.strides}")
            wantD = np.abs(Ai) @ np.abs(Bi)
            if not np.array_equal(D, wantD.astype(np.float64)):
                fails.append(f"integer D {M}x{N}x{K}")
    return fails


def pin_closed_forms(gemm_fn):
    fails = []
    M, N, K = 9, 10, 37
    ones_a = np.full((M, K), 0x3F80, np.uint16)
    ones_b = np.full((K, N), 0x3F80, np.uint16)
    C, D = gemm_fn(ones_a, ones_b)
    if not (np.all(C == K) and np.all(D == K)):
        fails.append("ones.ones != K")
    d = rand_bf16((1, M), 21)[0]
    Dg = np.zeros((M, M), np.uint16)
    Dg[np.arange(M), np.arange(M)] = d
    B = rand_bf16((M, N), 22)
    C, _ = gemm_fn(Dg, B)
    if not np.array_equal(C, bf16_to_f64(d)[:, None] * bf16_to_f64(B)):
        fails.append("diag(d).B != d_i B_ij")
    # textbook example: [[1,2,3],[4,5,6]] . [[7,8],[9,10],[11,12]] = [[58,64],[139,154]]
    A = synth.f64_to_bf16_bits(np.array([[1, 2, 3], [4, 5, 6]], np.float64))
    B = synth.f64_to_bf16_bits(np.array([[7, 8], [9, 10], [11, 12]], np.float64))
    C, _ = gemm_fn(A, B)
    if not np.array_equal(C, np.array([[58, 64], [139, 154]], np.float64)):
        fails.append("textbook 2x3.3x2 example")
    # negative entries: sign handling in C and D
    A = synth.f64_to_bf16_bits(np.array([[-1.0, 2.0]]))
    B = synth.f64_to_bf16_bits(np.array([[3.0], [-0.5]]))
    C, D = gemm_fn(A, B)
    if not (C[0, 0] == -4.0 and D[0, 0] == 4.0):
        fails.append("signs: (-1*3 + 2*-0.5) = -4, |.| sum = 4")
    return fails


def pin_layout(gemm_fn):
    """A column-major B (transposed view) gives bitwise the row-major result."""
    fails = []
    A = rand_bf16((20, 45), 31)
    Bt = rand_bf16((23, 45), 32)
    C1, D1 = gemm_fn(A, np.ascontiguousarray(Bt.T))
    C2, D2 = gemm_fn(A, Bt.T)
    if not (np.array_equal(C1, C2) and np.array_equal(D1, D2)):
        fails.append("column-major B differs from row-major B")
    # a strided A (a sub-block of a wider array) equals its contiguous copy
    big = rand_bf16((20, 64), 33)
    C3, _ = gemm_fn(big[:, 3:48], np.ascontiguousarray(Bt.T))
    C4, _ = gemm_fn(np.ascontiguousarray(big[:, 3:48]), np.ascontiguousarray(Bt.T))
    if not np.array_equal(C3, C4):
        fails.append("strided A differs from contiguous A")
    return fails


ALL_PINS = (pin_bruteforce, pin_identity, pin_permutation, pin_integer,
            pin_closed_forms, pin_layout)


# ------------------------------------------------------------- the real pins

def _full(lib=None):
    return lambda A, B: oracle.gemm(A, B, lib=lib)


def _at(lib=None):
    def f(A, B):
        M, N = A.shape[0], B.shape[1]
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        c, d = oracle.gemm_at(A, B, ii.ravel(), jj.ravel(), lib=lib)
        return c.reshape(M, N), d.reshape(M, N)
    return f


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_triple_loop_pins(pin):
    assert pin(_full()) == []


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_elementwise_pins(pin):
    assert pin(_at()) == []


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_blas_pins(pin):
    if pin is pin_layout:
        # the library product is not claimed bitwise across layouts, only
        # within the fp64 bound, which pin_bruteforce checks
        return
    assert pin(lambda A, B: oracle.gemm_blas(A, B)) == []


def test_blas_matches_triple_loop_within_fp64_bound():
    A = rand_bf16((70, 300), 41)
    B = rand_bf16((300, 90), 42)
    C1, D1 = oracle.gemm(A, B)
    C2, D2 = oracle.gemm_blas(A, B)
    assert np.all(np.abs(C1 - C2) <= 2 * 300 * 2.0 ** -53 * D1)
    assert np.all(np.abs(D1 - D2) <= 2 * 300 * 2.0 ** -53 * D1)


def test_empty_and_zero_k():
    A = np.zeros((4, 0), np.uint16)
    B = np.zeros((0, 6), np.uint16)
    C, D = oracle.gemm(A, B)
    assert C.shape == (4, 6) and np.all(C == 0) and np.all(D == 0)
    C, D = oracle.gemm(np.zeros((0, 5), np.uint16), np.zeros((5, 3), np.uint16))
    assert C.shape == (0, 3)


def test_threads_do_not_change_sums():
    A = rand_bf16((37, 500), 51)
    B = rand_bf16((500, 29), 52)
    C1, D1 = oracle.gemm(A, B, threads=1)
    C8, D8 = oracle.gemm(A, B, threads=8)
    assert np.array_equal(C1, C8) and np.array_equal(D1, D8)
    c, d = oracle.gemm_at(A, B, np.arange(37) % 37, np.arange(37) % 29)
    assert np.array_equal(c, C1[np.arange(37), np.arange(37) % 29])


# --------------------------------------------------- planted mistakes (mutants)
# Each mutant is a copy of gemm_oracle.c with one plausible mistake, compiled
# on the CPU into a temporary library; at least one pin must fail on it.

MUTANTS = {
    "dropped_last_term": [("for (int64_t k = 0; k < K; ++k) {\n      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);\n      const double* b",
                           "for (int64_t k = 0; k < K - 1; ++k) {\n      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);\n      const double* b"),
                          ("for (int64_t k = 0; k < K; ++k) {\n      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);\n      const double b",
                           "for (int64_t k = 0; k < K - 1; ++k) {\n      const double a = oracle_bf16_to_f64(A[i * a_m + k * a_k]);\n      const double b")],
    "wrong_sign": [("c[j] += a * b[j];", "c[j] -= a * b[j];"), ("s += a * b;", "s -= a * b;")],
    "transposed_A_index": [("A[i * a_m + k * a_k]", "A[k * a_m + i * a_k]")],
    "B_strides_swapped": [("oracle_decode(B, K, N, b_k, b_n, B64);", "oracle_decode(B, K, N, b_n, b_k, B64);"),
                          ("B[k * b_k + j * b_n]", "B[k * b_n + j * b_k]")],
    "wrong_column": [("c[j] += a * b[j];", "c[j] += a * b[(j + 1) % N];"),
                     ("const int64_t i = ii[t], j = jj[t];", "const int64_t i = ii[t], j = jj[t] > 0 ? jj[t] - 1 : 0;")],
    "abs_missing_in_D": [("d[j] += aa * fabs(b[j]);", "d[j] += aa * b[j];"),
                         ("sa += fabs(a) * fabs(b);", "sa += fabs(a) * b;")],
    "bf16_decode_low_half": [("uint32_t u = ((uint32_t)h) << 16;", "uint32_t u = ((uint32_t)h) << 15;")],
}


def _build_mutant(d, name):
    src = open(os.path.join(os.path.dirname(oracle.__file__), "gemm_oracle.c")).read()
    s = src
    for old, new in MUTANTS[name]:
        assert old in s, (name, old)
        s = s.replace(old, new)
    c = d / f"{name}.c"
    c.write_text(s)
    so = d / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                    "-o", str(so), str(c), "-lm"], check=True)
    return so


def test_mutant_driver_control():
    """The unmodified oracle passes every pin through the same driver."""
    driver = os.path.join(os.path.dirname(__file__), "_mutant_driver.py")
    oracle.build(force=False)
    r = subprocess.run([sys.executable, driver, oracle.lib_path()], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 3, r.stdout + r.stderr


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_are_caught(tmp_path, name):
    """Run every pin against the mutant in a child process (a mutant that
    indexes out of range may crash, which also counts as caught)."""
    so = _build_mutant(tmp_path, name)
    driver = os.path.join(os.path.dirname(__file__), "_mutant_driver.py")
    r = subprocess.run([sys.executable, driver, str(so)], capture_output=True, text=True,
                       timeout=300, env={**os.environ, "OMP_NUM_THREADS": "2"})
    # exit 0: at least one pin failed for both entry points; 3: some entry
    # point passed every pin; a negative code: the mutant crashed the child
    assert r.returncode != 3, f"mutant {name} not caught:\n{r.stdout}\n{r.stderr}"
    assert r.returncode in (0,) or r.returncode < 0, r.stderr


# ------------------------------------------------------------- bf16 rounding

def _golden_rne():
    rows = []
    for line in open(os.path.join(GOLDEN, "bf16_rne_cases.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        tok = re.split(r"\s+", line, maxsplit=2)
        v = float(tok[0]) if tok[0] in ("inf", "-inf", "nan") else float.fromhex(tok[0])
        rows.append((v, int(tok[1], 16), tok[2]))
    return rows


def test_rne_golden_cases():
    rows = _golden_rne()
    assert len(rows) >= 20
    got = rne_bf16(np.array([r[0] for r in rows]))
    for (v, want, why), g in zip(rows, got):
        assert int(g) == want, f"{v!r}: got {int(g):#06x} want {want:#06x} ({why})"


def test_generator_rounding_matches_golden():
    rows = [r for r in _golden_rne() if np.isfinite(r[0]) and abs(r[0]) < 2.0 ** 120
            and (r[0] == 0 or abs(r[0]) >= 2.0 ** -100)]
    got = synth.f64_to_bf16_bits(np.array([r[0] for r in rows]))
    for (v, want, why), g in zip(rows, got):
        assert int(g) == want, f"{v!r}: got {int(g):#06x} want {want:#06x} ({why})"


def test_rne_matches_torch_on_fp32_values():
    """For values already exact in fp32, one rounding fp64->bf16 equals torch's
    fp32->bf16 conversion (an independent library routine)."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(7)
    x32 = np.concatenate([
        rng.standard_normal(20000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-30).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    # exact ties in fp32: a bf16 value plus half of its ulp
    base = rng.standard_normal(2000).astype(np.float32)
    u = base.view(np.uint32) & np.uint32(0xFFFF0000)
    x32 = np.concatenate([x32, (u | np.uint32(0x8000)).view(np.float32)])
    ours = rne_bf16(x32.astype(np.float64))
    theirs = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


def test_rne_mutant_ties_away_is_caught():
    """A plausible mistake (ties away from zero) fails the golden table."""
    def mutant(x):
        x = np.asarray(x, np.float64)
        _, e = np.frexp(np.abs(x))
        q = np.maximum(e - 8, -133)
        r = np.sign(x) * np.ldexp(np.floor(np.ldexp(np.abs(x), -q) + 0.5), q)
        with np.errstate(over="ignore"):
            return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    rows = [r for r in _golden_rne() if np.isfinite(r[0])]
    got = mutant(np.array([r[0] for r in rows]))
    assert any(int(g) != r[1] for r, g in zip(rows, got))


def test_bf16_decode_closed_forms():
    bits = np.array([0x3F80, 0xBF80, 0x4040, 0x0001, 0x7F7F, 0x0000, 0x8000, 0x7F80], np.uint16)
    want = [1.0, -1.0, 3.0, 2.0 ** -133, (2 - 2.0 ** -7) * 2.0 ** 127, 0.0, -0.0, np.inf]
    got = bf16_to_f64(bits)
    assert list(got) == want
    assert np.signbit(got[6])


# ------------------------------------------------------------- checkers

def test_check_f32_bounds():
    C = np.array([[1.0, -2.0, 0.0]])
    D = np.array([[10.0, 10.0, 0.0]])
    assert oracle.check_f32(np.array([[1.0 + 9e-5, -2.0 - 9e-5, 0.0]]), C, D).ok
    r = oracle.check_f32(np.array([[1.0 + 1.1e-4, -2.0, 0.0]]), C, D)
    assert not r.ok and r.n_bad == 1 and r.first_bad == (0, 0)
    assert not oracle.check_f32(np.array([[1.0, -2.0, 1e-30]]), C, D).ok   # D == 0 needs exact 0
    assert not oracle.check_f32(np.array([[np.nan, -2.0, 0.0]]), C, D).ok


def test_check_bf16_bracket():
    C = np.array([1.0 + 2.0 ** -9])        # a quarter ulp above 1.0: RNE gives 1.0
    D = np.array([1e-9])                   # tiny tolerance: only the RNE value passes
    ok_bits = rne_bf16(C)
    assert int(ok_bits[0]) == 0x3F80
    assert oracle.check_bf16(ok_bits, C, D).ok
    assert not oracle.check_bf16(np.array([0x3F81], np.uint16), C, D).ok
    assert not oracle.check_bf16(np.array([0x3F7F], np.uint16), C, D).ok
    # an exact tie: an accumulator a hair above or below it rounds either way,
    # so with any positive tolerance both neighbours are acceptable
    T = np.array([1.0 + 2.0 ** -8])
    assert oracle.check_bf16(np.array([0x3F80], np.uint16), T, D).ok
    assert oracle.check_bf16(np.array([0x3F81], np.uint16), T, D).ok
    assert not oracle.check_bf16(np.array([0x3F82], np.uint16), T, D).ok
    # with zero tolerance only the even neighbour of the tie passes
    assert not oracle.check_bf16(np.array([0x3F81], np.uint16), T, np.array([0.0])).ok
    assert not oracle.check_bf16(np.array([0x7FC0], np.uint16), C, np.array([1.0])).ok


def test_check_exact():
    C = np.array([[3.0, -7.0], [0.0, 1.0 + 2.0 ** -8]])
    assert oracle.check_exact(np.array([[3.0, -7.0], [-0.0, 1.0 + 2.0 ** -8]], np.float32), C, False).ok
    assert not oracle.check_exact(np.array([[3.0, -7.0], [0.0, 1.0]], np.float32), C, False).ok
    assert oracle.check_exact(rne_bf16(C), C, True).ok

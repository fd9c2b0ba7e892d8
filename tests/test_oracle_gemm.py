"""Pins for the fp64 GEMM oracle (CPU only).

Each pin comes from outside the oracle:
- Decoders are checked against torch's own float8_e4m3fn / bfloat16
  conversions and against closed-form values of the formats.
- Tiny problems are checked against exact rational arithmetic
  (fractions.Fraction) over torch-decoded inputs.
- A single expert reduces to a textbook GEMM: numpy float64 matmul.
- The fp8 result is checked against the per-128-group promotion form in exact
  arithmetic: sum over groups of (group dot product) * a_scale * b_scale.
- Integer inputs with small sums must come out exact.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl
from oracle import gemm as og


@pytest.fixture(scope="module", autouse=True)
def _built():
    og.build()
    og._lib = None
    og.lib()


# ------------------------------------------------------------- decoders


def test_e4m3_decoder_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for c in range(256):
        got = og.dec_e4m3(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == ref[c], hex(c)


def test_e4m3_closed_forms():
    assert og.dec_e4m3(0x7E) == 448.0              # largest finite
    assert og.dec_e4m3(0x01) == 2.0 ** -9          # smallest subnormal
    assert og.dec_e4m3(0x08) == 2.0 ** -6          # smallest normal
    assert og.dec_e4m3(0x38) == 1.0
    assert og.dec_e4m3(0xB8) == -1.0
    assert og.dec_e4m3(0x00) == 0.0


def test_bf16_decoder():
    """Every one of the 2^16 bf16 codes against torch's conversion (NaNs as NaNs)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = np.array([og.dec_bf16(int(b)) for b in bits.tolist()])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert og.dec_bf16(0x3F80) == 1.0 and og.dec_bf16(0xC000) == -2.0


# ------------------------------------------------------------- helpers


def _frac(t: torch.Tensor):
    """Exact rational values of a tensor (decoded by torch)."""
    return np.vectorize(Fraction, otypes=[object])(t.to(torch.float64).numpy())


def _exact_contiguous(A, B, counts, seg_align, As=None, Bs=None):
    """C rows by exact rational arithmetic straight from the definition."""
    a, b = _frac(A), _frac(B)
    if As is not None:
        sa, sb = _frac(As), _frac(Bs)
        for r in range(a.shape[0]):
            for k in range(a.shape[1]):
                a[r, k] *= sa[r, k // 128]
        for e in range(b.shape[0]):
            for k in range(b.shape[1]):
                for n in range(b.shape[2]):
                    b[e, k, n] *= sb[e, k // 128, n // 128]
    out = {}
    off = 0
    for e, m in enumerate(counts):
        for r in range(m):
            row = off + r
            out[row] = [sum(a[row, k] * b[e, k, n] for k in range(a.shape[1])) for n in range(b.shape[2])]
        off += -(-m // seg_align) * seg_align
    return out


def _small_bf16(shape, seed, lo=-1.0, hi=1.0):
    return wl.to_bf16(wl.fp32_uniform(shape, lo, hi, seed))


# ------------------------------------------------------------- contiguous


@pytest.mark.parametrize("seg_align", [1, 4])
def test_contiguous_bf16_exact_rational(seg_align):
    counts = [3, 0, 5, 1]
    rows_total = sum(-(-c // seg_align) * seg_align for c in counts)
    K, N = 7, 5
    A = _small_bf16((rows_total, K), 11)
    B = _small_bf16((len(counts), K, N), 12)
    exact = _exact_contiguous(A, B, counts, seg_align)
    got = og.contiguous(A, B, counts, list(range(rows_total)), seg_align=seg_align)
    for r in range(rows_total):
        if r in exact:
            assert [float(x) for x in exact[r]] == got[r].tolist()
        else:
            assert np.isnan(got[r]).all()                 # row belongs to no expert


def test_contiguous_b_layouts_agree():
    counts = [4, 2]
    A = _small_bf16((6, 9), 1)
    B = _small_bf16((2, 9, 6), 2)
    kn = og.contiguous(A, B, counts, range(6), b_layout=og.B_KN)
    nk = og.contiguous(A, B.transpose(1, 2).contiguous(), counts, range(6), b_layout=og.B_NK)
    assert np.array_equal(kn, nk)


def test_single_expert_is_textbook_gemm():
    A = _small_bf16((37, 64), 3)
    B = _small_bf16((1, 64, 48), 4)
    got = og.contiguous(A, B, [37], range(37))
    ref = A.to(torch.float64).numpy() @ B[0].to(torch.float64).numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_integer_inputs_exact():
    g = torch.Generator().manual_seed(5)
    A = torch.randint(-1, 2, (40, 200), generator=g).to(torch.bfloat16)
    B = torch.randint(-1, 2, (3, 200, 33), generator=g).to(torch.bfloat16)
    counts = [10, 0, 30]
    got = og.contiguous(A, B, counts, range(40))
    ref = np.concatenate([A[:10].double().numpy() @ B[0].double().numpy(),
                          A[10:].double().numpy() @ B[2].double().numpy()])
    assert np.array_equal(got, ref)


def test_contiguous_fp8_exact_rational_and_group_form():
    counts = [2, 0, 3]
    K, N = 256, 128
    x = wl.fp32_normal((5, K), 1.0, 21)
    w = wl.fp32_normal((3, K, N), 1.0, 22)
    qa, sa = wl.quantize_rows_e4m3(x)
    qb, sb = wl.quantize_blocks_e4m3(w)
    # a few output columns suffice for the exact check
    got = og.contiguous(qa, qb, counts, range(5), A_scale=sa, B_scale=sb)
    exact = _exact_contiguous(qa, qb, counts, 1, sa, sb)
    # fp64 summation bound: |got - exact| <= gamma_K * sum_k |a_k b_k|, gamma_K ~ K * 2^-53
    absum = _exact_contiguous(qa.view(torch.uint8).bitwise_and(0x7F).view(torch.float8_e4m3fn), 
                              qb.view(torch.uint8).bitwise_and(0x7F).view(torch.float8_e4m3fn),
                              counts, 1, sa.abs(), sb.abs())
    gamma = 2 * K * 2.0 ** -53
    for r, row in exact.items():
        for n in range(N):
            assert abs(got[r, n] - float(row[n])) <= gamma * float(absum[r][n])
    # per-group promotion form: sum_kb (sum_{k in kb} qa*qb) * a_s[r,kb] * b_s[e,kb,n/128]
    a, b = _frac(qa), _frac(qb)
    fa, fb = _frac(sa), _frac(sb)
    e_of = {0: 0, 1: 0, 2: 2, 3: 2, 4: 2}
    for r in range(5):
        e = e_of[r]
        for n in (0, 77, 127):
            tot = Fraction(0)
            for kb in range(K // 128):
                part = sum(a[r, k] * b[e, k, n] for k in range(kb * 128, kb * 128 + 128))
                tot += part * fa[r, kb] * fb[e, kb, n // 128]
            assert abs(got[r, n] - float(tot)) <= gamma * float(absum[r][n])


def test_contiguous_rejects_rows_outside_buffer():
    A = _small_bf16((4, 3), 1)
    B = _small_bf16((1, 3, 2), 2)
    with pytest.raises(ValueError):
        og.contiguous(A, B, [4], [4])


# ------------------------------------------------------------- masked


def test_masked_exact_and_invalid_rows():
    G, cap, K, N = 3, 6, 5, 4
    A = _small_bf16((G, cap, K), 31)
    B = _small_bf16((G, K, N), 32)
    mm = [2, 0, 6]
    reqs = [(e, r) for e in range(G) for r in range(cap)]
    got = og.masked(A, B, mm, [e for e, _ in reqs], [r for _, r in reqs])
    a, b = _frac(A), _frac(B)
    for i, (e, r) in enumerate(reqs):
        if r < mm[e]:
            ref = [float(sum(a[e, r, k] * b[e, k, n] for k in range(K))) for n in range(N)]
            assert got[i].tolist() == ref
        else:
            assert np.isnan(got[i]).all()


def test_masked_equals_contiguous_at_capacity_offsets():
    G, cap, K, N = 2, 8, 16, 8
    A = _small_bf16((G, cap, K), 41)
    B = _small_bf16((G, K, N), 42)
    mm = [5, 8]
    m = og.masked(A, B, mm, [0] * 5 + [1] * 8, list(range(5)) + list(range(8)))
    c = og.contiguous(A.reshape(G * cap, K), B, mm, list(range(5)) + list(range(8, 16)), seg_align=cap)
    assert np.array_equal(m, c)


# ------------------------------------------------------------- k-grouped


def test_k_grouped_exact_and_empty_expert():
    t = [3, 0, 4]
    T, Mw, Nw = 7, 5, 6
    X = _small_bf16((T, Mw), 51)
    dY = _small_bf16((T, Nw), 52)
    reqs = [(e, i) for e in range(3) for i in range(Mw)]
    got = og.k_grouped(X, dY, t, [e for e, _ in reqs], [i for _, i in reqs])
    x, y = _frac(X), _frac(dY)
    offs = [0, 3, 3, 7]
    for q, (e, i) in enumerate(reqs):
        ref = [float(sum(x[s, i] * y[s, j] for s in range(offs[e], offs[e + 1]))) for j in range(Nw)]
        assert got[q].tolist() == ref
    assert not got[[q for q, (e, _) in enumerate(reqs) if e == 1]].any()   # empty sum is 0


def test_k_grouped_is_transposed_product():
    t = [20, 13]
    X = _small_bf16((33, 24), 61)
    dY = _small_bf16((33, 16), 62)
    got = og.k_grouped(X, dY, t, [1] * 24, list(range(24)))
    ref = X[20:].double().numpy().T @ dY[20:].double().numpy()
    assert np.allclose(got, ref, rtol=1e-13, atol=1e-13)


# ------------------------------------------------------------- metric


def test_rel_frobenius():
    ref = np.array([3.0, 4.0])
    assert og.rel_frobenius(ref, ref) == 0.0
    assert og.rel_frobenius(np.array([3.0, 4.5]), ref) == pytest.approx(0.1)
    assert og.rel_frobenius(np.zeros(2), np.zeros(2)) == 0.0
    assert og.rel_frobenius(np.ones(2), np.zeros(2)) == float("inf")


def test_bf16_rounding_alone_sits_under_the_bar():
    """Rounding an exact Gaussian GEMM result once to bf16 costs ~1.7e-3 < 2e-3."""
    A = wl.to_bf16(wl.fp32_normal((256, 512), 512 ** -0.5, 71))
    B = wl.to_bf16(wl.fp32_normal((1, 512, 256), 512 ** -0.5, 72))
    ref = og.contiguous(A, B, [256], range(256))
    rounded = torch.from_numpy(ref).to(torch.bfloat16).double().numpy()
    err = og.rel_frobenius(rounded, ref)
    assert 1.0e-3 < err < 2.0e-3

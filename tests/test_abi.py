"""The C ABI on the host (no GPU needed): the library loads and exports every
symbol include/moegg.h declares, and host-side validation rejects bad
arguments before anything is enqueued.  No call here reaches a launch."""
import ctypes
import re

import pytest

import moe_grouped_gemm_sizes_amd as mg


def declared_functions():
    src = open(mg.HEADER_PATH).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moegg_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(mg.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = mg.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.moegg_version() >> 16 == 0


def test_status_strings():
    L = mg.lib()
    for s in range(5):
        assert L.moegg_status_string(s)
    assert L.moegg_status_string(99) == b"unknown status"


def test_workspace_bytes():
    L = mg.lib()
    assert L.moegg_workspace_bytes(0, 10) == 0
    assert L.moegg_workspace_bytes(4097, 10) == 0
    assert L.moegg_workspace_bytes(8, -1) == 0
    small = L.moegg_workspace_bytes(8, 132)
    big = L.moegg_workspace_bytes(8, 1 << 20)
    assert small > 0 and small % 256 == 0
    assert big >= small + 16 * ((1 << 20) // 64)          # one 16-byte entry per 64-row tile


FAKE = ctypes.c_void_p(0x100000)        # aligned, never dereferenced: validation fails first


def contiguous(**kw):
    args = dict(A=FAKE, A_scale=None, B=FAKE, B_scale=None, C=FAKE, m=FAKE, G=8, rows=132, K=512, N=256,
                align=1, dtype=mg.BF16, layout=mg.B_KN, block_m=0, ws=FAKE, ws_bytes=1 << 20)
    args.update(kw)
    return mg.lib().moegg_grouped_gemm_contiguous(*args.values(), None)


@pytest.mark.parametrize("kw,status", [
    (dict(A=None), mg.ERR_INVALID_ARG),
    (dict(m=None), mg.ERR_INVALID_ARG),
    (dict(G=0), mg.ERR_INVALID_ARG),
    (dict(G=5000), mg.ERR_INVALID_ARG),
    (dict(K=100), mg.ERR_UNSUPPORTED),
    (dict(N=200), mg.ERR_UNSUPPORTED),
    (dict(dtype=7), mg.ERR_INVALID_ARG),
    (dict(layout=7), mg.ERR_INVALID_ARG),
    (dict(dtype=mg.FP8_E4M3), mg.ERR_INVALID_ARG),                 # fp8 without scales
    (dict(dtype=mg.FP8_E4M3, A_scale=FAKE, B_scale=FAKE, K=192), mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_SCALE_KM), mg.ERR_INVALID_ARG),         # transposed fp32 scales, none given
    (dict(dtype=mg.FP8_E4M3_SCALE_KM, A_scale=FAKE, B_scale=FAKE, K=192), mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_SCALE_KM, A_scale=ctypes.c_void_p(0x100002), B_scale=FAKE), mg.ERR_INVALID_ARG),
    # transposed scales beyond 32-bit offsets: K/128 * rows fp32 scales over 4 GiB, E8M0 bytes over 4 GiB
    (dict(dtype=mg.FP8_E4M3_SCALE_KM, A_scale=FAKE, B_scale=FAKE, K=7168, rows=20_000_000), mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_E8M0, A_scale=FAKE, B_scale=FAKE, N=512, K=131072, rows=40_000_000),
     mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_E8M0), mg.ERR_INVALID_ARG),            # E8M0 without scales
    (dict(dtype=mg.FP8_E4M3_E8M0, A_scale=FAKE, B_scale=FAKE, N=768), mg.ERR_UNSUPPORTED),   # N % 512
    (dict(dtype=mg.FP8_E4M3_E8M0, A_scale=FAKE, B_scale=FAKE, N=512, rows=130), mg.ERR_UNSUPPORTED),  # rows % 4
    (dict(dtype=mg.FP8_E4M3_E8M0, A_scale=FAKE, B_scale=ctypes.c_void_p(0x100002), N=512), mg.ERR_INVALID_ARG),
    (dict(dtype=mg.FP8_E4M3_FP4_E2M1), mg.ERR_INVALID_ARG),        # fp4 weights without scales
    (dict(dtype=mg.FP8_E4M3_FP4_E2M1, A_scale=FAKE, B_scale=FAKE, N=512), mg.ERR_UNSUPPORTED),   # [G,K,N] fp4
    (dict(dtype=mg.FP8_E4M3_FP4_E2M1, A_scale=FAKE, B_scale=FAKE, N=768, layout=mg.B_NK), mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_FP4_E2M1, A_scale=FAKE, B_scale=FAKE, N=512, layout=mg.B_NK, rows=130),
     mg.ERR_UNSUPPORTED),
    (dict(dtype=mg.FP8_E4M3_FP4_E2M1, A_scale=FAKE, B_scale=FAKE, N=512, layout=mg.B_NK, K=192),
     mg.ERR_UNSUPPORTED),
    (dict(block_m=32), mg.ERR_UNSUPPORTED),
    (dict(block_m=-2), mg.ERR_UNSUPPORTED),
    (dict(align=0), mg.ERR_INVALID_ARG),
    (dict(rows=-1), mg.ERR_INVALID_ARG),
    (dict(ws=None), mg.ERR_WORKSPACE),
    (dict(ws_bytes=64), mg.ERR_WORKSPACE),
    (dict(ws=ctypes.c_void_p(0x100010)), mg.ERR_WORKSPACE),        # not 256-byte aligned
    (dict(A=ctypes.c_void_p(0x100001)), mg.ERR_INVALID_ARG),       # not 16-byte aligned
])
def test_contiguous_validation(kw, status):
    assert contiguous(**kw) == status


def test_masked_validation():
    L = mg.lib()
    f = L.moegg_grouped_gemm_masked
    ok = [FAKE, None, FAKE, None, FAKE, FAKE, 32, 256, 2048, 7168, mg.BF16, mg.B_KN, None, 0, None]
    bad_cap = list(ok)
    bad_cap[7] = 0
    assert f(*bad_cap) == mg.ERR_INVALID_ARG
    bad_n = list(ok)
    bad_n[9] = 100
    assert f(*bad_n) == mg.ERR_UNSUPPORTED
    small_ws = list(ok)
    small_ws[12], small_ws[13] = FAKE, 16
    assert f(*small_ws) == mg.ERR_WORKSPACE
    e8m0 = list(ok)                         # E8M0 scale bytes [K/128, G * cap] need G * cap % 4 == 0
    e8m0[1], e8m0[3], e8m0[6], e8m0[7], e8m0[10] = FAKE, FAKE, 31, 255, mg.FP8_E4M3_E8M0
    assert f(*e8m0) == mg.ERR_UNSUPPORTED
    w4 = list(e8m0)                         # fp4 weights: K-contiguous only, then the same row rule
    w4[10] = mg.FP8_E4M3_FP4_E2M1
    assert f(*w4) == mg.ERR_UNSUPPORTED
    w4[11] = mg.B_NK
    assert f(*w4) == mg.ERR_UNSUPPORTED
    e8n = list(e8m0)                        # E8M0 also needs N % 512 == 0
    e8n[6], e8n[7], e8n[9] = 32, 256, 7168 + 256
    assert f(*e8n) == mg.ERR_UNSUPPORTED


def test_k_grouped_validation():
    f = mg.lib().moegg_grouped_gemm_k_grouped
    assert f(None, FAKE, FAKE, FAKE, 16, 100, 2048, 7168, FAKE, 1 << 20, None) == mg.ERR_INVALID_ARG
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 100, 2000, 7168, FAKE, 1 << 20, None) == mg.ERR_UNSUPPORTED
    assert f(FAKE, FAKE, FAKE, FAKE, 16, 100, 2048, 7168, None, 0, None) == mg.ERR_WORKSPACE


def test_schedule_validation():
    f = mg.lib().moegg_schedule
    assert f(None, 8, 132, 1, 0, 256, FAKE, 1 << 20, None) == mg.ERR_INVALID_ARG
    assert f(FAKE, 8, 132, 1, 48, 256, FAKE, 1 << 20, None) == mg.ERR_UNSUPPORTED
    assert f(FAKE, 8, 132, 1, 0, 256, FAKE, 8, None) == mg.ERR_WORKSPACE
    assert f(FAKE, 8, 132, 1, 0, 0, FAKE, 1 << 20, None) == mg.ERR_INVALID_ARG


def test_scheduled_validation():
    f = mg.lib().moegg_grouped_gemm_contiguous_scheduled
    args = [FAKE, None, FAKE, None, FAKE, 8, 132, 512, 256, mg.BF16, mg.B_KN, 0, FAKE, 1 << 20, None]
    bad = list(args); bad[12] = None
    assert f(*bad) == mg.ERR_WORKSPACE
    bad = list(args); bad[11] = 96
    assert f(*bad) == mg.ERR_UNSUPPORTED
    bad = list(args); bad[0] = None
    assert f(*bad) == mg.ERR_INVALID_ARG


def test_schedule_exemplar_validation():
    f = mg.lib().moegg_schedule_exemplar
    ok = [FAKE, 8, 132, 1, 256, FAKE, 4, 0, FAKE, 1 << 20, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)
    assert call(a0=None) == mg.ERR_INVALID_ARG          # counts
    assert call(a1=0) == mg.ERR_INVALID_ARG             # G
    assert call(a4=0) == mg.ERR_INVALID_ARG             # N
    assert call(a5=None) == mg.ERR_INVALID_ARG          # table
    assert call(a6=0) == mg.ERR_INVALID_ARG             # empty table
    assert call(a6=257) == mg.ERR_UNSUPPORTED           # more than MOEGG_MAX_EXEMPLARS
    assert call(a7=-1) == mg.ERR_INVALID_ARG            # negative hysteresis
    assert call(a8=None) == mg.ERR_WORKSPACE
    assert call(a9=16) == mg.ERR_WORKSPACE
    assert mg.lib().moegg_selection_read(None, None, None) == mg.ERR_INVALID_ARG


def test_exemplar_struct_matches_the_header():
    src = open(mg.HEADER_PATH).read()
    assert "int32_t lorenz[8];" in src and mg.EXEMPLAR_FIELDS == 10
    assert ctypes.sizeof(mg._Selection) == 48


def test_swiglu_validation():
    f = mg.lib().moegg_grouped_gemm_swiglu_scheduled
    ok = [FAKE, None, FAKE, None, FAKE, None, 8, 132, 512, 128, mg.BF16, mg.B_NK, 0, FAKE, 1 << 20, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(0, None) == mg.ERR_INVALID_ARG              # A
    assert call(9, 0) == mg.ERR_INVALID_ARG                 # I
    assert call(9, 64) == mg.ERR_UNSUPPORTED                # 2I % 256
    assert call(11, mg.B_KN) == mg.ERR_UNSUPPORTED          # W1 must be K-contiguous
    assert call(10, mg.FP8_E4M3_E8M0) == mg.ERR_INVALID_ARG  # no scales given
    assert call(13, None) == mg.ERR_WORKSPACE
    assert call(12, 48) == mg.ERR_UNSUPPORTED               # block_m
    assert call(5, ctypes.c_void_p(0x100002)) == mg.ERR_INVALID_ARG   # H_scale alignment


def test_expert_mlp_fused_validation():
    f = mg.lib().moegg_expert_mlp_fused
    ok = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 8, 132, 512, 256, 512, 1, mg.FP8_E4M3,
          mg.B_NK, FAKE, 1 << 20, None]

    def call(i, v):
        a = list(ok)
        a[i] = v
        return f(*a)
    assert call(9, None) == mg.ERR_INVALID_ARG              # m_sizes
    assert call(0, None) == mg.ERR_INVALID_ARG              # A
    assert call(7, None) == mg.ERR_INVALID_ARG              # H_scale
    assert call(13, 0) == mg.ERR_INVALID_ARG                # I
    assert call(13, 64) == mg.ERR_UNSUPPORTED               # 2I % 256
    assert call(14, 128) == mg.ERR_UNSUPPORTED              # N2 % 256
    assert call(16, mg.BF16) == mg.ERR_UNSUPPORTED          # e4m3 with fp32 scales only
    assert call(17, mg.B_KN) == mg.ERR_UNSUPPORTED          # weights must be K-contiguous
    assert call(18, None) == mg.ERR_WORKSPACE
    assert call(19, 1024) == mg.ERR_WORKSPACE               # too small


def test_read_validation():
    L = mg.lib()
    assert L.moegg_stats_read(None, None, None) == mg.ERR_INVALID_ARG
    n = ctypes.c_int64(0)
    assert L.moegg_tile_list_read(FAKE, None, 5, ctypes.byref(n), None) == mg.ERR_INVALID_ARG


def test_k_grouped_accepts_null_operands_only_without_rows():
    f = mg.lib().moegg_grouped_gemm_k_grouped
    # T = 0: X and dY are never read, so NULL passes validation (and fails later only on the workspace)
    assert f(None, None, FAKE, FAKE, 16, 0, 2048, 7168, None, 0, None) == mg.ERR_WORKSPACE
    assert f(None, None, FAKE, FAKE, 16, 1, 2048, 7168, None, 0, None) == mg.ERR_INVALID_ARG


def test_scale_km_dtype_code():
    """scale_km selects the transposed-fp32-scale format, and only for e4m3 with fp32 scales."""
    import torch
    G, rows, K, N = 2, 4, 128, 256
    a8 = torch.empty(rows, K, dtype=torch.float8_e4m3fn)
    b8 = torch.empty(G, K, N, dtype=torch.float8_e4m3fn)
    bs = torch.empty(G, 1, 2)
    assert mg._operands(rows, K, a8, torch.empty(1, rows), b8, bs, G, mg.B_KN, True) == (mg.FP8_E4M3_SCALE_KM, N)
    assert mg._operands(rows, K, a8, torch.empty(rows, 1), b8, bs, G, mg.B_KN, False) == (mg.FP8_E4M3, N)
    with pytest.raises(ValueError):
        mg._operands(rows, K, torch.empty(rows, K, dtype=torch.bfloat16), None,
                     torch.empty(G, K, N, dtype=torch.bfloat16), None, G, mg.B_KN, True)
    with pytest.raises(ValueError):
        mg._operands(rows, K, a8, torch.empty(1, rows, dtype=torch.uint8), b8, bs.to(torch.uint8), G, mg.B_KN, True)


def _stats_from_oracle(counts):
    from oracle import accounting as acc
    s = acc.summary(counts)
    P = [s["P"][q] for q in mg.Q_VALUES]
    return mg.Stats(s["U"], s["P"][16], s["tiles"][256], s["active"], s["sum_sq"], 0,
                    dict(zip(mg.Q_VALUES, P)), 256, 0), s


@pytest.mark.parametrize("counts", [
    [17, 17, 17, 17, 16, 16, 16, 16], [100, 32, 0, 0, 0, 0, 0, 0], [0, 0, 0], [1],
    [4, 1026, 1799, 166, 694, 753, 0, 16, 0, 240, 1119, 19, 6, 0, 46, 659,
     10, 0, 112, 808, 181, 0, 28, 22, 90, 0, 176, 0, 37, 5, 10, 22],
    [2 ** 31 - 1, 3],
])
def test_stats_report_matches_the_exact_ratios(counts):
    """moegg_stats_report (host C) against the oracle's exact Fractions: each ratio
    is the exact one rounded to double (within one ulp)."""
    import math
    from fractions import Fraction
    from oracle import accounting as acc
    st, s = _stats_from_oracle(counts)
    r = st.report()

    def close(got, exact):
        return got == float(exact) or abs(got - float(exact)) <= math.ulp(float(exact))
    assert close(r.effective_experts, s["effective_experts"])
    for q in mg.Q_VALUES:
        assert close(r.padding_fraction[q], acc.padding_fraction(counts, q))
        P = s["P"][q]
        assert close(r.useful_share[q], Fraction(s["U"], P) if P else 0)
    P16 = s["P"][16]
    assert close(r.exec_padding_fraction, Fraction(P16 - s["U"], P16) if P16 else 0)
    assert close(r.physical_over_effective, Fraction(P16, s["U"]) if s["U"] else 0)


def test_stats_report_worked_values():
    """The padding page's printed values, through the library's report."""
    st, _ = _stats_from_oracle([17, 17, 17, 17, 16, 16, 16, 16])
    r = st.report()
    assert [round(100 * r.padding_fraction[q], 2) for q in (8, 16, 32)] == [17.5, 31.25, 48.44]
    assert round(100 * r.useful_share[8], 1) == 82.5 and round(100 * r.useful_share[32], 1) == 51.6
    assert 7.9 < r.effective_experts < 8
    st, _ = _stats_from_oracle([100, 32, 0, 0, 0, 0, 0, 0])
    r = st.report()
    assert round(100 * r.padding_fraction[8], 1) == 2.9 and round(100 * r.padding_fraction[32], 1) == 17.5
    assert round(r.effective_experts, 2) == 1.58


def test_stats_report_rejects_bad_input():
    L = mg.lib()
    assert L.moegg_stats_report(None, None) == mg.ERR_INVALID_ARG
    st = mg._Stats()
    st.U = -1
    assert L.moegg_stats_report(ctypes.byref(st), ctypes.byref(mg._Report())) == mg.ERR_INVALID_ARG

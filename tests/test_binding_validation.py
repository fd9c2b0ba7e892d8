"""The Python binding checks every tensor it hands to the C ABI (CPU only).

The library sees plain pointers, so a buffer that is too small or of the wrong
type would make a kernel read or write outside it.  The binding therefore
checks the shape, dtype and device of every operand against the sizes it
passes, and raises ValueError naming the argument before any library call.
Each case below builds a correct set of (CPU) tensors, changes one of them,
and expects that argument's name in the error; the unchanged set gets as far as
the device check.
"""
import pytest
import torch

import moe_grouped_gemm_sizes_amd as mg

E4M3 = torch.float8_e4m3fn
G, ROWS, K, N = 3, 40, 256, 512


def t(*shape, dtype=torch.float32):
    return torch.zeros(*shape, dtype=dtype)


def contiguous_args(dtype="bf16", b_layout=mg.B_KN):
    kw = dict(m_sizes=t(G, dtype=torch.int32), ws=t(mg.workspace_bytes(G, ROWS), dtype=torch.uint8),
              C=t(ROWS, N, dtype=torch.bfloat16), b_layout=b_layout)
    bshape = (G, K, N) if b_layout == mg.B_KN else (G, N, K)
    if dtype == "bf16":
        kw.update(A=t(ROWS, K, dtype=torch.bfloat16), B=t(*bshape, dtype=torch.bfloat16))
    elif dtype == "fp8":
        kw.update(A=t(ROWS, K, dtype=E4M3), B=t(*bshape, dtype=E4M3), A_scale=t(ROWS, K // 128),
                  B_scale=t(G, K // 128, N // 128))
    elif dtype == "fp8_km":
        kw.update(A=t(ROWS, K, dtype=E4M3), B=t(*bshape, dtype=E4M3), A_scale=t(K // 128, ROWS),
                  B_scale=t(G, K // 128, N // 128), scale_km=True)
    elif dtype == "e8m0":
        kw.update(A=t(ROWS, K, dtype=E4M3), B=t(*bshape, dtype=E4M3), A_scale=t(K // 128, ROWS, dtype=torch.uint8),
                  B_scale=t(G, K // 128, N // 128, dtype=torch.uint8))
    elif dtype == "fp4":
        kw.update(A=t(ROWS, K, dtype=E4M3), B=t(G, N, K // 2, dtype=torch.uint8),
                  A_scale=t(K // 128, ROWS, dtype=torch.uint8), B_scale=t(G, K // 128, N // 128, dtype=torch.uint8),
                  b_layout=mg.B_NK)
    return kw


def call_contiguous(kw):
    mg.grouped_gemm_contiguous(**kw)


@pytest.mark.parametrize("dtype,layout", [("bf16", mg.B_KN), ("bf16", mg.B_NK), ("fp8", mg.B_NK),
                                          ("fp8_km", mg.B_KN), ("e8m0", mg.B_NK), ("fp4", mg.B_NK)])
def test_contiguous_correct_arguments_reach_the_device_check(dtype, layout):
    with pytest.raises(ValueError, match="device tensor expected"):
        call_contiguous(contiguous_args(dtype, layout))


@pytest.mark.parametrize("dtype,change,name", [
    ("bf16", dict(C=t(ROWS - 1, N, dtype=torch.bfloat16)), "C: shape"),
    ("bf16", dict(C=t(ROWS, N, dtype=torch.float32)), "C: dtype"),
    ("bf16", dict(B=t(G + 1, K, N, dtype=torch.bfloat16)), "B: shape"),
    ("bf16", dict(B=t(G, K + 64, N, dtype=torch.bfloat16)), "B: shape"),
    ("bf16", dict(B=t(G, K, N, dtype=E4M3)), "B: dtype"),
    ("bf16", dict(A_scale=t(ROWS, 2)), "A_scale: must be None"),
    ("bf16", dict(m_sizes=t(G, dtype=torch.int64)), "m_sizes: dtype"),
    ("bf16", dict(m_sizes=t(G, 1, dtype=torch.int32)), "m_sizes: shape"),
    ("bf16", dict(ws=t(64, dtype=torch.uint8)), "ws: 64 bytes"),
    ("bf16", dict(A=t(ROWS, K)), "A: dtype"),
    ("fp8", dict(A_scale=t(ROWS, K // 128 + 1)), "A_scale: shape"),
    ("fp8", dict(A_scale=t(K // 128, ROWS)), "A_scale: shape"),
    ("fp8", dict(B_scale=t(G, K // 128, N // 256)), "B_scale: shape"),
    ("fp8", dict(B_scale=None), "need A_scale and B_scale"),
    ("fp8", dict(B=t(G, K, N, dtype=torch.bfloat16)), "B: dtype"),
    ("fp8_km", dict(A_scale=t(ROWS, K // 128)), "A_scale: shape"),
    ("e8m0", dict(B_scale=t(G, K // 128, N // 128)), "B_scale: dtype"),
    ("e8m0", dict(A_scale=t(ROWS, K // 128, dtype=torch.uint8)), "A_scale: shape"),
    ("fp4", dict(B=t(G, N, K, dtype=torch.uint8)), "B: shape"),
    ("fp4", dict(b_layout=mg.B_KN), r"\(B_NK\) or its panels"),
    ("fp4", dict(b_layout=mg.B_NK_PANEL), "B: shape"),
])
def test_contiguous_mismatch_raises(dtype, change, name):
    kw = contiguous_args(dtype, mg.B_KN if dtype in ("bf16", "fp8_km") else mg.B_NK)
    kw.update(change)
    with pytest.raises(ValueError, match=name):
        call_contiguous(kw)


def test_contiguous_scheduled_checks_against_G():
    kw = contiguous_args("bf16")
    kw.pop("m_sizes")
    with pytest.raises(ValueError, match="device tensor expected"):
        mg.grouped_gemm_contiguous_scheduled(G=G, **kw)
    with pytest.raises(ValueError, match="B: shape"):
        mg.grouped_gemm_contiguous_scheduled(G=G + 1, **kw)


def masked_args(dtype="bf16"):
    cap = 16
    kw = dict(masked_m=t(G, dtype=torch.int32), C=t(G, cap, N, dtype=torch.bfloat16),
              ws=t(mg.workspace_bytes(G, G * cap), dtype=torch.uint8), b_layout=mg.B_KN)
    if dtype == "bf16":
        kw.update(A=t(G, cap, K, dtype=torch.bfloat16), B=t(G, K, N, dtype=torch.bfloat16))
    else:
        kw.update(A=t(G, cap, K, dtype=E4M3), B=t(G, K, N, dtype=E4M3), A_scale=t(G, cap, K // 128),
                  B_scale=t(G, K // 128, N // 128))
    return kw


@pytest.mark.parametrize("dtype,change,name", [
    ("bf16", dict(C=t(G, 15, N, dtype=torch.bfloat16)), "C: shape"),
    ("bf16", dict(masked_m=t(G + 1, dtype=torch.int32)), "masked_m: shape"),
    ("bf16", dict(B=t(G, K, N + 128, dtype=torch.bfloat16)), "C: shape"),
    ("bf16", dict(ws=t(8, dtype=torch.uint8)), "ws: 8 bytes"),
    ("fp8", dict(A_scale=t(G * 16, K // 128)), "A_scale: shape"),
    ("fp8", dict(B_scale=t(G, K // 128, 1)), "B_scale: shape"),
])
def test_masked_mismatch_raises(dtype, change, name):
    kw = masked_args(dtype)
    with pytest.raises(ValueError, match="device tensor expected"):
        mg.grouped_gemm_masked(**kw)
    kw.update(change)
    with pytest.raises(ValueError, match=name):
        mg.grouped_gemm_masked(**kw)


def swiglu_args():
    I = 256
    return dict(A=t(ROWS, K, dtype=E4M3), W1=t(G, 2 * I, K, dtype=E4M3), H=t(ROWS, I, dtype=E4M3),
                G=G, ws=t(mg.workspace_bytes(G, ROWS), dtype=torch.uint8), A_scale=t(ROWS, K // 128),
                W1_scale=t(G, K // 128, 2 * I // 128), H_scale=t(ROWS, I // 128))


@pytest.mark.parametrize("change,name", [
    (dict(H=t(ROWS, 128, dtype=E4M3)), "H: shape"),
    (dict(H_scale=t(2, ROWS)), "H_scale: shape"),
    (dict(H=t(ROWS, 256, dtype=torch.bfloat16)), "H: dtype"),
    (dict(W1=t(G, 384, K, dtype=E4M3), W1_scale=t(G, K // 128, 3)), "multiple of 256"),
])
def test_swiglu_mismatch_raises(change, name):
    kw = swiglu_args()
    with pytest.raises(ValueError, match="device tensor expected"):
        mg.grouped_gemm_swiglu_scheduled(**kw)
    kw.update(change)
    with pytest.raises(ValueError, match=name):
        mg.grouped_gemm_swiglu_scheduled(**kw)


def k_grouped_args(fp8=False):
    T, Mw, Nw = 300, 256, 512
    d = E4M3 if fp8 else torch.bfloat16
    kw = dict(X=t(T, Mw, dtype=d), dY=t(T, Nw, dtype=d), dW=t(G, Mw, Nw), t_sizes=t(G, dtype=torch.int32),
              ws=t(mg.workspace_bytes(G, 0), dtype=torch.uint8))
    if fp8:
        kw.update(X_scale=t(6, Mw), dY_scale=t(6, Nw))
    return kw


@pytest.mark.parametrize("fp8,change,name", [
    (False, dict(dW=t(G, 256, 256)), "dW: shape"),
    (False, dict(dW=t(G, 256, 512, dtype=torch.bfloat16)), "dW: dtype"),
    (False, dict(dY=t(299, 512, dtype=torch.bfloat16)), "dY: shape"),
    (False, dict(X_scale=t(6, 256)), "X_scale: must be None"),
    (True, dict(dY=t(300, 512, dtype=torch.bfloat16)), "dY: dtype"),
    (True, dict(X_scale=t(6, 512)), "X_scale: shape"),
    (True, dict(dY_scale=t(5, 512)), "dY_scale: shape"),
    (True, dict(X_scale=None), "X_scale: tensor expected"),
    (True, dict(dY_scale=t(6, 512, dtype=torch.uint8)), "dY_scale: dtype"),
    (True, dict(X_scale=t(6, 256, dtype=torch.int32)), "X_scale: dtype"),
])
def test_k_grouped_mismatch_raises(fp8, change, name):
    kw = k_grouped_args(fp8)
    with pytest.raises(ValueError, match="device tensor expected"):
        mg.grouped_gemm_k_grouped(**kw)
    kw.update(change)
    with pytest.raises(ValueError, match=name):
        mg.grouped_gemm_k_grouped(**kw)


def test_schedule_checks_counts_and_workspace():
    with pytest.raises(ValueError, match="m_sizes: dtype"):
        mg.schedule(t(4, dtype=torch.int64), 100, t(4096, dtype=torch.uint8))
    with pytest.raises(ValueError, match="ws: 16 bytes"):
        mg.schedule(t(4, dtype=torch.int32), 100, t(16, dtype=torch.uint8))


def test_k_scale_groups():
    assert mg.k_scale_groups([0, 1, 128, 129, 256, -5]) == 0 + 1 + 1 + 2 + 2 + 0


def test_pack_panels_index_mapping():
    """pack_panels places B[e, k, n] where the panel layouts say (checked element by element)."""
    G, K, N = 2, 256, 512
    B = torch.arange(G * K * N, dtype=torch.int64).reshape(G, K, N)
    kn = mg.pack_panels(B, mg.B_KN_PANEL, 256)
    assert kn.shape == (G, N // 256, K, 256)
    for e, k, n in [(0, 0, 0), (1, 255, 511), (0, 17, 300), (1, 128, 255), (1, 3, 256)]:
        assert kn[e, n // 256, k, n % 256] == B[e, k, n]
    Bh = B.to(torch.int16)                                   # 2-byte elements: S = 64
    nk = mg.pack_panels(Bh, mg.B_NK_PANEL, 128)
    assert nk.shape == (G, N // 128, K // 64, 128, 64)
    for e, k, n in [(0, 0, 0), (1, 255, 511), (0, 70, 300), (1, 191, 129)]:
        assert nk[e, n // 128, k // 64, n % 128, k % 64] == Bh[e, k, n]
    B8 = B.to(torch.uint8).view(torch.float8_e4m3fn)         # 1-byte elements: S = 128
    nk8 = mg.pack_panels(B8, mg.B_NK_PANEL, 256).view(torch.uint8)
    assert nk8.shape == (G, N // 256, K // 128, 256, 128)
    assert nk8[1, 1, 1, 7, 5] == B8.view(torch.uint8)[1, 128 + 5, 256 + 7]


def test_panel_shapes_are_checked():
    kw = contiguous_args("bf16")
    kw["b_layout"] = mg.B_KN_PANEL
    kw["B"] = t(G, N // 256, K, 256, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="device tensor expected"):
        call_contiguous(kw)
    kw["B"] = t(G, N // 128, K, 128, dtype=torch.bfloat16)     # masked panel width on a contiguous call
    with pytest.raises(ValueError, match="B: shape"):
        call_contiguous(kw)


def mlp_args(scale_km=False):
    I, N2 = 256, 512
    return dict(A=t(ROWS, K, dtype=E4M3), W1=t(G, 2 * I, K, dtype=E4M3), W2=t(G, N2, I, dtype=E4M3),
                H=t(ROWS, I, dtype=E4M3), Y=t(ROWS, N2, dtype=torch.bfloat16), m_sizes=t(G, dtype=torch.int32),
                ws=t(mg.workspace_bytes(G, ROWS), dtype=torch.uint8),
                A_scale=t(K // 128, ROWS) if scale_km else t(ROWS, K // 128), W1_scale=t(G, K // 128, 2 * I // 128),
                W2_scale=t(G, I // 128, N2 // 128), H_scale=t(I // 128, ROWS) if scale_km else t(ROWS, I // 128),
                scale_km=scale_km)


@pytest.mark.parametrize("scale_km", [False, True])
def test_expert_mlp_fused_correct_arguments_reach_the_device_check(scale_km):
    with pytest.raises(ValueError, match="device tensor expected"):
        mg.expert_mlp_fused(**mlp_args(scale_km))


@pytest.mark.parametrize("change,name", [
    (dict(H=t(ROWS, 384, dtype=E4M3)), "H: shape"),
    (dict(H_scale=t(ROWS, 1)), "H_scale: shape"),
    (dict(Y=t(ROWS, 512)), "Y: dtype"),
    (dict(Y=t(ROWS, 256, dtype=torch.bfloat16)), "Y: shape"),
    (dict(W2=t(G, 512, 384, dtype=E4M3)), "B: shape"),
    (dict(W1=t(G, 384, K, dtype=E4M3), W1_scale=t(G, K // 128, 3)), "multiple of 256"),
    (dict(A=t(ROWS, K, dtype=torch.bfloat16)), "A: dtype"),
    (dict(m_sizes=t(G, dtype=torch.int64)), "m_sizes: dtype"),
    (dict(ws=t(16, dtype=torch.uint8)), "ws:"),
])
def test_expert_mlp_fused_mismatch_raises(change, name):
    kw = mlp_args()
    kw.update(change)
    with pytest.raises(ValueError, match=name):
        mg.expert_mlp_fused(**kw)


def test_pack_panels_fp4():
    """Packed E2M1 [G, N, K/2] -> [G, N/P, K/128, P, 64]: K step s of panel p holds
    rows p*P .. p*P+P-1, bytes 64 s .. 64 s + 63 of each, in row order."""
    G, N, K, P = 2, 512, 512, 256
    B = torch.randint(0, 256, (G, N, K // 2), dtype=torch.uint8)
    Q = mg.pack_panels(B, mg.B_NK_PANEL, P)
    assert Q.shape == (G, N // P, K // 128, P, 64)
    for g, p, s, r in ((0, 0, 0, 0), (1, 1, 3, 255), (0, 1, 2, 17), (1, 0, 1, 200)):
        assert torch.equal(Q[g, p, s, r], B[g, p * P + r, 64 * s:64 * s + 64])
    with pytest.raises(ValueError, match="B_NK_PANEL panel layout only"):
        mg.pack_panels(B, mg.B_KN_PANEL, P)
    with pytest.raises(ValueError, match="must be 0"):
        mg.pack_panels(B[:, :, :96].contiguous(), mg.B_NK_PANEL, P)

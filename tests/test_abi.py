"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments with the documented status before
anything is enqueued (all of these return before any HIP call)."""
import ctypes
import os
import re

import pytest

import mxfp8_block_scaled_mx_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp8.h")

OK, EINVAL, ESHAPE, EALIGN, EWORKSPACE, EHIP, EUNSUPPORTED = range(7)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(mx.lib_path()):
        pytest.skip("library not built")
    return mx.load()


def test_exports_every_declared_symbol(L):
    decl = re.findall(r"MX_API\s+[\w\s\*]+?\b(\w+)\s*\(", open(HEADER).read())
    assert set(decl) >= {"mx_quantize", "mx_grouped_gemm", "grouped_mlp_fwd", "grouped_mlp_bwd",
                         "grouped_mlp_sizes", "mx_status_string", "mx_last_error", "mx_version"}
    for name in decl:
        assert hasattr(L, name), name
    assert L.mx_version() == 1
    assert L.mx_status_string(ESHAPE) == b"MX_ESHAPE"


FAKE = ctypes.c_void_p(0x100000)       # never dereferenced: validation fails first


def _q(L, x=FAKE, dt=0, rows=64, cols=64, gs=None, ng=0, qr=FAKE, sr=FAKE, qc=None, sc=None):
    return L.mx_quantize(x, dt, rows, cols, gs, ng, qr, sr, qc, sc, None)


def test_quantize_argument_errors(L):
    assert _q(L, x=None) == EINVAL
    assert _q(L, dt=7) == EINVAL
    assert _q(L, qr=None, sr=None) == EINVAL                   # nothing requested
    assert _q(L, sr=None) == EINVAL                            # half a pair
    assert _q(L, cols=48) == ESHAPE                            # cols % 32
    assert _q(L, cols=0) == ESHAPE
    assert _q(L, rows=-1) == ESHAPE
    assert _q(L, gs=mx._i64_array([30, 30]), ng=2) == ESHAPE   # sum != rows
    assert _q(L, gs=mx._i64_array([80, -16]), ng=2) == ESHAPE
    assert _q(L, gs=mx._i64_array([1] * 200), ng=200, rows=200) == EUNSUPPORTED
    assert _q(L, x=ctypes.c_void_p(0x100008)) == EALIGN
    assert b"mx_quantize" in L.mx_last_error()


def _g(L, mode=0, G=2, sizes=(32, 32), M=64, N=64, K=64, lda=64, ldb=64, bgs=4096, c_dt=1,
       ldc=64, cgs=0, acc=0, a=FAKE, c=FAKE):
    return L.mx_grouped_gemm(mode, G, mx._i64_array(sizes), M, N, K, a, FAKE, lda, FAKE, FAKE, ldb,
                             bgs, c, c_dt, ldc, cgs, acc, None)


def test_gemm_argument_errors(L):
    assert _g(L, mode=5) == EINVAL
    assert _g(L, G=0) == EINVAL
    assert _g(L, G=129, sizes=[0] * 129) == EUNSUPPORTED
    assert _g(L, a=None) == EINVAL
    assert _g(L, c_dt=4) == EINVAL
    assert _g(L, acc=1, c_dt=0) == EUNSUPPORTED                 # bf16 accumulate
    assert _g(L, K=48) == ESHAPE
    assert _g(L, N=48, ldc=48) == ESHAPE
    assert _g(L, lda=32) == ESHAPE                              # lda < K
    assert _g(L, ldc=32) == ESHAPE
    assert _g(L, sizes=(32, 16)) == ESHAPE                      # sum != M
    assert _g(L, bgs=48) == ESHAPE
    assert _g(L, mode=1, sizes=(40, 20), K=64) == ESHAPE        # sum of padded sizes is 96
    assert _g(L, a=ctypes.c_void_p(0x100004)) == EALIGN


def _dims(E=2, R=64, H=128, F=128):
    return mx._Dims(E, R, H, F)


def test_mlp_sizes_and_errors(L):
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    d = _dims()
    assert L.grouped_mlp_sizes(ctypes.byref(d), mx._i64_array([40, 24]), ctypes.byref(f),
                               ctypes.byref(s), ctypes.byref(b)) == OK
    assert f.value > 0 and s.value > 0 and b.value > 0
    # sizes grow with R and cover at least the dominant buffers
    R, H, F, E = 64, 128, 128, 2
    assert f.value >= E * 2 * F * H + E * H * F + R * H + R * F
    assert s.value >= R * 2 * F * 2
    assert L.grouped_mlp_sizes(ctypes.byref(d), mx._i64_array([40, 20]), None, None, None) == ESHAPE
    assert L.grouped_mlp_sizes(ctypes.byref(_dims(H=48)), mx._i64_array([40, 24]), None, None, None) == ESHAPE
    assert L.grouped_mlp_sizes(ctypes.byref(_dims(F=96)), mx._i64_array([40, 24]), None, None, None) == ESHAPE
    assert L.grouped_mlp_sizes(None, mx._i64_array([40, 24]), None, None, None) == EINVAL
    assert L.grouped_mlp_sizes(ctypes.byref(_dims(E=0)), mx._i64_array([64]), None, None, None) == EINVAL
    ws = ctypes.c_void_p(0x100000)
    # workspace too small, then saved too small: rejected before any launch
    assert L.grouped_mlp_fwd(ctypes.byref(d), mx._i64_array([40, 24]), FAKE, None, FAKE, FAKE, FAKE,
                             None, 0, ws, f.value - 1, None) == EWORKSPACE
    assert L.grouped_mlp_fwd(ctypes.byref(d), mx._i64_array([40, 24]), FAKE, None, FAKE, FAKE, FAKE,
                             ws, s.value - 256, ws, f.value, None) == EWORKSPACE
    assert L.grouped_mlp_fwd(ctypes.byref(d), mx._i64_array([40, 24]), None, None, FAKE, FAKE, FAKE,
                             None, 0, ws, f.value, None) == EINVAL
    assert L.grouped_mlp_fwd(ctypes.byref(d), mx._i64_array([40, 24]), FAKE, None, FAKE, FAKE, FAKE,
                             None, 0, ctypes.c_void_p(0x100010), f.value, None) == EALIGN
    assert L.grouped_mlp_bwd(ctypes.byref(d), mx._i64_array([40, 24]), FAKE, None, ws, s.value, FAKE,
                             None, FAKE, FAKE, 1, ws, b.value - 1, None) == EWORKSPACE
    assert L.grouped_mlp_bwd(ctypes.byref(d), mx._i64_array([40, 24]), FAKE, None, None, s.value, FAKE,
                             None, FAKE, FAKE, 1, ws, b.value, None) == EINVAL


def test_weight_cache_sizes_and_errors(L):
    n = ctypes.c_size_t()
    E, H, F = 2, 128, 256
    assert L.grouped_mlp_weight_cache_bytes(ctypes.byref(_dims(E=E, H=H, F=F)), ctypes.byref(n)) == OK
    codes = 2 * (E * 2 * F * H + E * H * F)          # both layouts of W1 and W2
    assert codes * (1 + 1 / 32) <= n.value <= codes * (1 + 1 / 32) + 8 * 256
    assert L.grouped_mlp_weight_cache_bytes(ctypes.byref(_dims(H=96)), ctypes.byref(n)) == ESHAPE
    assert L.grouped_mlp_weight_cache_bytes(None, ctypes.byref(n)) == EINVAL
    assert L.grouped_mlp_weight_cache_bytes(ctypes.byref(_dims()), None) == EINVAL
    d = _dims(E=E, H=H, F=F)
    cb = ctypes.c_size_t()
    L.grouped_mlp_weight_cache_bytes(ctypes.byref(d), ctypes.byref(cb))
    ws = ctypes.c_void_p(0x100000)
    assert L.grouped_mlp_quantize_weights(ctypes.byref(d), FAKE, FAKE, ws, cb.value - 1, None) == EWORKSPACE
    assert L.grouped_mlp_quantize_weights(ctypes.byref(d), None, FAKE, ws, cb.value, None) == EINVAL
    assert L.grouped_mlp_quantize_weights(ctypes.byref(d), FAKE, FAKE, None, cb.value, None) == EINVAL
    assert L.grouped_mlp_quantize_weights(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x100010), cb.value,
                                          None) == EALIGN
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    split = mx._i64_array([40, 24])
    assert L.grouped_mlp_sizes(ctypes.byref(d), split, ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)) == OK
    assert L.grouped_mlp_fwd_cached(ctypes.byref(d), split, FAKE, None, ws, cb.value - 1, FAKE, None, 0, ws,
                                    f.value, None) == EWORKSPACE
    assert L.grouped_mlp_fwd_cached(ctypes.byref(d), split, FAKE, None, None, cb.value, FAKE, None, 0, ws,
                                    f.value, None) == EINVAL
    assert L.grouped_mlp_fwd_cached(ctypes.byref(d), split, FAKE, None, ws, cb.value, FAKE, None, 0, ws,
                                    f.value - 1, None) == EWORKSPACE
    assert L.grouped_mlp_bwd_cached(ctypes.byref(d), split, FAKE, None, ws, cb.value - 1, ws, s.value, FAKE,
                                    None, FAKE, FAKE, 1, ws, b.value, None) == EWORKSPACE
    assert L.grouped_mlp_bwd_cached(ctypes.byref(d), split, FAKE, None, ws, cb.value, None, s.value, FAKE,
                                    None, FAKE, FAKE, 1, ws, b.value, None) == EINVAL


def test_product_has_no_oracle_dependency():
    """The product package never imports the test oracle."""
    pkg = os.path.join(ROOT, "mxfp8_block_scaled_mx_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn


def test_library_defines_every_kernel_stub(L):
    """Every kernel the host code launches has its host stub in the library
    (a host-pass problem in a kernel body silently drops the stub and leaves
    an undefined symbol that only fails at load time on the GPU machine)."""
    import subprocess
    out = subprocess.run(["nm", "-C", "--undefined-only", mx.lib_path()], capture_output=True, text=True).stdout
    assert "device_stub" not in out, [l for l in out.splitlines() if "device_stub" in l][:5]


def test_moe_dispatch_combine_argument_errors(L):
    assert L.mx_moe_dispatch_workspace_bytes(100, 2, 8) == ((200 + 255) // 256 * 8 + 1) * 4
    assert L.mx_moe_dispatch_workspace_bytes(100, 2, 0) == 0
    ws = ctypes.c_void_p(0x100000)

    def d(x=FAKE, idx=FAKE, w=None, T=100, H=64, k=2, E=8, xp=FAKE, pp=None, wsb=1 << 20):
        return L.mx_moe_dispatch(x, idx, w, T, H, k, E, xp, pp, FAKE, FAKE, FAKE, ws, wsb, None)

    assert d(H=60) == ESHAPE
    assert d(k=0) == EINVAL
    assert d(E=129) == EUNSUPPORTED
    assert d(x=None) == EINVAL                       # x without x_perm
    assert d(xp=None) == EINVAL
    assert d(w=FAKE) == EINVAL                       # weights without probs_perm
    assert d(x=ctypes.c_void_p(0x100008)) == EALIGN
    assert d(wsb=16) == EWORKSPACE
    assert L.mx_moe_combine(FAKE, FAKE, 10, 60, 2, FAKE, None) == ESHAPE
    assert L.mx_moe_combine(None, FAKE, 10, 64, 2, FAKE, None) == EINVAL
    assert L.mx_moe_combine(FAKE, FAKE, 10, 64, 2, ctypes.c_void_p(0x100004), None) == EALIGN


def test_quantize_fp4_argument_errors(L):
    assert L.mx_quantize_fp4(FAKE, 4, 48, FAKE, FAKE, None, None, None) == ESHAPE
    assert L.mx_quantize_fp4(FAKE, -1, 64, FAKE, FAKE, None, None, None) == ESHAPE
    assert L.mx_quantize_fp4(FAKE, 40, 64, None, None, FAKE, FAKE, None) == ESHAPE   # rows % 32
    assert L.mx_quantize_fp4(None, 4, 64, FAKE, FAKE, None, None, None) == EINVAL
    assert L.mx_quantize_fp4(FAKE, 4, 64, None, None, None, None, None) == EINVAL   # nothing requested
    assert L.mx_quantize_fp4(FAKE, 4, 64, FAKE, None, None, None, None) == EINVAL   # half a pair
    assert L.mx_quantize_fp4(FAKE, 4, 64, ctypes.c_void_p(0x100008), FAKE, None, None, None) == EALIGN


def test_gemm_fp4_errors(L):
    g = L.mx_gemm_fp4
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 96, FAKE, 0, None) == ESHAPE      # k % 64
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 0, FAKE, 0, None) == ESHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, -1, 4, 64, FAKE, 0, None) == ESHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 2, None) == EINVAL      # dtype
    assert g(None, FAKE, FAKE, FAKE, 4, 4, 64, FAKE, 0, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, None, 4, 4, 64, FAKE, 1, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 64, ctypes.c_void_p(0x100008), 0, None) == EALIGN
    assert g(FAKE, FAKE, FAKE, FAKE, 4, 4, 1 << 27, FAKE, 0, None) == EUNSUPPORTED
    assert g(None, None, None, None, 0, 4, 64, None, 0, None) == OK             # empty: no-op


def test_grouped_gemm_fp4_errors(L):
    g = L.mx_grouped_gemm_fp4
    sz = (ctypes.c_int64 * 3)(4, 0, 8)
    neg = (ctypes.c_int64 * 2)(4, -1)
    assert g(FAKE, FAKE, FAKE, FAKE, sz, 0, 4, 64, FAKE, 0, None) == EINVAL      # no groups
    assert g(FAKE, FAKE, FAKE, FAKE, sz, 129, 4, 64, FAKE, 0, None) == EINVAL    # > MX_MAX_GROUPS
    assert g(FAKE, FAKE, FAKE, FAKE, None, 3, 4, 64, FAKE, 0, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, neg, 2, 4, 64, FAKE, 0, None) == ESHAPE
    assert g(FAKE, FAKE, FAKE, FAKE, sz, 3, 4, 32, FAKE, 0, None) == ESHAPE     # k % 64
    assert g(FAKE, FAKE, None, FAKE, sz, 3, 4, 64, FAKE, 0, None) == EINVAL
    assert g(FAKE, FAKE, FAKE, FAKE, sz, 3, 4, 64, ctypes.c_void_p(0x100008), 1, None) == EALIGN
    zero = (ctypes.c_int64 * 2)(0, 0)
    assert g(None, None, None, None, zero, 2, 4, 64, None, 0, None) == OK        # no rows: no-op


def test_fp4_gemm_wrappers_reject_mismatched_shapes():
    # the C ABI takes plain pointers; the binding checks the operand shapes
    # before any call, so a narrower B can never be read past its end
    import torch
    u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
    with pytest.raises(ValueError):
        mx.mx_gemm_fp4(u8(4, 32), u8(4, 2), u8(8, 16), u8(8, 1))          # B narrower than A
    with pytest.raises(ValueError):
        mx.mx_gemm_fp4(u8(4, 32), u8(4, 1), u8(8, 32), u8(8, 2))          # A scales too short
    with pytest.raises(ValueError):
        mx.mx_gemm_fp4(u8(4, 32), u8(4, 2), u8(8, 32), u8(8, 2), out=torch.zeros(4, 7))
    with pytest.raises(ValueError):
        mx.mx_grouped_gemm_fp4(u8(5, 32), u8(5, 2), u8(2, 8, 32), u8(2, 8, 2), [2, 2])   # sizes != rows
    with pytest.raises(ValueError):
        mx.mx_grouped_gemm_fp4(u8(4, 32), u8(4, 2), u8(3, 8, 32), u8(3, 8, 2), [2, 2])   # groups != weights


def test_cast_wrappers_reject_bad_inputs():
    # a float32, strided, 1-D or host x would be read as packed bf16 from its
    # data pointer; the bindings refuse it before any device call
    import torch
    bad = [torch.zeros(4, 64, dtype=torch.float32),                 # fp32 (FP4 cast takes bf16 only)
           torch.zeros(64, 8, dtype=torch.bfloat16).t(),            # strided
           torch.zeros(256, dtype=torch.bfloat16),                  # 1-D
           torch.zeros(4, 64, dtype=torch.bfloat16)]                # host memory
    for x in bad:
        with pytest.raises(ValueError):
            mx.mx_quantize_fp4(x)
    for x in bad[1:] + [torch.zeros(4, 64, dtype=torch.float16)]:
        with pytest.raises(ValueError):
            mx.quantize(x)


def test_mlp_intermediates_offsets(L):
    # the intermediates lie inside the buffers grouped_mlp_sizes sizes, in
    # disjoint regions large enough for their layouts
    E, R, H, F = 3, 100, 256, 384
    split = [37, 0, 63]
    fws, sv, bws = mx.mlp_sizes(E, R, H, F, split)
    o = mx.mlp_intermediates(E, R, H, F, split)
    P = sum((m + 31) // 32 * 32 for m in split)
    nq = sum(-(-((m + 31) // 32 * 32) // 128) for m in split)
    assert o["nq_col"] == nq
    R32 = -(-R // 32) * 32
    regions = {
        "fwd": [(o["a_row_codes"], R * F), (o["a_row_scales"], R32 * F // 32)],
        "saved": [(o["h1"], R * 2 * F * 2), (o["a_col_codes"], F * P), (o["a_col_scales"], F // 32 * nq * 128)],
        "bwd": [(o["dh1_row_codes"], R * 2 * F), (o["dh1_row_scales"], R32 * 2 * F // 32),
                (o["dh1_col_codes"], 2 * F * P), (o["dh1_col_scales"], 2 * F // 32 * nq * 128)],
    }
    for key, total in (("fwd", fws), ("saved", sv), ("bwd", bws)):
        spans = sorted(regions[key])
        for (a, n), (b, _) in zip(spans, spans[1:]):
            assert a + n <= b, key
        assert all(a % 256 == 0 and a + n <= total for a, n in spans), key
    with pytest.raises(mx.MXError):
        mx.mlp_intermediates(E, R, H, F, [37, 0, 62])           # split does not sum to R
    assert L.grouped_mlp_intermediates(ctypes.byref(_dims()), mx._i64_array([40, 24]), None) == EINVAL


def test_moe_dispatch_noalloc_limits(L):
    # validated before the scratch array is touched: sizes past its 65536
    # words, and the usual argument errors
    def d(T=100, H=64, k=2, E=8, x=FAKE, xp=FAKE):
        return L.mx_moe_dispatch_noalloc(x, FAKE, None, T, H, k, E, xp, None, FAKE, FAKE, FAKE, None)

    assert d(T=65536, E=128) == EUNSUPPORTED          # ceil(131072 / 256) * 128 + 1 words
    assert d(H=60) == ESHAPE
    assert d(E=129) == EUNSUPPORTED
    assert d(x=None) == EINVAL
    assert d(x=ctypes.c_void_p(0x100008)) == EALIGN


def test_device_split_sizes_cover_every_split(L):
    # the device-split layout holds the largest padded total any split of R
    # rows can reach, so it is at least the host-split size of each split
    E, R, H, F = 4, 100, 128, 128
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    assert L.grouped_mlp_sizes_device_split(ctypes.byref(_dims(E, R, H, F)), ctypes.byref(f), ctypes.byref(s),
                                            ctypes.byref(b)) == OK
    for split in ([100, 0, 0, 0], [25, 25, 25, 25], [1, 1, 1, 97], [33, 33, 33, 1], [0, 0, 0, 100]):
        hf, hs, hb = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
        assert L.grouped_mlp_sizes(ctypes.byref(_dims(E, R, H, F)), mx._i64_array(split), ctypes.byref(hf),
                                   ctypes.byref(hs), ctypes.byref(hb)) == OK
        # (less the host call's split-K partials, which the device-split call does not use)
        split_k = min(sum(-(-m // 256) for m in split) * -(-H // 256), 128) * 4 * 256 * 256 * 4
        assert hs.value <= s.value, split
        assert hf.value - split_k <= f.value and hb.value - split_k <= b.value, split
    assert L.grouped_mlp_sizes_device_split(ctypes.byref(_dims(E, R, 96, F)), None, None, None) == ESHAPE
    assert L.grouped_mlp_sizes_device_split(None, None, None, None) == EINVAL


def test_device_split_argument_errors(L):
    E, R, H, F = 2, 64, 128, 128
    d = _dims(E, R, H, F)
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    L.grouped_mlp_sizes_device_split(ctypes.byref(d), ctypes.byref(f), ctypes.byref(s), ctypes.byref(b))
    ws = ctypes.c_void_p(0x100000)

    def fwd(split=FAKE, w1=FAKE, cache=None, fb=f.value, rt=None, tokens=0):
        return L.grouped_mlp_fwd_device_split(ctypes.byref(d), split, FAKE, tokens, rt, None, w1, FAKE, cache, 0,
                                              FAKE, None, 0, ws, fb, None)

    assert fwd(split=None) == EINVAL
    assert fwd(split=ctypes.c_void_p(0x100004)) == EALIGN
    assert fwd(fb=f.value - 1) == EWORKSPACE
    assert fwd(w1=None) == EINVAL                                   # no weights and no cache
    assert fwd(cache=ws) == EWORKSPACE                              # cache of 0 bytes
    assert fwd(rt=FAKE, tokens=-1) == ESHAPE
    assert L.grouped_mlp_bwd_device_split(ctypes.byref(d), None, FAKE, 0, None, None, None, 0, ws, s.value, FAKE,
                                          None, FAKE, FAKE, 0, ws, b.value, None) == EINVAL
    assert L.grouped_mlp_bwd_device_split(ctypes.byref(d), FAKE, FAKE, 0, None, None, None, 0, ws, s.value - 1,
                                          FAKE, None, FAKE, FAKE, 0, ws, b.value, None) == EWORKSPACE


def test_fp4_wgrad_and_grouped_cast_argument_errors(L):
    sizes = mx._i64_array([20, 44])
    def cast(rows=64, cols=64, sz=sizes, g=2, x=FAKE, q=FAKE):
        return L.mx_quantize_fp4_colwise_grouped(x, rows, cols, sz, g, q, FAKE, None)
    assert cast(cols=48) == ESHAPE
    assert cast(rows=63) == ESHAPE                       # sizes do not sum to rows
    assert cast(g=0) == EINVAL
    assert cast(q=None) == EINVAL
    assert cast(x=ctypes.c_void_p(0x100008)) == EALIGN
    def wg(g=2, m=64, n=64, sz=sizes, c=FAKE, a=FAKE):
        return L.mx_grouped_gemm_fp4_wgrad(a, FAKE, FAKE, FAKE, sz, g, m, n, c, 0, None)
    assert wg(g=0) == EINVAL
    assert wg(g=129, sz=mx._i64_array([1] * 129)) == EINVAL
    assert wg(m=-1) == ESHAPE
    assert wg(sz=mx._i64_array([20, -4])) == ESHAPE
    assert wg(c=None) == EINVAL
    assert wg(a=ctypes.c_void_p(0x100008)) == EALIGN
    assert wg(m=0) == OK                                 # nothing to compute, nothing enqueued


def test_device_copy_argument_errors(L):
    # checked before any launch; a zero-byte copy enqueues nothing
    assert L.mx_device_copy(FAKE, FAKE, 24, None) == ESHAPE
    assert L.mx_device_copy(FAKE, FAKE, -16, None) == ESHAPE
    assert L.mx_device_copy(None, FAKE, 16, None) == EINVAL
    assert L.mx_device_copy(ctypes.c_void_p(0x100008), FAKE, 16, None) == EALIGN
    assert L.mx_device_copy(None, None, 0, None) == 0


def test_mlp_bindings_reject_tensors_that_disagree_with_the_dims():
    # the C ABI trusts the sizes it is given, so a smaller tensor would be read
    # past its end; the bindings compare every tensor with the dims first
    # (shapes and dtypes before the device, so these checks run on the CPU)
    import torch
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    E, R, H, F = 2, 64, 256, 64
    x, w1, w2 = bf(R, H), bf(E, 2 * F, H), bf(E, H, F)
    with pytest.raises(ValueError, match="w1"):
        mx.grouped_mlp_fwd(x, None, bf(E, H, 2 * F), w2, [32, 32])          # W1 given as [E, H, 2F]
    with pytest.raises(ValueError, match="w2"):
        mx.grouped_mlp_fwd(x, None, w1, bf(E, F, H), [32, 32])
    with pytest.raises(ValueError, match="split_sizes"):
        mx.grouped_mlp_fwd(x, None, w1, w2, [32, 31])
    with pytest.raises(ValueError, match="probs"):
        mx.grouped_mlp_fwd(x, torch.zeros(R + 1), w1, w2, [32, 32])
    with pytest.raises(ValueError, match="CUDA"):
        mx.grouped_mlp_fwd(x, None, w1, w2, [32, 32])                      # consistent, but host memory
    with pytest.raises(ValueError, match="dy"):
        mx.grouped_mlp_bwd(bf(R, H + 32), None, mx.MLPState(None, (E, R, H, F), [32, 32]))
    with pytest.raises(ValueError, match="topk_idx"):
        mx.mx_moe_dispatch(x, torch.zeros((R, 2), dtype=torch.int64), None, E)
    with pytest.raises(ValueError, match="a_q"):
        u8 = lambda *s: torch.zeros(s, dtype=torch.uint8)
        mx.grouped_gemm(mx.MX_GROUP_M, [64], u8(64, 128), u8(64, 4), u8(32, 128), u8(32, 4), N=32, K=128,
                        out=torch.zeros((64, 32)))


def test_fp4_mlp_sizes_and_argument_errors(L):
    E, R, H, F = 3, 300, 256, 384
    split = mx._i64_array([100, 0, 200])
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    d = _dims(E, R, H, F)
    assert L.grouped_mlp_fp4_sizes(ctypes.byref(d), split, ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)) == OK
    P = 128 + 0 + 224                                   # per-expert rows padded to 32
    # the forward holds at least H1 in fp32 and the 4-bit rowwise copies of A
    # and W1; the saved buffer at least H1 in bf16 and the 4-bit columnwise
    # copies of A, X, W1 and W2; the backward at least dA in fp32, dH1's two
    # 4-bit copies and the per-tile dprobs partials (A and dH1 are cast as they
    # are formed, with no fp32 copy)
    assert f.value >= R * 2 * F * 4 + R * F // 2 + E * 2 * F * H // 2
    assert s.value >= R * 2 * F * 2 + (F + H) * P // 2 + E * 3 * F * H // 2
    assert b.value >= R * F * 4 + R * 2 * F // 2 + 2 * F * P // 2 + F // 64 * R * 4
    assert L.grouped_mlp_fp4_sizes(ctypes.byref(_dims(E, R, 96, F)), split, None, None, None) == ESHAPE
    assert L.grouped_mlp_fp4_sizes(ctypes.byref(d), mx._i64_array([100, 0, 199]), None, None, None) == ESHAPE
    assert L.grouped_mlp_fp4_sizes(None, split, None, None, None) == EINVAL
    ws = f.value

    def fwd(x=FAKE, w=FAKE, y=FAKE, wsb=ws, saved=None, sb=0):
        return L.grouped_mlp_fwd_fp4(ctypes.byref(d), split, x, None, w, FAKE, y, saved, sb, FAKE, wsb, None)
    assert fwd(x=None) == EINVAL
    assert fwd(w=None) == EINVAL
    assert fwd(y=ctypes.c_void_p(0x100008)) == EALIGN
    assert fwd(wsb=ws - 1) == EWORKSPACE
    assert fwd(saved=FAKE, sb=s.value - 1) == EWORKSPACE

    def bwd(saved=FAKE, sb=s.value, wsb=b.value, dw1=FAKE):
        return L.grouped_mlp_bwd_fp4(ctypes.byref(d), split, FAKE, None, saved, sb, FAKE, None, dw1, FAKE, 0,
                                     FAKE, wsb, None)
    assert bwd(saved=None) == EINVAL
    assert bwd(dw1=None) == EINVAL
    assert bwd(sb=s.value - 1) == EWORKSPACE
    assert bwd(wsb=b.value - 1) == EWORKSPACE


def test_fp4_mlp_bindings_check_state_and_shapes():
    import torch
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    E, R, H, F = 2, 64, 256, 64
    with pytest.raises(ValueError, match="w1"):
        mx.grouped_mlp_fwd_fp4(bf(R, H), None, bf(E, H, 2 * F), bf(E, H, F), [32, 32])
    with pytest.raises(ValueError, match="MXFP4 forward"):
        mx.grouped_mlp_bwd_fp4(bf(R, H), None, mx.MLPState(None, (E, R, H, F), [32, 32]))     # an MXFP8 state
    with pytest.raises(ValueError, match="MXFP8"):
        mx.grouped_mlp_bwd(bf(R, H), None, mx.MLPState(None, (E, R, H, F), [32, 32], fmt="mxfp4"))


def _fake_cache(fmt, E=2, H=256, F=64):
    """A WeightCache object without a device buffer (the bindings' checks
    below run before any device call)."""
    c = mx.WeightCache.__new__(mx.WeightCache)
    c.ehf, c.fmt, c.buf = (E, H, F), fmt, None
    return c


def test_cached_states_pair_with_their_cache():
    """A state from a cached forward holds no weight copies: the uncached
    backward refuses it, and a cached backward takes only the cache (and
    format) that made it."""
    import torch
    bf = lambda *s: torch.zeros(s, dtype=torch.bfloat16)
    E, R, H, F = 2, 64, 256, 64
    c8, c4 = _fake_cache("mxfp8"), _fake_cache("mxfp4")
    st8 = mx.MLPState(None, (E, R, H, F), [32, 32], cache=c8)
    st4 = mx.MLPState(None, (E, R, H, F), [32, 32], fmt="mxfp4", cache=c4)
    with pytest.raises(ValueError, match="cached forward"):
        mx.grouped_mlp_bwd(bf(R, H), None, st8)
    with pytest.raises(ValueError, match="cached forward"):
        mx.grouped_mlp_bwd_fp4(bf(R, H), None, st4)
    with pytest.raises(ValueError, match="this weight cache"):
        mx.grouped_mlp_bwd_cached(bf(R, H), None, st8, _fake_cache("mxfp8"))
    with pytest.raises(ValueError, match="this weight cache"):
        mx.grouped_mlp_bwd_fp4_cached(bf(R, H), None, st4, _fake_cache("mxfp4"))
    with pytest.raises(ValueError, match="MXFP4 weight cache"):
        mx.grouped_mlp_bwd_fp4_cached(bf(R, H), None, st4, c8)
    with pytest.raises(ValueError, match="MXFP8 weight cache"):
        mx.grouped_mlp_bwd_cached(bf(R, H), None, st8, c4)
    with pytest.raises(ValueError, match="MXFP4 forward"):
        mx.grouped_mlp_bwd_fp4_cached(bf(R, H), None, mx.MLPState(None, (E, R, H, F), [32, 32], cache=c4), c4)
    with pytest.raises(ValueError, match="mxfp8"):
        mx.grouped_mlp_fwd_fp4_cached(bf(R, H), None, c8, [32, 32])
    with pytest.raises(ValueError, match="mxfp4"):
        mx.grouped_mlp_fwd_cached(bf(R, H), None, c4, [32, 32])
    with pytest.raises(ValueError, match="unknown format"):
        mx.WeightCache(E, H, F, fmt="nvfp4")


def test_fp4_weight_cache_sizes_and_errors(L):
    E, H, F = 2, 256, 128
    n = ctypes.c_size_t()
    d = _dims(E=E, H=H, F=F)
    assert L.grouped_mlp_fp4_weight_cache_bytes(ctypes.byref(d), ctypes.byref(n)) == OK
    codes = (E * 2 * F * H + E * H * F)               # both layouts of W1 and W2, two codes per byte
    assert codes * (1 + 1 / 16) <= n.value <= codes * (1 + 1 / 16) + 8 * 256
    assert L.grouped_mlp_fp4_weight_cache_bytes(ctypes.byref(_dims(H=96)), ctypes.byref(n)) == ESHAPE
    assert L.grouped_mlp_fp4_weight_cache_bytes(None, ctypes.byref(n)) == EINVAL
    assert L.grouped_mlp_fp4_weight_cache_bytes(ctypes.byref(d), None) == EINVAL
    cb = ctypes.c_size_t()
    L.grouped_mlp_fp4_weight_cache_bytes(ctypes.byref(d), ctypes.byref(cb))
    ws = ctypes.c_void_p(0x100000)
    assert L.grouped_mlp_fp4_quantize_weights(ctypes.byref(d), FAKE, FAKE, ws, cb.value - 1, None) == EWORKSPACE
    assert L.grouped_mlp_fp4_quantize_weights(ctypes.byref(d), None, FAKE, ws, cb.value, None) == EINVAL
    assert L.grouped_mlp_fp4_quantize_weights(ctypes.byref(d), FAKE, FAKE, None, cb.value, None) == EINVAL
    assert L.grouped_mlp_fp4_quantize_weights(ctypes.byref(d), FAKE, FAKE, ctypes.c_void_p(0x100010), cb.value,
                                              None) == EALIGN
    assert L.grouped_mlp_fp4_quantize_weights(None, FAKE, FAKE, ws, cb.value, None) == EINVAL
    f, s, b = ctypes.c_size_t(), ctypes.c_size_t(), ctypes.c_size_t()
    split = mx._i64_array([40, 24])
    d = _dims(E=E, R=64, H=H, F=F)
    assert L.grouped_mlp_fp4_sizes(ctypes.byref(d), split, ctypes.byref(f), ctypes.byref(s), ctypes.byref(b)) == OK
    fwd = lambda cache=ws, cbytes=cb.value, wsb=f.value, x=FAKE: L.grouped_mlp_fwd_fp4_cached(
        ctypes.byref(d), split, x, None, cache, cbytes, FAKE, None, 0, ws, wsb, None)
    assert fwd(cbytes=cb.value - 1) == EWORKSPACE
    assert fwd(cache=None) == EINVAL
    assert fwd(cache=ctypes.c_void_p(0x100010)) == EALIGN
    assert fwd(wsb=f.value - 1) == EWORKSPACE
    assert fwd(x=None) == EINVAL
    bwd = lambda cache=ws, cbytes=cb.value, saved=ws, sb=s.value, wsb=b.value: L.grouped_mlp_bwd_fp4_cached(
        ctypes.byref(d), split, FAKE, None, cache, cbytes, saved, sb, FAKE, None, FAKE, FAKE, 1, ws, wsb, None)
    assert bwd(cbytes=cb.value - 1) == EWORKSPACE
    assert bwd(cache=None) == EINVAL
    assert bwd(saved=None) == EINVAL
    assert bwd(sb=s.value - 1) == EWORKSPACE
    assert bwd(wsb=b.value - 1) == EWORKSPACE


def test_nvfp4_argument_errors(L):
    amax = FAKE
    def cast(rows=32, cols=64, q=FAKE, qc=None, am=amax, x=FAKE):
        return L.mx_quantize_nvfp4(x, rows, cols, q, FAKE if q is not None else None, qc,
                                   FAKE if qc is not None else None, am, None)
    assert cast(cols=40) == ESHAPE
    assert cast(rows=24, qc=FAKE) == ESHAPE                # columnwise copy needs rows % 16 == 0
    assert cast(q=None) == EINVAL                           # no output
    assert cast(am=None) == EINVAL
    assert cast(x=ctypes.c_void_p(0x100008)) == EALIGN
    assert cast(am=ctypes.c_void_p(0x100002)) == EALIGN
    def gemm(k=256, am=amax, bs=FAKE, n=64):
        return L.mx_gemm_nvfp4(FAKE, FAKE, am, FAKE, bs, amax, 64, n, k, FAKE, 0, None)
    assert gemm(k=192) == ESHAPE                            # k must be a multiple of 128
    assert gemm(am=None) == EINVAL
    assert gemm(bs=ctypes.c_void_p(0x100004)) == EALIGN    # scales 8-byte aligned
    assert gemm(n=0) == OK                                  # nothing to compute
    assert L.mx_grouped_gemm_nvfp4(FAKE, FAKE, amax, FAKE, FAKE, amax, mx._i64_array([1]), 0, 64, 256, FAKE, 0,
                                   None) == EINVAL


def test_fp4_mlp_rejects_grids_past_32_bits(L):
    # 2^24 rows of one expert and F = 2^20: every dimension and the padded row
    # count are in range, but the columnwise cast of the [R, 2F] gradient takes
    # 2^17 row tiles x 2^15 column tiles = 2^32 workgroups
    E, R, H, F = 1, 1 << 24, 4096, 1 << 20
    split = mx._i64_array([R // E] * E)
    assert L.grouped_mlp_fp4_sizes(ctypes.byref(_dims(E, R, H, F)), split, None, None, None) == EUNSUPPORTED

"""The allocation-free token dispatch (mx_moe_dispatch_noalloc), called
through the C ABI, against mx_moe_dispatch with a caller workspace on the same
inputs: bit-identical routed rows, routing weights, permutation, row tokens
and counts, on two calls in a row, the second with fewer tokens (the shared
scratch array keeps the first call's contents). Token routing as in
"Efficient MoE training for biological foundation models" (Dense vs. MoE
scaling; Key technical approaches item 1: per-expert groups with counts)."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as wl
from tests.gpu_util import dev_bf16

pytestmark = pytest.mark.gpu


def _outputs(T, H, k, E, dev):
    return dict(x_perm=torch.full((T * k, H), 7.0, dtype=torch.bfloat16, device=dev),
                probs=torch.full((T * k,), -1.0, dtype=torch.float32, device=dev),
                perm=torch.full((T, k), -7, dtype=torch.int32, device=dev),
                row_token=torch.full((T * k,), -7, dtype=torch.int32, device=dev),
                counts=torch.full((E,), -7, dtype=torch.int64, device=dev))


def _dispatch(mx, noalloc, x, idx, w, E, out):
    L = mx.load()
    T, H = x.shape
    k = idx.shape[1]
    p = mx._ptr
    args = (p(x), p(idx), p(w), T, H, k, E, p(out["x_perm"]), p(out["probs"]), p(out["perm"]),
            p(out["row_token"]), p(out["counts"]))
    if noalloc:
        st = L.mx_moe_dispatch_noalloc(*args, mx._stream())
    else:
        ws = mx._byte_buffer(L.mx_moe_dispatch_workspace_bytes(T, k, E), x.device)
        st = L.mx_moe_dispatch(*args, p(ws), ws.numel(), mx._stream())
    mx._check(st)


@pytest.mark.parametrize("shapes", [((8192, 4096, 8), (1000, 512, 8)), ((3000, 256, 128), (257, 256, 5))])
def test_noalloc_dispatch_matches_workspace_dispatch(gpu_lib, shapes):
    dev = torch.device("cuda")
    for i, (T, H, E) in enumerate(shapes):
        print(f"[no_alloc] call {i}: tokens={T} hidden={H} experts={E}", flush=True)
        c = wl.make_dispatch_inputs(T, E, H, seed=90 + i)
        idx = c["topk_idx"].copy()
        idx[::97, 1] = E            # dropped entries (expert out of range)
        x = dev_bf16(c["x"])
        idx_d = torch.from_numpy(idx).to(dev)
        w = torch.from_numpy(c["topk_w"]).to(dev)
        ref = _outputs(T, H, 2, E, dev)
        got = _outputs(T, H, 2, E, dev)
        _dispatch(gpu_lib, False, x, idx_d, w, E, ref)
        _dispatch(gpu_lib, True, x, idx_d, w, E, got)
        torch.cuda.synchronize()
        n = int(ref["counts"].sum())
        assert n == int((idx < E).sum())
        for key in ("probs", "perm", "row_token", "counts"):
            assert torch.equal(got[key], ref[key]), key
        assert torch.equal(got["x_perm"][:n].view(torch.int16), ref["x_perm"][:n].view(torch.int16))


def test_noalloc_dispatch_rejects_requests_above_its_scratch(gpu_lib):
    L = gpu_lib.load()
    fake = ctypes.c_void_p(0x100000)
    # ceil(65536 * 2 / 256) * 128 + 1 > 65536 words: refused before any launch
    st = L.mx_moe_dispatch_noalloc(fake, fake, None, 65536, 64, 2, 128, fake, None, fake, fake, fake, None)
    assert st == 6                                        # MX_EUNSUPPORTED

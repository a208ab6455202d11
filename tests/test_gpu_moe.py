"""GPU parity of token dispatch and combine (mx_moe_dispatch, mx_moe_combine)
against the oracle (readings R12, R13): bit-exact routed rows, permutation,
token of each row, routing weight of each row and per-expert counts; the
combine bit-exact for top-2 (the fp32 sum of two bf16 values rounds to the
same bf16 as the float64 sum) and for integer-valued rows at top-3."""
import numpy as np
import pytest
import torch

import oracle as orc
import workloads as wl
from tests.gpu_util import to_np

pytestmark = pytest.mark.gpu


def _dev_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _check_dispatch(mx, x_bits, idx, w, E):
    want = orc.moe_dispatch(x_bits, idx, w, E)
    x_perm, probs, perm, row_token, counts = mx.mx_moe_dispatch(
        _dev_bits(x_bits), torch.from_numpy(idx).cuda(),
        None if w is None else torch.from_numpy(w).cuda(), E)
    torch.cuda.synchronize()
    R = int(want["counts"].sum())
    assert np.array_equal(counts.cpu().numpy(), want["counts"])
    assert np.array_equal(perm.cpu().numpy(), want["perm"])
    assert np.array_equal(row_token.cpu().numpy()[:R], want["row_token"])
    assert np.array_equal(_bits(x_perm)[:R], want["x_perm"])
    if w is not None:
        assert np.array_equal(probs.cpu().numpy()[:R], want["probs_perm"])
    # routing only (no row copy): the same routing outputs
    none, probs2, perm2, row_token2, counts2 = mx.mx_moe_dispatch(
        _dev_bits(x_bits), torch.from_numpy(idx).cuda(),
        None if w is None else torch.from_numpy(w).cuda(), E, gather=False)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(perm2, perm) and torch.equal(counts2, counts)
    assert torch.equal(row_token2[:R], row_token[:R])
    if w is not None:
        assert torch.equal(probs2[:R], probs[:R])
    return perm, want


@pytest.mark.parametrize("T,k,E,H", [(300, 2, 8, 64), (1000, 1, 3, 32), (257, 3, 128, 8), (0, 2, 4, 64)])
def test_dispatch_and_combine_small(gpu_lib, T, k, E, H):
    rng = np.random.default_rng(50 + T + k)
    x = wl.normal_bf16(rng, (T, H), 1.0)
    idx = np.array([rng.permutation(E)[:k] for _ in range(T)], dtype=np.int32).reshape(T, k)
    if T > 10:
        idx[3, 0] = -1                                  # dropped entries
        idx[7, k - 1] = E
    w = rng.uniform(0, 1, size=(T, k)).astype(np.float32)
    perm, want = _check_dispatch(gpu_lib, x, idx, w, E)
    R = int(want["counts"].sum())
    if k == 3:      # integer-valued rows: every fp32 partial sum is exact
        y_perm = wl.bf16_bits_from_f32(rng.integers(-64, 64, size=(max(R, 1), H)).astype(np.float32))
    else:
        y_perm = wl.normal_bf16(rng, (max(R, 1), H), 1.0)
    y = gpu_lib.mx_moe_combine(_dev_bits(y_perm), perm)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y), orc.moe_combine(y_perm, want["perm"]))


def test_dispatch_and_combine_full_size(gpu_lib):
    """8192 tokens, top-2 of 8 experts with skewed loads, hidden 4096 (the
    Mixtral-shaped forward workload's routing shape)."""
    c = wl.make_dispatch_inputs(8192, 8, 4096, seed=60)
    perm, want = _check_dispatch(gpu_lib, c["x"], c["topk_idx"], c["topk_w"], 8)
    y = gpu_lib.mx_moe_combine(_dev_bits(c["y_perm"]), perm)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(y), orc.moe_combine(c["y_perm"], want["perm"]))


@pytest.mark.parametrize("T,E,H,F", [(300, 4, 256, 384), (2048, 8, 512, 256)])
def test_mlp_forward_with_fused_gather_equals_dispatch_then_forward(gpu_lib, T, E, H, F):
    """grouped_mlp_fwd_gather (the X cast reads token rows through row_token)
    is bit-identical to mx_moe_dispatch followed by grouped_mlp_fwd on the
    routed copy, forward and backward (saved state), with one expert empty
    and a few dropped entries; and the combine of the forward output matches
    the oracle's combine of the same routed output."""
    mx = gpu_lib
    rng = np.random.default_rng(70 + T)
    x = wl.normal_bf16(rng, (T, H), 1.0)
    logits = rng.standard_normal((T, E))
    logits[:, 1] = -50.0                                   # expert 1 gets no tokens
    idx, w = wl.top2_picks(logits, np.zeros(E))
    idx[5, 1] = -1
    w1 = wl.normal_bf16(rng, (E, 2 * F, H), 0.02)
    w2 = wl.normal_bf16(rng, (E, H, F), 0.02)
    xt, w1t, w2t = _dev_bits(x), _dev_bits(w1), _dev_bits(w2)
    x_perm, probs, perm, row_token, counts = mx.mx_moe_dispatch(xt, torch.from_numpy(idx).cuda(),
                                                                torch.from_numpy(w).cuda(), E)
    split = counts.cpu().tolist()
    R = sum(split)
    assert split[1] == 0 and R == 2 * T - 1
    y_ref, st_ref = mx.grouped_mlp_fwd(x_perm[:R].contiguous(), probs[:R].contiguous(), w1t, w2t, split)
    y, st = mx.grouped_mlp_fwd_gather(xt, row_token[:R].contiguous(), probs[:R].contiguous(), w1t, w2t, split)
    dy = _dev_bits(wl.normal_bf16(rng, (R, H), 1e-3))
    ref = mx.grouped_mlp_bwd(dy, probs[:R].contiguous(), st_ref)
    got = mx.grouped_mlp_bwd(dy, probs[:R].contiguous(), st)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)
    out = mx.mx_moe_combine(y, perm)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(out), orc.moe_combine(_bits(y), perm.cpu().numpy()))
    # backward with dY gathered from the tokens' output gradient by the dY cast
    # (the gradient of the combine) equals the backward on the gathered copy
    dy_tok = _dev_bits(wl.normal_bf16(rng, (T, H), 1e-3))
    dy_perm = dy_tok[row_token[:R].long()].contiguous()
    ref = mx.grouped_mlp_bwd(dy_perm, probs[:R].contiguous(), st)
    got = mx.grouped_mlp_bwd_gather(dy_tok, row_token[:R].contiguous(), probs[:R].contiguous(), st)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b)

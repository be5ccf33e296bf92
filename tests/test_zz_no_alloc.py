"""The allocation-free factor (gptq_factor_noalloc, through the C ABI) against gptq_factor.

Collected last on purpose (a failure here must not hide the other GPU tests).

Two calls in a row on the library's static scratch, the second with a smaller matrix, so the second
runs on whatever the first left in the shared array. Each must give, bit for bit, the U and perm of
gptq_factor with a workspace of its own (the same kernels, on one stream instead of two), and meet
the factor's parity bar against the float64 oracle (float32 LAPACK's error on the same matrix).
"""

import numpy as np
import pytest

import synth
from gpu_util import FACTOR_VS_LAPACK, factor_errors, lapack_f32_factor, torch_cuda
from oracle import gptq_ref as ref

pytestmark = pytest.mark.gpu


def _hessian(d, seed, act):
    case = synth.make_case(name="na", seed=seed, rows=16, d=d, n=3 * d + 64, w_std=0.02, w_dtype="f16",
                           x_dist="laplace", x_dtype="f32", outlier_frac=0.01, outlier_scale=20.0, chunk=8192,
                           bits=4, group_size=128, block_size=128, act_order=act)
    H64, n = ref.hessian([synth.to_f64(synth.x_chunk(case, 0), "f32")])
    return H64.astype(np.float32), n


def test_factor_noalloc_matches_factor_on_two_calls():
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    # the second call is smaller; the first is wide enough for grouped Cholesky steps and paired
    # inverse steps
    for d, act, seed in ((8300, True, 61), (390, False, 62)):
        print(f"[noalloc] d={d} act_order={act}", flush=True)
        H32, n = _hessian(d, seed, act)
        Hd = torch.from_numpy(H32).cuda()
        p = g.Params(act_order=act, damp=0.01)
        U_ref, perm_ref = g.gptq_factor(Hd, n, p)
        U = torch.full((d, d), float("nan"), dtype=torch.float32, device="cuda")
        perm = torch.full((d,), -1, dtype=torch.int32, device="cuda")
        U2, perm2 = g.gptq_factor_noalloc(Hd, n, p, U, perm)
        torch.cuda.synchronize()
        assert U2.data_ptr() == U.data_ptr() and perm2.data_ptr() == perm.data_ptr()
        Ua, Ub = U.cpu().numpy(), U_ref.cpu().numpy()
        assert np.array_equal(Ua.view(np.uint32), Ub.view(np.uint32)), "U differs from gptq_factor's"
        assert np.array_equal(perm.cpu().numpy(), perm_ref.cpu().numpy())
        # the oracle's bar, on the processing order the GPU chose (checked: descending diag(H) with
        # act-order, the identity without)
        gp = perm.cpu().numpy().astype(np.int64)
        assert np.array_equal(np.sort(gp), np.arange(d))
        if act:
            dk = np.diag(H32.astype(np.float64))[gp]
            assert np.all(dk[1:] <= dk[:-1] * (1 + 1e-6))
        else:
            assert np.array_equal(gp, np.arange(d))
        Hh, _, _ = ref.damp_and_order(H32.astype(np.float64), n, 0.01, act, perm=gp if act else None)
        Uo = ref.inverse_cholesky_upper(Hh)
        err, resid = factor_errors(Ua, Hh, Uo)
        err32, resid32 = factor_errors(lapack_f32_factor(Hh), Hh, Uo)
        assert err <= FACTOR_VS_LAPACK * err32 and resid <= FACTOR_VS_LAPACK * resid32, (err, err32, resid, resid32)


def test_factor_noalloc_in_place_and_limits():
    """U == H works as for gptq_factor; a d above the scratch's maximum is rejected on the host."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    H32, n = _hessian(260, 63, True)
    p = g.Params(act_order=True, damp=0.01)
    U_ref, perm_ref = g.gptq_factor(torch.from_numpy(H32).cuda(), n, p)
    Hi = torch.from_numpy(H32).cuda()
    perm = torch.empty(260, dtype=torch.int32, device="cuda")
    g.gptq_factor_noalloc(Hi, n, p, Hi, perm)
    torch.cuda.synchronize()
    assert np.array_equal(Hi.cpu().numpy().view(np.uint32), U_ref.cpu().numpy().view(np.uint32))
    assert np.array_equal(perm.cpu().numpy(), perm_ref.cpu().numpy())
    big = g.GPTQ_FACTOR_NOALLOC_MAX_D + 1
    Hb = torch.zeros((big, big), dtype=torch.float32, device="cuda")
    with pytest.raises(g.GPTQError) as ei:
        g.gptq_factor_noalloc(Hb, 10, p, Hb, torch.empty(big, dtype=torch.int32, device="cuda"))
    assert ei.value.status == g.GPTQ_EUNSUPPORTED

"""GPU parity of hr_w8a8_gemm (both operands one int8 code per element:
the W4A4 GEMM with its codes held in int8, and W8A8) against the oracle, on
the tile kernel (M > 16, N a multiple of 128) and the simple kernel (other
shapes).  All calls go through the C ABI (the ctypes binding)."""
import numpy as np
import pytest
import torch

import hr_inputs
import oracle
from parity import check_gemm

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _hr():
    import hadamard_rotation_int4_amd as hr
    return hr


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _run(gi, group, scale_mode="f16", rows=None):
    hr = _hr()
    sd = np.float16 if scale_mode == "f16" else np.float32
    sa, sw = gi.a_scales.astype(sd), gi.w_scales.astype(sd)
    c, acc = hr.w8a8_gemm(_t(gi.a_codes), _t(sa), _t(gi.w_codes), _t(sw), group, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w8a8_gemm(gi.a_codes, sa, gi.w_codes, sw, group, rows=rows,
                                                  return_sums=True)
    cg, ag = c.cpu().numpy(), acc.cpu().numpy()
    if rows is not None:
        cg, ag = cg[rows], ag[rows]
    check_gemm(cg, c_ref, bound, ag, acc_ref)
    # the call without group sums is another kernel instance: same output
    c2 = hr.w8a8_gemm(_t(gi.a_codes), _t(sa), _t(gi.w_codes), _t(sw), group)
    assert torch.equal(c2, c)


@pytest.mark.parametrize("M,N,K,group", [(128, 128, 256, 128), (100, 256, 1024, 128),
                                         (130, 128, 512, 64), (256, 384, 2048, 256),
                                         (17, 128, 768, 128), (300, 256, 4096, 64)])
@pytest.mark.parametrize("code_max", [7, 127])
def test_w8a8_tile(M, N, K, group, code_max):
    """Tile kernel: ragged M, every group size, int4-valued and full-range codes."""
    gi = hr_inputs.gemm_i8_inputs(M=M, N=N, K=K, group=group, seed=700 + M + K, code_max=code_max)
    _run(gi, group)


@pytest.mark.parametrize("group", [64, 128, 256])
def test_w8a8_tile_fp32_scales(group):
    gi = hr_inputs.gemm_i8_inputs(M=192, N=256, K=1024, group=group, seed=760 + group, code_max=127)
    _run(gi, group, "f32")


@pytest.mark.parametrize("M,N,K,group", [(16, 256, 512, 128), (5, 64, 256, 64), (1, 192, 1024, 256),
                                         (64, 192, 512, 128)])
def test_w8a8_simple_kernel_shapes(M, N, K, group):
    """M <= 16 or N not a multiple of 128: the simple kernel's int8-weight mode."""
    gi = hr_inputs.gemm_i8_inputs(M=M, N=N, K=K, group=group, seed=780 + M, code_max=127)
    _run(gi, group)


def test_w8a8_extreme_codes():
    """-128 * -128 over whole groups: the largest int32 group sums."""
    M, N, K, G = 128, 128, 512, 256
    a = np.full((M, K), -128, dtype=np.int8)
    a[1::2] = 127
    w = np.full((N, K), -128, dtype=np.int8)
    ones_a = np.ones((M, K // G), np.float16)
    ones_w = np.ones((N, K // G), np.float16)
    gi = hr_inputs.GemmI8Inputs(a, ones_a, w, ones_w, M, N, K, G)
    _run(gi, G)


def test_w8a8_equals_w4a4_on_int4_codes():
    """int4-valued codes: the int8-held GEMM matches the packed W4A4 GEMM bit for bit."""
    hr = _hr()
    gi = hr_inputs.gemm_i8_inputs(M=256, N=256, K=1024, group=128, seed=790)
    sa, sw = _t(gi.a_scales), _t(gi.w_scales)
    c8, a8 = hr.w8a8_gemm(_t(gi.a_codes), sa, _t(gi.w_codes), sw, 128, group_acc=True)
    c4, a4 = hr.w4a4_gemm(_t(oracle.quant.pack_int4(gi.a_codes)), sa,
                          _t(oracle.quant.pack_int4(gi.w_codes)), sw, 128, group_acc=True)
    assert torch.equal(a8, a4)
    assert torch.equal(c8, c4)


def test_w8a8_4096():
    """The bench workload: 4096^3, G = 128, int4-valued codes held in int8; sampled rows."""
    gi = hr_inputs.gemm_i8_inputs(M=4096, N=4096, K=4096, group=128)
    rows = np.unique(np.concatenate([np.random.default_rng(7).choice(4096, 20, replace=False),
                                     [0, 4095]]))
    _run(gi, 128, rows=rows)

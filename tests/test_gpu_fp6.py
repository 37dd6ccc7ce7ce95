"""GPU parity of the fp6 path (hr_w4a4_to_fp6, hr_w4a4_gemm_fp6) against the
oracle, through the C ABI.  The tiled format is decoded here from its
definition: a slot is 32 codes of a row in 24 bytes, code 32 j + e of the slot
in bits 6 e .. 6 e + 5 of its 192-bit little-endian value, field = (q < 0) << 5
| |q|; panel p (128 rows), block b (128 codes) is the 12288-byte tile at
(p * K / 128 + b) * 12288, holding slots h and h + 2 of the panel's row r at
h * 6144 + r * 48 + 24 * (slot // 2)."""
import numpy as np
import pytest
import torch

import hr_inputs
import oracle
from parity import check_gemm, check_quant

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _hr():
    import hadamard_rotation_int4_amd as hr
    return hr


def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def decode_fp6_tiles(f6: np.ndarray, rows: int) -> np.ndarray:
    """Tiled fp6 bytes [padded rows][K*3/4] -> int codes [padded rows][K]
    (from the format definition); checks every field is a valid code."""
    prow, nb = f6.shape
    K = nb * 4 // 3
    flat = f6.reshape(-1)
    out = np.empty((prow, K), dtype=np.int64)
    for r in range(prow):
        p, rr = divmod(r, 128)
        for j in range(K // 32):
            b, sl = divmod(j, 4)
            at = (p * (K // 128) + b) * 12288 + (sl & 1) * 6144 + rr * 48 + (sl >> 1) * 24
            bits = int.from_bytes(flat[at:at + 24].tobytes(), "little")
            for e in range(32):
                f = (bits >> (6 * e)) & 0x3F
                assert f & 0x10 == 0 and (f & 0x0F) <= 8, (r, j, e, f)
                out[r, 32 * j + e] = -(f & 0x0F) if f & 0x20 else (f & 0x0F)
    return out


def decode_fp6_tiles_np(f6: np.ndarray, rows: int) -> np.ndarray:
    """The same decoding as decode_fp6_tiles, vectorised with numpy (for the
    larger cases): [padded rows][K*3/4] bytes -> int codes [rows][K]; only
    the first rows are checked and returned (padding rows may hold anything)."""
    prow, nb = f6.shape
    K = nb * 4 // 3
    P, KB = prow // 128, K // 128
    t = f6.reshape(P, KB, 2, 128, 2, 24)              # panel, block, plane h, row, slot pair, 24 bytes
    bits = np.unpackbits(t, axis=-1, bitorder="little").reshape(P, KB, 2, 128, 2, 32, 6)
    f = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)      # [P][KB][h][r][pair][e]
    # slot j of a block = plane j & 1, pair j >> 1
    f = f.transpose(0, 3, 1, 4, 2, 5).reshape(P * 128, K)[:rows]  # panel, row, block, pair, plane, e
    assert not (f & 0x10).any() and ((f & 0x0F) <= 8).all()
    return np.where(f & 0x20, -(f & 0x0F), f & 0x0F)


def _all_nibble_codes(rng, rows, K):
    """Packed codes with every nibble pattern, -8 included."""
    return rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)


@pytest.mark.parametrize("rows,K", [(1, 128), (5, 256), (130, 384), (33, 4096)])
def test_int4_to_fp6_matches_codes(rows, K):
    """Every code lands in its place in the tiles; padding rows are zeros
    (the output buffer starts as 0xFF bytes, so nothing is left unwritten)."""
    hr = _hr()
    codes = _all_nibble_codes(np.random.default_rng(rows + K), rows, K)
    out = torch.full((hr.fp6_rows(rows), K * 3 // 4), 255, dtype=torch.uint8, device=DEV)
    f6 = hr.w4a4_to_fp6(_t(codes), out=out).cpu().numpy()
    assert f6.shape == ((rows + 127) // 128 * 128, K * 3 // 4)
    dec = decode_fp6_tiles(f6, rows)
    np.testing.assert_array_equal(dec[:rows], oracle.quant.unpack_int4(codes).astype(np.int64))
    assert not dec[rows:].any()


@pytest.mark.parametrize("dtype", [np.float16, np.float32])
@pytest.mark.parametrize("rows,K,G", [(1, 128, 128), (130, 768, 256), (257, 1024, 128)])
def test_int4_to_fp6_scales(dtype, rows, K, G):
    """The scales come out transposed to [K/G][padded rows], bit for bit, with
    zeros in the padding rows; the tiles match the codes-only call."""
    hr = _hr()
    rng = np.random.default_rng(rows + K + G)
    codes = _all_nibble_codes(rng, rows, K)
    sc = (rng.random((rows, K // G)) + 0.01).astype(dtype)
    P = hr.fp6_rows(rows)
    o_s = torch.full((K // G, P), 7.0, dtype=torch.float16 if dtype == np.float16 else torch.float32, device=DEV)
    f6, st = hr.w4a4_to_fp6(_t(codes), _t(sc), G, out_scales=o_s)
    ref = np.zeros((K // G, P), dtype=dtype)
    ref[:, :rows] = sc.T
    np.testing.assert_array_equal(st.cpu().numpy().view(np.uint8), ref.view(np.uint8))
    assert torch.equal(f6, hr.w4a4_to_fp6(_t(codes)))


def _gemm_case(M, N, K, G, seed, scale_mode, all_nibbles=False):
    gi = hr_inputs.gemm_inputs(M=M, N=N, K=K, group=G, seed=seed)
    a, w = gi.a_codes, gi.w_codes
    if all_nibbles:
        rng = np.random.default_rng(seed)
        a, w = _all_nibble_codes(rng, M, K), _all_nibble_codes(rng, N, K)
    sa, sw = gi.a_scales, gi.w_scales
    if scale_mode == "f32":
        sa, sw = sa.astype(np.float32), sw.astype(np.float32)
    return a, w, sa, sw


@pytest.mark.parametrize("G", [128, 256])
@pytest.mark.parametrize("M", [1, 130, 256, 300])
@pytest.mark.parametrize("scale_mode", ["f16", "f32"])
def test_gemm_fp6_parity(G, M, scale_mode):
    """Several 128-row panels with a ragged last one (M = 130, 300), one
    panel (M = 1), whole panels (M = 256)."""
    hr = _hr()
    N, K = 256, 1024
    a, w, sa, sw = _gemm_case(M, N, K, G, 800 + M + G, scale_mode, all_nibbles=(M in (130, 300)))
    (a6, st_a), (w6, st_w) = hr.w4a4_to_fp6(_t(a), _t(sa), G), hr.w4a4_to_fp6(_t(w), _t(sw), G)
    c, acc = hr.w4a4_gemm_fp6(a6, st_a, w6, st_w, G, M, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(a, sa, w, sw, G, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    c2 = hr.w4a4_gemm_fp6(a6, st_a, w6, st_w, G, M)
    assert torch.equal(c, c2)


@pytest.mark.parametrize("K,G", [(128, 128), (384, 128), (640, 128), (512, 256), (1280, 256)])
def test_gemm_fp6_stage_counts(K, G):
    """K from one stage up, through every remainder of the three-stage
    pipeline (and of six stages for G = 256)."""
    hr = _hr()
    M, N = 70, 128
    a, w, sa, sw = _gemm_case(M, N, K, G, 860 + K + G, "f16", all_nibbles=True)
    (a6, st_a), (w6, st_w) = hr.w4a4_to_fp6(_t(a), _t(sa), G), hr.w4a4_to_fp6(_t(w), _t(sw), G)
    c, acc = hr.w4a4_gemm_fp6(a6, st_a, w6, st_w, G, M, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(a, sa, w, sw, G, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)


def test_gemm_fp6_long_k():
    """K = 65536 (the largest accepted): 512 groups per output."""
    hr = _hr()
    a, w, sa, sw = _gemm_case(64, 128, 65536, 128, 840, "f16", all_nibbles=True)
    (a6, st_a), (w6, st_w) = hr.w4a4_to_fp6(_t(a), _t(sa), 128), hr.w4a4_to_fp6(_t(w), _t(sw), 128)
    c, acc = hr.w4a4_gemm_fp6(a6, st_a, w6, st_w, 128, 64, group_acc=True)
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(a, sa, w, sw, 128, return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)


def test_gemm_fp6_4096_sampled():
    """The 4096^3 G = 128 workload: every output of 48 sampled rows (and the
    first and last) against the oracle, and the whole product against the int8
    kernel's within the GEMM tolerance."""
    hr = _hr()
    gi = hr_inputs.gemm_inputs(M=4096)
    a6, st_a = hr.w4a4_to_fp6(_t(gi.a_codes), _t(gi.a_scales), 128)
    w6, st_w = hr.w4a4_to_fp6(_t(gi.w_codes), _t(gi.w_scales), 128)
    c = hr.w4a4_gemm_fp6(a6, st_a, w6, st_w, 128, 4096)
    rows = np.unique(np.concatenate([np.random.default_rng(850).choice(4096, 48, replace=False), [0, 4095]]))
    c_ref, _, bound = oracle.gemm.w4a4_gemm(gi.a_codes, gi.a_scales, gi.w_codes, gi.w_scales, 128, rows=rows,
                                            return_sums=True)
    check_gemm(c[torch.from_numpy(rows).to(DEV)].cpu().numpy(), c_ref, bound)
    c8 = hr.w4a4_gemm(_t(gi.a_codes), _t(gi.a_scales), _t(gi.w_codes), _t(gi.w_scales), 128)
    diff = (c - c8).abs().max().item()
    assert diff <= 1e-5 * float(np.abs(bound).max()), diff


@pytest.mark.parametrize("rows", [1, 130, 300])
@pytest.mark.parametrize("n", [2048, 4096])
@pytest.mark.parametrize("G", [128, 256])
@pytest.mark.parametrize("scale_mode", ["f16", "f32"])
def test_rotate_quant_fp6(rows, n, G, scale_mode):
    """hr_rotate_quant_fp6: the tiles hold the oracle's codes of the rotated
    rows and the transposed scales its scales (the parity rules of the int4
    path), and they equal the int4 entry's codes and scales bit for bit."""
    hr = _hr()
    ri = hr_inputs.rht_inputs(rows=rows, n=n, seed=870 + rows + n + G)
    x, d = ri.x.to(DEV), _t(ri.signs)
    sdt = torch.float16 if scale_mode == "f16" else torch.float32
    tiles, st = hr.rotate_quant_fp6(x, G, d, scale_dtype=sdt)
    assert tiles.shape == (hr.fp6_rows(rows), n * 3 // 4) and st.shape == (n // G, hr.fp6_rows(rows))
    q = decode_fp6_tiles_np(tiles.cpu().numpy(), rows)
    sc = st.cpu().numpy()[:, :rows].T.copy()
    y64 = oracle.hadamard.rht(ri.x.float().numpy(), ri.signs)
    check_quant(oracle.quant.pack_int4(q), sc, y64, G, scale_mode)
    codes4, scales4 = hr.rotate_quant_int4(x, G, d, scale_dtype=sdt)
    np.testing.assert_array_equal(q, oracle.quant.unpack_int4(codes4.cpu().numpy()))
    np.testing.assert_array_equal(sc.view(np.uint8), scales4.cpu().numpy().view(np.uint8))


@pytest.mark.parametrize("M", [16, 300])
def test_rotate_quant_fp6_then_gemm(M):
    """bf16 activations -> hr_rotate_quant_fp6 -> hr_w4a4_gemm_fp6 against the
    oracle GEMM on the activation codes the tiles hold and the weight codes
    (int32 group sums exact); the padding rows were never written."""
    hr = _hr()
    N, K, G = 256, 4096, 128
    ri = hr_inputs.rht_inputs(rows=M, n=K, seed=880 + M)
    gi = hr_inputs.gemm_inputs(M=1, N=N, K=K, group=G, seed=881)
    x, d = ri.x.to(DEV), _t(ri.signs)
    tiles = torch.full((hr.fp6_rows(M), K * 3 // 4), 0xFF, dtype=torch.uint8, device=DEV)
    st = torch.full((K // G, hr.fp6_rows(M)), float("nan"), dtype=torch.float16, device=DEV)
    hr.rotate_quant_fp6(x, G, d, out=tiles, out_scales=st)
    w6, stw = hr.w4a4_to_fp6(_t(gi.w_codes), _t(gi.w_scales), G)
    c, acc = hr.w4a4_gemm_fp6(tiles, st, w6, stw, G, M, group_acc=True)
    a_codes = oracle.quant.pack_int4(decode_fp6_tiles_np(tiles.cpu().numpy(), M))
    a_scales = st.cpu().numpy()[:, :M].T.copy()
    c_ref, acc_ref, bound = oracle.gemm.w4a4_gemm(a_codes, a_scales, gi.w_codes, gi.w_scales, G,
                                                  return_sums=True)
    check_gemm(c.cpu().numpy(), c_ref, bound, acc.cpu().numpy(), acc_ref)
    assert torch.isfinite(c).all()


def _sample(rows, k, seed=0):
    idx = np.random.default_rng(seed).choice(rows, size=k, replace=False)
    return np.unique(np.concatenate([idx, [0, rows - 1]]))


@pytest.mark.parametrize("rows,n", [(65536, 2048), (4096, 4096)])
def test_rotate_quant_fp6_fullsize(rows, n):
    """The headline shape (bf16 65536 x 2048) and the GEMM's activation
    shape (4096 x 4096), G = 128, fp16 scales: every row's decoded tile codes
    and every transposed scale equal the int4 entry's bit for bit, and a
    seeded sample of rows (plus the first and last) matches the oracle."""
    hr = _hr()
    ri = hr_inputs.rht_inputs(rows=rows, n=n)
    x, d = ri.x.to(DEV), _t(ri.signs)
    tiles, st = hr.rotate_quant_fp6(x, 128, d)
    codes4, scales4 = hr.rotate_quant_int4(x, 128, d)
    tiles_np, c4 = tiles.cpu().numpy(), codes4.cpu().numpy()
    for r0 in range(0, rows, 4096):
        nr = min(4096, rows - r0)
        q = decode_fp6_tiles_np(tiles_np[r0:r0 + (nr + 127) // 128 * 128], nr)
        np.testing.assert_array_equal(q, oracle.quant.unpack_int4(c4[r0:r0 + nr]))
    sc = st.cpu().numpy()[:, :rows].T
    np.testing.assert_array_equal(sc.view(np.uint16), scales4.cpu().numpy().view(np.uint16))
    sample = _sample(rows, 64, seed=n)
    q = np.concatenate([decode_fp6_tiles_np(tiles_np[r // 128 * 128:(r // 128 + 1) * 128], r % 128 + 1)[-1:]
                        for r in sample])
    y64 = oracle.hadamard.rht(ri.x[sample].float().numpy(), ri.signs)
    check_quant(oracle.quant.pack_int4(q), sc[sample], y64, 128, "f16")


@pytest.mark.parametrize("rows,n", [(5, 2048), (131, 4096)])
def test_rotate_quant_fp6_tiny_fp32_scales(rows, n):
    """Delta rows c e_0 with c = 2^-120 (bf16): every rotated value is
    +-c / sqrt(n), the fp32 scale is below 2^-128 (its reciprocal would
    overflow; the quantizer rescales by 2^64) and every code is +-7; the
    tiles hold those codes and the transposed scales match the oracle's."""
    hr = _hr()
    d = hr_inputs.sign_vector(np.random.default_rng(502), n)
    x = np.zeros((rows, n), dtype=np.float32)
    x[:, 0] = np.float32(2.0 ** -120)
    x[1::2, 0] *= -1
    xt = torch.from_numpy(x).to(torch.bfloat16)
    tiles, st = hr.rotate_quant_fp6(xt.to(DEV), 128, _t(d), scale_dtype=torch.float32)
    q = decode_fp6_tiles_np(tiles.cpu().numpy(), rows)
    s = st.cpu().numpy()[:, :rows].T.copy()
    y64 = oracle.hadamard.rht(x, d)
    assert np.all(s < 2.0 ** -128) and np.all(s > 0)
    assert np.all(np.abs(q) == 7)
    check_quant(oracle.quant.pack_int4(q), s, y64, 128, "f32")

"""Parity of gptq_dequant_gemm, the stored layer's product y = x W^T, with the float64 oracle.

Two kinds of check:
* exact: integer inputs in [-2, 2], power-of-two scales and zeros within [-4, 20) keep every partial
  sum an exactly representable fp32 value, whatever the summation order, so the kernels must equal
  the oracle bit for bit;
* bounded: normal inputs and log-uniform scales, compared with the oracle within the error bound of
  the kernels' fp32 summation, 2 (d / 64 + 48) u sum_k |x_k| s (q_k + |z|), u = 2^-24 (a lane sums
  at most d / 64 columns, a 32-column chunk adds at most 34 roundings, the wave reduction 7).
"""

import numpy as np
import pytest

from gpu_util import dev_tensor, gpu_layer, torch_cuda
import synth
from oracle import gptq_ref as ref

pytestmark = pytest.mark.gpu

U32 = 2.0 ** -24


def _groups(L, d):
    g = d if L.group_size <= 0 else L.group_size
    return np.arange(d) // g if L.g_idx is None else L.g_idx.astype(np.int64)


def _bound(x64, L, d):
    G = _groups(L, d)
    s = L.scales.astype(np.float64)[:, G]
    z = np.abs(L.zeros.astype(np.float64))[:, G]
    S = np.abs(x64) @ (s * (L.codes.astype(np.float64) + z)).T
    return 2.0 * (d / 64 + 48) * U32 * S


def _gpu(L, x, xdtype, d, bits=4, pass_gidx=True, ldx_pad=0, gidx_offset=0, dense=False):
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    codes = dev_tensor(L.codes, "u8")
    packed = g.gptq_pack_dense(codes, bits) if dense else g.gptq_pack(codes, bits)
    xs = x
    if ldx_pad:
        xs = np.zeros((x.shape[0], d + ldx_pad), dtype=x.dtype)
        xs[:, :d] = x
    xd = dev_tensor(xs, xdtype)[:, :d]
    gi = None
    if L.g_idx is not None and pass_gidx:
        # gidx_offset > 0 hands over a g_idx that is not 16-byte aligned (a view one element in)
        gi = dev_tensor(np.concatenate([np.zeros(gidx_offset, np.int32), L.g_idx]), "i32")[gidx_offset:]
    y = g.gptq_dequant_gemm(xd, packed, dev_tensor(L.scales, "f32"), dev_tensor(L.zeros, "i32"), d, L.group_size,
                            g_idx=gi, bits=bits, dense=dense)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def _oracle(L, x64, d, bits=4, dense=False):
    gidx = _groups(L, d)
    packed = ref.pack_dense(L.codes, bits) if dense else ref.pack(L.codes, bits)
    return ref.dequant_matmul(x64, packed, L.scales, L.zeros, gidx, d, bits, dense)


EXACT_CASES = [
    # (name, x dtype, rows, d, m, group_size, act_order)
    ("fast g128", "f16", 300, 4096, 5, 128, False),
    ("fast per-row group", "f16", 37, 2080, 1, 0, False),
    ("fast g32 m8", "f16", 64, 1024, 8, 32, False),
    ("general g16", "f16", 33, 512, 3, 16, False),
    ("general act-order f16", "f16", 300, 4096, 5, 128, True),
    ("general act-order bf16", "bf16", 40, 2048, 2, 64, True),
    ("general f32 g128", "f32", 40, 1024, 4, 128, False),
    ("general d%32 and m=9", "f16", 9, 136, 9, 8, False),
]


@pytest.mark.parametrize("name,xdt,rows,d,m,gs,act", EXACT_CASES, ids=[c[0] for c in EXACT_CASES])
def test_exact_inputs_bit_identical(name, xdt, rows, d, m, gs, act):
    print(f"[dequant exact] {name}: rows {rows} d {d} m {m} g {gs} act {act} x {xdt}", flush=True)
    L = synth.stored_layer(11, rows, d, 4, gs, act_order=act, exact=True)
    x = synth.inference_x(12, m, d, xdt, exact=True)
    y = _gpu(L, x, xdt, d)
    want = _oracle(L, synth.to_f64(x, xdt), d)
    assert np.array_equal(y.astype(np.float64), want)


MFMA_CASES = [
    # (rows, d, m, group_size): the matrix-core kernel takes fp16 inputs, 3..16 rows per pass and
    # groups of whole 128-column units; 16, 8 or 4 waves per workgroup by the row count
    (300, 4096, 3, 128),
    (300, 1152, 16, 128),       # an odd number of 128-column units
    (45, 384, 17, 0),           # 16 rows on the matrix cores, then one on the dot2 kernel
    (45, 384, 18, 0),           # then two on the dot2 kernel
    (8200, 512, 5, 256),        # 8 waves per workgroup
    (12300, 256, 33, 128),      # 4 waves per workgroup; passes of 16, 16 and 1
]


@pytest.mark.parametrize("rows,d,m,gs", MFMA_CASES, ids=[f"r{c[0]}-d{c[1]}-m{c[2]}-g{c[3]}" for c in MFMA_CASES])
def test_matrix_core_kernel_exact(rows, d, m, gs):
    print(f"[dequant mfma exact] rows {rows} d {d} m {m} g {gs}", flush=True)
    L = synth.stored_layer(21, rows, d, 4, gs, exact=True)
    x = synth.inference_x(22, m, d, "f16", exact=True)
    y = _gpu(L, x, "f16", d)
    assert np.array_equal(y.astype(np.float64), _oracle(L, synth.to_f64(x, "f16"), d))


LAYOUT_CASES = [
    # (bits, dense, x dtype, rows, d, m, group_size, act_order)
    (8, False, "f16", 70, 1024, 1, 128, False),
    (8, False, "bf16", 33, 512, 5, 64, True),
    (5, False, "f32", 20, 256, 2, 0, False),
    (3, True, "f16", 70, 2048, 1, 128, False),
    (3, True, "f16", 40, 1056, 9, 32, True),
    (2, True, "bf16", 33, 512, 3, 64, False),
    (5, True, "f16", 25, 96 * 8, 2, 96, False),
    (7, True, "f32", 17, 32 * 8, 4, 0, True),
    (4, True, "f16", 64, 1024, 3, 128, False),     # dense at 4 bits is the nibble layout
]


@pytest.mark.parametrize("bits,dense,xdt,rows,d,m,gs,act", LAYOUT_CASES,
                         ids=[f"{c[0]}bit-{'dense' if c[1] else 'fields'}-{c[2]}-m{c[5]}" for c in LAYOUT_CASES])
def test_storage_layouts_exact(bits, dense, xdt, rows, d, m, gs, act):
    """Byte fields (5 to 8 bits) and dense bit streams (codes straddling words) through the product."""
    print(f"[dequant layout] bits {bits} dense {dense} x {xdt} rows {rows} d {d} m {m} g {gs} act {act}", flush=True)
    L = synth.stored_layer(23, rows, d, bits, gs, act_order=act, exact=True)
    x = synth.inference_x(24, m, d, xdt, exact=True)
    y = _gpu(L, x, xdt, d, bits=bits, dense=dense)
    assert np.array_equal(y.astype(np.float64), _oracle(L, synth.to_f64(x, xdt), d, bits, dense))


@pytest.mark.parametrize("m", [5, 16])
def test_matrix_core_kernel_far_zeros_exact(m):
    """Zeros far outside the code range (groups of one sign far from zero) through the matrix-core
    kernel, which subtracts z sum x in fp32 after the product. Exact inputs, so bit-identical."""
    rows, d = 40, 256
    L = synth.stored_layer(25, rows, d, 4, 128, exact=True)
    zeros = L.zeros.copy()
    zeros[3, 0], zeros[7, 1], zeros[20, 0] = 3000, -2500, 1001
    L = synth.StoredLayer(L.codes, L.scales, zeros, None, 128)
    x = synth.inference_x(26, m, d, "f16", exact=True)
    y = _gpu(L, x, "f16", d)
    assert np.array_equal(y.astype(np.float64), _oracle(L, synth.to_f64(x, "f16"), d))


@pytest.mark.parametrize("rows,m", [(8200, 2), (4100, 1), (4100, 8), (8193, 4)])
def test_rows_per_wave_variants_exact(rows, m):
    """Row counts that select four, two and one weight rows per wave, each with a ragged last wave."""
    print(f"[dequant rows/wave] rows {rows} m {m}", flush=True)
    d = 256
    L = synth.stored_layer(13, rows, d, 4, 64, exact=True)
    x = synth.inference_x(14, m, d, "f16", exact=True)
    y = _gpu(L, x, "f16", d)
    assert np.array_equal(y.astype(np.float64), _oracle(L, synth.to_f64(x, "f16"), d))


BOUND_CASES = [
    ("fast g128", "f16", 500, 4096, 1, 128, False, 0),
    ("mfma g128", "f16", 500, 4096, 3, 128, False, 0),
    ("mfma per-row m16", "f16", 300, 8192, 16, 0, False, 0),
    ("fast per-row 3-bit", "f16", 64, 8192, 1, 0, False, 0),
    ("general act-order", "f16", 200, 4096, 4, 128, True, 0),
    ("general act-order unaligned g_idx", "f16", 70, 1024, 1, 64, True, 0),
    ("general act-order many groups", "f16", 70, 8192, 2, 16, True, 0),     # tables too big for LDS
    ("general unaligned x", "f16", 50, 2048, 2, 128, False, 3),
    ("general bf16", "bf16", 50, 2048, 6, 32, False, 0),
    ("general f32", "f32", 50, 2048, 16, 128, True, 0),
]


@pytest.mark.parametrize("name,xdt,rows,d,m,gs,act,pad", BOUND_CASES, ids=[c[0] for c in BOUND_CASES])
def test_normal_inputs_within_bound(name, xdt, rows, d, m, gs, act, pad):
    print(f"[dequant bound] {name}: rows {rows} d {d} m {m} g {gs} act {act} x {xdt} pad {pad}", flush=True)
    bits = 3 if "3-bit" in name else 4
    L = synth.stored_layer(15, rows, d, bits, gs, act_order=act)
    x = synth.inference_x(16, m, d, xdt)
    y = _gpu(L, x, xdt, d, bits=bits, ldx_pad=pad, gidx_offset=1 if "unaligned g_idx" in name else 0)
    y = y.astype(np.float64)
    x64 = synth.to_f64(x, xdt)
    want = _oracle(L, x64, d, bits)
    err = np.abs(y - want)
    tol = _bound(x64, L, d)
    assert np.all(err <= tol), (err.max(), tol[err > tol][:4])


def test_without_g_idx_matches_with_identity_groups():
    """Passing g_idx = k // g explicitly (the general kernel) and passing none (the fast kernel) agree
    exactly on exact inputs."""
    d, rows = 2048, 100
    L = synth.stored_layer(17, rows, d, 4, 128, exact=True)
    x = synth.inference_x(18, 4, d, "f16", exact=True)
    L2 = synth.StoredLayer(L.codes, L.scales, L.zeros, (np.arange(d) // 128).astype(np.int32), 128)
    assert np.array_equal(_gpu(L, x, "f16", d), _gpu(L2, x, "f16", d))


@pytest.mark.parametrize("act", [False, True])
def test_quantized_layer_end_to_end(act):
    """A layer through the four solver calls, then its stored outputs through gptq_dequant_gemm."""
    print(f"[dequant end-to-end] act {act}", flush=True)
    case = synth.make_case("dq_e2e", seed=19, rows=96, d=256, n=1024, bits=4, group_size=32, block_size=32,
                           act_order=act)
    W, chunks, out = gpu_layer(case)
    L = synth.StoredLayer(out["codes"], out["scales"], out["zeros"], out["g_idx"] if act else None, 32)
    x = synth.inference_x(20, 5, 256, "f16")
    x64 = synth.to_f64(x, "f16")
    y = _gpu(L, x, "f16", 256).astype(np.float64)
    want = ref.dequant_matmul(x64, ref.pack(out["codes"], 4), out["scales"], out["zeros"], out["g_idx"], 256)
    assert np.all(np.abs(y - want) <= _bound(x64, L, 256))


# ------------------------------------------------------------------ the benchmark's stored layers

def _bench_layers():
    import bench
    return bench.DEQUANT_LAYERS


@pytest.mark.parametrize("name,m", [("fc2", 1), ("fc2", 4), ("q_proj", 16), ("down_proj", 1), ("down_proj", 8)])
def test_benchmark_layers_full_size(name, m):
    """bench.py --dequant's stored layers at full size, in the launch configuration it times: the
    bench's own seeded layer and inputs within the error bound, and exact inputs bit for bit, on 64
    sampled weight rows the oracle computes one by one."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    rows, d, bits, gs, act = _bench_layers()[name]
    print(f"[dequant full size] {name} {rows}x{d} {bits}-bit g{gs} act {act} m {m}", flush=True)
    sample = np.sort(np.random.default_rng(7).choice(rows, 64, replace=False))
    for exact in (False, True):
        L = synth.stored_layer(400 if not exact else 402, rows, d, bits, gs, act_order=act, exact=exact)
        x = synth.inference_x(401 if not exact else 403, m, d, "f16", exact=exact)
        codes = torch.from_numpy(L.codes).cuda()
        packed = g.gptq_pack(codes, bits)
        del codes
        y = g.gptq_dequant_gemm(torch.from_numpy(x).cuda(), packed, torch.from_numpy(L.scales).cuda(),
                                torch.from_numpy(L.zeros).cuda(), d, gs,
                                g_idx=torch.from_numpy(L.g_idx).cuda() if act else None, bits=bits)
        torch.cuda.synchronize()
        y = y.cpu().numpy().astype(np.float64)[:, sample]
        Ls = synth.StoredLayer(L.codes[sample], L.scales[sample], L.zeros[sample], L.g_idx, gs)
        x64 = synth.to_f64(x, "f16")
        want = _oracle(Ls, x64, d, bits)
        if exact:
            assert np.array_equal(y, want)
        else:
            assert np.all(np.abs(y - want) <= _bound(x64, Ls, d))
        del packed, L


def test_three_bit_layer_dense_end_to_end():
    """A 3-bit layer through the solver on the GPU, stored as a dense bit stream (3 bits per code)
    and multiplied straight from it, against the oracle on the same stored outputs."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    case = synth.make_case("dq_dense", seed=27, rows=80, d=384, n=1500, bits=3, group_size=128, block_size=128,
                           act_order=True)
    W, chunks, out = gpu_layer(case)
    packed = g.gptq_pack_dense(torch.from_numpy(out["codes"]).cuda(), 3)
    assert np.array_equal(packed.cpu().numpy(), ref.pack_dense(out["codes"], 3))
    x = synth.inference_x(28, 4, 384, "f16")
    y = g.gptq_dequant_gemm(torch.from_numpy(x).cuda(), packed, torch.from_numpy(out["scales"]).cuda(),
                            torch.from_numpy(out["zeros"]).cuda(), 384, 128,
                            g_idx=torch.from_numpy(out["g_idx"]).cuda(), bits=3, dense=True)
    torch.cuda.synchronize()
    x64 = synth.to_f64(x, "f16")
    want = ref.dequant_matmul(x64, ref.pack_dense(out["codes"], 3), out["scales"], out["zeros"], out["g_idx"], 384,
                              3, True)
    L = synth.StoredLayer(out["codes"], out["scales"], out["zeros"], out["g_idx"], 128)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - want) <= _bound(x64, L, 384))


# ------------------------------------------------------------------ act-order layers stored in processing order

@pytest.mark.parametrize("xdt,rows,d,m,gs,exact", [("f16", 300, 4096, 1, 128, True), ("f16", 200, 2048, 5, 128, True),
                                                   ("f16", 100, 1024, 2, 64, False), ("bf16", 40, 512, 3, 32, True)])
def test_act_order_reordered_product(xdt, rows, d, m, gs, exact):
    """An act-order layer packed in processing order (groups contiguous) times inputs gathered by the
    same order equals the oracle's product of the stored layer in its original order: exactly on
    exact inputs, within the bound otherwise."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    print(f"[dequant reordered] x {xdt} rows {rows} d {d} m {m} g {gs} exact {exact}", flush=True)
    L = synth.stored_layer(29, rows, d, 4, gs, act_order=True, exact=exact)
    order = np.argsort(L.g_idx, kind="stable").astype(np.int32)
    assert np.array_equal(L.g_idx[order], np.arange(d) // gs)
    x = synth.inference_x(30, m, d, xdt, exact=exact)
    od = torch.from_numpy(order).cuda()
    packed = g.gptq_pack_ordered(torch.from_numpy(L.codes).cuda(), 4, od)
    assert np.array_equal(packed.cpu().numpy(), ref.pack(L.codes[:, order], 4))
    xd = dev_tensor(x, xdt)
    xp = g.gptq_permute_columns(xd, od)
    torch.cuda.synchronize()
    xin = x if xdt != "bf16" else x.view(np.uint16)
    got_xp = xp.cpu().view(torch.int16).numpy().view(np.uint16) if xdt == "bf16" else xp.cpu().numpy()
    assert np.array_equal(got_xp, xin[:, order])
    y = g.gptq_dequant_gemm(xp, packed, torch.from_numpy(L.scales).cuda(), torch.from_numpy(L.zeros).cuda(), d, gs)
    torch.cuda.synchronize()
    y = y.cpu().numpy().astype(np.float64)
    x64 = synth.to_f64(x, xdt)
    want = _oracle(L, x64, d)
    if exact:
        assert np.array_equal(y, want)
    else:
        assert np.all(np.abs(y - want) <= _bound(x64, L, d))


def test_act_order_layer_reordered_end_to_end():
    """A layer solved with act-order on the GPU, stored in its processing order (the factor's perm)
    and multiplied on reordered inputs, against the oracle's product of the standard stored layer."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    case = synth.make_case("dq_ord", seed=31, rows=96, d=512, n=2048, bits=4, group_size=128, block_size=128,
                           act_order=True)
    W, chunks, out = gpu_layer(case)
    od = torch.from_numpy(out["perm"].astype(np.int32)).cuda()
    packed = g.gptq_pack_ordered(torch.from_numpy(out["codes"]).cuda(), 4, od)
    x = synth.inference_x(32, 6, 512, "f16")
    xp = g.gptq_permute_columns(torch.from_numpy(x).cuda(), od)
    y = g.gptq_dequant_gemm(xp, packed, torch.from_numpy(out["scales"]).cuda(), torch.from_numpy(out["zeros"]).cuda(),
                            512, 128)
    torch.cuda.synchronize()
    x64 = synth.to_f64(x, "f16")
    want = ref.dequant_matmul(x64, ref.pack(out["codes"], 4), out["scales"], out["zeros"], out["g_idx"], 512)
    L = synth.StoredLayer(out["codes"], out["scales"], out["zeros"], out["g_idx"], 128)
    assert np.all(np.abs(y.cpu().numpy().astype(np.float64) - want) <= _bound(x64, L, 512))


@pytest.mark.parametrize("m,act", [(1, False), (5, False), (3, True)])
def test_deterministic_and_strided_output(m, act):
    """Two calls give bit-identical results (no atomics; fixed reduction order), and an output with a
    row pitch wider than rows leaves its padding untouched."""
    torch = torch_cuda()
    import post_weight_quantization_20_amd as g
    rows, d = 1000, 2048
    L = synth.stored_layer(33, rows, d, 4, 128, act_order=act)
    x = torch.from_numpy(synth.inference_x(34, m, d, "f16")).cuda()
    packed = g.gptq_pack(torch.from_numpy(L.codes).cuda(), 4)
    sc, ze = torch.from_numpy(L.scales).cuda(), torch.from_numpy(L.zeros).cuda()
    gi = torch.from_numpy(L.g_idx).cuda() if act else None
    y1 = g.gptq_dequant_gemm(x, packed, sc, ze, d, 128, g_idx=gi)
    big = torch.full((m, rows + 24), 7.0, dtype=torch.float32, device="cuda")
    y2 = g.gptq_dequant_gemm(x, packed, sc, ze, d, 128, g_idx=gi, y=big[:, :rows])
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.all(big[:, rows:] == 7.0)

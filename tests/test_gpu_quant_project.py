"""GPU parity of qsvd_quantize_latent (bit-exact codes and scales) and
qsvd_project (bit-exact int8 path, tolerance for bf16) against the oracle."""
import numpy as np
import pytest

import oracle
import synth
from gpu_util import bf16_bits, dev, empty, host, say

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu


def run_quant(x, in_dt, hadamard, bits, group):
    import torch
    M, n = x.shape
    codes = empty((M, n if bits == 8 else n // 2), torch.int8 if bits == 8 else torch.uint8)
    nsc = 1 if group == 0 else n // group
    scales = empty((M, nsc) if group else (M,), torch.float32)
    q.qsvd_quantize_latent(dev(x), in_dt, M, n, hadamard, q.I8 if bits == 8 else q.I4, group,
                           codes, scales)
    torch.cuda.synchronize()
    c = codes.cpu().numpy()
    if bits == 4:
        c = oracle.unpack_int4(c)
    return c, scales.cpu().numpy()


def rows(M, n, seed, dtype):
    g = np.random.default_rng(seed)
    x = g.standard_normal((M, n))
    ch = synth.outlier_channels(n, 0.01, g)
    x[:, ch] *= 50.0
    x[M // 3:M // 3 + 1] = 0.0          # a zero row
    if M > 5:
        x[5] = 0.0
        x[5, n // 2] = -3.0              # single spike
    if dtype == "bf16":
        bits = synth.to_bf16_bits(x)
        return bits, oracle.bf16_decode(bits), q.BF16
    f = x.astype(np.float32)
    return f, f.astype(np.float64), q.F32


CASES = [
    # M, n, in dtype, hadamard, bits, group
    (1, 128, "f32", 128, 8, 0),
    (7, 768, "f32", 128, 4, 128),
    (300, 1536, "f32", 128, 8, 0),
    (300, 4096, "bf16", 128, 8, 0),
    (64, 5120, "bf16", 128, 8, 0),
    (33, 8192, "bf16", 128, 4, 128),
    (129, 2304, "f32", 128, 4, 128),
    (50, 24, "f32", 0, 8, 0),
    (50, 520, "bf16", 0, 4, 0),
    (20, 256, "f32", 0, 4, 128),
    (1000, 768, "f32", 128, 4, 128),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "M{}n{}{}h{}i{}g{}".format(*c))
def test_rotate_quantize_bit_exact(case):
    M, n, dt, had, bits, group = case
    say(f"case: quantize {case}")
    x, xv, in_dt = rows(M, n, seed=M * 7 + n, dtype=dt)
    codes, scales = run_quant(x, in_dt, had, bits, group)
    ref_c, ref_s = oracle.rotate_quantize(xv, had, bits, group)
    assert np.array_equal(codes, ref_c)
    assert np.array_equal(scales.reshape(ref_s.shape).view(np.uint32), ref_s.view(np.uint32))


def test_quantize_exact_ties_without_rotation():
    """Rows whose quotients fall exactly on k + 1/2 round to the even code."""
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "quantiser_cases.json")))
    for case in g["cases"]:
        y = np.array(case["y"], dtype=np.float32)
        x = np.zeros((1, 8), np.float32)
        x[0] = y
        codes, scales = run_quant(x, q.F32, 0, case["bits"], 0)
        assert codes[0].tolist() == case["codes"], case["name"]


def test_quantize_empty_rows_is_noop():
    import torch
    codes = torch.full((4, 128), 5, dtype=torch.int8, device="cuda")
    scales = torch.full((4,), 2.0, device="cuda")
    x = torch.zeros((4, 128), device="cuda")
    q.qsvd_quantize_latent(x, q.F32, 0, 128, 128, q.I8, 0, codes, scales)
    torch.cuda.synchronize()
    assert int(codes.min()) == 5 and float(scales.min()) == 2.0


# ------------------------------------------------------------------ projection
def run_project_i8(A, sa, W, sw, out_bf16=False):
    import torch
    M, K = A.shape
    N = W.shape[1]
    Wt = dev(np.ascontiguousarray(W.T))
    C = empty((M, N), torch.bfloat16 if out_bf16 else torch.float32)
    q.qsvd_project(dev(A), q.I8, dev(sa), M, K, Wt, q.I8, dev(sw) if sw is not None else None, N,
                   C, q.BF16 if out_bf16 else q.F32)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,K,N", [(1, 64, 16), (33, 128, 48), (257, 4096, 1536), (130, 512, 272),
                                   (77, 192, 48), (300, 1088, 2048), (1000, 4096, 400),
                                   (512, 2048, 8192)])
def test_project_int8_bit_exact(M, K, N):
    say(f"case: project int8 M={M} K={K} N={N}")
    g = np.random.default_rng(M + K + N)
    A = g.integers(-127, 128, size=(M, K)).astype(np.int8)
    W = g.integers(-127, 128, size=(K, N)).astype(np.int8)
    sa = (g.random(M) * 1e-2 + 1e-4).astype(np.float32)
    sw = (g.random(N) * 1e-2 + 1e-4).astype(np.float32)
    C = host(run_project_i8(A, sa, W, sw))
    ref = oracle.project_int8(A, sa, W, sw)
    assert np.array_equal(C, ref)
    # extreme accumulators: all +127 * +127
    A2 = np.full((3, K), 127, np.int8)
    W2 = np.full((K, 16), -127, np.int8)
    C2 = host(run_project_i8(A2, np.ones(3, np.float32), W2, None))
    assert np.array_equal(C2, oracle.project_int8(A2, np.ones(3, np.float32), W2, np.ones(16)))


def test_project_int8_bf16_output():
    g = np.random.default_rng(4)
    A = g.integers(-127, 128, size=(100, 256)).astype(np.int8)
    W = g.integers(-127, 128, size=(256, 64)).astype(np.int8)
    sa = (g.random(100) * 1e-2).astype(np.float32)
    sw = (g.random(64) * 1e-2).astype(np.float32)
    C = run_project_i8(A, sa, W, sw, out_bf16=True)
    ref = oracle.bf16_round(oracle.project_int8(A, sa, W, sw))
    assert np.array_equal(host(C), ref)


@pytest.mark.parametrize("M,K,N", [(5, 64, 16), (300, 4096, 1536), (129, 1024, 2304)])
def test_project_bf16(M, K, N):
    import torch
    say(f"case: project bf16 M={M} K={K} N={N}")
    g = np.random.default_rng(K + N)
    X = synth.to_bf16_bits(g.standard_normal((M, K)))
    W = synth.to_bf16_bits(g.standard_normal((K, N)) / np.sqrt(K))
    cs = (g.random(N) + 0.5).astype(np.float32)
    C = empty((M, N), torch.float32)
    Wt = dev(np.ascontiguousarray(W.T))
    q.qsvd_project(dev(X), q.BF16, None, M, K, Wt, q.BF16, dev(cs), N, C, q.F32)
    torch.cuda.synchronize()
    ref = oracle.project_real(oracle.bf16_decode(X), oracle.bf16_decode(W)) * cs
    got = host(C)
    # float32 accumulation over K products: |err| <= K * 2^-24 * sum|x w| (loose bound)
    bound = K * 2.0 ** -24 * (np.abs(oracle.bf16_decode(X)) @ np.abs(oracle.bf16_decode(W))) * cs
    assert np.all(np.abs(got - ref) <= bound + 1e-30)
    assert oracle.rel_l2(got, ref) < 1e-5


def run_project_i4(A, sa, W, sw, out_bf16=False):
    """A int8 codes [M][K] (int4 range), W int8 codes [K][N]; X packed on the host,
    W packed by qsvd_pack_weight (checked against the host packing)."""
    import torch
    M, K = A.shape
    N = W.shape[1]
    Wp = empty((N, K // 2), torch.uint8)
    q.qsvd_pack_weight(dev(W), q.I4, K, N, Wp)
    torch.cuda.synchronize()
    assert np.array_equal(Wp.cpu().numpy(), oracle.pack_int4(np.ascontiguousarray(W.T)))
    C = empty((M, N), torch.bfloat16 if out_bf16 else torch.float32)
    q.qsvd_project(dev(oracle.pack_int4(A)), q.I4, dev(sa), M, K, Wp, q.I4,
                   dev(sw) if sw is not None else None, N, C, q.BF16 if out_bf16 else q.F32)
    torch.cuda.synchronize()
    return C


@pytest.mark.parametrize("M,K,N", [(1, 128, 16), (77, 1152, 48), (257, 4096, 1536), (130, 512, 272),
                                   (300, 2048, 8192), (1000, 4096, 400)])
def test_project_int4_bit_exact(M, K, N):
    say(f"case: project W4A4 M={M} K={K} N={N}")
    g = np.random.default_rng(M + 3 * K + N)
    A = g.integers(-8, 8, size=(M, K)).astype(np.int8)      # the full nibble range
    W = g.integers(-8, 8, size=(K, N)).astype(np.int8)
    sa = (g.random(M) * 1e-2 + 1e-4).astype(np.float32)
    sw = (g.random(N) * 1e-2 + 1e-4).astype(np.float32)
    C = host(run_project_i4(A, sa, W, sw))
    assert np.array_equal(C, oracle.project_int8(A, sa, W, sw))
    # extreme sums: all -8 * -8
    A2 = np.full((3, K), -8, np.int8)
    W2 = np.full((K, 16), -8, np.int8)
    C2 = host(run_project_i4(A2, np.ones(3, np.float32), W2, None))
    assert np.array_equal(C2, oracle.project_int8(A2, np.ones(3, np.float32), W2, np.ones(16)))


def test_project_int4_bf16_output():
    g = np.random.default_rng(8)
    A = g.integers(-7, 8, size=(100, 256)).astype(np.int8)
    W = g.integers(-7, 8, size=(256, 64)).astype(np.int8)
    sa = (g.random(100) * 1e-2).astype(np.float32)
    sw = (g.random(64) * 1e-2).astype(np.float32)
    C = run_project_i4(A, sa, W, sw, out_bf16=True)
    assert np.array_equal(host(C), oracle.bf16_round(oracle.project_int8(A, sa, W, sw)))


def test_pack_weight_transposes():
    import torch
    g = np.random.default_rng(0)
    for dt, arr in ((q.I8, g.integers(-127, 128, (37, 70)).astype(np.int8)),
                    (q.BF16, synth.to_bf16_bits(g.standard_normal((65, 33)))),
                    (q.F32, g.standard_normal((3, 129)).astype(np.float32))):
        W = dev(arr)
        out = torch.empty((arr.shape[1], arr.shape[0]), dtype=W.dtype, device="cuda")
        q.qsvd_pack_weight(W, dt, arr.shape[0], arr.shape[1], out)
        torch.cuda.synchronize()
        if dt == q.BF16:
            assert np.array_equal(bf16_bits(out), arr.T)
        else:
            assert np.array_equal(out.cpu().numpy(), arr.T)

"""Helpers for the GPU parity tests: host <-> device copies and one-call wrappers
around the C ABI (through the Python binding)."""
from __future__ import annotations

import math
import sys

import numpy as np

import rank_latent_attention_amd as q

DEV = "cuda"


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray):
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


def host(t) -> np.ndarray:
    """device tensor -> numpy (bf16 -> float64 values; float32 -> float64)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    if t.dtype == torch.float32:
        return t.cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=dtype, device=DEV)


def workspace(nbytes: int):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=DEV)


def decode(qv, q_dtype, C, c_dtype, Wk, Wv, wu_dtype, b, L, r, heads, d, scale, *,
           c_scales=None, c_group=0, wsk=None, wsv=None, splits=0, o_dtype=None):
    """Run qsvd_decode_attn on device tensors; returns the output tensor."""
    import torch
    if o_dtype is None:
        o_dtype = q.F32 if c_dtype == q.F32 else q.BF16
    O = empty((b, heads, d), torch.float32 if o_dtype == q.F32 else torch.bfloat16)
    nbytes = q.qsvd_decode_workspace_bytes(b, L, r, heads, d, c_dtype, splits)
    assert nbytes > 0
    ws = workspace(nbytes)
    q.qsvd_decode_attn(qv, q_dtype, C, c_dtype, c_scales, c_group, Wk, Wv, wu_dtype, wsk, wsv,
                       b, L, r, heads, d, scale, splits, O, o_dtype, ws)
    torch.cuda.synchronize()
    return O


def decode_case_on_gpu(cs, splits=0, o_dtype=None, q_override=None):
    """Decode a synth.DecodeCase (float32 or bf16 storage) on the GPU."""
    dt = q.F32 if cs.dtype == "f32" else q.BF16
    qv = dev(cs.q if q_override is None else q_override)
    O = decode(qv, dt, dev(cs.C), dt, dev(cs.Wu_k), dev(cs.Wu_v), dt, cs.b, cs.L, cs.r, cs.heads,
               cs.d, cs.softmax_scale, splits=splits, o_dtype=o_dtype)
    return host(O)


def values(cs_array, dtype: str) -> np.ndarray:
    """Exact float64 values of a stored input (float32 or bf16 bits)."""
    import oracle
    if dtype == "bf16":
        return oracle.bf16_decode(cs_array)
    return np.asarray(cs_array, np.float64)


def check_rows(got, ref, tol: float, label: str = "", row_tol: float | None = None) -> float:
    """Assert the whole-output relative L2 error and the error of every
    (sequence, head) row are within tol.

    A single wrong row barely moves the whole-output norm (one of b * heads
    rows), so each row is held to the bound on its own.  A row is judged
    against max(its own norm, a quarter of the RMS row norm), so that a row
    whose reference nearly cancels (a near-uniform average of values) is not
    held to a relative bound on a vanishing norm.  Returns the worst row error.
    """
    import oracle
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    whole = oracle.rel_l2(got, ref)
    rows_g = got.reshape(-1, got.shape[-1])
    rows_r = ref.reshape(-1, ref.shape[-1])
    norms = np.linalg.norm(rows_r, axis=1)
    floor = 0.25 * math.sqrt(float(np.mean(norms ** 2)))
    errs = np.linalg.norm(rows_g - rows_r, axis=1) / np.maximum(norms, max(floor, 1e-300))
    worst = int(np.argmax(errs))
    say(f"  {label} rel-L2 {whole:.2e}, worst row {worst} {errs[worst]:.2e}")
    assert whole <= tol, f"{label}: whole-output rel-L2 {whole:.3e} > {tol}"
    rt = tol if row_tol is None else row_tol
    assert errs[worst] <= rt, f"{label}: row {worst} (sequence {worst // got.shape[-2] if got.ndim > 2 else 0}) rel-L2 {errs[worst]:.3e} > {rt}"
    return float(errs[worst])

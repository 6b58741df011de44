"""qsvd_decode_attn_noalloc (no workspace argument, library-owned scratch)
against qsvd_decode_attn (caller workspace) through the C ABI.

The two entry points run the same kernels on the same plan, so their outputs
must agree bitwise.  Two calls in a row, the second with a smaller batch and
cache, check that the shared scratch needs no clearing between calls; the
first output is also held to the oracle's tolerance.  A shape whose plan
exceeds the 64 MiB scratch is rejected with QSVD_ERR_WORKSPACE.
"""
import math

import numpy as np
import pytest

import oracle
import synth
from gpu_util import decode, dev, empty, host, say

import rank_latent_attention_amd as q

pytestmark = pytest.mark.gpu


def _pair(cs, o_dtype):
    import torch
    ref = decode(dev(cs.q), q.BF16, dev(cs.C), q.BF16, dev(cs.Wu_k), dev(cs.Wu_v), q.BF16, cs.b, cs.L,
                 cs.r, cs.heads, cs.d, cs.softmax_scale, o_dtype=o_dtype)
    O = empty((cs.b, cs.heads, cs.d), torch.float32 if o_dtype == q.F32 else torch.bfloat16)
    q.qsvd_decode_attn_noalloc(dev(cs.q), q.BF16, dev(cs.C), q.BF16, None, 0, dev(cs.Wu_k), dev(cs.Wu_v),
                               q.BF16, None, None, cs.b, cs.L, cs.r, cs.heads, cs.d, cs.softmax_scale, 0,
                               O, o_dtype)
    torch.cuda.synchronize()
    return host(O), host(ref)


def test_noalloc_matches_workspace_entry_point():
    say("case: no-alloc decode, E=2048 16x128 r=1536 b=4 L=3000, then E=1024 8x128 r=512 b=2 L=333")
    big = synth.decode_case(2048, 16, 128, 1536, 4, 3000, dtype="bf16", hadamard=128, seed=61)
    got, ref = _pair(big, q.BF16)
    assert np.array_equal(got, ref)
    want = oracle.attend_explicit(oracle.bf16_decode(big.q), oracle.bf16_decode(big.C),
                                  oracle.bf16_decode(big.Wu_k), oracle.bf16_decode(big.Wu_v), big.heads,
                                  big.d, big.softmax_scale)
    err = oracle.rel_l2(got, want)
    say(f"  first call: bitwise equal, rel-L2 vs oracle {err:.2e}")
    assert err <= 2e-2
    small = synth.decode_case(1024, 8, 128, 512, 2, 333, dtype="bf16", hadamard=128, seed=62)
    got2, ref2 = _pair(small, q.F32)
    assert np.array_equal(got2, ref2)
    say("  second, smaller call: bitwise equal")


def test_noalloc_rejects_a_plan_beyond_the_scratch():
    import torch
    b, L, r, heads, d, splits = 16, 65536, 1536, 32, 128, 64   # ~100 MB of split partials
    assert q.qsvd_decode_workspace_bytes(b, L, r, heads, d, q.BF16, splits) > (64 << 20)
    t = torch.empty(16, dtype=torch.bfloat16, device="cuda")   # rejected before any launch
    with pytest.raises(q.QsvdError) as e:
        q.qsvd_decode_attn_noalloc(t, q.BF16, t, q.BF16, None, 0, t, t, q.BF16, None, None, b, L, r, heads,
                                   d, 1 / math.sqrt(d), splits, t, q.BF16)
    assert e.value.status == -3 and "scratch" in str(e.value)

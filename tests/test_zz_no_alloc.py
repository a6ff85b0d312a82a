"""The allocation-free decode attention entry point against the one that
takes a workspace, through the C ABI.

kvpop_decode_attend_noalloc keeps the split partial states in the
library's fixed device array instead of a caller workspace (for callers
that cannot allocate).  Two calls in a row, the second on a smaller input
(so the array holds the first call's partials when the second starts), must
each give o and lse equal bit for bit to kvpop_decode_attend's, and within
the decode tolerance of the oracle (o |d| <= 1e-5 + 2e-3 |ref| for fp32
output, + 2^-8 |ref| for bf16; lse |d| <= 1e-4).  A shape whose partials
would not fit the array is refused before any launch.
"""
import pytest
import torch

import oracle
import synth
from gpu_util import O_ATOL, O_RTOL, assert_close, ensure_built, f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kv():
    return ensure_built()


def _case(B, Hq, Hkv, n, D, seed):
    kc = synth.bf16(synth.normal((B, Hkv, n, D), seed, std=0.5))
    vc = synth.bf16(synth.normal((B, Hkv, n, D), seed + 1))
    g = torch.Generator().manual_seed(seed + 2)
    sp = torch.arange(n, dtype=torch.int32).expand(B, Hkv, n).contiguous()
    sp = torch.where(torch.rand((B, Hkv, n), generator=g) < 0.1, torch.full_like(sp, -1), sp)
    q = synth.bf16(synth.normal((B, Hq, D), seed + 3, std=0.5))
    return q, kc, vc, sp


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_decode_matches_workspace_entry_point(kv, out_dtype):
    # few rows, so both launches split their slots and use the array;
    # the second input is smaller than the first
    for i, (B, Hq, Hkv, n, D) in enumerate([(1, 32, 8, 4096, 128), (1, 8, 2, 1000, 64)]):
        need = kv.workspace_bytes(kv.OP_DECODE, kv.dims(B, Hq, Hkv, n, D))
        assert 0 < need <= kv.DECODE_NOALLOC_SCRATCH_BYTES, need
        q, kc, vc, sp = (t.cuda() for t in _case(B, Hq, Hkv, n, D, seed=40 + i))
        print(f"noalloc decode call {i}: B={B} Hq={Hq} Hkv={Hkv} n={n} D={D}", flush=True)
        o1, l1 = kv.decode_attend(q, kc, vc, sp, out_dtype=out_dtype)
        o2, l2 = kv.decode_attend_noalloc(q, kc, vc, sp, out_dtype=out_dtype)
        torch.cuda.synchronize()
        assert torch.equal(o1.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           o2.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32)), i
        assert torch.equal(l1.view(torch.int32), l2.view(torch.int32)), i
        oo, ol = oracle.decode_attend(f32(q), f32(kc), f32(vc), sp.cpu().numpy())
        extra = 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0
        assert_close(f32(o2), oo, O_ATOL, O_RTOL + extra, f"call {i}: o")
        assert_close(f32(l2), ol, 1e-4, 0.0, f"call {i}: lse")


def test_noalloc_decode_refuses_oversized_partials(kv):
    """A single 128-head group over 200000 slots splits into more partials
    than the array holds: the call returns 'workspace too small' and writes
    nothing."""
    B, Hq, Hkv, n, D = 1, 128, 1, 200000, 128
    need = kv.workspace_bytes(kv.OP_DECODE, kv.dims(B, Hq, Hkv, n, D))
    assert need > kv.DECODE_NOALLOC_SCRATCH_BYTES, need
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((B, Hkv, n, D), dtype=torch.bfloat16, device="cuda")
    sp = torch.zeros((B, Hkv, n), dtype=torch.int32, device="cuda")
    o = torch.full((B, Hq, D), 3.0, device="cuda")
    with pytest.raises(kv.KvpopError) as e:
        kv.decode_attend_noalloc(q, kc, kc, sp, out=o)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert bool((o == 3.0).all())

"""CPU-side checks of the C ABI: the library loads, exports every function
include/kvpop.h declares, and rejects invalid arguments on the host before
any launch (no GPU is touched: every call below fails validation).
"""
import ctypes
import os
import re

import pytest

import future_attention_scoring_kvpop_amd as kv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvpop.h")
P = ctypes.c_void_p
GOOD = P(0x10000)  # aligned, never dereferenced: validation fails first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(kv.LIB_PATH):
        from future_attention_scoring_kvpop_amd import build
        build.build()
    return kv.lib()


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kvpop_[a-z_]+)\s*\(", text))


def test_exports_match_header(lib):
    names = declared()
    assert names == set(kv.EXPORTS), names ^ set(kv.EXPORTS)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvpop_abi_version() == 3
    for s in range(5):
        assert lib.kvpop_status_string(s)


def test_dims_validation(lib):
    def fwd(d):
        return lib.kvpop_fwd_lse(ctypes.byref(d), GOOD, GOOD, None, GOOD, None, 0, None, 0, None)

    assert lib.kvpop_fwd_lse(None, GOOD, GOOD, None, GOOD, None, 0, None, 0, None) == 1
    assert fwd(kv.dims(0, 32, 8, 4096, 128)) == 1
    assert fwd(kv.dims(1, 32, 8, 0, 128)) == 1
    assert fwd(kv.dims(1, 30, 8, 4096, 128)) == 1   # Hq % Hkv
    assert fwd(kv.dims(1, 24, 8, 4096, 128)) == 2   # group of 3
    assert fwd(kv.dims(1, 32, 8, 4096, 96)) == 2    # head dim
    assert fwd(kv.dims(1, 32, 8, 4096, 128, float("nan"))) == 1
    d = kv.dims(1, 2, 1, 4096, 128)
    need = kv.workspace_bytes(kv.OP_FWD_LSE, d)
    assert need > 0  # few row blocks: long causal rows are split
    assert lib.kvpop_fwd_lse(ctypes.byref(d), None, GOOD, None, GOOD, None, 0, GOOD, need, None) == 1
    assert lib.kvpop_fwd_lse(ctypes.byref(d), P(0x10008), GOOD, None, GOOD, None, 0, GOOD, need, None) == 1  # misaligned
    assert lib.kvpop_fwd_lse(ctypes.byref(d), GOOD, GOOD, None, GOOD, None, 0, None, need, None) == 1
    assert lib.kvpop_fwd_lse(ctypes.byref(d), GOOD, GOOD, None, GOOD, None, 0, GOOD, need - 8, None) == 3
    for big in (kv.dims(1, 32, 8, 32768, 128), kv.dims(1, 32, 8, 4096, 128)):
        assert kv.workspace_bytes(kv.OP_FWD_LSE, big) == 0  # enough row blocks: no split
    # the attention output: v and o together, 16-byte aligned, a valid type,
    # and room for V^T (64-key padded rows)
    d = kv.dims(1, 32, 8, 100, 128)
    need = kv.workspace_bytes(kv.OP_FWD_ATTN, d)
    assert need == 1 * 8 * 128 * 128 * 2

    def att(v=GOOD, o=GOOD, o_dtype=0, ws=GOOD, nbytes=need):
        return lib.kvpop_fwd_lse(ctypes.byref(d), GOOD, GOOD, v, GOOD, o, o_dtype, ws, nbytes, None)

    assert att(v=None) == 1
    assert att(o=None) == 1
    assert att(o_dtype=2) == 1
    assert att(o=P(0x10008)) == 1
    assert att(ws=None) == 1
    assert att(ws=P(0x10010)) == 1  # V^T workspace: 256-byte aligned
    assert att(nbytes=need - 1) == 3
    sp = lib.kvpop_fwd_lse_sparse
    assert sp(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, 64, GOOD, None, 0, GOOD, need, None) == 1
    assert sp(ctypes.byref(d), GOOD, GOOD, GOOD, GOOD, 64, GOOD, GOOD, 0, GOOD, need - 1, None) == 3


def test_target_validation(lib):
    d = kv.dims(1, 32, 8, 4096, 128)
    need = kv.workspace_bytes(kv.OP_FUTURE_TARGET, d, 128)
    assert need > 0

    def call(window=128, agg=0, ws=GOOD, nbytes=need, mass=GOOD):
        return lib.kvpop_future_attn_target(ctypes.byref(d), GOOD, GOOD, GOOD, window, -1, agg, 0,
                                            mass, None, ws, nbytes, None)

    assert call(window=-1) == 1
    assert call(agg=3) == 1
    assert call(mass=None) == 1
    assert call(ws=None) == 1
    assert call(ws=P(0x10010)) == 1           # workspace must be 256-byte aligned
    assert call(nbytes=need - 4) == 3
    # one group's Q rows are addressed by 32-bit offsets: G * S * D * 2 < 2 GiB
    big = kv.dims(1, 64, 8, 1 << 20, 128)
    assert lib.kvpop_future_attn_target(ctypes.byref(big), GOOD, GOOD, GOOD, 128, -1, 0, 0,
                                        GOOD, None, GOOD, 1 << 40, None) == 2


def test_select_validation(lib):
    def call(B=1, H=8, S=4096, D=128, s=4, w=128, budget=1024, scores=GOOD, k=None, v=None,
             kc=None, vc=None, pos=GOOD):
        return lib.kvpop_evict_select(B, H, S, D, s, w, budget, scores, k, v, pos, None, kc, vc, None)

    assert call(budget=100) == 1              # budget < s + w
    assert call(s=-1) == 1
    assert call(w=-1) == 1
    assert call(scores=None) == 1
    assert call(pos=None) == 1
    assert call(k=GOOD) == 1                  # k without v
    assert call(k=GOOD, v=GOOD) == 1          # no cache outputs
    assert call(kc=GOOD, vc=GOOD) == 1        # cache outputs without inputs
    assert call(k=GOOD, v=GOOD, kc=GOOD, vc=GOOD, D=96) == 2


def test_decode_validation(lib):
    # 64 x 8 (b, KV head) rows fill the device alone: no split, no workspace
    assert kv.workspace_bytes(kv.OP_DECODE, kv.dims(64, 32, 8, 4096, 128)) == 0
    d = kv.dims(1, 32, 8, 4096, 128)  # 8 rows: slots are split, partials need room
    need = kv.workspace_bytes(kv.OP_DECODE, d)
    assert need > 0

    def call(o_dtype=0, ws=GOOD, nbytes=need, sp=GOOD):
        return lib.kvpop_decode_attend(ctypes.byref(d), GOOD, GOOD, GOOD, sp, GOOD, o_dtype, None,
                                       ws, nbytes, None)

    assert call(o_dtype=2) == 1
    assert call(sp=None) == 1
    assert call(ws=None) == 1
    assert call(nbytes=need - 1) == 3


def test_decode_noalloc_validation(lib):
    """The allocation-free decode entry point: the same argument checks as
    kvpop_decode_attend, and a refusal (workspace too small) for shapes whose
    split partials exceed the library's fixed array."""
    d = kv.dims(1, 32, 8, 4096, 128)
    assert 0 < kv.workspace_bytes(kv.OP_DECODE, d) <= kv.DECODE_NOALLOC_SCRATCH_BYTES

    def call(dd=d, o_dtype=0, sp=GOOD, q=GOOD):
        return lib.kvpop_decode_attend_noalloc(ctypes.byref(dd) if dd is not None else None, q,
                                               GOOD, GOOD, sp, GOOD, o_dtype, None, None)

    assert call(dd=None) == 1
    assert call(o_dtype=2) == 1
    assert call(sp=None) == 1
    assert call(q=P(0x10008)) == 1  # misaligned
    big = kv.dims(1, 128, 1, 200000, 128)
    assert kv.workspace_bytes(kv.OP_DECODE, big) > kv.DECODE_NOALLOC_SCRATCH_BYTES
    assert call(dd=big) == 3


def test_mlp_and_cache_step_validation(lib):
    assert lib.kvpop_score_mlp(1, 8, 10, 128, 65, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None) == 2
    assert lib.kvpop_score_mlp(1, 8, 10, 96, 64, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None) == 2
    assert lib.kvpop_score_mlp(1, 8, 10, 128, 64, None, GOOD, GOOD, GOOD, GOOD, GOOD, None) == 1

    def step(window=256, delay=16, budget=4096, w1=None, sr=GOOD, hidden=64, pos=40000):
        return lib.kvpop_cache_step(64, 8, 128, 4, window, budget, delay, pos, GOOD, GOOD, w1, GOOD,
                                    GOOD, GOOD, hidden, sr, GOOD, GOOD, GOOD, GOOD, None)

    assert step(window=0) == 1
    assert step(delay=256) == 1               # delay must stay inside the window
    assert step(delay=-1) == 1
    assert step(budget=200) == 1
    assert step(pos=-1) == 1
    assert step(w1=GOOD) == 1                 # both an MLP and given scores
    # neither is valid (no delayed scoring): it passes validation and would launch
    assert step(w1=GOOD, sr=None, hidden=65) == 2


def test_decode_step_validation(lib):
    d = kv.dims(64, 32, 8, 4096, 128)

    def call(d=d, window=256, delay=16, w1=None, sr=GOOD, hidden=64, o_dtype=0, pos=40000, q=GOOD):
        return lib.kvpop_decode_step(ctypes.byref(d), 4, window, delay, pos, GOOD, GOOD, w1, GOOD,
                                     GOOD, GOOD, hidden, sr, GOOD, GOOD, GOOD, GOOD, q, GOOD,
                                     o_dtype, None, None, 0, None)

    assert call(window=0) == 1
    assert call(delay=256) == 1
    assert call(pos=-1) == 1
    assert call(q=None) == 1
    assert call(o_dtype=2) == 1
    assert call(w1=GOOD) == 1                 # both an MLP and given scores
    assert call(w1=GOOD, sr=None, hidden=65) == 2
    assert call(d=kv.dims(64, 32, 8, 200, 128)) == 1  # budget < s + w
    assert call(d=kv.dims(64, 32, 8, 4096, 96)) == 2  # head dim


def test_python_binding_rejects_host_tensors():
    import torch
    with pytest.raises(ValueError):
        kv.fwd_lse(torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16),
                   torch.zeros(1, 1, 4, 64, dtype=torch.bfloat16))


def test_running_topk_and_sparse_lse_validation(lib):
    # every call below fails its host-side checks before any launch
    rt = lib.kvpop_running_topk
    assert rt(1, 8, 4096, 4, 128, 100, GOOD, None, GOOD, None, None, 0, None) == 1   # budget < s + w
    assert rt(1, 8, 4096, -1, 128, 1024, GOOD, None, GOOD, None, None, 0, None) == 1
    assert rt(1, 8, 4096, 4, -2, 1024, GOOD, None, GOOD, None, None, 0, None) == 1
    assert rt(0, 8, 4096, 4, 128, 1024, GOOD, None, GOOD, None, None, 0, None) == 1
    assert rt(1, 8, 4096, 4, 128, 1024, None, None, GOOD, None, None, 0, None) == 1
    assert rt(1, 8, 4096, 4, 128, 1024, GOOD, None, None, None, None, 0, None) == 1
    assert rt(1, 8, 4096, 4, 128, 1024, P(0x10002), None, GOOD, None, None, 0, None) == 1  # misaligned
    assert rt(1, 8, 4096, 4, 128, 1024, GOOD, P(0x10001), GOOD, None, None, 0, None) == 1
    assert rt(1, 8, (1 << 24) + 1, 4, 128, 1024, GOOD, None, GOOD, None, None, 0, None) == 2  # longest row 2^24
    # rows up to 8192 tokens need no workspace; longer rows do
    wsb = lib.kvpop_running_topk_workspace_bytes
    assert wsb(1, 8, 8192, 4) == 0 and wsb(1, 8, 4096, 4) == 0
    need = wsb(1, 8, 16384, 4)
    assert need >= 8 * 16384 * 4 * 8 and wsb(2, 8, 16384, 4) == 2 * need
    assert wsb(1, 8, (1 << 24) + 1, 4) == 0 and wsb(0, 8, 16384, 4) == 0
    assert rt(1, 8, 16384, 4, 128, 1024, GOOD, None, GOOD, None, None, 0, None) == 1     # no workspace
    assert rt(1, 8, 16384, 4, 128, 1024, GOOD, None, GOOD, None, P(0x10008), need, None) == 1  # misaligned
    assert rt(1, 8, 16384, 4, 128, 1024, GOOD, None, GOOD, None, GOOD, need - 16, None) == 3   # too small
    sp = lib.kvpop_fwd_lse_sparse
    d = kv.dims(1, 32, 8, 4096, 128)
    assert sp(ctypes.byref(d), GOOD, GOOD, None, None, 0, GOOD, None, 0, None, 0, None) == 1     # no mask
    assert sp(ctypes.byref(d), GOOD, GOOD, None, P(0x10002), 0, GOOD, None, 0, None, 0, None) == 1
    assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, -1, GOOD, None, 0, None, 0, None) == 1    # budget < 0
    assert sp(None, GOOD, GOOD, None, GOOD, 0, GOOD, None, 0, None, 0, None) == 1
    d = kv.dims(1, 32, 8, 4096, 96)
    assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, 0, GOOD, None, 0, None, 0, None) == 2      # D = 96
    d = kv.dims(1, 32, 8, 4096, 128)
    need = lib.kvpop_workspace_bytes(3, ctypes.byref(d), 0)
    assert need == lib.kvpop_workspace_bytes(2, ctypes.byref(d), 0)
    if need:
        assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, 0, GOOD, None, 0, GOOD, need - 16, None) == 3
    # with a budget: a header per block of 32 queries (8 heads x 128 blocks),
    # then 1024 + 32 listed keys per block
    need = lib.kvpop_workspace_bytes(3, ctypes.byref(d), 1024)
    assert need == 8 * 128 * 8 + 8 * 128 * 1088 * 4
    assert lib.kvpop_workspace_bytes(3, ctypes.byref(d), -1) == 0
    assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, 1024, GOOD, None, 0, None, 0, None) == 1   # no workspace
    assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, 1024, GOOD, None, 0, P(0x10010), need, None) == 1  # 256 B
    assert sp(ctypes.byref(d), GOOD, GOOD, None, GOOD, 1024, GOOD, None, 0, GOOD, need - 1, None) == 3


def test_mlstm_step_validation(lib):
    def weights(feat=32, vdim=64, missing=None):
        ptrs = {n: 0x10000 for n in ("wk", "wr", "wv", "wi", "bi", "wf", "bf", "wo", "bo")}
        if missing:
            ptrs[missing] = None
        return kv.MlstmWeights(feat, vdim, *[ptrs[n] for n in ("wk", "wr", "wv", "wi", "bi", "wf",
                                                               "bf", "wo", "bo")])

    def call(w=None, D=128, window=256, budget=4096, pos=40000, state=GOOD, ss=GOOD, kc=GOOD):
        w = w if w is not None else weights()
        return lib.kvpop_mlstm_step(64, 8, D, 4, window, budget, pos, GOOD, GOOD, kc, kc,
                                    ctypes.byref(w), state, ss, None)

    assert call(window=0) == 1
    assert call(budget=200) == 1
    assert call(pos=-1) == 1
    assert call(D=96) == 2
    assert call(w=weights(feat=16)) == 2
    assert call(w=weights(vdim=32)) == 2
    assert call(w=weights(missing="wo")) == 1
    assert call(state=None) == 1
    assert call(state=P(0x10004)) == 1        # state rows need 16-byte alignment
    assert call(kc=None) == 1                 # a readout needs the caches
    assert lib.kvpop_mlstm_step(64, 8, 128, 4, 256, 4096, 0, GOOD, GOOD, GOOD, GOOD, None, GOOD,
                                GOOD, None) == 1

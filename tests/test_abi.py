"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, rejects bad host arguments before touching the device, and its
host-only cost-table call matches the oracle bit for bit.  No device compute
is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libspecverify.h")

sv = pytest.importorskip("adaptive_draft_verification_amd",
                         reason="libspecverify.so not built (python adaptive_draft_verification_amd/build.py)")

FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first
WS43 = sv.sv_verify_workspace_bytes(4, 3)  # the verify calls below: 4 requests, k_max 3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sv_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert "sv_verify" in names and "sv_budget_select" in names and "sv_pack_varlen" in names
    lib = ctypes.CDLL(sv.LIB_PATH)
    for name in names:
        assert hasattr(lib, name), name
    assert sorted(sv.EXPORTED) == names


def test_status_strings():
    for s in range(9):
        assert sv.sv_status_str(s)
    assert sv.sv_status_str(99) == "unknown status"


def test_workspace_sizes():
    # 8 parts per row: a 16-byte record per part of each of the 2K+1 rows, and an
    # 8-byte feature record per part of each of the K draft rows
    assert sv.sv_verify_workspace_bytes(256, 7) == 256 * 15 * 8 * 16 + 256 * 7 * 8 * 8
    assert sv.sv_verify_workspace_bytes(-1, 7) == 0
    assert sv.sv_verify_workspace_bytes(1, 65) == 0
    assert sv.sv_verify_workspace_bytes(sv.SV_MAX_VERIFY_SLOTS // 15 + 1, 7) == 0
    assert sv.sv_verify_workspace_bytes(sv.SV_MAX_VERIFY_SLOTS // 15, 7) > 0
    # a 16-byte header, then an int32 rank and an fp32 survival per slot
    assert sv.sv_budget_workspace_bytes(256, 7) == 16 + 1792 * 8
    assert sv.sv_budget_workspace_bytes(8192, 1) == 16 + 8192 * 8
    assert sv.sv_budget_workspace_bytes(3, 0) == 16
    assert sv.sv_budget_workspace_bytes(0, 5) == 0
    assert sv.sv_budget_workspace_bytes(2048, 5) == 0   # over the slot limit: call is refused
    assert sv.sv_budget_workspace_bytes(1, 65) == 0     # over the draft limit: call is refused


@pytest.mark.parametrize("granule", [1, 2, 16])
def test_cost_table_prepare_matches_oracle(granule):
    rng = np.random.default_rng(granule)
    raw = (1 + rng.uniform(0, 1, 4097) * np.linspace(1, 5, 4097)).astype(np.float32)
    out_len = 4097 - granule
    got = sv.sv_cost_table_prepare(raw, granule, out_len)
    want = oracle.cost_table_prepare(raw, granule, out_len)
    np.testing.assert_array_equal(got, want)


def test_cost_table_prepare_errors():
    raw = np.ones(10, dtype=np.float32)
    with pytest.raises(sv.SvError) as e:
        sv.sv_cost_table_prepare(raw, 16, 10)
    assert e.value.status == sv.SV_ERR_SHAPE
    bad = raw.copy()
    bad[4] = np.inf
    with pytest.raises(sv.SvError) as e:
        sv.sv_cost_table_prepare(bad, 1, 5)
    assert e.value.status == sv.SV_ERR_VALUE
    with pytest.raises(sv.SvError) as e:
        sv.sv_cost_table_prepare(raw, 0, 5)
    assert e.value.status == sv.SV_ERR_SHAPE
    lib = sv._lib
    assert lib.sv_cost_table_prepare(None, 10, 1, FAKE, 5) == sv.SV_ERR_NULL


def budget(**kw):
    args = dict(conf=FAKE, draft_len=FAKE, n_req=4, k_max=3, cost=FAKE, cost_len=17, t_base=4,
                n_bonus=4, kept=FAKE, budget=FAKE, survival=None, dev_error=None, ws=None,
                ws_bytes=0, stream=None)
    args.update(kw)
    return sv._lib.sv_budget_select(*args.values())


def allocate(**kw):
    args = dict(conf=FAKE, draft_len=FAKE, n_req=4, k_max=3, budget_in=FAKE, kept=FAKE,
                budget_used=None, survival=None, dev_error=None, ws=FAKE,
                ws_bytes=sv.sv_budget_workspace_bytes(4, 3), stream=None)
    args.update(kw)
    return sv._lib.sv_budget_allocate(*args.values())


def test_budget_allocate_host_validation():
    assert allocate(n_req=-1) == sv.SV_ERR_SHAPE
    assert allocate(k_max=-1) == sv.SV_ERR_SHAPE
    assert allocate(n_req=2048, k_max=5) == sv.SV_ERR_SHAPE   # > 8192 slots
    assert allocate(n_req=8193, k_max=0) == sv.SV_ERR_SHAPE   # > 8192 requests
    assert allocate(n_req=1, k_max=65) == sv.SV_ERR_SHAPE     # > 64 drafts
    for key in ("budget_in", "conf", "draft_len", "kept"):
        assert allocate(**{key: None}) == sv.SV_ERR_NULL, key
    assert allocate(ws=None) == sv.SV_ERR_WORKSPACE
    assert allocate(ws_bytes=sv.sv_budget_workspace_bytes(4, 3) - 1) == sv.SV_ERR_WORKSPACE


def select_pack(**kw):
    args = dict(conf=FAKE, draft_len=FAKE, n_req=4, k_max=3, cost=FAKE, cost_len=17, t_base=4,
                n_bonus=4, last_token=FAKE, draft_tokens=FAKE, kept=FAKE, budget=FAKE,
                survival=None, cu_rows=FAKE, row_req=FAKE, row_pos=FAKE, packed=FAKE,
                dev_error=None, ws=FAKE, ws_bytes=sv.sv_budget_workspace_bytes(4, 3), stream=None)
    args.update(kw)
    return sv._lib.sv_budget_select_pack(*args.values())


def allocate_pack(**kw):
    args = dict(conf=FAKE, draft_len=FAKE, n_req=4, k_max=3, budget_in=FAKE, last_token=FAKE,
                draft_tokens=FAKE, kept=FAKE, budget_used=None, survival=None, cu_rows=FAKE,
                row_req=FAKE, row_pos=FAKE, packed=FAKE, dev_error=None, ws=FAKE,
                ws_bytes=sv.sv_budget_workspace_bytes(4, 3), stream=None)
    args.update(kw)
    return sv._lib.sv_budget_allocate_pack(*args.values())


def test_fused_budget_pack_host_validation():
    for call, own in ((select_pack, ("cost", "budget")), (allocate_pack, ("budget_in",))):
        for key in own + ("conf", "draft_len", "kept", "last_token", "draft_tokens", "cu_rows",
                          "row_req", "row_pos", "packed"):
            assert call(**{key: None}) == sv.SV_ERR_NULL, (call.__name__, key)
        assert call(n_req=-1) == sv.SV_ERR_SHAPE
        assert call(n_req=2048, k_max=5) == sv.SV_ERR_SHAPE
        assert call(n_req=1, k_max=65) == sv.SV_ERR_SHAPE
        assert call(ws=None) == sv.SV_ERR_WORKSPACE
    assert select_pack(cost_len=16) == sv.SV_ERR_SHAPE
    assert select_pack(t_base=-1) == sv.SV_ERR_VALUE


def test_budget_select_host_validation():
    assert budget(cost_len=16) == sv.SV_ERR_SHAPE          # needs t_base + n*k + 1
    assert budget(n_req=-1) == sv.SV_ERR_SHAPE
    assert budget(k_max=-2) == sv.SV_ERR_SHAPE
    assert budget(n_req=2048, k_max=5, cost_len=20000) == sv.SV_ERR_SHAPE  # > 8192 slots
    assert budget(n_req=8193, k_max=0, cost_len=20000) == sv.SV_ERR_SHAPE  # > 8192 requests
    assert budget(n_req=1, k_max=65, cost_len=200) == sv.SV_ERR_SHAPE      # > 64 drafts
    assert budget(t_base=-1) == sv.SV_ERR_VALUE
    assert budget(n_bonus=-1) == sv.SV_ERR_VALUE
    assert budget(cost=None) == sv.SV_ERR_NULL
    assert budget(budget=None) == sv.SV_ERR_NULL
    assert budget(conf=None) == sv.SV_ERR_NULL
    assert budget(kept=None) == sv.SV_ERR_NULL
    need = sv.sv_budget_workspace_bytes(4, 3)
    assert need > 0
    assert budget() == sv.SV_ERR_WORKSPACE
    assert budget(ws=FAKE, ws_bytes=need - 1) == sv.SV_ERR_WORKSPACE


def uniform_k(**kw):
    args = dict(conf=FAKE, draft_len=FAKE, n_req=4, k_max=3, cost=FAKE, cost_len=17, t_base=4,
                n_bonus=4, kept=FAKE, k_out=FAKE, scores=None, dev_error=None, stream=None)
    args.update(kw)
    return sv._lib.sv_uniform_k_select(*args.values())


def test_uniform_k_host_validation():
    assert uniform_k(cost_len=16) == sv.SV_ERR_SHAPE          # needs t_base + n*k + 1
    assert uniform_k(n_req=-1) == sv.SV_ERR_SHAPE
    assert uniform_k(k_max=65, cost_len=300) == sv.SV_ERR_SHAPE
    assert uniform_k(n_req=2048, k_max=5, cost_len=20000) == sv.SV_ERR_SHAPE
    assert uniform_k(t_base=-1) == sv.SV_ERR_VALUE
    assert uniform_k(n_bonus=-1) == sv.SV_ERR_VALUE
    for key in ("conf", "draft_len", "cost", "kept", "k_out"):
        assert uniform_k(**{key: None}) == sv.SV_ERR_NULL, key
    # no requests: nothing needs the request arrays
    assert uniform_k(n_req=0, conf=None, draft_len=None, kept=None, cost_len=5,
                     k_out=None) == sv.SV_ERR_NULL  # k_out is always written


def pack(**kw):
    args = dict(kept=FAKE, last_token=FAKE, draft_tokens=FAKE, n_req=4, k_max=3, cu_rows=FAKE,
                row_req=FAKE, row_pos=FAKE, packed=FAKE, dev_error=None, stream=None)
    args.update(kw)
    return sv._lib.sv_pack_varlen(*args.values())


def test_pack_host_validation():
    assert pack(n_req=-1) == sv.SV_ERR_SHAPE
    assert pack(k_max=-1) == sv.SV_ERR_SHAPE
    assert pack(n_req=2**30, k_max=7) == sv.SV_ERR_SHAPE
    for key in ("kept", "last_token", "draft_tokens", "cu_rows", "row_req", "row_pos", "packed"):
        assert pack(**{key: None}) == sv.SV_ERR_NULL, key


def verify(**kw):
    args = dict(target=FAKE, target_ld=32, target_rows=16, draft=FAKE, draft_ld=32,
                dtype=sv.SV_F32, vocab=32, draft_tokens=FAKE, cu_rows=FAKE, n_req=4, k_max=3,
                mode=sv.SV_STOCHASTIC, temperature=1.0, seed=0, step=0, out_tokens=FAKE,
                out_accepted=FAKE, out_p=None, out_q=None, out_resid=None, out_qh=None,
                out_qm=None, dev_error=None, ws=FAKE, ws_bytes=WS43, stream=None)
    args.update(kw)
    return sv._lib.sv_verify(*args.values())


def test_verify_host_validation():
    assert verify(dtype=7) == sv.SV_ERR_DTYPE
    assert verify(mode=5) == sv.SV_ERR_VALUE
    assert verify(n_req=-1) == sv.SV_ERR_SHAPE
    assert verify(k_max=65) == sv.SV_ERR_SHAPE
    # the batch bound: n_req * (2 k_max + 1) row slots at most SV_MAX_VERIFY_SLOTS, so
    # that the pass-1 grid (up to 8 parts of 512 threads per slot) stays below 2^32
    # work-items; checked before the workspace, which is then sized 0
    big = sv.SV_MAX_VERIFY_SLOTS // 15
    assert verify(n_req=big + 1, k_max=7, ws_bytes=2**62) == sv.SV_ERR_SHAPE
    assert verify(n_req=2**31 - 1, k_max=64, ws_bytes=2**62) == sv.SV_ERR_SHAPE
    assert verify(n_req=big, k_max=7, ws=None) == sv.SV_ERR_WORKSPACE
    assert sv.SV_MAX_VERIFY_SLOTS * 8 * 512 < 2**32
    assert verify(vocab=0) == sv.SV_ERR_SHAPE
    assert verify(vocab=2**20 + 1, target_ld=2**21, draft_ld=2**21) == sv.SV_ERR_SHAPE
    assert verify(target_ld=31) == sv.SV_ERR_SHAPE
    assert verify(draft_ld=31) == sv.SV_ERR_SHAPE
    assert verify(target_rows=-1) == sv.SV_ERR_SHAPE
    assert verify(temperature=0.0) == sv.SV_ERR_VALUE
    assert verify(temperature=-1.0) == sv.SV_ERR_VALUE
    assert verify(temperature=float("nan")) == sv.SV_ERR_VALUE
    assert verify(temperature=float("inf")) == sv.SV_ERR_VALUE
    assert verify(temperature=1e-39) == sv.SV_ERR_VALUE
    assert verify(ws_bytes=WS43 - 1) == sv.SV_ERR_WORKSPACE
    assert verify(ws=None) == sv.SV_ERR_WORKSPACE
    for key in ("target", "cu_rows", "out_tokens", "out_accepted", "draft_tokens", "draft"):
        assert verify(**{key: None}) == sv.SV_ERR_NULL, key
    # greedy needs no draft logits, no draft stride and no temperature; it then
    # fails only on the (deliberately) missing workspace, still before any launch
    assert verify(mode=sv.SV_GREEDY, draft=None, draft_ld=0, temperature=0.0,
                  ws=None) == sv.SV_ERR_WORKSPACE
    # nothing to do: OK without touching anything
    assert verify(n_req=0, target=None, ws=None) == sv.SV_OK


def test_verify_stages_validation():
    base = dict(target=FAKE, target_ld=32, target_rows=16, draft=FAKE, draft_ld=32,
                dtype=sv.SV_F32, vocab=32, draft_tokens=FAKE, cu_rows=FAKE, n_req=4, k_max=3,
                mode=sv.SV_STOCHASTIC, temperature=1.0, seed=0, step=0, out_tokens=FAKE,
                out_accepted=FAKE, out_p=None, out_q=None, out_resid=None, out_qh=None,
                out_qm=None, dev_error=None, ws=FAKE, ws_bytes=WS43)
    for bad in (0, 4, -1):
        assert sv._lib.sv_verify_stages(*base.values(), bad, None) == sv.SV_ERR_VALUE
    base["ws"] = None
    for ok in (1, 2, 3):
        assert sv._lib.sv_verify_stages(*base.values(), ok, None) == sv.SV_ERR_WORKSPACE


def test_calibration_host_validation():
    lib = sv._lib
    assert lib.sv_accept_stats(FAKE, FAKE, -1, 3, FAKE, FAKE, FAKE, None) == sv.SV_ERR_SHAPE
    assert lib.sv_accept_stats(FAKE, FAKE, 4, 65, FAKE, FAKE, FAKE, None) == sv.SV_ERR_SHAPE
    assert lib.sv_accept_stats(FAKE, FAKE, 4, 3, FAKE, FAKE, None, None) == sv.SV_ERR_NULL
    assert lib.sv_accept_stats(None, FAKE, 4, 3, FAKE, FAKE, FAKE, None) == sv.SV_ERR_NULL
    upd = lambda th, q, acc, cu, n, k, lr: lib.sv_calibrate_update(th, q, None, None, acc, cu, n,
                                                                    k, lr, None, None)
    assert upd(FAKE, FAKE, FAKE, FAKE, 4, 65, 0.1) == sv.SV_ERR_SHAPE
    assert upd(FAKE, FAKE, FAKE, FAKE, 4, 3, -0.1) == sv.SV_ERR_VALUE
    assert lib.sv_calibrate_update(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 3, float("nan"), None,
                                   None) == sv.SV_ERR_VALUE
    assert upd(None, FAKE, FAKE, FAKE, 4, 3, 0.1) == sv.SV_ERR_NULL
    assert upd(FAKE, None, FAKE, FAKE, 4, 3, 0.1) == sv.SV_ERR_NULL
    assert upd(FAKE, FAKE, None, FAKE, 4, 3, 0.1) == sv.SV_ERR_NULL
    pred = lambda th, q, n, k, conf: lib.sv_calibrate_predict(th, q, None, None, n, k, conf, None)
    assert pred(FAKE, FAKE, 4, 65, FAKE) == sv.SV_ERR_SHAPE
    assert pred(FAKE, None, 4, 3, FAKE) == sv.SV_ERR_NULL
    assert pred(None, None, 0, 3, None) == sv.SV_OK


def test_philox_host_validation():
    assert sv._lib.sv_philox_uniforms(0, 0, -1, 3, FAKE, FAKE, None) == sv.SV_ERR_SHAPE
    assert sv._lib.sv_philox_uniforms(0, 0, 2, 3, None, FAKE, None) == sv.SV_ERR_NULL
    assert sv._lib.sv_philox_uniforms(0, 0, 0, 3, None, None, None) == sv.SV_OK


def test_binding_rejects_host_tensors():
    import torch
    conf = torch.zeros(2, 2)
    with pytest.raises(ValueError):
        sv.budget_select(conf, torch.zeros(2, dtype=torch.int32), torch.ones(9), 2, 2)


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defines = dict(re.findall(r"#define\s+(SV_\w+)\s+(\d+)", text))
    assert "SV_MAX_VERIFY_SLOTS" in defines
    for name, value in defines.items():
        if hasattr(sv, name):
            assert getattr(sv, name) == int(value), name
    # the enums: every named value, and the binding has each of them
    blocks = re.findall(r"typedef enum\s*\{(.*?)\}", text, re.S)
    enums = dict(re.findall(r"\b(SV_\w+)\s*=\s*(\d+)", " ".join(blocks)))
    assert enums["SV_ERR_DATA"] == "8" and enums["SV_BF16"] == "1"
    for name, value in enums.items():
        if not name.endswith("_"):  # range markers (every int32 a value of the type)
            assert getattr(sv, name) == int(value), name


def test_verify_noalloc_host_validation():
    """sv_verify_noalloc's checks run before any HIP call: sv_verify's own, then the
    static workspace's capacity."""
    def call(**kw):
        args = dict(target=FAKE, target_ld=32, target_rows=16, draft=FAKE, draft_ld=32,
                    dtype=sv.SV_F32, vocab=32, draft_tokens=FAKE, cu_rows=FAKE, n_req=4,
                    k_max=3, mode=sv.SV_STOCHASTIC, temperature=1.0, seed=0, step=0,
                    out_tokens=FAKE, out_accepted=FAKE, out_p=None, out_q=None, out_resid=None,
                    out_qh=None, out_qm=None, dev_error=None, stream=None)
        args.update(kw)
        return sv._lib.sv_verify_noalloc(*args.values())
    per_req = (2 * 7 + 1) * 128 + 7 * 64
    over = sv.SV_NOALLOC_WS_BYTES // per_req + 1
    assert call(n_req=over, k_max=7) == sv.SV_ERR_CAPACITY
    assert call(n_req=over - 1, k_max=7, target=None) == sv.SV_ERR_NULL  # fits: other checks
    assert call(dtype=9) == sv.SV_ERR_DTYPE
    assert call(k_max=65) == sv.SV_ERR_SHAPE
    assert call(temperature=0.0) == sv.SV_ERR_VALUE
    assert call(n_req=0, target=None) == sv.SV_OK
    assert sv.sv_status_str(sv.SV_ERR_CAPACITY)

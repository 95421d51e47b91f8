"""sv_verify_noalloc (its workspace a static per-GPU array; the call allocates
nothing) against sv_verify (the caller's workspace), through the C ABI.

Two calls in a row, the second on a smaller batch than the first (the array
keeps the first call's records), each compared with sv_verify output for
output (the same kernels: identical bits) and with the oracle under the parity
rules; then a third, larger call again.  A batch beyond the array's size is
refused before anything is launched.  Last, one call recorded in a HIP graph
(the first call on the GPU, made eagerly, looks up the array's address; the
recorded call only launches kernels) replays over new inputs in its buffers,
each replay equal to eager sv_verify bit for bit."""

import numpy as np
import pytest
import torch

import adaptive_draft_verification_amd as sv
import oracle
import workloads

from parity import compare_verify, logits_dtype, to_dev, workload_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, scope="module")
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _outputs(n, k, fill):
    dev = "cuda"
    return dict(out_tokens=torch.full((n, k + 1), fill, dtype=torch.int32, device=dev),
                out_accepted=torch.full((n,), fill, dtype=torch.int32, device=dev),
                out_p_draft=torch.full((n, k), float(fill), device=dev),
                out_q_draft=torch.full((n, k), float(fill), device=dev),
                out_residual_mass=torch.full((n,), float(fill), device=dev),
                out_q_entropy=torch.full((n, k), float(fill), device=dev),
                out_q_max=torch.full((n, k), float(fill), device=dev),
                dev_error=torch.zeros(1, dtype=torch.int32, device=dev))


def _both(name, mode, features, seed, step):
    w = workloads.make(name)
    kept = w.draft_len
    target, draft, toks, cu = workload_inputs(w, kept, mode)
    ldt = logits_dtype(w)
    t, d = to_dev(target, ldt), (None if draft is None else to_dev(draft, ldt))
    toks_d, cu_d = to_dev(np.asarray(toks, np.int32)), to_dev(np.asarray(cu, np.int32))
    m = sv.SV_GREEDY if mode == "greedy" else sv.SV_STOCHASTIC
    n, k = w.n, w.k_max
    ref = _outputs(n, k, -7)
    ws = torch.empty(sv.sv_verify_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    feat = {} if features else dict(out_q_entropy=None, out_q_max=None)
    sv.sv_verify(t, d, toks_d, cu_d, m, w.tau, seed, step, ws=ws, **{**ref, **feat})
    got = _outputs(n, k, -9)
    sv.sv_verify_noalloc(t, d, toks_d, cu_d, m, w.tau, seed, step, **{**got, **feat})
    torch.cuda.synchronize()
    for key in ref:
        if key in feat:
            continue
        a, b = ref[key].cpu().numpy(), got[key].cpu().numpy()
        np.testing.assert_array_equal(a.view(np.uint32) if a.dtype == np.float32 else a,
                                      b.view(np.uint32) if b.dtype == np.float32 else b,
                                      err_msg=f"{name} {mode} {key}")
    g = {k2: v.cpu().numpy() for k2, v in got.items() if k2 not in feat}
    g = {("tokens" if k2 == "out_tokens" else k2.replace("out_", "")): v for k2, v in g.items()}
    compare_verify(g, target, draft, toks, cu, k, w.vocab, mode, w.tau, seed, step)
    return n


def test_noalloc_matches_sv_verify_on_two_calls_in_a_row():
    n1 = _both("b64_v128256", "stochastic", True, 3, 1)
    n2 = _both("b16_v32000", "stochastic", False, 4, 2)   # smaller, over the first's records
    assert n2 < n1
    _both("tiny", "greedy", False, 0, 0)                  # smaller still, greedy
    _both("b64_v128256", "stochastic", False, 5, 3)       # larger again


def test_noalloc_refuses_a_batch_beyond_its_array():
    per_req = (2 * 7 + 1) * 128 + 7 * 64
    n = sv.SV_NOALLOC_WS_BYTES // per_req + 1
    assert sv.sv_verify_workspace_bytes(n, 7) > sv.SV_NOALLOC_WS_BYTES
    target = torch.zeros(8, 64, dtype=torch.bfloat16, device="cuda")
    draft = torch.zeros(n * 7, 64, dtype=torch.bfloat16, device="cuda")
    toks = torch.zeros(n, 7, dtype=torch.int32, device="cuda")
    cu = torch.zeros(n + 1, dtype=torch.int32, device="cuda")
    out = _outputs(n, 7, -3)
    with pytest.raises(sv.SvError) as e:
        sv.sv_verify_noalloc(target, draft, toks, cu, sv.SV_STOCHASTIC, 1.0, 0, 0, **out)
    assert e.value.status == sv.SV_ERR_CAPACITY
    torch.cuda.synchronize()
    assert (out["out_tokens"] == -3).all() and (out["out_accepted"] == -3).all()


def _outs(n, k):
    dev = "cuda"
    return dict(out_tokens=torch.full((n, k + 1), -7, dtype=torch.int32, device=dev),
                out_accepted=torch.full((n,), -7, dtype=torch.int32, device=dev),
                out_p_draft=torch.full((n, k), -7.0, device=dev),
                out_q_draft=torch.full((n, k), -7.0, device=dev),
                out_residual_mass=torch.full((n,), -7.0, device=dev),
                dev_error=torch.zeros(1, dtype=torch.int32, device=dev))


def _same(a, b, what):
    for key in a:
        x, y = a[key].cpu().numpy(), b[key].cpu().numpy()
        np.testing.assert_array_equal(x.view(np.uint32) if x.dtype == np.float32 else x,
                                      y.view(np.uint32) if y.dtype == np.float32 else y,
                                      err_msg=f"{what} {key}")


def test_noalloc_replays_from_a_graph():
    w = workloads.make("b64_v128256")
    n, k = w.n, w.k_max
    ldt = logits_dtype(w)
    # three input sets of one shape: the graph reads whatever the buffers hold
    sets = []
    for i in range(3):
        rng_w = workloads.make("b64_v128256")
        target, draft, toks, cu = workload_inputs(rng_w, w.draft_len, "stochastic")
        if i:
            target = np.roll(target, 37 * i, axis=1)
            draft = np.roll(draft, 37 * i, axis=1)
        sets.append((target, draft, toks, cu))
    t = to_dev(sets[0][0], ldt)
    d = to_dev(sets[0][1], ldt)
    toks_d = to_dev(np.asarray(sets[0][2], np.int32))
    cu_d = to_dev(np.asarray(sets[0][3], np.int32))
    got = _outs(n, k)
    kw = dict(out_q_entropy=None, out_q_max=None)
    # eager first call on this GPU, then record one call on a side stream
    sv.sv_verify_noalloc(t, d, toks_d, cu_d, sv.SV_STOCHASTIC, w.tau, 11, 5, **got, **kw)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            sv.sv_verify_noalloc(t, d, toks_d, cu_d, sv.SV_STOCHASTIC, w.tau, 11, 5, **got,
                                 **kw)
    torch.cuda.synchronize()
    ws = torch.empty(sv.sv_verify_workspace_bytes(n, k), dtype=torch.uint8, device="cuda")
    for i in (1, 2, 0, 1):
        target, draft, _, _ = sets[i]
        t.copy_(torch.from_numpy(target).to(ldt))
        d.copy_(torch.from_numpy(draft).to(ldt))
        for key, v in got.items():
            v.fill_(0 if key == "dev_error" else -3)   # dev_error only gathers bits
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = _outs(n, k)
        sv.sv_verify(t, d, toks_d, cu_d, sv.SV_STOCHASTIC, w.tau, 11, 5, ws=ws, **ref, **kw)
        torch.cuda.synchronize()
        _same(ref, got, f"replay of input set {i}")
        assert int(got["dev_error"][0]) == 0

"""Python binding of libspecverify (argument marshalling only).

Every step of the verify path runs in the HIP kernels of libspecverify.so,
built in-tree by ``adaptive_draft_verification_amd/build.py``.  PyTorch supplies
device memory and streams; nothing here computes.  Importing this module
fails loudly if the library has not been built: there is no fallback.

The functions keep the C names (sv_budget_select, sv_pack_varlen, sv_verify,
...) and take torch tensors; shapes are read from the tensors, the stream is
torch's current stream unless one is given.  A non-OK status raises SvError.
"""

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_DTYPE, SV_ERR_VALUE, SV_ERR_WORKSPACE, SV_ERR_LAUNCH, \
    SV_ERR_CAPACITY, SV_ERR_DATA = range(9)
SV_F32, SV_BF16 = 0, 1
SV_STOCHASTIC, SV_GREEDY = 0, 1
SV_DEV_BAD_CU_ROWS, SV_DEV_BAD_TOKEN, SV_DEV_NONFINITE = 1, 2, 4
SV_DEV_BAD_DRAFT_LEN, SV_DEV_BAD_COST, SV_DEV_BAD_KEPT = 8, 16, 32
SV_MAX_BUDGET_SLOTS, SV_MAX_DRAFT, SV_MAX_VOCAB = 8192, 64, 1048576
SV_MAX_VERIFY_SLOTS = 524288
SV_NOALLOC_WS_BYTES = 8388608

EXPORTED = ["sv_status_str", "sv_budget_workspace_bytes", "sv_verify_workspace_bytes",
            "sv_cost_table_prepare", "sv_budget_select", "sv_budget_allocate",
            "sv_budget_select_pack", "sv_budget_allocate_pack",
            "sv_uniform_k_select", "sv_pack_varlen",
            "sv_verify",
            "sv_verify_stages", "sv_verify_noalloc", "sv_accept_stats", "sv_calibrate_update", "sv_calibrate_predict",
            "sv_philox_uniforms"]


class SvError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {_lib.sv_status_str(status).decode()} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python adaptive_draft_verification_amd/build.py` "
                          "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u64, f32, sz = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint64, ctypes.c_float, ctypes.c_size_t)
    sig = {
        "sv_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "sv_budget_workspace_bytes": (sz, [i32, i32]),
        "sv_verify_workspace_bytes": (sz, [i32, i32]),
        "sv_cost_table_prepare": (ctypes.c_int, [vp, i32, i32, vp, i32]),
        "sv_budget_select": (ctypes.c_int, [vp, vp, i32, i32, vp, i32, i32, i32, vp, vp, vp, vp,
                                            vp, sz, vp]),
        "sv_budget_allocate": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sv_budget_select_pack": (ctypes.c_int, [vp, vp, i32, i32, vp, i32, i32, i32, vp, vp, vp,
                                                 vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "sv_budget_allocate_pack": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                   vp, vp, vp, vp, vp, sz, vp]),
        "sv_uniform_k_select": (ctypes.c_int, [vp, vp, i32, i32, vp, i32, i32, i32, vp, vp, vp,
                                               vp, vp]),
        "sv_pack_varlen": (ctypes.c_int, [vp, vp, vp, i32, i32, vp, vp, vp, vp, vp, vp]),
        "sv_verify": (ctypes.c_int, [vp, i64, i64, vp, i64, ctypes.c_int, i32, vp, vp, i32, i32,
                                     ctypes.c_int, f32, u64, u64, vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]),
        "sv_verify_stages": (ctypes.c_int, [vp, i64, i64, vp, i64, ctypes.c_int, i32, vp, vp, i32,
                                            i32, ctypes.c_int, f32, u64, u64, vp, vp, vp, vp, vp,
                                            vp, vp, vp, vp, sz, i32, vp]),
        "sv_verify_noalloc": (ctypes.c_int, [vp, i64, i64, vp, i64, ctypes.c_int, i32, vp, vp,
                                             i32, i32, ctypes.c_int, f32, u64, u64, vp, vp, vp,
                                             vp, vp, vp, vp, vp, vp]),
        "sv_accept_stats": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, vp, vp]),
        "sv_calibrate_update": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, i32, i32, f32, vp, vp]),
        "sv_calibrate_predict": (ctypes.c_int, [vp, vp, vp, vp, i32, i32, vp, vp]),
        "sv_philox_uniforms": (ctypes.c_int, [u64, u64, i32, i32, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(t, dtype, name, ndim=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")


def _check(status, where):
    if status != SV_OK:
        raise SvError(status, where)


def sv_status_str(status):
    return _lib.sv_status_str(status).decode()


def sv_budget_workspace_bytes(n_req, k_max):
    return int(_lib.sv_budget_workspace_bytes(n_req, k_max))


def sv_verify_workspace_bytes(n_req, k_max):
    return int(_lib.sv_verify_workspace_bytes(n_req, k_max))


def sv_cost_table_prepare(raw, granule, out_len):
    """Host call: shaped cost table (numpy fp32 in, numpy fp32 out)."""
    raw = np.ascontiguousarray(raw, dtype=np.float32)
    out = np.zeros(int(out_len), dtype=np.float32)
    _check(_lib.sv_cost_table_prepare(raw.ctypes.data_as(ctypes.c_void_p), len(raw), int(granule),
                                      out.ctypes.data_as(ctypes.c_void_p), int(out_len)),
           "sv_cost_table_prepare")
    return out


def sv_budget_select(conf, draft_len, cost, t_base, n_bonus, kept, budget, survival=None,
                     dev_error=None, stream=None, ws=None):
    """conf [n, k_max] f32, draft_len [n] i32, cost [L] f32 -> kept [n] i32, budget [1] i32.

    ws: device uint8 tensor of at least sv_budget_workspace_bytes(n, k_max) bytes."""
    _dev(conf, torch.float32, "conf", 2)
    _dev(draft_len, torch.int32, "draft_len", 1)
    _dev(cost, torch.float32, "cost", 1)
    _dev(kept, torch.int32, "kept", 1)
    _dev(budget, torch.int32, "budget", 1)
    _dev(survival, torch.float32, "survival", 2)
    _dev(dev_error, torch.int32, "dev_error", 1)
    _dev(ws, torch.uint8, "ws", 1)
    n, k_max = conf.shape
    if draft_len.numel() != n or kept.numel() != n or budget.numel() < 1:
        raise ValueError("draft_len, kept must have n entries and budget one")
    if survival is not None and tuple(survival.shape) != (n, k_max):
        raise ValueError("survival must be [n, k_max]")
    _check(_lib.sv_budget_select(_ptr(conf), _ptr(draft_len), n, k_max, _ptr(cost), cost.numel(),
                                 int(t_base), int(n_bonus), _ptr(kept), _ptr(budget),
                                 _ptr(survival), _ptr(dev_error), _ptr(ws), 0 if ws is None else ws.numel(),
                                 _stream(stream)),
           "sv_budget_select")


def sv_budget_allocate(conf, draft_len, budget_in, kept, budget_used=None, survival=None,
                       dev_error=None, stream=None, ws=None):
    """conf [n, k_max] f32, draft_len [n] i32, budget_in [1] i32 (device) -> kept [n] i32.

    ws: device uint8 tensor of at least sv_budget_workspace_bytes(n, k_max) bytes."""
    _dev(conf, torch.float32, "conf", 2)
    _dev(draft_len, torch.int32, "draft_len", 1)
    _dev(budget_in, torch.int32, "budget_in", 1)
    _dev(kept, torch.int32, "kept", 1)
    _dev(budget_used, torch.int32, "budget_used", 1)
    _dev(survival, torch.float32, "survival", 2)
    _dev(dev_error, torch.int32, "dev_error", 1)
    _dev(ws, torch.uint8, "ws", 1)
    n, k_max = conf.shape
    if draft_len.numel() != n or kept.numel() != n or budget_in.numel() < 1:
        raise ValueError("draft_len, kept must have n entries and budget_in one")
    if survival is not None and tuple(survival.shape) != (n, k_max):
        raise ValueError("survival must be [n, k_max]")
    _check(_lib.sv_budget_allocate(_ptr(conf), _ptr(draft_len), n, k_max, _ptr(budget_in),
                                   _ptr(kept), _ptr(budget_used), _ptr(survival), _ptr(dev_error),
                                   _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream)),
           "sv_budget_allocate")


def _pack_outputs(n, k_max, last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens):
    for name, t in (("last_token", last_token), ("cu_rows", cu_rows), ("row_req", row_req),
                    ("row_pos", row_pos), ("packed_tokens", packed_tokens)):
        _dev(t, torch.int32, name, 1)
    _dev(draft_tokens, torch.int32, "draft_tokens", 2)
    cap = n * (k_max + 1)
    if tuple(draft_tokens.shape) != (n, k_max) or last_token.numel() != n \
            or cu_rows.numel() != n + 1:
        raise ValueError("draft_tokens [n, k_max], last_token [n], cu_rows [n+1]")
    if row_req.numel() != cap or row_pos.numel() != cap or packed_tokens.numel() != cap:
        raise ValueError("row maps need n*(k_max+1) entries")


def sv_budget_select_pack(conf, draft_len, cost, t_base, n_bonus, last_token, draft_tokens, kept,
                          budget, cu_rows, row_req, row_pos, packed_tokens, survival=None,
                          dev_error=None, stream=None, ws=None):
    """sv_budget_select then sv_pack_varlen, one launch fewer (same tensors as the two)."""
    for name, t, nd in (("conf", conf, 2), ("draft_len", draft_len, 1), ("cost", cost, 1),
                        ("kept", kept, 1), ("budget", budget, 1)):
        _dev(t, torch.float32 if name in ("conf", "cost") else torch.int32, name, nd)
    _dev(survival, torch.float32, "survival", 2)
    _dev(dev_error, torch.int32, "dev_error", 1)
    _dev(ws, torch.uint8, "ws", 1)
    n, k_max = conf.shape
    if draft_len.numel() != n or kept.numel() != n or budget.numel() < 1:
        raise ValueError("draft_len, kept must have n entries and budget one")
    _pack_outputs(n, k_max, last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens)
    _check(_lib.sv_budget_select_pack(_ptr(conf), _ptr(draft_len), n, k_max, _ptr(cost),
                                      cost.numel(), int(t_base), int(n_bonus), _ptr(last_token),
                                      _ptr(draft_tokens), _ptr(kept), _ptr(budget),
                                      _ptr(survival), _ptr(cu_rows), _ptr(row_req), _ptr(row_pos),
                                      _ptr(packed_tokens), _ptr(dev_error), _ptr(ws),
                                      0 if ws is None else ws.numel(), _stream(stream)),
           "sv_budget_select_pack")


def sv_budget_allocate_pack(conf, draft_len, budget_in, last_token, draft_tokens, kept, cu_rows,
                            row_req, row_pos, packed_tokens, budget_used=None, survival=None,
                            dev_error=None, stream=None, ws=None):
    """sv_budget_allocate then sv_pack_varlen, one launch fewer."""
    _dev(conf, torch.float32, "conf", 2)
    for name, t in (("draft_len", draft_len), ("budget_in", budget_in), ("kept", kept),
                    ("budget_used", budget_used), ("dev_error", dev_error)):
        _dev(t, torch.int32, name, 1)
    _dev(survival, torch.float32, "survival", 2)
    _dev(ws, torch.uint8, "ws", 1)
    n, k_max = conf.shape
    if draft_len.numel() != n or kept.numel() != n or budget_in.numel() < 1:
        raise ValueError("draft_len, kept must have n entries and budget_in one")
    _pack_outputs(n, k_max, last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens)
    _check(_lib.sv_budget_allocate_pack(_ptr(conf), _ptr(draft_len), n, k_max, _ptr(budget_in),
                                        _ptr(last_token), _ptr(draft_tokens), _ptr(kept),
                                        _ptr(budget_used), _ptr(survival), _ptr(cu_rows),
                                        _ptr(row_req), _ptr(row_pos), _ptr(packed_tokens),
                                        _ptr(dev_error), _ptr(ws),
                                        0 if ws is None else ws.numel(), _stream(stream)),
           "sv_budget_allocate_pack")


def sv_uniform_k_select(conf, draft_len, cost, t_base, n_bonus, kept, k_out, scores=None,
                        dev_error=None, stream=None):
    """conf [n, k_max] f32, draft_len [n] i32, cost [L] f32 -> kept [n] i32, k_out [1] i32,
    scores [k_max + 1] f64 (optional)."""
    _dev(conf, torch.float32, "conf", 2)
    _dev(draft_len, torch.int32, "draft_len", 1)
    _dev(cost, torch.float32, "cost", 1)
    _dev(kept, torch.int32, "kept", 1)
    _dev(k_out, torch.int32, "k_out", 1)
    _dev(scores, torch.float64, "scores", 1)
    _dev(dev_error, torch.int32, "dev_error", 1)
    n, k_max = conf.shape
    if draft_len.numel() != n or kept.numel() != n or k_out.numel() < 1:
        raise ValueError("draft_len, kept must have n entries and k_out one")
    if scores is not None and scores.numel() != k_max + 1:
        raise ValueError("scores must have k_max + 1 entries")
    _check(_lib.sv_uniform_k_select(_ptr(conf), _ptr(draft_len), n, k_max, _ptr(cost),
                                    cost.numel(), int(t_base), int(n_bonus), _ptr(kept),
                                    _ptr(k_out), _ptr(scores), _ptr(dev_error), _stream(stream)),
           "sv_uniform_k_select")


def sv_pack_varlen(kept, last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens,
                   dev_error=None, stream=None):
    """kept [n], last_token [n], draft_tokens [n, k_max] -> cu_rows [n+1], row maps [n(k_max+1)]."""
    for name, t in (("kept", kept), ("last_token", last_token), ("cu_rows", cu_rows),
                    ("row_req", row_req), ("row_pos", row_pos), ("packed_tokens", packed_tokens)):
        _dev(t, torch.int32, name, 1)
    _dev(draft_tokens, torch.int32, "draft_tokens", 2)
    _dev(dev_error, torch.int32, "dev_error", 1)
    n, k_max = draft_tokens.shape
    cap = n * (k_max + 1)
    if kept.numel() != n or last_token.numel() != n or cu_rows.numel() != n + 1:
        raise ValueError("kept/last_token need n entries, cu_rows n+1")
    if row_req.numel() != cap or row_pos.numel() != cap or packed_tokens.numel() != cap:
        raise ValueError("row maps need n*(k_max+1) entries")
    _check(_lib.sv_pack_varlen(_ptr(kept), _ptr(last_token), _ptr(draft_tokens), n, k_max,
                               _ptr(cu_rows), _ptr(row_req), _ptr(row_pos), _ptr(packed_tokens),
                               _ptr(dev_error), _stream(stream)),
           "sv_pack_varlen")


_DTYPES = {torch.bfloat16: SV_BF16, torch.float32: SV_F32}


def _verify_args(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                 out_tokens, out_accepted, ws, out_p_draft, out_q_draft, out_residual_mass,
                 dev_error, vocab, out_q_entropy, out_q_max):
    if target.dtype not in _DTYPES:
        raise ValueError("logits must be bfloat16 or float32")
    _dev(target, target.dtype, "target", 2)
    if draft is not None:
        _dev(draft, target.dtype, "draft", 2)
    _dev(draft_tokens, torch.int32, "draft_tokens", 2)
    _dev(cu_rows, torch.int32, "cu_rows", 1)
    _dev(out_tokens, torch.int32, "out_tokens", 2)
    _dev(out_accepted, torch.int32, "out_accepted", 1)
    _dev(ws, torch.uint8, "ws", 1)
    for name, t in (("out_p_draft", out_p_draft), ("out_q_draft", out_q_draft),
                    ("out_q_entropy", out_q_entropy), ("out_q_max", out_q_max)):
        _dev(t, torch.float32, name, 2)
    _dev(out_residual_mass, torch.float32, "out_residual_mass", 1)
    _dev(dev_error, torch.int32, "dev_error", 1)
    n, k_max = draft_tokens.shape
    V = target.shape[1] if vocab is None else int(vocab)
    if cu_rows.numel() != n + 1 or tuple(out_tokens.shape) != (n, k_max + 1) \
            or out_accepted.numel() != n:
        raise ValueError("cu_rows [n+1], out_tokens [n, k_max+1], out_accepted [n]")
    if draft is not None and draft.shape[0] < n * k_max:
        raise ValueError("draft must hold n*k_max rows")
    for t in (out_p_draft, out_q_draft, out_q_entropy, out_q_max):
        if t is not None and tuple(t.shape) != (n, k_max):
            raise ValueError("out_p_draft, out_q_draft, out_q_entropy, out_q_max must be "
                             "[n, k_max]")
    if out_residual_mass is not None and out_residual_mass.numel() != n:
        raise ValueError("out_residual_mass must have n entries")
    return [_ptr(target), target.shape[1], target.shape[0], _ptr(draft),
            0 if draft is None else draft.shape[1], _DTYPES[target.dtype], V,
            _ptr(draft_tokens), _ptr(cu_rows), n, k_max, int(mode), float(temperature),
            int(seed), int(step), _ptr(out_tokens), _ptr(out_accepted), _ptr(out_p_draft),
            _ptr(out_q_draft), _ptr(out_residual_mass), _ptr(out_q_entropy), _ptr(out_q_max),
            _ptr(dev_error), _ptr(ws), 0 if ws is None else ws.numel()]


def sv_verify(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step, out_tokens,
              out_accepted, ws, out_p_draft=None, out_q_draft=None, out_residual_mass=None,
              dev_error=None, vocab=None, stream=None, out_q_entropy=None, out_q_max=None):
    """target [rows, >=V] and draft [n*k_max, >=V] (bf16 or f32, row stride = shape[1]);
    draft_tokens [n, k_max] i32; cu_rows [n+1] i32; ws: uint8 device buffer of
    sv_verify_workspace_bytes(n, k_max) bytes; out_q_entropy / out_q_max [n, k_max] f32
    ask pass 1 for the draft-row features."""
    args = _verify_args(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                        out_tokens, out_accepted, ws, out_p_draft, out_q_draft,
                        out_residual_mass, dev_error, vocab, out_q_entropy, out_q_max)
    _check(_lib.sv_verify(*args, _stream(stream)), "sv_verify")


def sv_verify_stages(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                     out_tokens, out_accepted, ws, stages, out_p_draft=None, out_q_draft=None,
                     out_residual_mass=None, dev_error=None, vocab=None, stream=None,
                     out_q_entropy=None, out_q_max=None):
    """sv_verify restricted to pass 1 (stages=1), pass 2 (stages=2) or both (3)."""
    args = _verify_args(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                        out_tokens, out_accepted, ws, out_p_draft, out_q_draft,
                        out_residual_mass, dev_error, vocab, out_q_entropy, out_q_max)
    _check(_lib.sv_verify_stages(*args, int(stages), _stream(stream)), "sv_verify_stages")


def sv_verify_noalloc(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                      out_tokens, out_accepted, out_p_draft=None, out_q_draft=None,
                      out_residual_mass=None, dev_error=None, vocab=None, stream=None,
                      out_q_entropy=None, out_q_max=None):
    """sv_verify without a workspace argument: the library's static per-GPU array
    serves as the workspace (the call allocates nothing; overlapping calls on one
    GPU race on it)."""
    args = _verify_args(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                        out_tokens, out_accepted, None, out_p_draft, out_q_draft,
                        out_residual_mass, dev_error, vocab, out_q_entropy, out_q_max)
    _check(_lib.sv_verify_noalloc(*args[:-2], _stream(stream)), "sv_verify_noalloc")


def sv_accept_stats(accepted, cu_rows, attempted, accepted_at, totals, stream=None):
    """accepted [n] i32, cu_rows [n+1] i32 -> adds to attempted/accepted_at [k_max] and
    totals [2] (int64 device tensors holding uint64 counts)."""
    _dev(accepted, torch.int32, "accepted", 1)
    _dev(cu_rows, torch.int32, "cu_rows", 1)
    for name, t in (("attempted", attempted), ("accepted_at", accepted_at), ("totals", totals)):
        _dev(t, torch.int64, name, 1)
    n = accepted.numel()
    k_max = attempted.numel()
    if cu_rows.numel() != n + 1 or accepted_at.numel() != k_max or totals.numel() < 2:
        raise ValueError("cu_rows [n+1], attempted/accepted_at [k_max], totals [2]")
    _check(_lib.sv_accept_stats(_ptr(accepted), _ptr(cu_rows), n, k_max, _ptr(attempted),
                                _ptr(accepted_at), _ptr(totals), _stream(stream)),
           "sv_accept_stats")


def _features(q_draft, q_entropy, q_max):
    _dev(q_draft, torch.float32, "q_draft", 2)
    for name, t in (("q_entropy", q_entropy), ("q_max", q_max)):
        _dev(t, torch.float32, name, 2)
        if t is not None and t.shape != q_draft.shape:
            raise ValueError(f"{name} must have q_draft's shape")
    return q_draft.shape


def sv_calibrate_update(theta, q_draft, accepted, cu_rows, lr, count_out=None, stream=None,
                        q_entropy=None, q_max=None):
    """theta [k_max+3] f32 (in place); q_draft, q_entropy, q_max [n, k_max] f32 (the last
    two may be None: feature 0); accepted [n]; cu_rows [n+1]."""
    _dev(theta, torch.float32, "theta", 1)
    _dev(accepted, torch.int32, "accepted", 1)
    _dev(cu_rows, torch.int32, "cu_rows", 1)
    _dev(count_out, torch.int32, "count_out", 1)
    n, k_max = _features(q_draft, q_entropy, q_max)
    if theta.numel() != k_max + 3 or accepted.numel() != n or cu_rows.numel() != n + 1:
        raise ValueError("theta [k_max+3], accepted [n], cu_rows [n+1]")
    _check(_lib.sv_calibrate_update(_ptr(theta), _ptr(q_draft), _ptr(q_entropy), _ptr(q_max),
                                    _ptr(accepted), _ptr(cu_rows), n, k_max, float(lr),
                                    _ptr(count_out), _stream(stream)),
           "sv_calibrate_update")


def sv_calibrate_predict(theta, q_draft, conf, stream=None, q_entropy=None, q_max=None):
    """conf [n, k_max] f32 <- sigmoid(alpha_j + beta . x(q, entropy, max prob))."""
    _dev(theta, torch.float32, "theta", 1)
    _dev(conf, torch.float32, "conf", 2)
    n, k_max = _features(q_draft, q_entropy, q_max)
    if theta.numel() != k_max + 3 or tuple(conf.shape) != (n, k_max):
        raise ValueError("theta [k_max+3], conf [n, k_max]")
    _check(_lib.sv_calibrate_predict(_ptr(theta), _ptr(q_draft), _ptr(q_entropy), _ptr(q_max), n,
                                     k_max, _ptr(conf), _stream(stream)),
           "sv_calibrate_predict")


def sv_philox_uniforms(seed, step, u, v, stream=None):
    """u, v [n, n_pos] f32 <- the uniforms sv_verify draws for (r, j, step)."""
    _dev(u, torch.float32, "u", 2)
    _dev(v, torch.float32, "v", 2)
    n, n_pos = u.shape
    if tuple(v.shape) != (n, n_pos):
        raise ValueError("u and v must have the same shape")
    _check(_lib.sv_philox_uniforms(int(seed), int(step), n, n_pos, _ptr(u), _ptr(v),
                                   _stream(stream)),
           "sv_philox_uniforms")


# ----------------------------------------------------------------------------
# Allocating conveniences over the calls above (outputs are new device tensors).

def budget_select(conf, draft_len, cost, t_base, n_bonus, stream=None):
    dev = conf.device
    n, k_max = conf.shape
    kept = torch.empty(n, dtype=torch.int32, device=dev)
    budget = torch.empty(1, dtype=torch.int32, device=dev)
    survival = torch.empty(n, k_max, dtype=torch.float32, device=dev)
    err = torch.zeros(1, dtype=torch.int32, device=dev)
    ws = torch.empty(max(1, sv_budget_workspace_bytes(n, k_max)), dtype=torch.uint8, device=dev)
    sv_budget_select(conf, draft_len, cost, t_base, n_bonus, kept, budget, survival, err, stream,
                     ws=ws)
    return dict(kept=kept, budget=budget, survival=survival, dev_error=err)


def budget_allocate(conf, draft_len, budget_in, stream=None, ws=None):
    dev = conf.device
    n, k_max = conf.shape
    out = dict(kept=torch.empty(n, dtype=torch.int32, device=dev),
               budget_used=torch.empty(1, dtype=torch.int32, device=dev),
               survival=torch.empty(n, k_max, dtype=torch.float32, device=dev),
               dev_error=torch.zeros(1, dtype=torch.int32, device=dev))
    if ws is None:
        ws = torch.empty(max(1, sv_budget_workspace_bytes(n, k_max)), dtype=torch.uint8,
                         device=dev)
    sv_budget_allocate(conf, draft_len, budget_in, out["kept"], out["budget_used"],
                       out["survival"], out["dev_error"], stream, ws=ws)
    return out


def uniform_k_select(conf, draft_len, cost, t_base, n_bonus, stream=None):
    dev = conf.device
    n, k_max = conf.shape
    out = dict(kept=torch.empty(n, dtype=torch.int32, device=dev),
               k=torch.empty(1, dtype=torch.int32, device=dev),
               scores=torch.empty(k_max + 1, dtype=torch.float64, device=dev),
               dev_error=torch.zeros(1, dtype=torch.int32, device=dev))
    sv_uniform_k_select(conf, draft_len, cost, t_base, n_bonus, out["kept"], out["k"],
                        out["scores"], out["dev_error"], stream)
    return out


def pack_varlen(kept, last_token, draft_tokens, stream=None):
    dev = kept.device
    n, k_max = draft_tokens.shape
    cap = n * (k_max + 1)
    out = dict(cu_rows=torch.empty(n + 1, dtype=torch.int32, device=dev),
               row_req=torch.empty(cap, dtype=torch.int32, device=dev),
               row_pos=torch.empty(cap, dtype=torch.int32, device=dev),
               packed_tokens=torch.empty(cap, dtype=torch.int32, device=dev),
               dev_error=torch.zeros(1, dtype=torch.int32, device=dev))
    sv_pack_varlen(kept, last_token, draft_tokens, out["cu_rows"], out["row_req"],
                   out["row_pos"], out["packed_tokens"], out["dev_error"], stream)
    return out


def verify(target, draft, draft_tokens, cu_rows, mode, temperature=1.0, seed=0, step=0,
           vocab=None, stream=None, stages=None, ws=None, features=False):
    """Allocating wrapper: sv_verify, or sv_verify_stages(stages) when `stages` is given.
    ws: a workspace to reuse.  features: also return the draft-row features q_entropy and
    q_max (pass 1 then accumulates them)."""
    dev = target.device
    n, k_max = draft_tokens.shape
    if ws is None:
        ws = torch.zeros(max(1, sv_verify_workspace_bytes(n, k_max)), dtype=torch.uint8,
                         device=dev)
    out = dict(tokens=torch.empty(n, k_max + 1, dtype=torch.int32, device=dev),
               accepted=torch.empty(n, dtype=torch.int32, device=dev),
               p_draft=torch.empty(n, k_max, dtype=torch.float32, device=dev),
               q_draft=torch.empty(n, k_max, dtype=torch.float32, device=dev),
               residual_mass=torch.empty(n, dtype=torch.float32, device=dev),
               dev_error=torch.zeros(1, dtype=torch.int32, device=dev))
    if features:
        out["q_entropy"] = torch.empty(n, k_max, dtype=torch.float32, device=dev)
        out["q_max"] = torch.empty(n, k_max, dtype=torch.float32, device=dev)
    feat = dict(out_q_entropy=out.get("q_entropy"), out_q_max=out.get("q_max"))
    if stages is None:
        sv_verify(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                  out["tokens"], out["accepted"], ws, out["p_draft"], out["q_draft"],
                  out["residual_mass"], out["dev_error"], vocab, stream, **feat)
    else:
        sv_verify_stages(target, draft, draft_tokens, cu_rows, mode, temperature, seed, step,
                         out["tokens"], out["accepted"], ws, stages, out["p_draft"],
                         out["q_draft"], out["residual_mass"], out["dev_error"], vocab, stream,
                         **feat)
    return out

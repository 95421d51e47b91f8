"""Varlen packing of kept verify rows — oracle side (test infrastructure).

agentlens page "vLLM DSpark을 활용한 적응형 검증(Adaptive Verification)",
section "기술적 구현 및 CUDA Graphs", item Graph Capture: one decode shape
holds any mix of 1 .. num_speculative_tokens+1 query tokens per request; and
section "설정 및 재현": the capture size is (num_speculative_tokens + 1) *
max_num_seq — here the row capacity n * (k_max + 1).  The PyTorch-KR DSD
page, section "비동기 스케줄링(Async Scheduling)과의 호환", fills slots whose
ids are unknown with -1; unused capacity rows here carry -1 the same way.

Request r owns rows cu_rows[r] .. cu_rows[r] + b_r.  Row i of request r is the
target position that follows i accepted drafts: row 0 carries the request's
last emitted token, row i > 0 carries draft token i-1.
"""

import numpy as np

DEV_BAD_KEPT = 32


def pack_varlen(kept, last_token, draft_tokens, k_max):
    """Return dict(cu_rows, row_req, row_pos, packed_tokens, dev_error)."""
    n = len(kept)
    cap = n * (k_max + 1)
    draft_tokens = np.asarray(draft_tokens).reshape(n, k_max) if k_max > 0 else \
        np.zeros((n, 0), dtype=np.int32)
    err = 0
    b = np.zeros(n, dtype=np.int64)
    for r in range(n):
        v = int(kept[r])
        if v < 0 or v > k_max:
            err |= DEV_BAD_KEPT
            v = min(max(v, 0), k_max)
        b[r] = v
    cu_rows = np.zeros(n + 1, dtype=np.int32)
    for r in range(n):
        cu_rows[r + 1] = cu_rows[r] + b[r] + 1
    row_req = np.full(cap, -1, dtype=np.int32)
    row_pos = np.full(cap, -1, dtype=np.int32)
    packed = np.full(cap, -1, dtype=np.int32)
    for r in range(n):
        for i in range(int(b[r]) + 1):
            row = cu_rows[r] + i
            row_req[row] = r
            row_pos[row] = i
            packed[row] = int(last_token[r]) if i == 0 else int(draft_tokens[r, i - 1])
    return dict(cu_rows=cu_rows, row_req=row_req, row_pos=row_pos,
                packed_tokens=packed, dev_error=err)

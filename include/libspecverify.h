/*
 * libspecverify — the batched speculative-decoding verify step on AMD Instinct
 * MI355X (gfx950): adaptive budget selection, varlen packing of the kept
 * rows, and full-vocabulary verification (stochastic or greedy).
 *
 * Pages this interface follows (cited by title and section):
 *  - FOS Study blog "추측 디코딩과 vLLM 적응형 검증" (Speculative decoding and
 *    vLLM adaptive verification);
 *  - agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive Verification)";
 *  - PyTorch-KR "Hardware-Aware Dynamic Speculative Decoding (DSD), feat.
 *    Cohere".
 *
 * Conventions for every call below.
 *  - Array arguments are caller-owned DEVICE pointers unless marked "host".
 *    The library allocates nothing and keeps no state between calls.
 *  - Every call only enqueues work on `stream` (a hipStream_t passed as an
 *    opaque pointer; NULL is the default stream) and never synchronises, so
 *    outputs are valid once the stream has reached that point.
 *  - The return value reports faults the host can see before anything is
 *    enqueued (null pointers, sizes, out-of-range scalars, short workspace):
 *    then nothing is launched and no output is touched.  SV_ERR_LAUNCH means
 *    the HIP runtime refused a launch.
 *  - Faults that only the data on the device can show are ORed into
 *    *dev_error (SV_DEV_* bits below; the library never clears it, so zero it
 *    before the call).  dev_error may be NULL.  Kernels never read or write
 *    past the bounds the host validated, whatever the device data holds: the
 *    crash write-up on the FOS page (section "적응형 검증이 GPU 오류와 엮인
 *    사례") is about a kernel that trusted a length it was not given.
 *  - Layouts are row-major; int32 token ids; "-1" marks an empty slot, as the
 *    -1 placeholders of the DSD page (section "비동기 스케줄링(Async
 *    Scheduling)과의 호환").
 *  - Two environment variables, read at every call, serve debugging only (the
 *    FOS crash write-up: a device fault surfaces at the next synchronisation,
 *    not where it happened).  SV_FORCE_SYNC=1: after its launches a call
 *    waits for its stream (not while the stream is being captured into a
 *    graph) and returns SV_ERR_LAUNCH if one of its kernels failed, so the
 *    failing call is the one that reports it.  SV_DEBUG_CHECKS=1: before
 *    launching, sv_verify and sv_verify_stages, the budget calls and
 *    sv_pack_varlen copy their index inputs (row offsets, draft ids, draft
 *    lengths, kept counts) to the host, wait for them (not while capturing)
 *    and return SV_ERR_DATA, launching nothing, where the kernels would set a
 *    dev_error bit for them.  Both make calls synchronous and slow; neither
 *    changes any result.  sv_verify_noalloc honours SV_FORCE_SYNC only (its
 *    contract is to allocate nothing, host memory included).
 */
#ifndef LIBSPECVERIFY_H
#define LIBSPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SV_OK = 0,
    SV_ERR_NULL = 1,      /* a required pointer is NULL                        */
    SV_ERR_SHAPE = 2,     /* a size or stride is out of range                  */
    SV_ERR_DTYPE = 3,     /* unknown sv_dtype                                  */
    SV_ERR_VALUE = 4,     /* a scalar is out of range (temperature, mode, ...) */
    SV_ERR_WORKSPACE = 5, /* workspace missing or smaller than required        */
    SV_ERR_LAUNCH = 6,    /* the HIP runtime refused a kernel launch, or one failed
                             (SV_FORCE_SYNC)                                   */
    SV_ERR_CAPACITY = 7,  /* the batch needs more than a static workspace holds */
    SV_ERR_DATA = 8,      /* index data on the device is inconsistent
                             (SV_DEBUG_CHECKS only)                            */
    SV_STATUS_RANGE_LO_ = -2147483647 - 1, /* range markers, never returned: every */
    SV_STATUS_RANGE_HI_ = 2147483647       /* int32 is a value of the type         */
} sv_status;

/* The range markers make every int32 a value of the type (C++ gives an enum
 * only the range of its enumerators), so that the library can refuse an
 * unknown dtype or mode that a caller passes as a plain int. */
typedef enum {
    SV_F32 = 0,
    SV_BF16 = 1,
    SV_DTYPE_RANGE_LO_ = -2147483647 - 1,
    SV_DTYPE_RANGE_HI_ = 2147483647
} sv_dtype;
typedef enum {
    SV_STOCHASTIC = 0,
    SV_GREEDY = 1,
    SV_MODE_RANGE_LO_ = -2147483647 - 1,
    SV_MODE_RANGE_HI_ = 2147483647
} sv_mode;

/* Device error bits (ORed into *dev_error). */
#define SV_DEV_BAD_CU_ROWS   1  /* a request's row range is inconsistent or exceeds target_rows */
#define SV_DEV_BAD_TOKEN     2  /* a kept draft id is outside [0, vocab)                        */
#define SV_DEV_NONFINITE     4  /* a needed logit row holds NaN or +inf, or only -inf            */
#define SV_DEV_BAD_DRAFT_LEN 8  /* a draft length is outside [0, k_max] (clamped)                */
#define SV_DEV_BAD_COST      16 /* a consulted cost entry is not finite and > 0 (never chosen)   */
#define SV_DEV_BAD_KEPT      32 /* a kept count is outside [0, k_max] (clamped)                  */

/* Limits checked on the host. */
#define SV_MAX_BUDGET_SLOTS 8192   /* n_req and n_req * k_max for sv_budget_select (LDS-resident) */
#define SV_MAX_DRAFT        64     /* k_max for sv_verify (one wave64 ballot covers a request) and sv_budget_select */
#define SV_MAX_VOCAB        1048576
#define SV_NOALLOC_WS_BYTES 8388608   /* sv_verify_noalloc's static workspace per GPU (8 MiB) */
#define SV_MAX_VERIFY_SLOTS 524288     /* n_req * (2*k_max + 1) for sv_verify: its pass-1 grid (up to
                                           8 parts of 512 threads per row slot) stays below 2^32 work-items */

const char* sv_status_str(sv_status s);

/*
 * Workspace bytes the device calls need (0 = none; pass ws = NULL then; also 0
 * for shapes the call rejects).  sv_verify keeps one 16-byte statistics record
 * per candidate row part and one 8-byte feature record per draft row part.
 */
size_t sv_budget_workspace_bytes(int32_t n_req, int32_t k_max);
size_t sv_verify_workspace_bytes(int32_t n_req, int32_t k_max);

/*
 * sv_cost_table_prepare — HOST ONLY (no device work).
 *
 * agentlens page, section "기술적 구현 및 CUDA Graphs": the engine profiles
 * the step cost per token count at start-up (item Cost Modeling), forces the
 * curve to be monotone to absorb profiling noise and tile effects, and prices
 * a batch at the next captured graph size (item CUDA Graph Padding: 121 tokens
 * cost what 128 do).  Here: out[t] = max(raw[0 .. ceil_g(t)]) for
 * t = 0 .. out_len-1, where ceil_g rounds up to a multiple of `granule`
 * (granule 1 = no padding).
 *
 * raw:  host, raw_len fp32 profiled costs, each finite and > 0.
 * out:  host, out_len fp32 (may not alias raw).
 * Errors: SV_ERR_NULL; SV_ERR_SHAPE if granule < 1, out_len < 1 or
 * raw_len < ceil_g(out_len-1) + 1; SV_ERR_VALUE if a raw entry is not finite
 * and > 0 (out untouched).
 */
sv_status sv_cost_table_prepare(const float* raw, int32_t raw_len, int32_t granule,
                                float* out, int32_t out_len);

/*
 * sv_budget_select — adaptive verification budget.
 *
 * FOS page, section "적응형 검증 > 동작", steps 1-3, and agentlens page,
 * section "DSpark 신뢰도 스케줄링 메커니즘" (Global Top-B Selection, Budget
 * Calculation):
 *  1. survival s[r, j-1] = c[r,0] * ... * c[r,j-1] for draft position
 *     j = 1..draft_len[r], taken left to right in fp32 (round to nearest),
 *     each confidence clamped to [0, 1] with NaN read as 0;
 *  2. every draft slot of the batch ranked by survival, descending; ties to
 *     the lower request, then the lower position — so each request's kept
 *     slots are a front prefix;
 *  3. B = the smallest maximiser over B = 0 .. sum(draft_len) of
 *     (n_bonus + S(B)) / cost[t_base + B], where S(B) is the sum of the B best
 *     survivals, taken exactly as sum(floor(s * 2^40)) * 2^-40 and the ratio
 *     in fp64;
 *  4. kept[r] = number of request r's slots among the first B.
 *
 * conf:      [n_req, k_max] fp32 per-position acceptance estimates.
 * draft_len: [n_req] int32 drafts written per request (clamped into
 *            [0, k_max], SV_DEV_BAD_DRAFT_LEN).
 * cost:      [cost_len] fp32 step cost by token count, already shaped (see
 *            sv_cost_table_prepare); cost_len >= t_base + n_req*k_max + 1.
 *            Entries consulted that are not finite and > 0 are never chosen
 *            (SV_DEV_BAD_COST); if none is usable B = 0.
 * t_base:    non-draft tokens in the step (one per request for pure decode).
 * n_bonus:   bonus tokens (one per sampling request).
 * kept:      [n_req] int32 out.   budget: [1] int32 out (B).
 * survival:  [n_req, k_max] fp32 out, or NULL (0 past draft_len).
 * ws:        device scratch of sv_budget_workspace_bytes(n_req, k_max) bytes
 *            (16 + 8 * n_req * k_max: slot ranks and rank-ordered survivals;
 *            needs no initialisation, garbage afterwards).  May be NULL when
 *            that size is 0 (n_req = 0).  Calls that overlap in time must
 *            not share a workspace.
 * Launch: two kernels on `stream`.  The first ranks every slot: one
 * 1024-thread workgroup per 16 slots counts, for each of its slots, the
 * keys of the whole batch ordered before it (the keys staged in LDS).  The
 * second, one workgroup of 1024 threads, scans the rank-ordered survivals
 * and picks B.
 * Errors: SV_ERR_NULL; SV_ERR_SHAPE if n_req < 0, k_max < 0, k_max > SV_MAX_DRAFT,
 * n_req or n_req * k_max > SV_MAX_BUDGET_SLOTS, or cost_len too short; SV_ERR_VALUE if
 * t_base < 0 or n_bonus < 0; SV_ERR_WORKSPACE if ws is NULL or ws_bytes is
 * short while the workspace size is nonzero.
 */
sv_status sv_budget_select(const float* conf, const int32_t* draft_len, int32_t n_req,
                           int32_t k_max, const float* cost, int32_t cost_len, int32_t t_base,
                           int32_t n_bonus, int32_t* kept, int32_t* budget, float* survival,
                           int32_t* dev_error, void* ws, size_t ws_bytes, void* stream);

/*
 * sv_budget_allocate — the slots of a budget B sized elsewhere.
 *
 * agentlens page, section "DSpark 신뢰도 스케줄링 메커니즘", item Execution
 * Pipeline: the budget is sized from the previous step's (double-buffered)
 * confidences, ahead of the step, and only the allocation of slots to
 * requests runs with the current step's.  Here B is read on the device
 * (budget_in, e.g. the `budget` sv_budget_select wrote for the previous
 * step's confidences, copied to the host asynchronously to size the batch)
 * and the current confidences are ranked exactly as in sv_budget_select
 * steps 1-2; kept[r] = number of request r's slots among the first
 * min(max(B, 0), total slots).
 *
 * conf, draft_len, survival, ws: as sv_budget_select (same workspace size).
 * budget_in:   [1] int32 device, B (a B above the current slot count keeps
 *              every slot; B <= 0 keeps none).
 * kept:        [n_req] int32 out.
 * budget_used: [1] int32 out, the B applied after clamping, or NULL.
 * Launch: the rank kernel of sv_budget_select, then one 1024-thread
 * workgroup that counts each request's slots ranked below B.
 * Errors: SV_ERR_NULL (budget_in always; conf, draft_len, kept when there
 * are requests); SV_ERR_SHAPE as sv_budget_select; SV_ERR_WORKSPACE.
 */
sv_status sv_budget_allocate(const float* conf, const int32_t* draft_len, int32_t n_req,
                             int32_t k_max, const int32_t* budget_in, int32_t* kept,
                             int32_t* budget_used, float* survival, int32_t* dev_error, void* ws,
                             size_t ws_bytes, void* stream);

/*
 * sv_budget_select_pack, sv_budget_allocate_pack — sv_budget_select (or
 * sv_budget_allocate) followed by sv_pack_varlen in one launch fewer: the
 * workgroup that counts the kept slots also writes the packed layout
 * (cu_rows, row_req, row_pos, packed_tokens exactly as sv_pack_varlen
 * documents them, from the kept counts it has just computed, which are
 * always inside [0, k_max]).  Arguments, sizes, workspace and errors: the
 * union of the two calls' (the budget's limits apply).
 */
sv_status sv_budget_select_pack(const float* conf, const int32_t* draft_len, int32_t n_req,
                                int32_t k_max, const float* cost, int32_t cost_len,
                                int32_t t_base, int32_t n_bonus, const int32_t* last_token,
                                const int32_t* draft_tokens, int32_t* kept, int32_t* budget,
                                float* survival, int32_t* cu_rows, int32_t* row_req,
                                int32_t* row_pos, int32_t* packed_tokens, int32_t* dev_error,
                                void* ws, size_t ws_bytes, void* stream);
sv_status sv_budget_allocate_pack(const float* conf, const int32_t* draft_len, int32_t n_req,
                                  int32_t k_max, const int32_t* budget_in,
                                  const int32_t* last_token, const int32_t* draft_tokens,
                                  int32_t* kept, int32_t* budget_used, float* survival,
                                  int32_t* cu_rows, int32_t* row_req, int32_t* row_pos,
                                  int32_t* packed_tokens, int32_t* dev_error, void* ws,
                                  size_t ws_bytes, void* stream);

/*
 * sv_uniform_k_select — one draft length K for the whole batch, by goodput.
 *
 * "Hardware-Aware Dynamic Speculative Decoding (DSD), feat. Cohere", section
 * "동적 추측 디코딩(DSD)의 핵심 아이디어": the number of drafts is chosen per
 * step from the model/hardware interaction by maximising goodput =
 * acceptance length / inter-token latency (more drafts while memory-bound,
 * fewer once compute-bound).  Here, with the survivals s of
 * sv_budget_select (same clamping, fp32 products):
 *   K* = the smallest maximiser over K = 0 .. k_max of
 *        (n_bonus + S(K)) / cost[t_base + T(K)],
 *   S(K) = sum over r of the survivals of r's first min(K, K_r) drafts, taken
 *          exactly as sum(floor(s * 2^40)) * 2^-40, the ratio in fp64;
 *   T(K) = sum over r of min(K, K_r) (drafts verified);
 *   kept[r] = min(K*, K_r).
 * The acceptance length is the FOS page's (section "평균 수락 길이"): one
 * plus the survivals of the drafts verified.
 *
 * conf, draft_len, cost, t_base, n_bonus: as for sv_budget_select.
 * kept:    [n_req] int32 out.   k_out: [1] int32 out (K*).
 * scores:  [k_max + 1] fp64 out (the goodput of every K; -inf where the cost
 *          entry is unusable), or NULL.
 * Launch: one workgroup of 1024 threads; no workspace.
 * Errors: as for sv_budget_select (SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_VALUE);
 * device bits SV_DEV_BAD_DRAFT_LEN, SV_DEV_BAD_COST.
 */
sv_status sv_uniform_k_select(const float* conf, const int32_t* draft_len, int32_t n_req,
                              int32_t k_max, const float* cost, int32_t cost_len, int32_t t_base,
                              int32_t n_bonus, int32_t* kept, int32_t* k_out, double* scores,
                              int32_t* dev_error, void* stream);

/*
 * sv_pack_varlen — lay the kept rows out as one varlen decode batch.
 *
 * agentlens page, section "기술적 구현 및 CUDA Graphs", item Graph Capture:
 * one decode shape holds 1 .. k+1 query tokens per request; section "설정 및
 * 재현": capacity (k + 1) * max_num_seq.  Request r owns rows
 * cu_rows[r] .. cu_rows[r] + kept[r]; row 0 of a request carries its last
 * emitted token, row i > 0 draft token i-1.
 *
 * kept:          [n_req] int32 (clamped into [0, k_max], SV_DEV_BAD_KEPT).
 * last_token:    [n_req] int32.   draft_tokens: [n_req, k_max] int32.
 * cu_rows:       [n_req + 1] int32 out: exclusive scan of kept + 1.
 * row_req, row_pos, packed_tokens: [n_req * (k_max + 1)] int32 out; rows past
 *                cu_rows[n_req] hold -1.
 * Launch: one workgroup.
 * Errors: SV_ERR_NULL; SV_ERR_SHAPE if n_req < 0 or k_max < 0 or the
 * capacity overflows int32.
 */
sv_status sv_pack_varlen(const int32_t* kept, const int32_t* last_token,
                         const int32_t* draft_tokens, int32_t n_req, int32_t k_max,
                         int32_t* cu_rows, int32_t* row_req, int32_t* row_pos,
                         int32_t* packed_tokens, int32_t* dev_error, void* stream);

/*
 * sv_verify — full-vocabulary verification of every kept row.
 *
 * FOS page, section "추측 디코딩이란": drafts are checked from the front and
 * accepted up to the first mismatch; the target's own token fills the
 * mismatch, or follows the last draft if all are accepted (bonus token;
 * section "평균 수락 길이").  Section "속도, 메모리, 정확도에 주는 영향", row
 * 정확도: with rejection sampling the output law is the target's.
 *
 * Stochastic mode, per request r with b = cu_rows[r+1] - cu_rows[r] - 1:
 *   p_j = softmax(target row j / T), q_j = softmax(draft row j / T);
 *   (u_j, v_j) = Philox4x32-10 (Salmon et al., SC'11) with key = seed and
 *   counter = (r, j, step low, step high), u from word 0 and v from word 1 as
 *   (word >> 8) * 2^-24;
 *   draft d_j accepted iff u_j < min(1, p_j(d_j) / q_j(d_j)), the ratio taken
 *   as 2^(log2 p - log2 q) so that it stays exact-to-rounding when p or q
 *   falls below fp32's normal range (q = 0 accepts iff p > 0);
 *   L = first rejected position, else b;
 *   token at L: if L < b, the smallest id x with C(x) > v_L * W for
 *   C the running sum of w = max(0, p_L - q_L) and W its total (p_L if W = 0);
 *   if L = b, the same draw from p_b.
 * Greedy mode: d_j accepted iff it is the argmax (lowest id on ties) of target
 *   row j; the token at L is that argmax.  draft_logits may be NULL and
 *   temperature is ignored.
 *
 * target_logits: packed target rows, row cu_rows[r] + j at
 *                target_logits + (cu_rows[r] + j) * target_ld elements;
 *                target_rows = rows the buffer holds (a request whose rows
 *                pass it is a fault, SV_DEV_BAD_CU_ROWS).
 * draft_logits:  [n_req * k_max] draft rows, row r*k_max + j at stride
 *                draft_ld elements (stochastic mode).
 * dtype:         SV_BF16 or SV_F32, same for both.  Rows whose start is
 *                16-byte aligned take the vector path; others are read
 *                element-wise (slower, same result).
 * draft_tokens:  [n_req, k_max] int32 (ids outside [0, vocab) at a kept
 *                position: SV_DEV_BAD_TOKEN).
 * cu_rows:       [n_req + 1] int32, as written by sv_pack_varlen.
 * temperature:   > 0 and finite in stochastic mode.
 * out_tokens:    [n_req, k_max + 1] int32: accepted drafts, then the token at
 *                L, then -1.   out_accepted: [n_req] int32 L.
 * out_p_draft, out_q_draft: [n_req, k_max] fp32 p_j(d_j), q_j(d_j) for j < b,
 *                -1 elsewhere and in greedy mode; may be NULL.
 * out_residual_mass: [n_req] fp32 sum max(0, p_L - q_L) when a draft was
 *                rejected in stochastic mode, else -1; may be NULL.
 * out_q_entropy, out_q_max: [n_req, k_max] fp32 draft-row features for
 *                acceptance prediction (same page, section "켜는 방법과
 *                제약": a drafter without a confidence head gets its
 *                estimates from a small model over its logits): the entropy
 *                in bits, -sum_x q_j(x) log2 q_j(x), and the largest
 *                probability max_x q_j(x) of draft row j, for j < b in
 *                stochastic mode; -1 elsewhere and in greedy mode (draft rows
 *                are not read there).  May be NULL; when either is given,
 *                pass 1 accumulates them while it streams the draft rows.
 * A faulty request (any SV_DEV_* bit of its own) writes -1 to all of its
 * outputs.
 * Numerics: fp32.  Each probability carries a few fp32 ulps of error (the
 * exp2 instruction, the rounding of its exponent, the normalisations), which
 * p(d), q(d) and the residual mass inherit; the token at L is the draw above
 * with its cumulative weights rounded to fp32.  Repeated calls with the same
 * arguments give bit-identical outputs, on any stream.
 * ws:            sv_verify_workspace_bytes(n_req, k_max) bytes (per-part
 *                row statistics and draft-row feature sums passed from the
 *                first launch to the second).  Calls that overlap in time
 *                must not share a workspace.
 * Launch: two kernels.  Pass 1: one 512-thread workgroup per candidate row
 * part, rows cut into ceil(vocab / 131072) <= 8 parts (n_req * (2*k_max + 1)
 * rows stochastic, n_req * (k_max + 1) greedy; workgroups beyond the kept
 * rows do nothing).  Pass 2: one workgroup per request (1024 threads
 * stochastic, 64 greedy) merges the parts, decides and draws.
 * Errors: SV_ERR_NULL; SV_ERR_DTYPE; SV_ERR_SHAPE if n_req < 0, k_max outside
 * [0, SV_MAX_DRAFT], n_req * (2*k_max + 1) > SV_MAX_VERIFY_SLOTS, vocab outside
 * [1, SV_MAX_VOCAB], a stride below vocab or target_rows < 0; SV_ERR_VALUE for
 * an unknown mode or a bad temperature; SV_ERR_WORKSPACE.
 */
sv_status sv_verify(const void* target_logits, int64_t target_ld, int64_t target_rows,
                    const void* draft_logits, int64_t draft_ld, sv_dtype dtype, int32_t vocab,
                    const int32_t* draft_tokens, const int32_t* cu_rows, int32_t n_req,
                    int32_t k_max, sv_mode mode, float temperature, uint64_t seed, uint64_t step,
                    int32_t* out_tokens, int32_t* out_accepted, float* out_p_draft,
                    float* out_q_draft, float* out_residual_mass, float* out_q_entropy,
                    float* out_q_max, int32_t* dev_error, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * sv_verify_stages — sv_verify split at its two launches, for callers that
 * time or schedule the passes on their own.  Same arguments and checks as
 * sv_verify, plus `stages`: 1 = pass 1 only (row statistics into ws),
 * 2 = pass 2 only (decisions, draws and outputs from the ws that a pass 1
 * with the same arguments filled earlier on the same stream; the draft-row
 * features are read back only if that pass 1 was asked for them too), 3 =
 * both (identical to sv_verify).  Errors: as sv_verify; SV_ERR_VALUE if
 * stages is not 1, 2 or 3.
 */
sv_status sv_verify_stages(const void* target_logits, int64_t target_ld, int64_t target_rows,
                           const void* draft_logits, int64_t draft_ld, sv_dtype dtype,
                           int32_t vocab, const int32_t* draft_tokens, const int32_t* cu_rows,
                           int32_t n_req, int32_t k_max, sv_mode mode, float temperature,
                           uint64_t seed, uint64_t step, int32_t* out_tokens,
                           int32_t* out_accepted, float* out_p_draft, float* out_q_draft,
                           float* out_residual_mass, float* out_q_entropy, float* out_q_max,
                           int32_t* dev_error, void* ws, size_t ws_bytes, int32_t stages,
                           void* stream);

/*
 * sv_verify_noalloc — sv_verify for callers that cannot allocate device
 * memory: work recorded under HIP graph capture, serving loops and harnesses
 * that forbid hipMalloc.  Same arguments, checks, kernels and results as
 * sv_verify, without ws and ws_bytes: the per-part statistics pass 1 hands to
 * pass 2 live in a static device array of SV_NOALLOC_WS_BYTES bytes, one copy
 * per GPU, held from the library's load until the process ends (its address
 * is looked up once per GPU, on the first call there).  The call allocates
 * and frees nothing.
 * Limit: sv_verify_workspace_bytes(n_req, k_max) <= SV_NOALLOC_WS_BYTES, i.e.
 * n_req * ((2*k_max + 1) * 128 + k_max * 64) bytes (256 requests x 7 drafts:
 * 606,208 bytes; at most 3542 requests at k_max = 7); larger batches return
 * SV_ERR_CAPACITY before anything is launched.
 * Sharing: every call on one GPU uses that GPU's one array, which keeps the
 * last call's contents (nothing in it needs clearing: every record pass 2
 * reads is written by pass 1 of the same call).  Calls that overlap in time
 * on one GPU (two streams, or two host threads) race on the array and must
 * be serialised by the caller.  `stream` selects the GPU (NULL: the current
 * device's null stream).
 * Errors: those of sv_verify except SV_ERR_WORKSPACE; SV_ERR_CAPACITY as
 * above; SV_ERR_LAUNCH if the runtime cannot name the stream's device or the
 * array's address, or refuses a launch.
 */
sv_status sv_verify_noalloc(const void* target_logits, int64_t target_ld, int64_t target_rows,
                            const void* draft_logits, int64_t draft_ld, sv_dtype dtype,
                            int32_t vocab, const int32_t* draft_tokens, const int32_t* cu_rows,
                            int32_t n_req, int32_t k_max, sv_mode mode, float temperature,
                            uint64_t seed, uint64_t step, int32_t* out_tokens,
                            int32_t* out_accepted, float* out_p_draft, float* out_q_draft,
                            float* out_residual_mass, float* out_q_entropy, float* out_q_max,
                            int32_t* dev_error, void* stream);

/*
 * Acceptance statistics and online calibration of the per-position
 * acceptance estimates.  FOS page, section "켜는 방법과 제약" (for model-based
 * drafters without a confidence head, a small logistic model predicts
 * acceptance from the draft's logits and is recalibrated while serving from
 * the verification results), the measurement checklist (per-position
 * acceptance rate and mean acceptance length) and section "평균 수락 길이".
 *
 * Outcomes come from sv_verify: request r kept b_r = cu_rows[r+1] - cu_rows[r]
 * - 1 drafts and accepted L_r = accepted[r]; it verified positions
 * 0 .. min(L_r, b_r - 1), accepting those below L_r and rejecting L_r when
 * L_r < b_r.  Requests with L_r < 0 (a fault) or outside
 * 0 <= L_r <= b_r <= k_max are skipped.
 */

/*
 * sv_accept_stats — add one step's counters to running totals (device
 * uint64, caller-owned, never cleared by the library).
 * attempted[j] += requests that verified position j; accepted_at[j] += those
 * that accepted it ([k_max] each: accepted_at/attempted is position j's
 * conditional acceptance); totals[0] += requests counted, totals[1] += their
 * emitted tokens sum(L_r + 1) (totals[1] / totals[0] = mean acceptance
 * length).  One workgroup.  Errors: SV_ERR_SHAPE (n_req < 0, k_max outside
 * [0, SV_MAX_DRAFT]), SV_ERR_NULL.
 */
sv_status sv_accept_stats(const int32_t* accepted, const int32_t* cu_rows, int32_t n_req,
                          int32_t k_max, uint64_t* attempted, uint64_t* accepted_at,
                          uint64_t* totals, void* stream);

/*
 * The logistic acceptance model over three features of draft row j of
 * request r, all reported by sv_verify:
 *   c_j = sigmoid(alpha_j + beta_1 x_1 + beta_2 x_2 + beta_3 x_3),
 *   x_1 = log2 q_j(d_j) clamped to [-64, 0] (q <= 0 or NaN reads as -64),
 *   x_2 = the row's entropy in bits clamped to [0, 64],
 *   x_3 = the row's largest probability clamped to [0, 1]
 * (NaN or a negative value reads as 0 for x_2 and x_3, and so does a feature
 * array passed as NULL).  theta = [alpha_0 .. alpha_{k_max-1}, beta_1,
 * beta_2, beta_3]: device fp32 [k_max + 3].
 * q_draft, q_entropy, q_max: [n_req, k_max] fp32, sv_verify's out_q_draft,
 * out_q_entropy and out_q_max (q_entropy and q_max may be NULL).
 */

/*
 * sv_calibrate_update — one gradient step of the model on the mean log-loss
 * of the verified positions: theta -= lr * grad / N (theta updated in
 * place).  count_out: [1] int32, N (or NULL).  One workgroup; fixed-order
 * reductions (deterministic).  Errors: SV_ERR_SHAPE, SV_ERR_NULL,
 * SV_ERR_VALUE (lr negative or not finite).
 */
sv_status sv_calibrate_update(float* theta, const float* q_draft, const float* q_entropy,
                              const float* q_max, const int32_t* accepted,
                              const int32_t* cu_rows, int32_t n_req, int32_t k_max, float lr,
                              int32_t* count_out, void* stream);

/*
 * sv_calibrate_predict — conf[r, j] = c_j of request r: the per-position
 * acceptance estimates sv_budget_select and sv_uniform_k_select read.
 * conf: [n_req, k_max] fp32.  Errors: SV_ERR_SHAPE, SV_ERR_NULL.
 */
sv_status sv_calibrate_predict(const float* theta, const float* q_draft, const float* q_entropy,
                               const float* q_max, int32_t n_req, int32_t k_max, float* conf,
                               void* stream);

/*
 * sv_philox_uniforms — the (u, v) pairs sv_verify draws, for inspection.
 * u, v: [n_req, n_pos] fp32 out for counters (r, j, step) with r < n_req,
 * j < n_pos.  Errors: SV_ERR_NULL; SV_ERR_SHAPE if a size is negative.
 */
sv_status sv_philox_uniforms(uint64_t seed, uint64_t step, int32_t n_req, int32_t n_pos,
                             float* u, float* v, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSPECVERIFY_H */

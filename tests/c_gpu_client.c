/* A plain C caller of the whole path on a GPU, through the C ABI alone:
 * budget and packing in one call, the target rows gathered into the packed
 * layout the offsets describe (what a varlen target forward writes), then
 * stochastic verification.  It reads its inputs from the files a test writes
 * into the directory given as argv[1] and prints every output, one
 * "name value..." line each; tests/test_c_client.py checks them against the
 * oracle.
 *
 * Files (little-endian, row-major): meta.txt "n k V cost_len t_base n_bonus
 * seed step temperature"; conf.f32 [n, k]; draft_len.i32 [n]; cost.f32
 * [cost_len]; last_token.i32 [n]; draft_tokens.i32 [n, k]; target.f32
 * [n * (k + 1), V] (request r's row j at r * (k + 1) + j); draft.f32 [n * k, V]. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "libspecverify.h"

#define CHECK_HIP(x)                                                               \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
            return 1;                                                              \
        }                                                                          \
    } while (0)
#define CHECK_SV(x)                                                                \
    do {                                                                           \
        sv_status s_ = (x);                                                        \
        if (s_ != SV_OK) {                                                         \
            fprintf(stderr, "%s failed: %s\n", #x, sv_status_str(s_));             \
            return 1;                                                              \
        }                                                                          \
    } while (0)

static void* read_file(const char* dir, const char* name, size_t bytes) {
    char path[4096];
    FILE* f;
    void* buf;
    snprintf(path, sizeof path, "%s/%s", dir, name);
    f = fopen(path, "rb");
    if (!f) return NULL;
    buf = malloc(bytes ? bytes : 1);
    if (buf && fread(buf, 1, bytes, f) != bytes) {
        free(buf);
        buf = NULL;
    }
    fclose(f);
    return buf;
}

static hipError_t upload(void** dev, const void* host, size_t bytes) {
    hipError_t e = hipMalloc(dev, bytes ? bytes : 4);
    if (e != hipSuccess || bytes == 0) return e;
    return hipMemcpy(*dev, host, bytes, hipMemcpyHostToDevice);
}

static void print_i32(const char* name, const int32_t* v, long count) {
    long i;
    printf("%s", name);
    for (i = 0; i < count; ++i) printf(" %d", (int)v[i]);
    printf("\n");
}

static void print_f32(const char* name, const float* v, long count) {
    long i;
    printf("%s", name);
    for (i = 0; i < count; ++i) printf(" %.9g", (double)v[i]);
    printf("\n");
}

int main(int argc, char** argv) {
    int n, k, V, cost_len, t_base, n_bonus;
    unsigned long long seed, step;
    float tau;
    char path[4096];
    FILE* meta;
    float *conf, *cost, *target, *draft, *packed, *p_d, *q_d, *resid;
    int32_t *draft_len, *last_token, *draft_tokens, *kept, *cu, *tokens, *accepted;
    int32_t budget = -1, dev_error = 0;
    void *d_conf, *d_dl, *d_cost, *d_last, *d_dtok, *d_kept, *d_budget, *d_err, *d_bws;
    void *d_cu, *d_row_req, *d_row_pos, *d_packed_tok, *d_target, *d_draft, *d_vws;
    void *d_tokens, *d_accepted, *d_p, *d_q, *d_resid;
    size_t bws, vws, row_bytes;
    long rows, cap, r, j;

    if (argc != 2) {
        fprintf(stderr, "usage: %s <input directory>\n", argv[0]);
        return 2;
    }
    snprintf(path, sizeof path, "%s/meta.txt", argv[1]);
    meta = fopen(path, "r");
    if (!meta || fscanf(meta, "%d %d %d %d %d %d %llu %llu %f", &n, &k, &V, &cost_len, &t_base,
                        &n_bonus, &seed, &step, &tau) != 9) {
        fprintf(stderr, "cannot read %s\n", path);
        return 2;
    }
    fclose(meta);
    if (n < 1 || k < 1 || V < 1 || cost_len < 1 || (long)n * (k + 1) * V > (1L << 28)) {
        fprintf(stderr, "sizes out of range\n");
        return 2;
    }
    cap = (long)n * (k + 1);
    row_bytes = (size_t)V * sizeof(float);
    conf = read_file(argv[1], "conf.f32", (size_t)n * k * sizeof(float));
    draft_len = read_file(argv[1], "draft_len.i32", (size_t)n * sizeof(int32_t));
    cost = read_file(argv[1], "cost.f32", (size_t)cost_len * sizeof(float));
    last_token = read_file(argv[1], "last_token.i32", (size_t)n * sizeof(int32_t));
    draft_tokens = read_file(argv[1], "draft_tokens.i32", (size_t)n * k * sizeof(int32_t));
    target = read_file(argv[1], "target.f32", (size_t)cap * row_bytes);
    draft = read_file(argv[1], "draft.f32", (size_t)n * k * row_bytes);
    if (!conf || !draft_len || !cost || !last_token || !draft_tokens || !target || !draft) {
        fprintf(stderr, "missing input file\n");
        return 2;
    }

    /* budget and packing */
    bws = sv_budget_workspace_bytes(n, k);
    CHECK_HIP(upload(&d_conf, conf, (size_t)n * k * sizeof(float)));
    CHECK_HIP(upload(&d_dl, draft_len, (size_t)n * sizeof(int32_t)));
    CHECK_HIP(upload(&d_cost, cost, (size_t)cost_len * sizeof(float)));
    CHECK_HIP(upload(&d_last, last_token, (size_t)n * sizeof(int32_t)));
    CHECK_HIP(upload(&d_dtok, draft_tokens, (size_t)n * k * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_kept, (size_t)n * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_budget, sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_err, sizeof(int32_t)));
    CHECK_HIP(hipMemset(d_err, 0, sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_bws, bws));
    CHECK_HIP(hipMalloc(&d_cu, (size_t)(n + 1) * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_row_req, (size_t)cap * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_row_pos, (size_t)cap * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_packed_tok, (size_t)cap * sizeof(int32_t)));
    CHECK_SV(sv_budget_select_pack(d_conf, d_dl, n, k, d_cost, cost_len, t_base, n_bonus,
                                   d_last, d_dtok, d_kept, d_budget, NULL, d_cu, d_row_req,
                                   d_row_pos, d_packed_tok, d_err, d_bws, bws, NULL));
    kept = malloc((size_t)n * sizeof(int32_t));
    cu = malloc((size_t)(n + 1) * sizeof(int32_t));
    if (!kept || !cu) return 2;
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(kept, d_kept, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(cu, d_cu, (size_t)(n + 1) * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&budget, d_budget, sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&dev_error, d_err, sizeof(int32_t), hipMemcpyDeviceToHost));
    printf("budget %d\n", (int)budget);
    printf("budget_dev_error %d\n", (int)dev_error);
    print_i32("kept", kept, n);
    print_i32("cu_rows", cu, n + 1);

    /* the packed target rows: request r's rows 0..kept[r] at cu[r] + j */
    rows = cu[n];
    if (rows < n || rows > cap) {
        fprintf(stderr, "bad packed row count %ld\n", rows);
        return 1;
    }
    packed = malloc((size_t)rows * row_bytes);
    if (!packed) return 2;
    for (r = 0; r < n; ++r)
        for (j = 0; j <= kept[r]; ++j)
            memcpy((char*)packed + (size_t)(cu[r] + j) * row_bytes,
                   (const char*)target + (size_t)(r * (k + 1) + j) * row_bytes, row_bytes);

    /* verification */
    vws = sv_verify_workspace_bytes(n, k);
    CHECK_HIP(upload(&d_target, packed, (size_t)rows * row_bytes));
    CHECK_HIP(upload(&d_draft, draft, (size_t)n * k * row_bytes));
    CHECK_HIP(hipMalloc(&d_vws, vws));
    CHECK_HIP(hipMalloc(&d_tokens, (size_t)cap * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_accepted, (size_t)n * sizeof(int32_t)));
    CHECK_HIP(hipMalloc(&d_p, (size_t)n * k * sizeof(float)));
    CHECK_HIP(hipMalloc(&d_q, (size_t)n * k * sizeof(float)));
    CHECK_HIP(hipMalloc(&d_resid, (size_t)n * sizeof(float)));
    CHECK_HIP(hipMemset(d_err, 0, sizeof(int32_t)));
    CHECK_SV(sv_verify(d_target, V, rows, d_draft, V, SV_F32, V, d_dtok, d_cu, n, k,
                       SV_STOCHASTIC, tau, (uint64_t)seed, (uint64_t)step, d_tokens, d_accepted,
                       d_p, d_q, d_resid, NULL, NULL, d_err, d_vws, vws, NULL));
    tokens = malloc((size_t)cap * sizeof(int32_t));
    accepted = malloc((size_t)n * sizeof(int32_t));
    p_d = malloc((size_t)n * k * sizeof(float));
    q_d = malloc((size_t)n * k * sizeof(float));
    resid = malloc((size_t)n * sizeof(float));
    if (!tokens || !accepted || !p_d || !q_d || !resid) return 2;
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(tokens, d_tokens, (size_t)cap * sizeof(int32_t), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(accepted, d_accepted, (size_t)n * sizeof(int32_t),
                        hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(p_d, d_p, (size_t)n * k * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(q_d, d_q, (size_t)n * k * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(resid, d_resid, (size_t)n * sizeof(float), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&dev_error, d_err, sizeof(int32_t), hipMemcpyDeviceToHost));
    printf("verify_dev_error %d\n", (int)dev_error);
    print_i32("tokens", tokens, cap);
    print_i32("accepted", accepted, n);
    print_f32("p_draft", p_d, (long)n * k);
    print_f32("q_draft", q_d, (long)n * k);
    print_f32("residual_mass", resid, n);
    return 0;
}

// Varlen packing of the kept verify rows on one workgroup (gfx950).
//
// agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive Verification)",
// section "기술적 구현 및 CUDA Graphs" (Graph Capture: any mix of 1 .. k+1
// query tokens per request in one decode shape) and section "설정 및 재현"
// (capacity (k+1) * max_num_seq).  Request r owns rows cu_rows[r] ..
// cu_rows[r] + kept[r]; row 0 carries the last emitted token, row i > 0 draft
// i-1; capacity rows past cu_rows[n] hold -1.
//
// One workgroup walks the requests in chunks of 1024 with a running carry;
// each thread writes its own request's rows as soon as it knows its offset.
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kPackThreads = 1024;
constexpr int kPackWaves = kPackThreads / kWave;

__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const int32_t* __restrict__ kept, const int32_t* __restrict__ last_token,
    const int32_t* __restrict__ draft_tokens, int n_req, int k_max, int32_t* __restrict__ cu_rows,
    int32_t* __restrict__ row_req, int32_t* __restrict__ row_pos,
    int32_t* __restrict__ packed_tokens, int32_t* dev_error) {
    __shared__ int32_t wave_tot[kPackWaves];
    __shared__ int32_t err_s;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    if (tid == 0) err_s = 0;
    int carry = 0;
    int my_err = 0;
    for (int base = 0; base < n_req; base += kPackThreads) {
        const int r = base + tid;
        int b = 0;
        if (r < n_req) {
            b = kept[r];
            if (b < 0 || b > k_max) {
                my_err |= SV_DEV_BAD_KEPT;
                b = b < 0 ? 0 : k_max;
            }
        }
        const int cnt = r < n_req ? b + 1 : 0;
        const int incl = wave_incl_sum_dpp<int>(cnt, lane);
        __syncthreads();  // wave_tot reuse across chunks
        if (lane == kWave - 1) wave_tot[wave] = incl;
        __syncthreads();
        if (wave == 0) {
            int t = lane < kPackWaves ? wave_tot[lane] : 0;
            t = wave_incl_sum_dpp<int>(t, lane);
            if (lane < kPackWaves) wave_tot[lane] = t;
        }
        __syncthreads();
        const int start = carry + (wave == 0 ? 0 : wave_tot[wave - 1]) + incl - cnt;
        if (r < n_req) {
            cu_rows[r] = start;
            row_req[start] = r;
            row_pos[start] = 0;
            packed_tokens[start] = last_token[r];
            for (int i = 1; i <= b; ++i) {
                row_req[start + i] = r;
                row_pos[start + i] = i;
                packed_tokens[start + i] = draft_tokens[(int64_t)r * k_max + (i - 1)];
            }
        }
        carry += wave_tot[kPackWaves - 1];
    }
    if (tid == 0) cu_rows[n_req] = carry;
    const int cap = n_req * (k_max + 1);
    for (int row = carry + tid; row < cap; row += kPackThreads) {
        row_req[row] = -1;
        row_pos[row] = -1;
        packed_tokens[row] = -1;
    }
    if (my_err) atomicOr(&err_s, my_err);
    __syncthreads();
    if (tid == 0) raise_error(dev_error, err_s);
}

}  // namespace

hipError_t launch_pack(const int32_t* kept, const int32_t* last_token,
                       const int32_t* draft_tokens, int n_req, int k_max, int32_t* cu_rows,
                       int32_t* row_req, int32_t* row_pos, int32_t* packed_tokens,
                       int32_t* dev_error, hipStream_t stream) {
    hipLaunchKernelGGL(pack_kernel, dim3(1), dim3(kPackThreads), 0, stream, kept, last_token,
                       draft_tokens, n_req, k_max, cu_rows, row_req, row_pos, packed_tokens,
                       dev_error);
    return hipGetLastError();
}

}  // namespace sv

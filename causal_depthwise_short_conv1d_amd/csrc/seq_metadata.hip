// Token -> (request, first row) metadata in one launch -- Inkling sconv.py,
// sconv_seq_metadata / _seq_metadata_kernel.  Every row below num_actual gets
// its owning request (the largest j < num_reqs with qsl[j] <= row, so that
// empty requests are passed over) and that request's first row; rows in
// [num_actual, num_padded) get 0 / 0.  One lane per row; the binary search
// reads query_start_loc through the caches (a few KiB at most).
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kMetaBlock = 256;

__global__ __launch_bounds__(kMetaBlock) void seq_metadata_kernel(
    const int32_t *qsl, int32_t num_reqs, int32_t num_actual, int32_t num_padded,
    int32_t *seq_idx, int32_t *query_start) {
    const int32_t t = int32_t(blockIdx.x) * kMetaBlock + int32_t(threadIdx.x);
    if (t >= num_padded) return;
    int32_t r = 0, q = 0;
    if (t < num_actual) {
        r = seq_search(qsl, num_reqs, t);
        q = qsl[r];
    }
    seq_idx[t] = r;
    query_start[t] = q;
}

}  // namespace

hipError_t launch_seq_metadata(const int32_t *qsl, int32_t num_reqs, int32_t num_actual,
                               int32_t num_padded, int32_t *seq_idx, int32_t *query_start,
                               hipStream_t s) {
    const dim3 grid(uint32_t((int64_t(num_padded) + kMetaBlock - 1) / kMetaBlock));
    seq_metadata_kernel<<<grid, dim3(kMetaBlock), 0, s>>>(qsl, num_reqs, num_actual,
                                                          num_padded, seq_idx, query_start);
    return hipGetLastError();
}

}  // namespace sconv

// Decode-time update: every batch entry feeds seqlen (usually 1) new tokens
// that continue from its cached state, then the state is shifted to hold the
// last width-1 inputs -- tokenspeed causal_conv1d.py, causal_conv1d_update /
// _causal_conv1d_update_kernel (non-speculative path).
//
// The work is tiny (about 100 KiB at dim 4096) and latency-bound: one lane
// per (entry, channel), all loads of a lane independent of each other, so a
// launch costs one memory round trip plus the stores.  Each lane reads its
// inputs before writing its outputs, which makes out == x (in place, as the
// page computes) safe.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kUpdBlock = 256;

template <int W, bool SILU>
__global__ __launch_bounds__(kUpdBlock) void update_decode_kernel(UpdParams p, uint32_t cblocks) {
    const uint32_t b = blockIdx.x / cblocks;
    const int32_t c = int32_t((blockIdx.x % cblocks) * kUpdBlock + threadIdx.x);
    if (int32_t(b) >= p.batch || c >= p.dim) return;
    const int64_t line = p.cache_idx ? int64_t(p.cache_idx[b]) : int64_t(b);
    if ((p.cache_idx && line == p.pad_slot_id) || line < 0 || line >= p.num_lines) return;

    uint16_t *st = p.cs + line * p.cs_sl + int64_t(c) * p.cs_sd;
    uint16_t win[W - 1];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) win[k] = st[k * p.cs_st];
    float wf[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wf[k] = bf_one(p.w[int64_t(c) * p.w_sd + k]);
    const float b0 = p.bias ? bf_one(p.bias[c]) : 0.0f;

    const uint16_t *xp = p.x + int64_t(b) * p.x_sb + int64_t(c) * p.x_sd;
    uint16_t *op = p.out + int64_t(b) * p.o_sb + int64_t(c) * p.o_sd;
    for (int32_t t = 0; t < p.seqlen; ++t) {
        const uint16_t xb = xp[int64_t(t) * p.x_st];
        float acc = b0;
#pragma unroll
        for (int k = 0; k < W - 1; ++k) acc = __builtin_fmaf(wf[k], bf_one(win[k]), acc);
        acc = __builtin_fmaf(wf[W - 1], bf_one(xb), acc);
        op[int64_t(t) * p.o_st] = to_bf16(act<SILU>(acc));
#pragma unroll
        for (int k = 0; k + 1 < W - 1; ++k) win[k] = win[k + 1];
        win[W - 2] = xb;
    }
#pragma unroll
    for (int k = 0; k < W - 1; ++k) st[k * p.cs_st] = win[k];
}

template <int W>
hipError_t launch_w(const UpdParams &p, bool silu, hipStream_t s) {
    const uint32_t cblocks = uint32_t((p.dim + kUpdBlock - 1) / kUpdBlock);
    const dim3 grid(cblocks * uint32_t(p.batch)), block(kUpdBlock);
    if (silu) update_decode_kernel<W, true><<<grid, block, 0, s>>>(p, cblocks);
    else update_decode_kernel<W, false><<<grid, block, 0, s>>>(p, cblocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_update_decode(const UpdParams &p, int width, bool silu, hipStream_t s) {
    switch (width) {
        case 2: return launch_w<2>(p, silu, s);
        case 3: return launch_w<3>(p, silu, s);
        case 4: return launch_w<4>(p, silu, s);
        case 5: return launch_w<5>(p, silu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

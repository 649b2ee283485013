// Varlen forward for channel-contiguous (T, dim) storage -- the layout the
// tokenspeed causal_conv1d.py launcher (causal_conv1d_fn) requires for its
// packed continuous-batching input.
//
// Decomposition: a wave owns a [bt tokens x 512 channels] tile; each lane
// owns 8 adjacent channels (one 16-byte vector per token row, 1 KiB per wave
// per row, fully coalesced) and walks the tile's tokens keeping the previous
// width-1 inputs of its channels in registers.  All lanes of a wave share the
// token, so the sequence bookkeeping is wave-uniform.
//
// Ownership of a sequence's history: the tile holding the sequence's first
// token processes the first width-1 tokens of that sequence (spilling past
// its end when needed) and the next tile skips them.  That tile is the only
// reader of the cached state and writes the new state right after reading
// it, so the state write cannot overtake another reader.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kUnroll = 4;

template <int W, bool SILU>
__device__ __forceinline__ void run_segment(const FwdClParams &p, const SeqInfo &si,
                                            int64_t b, int64_t e, bool head, int32_t c0,
                                            int nv, const float (&wf)[W][kVec],
                                            const float (&bf)[kVec]) {
    float win[W - 1][kVec];
    if (head) {
        uint16_t h[W - 1][kVec];
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
#pragma unroll
            for (int ch = 0; ch < kVec; ++ch)
                h[k][ch] = (si.init && ch < nv)
                               ? p.sb.cs[si.line * p.sb.cs_sl + int64_t(c0 + ch) * p.sb.cs_sd +
                                         k * p.sb.cs_st]
                               : uint16_t(0);
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
#pragma unroll
            for (int ch = 0; ch < kVec; ++ch) win[k][ch] = bf_one(h[k][ch]);
        if (p.sb.cs) {
            // new state = the last width-1 entries of (history ++ sequence)
            const int64_t L = si.end - si.start;
            uint16_t nh[W - 1][kVec];
#pragma unroll
            for (int k = 0; k < W - 1; ++k) {
                const int64_t m = L + k;
                if (m < W - 1) {
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) nh[k][ch] = h[m][ch];
                } else {
                    const u32x4 v = ld8_partial(p.x + (si.start + m - (W - 1)) * p.x_st + c0, nv);
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) nh[k][ch] = lane_elem(v, ch);
                }
            }
#pragma unroll
            for (int k = 0; k < W - 1; ++k)
#pragma unroll
                for (int ch = 0; ch < kVec; ++ch)
                    if (ch < nv)
                        p.sb.cs[si.line * p.sb.cs_sl + int64_t(c0 + ch) * p.sb.cs_sd +
                                k * p.sb.cs_st] = nh[k][ch];
        }
    } else {
        // interior: the previous width-1 rows belong to the same sequence
#pragma unroll
        for (int k = 0; k < W - 1; ++k) {
            const u32x4 v = ld8_partial(p.x + (b - (W - 1) + k) * p.x_st + c0, nv);
            unpack8(v, win[k]);
        }
    }

    for (int64_t t = b; t < e; t += kUnroll) {
        const int n = (e - t) < kUnroll ? int(e - t) : kUnroll;
        u32x4 xv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            if (u < n) xv[u] = ld8_partial(p.x + (t + u) * p.x_st + c0, nv);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u < n) {
                float xf[kVec], o[kVec];
                unpack8(xv[u], xf);
#pragma unroll
                for (int ch = 0; ch < kVec; ++ch) {
                    float acc = bf[ch];
#pragma unroll
                    for (int k = 0; k < W - 1; ++k) acc = __builtin_fmaf(wf[k][ch], win[k][ch], acc);
                    acc = __builtin_fmaf(wf[W - 1][ch], xf[ch], acc);
                    o[ch] = act<SILU>(acc);
                }
                st8_partial(p.out + (t + u) * p.o_st + c0, pack8(o), nv, true);
#pragma unroll
                for (int k = 0; k + 1 < W - 1; ++k)
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) win[k][ch] = win[k + 1][ch];
#pragma unroll
                for (int ch = 0; ch < kVec; ++ch) win[W - 2][ch] = xf[ch];
            }
        }
    }
}

template <int W, bool SILU>
__global__ __launch_bounds__(kClWavesPerBlock * kWaveSize) void fwd_chanlast_kernel(FwdClParams p) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = threadIdx.x / kWaveSize;
    const uint32_t wt = xcd_tile(blockIdx.x, gridDim.x) * kClWavesPerBlock + wave;
    const int32_t slab = int32_t(wt % uint32_t(p.n_slabs));
    const int32_t tt = int32_t(wt / uint32_t(p.n_slabs));
    if (tt >= p.n_tiles) return;

    const int32_t c0 = slab * kSlab + lane * kVec;
    int nv = p.dim - c0;
    nv = nv < 0 ? 0 : (nv > kVec ? kVec : nv);

    float wf[W][kVec], bf[kVec];
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) {
        const bool ok = ch < nv;
#pragma unroll
        for (int k = 0; k < W; ++k) wf[k][ch] = ok ? bf_one(p.w[int64_t(c0 + ch) * p.w_sd + k]) : 0.0f;
        bf[ch] = (ok && p.bias) ? bf_one(p.bias[c0 + ch]) : 0.0f;
    }

    const int64_t T = p.sb.total_T;
    const int64_t tile_start = int64_t(tt) * p.bt;
    const int64_t tile_end = (tile_start + p.bt) < T ? (tile_start + p.bt) : T;
    int32_t s = seq_search(p.sb.qsl, p.sb.batch, tile_start);
    int64_t t = tile_start;
    while (t < tile_end) {
        const SeqInfo si = seq_info(p.sb, p.sb.qsl, s);
        if (si.end <= t) {                 // finished (or empty) sequence
            if (++s >= p.sb.batch) break;
            continue;
        }
        if (si.start > t) {                // tokens no sequence covers
            t = si.start;
            continue;
        }
        int64_t b = t;
        int64_t e = si.end < tile_end ? si.end : tile_end;
        const int64_t tl0 = t - si.start;
        if (tl0 >= 1 && tl0 <= W - 2) {    // this sequence's head belongs to the previous tile
            const int64_t hend = si.start + (W - 1);
            b = hend < si.end ? hend : si.end;
        }
        const bool head = (b == si.start);
        if (head) {                        // finish the head even past the tile end
            const int64_t hend = si.start + (W - 1) < si.end ? si.start + (W - 1) : si.end;
            e = e > hend ? e : hend;
        }
        if (!si.skip && b < e && nv > 0) run_segment<W, SILU>(p, si, b, e, head, c0, nv, wf, bf);
        t = b > e ? b : e;
        if (t >= si.end && ++s >= p.sb.batch) break;
    }
}

template <int W>
hipError_t launch_w(const FwdClParams &p, bool silu, hipStream_t s) {
    const uint64_t waves = uint64_t(p.n_tiles) * uint64_t(p.n_slabs);
    const uint32_t blocks = uint32_t((waves + kClWavesPerBlock - 1) / kClWavesPerBlock);
    const dim3 grid(blocks), block(kClWavesPerBlock * kWaveSize);
    if (silu) fwd_chanlast_kernel<W, true><<<grid, block, 0, s>>>(p);
    else fwd_chanlast_kernel<W, false><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_chanlast(const FwdClParams &p, int width, bool silu, hipStream_t s) {
    switch (width) {
        case 2: return launch_w<2>(p, silu, s);
        case 3: return launch_w<3>(p, silu, s);
        case 4: return launch_w<4>(p, silu, s);
        case 5: return launch_w<5>(p, silu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

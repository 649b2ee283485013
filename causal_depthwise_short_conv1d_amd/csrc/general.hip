// General-stride kernels: the varlen forward and the paged insert + conv for
// every layout the vector kernels do not take -- any non-negative element
// strides (sliced, offset, pitched, broadcast or transposed views), bases
// aligned only to their element size, stream widths and D offsets of any
// size, and tensors of 2^32 elements or more (all offsets are 64-bit).
//
// They compute exactly what the vector kernels compute (same tap order:
// bf16 pairs on the dot2 unit, the odd last tap by fma, one rounding), one
// output element per lane:
//   * forward (tokenspeed causal_conv1d.py, causal_conv1d_fn): a tile is
//     kGenTile lanes along the axis of x with the smaller stride -- tokens of
//     one channel, or channels of one token -- so each of a wave's loads
//     covers consecutive addresses whenever the layout has a unit axis.  A
//     lane reads its width taps straight from x (neighbouring lanes share
//     them through the cache).  The lane holding a sequence's first token is
//     the single reader and writer of its history: it computes the first
//     min(L, width-1) outputs, which are the only ones that read the state,
//     and then writes the new state; the lanes of the next width-2 tokens do
//     nothing.
//   * paged step (Inkling sconv.py, fused_sconv): a tile is one token row of
//     kGenTile channels of one stream; the lane resolves its token's request,
//     reads each tap from x (rows inside the forward) or from the cache
//     through block_table (earlier positions), and inserts its input.  The
//     cache is read only at positions before the request's first row, which
//     no row of the call writes, so the result is the snapshot the page
//     defines.
// Grids are capped at kGenMaxBlocks workgroups; a workgroup walks tiles
// blockIdx.x, blockIdx.x + gridDim.x, ... until none are left.
#include "sconv_device.h"

namespace sconv {

namespace {

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// bias + sum_j w[j] * u[j]: taps in bf16 pairs on the dot2 unit (exact
// products, fp32 sums), then the odd last tap, as the vector kernels order
// them.
template <int W>
__device__ __forceinline__ float taps(const uint16_t (&u)[W], const uint16_t (&w)[W], float bias) {
    float acc = bias;
#pragma unroll
    for (int q = 0; q < W / 2; ++q)
        acc = dot2(uint32_t(u[2 * q]) | (uint32_t(u[2 * q + 1]) << 16),
                   uint32_t(w[2 * q]) | (uint32_t(w[2 * q + 1]) << 16), acc);
    if constexpr (W & 1) acc = __builtin_fmaf(bf_one(w[W - 1]), bf_one(u[W - 1]), acc);
    return acc;
}

template <int W, bool SILU>
__global__ __launch_bounds__(kGenTile) void fwd_general_kernel(FwdGenParams p) {
    constexpr int H = W - 1;
    __shared__ int32_t s_qsl[kQslLdsMax];
    const bool use_lds = p.sb.batch + 1 <= kQslLdsMax;
    if (use_lds) {
        for (int i = threadIdx.x; i <= p.sb.batch; i += kGenTile) s_qsl[i] = p.sb.qsl[i];
        __syncthreads();
    }
    const int32_t *qsl = use_lds ? s_qsl : p.sb.qsl;

    for (int64_t tile = blockIdx.x; tile < p.n_tiles; tile += gridDim.x) {
        const int64_t major = tile / p.tiles_per_line;
        const int64_t minor = (tile - major * p.tiles_per_line) * kGenTile + threadIdx.x;
        const int64_t c = p.lanes_on_tokens ? major : minor;
        const int64_t t = p.lanes_on_tokens ? minor : major;
        if (c >= p.dim || t >= p.T) continue;
        const SeqInfo si = seq_info(p.sb, qsl, seq_search(qsl, p.sb.batch, t));
        if (si.skip || t < si.start || t >= si.end) continue;
        const int64_t i = t - si.start;           // position inside the sequence
        if (i > 0 && i < H) continue;             // the sequence's head lane computes it

        uint16_t w[W];
#pragma unroll
        for (int j = 0; j < W; ++j) w[j] = p.w[c * p.w_sd + j];
        const float b = p.bias ? bf_one(p.bias[c]) : 0.0f;
        const uint16_t *xc = p.x + c * p.x_sd;

        if (i >= H) {                             // every tap inside the sequence
            uint16_t u[W];
#pragma unroll
            for (int j = 0; j < W; ++j) u[j] = xc[(t - H + j) * p.x_st];
            p.out[c * p.o_sd + t * p.o_st] = to_bf16(act<SILU>(taps<W>(u, w, b)));
            continue;
        }

        // Head lane: u = history ++ x of the sequence; u[k] for k < H is the
        // cached history (zero without one), u[k] for k >= H is
        // x[start + k - H].
        const int64_t L = si.end - si.start;
        uint16_t *line = p.sb.cs ? p.sb.cs + si.line * p.sb.cs_sl + c * p.sb.cs_sd : nullptr;
        uint16_t h[H];
#pragma unroll
        for (int k = 0; k < H; ++k) h[k] = si.init ? line[k * p.sb.cs_st] : uint16_t(0);
        // outputs 0 .. min(L, H) - 1: output o reads u[o .. o + H]
#pragma unroll
        for (int o = 0; o < H; ++o) {
            if (o < L) {
                uint16_t u[W];
#pragma unroll
                for (int j = 0; j < W; ++j)
                    u[j] = o + j < H ? h[o + j < H ? o + j : 0] : xc[(si.start + o + j - H) * p.x_st];
                p.out[c * p.o_sd + (si.start + o) * p.o_st] = to_bf16(act<SILU>(taps<W>(u, w, b)));
            }
        }
        // new state: the last H entries of u, u[L + k]
        if (p.sb.cs) {
            uint16_t nh[H];
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int64_t e = L + k;
                uint16_t v = 0;
#pragma unroll
                for (int m = 0; m < H; ++m)
                    if (e == m) v = h[m];
                nh[k] = e < H ? v : xc[(si.start + e - H) * p.x_st];
            }
#pragma unroll
            for (int k = 0; k < H; ++k) line[k * p.sb.cs_st] = nh[k];
        }
    }
}

template <int W, bool SILU, bool RESID>
__global__ __launch_bounds__(kGenTile) void paged_general_kernel(PagedGenParams p) {
    constexpr int H = W - 1;
    int64_t actual = p.num_reqs > 0 ? int64_t(p.qsl[p.num_reqs]) : 0;
    actual = actual < 0 ? 0 : (actual > p.T ? p.T : actual);

    for (int64_t tile = blockIdx.x; tile < p.n_tiles; tile += gridDim.x) {
        const int64_t t = tile / p.cols;
        const int32_t col = int32_t(tile - t * p.cols);
        int si = 0;                               // the tile's stream
#pragma unroll
        for (int k = 1; k < kMaxPagedStreams; ++k)
            if (k < p.num_streams && p.s[k].slab0 <= col) si = k;
        const PagedStream &st = p.s[si];
        const int64_t c = int64_t(col - st.slab0) * kGenTile + threadIdx.x;
        if (c >= st.C) continue;

        const int64_t slot = p.slot[t];
        const int64_t pos = p.pos[t];
        const bool pad = slot < 0 || t >= actual;
        const uint16_t xt = st.x[t * st.x_st + c];
        // the channel's element of a cache slot: head c / ws, D off_s + c % ws
        const int64_t cidx = (c / st.ws) * p.c_sh + st.off_s + c % st.ws;

        float acc = 0.0f;
        if (!pad) {
            const int32_t r = seq_search(p.qsl, p.num_reqs, t);
            const int64_t qs = p.qsl[r];
            uint16_t u[W], w[W];
#pragma unroll
            for (int j = 0; j < W; ++j) {
                w[j] = st.w[c * st.w_sd + j];
                const int64_t src = pos - H + j;  // absolute position of tap j
                const int64_t row = t - H + j;    // its row, if inside this forward
                uint16_t v = 0;
                if (src >= 0) {
                    if (row >= qs && row >= 0) {     // (row >= 0 holds for a valid query_start_loc)
                        v = st.x[row * st.x_st + c];
                    } else {
                        const int64_t lblk = src / p.block_size;
                        if (lblk < p.max_blocks) {
                            const int64_t blk = p.bt[int64_t(r) * p.bt_sr + lblk];
                            if (blk >= 0 && blk < p.num_blocks)
                                v = p.cache[blk * p.c_sb + (src % p.block_size) * p.c_sn + cidx];
                        }
                    }
                }
                u[j] = v;
            }
            acc = taps<W>(u, w, st.bias ? bf_one(st.bias[c]) : 0.0f);
        }
        float o = act<SILU>(acc);
        if constexpr (RESID) o += bf_one(xt);
        st.out[t * st.o_st + c] = to_bf16(o);
        if (!pad) {
            const int64_t blk = slot / p.block_size;
            if (blk < p.num_blocks)
                p.cache[blk * p.c_sb + (slot % p.block_size) * p.c_sn + cidx] = xt;
        }
    }
}

dim3 gen_grid(int64_t n_tiles) {
    return dim3(uint32_t(n_tiles < kGenMaxBlocks ? n_tiles : kGenMaxBlocks));
}

template <int W>
hipError_t fwd_w(const FwdGenParams &p, bool silu, hipStream_t s) {
    if (silu) fwd_general_kernel<W, true><<<gen_grid(p.n_tiles), kGenTile, 0, s>>>(p);
    else fwd_general_kernel<W, false><<<gen_grid(p.n_tiles), kGenTile, 0, s>>>(p);
    return hipGetLastError();
}

template <int W, bool SILU>
hipError_t paged_ws(const PagedGenParams &p, bool residual, hipStream_t s) {
    if (residual) paged_general_kernel<W, SILU, true><<<gen_grid(p.n_tiles), kGenTile, 0, s>>>(p);
    else paged_general_kernel<W, SILU, false><<<gen_grid(p.n_tiles), kGenTile, 0, s>>>(p);
    return hipGetLastError();
}

template <int W>
hipError_t paged_w(const PagedGenParams &p, bool silu, bool residual, hipStream_t s) {
    return silu ? paged_ws<W, true>(p, residual, s) : paged_ws<W, false>(p, residual, s);
}

}  // namespace

hipError_t launch_fwd_general(const FwdGenParams &p, int width, bool silu, hipStream_t s) {
    switch (width) {
        case 2: return fwd_w<2>(p, silu, s);
        case 3: return fwd_w<3>(p, silu, s);
        case 4: return fwd_w<4>(p, silu, s);
        case 5: return fwd_w<5>(p, silu, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_paged_general(const PagedGenParams &p, int width, bool silu, bool residual,
                                hipStream_t s) {
    switch (width) {
        case 2: return paged_w<2>(p, silu, residual, s);
        case 3: return paged_w<3>(p, silu, residual, s);
        case 4: return paged_w<4>(p, silu, residual, s);
        case 5: return paged_w<5>(p, silu, residual, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

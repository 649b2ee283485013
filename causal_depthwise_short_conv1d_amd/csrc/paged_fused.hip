// Paged sliding-window insert + depthwise causal conv in one launch --
// Inkling sconv.py, fused_sconv / _fused_sconv_kernel, with the
// token -> request search of its _seq_metadata_kernel done in-kernel.
//
// Decomposition: a wave owns [kPagedBT tokens x 512 channels]; each lane owns
// 8 adjacent channels, which lie in one head (ws % 8 == 0), so every cache
// access of a lane is one 16-byte vector at D offset off_s + c % ws.
// Latency, not bandwidth, is the hazard here (decode rows are pure gathers
// through block_table): the per-token metadata of the tile -- slot,
// position, request, and for every tap whether it is zero, a row of x, or a
// cached slot -- is resolved first, one token per lane, all loads in
// parallel; the token loop then broadcasts it with readlane and keeps
// kUnroll tokens' loads in flight.
//
// Taps inside the forward read the immutable x (the previous width-1 rows
// are kept in registers); only pre-forward positions are read from the
// cache, so the inserts of this launch are never read back by it.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kUnroll = 4;
constexpr int kTapZero = -2;    // position before 0, pad row, or unmapped block
constexpr int kTapIntra = -1;   // a row of x inside this forward

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), lane));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(uint64_t(v) >> 32)), lane));
    return int64_t((uint64_t(hi) << 32) | lo);
}

template <int W, bool SILU, bool RESID>
__global__ __launch_bounds__(kPagedWavesPerBlock * kWaveSize) void paged_fused_kernel(PagedParams p) {
    __shared__ int32_t s_qsl[kQslLdsMax];
    const bool use_lds = p.num_reqs + 1 <= kQslLdsMax;
    if (use_lds) {
        for (int i = threadIdx.x; i <= p.num_reqs; i += blockDim.x) s_qsl[i] = p.qsl[i];
        __syncthreads();
    }
    const int32_t *qsl = use_lds ? s_qsl : p.qsl;

    const int lane = threadIdx.x & (kWaveSize - 1);
    // wave index within the block: uniform, and marked so for the compiler
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t wt = blockIdx.x * kPagedWavesPerBlock + wave;
    const int32_t slab = int32_t(wt % uint32_t(p.n_slabs));
    const int32_t tt = int32_t(wt / uint32_t(p.n_slabs));
    if (tt >= p.n_tiles) return;

    const int32_t c0 = slab * kSlab + lane * kVec;
    int nv = p.C - c0;
    nv = nv < 0 ? 0 : (nv > kVec ? kVec : nv);
    const int32_t cc = nv > 0 ? c0 : 0;                 // keeps idle lanes' addresses in range
    const int64_t lane_off = int64_t(cc / p.ws) * p.c_sh + (p.off_s + cc % p.ws);

    float wf[W][kVec], bf[kVec];
#pragma unroll
    for (int ch = 0; ch < kVec; ++ch) {
        const bool ok = ch < nv;
#pragma unroll
        for (int k = 0; k < W; ++k) wf[k][ch] = ok ? bf_one(p.w[int64_t(c0 + ch) * p.w_sd + k]) : 0.0f;
        bf[ch] = (ok && p.bias) ? bf_one(p.bias[c0 + ch]) : 0.0f;
    }

    const int64_t tile_start = int64_t(tt) * kPagedBT;
    const int n_tok = int((p.T - tile_start) < kPagedBT ? (p.T - tile_start) : kPagedBT);
    int64_t actual = p.num_reqs > 0 ? int64_t(qsl[p.num_reqs]) : 0;
    actual = actual < 0 ? 0 : (actual > p.T ? p.T : actual);

    // Per-token metadata, token tile_start + lane in lane `lane`.
    int64_t m_slot = -1;
    int32_t m_pad = 1;
    int64_t m_qs = 0;
    int64_t m_tap[W - 1];
#pragma unroll
    for (int j = 0; j < W - 1; ++j) m_tap[j] = kTapZero;
    if (lane < n_tok) {
        const int64_t t = tile_start + lane;
        m_slot = p.slot[t];
        const int64_t pos = p.pos[t];
        m_pad = (m_slot < 0 || t >= actual) ? 1 : 0;
        if (!m_pad) {
            const int32_t r = seq_search(qsl, p.num_reqs, t);
            m_qs = qsl[r];
#pragma unroll
            for (int j = 0; j < W - 1; ++j) {
                const int64_t src = pos - (W - 1) + j;
                const int64_t row = t - (W - 1) + j;
                if (src < 0) continue;
                if (row >= m_qs) { m_tap[j] = kTapIntra; continue; }
                const int64_t lblk = src / p.block_size;
                if (lblk >= p.max_blocks) continue;
                const int64_t blk = p.bt[int64_t(r) * p.bt_sr + lblk];
                if (blk < 0 || blk >= p.num_blocks) continue;
                m_tap[j] = blk * p.block_size + src % p.block_size;
            }
        }
    }

    // Previous width-1 rows of x for the tile's first tokens; rows before
    // the first token's request are never an intra tap of this tile.
    const int64_t qs0 = readlane64(m_qs, 0);
    float win[W - 1][kVec];
#pragma unroll
    for (int k = 0; k < W - 1; ++k) {
        const int64_t row = tile_start - (W - 1) + k;
        if (row >= 0 && row >= qs0) {
            const u32x4 v = ld8_partial(p.x + row * p.x_st + cc, nv);
            unpack8(v, win[k]);
        } else {
#pragma unroll
            for (int ch = 0; ch < kVec; ++ch) win[k][ch] = 0.0f;
        }
    }
    // Lanes past the last channel (nv == 0) stay active: they may hold token
    // metadata that the loop below reads with readlane.  Their memory
    // accesses are empty (nv == 0).
    for (int u0 = 0; u0 < n_tok; u0 += kUnroll) {
        u32x4 xv[kUnroll];
        u32x4 g[kUnroll][W - 1];
        int64_t taps[kUnroll][W - 1];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u0 + u < n_tok) {
                const int64_t t = tile_start + u0 + u;
                xv[u] = ld8_partial(p.x + t * p.x_st + cc, nv);
#pragma unroll
                for (int j = 0; j < W - 1; ++j) {
                    taps[u][j] = readlane64(m_tap[j], u0 + u);
                    if (taps[u][j] >= 0) {
                        const int64_t blk = taps[u][j] / p.block_size;
                        const int64_t n = taps[u][j] % p.block_size;
                        g[u][j] = ld8_partial(p.cache + blk * p.c_sb + n * p.c_sn + lane_off, nv);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (u0 + u < n_tok) {
                const int uu = u0 + u;
                const int64_t t = tile_start + uu;
                const int64_t slot = readlane64(m_slot, uu);
                const bool pad = __builtin_amdgcn_readlane(m_pad, uu) != 0;
                float xf[kVec], o[kVec];
                unpack8(xv[u], xf);
                if (!pad) {
                    const int64_t blk = slot / p.block_size;
                    if (blk < p.num_blocks)
                        st8_partial(p.cache + blk * p.c_sb + (slot % p.block_size) * p.c_sn + lane_off,
                                    xv[u], nv, false);
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) o[ch] = bf[ch];
#pragma unroll
                    for (int j = 0; j < W - 1; ++j) {
                        if (taps[u][j] == kTapIntra) {
#pragma unroll
                            for (int ch = 0; ch < kVec; ++ch) o[ch] = __builtin_fmaf(wf[j][ch], win[j][ch], o[ch]);
                        } else if (taps[u][j] >= 0) {
                            float gf[kVec];
                            unpack8(g[u][j], gf);
#pragma unroll
                            for (int ch = 0; ch < kVec; ++ch) o[ch] = __builtin_fmaf(wf[j][ch], gf[ch], o[ch]);
                        }
                    }
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) o[ch] = __builtin_fmaf(wf[W - 1][ch], xf[ch], o[ch]);
                } else {
#pragma unroll
                    for (int ch = 0; ch < kVec; ++ch) o[ch] = 0.0f;
                }
#pragma unroll
                for (int ch = 0; ch < kVec; ++ch) {
                    o[ch] = act<SILU>(o[ch]);
                    if constexpr (RESID) o[ch] += xf[ch];
                }
                st8_partial(p.out + t * p.o_st + cc, pack8(o), nv, true);
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
hipError_t launch_ws(const PagedParams &p, bool residual, hipStream_t s) {
    const uint64_t waves = uint64_t(p.n_tiles) * uint64_t(p.n_slabs);
    const uint32_t blocks = uint32_t((waves + kPagedWavesPerBlock - 1) / kPagedWavesPerBlock);
    const dim3 grid(blocks), block(kPagedWavesPerBlock * kWaveSize);
    if (residual) paged_fused_kernel<W, SILU, true><<<grid, block, 0, s>>>(p);
    else paged_fused_kernel<W, SILU, false><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
}

template <int W>
hipError_t launch_w(const PagedParams &p, bool silu, bool residual, hipStream_t s) {
    return silu ? launch_ws<W, true>(p, residual, s) : launch_ws<W, false>(p, residual, s);
}

}  // namespace

hipError_t launch_paged_fused(const PagedParams &p, int width, bool silu, bool residual,
                              hipStream_t s) {
    switch (width) {
        case 2: return launch_w<2>(p, silu, residual, s);
        case 3: return launch_w<3>(p, silu, residual, s);
        case 4: return launch_w<4>(p, silu, residual, s);
        case 5: return launch_w<5>(p, silu, residual, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

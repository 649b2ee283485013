// Paged sliding-window insert + depthwise causal conv in one launch --
// Inkling sconv.py, fused_sconv / _fused_sconv_kernel, with the
// token -> request search of its _seq_metadata_kernel done in-kernel.  One
// launch may carry several of the conv streams that share the cache (the
// page's module docstring: K, V, attention output and MLP output, each at its
// own D sub-range): they share the per-token metadata and differ only in
// their rows of x / out, taps and D offsets.
//
// Decomposition: a wave owns [BT tokens x 256 channels of one stream]
// (the slabs of all streams are numbered consecutively; BT is 16, or 8 for
// a step that would not fill the chip once with 16); each lane owns
// 4 adjacent channels, which lie in one head (ws % 8 == 0), so every cache
// access of a lane is one 8-byte vector at D offset off_s + c % ws.
// Latency, not bandwidth, is the hazard here (decode rows are pure gathers
// through block_table): the per-token metadata of the tile -- slot,
// position, request, and for every tap whether it is zero, a row of x, or a
// cached slot -- is resolved first, one token per lane, all loads in
// parallel; the token loop then broadcasts it with readlane and keeps
// kPagedUnroll tokens' loads (rows and gathers) in flight.
//
// Every access goes through a buffer descriptor whose base is wave-uniform
// (the tile's rows of x / out, or the physical block of a cached position),
// so the in-flight rows cost no address registers and the descriptors are
// built on the scalar unit.  Taps inside the forward read the immutable x
// (the previous width-1 rows are kept in registers); only pre-forward
// positions are read from the cache, so the inserts of this launch are never
// read back by it.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kPCpl = 4;                        // channels per lane
constexpr int kPSlab = kPagedSlab;              // channels per wave (256)
static_assert(kPSlab == kWaveSize * kPCpl, "paged slab = 64 lanes x 4 channels");
constexpr int kPagedUnroll = 4;                 // tokens in flight per lane
constexpr int kTapZero = -2;                    // position before 0, pad row, unmapped block
constexpr int kTapIntra = -1;                   // a row of x inside this forward
constexpr int kNt = 2;                          // non-temporal cache policy bit

__device__ __forceinline__ int64_t readlane64(int64_t v, int lane) {
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), lane));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(uint64_t(v) >> 32)), lane));
    return int64_t((uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// (channel ch of row a, channel ch of row b) as one bf16 pair.
__device__ __forceinline__ uint32_t cross_pair(const u32x2 &ra, const u32x2 &rb, int ch) {
    const uint32_t da = (ch >> 1) ? ra.y : ra.x, db = (ch >> 1) ? rb.y : rb.x;
    return __builtin_amdgcn_perm(db, da, (ch & 1) ? 0x07060302u : 0x05040100u);
}

typedef unsigned int ui32x2 __attribute__((ext_vector_type(2)));

// A buffer descriptor over `bytes` bytes from `base` (offsets past the end
// read 0 / drop the write).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<void *>(base), short(0),
        int(bytes < 0 ? 0 : (bytes < 0x7fffffff ? bytes : 0x7fffffff)), 0x00020000);
}
template <int AUX>
__device__ __forceinline__ u32x2 ld8(__amdgpu_buffer_rsrc_t r, uint32_t voff, int64_t soff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, int(soff), AUX));
}
template <int AUX>
__device__ __forceinline__ void st8(__amdgpu_buffer_rsrc_t r, uint32_t voff, int64_t soff,
                                    const u32x2 &v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(ui32x2, v), r, voff, int(soff), AUX);
}

template <int W, bool SILU, bool RESID, int BT>
__global__ __launch_bounds__(kPagedWavesPerBlock * kWaveSize) void paged_fused_kernel(PagedParams p) {
    constexpr int H = W - 1;
    __shared__ int32_t s_qsl[kQslLdsMax];
    const int lane = threadIdx.x & (kWaveSize - 1);
    // wave index within the block: uniform, and marked so for the compiler
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t wt = blockIdx.x * kPagedWavesPerBlock + wave;
    const int32_t gslab = int32_t(wt % uint32_t(p.total_slabs));
    const int32_t tt = int32_t(wt / uint32_t(p.total_slabs));
    // the wave's stream: the last one whose first slab is at or below gslab
    int si = 0;
#pragma unroll
    for (int i = 1; i < kMaxPagedStreams; ++i)
        if (i < p.num_streams && p.s[i].slab0 <= gslab) si = i;
    const PagedStream &st = p.s[si];
    const int32_t slab = gslab - st.slab0;

    int32_t c0 = slab * kPSlab + lane * kPCpl;
    const bool active = c0 < st.C;
    if (!active) c0 = 0;                 // idle lane: in-range reads, no writes
    // byte offsets of the lane's 4 channels inside a block and inside a row
    const uint32_t coff = uint32_t((int64_t(c0 / st.ws) * p.c_sh + (st.off_s + c0 % st.ws)) * 2);
    const uint32_t xoff = uint32_t(c0) * 2;
    // store offsets: an idle lane's stores land past every extent (dropped)
    const uint32_t coff_st = active ? coff : kOob;
    const uint32_t xoff_st = active ? xoff : kOob;

    // What depends only on the tile is issued before the query_start_loc
    // staging and the metadata round trips: the token's slot and position
    // (lane = token) and the width-1 rows before the tile.  A wave past the
    // last tile reads clamped addresses and zeros, and stops after the
    // barrier.  (Issuing the tile's own rows here as well was measured: it
    // raises registers and was slower.)
    const int64_t tile_start = int64_t(tt) * BT;
    const int64_t xbase = tile_start >= H ? tile_start - H : 0;
    const __amdgpu_buffer_rsrc_t xr =
        rsrc(st.x + xbase * st.x_st, (p.T - xbase - 1) * st.x_st * 2 + int64_t(st.C) * 2);
    u32x2 win[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const int64_t row = tile_start - H + k;
        win[k] = ld8<kNt>(xr, xoff, row >= 0 ? (row - xbase) * st.x_st * 2 : int64_t(kOob));
    }
    const int64_t t_lane = tile_start + (lane < BT ? lane : 0);
    const int64_t t_safe = t_lane < p.T ? t_lane : p.T - 1;
    const int64_t slot_l = p.slot[t_safe];
    const int64_t pos_l = p.pos[t_safe];

    const bool use_lds = p.num_reqs + 1 <= kQslLdsMax;
    if (use_lds) {
        for (int i = threadIdx.x; i <= p.num_reqs; i += kPagedWavesPerBlock * kWaveSize) s_qsl[i] = p.qsl[i];
        __syncthreads();
    }
    const int32_t *qsl = use_lds ? s_qsl : p.qsl;
    if (tt >= p.n_tiles) return;

    // taps: pair q of channel ch is (w[ch][2q], w[ch][2q+1]); odd last tap fp32
    uint32_t wp[W / 2 > 0 ? W / 2 : 1][kPCpl];
    float wl[kPCpl], bf[kPCpl];
    const Rsrc br = make_rsrc(st.bias ? st.bias : st.w, st.bias ? int64_t(st.C) * 2 : 0);
    if (st.w_sd == W && int64_t(st.C) * W * 2 < kMaxDescriptorSpan &&
        (reinterpret_cast<uintptr_t>(st.w) & 15) == 0 &&
        (reinterpret_cast<uintptr_t>(st.bias) & 7) == 0) {
        // contiguous weights: three or fewer wide loads per lane
        const Rsrc wr = make_rsrc(st.w, int64_t(st.C) * W * 2);
        load_taps4<W>(wr, uint32_t(c0) * W * 2, br, uint32_t(c0) * 2, wp, wl, bf);
    } else {
#pragma unroll
        for (int ch = 0; ch < kPCpl; ++ch) {
            const uint16_t *w = st.w + int64_t(c0 + ch) * st.w_sd;
#pragma unroll
            for (int q = 0; q < W / 2; ++q) wp[q][ch] = uint32_t(w[2 * q]) | (uint32_t(w[2 * q + 1]) << 16);
            wl[ch] = (W & 1) ? bf_one(w[W - 1]) : 0.0f;
            bf[ch] = bf_one(buf_ld16(br, uint32_t(c0 + ch) * 2));
        }
    }

    const int n_tok = int((p.T - tile_start) < BT ? (p.T - tile_start) : BT);
    int64_t actual = p.num_reqs > 0 ? int64_t(qsl[p.num_reqs]) : 0;
    actual = actual < 0 ? 0 : (actual > p.T ? p.T : actual);

    // Per-token metadata, token tile_start + lane in lane `lane`, as 32-bit
    // values (the token loop broadcasts them with readlane, so every cache
    // address below is built on the scalar unit):
    //   m_sblk / m_sn : physical block / slot of the insert (m_sblk < 0: none)
    //   m_tblk / m_tn : per tap, the block / slot of a cached position, or
    //                   kTapIntra (a row of x) or kTapZero.
    // Every lane resolves its token without a branch around a load (a load
    // under a lane-dependent branch would wait before the branch joins, and
    // the block-table reads of a tile's taps would become a chain of round
    // trips): lanes past the tile, pads and taps without a table entry read
    // valid stand-in addresses and their values are discarded.
    const int64_t tl = tile_start + lane;      // the lane's token
    const bool tok = lane < n_tok;
    const int64_t slot = slot_l;
    const int64_t pos = pos_l;
    const int32_t m_pad = (!tok || slot < 0 || tl >= actual) ? 1 : 0;
    const bool ins = !m_pad && slot < p.slot_lim;
    const uint32_t s32 = ins ? uint32_t(slot) : 0u;
    const uint32_t sblk = p.div_n.div(s32);
    const int32_t m_sblk = ins ? int32_t(sblk) : -1;
    const int32_t m_sn = int32_t(s32 - sblk * uint32_t(p.block_size));
    const int32_t r = seq_search(qsl, p.num_reqs, tok ? tl : tile_start);
    const int64_t qs_r = qsl[r];
    const int64_t m_qs = m_pad ? 0 : qs_r;
    int32_t m_tblk[H], m_tn[H], lb_v[H];
    bool need[H];
    bool any = false;
#pragma unroll
    for (int j = 0; j < H; ++j) {
        const int64_t src = pos - H + j;
        const int64_t row = tl - H + j;
        const bool live = !m_pad && src >= 0;
        const bool intra = live && row >= qs_r;
        need[j] = live && !intra && src < p.src_lim;
        any = any || need[j];
        const uint32_t c32 = need[j] ? uint32_t(src) : 0u;
        const uint32_t lb = p.div_n.div(c32);
        lb_v[j] = int32_t(lb);
        m_tn[j] = int32_t(c32 - lb * uint32_t(p.block_size));
        m_tblk[j] = intra ? kTapIntra : kTapZero;
    }
    // Most tiles of a prefill chunk take every tap from x: their waves skip
    // the block-table round trip (a wave-uniform branch).
    if (__builtin_amdgcn_ballot_w64(any) != 0) {
        asm volatile("");                                   // keeps this a branch
        int32_t bt_v[H];
#pragma unroll
        for (int j = 0; j < H; ++j) bt_v[j] = *(need[j] ? p.bt + (int64_t(r) * p.bt_sr + lb_v[j]) : p.bt_rd);
#pragma unroll
        for (int j = 0; j < H; ++j)
            if (need[j] && bt_v[j] >= 0 && bt_v[j] < p.num_blocks) m_tblk[j] = bt_v[j];
    }

    const __amdgpu_buffer_rsrc_t orr =
        rsrc(st.out + tile_start * st.o_st, (p.T - tile_start - 1) * st.o_st * 2 + int64_t(st.C) * 2);

    // Previous width-1 rows of x for the tile's first tokens; rows before
    // the first token's request are never an intra tap of this tile.
    const int64_t qs0 = readlane64(m_qs, 0);
#pragma unroll
    for (int k = 0; k < H; ++k)
        if (tile_start - H + k < qs0) win[k] = u32x2{0u, 0u};

    for (int u0 = 0; u0 < n_tok; u0 += kPagedUnroll) {
        u32x2 xv[kPagedUnroll];
        u32x2 g[kPagedUnroll][H];
#pragma unroll
        for (int u = 0; u < kPagedUnroll; ++u) {
            if (u0 + u < n_tok) {
                const int64_t t = tile_start + u0 + u;
                xv[u] = ld8<kNt>(xr, xoff, (t - xbase) * st.x_st * 2);
#pragma unroll
                for (int j = 0; j < H; ++j) {
                    const int32_t blk = __builtin_amdgcn_readlane(m_tblk[j], u0 + u);
                    g[u][j] = u32x2{0u, 0u};
                    if (blk >= 0) {
                        const int32_t n = __builtin_amdgcn_readlane(m_tn[j], u0 + u);
                        const __amdgpu_buffer_rsrc_t cr = rsrc(p.cache + int64_t(blk) * p.c_sb, p.c_sb * 2);
                        g[u][j] = ld8<0>(cr, coff, int64_t(n) * p.c_sn * 2);
                    }
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kPagedUnroll; ++u) {
            if (u0 + u < n_tok) {
                const int uu = u0 + u;
                const int64_t t = tile_start + uu;
                const bool pad = __builtin_amdgcn_readlane(m_pad, uu) != 0;
                float o[kPCpl];
                if (!pad) {
                    const int32_t sblk = __builtin_amdgcn_readlane(m_sblk, uu);
                    if (sblk >= 0) {
                        const int32_t sn = __builtin_amdgcn_readlane(m_sn, uu);
                        const __amdgpu_buffer_rsrc_t cr = rsrc(p.cache + int64_t(sblk) * p.c_sb, p.c_sb * 2);
                        st8<0>(cr, coff_st, int64_t(sn) * p.c_sn * 2, xv[u]);
                    }
                    // the taps' input rows: a window row, a cached row or zero
                    u32x2 in[W];
#pragma unroll
                    for (int j = 0; j < H; ++j)
                        in[j] = __builtin_amdgcn_readlane(m_tblk[j], uu) == kTapIntra ? win[j] : g[u][j];
                    in[H] = xv[u];
#pragma unroll
                    for (int ch = 0; ch < kPCpl; ++ch) {
                        float acc = bf[ch];
#pragma unroll
                        for (int q = 0; q < W / 2; ++q)
                            acc = dot2(cross_pair(in[2 * q], in[2 * q + 1], ch), wp[q][ch], acc);
                        if constexpr (W & 1) {
                            const uint32_t d = (ch >> 1) ? xv[u].y : xv[u].x;
                            acc = __builtin_fmaf(wl[ch], (ch & 1) ? bf_hi(d) : bf_lo(d), acc);
                        }
                        o[ch] = acc;
                    }
                } else {
#pragma unroll
                    for (int ch = 0; ch < kPCpl; ++ch) o[ch] = 0.0f;
                }
#pragma unroll
                for (int ch = 0; ch < kPCpl; ++ch) {
                    o[ch] = act<SILU>(o[ch]);
                    if constexpr (RESID) {
                        const uint32_t d = (ch >> 1) ? xv[u].y : xv[u].x;
                        o[ch] += (ch & 1) ? bf_hi(d) : bf_lo(d);
                    }
                }
                // a temporal store: the L2 gathers each output row from the
                // pieces the waves of its other slabs write
                st8<0>(orr, xoff_st, (t - tile_start) * st.o_st * 2,
                       u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
#pragma unroll
                for (int k = 0; k + 1 < H; ++k) win[k] = win[k + 1];
                win[H - 1] = xv[u];
            }
        }
    }
}

template <int W, bool SILU>
hipError_t launch_ws(const PagedParams &p, bool residual, hipStream_t s) {
    const uint64_t waves = uint64_t(p.n_tiles) * uint64_t(p.total_slabs);
    const uint32_t blocks = uint32_t((waves + kPagedWavesPerBlock - 1) / kPagedWavesPerBlock);
    const dim3 grid(blocks), block(kPagedWavesPerBlock * kWaveSize);
    if (p.tile_bt == kPagedBTSmall) {
        if (residual) paged_fused_kernel<W, SILU, true, kPagedBTSmall><<<grid, block, 0, s>>>(p);
        else paged_fused_kernel<W, SILU, false, kPagedBTSmall><<<grid, block, 0, s>>>(p);
    } else {
        if (residual) paged_fused_kernel<W, SILU, true, kPagedBT><<<grid, block, 0, s>>>(p);
        else paged_fused_kernel<W, SILU, false, kPagedBT><<<grid, block, 0, s>>>(p);
    }
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

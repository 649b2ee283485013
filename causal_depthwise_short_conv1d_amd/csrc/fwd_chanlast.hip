// Varlen forward for channel-contiguous (T, dim) storage -- the layout the
// tokenspeed causal_conv1d.py launcher (causal_conv1d_fn) requires for its
// packed continuous-batching input.
//
// Decomposition: a wave owns a [bt tokens x 256 channels] tile; each lane
// owns 4 adjacent channels (one 8-byte vector per token row, 512 B per wave
// per row, fully coalesced), keeps 8 rows in flight, and walks the tile's
// tokens keeping the previous width-1 input rows in registers, still packed.
// The taps pair two rows' values of a channel with one byte permute and
// accumulate them with the gfx950 dot2 instruction (exact products, fp32
// sums); keeping rows and weights packed halves the registers, which is what
// sets the occupancy of this streaming kernel.  A pair of consecutive rows
// serves every second output after it, so the tile walk forms each pair
// once.  All lanes of a wave share the token, so the sequence bookkeeping is
// wave-uniform, and a lane with no channels stores through an offset past
// the descriptor's extent rather than behind a branch.
//
// Ownership of a sequence's history: the tile holding the sequence's first
// token processes the first width-1 tokens of that sequence (spilling past
// its end when needed) and the next tile skips them.  That tile is the only
// reader of the cached state and writes the new state right after reading
// it, so the state write cannot overtake another reader.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kUnroll = 8;                     // token rows per batch (two batches in flight)

// A lane's taps for its 4 channels, packed for dot2: pair q of channel ch is
// (w[ch][2q], w[ch][2q+1]); an odd last tap and the bias are fp32.
template <int W>
struct LaneTaps {
    uint32_t wp[W / 2 > 0 ? W / 2 : 1][kCpl];
    float wl[kCpl];
    float b[kCpl];
};

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// (channel ch of row a, channel ch of row b) as one bf16 pair.
__device__ __forceinline__ uint32_t cross_pair(const u32x2 &ra, const u32x2 &rb, int ch) {
    const uint32_t da = (ch >> 1) ? ra.y : ra.x, db = (ch >> 1) ? rb.y : rb.x;
    return __builtin_amdgcn_perm(db, da, (ch & 1) ? 0x07060302u : 0x05040100u);
}

template <bool FULL>
__device__ __forceinline__ u32x2 ld_row(const uint16_t *p, int nv) {
    if constexpr (FULL) {
        return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));   // idle lanes read channel 0
    } else {
        uint32_t e[kCpl];
#pragma unroll
        for (int i = 0; i < kCpl; ++i) e[i] = i < nv ? p[i] : 0u;
        return u32x2{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
    }
}
template <bool FULL>
__device__ __forceinline__ void st_row(uint16_t *p, const u32x2 &v, int nv) {
    if constexpr (FULL) {
        if (nv > 0) __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(p));
    } else {
        const uint32_t w[2] = {v.x, v.y};
#pragma unroll
        for (int i = 0; i < kCpl; ++i)
            if (i < nv) p[i] = uint16_t((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
    }
}
__device__ __forceinline__ uint16_t row_elem(const u32x2 &v, int i) {
    return uint16_t((((i >> 1) ? v.y : v.x) >> ((i & 1) * 16)) & 0xffffu);
}

// Rows of a (T, pitch) bf16 tensor seen through a buffer descriptor based at
// row `base`: a row's byte offset is a wave-uniform scalar, the lane's
// channel offset the only vector operand, so the rows kept in flight cost no
// address registers.  Offsets past `bytes` read 0 / drop the write.
struct Rows {
    __amdgpu_buffer_rsrc_t rsrc;
    int64_t base;
    int64_t pitch;   // bytes
};
__device__ __forceinline__ Rows make_rows(const uint16_t *t, int64_t base, int64_t stride,
                                          int64_t rows_total, int32_t dim) {
    Rows r;
    r.base = base;
    r.pitch = stride * 2;
    // last row's channels end the extent (the row stride may be 0 when T == 1);
    // a base past the last row gives an empty descriptor
    const int64_t bytes = base < rows_total ? (rows_total - base - 1) * r.pitch + int64_t(dim) * 2 : 0;
    r.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(t + base * stride), short(0),
                                               int(bytes < 0x7fffffff ? bytes : 0x7fffffff),
                                               0x00020000);
    return r;
}
constexpr int kNt = 2;   // non-temporal cache policy bit of buffer accesses
__device__ __forceinline__ u32x2 ld_rows(const Rows &r, int64_t row, uint32_t voff) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                         r.rsrc, voff, int((row - r.base) * r.pitch), kNt));
}
__device__ __forceinline__ void st_rows(const Rows &r, int64_t row, uint32_t voff, const u32x2 &v) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned int, v),
                                          r.rsrc, voff, int((row - r.base) * r.pitch), kNt);
}

// Outputs of one token row: the taps' inputs are the H window rows (oldest
// first) and the row itself.
template <int W, bool SILU>
__device__ __forceinline__ u32x2 conv_row(const LaneTaps<W> &tp, const u32x2 (&win)[W - 1],
                                          const u32x2 &x) {
    constexpr int H = W - 1;
    float o[kCpl];
#pragma unroll
    for (int ch = 0; ch < kCpl; ++ch) {
        float acc = tp.b[ch];
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const u32x2 &ra = win[2 * q];
            const u32x2 &rb = (2 * q + 1 < H) ? win[(2 * q + 1) < H ? 2 * q + 1 : 0] : x;
            acc = dot2(cross_pair(ra, rb, ch), tp.wp[q][ch], acc);
        }
        if constexpr (W & 1) {
            const uint32_t d = (ch >> 1) ? x.y : x.x;
            acc = __builtin_fmaf(tp.wl[ch], (ch & 1) ? bf_hi(d) : bf_lo(d), acc);
        }
        o[ch] = act<SILU>(acc);
    }
    return u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

// The 4 cross-row pairs (x[s-1][ch], x[s][ch]) of a lane's channels.
struct RowPairs {
    uint32_t v[kCpl];
};
__device__ __forceinline__ RowPairs row_pairs(const u32x2 &ra, const u32x2 &rb) {
    RowPairs r;
#pragma unroll
    for (int ch = 0; ch < kCpl; ++ch) r.v[ch] = cross_pair(ra, rb, ch);
    return r;
}

// conv_row from pairs: pw[k] holds the pairs ending at row t-(W-2)+k, so
// tap pair q is pw[2q] (the newest, pw[W-2], ends at row t itself).  Each
// pair is formed once and serves every second row after it; the sums are
// the same, in the same order, as conv_row's.
template <int W, bool SILU>
__device__ __forceinline__ u32x2 conv_row_pairs(const LaneTaps<W> &tp,
                                                const RowPairs (&pw)[W - 1], const u32x2 &x) {
    float o[kCpl];
#pragma unroll
    for (int ch = 0; ch < kCpl; ++ch) {
        float acc = tp.b[ch];
#pragma unroll
        for (int q = 0; q < W / 2; ++q) acc = dot2(pw[2 * q].v[ch], tp.wp[q][ch], acc);
        if constexpr (W & 1) {
            const uint32_t d = (ch >> 1) ? x.y : x.x;
            acc = __builtin_fmaf(tp.wl[ch], (ch & 1) ? bf_hi(d) : bf_lo(d), acc);
        }
        o[ch] = act<SILU>(acc);
    }
    return u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

template <int W, bool SILU, bool FULL>
__device__ __forceinline__ void run_segment(const FwdClParams &p, const SeqInfo &si,
                                            int64_t b, int64_t e, bool head, int32_t c0,
                                            int nv, const LaneTaps<W> &tp) {
    constexpr int H = W - 1;
    // Row addresses are wave-uniform (scalar registers); only the lane's
    // channel offset c0 lives in a vector register.
    u32x2 win[H];
    if (head) {
        // One state line through a buffer descriptor: element (c, k) at byte
        // 2*(c*cs_sd + k*cs_st) from the line start (the host bounds a line's
        // extent below 2 GiB); only the lane's channel offsets are vectors.
        // Every load below is issued unconditionally (a descriptor of zero
        // extent, or an out-of-range offset, reads 0), so none waits for
        // another.
        const bool has_cs = p.sb.cs != nullptr;
        const Rsrc cs = make_rsrc(has_cs ? p.sb.cs + si.line * p.sb.cs_sl : p.x,
                                  has_cs ? 0x7fffffff : 0);
        const Rsrc hist = make_rsrc(has_cs ? p.sb.cs + si.line * p.sb.cs_sl : p.x,
                                    has_cs && si.init ? 0x7fffffff : 0);
        uint32_t coff[kCpl];
#pragma unroll
        for (int ch = 0; ch < kCpl; ++ch)
            coff[ch] = ch < nv ? uint32_t(int64_t(c0 + ch) * p.sb.cs_sd * 2) : kOob;
        // the cached history, packed as it arrives
#pragma unroll
        for (int k = 0; k < H; ++k) {
            uint32_t d[2] = {0u, 0u};
#pragma unroll
            for (int ch = 0; ch < kCpl; ++ch)
                d[ch >> 1] |= uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                                  hist, coff[ch], int(k * p.sb.cs_st * 2), 0))
                              << (16 * (ch & 1));
            win[k] = u32x2{d[0], d[1]};
        }
        if (has_cs) {
            // new state = the last width-1 entries of (history ++ sequence):
            // rows of the sequence are loaded (those before its start read 0)
            // and the history entries are picked after the loads
            const int64_t L = si.end - si.start;
            u32x2 tail[H];
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int64_t row = si.start + L + k - H;
                const bool in = row >= si.start;
                const Rows rk = make_rows(p.x, in ? row : si.start, p.x_st, si.end, p.dim);
                tail[k] = FULL ? __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                                     rk.rsrc, in ? uint32_t(c0) * 2 : kOob, 0, 0))
                               : (in ? ld_row<FULL>(p.x + row * p.x_st + c0, nv) : u32x2{0u, 0u});
            }
            u32x2 nh[H];
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int64_t m = L + k;
                u32x2 hv = win[0];
#pragma unroll
                for (int q = 1; q < H; ++q)
                    if (m == q) hv = win[q];
                nh[k] = m < H ? hv : tail[k];
            }
#pragma unroll
            for (int k = 0; k < H; ++k)
#pragma unroll
                for (int ch = 0; ch < kCpl; ++ch)
                    __builtin_amdgcn_raw_buffer_store_b16(row_elem(nh[k], ch), cs, coff[ch],
                                                          int(k * p.sb.cs_st * 2), 0);
        }
    }
    const int64_t base = head ? b : b - H;
    // both descriptors end with the segment: rows past it read 0, store nothing
    const Rows xr = make_rows(p.x, base, p.x_st, e, p.dim);
    const Rows orr = make_rows(p.out, base, p.o_st, e, p.dim);
    const uint32_t voff = uint32_t(c0) * 2;
    if (!head) {
        // interior: the previous width-1 rows belong to the same sequence
#pragma unroll
        for (int k = 0; k < H; ++k)
            win[k] = FULL ? ld_rows(xr, b - H + k, voff)
                          : ld_row<FULL>(p.x + (b - H + k) * p.x_st + c0, nv);
    }

    // Software-pipelined rows: the next kUnroll rows are issued before the
    // current ones are computed (rows past the segment read 0), which keeps a
    // wave's loads in flight through its arithmetic.
    u32x2 xn[kUnroll];
    if constexpr (FULL) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) xn[u] = ld_rows(xr, b + u, voff);
    }
    const uint32_t soff = nv > 0 ? voff : kOob;    // idle lanes store past the extent
    // pw[k] = pairs ending at row t-H+1+k; the newest is formed at each row
    RowPairs pw[H];
#pragma unroll
    for (int k = 0; k + 1 < H; ++k) pw[k] = row_pairs(win[k], win[k + 1]);
    u32x2 prev = win[H - 1];
    for (int64_t t = b; t < e; t += kUnroll) {
        const int n = (e - t) < kUnroll ? int(e - t) : kUnroll;
        u32x2 xv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if constexpr (FULL) {
                xv[u] = xn[u];
                xn[u] = ld_rows(xr, t + kUnroll + u, voff);          // next batch; past the segment: 0
            } else if (u < n) {
                xv[u] = ld_row<FULL>(p.x + (t + u) * p.x_st + c0, nv);
            }
        }
        auto row = [&](int u) {
            pw[H - 1] = row_pairs(prev, xv[u]);
            const u32x2 o = conv_row_pairs<W, SILU>(tp, pw, xv[u]);
            if constexpr (FULL) {
                st_rows(orr, t + u, soff, o);                  // idle lanes: dropped
            } else {
                st_row<FULL>(p.out + (t + u) * p.o_st + c0, o, nv);
            }
#pragma unroll
            for (int k = 0; k + 1 < H; ++k) pw[k] = pw[k + 1];
            prev = xv[u];
        };
        // a whole batch runs unguarded, so the window shifts are renamings
        if (n == kUnroll) {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) row(u);
        } else {
#pragma unroll
            for (int u = 0; u < kUnroll; ++u)
                if (u < n) row(u);
        }
    }
}

// Taps of a lane's channels (slab `slab`, lane channels from c0), loaded
// without branches: channels past dim, and a missing bias, read 0.
template <int W, bool FULL>
__device__ __forceinline__ LaneTaps<W> lane_taps(const FwdClParams &p, int32_t slab, int lane) {
    const int32_t c_lo = slab * kClSlab;
    const int32_t n_ch = p.dim - c_lo < kClSlab ? p.dim - c_lo : kClSlab;
    const Rsrc wr = make_rsrc(p.w + int64_t(c_lo) * p.w_sd, int64_t(n_ch) * p.w_sd * 2);
    const Rsrc br = make_rsrc(p.bias ? p.bias + c_lo : p.w, p.bias ? int64_t(n_ch) * 2 : 0);
    LaneTaps<W> tp;
    const bool wide = FULL && p.w_sd == W && (reinterpret_cast<uintptr_t>(p.w) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(p.bias) & 7) == 0;
    if (wide) {
        // contiguous weights, whole lanes: three or fewer wide loads
        const uint32_t lc0 = uint32_t(lane * kCpl);
        load_taps4<W>(wr, lc0 < uint32_t(n_ch) ? lc0 * W * 2 : kOob, br,
                      lc0 < uint32_t(n_ch) ? lc0 * 2 : kOob, tp.wp, tp.wl, tp.b);
    } else {
#pragma unroll
        for (int ch = 0; ch < kCpl; ++ch) {
            const int32_t lc = lane * kCpl + ch;          // channel within the slab
            const uint32_t wo = lc < n_ch ? uint32_t(int64_t(lc) * p.w_sd * 2) : kOob;
#pragma unroll
            for (int q = 0; q < W / 2; ++q)
                tp.wp[q][ch] = uint32_t(buf_ld16(wr, wo + 4 * q)) |
                               (uint32_t(buf_ld16(wr, wo + 4 * q + 2)) << 16);
            tp.wl[ch] = (W & 1) ? bf_one(buf_ld16(wr, wo + 2 * (W - 1))) : 0.0f;
            tp.b[ch] = bf_one(buf_ld16(br, lc < n_ch ? uint32_t(lc) * 2 : kOob));
        }
    }
    return tp;
}

// Tokens [tile_start, tile_end) of one slab, sequence by sequence: each
// sequence's stretch inside the tile is a segment; a sequence's first
// width-1 tokens belong to the tile that holds its first token.
template <int W, bool SILU, bool FULL>
__device__ __forceinline__ void run_tile(const FwdClParams &p, int64_t tile_start, int64_t tile_end,
                                         int32_t c0, int nv, const LaneTaps<W> &tp) {
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
        // Every lane runs the segment (the control flow stays wave-uniform, so
        // row addresses stay scalar); lanes past the last channel read channel
        // 0 and store nothing.
        if (!si.skip && b < e) run_segment<W, SILU, FULL>(p, si, b, e, head, c0, nv, tp);
        t = b > e ? b : e;
        if (t >= si.end && ++s >= p.sb.batch) break;
    }
}

template <int W, bool SILU, bool FULL>
__global__ __launch_bounds__(kClWavesPerBlock * kWaveSize) void fwd_chanlast_kernel(FwdClParams p) {
    const int lane = threadIdx.x & (kWaveSize - 1);
    // wave index within the block: uniform, and marked so for the compiler
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t wt = blockIdx.x * kClWavesPerBlock + wave;
    const uint32_t tq = p.div_slabs.div(wt);
    const int32_t slab = int32_t(wt - tq * uint32_t(p.n_slabs));
    const int32_t tt = int32_t(tq);
    if (tt >= p.n_tiles) return;

    int32_t c0 = slab * kClSlab + lane * kCpl;
    int nv = p.dim - c0;
    nv = nv < 0 ? 0 : (nv > kCpl ? kCpl : nv);
    if (nv == 0) c0 = 0;                   // idle lane: in-range reads, no writes
    const LaneTaps<W> tp = lane_taps<W, FULL>(p, slab, lane);

    const int64_t T = p.sb.total_T;
    const int64_t tile_start = int64_t(tt) * p.bt;
    const int64_t tile_end = (tile_start + p.bt) < T ? (tile_start + p.bt) : T;
    run_tile<W, SILU, FULL>(p, tile_start, tile_end, c0, nv, tp);
}

// One sequence in (T, dim) storage, whole lanes (dim % 4 == 0), T >= 64.
// A workgroup owns four consecutive 8-row tiles of one 256-channel slab.
// Each wave issues its 8 rows at once; wave 0 also issues the width-1 rows
// before the group.  Every other wave takes its history from the previous
// wave's last width-1 rows, passed through LDS, so a halo costs no second
// HBM read.  (With 8-row tiles, reading every tile's halo from memory costs
// 7% of a copy of the same bytes.)  Group 0's wave 0 holds the sequence's
// head: it reads the cached history and writes the new state (the last
// width-1 rows), and is the only reader and writer of that line.  When the
// sequence does not cover exactly [0, T) (query_start_loc is only known on
// the device), every wave runs the general tile routine on its 8-row tile,
// with the same tiles as fwd_chanlast_kernel at bt = 8.
constexpr int kOneRows = 8;                      // rows per wave
constexpr int kOneGroup = kClWavesPerBlock * kOneRows;   // rows per workgroup

template <int W, bool SILU>
__global__ __launch_bounds__(kClWavesPerBlock * kWaveSize) void fwd_cl_one_kernel(FwdClParams p,
                                                                                  int32_t n_groups) {
    constexpr int H = W - 1;
    __shared__ u32x2 edge[kClWavesPerBlock][H][kWaveSize];   // each wave's last H rows
    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t gq = p.div_slabs.div(blockIdx.x);
    const int32_t slab = int32_t(blockIdx.x - gq * uint32_t(p.n_slabs));
    const int32_t grp = int32_t(gq);
    if (grp >= n_groups) return;                     // the whole workgroup

    int32_t c0 = slab * kClSlab + lane * kCpl;
    const int nv = c0 < p.dim ? kCpl : 0;            // whole lanes
    if (nv == 0) c0 = 0;                             // idle lane: in-range reads, no writes
    const uint32_t voff = uint32_t(c0) * 2;
    const uint32_t soff = nv > 0 ? voff : kOob;
    const int64_t T = p.sb.total_T;
    const int64_t g0 = int64_t(grp) * kOneGroup;
    const int64_t t0 = g0 + int64_t(wave) * kOneRows;

    // The sequence's description comes through the scalar cache (a query
    // every wave of a CU shares).  Whether the sequence covers [0, T) is
    // decided before the rows are issued: rows in flight across the general
    // routine would keep their registers and cost occupancy.
    const SeqInfo si = seq_info_scalar(p.sb, 0);
    const LaneTaps<W> tp = lane_taps<W, true>(p, slab, lane);
    if (!(si.start == 0 && si.end == T)) {           // uniform across the launch
        const int64_t te = t0 + kOneRows < T ? t0 + kOneRows : T;
        if (t0 < T) run_tile<W, SILU, true>(p, t0, te, c0, nv, tp);
        return;
    }
    if (si.skip) return;                             // padded sequence: nothing to write

    // the group's rows and the H before it, through one descriptor based at
    // the first of them (rows past T read 0)
    const int64_t base = g0 >= H ? g0 - H : 0;
    const Rows xr = make_rows(p.x, base, p.x_st, T, p.dim);
    u32x2 xv[kOneRows];
#pragma unroll
    for (int u = 0; u < kOneRows; ++u) xv[u] = ld_rows(xr, t0 + u, voff);
    u32x2 win[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        const int64_t row = g0 - H + k;
        const bool mine = wave == 0 && row >= 0;
        win[k] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(
                     xr.rsrc, mine ? voff : kOob, mine ? int((row - base) * xr.pitch) : 0, kNt));
    }
    // Rows H.. of the wave read only its own rows: they are computed and
    // stored as the rows arrive, before the workgroup waits on its slowest
    // wave for the halos.
    const Rows orr = make_rows(p.out, t0, p.o_st, T, p.dim);
#pragma unroll
    for (int u = H; u < kOneRows; ++u) {
        u32x2 own[H];
#pragma unroll
        for (int k = 0; k < H; ++k) own[k] = xv[u - H + k];
        const u32x2 o = conv_row<W, SILU>(tp, own, xv[u]);
        st_rows(orr, t0 + u, soff, o);     // rows past T, idle lanes: dropped
    }
#pragma unroll
    for (int k = 0; k < H; ++k) edge[wave][k][lane] = xv[kOneRows - H + k];
    __syncthreads();
    if (wave > 0) {
#pragma unroll
        for (int k = 0; k < H; ++k) win[k] = edge[wave - 1][k][lane];
    } else if (grp == 0) {
        // the sequence head: cached history (or zeros), then the new state
        // = rows T-H .. T-1 (T >= 64 > H), written after the history is read
        const bool has_cs = p.sb.cs != nullptr;
        const Rsrc cs = make_rsrc(has_cs ? p.sb.cs + si.line * p.sb.cs_sl : p.x,
                                  has_cs ? 0x7fffffff : 0);
        const Rsrc hist = make_rsrc(has_cs ? p.sb.cs + si.line * p.sb.cs_sl : p.x,
                                    has_cs && si.init ? 0x7fffffff : 0);
        uint32_t coff[kCpl];
#pragma unroll
        for (int ch = 0; ch < kCpl; ++ch)
            coff[ch] = nv > 0 ? uint32_t(int64_t(c0 + ch) * p.sb.cs_sd * 2) : kOob;
        const Rows tr = make_rows(p.x, T - H, p.x_st, T, p.dim);
        u32x2 tail[H];
#pragma unroll
        for (int k = 0; k < H; ++k) {
            uint32_t d[2] = {0u, 0u};
#pragma unroll
            for (int ch = 0; ch < kCpl; ++ch)
                d[ch >> 1] |= uint32_t(__builtin_amdgcn_raw_buffer_load_b16(
                                  hist, coff[ch], int(k * p.sb.cs_st * 2), 0))
                              << (16 * (ch & 1));
            win[k] = u32x2{d[0], d[1]};
            tail[k] = ld_rows(tr, T - H + k, voff);
        }
        if (has_cs) {
#pragma unroll
            for (int k = 0; k < H; ++k)
#pragma unroll
                for (int ch = 0; ch < kCpl; ++ch)
                    __builtin_amdgcn_raw_buffer_store_b16(row_elem(tail[k], ch), cs, coff[ch],
                                                          int(k * p.sb.cs_st * 2), 0);
        }
    }

    // rows 0 .. H-1, whose windows reach into the halo
#pragma unroll
    for (int u = 0; u < H; ++u) {
        const u32x2 o = conv_row<W, SILU>(tp, win, xv[u]);
        st_rows(orr, t0 + u, soff, o);     // rows past T, idle lanes: dropped
#pragma unroll
        for (int k = 0; k + 1 < H; ++k) win[k] = win[k + 1];
        win[H - 1] = xv[u];
    }
}

// The varlen kernel's waves keep their tile's rows in flight; at the six
// or seven resident workgroups per CU that its registers allow, the memory
// queues run deeper than they need to.  An LDS reservation the kernel never
// touches caps a CU at five workgroups (5 x 32 KiB of gfx950's 160 KiB):
// measured 1.6-3% faster on the 64-sequence dim-8192 batch at widths 2-5.
// (The one-sequence kernel is best at full occupancy.)
constexpr uint32_t kClCapLds = 32768;

template <int W>
hipError_t launch_w(const FwdClParams &p, bool silu, hipStream_t s) {
    const uint64_t waves = uint64_t(p.n_tiles) * uint64_t(p.n_slabs);
    const uint32_t blocks = uint32_t((waves + kClWavesPerBlock - 1) / kClWavesPerBlock);
    const dim3 grid(blocks), block(kClWavesPerBlock * kWaveSize);
    const bool full = p.dim % kCpl == 0;
    const int64_t pitch = (p.x_st > p.o_st ? p.x_st : p.o_st) * 2;
    if (p.sb.batch <= 1 && full && p.bt == kOneRows && p.sb.total_T >= 64 &&
        int64_t(kOneGroup + W) * pitch + int64_t(p.dim) * 2 < kMaxDescriptorSpan) {
        // one sequence: four 8-row tiles per workgroup, halos through LDS
        const int32_t n_groups = int32_t((p.sb.total_T + kOneGroup - 1) / kOneGroup);
        const dim3 g(uint32_t(n_groups) * uint32_t(p.n_slabs));
        if (silu) fwd_cl_one_kernel<W, true><<<g, block, 0, s>>>(p, n_groups);
        else fwd_cl_one_kernel<W, false><<<g, block, 0, s>>>(p, n_groups);
        return hipGetLastError();
    }
    if (silu && full) fwd_chanlast_kernel<W, true, true><<<grid, block, kClCapLds, s>>>(p);
    else if (silu) fwd_chanlast_kernel<W, true, false><<<grid, block, kClCapLds, s>>>(p);
    else if (full) fwd_chanlast_kernel<W, false, true><<<grid, block, kClCapLds, s>>>(p);
    else fwd_chanlast_kernel<W, false, false><<<grid, block, kClCapLds, s>>>(p);
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

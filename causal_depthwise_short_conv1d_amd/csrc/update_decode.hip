// Decode-time update: every batch entry feeds seqlen (usually 1) new tokens
// that continue from its cached state -- tokenspeed causal_conv1d.py,
// causal_conv1d_update / _causal_conv1d_update_kernel, including the options
// of that kernel and its docstring:
//   * speculative decoding: num_accepted_tokens moves the start of the
//     history window to column num_accepted - 1 of the state line; without
//     saved windows the line is rewritten as the history minus its oldest
//     input followed by every new input, so that the next call's acceptance
//     count selects the window that ends with the last accepted token;
//   * saved windows: the width-1 inputs that end with token t go to
//     intermediate[b][t] and/or to the line output_state_indices[b][t]
//     (then the state is not updated in place);
//   * ring-buffer states (cache_seqlens): input n of a stream lives at column
//     n mod state_len.
// Without options the state becomes the last width-1 inputs of
// history ++ x.
//
// The work is tiny (about 100 KiB at dim 4096) and latency-bound: one lane
// per (entry, channel); the per-entry option values are wave-uniform loads.
// Each lane reads its history before writing any state and loads a group of
// up to four inputs before storing their outputs, which makes out == x (in
// place, as the page computes) and a saved window aimed at the entry's own
// line safe.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kUpdBlock = 256;
constexpr int kUpdGroup = 4;   // inputs loaded ahead of their outputs

template <int W, bool SILU>
__global__ __launch_bounds__(kUpdBlock) void update_kernel(UpdParams p, uint32_t cblocks) {
    constexpr int H = W - 1;
    const uint32_t b = blockIdx.x / cblocks;            // the entry (workgroup-uniform)
    const int32_t c0 = int32_t((blockIdx.x % cblocks) * kUpdBlock);
    const int32_t c = c0 + int32_t(threadIdx.x);
    if (int32_t(b) >= p.batch || c >= p.dim) return;
    const int32_t nch = p.dim - c0 < kUpdBlock ? p.dim - c0 : kUpdBlock;
    const uint32_t lc = uint32_t(threadIdx.x);

    // The first group of inputs, the taps and the bias go out first, with no
    // branch: they depend on the launch arguments alone.  An input past
    // seqlen re-reads the first one and is discarded; the bias comes through
    // a descriptor based at the workgroup's first channel (none reads 0).
    const int32_t g0 = p.seqlen < kUpdGroup ? p.seqlen : kUpdGroup;
    const uint16_t *xp = p.x + int64_t(b) * p.x_sb + int64_t(c) * p.x_sd;
    uint16_t xv0[kUpdGroup];
#pragma unroll
    for (int i = 0; i < kUpdGroup; ++i) {
        const uint16_t v = xp[int64_t(i < g0 ? i : 0) * p.x_st];   // always a valid input
        xv0[i] = i < g0 ? v : uint16_t(0);
    }
    // (plain loads for the taps: the compiler merges a lane's W adjacent
    // values into one wide load, which a descriptor load would not get)
    float wf[W];
#pragma unroll
    for (int k = 0; k < W; ++k) wf[k] = bf_one(p.w[int64_t(c) * p.w_sd + k]);
    const Rsrc br = make_rsrc(p.bias ? p.bias + c0 : p.w, p.bias ? int64_t(nch) * 2 : 0);
    const float b0 = bf_one(buf_ld16(br, lc * 2));

    // The entry's line and option values, read together through the scalar
    // cache (a missing array reads a stand-in dword of x, discarded).
    const void *sx = reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(p.x) & ~uintptr_t(3));
    const int32_t ci = int32_t(sld_u32(p.cache_idx ? static_cast<const void *>(p.cache_idx + b) : sx));
    const int32_t na = int32_t(sld_u32(p.num_acc ? static_cast<const void *>(p.num_acc + b) : sx));
    const int32_t seen = int32_t(sld_u32(p.ring_seen ? static_cast<const void *>(p.ring_seen + b) : sx));
    const int64_t line = p.cache_idx ? int64_t(ci) : int64_t(b);
    if ((p.cache_idx && line == p.pad_slot_id) || line < 0 || line >= p.num_lines) return;

    const int32_t L = p.state_len;
    int32_t off = 0;     // first history column (speculative decoding)
    int32_t rcol = 0;    // ring: column of the next input
    if (p.num_acc) {
        off = na - 1;
        if (off < 0 || off > L - H) return;
    }
    if (p.ring_seen) {
        if (seen < 0) return;
        rcol = seen % L;
    }
    const bool spec = p.num_acc != nullptr;
    const bool ring = p.ring_seen != nullptr;
    const bool saved = p.inter != nullptr || p.out_idx != nullptr;

    uint16_t *row = p.cs + line * p.cs_sl + int64_t(c) * p.cs_sd;
    uint16_t win[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        int32_t col = off + k;
        if (ring) {
            col = rcol - H + k;
            if (col < 0) col += L;          // H <= L, so one wrap suffices
        }
        win[k] = row[int64_t(col) * p.cs_st];
    }

    // Speculative roll: the line restarts with the history minus its oldest
    // input (the new inputs follow at columns H-1 onward).
    if (spec && !saved) {
#pragma unroll
        for (int k = 0; k + 1 < H; ++k) row[int64_t(k) * p.cs_st] = win[k + 1];
    }

    uint16_t *op = p.out + int64_t(b) * p.o_sb + int64_t(c) * p.o_sd;
    const int32_t ring_from = p.seqlen - L;    // ring: earlier inputs are overwritten anyway
    for (int32_t t0 = 0; t0 < p.seqlen; t0 += kUpdGroup) {
        uint16_t xv[kUpdGroup];
        if (t0 == 0) {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i) xv[i] = xv0[i];
        } else {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i)
                xv[i] = t0 + i < p.seqlen ? xp[int64_t(t0 + i) * p.x_st] : uint16_t(0);
        }
#pragma unroll
        for (int i = 0; i < kUpdGroup; ++i) {
            const int32_t t = t0 + i;
            if (t >= p.seqlen) break;
            float acc = b0;
#pragma unroll
            for (int k = 0; k < H; ++k) acc = __builtin_fmaf(wf[k], bf_one(win[k]), acc);
            acc = __builtin_fmaf(wf[H], bf_one(xv[i]), acc);
            op[int64_t(t) * p.o_st] = to_bf16(act<SILU>(acc));
#pragma unroll
            for (int k = 0; k + 1 < H; ++k) win[k] = win[k + 1];
            win[H - 1] = xv[i];

            if (p.inter) {
                uint16_t *ip = p.inter + int64_t(b) * p.i_sb + int64_t(t) * p.i_st +
                               int64_t(c) * p.i_sd;
#pragma unroll
                for (int k = 0; k < H; ++k) ip[int64_t(k) * p.i_sk] = win[k];
            }
            if (p.out_idx) {
                const int64_t dst = p.out_idx[int64_t(b) * p.oi_sb + int64_t(t) * p.oi_st];
                if (dst >= 0 && dst < p.num_lines) {
                    uint16_t *dp = p.cs + dst * p.cs_sl + int64_t(c) * p.cs_sd;
#pragma unroll
                    for (int k = 0; k < H; ++k) dp[int64_t(k) * p.cs_st] = win[k];
                }
            }
            if (!saved) {
                if (ring) {
                    if (t >= ring_from) row[int64_t(rcol) * p.cs_st] = xv[i];
                    rcol = rcol + 1 == L ? 0 : rcol + 1;
                } else if (spec) {
                    row[int64_t(H - 1 + t) * p.cs_st] = xv[i];
                }
            }
        }
    }
    if (!saved && !ring && !spec) {
#pragma unroll
        for (int k = 0; k < H; ++k) row[int64_t(k) * p.cs_st] = win[k];
    }
}

// The same update with four adjacent channels per lane, for x, out, the
// state lines and the saved windows all unit-stride along dim (the layout a
// verify step keeps its states in).  Every access is then one 8-byte vector
// instead of four 2-byte ones: at one lane per channel the address unit,
// not the bytes, bounds a launch of this size.  The arithmetic and the
// order of every read and write per channel are those of update_kernel.
constexpr int kVecCh = 4;

__device__ __forceinline__ u32x2 ld4ch(const uint16_t *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ void st4ch(uint16_t *p, const u32x2 &v) { *reinterpret_cast<u32x2 *>(p) = v; }
__device__ __forceinline__ float ch_of(const u32x2 &v, int ch) {
    const uint32_t d = (ch >> 1) ? v.y : v.x;
    return (ch & 1) ? bf_hi(d) : bf_lo(d);
}

// WIDE: the weights are packed (row pitch W) and 16-byte aligned, so a lane's
// four channels' taps are 4W adjacent values, read as W/2 16-byte vectors
// (W even) or W 8-byte vectors (W odd).
template <int W, bool SILU, bool WIDE>
__global__ __launch_bounds__(kUpdBlock) void update_vec_kernel(UpdParams p, uint32_t cblocks) {
    constexpr int H = W - 1;
    const uint32_t b = blockIdx.x / cblocks;            // the entry (workgroup-uniform)
    const int32_t c = int32_t(((blockIdx.x % cblocks) * kUpdBlock + threadIdx.x) * kVecCh);
    if (int32_t(b) >= p.batch || c >= p.dim) return;

    const int32_t g0 = p.seqlen < kUpdGroup ? p.seqlen : kUpdGroup;
    const uint16_t *xp = p.x + int64_t(b) * p.x_sb + c;
    u32x2 xv0[kUpdGroup];
#pragma unroll
    for (int i = 0; i < kUpdGroup; ++i) {
        const u32x2 v = ld4ch(xp + int64_t(i < g0 ? i : 0) * p.x_st);   // always a valid input
        xv0[i] = i < g0 ? v : u32x2{0u, 0u};
    }
    float wf[kVecCh][W];
    if constexpr (WIDE) {
        constexpr int kWD = 2 * W;                      // dwords of the lane's taps
        uint32_t wd[kWD];
        const uint16_t *wq = p.w + int64_t(c) * W;
        if constexpr ((W & 1) == 0) {
#pragma unroll
            for (int i = 0; i < kWD / 4; ++i) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(wq + 8 * i);
                wd[4 * i] = v.x; wd[4 * i + 1] = v.y; wd[4 * i + 2] = v.z; wd[4 * i + 3] = v.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kWD / 2; ++i) {
                const u32x2 v = ld4ch(wq + 4 * i);
                wd[2 * i] = v.x; wd[2 * i + 1] = v.y;
            }
        }
#pragma unroll
        for (int ch = 0; ch < kVecCh; ++ch)
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int e = ch * W + k;
                wf[ch][k] = (e & 1) ? bf_hi(wd[e >> 1]) : bf_lo(wd[e >> 1]);
            }
    } else {
#pragma unroll
        for (int ch = 0; ch < kVecCh; ++ch)
#pragma unroll
            for (int k = 0; k < W; ++k) wf[ch][k] = bf_one(p.w[int64_t(c + ch) * p.w_sd + k]);
    }
    // without a bias the first input stands in and is discarded
    const u32x2 bv = ld4ch(p.bias ? p.bias + c : xp);
    float b0[kVecCh];
#pragma unroll
    for (int ch = 0; ch < kVecCh; ++ch) b0[ch] = p.bias ? ch_of(bv, ch) : 0.0f;

    const void *sx = reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(p.x) & ~uintptr_t(3));
    const int32_t ci = int32_t(sld_u32(p.cache_idx ? static_cast<const void *>(p.cache_idx + b) : sx));
    const int32_t na = int32_t(sld_u32(p.num_acc ? static_cast<const void *>(p.num_acc + b) : sx));
    const int32_t seen = int32_t(sld_u32(p.ring_seen ? static_cast<const void *>(p.ring_seen + b) : sx));
    const int64_t line = p.cache_idx ? int64_t(ci) : int64_t(b);
    if ((p.cache_idx && line == p.pad_slot_id) || line < 0 || line >= p.num_lines) return;

    const int32_t L = p.state_len;
    int32_t off = 0;
    int32_t rcol = 0;
    if (p.num_acc) {
        off = na - 1;
        if (off < 0 || off > L - H) return;
    }
    if (p.ring_seen) {
        if (seen < 0) return;
        rcol = seen % L;
    }
    const bool spec = p.num_acc != nullptr;
    const bool ring = p.ring_seen != nullptr;
    const bool saved = p.inter != nullptr || p.out_idx != nullptr;

    uint16_t *row = p.cs + line * p.cs_sl + c;
    u32x2 win[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        int32_t col = off + k;
        if (ring) {
            col = rcol - H + k;
            if (col < 0) col += L;
        }
        win[k] = ld4ch(row + int64_t(col) * p.cs_st);
    }
    if (spec && !saved) {
#pragma unroll
        for (int k = 0; k + 1 < H; ++k) st4ch(row + int64_t(k) * p.cs_st, win[k + 1]);
    }

    uint16_t *op = p.out + int64_t(b) * p.o_sb + c;
    const int32_t ring_from = p.seqlen - L;
    for (int32_t t0 = 0; t0 < p.seqlen; t0 += kUpdGroup) {
        u32x2 xv[kUpdGroup];
        if (t0 == 0) {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i) xv[i] = xv0[i];
        } else {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i)
                xv[i] = t0 + i < p.seqlen ? ld4ch(xp + int64_t(t0 + i) * p.x_st) : u32x2{0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kUpdGroup; ++i) {
            const int32_t t = t0 + i;
            if (t >= p.seqlen) break;
            float o[kVecCh];
#pragma unroll
            for (int ch = 0; ch < kVecCh; ++ch) {
                float acc = b0[ch];
#pragma unroll
                for (int k = 0; k < H; ++k) acc = __builtin_fmaf(wf[ch][k], ch_of(win[k], ch), acc);
                acc = __builtin_fmaf(wf[ch][H], ch_of(xv[i], ch), acc);
                o[ch] = act<SILU>(acc);
            }
            st4ch(op + int64_t(t) * p.o_st, u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
#pragma unroll
            for (int k = 0; k + 1 < H; ++k) win[k] = win[k + 1];
            win[H - 1] = xv[i];

            if (p.inter) {
                uint16_t *ip = p.inter + int64_t(b) * p.i_sb + int64_t(t) * p.i_st + c;
#pragma unroll
                for (int k = 0; k < H; ++k) st4ch(ip + int64_t(k) * p.i_sk, win[k]);
            }
            if (p.out_idx) {
                const int64_t dst = p.out_idx[int64_t(b) * p.oi_sb + int64_t(t) * p.oi_st];
                if (dst >= 0 && dst < p.num_lines) {
                    uint16_t *dp = p.cs + dst * p.cs_sl + c;
#pragma unroll
                    for (int k = 0; k < H; ++k) st4ch(dp + int64_t(k) * p.cs_st, win[k]);
                }
            }
            if (!saved) {
                if (ring) {
                    if (t >= ring_from) st4ch(row + int64_t(rcol) * p.cs_st, xv[i]);
                    rcol = rcol + 1 == L ? 0 : rcol + 1;
                } else if (spec) {
                    st4ch(row + int64_t(H - 1 + t) * p.cs_st, xv[i]);
                }
            }
        }
    }
    if (!saved && !ring && !spec) {
#pragma unroll
        for (int k = 0; k < H; ++k) st4ch(row + int64_t(k) * p.cs_st, win[k]);
    }
}

// The plain update (no options) on states stored token-contiguous with
// exactly width-1 columns, the usual decode cache: four adjacent channels'
// histories are one run of 4(W-1) values, read and rewritten as W-1
// 8-byte vectors; x and out as in update_vec_kernel.  The arithmetic is that
// of update_kernel.
template <int W, bool SILU>
__global__ __launch_bounds__(kUpdBlock) void update_run_kernel(UpdParams p, uint32_t cblocks) {
    constexpr int H = W - 1;
    const uint32_t b = blockIdx.x / cblocks;
    const int32_t c = int32_t(((blockIdx.x % cblocks) * kUpdBlock + threadIdx.x) * kVecCh);
    if (int32_t(b) >= p.batch || c >= p.dim) return;

    const int32_t g0 = p.seqlen < kUpdGroup ? p.seqlen : kUpdGroup;
    const uint16_t *xp = p.x + int64_t(b) * p.x_sb + c;
    u32x2 xv0[kUpdGroup];
#pragma unroll
    for (int i = 0; i < kUpdGroup; ++i) {
        const u32x2 v = ld4ch(xp + int64_t(i < g0 ? i : 0) * p.x_st);
        xv0[i] = i < g0 ? v : u32x2{0u, 0u};
    }
    float wf[kVecCh][W];
#pragma unroll
    for (int ch = 0; ch < kVecCh; ++ch)
#pragma unroll
        for (int k = 0; k < W; ++k) wf[ch][k] = bf_one(p.w[int64_t(c + ch) * p.w_sd + k]);
    const u32x2 bv = ld4ch(p.bias ? p.bias + c : xp);
    float b0[kVecCh];
#pragma unroll
    for (int ch = 0; ch < kVecCh; ++ch) b0[ch] = p.bias ? ch_of(bv, ch) : 0.0f;

    const void *sx = reinterpret_cast<const void *>(reinterpret_cast<uintptr_t>(p.x) & ~uintptr_t(3));
    const int32_t ci = int32_t(sld_u32(p.cache_idx ? static_cast<const void *>(p.cache_idx + b) : sx));
    const int64_t line = p.cache_idx ? int64_t(ci) : int64_t(b);
    if ((p.cache_idx && line == p.pad_slot_id) || line < 0 || line >= p.num_lines) return;

    // the four histories: value k of channel ch is element ch*H + k of the run
    uint16_t *run = p.cs + line * p.cs_sl + int64_t(c) * H;
    uint32_t hd[2 * H];
#pragma unroll
    for (int i = 0; i < H; ++i) {
        const u32x2 v = ld4ch(run + 4 * i);
        hd[2 * i] = v.x;
        hd[2 * i + 1] = v.y;
    }
    uint32_t win[kVecCh][H];                           // bf16 bits, oldest first
#pragma unroll
    for (int ch = 0; ch < kVecCh; ++ch)
#pragma unroll
        for (int k = 0; k < H; ++k) {
            const int e = ch * H + k;
            win[ch][k] = (hd[e >> 1] >> (16 * (e & 1))) & 0xffffu;
        }

    uint16_t *op = p.out + int64_t(b) * p.o_sb + c;
    for (int32_t t0 = 0; t0 < p.seqlen; t0 += kUpdGroup) {
        u32x2 xv[kUpdGroup];
        if (t0 == 0) {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i) xv[i] = xv0[i];
        } else {
#pragma unroll
            for (int i = 0; i < kUpdGroup; ++i)
                xv[i] = t0 + i < p.seqlen ? ld4ch(xp + int64_t(t0 + i) * p.x_st) : u32x2{0u, 0u};
        }
#pragma unroll
        for (int i = 0; i < kUpdGroup; ++i) {
            const int32_t t = t0 + i;
            if (t >= p.seqlen) break;
            float o[kVecCh];
#pragma unroll
            for (int ch = 0; ch < kVecCh; ++ch) {
                float acc = b0[ch];
#pragma unroll
                for (int k = 0; k < H; ++k) acc = __builtin_fmaf(wf[ch][k], bf_one(uint16_t(win[ch][k])), acc);
                acc = __builtin_fmaf(wf[ch][H], ch_of(xv[i], ch), acc);
                o[ch] = act<SILU>(acc);
                const uint32_t d = (ch >> 1) ? xv[i].y : xv[i].x;
#pragma unroll
                for (int k = 0; k + 1 < H; ++k) win[ch][k] = win[ch][k + 1];
                win[ch][H - 1] = (d >> (16 * (ch & 1))) & 0xffffu;
            }
            st4ch(op + int64_t(t) * p.o_st, u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])});
        }
    }
    // the new histories, written back as the same run
#pragma unroll
    for (int i = 0; i < 2 * H; ++i) {
        const int e0 = 2 * i, e1 = 2 * i + 1;
        hd[i] = win[e0 / H][e0 % H] | (win[e1 / H][e1 % H] << 16);
    }
#pragma unroll
    for (int i = 0; i < H; ++i) st4ch(run + 4 * i, u32x2{hd[2 * i], hd[2 * i + 1]});
}

// Whether every tensor the update touches holds four adjacent channels as
// one aligned 8-byte vector.
bool vec_layout(const UpdParams &p) {
    auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; };
    auto m4 = [](int64_t v) { return (v & 3) == 0; };
    if (p.dim % kVecCh != 0 || p.x_sd != 1 || p.o_sd != 1 || p.cs_sd != 1) return false;
    if (!al(p.x) || !al(p.out) || !al(p.cs) || (p.bias && !al(p.bias))) return false;
    const bool one = p.seqlen == 1;                     // token strides unused
    if (!m4(p.x_sb) || !m4(p.o_sb) || !m4(p.cs_sl) || !m4(p.cs_st) ||
        !(one || (m4(p.x_st) && m4(p.o_st))))
        return false;
    if (p.inter && (p.i_sd != 1 || !al(p.inter) || !m4(p.i_sb) || !(one || m4(p.i_st)) ||
                    !m4(p.i_sk)))
        return false;
    return true;
}

// Whether the update is the plain one on (lines, dim, width-1) token-
// contiguous states, with x and out as vec_layout requires.
bool run_layout(const UpdParams &p, int width) {
    auto al = [](const void *q) { return (reinterpret_cast<uintptr_t>(q) & 7) == 0; };
    auto m4 = [](int64_t v) { return (v & 3) == 0; };
    const bool one = p.seqlen == 1;
    if (p.num_acc || p.ring_seen || p.inter || p.out_idx) return false;
    if (p.state_len != width - 1 || p.cs_st != 1 || p.cs_sd != width - 1) return false;
    if (p.dim % kVecCh != 0 || p.x_sd != 1 || p.o_sd != 1) return false;
    if (!al(p.x) || !al(p.out) || !al(p.cs) || (p.bias && !al(p.bias))) return false;
    return m4(p.x_sb) && m4(p.o_sb) && m4(p.cs_sl) && (one || (m4(p.x_st) && m4(p.o_st)));
}

template <int W>
hipError_t launch_w(const UpdParams &p, bool silu, hipStream_t s) {
    if (run_layout(p, W)) {
        const int32_t lanes = p.dim / kVecCh;
        const uint32_t cblocks = uint32_t((lanes + kUpdBlock - 1) / kUpdBlock);
        const dim3 grid(cblocks * uint32_t(p.batch)), block(kUpdBlock);
        if (silu) update_run_kernel<W, true><<<grid, block, 0, s>>>(p, cblocks);
        else update_run_kernel<W, false><<<grid, block, 0, s>>>(p, cblocks);
        return hipGetLastError();
    }
    if (vec_layout(p)) {
        const int32_t lanes = p.dim / kVecCh;
        const uint32_t cblocks = uint32_t((lanes + kUpdBlock - 1) / kUpdBlock);
        const dim3 grid(cblocks * uint32_t(p.batch)), block(kUpdBlock);
        const bool wide = p.w_sd == W && (reinterpret_cast<uintptr_t>(p.w) & 15) == 0;
        if (silu && wide) update_vec_kernel<W, true, true><<<grid, block, 0, s>>>(p, cblocks);
        else if (silu) update_vec_kernel<W, true, false><<<grid, block, 0, s>>>(p, cblocks);
        else if (wide) update_vec_kernel<W, false, true><<<grid, block, 0, s>>>(p, cblocks);
        else update_vec_kernel<W, false, false><<<grid, block, 0, s>>>(p, cblocks);
        return hipGetLastError();
    }
    const uint32_t cblocks = uint32_t((p.dim + kUpdBlock - 1) / kUpdBlock);
    const dim3 grid(cblocks * uint32_t(p.batch)), block(kUpdBlock);
    if (silu) update_kernel<W, true><<<grid, block, 0, s>>>(p, cblocks);
    else update_kernel<W, false><<<grid, block, 0, s>>>(p, cblocks);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_update(const UpdParams &p, int width, bool silu, hipStream_t s) {
    switch (width) {
        case 2: return launch_w<2>(p, silu, s);
        case 3: return launch_w<3>(p, silu, s);
        case 4: return launch_w<4>(p, silu, s);
        case 5: return launch_w<5>(p, silu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

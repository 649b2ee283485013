// Varlen forward for token-contiguous (dim, T) storage -- the layout of the
// atrex-bench #003 "causal_conv1d" inputs (section "Input Generation"), with
// the batch semantics of tokenspeed causal_conv1d.py (_causal_conv1d_fwd_kernel).
//
// Decomposition: x is streamed as one flat array of dim*T bf16 in aligned
// 16-byte chunks (8 elements); chunk k covers flat elements 8k..8k+7, i.e.
// channel c = i / T, token t = i % T of each element.  A wave owns
// kTokRounds rounds of 64 consecutive chunks, so each load instruction moves
// 1 KiB of contiguous memory whatever T is (rows start misaligned whenever
// T % 8 != 0).  The width-1 history of a chunk is the tail of the previous
// chunk: it comes from the neighbouring lane with a cross-lane permute, and
// lane 0 takes lane 63's tail from the previous round (one 8-byte load per
// wave for round 0).
//
// The path is bound by memory only if the ALU work per 16-byte chunk stays
// small (at 8 TB/s a CU has ~150 lane-instructions per chunk), so the fast
// path is built to be lean:
//   * when T >= 2048 a wave's 2048 elements span at most two channel rows:
//     the channel, the row start and the weights are wave-uniform values and
//     each lane only picks one of two (no per-lane division, no gathers);
//   * the taps run on packed bf16 pairs with the gfx950 dot2 instruction
//     (two products accumulated into fp32 per instruction, exact products),
//     so x is never unpacked for the taps; an odd last tap uses one fma.
// Chunks that touch a row or sequence boundary, the first width-1 tokens of
// a sequence, or the ragged tail (about 0.1% of chunks at the benchmark's
// sizes) are deferred and redone element by element after the fast rounds.
// The element holding a sequence's first token owns that sequence's history:
// it alone reads the cached state, computes the first width-1 outputs
// (possibly spilling into the next chunk) and writes the new state, so no
// other lane can read a state that has already been overwritten.
#include "sconv_device.h"

namespace sconv {

namespace {

constexpr int kChunksPerWave = kWaveSize * kTokRounds;
constexpr uint32_t kWaveElems = kChunksPerWave * kVec;
constexpr int kShortMinT = 16;                    // shortest row of the short-row kernel
constexpr int kShortWaves = 256 * 8;             // waves that keep ~8 per CU busy
constexpr int kLongWaves = 4;                     // waves per long-row block (fewer, larger
                                                  // workgroups dispatch faster at 10^5 waves)
constexpr int kLongRounds = 4;                    // 64-chunk rounds per long-row wave (measured:
                                                  // 1 and 2 repeat the wave setup too often)
constexpr int kLongRoundsMid = 3;                 // rounds for kLongMidLo <= T < kLongMidHi
constexpr uint32_t kLongMidLo = 3072;             // (measured on gfx950: 3 rounds are 1.3-3.5%
constexpr uint32_t kLongMidHi = 10000;            // faster at T 3100-9999, 5% slower at T 2048,
                                                  // where 4 rounds are exactly one row per wave)
// Four-round waves each keep 4 KiB of loads in flight; at six resident
// workgroups per CU (what the registers allow) the memory queues run deeper
// than they need to.  From T 10000 on, an LDS reservation the kernel never
// touches caps a CU at five (5 x 32 KiB of gfx950's 160 KiB): measured
// 1.4-1.7% faster at T 11027, 14807 and 20000.  Three-round waves
// (T 3072-9999) and four-round waves below T 3072 are best at six.
#ifndef SCONV_LONG_FOUR_ROUND_LDS
#define SCONV_LONG_FOUR_ROUND_LDS 32768
#endif
constexpr uint32_t kLongFourRoundLds = SCONV_LONG_FOUR_ROUND_LDS;

// Weights of one channel for the dot2 path: taps as packed bf16 pairs
// (w[2p], w[2p+1]), the odd last tap and the bias as fp32.
template <int W>
struct PairTaps {
    uint32_t wp[W / 2];
    float wl;
    float b;
};

template <int W>
__device__ __forceinline__ PairTaps<W> load_pair_taps(const FwdTokParams &p, uint32_t c) {
    PairTaps<W> r;
    const uint16_t *w = p.w + int64_t(c) * p.w_sd;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) r.wp[q] = uint32_t(w[2 * q]) | (uint32_t(w[2 * q + 1]) << 16);
    r.wl = (W & 1) ? bf_one(w[W - 1]) : 0.0f;
    r.b = p.bias ? bf_one(p.bias[c]) : 0.0f;
    return r;
}

template <int W>
__device__ __forceinline__ PairTaps<W> uniform(PairTaps<W> t) {
#pragma unroll
    for (int q = 0; q < W / 2; ++q) t.wp[q] = __builtin_amdgcn_readfirstlane(t.wp[q]);
    t.wl = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(t.wl)));
    t.b = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(t.b)));
    return t;
}

template <int W>
__device__ __forceinline__ PairTaps<W> select(bool b, const PairTaps<W> &tb, const PairTaps<W> &ta) {
    PairTaps<W> r;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) r.wp[q] = b ? tb.wp[q] : ta.wp[q];
    r.wl = b ? tb.wl : ta.wl;
    r.b = b ? tb.b : ta.b;
    return r;
}

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// The 12 elements e[0..11] before and in a chunk: e[0..3] are elements 4..7
// of the previous chunk (dwords hz, hw), e[4..11] the chunk (v).  Pair m is
// (e[m], e[m+1]); elem m is e[m] widened.
struct Window {
    uint32_t d[6];
    __device__ __forceinline__ uint32_t pair(int m) const {
        return (m & 1) ? __builtin_amdgcn_alignbit(d[(m + 1) >> 1], d[(m - 1) >> 1], 16)
                       : d[m >> 1];
    }
    __device__ __forceinline__ float elem(int m) const {
        return (m & 1) ? bf_hi(d[m >> 1]) : bf_lo(d[m >> 1]);
    }
};

// 8 outputs of a chunk whose every tap lies in the window.
template <int W, bool SILU>
__device__ __forceinline__ u32x4 fast_chunk(const Window &win, const PairTaps<W> &tp) {
    constexpr int H = W - 1;            // history length
    constexpr int B = 4 - H;            // e index of u[0]
    float o[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        float acc = tp.b;
#pragma unroll
        for (int q = 0; q < W / 2; ++q) acc = dot2(win.pair(B + j + 2 * q), tp.wp[q], acc);
        if constexpr (W & 1) acc = __builtin_fmaf(tp.wl, win.elem(B + j + W - 1), acc);
        o[j] = act<SILU>(acc);
    }
    return pack8(o);
}

// The history h[0..H) packed four 16-bit entries to a 64-bit value, and entry
// h[H+l] (l in [-H, -1]) read back by shifting.  Arithmetic, not an array:
// a select chain over an array indexed by a lane-dependent l gets folded
// into an indexed load, the array then moves to LDS, and indexing it costs
// every wave a read of the dispatch packet -- about 15 us per launch.
template <int H>
__device__ __forceinline__ uint64_t pack_hist(const uint32_t (&h)[H]) {
    uint64_t v = 0;
#pragma unroll
    for (int k = 0; k < H; ++k) v |= uint64_t(h[k] & 0xffffu) << (16 * k);
    return v;
}
template <int H>
__device__ __forceinline__ uint32_t hist_bits(uint64_t hv, int l) {
    return uint32_t(hv >> (16 * (H + l))) & 0xffffu;
}

// A chunk that holds part of the first width-1 tokens of a row whose head is
// at flat index hp (the chunk may also end the previous row).  It is the fast
// chunk twice: once on the window as loaded with the previous row's taps
// (right for elements before hp), once on a copy whose positions in
// [hp-H, hp) hold the cached history h, with the head row's taps (right for
// elements from hp on); the two are merged element by element.  head_merge
// takes the first of the two, `a`, already computed.
template <int W, bool SILU>
__device__ __forceinline__ u32x4 head_merge(const u32x4 &a, const Window &win, uint32_t i0, uint32_t hp,
                                            const PairTaps<W> &t_head, const uint32_t (&h)[W - 1]) {
    constexpr int H = W - 1;
    const uint64_t hv = pack_hist<H>(h);
    Window wh = win;
#pragma unroll
    for (int d = 0; d < 6; ++d) {
        uint32_t lo = wh.d[d] & 0xffffu, hi = wh.d[d] >> 16;
        const int l0 = int(i0 - 4 + 2 * d) - int(hp);          // position relative to the head
        if (l0 >= -H && l0 < 0) lo = hist_bits<H>(hv, l0);
        if (l0 + 1 >= -H && l0 + 1 < 0) hi = hist_bits<H>(hv, l0 + 1);
        wh.d[d] = lo | (hi << 16);
    }
    const u32x4 b = fast_chunk<W, SILU>(wh, t_head);
    const uint32_t k = hp > i0 ? hp - i0 : 0;              // elements [0, k) end the previous row
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
    uint32_t r[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t lo = (2 * d < int(k) ? av[d] : bv[d]) & 0xffffu;
        const uint32_t hi = (2 * d + 1 < int(k) ? av[d] : bv[d]) & 0xffff0000u;
        r[d] = lo | hi;
    }
    return u32x4{r[0], r[1], r[2], r[3]};
}
template <int W, bool SILU>
__device__ __forceinline__ u32x4 head_chunk(const Window &win, uint32_t i0, uint32_t hp,
                                            const PairTaps<W> &t_prev, const PairTaps<W> &t_head,
                                            const uint32_t (&h)[W - 1]) {
    return head_merge<W, SILU>(fast_chunk<W, SILU>(win, t_prev), win, i0, hp, t_head, h);
}

// Scalar weights for the element-by-element path.
template <int W>
struct Taps {
    float w[W];
    float b;
};

template <int W>
__device__ __forceinline__ Taps<W> load_taps(const FwdTokParams &p, uint32_t c) {
    Taps<W> r;
#pragma unroll
    for (int k = 0; k < W; ++k) r.w[k] = bf_one(p.w[int64_t(c) * p.w_sd + k]);
    r.b = p.bias ? bf_one(p.bias[c]) : 0.0f;
    return r;
}

// Sequence of token t, reusing the lane's previous answer when it still holds.
struct SeqCache {
    int32_t s = -1;
    SeqInfo si;
    __device__ __forceinline__ const SeqInfo &get(const SeqBatch &sb, const int32_t *qsl, int64_t t) {
        if (s < 0 || t < si.start || t >= si.end) {
            s = sb.batch == 1 ? 0 : seq_search(qsl, sb.batch, t);
            si = seq_info(sb, qsl, s);
        }
        return si;
    }
};

// Element-by-element processing of one chunk (all loads from memory).
template <int W, bool SILU>
__device__ void slow_chunk(const FwdTokParams &p, const int32_t *qsl, uint32_t i0) {
    constexpr int H = W - 1;
    const uint32_t T = p.T;
    uint32_t c = p.divT.div(i0);
    uint32_t t = i0 - c * T;
    Taps<W> tp = load_taps<W>(p, c);
    SeqCache sc;
    for (int j = 0; j < kVec; ++j) {
        const uint32_t i = i0 + j;
        if (i >= p.n_elems) break;
        if (j > 0 && ++t == T) {           // crossed into the next channel row
            t = 0;
            ++c;
            tp = load_taps<W>(p, c);
        }
        const SeqInfo &si = sc.get(p.sb, qsl, t);
        if (si.skip || int64_t(t) < si.start || int64_t(t) >= si.end) continue;
        const int64_t tl = int64_t(t) - si.start;
        if (tl >= 1 && tl <= H - 1) continue;      // owned by the sequence's first token
        const uint16_t *xrow = p.x + size_t(c) * T;
        uint16_t *orow = p.out + size_t(c) * T;
        if (tl >= H) {                              // every tap inside the sequence
            float acc = tp.b;
#pragma unroll
            for (int k = 0; k < W; ++k) acc = __builtin_fmaf(tp.w[k], bf_one(xrow[t - H + k]), acc);
            orow[t] = to_bf16(act<SILU>(acc));
            continue;
        }
        // tl == 0: the history owner of (sequence, channel).
        const uint16_t *xseq = xrow + si.start;
        uint16_t h[H];
#pragma unroll
        for (int k = 0; k < H; ++k)
            h[k] = si.init ? p.sb.cs[si.line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd + k * p.sb.cs_st]
                           : uint16_t(0);
        const int64_t L = si.end - si.start;
        const int nq = L < H ? int(L) : H;
#pragma unroll
        for (int q = 0; q < H; ++q) {
            if (q >= nq) break;
            float acc = tp.b;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int idx = q - H + k;          // compile-time after unrolling
                const uint16_t v = idx >= 0 ? xseq[idx] : h[H + idx];
                acc = __builtin_fmaf(tp.w[k], bf_one(v), acc);
            }
            orow[si.start + q] = to_bf16(act<SILU>(acc));
        }
        if (p.sb.cs) {
            uint16_t nh[H];
#pragma unroll
            for (int k = 0; k < H; ++k) {
                const int64_t m = L + k;            // index into h ++ x
                uint16_t hv = 0;
#pragma unroll
                for (int q = 0; q < H; ++q)
                    if (m == q) hv = h[q];
                nh[k] = m < H ? hv : xseq[m - H];
            }
#pragma unroll
            for (int k = 0; k < H; ++k)
                p.sb.cs[si.line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd + k * p.sb.cs_st] = nh[k];
        }
    }
}

// Tap k of a PairTaps as fp32.
template <int W>
__device__ __forceinline__ float tap_of(const PairTaps<W> &t, int k) {
    if ((W & 1) && k == W - 1) return t.wl;
    const uint32_t pr = t.wp[k >> 1];
    return (k & 1) ? bf_hi(pr) : bf_lo(pr);
}

// Channel c's taps and bias through the scalar cache (with no bias the
// stand-in read is masked to 0).
template <int W>
__device__ __forceinline__ PairTaps<W> sload_pair_taps(const FwdTokParams &p, uint32_t c) {
    const U16Run<W> w = sld_run<W>(p.w + int64_t(c) * p.w_sd);
    PairTaps<W> r;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) r.wp[q] = w.d[q];
    r.wl = (W & 1) ? bf_one(uint16_t(w.elem(W - 1))) : 0.0f;
    r.b = bf_one(uint16_t(sld_u16(p.bias_rd + c) & p.bias_mask));
    return r;
}

// One sequence whose rows are at least one wave long (T >= 2048): every
// wave spans at most two rows and contains at most one row head.  The head's
// history (state), the row's last width-1 inputs (the new state) and both
// rows' taps are wave-uniform values read with scalar loads issued right
// after the wave's x loads, so they complete under them; the head chunks are
// computed in registers and one lane writes the new state after the wave's
// reads.  A head belongs to the wave that holds its last history-reading
// token, so a head that straddles two waves is computed by the second one,
// from its 4-element halo and the history; the first leaves those elements
// alone.  No wave waits on a second round trip for these rare heads (an
// element path with several dependent loads made a few waves the tail of
// the grid).  Only the ragged last chunk of the array and a sequence that
// does not cover every token take the element path.
template <int W, bool SILU, int ROUNDS>
__global__ __launch_bounds__(kLongWaves * kWaveSize) void fwd_tok_long_kernel(FwdTokParams p) {
    constexpr uint32_t kCPW = ROUNDS * kWaveSize;           // chunks per wave
    constexpr uint32_t kWE = kCPW * kVec;                   // elements per wave
    constexpr int H = W - 1;
    constexpr uint32_t kNone = 0xffffffffu;
    const int lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t wbase = (blockIdx.x * kLongWaves + wave) * kCPW;
    if (wbase >= p.n_chunks) return;

    // The wave's x goes out first.  Everything else it needs is wave-uniform
    // and read with scalar loads that complete under the x loads, so a wave
    // waits for one memory round trip before it computes.  Full chunks go
    // through a descriptor that ends at the last one, so the loads need no
    // branch (the ragged last chunk reads 0 here).
    const uint32_t T = p.T;
    const uint32_t n_full = p.n_elems / kVec;
    constexpr int kNt = 2;                                  // non-temporal cache policy bit
    const uint32_t n_mine = wbase < n_full ? (n_full - wbase < kCPW ? n_full - wbase : kCPW) : 0u;
    const Rsrc xr = make_rsrc(p.x + size_t(wbase) * kVec, int64_t(n_mine) * 16);
    const Rsrc outr = make_rsrc(p.out + size_t(wbase) * kVec, int64_t(n_mine) * 16);
    u32x4 v[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) v[r] = buf_ld128<kNt>(xr, uint32_t(r * kWaveSize + lane) * 16u);
    asm volatile("" ::: "memory");                          // the x loads go out first

    // Wave-uniform rows, head and history.
    const uint32_t e_first = wbase * kVec;
    const uint32_t e_last = (e_first + kWE <= p.n_elems ? e_first + kWE : p.n_elems) - 1;
    const uint32_t cA = p.divT.div(e_first);
    const uint32_t row_a = cA * T, row_end = row_a + T;
    // The wave owns the head of a row (its first width-1 tokens, the ones
    // that read the history) when it holds the head's last token: row cA's
    // head when the wave starts at most width-2 tokens into the row (those
    // first tokens then lie just before the wave), or row cA+1's head when
    // it ends inside the wave.  A head of row cA+1 that runs past the wave's
    // end belongs to the next wave: this wave leaves its first tokens alone.
    uint32_t hp = kNone, R = 0;
    if (e_first - row_a <= uint32_t(H - 1)) { hp = row_a; R = cA; }
    else if (uint64_t(row_end) + (H - 1) <= e_last) { hp = row_end; R = cA + 1; }
    const bool next_head = row_end <= e_last && uint64_t(row_end) + (H - 1) > e_last;
    // The elements around a row boundary are computed one per lane after
    // the rounds, and the chunks that hold them are not stored by the
    // rounds.  Span A: the chunks that hold the wave's head (from the head
    // itself when it starts just before the wave), at most 16 elements, for
    // lanes 0..15.  Span B: the start of the chunk that holds the next
    // wave's head, up to that head (1..7 elements), for lanes 16..23.  Each
    // of these lanes reads its element's width inputs with 2-byte loads
    // issued here, right after the x loads: the spans follow from the row
    // geometry alone, so no scalar load stands before them.
    const uint32_t fa0 = hp != kNone ? (hp < e_first ? hp : hp & ~uint32_t(kVec - 1)) : 0u;
    const uint32_t fa1 = hp != kNone ? ((hp + (H - 1)) & ~uint32_t(kVec - 1)) + kVec : 0u;
    const uint32_t fb0 = row_end & ~uint32_t(kVec - 1);
    const uint32_t nb_rows = next_head ? row_end - fb0 : 0u;
    const bool in_a = lane < 16;
    const uint32_t fe = in_a ? fa0 + uint32_t(lane) : fb0 + uint32_t(lane - 16);
    const bool f_in = in_a ? fe < fa1 : uint32_t(lane - 16) < nb_rows;
    // span offsets are relative to 8 elements before the wave
    const uint32_t xb = e_first >= kVec ? e_first - kVec : 0u;
    const Rsrc xfr = make_rsrc(p.x + xb, int64_t(p.n_elems - xb) * 2);
    const Rsrc ofr = make_rsrc(p.out + xb, int64_t(p.n_elems - xb) * 2);
    // One 12-byte load from the dword holding input 0 covers the width
    // inputs (at most 6 elements from there).  Inputs before x occur only
    // in the array's first wave (the first row's head, whose inputs before
    // token 0 are history): such a lane loads from x's start instead.
    const int64_t p0 = int64_t(fe) - H;
    const bool f_neg = p0 < int64_t(xb);
    const uint32_t f_odd = f_neg ? 0u : uint32_t(p0) & 1u;
    const uint32_t f_off = f_neg ? 0u : uint32_t(p0 - int64_t(xb)) * 2u - f_odd * 2u;
    const u32x3 fr = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(
        xfr, f_in ? f_off : kOob, 0, 0));
    asm volatile("" ::: "memory");                          // and the span loads next
    // the 4 elements before the wave: lane 0's halo in round 0
    const uint16_t *pp = p.x + (wbase > 0 ? size_t(wbase) * kVec - 4 : 0);
    uint32_t prev_z = sld_u32(pp), prev_w = sld_u32(pp + 2);
    if (wbase == 0) prev_z = prev_w = 0;

    // Sequence 0: its token range, cache line and whether it has a history.
    const int64_t q0 = int32_t(sld_u32(p.sb.qsl)), q1 = int32_t(sld_u32(p.sb.qsl + 1));
    const int32_t ci = int32_t(sld_u32(p.ci_rd));
    const uint32_t hiv = sld_u8(p.hi_rd);
    const int64_t line = p.sb.cache_idx ? int64_t(ci) : 0;
    const bool skip = (p.sb.cache_idx && line == p.sb.pad_slot_id) ||
                      (p.sb.cs && (line < 0 || line >= p.sb.num_lines));
    const bool init = p.sb.cs && p.sb.has_init && hiv != 0;
    const bool simple = q0 <= 0 && q1 >= int64_t(T);       // the sequence covers every token

    const bool live = !skip;                                // padded sequence: nothing to do
    // A span is computed when the whole row is one sequence that is not padded.
    const bool own_head = simple && hp != kNone && live;
    const uint32_t nb = simple && live ? nb_rows : 0u;
    const bool fvalid = f_in && simple && live;
    const PairTaps<W> tA = sload_pair_taps<W>(p, cA);
    const PairTaps<W> tB = sload_pair_taps<W>(p, cA + 1 < uint32_t(p.dim) ? cA + 1 : cA);
    const PairTaps<W> &t_head = (R == cA) ? tA : tB;
    // Waves that hold a row head also read its history (the cached state,
    // read by this wave only) and the row's last width-1 inputs (the new
    // state).  The loads still go out before the wave waits for its x.
    uint32_t hb[H];
    U16Run<H> nh;
#pragma unroll
    for (int k = 0; k < H; ++k) hb[k] = 0;
#pragma unroll
    for (int i = 0; i < H / 2 + 1; ++i) nh.d[i] = 0;
    if (own_head) {
        asm volatile("");                                   // keeps this a branch
        nh = sld_run<H>(p.x + size_t(R) * T + (T - H));
        if (init) {
#pragma unroll
            for (int k = 0; k < H; ++k)
                hb[k] = sld_u16(p.sb.cs + (line * p.sb.cs_sl + int64_t(R) * p.sb.cs_sd + k * p.sb.cs_st));
        }
    }
#pragma unroll
    for (int k = 0; k < H; ++k) pin_sgpr(hb[k]);
#pragma unroll
    for (int i = 0; i < H / 2 + 1; ++i) pin_sgpr(nh.d[i]);

    // chunks (relative to the wave) the rounds leave to the lanes above
    const uint32_t sa0 = fa0 < e_first ? 0u : fa0 / kVec - wbase;
    const uint32_t na = fa1 > fa0 ? (fa1 - 1) / kVec - wbase + 1 - sa0 : 0u;
    const uint32_t sbr = nb ? fb0 / kVec - wbase : kNone;

    // Halo of every round first (each permute waits only for its own load).
    const int src_lane = (lane + kWaveSize - 1) & (kWaveSize - 1);
    uint32_t hz[ROUNDS], hw[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const uint32_t rz = uint32_t(__shfl(int(v[r].z), src_lane));
        const uint32_t rw = uint32_t(__shfl(int(v[r].w), src_lane));
        hz[r] = lane == 0 ? prev_z : rz;
        hw[r] = lane == 0 ? prev_w : rw;
        prev_z = rz;
        prev_w = rw;
    }

    // Chunks computed and stored round by round.  Element-path chunks are
    // only marked here.
    uint32_t slow = 0;
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const uint32_t rel = uint32_t(r * kWaveSize + lane);
        const uint32_t chunk = wbase + rel;
        const uint32_t i0 = chunk * kVec;
        const bool is_slow = !simple || chunk >= n_full;
        const bool spanned = rel - sa0 < na || rel == sbr;
        Window win;
        win.d[0] = hz[r];
        win.d[1] = hw[r];
        win.d[2] = v[r].x;
        win.d[3] = v[r].y;
        win.d[4] = v[r].z;
        win.d[5] = v[r].w;
        // Every lane computes its chunk and stores it through a descriptor
        // (a lane with nothing to store writes past its end): no branch
        // stands between the wave's loads and the taps' first use.
        const u32x4 o = fast_chunk<W, SILU>(win, select(i0 >= row_end, tB, tA));
        const bool mine = live && chunk < p.n_chunks;
        if (mine && is_slow) slow |= 1u << r;
        __builtin_amdgcn_raw_buffer_store_b128(o, outr,
                                               mine && !is_slow && !spanned ? rel * 16u : kOob,
                                               0, kNt);
    }
    // The spanned elements, one per lane: the head's taps from the head on
    // (its first width-1 tokens read the history in place of the previous
    // row), the previous row's taps before it.  The same pairwise
    // accumulation as the rounds.
    if (own_head || nb != 0) {                              // wave-uniform
        asm volatile("");
        const bool head_side = in_a && fe >= hp;
        const PairTaps<W> tf = select(head_side, t_head, tA);
        const uint64_t hv = pack_hist<H>(hb);
        // the loaded inputs shifted down by the odd element, two per dword
        const uint32_t g0 = __builtin_amdgcn_alignbit(fr.y, fr.x, 16 * f_odd);
        const uint32_t g1 = __builtin_amdgcn_alignbit(fr.z, fr.y, 16 * f_odd);
        const uint32_t g2 = f_odd ? fr.z >> 16 : fr.z;
        const uint32_t gv[3] = {g0, g1, g2};
        uint32_t xin[W];
#pragma unroll
        for (int k = 0; k < W; ++k) xin[k] = (gv[k >> 1] >> (16 * (k & 1))) & 0xffffu;
        if (wbase == 0) {                                   // wave-uniform: the first wave
            asm volatile("");
            // a lane whose inputs start sh tokens before x read x from its
            // start: input k >= sh is element k - sh of that run
            const int32_t sh = f_neg ? int32_t(int64_t(xb) - p0) : 0;
            const uint32_t fw[3] = {fr.x, fr.y, fr.z};
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int32_t i = k - sh;
                const uint32_t ii = i < 0 ? 0u : uint32_t(i);
                const uint32_t dw = (ii >> 1) == 0 ? fw[0] : ((ii >> 1) == 1 ? fw[1] : fw[2]);
                if (sh > 0) xin[k] = (dw >> (16 * (ii & 1))) & 0xffffu;
            }
        }
        uint32_t u[W];
#pragma unroll
        for (int k = 0; k < W; ++k) {
            const uint32_t hi = fe - hp + uint32_t(k);      // history index when < H
            const uint32_t hbits = uint32_t(hv >> (16 * (hi < uint32_t(H) ? hi : 0u))) & 0xffffu;
            u[k] = head_side && hi < uint32_t(H) ? hbits : xin[k];
        }
        float acc = tf.b;
#pragma unroll
        for (int q = 0; q < W / 2; ++q) acc = dot2(u[2 * q] | (u[2 * q + 1] << 16), tf.wp[q], acc);
        if constexpr (W & 1) acc = __builtin_fmaf(tf.wl, bf_one(uint16_t(u[W - 1])), acc);
        __builtin_amdgcn_raw_buffer_store_b16(to_bf16(act<SILU>(acc)), ofr,
                                              fvalid ? (fe - xb) * 2u : kOob, 0, 0);
    }
    // One lane replaces the history this wave read with the row's last
    // width-1 inputs.
    if (own_head && p.sb.cs && lane == 0) {
#pragma unroll
        for (int k = 0; k < H; ++k)
            p.sb.cs[line * p.sb.cs_sl + int64_t(R) * p.sb.cs_sd + k * p.sb.cs_st] = uint16_t(nh.elem(k));
    }
#pragma unroll 1
    for (int r = 0; r < ROUNDS; ++r)
        if (slow & (1u << r)) slow_chunk<W, SILU>(p, p.sb.qsl, (wbase + r * kWaveSize + lane) * kVec);
}

// Taps of channel row `lr` of a wave-local weight descriptor (row pitch
// w_sd elements), loaded without branches (past the extent: 0).
template <int W>
__device__ __forceinline__ PairTaps<W> buf_pair_taps(Rsrc wr, Rsrc br, uint32_t lr, int64_t w_sd) {
    PairTaps<W> t;
    const uint32_t o = uint32_t(int64_t(lr) * w_sd) * 2;
#pragma unroll
    for (int q = 0; q < W / 2; ++q)
        t.wp[q] = uint32_t(buf_ld16(wr, o + 4 * q)) | (uint32_t(buf_ld16(wr, o + 4 * q + 2)) << 16);
    t.wl = (W & 1) ? bf_one(buf_ld16(wr, o + 2 * (W - 1))) : 0.0f;
    t.b = bf_one(buf_ld16(br, lr * 2));
    return t;
}

// Lane `src`'s PairTaps (a cross-lane permute per value).
template <int W>
__device__ __forceinline__ PairTaps<W> shfl_taps(const PairTaps<W> &t, int src) {
    PairTaps<W> r;
#pragma unroll
    for (int q = 0; q < W / 2; ++q) r.wp[q] = uint32_t(__shfl(int(t.wp[q]), src));
    r.wl = (W & 1) ? __shfl(t.wl, src) : 0.0f;
    r.b = __shfl(t.b, src);
    return r;
}

// One sequence whose rows are short (kShortMinT <= T < one wave): a chunk
// holds at most one row start, and every element of a chunk before that
// start has its whole window inside its own row (T >= 16 > 8 + width-1).
//
// The rows a wave touches (at most ROUNDS*512/T + 2 <= 64) are handled by
// "row lanes": lane j loads, once per wave, the taps of row c_first + j and,
// when that row starts inside the wave, its cached history, its first
// width-1 inputs and its last width-1 inputs -- and writes the row's new
// state, so the one reader of a history is also its one writer.  A chunk
// lane takes its row's taps, and for a row start inside its chunk the
// history and head inputs, from the row lane with cross-lane permutes; it
// computes that chunk with head_chunk and the head outputs that spill into
// the next chunk, which leaves them alone.  A wave thus issues ROUNDS chunk
// loads plus a fixed handful of row loads, all up front and unconditional
// (through descriptors based at the wave's own rows; out-of-range offsets
// read 0): one memory round trip per wave.
template <int W, bool SILU, int ROUNDS>
__global__ __launch_bounds__(kWaveSize) void fwd_tok_short_kernel(FwdTokParams p) {
    constexpr int H = W - 1;
    constexpr uint32_t kNone = 0xffffffffu;
    constexpr int kNt = 2;
    const int lane = threadIdx.x;
    const uint32_t wbase = blockIdx.x * uint32_t(ROUNDS * kWaveSize);
    if (wbase >= p.n_chunks) return;
    const uint32_t T = p.T;
    const uint32_t n_full = p.n_elems / kVec;

    // The wave's elements [e0, e_end) and rows [c_first, c_last]; a row that
    // starts in a full chunk of the wave is owned by the wave.
    const uint32_t e0 = wbase * kVec;
    const uint32_t e_end = e0 + uint32_t(ROUNDS * kWaveSize * kVec) < p.n_elems
                               ? e0 + uint32_t(ROUNDS * kWaveSize * kVec) : p.n_elems;
    const uint32_t own_end = e_end < n_full * kVec ? e_end : n_full * kVec;
    const uint32_t c_first = p.divT.div(e0);
    const uint32_t c_last = p.divT.div(e_end - 1);
    const uint32_t n_rows = c_last - c_first + 1;
    const uint32_t xb0 = e0 >= uint32_t(kVec) ? e0 - kVec : 0;      // keeps the halo in range
    const uint32_t x_hi = uint64_t(e_end) + T < p.n_elems ? e_end + T : p.n_elems;
    const Rsrc xr = make_rsrc(p.x + xb0, int64_t(x_hi - xb0) * 2);
    const Rsrc wr = make_rsrc(p.w + int64_t(c_first) * p.w_sd, int64_t(n_rows) * p.w_sd * 2);
    const Rsrc br = make_rsrc(p.bias ? p.bias + c_first : p.x, p.bias ? int64_t(n_rows) * 2 : 0);

    // chunk loads first: they depend on the launch arguments alone
    u32x4 v[ROUNDS];
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const uint32_t chunk = wbase + r * kWaveSize + lane;
        v[r] = buf_ld128<kNt>(xr, chunk < n_full ? (chunk * kVec - xb0) * 2 : kOob);
    }
    const u32x2 prev = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(xr, lane == 0 && wbase > 0 ? (e0 - 4 - xb0) * 2
                                                                                : kOob, 0, 0));
    // row loads: lane j <-> row c_first + j
    const uint32_t my_row = c_first + uint32_t(lane);
    const bool row_in = uint32_t(lane) < n_rows;
    const uint32_t my_hp = my_row * T;
    const bool row_own = row_in && my_hp >= e0 && my_hp < own_end;
    const PairTaps<W> rt = buf_pair_taps<W>(wr, br, row_in ? uint32_t(lane) : 0x7fffu, p.w_sd);
    uint32_t rh[H], rx[H], rn[H];
#pragma unroll
    for (int k = 0; k < H; ++k) {
        rx[k] = buf_ld16(xr, row_own ? (my_hp + k - xb0) * 2 : kOob);
        rn[k] = buf_ld16(xr, row_own ? (my_hp + T - H + k - xb0) * 2 : kOob);
    }
    // the sequence's description through the scalar cache, then the owned
    // rows' cached histories (their line is known only now)
    const SeqInfo s0 = seq_info_scalar(p.sb, 0);
    const bool state_ok = p.sb.cs != nullptr && !s0.skip;
    const Rsrc sr = make_rsrc(state_ok ? p.sb.cs + s0.line * p.sb.cs_sl + int64_t(c_first) * p.sb.cs_sd
                                       : p.x,
                              state_ok ? (int64_t(n_rows - 1) * p.sb.cs_sd + int64_t(H - 1) * p.sb.cs_st + 1) * 2
                                       : 0);
#pragma unroll
    for (int k = 0; k < H; ++k)
        rh[k] = buf_ld16(sr, row_own ? uint32_t(int64_t(lane) * p.sb.cs_sd + int64_t(k) * p.sb.cs_st) * 2
                                     : kOob);

    if (s0.skip) return;                                // padded sequence: nothing to do
    // the sequence is not the whole row, or (never, with the host's choice of
    // ROUNDS) the wave spans more rows than it has lanes: element path
    if (s0.start != 0 || s0.end != int64_t(T) || n_rows > uint32_t(kWaveSize)) {
#pragma unroll 1
        for (int r = 0; r < ROUNDS; ++r) {
            const uint32_t chunk = wbase + r * kWaveSize + lane;
            if (chunk < p.n_chunks) slow_chunk<W, SILU>(p, p.sb.qsl, chunk * kVec);
        }
        return;
    }
    const bool init = s0.init;
    // packed per-row history and head inputs, to be permuted to chunk lanes
    uint32_t hpk[(H + 1) / 2], xpk[(H + 1) / 2];
#pragma unroll
    for (int k = 0; k < (H + 1) / 2; ++k) {
        const uint32_t h0 = init ? rh[2 * k] : 0u;
        const uint32_t h1 = (2 * k + 1 < H && init) ? rh[2 * k + 1 < H ? 2 * k + 1 : 0] : 0u;
        hpk[k] = (h0 & 0xffffu) | (h1 << 16);
        xpk[k] = (rx[2 * k] & 0xffffu) | ((2 * k + 1 < H ? rx[2 * k + 1 < H ? 2 * k + 1 : 0] : 0u) << 16);
    }

    uint32_t prev_z = prev.x, prev_w = prev.y;
    const int src_lane = (lane + kWaveSize - 1) & (kWaveSize - 1);
#pragma unroll
    for (int r = 0; r < ROUNDS; ++r) {
        const uint32_t rz = uint32_t(__shfl(int(v[r].z), src_lane));
        const uint32_t rw = uint32_t(__shfl(int(v[r].w), src_lane));
        Window win;
        win.d[0] = lane == 0 ? prev_z : rz;
        win.d[1] = lane == 0 ? prev_w : rw;
        win.d[2] = v[r].x;
        win.d[3] = v[r].y;
        win.d[4] = v[r].z;
        win.d[5] = v[r].w;
        prev_z = rz;
        prev_w = rw;

        const uint32_t chunk = wbase + r * kWaveSize + lane;
        const uint32_t i0 = (chunk < n_full ? chunk : wbase) * kVec;
        const uint32_t c = p.divT.div(i0);
        const uint32_t t0 = i0 - c * T;
        uint32_t hp = kNone, hrow = c, lead = 0;
        if (t0 == 0) hp = i0;
        else if (t0 + kVec > T) { hp = i0 + (T - t0); hrow = c + 1; }   // next row starts inside
        else if (t0 < uint32_t(H)) lead = H - t0;      // those outputs belong to the row's owner
        const PairTaps<W> ta = shfl_taps<W>(rt, int(c - c_first));
        const PairTaps<W> tb = shfl_taps<W>(rt, int(hrow - c_first));
        uint32_t h2[(H + 1) / 2], x2[(H + 1) / 2];
#pragma unroll
        for (int k = 0; k < (H + 1) / 2; ++k) {
            h2[k] = uint32_t(__shfl(int(hpk[k]), int(hrow - c_first)));
            x2[k] = uint32_t(__shfl(int(xpk[k]), int(hrow - c_first)));
        }
        if (chunk >= n_full) continue;                 // ragged tail: element path below

        if (hp == kNone) {
            const u32x4 o = fast_chunk<W, SILU>(win, ta);
            if (lead == 0) {
                st16_stream(p.out + size_t(i0), o);
            } else {
#pragma unroll
                for (int j = 0; j < kVec; ++j)
                    if (j >= int(lead)) p.out[size_t(i0) + j] = lane_elem(o, j);
            }
            continue;
        }
        uint32_t h[H];
#pragma unroll
        for (int k = 0; k < H; ++k) h[k] = (h2[k >> 1] >> ((k & 1) * 16)) & 0xffffu;
        st16_stream(p.out + size_t(i0), head_chunk<W, SILU>(win, i0, hp, ta, tb, h));
        // head outputs past the chunk: u = history ++ row, output j uses u[j .. j+H]
#pragma unroll
        for (int j = 0; j < H; ++j) {
            if (hp + j < i0 + kVec) continue;
            float acc = tb.b;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int m = j + k;                   // index into history ++ row
                const uint32_t bits = m < H ? (h2[m >> 1] >> ((m & 1) * 16))
                                            : (x2[(m - H) >> 1] >> (((m - H) & 1) * 16));
                acc = __builtin_fmaf(tap_of<W>(tb, k), bf_one(uint16_t(bits & 0xffffu)), acc);
            }
            p.out[size_t(hp) + j] = to_bf16(act<SILU>(acc));
        }
    }
    // the row lanes write the new states of the rows this wave owns
    if (row_own && p.sb.cs) {
        uint16_t *cs_line = p.sb.cs + s0.line * p.sb.cs_sl;
#pragma unroll
        for (int k = 0; k < H; ++k)
            cs_line[int64_t(my_row) * p.sb.cs_sd + k * p.sb.cs_st] = uint16_t(rn[k]);
    }
#pragma unroll 1
    for (int r = 0; r < ROUNDS; ++r) {
        const uint32_t chunk = wbase + r * kWaveSize + lane;
        if (chunk >= n_full && chunk < p.n_chunks) slow_chunk<W, SILU>(p, p.sb.qsl, chunk * kVec);
    }
}

// One sequence with very short rows (T < kShortMinT): one lane per channel
// row holds the row's history and inputs in registers.
constexpr int kRowsBlock = 256;

template <int W, bool SILU>
__global__ __launch_bounds__(kRowsBlock) void fwd_tok_rows_kernel(FwdTokParams p) {
    constexpr int H = W - 1;
    constexpr int kMaxT = kShortMinT - 1;
    const uint32_t c0 = blockIdx.x * uint32_t(kRowsBlock);            // the block's first row
    const int32_t c = int32_t(c0) + int32_t(threadIdx.x);
    if (c >= p.dim) return;
    // The block's rows and taps go out first, through descriptors based at
    // the block's first row (wave-uniform), so no load waits on a branch:
    // a lane reads its whole row (T < 16; past T reads 0).
    const uint32_t n_rows = uint32_t(p.dim) - c0 < uint32_t(kRowsBlock) ? uint32_t(p.dim) - c0
                                                                         : uint32_t(kRowsBlock);
    const uint32_t T = p.T;
    const Rsrc xr = make_rsrc(p.x + size_t(c0) * T, int64_t(n_rows) * T * 2);
    const uint32_t xo = uint32_t(threadIdx.x) * T;
    uint16_t row[kMaxT];
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) row[t] = buf_ld16(xr, uint32_t(t) < T ? (xo + t) * 2 : kOob);
    const Rsrc wr = make_rsrc(p.w + int64_t(c0) * p.w_sd, int64_t(n_rows) * p.w_sd * 2);
    const Rsrc br = make_rsrc(p.bias_rd + c0, p.bias ? int64_t(n_rows) * 2 : 0);
    Taps<W> tp;
#pragma unroll
    for (int k = 0; k < W; ++k)
        tp.w[k] = bf_one(buf_ld16(wr, uint32_t(int64_t(threadIdx.x) * p.w_sd + k) * 2));
    tp.b = bf_one(buf_ld16(br, uint32_t(threadIdx.x) * 2));
    const SeqInfo s0 = seq_info_scalar(p.sb, 0);
    // the cached history: a descriptor over the block's rows of the line
    const bool rd = s0.init && !s0.skip;
    const Rsrc hr = make_rsrc(rd ? p.sb.cs + s0.line * p.sb.cs_sl + int64_t(c0) * p.sb.cs_sd : p.x,
                              rd ? (int64_t(n_rows - 1) * p.sb.cs_sd + int64_t(H - 1) * p.sb.cs_st + 1) * 2 : 0);
    uint16_t u[H + kMaxT];
#pragma unroll
    for (int k = 0; k < H; ++k)
        u[k] = buf_ld16(hr, uint32_t(int64_t(threadIdx.x) * p.sb.cs_sd + int64_t(k) * p.sb.cs_st) * 2);
    if (s0.skip) return;
    const int32_t a = int32_t(s0.start), L = int32_t(s0.end - s0.start);
    if (L <= 0) return;
    if (a == 0) {                                        // uniform: the row from its start
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) u[H + t] = t < L ? row[t] : uint16_t(0);
    } else {
        const uint16_t *xs = p.x + size_t(c) * T + a;
#pragma unroll
        for (int t = 0; t < kMaxT; ++t) u[H + t] = t < L ? xs[t] : uint16_t(0);
    }
    uint16_t *orow = p.out + size_t(c) * T + a;
#pragma unroll
    for (int t = 0; t < kMaxT; ++t) {
        if (t >= L) break;
        float acc = tp.b;
#pragma unroll
        for (int k = 0; k < W; ++k) acc = __builtin_fmaf(tp.w[k], bf_one(u[t + k]), acc);
        orow[t] = to_bf16(act<SILU>(acc));
    }
    if (p.sb.cs) {
        // new state: u[L .. L+H), picked without dynamic indexing
        uint16_t *st = p.sb.cs + s0.line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd;
#pragma unroll
        for (int k = 0; k < H; ++k) {
            uint16_t hv = 0;
#pragma unroll
            for (int m = 0; m < H + kMaxT; ++m)
                if (m == L + k) hv = u[m];
            st[k * p.sb.cs_st] = hv;
        }
    }
}

// A batch of sequences in rows of at least one wave (total tokens T >=
// 2048), in two launches of one kernel on the same stream:
//   * chunk workgroups stream x as the long kernel does (a wave spans at most
//     two rows, so the row and its taps are wave-uniform), compute every
//     chunk from the plain window and store every element of an unpadded
//     sequence, whole chunks wherever a chunk holds no padded or uncovered
//     token.  A sequence's first width-1 outputs come out wrong here (their
//     windows reach into the previous sequence).  They never touch a state.
//   * head workgroups, launched after them, give one lane to each
//     (sequence, channel): it reads the cached history (when the sequence
//     continues from it), rewrites the first width-1 outputs, and writes the
//     new state -- the single reader and writer of that history.
// Stream order puts every head write after the chunk writes it replaces.
// (Leaving the head elements to the head lanes alone split every line that
// holds a sequence start between two writers and cost each boundary chunk
// several narrow stores: measured 8% of the batch.)
// query_start_loc and the per-sequence lines and flags are staged in LDS.
constexpr int kVarWaves = 4;                      // waves per block sharing the staged tables
constexpr uint32_t kHeadChans = 16;               // channels of a head workgroup
constexpr uint32_t kHeadSeqs = kVarWaves * kWaveSize / kHeadChans;   // its sequences (16)

// K adjacent bf16 values from p through vector loads of only the dwords
// that hold them (as sld_run, in vector registers).
template <int K>
__device__ __forceinline__ U16Run<K> vld_run(const uint16_t *p) {
    constexpr int N = K / 2 + 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uint32_t *q = reinterpret_cast<const uint32_t *>(a & ~uintptr_t(3));
    const uint32_t m = uint32_t(a >> 1) & 1u;
    uint32_t raw[N];
#pragma unroll
    for (int i = 0; i < N - 1; ++i) raw[i] = q[i];
    raw[N - 1] = (K & 1) ? q[N - 1] : q[N - 2 + m];
    U16Run<K> r;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint64_t hi = i + 1 < N ? uint64_t(raw[i + 1]) << 32 : 0;
        r.d[i] = uint32_t((hi | raw[i]) >> (16 * m));
    }
    return r;
}

// K adjacent bf16 values from element `flat` of a descriptor's array, in
// one load of the dwords that hold them (past the extent: 0).
template <int K>
__device__ __forceinline__ U16Run<K> bld_run(Rsrc r, uint32_t flat) {
    constexpr int N = K / 2 + 1;
    const uint32_t m = flat & 1u;
    const uint32_t off = (flat - m) * 2u;
    uint32_t raw[N];
    if constexpr (N == 1) {
        raw[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
    } else if constexpr (N == 2) {
        const u32x2 v = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
        raw[0] = v.x; raw[1] = v.y;
    } else {
        const u32x3 v = __builtin_bit_cast(u32x3, __builtin_amdgcn_raw_buffer_load_b96(r, off, 0, 0));
        raw[0] = v.x; raw[1] = v.y; raw[2] = v.z;
    }
    U16Run<K> res;
#pragma unroll
    for (int i = 0; i < N; ++i)
        res.d[i] = __builtin_amdgcn_alignbit(i + 1 < N ? raw[i + 1 < N ? i + 1 : 0] : 0u, raw[i], 16 * m);
    return res;
}

template <int W, bool SILU, bool SMALLB>
__global__ __launch_bounds__(kVarWaves * kWaveSize) void fwd_tok_varlen_kernel(FwdTokParams p,
                                                                                uint32_t chunk_blocks,
                                                                                uint32_t block0) {
    constexpr int H = W - 1;
    // The table: staged in LDS for the workgroup, or (batches of at most 64
    // sequences) copied by each wave from its lanes' registers into its own
    // LDS rows, which needs no barrier.
    __shared__ int32_t qsl[SMALLB ? 1 : kQslLdsMax];    // the host guarantees batch + 1 fits
    __shared__ uint8_t skip_of[SMALLB ? 1 : kQslLdsMax];
    __shared__ int32_t wqsl[SMALLB ? kVarWaves : 1][kWaveSize + 1];
    __shared__ uint8_t wskip[SMALLB ? kVarWaves : 1][kWaveSize];
    const int32_t B = p.sb.batch;
    const uint32_t T = p.T;

    // A chunk wave issues its x loads before the table is staged (or, for
    // small batches, right after reading its lanes' entries), so the
    // staging's round trip and barrier overlap them.  Full chunks go through
    // a descriptor that ends at the last one (no branch); only the last wave
    // reads a ragged last chunk element by element.  The wave-uniform rows'
    // taps and the 4 elements before the wave are scalar loads issued next.
    const int lane = threadIdx.x & (kWaveSize - 1);
    const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWaveSize);
    const uint32_t bid = blockIdx.x + block0;               // chunk blocks, then head blocks
    if (bid >= chunk_blocks) {
        // ---- head lanes, in their own launch after the chunk lanes' (no
        // staging: a lane reads only its own sequence's entries).  A
        // workgroup takes kHeadSeqs sequences x kHeadChans channels (channel
        // fastest), the workgroups of one channel group next to each other.  Sequence s's last inputs and s+1's first
        // inputs lie in the same line of a row, so neighbouring sequences'
        // lanes read each row's boundary lines once from HBM; a sequence's
        // states are kHeadChans * (width-1) contiguous values.
        const uint32_t hb = bid - chunk_blocks;
        const uint32_t sgroups = (uint32_t(B) + kHeadSeqs - 1) / kHeadSeqs;
        const uint32_t cg = hb / sgroups, sg = hb - cg * sgroups;
        const int32_t sq = int32_t(sg * kHeadSeqs + threadIdx.x / kHeadChans);
        const uint32_t c = cg * kHeadChans + threadIdx.x % kHeadChans;
        if (sq >= B || c >= uint32_t(p.dim)) return;
        // the lane's own sequence entries, its taps: one round trip
        const int32_t q0 = p.sb.qsl[sq], q1 = p.sb.qsl[sq + 1];
        const int64_t line = p.sb.cache_idx ? int64_t(p.sb.cache_idx[sq]) : int64_t(sq);
        const bool init = p.sb.cs && p.sb.has_init && p.sb.has_init[sq] != 0;
        const Taps<W> tp = load_taps<W>(p, c);
        const int64_t st = q0 < 0 ? 0 : (q0 > int32_t(T) ? int64_t(T) : int64_t(q0));
        const int64_t en = q1 < st ? st : (q1 > int32_t(T) ? int64_t(T) : int64_t(q1));
        const int64_t L = en - st;
        const bool skip = (p.sb.cache_idx && line == p.sb.pad_slot_id) ||
                          (p.sb.cs && (line < 0 || line >= p.sb.num_lines));
        if (L <= 0 || skip) return;
        // every load at once, from addresses valid whether or not the value is
        // wanted (the values are selected afterwards)
        const size_t row0 = size_t(c) * T;
        const uint16_t *hbase = init ? p.sb.cs + line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd : p.x + row0;
        // the sequence's first and last width-1 inputs as two runs of the row
        // (a first run that would pass the row's end starts d earlier)
        const int64_t xs = st + H <= int64_t(T) ? st : int64_t(T) - H;
        const int d = int(st - xs);
        // (one load per run through a descriptor at x when x spans less than
        // 2^31 bytes, else the dwords one by one).  The descriptor ends with
        // the dword that holds x's last element, which the one-by-one reads
        // touch as well; a dword-aligned read that holds a valid element
        // stays in its page, and dwords past that end read 0.
        U16Run<H> xrun, nrun;
        const int64_t ns = L >= H ? en - H : xs;
        const int64_t x_bytes = (int64_t(p.n_elems) * 2 + 3) & ~int64_t(3);
        if (x_bytes < (int64_t(1) << 31)) {                     // launch-uniform
            const Rsrc xa = make_rsrc(p.x, x_bytes);
            xrun = bld_run<H>(xa, uint32_t(row0 + size_t(xs)));
            nrun = bld_run<H>(xa, uint32_t(row0 + size_t(ns)));
        } else {
            xrun = vld_run<H>(p.x + row0 + size_t(xs));
            nrun = vld_run<H>(p.x + row0 + size_t(ns));
        }
        uint32_t h[H], xh[H], nb[H];
#pragma unroll
        for (int q = 0; q < H; ++q) {
            const uint16_t hv = hbase[init ? q * p.sb.cs_st : 0];
            uint32_t xv = xrun.elem(q);
#pragma unroll
            for (int e = 1; e < H; ++e)
                if (d == e && q + e < H) xv = xrun.elem(q + e < H ? q + e : 0);
            h[q] = init ? hv : 0u;
            xh[q] = q < L ? xv : 0u;
            nb[q] = nrun.elem(q);
        }
        // outputs j < min(L, H): u = history ++ sequence, output j uses u[j .. j+H]
#pragma unroll
        for (int j = 0; j < H; ++j) {
            if (j >= L) break;
            float acc = tp.b;
#pragma unroll
            for (int k = 0; k < W; ++k) {
                const int m = j + k;                   // compile-time: a register, not an index
                const uint32_t bits = m < H ? h[m < H ? m : 0] : xh[m - H < H ? m - H : 0];
                acc = __builtin_fmaf(tp.w[k], bf_one(uint16_t(bits)), acc);
            }
            p.out[row0 + size_t(st) + j] = to_bf16(act<SILU>(acc));
        }
        if (p.sb.cs) {
            // new state: the last H entries of history ++ sequence
#pragma unroll
            for (int q = 0; q < H; ++q) {
                uint32_t bits = nb[q];
#pragma unroll
                for (int e = 0; e < H; ++e) {
                    if (L + q == e) bits = h[e];
                    if (L < H && L + q == H + e) bits = xh[e];
                }
                p.sb.cs[line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd + q * p.sb.cs_st] = uint16_t(bits);
            }
        }
        return;
    }

    const uint32_t wbase = (bid * kVarWaves + wave) * uint32_t(kChunksPerWave);
    const uint32_t n_full = p.n_elems / kVec;
    const bool chunk_wave = bid < chunk_blocks && wbase < p.n_chunks;
    constexpr int kNt = 2;                                  // non-temporal cache policy bit
    const uint32_t n_mine = chunk_wave && wbase < n_full
                                ? (n_full - wbase < uint32_t(kChunksPerWave) ? n_full - wbase : uint32_t(kChunksPerWave))
                                : 0u;
    const uint32_t e_first = wbase * kVec;
    const uint32_t cA = chunk_wave ? p.divT.div(e_first) : 0u;
    // wave-uniform rows (at most two)
    const uint32_t row_a = cA * T, row_end = row_a + T;
    const uint32_t e_end = e_first + kWaveElems <= p.n_elems ? e_first + kWaveElems : p.n_elems;

    // Batches of at most 64 sequences read the table first, one sequence per
    // lane (the lanes keep it; the chunk path below copies it into the
    // wave's LDS rows).  A chunk whose tokens all lie in padded sequences is
    // never stored and feeds no stored output (an output at position width-1
    // or later of a sequence reads that sequence's inputs only; earlier ones
    // are rewritten by the head launch), so its load is skipped.  Larger
    // batches load every chunk.
    uint32_t dead = 0;                                      // bit r: round r's chunk
    int32_t a = 0, b = 0;                                   // lane q: query_start_loc[q], [q+1]
    bool pad = false;                                       // lane q: sequence q is padded
    if (SMALLB && chunk_wave) {
        if (lane < B) {
            a = p.sb.qsl[lane];
            b = p.sb.qsl[lane + 1];
            const int64_t line = p.sb.cache_idx ? int64_t(p.sb.cache_idx[lane]) : int64_t(lane);
            pad = (p.sb.cache_idx && line == p.sb.pad_slot_id) ||
                  (p.sb.cs && (line < 0 || line >= p.sb.num_lines));
        }
        // the sequence's tokens clamped into [0, T], as the chunk lanes see them
        const int32_t st = a < 0 ? 0 : (int64_t(a) > int64_t(T) ? int32_t(T) : a);
        const int32_t en = b < st ? st : (int64_t(b) > int64_t(T) ? int32_t(T) : b);
        const int64_t ta0 = int64_t(e_first) - int64_t(row_a);           // row A: [ta0, ta1)
        const int64_t ta1 = int64_t(e_end < row_end ? e_end : row_end) - int64_t(row_a);
        const int64_t tb1 = e_end > row_end ? int64_t(e_end - row_end) : 0;   // row B: [0, tb1)
        uint64_t m = __ballot(pad && st < en && ((st < ta1 && en > ta0) || st < tb1));
        while (m) {
            const int q = __builtin_ctzll(m);
            m &= m - 1;
            const uint32_t s = uint32_t(__builtin_amdgcn_readlane(st, q));
            const uint32_t e = uint32_t(__builtin_amdgcn_readlane(en, q));
#pragma unroll
            for (int r = 0; r < kTokRounds; ++r) {
                const uint32_t i0 = (wbase + r * kWaveSize + lane) * kVec;
                // the chunk's first token in its row (a chunk across the row end: none)
                const uint32_t t = i0 + kVec <= row_end ? i0 - row_a : (i0 >= row_end ? i0 - row_end : kOob);
                if (t != kOob && t >= s && t + kVec <= e) dead |= 1u << r;
            }
        }
    }

    const Rsrc xr = make_rsrc(p.x + size_t(chunk_wave ? wbase : 0) * kVec, int64_t(n_mine) * 16);
    u32x4 v[kTokRounds];
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r)
        v[r] = buf_ld128<kNt>(xr, (dead >> r) & 1u ? kOob : uint32_t(r * kWaveSize + lane) * 16u);
    if (chunk_wave && n_mine < uint32_t(kChunksPerWave) && n_full < p.n_chunks) {
#pragma unroll
        for (int r = 0; r < kTokRounds; ++r) {
            const uint32_t ch = wbase + r * kWaveSize + lane;
            if (ch == n_full) v[r] = ld8_partial(p.x + size_t(ch) * kVec, int(p.n_elems - ch * kVec));
        }
    }
    const uint16_t *pp = p.x + (chunk_wave && wbase > 0 ? size_t(wbase) * kVec - 4 : 0);
    uint32_t prev_z = sld_u32(pp), prev_w = sld_u32(pp + 2);
    if (!chunk_wave || wbase == 0) prev_z = prev_w = 0;
    const PairTaps<W> tA = sload_pair_taps<W>(p, cA);
    const PairTaps<W> tB = sload_pair_taps<W>(p, cA + 1 < uint32_t(p.dim) ? cA + 1 : cA);

    if constexpr (!SMALLB) {
        for (int i = threadIdx.x; i <= B; i += kVarWaves * kWaveSize) {
            qsl[i] = p.sb.qsl[i];
            if (i < B) {
                const int64_t line = p.sb.cache_idx ? int64_t(p.sb.cache_idx[i]) : int64_t(i);
                skip_of[i] = (p.sb.cache_idx && line == p.sb.pad_slot_id) ||
                             (p.sb.cs && (line < 0 || line >= p.sb.num_lines));
            }
        }
        __syncthreads();
    }

    // ---- chunk lanes
    if (!chunk_wave) return;
    if constexpr (SMALLB) {
        if (lane < B) {
            wqsl[wave][lane] = a;
            wskip[wave][lane] = pad ? 1 : 0;
        }
        if (lane == B - 1) wqsl[wave][B] = b;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's rows, before its reads
    }
    const int32_t *tq = SMALLB ? &wqsl[wave][0] : qsl;
    const uint8_t *tskip = SMALLB ? &wskip[wave][0] : skip_of;

    // sequence bounds clamped into [0, T], as the head lanes see them
    auto bounds = [&](int32_t q, int64_t &st, int64_t &en) {
        st = tq[q] < 0 ? 0 : (tq[q] > int32_t(T) ? int64_t(T) : int64_t(tq[q]));
        en = tq[q + 1] < st ? st : (tq[q + 1] > int32_t(T) ? int64_t(T) : int64_t(tq[q + 1]));
    };
    // the sequence of the wave's first element; lanes of the first row walk
    // forward from it (a wave spans a few sequences), the second row searches
    int32_t s_wave;
    if constexpr (SMALLB) {
        // the last sequence starting at or before the wave's first token:
        // one ballot over the lanes' starts instead of a search
        const uint32_t n = uint32_t(__builtin_popcountll(
            __ballot(lane < B && int64_t(a) <= int64_t(e_first - row_a))));
        s_wave = n > 0 ? int32_t(n) - 1 : 0;
    } else {
        s_wave = __builtin_amdgcn_readfirstlane(seq_search(tq, B, int64_t(e_first - row_a)));
    }

    const int src_lane = (lane + kWaveSize - 1) & (kWaveSize - 1);
    uint32_t hz[kTokRounds], hw[kTokRounds];
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t rz = uint32_t(__shfl(int(v[r].z), src_lane));
        const uint32_t rw = uint32_t(__shfl(int(v[r].w), src_lane));
        hz[r] = lane == 0 ? prev_z : rz;
        hw[r] = lane == 0 ? prev_w : rw;
        prev_z = rz;
        prev_w = rw;
    }

    // A wave inside one row whose tokens all belong to unpadded sequences
    // stores every chunk whole, with no per-lane sequence work (the first
    // width-1 outputs of the sequences that start in it are rewritten by the
    // head launch).  Deciding it is a short wave-uniform walk of the table.
    bool plain = e_end <= row_end;
    if (plain) {
        asm volatile("");
        const int64_t ta0 = int64_t(e_first) - int64_t(row_a);     // the wave's tokens [ta0, ta1)
        const int64_t ta1 = ta0 + int64_t(e_end - e_first);
        if constexpr (SMALLB) {
            plain = int64_t(__builtin_amdgcn_readlane(a, 0)) <= ta0 &&
                    int64_t(__builtin_amdgcn_readlane(b, B - 1)) >= ta1 &&
                    __ballot(lane < B && lane >= s_wave && int64_t(a) < ta1 && pad) == 0;
        } else {
            plain = int64_t(__builtin_amdgcn_readfirstlane(tq[0])) <= ta0 &&
                    int64_t(__builtin_amdgcn_readfirstlane(tq[B])) >= ta1;
            for (int32_t q = s_wave; plain && q < B; ++q) {
                if (int64_t(__builtin_amdgcn_readfirstlane(tq[q])) >= ta1) break;
                if (__builtin_amdgcn_readfirstlane(int32_t(tskip[q])) != 0) plain = false;
            }
        }
    }
    if (plain) {
        asm volatile("");
        const Rsrc outr = make_rsrc(p.out + size_t(wbase) * kVec, int64_t(n_mine) * 16);
#pragma unroll
        for (int r = 0; r < kTokRounds; ++r) {
            const uint32_t rel = uint32_t(r * kWaveSize + lane);
            const uint32_t chunk = wbase + rel;
            Window win;
            win.d[0] = hz[r];
            win.d[1] = hw[r];
            win.d[2] = v[r].x;
            win.d[3] = v[r].y;
            win.d[4] = v[r].z;
            win.d[5] = v[r].w;
            const u32x4 o = fast_chunk<W, SILU>(win, tA);
            // full chunks through the descriptor (past its end: dropped)
            __builtin_amdgcn_raw_buffer_store_b128(o, outr, rel * 16u, 0, kNt);
            if (chunk == n_full && chunk < p.n_chunks)               // the ragged last chunk
                st8_partial(p.out + size_t(chunk) * kVec, o, int(p.n_elems - chunk * kVec), true);
        }
        return;
    }

#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t chunk = wbase + r * kWaveSize + lane;
        if (chunk >= p.n_chunks) continue;
        const uint32_t i0 = chunk * kVec;
        const uint32_t n = chunk < n_full ? uint32_t(kVec) : p.n_elems - i0;   // elements present
        const bool in_b = i0 >= row_end;
        const int64_t t0 = int64_t(i0) - int64_t(in_b ? row_end : row_a);
        // the sequence of the first element, and whether the chunk is plain:
        // one row, unpadded sequences only
        int32_t sq = in_b ? seq_search(tq, B, t0) : s_wave;
        if (!in_b)
            while (sq + 1 < B && tq[sq + 1] <= t0) ++sq;
        int64_t st, en;
        bounds(sq, st, en);
        const bool row_cross = !in_b && i0 + n > row_end;
        auto bits = [](int64_t a, int64_t b) {         // elements [a, b) of a chunk, 0 <= a <= b <= 8
            return ((1u << uint32_t(b)) - 1u) & ~((1u << uint32_t(a)) - 1u);
        };
        // The common cases without a loop: a whole chunk inside one row that
        // starts inside sequence sq and holds at most one more sequence
        // start.  An element is kept when its sequence is not padded.  (The
        // next sequence's bounds and pad flag are read with sq's, in one
        // round of LDS reads.)
        uint32_t keep = 0;                             // bit j: store element j
        bool done = false;
        if (n == uint32_t(kVec) && !row_cross && t0 >= st && t0 < en) {
            const int64_t ea = en - t0 < kVec ? en - t0 : kVec;     // elements of sq: [0, ea)
            const int64_t ka = st - t0 > 0 ? st - t0 : 0;            // the first of sq
            const int32_t s2 = sq + 1 < B ? sq + 1 : sq;
            int64_t st2, en2;
            bounds(s2, st2, en2);
            const bool pad1 = tskip[sq] != 0, pad2 = tskip[s2] != 0;
            if (ka < ea && !pad1) keep = bits(ka, ea);
            if (ea == kVec) {
                done = true;
            } else if (s2 != sq && st2 == en && en2 >= t0 + kVec) {
                const int64_t kb = st2 - t0;                         // == ea
                if (kb < kVec && !pad2) keep |= bits(kb, kVec);
                done = true;
            }
        }
        if (!done) {
            keep = 0;
            // segment by segment (a run of elements of one sequence of one
            // row): keep those of an unpadded sequence
            int64_t row_base = in_b ? int64_t(row_end) : int64_t(row_a);
            uint32_t j = 0;
            while (j < n) {
                int64_t t = int64_t(i0) + j - row_base;
                if (t >= int64_t(T)) {                 // crossed into the next row
                    row_base += T;
                    t -= T;
                    sq = seq_search(tq, B, t);
                    bounds(sq, st, en);
                } else if (t >= en) {
                    while (sq + 1 < B && tq[sq + 1] <= t) ++sq;
                    bounds(sq, st, en);
                }
                if (t < st || t >= en) {               // a token no sequence covers
                    ++j;
                    continue;
                }
                const uint32_t jend = uint32_t(en - t) < n - j ? j + uint32_t(en - t) : n;
                if (!tskip[sq]) keep |= ((1u << jend) - 1u) & ~((1u << j) - 1u);
                j = jend;
            }
        }
        if (!keep) continue;
        Window win;
        win.d[0] = hz[r];
        win.d[1] = hw[r];
        win.d[2] = v[r].x;
        win.d[3] = v[r].y;
        win.d[4] = v[r].z;
        win.d[5] = v[r].w;
        u32x4 o = fast_chunk<W, SILU>(win, in_b ? tB : tA);
        if (row_cross) {                               // elements from row_end on use the next row's taps
            const u32x4 ob = fast_chunk<W, SILU>(win, tB);
            const uint32_t kb = row_end - i0;
            const uint32_t av[4] = {o.x, o.y, o.z, o.w}, bv[4] = {ob.x, ob.y, ob.z, ob.w};
            uint32_t rr[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t lo = (2 * d < int(kb) ? av[d] : bv[d]) & 0xffffu;
                const uint32_t hi = (2 * d + 1 < int(kb) ? av[d] : bv[d]) & 0xffff0000u;
                rr[d] = lo | hi;
            }
            o = u32x4{rr[0], rr[1], rr[2], rr[3]};
        }
        if (keep == 0xffu) {
            st16_stream(p.out + size_t(i0), o);
        } else {
            // a pair of kept elements is one 4-byte store, a lone one a
            // 2-byte store (the chunk is 16-byte aligned)
            const uint32_t ov[4] = {o.x, o.y, o.z, o.w};
            uint32_t *o32 = reinterpret_cast<uint32_t *>(p.out + size_t(i0));
#pragma unroll
            for (int d = 0; d < kVec / 2; ++d) {
                const uint32_t m2 = (keep >> (2 * d)) & 3u;
                if (m2 == 3u) o32[d] = ov[d];
                else if (m2 == 1u) p.out[size_t(i0) + 2 * d] = uint16_t(ov[d] & 0xffffu);
                else if (m2 == 2u) p.out[size_t(i0) + 2 * d + 1] = uint16_t(ov[d] >> 16);
            }
        }
    }
}

template <int W, bool SILU, bool VARLEN>
__global__ __launch_bounds__(kTokWavesPerBlock * kWaveSize) void fwd_tokmajor_kernel(FwdTokParams p) {
    constexpr int H = W - 1;
    __shared__ int32_t s_qsl[VARLEN ? kQslLdsMax : 1];
    const int32_t *qsl = p.sb.qsl;
    if constexpr (VARLEN) {
        if (p.sb.batch + 1 <= kQslLdsMax) {
            for (int i = threadIdx.x; i <= p.sb.batch; i += kTokWavesPerBlock * kWaveSize)
                s_qsl[i] = p.sb.qsl[i];
            __syncthreads();
            qsl = s_qsl;
        }
    }

    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = threadIdx.x / kWaveSize;
    const uint32_t tile = blockIdx.x;
    const uint32_t wbase = (tile * kTokWavesPerBlock + wave) * uint32_t(kChunksPerWave);
    if (wbase >= p.n_chunks) return;

    const uint32_t T = p.T;
    const uint32_t n_full = p.n_elems / kVec;

    // Issue every load of the wave first.
    u32x4 v[kTokRounds];
    if (wbase + kChunksPerWave <= n_full) {
#pragma unroll
        for (int r = 0; r < kTokRounds; ++r)
            v[r] = ld16(p.x + size_t(wbase + r * kWaveSize + lane) * kVec);
    } else {
#pragma unroll
        for (int r = 0; r < kTokRounds; ++r) {
            const uint32_t ch = wbase + r * kWaveSize + lane;
            if (ch < n_full) v[r] = ld16(p.x + size_t(ch) * kVec);
            else v[r] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t prev_z = 0, prev_w = 0;     // lane 0: tail (elements 4..7) of the chunk before
    if (lane == 0 && wbase > 0) {
        const u32x2 t2 = *reinterpret_cast<const u32x2 *>(p.x + size_t(wbase) * kVec - 4);
        prev_z = t2.x;
        prev_w = t2.y;
    }

    // Wave-uniform row bookkeeping.
    const uint32_t e_first = wbase * kVec;
    const uint32_t cA = p.divT.div(e_first);
    const uint32_t row_end = (cA + 1) * T;                 // first element of row cA+1
    const uint32_t e_last = (e_first + kWaveElems <= p.n_elems ? e_first + kWaveElems : p.n_elems) - 1;
    const bool two_rows = uint64_t(e_last) < uint64_t(row_end) + T;
    PairTaps<W> tA, tB;
    if (two_rows) {
        tA = uniform(load_pair_taps<W>(p, cA));
        tB = (cA + 1 < uint32_t(p.dim)) ? uniform(load_pair_taps<W>(p, cA + 1)) : tA;
    }
    SeqInfo s0;
    if constexpr (!VARLEN) s0 = seq_info(p.sb, qsl, 0);
    SeqCache sc;

    // Halo of every round first (each permute waits only for its own load).
    const int src_lane = (lane + kWaveSize - 1) & (kWaveSize - 1);
    uint32_t hz[kTokRounds], hw[kTokRounds];
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t rz = uint32_t(__shfl(int(v[r].z), src_lane));
        const uint32_t rw = uint32_t(__shfl(int(v[r].w), src_lane));
        hz[r] = lane == 0 ? prev_z : rz;
        hw[r] = lane == 0 ? prev_w : rw;
        prev_z = rz;
        prev_w = rw;
    }

    // Compute every fast chunk into registers, then store them back to back:
    // a store inside the round loop would make the next round wait for it.
    u32x4 o[kTokRounds];
    uint32_t done = 0, slow = 0;
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t chunk = wbase + r * kWaveSize + lane;
        if (chunk >= p.n_chunks) continue;
        const uint32_t i0 = chunk * kVec;
        uint32_t t0;
        PairTaps<W> tp;
        if (two_rows) {
            const bool in_b = i0 >= row_end;
            t0 = i0 - (in_b ? row_end : row_end - T);
            tp = select(in_b, tB, tA);
        } else {
            const uint32_t c = p.divT.div(i0);
            t0 = i0 - c * T;
            tp = load_pair_taps<W>(p, c);
        }
        bool fast = chunk < n_full && t0 + kVec <= T;
        if (fast) {
            const SeqInfo &si = VARLEN ? sc.get(p.sb, qsl, t0) : s0;
            fast = !si.skip && int64_t(t0) >= si.start + H && int64_t(t0) + kVec <= si.end;
        }
        if (fast) {
            Window win;
            win.d[0] = hz[r];
            win.d[1] = hw[r];
            win.d[2] = v[r].x;
            win.d[3] = v[r].y;
            win.d[4] = v[r].z;
            win.d[5] = v[r].w;
            o[r] = fast_chunk<W, SILU>(win, tp);
            done |= 1u << r;
        } else {
            slow |= 1u << r;
        }
    }
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r)
        if (done & (1u << r))
            st16_stream(p.out + size_t(wbase + r * kWaveSize + lane) * kVec, o[r]);
    // Deferred boundary chunks (rare): element by element.
#pragma unroll 1
    for (int r = 0; r < kTokRounds; ++r)
        if (slow & (1u << r)) slow_chunk<W, SILU>(p, qsl, (wbase + r * kWaveSize + lane) * kVec);
}

template <int W, bool SILU>
hipError_t launch_ws(const FwdTokParams &p, hipStream_t s) {
    const uint32_t blocks = (p.n_chunks + kTokWavesPerBlock * kChunksPerWave - 1) /
                            (kTokWavesPerBlock * kChunksPerWave);
    const dim3 grid(blocks), block(kTokWavesPerBlock * kWaveSize);
    if (p.sb.batch > 1 && p.T >= kWaveElems && p.sb.batch + 1 <= kQslLdsMax) {
        const uint32_t waves = (p.n_chunks + kChunksPerWave - 1) / kChunksPerWave;
        const uint32_t chunk_blocks = (waves + kVarWaves - 1) / kVarWaves;
        const uint32_t head_blocks = ((uint32_t(p.sb.batch) + kHeadSeqs - 1) / kHeadSeqs) *
                                     ((uint32_t(p.dim) + kHeadChans - 1) / kHeadChans);
        // chunk workgroups, then (stream-ordered) the head workgroups that
        // rewrite each sequence's first outputs and write its state
        // (batches of at most 64 sequences keep the table in registers)
        if (p.sb.batch <= kWaveSize)
            fwd_tok_varlen_kernel<W, SILU, true><<<dim3(chunk_blocks), dim3(kVarWaves * kWaveSize), 0, s>>>(
                p, chunk_blocks, 0u);
        else
            fwd_tok_varlen_kernel<W, SILU, false><<<dim3(chunk_blocks), dim3(kVarWaves * kWaveSize), 0, s>>>(
                p, chunk_blocks, 0u);
        const hipError_t e1 = hipGetLastError();
        if (e1 != hipSuccess) return e1;
        fwd_tok_varlen_kernel<W, SILU, false><<<dim3(head_blocks), dim3(kVarWaves * kWaveSize), 0, s>>>(
            p, chunk_blocks, chunk_blocks);
    } else if (p.sb.batch > 1) {
        fwd_tokmajor_kernel<W, SILU, true><<<grid, block, 0, s>>>(p);
    } else if (p.T >= kWaveElems) {
        const dim3 b(kLongWaves * kWaveSize);
        if (p.T >= kLongMidLo && p.T < kLongMidHi) {
            constexpr uint32_t kLB = kLongWaves * kLongRoundsMid * kWaveSize;
            const dim3 g((p.n_chunks + kLB - 1) / kLB);
            fwd_tok_long_kernel<W, SILU, kLongRoundsMid><<<g, b, 0, s>>>(p);
        } else {
            constexpr uint32_t kLB = kLongWaves * kLongRounds * kWaveSize;
            const dim3 g((p.n_chunks + kLB - 1) / kLB);
            const uint32_t lds = p.T >= kLongMidHi ? kLongFourRoundLds : 0u;
            fwd_tok_long_kernel<W, SILU, kLongRounds><<<g, b, lds, s>>>(p);
        }
    } else if (p.T >= uint32_t(kShortMinT)) {
        // Rounds per wave, measured on gfx950: one round (the most waves in
        // flight) up to 512K chunks, two from there, four from 2M, where a
        // wave's row loads are worth amortising; a wave's rows
        // (ROUNDS*512/T + 2) must fit its 64 lanes.
        const uint32_t T = p.T;
        if (T >= 64 && p.n_chunks >= uint32_t(16 * kShortWaves * kWaveSize)) {
            const dim3 g((p.n_chunks + 4 * kWaveSize - 1) / (4 * kWaveSize));
            fwd_tok_short_kernel<W, SILU, 4><<<g, dim3(kWaveSize), 0, s>>>(p);
        } else if (T >= 32 && p.n_chunks >= uint32_t(4 * kShortWaves * kWaveSize)) {
            const dim3 g((p.n_chunks + 2 * kWaveSize - 1) / (2 * kWaveSize));
            fwd_tok_short_kernel<W, SILU, 2><<<g, dim3(kWaveSize), 0, s>>>(p);
        } else {
            const dim3 g((p.n_chunks + kWaveSize - 1) / kWaveSize);
            fwd_tok_short_kernel<W, SILU, 1><<<g, dim3(kWaveSize), 0, s>>>(p);
        }
    } else {
        const dim3 g((uint32_t(p.dim) + kRowsBlock - 1) / kRowsBlock);
        fwd_tok_rows_kernel<W, SILU><<<g, dim3(kRowsBlock), 0, s>>>(p);
    }
    return hipGetLastError();
}

template <int W>
hipError_t launch_w(const FwdTokParams &p, bool silu, hipStream_t s) {
    return silu ? launch_ws<W, true>(p, s) : launch_ws<W, false>(p, s);
}

}  // namespace

hipError_t launch_fwd_tokmajor(const FwdTokParams &p, int width, bool silu, hipStream_t s) {
    switch (width) {
        case 2: return launch_w<2>(p, silu, s);
        case 3: return launch_w<3>(p, silu, s);
        case 4: return launch_w<4>(p, silu, s);
        case 5: return launch_w<5>(p, silu, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace sconv

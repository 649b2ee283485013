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
// chunk: it comes from the neighbouring lane with a cross-lane rotate, and
// lane 0 takes lane 63's tail from the previous round (one 8-byte load per
// wave for round 0).
//
// Fast path: the chunk lies inside one row and one sequence, at least
// width-1 tokens past the sequence start -> all taps are in registers.
// Slow path (rare: row or sequence boundaries, the first width-1 tokens of a
// sequence, the ragged tail): element by element.  The element holding a
// sequence's first token owns that sequence's history: it alone reads the
// cached state, computes the first width-1 outputs (possibly spilling into
// the next chunk) and writes the new state, so no other lane can read a
// state that has already been overwritten.
#include "sconv_device.h"

namespace sconv {

namespace {

// Weights and bias of one channel, widened to fp32.
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

// One element whose taps lie partly in the history h (bits, oldest first):
// element with local index tl < width-1 reads h for negative offsets.
template <int W, bool SILU>
__device__ __forceinline__ uint16_t head_output(const Taps<W> &tp, const uint16_t *h,
                                                const uint16_t *xseq, int tl) {
    float acc = tp.b;
#pragma unroll
    for (int k = 0; k < W; ++k) {
        const int idx = tl - (W - 1) + k;
        const uint16_t v = idx >= 0 ? xseq[idx] : h[(W - 1) + idx];
        acc = __builtin_fmaf(tp.w[k], bf_one(v), acc);
    }
    return to_bf16(act<SILU>(acc));
}

// Element-by-element processing of one chunk.  e[] holds the bits of flat
// elements i0-(W-1) .. i0+7 (entries before element 0 of the tensor are
// never used: such elements are the start of row 0 and read history).
template <int W, bool SILU>
__device__ void slow_chunk(const FwdTokParams &p, const int32_t *qsl, uint32_t i0,
                           const uint16_t *e, uint32_t cA, const Taps<W> &tA,
                           const Taps<W> &tB) {
    const uint32_t T = p.T;
    uint32_t c = p.divT.div(i0);
    uint32_t t = i0 - c * T;
    Taps<W> tp = (c == cA) ? tA : (c == cA + 1 ? tB : load_taps<W>(p, c));
    int32_t s = -1;
    SeqInfo si;
    si.start = 0; si.end = 0; si.line = 0; si.skip = true; si.init = false;
    for (int j = 0; j < 8; ++j) {
        const uint32_t i = i0 + j;
        if (i >= p.n_elems) break;
        if (j > 0 && ++t == T) {           // crossed into the next channel row
            t = 0;
            ++c;
            tp = (c == cA) ? tA : (c == cA + 1 ? tB : load_taps<W>(p, c));
        }
        if (s < 0 || int64_t(t) < si.start || int64_t(t) >= si.end) {
            s = p.sb.batch == 1 ? 0 : seq_search(qsl, p.sb.batch, t);
            si = seq_info(p.sb, qsl, s);
        }
        if (si.skip || int64_t(t) < si.start || int64_t(t) >= si.end) continue;
        const int64_t tl = int64_t(t) - si.start;
        if (tl >= 1 && tl <= W - 2) continue;      // owned by the sequence's first token
        uint16_t *orow = p.out + size_t(c) * T;
        if (tl >= W - 1) {                          // every tap inside the row window
            float acc = tp.b;
#pragma unroll
            for (int k = 0; k < W; ++k) acc = __builtin_fmaf(tp.w[k], bf_one(e[j + k]), acc);
            orow[t] = to_bf16(act<SILU>(acc));
            continue;
        }
        // tl == 0: the history owner of (sequence, channel).
        const uint16_t *xseq = p.x + size_t(c) * T + si.start;
        uint16_t h[W - 1];
#pragma unroll
        for (int k = 0; k < W - 1; ++k)
            h[k] = si.init ? p.sb.cs[si.line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd +
                                     k * p.sb.cs_st]
                           : uint16_t(0);
        const int64_t L = si.end - si.start;
        const int nq = L < (W - 1) ? int(L) : (W - 1);
        for (int q = 0; q < nq; ++q) orow[si.start + q] = head_output<W, SILU>(tp, h, xseq, q);
        if (p.sb.cs) {
            uint16_t nh[W - 1];
#pragma unroll
            for (int k = 0; k < W - 1; ++k) {
                const int64_t m = L + k;            // index into h ++ x
                nh[k] = m < (W - 1) ? h[m] : xseq[m - (W - 1)];
            }
#pragma unroll
            for (int k = 0; k < W - 1; ++k)
                p.sb.cs[si.line * p.sb.cs_sl + int64_t(c) * p.sb.cs_sd + k * p.sb.cs_st] = nh[k];
        }
    }
}

template <int W, bool SILU>
__global__ __launch_bounds__(kTokWavesPerBlock * kWaveSize) void fwd_tokmajor_kernel(FwdTokParams p) {
    __shared__ int32_t s_qsl[kQslLdsMax];
    const bool use_lds = p.sb.batch > 1 && p.sb.batch + 1 <= kQslLdsMax;
    if (use_lds) {
        for (int i = threadIdx.x; i <= p.sb.batch; i += blockDim.x) s_qsl[i] = p.sb.qsl[i];
        __syncthreads();
    }
    const int32_t *qsl = use_lds ? s_qsl : p.sb.qsl;

    const int lane = threadIdx.x & (kWaveSize - 1);
    const int wave = threadIdx.x / kWaveSize;
    const uint32_t tile = xcd_tile(blockIdx.x, gridDim.x);
    const uint32_t wbase = (tile * kTokWavesPerBlock + wave) * uint32_t(kWaveSize * kTokRounds);
    if (wbase >= p.n_chunks) return;

    const uint32_t T = p.T;
    const uint32_t n_full = p.n_elems / kVec;

    // Issue every load of the wave first.
    u32x4 v[kTokRounds];
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t ch = wbase + r * kWaveSize + lane;
        if (ch < n_full) {
            v[r] = ld16(p.x + size_t(ch) * kVec);
        } else if (ch < p.n_chunks) {
            v[r] = ld8_partial(p.x + size_t(ch) * kVec, int(p.n_elems - ch * kVec));
        } else {
            v[r] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    uint32_t prev_z = 0, prev_w = 0;     // lane 0: tail (elements 4..7) of the chunk before
    if (lane == 0 && wbase > 0) {
        const u32x2 t2 = *reinterpret_cast<const u32x2 *>(p.x + size_t(wbase) * kVec - 4);
        prev_z = t2.x;
        prev_w = t2.y;
    }

    // The wave spans at most a few rows; the first two rows' taps are uniform.
    const uint32_t cA = p.divT.div(wbase * kVec);
    const Taps<W> tA = load_taps<W>(p, cA);
    const Taps<W> tB = (cA + 1 < uint32_t(p.dim)) ? load_taps<W>(p, cA + 1) : tA;
    SeqInfo s0;
    if (p.sb.batch == 1) s0 = seq_info(p.sb, qsl, 0);

    const int src_lane = (lane + kWaveSize - 1) & (kWaveSize - 1);
#pragma unroll
    for (int r = 0; r < kTokRounds; ++r) {
        const uint32_t rz = uint32_t(__shfl(int(v[r].z), src_lane));
        const uint32_t rw = uint32_t(__shfl(int(v[r].w), src_lane));
        const uint32_t hz = lane == 0 ? prev_z : rz;
        const uint32_t hw = lane == 0 ? prev_w : rw;
        prev_z = rz;
        prev_w = rw;

        const uint32_t chunk = wbase + r * kWaveSize + lane;
        if (chunk >= p.n_chunks) continue;
        const uint32_t i0 = chunk * kVec;
        const uint32_t c = p.divT.div(i0);
        const uint32_t t0 = i0 - c * T;

        bool fast = chunk < n_full && t0 + kVec <= T;
        if (fast) {
            SeqInfo si;
            if (p.sb.batch == 1) si = s0;
            else si = seq_info(p.sb, qsl, seq_search(qsl, p.sb.batch, t0));
            fast = !si.skip && int64_t(t0) >= si.start + (W - 1) && int64_t(t0) + kVec <= si.end;
        }
        if (fast) {
            float e[kVec + W - 1];
            const float hh[4] = {bf_lo(hz), bf_hi(hz), bf_lo(hw), bf_hi(hw)};
#pragma unroll
            for (int k = 0; k < W - 1; ++k) e[k] = hh[4 - (W - 1) + k];
            unpack8(v[r], e + (W - 1));
            const Taps<W> tp = (c == cA) ? tA : (c == cA + 1 ? tB : load_taps<W>(p, c));
            float o[kVec];
#pragma unroll
            for (int j = 0; j < kVec; ++j) {
                float acc = tp.b;
#pragma unroll
                for (int k = 0; k < W; ++k) acc = __builtin_fmaf(tp.w[k], e[j + k], acc);
                o[j] = act<SILU>(acc);
            }
            st16_stream(p.out + size_t(i0), pack8(o));
        } else {
            uint16_t eb[kVec + W - 1];
            const uint16_t hb[4] = {uint16_t(hz & 0xffffu), uint16_t(hz >> 16),
                                    uint16_t(hw & 0xffffu), uint16_t(hw >> 16)};
#pragma unroll
            for (int k = 0; k < W - 1; ++k) eb[k] = hb[4 - (W - 1) + k];
#pragma unroll
            for (int k = 0; k < kVec; ++k) eb[W - 1 + k] = lane_elem(v[r], k);
            slow_chunk<W, SILU>(p, qsl, i0, eb, cA, tA, tB);
        }
    }
}

template <int W>
hipError_t launch_w(const FwdTokParams &p, bool silu, hipStream_t s) {
    const uint32_t per_block = kTokWavesPerBlock * kWaveSize * kTokRounds;
    const uint32_t blocks = (p.n_chunks + per_block - 1) / per_block;
    const dim3 grid(blocks), block(kTokWavesPerBlock * kWaveSize);
    if (silu) fwd_tokmajor_kernel<W, true><<<grid, block, 0, s>>>(p);
    else fwd_tokmajor_kernel<W, false><<<grid, block, 0, s>>>(p);
    return hipGetLastError();
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

// Kernel parameter blocks and launcher declarations shared by the C ABI
// (sconv_api.hip) and the kernel translation units.  Host and device code
// both see these structs: the host fills them, kernels take them by value.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace sconv {

// Exact unsigned 32-bit division by a launch constant d >= 1: with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d == (umulhi(m, n) + n) >> l for every n < 2^32 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994).
struct FastDivU32 {
    uint32_t d;
    uint32_t m;
    uint32_t l;

    static FastDivU32 make(uint32_t d) {
        FastDivU32 f;
        f.d = d;
        uint32_t l = 0;
        while (l < 32 && (uint64_t(1) << l) < d) ++l;
        f.l = l;
        f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
        return f;
    }
    __host__ __device__ uint32_t div(uint32_t n) const {
#if defined(__HIP_DEVICE_COMPILE__)
        uint32_t hi = __umulhi(m, n);
#else
        uint32_t hi = uint32_t((uint64_t(m) * n) >> 32);
#endif
        return uint32_t((uint64_t(hi) + n) >> l);
    }
};

// Everything about the varlen batch that the forward kernels share.
struct SeqBatch {
    const int32_t *qsl;          // [batch + 1]
    const int32_t *cache_idx;    // [batch] or null (line = sequence id)
    const uint8_t *has_init;     // [batch] or null (all false)
    uint16_t *cs;                // conv states or null
    int64_t cs_sl, cs_sd, cs_st; // state strides (line, channel, column)
    int64_t num_lines;
    int32_t batch;
    int32_t pad_slot_id;
    int64_t total_T;
};

struct FwdTokParams {          // token-contiguous (dim, T) storage
    const uint16_t *x;
    uint16_t *out;
    const uint16_t *w;
    int64_t w_sd;
    const uint16_t *bias;      // or null
    SeqBatch sb;
    uint32_t T;                // total tokens (row length)
    FastDivU32 divT;
    uint32_t n_elems;          // dim * T
    uint32_t n_chunks;         // ceil(n_elems / 8)
    int32_t dim;
    // Always-readable stand-ins, so wave-uniform reads need no branch: the
    // bias (or the weights, masked to 0 when there is no bias), the cache
    // indices and has_initial_state (or query_start_loc when absent).
    const uint16_t *bias_rd;
    uint32_t bias_mask;        // 0xffff with a bias, else 0
    const int32_t *ci_rd;
    const uint8_t *hi_rd;
};

struct FwdClParams {           // channel-contiguous (T, dim) storage
    const uint16_t *x;
    uint16_t *out;
    int64_t x_st, o_st;        // row strides (elements, multiples of 8)
    const uint16_t *w;
    int64_t w_sd;
    const uint16_t *bias;
    SeqBatch sb;
    int32_t dim;
    int32_t n_slabs;           // ceil(dim / 256): 256-channel slabs
    FastDivU32 div_slabs;      // division by n_slabs (a wave's tile and slab)
    int32_t bt;                // tokens per wave tile
    int32_t n_tiles;           // ceil(T / bt)
};

// Any storage of x / out: element (c, t) at c * sd + t * st, 64-bit offsets,
// bases aligned to 2 bytes only.  Work is cut into tiles of kGenTile lanes
// along whichever axis of x has the smaller stride, so a wave's reads are
// as close together as the layout allows.
struct FwdGenParams {
    const uint16_t *x;
    uint16_t *out;
    int64_t x_sd, x_st, o_sd, o_st;
    const uint16_t *w;
    int64_t w_sd;
    const uint16_t *bias;      // or null
    SeqBatch sb;
    int32_t dim;
    int64_t T;
    bool lanes_on_tokens;      // a tile is kGenTile tokens of one channel, else
                               // kGenTile channels of one token
    int64_t tiles_per_line;    // tiles along the lane axis
    int64_t n_tiles;
};

struct UpdParams {
    const uint16_t *x;
    int64_t x_sb, x_sd, x_st;
    uint16_t *out;
    int64_t o_sb, o_sd, o_st;
    const uint16_t *w;
    int64_t w_sd;
    const uint16_t *bias;
    uint16_t *cs;
    int64_t cs_sl, cs_sd, cs_st;
    int64_t num_lines;
    const int32_t *cache_idx;
    const int32_t *ring_seen;     // cache_seqlens: inputs seen per entry (ring states)
    const int32_t *num_acc;       // num_accepted_tokens (speculative decoding)
    uint16_t *inter;              // per-step windows [batch][steps][dim][width-1]
    int64_t i_sb, i_st, i_sd, i_sk;
    const int32_t *out_idx;       // per-step destination lines [batch][seqlen]
    int64_t oi_sb, oi_st;
    int32_t state_len;
    int32_t batch, dim, seqlen, pad_slot_id;
};

constexpr int kMaxPagedStreams = 8;              // streams of one paged launch

// One conv stream of the paged cache: its own input / output rows, taps and
// D sub-range [off_s, off_s + ws) of every head; C = num_heads * ws.
struct PagedStream {
    const uint16_t *x;
    uint16_t *out;
    const uint16_t *w;
    const uint16_t *bias;
    int64_t x_st, o_st, w_sd;
    int32_t off_s, ws, C;
    int32_t slab0;      // index of the stream's first 256-channel slab in the launch
};

struct PagedParams {
    PagedStream s[kMaxPagedStreams];
    int32_t num_streams;
    int32_t total_slabs;
    uint16_t *cache;
    int64_t c_sb, c_sh, c_sn;
    int64_t num_blocks;
    int32_t block_size;
    const int64_t *pos;
    const int64_t *slot;
    const int32_t *qsl;
    int32_t num_reqs;
    const int32_t *bt;
    int64_t bt_sr;
    int32_t max_blocks;
    int64_t T;
    int32_t tile_bt;           // tokens per tile: kPagedBT or kPagedBTSmall
    int32_t n_tiles;           // ceil(T / tile_bt)
    // Slot and position arithmetic in 32 bits: the host bounds every valid
    // slot (slot_lim = num_blocks * block_size) and every position with a
    // block-table entry (src_lim = max_blocks * block_size) below 2^31.
    FastDivU32 div_n;          // division by block_size
    int64_t slot_lim;
    int64_t src_lim;
    const int32_t *bt_rd;      // the block table, or query_start_loc when it is empty
};

// The paged step for any layout: strides and D offsets of any size, bases
// aligned to their element size, 64-bit slot arithmetic.  A tile is one
// token row of kGenTile channels of one stream; the streams' channel tiles
// are numbered consecutively (PagedStream::slab0 is a stream's first).
struct PagedGenParams {
    PagedStream s[kMaxPagedStreams];
    int32_t num_streams;
    int64_t cols;              // channel tiles of all streams
    uint16_t *cache;
    int64_t c_sb, c_sh, c_sn;
    int64_t num_blocks;
    int32_t block_size;
    const int64_t *pos;
    const int64_t *slot;
    const int32_t *qsl;
    int32_t num_reqs;
    const int32_t *bt;         // or null when no request has a table entry
    int64_t bt_sr;
    int32_t max_blocks;
    int64_t T;
    int64_t n_tiles;           // T * cols
};

// Launchers: each enqueues one kernel and returns hipGetLastError().
hipError_t launch_fwd_tokmajor(const FwdTokParams &p, int width, bool silu, hipStream_t s);
hipError_t launch_fwd_chanlast(const FwdClParams &p, int width, bool silu, hipStream_t s);
hipError_t launch_update(const UpdParams &p, int width, bool silu, hipStream_t s);
hipError_t launch_seq_metadata(const int32_t *qsl, int32_t num_reqs, int32_t num_actual,
                               int32_t num_padded, int32_t *seq_idx, int32_t *query_start,
                               hipStream_t s);
hipError_t launch_paged_fused(const PagedParams &p, int width, bool silu, bool residual,
                              hipStream_t s);
hipError_t launch_fwd_general(const FwdGenParams &p, int width, bool silu, hipStream_t s);
hipError_t launch_paged_general(const PagedGenParams &p, int width, bool silu, bool residual,
                                hipStream_t s);

// Tile geometry used by both the host (grid sizes) and the kernels.
constexpr int kWaveSize = 64;
constexpr int kVec = 8;                          // bf16 per 16-byte vector
constexpr int kSlab = kWaveSize * kVec;          // channels per wave (512)
constexpr int kTokWavesPerBlock = 1;
constexpr int kTokRounds = 4;                    // 64-chunk rounds per wave
constexpr int kClWavesPerBlock = 4;
constexpr int kCpl = 4;                          // channels per lane, channel-contiguous
constexpr int kClSlab = kWaveSize * kCpl;        // channels per wave there (256)
constexpr int kPagedWavesPerBlock = 4;
constexpr int kPagedBT = 16;                     // tokens per paged wave tile (the larger size)
constexpr int kPagedBTSmall = 8;                 // tile for steps of under one generation of waves
constexpr int64_t kPagedFillWaves = 256 * 32;    // waves that fill the chip once
constexpr int kPagedSlab = 256;                  // channels per paged wave (4 per lane)
// Buffer-descriptor offsets are 32-bit: rows, state lines and cache blocks
// reached through one descriptor must span less than this many bytes.
constexpr int64_t kMaxDescriptorSpan = int64_t(1) << 31;
constexpr int kQslLdsMax = 2048;                 // qsl entries staged in LDS
constexpr int kGenTile = 256;                    // lanes (one workgroup) per general-stride tile
constexpr int64_t kGenMaxBlocks = int64_t(1) << 20;  // general-stride grid cap (tile loop beyond)

}  // namespace sconv

// libsconv C ABI: host-side validation, layout dispatch and launch.
// Nothing here touches device memory or synchronises.  A successful call
// enqueues one kernel on the caller's stream: a vector kernel when the
// layout allows one, else the general-stride kernel (a token-contiguous
// forward of 2^32 elements or more enqueues one launch per channel group).
#include <stddef.h>
#include <initializer_list>
#include <stdint.h>

#include "sconv.h"
#include "sconv_params.h"

using namespace sconv;

namespace {

constexpr int kVersionMajor = 1;
constexpr int kMaxWidthHistory = SCONV_MAX_WIDTH - 1;
static_assert(kMaxPagedStreams == SCONV_MAX_PAGED_STREAMS, "stream table size");
constexpr int kVersionMinor = 4;

// Byte range [lo, hi) covered by a strided bf16 tensor; empty when a size is 0.
struct Span {
    uintptr_t lo = 0, hi = 0;
    bool empty() const { return hi <= lo; }
};

Span span_of(const void *p, std::initializer_list<int64_t> sizes,
             std::initializer_list<int64_t> strides, int64_t elem = 2) {
    Span s;
    if (!p) return s;
    int64_t last = 0;
    auto st = strides.begin();
    for (int64_t n : sizes) {
        if (n <= 0) return s;
        last += (n - 1) * *st++;
    }
    s.lo = reinterpret_cast<uintptr_t>(p);
    s.hi = s.lo + uintptr_t((last + 1) * elem);
    return s;
}

bool overlap(const Span &a, const Span &b) {
    return !a.empty() && !b.empty() && a.lo < b.hi && b.lo < a.hi;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// No two elements of a strided tensor share an address: taken in order of
// stride, every dimension of size > 1 steps past the whole span of the
// smaller ones.  Outputs and written caches must pass (their elements are
// written by different lanes); inputs may be any view, broadcasts included.
bool non_overlapping(std::initializer_list<int64_t> sizes, std::initializer_list<int64_t> strides) {
    int64_t n[4], st[4];
    int k = 0;
    auto sp = strides.begin();
    for (int64_t s : sizes) {
        const int64_t d = *sp++;
        if (s <= 1) continue;
        int i = k++;
        for (; i > 0 && st[i - 1] > d; --i) { n[i] = n[i - 1]; st[i] = st[i - 1]; }
        n[i] = s;
        st[i] = d;
    }
    int64_t span = 1;          // one past the largest offset of the dimensions so far
    for (int i = 0; i < k; ++i) {
        if (st[i] < span) return false;
        span += st[i] * (n[i] - 1);
    }
    return true;
}

int launch_status(hipError_t e) { return e == hipSuccess ? SCONV_OK : SCONV_ERR_LAUNCH; }

// Channel-contiguous storage: unit channel stride, 16-byte aligned rows.
bool chanlast_ok(int64_t sd, int64_t st, int64_t dim, int64_t T) {
    return sd == 1 && (T == 1 || (st >= dim && st % kVec == 0));
}
// Token-contiguous storage: a compact (dim, T) array.
bool tokmajor_ok(int64_t sd, int64_t st, int64_t dim, int64_t T) {
    return (st == 1 || T == 1) && (dim == 1 || sd == T);
}

// Tokens per channel-contiguous wave tile (measured on gfx950): a single
// sequence runs fastest with 8-token tiles at every length -- one batch of
// rows per wave, the most waves in flight, the halo rows re-read from L2.
// A batch of sequences pays a search of query_start_loc and a segment split
// per tile, so it takes the tile that leaves ~32 waves per CU, between 16
// and 128 tokens.
int32_t chanlast_tile(int64_t T, int32_t n_slabs, int32_t batch) {
    if (batch <= 1) return 8;
    const int64_t target_waves = 256 * 32;
    int64_t bt = (T * n_slabs + target_waves - 1) / target_waves;
    bt = (bt + 7) / 8 * 8;
    if (bt < 16) bt = 16;
    if (bt > 128) bt = 128;
    return int32_t(bt);
}

}  // namespace

extern "C" {

const char *sconv_status_string(int status) {
    switch (status) {
        case SCONV_OK: return "ok";
        case SCONV_ERR_NULL: return "required pointer is null";
        case SCONV_ERR_SHAPE: return "invalid or inconsistent size";
        case SCONV_ERR_STRIDE: return "unsupported stride / layout";
        case SCONV_ERR_WIDTH: return "width outside 2..5";
        case SCONV_ERR_ALIAS: return "output overlaps an input";
        case SCONV_ERR_ALIGN: return "pointer not aligned to its element size";
        case SCONV_ERR_ARG: return "invalid enumerated argument";
        case SCONV_ERR_LAUNCH: return "kernel launch failed";
        default: return "unknown status";
    }
}

int sconv_version(void) { return (kVersionMajor << 16) | kVersionMinor; }

int conv1d_fwd_varlen(const void *x, int64_t x_stride_dim, int64_t x_stride_tok,
                      const void *weight, int64_t w_stride_dim, const void *bias,
                      void *conv_states, int64_t cs_stride_line, int64_t cs_stride_dim,
                      int64_t cs_stride_tok, int64_t num_cache_lines,
                      const int32_t *cache_indices, const uint8_t *has_initial_state,
                      const int32_t *query_start_loc, int32_t batch, int64_t total_tokens,
                      int32_t dim, int32_t width, int32_t activation, int32_t pad_slot_id,
                      void *out, int64_t o_stride_dim, int64_t o_stride_tok,
                      hipStream_t stream) {
    if (width < SCONV_MIN_WIDTH || width > SCONV_MAX_WIDTH) return SCONV_ERR_WIDTH;
    if (activation != SCONV_ACT_NONE && activation != SCONV_ACT_SILU) return SCONV_ERR_ARG;
    if (batch < 0 || total_tokens < 0 || dim < 0 || num_cache_lines < 0) return SCONV_ERR_SHAPE;
    if (total_tokens > INT32_MAX) return SCONV_ERR_SHAPE;       // offsets are int32
    if (batch == 0 || total_tokens == 0 || dim == 0) return SCONV_OK;
    if (!x || !weight || !query_start_loc || !out) return SCONV_ERR_NULL;
    if (has_initial_state && !conv_states) return SCONV_ERR_NULL;
    if (x_stride_dim < 0 || x_stride_tok < 0 || o_stride_dim < 0 || o_stride_tok < 0 ||
        cs_stride_line < 0 || cs_stride_dim < 0 || cs_stride_tok < 0 || w_stride_dim < 0)
        return SCONV_ERR_STRIDE;
    if (conv_states) {
        if (num_cache_lines < 1) return SCONV_ERR_SHAPE;
        if (!cache_indices && num_cache_lines < batch) return SCONV_ERR_SHAPE;
    }
    if (!aligned(x, 2) || !aligned(out, 2) || !aligned(weight, 2) || !aligned(bias, 2) ||
        !aligned(conv_states, 2) || !aligned(cache_indices, 4) || !aligned(query_start_loc, 4))
        return SCONV_ERR_ALIGN;

    const int64_t T = total_tokens;
    // outputs and states are written element by element: no two may coincide
    if (!non_overlapping({dim, T}, {o_stride_dim, o_stride_tok})) return SCONV_ERR_STRIDE;
    if (conv_states && !non_overlapping({num_cache_lines, dim, width - 1},
                                        {cs_stride_line, cs_stride_dim, cs_stride_tok}))
        return SCONV_ERR_STRIDE;
    const Span sx = span_of(x, {dim, T}, {x_stride_dim, x_stride_tok});
    const Span so = span_of(out, {dim, T}, {o_stride_dim, o_stride_tok});
    const Span sw = span_of(weight, {dim, width}, {w_stride_dim, 1});
    const Span sbias = span_of(bias, {dim}, {1});
    const Span scs = span_of(conv_states, {num_cache_lines, dim, width - 1},
                             {cs_stride_line, cs_stride_dim, cs_stride_tok});
    if (overlap(so, sx) || overlap(so, scs) || overlap(so, sw) || overlap(so, sbias) ||
        overlap(scs, sx) || overlap(scs, sw) || overlap(scs, sbias))
        return SCONV_ERR_ALIAS;

    SeqBatch sb;
    sb.qsl = query_start_loc;
    sb.cache_idx = cache_indices;
    sb.has_init = has_initial_state;
    sb.cs = static_cast<uint16_t *>(conv_states);
    sb.cs_sl = cs_stride_line;
    sb.cs_sd = cs_stride_dim;
    sb.cs_st = cs_stride_tok;
    sb.num_lines = conv_states ? num_cache_lines : 0;
    sb.batch = batch;
    sb.pad_slot_id = pad_slot_id;
    sb.total_T = T;
    const bool silu = activation == SCONV_ACT_SILU;

    // The vector kernels read x and out in 16-byte pieces and whole weight
    // rows through buffer descriptors; every other layout takes the
    // general-stride kernel.
    const bool vec_ok = aligned(x, 16) && aligned(out, 16) && w_stride_dim >= width;
    // one descriptor spans a state line's channels
    const int64_t line_span =
        conv_states ? ((int64_t(dim) - 1) * cs_stride_dim + int64_t(width - 2) * cs_stride_tok + 1) * 2
                    : 0;

    // A single token is both layouts at once; the per-row kernel of the
    // token-contiguous path (one lane per channel) serves it with the
    // shortest chain of reads.
    const bool one_token_rows = T == 1 && batch <= 1 && tokmajor_ok(x_stride_dim, x_stride_tok, dim, T) &&
                                tokmajor_ok(o_stride_dim, o_stride_tok, dim, T);
    if (vec_ok && !one_token_rows && chanlast_ok(x_stride_dim, x_stride_tok, dim, T) &&
        chanlast_ok(o_stride_dim, o_stride_tok, dim, T)) {
        FwdClParams p;
        p.x = static_cast<const uint16_t *>(x);
        p.out = static_cast<uint16_t *>(out);
        p.x_st = T == 1 ? 0 : x_stride_tok;
        p.o_st = T == 1 ? 0 : o_stride_tok;
        p.w = static_cast<const uint16_t *>(weight);
        p.w_sd = w_stride_dim;
        p.bias = static_cast<const uint16_t *>(bias);
        p.sb = sb;
        p.dim = dim;
        p.n_slabs = (dim + kClSlab - 1) / kClSlab;
        p.div_slabs = FastDivU32::make(uint32_t(p.n_slabs));
        p.bt = chanlast_tile(T, p.n_slabs, batch);
        // one descriptor spans a tile's rows (plus the spilled head) and one
        // state line
        const int64_t row_span = int64_t(p.bt + 2 * kMaxWidthHistory) *
                                     (x_stride_tok > o_stride_tok ? x_stride_tok : o_stride_tok) * 2 +
                                 int64_t(dim) * 2;
        p.n_tiles = int32_t((T + p.bt - 1) / p.bt);
        if (row_span < kMaxDescriptorSpan && line_span < kMaxDescriptorSpan &&
            uint64_t(p.n_tiles) * uint64_t(p.n_slabs) < (uint64_t(1) << 31))
            return launch_status(launch_fwd_chanlast(p, width, silu, stream));
    } else if (vec_ok && line_span < kMaxDescriptorSpan &&
               tokmajor_ok(x_stride_dim, x_stride_tok, dim, T) &&
               tokmajor_ok(o_stride_dim, o_stride_tok, dim, T)) {
        // The token-contiguous kernels index a (dim, T) array with 32-bit
        // element offsets.  Channels are independent, so a larger array is
        // run as consecutive channel groups of fewer than 2^32 elements,
        // each a compact (group, T) array of its own (one launch per group;
        // groups start on 16-byte boundaries).
        int64_t group = dim;
        if (uint64_t(dim) * uint64_t(T) >= (uint64_t(1) << 32)) {
            group = int64_t((uint64_t(1) << 32) - 1) / T;
            if (T % kVec) group -= group % kVec;
        }
        if (group > 0) {
            for (int64_t c0 = 0; c0 < dim; c0 += group) {
                const int64_t g = dim - c0 < group ? dim - c0 : group;
                const uint64_t n = uint64_t(g) * uint64_t(T);
                FwdTokParams p;
                p.x = static_cast<const uint16_t *>(x) + c0 * T;
                p.out = static_cast<uint16_t *>(out) + c0 * T;
                p.w = static_cast<const uint16_t *>(weight) + c0 * w_stride_dim;
                p.w_sd = w_stride_dim;
                p.bias = bias ? static_cast<const uint16_t *>(bias) + c0 : nullptr;
                p.sb = sb;
                if (conv_states) p.sb.cs = sb.cs + c0 * cs_stride_dim;
                p.T = uint32_t(T);
                p.divT = FastDivU32::make(uint32_t(T));
                p.n_elems = uint32_t(n);
                p.n_chunks = uint32_t((n + kVec - 1) / kVec);
                p.dim = int32_t(g);
                p.bias_rd = p.bias ? p.bias : p.w;
                p.bias_mask = p.bias ? 0xffffu : 0u;
                p.ci_rd = sb.cache_idx ? sb.cache_idx : sb.qsl;
                p.hi_rd = sb.has_init ? sb.has_init : reinterpret_cast<const uint8_t *>(sb.qsl);
                const int rc = launch_status(launch_fwd_tokmajor(p, width, silu, stream));
                if (rc != SCONV_OK) return rc;
            }
            return SCONV_OK;
        }
    }

    FwdGenParams g;
    g.x = static_cast<const uint16_t *>(x);
    g.out = static_cast<uint16_t *>(out);
    g.x_sd = x_stride_dim;
    g.x_st = x_stride_tok;
    g.o_sd = o_stride_dim;
    g.o_st = o_stride_tok;
    g.w = static_cast<const uint16_t *>(weight);
    g.w_sd = w_stride_dim;
    g.bias = static_cast<const uint16_t *>(bias);
    g.sb = sb;
    g.dim = dim;
    g.T = T;
    // lanes along the axis of x with the smaller stride
    g.lanes_on_tokens = dim == 1 || (T > 1 && x_stride_tok < x_stride_dim);
    const int64_t lane_axis = g.lanes_on_tokens ? T : dim;
    g.tiles_per_line = (lane_axis + kGenTile - 1) / kGenTile;
    g.n_tiles = (g.lanes_on_tokens ? int64_t(dim) : T) * g.tiles_per_line;
    return launch_status(launch_fwd_general(g, width, silu, stream));
}

int conv1d_update(const void *x, int64_t x_stride_seq, int64_t x_stride_dim,
                  int64_t x_stride_tok, const void *weight, int64_t w_stride_dim,
                  const void *bias, void *conv_state, int64_t cs_stride_line,
                  int64_t cs_stride_dim, int64_t cs_stride_tok, int64_t num_cache_lines,
                  int32_t state_len, const int32_t *cache_indices,
                  const int32_t *cache_seqlens, const int32_t *num_accepted_tokens,
                  void *intermediate, int64_t it_stride_seq, int64_t it_stride_step,
                  int64_t it_stride_dim, int64_t it_stride_win,
                  const int32_t *output_state_indices, int64_t osi_stride_seq,
                  int64_t osi_stride_step, int32_t batch, int32_t dim, int32_t seqlen,
                  int32_t width, int32_t activation, int32_t pad_slot_id, void *out,
                  int64_t o_stride_seq, int64_t o_stride_dim, int64_t o_stride_tok,
                  hipStream_t stream) {
    if (width < SCONV_MIN_WIDTH || width > SCONV_MAX_WIDTH) return SCONV_ERR_WIDTH;
    if (activation != SCONV_ACT_NONE && activation != SCONV_ACT_SILU) return SCONV_ERR_ARG;
    const bool saved = intermediate || output_state_indices;
    if (cache_seqlens && (num_accepted_tokens || saved)) return SCONV_ERR_ARG;
    if (batch < 0 || dim < 0 || seqlen < 0 || num_cache_lines < 0) return SCONV_ERR_SHAPE;
    if (state_len < width - 1) return SCONV_ERR_SHAPE;
    if (num_accepted_tokens && !saved && int64_t(state_len) < int64_t(width) - 2 + seqlen)
        return SCONV_ERR_SHAPE;
    if (batch == 0 || dim == 0 || seqlen == 0) return SCONV_OK;
    if (!x || !weight || !conv_state || !out) return SCONV_ERR_NULL;
    if (x_stride_seq < 0 || x_stride_dim < 0 || x_stride_tok < 0 || o_stride_seq < 0 ||
        o_stride_dim < 0 || o_stride_tok < 0 || cs_stride_line < 0 || cs_stride_dim < 0 ||
        cs_stride_tok < 0 || it_stride_seq < 0 || it_stride_step < 0 || it_stride_dim < 0 ||
        it_stride_win < 0 || osi_stride_seq < 0 || osi_stride_step < 0 || w_stride_dim < 0)
        return SCONV_ERR_STRIDE;
    // outputs, states and saved windows are written element by element
    if (!non_overlapping({batch, dim, seqlen}, {o_stride_seq, o_stride_dim, o_stride_tok}) ||
        !non_overlapping({num_cache_lines, dim, state_len},
                         {cs_stride_line, cs_stride_dim, cs_stride_tok}) ||
        (intermediate && !non_overlapping({batch, seqlen, dim, width - 1},
                                          {it_stride_seq, it_stride_step, it_stride_dim,
                                           it_stride_win})))
        return SCONV_ERR_STRIDE;
    if (num_cache_lines < 1 || (!cache_indices && num_cache_lines < batch)) return SCONV_ERR_SHAPE;
    if (!aligned(x, 2) || !aligned(out, 2) || !aligned(weight, 2) || !aligned(bias, 2) ||
        !aligned(conv_state, 2) || !aligned(intermediate, 2) || !aligned(cache_indices, 4) ||
        !aligned(cache_seqlens, 4) || !aligned(num_accepted_tokens, 4) ||
        !aligned(output_state_indices, 4))
        return SCONV_ERR_ALIGN;
    const uint64_t cblocks = (uint64_t(dim) + 255) / 256;
    if (cblocks * uint64_t(batch) >= (uint64_t(1) << 31)) return SCONV_ERR_SHAPE;

    const Span sx = span_of(x, {batch, dim, seqlen}, {x_stride_seq, x_stride_dim, x_stride_tok});
    const Span so = span_of(out, {batch, dim, seqlen}, {o_stride_seq, o_stride_dim, o_stride_tok});
    const Span scs = span_of(conv_state, {num_cache_lines, dim, state_len},
                             {cs_stride_line, cs_stride_dim, cs_stride_tok});
    const Span sw = span_of(weight, {dim, width}, {w_stride_dim, 1});
    const Span sbias = span_of(bias, {dim}, {1});
    const Span sit = span_of(intermediate, {batch, seqlen, dim, width - 1},
                             {it_stride_seq, it_stride_step, it_stride_dim, it_stride_win});
    const bool in_place = out == x && o_stride_seq == x_stride_seq &&
                          o_stride_dim == x_stride_dim && o_stride_tok == x_stride_tok;
    if ((!in_place && overlap(so, sx)) || overlap(so, scs) || overlap(so, sw) ||
        overlap(so, sbias) || overlap(scs, sx) || overlap(scs, sw) || overlap(scs, sbias) ||
        overlap(sit, sx) || overlap(sit, so) || overlap(sit, scs) || overlap(sit, sw) ||
        overlap(sit, sbias))
        return SCONV_ERR_ALIAS;

    UpdParams p;
    p.x = static_cast<const uint16_t *>(x);
    p.x_sb = x_stride_seq;
    p.x_sd = x_stride_dim;
    p.x_st = x_stride_tok;
    p.out = static_cast<uint16_t *>(out);
    p.o_sb = o_stride_seq;
    p.o_sd = o_stride_dim;
    p.o_st = o_stride_tok;
    p.w = static_cast<const uint16_t *>(weight);
    p.w_sd = w_stride_dim;
    p.bias = static_cast<const uint16_t *>(bias);
    p.cs = static_cast<uint16_t *>(conv_state);
    p.cs_sl = cs_stride_line;
    p.cs_sd = cs_stride_dim;
    p.cs_st = cs_stride_tok;
    p.num_lines = num_cache_lines;
    p.cache_idx = cache_indices;
    p.ring_seen = cache_seqlens;
    p.num_acc = num_accepted_tokens;
    p.inter = static_cast<uint16_t *>(intermediate);
    p.i_sb = it_stride_seq;
    p.i_st = it_stride_step;
    p.i_sd = it_stride_dim;
    p.i_sk = it_stride_win;
    p.out_idx = output_state_indices;
    p.oi_sb = osi_stride_seq;
    p.oi_st = osi_stride_step;
    p.state_len = state_len;
    p.batch = batch;
    p.dim = dim;
    p.seqlen = seqlen;
    p.pad_slot_id = pad_slot_id;
    return launch_status(launch_update(p, width, activation == SCONV_ACT_SILU, stream));
}

int conv1d_update_decode(const void *x, int64_t x_stride_seq, int64_t x_stride_dim,
                         int64_t x_stride_tok, const void *weight, int64_t w_stride_dim,
                         const void *bias, void *conv_state, int64_t cs_stride_line,
                         int64_t cs_stride_dim, int64_t cs_stride_tok, int64_t num_cache_lines,
                         const int32_t *cache_indices, int32_t batch, int32_t dim, int32_t seqlen,
                         int32_t width, int32_t activation, int32_t pad_slot_id, void *out,
                         int64_t o_stride_seq, int64_t o_stride_dim, int64_t o_stride_tok,
                         hipStream_t stream) {
    if (width < SCONV_MIN_WIDTH || width > SCONV_MAX_WIDTH) return SCONV_ERR_WIDTH;
    return conv1d_update(x, x_stride_seq, x_stride_dim, x_stride_tok, weight, w_stride_dim, bias,
                         conv_state, cs_stride_line, cs_stride_dim, cs_stride_tok,
                         num_cache_lines, width - 1, cache_indices, nullptr, nullptr, nullptr,
                         0, 0, 0, 0, nullptr, 0, 0, batch, dim, seqlen, width, activation,
                         pad_slot_id, out, o_stride_seq, o_stride_dim, o_stride_tok, stream);
}

int sconv_seq_metadata(const int32_t *query_start_loc, int32_t num_reqs,
                       int64_t num_actual_tokens, int64_t num_padded_tokens,
                       int32_t *seq_idx_out, int64_t seq_idx_capacity,
                       int32_t *query_start_out, int64_t query_start_capacity,
                       hipStream_t stream) {
    if (num_padded_tokens < 0) num_padded_tokens = num_actual_tokens;
    if (num_actual_tokens < 0 || num_reqs < 0) return SCONV_ERR_SHAPE;
    if (num_padded_tokens < num_actual_tokens) return SCONV_ERR_SHAPE;
    if (num_padded_tokens > seq_idx_capacity || num_padded_tokens > query_start_capacity)
        return SCONV_ERR_SHAPE;
    if (num_padded_tokens > INT32_MAX) return SCONV_ERR_SHAPE;
    if (num_actual_tokens > 0 && num_reqs < 1) return SCONV_ERR_SHAPE;
    if (num_padded_tokens == 0) return SCONV_OK;
    if (!seq_idx_out || !query_start_out || (num_actual_tokens > 0 && !query_start_loc))
        return SCONV_ERR_NULL;
    if (!aligned(query_start_loc, 4) || !aligned(seq_idx_out, 4) || !aligned(query_start_out, 4))
        return SCONV_ERR_ALIGN;
    const Span si = span_of(seq_idx_out, {num_padded_tokens}, {1}, 4);
    const Span sq = span_of(query_start_out, {num_padded_tokens}, {1}, 4);
    const Span sl = span_of(num_actual_tokens > 0 ? query_start_loc : nullptr,
                            {int64_t(num_reqs) + 1}, {1}, 4);
    if (overlap(si, sq) || overlap(si, sl) || overlap(sq, sl)) return SCONV_ERR_ALIAS;
    return launch_status(launch_seq_metadata(query_start_loc, num_reqs,
                                             int32_t(num_actual_tokens),
                                             int32_t(num_padded_tokens), seq_idx_out,
                                             query_start_out, stream));
}

int sconv_paged_fused_multi(int32_t num_streams, const void *const *x,
                            const int64_t *x_stride_tok, const void *const *weight,
                            const int64_t *w_stride_dim, const void *const *bias,
                            const int32_t *off_s, const int32_t *ws, void *const *out,
                            const int64_t *o_stride_tok, void *cache, int64_t c_stride_blk,
                            int64_t c_stride_head, int64_t c_stride_slot, int64_t num_blocks,
                            int32_t num_heads, int32_t block_size, int32_t head_dim,
                            const int64_t *positions, const int64_t *slot_mapping,
                            const int32_t *query_start_loc, int32_t num_reqs,
                            const int32_t *block_table, int64_t bt_stride_req,
                            int32_t max_blocks, int64_t num_tokens, int32_t width,
                            int32_t activation, int32_t use_residual, hipStream_t stream) {
    if (width < SCONV_MIN_WIDTH || width > SCONV_MAX_WIDTH) return SCONV_ERR_WIDTH;
    if (activation != SCONV_ACT_NONE && activation != SCONV_ACT_SILU) return SCONV_ERR_ARG;
    if (use_residual != 0 && use_residual != 1) return SCONV_ERR_ARG;
    if (num_streams < 1 || num_streams > SCONV_MAX_PAGED_STREAMS) return SCONV_ERR_SHAPE;
    if (!x || !x_stride_tok || !weight || !w_stride_dim || !off_s || !ws || !out ||
        !o_stride_tok)
        return SCONV_ERR_NULL;
    if (num_tokens < 0 || num_reqs < 0 || max_blocks < 0 || num_blocks < 0) return SCONV_ERR_SHAPE;
    if (num_heads < 1 || block_size < 1 || head_dim < 1) return SCONV_ERR_SHAPE;
    for (int i = 0; i < num_streams; ++i)
        if (ws[i] < 1 || off_s[i] < 0 || int64_t(off_s[i]) + ws[i] > head_dim)
            return SCONV_ERR_SHAPE;
    // every stream writes its own D sub-range of the inserted slots
    for (int i = 0; i < num_streams; ++i)
        for (int j = i + 1; j < num_streams; ++j)
            if (off_s[i] < off_s[j] + ws[j] && off_s[j] < off_s[i] + ws[i]) return SCONV_ERR_ALIAS;
    if (num_tokens == 0) return SCONV_OK;
    if (num_tokens > INT32_MAX) return SCONV_ERR_SHAPE;
    if (!cache || !positions || !slot_mapping || !query_start_loc ||
        (num_reqs > 0 && max_blocks > 0 && !block_table))
        return SCONV_ERR_NULL;
    if (bt_stride_req < 0 || c_stride_blk < 0 || c_stride_head < 0 || c_stride_slot < 0)
        return SCONV_ERR_STRIDE;
    if (!aligned(cache, 2) || !aligned(positions, 8) || !aligned(slot_mapping, 8) ||
        !aligned(query_start_loc, 4) || !aligned(block_table, 4))
        return SCONV_ERR_ALIGN;
    // inserts write cache elements: no two slots / heads may share one
    if (!non_overlapping({num_blocks, num_heads, block_size, head_dim},
                         {c_stride_blk, c_stride_head, c_stride_slot, 1}))
        return SCONV_ERR_STRIDE;
    const Span sc = span_of(cache, {num_blocks, num_heads, block_size, head_dim},
                            {c_stride_blk, c_stride_head, c_stride_slot, 1});

    // The vector kernel moves 4 channels of one head per lane in 8-byte
    // pieces through buffer descriptors, with 32-bit slot arithmetic; other
    // layouts take the general-stride kernel.
    bool vec_ok = aligned(cache, 16) && c_stride_blk % kVec == 0 && c_stride_head % kVec == 0 &&
                  c_stride_slot % kVec == 0 && c_stride_blk * 2 < kMaxDescriptorSpan &&
                  num_blocks * int64_t(block_size) < (int64_t(1) << 31) &&
                  int64_t(max_blocks) * block_size < (int64_t(1) << 31);

    PagedParams p;
    Span sx[kMaxPagedStreams], so[kMaxPagedStreams], sw[kMaxPagedStreams], sb[kMaxPagedStreams];
    int64_t total_slabs = 0, total_cols = 0;
    for (int i = 0; i < num_streams; ++i) {
        const void *bi = bias ? bias[i] : nullptr;
        if (!x[i] || !weight[i] || !out[i]) return SCONV_ERR_NULL;
        const int64_t C = int64_t(num_heads) * ws[i];
        if (C > INT32_MAX) return SCONV_ERR_SHAPE;
        if (x_stride_tok[i] < 0 || o_stride_tok[i] < 0 || w_stride_dim[i] < 0)
            return SCONV_ERR_STRIDE;
        // rows of out are written element by element: they may not overlap
        if (!non_overlapping({num_tokens, C}, {o_stride_tok[i], 1})) return SCONV_ERR_STRIDE;
        if (!aligned(x[i], 2) || !aligned(out[i], 2) || !aligned(weight[i], 2) || !aligned(bi, 2))
            return SCONV_ERR_ALIGN;
        // one descriptor spans a tile's rows of x (with the width-1 before it) or of out
        const int64_t row_span = int64_t(kPagedBT + SCONV_MAX_WIDTH) *
                                     (x_stride_tok[i] > o_stride_tok[i] ? x_stride_tok[i]
                                                                        : o_stride_tok[i]) * 2 +
                                 C * 2;
        vec_ok = vec_ok && ws[i] % kVec == 0 && off_s[i] % kVec == 0 &&
                 x_stride_tok[i] % kVec == 0 && o_stride_tok[i] % kVec == 0 &&
                 x_stride_tok[i] >= C && aligned(x[i], 16) && aligned(out[i], 16) &&
                 row_span < kMaxDescriptorSpan;
        sx[i] = span_of(x[i], {num_tokens, C}, {x_stride_tok[i], 1});
        so[i] = span_of(out[i], {num_tokens, C}, {o_stride_tok[i], 1});
        sw[i] = span_of(weight[i], {C, width}, {w_stride_dim[i], 1});
        sb[i] = span_of(bi, {C}, {1});
        PagedStream &st = p.s[i];
        st.x = static_cast<const uint16_t *>(x[i]);
        st.out = static_cast<uint16_t *>(out[i]);
        st.w = static_cast<const uint16_t *>(weight[i]);
        st.bias = static_cast<const uint16_t *>(bi);
        st.x_st = x_stride_tok[i];
        st.o_st = o_stride_tok[i];
        st.w_sd = w_stride_dim[i];
        st.off_s = off_s[i];
        st.ws = ws[i];
        st.C = int32_t(C);
        st.slab0 = int32_t(total_slabs);
        total_slabs += (C + kPagedSlab - 1) / kPagedSlab;
        total_cols += (C + kGenTile - 1) / kGenTile;
    }
    for (int i = num_streams; i < kMaxPagedStreams; ++i) p.s[i] = p.s[0];
    // outputs overlap nothing; the cache overlaps no input
    for (int i = 0; i < num_streams; ++i) {
        if (overlap(so[i], sc) || overlap(sc, sx[i]) || overlap(sc, sw[i]) || overlap(sc, sb[i]))
            return SCONV_ERR_ALIAS;
        for (int j = 0; j < num_streams; ++j)
            if (overlap(so[i], sx[j]) || overlap(so[i], sw[j]) || overlap(so[i], sb[j]) ||
                (j != i && overlap(so[i], so[j])))
                return SCONV_ERR_ALIAS;
    }
    const bool silu = activation == SCONV_ACT_SILU;

    if (vec_ok) {
        p.num_streams = num_streams;
        p.cache = static_cast<uint16_t *>(cache);
        p.c_sb = c_stride_blk;
        p.c_sh = c_stride_head;
        p.c_sn = c_stride_slot;
        p.num_blocks = num_blocks;
        p.block_size = block_size;
        p.pos = positions;
        p.slot = slot_mapping;
        p.qsl = query_start_loc;
        p.num_reqs = num_reqs;
        p.bt = block_table;
        p.bt_sr = bt_stride_req;
        p.max_blocks = block_table ? max_blocks : 0;
        p.div_n = FastDivU32::make(uint32_t(block_size));
        p.slot_lim = num_blocks * int64_t(block_size);
        p.src_lim = int64_t(p.max_blocks) * block_size;
        p.bt_rd = (block_table && num_reqs > 0 && max_blocks > 0) ? block_table : query_start_loc;
        p.T = num_tokens;
        // A step that would not fill the chip once with 16-token tiles takes
        // 8-token tiles: twice the waves, each with half the chain of round trips.
        const int64_t tiles16 = (num_tokens + kPagedBT - 1) / kPagedBT;
        p.tile_bt = tiles16 * total_slabs < kPagedFillWaves ? kPagedBTSmall : kPagedBT;
        p.n_tiles = int32_t((num_tokens + p.tile_bt - 1) / p.tile_bt);
        p.total_slabs = int32_t(total_slabs);
        if (uint64_t(p.n_tiles) * uint64_t(total_slabs) < (uint64_t(1) << 31))
            return launch_status(launch_paged_fused(p, width, silu, use_residual != 0, stream));
    }

    PagedGenParams g;
    for (int i = 0; i < kMaxPagedStreams; ++i) g.s[i] = p.s[i];
    int64_t col0 = 0;
    for (int i = 0; i < num_streams; ++i) {
        g.s[i].slab0 = int32_t(col0);
        col0 += (int64_t(g.s[i].C) + kGenTile - 1) / kGenTile;
    }
    for (int i = num_streams; i < kMaxPagedStreams; ++i) g.s[i] = g.s[0];
    g.num_streams = num_streams;
    g.cols = total_cols;
    g.cache = static_cast<uint16_t *>(cache);
    g.c_sb = c_stride_blk;
    g.c_sh = c_stride_head;
    g.c_sn = c_stride_slot;
    g.num_blocks = num_blocks;
    g.block_size = block_size;
    g.pos = positions;
    g.slot = slot_mapping;
    g.qsl = query_start_loc;
    g.num_reqs = num_reqs;
    g.bt = block_table;
    g.bt_sr = bt_stride_req;
    g.max_blocks = block_table ? max_blocks : 0;
    g.T = num_tokens;
    g.n_tiles = num_tokens * total_cols;
    return launch_status(launch_paged_general(g, width, silu, use_residual != 0, stream));
}

int sconv_paged_fused(const void *x, int64_t x_stride_tok, const void *weight,
                      int64_t w_stride_dim, const void *bias, void *cache, int64_t c_stride_blk,
                      int64_t c_stride_head, int64_t c_stride_slot, int64_t num_blocks,
                      int32_t num_heads, int32_t block_size, int32_t head_dim, int32_t off_s,
                      int32_t ws, const int64_t *positions, const int64_t *slot_mapping,
                      const int32_t *query_start_loc, int32_t num_reqs,
                      const int32_t *block_table, int64_t bt_stride_req, int32_t max_blocks,
                      int64_t num_tokens, int32_t width, int32_t activation,
                      int32_t use_residual, void *out, int64_t o_stride_tok,
                      hipStream_t stream) {
    if (num_tokens > 0 && (!x || !weight || !out)) return SCONV_ERR_NULL;
    return sconv_paged_fused_multi(1, &x, &x_stride_tok, &weight, &w_stride_dim, &bias, &off_s,
                                   &ws, &out, &o_stride_tok, cache, c_stride_blk, c_stride_head,
                                   c_stride_slot, num_blocks, num_heads, block_size, head_dim,
                                   positions, slot_mapping, query_start_loc, num_reqs,
                                   block_table, bt_stride_req, max_blocks, num_tokens, width,
                                   activation, use_residual, stream);
}

}  // extern "C"

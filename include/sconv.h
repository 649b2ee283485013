/*
 * sconv.h -- C ABI of libsconv, a gfx950 (MI355X) library for the causal
 * depthwise short convolution (width 2..5) used by hybrid / linear-attention
 * language models.
 *
 * The operation, in the notation of the pages it comes from:
 *
 *   For a sequence s with inputs x[c][t], t < L, a per-channel history
 *   h[c][k], k < W-1 (the cached last W-1 inputs, oldest first), weights
 *   w[c][j], j < W, and bias b[c]:
 *     u[c] = h[c] ++ x[c]
 *     y[c][t] = b[c] + sum_j w[c][j] * u[c][t+j]       (fp32 accumulation)
 *     out[c][t] = bf16(silu(y))  or  bf16(y)            (one rounding, RNE)
 *     new h[c][k] = u[c][L+k]                           (last W-1 of u)
 *
 *   -- atrex-bench operator #003 "causal_conv1d", section "Reference
 *      Implementation" (prefix by state, depthwise conv1d, last T outputs,
 *      SiLU); tokenspeed causal_conv1d.py, causal_conv1d_fn and
 *      causal_conv1d_update (varlen batches, cache lines, pads, state
 *      update); Inkling sconv.py, fused_sconv (paged sliding-window cache).
 *
 * Conventions shared by every entry point:
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library keeps no pointer after it returns, but the work it enqueues
 *     reads and writes them asynchronously: they must stay valid until the
 *     stream reaches that work.
 *   - bf16 tensors are passed as void* (IEEE bfloat16 bit patterns).  Index
 *     arrays are int32 (query_start_loc, cache_indices, block_table), int64
 *     (positions, slot_mapping) or bytes (has_initial_state, 0 = false).
 *   - Strides are in ELEMENTS and must be non-negative; any such view is
 *     accepted (sliced, pitched, offset, transposed, broadcast inputs).  A
 *     tensor the call WRITES (outputs, states, caches, saved windows) must
 *     not have two elements at one address (else SCONV_ERR_STRIDE).  Pointers
 *     need only their element's alignment: 2 bytes for bf16, 4 for int32,
 *     8 for int64.  Layouts decide only the speed: each call documents the
 *     ones its vector kernels take; every other layout runs a general-stride
 *     kernel (one lane per element, 64-bit offsets) with the same results.
 *   - The library allocates nothing, never reads device memory on the host
 *     and never synchronises: each call validates its host arguments, then
 *     enqueues one kernel on `stream` (NULL = the default stream) and
 *     returns.  Two forms enqueue more, all on `stream`: a token-contiguous
 *     forward of 2^32 or more elements (one kernel per channel group), and a
 *     token-contiguous batch of several sequences with rows of at least 2048
 *     tokens (a streaming kernel, then one that rewrites each sequence's
 *     first width-1 outputs and writes its state).  Calls are therefore safe
 *     to capture in a HIP graph.
 *   - Return value: SCONV_OK, or a negative sconv_status.  On any error
 *     other than SCONV_ERR_LAUNCH nothing is enqueued.  An empty problem
 *     (zero tokens, zero sequences) returns SCONV_OK without enqueueing
 *     anything.
 *   - Device data is not validated on the host (it is never read there).
 *     Kernels guard every data-dependent index: a cache line outside
 *     [0, num_cache_lines) skips its sequence, a block id outside
 *     [0, num_blocks) reads as zero / drops the insert, and token offsets
 *     are clamped into the tensor.  Results for such inputs are defined by
 *     these rules only; the memory accessed always stays inside the tensors.
 *   - Calls that write the same cache lines / blocks must be ordered by the
 *     caller (same stream, or events); concurrent writers race.
 */
#ifndef SCONV_H
#define SCONV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sconv_status {
    SCONV_OK = 0,
    SCONV_ERR_NULL = -1,    /* a required pointer is NULL                       */
    SCONV_ERR_SHAPE = -2,   /* a size is negative, inconsistent or too large    */
    SCONV_ERR_STRIDE = -3,  /* a negative stride, or written elements overlap   */
    SCONV_ERR_WIDTH = -4,   /* width outside [SCONV_MIN_WIDTH, SCONV_MAX_WIDTH] */
    SCONV_ERR_ALIAS = -5,   /* an output overlaps an input it must not overlap  */
    SCONV_ERR_ALIGN = -6,   /* a pointer not aligned to its element size        */
    SCONV_ERR_ARG = -7,     /* an enumerated argument (activation, ...) is bad  */
    SCONV_ERR_LAUNCH = -8   /* the HIP runtime refused the launch               */
} sconv_status;

#define SCONV_MIN_WIDTH 2
#define SCONV_MAX_WIDTH 5
#define SCONV_MAX_PAGED_STREAMS 8   /* conv streams of one sconv_paged_fused_multi call */
#define SCONV_ACT_NONE 0
#define SCONV_ACT_SILU 1

/* Human-readable name of a status code (static storage, never NULL). */
const char *sconv_status_string(int status);

/* Library ABI version: (major << 16) | minor. */
int sconv_version(void);

/*
 * conv1d_fwd_varlen -- prefill over a packed batch of variable-length
 * sequences, each continued from (and writing back) its conv state.
 * Follows tokenspeed causal_conv1d.py, causal_conv1d_fn /
 * _causal_conv1d_fwd_kernel, with the arithmetic of the atrex-bench #003
 * reference forward.
 *
 * x            logical [dim][total_tokens] bf16; element (c, t) at
 *              x[c*x_stride_dim + t*x_stride_tok], any strides.  The vector
 *              kernels take two storages, when x and out are both in one of
 *              them, 16-byte aligned, and w_stride_dim >= width:
 *                token-contiguous: x_stride_tok == 1 and
 *                  x_stride_dim == total_tokens (a compact (dim, T) array,
 *                  the benchmark page's layout);
 *                channel-contiguous: x_stride_dim == 1, x_stride_tok >= dim
 *                  and a multiple of 8 (the (T, dim) layout the tokenspeed
 *                  launcher requires).  With total_tokens == 1 the token
 *                  stride is ignored.
 *              Any other layout (a slice x[:, a:b], a (T, dim) batch of
 *              pitch dim with dim % 8 != 0, an offset view, out stored
 *              unlike x, ...) takes the general-stride kernel.
 * weight       logical [dim][width] bf16, element (c, j) at
 *              weight[c*w_stride_dim + j] (unit width stride, as the page
 *              asserts); w_stride_dim may be anything >= 0 (0 broadcasts one
 *              set of taps to every channel).
 * bias         [dim] bf16, or NULL for no bias.
 * conv_states  logical [num_cache_lines][dim][width-1] bf16, element
 *              (l, c, k) at conv_states[l*cs_stride_line + c*cs_stride_dim
 *              + k*cs_stride_tok]; column 0 is the oldest input.  Read as the
 *              history of sequences with has_initial_state set, and
 *              overwritten in place with the last width-1 inputs of every
 *              processed sequence of non-zero length.  NULL: zero history,
 *              no state written.
 * cache_indices  [batch] int32: the cache line of each sequence; an entry
 *              equal to pad_slot_id marks a padded sequence, which is skipped
 *              entirely (no output, no state).  NULL: sequence s uses line s.
 * has_initial_state  [batch] bytes, non-zero = continue from the cached
 *              state; NULL = all false.  Requires conv_states.
 * query_start_loc  [batch+1] int32 token offsets: 0, then the running sum of
 *              the lengths; the last entry must equal total_tokens.
 * activation   SCONV_ACT_NONE or SCONV_ACT_SILU ("silu" / "swish").
 * out          logical [dim][total_tokens] bf16 (strides o_stride_dim /
 *              o_stride_tok).  Its address range must not overlap those of
 *              x or conv_states.  Rows of skipped sequences are left
 *              untouched.
 * Errors: NULL x/weight/query_start_loc/out (when there is work), or
 *   has_initial_state without conv_states -> SCONV_ERR_NULL; bad sizes,
 *   conv_states narrower than the lines cache_indices may not check ->
 *   SCONV_ERR_SHAPE; a negative stride, or out / conv_states with two
 *   elements at one address -> SCONV_ERR_STRIDE; a bf16 pointer not 2-byte
 *   or an index array not 4-byte aligned -> SCONV_ERR_ALIGN; overlap ->
 *   SCONV_ERR_ALIAS.
 */
int conv1d_fwd_varlen(const void *x, int64_t x_stride_dim, int64_t x_stride_tok,
                      const void *weight, int64_t w_stride_dim,
                      const void *bias,
                      void *conv_states, int64_t cs_stride_line,
                      int64_t cs_stride_dim, int64_t cs_stride_tok,
                      int64_t num_cache_lines,
                      const int32_t *cache_indices,
                      const uint8_t *has_initial_state,
                      const int32_t *query_start_loc,
                      int32_t batch, int64_t total_tokens, int32_t dim,
                      int32_t width, int32_t activation, int32_t pad_slot_id,
                      void *out, int64_t o_stride_dim, int64_t o_stride_tok,
                      hipStream_t stream);

/*
 * conv1d_update_decode -- decode-time update: each of `batch` entries feeds
 * `seqlen` new tokens (seqlen == 1 for plain decode) continuing from its
 * cached state, which is then shifted to hold the last width-1 inputs.
 * Follows tokenspeed causal_conv1d.py, causal_conv1d_update /
 * _causal_conv1d_update_kernel (without speculative decoding; conv1d_update
 * below adds the page's options).
 *
 * x            logical [batch][dim][seqlen] bf16 at
 *              x[b*x_stride_seq + c*x_stride_dim + t*x_stride_tok].
 * weight, bias as for conv1d_fwd_varlen.
 * conv_state   logical [num_cache_lines][dim][width-1] bf16 (any strides),
 *              always read as the history and updated in place.
 * cache_indices  [batch] int32 or NULL (entry b uses line b, and then
 *              num_cache_lines must be >= batch); pad_slot_id skips an entry.
 * out          logical [batch][dim][seqlen] bf16.  It may be exactly x
 *              (same pointer and strides: the page computes in place);
 *              any other overlap with x, and any overlap with conv_state, is
 *              SCONV_ERR_ALIAS.
 */
int conv1d_update_decode(const void *x, int64_t x_stride_seq, int64_t x_stride_dim,
                         int64_t x_stride_tok,
                         const void *weight, int64_t w_stride_dim,
                         const void *bias,
                         void *conv_state, int64_t cs_stride_line,
                         int64_t cs_stride_dim, int64_t cs_stride_tok,
                         int64_t num_cache_lines,
                         const int32_t *cache_indices,
                         int32_t batch, int32_t dim, int32_t seqlen,
                         int32_t width, int32_t activation, int32_t pad_slot_id,
                         void *out, int64_t o_stride_seq, int64_t o_stride_dim,
                         int64_t o_stride_tok,
                         hipStream_t stream);

/*
 * conv1d_update -- the decode update with the options of the same page
 * (tokenspeed causal_conv1d.py, causal_conv1d_update /
 * _causal_conv1d_update_kernel and its docstring): speculative decoding
 * (num_accepted_tokens, intermediate windows, output_state_indices) and
 * ring-buffer states (cache_seqlens).  conv1d_update_decode is this call with
 * state_len = width-1 and every option NULL.
 *
 * x, weight, bias, out, cache_indices, pad_slot_id: as for
 *              conv1d_update_decode (out may be exactly x).
 * conv_state   logical [num_cache_lines][dim][state_len] bf16 (any strides),
 *              state_len >= width-1.  The page asks for a unit dim stride;
 *              any stride works here.
 * Per entry b, the history (the width-1 inputs before x[b][.][0]) is
 *   cache_seqlens given: columns (cache_seqlens[b] - (width-1) + k) mod
 *              state_len, k = 0..width-2 (input n of the stream lives at
 *              column n mod state_len, and cache_seqlens[b] inputs have been
 *              seen);
 *   num_accepted_tokens given: columns num_accepted_tokens[b] - 1 + k;
 *   otherwise: columns k.
 * Outputs are act(bias + sum_j w[j] u[t+j]) over u = history ++ x[b], as for
 * every other call.  The window after step t is u[t+1 .. t+width-1], the
 * width-1 inputs that end with x[b][.][t].
 * intermediate [batch][>= seqlen][dim][width-1] bf16 or NULL, element
 *              (b, t, c, k) at intermediate[b*it_stride_seq + t*it_stride_step
 *              + c*it_stride_dim + k*it_stride_win]: receives the window after
 *              every step t.  Indexed by batch position, not by cache line.
 * output_state_indices  [batch][seqlen] int32 or NULL, element (b, t) at
 *              [b*osi_stride_seq + t*osi_stride_step]: a line in
 *              [0, num_cache_lines) receives the window after step t in its
 *              columns 0..width-2; other values write nothing.  A destination
 *              line must not be one that another entry of the same call reads
 *              (the entry's own line is fine: an entry reads before it writes).
 * State update in place, only when neither intermediate nor
 *   output_state_indices is given:
 *   cache_seqlens: x[b][.][t] goes to column (cache_seqlens[b] + t) mod
 *              state_len (when seqlen > state_len only the last state_len
 *              inputs remain);
 *   num_accepted_tokens: columns 0 .. width-3+seqlen receive u[1 ..], the
 *              history minus its oldest input followed by all of x[b]; the
 *              next call's num_accepted_tokens = a then reads the window that
 *              ends with the a-th input of this call.  Needs state_len >=
 *              width-2+seqlen (else SCONV_ERR_SHAPE);
 *   otherwise: columns 0..width-2 receive the last width-1 inputs of u.
 * An entry is skipped entirely (no output, no state, no window) when its line
 * is pad_slot_id or outside [0, num_cache_lines), when num_accepted_tokens[b]
 * is below 1 or above state_len - width + 2, or when cache_seqlens[b] is
 * negative.
 * Layouts and speed (results do not depend on the layout): with dim % 4 ==
 *   0, x and out of unit dim stride and every base and stride keeping four
 *   channels 8-byte aligned, a lane handles four channels with 8-byte
 *   accesses when either (a) the call has no option and conv_state is
 *   [lines][dim][width-1] token-contiguous (the usual decode cache), or (b)
 *   conv_state (and intermediate, when given) has unit dim stride.  Other
 *   layouts take one lane per channel with 2-byte accesses, which bounds
 *   large batches by the address unit (about 1.5-2x slower there).
 * Errors: as for conv1d_update_decode; cache_seqlens together with any of
 *   the three speculative options -> SCONV_ERR_ARG; state_len < width-1 ->
 *   SCONV_ERR_SHAPE; intermediate overlapping x, out, conv_state, weight or
 *   bias -> SCONV_ERR_ALIAS; index arrays must be 4-byte aligned.
 */
int conv1d_update(const void *x, int64_t x_stride_seq, int64_t x_stride_dim,
                  int64_t x_stride_tok,
                  const void *weight, int64_t w_stride_dim,
                  const void *bias,
                  void *conv_state, int64_t cs_stride_line,
                  int64_t cs_stride_dim, int64_t cs_stride_tok,
                  int64_t num_cache_lines, int32_t state_len,
                  const int32_t *cache_indices,
                  const int32_t *cache_seqlens,
                  const int32_t *num_accepted_tokens,
                  void *intermediate, int64_t it_stride_seq, int64_t it_stride_step,
                  int64_t it_stride_dim, int64_t it_stride_win,
                  const int32_t *output_state_indices, int64_t osi_stride_seq,
                  int64_t osi_stride_step,
                  int32_t batch, int32_t dim, int32_t seqlen,
                  int32_t width, int32_t activation, int32_t pad_slot_id,
                  void *out, int64_t o_stride_seq, int64_t o_stride_dim,
                  int64_t o_stride_tok,
                  hipStream_t stream);

/*
 * sconv_seq_metadata -- per-token request metadata in one launch, for callers
 * that keep persistent seq_idx / query_start buffers (Inkling sconv.py,
 * sconv_seq_metadata / _seq_metadata_kernel).  sconv_paged_fused derives the
 * same values inside its own kernel and does not need them.
 *
 * query_start_loc  [num_reqs+1] int32, non-decreasing row offsets (device).
 *              Read only when num_actual_tokens > 0.
 * Rows t < num_actual_tokens get seq_idx_out[t] = the largest j < num_reqs
 * with query_start_loc[j] <= t (an empty request is passed over) and
 * query_start_out[t] = query_start_loc[seq_idx_out[t]].  Rows in
 * [num_actual_tokens, num_padded_tokens) get 0 / 0; such padded rows must
 * carry slot_mapping == -1 in the paged call.  num_padded_tokens < 0 means
 * num_actual_tokens.
 * seq_idx_out, query_start_out  int32 device arrays with room for
 *              seq_idx_capacity / query_start_capacity entries.
 * Errors: num_padded_tokens < num_actual_tokens, or above either capacity
 *   or INT32_MAX, or num_reqs < 1 with actual tokens -> SCONV_ERR_SHAPE (the
 *   page raises for the first three); NULL arrays -> SCONV_ERR_NULL;
 *   misaligned -> SCONV_ERR_ALIGN; overlapping arrays -> SCONV_ERR_ALIAS.
 */
int sconv_seq_metadata(const int32_t *query_start_loc, int32_t num_reqs,
                       int64_t num_actual_tokens, int64_t num_padded_tokens,
                       int32_t *seq_idx_out, int64_t seq_idx_capacity,
                       int32_t *query_start_out, int64_t query_start_capacity,
                       hipStream_t stream);

/*
 * sconv_paged_fused -- one launch that inserts every token's input into a
 * paged sliding-window cache and convolves the width taps ending at its
 * absolute position.  Follows Inkling sconv.py, fused_sconv /
 * _fused_sconv_kernel; the token -> request lookup of its
 * _seq_metadata_kernel is done inside the kernel from query_start_loc.
 *
 * x            [num_tokens][C] bf16, C = num_heads * ws, channel stride 1,
 *              row stride x_stride_tok (any); head-major channels: channel
 *              c is head c / ws, cache D-index off_s + c % ws.
 * weight       [C][width] bf16 (unit width stride, any row stride), bias
 *              [C] or NULL (the page has none).
 * cache        [num_blocks][num_heads][block_size][head_dim] bf16 with unit
 *              D stride (the page asserts it; there is no D stride
 *              argument); strides c_stride_blk / c_stride_head /
 *              c_stride_slot, no two elements at one address.  It holds the
 *              conv input of every absolute position: position p of request
 *              r lives in block block_table[r*bt_stride_req + p /
 *              block_size], slot p % block_size, D range [off_s, off_s + ws),
 *              off_s + ws <= head_dim (else SCONV_ERR_SHAPE).
 *              The vector kernel runs when ws, off_s, the row strides and
 *              the cache strides are multiples of 8, x, out and the cache
 *              are 16-byte aligned, and num_blocks * block_size and
 *              max_blocks * block_size are below 2^31 (32-bit slot
 *              arithmetic); other layouts take the general-stride kernel.
 * positions    [num_tokens] int64 absolute position of each row.
 * slot_mapping [num_tokens] int64 flat slot block*block_size + offset of
 *              each row; < 0 marks a pad row.
 * query_start_loc [num_reqs+1] int32 row offsets of the requests; rows at or
 *              past query_start_loc[num_reqs] are pad rows.
 * block_table  [num_reqs][>= max_blocks] int32.
 * For a non-pad row t of request r (first row qs) at position p, tap j
 * (0..width-1) covers position p-(width-1)+j: zero before position 0, the
 * input row t-(width-1)+j when that row is >= qs (inside this forward),
 * else the cached value.  y = bias + sum of taps; silu if asked; + x[t] if
 * use_residual; one bf16 rounding.  Pad rows are neither convolved nor
 * inserted: out = x (use_residual) or 0.  The cache is read as it was
 * before the call (rows inside the forward are never read back from it),
 * which requires the blocks written by one request not to be read as
 * pre-forward taps by another.
 * out          [num_tokens][C] bf16 with row stride o_stride_tok (rows may
 *              not overlap: o_stride_tok >= C when num_tokens > 1); its
 *              address range must not overlap x or the cache.
 */
int sconv_paged_fused(const void *x, int64_t x_stride_tok,
                      const void *weight, int64_t w_stride_dim,
                      const void *bias,
                      void *cache, int64_t c_stride_blk, int64_t c_stride_head,
                      int64_t c_stride_slot,
                      int64_t num_blocks, int32_t num_heads, int32_t block_size,
                      int32_t head_dim, int32_t off_s, int32_t ws,
                      const int64_t *positions, const int64_t *slot_mapping,
                      const int32_t *query_start_loc, int32_t num_reqs,
                      const int32_t *block_table, int64_t bt_stride_req,
                      int32_t max_blocks,
                      int64_t num_tokens, int32_t width, int32_t activation,
                      int32_t use_residual,
                      void *out, int64_t o_stride_tok,
                      hipStream_t stream);

/*
 * sconv_paged_fused_multi -- sconv_paged_fused for several conv streams that
 * share one paged cache, in one launch.  The paged page's module docstring
 * describes four such streams per layer (K, V, attention output, MLP output),
 * each occupying its own D sub-range [off_s, off_s + ws) of every head of the
 * same cache; every stream computes exactly what sconv_paged_fused computes
 * for it, with the shared positions, slot_mapping, query_start_loc and
 * block_table.  The streams share the per-token metadata work of the launch.
 *
 * num_streams  1..SCONV_MAX_PAGED_STREAMS.
 * x, x_stride_tok, weight, w_stride_dim, off_s, ws, out, o_stride_tok:
 *              HOST arrays of num_streams entries holding what
 *              sconv_paged_fused takes for one stream (device pointers and
 *              element strides; stream i has C_i = num_heads * ws[i]
 *              channels).
 * bias         NULL (no stream has a bias) or a HOST array of num_streams
 *              device pointers, each NULL or [C_i] bf16.
 * cache ... use_residual: as for sconv_paged_fused, shared by all streams.
 * The D sub-ranges must be pairwise disjoint (else SCONV_ERR_ALIAS: two
 * streams would insert into the same cache elements); no output may overlap
 * any input, another output or the cache.  Other errors as for
 * sconv_paged_fused; a NULL host array -> SCONV_ERR_NULL.
 */
int sconv_paged_fused_multi(int32_t num_streams,
                            const void *const *x, const int64_t *x_stride_tok,
                            const void *const *weight, const int64_t *w_stride_dim,
                            const void *const *bias,
                            const int32_t *off_s, const int32_t *ws,
                            void *const *out, const int64_t *o_stride_tok,
                            void *cache, int64_t c_stride_blk, int64_t c_stride_head,
                            int64_t c_stride_slot, int64_t num_blocks,
                            int32_t num_heads, int32_t block_size, int32_t head_dim,
                            const int64_t *positions, const int64_t *slot_mapping,
                            const int32_t *query_start_loc, int32_t num_reqs,
                            const int32_t *block_table, int64_t bt_stride_req,
                            int32_t max_blocks, int64_t num_tokens, int32_t width,
                            int32_t activation, int32_t use_residual,
                            hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SCONV_H */

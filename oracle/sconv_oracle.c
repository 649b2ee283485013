/*
 * sconv_oracle.c -- plain, slow CPU oracle for the causal depthwise short
 * convolution.  TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and
 * the benchmark's CPU-baseline leg call it; the library never does.  It shares
 * no code, header, table or helper with the HIP implementation.
 *
 * Arithmetic: every value is widened from bf16 to double, taps are summed in
 * double, SiLU is evaluated in double, and the result is rounded ONCE to bf16
 * (round to nearest, ties to even).  State / cache writes are bit copies.
 *
 * Sources (the three pages this library is built from):
 *  [P3] atrex-bench operator #003 "causal_conv1d", section "Reference
 *       Implementation": Model.forward prefixes the input with the last
 *       width-1 state columns, runs a depthwise (groups = dim) conv1d with
 *       bias, keeps the last T outputs and applies SiLU.
 *  [P1] tokenspeed causal_conv1d.py: _causal_conv1d_fwd_kernel /
 *       causal_conv1d_fn (varlen batch through query_start_loc, cache line
 *       selection through cache_indices with a pad id, has_initial_state,
 *       conv_state update with the last width-1 inputs) and
 *       _causal_conv1d_update_kernel / causal_conv1d_update (decode).
 *  [P2] Inkling sconv.py: _fused_sconv_kernel / fused_sconv (paged
 *       sliding-window cache insert + conv + SiLU + residual) and
 *       _seq_metadata_kernel (token -> request search).
 *
 * Readings taken where the pages are silent or garbled are listed at each
 * function.  All pointers are host pointers; strides are in elements.
 * Every function returns 0, or -1 on an argument it cannot handle.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_WIDTH 16

/* ---------------------------------------------------------------- bf16 -- */

/* bf16 is the top half of an IEEE binary32; widening is exact. */
double oracle_bf16_to_f64(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Round a double straight to bf16, nearest-even, in one step (no detour
 * through float, which would round twice).  bf16 keeps 8 significant bits and
 * float's exponent range: normal numbers have exponent >= -126, below that the
 * grid spacing stays 2^-133 (subnormals).  NaN becomes the canonical quiet
 * NaN 0x7FC0; magnitudes that round past the largest finite value become inf. */
uint16_t oracle_f64_to_bf16(double v)
{
    if (isnan(v))
        return 0x7FC0;
    if (isinf(v))
        return signbit(v) ? 0xFF80 : 0x7F80;
    if (v == 0.0)
        return signbit(v) ? 0x8000 : 0x0000;
    int e;
    (void)frexp(v, &e);          /* |v| = m * 2^e with m in [0.5, 1) */
    int lead = e - 1;            /* exponent of the leading bit */
    if (lead < -126)
        lead = -126;             /* subnormal range: fixed spacing */
    int ulp_exp = lead - 7;      /* 8 significant bits */
    double r = nearbyint(ldexp(v, -ulp_exp));   /* default mode: ties-to-even */
    double q = ldexp(r, ulp_exp);
    if (fabs(q) >= 0x1p128)
        return signbit(v) ? 0xFF80 : 0x7F80;
    float f = (float)q;          /* exact: q has <= 8 significant bits */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16);
}

/* SiLU / swish, a * sigmoid(a), written as a / (1 + e^-a) [P1 fwd kernel
 * epilogue; P2 uses a*sigmoid(a); P3 uses F.silu -- all the same function]. */
double oracle_silu(double a)
{
    return a / (1.0 + exp(-a));
}

/* ------------------------------------------------------- varlen forward -- */

/*
 * Varlen prefill with a per-sequence conv state [P1 causal_conv1d_fn /
 * _causal_conv1d_fwd_kernel; definition from P3 Model.forward].
 *
 * x      : logical [dim][total_T], element (c, t) at x[c*x_sd + t*x_st]
 * weight : logical [dim][width],   element (c, j) at weight[c*w_sd + j*w_sw]
 * bias   : [dim] or NULL
 * conv_states : logical [num_lines][dim][width-1], element (l, c, k) at
 *          conv_states[l*cs_sl + c*cs_sd + k*cs_st]; column 0 is the oldest
 *          input.  May be NULL (no history, no state write).
 * cache_indices : [batch] or NULL (then sequence s uses line s)
 * has_init : [batch] bytes (0 / non-0) or NULL (all false)
 * qsl    : [batch+1] token offsets, qsl[0] = 0, non-decreasing
 * out    : logical [dim][total_T] with strides o_sd, o_st
 *
 * For sequence s with tokens [qsl[s], qsl[s+1]) and length L:
 *   h[c][k]  = has_init[s] ? conv_states[line][c][k] : 0      (k < width-1)
 *   u[c]     = h[c] ++ x[c][qsl[s] .. qsl[s+1])                (length width-1+L)
 *   y[c][t]  = bias[c] + sum_j weight[c][j] * u[c][t + j]       (t < L)
 *   out[c][qsl[s]+t] = bf16(silu?(y))
 *   conv_states[line][c][k] = u[c][L + k]  (the last width-1 entries of u)
 * Readings: a sequence whose line equals pad_slot_id (only when cache_indices
 * is given) or lies outside [0, num_lines) (only when conv_states is given) is
 * skipped: its outputs and every state line stay untouched.  A zero-length
 * sequence writes nothing.  has_init without conv_states means zero history.
 */
int oracle_fwd_varlen(const uint16_t *x, int64_t x_sd, int64_t x_st,
                      const uint16_t *weight, int64_t w_sd, int64_t w_sw,
                      const uint16_t *bias,
                      uint16_t *conv_states, int64_t cs_sl, int64_t cs_sd,
                      int64_t cs_st, int64_t num_lines,
                      const int32_t *cache_indices, const uint8_t *has_init,
                      const int32_t *qsl, int32_t batch, int32_t dim,
                      int32_t width, int32_t silu, int32_t pad_slot_id,
                      uint16_t *out, int64_t o_sd, int64_t o_st)
{
    if (width < 1 || width > ORACLE_MAX_WIDTH || dim < 0 || batch < 0)
        return -1;
    const int hist = width - 1;

    for (int32_t s = 0; s < batch; ++s) {
        const int64_t start = qsl[s];
        const int64_t len = (int64_t)qsl[s + 1] - start;
        int64_t line = cache_indices ? (int64_t)cache_indices[s] : (int64_t)s;
        if (cache_indices && line == pad_slot_id)
            continue;
        if (conv_states && (line < 0 || line >= num_lines))
            continue;
        if (len <= 0)
            continue;
        const int init = (conv_states && has_init && has_init[s]) ? 1 : 0;

        /* u as raw bf16 bits so that the state write is a bit copy. */
        uint16_t *u = (uint16_t *)malloc((size_t)(hist + len) * sizeof(uint16_t));
        if (!u)
            return -1;
        for (int32_t c = 0; c < dim; ++c) {
            for (int k = 0; k < hist; ++k)
                u[k] = init ? conv_states[line * cs_sl + c * cs_sd + k * cs_st] : 0;
            for (int64_t t = 0; t < len; ++t)
                u[hist + t] = x[c * x_sd + (start + t) * x_st];

            for (int64_t t = 0; t < len; ++t) {
                double acc = bias ? oracle_bf16_to_f64(bias[c]) : 0.0;
                for (int j = 0; j < width; ++j)
                    acc += oracle_bf16_to_f64(weight[c * w_sd + j * w_sw]) *
                           oracle_bf16_to_f64(u[t + j]);
                if (silu)
                    acc = oracle_silu(acc);
                out[c * o_sd + (start + t) * o_st] = oracle_f64_to_bf16(acc);
            }
            if (conv_states)
                for (int k = 0; k < hist; ++k)
                    conv_states[line * cs_sl + c * cs_sd + k * cs_st] = u[len + k];
        }
        free(u);
    }
    return 0;
}

/* -------------------------------------------------------- decode update -- */

/*
 * Decode-time update [P1 causal_conv1d_update / _causal_conv1d_update_kernel]:
 * x is logical [batch][dim][seqlen]; every entry continues from its cached
 * state (the history is always the state), the state becomes the last
 * width-1 entries of state ++ x, and out receives the outputs.  out may be
 * the same buffer as x (the page writes the result in place): each entry's
 * inputs are copied before any output is written.
 * Readings: seqlen > 1 follows the same "last width-1 of state ++ x" rule as
 * the forward; an entry whose line equals pad_slot_id (cache_indices given) or
 * is outside [0, num_lines) is skipped.
 */
int oracle_update_decode(const uint16_t *x, int64_t x_sb, int64_t x_sd, int64_t x_st,
                         const uint16_t *weight, int64_t w_sd, int64_t w_sw,
                         const uint16_t *bias,
                         uint16_t *conv_state, int64_t cs_sl, int64_t cs_sd,
                         int64_t cs_st, int64_t num_lines,
                         const int32_t *cache_indices, int32_t batch, int32_t dim,
                         int32_t seqlen, int32_t width, int32_t silu,
                         int32_t pad_slot_id,
                         uint16_t *out, int64_t o_sb, int64_t o_sd, int64_t o_st)
{
    if (width < 1 || width > ORACLE_MAX_WIDTH || dim < 0 || batch < 0 || seqlen < 0)
        return -1;
    const int hist = width - 1;
    uint16_t *u = (uint16_t *)malloc((size_t)(hist + seqlen + 1) * sizeof(uint16_t));
    if (!u)
        return -1;
    for (int32_t b = 0; b < batch; ++b) {
        int64_t line = cache_indices ? (int64_t)cache_indices[b] : (int64_t)b;
        if (cache_indices && line == pad_slot_id)
            continue;
        if (line < 0 || line >= num_lines)
            continue;
        for (int32_t c = 0; c < dim; ++c) {
            for (int k = 0; k < hist; ++k)
                u[k] = conv_state[line * cs_sl + c * cs_sd + k * cs_st];
            for (int32_t t = 0; t < seqlen; ++t)
                u[hist + t] = x[b * x_sb + c * x_sd + t * x_st];
            for (int32_t t = 0; t < seqlen; ++t) {
                double acc = bias ? oracle_bf16_to_f64(bias[c]) : 0.0;
                for (int j = 0; j < width; ++j)
                    acc += oracle_bf16_to_f64(weight[c * w_sd + j * w_sw]) *
                           oracle_bf16_to_f64(u[t + j]);
                if (silu)
                    acc = oracle_silu(acc);
                out[b * o_sb + c * o_sd + t * o_st] = oracle_f64_to_bf16(acc);
            }
            for (int k = 0; k < hist; ++k)
                conv_state[line * cs_sl + c * cs_sd + k * cs_st] = u[seqlen + k];
        }
    }
    free(u);
    return 0;
}

/*
 * General decode update with the speculative-decoding and circular-buffer
 * options of the same page [P1 causal_conv1d_update /
 * _causal_conv1d_update_kernel: num_accepted_tokens, intermediate_conv_window,
 * output_state_indices; cache_seqlens as its docstring describes it].
 *
 * x           : logical [batch][dim][seqlen]
 * conv_state  : logical [num_lines][dim][state_len], state_len >= width-1
 * cache_seqlens : [batch] or NULL.  Given: the line is a ring of state_len
 *          inputs; input number n of the stream sits at slot n mod state_len
 *          and cache_seqlens[b] inputs have been seen so far.
 * num_accepted : [batch] or NULL.  Given (speculative decoding): the history
 *          window starts at column num_accepted[b] - 1 of the line.
 * inter   : logical [batch][steps >= seqlen][dim][width-1] or NULL; element
 *          (b, t, c, k) at inter[b*i_sb + t*i_st + c*i_sd + k*i_sk].
 * out_idx : logical [batch][seqlen] line numbers or NULL, element (b, t) at
 *          out_idx[b*oi_sb + t*oi_st].
 *
 * For entry b and channel c, with W = width:
 *   h[k] (k < W-1), the history:
 *     ring:  state[(cache_seqlens[b] - (W-1) + k) mod state_len]
 *     else:  state[off + k], off = num_accepted ? num_accepted[b] - 1 : 0
 *   u = h ++ x[b][c][0..seqlen), out[t] = act(bias + sum_j w[j] u[t+j])
 *   win_t = u[t+1 .. t+W-1], the W-1 inputs that end with x[t]
 *   inter given:    inter[b][t][c][k] = win_t[k]
 *   out_idx given:  state[out_idx[b][t]][c][k] = win_t[k] for every t whose
 *                   index lies in [0, num_lines)
 *   state update in place, only when neither inter nor out_idx is given:
 *     ring:  x[t] goes to slot (cache_seqlens[b] + t) mod state_len (for the
 *            last min(seqlen, state_len) tokens: later tokens overwrite)
 *     speculative:  state[k] = u[1 + k] for k < W-2+seqlen, i.e. the history
 *            minus its oldest input, then all of x (the page's comment: the
 *            state becomes history2..historyM, draft1..draftN, and the next
 *            call's num_accepted picks the window that ends with the last
 *            accepted draft)
 *     plain: state[k] = u[seqlen + k] for k < W-1 (the decode rule above)
 * Readings (all defensive, the page leaves them open): an entry whose line is
 * pad_slot_id or out of range, whose num_accepted[b] - 1 + W-1 exceeds
 * state_len or is below W-1 (num_accepted < 1), or whose cache_seqlens[b] is
 * negative, is skipped entirely; the ring option excludes the three
 * speculative ones; without inter/out_idx a speculative call needs
 * state_len >= W-2+seqlen.  Every read of an entry happens before its writes,
 * so out may be x and out_idx may name the entry's own line.
 */
int oracle_update_general(const uint16_t *x, int64_t x_sb, int64_t x_sd, int64_t x_st,
                          const uint16_t *weight, int64_t w_sd, int64_t w_sw,
                          const uint16_t *bias,
                          uint16_t *conv_state, int64_t cs_sl, int64_t cs_sd,
                          int64_t cs_st, int64_t num_lines, int32_t state_len,
                          const int32_t *cache_indices, const int32_t *cache_seqlens,
                          const int32_t *num_accepted,
                          uint16_t *inter, int64_t i_sb, int64_t i_st, int64_t i_sd,
                          int64_t i_sk,
                          const int32_t *out_idx, int64_t oi_sb, int64_t oi_st,
                          int32_t batch, int32_t dim, int32_t seqlen, int32_t width,
                          int32_t silu, int32_t pad_slot_id,
                          uint16_t *out, int64_t o_sb, int64_t o_sd, int64_t o_st)
{
    if (width < 1 || width > ORACLE_MAX_WIDTH || dim < 0 || batch < 0 || seqlen < 0 ||
        state_len < width - 1)
        return -1;
    const int ring = cache_seqlens != NULL;
    const int spec = num_accepted != NULL;
    const int scatter = inter != NULL || out_idx != NULL;
    if (ring && (spec || scatter || state_len < 1))
        return -1;
    if (spec && !scatter && state_len < width - 2 + seqlen)
        return -1;
    const int hist = width - 1;
    uint16_t *u = (uint16_t *)malloc((size_t)(hist + seqlen + 1) * sizeof(uint16_t));
    if (!u)
        return -1;
    for (int32_t b = 0; b < batch; ++b) {
        const int64_t line = cache_indices ? (int64_t)cache_indices[b] : (int64_t)b;
        if (cache_indices && line == pad_slot_id)
            continue;
        if (line < 0 || line >= num_lines)
            continue;
        int64_t off = 0;
        if (spec) {
            off = (int64_t)num_accepted[b] - 1;
            if (off < 0 || off + hist > state_len)
                continue;
        }
        if (ring && cache_seqlens[b] < 0)
            continue;
        for (int32_t c = 0; c < dim; ++c) {
            uint16_t *row = conv_state + line * cs_sl + c * cs_sd;
            for (int k = 0; k < hist; ++k) {
                int64_t col = off + k;
                if (ring) {
                    col = ((int64_t)cache_seqlens[b] - hist + k) % state_len;
                    if (col < 0)
                        col += state_len;
                }
                u[k] = row[col * cs_st];
            }
            for (int32_t t = 0; t < seqlen; ++t)
                u[hist + t] = x[b * x_sb + c * x_sd + t * x_st];
            for (int32_t t = 0; t < seqlen; ++t) {
                double acc = bias ? oracle_bf16_to_f64(bias[c]) : 0.0;
                for (int j = 0; j < width; ++j)
                    acc += oracle_bf16_to_f64(weight[c * w_sd + j * w_sw]) *
                           oracle_bf16_to_f64(u[t + j]);
                if (silu)
                    acc = oracle_silu(acc);
                out[b * o_sb + c * o_sd + t * o_st] = oracle_f64_to_bf16(acc);
            }
            for (int32_t t = 0; t < seqlen; ++t) {
                if (inter)
                    for (int k = 0; k < hist; ++k)
                        inter[b * i_sb + t * i_st + c * i_sd + k * i_sk] = u[t + 1 + k];
                if (out_idx) {
                    const int64_t dst = out_idx[b * oi_sb + t * oi_st];
                    if (dst >= 0 && dst < num_lines)
                        for (int k = 0; k < hist; ++k)
                            conv_state[dst * cs_sl + c * cs_sd + k * cs_st] = u[t + 1 + k];
                }
            }
            if (scatter)
                continue;
            if (ring) {
                const int32_t first = seqlen > state_len ? seqlen - state_len : 0;
                for (int32_t t = first; t < seqlen; ++t) {
                    const int64_t col = ((int64_t)cache_seqlens[b] + t) % state_len;
                    row[col * cs_st] = u[hist + t];
                }
            } else if (spec) {
                for (int k = 0; k < hist - 1 + seqlen; ++k)
                    row[k * cs_st] = u[1 + k];
            } else {
                for (int k = 0; k < hist; ++k)
                    row[k * cs_st] = u[seqlen + k];
            }
        }
    }
    free(u);
    return 0;
}

/* ---------------------------------------------------- paged fused step -- */

/* Request owning token row t: the largest j in [0, num_reqs) with
 * qsl[j] <= t [P2 _seq_metadata_kernel]. Written as a linear scan. */
static int32_t oracle_request_of(const int32_t *qsl, int32_t num_reqs, int64_t t)
{
    int32_t r = 0;
    for (int32_t j = 0; j < num_reqs; ++j)
        if ((int64_t)qsl[j] <= t)
            r = j;
    return r;
}

/*
 * Paged sliding-window insert + depthwise conv [P2 _fused_sconv_kernel].
 *
 * x      : [T][C] with row stride x_st, C = num_heads * ws; channel c lives in
 *          head c / ws at cache D-index off_s + c % ws.
 * cache  : [num_blocks][num_heads][block_size][head_dim], element
 *          (b, h, n, d) at cache[b*c_sb + h*c_sh + n*c_sn + d]; it holds the
 *          conv INPUT at every absolute position, position p of a request in
 *          block block_table[r][p / block_size], slot p % block_size.
 * positions / slot_mapping : [T] int64; slot < 0 marks a pad row.
 * qsl    : [num_reqs+1]; block_table element (r, i) at block_table[r*bt_sr + i].
 *
 * Snapshot semantics: all taps read the cache as it was before the call,
 * then every non-pad row's input is inserted at its slot.  For a non-pad row t
 * of request r (first row qstart = qsl[r]) at position p:
 *   tap j (0..W-1) covers position src = p - (W-1) + j and row = t - (W-1) + j;
 *   value = 0                      if src < 0
 *         = x[row][c]              if row >= qstart (inside this forward)
 *         = cache[bt[r][src/N]][c/ws][src%N][off_s + c%ws]   otherwise
 *   y = bias[c] + sum_j weight[c][j] * value_j ; y = silu(y) if asked;
 *   y += x[t][c] if residual ; out[t][c] = bf16(y).
 * Pad rows (slot < 0, or rows at or past qsl[num_reqs]) are not convolved
 * (y = 0, bias not added), are not inserted, and out = bf16(silu?(0) + x)
 * with residual, i.e. x itself, else 0.
 * Readings: a cached tap whose logical block is >= max_blocks, or whose block
 * id is outside [0, num_blocks), contributes 0; an insert whose slot block is
 * outside [0, num_blocks) is dropped.
 */
int oracle_paged(const uint16_t *x, int64_t x_st,
                 const uint16_t *weight, int64_t w_sd, int64_t w_sw,
                 const uint16_t *bias,
                 uint16_t *cache, int64_t c_sb, int64_t c_sh, int64_t c_sn,
                 int64_t num_blocks, int32_t num_heads, int32_t block_size,
                 int32_t off_s, int32_t ws,
                 const int64_t *positions, const int64_t *slot_mapping,
                 const int32_t *qsl, int32_t num_reqs,
                 const int32_t *block_table, int64_t bt_sr, int32_t max_blocks,
                 int64_t num_tokens, int32_t width, int32_t silu,
                 int32_t residual, uint16_t *out, int64_t o_st)
{
    if (width < 1 || width > ORACLE_MAX_WIDTH || num_heads < 0 || ws < 0 ||
        block_size < 1 || num_reqs < 0 || num_tokens < 0)
        return -1;
    const int64_t C = (int64_t)num_heads * ws;
    const int64_t actual = num_reqs > 0 ? (int64_t)qsl[num_reqs] : 0;

    /* Phase 1: every output from the pre-call cache. */
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int pad = slot_mapping[t] < 0 || t >= actual;
        const int32_t r = pad ? 0 : oracle_request_of(qsl, num_reqs, t);
        const int64_t qstart = pad ? 0 : qsl[r];
        const int64_t pos = positions[t];
        for (int64_t c = 0; c < C; ++c) {
            const int64_t head = c / ws;
            const int64_t d = off_s + c % ws;
            double acc = 0.0;
            if (!pad) {
                acc = bias ? oracle_bf16_to_f64(bias[c]) : 0.0;
                for (int j = 0; j < width; ++j) {
                    const int64_t src = pos - (width - 1) + j;
                    const int64_t row = t - (width - 1) + j;
                    double v = 0.0;
                    if (src < 0) {
                        v = 0.0;
                    } else if (row >= qstart) {
                        v = oracle_bf16_to_f64(x[row * x_st + c]);
                    } else {
                        const int64_t lblk = src / block_size;
                        if (lblk < max_blocks) {
                            const int64_t blk = block_table[r * bt_sr + lblk];
                            if (blk >= 0 && blk < num_blocks)
                                v = oracle_bf16_to_f64(
                                    cache[blk * c_sb + head * c_sh +
                                          (src % block_size) * c_sn + d]);
                        }
                    }
                    acc += oracle_bf16_to_f64(weight[c * w_sd + j * w_sw]) * v;
                }
            }
            if (silu)
                acc = oracle_silu(acc);
            if (residual)
                acc += oracle_bf16_to_f64(x[t * x_st + c]);
            out[t * o_st + c] = oracle_f64_to_bf16(acc);
        }
    }

    /* Phase 2: insert the inputs of the non-pad rows. */
    for (int64_t t = 0; t < num_tokens; ++t) {
        const int64_t slot = slot_mapping[t];
        if (slot < 0 || t >= actual)
            continue;
        const int64_t blk = slot / block_size;
        const int64_t n = slot % block_size;
        if (blk >= num_blocks)
            continue;
        for (int64_t c = 0; c < C; ++c)
            cache[blk * c_sb + (c / ws) * c_sh + n * c_sn + off_s + c % ws] =
                x[t * x_st + c];
    }
    return 0;
}

/* Token -> (request, first row) metadata [P2 _seq_metadata_kernel]: rows
 * below num_actual get the owning request and its first row, rows in
 * [num_actual, num_padded) get 0 / 0. */
int oracle_seq_metadata(const int32_t *qsl, int32_t num_reqs, int64_t num_actual,
                        int64_t num_padded, int32_t *seq_idx, int32_t *query_start)
{
    if (num_padded < num_actual || num_reqs < 1)
        return -1;
    for (int64_t t = 0; t < num_padded; ++t) {
        if (t < num_actual) {
            const int32_t r = oracle_request_of(qsl, num_reqs, t);
            seq_idx[t] = r;
            query_start[t] = qsl[r];
        } else {
            seq_idx[t] = 0;
            query_start[t] = 0;
        }
    }
    return 0;
}

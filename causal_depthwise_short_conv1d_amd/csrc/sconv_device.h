// Device-side helpers for the gfx950 short-conv kernels: bf16 packing,
// 16-byte vector memory access, SiLU, and the varlen sequence lookup.
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

#include "sconv_params.h"

namespace sconv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ------------------------------------------------------------------ bf16 --
// A bf16 is the upper half of a binary32, so widening is a shift or a mask.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf_one(uint16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// fp32 -> bf16 round-to-nearest-even; gfx950 converts a pair in one
// instruction (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
__device__ __forceinline__ uint16_t to_bf16(float v) {
    return uint16_t(pack_bf16x2(v, 0.0f) & 0xffffu);
}

// Unpack 8 bf16 held in a 16-byte vector into floats.
__device__ __forceinline__ void unpack8(const u32x4 &v, float f[8]) {
    f[0] = bf_lo(v.x); f[1] = bf_hi(v.x);
    f[2] = bf_lo(v.y); f[3] = bf_hi(v.y);
    f[4] = bf_lo(v.z); f[5] = bf_hi(v.z);
    f[6] = bf_lo(v.w); f[7] = bf_hi(v.w);
}
__device__ __forceinline__ u32x4 pack8(const float f[8]) {
    u32x4 r;
    r.x = pack_bf16x2(f[0], f[1]);
    r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]);
    r.w = pack_bf16x2(f[6], f[7]);
    return r;
}

// ------------------------------------------------------------------ SiLU --
// silu(a) = a * sigmoid(a) = a / (1 + e^-a), with the hardware exp2 and
// reciprocal (about 1 ulp each, far below the bf16 output rounding).
template <bool SILU>
__device__ __forceinline__ float act(float a) {
    if constexpr (SILU) {
        const float e = __builtin_amdgcn_exp2f(a * -1.4426950408889634f);
        return a * __builtin_amdgcn_rcpf(1.0f + e);
    } else {
        return a;
    }
}

// -------------------------------------------------------- vector memory --
__device__ __forceinline__ u32x4 ld16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
// Streaming (non-temporal) load for data read exactly once.
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16_stream(uint16_t *p, const u32x4 &v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}
__device__ __forceinline__ void st16(uint16_t *p, const u32x4 &v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// 8 consecutive channels of which only the first n (0..8) exist: a full
// vector access when n == 8, element accesses otherwise (zero filled).
__device__ __forceinline__ u32x4 ld8_partial(const uint16_t *p, int n) {
    if (n >= 8) return ld16(p);
    uint16_t e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) e[i] = (i < n) ? p[i] : uint16_t(0);
    u32x4 r;
    r.x = e[0] | (uint32_t(e[1]) << 16);
    r.y = e[2] | (uint32_t(e[3]) << 16);
    r.z = e[4] | (uint32_t(e[5]) << 16);
    r.w = e[6] | (uint32_t(e[7]) << 16);
    return r;
}
__device__ __forceinline__ void st8_partial(uint16_t *p, const u32x4 &v, int n, bool stream) {
    if (n >= 8) {
        if (stream) st16_stream(p, v); else st16(p, v);
        return;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < n) p[i] = uint16_t((w[i >> 1] >> ((i & 1) * 16)) & 0xffffu);
}
__device__ __forceinline__ uint16_t lane_elem(const u32x4 &v, int i) {
    const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
    return uint16_t((w >> ((i & 1) * 16)) & 0xffffu);
}

// ---------------------------------------------------- buffer descriptors --
// A load through a buffer descriptor whose offset lies past the descriptor's
// extent returns 0 without touching memory (a store is dropped).  Latency-
// critical paths use this to issue every load unconditionally -- a load under
// a branch makes the compiler wait for it before the branch joins, which
// turns a handful of independent loads into a chain of round trips.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOob = 0x80000000u;            // an offset past every extent

// `bytes` is clamped to [0, 2^31 - 1]; 0 makes every access out of range.
__device__ __forceinline__ Rsrc make_rsrc(const void *base, int64_t bytes) {
    const int n = bytes <= 0 ? 0 : (bytes < 0x7fffffff ? int(bytes) : 0x7fffffff);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), short(0), n, 0x00020000);
}
__device__ __forceinline__ uint16_t buf_ld16(Rsrc r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
template <int AUX>
__device__ __forceinline__ u32x4 buf_ld128(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, AUX));
}

// Taps of 4 adjacent channels whose weights are stored contiguously
// (row stride == width): 4*W bf16 = 8W bytes from byte `off` of `wr`, read
// with 16- and 8-byte loads (W * 8 = 16, 24, 32, 40 bytes for W = 2..5; the
// offset is a multiple of 8W, so every load is 8-byte aligned).  Pair q of
// channel ch is (w[ch][2q], w[ch][2q+1]) as packed bf16, wl[ch] the odd last
// tap; bias (4 bf16 at byte `boff` of `br`) as fp32.
template <int W>
__device__ __forceinline__ void load_taps4(Rsrc wr, uint32_t off, Rsrc br, uint32_t boff,
                                           uint32_t (&wp)[W / 2 > 0 ? W / 2 : 1][4],
                                           float (&wl)[4], float (&b)[4]) {
    constexpr int kDw = 2 * W;                 // dwords of the 4 channels' taps
    uint32_t d[kDw];
#pragma unroll
    for (int i = 0; i + 4 <= kDw; i += 4) {
        const u32x4 v = buf_ld128<0>(wr, off + 4 * i);
        d[i] = v.x; d[i + 1] = v.y; d[i + 2] = v.z; d[i + 3] = v.w;
    }
    if constexpr (kDw % 4 == 2) {
        const u32x2 v = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(wr, off + 4 * (kDw - 2), 0, 0));
        d[kDw - 2] = v.x; d[kDw - 1] = v.y;
    }
    // element e of the 4W is half (e & 1) of dword e / 2
#pragma unroll
    for (int ch = 0; ch < 4; ++ch) {
#pragma unroll
        for (int q = 0; q < W / 2; ++q) {
            const int e = ch * W + 2 * q;
            wp[q][ch] = (e & 1) ? __builtin_amdgcn_alignbit(d[(e + 1) / 2], d[e / 2], 16) : d[e / 2];
        }
        const int el = ch * W + W - 1;
        wl[ch] = (W & 1) ? ((el & 1) ? bf_hi(d[el / 2]) : bf_lo(d[el / 2])) : 0.0f;
    }
    const u32x2 bv = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(br, boff, 0, 0));
    b[0] = bf_lo(bv.x); b[1] = bf_hi(bv.x); b[2] = bf_lo(bv.y); b[3] = bf_hi(bv.y);
}

// -------------------------------------------------- wave-uniform loads --
// Reads of read-only, wave-uniform data through the scalar cache (constant
// address space): they take no vector-memory issue slots and land directly
// in scalar registers.  Only whole dwords that hold a wanted byte are read,
// so no access leaves the dword-aligned span of the data.
typedef const __attribute__((address_space(4))) uint32_t KU32;

__device__ __forceinline__ KU32 *kptr(uintptr_t a) { return reinterpret_cast<KU32 *>(a); }

__device__ __forceinline__ uint32_t sld_u32(const void *p) {
    return *kptr(reinterpret_cast<uintptr_t>(p));
}
__device__ __forceinline__ uint32_t sld_u16(const uint16_t *p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return (*kptr(a & ~uintptr_t(3)) >> ((a & 2) * 8)) & 0xffffu;
}
__device__ __forceinline__ uint32_t sld_u8(const uint8_t *p) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return (*kptr(a & ~uintptr_t(3)) >> ((a & 3) * 8)) & 0xffu;
}

// K consecutive 16-bit values from p (wave-uniform, 2-byte aligned) as
// dwords: value k is bits [16(k&1), 16(k&1)+16) of d[k/2], so d[q] is the
// pair (2q, 2q+1) whatever the alignment of p.
// Marks a wave-uniform value as used at this point: its load completes here
// instead of being sunk into the (branch) block that first reads it.
__device__ __forceinline__ void pin_sgpr(uint32_t v) { asm volatile("" ::"s"(v)); }

template <int K>
struct U16Run {
    uint32_t d[K / 2 + 1];
    __device__ __forceinline__ uint32_t elem(int k) const { return (d[k >> 1] >> (16 * (k & 1))) & 0xffffu; }
};
template <int K>
__device__ __forceinline__ U16Run<K> sld_run(const uint16_t *p) {
    constexpr int N = K / 2 + 1;
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uintptr_t q = a & ~uintptr_t(3);
    const uint32_t m = uint32_t(a >> 1) & 1u;             // 1 when p is not dword aligned
    // The run spans dwords 0..K/2 except for an even K at an aligned p, which
    // ends at dword K/2 - 1; that dword is then read twice instead.
    uint32_t raw[N];
#pragma unroll
    for (int i = 0; i < N - 1; ++i) raw[i] = kptr(q)[i];
    raw[N - 1] = (K & 1) ? kptr(q)[N - 1] : kptr(q + 4 * (N - 2 + m))[0];
    U16Run<K> r;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint64_t hi = i + 1 < N ? uint64_t(raw[i + 1]) << 32 : 0;
        r.d[i] = uint32_t((hi | raw[i]) >> (16 * m));
    }
    return r;
}

// -------------------------------------------------- varlen sequence lookup --
// Largest j in [0, n) with qsl[j] <= t (the token -> sequence search of the
// Inkling page's metadata kernel).  Works for any qsl contents: the result
// is always a valid index.
__device__ __forceinline__ int32_t seq_search(const int32_t *qsl, int32_t n, int64_t t) {
    int32_t lo = 0, hi = n - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi + 1) >> 1;
        if (int64_t(qsl[mid]) <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// What the forward kernels need to know about one sequence.
struct SeqInfo {
    int64_t start, end;   // token range, clamped into [0, total_T]
    int64_t line;         // cache line
    bool skip;            // padded, or its line is out of range
    bool init;            // continue from the cached state
};

__device__ __forceinline__ SeqInfo seq_info(const SeqBatch &sb, const int32_t *qsl, int32_t s) {
    SeqInfo si;
    int64_t a = qsl[s], b = qsl[s + 1];
    a = a < 0 ? 0 : (a > sb.total_T ? sb.total_T : a);
    b = b < a ? a : (b > sb.total_T ? sb.total_T : b);
    si.start = a;
    si.end = b;
    si.line = sb.cache_idx ? int64_t(sb.cache_idx[s]) : int64_t(s);
    si.skip = (sb.cache_idx && si.line == sb.pad_slot_id) ||
              (sb.cs && (si.line < 0 || si.line >= sb.num_lines));
    si.init = sb.cs && sb.has_init && sb.has_init[s] != 0;
    return si;
}

// seq_info() of sequence s (wave-uniform) with every read a scalar load at
// an address that is always readable (a null array reads query_start_loc
// instead), so the reads need no branch and can overlap earlier loads.
__device__ __forceinline__ SeqInfo seq_info_scalar(const SeqBatch &sb, int32_t s) {
    SeqInfo si;
    int64_t a = int32_t(sld_u32(sb.qsl + s)), b = int32_t(sld_u32(sb.qsl + s + 1));
    a = a < 0 ? 0 : (a > sb.total_T ? sb.total_T : a);
    b = b < a ? a : (b > sb.total_T ? sb.total_T : b);
    si.start = a;
    si.end = b;
    const int32_t ci = int32_t(sld_u32(sb.cache_idx ? sb.cache_idx + s : sb.qsl));
    const uint32_t hi = sld_u8(sb.has_init ? sb.has_init + s : reinterpret_cast<const uint8_t *>(sb.qsl));
    si.line = sb.cache_idx ? int64_t(ci) : int64_t(s);
    si.skip = (sb.cache_idx && si.line == sb.pad_slot_id) ||
              (sb.cs && (si.line < 0 || si.line >= sb.num_lines));
    si.init = sb.cs && sb.has_init && hi != 0;
    return si;
}

}  // namespace sconv

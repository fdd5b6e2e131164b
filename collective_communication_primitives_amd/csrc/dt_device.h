// dt_device.h -- device-side building blocks shared by the HIP kernels:
// 16-byte vector memory access, bf16 <-> fp32 conversion and the element
// operators of the rank fold.
//
// The fold follows the DTorch same-device AllReduce (page "集合通信组件",
// sec. 2.3): start from rank 0's element and combine ranks 1..P-1 in rank
// order.  Accumulation is fp32 for fp32 and bf16 data (one round to nearest
// even at the end) and int32 (wrapping) for int32 data.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dt {

enum : int { kF32 = 0, kBF16 = 1, kI32 = 2 };
enum : int { kSum = 0, kMax = 1, kMin = 2, kAvg = 3 };

constexpr int kMaxRanks = 16;
constexpr int kBlock = 256;  // threads per workgroup: four 64-wide waves

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- memory --
// Every byte is touched once per launch.  Whether a side carries the
// non-temporal hint is chosen per kernel from measurements on the MI355X
// (1.1 GiB working sets, beyond the Infinity Cache): with reads dominating
// (P-to-1 fold), non-temporal loads and device-scope stores are fastest; with
// writes dominating (1-to-P fan-out), plain loads and non-temporal
// device-scope stores; for the balanced P-to-P fold and for 1-to-1 copies,
// both non-temporal.
__device__ __forceinline__ u32x4 load16(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void store16(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}
template <bool NT>
__device__ __forceinline__ u32x4 load16_h(const void* p) {
    if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    else return *reinterpret_cast<const u32x4*>(p);
}

// Buffer-instruction access.  A workgroup describes each contiguous range it
// touches with a buffer resource (base address in scalar registers, byte
// range) and addresses lanes with 32-bit offsets.  The hardware checks every
// access against the range: a 16-byte load at or past the end returns zeros
// and a store there is dropped, so a ragged last tile needs no per-lane
// branch.  The last operand selects the cache policy of the access:
// bit 1 = non-temporal, bit 4 = device scope (the store is written through
// the XCD's L2 towards memory instead of staying there dirty until the
// kernel ends).  Ranges are at most a few tiles, far below the 4 GiB limit.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kPolNT = 2;
constexpr int kPolDevice = 16;
constexpr int kRsrcFlags = 0x00020000;  // word 3: 32-bit data format, raw (stride 0) addressing

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), kRsrcFlags);
}
template <int POL>
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, POL);
}
template <int POL>
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, u32x4 v) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(off), 0, POL);
}

// Bytes [s, s + 16) of the 32 bytes lo:hi (little endian), 0 <= s <= 15,
// s the same in every lane: a 16-byte vector of a source that is not
// 16-byte aligned, built from the two aligned vectors around it.  The word
// selection branches on the uniform s / 4; v_alignbyte joins two words.
__device__ __forceinline__ u32x4 funnel16(u32x4 lo, u32x4 hi, uint32_t s) {
    const uint32_t b = s & 3u;
    u32x4 o;
    switch (s >> 2) {
        case 0:
            o[0] = __builtin_amdgcn_alignbyte(lo[1], lo[0], b);
            o[1] = __builtin_amdgcn_alignbyte(lo[2], lo[1], b);
            o[2] = __builtin_amdgcn_alignbyte(lo[3], lo[2], b);
            o[3] = __builtin_amdgcn_alignbyte(hi[0], lo[3], b);
            break;
        case 1:
            o[0] = __builtin_amdgcn_alignbyte(lo[2], lo[1], b);
            o[1] = __builtin_amdgcn_alignbyte(lo[3], lo[2], b);
            o[2] = __builtin_amdgcn_alignbyte(hi[0], lo[3], b);
            o[3] = __builtin_amdgcn_alignbyte(hi[1], hi[0], b);
            break;
        case 2:
            o[0] = __builtin_amdgcn_alignbyte(lo[3], lo[2], b);
            o[1] = __builtin_amdgcn_alignbyte(hi[0], lo[3], b);
            o[2] = __builtin_amdgcn_alignbyte(hi[1], hi[0], b);
            o[3] = __builtin_amdgcn_alignbyte(hi[2], hi[1], b);
            break;
        default:
            o[0] = __builtin_amdgcn_alignbyte(hi[0], lo[3], b);
            o[1] = __builtin_amdgcn_alignbyte(hi[1], hi[0], b);
            o[2] = __builtin_amdgcn_alignbyte(hi[2], hi[1], b);
            o[3] = __builtin_amdgcn_alignbyte(hi[3], hi[2], b);
            break;
    }
    return o;
}

// Aligned loads over the part of a byte range [s, s + n) that one tile
// reads, for kernels that shift vectors: the tile's loads start at offset o_t
// from s (o_t + s aligned, o_t may be negative) and span `span` bytes.  The
// window is a buffer resource over the aligned vectors of that span which
// hold at least one byte of the range, so a load at any offset outside them
// (before the range's first vector or past its last) returns zeros without
// touching memory, and the lanes at a range's two ends load like the rest.
struct LoadWindow {
    rsrc_t r;
    int64_t b;  // offset from s of the resource's first byte
};
__device__ __forceinline__ LoadWindow load_window(const char* s, int64_t n, int64_t o_t, int64_t span) {
    const int64_t head = int64_t(reinterpret_cast<uintptr_t>(s) & 15u);
    const int64_t o_end = ((head + n + 15) & ~int64_t(15)) - head;  // past the range's last aligned vector
    const int64_t b = o_t > -head ? o_t : -head;
    const int64_t e = o_t + span < o_end ? o_t + span : o_end;
    return LoadWindow{make_rsrc(s + b, uint32_t(e > b ? e - b : 0)), b};
}
// The aligned vector at s + o (o - w.b wraps to far past the window when o < w.b).
template <int POL>
__device__ __forceinline__ u32x4 window_load(const LoadWindow& w, int64_t o) {
    return bload16<POL>(w.r, uint32_t(o - w.b));
}
// Bytes [o + sm, o + sm + 16) of the range: the aligned vectors at o and o + 16
// joined (sm = 0: the one at o).
template <int POL>
__device__ __forceinline__ u32x4 window_load_shifted(const LoadWindow& w, int64_t o, uint32_t sm) {
    const u32x4 lo = window_load<POL>(w, o);
    if (sm == 0) return lo;
    return funnel16(lo, window_load<POL>(w, o + 16), sm);
}
// The 16 bytes at p (p & 15 == misalign, uniform across the lanes) from
// aligned loads: the one aligned vector holding them, or the two around them.
// Each of those vectors holds at least one of the 16 bytes, so none reaches a
// page that the bytes themselves do not touch.
template <bool NT>
__device__ __forceinline__ u32x4 load16_any(const char* p, uint32_t misalign) {
    const char* a = p - misalign;
    const u32x4 lo = load16_h<NT>(a);
    if (misalign == 0) return lo;
    return funnel16(lo, load16_h<NT>(a + 16), misalign);
}
// Elements of v (ES bytes each, little endian) between its bytes j0 and j1
// that fall inside [0, n) when v's byte 0 is byte `at` of a range at d:
// one store each.
template <int ES>
__device__ __forceinline__ void store_vec_elems(char* d, int64_t at, const u32x4& v, int j0, int j1, int64_t n) {
#pragma unroll
    for (int j = 0; j < 16; j += ES) {
        if (j < j0 || j >= j1 || at + j < 0 || at + j >= n) continue;
        if constexpr (ES == 2) *reinterpret_cast<uint16_t*>(d + at + j) = uint16_t(v[j >> 2] >> ((j & 2) * 8));
        else *reinterpret_cast<uint32_t*>(d + at + j) = v[j >> 2];
    }
}
// Byte j of a vector.
__device__ __forceinline__ char vec_byte(const u32x4& x, int j) { return char(x[j >> 2] >> ((j & 3) * 8)); }

// ------------------------------------------------------------------- bf16 --
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_at(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// fp32 -> bf16 bits, round to nearest with ties to even, computed on the
// integer pattern; a NaN keeps its sign and top payload bits and gets the
// quiet bit; overflow to infinity comes out of the carry.
__device__ __forceinline__ uint32_t to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
    uint32_t quiet = (u >> 16) | 0x40u;
    return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? quiet : rounded;
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return to_bf16(lo) | (to_bf16(hi) << 16);
}

// -------------------------------------------------------------- operators --
// Max/min: strict compare, the accumulator wins ties (earlier rank, also
// between +0 and -0); the first NaN met is kept.  Avg folds as a sum and
// divides once at the end (finish()).
template <int OP>
__device__ __forceinline__ float combine(float a, float v) {
    if constexpr (OP == kSum || OP == kAvg) {
        return a + v;
    } else {
        const bool a_nan = a != a;
        const bool v_nan = v != v;
        const bool take = (OP == kMax) ? (v > a) : (v < a);
        return a_nan ? a : ((v_nan || take) ? v : a);
    }
}

template <int OP>
__device__ __forceinline__ int32_t combine(int32_t a, int32_t v) {
    if constexpr (OP == kSum || OP == kAvg) {
        return int32_t(uint32_t(a) + uint32_t(v));
    } else if constexpr (OP == kMax) {
        return v > a ? v : a;
    } else {
        return v < a ? v : a;
    }
}

// The mean: one IEEE division of the fp32 sum (correctly rounded), or C's
// truncating division of the wrapped int32 sum, by the rank count.
template <int OP>
__device__ __forceinline__ float finish(float a, int nr) {
    if constexpr (OP == kAvg) return a / float(nr);
    else return a;
}
template <int OP>
__device__ __forceinline__ int32_t finish(int32_t a, int nr) {
    if constexpr (OP == kAvg) return a / nr;
    else return a;
}

// Elements per 16-byte vector.
template <int DT>
struct Elems {
    static constexpr int value = DT == kBF16 ? 8 : 4;
};

// Fold P vectors (x[0..P-1]) element-wise in rank order.  NR = live ranks
// (runtime, NR <= P); with NR == P the selects fold away.  A slot past the
// live ranks is combined and its result discarded by a select, not skipped
// by a branch: a branch lets the compiler sink that slot's load into it,
// which then waits for every load in turn instead of keeping them all in
// flight.
template <int DT, int OP, int P>
__device__ __forceinline__ u32x4 fold_vec(const u32x4 (&x)[P], int nr) {
    u32x4 out;
    if constexpr (DT == kBF16) {
        float acc[8];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            acc[2 * i] = bf16_lo(x[0][i]);
            acc[2 * i + 1] = bf16_hi(x[0][i]);
        }
#pragma unroll
        for (int r = 1; r < P; r++) {
            const bool live = r < nr;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float lo = combine<OP>(acc[2 * i], bf16_lo(x[r][i]));
                const float hi = combine<OP>(acc[2 * i + 1], bf16_hi(x[r][i]));
                acc[2 * i] = live ? lo : acc[2 * i];
                acc[2 * i + 1] = live ? hi : acc[2 * i + 1];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) out[i] = pack_bf16(finish<OP>(acc[2 * i], nr), finish<OP>(acc[2 * i + 1], nr));
    } else if constexpr (DT == kF32) {
        float acc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) acc[i] = __uint_as_float(x[0][i]);
#pragma unroll
        for (int r = 1; r < P; r++) {
            const bool live = r < nr;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const float c = combine<OP>(acc[i], __uint_as_float(x[r][i]));
                acc[i] = live ? c : acc[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) out[i] = __float_as_uint(finish<OP>(acc[i], nr));
    } else {
        int32_t acc[4];
#pragma unroll
        for (int i = 0; i < 4; i++) acc[i] = int32_t(x[0][i]);
#pragma unroll
        for (int r = 1; r < P; r++) {
            const bool live = r < nr;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int32_t c = combine<OP>(acc[i], int32_t(x[r][i]));
                acc[i] = live ? c : acc[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 4; i++) out[i] = uint32_t(finish<OP>(acc[i], nr));
    }
    return out;
}

// One element: fold element e of the P rank buffers (element-wise path),
// returned as the result's bit pattern (bf16 in the low 16 bits).  P is a
// compile-time count, so the P loads unroll and all go out before the fold
// (with a run-time count the loop folded as it loaded and waited for each
// load in turn).
template <int DT, int OP, int P>
__device__ __forceinline__ uint32_t fold_elem_bits(const void* const* src, size_t e) {
    uint32_t w[P];
#pragma unroll
    for (int r = 0; r < P; r++) {
        if constexpr (DT == kBF16) w[r] = static_cast<const uint16_t*>(src[r])[e];
        else w[r] = static_cast<const uint32_t*>(src[r])[e];
    }
    if constexpr (DT == kI32) {
        int32_t acc = int32_t(w[0]);
#pragma unroll
        for (int r = 1; r < P; r++) acc = combine<OP>(acc, int32_t(w[r]));
        return uint32_t(finish<OP>(acc, P));
    } else if constexpr (DT == kF32) {
        float acc = __uint_as_float(w[0]);
#pragma unroll
        for (int r = 1; r < P; r++) acc = combine<OP>(acc, __uint_as_float(w[r]));
        return __float_as_uint(finish<OP>(acc, P));
    } else {
        float acc = bf16_at(uint16_t(w[0]));
#pragma unroll
        for (int r = 1; r < P; r++) acc = combine<OP>(acc, bf16_at(uint16_t(w[r])));
        return to_bf16(finish<OP>(acc, P));
    }
}
// Element de of dst takes the bits of one element.
template <int DT>
__device__ __forceinline__ void store_elem(void* dst, size_t de, uint32_t bits) {
    if constexpr (DT == kBF16) static_cast<uint16_t*>(dst)[de] = uint16_t(bits);
    else static_cast<uint32_t*>(dst)[de] = bits;
}
template <int DT, int OP, int P>
__device__ __forceinline__ void fold_elem(const void* const* src, size_t e, void* dst, size_t de) {
    store_elem<DT>(dst, de, fold_elem_bits<DT, OP, P>(src, e));
}

}  // namespace dt

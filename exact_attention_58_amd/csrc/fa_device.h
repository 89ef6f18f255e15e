// fa_device.h -- device helpers shared by the forward and backward kernels (gfx950):
// vector types, MFMA wrappers for the 16-bit types, LDS access helpers, workgroup order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.693147180559945309417f;
// Workgroups are dispatched round-robin over the 8 XCDs. Renumber them so that
// consecutive logical tiles (the query tiles of one head) run on the same XCD and
// share its L2 for K and V.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int kXcds = 8;
    const int per = total / kXcds, rem = total % kXcds;
    const int x = bid % kXcds, slot = bid / kXcds;
    return x * per + (x < rem ? x : rem) + slot;
}

// Workgroup bid of a grid of n_pairs x n_tiles workgroups -> (pair, tile), every XCD owning
// a contiguous run of pairs (workgroups are dealt to the XCDs in turn). Pair-major inside an
// XCD by default: consecutive workgroups share one pair's K and V in the XCD's L2. With
// tile_major, and when the pairs split evenly over the XCDs, the XCD's pairs go in groups of
// G, tile-major inside a group: in causal grids tile t has the same work in every pair, so
// when tile 0 is the heaviest the heavy tiles of a group start together and the next
// group's heavy tiles fill in behind the light ones (longest job first), where pair-major
// order would start the heavy tiles of the XCD's last pairs after everything else. G starts
// as the smallest group whose tiles fill the `slots` workgroups an XCD holds at once (a
// larger G balances no better and only spreads the XCD's L2 over more pairs' K and V), and is
// then evened out over the groups that take: 4 pairs with a smallest group of 3 run as one
// group of 4, not 3 + 1, whose lone last pair would run its heavy tiles at the end (causal
// bf16 B2 H16 N2048 d64: 39.5 -> 32.5 us, B8 H16 N1536 d128: 118-127 -> 103-110 us). The last
// group may still be smaller.
struct PairTile {
    int pair, tile;
};
__device__ inline PairTile xcd_pair_tile(int bid, int total, int n_tiles, int n_pairs, bool tile_major,
                                         int slots) {
    constexpr int kXcds = 8;
    if (tile_major && n_pairs % kXcds == 0) {
        const int per = n_pairs / kXcds;
        const int x = bid % kXcds, slot = bid / kXcds;
        const int g0 = min(per, (slots + n_tiles - 1) / n_tiles);
        const int g = (per + per / g0 - 1) / (per / g0);  // per / g0 groups of equal size
        const int full = per / g;                 // groups of g pairs
        int grp = slot / (g * n_tiles);
        const int gs = grp < full ? g : per - full * g;  // pairs in this group
        grp = min(grp, full);
        const int r = slot - grp * g * n_tiles;
        const int t = r / gs;
        return {x * per + grp * g + (r - t * gs), t};
    }
    const int wg = xcd_remap(bid, total);
    const int p = wg / n_tiles;
    return {p, wg - p * n_tiles};
}

// (NaN-propagating maximum / minimum: no canonicalising copies; equal to fmaxf / fminf on
// scores and -inf)
__device__ inline float wave_half_max(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_maximum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float wave_half_min(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __builtin_elementwise_minimum(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float wave_half_sum(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E), fully unrolled.
template <int B, int E, typename F>
__device__ __attribute__((always_inline)) inline void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------- 16-bit types

template <typename T> struct Half;
template <> struct Half<__bf16> {
    static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    static __device__ inline unsigned pack2(float a, float b) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return __builtin_bit_cast(unsigned, v);
    }
    static __device__ inline uint16_t one(float a) { return __builtin_bit_cast(uint16_t, (__bf16)a); }
    // the two values of a packed pair as fp32 (exact)
    static __device__ inline float lo(unsigned u) { return __uint_as_float(u << 16); }
    static __device__ inline float hi(unsigned u) { return __uint_as_float(u & 0xffff0000u); }
};
template <> struct Half<_Float16> {
    static __device__ inline f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ inline unsigned pack2(float a, float b) {
        typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
        f16x2 v = {(_Float16)a, (_Float16)b};
        return __builtin_bit_cast(unsigned, v);
    }
    static __device__ inline uint16_t one(float a) { return __builtin_bit_cast(uint16_t, (_Float16)a); }
    static __device__ inline float lo(unsigned u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu)); }
    static __device__ inline float hi(unsigned u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }
};

__device__ inline u32x2 lds_read_tr16(const uint16_t* p) {
    i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
    return __builtin_bit_cast(u32x2, t);
}

// LDS reads issued through inline asm, for kernels that also fill LDS with direct HBM->LDS
// loads: the compiler cannot prove that a read does not alias an in-flight load and would
// otherwise wait for every outstanding load before each LDS read. The kernel's own barrier
// schedule guarantees that the buffers read are not being written, and the reads' completion
// is awaited explicitly (lgkm_wait) with a count known at compile time.
template <int OFF>
__device__ inline u32x4 lds_rd128(unsigned addr) {
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
template <int OFF>
__device__ inline u32x2 lds_rdtr16(unsigned addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
// Waits until at most N LDS/scalar-memory operations are outstanding; tied to `x` so that
// the consumer of x cannot be scheduled above the wait.
template <int N>
__device__ inline void lgkm_wait(u32x4& x) {
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "n"(N));
}
// Workgroup barrier without the memory fence __syncthreads() adds: that fence waits for every
// outstanding HBM->LDS load of the issuing wave. Kernels using it order LDS traffic
// themselves: loads are awaited with an explicit s_waitcnt vmcnt(0) one phase later, and LDS
// reads are awaited before their results are used.
__device__ inline void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }
__device__ inline unsigned lds_addr(const void* p) {
    return (unsigned)(uintptr_t)(const FA_LDS void*)(p);
}

// Raw buffer resource over the `nbytes` bytes at p (clamped to [0, 2^31 - 1]): loads through
// it at byte offsets past nbytes return zeros without touching memory (the buffer range
// check), so a tile that runs past the end of a tensor needs no per-chunk branch. Word 3 is
// the gfx9-family format (32-bit data, no swizzle); p, nbytes must be wave-uniform.
__device__ inline __amdgpu_buffer_rsrc_t buffer_rsrc(const void* p, int64_t nbytes) {
    const int n = nbytes <= 0 ? 0 : nbytes > 0x7fffffff ? 0x7fffffff : (int)nbytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, n, 0x00020000);
}
// An offset past any range buffer_rsrc makes: its loads return zeros.
constexpr unsigned kBufferVoid = 0x80000000u;
// 16 bytes at byte offset `off` of a buffer resource (zeros past its range).
__device__ inline u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One 16-byte chunk (8 elements) of row `row`, columns [col, col+8), zero outside
// [0, nrows) x [0, ncols). VEC: rows are 16-byte aligned and ncols % 8 == 0.
template <bool VEC>
__device__ inline u32x4 load_chunk16(const uint16_t* base, int row, int col, int nrows, int ncols) {
    u32x4 r = {0u, 0u, 0u, 0u};
    if (row >= nrows) return r;
    const uint16_t* p = base + (int64_t)row * ncols + col;
    if (VEC) {
        if (col < ncols) r = *(const u32x4*)p;
    } else {
        uint16_t e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = (col + i < ncols) ? p[i] : (uint16_t)0;
        r[0] = e[0] | ((unsigned)e[1] << 16);
        r[1] = e[2] | ((unsigned)e[3] << 16);
        r[2] = e[4] | ((unsigned)e[5] << 16);
        r[3] = e[6] | ((unsigned)e[7] << 16);
    }
    return r;
}

// One 16-byte chunk (4 floats) of row `row`, columns [col, col+4), zero outside
// [0, nrows) x [0, ncols). VEC: rows are 16-byte aligned and ncols % 4 == 0.
template <bool VEC>
__device__ inline f32x4 load_chunk32(const float* base, int row, int col, int nrows, int ncols) {
    f32x4 r = {0.f, 0.f, 0.f, 0.f};
    if (row >= nrows) return r;
    const float* p = base + (int64_t)row * ncols + col;
    if (VEC) {
        if (col < ncols) r = *(const f32x4*)p;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) r[i] = (col + i < ncols) ? p[i] : 0.0f;
    }
    return r;
}

}  // namespace fa

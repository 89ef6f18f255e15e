// fa_fwd_kernels.hip -- exact attention forward kernels for gfx950 (MI355X, CDNA4).
//
// The method (page "flash_attention_2.cu", forward kernel): for a block of query
// rows, walk the key/value tiles keeping a running row max m, a running row sum l
// and an output accumulator O; for each tile compute the scores, the new max,
// P = exp(S - m), rescale l and O by exp(m_old - m_new), add rowsum(P) and P.V;
// at the end O /= l and L = m + ln(l). The loop order follows the "swapped" order
// discussed on page "parallel execution of read/write operations (paper vs
// implementation)": one workgroup owns its query rows for the whole key loop, so
// O starts at zero in registers and is written once. The grid covers (query
// tile, head, batch), the query-parallel forward of page "Meta's xFormers has
// Attention kernel written in CUTLASS".
//
// gfx950 mapping (one wave = 64 lanes owns 32 query rows):
//  * S^T = K Q^T on MFMA 32x32x16 (16-bit) or 32x32x2 (fp32). With keys as the
//    MFMA rows and queries as the columns, each lane holds one query (column
//    lane%32) and 16 keys per 32-key block, so the row max and row sum are
//    lane-local plus one v_permlane32_swap between the two lane halves.
//  * The S^T accumulator is, register for register, the B operand of the next
//    product O^T = V^T P^T once the keys of the reduction are enumerated in the
//    accumulator's order (any order of the keys gives the same sum). V^T is read
//    from LDS with ds_read_b64_tr_b16, which hands each lane 4 consecutive keys
//    of one head-dim column.
//  * The online softmax uses exp2 with the scale folded into log2(e) (page "Add
//    Fused Multi-Head Attention example"); P is rounded to the input type for
//    the PV product while l sums the fp32 P.
//  * K/V tiles are loaded from HBM with 16-byte coalesced loads into registers
//    one tile ahead of their use and stored to LDS behind a barrier.
//  * Keys past Nk are zero in LDS and masked to -inf; the causal mask keeps key
//    j for query i iff j <= i; tiles wholly above the diagonal are skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_internal.h"

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
// Running-max refresh threshold in log2 units: O and l are rescaled only when a
// row's max grows by more than this, otherwise the old max stays the reference.
// The result is unchanged (numerator and denominator share the reference) and
// the unnormalised weights stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;

// Workgroups are dispatched round-robin over the 8 XCDs. Renumber them so that
// consecutive logical tiles (the query tiles of one head) run on the same XCD and
// share its L2 for K and V.
__device__ inline int xcd_remap(int bid, int total) {
    constexpr int kXcds = 8;
    const int per = total / kXcds, rem = total % kXcds;
    const int x = bid % kXcds, slot = bid / kXcds;
    return x * per + (x < rem ? x : rem) + slot;
}

__device__ inline float wave_half_max(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float wave_half_min(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fminf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}
__device__ inline float wave_half_sum(float x) {
    u32x2 s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
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
};

__device__ inline u32x2 lds_read_tr16(const uint16_t* p) {
    i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS i16x4*)(p));
    return __builtin_bit_cast(u32x2, t);
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

// 16-bit forward kernel. DP: padded head dim (32, 64, 96, 128). Workgroup = 4 waves
// = 128 query rows; K/V tiles of 64 keys.
template <typename T, int DP, bool CAUSAL, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd16_kernel(FwdArgs a, int n_qtiles) {
    constexpr int NW = 4, BR = 32 * NW, BC = 64;
    constexpr int KST = DP + 8;   // K row stride (elements): 16-byte pad, conflict-free b128 reads
    constexpr int VST = DP + 16;  // V row stride: 32-byte pad, conflict-free transposed reads
    constexpr int CPR = DP / 8;   // 16-byte chunks per row
    constexpr int CH = BC * CPR / (64 * NW);  // chunks per thread per tile
    static_assert(BC * CPR % (64 * NW) == 0, "tile load split");
    constexpr int NDS = DP / 16;  // k-steps of the QK^T product
    constexpr int NDB = DP / 32;  // 32-wide head-dim blocks of O^T

    __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * KST];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[BC * VST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = wg / n_qtiles;
    int qt = wg - bh * n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int q0 = qt * BR;
    const int r0w = q0 + wave * 32;
    const int myq = r0w + l32;

    const uint16_t* qg = (const uint16_t*)a.q + (int64_t)bh * Nq * d;
    const uint16_t* kg = (const uint16_t*)a.k + (int64_t)bh * Nk * d;
    const uint16_t* vg = (const uint16_t*)a.v + (int64_t)bh * Nk * d;

    // Q fragments (B operand of S^T = K Q^T): lane holds Q[myq][16*ds + 8*h32 + 0..7]
    u32x4 qf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = load_chunk16<VEC>(qg, myq, ds * 16 + 8 * h32, Nq, d);

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;

    u32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int chunk = tid + c * 64 * NW;
            const int row = chunk / CPR, col = (chunk % CPR) * 8;
            kreg[c] = load_chunk16<VEC>(kg, j * BC + row, col, Nk, d);
            vreg[c] = load_chunk16<VEC>(vg, j * BC + row, col, Nk, d);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int chunk = tid + c * 64 * NW;
            const int row = chunk / CPR, col = (chunk % CPR) * 8;
            *(u32x4*)(Ks + row * KST + col) = kreg[c];
            *(u32x4*)(Vs + row * VST + col) = vreg[c];
        }
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float c = a.scale_log2;

    load_tile(0);
    for (int j = 0; j < n_tiles; ++j) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (j + 1 < n_tiles) load_tile(j + 1);

        const int k0 = j * BC;
        if (CAUSAL && k0 > r0w + 31) continue;  // every key of the tile is above this wave's rows

        // ---- S^T = K Q^T: two 32-key blocks
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            s[kb] = f32x16{};
            const uint16_t* kp = Ks + (kb * 32 + l32) * KST + 8 * h32;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s[kb] = Half<T>::mfma(*(const u32x4*)(kp + ds * 16), qf[ds], s[kb]);
        }

        // ---- masks and tile max (log2 units)
        const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > r0w);
        float mt;
        if (masked) {
            mt = kNegInf;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                    const bool ok = key < Nk && (!CAUSAL || key <= myq);
                    const float t = ok ? s[kb][r] * c : kNegInf;
                    s[kb][r] = t;
                    mt = fmaxf(mt, t);
                }
            mt = wave_half_max(mt);
        } else {
            float mx = s[0][0];
            if (c >= 0.0f) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mx = wave_half_max(mx);
            } else {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fminf(mx, s[kb][r]);
                mx = wave_half_min(mx);
            }
            mt = mx * c;
        }

        // ---- lazy rescale of the running state
        const float m_cand = fmaxf(m_run, mt);
        if (__any(m_cand > m_run + kRescaleThreshold)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
            m_run = m_cand;
        }

        // ---- P = exp2(S*c - m), row sum, 16-bit pack
        unsigned pk[2][8];
        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                float p0, p1;
                if (masked) {
                    p0 = __builtin_amdgcn_exp2f(s[kb][r] - m_run);
                    p1 = __builtin_amdgcn_exp2f(s[kb][r + 1] - m_run);
                } else {
                    p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_run));
                    p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], c, -m_run));
                }
                lsum += p0 + p1;
                pk[kb][r >> 1] = Half<T>::pack2(p0, p1);
            }
        l_run += lsum;

        // ---- O^T += V^T P^T: 4 k-steps of 16 keys
        const int i16 = lane & 15, g16 = (lane >> 4) & 1;
#pragma unroll
        for (int t = 0; t < BC / 16; ++t) {
            const u32x4 pb = {pk[t >> 1][4 * (t & 1) + 0], pk[t >> 1][4 * (t & 1) + 1],
                              pk[t >> 1][4 * (t & 1) + 2], pk[t >> 1][4 * (t & 1) + 3]};
            const int rowa = t * 16 + 4 * h32 + (i16 >> 2);
            const uint16_t* vp = Vs + rowa * VST + 16 * g16 + 4 * (i16 & 3);
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x2 lo = lds_read_tr16(vp + db * 32);
                const u32x2 hi = lds_read_tr16(vp + 8 * VST + db * 32);
                const u32x4 va = {lo[0], lo[1], hi[0], hi[1]};
                oacc[db] = Half<T>::mfma(va, pb, oacc[db]);
            }
        }
    }

    // ---- epilogue: O = O / l, L = (m + log2 l) ln 2
    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < Nq) {
        uint16_t* og = (uint16_t*)a.o + ((int64_t)bh * Nq + myq) * d;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * h32;
                const float o0 = oacc[db][4 * g + 0] * inv, o1 = oacc[db][4 * g + 1] * inv;
                const float o2 = oacc[db][4 * g + 2] * inv, o3 = oacc[db][4 * g + 3] * inv;
                if (VEC) {
                    if (d0 < d) {
                        u32x2 w = {Half<T>::pack2(o0, o1), Half<T>::pack2(o2, o3)};
                        *(u32x2*)(og + d0) = w;
                    }
                } else {
                    if (d0 + 0 < d) og[d0 + 0] = Half<T>::one(o0);
                    if (d0 + 1 < d) og[d0 + 1] = Half<T>::one(o1);
                    if (d0 + 2 < d) og[d0 + 2] = Half<T>::one(o2);
                    if (d0 + 3 < d) og[d0 + 3] = Half<T>::one(o3);
                }
            }
        if (h32 == 0) a.lse[(int64_t)bh * Nq + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- fp32

// One 16-byte chunk (4 floats) of row `row`, columns [col, col+4), zero outside.
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

// fp32 forward kernel on v_mfma_f32_32x32x2_f32. The head-dim reduction of S^T is
// enumerated as d = h32*(DP/2) + ds so each lane loads half a contiguous row of Q
// and of K. P stays fp32 for the PV product.
template <int DP, int BC, bool CAUSAL, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd32_kernel(FwdArgs a, int n_qtiles) {
    constexpr int NW = 4, BR = 32 * NW;
    constexpr int KST = DP + 4;  // floats; 16-byte pad
    constexpr int VST = DP;      // floats
    constexpr int CPR = DP / 4;
    constexpr int CH = BC * CPR / (64 * NW);
    static_assert(BC * CPR % (64 * NW) == 0, "tile load split");
    constexpr int HALF = DP / 2;
    constexpr int NKB = BC / 32;
    constexpr int NDB = DP / 32;

    __shared__ __attribute__((aligned(16))) float Ks[BC * KST];
    __shared__ __attribute__((aligned(16))) float Vs[BC * VST];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;

    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int bh = wg / n_qtiles;
    int qt = wg - bh * n_qtiles;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int q0 = qt * BR;
    const int r0w = q0 + wave * 32;
    const int myq = r0w + l32;

    const float* qg = (const float*)a.q + (int64_t)bh * Nq * d;
    const float* kg = (const float*)a.k + (int64_t)bh * Nk * d;
    const float* vg = (const float*)a.v + (int64_t)bh * Nk * d;

    // Q: lane holds Q[myq][h32*HALF + 0..HALF-1]
    float qf[HALF];
#pragma unroll
    for (int c4 = 0; c4 < HALF / 4; ++c4) {
        const f32x4 t = load_chunk32<VEC>(qg, myq, h32 * HALF + 4 * c4, Nq, d);
        qf[4 * c4 + 0] = t[0];
        qf[4 * c4 + 1] = t[1];
        qf[4 * c4 + 2] = t[2];
        qf[4 * c4 + 3] = t[3];
    }

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;

    f32x4 kreg[CH], vreg[CH];
    auto load_tile = [&](int j) {
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
            const int chunk = tid + cc * 64 * NW;
            const int row = chunk / CPR, col = (chunk % CPR) * 4;
            kreg[cc] = load_chunk32<VEC>(kg, j * BC + row, col, Nk, d);
            vreg[cc] = load_chunk32<VEC>(vg, j * BC + row, col, Nk, d);
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
            const int chunk = tid + cc * 64 * NW;
            const int row = chunk / CPR, col = (chunk % CPR) * 4;
            *(f32x4*)(Ks + row * KST + col) = kreg[cc];
            *(f32x4*)(Vs + row * VST + col) = vreg[cc];
        }
    };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float c = a.scale_log2;

    load_tile(0);
    for (int j = 0; j < n_tiles; ++j) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (j + 1 < n_tiles) load_tile(j + 1);

        const int k0 = j * BC;
        if (CAUSAL && k0 > r0w + 31) continue;

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
            const float* kp = Ks + (kb * 32 + l32) * KST + h32 * HALF;
#pragma unroll
            for (int c4 = 0; c4 < HALF / 4; ++c4) {
                const f32x4 kv = *(const f32x4*)(kp + 4 * c4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[4 * c4 + e], s[kb], 0, 0, 0);
            }
        }

        const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > r0w);
        float mt;
        if (masked) {
            mt = kNegInf;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                    const bool ok = key < Nk && (!CAUSAL || key <= myq);
                    const float t = ok ? s[kb][r] * c : kNegInf;
                    s[kb][r] = t;
                    mt = fmaxf(mt, t);
                }
            mt = wave_half_max(mt);
        } else {
            float mx = s[0][0];
            if (c >= 0.0f) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
                mx = wave_half_max(mx);
            } else {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fminf(mx, s[kb][r]);
                mx = wave_half_min(mx);
            }
            mt = mx * c;
        }

        const float m_cand = fmaxf(m_run, mt);
        if (__any(m_cand > m_run + kRescaleThreshold)) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
            l_run *= alpha;
#pragma unroll
            for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
            m_run = m_cand;
        }

        float lsum = 0.0f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const float p = masked ? __builtin_amdgcn_exp2f(s[kb][r] - m_run)
                                       : __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -m_run));
                s[kb][r] = p;
                lsum += p;
            }
        l_run += lsum;

        // O^T += V^T P^T, one key per lane half per MFMA: k-step r of block kb is
        // key kb*32 + 8*(r/4) + 4*h32 + r%4, the key the lane's S^T register r holds.
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                const float* vp = Vs + key * VST + l32;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[db * 32], s[kb][r], oacc[db], 0, 0, 0);
            }
    }

    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < Nq) {
        float* og = (float*)a.o + ((int64_t)bh * Nq + myq) * d;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * h32;
                const f32x4 w = {oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv,
                                 oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv};
                if (VEC) {
                    if (d0 < d) *(f32x4*)(og + d0) = w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < d) og[d0 + e] = w[e];
                }
            }
        if (h32 == 0) a.lse[(int64_t)bh * Nq + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- launch

template <typename K>
static int launch(K kernel, const FwdArgs& a, int br, hipStream_t st) {
    const int n_qtiles = (a.Nq + br - 1) / br;
    const int64_t total = (int64_t)n_qtiles * a.B * a.H;
    hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(256), 0, st, a, n_qtiles);
    return (int)hipGetLastError();
}

template <typename T, int DP>
static int launch16(const FwdArgs& a, bool vec, hipStream_t st) {
    if (a.causal) {
        return vec ? launch(fwd16_kernel<T, DP, true, true>, a, 128, st)
                   : launch(fwd16_kernel<T, DP, true, false>, a, 128, st);
    }
    return vec ? launch(fwd16_kernel<T, DP, false, true>, a, 128, st)
               : launch(fwd16_kernel<T, DP, false, false>, a, 128, st);
}

template <int DP, int BC>
static int launch32(const FwdArgs& a, bool vec, hipStream_t st) {
    if (a.causal) {
        return vec ? launch(fwd32_kernel<DP, BC, true, true>, a, 128, st)
                   : launch(fwd32_kernel<DP, BC, true, false>, a, 128, st);
    }
    return vec ? launch(fwd32_kernel<DP, BC, false, true>, a, 128, st)
               : launch(fwd32_kernel<DP, BC, false, false>, a, 128, st);
}

int launch_fwd(const FwdArgs& a, const TileConfig& cfg, bool vec, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.dtype == 2 || a.dtype == 1) {
        const bool bf = a.dtype == 2;
        switch (cfg.dpad) {
            case 32: return bf ? launch16<__bf16, 32>(a, vec, st) : launch16<_Float16, 32>(a, vec, st);
            case 64: return bf ? launch16<__bf16, 64>(a, vec, st) : launch16<_Float16, 64>(a, vec, st);
            case 96: return bf ? launch16<__bf16, 96>(a, vec, st) : launch16<_Float16, 96>(a, vec, st);
            case 128: return bf ? launch16<__bf16, 128>(a, vec, st) : launch16<_Float16, 128>(a, vec, st);
            default: return (int)hipErrorInvalidValue;
        }
    }
    switch (cfg.dpad) {
        case 32: return launch32<32, 64>(a, vec, st);
        case 64: return launch32<64, 64>(a, vec, st);
        case 96: return launch32<96, 64>(a, vec, st);
        case 128: return launch32<128, 32>(a, vec, st);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fa

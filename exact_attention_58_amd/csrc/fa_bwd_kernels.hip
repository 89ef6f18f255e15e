// fa_bwd_kernels.hip -- exact attention backward kernels for gfx950 (MI355X, CDNA4).
//
// The gradients (page "flash_attention_2.cu", backward kernel): with D_i = rowsum(dO_i * O_i)
// and P_ij = exp(scale * q_i . k_j - L_i) recomputed from the forward's logsumexp L,
//     dV_j += P_ij dO_i,   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i),
//     dQ_i += scale dS_ij k_j,   dK_j += scale dS_ij q_i.
// That page accumulates dQ with atomic adds from a loop over key tiles; here three kernels
// share the work without atomics:
//  * row terms: D = rowsum(dO * O) per query row (fp32, into a caller's workspace);
//  * dK, dV: looping over query tiles of 128 (d <= 64) or 64; up to d = 96 one workgroup per
//    256 keys (8 waves x 32 keys) or, on small grids, 128 keys (4 waves); above, one per 128
//    keys (8 waves in two roles that split each 32-key block's products);
//  * dQ: one workgroup per 256 queries (8 waves x 32) or, on small grids, 128 (4 waves),
//    looping over key tiles of 128 (d <= 64, and d <= 96 with 8 waves) or 64.
// Both tile kernels recompute S and dP on MFMA 32x32x16 (16-bit operands, fp32 accumulate);
// P and dS are rounded to the input type for the products that consume them.
//
// Layouts, per wave (lane = 32 * h32 + l32):
//  * dK/dV kernel: S = Q K^T and dP = dO V^T with this wave's keys as the MFMA columns, so a
//    lane holds one key and 16 queries per 32-query block; the accumulator is, register for
//    register, the A operand of dV += P^T dO and dK += dS^T Q once the queries of the
//    reduction are enumerated in the accumulator's order; dO^T and Q^T come from LDS through
//    ds_read_b64_tr_b16. dK and dV accumulate as [key][head-dim] blocks.
//  * dQ kernel: S^T = K Q^T and dP^T = V dO^T with this wave's queries as the columns (the
//    forward's layout), so dS^T is the B operand of dQ^T += K^T dS^T.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr float kLog2e = 1.4426950408889634074f;
// workgroups an XCD holds at once (two waves per SIMD): 32 CUs x two 4-wave workgroups, or
// 32 CUs x one 8-wave workgroup
constexpr int kXcdSlots = 64, kXcdSlots8 = 32;

// Row terms: delta[r] = sum_c dO[r][c] O[r][c] for every flat query row r (d % 8 == 0, d <= 128).
// Sixteen lanes share a row, one 16-byte chunk each, so a wave reads four whole rows of O and
// of dO per instruction (coalesced); the sixteen partial sums meet through lane shuffles.
template <typename T>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void bwd_delta_kernel(const uint16_t* o, const uint16_t* dout, float* delta, int64_t rows, int d) {
    const int sub = threadIdx.x & 15;
    const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    float acc = 0.0f;
    if (r < rows && sub * 8 < d) {
        const u32x4 a = *(const u32x4*)(o + r * d + sub * 8);
        const u32x4 b = *(const u32x4*)(dout + r * d + sub * 8);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = __builtin_fmaf(Half<T>::lo(a[i]), Half<T>::lo(b[i]), acc);
            acc = __builtin_fmaf(Half<T>::hi(a[i]), Half<T>::hi(b[i]), acc);
        }
    }
    // every lane takes part in the shuffles, also past the last row
#pragma unroll
    for (int m = 8; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 16);
    if (r < rows && sub == 0) delta[r] = acc;
}

// One element of a row-major buffer of type E (fp32, or a 16-bit type), as fp32 (exact).
template <typename E>
__device__ inline float elem(const void* p, int64_t i) {
    if constexpr (std::is_same<E, float>::value) {
        return ((const float*)p)[i];
    } else if constexpr (std::is_same<E, __bf16>::value) {
        return __uint_as_float((unsigned)((const uint16_t*)p)[i] << 16);
    } else {
        return (float)((const _Float16*)p)[i];
    }
}

// Row terms for any element type, head dim and alignment: sixteen lanes share a row and walk
// its elements sixteen apart (each load instruction reads 16 consecutive elements of four
// rows), then meet through lane shuffles.
template <typename E>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void bwd_delta_any_kernel(const void* o, const void* dout, float* delta, int64_t rows, int d) {
    const int sub = threadIdx.x & 15;
    const int64_t r = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    float acc = 0.0f;
    if (r < rows)
        for (int c = sub; c < d; c += 16) acc = __builtin_fmaf(elem<E>(o, r * d + c), elem<E>(dout, r * d + c), acc);
#pragma unroll
    for (int m = 8; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 16);
    if (r < rows && sub == 0) delta[r] = acc;
}

// LDS layout of the 16-bit tiles (Q, dO, K, V: rows x DP). Swizzled (d = 32, 64, 128): rows of
// P 16-byte chunks, P = 4 or 12 (mod 16), and chunk c of row r at position c ^ ((r >> 2) & 3)
// of its row (the low two bits of the chunk index permuted by the row's next two bits). On 64
// banks of 4 bytes this serves both reads of a tile without conflicts: a b128 read of one
// chunk from 16 consecutive rows (16 lanes at a time: row pitch and permutation spread them
// over the 16 bank groups) and a transposed b64 read of 4 consecutive chunks from 4 rows (32
// lanes at a time: the pitch puts the 4 rows in 4 distinct groups of 4 chunks). The plain
// pitch of CPR + 1 chunks serves only the first and costs the second 2-4x its cycles; d = 96
// keeps it, since the swizzle's two extra address registers make its kernels spill.
template <int DP>
struct Tile16 {
    static constexpr bool SWZ = DP != 96;
    static constexpr int CPR = DP / 8;                                     // chunks of data per row
    static constexpr int P = !SWZ ? CPR + 1 : CPR % 8 == 0 ? CPR + 4 : CPR;  // chunks per LDS row
    static constexpr int STR = 8 * P;                                      // elements per LDS row
    static_assert(!SWZ || P % 8 == 4, "row pitch of 4 or 12 chunks mod 16");
    // element offset of chunk c of row r
    __device__ static int off(int r, int c) {
        return r * STR + 8 * (SWZ ? (c & ~3) | ((c & 3) ^ ((r >> 2) & 3)) : c);
    }
};

// Row-major operand reads of a Tile16 tile: lane (h32, l32) reads chunk 2 ds + h32 of row
// R + l32 (R % 16 == 0). Swizzled, with z = h32 ^ ((l32 >> 2) & 3), that chunk sits at
// position 4 (ds >> 1) + (z or z ^ 2 by the parity of ds): two offsets per lane, the rest
// constant.
template <int DP>
struct RowFrag {
    int o0, o1;
    __device__ explicit RowFrag(int lane) {
        const int h32 = lane >> 5, l32 = lane & 31;
        if constexpr (Tile16<DP>::SWZ) {
            o0 = l32 * Tile16<DP>::STR + 8 * (h32 ^ ((l32 >> 2) & 3));
            o1 = o0 ^ 16;  // l32 * STR is a multiple of 32 elements
        } else {
            o0 = l32 * Tile16<DP>::STR + 8 * h32;
            o1 = o0 + 16;
        }
    }
    __device__ __attribute__((always_inline)) u32x4 operator()(const uint16_t* tile, int R, int ds) const {
        return *(const u32x4*)(tile + (ds & 1 ? o1 : o0) + R * Tile16<DP>::STR + 32 * (ds >> 1));
    }
};

// Tile of ROWS rows x DP columns (16-bit) staged by NT threads through registers into LDS in
// the Tile16 layout; rows >= nrows and columns >= d are zero. VEC: 16-byte rows (d % 8 == 0,
// aligned). Each wave moves a contiguous run of CH x 64 chunks, one 1 KB instruction after
// another (0-2% faster than every wave taking every (NT/64)-th KB; the same bits).
template <int DP, bool VEC, int NT = 256, int ROWS = 64>
struct TileCopy {
    static constexpr int CPR = DP / 8;                // 16-byte chunks per row
    static constexpr int CH = (ROWS * CPR + NT - 1) / NT;  // chunks per thread (the last maybe partial)
    u32x4 r[CH];
    // VEC: byte offset of this thread's chunk within a tile, or an offset past any buffer
    // (a chunk past d, or a thread without a chunk) that the load's range check turns into 0
    unsigned voff[CH];
    __device__ __attribute__((always_inline)) void init(int d, int tid) {
        if constexpr (VEC) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 8;
                const bool ok = (ROWS * CPR % NT == 0 || chunk < ROWS * CPR) && col < d;
                voff[c] = ok ? (unsigned)(row * d + col) * 2u : kBufferVoid;
            }
        }
    }
    // VEC: buffer loads over rows [row0, nrows) of the tensor, so rows past nrows read as
    // zeros by the hardware's range check, without a branch per chunk
    __device__ __attribute__((always_inline)) void load(const uint16_t* base, int row0, int nrows, int d, int tid) {
        if constexpr (VEC) {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base + (int64_t)row0 * d, (int64_t)(nrows - row0) * d * 2);
#pragma unroll
            for (int c = 0; c < CH; ++c) r[c] = buffer_load16(rs, voff[c]);
        } else {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 8;
                if (ROWS * CPR % NT == 0 || chunk < ROWS * CPR) r[c] = load_chunk16<VEC>(base, row0 + row, col, nrows, d);
            }
        }
    }
    __device__ __attribute__((always_inline)) void store(uint16_t* lds, int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
            const int row = chunk / CPR;
            if (ROWS * CPR % NT == 0 || chunk < ROWS * CPR) *(u32x4*)(lds + Tile16<DP>::off(row, chunk % CPR)) = r[c];
        }
    }
};

// Transposed fragment of a Tile16 tile (rows = reduction index): lane gets rows
// R + 4 h32 + {0..3} and R + 8 + 4 h32 + {0..3} of column C + 16 g16 + i16, the B (or A)
// operand of a 32x32x16 product whose reduction runs over 16 rows in accumulator order
// (R % 16 == 0, C % 32 == 0). Each lane reads 4 elements of chunk C/8 + y, y = 2 g16 +
// (i16 & 3) / 2, whose position in the first row group is y ^ h32 ((row >> 2) & 3 = h32) and
// in the second y ^ h32 ^ 2.
template <int DP>
__device__ __attribute__((always_inline)) inline u32x4 tr_frag(const uint16_t* tile, int R, int C, int lane) {
    constexpr int STR = Tile16<DP>::STR;
    const int h32 = lane >> 5, i16 = lane & 15, g16 = (lane >> 4) & 1;
    const int row = R + 4 * h32 + (i16 >> 2);
    const int y = 2 * g16 + ((i16 & 3) >> 1), e = 4 * (i16 & 1);
    const int k = Tile16<DP>::SWZ ? h32 : 0;
    const u32x2 lo = lds_read_tr16(tile + row * STR + C + 8 * (y ^ k) + e);
    const u32x2 hi = lds_read_tr16(tile + (row + 8) * STR + C + 8 * (Tile16<DP>::SWZ ? y ^ k ^ 2 : y) + e);
    return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// ---------------------------------------------------------------- dK, dV

// dK and dV together for d <= 96, NW waves of 32 keys, two per SIMD: one wave's LDS reads and
// staged loads then overlap the other's products, about 1.5x the throughput of one wave per
// SIMD.
template <typename T, int DP, bool CAUSAL, bool VEC, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_kernel(BwdArgs a, int n_ktiles) {
    static_assert(DP <= 96, "above d = 96: bwd_dkdv_pair_kernel");
    // keys per workgroup, queries per tile (128 where the registers allow: half the barriers)
    constexpr int BK = 32 * NW, BQ = DP <= 64 ? 128 : 64;
    constexpr int STR = Tile16<DP>::STR;
    constexpr int NDS = DP / 16, NDB = DP / 32;
    __shared__ __attribute__((aligned(16))) uint16_t Qs[BQ * STR];
    __shared__ __attribute__((aligned(16))) uint16_t Gs[BQ * STR];  // dO
    __shared__ __attribute__((aligned(16))) float Ls[BQ];
    __shared__ __attribute__((aligned(16))) float Ds[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    // causal: key tile 0 sees every query tile, the heaviest; tile-major dispatch per XCD
    const PairTile pt = xcd_pair_tile(blockIdx.x, gridDim.x, n_ktiles, a.B * a.H, CAUSAL, NW == 8 ? kXcdSlots8 : kXcdSlots);
    const int bh = pt.pair, kt = pt.tile;
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * wave;
    const int mykey = kw0 + l32;

    const uint16_t* qg = (const uint16_t*)a.q + (int64_t)bh * Nq * d;
    const uint16_t* kg = (const uint16_t*)a.k + (int64_t)bh * Nk * d;
    const uint16_t* vg = (const uint16_t*)a.v + (int64_t)bh * Nk * d;
    const uint16_t* gg = (const uint16_t*)a.dout + (int64_t)bh * Nq * d;
    const float* lg = a.lse + (int64_t)bh * Nq;
    const float* dg = a.delta + (int64_t)bh * Nq;

    // this wave's keys as B operands: lane holds K[mykey][16 ds + 8 h32 + 0..7] (V likewise)
    u32x4 kf[NDS], vf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        kf[ds] = load_chunk16<VEC>(kg, mykey, ds * 16 + 8 * h32, Nk, d);
        vf[ds] = load_chunk16<VEC>(vg, mykey, ds * 16 + 8 * h32, Nk, d);
    }

    f32x16 dva[NDB], dka[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dva[i] = dka[i] = f32x16{};
    const float c = a.scale_log2;

    // query tiles that see any key of this workgroup (causal: queries >= k0)
    const int qt0 = CAUSAL ? k0 / BQ : 0;
    const int n_qt = (Nq + BQ - 1) / BQ;
    TileCopy<DP, VEC, 64 * NW, BQ> qc, gc;
    qc.init(d, tid);
    gc.init(d, tid);
    const RowFrag<DP> rf(lane);
    float lrow = 0.0f, drow = 0.0f;
    auto load_tile = [&](int qt) __attribute__((always_inline)) {
        qc.load(qg, qt * BQ, Nq, d, tid);
        gc.load(gg, qt * BQ, Nq, d, tid);
        if (tid < BQ) {
            const int q = qt * BQ + tid;
            lrow = q < Nq ? lg[q] * kLog2e : 0.0f;
            drow = q < Nq ? dg[q] : 0.0f;
        }
    };
    if (qt0 < n_qt) load_tile(qt0);
    for (int qt = qt0; qt < n_qt; ++qt) {
        __syncthreads();
        qc.store(Qs, tid);
        gc.store(Gs, tid);
        if (tid < BQ) {
            Ls[tid] = lrow;
            Ds[tid] = drow;
        }
        __syncthreads();
        if (qt + 1 < n_qt) load_tile(qt + 1);
        const int q0 = qt * BQ;
        // a causal wave skips tiles whose queries all precede its keys
        if (CAUSAL && q0 + BQ - 1 < kw0) continue;

#pragma unroll
        for (int qb = 0; qb < BQ / 32; ++qb) {
            // S = Q K^T and dP = dO V^T for 32 queries x this wave's 32 keys
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = Half<T>::mfma(rf(Qs, qb * 32, ds), kf[ds], s);
                dp = Half<T>::mfma(rf(Gs, qb * 32, ds), vf[ds], dp);
            }
            // register r: query q0 + qb*32 + 8 (r/4) + 4 h32 + r%4, key mykey. The weight is
            // kept iff off = 8 (r/4) + r%4 >= lo: lo puts the causal diagonal (q >= mykey) in
            // one compare per register and masks every query of a key past Nk. Padded query
            // rows (q >= Nq) need no test: their Q, dO, L and D are zero, so the weight
            // exp2(0) = 1 meets dO = 0 and dP - D = 0 and adds nothing.
            const int lo = mykey >= Nk ? 64 : CAUSAL ? mykey - q0 - qb * 32 - 4 * h32 : -64;
            // every weight of the block kept (all keys below Nk, all queries on or past the
            // diagonal): the wave skips the compares
            const bool full = kw0 + 32 <= Nk && (!CAUSAL || kw0 + 31 <= q0 + qb * 32);
            unsigned ppk[8], spk[8];
            auto weights = [&](auto masked_c) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int ql = qb * 32 + 8 * g + 4 * h32;
                    const f32x4 lv = *(const f32x4*)(Ls + ql);
                    const f32x4 dv = *(const f32x4*)(Ds + ql);
                    float pv[4], sv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float p = !MASKED || 8 * g + e >= lo
                                            ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c, -lv[e]))
                                            : 0.0f;
                        pv[e] = p;
                        sv[e] = p * (dp[4 * g + e] - dv[e]);
                    }
                    ppk[2 * g] = Half<T>::pack2(pv[0], pv[1]);
                    ppk[2 * g + 1] = Half<T>::pack2(pv[2], pv[3]);
                    spk[2 * g] = Half<T>::pack2(sv[0], sv[1]);
                    spk[2 * g + 1] = Half<T>::pack2(sv[2], sv[3]);
                }
            };
            // (the unmasked copy only for 16-byte rows: the element-wise instances have no
            // registers to spare for it)
            if (VEC && full) weights(std::false_type{});
            else weights(std::true_type{});
            // dV += P^T dO and dK += dS^T Q over the two 16-query steps of this block
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const u32x4 pa = {ppk[4 * t], ppk[4 * t + 1], ppk[4 * t + 2], ppk[4 * t + 3]};
                const u32x4 sa = {spk[4 * t], spk[4 * t + 1], spk[4 * t + 2], spk[4 * t + 3]};
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const u32x4 gb = tr_frag<DP>(Gs, qb * 32 + 16 * t, db * 32, lane);
                    dva[db] = Half<T>::mfma(pa, gb, dva[db]);
                    const u32x4 qbf = tr_frag<DP>(Qs, qb * 32 + 16 * t, db * 32, lane);
                    dka[db] = Half<T>::mfma(sa, qbf, dka[db]);
                }
            }
        }
    }

    // register r of block db: key kw0 + 8 (r/4) + 4 h32 + r%4, column db*32 + l32
    uint16_t* dkg = (uint16_t*)a.dk + (int64_t)bh * Nk * d;
    uint16_t* dvg = (uint16_t*)a.dv + (int64_t)bh * Nk * d;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + l32;
        if (col >= d) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            if (key < Nk) {
                dvg[(int64_t)key * d + col] = Half<T>::one(dva[db][r]);
                dkg[(int64_t)key * d + col] = Half<T>::one(dka[db][r] * sc);
            }
        }
    }
}


// dK and dV for d > 96, with the products of each 32-key block on two waves that share a
// SIMD. Wave w < KB (role A) computes S = Q K^T, P and dV += P^T dO; wave w + KB (role B)
// computes dP = dO V^T and, from the P that role A passes through LDS in fp32, dS = P (dP - D)
// and dK += dS^T Q. Each holds half the accumulators and resident key fragments of the fused
// kernel, so both fit two waves per SIMD, and S is computed once (separate dV and dK kernels
// would each compute it). The gradients are those of the fused kernel bit for bit. The query loop runs in
// steps of 32 queries; B handles step i - 1 while A handles step i, so neither waits for the
// other within a step, and a workgroup barrier ends each step. Query tiles (64 rows of Q and
// dO, with L and D) have two LDS buffers: tile t is read in steps 2t..2t+2 and tile t+2 is
// stored into the same buffer in step 2t+3; its loads are issued two steps earlier and stay
// in flight across the barriers (a plain s_barrier after an LDS-only wait).
template <typename T, int DP, bool CAUSAL, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv_pair_kernel(BwdArgs a, int n_ktiles) {
    constexpr int KB = 4;  // key blocks of 32 per workgroup (one per SIMD)
    constexpr int NT = 128 * KB;
    constexpr int BK = 32 * KB, BQ = 64;
    constexpr int STR = Tile16<DP>::STR;
    constexpr int NDS = DP / 16, NDB = DP / 32;
    __shared__ __attribute__((aligned(16))) uint16_t Qsb[2][BQ * STR];
    __shared__ __attribute__((aligned(16))) uint16_t Gsb[2][BQ * STR];  // dO
    __shared__ __attribute__((aligned(16))) float Lsb[2][BQ];
    __shared__ __attribute__((aligned(16))) float Dsb[2][BQ];
    // P of one step per key block, [buffer][key block][register group][lane]: lane-contiguous
    // 16-byte rows, so the writes and reads of a register group are conflict-free
    __shared__ __attribute__((aligned(16))) f32x4 Pb[2][KB][4][64];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    const int kbk = wave % KB;
    // one workgroup per CU: an XCD holds 32 at once
    const PairTile pt = xcd_pair_tile(blockIdx.x, gridDim.x, n_ktiles, a.B * a.H, CAUSAL, kXcdSlots8);
    const int bh = pt.pair, kt = pt.tile;
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * kbk;
    const int mykey = kw0 + l32;

    const uint16_t* qg = (const uint16_t*)a.q + (int64_t)bh * Nq * d;
    const uint16_t* kg = (const uint16_t*)a.k + (int64_t)bh * Nk * d;
    const uint16_t* vg = (const uint16_t*)a.v + (int64_t)bh * Nk * d;
    const uint16_t* gg = (const uint16_t*)a.dout + (int64_t)bh * Nq * d;
    const float* lg = a.lse + (int64_t)bh * Nq;
    const float* dg = a.delta + (int64_t)bh * Nq;
    const float c = a.scale_log2;

    // query tiles that see any key of this workgroup (causal: queries >= k0)
    const int qt0 = CAUSAL ? k0 / BQ : 0;
    const int nt = max((Nq + BQ - 1) / BQ - qt0, 0);
    const int n_steps = nt > 0 ? 2 * nt + 1 : 0;
    TileCopy<DP, VEC, NT> qc, gc;
    qc.init(d, tid);
    gc.init(d, tid);
    const RowFrag<DP> rf(lane);
    float lrow = 0.0f, drow = 0.0f;
    auto load_tile = [&](int t) __attribute__((always_inline)) {
        const int r0 = (qt0 + t) * BQ;
        qc.load(qg, r0, Nq, d, tid);
        gc.load(gg, r0, Nq, d, tid);
        if (tid < BQ) {
            const int q = r0 + tid;
            lrow = q < Nq ? lg[q] * kLog2e : 0.0f;
            drow = q < Nq ? dg[q] : 0.0f;
        }
    };
    auto store_tile = [&](int b) __attribute__((always_inline)) {
        qc.store(Qsb[b], tid);
        gc.store(Gsb[b], tid);
        if (tid < BQ) {
            Lsb[b][tid] = lrow;
            Dsb[b][tid] = drow;
        }
    };
    if (nt > 0) {
        load_tile(0);
        store_tile(0);
    }
    if (nt > 1) {
        load_tile(1);
        store_tile(1);
    }
    if (nt > 2) load_tile(2);
    __syncthreads();
    // LDS writes of this step done, then the workgroup barrier; loads stay in flight
    auto end_step = [&]() __attribute__((always_inline)) {
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // tile staging of step s (every wave): tile t = (s + 1) / 2 into its buffer at odd s >= 3,
    // then the loads of tile t + 1
    auto stage = [&](int s) __attribute__((always_inline)) {
        if (s >= 3 && (s & 1)) {
            const int t = (s + 1) >> 1;
            if (t < nt) {
                store_tile(t & 1);
                if (t + 1 < nt) load_tile(t + 1);
            }
        }
    };
    // step index i -> (tile, 32-query block); a causal step whose queries all precede the
    // wave's keys is skipped by both roles alike
    auto step_active = [&](int i) __attribute__((always_inline)) {
        return !(CAUSAL && (qt0 + (i >> 1)) * BQ + (i & 1) * 32 + 31 < kw0);
    };
    uint16_t* dkg = (uint16_t*)a.dk + (int64_t)bh * Nk * d;
    uint16_t* dvg = (uint16_t*)a.dv + (int64_t)bh * Nk * d;
    // register r of block db: key kw0 + 8 (r/4) + 4 h32 + r%4, column db*32 + l32
    auto write_grad = [&](uint16_t* out, const f32x16 (&acc)[NDB], float sc) __attribute__((always_inline)) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = db * 32 + l32;
            if (col >= d) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                if (key < Nk) out[(int64_t)key * d + col] = Half<T>::one(acc[db][r] * sc);
            }
        }
    };

    if (wave < KB) {
        // role A: S, P, dV
        u32x4 kf[NDS];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) kf[ds] = load_chunk16<VEC>(kg, mykey, ds * 16 + 8 * h32, Nk, d);
        f32x16 dva[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) dva[i] = f32x16{};
        for (int s = 0; s < n_steps; ++s) {
            stage(s);
            if (s < 2 * nt && step_active(s)) {
                const int b = (s >> 1) & 1, qb = s & 1;
                const int qbase = (qt0 + (s >> 1)) * BQ + qb * 32;
                f32x16 sacc = f32x16{};
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) sacc = Half<T>::mfma(rf(Qsb[b], qb * 32, ds), kf[ds], sacc);
                // register r: query qbase + 8 (r/4) + 4 h32 + r%4, key mykey; kept iff
                // 8 (r/4) + r%4 >= lo (key past Nk: none; causal: on or below the diagonal).
                // Padded query rows need no test: their Q, dO and L are zero, and their weight
                // of 1 meets dO = 0 (and dP - D = 0 in role B).
                const int lo = mykey >= Nk ? 64 : CAUSAL ? mykey - qbase - 4 * h32 : -64;
                const bool full = kw0 + 32 <= Nk && (!CAUSAL || kw0 + 31 <= qbase);
                unsigned ppk[8];
                auto weights = [&](auto masked_c) __attribute__((always_inline)) {
                    constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const f32x4 lv = *(const f32x4*)(Lsb[b] + qb * 32 + 8 * g + 4 * h32);
                        f32x4 pv;
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            pv[e] = !MASKED || 8 * g + e >= lo
                                        ? __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[4 * g + e], c, -lv[e]))
                                        : 0.0f;
                        Pb[s & 1][kbk][g][lane] = pv;
                        ppk[2 * g] = Half<T>::pack2(pv[0], pv[1]);
                        ppk[2 * g + 1] = Half<T>::pack2(pv[2], pv[3]);
                    }
                };
                if (full) weights(std::false_type{});
                else weights(std::true_type{});
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 pa = {ppk[4 * t], ppk[4 * t + 1], ppk[4 * t + 2], ppk[4 * t + 3]};
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dva[db] = Half<T>::mfma(pa, tr_frag<DP>(Gsb[b], qb * 32 + 16 * t, db * 32, lane), dva[db]);
                }
            }
            end_step();
        }
        write_grad(dvg, dva, 1.0f);
    } else {
        // role B, one step behind: dP, dS, dK
        u32x4 vf[NDS];
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) vf[ds] = load_chunk16<VEC>(vg, mykey, ds * 16 + 8 * h32, Nk, d);
        f32x16 dka[NDB];
#pragma unroll
        for (int i = 0; i < NDB; ++i) dka[i] = f32x16{};
        for (int s = 0; s < n_steps; ++s) {
            stage(s);
            const int i = s - 1;
            if (i >= 0 && step_active(i)) {
                const int b = (i >> 1) & 1, qb = i & 1;
                f32x16 dp = f32x16{};
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) dp = Half<T>::mfma(rf(Gsb[b], qb * 32, ds), vf[ds], dp);
                unsigned spk[8];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const f32x4 dv = *(const f32x4*)(Dsb[b] + qb * 32 + 8 * g + 4 * h32);
                    const f32x4 pv = Pb[i & 1][kbk][g][lane];
                    float sv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) sv[e] = pv[e] * (dp[4 * g + e] - dv[e]);
                    spk[2 * g] = Half<T>::pack2(sv[0], sv[1]);
                    spk[2 * g + 1] = Half<T>::pack2(sv[2], sv[3]);
                }
#pragma unroll
                for (int t = 0; t < 2; ++t) {
                    const u32x4 sa = {spk[4 * t], spk[4 * t + 1], spk[4 * t + 2], spk[4 * t + 3]};
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        dka[db] = Half<T>::mfma(sa, tr_frag<DP>(Qsb[b], qb * 32 + 16 * t, db * 32, lane), dka[db]);
                }
            }
            end_step();
        }
        write_grad(dkg, dka, a.scale);
    }
}

// ---------------------------------------------------------------- dQ

// Two waves per SIMD at every head dim (the registers fit 256 per wave).
template <typename T, int DP, bool CAUSAL, bool VEC, int NW>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(BwdArgs a, int n_qtiles) {
    // queries per workgroup, keys per tile (128 where the registers allow: half the barriers)
    constexpr int BR = 32 * NW, BC = DP <= 64 || (DP <= 96 && NW == 8) ? 128 : 64;
    constexpr int STR = Tile16<DP>::STR;
    constexpr int NDS = DP / 16, NDB = DP / 32;
    __shared__ __attribute__((aligned(16))) uint16_t Ks[BC * STR];
    __shared__ __attribute__((aligned(16))) uint16_t Vs[BC * STR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    const PairTile pt = xcd_pair_tile(blockIdx.x, gridDim.x, n_qtiles, a.B * a.H, CAUSAL, NW == 8 ? kXcdSlots8 : kXcdSlots);
    const int bh = pt.pair;
    int qt = pt.tile;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first (tile-major dispatch per XCD)
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int q0 = qt * BR;
    const int r0w = q0 + 32 * wave;
    const int myq = r0w + l32;

    const uint16_t* qg = (const uint16_t*)a.q + (int64_t)bh * Nq * d;
    const uint16_t* kg = (const uint16_t*)a.k + (int64_t)bh * Nk * d;
    const uint16_t* vg = (const uint16_t*)a.v + (int64_t)bh * Nk * d;
    const uint16_t* gg = (const uint16_t*)a.dout + (int64_t)bh * Nq * d;

    // this wave's queries as B operands: lane holds Q[myq][16 ds + 8 h32 + 0..7] (dO likewise)
    u32x4 qf[NDS], gf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
        qf[ds] = load_chunk16<VEC>(qg, myq, ds * 16 + 8 * h32, Nq, d);
        gf[ds] = load_chunk16<VEC>(gg, myq, ds * 16 + 8 * h32, Nq, d);
    }
    const float lq = myq < Nq ? a.lse[(int64_t)bh * Nq + myq] * kLog2e : 0.0f;
    const float dq = myq < Nq ? a.delta[(int64_t)bh * Nq + myq] : 0.0f;
    const float c = a.scale_log2;

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;

    f32x16 dqa[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqa[i] = f32x16{};

    TileCopy<DP, VEC, 64 * NW, BC> kc, vc;
    kc.init(d, tid);
    vc.init(d, tid);
    const RowFrag<DP> rf(lane);
    kc.load(kg, 0, Nk, d, tid);
    vc.load(vg, 0, Nk, d, tid);
    for (int j = 0; j < n_tiles; ++j) {
        __syncthreads();
        kc.store(Ks, tid);
        vc.store(Vs, tid);
        __syncthreads();
        if (j + 1 < n_tiles) {
            kc.load(kg, (j + 1) * BC, Nk, d, tid);
            vc.load(vg, (j + 1) * BC, Nk, d, tid);
        }
        const int k0 = j * BC;
        if (CAUSAL && k0 > r0w + 31) continue;

        // S^T = K Q^T and dP^T = V dO^T: BC/32 blocks of 32 keys; register r of block kb is key
        // k0 + kb*32 + 8 (r/4) + 4 h32 + r%4, query myq
        unsigned pk[BC / 32][8];
#pragma unroll
        for (int kb = 0; kb < BC / 32; ++kb) {
            f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) {
                s = Half<T>::mfma(rf(Ks, kb * 32, ds), qf[ds], s);
                dp = Half<T>::mfma(rf(Vs, kb * 32, ds), gf[ds], dp);
            }
            const int lim = (CAUSAL ? min(Nk - 1, myq) : Nk - 1) - k0 - kb * 32 - 4 * h32;
            // every key of the block below Nk and (causal) at or before every query of the wave
            const bool full = k0 + kb * 32 + 32 <= Nk && (!CAUSAL || k0 + kb * 32 + 31 <= r0w);
            auto weights = [&](auto masked_c) __attribute__((always_inline)) {
                constexpr bool MASKED = decltype(masked_c)::value;
                float sv[16];
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int off = 8 * (r >> 2) + (r & 3);
                    const float p = !MASKED || off <= lim ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lq)) : 0.0f;
                    sv[r] = p * (dp[r] - dq);
                }
#pragma unroll
                for (int r = 0; r < 16; r += 2) pk[kb][r >> 1] = Half<T>::pack2(sv[r], sv[r + 1]);
            };
            // (the unmasked copy not for causal d = 128 at 4 waves, where it does not fit the
            // registers; 8 waves stage half as many chunks per thread)
            if ((DP <= 96 || !CAUSAL || NW == 8) && VEC && full) weights(std::false_type{});
            else weights(std::true_type{});
        }
        // dQ^T += K^T dS^T: BC/16 steps of 16 keys
#pragma unroll
        for (int t = 0; t < BC / 16; ++t) {
            const u32x4 sb = {pk[t >> 1][4 * (t & 1) + 0], pk[t >> 1][4 * (t & 1) + 1],
                              pk[t >> 1][4 * (t & 1) + 2], pk[t >> 1][4 * (t & 1) + 3]};
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const u32x4 ka = tr_frag<DP>(Ks, 16 * t, db * 32, lane);
                dqa[db] = Half<T>::mfma(ka, sb, dqa[db]);
            }
        }
    }

    // register r of block db: column db*32 + 8 (r/4) + 4 h32 + r%4, query myq
    if (myq < Nq) {
        uint16_t* og = (uint16_t*)a.dq + ((int64_t)bh * Nq + myq) * d;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * h32;
                if (VEC) {
                    if (d0 < d) {
                        u32x2 w = {Half<T>::pack2(dqa[db][4 * g + 0] * sc, dqa[db][4 * g + 1] * sc),
                                   Half<T>::pack2(dqa[db][4 * g + 2] * sc, dqa[db][4 * g + 3] * sc)};
                        *(u32x2*)(og + d0) = w;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < d) og[d0 + e] = Half<T>::one(dqa[db][4 * g + e] * sc);
                }
            }
    }
}

// ---------------------------------------------------------------- fp32

// Tile of ROWS rows x DP columns (fp32) staged through registers into LDS rows of STR floats;
// rows >= nrows and columns >= d are zero. VEC: 16-byte rows (d % 4 == 0, aligned buffers).
// Each wave moves a contiguous run of chunks, as in TileCopy.
template <int ROWS, int DP, int STR, bool VEC>
struct TileCopy32 {
    static constexpr int CPR = DP / 4;                  // 16-byte chunks per row
    static constexpr int CH = ROWS * CPR / 256;         // chunks per thread
    static_assert(ROWS * CPR % 256 == 0, "tile split");
    f32x4 r[CH];
    unsigned voff[CH];  // VEC: byte offset of this thread's chunk in a tile (as in TileCopy)
    __device__ __attribute__((always_inline)) void init(int d, int tid) {
        if constexpr (VEC) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 4;
                voff[c] = col < d ? (unsigned)(row * d + col) * 4u : kBufferVoid;
            }
        }
    }
    __device__ __attribute__((always_inline)) void load(const float* base, int row0, int nrows, int d, int tid) {
        if constexpr (VEC) {
            const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base + (int64_t)row0 * d, (int64_t)(nrows - row0) * d * 4);
#pragma unroll
            for (int c = 0; c < CH; ++c) r[c] = __builtin_bit_cast(f32x4, buffer_load16(rs, voff[c]));
        } else {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 4;
                r[c] = load_chunk32<VEC>(base, row0 + row, col, nrows, d);
            }
        }
    }
    __device__ __attribute__((always_inline)) void store(float* lds, int tid) const {
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
            const int row = chunk / CPR, col = (chunk % CPR) * 4;
            *(f32x4*)(lds + row * STR + col) = r[c];
        }
    }
};

// Half a row of fp32 (HALF = DP/2 values from column h32*HALF) into registers: the B operand
// of a 32x32x2 fp32 product whose reduction over the head dim runs as d = h32*HALF + i.
template <int HALF, bool VEC>
__device__ __attribute__((always_inline)) inline void load_half_row(float (&dst)[HALF], const float* base, int row,
                                                                    int nrows, int d, int h32) {
#pragma unroll
    for (int c4 = 0; c4 < HALF / 4; ++c4) {
        const f32x4 t = load_chunk32<VEC>(base, row, h32 * HALF + 4 * c4, nrows, d);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[4 * c4 + e] = t[e];
    }
}

// fp32 dK, dV on v_mfma_f32_32x32x2_f32, the layout of the fp32 forward mirrored: one
// workgroup per 128 keys (4 waves x 32 keys), looping over query tiles of 32. S = Q K^T and
// dP = dO V^T take this wave's keys as the MFMA columns (K and V half rows in registers, Q and
// dO read from LDS along the head dim), so a lane holds one key and 16 queries; register r of
// S is then, with the queries of the reduction enumerated in accumulator order, the A operand
// of dV += P^T dO (and dS of dK += dS^T Q), whose B operand is one dO (Q) row element per lane
// read from LDS. MODE 0 computes dK and dV, MODE 1 only dV (S, P, P^T dO) and MODE 2 only dK
// (S, dP, dS, dS^T Q): above d = 64 the two single-gradient kernels each recompute S but hold
// half the accumulators.
template <int DP, bool CAUSAL, int MODE, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(DP <= 64 || MODE == 1 ? 2 : 1, DP <= 64 || MODE == 1 ? 2 : 1)))
void bwd32_dkdv_kernel(BwdArgs a, int n_ktiles) {
    constexpr bool DO_DV = MODE != 2, DO_DK = MODE != 1;
    constexpr int BK = 128, BQ = 32;  // keys per workgroup, queries per tile
    constexpr int STR = DP + 4;       // LDS row stride (floats): 16-byte pad
    constexpr int HALF = DP / 2, NDB = DP / 32;
    __shared__ __attribute__((aligned(16))) float Qs[BQ * STR];
    __shared__ __attribute__((aligned(16))) float Gs[BQ * STR];  // dO
    __shared__ __attribute__((aligned(16))) float Ls[BQ];
    __shared__ __attribute__((aligned(16))) float Ds[BQ];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    const PairTile pt = xcd_pair_tile(blockIdx.x, gridDim.x, n_ktiles, a.B * a.H, CAUSAL, kXcdSlots);
    const int bh = pt.pair, kt = pt.tile;
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int k0 = kt * BK;
    const int kw0 = k0 + 32 * wave;
    const int mykey = kw0 + l32;

    const float* qg = (const float*)a.q + (int64_t)bh * Nq * d;
    const float* kg = (const float*)a.k + (int64_t)bh * Nk * d;
    const float* vg = (const float*)a.v + (int64_t)bh * Nk * d;
    const float* gg = (const float*)a.dout + (int64_t)bh * Nq * d;
    const float* lg = a.lse + (int64_t)bh * Nq;
    const float* dg = a.delta + (int64_t)bh * Nq;

    // this wave's keys as B operands: lane holds K[mykey][h32*HALF + i] (V likewise)
    float kf[HALF], vf[HALF];
    load_half_row<HALF, VEC>(kf, kg, mykey, Nk, d, h32);
    if constexpr (DO_DK) load_half_row<HALF, VEC>(vf, vg, mykey, Nk, d, h32);

    f32x16 dva[NDB], dka[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dva[i] = dka[i] = f32x16{};
    const float c = a.scale_log2;

    // query tiles that see any key of this workgroup (causal: queries >= k0)
    const int qt0 = CAUSAL ? k0 / BQ : 0;
    const int n_qt = (Nq + BQ - 1) / BQ;
    TileCopy32<BQ, DP, STR, VEC> qc, gc;
    qc.init(d, tid);
    gc.init(d, tid);
    float lrow = 0.0f, drow = 0.0f;
    auto load_tile = [&](int qt) __attribute__((always_inline)) {
        qc.load(qg, qt * BQ, Nq, d, tid);
        gc.load(gg, qt * BQ, Nq, d, tid);
        if (tid < BQ) {
            const int q = qt * BQ + tid;
            lrow = q < Nq ? lg[q] * kLog2e : 0.0f;
            drow = q < Nq ? dg[q] : 0.0f;
        }
    };
    if (qt0 < n_qt) load_tile(qt0);
    for (int qt = qt0; qt < n_qt; ++qt) {
        __syncthreads();
        qc.store(Qs, tid);
        gc.store(Gs, tid);
        if (tid < BQ) {
            Ls[tid] = lrow;
            Ds[tid] = drow;
        }
        __syncthreads();
        if (qt + 1 < n_qt) load_tile(qt + 1);
        const int q0 = qt * BQ;
        // a causal wave skips tiles whose queries all precede its keys
        if (CAUSAL && q0 + BQ - 1 < kw0) continue;

        // S = Q K^T and dP = dO V^T: 32 queries x this wave's 32 keys; register r holds query
        // q0 + 8 (r/4) + 4 h32 + r%4 and key mykey
        f32x16 s = f32x16{}, dp = f32x16{};
        const float* qp = Qs + l32 * STR + h32 * HALF;
        const float* gp = Gs + l32 * STR + h32 * HALF;
#pragma unroll
        for (int c4 = 0; c4 < HALF / 4; ++c4) {
            const f32x4 qa = *(const f32x4*)(qp + 4 * c4);
            f32x4 ga = {};
            if constexpr (DO_DK) ga = *(const f32x4*)(gp + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(qa[e], kf[4 * c4 + e], s, 0, 0, 0);
                if constexpr (DO_DK) dp = __builtin_amdgcn_mfma_f32_32x32x2f32(ga[e], vf[4 * c4 + e], dp, 0, 0, 0);
            }
        }
        // the weight is kept iff off = 8 (r/4) + r%4 >= lo (the causal diagonal and the key
        // tail in one compare); padded query rows have zero Q, dO, L and D and add nothing
        const int lo = mykey >= Nk ? 64 : CAUSAL ? mykey - q0 - 4 * h32 : -64;
        float pr[16], dsr[16];
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const int ql = 8 * g + 4 * h32;
            const f32x4 lv = *(const f32x4*)(Ls + ql);
            f32x4 dv = {};
            if constexpr (DO_DK) dv = *(const f32x4*)(Ds + ql);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float p = 8 * g + e >= lo ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * g + e], c, -lv[e])) : 0.0f;
                pr[4 * g + e] = p;
                if constexpr (DO_DK) dsr[4 * g + e] = p * (dp[4 * g + e] - dv[e]);
            }
        }
        // dV += P^T dO and dK += dS^T Q: k-step r reduces over the two queries lane halves hold
        // in register r; the B operand is that query's row, one element per lane
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = 8 * (r >> 2) + 4 * h32 + (r & 3);
            const float* grow = Gs + row * STR + l32;
            const float* qrow = Qs + row * STR + l32;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if constexpr (DO_DV) dva[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(pr[r], grow[db * 32], dva[db], 0, 0, 0);
                if constexpr (DO_DK) dka[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(dsr[r], qrow[db * 32], dka[db], 0, 0, 0);
            }
        }
    }

    // register r of block db: key kw0 + 8 (r/4) + 4 h32 + r%4, column db*32 + l32
    float* dkg = (float*)a.dk + (int64_t)bh * Nk * d;
    float* dvg = (float*)a.dv + (int64_t)bh * Nk * d;
    const float sc = a.scale;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        const int col = db * 32 + l32;
        if (col >= d) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = kw0 + 8 * (r >> 2) + 4 * h32 + (r & 3);
            if (key < Nk) {
                if constexpr (DO_DV) dvg[(int64_t)key * d + col] = dva[db][r];
                if constexpr (DO_DK) dkg[(int64_t)key * d + col] = dka[db][r] * sc;
            }
        }
    }
}

// fp32 dQ on v_mfma_f32_32x32x2_f32: one workgroup per 128 queries (4 waves x 32), looping over
// key tiles of 32, in the fp32 forward's layout: S^T = K Q^T and dP^T = V dO^T with this wave's
// queries as the columns (Q and dO half rows in registers, K and V from LDS along the head
// dim), so dS^T register r is the B operand of dQ^T += K^T dS^T, whose A operand is one K row
// element per lane read from LDS.
template <int DP, bool CAUSAL, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(DP <= 64 ? 2 : 1, DP <= 64 ? 2 : 1)))
void bwd32_dq_kernel(BwdArgs a, int n_qtiles) {
    constexpr int BR = 128, BC = 32;  // queries per workgroup, keys per tile
    constexpr int STR = DP + 4;
    constexpr int HALF = DP / 2, NDB = DP / 32;
    __shared__ __attribute__((aligned(16))) float Ks[BC * STR];
    __shared__ __attribute__((aligned(16))) float Vs[BC * STR];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    const PairTile pt = xcd_pair_tile(blockIdx.x, gridDim.x, n_qtiles, a.B * a.H, CAUSAL, kXcdSlots);
    const int bh = pt.pair;
    int qt = pt.tile;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    const int Nq = a.Nq, Nk = a.Nk, d = a.d;
    const int q0 = qt * BR;
    const int r0w = q0 + 32 * wave;
    const int myq = r0w + l32;

    const float* qg = (const float*)a.q + (int64_t)bh * Nq * d;
    const float* kg = (const float*)a.k + (int64_t)bh * Nk * d;
    const float* vg = (const float*)a.v + (int64_t)bh * Nk * d;
    const float* gg = (const float*)a.dout + (int64_t)bh * Nq * d;

    float qf[HALF], gf[HALF];
    load_half_row<HALF, VEC>(qf, qg, myq, Nq, d, h32);
    load_half_row<HALF, VEC>(gf, gg, myq, Nq, d, h32);
    const float lq = myq < Nq ? a.lse[(int64_t)bh * Nq + myq] * kLog2e : 0.0f;
    const float dq = myq < Nq ? a.delta[(int64_t)bh * Nq + myq] : 0.0f;
    const float c = a.scale_log2;

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;

    f32x16 dqa[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) dqa[i] = f32x16{};

    TileCopy32<BC, DP, STR, VEC> kc, vc;
    kc.init(d, tid);
    vc.init(d, tid);
    kc.load(kg, 0, Nk, d, tid);
    vc.load(vg, 0, Nk, d, tid);
    for (int j = 0; j < n_tiles; ++j) {
        __syncthreads();
        kc.store(Ks, tid);
        vc.store(Vs, tid);
        __syncthreads();
        if (j + 1 < n_tiles) {
            kc.load(kg, (j + 1) * BC, Nk, d, tid);
            vc.load(vg, (j + 1) * BC, Nk, d, tid);
        }
        const int k0 = j * BC;
        if (CAUSAL && k0 > r0w + 31) continue;

        // S^T = K Q^T and dP^T = V dO^T: register r is key k0 + 8 (r/4) + 4 h32 + r%4, query myq
        f32x16 s = f32x16{}, dp = f32x16{};
        const float* kp = Ks + l32 * STR + h32 * HALF;
        const float* vp = Vs + l32 * STR + h32 * HALF;
#pragma unroll
        for (int c4 = 0; c4 < HALF / 4; ++c4) {
            const f32x4 ka = *(const f32x4*)(kp + 4 * c4);
            const f32x4 va = *(const f32x4*)(vp + 4 * c4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s = __builtin_amdgcn_mfma_f32_32x32x2f32(ka[e], qf[4 * c4 + e], s, 0, 0, 0);
                dp = __builtin_amdgcn_mfma_f32_32x32x2f32(va[e], gf[4 * c4 + e], dp, 0, 0, 0);
            }
        }
        const int lim = (CAUSAL ? min(Nk - 1, myq) : Nk - 1) - k0 - 4 * h32;
        float dsr[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + (r & 3);
            const float p = off <= lim ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c, -lq)) : 0.0f;
            dsr[r] = p * (dp[r] - dq);
        }
        // dQ^T += K^T dS^T: k-step r reduces over the two keys lane halves hold in register r
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const float* krow = Ks + (8 * (r >> 2) + 4 * h32 + (r & 3)) * STR + l32;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                dqa[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(krow[db * 32], dsr[r], dqa[db], 0, 0, 0);
        }
    }

    // register r of block db: column db*32 + 8 (r/4) + 4 h32 + r%4, query myq
    if (myq < Nq) {
        float* og = (float*)a.dq + ((int64_t)bh * Nq + myq) * d;
        const float sc = a.scale;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * h32;
                const f32x4 w = {dqa[db][4 * g + 0] * sc, dqa[db][4 * g + 1] * sc, dqa[db][4 * g + 2] * sc,
                                 dqa[db][4 * g + 3] * sc};
                if (VEC) {
                    if (d0 < d) *(f32x4*)(og + d0) = w;
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (d0 + e < d) og[d0 + e] = w[e];
                }
            }
    }
}

template <int DP, bool VEC>
int launch_bwd32(const BwdArgs& a, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.H * a.Nq;
    if ((rows + 15) / 16 > INT32_MAX) return (int)hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_delta_any_kernel<float>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                       a.o, a.dout, a.delta, rows, a.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const int n_kt = (a.Nk + 127) / 128;
    const unsigned g1 = (unsigned)((int64_t)n_kt * a.B * a.H);
    if constexpr (DP <= 64) {
        if (a.causal)
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, true, 0, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
        else
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, false, 0, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
    } else {
        // dV and dK as two kernels, each holding half the accumulators
        if (a.causal) {
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, true, 1, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, true, 2, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
        } else {
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, false, 1, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
            hipLaunchKernelGGL((bwd32_dkdv_kernel<DP, false, 2, VEC>), dim3(g1), dim3(256), 0, st, a, n_kt);
        }
    }
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const int n_qt = (a.Nq + 127) / 128;
    const unsigned g2 = (unsigned)((int64_t)n_qt * a.B * a.H);
    if (a.causal)
        hipLaunchKernelGGL((bwd32_dq_kernel<DP, true, VEC>), dim3(g2), dim3(256), 0, st, a, n_qt);
    else
        hipLaunchKernelGGL((bwd32_dq_kernel<DP, false, VEC>), dim3(g2), dim3(256), 0, st, a, n_qt);
    return (int)hipGetLastError();
}

// NW-wave launches of the 16-bit dK/dV (d <= 96) and dQ kernels, 32 rows per wave. More waves
// share each staged tile, so each stages less of it (8 waves measured 2-7% faster than 4 on
// grids of two or more workgroups per CU); fewer rows per workgroup balance small grids
// better. The results are the same bit for bit: every wave sums the same tiles in the same order.
template <typename T, int DP, bool VEC, int NW>
void launch_dkdv16(const BwdArgs& a, hipStream_t st) {
    const int n_kt = (a.Nk + 32 * NW - 1) / (32 * NW);
    const unsigned g = (unsigned)((int64_t)n_kt * a.B * a.H);
    if (a.causal)
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, DP, true, VEC, NW>), dim3(g), dim3(64 * NW), 0, st, a, n_kt);
    else
        hipLaunchKernelGGL((bwd_dkdv_kernel<T, DP, false, VEC, NW>), dim3(g), dim3(64 * NW), 0, st, a, n_kt);
}
template <typename T, int DP, bool VEC, int NW>
void launch_dq16(const BwdArgs& a, hipStream_t st) {
    const int n_qt = (a.Nq + 32 * NW - 1) / (32 * NW);
    const unsigned g = (unsigned)((int64_t)n_qt * a.B * a.H);
    if (a.causal)
        hipLaunchKernelGGL((bwd_dq_kernel<T, DP, true, VEC, NW>), dim3(g), dim3(64 * NW), 0, st, a, n_qt);
    else
        hipLaunchKernelGGL((bwd_dq_kernel<T, DP, false, VEC, NW>), dim3(g), dim3(64 * NW), 0, st, a, n_qt);
}

template <typename T, int DP, bool VEC>
int launch_bwd_t(const BwdArgs& a, hipStream_t st) {
    const int64_t rows = (int64_t)a.B * a.H * a.Nq;
    static_assert(DP <= 128, "row terms: at most 16 chunks of 8 per row");
    if ((rows + 15) / 16 > INT32_MAX) return (int)hipErrorInvalidConfiguration;
    if (VEC)
        hipLaunchKernelGGL(bwd_delta_kernel<T>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                           (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows, a.d);
    else
        hipLaunchKernelGGL(bwd_delta_any_kernel<T>, dim3((unsigned)((rows + 15) / 16)), dim3(256), 0, st,
                           a.o, a.dout, a.delta, rows, a.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    // dK, dV up to d = 96 and dQ: 8-wave workgroups (256 rows) while their grid still gives
    // every CU two, else 4-wave ones (128 rows)
    const bool wide_k = (int64_t)((a.Nk + 255) / 256) * a.B * a.H >= 2 * (int64_t)a.num_cus;
    const bool wide_q = (int64_t)((a.Nq + 255) / 256) * a.B * a.H >= 2 * (int64_t)a.num_cus;
    if constexpr (DP <= 96) {
        if (wide_k) launch_dkdv16<T, DP, VEC, 8>(a, st);
        else launch_dkdv16<T, DP, VEC, 4>(a, st);
    } else {
        // above d = 96 the accumulators of both gradients no longer fit one wave at two waves
        // per SIMD: the two-role kernel, 128 keys per workgroup
        const int n_kt = (a.Nk + 127) / 128;
        const unsigned g1 = (unsigned)((int64_t)n_kt * a.B * a.H);
        if (a.causal)
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, DP, true, VEC>), dim3(g1), dim3(512), 0, st, a, n_kt);
        else
            hipLaunchKernelGGL((bwd_dkdv_pair_kernel<T, DP, false, VEC>), dim3(g1), dim3(512), 0, st, a, n_kt);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    if (wide_q) launch_dq16<T, DP, VEC, 8>(a, st);
    else launch_dq16<T, DP, VEC, 4>(a, st);
    return (int)hipGetLastError();
}

template <typename T, bool VEC>
int launch_bwd_16(const BwdArgs& a, int dpad, hipStream_t st) {
    switch (dpad) {
        case 32: return launch_bwd_t<T, 32, VEC>(a, st);
        case 64: return launch_bwd_t<T, 64, VEC>(a, st);
        case 96: return launch_bwd_t<T, 96, VEC>(a, st);
        case 128: return launch_bwd_t<T, 128, VEC>(a, st);
        default: return (int)hipErrorInvalidValue;
    }
}

template <bool VEC>
int launch_bwd_32(const BwdArgs& a, int dpad, hipStream_t st) {
    switch (dpad) {
        case 32: return launch_bwd32<32, VEC>(a, st);
        case 64: return launch_bwd32<64, VEC>(a, st);
        case 96: return launch_bwd32<96, VEC>(a, st);
        case 128: return launch_bwd32<128, VEC>(a, st);
        default: return (int)hipErrorInvalidValue;
    }
}

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxScratchDevices];  // per device, resolved on first use

}  // namespace

// Row-term workspace of the allocation-free backward entry point. In host code this name is a
// host-side stand-in: kernels receive the device address hipGetSymbolAddress reports for the
// current device, never the name itself.
static __device__ __align__(256) float scratch[kBwdScratchFloats];

int bwd_scratch(float** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    if (dev < 0 || dev >= kMaxScratchDevices) return (int)hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return (int)e;
        g_scratch_ptr[dev] = (float*)p;
    }
    *out = g_scratch_ptr[dev];
    return (int)hipSuccess;
}

int launch_bwd(const BwdArgs& a, int dpad, bool vec, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.dtype == 0) return vec ? launch_bwd_32<true>(a, dpad, st) : launch_bwd_32<false>(a, dpad, st);
    if (a.dtype == 2) return vec ? launch_bwd_16<__bf16, true>(a, dpad, st) : launch_bwd_16<__bf16, false>(a, dpad, st);
    return vec ? launch_bwd_16<_Float16, true>(a, dpad, st) : launch_bwd_16<_Float16, false>(a, dpad, st);
}

}  // namespace fa

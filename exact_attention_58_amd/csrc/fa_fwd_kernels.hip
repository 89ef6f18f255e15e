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
//    the PV product while l sums the fp32 weights. The fp32 path keeps P in fp32.
//  * K/V tiles are loaded from HBM with 16-byte coalesced loads into registers
//    one tile ahead of their use and stored to LDS behind a barrier.
//  * Keys past Nk are zero in LDS and masked to -inf; the causal mask keeps key
//    j for query i iff j <= i; tiles wholly above the diagonal are skipped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// Running-max refresh threshold in log2 units: O and l are rescaled only when a
// row's max grows by more than this, otherwise the old max stays the reference.
// The result is unchanged (numerator and denominator share the reference) and
// the unnormalised weights stay below 2^8.
constexpr float kRescaleThreshold = 8.0f;

// The rows of one (batch, head) pair. Dense inputs are [B,H,N,d]: pair bh starts at row bh*N
// of every tensor. Packed sequences of different lengths (page "Meta's xFormers has Attention
// kernel written in CUTLASS": fixed and variable lengths served by one kernel) are
// [H, total, d]: sequence b of head h starts at row h*total + cu[b]. Offsets are clamped into
// [0, total] and lengths to the launch's maxima, so offsets that break their documented
// contract cannot move an access outside the tensors.
struct Slice {
    int64_t q0, k0;  // first query row and first key row of the pair
    int nq, nk;      // its query and key counts
};
__device__ __attribute__((always_inline)) inline Slice slice_of(const FwdArgs& a, int bh) {
    if (a.cu_q == nullptr) return {(int64_t)bh * a.Nq, (int64_t)bh * a.Nk, a.Nq, a.Nk};
    const int b = bh / a.H, h = bh - b * a.H;
    const int64_t qs = min(max((int64_t)a.cu_q[b], (int64_t)0), a.tq);
    const int64_t qe = min(max((int64_t)a.cu_q[b + 1], qs), a.tq);
    const int64_t ks = min(max((int64_t)a.cu_k[b], (int64_t)0), a.tk);
    const int64_t ke = min(max((int64_t)a.cu_k[b + 1], ks), a.tk);
    return {h * a.tq + qs, h * a.tk + ks, (int)min(qe - qs, (int64_t)a.Nq), (int)min(ke - ks, (int64_t)a.Nk)};
}

// Workgroup -> (batch-head pair, query tile). Workgroups are dealt to the 8 XCDs in turn.
// Dense inputs give every pair the same work, so each XCD takes a contiguous run of pairs
// (xcd_remap) and keeps their K and V in its own L2. Packed sequences give each pair work in
// proportion to its sequence's length, and contiguous runs would load one XCD with the
// longest sequences; there pair p goes to XCD p % 8 with all its query tiles, which spreads
// every sequence's heads over all XCDs (a bijection when the pair count is a multiple of 8,
// otherwise the dense order is kept).
// Causal grids run tiles heaviest first (the kernels reverse qt) and take the XCD-local
// grouped tile-major order of xcd_pair_tile, so the heavy tiles of an XCD's pairs start
// before the light ones. Dense pairs all have equal work; packed sequences differ in
// length, and tile-major order over their pairs still starts the longest sequences' last
// query tiles first (simulated with the bench's packed lengths: 220 -> 212 tile-units per
// XCD against an ideal of 204).
struct TileId {
    int bh, qt;
};
// slots: the workgroups one group of pairs should hold at least. The 4-wave kernels pass what
// an XCD holds at once (32 CUs x 2 or 3, their waves per SIMD); the ping-pong kernel passes
// twice its 32 resident ones,
// which measured about 2% faster on dense causal grids of 2 or more pairs per XCD (packed
// batches: 32).
__device__ __attribute__((always_inline)) inline TileId tile_of(const FwdArgs& a, int n_qtiles, int slots) {
    const int i = blockIdx.x;
    if (a.slots > 0) slots = a.slots;
    const PairTile pt = xcd_pair_tile(i, gridDim.x, n_qtiles, a.B * a.H, a.causal, slots);
    if (a.cu_q != nullptr && (a.B * a.H) % 8 == 0) {
        // XCD x takes pairs x, x + 8, x + 16, ...: its m-th pair is the m-th of its run above
        const int x = i & 7;
        return {x + 8 * (pt.pair - x * ((a.B * a.H) >> 3)), pt.tile};
    }
    return {pt.pair, pt.tile};
}

// Query rows [r0, r0 + br) of a sequence that has queries but no keys: the softmax sum is
// empty, so O = 0 and L = ln 0 = -inf. Every thread of the workgroup takes part.
template <typename E>
__device__ void write_empty_rows(const FwdArgs& a, const Slice& sl, int r0, int br) {
    const int rows = min(br, sl.nq - r0);
    E* o = (E*)a.o + (sl.q0 + r0) * a.d;
    for (int i = threadIdx.x; i < rows * a.d; i += blockDim.x) o[i] = E(0);
    for (int i = threadIdx.x; i < rows; i += blockDim.x) a.lse[sl.q0 + r0 + i] = kNegInf;
}

// Maximum of the NKB*16 values of s as a balanced tree (v_maximum3), so the dependency chain
// is logarithmic in the number of values instead of linear. MIN selects the minimum instead.
// The NaN-propagating maximum needs no canonicalising copies of the MFMA results, which the
// IEEE maxnum (fmaxf) adds before each v_max; on scores and -inf the two agree.
template <int NKB, bool MIN>
__device__ __attribute__((always_inline)) inline float tile_extreme(const f32x16 (&s)[NKB]) {
    float v[NKB * 16];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[kb * 16 + r] = s[kb][r];
    int n = NKB * 16;
#pragma unroll
    for (int step = 0; step < 6; ++step) {
        if (n == 1) break;
        const int m = (n + 2) / 3;
#pragma unroll
        for (int i = 0; i < m; ++i) {
            const float a = v[3 * i];
            const float b = 3 * i + 1 < n ? v[3 * i + 1] : a;
            const float c = 3 * i + 2 < n ? v[3 * i + 2] : a;
            v[i] = MIN ? __builtin_elementwise_minimum(__builtin_elementwise_minimum(a, b), c)
                       : __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
        }
        n = m;
    }
    return v[0];
}

// First half of an online-softmax step on a tile of S^T held as NKB blocks of 32 keys (lane:
// one query, 16 keys per block): apply the key-tail and causal masks and return the tile's
// row max in log2 units; *cc receives the factor that turns s into log2 units (the scale for
// unmasked tiles, 1 for masked tiles, whose s this function scales in place). Unmasked
// tiles skip the per-element scaling: for c >= 0 the max of s*c is c*max(s), for c < 0 it
// is c*min(s), and the scale folds into the exp2 argument's FMA.
template <int NKB, bool CAUSAL>
__device__ __attribute__((always_inline)) inline float tile_max_log2(f32x16 (&s)[NKB], float c, bool masked,
                                                                     int k0, int Nk, int myq, int h32,
                                                                     float* cc) {
    if (masked) {
        // key = k0 + 4*h32 + off with a compile-time offset per register: visible iff
        // key <= Nk - 1 and (causal) key <= myq, i.e. off <= lim
        const int lim = (CAUSAL ? min(Nk - 1, myq) : Nk - 1) - k0 - 4 * h32;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int off = kb * 32 + 8 * (r >> 2) + (r & 3);
                s[kb][r] = off <= lim ? s[kb][r] * c : kNegInf;
            }
        *cc = 1.0f;
        return wave_half_max(tile_extreme<NKB, false>(s));
    }
    *cc = c;
    if (c >= 0.0f) return wave_half_max(tile_extreme<NKB, false>(s)) * c;
    return wave_half_min(tile_extreme<NKB, true>(s)) * c;
}

// Second half: refresh (m, l, O) when the row max grew by more than the threshold, then
// replace s by the unnormalised weights exp2(s*cc - m). The caller adds the weights to l.
template <int NKB, int NDB>
__device__ __attribute__((always_inline)) inline void tile_exp(f32x16 (&s)[NKB], f32x16 (&oacc)[NDB],
                                                               float& m_run, float& l_run, float mt,
                                                               float cc) {
    const float m_cand = __builtin_elementwise_maximum(m_run, mt);
    if (__any(m_cand > m_run + kRescaleThreshold)) {
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_cand);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
        m_run = m_cand;
    }
    const float nm = -m_run;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], cc, nm));
}

// Whole online-softmax step (masks, max, rescale, exp) for kernels that run it in one place.
template <int NKB, int NDB, bool CAUSAL>
__device__ __attribute__((always_inline)) inline void softmax_step(
        f32x16 (&s)[NKB], f32x16 (&oacc)[NDB], float& m_run, float& l_run, float c, bool masked,
        int k0, int Nk, int myq, int h32) {
    float cc;
    const float mt = tile_max_log2<NKB, CAUSAL>(s, c, masked, k0, Nk, myq, h32, &cc);
    tile_exp<NKB, NDB>(s, oacc, m_run, l_run, mt, cc);
}

// Sum of the weights of a tile as a balanced tree (fp32 path).
template <int NKB>
__device__ __attribute__((always_inline)) inline float tile_sum(const f32x16 (&s)[NKB]) {
    float v[NKB * 16];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) v[kb * 16 + r] = s[kb][r];
#pragma unroll
    for (int n = NKB * 16; n > 1; n /= 2)
#pragma unroll
        for (int i = 0; i < n / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
    return v[0];
}

// Packs the tile's weights to the 16-bit type (pk[kb][r/2] holds keys r, r+1 of block kb) and
// returns the sum of the fp32 weights (a balanced tree). l sums the fp32 weights, not the
// rounded ones: a 16-bit weight carries up to 2^-8 relative rounding error, which a row with
// few visible keys would pass straight into L = m + ln(l).
template <typename T, int NKB>
__device__ __attribute__((always_inline)) inline float pack_and_sum(const f32x16 (&s)[NKB], unsigned (&pk)[NKB][8]) {
    const float sum = tile_sum<NKB>(s);
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; r += 2) pk[kb][r >> 1] = Half<T>::pack2(s[kb][r], s[kb][r + 1]);
    return sum;
}

// 16-bit forward kernel. DP: padded head dim (32 ... 256). Workgroup = 4 waves; K/V
// tiles of 64 keys. SPLIT = 1: 4 row blocks of 32 = 128 query rows, every wave walks all
// key tiles. SPLIT = 2 (grids too small to fill the chip): 2 row blocks = 64
// rows, and the two waves of a row block each walk one half of the key tiles (two tiles
// staged per step); at the end the second half's (O, m, l) pass through LDS and the first
// half merges them: m = max(m1, m2), l = l1 2^(m1-m) + l2 2^(m2-m), O likewise, the same
// exact combination the online recurrence makes tile by tile.
// Head dims up to 32 run 128-key tiles (half the barriers and reductions per key, where the
// softmax's vector work dominates). Without the key split, head dims up to 64 compile for
// three waves per SIMD (at most 168 registers; non-causal d = 64: 16-19% faster on short
// sequences, 7-8% on small grids; causal B4 H32 N2048 d64: 106 -> 91 us), and so does
// non-causal d = 96 over 16-byte rows (B16 H64 N512: 156 -> 138 us; its element-wise instance
// would spill). The key split at d = 64 takes three as well (causal B1 H16 N4096: 62 -> 54 us;
// at d = 32 it would spill).
template <int DP, int SPLIT, bool CAUSAL, bool VEC>
constexpr int fwd16_waves_per_simd() {
    return DP > 128 ? 1
           : ((SPLIT == 1 && (DP <= 64 || (DP == 96 && !CAUSAL && VEC))) ||
              (SPLIT == 2 && DP == 64))
               ? 3
               : 2;
}

template <typename T, int DP, bool CAUSAL, bool VEC, int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256),
                          amdgpu_waves_per_eu(fwd16_waves_per_simd<DP, SPLIT, CAUSAL, VEC>(), fwd16_waves_per_simd<DP, SPLIT, CAUSAL, VEC>())))
void fwd16_kernel(FwdArgs a, int n_qtiles) {
    // Causal grids split too: a workgroup's rows start at q0 = 64 t and its key tiles end at
    // its diagonal, so the second half starts at key 64 ceil((t + 1) / 2) <= q0 and every row
    // sees a key of the first tile it processes (for t = 0 the second half has no tile and
    // merges as zero weight).
    static_assert(SPLIT == 1 || SPLIT == 2, "one or two key halves");
    // K/V tiles of 64 keys; 128 up to DP = 32; 32 at DP = 256, where 64-key tiles staged
    // through registers no longer fit the 512 registers of one wave per SIMD
    constexpr int NW = 4, RB = NW / SPLIT, BR = 32 * RB, BC = DP > 224 ? 32 : DP <= 32 ? 128 : 64;
    constexpr int NKB = BC / 32;
    constexpr int KST = DP + 8;   // K row stride (elements): 16-byte pad, conflict-free b128 reads
    // V row stride: 4 consecutive rows must start in 4 distinct quarters of the 16 bank groups
    // (the transposed read serves 4 rows x 4 chunks at once), i.e. a pitch of 4 or 12 chunks
    // mod 16: head dims whose chunk count is a multiple of 8 (64, 128, 192, 256) get 4 pad
    // chunks, the others (32, 96, 160, 224) already have one.
    constexpr int VST = (DP / 8) % 8 == 0 ? DP + 32 : DP;
    constexpr int CPR = DP / 8;   // 16-byte chunks per row
    constexpr int CH = BC * CPR / (64 * NW);  // chunks per thread per tile
    static_assert(BC * CPR % (64 * NW) == 0, "tile load split");
    constexpr int NDS = DP / 16;  // k-steps of the QK^T product
    constexpr int NDB = DP / 32;  // 32-wide head-dim blocks of O^T

    // SPLIT tile buffers; after the key loop the same memory carries the split merge
    constexpr int TILE_ELEMS = BC * KST + BC * VST;
    constexpr int MERGE_FLOATS = SPLIT > 1 ? RB * (NDB * 16 + 2) * 64 : 0;
    constexpr int SMEM_B = SPLIT * TILE_ELEMS * 2 > MERGE_FLOATS * 4 ? SPLIT * TILE_ELEMS * 2 : MERGE_FLOATS * 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[SMEM_B];
    auto Ksb = [&](int h) __attribute__((always_inline)) { return (uint16_t*)smem + h * TILE_ELEMS; };
    auto Vsb = [&](int h) __attribute__((always_inline)) { return (uint16_t*)smem + h * TILE_ELEMS + BC * KST; };

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    const int rbk = wave % RB, half = wave / RB;  // row block, key half

    // an XCD holds 32 CUs x (workgroups per CU) of these at once
    const TileId wt = tile_of(a, n_qtiles, 32 * fwd16_waves_per_simd<DP, SPLIT, CAUSAL, VEC>());
    const int bh = wt.bh;
    int qt = wt.qt;
    if (CAUSAL) qt = n_qtiles - 1 - qt;  // longest rows first
    const Slice sl = slice_of(a, bh);
    const int Nq = sl.nq, Nk = sl.nk, d = a.d;
    const int q0 = qt * BR;
    if (q0 >= Nq) return;  // a packed sequence shorter than the longest
    if (Nk == 0) return write_empty_rows<uint16_t>(a, sl, q0, BR);
    const int r0w = q0 + rbk * 32;
    const int myq = r0w + l32;

    const uint16_t* qg = (const uint16_t*)a.q + sl.q0 * d;
    const uint16_t* kg = (const uint16_t*)a.k + sl.k0 * d;
    const uint16_t* vg = (const uint16_t*)a.v + sl.k0 * d;

    // Q fragments (B operand of S^T = K Q^T): lane holds Q[myq][16*ds + 8*h32 + 0..7]
    u32x4 qf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = load_chunk16<VEC>(qg, myq, ds * 16 + 8 * h32, Nq, d);

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n_tiles = (kv_end + BC - 1) / BC;
    // key half h walks tiles [h * n_steps, min(n_tiles, (h + 1) * n_steps))
    const int n_steps = (n_tiles + SPLIT - 1) / SPLIT;

    // step i stages tile h * n_steps + i of every half h (rows past Nk load as zeros). With
    // 16-byte rows the chunks load through buffer resources that end at row Nk (or hold
    // nothing for a tile past the last), at per-thread offsets fixed for every tile. Each
    // wave moves a contiguous run of CH x 64 chunks (0-3% faster than every wave taking every
    // fourth KB; the same bits).
    u32x4 kreg[SPLIT][CH], vreg[SPLIT][CH];
    unsigned voff[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
        const int row = chunk / CPR, col = (chunk % CPR) * 8;
        voff[c] = col < d ? (unsigned)(row * d + col) * 2u : kBufferVoid;
    }
    auto load_tile = [&](int i) __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPLIT; ++h) {
            const int j = h * n_steps + i;
            if constexpr (VEC) {
                const int64_t nb = j < n_tiles ? (int64_t)(Nk - j * BC) * d * 2 : 0;
                const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg + (int64_t)j * BC * d, nb);
                const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg + (int64_t)j * BC * d, nb);
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    kreg[h][c] = buffer_load16(rk, voff[c]);
                    vreg[h][c] = buffer_load16(rv, voff[c]);
                }
            } else {
#pragma unroll
                for (int c = 0; c < CH; ++c) {
                    const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                    const int row = chunk / CPR, col = (chunk % CPR) * 8;
                    kreg[h][c] = load_chunk16<VEC>(kg, j * BC + row, col, j < n_tiles ? Nk : 0, d);
                    vreg[h][c] = load_chunk16<VEC>(vg, j * BC + row, col, j < n_tiles ? Nk : 0, d);
                }
            }
        }
    };
    auto store_tile = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int h = 0; h < SPLIT; ++h)
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                const int chunk = (tid >> 6) * (CH * 64) + c * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 8;
                *(u32x4*)(Ksb(h) + row * KST + col) = kreg[h][c];
                *(u32x4*)(Vsb(h) + row * VST + col) = vreg[h][c];
            }
    };
    const uint16_t* Ks = Ksb(half);
    const uint16_t* Vs = Vsb(half);

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float c = a.scale_log2;

    load_tile(0);
    for (int i = 0; i < n_steps; ++i) {
        __syncthreads();
        store_tile();
        __syncthreads();
        if (i + 1 < n_steps) load_tile(i + 1);

        const int j = half * n_steps + i;
        if (SPLIT > 1 && j >= n_tiles) continue;  // the last half may have one tile less
        const int k0 = j * BC;
        if (CAUSAL && k0 > r0w + 31) continue;  // every key of the tile is above this wave's rows

        // ---- S^T = K Q^T: two 32-key blocks
        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            s[kb] = f32x16{};
            const uint16_t* kp = Ks + (kb * 32 + l32) * KST + 8 * h32;
#pragma unroll
            for (int ds = 0; ds < NDS; ++ds) s[kb] = Half<T>::mfma(*(const u32x4*)(kp + ds * 16), qf[ds], s[kb]);
        }

        // ---- online softmax, then pack P to the 16-bit type
        // softmax at normal priority, MFMA stretches raised: on a SIMD shared by two
        // workgroups the products of one take precedence and the other's softmax fills in
        __builtin_amdgcn_s_setprio(0);
        const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > r0w);
        softmax_step<NKB, NDB, CAUSAL>(s, oacc, m_run, l_run, c, masked, k0, Nk, myq, h32);
        unsigned pk[NKB][8];
        l_run += pack_and_sum<T, NKB>(s, pk);
        __builtin_amdgcn_s_setprio(1);

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

    if constexpr (SPLIT > 1) {
        // ---- merge the key halves: half 1 hands (O, m, l) to half 0 through LDS
        // (lane-contiguous rows of 64 floats: conflict-free)
        constexpr int NV = NDB * 16 + 2;
        float* mrg = (float*)smem + rbk * NV * 64;
        __syncthreads();  // every wave is done with the tile buffers
        if (half == 1) {
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) mrg[(db * 16 + r) * 64 + lane] = oacc[db][r];
            mrg[(NV - 2) * 64 + lane] = m_run;
            mrg[(NV - 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (half == 1) return;
        const float m2 = mrg[(NV - 2) * 64 + lane], l2 = mrg[(NV - 1) * 64 + lane];
        const float m = fmaxf(m_run, m2);  // finite: half 0 has seen key tile 0
        const float a1 = __builtin_amdgcn_exp2f(m_run - m), a2 = __builtin_amdgcn_exp2f(m2 - m);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a1 + mrg[(db * 16 + r) * 64 + lane] * a2;
        l_run = l_run * a1 + l2 * a2;
        m_run = m;
    }

    // ---- epilogue: O = O / l, L = (m + log2 l) ln 2
    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < Nq) {
        uint16_t* og = (uint16_t*)a.o + (sl.q0 + myq) * d;
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
        if (h32 == 0) a.lse[sl.q0 + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- 16-bit, two-group ping-pong

// Reduction op r of an in-place pairwise tree over P values (levels of P/2, P/4, ..., 1 ops
// in that order): the slot it writes, part[o] = part[2o] + part[2o+1].
template <int P>
constexpr int tree_slot(int r) {
    int base = 0;
    for (int n = P / 2; n >= 1; n /= 2) {
        if (r < base + n) return r - base;
        base += n;
    }
    return 0;
}

// LDS layouts of the K and V tiles. The LDS serves 256 bytes per clock over 64 four-byte
// banks, i.e. 16 bank groups of 16 bytes; a b128 read is served 16 lanes at a time and a
// 64-bit transposed read 32 lanes at a time. A K fragment read takes one 16-byte chunk from
// each of 16 consecutive key rows, a V^T fragment read 4 aligned chunks from each of 4
// consecutive key rows: each must fall in 16 distinct bank groups, and every operand address
// stays a per-lane base plus an immediate offset. A tile is filled by 1 KB copy instructions
// (lane i writes 16-byte slot i), so the layout is chosen by where each slot loads from.
//  * Dense (rows of 4, 8 or 16 chunks): no padding slots, so a copy moves only data. A
//    256-byte K line holds chunks 2m and 2m+1 of 8 consecutive rows, chunk c of row r in slot
//    2(r&7) + ((c ^ (r >> 3)) & 1): the 16 rows of a read lie in two lines, one per slot
//    parity. A V line holds 4 aligned chunks of 4 consecutive rows, which is exactly what one
//    half-wave of a transposed read takes. One copy instruction covers whole rows or whole
//    128-byte row segments.
//  * Padded (d = 96): K rows of 13 chunks (odd, so 16 consecutive rows spread over the 16
//    groups) and V rows of 12 (12 mod 16 spreads 4 rows x 4 chunks). Here the dense lines
//    would cut the 192-byte rows into pieces of 32 and 64 bytes.
template <int DP> struct KvLayout {
    static constexpr int CPR = DP / 8;  // 16-byte data chunks per row
    static constexpr bool DENSE = (CPR & (CPR - 1)) == 0;
    static constexpr int KP = DENSE ? CPR : CPR + 1, VP = CPR;  // slots per row
    // key row r and chunk c that slot p of a K (isk) or V tile holds
    __device__ static void slot_rc(bool isk, int p, int& r, int& c) {
        const int line = p >> 4, q = p & 15;
        if (!DENSE) {
            const int pitch = isk ? KP : VP;
            r = p / pitch;
            c = p - r * pitch;
        } else if (isk) {
            r = 8 * (line / (CPR / 2)) + (q >> 1);
            c = 2 * (line % (CPR / 2)) + ((q ^ (r >> 3)) & 1);
        } else {
            r = 4 * (line / (CPR / 4)) + (q >> 2);
            c = 4 * (line % (CPR / 4)) + (q & 3);
        }
    }
    // K fragment of key rows 32kb + l32, chunk 2ds + h32: per-lane base + koff(kb, ds)
    __device__ static unsigned kbase(int l32, int h32) {
        return DENSE ? (l32 >> 3) * (CPR / 2) * 256 + 32 * (l32 & 7) + 16 * ((h32 ^ (l32 >> 3)) & 1)
                     : l32 * KP * 16 + h32 * 16;
    }
    static constexpr int koff(int kb, int ds) { return DENSE ? kb * CPR * 512 + ds * 256 : kb * 32 * KP * 16 + ds * 32; }
    // V^T fragment: lane (i16, g16, h32) reads key row 16t + 8hi + 4h32 + i16/4, bytes
    // 64db + 32g16 + 8(i16 & 3) of it: per-lane base + voff(t, db, hi)
    __device__ static unsigned vbase(int h32, int i16, int g16) {
        return DENSE ? h32 * (CPR / 4) * 256 + (i16 >> 2) * 64 + 32 * g16 + 8 * (i16 & 3)
                     : (4 * h32 + (i16 >> 2)) * VP * 16 + (16 * g16 + 4 * (i16 & 3)) * 2;
    }
    static constexpr int voff(int t, int db, int hi) {
        return DENSE ? (4 * t + 2 * hi) * (CPR / 4) * 256 + db * 256 : (16 * t + 8 * hi) * VP * 16 + db * 64;
    }
};

// 16-bit forward kernel for aligned inputs with d % 8 == 0: 8 waves in two groups of four.
// While one group runs its MFMA phase the other runs its softmax phase; a workgroup barrier
// separates the phases, so on each SIMD (one wave of each group) the matrix core and the
// vector ALU work at the same time. Global phase 2m is group 0's MFMA phase m and group 1's
// softmax phase m-1; phase 2m+1 is group 1's MFMA phase m and group 0's softmax phase m.
//  * MFMA phase j: O^T += V_{j-1}^T P_{j-1}^T, then S^T_j = K_j Q^T. Around the MFMAs the
//    wave also folds the fp32 weights of tile j-1 into l, and after the last MFMA applies
//    the masks and takes the row max of S_j.
//  * Softmax phase j: the wave's share of the direct HBM->LDS copies of tile j+2 (group 0
//    copies K_{j+2}, group 1 V_{j+2}),
//    the rescale test, exp2 of the tile, packing P_j to 16 bits, and the first PV operands
//    of the next MFMA phase (read ahead of the barrier).
// Copies are issued from the softmax phase because issuing them stalls the issuing wave for
// a while; there the stall does not hold up the matrix core. The copies a group issues in
// its softmax phase j are awaited in global phase 2j+3 (group 0 at the start of its
// softmax phase j+1, group 1 at the end of its MFMA phase j+1), so they are in LDS when
// the barrier ending that phase lets group 0 start MFMA phase j+2. K has three LDS buffers (K_j is read
// in MFMA phase j), V four (V_j is read at the end of softmax phase j and in MFMA phase
// j+1), so no buffer is rewritten while either group may still read it. Tail rows of K/V
// are clamped to row Nk-1. Both groups run one loop body (their differences are scalar
// flags), so the accumulators keep fixed registers. Every MFMA phase runs the full program:
// the first one multiplies a zero P by the resident V_0, and a causal wave past its diagonal
// runs fully masked tiles whose weights are exactly zero; the phases are barrier-bound, so
// neither costs time.
// Key tiles hold 64 keys, and 128 up to DP = 64: there a 64-key phase is short (16 MFMAs),
// and the longer tile halves the barriers, row-max reductions and rescale tests per key
// (about 7% faster at d = 64; three K and four V buffers of 128 keys take 112 KB of LDS).
template <typename T, int DP, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fwd16_pp_kernel(FwdArgs a, int n_qtiles) {
    constexpr int WPG = 4, NWAVE = 2 * WPG;
    constexpr int BR = 32 * NWAVE, BC = pp_keys(DP);
    constexpr int NKB = BC / 32;
    using L = KvLayout<DP>;
    constexpr int KTILEB = BC * L::KP * 16, VTILEB = BC * L::VP * 16;
    constexpr int NDS = DP / 16;
    constexpr int NDB = DP / 32;

    constexpr int NKBUF = 3, NVBUF = 4;
    __shared__ __attribute__((aligned(16))) uint8_t smem[NKBUF * KTILEB + NVBUF * VTILEB];

    const int tid = threadIdx.x, lane = tid & 63;
    // wave index through readfirstlane: the group branch below is a scalar branch, so
    // each wave executes only its own group's barriers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h32 = lane >> 5, l32 = lane & 31;
    const int grp = wave / WPG, wig = wave % WPG;

    // packed batches keep groups of 32 workgroups: with 64 the causal bench batch (16
    // sequences of 533..3973) ran 10-14% slower, its groups then mixing sequences
    const TileId wt = tile_of(a, n_qtiles, a.cu_q != nullptr ? 32 : 64);
    const int bh = wt.bh;
    int qt = wt.qt;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
    const Slice sl = slice_of(a, bh);
    const int Nq = sl.nq, Nk = sl.nk, d = a.d;
    const int q0 = qt * BR;
    if (q0 >= Nq) return;  // a packed sequence shorter than the longest
    if (Nk == 0) return write_empty_rows<uint16_t>(a, sl, q0, BR);
    const int r0w = q0 + grp * 32 * WPG + wig * 32;
    const int myq = r0w + l32;

    const uint16_t* qg = (const uint16_t*)a.q + sl.q0 * d;
    const uint16_t* kg = (const uint16_t*)a.k + sl.k0 * d;
    const uint16_t* vg = (const uint16_t*)a.v + sl.k0 * d;

    u32x4 qf[NDS];
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) qf[ds] = load_chunk16<true>(qg, myq, ds * 16 + 8 * h32, Nq, d);

    int kv_end = Nk;
    if (CAUSAL) kv_end = min(Nk, min(q0 + BR, Nq));
    const int n = (kv_end + BC - 1) / BC;
    const int dchunks = d / 8;

    // Direct HBM->LDS copy of the K and V tiles in the KvLayout. The copy of a tile pair is
    // KI + VI wave instructions (64 lanes x 16 B, wave-uniform LDS destination, lane i ->
    // +16*i): group 0 issues those of K and group 1 those of V, each wave a contiguous run
    // (4 KB of consecutive rows of one tile at d = 64 and 128; measured 1-2% faster than
    // spreading every wave's copies over both tiles, the same bits). A lane on a padding slot
    // loads a valid chunk of its row into the padding, which is never read, so the copy of a
    // full tile needs no lane mask. Chunks past d (DP > d) repeat the row's last
    // data chunk: finite, and Q is zero there, so they add nothing to the scores. A tile that
    // runs past Nk repeats row Nk-1 in its tail rows (finite; their scores are masked and
    // their weights are zero); only that last tile takes the slower clamped path.
    constexpr int KI = L::KP * BC / 64, VI = L::VP * BC / 64;  // copy instructions per K / V tile
    constexpr int NKW = (KI + WPG - 1) / WPG, NVW = (VI + WPG - 1) / WPG;
    constexpr int NCP = NKW > NVW ? NKW : NVW;
    const bool kgrp = grp == 0;
    auto cidx = [&](int it) __attribute__((always_inline)) { return kgrp ? wig * NKW + it : KI + wig * NVW + it; };
    auto cvalid = [&](int it) __attribute__((always_inline)) {
        return kgrp ? it < NKW && wig * NKW + it < KI : it < NVW && wig * NVW + it < VI;
    };
    unsigned coff[NCP];  // lane's byte offset within a full tile (row r, column chunk)
#pragma unroll
    for (int it = 0; it < NCP; ++it) {
        const int c = cvalid(it) ? cidx(it) : 0;
        const int idx = c < KI ? c : c - KI;
        int r, cch;
        L::slot_rc(c < KI, idx * 64 + lane, r, cch);
        coff[it] = (unsigned)(r * d + min(cch, dchunks - 1) * 8) * 2u;
    }
    auto kbuf = [&](int j) __attribute__((always_inline)) { return smem + (j % NKBUF) * KTILEB; };
    auto vbuf = [&](int j) __attribute__((always_inline)) { return smem + NKBUF * KTILEB + (j % NVBUF) * VTILEB; };
    // copy instruction `it` of this wave for tile m (wave-uniform branches only)
    auto issue_copy = [&](int it, int m) __attribute__((always_inline)) {
        const int c = cidx(it);
        if (m >= n || !cvalid(it)) return;
        const bool isk = c < KI;
        const int idx = isk ? c : c - KI;
        const uint8_t* tile = (const uint8_t*)((isk ? kg : vg) + (int64_t)m * BC * d);
        uint8_t* dst = (isk ? kbuf(m) : vbuf(m)) + idx * 1024;
        if (m * BC + BC <= Nk) {
            __builtin_amdgcn_global_load_lds((const void*)(tile + coff[it]), (FA_LDS void*)dst, 16, 0, 0);
        } else {
            int r, cch;
            L::slot_rc(isk, idx * 64 + lane, r, cch);
            const int rr = min(r, Nk - 1 - m * BC);
            const unsigned off = (unsigned)(rr * d + min(cch, dchunks - 1) * 8) * 2u;
            __builtin_amdgcn_global_load_lds((const void*)(tile + off), (FA_LDS void*)dst, 16, 0, 0);
        }
    };
    auto issue_tiles = [&](int m) __attribute__((always_inline)) {  // all of K_m and V_m
#pragma unroll
        for (int it = 0; it < NCP; ++it) issue_copy(it, m);
    };
    auto wait_loads = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float c = a.scale_log2;
    f32x16 s[NKB];
    unsigned pk[NKB][8];
#pragma unroll
    for (int i = 0; i < 8 * NKB; ++i) pk[i / 8][i % 8] = 0u;

    // MFMA phase as one unrolled micro-program: NQ MFMAs of S^T_j = K_j Q^T (k-step ds of key
    // block kb) then NP MFMAs of O^T += V_{j-1}^T P_{j-1}^T (key step t of head-dim block db).
    // Each MFMA's LDS operand is read LA MFMAs ahead into a small ring, and scheduling
    // barriers keep that order, so the one wave of this group on the SIMD keeps the matrix
    // core fed while the LDS reads of the next MFMAs are in flight. A QK operand is one b128
    // read, a PV operand two transposed b64 reads: at most 2*LA LDS reads are outstanding.
    constexpr int NQ = NKB * NDS, NP = (BC / 16) * NDB;
    constexpr int LA = 6;
    const int i16 = lane & 15, g16 = (lane >> 4) & 1;
    // per-lane operand bases (LDS byte addresses); every fragment is base + compile-time offset
    const unsigned kbase = L::kbase(l32, h32);
    const unsigned vbase = L::vbase(h32, i16, g16);
    const unsigned smem_a = lds_addr(smem);
    auto kaddr = [&](int j) __attribute__((always_inline)) { return smem_a + (j % NKBUF) * KTILEB + kbase; };
    auto vaddr = [&](int j) __attribute__((always_inline)) { return smem_a + NKBUF * KTILEB + (j % NVBUF) * VTILEB + vbase; };
    auto fetch = [&](auto ic, unsigned ka, unsigned va) __attribute__((always_inline)) -> u32x4 {
        constexpr int i = decltype(ic)::value;
        if constexpr (i < NP) {
            constexpr int t = i / NDB, db = i % NDB;
            const u32x2 lo = lds_rdtr16<L::voff(t, db, 0)>(va);
            const u32x2 hi = lds_rdtr16<L::voff(t, db, 1)>(va);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
        } else {
            constexpr int qi = i - NP, ds = qi / NKB, kb = qi % NKB;
            return lds_rd128<L::koff(kb, ds)>(ka);
        }
    };
    u32x4 ring[LA];
    // first operands of the PV product on tile jp (at most LA, all of them V fragments),
    // read before the MFMA phase starts
    constexpr int NPRE = LA < NP ? LA : NP;
    auto prefetch_pv = [&](int jp) __attribute__((always_inline)) {
        const unsigned va = vaddr(jp);
        static_for<0, NPRE>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            ring[i] = fetch(std::integral_constant<int, i>{}, 0u, va);
        });
    };
    // DO_PV: accumulate P V of tile jp (its first LA operands already in the ring);
    // DO_QK: compute S^T_j. Both compile-time so the unrolled program and its ring are static.
    // partial sums of the previous tile's weights (tree folded around the MFMAs)
    constexpr int NPART = 8 * NKB;  // pair sums of the tile's 16 NKB weights
    float part[NPART];
    auto mphase_t = [&](auto do_qk_c, auto do_pv_c, int j, int jp) __attribute__((always_inline)) {
        constexpr bool DO_QK = decltype(do_qk_c)::value, DO_PV = decltype(do_pv_c)::value;
        static_assert(DO_PV, "the MFMA phase always folds the previous tile's weights");
        constexpr int first = 0, end = DO_QK ? NP + NQ : NP;
        const unsigned ka = kaddr(j), va = vaddr(jp);
        // ring slots not filled ahead of the barrier: the QK operands among the first LA
        // when the PV product is shorter than LA
        static_for<NPRE, LA>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            if constexpr (first + i < end) ring[i] = fetch(std::integral_constant<int, first + i>{}, ka, va);
        });
        static_for<first, end>([&](auto ic) __attribute__((always_inline)) {
            constexpr int i = decltype(ic)::value;
            constexpr int slot = (i - first) % LA;
            u32x4 op = ring[slot];
            if constexpr (i + LA < end) ring[slot] = fetch(std::integral_constant<int, i + LA>{}, ka, va);
            // operations issued after fetch i and still allowed in flight
            constexpr int last_issued = (i + LA < end) ? i + LA : end - 1;
            constexpr int pending = [&]() constexpr {
                int c = 0;
                for (int q = i + 1; q <= last_issued; ++q) c += (q < NP ? 2 : 1);
                return c;
            }();
            lgkm_wait<pending>(op);
            if constexpr (i < NP) {
                constexpr int t = i / NDB, db = i % NDB;
                const u32x4 pb = {pk[t >> 1][4 * (t & 1) + 0], pk[t >> 1][4 * (t & 1) + 1],
                                  pk[t >> 1][4 * (t & 1) + 2], pk[t >> 1][4 * (t & 1) + 3]};
                oacc[db] = Half<T>::mfma(op, pb, oacc[db]);
                // first tree level of the previous tile's weight sum (s still holds them):
                // pair q of the NPART is added at PV step q mod NP
                static_for<0, NPART>([&](auto qc) __attribute__((always_inline)) {
                    constexpr int q = decltype(qc)::value;
                    if constexpr (q % NP == i) part[q] = s[q >> 3][2 * (q & 7)] + s[q >> 3][2 * (q & 7) + 1];
                });
            } else {
                constexpr int qi = i - NP, ds = qi / NKB, kb = qi % NKB;
                // the first k-step of each key block starts from a zero accumulator
                s[kb] = Half<T>::mfma(op, qf[ds], ds == 0 ? f32x16{} : s[kb]);
                // remaining tree levels (NPART / 2, ..., 2, 1 partial sums = reduction ops
                // 0..NPART-2, in dependency order), spread over the NQ QK steps
                static_for<(qi * (NPART - 1)) / NQ, ((qi + 1) * (NPART - 1)) / NQ>([&](auto rc) __attribute__((always_inline)) {
                    constexpr int r = decltype(rc)::value;
                    constexpr int o = tree_slot<NPART>(r);
                    part[o] = part[2 * o] + part[2 * o + 1];
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (!DO_QK) {
#pragma unroll
            for (int n2 = NPART / 2; n2 >= 1; n2 /= 2)
#pragma unroll
                for (int i = 0; i < n2; ++i) part[i] = part[2 * i] + part[2 * i + 1];
        }
        l_run += part[0];
    };
    using yes = std::integral_constant<bool, true>;
    using no = std::integral_constant<bool, false>;
    float mt = 0.0f, cc = 1.0f;
    auto tile_max = [&](int j) __attribute__((always_inline)) {
        const int k0 = j * BC;
        const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > r0w);
        mt = tile_max_log2<NKB, CAUSAL>(s, c, masked, k0, Nk, myq, h32, &cc);
    };
    auto softmax = [&]() __attribute__((always_inline)) {
        tile_exp<NKB, NDB>(s, oacc, m_run, l_run, mt, cc);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; r += 2) pk[kb][r >> 1] = Half<T>::pack2(s[kb][r], s[kb][r + 1]);
    };

    // prologue: K_0, V_0, K_1, V_1 resident before the first phase
    issue_tiles(0);
    issue_tiles(1);
    wait_loads();
    __syncthreads();
    prefetch_pv(0);  // operands of the first (zero-weight) PV product
#pragma unroll
    for (int i = 0; i < 16 * NKB; ++i) s[i / 16][i % 16] = 0.0f;  // no previous tile to fold into l

    const bool g0 = grp == 0;
    if (!g0) barrier_nofence();  // group 1 starts one phase later
    for (int j = 0; j < n; ++j) {
        // MFMA phase: group 0 in global phase 2j, group 1 in 2j+1
        mphase_t(yes{}, yes{}, j, j > 0 ? j - 1 : 0);
        tile_max(j);
        __builtin_amdgcn_sched_barrier(0);
        // this wave's copies of tile j+1 (issued in its previous softmax phase) must land
        // before the barrier that ends global phase 2j+1: group 1 waits at the end of this
        // MFMA phase, group 0 right after the barrier (its phase 2j+1 is the next one)
        if (!g0) wait_loads();
        barrier_nofence();
        if (g0) wait_loads();
        // softmax phase: group 0 in global phase 2j+1, group 1 in 2j+2
        issue_tiles(j + 2);
        softmax();
        prefetch_pv(j);
        __builtin_amdgcn_sched_barrier(0);
        barrier_nofence();
    }
    mphase_t(no{}, yes{}, n - 1, n - 1);
    if (g0) barrier_nofence();

    // epilogue: O = O / l, L = (m + log2 l) ln 2
    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < Nq) {
        uint16_t* og = (uint16_t*)a.o + (sl.q0 + myq) * d;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d0 = db * 32 + 8 * g + 4 * h32;
                if (d0 < d) {
                    u32x2 w = {Half<T>::pack2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                               Half<T>::pack2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
                    *(u32x2*)(og + d0) = w;
                }
            }
        if (h32 == 0) a.lse[sl.q0 + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- fp32

// fp32 forward kernel on v_mfma_f32_32x32x2_f32. The head-dim reduction of S^T is
// enumerated as d = h32*(DP/2) + ds so each lane loads half a contiguous row of Q
// and of K. P stays fp32 for the PV product. SPLIT = 2 (grids too small to fill the chip)
// works as in the 16-bit kernel: 64 rows per workgroup, the two waves of a row block each
// walk one half of the key tiles (one LDS tile buffer per half) and the halves' (O, m, l)
// merge through LDS at the end. SPLIT = 4 (still smaller grids) gives a workgroup one row
// block of 32 rows whose four waves each walk a quarter of the key tiles (32-key tiles, so
// the four staged tiles fit the registers), merged the same way in quarter order: on the
// fp32 matrix core a wave's chain of products is what a small grid waits for, and the
// quarters cut it by half again. Causal grids may split too: every tile a workgroup
// processes starts at or before its first row q0 (its tiles end at its diagonal, and the
// last one starts at most at q0), so every row sees a key of the first tile of each part;
// a part with no tile (small t) merges as zero weight.
template <int DP, int BC, bool CAUSAL, bool VEC, int SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(2, 2)))
void fwd32_kernel(FwdArgs a, int n_qtiles) {
    static_assert(SPLIT == 1 || SPLIT == 2 || SPLIT == 4, "one, two or four key parts");
    constexpr int NW = 4, RB = NW / SPLIT, BR = 32 * RB;
    constexpr int KST = DP + 4;  // floats; 16-byte pad
    constexpr int VST = DP;      // floats
    constexpr int CPR = DP / 4;
    constexpr int CH = BC * CPR / (64 * NW);
    static_assert(BC * CPR % (64 * NW) == 0, "tile load split");
    constexpr int HALF = DP / 2;
    constexpr int NKB = BC / 32;
    constexpr int NDB = DP / 32;

    // One K/V buffer per key half, two barriers per tile: tile j+1 is stored once every wave
    // has read tile j, and its loads are in flight while tile j is computed. (Two buffers with
    // one barrier per tile, where two workgroups still fit the LDS, measured slower: fp32 B4
    // H4 N4096 d64 524 vs 504 us, d128 994 vs 980 us, causal B1 H16 N4096 d128 595 vs 588 us.)
    constexpr int NBUF = SPLIT;
    __shared__ __attribute__((aligned(16))) float Ks[NBUF][BC * KST];
    __shared__ __attribute__((aligned(16))) float Vs[NBUF][BC * VST];
    static_assert(SPLIT == 1 || (SPLIT - 1) * RB * (NDB * 16 + 2) * 64 <= NBUF * BC * KST, "merge fits the K buffers");

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h32 = lane >> 5, l32 = lane & 31;
    const int rbk = wave % RB, half = wave / RB;  // row block, key half

    const TileId wt = tile_of(a, n_qtiles, 64);
    const int bh = wt.bh;
    int qt = wt.qt;
    if (CAUSAL) qt = n_qtiles - 1 - qt;
    const Slice sl = slice_of(a, bh);
    const int Nq = sl.nq, Nk = sl.nk, d = a.d;
    const int q0 = qt * BR;
    if (q0 >= Nq) return;  // a packed sequence shorter than the longest
    if (Nk == 0) return write_empty_rows<float>(a, sl, q0, BR);
    const int r0w = q0 + rbk * 32;
    const int myq = r0w + l32;

    const float* qg = (const float*)a.q + sl.q0 * d;
    const float* kg = (const float*)a.k + sl.k0 * d;
    const float* vg = (const float*)a.v + sl.k0 * d;

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

    // staging of SPLIT tiles (one per key part; rows past Nk load as zeros). With 16-byte
    // rows the chunks load through buffer resources that end at row Nk (or hold nothing for
    // a tile past the last), at per-thread offsets fixed for every tile; each wave moves a
    // contiguous run of chunks.
    f32x4 kreg[SPLIT][CH], vreg[SPLIT][CH];
    unsigned voff[CH];
#pragma unroll
    for (int cc = 0; cc < CH; ++cc) {
        const int chunk = (tid >> 6) * (CH * 64) + cc * 64 + (tid & 63);
        const int row = chunk / CPR, col = (chunk % CPR) * 4;
        voff[cc] = col < d ? (unsigned)(row * d + col) * 4u : kBufferVoid;
    }
    auto load_tile_h = [&](int h, int j) __attribute__((always_inline)) {
        if constexpr (VEC) {
            const int64_t nb = j < n_tiles ? (int64_t)(Nk - j * BC) * d * 4 : 0;
            const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kg + (int64_t)j * BC * d, nb);
            const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vg + (int64_t)j * BC * d, nb);
#pragma unroll
            for (int cc = 0; cc < CH; ++cc) {
                kreg[h][cc] = __builtin_bit_cast(f32x4, buffer_load16(rk, voff[cc]));
                vreg[h][cc] = __builtin_bit_cast(f32x4, buffer_load16(rv, voff[cc]));
            }
        } else {
#pragma unroll
            for (int cc = 0; cc < CH; ++cc) {
                const int chunk = (tid >> 6) * (CH * 64) + cc * 64 + (tid & 63);
                const int row = chunk / CPR, col = (chunk % CPR) * 4;
                kreg[h][cc] = load_chunk32<VEC>(kg, j * BC + row, col, j < n_tiles ? Nk : 0, d);
                vreg[h][cc] = load_chunk32<VEC>(vg, j * BC + row, col, j < n_tiles ? Nk : 0, d);
            }
        }
    };
    auto store_tile_h = [&](int h, int b) __attribute__((always_inline)) {
#pragma unroll
        for (int cc = 0; cc < CH; ++cc) {
            const int chunk = (tid >> 6) * (CH * 64) + cc * 64 + (tid & 63);
            const int row = chunk / CPR, col = (chunk % CPR) * 4;
            *(f32x4*)(Ks[b] + row * KST + col) = kreg[h][cc];
            *(f32x4*)(Vs[b] + row * VST + col) = vreg[h][cc];
        }
    };
    auto load_tile = [&](int j) __attribute__((always_inline)) { load_tile_h(0, j); };
    auto store_tile = [&](int b) __attribute__((always_inline)) { store_tile_h(0, b); };

    f32x16 oacc[NDB];
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
    float m_run = kNegInf, l_run = 0.0f;
    const float c = a.scale_log2;

    // one key tile: QK^T, masks and online softmax, PV (Kb / Vb: the LDS buffer holding it)
    auto tile = [&](int j, const float* Kb, const float* Vb) __attribute__((always_inline)) {
        const int k0 = j * BC;
        // a causal wave skips tiles wholly above its rows (the workgroup still loads them
        // for its other waves)
        if (!CAUSAL || k0 <= r0w + 31) {
            f32x16 s[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                s[kb] = f32x16{};
                const float* kp = Kb + (kb * 32 + l32) * KST + h32 * HALF;
#pragma unroll
                for (int c4 = 0; c4 < HALF / 4; ++c4) {
                    const f32x4 kv = *(const f32x4*)(kp + 4 * c4);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[e], qf[4 * c4 + e], s[kb], 0, 0, 0);
                }
            }

            // the MFMA stretches run at raised wave priority, so on a SIMD shared by two
            // workgroups the matrix products of one take precedence over the softmax of
            // the other, which fills the gaps
            __builtin_amdgcn_s_setprio(0);
            const bool masked = (k0 + BC > Nk) || (CAUSAL && k0 + BC - 1 > r0w);
            softmax_step<NKB, NDB, CAUSAL>(s, oacc, m_run, l_run, c, masked, k0, Nk, myq, h32);
            l_run += tile_sum<NKB>(s);
            __builtin_amdgcn_s_setprio(1);

            // O^T += V^T P^T, one key per lane half per MFMA: k-step r of block kb is
            // key kb*32 + 8*(r/4) + 4*h32 + r%4, the key the lane's S^T register r holds.
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = kb * 32 + 8 * (r >> 2) + 4 * h32 + (r & 3);
                    const float* vp = Vb + key * VST + l32;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vp[db * 32], s[kb][r], oacc[db], 0, 0, 0);
                }
        }
    };
    if constexpr (SPLIT > 1) {
        // step i stages tile h * n_steps + i of each part h into buffer h
        const int n_steps = (n_tiles + SPLIT - 1) / SPLIT;
#pragma unroll
        for (int h = 0; h < SPLIT; ++h) load_tile_h(h, h * n_steps);
        for (int i = 0; i < n_steps; ++i) {
            __syncthreads();
#pragma unroll
            for (int h = 0; h < SPLIT; ++h) store_tile_h(h, h);
            __syncthreads();
            if (i + 1 < n_steps) {
#pragma unroll
                for (int h = 0; h < SPLIT; ++h) load_tile_h(h, h * n_steps + i + 1);
            }
            const int j = half * n_steps + i;
            if (j < n_tiles) tile(j, Ks[half], Vs[half]);  // a later part may have fewer tiles
        }
        // merge the key parts: parts 1.. hand (O, m, l) to part 0 through LDS (lane-contiguous
        // rows of 64 floats); part 0 adds them in part order
        constexpr int NV = NDB * 16 + 2;
        auto mrg = [&](int h) __attribute__((always_inline)) { return &Ks[0][0] + ((h - 1) * RB + rbk) * NV * 64; };
        __syncthreads();  // every wave is done with the tile buffers
        if (half > 0) {
            float* w = mrg(half);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) w[(db * 16 + r) * 64 + lane] = oacc[db][r];
            w[(NV - 2) * 64 + lane] = m_run;
            w[(NV - 1) * 64 + lane] = l_run;
        }
        __syncthreads();
        if (half > 0) return;
        float m = m_run;  // finite: part 0 has seen key tile 0
#pragma unroll
        for (int h = 1; h < SPLIT; ++h) m = fmaxf(m, mrg(h)[(NV - 2) * 64 + lane]);
        const float a0 = __builtin_amdgcn_exp2f(m_run - m);
#pragma unroll
        for (int h = 1; h < SPLIT; ++h) {
            const float* w = mrg(h);
            const float ah = __builtin_amdgcn_exp2f(w[(NV - 2) * 64 + lane] - m);
            const float lh = w[(NV - 1) * 64 + lane];
            if (h == 1) {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] = oacc[db][r] * a0 + w[(db * 16 + r) * 64 + lane] * ah;
                l_run = l_run * a0 + lh * ah;
            } else {
#pragma unroll
                for (int db = 0; db < NDB; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r) oacc[db][r] += w[(db * 16 + r) * 64 + lane] * ah;
                l_run += lh * ah;
            }
        }
        m_run = m;
    } else {
        load_tile(0);
        for (int j = 0; j < n_tiles; ++j) {
            __syncthreads();
            store_tile(0);
            __syncthreads();
            if (j + 1 < n_tiles) load_tile(j + 1);
            tile(j, Ks[0], Vs[0]);
        }
    }

    const float l_tot = wave_half_sum(l_run);
    const float inv = 1.0f / l_tot;
    if (myq < Nq) {
        float* og = (float*)a.o + (sl.q0 + myq) * d;
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
        if (h32 == 0) a.lse[sl.q0 + myq] = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    }
}

// ---------------------------------------------------------------- launch

constexpr size_t kLdsPerCu = 160 * 1024;

// occ > 0 caps the workgroups a CU holds at once: each launch also reserves unused dynamic
// LDS so that one workgroup's share is kLdsPerCu / occ (no reservation when the kernel's
// own LDS already exceeds that share).
// Static LDS bytes of a kernel, asked of the runtime once per kernel (the code object is the
// same on every gfx950 device) and remembered.
static hipError_t static_lds(const void* fn, size_t* out) {
    struct Entry {
        const void* fn;
        size_t lds;
    };
    static std::mutex mu;
    static Entry cache[128];
    static int used = 0;
    std::lock_guard<std::mutex> lk(mu);
    for (int i = 0; i < used; ++i)
        if (cache[i].fn == fn) {
            *out = cache[i].lds;
            return hipSuccess;
        }
    hipFuncAttributes attr;
    const hipError_t e = hipFuncGetAttributes(&attr, fn);
    if (e != hipSuccess) return e;
    if (used < 128) cache[used++] = Entry{fn, attr.sharedSizeBytes};
    *out = attr.sharedSizeBytes;
    return hipSuccess;
}

template <typename K>
static int launch(K kernel, const FwdArgs& a, int br, hipStream_t st, int threads, int occ) {
    const int n_qtiles = (a.Nq + br - 1) / br;
    const int64_t total = (int64_t)n_qtiles * a.B * a.H;
    size_t dyn = 0;
    if (occ > 0) {
        size_t lds = 0;
        const hipError_t e = static_lds(reinterpret_cast<const void*>(kernel), &lds);
        if (e != hipSuccess) return (int)e;
        const size_t share = kLdsPerCu / (size_t)occ;
        if (share > lds) dyn = share - lds;
    }
    hipLaunchKernelGGL(kernel, dim3((unsigned)total), dim3(threads), dyn, st, a, n_qtiles);
    return (int)hipGetLastError();
}

template <typename T, int DP>
static int launch16(const FwdArgs& a, const TileConfig& cfg, bool vec, hipStream_t st) {
    if constexpr (DP <= 128) {
        if (cfg.waves == 8) {  // aligned, d % 8 == 0 (checked by the caller)
            if (a.causal) return launch(fwd16_pp_kernel<T, DP, true>, a, cfg.br, st, 512, cfg.occ);
            return launch(fwd16_pp_kernel<T, DP, false>, a, cfg.br, st, 512, cfg.occ);
        }
    }
    if constexpr (DP <= 128) {
        if (cfg.br == 64) {  // key split in two (small grids)
            if (a.causal)
                return vec ? launch(fwd16_kernel<T, DP, true, true, 2>, a, 64, st, 256, cfg.occ)
                           : launch(fwd16_kernel<T, DP, true, false, 2>, a, 64, st, 256, cfg.occ);
            return vec ? launch(fwd16_kernel<T, DP, false, true, 2>, a, 64, st, 256, cfg.occ)
                       : launch(fwd16_kernel<T, DP, false, false, 2>, a, 64, st, 256, cfg.occ);
        }
    }
    if (a.causal) {
        return vec ? launch(fwd16_kernel<T, DP, true, true, 1>, a, 128, st, 256, cfg.occ)
                   : launch(fwd16_kernel<T, DP, true, false, 1>, a, 128, st, 256, cfg.occ);
    }
    return vec ? launch(fwd16_kernel<T, DP, false, true, 1>, a, 128, st, 256, cfg.occ)
               : launch(fwd16_kernel<T, DP, false, false, 1>, a, 128, st, 256, cfg.occ);
}

template <int DP, int BC>
static int launch32(const FwdArgs& a, const TileConfig& cfg, bool vec, hipStream_t st) {
    if constexpr (DP <= 96) {
        if (cfg.br == 32) {  // key split in four, 32-key tiles (d <= 96: checked by the caller)
            if (a.causal)
                return vec ? launch(fwd32_kernel<DP, 32, true, true, 4>, a, 32, st, 256, cfg.occ)
                           : launch(fwd32_kernel<DP, 32, true, false, 4>, a, 32, st, 256, cfg.occ);
            return vec ? launch(fwd32_kernel<DP, 32, false, true, 4>, a, 32, st, 256, cfg.occ)
                       : launch(fwd32_kernel<DP, 32, false, false, 4>, a, 32, st, 256, cfg.occ);
        }
        if (cfg.br == 64) {  // key split in two (d <= 96: checked by the caller)
            if (a.causal)
                return vec ? launch(fwd32_kernel<DP, BC, true, true, 2>, a, 64, st, 256, cfg.occ)
                           : launch(fwd32_kernel<DP, BC, true, false, 2>, a, 64, st, 256, cfg.occ);
            return vec ? launch(fwd32_kernel<DP, BC, false, true, 2>, a, 64, st, 256, cfg.occ)
                       : launch(fwd32_kernel<DP, BC, false, false, 2>, a, 64, st, 256, cfg.occ);
        }
    }
    if constexpr (DP <= 64) {
        if (cfg.bc == 128) {  // 128-key tiles (16-byte rows: checked by the caller)
            if (a.causal) return launch(fwd32_kernel<DP, 128, true, true, 1>, a, 128, st, 256, cfg.occ);
            return launch(fwd32_kernel<DP, 128, false, true, 1>, a, 128, st, 256, cfg.occ);
        }
    }
    if (a.causal) {
        return vec ? launch(fwd32_kernel<DP, BC, true, true, 1>, a, 128, st, 256, cfg.occ)
                   : launch(fwd32_kernel<DP, BC, true, false, 1>, a, 128, st, 256, cfg.occ);
    }
    return vec ? launch(fwd32_kernel<DP, BC, false, true, 1>, a, 128, st, 256, cfg.occ)
               : launch(fwd32_kernel<DP, BC, false, false, 1>, a, 128, st, 256, cfg.occ);
}

int launch_fwd(const FwdArgs& a, const TileConfig& cfg, bool vec, void* stream) {
    hipStream_t st = (hipStream_t)stream;
    if (a.dtype == 2 || a.dtype == 1) {
        const bool bf = a.dtype == 2;
        switch (cfg.dpad) {
            case 32: return bf ? launch16<__bf16, 32>(a, cfg, vec, st) : launch16<_Float16, 32>(a, cfg, vec, st);
            case 64: return bf ? launch16<__bf16, 64>(a, cfg, vec, st) : launch16<_Float16, 64>(a, cfg, vec, st);
            case 96: return bf ? launch16<__bf16, 96>(a, cfg, vec, st) : launch16<_Float16, 96>(a, cfg, vec, st);
            case 128: return bf ? launch16<__bf16, 128>(a, cfg, vec, st) : launch16<_Float16, 128>(a, cfg, vec, st);
            case 160: return bf ? launch16<__bf16, 160>(a, cfg, vec, st) : launch16<_Float16, 160>(a, cfg, vec, st);
            case 192: return bf ? launch16<__bf16, 192>(a, cfg, vec, st) : launch16<_Float16, 192>(a, cfg, vec, st);
            case 224: return bf ? launch16<__bf16, 224>(a, cfg, vec, st) : launch16<_Float16, 224>(a, cfg, vec, st);
            case 256: return bf ? launch16<__bf16, 256>(a, cfg, vec, st) : launch16<_Float16, 256>(a, cfg, vec, st);
            default: return (int)hipErrorInvalidValue;
        }
    }
    switch (cfg.dpad) {
        case 32: return launch32<32, 64>(a, cfg, vec, st);
        case 64: return launch32<64, 64>(a, cfg, vec, st);
        case 96: return launch32<96, 64>(a, cfg, vec, st);
        case 128: return launch32<128, 32>(a, cfg, vec, st);
        default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fa

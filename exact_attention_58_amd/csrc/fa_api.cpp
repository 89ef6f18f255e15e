// fa_api.cpp -- C-ABI front end: argument checks, tile selection, launch.
//
// Argument checks run before any HIP call, so every error path can be exercised
// without a GPU. The tile selector is a pure function of the sizes and the
// compute-unit count: the analogue of choosing a tile size that fits the
// on-chip memory and failing with an error when none does (page "Flash
// Attention Shared Memory constraint", the group-size search).
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace fa {

namespace {

constexpr int kMaxDim = 256;      // 16-bit forward
constexpr int kMaxDim32 = 128;    // fp32 forward and the backward
constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];  // 0 = not queried yet

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

int dev_num_cus(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_num_cus[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
        v = 256;
    g_num_cus[dev].store(v, std::memory_order_relaxed);
    return v;
}

fa_status check_args(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d) {
    if (dtype != FA_F32 && dtype != FA_F16 && dtype != FA_BF16) return FA_EINVAL;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_EINVAL;
    int64_t bh, t;
    if (!mul_ok(B, H, &bh)) return FA_EINVAL;
    if (!mul_ok(bh, Nq, &t) || !mul_ok(t, d, &t)) return FA_EINVAL;
    if (!mul_ok(bh, Nk, &t) || !mul_ok(t, d, &t)) return FA_EINVAL;
    if (d > kMaxDim || (dtype == FA_F32 && d > kMaxDim32)) return FA_EUNSUPPORTED;
    // 32-bit index arithmetic inside one (batch, head): rows and row*d must fit.
    if (Nq * d > INT32_MAX || Nk * d > INT32_MAX) return FA_EUNSUPPORTED;
    if (B > INT32_MAX || H > INT32_MAX) return FA_EUNSUPPORTED;
    return FA_OK;
}

// Shared tail of fa_fwd and fa_fwd_varlen once the sizes are valid: alignment, tile choice,
// launch. cu_q == nullptr selects the dense layout; otherwise Nq, Nk are the longest lengths.
fa_status run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_q,
                  const int32_t* cu_k, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t tq,
                  int64_t tk, int64_t d, float scale, int causal, fa_dtype dtype, void* stream);

}  // namespace

int select_config(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int causal,
                  int num_cus, bool aligned, TileConfig* out) {
    TileConfig c{};
    c.dpad = (int)((d + 31) / 32) * 32;
    c.waves = 4;
    c.br = 32 * c.waves;
    if (dtype == FA_F32) {
        c.bc = c.dpad > 96 ? 32 : 64;
    } else {
        c.bc = 64;
        // Two-group ping-pong kernel (8 waves, 256 rows) when the inputs allow 16-byte
        // loads, its grid still gives every compute unit a workgroup and the key loop is
        // long enough for its pipeline to pay off. Short key sequences (<= 512, HBM-bound)
        // go to the 4-wave kernel, whose smaller workgroups overlap their loads better
        // (bf16 d=128, N=128: 4.7 vs 2.8 TB/s on MI355X).
        const int64_t wgs256 = (Nq + 255) / 256 * B * H;
        const int64_t wgs128 = (Nq + 127) / 128 * B * H;
        if (d > 128) {
            // head dims past 128: the 4-wave kernel, one wave per SIMD
        } else if (aligned && d % 8 == 0 && wgs256 >= num_cus && Nk > 512) {
            c.waves = 8;
            c.br = 256;
        } else if (!causal && c.dpad <= 96 && wgs128 < num_cus && Nk > 2 * c.bc) {
            // too few 128-row workgroups to fill the chip: 64 rows per workgroup, each row
            // block's keys walked in two halves by two waves and merged at the end
            c.br = 64;
        }
    }
    // The grid must stay within the 32-bit launch limit.
    const int64_t n_qtiles = (Nq + c.br - 1) / c.br;
    if (n_qtiles * B * H > INT32_MAX) return FA_EUNSUPPORTED;
    *out = c;
    return FA_OK;
}

namespace {

fa_status run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, const int32_t* cu_q,
                  const int32_t* cu_k, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t tq,
                  int64_t tk, int64_t d, float scale, int causal, fa_dtype dtype, void* stream) {
    const int esz = dtype == FA_F32 ? 4 : 2;
    if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) % esz != 0 ||
        (uintptr_t)lse % 4 != 0)
        return FA_EINVAL;
    const bool vec = (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) % 16 == 0) &&
                     (d * esz) % 16 == 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FA_ELAUNCH;
    TileConfig cfg;
    int rc = select_config(dtype, B, H, Nq, Nk, d, causal, dev_num_cus(dev), vec, &cfg);
    if (rc != FA_OK) return (fa_status)rc;
    FwdArgs a{};
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    a.B = (int)B;
    a.H = (int)H;
    a.Nq = (int)Nq;
    a.Nk = (int)Nk;
    a.d = (int)d;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.causal = causal ? 1 : 0;
    a.dtype = (int)dtype;
    a.cu_q = cu_q;
    a.cu_k = cu_k;
    a.tq = tq;
    a.tk = tk;
    return launch_fwd(a, cfg, vec, stream) == 0 ? FA_OK : FA_ELAUNCH;
}

}  // namespace

}  // namespace fa

extern "C" {

const char* fa_status_str(fa_status s) {
    switch (s) {
        case FA_OK: return "FA_OK: success";
        case FA_EINVAL: return "FA_EINVAL: invalid argument";
        case FA_EUNSUPPORTED: return "FA_EUNSUPPORTED: no kernel for this request";
        case FA_ELAUNCH: return "FA_ELAUNCH: kernel launch failed";
    }
    return "unknown fa_status";
}

int fa_version(void) { return 1; }

fa_status fa_select_config(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                           int causal, int num_cus, int* Br, int* Bc, int* waves, int* dpad) {
    fa_status st = fa::check_args(dtype, B, H, Nq, Nk, d);
    if (st != FA_OK) return st;
    fa::TileConfig cfg;
    int rc = fa::select_config(dtype, B, H, Nq, Nk, d, causal, num_cus > 0 ? num_cus : 256, true, &cfg);
    if (rc != FA_OK) return (fa_status)rc;
    if (Br) *Br = cfg.br;
    if (Bc) *Bc = cfg.bc;
    if (waves) *waves = cfg.waves;
    if (dpad) *dpad = cfg.dpad;
    return FA_OK;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                 int64_t H, int64_t Nq, int64_t Nk, int64_t d, float scale, int causal,
                 fa_dtype dtype, void* stream) {
    if (!q || !k || !v || !o || !lse) return FA_EINVAL;
    if (!std::isfinite(scale)) return FA_EINVAL;
    fa_status st = fa::check_args(dtype, B, H, Nq, Nk, d);
    if (st != FA_OK) return st;
    return fa::run_fwd(q, k, v, o, lse, nullptr, nullptr, B, H, Nq, Nk, 0, 0, d, scale, causal, dtype,
                       stream);
}

fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t B,
                        int64_t H, int64_t total_q, int64_t total_k, int64_t max_seqlen_q,
                        int64_t max_seqlen_k, int64_t d, float scale, int causal, fa_dtype dtype,
                        void* stream) {
    if (!q || !k || !v || !o || !lse || !cu_seqlens_q || !cu_seqlens_k) return FA_EINVAL;
    if (((uintptr_t)cu_seqlens_q | (uintptr_t)cu_seqlens_k) % 4 != 0) return FA_EINVAL;
    if (!std::isfinite(scale)) return FA_EINVAL;
    if (total_q < 1 || total_k < 1 || max_seqlen_q < 1 || max_seqlen_k < 1 ||
        max_seqlen_q > total_q || max_seqlen_k > total_k)
        return FA_EINVAL;
    // every tensor as one (batch = 1, head) stack of `total` rows, and every sequence as a
    // (batch, head) slice of the longest lengths: both must pass the dense limits
    fa_status st = fa::check_args(dtype, B, H, max_seqlen_q, max_seqlen_k, d);
    if (st != FA_OK) return st;
    st = fa::check_args(dtype, 1, H, total_q, total_k, d);
    if (st != FA_OK) return st;
    return fa::run_fwd(q, k, v, o, lse, cu_seqlens_q, cu_seqlens_k, B, H, max_seqlen_q, max_seqlen_k,
                       total_q, total_k, d, scale, causal, dtype, stream);
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta, int64_t B, int64_t H,
                 int64_t Nq, int64_t Nk, int64_t d, float scale, int causal, fa_dtype dtype,
                 void* stream) {
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA_EINVAL;
    if (!std::isfinite(scale)) return FA_EINVAL;
    fa_status st = fa::check_args(dtype, B, H, Nq, Nk, d);
    if (st != FA_OK) return st;
    const uintptr_t all16 = (uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
                            (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv;
    if (all16 % 2 != 0 || (uintptr_t)lse % 4 != 0 || (uintptr_t)delta % 4 != 0) return FA_EINVAL;
    // the backward kernels exist for the 16-bit types on 16-byte rows, d <= 128, only
    if (dtype == FA_F32 || d % 8 != 0 || d > fa::kMaxDim32 || all16 % 16 != 0) return FA_EUNSUPPORTED;
    fa::BwdArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.dout = dout;
    a.lse = lse;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    a.B = (int)B;
    a.H = (int)H;
    a.Nq = (int)Nq;
    a.Nk = (int)Nk;
    a.d = (int)d;
    a.scale = scale;
    a.scale_log2 = (float)((double)scale * 1.4426950408889634074);
    a.causal = causal ? 1 : 0;
    a.dtype = (int)dtype;
    const int dpad = (int)((d + 31) / 32) * 32;
    return fa::launch_bwd(a, dpad, stream) == 0 ? FA_OK : FA_ELAUNCH;
}

}  // extern "C"

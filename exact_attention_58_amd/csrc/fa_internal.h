// fa_internal.h -- interface between the C-ABI front end (fa_api.cpp) and the
// HIP kernels (fa_fwd_kernels.hip, fa_bwd_kernels.hip). Not installed, not part of the ABI.
#pragma once

#include <stdint.h>

namespace fa {

// Everything a forward kernel needs, already validated by the front end.
struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, Nq, Nk, d;  // packed sequences: Nq, Nk are the longest lengths
    float scale_log2;  // softmax scale times log2(e): scores enter exp2 directly
    int causal;
    int dtype;         // fa_dtype value
    // Packed sequences of different lengths (null for the dense [B,H,N,d] layout): device
    // offsets, B+1 each; tensors are [H, tq, d] (keys [H, tk, d]), lse is [H, tq].
    const int* cu_q;
    const int* cu_k;
    int64_t tq, tk;
    // causal grids: workgroups an XCD takes per group of batch-head pairs in the
    // heaviest-tile-first order (0: the kernel's own, its resident workgroups per XCD)
    int slots;
};

// Tile configuration chosen by the selector.
struct TileConfig {
    int br;     // query rows per workgroup (32 per wave)
    int bc;     // keys per K/V tile
    int waves;  // waves per workgroup
    int dpad;   // head dimension the kernel is compiled for (multiple of 32, >= d)
    // Knobs that leave every result bit-identical:
    int occ;    // at most this many workgroups per CU (1..4), by reserving LDS; 0: no cap
    int group;  // FwdArgs::slots for causal grids (8..1024); 0: the kernel's own
};

// Keys per K/V tile of the 16-bit ping-pong kernel for a padded head dim.
constexpr int pp_keys(int dpad) { return dpad <= 64 ? 128 : 64; }
// Keys per K/V tile of the fp32 kernel: 128 up to d = 64 for 128-row workgroups over
// 16-byte rows, 32 above d = 96 and for the four-way key split (32-row workgroups), else 64
// (the two-way key split and element-wise rows keep 64).
constexpr int f32_keys(int dpad, int br, bool aligned) {
    return dpad > 96 || br == 32 ? 32 : (dpad <= 64 && br == 128 && aligned) ? 128 : 64;
}

// Pure selection logic (no HIP calls). Returns 0 on success, 2 if no kernel fits.
// `aligned`: all buffers 16-byte aligned and d*element_size a multiple of 16.
int select_config(int dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                  int causal, int num_cus, bool aligned, TileConfig* out);

// Launches the kernel for `cfg` on `stream`; returns the hipError_t of the launch as int.
int launch_fwd(const FwdArgs& a, const TileConfig& cfg, bool vec, void* stream);

// Everything the backward kernels need, already validated by the front end (d <= 128).
struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const void* dout;
    const float* lse;
    void* dq;
    void* dk;
    void* dv;
    float* delta;      // [B,H,Nq] workspace: rowsum(dO * O)
    int B, H, Nq, Nk, d;
    float scale;       // softmax scale
    float scale_log2;  // scale times log2(e)
    int causal;
    int dtype;
    int num_cus;       // compute units of the device (the workgroup size of two kernels)
};

// Launches the backward kernels (row terms, dK/dV, dQ) on `stream`; `vec`: every buffer
// 16-byte aligned and d * element size a multiple of 16. Returns the hipError_t as int.
int launch_bwd(const BwdArgs& a, int dpad, bool vec, void* stream);

// The backward's own row-term workspace for callers that cannot allocate: a file-scope device
// array of kBwdScratchFloats fp32 values (4 MiB, one value per query row) that every GPU the
// library runs on holds until the process ends. bwd_scratch() gives its address on the current
// device (resolved once per device); returns the hipError_t as int. Calls that overlap on one
// GPU share the array and race.
constexpr int64_t kBwdScratchFloats = (int64_t)1 << 20;
int bwd_scratch(float** out);

}  // namespace fa

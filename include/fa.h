/*
 * fa.h -- C ABI of the MI355X (gfx950) exact attention forward library.
 *
 * One operation: exact scaled-dot-product attention forward with its per-row
 * logsumexp,
 *
 *     O = softmax(scale * Q K^T + mask) V,      L_i = ln sum_j exp(scale * q_i . k_j)
 *
 * computed tile by tile with the online-softmax recurrence (running row max m,
 * running row sum l, rescaled output accumulator), so the N x N score matrix
 * never reaches device memory. Sources on the pages:
 *   - page "flash_attention_2.cu" (leloykun/flash-hyperbolic-attention-minimal),
 *     forward kernel and its host wrapper: the recurrence m, l, O; the final
 *     O / l and L = m + log(l); the causal guard (key j visible to query i iff
 *     j <= i); the wrapper returning {O, L} for [B, nh, N, d] inputs.
 *   - page "Meta's xFormers has Attention kernel written in CUTLASS": parallel
 *     work over queries as well as batch and heads in the forward pass; fp32
 *     accumulation with a 16-bit output; residual handling for arbitrary
 *     query and key lengths.
 *   - page "Add Fused Multi-Head Attention example" (cuTile.jl PR #16): the
 *     additive -Inf padding mask for keys beyond the key length, and exp2 with
 *     the scale multiplied by 1/ln 2.
 *   - page "Flash Attention Shared Memory constraint" (NNkernels.jl issue #10):
 *     a tile configuration has to fit the on-chip memory, and the library
 *     reports an error when none does.
 *
 * Everything here is plain C; the only HIP type is hipStream_t (passed as
 * void* so that this header needs no HIP include).
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. lse is always fp32. */
typedef enum {
    FA_F32 = 0,  /* IEEE binary32; computed on fp32 MFMA, P kept in fp32      */
    FA_F16 = 1,  /* IEEE binary16; fp16 MFMA operands, fp32 accumulation      */
    FA_BF16 = 2  /* bfloat16; bf16 MFMA operands, fp32 accumulation           */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_EINVAL = 1,       /* bad argument: null pointer, size < 1, unknown dtype,
                            non-finite scale, sizes whose products overflow    */
    FA_EUNSUPPORTED = 2, /* valid request with no kernel for it (d > 256;      
                            fp32 with d > 128)                              */
    FA_ELAUNCH = 3       /* the HIP runtime reported an error at launch        */
} fa_status;

/*
 * fa_fwd -- attention forward on the device, asynchronous on `stream`.
 *
 * Arguments
 *   q      [B, H, Nq, d] device buffer, row-major, element type `dtype`
 *   k, v   [B, H, Nk, d] device buffers, row-major, element type `dtype`
 *   o      [B, H, Nq, d] device buffer written in full, element type `dtype`
 *          (fp32 accumulator rounded to nearest even)
 *   lse    [B, H, Nq] fp32 device buffer written in full: L = m + ln(l), the
 *          natural-log logsumexp of the scaled, masked scores of each row
 *   B, H, Nq, Nk, d   sizes, each >= 1; d <= 256 for fp16/bf16, d <= 128 for fp32
 *   scale  multiplies q . k before the mask and the softmax; any finite value
 *          (0 and negative values included); 1/sqrt(d) is the usual choice
 *   causal 0: every key is visible. non-zero: key j is visible to query i iff
 *          j <= i (top-left alignment, also when Nq != Nk), so every row sees
 *          key 0 and no row is empty
 *   dtype  element type of q, k, v, o
 *   stream hipStream_t to launch on (NULL = the null stream of the current
 *          device). The current HIP device must own all five buffers.
 *
 * Ownership: the caller allocates every buffer; the library allocates
 * nothing, keeps no per-call state and never synchronises. o must not alias
 * q, k or v; lse must not alias anything. Buffers only need the alignment of
 * their element type; 16-byte alignment (and d a multiple of 8 for 16-bit
 * types, of 4 for fp32) enables the vectorised loads.
 *
 * Errors: arguments are checked before any HIP call. FA_EINVAL and
 * FA_EUNSUPPORTED leave o and lse untouched. FA_ELAUNCH is returned when
 * hipGetLastError() reports a failure after the launch.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                 float scale, int causal, fa_dtype dtype, void* stream);

/*
 * fa_fwd_varlen -- attention forward over a packed batch of sequences of different
 * lengths in one launch, asynchronous on `stream`.
 *
 * Page "Meta's xFormers has Attention kernel written in CUTLASS" (the grouped-GEMM
 * discussion) asks for fixed and variable sequence lengths served by one kernel. Each
 * sequence is its own attention problem: its queries see only its own keys, and the causal
 * mask counts positions from the sequence's start (key j visible to query i iff j <= i).
 * A sequence with queries but no keys has an empty softmax sum: its rows get O = 0 and
 * L = -inf.
 *
 * Arguments
 *   q, o   [H, total_q, d] device buffers, row-major, element type `dtype`: every head
 *          holds the B sequences' query rows back to back
 *   k, v   [H, total_k, d] device buffers, row-major, likewise for the key rows
 *   lse    [H, total_q] fp32 device buffer
 *   cu_seqlens_q, cu_seqlens_k   device int32 arrays of B+1 offsets: sequence b owns query
 *          rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
 *          cu_seqlens_k[b+1]-1 of every head. They must start at 0, never decrease, end at
 *          total_q (resp. total_k), and no sequence may be longer than max_seqlen_q (resp.
 *          max_seqlen_k). Zero-length sequences are allowed.
 *   B      number of sequences (>= 1)
 *   H, d, scale, causal, dtype, stream   as for fa_fwd
 *   total_q, total_k           rows per head (>= 1)
 *   max_seqlen_q, max_seqlen_k the longest query and key sequence (1 .. total); they set
 *          the grid, which has a workgroup for every (query tile of the longest sequence,
 *          head, sequence); tiles past a sequence's end return at once.
 *
 * The offsets live on the device, so the library cannot check them without a
 * synchronisation and does not: offsets that break the rules above give unspecified
 * values in o and lse (the kernels clamp every offset into [0, total] and every length to
 * its maximum, so no access leaves the buffers). Rows of o and lse that belong to no
 * sequence are not written.
 *
 * Ownership and errors: as fa_fwd. FA_EINVAL also for null or misaligned offset arrays and
 * for totals or maxima below 1 or maxima above their totals; FA_EUNSUPPORTED for sizes whose
 * dense equivalent (B sequences of the maximum lengths, or one batch of the totals) fa_fwd
 * would reject.
 */
fa_status fa_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int64_t B, int64_t H, int64_t total_q, int64_t total_k,
                        int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t d,
                        float scale, int causal, fa_dtype dtype, void* stream);

/*
 * fa_fwd_config -- fa_fwd with the tile configuration given instead of chosen.
 *
 * Br, Bc, waves: query rows per workgroup, keys per K/V tile and waves per workgroup, as
 * fa_select_config and fa_tune_fwd report them. The kernels that exist: for fp16/bf16,
 * the ping-pong kernel (256, Bc, 8) with Bc = 128 keys for d <= 64 and 64 above, when every
 * buffer is 16-byte aligned, d % 8 == 0 and d <= 128; the 4-wave kernel
 * (128, Bc, 4) and its two-way key split (64, Bc, 4, d <= 128), with Bc = 128 keys for
 * d <= 32, 32 for d > 224 and 64 otherwise. For fp32, (128, 128, 4) for d <= 64 when every
 * buffer is 16-byte aligned and d % 4 == 0, otherwise (128, 64, 4) for d <= 96; (128, 32, 4)
 * above d = 96; and the key splits (64, 64, 4) and (32, 32, 4) when d <= 96. Any other
 * triple returns FA_EUNSUPPORTED before any HIP call.
 * Two knobs change only where and when workgroups run, never a result bit:
 *  - occ (0..4): at most occ workgroups on one CU at a time, by reserving unused LDS
 *    (160 KB / occ per workgroup); 0 = as many as the registers and LDS allow.
 *  - group (0 or 8..1024): causal grids hand each XCD its batch-head pairs in groups, the
 *    longest query tiles of a group first; group is the number of workgroups that such a
 *    group should hold at least (0 = the workgroups the kernel keeps resident per XCD).
 *    Non-causal grids ignore it.
 * Values outside these ranges return FA_EUNSUPPORTED.
 * Everything else (arguments, ownership, errors) is as for fa_fwd; the result is the same
 * up to the order of the fp32 sums.
 */
fa_status fa_fwd_config(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                        float scale, int causal, fa_dtype dtype, int Br, int Bc, int waves,
                        int occ, int group, void* stream);

/*
 * fa_tune_fwd -- measure every tile configuration that exists for this problem and keep
 * the fastest.
 *
 * The pages' kernels pick tile sizes by hand and by search (page "Flash Attention Shared
 * Memory constraint", the group-size search; page "Add Fused Multi-Head Attention example":
 * its Python counterpart searches a space of hand-picked configurations). Here each
 * configuration fa_fwd_config accepts (with both knobs 0) runs once untimed. The first of them then runs
 * untimed for about 20 ms of GPU time, so that the GPU's clock has left its idle state.
 * After that, two rounds time `reps` launches (1..1000) of every configuration between two
 * HIP events on `stream`. Each configuration keeps its faster round. From the fastest, the
 * knobs of fa_fwd_config are then varied one at a time in two more rounds timed the same
 * way: occ = 1 for 4-wave configurations, and for causal problems whose B*H pairs split
 * evenly over the 8 XCDs those of group = 16, 32, 64, 128 that put a different number of
 * pairs in a group than the built-in order does; a variant replaces it only if faster. The result is written to *Br, *Bc, *waves, *occ,
 * *group (each may be NULL) and remembered for this
 * exact problem (current device, dtype, B, H, Nq, Nk, d, causal). Later fa_fwd calls on the
 * same problem launch it instead of the built-in choice, as long as the buffers allow it
 * (a ping-pong or 128-key fp32 choice needs 16-byte aligned buffers). The record holds up to 256 problems;
 * beyond that the oldest is replaced.
 *
 * q, k, v, o, lse, sizes, scale, causal, dtype, stream: as for fa_fwd. On FA_OK, o and lse
 * hold the result of the chosen configuration.
 *
 * Unlike fa_fwd this call blocks: it waits for the timed launches to finish. It creates
 * two HIP events for its own duration and allocates no device memory.
 *
 * Errors: as fa_fwd, plus FA_EINVAL for reps outside 1..1000. FA_ELAUNCH if a launch or
 * an event call fails; the record is then unchanged.
 */
fa_status fa_tune_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                      float scale, int causal, fa_dtype dtype, int reps, void* stream,
                      int* Br, int* Bc, int* waves, int* occ, int* group);

/* Forgets every configuration fa_tune_fwd recorded (all devices). */
void fa_tune_clear(void);

/*
 * fa_bwd -- gradients of the attention forward, asynchronous on `stream`.
 *
 * Given the forward's inputs q, k, v, its outputs o and lse (as fa_fwd wrote them, same
 * scale and causal flag) and the upstream gradient dout = dL/dO, writes
 *     dq = dL/dQ, dk = dL/dK, dv = dL/dV
 * by the updates of the backward kernel on page "flash_attention_2.cu" (backward kernel:
 * D_i = rowsum(dO_i * O_i), P = exp(scale QK^T - L), dV += P^T dO, dP = dO V^T,
 * dS = P (dP - D), dQ += scale dS K, dK += scale dS^T Q), without its atomic adds.
 *
 * Arguments
 *   q, dout, dq     [B, H, Nq, d] device buffers, row-major, element type `dtype`
 *   k, v, dk, dv    [B, H, Nk, d] device buffers, row-major, element type `dtype`
 *   o               [B, H, Nq, d] the forward output, element type `dtype`
 *   lse             [B, H, Nq] fp32, the forward's natural-log logsumexp
 *   delta           [B, H, Nq] fp32 device workspace the call overwrites (rowsum(dO * O))
 *   B, H, Nq, Nk, d, scale, causal, dtype, stream   as for fa_fwd
 *
 * dq, dk, dv are written in full (fp32 accumulation, rounded to nearest even); keys that no
 * query sees (causal with Nk > Nq) get zero gradients. The caller allocates every buffer,
 * including the workspace; the library allocates nothing. dq, dk, dv and delta must not
 * alias each other or any input.
 *
 * Every dtype of fa_fwd is served, with 1 <= d <= 128: fp32 inputs on fp32 MFMA with P and dS
 * kept in fp32; fp16/bf16 inputs with P and dS rounded to the input type for the products that
 * consume them. Buffers need only their element's alignment; 16-byte aligned buffers with
 * d * element size a multiple of 16 take vectorised loads.
 *
 * Errors: as fa_fwd (checked before any HIP call), plus FA_EINVAL for a null or misaligned
 * delta, and FA_EUNSUPPORTED for d > 128.
 */
fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv, float* delta,
                 int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                 float scale, int causal, fa_dtype dtype, void* stream);

/*
 * fa_bwd_noalloc -- fa_bwd without the caller's workspace, for callers that cannot allocate
 * device memory or pass one (code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation).
 *
 * Same arguments, results and errors as fa_bwd minus `delta`: the row terms live in a
 * file-scope device array of the library (4 MiB, one fp32 per query row) that each GPU the
 * library runs on holds until the process ends; its address is looked up once per device on
 * the first call there. The call itself allocates nothing.
 *
 * Limit: B * H * Nq <= 1048576 query rows; larger requests return FA_EUNSUPPORTED before any
 * HIP call. The array is overwritten in full by every call before it is read, so nothing has
 * to be cleared, but all calls on one GPU share it: calls that overlap on one GPU (two
 * streams, two threads) race and give undefined gradients. FA_ELAUNCH also when the array's
 * device address cannot be obtained.
 */
fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d,
                         float scale, int causal, fa_dtype dtype, void* stream);

/*
 * fa_status_str -- static description of a status code (never NULL). The error classes
 * follow page "Flash Attention Shared Memory constraint", where the library reports an error
 * instead of running when no tile configuration fits the request: FA_EUNSUPPORTED is that
 * case here, kept apart from malformed arguments (FA_EINVAL) and runtime failures
 * (FA_ELAUNCH).
 */
const char* fa_status_str(fa_status s);

/*
 * fa_select_config -- the tile configuration fa_fwd would launch on the current device for
 * these sizes, without launching anything: the query rows per workgroup (*Br), the keys per
 * K/V tile (*Bc) and the waves per workgroup (*waves). Any output pointer may be NULL.
 *
 * Page "Flash Attention Shared Memory constraint" searches for a tile size that fits the
 * on-chip memory and fails with an error when none does; page "Add Fused Multi-Head
 * Attention example" picks its tile sizes per problem. Here the choice is a function of the
 * sizes and of the device's compute-unit count, which is read from the current HIP device
 * (once per device, cached); with no device visible it assumes MI355X's 256. It is
 * fa_select_config_cus with that count and the padded head dimension dropped. The answer
 * assumes 16-byte aligned buffers; fa_fwd on unaligned buffers (or a 16-bit d that is not a
 * multiple of 8) uses the 4-wave, 128-row kernel (for fp32 with 64-key tiles up to d = 96),
 * and a configuration recorded by fa_tune_fwd for the same problem replaces it.
 *
 * Errors: FA_EINVAL / FA_EUNSUPPORTED exactly as fa_fwd for the same sizes and dtype.
 */
fa_status fa_select_config(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                           int64_t d, int causal, int* Br, int* Bc, int* waves);

/*
 * fa_select_config_cus -- the same choice as a pure function of the sizes and a given
 * compute-unit count `num_cus` (<= 0 means 256), with no HIP call at all, so that the rules
 * can be checked for any device on a machine without one. Also writes the padded head
 * dimension the kernel is compiled for (*dpad, a multiple of 32). The rules:
 *  - fp16/bf16: the two-group ping-pong kernel (256 rows, 8 waves; 128-key tiles up to
 *    d = 64, 64-key tiles above) for aligned rows with d % 8 == 0 and 32 < d <= 128, when
 *    its grid has at least 5/8 of a workgroup per CU (one per CU for causal grids) and the
 *    key length passes the crossover (more than 512 keys, or 1536 for d <= 96 on grids of at
 *    least three 128-row workgroups per CU; causal: more than 2048, or for d <= 64 more than
 *    2560, 4096 on grids of at least eight 128-row workgroups per CU),
 *    except causal grids with d <= 96 and at most two 128-row workgroups per
 *    CU; otherwise the 4-wave kernel (128 rows; 128-key tiles up to d = 32, 32-key tiles
 *    above d = 224), or its two-way key split (64 rows, d <= 128) for grids of at most one
 *    128-row workgroup per CU (1.5 for d <= 64; two for causal grids).
 *  - fp32: one 4-wave kernel per head dim (128 rows; 128-key tiles up to d = 64, 64-key
 *    tiles up to d = 96, 32-key tiles above), or its two-way key split (64 rows, d <= 96)
 *    below two 128-row workgroups per CU (one per CU for non-causal d > 64, four per CU
 *    for causal grids), and within that its four-way split (32 rows, 32-key tiles) for
 *    grids of at most one 32-row workgroup per CU (causal grids: four, two for d = 96).
 * The scheduling knobs of fa_fwd_config that the built-in rules set (dispatch groups of 128
 * for the causal fp32 two-way key split and for causal 16-bit 4-wave grids up to d = 32, and
 * one workgroup per CU for causal fp32 grids above d = 96 with at most two 128-row
 * workgroups per CU) are not reported; they change no result bit.
 */
fa_status fa_select_config_cus(fa_dtype dtype, int64_t B, int64_t H, int64_t Nq, int64_t Nk,
                               int64_t d, int causal, int num_cus,
                               int* Br, int* Bc, int* waves, int* dpad);

/*
 * fa_version -- the library's interface version (2: fa_select_config with the signature
 * above, fa_select_config_cus and fa_bwd_noalloc). The Python binding refuses a library
 * older than the interface it was written for. Versioning an ABI is the library's own
 * practice; the pages prescribe none.
 */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */

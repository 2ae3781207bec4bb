/* Top-k sparse multi-query attention, forward and backward, for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libsparse_mqa.so. Every function takes plain device pointers, sizes and a HIP
 * stream (passed as void*, a hipStream_t; NULL = the default stream), enqueues its kernels on
 * that stream and returns an int status (SMQA_OK = 0). Nothing here allocates, frees or
 * synchronises; the caller owns every buffer. All tensors are dense, contiguous, row-major,
 * in exactly the layouts below; bf16 tensors are passed as raw 16-bit words.
 *
 * The operation is the one documented on two NeMo AutoModel DeepSeek-V4 kernel pages:
 * "...kernels.tilelang_sparse_mla_fwd" (API entry sparse_mqa_fwd_interface) and
 * "...kernels.tilelang_sparse_mla_bwd" (API entry sparse_mqa_bwd_interface and the
 * preprocess / bwd / postprocess factories). For batch b, token s, head h, and slot t with
 * i = topk_idxs[b,s,t]:
 *   - slot t takes part iff 0 <= i < S_kv; any other value (negative, >= S_kv) is masked
 *     and its kv row is never read (fwd page, topk_idxs note);
 *   - score z_t = sm_scale * <q[b,s,h,:], kv[b,i,:]>; kv is both key and value (kv note);
 *   - the softmax denominator is Z = sum_t exp(z_t) + exp(attn_sink[h]) (attn_sink note);
 *   - O[b,s,h,:] = sum_t exp(z_t)/Z * kv[b,i,:] (bf16), LSE[b,s,h] = log2 Z (fp32; the
 *     reference_rounding note says the kept LSE is base 2);
 *   - sm_scale: a NaN value selects the default D^-0.5 (sm_scale note).
 * A token with no valid slot gets O = 0; its LSE is attn_sink[h]*log2(e), or -inf if the sink
 * is -inf. Duplicate indices within a token count once per slot.
 * Backward (bwd page): given dO, the forward's bf16 O and fp32 LSE,
 *   Delta = <O, dO>, P_t = 2^(z_t*log2 e - LSE), dS_t = P_t*(<dO, kv_i> - Delta),
 *   dQ = sm_scale * sum_t dS_t kv_i (bf16), dKV[b,j,:] = sum over (s,t) with i = j of
 *   sum_h (sm_scale*dS_t*q[b,s,h,:] + P_t*dO[b,s,h,:]), accumulated in fp32 (accum_dtype)
 *   and returned as bf16, or as the fp32 accumulator itself (return_dkv_accum_dtype).
 *
 * Shapes (all int64): B batch, S query tokens, S_kv kv rows, H heads, D head dim, topk slots.
 *   q, O, dO, dQ : [B, S, H, D] bf16       kv, dKV  : [B, S_kv, D] bf16 (dKV fp32 if asked)
 *   attn_sink    : [H] fp32                topk_idxs: [B, S, topk] int32
 *   LSE, Delta   : [B, S, H] fp32          dKV accumulator: [B, S_kv, D] fp32
 * Supported (H, D): D in {128, 256, 512} with H in {16, 32} or any multiple of 64 up to 1024; D = 64 with H in
 * {16, 32}.
 * 1 <= topk <= 2^30, S_kv <= 2^31 - 1, B*S*max(1, H/64) < 2^23 (one workgroup of up to 512
 * threads per token and block of 64 heads, and a launch holds fewer than 2^32 threads).
 * Pointers to bf16 tensors (q, kv, O, dO, dQ, dKV), the fp32 dKV accumulator and the workspace
 * must be 16-byte aligned; fp32 vectors (attn_sink, LSE, Delta) and topk_idxs 4-byte aligned.
 * Outputs must not overlap inputs or each other (SMQA_ERR_ALIAS).
 * Out-of-range indices are data, not errors. Results are undefined if q, kv or dO hold
 * non-finite values. Calls on one stream are ordered; concurrent calls writing the same
 * outputs race.
 */
#ifndef SPARSE_MQA_H
#define SPARSE_MQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SMQA_OK = 0,
  SMQA_ERR_NULL = 1,        /* a required pointer is NULL */
  SMQA_ERR_SHAPE = 2,       /* a size is <= 0 or beyond a stated limit */
  SMQA_ERR_UNSUPPORTED = 3, /* (H, D) has no compiled kernel, or one batch's kv rows
                               (S_kv * D * 2 bytes) reach 4 GiB */
  SMQA_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned */
  SMQA_ERR_ALIAS = 5,       /* an output overlaps an input or another output */
  SMQA_ERR_WORKSPACE = 6,   /* workspace missing or smaller than sparse_mqa_bwd_workspace_bytes */
  SMQA_ERR_HIP = 7,         /* a kernel launch failed (hipGetLastError) */
  SMQA_ERR_ARG = 8          /* another invalid argument (e.g. a non-finite, non-NaN sm_scale) */
};

/* Forward (fwd page, sparse_mqa_fwd_interface). Reads q, kv, attn_sink, topk_idxs; writes
 * o [B,S,H,D] bf16 and lse [B,S,H] fp32 (log2 units). sm_scale = NaN selects D^-0.5.
 * reference_rounding (fwd page, the option of that name): 0 forms each score as
 * fp32(dot * fp32(sm_scale * log2 e)) and runs the softmax in base 2; 1 rounds the scaled logit
 * fp32(dot * sm_scale) in natural units, subtracts the running max there and only then changes
 * to base 2 for the exponential; LSE is log2 units in both. Other values: SMQA_ERR_ARG. */
int sparse_mqa_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs,
                   void* o, float* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                   int64_t topk, float sm_scale, int reference_rounding, void* stream);

/* Backward workspace. sparse_mqa_bwd and sparse_mqa_bwd_dkv take a device workspace: Delta
 * [B,S,H] fp32 (sparse_mqa_bwd only), the kv row norms (which bound dS, so that dS can enter the
 * dKV product as a scaled fp16 operand), the staging plan (one bit per kv row and token of a
 * chunk, with pair counts and scanned offsets), and the staging rows of the
 * segmented dKV scatter-add (one row per valid (token, slot) pair and 64-head block, and one spare
 * row per token and head block that absorbs the stores of masked slots; a row is D int16 values
 * with one power-of-two exponent per segment of up to 128 values -- block floating point -- summed
 * in fp32).
 * sparse_mqa_bwd_workspace_bytes is the size for one pass over all tokens (an upper bound that
 * assumes every slot valid); any size >= sparse_mqa_bwd_workspace_min_bytes also works (the smaller
 * of that and token chunks of one with an fp32 running sum), and the tokens are then processed in
 * the largest chunks that fit. Both return 0 for invalid sizes. */
size_t sparse_mqa_bwd_workspace_bytes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                                      int64_t topk);
size_t sparse_mqa_bwd_workspace_min_bytes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                                          int64_t topk);

/* Backward (bwd page, sparse_mqa_bwd_interface): preprocess (Delta), the dKV kernel with its
 * segmented scatter-add and per-row reduction (which also performs the fp32 -> bf16
 * postprocess), and dQ: at D = 512 with H a multiple of 64 from the dS the dKV kernel stores in
 * the workspace, otherwise from a kernel that recomputes S and dP. dq [B,S,H,D] bf16. dkv [B,S_kv,D]: bf16 if dkv_fp32 == 0, else fp32 (the
 * fp32 sums themselves). The call overwrites dq and dkv; it never accumulates into them. Rows no
 * valid slot references come out exactly 0. attn_sink is accepted for the documented signature;
 * the LSE already includes the sink, so dQ and dKV do not read it. Results are bitwise
 * reproducible from call to call as long as no token lists a kv row twice (top-k selections never
 * do): nothing in the staged path depends on the order in which workgroups run.
 * Precondition on lse (as the bwd page's parameter list implies, it is the forward's output for
 * the same q, kv, attn_sink, topk_idxs and sm_scale): lse[b,s,h] must be at least log2 of the
 * head's softmax denominator, so that every P_t <= 1. The dKV kernels size the fixed-point range of
 * their fp16 dS operand from that (and from Delta and the kv row norms); a smaller lse makes P
 * exceed 1, and dS values beyond the range are then saturated (wrong dKV, status still SMQA_OK).
 * o enters only through Delta and may be any bf16 tensor. */
int sparse_mqa_bwd(const void* q, const void* kv, const float* attn_sink, const void* o,
                   const void* d_o, const int32_t* topk_idxs, const float* lse, void* dq, void* dkv,
                   int dkv_fp32, void* workspace, size_t workspace_bytes, int64_t B, int64_t S,
                   int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale, void* stream);

/* Size of the static scratch of sparse_mqa_bwd_noalloc: 128 MiB per device. */
#define SMQA_BWD_SCRATCH_BYTES ((size_t)128 << 20)

/* sparse_mqa_bwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same computation and results, with
 * the workspace taken from a static device array of SMQA_BWD_SCRATCH_BYTES that the library holds
 * on each device it runs on until the process ends. The call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine); the caller still passes every input and output.
 * - Sizes whose smallest workspace (sparse_mqa_bwd_workspace_min_bytes) exceeds
 *   SMQA_BWD_SCRATCH_BYTES are refused with SMQA_ERR_WORKSPACE before anything is enqueued; sizes
 *   whose one-pass workspace (sparse_mqa_bwd_workspace_bytes) exceeds it run in token chunks, so
 *   dkv may differ from sparse_mqa_bwd's one-pass result in fp32 summation order.
 * - The stream must belong to the current device (else SMQA_ERR_ARG); the first call on a device
 *   looks up that device's copy of the array (hipGetSymbolAddress).
 * - Every call on one device shares that device's array: calls that overlap in time on one device
 *   (different streams, or different threads without ordering) race and give wrong results. The
 *   kernels clear what they need, so the array's contents from an earlier call do not matter.
 * Other arguments, statuses and results as for sparse_mqa_bwd. */
int sparse_mqa_bwd_noalloc(const void* q, const void* kv, const float* attn_sink, const void* o,
                           const void* d_o, const int32_t* topk_idxs, const float* lse, void* dq,
                           void* dkv, int dkv_fp32, int64_t B, int64_t S, int64_t S_kv, int64_t H,
                           int64_t D, int64_t topk, float sm_scale, void* stream);

/* Stage: Delta[b,s,h] = sum_d O*dO in fp32 (bwd page, preprocess factory). */
int sparse_mqa_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t B, int64_t S,
                              int64_t H, int64_t D, void* stream);

/* Gradient of the attention sink (bwd page: attn_sink is an input of the backward; fwd page:
 * the sink is a per-head denominator bias with no value vector). With p_sink = exp(sink_h) / Z =
 * 2^(sink_h log2 e - LSE) and Delta = <O, dO> (sparse_mqa_bwd_preprocess):
 *   d_sink[h] = -sum_{b,s} 2^(sink_h log2 e - lse[b,s,h]) * delta[b,s,h]        (fp32)
 * lse and delta are [B,S,H] fp32, attn_sink and d_sink [H] fp32; a -inf sink gets 0. The
 * reduction order is fixed (deterministic). d_sink must not overlap the inputs. */
int sparse_mqa_bwd_dsink(const float* lse, const float* delta, const float* attn_sink, float* d_sink, int64_t B,
                         int64_t S, int64_t H, void* stream);

/* Stage: dQ alone (bwd page, bwd factory): writes dq (bf16) from q, kv, dO, indices, LSE, Delta. */
int sparse_mqa_bwd_dq(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                      const float* lse, const float* delta, void* dq, int64_t B, int64_t S,
                      int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale, void* stream);

/* Stage: dKV alone (bwd page, bwd and postprocess factories) with the segmented scatter-add:
 * writes dkv (bf16, or fp32 if dkv_fp32) completely. Workspace as for sparse_mqa_bwd without the
 * Delta part (sparse_mqa_bwd_workspace_bytes minus Delta's bytes is enough for one pass). */
int sparse_mqa_bwd_dkv(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                       const float* lse, const float* delta, void* dkv, int dkv_fp32, void* workspace,
                       size_t workspace_bytes, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                       int64_t topk, float sm_scale, void* stream);

/* The steps of sparse_mqa_bwd's staged pass over all tokens, for callers that schedule or time them
 * separately (bwd page, bwd factory: the dKV scatter-add, and dQ). They need a workspace that holds
 * every token (at least sparse_mqa_bwd_workspace_bytes minus Delta's bytes; SMQA_ERR_WORKSPACE
 * otherwise) and must run in this order with the same workspace and sizes:
 *   prepare   marks every valid (token, kv row) pair in a bitmap and gives each valid slot its
 *             staging row: a kv row's rows are contiguous, in an order fixed by the
 *             token indices;
 *   partials  computes every valid slot's dKV contribution row into the staging rows; at D = 512
 *             with H a multiple of 64 it also stores dS = P (dP - Delta) (bf16) in the workspace;
 *   dq        (sparse_mqa_bwd_dkv_dq; D = 512 with H a multiple of 64, else SMQA_ERR_UNSUPPORTED)
 *             writes dq [B,S,H,D] bf16 = sm_scale * sum_t dS_t kv_i from that dS and the kv rows;
 *   reduce    sums each kv row's staging rows and writes dkv (bf16, or fp32 if dkv_fp32).
 * dq and reduce may run in either order after partials. prepare reads only topk_idxs, so it may
 * run on another stream, e.g. beside the forward, as long as the caller orders it after the
 * workspace's previous use and before partials (events); the other steps go on one stream. */
int sparse_mqa_bwd_dkv_prepare(const int32_t* topk_idxs, void* workspace, size_t workspace_bytes,
                               int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                               void* stream);
int sparse_mqa_bwd_dkv_partials(const void* q, const void* kv, const void* d_o,
                                const int32_t* topk_idxs, const float* lse, const float* delta,
                                void* workspace, size_t workspace_bytes, int64_t B, int64_t S,
                                int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                                void* stream);
int sparse_mqa_bwd_dkv_dq(const void* kv, const int32_t* topk_idxs, void* dq, void* workspace,
                          size_t workspace_bytes, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                          int64_t topk, float sm_scale, void* stream);
int sparse_mqa_bwd_dkv_reduce(void* dkv, int dkv_fp32, void* workspace, size_t workspace_bytes,
                              int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                              void* stream);

/* Stage, workspace-free variant of the main backward (bwd page, bwd factory: its fp32 accumulator
 * [B,S_kv,D], accum_dtype, that the postprocess factory then converts): writes dq and adds every
 * valid slot's dKV contribution into dkv_accum [B,S_kv,D] fp32 with fp32 atomic adds. dkv_accum
 * must be zeroed by the caller first; rows no slot references are untouched. Slower than the staged
 * path on MI355X (the fp32 atomic rate bounds it) but needs no staging memory. The order of the
 * atomic adds, and so the last bits of dkv_accum, may vary from call to call. */
int sparse_mqa_bwd_main(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                        const float* lse, const float* delta, void* dq, float* dkv_accum, int64_t B,
                        int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                        void* stream);

/* Stage: dkv[b,j,d] = bf16(dkv_accum[b,j,d]) with round-to-nearest-even (bwd page,
 * postprocess factory). */
int sparse_mqa_bwd_postprocess(const float* dkv_accum, void* dkv, int64_t B, int64_t S_kv,
                               int64_t D, void* stream);

/* Static string naming a status code. */
const char* sparse_mqa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_MQA_H */

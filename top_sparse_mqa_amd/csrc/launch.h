// Kernel launchers behind the C ABI. Arguments arrive validated (abi.cpp); these only pick
// the compiled instance and enqueue on the given stream.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smqa {

struct FwdArgs {
  const void* q;
  const void* kv;
  const float* sink;
  const int32_t* idx;
  void* o;
  float* lse;
  int64_t B, S, S_kv, H, D, topk;
  float sm_scale;
  int reference_rounding;  // 1: fp32 scaled logits in natural units (fwd page option)
};

struct BwdMainArgs {
  const void* q;
  const void* kv;
  const void* d_o;
  const int32_t* idx;
  const float* lse;
  const float* delta;
  void* dq;
  float* dkv_accum;       // atomic mode: pre-zeroed fp32 accumulator [B,S_kv,D]
  const int32_t* pos;     // staging mode: staging row of each slot of the chunk (-1 if masked)
  uint16_t* stage;        // staging mode: contribution rows (int16 block floating point); nullptr: atomic mode
  int8_t* stage_exp;      // staging mode: one power-of-two exponent per row segment (stage_segments)
  const float* row_norm;  // staging mode: |kv_r| of every kv row (launch_kv_row_norm)
  int64_t B, S, S_kv, H, D, topk;
  float sm_scale;
  int64_t token0;         // first token of the chunk (dKV kernel)
  int64_t n_chunk;        // tokens in the chunk (dKV kernel)
  uint16_t* ds = nullptr; // staging mode at D = 512 with 64-head blocks: the dKV kernel also stores
                          // dS (bf16, [chunk token][head block][32-slot block][64][32]) here
};

// The dS store and the dQ kernel that reads it (bwd_dq_ds_kernel) serve D = 512 with H a multiple of
// 64; other shapes compute dQ with the recompute kernel.
inline bool dq_from_ds(int64_t H, int64_t D) { return D == 512 && H % 64 == 0; }
// Bytes of the dS store for n_chunk tokens.
inline int64_t ds_bytes(int64_t n_chunk, int64_t H, int64_t topk) {
  return n_chunk * (H / 64) * ((topk + 31) / 32) * 64 * 32 * 2;
}

// Heads handled by one backward workgroup, and workgroups per token.
inline int bwd_heads_per_wg(int64_t H) { return H >= 64 ? 64 : (int)H; }
inline int bwd_hblocks(int64_t H) { return (int)(H / bwd_heads_per_wg(H)); }
// Exponent segments per staging row: one per min(128, d-range of a backward wave) values.
inline int stage_segments(int64_t H, int64_t D) {
  const int64_t dw = D / (bwd_heads_per_wg(H) / 16);
  return (int)(D / (dw < 128 ? dw : 128));
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t rows, int64_t D,
                                 hipStream_t st);
hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st);
// norm[r] = |kv_r| (fp32) for rows kv[0 .. rows) of D bf16.
hipError_t launch_kv_row_norm(const void* kv, int64_t rows, int64_t D, float* norm, hipStream_t st);
// d_sink[h] = -sum_t 2^(sink_h log2 e - lse[t,h]) * delta[t,h] over tokens t (one workgroup per head).
hipError_t launch_bwd_dsink(const float* lse, const float* delta, const float* sink, float* d_sink, int64_t tokens,
                            int64_t H, hipStream_t st);
// which: 1 = dQ kernel (all tokens), 2 = dKV kernel (chunk; atomic or staging mode), 3 = both.
hipError_t launch_bwd_main(const BwdMainArgs& a, int which, hipStream_t st);
// dQ of the chunk's tokens [a.token0, a.token0 + a.n_chunk) from the dS the dKV kernel stored in a.ds
// (dq_from_ds shapes only).
hipError_t launch_bwd_dq_ds(const BwdMainArgs& a, hipStream_t st);
// Staging-row assignment for the tokens [token0, token0 + n_chunk). `plan` holds 3 *
// dkv_bitmap_words 32-bit words: {bitmap word, pair count} per word, then the cursors (written or
// cleared here). Marks every valid
// (token, kv row) pair, scans the words' pair counts into offset[0 .. words] and writes each valid
// slot's first staging row into pos (-1 for masked slots). Positions depend on the indices only
// unless a token selects a row more than once.
hipError_t launch_dkv_prepare(const int32_t* idx, uint32_t* plan, int32_t* offset, int32_t* tile_sum, int32_t* pos,
                              int64_t B, int64_t S, int64_t S_kv, int64_t topk, int n_hblk, int64_t token0,
                              int64_t n_chunk, hipStream_t st);
int64_t scan_tiles(int64_t n);
// Words of the selection bitmap per kv row for a chunk of n_chunk tokens: a row takes bits from the
// tokens of its own batch only, so ceil(min(n_chunk, S) / 32). dkv_bitmap_words: for n_rows rows,
// also the number of scanned offsets before the final total.
int64_t dkv_row_words(int64_t n_chunk, int64_t S);
int64_t dkv_bitmap_words(int64_t n_rows, int64_t n_chunk, int64_t S);
// Per kv row: sum of its staging segment [offset[row * stride], offset[(row + 1) * stride])
// (+ acc if accumulate); writes acc (fp32) and/or out (bf16).
hipError_t launch_reduce_rows(const uint16_t* stage, const int8_t* stage_exp, int nseg, const int32_t* offset,
                              int64_t stride, float* acc, void* out_bf16, int accumulate, int64_t n_rows, int64_t D,
                              hipStream_t st);
hipError_t launch_bwd_postprocess(const float* acc, void* dkv, int64_t n, hipStream_t st);

}  // namespace smqa

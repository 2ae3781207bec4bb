// CPU oracle for top-k sparse multi-query attention, forward and backward.
//
// TEST INFRASTRUCTURE ONLY. This file is the correctness reference that the HIP
// kernels are checked against. Only the tests, the smoke check and the bench's
// cpu_baseline leg may load it; the product path (top_sparse_mqa_amd) never does.
// It shares no code, header, table or helper with the HIP library.
//
// What it computes follows two NeMo AutoModel DeepSeek-V4 kernel pages:
//   page "...kernels.tilelang_sparse_mla_fwd", API entry sparse_mqa_fwd_interface and its
//     parameter notes (q, kv, attn_sink, topk_idxs, sm_scale, reference_rounding, Returns);
//   page "...kernels.tilelang_sparse_mla_bwd", API entry sparse_mqa_bwd_interface with its
//     parameter list, and the factories preprocess / bwd / postprocess (accum_dtype).
// The pages print no formulas. The definitions below are the plain reading of those
// parameter notes (each reading is listed in the design notes):
//   for batch b, query token s, head h, slot t with i = topk_idxs[b,s,t]:
//     slot t takes part  <=>  0 <= i < S_kv          (topk_idxs note: other values are masked)
//     z_t   = sm_scale * <q[b,s,h,:], kv[b,i,:]>     (kv note: one tensor serves as keys and values)
//     Z     = sum_{valid t} exp(z_t) + exp(attn_sink[h])   (attn_sink note: a per-head term in
//                                                       the softmax denominator)
//     O     = sum_{valid t} exp(z_t) / Z * kv[b,i,:]
//     LSE   = log2(Z)                                (reference_rounding note: the LSE the forward
//                                                       keeps for the backward is base 2)
//   backward of L(q, kv) with dL/dO = dO, given O (bf16, as passed in) and LSE:
//     P_t   = 2^(z_t * log2(e) - LSE),   dP_t = <dO[b,s,h,:], kv[b,i,:]>
//     Delta = <O[b,s,h,:], dO[b,s,h,:]>              (the preprocess step)
//     dS_t  = P_t * (dP_t - Delta)
//     dQ[b,s,h,:] = sm_scale * sum_{valid t} dS_t * kv[b,i,:]
//     dKV[b,j,:]  = sum_{s,t : i = j} sum_h ( sm_scale * dS_t * q[b,s,h,:] + P_t * dO[b,s,h,:] )
//
// Every input arrives already widened to the working precision R (bf16 -> fp32 is
// exact; the caller does it). R = float is the fp32-accumulation instance the pages
// name (accum_dtype = float32); R = double is used for finite differences and as a
// cross-check. Sums over d run in ascending d; sums over slots in ascending t. The file is
// built with -ffp-contract=off: each multiply and each add rounds on its own, as written.
// OpenMP parallelises over independent tokens (forward, dQ) or independent kv rows
// (dKV); no result depends on the thread count.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <vector>
#include <omp.h>

namespace {

constexpr double kLog2e = 1.4426950408889634073599246810019;

inline bool in_range(int32_t i, int64_t S_kv) { return i >= 0 && (int64_t)i < S_kv; }

struct Shape {
  int64_t B, S, S_kv, H, D, topk;
};

// Forward for one token (b, s): O[H][D] and LSE[H] (log2 units).
template <class R>
void fwd_token(const Shape& sh, const R* q, const R* kv, const float* sink, const int32_t* idx,
               R sm_scale, int64_t token, R* o_out, R* lse_out) {
  const int64_t H = sh.H, D = sh.D, K = sh.topk;
  const int64_t b = token / sh.S;
  const R* q_tok = q + token * H * D;
  const int32_t* idx_tok = idx + token * K;
  const R* kv_b = kv + b * sh.S_kv * D;

  // q transposed to [D][H] so the head loop is innermost; each score still sums over d in order.
  std::vector<R> qT(D * H);
  for (int64_t h = 0; h < H; h++)
    for (int64_t d = 0; d < D; d++) qT[d * H + h] = q_tok[h * D + d];

  std::vector<R> z(K * H, R(0));
  std::vector<char> valid(K);
  for (int64_t t = 0; t < K; t++) {
    valid[t] = in_range(idx_tok[t], sh.S_kv);
    if (!valid[t]) continue;
    const R* row = kv_b + (int64_t)idx_tok[t] * D;
    R* zt = &z[t * H];
    for (int64_t d = 0; d < D; d++) {
      const R kd = row[d];
      for (int64_t h = 0; h < H; h++) zt[h] += qT[d * H + h] * kd;
    }
    for (int64_t h = 0; h < H; h++) zt[h] *= sm_scale;
  }

  std::vector<R> acc(D);
  for (int64_t h = 0; h < H; h++) {
    const R s_h = (R)sink[h];
    R m = s_h;
    for (int64_t t = 0; t < K; t++)
      if (valid[t] && z[t * H + h] > m) m = z[t * H + h];
    R* o = o_out + h * D;
    if (m == -std::numeric_limits<R>::infinity()) {
      // no valid slot and a -inf sink: the denominator is empty; output zero, LSE -inf.
      for (int64_t d = 0; d < D; d++) o[d] = R(0);
      lse_out[h] = -std::numeric_limits<R>::infinity();
      continue;
    }
    R l = std::exp(s_h - m);
    for (int64_t d = 0; d < D; d++) acc[d] = R(0);
    for (int64_t t = 0; t < K; t++) {
      if (!valid[t]) continue;
      const R w = std::exp(z[t * H + h] - m);
      l += w;
      const R* row = kv_b + (int64_t)idx_tok[t] * D;
      for (int64_t d = 0; d < D; d++) acc[d] += w * row[d];
    }
    for (int64_t d = 0; d < D; d++) o[d] = acc[d] / l;
    lse_out[h] = (m + std::log(l)) * (R)kLog2e;
  }
}

// dQ and Delta for one token.
template <class R>
void dq_token(const Shape& sh, const R* q, const R* kv, const R* o, const R* dout, const int32_t* idx,
              const R* lse, R sm_scale, int64_t token, R* dq_out, R* delta_out) {
  const int64_t H = sh.H, D = sh.D, K = sh.topk;
  const int64_t b = token / sh.S;
  const R* q_tok = q + token * H * D;
  const R* do_tok = dout + token * H * D;
  const R* o_tok = o + token * H * D;
  const int32_t* idx_tok = idx + token * K;
  const R* kv_b = kv + b * sh.S_kv * D;
  const R* lse_tok = lse + token * H;

  std::vector<R> delta(H);
  for (int64_t h = 0; h < H; h++) {
    R a = 0;
    for (int64_t d = 0; d < D; d++) a += o_tok[h * D + d] * do_tok[h * D + d];
    delta[h] = a;
    if (delta_out) delta_out[h] = a;
  }

  std::vector<R> qT(D * H), doT(D * H);
  for (int64_t h = 0; h < H; h++)
    for (int64_t d = 0; d < D; d++) {
      qT[d * H + h] = q_tok[h * D + d];
      doT[d * H + h] = do_tok[h * D + d];
    }

  std::vector<R> z(H), dp(H), acc(H * D, R(0));
  for (int64_t t = 0; t < K; t++) {
    if (!in_range(idx_tok[t], sh.S_kv)) continue;
    const R* row = kv_b + (int64_t)idx_tok[t] * D;
    for (int64_t h = 0; h < H; h++) z[h] = dp[h] = R(0);
    for (int64_t d = 0; d < D; d++) {
      const R kd = row[d];
      for (int64_t h = 0; h < H; h++) {
        z[h] += qT[d * H + h] * kd;
        dp[h] += doT[d * H + h] * kd;
      }
    }
    for (int64_t h = 0; h < H; h++) {
      const R score = z[h] * sm_scale;
      const R p = std::exp2(score * (R)kLog2e - lse_tok[h]);
      const R ds = p * (dp[h] - delta[h]);
      R* a = &acc[h * D];
      for (int64_t d = 0; d < D; d++) a[d] += ds * row[d];
    }
  }
  for (int64_t i = 0; i < H * D; i++) dq_out[i] = sm_scale * acc[i];
}

// dKV for one kv row (b, j): the sum over every (s, t) whose index is j, in ascending (s, t).
template <class R>
void dkv_row(const Shape& sh, const R* q, const R* kv, const R* dout, const int32_t* idx, const R* lse,
             const R* delta, R sm_scale, int64_t b, int64_t j, const int64_t* refs, int64_t nrefs, R* out) {
  const int64_t H = sh.H, D = sh.D;
  const R* row = kv + (b * sh.S_kv + j) * D;
  for (int64_t d = 0; d < D; d++) out[d] = R(0);
  for (int64_t r = 0; r < nrefs; r++) {
    const int64_t token = refs[r];  // b*S + s
    const R* q_tok = q + token * H * D;
    const R* do_tok = dout + token * H * D;
    for (int64_t h = 0; h < H; h++) {
      const R* qh = q_tok + h * D;
      const R* doh = do_tok + h * D;
      R z = 0, dp = 0;
      for (int64_t d = 0; d < D; d++) z += qh[d] * row[d];
      for (int64_t d = 0; d < D; d++) dp += doh[d] * row[d];
      const R score = z * sm_scale;
      const R p = std::exp2(score * (R)kLog2e - lse[token * H + h]);
      const R ds = p * (dp - delta[token * H + h]);
      const R a = sm_scale * ds;
      for (int64_t d = 0; d < D; d++) out[d] += a * qh[d] + p * doh[d];
    }
  }
}

template <class R>
void run_fwd(const R* q, const R* kv, const float* sink, const int32_t* idx, int64_t B, int64_t S, int64_t S_kv,
             int64_t H, int64_t D, int64_t topk, double sm_scale, const int64_t* tokens, int64_t n_tokens,
             R* o_out, R* lse_out) {
  const Shape sh{B, S, S_kv, H, D, topk};
  const int64_t n = tokens ? n_tokens : B * S;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < n; k++) {
    const int64_t token = tokens ? tokens[k] : k;
    fwd_token<R>(sh, q, kv, sink, idx, (R)sm_scale, token, o_out + k * H * D, lse_out + k * H);
  }
}

template <class R>
void run_dq(const R* q, const R* kv, const R* o, const R* dout, const int32_t* idx, const R* lse, int64_t B,
            int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, double sm_scale, const int64_t* tokens,
            int64_t n_tokens, R* dq_out, R* delta_out) {
  const Shape sh{B, S, S_kv, H, D, topk};
  const int64_t n = tokens ? n_tokens : B * S;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < n; k++) {
    const int64_t token = tokens ? tokens[k] : k;
    dq_token<R>(sh, q, kv, o, dout, idx, lse, (R)sm_scale, token, dq_out + k * H * D,
                delta_out ? delta_out + k * H : nullptr);
  }
}

template <class R>
void run_dkv(const R* q, const R* kv, const R* o, const R* dout, const int32_t* idx, const R* lse, int64_t B,
             int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, double sm_scale, const int64_t* rows,
             int64_t n_rows, R* dkv_out) {
  const Shape sh{B, S, S_kv, H, D, topk};
  // Delta for every token (each dKV row may need any token's).
  std::vector<R> delta(B * S * H);
#pragma omp parallel for schedule(static)
  for (int64_t th = 0; th < B * S * H; th++) {
    R a = 0;
    for (int64_t d = 0; d < D; d++) a += o[th * D + d] * dout[th * D + d];
    delta[th] = a;
  }
  // Which (b, j) rows are wanted; reference lists are kept only for those.
  const int64_t n = rows ? n_rows : B * S_kv;
  std::vector<int64_t> slot_of(B * S_kv, -1);
  for (int64_t k = 0; k < n; k++) slot_of[rows ? rows[k] : k] = k;
  std::vector<std::vector<int64_t>> refs(n);
  for (int64_t token = 0; token < B * S; token++) {
    const int64_t b = token / S;
    for (int64_t t = 0; t < topk; t++) {
      const int32_t i = idx[token * topk + t];
      if (!in_range(i, S_kv)) continue;
      const int64_t k = slot_of[b * S_kv + i];
      if (k >= 0) refs[k].push_back(token);
    }
  }
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t k = 0; k < n; k++) {
    const int64_t bj = rows ? rows[k] : k;
    dkv_row<R>(sh, q, kv, dout, idx, lse, delta.data(), (R)sm_scale, bj / S_kv, bj % S_kv, refs[k].data(),
               (int64_t)refs[k].size(), dkv_out + k * D);
  }
}

}  // namespace

extern "C" {

// Forward. q [B,S,H,D], kv [B,S_kv,D] widened to R; sink [H] fp32; idx [B,S,topk] int32.
// tokens: optional list of flat token ids (b*S + s); NULL means every token.
// o_out [n,H,D] and lse_out [n,H] are compact over the listed tokens.
void oracle_fwd_f32(const float* q, const float* kv, const float* sink, const int32_t* idx, int64_t B, int64_t S,
                    int64_t S_kv, int64_t H, int64_t D, int64_t topk, double sm_scale, const int64_t* tokens,
                    int64_t n_tokens, float* o_out, float* lse_out) {
  run_fwd<float>(q, kv, sink, idx, B, S, S_kv, H, D, topk, sm_scale, tokens, n_tokens, o_out, lse_out);
}
void oracle_fwd_f64(const double* q, const double* kv, const float* sink, const int32_t* idx, int64_t B, int64_t S,
                    int64_t S_kv, int64_t H, int64_t D, int64_t topk, double sm_scale, const int64_t* tokens,
                    int64_t n_tokens, double* o_out, double* lse_out) {
  run_fwd<double>(q, kv, sink, idx, B, S, S_kv, H, D, topk, sm_scale, tokens, n_tokens, o_out, lse_out);
}

// dQ (and Delta) for listed tokens. o and dout [B,S,H,D]; lse [B,S,H] (log2 units).
void oracle_dq_f32(const float* q, const float* kv, const float* o, const float* dout, const int32_t* idx,
                   const float* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                   double sm_scale, const int64_t* tokens, int64_t n_tokens, float* dq_out, float* delta_out) {
  run_dq<float>(q, kv, o, dout, idx, lse, B, S, S_kv, H, D, topk, sm_scale, tokens, n_tokens, dq_out, delta_out);
}
void oracle_dq_f64(const double* q, const double* kv, const double* o, const double* dout, const int32_t* idx,
                   const double* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                   double sm_scale, const int64_t* tokens, int64_t n_tokens, double* dq_out, double* delta_out) {
  run_dq<double>(q, kv, o, dout, idx, lse, B, S, S_kv, H, D, topk, sm_scale, tokens, n_tokens, dq_out, delta_out);
}

// dKV rows. rows: optional list of flat kv row ids (b*S_kv + j); NULL means every row.
// dkv_out [n,D] compact over the listed rows.
void oracle_dkv_f32(const float* q, const float* kv, const float* o, const float* dout, const int32_t* idx,
                    const float* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                    double sm_scale, const int64_t* rows, int64_t n_rows, float* dkv_out) {
  run_dkv<float>(q, kv, o, dout, idx, lse, B, S, S_kv, H, D, topk, sm_scale, rows, n_rows, dkv_out);
}
void oracle_dkv_f64(const double* q, const double* kv, const double* o, const double* dout, const int32_t* idx,
                    const double* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                    double sm_scale, const int64_t* rows, int64_t n_rows, double* dkv_out) {
  run_dkv<double>(q, kv, o, dout, idx, lse, B, S, S_kv, H, D, topk, sm_scale, rows, n_rows, dkv_out);
}

int oracle_num_threads(void) { return omp_get_max_threads(); }

}  // extern "C"

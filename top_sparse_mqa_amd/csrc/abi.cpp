// C ABI of libsparse_mqa: argument validation and dispatch. Every check runs before any HIP
// call, so invalid arguments are rejected without touching the device.
#include "../../include/sparse_mqa.h"
#include "launch.h"

#include <cmath>
#include <cstdint>

namespace {

bool supported(int64_t H, int64_t D) {
  if (D == 512) return H == 16 || H == 32 || H == 64 || H == 128;
  if (D == 64) return H == 16 || H == 32;
  return false;
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }

// Element count of a product of dims, or -1 on overflow.
int64_t count(std::initializer_list<int64_t> dims) {
  int64_t n = 1;
  for (int64_t d : dims)
    if (!mul_ok(n, d, &n)) return -1;
  return n;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

struct Span {
  const void* p;
  int64_t bytes;
};
bool overlap(Span a, Span b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = (uintptr_t)a.p, b0 = (uintptr_t)b.p;
  return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Common shape checks of the forward / backward: sizes positive, counts representable,
// grid sizes within launch limits.
int check_shapes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk) {
  if (B <= 0 || S <= 0 || S_kv <= 0 || H <= 0 || D <= 0 || topk <= 0) return SMQA_ERR_SHAPE;
  if (S_kv > INT32_MAX || topk > INT32_MAX / 2 || S > INT32_MAX) return SMQA_ERR_SHAPE;
  const int64_t tokens = count({B, S});
  if (tokens < 0 || tokens > (int64_t)INT32_MAX / 8) return SMQA_ERR_SHAPE;
  if (count({B, S, H, D}) < 0 || count({B, S_kv, D}) < 0 || count({B, S, topk}) < 0) return SMQA_ERR_SHAPE;
  if (!supported(H, D)) return SMQA_ERR_UNSUPPORTED;
  return SMQA_OK;
}

int resolve_scale(float in, int64_t D, float* out) {
  if (std::isnan(in)) {
    *out = (float)(1.0 / std::sqrt((double)D));
    return SMQA_OK;
  }
  if (!std::isfinite(in)) return SMQA_ERR_ARG;
  *out = in;
  return SMQA_OK;
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* sparse_mqa_status_string(int status) {
  switch (status) {
    case SMQA_OK: return "ok";
    case SMQA_ERR_NULL: return "a required pointer is NULL";
    case SMQA_ERR_SHAPE: return "a size is <= 0 or beyond a supported limit";
    case SMQA_ERR_UNSUPPORTED: return "unsupported (H, D): no compiled kernel";
    case SMQA_ERR_ALIGN: return "a tensor pointer is not 16-byte aligned";
    case SMQA_ERR_ALIAS: return "an output overlaps an input or another output";
    case SMQA_ERR_WORKSPACE: return "workspace missing or too small";
    case SMQA_ERR_HIP: return "HIP kernel launch failed";
    case SMQA_ERR_ARG: return "invalid argument";
    default: return "unknown status";
  }
}

int sparse_mqa_fwd(const void* q, const void* kv, const float* attn_sink, const int32_t* topk_idxs, void* o,
                   float* lse, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                   float sm_scale, void* stream) {
  if (!q || !kv || !attn_sink || !topk_idxs || !o || !lse) return SMQA_ERR_NULL;
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned4(lse) || !aligned4(attn_sink) ||
      !aligned4(topk_idxs))
    return SMQA_ERR_ALIGN;
  float scale;
  if ((st = resolve_scale(sm_scale, D, &scale))) return st;
  const int64_t qb = count({B, S, H, D}) * 2, kvb = count({B, S_kv, D}) * 2;
  const Span so{o, qb}, sl{lse, count({B, S, H}) * 4};
  const Span ins[] = {{q, qb}, {kv, kvb}, {attn_sink, H * 4}, {topk_idxs, count({B, S, topk}) * 4}};
  for (const Span& s : ins)
    if (overlap(so, s) || overlap(sl, s)) return SMQA_ERR_ALIAS;
  if (overlap(so, sl)) return SMQA_ERR_ALIAS;
  smqa::FwdArgs a{q, kv, attn_sink, topk_idxs, o, lse, B, S, S_kv, H, D, topk, scale};
  return smqa::launch_fwd(a, (hipStream_t)stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

size_t sparse_mqa_bwd_workspace_bytes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D) {
  if (B <= 0 || S <= 0 || S_kv <= 0 || H <= 0 || D <= 0) return 0;
  const int64_t nd = count({B, S, H}), na = count({B, S_kv, D});
  if (nd < 0 || na < 0) return 0;
  return round256((size_t)nd * 4) + round256((size_t)na * 4);
}

int sparse_mqa_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t B, int64_t S, int64_t H,
                              int64_t D, void* stream) {
  if (!o || !d_o || !delta) return SMQA_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return SMQA_ERR_SHAPE;
  if (D != 64 && D != 512) return SMQA_ERR_UNSUPPORTED;
  const int64_t rows = count({B, S, H});
  if (rows < 0 || count({B, S, H, D}) < 0) return SMQA_ERR_SHAPE;
  if (!aligned16(o) || !aligned16(d_o) || !aligned4(delta)) return SMQA_ERR_ALIGN;
  const Span sd{delta, rows * 4};
  if (overlap(sd, {o, rows * D * 2}) || overlap(sd, {d_o, rows * D * 2})) return SMQA_ERR_ALIAS;
  return smqa::launch_bwd_preprocess(o, d_o, delta, rows, D, (hipStream_t)stream) == hipSuccess ? SMQA_OK
                                                                                                 : SMQA_ERR_HIP;
}

static int bwd_main_checked(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                            const float* lse, const float* delta, void* dq, float* dkv_accum, int64_t B,
                            int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float scale, int which,
                            hipStream_t stream) {
  smqa::BwdMainArgs a{q, kv, d_o, topk_idxs, lse, delta, dq, dkv_accum, B, S, S_kv, H, D, topk, scale};
  return smqa::launch_bwd_main(a, which, stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

// Validation shared by the main-stage entry points; which = 1 (dQ), 2 (dKV) or 3 (both).
static int bwd_main_entry(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                          const float* lse, const float* delta, void* dq, float* dkv_accum, int64_t B, int64_t S,
                          int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale, int which,
                          void* stream) {
  if (!q || !kv || !d_o || !topk_idxs || !lse || !delta) return SMQA_ERR_NULL;
  if (((which & 1) && !dq) || ((which & 2) && !dkv_accum)) return SMQA_ERR_NULL;
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(d_o) || !aligned4(lse) || !aligned4(delta) ||
      !aligned4(topk_idxs))
    return SMQA_ERR_ALIGN;
  if (((which & 1) && !aligned16(dq)) || ((which & 2) && !aligned16(dkv_accum))) return SMQA_ERR_ALIGN;
  float scale;
  if ((st = resolve_scale(sm_scale, D, &scale))) return st;
  const int64_t qb = count({B, S, H, D}) * 2, ab = count({B, S_kv, D}) * 4;
  const Span sdq{(which & 1) ? dq : nullptr, qb}, sacc{(which & 2) ? dkv_accum : nullptr, ab};
  const Span ins[] = {{q, qb}, {kv, count({B, S_kv, D}) * 2}, {d_o, qb}, {topk_idxs, count({B, S, topk}) * 4},
                      {lse, count({B, S, H}) * 4}, {delta, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdq, s) || overlap(sacc, s)) return SMQA_ERR_ALIAS;
  if (overlap(sdq, sacc)) return SMQA_ERR_ALIAS;
  return bwd_main_checked(q, kv, d_o, topk_idxs, lse, delta, dq, dkv_accum, B, S, S_kv, H, D, topk, scale, which,
                          (hipStream_t)stream);
}

int sparse_mqa_bwd_main(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                        const float* lse, const float* delta, void* dq, float* dkv_accum, int64_t B, int64_t S,
                        int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale, void* stream) {
  return bwd_main_entry(q, kv, d_o, topk_idxs, lse, delta, dq, dkv_accum, B, S, S_kv, H, D, topk, sm_scale, 3,
                        stream);
}

int sparse_mqa_bwd_dq(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs, const float* lse,
                      const float* delta, void* dq, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                      int64_t topk, float sm_scale, void* stream) {
  return bwd_main_entry(q, kv, d_o, topk_idxs, lse, delta, dq, nullptr, B, S, S_kv, H, D, topk, sm_scale, 1,
                        stream);
}

int sparse_mqa_bwd_dkv(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                       const float* lse, const float* delta, float* dkv_accum, int64_t B, int64_t S, int64_t S_kv,
                       int64_t H, int64_t D, int64_t topk, float sm_scale, void* stream) {
  return bwd_main_entry(q, kv, d_o, topk_idxs, lse, delta, nullptr, dkv_accum, B, S, S_kv, H, D, topk, sm_scale,
                        2, stream);
}

int sparse_mqa_bwd_postprocess(const float* dkv_accum, void* dkv, int64_t B, int64_t S_kv, int64_t D,
                               void* stream) {
  if (!dkv_accum || !dkv) return SMQA_ERR_NULL;
  if (B <= 0 || S_kv <= 0 || D <= 0 || (D % 8) != 0) return SMQA_ERR_SHAPE;
  const int64_t n = count({B, S_kv, D});
  if (n < 0) return SMQA_ERR_SHAPE;
  if (!aligned16(dkv_accum) || !aligned16(dkv)) return SMQA_ERR_ALIGN;
  if (overlap({dkv_accum, n * 4}, {dkv, n * 2})) return SMQA_ERR_ALIAS;
  return smqa::launch_bwd_postprocess(dkv_accum, dkv, n, (hipStream_t)stream) == hipSuccess ? SMQA_OK
                                                                                           : SMQA_ERR_HIP;
}

int sparse_mqa_bwd(const void* q, const void* kv, const float* attn_sink, const void* o, const void* d_o,
                   const int32_t* topk_idxs, const float* lse, void* dq, void* dkv, int dkv_fp32, void* workspace,
                   size_t workspace_bytes, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                   int64_t topk, float sm_scale, void* stream) {
  if (!q || !kv || !attn_sink || !o || !d_o || !topk_idxs || !lse || !dq || !dkv) return SMQA_ERR_NULL;
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(o) || !aligned16(d_o) || !aligned16(dq) || !aligned16(dkv) ||
      !aligned4(lse) || !aligned4(attn_sink) || !aligned4(topk_idxs))
    return SMQA_ERR_ALIGN;
  float scale;
  if ((st = resolve_scale(sm_scale, D, &scale))) return st;
  const size_t need_delta = round256((size_t)count({B, S, H}) * 4);
  const size_t need = dkv_fp32 ? need_delta : sparse_mqa_bwd_workspace_bytes(B, S, S_kv, H, D);
  if (!workspace || workspace_bytes < need) return SMQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SMQA_ERR_ALIGN;
  const int64_t qb = count({B, S, H, D}) * 2, nkv = count({B, S_kv, D});
  const Span sdq{dq, qb}, sdkv{dkv, nkv * (dkv_fp32 ? 4 : 2)}, sws{workspace, (int64_t)need};
  const Span ins[] = {{q, qb}, {kv, nkv * 2}, {attn_sink, H * 4}, {o, qb}, {d_o, qb},
                      {topk_idxs, count({B, S, topk}) * 4}, {lse, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdq, s) || overlap(sdkv, s) || overlap(sws, s)) return SMQA_ERR_ALIAS;
  if (overlap(sdq, sdkv) || overlap(sdq, sws) || overlap(sdkv, sws)) return SMQA_ERR_ALIAS;

  hipStream_t hs = (hipStream_t)stream;
  float* delta = (float*)workspace;
  float* acc = dkv_fp32 ? (float*)dkv : (float*)((char*)workspace + need_delta);
  const int64_t rows = count({B, S, H});
  if (smqa::launch_bwd_preprocess(o, d_o, delta, rows, D, hs) != hipSuccess) return SMQA_ERR_HIP;
  if (smqa::launch_fill_zero_f32(acc, nkv, hs) != hipSuccess) return SMQA_ERR_HIP;
  if ((st = bwd_main_checked(q, kv, d_o, topk_idxs, lse, delta, dq, acc, B, S, S_kv, H, D, topk, scale, 3, hs)))
    return st;
  if (!dkv_fp32 && smqa::launch_bwd_postprocess(acc, dkv, nkv, hs) != hipSuccess) return SMQA_ERR_HIP;
  return SMQA_OK;
}

}  // extern "C"

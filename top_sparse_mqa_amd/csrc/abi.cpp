// C ABI of libsparse_mqa: argument validation and dispatch. Every check runs before any HIP
// call, so invalid arguments are rejected without touching the device.
#include "../../include/sparse_mqa.h"
#include "launch.h"

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

namespace {

// D = 128, 256 or 512: H = 16 or 32 (one workgroup per token), or any multiple of 64 up to 1024
// (H / 64 workgroups of 64 heads per token). D = 64: H = 16 or 32.
bool supported(int64_t H, int64_t D) {
  if (D == 128 || D == 256 || D == 512) return H == 16 || H == 32 || (H % 64 == 0 && H >= 64 && H <= 1024);
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
  // One workgroup of up to 512 threads per (token, block of 64 heads): a launch may hold at most
  // 2^32 - 1 threads, so the workgroup count stays below 2^23. (The per-row and per-element kernels
  // loop over their work and cap their grids.)
  int64_t wgs = 0;
  if (tokens < 0 || !mul_ok(tokens, H > 64 ? H / 64 : 1, &wgs) || wgs >= ((int64_t)1 << 23)) return SMQA_ERR_SHAPE;
  if (count({B, S, H, D}) < 0 || count({B, S_kv, D}) < 0 || count({B, S, topk}) < 0) return SMQA_ERR_SHAPE;
  if (!supported(H, D)) return SMQA_ERR_UNSUPPORTED;
  // the tile gathers address one batch's kv rows through a 32-bit byte range
  if (S_kv * D * 2 > (int64_t)UINT32_MAX) return SMQA_ERR_UNSUPPORTED;
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
                   float sm_scale, int reference_rounding, void* stream) {
  if (!q || !kv || !attn_sink || !topk_idxs || !o || !lse) return SMQA_ERR_NULL;
  if (reference_rounding != 0 && reference_rounding != 1) return SMQA_ERR_ARG;
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
  smqa::FwdArgs a{q, kv, attn_sink, topk_idxs, o, lse, B, S, S_kv, H, D, topk, scale, reference_rounding};
  return smqa::launch_fwd(a, (hipStream_t)stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------------------------
// Backward workspace: [Delta (full bwd only)] [kv row norms] [selection bitmap words (bits and pair
// count; after the scan, bits and the word's prefix inside its scan tile), cursors] [offsets]
// [scan tiles] [acc (multi-chunk, bf16 output only)] [pos: chunk*topk int32] [staging rows:
// chunk*(topk+1)*n_hblk rows of D int16] [their exponents] [dS (full bwd at D = 512)]. The bitmap
// part and the offsets scale with the chunk (one bit per kv row and chunk token).

namespace {

struct DkvPlan {
  size_t kvn, bits, offset, tiles, acc, pos, stage, stage_exp, ds;  // byte offsets into the workspace
  int64_t chunk;                                               // tokens per chunk
  bool use_acc;                                                // a separate fp32 accumulator in the workspace
  size_t end;                                                  // bytes used
};

// Lay out the dKV part of the workspace from `base` for token chunks of `chunk` tokens; returns the
// end offset.
size_t dkv_layout(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, int64_t chunk,
                  bool use_acc, bool with_ds, size_t base, DkvPlan* p) {
  const int64_t n_rows = B * S_kv, words = smqa::dkv_bitmap_words(n_rows, chunk, S);
  size_t o = base;
  p->kvn = o;  // kv row norms
  o += round256((size_t)n_rows * 4);
  p->bits = o;  // selection bitmap, pair counts and cursors, cleared as whole 16-byte pieces
  o += round256((size_t)(3 * words + 4) * 4);
  p->offset = o;
  o += round256((size_t)(words + 1) * 4);
  p->tiles = o;
  o += round256((size_t)smqa::scan_tiles(words) * 4);
  p->use_acc = use_acc;
  p->acc = use_acc ? o : 0;
  if (use_acc) o += round256((size_t)n_rows * D * 4);
  p->pos = o;
  o += round256((size_t)chunk * topk * 4);
  // one staging row per slot and head block, and one spare row per token and head block that takes
  // the stores of the token's masked slots
  const size_t rows = (size_t)chunk * (topk + 1) * smqa::bwd_hblocks(H);
  p->stage = o;
  o += round256(rows * D * 2);
  p->stage_exp = o;
  o += round256(rows * smqa::stage_segments(H, D));
  // the dS the dKV kernel stores for the dQ kernel (full backward at D = 512, 64-head blocks)
  p->ds = with_ds ? o : 0;
  if (with_ds) o += round256((size_t)smqa::ds_bytes(chunk, H, topk));
  p->chunk = chunk;
  p->end = o;
  return o;
}

// Lay out the dKV part of the workspace starting at `base`: one pass over all tokens if it fits,
// else the largest token chunk that fits, with an fp32 running sum; false if `bytes` cannot hold
// even one token's staging.
// Most tokens one dKV pass may take: staging row indices are 32-bit, and the scan of the bitmap
// words runs one workgroup per 4096 words (a launch holds fewer than 2^24 workgroups of 256
// threads). 0 if not even one token fits.
int64_t max_chunk_tokens(int64_t B, int64_t S_kv, int64_t H, int64_t topk) {
  int64_t max_chunk = (int64_t)(INT32_MAX / ((topk + 1) * smqa::bwd_hblocks(H)));
  const int64_t max_nw = (((int64_t)1 << 24) - 1) * 4096 / (B * S_kv);
  if (max_nw * 32 < max_chunk) max_chunk = max_nw * 32;
  return max_chunk < 0 ? 0 : max_chunk;
}

bool plan_dkv(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, bool dkv_fp32, bool with_ds,
              size_t base, size_t bytes, DkvPlan* p) {
  const int64_t tokens = B * S;
  const int64_t max_chunk = max_chunk_tokens(B, S_kv, H, topk);
  if (max_chunk < 1) return false;
  if (tokens <= max_chunk && dkv_layout(B, S, S_kv, H, D, topk, tokens, false, with_ds, base, p) <= bytes) return true;
  const bool use_acc = !dkv_fp32;
  if (dkv_layout(B, S, S_kv, H, D, topk, 1, use_acc, with_ds, base, p) > bytes) return false;
  int64_t lo = 1, hi = tokens < max_chunk ? tokens : max_chunk;
  while (lo < hi) {  // the largest chunk that fits (the layout grows with the chunk)
    const int64_t mid = lo + (hi - lo + 1) / 2;
    if (dkv_layout(B, S, S_kv, H, D, topk, mid, use_acc, with_ds, base, p) <= bytes) lo = mid;
    else hi = mid - 1;
  }
  dkv_layout(B, S, S_kv, H, D, topk, lo, use_acc, with_ds, base, p);
  return true;
}

size_t delta_bytes(int64_t B, int64_t S, int64_t H) { return round256((size_t)(B * S * H) * 4); }

bool sizes_ok(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk) {
  return check_shapes(B, S, S_kv, H, D, topk) == SMQA_OK;
}

// The staged dKV pass over all tokens, chunked as the plan says. dkv: bf16 or fp32 output. When the
// plan has a dS region, the dKV kernel also stores dS and dQ (dq) is computed from it chunk by chunk.
int run_dkv(const void* q, const void* kv, const void* d_o, const int32_t* idx, const float* lse, const float* delta,
            void* dkv, int dkv_fp32, void* dq, char* ws, const DkvPlan& p, int64_t B, int64_t S, int64_t S_kv,
            int64_t H, int64_t D, int64_t topk, float scale, hipStream_t st) {
  const int64_t tokens = B * S, n_rows = B * S_kv;
  uint32_t* bits = (uint32_t*)(ws + p.bits);
  int32_t* offset = (int32_t*)(ws + p.offset);
  int32_t* tiles = (int32_t*)(ws + p.tiles);
  int32_t* pos = (int32_t*)(ws + p.pos);
  uint16_t* stage = (uint16_t*)(ws + p.stage);
  int8_t* stage_exp = (int8_t*)(ws + p.stage_exp);
  float* acc = dkv_fp32 ? (float*)dkv : (p.use_acc ? (float*)(ws + p.acc) : nullptr);
  float* kvn = (float*)(ws + p.kvn);
  if (smqa::launch_kv_row_norm(kv, n_rows, D, kvn, st) != hipSuccess) return SMQA_ERR_HIP;
  for (int64_t t0 = 0; t0 < tokens; t0 += p.chunk) {
    const int64_t n = (tokens - t0) < p.chunk ? (tokens - t0) : p.chunk;
    if (smqa::launch_dkv_prepare(idx, bits, offset, tiles, pos, B, S, S_kv, topk, smqa::bwd_hblocks(H), t0, n, st) !=
        hipSuccess)
      return SMQA_ERR_HIP;
    smqa::BwdMainArgs a{q, kv, d_o, idx, lse, delta, dq, nullptr, pos, stage, stage_exp, kvn, B, S, S_kv, H,
                        D, topk, scale, t0, n, p.ds ? (uint16_t*)(ws + p.ds) : nullptr};
    if (smqa::launch_bwd_main(a, 2, st) != hipSuccess) return SMQA_ERR_HIP;
    if (p.ds && smqa::launch_bwd_dq_ds(a, st) != hipSuccess) return SMQA_ERR_HIP;
    const bool last = t0 + n >= tokens;
    void* out16 = (!dkv_fp32 && last) ? dkv : nullptr;
    if (smqa::launch_reduce_rows(stage, stage_exp, smqa::stage_segments(H, D), offset,
                                 smqa::dkv_row_words(n, S), acc, out16, t0 > 0 ? 1 : 0, n_rows, D,
                                 st) != hipSuccess)
      return SMQA_ERR_HIP;
  }
  return SMQA_OK;
}

int check_bwd_inputs(const void* q, const void* kv, const void* d_o, const int32_t* idx, const float* lse,
                     int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                     float* scale) {
  if (!q || !kv || !d_o || !idx || !lse) return SMQA_ERR_NULL;
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!aligned16(q) || !aligned16(kv) || !aligned16(d_o) || !aligned4(lse) || !aligned4(idx)) return SMQA_ERR_ALIGN;
  return resolve_scale(sm_scale, D, scale);
}

// Argument checks of the full backward on a workspace of workspace_bytes at `workspace` (which may be
// null when check_ws_ptr is false: the allocation-free entry point learns its address only after
// the checks, and its scratch overlaps no caller buffer). Fills the scale and the dKV plan.
int bwd_validate(const void* q, const void* kv, const float* attn_sink, const void* o, const void* d_o,
                 const int32_t* topk_idxs, const float* lse, void* dq, void* dkv, int dkv_fp32, void* workspace,
                 size_t workspace_bytes, bool check_ws_ptr, int64_t B, int64_t S, int64_t S_kv, int64_t H,
                 int64_t D, int64_t topk, float sm_scale, float* scale, DkvPlan* p) {
  int st = check_bwd_inputs(q, kv, d_o, topk_idxs, lse, B, S, S_kv, H, D, topk, sm_scale, scale);
  if (st) return st;
  if (!attn_sink || !o || !dq || !dkv) return SMQA_ERR_NULL;
  if (check_ws_ptr && !workspace) return SMQA_ERR_WORKSPACE;
  if (!aligned16(o) || !aligned16(dq) || !aligned16(dkv) || !aligned4(attn_sink) || !aligned16(workspace))
    return SMQA_ERR_ALIGN;
  const size_t dbytes = delta_bytes(B, S, H);
  if (workspace_bytes < dbytes ||
      !plan_dkv(B, S, S_kv, H, D, topk, dkv_fp32 != 0, smqa::dq_from_ds(H, D), dbytes, workspace_bytes, p))
    return SMQA_ERR_WORKSPACE;
  const int64_t qb = count({B, S, H, D}) * 2, nkv = count({B, S_kv, D});
  const Span sdq{dq, qb}, sdkv{dkv, nkv * (dkv_fp32 ? 4 : 2)}, sws{workspace, (int64_t)p->end};
  const Span ins[] = {{q, qb}, {kv, nkv * 2}, {attn_sink, H * 4}, {o, qb}, {d_o, qb},
                      {topk_idxs, count({B, S, topk}) * 4}, {lse, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdq, s) || overlap(sdkv, s) || overlap(sws, s)) return SMQA_ERR_ALIAS;
  if (overlap(sdq, sdkv) || overlap(sdq, sws) || overlap(sdkv, sws)) return SMQA_ERR_ALIAS;
  return SMQA_OK;
}

// The full backward (preprocess, staged dKV in as many token chunks as the plan says, dQ) on a
// validated workspace; sparse_mqa_bwd and sparse_mqa_bwd_noalloc differ only in where it comes from.
int bwd_launch(const void* q, const void* kv, const void* o, const void* d_o, const int32_t* topk_idxs,
               const float* lse, void* dq, void* dkv, int dkv_fp32, void* workspace, const DkvPlan& p, int64_t B,
               int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float scale, void* stream) {
  hipStream_t hs = (hipStream_t)stream;
  float* delta = (float*)workspace;
  if (smqa::launch_bwd_preprocess(o, d_o, delta, count({B, S, H}), D, hs) != hipSuccess) return SMQA_ERR_HIP;
  const int st = run_dkv(q, kv, d_o, topk_idxs, lse, delta, dkv, dkv_fp32, dq, (char*)workspace, p, B, S, S_kv, H,
                         D, topk, scale, hs);
  if (st) return st;
  if (p.ds) return SMQA_OK;  // dQ came from the stored dS
  smqa::BwdMainArgs a{q, kv, d_o, topk_idxs, lse, delta, dq, nullptr, nullptr, nullptr, nullptr, nullptr, B, S, S_kv, H,
                      D, topk, scale, 0, B * S};
  return smqa::launch_bwd_main(a, 1, hs) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

// Workspace of sparse_mqa_bwd_noalloc, for callers that cannot allocate device memory: one
// SMQA_BWD_SCRATCH_BYTES array per device, created with the library's code object on each device it
// runs on and held until the process ends. Host code never passes this name to a kernel (on the host
// it is only a stand-in for the symbol): the device address of each device's copy comes from
// hipGetSymbolAddress, taken once per device with that device current.
static __device__ __align__(256) char scratch[SMQA_BWD_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];  // device address of `scratch` per device, once known
std::mutex g_scratch_mu;

// Device address of the scratch array of the device `stream` runs on, which must be the current
// device (hipGetSymbolAddress resolves the symbol for the current device).
int scratch_for_stream(hipStream_t stream, void** out) {
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return SMQA_ERR_HIP;
  if (stream) {
    hipDevice_t sd = -1;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return SMQA_ERR_HIP;
    if ((int)sd != cur) return SMQA_ERR_ARG;
  }
  if (cur < 0 || cur >= kMaxDevices) return SMQA_ERR_UNSUPPORTED;
  void* p = g_scratch_addr[cur].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_addr[cur].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SMQA_ERR_HIP;
      g_scratch_addr[cur].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SMQA_OK;
}

}  // namespace

extern "C" {

size_t sparse_mqa_bwd_workspace_bytes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk) {
  if (!sizes_ok(B, S, S_kv, H, D, topk)) return 0;
  DkvPlan p;
  return delta_bytes(B, S, H) + dkv_layout(B, S, S_kv, H, D, topk, B * S, false, smqa::dq_from_ds(H, D), 0, &p);
}

size_t sparse_mqa_bwd_workspace_min_bytes(int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk) {
  if (!sizes_ok(B, S, S_kv, H, D, topk)) return 0;
  const int64_t max_chunk = max_chunk_tokens(B, S_kv, H, topk);
  if (max_chunk < 1) return 0;
  DkvPlan p;
  // token chunks of one (with the fp32 running sum), or a single pass over all tokens when that
  // takes less (few tokens over many kv rows)
  const bool with_ds = smqa::dq_from_ds(H, D);
  const size_t chunked = dkv_layout(B, S, S_kv, H, D, topk, 1, true, with_ds, 0, &p);
  size_t low = chunked;
  if (B * S <= max_chunk) {
    const size_t one_pass = dkv_layout(B, S, S_kv, H, D, topk, B * S, false, with_ds, 0, &p);
    if (one_pass < low) low = one_pass;
  }
  return delta_bytes(B, S, H) + low;
}

int sparse_mqa_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t B, int64_t S, int64_t H,
                              int64_t D, void* stream) {
  if (!o || !d_o || !delta) return SMQA_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0 || D <= 0) return SMQA_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256 && D != 512) return SMQA_ERR_UNSUPPORTED;
  const int64_t rows = count({B, S, H});
  if (rows < 0 || count({B, S, H, D}) < 0) return SMQA_ERR_SHAPE;
  if (!aligned16(o) || !aligned16(d_o) || !aligned4(delta)) return SMQA_ERR_ALIGN;
  const Span sd{delta, rows * 4};
  if (overlap(sd, {o, rows * D * 2}) || overlap(sd, {d_o, rows * D * 2})) return SMQA_ERR_ALIAS;
  return smqa::launch_bwd_preprocess(o, d_o, delta, rows, D, (hipStream_t)stream) == hipSuccess ? SMQA_OK
                                                                                                 : SMQA_ERR_HIP;
}

int sparse_mqa_bwd_dsink(const float* lse, const float* delta, const float* attn_sink, float* d_sink, int64_t B,
                         int64_t S, int64_t H, void* stream) {
  if (!lse || !delta || !attn_sink || !d_sink) return SMQA_ERR_NULL;
  if (B <= 0 || S <= 0 || H <= 0 || H > 65536) return SMQA_ERR_SHAPE;
  const int64_t rows = count({B, S, H});
  if (rows < 0) return SMQA_ERR_SHAPE;
  if (!aligned4(lse) || !aligned4(delta) || !aligned4(attn_sink) || !aligned4(d_sink)) return SMQA_ERR_ALIGN;
  const Span out{d_sink, H * 4};
  if (overlap(out, {lse, rows * 4}) || overlap(out, {delta, rows * 4}) || overlap(out, {attn_sink, H * 4}))
    return SMQA_ERR_ALIAS;
  return smqa::launch_bwd_dsink(lse, delta, attn_sink, d_sink, B * S, H, (hipStream_t)stream) == hipSuccess
             ? SMQA_OK
             : SMQA_ERR_HIP;
}

int sparse_mqa_bwd_dq(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs, const float* lse,
                      const float* delta, void* dq, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D,
                      int64_t topk, float sm_scale, void* stream) {
  float scale;
  int st = check_bwd_inputs(q, kv, d_o, topk_idxs, lse, B, S, S_kv, H, D, topk, sm_scale, &scale);
  if (st) return st;
  if (!delta || !dq) return SMQA_ERR_NULL;
  if (!aligned4(delta) || !aligned16(dq)) return SMQA_ERR_ALIGN;
  const int64_t qb = count({B, S, H, D}) * 2;
  const Span sdq{dq, qb};
  const Span ins[] = {{q, qb}, {kv, count({B, S_kv, D}) * 2}, {d_o, qb}, {topk_idxs, count({B, S, topk}) * 4},
                      {lse, count({B, S, H}) * 4}, {delta, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdq, s)) return SMQA_ERR_ALIAS;
  smqa::BwdMainArgs a{q, kv, d_o, topk_idxs, lse, delta, dq, nullptr, nullptr, nullptr, nullptr, nullptr, B, S, S_kv, H,
                      D, topk, scale, 0, B * S};
  return smqa::launch_bwd_main(a, 1, (hipStream_t)stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

int sparse_mqa_bwd_dkv(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs, const float* lse,
                       const float* delta, void* dkv, int dkv_fp32, void* workspace, size_t workspace_bytes,
                       int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                       void* stream) {
  float scale;
  int st = check_bwd_inputs(q, kv, d_o, topk_idxs, lse, B, S, S_kv, H, D, topk, sm_scale, &scale);
  if (st) return st;
  if (!delta || !dkv) return SMQA_ERR_NULL;
  if (!workspace) return SMQA_ERR_WORKSPACE;
  if (!aligned4(delta) || !aligned16(dkv) || !aligned16(workspace)) return SMQA_ERR_ALIGN;
  DkvPlan p;
  if (!plan_dkv(B, S, S_kv, H, D, topk, dkv_fp32 != 0, false, 0, workspace_bytes, &p)) return SMQA_ERR_WORKSPACE;
  const int64_t qb = count({B, S, H, D}) * 2, nkv = count({B, S_kv, D});
  const Span sdkv{dkv, nkv * (dkv_fp32 ? 4 : 2)}, sws{workspace, (int64_t)p.end};
  const Span ins[] = {{q, qb}, {kv, nkv * 2}, {d_o, qb}, {topk_idxs, count({B, S, topk}) * 4},
                      {lse, count({B, S, H}) * 4}, {delta, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdkv, s) || overlap(sws, s)) return SMQA_ERR_ALIAS;
  if (overlap(sdkv, sws)) return SMQA_ERR_ALIAS;
  return run_dkv(q, kv, d_o, topk_idxs, lse, delta, dkv, dkv_fp32, nullptr, (char*)workspace, p, B, S, S_kv, H, D, topk, scale,
                 (hipStream_t)stream);
}

// The three steps of a single-pass staged dKV, for callers that schedule or time them separately.
// They need a workspace that holds every token (sparse_mqa_bwd_workspace_bytes minus Delta's part)
// and must run in order on one stream with the same workspace and sizes.
static int single_pass_plan(void* workspace, size_t workspace_bytes, int64_t B, int64_t S, int64_t S_kv, int64_t H,
                            int64_t D, int64_t topk, int dkv_fp32, DkvPlan* p) {
  if (!workspace) return SMQA_ERR_WORKSPACE;
  if (!aligned16(workspace)) return SMQA_ERR_ALIGN;
  if (!plan_dkv(B, S, S_kv, H, D, topk, dkv_fp32 != 0, smqa::dq_from_ds(H, D), 0, workspace_bytes, p) ||
      p->chunk != B * S)
    return SMQA_ERR_WORKSPACE;
  return SMQA_OK;
}

int sparse_mqa_bwd_dkv_prepare(const int32_t* topk_idxs, void* workspace, size_t workspace_bytes, int64_t B,
                               int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, void* stream) {
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!topk_idxs) return SMQA_ERR_NULL;
  if (!aligned4(topk_idxs)) return SMQA_ERR_ALIGN;
  DkvPlan p;
  if ((st = single_pass_plan(workspace, workspace_bytes, B, S, S_kv, H, D, topk, 0, &p))) return st;
  if (overlap(Span{workspace, (int64_t)p.end}, Span{topk_idxs, count({B, S, topk}) * 4})) return SMQA_ERR_ALIAS;
  char* ws = (char*)workspace;
  if (smqa::launch_dkv_prepare(topk_idxs, (uint32_t*)(ws + p.bits), (int32_t*)(ws + p.offset),
                               (int32_t*)(ws + p.tiles), (int32_t*)(ws + p.pos), B, S, S_kv, topk,
                               smqa::bwd_hblocks(H), 0, B * S, (hipStream_t)stream) != hipSuccess)
    return SMQA_ERR_HIP;
  return SMQA_OK;
}

int sparse_mqa_bwd_dkv_partials(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                                const float* lse, const float* delta, void* workspace, size_t workspace_bytes,
                                int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                                float sm_scale, void* stream) {
  float scale;
  int st = check_bwd_inputs(q, kv, d_o, topk_idxs, lse, B, S, S_kv, H, D, topk, sm_scale, &scale);
  if (st) return st;
  if (!delta) return SMQA_ERR_NULL;
  if (!aligned4(delta)) return SMQA_ERR_ALIGN;
  DkvPlan p;
  if ((st = single_pass_plan(workspace, workspace_bytes, B, S, S_kv, H, D, topk, 0, &p))) return st;
  const int64_t qb = count({B, S, H, D}) * 2;
  const Span sws{workspace, (int64_t)p.end};
  const Span ins[] = {{q, qb}, {kv, count({B, S_kv, D}) * 2}, {d_o, qb}, {topk_idxs, count({B, S, topk}) * 4},
                      {lse, count({B, S, H}) * 4}, {delta, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sws, s)) return SMQA_ERR_ALIAS;
  char* ws = (char*)workspace;
  float* kvn = (float*)(ws + p.kvn);
  if (smqa::launch_kv_row_norm(kv, B * S_kv, D, kvn, (hipStream_t)stream) != hipSuccess) return SMQA_ERR_HIP;
  smqa::BwdMainArgs a{q, kv, d_o, topk_idxs, lse, delta, nullptr, nullptr, (const int32_t*)(ws + p.pos),
                      (uint16_t*)(ws + p.stage), (int8_t*)(ws + p.stage_exp), kvn, B, S, S_kv, H, D, topk, scale, 0,
                      B * S, p.ds ? (uint16_t*)(ws + p.ds) : nullptr};
  if (smqa::launch_bwd_main(a, 2, (hipStream_t)stream) != hipSuccess) return SMQA_ERR_HIP;
  return SMQA_OK;
}

int sparse_mqa_bwd_dkv_dq(const void* kv, const int32_t* topk_idxs, void* dq, void* workspace, size_t workspace_bytes,
                          int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                          void* stream) {
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!smqa::dq_from_ds(H, D)) return SMQA_ERR_UNSUPPORTED;
  if (!kv || !topk_idxs || !dq) return SMQA_ERR_NULL;
  if (!aligned16(kv) || !aligned4(topk_idxs) || !aligned16(dq)) return SMQA_ERR_ALIGN;
  float scale;
  if ((st = resolve_scale(sm_scale, D, &scale))) return st;
  DkvPlan p;
  if ((st = single_pass_plan(workspace, workspace_bytes, B, S, S_kv, H, D, topk, 0, &p))) return st;
  const Span sdq{dq, count({B, S, H, D}) * 2};
  const Span others[] = {{kv, count({B, S_kv, D}) * 2}, {topk_idxs, count({B, S, topk}) * 4},
                         {workspace, (int64_t)p.end}};
  for (const Span& s : others)
    if (overlap(sdq, s)) return SMQA_ERR_ALIAS;
  char* ws = (char*)workspace;
  smqa::BwdMainArgs a{nullptr, kv, nullptr, topk_idxs, nullptr, nullptr, dq, nullptr, nullptr, nullptr, nullptr,
                      nullptr, B, S, S_kv, H, D, topk, scale, 0, B * S, (uint16_t*)(ws + p.ds)};
  return smqa::launch_bwd_dq_ds(a, (hipStream_t)stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
}

int sparse_mqa_bwd_dkv_reduce(void* dkv, int dkv_fp32, void* workspace, size_t workspace_bytes, int64_t B,
                              int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, void* stream) {
  int st = check_shapes(B, S, S_kv, H, D, topk);
  if (st) return st;
  if (!dkv) return SMQA_ERR_NULL;
  if (!aligned16(dkv)) return SMQA_ERR_ALIGN;
  DkvPlan p;
  if ((st = single_pass_plan(workspace, workspace_bytes, B, S, S_kv, H, D, topk, dkv_fp32, &p))) return st;
  if (overlap(Span{workspace, (int64_t)p.end}, Span{dkv, count({B, S_kv, D}) * (dkv_fp32 ? 4 : 2)}))
    return SMQA_ERR_ALIAS;
  char* ws = (char*)workspace;
  if (smqa::launch_reduce_rows((const uint16_t*)(ws + p.stage), (const int8_t*)(ws + p.stage_exp),
                               smqa::stage_segments(H, D), (const int32_t*)(ws + p.offset),
                               smqa::dkv_row_words(B * S, S), dkv_fp32 ? (float*)dkv : nullptr,
                               dkv_fp32 ? nullptr : dkv, 0, B * S_kv, D,
                               (hipStream_t)stream) != hipSuccess)
    return SMQA_ERR_HIP;
  return SMQA_OK;
}

int sparse_mqa_bwd_main(const void* q, const void* kv, const void* d_o, const int32_t* topk_idxs,
                        const float* lse, const float* delta, void* dq, float* dkv_accum, int64_t B, int64_t S,
                        int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale, void* stream) {
  float scale;
  int st = check_bwd_inputs(q, kv, d_o, topk_idxs, lse, B, S, S_kv, H, D, topk, sm_scale, &scale);
  if (st) return st;
  if (!delta || !dq || !dkv_accum) return SMQA_ERR_NULL;
  if (!aligned4(delta) || !aligned16(dq) || !aligned16(dkv_accum)) return SMQA_ERR_ALIGN;
  const int64_t qb = count({B, S, H, D}) * 2, ab = count({B, S_kv, D}) * 4;
  const Span sdq{dq, qb}, sacc{dkv_accum, ab};
  const Span ins[] = {{q, qb}, {kv, count({B, S_kv, D}) * 2}, {d_o, qb}, {topk_idxs, count({B, S, topk}) * 4},
                      {lse, count({B, S, H}) * 4}, {delta, count({B, S, H}) * 4}};
  for (const Span& s : ins)
    if (overlap(sdq, s) || overlap(sacc, s)) return SMQA_ERR_ALIAS;
  if (overlap(sdq, sacc)) return SMQA_ERR_ALIAS;
  smqa::BwdMainArgs a{q, kv, d_o, topk_idxs, lse, delta, dq, dkv_accum, nullptr, nullptr, nullptr, nullptr, B, S, S_kv,
                      H, D, topk, scale, 0, B * S};
  return smqa::launch_bwd_main(a, 3, (hipStream_t)stream) == hipSuccess ? SMQA_OK : SMQA_ERR_HIP;
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
                   size_t workspace_bytes, int64_t B, int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk,
                   float sm_scale, void* stream) {
  float scale;
  DkvPlan p;
  const int st = bwd_validate(q, kv, attn_sink, o, d_o, topk_idxs, lse, dq, dkv, dkv_fp32, workspace, workspace_bytes,
                              true, B, S, S_kv, H, D, topk, sm_scale, &scale, &p);
  if (st) return st;
  return bwd_launch(q, kv, o, d_o, topk_idxs, lse, dq, dkv, dkv_fp32, workspace, p, B, S, S_kv, H, D, topk, scale,
                    stream);
}

int sparse_mqa_bwd_noalloc(const void* q, const void* kv, const float* attn_sink, const void* o, const void* d_o,
                           const int32_t* topk_idxs, const float* lse, void* dq, void* dkv, int dkv_fp32, int64_t B,
                           int64_t S, int64_t S_kv, int64_t H, int64_t D, int64_t topk, float sm_scale,
                           void* stream) {
  // every argument check first, against a workspace of the scratch's size; then the scratch's
  // address (the only HIP calls before the launches: device queries and, once per device, the
  // symbol lookup)
  float scale;
  DkvPlan p;
  int st = bwd_validate(q, kv, attn_sink, o, d_o, topk_idxs, lse, dq, dkv, dkv_fp32, nullptr,
                        (size_t)SMQA_BWD_SCRATCH_BYTES, false, B, S, S_kv, H, D, topk, sm_scale, &scale, &p);
  if (st) return st;
  void* ws = nullptr;
  if ((st = scratch_for_stream((hipStream_t)stream, &ws))) return st;
  return bwd_launch(q, kv, o, d_o, topk_idxs, lse, dq, dkv, dkv_fp32, ws, p, B, S, S_kv, H, D, topk, scale, stream);
}

}  // extern "C"

// Backward kernels of top-k sparse MQA for gfx950 (see include/sparse_mqa.h for the contract).
//
//   preprocess   Delta[b,s,h] = <O, dO> in fp32                       (HBM stream)
//   fill_zero    clears the fp32 dKV accumulator (a kernel, so the sequence is graph-safe)
//   bwd_dq       per token: S^T, dP^T, P, dS, dQ^T += K^T dS^T      (bf16 MFMA 16x16x32)
//   bwd_dkv      per token: S^T, dP^T, P, dS, then dKV rows of the block
//                = (sm_scale dS)^T Q + P^T dO over all heads          (bf16 MFMA 32x32x16)
//                and a fp32 atomic add of each valid row into the accumulator. P and
//                sm_scale*dS enter this product as hi + lo bf16 pairs (two MFMAs each): a
//                kv row sums thousands of heavily cancelling terms, and single-bf16
//                coefficients leave errors of several percent of the result there.
//   postprocess  fp32 accumulator -> bf16 (round to nearest even)
// dQ and dKV run as two kernels: the per-token state both need (Q and dO in two layouts plus
// the dQ accumulator) does not fit one workgroup's registers at H = 64, D = 512.
// Both kernels gather a block of 32 slots into LDS with direct-to-LDS loads, double-buffered.
#include "device_common.h"
#include "launch.h"

namespace smqa {

__device__ __attribute__((aligned(16))) uint4 g_zero_row_bwd[64];

// Tile swizzle for the backward: 16 consecutive rows at one chunk and 8 consecutive rows at two
// adjacent chunks (the footprint of a transposing read over 32 lanes) both avoid bank conflicts.
__device__ __forceinline__ int bwd_swz(int row) {
  const int r = row & 15;
  return ((r & 7) << 1) | (r >> 3);
}
template <int D>
__device__ __forceinline__ int bwd_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ (bwd_swz(row) & (D / 8 - 1))) << 4);
}

// ---------------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, float* __restrict__ delta,
             int64_t rows) {
  constexpr int LPR = D / 8;   // lanes per row (16 bytes each)
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row = ((int64_t)blockIdx.x * 4 + w) * RPW + lane / LPR;
  const int chunk = lane % LPR;
  float s = 0.f;
  if (row < rows) {
    const bf16x8 a = load_bf16x8(o + row * D + chunk * 8);
    const bf16x8 c = load_bf16x8(dout + row * D + chunk * 8);
#pragma unroll
    for (int e = 0; e < 8; e++) s += (float)a[e] * (float)c[e];
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (row < rows && chunk == 0) delta[row] = s;
}

__global__ void __launch_bounds__(256) fill_zero_kernel(float4* __restrict__ p, int64_t n4) {
  const float4 z = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) p[i] = z;
}

__global__ void __launch_bounds__(256)
postprocess_kernel(const float4* __restrict__ acc, uint4* __restrict__ out, int64_t n8) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (int64_t)gridDim.x * 256) {
    const float4 a = acc[2 * i], c = acc[2 * i + 1];
    bf16x8 v;
    v[0] = (__bf16)a.x; v[1] = (__bf16)a.y; v[2] = (__bf16)a.z; v[3] = (__bf16)a.w;
    v[4] = (__bf16)c.x; v[5] = (__bf16)c.y; v[6] = (__bf16)c.z; v[7] = (__bf16)c.w;
    out[i] = __builtin_bit_cast(uint4, v);
  }
}

// ---------------------------------------------------------------------------------------------
// Shared pieces of the two main backward kernels. Workgroup = NW waves for one (token, block of
// 16*NW heads); wave w owns heads 16w..16w+15 for S^T and dP^T.
template <int D, int NW>
struct BwdCommon {
  static constexpr int T = 32;
  static constexpr int ROWB = D * 2;
  static constexpr int CPR = D / 8;
  static constexpr int TB = T * ROWB;
  static constexpr int RPI = 1024 / ROWB;
  static constexpr int NINSTR = T / RPI;
};

template <int D, int NW>
__device__ __forceinline__ void bwd_issue_tile(const char* kv_b, int32_t my_idx, uint64_t mask, char* tile,
                                               int lane, int w) {
  using C = BwdCommon<D, NW>;
  for (int ins = w; ins < C::NINSTR; ins += NW) {
    const int r = ins * C::RPI + lane / C::CPR;
    const int p = lane % C::CPR;
    const int c = p ^ (bwd_swz(r) & (C::CPR - 1));
    const int32_t ri = __shfl(my_idx, r);
    const bool v = (mask >> r) & 1ull;
    const char* src = v ? kv_b + (int64_t)ri * C::ROWB + c * 16 : (const char*)g_zero_row_bwd + c * 16;
    dma16(src, tile + ins * 1024);
  }
}

// S^T and dP^T of one 32-slot block for this wave's 16 heads: C layout lane l holds head
// (l & 15) and slots 16 mt + 4 (l>>4) + r.
template <int D>
__device__ __forceinline__ void bwd_scores(const char* tile, const bf16x8* qb, const bf16x8* dob, int lane,
                                           f32x4* sacc, f32x4* dpacc) {
  const int g = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) { sacc[mt][r] = 0.f; dpacc[mt][r] = 0.f; }
#pragma unroll
  for (int ks = 0; ks < D / 32; ks++) {
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      const bf16x8 a = lds_load16(tile + bwd_off<D>(16 * mt + (lane & 15), 4 * ks + g));
      sacc[mt] = mfma16(a, qb[ks], sacc[mt]);
      dpacc[mt] = mfma16(a, dob[ks], dpacc[mt]);
    }
  }
}

// ---------------------------------------------------------------------------------------------
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
              const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
              uint16_t* __restrict__ dq, int S, int64_t S_kv, int H, int topk, float sm_scale, float scale_log2,
              int n_hblk, int n_tokens) {
  using C = BwdCommon<D, NW>;
  constexpr int T = C::T;
  __shared__ __attribute__((aligned(16))) char smem[2 * C::TB];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4;
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int head = hblk * 16 * NW + 16 * w + (lane & 15);

  bf16x8 qb[D / 32], dob[D / 32];
  {
    const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 32; ks++) {
      qb[ks] = load_bf16x8(q + off + 32 * ks);
      dob[ks] = load_bf16x8(dout + off + 32 * ks);
    }
  }
  const float lse_h = lse[token * H + head];
  const float delta_h = delta[token * H + head];

  f32x4 dqacc[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; dt++)
#pragma unroll
    for (int r = 0; r < 4; r++) dqacc[dt][r] = 0.f;

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const char* kv_b = (const char*)(kv + b * S_kv * D);
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };

  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) bwd_issue_tile<D, NW>(kv_b, idx_cur, mask_cur, smem, lane, w);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;

  for (int blk = 0; blk < nblk; blk++) {
    const int buf = blk & 1;
    wait_all_mem();
    __syncthreads();
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) {
      mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
      if (mask_nxt) bwd_issue_tile<D, NW>(kv_b, idx_nxt, mask_nxt, smem + (buf ^ 1) * C::TB, lane, w);
    }
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) continue;

    const char* tile = smem + buf * C::TB;
    f32x4 sacc[2], dpacc[2];
    bwd_scores<D>(tile, qb, dob, lane, sacc, dpacc);
    // dS as the B operand of dQ^T = K^T dS^T: element e <-> slot 4g + e (e < 4), 16 + 4g + e - 4.
    bf16x8 dsb;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = 16 * mt + 4 * g + r;
        const float p = ((mask >> t) & 1ull) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
        dsb[4 * mt + r] = (__bf16)(p * (dpacc[mt][r] - delta_h));
      }
    const int t0 = 4 * g + ((lane & 15) >> 2);
#pragma unroll
    for (int dt = 0; dt < D / 16; dt++) {
      const int d = 16 * dt + 4 * (lane & 3);
      const int hoff = (d & 4) ? 8 : 0;
      const s16x4 lo = lds_load_tr(tile + bwd_off<D>(t0, d >> 3) + hoff);
      const s16x4 hi = lds_load_tr(tile + bwd_off<D>(t0 + 16, d >> 3) + hoff);
      dqacc[dt] = mfma16(join_tr(lo, hi), dsb, dqacc[dt]);
    }
  }

  // dQ^T C layout: lane holds head (lane & 15), d = 16 dt + 4 g + r.
  uint16_t* dqrow = dq + (token * H + head) * (int64_t)D;
#pragma unroll
  for (int dt = 0; dt < D / 16; dt++)
    *(uint2*)(dqrow + 16 * dt + 4 * g) = pack4_bf16(dqacc[dt][0] * sm_scale, dqacc[dt][1] * sm_scale,
                                                    dqacc[dt][2] * sm_scale, dqacc[dt][3] * sm_scale);
}

// ---------------------------------------------------------------------------------------------
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
bwd_dkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
               const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
               float* __restrict__ dkv_acc, int S, int64_t S_kv, int H, int topk, float sm_scale,
               float scale_log2, int n_hblk, int n_tokens) {
  using C = BwdCommon<D, NW>;
  constexpr int T = C::T;
  constexpr int HB = 16 * NW;   // heads of this workgroup
  constexpr int DW = D / NW;    // d-columns of dKV owned by one wave
  constexpr int NDT = DW / 32;
  constexpr int KS = HB / 16;   // 16-head k-steps of the dKV product
  static_assert(NDT >= 1, "each wave needs at least one 32-wide d tile");
  constexpr int SB = HB * T * 2;  // bytes of one [HB][T] bf16 buffer
  __shared__ __attribute__((aligned(16))) char smem[2 * C::TB + 4 * SB];
  char* dsbuf = smem + 2 * C::TB;  // hi parts
  char* pbuf = dsbuf + SB;
  char* dslo = pbuf + SB;          // lo parts: x - float(bf16(x)), rounded to bf16
  char* plo = dslo + SB;

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, kg = lane >> 5;
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int hrow = 16 * w + (lane & 15);          // head within the workgroup's block
  const int head = hblk * HB + hrow;

  // (1) Q and dO with heads along k, as B operands of dKV = (sm_scale dS)^T Q + P^T dO:
  // lane l holds d = w*DW + 32 dt + (l & 31) and heads 16 ks + 8 kg .. +7, read with transposing
  // LDS loads from a row-major [HB][D] staging copy (the tile buffers are free at this point).
  static_assert(HB * D * 2 <= 2 * C::TB, "staging copy must fit the tile buffers");
  bf16x8 qv[NDT][KS], dov[NDT][KS];
  {
    const int64_t base = (token * H + (int64_t)hblk * HB) * D;
    for (int pass = 0; pass < 2; pass++) {
      const uint16_t* src = (pass == 0 ? q : dout) + base;
      for (int i = threadIdx.x; i < HB * D / 8; i += NW * 64)
        *(uint4*)(smem + 16 * i) = *(const uint4*)(src + 8 * i);
      __syncthreads();
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const int h0 = 16 * ks + 8 * kg + ((lane & 15) >> 2);
          const int d = w * DW + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const s16x4 lo = lds_load_tr(smem + (h0 * D + d) * 2);
          const s16x4 hi = lds_load_tr(smem + ((h0 + 4) * D + d) * 2);
          if (pass == 0) qv[dt][ks] = join_tr(lo, hi);
          else dov[dt][ks] = join_tr(lo, hi);
        }
      __syncthreads();
    }
  }
  // (2) Q and dO with d along k, as B operands of S^T and dP^T (this wave's 16 heads).
  bf16x8 qb[D / 32], dob[D / 32];
  {
    const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < D / 32; ks++) {
      qb[ks] = load_bf16x8(q + off + 32 * ks);
      dob[ks] = load_bf16x8(dout + off + 32 * ks);
    }
  }
  const float lse_h = lse[token * H + head];
  const float delta_h = delta[token * H + head];

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const char* kv_b = (const char*)(kv + b * S_kv * D);
  float* acc_b = dkv_acc + b * S_kv * D;
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };

  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) bwd_issue_tile<D, NW>(kv_b, idx_cur, mask_cur, smem, lane, w);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;

  for (int blk = 0; blk < nblk; blk++) {
    const int buf = blk & 1;
    wait_all_mem();
    __syncthreads();  // tile ready; dsbuf / pbuf of the previous block fully consumed
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) {
      mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
      if (mask_nxt) bwd_issue_tile<D, NW>(kv_b, idx_nxt, mask_nxt, smem + (buf ^ 1) * C::TB, lane, w);
    }
    const int32_t idx_this = idx_cur;
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) continue;

    const char* tile = smem + buf * C::TB;
    f32x4 sacc[2], dpacc[2];
    bwd_scores<D>(tile, qb, dob, lane, sacc, dpacc);
    // P and sm_scale*dS, stored [head][slot] in bf16 (four consecutive slots per lane).
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      float p[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const int t = 16 * mt + 4 * g + r;
        p[r] = ((mask >> t) & 1ull) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
        ds[r] = sm_scale * p[r] * (dpacc[mt][r] - delta_h);
      }
      float plr[4], dslr[4];
#pragma unroll
      for (int r = 0; r < 4; r++) {
        plr[r] = p[r] - (float)(__bf16)p[r];
        dslr[r] = ds[r] - (float)(__bf16)ds[r];
      }
      const int off = (hrow * T + 16 * mt + 4 * g) * 2;
      *(uint2*)(pbuf + off) = pack4_bf16(p[0], p[1], p[2], p[3]);
      *(uint2*)(dsbuf + off) = pack4_bf16(ds[0], ds[1], ds[2], ds[3]);
      *(uint2*)(plo + off) = pack4_bf16(plr[0], plr[1], plr[2], plr[3]);
      *(uint2*)(dslo + off) = pack4_bf16(dslr[0], dslr[1], dslr[2], dslr[3]);
    }
    __syncthreads();

    // dKV rows of the block for this wave's d-range. A operand = [slot][head] via transposing
    // reads of the [head][slot] buffers: lane l holds slot (l & 31), heads 16 ks + 8 kg .. +7.
    int32_t rowi[16];
#pragma unroll
    for (int r = 0; r < 16; r++) rowi[r] = __shfl(idx_this, 8 * (r >> 2) + 4 * kg + (r & 3));
    const int hl = 8 * kg + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int dt = 0; dt < NDT; dt++) {
      f32x16 c;
#pragma unroll
      for (int r = 0; r < 16; r++) c[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const int o0 = (16 * ks + hl) * T * 2 + tcol * 2, o1 = o0 + 4 * T * 2;
        const bf16x8 ads = join_tr(lds_load_tr(dsbuf + o0), lds_load_tr(dsbuf + o1));
        const bf16x8 adl = join_tr(lds_load_tr(dslo + o0), lds_load_tr(dslo + o1));
        const bf16x8 aph = join_tr(lds_load_tr(pbuf + o0), lds_load_tr(pbuf + o1));
        const bf16x8 apl = join_tr(lds_load_tr(plo + o0), lds_load_tr(plo + o1));
        c = mfma32(ads, qv[dt][ks], c);
        c = mfma32(adl, qv[dt][ks], c);
        c = mfma32(aph, dov[dt][ks], c);
        c = mfma32(apl, dov[dt][ks], c);
      }
      // C layout: lane holds d = w*DW + 32 dt + (lane & 31), slots 8 (r>>2) + 4 kg + (r&3).
      const int d = w * DW + 32 * dt + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int t = 8 * (r >> 2) + 4 * kg + (r & 3);
        if ((mask >> t) & 1ull) unsafeAtomicAdd(acc_b + (int64_t)rowi[r] * D + d, c[r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t rows, int64_t D,
                                 hipStream_t st) {
  const int64_t rpb = 4 * (64 / (D / 8));  // rows per 256-thread block
  const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(256);
  if (D == 512)
    hipLaunchKernelGGL(delta_kernel<512>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else if (D == 64)
    hipLaunchKernelGGL(delta_kernel<64>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fill_zero_f32(float* p, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  int64_t blocks = (n4 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (float4*)p, n4);
  return hipGetLastError();
}

hipError_t launch_bwd_postprocess(const float* acc, void* dkv, int64_t n, hipStream_t st) {
  const int64_t n8 = n / 8;
  int64_t blocks = (n8 + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(postprocess_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (const float4*)acc, (uint4*)dkv, n8);
  return hipGetLastError();
}

template <int D, int NW>
static hipError_t launch_bwd_main_t(const BwdMainArgs& a, int which, hipStream_t st) {
  const int n_hblk = (int)(a.H / (16 * NW));
  const int n_tokens = (int)(a.B * a.S);
  const dim3 grid((unsigned)(n_tokens * n_hblk)), block(NW * 64);
  const float sl2 = a.sm_scale * kLog2e;
  if (which & 1) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), grid, block, 0, st, (const uint16_t*)a.q, (const uint16_t*)a.kv,
                       (const uint16_t*)a.d_o, a.idx, a.lse, a.delta, (uint16_t*)a.dq, (int)a.S, a.S_kv, (int)a.H,
                       (int)a.topk, a.sm_scale, sl2, n_hblk, n_tokens);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(which & 2)) return hipSuccess;
  hipLaunchKernelGGL((bwd_dkv_kernel<D, NW>), grid, block, 0, st, (const uint16_t*)a.q, (const uint16_t*)a.kv,
                     (const uint16_t*)a.d_o, a.idx, a.lse, a.delta, a.dkv_accum, (int)a.S, a.S_kv, (int)a.H,
                     (int)a.topk, a.sm_scale, sl2, n_hblk, n_tokens);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdMainArgs& a, int which, hipStream_t st) {
  const int hb = a.H >= 64 ? 64 : (int)a.H;
  if (a.D == 512) {
    if (hb == 64) return launch_bwd_main_t<512, 4>(a, which, st);
    if (hb == 32) return launch_bwd_main_t<512, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<512, 1>(a, which, st);
  } else if (a.D == 64) {
    if (hb == 32) return launch_bwd_main_t<64, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<64, 1>(a, which, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace smqa

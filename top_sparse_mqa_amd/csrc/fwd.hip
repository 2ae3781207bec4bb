// Forward kernel of top-k sparse MQA for gfx950 (see include/sparse_mqa.h for the contract).
//
// One workgroup per (query token, block of up to 64 heads). All heads of a token share the
// gathered kv rows, so each block of 64 slots is gathered once into LDS (direct-to-LDS
// global_load_lds_dwordx4, double-buffered) and used by every head:
//   S^T[slot, head] = K[slot, :] . Q[head, :]^T    bf16 MFMA 32x32x16, K from LDS, Q in VGPRs
//   online softmax in log2 units, sink folded into the running max and sum
//   O^T[d, head]   += V^T[d, slot] . P^T[slot, head]  bf16 MFMA, V^T read with ds_read_b64_tr_b16
// Waves are (head group of 32) x (half). For S^T a wave owns 32 slots of the block; for the
// P.V product it owns half of D. The two halves of a head group swap their block maxima and
// their bf16 P through LDS.
#include "device_common.h"
#include "launch.h"

namespace smqa {

// Source of masked slots' tile rows: masked slots are never read from kv.
__device__ __attribute__((aligned(16))) uint4 g_zero_row[64];

__device__ __forceinline__ int fwd_swz(int row) {
  const int r = row & 15;
  return ((r & 3) << 2) | (r >> 2);
}
template <int D>
__device__ __forceinline__ int fwd_off(int row, int chunk) {
  return row * (D * 2) + ((chunk ^ (fwd_swz(row) & (D / 8 - 1))) << 4);
}

template <int D, int NHG>
__global__ void __launch_bounds__(NHG * 128)
fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
           const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int S,
           int64_t S_kv, int H, int topk, float scale_log2, int n_hblk, int n_tokens) {
  constexpr int T = 64;
  constexpr int NW = 2 * NHG;
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int TB = T * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int NINSTR = T / RPI;
  constexpr int MAXB = NHG * 2 * 32 * 4;
  constexpr int PB = NHG * 2 * 2 * 64 * 16;
  __shared__ __attribute__((aligned(16))) char smem[2 * TB + MAXB + PB + MAXB];
  char* tiles = smem;
  float* maxbuf = (float*)(smem + 2 * TB);
  uint4* pbuf = (uint4*)(smem + 2 * TB + MAXB);
  float* lbuf = (float*)(smem + 2 * TB + MAXB + PB);

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hg = w >> 1, half = w & 1;
  const int kg = lane >> 5;
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;  // heavier (later) tokens first
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int head = hblk * 32 * NHG + 32 * hg + (lane & 31);
  const bool head_ok = head < H;

  // Q as the B operand of S^T = K Q^T: lane holds head (lane & 31), d = 16 ks + 8 kg .. +7.
  bf16x8 qb[D / 16];
  {
    const uint16_t* qrow = q + (token * H + (head_ok ? head : 0)) * (int64_t)D + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) qb[ks] = head_ok ? load_bf16x8(qrow + 16 * ks) : zero_bf16x8();
  }
  const float sink2 = head_ok ? sink[head] * kLog2e : 0.f;
  float m_run = sink2;
  // The sink's term of the denominator is carried by one lane per head.
  float l_run = (half == 0 && kg == 0 && sink2 != -INFINITY) ? 1.f : 0.f;

  f32x16 oacc[D / 64];
#pragma unroll
  for (int dt = 0; dt < D / 64; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[dt][r] = 0.f;

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const char* kv_b = (const char*)(kv + b * S_kv * D);

  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return t < topk ? idx_tok[t] : -1;
  };
  auto issue_tile = [&](int32_t my_idx, uint64_t mask, int buf) {
    char* tile = tiles + buf * TB;
    for (int ins = w; ins < NINSTR; ins += NW) {
      const int r = ins * RPI + lane / CPR;
      const int p = lane % CPR;
      const int c = p ^ (fwd_swz(r) & (CPR - 1));
      const int32_t ri = __shfl(my_idx, r);
      const bool v = (mask >> r) & 1ull;
      const char* src = v ? kv_b + (int64_t)ri * ROWB + c * 16 : (const char*)g_zero_row + c * 16;
      dma16(src, tile + ins * 1024);
    }
  };

  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) issue_tile(idx_cur, mask_cur, 0);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;

  for (int blk = 0; blk < nblk; blk++) {
    const int buf = blk & 1;
    wait_all_mem();
    __syncthreads();  // tile blk is in LDS; every wave is done with block blk-1
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) {
      mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
      if (mask_nxt) issue_tile(idx_nxt, mask_nxt, buf ^ 1);
    }
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) continue;

    const char* tile = tiles + buf * TB;
    // ---- S^T for this wave's 32 slots x 32 heads
    f32x16 sacc0, sacc1;
#pragma unroll
    for (int r = 0; r < 16; r++) { sacc0[r] = 0.f; sacc1[r] = 0.f; }
    const int arow = 32 * half + (lane & 31);
#pragma unroll
    for (int ks = 0; ks < D / 16; ks += 2) {
      const bf16x8 a0 = lds_load16(tile + fwd_off<D>(arow, 2 * ks + kg));
      const bf16x8 a1 = lds_load16(tile + fwd_off<D>(arow, 2 * ks + 2 + kg));
      sacc0 = mfma32(a0, qb[ks], sacc0);
      sacc1 = mfma32(a1, qb[ks + 1], sacc1);
    }
    // ---- masked scores in log2 units, block max per head
    float s2[16];
    float bmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int t = 32 * half + 8 * (r >> 2) + 4 * kg + (r & 3);
      const float v = (sacc0[r] + sacc1[r]) * scale_log2;
      s2[r] = ((mask >> t) & 1ull) ? v : -INFINITY;
      bmax = fmaxf(bmax, s2[r]);
    }
    bmax = wave_max_xor32(bmax);
    float* mb = maxbuf + hg * 64;
    if (kg == 0) mb[half * 32 + (lane & 31)] = bmax;
    __syncthreads();
    const float pmax = mb[(half ^ 1) * 32 + (lane & 31)];
    const float m_new = fmaxf(m_run, fmaxf(bmax, pmax));  // finite: the block has a valid slot
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;

    float psum = 0.f;
    bf16x8 pown[2];
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const float p = exp2f(s2[r] - m_new);
      psum += p;
      pown[r >> 3][r & 7] = (__bf16)p;
    }
    l_run = l_run * alpha + psum;

    uint4* pb = pbuf + hg * 256;
    pb[half * 128 + lane] = __builtin_bit_cast(uint4, pown[0]);
    pb[half * 128 + 64 + lane] = __builtin_bit_cast(uint4, pown[1]);
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < D / 64; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] *= alpha;
    }
    __syncthreads();
    bf16x8 ppart[2];
    ppart[0] = __builtin_bit_cast(bf16x8, pb[(half ^ 1) * 128 + lane]);
    ppart[1] = __builtin_bit_cast(bf16x8, pb[(half ^ 1) * 128 + 64 + lane]);

    // ---- O^T[d, head] += V^T[d, slot] P^T[slot, head] over the 64 slots, for this wave's half of D.
    // k-order of a 16-slot step (hs, j): element e <-> slot 32 hs + 16 j + 8 (e>>2) + 4 kg + (e&3),
    // which is the C-layout order of S^T, so P needs no shuffle.
    const int dbase = half * (D / 2);
#pragma unroll
    for (int hs = 0; hs < 2; hs++) {
#pragma unroll
      for (int j = 0; j < 2; j++) {
        const bf16x8 bop = (hs == half) ? pown[j] : ppart[j];
        const int t0 = 32 * hs + 16 * j + 4 * kg + ((lane & 15) >> 2);
#pragma unroll
        for (int dt = 0; dt < D / 64; dt++) {
          const int d = dbase + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          const int hoff = (d & 4) ? 8 : 0;
          const s16x4 lo = lds_load_tr(tile + fwd_off<D>(t0, d >> 3) + hoff);
          const s16x4 hi = lds_load_tr(tile + fwd_off<D>(t0 + 8, d >> 3) + hoff);
          oacc[dt] = mfma32(join_tr(lo, hi), bop, oacc[dt]);
        }
      }
    }
  }

  // ---- epilogue: total denominator, normalise, store O (bf16) and LSE (log2)
  float ltot = l_run + __shfl_xor(l_run, 32);
  float* lb = lbuf + hg * 64;
  if (kg == 0) lb[half * 32 + (lane & 31)] = ltot;
  __syncthreads();
  ltot += lb[(half ^ 1) * 32 + (lane & 31)];
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (head_ok) {
    uint16_t* orow = out + (token * H + head) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < D / 64; dt++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int d = half * (D / 2) + 32 * dt + 8 * r4 + 4 * kg;
        *(uint2*)(orow + d) = pack4_bf16(oacc[dt][4 * r4] * inv, oacc[dt][4 * r4 + 1] * inv,
                                         oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv);
      }
    if (half == 0 && kg == 0) lse[token * H + head] = ltot > 0.f ? m_run + log2f(ltot) : -INFINITY;
  }
}

template <int D, int NHG>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int n_hblk = (int)((a.H + 32 * NHG - 1) / (32 * NHG));
  const int n_tokens = (int)(a.B * a.S);
  const dim3 grid((unsigned)(n_tokens * n_hblk)), block(NHG * 128);
  hipLaunchKernelGGL((fwd_kernel<D, NHG>), grid, block, 0, st, (const uint16_t*)a.q, (const uint16_t*)a.kv,
                     a.sink, a.idx, (uint16_t*)a.o, a.lse, (int)a.S, a.S_kv, (int)a.H, (int)a.topk,
                     a.sm_scale * kLog2e, n_hblk, n_tokens);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.D == 512) return a.H <= 32 ? launch_fwd_t<512, 1>(a, st) : launch_fwd_t<512, 2>(a, st);
  if (a.D == 64) return a.H <= 32 ? launch_fwd_t<64, 1>(a, st) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

}  // namespace smqa

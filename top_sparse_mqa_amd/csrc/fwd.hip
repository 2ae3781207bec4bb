// Forward kernels of top-k sparse MQA for gfx950 (see include/sparse_mqa.h for the contract).
// fwd_ws_kernel (below) serves D = 512 with blocks of 64 heads; fwd_kernel serves every other
// shape.
//
// One workgroup per (query token, block of up to 64 heads). All heads of a token share the
// gathered kv rows, so each block of 64 slots is gathered once into LDS (direct-to-LDS
// global_load_lds_dwordx4, double-buffered) and used by every head:
//   S^T[slot, head] = K[slot, :] . Q[head, :]^T    bf16 MFMA 32x32x16, K from LDS, Q in VGPRs
//   online softmax in log2 units, sink folded into the running max and sum
//   (RR: the scaled logit is rounded to fp32 in natural units first, and the max is subtracted
//   before the change to base 2; LSE is written in log2 units either way)
//   O^T[d, head]   += V^T[d, slot] . P^T[slot, head]  bf16 MFMA, V^T read with ds_read_b64_tr_b16
// Waves are (head group of 32) x (half of D). Each wave keeps Q for its half of D, computes a
// partial S^T over that half for all 64 slots, and swaps the fp32 partials with the other half
// through LDS; both then hold the full scores, run the softmax redundantly and accumulate O for
// their own half of D.
#include "device_common.h"
#include "launch.h"

namespace smqa {

// Source of masked slots' tile rows: masked slots are never read from kv.
__device__ __attribute__((aligned(16))) uint4 g_zero_row[64];

__device__ __forceinline__ int fwd_swz(int row) {
  const int r = row & 15;
  return ((r & 3) << 2) | (r >> 2);
}

// score_scale multiplies the fp32 dot product: sm_scale * log2(e) (scores in log2 units), or
// sm_scale alone when RR (scores in natural units, the fwd page's reference_rounding option).
template <int D, int NHG, bool RR>
__global__ void __launch_bounds__(NHG * 128)
fwd_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
           const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int S,
           int64_t S_kv, int H, int topk, float score_scale, int n_hblk, int n_tokens) {
  // EU turns a difference of scores into log2 units; MAXSTEP is 8 in log2 units.
  constexpr float EU = RR ? kLog2e : 1.f;
  constexpr float MAXSTEP = RR ? 8.f * 0.693147180559945309f : 8.f;
  constexpr int T = 64;           // slots per block
  constexpr int NW = 2 * NHG;     // waves
  constexpr int DH = D / 2;       // d-columns owned by one wave of a head-group pair
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int TB = T * ROWB;
  constexpr int RPI = 1024 / ROWB;
  constexpr int NINSTR = T / RPI;
  constexpr int XB = 2 * 16 * 64 * 4;  // one wave's partial S^T: 2 tiles x 16 regs x 64 lanes fp32
  constexpr int KS = DH / 16;          // k-steps of the S^T product
  constexpr int NDT = DH / 32;         // 32-wide d tiles of O^T
  constexpr int PFS = 4;               // S fragment reads in flight
  constexpr int NFV = 4 * NDT;         // V fragments per block
  constexpr int PFV = NFV < 4 ? NFV : 4;  // V fragment reads in flight
  // The two tile buffers are distinct LDS arrays and the block loop is unrolled by two, so every
  // read names its buffer at compile time and is not made to wait for the gather in flight into
  // the other one.
  __shared__ __attribute__((aligned(16))) char tile0[TB];
  __shared__ __attribute__((aligned(16))) char tile1[TB];
  __shared__ __attribute__((aligned(16))) char xbuf[NW * XB];

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

  // Q for this wave's half of D, as the B operand of S^T = K Q^T:
  // lane holds head (lane & 31), d = half*DH + 16 ks + 8 kg .. +7.
  bf16x8 qb[KS];
  {
    const uint16_t* qrow = q + (token * H + (head_ok ? head : 0)) * (int64_t)D + half * DH + 8 * kg;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) qb[ks] = head_ok ? load_bf16x8(qrow + 16 * ks) : zero_bf16x8();
#pragma unroll
    for (int ks = 0; ks < KS; ks++) keep_in_agpr(qb[ks]);
  }
  const float sink2 = head_ok ? (RR ? sink[head] : sink[head] * kLog2e) : 0.f;
  float m_run = sink2;
  // The sink's share of the denominator is carried by the kg == 0 lane of each head.
  float l_run = (kg == 0 && sink2 != -INFINITY) ? 1.f : 0.f;

  f32x16 oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) oacc[dt][r] = 0.f;

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const char* kv_b = (const char*)(kv + b * S_kv * D);

  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return t < topk ? idx_tok[t] : -1;
  };
  const int wu = __builtin_amdgcn_readfirstlane(w);  // wave index as a scalar
  auto issue_tile = [&](int32_t my_idx, uint64_t mask, char* tile) {
    if constexpr (RPI == 1) {
      // One kv row per instruction, through a buffer resource: row index and validity are
      // wave-uniform, the row offset goes in the scalar offset; masked rows read the zero row.
      // The lane id is passed through an empty asm so the per-row lane offsets are computed
      // here instead of being hoisted out of the block loop into 16 live registers.
      const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv_b, (int)(uint32_t)(S_kv * ROWB));
      const __amdgpu_buffer_rsrc_t rz = make_rsrc(g_zero_row, ROWB);
      int ln = lane;
      asm volatile("" : "+v"(ln));
#pragma unroll
      for (int i = 0; i < NINSTR / NW; i++) {
        const int r = wu + NW * i;
        const int32_t ri = __builtin_amdgcn_readlane(my_idx, r);
        const uint32_t voff = (uint32_t)((ln ^ (fwd_swz(r) & (CPR - 1))) << 4);
        if ((mask >> r) & 1ull) dma16_buf(rk, voff, (uint32_t)ri * ROWB, tile + r * ROWB);
        else dma16_buf(rz, voff, 0, tile + r * ROWB);
      }
    } else {
      for (int ins = wu; ins < NINSTR; ins += NW) {
        const int r = ins * RPI + lane / CPR;
        const int p = lane % CPR;
        const int c = p ^ (fwd_swz(r) & (CPR - 1));
        const int32_t ri = __shfl(my_idx, r);
        const bool v = (mask >> r) & 1ull;
        const char* src = v ? kv_b + (int64_t)ri * ROWB + c * 16 : (const char*)g_zero_row + c * 16;
        dma16(src, tile + ins * 1024);
      }
    }
  };

  // Per-lane parts of the LDS addresses, fixed for the whole kernel. The XOR swizzle only touches
  // the low four chunk bits, so chunks 16 apart differ by 256 bytes (an instruction offset).
  // S^T reads: row (lane & 31) (+32 for the second tile), chunk half*DH/8 + 2 ks + kg.
  constexpr int KSJ = KS < 8 ? KS : 8;
  const int arow = lane & 31;
  int qk_off[KSJ];
#pragma unroll
  for (int j = 0; j < KSJ; j++)
    qk_off[j] = arow * ROWB + (((half * (DH / 8) + 2 * j + kg) ^ (fwd_swz(arow) & (CPR - 1))) << 4);
  // V^T reads: row t0 (+8 for the upper k-half), chunk c0 + 4 dt; pv_off[a][k] covers dt % NK == k.
  const int t0 = 4 * kg + ((lane & 15) >> 2);
  const int c0 = (half * DH + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) >> 3;
  const int hoff = (lane & 1) ? 8 : 0;
  constexpr int NK = NDT < 4 ? NDT : 4;
  int pv_off[2][NK];
#pragma unroll
  for (int a = 0; a < 2; a++)
#pragma unroll
    for (int k = 0; k < NK; k++)
      pv_off[a][k] = (t0 + 8 * a) * ROWB + (((c0 + 4 * k) ^ (fwd_swz(t0 + 8 * a) & (CPR - 1))) << 4) + hoff;
  float4* xmine = (float4*)(xbuf + w * XB);
  const float4* xpart = (const float4*)(xbuf + (w ^ 1) * XB);

  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) issue_tile(idx_cur, mask_cur, tile0);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;

  auto block = [&](auto buf_tag, int blk) {
    constexpr int BUF = decltype(buf_tag)::value;
    const char* tile = BUF ? tile1 : tile0;
    char* other = BUF ? tile0 : tile1;
    wait_all_mem();
    __syncthreads();  // tile blk is in LDS; every wave is done with block blk-1
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) {
      mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
      if (mask_nxt) issue_tile(idx_nxt, mask_nxt, other);
    }
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) return;

    // ---- partial S^T over this wave's half of D, for all 64 slots (two 32-slot tiles).
    // Fragment i = (ks, mt) = (i / 2, i % 2); PFS reads run ahead of their MFMAs, every stage
    // fenced so the scheduler keeps that distance.
    f32x16 sacc[2];
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) sacc[mt][r] = 0.f;
    {
      constexpr int NF = 2 * KS, NB = PFS + 1;
      auto sfrag = [&](int i) {
        const int ks = i >> 1, mt = i & 1;
        return lds_load16(tile + qk_off[ks % KSJ] + 256 * (ks / KSJ) + 32 * mt * ROWB);
      };
      bf16x8 fr[NB];
#pragma unroll
      for (int i = 0; i < PFS; i++) fr[i] = sfrag(i);
#pragma unroll
      for (int i = 0; i < NF; i++) {
        __builtin_amdgcn_sched_barrier(0);
        if (i + PFS < NF) fr[(i + PFS) % NB] = sfrag(i + PFS);
        sacc[i & 1] = mfma32(fr[i % NB], qb[i >> 1], sacc[i & 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // ---- swap partial sums with the other half of the head group
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++)
        xmine[(mt * 4 + r4) * 64 + lane] = make_float4(sacc[mt][4 * r4], sacc[mt][4 * r4 + 1],
                                                       sacc[mt][4 * r4 + 2], sacc[mt][4 * r4 + 3]);
    lds_barrier();  // partial sums visible; the next tile's gather stays in flight
    // the first V fragments are read while the softmax below runs
    constexpr int NBV = PFV + 1;
    auto vfrag = [&](int i) {
      // i = (k-step kk = (mt, j), d tile dt); k-step kk covers slots 16 kk .. 16 kk + 15
      const int kk = i / NDT, dt = i % NDT;
      const int imm = 16 * kk * ROWB + 256 * (dt / NK);
      return join_tr(lds_load_tr(tile + pv_off[0][dt % NK] + imm), lds_load_tr(tile + pv_off[1][dt % NK] + imm));
    };
    bf16x8 fv[NBV];
#pragma unroll
    for (int i = 0; i < PFV; i++) fv[i] = vfrag(i);

    float bmax = -INFINITY;
    // validity of this lane's slots, bit 32 mt + 8 r4 + i for C element (mt, 4 r4 + i); one
    // variable shift keeps the compiler from hoisting per-slot 64-bit masks out of the loop
    const uint64_t vb = mask >> (4 * kg);
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const float4 o = xpart[(mt * 4 + r4) * 64 + lane];
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const int r = 4 * r4 + i;
          const float v = (sacc[mt][r] + ov[i]) * score_scale;
          sacc[mt][r] = ((vb >> (32 * mt + 8 * r4 + i)) & 1ull) ? v : -INFINITY;
          bmax = fmaxf(bmax, sacc[mt][r]);
        }
      }
    bmax = wave_max_xor32(bmax);  // block max of this head over the 64 slots
    // The running max only moves when the block exceeds it by more than 8 (log2 units), so P
    // stays <= 2^8 and the O rescale below runs on a few blocks only; O / l and m + log2(l)
    // do not depend on where the max sits.
    const float m_new = (bmax > m_run + MAXSTEP) ? bmax : m_run;  // bmax is finite: a slot is valid
    const float alpha = fast_exp2((m_run - m_new) * EU);
    m_run = m_new;

    float psum = 0.f;
    bf16x8 pb[2][2];  // B operand of O^T += V^T P^T: k-step (mt, j)
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const float p = fast_exp2((sacc[mt][r] - m_new) * EU);
        psum += p;
        pb[mt][r >> 3][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][r] *= alpha;
    }

    // ---- O^T[d, head] += V^T[d, slot] P^T[slot, head] over the 64 slots, this wave's half of D.
    // k-order of step (mt, j): element e <-> slot 32 mt + 16 j + 8 (e>>2) + 4 kg + (e&3), the
    // C-layout order of S^T, so P needs no shuffle.
#pragma unroll
    for (int i = 0; i < NFV; i++) {
      __builtin_amdgcn_sched_barrier(0);
      if (i + PFV < NFV) fv[(i + PFV) % NBV] = vfrag(i + PFV);
      const int kk = i / NDT, dt = i % NDT;
      oacc[dt] = mfma32(fv[i % NBV], pb[kk >> 1][kk & 1], oacc[dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    block(IntTag<0>{}, blk);
    if (blk + 1 < nblk) block(IntTag<1>{}, blk + 1);
  }

  // ---- epilogue: normalise, store O (bf16) and LSE (log2)
  const float ltot = l_run + __shfl_xor(l_run, 32);
  const float inv = ltot > 0.f ? 1.f / ltot : 0.f;
  if (head_ok) {
    uint16_t* orow = out + (token * H + head) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int d = half * DH + 32 * dt + 8 * r4 + 4 * kg;
        *(uint2*)(orow + d) = pack4_bf16(oacc[dt][4 * r4] * inv, oacc[dt][4 * r4 + 1] * inv,
                                         oacc[dt][4 * r4 + 2] * inv, oacc[dt][4 * r4 + 3] * inv);
      }
    if (half == 0 && kg == 0)
      lse[token * H + head] = ltot > 0.f ? (RR ? (m_run + logf(ltot)) * kLog2e : m_run + log2f(ltot)) : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------------
// Forward with specialised waves, for D = 512 and blocks of 64 heads: eight waves, two per SIMD,
// in two roles. RR as in fwd_kernel (scores in natural units, the max subtracted before the change
// to base 2).
//   Score waves (0-3) gather the 32-slot kv tiles (one 1 KiB row per direct-to-LDS instruction)
//   and compute S^T for 16 heads each (16x16x32 MFMAs, Q in AGPRs), then the online softmax
//   (running max and sum per head, sink included) and hand P (bf16, [head][slot]) and each head's
//   rescale factor to the O waves through LDS.
//   O waves (4-7) hold O^T for 128 d-columns of all 64 heads in registers and accumulate V^T P^T
//   one block behind (32x32x16 MFMAs, V^T from transposing LDS reads).
// Stage j runs block j on the score waves and block j - 1 on the O waves, and ends with one
// workgroup barrier; three tile buffers let the gather of tile j + 1 land in the one the O waves
// finished with. Both roles pass the same barriers (one before the stages, nblk + 1 stages, one
// before the epilogue). A SIMD thus overlaps one role's gather issue, softmax and LDS traffic
// with the other's MFMAs; with one wave per SIMD (fwd_kernel) they run one after another.
// Maximum over lanes l, l ^ 16, l ^ 32 and l ^ 48, with the two lane-swap instructions (no LDS
// round trip): a 16-lane swap leaves a lane holding its own value and that of l ^ 16, a 32-lane
// swap then pairs l with l ^ 32.
__device__ __forceinline__ float max_xor16_32(float m) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

__device__ __forceinline__ int fws_swz(int row) {
  const int r = row & 15;
  return ((r & 1) << 2) ^ (r & 10) ^ (((r >> 2) & 1) * 9);
}

template <int D, bool RR>
__global__ void __launch_bounds__(512)
fwd_ws_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const float* __restrict__ sink,
              const int32_t* __restrict__ idx, uint16_t* __restrict__ out, float* __restrict__ lse, int S,
              int64_t S_kv, int H, int topk, float score_scale, int n_hblk, int n_tokens) {
  constexpr int T = 32;           // slots per block
  constexpr int HB = 64;          // heads per workgroup
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int TB = T * ROWB;
  constexpr int KS = D / 32;      // k-steps of S^T
  constexpr int NF = 2 * KS;      // score fragments (k-step, 16-slot half)
  constexpr int PF = 6;           // score fragment reads in flight
  constexpr int NP = T / 8;       // gather instructions per wave and tile
  constexpr int DW = D / 4;       // O^T d-columns per O wave
  constexpr int NDT = DW / 32;    // its 32-wide d tiles
  constexpr int PB = HB * T * 2;  // bytes of one P buffer
  // EU turns a difference of scores into log2 units; MAXSTEP is 8 in log2 units.
  constexpr float EU = RR ? kLog2e : 1.f;
  constexpr float MAXSTEP = RR ? 8.f * 0.693147180559945309f : 8.f;
  static_assert(ROWB == 1024 && NDT * 32 == DW, "one kv row per gather instruction");
  __shared__ __attribute__((aligned(16))) char tile0[TB];
  __shared__ __attribute__((aligned(16))) char tile1[TB];
  __shared__ __attribute__((aligned(16))) char tile2[TB];
  __shared__ __attribute__((aligned(16))) char pbuf0[PB];
  __shared__ __attribute__((aligned(16))) char pbuf1[PB];
  __shared__ __attribute__((aligned(16))) char pbuf2[PB];
  __shared__ float alpha_s[3][HB];
  __shared__ float fin_l[HB];
  __shared__ __attribute__((aligned(16))) int32_t idx_ring[IdxRing::SLOTS];  // the token's indices
  __shared__ int last_s[4];  // last valid slot seen by each score wave

  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;  // heavier (later) tokens first
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  // Blocks after the last one holding a valid slot are skipped (when the ring holds every block):
  // a selection shorter than topk is padded with masked slots at its end.
  int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };
  // the score waves fill the ring; both roles read it
  const IdxRing ring{idx_ring, idx_tok, topk};
  auto read_idx = [&](int blk) -> int32_t { return ring.read(blk, lane); };
  auto tile_at = [&](int k) -> char* { return k == 0 ? tile0 : (k == 1 ? tile1 : tile2); };
  auto pbuf_at = [&](int k) -> char* { return k == 0 ? pbuf0 : (k == 1 ? pbuf1 : pbuf2); };
  // Every wave gathers an eighth of each tile, one kv row per instruction (masked rows read the zero
  // row): part k of wave wu is row wu + 8 k. The score waves spread their parts over the score loop;
  // the O waves issue theirs first thing in the stage. The buffer a stage gathers into is read by
  // neither role during that stage.
  const char* kv_b = (const char*)(kv + b * S_kv * D);
  auto gpart = [&](int r, int32_t my_idx, uint64_t mask, char* tile) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int32_t ri = __builtin_amdgcn_readlane(my_idx, r);
    const uint32_t voff = (uint32_t)((ln ^ (fws_swz(r) & (CPR - 1))) << 4);
    const bool v = (mask >> r) & 1ull;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv_b, (int)(uint32_t)(S_kv * ROWB));
    const __amdgpu_buffer_rsrc_t rz = make_rsrc(g_zero_row, ROWB);
    dma16_buf(v ? rk : rz, voff, v ? (uint32_t)ri * ROWB : 0u, tile + r * ROWB);
  };
  const int32_t idx0 = load_idx(0);
  const uint64_t mask0 = __ballot(slot_in_range(idx0, S_kv));
  if (mask0) {  // tile 0: all eight waves, rows wu + 8 k
#pragma unroll
    for (int k = 0; k < T / 8; k++) gpart(wu + 8 * k, idx0, mask0, tile0);
  }

  if (wu < 4) {
    // ---------------- score waves: wave wu owns heads 16 wu .. 16 wu + 15 ----------------
    const int g = lane >> 4;
    const int hrow = 16 * wu + (lane & 15);
    const int head = hblk * HB + hrow;
    // Q as the B operand of S^T = K Q^T: lane holds head (lane & 15), d = 32 ks + 8 g .. +7. It
    // stays in ordinary vector registers: with no accumulation registers in use the whole 256-register
    // budget of two waves per SIMD goes to them, which the O waves' 128-register accumulator needs.
    bf16x8 qb[KS];
    {
      const uint16_t* qrow = q + (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) qb[ks] = load_bf16x8(qrow + 32 * ks);
    }
    const float sink2 = RR ? sink[head] : sink[head] * kLog2e;
    float m_run = sink2;
    // the sink's share of the denominator is carried by the g == 0 lane of each head
    float l_run = (g == 0 && sink2 != -INFINITY) ? 1.f : 0.f;
    // score fragment offsets: rows lane & 15 (+16 for the second half), chunk 4 ks + g, swizzled
    // by the row's low bits (fragments four k-steps apart differ by 256 bytes)
    int sc_off[4];
    {
      const int row = lane & 15;
#pragma unroll
      for (int j = 0; j < 4; j++) sc_off[j] = row * ROWB + (((4 * j + g) ^ (fws_swz(row) & (CPR - 1))) << 4);
    }
    uint64_t mask_cur = mask0;
    {
      int32_t v0[4], v1[4];
      ring.fetch(0, wu, lane, v0);
      if (nblk > 32) ring.fetch(32, wu, lane, v1);
      wait_all_mem();
      ring.store(0, wu, lane, v0);
      if (nblk > 32) ring.store(32, wu, lane, v1);
      int last = -1;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        if (slot_in_range(v0[k], S_kv)) last = max(last, 256 * k + 64 * wu + lane);
        if (nblk > 32 && slot_in_range(v1[k], S_kv)) last = max(last, 1024 + 256 * k + 64 * wu + lane);
      }
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) last = max(last, __shfl_xor(last, o));
      if (lane == 0) last_s[wu] = last;
    }
    __syncthreads();  // tile 0 and the first index blocks are in LDS
    if (nblk <= 64) nblk = __builtin_amdgcn_readfirstlane((max(max(last_s[0], last_s[1]), max(last_s[2], last_s[3])) + T) / T);
    int32_t idx_nxt = read_idx(1);
    uint64_t mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));

    auto sblock = [&](auto buf_tag, int blk) {
      constexpr int BUF = decltype(buf_tag)::value;
      const char* tile = tile_at(BUF);
      char* nxt = tile_at((BUF + 1) % 3);
      char* pw = pbuf_at(BUF) + (hrow * T + 4 * g) * 2;
      if (blk < nblk) {
        const uint64_t mask = mask_cur, mask_g = mask_nxt;
        const int32_t idx_g = idx_nxt;
        const int32_t idx_new = read_idx(blk + 2);
        // blocks blk + 32 .. blk + 63 go where blocks blk - 32 .. blk - 1 were (read by neither role
        // from here on); they land in the ring at the end of this stage
        const bool refill = IdxRing::refill_at(blk, nblk);
        int32_t iv[4];
        if (refill) ring.fetch(blk + 32, wu, lane, iv);
        if (mask == 0) {
          if (mask_g) {
#pragma unroll
            for (int k = 0; k < NP; k++) gpart(wu + 8 * k, idx_g, mask_g, nxt);
          }
        } else {
          // S^T for the block: fragment i = (k-step i / 2, half i % 2); PF reads run ahead, every
          // stage fenced; the next tile's gather goes out in parts (the zero row when there is no
          // next block, into a buffer nothing reads before the next wait)
          f32x4 sacc[2];
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int r = 0; r < 4; r++) sacc[mt][r] = 0.f;
          auto frag = [&](int i) {
            const int ks = i >> 1, mt = i & 1;
            return lds_load16(tile + sc_off[ks % 4] + 256 * (ks / 4) + mt * 16 * ROWB);
          };
          constexpr int NB = PF + 1;
          bf16x8 fr[NB];
#pragma unroll
          for (int i = 0; i < PF; i++) fr[i] = frag(i);
          static_for<NF>([&](auto it) {
            constexpr int i = decltype(it)::value;
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (i + PF < NF) fr[(i + PF) % NB] = frag(i + PF);
            sacc[i & 1] = mfma16(fr[i % NB], qb[i >> 1], sacc[i & 1]);
            if constexpr (i % (NF / NP) == NF / NP / 2) gpart(wu + 8 * (i / (NF / NP)), idx_g, mask_g, nxt);
          });
          __builtin_amdgcn_sched_barrier(0);
          // online softmax (log2 units, or natural units under RR); this lane holds head hrow,
          // slots 16 mt + 4 g + r
          const uint32_t vb = (uint32_t)(mask >> (4 * g));
          float sv[8];
          float bmax = -INFINITY;
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const float v = ((vb >> (16 * mt + r)) & 1u) ? sacc[mt][r] * score_scale : -INFINITY;
              sv[4 * mt + r] = v;
              bmax = fmaxf(bmax, v);
            }
          bmax = max_xor16_32(bmax);
          // the running max only moves when the block exceeds it by more than 8, so P <= 2^8 and
          // the O rescale runs on few blocks; O / l and m + log2(l) do not depend on where it sits
          const float m_new = (bmax > m_run + MAXSTEP) ? bmax : m_run;  // bmax is finite: a slot is valid
          const float alpha = fast_exp2((m_run - m_new) * EU);
          m_run = m_new;
          float ps = 0.f;
          float p[8];
#pragma unroll
          for (int k = 0; k < 8; k++) {
            p[k] = fast_exp2((sv[k] - m_new) * EU);
            ps += p[k];
          }
          l_run = l_run * alpha + ps;
#pragma unroll
          for (int mt = 0; mt < 2; mt++)
            *(uint2*)(pw + 32 * mt) = pack4_bf16(p[4 * mt], p[4 * mt + 1], p[4 * mt + 2], p[4 * mt + 3]);
          if (g == 0) alpha_s[BUF][hrow] = alpha;
        }
        mask_cur = mask_g;
        mask_nxt = __ballot(slot_in_range(idx_new, S_kv));
        idx_nxt = idx_new;
        wait_all_mem();  // this wave's part of tile blk + 1
        if (refill) ring.store(blk + 32, wu, lane, iv);
      }
      lds_barrier();
    };
    for (int blk = 0; blk <= nblk; blk += 3) {
      sblock(IntTag<0>{}, blk);
      if (blk + 1 <= nblk) sblock(IntTag<1>{}, blk + 1);
      if (blk + 2 <= nblk) sblock(IntTag<2>{}, blk + 2);
    }
    // denominator of each head: the four lanes (g) of the head hold parts of it
    const float l1 = l_run + __shfl_xor(l_run, 16);
    const float ltot = l1 + __shfl_xor(l1, 32);
    if (g == 0) {
      fin_l[hrow] = ltot;
      lse[token * H + head] = ltot > 0.f ? (RR ? (m_run + logf(ltot)) * kLog2e : m_run + log2f(ltot)) : -INFINITY;
    }
    __syncthreads();  // the denominators are in LDS
  } else {
    // ---------- O waves: wave 4 + ow owns d-columns ow DW .. ow DW + DW - 1 of all heads ----------
    const int ow = wu - 4;
    // O^T[d, head] for d tile dt and head half hh: lane holds head 32 hh + (lane & 31),
    // d = ow DW + 32 dt + 8 (r >> 2) + 4 (lane >> 5) + (r & 3)
    f32x16 oacc[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int r = 0; r < 16; r++) oacc[dt][hh][r] = 0.f;
    // masks of the blocks in flight, slot k holding blocks k, k + 3, ...: at the top of stage j the
    // mask of block j - 1 (products) is in slot (j + 2) % 3, and stage j sets slot (j + 1) % 3 (gather)
    uint64_t mask_s[3];
    mask_s[0] = mask0;
    mask_s[2] = 0;
    wait_all_mem();
    __syncthreads();  // tile 0 and the first index blocks are in LDS
    if (nblk <= 64) nblk = __builtin_amdgcn_readfirstlane((max(max(last_s[0], last_s[1]), max(last_s[2], last_s[3])) + T) / T);
    // indices of the block gathered in the next stage (read one stage ahead, so that no stage waits
    // on an index read before its gather)
    int32_t idx_nx = read_idx(1);

    // V^T A fragments of a block run one stage ahead: stage j reads block j's (its tile landed at
    // the end of stage j - 1) into register set j % 2 while its MFMAs use block j - 1's from the
    // other set, so only the P^T fragments' LDS round trip stays in front of the stage's products.
    // For k-step kk (slots 16 kk .. +15) lane l gets d = dbase + (l & 31) and slots s0 .. s0 + 7,
    // s0 = 16 kk + 8 (l >> 5), from two transposing reads four rows apart.
    bf16x8 va_s[2][2][NDT];
    auto read_v = [&](const char* tile, bf16x8 (&va)[2][NDT]) {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int vrow = 8 * (ln >> 5) + ((ln & 15) >> 2);
      const int vch = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
      const int hoff = 8 * (ln & 1);
#pragma unroll
      for (int kk = 0; kk < 2; kk++)
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
          const int r0 = 16 * kk + vrow, c = ow * (DW / 8) + 4 * dt + vch;
          const char* p0 = tile + r0 * ROWB + ((c ^ (fws_swz(r0) & (CPR - 1))) << 4) + hoff;
          const char* p1 = tile + (r0 + 4) * ROWB + ((c ^ (fws_swz(r0 + 4) & (CPR - 1))) << 4) + hoff;
          va[kk][dt] = join_tr(lds_load_tr(p0), lds_load_tr(p1));
        }
    };
    auto oblock = [&](auto buf_tag, int j) {
      constexpr int J = decltype(buf_tag)::value;
      constexpr int BUF = J % 3;
      constexpr int PBUF = (BUF + 2) % 3;  // block j - 1 went through buffers (j - 1) % 3
      constexpr int VS = J % 2;            // register set of block j's V^T fragments
      // the tile gather first (its indices were read a stage ahead), then the LDS reads: the P^T B
      // fragments of block j - 1 and its rescale factors (lane holds head 32 hh + (l & 31), slots
      // 16 kk + 8 (l >> 5) .. +7), block j's V^T fragments and the next stage's indices
      if (j + 1 < nblk) {  // this wave's rows of tile j + 1
        const uint64_t mask_g = __ballot(slot_in_range(idx_nx, S_kv));
        mask_s[(BUF + 1) % 3] = mask_g;
        if (mask_g) {
#pragma unroll
          for (int k = 0; k < NP; k++) gpart(wu + 8 * k, idx_nx, mask_g, tile_at((BUF + 1) % 3));
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      const uint64_t mask = (j >= 1 && j <= nblk) ? mask_s[(BUF + 2) % 3] : 0ull;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      bf16x8 pv[2][2];
      float a0 = 1.f, a1 = 1.f;
      if (mask) {
        const char* pp = pbuf_at(PBUF);
        a0 = alpha_s[PBUF][ln & 31];
        a1 = alpha_s[PBUF][32 + (ln & 31)];
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
          for (int hh = 0; hh < 2; hh++)
            pv[kk][hh] = lds_load16(pp + ((32 * hh + (ln & 31)) * T + 16 * kk + 8 * (ln >> 5)) * 2);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (j < nblk && mask_s[BUF] != 0ull) read_v(tile_at(BUF), va_s[VS]);  // block j's V^T
      idx_nx = read_idx(j + 2);
      __builtin_amdgcn_sched_barrier(0);
      if (mask) {
        if (__any(a0 != 1.f || a1 != 1.f)) {
#pragma unroll
          for (int dt = 0; dt < NDT; dt++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              oacc[dt][0][r] *= a0;
              oacc[dt][1][r] *= a1;
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; kk++)
#pragma unroll
          for (int dt = 0; dt < NDT; dt++) {
            oacc[dt][0] = mfma32(va_s[1 - VS][kk][dt], pv[kk][0], oacc[dt][0]);
            oacc[dt][1] = mfma32(va_s[1 - VS][kk][dt], pv[kk][1], oacc[dt][1]);
          }
      }
      wait_all_mem();  // this wave's rows of tile j + 1
      lds_barrier();
    };
    for (int j = 0; j <= nblk; j += 6) {
      oblock(IntTag<0>{}, j);
      if (j + 1 <= nblk) oblock(IntTag<1>{}, j + 1);
      if (j + 2 <= nblk) oblock(IntTag<2>{}, j + 2);
      if (j + 3 <= nblk) oblock(IntTag<3>{}, j + 3);
      if (j + 4 <= nblk) oblock(IntTag<4>{}, j + 4);
      if (j + 5 <= nblk) oblock(IntTag<5>{}, j + 5);
    }
    __syncthreads();  // the denominators are in LDS
    // epilogue: normalise and store O (bf16), four consecutive d per 8-byte store
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      const int hr = 32 * hh + (lane & 31);
      const float l = fin_l[hr];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* orow = out + (token * H + hblk * HB + hr) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int d = ow * DW + 32 * dt + 8 * r4 + 4 * (lane >> 5);
          *(uint2*)(orow + d) = pack4_bf16(oacc[dt][hh][4 * r4] * inv, oacc[dt][hh][4 * r4 + 1] * inv,
                                           oacc[dt][hh][4 * r4 + 2] * inv, oacc[dt][hh][4 * r4 + 3] * inv);
        }
    }
  }
  wait_all_mem();
}

template <int D, int NHG, bool RR>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t st) {
  const int n_hblk = (int)((a.H + 32 * NHG - 1) / (32 * NHG));
  const int n_tokens = (int)(a.B * a.S);
  const dim3 grid((unsigned)(n_tokens * n_hblk)), block(NHG * 128);
  hipLaunchKernelGGL((fwd_kernel<D, NHG, RR>), grid, block, 0, st, (const uint16_t*)a.q, (const uint16_t*)a.kv,
                     a.sink, a.idx, (uint16_t*)a.o, a.lse, (int)a.S, a.S_kv, (int)a.H, (int)a.topk,
                     RR ? a.sm_scale : a.sm_scale * kLog2e, n_hblk, n_tokens);
  return hipGetLastError();
}

template <bool RR>
static hipError_t launch_fwd_rr(const FwdArgs& a, hipStream_t st) {
  if (a.D == 512 && a.H % 64 == 0) {  // blocks of 64 heads: the specialised-wave kernel
    const int n_hblk = (int)(a.H / 64);
    const int n_tokens = (int)(a.B * a.S);
    hipLaunchKernelGGL((fwd_ws_kernel<512, RR>), dim3((unsigned)(n_tokens * n_hblk)), dim3(512), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, a.sink, a.idx, (uint16_t*)a.o, a.lse, (int)a.S,
                       a.S_kv, (int)a.H, (int)a.topk, RR ? a.sm_scale : a.sm_scale * kLog2e, n_hblk, n_tokens);
    return hipGetLastError();
  }
  if (a.D == 512) return a.H <= 32 ? launch_fwd_t<512, 1, RR>(a, st) : hipErrorInvalidValue;
  if (a.D == 256) return a.H <= 32 ? launch_fwd_t<256, 1, RR>(a, st) : launch_fwd_t<256, 2, RR>(a, st);
  if (a.D == 128) return a.H <= 32 ? launch_fwd_t<128, 1, RR>(a, st) : launch_fwd_t<128, 2, RR>(a, st);
  if (a.D == 64) return a.H <= 32 ? launch_fwd_t<64, 1, RR>(a, st) : hipErrorInvalidValue;
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  return a.reference_rounding ? launch_fwd_rr<true>(a, st) : launch_fwd_rr<false>(a, st);
}

}  // namespace smqa

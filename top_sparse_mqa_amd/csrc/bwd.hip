// Backward kernels of top-k sparse MQA for gfx950 (see include/sparse_mqa.h for the contract).
//
//   preprocess   Delta[b,s,h] = <O, dO> in fp32                       (HBM stream)
//   fill_zero    clears the fp32 dKV accumulator (a kernel, so the sequence is graph-safe)
//   bwd_dq       per token: S^T, dP^T, P, dS, dQ^T += K^T dS^T      (bf16 MFMA 16x16x32)
//   bwd_dkv      per token: S^T, dP^T, P, dS, then dKV^T for the block's slots
//                = Q^T (sm_scale dS) + dO^T P over all heads            (MFMA 32x32x16)
//                and either a plain store of each valid row into its staging row (segmented
//                scatter-add, below) or a fp32 atomic add into the accumulator. A kv row sums
//                thousands of heavily cancelling terms, and 8-bit-mantissa coefficients leave
//                errors of several percent of the result there, so the products run on fp16
//                operands (11 bits) under per-token power-of-two scales, with dS as a hi + lo
//                pair (three MFMAs per k-step): staged, Q and dS as fp16 (dS's scale bounded by
//                the token's kv row norms, kv_row_norm, and Delta); atomic, Q stays bf16 against
//                a bf16 hi + lo pair of dS. P and dO enter as fp16 in both. Staged rows are int16
//                block floating point (one exponent per segment of up to 128 values).
//   bwd_dkv_ws   the staged bwd_dkv at 64 heads per workgroup and D = 512, with specialised
//                waves: score waves (gather, S^T, dP^T, P, dS) and product waves (dKV^T, staging
//                stores) share each SIMD, one block apart; the score waves also store dS (bf16,
//                in the dQ kernel's MFMA operand order) for bwd_dq_ds
//   bwd_dq_ds    at D = 512 with 64-head blocks: dQ = sm_scale dS K from that dS, gathering the
//                same kv rows (2HD flops per pair instead of the recompute's 6HD)
//   postprocess  fp32 accumulator -> bf16 (round to nearest even)
// dQ and dKV run as two kernels: the per-token state both need (Q and dO in two layouts plus
// the dQ accumulator) does not fit one workgroup's registers at H = 64, D = 512. Where the dS
// store exists the dQ kernel reads it; elsewhere (other shapes, and the standalone dQ stage) it
// recomputes S and dP. Every kernel gathers a block of 32 slots into LDS with direct-to-LDS loads
// and stops after the token's last block that holds a valid slot.
#include <type_traits>

#include "device_common.h"
#include "launch.h"

namespace smqa {

__device__ __attribute__((aligned(16))) uint4 g_zero_row_bwd[64];

// Tile swizzle for the backward (16-byte chunk c of row r sits at c ^ bwd_swz(r)): a GF(2)-linear
// map of the row's low four bits under which both tile reads are free of LDS bank conflicts on
// gfx950 -- the score read (rows lane & 15 at one chunk per 16-lane group, 16-byte reads) and the
// dQ transposing read (rows 4 (lane >> 4) + ((lane & 15) >> 2) at two adjacent chunks). Chosen by
// measuring the bank-conflict counter over candidate maps; simpler maps such as
// ((r & 7) << 1) | (r >> 3) leave the score read 2-way conflicted.
__device__ __forceinline__ int bwd_swz(int row) {
  const int r = row & 15;
  return ((r & 1) << 2) ^ (r & 10) ^ (((r >> 2) & 1) * 9);
}

// Maximum of lanes l and l ^ 32 (one cross-half lane swap).
__device__ __forceinline__ float half_swap_max(float m) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(m, fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1])));
}

// Staging rows are block floating point: D int16 values plus one int8 exponent per segment of up
// to 128 values, value = k * 2^e. A segment's exponent puts its largest magnitude m in
// [2^14, 32767.5), so every value of the segment errs by at most m * 2^-15 after rounding to the
// nearest integer. Summed over the thousands of rows a kv row collects, this absolute bound per
// value is what matters: against fp16 values (11 significant bits each) it cuts the error of the
// sums several-fold at the same 2 bytes per value, half the traffic of fp32 rows.
//
// Exponent of a segment whose largest magnitude is m (0 for m = 0): m * 2^-e lies in
// [2^14, 32767.5), so no value of the segment rounds beyond the int16 range.
__device__ __forceinline__ int bfp16_exponent(float m) {
  if (!(m > 0.f && m <= 3.4028235e38f)) return 0;
  int e = __builtin_amdgcn_frexp_expf(m) - 15;
  if (__builtin_amdgcn_ldexpf(m, -e) >= 32767.5f) e++;
  return e;
}
// Two values times sc (a power of two) rounded to the nearest integers, as an int16 pair (a in the
// low half). Adding 1.5 * 2^23 leaves round(x) in the low mantissa bits of the sum for |x| < 2^22,
// and the fma rounds only once, so this is round-to-nearest-even of a * sc exactly.
__device__ __forceinline__ uint32_t bfp16_pair(float a, float b, float sc) {
  constexpr float kRound = 12582912.0f;
  const uint32_t ia = __float_as_uint(__builtin_fmaf(a, sc, kRound));
  const uint32_t ib = __float_as_uint(__builtin_fmaf(b, sc, kRound));
  return __builtin_amdgcn_perm(ib, ia, 0x05040100u);
}
// Block-floating-point encoding of one staging-row segment whose values this lane holds in the NT
// MFMA accumulators c (lanes l and l ^ 32 together hold the segment): picks the exponent from the segment's
// largest magnitude, pre-scales rows of tiny values so that 2^-e stays a normal float, and returns
// the scale sc to apply to the values and the exponent to store (e + so, the product's 2^-so
// undone). Segments whose values are all below 2^-112 are stored as zeros.
template <int NT>
__device__ __forceinline__ float bfp16_scale(f32x16 (&c)[NT], int so, int* es_out) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < NT; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) mx = fmaxf(mx, fabsf(c[i][r]));
  int e = bfp16_exponent(half_swap_max(mx));
  if (__ballot(e < -126)) {
    const int pre = e < -126 ? -126 - e : 0;
#pragma unroll
    for (int i = 0; i < NT; i++)
#pragma unroll
      for (int r = 0; r < 16; r++) c[i][r] = __builtin_amdgcn_ldexpf(c[i][r], pre);
    e += pre;
  }
  int es = e + so;
  float sc = __builtin_amdgcn_ldexpf(1.0f, -e);
  if (es < -127) {
    es = 0;
    sc = 0.f;
  }
  *es_out = es > 127 ? 127 : es;
  return sc;
}
// Offset (in bf16 elements, within one 64-head x 32-slot block) of dS[head][slot] in the stored dS:
// the dQ kernel's MFMA B fragments in order, fragment f = 2 (slot >> 4) + (head >> 5) of 64 lanes x 8
// values, lane (head & 31) + 32 ((slot >> 3) & 1) holding slots 8 (slot >> 3) .. +7 of its head.
__device__ __forceinline__ int ds_fragment_offset(int head, int slot) {
  return (2 * (slot >> 4) + (head >> 5)) * 512 + ((head & 31) + 32 * ((slot >> 3) & 1)) * 8 + (slot & 7);
}
// Bound on |sm_scale * dS| over a token's valid slots and a block of heads, for the scale of the dS
// operand of the dKV product: with P <= 1 (the LSE passed in is at least the log of each head's
// softmax denominator, as the forward's is), |dS| <= |dP| + |Delta|, and |dP| = |<dO_h, kv_t>| <=
// sqrt(D) max|dO| max_t |kv_t| (Cauchy-Schwarz); |Delta| is taken from the Delta passed in
// (max_delta = its largest magnitude over the block's heads).
__device__ __forceinline__ float dS_operand_bound(float sm_scale, int D, float max_do, float max_row_norm,
                                                  float max_delta) {
  return fabsf(sm_scale) * (sqrtf((float)D) * max_do * max_row_norm + max_delta);
}
// dS as an fp16 pair hi + lo (lo = the rounding error of hi, itself rounded to fp16): with a single
// fp16 dS operand the dKV product's rounding dominates the error of heavily shared rows.
__device__ __forceinline__ void f16_hilo4(const float (&x)[4], uint2* hi, uint2* lo) {
  const f16x2 h01 = __builtin_convertvector((f32x2){x[0], x[1]}, f16x2);
  const f16x2 h23 = __builtin_convertvector((f32x2){x[2], x[3]}, f16x2);
  const f16x2 l01 = __builtin_convertvector((f32x2){x[0] - (float)h01[0], x[1] - (float)h01[1]}, f16x2);
  const f16x2 l23 = __builtin_convertvector((f32x2){x[2] - (float)h23[0], x[3] - (float)h23[1]}, f16x2);
  *hi = make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
  *lo = make_uint2(__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23));
}

// ---------------------------------------------------------------------------------------------
template <int D>
__global__ void __launch_bounds__(256)
delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout, float* __restrict__ delta,
             int64_t rows) {
  constexpr int LPR = D / 8;   // lanes per row (16 bytes each)
  constexpr int RPW = 64 / LPR;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int chunk = lane % LPR;
  // workgroups loop over groups of 4 * RPW rows (the grid is capped)
  for (int64_t g = blockIdx.x; g * 4 * RPW < rows; g += gridDim.x) {
    const int64_t row = (g * 4 + w) * RPW + lane / LPR;
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
}

// d_sink[h] = -sum over tokens of 2^(sink_h log2 e - LSE) * Delta: the sink adds exp(sink_h) to
// the softmax denominator and has no value vector, so its weight 2^(sink log2 e - LSE) scales
// -<O, dO> (bwd page, attn_sink input; fwd page, attn_sink note). One workgroup per head; the
// threads' partial sums are combined in a fixed order, so the result is deterministic. A sink of
// -inf has weight 0 (its gradient is 0, and -inf - LSE is never formed).
__global__ void __launch_bounds__(256)
dsink_kernel(const float* __restrict__ lse, const float* __restrict__ delta, const float* __restrict__ sink,
             float* __restrict__ d_sink, int64_t tokens, int H) {
  __shared__ float part[4];
  const int h = blockIdx.x;
  const float sl = sink[h] * kLog2e;
  float acc = 0.f;
  if (sl > -__builtin_inff()) {
    for (int64_t t = threadIdx.x; t < tokens; t += 256) {
      const int64_t i = t * H + h;
      acc += exp2f(sl - lse[i]) * delta[i];
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) d_sink[h] = -((part[0] + part[1]) + (part[2] + part[3]));
}

// Row norms |kv_r| (fp32) of all B * S_kv rows; LPR lanes per row, 16 bytes each.
template <int D>
__global__ void __launch_bounds__(256)
kv_row_norm_kernel(const uint16_t* __restrict__ kv, int64_t rows, float* __restrict__ norm) {
  constexpr int LPR = D / 8;
  constexpr int RPB = 256 / LPR;  // rows per workgroup pass
  const int t = threadIdx.x;
  for (int64_t r = (int64_t)blockIdx.x * RPB + t / LPR; r - t / LPR < rows; r += (int64_t)gridDim.x * RPB) {
    float ss = 0.f;
    if (r < rows) {
      const bf16x8 v = load_bf16x8(kv + r * D + 8 * (t % LPR));
#pragma unroll
      for (int e = 0; e < 8; e++) ss += (float)v[e] * (float)v[e];
    }
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) ss += __shfl_xor(ss, off);
    if (r < rows && t % LPR == 0) norm[r] = sqrtf(ss);
  }
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
  static constexpr int KS = D / 32;              // k-steps of the score products
  static constexpr int KSJ = KS < 4 ? KS : 4;    // distinct per-lane score-fragment offsets
  static constexpr int NDQ = D / 16;             // 16-wide d tiles of dQ
  static constexpr int DQJ = NDQ < 8 ? NDQ : 8;  // distinct per-lane dQ-fragment offsets
};

// Tile rows are gathered with direct-to-LDS loads. With 1 KiB rows (D = 512) one instruction
// moves one row: its kv row index is read from the index lane into a scalar register and the lane
// offset carries the row's chunk swizzle; smaller rows take several rows per instruction. A wave
// issues its share of a tile as NP instructions.
template <int D, int NW>
struct BwdGather {
  using C = BwdCommon<D, NW>;
  static constexpr int NP = C::RPI == 1 ? C::T / NW : (C::NINSTR + NW - 1) / NW;
  const char* kv_b;
  __amdgpu_buffer_rsrc_t rk, rz;  // kv rows of this batch; the zero row (masked slots)

  __device__ __forceinline__ BwdGather(const char* kv_b_, int64_t S_kv)
      : kv_b(kv_b_), rk(make_rsrc(kv_b_, (int)(uint32_t)(S_kv * C::ROWB))), rz(make_rsrc(g_zero_row_bwd, C::ROWB)) {}

  // part k of this wave's share of the tile whose slots' indices sit in my_idx (lane t = slot t)
  __device__ __forceinline__ void part(int k, int32_t my_idx, uint64_t mask, char* tile, int lane, int wu) const {
    if constexpr (C::RPI == 1) {
      const int r = wu + NW * k;
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int32_t ri = __builtin_amdgcn_readlane(my_idx, r);
      const uint32_t voff = (uint32_t)((ln ^ (bwd_swz(r) & (C::CPR - 1))) << 4);
      // branch-free: the row's resource and offset are selected (scalar selects)
      const bool v = (mask >> r) & 1ull;
      dma16_buf(v ? rk : rz, voff, v ? (uint32_t)ri * C::ROWB : 0u, tile + r * C::ROWB);
    } else {
      const int ins = wu + NW * k;
      if (NP * NW == C::NINSTR || ins < C::NINSTR) {
        const int r = ins * C::RPI + lane / C::CPR;
        const int p = lane % C::CPR;
        const int c = p ^ (bwd_swz(r) & (C::CPR - 1));
        const int32_t ri = __shfl(my_idx, r);
        const bool v = (mask >> r) & 1ull;
        const char* src = v ? kv_b + (int64_t)ri * C::ROWB + c * 16 : (const char*)g_zero_row_bwd + c * 16;
        dma16(src, tile + ins * 1024);
      }
    }
  }
  __device__ __forceinline__ void all(int32_t my_idx, uint64_t mask, char* tile, int lane, int wu) const {
#pragma unroll
    for (int k = 0; k < NP; k++) part(k, my_idx, mask, tile, lane, wu);
  }
};

// Per-lane byte offsets of the score A fragments inside a tile: fragment (ks, mt) = rows
// 16 mt + (lane & 15), chunk 4 ks + (lane >> 4). The swizzle only touches the low four chunk
// bits, so fragments 4 k-steps apart differ by 256 bytes and mt by 16 rows (instruction offsets).
template <int D>
__device__ __forceinline__ void bwd_score_offsets(int lane, int* sc_off) {
  using C = BwdCommon<D, 1>;
  const int row = lane & 15, g = lane >> 4;
#pragma unroll
  for (int j = 0; j < C::KSJ; j++) sc_off[j] = row * C::ROWB + (((4 * j + g) ^ (bwd_swz(row) & (C::CPR - 1))) << 4);
}

// S^T and dP^T of one 32-slot block for this wave's 16 heads (C layout: lane l holds head
// (l & 15) and slots 16 mt + 4 (l>>4) + r). Fragment i is (ks, mt) = (i / 2, i % 2). PF fragment
// reads run ahead of the MFMAs that use them; every stage is fenced so the scheduler cannot pull
// a read down to its use, which would expose the full LDS latency on each MFMA. stage_hook(i)
// runs inside stage i (the dKV kernel issues the previous block's stores there).
template <int D, int PF, typename Hook>
__device__ __forceinline__ void bwd_scores(const char* tile, const int* sc_off, const bf16x8* qb,
                                           const bf16x8* dob, f32x4* sacc, f32x4* dpacc, Hook&& stage_hook) {
  using C = BwdCommon<D, 1>;
  constexpr int NF = 2 * C::KS;
  constexpr int PFE = PF < NF ? PF : NF;  // reads in flight
  constexpr int NB = PFE + 1;
  auto frag = [&](int i) {
    const int ks = i >> 1, mt = i & 1;
    return lds_load16(tile + sc_off[ks % C::KSJ] + 256 * (ks / C::KSJ) + mt * 16 * C::ROWB);
  };
#pragma unroll
  for (int mt = 0; mt < 2; mt++)
#pragma unroll
    for (int r = 0; r < 4; r++) { sacc[mt][r] = 0.f; dpacc[mt][r] = 0.f; }
  bf16x8 fr[NB];
#pragma unroll
  for (int i = 0; i < PFE; i++) fr[i] = frag(i);
  static_for<NF>([&](auto it) {
    constexpr int i = decltype(it)::value;
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (i + PFE < NF) fr[(i + PFE) % NB] = frag(i + PFE);
    constexpr int ks = i >> 1, mt = i & 1;
    sacc[mt] = mfma16(fr[i % NB], qb[ks], sacc[mt]);
    dpacc[mt] = mfma16(fr[i % NB], dob[ks], dpacc[mt]);
    stage_hook(it);
  });
  __builtin_amdgcn_sched_barrier(0);
}

// ---------------------------------------------------------------------------------------------
// The two tile buffers are distinct LDS arrays and the block loop is unrolled by two, so every
// read names the buffer it reads at compile time. The compiler can then tell a read of one buffer
// from the gather in flight into the other; with a single array it makes each transposing read
// wait for all outstanding gathers.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
bwd_dq_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
              const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
              uint16_t* __restrict__ dq, int S, int64_t S_kv, int H, int topk, float sm_scale, float scale_log2,
              int n_hblk, int n_tokens) {
  using C = BwdCommon<D, NW>;
  constexpr int T = C::T;
  constexpr int PF = 6;
  constexpr int PFQ = C::NDQ < 6 ? C::NDQ : 6, NBQ = PFQ + 1;  // dQ fragment reads in flight
  __shared__ __attribute__((aligned(16))) char tile0[C::TB];
  __shared__ __attribute__((aligned(16))) char tile1[C::TB];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int g = lane >> 4;
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int head = hblk * 16 * NW + 16 * w + (lane & 15);

  bf16x8 qb[C::KS], dob[C::KS];
  {
    const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
      qb[ks] = load_bf16x8(q + off + 32 * ks);
      dob[ks] = load_bf16x8(dout + off + 32 * ks);
    }
    // after all loads are issued: pinning waits for the value
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
      keep_in_agpr(qb[ks]);
      keep_in_agpr(dob[ks]);
    }
  }
  const float lse_h = lse[token * H + head];
  const float delta_h = delta[token * H + head];

  f32x4 dqacc[C::NDQ];
#pragma unroll
  for (int dt = 0; dt < C::NDQ; dt++)
#pragma unroll
    for (int r = 0; r < 4; r++) dqacc[dt][r] = 0.f;

  int sc_off[C::KSJ];
  bwd_score_offsets<D>(lane, sc_off);
  // dQ^T A fragments (16 d x 32 slots, read transposed): lane rows t0 and t0 + 16 of the tile,
  // d = 16 dt + 4 (lane & 3) -> chunk 2 dt + ((lane & 3) >> 1), byte 8 (lane & 1) of the chunk.
  const int t0 = 4 * g + ((lane & 15) >> 2);
  int dq_off[C::DQJ];
#pragma unroll
  for (int j = 0; j < C::DQJ; j++)
    dq_off[j] = t0 * C::ROWB + (((2 * j + ((lane & 3) >> 1)) ^ (bwd_swz(t0) & (C::CPR - 1))) << 4) + 8 * (lane & 1);

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  using G = BwdGather<D, NW>;
  const G gather((const char*)(kv + b * S_kv * D), S_kv);
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };

  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) gather.all(idx_cur, mask_cur, tile0, lane, wu);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;

  auto block = [&](auto buf_tag, int blk) {
    constexpr int BUF = decltype(buf_tag)::value;
    char* tile = BUF ? tile1 : tile0;
    char* other = BUF ? tile0 : tile1;
    wait_all_mem();
    __syncthreads();
    // the next tile's gather goes out at once: spread over the score loop (one part every few
    // stages) it measured slower in this kernel
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) {
      mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
      if (mask_nxt) gather.all(idx_nxt, mask_nxt, other, lane, wu);
    }
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) return;

    f32x4 sacc[2], dpacc[2];
    bwd_scores<D, PF>(tile, sc_off, qb, dob, sacc, dpacc, [](int) {});

    auto dfrag = [&](int dt) {
      const char* p = tile + dq_off[dt % C::DQJ] + 256 * (dt / C::DQJ);
      return join_tr(lds_load_tr(p), lds_load_tr(p + 16 * C::ROWB));
    };
    // the first dQ fragments are read while the softmax below runs
    bf16x8 fq[NBQ];
#pragma unroll
    for (int i = 0; i < PFQ; i++) fq[i] = dfrag(i);

    // dS as the B operand of dQ^T = K^T dS^T: element e <-> slot 4g + e (e < 4), 16 + 4g + e - 4.
    // validity of this lane's slots 4g + r (bit r) and 16 + 4g + r (bit 16 + r); extracting the
    // lane's bits with one variable shift keeps the compiler from hoisting per-slot 64-bit masks
    const uint32_t vb = (uint32_t)(mask >> (4 * g));
    bf16x8 dsb;
#pragma unroll
    for (int mt = 0; mt < 2; mt++)
#pragma unroll
      for (int r = 0; r < 4; r++) {
        const float p = ((vb >> (16 * mt + r)) & 1u) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
        dsb[4 * mt + r] = (__bf16)(p * (dpacc[mt][r] - delta_h));
      }
#pragma unroll
    for (int dt = 0; dt < C::NDQ; dt++) {
      __builtin_amdgcn_sched_barrier(0);
      if (dt + PFQ < C::NDQ) fq[(dt + PFQ) % NBQ] = dfrag(dt + PFQ);
      dqacc[dt] = mfma16(fq[dt % NBQ], dsb, dqacc[dt]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    block(IntTag<0>{}, blk);
    if (blk + 1 < nblk) block(IntTag<1>{}, blk + 1);
  }

  // dQ^T C layout: lane holds head (lane & 15), d = 16 dt + 4 g + r.
  uint16_t* dqrow = dq + (token * H + head) * (int64_t)D;
#pragma unroll
  for (int dt = 0; dt < C::NDQ; dt++)
    *(uint2*)(dqrow + 16 * dt + 4 * g) = pack4_bf16(dqacc[dt][0] * sm_scale, dqacc[dt][1] * sm_scale,
                                                    dqacc[dt][2] * sm_scale, dqacc[dt][3] * sm_scale);
}

// ---------------------------------------------------------------------------------------------
// dQ with specialised waves, for D = 512 and blocks of 64 heads: eight waves, two per SIMD.
//   Score waves (0-3) compute S^T and dP^T for 16 heads each (16x16x32 MFMAs), then P and
//   dS = P (dP - Delta), and hand dS (bf16, [head][slot]) to the dQ waves through LDS.
//   dQ waves (4-7) hold dQ^T for 128 d-columns of all 64 heads, add K^T dS^T one block behind
//   (32x32x16 MFMAs, K^T from transposing reads of the same tile) and gather the tiles.
// Stage j runs block j on the score waves and block j - 1 on the dQ waves and ends with one
// workgroup barrier; three tile buffers let the dQ waves gather tile j + 1 during stage j (the
// buffer neither role reads then). Q and dO stay in ordinary vector registers, so the whole
// 256-register budget of two waves per SIMD is there for them and for the dQ accumulator.
template <int D>
__global__ void __launch_bounds__(512)
bwd_dq_ws_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
                 const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
                 uint16_t* __restrict__ dq, int S, int64_t S_kv, int H, int topk, float sm_scale, float scale_log2,
                 int n_hblk, int n_tokens) {
  using C = BwdCommon<D, 4>;
  constexpr int T = C::T;
  constexpr int HB = 64;
  constexpr int ROWB = C::ROWB, CPR = C::CPR, TB = C::TB;
  constexpr int PF = 6;
  constexpr int NP = T / 4;       // gather instructions per dQ wave (the dQ waves gather every row)
  constexpr int DW = D / 4;       // dQ^T d-columns per dQ wave
  constexpr int NDT = DW / 32;
  constexpr int DB = HB * T * 2;  // bytes of one dS buffer
  static_assert(ROWB == 1024 && NDT * 32 == DW, "one kv row per gather instruction");
  __shared__ __attribute__((aligned(16))) char tile0[TB];
  __shared__ __attribute__((aligned(16))) char tile1[TB];
  __shared__ __attribute__((aligned(16))) char tile2[TB];
  __shared__ __attribute__((aligned(16))) char dsb0[DB];
  __shared__ __attribute__((aligned(16))) char dsb1[DB];
  __shared__ __attribute__((aligned(16))) char dsb2[DB];

  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x;
  const int64_t token = (int64_t)n_tokens - 1 - item / n_hblk;  // heavier (later) tokens first
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };
  auto tile_at = [&](int k) -> char* { return k == 0 ? tile0 : (k == 1 ? tile1 : tile2); };
  auto dsb_at = [&](int k) -> char* { return k == 0 ? dsb0 : (k == 1 ? dsb1 : dsb2); };
  // Part k of dQ wave wu - 4's share of a tile: row (wu - 4) + 4 k, one kv row per instruction,
  // masked rows read the zero row; the row's 16-byte chunks are swizzled as the score and
  // transposing reads expect. Only the dQ waves gather: the score waves' 64 MFMAs per block make
  // them the longer role, and gathering from their score loop cost ~10%.
  const char* kv_b = (const char*)(kv + b * S_kv * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv_b, (int)(uint32_t)(S_kv * ROWB));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g_zero_row_bwd, ROWB);
  auto gpart = [&](int k, int32_t my_idx, uint64_t mask, char* tile) {
    const int r = (wu - 4) + 4 * k;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int32_t ri = __builtin_amdgcn_readlane(my_idx, r);
    const uint32_t voff = (uint32_t)((ln ^ (bwd_swz(r) & (CPR - 1))) << 4);
    const bool v = (mask >> r) & 1ull;
    dma16_buf(v ? rk : rz, voff, v ? (uint32_t)ri * ROWB : 0u, tile + r * ROWB);
  };
  const int32_t idx0 = load_idx(0);
  const uint64_t mask0 = __ballot(slot_in_range(idx0, S_kv));
  if (mask0 && wu >= 4) {
#pragma unroll
    for (int k = 0; k < NP; k++) gpart(k, idx0, mask0, tile0);
  }

  if (wu < 4) {
    // ---------------- score waves: wave wu owns heads 16 wu .. 16 wu + 15 ----------------
    const int g = lane >> 4;
    const int hrow = 16 * wu + (lane & 15);
    const int head = hblk * HB + hrow;
    bf16x8 qb[C::KS], dob[C::KS];
    {
      const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < C::KS; ks++) {
        qb[ks] = load_bf16x8(q + off + 32 * ks);
        dob[ks] = load_bf16x8(dout + off + 32 * ks);
      }
    }
    const float lse_h = lse[token * H + head];
    const float delta_h = delta[token * H + head];
    int sc_off[C::KSJ];
    bwd_score_offsets<D>(lane, sc_off);
    const int dw_off = (hrow * T + 4 * g) * 2;  // dS writes: head hrow, slots 16 mt + 4 g .. +3
    uint64_t mask_cur = mask0;
    uint64_t mask_nxt = __ballot(slot_in_range(nblk > 1 ? load_idx(1) : -1, S_kv));
    __syncthreads();  // tile 0 is complete (the dQ waves' gathers)

    auto sblock = [&](auto buf_tag, int blk) {
      constexpr int BUF = decltype(buf_tag)::value;
      const char* tile = tile_at(BUF);
      char* dw = dsb_at(BUF) + dw_off;
      if (blk < nblk) {
        const uint64_t mask = mask_cur;
        const int32_t idx_new = blk + 2 < nblk ? load_idx(blk + 2) : -1;
        if (mask != 0) {
          f32x4 sacc[2], dpacc[2];
          bwd_scores<D, PF>(tile, sc_off, qb, dob, sacc, dpacc, [](int) {});
          const uint32_t vb = (uint32_t)(mask >> (4 * g));
#pragma unroll
          for (int mt = 0; mt < 2; mt++) {
            float ds[4];
#pragma unroll
            for (int r = 0; r < 4; r++) {
              const float p = ((vb >> (16 * mt + r)) & 1u) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
              ds[r] = p * (dpacc[mt][r] - delta_h);
            }
            *(uint2*)(dw + 32 * mt) = pack4_bf16(ds[0], ds[1], ds[2], ds[3]);
          }
        }
        mask_cur = mask_nxt;
        mask_nxt = __ballot(slot_in_range(idx_new, S_kv));
      }
      lds_barrier();
    };
    for (int blk = 0; blk <= nblk; blk += 3) {
      sblock(IntTag<0>{}, blk);
      if (blk + 1 <= nblk) sblock(IntTag<1>{}, blk + 1);
      if (blk + 2 <= nblk) sblock(IntTag<2>{}, blk + 2);
    }
  } else {
    // ------- dQ waves: wave 4 + qw owns d-columns qw DW .. qw DW + DW - 1 of all 64 heads -------
    const int qw = wu - 4;
    // dQ^T[d, head] for d tile dt and head half hh: lane holds head 32 hh + (lane & 31),
    // d = qw DW + 32 dt + 8 (r >> 2) + 4 (lane >> 5) + (r & 3)
    f32x16 acc[NDT][2];
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int hh = 0; hh < 2; hh++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[dt][hh][r] = 0.f;
    // indices of blocks j - 1 (products), j and j + 1 (gather) at the top of stage j
    int32_t idx_m1 = -1, idx_0 = idx0, idx_p1 = nblk > 1 ? load_idx(1) : -1;
    wait_all_mem();
    __syncthreads();  // tile 0 is complete

    auto qblock = [&](auto buf_tag, int j) {
      constexpr int BUF = decltype(buf_tag)::value;
      constexpr int PBUF = (BUF + 2) % 3;  // block j - 1 went through buffers (j - 1) % 3
      const int32_t idx_this = idx_m1;
      if (j + 1 < nblk) {  // this wave's rows of tile j + 1, issued before its products
        const uint64_t mask_g = __ballot(slot_in_range(idx_p1, S_kv));
        if (mask_g) {
#pragma unroll
          for (int k = 0; k < NP; k++) gpart(k, idx_p1, mask_g, tile_at((BUF + 1) % 3));
        }
      }
      idx_m1 = idx_0;
      idx_0 = idx_p1;
      idx_p1 = j + 2 < nblk ? load_idx(j + 2) : -1;
      if (j >= 1 && j <= nblk) {
        const uint64_t mask = __ballot(slot_in_range(idx_this, S_kv));
        if (mask) {
          int ln = lane;
          asm volatile("" : "+v"(ln));
          const char* tile = tile_at(PBUF);
          const char* dsp = dsb_at(PBUF);
          // K^T A fragments: for k-step kk (slots 16 kk .. +15), lane l gets d = dbase + (l & 31) and
          // slots 16 kk + 8 (l >> 5) .. +7, from two transposing reads four rows apart
          const int krow = 8 * (ln >> 5) + ((ln & 15) >> 2);
          const int kch = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1);
          const int hoff = 8 * (ln & 1);
          auto kfrag = [&](int kk, int dt) {
            const int r0 = 16 * kk + krow, c = qw * (DW / 8) + 4 * dt + kch;
            const char* p0 = tile + r0 * ROWB + ((c ^ (bwd_swz(r0) & (CPR - 1))) << 4) + hoff;
            const char* p1 = tile + (r0 + 4) * ROWB + ((c ^ (bwd_swz(r0 + 4) & (CPR - 1))) << 4) + hoff;
            return join_tr(lds_load_tr(p0), lds_load_tr(p1));
          };
#pragma unroll
          for (int kk = 0; kk < 2; kk++) {
            // dS^T B fragments: lane holds head 32 hh + (l & 31), slots 16 kk + 8 (l >> 5) .. +7
            bf16x8 dv[2];
#pragma unroll
            for (int hh = 0; hh < 2; hh++)
              dv[hh] = lds_load16(dsp + ((32 * hh + (ln & 31)) * T + 16 * kk + 8 * (ln >> 5)) * 2);
            bf16x8 ka[NDT];
#pragma unroll
            for (int dt = 0; dt < NDT; dt++) ka[dt] = kfrag(kk, dt);
#pragma unroll
            for (int dt = 0; dt < NDT; dt++) {
              acc[dt][0] = mfma32(ka[dt], dv[0], acc[dt][0]);
              acc[dt][1] = mfma32(ka[dt], dv[1], acc[dt][1]);
            }
          }
        }
      }
      wait_all_mem();  // this wave's rows of tile j + 1
      lds_barrier();
    };
    for (int j = 0; j <= nblk; j += 3) {
      qblock(IntTag<0>{}, j);
      if (j + 1 <= nblk) qblock(IntTag<1>{}, j + 1);
      if (j + 2 <= nblk) qblock(IntTag<2>{}, j + 2);
    }
    // dQ = sm_scale * (dS K), bf16, four consecutive d per 8-byte store
#pragma unroll
    for (int hh = 0; hh < 2; hh++) {
      uint16_t* row = dq + (token * H + hblk * HB + 32 * hh + (lane & 31)) * (int64_t)D;
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
          const int d = qw * DW + 32 * dt + 8 * r4 + 4 * (lane >> 5);
          *(uint2*)(row + d) = pack4_bf16(acc[dt][hh][4 * r4] * sm_scale, acc[dt][hh][4 * r4 + 1] * sm_scale,
                                          acc[dt][hh][4 * r4 + 2] * sm_scale, acc[dt][hh][4 * r4 + 3] * sm_scale);
        }
    }
  }
  wait_all_mem();
}

// ---------------------------------------------------------------------------------------------
// dQ from the dS that the staged dKV kernel stores (D = 512, blocks of 64 heads): per (token, head
// block), dQ^T[d, head] = sm_scale * sum over blocks of K^T[d, slot] dS^T[slot, head]. No S or dP
// recompute: the kernel only gathers the kv tiles and copies dS (bf16, as bwd_dq_ws_kernel rounds it,
// so the two give the same dQ bit for bit).
// Eight waves, two per SIMD. Wave w owns d-columns 64 w .. 64 w + 63 of all 64 heads (dQ^T
// accumulators) and gathers rows w, w + 8, w + 16, w + 24 of every tile; waves 0-3 also copy one
// 1 KiB fragment each of the block's dS (stored in B-fragment order) into LDS, so dS crosses the
// vector memory path once per workgroup instead of once per wave. Two buffers of each: during block
// j the copies for block j + 1 are in flight, and at 72 KiB of LDS and at most 128 registers two
// workgroups share a CU, each covering the other's waits (against three buffers and one workgroup
// per CU: 0.62 against 0.76 ms on the headline workload, 5.7 against 6.6 ms on the long-context
// one, 2.55-2.62 against 2.50-2.57 ms with a 256 MiB kv table). Every stage issues its vector
// memory instructions in one fixed order (masked rows and tiles past the end read the zero row; dS
// copies past the end repeat the last block), so the wait at the top of a stage for block j's
// copies, the wave's newest accesses, is a plain vmcnt(0); the copies are issued so that the
// compiler adds no waits of its own (dma16_buf_unordered).
template <int D>
__global__ void __launch_bounds__(512, 2)
bwd_dq_ds_kernel(const uint16_t* __restrict__ kv, const int32_t* __restrict__ idx, const uint16_t* __restrict__ ds,
                 uint16_t* __restrict__ dq, int S, int64_t S_kv, int H, int topk, float sm_scale, int n_hblk,
                 int token0, int n_tokens) {
  constexpr int T = 32, HB = 64, NWV = 8;
  constexpr int ROWB = D * 2, CPR = D / 8, TB = T * ROWB;
  constexpr int DSB = HB * T * 2;  // bytes of one block's dS
  constexpr int DW = D / NWV;      // d-columns per wave
  constexpr int NDT = DW / 32;     // 32-wide d tiles per wave
  constexpr int NP = T / NWV;      // gather rows per wave and tile
  static_assert(ROWB == 1024 && NDT * 32 == DW && NP == 4, "one kv row per gather instruction, four per wave");
  __shared__ __attribute__((aligned(16))) char tile0[TB];
  __shared__ __attribute__((aligned(16))) char tile1[TB];
  __shared__ __attribute__((aligned(16))) char dsb0[DSB];
  __shared__ __attribute__((aligned(16))) char dsb1[DSB];
  __shared__ int last_s[NWV];

  const int lane = threadIdx.x & 63;
  const int wu = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int item = blockIdx.x;
  const int64_t ctok = (int64_t)n_tokens - 1 - item / n_hblk;  // heavier (later) tokens first
  const int64_t token = token0 + ctok;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int nblk_all = (topk + T - 1) / T;  // blocks of the dS store layout
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const uint16_t* ds_tok = ds + (ctok * n_hblk + hblk) * (int64_t)nblk_all * (HB * T);
  // The stages run over the blocks up to the last one holding a valid slot (a selection shorter than
  // topk is padded with masked slots at its end; the dKV kernel stores no dS for blocks past it). The
  // index scan's loads go out first, so the wait for them covers nothing else.
  int last = -1;
  {
    constexpr int U = 4;
    for (int t0 = threadIdx.x; t0 < topk; t0 += U * NWV * 64) {
      int32_t v[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int t = t0 + u * NWV * 64;
        v[u] = t < topk ? idx_tok[t] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; u++)
        if (slot_in_range(v[u], S_kv)) last = max(last, t0 + u * NWV * 64);
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) last = max(last, __shfl_xor(last, o));
    if (lane == 0) last_s[wu] = last;
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < NWV; k++) last = max(last, last_s[k]);
  const int nblk = __builtin_amdgcn_readfirstlane((last + T) / T);
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (blk < nblk && lane < T && t < topk) ? idx_tok[t] : -1;
  };
  auto tile_at = [&](int k) -> char* { return k == 0 ? tile0 : tile1; };
  auto dsb_at = [&](int k) -> char* { return k == 0 ? dsb0 : dsb1; };
  const char* kv_b = (const char*)(kv + b * S_kv * D);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(kv_b, (int)(uint32_t)(S_kv * ROWB));
  const __amdgpu_buffer_rsrc_t rz = make_rsrc(g_zero_row_bwd, ROWB);
  // this wave's NP rows of tile blk's buffer (always NP instructions: masked rows read the zero row),
  // then (waves 0-3) fragment w of block blk's dS
  auto copy_block = [&](int blk, int32_t my_idx, char* tile, char* dsbuf) {
    const uint64_t mask = __ballot(slot_in_range(my_idx, S_kv));
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int k = 0; k < NP; k++) {
      const int r = wu + NWV * k;
      const int32_t ri = __builtin_amdgcn_readlane(my_idx, r);
      const uint32_t voff = (uint32_t)((ln ^ (bwd_swz(r) & (CPR - 1))) << 4);
      const bool v = (mask >> r) & 1ull;
      dma16_buf_unordered(v ? rk : rz, voff, v ? (uint32_t)ri * ROWB : 0u, tile + r * ROWB);
    }
    if (wu < 4) {
      const uint16_t* src = ds_tok + (int64_t)(blk < nblk_all ? blk : nblk_all - 1) * (HB * T);
      dma16_buf_unordered(make_rsrc(src, DSB), (uint32_t)(ln << 4), (uint32_t)(wu * 1024), dsbuf + wu * 1024);
    }
  };
  // K^T A fragments: for k-step kk (slots 16 kk .. +15) lane l gets d = 64 w + 32 dt + (l & 31) and
  // slots 16 kk + 8 (l >> 5) .. +7, from two transposing reads four rows apart
  const int krow = 8 * (lane >> 5) + ((lane & 15) >> 2);
  const int kch = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
  const int hoff = 8 * (lane & 1);

  f32x16 acc[NDT][2];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int hh = 0; hh < 2; hh++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[dt][hh][r] = 0.f;

  // indices of blocks j and j + 1 at the top of stage j
  int32_t ia = load_idx(0), ib = load_idx(1);
  copy_block(0, ia, tile0, dsb0);
  __builtin_amdgcn_sched_barrier(0);

  // Stage j issues, in this order: the index of block j + 2 (none past the end), then the copies of
  // block j + 1. At the top of stage j the copies of block j (stage j - 1), the newest accesses of
  // every wave, are needed.
  auto stage = [&](auto buf_tag, int j) {
    constexpr int BUF = decltype(buf_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0); lgkmcnt and expcnt at their maxima
    lds_barrier();  // every wave's copies of block j; every wave done with the buffers of block j - 1
    const uint64_t mask = __ballot(slot_in_range(ia, S_kv));
    const int32_t ic = load_idx(j + 2);
    __builtin_amdgcn_sched_barrier(0);
    copy_block(j + 1, ib, tile_at(1 - BUF), dsb_at(1 - BUF));  // into the buffers of block j - 1
    __builtin_amdgcn_sched_barrier(0);
    if (mask) {
      const char* tile = tile_at(BUF);
      const char* dsp = dsb_at(BUF) + 16 * lane;
#pragma unroll
      for (int kk = 0; kk < 2; kk++) {
        bf16x8 ka[NDT], dv[2];
#pragma unroll
        for (int hh = 0; hh < 2; hh++) dv[hh] = lds_load16(dsp + (2 * kk + hh) * 1024);
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
          const int r0 = 16 * kk + krow, c = wu * (DW / 8) + 4 * dt + kch;
          const char* p0 = tile + r0 * ROWB + ((c ^ (bwd_swz(r0) & (CPR - 1))) << 4) + hoff;
          const char* p1 = tile + (r0 + 4) * ROWB + ((c ^ (bwd_swz(r0 + 4) & (CPR - 1))) << 4) + hoff;
          ka[dt] = join_tr(lds_load_tr(p0), lds_load_tr(p1));
        }
#pragma unroll
        for (int dt = 0; dt < NDT; dt++) {
          acc[dt][0] = mfma32(ka[dt], dv[0], acc[dt][0]);
          acc[dt][1] = mfma32(ka[dt], dv[1], acc[dt][1]);
        }
      }
    }
    ia = ib;
    ib = ic;
  };
  for (int j = 0; j < nblk; j += 2) {
    stage(IntTag<0>{}, j);
    if (j + 1 < nblk) stage(IntTag<1>{}, j + 1);
  }
  wait_all_mem();  // no copy may still write LDS when the workgroup ends
  // dQ = sm_scale * (dS K), bf16; dQ^T C layout: lane holds head 32 hh + (lane & 31),
  // d = 64 w + 32 dt + 8 (r >> 2) + 4 (lane >> 5) + (r & 3)
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    uint16_t* row = dq + (token * H + hblk * HB + 32 * hh + (lane & 31)) * (int64_t)D;
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int r4 = 0; r4 < 4; r4++) {
        const int d = wu * DW + 32 * dt + 8 * r4 + 4 * (lane >> 5);
        *(uint2*)(row + d) = pack4_bf16(acc[dt][hh][4 * r4] * sm_scale, acc[dt][hh][4 * r4 + 1] * sm_scale,
                                        acc[dt][hh][4 * r4 + 2] * sm_scale, acc[dt][hh][4 * r4 + 3] * sm_scale);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// STAGED: every valid slot's dKV row goes to its staging row (pos, stage, stage_exp); otherwise it
// is added into the fp32 accumulator dkv_acc with fp32 atomics (the workspace-free variant).
template <int D, int NW, bool STAGED>
__global__ void __launch_bounds__(NW * 64)
bwd_dkv_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
               const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
               float* __restrict__ dkv_acc, const int32_t* __restrict__ pos, uint16_t* __restrict__ stage,
               int8_t* __restrict__ stage_exp, const float* __restrict__ row_norm, int S, int64_t S_kv, int H,
               int topk, float sm_scale, float scale_log2, int n_hblk, int token0, int n_tokens) {
  using C = BwdCommon<D, NW>;
  using G = BwdGather<D, NW>;
  constexpr int T = C::T;
  constexpr int PF = 6;
  constexpr int HB = 16 * NW;   // heads of this workgroup
  constexpr int DW = D / NW;    // d-columns of dKV owned by one wave
  constexpr int NDT = DW / 32;  // 32-wide d tiles of one wave
  constexpr int DG = NDT < 4 ? NDT : 4;  // d tiles accumulated together
  constexpr int KH = HB / 16;   // 16-head k-steps of the dKV product
  constexpr int NFS = 2 * C::KS;  // score stages
  static_assert(NDT >= 1 && NDT % DG == 0, "each wave needs whole groups of 32-wide d tiles");
  constexpr int SB = HB * T * 2;  // bytes of one [HB][T] bf16 buffer
  __shared__ __attribute__((aligned(16))) char tile0[C::TB];
  __shared__ __attribute__((aligned(16))) char tile1[C::TB];
  // B operands of the dKV product, each [head][slot]: the hi and lo parts of the dS operand, then
  // fp16 P. Staged: fp16 hi + lo of sm_scale * dS * 2^(sq - so). Atomic (no kv_norm bound): bf16
  // hi + lo of sm_scale * dS * 2^-so (lo = x - float(bf16(x)), rounded).
  constexpr int NB = 3;
  __shared__ __attribute__((aligned(16))) char pds[NB * SB];
  __shared__ float red[4][NW];
  // Staging-store transpose. The dKV^T accumulator gives each lane one slot row and runs of four
  // consecutive d; they go to this wave's [32 slots][SEGW d] int16 buffer as 8-byte writes and come
  // back as 16-byte pieces of whole row segments, so one store instruction covers LPR * 16
  // contiguous bytes of each of RPS rows. Rows are unpadded and their 16-byte chunks XOR-swizzled
  // by the row's low bits (obuf_chunk): the read-back is conflict-free and the writes (32 rows at
  // one column) 2-way. (A padded pitch that makes the writes conflict-free too leaves the rows
  // 8-byte aligned, and the compiler then makes every read-back wait for the gathers in flight.)
  constexpr int SEGW = DG * 32;         // d values per wave group = one staging exponent segment
  constexpr int NSEG = D / SEGW;        // exponents per staging row
  constexpr int OP = SEGW * 2;
  __shared__ __attribute__((aligned(16))) char obuf[NW][T * OP];
  // read-back geometry of the transpose: RPS slot rows of LPR lanes (16 bytes each) per instruction
  constexpr int LPR = SEGW / 8, RPS = 64 / LPR, NI = T / RPS;
  auto obuf_chunk = [](int row, int chunk) { return ((chunk ^ (row & (LPR - 1))) << 4); };
  // With one d group per wave the stores of a block are deferred: the block leaves its rows in
  // obuf (and their staging row indices in obdst) and the next block issues them from inside its
  // score loop, one every other stage. A wave issues in order, so stores issued in one burst
  // would stall its MFMAs behind the memory pipeline.
  constexpr bool DEFER = STAGED && (NDT == DG);
  __shared__ int32_t obdst[NW][T];

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int g = lane >> 4, kg = lane >> 5;
  const int item = blockIdx.x;
  const int64_t ctok = (int64_t)n_tokens - 1 - item / n_hblk;  // token within the chunk
  const int64_t token = token0 + ctok;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int hrow = 16 * w + (lane & 15);          // head within the workgroup's block
  // staged: every valid slot owns n_hblk consecutive staging rows from pos[]
  const int32_t* pos_tok = STAGED ? pos + ctok * (int64_t)topk : nullptr;
  const int head = hblk * HB + hrow;

  // (1) Q and dO with heads along k, as A operands of dKV^T = Q^T (sm_scale dS) + dO^T P:
  // lane l holds d = w*DW + 32 dt + (l & 31) and heads 16 ks + 8 kg .. +7, read with transposing
  // LDS loads from a row-major [HB][D] staging copy held in the two tile buffers (heads
  // 0 .. HH-1 in tile0, the rest in tile1; the buffers are free at this point).
  // P enters as fp16 (11 significant bits; bf16 P leaves errors of several percent on heavily
  // shared rows), so dO does too, scaled by 2^-so with so from this workgroup's max |dO|: every
  // bf16 value within 2^28 of the max converts exactly. Staged, Q is fp16 as well, scaled by 2^-sq
  // from max |q|, and the dS operand is sm_scale * dS * 2^(sq - so) in fp16, so both products
  // carry 2^-so, which the staged rows' exponents undo. so is raised where needed so that the dS
  // operand stays inside the fp16 range (dS_operand_bound: P <= 1, Cauchy-Schwarz for dP, the
  // block's largest |Delta|), with max_t |kv_t| over the token's valid slots from the per-row norms
  // in row_norm. The dS operand is an fp16 hi + lo pair. The atomic variant has no row norms: Q
  // stays bf16 and dS goes in as a hi + lo pair of bf16. Both run three MFMAs per k-step.
  constexpr int HH = C::TB / (D * 2);  // heads per tile buffer
  static_assert(HB <= 2 * HH && HH % 16 == 0, "staging copy must fit the tile buffers");
  constexpr int NPT = HB * D / 8 / (NW * 64);  // 16-byte pieces per thread
  using QV = std::conditional_t<STAGED, f16x8, bf16x8>;
  QV qv[NDT][KH];
  f16x8 dov[NDT][KH];
  int so = 0, sqo = 0;  // dO scale exponent; dS operand exponent sq - so (staged)
  {
    const int64_t base = (token * H + (int64_t)hblk * HB) * D;
    auto piece = [&](int i) -> char* {  // staging-copy address of 16-byte piece i
      const int h = i / (D / 8);
      return h < HH ? tile0 + 16 * i : tile1 + 16 * (i - HH * (D / 8));
    };
    auto read_frags = [&](auto&& put) {
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int ks = 0; ks < KH; ks++) {
          const int hb0 = 16 * ks;  // first head of the k-step: all 16 sit in one buffer
          const char* sb = hb0 < HH ? tile0 : tile1;
          const int h0 = hb0 % HH + 8 * kg + ((lane & 15) >> 2);
          const int d = w * DW + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          put(dt, ks, join_tr(lds_load_tr(sb + (h0 * D + d) * 2), lds_load_tr(sb + ((h0 + 4) * D + d) * 2)));
        }
    };
    uint4 rq[NPT], rd[NPT];
    float mq = 0.f, md = 0.f, mv = 0.f, mdl = 0.f;
    if constexpr (STAGED) {  // largest norm among this token's referenced kv rows; largest |Delta|
      if (threadIdx.x < HB) mdl = fabsf(delta[token * H + (int64_t)hblk * HB + threadIdx.x]);
      const int32_t* it = idx + token * (int64_t)topk;
      const float* nb = row_norm + b * S_kv;
      constexpr int U = 8;  // independent index loads, then independent norm loads
      for (int t0 = threadIdx.x; t0 < topk; t0 += U * NW * 64) {
        int32_t v[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
          const int t = t0 + u * NW * 64;
          v[u] = t < topk ? it[t] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; u++)
          if (slot_in_range(v[u], S_kv)) mv = fmaxf(mv, nb[v[u]]);
      }
    }
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      rq[k] = *(const uint4*)(q + base + 8 * (threadIdx.x + k * NW * 64));
      rd[k] = *(const uint4*)(dout + base + 8 * (threadIdx.x + k * NW * 64));
    }
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, rq[k]), c = __builtin_bit_cast(bf16x8, rd[k]);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        mq = fmaxf(mq, fabsf((float)a[e]));
        md = fmaxf(md, fabsf((float)c[e]));
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      mq = fmaxf(mq, __shfl_xor(mq, o));
      md = fmaxf(md, __shfl_xor(md, o));
      mv = fmaxf(mv, __shfl_xor(mv, o));
      mdl = fmaxf(mdl, __shfl_xor(mdl, o));
    }
    if (lane == 0) {
      red[0][w] = mq;
      red[1][w] = md;
      red[2][w] = mv;
      red[3][w] = mdl;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NW; k++) {
      mq = fmaxf(mq, red[0][k]);
      md = fmaxf(md, red[1][k]);
      mv = fmaxf(mv, red[2][k]);
      mdl = fmaxf(mdl, red[3][k]);
    }
    // scaled maxima stay below 2^15
    const int sq = (STAGED && mq > 0.f && mq <= 3.4028235e38f) ? __builtin_amdgcn_frexp_expf(mq) - 15 : 0;
    if (md > 0.f && md <= 3.4028235e38f) {
      so = __builtin_amdgcn_frexp_expf(md) - 15;
      if constexpr (STAGED) {
        const float bound = dS_operand_bound(sm_scale, D, md, mv, mdl);
        if (bound > 0.f && bound <= 3.4028235e38f) {
          const int sd = __builtin_amdgcn_frexp_expf(bound) + sq - 15;
          so = so > sd ? so : sd;
        }
      }
      so = so < -100 ? -100 : (so > 100 ? 100 : so);
    }
    sqo = sq - so;
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      if constexpr (STAGED) {
        const bf16x8 v = __builtin_bit_cast(bf16x8, rq[k]);
        f16x8 hv;
#pragma unroll
        for (int e = 0; e < 8; e++) hv[e] = (_Float16)__builtin_amdgcn_ldexpf((float)v[e], -sq);
        *(f16x8*)piece(threadIdx.x + k * NW * 64) = hv;
      } else {
        *(uint4*)piece(threadIdx.x + k * NW * 64) = rq[k];
      }
    }
    __syncthreads();
    read_frags([&](int dt, int ks, bf16x8 v) { qv[dt][ks] = __builtin_bit_cast(QV, v); });
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, rd[k]);
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; e++) hv[e] = (_Float16)__builtin_amdgcn_ldexpf((float)v[e], -so);
      *(f16x8*)piece(threadIdx.x + k * NW * 64) = hv;
    }
    __syncthreads();
    read_frags([&](int dt, int ks, bf16x8 v) { dov[dt][ks] = __builtin_bit_cast(f16x8, v); });
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int ks = 0; ks < KH; ks++) {
        keep_in_agpr(qv[dt][ks]);
        keep_in_agpr(dov[dt][ks]);
      }
  }
  // (2) Q and dO with d along k, as B operands of S^T and dP^T (this wave's 16 heads).
  bf16x8 qb[C::KS], dob[C::KS];
  {
    const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
      qb[ks] = load_bf16x8(q + off + 32 * ks);
      dob[ks] = load_bf16x8(dout + off + 32 * ks);
    }
    // after all loads are issued: pinning waits for the value
#pragma unroll
    for (int ks = 0; ks < C::KS; ks++) {
      keep_in_agpr(qb[ks]);
      keep_in_agpr(dob[ks]);
    }
  }
  const float lse_h = lse[token * H + head];
  const float delta_h = delta[token * H + head];

  int sc_off[C::KSJ];
  bwd_score_offsets<D>(lane, sc_off);
  // P/dS writes: head hrow, slots 16 mt + 4 g .. +3 (8 bytes). Reads (B operand of dKV^T): lane l
  // gets slot (l & 31) and heads 16 ks + 8 kg .. +7 from two transposing reads 4 heads apart.
  const int pw_off = (hrow * T + 4 * g) * 2;
  const int pr_off = ((8 * kg + ((lane & 15) >> 2)) * T + 16 * ((lane >> 4) & 1) + 4 * (lane & 3)) * 2;

  const int nblk = (topk + T - 1) / T;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  const G gather((const char*)(kv + b * S_kv * D), S_kv);
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };
  auto load_pos = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (STAGED && lane < T && t < topk) ? pos_tok[t] : -1;
  };

  int32_t pos_cur = load_pos(0);
  int32_t pos_nxt = nblk > 1 ? load_pos(1) : -1;
  int32_t idx_cur = load_idx(0);
  uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
  if (mask_cur) gather.all(idx_cur, mask_cur, tile0, lane, wu);
  int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;
  wait_all_mem();

  // 16-byte piece lane % LPR of transpose row (k * RPS + lane / LPR)
  auto rdpiece = [&](int k) -> i32x4 {
    const int row = k * RPS + lane / LPR;
    return *(const i32x4*)(obuf[w] + row * OP + obuf_chunk(row, lane % LPR));
  };
  // Deferred staging stores (one d group per wave): the rows a block leaves in the transpose
  // buffer, with their staging rows in obdst, go out during the next non-empty block's dKV
  // product, SPK rows per k-step, each read from LDS one k-step ahead of its store. obdst starts at
  // the spare row, so the first block's stores write the unused buffer there; a block without valid
  // slots leaves the buffer alone and the next one stores the same rows again (same values).
  const int32_t spare = (n_tokens * topk + (int32_t)ctok) * n_hblk + hblk;
  constexpr int SPK = (NI + KH - 1) / KH;  // stores per k-step of the dKV product
  int pending_e = 0;                       // exponent of slot row lane & 31
  if constexpr (DEFER) {
    if (lane < T) obdst[w][lane] = spare;
  }
  const int dlane = w * DW + 8 * (lane % LPR);  // first d of this lane's 8 values
  i32x4 dv[SPK];
  int32_t dd[SPK], ddx = 0;
  auto dread = [&](int k) {
    if (k < NI) {
      dv[k % SPK] = rdpiece(k);
      dd[k % SPK] = obdst[w][k * RPS + lane / LPR];
    }
  };
  auto dstore = [&](int k) {
    if (k < NI) __builtin_nontemporal_store(dv[k % SPK], (i32x4*)(stage + (int64_t)dd[k % SPK] * D + dlane));
  };
  auto eread = [&]() { ddx = obdst[w][lane & 31]; };
  auto estore = [&]() {
    if (lane < T) stage_exp[(int64_t)ddx * NSEG + w * (DW / SEGW)] = (int8_t)pending_e;
  };

  // Each wave waits for its own part of tile blk + 1 right before it stores the rows of tile blk,
  // so the barrier at the top of the next block finds the tile complete without draining stores.
  auto block = [&](auto buf_tag, int blk) {
    constexpr int BUF = decltype(buf_tag)::value;
    const char* tile = BUF ? tile1 : tile0;
    char* other = BUF ? tile0 : tile1;
    // tile blk complete (each wave waited for its part before its previous stores); the P/dS
    // buffers of the previous block fully consumed. The stores themselves stay in flight.
    lds_barrier();
    // the next tile is gathered in parts from inside this block's score loop, one every NFS / NP
    // stages; the previous block's staging stores go out during this block's dKV product, so the
    // two streams of vector memory instructions do not queue up behind each other
    uint64_t mask_nxt = 0;
    if (blk + 1 < nblk) mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
    const int32_t idx_g = idx_nxt;
    const int32_t idx_this = idx_cur;
    idx_cur = idx_nxt;
    idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
    const int32_t pos_this = pos_cur;
    pos_cur = pos_nxt;
    pos_nxt = blk + 2 < nblk ? load_pos(blk + 2) : -1;
    const uint64_t mask = mask_cur;
    mask_cur = mask_nxt;
    if (mask == 0) {
      if (mask_nxt) gather.all(idx_g, mask_nxt, other, lane, wu);
      wait_all_mem();
      return;
    }
    // unconditional and branch-free: with no next block (mask_nxt == 0) the parts read the zero row
    // into the idle buffer, which nothing reads before the next wait
    auto gather_hook = [&](int i) {
#pragma unroll
      for (int k = 0; k < G::NP; k++)
        if (i == (k * NFS) / G::NP + NFS / G::NP / 2) gather.part(k, idx_g, mask_nxt, other, lane, wu);
    };

    f32x4 sacc[2], dpacc[2];
    bwd_scores<D, PF>(tile, sc_off, qb, dob, sacc, dpacc, gather_hook);
    // validity of this lane's slots 4g + r (bit r) and 16 + 4g + r (bit 16 + r), one variable shift
    const uint32_t vb = (uint32_t)(mask >> (4 * g));
#pragma unroll
    for (int mt = 0; mt < 2; mt++) {
      float p[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; r++)
        p[r] = ((vb >> (16 * mt + r)) & 1u) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
      char* wp = pds + pw_off + 32 * mt;
      if constexpr (STAGED) {
#pragma unroll
        for (int r = 0; r < 4; r++)  // saturated to the fp16 range: only inputs outside the bound's assumptions reach it
          ds[r] = __builtin_amdgcn_fmed3f(
              __builtin_amdgcn_ldexpf(sm_scale * p[r] * (dpacc[mt][r] - delta_h), sqo), -65504.f, 65504.f);
        f16_hilo4(ds, (uint2*)(wp), (uint2*)(wp + SB));
      } else {
        float dslr[4];
#pragma unroll
        for (int r = 0; r < 4; r++) {
          ds[r] = __builtin_amdgcn_ldexpf(sm_scale * p[r] * (dpacc[mt][r] - delta_h), -so);
          dslr[r] = ds[r] - (float)(__bf16)ds[r];
        }
        *(uint2*)(wp) = pack4_bf16(ds[0], ds[1], ds[2], ds[3]);
        *(uint2*)(wp + SB) = pack4_bf16(dslr[0], dslr[1], dslr[2], dslr[3]);
      }
      const f16x2 p01 = __builtin_convertvector((f32x2){p[0], p[1]}, f16x2);
      const f16x2 p23 = __builtin_convertvector((f32x2){p[2], p[3]}, f16x2);
      *(uint2*)(wp + (NB - 1) * SB) = make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
    }
    lds_barrier();  // P/dS visible to all waves; the next tile's gather stays in flight

    // 2^-so dKV^T[d, slot] for this wave's d-range, DG tiles of 32 d at a time, k over the block's
    // heads: Q^T dS_hi + Q^T dS_lo + (2^-so dO)^T P, with Q scaled by 2^-sq and dS by 2^(sq-so)
    // (fp16) staged, Q and dS by 2^-so (bf16) atomic.
    // C layout: lane holds slot (lane & 31), d = w*DW + 32 dt + 8 (r >> 2) + 4 kg + (r & 3).
    // Masked slots store into this workgroup's spare row (after all staging rows of the chunk),
    // so the stores need no per-slot branches.
    const int32_t dst_this = slot_in_range(idx_this, S_kv) ? pos_this + hblk : spare;
    int32_t rowi[NI];
    if constexpr (STAGED && !DEFER) {
#pragma unroll
      for (int n = 0; n < NI; n++) rowi[n] = __shfl(dst_this, n * RPS + lane / LPR);
    }
    char* ob = obuf[w] + (lane & 31) * OP + 8 * kg;  // this lane's slot row in the transpose
    auto bfrag = [&](int ks, int m) {
      const char* p = pds + m * SB + pr_off + ks * 16 * T * 2;
      return join_tr(lds_load_tr(p), lds_load_tr(p + 4 * T * 2));
    };
#pragma unroll
    for (int dg = 0; dg < NDT / DG; dg++) {
      f32x16 c[DG];
#pragma unroll
      for (int i = 0; i < DG; i++)
#pragma unroll
        for (int r = 0; r < 16; r++) c[i][r] = 0.f;
      bf16x8 bcur[NB], bnxt[NB];
#pragma unroll
      for (int m = 0; m < NB; m++) bcur[m] = bfrag(0, m);
      if constexpr (DEFER) {
        eread();
#pragma unroll
        for (int k = 0; k < SPK; k++) dread(k);
      }
#pragma unroll
      for (int ks = 0; ks < KH; ks++) {
        __builtin_amdgcn_sched_barrier(0);
        if (ks + 1 < KH) {
#pragma unroll
          for (int m = 0; m < NB; m++) bnxt[m] = bfrag(ks + 1, m);
        }
        if constexpr (DEFER) {
          // the previous block's rows of this k-step, then the reads for the next one
          if (ks == 0) estore();
#pragma unroll
          for (int k = SPK * ks; k < SPK * (ks + 1); k++) dstore(k);
#pragma unroll
          for (int k = SPK * (ks + 1); k < SPK * (ks + 2); k++) dread(k);
        }
#pragma unroll
        for (int m = 0; m < NB; m++)
#pragma unroll
          for (int i = 0; i < DG; i++) {
            const int dt = dg * DG + i;
            if (m == NB - 1) c[i] = mfma32h(dov[dt][ks], __builtin_bit_cast(f16x8, bcur[m]), c[i]);
            else if constexpr (STAGED) c[i] = mfma32h(qv[dt][ks], __builtin_bit_cast(f16x8, bcur[m]), c[i]);
            else c[i] = mfma32(qv[dt][ks], bcur[m], c[i]);
          }
        if (ks + 1 < KH) {
#pragma unroll
          for (int m = 0; m < NB; m++) bcur[m] = bnxt[m];
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (!STAGED) {
        if (dg == NDT / DG - 1) wait_all_mem();  // this wave's part of tile blk + 1
        // fp32 atomics of the valid slots' values (lane: slot lane & 31)
        const int32_t kvrow = __shfl(idx_this, lane & 31);
        if ((mask >> (lane & 31)) & 1ull) {
          float* p = dkv_acc + (b * S_kv + kvrow) * D + w * DW + SEGW * dg + 4 * kg;
#pragma unroll
          for (int i = 0; i < DG; i++)
#pragma unroll
            for (int r = 0; r < 16; r++)
              unsafeAtomicAdd(p + 32 * i + 8 * (r >> 2) + (r & 3), __builtin_amdgcn_ldexpf(c[i][r], so));
        }
        continue;
      }
      // one exponent per slot row segment (this lane and lane ^ 32 hold the row's values), then
      // int16 runs of four d into this wave's transpose buffer
      int es;
      const float sc = bfp16_scale(c, so, &es);
#pragma unroll
      for (int i = 0; i < DG; i++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          *(i32x2*)(ob + obuf_chunk(lane & 31, 4 * i + j)) =
              i32x2{(int)bfp16_pair(c[i][4 * j], c[i][4 * j + 1], sc), (int)bfp16_pair(c[i][4 * j + 2], c[i][4 * j + 3], sc)};
      if constexpr (DEFER) {
        if (lane < T) obdst[w][lane] = dst_this;
        wait_all_mem();  // this wave's part of tile blk + 1
        pending_e = es;
        continue;
      }
      if (dg == NDT / DG - 1) wait_all_mem();  // this wave's part of tile blk + 1
      // row reads: lane covers 8 consecutive d of slot row n*RPS + lane/LPR
      const int d0 = w * DW + SEGW * dg + 8 * (lane % LPR);
#pragma unroll
      for (int n = 0; n < NI; n++) {
        const i32x4 v = rdpiece(n);
        __builtin_nontemporal_store(v, (i32x4*)(stage + (int64_t)rowi[n] * D + d0));
      }
      // the row exponents of this group (lane < 32 holds slot row lane)
      if (lane < T) stage_exp[(int64_t)dst_this * NSEG + (w * DW + SEGW * dg) / SEGW] = (int8_t)es;
    }
  };
  for (int blk = 0; blk < nblk; blk += 2) {
    block(IntTag<0>{}, blk);
    if (blk + 1 < nblk) block(IntTag<1>{}, blk + 1);
  }
  if constexpr (DEFER) {  // the last block's rows
    eread();
    estore();
#pragma unroll
    for (int k = 0; k < NI; k++) {
      dread(k);
      dstore(k);
    }
  }
  wait_all_mem();  // no gather may still write LDS when the workgroup ends
}

// ---------------------------------------------------------------------------------------------
// Staged dKV with specialised waves: 2 NW waves per workgroup, two per SIMD. Score waves
// (0 .. NW-1) gather the kv tiles and produce S^T, dP^T, P and dS of block j for 16 heads each, as
// bwd_dkv_kernel does; product waves (NW .. 2NW-1) run the dKV^T product of block j - 1 for a
// d-range of DW each and store its staging rows. Each SIMD holds one wave of each kind, so the
// gather and store issue, the softmax and the transposes of one wave overlap the MFMAs of the
// other (with one wave per SIMD they run one after another). Stage j ends with one workgroup
// barrier that hands block j's P/dS buffer to the product waves; every wave passes the same number
// of barriers whatever its role (five in the set-up, then nblk + 1 stages). Numerics and staging
// format are those of bwd_dkv_kernel<D, NW, true>.
template <int D, int NW>
__global__ void __launch_bounds__(NW * 128)
bwd_dkv_ws_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ kv, const uint16_t* __restrict__ dout,
                  const int32_t* __restrict__ idx, const float* __restrict__ lse, const float* __restrict__ delta,
                  const int32_t* __restrict__ pos, uint16_t* __restrict__ stage, int8_t* __restrict__ stage_exp,
                  const float* __restrict__ row_norm, int S, int64_t S_kv, int H, int topk, float sm_scale,
                  float scale_log2, int n_hblk, int token0, int n_tokens, uint16_t* __restrict__ ds_out) {
  using C = BwdCommon<D, NW>;
  using G = BwdGather<D, NW>;
  constexpr int T = C::T;
  constexpr int PF = 6;
  constexpr int NWT = 2 * NW;   // waves of the workgroup
  constexpr int HB = 16 * NW;   // heads of this workgroup
  constexpr int DW = D / NW;    // d-columns of dKV owned by one product wave
  constexpr int NDT = DW / 32;  // its 32-wide d tiles, accumulated together
  constexpr int KH = HB / 16;   // 16-head k-steps of the dKV product
  constexpr int NFS = 2 * C::KS;
  static_assert(NDT >= 1 && NDT <= 4, "one group of at most four 32-wide d tiles per product wave");
  constexpr int SB = HB * T * 2;  // bytes of one [HB][T] fp16 buffer
  __shared__ __attribute__((aligned(16))) char tile0[C::TB];
  __shared__ __attribute__((aligned(16))) char tile1[C::TB];
  // dS operand (hi, then lo) then P of a block, each [head][slot] fp16; block j goes through
  // pds<j & 1>
  __shared__ __attribute__((aligned(16))) char pds0[3 * SB];
  __shared__ __attribute__((aligned(16))) char pds1[3 * SB];
  __shared__ float red[4][NWT];
  __shared__ int red_last[NWT];
  // staging-store transpose per product wave, as in bwd_dkv_kernel (one exponent segment = DW)
  constexpr int SEGW = NDT * 32;
  constexpr int NSEG = D / SEGW;
  constexpr int OP = SEGW * 2;
  __shared__ __attribute__((aligned(16))) char obuf[NW][T * OP];
  constexpr int LPR = SEGW / 8, RPS = 64 / LPR, NI = T / RPS;
  auto obuf_chunk = [](int row, int chunk) { return ((chunk ^ (row & (LPR - 1))) << 4); };

  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int g = lane >> 4, kg = lane >> 5;
  const int item = blockIdx.x;
  const int64_t ctok = (int64_t)n_tokens - 1 - item / n_hblk;  // token within the chunk
  const int64_t token = token0 + ctok;
  const int hblk = item % n_hblk;
  const int64_t b = token / S;
  const int nblk_all = (topk + T - 1) / T;  // blocks of the dS store layout
  // blocks processed: those up to the last one holding a valid slot (set after the index scan below;
  // a selection shorter than topk is padded with masked slots at its end)
  int nblk = nblk_all;
  const int32_t* idx_tok = idx + token * (int64_t)topk;
  auto load_idx = [&](int blk) -> int32_t {
    const int t = blk * T + lane;
    return (lane < T && t < topk) ? idx_tok[t] : -1;
  };

  // (1) Per-token scales (all waves): Q as fp16 times 2^-sq, dO times 2^-so, the dS operand times
  // 2^(sq - so), with sq, so from max |q|, max |dO| and the largest row norm among the token's
  // valid slots, exactly as bwd_dkv_kernel derives them. Q and dO then pass through a row-major
  // [HB][D] fp16 copy in the tile buffers, from which the product waves read them transposed.
  constexpr int HH = C::TB / (D * 2);  // heads per tile buffer
  static_assert(HB <= 2 * HH && HH % 16 == 0, "staging copy must fit the tile buffers");
  constexpr int NPT = HB * D / 8 / (NWT * 64);  // 16-byte pieces per thread
  static_assert(NPT >= 1 && NPT * NWT * 64 * 8 == HB * D, "whole pieces per thread");
  auto piece = [&](int i) -> char* {
    const int h = i / (D / 8);
    return h < HH ? tile0 + 16 * i : tile1 + 16 * (i - HH * (D / 8));
  };
  uint4 rq[NPT], rd[NPT];
  f16x8 hd[NPT];  // dO pieces as fp16 times 2^-so, written to the copy once Q has been read
  int so = 0, sqo = 0;
  {
    const int64_t base = (token * H + (int64_t)hblk * HB) * D;
    float mq = 0.f, md = 0.f, mv = 0.f;
    float mdl = threadIdx.x < HB ? fabsf(delta[token * H + (int64_t)hblk * HB + threadIdx.x]) : 0.f;
    int last = -1;  // last valid slot
    const float* nb = row_norm + b * S_kv;
    constexpr int U = 8;  // independent index loads, then independent norm loads
    for (int t0 = threadIdx.x; t0 < topk; t0 += U * NWT * 64) {
      int32_t v[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const int t = t0 + u * NWT * 64;
        v[u] = t < topk ? idx_tok[t] : -1;
      }
#pragma unroll
      for (int u = 0; u < U; u++)
        if (slot_in_range(v[u], S_kv)) {
          mv = fmaxf(mv, nb[v[u]]);
          last = max(last, t0 + u * NWT * 64);
        }
    }
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      rq[k] = *(const uint4*)(q + base + 8 * (threadIdx.x + k * NWT * 64));
      rd[k] = *(const uint4*)(dout + base + 8 * (threadIdx.x + k * NWT * 64));
    }
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, rq[k]), c = __builtin_bit_cast(bf16x8, rd[k]);
#pragma unroll
      for (int e = 0; e < 8; e++) {
        mq = fmaxf(mq, fabsf((float)a[e]));
        md = fmaxf(md, fabsf((float)c[e]));
      }
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      mq = fmaxf(mq, __shfl_xor(mq, o));
      md = fmaxf(md, __shfl_xor(md, o));
      mv = fmaxf(mv, __shfl_xor(mv, o));
      mdl = fmaxf(mdl, __shfl_xor(mdl, o));
      last = max(last, __shfl_xor(last, o));
    }
    if (lane == 0) {
      red_last[w] = last;
      red[0][w] = mq;
      red[1][w] = md;
      red[2][w] = mv;
      red[3][w] = mdl;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < NWT; k++) {
      mq = fmaxf(mq, red[0][k]);
      md = fmaxf(md, red[1][k]);
      mv = fmaxf(mv, red[2][k]);
      mdl = fmaxf(mdl, red[3][k]);
      last = max(last, red_last[k]);
    }
    nblk = __builtin_amdgcn_readfirstlane((last + T) / T);
    const int sq = (mq > 0.f && mq <= 3.4028235e38f) ? __builtin_amdgcn_frexp_expf(mq) - 15 : 0;
    if (md > 0.f && md <= 3.4028235e38f) {
      so = __builtin_amdgcn_frexp_expf(md) - 15;
      const float bound = dS_operand_bound(sm_scale, D, md, mv, mdl);
      if (bound > 0.f && bound <= 3.4028235e38f) {
        const int sd = __builtin_amdgcn_frexp_expf(bound) + sq - 15;
        so = so > sd ? so : sd;
      }
      so = so < -100 ? -100 : (so > 100 ? 100 : so);
    }
    sqo = sq - so;
#pragma unroll
    for (int k = 0; k < NPT; k++) {
      const bf16x8 v = __builtin_bit_cast(bf16x8, rq[k]), c = __builtin_bit_cast(bf16x8, rd[k]);
      f16x8 hv;
#pragma unroll
      for (int e = 0; e < 8; e++) {
        hv[e] = (_Float16)__builtin_amdgcn_ldexpf((float)v[e], -sq);
        hd[k][e] = (_Float16)__builtin_amdgcn_ldexpf((float)c[e], -so);
      }
      *(f16x8*)piece(threadIdx.x + k * NWT * 64) = hv;
    }
  }
  __syncthreads();  // the Q copy is complete
  auto put_dout = [&]() {
#pragma unroll
    for (int k = 0; k < NPT; k++) *(f16x8*)piece(threadIdx.x + k * NWT * 64) = hd[k];
  };

  if (wu < NW) {
    // ---------------- score waves: wave wu owns heads 16 wu .. 16 wu + 15 ----------------
    const int hrow = 16 * wu + (lane & 15);
    const int head = hblk * HB + hrow;
    bf16x8 qb[C::KS], dob[C::KS];
    {
      const int64_t off = (token * H + head) * (int64_t)D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < C::KS; ks++) {
        qb[ks] = load_bf16x8(q + off + 32 * ks);
        dob[ks] = load_bf16x8(dout + off + 32 * ks);
      }
      // after all loads are issued: pinning waits for the value
#pragma unroll
      for (int ks = 0; ks < C::KS; ks++) {
        keep_in_agpr(qb[ks]);
        keep_in_agpr(dob[ks]);
      }
    }
    const float lse_h = lse[token * H + head];
    const float delta_h = delta[token * H + head];
    __syncthreads();  // the product waves have read Q
    put_dout();
    __syncthreads();  // the dO copy is complete
    __syncthreads();  // the product waves have read dO: the tile buffers are free

    int sc_off[C::KSJ];
    bwd_score_offsets<D>(lane, sc_off);
    const int pw_off = (hrow * T + 4 * g) * 2;  // P/dS writes: head hrow, slots 16 mt + 4 g .. +3
    // dS output, per (chunk token, head block, 32-slot block) in the order of the dQ kernel's MFMA B
    // fragments: fragment f = 2 kk + hh is 64 lanes x 8 values, lane l holding head 32 hh + (l & 31)
    // and slots 16 kk + 8 (l >> 5) .. +7 (ds_fragment_offset). This lane's values (head hrow, slots
    // 16 mt + 4 g .. +3) are 8 contiguous bytes of fragment 2 mt + (hrow >> 5).
    const int64_t ds_off = (ctok * n_hblk + hblk) * (int64_t)nblk_all * (HB * T) + ds_fragment_offset(hrow, 4 * g);
    const G gather((const char*)(kv + b * S_kv * D), S_kv);
    int32_t idx_cur = load_idx(0);
    uint64_t mask_cur = __ballot(slot_in_range(idx_cur, S_kv));
    if (mask_cur) gather.all(idx_cur, mask_cur, tile0, lane, wu);
    int32_t idx_nxt = nblk > 1 ? load_idx(1) : -1;
    wait_all_mem();
    __syncthreads();  // tile 0 is complete

    auto sblock = [&](auto buf_tag, int blk) {
      constexpr int BUF = decltype(buf_tag)::value;
      const char* tile = BUF ? tile1 : tile0;
      char* other = BUF ? tile0 : tile1;
      char* pw = (BUF ? pds1 : pds0) + pw_off;
      if (blk < nblk) {
        uint64_t mask_nxt = 0;
        if (blk + 1 < nblk) mask_nxt = __ballot(slot_in_range(idx_nxt, S_kv));
        const int32_t idx_g = idx_nxt;
        idx_cur = idx_nxt;
        idx_nxt = blk + 2 < nblk ? load_idx(blk + 2) : -1;
        const uint64_t mask = mask_cur;
        mask_cur = mask_nxt;
        if (mask == 0) {
          if (mask_nxt) gather.all(idx_g, mask_nxt, other, lane, wu);
        } else {
          // the next tile goes out in parts from inside the score loop; with no next block the parts
          // read the zero row into the idle buffer, which nothing reads before the next wait
          auto gather_hook = [&](int i) {
#pragma unroll
            for (int k = 0; k < G::NP; k++)
              if (i == (k * NFS) / G::NP + NFS / G::NP / 2) gather.part(k, idx_g, mask_nxt, other, lane, wu);
          };
          f32x4 sacc[2], dpacc[2];
          bwd_scores<D, PF>(tile, sc_off, qb, dob, sacc, dpacc, gather_hook);
          const uint32_t vb = (uint32_t)(mask >> (4 * g));
#pragma unroll
          for (int mt = 0; mt < 2; mt++) {
            float p[4], ds[4];
#pragma unroll
            for (int r = 0; r < 4; r++)
              p[r] = ((vb >> (16 * mt + r)) & 1u) ? fast_exp2(sacc[mt][r] * scale_log2 - lse_h) : 0.f;
#pragma unroll
            for (int r = 0; r < 4; r++)  // saturated to the fp16 range: only inputs outside the bound's assumptions reach it
              ds[r] = __builtin_amdgcn_fmed3f(
                  __builtin_amdgcn_ldexpf(sm_scale * p[r] * (dpacc[mt][r] - delta_h), sqo), -65504.f, 65504.f);
            f16_hilo4(ds, (uint2*)(pw + 32 * mt), (uint2*)(pw + 32 * mt + SB));
            if (ds_out)  // dS = P (dP - Delta) in bf16 for the dQ kernel (bwd_dq_ds_kernel)
              *(uint2*)(ds_out + ds_off + (int64_t)blk * (HB * T) + mt * 1024) =
                  pack4_bf16(p[0] * (dpacc[mt][0] - delta_h), p[1] * (dpacc[mt][1] - delta_h),
                             p[2] * (dpacc[mt][2] - delta_h), p[3] * (dpacc[mt][3] - delta_h));
            const f16x2 p01 = __builtin_convertvector((f32x2){p[0], p[1]}, f16x2);
            const f16x2 p23 = __builtin_convertvector((f32x2){p[2], p[3]}, f16x2);
            *(uint2*)(pw + 32 * mt + 2 * SB) =
                make_uint2(__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23));
          }
        }
        wait_all_mem();  // this wave's part of tile blk + 1
      }
      lds_barrier();
    };
    for (int blk = 0; blk <= nblk; blk += 2) {
      sblock(IntTag<0>{}, blk);
      if (blk + 1 <= nblk) sblock(IntTag<1>{}, blk + 1);
    }
  } else {
    // -------- product waves: wave NW + kw owns dKV columns kw DW .. kw DW + DW - 1 --------
    const int kw = wu - NW;
    // Q and dO with heads along k, as A operands of dKV^T: lane l holds d = kw DW + 32 dt + (l & 31)
    // and heads 16 ks + 8 kg .. +7, read with transposing LDS loads from the row-major copy
    f16x8 qv[NDT][KH], dov[NDT][KH];
    auto read_frags = [&](f16x8 (&dst)[NDT][KH]) {
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int ks = 0; ks < KH; ks++) {
          const int hb0 = 16 * ks;  // first head of the k-step: all 16 sit in one buffer
          const char* sb = hb0 < HH ? tile0 : tile1;
          const int h0 = hb0 % HH + 8 * kg + ((lane & 15) >> 2);
          const int d = kw * DW + 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
          dst[dt][ks] = __builtin_bit_cast(
              f16x8, join_tr(lds_load_tr(sb + (h0 * D + d) * 2), lds_load_tr(sb + ((h0 + 4) * D + d) * 2)));
        }
    };
    read_frags(qv);
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int ks = 0; ks < KH; ks++) keep_in_agpr(qv[dt][ks]);
    __syncthreads();  // all product waves have read Q
    put_dout();
    __syncthreads();  // the dO copy is complete
    read_frags(dov);
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int ks = 0; ks < KH; ks++) keep_in_agpr(dov[dt][ks]);
    __syncthreads();  // all product waves have read dO

    const int32_t* pos_tok = pos + ctok * (int64_t)topk;
    auto load_pos = [&](int blk) -> int32_t {
      const int t = blk * T + lane;
      return (lane < T && t < topk) ? pos_tok[t] : -1;
    };
    // masked slots of a partly valid block store into this workgroup's spare row (after all staging
    // rows of the chunk), so the stores need no per-slot branches
    const int32_t spare = (n_tokens * topk + (int32_t)ctok) * n_hblk + hblk;
    int32_t idx_cur = load_idx(0), pos_cur = load_pos(0);
    __syncthreads();  // tile 0 is complete (the score waves' set-up)

    // A block's products go to c; finish() then writes them out (exponent, int16 transpose, staging
    // stores) before the stage ends. The stores thus share the vector memory path with the score
    // waves' softmax rather than with their gathers; finishing each block at the top of the next
    // stage instead (over the score waves' MFMAs and gathers) measured no faster, as that path
    // bounds the kernel.
    f32x16 c[NDT];
    int32_t dst_c = 0;  // staging row of slot lane & 31 of the block in c (lanes < T)
    auto finish = [&]() {
      // per-lane addresses are derived here from an opaque copy of the lane id, so that the
      // compiler does not hoist them out of the block loop and hold them in registers
      int ln = lane;
      asm volatile("" : "+v"(ln));
      // one exponent per slot row segment (this lane and lane ^ 32 hold the row's values)
      int es;
      const float sc = bfp16_scale(c, so, &es);
      // int16 runs of four d into this wave's transpose buffer (C layout: lane holds slot lane & 31,
      // d = kw DW + 32 i + 8 (r >> 2) + 4 kg + (r & 3))
      char* ob = obuf[kw] + (ln & 31) * OP + 8 * (ln >> 5);
#pragma unroll
      for (int i = 0; i < NDT; i++)
#pragma unroll
        for (int jj = 0; jj < 4; jj++)
          *(i32x2*)(ob + obuf_chunk(ln & 31, 4 * i + jj)) =
              i32x2{(int)bfp16_pair(c[i][4 * jj], c[i][4 * jj + 1], sc), (int)bfp16_pair(c[i][4 * jj + 2], c[i][4 * jj + 3], sc)};
      // row read-back: lane covers d0 .. d0 + 7 of slot row n RPS + lane / LPR
      const int d0 = kw * DW + 8 * (ln % LPR);
#pragma unroll
      for (int n = 0; n < NI; n++) {
        const int row = n * RPS + ln / LPR;
        const i32x4 v = *(const i32x4*)(obuf[kw] + row * OP + obuf_chunk(row, ln % LPR));
        const int32_t rowi = __shfl(dst_c, row);
        __builtin_nontemporal_store(v, (i32x4*)(stage + (int64_t)rowi * D + d0));
      }
      if (lane < T) stage_exp[(int64_t)dst_c * NSEG + kw] = (int8_t)es;
    };
    auto pblock = [&](auto buf_tag, int j) {
      constexpr int BUF = decltype(buf_tag)::value;
      if (j >= 1) {
        const int blk = j - 1;
        const int32_t idx_this = idx_cur, pos_this = pos_cur;
        if (blk + 1 < nblk) {
          idx_cur = load_idx(blk + 1);
          pos_cur = load_pos(blk + 1);
        }
        const bool valid = slot_in_range(idx_this, S_kv);
        const uint64_t mask = __ballot(valid);
        if (mask) {
          int ln = lane;
          asm volatile("" : "+v"(ln));
          // dKV^T B fragments: lane l gets slot (l & 31) and heads 16 ks + 8 kg .. +7, two
          // transposing reads 4 heads apart; block j - 1 went through pds<(j - 1) & 1>
          const char* pr = (BUF ? pds0 : pds1) +
                           ((8 * (ln >> 5) + ((ln & 15) >> 2)) * T + 16 * ((ln >> 4) & 1) + 4 * (ln & 3)) * 2;
          dst_c = valid ? pos_this + hblk : spare;
          auto bfrag = [&](int ks, int m) {
            const char* p = pr + m * SB + ks * 16 * T * 2;
            return __builtin_bit_cast(f16x8, join_tr(lds_load_tr(p), lds_load_tr(p + 4 * T * 2)));
          };
          // 2^-so dKV^T[d, slot] = (2^-sq Q)^T (2^(sq-so) sm_scale (dS_hi + dS_lo)) + (2^-so dO)^T P
#pragma unroll
          for (int i = 0; i < NDT; i++)
#pragma unroll
            for (int r = 0; r < 16; r++) c[i][r] = 0.f;
          f16x8 bcur[3], bnxt[3];
#pragma unroll
          for (int m = 0; m < 3; m++) bcur[m] = bfrag(0, m);
#pragma unroll
          for (int ks = 0; ks < KH; ks++) {
            __builtin_amdgcn_sched_barrier(0);
            if (ks + 1 < KH) {
#pragma unroll
              for (int m = 0; m < 3; m++) bnxt[m] = bfrag(ks + 1, m);
            }
#pragma unroll
            for (int i = 0; i < NDT; i++) c[i] = mfma32h(qv[i][ks], bcur[0], c[i]);
#pragma unroll
            for (int i = 0; i < NDT; i++) c[i] = mfma32h(qv[i][ks], bcur[1], c[i]);
#pragma unroll
            for (int i = 0; i < NDT; i++) c[i] = mfma32h(dov[i][ks], bcur[2], c[i]);
            if (ks + 1 < KH) {
#pragma unroll
              for (int m = 0; m < 3; m++) bcur[m] = bnxt[m];
            }
          }
          __builtin_amdgcn_sched_barrier(0);
          finish();
        }
      }
      lds_barrier();
    };
    for (int j = 0; j <= nblk; j += 2) {
      pblock(IntTag<0>{}, j);
      if (j + 1 <= nblk) pblock(IntTag<1>{}, j + 1);
    }
  }
  wait_all_mem();
}

// ---------------------------------------------------------------------------------------------
// Segmented scatter-add of dKV. Every valid (token, slot) pair gets n_hblk consecutive rows of a
// staging buffer, grouped by kv row and, within a row, in an order fixed by the token indices (a
// token with place k among its batch's tokens of the chunk sorts by (k % nw, k / nw), nw below). The
// dKV kernel stores each contribution row there with plain stores, and reduce_rows sums each kv
// row's segment in that order. This moves the payload through the store and streaming-read paths
// instead of the fp32 atomic units, and the result does not depend on the order in which
// workgroups run.
//
// The plan takes no global atomics on the common path. For a chunk of n_chunk tokens, kv row `row`
// of batch b has nw = ceil(min(n_chunk, S) / 32) words of a selection bitmap covering batch b's
// tokens of the chunk, and the token with place k among them owns bit k / nw of word k % nw; a set
// bit records that the token selects the row. Next to each word sits the count of its pairs (word
// e = row * nw + word is stored as {bits, count} at bc[plan_word(row, word)]). An exclusive scan of
// n_hblk * count over the words in (row, word) order gives each word the staging row of its first
// pair. In a word whose count equals its popcount (each of its tokens selects the row once, as
// top-k selections do), a pair's staging row is that plus n_hblk times the word's pairs below its
// bit: positions then depend on the indices only, and row r's segment is
// [offset[r nw], offset[(r + 1) nw]). A word with duplicate (token, row) pairs hands out its range
// [offset[e], offset[e + 1]) through an atomic cursor cur[e] instead.

// One workgroup per (word column w0, tile of MARK_ROWS kv rows): for each batch with rows in the
// tile, the (up to 32) tokens with places w0 + nw j own every word of the column, so the workgroup
// builds the tile's words in LDS (LDS atomics) and writes them out with plain stores. 32 KiB of LDS
// lets a workgroup sit beside a forward workgroup (~117 KiB) on one CU when the plan runs on a side
// stream.
constexpr int MARK_ROWS = 4096;
// Storage place of word w of kv row `row` among the n_rows * nw words: tile-major, so that the mark
// kernel's workgroup (word column w, tile of MARK_ROWS rows) writes its words as one contiguous run
// (the last tile holds fewer rows). The scan walks the words in (row, word) order through this map.
__device__ __forceinline__ int64_t plan_word(int64_t row, int64_t w, int64_t nw, int64_t n_rows) {
  const int64_t t = row / MARK_ROWS, r0 = t * MARK_ROWS;
  const int64_t rows_t = n_rows - r0 < MARK_ROWS ? n_rows - r0 : MARK_ROWS;
  return r0 * nw + w * rows_t + (row - r0);
}

__global__ void __launch_bounds__(256)
mark_kernel(const int32_t* __restrict__ idx, int2* __restrict__ bc, int64_t token0, int64_t n_chunk, int64_t S,
            int64_t S_kv, int topk, int64_t nw, int64_t n_rows) {
  __shared__ uint32_t lb[MARK_ROWS];
  __shared__ int32_t lc[MARK_ROWS];
  const int64_t n_units = nw * ((n_rows + MARK_ROWS - 1) / MARK_ROWS);
  const int64_t c_lo = token0 / S, c_hi = (token0 + n_chunk - 1) / S;  // batches of the chunk
  for (int64_t u = blockIdx.x; u < n_units; u += gridDim.x) {  // the grid is capped
    const int64_t w0 = u % nw;
    const int64_t r0 = (u / nw) * MARK_ROWS;
    const int nr = (int)(n_rows - r0 < MARK_ROWS ? n_rows - r0 : MARK_ROWS);
    for (int r = threadIdx.x; r < nr; r += 256) {
      lb[r] = 0u;
      lc[r] = 0;
    }
    __syncthreads();
    // the batches with rows in this tile; a row of batch b takes bits from batch b's tokens only
    const int64_t b_lo = r0 / S_kv, b_hi = (r0 + nr - 1) / S_kv;
    for (int64_t b = (b_lo > c_lo ? b_lo : c_lo); b <= (b_hi < c_hi ? b_hi : c_hi); b++) {
      const int64_t first = token0 > b * S ? token0 : b * S;
      const int64_t last = token0 + n_chunk < (b + 1) * S ? token0 + n_chunk : (b + 1) * S;
      const int64_t rb = b * S_kv - r0;  // the batch's rows, relative to the tile
      // the column's tokens one after another, each token's indices in chunks of MU per thread
      // whose loads all go out before the chunk's LDS atomics
      constexpr int MU = 8;
      for (int j = 0; j < 32; j++) {
        const int64_t token = first + w0 + nw * j;
        if (token >= last) break;
        const int32_t* it = idx + token * topk;
        for (int t0 = threadIdx.x; t0 < topk; t0 += MU * 256) {
          int32_t v[MU];
#pragma unroll
          for (int u = 0; u < MU; u++) v[u] = t0 + u * 256 < topk ? it[t0 + u * 256] : -1;
#pragma unroll
          for (int u = 0; u < MU; u++) {
            if (slot_in_range(v[u], S_kv)) {
              const int64_t r = rb + v[u];
              if (r >= 0 && r < nr) {
                atomicOr(lb + r, 1u << j);
                atomicAdd(lc + r, 1);
              }
            }
          }
        }
      }
    }
    __syncthreads();
    int2* out = bc + plan_word(r0, w0, nw, n_rows);  // the column's words of this tile, contiguous
    for (int r = threadIdx.x; r < nr; r += 256) out[r] = make_int2((int)lb[r], lc[r]);
    __syncthreads();  // lb and lc are cleared for the next unit
  }
}

// Exclusive scan of the words' staging-row counts, in tiles of SCAN_TILE words (below).
constexpr int SCAN_TILE = 4096;  // 256 threads x 16

// pos[ct, slot] = the slot's first staging row, or -1 for a masked slot. Workgroup unit u covers
// POS_SLOTS slots of chunk token u / tpt (tpt units per token), so the token and batch come from
// one wave-uniform division per unit; a thread takes four slots 256 apart and issues each level of
// its loads (indices, then the words and tile bases they name) for all four before using any. A
// word's first staging row is its scan tile's base plus its prefix inside the tile, both left by
// the scan, so each slot reads one word at random.
constexpr int POS_PER_THREAD = 4;
constexpr int POS_SLOTS = 256 * POS_PER_THREAD;
__global__ void __launch_bounds__(256)
position_kernel(const int32_t* __restrict__ idx, const int2* __restrict__ bc, int32_t* __restrict__ cur,
                const int32_t* __restrict__ tile_base, int32_t* __restrict__ pos, int64_t token0, int64_t n_chunk,
                int64_t S, int64_t S_kv, int topk, int64_t nw, int n_hblk, int64_t n_rows) {
  constexpr int PU = POS_PER_THREAD;
  const int64_t tpt = (topk + POS_SLOTS - 1) / POS_SLOTS;
  for (int64_t u = blockIdx.x; u < n_chunk * tpt; u += gridDim.x) {
    const int64_t ct = u / tpt;
    const int t0 = (int)(u - ct * tpt) * POS_SLOTS + (int)threadIdx.x;
    const int64_t token = token0 + ct;
    const int64_t b = token / S;
    const int64_t k = token - (token0 > b * S ? token0 : b * S);  // the token's place among its batch's
    int32_t v[PU];
#pragma unroll
    for (int q = 0; q < PU; q++) v[q] = t0 + 256 * q < topk ? idx[token * topk + t0 + 256 * q] : -1;
    // words after scan_tiles_kernel: {bits, prefix inside the scan tile | duplicate flag}; e is the
    // word's place in (row, word) order (scan tiles, cursors), pw where it is stored
    int64_t e[PU];
    int2 w[PU];
    int32_t tb[PU];
#pragma unroll
    for (int q = 0; q < PU; q++) {
      const bool ok = slot_in_range(v[q], S_kv);
      e[q] = ok ? (b * S_kv + v[q]) * nw + k % nw : -1;
      w[q] = ok ? bc[plan_word(b * S_kv + v[q], k % nw, nw, n_rows)] : make_int2(0, 0);
      tb[q] = ok ? tile_base[e[q] / SCAN_TILE] : 0;
    }
#pragma unroll
    for (int q = 0; q < PU; q++) {
      int32_t r = -1;
      if (e[q] >= 0) {
        const int32_t off = tb[q] + (w[q].y & 0x7FFFFFFF);  // the word's first staging row
        if (w[q].y >= 0)
          r = off + n_hblk * __popc((uint32_t)w[q].x & ((1u << (k / nw)) - 1u));
        else
          r = off + atomicAdd(cur + e[q], n_hblk);  // a word with duplicate pairs
      }
      if (t0 + 256 * q < topk) pos[ct * topk + t0 + 256 * q] = r;
    }
  }
}

// Exclusive scan of n int32 counts into offset[0..n] (offset[n] = total), three passes:
// per-tile scans of SCAN_TILE elements, a scan of the tile totals, then the tile bases.

__device__ __forceinline__ int32_t block_exclusive_scan_256(int32_t v, int32_t* sh, int32_t* total) {
  // v: this thread's value; returns the exclusive prefix over the 256 threads of the block.
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int32_t x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int32_t base = 0;
  for (int i = 0; i < w; i++) base += sh[i];
  *total = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return base + x - v;
}

// Scan input: element e is n_hblk times word e's pair count, the staging rows of its pairs. The
// tile passes through LDS (element l at l + l / 32, against bank conflicts) so that global loads
// and stores run along consecutive elements while each thread scans 16 consecutive ones. The word
// then trades its count for what position_kernel needs: its exclusive prefix inside the tile, with
// bit 31 set when the count exceeds the popcount (a word holding duplicate pairs); the tile's base
// comes from tile_sum once the totals are scanned.
__global__ void __launch_bounds__(256)
scan_tiles_kernel(int2* __restrict__ bc, int32_t* __restrict__ out, int32_t* __restrict__ tile_sum,
                  int64_t n, int n_hblk, int64_t nw, int64_t n_rows) {
  __shared__ int32_t sh[4];
  __shared__ int32_t sv[SCAN_TILE + SCAN_TILE / 32];
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE;
  const int t = threadIdx.x;
  // element base + l is word (w0 + l) % nw of row row0 + (w0 + l) / nw
  const int64_t row0 = base / nw;
  const uint32_t w0 = (uint32_t)(base - row0 * nw), unw = (uint32_t)nw;
  int64_t pw[16];
  int2 wd[16];
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int l = 256 * i + t;
    const uint32_t x = w0 + (uint32_t)l;
    pw[i] = plan_word(row0 + x / unw, x % unw, nw, n_rows);
    wd[i] = base + l < n ? bc[pw[i]] : make_int2(0, 0);
    sv[l + l / 32] = n_hblk * wd[i].y;
  }
  __syncthreads();
  int32_t v[16];
  int32_t s = 0;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int l = 16 * t + i;
    v[i] = sv[l + l / 32];
    s += v[i];
  }
  int32_t total;
  int32_t run = block_exclusive_scan_256(s, sh, &total);
#pragma unroll
  for (int i = 0; i < 16; i++) {  // each thread overwrites only the elements it read
    const int l = 16 * t + i;
    sv[l + l / 32] = run;
    run += v[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const int l = 256 * i + t;
    if (base + l < n) {
      const int32_t ex = sv[l + l / 32];
      out[base + l] = ex;
      const bool dup = wd[i].y != __popc((uint32_t)wd[i].x);
      bc[pw[i]] = make_int2(wd[i].x, dup ? (int32_t)(0x80000000u | (uint32_t)ex) : ex);
    }
  }
  if (t == 0) tile_sum[blockIdx.x] = total;
}

// Single workgroup: exclusive scan of the tile totals (in place), total into out[n].
__global__ void __launch_bounds__(256)
scan_totals_kernel(int32_t* __restrict__ tile_sum, int64_t n_tiles, int32_t* __restrict__ out, int64_t n) {
  __shared__ int32_t sh[4];
  int32_t carry = 0;
  for (int64_t b0 = 0; b0 < n_tiles; b0 += 256) {
    const int64_t i = b0 + threadIdx.x;
    const int32_t v = i < n_tiles ? tile_sum[i] : 0;
    int32_t total;
    const int32_t ex = block_exclusive_scan_256(v, sh, &total);
    if (i < n_tiles) tile_sum[i] = carry + ex;
    carry += total;
  }
  if (threadIdx.x == 0) out[n] = carry;
}

__global__ void __launch_bounds__(256)
scan_add_kernel(int32_t* __restrict__ out, const int32_t* __restrict__ tile_sum, int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * SCAN_TILE + threadIdx.x;
  const int32_t add = tile_sum[blockIdx.x];
#pragma unroll
  for (int i = 0; i < 16; i++)
    if (base + 256 * i < n) out[base + 256 * i] += add;
}

// One workgroup per kv row: sum the row's staging segment in fp32 (fixed order), optionally add
// the running accumulator (earlier token chunks), then write fp32 and/or bf16 output.
template <int D>
__global__ void __launch_bounds__(256)
reduce_rows_kernel(const uint16_t* __restrict__ stage, const int8_t* __restrict__ stage_exp, int nseg,
                   const int32_t* __restrict__ offset, int64_t stride, f32x4* __restrict__ acc,
                   uint4* __restrict__ out_bf16, int accumulate, int64_t n_rows) {
  // Workgroups loop over kv rows (the grid is capped); a row's segment is
  // [offset[row * stride], offset[(row + 1) * stride]).
  // Thread c of a group takes values 8c .. 8c+7 of every NG-th staging row of the segment.
  constexpr int F8 = D / 8;         // 16-byte pieces of int16 per row
  constexpr int NG = 256 / F8;      // thread groups
  static_assert(NG >= 1 && 256 % F8 == 0, "row width");
  __shared__ f32x4 part[NG][F8][2];
  const int g = threadIdx.x / F8, c = threadIdx.x % F8;
  f32x4 lo, hi;
  // values 8c .. 8c+7 of a row: int16 pairs (the lower value in the low half) times 2^e
  auto lo16 = [](int x) { return (float)(int)(int16_t)(uint16_t)(uint32_t)x; };
  auto hi16 = [](int x) { return (float)(x >> 16); };
  auto add = [&](const i32x4& raw, int e) {
#pragma unroll
    for (int k = 0; k < 2; k++) {
      lo[2 * k] += __builtin_amdgcn_ldexpf(lo16(raw[k]), e);
      lo[2 * k + 1] += __builtin_amdgcn_ldexpf(hi16(raw[k]), e);
      hi[2 * k] += __builtin_amdgcn_ldexpf(lo16(raw[2 + k]), e);
      hi[2 * k + 1] += __builtin_amdgcn_ldexpf(hi16(raw[2 + k]), e);
    }
  };
  auto ld = [&](int32_t i) { return __builtin_nontemporal_load((const i32x4*)(stage + (int64_t)i * D) + c); };
  const int seg = 8 * c * nseg / D;  // exponent segment of this thread's 8 values
  auto lde = [&](int32_t i) { return (int)stage_exp[(int64_t)i * nseg + seg]; };
  for (int64_t row = blockIdx.x; row < n_rows; row += gridDim.x) {
    const int32_t beg = offset[row * stride], end = offset[(row + 1) * stride];
    lo = f32x4{0.f, 0.f, 0.f, 0.f};
    hi = lo;
    int32_t i = beg + g;
    // eight rows in flight per thread, then four, then one (the order of the sums stays row order)
    for (; i + 7 * NG < end; i += 8 * NG) {
      i32x4 r[8];
      int e[8];
#pragma unroll
      for (int k = 0; k < 8; k++) r[k] = ld(i + k * NG);
#pragma unroll
      for (int k = 0; k < 8; k++) e[k] = lde(i + k * NG);
#pragma unroll
      for (int k = 0; k < 8; k++) add(r[k], e[k]);
    }
    for (; i + 3 * NG < end; i += 4 * NG) {
      const i32x4 r0 = ld(i), r1 = ld(i + NG), r2 = ld(i + 2 * NG), r3 = ld(i + 3 * NG);
      const int e0 = lde(i), e1 = lde(i + NG), e2 = lde(i + 2 * NG), e3 = lde(i + 3 * NG);
      add(r0, e0);
      add(r1, e1);
      add(r2, e2);
      add(r3, e3);
    }
    for (; i < end; i += NG) add(ld(i), lde(i));
    part[g][c][0] = lo;
    part[g][c][1] = hi;
    __syncthreads();
    if (g == 0) {
      f32x4 t0 = part[0][c][0], t1 = part[0][c][1];
      for (int k = 1; k < NG; k++) {
        t0 += part[k][c][0];
        t1 += part[k][c][1];
      }
      if (accumulate) {
        t0 += acc[row * (D / 4) + 2 * c];
        t1 += acc[row * (D / 4) + 2 * c + 1];
      }
      if (acc) {
        acc[row * (D / 4) + 2 * c] = t0;
        acc[row * (D / 4) + 2 * c + 1] = t1;
      }
      if (out_bf16) {
        const uint2 a = pack4_bf16(t0[0], t0[1], t0[2], t0[3]), b = pack4_bf16(t1[0], t1[1], t1[2], t1[3]);
        out_bf16[row * F8 + c] = make_uint4(a.x, a.y, b.x, b.y);
      }
    }
    __syncthreads();  // part is rewritten for the next row
  }
}

// ---------------------------------------------------------------------------------------------
hipError_t launch_bwd_preprocess(const void* o, const void* d_o, float* delta, int64_t rows, int64_t D,
                                 hipStream_t st) {
  const int64_t rpb = 4 * (64 / (D / 8));  // rows per 256-thread block and pass
  const int64_t groups = (rows + rpb - 1) / rpb;
  const dim3 grid((unsigned)(groups < (1 << 20) ? groups : (1 << 20))), block(256);
  if (D == 512)
    hipLaunchKernelGGL(delta_kernel<512>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else if (D == 256)
    hipLaunchKernelGGL(delta_kernel<256>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else if (D == 128)
    hipLaunchKernelGGL(delta_kernel<128>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else if (D == 64)
    hipLaunchKernelGGL(delta_kernel<64>, grid, block, 0, st, (const uint16_t*)o, (const uint16_t*)d_o, delta, rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_bwd_dsink(const float* lse, const float* delta, const float* sink, float* d_sink, int64_t tokens,
                            int64_t H, hipStream_t st) {
  hipLaunchKernelGGL(dsink_kernel, dim3((unsigned)H), dim3(256), 0, st, lse, delta, sink, d_sink, tokens, (int)H);
  return hipGetLastError();
}

hipError_t launch_kv_row_norm(const void* kv, int64_t rows, int64_t D, float* norm, hipStream_t st) {
  const int64_t per_block = 256 / (D / 8);
  int64_t g = (rows + per_block - 1) / per_block;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  if (D == 512)
    hipLaunchKernelGGL(kv_row_norm_kernel<512>, dim3((unsigned)g), dim3(256), 0, st, (const uint16_t*)kv, rows, norm);
  else if (D == 256)
    hipLaunchKernelGGL(kv_row_norm_kernel<256>, dim3((unsigned)g), dim3(256), 0, st, (const uint16_t*)kv, rows, norm);
  else if (D == 128)
    hipLaunchKernelGGL(kv_row_norm_kernel<128>, dim3((unsigned)g), dim3(256), 0, st, (const uint16_t*)kv, rows, norm);
  else if (D == 64)
    hipLaunchKernelGGL(kv_row_norm_kernel<64>, dim3((unsigned)g), dim3(256), 0, st, (const uint16_t*)kv, rows, norm);
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
  const float sl2 = a.sm_scale * kLog2e;
  if constexpr (NW == 4 && D == 512) {
    if (which & 1) {  // 64 heads at D = 512: the specialised-wave dQ kernel
      const int n_tokens = (int)(a.B * a.S);
      hipLaunchKernelGGL((bwd_dq_ws_kernel<D>), dim3((unsigned)(n_tokens * n_hblk)), dim3(512), 0, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.kv, (const uint16_t*)a.d_o, a.idx, a.lse, a.delta,
                         (uint16_t*)a.dq, (int)a.S, a.S_kv, (int)a.H, (int)a.topk, a.sm_scale, sl2, n_hblk, n_tokens);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
      which &= ~1;
    }
  }
  if (which & 1) {
    const int n_tokens = (int)(a.B * a.S);
    hipLaunchKernelGGL((bwd_dq_kernel<D, NW>), dim3((unsigned)(n_tokens * n_hblk)), dim3(NW * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, (const uint16_t*)a.d_o, a.idx, a.lse, a.delta,
                       (uint16_t*)a.dq, (int)a.S, a.S_kv, (int)a.H, (int)a.topk, a.sm_scale, sl2, n_hblk, n_tokens);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!(which & 2)) return hipSuccess;
  if (a.stage) {
    // 64 heads at D = 512: the specialised-wave kernel (eight waves, two per SIMD)
    if constexpr (NW == 4 && D == 512)
      hipLaunchKernelGGL((bwd_dkv_ws_kernel<D, NW>), dim3((unsigned)(a.n_chunk * n_hblk)), dim3(NW * 128), 0, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.kv, (const uint16_t*)a.d_o, a.idx, a.lse, a.delta,
                         a.pos, a.stage, a.stage_exp, a.row_norm, (int)a.S, a.S_kv, (int)a.H, (int)a.topk, a.sm_scale,
                         sl2, n_hblk, (int)a.token0, (int)a.n_chunk, a.ds);
    else
      hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, true>), dim3((unsigned)(a.n_chunk * n_hblk)), dim3(NW * 64), 0, st,
                         (const uint16_t*)a.q, (const uint16_t*)a.kv, (const uint16_t*)a.d_o, a.idx, a.lse, a.delta,
                         nullptr, a.pos, a.stage, a.stage_exp, a.row_norm, (int)a.S, a.S_kv, (int)a.H, (int)a.topk,
                         a.sm_scale, sl2, n_hblk, (int)a.token0, (int)a.n_chunk);
  } else {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, NW, false>), dim3((unsigned)(a.n_chunk * n_hblk)), dim3(NW * 64), 0, st,
                       (const uint16_t*)a.q, (const uint16_t*)a.kv, (const uint16_t*)a.d_o, a.idx, a.lse, a.delta,
                       a.dkv_accum, nullptr, nullptr, nullptr, nullptr, (int)a.S, a.S_kv, (int)a.H, (int)a.topk,
                       a.sm_scale, sl2, n_hblk, (int)a.token0, (int)a.n_chunk);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_dq_ds(const BwdMainArgs& a, hipStream_t st) {
  if (!dq_from_ds(a.H, a.D) || !a.ds) return hipErrorInvalidValue;
  const int n_hblk = (int)(a.H / 64);
  hipLaunchKernelGGL((bwd_dq_ds_kernel<512>), dim3((unsigned)(a.n_chunk * n_hblk)), dim3(512), 0, st,
                     (const uint16_t*)a.kv, a.idx, (const uint16_t*)a.ds, (uint16_t*)a.dq, (int)a.S, a.S_kv,
                     (int)a.H, (int)a.topk, a.sm_scale, n_hblk, (int)a.token0, (int)a.n_chunk);
  return hipGetLastError();
}

hipError_t launch_bwd_main(const BwdMainArgs& a, int which, hipStream_t st) {
  const int hb = bwd_heads_per_wg(a.H);
  if (a.D == 512) {
    if (hb == 64) return launch_bwd_main_t<512, 4>(a, which, st);
    if (hb == 32) return launch_bwd_main_t<512, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<512, 1>(a, which, st);
  } else if (a.D == 256) {
    if (hb == 64) return launch_bwd_main_t<256, 4>(a, which, st);
    if (hb == 32) return launch_bwd_main_t<256, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<256, 1>(a, which, st);
  } else if (a.D == 128) {
    if (hb == 64) return launch_bwd_main_t<128, 4>(a, which, st);
    if (hb == 32) return launch_bwd_main_t<128, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<128, 1>(a, which, st);
  } else if (a.D == 64) {
    if (hb == 32) return launch_bwd_main_t<64, 2>(a, which, st);
    if (hb == 16) return launch_bwd_main_t<64, 1>(a, which, st);
  }
  return hipErrorInvalidValue;
}

static unsigned grid_for(int64_t n, int64_t per_block, int64_t cap = 65536) {
  int64_t g = (n + per_block - 1) / per_block;
  if (g > cap) g = cap;
  return (unsigned)(g < 1 ? 1 : g);
}

int64_t scan_tiles(int64_t n) { return (n + SCAN_TILE - 1) / SCAN_TILE; }
int64_t dkv_row_words(int64_t n_chunk, int64_t S) { return ((n_chunk < S ? n_chunk : S) + 31) / 32; }
int64_t dkv_bitmap_words(int64_t n_rows, int64_t n_chunk, int64_t S) { return n_rows * dkv_row_words(n_chunk, S); }

hipError_t launch_dkv_prepare(const int32_t* idx, uint32_t* plan, int32_t* offset, int32_t* tile_sum, int32_t* pos,
                              int64_t B, int64_t S, int64_t S_kv, int64_t topk, int n_hblk, int64_t token0,
                              int64_t n_chunk, hipStream_t st) {
  const int64_t nw = dkv_row_words(n_chunk, S), n_rows = B * S_kv;
  const int64_t n = dkv_bitmap_words(n_rows, n_chunk, S);
  int2* bc = (int2*)plan;             // {bits, count} per word, written whole by mark_kernel
  int32_t* cur = (int32_t*)(plan + 2 * n);  // cursors of words with duplicate pairs
  hipError_t e = launch_fill_zero_f32((float*)cur, (n + 3) / 4 * 4, st);
  if (e != hipSuccess) return e;
  const int64_t mark_units = nw * ((n_rows + MARK_ROWS - 1) / MARK_ROWS);
  hipLaunchKernelGGL(mark_kernel, dim3(grid_for(mark_units, 1, 1 << 20)), dim3(256), 0, st, idx, bc, token0, n_chunk,
                     S, S_kv, (int)topk, nw, n_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t tiles = scan_tiles(n);
  hipLaunchKernelGGL(scan_tiles_kernel, dim3((unsigned)tiles), dim3(256), 0, st, bc, offset, tile_sum, n, n_hblk, nw,
                     n_rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_totals_kernel, dim3(1), dim3(256), 0, st, tile_sum, tiles, offset, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(scan_add_kernel, dim3((unsigned)tiles), dim3(256), 0, st, offset, (const int32_t*)tile_sum, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t n_units = n_chunk * ((topk + POS_SLOTS - 1) / POS_SLOTS);
  hipLaunchKernelGGL(position_kernel, dim3(grid_for(n_units, 1)), dim3(256), 0, st, idx, (const int2*)bc, cur,
                     (const int32_t*)tile_sum, pos, token0, n_chunk, S, S_kv, (int)topk, nw, n_hblk, n_rows);
  return hipGetLastError();
}

hipError_t launch_reduce_rows(const uint16_t* stage, const int8_t* stage_exp, int nseg, const int32_t* offset,
                              int64_t stride, float* acc, void* out_bf16, int accumulate, int64_t n_rows, int64_t D,
                              hipStream_t st) {
  const dim3 grid((unsigned)(n_rows < (1 << 22) ? n_rows : (1 << 22)));
  if (D == 512)
    hipLaunchKernelGGL(reduce_rows_kernel<512>, grid, dim3(256), 0, st, stage, stage_exp, nseg, offset, stride,
                       (f32x4*)acc, (uint4*)out_bf16, accumulate, n_rows);
  else if (D == 256)
    hipLaunchKernelGGL(reduce_rows_kernel<256>, grid, dim3(256), 0, st, stage, stage_exp, nseg, offset, stride,
                       (f32x4*)acc, (uint4*)out_bf16, accumulate, n_rows);
  else if (D == 128)
    hipLaunchKernelGGL(reduce_rows_kernel<128>, grid, dim3(256), 0, st, stage, stage_exp, nseg, offset, stride,
                       (f32x4*)acc, (uint4*)out_bf16, accumulate, n_rows);
  else if (D == 64)
    hipLaunchKernelGGL(reduce_rows_kernel<64>, grid, dim3(256), 0, st, stage, stage_exp, nseg, offset, stride,
                       (f32x4*)acc, (uint4*)out_bf16, accumulate, n_rows);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace smqa

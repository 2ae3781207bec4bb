// Device-side helpers shared by the gfx950 kernels of libsparse_mqa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace smqa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define SMQA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.44269504088896340736f;

// v_mfma_f32_32x32x16_bf16. Operand lane layout: lane l holds row/col (l & 31) and eight
// k-values of k-group (l >> 5); C lane l holds column (l & 31), rows 8*(r/4) + 4*(l>>5) + r%4.
// Any k-permutation is fine as long as A and B use the same one.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x32_bf16. Lane l holds row/col (l & 15) and k-group (l >> 4); C lane l holds
// column (l & 15), rows 4*(l>>4) + r.
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_f16: operand layouts as mfma32.
__device__ __forceinline__ f32x16 mfma32h(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds_load16(const char* p) {
  return *(const SMQA_LDS bf16x8*)(const SMQA_LDS char*)p;
}
// ds_read_b64_tr_b16. Within each group of 16 lanes, lane 4*r + c points at row r, columns
// 4c..4c+3 of a 4x16 block of 16-bit elements; lane j receives column j of rows 0..3.
__device__ __forceinline__ s16x4 lds_load_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((SMQA_LDS s16x4*)(SMQA_LDS char*)p);
}
// Concatenate two 4-element transposing reads into one 8-element MFMA operand. Built with a
// whole-vector shuffle and one bitcast: element-wise insertion of bit-cast halves has been
// observed to compile into lane-duplicating v_perm sequences.
__device__ __forceinline__ bf16x8 join_tr(s16x4 lo, s16x4 hi) {
  const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8, v);
}
// 16-byte global -> LDS copy without a register round trip (global_load_lds_dwordx4).
// lds_base must be the same for the whole wave; lane l lands at lds_base + 16*l.
__device__ __forceinline__ void dma16(const void* gsrc, char* lds_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (SMQA_LDS void*)(SMQA_LDS char*)lds_base, 16, 0, 0);
}
// Buffer resource over [base, base + bytes) for raw (unswizzled, stride 0) buffer loads. The
// record count is an unsigned 32-bit field: `bytes` carries its bit pattern, so a range must stay
// below 4 GiB (the library refuses kv tensors whose rows of one batch reach that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
// 16-byte global -> LDS copy through a buffer resource (buffer_load_dwordx4 ... lds): lane l reads
// rsrc + soff + voff and lands at lds_base + 16*l. Unlike the global_ form this is not a FLAT
// instruction, so the compiler keeps exact LDS wait counts for reads issued while it is in flight.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, char* lds_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SMQA_LDS void*)(SMQA_LDS char*)lds_base, 16, voff, soff, 0, 0);
}
// dma16_buf whose LDS destination the compiler cannot trace to an LDS variable. The compiler then
// adds no wait of its own before later LDS reads (it cannot tell which reads the copy feeds), so the
// caller must order every read of the destination after the copy itself: an explicit vmcnt wait for
// the copy, then a barrier for the other waves' copies. Used where several tiles are in flight.
__device__ __forceinline__ void dma16_buf_unordered(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                                    char* lds_base) {
  uint32_t a = (uint32_t)(uintptr_t)(SMQA_LDS char*)lds_base;
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (SMQA_LDS void*)(uintptr_t)a, 16, voff, soff, 0, 0);
}
// dma16 (global_load_lds_dwordx4) whose LDS destination the compiler cannot trace, with the same
// contract as dma16_buf_unordered: the caller orders every read of the destination after the copy.
__device__ __forceinline__ void dma16_unordered(const void* gsrc, char* lds_base) {
  uint32_t a = (uint32_t)(uintptr_t)(SMQA_LDS char*)lds_base;
  asm volatile("" : "+s"(a));
  __builtin_amdgcn_global_load_lds(gsrc, (SMQA_LDS void*)(uintptr_t)a, 16, 0, 0);
}
// A token's top-k indices staged in LDS in blocks of 32 slots, 32 blocks at a time, in a ring of 64
// blocks. Reading a block's indices from global memory inside a block loop puts one memory latency
// into every stage (each block's indices are a fresh cache line, and a stage that ends waiting for
// its gathers waits for that load too); from the ring the read is an LDS access. Four waves (256
// lanes, wave number w4 = 0..3) fetch blocks c .. c + 31 with four coalesced loads a lane (-1 past
// topk) and write them in once a wait of their own has covered the loads, so a fetch issued at the
// top of a stage lands at its end. The slots of blocks c .. c + 31 are those of blocks c - 64 ..
// c - 33, and, for a refill at c = blk + 32 issued in stage blk, of blocks blk - 32 .. blk - 1.
struct IdxRing {
  static constexpr int T = 32;
  static constexpr int SLOTS = 64 * T;
  int32_t* ring;         // SLOTS ints of LDS
  const int32_t* src;    // the token's topk indices
  int topk;
  __device__ __forceinline__ void fetch(int c, int w4, int lane, int32_t (&v)[4]) const {
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int t = c * T + 256 * k + 64 * w4 + lane;
      v[k] = t < topk ? src[t] : -1;
    }
  }
  __device__ __forceinline__ void store(int c, int w4, int lane, const int32_t (&v)[4]) const {
#pragma unroll
    for (int k = 0; k < 4; k++) ring[(c * T + 256 * k + 64 * w4 + lane) & (SLOTS - 1)] = v[k];
  }
  // block blk's index of this lane (lanes >= 32 and slots past topk: -1)
  __device__ __forceinline__ int32_t read(int blk, int lane) const {
    const int32_t v = ring[(blk * T + (lane & (T - 1))) & (SLOTS - 1)];
    return (lane < T && blk * T + lane < topk) ? v : -1;
  }
  // whether stage blk refills blocks blk + 32 .. blk + 63 (the first 64 blocks are fetched up front)
  __device__ __forceinline__ static bool refill_at(int blk, int nblk) {
    return blk >= 32 && (blk & 31) == 0 && blk + 32 < nblk;
  }
};
// Workgroup barrier that publishes this wave's LDS writes only. __syncthreads() also waits for
// every outstanding global access, including tile gathers still in flight for a later block; this
// waits for the LDS counter alone, and the empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left at their maxima
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// Wait for all outstanding memory operations of this wave (including LDS DMA).
__device__ __forceinline__ void wait_all_mem() { __builtin_amdgcn_s_waitcnt(0); }

// Pins a long-lived MFMA operand to the accumulator register file (an MFMA reads its A and B
// operands from there directly), leaving the vector registers to accumulators and in-flight
// fragments.
__device__ __forceinline__ void keep_in_agpr(bf16x8& v) { asm volatile("" : "+a"(v)); }
__device__ __forceinline__ void keep_in_agpr(f16x8& v) { asm volatile("" : "+a"(v)); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *(const uint4*)p);
}
__device__ __forceinline__ bf16x8 zero_bf16x8() { return __builtin_bit_cast(bf16x8, make_uint4(0, 0, 0, 0)); }

__device__ __forceinline__ bool slot_in_range(int32_t i, int64_t S_kv) {
  return i >= 0 && (int64_t)i < S_kv;
}

__device__ __forceinline__ uint2 pack4_bf16(float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  return __builtin_bit_cast(uint2, v);
}


// Maximum over the four lanes of a hardware quad (DPP quad permutations, no LDS traffic).
__device__ __forceinline__ float quad_max(float m) {
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0xB1, 0xF, 0xF, true)));
  m = fmaxf(m, __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, m), 0x4E, 0xF, 0xF, true)));
  return m;
}

// Compile-time integer tag, used to instantiate a loop body once per LDS buffer.
template <int V>
struct IntTag {
  static constexpr int value = V;
  __device__ constexpr operator int() const { return V; }
};

// f(IntTag<0>{}), ..., f(IntTag<N-1>{}): a loop unrolled by construction, for pipelines whose
// stages must see their index as a constant (the unroller may decline a large body).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IntTag<I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float wave_max_xor32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// 2^x with the hardware v_exp_f32 (no denormal-range fix-up): used for softmax weights, whose
// arguments are <= 8 here and whose tiny results only feed bf16 operands and fp32 sums.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace smqa

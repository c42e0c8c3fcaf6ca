// Device helpers shared by the gfx950 attention kernels: vector types, 16-byte
// memory access, bf16/fp16 packing and the MFMA shapes the kernels use.
//
// MFMA accumulator layouts relied on (CDNA3/CDNA4 matrix cores, wave64):
//   v_mfma_f32_32x32x16_{bf16,f16}: A row m = lane % 32, B column n = lane % 32,
//     each lane supplying 8 consecutive-k elements of its row/column; the 16
//     accumulators of lane l hold D[8*(i/4) + 4*(l/32) + i%4][l % 32], i = 0..15.
//   v_mfma_f32_16x16x32_{bf16,f16}: A row m = lane % 16, B column n = lane % 16;
//     the 4 accumulators of lane l hold D[4*(l/16) + i][l % 16], i = 0..3.
// A and B use the same (lane group, slot) -> k assignment, so any consistent
// relabelling of the contraction index between the two operands is exact.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

struct bf16_t {};  // tag types for the 16-bit input formats
struct f16_t {};

template <typename T> struct in_traits;
template <> struct in_traits<bf16_t> {
  typedef bf16x8 vec8;
  // Pack two fp32 into two bf16 (round to nearest even) in one dword.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  // c + the two 16-bit values packed in p (v_dot2c_f32_bf16 with (1, 1)).
  static __device__ __forceinline__ float sum2(uint32_t p, float c) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, p),
                                           bf16x2{(__bf16)1.0f, (__bf16)1.0f}, c, false);
  }
  static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <> struct in_traits<f16_t> {
  typedef f16x8 vec8;
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
  }
  static __device__ __forceinline__ float sum2(uint32_t p, float c) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, p),
                                  f16x2{(_Float16)1.0f, (_Float16)1.0f}, c, false);
  }
  static __device__ __forceinline__ f32x16 mma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 mma16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
};

// Output element stores. `n` consecutive fp32 values go to `dst` (n = 4).
struct out_bf16 {};
struct out_f16 {};
struct out_f32 {};

__device__ __forceinline__ void store4(out_f32, void* dst, float a, float b, float c, float d) {
  *(f32x4*)dst = f32x4{a, b, c, d};
}
__device__ __forceinline__ void store4(out_bf16, void* dst, float a, float b, float c, float d) {
  *(u32x2*)dst = u32x2{in_traits<bf16_t>::pack2(a, b), in_traits<bf16_t>::pack2(c, d)};
}
__device__ __forceinline__ void store4(out_f16, void* dst, float a, float b, float c, float d) {
  *(u32x2*)dst = u32x2{in_traits<f16_t>::pack2(a, b), in_traits<f16_t>::pack2(c, d)};
}
template <typename O> struct out_size;
template <> struct out_size<out_f32> { static constexpr int bytes = 4; };
template <> struct out_size<out_bf16> { static constexpr int bytes = 2; };
template <> struct out_size<out_f16> { static constexpr int bytes = 2; };

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *(const u32x4*)p; }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j passes the address
// of row r0 + j / 4, columns c0 + 4 * (j % 4) .. + 3 of a row-major 16-bit
// matrix in LDS and receives column c0 + j of rows r0 .. r0 + 3 (4 elements).
// It turns a row-major tile into MFMA operands that need consecutive rows per
// lane (the keys of the P V product).
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
  return __builtin_bit_cast(u32x2, r);
}

// Swap values between lane l and lane l ^ 32.
__device__ __forceinline__ float xor32(float v) { return __shfl_xor(v, 32, 64); }
__device__ __forceinline__ float xor16(float v) { return __shfl_xor(v, 16, 64); }

// Block index remap so that consecutive logical blocks share one XCD (the
// hardware hands workgroups to the 8 XCDs round-robin by dispatch order).
// Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int pid, int n) {
  const int x = pid & 7, s = pid >> 3;
  const int q = n >> 3, r = n & 7;
  return x < r ? x * (q + 1) + s : r * (q + 1) + (x - r) * q + s;
}

// LDS-race debug build (compiled with -DFA_LDS_DEBUG=1 into a library of its
// own): every LDS hand-off below also waits for all of the wave's
// vector-memory operations (global-to-LDS copies included), every partial
// vmcnt wait waits for all of them, and the loops over the workgroup-shared
// K/V stages end each step with a full barrier (debug_step_barrier). The
// arithmetic and its order are unchanged, so the debug library's results must
// equal the fast build's bit for bit; a difference means a stage was read
// before its copy landed or overwritten while another wave still read it.
#ifndef FA_LDS_DEBUG
#define FA_LDS_DEBUG 0
#endif

// Wave-local ordering of LDS accesses (all lanes' earlier LDS ops completed
// before later ones are issued; also a compiler barrier).
__device__ __forceinline__ void wave_lds_sync() {
#if FA_LDS_DEBUG
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
#else
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
}

// Workgroup barrier for LDS traffic only: this wave's LDS operations are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// outstanding global loads, so prefetches stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
#if FA_LDS_DEBUG
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
#else
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#endif
}

// End of one step of a loop over workgroup-shared LDS stages: a full barrier
// in the debug build, nothing otherwise. Only for places that every wave of
// the workgroup reaches equally often (beside an lds_barrier of the same loop).
__device__ __forceinline__ void debug_step_barrier() {
#if FA_LDS_DEBUG
  lds_barrier();
#endif
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (they retire in issue order).
template <int N> __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
#if FA_LDS_DEBUG
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#else
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
#endif
}

// LDS byte address (offset in the workgroup's LDS) of a __shared__ pointer.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// Direct global -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4)
// from a wave-uniform 64-bit base (SGPRs) plus a per-lane 32-bit byte offset:
// lane l's 16 bytes land at LDS address lds_base + 16 * l; lds_base is
// wave-uniform and goes through M0, which is restored afterwards. (The
// instruction's immediate offset is left at 0: it would move the LDS side too.)
// Issued from inline assembly so the compiler does not add a full vmcnt(0)
// wait before every later LDS read; callers wait with wait_vmcnt<N>(), which
// counts these copies like any vector load (they retire in issue order).
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(sbase), "s"(__builtin_amdgcn_readfirstlane(lds_base))
      : "memory");
}

__device__ __forceinline__ u32x4 lds16(const char* p) { return *(const u32x4*)p; }

// max / sum of a value over lanes l and l ^ 16 (v_permlane16_swap exchanges
// the odd and even 16-lane rows of its two operands; no LDS).
__device__ __forceinline__ float max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// max / sum of a value over lanes l and l ^ 32 (v_permlane32_swap, no LDS).
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Flip the sign of the 8 bf16/fp16 values of a fragment (a negative scale is
// applied as |scale| on -Q so the running max stays a max).
__device__ __forceinline__ u32x4 neg16x8(u32x4 v) {
  return v ^ u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
}

// LDS tile layout shared by the direct-to-LDS copies: a tile of 16-byte chunks
// (row r = key or token, chunk c) is cut into 8 x 8 blocks, one block per copy
// instruction (8 rows x 128 contiguous bytes of global memory). Inside block
// (RB = r >> 3, CB = c >> 3) the chunk sits at slot
//     8 * (g ^ (RB & 1)) + (rho ^ 4 * ((g >> 1) & 1)),   g = c & 7, rho = r & 7,
// which spreads both MFMA operand read patterns over all 64 banks: 16
// consecutive rows of one chunk (ds_read_b128 key reads), and 4 or 8 rows of
// 2 or 4 adjacent chunks (ds_read_b64_tr_b16 value reads).
__device__ __forceinline__ int blk_slot(int r, int c) {
  const int g = c & 7;
  return 8 * (g ^ ((r >> 3) & 1)) + ((r & 7) ^ (4 * ((g >> 1) & 1)));
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E - 1, each
// a separate instantiation, so indices into register arrays stay constants
// without relying on the loop unroller.
template <int B, int E, typename F> __device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Online-softmax rescale threshold in log2 units: the running max is moved
// only when a tile's max exceeds it by more than this, so probabilities stay
// <= 2^8 and the O rescale (a pass over all accumulators) is rare.
constexpr float RESCALE_LOG2 = 8.0f;

}  // namespace fa

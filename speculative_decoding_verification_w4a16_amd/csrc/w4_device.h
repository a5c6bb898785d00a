// Device helpers shared by the verify-linear kernels (w4a16_kernels.hip)
// and the verify-pass kernel (w4_pass.hip): vector types, the exact unpack
// of packed codes into bf16 operands, fp16/bf16 conversions, the bf16 dot,
// cache-policy loads and stores, and the LDS-only workgroup barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

namespace w4 {

// A wave-uniform value copied into a VGPR (once, at kernel start).  With the
// unpack mask in an SGPR and the magic value in a VGPR the compiler forms one
// v_and_or_b32 per bf16 pair; with both in SGPRs it needs an AND and an OR
// (a VALU op may read only one SGPR), and with literals it cannot fuse at all.
__device__ __forceinline__ uint32_t to_vgpr(uint32_t s) {
    uint32_t v;
    asm volatile("v_mov_b32 %0, %1" : "=v"(v) : "s"(s));
    return v;
}

// 8 packed codes -> 4 bf16 pairs (16 + q): dword d holds k offsets 2d, 2d+1.
// One v_alignbit_b32 (a rotate) and one v_and_or_b32 per pair, 7 VALU ops
// per word.  `mask` (0x00780078) and `magic` (0x41804180) arrive as kernel
// arguments so that the compiler keeps them in registers and forms one
// v_and_or_b32 per pair (with literal constants it emits a separate AND and
// OR).  Plain C, not inline asm, so the compiler's MFMA operand hazard checks
// see every write.
__device__ __forceinline__ u32x4 unpack_biased(uint32_t w, uint32_t mask, uint32_t magic) {
    u32x4 r;
    r[0] = (w & mask) | magic;
    r[1] = (__builtin_amdgcn_alignbit(w, w, 4) & mask) | magic;
    r[2] = (__builtin_amdgcn_alignbit(w, w, 8) & mask) | magic;
    r[3] = (__builtin_amdgcn_alignbit(w, w, 12) & mask) | magic;
    return r;
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// The bias of the unpacked operands (bf16 16 + q), and the unpack's mask and
// magic value (kernel arguments, see unpack_biased).
constexpr float kCodeBias = 16.0f;
constexpr uint32_t kNibbleMask = 0x00780078u;
constexpr uint32_t kBiasMagic = 0x41804180u;

// 16 + z for nibble j of a packed zero word, exact in fp32.
__device__ __forceinline__ float biased_zero(uint32_t zw, int j) {
    return (float)(16u + ((zw >> (4 * j)) & 15u));
}

// a . b + acc over one bf16 pair each, fp32 accumulation (v_dot2_f32_bf16).
// Arguments are plain dwords: hipcc miscompiles __builtin_bit_cast applied
// directly to an element of an ext_vector (it reads element 0), so vector
// elements are always copied into a scalar first.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), acc, false);
}

// fp32 -> bf16, round to nearest, ties to even (NaN stays a quiet NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x0040u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Workgroup barrier for an LDS producer/consumer hand-off.  It waits for this
// wave's LDS operations only: __syncthreads() also waits for every
// outstanding global load, which would drain the weight ring at each stage.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds + 16 l (the LDS line address travels in M0, wave-uniform).  Issued
// from inline asm so the compiler's wait-count pass does not see it; callers
// wait for it with an explicit s_waitcnt vmcnt.
__device__ __forceinline__ void lds_dma16(const void* src, void* lds) {
    const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_ptr_t)lds);
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(m) : "memory", "m0");
}

// Split-K partial sums travel through device memory with agent-scope (sc1)
// stores and loads, which are made visible at, and read from, the device
// coherence point directly.  No L2 write-back or invalidate is needed; those
// (what __threadfence() emits) serialise per XCD and cost far more than the
// kernel itself when every workgroup issues them.
__device__ __forceinline__ void store_partial(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Non-temporal loads for the streaming kernels (M <= 16).  Every packed
// weight, scale and zero byte is read once per call, while the activation
// rows are re-read by every wave from L2; marking the one-pass stream
// non-temporal keeps it from evicting them.  Measured on MI355X: 5-12 % off
// the M = 1 and M = 5 linears (lm_head at M = 1: 101 -> 89 us).  The LDS-ring
// kernel keeps ordinary loads (no gain there: its activations sit in LDS, and
// its row slices re-read a tile's weights from L2).
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
    const uint64_t v = __builtin_nontemporal_load((const uint64_t*)p);
    return make_uint2((uint32_t)v, (uint32_t)(v >> 32));
}
__device__ __forceinline__ uint32_t load_stream(const uint16_t* p) { return __builtin_nontemporal_load(p); }

__device__ __forceinline__ void decode_scales(uint2 sv, float (&sj)[4]) {
    sj[0] = f16_bits_to_f32(sv.x & 0xFFFFu);
    sj[1] = f16_bits_to_f32(sv.x >> 16);
    sj[2] = f16_bits_to_f32(sv.y & 0xFFFFu);
    sj[3] = f16_bits_to_f32(sv.y >> 16);
}


constexpr uint32_t kOnesBf16x2 = 0x3F803F80u;  // bf16 (1.0, 1.0)
}  // namespace w4

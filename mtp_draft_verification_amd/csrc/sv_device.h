// sv_device.h -- device-side helpers shared by the libspecverify kernels
// (CDNA4 / gfx950 only: 64-lane wavefronts, bf16 MFMA, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/specverify.h"

namespace sv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

// ---------------------------------------------------------------------------
// bf16 <-> fp32 (bit-level; round-to-nearest-even, NaN kept quiet)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
// round-to-nearest-even pack of two floats (one v_cvt_pk_bf16_f32 on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float round_bf16(float f) { return __uint_as_float(f32_to_bf16_bits(f) << 16); }

// 16-byte vector of 8 bf16 <-> the MFMA operand type
union V16 {
  uint4 u;
  uint32_t w[4];
  bf16x8_t b;
};

// ---------------------------------------------------------------------------
// MFMA: D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).
// Lane l supplies row (l % 16) of A and column (l % 16) of B, eight k-values each
// (lane group l / 16 selects which eight); the accumulator lane l holds column
// (l % 16), rows 4 * (l / 16) + {0,1,2,3}.  Any fixed assignment of k-values to
// (lane group, slot) gives the same product as long as A and B use the same one.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4_t mfma16x16x32(const bf16x8_t& a, const bf16x8_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ int shfl_xor_i(int v, int m) { return __shfl_xor(v, m, 64); }

// Max / sum over the four 16-lane rows of a wave (lanes l, l^16, l^32, l^48), with the
// gfx950 row-swap instructions (plain vector ALU ops, no trip through the LDS unit like
// a general shuffle).  v_permlane16_swap(x, x) leaves rows (0,0,2,2) in its first result
// and (1,1,3,3) in its second; v_permlane32_swap(y, y) leaves (0,1,0,1) and (2,3,2,3).
// The sum is (x0 + x1) + (x2 + x3) in every row, as the xor-16-then-32 shuffle gives.
__device__ __forceinline__ float row4_max(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float row4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float s = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(s), __float_as_uint(s), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// "a beats b" in the order (value descending, id ascending); id < 0 is an empty slot.
// Written with bitwise operators and selects below, so that lanes never diverge.
__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
  return (ai >= 0) & ((bi < 0) | (av > bv) | ((av == bv) & (ai < bi)));
}

// running best-two under `beats`
struct Top2 {
  float v1, v2;
  int i1, i2;
  __device__ __forceinline__ void init() { v1 = v2 = kNegInf; i1 = i2 = -1; }
  __device__ __forceinline__ void push(float v, int i) {
    const bool w1 = beats(v, i, v1, i1), w2 = beats(v, i, v2, i2);
    const float nv2 = w1 ? v1 : (w2 ? v : v2);
    const int ni2 = w1 ? i1 : (w2 ? i : i2);
    v1 = w1 ? v : v1;
    i1 = w1 ? i : i1;
    v2 = nv2;
    i2 = ni2;
  }
  // merge another running pair whose ids are disjoint from ours: if the other's best
  // wins, the second is the better of our best and the other's second; otherwise
  // the other's best may still displace our second
  __device__ __forceinline__ void merge(float ov1, int oi1, float ov2, int oi2) {
    const bool a = beats(ov1, oi1, v1, i1);
    const bool b = beats(v1, i1, ov2, oi2);
    const bool c = beats(ov1, oi1, v2, i2);
    const float nv2 = a ? (b ? v1 : ov2) : (c ? ov1 : v2);
    const int ni2 = a ? (b ? i1 : oi2) : (c ? oi1 : i2);
    v1 = a ? ov1 : v1;
    i1 = a ? oi1 : i1;
    v2 = nv2;
    i2 = ni2;
  }
  __device__ __forceinline__ void merge_xor(int m) {
    float ov1 = shfl_xor_f(v1, m), ov2 = shfl_xor_f(v2, m);
    int oi1 = shfl_xor_i(i1, m), oi2 = shfl_xor_i(i2, m);
    merge(ov1, oi1, ov2, oi2);
  }
};

// online log-sum-exp state in natural-log units: value = m + log(s)
struct LSE {
  float m, s;
  __device__ __forceinline__ void init() { m = kNegInf; s = 0.f; }
  __device__ __forceinline__ void merge(float om, float os) {
    if (om == kNegInf) return;
    if (m == kNegInf) { m = om; s = os; return; }
    float M = fmaxf(m, om);
    s = s * exp2f((m - M) * kLog2e) + os * exp2f((om - M) * kLog2e);
    m = M;
  }
  __device__ __forceinline__ void merge_xor(int k) {
    float om = shfl_xor_f(m, k), os = shfl_xor_f(s, k);
    merge(om, os);
  }
};

__device__ __forceinline__ void set_status(int32_t* st, int32_t bits) {
  if (st) atomicOr(st, bits);
}

// gelu, tanh form: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))
__device__ __forceinline__ float gelu_tanh(float x) {
  const float c = 0.7978845608028654f;
  return 0.5f * x * (1.f + tanhf(c * (x + 0.044715f * x * x * x)));
}

// Gumbel noise from a uniform in [0,1): -log(-log u); u == 0 gives -inf.
__device__ __forceinline__ float gumbel(float u) { return -logf(-logf(u)); }

// ---------------------------------------------------------------------------
// HBM -> LDS streaming (direct-to-LDS DMA) and LDS-only barriers
// ---------------------------------------------------------------------------
// 16 bytes per lane from global memory straight into LDS at (lds_base + 16 * lane),
// gaddr = base (wave-uniform) + off (per lane, bytes).  Issued from inline asm so the
// compiler, which cannot tell which ring stage a DMA writes, does not stall every LDS
// read on it; completion is waited for explicitly with wait_vm.  M0 (the LDS base)
// is saved and restored around the instruction.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const void*)p);
}
// ORDERED = false drops the memory clobber, so the compiler may move ordinary LDS
// reads and MFMAs across the DMA.  Only for a DMA into a ring stage that no code
// between the surrounding barriers reads: its ordering against the reads of that
// stage is carried by the barrier and wait statements (volatile asm, which keep
// their relative order, each with a memory clobber).
// NT sets the non-temporal hint: for data a call streams once (weights, KV tiles),
// which then is not allocated in the caches.  A ring streamed this way measured
// about 7.1 TB/s on MI355X against about 6.1 TB/s without the hint; data that other
// workgroups read again (activations) keeps the default policy.
template <bool ORDERED = true, bool NT = false>
__device__ __forceinline__ void dma16(const void* base_in, uint32_t off, uint32_t lds_base) {
  // the base is wave-uniform by construction; say so, so that it lives in SGPRs
  const uint64_t bu = (uint64_t)(uintptr_t)base_in;
  // (readfirstlane yields an int: widen each half as unsigned, never sign-extend)
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(bu >> 32));
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)bu);
  const uint64_t b64 = (hi << 32) | lo;
  const void* base = (const void*)(uintptr_t)b64;
  lds_base = __builtin_amdgcn_readfirstlane(lds_base);
  uint32_t saved;
  if constexpr (ORDERED && NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_base)
        : "memory");
  } else if constexpr (NT) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2 nt\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_base));
  } else if constexpr (ORDERED) {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_base)
        : "memory");
  } else {
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "global_load_lds_dwordx4 %1, %2\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(off), "s"(base), "s"(lds_base));
  }
}

// raw buffer descriptor word 3 for gfx950 (32-bit elements, no swizzle) and the
// sc1 cache policy: stores write through to, and loads read from, the device's
// coherence point, so workgroups on different XCDs (each with its own L2) can hand
// data to each other inside one kernel
constexpr int kBufferWord3 = 0x00020000;
constexpr int kCoherent = 16;

// wait until at most N of this wave's vector memory operations are outstanding
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait for all but `ahead` ring stages of NI operations each (ahead <= 6; callers
// guarantee ahead * NI <= 63, larger `ahead` waits for everything)
template <int NI>
__device__ __forceinline__ void wait_stages(int ahead) {
  switch (ahead) {
    case 0: wait_vm_n<0>(); break;
    case 1: wait_vm_n<(NI < 63 ? NI : 0)>(); break;
    case 2: wait_vm_n<(2 * NI < 63 ? 2 * NI : 0)>(); break;
    case 3: wait_vm_n<(3 * NI < 63 ? 3 * NI : 0)>(); break;
    case 4: wait_vm_n<(4 * NI < 63 ? 4 * NI : 0)>(); break;
    case 5: wait_vm_n<(5 * NI < 63 ? 5 * NI : 0)>(); break;
    case 6: wait_vm_n<(6 * NI < 63 ? 6 * NI : 0)>(); break;
    default: wait_vm_n<0>(); break;
  }
}

// Workgroup barrier for LDS traffic only: this wave's LDS writes have completed,
// but DMA into LDS still in flight is not waited for (each stage waits for its own
// DMA explicitly), which keeps the ring's prefetches going across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace sv

// Device helpers shared by the gfx950 kernels of the NF4 QLoRA library.
//
// Arithmetic rules kept everywhere (they make the results bit-reproducible
// against an independent implementation): one IEEE fp32 rounding per
// operation, no contraction into fused multiply-add (-ffp-contract=off plus
// the pragma below), correctly rounded fp32 division, fp32 denormals kept.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace qnf4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBlock = 64;     // NF4 absmax block (elements)
constexpr int kDqBlock = 256;  // constants per double-quantization group

// NF4 levels and the 15 decision thresholds, passed to kernels by value.
struct Codebook {
  float q[16];
  float t[15];  // largest fp32 <= midpoint of q[j], q[j+1]
};

// ---------------------------------------------------------------------------
// bf16
// ---------------------------------------------------------------------------

// Two fp32 values rounded to bf16 (nearest, ties to even) and packed; `lo`
// lands in bits 0..15.  Lowers to v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t p;
  p.x = (__bf16)lo;
  p.y = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, p);
}

// The same into IEEE binary16 (nearest, ties to even, subnormals kept):
// v_cvt_f16_f32 under the default rounding and denormal modes.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  f16x2_t p;
  p.x = (_Float16)lo;
  p.y = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, p);
}
// Two values rounded into the 16-bit compute format (F16: binary16, else bf16).
template <bool F16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (F16) {
    return pack_f16x2(lo, hi);
  } else {
    return pack_bf16x2(lo, hi);
  }
}
// A 16-bit compute-format value widened to fp32 (exact).
template <bool F16>
__device__ __forceinline__ float widen16(uint32_t v16) {
  if constexpr (F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)v16);
  } else {
    return __uint_as_float(v16 << 16);
  }
}

__device__ __forceinline__ float bf16lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) {
  return __uint_as_float((uint32_t)v << 16);
}

// ---------------------------------------------------------------------------
// OCP FP8 E4M3 (bias 7, 3 mantissa bits, max 448, subnormals to 2^-9)
// ---------------------------------------------------------------------------

__device__ __forceinline__ float e4m3_to_f32(uint32_t e) {
  const uint32_t sign = (e & 0x80u) << 24;
  const uint32_t ex = (e >> 3) & 15u;
  const uint32_t m = e & 7u;
  // normal: exponent ex - 7, mantissa m/8; subnormal (ex == 0): m * 2^-9
  const float normal = __uint_as_float(((ex + 120u) << 23) | (m << 20));
  const float sub = (float)m * 0x1p-9f;
  const float mag = ex ? normal : sub;
  return __uint_as_float(__float_as_uint(mag) | sign);
}

// Nearest E4M3 of a finite fp32 value, ties to the even mantissa, magnitudes
// >= 448 saturate to 448; the sign bit is the sign of y (-0 -> 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(y);
  uint32_t code;
  if (!(a < 448.0f)) {
    code = 0x7Eu;
  } else if (a < 0x1p-6f) {
    // subnormal grid of spacing 2^-9: a * 512 is exact, rintf rounds half-even
    code = (uint32_t)rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits with round-to-nearest-even on the fp32 pattern; a
    // carry moves into the exponent, which is the right result
    const uint32_t ua = u & 0x7fffffffu;
    const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return code | sign;
}

// c' = fl32(fl32(dec(e) * s) + mu): two roundings, no fused multiply-add.
__device__ __forceinline__ float decode_constant(uint32_t e, float s, float mu) {
  const float p = __fmul_rn(e4m3_to_f32(e), s);
  return __fadd_rn(p, mu);
}

// ---------------------------------------------------------------------------
// MFMA: D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16)
// Lane l supplies A row (l % 16) and B column (l % 16), 8 consecutive
// reduction elements each (the same reduction slots for A and B), and
// receives D rows 4*(l/16) + v, v = 0..3, of column l % 16.
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// The same layout for either 16-bit compute format (F16: v_mfma_f32_16x16x32_f16).
template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(const u32x4_t a, const u32x4_t b, f32x4_t c) {
  if constexpr (F16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  } else {
    return mfma_16x16x32(a, b, c);
  }
}

// ---------------------------------------------------------------------------
// Buffer loads: a scalar resource (base, size in bytes) plus a per-lane 32-bit
// byte offset and a scalar byte offset.  Reads at or past `bytes` return zero
// and never fault, which is how ragged tile edges are handled without
// per-lane branches.
// ---------------------------------------------------------------------------

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)b, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x2_t buf_load8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ uint32_t buf_load2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
}
__device__ __forceinline__ uint32_t buf_load1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

// Asynchronous copy of 16 bytes per lane from a buffer straight into LDS:
// lane i's bytes land at lds + 16*i (the whole wave fills 1 KB starting at the
// wave-uniform `lds`).  Reads past the resource's size deliver zeros.
__device__ __forceinline__ void buf_load_lds16(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           (int)voff, (int)soff, 0, 0);
}

// The same for 4 bytes per lane: lane i's dword lands at lds + 4*i.
__device__ __forceinline__ void buf_load_lds4(rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4,
                                           (int)voff, (int)soff, 0, 0);
}

// LDS as explicit 32-bit byte addresses: lets table lookups be formed as
// base | (code * 2) (two VALU ops) when the table base is 32-byte aligned.
typedef __attribute__((address_space(3))) uint16_t lds_u16_t;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)(p);
}
__device__ __forceinline__ uint16_t lds_read_u16(uint32_t a) {
  return *(const lds_u16_t*)(uintptr_t)a;
}
// v = hi + lo with hi = RNE_bf16(v) and lo = RNE_bf16(v - hi): the pair
// carries about 16 significant bits of an fp32 value into bf16 products.
__device__ __forceinline__ void split_hilo(float v, uint16_t& hi, uint16_t& lo) {
  const uint32_t h = pack_bf16x2(v, 0.0f) & 0xffffu;
  const float rem = __fsub_rn(v, __uint_as_float(h << 16));
  hi = (uint16_t)h;
  lo = (uint16_t)(pack_bf16x2(rem, 0.0f) & 0xffffu);
}
// The same split into the 16-bit compute format (binary16 pairs carry about
// 22 significant bits while the low part stays above the subnormal range).
template <bool F16>
__device__ __forceinline__ void split_hilo16(float v, uint16_t& hi, uint16_t& lo) {
  if constexpr (F16) {
    const uint32_t h = pack_f16x2(v, 0.0f) & 0xffffu;
    const float rem = __fsub_rn(v, widen16<true>(h));
    hi = (uint16_t)h;
    lo = (uint16_t)(pack_f16x2(rem, 0.0f) & 0xffffu);
  } else {
    split_hilo(v, hi, lo);
  }
}

// Returns x unchanged, but hides where it came from: values derived from it
// are computed where they are used instead of being hoisted out of a loop,
// where each would hold a register for the whole loop.
template <typename T>
__device__ __forceinline__ T opaque(T x) {
  asm volatile("" : "+v"(x));
  return x;
}
// 2 * (4-bit code at bit `pos` of w), as a byte offset into a bf16 table.
__device__ __forceinline__ uint32_t code_x2(uint32_t w, int pos) {
  return pos == 0 ? ((w << 1) & 0x1Eu) : ((w >> (pos - 1)) & 0x1Eu);
}

// Copies into LDS written as inline assembly.  The compiler does not see
// their LDS writes, so it inserts no waits of its own in front of LDS reads
// (with the builtins above it must assume any LDS read may alias a copy in
// flight and waits for all of them); the caller orders every read of copied
// data after wait_vmem()/wait_vmem_le<>() and, across waves, a barrier.
// The resource is passed as its four descriptor words (held in SGPRs).
typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4_t rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  const int64_t b = bytes < 0 ? 0 : (bytes > 0x7fffffffLL ? 0x7fffffffLL : bytes);
  i32x4_t r;
  r.x = __builtin_amdgcn_readfirstlane((int32_t)(uint32_t)a);
  r.y = __builtin_amdgcn_readfirstlane((int32_t)((a >> 32) & 0xffffu));  // stride 0
  r.z = __builtin_amdgcn_readfirstlane((int32_t)b);                       // bytes
  r.w = 0x00020000;                                                      // raw dwords
  return r;
}
// lane i's 16 bytes at (voff + soff) land at lds + 16*i (lds wave-uniform)
__device__ __forceinline__ void dma_lds16(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r), "s"(so)
               : "memory", "m0");
}
// lane i's dword at (voff + soff) lands at lds + 4*i
__device__ __forceinline__ void dma_lds4(i32x4_t r, const void* lds, uint32_t voff, uint32_t soff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_offset(lds));
  const uint32_t so = __builtin_amdgcn_readfirstlane(soff);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0), "v"(voff), "s"(r), "s"(so)
               : "memory", "m0");
}

// Waits until every vector-memory load issued by this wave has completed
// (including copies into LDS, which the compiler does not track).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// Waits until at most N vector-memory loads of this wave are outstanding
// (loads complete in issue order, so the older ones are done).  N < 64.
// Callers that read LDS filled by copies put a compiler barrier after it.
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

}  // namespace qnf4

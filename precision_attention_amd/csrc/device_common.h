// device_common.h -- gfx950 building blocks shared by the kernels of this library.
//
// Operand layouts of the block-scaled MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4), as
// measured on MI355X:
//  - A (32 x 64, row-major in M x K) and B (64 x 32, K x N): lane l supplies row/column
//    l % 32; its 256-bit operand register holds 32 K-elements. FP4: nibble j (dword j/8,
//    low nibble first) is K-element (l/32)*32 + j, and the 32 nibbles form one scale block
//    whose E8M0 scale is the lane's own scale byte. FP8: byte j; bytes 0-15 of lanes r and
//    r+32 form scale block 0 (scale from lane r), bytes 16-31 form block 1 (scale from lane
//    r+32). Elements of A and B pair up when they sit at the same byte/nibble index of
//    lanes in the same half.
//  - C/D (32 x 32 fp32): lane l, register i holds row 8*(i/4) + 4*(l/32) + i%4, column l%32.
// Converters: cvt_scalef32_pk_fp4_f32 rounds x/scale to nearest even E2M1 (saturating,
// sign kept); cvt_scalef32_pk_fp8_f32 rounds to nearest even E4M3 but does NOT saturate
// (|x| > 464 becomes the NaN code 0x7F or 0xFF by sign; 464 rounds to 448), so callers clamp
// first or, for non-negative inputs, saturate the packed codes (sat_e4m3_nonneg).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4attn {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef short v2s __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: do not keep it in the caches).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// MFMA element-format codes (cbsz / blgp fields).
constexpr int kFmtFP8 = 0;
constexpr int kFmtFP4 = 4;

// c = log2(e) / sqrt(D) rounded once to binary32.
__host__ __device__ constexpr float log2e_over_sqrt_d(int D) {
  return D == 128 ? 0x1.0527dcp-3f : 0x1.715476p-3f;  // 0x3E0293EE, 0x3E38AA3B
}
__host__ __device__ constexpr float inv_sqrt_d(int D) { return D == 128 ? 0x1.6a09e6p-4f : 0.125f; }

template <int FA, int FB, int OPSA, int OPSB>
__device__ __forceinline__ v16f mfma_scaled(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FA, FB, OPSA, sa, OPSB, sb);
}

// Exact binary32 helpers that the compiler may not contract or reassociate.
__device__ __forceinline__ float fsub_rn(float a, float b) { return __fsub_rn(a, b); }
__device__ __forceinline__ float fmul_rn(float a, float b) { return __fmul_rn(a, b); }

// Pack 8 floats (already divided by their block scale) into one dword of E2M1 codes,
// element 0 in the low nibble.
__device__ __forceinline__ uint32_t pack8_fp4(const float* x) {
  uint32_t w = __float_as_uint(x[0]);  // every byte is written: any initial value (no extra move)
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[0], x[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[2], x[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[4], x[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, x[6], x[7], 1.0f, 3);
  return w;
}

// Pack 4 floats into one dword of E4M3 codes (element 0 in the low byte). Inputs must
// already satisfy |x| <= 448, or be non-negative and go through sat_e4m3_nonneg.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  v2s w = __builtin_bit_cast(v2s, a);  // both halves are written: any initial value (no extra move)
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, 1.0f, true);
  uint32_t r;
  __builtin_memcpy(&r, &w, 4);
  return r;
}

// Saturation of four E4M3 codes of non-negative values converted without a clamp: the converter
// writes 0x7F (NaN) for an input that rounds above 448 (measured; 464 itself rounds to 448), and
// such a byte becomes 0x7E (448), the saturating result. Every byte is at most 0x7F, so adding 1
// to each byte carries into no other, bit 7 of a sum byte is set exactly for 0x7F, and flipping
// bit 0 of those bytes gives 0x7E.
__device__ __forceinline__ uint32_t sat_e4m3_nonneg(uint32_t w) {
  return w ^ (((w + 0x01010101u) >> 7) & 0x01010101u);
}

// Direct global -> LDS loads (global_load_lds): lane l of one instruction writes its
// `size` bytes at LDS address lds + size*l (measured on MI355X for 16 and 4 bytes; the
// 1-byte form writes one zero-extended dword per lane, at lds + 4*l). `lds` must be the same
// for all lanes of the wave. Completion is tracked by vmcnt: wait_dma() before the barrier
// that publishes the data.
typedef uint8_t lds_char;
typedef uint32_t lds_u32;
__device__ __forceinline__ void dma16(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 4, 0, 0);
}
__device__ __forceinline__ void dma1(const void* g, lds_char* l) {
  __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)g,
                                   (__attribute__((address_space(3))) void*)l, 1, 0, 0);
}
__device__ __forceinline__ void wait_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// The same loads issued as inline assembly, invisible to the compiler's wait-count insertion:
// it cannot always prove that a fragment read from one LDS buffer does not alias a DMA into
// another and would then wait for the DMA in flight. Users order every DMA before the reads of
// its data with wait_dma() and a workgroup barrier. M0 holds the (wave-uniform) LDS base, one
// wait state before the load; kernels using these keep nothing else in M0.
__device__ __forceinline__ uint32_t lds_addr(const lds_char* l) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) lds_char*)l;
}
// p as an SGPR pair (readfirstlane of both halves; p must be wave-uniform): the asm operands
// below are scalar registers, which the compiler could otherwise leave in VGPRs.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
// base: wave-uniform global address (SGPR pair); off: per-lane unsigned 32-bit byte offset;
// lds: wave-uniform LDS byte address of the 64-lane destination
__device__ __forceinline__ void dma16_async(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma4_async(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
__device__ __forceinline__ void dma1_async(const void* base, uint32_t off, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_ubyte %0, %1" ::"v"(off), "s"(uniform_ptr(base)),
               "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Swap the upper 32 lanes of a with the lower 32 lanes of b (v_permlane32_swap).
__device__ __forceinline__ void permlane32_swap(uint32_t& a, uint32_t& b) {
  auto r = __builtin_amdgcn_permlane32_swap(a, b, false, false);
  a = r[0];
  b = r[1];
}

// max over lanes l and l^32, result in both.
__device__ __forceinline__ float max_across_halves(float x) {
  uint32_t a = __float_as_uint(x), b = a;
  permlane32_swap(a, b);
  return __builtin_elementwise_maximum(__uint_as_float(a), __uint_as_float(b));
}

// bf16 bits of x rounded to nearest, ties to even (x finite).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Per-wave LDS tile of the output epilogue: 32 rows of D bf16 plus 8 bytes, so that the 32 rows
// that one 32-lane pass of 8-byte writes touches fall on distinct bank pairs.
template <int D>
struct OStage {
  static constexpr int kRow = 2 * D + 8;
  static constexpr int kBytes = 32 * kRow;
};

// Output epilogue of one wave that holds O^T for 32 queries q0 + (lane % 32) in the MFMA C
// layout (acc[t][4a + i] is d = 32t + 8a + 4*(lane / 32) + i): O = O^T * (1/l) rounded to bf16,
// LSE = m / sqrt(D) + ln(l). The rows pass through this wave's LDS tile `stage`
// (OStage<D>::kBytes) and leave as whole rows, 16 bytes per lane and D/8 lanes per row, so that
// every (non-temporal) store instruction writes 64*16 contiguous bytes of O. o and lse point at
// this (batch, head)'s [N, D] and [N] slices; rows q >= N are not written. Every wave of the
// workgroup calls it (it holds workgroup barriers), after the last read of whatever LDS `stage`
// overlaps. LOG2_ANCHOR: m is an integer log2 anchor and LSE = (m + log2 l) ln 2.
template <int D, bool LOG2_ANCHOR = false>
__device__ __forceinline__ void store_o_lse_rows(const v16f (&acc)[D / 32], float l, float m, uint16_t* o, float* lse,
                                                 int N, int q0, int lane, uint8_t* stage) {
#pragma clang fp contract(off)
  constexpr int RS = OStage<D>::kRow;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  const int half = lane >> 5, col = lane & 31;
  __syncthreads();  // every wave is past its last read of the K/V buffers that `stage` overlaps
  const float inv = 1.0f / l;
#pragma unroll
  for (int t = 0; t < D / 32; t++)
#pragma unroll
    for (int aa = 0; aa < 4; aa++) {
      uint2 w;
      w.x = bf16_rne(acc[t][4 * aa + 0] * inv) | (bf16_rne(acc[t][4 * aa + 1] * inv) << 16);
      w.y = bf16_rne(acc[t][4 * aa + 2] * inv) | (bf16_rne(acc[t][4 * aa + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(stage + col * RS + (t * 32 + 8 * aa + 4 * half) * 2) = w;
    }
  if (half == 0 && q0 + col < N) {
    if constexpr (LOG2_ANCHOR)
      lse[q0 + col] = (m + __builtin_amdgcn_logf(l)) * 0.69314718f;
    else
      lse[q0 + col] = m * inv_sqrt_d(D) + __builtin_amdgcn_logf(l) * 0.69314718f;  // not contracted
  }
  __syncthreads();  // the tile is complete before any lane reads it back
  const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; i++) {
    const int r = i * RPI + rr;
    const uint2 lo = *reinterpret_cast<const uint2*>(stage + r * RS + cc * 16);
    const uint2 hi = *reinterpret_cast<const uint2*>(stage + r * RS + cc * 16 + 8);
    if (q0 + r < N) {  // streaming store: O is not read again by this kernel
      u32x4 w;
      w[0] = lo.x; w[1] = lo.y; w[2] = hi.x; w[3] = hi.y;
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o + (int64_t)(q0 + r) * D + cc * 8));
    }
  }
}

}  // namespace fp4attn

// quant.hip -- MX quantizer: bf16 -> MXFP4 (E2M1) or MXFP8 (E4M3) with one E8M0 scale per
// 32 elements, along D (row-major output) or along the sequence (transposed output).
//
// Rule (OCP MX v1.0, the pages' "power-of-two block scales"; gist.science summary of
// "Hardware-Aware FP4 FlashAttention-4", Methodology 1 "Format Selection" and Methodology 2
// "Gradient Formats"): e = floor(log2 amax) - emax (emax 2 for E2M1, 8 for E4M3), clamped to
// [-127, 127]; element = RNE(x / 2^e) on the element grid, saturating, sign kept.
//
// x / 2^e is built exactly from the bfloat16 bits by exponent arithmetic (so the result does
// not depend on the denormal mode); the rounding is done by the hardware converters, whose
// round-to-nearest-even behaviour matches the rule for every finite input (E4M3 inputs are
// clamped to +-448 first because that converter does not saturate).
//
// Both kernels are HBM-streaming: each bf16 element is read once and its code written once.
#include "device_common.h"
#include "kernels.h"

namespace fp4attn {

// Block exponent from the largest |x| given as 15-bit bf16 magnitude bits.
template <int EMAX>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 7) - 127 - EMAX;
  return e < -127 ? -127 : e;
}

// y = x / 2^e as binary32, exactly, from bf16 bits h. |y| < 2^(emax+1) by construction of e;
// values that would be binary32-subnormal are returned as signed zero (they round to zero
// in both element formats).
__device__ __forceinline__ float scaled_bf16(uint32_t h, int e) {
  const uint32_t sign = (h & 0x8000u) << 16;
  const int E = (int)((h >> 7) & 0xFFu);
  const uint32_t M = h & 0x7Fu;
  uint32_t mag = 0;
  if (E != 0) {
    const int ye = E - e;
    if (ye >= 1) mag = ((uint32_t)ye << 23) | (M << 16);
  } else if (M != 0) {
    const uint32_t b = __float_as_uint((float)M);  // exact; value M * 2^-133 before scaling
    const int ye = (int)(b >> 23) - 133 - e;
    if (ye >= 1) mag = ((uint32_t)ye << 23) | (b & 0x7FFFFFu);
  }
  return __uint_as_float(sign | mag);
}

__device__ __forceinline__ float clamp448(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }

// ---------------------------------------------------------------- along D
// A lane converts 8 consecutive elements (one 16-byte unit); 4 consecutive lanes share a
// 32-element block and exchange their partial |max| with two xor shuffles. Each lane handles
// kUnits units spaced one workgroup apart, loading all of them before converting any, so
// enough loads are in flight to cover the memory latency.
constexpr int kUnits = 4;

template <int FMT>
__device__ __forceinline__ void quant_unit_d(const uint4 v, uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                             int64_t u) {
  constexpr int EMAX = (FMT == kMXFP4) ? 2 : 8;
  uint32_t h[8] = {v.x & 0xFFFFu, v.x >> 16, v.y & 0xFFFFu, v.y >> 16,
                   v.z & 0xFFFFu, v.z >> 16, v.w & 0xFFFFu, v.w >> 16};
  uint32_t amax = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) amax = max(amax, h[i] & 0x7FFFu);
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 1));
  amax = max(amax, (uint32_t)__shfl_xor((int)amax, 2));
  const int e = block_exponent<EMAX>(amax);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; i++) y[i] = scaled_bf16(h[i], e);
  if constexpr (FMT == kMXFP4) {
    reinterpret_cast<uint32_t*>(codes)[u] = pack8_fp4(y);
  } else {
    uint2 w;
    w.x = pack4_fp8(clamp448(y[0]), clamp448(y[1]), clamp448(y[2]), clamp448(y[3]));
    w.y = pack4_fp8(clamp448(y[4]), clamp448(y[5]), clamp448(y[6]), clamp448(y[7]));
    reinterpret_cast<uint2*>(codes)[u] = w;
  }
  if ((u & 3) == 0) scales[u >> 2] = (uint8_t)(e + 127);
}

template <int FMT>
__global__ void __launch_bounds__(256) quant_along_d_kernel(const uint16_t* __restrict__ x,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales, int64_t nunits) {
  const int64_t span = (int64_t)256 * kUnits;
  for (int64_t u0 = (int64_t)blockIdx.x * span + threadIdx.x; u0 < nunits; u0 += (int64_t)gridDim.x * span) {
    // nunits is a multiple of 4 and the 4 lanes of a block are consecutive, so a block's lanes
    // are all in range or all out of range: the shuffles never mix the two
    uint4 v[kUnits];
#pragma unroll
    for (int k = 0; k < kUnits; k++) {
      const int64_t u = u0 + (int64_t)k * 256;
      v[k] = u < nunits ? load_stream16(reinterpret_cast<const uint4*>(x) + u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kUnits; k++) {
      const int64_t u = u0 + (int64_t)k * 256;
      if (u < nunits) quant_unit_d<FMT>(v[k], codes, scales, u);
    }
  }
}

// ---------------------------------------------------------------- along the sequence
// A workgroup stages a tile of 128 keys x D bf16 in LDS (coalesced 16-byte loads), then each
// lane takes one pair of columns (d, d+1) of one 32-key block, reads them down the tile, and
// writes the block's codes contiguously into the transposed output rows d and d+1.
template <int FMT, int D>
__global__ void __launch_bounds__(256) quant_along_seq_kernel(const uint16_t* __restrict__ x,
                                                              uint8_t* __restrict__ codes,
                                                              uint8_t* __restrict__ scales, int N) {
  constexpr int TK = 128;
  constexpr int RS = D / 2 + 1;  // LDS row stride in dwords (odd: column reads stay conflict-free)
  constexpr int EMAX = (FMT == kMXFP4) ? 2 : 8;
  constexpr int BITS = (FMT == kMXFP4) ? 4 : 8;
  __shared__ uint32_t tile[TK * RS];
  const int64_t bh = blockIdx.y;
  const int k0 = blockIdx.x * TK;
  const int nk = min(TK, N - k0);  // a multiple of 32
  const uint16_t* xb = x + ((int64_t)bh * N + k0) * D;
  constexpr int CH = D / 8;
  constexpr int PER = TK * CH / 256;  // 16-byte chunks per lane on a full tile
  if (nk == TK) {
    uint4 v[PER];  // all loads in flight before the first LDS store
#pragma unroll
    for (int r = 0; r < PER; r++) {
      const int t = threadIdx.x + r * 256;
      v[r] = load_stream16(reinterpret_cast<const uint4*>(xb + (int64_t)(t / CH) * D) + t % CH);
    }
#pragma unroll
    for (int r = 0; r < PER; r++) {
      const int t = threadIdx.x + r * 256;
      uint32_t* dst = tile + (t / CH) * RS + (t % CH) * 4;
      dst[0] = v[r].x;
      dst[1] = v[r].y;
      dst[2] = v[r].z;
      dst[3] = v[r].w;
    }
  } else {
    for (int t = threadIdx.x; t < nk * CH; t += 256) {
      const int key = t / CH, c = t % CH;
      const uint4 v = load_stream16(reinterpret_cast<const uint4*>(xb + (int64_t)key * D) + c);
      uint32_t* dst = tile + key * RS + c * 4;
      dst[0] = v.x;
      dst[1] = v.y;
      dst[2] = v.z;
      dst[3] = v.w;
    }
  }
  __syncthreads();
  constexpr int NP = D / 2;  // column pairs
  const int64_t row_bytes = (int64_t)N * BITS / 8;
  for (int t = threadIdx.x; t < NP * (TK / 32); t += 256) {
    const int p = t % NP, kb = t / NP;
    if (kb * 32 >= nk) continue;
    uint32_t amax_lo = 0, amax_hi = 0;
    uint32_t w[32];
#pragma unroll
    for (int i = 0; i < 32; i++) {
      w[i] = tile[(kb * 32 + i) * RS + p];
      amax_lo = max(amax_lo, w[i] & 0x7FFFu);
      amax_hi = max(amax_hi, (w[i] >> 16) & 0x7FFFu);
    }
    const int e_lo = block_exponent<EMAX>(amax_lo), e_hi = block_exponent<EMAX>(amax_hi);
    const int64_t d_lo = (int64_t)bh * D + 2 * p;
    uint8_t* out_lo = codes + d_lo * row_bytes + (int64_t)(k0 + kb * 32) * BITS / 8;
    uint8_t* out_hi = out_lo + row_bytes;
    if constexpr (FMT == kMXFP4) {
      uint32_t lo[4], hi[4];
#pragma unroll
      for (int q = 0; q < 4; q++) {
        float a[8], b[8];
#pragma unroll
        for (int j = 0; j < 8; j++) {
          a[j] = scaled_bf16(w[8 * q + j] & 0xFFFFu, e_lo);
          b[j] = scaled_bf16(w[8 * q + j] >> 16, e_hi);
        }
        lo[q] = pack8_fp4(a);
        hi[q] = pack8_fp4(b);
      }
      *reinterpret_cast<uint4*>(out_lo) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      *reinterpret_cast<uint4*>(out_hi) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    } else {
      uint32_t lo[8], hi[8];
#pragma unroll
      for (int q = 0; q < 8; q++) {
        float a[4], b[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          a[j] = clamp448(scaled_bf16(w[4 * q + j] & 0xFFFFu, e_lo));
          b[j] = clamp448(scaled_bf16(w[4 * q + j] >> 16, e_hi));
        }
        lo[q] = pack4_fp8(a[0], a[1], a[2], a[3]);
        hi[q] = pack4_fp8(b[0], b[1], b[2], b[3]);
      }
      uint4* ol = reinterpret_cast<uint4*>(out_lo);
      uint4* oh = reinterpret_cast<uint4*>(out_hi);
      ol[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
      ol[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
      oh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
      oh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
    }
    const int64_t srow = (int64_t)N / 32;
    scales[d_lo * srow + k0 / 32 + kb] = (uint8_t)(e_lo + 127);
    scales[(d_lo + 1) * srow + k0 / 32 + kb] = (uint8_t)(e_hi + 127);
  }
}

// ---------------------------------------------------------------- launchers
hipError_t launch_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, int fmt, int axis, int64_t BH,
                           int N, int D, hipStream_t stream) {
  if (axis == kAlongD) {
    const int64_t nunits = BH * N * D / 8;
    int64_t blocks = (nunits + 256 * kUnits - 1) / (256 * kUnits);
    const int64_t cap = 256 * 8;  // enough resident waves to saturate HBM; grid-stride beyond
    if (blocks > cap) blocks = cap;
    if (fmt == kMXFP4)
      quant_along_d_kernel<kMXFP4><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(x, codes, scales, nunits);
    else
      quant_along_d_kernel<kMXFP8><<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(x, codes, scales, nunits);
  } else {
    const dim3 grid((unsigned)((N + 127) / 128), (unsigned)BH);
    if (D == 128) {
      if (fmt == kMXFP4) quant_along_seq_kernel<kMXFP4, 128><<<grid, dim3(256), 0, stream>>>(x, codes, scales, N);
      else quant_along_seq_kernel<kMXFP8, 128><<<grid, dim3(256), 0, stream>>>(x, codes, scales, N);
    } else {
      if (fmt == kMXFP4) quant_along_seq_kernel<kMXFP4, 64><<<grid, dim3(256), 0, stream>>>(x, codes, scales, N);
      else quant_along_seq_kernel<kMXFP8, 64><<<grid, dim3(256), 0, stream>>>(x, codes, scales, N);
    }
  }
  return hipGetLastError();
}

}  // namespace fp4attn

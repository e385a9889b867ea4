// quant.hip -- MX quantizer: bf16 -> MXFP4 (E2M1) or MXFP8 (E4M3) with one E8M0 scale per
// 32 elements, along D (row-major output) or along the sequence (transposed output).
//
// Rule (OCP MX v1.0, the pages' "power-of-two block scales"; gist.science summary of
// "Hardware-Aware FP4 FlashAttention-4", Methodology 1 "Format Selection" and Methodology 2
// "Gradient Formats"): e = floor(log2 amax) - emax (emax 2 for E2M1, 8 for E4M3), clamped to
// [-127, 127]; element = RNE(x / 2^e) on the element grid, saturating, sign kept.
//
// The block exponent comes from the bf16 magnitude bits (integer max over the block). The
// division by 2^e and the rounding are one hardware conversion: the scale operand of
// v_cvt_scalef32_pk_{fp4,fp8}_f32 divides by 2^(its exponent field - 127) exactly, field 0
// meaning 2^-127, subnormal inputs included, then rounds to nearest even. E4M3 inputs are
// clamped to +-448 * 2^e first because that converter does not saturate; E2M1 saturates.
//
// One launch runs up to kMaxQuantJobs tensors (the forward's Q, K and V together): each
// workgroup finds its job from the jobs' first-workgroup indices. Every bf16 element is read
// once and every code written once, in two work shapes:
//  - along D: HBM-streaming and LDS-free. As an option it also reads a second bf16 tensor y of
//    the same shape and writes, per row i, -sum_d x_id y_id (fp32) and -fp32(lse_i log2 e): the
//    backward's -Delta and -LSE log2 e, formed while dO is quantized.
//  - along the sequence: a workgroup stages one 256-key tile of codes and scales in dynamic
//    LDS (up to about 35 KB) and stores whole transposed row spans.
#include "device_common.h"
#include "kernels.h"

namespace fp4attn {
namespace {

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// largest 15-bit magnitude among the two bf16 halves of each word, per half
__device__ __forceinline__ uint32_t pk_absmax(uint32_t a, uint32_t b) {
  u16x2 x, y;
  const uint32_t ma = a & 0x7FFF7FFFu, mb = b & 0x7FFF7FFFu;
  __builtin_memcpy(&x, &ma, 4);
  __builtin_memcpy(&y, &mb, 4);
  const u16x2 m = __builtin_elementwise_max(x, y);
  uint32_t r;
  __builtin_memcpy(&r, &m, 4);
  return r;
}
__device__ __forceinline__ uint32_t pk_max(uint32_t a, uint32_t b) {
  u16x2 x, y;
  __builtin_memcpy(&x, &a, 4);
  __builtin_memcpy(&y, &b, 4);
  const u16x2 m = __builtin_elementwise_max(x, y);
  uint32_t r;
  __builtin_memcpy(&r, &m, 4);
  return r;
}

// Block exponent from the largest |x| given as 15-bit bf16 magnitude bits: floor(log2) is the
// biased exponent field minus 127 (a subnormal or zero maximum lands below -127 and clamps).
template <int EMAX>
__device__ __forceinline__ int block_exponent(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 7) - 127 - EMAX;
  return e < -127 ? -127 : e;
}
// the converter scale operand for 2^e (exponent field e + 127; 0 stands for 2^-127)
__device__ __forceinline__ float cvt_scale(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
// 448 * 2^e, the largest input that stays finite in E4M3 after the division by 2^e
__device__ __forceinline__ float e4m3_bound(int e) { return __uint_as_float(((uint32_t)(e + 135) << 23) | 0x600000u); }

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// E2M1 codes of the 8 bf16 values in 4 words (element 0 in the low nibble), scaled by 2^-e
__device__ __forceinline__ uint32_t fp4_of_words(const uint32_t* w, float sc) {
  uint32_t r = 0;
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w[0]), bf16_hi(w[0]), sc, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w[1]), bf16_hi(w[1]), sc, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w[2]), bf16_hi(w[2]), sc, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, bf16_lo(w[3]), bf16_hi(w[3]), sc, 3);
  return r;
}
// E4M3 codes of 4 values (element 0 in the low byte), clamped to +-bound, scaled by 2^-e
__device__ __forceinline__ uint32_t fp8_of4(float a, float b, float c, float d, float bound, float sc) {
  v2s r = {0, 0};
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(a, -bound, bound),
                                               __builtin_amdgcn_fmed3f(b, -bound, bound), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(c, -bound, bound),
                                               __builtin_amdgcn_fmed3f(d, -bound, bound), sc, true);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}

// max over the 4 lanes of a quad (DPP quad permutations xor 1 and xor 2)
__device__ __forceinline__ uint32_t quad_max(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return x;
}

constexpr int kThreadsQ = 256;

// ---------------------------------------------------------------- along D
// A lane converts 8 consecutive elements (one 16-byte unit); the 4 lanes of a quad share a
// 32-element block. A workgroup takes kUnitsD consecutive groups of 256 units, all loads
// issued before the first conversion.
//
// With a second tensor y (the backward's O beside dO), the job also forms each row's
// -sum_d x_id y_id: a lane multiplies its unit with y's, the D/8 lanes of a row (consecutive
// lanes, a row never straddles two waves) sum by xor shuffles, and the row's first lane writes
// the sum and -fp32(LSE log2 e). x is then read once for its codes and the row sums together.
constexpr int kUnitsD = 8;
constexpr int kUnitsPerBlockD = kThreadsQ * kUnitsD;

// sum of the 8 products of two units of bf16 pairs, in a fixed order, without contraction
__device__ __forceinline__ float unit_dot(const uint4& a, const uint4& b) {
#pragma clang fp contract(off)
  const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
  float s = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    s += bf16_lo(aw[i]) * bf16_lo(bw[i]);
    s += bf16_hi(aw[i]) * bf16_hi(bw[i]);
  }
  return s;
}

template <int FMT, int D, bool DOT>
__device__ __forceinline__ void along_d(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                        uint8_t* __restrict__ scales, int64_t nunits, int64_t blk,
                                        const uint16_t* __restrict__ y, const float* __restrict__ lse,
                                        float* __restrict__ ndot, float* __restrict__ nl) {
  constexpr int EMAX = (FMT == kMXFP4) ? 2 : 8;
  constexpr int TPR = D / 8;  // units per row
  const int64_t u0 = blk * kUnitsPerBlockD + threadIdx.x;
  // nunits is a multiple of 4 and quads are 4 consecutive units: a quad is wholly in range or
  // wholly out of it, so the quad maximum never mixes the two (rows likewise, TPR units each)
  uint4 v[kUnitsD];
#pragma unroll
  for (int k = 0; k < kUnitsD; k++) {
    const int64_t u = u0 + (int64_t)k * kThreadsQ;
    v[k] = u < nunits ? load_stream16(reinterpret_cast<const uint4*>(x) + u) : make_uint4(0, 0, 0, 0);
  }
  if (DOT && y != nullptr) {  // uniform over the workgroup
    uint4 yv[kUnitsD];
#pragma unroll
    for (int k = 0; k < kUnitsD; k++) {
      const int64_t u = u0 + (int64_t)k * kThreadsQ;
      yv[k] = u < nunits ? load_stream16(reinterpret_cast<const uint4*>(y) + u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int k = 0; k < kUnitsD; k++) {
      const int64_t u = u0 + (int64_t)k * kThreadsQ;
      float s = unit_dot(yv[k], v[k]);
#pragma unroll
      for (int m = TPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m);
      if (u < nunits && (u % TPR) == 0) {
        const int64_t row = u / TPR;
        ndot[row] = -s;
        nl[row] = -fmul_rn(lse[row], 1.44269504f);
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kUnitsD; k++) {
    const int64_t u = u0 + (int64_t)k * kThreadsQ;
    const uint32_t w[4] = {v[k].x, v[k].y, v[k].z, v[k].w};
    const uint32_t m2 = pk_max(pk_absmax(w[0], w[1]), pk_absmax(w[2], w[3]));
    const uint32_t amax = quad_max(max(m2 & 0xFFFFu, m2 >> 16));
    const int e = block_exponent<EMAX>(amax);
    const float sc = cvt_scale(e);
    if (u < nunits) {
      if constexpr (FMT == kMXFP4) {
        reinterpret_cast<uint32_t*>(codes)[u] = fp4_of_words(w, sc);
      } else {
        const float bound = e4m3_bound(e);
        uint2 o;
        o.x = fp8_of4(bf16_lo(w[0]), bf16_hi(w[0]), bf16_lo(w[1]), bf16_hi(w[1]), bound, sc);
        o.y = fp8_of4(bf16_lo(w[2]), bf16_hi(w[2]), bf16_lo(w[3]), bf16_hi(w[3]), bound, sc);
        reinterpret_cast<uint2*>(codes)[u] = o;
      }
      if ((u & 3) == 0) scales[u >> 2] = (uint8_t)(e + 127);
    }
  }
}

// ---------------------------------------------------------------- along the sequence
// A workgroup takes one tile of kKbSeq<D> consecutive 32-key blocks of one (batch, head): 256
// keys at D = 128, 512 at D = 64 (the tile's last blocks may lie past N, then they are skipped).
// A lane takes one column pair (d, d+1) of a key block: it reads the pair's dword from each of
// the block's 32 rows (a wave's lanes cover whole rows, so every row read is coalesced) for two
// key blocks, loading both before converting either. The codes and scales go to an LDS tile
// laid out like the transposed output; after a barrier the workgroup copies each output row's
// span of the tile to global memory in 16-byte pieces, so every global store is contiguous
// along the row (a lane's own codes alone would make 16-byte fragments, one row per lane).
template <int D>
constexpr int kKbSeq = 8 * (128 / D);
// bytes of one output row's span in a tile, and the LDS row stride (padded by 16 bytes)
template <int FMT, int D>
constexpr int kSeqRowBytes = kKbSeq<D> * 32 * ((FMT == kMXFP4) ? 4 : 8) / 8;
template <int FMT, int D>
constexpr int kSeqLdsBytes = D * (kSeqRowBytes<FMT, D> + 16) + D * kKbSeq<D>;

template <int FMT, int D>
__device__ __forceinline__ void seq_convert(const uint32_t* w, uint8_t* __restrict__ ctile, uint8_t* __restrict__ stile,
                                            int l, int p) {
  constexpr int EMAX = (FMT == kMXFP4) ? 2 : 8;
  constexpr int RS = kSeqRowBytes<FMT, D> + 16;
  uint32_t m = pk_absmax(w[0], w[1]);
#pragma unroll
  for (int i = 2; i < 32; i += 2) m = pk_max(m, pk_absmax(w[i], w[i + 1]));
  const int e_lo = block_exponent<EMAX>(m & 0xFFFFu), e_hi = block_exponent<EMAX>(m >> 16);
  const float s_lo = cvt_scale(e_lo), s_hi = cvt_scale(e_hi);
  uint8_t* out_lo = ctile + (2 * p) * RS;
  uint8_t* out_hi = out_lo + RS;
  if constexpr (FMT == kMXFP4) {
    uint32_t lo[4], hi[4];
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const uint32_t* ww = w + 8 * q;
      uint32_t a = 0, b = 0;
      a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, bf16_lo(ww[0]), bf16_lo(ww[1]), s_lo, 0);
      a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, bf16_lo(ww[2]), bf16_lo(ww[3]), s_lo, 1);
      a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, bf16_lo(ww[4]), bf16_lo(ww[5]), s_lo, 2);
      a = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(a, bf16_lo(ww[6]), bf16_lo(ww[7]), s_lo, 3);
      b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, bf16_hi(ww[0]), bf16_hi(ww[1]), s_hi, 0);
      b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, bf16_hi(ww[2]), bf16_hi(ww[3]), s_hi, 1);
      b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, bf16_hi(ww[4]), bf16_hi(ww[5]), s_hi, 2);
      b = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(b, bf16_hi(ww[6]), bf16_hi(ww[7]), s_hi, 3);
      lo[q] = a;
      hi[q] = b;
    }
    *reinterpret_cast<uint4*>(out_lo + l * 16) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    *reinterpret_cast<uint4*>(out_hi + l * 16) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  } else {
    const float b_lo = e4m3_bound(e_lo), b_hi = e4m3_bound(e_hi);
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int q = 0; q < 8; q++) {
      const uint32_t* ww = w + 4 * q;
      lo[q] = fp8_of4(bf16_lo(ww[0]), bf16_lo(ww[1]), bf16_lo(ww[2]), bf16_lo(ww[3]), b_lo, s_lo);
      hi[q] = fp8_of4(bf16_hi(ww[0]), bf16_hi(ww[1]), bf16_hi(ww[2]), bf16_hi(ww[3]), b_hi, s_hi);
    }
    uint4* ol = reinterpret_cast<uint4*>(out_lo + l * 32);
    uint4* oh = reinterpret_cast<uint4*>(out_hi + l * 32);
    ol[0] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    ol[1] = make_uint4(lo[4], lo[5], lo[6], lo[7]);
    oh[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
    oh[1] = make_uint4(hi[4], hi[5], hi[6], hi[7]);
  }
  stile[(2 * p) * kKbSeq<D> + l] = (uint8_t)(e_lo + 127);
  stile[(2 * p + 1) * kKbSeq<D> + l] = (uint8_t)(e_hi + 127);
}

template <int FMT, int D>
__device__ __forceinline__ void along_seq(const uint16_t* __restrict__ x, uint8_t* __restrict__ codes,
                                          uint8_t* __restrict__ scales, int N, int64_t blk, uint8_t* smem) {
  constexpr int PAIRS = D / 2;
  constexpr int KB = kKbSeq<D>;
  constexpr int BITS = (FMT == kMXFP4) ? 4 : 8;
  constexpr int RB = kSeqRowBytes<FMT, D>, RS = RB + 16, CPR = RB / 16;
  uint8_t* ctile = smem;
  uint8_t* stile = smem + D * RS;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int p = lane % PAIRS;
  const int nb = N / 32, tpb = (nb + KB - 1) / KB;
  const int64_t bh = blk / tpb;
  const int kb0 = (int)(blk % tpb) * KB;
  const int nvalid = min(KB, nb - kb0);
  // the lane's two key blocks within the tile, 128/D apart
  const int lA = wave * 2 * (128 / D) + lane / PAIRS, lB = lA + (128 / D);
  const bool okA = lA < nvalid, okB = lB < nvalid;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(x + (bh * N + (int64_t)kb0 * 32) * D) + p;
  uint32_t w[2][32];
  if (okA) {
#pragma unroll
    for (int i = 0; i < 32; i++) w[0][i] = __builtin_nontemporal_load(src + (lA * 32 + i) * PAIRS);
  }
  if (okB) {
#pragma unroll
    for (int i = 0; i < 32; i++) w[1][i] = __builtin_nontemporal_load(src + (lB * 32 + i) * PAIRS);
  }
  if (okA) seq_convert<FMT, D>(w[0], ctile, stile, lA, p);
  if (okB) seq_convert<FMT, D>(w[1], ctile, stile, lB, p);
  __syncthreads();
  // codes: D rows of RB bytes, the first nvalid blocks' worth of each row is in range
  const int64_t row_bytes = (int64_t)N * BITS / 8;
  const int vbytes = nvalid * 32 * BITS / 8;
  uint8_t* gcodes = codes + bh * D * row_bytes + (int64_t)kb0 * 32 * BITS / 8;
#pragma unroll
  for (int i = 0; i < D * CPR / kThreadsQ; i++) {
    const int c = i * kThreadsQ + (int)threadIdx.x;
    const int r = c / CPR, col = (c % CPR) * 16;
    if (col < vbytes) {
      const uint4 v = *reinterpret_cast<const uint4*>(ctile + r * RS + col);
      __builtin_nontemporal_store(u32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<u32x4*>(gcodes + r * row_bytes + col));
    }
  }
  // scales: D rows of KB bytes; one row per thread, whole when the tile is full and aligned
  if ((int)threadIdx.x < D) {
    const int r = threadIdx.x;
    const uint8_t* s = stile + r * KB;
    uint8_t* g = scales + (bh * D + r) * nb + kb0;
    if (nvalid == KB && ((uintptr_t)g % KB) == 0) {
      if constexpr (KB == 8) *reinterpret_cast<uint2*>(g) = *reinterpret_cast<const uint2*>(s);
      else *reinterpret_cast<uint4*>(g) = *reinterpret_cast<const uint4*>(s);
    } else {
      for (int k = 0; k < nvalid; k++) g[k] = s[k];
    }
  }
}

struct QuantJob {
  const uint16_t* x;
  uint8_t* codes;
  uint8_t* scales;
  const uint16_t* y;  // optional row dot products (along D): see along_d
  const float* lse;
  float* ndot;
  float* nl;
  int64_t work;  // along D: 16-byte units; along the sequence: unused (tiles from rows and N)
  int fmt, axis;
  int block0;    // first workgroup of this job
};
struct QuantBatch {
  QuantJob job[kMaxQuantJobs];
  int njobs;
  int N;
};

// DOT: some job has row dot products (a separate instance, as their loads take 32 more VGPRs)
template <int D, bool DOT>
__global__ void __launch_bounds__(kThreadsQ) quant_kernel(QuantBatch b) {
  extern __shared__ __align__(16) uint8_t qsmem[];
  const int bid = (int)blockIdx.x;
  int j = 0;
#pragma unroll
  for (int i = 1; i < kMaxQuantJobs; i++)
    if (i < b.njobs && bid >= b.job[i].block0) j = i;
  const QuantJob& jb = b.job[j];
  const int64_t blk = bid - jb.block0;
  if (jb.axis == kAlongD) {
    if (jb.fmt == kMXFP4) along_d<kMXFP4, D, DOT>(jb.x, jb.codes, jb.scales, jb.work, blk, jb.y, jb.lse, jb.ndot, jb.nl);
    else along_d<kMXFP8, D, DOT>(jb.x, jb.codes, jb.scales, jb.work, blk, jb.y, jb.lse, jb.ndot, jb.nl);
  } else {
    if (jb.fmt == kMXFP4) along_seq<kMXFP4, D>(jb.x, jb.codes, jb.scales, b.N, blk, qsmem);
    else along_seq<kMXFP8, D>(jb.x, jb.codes, jb.scales, b.N, blk, qsmem);
  }
}

}  // namespace

// ---------------------------------------------------------------- launchers
hipError_t launch_quantize_batch(const QuantTask* tasks, int count, int N, int D, hipStream_t stream) {
  if (count < 1 || count > kMaxQuantJobs) return hipErrorInvalidValue;
  QuantBatch b{};
  int64_t blocks = 0;
  size_t smem = 0;  // the LDS tile of the along-sequence jobs (the largest format among them)
  bool any_dot = false;
  // The along-sequence jobs take the first workgroups: each of their workgroups loads, converts
  // and stores a whole tile in turn and takes longer than an along-D workgroup, so started first
  // they overlap the along-D work instead of finishing the launch on their own (the jobs are
  // independent; the order changes no result).
  int order[kMaxQuantJobs], n = 0;
  for (int i = 0; i < count; i++)
    if (tasks[i].axis != kAlongD) order[n++] = i;
  for (int i = 0; i < count; i++)
    if (tasks[i].axis == kAlongD) order[n++] = i;
  for (int i = 0; i < count; i++) {
    const QuantTask& t = tasks[order[i]];
    QuantJob& j = b.job[i];
    j.x = t.x;
    j.codes = t.codes;
    j.scales = t.scales;
    j.fmt = t.fmt;
    j.axis = t.axis;
    const bool dot = t.y != nullptr;
    if (dot != (t.lse != nullptr) || dot != (t.ndot != nullptr) || dot != (t.nl != nullptr) ||
        (dot && t.axis != kAlongD))
      return hipErrorInvalidValue;
    j.y = t.y;
    j.lse = t.lse;
    j.ndot = t.ndot;
    j.nl = t.nl;
    any_dot = any_dot || dot;
    j.block0 = (int)blocks;
    if (t.axis == kAlongD) {
      j.work = t.rows * N * D / 8;
      blocks += (j.work + kUnitsPerBlockD - 1) / kUnitsPerBlockD;
    } else {
      const int per = D == 128 ? kKbSeq<128> : kKbSeq<64>;
      j.work = 0;
      blocks += t.rows * ((N / 32 + per - 1) / per);
      const size_t need = D == 128 ? (t.fmt == kMXFP4 ? kSeqLdsBytes<kMXFP4, 128> : kSeqLdsBytes<kMXFP8, 128>)
                                   : (t.fmt == kMXFP4 ? kSeqLdsBytes<kMXFP4, 64> : kSeqLdsBytes<kMXFP8, 64>);
      smem = need > smem ? need : smem;
    }
  }
  b.njobs = count;
  b.N = N;
  if (blocks == 0) return hipSuccess;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)blocks), block(kThreadsQ);
  if (D == 128) {
    if (any_dot) quant_kernel<128, true><<<grid, block, smem, stream>>>(b);
    else quant_kernel<128, false><<<grid, block, smem, stream>>>(b);
  } else {
    if (any_dot) quant_kernel<64, true><<<grid, block, smem, stream>>>(b);
    else quant_kernel<64, false><<<grid, block, smem, stream>>>(b);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, int fmt, int axis, int64_t BH, int N,
                           int D, hipStream_t stream) {
  const QuantTask t{x, codes, scales, BH, fmt, axis};
  return launch_quantize_batch(&t, 1, N, D, stream);
}

}  // namespace fp4attn

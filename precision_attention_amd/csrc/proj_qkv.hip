// proj_qkv.hip -- the QKV projection with the MX quantization in its epilogue.
//
// Q, K, V = X Wq^T, X Wk^T, X Wv^T on the BF16 MFMA with fp32 accumulation, and the epilogue
// writes the quantized tensors the attention kernels read, from the fp32 accumulators: no bf16
// copy of Q, K or V is formed (gist.science summary of "Hardware-Aware FP4 FlashAttention-4",
// Methodology 2 "Quantized Causal Backward", *Gradient Formats*: the projection epilogues publish
// the quantized operands and their FP8 row/column views; Results, *Training Performance*).
// Outputs: Q and K as MXFP4 along D, V along the sequence (MXFP4 for Direct-P, MXFP8 for the FP8
// routes) and, as an option, the backward's MXFP8 views: Q and K along the sequence, V along D.
// The MX rule is the quantizer's (OCP MX v1.0 block exponent floor(log2 amax) - emax, RNE codes,
// saturating), applied to the fp32 sums.
//
// Weight layout: one linear layer's weight, [(H + 2 Hkv) D, Dm] row-major (output features by
// input features): the rows of Wq (H heads of D rows), then Wk, then Wv. X is [B, N, Dm].
//
// A workgroup (8 waves, two per SIMD) computes a tile of 256 tokens x 128 features: wave w holds
// tokens 64 (w / 2) .. +63 and features 64 (w % 2) .. +63 as 2 x 2 tiles of the 32x32x16 BF16 MFMA,
// with lanes indexed by feature and registers by token; while one wave of a SIMD waits on its
// loads or fragments, the other issues MFMAs. The model dimension runs in stages of 64:
// both operand tiles (256 and 128 rows of 128 bytes) are fetched two stages ahead into three
// rotating LDS buffers by direct global->LDS loads, 16-byte chunks XOR-swizzled by row so that the
// fragment reads are conflict-free; one wait and one barrier per stage, the next loads issued
// half at a time between the MFMA steps. Tiles are numbered so that
// the 32 workgroups an XCD runs at once cover 4 token tiles x 8 feature tiles. The epilogue writes the
// fp32 tile to LDS (reusing the buffers) and quantizes it from there: along D a lane takes 8
// consecutive features of a token and a quad shares each 32-feature block; along the sequence a
// lane takes one feature over a 32-token block, and the 8 blocks of a feature sit in 8
// consecutive lanes, so each store instruction writes whole 128- or 256-byte row spans of the
// transposed layout.
#include <atomic>

#include "device_common.h"
#include "kernels.h"

namespace fp4attn {
namespace {

constexpr int kPM = 256;                        // tokens per tile
constexpr int kPN = 128;                        // features per tile
constexpr int kPK = 64;                         // model-dimension elements per stage
constexpr int kPThreads = 512;                  // 8 waves
constexpr int kRowBytes = kPK * 2;              // one operand row of a stage: 128 bytes
constexpr int kABytes = kPM * kRowBytes;        // 32 KiB
constexpr int kStageBytes = kABytes + kPN * kRowBytes;  // 48 KiB
constexpr int kStages = 3;
constexpr int kLoadsPerWave = kStageBytes / 1024 / (kPThreads / 64);   // 1 KiB per wave instruction: 6
// the fp32 epilogue tile: [256][128] with 4 dwords of skew per 32 rows
constexpr int kEpiDwords = kPM * kPN + (kPM / 32) * 4;
constexpr int kSmem = kStages * kStageBytes;
static_assert(kEpiDwords * 4 <= kSmem, "the epilogue tile reuses the stage buffers");
// tiles an XCD's 32 CUs run at once: 4 token tiles x 8 feature tiles
constexpr int kSbT = 4, kSbF = 8;

__device__ __forceinline__ int epi(int r, int c) { return r * kPN + (r >> 5) * 4 + c; }
// physical 16-byte chunk of logical chunk c in operand row r: rows r and r + 2 of a 16-row
// read phase land in different bank groups
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

// the fp32 block exponent: floor(log2 amax) is the biased exponent field minus 127 (a zero or
// subnormal maximum lands below -127 and clamps)
template <int EMAX>
__device__ __forceinline__ int block_exp_f32(uint32_t amax_bits) {
  const int e = (int)(amax_bits >> 23) - 127 - EMAX;
  return e < -127 ? -127 : e;
}
__device__ __forceinline__ float scale_of(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
// 448 * 2^e: the largest input that stays finite in E4M3 after the division by 2^e
__device__ __forceinline__ float e4m3_limit(int e) { return __uint_as_float(((uint32_t)(e + 135) << 23) | 0x600000u); }

__device__ __forceinline__ uint32_t fp4x8(const float* x, float sc) {
  uint32_t r = __float_as_uint(x[0]);  // every byte is written
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[0], x[1], sc, 0);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[2], x[3], sc, 1);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[4], x[5], sc, 2);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[6], x[7], sc, 3);
  return r;
}
__device__ __forceinline__ uint32_t fp8x4(const float* x, float lim, float sc) {
  v2s r = __builtin_bit_cast(v2s, x[0]);  // both halves are written
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(x[0], -lim, lim),
                                               __builtin_amdgcn_fmed3f(x[1], -lim, lim), sc, false);
  r = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(r, __builtin_amdgcn_fmed3f(x[2], -lim, lim),
                                               __builtin_amdgcn_fmed3f(x[3], -lim, lim), sc, true);
  uint32_t u;
  __builtin_memcpy(&u, &r, 4);
  return u;
}
__device__ __forceinline__ uint32_t quad_umax(uint32_t x) {
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xF, 0xF, false));  // [1,0,3,2]
  x = max(x, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xF, 0xF, false));  // [2,3,0,1]
  return x;
}

// Along D over one head slice (256 tokens x D features of the tile, at column c0): FMT 1 = MXFP4,
// 2 = MXFP8. codes/scales point at the head's token tok0; rows at or beyond nvalid are not stored.
template <int D, int FMT>
__device__ __forceinline__ void epi_along_d(const float* T, int c0, uint8_t* codes, uint8_t* scales, int nvalid) {
  constexpr int CPR = D / 8;  // 8-feature units per token
  constexpr int EMAX = FMT == kMXFP4 ? 2 : 8;
#pragma unroll 2
  for (int it = 0; it < kPM * CPR / kPThreads; it++) {
    const int u = it * kPThreads + threadIdx.x;
    const int row = u / CPR, ch = u % CPR;
    const float4 a = *reinterpret_cast<const float4*>(T + epi(row, c0 + ch * 8));
    const float4 b = *reinterpret_cast<const float4*>(T + epi(row, c0 + ch * 8 + 4));
    const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 8; i++) m = max(m, __float_as_uint(x[i]) & 0x7FFFFFFFu);
    m = quad_umax(m);
    const int e = block_exp_f32<EMAX>(m);
    const float sc = scale_of(e);
    if (row < nvalid) {
      if constexpr (FMT == kMXFP4) {
        *reinterpret_cast<uint32_t*>(codes + (int64_t)row * (D / 2) + ch * 4) = fp4x8(x, sc);
      } else {
        const float lim = e4m3_limit(e);
        const uint2 w = make_uint2(fp8x4(x, lim, sc), fp8x4(x + 4, lim, sc));
        *reinterpret_cast<uint2*>(codes + (int64_t)row * D + ch * 8) = w;
      }
      if ((ch & 3) == 0) scales[(int64_t)row * (D / 32) + ch / 4] = (uint8_t)(e + 127);
    }
  }
}

// Along the sequence over one head slice: lane (tid % 8) takes token block tid % 8 of feature
// tid / 8 (+ 32 per step). codes/scales point at the head's feature 0; the token tile starts at
// tok0 (a multiple of 256) in rows of N tokens; blocks at or beyond nvalid tokens are not stored.
template <int D, int FMT>
__device__ __forceinline__ void epi_along_seq(const float* T, int c0, uint8_t* codes, uint8_t* scales, int N,
                                              int tok0, int nvalid) {
  constexpr int EMAX = FMT == kMXFP4 ? 2 : 8;
  const int blk = threadIdx.x & 7;
  const bool store = blk * 32 < nvalid;
#pragma unroll 1
  for (int g = 0; g < D / (kPThreads / 8); g++) {
    const int d = g * (kPThreads / 8) + (threadIdx.x >> 3);
    float x[32];
#pragma unroll
    for (int t = 0; t < 32; t++) x[t] = T[epi(blk * 32 + t, c0 + d)];
    uint32_t m = 0;
#pragma unroll
    for (int t = 0; t < 32; t++) m = max(m, __float_as_uint(x[t]) & 0x7FFFFFFFu);
    const int e = block_exp_f32<EMAX>(m);
    const float sc = scale_of(e);
    if (store) {
      if constexpr (FMT == kMXFP4) {
        uint4 w;
        w.x = fp4x8(x, sc);
        w.y = fp4x8(x + 8, sc);
        w.z = fp4x8(x + 16, sc);
        w.w = fp4x8(x + 24, sc);
        *reinterpret_cast<uint4*>(codes + (int64_t)d * (N / 2) + (tok0 + blk * 32) / 2) = w;
      } else {
        const float lim = e4m3_limit(e);
        uint4 w0, w1;
        w0.x = fp8x4(x, lim, sc);
        w0.y = fp8x4(x + 4, lim, sc);
        w0.z = fp8x4(x + 8, lim, sc);
        w0.w = fp8x4(x + 12, lim, sc);
        w1.x = fp8x4(x + 16, lim, sc);
        w1.y = fp8x4(x + 20, lim, sc);
        w1.z = fp8x4(x + 24, lim, sc);
        w1.w = fp8x4(x + 28, lim, sc);
        uint4* p = reinterpret_cast<uint4*>(codes + (int64_t)d * N + tok0 + blk * 32);
        p[0] = w0;
        p[1] = w1;
      }
      scales[(int64_t)d * (N / 32) + tok0 / 32 + blk] = (uint8_t)(e + 127);
    }
  }
}

// The quantizing epilogue over one 128-feature slice of the fp32 tile T (features f0 .. f0 + 127 of
// tokens tok0 .. tok0 + 255 of batch b): each D-feature head slice in it goes to its outputs.
template <int D>
__device__ __forceinline__ void epilogue_slice(const ProjArgs& a, const float* T, int b, int tok0, int f0, int nvalid) {
#pragma unroll 1
  for (int sl = 0; sl < kPN / D; sl++) {
    const int f = f0 + sl * D;  // the slice's first feature; uniform over the workgroup
    if (f >= a.F) break;
    const int hd = f / D;
    const int c0 = sl * D;
    if (hd < a.H) {  // Q
      const int64_t bh = (int64_t)b * a.H + hd;
      epi_along_d<D, kMXFP4>(T, c0, a.q + (bh * a.N + tok0) * (D / 2), a.qs + (bh * a.N + tok0) * (D / 32), nvalid);
      if (a.q8) epi_along_seq<D, kMXFP8>(T, c0, a.q8 + bh * D * a.N, a.q8s + bh * D * (a.N / 32), a.N, tok0, nvalid);
    } else if (hd < a.H + a.Hkv) {  // K
      const int64_t bh = (int64_t)b * a.Hkv + (hd - a.H);
      epi_along_d<D, kMXFP4>(T, c0, a.k + (bh * a.N + tok0) * (D / 2), a.ks + (bh * a.N + tok0) * (D / 32), nvalid);
      if (a.k8) epi_along_seq<D, kMXFP8>(T, c0, a.k8 + bh * D * a.N, a.k8s + bh * D * (a.N / 32), a.N, tok0, nvalid);
    } else {  // V
      const int64_t bh = (int64_t)b * a.Hkv + (hd - a.H - a.Hkv);
      if (a.v_fp8)
        epi_along_seq<D, kMXFP8>(T, c0, a.v + bh * D * a.N, a.vs + bh * D * (a.N / 32), a.N, tok0, nvalid);
      else
        epi_along_seq<D, kMXFP4>(T, c0, a.v + bh * D * (a.N / 2), a.vs + bh * D * (a.N / 32), a.N, tok0, nvalid);
      if (a.v8) epi_along_d<D, kMXFP8>(T, c0, a.v8 + (bh * a.N + tok0) * D, a.v8s + (bh * a.N + tok0) * (D / 32), nvalid);
    }
  }
}

template <int D>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void proj_qkv_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) lds_char smem[kSmem];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntt = (a.N + kPM - 1) / kPM;
  const int nft = (a.F + kPN - 1) / kPN;
  // XCD-aware numbering: workgroup i runs on XCD i % 8; its j-th workgroup there belongs to
  // super-block (j / 32) * 8 + i % 8 of 4 token tiles x 8 feature tiles, whose 32 workgroups run
  // at the same time and share the XCD's L2 (4 X tiles and 8 weight tiles)
  const int tiles_t = a.B * ntt;
  const int nsb_t = (tiles_t + kSbT - 1) / kSbT;
  const int j = blockIdx.x >> 3;
  const int sb = (j / (kSbT * kSbF)) * 8 + (blockIdx.x & 7);
  const int r = j % (kSbT * kSbF);
  const int bt = (sb % nsb_t) * kSbT + r % kSbT;
  const int ft = (sb / nsb_t) * kSbF + r / kSbT;
  if (bt >= tiles_t || ft >= nft) return;  // the padding of the last super-blocks
  const int b = bt / ntt;
  const int tok0 = (bt % ntt) * kPM;
  const int f0 = ft * kPN;
  const int nvalid = min(kPM, a.N - tok0);

  // ---- loads: this wave's 6 instructions per stage, 8 operand rows of 128 bytes each ----
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x) + ((int64_t)b * a.N + tok0) * a.Dm * 2;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(a.w) + (int64_t)f0 * a.Dm * 2;
  uint32_t off[kLoadsPerWave];
#pragma unroll
  for (int i = 0; i < kLoadsPerWave; i++) {
    const int gi = wave * kLoadsPerWave + i;  // 0..31 rows of X, 32..47 rows of W, 8 rows each
    const int row = (gi < 32 ? gi : gi - 32) * 8 + (lane >> 3);
    const int c = swz(row, lane & 7);        // the global chunk this lane's LDS slot holds
    // rows past the end re-read the last valid row (never stored)
    const int src = gi < 32 ? min(row, a.N - tok0 - 1) : min(row, a.F - f0 - 1);
    off[i] = (uint32_t)src * (uint32_t)(a.Dm * 2) + (uint32_t)c * 16u;
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue_part = [&](int s, int buf, int p, int np) {
    const uint8_t* xs = xb + (int64_t)s * kRowBytes;
    const uint8_t* ws = wb + (int64_t)s * kRowBytes;
#pragma unroll
    for (int i = p * (kLoadsPerWave / np); i < (p + 1) * (kLoadsPerWave / np); i++) {
      const int gi = wave * kLoadsPerWave + i;
      dma16_async(gi < 32 ? xs : ws, off[i], lds0 + buf * kStageBytes + gi * 1024);
    }
  };
  auto issue = [&](int s, int buf) {
    const uint8_t* xs = xb + (int64_t)s * kRowBytes;
    const uint8_t* ws = wb + (int64_t)s * kRowBytes;
#pragma unroll
    for (int i = 0; i < kLoadsPerWave; i++) {
      const int gi = wave * kLoadsPerWave + i;
      const uint32_t dst = lds0 + buf * kStageBytes + gi * 1024;
      dma16_async(gi < 32 ? xs : ws, off[i], dst);
    }
  };

  // ---- fragments: lane row (lane & 31), chunk 2 k16 + (lane >> 5) ----
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, hf = lane >> 5;
  uint32_t frag_off[4];
#pragma unroll
  for (int k = 0; k < 4; k++) frag_off[k] = lr * kRowBytes + swz(lr, 2 * k + hf) * 16;

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;

  const int S = a.Dm / kPK;
  issue(0, 0);
  if (S > 1) issue(1, 1);
  for (int s = 0; s < S; s++) {
    // this stage's loads are done when at most the next stage's 6 are still in flight
    if (s + 1 < S) asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    const lds_char* sa = smem + (s % kStages) * kStageBytes + wm * 64 * kRowBytes;
    const lds_char* sb = smem + (s % kStages) * kStageBytes + kABytes + wn * 64 * kRowBytes;
    v8bf fa[2][2], fb[2][2];
    auto ld = [&](int k, v8bf (&a4)[2], v8bf (&b2)[2]) {
#pragma unroll
      for (int i = 0; i < 2; i++)
        a4[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(sa + i * 32 * kRowBytes + frag_off[k]));
#pragma unroll
      for (int j = 0; j < 2; j++)
        b2[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(sb + j * 32 * kRowBytes + frag_off[k]));
    };
    // fragments one k16 step ahead of the MFMAs; the scheduling groups pin that order (the
    // compiler otherwise issues each read just before its MFMA)
    ld(0, fa[0], fb[0]);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      // half of stage s + 2's loads before every other k16 step: a burst of all of them holds up
      // the wave's in-order issue, MFMAs included
      if (s + 2 < S && (k & 1) == 0) issue_part(s + 2, (s + 2) % kStages, k >> 1, 2);
      if (k < 3) ld(k + 1, fa[(k + 1) & 1], fb[(k + 1) & 1]);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k & 1][i], fb[k & 1][j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  }
  __syncthreads();  // every wave is done reading the stage buffers

  // ---- epilogue: the fp32 tile through LDS ----
  float* T = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int row = wm * 64 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
        T[epi(row, wn * 64 + j * 32 + lr)] = acc[i][j][r];
      }
  __syncthreads();

  epilogue_slice<D>(a, T, b, tok0, f0, nvalid);
}


// ---- the wide tile: 256 tokens x 256 features ----
// For launches with many tiles. Wave w holds tokens 128 (w / 4) .. +127 and features 64 (w % 4) ..
// +63 as 4 x 2 MFMA tiles: 6 fragment reads per 8 MFMAs where the 256 x 128 tile takes 4 per 4, so
// the LDS reads per MFMA drop by a quarter. The model dimension runs in stages of 32 (rows of 64
// bytes, 32 KiB per stage) through four LDS buffers: stage s + 3 is fetched while stage s is read.
// One barrier per stage, placed between the stage's two k16 steps: after it a wave fetches the next
// stage's first fragments, so the MFMAs never wait on a fragment read that follows a barrier. The
// accumulators take the same k16 steps in the same order as in the 256 x 128 kernel, so the two
// give bit-identical outputs. The epilogue runs twice, once per 128-feature half, through the same
// fp32 tile in LDS.
constexpr int kWN = 256;                         // features per wide tile
constexpr int kWK = 32;                          // model-dimension elements per stage
constexpr int kWRow = kWK * 2;                   // one operand row of a stage: 64 bytes
constexpr int kWOp = kPM * kWRow;                // one operand's rows of a stage: 16 KiB
constexpr int kWStage = 2 * kWOp;                // 32 KiB
constexpr int kWStages = 4;
constexpr int kWLoads = kWStage / 1024 / (kPThreads / 64);  // 1 KiB per wave instruction: 4
constexpr int kWSmem = kWStages * kWStage > kEpiDwords * 4 ? kWStages * kWStage : kEpiDwords * 4;
// physical 16-byte chunk of logical chunk c in a 64-byte row r: the four rows of one bank quarter in
// a 16-row read phase (r, r + 4, r + 8, r + 12) take four different chunks
__device__ __forceinline__ int wswz(int r, int c) { return c ^ ((r >> 2) & 3); }

template <int D>
__global__ __launch_bounds__(kPThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void proj_qkv_wide_kernel(const ProjArgs a) {
  __shared__ __attribute__((aligned(16))) lds_char smem[kWSmem];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int ntt = (a.N + kPM - 1) / kPM;
  const int nft = (a.F + kWN - 1) / kWN;
  // the XCD-aware numbering of the 256 x 128 kernel over the wide tiles
  const int tiles_t = a.B * ntt;
  const int nsb_t = (tiles_t + kSbT - 1) / kSbT;
  const int j = blockIdx.x >> 3;
  const int sb = (j / (kSbT * kSbF)) * 8 + (blockIdx.x & 7);
  const int r = j % (kSbT * kSbF);
  const int bt = (sb % nsb_t) * kSbT + r % kSbT;
  const int ft = (sb / nsb_t) * kSbF + r / kSbT;
  if (bt >= tiles_t || ft >= nft) return;  // the padding of the last super-blocks
  const int b = bt / ntt;
  const int tok0 = (bt % ntt) * kPM;
  const int f0 = ft * kWN;
  const int nvalid = min(kPM, a.N - tok0);

  // ---- loads: this wave's 4 instructions per stage, 16 operand rows of 64 bytes each ----
  const uint8_t* xb = reinterpret_cast<const uint8_t*>(a.x) + ((int64_t)b * a.N + tok0) * a.Dm * 2;
  const uint8_t* wb = reinterpret_cast<const uint8_t*>(a.w) + (int64_t)f0 * a.Dm * 2;
  uint32_t off[kWLoads];
#pragma unroll
  for (int i = 0; i < kWLoads; i++) {
    const int gi = wave * kWLoads + i;  // 0..15 rows of X, 16..31 rows of W, 16 rows each
    const int row = (gi & 15) * 16 + (lane >> 2);
    const int c = wswz(row, lane & 3);  // the global chunk this lane's LDS slot holds
    // rows past the end re-read the last valid row (never stored)
    const int src = gi < 16 ? min(row, a.N - tok0 - 1) : min(row, a.F - f0 - 1);
    off[i] = (uint32_t)src * (uint32_t)(a.Dm * 2) + (uint32_t)c * 16u;
  }
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int s, int buf) {
    const uint8_t* xs = xb + (int64_t)s * kWRow;
    const uint8_t* ws = wb + (int64_t)s * kWRow;
#pragma unroll
    for (int i = 0; i < kWLoads; i++) {
      const int gi = wave * kWLoads + i;
      dma16_async(gi < 16 ? xs : ws, off[i], lds0 + buf * kWStage + gi * 1024);
    }
  };

  // ---- fragments: lane row (lane & 31), chunk 2 k16 + (lane >> 5) ----
  const int wm = wave >> 2, wn = wave & 3;
  const int lr = lane & 31, hf = lane >> 5;
  uint32_t frag_off[2];
#pragma unroll
  for (int k = 0; k < 2; k++) frag_off[k] = lr * kWRow + wswz(lr, 2 * k + hf) * 16;
  auto ld = [&](int s, int k, v8bf (&a4)[4], v8bf (&b2)[2]) {
    const lds_char* sa = smem + (s % kWStages) * kWStage + wm * 128 * kWRow + frag_off[k];
    const lds_char* sb = smem + (s % kWStages) * kWStage + kWOp + wn * 64 * kWRow + frag_off[k];
#pragma unroll
    for (int i = 0; i < 4; i++) a4[i] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(sa + i * 32 * kWRow));
#pragma unroll
    for (int j = 0; j < 2; j++) b2[j] = __builtin_bit_cast(v8bf, *reinterpret_cast<const u32x4*>(sb + j * 32 * kWRow));
  };

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 2; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.0f;
  auto mma = [&](const v8bf (&a4)[4], const v8bf (&b2)[2]) {
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int j = 0; j < 2; j++) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a4[i], b2[j], acc[i][j], 0, 0, 0);
  };

  // wait until at most n stages' loads of this wave are in flight (n < kWStages - 1)
  auto wait_stages = [](int n) {
    if (n >= 3) asm volatile("s_waitcnt vmcnt(12)" ::: "memory");
    else if (n == 2) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
    else if (n == 1) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  static_assert(kWLoads == 4 && kWStages <= 5, "wait_stages counts 4 loads per stage, at most 3 stages");
  const int S = a.Dm / kWK;  // at least 2 (the model dimension is a multiple of 64)
#pragma unroll
  for (int t = 0; t < kWStages - 1; t++)
    if (t < S) issue(t, t);
  wait_stages(min(S, kWStages - 1) - 1);
  __syncthreads();
  v8bf fa[2][4], fb[2][2];
  ld(0, 0, fa[0], fb[0]);
  // the last stage is peeled: a path that skips the barrier would leave the compiler's count of
  // fragment reads in flight merged with this one, and the k16 step after the barrier would then
  // wait on the next stage's reads
  // the scheduling groups issue each k16 step's 6 fragment reads before the other step's 8 MFMAs
  // (left alone, the compiler shares their registers and issues the reads after 6 of the MFMAs)
  for (int s = 0; s + 1 < S; s++) {
    ld(s, 1, fa[1], fb[1]);
    mma(fa[0], fb[0]);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    // stage s + 1 has landed when at most the later stages' loads are still in flight; after the
    // barrier no wave reads stage s - 1's buffer again, and stage s + kWStages - 1 goes there (its
    // loads issued after this step's MFMAs, which would otherwise wait behind them)
    wait_stages(min(S - 2 - s, kWStages - 3));
    __syncthreads();
    ld(s + 1, 0, fa[0], fb[0]);
    mma(fa[1], fb[1]);
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    if (s + kWStages - 1 < S) issue(s + kWStages - 1, (s + kWStages - 1) % kWStages);
  }
  ld(S - 1, 1, fa[1], fb[1]);
  mma(fa[0], fb[0]);
  mma(fa[1], fb[1]);
  __syncthreads();  // every wave is done reading the stage buffers

  // ---- epilogue: one 128-feature half at a time through the fp32 tile in LDS ----
  float* T = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int h = 0; h < 2; h++) {
    if ((wn >> 1) == h) {
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int row = wm * 128 + i * 32 + 8 * (r >> 2) + 4 * hf + (r & 3);
            T[epi(row, (wn & 1) * 64 + j * 32 + lr)] = acc[i][j][r];
          }
    }
    __syncthreads();
    epilogue_slice<D>(a, T, b, tok0, f0 + h * kPN, nvalid);
    if (h == 0) __syncthreads();  // the second half overwrites the tile
  }
}

}  // namespace

namespace {
// compute units of the current device (256 on an MI355X; fewer on a partition of one), read once
// per device
int64_t device_cus() {
  static std::atomic<int> cached[64];  // zero-initialized (static storage); 0 = not read yet
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  if (dev < 64) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}
}  // namespace

hipError_t launch_proj_qkv(const ProjArgs& a, int D, int tile, hipStream_t stream, const KernelEvents& ev) {
  const int64_t tt = (int64_t)a.B * ((a.N + kPM - 1) / kPM);
  const int64_t nft = (a.F + kPN - 1) / kPN, nwt = (a.F + kWN - 1) / kWN;
  if (tile == 0) {
    // the wide tile where its rounds of workgroups (one per CU for either kernel) cover the chip at
    // least as well: half as many tiles of twice the work each, with no worse a last round
    const int64_t cus = device_cus();
    const int64_t rounds = (tt * nft + cus - 1) / cus, wrounds = (tt * nwt + cus - 1) / cus;
    tile = 2 * wrounds <= rounds ? kWN : kPN;
  }
  const bool wide = tile == kWN;
  const int64_t nsb = ((tt + kSbT - 1) / kSbT) * (((wide ? nwt : nft) + kSbF - 1) / kSbF);
  const dim3 grid((unsigned)(((nsb + 7) / 8) * 8 * kSbT * kSbF));
  if (wide) {
    if (D == 128) return launch_kernel(proj_qkv_wide_kernel<128>, grid, dim3(kPThreads), 0, stream, ev, a);
    return launch_kernel(proj_qkv_wide_kernel<64>, grid, dim3(kPThreads), 0, stream, ev, a);
  }
  if (D == 128) return launch_kernel(proj_qkv_kernel<128>, grid, dim3(kPThreads), 0, stream, ev, a);
  return launch_kernel(proj_qkv_kernel<64>, grid, dim3(kPThreads), 0, stream, ev, a);
}

}  // namespace fp4attn

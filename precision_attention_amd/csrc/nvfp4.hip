// nvfp4.hip -- NVFP4-style Q and K: the block quantizer and the Direct-P forward that consumes it.
//
// Format (gist.science summary of "Hardware-Aware FP4 FlashAttention-4", Methodology 1 "Format
// Selection": NVFP4 for Q and K, finer block scales than MXFP4): blocks of 16 consecutive elements
// along D, E2M1 elements, one E4M3 scale per block and a per-tensor scale 2^g chosen by the caller:
//   s = RNE_E4M3(amax / 6 / 2^g), saturating at 448 (zero when it rounds to zero);
//   code = RNE_E2M1(x / (s 2^g)), saturating, sign kept; magnitude 0 for every element when s = 0;
//   x_hat = E2M1(code) s 2^g, which has at most 6 significant bits and is exact in bf16.
// gfx950's scaled MFMA takes E8M0 scales per 32 elements only, so a product with E4M3 scales per
// 16 cannot run on it; the route computes S = Q_hat K_hat^T on the BF16 MFMA from the exact bf16
// expansions that the quantizer writes beside the codes, and forms P and P.V as Direct-P on the
// integer-log2 anchor (MXFP4 P and V, block-scaled FP4 MFMA, consistent normalizer).
//
// Quantizer: a lane takes 8 consecutive elements (16 bytes), a lane pair one 16-element block. The
// block scale is the E4M3 rounding of the correctly rounded fp32 quotient amax / 6 (times 2^-g,
// exact), which rounds as the exact quotient would: a bf16 value divided by 6 lies on an E4M3
// midpoint only when the exact quotient does. x / (s 2^g) is not exact in fp32, so each element's
// code comes from comparisons with the seven exact midpoints (midpoint x s x 2^g, at most 7
// significant bits), ties going to the even code.
//
// Forward: 8 waves x 32 queries per workgroup, keys in blocks of 64. Each wave holds its queries'
// Q_hat fragments (bf16) in registers; K_hat rows (bf16), V^T rows (MXFP4) and V scales of a block
// are fetched two blocks ahead into three rotating LDS buffers by direct global->LDS loads, one
// wait and one barrier per block. S^T = K_hat Q_hat^T on the 32x32x16 BF16 MFMA puts one query in
// each lane and, with K rows read in the order {0..3, 32..35, 4..7, ...}, the 32 keys of one P
// block in the 32 registers of a lane half's two tiles; the block exponent, the anchor guard, the
// codes, P.V and the normalizer are those of the anchored Direct-P kernel. Software pipeline: the
// next block's score MFMAs (into a second set of score registers, the block loop unrolled by two)
// are issued with this block's codes, so that they run under its VALU work.
#include "device_common.h"
#include "fwd_common.h"
#include "kernels.h"

namespace fp4attn {
namespace {

using fwd::max32;

// ------------------------------------------------------------------ quantizer

constexpr int kNvThreads = 256;

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const int e = (int)(c >> 3) & 15, m = (int)(c & 7);
  return e ? __builtin_amdgcn_ldexpf((float)(8 + m), e - 10) : __builtin_amdgcn_ldexpf((float)m, -9);
}
__device__ __forceinline__ float e2m1_mag(int c) {
  return c < 4 ? 0.5f * (float)c : (c == 7 ? 6.0f : (float)(c - 2));
}

__global__ __launch_bounds__(kNvThreads) void quant_nvfp4_kernel(const uint16_t* __restrict__ x,
                                                                 uint8_t* __restrict__ codes,
                                                                 uint8_t* __restrict__ scales,
                                                                 uint16_t* __restrict__ xhat, int64_t nunits,
                                                                 int g) {
  const int64_t stride = (int64_t)gridDim.x * kNvThreads;
  // nunits is even and pairs of units are adjacent lanes, so a pair is wholly in range or out
  for (int64_t u = (int64_t)blockIdx.x * kNvThreads + threadIdx.x; u - (threadIdx.x & 1) < nunits; u += stride) {
    const bool in = u < nunits;
    const uint4 v = in ? load_stream16(reinterpret_cast<const uint4*>(x) + u) : make_uint4(0, 0, 0, 0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) m = max(m, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));  // lane pair
    const float amax = __uint_as_float(m << 16);
    // the block scale: RNE E4M3 of amax / 6 / 2^g, clamped to 448 (the converter does not saturate)
    const float q = fminf(__builtin_amdgcn_ldexpf(__fdiv_rn(amax, 6.0f), -g), 448.0f);
    v2s sv = {0, 0};
    sv = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(sv, q, 0.0f, 1.0f, false);
    const uint32_t sc = (uint32_t)sv[0] & 0xFFu;
    const float sg = __builtin_amdgcn_ldexpf(e4m3_value(sc), g);
    const float t0 = 0.25f * sg, t1 = 0.75f * sg, t2 = 1.25f * sg, t3 = 1.75f * sg;
    const float t4 = 2.5f * sg, t5 = 3.5f * sg, t6 = 5.0f * sg;
    uint32_t packed = 0;
    uint32_t hat[4];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      const uint32_t h = (w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      const float a = __uint_as_float((h & 0x7FFFu) << 16);
      // midpoint k lies between codes k and k + 1; a tie goes to the even one
      int c = (a > t0) + (a >= t1) + (a > t2) + (a >= t3) + (a > t4) + (a >= t5) + (a > t6);
      if (sc == 0) c = 0;
      const uint32_t sign = h >> 15;
      packed |= (uint32_t)(c | (sign << 3)) << (4 * i);
      const uint32_t vb = (__float_as_uint(e2m1_mag(c) * sg) >> 16) | (sign << 15);  // exact in bf16
      if (i & 1) hat[i >> 1] |= vb << 16;
      else hat[i >> 1] = vb;
    }
    if (in) {
      reinterpret_cast<uint32_t*>(codes)[u] = packed;
      reinterpret_cast<uint4*>(xhat)[u] = make_uint4(hat[0], hat[1], hat[2], hat[3]);
      if ((u & 1) == 0) scales[u >> 1] = (uint8_t)sc;
    }
  }
}

// ------------------------------------------------------------------ forward

constexpr int kNvWaves = 8;
constexpr int kNvQTile = 32 * kNvWaves;
constexpr int kNvKB = 64;  // keys per block

template <int D>
struct NvSmem {
  static constexpr int kRow = 2 * D;                  // bytes of one K_hat row (bf16)
  static constexpr int kCh = kRow / 16;               // 16-byte chunks per K_hat row
  static constexpr int kBytes = kNvKB * kRow;
  static constexpr int vRow = kNvKB / 2;              // bytes of one V^T row (MXFP4) per block
  static constexpr int vCh = vRow / 16;               // 2
  static constexpr int vOff = kBytes;
  static constexpr int vsOff = vOff + D * vRow;       // V scales: one dword per byte, [32-key block][d]
  static constexpr int buf = vsOff + 2 * D * 4;
  static constexpr int kDma = kBytes / 1024;          // 16-byte-per-lane instructions
  static constexpr int vDma = D * vRow / 1024;
  static constexpr int vsDma = 2 * D / 64;            // 1-byte-per-lane instructions (dword slots)
  static constexpr int nDma = kDma + vDma + vsDma;
};

// physical 16-byte chunk of logical chunk c in K_hat row r: a fragment read phase of 16 lanes
// touches rows {0..3, 32..35, 4..7, 36..39} (+16 t, +64 offsets) at one logical chunk
template <int D>
__device__ __forceinline__ int nv_kchunk(int r, int c) {
  if constexpr (D == 128) return c ^ ((r & 3) | (((r >> 2) & 1) << 2) | (((r >> 5) & 1) << 3));  // 16 chunks
  else return c ^ (((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 5) & 1) << 2));  // 8 chunks, 2 rows / 256 B
}
// V^T row chunk swizzle (2 chunks per row per block)
__device__ __forceinline__ int nv_vchunk(int d, int c) { return c ^ ((d >> 3) & 1); }

template <int D>
__global__ void __launch_bounds__(64 * kNvWaves, 2) attn_fwd_nvfp4_kernel(NvFwdArgs a) {
  using L = NvSmem<D>;
  constexpr int DT = D / 32;
  constexpr int KS = D / 16;  // BF16 MFMA k-steps over D
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr int kSmem = 3 * L::buf > kNvWaves * OStage<D>::kBytes ? 3 * L::buf : kNvWaves * OStage<D>::kBytes;
  __shared__ __attribute__((aligned(16))) lds_char smem[kSmem];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;
  // workgroup -> (batch*head, query tile): each XCD takes a contiguous range of tiles
  const int nqt = (N + kNvQTile - 1) / kNvQTile;
  const int total = (int)gridDim.x;
  const int per = total / 8, rem = total % 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  const int qt = lin % nqt, bh = lin / nqt, h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int q0 = qt * kNvQTile + wave * 32;
  const int qi = q0 + col;
  const bool qvalid = qi < N;

  // this lane's Q_hat fragments: query qi, d = 16 s + 8 half .. +7
  v8bf qh[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) {
    uint4 t = make_uint4(0, 0, 0, 0);
    if (qvalid) t = *reinterpret_cast<const uint4*>(a.q + ((int64_t)bh * N + qi) * D + 16 * s + 8 * half);
    qh[s] = __builtin_bit_cast(v8bf, t);
  }

  // ---- staging: DMA instruction i of a block is issued by wave i % 8 ----
  const uint8_t* kh = reinterpret_cast<const uint8_t*>(a.k) + bhkv * N * D * 2;
  const uint8_t* vh = a.v + bhkv * D * (N / 2);
  const uint8_t* vsh = a.vs + bhkv * D * (N / 32);
  const uint32_t lds0 = lds_addr(smem);
  const int wv = __builtin_amdgcn_readfirstlane(wave);  // wave-uniform: the DMA choice is scalar
  auto issue = [&](int j, int buf) {
    const int kb0 = j * kNvKB;
    const uint32_t base = lds0 + buf * L::buf;
#pragma unroll
    for (int i = wv; i < L::nDma; i += kNvWaves) {
      if (i < L::kDma) {
        const int P = i * 64 + lane;  // 16-byte slot
        const int r = P / L::kCh, c = nv_kchunk<D>(r, P % L::kCh);
        const int gk = min(kb0 + r, N - 1);
        dma16_async(kh, (uint32_t)gk * (D * 2) + (uint32_t)c * 16, base + i * 1024);
      } else if (i < L::kDma + L::vDma) {
        const int P = (i - L::kDma) * 64 + lane;
        const int d = P / L::vCh, c = nv_vchunk(d, P % L::vCh);
        const int cc = (kb0 + c * 32 < N) ? c : 0;  // chunks past N re-read the block's first chunk
        dma16_async(vh, (uint32_t)d * (N / 2) + (uint32_t)(kb0 / 2 + cc * 16), base + L::vOff + (i - L::kDma) * 1024);
      } else {
        const int P = (i - L::kDma - L::vDma) * 64 + lane;  // dword slot: block e = P / D, row d
        const int d = P % D, e = P / D;
        dma1_async(vsh, (uint32_t)d * (N / 32) + (uint32_t)min(kb0 / 32 + e, N / 32 - 1),
                   base + L::vsOff + (i - L::kDma - L::vDma) * 256);
      }
    }
  };

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;
  v16f accl;
#pragma unroll
  for (int r = 0; r < 16; r++) accl[r] = 0.0f;
  v8i ones;
#pragma unroll
  for (int r = 0; r < 8; r++) ones[r] = 0x22222222;  // E2M1 1.0
  float anchor = -INFINITY;

  // lane-constant LDS offsets: K row krow(col) (+16 t), V^T row col (+32 t)
  const int krow = (((col >> 2) & 1) << 5) + ((col >> 3) << 2) + (col & 3);
  const int vb = L::vOff + col * L::vRow + nv_vchunk(col, half) * 16;
  const int vs_base = L::vsOff + (half * D + col) * 4;

  const int nkb = (N + kNvKB - 1) / kNvKB;

  // S^T tiles of the block staged at sb: tile t holds keys 32 half + 16 t + i (register i)
  auto scores = [&](const lds_char* sb, v16f (&sn)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int r = krow + 16 * t;
#pragma unroll
      for (int rr = 0; rr < 16; rr++) sn[t][rr] = 0.0f;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sb + r * L::kRow + nv_kchunk<D>(r, 2 * ks + half) * 16);
        sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kf), qh[ks], sn[t], 0, 0, 0);
      }
    }
  };

  // One key block j with its scores in sc, staged at sb; block j+1's scores are formed into sn
  // from sbn while block j's codes are generated (software pipeline: the BF16 MFMAs of the next
  // block run under this block's VALU work). After the last block they are formed from a stale
  // buffer and never read.
  auto block = [&](int j, v16f (&sc)[2], v16f (&sn)[2], const lds_char* sb, const lds_char* sbn)
      __attribute__((always_inline)) {
    const int kb0 = j * kNvKB;
    if (kb0 + kNvKB > N) {
      asm volatile("" ::: "memory");  // keeps this a branch: only a ragged last block takes it
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int i = 0; i < 16; i++)
          if (kb0 + half * 32 + 16 * t + i >= N) sc[t][i] = -INFINITY;
    }
    // block exponent of this lane half's 32-key block
    const float bm = max32(sc[0], sc[1]);
    float t = floorf(fmul_rn(bm, C));
    // the guard: move the anchor when a block sits more than 64 binades above it (on the first
    // block the anchor is -inf, so this sets it from the block's exponents)
    if (__builtin_amdgcn_ballot_w64(t - anchor > 64.0f)) {
      const float an = max_across_halves(__builtin_elementwise_maximum(t, anchor));
      const float f = __builtin_amdgcn_ldexpf(1.0f, (int)fmaxf(anchor - an, -150.0f));
#pragma unroll
      for (int tt = 0; tt < DT; tt++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[tt][r] *= f;
      accl[0] *= f;
      anchor = an;
    }
    t = __builtin_elementwise_maximum(t, anchor - 125.0f);
    scores(sbn, sn);
    // E2M1 codes of 2^(fmaf(S, c, 2 - t)); a fully masked half gives t = -inf -> clamped, codes 0
    v8i pf;
    const float off = 2.0f - t;
#pragma unroll
    for (int w = 0; w < 4; w++) {
      float x[8];
#pragma unroll
      for (int jj = 0; jj < 8; jj++) {
        const int idx = 8 * w + jj;
        x[jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[idx >> 4][idx & 15], C, off));
      }
      uint32_t u = __float_as_uint(x[0]);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[0], x[1], 1.0f, 0);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[2], x[3], 1.0f, 1);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[4], x[5], 1.0f, 2);
      u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[6], x[7], 1.0f, 3);
      pf[w] = (int)u;
    }
#pragma unroll
    for (int w = 4; w < 8; w++) pf[w] = 0;
    const int psc = (int)(t - anchor) + 125;
    // O^T += V^T P^T and l += 1^T P^T
#pragma unroll
    for (int tt = 0; tt < DT; tt++) {
      const uint4 v0 = *reinterpret_cast<const uint4*>(sb + vb + tt * 32 * L::vRow);
      v8i vf;
      vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w;
      vf[4] = vf[5] = vf[6] = vf[7] = 0;
      const int vsc = (int)*reinterpret_cast<const lds_u32*>(sb + vs_base + tt * 32 * 4);
      acc[tt] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(vf, pf, acc[tt], vsc, psc);
    }
    accl = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(ones, pf, accl, 127, psc);
    // the compiler interleaves the next block's score MFMAs with the codes (scheduling groups of
    // one MFMA per 4, 6 or 8 VALU instructions were 2-7 % slower)
  };

  // Block j is staged in buffer j % 3 (issued two blocks ahead); one wait and one barrier per
  // block, after which block j+1 has landed and block j-1's buffer is free. Blocks go in pairs
  // (alternating score registers); for an odd count a last step past the end has every key
  // masked (zero codes) and reads the last block's buffer (finite data).
  v16f sA[2], sB[2];
  issue(0, 0);
  if (nkb > 1) issue(1, 1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  scores(smem, sA);
  // buffer indices of blocks j, j+1, j+2, rotated per step (wave-uniform)
  int bj = 0, bj1 = 1, bj2 = 2;
  auto step = [&](int j, v16f (&sc)[2], v16f (&sn)[2]) __attribute__((always_inline)) {
    if (j > 0) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
    }
    if (j + 2 < nkb) issue(j + 2, bj2);
    // a step past the end reads the last block's buffer (block j - 1's)
    const int bc = j < nkb ? bj : (bj + 2) % 3;
    block(j, sc, sn, smem + bc * L::buf, smem + bj1 * L::buf);
    const int b0 = bj;
    bj = bj1;
    bj1 = bj2;
    bj2 = b0;
  };
  for (int j = 0; j < nkb; j += 2) {
    step(j, sA, sB);
    step(j + 1, sB, sA);
  }

  // ---- epilogue: O = O^T / l as whole bf16 rows, LSE = (A + log2 l) ln 2 ----
  store_o_lse_rows<D, true>(acc, accl[0], anchor, a.o + (int64_t)bh * N * D, a.lse + (int64_t)bh * N, N, q0, lane,
                            smem + wave * OStage<D>::kBytes);
}

}  // namespace

hipError_t launch_quantize_nvfp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, uint16_t* xhat, int64_t n,
                                 int g, hipStream_t stream) {
  const int64_t nunits = n / 8;
  const int64_t blocks = (nunits + kNvThreads - 1) / kNvThreads;
  const dim3 grid((unsigned)(blocks < 8192 ? blocks : 8192));
  quant_nvfp4_kernel<<<grid, kNvThreads, 0, stream>>>(x, codes, scales, xhat, nunits, g);
  return hipGetLastError();
}

hipError_t launch_attn_fwd_nvfp4(const NvFwdArgs& a, int D, hipStream_t stream, const KernelEvents& ev) {
  const int nqt = (a.N + kNvQTile - 1) / kNvQTile;
  const dim3 grid((unsigned)(a.B * a.H * nqt));
  if (D == 128) return launch_kernel(attn_fwd_nvfp4_kernel<128>, grid, dim3(64 * kNvWaves), 0, stream, ev, a);
  return launch_kernel(attn_fwd_nvfp4_kernel<64>, grid, dim3(64 * kNvWaves), 0, stream, ev, a);
}

}  // namespace fp4attn

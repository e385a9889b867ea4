// attn_bwd.hip -- backward of the causal FP4/FP8 route of "Hardware-Aware FP4
// FlashAttention-4" (gist.science technical summary, Methodology 2 "Quantized Causal
// Backward": Reconstruction, Gradient Formats; arXiv abstract).
//
// Probabilities are rebuilt from the saved MXFP4 Q/K and the forward's LSE (no separate score
// path); the four gradient products run on MXFP8 operands (E4M3 elements, one E8M0 scale per
// 32 along each product's contraction axis):
//   P  = 2^(fmaf(S, c, -fp32(LSE log2 e)))          S = Q K^T on the FP4 MFMA
//   dP = dO V^T          (dO, V blocked along D)      dS = P (dP - Delta), Delta = rowsum(dO O)
//   dV = P^T dO          (P, dO blocked along queries)
//   dK = scale dS^T Q    (dS, Q blocked along queries)
//   dQ = scale dS K      (dS, K blocked along keys)
//
// Three kernels:
//  - delta_kernel: Delta_i = sum_d dO_id O_id in fp32. dO's two MXFP8 views are produced by the
//    MX quantizer into the workspace.
//  - dkdv_kernel: one workgroup per (batch, KV head, 128-key tile), 4 waves x 32 keys. S and dP
//    are formed with keys in lanes and queries in registers (S = Q K^T, dP = dO V^T), so P and dS
//    come out of the MFMA already in the layout of the A operand of dV += P^T dO and
//    dK += dS^T Q; their MX blocks along queries span one lane pair (one permlane32 swap for the
//    block max). Loops over the query heads of the KV group and over 64-query blocks.
//  - dq_kernel: one workgroup per (batch, query head, 128-query tile), 4 waves x 32 queries, the
//    forward's orientation (queries in lanes, keys in registers): S^T = K Q^T, dP^T = V dO^T,
//    dS blocked along keys in-lane, dQ^T += K^T dS^T.
// Operand layouts of the 32x32x64 block-scaled MFMA: see device_common.h.
#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E8M0 exponent of an MXFP8 block from its largest magnitude (binary32):
// floor(log2 amax) - 8, clamped to [-127, 127]; amax == 0 gives -127.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return max(E - 127 - 8, -127);
}
// 2^-e as binary32 for e in [-127, 119]
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }
__device__ __forceinline__ float clamp448(float y) { return __builtin_amdgcn_fmed3f(y, -448.0f, 448.0f); }

// query (or key) held in register i of lane half h of a 32x32 MFMA output tile whose A rows
// were loaded in the order r -> perm32(r): the output's register i of half h is row h*16 + i.
__device__ __forceinline__ int perm32(int r) { return (((r >> 2) & 1) << 4) + ((r >> 3) << 2) + (r & 3); }

// ------------------------------------------------------------------------------------
// Delta_i = sum_d dO_id O_id (fp32). D/8 lanes per row, 16-byte loads, xor-shuffle sum.
template <int D>
__global__ void __launch_bounds__(kThreads) delta_kernel(const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
                                                         float* __restrict__ delta, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t row = t / TPR;
  const int part = (int)(t % TPR);
  float s = 0.0f;
  if (row < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + row * D + part * 8);
    const uint4 b = *reinterpret_cast<const uint4*>(dout + row * D + part * 8);
    const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      s += __uint_as_float(aw[i] << 16) * __uint_as_float(bw[i] << 16);
      s += __uint_as_float(aw[i] & 0xFFFF0000u) * __uint_as_float(bw[i] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int m = TPR / 2; m > 0; m >>= 1) s += __shfl_xor(s, m);
  if (row < rows && part == 0) delta[row] = s;
}

// ------------------------------------------------------------------------------------
struct BwdArgs {
  const uint8_t* q;    // MXFP4 along D [B*H][N][D/2], scales [B*H][N][D/32]
  const uint8_t* qs;
  const uint8_t* k;    // MXFP4 along D [B*Hkv][N][D/2]
  const uint8_t* ks;
  const uint8_t* q8;   // MXFP8 along queries [B*H][D][N], scales [B*H][D][N/32]
  const uint8_t* q8s;
  const uint8_t* k8;   // MXFP8 along keys [B*Hkv][D][N]
  const uint8_t* k8s;
  const uint8_t* v8;   // MXFP8 along D [B*Hkv][N][D], scales [B*Hkv][N][D/32]
  const uint8_t* v8s;
  const uint8_t* dod;  // dO MXFP8 along D [B*H][N][D]
  const uint8_t* dods;
  const uint8_t* doq;  // dO MXFP8 along queries [B*H][D][N]
  const uint8_t* doqs;
  const float* lse;    // [B*H][N]
  const float* delta;  // [B*H][N]
  uint16_t* dq;        // bf16 [B*H][N][D]
  uint16_t* dk;        // bf16 [B*Hkv][N][D]
  uint16_t* dv;
  int B, H, Hkv, N;
};

// ------------------------------------------------------------------------------------
// dK, dV. Workgroup: (batch, KV head, 128 keys); wave w owns keys k0 + 32w + (lane % 32).
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) dkdv_kernel(BwdArgs a) {
  constexpr int KS = D / 64;        // k-steps over D
  constexpr int DT = D / 32;        // 32-wide output tiles along D
  constexpr int QB = 64;            // queries per staged block
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr float SCALE = inv_sqrt_d(D);
  // LDS: Q rows (MXFP4) + scales, dO rows (MXFP8) + scales, Q^T and dO^T rows along queries
  // (MXFP8, 64 bytes each) + their two scale bytes, -LSE log2e and Delta.
  constexpr int oQ = 0, oQs = oQ + QB * D / 2, oDO = oQs + QB * 4, oDOs = oDO + QB * D;
  constexpr int oQT = oDOs + QB * 4, oQTs = oQT + D * QB, oDOT = oQTs + D * 4, oDOTs = oDOT + D * QB;
  constexpr int oNL = oDOTs + D * 4, oDL = oNL + QB * 4, kSmem = oDL + QB * 4;
  __shared__ __attribute__((aligned(16))) uint8_t sm[kSmem];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;
  const int ntile = (N + 127) / 128;
  const int kt = (int)blockIdx.x % ntile;
  const int bg = (int)blockIdx.x / ntile;  // b * Hkv + g
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int G = a.H / a.Hkv;
  const int k0 = kt * 128;
  const int kw0 = k0 + wave * 32;
  const int kl = kw0 + col;  // this lane's key (B operand column / A operand row)
  const bool kvalid = kl < N;
  const int64_t bhkv = (int64_t)bg;

  // this lane's K (MXFP4) and V (MXFP8) fragments: B operands of S = Q K^T and dP = dO V^T
  v8i kf[KS], vf[KS];
  uint32_t ksc = 0x7F7F7F7Fu, vsc = 0x7F7F7F7Fu;
  {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      uint4 t = make_uint4(0, 0, 0, 0), u0 = t, u1 = t;
      if (kvalid) {
        t = *reinterpret_cast<const uint4*>(a.k + (bhkv * N + kl) * (D / 2) + (2 * ks + half) * 16);
        const uint8_t* vrow = a.v8 + (bhkv * N + kl) * D + 64 * ks + half * 16;
        u0 = *reinterpret_cast<const uint4*>(vrow);
        u1 = *reinterpret_cast<const uint4*>(vrow + 32);
      }
      kf[ks][0] = t.x; kf[ks][1] = t.y; kf[ks][2] = t.z; kf[ks][3] = t.w;
      vf[ks][0] = u0.x; vf[ks][1] = u0.y; vf[ks][2] = u0.z; vf[ks][3] = u0.w;
      vf[ks][4] = u1.x; vf[ks][5] = u1.y; vf[ks][6] = u1.z; vf[ks][7] = u1.w;
    }
    if (kvalid) {
      if constexpr (D == 128) {
        ksc = *reinterpret_cast<const uint32_t*>(a.ks + (bhkv * N + kl) * 4);
        vsc = *reinterpret_cast<const uint32_t*>(a.v8s + (bhkv * N + kl) * 4);
      } else {
        ksc = *reinterpret_cast<const uint16_t*>(a.ks + (bhkv * N + kl) * 2);
        vsc = *reinterpret_cast<const uint16_t*>(a.v8s + (bhkv * N + kl) * 2);
      }
    }
    ksc >>= 8 * half;  // byte 2*ks: d-block 2*ks + half
    vsc >>= 8 * half;
  }

  v16f dvacc[DT], dkacc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) {
      dvacc[t][r] = 0.0f;
      dkacc[t][r] = 0.0f;
    }

  const int qstart = CAUSAL ? (k0 / QB) * QB : 0;
  for (int hh = 0; hh < G; hh++) {
    const int64_t bh = (int64_t)b * a.H + (int64_t)g * G + hh;
    for (int qb0 = qstart; qb0 < N; qb0 += QB) {
      // ---- stage the query block (all threads) ----
      __syncthreads();
      {
        // Q rows, MXFP4: QB x D/2 bytes
        for (int t = tid; t < QB * D / 32; t += kThreads) {
          const int r = t / (D / 32), c = t % (D / 32), q = qb0 + r;
          uint4 w = make_uint4(0, 0, 0, 0);
          if (q < N) w = *reinterpret_cast<const uint4*>(a.q + (bh * N + q) * (D / 2) + c * 16);
          *reinterpret_cast<uint4*>(sm + oQ + r * (D / 2) + c * 16) = w;
        }
        // dO rows, MXFP8: QB x D bytes
        for (int t = tid; t < QB * D / 16; t += kThreads) {
          const int r = t / (D / 16), c = t % (D / 16), q = qb0 + r;
          uint4 w = make_uint4(0, 0, 0, 0);
          if (q < N) w = *reinterpret_cast<const uint4*>(a.dod + (bh * N + q) * D + c * 16);
          *reinterpret_cast<uint4*>(sm + oDO + r * D + c * 16) = w;
        }
        // Q^T and dO^T rows along queries (MXFP8): D rows x QB bytes
        for (int t = tid; t < D * QB / 16; t += kThreads) {
          const int d = t / (QB / 16), c = t % (QB / 16), q = qb0 + c * 16;
          uint4 w1 = make_uint4(0, 0, 0, 0), w2 = w1;
          if (q < N) {
            w1 = *reinterpret_cast<const uint4*>(a.q8 + (bh * D + d) * N + q);
            w2 = *reinterpret_cast<const uint4*>(a.doq + (bh * D + d) * N + q);
          }
          *reinterpret_cast<uint4*>(sm + oQT + d * QB + c * 16) = w1;
          *reinterpret_cast<uint4*>(sm + oDOT + d * QB + c * 16) = w2;
        }
        if (tid < QB) {
          const int q = qb0 + tid;
          uint32_t s1 = 0x7F7F7F7Fu, s2 = 0x7F7F7F7Fu;
          float nl = 0.0f, dl = 0.0f;
          if (q < N) {
            if constexpr (D == 128) {
              s1 = *reinterpret_cast<const uint32_t*>(a.qs + (bh * N + q) * 4);
              s2 = *reinterpret_cast<const uint32_t*>(a.dods + (bh * N + q) * 4);
            } else {
              s1 = *reinterpret_cast<const uint16_t*>(a.qs + (bh * N + q) * 2);
              s2 = *reinterpret_cast<const uint16_t*>(a.dods + (bh * N + q) * 2);
            }
            nl = -fmul_rn(a.lse[bh * N + q], 1.44269504f);
            dl = a.delta[bh * N + q];
          }
          reinterpret_cast<uint32_t*>(sm + oQs)[tid] = s1;
          reinterpret_cast<uint32_t*>(sm + oDOs)[tid] = s2;
          reinterpret_cast<float*>(sm + oNL)[tid] = nl;
          reinterpret_cast<float*>(sm + oDL)[tid] = dl;
        }
        if (tid < D) {
          const int64_t srow = (bh * D + tid) * (N / 32) + qb0 / 32;
          const bool v1 = qb0 + 32 < N;
          const uint32_t a0 = a.q8s[srow], a1 = v1 ? a.q8s[srow + 1] : 127u;
          const uint32_t b0 = a.doqs[srow], b1 = v1 ? a.doqs[srow + 1] : 127u;
          reinterpret_cast<uint32_t*>(sm + oQTs)[tid] = a0 | (a1 << 8);
          reinterpret_cast<uint32_t*>(sm + oDOTs)[tid] = b0 | (b1 << 8);
        }
      }
      __syncthreads();
      if (CAUSAL && qb0 + QB - 1 < kw0) continue;  // every query of the block precedes every key of the wave

      // ---- S and dP tiles: lane = key kl; register i of half h = query qb0 + 32t + 16h + i ----
      v16f s[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int r = t * 32 + perm32(col);  // query row supplied by this lane as A operand
        const int qsc = (int)(reinterpret_cast<const uint32_t*>(sm + oQs)[r] >> (8 * half));
        const int dsc = (int)(reinterpret_cast<const uint32_t*>(sm + oDOs)[r] >> (8 * half));
        v16f z;
#pragma unroll
        for (int i = 0; i < 16; i++) z[i] = 0.0f;
        s[t] = z;
        dp[t] = z;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const uint4 qa = *reinterpret_cast<const uint4*>(sm + oQ + r * (D / 2) + (2 * ks + half) * 16);
          v8i af;
          af[0] = qa.x; af[1] = qa.y; af[2] = qa.z; af[3] = qa.w;
          const uint8_t* dorow = sm + oDO + r * D + 64 * ks + half * 16;
          const uint4 d0 = *reinterpret_cast<const uint4*>(dorow);
          const uint4 d1 = *reinterpret_cast<const uint4*>(dorow + 32);
          v8i bf;
          bf[0] = d0.x; bf[1] = d0.y; bf[2] = d0.z; bf[3] = d0.w;
          bf[4] = d1.x; bf[5] = d1.y; bf[6] = d1.z; bf[7] = d1.w;
          if (ks == 0) {
            s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(af, kf[0], s[t], qsc, (int)ksc);
            dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(bf, vf[0], dp[t], dsc, (int)vsc);
          } else {
            s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(af, kf[KS - 1], s[t], qsc, (int)ksc);
            dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 2, 2>(bf, vf[KS - 1], dp[t], dsc, (int)vsc);
          }
        }
      }
      // ---- P, dS; MXFP8 quantization along queries (block = one tile = lane pair) ----
      v8i pa, sa;
      int pscale[2], sscale[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int qrow0 = t * 32 + half * 16;
        float p[16], dsv[16];
        float pmax = 0.0f, smax = 0.0f;
#pragma unroll
        for (int i4 = 0; i4 < 4; i4++) {
          const float4 nl4 = reinterpret_cast<const float4*>(sm + oNL)[(qrow0 >> 2) + i4];
          const float4 dl4 = reinterpret_cast<const float4*>(sm + oDL)[(qrow0 >> 2) + i4];
          const float nlv[4] = {nl4.x, nl4.y, nl4.z, nl4.w}, dlv[4] = {dl4.x, dl4.y, dl4.z, dl4.w};
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const int i = 4 * i4 + j;
            const int q = qb0 + qrow0 + i;
            const bool vis = kvalid && q < N && (!CAUSAL || kl <= q);
            const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], C, nlv[j])) : 0.0f;
            p[i] = pv;
            dsv[i] = pv * (dp[t][i] - dlv[j]);
            pmax = fmaxf(pmax, pv);
            smax = fmaxf(smax, fabsf(dsv[i]));
          }
        }
        pmax = max_across_halves(pmax);
        smax = max_across_halves(smax);
        const int ep = mx8_exponent(pmax), es = mx8_exponent(smax);
        pscale[t] = ep + 127;
        sscale[t] = es + 127;
        const float fp = pow2_neg(ep), fs = pow2_neg(es);
#pragma unroll
        for (int w = 0; w < 4; w++) {
          pa[4 * t + w] = (int)pack4_fp8(fminf(p[4 * w] * fp, 448.0f), fminf(p[4 * w + 1] * fp, 448.0f),
                                         fminf(p[4 * w + 2] * fp, 448.0f), fminf(p[4 * w + 3] * fp, 448.0f));
          sa[4 * t + w] = (int)pack4_fp8(clamp448(dsv[4 * w] * fs), clamp448(dsv[4 * w + 1] * fs),
                                         clamp448(dsv[4 * w + 2] * fs), clamp448(dsv[4 * w + 3] * fs));
        }
      }
      // lane r supplies block 0 (queries qb0..+31, tile 0), lane r+32 block 1 (tile 1)
      const int psc = half ? pscale[1] : pscale[0];
      const int ssc = half ? sscale[1] : sscale[0];
      // ---- dV += P^T dO, dK += dS^T Q (contraction over the 64 queries) ----
#pragma unroll
      for (int t = 0; t < DT; t++) {
        const int d = t * 32 + col;
        const uint8_t* dorow = sm + oDOT + d * QB + half * 16;
        const uint8_t* qrow = sm + oQT + d * QB + half * 16;
        const uint4 a0 = *reinterpret_cast<const uint4*>(dorow), a1 = *reinterpret_cast<const uint4*>(dorow + 32);
        const uint4 b0 = *reinterpret_cast<const uint4*>(qrow), b1 = *reinterpret_cast<const uint4*>(qrow + 32);
        v8i bo, bq;
        bo[0] = a0.x; bo[1] = a0.y; bo[2] = a0.z; bo[3] = a0.w; bo[4] = a1.x; bo[5] = a1.y; bo[6] = a1.z; bo[7] = a1.w;
        bq[0] = b0.x; bq[1] = b0.y; bq[2] = b0.z; bq[3] = b0.w; bq[4] = b1.x; bq[5] = b1.y; bq[6] = b1.z; bq[7] = b1.w;
        const int dosc = (int)((reinterpret_cast<const uint32_t*>(sm + oDOTs)[d] >> (8 * half)) & 0xFFu);
        const int qtsc = (int)((reinterpret_cast<const uint32_t*>(sm + oQTs)[d] >> (8 * half)) & 0xFFu);
        dvacc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(pa, bo, dvacc[t], psc, dosc);
        dkacc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(sa, bq, dkacc[t], ssc, qtsc);
      }
    }
  }

  // ---- epilogue: row R of the output tiles is key kw0 + R, column d = 32t + lane%32 ----
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int i = 0; i < 16; i++) {
      const int key = kw0 + 8 * (i >> 2) + 4 * half + (i & 3);
      if (key < N) {
        const int64_t off = (bhkv * N + key) * D + t * 32 + col;
        a.dv[off] = (uint16_t)bf16_bits(dvacc[t][i]);
        a.dk[off] = (uint16_t)bf16_bits(dkacc[t][i] * SCALE);
      }
    }
}

// ------------------------------------------------------------------------------------
// dQ. Workgroup: (batch, query head, 128 queries); wave w owns queries q0 + 32w + lane % 32.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads) dq_kernel(BwdArgs a) {
  constexpr int KS = D / 64;
  constexpr int DT = D / 32;
  constexpr int KB = 64;
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr float SCALE = inv_sqrt_d(D);
  // LDS: K rows (MXFP4) + scales, V rows (MXFP8 along D) + scales, K^T rows along keys
  // (MXFP8, 64 bytes) + two scale bytes
  constexpr int oK = 0, oKs = oK + KB * D / 2, oV = oKs + KB * 4, oVs = oV + KB * D;
  constexpr int oKT = oVs + KB * 4, oKTs = oKT + D * KB, kSmem = oKTs + D * 4;
  __shared__ __attribute__((aligned(16))) uint8_t sm[kSmem];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;
  const int nqt = (N + 127) / 128;
  int qt = (int)blockIdx.x % nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int bh = (int)blockIdx.x / nqt;
  const int h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int q0 = qt * 128;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + col;
  const bool qvalid = qi < N;

  // this lane's Q (MXFP4) and dO (MXFP8 along D) fragments: B operands of S^T and dP^T
  v8i qf[KS], df[KS];
  uint32_t qsc = 0x7F7F7F7Fu, dsc = 0x7F7F7F7Fu;
  float nl = 0.0f, dl = 0.0f;
  {
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      uint4 t = make_uint4(0, 0, 0, 0), u0 = t, u1 = t;
      if (qvalid) {
        t = *reinterpret_cast<const uint4*>(a.q + ((int64_t)bh * N + qi) * (D / 2) + (2 * ks + half) * 16);
        const uint8_t* drow = a.dod + ((int64_t)bh * N + qi) * D + 64 * ks + half * 16;
        u0 = *reinterpret_cast<const uint4*>(drow);
        u1 = *reinterpret_cast<const uint4*>(drow + 32);
      }
      qf[ks][0] = t.x; qf[ks][1] = t.y; qf[ks][2] = t.z; qf[ks][3] = t.w;
      df[ks][0] = u0.x; df[ks][1] = u0.y; df[ks][2] = u0.z; df[ks][3] = u0.w;
      df[ks][4] = u1.x; df[ks][5] = u1.y; df[ks][6] = u1.z; df[ks][7] = u1.w;
    }
    if (qvalid) {
      if constexpr (D == 128) {
        qsc = *reinterpret_cast<const uint32_t*>(a.qs + ((int64_t)bh * N + qi) * 4);
        dsc = *reinterpret_cast<const uint32_t*>(a.dods + ((int64_t)bh * N + qi) * 4);
      } else {
        qsc = *reinterpret_cast<const uint16_t*>(a.qs + ((int64_t)bh * N + qi) * 2);
        dsc = *reinterpret_cast<const uint16_t*>(a.dods + ((int64_t)bh * N + qi) * 2);
      }
      nl = -fmul_rn(a.lse[(int64_t)bh * N + qi], 1.44269504f);
      dl = a.delta[(int64_t)bh * N + qi];
    }
    qsc >>= 8 * half;
    dsc >>= 8 * half;
  }

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;

  const int kend = CAUSAL ? min(N, q0 + 128) : N;
  for (int kb0 = 0; kb0 < kend; kb0 += KB) {
    __syncthreads();
    {
      for (int t = tid; t < KB * D / 32; t += kThreads) {
        const int r = t / (D / 32), c = t % (D / 32), kk = kb0 + r;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (kk < N) w = *reinterpret_cast<const uint4*>(a.k + (bhkv * N + kk) * (D / 2) + c * 16);
        *reinterpret_cast<uint4*>(sm + oK + r * (D / 2) + c * 16) = w;
      }
      for (int t = tid; t < KB * D / 16; t += kThreads) {
        const int r = t / (D / 16), c = t % (D / 16), kk = kb0 + r;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (kk < N) w = *reinterpret_cast<const uint4*>(a.v8 + (bhkv * N + kk) * D + c * 16);
        *reinterpret_cast<uint4*>(sm + oV + r * D + c * 16) = w;
      }
      for (int t = tid; t < D * KB / 16; t += kThreads) {
        const int d = t / (KB / 16), c = t % (KB / 16), kk = kb0 + c * 16;
        uint4 w = make_uint4(0, 0, 0, 0);
        if (kk < N) w = *reinterpret_cast<const uint4*>(a.k8 + (bhkv * D + d) * N + kk);
        *reinterpret_cast<uint4*>(sm + oKT + d * KB + c * 16) = w;
      }
      if (tid < KB) {
        const int kk = kb0 + tid;
        uint32_t s1 = 0x7F7F7F7Fu, s2 = 0x7F7F7F7Fu;
        if (kk < N) {
          if constexpr (D == 128) {
            s1 = *reinterpret_cast<const uint32_t*>(a.ks + (bhkv * N + kk) * 4);
            s2 = *reinterpret_cast<const uint32_t*>(a.v8s + (bhkv * N + kk) * 4);
          } else {
            s1 = *reinterpret_cast<const uint16_t*>(a.ks + (bhkv * N + kk) * 2);
            s2 = *reinterpret_cast<const uint16_t*>(a.v8s + (bhkv * N + kk) * 2);
          }
        }
        reinterpret_cast<uint32_t*>(sm + oKs)[tid] = s1;
        reinterpret_cast<uint32_t*>(sm + oVs)[tid] = s2;
      }
      if (tid < D) {
        const int64_t srow = (bhkv * D + tid) * (N / 32) + kb0 / 32;
        const uint32_t s0 = a.k8s[srow], s1 = (kb0 + 32 < N) ? a.k8s[srow + 1] : 127u;
        reinterpret_cast<uint32_t*>(sm + oKTs)[tid] = s0 | (s1 << 8);
      }
    }
    __syncthreads();
    if (CAUSAL && kb0 > qw0 + 31) continue;  // every key of the block follows every query of the wave

    // ---- S^T, dP^T: lane = query qi; register i of tile t = key kb0 + 32 half + 16 t + i ----
    v16f s[2], dp[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int key = (((col >> 2) & 1) << 5) + t * 16 + ((col >> 3) << 2) + (col & 3);
      const int ksc = (int)(reinterpret_cast<const uint32_t*>(sm + oKs)[key] >> (8 * half));
      const int vsc = (int)(reinterpret_cast<const uint32_t*>(sm + oVs)[key] >> (8 * half));
      v16f z;
#pragma unroll
      for (int i = 0; i < 16; i++) z[i] = 0.0f;
      s[t] = z;
      dp[t] = z;
#pragma unroll
      for (int ks = 0; ks < KS; ks++) {
        const uint4 kk = *reinterpret_cast<const uint4*>(sm + oK + key * (D / 2) + (2 * ks + half) * 16);
        v8i af;
        af[0] = kk.x; af[1] = kk.y; af[2] = kk.z; af[3] = kk.w;
        const uint8_t* vrow = sm + oV + key * D + 64 * ks + half * 16;
        const uint4 v0 = *reinterpret_cast<const uint4*>(vrow), v1 = *reinterpret_cast<const uint4*>(vrow + 32);
        v8i vf;
        vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w; vf[4] = v1.x; vf[5] = v1.y; vf[6] = v1.z; vf[7] = v1.w;
        if (ks == 0) {
          s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(af, qf[0], s[t], ksc, (int)qsc);
          dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(vf, df[0], dp[t], vsc, (int)dsc);
        } else {
          s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(af, qf[KS - 1], s[t], ksc, (int)qsc);
          dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 2, 2>(vf, df[KS - 1], dp[t], vsc, (int)dsc);
        }
      }
    }
    // ---- dS, MXFP8 along keys: the lane's 32 keys are one block ----
    float dsv[32];
    float smax = 0.0f;
#pragma unroll
    for (int idx = 0; idx < 32; idx++) {
      const int t = idx >> 4, i = idx & 15;
      const int key = kb0 + half * 32 + idx;
      const bool vis = qvalid && key < N && (!CAUSAL || key <= qi);
      const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], C, nl)) : 0.0f;
      dsv[idx] = pv * (dp[t][i] - dl);
      smax = fmaxf(smax, fabsf(dsv[idx]));
    }
    const int es = mx8_exponent(smax);
    const float fs = pow2_neg(es);
    uint32_t pw[8];
#pragma unroll
    for (int w = 0; w < 8; w++)
      pw[w] = pack4_fp8(clamp448(dsv[4 * w] * fs), clamp448(dsv[4 * w + 1] * fs), clamp448(dsv[4 * w + 2] * fs),
                        clamp448(dsv[4 * w + 3] * fs));
#pragma unroll
    for (int w = 0; w < 4; w++) permlane32_swap(pw[w], pw[w + 4]);
    v8i sb;
#pragma unroll
    for (int w = 0; w < 8; w++) sb[w] = (int)pw[w];
    const int ssc = es + 127;
    // ---- dQ^T += K^T dS^T (contraction over the 64 keys) ----
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const int d = t * 32 + col;
      const uint8_t* krow = sm + oKT + d * KB + half * 16;
      const uint4 a0 = *reinterpret_cast<const uint4*>(krow), a1 = *reinterpret_cast<const uint4*>(krow + 32);
      v8i kfr;
      kfr[0] = a0.x; kfr[1] = a0.y; kfr[2] = a0.z; kfr[3] = a0.w; kfr[4] = a1.x; kfr[5] = a1.y; kfr[6] = a1.z; kfr[7] = a1.w;
      const int ktsc = (int)((reinterpret_cast<const uint32_t*>(sm + oKTs)[d] >> (8 * half)) & 0xFFu);
      acc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(kfr, sb, acc[t], ktsc, ssc);
    }
  }

  if (qvalid) {
    uint16_t* orow = a.dq + ((int64_t)bh * N + qi) * D;
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int aa = 0; aa < 4; aa++) {
        const int d0 = t * 32 + 8 * aa + 4 * half;
        uint2 w;
        w.x = bf16_bits(acc[t][4 * aa + 0] * SCALE) | (bf16_bits(acc[t][4 * aa + 1] * SCALE) << 16);
        w.y = bf16_bits(acc[t][4 * aa + 2] * SCALE) | (bf16_bits(acc[t][4 * aa + 3] * SCALE) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
  }
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int ntile = (a.N + 127) / 128;
  dkdv_kernel<D, CAUSAL><<<dim3((unsigned)(ntile * a.B * a.Hkv)), dim3(kThreads), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dq_kernel<D, CAUSAL><<<dim3((unsigned)(ntile * a.B * a.H)), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
  const int64_t rows = B * H * N;
  // Delta (fp32) + dO MXFP8 along D (codes + scales) + dO MXFP8 along queries (codes + scales),
  // each region padded to 256 bytes
  auto pad = [](int64_t x) { return (x + 255) / 256 * 256; };
  return (size_t)(pad(rows * 4) + 2 * (pad(rows * D) + pad(rows * D / 32)));
}

hipError_t launch_attn_bwd(const BwdLaunch& l, int D, int causal, hipStream_t stream) {
  const int64_t rows = (int64_t)l.B * l.H * l.N;
  auto pad = [](int64_t x) { return (x + 255) / 256 * 256; };
  uint8_t* ws = (uint8_t*)l.workspace;
  float* delta = (float*)ws;
  uint8_t* dod = ws + pad(rows * 4);
  uint8_t* dods = dod + pad(rows * D);
  uint8_t* doq = dods + pad(rows * D / 32);
  uint8_t* doqs = doq + pad(rows * D);
  // Delta
  {
    const int64_t threads = rows * (D / 8);
    const unsigned blocks = (unsigned)((threads + kThreads - 1) / kThreads);
    if (D == 128) delta_kernel<128><<<blocks, kThreads, 0, stream>>>(l.o, l.dout, delta, rows);
    else delta_kernel<64><<<blocks, kThreads, 0, stream>>>(l.o, l.dout, delta, rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  // dO's two MXFP8 views
  hipError_t e = launch_quantize(l.dout, dod, dods, kMXFP8, kAlongD, (int64_t)l.B * l.H, l.N, D, stream);
  if (e != hipSuccess) return e;
  e = launch_quantize(l.dout, doq, doqs, kMXFP8, kAlongSeq, (int64_t)l.B * l.H, l.N, D, stream);
  if (e != hipSuccess) return e;
  BwdArgs a;
  a.q = l.q; a.qs = l.qs; a.k = l.k; a.ks = l.ks;
  a.q8 = l.q8; a.q8s = l.q8s; a.k8 = l.k8; a.k8s = l.k8s; a.v8 = l.v8; a.v8s = l.v8s;
  a.dod = dod; a.dods = dods; a.doq = doq; a.doqs = doqs;
  a.lse = l.lse; a.delta = delta; a.dq = l.dq; a.dk = l.dk; a.dv = l.dv;
  a.B = l.B; a.H = l.H; a.Hkv = l.Hkv; a.N = l.N;
  if (D == 128) return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
  return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
}

}  // namespace fp4attn

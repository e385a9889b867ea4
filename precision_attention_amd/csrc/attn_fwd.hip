// attn_fwd.hip -- FP4 attention forward on the block-scaled MFMA of gfx950.
//
// Two routes of "Hardware-Aware FP4 FlashAttention-4" (gist.science technical summary,
// Methodology 1 and 2; arXiv abstract):
//  - Direct-P (noncausal inference): MXFP4 Q/K/V; scores are mapped straight to E2M1
//    probability codes with one E8M0 scale per 32 keys; the normalizer is accumulated from
//    the same represented values the P.V product consumes ("Consistent Normalization").
//  - Causal training forward: MXFP4 Q/K (the saved state), FP8 (E4M3) P and V.
//
// Per 32-key block b of one query row, with running max m and c = log2(e)/sqrt(D):
//   e_b = max(floor(fp32(fp32(S_bmax - m) * c)) - emax, -127)     emax = 2 (E2M1) or 8 (E4M3)
//   u_j = fmaf(S_j, c, fp32(-fp32(m * c) - e_b))
//   P_j = RNE(2^u_j) on the element grid, scale 2^e_b
// The class boundaries of the Direct-P classification are the step points of RNE(2^u), so
// evaluating 2^u with the hardware exponential and rounding with the hardware converter
// realizes it ("selective native exponentials"); only scores within an ulp of a step point
// can land in the neighbouring class.
//
// Mapping onto the MI355X:
//  - workgroup = 4 waves = 128 queries of one (batch, head); each wave owns 32 queries.
//  - S^T = K Q^T on the 32x32x64 FP4 MFMA, so lane l holds query l%32 and, after permuting
//    the K rows at load time, the 32 consecutive keys of one P block in order; the block max
//    is an in-lane reduction and the row max needs one permlane32 swap.
//  - O^T = V^T P^T on the 32x32x64 MFMA (FP4 or FP8): the query stays in the lane, so the
//    running max, the rescale factor and the normalizer are per-lane scalars.
//  - l comes from one more MFMA with an all-ones V^T tile: the exact sum of the represented
//    probabilities, at 1/8 (D=128) of the P.V cost and no VALU work.
//  - K and V^T tiles of 64 keys are double-buffered in LDS with XOR-swizzled 16-byte chunks
//    (conflict-free fragment reads); the next block's global loads are in flight during the
//    current block's math.
//  - workgroups are numbered so that the query tiles of one head land on the same XCD
//    (shared L2 for that head's K and V).
#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

template <int D, bool FP8V>
struct FwdSmem {
  static constexpr int kRow = D / 2;                          // bytes of one MXFP4 K row
  static constexpr int kCh = D / 32;                          // 16-byte chunks per K row
  static constexpr int vRow = FP8V ? kKeyBlock : kKeyBlock / 2;  // bytes of one V^T row per block
  static constexpr int vCh = vRow / 16;                       // 16-byte chunks per V^T row
  static constexpr int vKeysPerCh = FP8V ? 16 : 32;
  static constexpr int ksOff = kKeyBlock * kRow;              // one dword of scales per key
  static constexpr int vOff = ksOff + kKeyBlock * 4;
  static constexpr int vsOff = vOff + D * vRow;               // two scale bytes per V^T row
  static constexpr int buf = vsOff + D * 2;
  static constexpr int vLoads = (D * vCh + kThreads - 1) / kThreads;
};

// XOR swizzles of 16-byte chunks; see the bank analysis in the design notes: with these,
// the 16 lanes of each ds_read_b128 phase touch 16 distinct bank groups.
template <int D>
__device__ __forceinline__ int k_chunk(int key, int c) {
  if constexpr (D == 128) return c ^ (((key >> 2) & 1) | (((key >> 5) & 1) << 1));
  else return c ^ ((key >> 5) & 1);
}
template <bool FP8V>
__device__ __forceinline__ int v_chunk(int d, int c) {
  if constexpr (FP8V) return c ^ ((d >> 2) & 3);
  else return c ^ ((d >> 3) & 1);
}

__device__ __forceinline__ uint32_t bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_kernel(FwdArgs a) {
  constexpr bool FP8V = CAUSAL;
  using L = FwdSmem<D, FP8V>;
  constexpr int DT = D / 32;          // 32-wide output tiles along D
  constexpr float EMAX = FP8V ? 8.0f : 2.0f;
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr int PF = FP8V ? kFmtFP8 : kFmtFP4;
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::buf];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;

  // ---- workgroup -> (batch*head, query tile), grouping each head's tiles on one XCD ----
  const int nqt = (N + kQueryTile - 1) / kQueryTile;
  const int total = (int)gridDim.x;
  const int per = total / 8, rem = total % 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  int qt = lin % nqt;
  if (CAUSAL) qt = nqt - 1 - qt;  // longest causal rows first
  const int bh = lin / nqt;
  const int h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int qrow0 = qt * kQueryTile;
  const int qwave0 = qrow0 + wave * 32;
  const int qi = qwave0 + col;
  const bool qvalid = qi < N;

  // ---- this lane's Q fragment (B operand of S^T = K Q^T): query qi, d-block 2*ks + half ----
  v8i qf0, qf1;
  uint32_t qsc;
  {
    uint4 t0 = make_uint4(0, 0, 0, 0), t1 = make_uint4(0, 0, 0, 0);
    uint32_t w = 0x7F7F7F7Fu;
    if (qvalid) {
      const uint8_t* qrow = a.q + ((int64_t)bh * N + qi) * (D / 2);
      t0 = *reinterpret_cast<const uint4*>(qrow + half * 16);
      if constexpr (D == 128) {
        t1 = *reinterpret_cast<const uint4*>(qrow + (2 + half) * 16);
        w = *reinterpret_cast<const uint32_t*>(a.qs + ((int64_t)bh * N + qi) * 4);
      } else {
        w = *reinterpret_cast<const uint16_t*>(a.qs + ((int64_t)bh * N + qi) * 2);
      }
    }
    qf0[0] = t0.x; qf0[1] = t0.y; qf0[2] = t0.z; qf0[3] = t0.w;
    qf1[0] = t1.x; qf1[1] = t1.y; qf1[2] = t1.z; qf1[3] = t1.w;
    qsc = w >> (8 * half);  // byte 2*ks of qsc is this lane's d-block 2*ks + half
  }

  const int kend = CAUSAL ? min(N, qrow0 + kQueryTile) : N;
  const int nkb = (kend + kKeyBlock - 1) / kKeyBlock;
  const int64_t vrow_bytes = FP8V ? (int64_t)N : (int64_t)N / 2;

  // ---- global -> register staging of one key block, then register -> LDS ----
  uint4 st_k = make_uint4(0, 0, 0, 0);
  uint32_t st_ks = 0, st_vs = 0;
  uint4 st_v[L::vLoads];
  auto load_stage = [&](int j) {
    const int kb0 = j * kKeyBlock;
    if (tid < kKeyBlock * L::kCh) {
      const int key = tid / L::kCh, c = tid % L::kCh, gk = kb0 + key;
      st_k = gk < N ? *reinterpret_cast<const uint4*>(a.k + (bhkv * N + gk) * (D / 2) + c * 16)
                    : make_uint4(0, 0, 0, 0);
    }
    if (tid < kKeyBlock) {
      const int gk = kb0 + tid;
      if constexpr (D == 128)
        st_ks = gk < N ? *reinterpret_cast<const uint32_t*>(a.ks + (bhkv * N + gk) * 4) : 0x7F7F7F7Fu;
      else
        st_ks = gk < N ? (uint32_t)*reinterpret_cast<const uint16_t*>(a.ks + (bhkv * N + gk) * 2) : 0x7F7Fu;
    }
#pragma unroll
    for (int u = 0; u < L::vLoads; u++) {
      const int t = tid + u * kThreads;
      if (t < D * L::vCh) {
        const int d = t / L::vCh, c = t % L::vCh;
        const int64_t off = (bhkv * D + d) * vrow_bytes + (FP8V ? kb0 : kb0 / 2) + c * 16;
        st_v[u] = (kb0 + c * L::vKeysPerCh < N) ? *reinterpret_cast<const uint4*>(a.v + off) : make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < D) {
      const int64_t srow = (bhkv * D + tid) * (N / 32) + kb0 / 32;
      const uint32_t lo = kb0 < N ? a.vs[srow] : 127u;
      const uint32_t hi = kb0 + 32 < N ? a.vs[srow + 1] : 127u;
      st_vs = lo | (hi << 8);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* sb = smem + buf * L::buf;
    if (tid < kKeyBlock * L::kCh) {
      const int key = tid / L::kCh, c = tid % L::kCh;
      *reinterpret_cast<uint4*>(sb + key * L::kRow + k_chunk<D>(key, c) * 16) = st_k;
    }
    if (tid < kKeyBlock) reinterpret_cast<uint32_t*>(sb + L::ksOff)[tid] = st_ks;
#pragma unroll
    for (int u = 0; u < L::vLoads; u++) {
      const int t = tid + u * kThreads;
      if (t < D * L::vCh) {
        const int d = t / L::vCh, c = t % L::vCh;
        *reinterpret_cast<uint4*>(sb + L::vOff + d * L::vRow + v_chunk<FP8V>(d, c) * 16) = st_v[u];
      }
    }
    if (tid < D) reinterpret_cast<uint16_t*>(sb + L::vsOff)[tid] = (uint16_t)st_vs;
  };

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;
  v16f accl;
#pragma unroll
  for (int r = 0; r < 16; r++) accl[r] = 0.0f;
  float m_run = -INFINITY;

  v8i ones;
#pragma unroll
  for (int r = 0; r < 8; r++) ones[r] = FP8V ? 0x38383838 : 0x22222222;  // E4M3 / E2M1 value 1.0

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int j = 0; j < nkb; j++) {
    const int kb0 = j * kKeyBlock;
    if (j + 1 < nkb) load_stage(j + 1);
    const uint8_t* sb = smem + (j & 1) * L::buf;
    const bool wave_active = !CAUSAL || kb0 <= qwave0 + 31;
    if (wave_active) {
      // ---- S^T tiles: lane holds keys kb0 + half*32 + t*16 + i (i = register) for query qi ----
      v16f s[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int key = (((col >> 2) & 1) << 5) + t * 16 + ((col >> 3) << 2) + (col & 3);
        const int ksc = (int)(reinterpret_cast<const uint32_t*>(sb + L::ksOff)[key] >> (8 * half));
        const uint4 k0 = *reinterpret_cast<const uint4*>(sb + key * L::kRow + k_chunk<D>(key, half) * 16);
        v8i kf;
        kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w;
        v16f z;
#pragma unroll
        for (int r = 0; r < 16; r++) z[r] = 0.0f;
        s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(kf, qf0, z, ksc, (int)qsc);
        if constexpr (D == 128) {
          const uint4 k1 = *reinterpret_cast<const uint4*>(sb + key * L::kRow + k_chunk<D>(key, 2 + half) * 16);
          kf[0] = k1.x; kf[1] = k1.y; kf[2] = k1.z; kf[3] = k1.w;
          s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(kf, qf1, s[t], ksc, (int)qsc);
        }
      }
      // ---- masks: keys past N, and the causal diagonal ----
      const bool need_mask = (kb0 + kKeyBlock > N) || (CAUSAL && kb0 + kKeyBlock - 1 > qwave0);
      if (need_mask) {
#pragma unroll
        for (int t = 0; t < 2; t++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int key = kb0 + half * 32 + t * 16 + i;
            const bool vis = key < N && (!CAUSAL || key <= qi);
            s[t][i] = vis ? s[t][i] : -INFINITY;
          }
      }
      // ---- block max (32 keys in-lane), row max over the key block, running max ----
      float bmax = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; i++) bmax = fmaxf(bmax, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; i++) bmax = fmaxf(bmax, s[1][i]);
      const float m_new = fmaxf(m_run, max_across_halves(bmax));
      if (__any(m_new > m_run)) {
        const float alpha = __builtin_amdgcn_exp2f(fmul_rn(fsub_rn(m_run, m_new), C));
#pragma unroll
        for (int t = 0; t < DT; t++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[t][r] *= alpha;
        accl[0] *= alpha;
      }
      m_run = m_new;
      // ---- probability codes of this lane's 32-key block ----
      const float d2 = fmul_rn(fsub_rn(bmax, m_new), C);
      const float ebf = fmaxf(floorf(d2) - EMAX, -127.0f);
      const float off = fsub_rn(-fmul_rn(m_new, C), ebf);
      const int psc = (int)ebf + 127;
      v8i pf;
      if constexpr (!FP8V) {
#pragma unroll
        for (int w = 0; w < 4; w++) {
          float x[8];
#pragma unroll
          for (int jj = 0; jj < 8; jj++) {
            const int idx = 8 * w + jj;
            x[jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[idx >> 4][idx & 15], C, off));
          }
          pf[w] = (int)pack8_fp4(x);
        }
      } else {
        uint32_t pw[8];
#pragma unroll
        for (int w = 0; w < 8; w++) {
          float x[4];
#pragma unroll
          for (int jj = 0; jj < 4; jj++) {
            const int idx = 4 * w + jj;
            x[jj] = fminf(__builtin_amdgcn_exp2f(__builtin_fmaf(s[idx >> 4][idx & 15], C, off)), 448.0f);
          }
          pw[w] = pack4_fp8(x[0], x[1], x[2], x[3]);
        }
        // FP8 operand: bytes 0-15 of lanes r, r+32 are scale block 0, bytes 16-31 block 1.
#pragma unroll
        for (int w = 0; w < 4; w++) permlane32_swap(pw[w], pw[w + 4]);
#pragma unroll
        for (int w = 0; w < 8; w++) pf[w] = (int)pw[w];
      }
      // ---- O^T += V^T P^T, l += 1^T P^T ----
#pragma unroll
      for (int t = 0; t < DT; t++) {
        const int d = t * 32 + col;
        const uint8_t* vrow = sb + L::vOff + d * L::vRow;
        v8i vf;
        const uint4 v0 = *reinterpret_cast<const uint4*>(vrow + v_chunk<FP8V>(d, half) * 16);
        vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w;
        if constexpr (FP8V) {
          const uint4 v1 = *reinterpret_cast<const uint4*>(vrow + v_chunk<FP8V>(d, 2 + half) * 16);
          vf[4] = v1.x; vf[5] = v1.y; vf[6] = v1.z; vf[7] = v1.w;
        }
        const int vsc = sb[L::vsOff + d * 2 + half];
        acc[t] = mfma_scaled<PF, PF, 0, 0>(vf, pf, acc[t], vsc, psc);
      }
      accl = mfma_scaled<PF, PF, 0, 0>(ones, pf, accl, 127, psc);
    }
    if (j + 1 < nkb) store_stage((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l in bf16, LSE = m / sqrt(D) + ln(l) ----
  if (qvalid) {
    const float l = accl[0];
    const float inv = 1.0f / l;
    uint16_t* orow = a.o + ((int64_t)bh * N + qi) * D;
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int aa = 0; aa < 4; aa++) {
        const int d0 = t * 32 + 8 * aa + 4 * half;
        uint2 w;
        w.x = bf16_rne(acc[t][4 * aa + 0] * inv) | (bf16_rne(acc[t][4 * aa + 1] * inv) << 16);
        w.y = bf16_rne(acc[t][4 * aa + 2] * inv) | (bf16_rne(acc[t][4 * aa + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(orow + d0) = w;
      }
    if (half == 0) a.lse[(int64_t)bh * N + qi] = m_run * inv_sqrt_d(D) + __builtin_amdgcn_logf(l) * 0.69314718f;
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdArgs& a, int D, int causal, hipStream_t stream) {
  const int nqt = (a.N + kQueryTile - 1) / kQueryTile;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(kThreads);
  if (D == 128) {
    if (causal) attn_fwd_kernel<128, true><<<grid, block, 0, stream>>>(a);
    else attn_fwd_kernel<128, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (causal) attn_fwd_kernel<64, true><<<grid, block, 0, stream>>>(a);
    else attn_fwd_kernel<64, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fp4attn

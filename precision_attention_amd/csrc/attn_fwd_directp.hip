// attn_fwd_directp.hip -- noncausal Direct-P forward ("Hardware-Aware FP4 FlashAttention-4",
// gist.science technical summary, Methodology 1 "Direct Mapping" and "Consistent
// Normalization"; arXiv abstract), as a two-group ping-pong on gfx950.
//
// Semantics (one query row, running max m, c = log2(e)/sqrt(D), key blocks of KB keys):
//   m_new = max(m, block max); O, l *= 2^((m - m_new) c)
//   per 32-key block b: e_b = max(floor(fp32(fp32(S_bmax - m_new) c)) - 2, -127)
//                       u_j = fmaf(S_j, c, fp32(-fp32(m_new c) - e_b))
//                       P_j = RNE_E2M1(2^u_j) * 2^e_b        (the step points of RNE(2^u) are
//                       the class boundaries of the Direct-P classification)
//   O += P V, l += sum_j P_j (the same represented values), O /= l at the end.
//
// Mapping: workgroup = 8 waves x 32 queries of one (batch, head). S^T = K Q^T on the 32x32x64
// FP4 MFMA puts one query in each lane and, with K rows permuted at load time, the 32 keys of
// one P block in the registers of one lane half; O^T = V^T P^T keeps the query in the lane, and
// l is one more MFMA against an all-ones tile.
//
// Ping-pong: waves 0-3 (group X) and 4-7 (group Y) share the four SIMDs pairwise. Every wave
// alternates a matrix phase M_k (S of block k, then P.V of block k-1: MFMA only) and a vector
// phase V_k (max, rescale and the E2M1 codes of block k: VALU only). Group Y runs one phase
// behind group X and a workgroup barrier closes every phase, so on each SIMD one wave keeps the
// matrix core busy while the other keeps the vector ALU busy:
//   phase:  0     1     2     3     4    ...
//   X:      M0    V0    M1    V1    M2
//   Y:      -     M0    V0    M1    V1
// LDS stage s (buffer s % 2) holds K of block s and V of block s-1, exactly what M_s reads; stage
// s+1 is loaded directly from global memory during phases 2s and 2s+1.
#include "fwd_common.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

using namespace fwd;

constexpr int kPPWaves = 8;
constexpr int kPPThreads = 64 * kPPWaves;
constexpr int kPPQueryTile = 32 * kPPWaves;

template <int D>
__global__ void __launch_bounds__(kPPThreads, 2) attn_fwd_directp_kernel(FwdArgs a) {
  using L = Smem<D, false>;
  constexpr int KB = L::KB, NSB = L::NSB;
  constexpr int DT = D / 32;
  constexpr float C = log2e_over_sqrt_d(D);
  // the two LDS buffers as distinct objects, so the compiler can see that the DMA into one
  // never aliases the fragment reads from the other
  __shared__ __attribute__((aligned(16))) lds_char smem0[L::buf];
  __shared__ __attribute__((aligned(16))) lds_char smem1[L::buf];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);  // 0: X, 1: Y (wave-uniform)
  const int N = a.N;
  const Tile tl = tile_of_block(N, false, kPPQueryTile);
  const int bh = tl.bh, h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int qi = tl.qt * kPPQueryTile + wave * 32 + col;
  const bool qvalid = qi < N;
  v8i qf0, qf1;
  const uint32_t qsc = load_q_fragment<D>(a, bh, qi, qvalid, half, qf0, qf1);
  const KVStager<D, false, kWaves, true> st(a, bhkv, wave & 3, lane);  // used by group X only
  const int nkb = (N + KB - 1) / KB;

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

  v16f s[2 * NSB];  // S^T tiles of the current block: tile 2q+t holds keys 64q + 32*half + 16t + i
  v8i pf[NSB];      // E2M1 codes of the current block (one 32-key block per lane half)
  int psc[NSB];     // their E8M0 scales
  float m_run = -INFINITY;

  // A-operand row of this lane inside a 64-key sub-block, and the lane's LDS fragment offsets.
  // Adding 16 or 64 to a key leaves bits 2 and 5 (the K swizzle inputs) unchanged, and adding
  // 32 to d leaves bits 2-3 (the V swizzle inputs) unchanged, so every fragment of a phase is one
  // of these bases plus a compile-time offset.
  const int krow = (((col >> 2) & 1) << 5) + ((col >> 3) << 2) + (col & 3);
  const int kb_lo = krow * L::kRow + k_chunk<D>(krow, half) * 16;
  const int kb_hi = krow * L::kRow + k_chunk<D>(krow, 2 + half) * 16;
  const int ks_base = D == 128 ? L::ksOff + krow * 4 : L::ksOff + (2 * krow + half) * 4;
  int vb[NSB];
#pragma unroll
  for (int q = 0; q < NSB; q++) vb[q] = L::vOff + col * L::vRow + v_chunk<L::vCh>(col, 2 * q + half) * 16;
  const int vs_base = L::vsOff + (col * L::vsRow + half) * 4;

  // ---- M_k: S of block k (k < nkb) and P.V of block k-1 (k >= 1), all from stage k ----
  auto matrix_phase = [&](const lds_char* sb, bool do_s, bool do_pv) __attribute__((always_inline)) {
    if (do_s) {
#pragma unroll
      for (int ti = 0; ti < 2 * NSB; ti++) {
        const int koff = ((ti >> 1) * 64 + 16 * (ti & 1));  // key offset of this tile
        const uint32_t ksw = *reinterpret_cast<const lds_u32*>(sb + ks_base + koff * 4 * L::ksPerKey);
        const int ksc = D == 128 ? (int)(ksw >> (8 * half)) : (int)ksw;
        const uint4 k0 = *reinterpret_cast<const uint4*>(sb + kb_lo + koff * L::kRow);
        v8i kf;
        kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w;
        v16f z;
#pragma unroll
        for (int r = 0; r < 16; r++) z[r] = 0.0f;
        s[ti] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(kf, qf0, z, ksc, (int)qsc);
        if constexpr (D == 128) {
          const uint4 k1 = *reinterpret_cast<const uint4*>(sb + kb_hi + koff * L::kRow);
          kf[0] = k1.x; kf[1] = k1.y; kf[2] = k1.z; kf[3] = k1.w;
          s[ti] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(kf, qf1, s[ti], ksc, (int)qsc);
        }
      }
    }
    if (do_pv) {
#pragma unroll
      for (int q = 0; q < NSB; q++) {
#pragma unroll
        for (int t = 0; t < DT; t++) {
          const uint4 v0 = *reinterpret_cast<const uint4*>(sb + vb[q] + t * 32 * L::vRow);
          v8i vf;
          vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w;
          const int vsc = (int)*reinterpret_cast<const lds_u32*>(sb + vs_base + (t * 32 * L::vsRow + 2 * q) * 4);
          acc[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(vf, pf[q], acc[t], vsc, psc[q]);
        }
        accl = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(ones, pf[q], accl, 127, psc[q]);
      }
    }
  };

  // ---- V_k: mask, block maxima, running max, rescale, E2M1 codes of block k ----
  auto vector_phase = [&](int k) __attribute__((always_inline)) {
    const int kb0 = k * KB;
    if (kb0 + KB > N) {
#pragma unroll
      for (int ti = 0; ti < 2 * NSB; ti++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = kb0 + (ti >> 1) * 64 + half * 32 + (ti & 1) * 16 + i;
          s[ti][i] = key < N ? s[ti][i] : -INFINITY;
        }
    }
    float bmax[NSB];
#pragma unroll
    for (int q = 0; q < NSB; q++) bmax[q] = max32(s[2 * q], s[2 * q + 1]);
    float mloc = bmax[0];
#pragma unroll
    for (int q = 1; q < NSB; q++) mloc = __builtin_elementwise_maximum(mloc, bmax[q]);
    const float m_new = __builtin_elementwise_maximum(m_run, max_across_halves(mloc));
    // rescale O and l when some row's max grew (not on the first block: they are still 0)
    if (k > 0 && __any(m_new > m_run)) {
      const float alpha = __builtin_amdgcn_exp2f(fmul_rn(fsub_rn(m_run, m_new), C));
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[t][r] *= alpha;
      accl[0] *= alpha;
    }
    m_run = m_new;
    const float mc = fmul_rn(m_new, C);
#pragma unroll
    for (int q = 0; q < NSB; q++) {
      const float d2 = fmul_rn(fsub_rn(bmax[q], m_new), C);
      const float ebf = fmaxf(floorf(d2) - 2.0f, -127.0f);
      const float off = fsub_rn(-mc, ebf);
      psc[q] = (int)ebf + 127;
#pragma unroll
      for (int w = 0; w < 4; w++) {
        float x[8];
#pragma unroll
        for (int jj = 0; jj < 8; jj++) {
          const int idx = 8 * w + jj;
          x[jj] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[2 * q + (idx >> 4)][idx & 15], C, off));
        }
        // every byte of the destination is written, so its initial value is irrelevant
        uint32_t u = __float_as_uint(x[0]);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[0], x[1], 1.0f, 0);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[2], x[3], 1.0f, 1);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[4], x[5], 1.0f, 2);
        u = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(u, x[6], x[7], 1.0f, 3);
        pf[q][w] = (int)u;
      }
    }
  };

  // stage s: K of block s (s < nkb) and V of block s-1 (s >= 1), into buffer s % 2
  auto issue_stage = [&](int s_, lds_char* sb) __attribute__((always_inline)) {
    if (s_ < nkb) st.issue_k(s_, sb);
    if (s_ >= 1) st.issue_v(s_ - 1, sb);
  };

  // Phases 2k and 2k+1, for k = 0 .. nkb. X runs M_k in phase 2k and V_k in phase 2k+1; Y runs
  // V_{k-1} in phase 2k and M_k in phase 2k+1. Group X alone stages the K/V tiles: it issues
  // stage k+1 at the start of phase 2k (when it holds the fewest live registers) and waits for
  // it at the end of phase 2k+1. The two groups run separate loops (the barriers pair up across
  // them), each unrolled over two blocks so that every LDS buffer choice is static and the
  // compiler can see that fragment reads never alias the DMA in flight. The barriers are bare
  // s_barrier instructions: a fenced __syncthreads would also wait for the stage in flight. LDS
  // is written only by the staging DMA, whose completion X waits for explicitly before the
  // barrier that closes phase 2k+1; a buffer is overwritten only after the barrier that follows
  // its last fragment reads, and those reads have returned before the MFMAs that use them issue.
  auto pair_x = [&](auto BC, int k) __attribute__((always_inline)) {
    constexpr int B = decltype(BC)::value;  // k % 2
    if (k + 1 <= nkb) issue_stage(k + 1, B ? smem0 : smem1);
    matrix_phase(B ? smem1 : smem0, k < nkb, k >= 1);
    __builtin_amdgcn_s_barrier();  // phase switch only: publishes no LDS data
    if (k < nkb) vector_phase(k);
    wait_dma();
    __builtin_amdgcn_s_barrier();  // stage k+1 has landed in LDS
  };
  auto pair_y = [&](auto BC, int k) __attribute__((always_inline)) {
    constexpr int B = decltype(BC)::value;
    if (k >= 1) vector_phase(k - 1);
    __builtin_amdgcn_s_barrier();
    matrix_phase(B ? smem1 : smem0, k < nkb, k >= 1);
    __builtin_amdgcn_s_barrier();
  };

  if (grp == 0) {
    issue_stage(0, smem0);
    wait_dma();
  }
  __syncthreads();
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  if (grp == 0) {
    for (int k = 0; k <= nkb; k += 2) {
      pair_x(B0(), k);
      if (k + 1 <= nkb) pair_x(B1(), k + 1);
    }
  } else {
    for (int k = 0; k <= nkb; k += 2) {
      pair_y(B0(), k);
      if (k + 1 <= nkb) pair_y(B1(), k + 1);
    }
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

hipError_t launch_attn_fwd_directp(const FwdArgs& a, int D, hipStream_t stream) {
  const int nqt = (a.N + kPPQueryTile - 1) / kPPQueryTile;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(kPPThreads);
  if (D == 128) attn_fwd_directp_kernel<128><<<grid, block, 0, stream>>>(a);
  else attn_fwd_directp_kernel<64><<<grid, block, 0, stream>>>(a);
  return hipGetLastError();
}

}  // namespace fp4attn

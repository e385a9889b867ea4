// attn_fwd_directp.hip -- noncausal Direct-P forward ("Hardware-Aware FP4 FlashAttention-4",
// gist.science technical summary, Methodology 1 "Direct Mapping" and "Consistent
// Normalization"; arXiv abstract), software-pipelined for gfx950.
//
// Semantics (one query row, running max m, c = log2(e)/sqrt(D), key blocks of 128 keys):
//   m_new = max(m, block max); O, l *= 2^((m - m_new) c)
//   per 32-key block b: e_b = max(floor(fp32(fp32(S_bmax - m_new) c)) - 2, -127)
//                       u_j = fmaf(S_j, c, fp32(-fp32(m_new c) - e_b))
//                       P_j = RNE_E2M1(2^u_j) * 2^e_b        (the step points of RNE(2^u) are
//                       the class boundaries of the Direct-P classification)
//   O += P V, l += sum_j P_j (the same represented values), O /= l at the end.
//
// Mapping: workgroup = 8 waves x 32 queries of one (batch, head), one workgroup per CU (two
// waves per SIMD, sharing each staged K/V block). S^T = K Q^T on the 32x32x64 FP4 MFMA puts one
// query in each lane and, with K rows permuted at load time, the 32 keys of one P block in the
// registers of one lane half; O^T = V^T P^T keeps the query in the lane, and l is one more MFMA
// against an all-ones tile.
//
// On gfx950 one wave issues a VALU instruction only every ~6.5 cycles (measured), well below
// the VALU pipe's rate, so each wave's own VALU stream is its critical path and the MFMAs must
// run underneath it. A key block is two 64-key sub-blocks held in score tiles {0,1} and {2,3}.
// Per block j:
//   max, rescale                     (the MFMAs of the previous block finish underneath)
//   codes(j, 0)
//   codes(j, 1)  ||  PV(j, 0), S(j+1, 0) -> tiles {0,1} (free once codes(j, 0) has run)
//                    S(j+1, 1) -> tiles {2,3}, then PV(j, 1), issued at the end: the next
//                    block's max waits only for the score MFMAs, its rescale for PV(j, 1)
// K/V tiles rotate through three LDS buffers filled by direct global->LDS loads two blocks
// ahead (inline assembly, ordered by an explicit wait and a barrier per block).
//
// ANCH: Direct-P on the integer-log2 anchor (the summary's Range Guarding: an anchor taken from a
// sample of the scores). Each 32-key block is normalized by its own leading binade,
// t_b = floor(fp32(S_bmax c)): u_j = fmaf(S_j, c, 2 - t_b), P_j = RNE_E2M1(2^u_j) * 2^(t_b - 2),
// so the codes depend on no row quantity and there is no running max. The accumulators are kept
// relative to a per-query integer anchor A (P's E8M0 byte is t_b - 2 - A + 127): A is set from the
// first key block's block exponents (the sample) and moved only when a later block's t_b exceeds it
// by more than 64 binades, with an exact power-of-two rescale of O and l (the guard; a wave-uniform
// branch that ordinary inputs take once, on the first block). A block more than 125 binades below
// A is clamped to byte 0 (its weight, below 2^-120 of l, is lost). LSE = (A + log2 l) ln 2.
#include "fwd_common.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

using namespace fwd;

// Scheduling-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSgVALU = 0x002 | 0x400;  // VALU including transcendentals
constexpr int kSgMFMA = 0x008;
constexpr int kSgDSRead = 0x100;

constexpr int kDPWaves = 8;
constexpr int kDPQueryTile = 32 * kDPWaves;


template <int D, bool ANCH>
__global__ void __launch_bounds__(64 * kDPWaves, 2) attn_fwd_directp_kernel(FwdArgs a) {
  constexpr int KB = key_block_for(D);
  using L = Smem<D, false, KB>;
  constexpr int NSB = L::NSB;  // 64-key sub-blocks per key block: 2 at D=128, 1 at D=64
  static_assert(NSB == 1 || NSB == 2, "one or two 64-key sub-blocks per key block");
  constexpr int DT = D / 32;
  constexpr int KS = D / 64;  // MFMA k-steps over D
  constexpr float C = log2e_over_sqrt_d(D);
  // three rotating K/V buffers; after the loop the same memory holds the output tiles
  constexpr int kSmem = 3 * L::buf > kDPWaves * OStage<D>::kBytes ? 3 * L::buf : kDPWaves * OStage<D>::kBytes;
  __shared__ __attribute__((aligned(16))) lds_char smem[kSmem];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;
  const Tile tl = tile_of_block(N, false, kDPQueryTile);
  const int bh = tl.bh, h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int qi = tl.qt * kDPQueryTile + wave * 32 + col;
  const bool qvalid = qi < N;
  v8i qf0, qf1;
  const uint32_t qsc = load_q_fragment<D>(a, bh, qi, qvalid, half, qf0, qf1);
  const KVStager<D, false, kDPWaves, true, KB> st(a, bhkv, wave, lane);
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
  float m_run = -INFINITY;  // running max (ANCH: the integer anchor A, as a float)

  // score tiles of the current block: tile 2q+t holds keys 64q + 32*half + 16t + i (register i)
  v16f s[2 * NSB];

  // Lane-constant LDS offsets. Adding 16 or 64 to a key leaves bits 2 and 5 (the K swizzle
  // inputs) unchanged, and adding 32 to d leaves bits 2-3 (the V swizzle inputs) unchanged, so
  // every fragment is one of these bases plus a compile-time offset.
  const int krow = (((col >> 2) & 1) << 5) + ((col >> 3) << 2) + (col & 3);
  const int kb_lo = krow * L::kRow + k_chunk<D>(krow, half) * 16;
  const int kb_hi = krow * L::kRow + k_chunk<D>(krow, 2 + half) * 16;
  const int ks_base = D == 128 ? L::ksOff + ks_slot(krow) * 4 : L::ksOff + (half * KB + ks_slot(krow)) * 4;
  const int vb0 = L::vOff + col * L::vRow + v_chunk<L::vCh>(col, half) * 16;
  const int vb1 = L::vOff + col * L::vRow + v_chunk<L::vCh>(col, 2 + half) * 16;
  const int vs_base = L::vsOff + (half * D + col) * 4;

  // S^T tiles 2q, 2q+1 of the block staged at sb
  auto scores = [&](const lds_char* sb, int q) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; t++) {
      const int koff = q * 64 + 16 * t;
      const uint32_t ksw = *reinterpret_cast<const lds_u32*>(sb + ks_base + (q * 64 + 32 * t) * 4);
      const int ksc = D == 128 ? (int)(ksw >> (8 * half)) : (int)ksw;
      const uint4 k0 = *reinterpret_cast<const uint4*>(sb + kb_lo + koff * L::kRow);
      v8i kf;
      kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w;
      v16f z;
#pragma unroll
      for (int r = 0; r < 16; r++) z[r] = 0.0f;
      s[2 * q + t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(kf, qf0, z, ksc, (int)qsc);
      if constexpr (KS == 2) {
        const uint4 k1 = *reinterpret_cast<const uint4*>(sb + kb_hi + koff * L::kRow);
        kf[0] = k1.x; kf[1] = k1.y; kf[2] = k1.z; kf[3] = k1.w;
        s[2 * q + t] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(kf, qf1, s[2 * q + t], ksc, (int)qsc);
      }
    }
  };

  // O^T += V^T P^T and l += 1^T P^T for sub-block q of the block staged at sb
  auto pv = [&](const lds_char* sb, int q, const v8i& pf, int psc) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < DT; t++) {
      const uint4 v0 = *reinterpret_cast<const uint4*>(sb + (q ? vb1 : vb0) + t * 32 * L::vRow);
      v8i vf;
      vf[0] = v0.x; vf[1] = v0.y; vf[2] = v0.z; vf[3] = v0.w;
      const int vsc = (int)*reinterpret_cast<const lds_u32*>(sb + vs_base + (2 * q * D + t * 32) * 4);
      acc[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(vf, pf, acc[t], vsc, psc);
    }
    accl = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(ones, pf, accl, 127, psc);
  };

  // E2M1 codes of 2^(fmaf(S, c, off)) for this lane's 32-key block of sub-block q
  auto codes_off = [&](int q, float off, v8i& pf) __attribute__((always_inline)) {
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
      pf[w] = (int)u;
    }
  };
  // running max: codes relative to m_run and the block's E8M0 scale
  auto codes = [&](int q, float bm, float mc, v8i& pf) __attribute__((always_inline)) -> int {
    const float d2 = fmul_rn(fsub_rn(bm, m_run), C);
    const float ebf = fmaxf(floorf(d2) - 2.0f, -127.0f);
    codes_off(q, fsub_rn(-mc, ebf), pf);
    return (int)ebf + 127;
  };
  // anchored: block exponent t (already clamped to >= A - 125), codes of 2^(S c - t + 2), and the
  // E8M0 byte t - 2 - A + 127 relative to the anchor
  auto codes_anch = [&](int q, float t, v8i& pf) __attribute__((always_inline)) -> int {
    codes_off(q, 2.0f - t, pf);
    return (int)(t - m_run) + 125;
  };

  // One key block j with its scores in s[], staged at sb (V) and, unless LAST, block j+1's K
  // staged at sbn.
  auto block = [&](auto LC, int j, const lds_char* sb, const lds_char* sbn) __attribute__((always_inline)) {
    constexpr bool LAST = decltype(LC)::value;
    if constexpr (LAST) {
      const int kb0 = j * KB;
      if (kb0 + KB > N) {
#pragma unroll
        for (int ti = 0; ti < 2 * NSB; ti++)
#pragma unroll
          for (int i = 0; i < 16; i++) {
            const int key = kb0 + (ti >> 1) * 64 + half * 32 + (ti & 1) * 16 + i;
            s[ti][i] = key < N ? s[ti][i] : -INFINITY;
          }
      }
    }
    const float bm0 = max32(s[0], s[1]);
    const float bm1 = NSB == 2 ? max32(s[2 * NSB - 2], s[2 * NSB - 1]) : bm0;
    if constexpr (ANCH) {
      // block exponents; a fully masked lane half gives -inf
      float t0 = floorf(fmul_rn(bm0, C)), t1 = floorf(fmul_rn(bm1, C));
      const float tm = __builtin_elementwise_maximum(t0, t1);
      // the guard: move the anchor when a block sits more than 64 binades above it (on the first
      // block the anchor is -inf, so this sets it from the block's exponents)
      if (__builtin_amdgcn_ballot_w64(tm - m_run > 64.0f)) {
        const float an = max_across_halves(__builtin_elementwise_maximum(tm, m_run));
        const float f = __builtin_amdgcn_ldexpf(1.0f, (int)fmaxf(m_run - an, -150.0f));
#pragma unroll
        for (int t = 0; t < DT; t++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[t][r] *= f;
        accl[0] *= f;
        m_run = an;
      }
      t0 = __builtin_elementwise_maximum(t0, m_run - 125.0f);
      t1 = __builtin_elementwise_maximum(t1, m_run - 125.0f);
      v8i pf0, pf1;
      const int psc0 = codes_anch(0, t0, pf0);
      if constexpr (NSB == 1) {
        pv(sb, 0, pf0, psc0);
        if constexpr (!LAST) scores(sbn, 0);
        return;
      }
      const int psc1 = codes_anch(NSB - 1, t1, pf1);
      // left to the compiler's scheduler: with no running max the block has fewer dependences, and
      // the scheduling groups of the running-max form were 3-5 % slower here
      pv(sb, 0, pf0, psc0);
      if constexpr (!LAST) scores(sbn, 0);
      if constexpr (!LAST) scores(sbn, NSB - 1);
      pv(sb, NSB - 1, pf1, psc1);
      return;
    }
    // running max; the rescale is unconditional (alpha = 1 exactly when a row's max is unchanged,
    // and 0 on the first block where O and l are still 0)
    const float m_new =
        __builtin_elementwise_maximum(m_run, max_across_halves(__builtin_elementwise_maximum(bm0, bm1)));
    const float alpha = __builtin_amdgcn_exp2f(fmul_rn(fsub_rn(m_run, m_new), C));
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[t][r] *= alpha;
    accl[0] *= alpha;
    m_run = m_new;
    const float mc = fmul_rn(m_new, C);
    v8i pf0, pf1;
    const int psc0 = codes(0, bm0, mc, pf0);
    if constexpr (NSB == 1) {
      // one sub-block: its P.V and the next block's scores follow the codes; the compiler
      // schedules them
      pv(sb, 0, pf0, psc0);
      if constexpr (!LAST) scores(sbn, 0);
      return;
    }
    const int psc1 = codes(NSB - 1, bm1, mc, pf1);
    pv(sb, 0, pf0, psc0);
    if constexpr (!LAST) scores(sbn, 0);
    if constexpr (!LAST) scores(sbn, NSB - 1);
    pv(sb, NSB - 1, pf1, psc1);
    // schedule: the second sub-block's codes run with the first sub-block's P.V and the next
    // block's first scores underneath; the rest issues at the end
    __builtin_amdgcn_sched_group_barrier(kSgVALU, 110, 0);  // max, rescale, codes(j, 0)
    __builtin_amdgcn_sched_group_barrier(kSgDSRead, 8, 0);
#pragma unroll
    for (int g = 0; g < DT + 1 + (LAST ? 0 : 2 * KS); g++) {
      __builtin_amdgcn_sched_group_barrier(kSgMFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSgVALU, 8, 0);
      __builtin_amdgcn_sched_group_barrier(kSgDSRead, 1, 0);
    }
  };

  // ---- prologue: blocks 0 and 1 staged, scores of block 0 ----
  st.issue(0, smem);
  if (nkb > 1) st.issue(1, smem + L::buf);
  wait_dma();
  __builtin_amdgcn_s_barrier();
  scores(smem, 0);
  if constexpr (NSB == 2) scores(smem, 1);

  int rb = 0;  // j % 3
  for (int j = 0; j + 1 < nkb; j++) {
    const int rn = rb == 2 ? 0 : rb + 1, r2 = rn == 2 ? 0 : rn + 1;
    if (j + 2 < nkb) st.issue(j + 2, smem + r2 * L::buf);
    block(std::false_type(), j, smem + rb * L::buf, smem + rn * L::buf);
    // block j+2 has landed (each wave waits for its own loads); buffer rb is free once every wave
    // is past its last fragment reads of block j
    wait_dma();
    __builtin_amdgcn_s_barrier();
    rb = rn;
  }
  block(std::true_type(), nkb - 1, smem + rb * L::buf, smem);

  // ---- epilogue: O = O^T / l in bf16 (whole rows through LDS), LSE = m / sqrt(D) + ln(l)
  // (ANCH: LSE = (A + log2 l) ln 2) ----
  store_o_lse_rows<D, ANCH>(acc, accl[0], m_run, a.o + (int64_t)bh * N * D, a.lse + (int64_t)bh * N, N,
                            tl.qt * kDPQueryTile + wave * 32, lane, smem + wave * OStage<D>::kBytes);
}

}  // namespace

hipError_t launch_attn_fwd_directp(const FwdArgs& a, int D, hipStream_t stream, const KernelEvents& ev,
                                   bool anchored) {
  const int nqt = (a.N + kDPQueryTile - 1) / kDPQueryTile;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(64 * kDPWaves);
  if (anchored) {
    if (D == 128) return launch_kernel(attn_fwd_directp_kernel<128, true>, grid, block, 0, stream, ev, a);
    return launch_kernel(attn_fwd_directp_kernel<64, true>, grid, block, 0, stream, ev, a);
  }
  if (D == 128) return launch_kernel(attn_fwd_directp_kernel<128, false>, grid, block, 0, stream, ev, a);
  return launch_kernel(attn_fwd_directp_kernel<64, false>, grid, block, 0, stream, ev, a);
}

}  // namespace fp4attn

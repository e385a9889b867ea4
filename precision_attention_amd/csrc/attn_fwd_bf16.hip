// attn_fwd_bf16.hip -- the FP4 forward's kernel design with bf16 operands on the bf16 MFMA
// (V_MFMA_F32_32X32X16_BF16). It exists to form the FP4-versus-BF16 throughput ratio that
// "Hardware-Aware FP4 FlashAttention-4" reports against a BF16 FlashAttention forward
// (gist.science technical summary, Key Contributions; Results "Throughput").
//
// Per 64-key block of one query row, reference point m (at most the row max so far),
// c = log2(e)/sqrt(D):
//   m' = max(m, block max); when some row of the wave has (m' - m) c > 8 (and on the first
//   block): O, l *= 2^((m - m') c), m = m'
//   P_j = 2^(fmaf(S_j, c, -fp32(m c))) in fp32 (at most 2^8); l += sum_j P_j (unrounded);
//   O += bf16(P) V.
// O = O / l and LSE = m / sqrt(D) + ln l do not depend on which m was used.
//
// The structure is that of the FP4 kernels (attn_fwd_directp.hip, nvfp4.hip): 8 waves x 32
// queries per workgroup, one workgroup per CU, two waves per SIMD; the K rows and V^T rows of a
// 64-key block are fetched two blocks ahead into three rotating LDS buffers by direct
// global->LDS loads, one wait and one barrier per block; S^T = K Q^T on the BF16 MFMA puts one
// query in each lane (Q in registers; K rows read in the order {0..3, 32..35, 4..7, ...}, which
// places the lane half's 32 keys in its registers), and the next block's score MFMAs (into a
// second set of score registers, the block loop unrolled by two) run under this block's
// softmax. O^T = V^T P^T keeps the query in the lane, so m, l and the rescale factor are
// per-lane. V comes transposed, [B, Hkv, D, N], as the FP4 routes' V comes from the quantizer's
// along-the-sequence layout.
#include "device_common.h"
#include "fwd_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

constexpr int kBfWaves = 8;
constexpr int kBfQTile = 32 * kBfWaves;
constexpr int kBfKB = 64;  // keys per block (one running-max update per block)
constexpr float kLazy = 8.0f;  // log2 of the largest P relative to the reference point

template <int D>
struct BfSmem {
  static constexpr int kRow = 2 * D;                 // bytes of one K row (bf16)
  static constexpr int kCh = kRow / 16;              // 16-byte chunks per K row
  static constexpr int kBytes = kBfKB * kRow;
  static constexpr int vRow = 2 * kBfKB;             // bytes of one V^T row (64 keys, bf16)
  static constexpr int vCh = vRow / 16;              // 8
  static constexpr int vOff = kBytes;
  static constexpr int buf = vOff + D * vRow;
  static constexpr int kDma = kBytes / 1024;         // 16-byte-per-lane instructions
  static constexpr int vDma = D * vRow / 1024;
  static constexpr int nDma = kDma + vDma;
};

// physical 16-byte chunk of logical chunk c in K row r: a fragment read phase of 16 lanes touches
// rows {0..3, 32..35, 4..7, 36..39} (+16 t) at one logical chunk
template <int D>
__device__ __forceinline__ int bf_kchunk(int r, int c) {
  if constexpr (D == 128) return c ^ ((r & 3) | (((r >> 2) & 1) << 2) | (((r >> 5) & 1) << 3));  // 16 chunks
  else return c ^ (((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 5) & 1) << 2));  // 8 chunks, 2 rows / 256 B
}
// physical chunk of logical chunk c (keys 8c .. 8c+7) in V^T row d: a read phase of 16 lanes
// touches rows d .. d+15 at one logical chunk; rows are 128 bytes, so (d & 1) and the XOR with
// bits 1-3 of d give the 16 rows 16 distinct bank groups
__device__ __forceinline__ int bf_vchunk(int d, int c) { return c ^ ((d >> 1) & 7); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  v2bf r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(64 * kBfWaves, 2) attn_fwd_bf16_kernel(FwdBf16Args a) {
  using L = BfSmem<D>;
  constexpr int DT = D / 32;
  constexpr int KS = D / 16;  // BF16 MFMA k-steps over D
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr int kSmem = 3 * L::buf > kBfWaves * OStage<D>::kBytes ? 3 * L::buf : kBfWaves * OStage<D>::kBytes;
  __shared__ __attribute__((aligned(16))) lds_char smem[kSmem];

  // the wave index is wave-uniform: readfirstlane lets the compiler keep what derives from it in
  // scalar registers and branch on it without exec masks
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5,
            col = lane & 31;
  const int N = a.N;
  // workgroup -> (batch*head, query tile): each XCD takes a contiguous range of tiles; causal:
  // the longest rows first
  const int nqt = (N + kBfQTile - 1) / kBfQTile;
  const int total = (int)gridDim.x;
  const int per = total / 8, rem = total % 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  int qt = lin % nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int bh = lin / nqt, h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int qrow0 = qt * kBfQTile;
  const int qwave0 = qrow0 + wave * 32;
  const int qi = qwave0 + col;
  const bool qvalid = qi < N;

  // this lane's Q fragments (B operand of S^T): query qi, d = 16 s + 8 half .. +7
  v8bf qf[KS];
#pragma unroll
  for (int s = 0; s < KS; s++) {
    uint4 t = make_uint4(0, 0, 0, 0);
    if (qvalid) t = *reinterpret_cast<const uint4*>(a.q + ((int64_t)bh * N + qi) * D + 16 * s + 8 * half);
    qf[s] = __builtin_bit_cast(v8bf, t);
  }
  // wait for the fragment loads here (vmcnt 0), not at their first use inside the block loop,
  // where the wait would also cover the staging loads in flight
  __builtin_amdgcn_s_waitcnt(0x0F70);

  // ---- staging: DMA instruction i of a block is issued by wave i % 8; rows past N read row
  // N-1 and V^T chunks past N the block's first chunk (finite data under masked keys) ----
  const void* kbase = uniform_ptr(reinterpret_cast<const uint8_t*>(a.k) + bhkv * N * D * 2);
  const void* vbase = uniform_ptr(reinterpret_cast<const uint8_t*>(a.vt) + bhkv * D * N * 2);
  const uint32_t lds0 = lds_addr(smem);
  auto issue = [&](int j, int buf) {
    const int kb0 = j * kBfKB;
    const uint32_t base = lds0 + buf * L::buf;
#pragma unroll
    for (int i = wave; i < L::nDma; i += kBfWaves) {
      if (i < L::kDma) {
        const int P = i * 64 + lane;  // 16-byte slot
        const int r = P / L::kCh, c = bf_kchunk<D>(r, P % L::kCh);
        const int gk = min(kb0 + r, N - 1);
        dma16_async(kbase, (uint32_t)gk * (D * 2) + (uint32_t)c * 16, base + i * 1024);
      } else {
        const int P = (i - L::kDma) * 64 + lane;
        const int d = P / L::vCh, c = bf_vchunk(d, P % L::vCh);
        const int cc = (kb0 + c * 8 < N) ? c : 0;
        dma16_async(vbase, (uint32_t)d * (N * 2) + (uint32_t)(kb0 + cc * 8) * 2, base + L::vOff + (i - L::kDma) * 1024);
      }
    }
  };

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  // lane-constant LDS offsets: K row krow (+16 t), V^T row col (+32 t; the chunk swizzle reads
  // bits of d that adding 32 leaves unchanged)
  const int krow = (((col >> 2) & 1) << 5) + ((col >> 3) << 2) + (col & 3);

  const int kend = CAUSAL ? min(N, qrow0 + kBfQTile) : N;
  const int nkb = (kend + kBfKB - 1) / kBfKB;

  // S^T tiles of the block staged at sb: tile t holds keys 32 half + 16 t + i (register i)
  // (the two tiles alternate, so that each fragment read has two MFMAs of slack)
  auto scores = [&](const lds_char* sb, v16f (&sn)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < 2; t++)
#pragma unroll
      for (int rr = 0; rr < 16; rr++) sn[t][rr] = 0.0f;
#pragma unroll
    for (int ks = 0; ks < KS; ks++)
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int r = krow + 16 * t;
        const u32x4 kf = *reinterpret_cast<const u32x4*>(sb + r * L::kRow + bf_kchunk<D>(r, 2 * ks + half) * 16);
        sn[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kf), qf[ks], sn[t], 0, 0, 0);
      }
  };

  // One key block j with its scores in sc, staged at sb; block j+1's scores are formed into sn
  // from sbn while block j's softmax runs (after the last block, from a stale buffer, never read).
  auto block = [&](int j, v16f (&sc)[2], v16f (&sn)[2], const lds_char* sb, const lds_char* sbn)
      __attribute__((always_inline)) {
    const int kb0 = j * kBfKB;
    // masks: keys past N (and a step past the end, wholly), and the causal diagonal
    const bool need_mask = (kb0 + kBfKB > N) || (CAUSAL && kb0 + kBfKB - 1 > qwave0);
    if (need_mask) {
      asm volatile("" ::: "memory");  // keeps this a branch: few blocks take it
#pragma unroll
      for (int t = 0; t < 2; t++)
#pragma unroll
        for (int i = 0; i < 16; i++) {
          const int key = kb0 + half * 32 + t * 16 + i;
          const bool vis = key < N && (!CAUSAL || key <= qi);
          sc[t][i] = vis ? sc[t][i] : -INFINITY;
        }
    }
    const float bmax = fwd::max32(sc[0], sc[1]);
    const float m_blk = __builtin_elementwise_maximum(m_run, max_across_halves(bmax));
    // The reference point m moves (with O and l rescaled) only when some row's max exceeds it by
    // more than 2^8 in P (every row on the first block): P = 2^((S - m) c) <= 2^8 stays exact to
    // bf16's relative precision, and the rescale's 65 multiplies run on a few blocks rather than
    // on most. O / l and LSE = m / sqrt(D) + ln l hold for any m at or below the row max.
    if (__any(fmul_rn(fsub_rn(m_blk, m_run), C) > kLazy)) {
      const float alpha = __builtin_amdgcn_exp2f(fmul_rn(fsub_rn(m_run, m_blk), C));
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[t][r] *= alpha;
      l_run *= alpha;
      m_run = m_blk;
    }
    scores(sbn, sn);
    // a row that has seen only masked keys keeps m = -inf: its P are 0 (not 2^nan)
    const float off = m_run == -INFINITY ? 0.0f : -fmul_rn(m_run, C);
    float p[32];
    float lsum = 0.0f;
#pragma unroll
    for (int idx = 0; idx < 32; idx++) {
      p[idx] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[idx >> 4][idx & 15], C, off));
      lsum += p[idx];
    }
    // l over both lane halves (keys 0-31 here, 32-63 in lane l^32)
    {
      uint32_t x0 = __float_as_uint(lsum), x1 = x0;
      permlane32_swap(x0, x1);
      l_run += __uint_as_float(x0) + __uint_as_float(x1);
    }
    // O^T += V^T P^T: k-step kk takes this lane half's keys 32 half + 8 kk .. +7 (A: V^T row
    // d = 32t + col at those keys; B: the lane's bf16 P at those keys)
#pragma unroll
    for (int kk = 0; kk < 4; kk++) {
      u32x4 pw;
#pragma unroll
      for (int w = 0; w < 4; w++) pw[w] = pack_bf16(p[8 * kk + 2 * w], p[8 * kk + 2 * w + 1]);
      const v8bf pb = __builtin_bit_cast(v8bf, pw);
#pragma unroll
      for (int t = 0; t < DT; t++) {
        const int d = t * 32 + col;
        const u32x4 vv = *reinterpret_cast<const u32x4*>(sb + L::vOff + d * L::vRow + bf_vchunk(d, 4 * half + kk) * 16);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, vv), pb, acc[t], 0, 0, 0);
      }
    }
  };

  // Block j is staged in buffer j % 3 (issued two blocks ahead); one wait and one barrier per
  // block, after which block j+1 has landed and block j-1's buffer is free. Blocks go in pairs
  // (alternating score registers); for an odd count a last step past the end has every key
  // masked and reads the last block's buffer. Under the causal mask a wave whose rows all precede
  // block j skips its math (every later block too).
  v16f sA[2], sB[2];
  issue(0, 0);
  if (nkb > 1) issue(1, 1);
  wait_dma();
  __syncthreads();
  scores(smem, sA);
  int bj = 0, bj1 = 1, bj2 = 2;  // buffers of blocks j, j+1, j+2
  auto step = [&](int j, v16f (&sc)[2], v16f (&sn)[2]) __attribute__((always_inline)) {
    if (j > 0) {
      wait_dma();
      __syncthreads();
    }
    if (j + 2 < nkb) issue(j + 2, bj2);
    const int bc = j < nkb ? bj : (bj + 2) % 3;
    if (!CAUSAL || j * kBfKB <= qwave0 + 31) block(j, sc, sn, smem + bc * L::buf, smem + bj1 * L::buf);
    const int b0 = bj;
    bj = bj1;
    bj1 = bj2;
    bj2 = b0;
  };
  for (int j = 0; j < nkb; j += 2) {
    step(j, sA, sB);
    step(j + 1, sB, sA);
  }
  // every wave is past its last fragment reads before the output tiles overwrite the buffers
  wait_dma();
  __syncthreads();

  // O = O^T / l in bf16 (whole rows through LDS), LSE = m / sqrt(D) + ln(l)
  store_o_lse_rows<D>(acc, l_run, m_run, a.o + (int64_t)bh * N * D, a.lse + (int64_t)bh * N, N, qwave0, lane,
                      smem + wave * OStage<D>::kBytes);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdBf16Args& a, int D, int causal, hipStream_t stream) {
  const int nqt = (a.N + kBfQTile - 1) / kBfQTile;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(64 * kBfWaves);
  if (D == 128) {
    if (causal) attn_fwd_bf16_kernel<128, true><<<grid, block, 0, stream>>>(a);
    else attn_fwd_bf16_kernel<128, false><<<grid, block, 0, stream>>>(a);
  } else {
    if (causal) attn_fwd_bf16_kernel<64, true><<<grid, block, 0, stream>>>(a);
    else attn_fwd_bf16_kernel<64, false><<<grid, block, 0, stream>>>(a);
  }
  return hipGetLastError();
}

}  // namespace fp4attn

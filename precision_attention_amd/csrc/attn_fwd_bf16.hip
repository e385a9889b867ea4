// attn_fwd_bf16.hip -- the same online-softmax forward loop with bf16 operands on the bf16
// MFMA (V_MFMA_F32_32X32X16_BF16). It exists to form the FP4-versus-BF16 throughput ratio
// that "Hardware-Aware FP4 FlashAttention-4" reports against a BF16 FlashAttention forward
// (gist.science technical summary, Key Contributions; Results "Throughput").
//
// P = 2^(fmaf(S, c, -m c)) in fp32, rounded to bf16 for the P.V product; the normalizer l
// sums the unrounded fp32 P. Keys are consumed in blocks of 64 with one running-max update
// per block, as in the FP4 kernels.
//
// Layout on the MI355X: 4 waves x 32 queries per workgroup; S^T = K Q^T with Q^T held in
// registers and K read from LDS ([key][d], 16-byte chunks XOR-swizzled); O^T = V^T P^T with V
// transposed into LDS ([d][key]) while it is staged, so each lane's MFMA operand is 8
// consecutive keys; lane l keeps query l%32, so m, l and the rescale factor are per-lane.
#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

template <int D>
struct Bf16Smem {
  static constexpr int kRow = D * 2;                 // bytes per K row
  static constexpr int kCh = kRow / 16;              // 16-byte chunks per K row
  static constexpr int vtRow = kKeyBlock * 2 + 16;   // bytes per V^T row (64 keys + pad)
  static constexpr int vtOff = kKeyBlock * kRow;
  static constexpr int buf = vtOff + D * vtRow;
  static constexpr int kLoads = kKeyBlock * kCh / kThreads;        // 16-byte K loads per thread
  static constexpr int vUnits = (kKeyBlock / 2) * (D / 8);         // (key pair, 8-d chunk)
  static constexpr int vLoads = vUnits / kThreads;
};

// K row chunk swizzle. One 16-lane phase of a fragment read touches keys {0..7, 32..39}
// (+16 t, +8) at one logical chunk: D=128 rows are 256 B (every row starts at bank 0), so
// the 16 keys need 16 distinct physical chunks; D=64 rows are 128 B (key parity picks the
// bank half), so each parity class needs 8 distinct chunks.
template <int D>
__device__ __forceinline__ int kb_chunk(int key, int c) {
  if constexpr (D == 128) return c ^ ((key & 7) | (((key >> 5) & 1) << 3));
  else return c ^ (((key >> 1) & 3) | (((key >> 5) & 1) << 2));
}

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  v2bf r = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, r);
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) attn_fwd_bf16_kernel(FwdBf16Args a) {
  using L = Bf16Smem<D>;
  constexpr int DT = D / 32;
  constexpr int KS = D / 16;  // k-steps of S^T
  constexpr float C = log2e_over_sqrt_d(D);
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * L::buf];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, half = lane >> 5, col = lane & 31;
  const int N = a.N;
  const int nqt = (N + kQueryTile - 1) / kQueryTile;
  const int total = (int)gridDim.x;
  const int per = total / 8, rem = total % 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  int qt = lin % nqt;
  if (CAUSAL) qt = nqt - 1 - qt;
  const int bh = lin / nqt;
  const int h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int qrow0 = qt * kQueryTile;
  const int qwave0 = qrow0 + wave * 32;
  const int qi = qwave0 + col;
  const bool qvalid = qi < N;

  // Q^T fragments: k-step ks covers d = 16*ks + 8*half + j.
  v8bf qf[KS];
  {
    const uint16_t* qrow = a.q + ((int64_t)bh * N + qi) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ks++) {
      u32x4 t = {0, 0, 0, 0};
      if (qvalid) t = *reinterpret_cast<const u32x4*>(qrow + 16 * ks + 8 * half);
      qf[ks] = __builtin_bit_cast(v8bf, t);
    }
  }

  const int kend = CAUSAL ? min(N, qrow0 + kQueryTile) : N;
  const int nkb = (kend + kKeyBlock - 1) / kKeyBlock;

  uint4 st_k[L::kLoads];
  uint4 st_v[L::vLoads][2];
  auto load_stage = [&](int j) {
    const int kb0 = j * kKeyBlock;
#pragma unroll
    for (int u = 0; u < L::kLoads; u++) {
      const int t = tid + u * kThreads;
      const int key = t / L::kCh, c = t % L::kCh, gk = kb0 + key;
      st_k[u] = gk < N ? *reinterpret_cast<const uint4*>(a.k + (bhkv * N + gk) * D + c * 8) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < L::vLoads; u++) {
      const int t = tid + u * kThreads;
      const int kp = t % (kKeyBlock / 2), c = t / (kKeyBlock / 2);
      const int g0 = kb0 + 2 * kp;
#pragma unroll
      for (int e = 0; e < 2; e++)
        st_v[u][e] = g0 + e < N ? *reinterpret_cast<const uint4*>(a.v + (bhkv * N + g0 + e) * D + c * 8)
                                : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* sb = smem + buf * L::buf;
#pragma unroll
    for (int u = 0; u < L::kLoads; u++) {
      const int t = tid + u * kThreads;
      const int key = t / L::kCh, c = t % L::kCh;
      *reinterpret_cast<uint4*>(sb + key * L::kRow + kb_chunk<D>(key, c) * 16) = st_k[u];
    }
#pragma unroll
    for (int u = 0; u < L::vLoads; u++) {
      const int t = tid + u * kThreads;
      const int kp = t % (kKeyBlock / 2), c = t / (kKeyBlock / 2);
      const uint32_t a0[4] = {st_v[u][0].x, st_v[u][0].y, st_v[u][0].z, st_v[u][0].w};
      const uint32_t a1[4] = {st_v[u][1].x, st_v[u][1].y, st_v[u][1].z, st_v[u][1].w};
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t lo = (a0[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
        const uint32_t hi = (a1[i / 2] >> (16 * (i & 1))) & 0xFFFFu;
        const int d = c * 8 + i;
        *reinterpret_cast<uint32_t*>(sb + L::vtOff + d * L::vtRow + kp * 4) = lo | (hi << 16);
      }
    }
  };

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;
  float m_run = -INFINITY, l_run = 0.0f;

  load_stage(0);
  store_stage(0);
  __syncthreads();

  for (int j = 0; j < nkb; j++) {
    const int kb0 = j * kKeyBlock;
    if (j + 1 < nkb) load_stage(j + 1);
    const uint8_t* sb = smem + (j & 1) * L::buf;
    const bool wave_active = !CAUSAL || kb0 <= qwave0 + 31;
    if (wave_active) {
      v16f s[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int key = (((col >> 2) & 1) << 5) + t * 16 + ((col >> 3) << 2) + (col & 3);
#pragma unroll
        for (int r = 0; r < 16; r++) s[t][r] = 0.0f;
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const int c = 2 * ks + half;  // 16-byte chunk: d = 16*ks + 8*half .. +7
          const u32x4 kk = *reinterpret_cast<const u32x4*>(sb + key * L::kRow + kb_chunk<D>(key, c) * 16);
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, kk), qf[ks], s[t], 0, 0, 0);
        }
      }
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
      float bmax = s[0][0];
#pragma unroll
      for (int i = 1; i < 16; i++) bmax = fmaxf(bmax, s[0][i]);
#pragma unroll
      for (int i = 0; i < 16; i++) bmax = fmaxf(bmax, s[1][i]);
      const float m_new = fmaxf(m_run, max_across_halves(bmax));
      if (__any(m_new > m_run)) {
        const float alpha = __builtin_amdgcn_exp2f((m_run - m_new) * C);
#pragma unroll
        for (int t = 0; t < DT; t++)
#pragma unroll
          for (int r = 0; r < 16; r++) acc[t][r] *= alpha;
        l_run *= alpha;
      }
      m_run = m_new;
      const float off = -(m_new * C);
      float p[32];
      float lsum = 0.0f;
#pragma unroll
      for (int idx = 0; idx < 32; idx++) {
        p[idx] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[idx >> 4][idx & 15], C, off));
        lsum += p[idx];
      }
      // l over both lane halves (keys 0-31 here, 32-63 in lane l^32)
      {
        uint32_t x0 = __float_as_uint(lsum), x1 = x0;
        permlane32_swap(x0, x1);
        l_run += __uint_as_float(x0) + __uint_as_float(x1);
      }
      // O^T += V^T P^T: k-step kk uses this lane's keys half*32 + 8*kk + jj
#pragma unroll
      for (int kk = 0; kk < 4; kk++) {
        u32x4 pw;
#pragma unroll
        for (int w = 0; w < 4; w++) pw[w] = pack_bf16(p[8 * kk + 2 * w], p[8 * kk + 2 * w + 1]);
        const v8bf pb = __builtin_bit_cast(v8bf, pw);
#pragma unroll
        for (int t = 0; t < DT; t++) {
          const int d = t * 32 + col;
          const u32x4 vv =
              *reinterpret_cast<const u32x4*>(sb + L::vtOff + d * L::vtRow + (half * 32 + 8 * kk) * 2);
          acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, vv), pb, acc[t], 0, 0, 0);
        }
      }
    }
    if (j + 1 < nkb) store_stage((j + 1) & 1);
    __syncthreads();
  }

  // O = O^T / l in bf16 (whole rows through LDS; both K/V buffers are free), LSE = m / sqrt(D) + ln(l)
  static_assert(2 * L::buf >= kWaves * OStage<D>::kBytes, "output tiles fit the K/V buffers");
  store_o_lse_rows<D>(acc, l_run, m_run, a.o + (int64_t)bh * N * D, a.lse + (int64_t)bh * N, N, qwave0, lane,
                      smem + wave * OStage<D>::kBytes);
}

}  // namespace

hipError_t launch_attn_fwd_bf16(const FwdBf16Args& a, int D, int causal, hipStream_t stream) {
  const int nqt = (a.N + kQueryTile - 1) / kQueryTile;
  const dim3 grid((unsigned)(nqt * a.H * a.B)), block(kThreads);
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

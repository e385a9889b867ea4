// attn_bwd.hip -- backward of the causal FP4/FP8 route of "Hardware-Aware FP4 FlashAttention-4"
// (gist.science technical summary, Methodology 2 "Quantized Causal Backward": Reconstruction,
// Gradient Formats; arXiv abstract).
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
// A quantizer launch first writes dO's two MXFP8 views into the workspace; its along-D job also
// reads O and writes -Delta_i = -sum_d dO_id O_id (fp32) and -fp32(LSE_i log2 e) per row.
// Then two kernels:
//  - dkdv_kernel: one workgroup per (batch, KV head, 128-key tile), 4 waves x 32 keys, the tile's
//    K and V fragments held in registers. S and dP are formed with keys in lanes and queries in
//    registers (S = Q K^T, dP = dO V^T), so P and dS come out of the MFMA already in the layout
//    of the A operand of dV += P^T dO and dK += dS^T Q; their MX blocks along queries span one
//    lane pair (one permlane32 swap for the block max). Loops over 64-query blocks and, inside,
//    the query heads of the KV group, in an order that keeps the group's workgroups on the same
//    block; each block's Q, dO rows and Q^T, dO^T rows are staged into LDS by direct
//    global->LDS loads one block ahead (double buffer).
//  - dq_kernel: one workgroup per (batch, query head, 128-query tile), 4 waves x 32 queries, the
//    forward's orientation (queries in lanes, keys in registers): S^T = K Q^T, dP^T = V dO^T,
//    dS blocked along keys in-lane, dQ^T += K^T dS^T; K, V rows and K^T rows staged one 64-key
//    block ahead.
// LDS rows use XOR-swizzled 16-byte chunks so that the 16 lanes of a fragment read hit distinct
// banks. The staging loads are issued as inline assembly (dma16_async and friends) and ordered
// by an explicit wait and a barrier per block. Operand layouts of the 32x32x64 block-scaled
// MFMA: see device_common.h.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace fp4attn {
namespace {

constexpr int kThreads = 256;
constexpr int kWavesB = 4;
constexpr int kThreadsKV = 2 * kWavesB * 64;  // dkdv: two groups of 4 waves

__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// E8M0 exponent of an MXFP8 block from its largest magnitude (binary32):
// floor(log2 amax) - 8, clamped to [-127, 127]; amax == 0 or subnormal gives -127.
__device__ __forceinline__ int mx8_exponent(float amax) {
  const int E = (int)((__float_as_uint(amax) >> 23) & 0xFFu);
  return max(E - 127 - 8, -127);
}
// IEEE-754-2019 maximum of three; lowers to v_maximum3_f32 (operands here are finite)
// 2^u in binary32 for the probability of query 0. For |u| < 2^-21, 2^u = 1 + u ln 2 to within
// 1e-13, so one fused multiply-add rounds it as a correctly rounded exponential would, whereas the
// hardware exponential may land on the other side of 1.0. The side matters: a probability one ulp
// below 1.0 heads its MXFP8 block with exponent -9 and saturates to 0.875 (the floor rule of the
// block exponent), 1.0 is exact. Query 0 of the causal route sees one key, so its probability is 1
// up to the rounding of LSE and sits at that edge in every head; other probabilities reach it only
// when one key holds all but 1e-7 of a row's weight.
constexpr float kLn2 = 0x1.62e430p-1f;  // binary32 ln 2
__device__ __forceinline__ float exp2_near_one(float u, float p) {
  return fabsf(u) < 0x1p-21f ? __builtin_fmaf(u, kLn2, 1.0f) : p;
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// The scale operand of the fp8 converters: only its exponent field is used (field 0 = 2^-127,
// measured), so the E8M0 code goes straight into the exponent bits; the converter then divides
// by 2^e exactly.
__device__ __forceinline__ float scale_operand(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
// 448 * 2^e: the largest value whose scaled code stays finite in E4M3 (the converter does not
// saturate); finite for every e the exponent rule produces
__device__ __forceinline__ float e4m3_limit(int e) {
  return __uint_as_float(((uint32_t)(e + 127 + 8) << 23) | 0x600000u);
}

// E4M3 codes of a/2^e .. d/2^e (inputs already within +-448 * 2^e), element 0 in the low byte.
__device__ __forceinline__ uint32_t pack4_fp8_scaled(float a, float b, float c, float d, float sc) {
  v2s w = __builtin_bit_cast(v2s, a);  // both halves are written: any initial value (no extra move)
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, a, b, sc, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, c, d, sc, true);
  uint32_t r;
  __builtin_memcpy(&r, &w, 4);
  return r;
}

// query (or key) held in register i of lane half h of a 32x32 MFMA output tile whose A rows
// were loaded in the order r -> perm32(r): the output's register i of half h is row h*16 + i.
__device__ __forceinline__ int perm32(int r) { return (((r >> 2) & 1) << 4) + ((r >> 3) << 2) + (r & 3); }

// XOR swizzles of the 16-byte chunks of LDS rows. A fragment read of 16 lanes touches one chunk
// of the rows {0..3, 16..19, 4..7, 20..23} (+8 for the other 16 lanes) -- the perm32 row set --
// or of 16 consecutive rows; each swizzle maps those 16 reads to distinct banks (64 banks x 4
// bytes) for its row length.
__device__ __forceinline__ int sw2_perm(int r) { return (r >> 4) & 1; }                              // 32-byte rows
__device__ __forceinline__ int sw4_perm(int r) { return ((r >> 2) & 1) | (((r >> 4) & 1) << 1); }    // 64-byte rows
__device__ __forceinline__ int sw8_perm(int r) {                                                     // 128-byte rows
  return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 4) & 1) << 2);
}
__device__ __forceinline__ int sw4_lin(int r) { return (r >> 2) & 3; }  // 64-byte rows, consecutive
// chunk position of logical chunk c of a perm32-read row holding D/2 (FP4) or D (FP8) bytes
template <int D>
__device__ __forceinline__ int swz_fp4_row(int r, int c) { return D == 128 ? (c ^ sw4_perm(r)) : (c ^ sw2_perm(r)); }
template <int D>
__device__ __forceinline__ int swz_fp8_row(int r, int c) { return D == 128 ? (c ^ sw8_perm(r)) : (c ^ sw4_perm(r)); }
// dq_kernel's K and V rows are read in the set {0..3, 32..35, 4..7, 36..39, ...} (+16): bit 5 of
// the key is the output lane half. Its swizzles use bits 2 and 5 (and bit 1 for 128-byte rows),
// which map each 16-lane read to 16 distinct bank groups.
// Wait for this wave's outstanding vector-memory loads with an instruction that the compiler's
// wait-count bookkeeping sees (vmcnt 0; expcnt and lgkmcnt left at their maxima). Register
// fragments loaded before a staged loop and first used inside it would otherwise get their wait
// at that first use, inside the loop, where it also waits for the staging loads in flight.
__device__ __forceinline__ void settle_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D>
__device__ __forceinline__ int swz_fp4_key(int r, int c) {
  return D == 128 ? (c ^ (((r >> 2) & 1) | (((r >> 5) & 1) << 1))) : (c ^ ((r >> 5) & 1));
}
template <int D>
__device__ __forceinline__ int swz_fp8_key(int r, int c) {
  return D == 128 ? (c ^ (((r >> 1) & 1) | (((r >> 2) & 1) << 1) | (((r >> 5) & 1) << 2)))
                  : (c ^ (((r >> 2) & 1) | (((r >> 5) & 1) << 1)));
}
// LDS dword slot of a key's scales inside a 64-key block: bits 4 and 5 swapped, so that the 32
// lanes of one 4-byte read pass (keys {0..3, 32..35, 4..7, ...}) hit 32 distinct banks
__device__ __forceinline__ int ks_slot(int key) { return (key & ~0x30) | ((key >> 1) & 0x10) | ((key << 1) & 0x20); }

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
  const float* nl;     // -fp32(LSE log2 e) [B*H][N]
  const float* ndelta;  // -Delta [B*H][N]
  uint16_t* dq;        // bf16 [B*H][N][D]
  uint16_t* dk;        // bf16 [B*Hkv][N][D]
  uint16_t* dv;
  int B, H, Hkv, N;
};

// ------------------------------------------------------------------------------------
// dK, dV. Workgroup: (batch, KV head, 128 keys); wave w owns keys k0 + 32w + (lane % 32).
template <int D>
struct DkdvSmem {
  static constexpr int QB = 64;                     // queries per staged block
  static constexpr int oQ = 0;                      // Q rows, MXFP4: QB x D/2
  static constexpr int oDO = oQ + QB * D / 2;       // dO rows, MXFP8: QB x D
  static constexpr int oQT = oDO + QB * D;          // Q^T rows along queries, MXFP8: D x QB
  static constexpr int oDOT = oQT + D * QB;         // dO^T rows: D x QB
  static constexpr int oQs = oDOT + D * QB;         // Q scales: [D/32 blocks (<= 2 used)][QB] dwords
  static constexpr int oDOs = oQs + 2 * QB * 4;     // dO scales, same layout
  static constexpr int oQTs = oDOs + 2 * QB * 4;    // Q^T scales: [2 query blocks][D] dwords
  static constexpr int oDOTs = oQTs + 2 * D * 4;    // dO^T scales
  static constexpr int oNL = oDOTs + 2 * D * 4;     // nl (fp32)
  static constexpr int oDL = oNL + QB * 4;          // Delta (fp32)
  static constexpr int buf = oDL + QB * 4;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreadsKV, 1) dkdv_kernel(BwdArgs a) {
  using L = DkdvSmem<D>;
  constexpr int QB = L::QB;
  constexpr int KS = D / 64;   // k-steps over D
  constexpr int DT = D / 32;   // 32-wide output tiles along D
  constexpr int QCH = D / 32;  // 16-byte chunks of a Q row
  constexpr int OCH = D / 16;  // 16-byte chunks of a dO row
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr float SCALE = inv_sqrt_d(D);
  // staging buffers: two for group 0, three for group 1 (which finishes each block one step
  // late); reused at a tile's end for the groups' partial dK, dV
  constexpr int kRed = 2 * kWavesB * DT * 16 * 64 * 4;
  constexpr int kSmem = 5 * L::buf > kRed ? 5 * L::buf : kRed;
  __shared__ __attribute__((aligned(16))) lds_char smem[kSmem];

  // the wave index is wave-uniform: readfirstlane lets the compiler keep what derives from it in
  // scalar registers and branch on it without exec masks
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5,
            col = lane & 31;
  // two groups of 4 waves: group grp takes the query blocks it = 2s + grp of each tile. Each
  // SIMD runs one wave of each group. Group 0 finishes a block within its step (S and dP
  // products, P and dS on the VALU, then the dV and dK products); group 1 issues the dV and dK
  // products of its previous block at the start of the next step, ahead of that step's S and dP
  // products, so that one wave of a SIMD has MFMA work queued while the other forms P and dS.
  const int grp = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int wv = __builtin_amdgcn_readfirstlane(wave & 3);
  lds_char* gsm = smem + grp * 2 * L::buf;
  const int nbuf = grp ? 3 : 2;
  const int N = a.N;
  const int ntile = (N + 127) / 128;
  // Consecutive workgroups cover all (batch, KV head) pairs of one tile position. Causal: the
  // workgroup at position pos runs key tile pos and then its mirror ntile-1-pos, so that every
  // workgroup carries the same number of query blocks.
  const int pos = (int)blockIdx.x / (a.B * a.Hkv);
  const int bg = (int)blockIdx.x % (a.B * a.Hkv);  // b * Hkv + g
  const int g = bg % a.Hkv, b = bg / a.Hkv;
  const int G = a.H / a.Hkv;
  const int ntw = (CAUSAL && ntile - 1 - pos != pos) ? 2 : 1;
  const int64_t bhkv = (int64_t)bg;

  // ---- staging of one query block (row bh, queries qb0 .. qb0+63) into buffer sb ----
  // Every region is filled by 64-lane loads (16 bytes per lane for rows, 4 or 1 byte for
  // scales) spread over the 4 waves; LDS slot P of a row region holds row P / chunks, chunk
  // (P % chunks) ^ swizzle(row). The per-lane source offsets inside a block are fixed, so they
  // are computed once; a block adds its uniform base. A block reaching past N takes the slow
  // path: rows past N read row N-1 and chunks past N the block's first chunk (finite data;
  // those queries are masked before they contribute).
  constexpr int nQ = QB * QCH / 64, nO = QB * OCH / 64, nT = D * 4 / 64;  // 64-lane loads per region
  constexpr int uQ = (nQ + kWavesB - 1) / kWavesB, uO = (nO + kWavesB - 1) / kWavesB, uT = (nT + kWavesB - 1) / kWavesB;
  // Load u of a region covers the rows 256/chunks * u further on; every swizzle reads only row
  // bits below 5 and those steps are multiples of 32, so load u keeps load 0's lane offset and
  // adds a uniform row step to its base.
  static_assert((256 / QCH) % 32 == 0 && (256 / OCH) % 32 == 0, "row steps keep the swizzle");
  const int nsb = N / 32;
  auto stage = [&](int64_t bh, int qb0, lds_char* sb) __attribute__((always_inline)) {
    const uint32_t sbl = lds_addr(sb);
    if (qb0 + QB <= N) {
      // the lane offsets, formed here from an opaque copy of the lane index: kept live across
      // the block they would take three registers, which the kernel does not have to spare
      int ln = lane;
      asm volatile("" : "+v"(ln));
      const int P = wv * 64 + ln;
      const int rq = P / QCH, ro = P / OCH, d = P / 4;
      const uint32_t offQ = (uint32_t)(rq * (D / 2) + swz_fp4_row<D>(rq, P % QCH) * 16);
      const uint32_t offO = (uint32_t)(ro * D + swz_fp8_row<D>(ro, P % OCH) * 16);
      const uint32_t offT = (uint32_t)(d * N + ((P % 4) ^ sw4_lin(d)) * 16);
      const uint8_t* bq = a.q + (bh * N + qb0) * (D / 2);
      const uint8_t* bo = a.dod + (bh * N + qb0) * D;
      const uint8_t* bt = a.q8 + bh * D * N + qb0;
      const uint8_t* bto = a.doq + bh * D * N + qb0;
#pragma unroll
      for (int u = 0; u < uQ; u++)
        if (wv + u * kWavesB < nQ) dma16_async(bq + u * (256 / QCH) * (D / 2), offQ, sbl + L::oQ + (wv + u * kWavesB) * 1024);
#pragma unroll
      for (int u = 0; u < uO; u++)
        if (wv + u * kWavesB < nO) dma16_async(bo + u * (256 / OCH) * D, offO, sbl + L::oDO + (wv + u * kWavesB) * 1024);
#pragma unroll
      for (int u = 0; u < uT; u++)
        if (wv + u * kWavesB < nT) {
          dma16_async(bt + (int64_t)u * 64 * N, offT, sbl + L::oQT + (wv + u * kWavesB) * 1024);
          dma16_async(bto + (int64_t)u * 64 * N, offT, sbl + L::oDOT + (wv + u * kWavesB) * 1024);
        }
    } else {
      const int qmax = N - 1;
      for (int i = wv; i < nQ; i += kWavesB) {
        const int P = i * 64 + lane, r = P / QCH;
        const int q = min(qb0 + r, qmax);
        dma16_async(a.q, (uint32_t)((bh * N + q) * (D / 2) + swz_fp4_row<D>(r, P % QCH) * 16), sbl + L::oQ + i * 1024);
      }
      for (int i = wv; i < nO; i += kWavesB) {
        const int P = i * 64 + lane, r = P / OCH;
        const int q = min(qb0 + r, qmax);
        dma16_async(a.dod, (uint32_t)((bh * N + q) * D + swz_fp8_row<D>(r, P % OCH) * 16), sbl + L::oDO + i * 1024);
      }
      for (int i = wv; i < nT; i += kWavesB) {
        const int P = i * 64 + lane, d = P / 4;
        const int c = (P % 4) ^ sw4_lin(d);
        const int cc = (qb0 + c * 16 < N) ? c : 0;
        const uint32_t off = (uint32_t)((bh * D + d) * N + qb0 + cc * 16);
        dma16_async(a.q8, off, sbl + L::oQT + i * 1024);
        dma16_async(a.doq, off, sbl + L::oDOT + i * 1024);
      }
    }
    // per-row scales, nl and Delta (rows past N clamped), and the Q^T / dO^T scales of query
    // blocks qb0/32 and qb0/32 + 1 for every d
    const uint32_t rowq = (uint32_t)(bh * N + min(qb0 + lane, N - 1));
    if (wv == 0) {
      if constexpr (D == 128) {
        dma4_async(a.qs, rowq * 4, sbl + L::oQs);
        dma4_async(a.dods, rowq * 4, sbl + L::oDOs);
      } else {
        // two scale bytes per row, one zero-extended dword slot each
        dma1_async(a.qs, rowq * 2, sbl + L::oQs);
        dma1_async(a.dods, rowq * 2, sbl + L::oDOs);
        dma1_async(a.qs, rowq * 2 + 1, sbl + L::oQs + QB * 4);
        dma1_async(a.dods, rowq * 2 + 1, sbl + L::oDOs + QB * 4);
      }
    } else if (wv == 1) {
      dma4_async(reinterpret_cast<const uint8_t*>(a.nl), rowq * 4, sbl + L::oNL);
      dma4_async(reinterpret_cast<const uint8_t*>(a.ndelta), rowq * 4, sbl + L::oDL);
    }
#pragma unroll
    for (int u = 0; u < (2 * (D / 64) + kWavesB - 1) / kWavesB; u++) {
      const int i = wv + u * kWavesB;
      if (i < 2 * (D / 64)) {
        const int blk = i / (D / 64), d0 = (i % (D / 64)) * 64;
        const uint32_t off = (uint32_t)((bh * D + d0 + lane) * nsb + min(qb0 / 32 + blk, nsb - 1));
        dma1_async(a.q8s, off, sbl + L::oQTs + (blk * D + d0) * 4);
        dma1_async(a.doqs, off, sbl + L::oDOTs + (blk * D + d0) * 4);
      }
    }
  };

  // Byte offsets of this lane's fragment reads inside a staged block. Tile t reads the Q / dO
  // row r = 32t + perm32(col) and the Q^T / dO^T row d = 32t + col; every swizzle reads only
  // row bits below 5, so tile t's offsets are tile 0's plus a constant.
  const int pc = perm32(col);
  uint32_t oq[KS], od[KS][2];
#pragma unroll
  for (int ks = 0; ks < KS; ks++) {
    oq[ks] = (uint32_t)(L::oQ + pc * (D / 2) + swz_fp4_row<D>(pc, 2 * ks + half) * 16);
    od[ks][0] = (uint32_t)(L::oDO + pc * D + swz_fp8_row<D>(pc, 4 * ks + half) * 16);
    od[ks][1] = (uint32_t)(L::oDO + pc * D + swz_fp8_row<D>(pc, 4 * ks + 2 + half) * 16);
  }
  const uint32_t orsc = (uint32_t)((D == 128 ? pc : half * QB + pc) * 4);  // row scales
  const uint32_t onl = (uint32_t)(half * 64);                                // nl / Delta
  const int swc = sw4_lin(col);
  const uint32_t ot0 = (uint32_t)(col * QB + (half ^ swc) * 16), ot1 = (uint32_t)(col * QB + ((2 + half) ^ swc) * 16);
  const uint32_t otsc = (uint32_t)((half * D + col) * 4);                    // Q^T / dO^T scales

  for (int tw = 0; tw < ntw; tw++) {
  const int kt = tw == 0 ? pos : ntile - 1 - pos;
  const int k0 = kt * 128;
  const int kw0 = k0 + wv * 32;
  const int kl = kw0 + col;  // this lane's key (B operand column / A operand row)
  const bool kvalid = kl < N;

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

  // query blocks: the causal range starts at the block holding key k0
  const int qstart = CAUSAL ? (k0 / QB) * QB : 0;
  const int nqb = (N - qstart + QB - 1) / QB;
  const int total = G * nqb;
  // block-major with the query heads innermost; the first tile (the longer, from its diagonal to
  // the last query block) runs from the last block down, the mirror tile from its diagonal up. At
  // block step t every workgroup of a KV group then stages block last - t or t - 2 of the same
  // head, whatever its tile position: the group's workgroups share one XCD's L2 (they are
  // numbered onto it) and read each staged block from HBM about once
  auto block_row = [&](int it) -> int64_t { return (int64_t)b * a.H + (int64_t)g * G + it % G; };
  auto block_q0 = [&](int it) -> int { return qstart + (tw == 0 ? nqb - 1 - it / G : it / G) * QB; };

  if (grp < total) stage(block_row(grp), block_q0(grp), gsm);
  wait_dma();
  __builtin_amdgcn_s_barrier();
  const int nsup = (total + 1) / 2;
  // dV += P^T dO, dK += dS^T Q for the block staged at blk, from its P and dS codes (contraction
  // over the block's 64 queries)
  auto dvdk = [&](const lds_char* blk, const v8i& pa, const v8i& sa, int psc, int ssc) __attribute__((always_inline)) {
  #pragma unroll
    for (int t = 0; t < DT; t++) {
      const lds_char* dorow = blk + L::oDOT + t * 32 * QB;
      const lds_char* qrow = blk + L::oQT + t * 32 * QB;
      const uint4 a0 = *reinterpret_cast<const uint4*>(dorow + ot0);
      const uint4 a1 = *reinterpret_cast<const uint4*>(dorow + ot1);
      const uint4 b0 = *reinterpret_cast<const uint4*>(qrow + ot0);
      const uint4 b1 = *reinterpret_cast<const uint4*>(qrow + ot1);
      v8i bo, bq;
      bo[0] = a0.x; bo[1] = a0.y; bo[2] = a0.z; bo[3] = a0.w; bo[4] = a1.x; bo[5] = a1.y; bo[6] = a1.z; bo[7] = a1.w;
      bq[0] = b0.x; bq[1] = b0.y; bq[2] = b0.z; bq[3] = b0.w; bq[4] = b1.x; bq[5] = b1.y; bq[6] = b1.z; bq[7] = b1.w;
      const int dosc = (int)*reinterpret_cast<const lds_u32*>(blk + L::oDOTs + otsc + t * 128);
      const int qtsc = (int)*reinterpret_cast<const lds_u32*>(blk + L::oQTs + otsc + t * 128);
      dvacc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(pa, bo, dvacc[t], psc, dosc);
      dkacc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(sa, bq, dkacc[t], ssc, qtsc);
    }
  };
  // the group's buffer of the current block (group 0: step % 2, group 1: step % 3), and group 1's
  // pending block: its P and dS codes and scales, finished at the start of the next step
  int bc = 0;
  v8i pa1, sa1;
  int psc1 = 127, ssc1 = 127;
  // One step: block 2 sp + grp of each group. MASK: the causal diagonal and the ragged query end
  // are applied; the steps whose blocks need neither run a body without them (two VALU
  // instructions per score fewer).
  auto step = [&](int sp, auto MC) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(MC)::value;
    const int it = 2 * sp + grp;
    const int bn = bc + 1 == nbuf ? 0 : bc + 1;  // block it + 2
    const lds_char* cur = gsm + bc * L::buf;
    if (grp && sp > 0 && it - 2 < total) dvdk(gsm + (bc == 0 ? nbuf - 1 : bc - 1) * L::buf, pa1, sa1, psc1, ssc1);
    if (it + 2 < total) stage(block_row(it + 2), block_q0(it + 2), gsm + bn * L::buf);
    if (it < total) {
      const int qb0 = block_q0(it);
      // Keys past N need no mask: their K and V fragments are zero, their rows of dK and dV
      // are never stored, and the MX blocks of P and dS run along queries, within one key.
      {
        v8i pa, sa;
        int pscale[2], sscale[2];
  #pragma unroll
        for (int t = 0; t < 2; t++) {
          // ---- S and dP tile t: lane = key kl; register i of half h = query qb0 + 32t + 16h + i ----
          int qsc, dsc;
          if constexpr (D == 128) {
            qsc = (int)(*reinterpret_cast<const lds_u32*>(cur + L::oQs + orsc + t * 128) >> (8 * half));
            dsc = (int)(*reinterpret_cast<const lds_u32*>(cur + L::oDOs + orsc + t * 128) >> (8 * half));
          } else {
            qsc = (int)*reinterpret_cast<const lds_u32*>(cur + L::oQs + orsc + t * 128);
            dsc = (int)*reinterpret_cast<const lds_u32*>(cur + L::oDOs + orsc + t * 128);
          }
          // dP accumulates onto -Delta of its query (register i: query qb0 + 32t + 16 half + i),
          // so the MFMA hands out dP - Delta
          v16f s, dp;
  #pragma unroll
          for (int i4 = 0; i4 < 4; i4++) {
            const float4 nd4 = *reinterpret_cast<const float4*>(cur + L::oDL + onl + t * 128 + i4 * 16);
            dp[4 * i4] = nd4.x; dp[4 * i4 + 1] = nd4.y; dp[4 * i4 + 2] = nd4.z; dp[4 * i4 + 3] = nd4.w;
          }
  #pragma unroll
          for (int i = 0; i < 16; i++) s[i] = 0.0f;
  #pragma unroll
          for (int ks = 0; ks < KS; ks++) {
            const uint4 qa = *reinterpret_cast<const uint4*>(cur + oq[ks] + t * 32 * (D / 2));
            v8i af;
            af[0] = qa.x; af[1] = qa.y; af[2] = qa.z; af[3] = qa.w;
            const uint4 d0 = *reinterpret_cast<const uint4*>(cur + od[ks][0] + t * 32 * D);
            const uint4 d1 = *reinterpret_cast<const uint4*>(cur + od[ks][1] + t * 32 * D);
            v8i bfr;
            bfr[0] = d0.x; bfr[1] = d0.y; bfr[2] = d0.z; bfr[3] = d0.w;
            bfr[4] = d1.x; bfr[5] = d1.y; bfr[6] = d1.z; bfr[7] = d1.w;
            if (ks == 0) {
              s = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(af, kf[0], s, qsc, (int)ksc);
              dp = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(bfr, vf[0], dp, dsc, (int)vsc);
            } else {
              s = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(af, kf[KS - 1], s, qsc, (int)ksc);
              dp = mfma_scaled<kFmtFP8, kFmtFP8, 2, 2>(bfr, vf[KS - 1], dp, dsc, (int)vsc);
            }
          }
          // ---- P, dS; MXFP8 along queries (block = this tile = lane pair) ----
          const int qrow0 = t * 32 + half * 16;
          // register i (query qb0 + qrow0 + i) is visible iff lo <= i < hi: the causal diagonal
          // and the ragged query end (hi is clamped at 0 for a group of 16 queries wholly past
          // N); each P is then ANDed with the sign-extended bit i of a per-lane mask (two VALU
          // instructions per score, where a compare and a select would take three)
          uint32_t vis = 0xFFFFu;
          if constexpr (MASK) {
            const int hi = kvalid ? min(max(N - (qb0 + qrow0), 0), 16) : 0;
            const int lo = CAUSAL ? min(max(kl - (qb0 + qrow0), 0), hi) : 0;
            // bits lo .. hi-1 set (0 <= lo <= hi <= 16): the visible registers of this lane
            vis = ((1u << (hi - lo)) - 1u) << lo;
          }
          float p[16], dsv[16];
          float pmax = 0.0f, smax = 0.0f;
  #pragma unroll
          for (int i4 = 0; i4 < 4; i4++) {
            const float4 nl4 = *reinterpret_cast<const float4*>(cur + L::oNL + onl + t * 128 + i4 * 16);
            const float nlv[4] = {nl4.x, nl4.y, nl4.z, nl4.w};
  #pragma unroll
            for (int j = 0; j < 4; j++) {
              const int i = 4 * i4 + j;
              const float u = __builtin_fmaf(s[i], C, nlv[j]);
              float pv = __builtin_amdgcn_exp2f(u);
              if constexpr (MASK) {
                // register 0 of tile 0 in the lower half of the first query block is query 0
                if (i == 0 && t == 0 && qb0 == 0 && half == 0) pv = exp2_near_one(u, pv);
                // all-ones or zero from bit i of vis; zero bits give +0.0f
                uint32_t keep;
                asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(keep) : "v"(vis), "s"(i));
                pv = __uint_as_float(__float_as_uint(pv) & keep);
              }
              p[i] = pv;
              dsv[i] = pv * dp[i];
            }
          }
  #pragma unroll
          for (int i = 0; i < 16; i += 2) {
            pmax = max3f(pmax, p[i], p[i + 1]);
            smax = max3f(smax, fabsf(dsv[i]), fabsf(dsv[i + 1]));
          }
          pmax = max_across_halves(pmax);
          smax = max_across_halves(smax);
          const int ep = mx8_exponent(pmax), es = mx8_exponent(smax);
          pscale[t] = ep + 127;
          sscale[t] = es + 127;
          const float fp = scale_operand(ep), fs = scale_operand(es);
          const float ls = e4m3_limit(es);
  #pragma unroll
          for (int w = 0; w < 4; w++) {
            // P is finite and >= +0 (masked entries are +0): saturated after the conversion
            pa[4 * t + w] = (int)sat_e4m3_nonneg(pack4_fp8_scaled(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3], fp));
            sa[4 * t + w] = (int)pack4_fp8_scaled(
                __builtin_amdgcn_fmed3f(dsv[4 * w], -ls, ls), __builtin_amdgcn_fmed3f(dsv[4 * w + 1], -ls, ls),
                __builtin_amdgcn_fmed3f(dsv[4 * w + 2], -ls, ls), __builtin_amdgcn_fmed3f(dsv[4 * w + 3], -ls, ls), fs);
          }
        }
        // lane r supplies block 0 (queries qb0..+31, tile 0), lane r+32 block 1 (tile 1)
        const int psc = half ? pscale[1] : pscale[0];
        const int ssc = half ? sscale[1] : sscale[0];
        // (both groups keep the codes, so that the pending ones are dead within a block)
        pa1 = pa;
        sa1 = sa;
        psc1 = psc;
        ssc1 = ssc;
        if (!grp) dvdk(cur, pa, sa, psc, ssc);
            }
    }
    // the next blocks have landed (each wave waits for its own loads); a buffer is staged again
    // only after every wave is past the step that last read it (group 0: this block's, group 1:
    // the previous block's, whose dV/dK products ran at this step's start)
    wait_dma();
    __builtin_amdgcn_s_barrier();
    bc = bn;
  };
  // The blocks that need the mask sit at the ends of the walk: the two on the causal diagonal
  // (query blocks k0 and k0 + 64; no query block precedes them) and a ragged last query block.
  // Walk positions [ka, kb) need neither; a step takes the unmasked body when the blocks of both
  // groups (it = 2 sp and 2 sp + 1) lie there, every other step the masked one.
  const bool ragged = qstart + nqb * QB > N;
  const int ndiag = CAUSAL ? min(2, nqb) : 0;
  const int ka = tw == 0 ? (ragged ? 1 : 0) : ndiag;
  const int kb = tw == 0 ? nqb - ndiag : nqb - (ragged ? 1 : 0);
  const int spa = min((ka * G + 1) / 2, nsup);
  const int spb = max(min(kb * G / 2, nsup), spa);
  for (int sp = 0; sp < spa; sp++) step(sp, std::true_type());
  for (int sp = spa; sp < spb; sp++) step(sp, std::false_type());
  for (int sp = spb; sp < nsup; sp++) step(sp, std::true_type());
  // group 1's last block (the loop's last step is 2 (nsup - 1) + 1)
  if (grp && nsup > 0 && 2 * (nsup - 1) + 1 < total) dvdk(gsm + (bc == 0 ? nbuf - 1 : bc - 1) * L::buf, pa1, sa1, psc1, ssc1);
  // every wave is past its reads of the staged blocks before the reduction area overwrites them
  __syncthreads();

  // ---- the two groups' partial sums: group 1 hands over its dV, group 0 its dK ----
  // area [quantity][wave][t][i/4][lane] (float4 slots): registers 4(i/4) .. 4(i/4)+3 of tile t;
  // each wave addresses its part from one base plus offsets below 16 KB
  {
    auto part = [&](int qn) __attribute__((always_inline)) {
      return smem + (qn * kWavesB + wv) * (DT * 4 * 1024) + lane * 16;
    };
    lds_char* wr = part(grp ? 0 : 1);
    if (grp) {
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          *reinterpret_cast<float4*>(wr + (t * 4 + j) * 1024) =
              make_float4(dvacc[t][4 * j], dvacc[t][4 * j + 1], dvacc[t][4 * j + 2], dvacc[t][4 * j + 3]);
    } else {
#pragma unroll
      for (int t = 0; t < DT; t++)
#pragma unroll
        for (int j = 0; j < 4; j++)
          *reinterpret_cast<float4*>(wr + (t * 4 + j) * 1024) =
              make_float4(dkacc[t][4 * j], dkacc[t][4 * j + 1], dkacc[t][4 * j + 2], dkacc[t][4 * j + 3]);
    }
    __syncthreads();
    // ---- row R of the output tiles is key kw0 + R, column d = 32t + lane%32; group 0 stores
    // dV, group 1 dK ----
    const lds_char* rd = part(grp ? 1 : 0);
    uint16_t* out = grp ? a.dk : a.dv;
    const float osc = grp ? SCALE : 1.0f;
#pragma unroll
    for (int t = 0; t < DT; t++)
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const float4 o = *reinterpret_cast<const float4*>(rd + (t * 4 + j) * 1024);
        const float ov[4] = {o.x, o.y, o.z, o.w};
#pragma unroll
        for (int c = 0; c < 4; c++) {
          const int i = 4 * j + c;
          const float v = (grp ? dkacc[t][i] : dvacc[t][i]) + ov[c];
          const int key = kw0 + 8 * j + 4 * half + c;
          if (key < N) out[(bhkv * N + key) * D + t * 32 + col] = (uint16_t)bf16_bits(v * osc);
        }
      }
  }
  // the reduction area is the next tile's staging space
  __syncthreads();
  }
}

// dQ epilogue of one wave that holds a [32 x D] fp32 tile transposed in the MFMA C layout
// (acc[t][4a + i] is column d = 32t + 8a + 4*(lane / 32) + i of row q0 + (lane % 32)): each value
// times mul, rounded to bf16, goes to row q0 + (lane % 32) of o ([N, D], rows q >= N are not
// written). The rows pass through this wave's LDS tile `stage` (OStage<D>::kBytes) and leave as
// whole rows, 16 bytes per lane and D/8 lanes per row, so that every (non-temporal) store
// instruction writes 64*16 contiguous bytes. Every wave of the workgroup calls it (it holds
// workgroup barriers), after the last read of whatever LDS `stage` overlaps.
template <int D>
__device__ __forceinline__ void store_rows_bf16(const v16f (&acc)[D / 32], float mul, uint16_t* o, int N, int q0,
                                                int lane, uint8_t* stage) {
#pragma clang fp contract(off)
  constexpr int RS = OStage<D>::kRow;
  constexpr int CPR = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;   // rows per store instruction
  const int half = lane >> 5, col = lane & 31;
  __syncthreads();  // every wave is past its last read of the LDS that `stage` overlaps
#pragma unroll
  for (int t = 0; t < D / 32; t++)
#pragma unroll
    for (int aa = 0; aa < 4; aa++) {
      uint2 w;
      w.x = bf16_rne(acc[t][4 * aa + 0] * mul) | (bf16_rne(acc[t][4 * aa + 1] * mul) << 16);
      w.y = bf16_rne(acc[t][4 * aa + 2] * mul) | (bf16_rne(acc[t][4 * aa + 3] * mul) << 16);
      *reinterpret_cast<uint2*>(stage + col * RS + (t * 32 + 8 * aa + 4 * half) * 2) = w;
    }
  __syncthreads();  // the tile is complete before any lane reads it back
  const int rr = lane / CPR, cc = lane % CPR;
#pragma unroll
  for (int i = 0; i < 32 / RPI; i++) {
    const int r = i * RPI + rr;
    const uint2 lo = *reinterpret_cast<const uint2*>(stage + r * RS + cc * 16);
    const uint2 hi = *reinterpret_cast<const uint2*>(stage + r * RS + cc * 16 + 8);
    if (q0 + r < N) {  // streaming store: the output is not read again by this kernel
      u32x4 w;
      w[0] = lo.x; w[1] = lo.y; w[2] = hi.x; w[3] = hi.y;
      __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(o + (int64_t)(q0 + r) * D + cc * 8));
    }
  }
}

// ------------------------------------------------------------------------------------
// dQ. Workgroup: (batch, query head, 128 queries); wave w owns queries q0 + 32w + lane % 32.
template <int D>
struct DqSmem {
  static constexpr int KB = 64;                  // keys per staged block
  static constexpr int oK = 0;                   // K rows, MXFP4: KB x D/2
  static constexpr int oV = oK + KB * D / 2;     // V rows, MXFP8 along D: KB x D
  static constexpr int oKT = oV + KB * D;        // K^T rows along keys, MXFP8: D x KB
  static constexpr int oKs = oKT + D * KB;       // K scales: [D/32 blocks (<= 2 used)][KB] dwords
  static constexpr int oVs = oKs + 2 * KB * 4;   // V scales, same layout
  static constexpr int oKTs = oVs + 2 * KB * 4;  // K^T scales: [2 key blocks][D] dwords
  static constexpr int buf = oKTs + 2 * D * 4;
};

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(kThreads, 2) dq_kernel(BwdArgs a) {
  using L = DqSmem<D>;
  constexpr int KB = L::KB;
  constexpr int KS = D / 64;
  constexpr int DT = D / 32;
  constexpr int KCH = D / 32, VCH = D / 16;
  constexpr float C = log2e_over_sqrt_d(D);
  constexpr float SCALE = inv_sqrt_d(D);
  __shared__ __attribute__((aligned(16))) lds_char smem[2 * L::buf];

  // the wave index is wave-uniform: readfirstlane lets the compiler keep what derives from it in
  // scalar registers and branch on it without exec masks
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, half = lane >> 5,
            col = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int N = a.N;
  const int nqt = (N + 127) / 128;
  // consecutive workgroups cover all (batch, head) rows of one query tile; the causal route's
  // heaviest tiles (latest queries) come first
  const int qt0 = (int)blockIdx.x / (a.B * a.H);
  int bh = (int)blockIdx.x % (a.B * a.H);
  // workgroup i runs on XCD i % 8: give each XCD a contiguous range of heads, so that the query
  // heads of a KV group share that XCD's L2 for the group's K and V
  if ((a.B * a.H) % 8 == 0) bh = (bh % 8) * (a.B * a.H / 8) + bh / 8;
  const int qt = CAUSAL ? nqt - 1 - qt0 : qt0;
  const int h = bh % a.H, b = bh / a.H;
  const int64_t bhkv = (int64_t)b * a.Hkv + h / (a.H / a.Hkv);
  const int q0 = qt * 128;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + col;
  const bool qvalid = qi < N;

  // this lane's Q (MXFP4) and dO (MXFP8 along D) fragments: B operands of S^T and dP^T
  v8i qf[KS], df[KS];
  uint32_t qsc = 0x7F7F7F7Fu, dsc = 0x7F7F7F7Fu;
  float nl = 0.0f, ndl = 0.0f;
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
      nl = a.nl[(int64_t)bh * N + qi];
      ndl = a.ndelta[(int64_t)bh * N + qi];
    }
    qsc >>= 8 * half;
    dsc >>= 8 * half;
  }
  settle_vmem();

  v16f acc[DT];
#pragma unroll
  for (int t = 0; t < DT; t++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[t][r] = 0.0f;

  // ---- staging of one 64-key block kb0 into buffer sb (same scheme as dkdv_kernel's) ----
  constexpr int nK = KB * KCH / 64, nV = KB * VCH / 64, nT = D * 4 / 64;
  constexpr int uK = (nK + kWavesB - 1) / kWavesB, uV = (nV + kWavesB - 1) / kWavesB, uT = (nT + kWavesB - 1) / kWavesB;
  // load u of the K and K^T regions: load 0's lane offset, base moved by a uniform row step of
  // 64 rows (the swizzles read row bits below 6); V rows step by 256 / VCH rows, which can flip
  // bit 5, so each V load keeps its own offset
  static_assert(uK == 1 || (256 / KCH) % 64 == 0, "K row steps keep the swizzle");
  uint32_t offK, offV[uV], offT;
  {
    const int P = wv * 64 + lane;
    const int rk = P / KCH, d = P / 4;
    offK = (uint32_t)(rk * (D / 2) + swz_fp4_key<D>(rk, P % KCH) * 16);
    offT = (uint32_t)(d * N + ((P % 4) ^ sw4_lin(d)) * 16);
  }
#pragma unroll
  for (int u = 0; u < uV; u++) {
    const int P = (wv + u * kWavesB) * 64 + lane, rv = P / VCH;
    offV[u] = (uint32_t)(rv * D + swz_fp8_key<D>(rv, P % VCH) * 16);
  }
  const int nsb = N / 32;
  auto stage = [&](int kb0, lds_char* sb) __attribute__((always_inline)) {
    const uint32_t sbl = lds_addr(sb);
    if (kb0 + KB <= N) {
      const uint8_t* bk = a.k + (bhkv * N + kb0) * (D / 2);
      const uint8_t* bv = a.v8 + (bhkv * N + kb0) * D;
      const uint8_t* bt = a.k8 + bhkv * D * N + kb0;
#pragma unroll
      for (int u = 0; u < uK; u++)
        if (wv + u * kWavesB < nK) dma16_async(bk + u * (256 / KCH) * (D / 2), offK, sbl + L::oK + (wv + u * kWavesB) * 1024);
#pragma unroll
      for (int u = 0; u < uV; u++)
        if (wv + u * kWavesB < nV) dma16_async(bv, offV[u], sbl + L::oV + (wv + u * kWavesB) * 1024);
#pragma unroll
      for (int u = 0; u < uT; u++)
        if (wv + u * kWavesB < nT) dma16_async(bt + (int64_t)u * 64 * N, offT, sbl + L::oKT + (wv + u * kWavesB) * 1024);
    } else {
      const int kmax = N - 1;
      for (int i = wv; i < nK; i += kWavesB) {
        const int P = i * 64 + lane, r = P / KCH;
        const int kk = min(kb0 + r, kmax);
        dma16_async(a.k, (uint32_t)((bhkv * N + kk) * (D / 2) + swz_fp4_key<D>(r, P % KCH) * 16), sbl + L::oK + i * 1024);
      }
      for (int i = wv; i < nV; i += kWavesB) {
        const int P = i * 64 + lane, r = P / VCH;
        const int kk = min(kb0 + r, kmax);
        dma16_async(a.v8, (uint32_t)((bhkv * N + kk) * D + swz_fp8_key<D>(r, P % VCH) * 16), sbl + L::oV + i * 1024);
      }
      for (int i = wv; i < nT; i += kWavesB) {
        const int P = i * 64 + lane, d = P / 4;
        const int c = (P % 4) ^ sw4_lin(d);
        const int cc = (kb0 + c * 16 < N) ? c : 0;
        dma16_async(a.k8, (uint32_t)((bhkv * D + d) * N + kb0 + cc * 16), sbl + L::oKT + i * 1024);
      }
    }
    // scale slot s holds key ks_slot(s)
    const uint32_t rowk = (uint32_t)(bhkv * N + min(kb0 + ks_slot(lane), N - 1));
    if (wv == 0) {
      if constexpr (D == 128) {
        dma4_async(a.ks, rowk * 4, sbl + L::oKs);
        dma4_async(a.v8s, rowk * 4, sbl + L::oVs);
      } else {
        dma1_async(a.ks, rowk * 2, sbl + L::oKs);
        dma1_async(a.v8s, rowk * 2, sbl + L::oVs);
        dma1_async(a.ks, rowk * 2 + 1, sbl + L::oKs + KB * 4);
        dma1_async(a.v8s, rowk * 2 + 1, sbl + L::oVs + KB * 4);
      }
    }
#pragma unroll
    for (int u = 0; u < (2 * (D / 64) + kWavesB - 1) / kWavesB; u++) {
      const int i = wv + u * kWavesB;
      if (i < 2 * (D / 64)) {
        const int blk = i / (D / 64), d0 = (i % (D / 64)) * 64;
        dma1_async(a.k8s, (uint32_t)((bhkv * D + d0 + lane) * nsb + min(kb0 / 32 + blk, nsb - 1)),
                   sbl + L::oKTs + (blk * D + d0) * 4);
      }
    }
  };

  // lane-constant K^T fragment offsets of row d = 32t + col (sw4_lin reads bits 2-3 of d, which
  // the 32-row tile step leaves unchanged)
  const int kto0 = L::oKT + col * KB + (half ^ sw4_lin(col)) * 16;
  const int kto1 = L::oKT + col * KB + ((2 + half) ^ sw4_lin(col)) * 16;
  // A-operand key rows of this lane: tile t register i holds key kb0 + 32*half + 16t + i
  int krow[2];
#pragma unroll
  for (int t = 0; t < 2; t++) krow[t] = (((col >> 2) & 1) << 5) + t * 16 + ((col >> 3) << 2) + (col & 3);

  const int kend = CAUSAL ? min(N, q0 + 128) : N;
  const int nkb = (kend + KB - 1) / KB;
  stage(0, smem);
  wait_dma();
  __builtin_amdgcn_s_barrier();
  // key block j staged at cur; the loop below is unrolled by two so that cur is a
  // compile-time buffer and every LDS fragment address a lane constant plus an immediate
  auto kblock = [&](int j, const lds_char* cur) __attribute__((always_inline)) {
    const int kb0 = j * KB;
    if (!CAUSAL || kb0 <= qw0 + 31) {
      // ---- S^T, dP^T: lane = query qi; register i of tile t = key kb0 + 32 half + 16 t + i ----
      v16f s[2], dp[2];
#pragma unroll
      for (int t = 0; t < 2; t++) {
        const int key = krow[t];
        int ksc, vsc;
        if constexpr (D == 128) {
          ksc = (int)(reinterpret_cast<const lds_u32*>(cur + L::oKs)[ks_slot(key)] >> (8 * half));
          vsc = (int)(reinterpret_cast<const lds_u32*>(cur + L::oVs)[ks_slot(key)] >> (8 * half));
        } else {
          ksc = (int)reinterpret_cast<const lds_u32*>(cur + L::oKs)[half * KB + ks_slot(key)];
          vsc = (int)reinterpret_cast<const lds_u32*>(cur + L::oVs)[half * KB + ks_slot(key)];
        }
        // dP^T accumulates onto -Delta of the lane's query, so the MFMA hands out dP - Delta
#pragma unroll
        for (int i = 0; i < 16; i++) {
          s[t][i] = 0.0f;
          dp[t][i] = ndl;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ks++) {
          const uint4 kk = *reinterpret_cast<const uint4*>(cur + L::oK + key * (D / 2) + swz_fp4_key<D>(key, 2 * ks + half) * 16);
          v8i af;
          af[0] = kk.x; af[1] = kk.y; af[2] = kk.z; af[3] = kk.w;
          const uint8_t* vrow = cur + L::oV + key * D;
          const uint4 v0 = *reinterpret_cast<const uint4*>(vrow + swz_fp8_key<D>(key, 4 * ks + half) * 16);
          const uint4 v1 = *reinterpret_cast<const uint4*>(vrow + swz_fp8_key<D>(key, 4 * ks + 2 + half) * 16);
          v8i vfr;
          vfr[0] = v0.x; vfr[1] = v0.y; vfr[2] = v0.z; vfr[3] = v0.w; vfr[4] = v1.x; vfr[5] = v1.y; vfr[6] = v1.z; vfr[7] = v1.w;
          if (ks == 0) {
            s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(af, qf[0], s[t], ksc, (int)qsc);
            dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(vfr, df[0], dp[t], vsc, (int)dsc);
          } else {
            s[t] = mfma_scaled<kFmtFP4, kFmtFP4, 2, 2>(af, qf[KS - 1], s[t], ksc, (int)qsc);
            dp[t] = mfma_scaled<kFmtFP8, kFmtFP8, 2, 2>(vfr, df[KS - 1], dp[t], vsc, (int)dsc);
          }
        }
      }
      // ---- dS, MXFP8 along keys: the lane's 32 keys are one block ----
      uint32_t pw[8];
      int es;
      auto dsblock = [&](auto MC) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(MC)::value;
        float dsv[32];
        float smax = 0.0f;
#pragma unroll
        for (int idx = 0; idx < 32; idx++) {
          const int t = idx >> 4, i = idx & 15;
          const float u = __builtin_fmaf(s[t][i], C, nl);
          float pv = __builtin_amdgcn_exp2f(u);
          if constexpr (MASK) {
            // key 0 of query 0 (register 0 of the lower half in the first key block)
            if (idx == 0 && kb0 == 0 && half == 0 && qi == 0) pv = exp2_near_one(u, pv);
            const int key = kb0 + half * 32 + idx;
            pv = (qvalid && key < N && (!CAUSAL || key <= qi)) ? pv : 0.0f;
          }
          dsv[idx] = pv * dp[t][i];
          smax = __builtin_elementwise_maximum(smax, fabsf(dsv[idx]));
        }
        es = mx8_exponent(smax);
        const float fs = scale_operand(es), ls = e4m3_limit(es);
#pragma unroll
        for (int w = 0; w < 8; w++)
          pw[w] = pack4_fp8_scaled(__builtin_amdgcn_fmed3f(dsv[4 * w], -ls, ls), __builtin_amdgcn_fmed3f(dsv[4 * w + 1], -ls, ls),
                                   __builtin_amdgcn_fmed3f(dsv[4 * w + 2], -ls, ls),
                                   __builtin_amdgcn_fmed3f(dsv[4 * w + 3], -ls, ls), fs);
      };
      // the mask is needed only on the causal diagonal or at a ragged end of the keys or queries
      const bool full = (!CAUSAL || kb0 + KB - 1 <= qw0) && kb0 + KB <= N && qw0 + 32 <= N;
      if (full) dsblock(std::false_type());
      else dsblock(std::true_type());
      // FP8 operand layout: bytes 0-15 of lanes r, r+32 form block 0, bytes 16-31 block 1
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
        const uint8_t* ktrow = cur + t * 32 * KB;
        const uint4 a0 = *reinterpret_cast<const uint4*>(ktrow + kto0);
        const uint4 a1 = *reinterpret_cast<const uint4*>(ktrow + kto1);
        v8i kfr;
        kfr[0] = a0.x; kfr[1] = a0.y; kfr[2] = a0.z; kfr[3] = a0.w; kfr[4] = a1.x; kfr[5] = a1.y; kfr[6] = a1.z; kfr[7] = a1.w;
        const int ktsc = (int)reinterpret_cast<const lds_u32*>(cur + L::oKTs)[half * D + d];
        acc[t] = mfma_scaled<kFmtFP8, kFmtFP8, 0, 0>(kfr, sb, acc[t], ktsc, ssc);
      }
    }
  };
  for (int j = 0; j < nkb; j += 2) {
    if (j + 1 < nkb) stage((j + 1) * KB, smem + L::buf);
    kblock(j, smem);
    wait_dma();
    __builtin_amdgcn_s_barrier();
    if (j + 1 >= nkb) break;
    if (j + 2 < nkb) stage((j + 2) * KB, smem);
    kblock(j + 1, smem + L::buf);
    wait_dma();
    __builtin_amdgcn_s_barrier();
  }

  // dQ = scale * dQ^T in bf16, whole rows through LDS (the staging buffers are free)
  static_assert(2 * L::buf >= kThreads / 64 * OStage<D>::kBytes, "output tiles fit the staging buffers");
  store_rows_bf16<D>(acc, SCALE, a.dq + (int64_t)bh * N * D, N, qw0, lane, smem + wave * OStage<D>::kBytes);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t stream) {
  const int ntile = (a.N + 127) / 128;
  // causal: one workgroup per mirror pair of key tiles
  const int npos = CAUSAL ? (ntile + 1) / 2 : ntile;
  dkdv_kernel<D, CAUSAL><<<dim3((unsigned)(npos * a.B * a.Hkv)), dim3(kThreadsKV), 0, stream>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dq_kernel<D, CAUSAL><<<dim3((unsigned)(ntile * a.B * a.H)), dim3(kThreads), 0, stream>>>(a);
  return hipGetLastError();
}

int64_t pad256(int64_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D) {
  const int64_t rows = B * H * N;
  // Delta and nl (fp32 each) + dO MXFP8 along D (codes + scales) + dO MXFP8 along queries
  // (codes + scales), each region padded to 256 bytes
  return (size_t)(2 * pad256(rows * 4) + 2 * (pad256(rows * D) + pad256(rows * D / 32)));
}

hipError_t launch_attn_bwd(const BwdLaunch& l, int D, int causal, hipStream_t stream) {
  const int64_t rows = (int64_t)l.B * l.H * l.N;
  uint8_t* ws = (uint8_t*)l.workspace;
  float* ndelta = (float*)ws;
  float* nl = (float*)(ws + pad256(rows * 4));
  uint8_t* dod = ws + 2 * pad256(rows * 4);
  uint8_t* dods = dod + pad256(rows * D);
  uint8_t* doq = dods + pad256(rows * D / 32);
  uint8_t* doqs = doq + pad256(rows * D);
  // dO's two MXFP8 views in one launch; the along-D job also reads O for -Delta and writes nl
  QuantTask views[2] = {{l.dout, dod, dods, (int64_t)l.B * l.H, kMXFP8, kAlongD},
                        {l.dout, doq, doqs, (int64_t)l.B * l.H, kMXFP8, kAlongSeq}};
  views[0].y = l.o;
  views[0].lse = l.lse;
  views[0].ndot = ndelta;
  views[0].nl = nl;
  hipError_t e = launch_quantize_batch(views, 2, l.N, D, stream);
  if (e != hipSuccess) return e;
  BwdArgs a;
  a.q = l.q; a.qs = l.qs; a.k = l.k; a.ks = l.ks;
  a.q8 = l.q8; a.q8s = l.q8s; a.k8 = l.k8; a.k8s = l.k8s; a.v8 = l.v8; a.v8s = l.v8s;
  a.dod = dod; a.dods = dods; a.doq = doq; a.doqs = doqs;
  a.nl = nl; a.ndelta = ndelta; a.dq = l.dq; a.dk = l.dk; a.dv = l.dv;
  a.B = l.B; a.H = l.H; a.Hkv = l.Hkv; a.N = l.N;
  if (D == 128) return causal ? launch_bwd_t<128, true>(a, stream) : launch_bwd_t<128, false>(a, stream);
  return causal ? launch_bwd_t<64, true>(a, stream) : launch_bwd_t<64, false>(a, stream);
}

}  // namespace fp4attn

// fwd_common.h -- pieces shared by the two forward kernels (the pipelined Direct-P kernel and
// the causal FP8 kernel): LDS layout of one key block, XOR swizzles, the direct global->LDS
// staging of a key block, the workgroup -> tile mapping, and small reductions.
#pragma once

#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace fp4attn {
namespace fwd {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

// LDS layout of one key block (K rows MXFP4, K scales, V^T rows, V^T scales).
template <int D, bool FP8V, int KB_ = key_block_for(D)>
struct Smem {
  static constexpr int KB = KB_;                             // keys per running-max update
  static constexpr int NSB = KB / 64;                        // 64-key sub-blocks (2 S^T tiles each)
  static constexpr int kRow = D / 2;                         // bytes of one MXFP4 K row
  static constexpr int kCh = D / 32;                         // 16-byte chunks per K row
  static constexpr int vRow = FP8V ? KB : KB / 2;            // bytes of one V^T row per block
  static constexpr int vCh = vRow / 16;                      // 16-byte chunks per V^T row
  static constexpr int vKeysPerCh = FP8V ? 16 : 32;
  static constexpr int vsRow = KB / 32;                      // V scale bytes per V^T row per block
  static constexpr int ksPerKey = D == 128 ? 1 : 2;          // LDS dwords of K scales per key
  // regions of one buffer, all filled by direct global->LDS loads:
  static constexpr int kBytes = KB * kRow;                   // K codes, swizzled 16-byte chunks
  static constexpr int ksOff = kBytes;                       // K scales: D=128 one dword (4 bytes) per
                                                             // key at dword ks_slot(key); D=64 one dword
                                                             // per scale byte b at b * KB + ks_slot(key)
  static constexpr int vOff = ksOff + KB * ksPerKey * 4;
  static constexpr int vsOff = vOff + D * vRow;              // V scales: one dword per scale byte, the
                                                             // 32-key block e of row d at e * D + d
  static constexpr int buf = vsOff + D * vsRow * 4;
  static constexpr int kDma = kBytes / 1024;                 // 16-byte-per-lane DMA instructions
  static constexpr int vDma = D * vRow / 1024;
  static constexpr int ksDma = KB * ksPerKey / 64;           // 4- or 1-byte-per-lane instructions
  static constexpr int vsDma = D * vsRow / 64;
};

// XOR swizzles of 16-byte chunks. A fragment read of 16 lanes touches, at one logical chunk,
// K rows {0..7, 32..39} (+4, +8, +16, +64 offsets) or V^T rows d..d+15; the swizzles below map
// those 16 reads to 16 distinct bank groups (64 banks x 4 bytes).
template <int D>
__device__ __forceinline__ int k_chunk(int key, int c) {
  if constexpr (D == 128) return c ^ (((key >> 2) & 1) | (((key >> 5) & 1) << 1));
  else return c ^ ((key >> 5) & 1);
}
template <int VCH>
__device__ __forceinline__ int v_chunk(int d, int c) {
  return c ^ ((d / (16 / VCH)) & (VCH - 1));
}

// LDS dword slot of a key's scales inside its block: bits 4 and 5 of the key swapped. The 32
// lanes of one 4-byte LDS read pass (which must hit distinct banks mod 32) read the keys
// {0..3, 32..35, 4..7, 36..39, ...} (+16, +64 offsets); swapped, those are 32 distinct dwords.
// An offset of 16 keys becomes 32 slots (key bit 4 is 0 in that set).
__host__ __device__ constexpr int ks_slot(int key) { return (key & ~0x30) | ((key >> 1) & 0x10) | ((key << 1) & 0x20); }

// max of 32 scores. IEEE-754-2019 maximum lowers to v_maximum3_f32 without the per-input
// canonicalization that fmaxf needs; scores are finite or -inf, so the two agree. Three-input
// groups keep the partial maxima independent.
__device__ __forceinline__ float fmax3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
__device__ __forceinline__ float max32(const v16f& a, const v16f& b) {
  const float m0 = fmax3(a[0], a[1], a[2]), m1 = fmax3(a[3], a[4], a[5]), m2 = fmax3(a[6], a[7], a[8]);
  const float m3 = fmax3(a[9], a[10], a[11]), m4 = fmax3(a[12], a[13], a[14]), m5 = fmax3(a[15], b[0], b[1]);
  const float m6 = fmax3(b[2], b[3], b[4]), m7 = fmax3(b[5], b[6], b[7]), m8 = fmax3(b[8], b[9], b[10]);
  const float m9 = fmax3(b[11], b[12], b[13]), m10 = __builtin_elementwise_maximum(b[14], b[15]);
  return fmax3(fmax3(m0, m1, m2), fmax3(m3, m4, m5), fmax3(fmax3(m6, m7, m8), m9, m10));
}

// Workgroup -> (batch*head, query tile). Consecutive workgroup ids go round-robin over the 8
// XCDs; the mapping gives each XCD a contiguous range of tiles, so the query tiles of one head
// share that XCD's L2 for the head's K and V. Causal: longest rows first.
struct Tile {
  int bh, qt;
};
__device__ __forceinline__ Tile tile_of_block(int N, bool causal, int qtile = kQueryTile) {
  const int nqt = (N + qtile - 1) / qtile;
  const int total = (int)gridDim.x;
  const int per = total / 8, rem = total % 8, xcd = (int)blockIdx.x % 8, slot = (int)blockIdx.x / 8;
  const int lin = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  Tile t;
  t.qt = lin % nqt;
  if (causal) t.qt = nqt - 1 - t.qt;
  t.bh = lin / nqt;
  return t;
}

// Direct global -> LDS staging of key block j of one KV head (global_load_lds: lane l of one
// instruction writes LDS base + size*l). The XOR swizzle is realized by the choice of the source
// chunk for each destination slot; slot i of a region is issued by wave i % NW. On a block that
// reaches past N the addresses are clamped into the tensors (rows past N read row N-1, chunks
// past N read the block's first chunk): those keys are masked to -inf before probabilities are
// formed, so only the finiteness of the clamped data matters. Addresses are a wave-uniform
// tensor base plus a per-lane 32-bit byte offset (tensors are below 2^31 bytes). ASYNC issues
// the loads as inline assembly (see dma16_async).
template <int D, bool FP8V, int NW = kWaves, bool ASYNC = false, int KB_ = key_block_for(D)>
struct KVStager {
  using L = Smem<D, FP8V, KB_>;
  static constexpr int KB = L::KB;
  static constexpr int kSlots = (L::kDma + NW - 1) / NW;
  static constexpr int vSlots = (L::vDma + NW - 1) / NW;
  static constexpr int ksSlots = (L::ksDma + NW - 1) / NW;
  static constexpr int vsSlots = (L::vsDma + NW - 1) / NW;
  static_assert(ksSlots == 1, "one K-scale DMA per wave at most");

  // destination: region byte offset `ro` inside the buffer sb (sbl = its LDS address)
  static __device__ __forceinline__ void d16(const uint8_t* base, uint32_t off, lds_char* sb, uint32_t sbl, int ro) {
    if constexpr (ASYNC) dma16_async(base, off, sbl + (uint32_t)ro);
    else dma16(base + off, sb + ro);
  }
  static __device__ __forceinline__ void d4(const uint8_t* base, uint32_t off, lds_char* sb, uint32_t sbl, int ro) {
    if constexpr (ASYNC) dma4_async(base, off, sbl + (uint32_t)ro);
    else dma4(base + off, sb + ro);
  }
  static __device__ __forceinline__ void d1(const uint8_t* base, uint32_t off, lds_char* sb, uint32_t sbl, int ro) {
    if constexpr (ASYNC) dma1_async(base, off, sbl + (uint32_t)ro);
    else dma1(base + off, sb + ro);
  }

  const FwdArgs* a;
  uint32_t k_head, ks_head, v_head, vs_head;  // byte offsets of this KV head's slabs
  uint32_t vrow_bytes;
  int nsblk, N, wave, lane;
  uint32_t k_off[kSlots], v_off[vSlots], vs_off[vsSlots], ks_off;

  __device__ __forceinline__ KVStager(const FwdArgs& args, int64_t bhkv, int wave_, int lane_) {
    a = &args;
    N = args.N;
    wave = __builtin_amdgcn_readfirstlane(wave_);
    lane = lane_;
    vrow_bytes = FP8V ? (uint32_t)N : (uint32_t)N / 2;
    nsblk = N / 32;
    k_head = (uint32_t)(bhkv * N * (D / 2));
    ks_head = (uint32_t)(bhkv * N * (D / 32));
    v_head = (uint32_t)(bhkv * D * vrow_bytes);
    vs_head = (uint32_t)(bhkv * D * nsblk);
#pragma unroll
    for (int u = 0; u < kSlots; u++) {
      const int P = (wave + u * NW) * 64 + lane;
      const int key = P / L::kCh, c = (P % L::kCh) ^ k_chunk<D>(key, 0);
      k_off[u] = (uint32_t)(key * (D / 2) + c * 16);
    }
#pragma unroll
    for (int u = 0; u < vSlots; u++) {
      const int P = (wave + u * NW) * 64 + lane;
      const int d = P / L::vCh, c = (P % L::vCh) ^ v_chunk<L::vCh>(d, 0);
      v_off[u] = (uint32_t)(d * vrow_bytes + c * 16);
    }
    {
      // K-scale slot P holds key ks_slot(P) (D=128), or byte P / KB of key ks_slot(P % KB) (D=64)
      const int P = wave * 64 + lane;
      ks_off = D == 128 ? (uint32_t)(ks_slot(P) * 4) : (uint32_t)(ks_slot(P % KB) * 2 + P / KB);
    }
#pragma unroll
    for (int u = 0; u < vsSlots; u++) {
      // V-scale slot P holds 32-key block P / D of row P % D
      const int P = (wave + u * NW) * 64 + lane;
      vs_off[u] = (uint32_t)((P % D) * nsblk + P / D);
    }
  }

  // K rows and K scales of block j
  __device__ __forceinline__ void issue_k(int j, lds_char* sb) const {
    const int kb0 = j * KB;
    const uint32_t sbl = lds_addr(sb);
    if (kb0 + KB <= N) {
      const uint32_t kb = k_head + (uint32_t)kb0 * (D / 2);
      const uint32_t ksb = ks_head + (uint32_t)kb0 * (D / 32);
#pragma unroll
      for (int u = 0; u < kSlots; u++)
        if (wave + u * NW < L::kDma) d16(a->k, kb + k_off[u], sb, sbl, (wave + u * NW) * 1024);
      if (wave < L::ksDma) {
        if constexpr (D == 128) d4(a->ks, ksb + ks_off, sb, sbl, L::ksOff + wave * 256);
        else d1(a->ks, ksb + ks_off, sb, sbl, L::ksOff + wave * 256);
      }
      return;
    }
#pragma unroll
    for (int i = wave; i < L::kDma; i += NW) {
      const int P = i * 64 + lane;
      const int key = P / L::kCh, c = (P % L::kCh) ^ (k_chunk<D>(key, 0));
      const int gk = min(kb0 + key, N - 1);
      d16(a->k, k_head + (uint32_t)gk * (D / 2) + c * 16, sb, sbl, i * 1024);
    }
#pragma unroll
    for (int i = wave; i < L::ksDma; i += NW) {
      const int P = i * 64 + lane;
      if constexpr (D == 128) {
        const int gk = min(kb0 + ks_slot(P), N - 1);
        d4(a->ks, ks_head + (uint32_t)gk * 4, sb, sbl, L::ksOff + i * 256);
      } else {
        const int gk = min(kb0 + ks_slot(P % KB), N - 1);
        d1(a->ks, ks_head + (uint32_t)gk * 2 + P / KB, sb, sbl, L::ksOff + i * 256);
      }
    }
  }

  // V^T rows and V scales of block j
  __device__ __forceinline__ void issue_v(int j, lds_char* sb) const {
    const int kb0 = j * KB;
    const uint32_t sbl = lds_addr(sb);
    if (kb0 + KB <= N) {
      const uint32_t vb = v_head + (uint32_t)(FP8V ? kb0 : kb0 / 2);
      const uint32_t vsb = vs_head + (uint32_t)(kb0 / 32);
#pragma unroll
      for (int u = 0; u < vSlots; u++)
        if (wave + u * NW < L::vDma) d16(a->v, vb + v_off[u], sb, sbl, L::vOff + (wave + u * NW) * 1024);
#pragma unroll
      for (int u = 0; u < vsSlots; u++)
        if (wave + u * NW < L::vsDma) d1(a->vs, vsb + vs_off[u], sb, sbl, L::vsOff + (wave + u * NW) * 256);
      return;
    }
#pragma unroll
    for (int i = wave; i < L::vDma; i += NW) {
      const int P = i * 64 + lane;
      const int d = P / L::vCh, c = (P % L::vCh) ^ v_chunk<L::vCh>(d, 0);
      const int cc = (kb0 + c * L::vKeysPerCh < N) ? c : 0;
      d16(a->v, v_head + (uint32_t)d * vrow_bytes + (uint32_t)(FP8V ? kb0 : kb0 / 2) + cc * 16, sb, sbl,
          L::vOff + i * 1024);
    }
#pragma unroll
    for (int i = wave; i < L::vsDma; i += NW) {
      const int P = i * 64 + lane;
      const int d = P % D, e = P / D;
      d1(a->vs, vs_head + (uint32_t)(d * nsblk + min(kb0 / 32 + e, nsblk - 1)), sb, sbl, L::vsOff + i * 256);
    }
  }

  __device__ __forceinline__ void issue(int j, lds_char* sb) const {
    issue_k(j, sb);
    issue_v(j, sb);
  }
};

// This lane's Q fragment (B operand of S^T = K Q^T): query qi, d-block 2*ks + half; byte 2*ks
// of the returned scale word is that block's E8M0 scale.
template <int D>
__device__ __forceinline__ uint32_t load_q_fragment(const FwdArgs& a, int bh, int qi, bool qvalid, int half, v8i& qf0,
                                                    v8i& qf1) {
  const int N = a.N;
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
  return w >> (8 * half);
}

}  // namespace fwd
}  // namespace fp4attn

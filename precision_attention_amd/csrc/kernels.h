// kernels.h -- internal launch interface between the C ABI and the HIP kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4attn {

// Optional profiling events bound to one kernel's own dispatch: start takes the kernel's start
// timestamp and stop its end timestamp (hipExtLaunchKernel), so no marker packet is added to
// the stream. Both null: a plain launch.
struct KernelEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t smem, hipStream_t stream,
                                const KernelEvents& ev, Args... args) {
  if (ev.start || ev.stop) hipExtLaunchKernelGGL(kernel, grid, block, smem, stream, ev.start, ev.stop, 0u, args...);
  else kernel<<<grid, block, smem, stream>>>(args...);
  return hipGetLastError();
}

constexpr int kMXFP4 = 1;
constexpr int kMXFP8 = 2;
constexpr int kAlongD = 0;
constexpr int kAlongSeq = 1;

// Keys per running-max update of the forward kernels (both routes): 128 for D = 128, 64 for
// D = 64.
constexpr int key_block_for(int D) { return D == 128 ? 128 : 64; }
constexpr int kKeyBlock = 64;  // the BF16 variant's key block
// Queries per workgroup of the forward kernels (4 waves x 32 queries).
constexpr int kQueryTile = 128;

hipError_t launch_quantize(const uint16_t* x, uint8_t* codes, uint8_t* scales, int fmt, int axis, int64_t BH, int N,
                           int D, hipStream_t stream);
// Several quantizations of [rows, N, D] bf16 tensors (same N and D) in one launch.
constexpr int kMaxQuantJobs = 4;
struct QuantTask {
  const uint16_t* x;
  uint8_t* codes;
  uint8_t* scales;
  int64_t rows;  // B * heads
  int fmt, axis;
  // along D only, optional (all set or all null): per row i of x, ndot[i] = -sum_d x_id y_id in
  // fp32 (y bf16, same shape as x) and nl[i] = -fp32(lse[i] log2 e)
  const uint16_t* y = nullptr;
  const float* lse = nullptr;
  float* ndot = nullptr;
  float* nl = nullptr;
};
hipError_t launch_quantize_batch(const QuantTask* tasks, int count, int N, int D, hipStream_t stream);

struct FwdArgs {
  const uint8_t* q;   // MXFP4 along D: codes [B*H][N][D/2], scales [B*H][N][D/32]
  const uint8_t* qs;
  const uint8_t* k;   // MXFP4 along D: codes [B*Hkv][N][D/2], scales [B*Hkv][N][D/32]
  const uint8_t* ks;
  const uint8_t* v;   // along the sequence: codes [B*Hkv][D][N*bits/8], scales [B*Hkv][D][N/32]
  const uint8_t* vs;
  uint16_t* o;        // bf16 [B*H][N][D]
  float* lse;         // [B*H][N]
  int B, H, Hkv, N;
};

// fp8 == false (noncausal only): Direct-P, MXFP4 P and V. fp8 == true: FP8 P and V, with the
// causal mask when causal == 1.
// anchored (Direct-P only): the integer-log2 anchor with the sampled-anchor range guard.
hipError_t launch_attn_fwd(const FwdArgs& a, int D, int causal, bool fp8, hipStream_t stream,
                           const KernelEvents& ev = KernelEvents(), bool anchored = false);
// the pipelined Direct-P kernel (causal == 0)
hipError_t launch_attn_fwd_directp(const FwdArgs& a, int D, hipStream_t stream, const KernelEvents& ev = KernelEvents(),
                                   bool anchored = false);

// QKV projection with the MX quantization in its epilogue. F = (H + 2 Hkv) D weight rows.
struct ProjArgs {
  const uint16_t* x;  // bf16 [B][N][Dm]
  const uint16_t* w;  // bf16 [F][Dm]: Wq rows, then Wk, then Wv
  uint8_t* q;         // MXFP4 along D: codes [B*H][N][D/2], scales [B*H][N][D/32]
  uint8_t* qs;
  uint8_t* k;         // MXFP4 along D: [B*Hkv][N][D/2]
  uint8_t* ks;
  uint8_t* v;         // along the sequence: codes [B*Hkv][D][N*bits/8], scales [B*Hkv][D][N/32]
  uint8_t* vs;
  uint8_t* q8;        // optional (all three or none): MXFP8 along the sequence [B*H][D][N]
  uint8_t* q8s;
  uint8_t* k8;        // MXFP8 along the sequence [B*Hkv][D][N]
  uint8_t* k8s;
  uint8_t* v8;        // MXFP8 along D [B*Hkv][N][D], scales [B*Hkv][N][D/32]
  uint8_t* v8s;
  int B, N, Dm, H, Hkv, F;
  int v_fp8;          // V in MXFP8 (else MXFP4)
};
// tile: 0 picks by the launch's size, 128 the 256 x 128 tile, 256 the 256 x 256 tile
hipError_t launch_proj_qkv(const ProjArgs& a, int D, int tile, hipStream_t stream, const KernelEvents& ev = KernelEvents());

// NVFP4-style Q and K: block quantizer (n elements, D a multiple of 16) and the Direct-P forward on
// the integer-log2 anchor with S from their bf16 expansions.
hipError_t launch_quantize_nvfp4(const uint16_t* x, uint8_t* codes, uint8_t* scales, uint16_t* xhat, int64_t n,
                                 int g, hipStream_t stream);
struct NvFwdArgs {
  const uint16_t* q;  // bf16 [B*H][N][D]: the NVFP4 expansion of Q
  const uint16_t* k;  // bf16 [B*Hkv][N][D]
  const uint8_t* v;   // MXFP4 along the sequence: codes [B*Hkv][D][N/2], scales [B*Hkv][D][N/32]
  const uint8_t* vs;
  uint16_t* o;        // bf16 [B*H][N][D]
  float* lse;         // [B*H][N]
  int B, H, Hkv, N;
};
hipError_t launch_attn_fwd_nvfp4(const NvFwdArgs& a, int D, hipStream_t stream, const KernelEvents& ev = KernelEvents());

struct FwdBf16Args {
  const uint16_t* q;  // [B*H][N][D]
  const uint16_t* k;  // [B*Hkv][N][D]
  const uint16_t* vt; // V transposed, [B*Hkv][D][N]
  uint16_t* o;
  float* lse;
  int B, H, Hkv, N;
};
hipError_t launch_attn_fwd_bf16(const FwdBf16Args& a, int D, int causal, hipStream_t stream);

struct BwdLaunch {
  const uint8_t* q;    // MXFP4 along D [B*H][N][D/2], scales [B*H][N][D/32]
  const uint8_t* qs;
  const uint8_t* k;    // MXFP4 along D [B*Hkv][N][D/2]
  const uint8_t* ks;
  const uint8_t* q8;   // MXFP8 along the sequence [B*H][D][N], scales [B*H][D][N/32]
  const uint8_t* q8s;
  const uint8_t* k8;   // MXFP8 along the sequence [B*Hkv][D][N]
  const uint8_t* k8s;
  const uint8_t* v8;   // MXFP8 along D [B*Hkv][N][D], scales [B*Hkv][N][D/32]
  const uint8_t* v8s;
  const uint16_t* o;   // bf16 [B*H][N][D]
  const uint16_t* dout;
  const float* lse;    // [B*H][N]
  uint16_t* dq;        // bf16 [B*H][N][D]
  uint16_t* dk;        // bf16 [B*Hkv][N][D]
  uint16_t* dv;
  void* workspace;     // bwd_workspace_bytes(B, H, N, D) bytes, 256-byte aligned regions inside
  int B, H, Hkv, N;
};
size_t bwd_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D);
hipError_t launch_attn_bwd(const BwdLaunch& l, int D, int causal, hipStream_t stream);

}  // namespace fp4attn

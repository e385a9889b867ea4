// clock_probe.hip -- the shader clock under load, for the throughput figures' fraction of peak at
// the clock the GPU actually runs (the published peaks assume 2.4 GHz; a GPU under sustained
// matrix work may run lower, and one GPU differs from another).
//
// Load: every CU runs two workgroups of four waves (two waves per SIMD), each wave a loop of one
// FP4 32x32x64 MFMA and sixteen VALU instructions (fused multiply-adds and exponentials on
// independent chains), about the proportion of the Direct-P forward's block loop (18 MFMAs
// against some 300 VALU instructions per key block). Wave 0 of each workgroup reads the shader
// cycle counter (s_memtime) and the constant-rate real-time counter (s_memrealtime) around the
// loop; cycles / ticks x the real-time rate is the clock.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "fp4attn.h"

namespace fp4attn {
namespace {

constexpr int kProbeThreads = 256;

__global__ void __launch_bounds__(kProbeThreads, 2) clock_probe_kernel(uint64_t* counts, int iters) {
  // 60 KB of LDS per workgroup: at most two workgroups per CU
  __shared__ float pad[15 * 1024];
  v16f acc[2];
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 16; i++) acc[j][i] = 0.0f;
  v8i a, b;
#pragma unroll
  for (int i = 0; i < 8; i++) {
    a[i] = 0x22222222 + (int)(threadIdx.x & 7);
    b[i] = 0x11111111 + i;
  }
  float f[8];
#pragma unroll
  for (int i = 0; i < 8; i++) f[i] = (float)(threadIdx.x & 63) * -1e-3f - 0.01f * (float)i;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime(), r0 = __builtin_amdgcn_s_memrealtime();
  for (int it = 0; it < iters; ++it) {
    acc[it & 1] = mfma_scaled<kFmtFP4, kFmtFP4, 0, 0>(a, b, acc[it & 1], 127, 127);
#pragma unroll
    for (int i = 0; i < 8; i++) f[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(f[i], 0.5f, -0.25f));
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; j++)
#pragma unroll
    for (int i = 0; i < 16; i++) s += acc[j][i];
#pragma unroll
  for (int i = 0; i < 8; i++) s += f[i];
  pad[threadIdx.x] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    // the results depend on the loop (they are written only when non-finite, which they are not)
    const float keep = pad[(threadIdx.x + 1) & (kProbeThreads - 1)];
    counts[2 * blockIdx.x] = (t1 - t0) + (__builtin_isfinite(keep) ? 0 : 1);
    counts[2 * blockIdx.x + 1] = r1 - r0;
  }
}

}  // namespace
}  // namespace fp4attn

extern "C" int fp4attn_clock_probe(uint64_t* counts, int nblocks, int iters, int* realtime_khz, void* stream) {
  if (counts == nullptr || realtime_khz == nullptr) return FP4ATTN_ERR_NULL;
  if (nblocks < 1 || nblocks > 4096 || iters < 1 || iters > (1 << 24)) return FP4ATTN_ERR_SHAPE;
  int dev = 0, khz = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FP4ATTN_ERR_LAUNCH;
  if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess) return FP4ATTN_ERR_LAUNCH;
  *realtime_khz = khz;
  fp4attn::clock_probe_kernel<<<dim3((unsigned)nblocks), dim3(fp4attn::kProbeThreads), 0, (hipStream_t)stream>>>(
      counts, iters);
  return hipGetLastError() == hipSuccess ? FP4ATTN_OK : FP4ATTN_ERR_LAUNCH;
}

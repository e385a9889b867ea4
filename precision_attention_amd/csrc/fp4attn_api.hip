// fp4attn_api.hip -- the C ABI declared in include/fp4attn.h: argument validation on the
// host (nothing is enqueued when it fails) and kernel launches on the caller's stream.
#include "fp4attn.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

using namespace fp4attn;

// Scratch of fp4attn_bwd_noalloc: the backward's workspace held in a static device array, for
// callers that cannot allocate device memory. Each device the library runs on holds its own copy
// until the process ends. In host code `scratch` is only a stand-in for the symbol: its device
// address is looked up once per device and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[FP4ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
void* scratch_ptr[kMaxDevices];
std::once_flag scratch_once[kMaxDevices];
hipError_t scratch_err[kMaxDevices];

// Device address of this device's scratch array (the device must be current), or null on error.
void* scratch_address(int dev) {
  std::call_once(scratch_once[dev], [dev] {
    void* p = nullptr;
    scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    scratch_ptr[dev] = scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  return scratch_ptr[dev];
}

}  // namespace

static_assert(kMaxQuantJobs == FP4ATTN_MAX_QUANT_JOBS, "batch size limit of the ABI and the kernels");

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

int check_sizes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D) {
  if (B < 0 || H < 1 || Hkv < 1 || N < 0 || D < 1) return FP4ATTN_ERR_SHAPE;
  if (H % Hkv != 0 || N % 32 != 0) return FP4ATTN_ERR_SHAPE;
  if (D != 64 && D != 128) return FP4ATTN_ERR_UNSUPPORTED;
  if (B * H * N * D >= kMaxElems || B * H > 65535) return FP4ATTN_ERR_SHAPE;
  return FP4ATTN_OK;
}

int check_mx(const fp4attn_mx* t, int fmt, int axis) {
  if (!t || !t->codes || !t->scales) return FP4ATTN_ERR_NULL;
  if (t->fmt != fmt || t->axis != axis) return FP4ATTN_ERR_FORMAT;
  if (!aligned16(t->codes) || !aligned16(t->scales)) return FP4ATTN_ERR_ALIGN;
  return FP4ATTN_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? FP4ATTN_OK : FP4ATTN_ERR_LAUNCH; }

}  // namespace

extern "C" {

size_t fp4attn_mx_codes_bytes(int fmt, int64_t B, int64_t heads, int64_t N, int64_t D) {
  if (B < 0 || heads < 0 || N < 0 || D < 0) return 0;
  const int64_t n = B * heads * N * D;
  if (fmt == FP4ATTN_MXFP4) return (size_t)(n / 2);
  if (fmt == FP4ATTN_MXFP8) return (size_t)n;
  return 0;
}

size_t fp4attn_mx_scales_bytes(int64_t B, int64_t heads, int64_t N, int64_t D) {
  if (B < 0 || heads < 0 || N < 0 || D < 0) return 0;
  return (size_t)(B * heads * N * D / 32);
}

int fp4attn_quantize_mx(const void* x_bf16, const fp4attn_mx* out, int64_t B, int64_t heads, int64_t N, int64_t D,
                        void* stream) {
  if (!x_bf16 || !out || !out->codes || !out->scales) return FP4ATTN_ERR_NULL;
  int rc = check_sizes(B, heads, heads, N, D);
  if (rc) return rc;
  if ((out->fmt != FP4ATTN_MXFP4 && out->fmt != FP4ATTN_MXFP8) ||
      (out->axis != FP4ATTN_ALONG_D && out->axis != FP4ATTN_ALONG_SEQ))
    return FP4ATTN_ERR_FORMAT;
  if (!aligned16(x_bf16) || !aligned16(out->codes) || !aligned16(out->scales)) return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  return launch_status(launch_quantize((const uint16_t*)x_bf16, (uint8_t*)out->codes, out->scales, out->fmt,
                                       out->axis, B * heads, (int)N, (int)D, (hipStream_t)stream));
}

int fp4attn_quantize_mx_batch(const fp4attn_quant_job* jobs, int count, int64_t B, int64_t N, int64_t D,
                              void* stream) {
  if (!jobs) return FP4ATTN_ERR_NULL;
  if (count < 1 || count > FP4ATTN_MAX_QUANT_JOBS) return FP4ATTN_ERR_SHAPE;
  QuantTask t[FP4ATTN_MAX_QUANT_JOBS];
  for (int i = 0; i < count; i++) {
    const fp4attn_quant_job& j = jobs[i];
    if (!j.x_bf16 || !j.out.codes || !j.out.scales) return FP4ATTN_ERR_NULL;
    const int rc = check_sizes(B, j.heads, j.heads, N, D);
    if (rc) return rc;
    if ((j.out.fmt != FP4ATTN_MXFP4 && j.out.fmt != FP4ATTN_MXFP8) ||
        (j.out.axis != FP4ATTN_ALONG_D && j.out.axis != FP4ATTN_ALONG_SEQ))
      return FP4ATTN_ERR_FORMAT;
    if (!aligned16(j.x_bf16) || !aligned16(j.out.codes) || !aligned16(j.out.scales)) return FP4ATTN_ERR_ALIGN;
    t[i] = QuantTask{(const uint16_t*)j.x_bf16, (uint8_t*)j.out.codes, j.out.scales, B * j.heads, j.out.fmt,
                     j.out.axis};
  }
  if (B == 0 || N == 0) return FP4ATTN_OK;
  return launch_status(launch_quantize_batch(t, count, (int)N, (int)D, (hipStream_t)stream));
}

int fp4attn_quantize_nvfp4(const void* x_bf16, void* codes, void* scales, void* xhat_bf16, int tensor_exp,
                           int64_t B, int64_t heads, int64_t N, int64_t D, void* stream) {
  if (!x_bf16 || !codes || !scales || !xhat_bf16) return FP4ATTN_ERR_NULL;
  const int rc = check_sizes(B, heads, heads, N, D);
  if (rc) return rc;
  if (tensor_exp < -100 || tensor_exp > 100) return FP4ATTN_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(codes) || !aligned16(scales) || !aligned16(xhat_bf16)) return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  return launch_status(launch_quantize_nvfp4((const uint16_t*)x_bf16, (uint8_t*)codes, (uint8_t*)scales,
                                             (uint16_t*)xhat_bf16, B * heads * N * D, tensor_exp,
                                             (hipStream_t)stream));
}

int fp4attn_fwd_nvfp4(const void* q_hat_bf16, const void* k_hat_bf16, const fp4attn_mx* v, void* o_bf16, float* lse,
                      int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, void* stream, void* start_event,
                      void* stop_event) {
  if (!q_hat_bf16 || !k_hat_bf16 || !o_bf16 || !lse) return FP4ATTN_ERR_NULL;
  int rc = check_sizes(B, H, Hkv, N, D);
  if (rc) return rc;
  if ((rc = check_mx(v, FP4ATTN_MXFP4, FP4ATTN_ALONG_SEQ))) return rc;
  if (!aligned16(q_hat_bf16) || !aligned16(k_hat_bf16) || !aligned16(o_bf16) || !aligned16(lse))
    return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  NvFwdArgs a{};
  a.q = (const uint16_t*)q_hat_bf16;
  a.k = (const uint16_t*)k_hat_bf16;
  a.v = (const uint8_t*)v->codes;
  a.vs = v->scales;
  a.o = (uint16_t*)o_bf16;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  return launch_status(launch_attn_fwd_nvfp4(a, (int)D, (hipStream_t)stream,
                                             KernelEvents{(hipEvent_t)start_event, (hipEvent_t)stop_event}));
}

int fp4attn_project_qkv_ex(const void* x_bf16, const void* w_bf16, const fp4attn_mx* q, const fp4attn_mx* k,
                           const fp4attn_mx* v, const fp4attn_mx* q8, const fp4attn_mx* k8, const fp4attn_mx* v8,
                           int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t Hkv, int64_t D, int tile,
                           void* stream) {
  if (!x_bf16 || !w_bf16 || !q || !k || !v) return FP4ATTN_ERR_NULL;
  if (tile != 0 && tile != 128 && tile != 256) return FP4ATTN_ERR_UNSUPPORTED;
  int rc = check_sizes(B, H, Hkv, N, D);
  if (rc) return rc;
  if (N < 32 || Dm < 64 || Dm % 64 != 0 || Dm > 65536 || B * N * Dm >= kMaxElems ||
      (H + 2 * Hkv) * D * Dm >= kMaxElems || B * N > (int64_t)1 << 24)
    return FP4ATTN_ERR_SHAPE;
  if (!aligned16(x_bf16) || !aligned16(w_bf16)) return FP4ATTN_ERR_ALIGN;
  if ((rc = check_mx(q, FP4ATTN_MXFP4, FP4ATTN_ALONG_D)) || (rc = check_mx(k, FP4ATTN_MXFP4, FP4ATTN_ALONG_D))) return rc;
  if ((rc = check_mx(v, v->fmt == FP4ATTN_MXFP8 ? FP4ATTN_MXFP8 : FP4ATTN_MXFP4, FP4ATTN_ALONG_SEQ))) return rc;
  const int nviews = (q8 != nullptr) + (k8 != nullptr) + (v8 != nullptr);
  if (nviews != 0 && nviews != 3) return FP4ATTN_ERR_FORMAT;
  if (nviews == 3 && ((rc = check_mx(q8, FP4ATTN_MXFP8, FP4ATTN_ALONG_SEQ)) ||
                      (rc = check_mx(k8, FP4ATTN_MXFP8, FP4ATTN_ALONG_SEQ)) ||
                      (rc = check_mx(v8, FP4ATTN_MXFP8, FP4ATTN_ALONG_D))))
    return rc;
  if (B == 0) return FP4ATTN_OK;
  ProjArgs a{};
  a.x = (const uint16_t*)x_bf16;
  a.w = (const uint16_t*)w_bf16;
  a.q = (uint8_t*)q->codes;
  a.qs = q->scales;
  a.k = (uint8_t*)k->codes;
  a.ks = k->scales;
  a.v = (uint8_t*)v->codes;
  a.vs = v->scales;
  if (nviews == 3) {
    a.q8 = (uint8_t*)q8->codes;
    a.q8s = q8->scales;
    a.k8 = (uint8_t*)k8->codes;
    a.k8s = k8->scales;
    a.v8 = (uint8_t*)v8->codes;
    a.v8s = v8->scales;
  }
  a.B = (int)B;
  a.N = (int)N;
  a.Dm = (int)Dm;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.F = (int)((H + 2 * Hkv) * D);
  a.v_fp8 = v->fmt == FP4ATTN_MXFP8;
  return launch_status(launch_proj_qkv(a, (int)D, tile, (hipStream_t)stream));
}

int fp4attn_project_qkv(const void* x_bf16, const void* w_bf16, const fp4attn_mx* q, const fp4attn_mx* k,
                        const fp4attn_mx* v, const fp4attn_mx* q8, const fp4attn_mx* k8, const fp4attn_mx* v8,
                        int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t Hkv, int64_t D, void* stream) {
  return fp4attn_project_qkv_ex(x_bf16, w_bf16, q, k, v, q8, k8, v8, B, N, Dm, H, Hkv, D, 0, stream);
}

}  // extern "C"

namespace {

int fwd_impl(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* v, void* o_bf16, float* lse, int64_t B,
             int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, unsigned flags, void* stream,
             const KernelEvents& ev) {
  if (!o_bf16 || !lse) return FP4ATTN_ERR_NULL;
  int rc;
  if ((rc = check_mx(q, FP4ATTN_MXFP4, FP4ATTN_ALONG_D))) return rc;
  if ((rc = check_mx(k, FP4ATTN_MXFP4, FP4ATTN_ALONG_D))) return rc;
  // causal: MXFP8 V; noncausal: MXFP4 V (Direct-P) or MXFP8 V (the FP8 P/V route)
  if (!v) return FP4ATTN_ERR_NULL;
  const int vfmt = causal ? FP4ATTN_MXFP8 : (v->fmt == FP4ATTN_MXFP8 ? FP4ATTN_MXFP8 : FP4ATTN_MXFP4);
  if ((rc = check_mx(v, vfmt, FP4ATTN_ALONG_SEQ))) return rc;
  if ((rc = check_sizes(B, H, Hkv, N, D))) return rc;
  if (causal != 0 && causal != 1) return FP4ATTN_ERR_UNSUPPORTED;
  if (flags & ~(unsigned)FP4ATTN_FWD_ANCHORED) return FP4ATTN_ERR_UNSUPPORTED;
  const bool anchored = (flags & FP4ATTN_FWD_ANCHORED) != 0;
  if (anchored && (causal || vfmt != FP4ATTN_MXFP4)) return FP4ATTN_ERR_UNSUPPORTED;
  if (!aligned16(o_bf16) || !aligned16(lse)) return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  FwdArgs a;
  a.q = (const uint8_t*)q->codes;
  a.qs = q->scales;
  a.k = (const uint8_t*)k->codes;
  a.ks = k->scales;
  a.v = (const uint8_t*)v->codes;
  a.vs = v->scales;
  a.o = (uint16_t*)o_bf16;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  return launch_status(launch_attn_fwd(a, (int)D, causal, vfmt == FP4ATTN_MXFP8, (hipStream_t)stream, ev, anchored));
}

}  // namespace

extern "C" {

int fp4attn_fwd(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* v, void* o_bf16, float* lse, int64_t B,
                int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, void* stream) {
  return fwd_impl(q, k, v, o_bf16, lse, B, H, Hkv, N, D, causal, 0u, stream, KernelEvents());
}

int fp4attn_fwd_ex(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* v, void* o_bf16, float* lse,
                   int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, unsigned flags, void* stream,
                   void* start_event, void* stop_event) {
  if ((start_event == nullptr) != (stop_event == nullptr)) return FP4ATTN_ERR_NULL;
  KernelEvents ev;
  ev.start = (hipEvent_t)start_event;
  ev.stop = (hipEvent_t)stop_event;
  return fwd_impl(q, k, v, o_bf16, lse, B, H, Hkv, N, D, causal, flags, stream, ev);
}

int fp4attn_fwd_bf16(const void* q_bf16, const void* k_bf16, const void* vt_bf16, void* o_bf16, float* lse, int64_t B,
                     int64_t H, int64_t Hkv, int64_t N, int64_t D, int causal, void* stream) {
  if (!q_bf16 || !k_bf16 || !vt_bf16 || !o_bf16 || !lse) return FP4ATTN_ERR_NULL;
  int rc = check_sizes(B, H, Hkv, N, D);
  if (rc) return rc;
  if (causal != 0 && causal != 1) return FP4ATTN_ERR_UNSUPPORTED;
  if (!aligned16(q_bf16) || !aligned16(k_bf16) || !aligned16(vt_bf16) || !aligned16(o_bf16) || !aligned16(lse))
    return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  FwdBf16Args a;
  a.q = (const uint16_t*)q_bf16;
  a.k = (const uint16_t*)k_bf16;
  a.vt = (const uint16_t*)vt_bf16;
  a.o = (uint16_t*)o_bf16;
  a.lse = lse;
  a.B = (int)B;
  a.H = (int)H;
  a.Hkv = (int)Hkv;
  a.N = (int)N;
  return launch_status(launch_attn_fwd_bf16(a, (int)D, causal, (hipStream_t)stream));
}

size_t fp4attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D) {
  if (check_sizes(B, H, Hkv, N, D) != FP4ATTN_OK) return 0;
  return bwd_workspace_bytes(B, H, N, D);
}

}  // extern "C"

namespace {

int bwd_impl(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* q8, const fp4attn_mx* k8,
             const fp4attn_mx* v8, const void* o_bf16, const void* do_bf16, const float* lse, void* dq_bf16,
             void* dk_bf16, void* dv_bf16, void* workspace, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t D,
             int causal, void* stream) {
  if (!o_bf16 || !do_bf16 || !lse || !dq_bf16 || !dk_bf16 || !dv_bf16 || !workspace) return FP4ATTN_ERR_NULL;
  int rc;
  if ((rc = check_mx(q, FP4ATTN_MXFP4, FP4ATTN_ALONG_D))) return rc;
  if ((rc = check_mx(k, FP4ATTN_MXFP4, FP4ATTN_ALONG_D))) return rc;
  if ((rc = check_mx(q8, FP4ATTN_MXFP8, FP4ATTN_ALONG_SEQ))) return rc;
  if ((rc = check_mx(k8, FP4ATTN_MXFP8, FP4ATTN_ALONG_SEQ))) return rc;
  if ((rc = check_mx(v8, FP4ATTN_MXFP8, FP4ATTN_ALONG_D))) return rc;
  if ((rc = check_sizes(B, H, Hkv, N, D))) return rc;
  if (causal != 0 && causal != 1) return FP4ATTN_ERR_UNSUPPORTED;
  if (!aligned16(o_bf16) || !aligned16(do_bf16) || !aligned16(lse) || !aligned16(dq_bf16) || !aligned16(dk_bf16) ||
      !aligned16(dv_bf16) || !aligned16(workspace))
    return FP4ATTN_ERR_ALIGN;
  if (B == 0 || N == 0) return FP4ATTN_OK;
  BwdLaunch l;
  l.q = (const uint8_t*)q->codes;
  l.qs = q->scales;
  l.k = (const uint8_t*)k->codes;
  l.ks = k->scales;
  l.q8 = (const uint8_t*)q8->codes;
  l.q8s = q8->scales;
  l.k8 = (const uint8_t*)k8->codes;
  l.k8s = k8->scales;
  l.v8 = (const uint8_t*)v8->codes;
  l.v8s = v8->scales;
  l.o = (const uint16_t*)o_bf16;
  l.dout = (const uint16_t*)do_bf16;
  l.lse = lse;
  l.dq = (uint16_t*)dq_bf16;
  l.dk = (uint16_t*)dk_bf16;
  l.dv = (uint16_t*)dv_bf16;
  l.workspace = workspace;
  l.B = (int)B;
  l.H = (int)H;
  l.Hkv = (int)Hkv;
  l.N = (int)N;
  return launch_status(launch_attn_bwd(l, (int)D, causal, (hipStream_t)stream));
}

}  // namespace

extern "C" {

int fp4attn_bwd(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* q8, const fp4attn_mx* k8,
                const fp4attn_mx* v8, const void* o_bf16, const void* do_bf16, const float* lse, void* dq_bf16,
                void* dk_bf16, void* dv_bf16, void* workspace, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                int64_t D, int causal, void* stream) {
  return bwd_impl(q, k, q8, k8, v8, o_bf16, do_bf16, lse, dq_bf16, dk_bf16, dv_bf16, workspace, B, H, Hkv, N, D,
                  causal, stream);
}

int fp4attn_bwd_noalloc(const fp4attn_mx* q, const fp4attn_mx* k, const fp4attn_mx* q8, const fp4attn_mx* k8,
                        const fp4attn_mx* v8, const void* o_bf16, const void* do_bf16, const float* lse,
                        void* dq_bf16, void* dk_bf16, void* dv_bf16, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                        int64_t D, int causal, void* stream) {
  const int rc = check_sizes(B, H, Hkv, N, D);
  if (rc) return rc;
  if (bwd_workspace_bytes(B, H, N, D) > (size_t)FP4ATTN_NOALLOC_SCRATCH_BYTES) return FP4ATTN_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4ATTN_ERR_LAUNCH;
  void* ws = scratch_address(dev);
  if (!ws) return FP4ATTN_ERR_LAUNCH;
  return bwd_impl(q, k, q8, k8, v8, o_bf16, do_bf16, lse, dq_bf16, dk_bf16, dv_bf16, ws, B, H, Hkv, N, D, causal,
                  stream);
}

int fp4attn_key_block(int64_t D, int causal) {
  (void)causal;  // both routes use the same key block
  if (D != 64 && D != 128) return 0;
  return key_block_for((int)D);
}

const char* fp4attn_status_str(int status) {
  switch (status) {
    case FP4ATTN_OK: return "ok";
    case FP4ATTN_ERR_NULL: return "a required pointer is NULL";
    case FP4ATTN_ERR_SHAPE: return "invalid sizes (negative, H % Hkv != 0, N % 32 != 0, or too large)";
    case FP4ATTN_ERR_UNSUPPORTED: return "unsupported head size or mode";
    case FP4ATTN_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case FP4ATTN_ERR_FORMAT: return "an operand has the wrong MX format or blocking axis";
    case FP4ATTN_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case FP4ATTN_ERR_SCRATCH:
      return "the sizes need more scratch than the static buffer of fp4attn_bwd_noalloc holds "
             "(FP4ATTN_NOALLOC_SCRATCH_BYTES); use fp4attn_bwd with a workspace";
    default: return "unknown status";
  }
}

}  // extern "C"

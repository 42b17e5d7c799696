// C ABI entry points: argument validation and dispatch to the gfx950 kernels.
// Every check happens before any HIP call, so invalid arguments never launch
// anything.  See include/fa.h for the contract.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "../../include/fa.h"
#include "fa_kernels.h"

namespace {

constexpr long kMaxElems = 1L << 40;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool finite_pos(float x) { return isfinite(x) && x > 0.f; }

// Shared size checks.  Returns FA_OK and sets *empty when there is no work.
fa_status check_sizes(int B, int H, int N, int d, bool* empty) {
  if (B < 0 || H < 0 || N < 0) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return d > 0 ? FA_ERR_UNSUPPORTED : FA_ERR_INVALID_ARG;
  const long bhn = (long)B * (long)H * (long)N;
  *empty = bhn == 0;
  if (bhn > kMaxElems / d) return FA_ERR_INVALID_ARG;
  // one workgroup per 32 rows at most: keep the grid inside 32 bits
  const long blocks = (long)B * (long)H * (((long)N + 31) / 32);
  if (blocks > 0x7fffffffL) return FA_ERR_INVALID_ARG;
  return FA_OK;
}

// An additive bias: null (none), or 16-byte aligned float32 with strides in
// elements that are non-negative multiples of 4, and one (b, h) slice --
// (N - 1) * sq + N elements -- addressable with 32-bit byte offsets (with room
// for the reads of a ragged last tile, which the kernels mask).
fa_status check_bias(const float* p, long long sb, long long sh, long long sq, int H, int N,
                     fa::Bias* b) {
  *b = fa::Bias{};
  if (!p) return FA_OK;
  if (!aligned(p, 16)) return FA_ERR_INVALID_ARG;
  if (sb < 0 || sh < 0 || sq < 0 || (sb & 3) || (sh & 3) || (sq & 3)) return FA_ERR_INVALID_ARG;
  const long long nn = N > 0 ? N : 1;
  if (sq > (1LL << 32) / nn) return FA_ERR_INVALID_ARG;
  const long long extent = (nn - 1) * sq + nn;
  if (extent * 4 + 4096 > (1LL << 32)) return FA_ERR_INVALID_ARG;
  b->p = p;
  b->sb = sb;
  b->sh = sh;
  b->sq = sq;
  b->H = H > 0 ? H : 1;
  b->head_bytes = (uint32_t)(extent * 4);
  return FA_OK;
}

size_t ws_bytes(long BH, int N) {
  const size_t delta = (size_t)BH * (size_t)N * sizeof(float);
  return (delta + 255) & ~(size_t)255;
}

// FA_FWD_SCHEDULE (read on every call): unset, empty or "interleaved", the
// default; "pingpong" or "rows64".  Anything else: -1.
int fwd_schedule() {
  const char* s = getenv("FA_FWD_SCHEDULE");
  if (!s || !*s || !strcmp(s, "interleaved")) return fa::kSchedInterleaved;
  if (!strcmp(s, "pingpong")) return fa::kSchedPingPong;
  if (!strcmp(s, "rows64")) return fa::kSchedRows64;
  return -1;
}

fa_status run_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int N, int d, float scale, int causal, int dtype, float q_descale,
                  float k_descale, float v_descale, const fa::Bias& bias, void* stream) {
  if (dtype != FA_FP32 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  bool empty = false;
  fa_status st = check_sizes(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if (!finite_pos(scale)) return FA_ERR_INVALID_ARG;
  if (dtype == FA_FP8_E4M3 &&
      (!finite_pos(q_descale) || !finite_pos(k_descale) || !finite_pos(v_descale)))
    return FA_ERR_INVALID_ARG;
  const int schedule = fwd_schedule();
  if (schedule < 0) return FA_ERR_INVALID_ARG;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (long)B * H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.v_descale = v_descale;
  a.bias = bias;
  a.schedule = schedule;
  a.stream = (hipStream_t)stream;
  hipError_t e;
  switch (dtype) {
    case FA_FP32: e = fa::launch_fwd_f32(a); break;
    case FA_BF16: e = fa::launch_fwd_bf16(a); break;
    default: e = fa::launch_fwd_fp8(a); break;
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                 int N, int d, float scale, int causal, int dtype, float q_descale,
                 float k_descale, float v_descale, void* stream) {
  return run_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, q_descale, k_descale,
                 v_descale, fa::Bias{}, stream);
}

fa_status fa_fwd_bias(const void* q, const void* k, const void* v, const float* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      void* o, float* lse, int B, int H, int N, int d, float scale, int causal,
                      int dtype, void* stream) {
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  fa::Bias b;
  const fa_status st = check_bias(bias, bias_stride_b, bias_stride_h, bias_stride_q, H, N, &b);
  if (st != FA_OK) return st;
  return run_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, 1.f, 1.f, 1.f, b, stream);
}

fa_status fa_fwd_mxfp8(const void* q, const void* k, const void* v, const void* q_scale,
                       const void* k_scale, const void* v_scale, void* o, float* lse, int B,
                       int H, int N, int d, float scale, int causal, void* stream) {
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  bool empty = false;
  fa_status st = check_sizes(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if (!finite_pos(scale)) return FA_ERR_INVALID_ARG;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !q_scale || !k_scale || !v_scale) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(q_scale, 4) || !aligned(k_scale, 4) || !aligned(v_scale, 4))
    return FA_ERR_INVALID_ARG;

  fa::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (long)B * H;
  a.N = N;
  a.d = d;
  a.scale = scale;
  a.causal = causal != 0;
  a.q_descale = a.k_descale = a.v_descale = 1.f;
  a.q_scale = (const uint8_t*)q_scale;
  a.k_scale = (const uint8_t*)k_scale;
  a.v_scale = (const uint8_t*)v_scale;
  a.stream = (hipStream_t)stream;
  return fa::launch_fwd_fp8(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_std_workspace_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_sizes(B, H, N, d, &empty) != FA_OK) return 0;
  const size_t ldp = ((size_t)N + 63) / 64 * 64;
  const size_t entries = (size_t)B * (size_t)H * (size_t)N * ldp;
  return (entries * 4 + 255) / 256 * 256 + (entries * 2 + 255) / 256 * 256;
}

fa_status fa_std_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     void* workspace, size_t workspace_bytes, int B, int H, int N, int d,
                     float scale, int causal, int dtype, void* stream) {
  if (dtype != FA_FP32 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  bool empty = false;
  const fa_status st = check_sizes(B, H, N, d, &empty);
  if (st != FA_OK) return st;
  if (dtype != FA_BF16) return FA_ERR_UNSUPPORTED;
  if (!finite_pos(scale)) return FA_ERR_INVALID_ARG;
  if (empty) return FA_OK;
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(workspace, 256))
    return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_std_workspace_size(B, H, N, d)) return FA_ERR_INVALID_ARG;
  // grids: 64 x 64 score tiles by B*H (the second and third grid dimensions
  // stay within 65535), one softmax workgroup per four rows
  if ((long)B * H > 65535 || (N + 63) / 64 > 65535) return FA_ERR_UNSUPPORTED;
  if (((long)B * H * N + 3) / 4 > 0x7fffffffL) return FA_ERR_INVALID_ARG;
  fa::StdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.BH = (long)B * H;
  a.N = N;
  a.d = d;
  a.ldp = (N + 63) / 64 * 64;
  a.scale = scale;
  a.causal = causal != 0;
  const size_t entries = (size_t)a.BH * (size_t)N * (size_t)a.ldp;
  a.s = static_cast<float*>(workspace);
  a.p = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + (entries * 4 + 255) / 256 * 256);
  a.stream = (hipStream_t)stream;
  return fa::launch_std_bf16(a) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  bool empty = false;
  if (check_sizes(B, H, N, d, &empty) != FA_OK) return 0;
  return ws_bytes((long)B * H, N);
}

}  // extern "C"

namespace {

enum { kStageDelta = 1, kStageDkDv = 2, kStageDq = 4 };

// Validation shared by the backward entry points (all but the workspace).
// Fills *a except a->delta; *empty is set when there is no work.
fa_status prepare_bwd(const void* q, const void* k, const void* v, const void* o,
                      const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                      int H, int N, int d, float scale, int causal, int dtype, void* stream,
                      const fa::Bias& bias, fa::BwdArgs* a, bool* empty) {
  if (dtype != FA_FP32 && dtype != FA_BF16 && dtype != FA_FP8_E4M3) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  fa_status st = check_sizes(B, H, N, d, empty);
  if (st != FA_OK) return st;
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  if (!finite_pos(scale)) return FA_ERR_INVALID_ARG;
  if (*empty) return FA_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
      !aligned(lse, 4))
    return FA_ERR_INVALID_ARG;
  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->dout = dout;
  a->lse = lse;
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->delta = nullptr;
  a->BH = (long)B * H;
  a->N = N;
  a->d = d;
  a->scale = scale;
  a->causal = causal != 0;
  a->bias = bias;
  a->stream = (hipStream_t)stream;
  return FA_OK;
}

fa_status launch_bwd(const fa::BwdArgs& a, int dtype, int stages) {
  hipError_t e = hipSuccess;
  if (dtype == FA_BF16) {
    // The bf16 dQ kernel forms delta itself and stores it for the dK/dV
    // kernel: dQ runs first and a full backward needs no delta launch.
    if ((stages & kStageDelta) && !(stages & kStageDq)) e = fa::launch_delta(a, true);
    if (e == hipSuccess && (stages & kStageDq)) e = fa::launch_dq_bf16(a);
    if (e == hipSuccess && (stages & kStageDkDv)) e = fa::launch_dkdv_bf16(a);
  } else {
    if (stages & kStageDelta) e = fa::launch_delta(a, false);
    if (e == hipSuccess && (stages & kStageDkDv)) e = fa::launch_dkdv_f32(a);
    if (e == hipSuccess && (stages & kStageDq)) e = fa::launch_dq_f32(a);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status run_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                  const float* lse, void* dq, void* dk, void* dv, void* workspace,
                  size_t workspace_bytes, int B, int H, int N, int d, float scale, int causal,
                  int dtype, void* stream, int stages, const fa::Bias& bias = fa::Bias{}) {
  fa::BwdArgs a;
  bool empty = false;
  const fa_status st = prepare_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal,
                                   dtype, stream, bias, &a, &empty);
  if (st != FA_OK || empty) return st;
  if (!workspace || !aligned(workspace, 4)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < ws_bytes((long)B * H, N)) return FA_ERR_INVALID_ARG;
  a.delta = (float*)workspace;
  return launch_bwd(a, dtype, stages);
}

}  // namespace

extern "C" {

#define FA_BWD_PARAMS                                                                           \
  const void *q, const void *k, const void *v, const void *o, const void *dout,                 \
      const float *lse, void *dq, void *dk, void *dv, void *workspace, size_t workspace_bytes, \
      int B, int H, int N, int d, float scale, int causal, int dtype, void *stream
#define FA_BWD_ARGS                                                                          \
  q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, H, N, d, scale, causal, \
      dtype, stream

fa_status fa_bwd(FA_BWD_PARAMS) {
  return run_bwd(FA_BWD_ARGS, kStageDelta | kStageDkDv | kStageDq);
}
fa_status fa_bwd_delta(FA_BWD_PARAMS) { return run_bwd(FA_BWD_ARGS, kStageDelta); }
fa_status fa_bwd_dkdv(FA_BWD_PARAMS) { return run_bwd(FA_BWD_ARGS, kStageDkDv); }
fa_status fa_bwd_dq(FA_BWD_PARAMS) { return run_bwd(FA_BWD_ARGS, kStageDq); }

fa_status fa_bwd_bias(const void* q, const void* k, const void* v, const float* bias,
                      long long bias_stride_b, long long bias_stride_h, long long bias_stride_q,
                      const void* o, const void* dout, const float* lse, void* dq, void* dk,
                      void* dv, void* workspace, size_t workspace_bytes, int B, int H, int N,
                      int d, float scale, int causal, int dtype, void* stream) {
  if (dtype == FA_FP8_E4M3) return FA_ERR_UNSUPPORTED;
  fa::Bias b;
  const fa_status st = check_bias(bias, bias_stride_b, bias_stride_h, bias_stride_q, H, N, &b);
  if (st != FA_OK) return st;
  return run_bwd(FA_BWD_ARGS, kStageDelta | kStageDkDv | kStageDq, b);
}

}  // extern "C"

// The allocation-free backward keeps delta (one float per row) in this
// device-global array instead of a caller's workspace.  Every GPU the library
// runs on holds its own copy, at its own address, until the process ends.  In
// host code the array's name is only a stand-in: its device address is looked
// up per device (once, with that device current) and only that address is
// handed to kernels.
static __device__ __align__(256) float scratch[FA_NOALLOC_MAX_ROWS];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_dev[kMaxDevices] = {};

// The device address of `scratch` on the current device, which must be the
// device of `stream` (the null stream: the current device).
fa_status scratch_address(void* stream, float** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (stream) {
    int sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if (sdev != dev) return FA_ERR_INVALID_ARG;
  }
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FA_ERR_HIP;
    g_scratch_dev[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_dev[dev];
  return FA_OK;
}

}  // namespace

extern "C" {

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                         int H, int N, int d, float scale, int causal, int dtype, void* stream) {
  fa::BwdArgs a;
  bool empty = false;
  fa_status st = prepare_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, H, N, d, scale, causal, dtype,
                             stream, fa::Bias{}, &a, &empty);
  if (st != FA_OK || empty) return st;
  if ((long)B * (long)H * (long)N > (long)FA_NOALLOC_MAX_ROWS) return FA_ERR_UNSUPPORTED;
  st = scratch_address(stream, &a.delta);
  if (st != FA_OK) return st;
  return launch_bwd(a, dtype, kStageDelta | kStageDkDv | kStageDq);
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK: return "ok";
    case FA_ERR_INVALID_ARG: return "invalid argument";
    case FA_ERR_UNSUPPORTED: return "unsupported configuration";
    case FA_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

}  // extern "C"

// Internal launcher interface between the C ABI (fa_api.hip) and the kernels.
// Arguments are validated by the caller; launchers only pick an instantiation
// and enqueue it on the given stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

// Additive bias on the scaled scores (float32), s_ij = scale q_i.k_j + b_ij;
// -inf masks a key.  Element (b, h, i, j) is p[b*sb + h*sh + i*sq + j]; strides
// are in elements (multiples of 4, or 0 to broadcast), p is 16-byte aligned.
// head_bytes = ((N - 1) sq + N) * 4, the extent of one (b, h) slice, < 2^32.
struct Bias {
  const float* p = nullptr;
  long long sb = 0, sh = 0, sq = 0;
  int H = 1;  // heads per batch entry: splits the combined index bh into (b, h)
  uint32_t head_bytes = 0;
  // Set by a launcher when every head of a batch entry reads the same bias
  // (sh = 0) and the grid allows it: workgroups running together on one XCD
  // then take kGroupHeads heads x `grouped` blocks (map_block_grouped);
  // 0: map_block's order.
  int grouped = 0;
};

// Forward schedules of the bf16 d = 128 kernels without a bias (the
// FA_FWD_SCHEDULE environment variable): the same results, different ways of
// overlapping the matrix products with the softmax arithmetic.
enum FwdSchedule : int {
  kSchedInterleaved = 0,  // fwd_bf16.hip: softmax woven into the next tile's products
  kSchedPingPong = 1,     // fwd_bf16_pp.hip: two wave groups alternate products and softmax
  kSchedRows64 = 2,       // fwd_bf16_w64.hip: 64 rows per wave, one wave per SIMD
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  long BH;  // batch * heads
  int N, d;
  float scale;
  bool causal;
  float q_descale, k_descale, v_descale;  // fp8 with per-tensor scales
  // fp8 with e8m0 block scales (all three set, or all null): Q and K
  // [BH][N][4] (bytes 0 .. d/32-1 used), V [BH][ceil(N/32)][d]
  const uint8_t* q_scale = nullptr;
  const uint8_t* k_scale = nullptr;
  const uint8_t* v_scale = nullptr;
  Bias bias;  // p == nullptr: none
  int schedule = kSchedInterleaved;  // bf16, d = 128, no bias
  hipStream_t stream;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;  // [BH * N] inside the workspace
  long BH;
  int N, d;
  float scale;
  bool causal;
  Bias bias;  // p == nullptr: none
  hipStream_t stream;
};

// Standard attention with S and P materialised in device memory (bf16 inputs):
// S float32 and P bfloat16, [BH][N][ldp] each, ldp = N rounded up to 64.
struct StdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  float* s;
  uint16_t* p;
  long BH;
  int N, d, ldp;
  float scale;
  bool causal;
  hipStream_t stream;
};

hipError_t launch_fwd_f32(const FwdArgs& a);
hipError_t launch_fwd_bf16(const FwdArgs& a);
hipError_t launch_fwd_bf16_pp(const FwdArgs& a);   // d = 128, no bias
hipError_t launch_fwd_bf16_w64(const FwdArgs& a);  // d = 128, no bias
hipError_t launch_fwd_fp8(const FwdArgs& a);
hipError_t launch_delta(const BwdArgs& a, bool bf16);
hipError_t launch_dkdv_f32(const BwdArgs& a);
hipError_t launch_dq_f32(const BwdArgs& a);
hipError_t launch_dkdv_bf16(const BwdArgs& a);
hipError_t launch_dq_bf16(const BwdArgs& a);  // also writes delta (from O and dO)
hipError_t launch_std_bf16(const StdArgs& a);

}  // namespace fa

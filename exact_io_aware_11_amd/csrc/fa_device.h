// Device-side building blocks shared by the gfx950 attention kernels.
//
// Matrix-core lane layouts used throughout (measured on gfx950 with an
// in-bounds probe, and relied on by every kernel):
//  v_mfma_f32_32x32x16_bf16  (A 32x16, B 16x32, C 32x32), lane l, g = l / 32:
//    A: lane l holds A[l % 32][8g .. 8g+7]
//    B: lane l holds B[8g .. 8g+7][l % 32]
//    C: lane l element i holds C[8(i/4) + 4g + i%4][l % 32]
//  Only the pairing of A's and B's k-slots matters to the product, so any
//  permutation of k applied to both operands is free; the kernels use that to
//  feed a C-layout tile straight back in as a B operand.
//  ds_read_b64_tr_b16: within each group of 16 lanes, output lane j element r
//    is element (j % 4) of the 8 bytes addressed by source lane 4r + j/4.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_kernels.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// The forward moves its reference row max only when a score exceeds it by
// more than this many powers of two (probabilities stay <= 2^16).
constexpr float kRescaleLog2 = 16.f;

__device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// fp8 (OCP e4m3fn) x fp8, K = 64 per instruction, unit block scales.
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

// fp8 e4m3 product with per-lane power-of-two (e8m0) block scales: byte
// OPA of sa scales this lane's k block of A, byte OPB of sb that of B.
template <int OPA, int OPB>
__device__ __forceinline__ f32x16 mfma_fp8_scaled(i32x8 a, i32x8 b, f32x16 c, uint32_t sa,
                                                  uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPA, (int)sa, OPB, (int)sb);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// This lane's index in the wave, computed where it is used: the asm is not
// merged with other computations of the lane id or hoisted out of a loop, so
// no register holds it (or values derived from it) across a long scan.
__device__ __forceinline__ int lane_id_here() {
  int l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// Raw buffer resource over `bytes` bytes at `base`.  Buffer loads at byte
// offsets past the end do not touch memory and deliver zeros (also into LDS),
// which is how tiles running past the sequence end are padded.
// num_records is a 32-bit unsigned field.  Longer extents saturate at
// 2^32 - 1: every resource here starts at the tile it serves and is read at
// offsets far below 2^32, so for those reads a saturated bound is as good as
// the true one (a wrapped count would turn in-range rows into zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const uint32_t n = bytes <= 0 ? 0u : bytes >= 0xFFFFFFFFL ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_bit_cast(int, n), 0x00020000);
}
// The same for a tile of `rows` rows of ROW_BYTES bytes (rows may be <= 0),
// saturated in 32-bit arithmetic: rows past the largest count that fits
// 2^32 - 1 bytes give 2^32 - 1.  The 64-bit form above needs a vector
// compare per call (gfx950 has no unsigned 64-bit scalar compare), which in
// the tile loops costs instructions and, in the dQ kernel with a bias, pushed
// the register allocation into heavy spilling.
template <int ROW_BYTES>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_tile_rsrc(const void* base, int rows) {
  constexpr int kMaxRows = (int)(0xFFFFFFFFu / ROW_BYTES);
  const uint32_t n =
      rows <= 0 ? 0u : rows >= kMaxRows ? 0xFFFFFFFFu : (uint32_t)rows * (uint32_t)ROW_BYTES;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           __builtin_bit_cast(int, n), 0x00020000);
}
// Loads into registers through a buffer resource (reads past num_records
// return zeros): 16 or 4 bytes per lane at voff + soff + imm.
template <int IMM = 0>
__device__ __forceinline__ f32x4 buffer_load_f32x4(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                   uint32_t soff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff + IMM, soff, 0));
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                                 uint32_t soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
// The (b, h) slice of an additive bias as a buffer resource.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const Bias& b, uint32_t bh) {
  const uint32_t bi = bh / (uint32_t)b.H, hi = bh - bi * (uint32_t)b.H;
  return make_rsrc(b.p + (long long)bi * b.sb + (long long)hi * b.sh, (long)b.head_bytes);
}

// Direct load of 16 bytes per lane, from byte offset voff of the resource, to
// LDS at dst + 16 * lane.  The LDS address is wave-uniform (it goes to M0).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, const void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, 0, 0, 0);
}

// The same with a wave-uniform byte offset soff added (scalar operand).
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t r, const void* dst, uint32_t voff,
                                           uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}

// Direct load of 4 bytes per lane (256 bytes per wave) to LDS at dst + 4 * lane.
__device__ __forceinline__ void load_lds4(__amdgpu_buffer_rsrc_t r, const void* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4,
                                           voff, 0, 0, 0);
}

// Workgroup barrier for the staged pipelines.  Before the barrier this wave's
// LDS reads and writes are complete (lgkmcnt 0) and at most VM of its vector
// memory operations -- the newest batch of direct HBM->LDS loads -- are still
// in flight.  (__syncthreads() would also drain those loads: its workgroup
// fence waits for vmcnt(0), which defeats prefetching.)  The "memory" clobber
// keeps the compiler from moving memory accesses across the barrier.
// Waitcnt immediate (gfx9): vmcnt in bits [3:0] and [15:14], expcnt [6:4]
// (7: no wait), lgkmcnt [11:8] (0: wait for all).
template <int VM>
__device__ __forceinline__ void wait_vm() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
}
template <int VM>
__device__ __forceinline__ void barrier_vm() {
  wait_vm<VM>();
  asm volatile("s_barrier" ::: "memory");
}

// max / sum of a value over lanes l and l ^ 32 (the two halves of a wave).
__device__ __forceinline__ float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16-byte LDS read of 8 bf16 (p points into a __shared__ array).
__device__ __forceinline__ bf16x8 lds_read_b128(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// Transposing 8-byte LDS read (see the layout note at the top); p points
// into a __shared__ array.
__device__ __forceinline__ bf16x4 lds_read_tr16(const uint16_t* p) {
  s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((FA_LDS s16x4*)(p));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 concat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Round-to-nearest-even float -> bfloat16 of 8 consecutive accumulator values.
__device__ __forceinline__ bf16x8 to_bf16x8(const f32x16& c, int first) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = (__bf16)c[first + e];
  return r;
}

// acc + sum of 8 bf16 values (v_dot2_f32_bf16 against (1, 1)).
__device__ __forceinline__ float sum_bf16x8(bf16x8 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const bf16x2 p = {v[e], v[e + 1]};
    acc = __builtin_amdgcn_fdot2_f32_bf16(p, one, acc, false);
  }
  return acc;
}

// Workgroup -> (head, block) mapping.  Workgroups are dispatched to the 8
// XCDs round-robin (id % 8), each XCD with its own L2.  When the grid divides
// by 8, XCD x is given a contiguous range of total/8 logical blocks, so the
// blocks of a few heads run on one XCD and share its L2 copy of those heads'
// tensors.  Causal work is uneven (a row block i sees i+1 key tiles; a key
// block j is seen by the row blocks from j on): there the XCD's range is
// walked block-major across its heads, heaviest blocks first, which keeps the
// end of the launch to light blocks.  order: 0 plain, 1 heavy blocks are the
// last indices (row blocks), 2 heavy blocks are the first (key blocks).
enum : int { kOrderPlain = 0, kOrderHeavyLast = 1, kOrderHeavyFirst = 2 };
__device__ __forceinline__ void map_block(uint32_t w, uint32_t n_blk, uint32_t total, int order,
                                          uint32_t& bh, uint32_t& blk) {
  if ((total & 7u) == 0u && order != kOrderPlain && ((total >> 3) % n_blk) == 0u) {
    const uint32_t hx = (total >> 3) / n_blk, r = w >> 3;
    bh = (w & 7u) * hx + r % hx;
    blk = order == kOrderHeavyLast ? n_blk - 1u - r / hx : r / hx;
    return;
  }
  uint32_t logical = w;
  if ((total & 7u) == 0u) logical = (w & 7u) * (total >> 3) + (w >> 3);
  bh = logical / n_blk;
  blk = logical - bh * n_blk;
  if (order == kOrderHeavyLast) blk = n_blk - 1u - blk;
}

// Mapping for a bias shared by the heads of a batch entry.  With map_block's
// plain order the workgroups that run together on one XCD take every block of
// one or two heads: they share those heads' tiles in L2, but each head reads
// the whole bias again.  Here the XCD's range of total/8 logical blocks is
// cut into groups of kGroupHeads heads x U blocks, heads minor, with U chosen
// so that a group is about what one XCD runs at once: each bias tile is then
// read by kGroupHeads workgroups and each Q/K/V tile by U, at about the same
// time.  Blocks ascend across groups (heavy first for causal key blocks);
// heavy_last reverses them (causal row blocks).  Requires total % 8 == 0,
// heads % kGroupHeads == 0 and n_blk % U == 0 (then it is a permutation).
constexpr uint32_t kGroupHeads = 8;
__device__ __forceinline__ void map_block_grouped(uint32_t w, uint32_t n_blk, uint32_t total,
                                                  uint32_t U, bool heavy_last, uint32_t& bh,
                                                  uint32_t& blk) {
  const uint32_t logical = (w & 7u) * (total >> 3) + (w >> 3);
  const uint32_t G = kGroupHeads * U;
  const uint32_t grp = logical / G, in = logical - grp * G;
  const uint32_t per_head_group = n_blk / U;  // block groups per head group
  const uint32_t hg = grp / per_head_group, bg = grp - hg * per_head_group;
  bh = hg * kGroupHeads + in % kGroupHeads;
  blk = bg * U + in / kGroupHeads;
  if (heavy_last) blk = n_blk - 1u - blk;
}

// Blocks per group for a launch over bh_count heads x n_blk blocks, or 0 when
// the grouped order does not apply (host side).
inline int group_blocks(const Bias& b, long bh_count, uint32_t n_blk, uint32_t want) {
  return b.p && b.sh == 0 && bh_count % (long)kGroupHeads == 0 && n_blk % want == 0 ? (int)want : 0;
}

// 16-byte-chunk XOR swizzle of a [rows][D] bf16 tile in LDS (D = 64 or 128).
// It serves the two read patterns the kernels use, both free of bank
// conflicts (64 banks x 4 bytes):
//  * ds_read_b128 of one logical chunk by 16 consecutive rows (A/B operands
//    along the head dimension): the 16 rows land in 16 different 16-byte
//    bank groups;
//  * ds_read_b64_tr_b16 of 4 consecutive logical chunks by 4 consecutive
//    rows (the transposed operand): the 16 (row, chunk) pairs land in 16
//    different bank groups.
// Rows are 256 bytes (D = 128, one full bank sweep) or 128 bytes (D = 64,
// two rows per sweep); the swizzle depends only on row % 16.
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int tile_off(int row, int chunk) {  // element offset
  return row * D + ((chunk ^ swz<D>(row)) << 3);
}

}  // namespace fa

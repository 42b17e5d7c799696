// Standard (materialising) attention, bfloat16: the method the pages set the
// IO-aware kernels against.  The reading notes ("5.4 FlashAttention (1/2/3)",
// standard attention) and the explainer's background section describe it:
// S = Q K^T is written to device memory, read back for a row-wise softmax,
// P is written to device memory, and read back once more for O = P V -- four
// passes over N x N matrices per head, where the flash kernels move only
// O(N d) bytes ("FlashAttention-1: eliminating IO", introduction).  It exists
// here as the measured baseline of that IO claim, not as the product path.
//
// Three launches on one stream:
//  1. std_scores_kernel: S = scale Q K^T, float32, one 64 x 64 tile per
//     workgroup (four waves, one 32 x 32 block each, v_mfma_f32_32x32x16_bf16
//     with both operands loaded straight from the row-major Q and K).
//  2. std_softmax_kernel: one wave per row: the row max and the sum of exp
//     over the visible keys (all, or j <= i under the causal mask) in one pass
//     with a running rescale, then P = exp(S - m) / l in bfloat16 (0 where
//     masked and in the row padding) and LSE = m + ln l.
//  3. std_pv_kernel: O = P V on the matrix cores, P (the B operand of
//     O^T = V^T P^T) loaded from the row-major P, V staged through LDS and
//     read transposed (ds_read_b64_tr_b16).  The masked part of P is zero and
//     is multiplied like the rest: standard attention does not skip it.
// S and P rows have a pitch of N rounded up to 64 elements.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kStdTile = 64;

// S tile (64 queries x 64 keys) of one head: wave w computes queries
// 32 (w / 2) .. +31 and keys 32 (w % 2) .. +31.  A = Q rows, B = K^T: lane l
// (g = l / 32) holds Q[i0 + l % 32][16 t + 8 g .. +7] and K[j0 + l % 32][same].
template <int D>
__global__ __launch_bounds__(256) void std_scores_kernel(const uint16_t* __restrict__ Q,
                                                         const uint16_t* __restrict__ K,
                                                         float* __restrict__ S, int N, int ldp,
                                                         float scale) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 5, r32 = lane & 31;
  const size_t bh = blockIdx.z;
  const int i0 = blockIdx.y * kStdTile + 32 * (wave >> 1);
  const int j0 = blockIdx.x * kStdTile + 32 * (wave & 1);
  const uint16_t* Qh = Q + bh * (size_t)N * D;
  const uint16_t* Kh = K + bh * (size_t)N * D;
  const int qi = i0 + r32, kj = j0 + r32;
  f32x16 acc = {};
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const bf16x8 a = qi < N ? *reinterpret_cast<const bf16x8*>(Qh + (size_t)qi * D + 16 * t + 8 * g)
                            : bf16x8{};
    const bf16x8 b = kj < N ? *reinterpret_cast<const bf16x8*>(Kh + (size_t)kj * D + 16 * t + 8 * g)
                            : bf16x8{};
    acc = mfma_bf16(a, b, acc);
  }
  // C layout: element e of lane l is row 8 (e / 4) + 4 g + e % 4, column l % 32.
  float* Sh = S + bh * (size_t)N * ldp;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int i = i0 + 8 * (e >> 2) + 4 * g + (e & 3);
    if (i < N && kj < N) Sh[(size_t)i * ldp + kj] = acc[e] * scale;
  }
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per row (four rows per workgroup).  Row i of head bh sees keys
// [0, vis) with vis = N, or i + 1 under the causal mask.
__global__ __launch_bounds__(256) void std_softmax_kernel(const float* __restrict__ S,
                                                          uint16_t* __restrict__ P,
                                                          float* __restrict__ LSE, long rows,
                                                          int N, int ldp, int causal) {
  const int lane = threadIdx.x & 63;
  const long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int i = (int)(row % N);
  const int vis = causal ? i + 1 : N;
  const float* Sr = S + (size_t)row * ldp;
  // running max and sum of exp over this lane's keys (lane, lane + 64, ...)
  float m = -INFINITY, l = 0.f;
  for (int j = lane; j < vis; j += 64) {
    const float s = Sr[j];
    if (s > m) {
      l = l * exp2_fast((m - s) * kLog2e) + 1.f;
      m = s;
    } else {
      l += exp2_fast((s - m) * kLog2e);
    }
  }
  const float mr = wave_max(m);
  const float lr = wave_sum(m == -INFINITY ? 0.f : l * exp2_fast((m - mr) * kLog2e));
  const float inv = 1.f / lr;
  uint16_t* Pr = P + (size_t)row * ldp;
  for (int j = lane; j < ldp; j += 64) {
    const float p = j < vis ? exp2_fast((Sr[j] - mr) * kLog2e) * inv : 0.f;
    Pr[j] = __builtin_bit_cast(uint16_t, (__bf16)p);
  }
  if (lane == 0) LSE[row] = mr + __logf(lr);
}

// O = P V for 64 queries of one head per workgroup: wave w owns queries
// 32 (w % 2) .. +31 and head dims D/2 (w / 2) .. +D/2-1, as O^T = V^T P^T on
// 32 x 32 blocks.  B = P^T: lane l holds P[i0 + l % 32][key0 + 8 g .. +7]
// (a 16-byte load from the row).  A = V^T: lane l holds V[key0 + 8 g .. +7]
// [d0 + l % 32], read from the LDS tile with two transposing reads: source lane
// s addresses the 4 head dims 16 ((s / 16) % 2) + 4 (s % 4) of key row
// 8 g + (s % 16) / 4 (+4 for the second read).
template <int D>
__global__ __launch_bounds__(256) void std_pv_kernel(const uint16_t* __restrict__ P,
                                                     const uint16_t* __restrict__ V,
                                                     uint16_t* __restrict__ O, int N, int ldp) {
  constexpr int NB = D / 64;  // 32-wide head-dim blocks per wave
  __shared__ __attribute__((aligned(1024))) uint16_t vt[kStdTile * D];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 5, r32 = lane & 31;
  const size_t bh = blockIdx.y;
  const int i0 = blockIdx.x * kStdTile + 32 * (wave & 1);
  const int d0 = (D / 2) * (wave >> 1);
  const uint16_t* Vh = V + bh * (size_t)N * D;
  const uint16_t* Pr = P + (bh * (size_t)N + (size_t)min(i0 + r32, N - 1)) * ldp;
  const int tr_row = 8 * g + ((lane & 15) >> 2);
  // (the swizzle depends on row % 16: the second read's rows, 4 further on,
  // have their own offsets; 16 rows further on the offsets repeat)
  int voff[NB][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const int d = d0 + 32 * nb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h) voff[nb][h] = tile_off<D>(tr_row + 4 * h, d >> 3) + (d & 7);
  }
  f32x16 acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x16{};
  for (int key0 = 0; key0 < N; key0 += kStdTile) {
    __syncthreads();  // the previous chunk's reads are done
    // stage V rows key0 .. key0 + 63 (zeros past N), 16 bytes per thread per pass
#pragma unroll
    for (int x = 0; x < kStdTile * D / 8 / 256; ++x) {
      const int c = x * 256 + tid, row = c / (D / 8), ch = c % (D / 8);
      bf16x8 val = {};
      if (key0 + row < N)
        val = *reinterpret_cast<const bf16x8*>(Vh + (size_t)(key0 + row) * D + 8 * ch);
      *reinterpret_cast<bf16x8*>(vt + tile_off<D>(row, ch)) = val;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < kStdTile / 16; ++ks) {
      const bf16x8 b = *reinterpret_cast<const bf16x8*>(Pr + key0 + 16 * ks + 8 * g);
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        acc[nb] = mfma_bf16(concat(lds_read_tr16(vt + voff[nb][0] + 16 * ks * D),
                                   lds_read_tr16(vt + voff[nb][1] + 16 * ks * D)),
                            b, acc[nb]);
      }
    }
  }
  // C layout of O^T: element e of lane l is head dim 8 (e / 4) + 4 g + e % 4 of
  // the block, query l % 32.
  const int qi = i0 + r32;
  if (qi < N) {
    uint16_t* Orow = O + (bh * (size_t)N + qi) * D;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[nb][4 * q4 + e];
        *reinterpret_cast<bf16x4*>(Orow + d0 + 32 * nb + 8 * q4 + 4 * g) = v;
      }
  }
}

template <int D>
hipError_t launch_std_t(const StdArgs& a) {
  const int tiles = (a.N + kStdTile - 1) / kStdTile;
  hipLaunchKernelGGL(std_scores_kernel<D>, dim3(tiles, tiles, (unsigned)a.BH), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, a.s, a.N, a.ldp,
                     a.scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long rows = a.BH * a.N;
  hipLaunchKernelGGL(std_softmax_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0,
                     a.stream, a.s, a.p, a.lse, rows, a.N, a.ldp, a.causal ? 1 : 0);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(std_pv_kernel<D>, dim3(tiles, (unsigned)a.BH), dim3(256), 0, a.stream,
                     (const uint16_t*)a.p, (const uint16_t*)a.v, (uint16_t*)a.o, a.N, a.ldp);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_std_bf16(const StdArgs& a) {
  return a.d == 64 ? launch_std_t<64>(a) : launch_std_t<128>(a);
}

}  // namespace fa

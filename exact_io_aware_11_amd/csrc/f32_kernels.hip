// float32 attention kernels (forward, delta, dK/dV, dQ) and the delta kernel
// for both float32 and bfloat16.
//
// What they compute follows "FlashAttention-1: eliminating IO": the forward
// of sections 10.2.1-10.2.3 (running max m, running sum l, unnormalised
// accumulator rescaled by alpha = exp(m_old - m_new), one final division,
// LSE = m + ln l), and the recompute backward of section 10.2.4
// (P = exp(S - LSE), dV = P^T dO, dP = dO V^T, dS = P o (dP - delta),
// dQ = scale dS K, dK = scale dS^T Q, delta_i = dO_i . O_i).
//
// Tiles are Br = Bc = 32 rows, the block sizes of the FA1 page's examples
// (sections 10.2.3 and 10.2.4).  These kernels serve float32 problems, which
// the pages use for their exactness checks; float32 on gfx950 has the same
// peak on the vector ALUs as on the matrix cores, so they are plain
// LDS-tiled FMA kernels with exact expf/logf.  One workgroup of 256 threads
// per (batch, head, 32-row block); 8 threads share a row.
//
// Optional additive bias on the scaled scores (explainer V2 section: mask and
// bias merged into the score stage), read straight from global memory; -inf
// masks a key, a row with no finite score gets O = 0 and LSE = -inf, and the
// backward gives such rows (LSE = -inf) P = 0.
#include <math.h>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int kBR = 32, kBC = 32;

__device__ __forceinline__ float group8_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 1, 8));
  x = fmaxf(x, __shfl_xor(x, 2, 8));
  x = fmaxf(x, __shfl_xor(x, 4, 8));
  return x;
}
__device__ __forceinline__ float group8_sum(float x) {
  x += __shfl_xor(x, 1, 8);
  x += __shfl_xor(x, 2, 8);
  x += __shfl_xor(x, 4, 8);
  return x;
}

// Rows [row0, row0 + rows) of a [N][D] matrix into an LDS tile, zero past N.
template <int D, int LD>
__device__ __forceinline__ void load_rows(float (*dst)[LD], const float* src, int row0, int rows,
                                          int N) {
  for (int x = threadIdx.x; x < rows * D; x += 256) {
    const int rr = x / D, c = x - rr * D, row = row0 + rr;
    dst[rr][c] = row < N ? src[(size_t)row * D + c] : 0.f;
  }
}

// Row `row` of the (b, h) slice of a bias, or null.
__device__ __forceinline__ const float* bias_row(const Bias& b, size_t bh, int row) {
  if (!b.p) return nullptr;
  const size_t bi = bh / (size_t)b.H, hi = bh - bi * (size_t)b.H;
  return b.p + (long long)bi * b.sb + (long long)hi * b.sh + (long long)row * b.sq;
}

}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_f32_kernel(const float* __restrict__ Q,
                                                      const float* __restrict__ K,
                                                      const float* __restrict__ V,
                                                      float* __restrict__ O,
                                                      float* __restrict__ LSE, int N, float scale,
                                                      Bias bias) {
  constexpr int DS = D / 8;
  __shared__ float Qs[kBR][D + 1], Ks[kBC][D + 1], Vs[kBC][D], Ps[kBR][kBC + 1];
  const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
  const int nq = (N + kBR - 1) / kBR;
  const size_t bh = blockIdx.x / nq;
  const int q0 = (int)(blockIdx.x - bh * nq) * kBR, qrow = q0 + r;
  const size_t head = bh * (size_t)N * D;
  load_rows<D, D + 1>(Qs, Q + head, q0, kBR, N);
  const float* brow = qrow < N ? bias_row(bias, bh, qrow) : nullptr;
  float acc[DS];
#pragma unroll
  for (int x = 0; x < DS; ++x) acc[x] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kBC) {
    __syncthreads();
    load_rows<D, D + 1>(Ks, K + head, k0, kBC, N);
    load_rows<D, D>(Vs, V + head, k0, kBC, N);
    __syncthreads();
    float s[4], mt = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = sub + 8 * cc, key = k0 + c;
      float dot = 0.f;
      for (int x = 0; x < D; ++x) dot = fmaf(Qs[r][x], Ks[c][x], dot);
      const bool vis = key < N && (!CAUSAL || key <= qrow);
      s[cc] = vis ? dot * scale + (brow ? brow[key] : 0.f) : -INFINITY;
      mt = fmaxf(mt, s[cc]);
    }
    mt = group8_max(mt);
    const float m_new = fmaxf(m, mt);
    // (m_new = -inf: no finite score yet; every p is 0 and nothing rescales)
    const float alpha = m_new == -INFINITY ? 1.f : expf(m - m_new);
    float rs = 0.f;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const float p = m_new == -INFINITY ? 0.f : expf(s[cc] - m_new);
      Ps[r][sub + 8 * cc] = p;
      rs += p;
    }
    rs = group8_sum(rs);
    l = l * alpha + rs;
    m = m_new;
    __syncthreads();
#pragma unroll
    for (int x = 0; x < DS; ++x) {
      const int d = sub * DS + x;
      float a = acc[x] * alpha;
      for (int c = 0; c < kBC; ++c) a = fmaf(Ps[r][c], Vs[c][d], a);
      acc[x] = a;
    }
  }
  if (qrow < N) {
    float* Orow = O + head + (size_t)qrow * D + sub * DS;
#pragma unroll
    for (int x = 0; x < DS; ++x) Orow[x] = l > 0.f ? acc[x] / l : 0.f;
    if (sub == 0) LSE[bh * N + qrow] = l > 0.f ? m + logf(l) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dkdv_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dK, float* __restrict__ dV, int N, float scale, Bias bias) {
  constexpr int DS = D / 8;
  __shared__ float Ks[kBC][D + 1], Vs[kBC][D + 1], Qs[kBR][D + 1], dOs[kBR][D + 1];
  __shared__ float Ps[kBR][kBC + 1], dSs[kBR][kBC + 1], lse_s[kBR], del_s[kBR];
  const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
  const int nk = (N + kBC - 1) / kBC;
  const size_t bh = blockIdx.x / nk;
  const int k0 = (int)(blockIdx.x - bh * nk) * kBC;
  const size_t head = bh * (size_t)N * D;
  load_rows<D, D + 1>(Ks, K + head, k0, kBC, N);
  load_rows<D, D + 1>(Vs, V + head, k0, kBC, N);
  float dk[DS], dv[DS];
#pragma unroll
  for (int x = 0; x < DS; ++x) dk[x] = dv[x] = 0.f;
  const int q_start = CAUSAL ? k0 : 0;  // earlier query tiles see none of these keys
  for (int q0 = q_start; q0 < N; q0 += kBR) {
    __syncthreads();
    load_rows<D, D + 1>(Qs, Q + head, q0, kBR, N);
    load_rows<D, D + 1>(dOs, dO + head, q0, kBR, N);
    if (tid < kBR) {
      const int q = q0 + tid;
      lse_s[tid] = q < N ? LSE[bh * N + q] : 0.f;
      del_s[tid] = q < N ? Delta[bh * N + q] : 0.f;
    }
    __syncthreads();
    const int q = q0 + r;
    const float* brow = q < N ? bias_row(bias, bh, q) : nullptr;
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = sub + 8 * cc, key = k0 + c;
      float sd = 0.f, dpd = 0.f;
      for (int x = 0; x < D; ++x) {
        sd = fmaf(Qs[r][x], Ks[c][x], sd);
        dpd = fmaf(dOs[r][x], Vs[c][x], dpd);
      }
      // (LSE = -inf: a row with no finite score, P = 0)
      const bool valid = key < N && q < N && (!CAUSAL || key <= q) && lse_s[r] != -INFINITY;
      const float p = valid ? expf(sd * scale + (brow ? brow[key] : 0.f) - lse_s[r]) : 0.f;
      Ps[r][c] = p;
      dSs[r][c] = p * (dpd - del_s[r]);
    }
    __syncthreads();
    const int kk = r;  // this thread's key row for accumulation
#pragma unroll
    for (int x = 0; x < DS; ++x) {
      const int d = sub * DS + x;
      float a = dv[x], b = dk[x];
      for (int rr = 0; rr < kBR; ++rr) {
        a = fmaf(Ps[rr][kk], dOs[rr][d], a);
        b = fmaf(dSs[rr][kk], Qs[rr][d], b);
      }
      dv[x] = a;
      dk[x] = b;
    }
  }
  const int key = k0 + r;
  if (key < N) {
#pragma unroll
    for (int x = 0; x < DS; ++x) {
      dK[head + (size_t)key * D + sub * DS + x] = dk[x] * scale;
      dV[head + (size_t)key * D + sub * DS + x] = dv[x];
    }
  }
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void bwd_dq_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    const float* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Delta,
    float* __restrict__ dQ, int N, float scale, Bias bias) {
  constexpr int DS = D / 8;
  __shared__ float Qs[kBR][D + 1], dOs[kBR][D + 1], Ks[kBC][D + 1], Vs[kBC][D + 1];
  __shared__ float dSs[kBR][kBC + 1];
  const int tid = threadIdx.x, r = tid >> 3, sub = tid & 7;
  const int nq = (N + kBR - 1) / kBR;
  const size_t bh = blockIdx.x / nq;
  const int q0 = (int)(blockIdx.x - bh * nq) * kBR, q = q0 + r;
  const size_t head = bh * (size_t)N * D;
  load_rows<D, D + 1>(Qs, Q + head, q0, kBR, N);
  load_rows<D, D + 1>(dOs, dO + head, q0, kBR, N);
  const float lse = q < N ? LSE[bh * N + q] : 0.f;
  const float del = q < N ? Delta[bh * N + q] : 0.f;
  const float* brow = q < N ? bias_row(bias, bh, q) : nullptr;
  float dq[DS];
#pragma unroll
  for (int x = 0; x < DS; ++x) dq[x] = 0.f;
  const int kv_end = CAUSAL ? min(N, q0 + kBR) : N;
  for (int k0 = 0; k0 < kv_end; k0 += kBC) {
    __syncthreads();
    load_rows<D, D + 1>(Ks, K + head, k0, kBC, N);
    load_rows<D, D + 1>(Vs, V + head, k0, kBC, N);
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < 4; ++cc) {
      const int c = sub + 8 * cc, key = k0 + c;
      float sd = 0.f, dpd = 0.f;
      for (int x = 0; x < D; ++x) {
        sd = fmaf(Qs[r][x], Ks[c][x], sd);
        dpd = fmaf(dOs[r][x], Vs[c][x], dpd);
      }
      const bool valid = key < N && q < N && (!CAUSAL || key <= q) && lse != -INFINITY;
      const float p = valid ? expf(sd * scale + (brow ? brow[key] : 0.f) - lse) : 0.f;
      dSs[r][c] = p * (dpd - del);
    }
    __syncthreads();
#pragma unroll
    for (int x = 0; x < DS; ++x) {
      const int d = sub * DS + x;
      float a = dq[x];
      for (int c = 0; c < kBC; ++c) a = fmaf(dSs[r][c], Ks[c][d], a);
      dq[x] = a;
    }
  }
  if (q < N) {
#pragma unroll
    for (int x = 0; x < DS; ++x) dQ[head + (size_t)q * D + sub * DS + x] = dq[x] * scale;
  }
}

// delta_i = sum_c dO_ic O_ic (FA1 page, section 10.2.4), float32 result.
// HBM-bound: a row takes LPR lanes (one 16-byte chunk of O and of dO per
// lane and pass, PER passes), and every lane works on R rows of its
// workgroup, issuing all its loads before any arithmetic so that enough
// bytes are in flight per CU to keep HBM busy.
template <bool BF16, int D>
struct DeltaShape {
  static constexpr int CH = BF16 ? D / 8 : D / 4;     // 16-byte chunks per row
  static constexpr int LPR = CH < 16 ? CH : 16;       // lanes per row
  static constexpr int PER = CH / LPR;                // chunks per lane and row
  static constexpr int R = 4;                         // rows per lane
  static constexpr int ROWS = R * 256 / LPR;          // rows per workgroup
};
template <bool BF16, int D>
__global__ __launch_bounds__(256) void delta_kernel(const void* __restrict__ Ov,
                                                    const void* __restrict__ dOv,
                                                    float* __restrict__ delta, long rows) {
  using S = DeltaShape<BF16, D>;
  constexpr int LPR = S::LPR, PER = S::PER, R = S::R, CH = S::CH;
  const int sub = threadIdx.x % LPR;
  const long row0 = (long)blockIdx.x * S::ROWS + threadIdx.x / LPR;  // rows row0 + (256 / LPR) r
  const uint4* o = reinterpret_cast<const uint4*>(Ov);
  const uint4* g = reinterpret_cast<const uint4*>(dOv);
  uint4 a[R][PER], b[R][PER];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const long row = row0 + (long)(256 / LPR) * r;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      if (row < rows) {
        a[r][c] = o[row * CH + sub + LPR * c];
        b[r][c] = g[row * CH + sub + LPR * c];
      } else {
        a[r][c] = b[r][c] = uint4{0u, 0u, 0u, 0u};
      }
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float acc = 0.f;
#pragma unroll
    for (int c = 0; c < PER; ++c) {
      if constexpr (BF16) {
        const bf16x8 x = __builtin_bit_cast(bf16x8, a[r][c]);
        const bf16x8 y = __builtin_bit_cast(bf16x8, b[r][c]);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)x[e], (float)y[e], acc);
      } else {
        const float4 x = __builtin_bit_cast(float4, a[r][c]);
        const float4 y = __builtin_bit_cast(float4, b[r][c]);
        acc = fmaf(x.x, y.x, acc);
        acc = fmaf(x.y, y.y, acc);
        acc = fmaf(x.z, y.z, acc);
        acc = fmaf(x.w, y.w, acc);
      }
    }
#pragma unroll
    for (int m = LPR / 2; m > 0; m /= 2) acc += __shfl_xor(acc, m, LPR);
    const long row = row0 + (long)(256 / LPR) * r;
    if (row < rows && sub == 0) delta[row] = acc;
  }
}

template <bool BF16, int D>
static void launch_delta_t(const BwdArgs& a, long rows) {
  constexpr int ROWS = DeltaShape<BF16, D>::ROWS;
  const dim3 grid((unsigned)((rows + ROWS - 1) / ROWS));
  hipLaunchKernelGGL((delta_kernel<BF16, D>), grid, dim3(256), 0, a.stream, a.o, a.dout, a.delta, rows);
}

hipError_t launch_delta(const BwdArgs& a, bool bf16) {
  const long rows = a.BH * (long)a.N;
  if (bf16) {
    if (a.d == 64) launch_delta_t<true, 64>(a, rows);
    else launch_delta_t<true, 128>(a, rows);
  } else {
    if (a.d == 64) launch_delta_t<false, 64>(a, rows);
    else launch_delta_t<false, 128>(a, rows);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t fwd_f32_t(const FwdArgs& a) {
  const long nq = (a.N + kBR - 1) / kBR;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nq)), dim3(256), 0,
                     a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                     (float*)a.o, a.lse, a.N, a.scale, a.bias);
  return hipGetLastError();
}

hipError_t launch_fwd_f32(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? fwd_f32_t<64, true>(a) : fwd_f32_t<64, false>(a);
  return a.causal ? fwd_f32_t<128, true>(a) : fwd_f32_t<128, false>(a);
}

template <int D, bool CAUSAL>
static hipError_t dkdv_f32_t(const BwdArgs& a) {
  const long nb = (a.N + kBC - 1) / kBC;
  hipLaunchKernelGGL((bwd_dkdv_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nb)), dim3(256), 0,
                     a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                     (const float*)a.dout, a.lse, a.delta, (float*)a.dk, (float*)a.dv, a.N,
                     a.scale, a.bias);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t dq_f32_t(const BwdArgs& a) {
  const long nb = (a.N + kBR - 1) / kBR;
  hipLaunchKernelGGL((bwd_dq_f32_kernel<D, CAUSAL>), dim3((unsigned)(a.BH * nb)), dim3(256), 0,
                     a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                     (const float*)a.dout, a.lse, a.delta, (float*)a.dq, a.N, a.scale, a.bias);
  return hipGetLastError();
}

hipError_t launch_dkdv_f32(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dkdv_f32_t<64, true>(a) : dkdv_f32_t<64, false>(a);
  return a.causal ? dkdv_f32_t<128, true>(a) : dkdv_f32_t<128, false>(a);
}

hipError_t launch_dq_f32(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dq_f32_t<64, true>(a) : dq_f32_t<64, false>(a);
  return a.causal ? dq_f32_t<128, true>(a) : dq_f32_t<128, false>(a);
}

}  // namespace fa

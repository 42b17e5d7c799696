// Forward attention, bfloat16 inputs, float32 accumulation, gfx950 MFMA.
//
// What it computes ("FlashAttention-1: eliminating IO", sections 10.2.1 to
// 10.2.3; explainer V2 section; reading notes code 3-1): for each query row,
// O = softmax(scale Q K^T) V and LSE = ln sum exp(scale q.k), in one pass over
// the key tiles with a running max m, a running sum l and an unnormalised
// accumulator rescaled by alpha = exp(m_old - m_new), and one division at the
// end.  Scores and probabilities live only in registers.
//
// Work split (explainer V2 section; FA1 page section 10.2.5): one workgroup
// of 4 waves per (batch, head, block of 128 query rows); each wave owns 32
// query rows and scans every visible key tile of 64 keys.
//
// gfx950 mapping:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) comes from LDS,
//    Q (B operand) stays in registers for the whole scan.  In the C layout a
//    lane then holds 16 keys of ONE query, so the row max is an in-lane max
//    plus one exchange between the wave's halves (v_permlane32_swap), and the
//    row sum needs no exchange until the end.
//  * O^T = V^T P^T: the probabilities are converted to bf16 in place and used
//    directly as the B operand (the C-layout key order is matched by reading
//    V with ds_read_b64_tr_b16 in the same order); the accumulator then holds
//    16 head dims of one query per lane, so the alpha rescale and the final
//    division are per-lane scalars.
//  * K and V tiles are double-buffered in LDS (16-byte XOR swizzle), staged
//    from HBM with 16-byte loads issued one tile ahead; one barrier per tile.
//  * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    uint32_t n_qblk, uint32_t total, float scale, float scale_log2) {
  constexpr int BM = 128, BN = 64, CH = D / 8, TILE = BN * D;
  constexpr int PER = BN * CH / 256;  // 16-byte chunks per thread per tensor per tile
  __shared__ __attribute__((aligned(16))) uint16_t lds[2][2][TILE];  // [buffer][K, V]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  uint32_t bh, qblk;
  map_block(blockIdx.x, n_qblk, total, CAUSAL, bh, qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  const int q0 = (int)qblk * BM + wave * 32;  // first query row of this wave
  const int qrow = q0 + r32;                  // the query of this lane's column

  // Q fragment as the B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8g .. +7].
  bf16x8 qf[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if (qrow < N) qf[t] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + 16 * t + 8 * g);
    else qf[t] = bf16x8{};
  }

  const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  uint4 kreg[PER], vreg[PER];
  auto gload = [&](int j) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int c = tid + 256 * x, row = c / CH, ch = c % CH, key = j * BN + row;
      if (key < N) {
        kreg[x] = *reinterpret_cast<const uint4*>(Kh + (size_t)key * D + ch * 8);
        vreg[x] = *reinterpret_cast<const uint4*>(Vh + (size_t)key * D + ch * 8);
      } else {
        kreg[x] = make_uint4(0, 0, 0, 0);
        vreg[x] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < PER; ++x) {
      const int c = tid + 256 * x, row = c / CH, ch = c % CH;
      *reinterpret_cast<uint4*>(&lds[buf][0][tile_off<D>(row, ch)]) = kreg[x];
      *reinterpret_cast<uint4*>(&lds[buf][1][tile_off<D>(row, ch)]) = vreg[x];
    }
  };

  // Per-lane source address pieces of the transposing V read.
  const int tr_src = lane & 15, tr_r = tr_src >> 2, tr_c = tr_src & 3;
  const int tr_n0 = 16 * ((lane >> 4) & 1);

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int j = 0; j < n_tiles; ++j) {
    const int buf = j & 1;
    if (j + 1 < n_tiles) gload(j + 1);
    const int key0 = j * BN;
    const bool active = !CAUSAL || key0 <= q0 + 31;
    if (active) {
      const uint16_t* Kt = lds[buf][0];
      const uint16_t* Vt = lds[buf][1];
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
        const int krow = 32 * b + r32;
#pragma unroll
        for (int t = 0; t < D / 16; ++t)
          s[b] = mfma_bf16(lds_read_b128(Kt + tile_off<D>(krow, 2 * t + g)), qf[t], s[b]);
      }
      const bool need_mask = (key0 + BN > N) || (CAUSAL && key0 + BN - 1 > q0);
      if (need_mask) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int key = key0 + 32 * b + 8 * (i >> 2) + 4 * g + (i & 3);
            if (key >= N || (CAUSAL && key > qrow)) s[b][i] = -INFINITY;
          }
      }
      float mx = s[0][0];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[b][i]);
      mx = halves_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast((m_run - m_new) * scale_log2);
      const float mneg = -m_new * scale_log2;
      // The row sum is taken over the float32 probabilities (so LSE carries
      // no bf16 rounding); P rounded to bf16 feeds the P V product.
      float rs = 0.f;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[b][i] = exp2_fast(fmaf(s[b][i], scale_log2, mneg));
          rs += s[b][i];
        }
      l_run = l_run * alpha + rs;
      m_run = m_new;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;

      bf16x8 pf[2][2];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int h = 0; h < 2; ++h) pf[b][h] = to_bf16x8(s[b], 8 * h);

#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int d = 32 * cb + tr_n0 + 4 * tr_c;
        const int ch = d >> 3, sub = d & 7;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int kr0 = 32 * b + 16 * h + 4 * g + tr_r;
            const int kr1 = kr0 + 8;
            const bf16x4 lo = lds_read_tr16(Vt + tile_off<D>(kr0, ch) + sub);
            const bf16x4 hi = lds_read_tr16(Vt + tile_off<D>(kr1, ch) + sub);
            acc[cb] = mfma_bf16(concat(lo, hi), pf[b][h], acc[cb]);
          }
      }
    }
    if (j + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_run);
  const float inv = 1.f / l_tot;
  if (qrow < N) {
    uint16_t* Orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * inv);
        *reinterpret_cast<bf16x4*>(Orow + 32 * cb + 8 * q4 + 4 * g) = v;
      }
    if (g == 0) LSE[(size_t)bh * N + qrow] = m_run * scale + __logf(l_tot);
  }
}

template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + 127) / 128);
  const uint32_t total = (uint32_t)(a.BH * n_qblk);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qblk, total, a.scale, a.scale * kLog2e);
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_fwd_bf16_t<64, true>(a) : launch_fwd_bf16_t<64, false>(a);
  return a.causal ? launch_fwd_bf16_t<128, true>(a) : launch_fwd_bf16_t<128, false>(a);
}

}  // namespace fa

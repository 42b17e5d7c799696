// Forward attention with OCP float8 e4m3fn Q, K, V and one scale per tensor,
// float32 accumulation, bfloat16 output, gfx950 MFMA (32x32x64 f8f6f4).
//
// What it computes: the same exact attention as the bf16 forward
// ("FlashAttention-1: eliminating IO", sections 10.2.1-10.2.3) on the real
// values decode(code) * descale of the inputs.  The explainer's V3 section
// describes the FP8 variant: FP8 matrix inputs, FP32 accumulation and scaling
// factors to keep values in range.  Here:
//  * S^T = K Q^T runs on fp8 codes; the descales q_descale * k_descale and
//    scale * log2(e) fold into the one FMA in front of v_exp_f32.
//  * P is formed already multiplied by 2^8 (the factor is folded into the
//    exponent, exp2(x + 8)) and rounded to e4m3fn for the P V product; 2^8
//    keeps the probabilities that matter in the format's normal range.  The
//    row sum l is kept, in the same units, from the float32 values, so the
//    factor cancels in O = acc / l; only the LSE removes it.
//  * Lazy rescale as in the bf16 forward, with the headroom the format
//    allows: the reference max moves only when a score exceeds it by enough
//    that 2^8 P could pass 448 (the largest e4m3fn value).
//  * V^T, the A operand of O^T = V^T P^T, needs 32 keys of one head dim per
//    lane; there is no byte-transposing LDS read in use here, so V is staged
//    to LDS already transposed: each thread loads a 4 keys x 4 bytes block
//    with dword loads, transposes it with v_perm_b32 and stores 4 dwords,
//    placing keys in the order the probabilities sit in the accumulator.
// Work split, pipeline and XCD mapping are those of the bf16 forward.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {
// 16-byte-chunk XOR swizzle for LDS tiles with RB-byte rows (RB in 64/128/256).
template <int RB>
__device__ __forceinline__ int off8(int row, int byte) {
  constexpr int RP = 256 / RB;      // rows per 256 bytes
  constexpr int CM = RB / 16 - 1;   // chunk mask
  const int s = (row / RP) & CM;
  return row * RB + ((((byte >> 4) ^ s)) << 4) + (byte & 15);
}

__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}
}  // namespace

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    uint16_t* __restrict__ O, float* __restrict__ LSE, int N, uint32_t n_qblk, uint32_t total,
    float c_score, float lse_scale, float out_scale, float grow_thr) {
  constexpr int BM = 128, BN = 64;
  constexpr int KCH = D / 16;                 // 16-byte chunks per K row
  constexpr int KPER = BN * KCH / 256;        // K chunks per thread
  constexpr int VBLK = (BN / 4) * (D / 4);    // 4x4-byte V blocks per tile
  constexpr int VPER = VBLK / 256;
  __shared__ __attribute__((aligned(16))) uint8_t ks[2][BN * D];  // K tile, [key][d]
  __shared__ __attribute__((aligned(16))) uint8_t vt[2][D * BN];  // V^T tile, [d][key slot]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 5, r32 = lane & 31;
  uint32_t bh, qblk;
  map_block(blockIdx.x, n_qblk, total, CAUSAL, bh, qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* Kh = K + head;
  const uint8_t* Vh = V + head;
  const int q0 = (int)qblk * BM + wave * 32;
  const int qrow = q0 + r32;

  // Q as the B operand: lane holds Q[qrow][64t + 32g .. +31].
  i32x8 qf[D / 64];
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    if (qrow < N) {
      const i32x4* p = reinterpret_cast<const i32x4*>(Q + head + (size_t)qrow * D + 64 * t + 32 * g);
      const i32x4 a = p[0], b = p[1];
      qf[t] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
    } else {
      qf[t] = i32x8{};
    }
  }

  const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  uint4 kreg[KPER];
  uint32_t vreg[VPER][4];
  auto gload = [&](int j) {
#pragma unroll
    for (int x = 0; x < KPER; ++x) {
      const int c = tid + 256 * x, row = c / KCH, ch = c % KCH, key = j * BN + row;
      kreg[x] = key < N ? *reinterpret_cast<const uint4*>(Kh + (size_t)key * D + ch * 16)
                        : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int y = 0; y < VPER; ++y) {
      const int x = tid + 256 * y, k4 = x / (D / 4), d4 = x % (D / 4);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = j * BN + 4 * k4 + r;
        vreg[y][r] = key < N ? *reinterpret_cast<const uint32_t*>(Vh + (size_t)key * D + 4 * d4) : 0u;
      }
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int x = 0; x < KPER; ++x) {
      const int c = tid + 256 * x, row = c / KCH, ch = c % KCH;
      *reinterpret_cast<uint4*>(&ks[buf][off8<D>(row, ch * 16)]) = kreg[x];
    }
#pragma unroll
    for (int y = 0; y < VPER; ++y) {
      const int x = tid + 256 * y, k4 = x / (D / 4), d4 = x % (D / 4);
      // 4x4 byte transpose: u[c] = (V[k+0][c], V[k+1][c], V[k+2][c], V[k+3][c])
      const uint32_t t0 = __builtin_amdgcn_perm(vreg[y][1], vreg[y][0], 0x05010400u);
      const uint32_t t1 = __builtin_amdgcn_perm(vreg[y][1], vreg[y][0], 0x07030602u);
      const uint32_t t2 = __builtin_amdgcn_perm(vreg[y][3], vreg[y][2], 0x05010400u);
      const uint32_t t3 = __builtin_amdgcn_perm(vreg[y][3], vreg[y][2], 0x07030602u);
      uint32_t u[4];
      u[0] = __builtin_amdgcn_perm(t2, t0, 0x05040100u);
      u[1] = __builtin_amdgcn_perm(t2, t0, 0x07060302u);
      u[2] = __builtin_amdgcn_perm(t3, t1, 0x05040100u);
      u[3] = __builtin_amdgcn_perm(t3, t1, 0x07060302u);
      // key 4*k4 of the tile sits in accumulator block b = key/32, row
      // 8*(i/4) + 4*gg with i%4 = 0; its slot in the B operand is 32*gg + 16*b + i.
      const int key = 4 * k4, w = key & 31;
      const int pos = 32 * ((w >> 2) & 1) + 16 * (key >> 5) + 4 * (w >> 3);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        *reinterpret_cast<uint32_t*>(&vt[buf][off8<BN>(4 * d4 + c, pos)]) = u[c];
    }
  };

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
      f32x16 s[2];
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        s[b] = f32x16{};
        const int krow = 32 * b + r32;
#pragma unroll
        for (int t = 0; t < D / 64; ++t) {
          const i32x4 lo = *reinterpret_cast<const i32x4*>(&ks[buf][off8<D>(krow, 64 * t + 32 * g)]);
          const i32x4 hi = *reinterpret_cast<const i32x4*>(&ks[buf][off8<D>(krow, 64 * t + 32 * g + 16)]);
          s[b] = mfma_fp8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), qf[t], s[b]);
        }
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
      float ma = fmaxf(s[0][0], s[1][0]), mb = fmaxf(s[0][1], s[1][1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        ma = fmaxf(ma, fmaxf(s[0][i], s[1][i]));
        mb = fmaxf(mb, fmaxf(s[0][i + 1], s[1][i + 1]));
      }
      const float mx = halves_max(fmaxf(ma, mb));
      if (__builtin_amdgcn_ballot_w64(mx > m_run + grow_thr) != 0) {  // rare
        const float m_new = fmaxf(m_run, mx);
        const float alpha = exp2_fast((m_run - m_new) * c_score);
        l_run *= alpha;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
        m_run = m_new;
      }
      const float mneg = 8.f - m_run * c_score;  // 2^8 P = exp2(S c - m c + 8)
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          s[b][i] = exp2_fast(fmaf(s[b][i], c_score, mneg));
          rs[2 * b + (i & 1)] += s[b][i];
        }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);

      i32x8 pf;
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int w = 0; w < 4; ++w)
          pf[4 * b + w] = (int)pack4_fp8(s[b][4 * w], s[b][4 * w + 1], s[b][4 * w + 2], s[b][4 * w + 3]);
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
        const int drow = 32 * cb + r32;
        const i32x4 lo = *reinterpret_cast<const i32x4*>(&vt[buf][off8<BN>(drow, 32 * g)]);
        const i32x4 hi = *reinterpret_cast<const i32x4*>(&vt[buf][off8<BN>(drow, 32 * g + 16)]);
        acc[cb] = mfma_fp8(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), pf, acc[cb]);
      }
    }
    if (j + 1 < n_tiles) lstore(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = halves_sum(l_run);
  const float f = out_scale / l_tot;
  if (qrow < N) {
    uint16_t* Orow = O + head + (size_t)qrow * D;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * f);
        *reinterpret_cast<bf16x4*>(Orow + 32 * cb + 8 * q4 + 4 * g) = v;
      }
    if (g == 0) LSE[(size_t)bh * N + qrow] = m_run * lse_scale + __logf(l_tot) - 8.f * kLn2;
  }
}

template <int D, bool CAUSAL>
static hipError_t fwd_fp8_t(const FwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + 127) / 128);
  const uint32_t total = (uint32_t)(a.BH * n_qblk);
  const float sdq = a.scale * a.q_descale * a.k_descale;
  // 2^8 P <= 448 while P <= 2^(log2(448) - 8): the reference max may lag the
  // true max by about that much (in log2 units) before a rescale is needed;
  // log2(440 / 256) leaves room for the rounding of v_exp_f32.
  const float headroom_log2 = 0.7814085f;  // log2(440 / 256)
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qblk, total, sdq * kLog2e, sdq,
                     a.v_descale, headroom_log2 / (sdq * kLog2e));
  return hipGetLastError();
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? fwd_fp8_t<64, true>(a) : fwd_fp8_t<64, false>(a);
  return a.causal ? fwd_fp8_t<128, true>(a) : fwd_fp8_t<128, false>(a);
}

}  // namespace fa

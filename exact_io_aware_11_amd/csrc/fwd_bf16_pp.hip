// Forward attention, bfloat16, head size 128, no bias: the ping-pong schedule.
//
// Same computation as fwd_bf16.hip ("FlashAttention-1: eliminating IO",
// sections 10.2.1-10.2.3): one pass over the key tiles with a running max, a
// running sum and an unnormalised accumulator (lazy rescale against the row
// max of every tile), one division at the end.
//
// What differs is the schedule.  The reading notes' three-generation table
// credits FA3 with ping-pong scheduling (one group's softmax overlapping
// another group's matrix products), and the explainer's V3 section with warp
// specialisation (loading and computing overlapped).  Transplanted to gfx950:
//  * One workgroup of 8 waves per (b, h, 256-row block; causal: two blocks
//    u and n-1-u); waves w and w + 4 share a SIMD and form groups 0 and 1.
//  * Every wave runs S_0, SOFT_0, GEMM_0, SOFT_1, GEMM_1, ... with SOFT_t the
//    mask, row max, exp, row sum and bf16 packing of tile t and GEMM_t the
//    products S_{t+1} = K_{t+1} Q^T and O^T += V_t^T P_t^T, one item per
//    barrier-separated phase, group 1 one phase behind group 0.  In every
//    phase one wave of a SIMD issues matrix products, at raised issue
//    priority (s_setprio), while the other works on the vector ALUs.
//  * Loading needs no wave of its own: the direct buffer -> LDS loads are
//    asynchronous and hold no registers, so each wave issues its share of
//    the next tiles at the start of a phase and only the barrier two phases
//    later waits for them.  (A dedicated producer wave would cost a full
//    wave's registers: every wave of a workgroup gets the same allocation.)
// The default schedule (fwd_bf16.hip) weaves the softmax of one tile into
// the products of the next inside every wave instead; this one is selected
// with FA_FWD_SCHEDULE=pingpong.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <bool CAUSAL>
__global__ __launch_bounds__(512, 1) void fwd_bf16_pp_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    uint32_t n_qblk, uint32_t total, float scale, float scale_log2, float grow_thr) {
  constexpr int D = 128, WAVES = 8, BM = 32 * WAVES, BN = 64, TILE = BN * D;
  constexpr int LPW = TILE * 2 / 1024 / WAVES;  // 1 KiB direct loads per wave per tile
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[TILE];
  auto ktile = [&](auto bufc) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lk0;
    else return lk1;
  };
  auto vtile = [&](auto bufc) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lv0;
    else return lv1;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int g = lane >> 5, r32 = lane & 31;
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;
  uint32_t bh, unit;
  map_block(blockIdx.x, n_units, total, kOrderPlain, bh, unit);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  int koff[D / 16];
#pragma unroll
  for (int t = 0; t < D / 16; ++t) koff[t] = tile_off<D>(r32, 2 * t + g);
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_n0 = 16 * ((lane >> 4) & 1);
  int voff[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const int d = 32 * cb + tr_n0 + 4 * tr_c;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) voff[cb][hf] = tile_off<D>(4 * g + tr_r + 8 * hf, d >> 3) + (d & 7);
  }
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    ldoff[x] = (uint32_t)(row * 2 * D + ((((byte % (2 * D)) >> 4) ^ swz<D>(row)) << 4));
  }
  auto stage = [&](const uint16_t* src, uint16_t* dst, int key0) __attribute__((always_inline)) {
    const auto r = make_tile_rsrc<2 * D>(src + (size_t)key0 * D, N - key0);
#pragma unroll
    for (int x = 0; x < LPW; ++x) load_lds16(r, dst + (wave * LPW + x) * 512, ldoff[x]);
  };
  // Phase 2t: K_{t+1} into K buffer (t+1)%2, V_t into V buffer t%2.
  auto loads_even = [&](auto tpar, int t) __attribute__((always_inline)) {
    if constexpr (decltype(tpar)::value == 0) {
      stage(Kh, lk1, (t + 1) * BN);
      stage(Vh, lv0, t * BN);
    } else {
      stage(Kh, lk0, (t + 1) * BN);
      stage(Vh, lv1, t * BN);
    }
  };

  auto body = [&](const uint32_t qblk) __attribute__((always_inline)) {
    const int q0 = (int)qblk * BM + wave * 32;
    const int qrow = q0 + r32;
    bf16x8 qf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      if (qrow < N) qf[t] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow * D + 16 * t + 8 * g);
      else qf[t] = bf16x8{};
    }
    const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
    const int n_tiles = (kv_end + BN - 1) / BN;
    const int j_full = min(CAUSAL ? (int)qblk * (BM / BN) : n_tiles, N / BN);

    f32x16 acc[D / 32];
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
    float m_run = -INFINITY, l_run = 0.f;
    f32x16 sc0, sc1;
    bf16x8 pk[4];

    auto rescale = [&](float mx) __attribute__((always_inline)) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2_fast((m_run - m_new) * scale_log2);
      l_run *= alpha;
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
      m_run = m_new;
    };
    auto soft = [&](int t) __attribute__((always_inline)) {
      if (t >= j_full) {
        const int key0 = t * BN;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 8 * (i >> 2) + 4 * g + (i & 3);
          if (key >= kv_end || (CAUSAL && key > qrow)) sc0[i] = -INFINITY;
          if (key + 32 >= kv_end || (CAUSAL && key + 32 > qrow)) sc1[i] = -INFINITY;
        }
      }
      float ma = fmaxf(sc0[0], sc1[0]), mb = fmaxf(sc0[1], sc1[1]);
#pragma unroll
      for (int i = 2; i < 16; i += 2) {
        ma = fmaxf(ma, fmaxf(sc0[i], sc1[i]));
        mb = fmaxf(mb, fmaxf(sc0[i + 1], sc1[i + 1]));
      }
      const float mx = halves_max(fmaxf(ma, mb));
      if (__builtin_amdgcn_ballot_w64(mx > m_run + grow_thr) != 0) rescale(mx);
      const float mneg = -m_run * scale_log2;
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        sc0[i] = exp2_fast(fmaf(sc0[i], scale_log2, mneg));
        sc1[i] = exp2_fast(fmaf(sc1[i], scale_log2, mneg));
        rs[i & 1] += sc0[i];
        rs[2 + (i & 1)] += sc1[i];
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
      pk[0] = to_bf16x8(sc0, 0);
      pk[1] = to_bf16x8(sc0, 8);
      pk[2] = to_bf16x8(sc1, 0);
      pk[3] = to_bf16x8(sc1, 8);
    };
    constexpr int DEPTH = 4, NS = 2 * (D / 16), NCB = D / 32;
    auto gemm = [&](auto kbufc, auto vbufc, auto has_pv) __attribute__((always_inline)) {
      constexpr int NOPS = NS + (decltype(has_pv)::value ? 4 * NCB : 0);
      const uint16_t* Kt = ktile(kbufc);
      const uint16_t* Vt = vtile(vbufc);
      auto fetch = [&](int k) __attribute__((always_inline)) -> bf16x8 {
        if (k < NS) return lds_read_b128(Kt + 32 * D * (k & 1) + koff[k >> 1]);
        const int kc = (k - NS) / NCB, cb = (k - NS) % NCB;
        return concat(lds_read_tr16(Vt + voff[cb][0] + 16 * D * kc),
                      lds_read_tr16(Vt + voff[cb][1] + 16 * D * kc));
      };
      __builtin_amdgcn_s_setprio(1);  // products first; the partner wave does vector work
      bf16x8 ring[DEPTH + 1];
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) ring[k] = fetch(k);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NOPS; ++k) {
        if (k + DEPTH < NOPS) ring[(k + DEPTH) % (DEPTH + 1)] = fetch(k + DEPTH);
        const bf16x8 a = ring[k % (DEPTH + 1)];
        if (k < NS) {
          const int t = k >> 1;
          if (k & 1) sc1 = mfma_bf16(a, qf[t], t == 0 ? f32x16{} : sc1);
          else sc0 = mfma_bf16(a, qf[t], t == 0 ? f32x16{} : sc0);
        } else {
          const int kc = (k - NS) / NCB, cb = (k - NS) % NCB;
          acc[cb] = mfma_bf16(a, pk[kc], acc[cb]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };

    // Phases in blocks of four.  Block u: group 0 runs GEMM_{2u-1}, SOFT_{2u},
    // GEMM_{2u}, SOFT_{2u+1}; group 1 runs SOFT_{2u-1}, GEMM_{2u-1}, SOFT_{2u},
    // GEMM_{2u}.  Block 0's GEMM_{-1} is S_0 alone and its SOFT_{-1} is empty.
    // The tile count is padded to even and one block is added so that both
    // groups finish GEMM_{n_tiles-1}; the items past it see only masked tiles.
    using PV = std::true_type;
    using NOPV = std::false_type;
    stage(Kh, lk0, 0);
    barrier_vm<0>();
    const int U = ((n_tiles + 1) & ~1) / 2 + 1;
    if (group == 0) {
      loads_even(B0{}, 0);
      gemm(B0{}, B1{}, NOPV{});  // S_0
      barrier_vm<2 * LPW>();
      soft(0);
      barrier_vm<0>();
      loads_even(B1{}, 1);
      gemm(B1{}, B0{}, PV{});  // GEMM_0
      barrier_vm<2 * LPW>();
      soft(1);
      barrier_vm<0>();
      for (int u = 1; u < U; ++u) {
        loads_even(B0{}, 2 * u);
        gemm(B0{}, B1{}, PV{});  // GEMM_{2u-1}
        barrier_vm<2 * LPW>();
        soft(2 * u);
        barrier_vm<0>();
        loads_even(B1{}, 2 * u + 1);
        gemm(B1{}, B0{}, PV{});  // GEMM_{2u}
        barrier_vm<2 * LPW>();
        soft(2 * u + 1);
        barrier_vm<0>();
      }
    } else {
      loads_even(B0{}, 0);
      barrier_vm<2 * LPW>();
      gemm(B0{}, B1{}, NOPV{});  // S_0
      barrier_vm<0>();
      loads_even(B1{}, 1);
      soft(0);
      barrier_vm<2 * LPW>();
      gemm(B1{}, B0{}, PV{});  // GEMM_0
      barrier_vm<0>();
      for (int u = 1; u < U; ++u) {
        loads_even(B0{}, 2 * u);
        soft(2 * u - 1);
        barrier_vm<2 * LPW>();
        gemm(B0{}, B1{}, PV{});  // GEMM_{2u-1}
        barrier_vm<0>();
        loads_even(B1{}, 2 * u + 1);
        soft(2 * u);
        barrier_vm<2 * LPW>();
        gemm(B1{}, B0{}, PV{});  // GEMM_{2u}
        barrier_vm<0>();
      }
    }
    wait_vm<0>();
    barrier_vm<0>();  // every wave is done with the tiles before the next block restages them

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
  };
  if constexpr (CAUSAL) {
    const uint32_t partner = n_qblk - 1 - unit;
    body(partner);
    if (partner != unit) body(unit);
  } else {
    body(unit);
  }
}

template <bool CAUSAL>
static hipError_t launch_pp_t(const FwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + 255) / 256);
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;
  const uint32_t total = (uint32_t)(a.BH * n_units);
  hipLaunchKernelGGL((fwd_bf16_pp_kernel<CAUSAL>), dim3(total), dim3(512), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qblk, total, a.scale, a.scale * kLog2e,
                     kRescaleLog2 / (a.scale * kLog2e));
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_pp(const FwdArgs& a) {
  return a.causal ? launch_pp_t<true>(a) : launch_pp_t<false>(a);
}

}  // namespace fa

// Backward attention, bfloat16 inputs and gradients, float32 accumulation,
// gfx950 MFMA.
//
// What it computes ("FlashAttention-1: eliminating IO", section 10.2.4): the
// probabilities are recomputed tile by tile from the saved log-sum-exp,
// P = exp(scale Q K^T - LSE), never stored; with delta_i = dO_i . O_i,
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - delta),
//   dK = scale dS^T Q,  dQ = scale dS K.
//
// Two kernels on one stream, dQ first, no atomics:
//  * dK/dV: one workgroup per (batch, head, block of 128 keys); each wave
//    holds 32 keys' K and V rows in registers and scans the query tiles of 64
//    rows that can see them (all, or those at or after the keys when causal).
//    S = Q K^T and dP = dO V^T come out with one key per lane column; P and
//    dS are then fed, converted to bf16, straight back as the B operand of
//    dV^T = dO^T P and dK^T = Q^T dS, whose A operands (dO^T, Q^T) are read
//    from the row-major LDS tiles with ds_read_b64_tr_b16.
//  * dQ: one workgroup per (batch, head, block of 128 queries); each wave
//    holds 32 queries' Q and dO rows in registers and scans the key tiles.
//    S^T = K Q^T and dP^T = V dO^T give one query per lane column (so LSE and
//    delta are per-lane scalars); dS^T feeds dQ^T = K^T dS^T with K^T read by
//    the transposing LDS read.  It forms delta from its rows of O and dO and
//    stores it for the dK/dV kernel, so no separate delta pass is needed.
// Recomputing S and dP in the dQ pass costs two extra matrix products over
// the five the method needs; it keeps every output written exactly once.
//
// Optional additive bias (explainer V2 section: mask and bias merged into the
// score stage): P = exp(scale S + bias - LSE); each tile's bias values are
// loaded during the previous tile (in the dQ pass they then become, as
// bias / scale, the starting value of the S^T accumulators); rows whose LSE
// is -inf (no finite score in the forward) get P = 0.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(256, 1) void bwd_dkdv_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const float* __restrict__ LSE, const float* __restrict__ Delta, uint16_t* __restrict__ dK,
    uint16_t* __restrict__ dV, int N, uint32_t n_kblk, uint32_t total, float scale,
    float scale_log2, Bias bias) {
  constexpr int BN = 128, BM = 64, TILE = BM * D;
  constexpr int LPW = TILE * 2 / 1024 / 4;  // 1 KiB direct loads per wave per tile
  constexpr int NT = D / 16, NCB = D / 32;
  // Q and dO tiles, two buffers each.  Four separate arrays, not one indexed
  // array: the compiler tells LDS variables apart, so reading one buffer
  // does not wait for the direct loads still filling the other.
  __shared__ __attribute__((aligned(1024))) uint16_t lq0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lq1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lo0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lo1[TILE];
  __shared__ __attribute__((aligned(16))) float lst[2][2][BM];      // [buffer][LSE*log2e, delta]

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  uint32_t bh, kblk;
  if (BIAS && bias.grouped) map_block_grouped(blockIdx.x, n_kblk, total, bias.grouped, false, bh, kblk);
  else map_block(blockIdx.x, n_kblk, total, CAUSAL ? kOrderHeavyFirst : kOrderPlain, bh, kblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* dOh = dO + head;
  const float* LSEh = LSE + (size_t)bh * N;
  const float* Dh = Delta + (size_t)bh * N;

  const int k0 = (int)kblk * BN + wave * 32;
  const int kcol = k0 + r32;  // this lane's key (C-layout column)

  // Additive bias: element i of query half qb of a tile at qbase is
  // (row qbase + 32 qb + 8 (i / 4) + 4 g + i % 4, key kcol); the lane part of
  // the byte offset is fixed, the row part wave-uniform (scalar offset).
  // Reads past the slice return zeros; key columns past N are never written.
  [[maybe_unused]] const auto brs = BIAS ? bias_rsrc(bias, bh) : make_rsrc(nullptr, 0);
  [[maybe_unused]] const uint32_t bvoff =
      BIAS ? (uint32_t)(((long long)min(kcol, N - 1) + 4LL * g * bias.sq) * 4) : 0u;
  [[maybe_unused]] float bsv[2][2][16];  // [buffer][query half][element]
  auto load_bias = [&](auto bufc, int qb, int i, int qbase) {
    constexpr int BB = decltype(bufc)::value;
    const uint32_t row = (uint32_t)(qbase + 32 * qb + 8 * (i >> 2) + (i & 3));
    bsv[BB][qb][i] = buffer_load_f32(brs, bvoff, (uint32_t)(row * bias.sq * 4));
  };

  // K and V rows as the B operands of S = Q K^T and dP = dO V^T.
  bf16x8 kf[NT], vf[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (kcol < N) {
      kf[t] = *reinterpret_cast<const bf16x8*>(K + head + (size_t)kcol * D + 16 * t + 8 * g);
      vf[t] = *reinterpret_cast<const bf16x8*>(V + head + (size_t)kcol * D + 16 * t + 8 * g);
    } else {
      kf[t] = bf16x8{};
      vf[t] = bf16x8{};
    }
  }

  // Per-lane LDS element offsets (the swizzle depends only on row % 16).
  int aoff[NT];  // Q / dO rows as A operands: row r32 (+32 qb), chunk 2t + g
#pragma unroll
  for (int t = 0; t < NT; ++t) aoff[t] = tile_off<D>(r32, 2 * t + g);
  // Q^T / dO^T by the transposing read: row 4g + r (+8) (+16h +32qb), head dim
  // 32cb + 16((lane/16)%2) + 4c for source lane (r, c) = ((lane%16)/4, lane%4).
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_n0 = 16 * ((lane >> 4) & 1);
  int toff[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int d = 32 * cb + tr_n0 + 4 * tr_c;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) toff[cb][hf] = tile_off<D>(4 * g + tr_r + 8 * hf, d >> 3) + (d & 7);
  }
  // Direct HBM -> LDS staging of Q and dO tiles (see the forward kernel):
  // fixed per-lane byte offsets into a buffer resource per tile.
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    ldoff[x] = (uint32_t)(row * 2 * D + ((((byte % (2 * D)) >> 4) ^ swz<D>(row)) << 4));
  }
  const int n_it = (N + BM - 1) / BM;
  const int it0 = CAUSAL ? ((int)kblk * BN) / BM : 0;
  // The resource of a tile ends at the head's end: rows past N arrive as
  // zeros, whose probabilities the +inf LSE below turns into exact zeros.  A
  // tile index past the end is harmless, so the last step stages
  // unconditionally.  Load L (0 .. 2 LPW - 1) of this wave's share: piece
  // L / 2 of Q (L even) or of dO (L odd).
  auto qtile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lq0;
    else return lq1;
  };
  auto otile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lo0;
    else return lo1;
  };
  auto tile_rsrc = [&](const uint16_t* src, int row0) {
    return make_tile_rsrc<2 * D>(src + (size_t)row0 * D, N - row0);
  };
  auto stage_one = [&](const __amdgpu_buffer_rsrc_t& qr, const __amdgpu_buffer_rsrc_t& orr,
                       auto bufc, int L) {
    const int x = L >> 1;
    if (L & 1) load_lds16(orr, otile(bufc) + (wave * LPW + x) * 512, ldoff[x]);
    else load_lds16(qr, qtile(bufc) + (wave * LPW + x) * 512, ldoff[x]);
  };
  auto stage = [&](int it, auto bufc) {
    const auto qr = tile_rsrc(Qh, it * BM);
    const auto orr = tile_rsrc(dOh, it * BM);
#pragma unroll
    for (int L = 0; L < 2 * LPW; ++L) stage_one(qr, orr, bufc, L);
  };
  // Threads 0..127 carry one LSE (0..63) or delta (64..127) of the next tile
  // in a register; it is used (scaled, stored to LDS) only at the end of the
  // current tile, so the load's latency hides behind the whole tile.
  float sreg = 0.f;
  const float* stat_src = wave == 0 ? LSEh : Dh;  // wave-uniform: stays in scalar registers
  auto load_stats = [&](int it) {
    const int q = it * BM + (tid & (BM - 1));
    if (tid < 2 * BM && q < N) sreg = stat_src[q];
  };
  // Query rows past N get LSE = +inf and delta = 0, so their P and dS are
  // exactly zero and no bounds test is needed on the query side.  Key columns
  // past N (K, V rows zero) only reach dK/dV columns that are never written.
  // delta is stored negated: it is the starting value of the dP accumulators,
  // which then hold dP - delta with no vector op.
  auto store_stats = [&](int it, int buf) {
    const int q = it * BM + (tid & (BM - 1));
    // (with a bias, an LSE of -inf -- a row with no finite score -- becomes
    // +inf too: its P is 0)
    const bool live = q < N && (!BIAS || sreg != -__builtin_inff());
    if (tid < 2 * BM)
      lst[buf][tid / BM][tid & (BM - 1)] =
          tid < BM ? (live ? sreg * kLog2e : __builtin_inff()) : (q < N ? -sreg : 0.f);
  };

  f32x16 adk[NCB], adv[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    adk[cb] = f32x16{};
    adv[cb] = f32x16{};
  }

  // One 32-query half qb of a 64-query tile:
  //  G_A(qb): S = Q_qb K^T and dP = dO_qb V^T (2 NT products, A from LDS rows)
  //  SOFT(qb): P = exp2(S log2e scale - LSE log2e), dS = P (dP - delta)
  //  G_B(qb): dV^T += dO_qb^T P and dK^T += Q_qb^T dS (4 NCB products, A by
  //           the transposing read, B = P / dS straight from the C layout)
  // Per tile: G_A(0); [G_A(1) | SOFT(0)]; [G_B(0) | SOFT(1)]; G_B(1), with
  // the softmax arithmetic of one half interleaved, element by element, into
  // the other half's products, and every operand fetched from LDS several
  // products ahead (sched_barrier keeps that order).
  f32x16 s[2], dp[2];
  bf16x8 pb[2][2], db[2][2];

  // Causal masking (key > query -> P = 0) is compiled only into the variant
  // used for the two query tiles that can straddle this block's diagonal.
  auto tile = [&](auto bufc, auto maskc, int it) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool masked = CAUSAL && decltype(maskc)::value;
    const uint16_t* Qt = qtile(bufc);
    const uint16_t* Ot = otile(bufc);
    const int qbase = it * BM;
    constexpr int NA = 2 * NT, NB = 4 * NCB, DEPTH = 4;
    // LSE*log2e and -delta of the 16 rows a lane sees in half qb, read once
    // (-delta in C-layout order, as the starting value of dP)
    f32x4 l2v[4];
    f32x16 ndl_init;
    // operand fetches
    auto fetch_a = [&](int qb, int k) -> bf16x8 {  // k-th product of G_A(qb)
      const uint16_t* base = (k & 1) ? Ot : Qt;
      return lds_read_b128(base + 32 * qb * D + aoff[k >> 1]);
    };
    auto fetch_b = [&](int qb, int k) -> bf16x8 {  // k-th product of G_B(qb)
      const int h = k / (2 * NCB), cb = (k >> 1) % NCB;
      const uint16_t* base = ((k & 1) ? Qt : Ot) + (32 * qb + 16 * h) * D;
      return concat(lds_read_tr16(base + toff[cb][0]), lds_read_tr16(base + toff[cb][1]));
    };
    auto op_a = [&](int qb, int k, const bf16x8& a) {
      if (k < 2) {
        if (k == 0) s[qb] = mfma_bf16(a, kf[0], f32x16{});
        else dp[qb] = mfma_bf16(a, vf[0], ndl_init);
      } else if (k & 1) {
        dp[qb] = mfma_bf16(a, vf[k >> 1], dp[qb]);
      } else {
        s[qb] = mfma_bf16(a, kf[k >> 1], s[qb]);
      }
    };
    auto op_b = [&](int qb, int k, const bf16x8& a) {
      const int h = k / (2 * NCB), cb = (k >> 1) % NCB;
      if (k & 1) adk[cb] = mfma_bf16(a, db[qb][h], adk[cb]);
      else adv[cb] = mfma_bf16(a, pb[qb][h], adv[cb]);
    };
    auto load_half_lse = [&](int qb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        l2v[q4] = *reinterpret_cast<const f32x4*>(&lst[BUF][0][32 * qb + 8 * q4 + 4 * g]);
    };
    auto load_half_ndelta = [&](int qb) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&lst[BUF][1][32 * qb + 8 * q4 + 4 * g]);
#pragma unroll
        for (int e = 0; e < 4; ++e) ndl_init[4 * q4 + e] = v[e];
      }
    };
    // softmax-backward arithmetic of element i (0..15) of half qb
    auto soft_elem = [&](int qb, int i) {
      const float l2 = l2v[i >> 2][i & 3];
      float arg = -l2;
      if constexpr (BIAS) arg = fmaf(bsv[BUF][qb][i], kLog2e, arg);
      float p = exp2_fast(fmaf(s[qb][i], scale_log2, arg));
      if constexpr (masked) {  // row of element i: qbase + 32 qb + 4 g + 8 (i / 4) + i % 4
        if (kcol - (qbase + 32 * qb + 4 * g) > 8 * (i >> 2) + (i & 3)) p = 0.f;
      }
      s[qb][i] = p;
      dp[qb][i] = p * dp[qb][i];  // dP - delta from the accumulator
      if ((i & 7) == 7) {
        pb[qb][i >> 3] = to_bf16x8(s[qb], i - 7);
        db[qb][i >> 3] = to_bf16x8(dp[qb], i - 7);
      }
    };
    // A fenced stream of NOPS products of group (kind, qb) with operands
    // fetched DEPTH ahead; `extra(k)` is softmax work woven in after product k.
    auto stream = [&](bool kind_b, int qb, int nops, auto extra) {
      bf16x8 ring[DEPTH + 1];
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) ring[k] = kind_b ? fetch_b(qb, k) : fetch_a(qb, k);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < nops; ++k) {
        if (k + DEPTH < nops)
          ring[(k + DEPTH) % (DEPTH + 1)] = kind_b ? fetch_b(qb, k + DEPTH) : fetch_a(qb, k + DEPTH);
        if (kind_b) op_b(qb, k, ring[k % (DEPTH + 1)]);
        else op_a(qb, k, ring[k % (DEPTH + 1)]);
        extra(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    auto none = [](int) {};
    // This wave's share of the next tile is issued one load every SEV
    // products over the first three streams: the CU moves only about 64 B
    // per clock from L2 into LDS, and a burst would stall the issuing waves.
    constexpr int SEV = (2 * NA + NB) / (2 * LPW);
    const auto qr = tile_rsrc(Qh, (it + 1) * BM);
    const auto orr = tile_rsrc(dOh, (it + 1) * BM);
    auto stage_at = [&](int op) {
      if (op % SEV == 0) stage_one(qr, orr, std::integral_constant<int, BUF ^ 1>{}, op / SEV);
    };
    load_half_lse(0);
    load_half_ndelta(0);
    stream(false, 0, NA, [&](int k) { stage_at(k); });
    load_half_ndelta(1);
    // the 16 softmax elements of a half are spread evenly over a stream
    stream(false, 1, NA, [&](int k) {
#pragma unroll
      for (int i = k * 16 / NA; i < (k + 1) * 16 / NA; ++i) soft_elem(0, i);
      stage_at(NA + k);
    });
    load_half_lse(1);
    stream(true, 0, NB, [&](int k) {
#pragma unroll
      for (int i = k * 16 / NB; i < (k + 1) * 16 / NB; ++i) soft_elem(1, i);
      stage_at(2 * NA + k);
    });
    if constexpr (BIAS) {  // the next tile's bias, two or four loads per product
      stream(true, 1, NB, [&](int k) {
#pragma unroll
        for (int e = k * 32 / NB; e < (k + 1) * 32 / NB; ++e)
          load_bias(std::integral_constant<int, BUF ^ 1>{}, e >> 4, e & 15, qbase + BM);
      });
    } else {
      stream(true, 1, NB, none);
    }
  };

  // Two-stage pipeline over query tiles: tile it+1 streams into the other
  // buffer while tile it is processed; one barrier per tile.  The barrier
  // waits only for this wave's loads of the tile about to be used.
  // Every wave runs every tile of its block: in the causal prologue a wave
  // whose keys all follow the tile's queries gets an all-zero P (a branch
  // around it costs more registers than the one idle tile saves).
  auto step = [&](auto bufc, auto maskc, int it) {
    constexpr int BUF = decltype(bufc)::value;
    barrier_vm<0>();  // tile `it` (loads of the previous step) visible to all
    load_stats(it + 1);
    tile(bufc, maskc, it);
    store_stats(it + 1, BUF ^ 1);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  stage(it0, B0{});
  load_stats(it0);
  store_stats(it0, 0);
  if constexpr (BIAS) {
#pragma unroll
    for (int e = 0; e < 32; ++e) load_bias(B0{}, e >> 4, e & 15, it0 * BM);
  }
  int it = it0;
  if (CAUSAL) {  // tiles it0 and it0 + 1 hold every (key > query) pair of the block
    // (it0 + 1 may lie past the end: its rows are all masked by the +inf LSE)
    step(B0{}, std::true_type{}, it);
    step(B1{}, std::true_type{}, it + 1);
    it += 2;
  }
  for (; it < n_it; it += 2) {
    step(B0{}, std::false_type{}, it);
    if (it + 1 < n_it) step(B1{}, std::false_type{}, it + 1);
  }
  wait_vm<0>();  // the last (unused) staging lands before the workgroup's LDS is released

  if (kcol < N) {
    uint16_t* dKrow = dK + head + (size_t)kcol * D;
    uint16_t* dVrow = dV + head + (size_t)kcol * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (__bf16)(adk[cb][4 * q4 + e] * scale);
          b[e] = (__bf16)adv[cb][4 * q4 + e];
        }
        *reinterpret_cast<bf16x4*>(dKrow + 32 * cb + 8 * q4 + 4 * g) = a;
        *reinterpret_cast<bf16x4*>(dVrow + 32 * cb + 8 * q4 + 4 * g) = b;
      }
  }
}

template <int D, bool CAUSAL, bool BIAS>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
    const uint16_t* __restrict__ O, const float* __restrict__ LSE, float* __restrict__ Delta,
    uint16_t* __restrict__ dQ, int N, uint32_t n_qblk, uint32_t total, float scale,
    float scale_log2, Bias bias) {
  constexpr int BM = 128, BN = 64, TILE = BN * D;
  constexpr int LPW = TILE * 2 / 1024 / 4;  // 1 KiB direct loads per wave per tile and tensor
  constexpr int NT = D / 16, NCB = D / 32;
  // K and V tiles, two buffers each, as four separate arrays (reading one
  // buffer must not wait for the direct loads filling the other).
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[TILE];
  auto ktile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lk0;
    else return lk1;
  };
  auto vtile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lv0;
    else return lv1;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  uint32_t bh, qblk;
  if (BIAS && bias.grouped) map_block_grouped(blockIdx.x, n_qblk, total, bias.grouped, CAUSAL, bh, qblk);
  else map_block(blockIdx.x, n_qblk, total, CAUSAL ? kOrderHeavyLast : kOrderPlain, bh, qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;

  const int q0 = (int)qblk * BM + wave * 32;
  const int qrow = q0 + r32;  // this lane's query (C-layout column)

  // Q and dO rows as the B operands of S^T = K Q^T and dP^T = V dO^T.
  bf16x8 qf[NT], of[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (qrow < N) {
      qf[t] = *reinterpret_cast<const bf16x8*>(Q + head + (size_t)qrow * D + 16 * t + 8 * g);
      of[t] = *reinterpret_cast<const bf16x8*>(dO + head + (size_t)qrow * D + 16 * t + 8 * g);
    } else {
      qf[t] = bf16x8{};
      of[t] = bf16x8{};
    }
  }
  // One query per lane column: LSE and delta are per-lane scalars.  (With a
  // bias, rows past N and rows with LSE = -inf -- no finite score -- take
  // +inf, so that their P is exactly 0 whatever the bias there.)
  float lse2 = qrow < N ? LSE[(size_t)bh * N + qrow] * kLog2e : 0.f;
  if constexpr (BIAS) lse2 = (qrow < N && lse2 != -__builtin_inff()) ? lse2 : __builtin_inff();
  // delta_i = sum_c dO_ic O_ic (FA1 page, section 10.2.4): the lane holds
  // head dims 16t + 8g .. +7 of its query's dO row; it reads the same part of
  // O, and the wave's two halves add their partial sums.  Stored for the
  // dK/dV pass, which runs after this one.
  float del;
  {
    float part = 0.f;
    if (qrow < N) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 o8 = *reinterpret_cast<const bf16x8*>(O + head + (size_t)qrow * D + 16 * t + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) part = fmaf((float)o8[e], (float)of[t][e], part);
      }
    }
    del = halves_sum(part);
    if (qrow < N && g == 0) Delta[(size_t)bh * N + qrow] = del;
  }
  // Additive bias of this lane's query row: as in the forward, element i of
  // key half b of a tile at key0 is key key0 + 32 b + 8 (i / 4) + 4 g + i % 4,
  // load x = 4 b + i / 4 of 16 bytes, component i % 4.  A tile's bias is
  // loaded during the previous tile's last product stream and, as bias /
  // scale, becomes the starting value of the S^T accumulators, so it is not
  // held while the softmax backward runs.
  [[maybe_unused]] const auto brs = BIAS ? bias_rsrc(bias, bh) : make_rsrc(nullptr, 0);
  [[maybe_unused]] const uint32_t bvoff =
      BIAS ? (uint32_t)((long long)min(qrow, N - 1) * bias.sq * 4 + 16 * g) : 0u;
  [[maybe_unused]] const float inv_scale = 1.f / scale;
  [[maybe_unused]] f32x4 bv[8];
  auto load_bias = [&](int x, int key0) {
    bv[x] = buffer_load_f32x4(brs, bvoff + 128 * (x >> 2) + 32 * (x & 3), (uint32_t)key0 * 4u);
  };

  // K / V rows as A operands: row r32 (+32 b), chunk 2t + g.
  int koff[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) koff[t] = tile_off<D>(r32, 2 * t + g);
  // K^T by the transposing read (as V in the forward): source lane
  // (r, c) = ((lane%16)/4, lane%4) reads key row 4g + r (+8) at head dim
  // 32cb + 16((lane/16)%2) + 4c.
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_n0 = 16 * ((lane >> 4) & 1);
  int toff[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    const int d = 32 * cb + tr_n0 + 4 * tr_c;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) toff[cb][hf] = tile_off<D>(4 * g + tr_r + 8 * hf, d >> 3) + (d & 7);
  }
  // Direct loads of K and V tiles through buffer resources that end at the
  // head's end (rows past N arrive as zeros: their K rows add nothing to dQ).
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    ldoff[x] = (uint32_t)(row * 2 * D + ((((byte % (2 * D)) >> 4) ^ swz<D>(row)) << 4));
  }
  auto tile_rsrc = [&](const uint16_t* src, int key0) {
    return make_tile_rsrc<2 * D>(src + (size_t)key0 * D, N - key0);
  };
  // Load L (0 .. 2 LPW - 1): piece L / 2 of K (L even) or of V (L odd).
  auto stage_one = [&](const __amdgpu_buffer_rsrc_t& kr, const __amdgpu_buffer_rsrc_t& vr,
                       auto bufc, int L) {
    const int x = L >> 1;
    if (L & 1) load_lds16(vr, vtile(bufc) + (wave * LPW + x) * 512, ldoff[x]);
    else load_lds16(kr, ktile(bufc) + (wave * LPW + x) * 512, ldoff[x]);
  };

  const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;
  // Tiles [0, j_full) are visible to every query of the block.  With a bias
  // a ragged last tile is masked too: its keys past N read a bias from beyond
  // the row, which must not reach an exp.
  const int j_full = BIAS ? min(CAUSAL ? (int)qblk * (BM / BN) : n_tiles, N / BN)
                          : (CAUSAL ? (int)qblk * (BM / BN) : n_tiles);

  f32x16 adq[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) adq[cb] = f32x16{};

  // One 32-key half b of a 64-key tile:
  //  G_A(b): S^T = K_b Q^T and dP^T = V_b dO^T (2 NT products, A from LDS rows)
  //  SOFT(b): P = exp2(S log2e scale - LSE log2e), dS = P (dP - delta)
  //  G_B(b): dQ^T += K_b^T dS_b^T (2 NCB products, A by the transposing read,
  //          B = dS straight from the C layout)
  // Per tile: G_A(0); [G_A(1) | SOFT(0)]; [G_B(0) | SOFT(1)]; G_B(1), the
  // softmax arithmetic of one half woven element by element into the other
  // half's products, every operand fetched DEPTH products ahead, and the next
  // tile's loads spread over the first three streams.
  f32x16 s[2], dp[2];
  bf16x8 db[2][2];
  auto tile = [&](auto bufc, auto maskc, int j) {
    constexpr int BUF = decltype(bufc)::value;
    constexpr bool masked = (CAUSAL || BIAS) && decltype(maskc)::value;
    using BN1 = std::integral_constant<int, BUF ^ 1>;
    const uint16_t* Kt = ktile(bufc);
    const uint16_t* Vt = vtile(bufc);
    const int key0 = j * BN;
    const auto kr = tile_rsrc(Kh, key0 + BN);
    const auto vr = tile_rsrc(Vh, key0 + BN);
    // Masked tiles: the lane id formed here, once per tile, rather than a
    // row index held in a register through the whole scan (which spilled).
    [[maybe_unused]] int ln_m = 0;
    if constexpr (masked) ln_m = lane_id_here();
    constexpr int NA = 2 * NT, NB = 2 * NCB, DEPTH = 4;
    auto fetch_a = [&](int b, int k) -> bf16x8 {  // k-th product of G_A(b)
      const uint16_t* base = ((k & 1) ? Vt : Kt) + 32 * D * b;
      return lds_read_b128(base + koff[k >> 1]);
    };
    auto fetch_b = [&](int b, int k) -> bf16x8 {  // k-th product of G_B(b)
      const int h = k / NCB, cb = k % NCB;
      const uint16_t* base = Kt + (32 * b + 16 * h) * D;
      return concat(lds_read_tr16(base + toff[cb][0]), lds_read_tr16(base + toff[cb][1]));
    };
    auto op_a = [&](int b, int k, const bf16x8& a) {
      const int t = k >> 1;
      if (k & 1) dp[b] = mfma_bf16(a, of[t], t == 0 ? f32x16{} : dp[b]);
      else s[b] = mfma_bf16(a, qf[t], t == 0 && !BIAS ? f32x16{} : s[b]);
    };
    auto op_b = [&](int b, int k, const bf16x8& a) {
      const int h = k / NCB, cb = k % NCB;
      adq[cb] = mfma_bf16(a, db[b][h], adq[cb]);
    };
    auto soft_elem = [&](int b, int i) {  // key of element i: key0 + 32 b + 8 (i / 4) + 4 g + i % 4
      float p = exp2_fast(fmaf(s[b][i], scale_log2, -lse2));
      if constexpr (masked && BIAS) {
        const int key = key0 + 32 * b + 8 * (i >> 2) + 4 * (ln_m >> 5) + (i & 3);
        if ((CAUSAL && key > q0 + (ln_m & 31)) || key >= N) p = 0.f;
      } else if constexpr (masked) {  // causal only
        const int key = key0 + 32 * b + 8 * (i >> 2) + 4 * (ln_m >> 5) + (i & 3);
        if (key > q0 + (ln_m & 31)) p = 0.f;
      }
      dp[b][i] = p * (dp[b][i] - del);
      if ((i & 7) == 7) db[b][i >> 3] = to_bf16x8(dp[b], i - 7);
    };
    auto stream = [&](bool kind_b, int b, int nops, auto extra) {
      bf16x8 ring[DEPTH + 1];
#pragma unroll
      for (int k = 0; k < DEPTH; ++k) ring[k] = kind_b ? fetch_b(b, k) : fetch_a(b, k);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < nops; ++k) {
        if (k + DEPTH < nops)
          ring[(k + DEPTH) % (DEPTH + 1)] = kind_b ? fetch_b(b, k + DEPTH) : fetch_a(b, k + DEPTH);
        if (kind_b) op_b(b, k, ring[k % (DEPTH + 1)]);
        else op_a(b, k, ring[k % (DEPTH + 1)]);
        extra(k);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    constexpr int SEV = (2 * NA + NB) / (2 * LPW);  // one load every SEV products
    auto stage_at = [&](int op) {
      if (op % SEV == 0 && op / SEV < 2 * LPW) stage_one(kr, vr, BN1{}, op / SEV);
    };
    auto init_bias = [&](int b, int i) { s[b][i] = bv[4 * b + (i >> 2)][i & 3] * inv_scale; };
    if constexpr (BIAS) {  // half 0 starts from its bias now, half 1 during G_A(0)
#pragma unroll
      for (int i = 0; i < 16; ++i) init_bias(0, i);
    }
    stream(false, 0, NA, [&](int k) {
      if constexpr (BIAS) {
#pragma unroll
        for (int i = k * 16 / NA; i < (k + 1) * 16 / NA; ++i) init_bias(1, i);
      }
      stage_at(k);
    });
    stream(false, 1, NA, [&](int k) {
#pragma unroll
      for (int i = k * 16 / NA; i < (k + 1) * 16 / NA; ++i) soft_elem(0, i);
      stage_at(NA + k);
    });
    stream(true, 0, NB, [&](int k) {
#pragma unroll
      for (int i = k * 16 / NB; i < (k + 1) * 16 / NB; ++i) soft_elem(1, i);
      stage_at(2 * NA + k);
    });
    if constexpr (BIAS) {  // the next tile's bias
      stream(true, 1, NB, [&](int k) {
#pragma unroll
        for (int x = k * 8 / NB; x < (k + 1) * 8 / NB; ++x) load_bias(x, key0 + BN);
      });
    } else {
      stream(true, 1, NB, [](int) {});
    }
  };

  auto step = [&](auto bufc, auto maskc, int j) {
    barrier_vm<0>();  // tile j (this wave's loads and everyone's) is in LDS
    tile(bufc, maskc, j);
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  {
    const auto kr = tile_rsrc(Kh, 0);
    const auto vr = tile_rsrc(Vh, 0);
#pragma unroll
    for (int L = 0; L < 2 * LPW; ++L) stage_one(kr, vr, B0{}, L);
  }
  if constexpr (BIAS) {
#pragma unroll
    for (int x = 0; x < 8; ++x) load_bias(x, 0);
  }
  int j = 0;
  for (; j + 2 <= j_full; j += 2) {
    step(B0{}, std::false_type{}, j);
    step(B1{}, std::false_type{}, j + 1);
  }
  if constexpr (CAUSAL && !BIAS) {
    // This wave's tiles end at n_use, the last one holding a key at or
    // before its last query (j_full < n_use: the block's first query sees
    // every earlier key).  For the workgroup's remaining diagonal tile the
    // wave only stages its share of the next tile and meets the barrier.
    const int n_use = min(n_tiles, (q0 + 31) / BN + 1);
    for (; j + 1 < n_use; j += 2) {
      step(B0{}, std::true_type{}, j);
      step(B1{}, std::true_type{}, j + 1);
    }
    if (j < n_use) step(B0{}, std::true_type{}, j++);
    auto idle = [&](auto bufc, int jj) {
      barrier_vm<0>();
      const auto kr = tile_rsrc(Kh, (jj + 1) * BN);
      const auto vr = tile_rsrc(Vh, (jj + 1) * BN);
#pragma unroll
      for (int L = 0; L < 2 * LPW; ++L)
        stage_one(kr, vr, std::integral_constant<int, decltype(bufc)::value ^ 1>{}, L);
    };
    for (; j < n_tiles; ++j) {
      if (j & 1) idle(B1{}, j);
      else idle(B0{}, j);
    }
  } else {
    for (; j < n_tiles; j += 2) {  // the causal diagonal tiles (masking any tile is correct)
      step(B0{}, std::true_type{}, j);
      if (j + 1 < n_tiles) step(B1{}, std::true_type{}, j + 1);
    }
  }
  wait_vm<0>();  // the last (unused) loads land before the workgroup's LDS is released

  // (the row is formed again from the lane id: keeping it, or the row
  // address, live through the tile loops costs a spilled register)
  const int ln_e = lane_id_here();
  const int qrow_e = q0 + (ln_e & 31), g_e = ln_e >> 5;
  if (qrow_e < N) {
    uint16_t* dQrow = dQ + head + (size_t)qrow_e * D;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)(adq[cb][4 * q4 + e] * scale);
        *reinterpret_cast<bf16x4*>(dQrow + 32 * cb + 8 * q4 + 4 * g_e) = v;
      }
  }
}

template <int D, bool CAUSAL, bool BIAS>
static hipError_t dkdv_bf16_t(const BwdArgs& a) {
  const uint32_t n_kblk = (uint32_t)((a.N + 127) / 128);
  const uint32_t total = (uint32_t)(a.BH * n_kblk);
  Bias bias = a.bias;
  // (causal: the heavy-first order already walks several heads block-major, and
  // groups would leave the heavy key blocks of a head group to one XCD)
  bias.grouped = CAUSAL ? 0 : group_blocks(bias, a.BH, n_kblk, 4);  // one workgroup per CU: 32 per XCD
  hipLaunchKernelGGL((bwd_dkdv_bf16_kernel<D, CAUSAL, BIAS>), dim3(total), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv,
                     a.N, n_kblk, total, a.scale, a.scale * kLog2e, bias);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool BIAS>
static hipError_t dq_bf16_t(const BwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + 127) / 128);
  const uint32_t total = (uint32_t)(a.BH * n_qblk);
  Bias bias = a.bias;
  bias.grouped = CAUSAL ? 0 : group_blocks(bias, a.BH, n_qblk, 8);  // two workgroups per CU: 64 per XCD
  hipLaunchKernelGGL((bwd_dq_bf16_kernel<D, CAUSAL, BIAS>), dim3(total), dim3(256), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, (const uint16_t*)a.o, a.lse, a.delta,
                     (uint16_t*)a.dq, a.N, n_qblk, total, a.scale, a.scale * kLog2e, bias);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t dkdv_bf16_b(const BwdArgs& a) {
  return a.bias.p ? dkdv_bf16_t<D, CAUSAL, true>(a) : dkdv_bf16_t<D, CAUSAL, false>(a);
}
template <int D, bool CAUSAL>
static hipError_t dq_bf16_b(const BwdArgs& a) {
  return a.bias.p ? dq_bf16_t<D, CAUSAL, true>(a) : dq_bf16_t<D, CAUSAL, false>(a);
}

hipError_t launch_dkdv_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dkdv_bf16_b<64, true>(a) : dkdv_bf16_b<64, false>(a);
  return a.causal ? dkdv_bf16_b<128, true>(a) : dkdv_bf16_b<128, false>(a);
}

hipError_t launch_dq_bf16(const BwdArgs& a) {
  if (a.d == 64) return a.causal ? dq_bf16_b<64, true>(a) : dq_bf16_b<64, false>(a);
  return a.causal ? dq_bf16_b<128, true>(a) : dq_bf16_b<128, false>(a);
}

}  // namespace fa

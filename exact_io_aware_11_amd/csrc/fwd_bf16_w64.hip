// Forward attention, bfloat16, head size 128, no bias: 64 query rows per wave
// (selected with FA_FWD_SCHEDULE=rows64; the default is fwd_bf16.hip).
//
// Same computation as fwd_bf16.hip ("FlashAttention-1: eliminating IO",
// sections 10.2.1-10.2.3; explainer V2 section; reading notes code 3-1): one
// pass over the key tiles with a running max, a running sum and an
// unnormalised accumulator, one division at the end; scores and
// probabilities live only in registers.
//
// What differs is the shape of the work, chosen for the gfx950 cost model:
//  * Each wave owns 64 query rows -- two 32-row blocks -- so every K and V
//    operand read from LDS feeds two matrix products instead of one: 0.75
//    LDS instructions (0.5 KiB) per product instead of 1.5 (1 KiB).  The
//    accumulators of 64 rows x 128 head dims take 128 registers more, so the
//    kernel runs one wave per SIMD (four waves, 256 rows, per CU) with the
//    whole register file: accumulators, scores and Q in VGPRs (the products
//    in their VGPR form), the compiler's overflow in AGPRs.  A single
//    wave issues independent matrix products as fast as two (measured);
//    the vector work between them has no second wave to hide behind.
//  * Key tiles of 32 keys.  With the CU to itself the workgroup has LDS to
//    spare, so K and V go through a four-slot ring and every tile is staged
//    two steps before it is used (a tile's direct HBM -> LDS loads are
//    issued two steps ahead), which hides the load latency the two-slot
//    kernel exposed.
//  * Per step: one fenced stream of 32 matrix products, S_{j+1} = K_{j+1} Q^T
//    for both row blocks (each K operand once), then O^T += V_j^T P_j^T for
//    both (each V^T operand once); the exp, row sum and bf16 packing of P_j
//    and, when needed, the mask (and on the SAFE path the row max) of
//    S_{j+1} ride between the products, with this wave's share of the loads.
//  * FAST / SAFE reference max.  FAST takes the row max on the block's first
//    tile only and keeps it: later probabilities exp(S - m) may exceed 1 by
//    any amount float32 holds, which changes no relative precision, and they
//    need no max, no rescale and no exchange between lanes.  A block whose
//    row sum ends past 2^64 or not finite, or whose accumulator is not
//    finite (P V left the float range), is recomputed on the SAFE path,
//    which takes the row max of every tile before forming its probabilities
//    (lazy rescale, as in fwd_bf16.hip).
//  * Causal: a workgroup takes row blocks u and n-1-u.  Every wave runs all
//    of the block's tiles (the diagonal ones past its rows give P = 0), so
//    that the step loops hold no branches.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {
constexpr int kD = 128, kBM = 256, kBN = 32, kTile = kBN * kD;  // kTile: elements of a K or V tile
constexpr int kLPW = kTile * 2 / 1024 / 4;  // 1 KiB direct loads per wave per tile and tensor (2)
constexpr int kLead = 2;                    // steps a tile is staged ahead of its use
constexpr int kLoadsPerStep = 2 * kLPW;     // this wave's loads issued per step (K, then V)
}  // namespace

template <bool CAUSAL>
__global__ __launch_bounds__(256, 1) void fwd_w64_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    uint32_t n_qblk, uint32_t total, float scale, float scale_log2, float grow_thr) {
  constexpr int D = kD, BM = kBM, BN = kBN, TILE = kTile, LPW = kLPW;
  // The K and V rings, four slots each, as eight separate arrays (reads of
  // one slot must not wait for the direct loads still filling another).
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk3[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv2[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv3[TILE];
  __shared__ int redo[2];
  auto ktile = [&](auto slotc) -> uint16_t* {
    constexpr int S = decltype(slotc)::value & 3;
    if constexpr (S == 0) return lk0;
    else if constexpr (S == 1) return lk1;
    else if constexpr (S == 2) return lk2;
    else return lk3;
  };
  auto vtile = [&](auto slotc) -> uint16_t* {
    constexpr int S = decltype(slotc)::value & 3;
    if constexpr (S == 0) return lv0;
    else if constexpr (S == 1) return lv1;
    else if constexpr (S == 2) return lv2;
    else return lv3;
  };
  using std::integral_constant;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 2) redo[tid] = 0;
  const int g = lane >> 5, r32 = lane & 31;
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;
  uint32_t bh, unit;
  map_block(blockIdx.x, n_units, total, kOrderPlain, bh, unit);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint16_t* Qh = Q + head;
  const uint16_t* Kh = K + head;
  const uint16_t* Vh = V + head;
  const float inv_scale_log2 = 1.f / scale_log2;

  // Per-lane element offsets inside a tile buffer.  K as the A operand of
  // S^T = K Q^T: row r32, chunk 2t + g.  V^T by the transposing read, in the
  // key order the S^T accumulator leaves P in: source lane (r, c) =
  // ((lane % 16) / 4, lane % 4) reads row 4g + r (+8 for the chunk's second
  // read, +16 kc for chunk kc) at head dim 32 cb + 16 ((lane / 16) % 2) + 4c.
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
  // Direct HBM -> LDS staging: load x of this wave fills bytes
  // [(wave * LPW + x) * 1024, +1024) of a tile buffer; each lane fetches the
  // logical 16-byte chunk that the swizzle places at its 16 bytes.
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    ldoff[x] = (uint32_t)(row * 2 * D + ((((byte % (2 * D)) >> 4) ^ swz<D>(row)) << 4));
  }
  auto tile_rsrc = [&](const uint16_t* src, int key0) __attribute__((always_inline)) {
    return make_tile_rsrc<2 * D>(src + (size_t)key0 * D, N - key0);
  };
  // This wave's share of K tile jk and V tile jv into their ring slots (K
  // first, then V: the order the barrier counts on).
  auto stage_kv = [&](auto kslot, int jk, auto vslot, int jv) __attribute__((always_inline)) {
    const auto kr = tile_rsrc(Kh, jk * BN);
    const auto vr = tile_rsrc(Vh, jv * BN);
#pragma unroll
    for (int x = 0; x < LPW; ++x) load_lds16(kr, ktile(kslot) + (wave * LPW + x) * 512, ldoff[x]);
#pragma unroll
    for (int x = 0; x < LPW; ++x) load_lds16(vr, vtile(vslot) + (wave * LPW + x) * 512, ldoff[x]);
  };

  auto body = [&](const uint32_t qblk, auto fastc) __attribute__((always_inline)) -> bool {
    constexpr bool FAST = decltype(fastc)::value;
    bool bad = false;
    const int q0 = (int)qblk * BM + wave * 64;  // first of this wave's 64 rows
    int qrow[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) qrow[s] = q0 + 32 * s + r32;

    // Q fragments (B operand of S^T): lane holds Q[qrow[s]][16 t + 8 g .. +7].
    bf16x8 qf[2][D / 16];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int t = 0; t < D / 16; ++t) {
        if (qrow[s] < N)
          qf[s][t] = *reinterpret_cast<const bf16x8*>(Qh + (size_t)qrow[s] * D + 16 * t + 8 * g);
        else
          qf[s][t] = bf16x8{};
      }

    const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
    const int n_tiles = (kv_end + BN - 1) / BN;
    // tiles [0, j_full) need no mask for any row of the block
    const int j_full = min(CAUSAL ? (int)qblk * (BM / BN) : n_tiles, N / BN);

    f32x16 acc[2][D / 32];
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) acc[s][cb] = f32x16{};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};

    // Rescale row block s to a new reference max (SAFE path; rare).
    auto rescale = [&](int s, float mx) __attribute__((always_inline)) {
      const float m_new = fmaxf(m_run[s], mx);
      const float alpha = exp2_fast((m_run[s] - m_new) * scale_log2);
      l_run[s] *= alpha;
      // one 16-register block at a time (keeps the temporaries few)
#pragma unroll
      for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[s][cb][i] *= alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
      m_run[s] = m_new;
    };
    // Lazy rescale against the row max of a tile's scores (see fwd_bf16.hip):
    // the reference moves only when a score exceeds it by grow_thr.
    auto guard = [&](int s, float mx) __attribute__((always_inline)) {
      mx = halves_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > m_run[s] + grow_thr) != 0) rescale(s, mx);
    };
    auto rowmax_guard = [&](const f32x16 (&sv)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float mx = sv[s][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) mx = fmaxf(mx, sv[s][i]);
        guard(s, mx);
      }
    };
    // Masked scores: keys past N, and under the causal mask keys after the query.
    // Element i of row block s of a tile at key0 is key key0 + 8 (i / 4) + 4 g + i % 4.
    auto mask_elem = [&](f32x16 (&sv)[2], int key0, int s, int i) __attribute__((always_inline)) {
      const int key = key0 + 8 * (i >> 2) + 4 * g + (i & 3);
      if (key >= N || (CAUSAL && key > qrow[s])) sv[s][i] = -INFINITY;
    };

    f32x16 sa[2], sb[2];  // scores of even (a) and odd (b) tiles, by row block
    auto sc_of = [&](auto parity) __attribute__((always_inline)) -> f32x16 (&)[2] {
      if constexpr (decltype(parity)::value == 0) return sa;
      else return sb;
    };
    using S0 = integral_constant<int, 0>;

    // Prologue: K_0 (scores of tile 0), then V_0, K_1, V_1, ..., K_kLead.
    stage_kv(S0{}, 0, S0{}, 0);
    stage_kv(integral_constant<int, 1>{}, 1, integral_constant<int, 1>{}, 1);
#pragma unroll
    for (int x = 0; x < LPW; ++x)
      load_lds16(tile_rsrc(Kh, 2 * BN), lk2 + (wave * LPW + x) * 512, ldoff[x]);
    // K_0 landed for everyone: its loads are followed by V_0, K_1, V_1, K_2
    static_assert(kLead == 2, "the prologue stages K_0 .. K_2 and V_0, V_1");
    barrier_vm<4 * LPW>();
#pragma unroll
    for (int s = 0; s < 2; ++s) sa[s] = mfma_bf16(lds_read_b128(lk0 + koff[0]), qf[s][0], f32x16{});
#pragma unroll
    for (int t = 1; t < D / 16; ++t) {
      const bf16x8 a = lds_read_b128(lk0 + koff[t]);
#pragma unroll
      for (int s = 0; s < 2; ++s) sa[s] = mfma_bf16(a, qf[s][t], sa[s]);
    }
    if (j_full == 0) {
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int i = 0; i < 16; ++i) mask_elem(sa, 0, s, i);
    }
    rowmax_guard(sa);

    // Step j (this wave has tile j + 1 too): barrier (K_{j+1} and V_j landed),
    // then one fenced stream of 32 products: S_{j+1} (16: K operand t feeds
    // row blocks 0 and 1) then O^T += V_j^T P_j^T (16: V^T operand (kc, cb)
    // feeds row blocks 0 and 1), operands fetched DEPTH operands ahead.  The
    // stores of P_j's three phases per element (scaled score, exp, row sum
    // and bf16 packing) ride on products 0 .. EXP_OPS+1 -- every 16-key chunk
    // is packed before its first product -- and the mask (SAFE: and row max)
    // of S_{j+1} on the last MAX_OPS products, after the S results are in.
    // This wave's loads of K_{j+1+kLead} and V_{j+kLead} go on the first ones.
    constexpr int NOPS = 32, NOPD = 16, DEPTH = 2, EXP_OPS = 22, MAX_OPS = 12;
    // element n of P_j in processing order: chunk 0 of blocks 0 and 1, then chunk 1
    auto elem_s = [](int n) { return (n >> 3) & 1; };
    auto elem_i = [](int n) { return (n & 7) + 8 * (n >> 4); };
    static_assert((15 * EXP_OPS) / 32 + 2 < 16, "chunk 0 packed before its first product");
    static_assert((31 * EXP_OPS) / 32 + 2 < 24, "chunk 1 packed before its first product");
    auto step = [&](auto slotc, auto maskc, int j) __attribute__((always_inline)) {
      constexpr int SL = decltype(slotc)::value;  // j % 4
      constexpr bool MASK_NEXT = decltype(maskc)::value;  // tile j + 1 needs the mask
      using PC = integral_constant<int, SL & 1>;
      using PN = integral_constant<int, (SL + 1) & 1>;
      f32x16(&sc)[2] = sc_of(PC{});
      f32x16(&sn)[2] = sc_of(PN{});
      barrier_vm<kLoadsPerStep * (kLead - 1)>();
      const uint16_t* Kt = ktile(integral_constant<int, SL + 1>{});
      const uint16_t* Vt = vtile(integral_constant<int, SL>{});
      float mneg[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) mneg[s] = -m_run[s] * scale_log2;
      const int key1 = (j + 1) * BN;
      const auto kres = tile_rsrc(Kh, (j + 1 + kLead) * BN);
      const auto vres = tile_rsrc(Vh, (j + kLead) * BN);
      uint16_t* Kdst = ktile(integral_constant<int, SL + 1 + kLead>{});
      uint16_t* Vdst = vtile(integral_constant<int, SL + kLead>{});
      bf16x8 pk[2][2];  // P_j in bf16: [row block][16-key chunk]
      auto fetch = [&](int o) __attribute__((always_inline)) -> bf16x8 {
        if (o < 8) return lds_read_b128(Kt + koff[o]);
        const int kc = (o - 8) >> 2, cb = (o - 8) & 3;
        return concat(lds_read_tr16(Vt + voff[cb][0] + 16 * D * kc),
                      lds_read_tr16(Vt + voff[cb][1] + 16 * D * kc));
      };
      auto op = [&](int k, const bf16x8& a) __attribute__((always_inline)) {
        const int s = k & 1;
        if (k < NOPD) {
          const int t = k >> 1;
          sn[s] = mfma_bf16(a, qf[s][t], t == 0 ? f32x16{} : sn[s]);
        } else {
          const int o = (k - NOPD) >> 1, kc = o >> 2, cb = o & 3;
          acc[s][cb] = mfma_bf16(a, pk[s][kc], acc[s][cb]);
        }
      };
      float lsum[2][2];
      auto pin = [](float& x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };
      auto phase = [&](int n, int ph) __attribute__((always_inline)) {
        const int s = elem_s(n), i = elem_i(n);
        float x = sc[s][i];
        if (ph == 0) {
          pin(x);
          x = fmaf(x, scale_log2, mneg[s]);
          pin(x);
        } else if (ph == 1) {
          x = exp2_fast(x);
          pin(x);
        } else {
          lsum[s][i & 1] = (i < 2) ? x : lsum[s][i & 1] + x;  // two partial sums per block
        }
        sc[s][i] = x;
        if (ph == 2 && (i & 7) == 7) pk[s][i >> 3] = to_bf16x8(sc[s], i - 7);
      };
      float mxp[2] = {-INFINITY, -INFINITY};
      auto extra = [&](int k) __attribute__((always_inline)) {
#pragma unroll
        for (int ph = 0; ph < 3; ++ph) {
          const int ks = k - ph;
          if (ks >= 0 && ks < EXP_OPS) {
#pragma unroll
            for (int n = ks * 32 / EXP_OPS; n < (ks + 1) * 32 / EXP_OPS; ++n) phase(n, ph);
          }
        }
        if (k >= NOPS - MAX_OPS) {  // mask (and SAFE: row max) of S_{j+1}
          const int r = k - (NOPS - MAX_OPS);
#pragma unroll
          for (int n = r * 32 / MAX_OPS; n < (r + 1) * 32 / MAX_OPS; ++n) {
            const int s = n >> 4, i = n & 15;
            if constexpr (MASK_NEXT) mask_elem(sn, key1, s, i);
            if constexpr (!FAST) {
              mxp[s] = fmaxf(mxp[s], sn[s][i]);
              pin(mxp[s]);
            }
          }
        }
        if (k % 2 == 0 && k / 2 < 2 * LPW) {  // loads: K_{j+1+kLead} pieces, then V_{j+kLead}
          const int x = (k / 2) % LPW;
          if (k / 2 >= LPW) load_lds16(vres, Vdst + (wave * LPW + x) * 512, ldoff[x]);
          else load_lds16(kres, Kdst + (wave * LPW + x) * 512, ldoff[x]);
        }
      };
      bf16x8 ring[DEPTH + 1];
#pragma unroll
      for (int o = 0; o < DEPTH; ++o) ring[o] = fetch(o);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NOPS; ++k) {
        const int o = k >> 1;
        if ((k & 1) == 0 && o + DEPTH < NOPD) ring[(o + DEPTH) % (DEPTH + 1)] = fetch(o + DEPTH);
        op(k, ring[o % (DEPTH + 1)]);
        extra(k);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) l_run[s] += lsum[s][0] + lsum[s][1];
      if constexpr (!FAST) {
#pragma unroll
        for (int s = 0; s < 2; ++s) guard(s, mxp[s]);
      }
    };
    // Every tile is a full step: the tile count is padded to a multiple of
    // four (padding tiles lie past the block's last key, so the mask makes
    // their probabilities exactly zero), and under the causal mask every wave
    // runs the block's diagonal tiles, the ones past its rows giving P = 0.
    // The last step's next-tile scores are never used.  So the loops hold no
    // branches: one over groups of four steps whose next tiles are full for
    // every row, one over the rest with the mask.
    const int n_steps = (n_tiles + 3) & ~3;
    auto group = [&](auto maskc, int j) __attribute__((always_inline)) {
      step(integral_constant<int, 0>{}, maskc, j);
      step(integral_constant<int, 1>{}, maskc, j + 1);
      step(integral_constant<int, 2>{}, maskc, j + 2);
      step(integral_constant<int, 3>{}, maskc, j + 3);
    };
    int j = 0;
    for (; j + 4 < j_full; j += 4) group(std::false_type{}, j);
    for (; j < n_steps; j += 4) group(std::true_type{}, j);
    wait_vm<0>();  // no direct load may still be landing when the block ends

#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const float l_tot = halves_sum(l_run[s]);
      // FAST: a row sum past 2^64 (or not finite), or an accumulator that
      // is not finite (P V past the float range: large values times large
      // probabilities), sends the block to the SAFE path.
      if constexpr (FAST) {
        uint32_t top = 0;  // largest |acc| bit pattern: >= 0x7f800000 means inf or NaN
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int i = 0; i < 16; ++i) top = max(top, __float_as_uint(acc[s][cb][i]) & 0x7fffffffu);
        bad = bad || !(__float_as_uint(l_tot) < 0x5f800000u) || top >= 0x7f800000u;
      }
      const float inv = 1.f / l_tot;
      if (qrow[s] < N) {
        uint16_t* Orow = O + head + (size_t)qrow[s] * D;
#pragma unroll
        for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            bf16x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[s][cb][4 * q4 + e] * inv);
            *reinterpret_cast<bf16x4*>(Orow + 32 * cb + 8 * q4 + 4 * g) = v;
            __builtin_amdgcn_sched_barrier(0);
          }
        if (g == 0) LSE[(size_t)bh * N + qrow[s]] = m_run[s] * scale + __logf(l_tot);
      }
    }
    return bad;
  };  // body

  auto run = [&](uint32_t qblk, int slot) __attribute__((always_inline)) {
    const bool bad = body(qblk, std::true_type{});
    if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) redo[slot] = 1;
    barrier_vm<0>();
    if (redo[slot] != 0) {  // uniform over the workgroup
      body(qblk, std::false_type{});
      barrier_vm<0>();
    }
  };
  if constexpr (CAUSAL) {
    const uint32_t partner = n_qblk - 1 - unit;
    run(partner, 0);  // the longer block first
    if (partner != unit) run(unit, 1);  // (uniform over the workgroup)
  } else {
    run(unit, 0);
  }
}

template <bool CAUSAL>
static hipError_t launch_w64_t(const FwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + kBM - 1) / kBM);
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;
  const uint32_t total = (uint32_t)(a.BH * n_units);
  hipLaunchKernelGGL((fwd_w64_kernel<CAUSAL>), dim3(total), dim3(256), 0, a.stream,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qblk, total, a.scale, a.scale * kLog2e,
                     kRescaleLog2 / (a.scale * kLog2e));
  return hipGetLastError();
}

hipError_t launch_fwd_bf16_w64(const FwdArgs& a) {
  return a.causal ? launch_w64_t<true>(a) : launch_w64_t<false>(a);
}

}  // namespace fa

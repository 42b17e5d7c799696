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
//  * Operand order (probe-verified for v_mfma_scale_f32_32x32x64_f8f6f4): of
//    the 64 k values of a product, bytes 0-15 of lanes l and l+32 form k
//    block 0 and bytes 16-31 form k block 1; the per-lane scale of lane l
//    (l+32) applies to block 0 (1) of its row or column.  Lane half g
//    therefore holds k = 16g + e and k = 32 + 16g + e (e < 16), so that the
//    two 32-wide blocks of a product are contiguous ranges -- the blocks that
//    microscaling formats scale.
//  * Key order: the K rows of a 32-key block are fed to the matrix core
//    permuted so that accumulator element (block b, i) of lane half g holds
//    key 32 b + 16 g + i.  A lane's 32 probabilities are then, in order, the
//    keys the P V product wants in its B operand, and V^T (the A operand)
//    comes straight from the row-major V tile by four ds_read_b64_tr_b8.
//  * Microscaled variant (MX): Q and K carry one power-of-two (e8m0) scale
//    per 32 consecutive head dims of a row, V one per 32 consecutive keys of
//    a head dim (blocks along the contraction of each product), applied by
//    the matrix core itself; the score needs no descale then.  The explainer's
//    V3 section names finer-grained scale management for FP8; per-tensor
//    scales are the coarse case.
//  * K and V tiles are staged HBM -> LDS with buffer loads (rows past N
//    arrive as zeros), double-buffered in four separate arrays, 16-byte XOR
//    swizzle; one fenced stream of matrix products per 64-key step with the
//    softmax arithmetic and the loads woven in, as in the bf16 forward.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {
typedef int i32x2 __attribute__((ext_vector_type(2)));

// 16-byte-chunk XOR swizzle of a [64 keys][D bytes] tile.  LDS serves a
// 16-byte read 16 lanes at a time and an 8-byte read 32 lanes at a time, 256
// bytes (64 four-byte banks, 256 / D tile rows) per pass.  The K reads of one
// pass cover 16 rows of the form {0..3, 4..7, 16..19, 20..23} (+8) at one
// chunk, the transposing V reads 8 consecutive rows at two adjacent chunks;
// the XOR value (bits of the row: 2, 1 and 4 at D = 128; 2 and 4 at D = 64)
// differs over the rows of a pass that share banks, so both are
// conflict-free.  It repeats every 32 rows: the second 32-key block of a
// tile reuses the first one's offsets.
template <int D>
__device__ __forceinline__ int sw8(int row) {
  if constexpr (D == 128) return (((row >> 1) & 3) << 1) | ((row >> 4) & 1);
  else return (((row >> 2) & 1) << 1) | ((row >> 4) & 1);
}
template <int D>
__device__ __forceinline__ int tile_byte(int row, int chunk) {
  return row * D + 16 * (chunk ^ sw8<D>(row));
}

// Four floats to four e4m3fn bytes.  Each conversion writes one 16-bit half of
// its destination and keeps the other; the first one is seeded with d's own
// bits (overwritten half by half), so no zero needs to be materialised.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, __float_as_int(d), true);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, w, false);
  return (uint32_t)w;
}
__device__ __forceinline__ i32x4 lds_read_i32x4(const uint8_t* p) {
  return *reinterpret_cast<const i32x4*>(p);
}
__device__ __forceinline__ i32x2 lds_read_tr8(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32(
      (__attribute__((address_space(3))) i32x2*)(const_cast<uint8_t*>(p)));
}
}  // namespace

template <int D, bool CAUSAL, bool MX>
__global__ __launch_bounds__(256, 2) void fwd_fp8_kernel(
    const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
    const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS,
    const uint8_t* __restrict__ VS, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    uint32_t n_qblk, uint32_t total, float c_score, float lse_scale, float out_scale,
    float grow_thr) {
  constexpr int BM = 128, BN = 64, TILE = BN * D;  // TILE in bytes
  constexpr int LPW = TILE / 1024 / 4;             // 1 KiB direct loads per wave per tile
  constexpr int NT = D / 64, NCB = D / 32;
  // One tile's K (or V) block scales: BN * D / 32 bytes, staged as 256.
  constexpr int SB = 256;
  __shared__ __attribute__((aligned(1024))) uint8_t lk0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lk1[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint8_t lv1[TILE];
  // Each wave's rows: its 32 Q rows come in (as whole rows, 16-byte direct
  // loads; 16-byte chunks XOR-swizzled by row / 2 at D = 128, row / 4 at
  // D = 64), and its 32 rows of O (bfloat16) go out through the same space,
  // so that both cross HBM as 16-byte accesses of consecutive addresses
  // instead of 16 (or 8) bytes from each of 32 rows per instruction.
  __shared__ __attribute__((aligned(1024))) uint8_t lrow[4 * 32 * 2 * D];
  auto ktile = [&](auto bufc) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(bufc)::value == 0) return lk0;
    else return lk1;
  };
  auto vtile = [&](auto bufc) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(bufc)::value == 0) return lv0;
    else return lv1;
  };
  // block scales of the K and V tiles (MX only), two buffers each
  __shared__ __attribute__((aligned(16))) uint8_t lks0[MX ? SB : 4];
  __shared__ __attribute__((aligned(16))) uint8_t lks1[MX ? SB : 4];
  __shared__ __attribute__((aligned(16))) uint8_t lvs0[MX ? SB : 4];
  __shared__ __attribute__((aligned(16))) uint8_t lvs1[MX ? SB : 4];
  auto kstile = [&](auto bufc) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(bufc)::value == 0) return lks0;
    else return lks1;
  };
  auto vstile = [&](auto bufc) __attribute__((always_inline)) -> uint8_t* {
    if constexpr (decltype(bufc)::value == 0) return lvs0;
    else return lvs1;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, r32 = lane & 31;
  uint32_t bh, qblk;
  map_block(blockIdx.x, n_qblk, total, CAUSAL ? kOrderHeavyLast : kOrderPlain, bh, qblk);
  const size_t head = (size_t)bh * (size_t)N * D;
  const uint8_t* Kh = K + head;
  const uint8_t* Vh = V + head;
  const int q0 = (int)qblk * BM + wave * 32;
  const int qrow = q0 + r32;

  // Q as the B operand: lane holds Q[qrow][64t + 16g .. +15] and
  // Q[qrow][64t + 32 + 16g .. +15] -- from the wave's LDS rows, read once
  // they have landed (with the first tiles, below).
  uint8_t* const lrw = lrow + wave * 32 * 2 * D;
  auto qrow_byte = [](int row, int chunk) __attribute__((always_inline)) {
    return row * D + 16 * (chunk ^ (D == 128 ? (row >> 1) & 7 : (row >> 2) & 3));
  };
  {
    const auto qres = make_tile_rsrc<D>(Q + head + (size_t)q0 * D, N - q0);
#pragma unroll
    for (int x = 0; x < D / 32; ++x) {
      const int byte = x * 1024 + 16 * lane, row = byte / D, chunk = (byte % D) >> 4;
      // (the lane fetches the logical chunk that the swizzle puts at its byte)
      const int lchunk = chunk ^ (D == 128 ? (row >> 1) & 7 : (row >> 2) & 3);
      load_lds16(qres, lrw + x * 1024, (uint32_t)(row * D + 16 * lchunk));
    }
  }
  i32x8 qf[NT];
  // MX: this row's four (D = 128) or two block scales in one word, shifted so
  // that byte 2t is the scale of this lane's k block of product t.
  uint32_t qsc = 0x7f7f7f7fu;
  if constexpr (MX) {
    if (qrow < N) {
      uint32_t w;
      w = *reinterpret_cast<const uint32_t*>(QS + ((size_t)bh * N + qrow) * 4);
      qsc = w >> (8 * g);
    }
  }
  const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // K as the A operand of block b: accumulator row rho reads tile row
  // 32b + 16((rho/4)%2) + 4(rho/8) + rho%4, so that accumulator element
  // (b, i) of lane half g is key 32b + 16g + i.  The swizzle of those rows
  // does not depend on b, so block 1 is block 0 plus 32 rows.  Head dims as
  // the k index: chunks 4t + g and 4t + 2 + g of the row.
  const int kr0 = 16 * ((r32 >> 2) & 1) + 4 * (r32 >> 3) + (r32 & 3);
  int koff[NT][2];
#pragma unroll
  for (int t = 0; t < NT; ++t)
#pragma unroll
    for (int h = 0; h < 2; ++h) koff[t][h] = tile_byte<D>(kr0, 4 * t + 2 * h + g);
  // V^T by the transposing read: in each 16-lane group q (lane / 16), source
  // lane s reads 8 bytes of tile row 16(q/2) + 8m + s/2 (+32 for m >= 2) at
  // head dim 32cb + 16(q%2) + 8(s%2); output lane j then holds head dim
  // 32cb + 16(q%2) + j of those 8 keys.  Reads m and m + 2 differ by 32 rows
  // and share the swizzle.
  const int tq = lane >> 4, ts = lane & 15;
  int voff[NCB][2];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int m = 0; m < 2; ++m)
      voff[cb][m] = tile_byte<D>(16 * (tq >> 1) + 8 * m + (ts >> 1), 2 * cb + (tq & 1)) + 8 * (ts & 1);
  // Direct HBM -> LDS staging (see the bf16 forward): fixed per-lane byte
  // offsets into a buffer resource per tile that ends at the head's end.
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / D;
    ldoff[x] = (uint32_t)(row * D + 16 * (((byte % D) >> 4) ^ sw8<D>(row)));
  }
  auto tile_rsrc = [&](const uint8_t* src, int key0) __attribute__((always_inline)) {
    return make_tile_rsrc<D>(src + (size_t)key0 * D, N - key0);
  };
  auto stage = [&](const uint8_t* src, uint8_t* dst, int key0) __attribute__((always_inline)) {
    const auto r = tile_rsrc(src, key0);
#pragma unroll
    for (int x = 0; x < LPW; ++x) load_lds16(r, dst + (wave * LPW + x) * 1024, ldoff[x]);
  };
  // MX block scales of a tile: K scales (one 4-byte word per key, bytes
  // 0 .. D/32-1 used) of its 64 keys and V scales [key block][D] of its two
  // 32-key blocks, staged by waves 0 (K, 256 bytes) and 1 (V, 2 D bytes).  A
  // tile past the end arrives as zeros (unused).
  const int nkb = (N + 31) / 32;
  auto kscale_rsrc = [&](int key0) __attribute__((always_inline)) {
    return make_tile_rsrc<4>(KS + ((size_t)bh * N + key0) * 4, N - key0);
  };
  auto vscale_rsrc = [&](int key0) __attribute__((always_inline)) {
    return make_tile_rsrc<D>(VS + ((size_t)bh * nkb + key0 / 32) * D, nkb - key0 / 32);
  };
  auto stage_kscale = [&](uint8_t* dst, int key0) __attribute__((always_inline)) {
    if constexpr (MX) {
      if (wave == 0) load_lds4(kscale_rsrc(key0), dst, 4 * lane);
    }
  };
  auto stage_vscale = [&](uint8_t* dst, int key0) __attribute__((always_inline)) {
    if constexpr (MX) {
      if (wave == 1) load_lds4(vscale_rsrc(key0), dst, 4 * lane);
    }
  };
  // Scale word of K row kr (tile-local), shifted so byte 2t is this lane's
  // k block of product t; V scale byte of head dim 32cb + r32, key block g.
  auto kscale_of = [&](const uint8_t* ks, int kr) __attribute__((always_inline)) -> uint32_t {
    if constexpr (!MX) return 0x7f7f7f7fu;
    else return *reinterpret_cast<const uint32_t*>(ks + 4 * kr) >> (8 * g);
  };
  auto vscale_of = [&](const uint8_t* vs, int cb) __attribute__((always_inline)) -> uint32_t {
    if constexpr (!MX) return 0x7fu;
    else return (uint32_t)vs[g * D + 32 * cb + r32];
  };

  f32x16 acc[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;

  auto fetch_k = [&](const uint8_t* Kt, int b, int t) __attribute__((always_inline)) -> i32x8 {
    const uint8_t* base = Kt + 32 * D * b;
    const i32x4 lo = lds_read_i32x4(base + koff[t][0]);
    const i32x4 hi = lds_read_i32x4(base + koff[t][1]);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto fetch_v = [&](const uint8_t* Vt, int cb) __attribute__((always_inline)) -> i32x8 {
    const i32x2 a = lds_read_tr8(Vt + voff[cb][0]);
    const i32x2 b = lds_read_tr8(Vt + voff[cb][1]);
    const i32x2 c = lds_read_tr8(Vt + voff[cb][0] + 32 * D);
    const i32x2 d = lds_read_tr8(Vt + voff[cb][1] + 32 * D);
    const i32x4 ab = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    const i32x4 cd = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(ab, cd, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  // S^T product t of block b (scales: byte 2t of the K and Q words).
  auto smfma = [&](int t, const i32x8& a, const f32x16& c, uint32_t ks) __attribute__((always_inline)) {
    if (t == 0) return mfma_fp8_scaled<0, 0>(a, qf[0], c, ks, qsc);
    return mfma_fp8_scaled<2, 2>(a, qf[NT - 1], c, ks, qsc);
  };
  auto scores = [&](const uint8_t* Kt, const uint8_t* ks, f32x16& s0, f32x16& s1) __attribute__((always_inline)) {
    const uint32_t ks0 = kscale_of(ks, kr0), ks1 = kscale_of(ks, kr0 + 32);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      s0 = smfma(t, fetch_k(Kt, 0, t), t == 0 ? f32x16{} : s0, ks0);
      s1 = smfma(t, fetch_k(Kt, 1, t), t == 0 ? f32x16{} : s1, ks1);
    }
  };
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2_fast((m_run - m_new) * c_score);
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
    m_run = m_new;
  };
  auto guard = [&](float mx) __attribute__((always_inline)) {
    mx = halves_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + grow_thr) != 0) rescale(mx);  // rare
  };
  // Key of accumulator element (b, i): key0 + 32 b + 16 g + i.
  auto apply_mask = [&](f32x16& s0, f32x16& s1, int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int key = key0 + 16 * g + i;
      if (key >= N || (CAUSAL && key > qrow)) s0[i] = -INFINITY;
      if (key + 32 >= N || (CAUSAL && key + 32 > qrow)) s1[i] = -INFINITY;
    }
  };
  auto rowmax_guard = [&](const f32x16& s0, const f32x16& s1) __attribute__((always_inline)) {
    float ma = fmaxf(s0[0], s1[0]), mb = fmaxf(s0[1], s1[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) {
      ma = fmaxf(ma, fmaxf(s0[i], s1[i]));
      mb = fmaxf(mb, fmaxf(s0[i + 1], s1[i + 1]));
    }
    guard(fmaxf(ma, mb));
  };

  const int j_full = min(CAUSAL ? (int)qblk * (BM / BN) : n_tiles, N / BN);
  f32x16 sa0, sa1, sb0, sb1;
  auto sc_lo = [&](auto parity) __attribute__((always_inline)) -> f32x16& {
    if constexpr (decltype(parity)::value == 0) return sa0;
    else return sb0;
  };
  auto sc_hi = [&](auto parity) __attribute__((always_inline)) -> f32x16& {
    if constexpr (decltype(parity)::value == 0) return sa1;
    else return sb1;
  };
  stage(Kh, lk0, 0);
  stage(Vh, lv0, 0);
  stage_kscale(lks0, 0);
  stage_vscale(lvs0, 0);
  barrier_vm<0>();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const i32x4 a = lds_read_i32x4(lrw + qrow_byte(r32, 4 * t + g));
    const i32x4 b = lds_read_i32x4(lrw + qrow_byte(r32, 4 * t + 2 + g));
    qf[t] = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
  }
  stage(Kh, lk1, BN);
  stage_kscale(lks1, BN);
  scores(lk0, lks0, sa0, sa1);
  if (j_full == 0) apply_mask(sa0, sa1, 0);
  rowmax_guard(sa0, sa1);

  // Step j < n_tiles - 1: one fenced stream, S_{j+1} (2 NT products) then
  // O^T += V_j^T P_j^T (NCB products), operands DEPTH products ahead.  The
  // exp / sum / fp8 packing of P_j rides on the S products (P_j is complete
  // before the first PV product), the mask and row max of S_{j+1} on the PV
  // products, and this wave's loads of K_{j+2} and V_{j+1} on the first ones.
  constexpr int DEPTH = 2, NS = 2 * NT, NOPS = NS + NCB;
  auto step = [&](auto parity, auto maskc, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    constexpr bool MASK_NEXT = decltype(maskc)::value;
    using PN = std::integral_constant<int, P ^ 1>;
    f32x16& sc0 = sc_lo(parity);
    f32x16& sc1 = sc_hi(parity);
    f32x16& sn0 = sc_lo(PN{});
    f32x16& sn1 = sc_hi(PN{});
    barrier_vm<0>();  // K_{j+1} and V_j have landed (this wave's loads and everyone's)
    const uint8_t* Kt = ktile(PN{});
    const uint8_t* Vt = vtile(parity);
    uint8_t* Kdst = ktile(parity);
    uint8_t* Vdst = vtile(PN{});
    const auto kres = tile_rsrc(Kh, (j + 2) * BN);
    const auto vres = tile_rsrc(Vh, (j + 1) * BN);
    const uint32_t ks0 = kscale_of(kstile(PN{}), kr0), ks1 = kscale_of(kstile(PN{}), kr0 + 32);
    uint32_t vsc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) vsc[cb] = vscale_of(vstile(parity), cb);
    const float mneg = 8.f - m_run * c_score;  // 2^8 P = exp2(S c - m c + 8)
    const int key1 = (j + 1) * BN;
    i32x8 pf;
    float lsum[2] = {0.f, 0.f};
    float mxp[2] = {-INFINITY, -INFINITY};
    auto fetch = [&](int k) __attribute__((always_inline)) -> i32x8 {
      if (k < NS) return fetch_k(Kt, k & 1, k >> 1);
      return fetch_v(Vt, k - NS);
    };
    auto op = [&](int k, const i32x8& a) __attribute__((always_inline)) {
      if (k < NS) {
        const int t = k >> 1;
        if (k & 1) sn1 = smfma(t, a, t == 0 ? f32x16{} : sn1, ks1);
        else sn0 = smfma(t, a, t == 0 ? f32x16{} : sn0, ks0);
      } else {
        acc[k - NS] = mfma_fp8_scaled<0, 0>(a, pf, acc[k - NS], vsc[k - NS], 0x7fu);
      }
    };
    // element e of P_j: block e / 16, index e % 16
    auto exp_elem = [&](int e) __attribute__((always_inline)) {
      const int i = e & 15;
      float x;
      if (e < 16) {
        x = exp2_fast(fmaf(sc0[i], c_score, mneg));
        sc0[i] = x;
      } else {
        x = exp2_fast(fmaf(sc1[i], c_score, mneg));
        sc1[i] = x;
      }
      lsum[e & 1] += x;
      if ((e & 3) == 3) {
        const f32x16& sv = e < 16 ? sc0 : sc1;
        pf[e >> 2] = (int)pack4_fp8(sv[i - 3], sv[i - 2], sv[i - 1], sv[i]);
      }
    };
    auto mask_next = [&](int i) __attribute__((always_inline)) {
      const int key = key1 + 16 * g + i;
      if (key >= N || (CAUSAL && key > qrow)) sn0[i] = -INFINITY;
      if (key + 32 >= N || (CAUSAL && key + 32 > qrow)) sn1[i] = -INFINITY;
    };
    auto extra = [&](int k) __attribute__((always_inline)) {
      if (k < NS) {
#pragma unroll
        for (int e = k * 32 / NS; e < (k + 1) * 32 / NS; ++e) exp_elem(e);
      } else {
        const int r = k - NS;
#pragma unroll
        for (int i = r * 16 / NCB; i < (r + 1) * 16 / NCB; ++i) {
          if constexpr (MASK_NEXT) mask_next(i);
          mxp[i & 1] = fmaxf(mxp[i & 1], fmaxf(sn0[i], sn1[i]));
          asm volatile("" : "+v"(mxp[i & 1]));  // one three-input max per element pair
        }
      }
      if (k < 2 * LPW) {  // loads: K_{j+2} pieces, then V_{j+1}
        const int x = k % LPW;
        if (k >= LPW) load_lds16(vres, Vdst + (wave * LPW + x) * 1024, ldoff[x]);
        else load_lds16(kres, Kdst + (wave * LPW + x) * 1024, ldoff[x]);
      }
      if (k == 0) {
        stage_kscale(kstile(parity), (j + 2) * BN);
        stage_vscale(vstile(PN{}), (j + 1) * BN);
      }
    };
    i32x8 ring[DEPTH + 1];
#pragma unroll
    for (int k = 0; k < DEPTH; ++k) ring[k] = fetch(k);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int k = 0; k < NOPS; ++k) {
      if (k + DEPTH < NOPS) ring[(k + DEPTH) % (DEPTH + 1)] = fetch(k + DEPTH);
      op(k, ring[k % (DEPTH + 1)]);
      extra(k);
      __builtin_amdgcn_sched_barrier(0);
    }
    l_run += lsum[0] + lsum[1];
    guard(fmaxf(mxp[0], mxp[1]));
  };
  // Last tile: P_j then O^T += V_j^T P_j^T.
  auto step_last = [&](auto parity) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;
    f32x16& s0 = sc_lo(parity);
    f32x16& s1 = sc_hi(parity);
    barrier_vm<0>();
    const float mneg = 8.f - m_run * c_score;
    float rs[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      s0[i] = exp2_fast(fmaf(s0[i], c_score, mneg));
      s1[i] = exp2_fast(fmaf(s1[i], c_score, mneg));
      rs[i & 1] += s0[i] + s1[i];
    }
    l_run += rs[0] + rs[1];
    i32x8 pf;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      pf[w] = (int)pack4_fp8(s0[4 * w], s0[4 * w + 1], s0[4 * w + 2], s0[4 * w + 3]);
      pf[4 + w] = (int)pack4_fp8(s1[4 * w], s1[4 * w + 1], s1[4 * w + 2], s1[4 * w + 3]);
    }
    const uint8_t* Vt = vtile(parity);
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb)
      acc[cb] = mfma_fp8_scaled<0, 0>(fetch_v(Vt, cb), pf, acc[cb], vscale_of(vstile(parity), cb), 0x7fu);
  };

  using NOMASK = std::false_type;
  using MASK = std::true_type;
  int j = 0;
  for (; j + 2 < j_full; j += 2) {
    step(B0{}, NOMASK{}, j);
    step(B1{}, NOMASK{}, j + 1);
  }
  for (; j + 2 < n_tiles; j += 2) {
    step(B0{}, MASK{}, j);
    step(B1{}, MASK{}, j + 1);
  }
  if (j + 1 < n_tiles) {
    step(B0{}, MASK{}, j);
    step_last(B1{});
  } else {
    step_last(B0{});
  }
  wait_vm<0>();

  const float l_tot = halves_sum(l_run);
  const float f = out_scale / l_tot;
  // O through the wave's LDS rows (bfloat16 rows of 2 D bytes, the bf16
  // tiles' swizzle): four runs of 4 head dims per 32 in as 8-byte writes,
  // whole rows out as 16-byte reads, stored 1 KiB of consecutive rows per
  // instruction.  (Row and half formed from a fresh lane id.)
  uint16_t* const low = reinterpret_cast<uint16_t*>(lrw);
  const int ln_e = lane_id_here();
  const int r_e = ln_e & 31, g_e = ln_e >> 5;
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * f);
      *reinterpret_cast<bf16x4*>(low + tile_off<D>(r_e, 4 * cb + q4) + 4 * g_e) = v;
    }
#pragma unroll
  for (int x = 0; x < D / 16; ++x) {
    const int byte = x * 1024 + 16 * ln_e, row = byte / (2 * D), chunk = (byte % (2 * D)) >> 4;
    const bf16x8 w = lds_read_b128(low + tile_off<D>(row, chunk));
    if (q0 + row < N) *reinterpret_cast<bf16x8*>(O + head + (size_t)(q0 + row) * D + 8 * chunk) = w;
  }
  if (g_e == 0 && q0 + r_e < N) LSE[(size_t)bh * N + q0 + r_e] = m_run * lse_scale + __logf(l_tot) - 8.f * kLn2;
}

template <int D, bool CAUSAL, bool MX>
static hipError_t fwd_fp8_t(const FwdArgs& a) {
  const uint32_t n_qblk = (uint32_t)((a.N + 127) / 128);
  const uint32_t total = (uint32_t)(a.BH * n_qblk);
  // MX: the scales are inside the products; per tensor: folded in here.
  const float sdq = MX ? a.scale : a.scale * a.q_descale * a.k_descale;
  const float vd = MX ? 1.f : a.v_descale;
  // 2^8 P <= 448 while P <= 2^(log2(448) - 8): the reference max may lag the
  // true max by about that much (in log2 units) before a rescale is needed;
  // log2(440 / 256) leaves room for the rounding of v_exp_f32.
  const float headroom_log2 = 0.7814085f;  // log2(440 / 256)
  hipLaunchKernelGGL((fwd_fp8_kernel<D, CAUSAL, MX>), dim3(total), dim3(256), 0, a.stream,
                     (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale,
                     a.k_scale, a.v_scale, (uint16_t*)a.o, a.lse, a.N, n_qblk, total,
                     sdq * kLog2e, sdq, vd, headroom_log2 / (sdq * kLog2e));
  return hipGetLastError();
}

template <bool MX>
static hipError_t fwd_fp8_any(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? fwd_fp8_t<64, true, MX>(a) : fwd_fp8_t<64, false, MX>(a);
  return a.causal ? fwd_fp8_t<128, true, MX>(a) : fwd_fp8_t<128, false, MX>(a);
}

hipError_t launch_fwd_fp8(const FwdArgs& a) {
  return a.q_scale ? fwd_fp8_any<true>(a) : fwd_fp8_any<false>(a);
}

}  // namespace fa

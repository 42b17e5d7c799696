// Forward attention, bfloat16 inputs, float32 accumulation, gfx950 MFMA.
//
// What it computes ("FlashAttention-1: eliminating IO", sections 10.2.1 to
// 10.2.3; explainer V2 section; reading notes code 3-1): for each query row,
// O = softmax(scale Q K^T) V and LSE = ln sum exp(scale q.k), in one pass over
// the key tiles with a running max m, a running sum l and an unnormalised
// accumulator rescaled by alpha = exp(m_old - m_new), and one division at the
// end.  Scores and probabilities live only in registers.
//
// Work split (explainer V2 section; FA1 page section 10.2.5): a workgroup of
// 4 or 8 waves handles a (batch, head, block of 128 or 256 query rows) --
// under the causal mask two blocks, u and n-1-u, one after the other, so that
// every workgroup visits the same number of key tiles; each wave owns 32 query
// rows and scans every visible key tile of 64 keys (32 with a bias at d = 128).
//
// gfx950 mapping:
//  * S^T = K Q^T on v_mfma_f32_32x32x16_bf16: K (A operand) comes from LDS,
//    Q (B operand) stays in registers for the whole scan.  In the C layout a
//    lane then holds 16 keys of ONE query per 32-key half of a tile, so the
//    row max is an in-lane max plus one exchange between the wave's halves
//    (v_permlane32_swap), and the row sum needs no exchange until the end.
//  * O^T = V^T P^T: the probabilities are converted to bf16 in place and used
//    directly as the B operand (the C-layout key order is matched by reading
//    V with ds_read_b64_tr_b16 in the same order); the accumulator then holds
//    16 head dims of one query per lane, so the alpha rescale and the final
//    division are per-lane scalars.
//  * K and V tiles are double-buffered in LDS (16-byte XOR swizzle), staged
//    from HBM with 16-byte loads issued one tile ahead; one barrier per tile.
//  * exp is v_exp_f32 (base 2) with scale*log2(e) folded into one FMA.
//  * Reference max, two paths.  FAST (no bias): the row max of the block's
//    first tile, kept for the whole block -- the final division cancels any
//    reference, so no per-tile max or rescale is needed -- and checked once
//    at the end: a row sum at 2^64 or beyond, or an accumulator that is not
//    finite, and the workgroup recomputes the block on the SAFE path.  SAFE
//    (with a bias, and as that fallback): the running max of the pages, with
//    a lazy rescale (the reference moves only when a tile exceeds it by
//    2^16 in probability).
//  * Optional additive bias (the explainer's V2 section merges mask and bias
//    into the score stage), -inf masking: a tile's bias (16 bytes of four
//    consecutive keys per load) is loaded at the start of the step two before
//    the one that forms its scores, and at the end of that step -- once the
//    registers of the scores it will occupy are free -- becomes, as bias /
//    scale, the starting value of the score accumulators.  Only one tile's
//    bias is held at a time.  A row that sees no finite score ends with O = 0
//    and LSE = -inf.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

// Blocks one workgroup may take (its FAST-path flags live in LDS).
constexpr int kFwdMaxSeq = 256;

// Two waves per SIMD (64 KiB of LDS per workgroup and at most 256 registers
// per wave: two workgroups of 4 waves or one of 8 per CU); at d = 64 without
// a bias three workgroups of 4 (32 KiB of LDS each; the kernel fits in a
// third of the register file with a prefetch depth of 3).  A bias at d = 128 takes
// 32-key tiles: two 64-key score tiles and a tile's bias do not fit in the
// registers of two workgroups per CU, one 32-key score tile less does.
template <int D, bool CAUSAL, int WAVES, bool BIAS>
__global__ __launch_bounds__(64 * WAVES, D == 64 && !BIAS ? 3 : 8 / WAVES) void fwd_bf16_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
    const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE, int N,
    uint32_t n_qblk, uint32_t total, float scale, float scale_log2, float grow_thr, Bias bias) {
  constexpr int BM = 32 * WAVES, BN = BIAS && D == 128 ? 32 : 64;
  constexpr int NH = BN / 32, TILE = BN * D;  // NH: 32-key halves per tile; TILE: elements of a K or V tile
  constexpr int LPW = TILE * 2 / 1024 / WAVES;  // 1 KiB direct loads per wave per tile
  // Two K and two V tile buffers as four separate arrays: the compiler tells
  // LDS variables apart, so reading one buffer does not wait for the direct
  // loads that are still filling another.
  __shared__ __attribute__((aligned(1024))) uint16_t lk0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lk1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t lv1[TILE];
  // Q rows, 32 per wave (each wave uses only its own; same swizzle as the K
  // tiles): they arrive from HBM as whole rows, 16-byte loads of consecutive
  // addresses, instead of 16 bytes from each of 32 rows per instruction.
  __shared__ __attribute__((aligned(1024))) uint16_t lq[BM * D];
  auto ktile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lk0;
    else return lk1;
  };
  auto vtile = [&](auto bufc) -> uint16_t* {
    if constexpr (decltype(bufc)::value == 0) return lv0;
    else return lv1;
  };
  using B0 = std::integral_constant<int, 0>;
  using B1 = std::integral_constant<int, 1>;
  // With a bias, the bias tiles: each wave stages the rows of its own 32
  // queries, BN float32 keys each (below).  Without, per block of this
  // workgroup, in order: set when the FAST path must be redone (zeroed here,
  // before the first barrier).  (Two bias workgroups per CU use all 160 KiB.)
  __shared__ __attribute__((aligned(1024))) int lside[BIAS ? BM * BN : kFwdMaxSeq];
  int* const redo = lside;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if constexpr (!BIAS)
    for (int i = tid; i < kFwdMaxSeq; i += 64 * WAVES) redo[i] = 0;
  const int g = lane >> 5, r32 = lane & 31;
  // Causal: a workgroup takes row blocks u and n_qblk - 1 - u, which together
  // visit the same number of key tiles for every u, so all workgroups carry
  // equal work and each pays its set-up once per two blocks.
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;
  // The (batch, head) of the current unit (a workgroup takes units blockIdx.x,
  // blockIdx.x + gridDim.x, ...).
  uint32_t bh = 0;
  size_t head = 0;
  const uint16_t *Kh = K, *Vh = V;
  uint16_t* const lqw = lq + wave * 32 * D;  // this wave's Q / O rows

  // A block's first loads, issued ahead of the block: this wave's Q rows into
  // its LDS rows (rows past N arrive as zeros) and its share of K_0 and V_0
  // into tile buffers 0.  (Offsets formed from a fresh lane id: nothing here
  // stays live through a scan.)
  auto row_off = [](uint32_t byte) __attribute__((always_inline)) -> uint32_t {
    const uint32_t row = byte / (2 * D);  // byte offset in global of the chunk the swizzle puts at `byte`
    return row * 2 * D + ((((byte % (2 * D)) >> 4) ^ (uint32_t)swz<D>((int)row)) << 4);
  };
  auto issue_q = [&](const uint16_t* Qhead, const uint32_t qblk) __attribute__((always_inline)) {
    const int q0 = (int)qblk * BM + wave * 32;
    const uint32_t ln = (uint32_t)lane_id_here();
    const auto qres = make_tile_rsrc<2 * D>(Qhead + (size_t)q0 * D, N - q0);
#pragma unroll
    for (int x = 0; x < D / 16; ++x) load_lds16(qres, lqw + x * 512, row_off(x * 1024u + 16u * ln));
  };
  auto issue_kv = [&](const uint16_t* Khead, const uint16_t* Vhead) __attribute__((always_inline)) {
    const uint32_t ln = (uint32_t)lane_id_here();
    const auto kres = make_tile_rsrc<2 * D>(Khead, N), vres = make_tile_rsrc<2 * D>(Vhead, N);
#pragma unroll
    for (int x = 0; x < LPW; ++x) {
      const uint32_t o = row_off((uint32_t)(wave * LPW + x) * 1024u + 16u * ln);
      load_lds16(kres, lk0 + (wave * LPW + x) * 512, o);
      load_lds16(vres, lv0 + (wave * LPW + x) * 512, o);
    }
  };
  // The next block's first loads, issued by each wave right after the current
  // block's last barrier (set by the caller before each block): its Q rows
  // (the Q rows of this block are in registers by then), and its K_0 and V_0
  // when tile buffers 0 are free -- the current block's last tile is in
  // buffers 1 (an even number of tiles), which the other waves may still read.
  bool pf_q = false, pf_kv = false;
  uint32_t pf_qb = 0;
  const uint16_t *pf_Qh = Q, *pf_Kh = K, *pf_Vh = V;
  auto on_last = [&]() __attribute__((always_inline)) {
    if (pf_q) issue_q(pf_Qh, pf_qb);
    if (pf_kv) issue_kv(pf_Kh, pf_Vh);
  };

  // FAST (no bias): the reference max is taken on the
  // block's first tile only and kept.  Later probabilities exp(S - m) may
  // exceed 1 by anything float32 holds, which costs no relative precision,
  // and need no per-tile max.  A block whose row sum ends at 2^64 or beyond
  // (or not finite), or whose accumulator is not finite (P V past the float
  // range), is recomputed on the SAFE path.  SAFE: the row max of every tile
  // before its probabilities are formed (lazy rescale).  Returns (per lane)
  // whether the block must be recomputed.
  auto body = [&](const uint32_t qblk, auto fastc) __attribute__((always_inline)) -> bool {
  constexpr bool FAST = decltype(fastc)::value;
  static_assert(!(FAST && BIAS), "the bias kernels take the SAFE path");
  bool bad = false;
  const int q0 = (int)qblk * BM + wave * 32;  // first query row of this wave
  const int qrow = q0 + r32;                  // the query of this lane's column

  // Additive bias: a buffer resource over this (b, h) slice and the byte
  // offset of this lane's row (rows past N read row N - 1; they are never
  // written).  Element i of key half h of a tile at key0 is key
  // key0 + 32 h + 8 (i / 4) + 4 g + i % 4: load x = 4 h + i / 4, component i % 4.
  [[maybe_unused]] const auto brs = BIAS ? bias_rsrc(bias, bh) : make_rsrc(nullptr, 0);
  [[maybe_unused]] const uint32_t bvoff =
      BIAS ? (uint32_t)((long long)min(qrow, N - 1) * bias.sq * 4 + 16 * g) : 0u;
  [[maybe_unused]] const float inv_scale = 1.f / scale;
  auto load_bias = [&](f32x4 (&bv)[4 * NH], int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < 4 * NH; ++x)
      bv[x] = buffer_load_f32x4(brs, bvoff + 128 * (x >> 2) + 32 * (x & 3), (uint32_t)key0 * 4u);
  };
  auto add_bias = [&](const f32x4 (&bv)[4 * NH], f32x16 (&s)[NH], int i) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) s[h][i] = fmaf(bv[4 * h + (i >> 2)][i & 3], inv_scale, s[h][i]);
  };
  // The bias in raw-score units as the starting value of a tile's score
  // accumulators: the matrix core then adds K Q^T to it.
  auto init_bias = [&](const f32x4 (&bv)[4 * NH], f32x16 (&s)[NH], int i) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) s[h][i] = bv[4 * h + (i >> 2)][i & 3] * inv_scale;
  };
  // Tiles after the first go through the wave's own LDS rows: direct loads
  // that cover whole bias rows (RPI rows of RB bytes per 1 KiB load: 8 or 4
  // cache lines, not the 32 of a 16-byte read from each row), then one
  // 16-byte read per 4 keys in the accumulator layout.  Row r keeps logical
  // 16-byte chunk c at physical chunk c ^ bswz(r), so that the 16 rows of a
  // read pass meet 16 different bank groups.  Each wave reads only the rows it
  // loaded, and loads a tile only after reading the one before: no barrier.
  // Rows past N load whatever the resource returns (zeros past the slice);
  // they are never written.
  constexpr int RB = BN * 4, RPI = 1024 / RB, LPR = RB / 16, NBL = BN / 8, NX = RB == 128 ? 2 : 4;
  auto bswz = [](int r) __attribute__((always_inline)) { return RB == 128 ? (r >> 1) & 7 : r & 15; };
  [[maybe_unused]] int* const lbw = lside + wave * 32 * BN;
  // per-lane byte offsets of the loads, by x % NX (the swizzle of row RPI x +
  // l / LPR depends on x only through x % NX); the row step RPI x is scalar
  [[maybe_unused]] uint32_t bld[NX];
  if constexpr (BIAS) {
    const int ln = lane_id_here(), u = ln / LPR;
#pragma unroll
    for (int x = 0; x < NX; ++x)
      bld[x] = (uint32_t)((long long)(q0 + u) * bias.sq * 4) + 16u * (uint32_t)((ln % LPR) ^ bswz(RPI * x + u));
  }
  auto stage_bias = [&](int key0) __attribute__((always_inline)) {
#pragma unroll
    for (int x = 0; x < NBL; ++x)
      load_lds16(brs, lbw + 256 * x, bld[x % NX],
                 (uint32_t)(RPI * x) * (uint32_t)bias.sq * 4u + (uint32_t)key0 * 4u);
  };
  auto read_bias = [&](f32x4 (&bv)[4 * NH]) __attribute__((always_inline)) {
    const int ln = lane_id_here(), r = ln & 31;
    const uint32_t z = (uint32_t)(wave * 32 * RB + r * RB + 16 * ((ln >> 5) ^ bswz(r)));
#pragma unroll
    for (int x = 0; x < 4 * NH; ++x)  // logical chunk 8 h + 2 j + g, x = 4 h + j
      bv[x] = *reinterpret_cast<const f32x4*>(
          reinterpret_cast<const char*>(lside) + (z ^ (uint32_t)(16 * (8 * (x >> 2) + 2 * (x & 3)))));
  };


  const int kv_end = CAUSAL ? min(N, (int)qblk * BM + BM) : N;
  const int n_tiles = (kv_end + BN - 1) / BN;

  // Per-lane element offsets inside one tile buffer (the swizzle depends only
  // on row % 16, so whole 16-row steps are plain constants added to these).
  int koff[D / 16];  // K as the A operand: row r32 (+32h), chunk 2t + g
#pragma unroll
  for (int t = 0; t < D / 16; ++t) koff[t] = tile_off<D>(r32, 2 * t + g);
  // Q fragment as the B operand of S^T = K Q^T: lane holds Q[qrow][16t + 8g .. +7]
  // (read from the wave's LDS rows once they have landed).
  bf16x8 qf[D / 16];
  // V by the transposing read: source lane (r, c) = ((lane%16)/4, lane%4) reads
  // row 4g + r (+8 for keys 8..15 of a 16-key step) at head dim 32cb + 16((lane/16)%2) + 4c.
  const int tr_r = (lane & 15) >> 2, tr_c = lane & 3, tr_n0 = 16 * ((lane >> 4) & 1);
  int voff[D / 32][2];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
    const int d = 32 * cb + tr_n0 + 4 * tr_c;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) voff[cb][hf] = tile_off<D>(4 * g + tr_r + 8 * hf, d >> 3) + (d & 7);
  }
  // Direct HBM -> LDS staging: load x of this wave fills bytes
  // [(wave*LPW + x) * 1024, +1024) of a tile buffer, lane l the 16 bytes at
  // +16 l.  Those bytes are physical chunk (16 l % 2D)/16 of tile row
  // (byte / 2D); the lane therefore fetches the logical chunk that the
  // swizzle puts there, at a byte offset in the tile that never changes.
  uint32_t ldoff[LPW];
#pragma unroll
  for (int x = 0; x < LPW; ++x) {
    const int byte = (wave * LPW + x) * 1024 + 16 * lane;
    const int row = byte / (2 * D);
    ldoff[x] = (uint32_t)(row * 2 * D + ((((byte % (2 * D)) >> 4) ^ swz<D>(row)) << 4));
  }
  // A tile's loads go through a buffer resource that starts at the tile and
  // ends at the head's end: rows past N arrive as zeros (those keys are
  // masked, so their scores never count and their P is exactly 0).
  auto tile_rsrc = [&](const uint16_t* src, int key0) __attribute__((always_inline)) {
    return make_tile_rsrc<2 * D>(src + (size_t)key0 * D, N - key0);
  };
  auto stage = [&](const uint16_t* src, uint16_t* dst, int key0) __attribute__((always_inline)) {
    const auto r = tile_rsrc(src, key0);
#pragma unroll
    for (int x = 0; x < LPW; ++x) load_lds16(r, dst + (wave * LPW + x) * 512, ldoff[x]);
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) acc[cb] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  // exp2 argument offset for the reference max; 0 while a row has seen no
  // finite score (all its scores so far are -inf, whose exp is 0).
  auto neg_ref = [&]() __attribute__((always_inline)) -> float {
    if constexpr (BIAS) return m_run == -INFINITY ? 0.f : -m_run * scale_log2;
    else return -m_run * scale_log2;
  };

  auto scores = [&](const uint16_t* Kt, f32x16 (&s)[NH]) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h) s[h] = mfma_bf16(lds_read_b128(Kt + 32 * D * h + koff[0]), qf[0], f32x16{});
#pragma unroll
    for (int t = 1; t < D / 16; ++t)
#pragma unroll
      for (int h = 0; h < NH; ++h) s[h] = mfma_bf16(lds_read_b128(Kt + 32 * D * h + koff[t]), qf[t], s[h]);
  };

  // O^T += V_j^T P_j^T with P_j in bf16 (the B operand exactly as the
  // accumulator layout left it, one operand per 16-key chunk; V read
  // transposed in the same key order).
  auto pv = [&](const uint16_t* Vt, const bf16x8 (&p)[2 * NH]) __attribute__((always_inline)) {
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb) {
      const uint16_t* vb = Vt + voff[cb][0];
      const uint16_t* vc = Vt + voff[cb][1];
#pragma unroll
      for (int kc = 0; kc < 2 * NH; ++kc)
        acc[cb] = mfma_bf16(concat(lds_read_tr16(vb + 16 * D * kc), lds_read_tr16(vc + 16 * D * kc)),
                            p[kc], acc[cb]);
    }
  };

  // Rescale to a new reference max (rare; see guard).
  auto rescale = [&](float mx) __attribute__((always_inline)) {
    const float m_new = fmaxf(m_run, mx);
    float alpha = exp2_fast((m_run - m_new) * scale_log2);
    if constexpr (BIAS) alpha = m_new == -INFINITY ? 1.f : alpha;  // nothing seen yet
    l_run *= alpha;
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[cb][i] *= alpha;
    m_run = m_new;
  };
  // Online softmax (FA1 page 10.2.2; reading notes code 3-1) against a
  // running reference max m_run.  Lazy rescale: m_run only moves when some
  // row's tile max exceeds it by more than grow_thr (2^16 in probability);
  // the accumulator and row sum are then rescaled by alpha = exp(m_old -
  // m_new).  Otherwise the probabilities exp(S - m_run) may reach 2^16,
  // which float32 accumulation and bf16 P hold exactly as well as values <= 1
  // -- any reference gives the same exact result.  The first tile always
  // moves m_run off -infinity.
  auto guard = [&](float mx) __attribute__((always_inline)) {  // mx: this lane's max over its scores of the tile
    mx = halves_max(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + grow_thr) != 0) rescale(mx);
  };
  auto rowmax_guard = [&](const f32x16 (&s)[NH]) __attribute__((always_inline)) {
    float mx = NH == 2 ? fmaxf(s[0][0], s[NH - 1][0]) : s[0][0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, NH == 2 ? fmaxf(s[0][i], s[NH - 1][i]) : s[0][i]);
    guard(mx);
  };
  // P = exp(S - m_run) in place; row sum over the float32 P; P in bf16 out.
  auto exps = [&](f32x16 (&s)[NH], bf16x8 (&p)[2 * NH]) __attribute__((always_inline)) {
    const float mneg = neg_ref();
    float rs[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) rs[h] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int h = 0; h < NH; ++h) s[h][i] = exp2_fast(fmaf(s[h][i], scale_log2, mneg));
#pragma unroll
      for (int h = 0; h < NH; ++h) rs[h] += s[h][i];
    }
    l_run += NH == 2 ? rs[0] + rs[NH - 1] : rs[0];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      p[2 * h] = to_bf16x8(s[h], 0);
      p[2 * h + 1] = to_bf16x8(s[h], 8);
    }
  };

  // Masked scores: keys past N, and under the causal mask keys after the
  // query.  Element i of key half h of a tile at key0 is key key0 + 32 h +
  // 8 (i / 4) + 4 g + i % 4; it is visible iff it is at most lim = N - 1
  // (causal: min(N - 1, qrow)).  With t = lim - key0 - 4 g (one value per lane
  // and tile) that is 32 h + 8 (i / 4) + i % 4 <= t: one compare with a
  // constant per element.  (The lane's row is formed from the lane id here,
  // not held through the scan.)
  auto mask_thr = [&](int key0) __attribute__((always_inline)) -> int {
    const int ln = lane_id_here();
    const int lim = CAUSAL ? min(N - 1, q0 + (ln & 31)) : N - 1;
    return lim - key0 - 4 * (ln >> 5);
  };
  auto mask_elem = [&](f32x16 (&s)[NH], int i, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < NH; ++h)
      if (32 * h + 8 * (i >> 2) + (i & 3) > t) s[h][i] = -INFINITY;
  };
  auto apply_mask = [&](f32x16 (&s)[NH], int key0) __attribute__((always_inline)) {
    const int t = mask_thr(key0);
#pragma unroll
    for (int i = 0; i < 16; ++i) mask_elem(s, i, t);
  };

  // Causal without a bias: this wave's tiles end at n_use, the last one with
  // a key at or before its last query; the workgroup's diagonal tiles past
  // it would give all-zero P and all-masked scores.  The wave stops its
  // products there, and for the rest of the workgroup's tiles only stages its
  // share and meets the barriers (its SIMD partner has the matrix core to
  // itself meanwhile).
  const int n_use = CAUSAL && !BIAS ? min(n_tiles, (q0 + 31) / BN + 1) : n_tiles;
  // Software pipeline: K runs one tile ahead of V.  At step j the LDS holds
  // K_{j+1} and V_j, and the registers hold S_j = K_j Q^T, masked, with its
  // reference max settled.  Tiles [0, j_full) need no mask for this wave's
  // rows; the rest (the causal diagonal, a ragged tail) are masked while
  // their scores are formed.  Causal without a bias, only the wave's last
  // tile: the wave's first row q0 is a multiple of 32, so every key of an
  // earlier 64-key tile lies before q0 and inside N.  The two score buffers
  // swap roles with the step parity, so nothing is copied.
  const int j_full = CAUSAL && !BIAS ? n_use - 1 : min(CAUSAL ? (int)qblk * (BM / BN) : n_tiles, N / BN);
  f32x16 sa[NH], sb[NH];  // scores of even (a) and odd (b) tiles, by key half
  auto sc_of = [&](auto parity) __attribute__((always_inline)) -> f32x16 (&)[NH] {
    if constexpr (decltype(parity)::value == 0) return sa;
    else return sb;
  };
  // Bias of tile t + 1: staged at the start of step t - 1 (tile 1 here; tile
  // 0 straight into registers) and turned into the starting value of S_{t+1}
  // at the end of that step, once P_{t-1} no longer needs the registers
  // S_{t+1} will use.
  [[maybe_unused]] f32x4 bv0[4 * NH], bv[4 * NH];
  if constexpr (BIAS) {
    load_bias(bv0, 0);
    stage_bias(BN);
  }
  barrier_vm<0>();  // the block's Q rows, K_0 and V_0 (issue()) have landed
  if constexpr (BIAS) read_bias(bv);
  {
    const int ln_r = lane_id_here();
#pragma unroll
    for (int t = 0; t < D / 16; ++t) qf[t] = lds_read_b128(lqw + tile_off<D>(ln_r & 31, 2 * t + (ln_r >> 5)));
  }
  stage(Kh, lk1, BN);  // (a tile past the end arrives as zeros; never used)
  scores(lk0, sa);
  if constexpr (BIAS) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      add_bias(bv0, sa, i);
      init_bias(bv, sb, i);
    }
  }
  if (j_full == 0) apply_mask(sa, 0);
  rowmax_guard(sa);

  // Step j < n_tiles - 1: one fenced stream of matrix products,
  // S_{j+1} = K_{j+1} Q^T (NS products, K from LDS) then O^T += V_j^T P_j^T
  // (V by the transposing read, key chunk by key chunk), every operand
  // fetched DEPTH products ahead.  The vector work rides between the
  // products: exp, row sum and bf16 packing of P_j over the first EXP_OPS + 2
  // products (each key chunk of P is complete before its first PV product),
  // the mask (when tile j+1 needs one) and row max of S_{j+1} over the last
  // MAX_OPS products, with a bias the starting value of S_{j+2} once P_j is
  // packed, and this wave's share of K_{j+2} and V_{j+1} issued one load every
  // 2 products early in the step, so that it has landed by the next barrier.
  constexpr int DEPTH = D == 64 ? 3 : 4;
  constexpr int NS = NH * (D / 16), NOPS = NS + 2 * NH * (D / 32);  // S products come first
  // The mask and row max of S_{j+1} read its finished scores: they ride on
  // PV products only (at d = 64 that leaves 8 of them).
  // (at d = 128 the exp phases spread over 26 of the 32 products, the most
  // the packing deadline of the last key chunk allows: +0.2-0.6 % over 24)
  constexpr int EXP_OPS = NH == 2 ? (D == 128 ? NS + 10 : NS + 2 * (D / 32)) : NS + 2;
  constexpr int MAX_OPS = NH == 2 ? (NOPS - NS < 12 ? NOPS - NS : 12) : 4;
  static_assert(NOPS - MAX_OPS >= NS, "the row max must not see partial scores");
  // the last element of key chunk kc (element 8 kc + 7 of half kc / 2) gets its phase (c), which
  // packs the chunk, in product slot (its phase-(a) slot) + 2, before the chunk's first PV product
  static_assert((7 * EXP_OPS) / (16 * NH) + 2 < NS, "chunk 0 packed before its first PV product");
  static_assert(((16 * NH - 1) * EXP_OPS) / (16 * NH) + 2 < NS + (2 * NH - 1) * (D / 32),
                "last chunk packed before its first PV product");
  auto step = [&](auto parity, auto maskc, int j) __attribute__((always_inline)) {
    constexpr int P = decltype(parity)::value;  // j % 2
    constexpr bool MASK_NEXT = decltype(maskc)::value;
    using PN = std::integral_constant<int, P ^ 1>;
    f32x16(&sc)[NH] = sc_of(parity);
    f32x16(&sn)[NH] = sc_of(PN{});
    barrier_vm<0>();  // this wave's pieces of K_{j+1} and V_j have landed, and everyone's
    const uint16_t* Kt = ktile(PN{});
    const uint16_t* Vt = vtile(parity);
    uint16_t* Vdst = vtile(PN{});
    uint16_t* Kdst = ktile(parity);
    const float mneg = neg_ref();
    const int key1 = (j + 1) * BN;
    // tile j + 2's bias, ahead of this step's staging loads
    if constexpr (BIAS) stage_bias(key1 + BN);
    const auto kres = tile_rsrc(Kh, (j + 2) * BN);
    const auto vres = tile_rsrc(Vh, (j + 1) * BN);
    bf16x8 pk[2 * NH];
    auto fetch = [&](int k) __attribute__((always_inline)) -> bf16x8 {
      if (k < NS) return lds_read_b128(Kt + 32 * D * (k % NH) + koff[k / NH]);
      const int kc = (k - NS) / (D / 32), cb = (k - NS) % (D / 32);
      return concat(lds_read_tr16(Vt + voff[cb][0] + 16 * D * kc),
                    lds_read_tr16(Vt + voff[cb][1] + 16 * D * kc));
    };
    auto op = [&](int k, const bf16x8& a) __attribute__((always_inline)) {
      if (k < NS) {
        const int t = k / NH, h = k % NH;
        sn[h] = mfma_bf16(a, qf[t], t == 0 && !BIAS ? f32x16{} : sn[h]);
      } else {
        const int kc = (k - NS) / (D / 32), cb = (k - NS) % (D / 32);
        acc[cb] = mfma_bf16(a, pk[kc], acc[cb]);
      }
    };
    // Element e of P_j (key half e / 16, element e % 16) in three phases
    // placed in three consecutive products, so that no instruction waits on
    // the one just before it: (a) the scaled, shifted score; (b) its exp; (c)
    // the row sum (two partial sums) and, closing a key chunk, the bf16
    // packing.  The empty volatile statements pin each phase to its product.
    float lsum[2] = {0.f, 0.f};
    auto pin = [](float& x) __attribute__((always_inline)) { asm volatile("" : "+v"(x)); };
    auto phase = [&](int e, int ph) __attribute__((always_inline)) {
      f32x16& sv = sc[e >> 4];
      const int i = e & 15;
      float x = sv[i];
      if (ph == 0) {
        pin(x);
        x = fmaf(x, scale_log2, mneg);
        pin(x);
      } else if (ph == 1) {
        x = exp2_fast(x);
        pin(x);
      } else {
        lsum[e & 1] = e < 2 ? x : lsum[e & 1] + x;
      }
      sv[i] = x;
      if (ph == 2 && (e & 7) == 7) pk[e >> 3] = to_bf16x8(sv, i - 7);
    };
    int mthr = 0;  // mask threshold of S_{j+1}, formed where its masking starts
    // Elements start phase (a) over products 0 .. EXP_OPS-1; phase (c) of the
    // last element of key chunk kc lands two products later, before product
    // NS + kc (D/32), the chunk's first PV product.
    float mxp[2] = {-INFINITY, -INFINITY};
    auto extra = [&](int k) __attribute__((always_inline)) {
#pragma unroll
      for (int ph = 0; ph < 3; ++ph) {
        const int ks = k - ph;
        if (ks >= 0 && ks < EXP_OPS) {
#pragma unroll
          for (int e = ks * 16 * NH / EXP_OPS; e < (ks + 1) * 16 * NH / EXP_OPS; ++e) phase(e, ph);
        }
      }
      if (k >= NOPS - MAX_OPS) {  // row max of S_{j+1} over the last MAX_OPS products
        const int r = k - (NOPS - MAX_OPS);
        if constexpr (MASK_NEXT)
          if (r == 0) mthr = mask_thr(key1);
#pragma unroll
        for (int i = r * 16 / MAX_OPS; i < (r + 1) * 16 / MAX_OPS; ++i) {
          if constexpr (MASK_NEXT) mask_elem(sn, i, mthr);
          if constexpr (!FAST) {
            mxp[i & 1] = fmaxf(mxp[i & 1], NH == 2 ? fmaxf(sn[0][i], sn[NH - 1][i]) : sn[0][i]);
            pin(mxp[i & 1]);
          }
        }
      }
      if constexpr (BIAS) {  // S_{j+2} starts from its bias, once P_j is packed
        constexpr int K0 = EXP_OPS + 2, NI = NOPS - K0;
        static_assert(NI > 0 && K0 >= 2, "no product left after the exp phases");
        if (k == K0 - 2) read_bias(bv);
        if (k >= K0) {
#pragma unroll
          for (int i = (k - K0) * 16 / NI; i < (k - K0 + 1) * 16 / NI; ++i) init_bias(bv, sc, i);
        }
      }
      if (k % 2 == 0 && k / 2 < 2 * LPW) {  // loads: K_{j+2} pieces, then V_{j+1}
        const int x = (k / 2) % LPW;
        if (k / 2 >= LPW) load_lds16(vres, Vdst + (wave * LPW + x) * 512, ldoff[x]);
        else load_lds16(kres, Kdst + (wave * LPW + x) * 512, ldoff[x]);
      }
    };
    bf16x8 ring[DEPTH + 1];
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
    if constexpr (!FAST) guard(fmaxf(mxp[0], mxp[1]));
  };
  // This wave's last tile j: no next scores; P_j then O^T += V_j^T P_j^T.
  // Under the causal mask a wave's last tile can come before the workgroup's
  // (n_use below); the wave then still stages its share of K_{j+2}, V_{j+1}.
  auto stage_next = [&](auto parity, int j) __attribute__((always_inline)) {
    using PN = std::integral_constant<int, decltype(parity)::value ^ 1>;
    const auto kres = tile_rsrc(Kh, (j + 2) * BN);
    const auto vres = tile_rsrc(Vh, (j + 1) * BN);
#pragma unroll
    for (int L = 0; L < 2 * LPW; ++L) {
      const int x = L % LPW;
      if (L >= LPW) load_lds16(vres, vtile(PN{}) + (wave * LPW + x) * 512, ldoff[x]);
      else load_lds16(kres, ktile(parity) + (wave * LPW + x) * 512, ldoff[x]);
    }
  };
  auto step_last = [&](auto parity, int j) __attribute__((always_inline)) {
    barrier_vm<0>();
    if (j + 1 < n_tiles) stage_next(parity, j);  // (causal: tiles past this wave's queries follow)
    else on_last();
    bf16x8 p[2 * NH];
    exps(sc_of(parity), p);
    pv(vtile(parity), p);
  };
  // Step j forms S_{j+1}, masked iff j + 1 >= j_full; steps run in pairs (the
  // parity picks the buffers), then the last tile.
  using NOMASK = std::false_type;
  using MASK = std::true_type;
  int j = 0;
  for (; j + 2 < j_full; j += 2) {
    step(B0{}, NOMASK{}, j);
    step(B1{}, NOMASK{}, j + 1);
  }
  if constexpr (CAUSAL && !BIAS) {
    // j_full = n_use - 1: only the step forming the wave's last tile masks
    if (j + 2 == j_full) {
      step(B0{}, NOMASK{}, j);
      step(B1{}, MASK{}, j + 1);
      j += 2;
    }
  } else {
    for (; j + 2 < n_use; j += 2) {
      step(B0{}, MASK{}, j);
      step(B1{}, MASK{}, j + 1);
    }
  }
  if (j + 1 < n_use) {  // two tiles left
    step(B0{}, MASK{}, j);
    step_last(B1{}, ++j);
  } else {
    step_last(B0{}, j);
  }
  if constexpr (CAUSAL && !BIAS) {
    for (++j; j < n_tiles; ++j) {  // tiles past this wave's queries
      barrier_vm<0>();
      if (j + 1 < n_tiles) {
        if (j & 1) stage_next(B1{}, j);
        else stage_next(B0{}, j);
      } else {
        on_last();
      }
    }
  }
  // (every tile load of this block has landed: each wave waited for its own
  // before the last barrier; only the next block's loads may be in flight)

  const float l_tot = halves_sum(l_run);
  if constexpr (FAST) {
    uint32_t top = 0;  // largest |acc| bit pattern: >= 0x7f800000 means inf or NaN
#pragma unroll
    for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
      for (int i = 0; i < 16; ++i) top = max(top, __float_as_uint(acc[cb][i]) & 0x7fffffffu);
    bad = bad || !(__float_as_uint(l_tot) < 0x5f800000u) || top >= 0x7f800000u;
  }
  // (with a bias, a row that saw no finite score has l = 0: O = 0, LSE = -inf)
  const bool empty_row = BIAS && l_tot == 0.f;
  const float inv = empty_row ? 0.f : 1.f / l_tot;
  // (the row formed again from the lane id: not held through the scan)
  const int ln_e = lane_id_here();
  const int r_e = ln_e & 31, g_e = ln_e >> 5, qrow_e = q0 + r_e;
  // O through 2 KiB of LDS per wave in K tile buffer 1 (free during the last
  // tile, whatever its parity), 32 head dims at a time: the lane's four runs
  // of 4 dims go in as 8-byte writes ([32 rows][64 bytes], 16-byte chunks
  // XOR-swizzled by row / 4, and the two 8-byte halves of a chunk swapped in
  // rows 16..31, so that 32 lanes' writes meet 64 different banks), and
  // leave as 16-byte reads of 16 rows x 64 bytes per instruction, stored as
  // 64 contiguous bytes per row.
  uint16_t* const low = lk1 + wave * 1024;
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (__bf16)(acc[cb][4 * q4 + e] * inv);
      *reinterpret_cast<bf16x4*>(low + r_e * 32 + ((q4 ^ ((r_e >> 2) & 3)) << 3) +
                                 4 * (g_e ^ (r_e >> 4))) = v;
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      const int row = 16 * x + (ln_e >> 2), c = ln_e & 3;
      bf16x8 w = lds_read_b128(low + row * 32 + ((c ^ ((row >> 2) & 3)) << 3));
      if (x == 1) w = __builtin_shufflevector(w, w, 4, 5, 6, 7, 0, 1, 2, 3);  // (halves swapped in rows 16..31)
      if (q0 + row < N) *reinterpret_cast<bf16x8*>(O + head + (size_t)(q0 + row) * D + 32 * cb + 8 * c) = w;
    }
  }
  if (g_e == 0 && qrow_e < N)
    LSE[(size_t)bh * N + qrow_e] = empty_row ? -INFINITY : m_run * scale + __logf(l_tot);
  return bad;
  };  // body

  // The workgroup's blocks run back to back: unit after unit, and under the
  // causal mask the pair's longer block first.  Each wave issues the next
  // block's Q rows (and, when tile buffers 0 are free, its K_0 and V_0) at the
  // current block's last barrier (on_last); otherwise every wave meets at a
  // barrier after the block and then issues them.  Without a bias every
  // block takes the FAST path and records in redo[] whether any lane of the
  // workgroup found it out of range; those blocks are computed again on the
  // SAFE path after the last one (overwriting their outputs).  With a bias:
  // the SAFE path.
  using RUNC = std::integral_constant<bool, !BIAS>;
  using SAFEC = std::false_type;
  auto tiles_of = [&](uint32_t qb) __attribute__((always_inline)) {
    const int kv_end = CAUSAL ? min(N, (int)qb * BM + BM) : N;
    return (kv_end + BN - 1) / BN;
  };
  // Block k (0, or 1 for the second block of a causal pair) of unit vb: its
  // (batch, head) and row block; false past the end or for a pair of one.
  auto locate = [&](uint32_t vb, int k, uint32_t& bh_o, uint32_t& qb_o) __attribute__((always_inline)) -> bool {
    if (vb >= total) return false;
    uint32_t unit;
    if (BIAS && bias.grouped) map_block_grouped(vb, n_units, total, bias.grouped, false, bh_o, unit);
    else map_block(vb, n_units, total, kOrderPlain, bh_o, unit);
    const uint32_t partner = CAUSAL ? n_qblk - 1 - unit : unit;
    qb_o = k == 0 ? partner : unit;
    return k == 0 || partner != unit;
  };
  // the block after (vb, k) in this workgroup's walk
  auto advance = [&](uint32_t& vb, int& k, uint32_t& bh_o, uint32_t& qb_o) __attribute__((always_inline)) -> bool {
    if (CAUSAL && k == 0) {
      k = 1;
      if (locate(vb, 1, bh_o, qb_o)) return true;
    }
    k = 0;
    vb += gridDim.x;
    return locate(vb, 0, bh_o, qb_o);
  };
  auto set_head = [&](uint32_t b) __attribute__((always_inline)) {
    bh = b;
    head = (size_t)b * (size_t)N * D;
    Kh = K + head;
    Vh = V + head;
  };
  {
    uint32_t vb = blockIdx.x, cbh = 0, cqb = 0;
    int k = 0, seq = 0;
    bool have = locate(vb, 0, cbh, cqb);
    if (have) {
      issue_q(Q + (size_t)cbh * (size_t)N * D, cqb);
      issue_kv(K + (size_t)cbh * (size_t)N * D, V + (size_t)cbh * (size_t)N * D);
    }
    while (have) {
      uint32_t nvb = vb, nbh = 0, nqb = 0;
      int nk = k;
      const bool next = advance(nvb, nk, nbh, nqb);
      const size_t nhead = (size_t)nbh * (size_t)N * D;
      const bool even = (tiles_of(cqb) & 1) == 0;
      pf_q = next;
      pf_kv = next && even;
      pf_qb = nqb;
      pf_Qh = Q + nhead;
      pf_Kh = K + nhead;
      pf_Vh = V + nhead;
      set_head(cbh);
      const bool bad = body(cqb, RUNC{});
      if constexpr (!BIAS)
        if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0) redo[seq] = 1;
      if (next && !even) {
        barrier_vm<63>();  // tile buffers 0 are read no more
        issue_kv(K + nhead, V + nhead);
      }
      ++seq;
      vb = nvb;
      k = nk;
      cbh = nbh;
      cqb = nqb;
      have = next;
    }
  }
  if constexpr (!BIAS) {
    pf_q = pf_kv = false;
    barrier_vm<63>();  // every flag is written, every tile read
    int s = 0;
    for (uint32_t vb = blockIdx.x; vb < total; vb += gridDim.x) {
      for (int k = 0; k < (CAUSAL ? 2 : 1); ++k) {
        uint32_t b, qb;
        if (!locate(vb, k, b, qb)) continue;
        if (__builtin_amdgcn_readfirstlane(redo[s]) != 0) {
          set_head(b);
          issue_q(Q + head, qb);
          issue_kv(Kh, Vh);
          body(qb, SAFEC{});
          barrier_vm<63>();
        }
        ++s;
      }
    }
  }
}

// Compute units of the current device (looked up once per device).
static int cu_count() {
  static std::atomic<int> known[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = -1;
  if (dev >= 0 && dev < 64) {
    const int n = known[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
  }
  int n = 0;
  if (dev < 0 || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev >= 0 && dev < 64) known[dev].store(n, std::memory_order_relaxed);
  return n;
}

template <int D, bool CAUSAL, int WAVES, bool BIAS>
static hipError_t launch_fwd_bf16_t(const FwdArgs& a) {
  constexpr int BM = 32 * WAVES;
  const uint32_t n_qblk = (uint32_t)((a.N + BM - 1) / BM);
  const uint32_t n_units = CAUSAL ? (n_qblk + 1) / 2 : n_qblk;  // row blocks paired when causal
  const uint32_t total = (uint32_t)(a.BH * n_units);
  // As many workgroups as the CUs hold at once (one of 8 waves at d = 128,
  // three of 4 at d = 64), each taking units blockIdx.x + k gridDim.x back to
  // back -- but never more than kFwdMaxSeq blocks per workgroup.
  constexpr int kPerCu = D == 64 && !BIAS ? 3 : 8 / WAVES;
  const uint64_t per = CAUSAL ? 2 : 1;
  const uint64_t slots = (uint64_t)cu_count() * kPerCu;
  const uint64_t least = ((uint64_t)total * per + kFwdMaxSeq - 1) / kFwdMaxSeq;
  // (With a bias, one unit per workgroup as launched: the dense-bias forward,
  // bound by its bias traffic, measured 10 % slower with the static walk than
  // with the hardware handing out units as CUs free up.)
  const uint32_t grid = BIAS ? total : (uint32_t)std::min<uint64_t>(total, std::max(slots, least));
  Bias bias = a.bias;
  bias.grouped = group_blocks(bias, a.BH, n_units, 8);  // two workgroups per CU: 64 per XCD
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, WAVES, BIAS>), dim3(grid), dim3(64 * WAVES), 0,
                     a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (uint16_t*)a.o, a.lse, a.N, n_qblk, total, a.scale, a.scale * kLog2e,
                     kRescaleLog2 / (a.scale * kLog2e), bias);
  return hipGetLastError();
}

// Waves per workgroup: at d = 128 eight (256 query rows, one workgroup per CU,
// still two waves per SIMD), so each K/V tile staged into LDS serves twice
// the rows; at d = 64 four (three workgroups, twelve waves, per CU), and four
// with a bias (both measured faster that way).
template <int D, bool CAUSAL>
static hipError_t launch_fwd_bf16_b(const FwdArgs& a) {
  return a.bias.p ? launch_fwd_bf16_t<D, CAUSAL, 4, true>(a)
                  : launch_fwd_bf16_t<D, CAUSAL, D == 128 ? 8 : 4, false>(a);
}

hipError_t launch_fwd_bf16(const FwdArgs& a) {
  if (a.d == 64) return a.causal ? launch_fwd_bf16_b<64, true>(a) : launch_fwd_bf16_b<64, false>(a);
  if (!a.bias.p && a.schedule == kSchedPingPong) return launch_fwd_bf16_pp(a);
  if (!a.bias.p && a.schedule == kSchedRows64) return launch_fwd_bf16_w64(a);
  return a.causal ? launch_fwd_bf16_b<128, true>(a) : launch_fwd_bf16_b<128, false>(a);
}

}  // namespace fa

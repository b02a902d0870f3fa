// partial_fwd.hip — one KV block folded into a context-parallel rank's
// attention state, for gfx950 (MI355X).
//
// Method: the per-block step of the FCP page ("从固定环到自由拓扑：FCP到底在
// 解决什么", §3.3): the local queries are cut into blocks, and for every key
// block the scores are formed, the running row maximum is raised if needed,
// the accumulator and running sum are rescaled by exp(old max - new max), and
// exp(score - max) is accumulated into both. Masking is causal by global
// position (zig-zag page "大模型长上下文训练的挑战与突破", §4.2; PCP page
// "大模型长序列显存优化：PCP与DCP序列并行实战指南", §3.5) and optionally limited to
// the query's own document; query heads share KV heads as in the Halo page's
// GQA support ("长上下文训练 256k 不难", Ulysses section).
//
// gfx950 design (not taken from the pages, which give no kernel):
//  * A workgroup is 8 wave64s in two groups of four; wave w runs on SIMD
//    w % 4, so each SIMD holds one wave of each group. Each wave owns 32 query
//    rows of one head; the workgroup owns 256 rows of one head, or 32..128
//    rows of 8..2 heads that share a KV head, so every K/V tile staged in LDS
//    feeds 256 (row, head) pairs.
//  * Ping-pong: the two groups alternate, barrier by barrier, between a
//    matrix phase (P V of tile t, then the scores of tile t+1, on the matrix
//    cores) and a vector phase (mask, row max, rescale, exp, row sum, bf16
//    pack of the next tile's scores). While one group's wave on a SIMD issues
//    MFMAs, the other group's wave on that SIMD does the softmax, so the
//    softmax costs little beyond the MFMA time. The matrix-phase wave runs at
//    raised priority (s_setprio) so its MFMAs are not held back.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator then holds, in each lane, 16
//    keys of ONE query row (lane % 32), so row max and row sum are in-lane
//    plus one v_permlane32_swap between the half-waves, and the same
//    registers, rounded to bf16, are directly the B operand of O^T = V^T P^T.
//    O^T keeps each lane on one query row too, so the rescale is a per-lane
//    scalar multiply. Q stays in registers for the whole call.
//  * K and V tiles (64 keys at d 128, 128 at d 64: the same bytes) and the
//    tile's key positions live in a ring of
//    four LDS stages, each its own LDS array. The first load groups go
//    global -> LDS with buffer_load_dwordx4 ... lds; in steady state each
//    iteration fetches the next group into registers (16-byte buffer loads
//    whose range check zero-fills rows past the block) and its matrix phase
//    ends by writing it to LDS, because direct-to-LDS loads stall issue once
//    a handful per CU are in flight. Tiles are row-major with an XOR swizzle
//    of 16-byte chunks; K is read with ds_read_b128 (rows = MFMA rows), V with
//    ds_read_b64_tr_b16, which hands each lane four consecutive keys of one
//    column — the V^T operand layout.
//  * Softmax runs in base 2 with the scale folded into one FMA per score.
//    The scores are exponentiated against the running max as it stands; no
//    row max is formed unless a lane's sum of the tile's probabilities
//    exceeds a bound (a new maximum) or a row has seen no key yet. Then the
//    tile's max is formed, the running max raised if the tile's exceeds it by
//    more than 2^8, and the exponentials taken again, so the O rescale is
//    rare (the final normalisation uses the same stale max, so the result is
//    unchanged).
//  * The operands of a matrix phase (V^T for P V, then K for the next
//    scores) are read from LDS as one stream a few MFMAs ahead, and the first
//    few are read at the end of the vector phase before it, so the matrix
//    cores do not wait for LDS at the start of a phase or between its two
//    products.
//  * The workgroup loads only the key range its rows can see; each wave masks
//    only tiles it does not see in full (tiles it cannot see at all are
//    computed and fully masked: within a workgroup's range that is at most a
//    tile or two per wave near a diagonal or a document start).
//  * Workgroup start is latency-bound (a few dependent memory round trips
//    before the first MFMA), so it is kept short: a workgroup that cannot see
//    the block is recognised from its first key alone and, when
//    accumulating, leaves at once (the merge would not change its state);
//    the key-range bounds are found by the whole wave, 64 probes per round,
//    the workgroup's and the wave's in the same rounds; and without
//    documents Q and the first three tiles are requested before the searches.
//  * Heavy (late-position) query tiles are scheduled first. When the head
//    groups split evenly over the 8 XCDs, workgroup ids are remapped so that
//    consecutive logical tiles (same KV head) run on the same XCD and share
//    its L2; otherwise the hardware's round-robin order is kept, so that no
//    XCD gets all the heaviest tiles. A document call may run from a host
//    plan (plan_varlen below): workgroup b then takes its logical tile (each
//    XCD's tiles by decreasing work) and every range its start would search
//    for from record b, and requests Q and its first tiles at once.
//  * A multi-block call (several blocks that have all arrived) runs the same
//    code in a loop over a table of blocks: each block gets its own
//    emptiness test, searches and tile loop, while the running max, running
//    sum and unnormalised O stay in registers, so O is written once.
//  * Float32 inputs use the same skeleton with v_mfma_f32_32x32x2_f32 and
//    32-key tiles.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "device_common.hpp"
#include "kernels.hpp"
#include "tile_io.hpp"

namespace cpattn {

constexpr int kWaves = 8;                 // two groups of four
constexpr int kThreads = kWaves * 64;

template <typename TIn, typename TOut, int D, bool VARLEN, bool MULTI>
__global__ __launch_bounds__(kThreads, 1) void partial_fwd_kernel(PartialParams p, BlockTable bt) {
  using C = Cfg<TIn, D, kWaves>;
  constexpr int NB = C::kNB;
  constexpr int BK = C::kBK;
  constexpr int NDT = C::kNDT;
  constexpr int NQ = C::kNQ;
  constexpr int TB = C::kTileBytes;
  constexpr int NS = 4;  // LDS stages of the K/V/position ring

  // LDS ring: a K tile, a V tile and the K tile's key positions per stage.
  // Every stage is its own array, so the compiler can see that reading one
  // stage does not alias the direct-to-LDS loads filling another and inserts
  // no wait for them (the ring's counted waits order them).
  static_assert(NS == 4, "four LDS stages");
  __shared__ __attribute__((aligned(1024))) char k_s0[TB], k_s1[TB], k_s2[TB], k_s3[TB];
  __shared__ __attribute__((aligned(1024))) char v_s0[TB], v_s1[TB], v_s2[TB], v_s3[TB];
  __shared__ __attribute__((aligned(16))) int32_t p_s0[BK], p_s1[BK], p_s2[BK], p_s3[BK];
  auto kst = [&](auto st) __attribute__((always_inline)) -> char CPATTN_LDS* {
    constexpr int k = decltype(st)::value;
    if constexpr (k == 0) return (char CPATTN_LDS*)k_s0;
    else if constexpr (k == 1) return (char CPATTN_LDS*)k_s1;
    else if constexpr (k == 2) return (char CPATTN_LDS*)k_s2;
    else return (char CPATTN_LDS*)k_s3;
  };
  auto vst = [&](auto st) __attribute__((always_inline)) -> char CPATTN_LDS* {
    constexpr int k = decltype(st)::value;
    if constexpr (k == 0) return (char CPATTN_LDS*)v_s0;
    else if constexpr (k == 1) return (char CPATTN_LDS*)v_s1;
    else if constexpr (k == 2) return (char CPATTN_LDS*)v_s2;
    else return (char CPATTN_LDS*)v_s3;
  };
  auto pst = [&](auto st) __attribute__((always_inline)) -> int32_t CPATTN_LDS* {
    constexpr int k = decltype(st)::value;
    if constexpr (k == 0) return (int32_t CPATTN_LDS*)p_s0;
    else if constexpr (k == 1) return (int32_t CPATTN_LDS*)p_s1;
    else if constexpr (k == 2) return (int32_t CPATTN_LDS*)p_s2;
    else return (int32_t CPATTN_LDS*)p_s3;
  };
  using S0 = std::integral_constant<int, 0>;
  using S1 = std::integral_constant<int, 1>;
  using S2 = std::integral_constant<int, 2>;
  using S3 = std::integral_constant<int, 3>;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool grp1 = wave >= kWaves / 2;   // ping-pong group
  const int g = lane >> 5;                // half-wave
  const int li = lane & 31;               // query row within the wave

  // A planned document call takes its logical tile, key ranges and document
  // starts from its record instead of searching for them (every value that
  // addresses memory is clamped into range: a wrong plan gives wrong
  // results, never an access outside the tensors).
  const int32_t* rec = nullptr;
  if constexpr (VARLEN && !MULTI) rec = p.wg_plan ? p.wg_plan + (int64_t)blockIdx.x * kPlanRec : nullptr;
  const int Lid = rec ? min(max(rec[kPlanTile], 0), p.n_wg - 1) : tile_order(blockIdx.x, p.n_wg, p.n_hgroups);
  const int hgrp = Lid / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (Lid % p.n_qtiles);  // late (heavier) rows first
  const int hsub = wave % p.g_wg, rb = wave / p.g_wg;
  const int h = hgrp * p.g_wg + hsub;
  const int hk = h / (p.hq / p.hkv);

  // row and key indices fit in 32 bits (the host checks lq, lk < 2^31), which
  // keeps the tile bookkeeping on the scalar unit
  const int lq = (int)p.lq;
  const int wg_r0 = qt * 32 * p.r_wg;
  const int wg_r1 = min(wg_r0 + 32 * p.r_wg, lq);
  const int r0 = wg_r0 + 32 * rb;
  const int r1 = min(r0 + 32, lq);
  const bool wave_active = r0 < lq;

  const int qi = min(r0 + li, lq - 1);     // this lane's query row (clamped)
  const bool row_valid = wave_active && (r0 + li < lq);

  const int64_t kv_stride = (int64_t)p.hkv * D * sizeof(TIn);
  const int kvoff = lane_voff<TIn, D, false, kWaves>(wave, lane, kv_stride);
  const int vvoff = lane_voff<TIn, D, true, kWaves>(wave, lane, kv_stride);

  // ---- the block being folded in ----
  // A single-block call folds in p's block; a multi-block call the blocks of
  // the table one after the other, with the running state kept in registers
  // between them. These are set at the top of each block.
  const void* kraw = p.k;                 // the block's key tensor
  const char* kbase = nullptr;            // its K and V rows of this KV head
  const char* vbase = nullptr;
  const int32_t* kpos = p.k_pos;          // its key positions
  int lk = 0;                             // its keys
  int kt_begin = 0, nt = 0;               // the workgroup's first tile and tile count
  int f_lo = 0, f_hi = 0;                 // keys every row of this wave sees
  auto set_block = [&](int blk) __attribute__((always_inline)) {
    const void* vraw = p.v;
    lk = (int)p.lk;
    if constexpr (MULTI) {
      kraw = bt.k[blk];
      vraw = bt.v[blk];
      kpos = bt.k_pos[blk];
      lk = bt.lk[blk];
    }
    kbase = (const char*)kraw + (int64_t)hk * D * sizeof(TIn);
    vbase = (const char*)vraw + (int64_t)hk * D * sizeof(TIn);
  };

  // Q operand (B of S^T = K Q^T), resident in registers for the whole call,
  // loaded once, with the first block the workgroup sees anything of.
  typedef typename std::conditional<C::kBf16, bf16x8_t, float>::type QReg;
  QReg qreg[NQ];
  bool q_loaded = false;
  auto load_q = [&]() __attribute__((always_inline)) {
    if (q_loaded) return;
    const TIn* qrow = (const TIn*)p.q + ((int64_t)qi * p.hq + h) * D;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      if constexpr (C::kBf16) qreg[ks] = *(const bf16x8_t*)(qrow + 16 * ks + 8 * g);
      else qreg[ks] = qrow[2 * ks + g];
    }
    q_loaded = true;
  };
  // G(-1) = {K(0)}, G(0) = {K(1), V(0)}, G(1) = {K(2), V(1)} of the tiles
  // from kt0 on, straight to LDS; n_avail = tiles that exist from kt0
  auto load_first = [&](int kt0, int n_avail) __attribute__((always_inline)) {
    const int32_t* psrc = p.causal ? kpos : (const int32_t*)kraw;
    load_tile<TIn, D, false, kWaves>(kst(S0{}), kbase, kv_stride, kt0 * BK, lk, wave, lane, kvoff);
    load_positions<kWaves, BK>(pst(S0{}), psrc, kt0 * BK, lk, wave, lane);
    if (1 < n_avail) {
      load_tile<TIn, D, false, kWaves>(kst(S1{}), kbase, kv_stride, (kt0 + 1) * BK, lk, wave, lane, kvoff);
      load_positions<kWaves, BK>(pst(S1{}), psrc, (kt0 + 1) * BK, lk, wave, lane);
    }
    load_tile<TIn, D, true, kWaves>(vst(S0{}), vbase, kv_stride, kt0 * BK, lk, wave, lane, vvoff);
    if (2 < n_avail) {
      load_tile<TIn, D, false, kWaves>(kst(S2{}), kbase, kv_stride, (kt0 + 2) * BK, lk, wave, lane, kvoff);
      load_positions<kWaves, BK>(pst(S2{}), psrc, (kt0 + 2) * BK, lk, wave, lane);
    }
    if (1 < n_avail)
      load_tile<TIn, D, true, kWaves>(vst(S1{}), vbase, kv_stride, (kt0 + 1) * BK, lk, wave, lane, vvoff);
  };

  const int32_t my_qpos = p.causal ? p.q_pos[qi] : 0;
  // A single-block call's first and last key, read with the first loads (the
  // emptiness test and the search shortcuts below use them).
  const int32_t k_first0 = (!MULTI && p.causal && p.lk > 0 && !rec) ? p.k_pos[0] : 0;
  const int32_t k_last0 = (!MULTI && p.causal && p.lk > 0 && !rec) ? p.k_pos[p.lk - 1] : 0;
  // Documents (the same for every block): the starts of the documents of the
  // workgroup's first row and of the wave's last row, and this lane's own. The
  // three document indices are searched together; when the wave's first and
  // last rows share a document (nearly always) every lane's start is that
  // document's; when they lie in adjacent documents a lane's start is the
  // last row's document start if its position has reached it, else the first
  // row's (rows ascend); only a wave across three or more documents searches
  // per lane.
  int32_t s_wg = 0, s_wave = 0, my_start = 0;
  if constexpr (VARLEN) {
    if (rec) {
      s_wave = rec[kPlanSLast + wave];
      const int32_t s_first = rec[kPlanSFirst + wave];
      my_start = (rec[kPlanFlags + wave] & 1) ? doc_start(p.cu_seqlens, p.n_seqs, my_qpos)
                                              : (my_qpos >= s_wave ? s_wave : s_first);
    } else if (p.causal) {
      const int32_t wq_lo = p.q_pos[wg_r0];
      const int32_t q_first = wave_active ? p.q_pos[r0] : p.q_pos[wg_r1 - 1];
      const int32_t q_last = wave_active ? p.q_pos[r1 - 1] : p.q_pos[wg_r1 - 1];
      int d[3];
      const int32_t* const cus[3] = {p.cu_seqlens, p.cu_seqlens, p.cu_seqlens};
      const int ns[3] = {p.n_seqs + 1, p.n_seqs + 1, p.n_seqs + 1};
      const int32_t xs[3] = {wq_lo, q_first, q_last};
      wave_upper_bounds<3>(cus, ns, xs, d);
      s_wg = p.cu_seqlens[d[0] > 0 ? d[0] - 1 : 0];
      s_wave = p.cu_seqlens[d[2] > 0 ? d[2] - 1 : 0];
      const int32_t s_first = p.cu_seqlens[d[1] > 0 ? d[1] - 1 : 0];
      my_start = d[1] == d[2]       ? s_wave
                 : d[2] == d[1] + 1 ? (my_qpos >= s_wave ? s_wave : s_first)
                                    : doc_start(p.cu_seqlens, p.n_seqs, my_qpos);
    }
  }

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = neg_inf();  // running max of scale*log2(e)*score (may lag the true max by < kTau)
  float l_run = 0.f;        // this lane's share of the running sum

  // ---- loads: group G(t) = {K(t+1) and its positions, V(t)}; tile t lives in stage t % NS ----
  // steady state: G(j) is fetched into registers ahead, then committed to its stages.
  // With d = 64 a tile's period is half as long, too short to cover the load
  // latency of a key range that streams from memory, and registers are to
  // spare: G(j) is then fetched two periods ahead into staging set j % 2.
  constexpr bool kDeep = false;
  constexpr int NSET = kDeep ? 2 : 1;
  u32x4_t kreg[NSET][C::kInst / kWaves], vreg[NSET][C::kInst / kWaves];
  int32_t preg[NSET] = {};
  // Rows past `lim` read nothing (zeros). The one-ahead fetch is issued only
  // for j < nt (for j = nt-1 the K part is past the range: zeros written to a
  // free stage); the two-ahead fetch is unconditional, so that the compiler's
  // count of loads in flight is the same on every path, and is all zeros for
  // groups past the workgroup's tiles.
  auto fetch_group = [&](int j, auto set) __attribute__((always_inline)) {
    constexpr int e = decltype(set)::value;
    const int j0 = (kt_begin + j) * BK;
    const int klim = (!kDeep || j + 1 < nt) ? lk : 0, vlim = (!kDeep || j < nt) ? lk : 0;
    fetch_tile<TIn, D, kWaves>(kreg[e], kbase, (int)kv_stride, j0 + BK, klim, wave, kvoff);
    preg[e] = fetch_positions<kWaves, BK>(p.causal ? kpos : nullptr, j0 + BK, klim, wave, lane);
    fetch_tile<TIn, D, kWaves>(vreg[e], vbase, (int)kv_stride, j0, vlim, wave, vvoff);
  };
  auto commit_group = [&](auto sk1, auto sv, auto set) __attribute__((always_inline)) {
    constexpr int e = decltype(set)::value;
    commit_tile<TIn, D, kWaves>(kst(sk1), kreg[e], wave, lane);
    commit_positions<kWaves, BK>(pst(sk1), preg[e], wave, lane);
    commit_tile<TIn, D, kWaves>(vst(sv), vreg[e], wave, lane);
  };

  // does every row of this wave see every key of tile t?
  auto tile_full = [&](int t) __attribute__((always_inline)) {
    const int j0 = (kt_begin + t) * BK;
    return j0 >= f_lo && j0 + BK <= f_hi;
  };

  // LDS byte offsets of this lane's MFMA operands (tile-relative, bf16).
  // K (A of S^T): row li of 32-key block jb, 16-byte chunk 2ks + g.
  // V^T (A of O^T): transposed 8-byte reads; row 32jb + 16h + vr (+8), column block dt.
  int kaddr[C::kBf16 ? NQ : 1];
  int vaddr[C::kBf16 ? NDT : 1];
  if constexpr (C::kBf16) {
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) kaddr[ks] = C::off_k(li, 2 * ks + g);
    const int vr = 4 * g + ((lane & 15) >> 2);              // row within a 16-key group
    const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column within a 32-column block
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const int col = 32 * dt + vc;
      vaddr[dt] = C::off_v(vr, col >> 3) + ((col & 7) << 1);
    }
  }

  f32x16_t sacc[NB];        // scores of the tile in flight (S^T, one query row per lane)
  uint32_t pk[NB][8];       // its probabilities packed to bf16 pairs (bf16 path)

  // ---- matrix phase pieces ----
  // The operand reads are software-pipelined by hand, RING_* operands ahead of
  // the MFMA that consumes them, and fenced with sched_barrier so that the
  // compiler keeps that order (left alone it reads each operand right before
  // its MFMA and waits out the LDS latency every time).
  constexpr int RING_K = 4;   // K operands in flight
  constexpr int RING_V = 4;   // V^T operands in flight
  // S^T = K Q^T for one tile: NQ*NB MFMAs.
  auto qk_tile = [&](const char CPATTN_LDS* kl) __attribute__((always_inline)) {
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) sacc[jb] = f32x16_t{};
    if constexpr (C::kBf16) {
      constexpr int NM = NQ * NB;
      auto rd = [&](int s) __attribute__((always_inline)) {
        return *(const bf16x8_t CPATTN_LDS*)(kl + kaddr[s / NB] + (s % NB) * 32 * C::kRowBytes);
      };
      bf16x8_t ka[RING_K];
#pragma unroll
      for (int s = 0; s < RING_K; ++s) ka[s] = rd(s);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int s = 0; s < NM; ++s) {
        sacc[s % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s % RING_K], qreg[s / NB], sacc[s % NB], 0, 0, 0);
        if (s + RING_K < NM) ka[s % RING_K] = rd(s + RING_K);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        const int d = 2 * ks + g;
        float a = *(const float CPATTN_LDS*)(kl + C::off_k(li, d >> 2) + ((d & 3) << 2));
        sacc[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qreg[ks], sacc[0], 0, 0, 0);
      }
    }
  };

  // O^T += V^T P^T for one tile.
  auto pv_tile = [&](const char CPATTN_LDS* vl) __attribute__((always_inline)) {
    if constexpr (C::kBf16) {
      constexpr int NM = 2 * NB * NDT;
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      // V^T operand of MFMA m = (jb, hf, dt): keys 32jb + 16hf + vr (and + 8), column block dt
      auto rd = [&](int m) __attribute__((always_inline)) {
        const int jb = m / (2 * NDT), hf = (m / NDT) % 2, dt = m % NDT;
        const int roff = (32 * jb + 16 * hf) * C::kRowBytes;
        i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t CPATTN_LDS*)(vl + vaddr[dt] + roff));
        i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (i16x4_t CPATTN_LDS*)(vl + vaddr[dt] + roff + 8 * C::kRowBytes));
        return __builtin_bit_cast(bf16x8_t, (i16x8)__builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      bf16x8_t va[RING_V];
#pragma unroll
      for (int m = 0; m < RING_V; ++m) va[m] = rd(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int jb = m / (2 * NDT), hf = (m / NDT) % 2, dt = m % NDT;
        const u32x4 bw = {pk[jb][4 * hf], pk[jb][4 * hf + 1], pk[jb][4 * hf + 2], pk[jb][4 * hf + 3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[m % RING_V], __builtin_bit_cast(bf16x8_t, bw), oacc[dt],
                                                           0, 0, 0);
        if (m + RING_V < NM) va[m % RING_V] = rd(m + RING_V);
        __builtin_amdgcn_sched_barrier(0);
      }
    } else {
      // float32: P stays in the score registers (already exponentiated)
#pragma unroll
      for (int ks = 0; ks < 16; ++ks) {
        const int row = 8 * (ks >> 2) + 4 * g + (ks & 3);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const int col = 32 * dt + li;
          float a = *(const float CPATTN_LDS*)(vl + C::off_v(row, col >> 2) + ((col & 3) << 2));
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, sacc[0][ks], oacc[dt], 0, 0, 0);
        }
      }
    }
  };

  // ---- bf16 matrix step: one operand stream over P V (tile t) then Q K^T (tile t+1) ----
  // The MFMAs of a matrix step read one operand each from LDS (V^T for P V,
  // K for Q K^T). They are read as a single stream, RING operands ahead of
  // the MFMA that uses them, so the first K operands are already in flight
  // while the last P V MFMAs run, and the first RING operands of a step are
  // read at the end of the vector step before it (its V tile was published
  // two barriers earlier), so the matrix cores do not wait for LDS at the
  // start of a step either.
  constexpr int RING = 6;
  constexpr int NPV = 2 * NB * NDT;       // MFMAs of P V per tile
  constexpr int NQK = NQ * NB;            // MFMAs of Q K^T per tile
  static_assert(!C::kBf16 || RING <= NPV, "the prefetched operands are V^T operands");
  bf16x8_t ring[RING];
  // operand u of a step: u < NPV: V^T block (jb, hf, dt) = keys 32jb + 16hf + vr (and + 8),
  // column block dt; otherwise K block s = u - NPV (row li of 32-key block s % NB, chunk 2(s / NB) + g)
  auto rd_op = [&](int u, const char CPATTN_LDS* vl, const char CPATTN_LDS* kl) __attribute__((always_inline)) {
    if constexpr (!C::kBf16) return bf16x8_t{};
    if (u < NPV) {
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const int jb = u / (2 * NDT), hf = (u / NDT) % 2, dt = u % NDT;
      const int roff = (32 * jb + 16 * hf) * C::kRowBytes;
      i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t CPATTN_LDS*)(vl + vaddr[dt] + roff));
      i16x4_t t1 =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t CPATTN_LDS*)(vl + vaddr[dt] + roff + 8 * C::kRowBytes));
      return __builtin_bit_cast(bf16x8_t, (i16x8)__builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    const int s = u - NPV;
    return *(const bf16x8_t CPATTN_LDS*)(kl + kaddr[s / NB] + (s % NB) * 32 * C::kRowBytes);
  };
  // the first RING operands of the next step (its V^T operands), issued before the phase barrier
  auto prefetch_step = [&](const char CPATTN_LDS* vl) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < RING; ++u) ring[u] = rd_op(u, vl, nullptr);
    __builtin_amdgcn_sched_barrier(0);
  };
  // MFMAs u0 .. u1-1 of a step (u0 = 0: P V first; u1 = NPV: no Q K^T; u0 = NPV: Q K^T only).
  // With `primed` the ring already holds operands u0 .. u0+RING-1.
  // `mid` runs after MFMA kMid has been issued (the ring's commit, so that its
  // LDS writes overlap the MFMAs still to come).
  constexpr int kMid = 22;
  auto run_step = [&](const char CPATTN_LDS* vl, const char CPATTN_LDS* kl, auto u0c, auto u1c, bool primed,
                      auto mid) __attribute__((always_inline)) {
    constexpr int u0 = decltype(u0c)::value, u1 = decltype(u1c)::value;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    if (!primed) {
#pragma unroll
      for (int u = u0; u < u0 + RING && u < u1; ++u) ring[(u - u0) % RING] = rd_op(u, vl, kl);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int u = u0; u < u1; ++u) {
      const int slot = (u - u0) % RING;
      if (u < NPV) {
        const int jb = u / (2 * NDT), hf = (u / NDT) % 2, dt = u % NDT;
        const u32x4 bw = {pk[jb][4 * hf], pk[jb][4 * hf + 1], pk[jb][4 * hf + 2], pk[jb][4 * hf + 3]};
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[slot], __builtin_bit_cast(bf16x8_t, bw), oacc[dt], 0,
                                                           0, 0);
      } else if constexpr (C::kBf16) {
        // (the first k-step of each key block starts from zero, so the scores'
        // registers are not live while P V still holds P)
        const int s = u - NPV;
        sacc[s % NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ring[slot], qreg[s / NB],
                                                               s < NB ? f32x16_t{} : sacc[s % NB], 0, 0, 0);
      }
      if (u + RING < u1) ring[slot] = rd_op(u + RING, vl, kl);
      if (u == kMid || (u1 <= kMid && u == u1 - 1)) mid();
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- vector phase: mask, max, rescale, exp, sum, pack of tile t's scores ----
  // Boundary tiles: lane register r of block jb is key 32jb + 8(r/4) + 4g + r%4
  // of the tile. Keys at or past lk and keys the lane's row cannot see get -inf.
  auto mask = [&](const int32_t CPATTN_LDS* kp, int t) __attribute__((always_inline)) {
    const int lim = min(lk - (kt_begin + t) * BK, BK);  // keys of the tile inside the block
    const int go = 4 * g;
    // (key go + jt + c < lim is tested as the constant jt + c < rem: held as
    // a key index per register, the tests' operands take a register each)
    const int rem = lim - go;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int jt = 32 * jb + 8 * rr;
        typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
        i32x4 kv = {0, 0, 0, 0};
        if (p.causal) kv = *(const i32x4 CPATTN_LDS*)(kp + go + jt);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          bool vis = jt + c < rem;
          if (p.causal) {
            vis = vis & (kv[c] <= my_qpos);
            if (VARLEN) vis = vis & (kv[c] >= my_start);
          }
          sacc[jb][4 * rr + c] = vis ? sacc[jb][4 * rr + c] : neg_inf();
        }
      }
  };
  // Raise the running max where tile t's max exceeds it by more than kTau
  // (base 2), rescaling the running sum and O accordingly.
  auto raise_max = [&]() __attribute__((always_inline)) {
    // (opaque start: the two passes would otherwise share one max, which the
    // compiler then forms ahead of the rare branch on every tile. With
    // documents the max is needed often, at every row's document start, and
    // the shared max measured faster there.)
    float mx = neg_inf();
    if constexpr (!VARLEN) pin(mx);
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[jb][r]);
    mx = half_swap_max(mx) * p.scale_log2;
    const bool raise = mx > m_run + kTau;
    if (__builtin_amdgcn_ballot_w64(raise)) {
      const float m_new = raise ? mx : m_run;
      const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;  // m_run = -inf -> 0
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = m_new;
    }
  };
  // exp2(scale*log2(e)*score - m) of the lane's scores: packed to bf16 as the
  // P operand (float32 inputs: written over the scores); returns their sum
  auto exps = [&](float m) __attribute__((always_inline)) -> float {
    float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[jb][r], p.scale_log2, -m));
        const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[jb][r + 1], p.scale_log2, -m));
        ls0 += e0;
        ls1 += e1;
        if constexpr (C::kBf16) {
          pk[jb][r / 2] = pack_bf16x2(e0, e1);
        } else {
          sacc[jb][r] = e0;
          sacc[jb][r + 1] = e1;
        }
      }
    return ls0 + ls1;
  };
  // A lane's partial row sum of a tile (16*NB probabilities) bounds each of
  // them, so a sum of at most 16*NB*2^kTau keeps every probability within
  // 2^(kTau + log2(16*NB)): the running max may then lag the true one by that
  // much, which only scales the accumulator and the sum alike.
  constexpr float kSumLim = 16.0f * NB * (float)(1 << (int)kTau);
  auto softmax_tile = [&](const int32_t CPATTN_LDS* kp, int t) __attribute__((always_inline)) {
    if (!tile_full(t)) mask(kp, t);
    float ls = 0.f;
    if constexpr (C::kBf16) {
      // Common case: exponentiate against the running max as it stands (no
      // row max is formed). If a lane's sum exceeds the bound (a new maximum,
      // or an overflow), or a row has seen no key yet, the wave forms the
      // tile's max, raises the running max and takes the exponentials again
      // (the scores are still in sacc); after a raise the sum is within the
      // bound, so there are at most two passes.
      bool redo = __builtin_amdgcn_ballot_w64(m_run == neg_inf()) != 0;
      for (int pass = 0; pass < 2; ++pass) {
        if (redo) raise_max();
        ls = exps((m_run == neg_inf()) ? 0.f : m_run);
        redo = __builtin_amdgcn_ballot_w64(!(ls <= kSumLim)) != 0;
        if (!redo) break;
      }
    } else {
      raise_max();
      ls = exps((m_run == neg_inf()) ? 0.f : m_run);
    }
    l_run += ls;
    // the vector phase's results exist before the barrier that follows it
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      if constexpr (C::kBf16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pin(pk[jb][i]);
      } else {
        pin(sacc[jb]);
      }
    }
    pin(l_run);
  };

  // ---- ping-pong schedule ----
  // Every wave runs the same program: for each tile t, the vector step of t,
  // a barrier, the matrix step of t (P V of t, scores of t+1), a barrier.
  // Group 1 starts one barrier later than group 0 (and group 0 ends with one
  // more), so at every phase one group is in its matrix step and the other
  // in its vector step. Tile j's K, positions and V live in stage j % NS.
  // Load group G(j) = {K(j+1), its positions, V(j)}. Iteration t fetches
  // G(t+2) into registers as it starts, and its matrix step ends by
  // committing them to the stages of K(t-1) and V(t-2), which every wave has
  // finished with by then in either group's phase offset. The barrier that
  // follows publishes the commit; its first readers (the matrix step of t+2,
  // the vector step of t+3) are at least one more barrier away for both
  // groups.
  using U0 = std::integral_constant<int, 0>;
  using UPV = std::integral_constant<int, NPV>;
  using UPQ = std::integral_constant<int, NPV + NQK>;
  // (`last`: tile t is the workgroup's last, so the step has no scores to form)
  auto iteration = [&](int t, auto sk, auto last) __attribute__((always_inline)) {
    constexpr int k = decltype(sk)::value;
    constexpr bool LAST = decltype(last)::value;
    const std::integral_constant<int, (k + 1) % NS> sn{};
    const std::integral_constant<int, (k + 2) % NS> s2{};
    const std::integral_constant<int, (k + 3) % NS> s3{};
    if constexpr (kDeep) {
      // fetch G(t+3) into set (t+3) % 2, commit G(t+2) from set (t+2) % 2
      // (t = k mod 4, so the parities are compile-time constants)
      fetch_group(t + 3, std::integral_constant<int, (k + 3) & 1>{});
      softmax_tile(pst(sk), t);
      prefetch_step(vst(sk));
      phase_barrier_reads();
      __builtin_amdgcn_s_setprio(1);
      // (the commit, zeros past the tiles, goes into free stages mid-step)
      auto mid = [&]() __attribute__((always_inline)) {
        commit_group(s3, s2, std::integral_constant<int, (k + 2) & 1>{});
      };
      if constexpr (LAST) run_step(vst(sk), kst(sn), U0{}, UPV{}, true, mid);
      else run_step(vst(sk), kst(sn), U0{}, UPQ{}, true, mid);
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
    } else {
      const std::integral_constant<int, 0> set0{};
      if (t + 2 < nt) fetch_group(t + 2, set0);
      softmax_tile(pst(sk), t);
      if constexpr (C::kBf16) {
        prefetch_step(vst(sk));
        phase_barrier_reads();
        __builtin_amdgcn_s_setprio(1);
        // the commit of G(t+2) (stages every wave has finished with) mid-step
        auto mid = [&]() __attribute__((always_inline)) {
          if (t + 2 < nt) commit_group(s3, s2, set0);
        };
        if constexpr (LAST) run_step(vst(sk), kst(sn), U0{}, UPV{}, true, mid);
        else run_step(vst(sk), kst(sn), U0{}, UPQ{}, true, mid);
      } else {
        phase_barrier();
        __builtin_amdgcn_s_setprio(1);
        pv_tile(vst(sk));
        if constexpr (!LAST) qk_tile(kst(sn));
        if (t + 2 < nt) commit_group(s3, s2, set0);
      }
      // Nothing is in flight here (the commit waited for its loads). Saying so
      // unconditionally keeps the compiler's wait analysis exact across the
      // conditional fetch/commit pair: otherwise it assumes the staging
      // registers may still be loading at the next fetch and waits there for
      // every load just issued.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      __builtin_amdgcn_s_setprio(0);
      phase_barrier();
    }
  };

  bool seen = false;  // the workgroup saw some key of some block
  for (int blk = 0; blk < (MULTI ? bt.n : 1); ++blk) {
    set_block(blk);
    // Rows that see none of a block's keys: when accumulating, a single-block
    // call leaves the state exactly as it is (the merge weights would be 1
    // and 0), so the workgroup stops here; otherwise the block is skipped.
    // Keys all after the workgroup's last query is the common case, decided
    // by one load before any search (the block's last key, read with it,
    // spares the searches below when the rows see the whole block).
    const int32_t k_first = MULTI ? ((p.causal && lk > 0) ? kpos[0] : 0) : k_first0;
    const int32_t k_last = MULTI ? ((p.causal && lk > 0) ? kpos[lk - 1] : 0) : k_last0;
    // (planned: the record's key range, empty when the rows see nothing)
    const int p_kb = rec ? min(max(rec[kPlanKb], 0), lk) : 0;
    const int p_ke = rec ? min(max(rec[kPlanKe], 0), lk) : 0;
    const bool none = rec ? !(p_ke > p_kb) : p.causal && (lk == 0 || k_first > p.q_pos[wg_r1 - 1]);
    if (none || lk <= 0) {
      if (!MULTI && p.accumulate) return;
      continue;
    }
    // Q and, without documents, the first K/V tiles (the workgroup's keys
    // then start at key 0) are requested before the key-range searches,
    // which run under their latency.
    load_q();
    const bool early = !VARLEN || rec;
    // (tiles past the workgroup's range go unread)
    if (early) load_first(p_kb / BK, rec ? (p_ke + BK - 1) / BK - p_kb / BK : (lk + BK - 1) / BK);

    // ---- key range of the workgroup, and the per-wave fully visible range ----
    // (wave-cooperative searches: the positions are ascending, and a lower
    // bound of x is the upper bound of x - 1; document starts are > INT32_MIN).
    // A search whose answer the block's first or last key already gives runs
    // over an empty range: rows at or after the block's last key see all of
    // it (the common case away from the diagonal), and a block whose first key
    // is at or after a document start has no key before it.
    int kb = 0, ke = lk;
    f_lo = 0;
    f_hi = lk;
    if (rec) {
      kb = p_kb;
      ke = p_ke;
      f_lo = min(max(rec[kPlanFLo + wave], 0), lk);
      f_hi = min(max(rec[kPlanFHi + wave], 0), lk);
    } else if (p.causal) {
      // (an inactive wave, past the last row, searches with its workgroup's last row)
      const int32_t wq_hi = p.q_pos[wg_r1 - 1];
      const int32_t q_lo = wave_active ? p.q_pos[r0] : wq_hi;
      const bool all_wg = k_last <= wq_hi, all_wave = k_last <= q_lo;  // (q_lo <= wq_hi)
      if constexpr (VARLEN) {
        // both ends of both ranges in the same rounds (the document starts are known)
        int r[4];
        const int32_t* const ks[4] = {kpos, kpos, kpos, kpos};
        const int ns[4] = {all_wg ? 0 : lk, all_wave ? 0 : lk, k_first >= s_wg ? 0 : lk, k_first >= s_wave ? 0 : lk};
        const int32_t xs[4] = {wq_hi, q_lo, s_wg - 1, s_wave - 1};
        wave_upper_bounds<4>(ks, ns, xs, r);
        ke = all_wg ? lk : r[0];
        f_hi = all_wave ? lk : r[1];
        kb = r[2];
        f_lo = r[3];
      } else if (!all_wave) {
        if (all_wg) f_hi = wave_upper_bound(kpos, lk, q_lo);
        else wave_upper_bound2(kpos, lk, wq_hi, q_lo, ke, f_hi);
      }
    }
    kt_begin = kb / BK;
    // tiles this workgroup loads (>= 1 without documents; none when its rows'
    // documents hold no key of the block, even off a tile boundary)
    nt = ke > kb ? (ke + BK - 1) / BK - kt_begin : 0;
    if (nt <= 0) {
      // (with documents the rows may still see nothing; tiles are loaded early
      // only without documents, but never leave with loads into LDS in flight)
      if (early) __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      continue;
    }
    seen = true;
    if (!early) load_first(kt_begin, nt);
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    phase_barrier();
    if constexpr (kDeep) fetch_group(2, std::integral_constant<int, 0>{});  // G(2), committed in iteration 0
    if constexpr (C::kBf16) run_step(vst(S0{}), kst(S0{}), UPV{}, UPQ{}, false, []() {});
    else qk_tile(kst(S0{}));
    if (grp1) phase_barrier();
    // tiles followed by another, then the last one (peeled, so that the
    // loop's matrix steps all have the same shape; a multi-block call runs
    // every tile through the loop instead, forming scores of a stale stage
    // after its last tile, which its registers cannot otherwise afford)
    using More = std::false_type;
    using Last = std::true_type;
    // (at d 64 the peeled copy of the step costs more registers than the
    // stale scores it saves: every tile goes through the loop there as well)
    constexpr bool kPeel = !MULTI && D != 64;
    const int nmore = kPeel ? nt - 1 : nt;
    for (int t = 0; t < nmore; t += NS) {
      iteration(t, S0{}, More{});
      if (t + 1 < nmore) iteration(t + 1, S1{}, More{});
      if (t + 2 < nmore) iteration(t + 2, S2{}, More{});
      if (t + 3 < nmore) iteration(t + 3, S3{}, More{});
    }
    if constexpr (kPeel)
    switch (nmore & 3) {
      case 0: iteration(nmore, S0{}, Last{}); break;
      case 1: iteration(nmore, S1{}, Last{}); break;
      case 2: iteration(nmore, S2{}, Last{}); break;
      default: iteration(nmore, S3{}, Last{}); break;
    }
    // (after this barrier no wave reads the ring, so the next block may refill it)
    if (!grp1) phase_barrier();
  }
  if (!seen && p.accumulate) return;

  // ---- finalise: O = acc / l, LSE = ln(l) + max; merge into the stored state if accumulating ----
  const float l_tot = half_swap_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv_l = empty ? 0.f : 1.0f / l_tot;
  const float lse_blk = empty ? neg_inf() : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;

  float w_old = 0.f, w_blk = 1.f, lse_out = lse_blk;
  float* lse_ptr = p.lse + (int64_t)h * lq + (r0 + li);
  // (the stored LSE is requested here and the stored O rows below before the
  // merge weights are formed, so the two reads share one round trip)
  const float lse_old = (p.accumulate && row_valid) ? *lse_ptr : neg_inf();
  if constexpr (sizeof(TOut) == 2) {
    // bf16 O goes out through LDS, which no wave reads any more: each lane
    // holds 4-column pieces of one row, so writing them straight out would
    // cover each 128-byte line of O with eight partial writes; staged as
    // rows, every store instruction writes whole lines (16 bytes a lane, the
    // lanes of a row side by side). Each wave stages its own 32 rows in one
    // stage array (row stride padded by 16 bytes against bank conflicts);
    // LDS operations of one wave complete in order.
    constexpr int RS = D * 2 + 16;           // staged row stride (bytes)
    constexpr int CH = D * 2 / 16;           // 16-byte chunks per row
    constexpr int RPP = 64 / CH;             // rows per pass of the wave
    static_assert(32 * RS <= TB, "a wave's rows fit in one stage array");
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    char CPATTN_LDS* stg = wave < 4 ? (wave == 0 ? kst(S0{}) : wave == 1 ? kst(S1{}) : wave == 2 ? kst(S2{}) : kst(S3{}))
                                    : (wave == 4 ? vst(S0{}) : wave == 5 ? vst(S1{}) : wave == 6 ? vst(S2{}) : vst(S3{}));
    TOut* obase = (TOut*)p.o + ((int64_t)r0 * p.hq + h) * D;  // row r0 of this wave's head
    const int64_t ostride = (int64_t)p.hq * D;                 // elements from one row to the next
    const int n_rows = wave_active ? min(32, lq - r0) : 0;
    const int prow = lane / CH, pchunk = lane % CH;            // this lane's place in a pass
    if (p.accumulate) {
      u32x4 orow[32 / RPP];
#pragma unroll
      for (int pass = 0; pass < 32 / RPP; ++pass) {
        const int row = pass * RPP + prow;
        orow[pass] = row < n_rows ? *(const u32x4*)(obase + row * ostride + pchunk * 8) : u32x4{0u, 0u, 0u, 0u};
      }
      if (row_valid) merge_weights(lse_old, lse_blk, w_old, w_blk, lse_out);
#pragma unroll
      for (int pass = 0; pass < 32 / RPP; ++pass) {
        const int row = pass * RPP + prow;
        if (row < n_rows) *(u32x4 CPATTN_LDS*)(stg + row * RS + pchunk * 16) = orow[pass];
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    }
    const float s_blk = w_blk * inv_l;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int dv = 32 * dt + 8 * rr + 4 * g;
        float v0 = oacc[dt][4 * rr] * s_blk, v1 = oacc[dt][4 * rr + 1] * s_blk;
        float v2 = oacc[dt][4 * rr + 2] * s_blk, v3 = oacc[dt][4 * rr + 3] * s_blk;
        u32x2 CPATTN_LDS* slot = (u32x2 CPATTN_LDS*)(stg + li * RS + dv * 2);
        if (p.accumulate) {
          const u32x2 old = *slot;
          v0 += w_old * bf16_bits_to_f32((uint16_t)(old.x & 0xFFFF));
          v1 += w_old * bf16_bits_to_f32((uint16_t)(old.x >> 16));
          v2 += w_old * bf16_bits_to_f32((uint16_t)(old.y & 0xFFFF));
          v3 += w_old * bf16_bits_to_f32((uint16_t)(old.y >> 16));
        }
        *slot = u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int pass = 0; pass < 32 / RPP; ++pass) {
      const int row = pass * RPP + prow;
      if (row < n_rows)
        *(u32x4*)(obase + row * ostride + pchunk * 8) = *(const u32x4 CPATTN_LDS*)(stg + row * RS + pchunk * 16);
    }
  } else {
    if (p.accumulate && row_valid) merge_weights(lse_old, lse_blk, w_old, w_blk, lse_out);
    const float s_blk = w_blk * inv_l;
    if (row_valid) {
      TOut* orow = (TOut*)p.o + ((int64_t)(r0 + li) * p.hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int dv = 32 * dt + 8 * rr + 4 * g;
          float v0 = oacc[dt][4 * rr] * s_blk, v1 = oacc[dt][4 * rr + 1] * s_blk;
          float v2 = oacc[dt][4 * rr + 2] * s_blk, v3 = oacc[dt][4 * rr + 3] * s_blk;
          float4* dst = (float4*)(orow + dv);
          if (p.accumulate) {
            float4 old = *dst;
            v0 += w_old * old.x; v1 += w_old * old.y; v2 += w_old * old.z; v3 += w_old * old.w;
          }
          *dst = make_float4(v0, v1, v2, v3);
        }
    }
  }
  if (g == 0 && row_valid) *lse_ptr = lse_out;
}

// ---------------------------------------------------------------------------

template <typename TIn, typename TOut, int D>
static hipError_t launch_typed(const PartialParams& p, const BlockTable& bt, bool varlen, bool multi,
                               hipStream_t stream) {
  dim3 grid(p.n_wg), block(kThreads);
  if (multi) {
    if (varlen) hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, true, true>), grid, block, 0, stream, p, bt);
    else hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, false, true>), grid, block, 0, stream, p, bt);
  } else {
    if (varlen) hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, true, false>), grid, block, 0, stream, p, bt);
    else hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, false, false>), grid, block, 0, stream, p, bt);
  }
  return hipGetLastError();
}

// Workgroup geometry: g_wg query heads of one KV group x r_wg blocks of 32
// rows (g_wg * r_wg = kWaves); returns the number of workgroups.
static int64_t set_geometry(PartialParams& p) {
  const int G = p.hq / p.hkv;
  p.g_wg = (G % 8 == 0) ? 8 : (G % 4 == 0) ? 4 : (G % 2 == 0) ? 2 : 1;
  p.r_wg = kWaves / p.g_wg;
  p.n_qtiles = (int32_t)((p.lq + 32 * p.r_wg - 1) / (32 * p.r_wg));
  p.n_hgroups = p.hq / p.g_wg;
  return (int64_t)p.n_qtiles * p.n_hgroups;
}

int64_t partial_workgroups(int64_t lq, int32_t hq, int32_t hkv) {
  PartialParams p{};
  p.lq = lq; p.hq = hq; p.hkv = hkv;
  return set_geometry(p);
}

// Host mirrors of the kernel's searches over ascending int32 arrays.
static int64_t host_upper_bound(const int32_t* a, int64_t n, int32_t x) {
  return std::upper_bound(a, a + n, x) - a;
}
static int64_t host_lower_bound(const int32_t* a, int64_t n, int32_t x) {
  return std::lower_bound(a, a + n, x) - a;
}

void plan_varlen(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk, const int32_t* cu_seqlens,
                 int32_t n_seqs, int32_t hq, int32_t hkv, int in_bf16, int head_dim, int32_t* plan) {
  PartialParams p{};
  p.lq = lq; p.hq = hq; p.hkv = hkv;
  const int64_t n = set_geometry(p);
  const int BK = in_bf16 ? (head_dim == 64 ? Cfg<__bf16, 64, kWaves>::kBK : Cfg<__bf16, 128, kWaves>::kBK)
                         : Cfg<float, 128, kWaves>::kBK;
  // document index (as the kernel's search: offsets <= x) and start of a position
  auto doc_idx = [&](int32_t x) { return host_upper_bound(cu_seqlens, (int64_t)n_seqs + 1, x); };
  auto doc_at = [&](int64_t d) { return cu_seqlens[d > 0 ? d - 1 : 0]; };
  // records by logical tile, then placed at their workgroup ids
  std::vector<int32_t> recs((size_t)n * kPlanRec, 0);
  std::vector<int64_t> work((size_t)n, 0);
  const int32_t k_first = lk > 0 ? k_pos[0] : 0, k_last = lk > 0 ? k_pos[lk - 1] : 0;
  for (int64_t L = 0; L < n; ++L) {
    int32_t* r = &recs[(size_t)L * kPlanRec];
    r[kPlanTile] = (int32_t)L;
    const int64_t qt = p.n_qtiles - 1 - L % p.n_qtiles;
    const int64_t wg_r0 = qt * 32 * p.r_wg, wg_r1 = std::min<int64_t>(wg_r0 + 32 * p.r_wg, lq);
    const int32_t wq_hi = q_pos[wg_r1 - 1];
    for (int w = 0; w < kWaves; ++w) {
      // wave w's rows (the kernel's rb = w / g_wg); an inactive wave uses the
      // workgroup's last row
      const int64_t r0 = wg_r0 + 32 * (w / p.g_wg), r1 = std::min<int64_t>(r0 + 32, lq);
      const bool active = r0 < lq;
      const int32_t q_first = active ? q_pos[r0] : wq_hi, q_last = active ? q_pos[r1 - 1] : wq_hi;
      const int64_t d1 = doc_idx(q_first), d2 = doc_idx(q_last);
      const int32_t s_first = doc_at(d1), s_last = doc_at(d2);
      r[kPlanSFirst + w] = s_first;
      r[kPlanSLast + w] = s_last;
      r[kPlanFlags + w] = d2 > d1 + 1 ? 1 : 0;  // three or more documents: per-lane starts
      // fully visible keys: from the last row's document start to the first row
      r[kPlanFLo + w] = (int32_t)(k_first >= s_last ? 0 : host_lower_bound(k_pos, lk, s_last));
      r[kPlanFHi + w] = (int32_t)(k_last <= q_first ? lk : host_upper_bound(k_pos, lk, q_first));
    }
    // the workgroup's keys: from its first row's document start to its last row
    if (lk == 0 || k_first > wq_hi) continue;  // sees nothing of the block (empty range)
    const int32_t s_wg = doc_at(doc_idx(q_pos[wg_r0]));
    const int64_t kb = k_first >= s_wg ? 0 : host_lower_bound(k_pos, lk, s_wg);
    const int64_t ke = k_last <= wq_hi ? lk : host_upper_bound(k_pos, lk, wq_hi);
    r[kPlanKb] = (int32_t)kb;
    r[kPlanKe] = (int32_t)ke;
    if (ke > kb) work[(size_t)L] = (ke + BK - 1) / BK - kb / BK;
  }
  // Workgroup id b runs on XCD b % 8; each XCD keeps the logical tiles the
  // default order gives it (shared K/V in its L2), heaviest first (longest
  // processing time first: the XCD's CUs then finish close together).
  for (int x = 0; x < 8; ++x) {
    std::vector<int32_t> ls;
    for (int64_t b = x; b < n; b += 8) ls.push_back(tile_order((int)b, (int)n, p.n_hgroups));
    std::stable_sort(ls.begin(), ls.end(), [&](int32_t a, int32_t c) {
      return work[(size_t)a] != work[(size_t)c] ? work[(size_t)a] > work[(size_t)c] : a < c;
    });
    size_t i = 0;
    for (int64_t b = x; b < n; b += 8)
      std::copy_n(&recs[(size_t)ls[i++] * kPlanRec], kPlanRec, plan + b * kPlanRec);
  }
}

static hipError_t launch_any(PartialParams p, const BlockTable& bt, int in_bf16, int out_bf16, int head_dim,
                             bool varlen, bool multi, hipStream_t stream) {
  const int64_t n_wg = set_geometry(p);
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  p.n_wg = (int32_t)n_wg;
  if (multi || !varlen) p.wg_plan = nullptr;
  if (in_bf16) {
    if (head_dim == 128) return out_bf16 ? launch_typed<__bf16, __bf16, 128>(p, bt, varlen, multi, stream)
                                         : launch_typed<__bf16, float, 128>(p, bt, varlen, multi, stream);
    return out_bf16 ? launch_typed<__bf16, __bf16, 64>(p, bt, varlen, multi, stream)
                    : launch_typed<__bf16, float, 64>(p, bt, varlen, multi, stream);
  }
  if (head_dim == 128) return launch_typed<float, float, 128>(p, bt, varlen, multi, stream);
  return launch_typed<float, float, 64>(p, bt, varlen, multi, stream);
}

hipError_t launch_partial(PartialParams p, int in_bf16, int out_bf16, int head_dim, bool varlen, hipStream_t stream) {
  BlockTable bt{};
  bt.n = 1;
  return launch_any(p, bt, in_bf16, out_bf16, head_dim, varlen, false, stream);
}

hipError_t launch_partial_multi(PartialParams p, const BlockTable& bt, int in_bf16, int out_bf16, int head_dim,
                                bool varlen, hipStream_t stream) {
  return launch_any(p, bt, in_bf16, out_bf16, head_dim, varlen, true, stream);
}

}  // namespace cpattn

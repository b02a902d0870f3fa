// partial_bwd.hip — gradients of one KV block's part of a context-parallel
// rank's attention, for gfx950 (MI355X).
//
// Method: training with context parallelism runs the backward pass over the
// same KV blocks as the forward (PCP page "大模型长序列显存优化：PCP与DCP序列并行
// 实战指南", §2.3), with the same global-position masks (§3.5; zig-zag page
// "大模型长上下文训练的挑战与突破", §4.2) and the same GQA head sharing (Halo page
// "长上下文训练 256k 不难", Ulysses section). The pages give no formulas for it;
// these are the gradients of the attention the forward computes. With each
// row's FINAL log-normaliser LSE (after every block was merged) and
// D = <dO, O>, the probabilities of a block's keys are P = exp(s - LSE), and
//     dV = P^T dO,  dP = dO V^T,  dS = P (dP - D),
//     dQ = scale dS K,  dK = scale dS^T Q.
// Because P uses the final LSE, the terms of one block are exactly that
// block's share of the full gradient: dQ is the sum over blocks, and a
// block's dK and dV are complete once every query row has been seen.
//
// gfx950 design (not taken from the pages, which give no kernel):
//  * Two kernels and no atomics. The key kernel: a workgroup of eight waves
//    owns 128 keys of one KV head (32 per producer/consumer pair of waves)
//    and walks the 32-row query tiles that can see them, for every query
//    head that reads that KV head, accumulating dK and dV in registers. The
//    query kernel: a workgroup of four waves owns 128 rows (32 per wave) of
//    one head and walks the 32-key tiles they can see, accumulating dQ (two
//    such workgroups share a CU). Both recompute S and dP (seven matrix
//    products per visible pair instead of five) in exchange for no atomic
//    traffic and run-to-run identical results.
//  * Each wave keeps its own side's operands in registers for the whole
//    call (K and V of its keys, or Q and dO of its rows) and streams the
//    other side through LDS stages (four for the key kernel, two for the
//    query kernel), fetched ahead into registers (16-byte buffer loads; the
//    range check zero-fills rows past the end).
//  * Orientation, with v_mfma_f32_32x32x16_bf16: the key kernel computes
//    S = Q K^T and dP = dO V^T, so each lane holds ONE key and 16 query rows;
//    P and dS, rounded to bf16, are then directly the B operands of
//    dV^T = dO^T P and dK^T = Q^T dS, whose A operands (dO^T, Q^T) are read
//    transposed from LDS with ds_read_b64_tr_b16, and the accumulators keep
//    each lane on its key. The query kernel is the mirror: S^T = K Q^T,
//    dP^T = V dO^T, one query row per lane (its LSE and D are scalars of
//    the lane), and dQ^T = K^T dS^T with K^T read transposed.
//  * Tiles are row-major in LDS with one XOR swizzle of 16-byte chunks that
//    keeps both the row reads (ds_read_b128, 16 rows at one chunk) and the
//    transposed reads (4 rows x 4 chunks) free of bank conflicts.
//  * Workgroup ids are remapped so that consecutive logical tiles run on
//    one XCD (shared L2) when the heads split evenly over the 8 XCDs (else
//    the hardware's round-robin order spreads the heavy tiles); the tiles
//    with the most work go first.
//  * With documents a query tile's work follows its rows' places in their
//    documents, not their positions: a planned call takes the query kernel's
//    order from a host plan (each XCD's tiles, most key tiles first).
//  * Several blocks present at once (MULTI): the key kernel's grid covers
//    every block's workgroups (a workgroup finds its block in a table of
//    running workgroup counts, then runs the per-block code unchanged), and
//    the query kernel's workgroups walk the blocks in order, so dQ stays in
//    the accumulators across them and is stored once.
#include <algorithm>
#include <type_traits>
#include <vector>

#include "device_common.hpp"
#include "kernels_bwd.hpp"
#include "tile_io.hpp"

namespace cpattn {

constexpr int kBwdThreads = 256;  // four waves

template <int D>
struct BwdTile {
  static constexpr int kRowBytes = 2 * D;              // one bf16 row
  static constexpr int kChunks = D / 8;                // 16-byte chunks per row
  static constexpr int kBytes = 32 * kRowBytes;        // a 32-row tile
  static constexpr int kUnits = kBytes / 16 / kBwdThreads;  // 16-byte loads per thread per tile
  static constexpr int kNQ = D / 16;                   // k-steps over the head dimension
  static constexpr int kNDT = D / 32;                  // 32-column blocks of the head dimension
  // chunk ^ swz(row): 16 consecutive rows at one chunk hit 16 distinct
  // 16-byte bank groups, and so do 4 consecutive rows x 4 consecutive chunks
  static constexpr int swz(int row) {
    if constexpr (D == 128) return ((row & 3) << 2) | ((row >> 2) & 3);
    else return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  }
  static constexpr int off(int row, int chunk) { return row * kRowBytes + ((chunk ^ swz(row)) << 4); }
};

// 32 rows of one head of a [n_rows][heads][D] bf16 tensor into registers:
// thread t holds 16-byte units t, t + 256, ... of the tile (row-major);
// rows at or past n_rows read as zeros.
template <int D>
__device__ __forceinline__ void fetch_rows(u32x4_t* regs, const char* head_base, int row_stride, int r0, int n_rows,
                                           int tid) {
  using T = BwdTile<D>;
  const int rows = clamp_rows(n_rows - r0, 32);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head_base + (int64_t)r0 * row_stride, (int64_t)rows * row_stride);
#pragma unroll
  for (int u = 0; u < T::kUnits; ++u) {
    const int unit = tid + kBwdThreads * u;
    regs[u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (unit / T::kChunks) * row_stride + (unit % T::kChunks) * 16,
                                                    0, 0);
  }
}

template <int D>
__device__ __forceinline__ void commit_rows(char CPATTN_LDS* tile, const u32x4_t* regs, int tid) {
  using T = BwdTile<D>;
#pragma unroll
  for (int u = 0; u < T::kUnits; ++u) {
    const int unit = tid + kBwdThreads * u;
    *(u32x4_t CPATTN_LDS*)(tile + T::off(unit / T::kChunks, unit % T::kChunks)) = regs[u];
  }
}

// Transposed operand: for a tile whose rows are the contraction index
// (32 of them) and whose columns are the output rows, the A operand of k-step
// hf (rows 16hf .. 16hf+15) and column block dt. The contraction order matches
// the accumulator layout of the B side: lane half g holds rows 16hf + 4g + 0..3
// and 16hf + 8 + 4g + 0..3. a0/a8 are the lane's byte offsets in rows 0..15
// and 8..23 (the swizzle differs between them).
__device__ __forceinline__ bf16x8_t read_tr(const char CPATTN_LDS* tile, int a0, int a8, int hf, int row_bytes) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t CPATTN_LDS*)(tile + a0 + 16 * hf * row_bytes));
  const i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4_t CPATTN_LDS*)(tile + a8 + 16 * hf * row_bytes));
  return __builtin_bit_cast(bf16x8_t, (i16x8)__builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7));
}

// this lane's transposed-read offsets (see read_tr) for column block dt
template <int D>
__device__ __forceinline__ void tr_offsets(int lane, int dt, int& a0, int& a8) {
  using T = BwdTile<D>;
  const int g = lane >> 5;
  const int vr = 4 * g + ((lane & 15) >> 2);              // row within a 16-row group
  const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  a0 = T::off(vr, col >> 3) + ((col & 7) << 1);
  a8 = T::off(vr + 8, col >> 3) + ((col & 7) << 1);
}

// A wave's 32 rows of float32 results (lane l: row l % 32, head-dimension
// entries 32dt + 8rr + 4(l/32) + 0..3 in acc[dt][4rr .. 4rr+3]), times mul,
// written to rows row0 .. row0+31 of a float32 tensor (row_stride floats
// apart, out pointing at the head's first column) through the LDS array
// stg (32 rows x D/2 floats), so that every store instruction writes whole
// 128-byte lines instead of 32 bytes of each of 32 rows: two passes of half
// the head dimension, 16-byte chunks of row r XORed with r (mod the chunks
// per row) against bank conflicts. Rows at or past n_valid are not written;
// with `add` the stored values are added to.
template <int D>
__device__ __forceinline__ void store_rows_lds(float* out, int64_t row_stride, int row0, int n_valid,
                                               char CPATTN_LDS* stg, const f32x16_t* acc, float mul, bool add,
                                               int lane) {
  constexpr int DTP = D / 64;         // 32-column blocks per pass
  constexpr int PCOLS = 32 * DTP;     // floats of a row per pass
  constexpr int CHK = PCOLS / 4;      // 16-byte chunks of a row per pass
  constexpr int RB = PCOLS * 4;       // staged row bytes
  constexpr int RPI = 64 / CHK;       // rows per read
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int g = lane >> 5, li = lane & 31;
  const int rl = lane / CHK, cl = lane % CHK;
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
#pragma unroll
    for (int dtp = 0; dtp < DTP; ++dtp)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const f32x16_t& a = acc[ps * DTP + dtp];
        const int c = 8 * dtp + 2 * rr + g;
        *(f32x4 CPATTN_LDS*)(stg + li * RB + ((c ^ (li & (CHK - 1))) << 4)) =
            f32x4{a[4 * rr] * mul, a[4 * rr + 1] * mul, a[4 * rr + 2] * mul, a[4 * rr + 3] * mul};
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int row = k * RPI + rl;
      f32x4 v = *(const f32x4 CPATTN_LDS*)(stg + row * RB + ((cl ^ (row & (CHK - 1))) << 4));
      if (row < n_valid) {
        f32x4* dst = (f32x4*)(out + (int64_t)(row0 + row) * row_stride + ps * PCOLS + 4 * cl);
        if (add) v += *dst;
        *dst = v;
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this pass's reads are done before the next one's writes
  }
}

// ---------------------------------------------------------------------------
// Key kernel: dK and dV of 128 keys of one KV head.
//
// Eight waves in producer/consumer pairs: wave i (producer) and wave i + 4
// (consumer) run on the same SIMD and own the same 32 keys. Per phase the
// producer turns S = Q K^T and dP = dO V^T of query tile t (K and V of its
// keys in registers) into P and dS, which it leaves in LDS, while its MFMAs
// already form S and dP of tile t+1;
// the consumer, meanwhile, folds tile t-1's P and dS into dV^T += dO^T P and
// dK^T += Q^T dS (its accumulators in registers). The two roles' register
// sets are disjoint (operands vs accumulators), so each fits beside the
// other on the SIMD, and the consumer's MFMAs run while the producer does
// its vector work. Query tiles pass through four LDS stages (the producer
// reads tiles t and t+1, the consumer tile t-1, tile t+2 is being written).

constexpr int kDkvThreads = 512;   // four producer and four consumer waves

template <int D, bool VARLEN, bool MULTI>
__global__ __launch_bounds__(kDkvThreads, 1) void bwd_dkv_kernel(BwdParams p, BwdBlocks bt) {
  using T = BwdTile<D>;
  constexpr int NQ = T::kNQ, NDT = T::kNDT, TB = T::kBytes;
  constexpr int NS = 4;                     // LDS stages of query tiles
  constexpr int RING = 4;                   // LDS operands in flight
  constexpr int U = TB / 16;                // 16-byte units of one tile
  constexpr int FT = kDkvThreads / 2;       // the consumer waves move the query tiles
  constexpr int NU = 2 * U / FT;            // units of the (Q, dO) pair per consumer thread
  static_assert(NU >= 1 && U % FT == 0, "each tile splits evenly over the consumer threads");
  __shared__ __attribute__((aligned(1024))) char q_s[NS][TB], o_s[NS][TB];
  __shared__ __attribute__((aligned(1024))) char x_s[2][4][4][1024];  // [buffer][key block][part][lane]
  __shared__ __attribute__((aligned(16))) float l_s[NS][32], d_s[NS][32];
  __shared__ __attribute__((aligned(16))) int32_t p_s[NS][32];
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool producer = wave < 4;
  const int kw = wave & 3;                  // the wave's 32-key block
  const int g = lane >> 5, li = lane & 31;
  int bid = blockIdx.x;
  if constexpr (MULTI) {
    // the block whose range of workgroups holds this one (blocks without
    // keys have empty ranges; the grid ends at the last block's end)
    int b = 0;
    while (b + 1 < bt.n && bid >= bt.wg_end[b]) ++b;
    bid -= b ? bt.wg_end[b - 1] : 0;
    p.k = bt.k[b];
    p.v = bt.v[b];
    p.k_pos = bt.k_pos[b];
    p.dk = bt.dk[b];
    p.dv = bt.dv[b];
    p.lk = bt.lk[b];
    p.n_tiles = (p.lk + 127) / 128;
    p.n_wg = p.n_tiles * p.hkv;
  }
  const int L = tile_order(bid, p.n_wg, p.hkv);
  const int hk = L / p.n_tiles;
  const int kt = L % p.n_tiles;  // early keys (seen by the most rows) first
  const int G = p.hq / p.hkv;
  const int lq = p.lq, lk = p.lk;
  const int wg_j0 = kt * 128, wg_j1 = min(wg_j0 + 128, lk);
  const int j0 = wg_j0 + 32 * kw;
  const int kj = min(j0 + li, lk - 1);              // this lane's key (clamped)
  const bool key_valid = j0 + li < lk;

  // rows that see the workgroup's keys
  int i_lo = 0, i_hi = lq;
  if (p.causal) {
    i_lo = wave_upper_bound(p.q_pos, lq, p.k_pos[wg_j0] - 1);
    if constexpr (VARLEN) i_hi = wave_upper_bound(p.q_pos, lq, doc_end(p.cu_seqlens, p.n_seqs, p.k_pos[wg_j1 - 1]) - 1);
  }
  const int nqt = i_hi > i_lo ? (i_hi - i_lo + 31) / 32 : 0;
  const int n_it = G * nqt;

  // ---- query tiles: (head, 32 rows) per iteration, head-major; tile t lives in stage t % 4 ----
  // The consumer waves (whose per-phase work is the lighter) move the tiles:
  // consumer thread c = tid - 256 moves 16-byte units c, c + 256, ... of the
  // pair (Q tile, dO tile); the producers only compute.
  const int ct = tid - FT;
  // Tile t+3 is fetched into registers (set (t+3) % 2) in phase t and written to
  // LDS at the end of phase t+1, so a load has two phases to arrive. The fetch
  // is issued in every phase, reading nothing past the last tile, so that the
  // compiler's count of loads in flight is the same on every path and its wait
  // before a commit covers only the older set.
  const int q_stride = p.hq * D * 2;
  u32x4_t xr[2][NU];
  float lr[2] = {0.f, 0.f}, dr[2] = {0.f, 0.f};
  int32_t pr[2] = {0, 0};
  int nr[2] = {0, 0};  // rows of the fetched tile inside the tensor
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;
  auto fetch = [&](int it, auto set) __attribute__((always_inline)) {
    constexpr int e = decltype(set)::value;
    const bool live = it < n_it;
    const int hh = hk * G + (live ? it / nqt : 0);
    const int i0 = live ? i_lo + 32 * (it % nqt) : lq;
    const int rows = clamp_rows(lq - i0, 32);          // 0 past the last tile: nothing is read
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      // (0 <= ct < FT and FT divides U: the tile of unit ct + FT u is known
      // from u alone, so the buffer base is scalar)
      const bool is_o = FT * u >= U;
      const int lu = ct + FT * u - (is_o ? U : 0);
      const char* base = (const char*)(is_o ? p.dout : p.q) + (int64_t)hh * D * 2 + (int64_t)i0 * q_stride;
      const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (int64_t)rows * q_stride);
      xr[e][u] = __builtin_amdgcn_raw_buffer_load_b128(rs, (lu / T::kChunks) * q_stride + (lu % T::kChunks) * 16,
                                                       0, 0);
    }
    // The rows' LSE, D and positions: lanes 0..31 of wave 4 read them. Every
    // consumer wave issues the same loads (the range is empty elsewhere and they
    // read nothing), so that all have the same loads in flight; row validity and
    // the base-2 conversion are applied at the commit, so nothing waits here.
    const int mine = wave == 4 ? rows : 0;
    nr[e] = rows;
    const int64_t lo = (int64_t)hh * lq + i0;
    lr[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.lse + lo, mine * 4), lane * 4, 0, 0));
    dr[e] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.delta + lo, mine * 4), lane * 4, 0, 0));
    pr[e] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(p.q_pos + i0, p.causal ? mine * 4 : 0), lane * 4, 0, 0);
  };
  auto commit = [&](int st, auto set) __attribute__((always_inline)) {
    constexpr int e = decltype(set)::value;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const bool is_o = FT * u >= U;
      const int lu = ct + FT * u - (is_o ? U : 0);
      char CPATTN_LDS* tile = (char CPATTN_LDS*)(is_o ? o_s[st] : q_s[st]);
      *(u32x4_t CPATTN_LDS*)(tile + T::off(lu / T::kChunks, lu % T::kChunks)) = xr[e][u];
    }
    if (ct >= 0 && ct < 32) {
      // base-2 LSE; rows past the end, or that see nothing, get +inf: P = 0
      const bool ok = ct < nr[e];
      l_s[st][ct] = (!ok || lr[e] == neg_inf()) ? __builtin_inff() : lr[e] * kLog2e;
      d_s[st][ct] = ok ? dr[e] : 0.f;
      p_s[st][ct] = (ok && p.causal) ? pr[e] : (int32_t)0x80000000;
    }
  };

  if (!producer) {
    fetch(0, P0{});
    commit(0, P0{});
    fetch(1, P1{});
    commit(1, P1{});
    fetch(2, P0{});
  }
  phase_barrier();

  if (producer) {
    // ---------------- producer: S, dP -> P, dS ----------------
    bf16x8_t kreg[NQ], vreg[NQ];  // B operands of S = Q K^T and dP = dO V^T
    {
      const int64_t off = ((int64_t)kj * p.hkv + hk) * D + 8 * g;
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        kreg[ks] = *(const bf16x8_t*)((const __bf16*)p.k + off + 16 * ks);
        vreg[ks] = *(const bf16x8_t*)((const __bf16*)p.v + off + 16 * ks);
      }
    }
    // a query row sees key j iff q_pos >= k_pos[j] and, with documents, q_pos < end of k's document
    const int32_t my_kpos = p.causal ? p.k_pos[kj] : 0;
    const int32_t my_kend = VARLEN ? doc_end(p.cu_seqlens, p.n_seqs, my_kpos) : 0;
    int ra[NQ];  // row reads: row li, chunk 2ks + g
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) ra[ks] = T::off(li, 2 * ks + g);
    // S and dP of the tile in stage st (rows: the tile's queries; column: this
    // lane's key), alternating; work(m) runs after MFMA m
    auto sdp = [&](int st, f32x16_t& s, f32x16_t& dp, auto work) __attribute__((always_inline)) {
      constexpr int NM = 2 * NQ;
      const char CPATTN_LDS* ql = (const char CPATTN_LDS*)q_s[st];
      const char CPATTN_LDS* ol = (const char CPATTN_LDS*)o_s[st];
      auto rd = [&](int m) __attribute__((always_inline)) {
        return *(const bf16x8_t CPATTN_LDS*)(((m & 1) ? ol : ql) + ra[m >> 1]);
      };
      bf16x8_t a[RING];
#pragma unroll
      for (int m = 0; m < RING; ++m) a[m] = rd(m);
      s = f32x16_t{};
      dp = f32x16_t{};
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        if (m & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], vreg[m >> 1], dp, 0, 0, 0);
        else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], kreg[m >> 1], s, 0, 0, 0);
        if (m + RING < NM) a[m % RING] = rd(m + RING);
        work(m);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // P = exp(s - LSE) on visible pairs, dS = P (dP - D) of rows 8rr + 4g + 0..3
    // (registers 4rr..4rr+3), packed to bf16 pairs; the rows' LSE, D and
    // positions are read one MFMA before the slice that uses them
    uint32_t pp[8], pd[8];
    f32x4 l4, d4;
    i32x4 q4;
    auto read_rows = [&](int st, int rr) __attribute__((always_inline)) {
      l4 = *(const f32x4 CPATTN_LDS*)((const float CPATTN_LDS*)l_s[st] + 8 * rr + 4 * g);
      d4 = *(const f32x4 CPATTN_LDS*)((const float CPATTN_LDS*)d_s[st] + 8 * rr + 4 * g);
      q4 = p.causal ? *(const i32x4 CPATTN_LDS*)((const int32_t CPATTN_LDS*)p_s[st] + 8 * rr + 4 * g)
                    : i32x4{0, 0, 0, 0};
    };
    // Without documents, a query tile whose first row is at or after the
    // wave's last key sees all of the wave's keys (rows past the end have
    // LSE +inf, so P = 0): no mask then.
    const int32_t wave_klast = __builtin_amdgcn_readfirstlane(p.causal ? p.k_pos[min(j0 + 31, lk - 1)] : 0);
    const bool keys_full = j0 + 32 <= lk;
    auto tile_full = [&](int st) __attribute__((always_inline)) {
      return keys_full &&
             (!p.causal || (!VARLEN && __builtin_amdgcn_readfirstlane(p_s[st][0]) >= wave_klast));
    };
    auto softmax_rr = [&](const f32x16_t& s, const f32x16_t& dp, int rr, auto masked) __attribute__((always_inline)) {
      constexpr bool M = decltype(masked)::value;
      float pv[4], dv[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        bool vis = true;
        if constexpr (M) {
          vis = key_valid;
          if (p.causal) {
            vis = vis & (q4[c] >= my_kpos);
            if (VARLEN) vis = vis & (q4[c] < my_kend);
          }
        }
        pv[c] = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * rr + c], p.scale_log2, -l4[c])) : 0.f;
        dv[c] = pv[c] * (dp[4 * rr + c] - d4[c]);
      }
      pp[2 * rr] = pack_bf16x2(pv[0], pv[1]);
      pp[2 * rr + 1] = pack_bf16x2(pv[2], pv[3]);
      pd[2 * rr] = pack_bf16x2(dv[0], dv[1]);
      pd[2 * rr + 1] = pack_bf16x2(dv[2], dv[3]);
    };
    // Phase k: P, dS of tile k (its S, dP formed in phase k - 1) in four slices
    // placed between the MFMAs of tile k+1's S, dP, so that the wave's vector
    // work overlaps its own matrix work.
    f32x16_t s_c = f32x16_t{}, dp_c = f32x16_t{};
    if (n_it > 0) sdp(0, s_c, dp_c, [](int) {});
    int st = 0;
    // phase k fetches tile k+3 into set fs = (k+3) % 2 and commits tile k+2 from set cs = (k+2) % 2
    auto phase = [&](int k, auto fs, auto cs) __attribute__((always_inline)) {
      (void)fs;
      (void)cs;
      if (k < n_it) {
        const int st1 = (st + 1) & (NS - 1);
        const bool full = tile_full(st);
        auto soft = [&](int rr) __attribute__((always_inline)) {
          if (full) softmax_rr(s_c, dp_c, rr, std::false_type{});
          else softmax_rr(s_c, dp_c, rr, std::true_type{});
        };
        // P, dS go to the stage the consumers read next phase (this phase's
        // consumers read the other one): rows 0-15 (slices 0, 1) and 16-31
        // (slices 2, 3), each half a 16-byte piece of P and one of dS per lane
        char CPATTN_LDS* xb = (char CPATTN_LDS*)x_s[k & 1][kw] + 16 * lane;
        auto put = [&](int h) __attribute__((always_inline)) {
          *(u32x4 CPATTN_LDS*)(xb + 1024 * h) = u32x4{pp[4 * h], pp[4 * h + 1], pp[4 * h + 2], pp[4 * h + 3]};
          *(u32x4 CPATTN_LDS*)(xb + 2048 + 1024 * h) =
              u32x4{pd[4 * h], pd[4 * h + 1], pd[4 * h + 2], pd[4 * h + 3]};
        };
        // At d 128 the first half is written as soon as slice 1 has formed it,
        // under the rest of the products (measured faster there; at d 64, with
        // half the products per phase, slower)
        constexpr bool kEarlyHalf = D == 128;
        if (k + 1 < n_it) {
          constexpr int SP = NQ / 2;  // MFMAs per slice
          static_assert(SP >= 2, "a slice's row reads go one MFMA ahead of it");
          f32x16_t s_n, dp_n;
          sdp(st1, s_n, dp_n, [&](int m) __attribute__((always_inline)) {
            if (m % SP == SP - 2) read_rows(st, m / SP);
            if (m % SP == SP - 1) {
              soft(m / SP);
              if (kEarlyHalf && m / SP == 1) put(0);
            }
          });
          s_c = s_n;
          dp_c = dp_n;
          if (!kEarlyHalf) put(0);
          put(1);
        } else {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            read_rows(st, rr);
            soft(rr);
          }
          put(0);
          put(1);
        }
      }
      phase_barrier();
      st = (st + 1) & (NS - 1);
    };
    for (int k = 0; k <= n_it; k += 2) {
      phase(k, P1{}, P0{});
      if (k + 1 <= n_it) phase(k + 1, P0{}, P1{});
    }
    return;
  }

  // ---------------- consumer: dV^T += dO^T P, dK^T += Q^T dS ----------------
  int ta0[NDT], ta8[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) tr_offsets<D>(lane, dt, ta0[dt], ta8[dt]);
  f32x16_t dk_acc[NDT], dv_acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk_acc[dt] = f32x16_t{};
    dv_acc[dt] = f32x16_t{};
  }
  int st = NS - 1;  // stage of tile k - 1
  auto phase = [&](int k, auto fs, auto cs) __attribute__((always_inline)) {
    fetch(k + 3, fs);
    if (k >= 1) {
      const char CPATTN_LDS* ql = (const char CPATTN_LDS*)q_s[st];
      const char CPATTN_LDS* ol = (const char CPATTN_LDS*)o_s[st];
      const char CPATTN_LDS* xb = (const char CPATTN_LDS*)x_s[(k - 1) & 1][kw] + 16 * lane;
      const u32x4 bp0 = *(const u32x4 CPATTN_LDS*)(xb), bp1 = *(const u32x4 CPATTN_LDS*)(xb + 1024);
      const u32x4 bd0 = *(const u32x4 CPATTN_LDS*)(xb + 2048), bd1 = *(const u32x4 CPATTN_LDS*)(xb + 3072);
      constexpr int NM = 4 * NDT;   // (hf, dt, dv|dk)
      auto rd = [&](int m) __attribute__((always_inline)) {
        const int hf = m / (2 * NDT), dt = (m >> 1) % NDT;
        return read_tr((m & 1) ? ql : ol, ta0[dt], ta8[dt], hf, T::kRowBytes);
      };
      bf16x8_t a[RING];
#pragma unroll
      for (int m = 0; m < RING; ++m) a[m] = rd(m);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int m = 0; m < NM; ++m) {
        const int hf = m / (2 * NDT), dt = (m >> 1) % NDT;
        if (m & 1)
          dk_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], __builtin_bit_cast(bf16x8_t, hf ? bd1 : bd0),
                                                               dk_acc[dt], 0, 0, 0);
        else
          dv_acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], __builtin_bit_cast(bf16x8_t, hf ? bp1 : bp0),
                                                               dv_acc[dt], 0, 0, 0);
        if (m + RING < NM) a[m % RING] = rd(m + RING);
        // the commit of tile k + 2 into stage (k + 2) % 4 (read by nobody since
        // tile k - 2 left it) halfway through the products, so that its LDS
        // writes run under the rest of them and the phase barrier has little to
        // drain; its loads were issued a phase earlier
        if (m == NM / 2 && k + 2 < n_it) commit((st + 3) & (NS - 1), cs);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (k == 0 && k + 2 < n_it) commit((st + 3) & (NS - 1), cs);  // phase 0 has no products; st is (k - 1) % 4
    phase_barrier();
    st = (st + 1) & (NS - 1);
  };
  for (int k = 0; k <= n_it; k += 2) {
    phase(k, P1{}, P0{});
    if (k + 1 <= n_it) phase(k + 1, P0{}, P1{});
  }

  // ---- store: lane li holds key j0 + li, head-dimension entries 32dt + 8rr + 4g + 0..3 ----
  // through the query stages, which no wave reads after the last barrier:
  // consumer c stages dK in q_s[c] and dV in o_s[c]
  const int n_keys = min(32, lk - j0);
  if (n_keys <= 0) return;
  const int cw = wave - 4;
  const int64_t kv_row = (int64_t)p.hkv * D;
  store_rows_lds<D>(p.dk + (int64_t)hk * D, kv_row, j0, n_keys, (char CPATTN_LDS*)q_s[cw], dk_acc, p.scale,
                    p.acc_dkv != 0, lane);
  store_rows_lds<D>(p.dv + (int64_t)hk * D, kv_row, j0, n_keys, (char CPATTN_LDS*)o_s[cw], dv_acc, 1.0f,
                    p.acc_dkv != 0, lane);
}

// ---------------------------------------------------------------------------
// Query kernel: dQ of 128 rows of one query head.

template <int D, bool VARLEN, bool MULTI>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdParams p, BwdBlocks bt) {
  using T = BwdTile<D>;
  constexpr int NQ = T::kNQ, NDT = T::kNDT, TB = T::kBytes;
  __shared__ __attribute__((aligned(1024))) char k_s0[TB], k_s1[TB], v_s0[TB], v_s1[TB];
  __shared__ __attribute__((aligned(16))) int32_t p_s0[32], p_s1[32];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5, li = lane & 31;
  // (a planned call: the host's order, clamped into range, so a wrong plan
  // gives wrong results but no access outside the tensors)
  const int L = (!MULTI && p.dq_order)
                    ? __builtin_amdgcn_readfirstlane(min(max(p.dq_order[blockIdx.x], 0), p.n_wg - 1))
                    : tile_order(blockIdx.x, p.n_wg, p.hq);
  const int h = L / p.n_tiles;
  const int qt = p.n_tiles - 1 - L % p.n_tiles;  // late rows (that see the most keys) first
  const int hk = h / (p.hq / p.hkv);
  const int lq = p.lq;
  const int wg_r0 = qt * 128, wg_r1 = min(wg_r0 + 128, lq);
  const int r0 = wg_r0 + 32 * wave;
  const int qi = min(r0 + li, lq - 1);              // this lane's row (clamped)
  const bool row_valid = r0 + li < lq;
  // Rows that see none of the block add nothing, and when accumulating dQ is
  // left as it is: the common case (the block's first key is after the
  // workgroup's last row) is decided by one load, before Q and dO are read.
  if (!MULTI && p.acc_dq && (p.lk == 0 || (p.causal && p.k_pos[0] > p.q_pos[wg_r1 - 1]))) return;

  // the wave's rows: B operands of S^T = K Q^T and dP^T = V dO^T
  bf16x8_t qreg[NQ], dreg[NQ];
  {
    const int64_t off = ((int64_t)qi * p.hq + h) * D + 8 * g;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      qreg[ks] = *(const bf16x8_t*)((const __bf16*)p.q + off + 16 * ks);
      dreg[ks] = *(const bf16x8_t*)((const __bf16*)p.dout + off + 16 * ks);
    }
  }
  const float l_raw = p.lse[(int64_t)h * lq + qi];
  const float lse2 = (!row_valid || l_raw == neg_inf()) ? __builtin_inff() : l_raw * kLog2e;
  const float dlt = row_valid ? p.delta[(int64_t)h * lq + qi] : 0.f;
  const int32_t my_qpos = p.causal ? p.q_pos[qi] : 0;
  const int32_t my_start = VARLEN ? doc_start(p.cu_seqlens, p.n_seqs, my_qpos) : 0;
  const int32_t wq_first = __builtin_amdgcn_readfirstlane(p.causal ? p.q_pos[min(r0, lq - 1)] : 0);  // rows ascend

  int ra[NQ];
#pragma unroll
  for (int ks = 0; ks < NQ; ++ks) ra[ks] = T::off(li, 2 * ks + g);
  int ta0[NDT], ta8[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) tr_offsets<D>(lane, dt, ta0[dt], ta8[dt]);

  f32x16_t acc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16_t{};

  // The blocks in order (one for a single-block call); dQ is summed in the
  // accumulators across them and stored once.
  bool seen = false;
  for (int blk = 0; blk < (MULTI ? bt.n : 1); ++blk) {
    const int lk = MULTI ? bt.lk[blk] : p.lk;
    const int32_t* kpos = MULTI ? bt.k_pos[blk] : p.k_pos;
    const void* kptr = MULTI ? bt.k[blk] : p.k;
    const void* vptr = MULTI ? bt.v[blk] : p.v;
    if (MULTI && (lk == 0 || (p.causal && kpos[0] > p.q_pos[wg_r1 - 1]))) continue;

    // keys the workgroup's rows can see
    int kb = 0, ke = lk;
    if (p.causal) {
      ke = wave_upper_bound(kpos, lk, p.q_pos[wg_r1 - 1]);
      if constexpr (VARLEN) kb = wave_upper_bound(kpos, lk, doc_start(p.cu_seqlens, p.n_seqs, p.q_pos[wg_r0]) - 1);
    }
    const int nt = ke > kb ? (ke - kb + 31) / 32 : 0;
    // (with documents the rows may still see nothing)
    if constexpr (MULTI) {
      if (nt == 0) continue;
    } else {
      if (nt == 0 && p.acc_dq) return;
    }
    seen = true;

    const int kv_stride = p.hkv * D * 2;
    const char* kbase = (const char*)kptr + (int64_t)hk * D * 2;
    const char* vbase = (const char*)vptr + (int64_t)hk * D * 2;
    u32x4_t kr[T::kUnits], vr[T::kUnits];
    int32_t pr = 0;
    auto fetch = [&](int t) __attribute__((always_inline)) {
      const int j0 = kb + 32 * t;
      fetch_rows<D>(kr, kbase, kv_stride, j0, lk, tid);
      fetch_rows<D>(vr, vbase, kv_stride, j0, lk, tid);
      if (tid < 32) pr = (p.causal && j0 + tid < lk) ? kpos[j0 + tid] : 0x7FFFFFFF;
    };
    auto commit = [&](int st) __attribute__((always_inline)) {
      commit_rows<D>(st ? (char CPATTN_LDS*)k_s1 : (char CPATTN_LDS*)k_s0, kr, tid);
      commit_rows<D>(st ? (char CPATTN_LDS*)v_s1 : (char CPATTN_LDS*)v_s0, vr, tid);
      if (tid < 32) (st ? p_s1 : p_s0)[tid] = pr;
    };

    if (nt > 0) {
      fetch(0);
      commit(0);
    }
    // (likewise before the loop: the Q and dO loads are done once the first
    // tile is committed, and with no tile the loop does not run)
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    phase_barrier();
    for (int t = 0; t < nt; ++t) {
      const int st = t & 1;
      if (t + 1 < nt) fetch(t + 1);
      const char CPATTN_LDS* kl = st ? (const char CPATTN_LDS*)k_s1 : (const char CPATTN_LDS*)k_s0;
      const char CPATTN_LDS* vl = st ? (const char CPATTN_LDS*)v_s1 : (const char CPATTN_LDS*)v_s0;
      const int32_t CPATTN_LDS* pl = st ? (const int32_t CPATTN_LDS*)p_s1 : (const int32_t CPATTN_LDS*)p_s0;

      // (the products run at raised priority: the other workgroup's wave on the
      // SIMD then issues its vector work around them rather than in their way)
      __builtin_amdgcn_s_setprio(1);
      // S^T = K Q^T, dP^T = V dO^T (rows: the tile's keys; column: this lane's query
      // row), alternating so that neither chain waits on its own previous MFMA;
      // operands read RING ahead
      constexpr int RING = 4;
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
      {
        constexpr int NM = 2 * NQ;
        auto rd = [&](int m) __attribute__((always_inline)) {
          return *(const bf16x8_t CPATTN_LDS*)(((m & 1) ? vl : kl) + ra[m >> 1]);
        };
        bf16x8_t a[RING];
#pragma unroll
        for (int m = 0; m < RING; ++m) a[m] = rd(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          if (m & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], dreg[m >> 1], dp, 0, 0, 0);
          else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], qreg[m >> 1], s, 0, 0, 0);
          if (m + RING < NM) a[m % RING] = rd(m + RING);
          __builtin_amdgcn_sched_barrier(0);
        }
      }

      __builtin_amdgcn_s_setprio(0);
      // dS^T = P (dP - D); register r is key 8(r/4) + 4g + r%4 of the tile.
      // Without documents, a tile of 32 keys inside the block that are all at
      // or before the wave's first row is seen in full by every row of the wave
      // (rows past the end have LSE +inf, so P = 0): no mask.
      const int lim = min(lk - (kb + 32 * t), 32);
      const bool full = lim == 32 && (!p.causal || (!VARLEN && __builtin_amdgcn_readfirstlane(pl[31]) <= wq_first));
      uint32_t pd[8];
      typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
      auto dsoft = [&](auto masked) __attribute__((always_inline)) {
        constexpr bool M = decltype(masked)::value;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          i32x4 k4 = {0, 0, 0, 0};
          if (M && p.causal) k4 = *(const i32x4 CPATTN_LDS*)(pl + 8 * rr + 4 * g);
          float dv[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            bool vis = true;
            if constexpr (M) {
              vis = 8 * rr + 4 * g + c < lim;
              if (p.causal) {
                vis = vis & (k4[c] <= my_qpos);
                if (VARLEN) vis = vis & (k4[c] >= my_start);
              }
            }
            const float pv = vis ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * rr + c], p.scale_log2, -lse2)) : 0.f;
            dv[c] = pv * (dp[4 * rr + c] - dlt);
          }
          pd[2 * rr] = pack_bf16x2(dv[0], dv[1]);
          pd[2 * rr + 1] = pack_bf16x2(dv[2], dv[3]);
        }
      };
      if (full) dsoft(std::false_type{});
      else dsoft(std::true_type{});

      __builtin_amdgcn_s_setprio(1);
      // dQ^T += K^T dS^T (K^T read transposed, RING ahead)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      {
        constexpr int NM = 2 * NDT;  // (hf, dt)
        const u32x4 bd[2] = {{pd[0], pd[1], pd[2], pd[3]}, {pd[4], pd[5], pd[6], pd[7]}};
        auto rd = [&](int m) __attribute__((always_inline)) {
          return read_tr(kl, ta0[m % NDT], ta8[m % NDT], m / NDT, T::kRowBytes);
        };
        bf16x8_t a[RING];
#pragma unroll
        for (int m = 0; m < RING; ++m) a[m] = rd(m);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NM; ++m) {
          acc[m % NDT] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[m % RING], __builtin_bit_cast(bf16x8_t, bd[m / NDT]),
                                                                 acc[m % NDT], 0, 0, 0);
          if (m + RING < NM) a[m % RING] = rd(m + RING);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (t + 1 < nt) commit(st ^ 1);
      // Nothing is in flight here (the commit waited for its loads). Saying so
      // keeps the compiler's wait analysis exact across the conditional commit:
      // otherwise it takes the skipped commit's loads as possibly pending and
      // waits in the next tile's matrix products for the tile fetch just
      // issued.
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
      phase_barrier();
    }
  }
  if (MULTI && !seen && p.acc_dq) return;

  // ---- store: lane holds row qi, head-dimension entries 32dt + 8rr + 4g + 0..3 ----
  // through the K/V stages, which no wave reads after the last barrier: wave w
  // stages its rows in stage array w
  const int n_rows = min(32, lq - r0);
  if (n_rows <= 0) return;
  char CPATTN_LDS* stg = wave == 0 ? (char CPATTN_LDS*)k_s0 : wave == 1 ? (char CPATTN_LDS*)k_s1
                       : wave == 2 ? (char CPATTN_LDS*)v_s0 : (char CPATTN_LDS*)v_s1;
  store_rows_lds<D>(p.dq + (int64_t)h * D, (int64_t)p.hq * D, r0, n_rows, stg, acc, p.scale, p.acc_dq != 0, lane);
}

// ---------------------------------------------------------------------------
// D = <dO, O> per (row, head): D/8 lanes per pair, 8 elements each.

template <typename TO, typename TD, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const void* o, const void* dout, float* delta, int64_t lq,
                                                        int32_t hq) {
  constexpr int LPP = D / 8;
  const int64_t pair = ((int64_t)blockIdx.x * 256 + threadIdx.x) / LPP;
  const int sub = threadIdx.x % LPP;
  const int64_t n = lq * hq;
  float acc = 0.f;
  if (pair < n) {
    const int64_t base = pair * D + 8 * sub;
    float a[8], b[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if constexpr (sizeof(TO) == 2) a[e] = (float)((const __bf16*)o)[base + e];
      else a[e] = ((const float*)o)[base + e];
      if constexpr (sizeof(TD) == 2) b[e] = (float)((const __bf16*)dout)[base + e];
      else b[e] = ((const float*)dout)[base + e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf(a[e], b[e], acc);
  }
#pragma unroll
  for (int m = LPP / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 64);
  if (pair < n && sub == 0) delta[(pair % hq) * lq + pair / hq] = acc;
}

// ---------------------------------------------------------------------------

int64_t bwd_query_workgroups(int64_t lq, int32_t hq) { return (lq + 127) / 128 * hq; }

void plan_bwd_query(const int32_t* q_pos, int64_t lq, const int32_t* k_pos, int64_t lk, const int32_t* cu_seqlens,
                    int32_t n_seqs, int32_t hq, int32_t* plan) {
  const int32_t n_tiles = (int32_t)((lq + 127) / 128);
  const int32_t n_wg = n_tiles * hq;
  // the kernel's searches: keys up to the tile's last row, from the start of
  // its first row's document
  auto upper = [](const int32_t* a, int64_t n, int32_t x) { return std::upper_bound(a, a + n, x) - a; };
  std::vector<int32_t> work((size_t)n_tiles);
  for (int32_t qt = 0; qt < n_tiles; ++qt) {
    const int64_t r0 = (int64_t)qt * 128, r1 = std::min<int64_t>(r0 + 128, lq);
    const int64_t ke = upper(k_pos, lk, q_pos[r1 - 1]);
    const int64_t d = upper(cu_seqlens, (int64_t)n_seqs + 1, q_pos[r0]);   // documents whose start <= the row
    const int32_t ds = cu_seqlens[std::max<int64_t>(d - 1, 0)];
    const int64_t kb = upper(k_pos, lk, ds - 1);
    work[(size_t)qt] = ke > kb ? (int32_t)((ke - kb + 31) / 32) : 0;
  }
  auto work_of = [&](int32_t L) { return work[(size_t)(n_tiles - 1 - L % n_tiles)]; };
  std::vector<int32_t> ls;
  for (int x = 0; x < 8; ++x) {
    ls.clear();
    for (int32_t b = x; b < n_wg; b += 8) ls.push_back(tile_order(b, n_wg, hq));
    std::stable_sort(ls.begin(), ls.end(), [&](int32_t a, int32_t c) {
      return work_of(a) != work_of(c) ? work_of(a) > work_of(c) : a < c;
    });
    size_t i = 0;
    for (int32_t b = x; b < n_wg; b += 8) plan[b] = ls[i++];
  }
}

template <int D, bool VARLEN>
static hipError_t launch_bwd_typed(BwdParams p, hipStream_t stream) {
  const BwdBlocks none{};
  if (p.lk > 0) {
    BwdParams a = p;
    a.n_tiles = (p.lk + 127) / 128;
    a.n_wg = a.n_tiles * p.hkv;
    hipLaunchKernelGGL((bwd_dkv_kernel<D, VARLEN, false>), dim3(a.n_wg), dim3(kDkvThreads), 0, stream, a, none);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.lq > 0) {
    BwdParams a = p;
    a.n_tiles = (p.lq + 127) / 128;
    a.n_wg = a.n_tiles * p.hq;
    hipLaunchKernelGGL((bwd_dq_kernel<D, VARLEN, false>), dim3(a.n_wg), dim3(kBwdThreads), 0, stream, a, none);
    return hipGetLastError();
  }
  return hipSuccess;
}

// bt.wg_end must hold the running sums of (lk_b + 127) / 128 * hkv.
template <int D, bool VARLEN>
static hipError_t launch_bwd_multi_typed(BwdParams p, const BwdBlocks& bt, hipStream_t stream) {
  const int32_t n_kwg = bt.n > 0 ? bt.wg_end[bt.n - 1] : 0;
  if (n_kwg > 0) {
    hipLaunchKernelGGL((bwd_dkv_kernel<D, VARLEN, true>), dim3(n_kwg), dim3(kDkvThreads), 0, stream, p, bt);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.lq > 0) {
    BwdParams a = p;
    a.n_tiles = (p.lq + 127) / 128;
    a.n_wg = a.n_tiles * p.hq;
    hipLaunchKernelGGL((bwd_dq_kernel<D, VARLEN, true>), dim3(a.n_wg), dim3(kBwdThreads), 0, stream, a, bt);
    return hipGetLastError();
  }
  return hipSuccess;
}

hipError_t launch_bwd(BwdParams p, int head_dim, bool varlen, hipStream_t stream) {
  if (head_dim == 128) return varlen ? launch_bwd_typed<128, true>(p, stream) : launch_bwd_typed<128, false>(p, stream);
  return varlen ? launch_bwd_typed<64, true>(p, stream) : launch_bwd_typed<64, false>(p, stream);
}

hipError_t launch_bwd_multi(BwdParams p, const BwdBlocks& bt, int head_dim, bool varlen, hipStream_t stream) {
  if (head_dim == 128)
    return varlen ? launch_bwd_multi_typed<128, true>(p, bt, stream) : launch_bwd_multi_typed<128, false>(p, bt, stream);
  return varlen ? launch_bwd_multi_typed<64, true>(p, bt, stream) : launch_bwd_multi_typed<64, false>(p, bt, stream);
}

template <int D>
static hipError_t launch_delta_d(const void* o, int o_bf16, const void* dout, int do_bf16, int64_t lq, int32_t hq,
                                 float* delta, hipStream_t stream) {
  const int64_t threads = lq * hq * (D / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  if (o_bf16 && do_bf16) hipLaunchKernelGGL((bwd_delta_kernel<__bf16, __bf16, D>), grid, block, 0, stream, o, dout, delta, lq, hq);
  else if (o_bf16) hipLaunchKernelGGL((bwd_delta_kernel<__bf16, float, D>), grid, block, 0, stream, o, dout, delta, lq, hq);
  else if (do_bf16) hipLaunchKernelGGL((bwd_delta_kernel<float, __bf16, D>), grid, block, 0, stream, o, dout, delta, lq, hq);
  else hipLaunchKernelGGL((bwd_delta_kernel<float, float, D>), grid, block, 0, stream, o, dout, delta, lq, hq);
  return hipGetLastError();
}

hipError_t launch_bwd_delta(const void* o, int o_bf16, const void* dout, int do_bf16, int64_t lq, int32_t hq,
                            int32_t head_dim, float* delta, hipStream_t stream) {
  if (lq * hq == 0) return hipSuccess;
  if (head_dim == 128) return launch_delta_d<128>(o, o_bf16, dout, do_bf16, lq, hq, delta, stream);
  return launch_delta_d<64>(o, o_bf16, dout, do_bf16, lq, hq, delta, stream);
}

}  // namespace cpattn

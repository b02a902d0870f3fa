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
//  * A workgroup is 4 wave64s. Each wave owns 32 query rows of one head; the
//    workgroup owns either 128 rows of one head or 32 rows of 4 heads that
//    share a KV head, so every K/V tile in LDS feeds 128 (row, head) pairs.
//  * Scores are computed transposed, S^T = K Q^T, with
//    v_mfma_f32_32x32x16_bf16: the accumulator then holds, in each lane, 16
//    keys of ONE query row (lane % 32), so row max and row sum are in-lane
//    plus one v_permlane32_swap between the half-waves, and the same
//    registers, rounded to bf16, are directly the B operand of O^T = V^T P^T.
//    O^T keeps each lane on one query row too, so the rescale is a per-lane
//    scalar multiply.
//  * K and V tiles (64 keys) go global -> LDS with global_load_lds_dwordx4
//    (no register staging), double-buffered, one barrier per tile. Both are
//    stored row-major with an XOR swizzle of 16-byte chunks; K is read with
//    ds_read_b128 (rows = MFMA rows), V with ds_read_b64_tr_b16, which hands
//    each lane four consecutive keys of one column — the V^T operand layout.
//  * Softmax runs in base 2 with the scale folded into one FMA per score.
//    The running max is raised only when a tile's max exceeds it by more than
//    2^8, so the O rescale is skipped on most tiles (the final normalisation
//    uses the same stale max, so the result is unchanged).
//  * Each wave classifies each key tile against its rows from the global
//    positions: tiles no row can see are skipped, tiles every row sees fully
//    run without a mask, only boundary tiles are masked. The workgroup loads
//    only the key range its rows can see.
//  * Workgroup ids are remapped so that consecutive logical tiles (same KV
//    head) run on the same XCD and share its L2; heavy (late-position) query
//    tiles are scheduled first.
//  * Float32 inputs use the same skeleton with v_mfma_f32_32x32x2_f32 and
//    32-key tiles.
#include <type_traits>

#include "device_common.hpp"
#include "kernels.hpp"

namespace cpattn {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

template <typename TIn, int D>
struct Cfg {
  static constexpr bool kBf16 = sizeof(TIn) == 2;
  static constexpr int kNB = kBf16 ? 2 : 1;           // 32-key blocks per tile
  static constexpr int kBK = 32 * kNB;                // keys per tile
  static constexpr int kRowBytes = D * (int)sizeof(TIn);
  static constexpr int kChunks = kRowBytes / 16;      // 16-byte chunks per row
  static constexpr int kTileBytes = kBK * kRowBytes;
  static constexpr int kInst = kTileBytes / 1024;     // direct-to-LDS instructions per tile
  static_assert(kInst % kWaves == 0, "tile must split evenly over the waves");

  // Swizzles (16-byte chunk index XOR row function). K is read as 16
  // consecutive rows at one chunk; V (bf16) as 4 consecutive rows x 4 chunks.
  __device__ static __forceinline__ int swz_k(int row) {
    if constexpr (kBf16) return D == 128 ? (row & 15) : ((row >> 1) & 7);
    else return row & 15;
  }
  __device__ static __forceinline__ int swz_v(int row) {
    if constexpr (kBf16) return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    else return row & 15;
  }
  __device__ static __forceinline__ int off_k(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz_k(row)) << 4);
  }
  __device__ static __forceinline__ int off_v(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz_v(row)) << 4);
  }
};

// Workgroup id -> logical tile id. Hardware dispatches consecutive workgroup
// ids round-robin over the 8 XCDs; this gives XCD x a contiguous range of
// logical ids, so tiles of the same head share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  int x = bid & 7, slot = bid >> 3;
  int q = n >> 3, rem = n & 7;
  return x * q + (x < rem ? x : rem) + slot;
}

// Issue this wave's share of the direct-to-LDS loads of one K or V tile.
template <typename TIn, int D, bool IS_V>
__device__ __forceinline__ void load_tile(char CPATTN_LDS* lds_tile, const char* gbase, int64_t row_stride,
                                          int64_t j0, int64_t lk, int wave, int lane) {
  using C = Cfg<TIn, D>;
#pragma unroll
  for (int it = 0; it < C::kInst / kWaves; ++it) {
    int inst = wave + kWaves * it;
    int o = inst * 1024 + lane * 16;
    int row = o / C::kRowBytes;
    int pchunk = (o % C::kRowBytes) >> 4;
    int chunk = pchunk ^ (IS_V ? C::swz_v(row) : C::swz_k(row));
    int64_t grow = j0 + row;
    grow = grow < lk ? grow : lk - 1;  // rows past the block end re-read a valid row; they are masked
    const char* src = gbase + grow * row_stride + chunk * 16;
    __builtin_amdgcn_global_load_lds((const void*)src, (void CPATTN_LDS*)(lds_tile + inst * 1024), 16, 0, 0);
  }
}

template <typename TIn, typename TOut, int D, bool VARLEN>
__global__ __launch_bounds__(kThreads, 2) void partial_fwd_kernel(PartialParams p) {
  using C = Cfg<TIn, D>;
  constexpr int NB = C::kNB;
  constexpr int BK = C::kBK;
  constexpr int NDT = D / 32;

  __shared__ __attribute__((aligned(1024))) char smem[4 * C::kTileBytes];  // [buf][K,V]
  char CPATTN_LDS* lds = (char CPATTN_LDS*)smem;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 5;        // half-wave
  const int li = lane & 31;       // query row within the wave

  const int L = xcd_remap(blockIdx.x, p.n_wg);
  const int hgrp = L / p.n_qtiles;
  const int qt = p.n_qtiles - 1 - (L % p.n_qtiles);  // late (heavier) rows first
  const int hsub = wave % p.g_wg, rb = wave / p.g_wg;
  const int h = hgrp * p.g_wg + hsub;
  const int hk = h / (p.hq / p.hkv);

  const int64_t lq = p.lq, lk = p.lk;
  const int64_t wg_r0 = (int64_t)qt * 32 * p.r_wg;
  const int64_t wg_r1 = imin64(wg_r0 + 32 * p.r_wg, lq);
  const int64_t r0 = wg_r0 + 32 * rb;
  const int64_t r1 = imin64(r0 + 32, lq);
  const bool wave_active = r0 < lq;

  // ---- key range of the workgroup, and per-wave classification bounds ----
  int64_t kb = 0, ke = lk;                              // workgroup's visible key range
  int64_t w_lo = 0, w_hi = lk, f_lo = 0, f_hi = lk;     // wave: visible range, fully visible range
  if (p.causal) {
    int32_t wq_hi = p.q_pos[wg_r1 - 1];
    ke = upper_bound_i32(p.k_pos, lk, wq_hi);
    if (VARLEN) kb = lower_bound_i32(p.k_pos, lk, doc_start(p.cu_seqlens, p.n_seqs, p.q_pos[wg_r0]));
    if (wave_active) {
      int32_t q_lo = p.q_pos[r0], q_hi = p.q_pos[r1 - 1];
      w_hi = upper_bound_i32(p.k_pos, lk, q_hi);
      f_hi = upper_bound_i32(p.k_pos, lk, q_lo);
      if (VARLEN) {
        w_lo = lower_bound_i32(p.k_pos, lk, doc_start(p.cu_seqlens, p.n_seqs, q_lo));
        f_lo = lower_bound_i32(p.k_pos, lk, doc_start(p.cu_seqlens, p.n_seqs, q_hi));
      }
    }
  }
  if (!wave_active) { w_lo = 0; w_hi = 0; }
  const int64_t kt_begin = kb / BK;
  const int64_t kt_end = (ke + BK - 1) / BK;

  // ---- this lane's query row ----
  const int64_t qi = imin64(r0 + li, lq - 1);
  const bool row_valid = wave_active && (r0 + li < lq);
  const int32_t my_qpos = p.causal ? p.q_pos[qi] : 0;
  const int32_t my_start = (VARLEN && p.causal) ? doc_start(p.cu_seqlens, p.n_seqs, my_qpos) : 0;

  // Q operand (B of S^T = K Q^T), resident in registers for the whole call.
  constexpr int NQ = C::kBf16 ? D / 16 : D / 2;
  typedef typename std::conditional<C::kBf16, bf16x8_t, float>::type QReg;
  QReg qreg[NQ];
  {
    const TIn* qrow = (const TIn*)p.q + (qi * p.hq + h) * (int64_t)D;
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      if constexpr (C::kBf16) qreg[ks] = *(const bf16x8_t*)(qrow + 16 * ks + 8 * g);
      else qreg[ks] = qrow[2 * ks + g];
    }
  }

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = neg_inf();  // running max of scale*log2(e)*score (may lag the true max by < kTau)
  float l_run = 0.f;        // this lane's share of the running sum

  const int64_t kv_stride = (int64_t)p.hkv * D * sizeof(TIn);
  const char* kbase = (const char*)p.k + (int64_t)hk * D * sizeof(TIn);
  const char* vbase = (const char*)p.v + (int64_t)hk * D * sizeof(TIn);

  if (kt_begin < kt_end) {
    load_tile<TIn, D, false>(lds, kbase, kv_stride, kt_begin * BK, lk, wave, lane);
    load_tile<TIn, D, true>(lds + C::kTileBytes, vbase, kv_stride, kt_begin * BK, lk, wave, lane);
  }

  for (int64_t kt = kt_begin; kt < kt_end; ++kt) {
    const int cur = (int)((kt - kt_begin) & 1);
    char CPATTN_LDS* kl = lds + cur * 2 * C::kTileBytes;
    char CPATTN_LDS* vl = kl + C::kTileBytes;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's loads of tile kt are in LDS
    __syncthreads();                     // everyone's are; and tile kt-1's buffer is free
    if (kt + 1 < kt_end) {
      char CPATTN_LDS* nk = lds + (cur ^ 1) * 2 * C::kTileBytes;
      load_tile<TIn, D, false>(nk, kbase, kv_stride, (kt + 1) * BK, lk, wave, lane);
      load_tile<TIn, D, true>(nk + C::kTileBytes, vbase, kv_stride, (kt + 1) * BK, lk, wave, lane);
    }

    const int64_t j0 = kt * BK, j1 = j0 + BK;
    if (j1 <= w_lo || j0 >= w_hi) continue;             // no row of this wave sees the tile
    const bool full = (j0 >= f_lo) && (j1 <= f_hi);     // every row sees every key

    // ---- S^T = K Q^T for NB blocks of 32 keys ----
    f32x16_t sacc[NB];
#pragma unroll
    for (int jb = 0; jb < NB; ++jb) {
      sacc[jb] = f32x16_t{};
      const int row = 32 * jb + li;
#pragma unroll
      for (int ks = 0; ks < NQ; ++ks) {
        if constexpr (C::kBf16) {
          bf16x8_t a = *(const bf16x8_t CPATTN_LDS*)(kl + C::off_k(row, 2 * ks + g));
          sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[ks], sacc[jb], 0, 0, 0);
        } else {
          const int d = 2 * ks + g;
          float a = *(const float CPATTN_LDS*)(kl + C::off_k(row, d >> 2) + ((d & 3) << 2));
          sacc[jb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qreg[ks], sacc[jb], 0, 0, 0);
        }
      }
    }

    // ---- mask boundary tiles: lane's register r of block jb is key 32jb + 8(r/4) + 4g + r%4 ----
    if (!full) {
#pragma unroll
      for (int jb = 0; jb < NB; ++jb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t j = j0 + 32 * jb + 8 * (r >> 2) + 4 * g + (r & 3);
          bool vis = j < lk;
          if (vis && p.causal) {
            const int32_t kp = p.k_pos[j];
            vis = kp <= my_qpos;
            if (VARLEN) vis = vis && kp >= my_start;
          }
          if (!vis) sacc[jb][r] = neg_inf();
        }
      }
    }

    // ---- online softmax (base 2) ----
    float mx = neg_inf();
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
    const float m_use = (m_run == neg_inf()) ? 0.f : m_run;
    float lsum = 0.f;
#pragma unroll
    for (int jb = 0; jb < NB; ++jb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float e = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[jb][r], p.scale_log2, -m_use));
        sacc[jb][r] = e;
        lsum += e;
      }
    l_run += lsum;

    // ---- O^T += V^T P^T ----
    if constexpr (C::kBf16) {
      uint32_t pk[NB][8];
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int r = 0; r < 8; ++r) pk[jb][r] = pack_bf16x2(sacc[jb][2 * r], sacc[jb][2 * r + 1]);
      const int vr = 4 * g + ((lane & 15) >> 2);             // row within a 16-key group
      const int vc = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // column within a 32-column block
#pragma unroll
      for (int jb = 0; jb < NB; ++jb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
          u32x4 bw = {pk[jb][4 * half], pk[jb][4 * half + 1], pk[jb][4 * half + 2], pk[jb][4 * half + 3]};
          bf16x8_t b = __builtin_bit_cast(bf16x8_t, bw);
          const int row = 32 * jb + 16 * half + vr;
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            const int col = 32 * dt + vc;
            const int cb = (col & 7) << 1;
            i16x4_t t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4_t CPATTN_LDS*)(vl + C::off_v(row, col >> 3) + cb));
            i16x4_t t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (i16x4_t CPATTN_LDS*)(vl + C::off_v(row + 8, col >> 3) + cb));
            typedef short i16x8 __attribute__((ext_vector_type(8)));
            i16x8 a16 = __builtin_shufflevector(t0, t1, 0, 1, 2, 3, 4, 5, 6, 7);
            oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a16), b, oacc[dt], 0, 0, 0);
          }
        }
    } else {
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
  }

  // ---- finalise: O = acc / l, LSE = ln(l) + max; merge into the stored state if accumulating ----
  const float l_tot = half_swap_sum(l_run);
  const bool empty = !(l_tot > 0.f);
  const float inv_l = empty ? 0.f : 1.0f / l_tot;
  const float lse_blk = empty ? neg_inf() : (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
  if (!row_valid) return;

  float w_old = 0.f, w_blk = 1.f, lse_out = lse_blk;
  float* lse_ptr = p.lse + (int64_t)h * lq + (r0 + li);
  if (p.accumulate) merge_weights(*lse_ptr, lse_blk, w_old, w_blk, lse_out);
  const float s_blk = w_blk * inv_l;
  TOut* orow = (TOut*)p.o + ((r0 + li) * p.hq + h) * (int64_t)D;
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int dv = 32 * dt + 8 * rr + 4 * g;
      float v0 = oacc[dt][4 * rr] * s_blk, v1 = oacc[dt][4 * rr + 1] * s_blk;
      float v2 = oacc[dt][4 * rr + 2] * s_blk, v3 = oacc[dt][4 * rr + 3] * s_blk;
      if constexpr (sizeof(TOut) == 2) {
        uint2* dst = (uint2*)(orow + dv);
        if (p.accumulate) {
          uint2 old = *dst;
          v0 += w_old * bf16_bits_to_f32((uint16_t)(old.x & 0xFFFF));
          v1 += w_old * bf16_bits_to_f32((uint16_t)(old.x >> 16));
          v2 += w_old * bf16_bits_to_f32((uint16_t)(old.y & 0xFFFF));
          v3 += w_old * bf16_bits_to_f32((uint16_t)(old.y >> 16));
        }
        *dst = make_uint2(pack_bf16x2(v0, v1), pack_bf16x2(v2, v3));
      } else {
        float4* dst = (float4*)(orow + dv);
        if (p.accumulate) {
          float4 old = *dst;
          v0 += w_old * old.x; v1 += w_old * old.y; v2 += w_old * old.z; v3 += w_old * old.w;
        }
        *dst = make_float4(v0, v1, v2, v3);
      }
    }
  if (g == 0) *lse_ptr = lse_out;
}

// ---------------------------------------------------------------------------

template <typename TIn, typename TOut, int D>
static hipError_t launch_typed(const PartialParams& p, bool varlen, hipStream_t stream) {
  dim3 grid(p.n_wg), block(kThreads);
  if (varlen) hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, true>), grid, block, 0, stream, p);
  else hipLaunchKernelGGL((partial_fwd_kernel<TIn, TOut, D, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_partial(PartialParams p, int in_bf16, int out_bf16, int head_dim, bool varlen, hipStream_t stream) {
  const int G = p.hq / p.hkv;
  p.g_wg = (G % kWaves == 0) ? kWaves : ((G % 2 == 0) ? 2 : 1);
  p.r_wg = kWaves / p.g_wg;
  p.n_qtiles = (int32_t)((p.lq + 32 * p.r_wg - 1) / (32 * p.r_wg));
  p.n_hgroups = p.hq / p.g_wg;
  const int64_t n_wg = (int64_t)p.n_qtiles * p.n_hgroups;
  if (n_wg <= 0) return hipSuccess;
  if (n_wg > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  p.n_wg = (int32_t)n_wg;
  if (in_bf16) {
    if (head_dim == 128) return out_bf16 ? launch_typed<__bf16, __bf16, 128>(p, varlen, stream)
                                         : launch_typed<__bf16, float, 128>(p, varlen, stream);
    return out_bf16 ? launch_typed<__bf16, __bf16, 64>(p, varlen, stream)
                    : launch_typed<__bf16, float, 64>(p, varlen, stream);
  }
  if (head_dim == 128) return launch_typed<float, float, 128>(p, varlen, stream);
  return launch_typed<float, float, 64>(p, varlen, stream);
}

}  // namespace cpattn

// tile_io.hpp — K/V tile staging for the partial-attention kernel
// (partial_fwd.hip): tile geometry and LDS swizzles,
// global -> LDS loads (direct and register-staged), the phase barrier and
// register pins. NW is the number of waves that share one tile's loads.
// The gradient kernels (partial_bwd.hip) use its buffer descriptors, scalar
// clamp, workgroup remap and phase barrier. Internal to the library.
#pragma once

#include "device_common.hpp"

namespace cpattn {

constexpr float kTau = 8.0f;  // lazy-rescale threshold (log2 units)

template <typename TIn, int D, int NW>
struct Cfg {
  static constexpr bool kBf16 = sizeof(TIn) == 2;
  // 32-key blocks per tile: 64 keys at d 128; 128 at d 64, so that a tile has
  // the bytes, MFMAs and registers of a d 128 one and the per-tile costs of
  // the phases (barriers, fetch, commit, checks) are spread over twice the keys
  static constexpr int kNB = kBf16 ? (D == 64 ? 4 : 2) : 1;
  static constexpr int kBK = 32 * kNB;                // keys per tile
  static constexpr int kRowBytes = D * (int)sizeof(TIn);
  static constexpr int kTileBytes = kBK * kRowBytes;
  static constexpr int kInst = kTileBytes / 1024;     // direct-to-LDS instructions per tile
  static constexpr int kRowsPerInst = 1024 / kRowBytes;
  static constexpr int kNQ = kBf16 ? D / 16 : D / 2;  // Q operand registers (MFMA k-steps of S^T)
  static constexpr int kNDT = D / 32;                 // 32-column blocks of O^T
  static constexpr int kPosPerWave = kBK / NW;        // key positions each wave stages
  static_assert(kInst % NW == 0, "tile must split evenly over the waves");

  // Swizzles (16-byte chunk index XOR row function). K is read as 16
  // consecutive rows at one chunk; V (bf16) as 4 consecutive rows x 4 chunks.
  static constexpr int swz_k(int row) {
    if constexpr (kBf16) return D == 128 ? (row & 15) : ((row >> 1) & 7);
    else return row & 15;
  }
  static constexpr int swz_v(int row) {
    if constexpr (kBf16) return D == 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2);
    else return row & 15;
  }
  static constexpr int off_k(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz_k(row)) << 4);
  }
  static constexpr int off_v(int row, int chunk) {
    return row * kRowBytes + ((chunk ^ swz_v(row)) << 4);
  }
  // the swizzles repeat every 16 rows (K) / 4 rows (bf16 V), a divisor of the
  // rows one wave's successive load instructions advance by
  static_assert((NW * kRowsPerInst) % 16 == 0, "load offsets must be instruction-invariant");
};

// Workgroup id -> logical tile id. Hardware dispatches consecutive workgroup
// ids round-robin over the 8 XCDs; this gives XCD x a contiguous range of
// logical ids, so tiles of the same head share that XCD's L2.
__host__ __device__ __forceinline__ int xcd_remap(int bid, int n) {
  int x = bid & 7, slot = bid >> 3;
  int q = n >> 3, rem = n & 7;
  return x * q + (x < rem ? x : rem) + slot;
}

// Logical tile of workgroup bid when the logical order is unit-major (a unit:
// a head or head group, its tiles heaviest first). With a multiple of 8 units
// each XCD gets whole units (xcd_remap: shared K/V in its L2, and every XCD
// the same mix of heavy and light tiles). Otherwise contiguous ranges would
// give one XCD all the heaviest tiles (two units of 4096 tiles: 1.75 times
// the mean work), so the hardware's round-robin order is kept, which hands
// every XCD every eighth tile of the heavy-first order.
__host__ __device__ __forceinline__ int tile_order(int bid, int n, int units) {
  return (units & 7) == 0 ? xcd_remap(bid, n) : bid;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  // raw buffer (stride 0): the record count is a byte count
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Lane part of the source offset of this lane's 16 bytes in a tile's
// direct-to-LDS instruction inst = wave + NW*it: the instruction fills LDS
// bytes [inst*1024, +1024) with rows inst*RPI .. +RPI-1 of the tile; lane
// `lane` writes 16 bytes at inst*1024 + 16*lane, which is physical chunk pc
// of row lr of those, and so must hold logical chunk pc ^ swz(row). The row
// offset inst*RPI*row_stride is added as a scalar.
template <typename TIn, int D, bool IS_V, int NW>
__device__ __forceinline__ int lane_voff(int wave, int lane, int64_t row_stride) {
  using C = Cfg<TIn, D, NW>;
  const int lr = (lane * 16) / C::kRowBytes;
  const int pc = ((lane * 16) % C::kRowBytes) >> 4;
  const int row = wave * C::kRowsPerInst + lr;
  const int chunk = pc ^ (IS_V ? C::swz_v(row) : C::swz_k(row));
  return lr * (int)row_stride + chunk * 16;
}

// Issue this wave's share of the direct-to-LDS loads of one K or V tile whose
// first row is r0. Rows at or past lk re-read the last valid row (they are
// masked); whole tiles in range need no per-lane arithmetic.
template <typename TIn, int D, bool IS_V, int NW>
__device__ __forceinline__ void load_tile(char CPATTN_LDS* lds_tile, const char* head_base, int64_t row_stride,
                                          int r0, int lk, int wave, int lane, int voff0) {
  using C = Cfg<TIn, D, NW>;
  constexpr int RPI = C::kRowsPerInst;
  const char* base = head_base + (int64_t)r0 * row_stride;
  const int rows = lk - r0;
  if (rows >= C::kBK) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (C::kBK - 1) * row_stride + C::kRowBytes);
#pragma unroll
    for (int it = 0; it < C::kInst / NW; ++it) {
      const int inst = wave + NW * it;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void CPATTN_LDS*)(lds_tile + inst * 1024), 16, voff0,
                                               inst * RPI * (int)row_stride, 0, 0);
    }
  } else {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(base, (rows - 1) * row_stride + C::kRowBytes);
    int ln = lane;
    asm volatile("" : "+v"(ln));  // the tail tile is rare: recompute its offsets here, keep no registers for them
    const int lr = (ln * 16) / C::kRowBytes;
#pragma unroll
    for (int it = 0; it < C::kInst / NW; ++it) {
      const int inst = wave + NW * it;
      const int row = inst * RPI + lr;
      const int rc = row < rows ? row : rows - 1;
      const int voff = lane_voff<TIn, D, IS_V, NW>(wave, ln, row_stride) + (rc - lr) * (int)row_stride;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void CPATTN_LDS*)(lds_tile + inst * 1024), 16, voff, 0, 0, 0);
    }
  }
}

// Key positions of a tile of BK keys: wave w loads entries [E*w, E*w+E),
// E = BK/NW, of the BK-entry stage (the last valid position repeated past
// lk), one instruction per wave. Without positions (non-causal calls) the
// same instruction reads the key tensor instead, into a stage nobody reads.
template <int NW, int BK>
__device__ __forceinline__ void load_positions(int32_t CPATTN_LDS* kp_tile, const int32_t* src, int r0, int lk,
                                               int wave, int lane) {
  constexpr int E = BK / NW;
  static_assert(E <= 64 && (E & (E - 1)) == 0, "a wave stages a power-of-two run of positions");
  const int rows = min(lk - r0, BK);
  const int e = E * wave + (lane & (E - 1));
  const int idx = e < rows ? e : rows - 1;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + r0, rows * 4);
  if (lane < E)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (void CPATTN_LDS*)(kp_tile + E * wave), 4, idx * 4, 0, 0, 0);
}

// Register-staged loads for the steady-state ring. Direct-to-LDS loads have a
// small in-flight budget per CU: once about sixteen are outstanding, issuing
// one more stalls the wave until an earlier one lands (hundreds of cycles when
// the data streams from HBM). Loads into registers issue in a few cycles
// however many are in flight, so the ring fetches the next load group into
// registers one phase pair ahead and writes it to LDS (ds_write_b128) when it
// is needed. The lane/instruction mapping is that of load_tile, so the LDS
// layout is the same.
//
// The fetch has no branches: the buffer descriptor covers exactly the tile's
// rows inside the block, and the hardware range check returns zeros for the
// lanes of rows past it (a tail tile's missing keys, or a whole tile past the
// end, which is then never read). Zero rows are harmless: their scores are
// masked and their probabilities are zero. The row offset goes into the
// per-lane offset, which the range check sees.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// n (wave-uniform) clamped to [0, hi], on the scalar unit. Written as plain
// min/max the clamp is selected as a vector instruction (v_med3) whose result
// is read back with readfirstlane: that needs a vector register for a moment,
// and the compiler picks one of the staging registers, which can make it wait
// for every load in flight. The result must stay scalar anyway (a buffer
// descriptor the compiler thinks may vary per lane costs a loop over lanes at
// every load).
__device__ __forceinline__ int clamp_rows(int n, int hi) {
  int r;
  asm("s_max_i32 %0, %1, 0\n\ts_min_i32 %0, %0, %2" : "=&s"(r) : "s"(n), "s"(hi));
  return r;
}

template <typename TIn, int D, int NW>
__device__ __forceinline__ void fetch_tile(u32x4_t* regs, const char* head_base, int row_stride, int r0, int lk,
                                           int wave, int voff0) {
  using C = Cfg<TIn, D, NW>;
  constexpr int RPI = C::kRowsPerInst;
  const int rows = clamp_rows(lk - r0, C::kBK);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head_base + (int64_t)r0 * row_stride, (int64_t)rows * row_stride);
#pragma unroll
  for (int it = 0; it < C::kInst / NW; ++it)
    regs[it] = __builtin_amdgcn_raw_buffer_load_b128(rs, voff0 + (wave + NW * it) * RPI * row_stride, 0, 0);
}

template <typename TIn, int D, int NW>
__device__ __forceinline__ void commit_tile(char CPATTN_LDS* lds_tile, const u32x4_t* regs, int wave, int lane) {
  using C = Cfg<TIn, D, NW>;
#pragma unroll
  for (int it = 0; it < C::kInst / NW; ++it)
    *(u32x4_t CPATTN_LDS*)(lds_tile + (wave + NW * it) * 1024 + lane * 16) = regs[it];
}

// Positions: lanes 0..E-1 of wave w (E = BK/NW) hold entries E*w.. (zero past
// the block, and everywhere when src is null: non-causal calls stage zeros
// nobody reads).
template <int NW, int BK>
__device__ __forceinline__ int32_t fetch_positions(const int32_t* src, int r0, int lk, int wave, int lane) {
  constexpr int E = BK / NW;
  const int rows = src ? clamp_rows(lk - r0, BK) : 0;
  return (int32_t)__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(src + r0, rows * 4),
                                                       (E * wave + (lane & (E - 1))) * 4, 0, 0);
}

template <int NW, int BK>
__device__ __forceinline__ void commit_positions(int32_t CPATTN_LDS* kp_tile, int32_t v, int wave, int lane) {
  constexpr int E = BK / NW;
  if (lane < E) kp_tile[E * wave + lane] = v;
}

// s_waitcnt immediate waiting until at most n vector-memory instructions are outstanding.
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Workgroup barrier between phases. Unlike __syncthreads() it carries no
// release fence, which would make every wave wait for ALL of its outstanding
// direct-to-LDS loads (the prefetch of later stages); the ring waits instead,
// before the barrier, for exactly the loads it needs. Each wave's LDS reads
// are complete (lgkmcnt(0)), and the "memory" clobber keeps the compiler from
// moving memory accesses across.
__device__ __forceinline__ void phase_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Workgroup barrier at the end of a phase that issued only LDS reads whose
// stages no wave rewrites before this wave's next phase_barrier() (which waits
// for them): the reads stay in flight across it.
__device__ __forceinline__ void phase_barrier_reads() { asm volatile("s_barrier" ::: "memory"); }

// Materialise a register value at this point of the program. The barrier above
// only orders memory accesses: left alone, the compiler sinks pure register
// work (the exponentials, packs and row sums of the vector phase) past it into
// the wave's own matrix phase, which serialises the two phases the schedule
// means to overlap across waves. An empty volatile asm that reads and writes
// the value keeps its computation before the next volatile asm (the barrier).
template <typename T>
__device__ __forceinline__ void pin(T& x) { asm volatile("" : "+v"(x)); }

}  // namespace cpattn

// Device-side building blocks for the gfx950 (CDNA4) attention kernels:
// MFMA operand types, LDS tile addressing, work-group -> tile mapping and the
// per-sequence geometry of dense and packed batches.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_params.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define FA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_32x32x16_bf16: C[32x32] += A[32x16] * B[16x32].
// Operand layout per lane l (wave64):  A row m = l % 32, B column n = l % 32;
// both hold 8 consecutive K slots selected by l / 32.  The result holds
// column n = l % 32 and rows 8*(i/4) + 4*(l/32) + i%4 for i = 0..15.
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b,
                                         const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 u) {
  return __builtin_bit_cast(bf16x8, u);
}

// Round 8 floats to bf16 (round to nearest even, v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2,
                                              float a3, float a4, float a5,
                                              float a6, float a7) {
  bf16x8 r;
  r[0] = (__bf16)a0; r[1] = (__bf16)a1; r[2] = (__bf16)a2; r[3] = (__bf16)a3;
  r[4] = (__bf16)a4; r[5] = (__bf16)a5; r[6] = (__bf16)a6; r[7] = (__bf16)a7;
  return r;
}

// The same operations for either 16-bit element type of the matrix
// operands: bf16 (F16 = false) or IEEE fp16 (F16 = true,
// v_mfma_f32_32x32x16_f16).  Operands move as raw 16-bit data in bf16x8
// containers; only the MFMA, the rounding of fp32 values to 16 bits (nearest
// even) and the element type of stores depend on the choice.
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <bool F16>
__device__ __forceinline__ f32x16 mfma32_t(const bf16x8& a, const bf16x8& b,
                                           const f32x16& c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
template <bool F16>
__device__ __forceinline__ bf16x8 pack8_t(float a0, float a1, float a2, float a3, float a4,
                                          float a5, float a6, float a7) {
  if constexpr (F16) {
    f16x8 r;
    r[0] = (_Float16)a0; r[1] = (_Float16)a1; r[2] = (_Float16)a2; r[3] = (_Float16)a3;
    r[4] = (_Float16)a4; r[5] = (_Float16)a5; r[6] = (_Float16)a6; r[7] = (_Float16)a7;
    return __builtin_bit_cast(bf16x8, r);
  } else {
    return pack_bf16x8(a0, a1, a2, a3, a4, a5, a6, a7);
  }
}
// Four fp32 values rounded to 16 bits, as the raw 8 bytes they are stored in
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
template <bool F16>
__device__ __forceinline__ uint2 pack4_t(float a0, float a1, float a2, float a3) {
  if constexpr (F16) {
    f16x4 w;
    w[0] = (_Float16)a0; w[1] = (_Float16)a1; w[2] = (_Float16)a2; w[3] = (_Float16)a3;
    return __builtin_bit_cast(uint2, w);
  } else {
    bf16x4 w;
    w[0] = (__bf16)a0; w[1] = (__bf16)a1; w[2] = (__bf16)a2; w[3] = (__bf16)a3;
    return __builtin_bit_cast(uint2, w);
  }
}

__device__ __forceinline__ float fast_exp2(float x) {
  return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

// max(x, x of lane l ^ 32) and x + (x of lane l ^ 32) in every lane, with one
// v_permlane32_swap (a vector ALU exchange of the two half-waves) instead of
// the LDS crossbar that a general shuffle uses.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x),
                                                  __builtin_bit_cast(unsigned, x), false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// ---------------------------------------------------------------- LDS tiles
// A K or V tile of R rows x D bf16 columns is stored row-major with its
// 16-byte chunks permuted inside each row: chunk c of row r lives at chunk
// c ^ swz<D>(r).  The permutation is chosen (and checked exhaustively on the
// host for 32- and 64-bank LDS) so that both access patterns below touch
// distinct banks within every LDS pass:
//   * 128-bit reads of one chunk from consecutive rows (MFMA A operand),
//   * transposing 64-bit reads of 4 aligned rows x 32 bytes per 16 lanes
//     (ds_read_b64_tr_b16), two such groups side by side per pass.
// D = 128 (16 chunks): rows r..r+15 map one chunk to 16 distinct offsets,
// and 4 aligned rows land in 4 distinct 64-byte groups.  D = 64 (8 chunks,
// two rows per 256 bytes): same-parity rows of 16 map to distinct offsets.
template <int D>
__host__ __device__ constexpr int swz(int r) {
  if constexpr (D == 128) {
    // bits 1..3 from r % 4 through the table {0, 6, 10, 12}, bit 0 = r/4 % 2,
    // bit 3 also flipped by r/8 % 2
    const int h = (0xCA60 >> ((r & 3) * 4)) & 0xF;
    return h ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 3);
  } else {
    const int r0 = r & 1, r1 = (r >> 1) & 1, r2 = (r >> 2) & 1, r3 = (r >> 3) & 1;
    return ((r1 ^ r3) << 2) | ((r0 ^ r2) << 1) | (r2 ^ r3);
  }
}

// Element offset of (row r, column col) in a swizzled tile with D columns.
template <int D>
__host__ __device__ constexpr int tile_off(int r, int col) {
  return r * D + ((((col >> 3) ^ swz<D>(r))) << 3) + (col & 7);
}

// ---------------------------------------------------------------- 8-bit tiles
// The FP8 forward stages two byte tiles per key block:
//   * K: 64 rows (keys) of D bytes;
//   * V^T: D rows (head-dimension columns) of 64 bytes (keys).
// Both are stored with their 16-byte chunks permuted inside each row (chunk c
// of row r at chunk c ^ swz(r)); the permutations are checked exhaustively on
// the host, for 32- and 64-bank LDS, against the reads the kernel issues:
//   * K: lane (m, h) of a wave (m = lane % 32, h = lane / 32) reads 16 bytes
//     at row k8_row(kb, m), chunk 4 st + 2 h + u (D = 128) or 2 h + u
//     (D = 64), for key block kb, k-step st and half u of its 32 bytes;
//   * V^T: lane (m, h) reads 16 bytes at row 32 db + m, chunk 2 h + u.
template <int D>
__host__ __device__ constexpr int swz_k8(int r) {
  if constexpr (D == 128)  // bits (r0 ^ r2, r1, r5) of the row
    return ((r ^ (r >> 2)) & 1) | (((r >> 1) & 1) << 1) | (((r >> 5) & 1) << 2);
  else  // 4 chunks: bits (r1 ^ r2, r5)
    return (((r >> 1) ^ (r >> 2)) & 1) | (((r >> 5) & 1) << 1);
}
__host__ __device__ constexpr int swz_v8(int r) {  // 4 chunks: bits (r1 ^ r3, r2)
  return (((r >> 1) ^ (r >> 3)) & 1) | (((r >> 2) & 1) << 1);
}
template <int D>
__host__ __device__ constexpr int k8_off(int r, int byte) {
  return r * D + ((((byte >> 4) ^ swz_k8<D>(r))) << 4) + (byte & 15);
}
__host__ __device__ constexpr int v8_off(int r, int byte) {
  return r * 64 + ((((byte >> 4) ^ swz_v8(r))) << 4) + (byte & 15);
}
// K-tile row read by A-operand row m of key block kb in the FP8 score
// product.  With this order the 32 x 32 result gives lane half h the scores
// of the 32 consecutive keys 32 h + 16 kb + i (i = 0..15), which is the
// order the P V product takes them in: P never needs a permutation.
__host__ __device__ constexpr int k8_row(int kb, int m) {
  return 32 * ((m >> 2) & 1) + 16 * kb + 4 * (m >> 3) + (m & 3);
}

// LDS reads at a lane byte offset plus a byte offset that is a compile-time
// constant after unrolling (whole rows, or a tile).  Keeping the lane part
// in one register and the rest constant lets every read of a tile reuse that
// register, with the constant in the instruction's offset field; computing
// the full swizzled offset per read instead costs one address register per
// distinct read.
//
// 128-bit read: one MFMA operand fragment (8 bf16 of one row) per lane.
__device__ __forceinline__ uint4 lds_read_b128_at(const __bf16* base, uint32_t lane_off,
                                                  uint32_t const_off) {
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = *(const FA_LDS u32x4*)((const FA_LDS char*)(const FA_LDS __bf16*)base +
                                         lane_off + const_off);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address
// of 4 consecutive bf16 (row j/4 of a 4-row block, columns 4*(j%4)..+3) and
// receives column j of that 4 x 16 block (one element from each of the 4
// rows).  Used to read V (or K, Q, dO) transposed for MFMA operands.
__device__ __forceinline__ bf16x4 lds_read_tr_at(const __bf16* base, uint32_t lane_off,
                                                 uint32_t const_off) {
  i16x4 t = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (FA_LDS i16x4*)((FA_LDS char*)(FA_LDS __bf16*)base + lane_off + const_off));
  return __builtin_bit_cast(bf16x4, t);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

// ---------------------------------------------------------------- LDS DMA
// Buffer loads that write straight into LDS (buffer_load_dwordx4 ... lds):
// lane l of a wave deposits its 16 bytes at lds_base + 16 l, so one wave
// instruction fills 1 KB of LDS.  The buffer descriptor bounds every access:
// a lane whose offset is past num_records reads zeros, which is how rows
// beyond the end of a sequence are zero-filled without a branch.
constexpr int kBufferRsrcWord3 = 0x00020000;  // gfx9-family raw buffer, 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_bytes,
                                           kBufferRsrcWord3);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, __bf16* lds_base,
                                      uint32_t voffset, uint32_t soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (FA_LDS void*)lds_base, 16, (int)voffset,
                                           (int)soffset, 0, 0);
}

// Per-lane byte offsets for staging a [ROWS x D] bf16 tile whose rows are
// `stride_bytes` apart in global memory into a swizzled LDS tile with
// WAVES waves.  Wave w issues instructions w*PER_WAVE .. +PER_WAVE-1; each
// instruction covers 1024 / (2 D) consecutive rows of the LDS tile, and lane
// l fills physical chunk l % (D/8) of its row, i.e. logical chunk
// (l % (D/8)) ^ swz(row).
template <int D, int ROWS, int WAVES>
struct TileDma {
  static constexpr int kChunks = D / 8;                 // 16-byte chunks per row
  static constexpr int kRowsPerInst = 64 / kChunks;     // rows per 1 KB instruction
  static constexpr int kInsts = ROWS / kRowsPerInst;    // instructions per tile
  static constexpr int kPerWave = kInsts / WAVES;
  static_assert(kInsts % WAVES == 0, "tile must split evenly over the waves");
  uint32_t voff[kPerWave];
  int first;  // first instruction index of this wave
  __device__ __forceinline__ TileDma(int wave, int lane, uint32_t stride_bytes) {
    first = wave * kPerWave;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int row = (first + i) * kRowsPerInst + lane / kChunks;
      const int chunk = (lane % kChunks) ^ swz<D>(row);
      voff[i] = (uint32_t)row * stride_bytes + (uint32_t)chunk * 16u;
    }
  }
  // Stage rows [j0, j0 + ROWS) of a tensor whose row 0 is at `g`; rows at or
  // past `limit` read as zero.  The descriptor spans at most the tile's own
  // rows, so its 32-bit byte range cannot wrap however far `limit` lies
  // beyond the tile (a tensor can exceed 4 GiB).
  __device__ __forceinline__ void issue(const __bf16* g, uint32_t stride_bytes, int j0,
                                        int limit, __bf16* lds) const {
    const int valid = min(limit - j0, ROWS);  // >= 1 inside the loops that call this
    const uint32_t nbytes = (uint32_t)(valid - 1) * stride_bytes + (uint32_t)D * 2u;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(g + (int64_t)j0 * (stride_bytes / 2), nbytes);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) dma16(r, lds + (first + i) * 512, voff[i]);
  }
};

// Additive-bias block of one wave: its 32 rows r0 .. r0 + 31 (lane row r32)
// from column j0 on, read four consecutive fp32 entries per load.  One
// buffer descriptor spans the block up to the last valid element (row lq - 1,
// column lk - 1), so a load in a row past the sequence, or past its last key
// in that last row, returns 0 with no branch; in the other rows, keys past
// the end read the next row's entries, which the key mask discards.  The
// byte range is at most (31 sq + lk) x 4, which the C API bounds below 2^32.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bias_rsrc(const float* bias_bh, int64_t sq,
                                                            int r0, int lq, int j0, int lk) {
  const int rows = min(lq - r0, 32);
  const uint32_t nbytes = rows > 0 ? (uint32_t)(((int64_t)(rows - 1) * sq + (lk - j0)) * 4) : 0u;
  return make_rsrc(bias_bh + (int64_t)r0 * sq + j0, nbytes);
}
// Entries (row r0 + r32, columns j0 + col .. + 3); lane_off = (r32 sq) x 4.
__device__ __forceinline__ f32x4 bias_load4(__amdgpu_buffer_rsrc_t rs, uint32_t lane_off,
                                            int col) {
  return __builtin_bit_cast(
      f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)(lane_off + (uint32_t)col * 4u), 0, 0));
}

// Barrier that publishes LDS-DMA data to the whole work-group: every wave
// first waits for its own outstanding buffer->LDS loads (vmcnt 0), then all
// waves meet.  The compiler's automatic waits only order a wave's reads after
// its own loads, which is not enough when other waves' loads fill the tile.
__device__ __forceinline__ void dma_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Stage synchronisation for race hunting.  Built with -DFA_DEBUG_SYNC,
// every staged copy completes (vmcnt 0) and the whole work-group meets after
// each copy is issued and after each tile is computed, so no copy into LDS
// overlaps any read of LDS; the optimised build must give the same bits.
// Without the macro it is nothing.
#ifdef FA_DEBUG_SYNC
#define FA_STAGE_SYNC()                                \
  do {                                                 \
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   \
    __syncthreads();                                   \
  } while (0)
#else
#define FA_STAGE_SYNC() \
  do {                  \
  } while (0)
#endif

// ---------------------------------------------------------------- scheduling
// Instruction-class masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008, kSchedDsRead = 0x100;

// ---------------------------------------------------------------- grid
// Work-groups are dispatched round-robin over the 8 XCDs (wg % 8), each with
// its own L2.  Renumber them so that a contiguous range of logical ids runs
// on one XCD: work that shares K/V (the query heads of one KV head) then
// shares that XCD's L2.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t wg, uint32_t n) {
  uint32_t xcd = wg % kNumXcd, slot = wg / kNumXcd;
  uint32_t per = n / kNumXcd, rem = n % kNumXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// Rows of one sequence of a dense or packed batch.
struct SeqSpan {
  int64_t q0, k0;  // first token row of the sequence in Q and in K/V
  int lq, lk;      // its query and key lengths
};

__device__ __forceinline__ SeqSpan seq_span(const int32_t* cu, int b, int nq,
                                            int nk) {
  SeqSpan s;
  if (cu) {
    int a = cu[b], e = cu[b + 1];
    s.q0 = s.k0 = a;
    s.lq = s.lk = e - a;
  } else {
    s.q0 = (int64_t)b * nq;
    s.k0 = (int64_t)b * nk;
    s.lq = nq;
    s.lk = nk;
  }
  return s;
}

// Index of (head h, token row t of sequence b) in an LSE-shaped fp32 array:
// dense [B, Hq, Nq], packed [Hq, T].
__device__ __forceinline__ int64_t lse_index(const int32_t* cu, int B, int Hq,
                                             int Nq, int b, int h, int64_t q0,
                                             int i) {
  if (cu) return (int64_t)h * cu[B] + q0 + i;
  return ((int64_t)b * Hq + h) * Nq + i;
}

// ---------------------------------------------------------------- dropout
// Counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011).  Per round the
// counter words (c0, c1, c2, c3) become
//     (hi(B * c2) ^ c1 ^ k0,  lo(B * c2),  hi(A * c0) ^ c3 ^ k1,  lo(A * c0))
// with A = 0xD2511F53, B = 0xCD9E8D57 and 64-bit products; the key (k0, k1)
// advances by (0x9E3779B9, 0xBB67AE85) between rounds.  The key is uniform
// over the wave (scalar registers); the counter is per lane.
__device__ __forceinline__ uint4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                               uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t a = (uint64_t)0xD2511F53u * c0;
    const uint64_t m = (uint64_t)0xCD9E8D57u * c2;
    // three-input XORs as one v_bitop3_b32 each (truth table 0x96)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(m >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(a >> 32), c3, k1, 0x96);
    c1 = (uint32_t)m;
    c3 = (uint32_t)a;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return make_uint4(c0, c1, c2, c3);
}

// Dropout generator call shared by the keys 16m + 4t + {0..3, 8..11} of
// query row i of (sequence b, query head h), for any such key j
// (m = j >> 4, t = (j >> 2) & 1): counter (2m + t, i, h, b).  Key j takes
// slot s = 4 ((j >> 3) & 1) + (j & 3): the 16-bit half s & 1 (0 low) of
// output word s >> 1, and is kept iff that half >= the 16-bit threshold.
__device__ __forceinline__ uint4 drop_call(int j, int i, int h, int b, uint32_t seed_lo,
                                           uint32_t seed_hi) {
  const uint32_t c0 = 2u * ((uint32_t)j >> 4) + (((uint32_t)j >> 2) & 1u);
  return philox4x32_10(c0, (uint32_t)i, (uint32_t)h, (uint32_t)b, seed_lo, seed_hi);
}
__device__ __forceinline__ uint32_t word_of(const uint4& w, int e) {  // e unrolled
  return e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
}
__device__ __forceinline__ uint32_t slot_of(const uint4& w, int s) {  // s unrolled, 0..7
  const uint32_t x = word_of(w, s >> 1);
  return (s & 1) ? (x >> 16) : (x & 0xFFFFu);
}

// Value of x in lane (l & ~3) + E: a broadcast inside each quad of lanes
// (DPP quad_perm, a VALU move).
template <int E>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, E | (E << 2) | (E << 4) | (E << 6),
                                               0xF, 0xF, false);
}

// Visibility of key j from query i (sequence-relative), delta = lk - lq.
template <bool CAUSAL, bool WINDOW>
__device__ __forceinline__ bool visible(int i, int j, int delta, int lk,
                                        int window) {
  bool ok = j < lk;
  if (CAUSAL) ok = ok && (j <= i + delta);
  if (WINDOW) ok = ok && (i + delta - j < window);
  return ok;
}

}  // namespace fa

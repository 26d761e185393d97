// FP8 (OCP E4M3) attention forward and the block quantizer that feeds it.
//
// llms.blog "FlashAttention: How IO-Aware Tiling and Online Softmax Solved
// Transformer Memory Bottlenecks", "FlashAttention-3: Asynchronous Execution
// on Hopper Architectures": the FP8 variant doubles the matrix throughput
// and keeps the error in check with block quantization and incoherent
// processing.  On gfx950 the 8-bit product is v_mfma_f32_32x32x64_f8f6f4
// (twice the bf16 rate, four times the work per instruction).
//
// Quantizer (one work-group per block of 64 tokens of one head): optional
// rotation x -> x D H / sqrt(d) of each row (random signs D from the
// caller, Sylvester-Hadamard H by butterflies: within a thread, then across
// the four lanes that hold one row), block amax, scale amax / 448, codes
// RNE_e4m3(clamp(x * (448 / amax))) -- every decision in fp32.  Q and K keep
// their token-major layout; V is written transposed ([B, H, d, keys], keys
// padded to a multiple of 64 with zeros) because the P V product reads V as
// its A operand with keys along the contraction, and 8-bit operands have no
// transposing read that would serve it.
//
// Attention: the bf16 forward's structure (fa_fwd_kernel.h) with 8-bit
// operands.  A wave owns 32 query rows; S^T = K Q^T and O^T += V^T P^T run on
// the x64 8-bit MFMA.  The K tile's rows are read in the order k8_row so that
// the S^T result gives each lane half 32 consecutive keys, exactly the K
// slots of the P operand: P is exponentiated, rounded to E4M3 and used in
// place.  Per-tile factors carry the block scales: the score multiplier is
// scale * log2(e) * sQ * sK(tile) (one multiply per tile), and V's block
// scale enters P's exponent as log2(sV(tile) / sV_ref), sV_ref the largest V
// scale the work-group visits, so that every P stays <= 2^(7 + 1.5) < 448
// and the accumulator needs no per-tile rescale; the normaliser l takes the
// tile's partial sum times sV_ref / sV(tile).  The running maximum is raised
// lazily (only when a row maximum grows by more than 1.5 in log2 units): P
// then stays within E4M3's range with 2^7 of headroom, so probabilities down
// to 2^-13 of the maximum remain normal numbers.

#include "fa_device.h"

namespace fa {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kBN8 = 64;             // keys per tile = tokens per scale block
constexpr float kSlack8 = 1.5f;      // log2 growth of a row maximum before rescaling
constexpr float kPHead8 = 7.0f;      // P is rounded as P * 2^7 (times sV / sV_ref)

// v_mfma_f32_32x32x64_f8f6f4 with both operands E4M3 (format 0), unscaled.
// Operand bytes: lane l holds row (A) or column (B) l % 32 and 32 K slots
// chosen by l / 32; A and B map bytes to K slots the same way, so any byte
// order works as long as both operands use it.
__device__ __forceinline__ f32x16 mfma_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

__device__ __forceinline__ i32x8 cat8(uint4 lo, uint4 hi) {
  i32x8 r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Four fp32 values rounded to E4M3 (v_cvt_pk_fp8_f32, nearest even), byte
// e of the result from value e.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float d) {
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// Buffer-to-LDS staging of a tile of ROWS rows of ROW_BYTES bytes (rows
// `stride` bytes apart in global memory) into a row-major LDS tile whose
// 16-byte chunks are permuted by `swz(row)`; as TileDma in fa_device.h, one
// wave instruction fills 1 KB.
template <int ROW_BYTES, int ROWS, int WAVES>
struct ByteTileDma {
  static constexpr int kChunks = ROW_BYTES / 16;
  static constexpr int kRowsPerInst = 64 / kChunks;
  static constexpr int kInsts = ROWS / kRowsPerInst;
  static constexpr int kPerWave = kInsts / WAVES;
  static_assert(kInsts % WAVES == 0, "tile must split evenly over the waves");
  uint32_t voff[kPerWave];
  int first;
  template <typename Swz>
  __device__ __forceinline__ ByteTileDma(int wave, int lane, uint32_t stride, Swz swz) {
    first = wave * kPerWave;
#pragma unroll
    for (int i = 0; i < kPerWave; ++i) {
      const int row = (first + i) * kRowsPerInst + lane / kChunks;
      const int chunk = (lane % kChunks) ^ swz(row);
      voff[i] = (uint32_t)row * stride + (uint32_t)chunk * 16u;
    }
  }
  // rows [0, valid) of the tile whose row 0 is at g; rows past `valid` read
  // as zero (the descriptor ends at the last valid row)
  __device__ __forceinline__ void issue(const uint8_t* g, uint32_t stride, int valid,
                                        uint8_t* lds) const {
    const uint32_t nbytes = (uint32_t)(valid - 1) * stride + (uint32_t)ROW_BYTES;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(g, nbytes);
#pragma unroll
    for (int i = 0; i < kPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (FA_LDS void*)(lds + (first + i) * 1024), 16,
                                               (int)voff[i], 0, 0, 0);
  }
};

// ------------------------------------------------------------ attention
// Four waves (128 query rows) per work-group: the compiler fits the d = 128
// instances in 162-168 registers, so three work-groups share a CU (32 KB of
// LDS each) and three waves a SIMD.  The kernel is bound by vector issue
// (the softmax is as long as in the bf16 kernel while the products take half
// the time), and a third wave fills more of the matrix core's idle cycles:
// 0.323 ms on the GQA prefill shape against 0.384 ms with eight-wave
// work-groups (one per CU, two waves per SIMD).  Asking for three waves per
// SIMD outright made the compiler spill 8-12 bytes per lane instead.
template <int D, int W, bool CAUSAL, bool WINDOW>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_fp8_kernel(Fp8FwdParams p) {
  constexpr int KS = D / 64;   // k-steps of the Q K^T contraction
  constexpr int DB = D / 32;   // 32-column blocks of the output
  constexpr int kBM = 32 * W;
  constexpr float kInf = __builtin_inff();

  __shared__ __attribute__((aligned(1024))) uint8_t k0[kBN8 * D];
  __shared__ __attribute__((aligned(1024))) uint8_t v0[D * kBN8];
  __shared__ __attribute__((aligned(1024))) uint8_t k1[kBN8 * D];
  __shared__ __attribute__((aligned(1024))) uint8_t v1[D * kBN8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  // ---- work partition: as the bf16 forward (KV head slowest, XCD ranges)
  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int G = p.group;
  const int gi = id % G;
  id /= G;
  const int t_ord = id % p.num_qtiles;
  id /= p.num_qtiles;
  const int b = id % p.B;
  const int hkv = id / p.B;
  const int h = hkv * G + gi;
  const int qt = CAUSAL ? (p.num_qtiles - 1 - t_ord) : t_ord;
  const int q_start = qt * kBM;
  if (q_start >= p.Nq) return;
  const int delta = p.Nk - p.Nq;
  const int q_end = min(q_start + kBM, p.Nq);
  int kv_lo = 0, kv_hi = p.Nk;
  if (CAUSAL) kv_hi = min(kv_hi, q_end + delta);
  if (WINDOW) kv_lo = max(0, q_start + delta - p.window + 1);
  kv_lo = (kv_lo / kBN8) * kBN8;

  const uint32_t kstride = (uint32_t)p.Hkv * D;
  const uint8_t* Kg = p.k + (int64_t)b * p.Nk * kstride + (int64_t)hkv * D;
  const uint8_t* Vg = p.v + ((int64_t)b * p.Hkv + hkv) * D * p.ldv;
  const ByteTileDma<D, kBN8, W> kdma(wave, lane, kstride, [](int r) { return swz_k8<D>(r); });
  const ByteTileDma<kBN8, D, W> vdma(wave, lane, (uint32_t)p.ldv,
                                     [](int r) { return swz_v8(r); });
  auto issue = [&](int j0, uint8_t* kb, uint8_t* vb) {
    kdma.issue(Kg + (int64_t)j0 * kstride, kstride, min(p.Nk - j0, kBN8), kb);
    vdma.issue(Vg + j0, (uint32_t)p.ldv, D, vb);
  };
  if (kv_lo < kv_hi) issue(kv_lo, k0, v0);
  FA_STAGE_SYNC();

  // ---- block scales of K and V for this (sequence, KV head); the largest V
  // scale of the visited tiles is the reference that keeps P <= 2^8.5
  const float* skp = p.sk + ((int64_t)b * p.Hkv + hkv) * p.nbk;
  const float* svp = p.sv + ((int64_t)b * p.Hkv + hkv) * p.nbk;
  float sref = 0.f;
  for (int t = kv_lo / kBN8 + lane; t * kBN8 < kv_hi; t += 64) sref = fmaxf(sref, svp[t]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) sref = fmaxf(sref, __shfl_xor(sref, off, 64));
  const float lsref = __log2f(sref);

  // ---- Q fragments (B operand of S^T): query qi, d bytes 64 st + 32 hl ..
  const int qi = q_start + wave * 32 + r32;
  i32x8 qf[KS];
  if (qi < p.Nq) {
    const uint8_t* qp = p.q + (((int64_t)b * p.Nq + qi) * p.Hq + h) * D + hl * 32;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qf[st] = cat8(*reinterpret_cast<const uint4*>(qp + 64 * st),
                    *reinterpret_cast<const uint4*>(qp + 64 * st + 16));
  } else {
#pragma unroll
    for (int st = 0; st < KS; ++st)
      for (int e = 0; e < 8; ++e) qf[st][e] = 0;
  }
  const int qblk = min((q_start + wave * 32) / kBN8, p.nbq - 1);
  // The tile loop always takes the row maximum with a positive multiplier:
  // a negative scale is applied as |scale| to -Q (the E4M3 sign bits
  // flipped, exact), so no runtime branch separates the score products from
  // the softmax.
  float c_q = p.scale_log2 * p.sq[((int64_t)b * p.Hq + h) * p.nbq + qblk];
  if (c_q < 0.f) {
    c_q = -c_q;
#pragma unroll
    for (int st = 0; st < KS; ++st) qf[st] = qf[st] ^ (int)0x80808080u;
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m_run = -kInf;  // reference maximum, log2 units
  float l_run = 0.f;    // this half-wave's share of 2^7 * sum_j 2^(x_j - m)

  const int qlo_w = q_start + wave * 32;
  const int qhi_w = min(qlo_w + 31, p.Nq - 1);
  // Lane parts of the LDS read offsets; key block kb adds 16 rows and output
  // block db 32 rows, neither of which changes the swizzle (a constant).
  uint32_t koff[KS][2], voff[2];
#pragma unroll
  for (int st = 0; st < KS; ++st)
#pragma unroll
    for (int u = 0; u < 2; ++u) koff[st][u] = k8_off<D>(k8_row(0, r32), 64 * st + 32 * hl + 16 * u);
#pragma unroll
  for (int u = 0; u < 2; ++u) voff[u] = v8_off(r32, 32 * hl + 16 * u);

  auto compute = [&](int j0, const uint8_t* kt, const uint8_t* vt) {
    bool active = qlo_w <= qhi_w;
    if (CAUSAL) active = active && (j0 <= qhi_w + delta);
    if (WINDOW) active = active && (j0 + kBN8 - 1 > qlo_w + delta - p.window);
    if (!active) return;
    bool need_mask = (j0 + kBN8 > p.Nk);
    if (CAUSAL) need_mask = need_mask || (j0 + kBN8 - 1 > qlo_w + delta);
    if (WINDOW) need_mask = need_mask || (qhi_w + delta - j0 >= p.window);
    const int tile = j0 / kBN8;
    // score -> log2 units; kept >= 1e-30 so that a masked score (-inf)
    // exponentiates to exactly 0 even if the product underflows (with it
    // every exp2(s cs - m) of such a tile still rounds as with cs = 0)
    const float cs = fmaxf(c_q * skp[tile], 1e-30f);
    const float lr = __log2f(svp[tile]) - lsref;      // <= 0: this tile's V scale
    const float lsc = fast_exp2(-lr);                 // sV_ref / sV(tile)

    // S^T for key blocks kb: lane half hl gets keys j0 + 32 hl + 16 kb + i
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const uint32_t rows = kb * 16 * D;
        const i32x8 a = cat8(lds_read_b128_at((const __bf16*)kt, koff[st][0], rows),
                             lds_read_b128_at((const __bf16*)kt, koff[st][1], rows));
        s[kb] = mfma_fp8(a, qf[st], s[kb]);
      }

    // A tile that straddles a mask boundary first sets each invisible score
    // to -inf (never the row maximum; exp2 of it is exactly 0), in a
    // separate, rarely taken block; then every tile takes the same update.
    auto key_of = [&](int kb, int i) { return j0 + 32 * hl + 16 * kb + i; };
    if (__builtin_expect(need_mask, 0)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!visible<CAUSAL, WINDOW>(qi, key_of(kb, i), delta, p.Nk, p.window))
            s[kb][i] = -kInf;
    }
    {
      float rm = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) rm = fmaxf(rm, s[kb][i]);
      rm = max_halves(rm);
      const float tmax = __builtin_isinf(rm) ? -kInf : rm * cs;
      float m_use = m_run;
      if (tmax > m_run + kSlack8) m_use = tmax;  // also when m_run = -inf
      const float m_sub = (m_use == -kInf) ? 0.f : m_use;
      const float alpha = fast_exp2(m_run - m_sub);
      m_run = m_use;
      l_run *= alpha;
      if (__ballot(alpha != 1.0f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }
      // P * 2^7 * sV(tile) / sV_ref, rounded to E4M3: byte 16 kb + i of the
      // P operand is key 32 hl + 16 kb + i, the K slot V^T uses for it
      const float neg = kPHead8 + lr - m_sub;
      i32x8 pk;
      float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 4) {
          float e[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) e[u] = fast_exp2(fmaf(s[kb][i + u], cs, neg));
          lsum0 += e[0] + e[2];
          lsum1 += e[1] + e[3];
          pk[kb * 4 + i / 4] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
      l_run = fmaf(lsum0 + lsum1, lsc, l_run);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t rows = db * 32 * kBN8;
        const i32x8 a = cat8(lds_read_b128_at((const __bf16*)vt, voff[0], rows),
                             lds_read_b128_at((const __bf16*)vt, voff[1], rows));
        acc[db] = mfma_fp8(a, pk, acc[db]);
      }
    }
  };

  // ---- main loop over K/V tiles, two buffers
  for (int j0 = kv_lo; j0 < kv_hi; j0 += 2 * kBN8) {
    dma_barrier();
    if (j0 + kBN8 < kv_hi) issue(j0 + kBN8, k1, v1);
    FA_STAGE_SYNC();
    compute(j0, k0, v0);
    FA_STAGE_SYNC();
    if (j0 + kBN8 >= kv_hi) break;
    dma_barrier();
    if (j0 + 2 * kBN8 < kv_hi) issue(j0 + 2 * kBN8, k0, v0);
    FA_STAGE_SYNC();
    compute(j0 + kBN8, k1, v1);
    FA_STAGE_SYNC();
  }

  // ---- epilogue: O = acc * sV_ref / l', LSE = ln 2 * (m + log2 l' - 7)
  const float l_tot = sum_halves(l_run);
  if (qi < p.Nq) {
    const float inv = (l_tot == 0.f) ? 0.f : sref / l_tot;
    __bf16* op = (__bf16*)p.o + (((int64_t)b * p.Nq + qi) * p.Hq + h) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 w = pack4_t<false>(acc[db][4 * r + 0] * inv, acc[db][4 * r + 1] * inv,
                                       acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + r * 8 + hl * 4) = w;
      }
    if (hl == 0) {
      const float m_sub = (m_run == -kInf) ? 0.f : m_run;
      const float lse = (l_tot == 0.f) ? -kInf : (m_sub + __log2f(l_tot) - kPHead8) * kLn2;
      p.lse[((int64_t)b * p.Hq + h) * p.Nq + qi] = lse;
    }
  }
}

template <int D, int W, bool CAUSAL, bool WINDOW>
hipError_t launch_fp8_w(Fp8FwdParams p, hipStream_t stream) {
  p.num_qtiles = (p.Nq + 32 * W - 1) / (32 * W);
  dim3 grid((unsigned)p.B * p.Hq * p.num_qtiles), block(64 * W);
  hipLaunchKernelGGL((fwd_fp8_kernel<D, W, CAUSAL, WINDOW>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D, int W>
hipError_t launch_fp8_d(const Fp8FwdParams& p, hipStream_t stream) {
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch_fp8_w<D, W, true, true>(p, stream)
               : launch_fp8_w<D, W, true, false>(p, stream);
  return win ? launch_fp8_w<D, W, false, true>(p, stream)
             : launch_fp8_w<D, W, false, false>(p, stream);
}

// ------------------------------------------------------------ quantizer
// One work-group of 256 threads per block of 64 tokens of one head; thread
// (r, part) holds token r's d/4 values part * d/4 .. (a row sits in four
// adjacent lanes).
template <int D, bool ROT, bool TRANSPOSE>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(QuantParams p) {
  constexpr int PER = D / 4;
  constexpr int kPitch = D + 4;  // LDS row pitch of the transpose staging
  __shared__ float red[4];
  __shared__ __attribute__((aligned(16))) uint8_t tr[TRANSPOSE ? 64 * kPitch : 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t id = blockIdx.x;
  const int t = id % p.nb;
  id /= p.nb;
  const int h = id % p.H;
  const int b = id / p.H;
  const int r = tid >> 2, part = tid & 3;
  const int n = t * 64 + r;

  float x[PER];
  if (n < p.N) {
    const uint4* src = reinterpret_cast<const uint4*>(
        (const __bf16*)p.x + (((int64_t)b * p.N + n) * p.H + h) * D + part * PER);
#pragma unroll
    for (int c = 0; c < PER / 8; ++c) {
      const bf16x8 v = as_bf16x8(src[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[8 * c + e] = (float)v[e];
    }
  } else {
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] = 0.f;
  }

  if constexpr (ROT) {
    // x D, then the Sylvester-Hadamard butterflies (a, c) -> (a + c, a - c)
    // over each bit of the column index: the low bits inside the thread,
    // the top two across the row's four lanes, then 1 / sqrt(d)
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] *= p.signs[part * PER + e];
#pragma unroll
    for (int hs = 1; hs < PER; hs <<= 1)
#pragma unroll
      for (int e = 0; e < PER; ++e)
        if (!(e & hs)) {
          const float a = x[e], c = x[e + hs];
          x[e] = a + c;
          x[e + hs] = a - c;
        }
#pragma unroll
    for (int m = 1; m <= 2; m <<= 1) {
      const bool upper = (part & m) != 0;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const float o = __shfl_xor(x[e], m, 64);
        x[e] = upper ? (o - x[e]) : (x[e] + o);
      }
    }
    const float norm = (D == 128) ? 0.08838834764831845f : 0.125f;  // 1 / sqrt(d)
#pragma unroll
    for (int e = 0; e < PER; ++e) x[e] *= norm;
  }

  float am = 0.f;
#pragma unroll
  for (int e = 0; e < PER; ++e) am = fmaxf(am, fabsf(x[e]));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
  if (lane == 0) red[wave] = am;
  __syncthreads();
  am = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // blocks below 2^-119 (448 / amax would overflow) quantize to zero, scale 1
  float scale = 1.0f, inv = 0.0f;
  if (am >= 0x1p-119f) {
    scale = am / 448.0f;
    inv = 448.0f / am;
  }
  if (tid == 0) p.scales[((int64_t)b * p.H + h) * p.nb + t] = scale;

  uint32_t w[PER / 4];
#pragma unroll
  for (int e = 0; e < PER; e += 4) {
    float y[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      y[u] = x[e + u] * inv;
      y[u] = y[u] > 448.0f ? 448.0f : (y[u] < -448.0f ? -448.0f : y[u]);
    }
    w[e / 4] = (uint32_t)pack_fp8x4(y[0], y[1], y[2], y[3]);
  }

  if constexpr (!TRANSPOSE) {
    if (n < p.N) {
      uint4* dst = reinterpret_cast<uint4*>(p.x8 + (((int64_t)b * p.N + n) * p.H + h) * D +
                                            part * PER);
#pragma unroll
      for (int c = 0; c < PER / 16; ++c)
        dst[c] = make_uint4(w[4 * c], w[4 * c + 1], w[4 * c + 2], w[4 * c + 3]);
    }
  } else {
    // stage the 64 x d codes (rows past N are zero), then write d rows of 64
    // keys: output row dc of this block = column dc of the staged tile
#pragma unroll
    for (int c = 0; c < PER / 4; ++c)
      *reinterpret_cast<uint32_t*>(tr + r * kPitch + part * PER + 4 * c) = w[c];
    __syncthreads();
    for (int c = tid; c < D * 4; c += 256) {
      const int dc = c >> 2, q = c & 3;
      uint32_t o[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t v = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) v |= (uint32_t)tr[(16 * q + 4 * k + j) * kPitch + dc] << (8 * j);
        o[k] = v;
      }
      *reinterpret_cast<uint4*>(p.x8 + (((int64_t)b * p.H + h) * D + dc) * p.ldn + t * 64 +
                                16 * q) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

template <int D>
hipError_t launch_quant_d(const QuantParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.B * p.H * p.nb), block(256);
  if (p.signs) {
    if (p.transpose)
      hipLaunchKernelGGL((quantize_fp8_kernel<D, true, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((quantize_fp8_kernel<D, true, false>), grid, block, 0, stream, p);
  } else {
    if (p.transpose)
      hipLaunchKernelGGL((quantize_fp8_kernel<D, false, true>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((quantize_fp8_kernel<D, false, false>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream) {
  return p.d == 128 ? launch_fp8_d<128, 4>(p, stream) : launch_fp8_d<64, 4>(p, stream);
}

hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream) {
  return p.d == 128 ? launch_quant_d<128>(p, stream) : launch_quant_d<64>(p, stream);
}

}  // namespace fa

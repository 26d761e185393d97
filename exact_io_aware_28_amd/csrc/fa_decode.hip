// Split-KV attention for a few query rows per sequence over a long key/value
// cache (single-token decode, short chunked prefill), bf16 in / bf16 out.
//
// klaylearn.com glossary "flash-attention", "Does FlashAttention speed up
// every LLM inference path?": with one new query position the cost is
// streaming the cached keys and values, not the score matrix.  So the grid
// runs over key ranges instead of query tiles:
//   1. decode_split: one wave per (sequence, KV head, 32-row block, key
//      split).  Its 32 rows are the (query head of the group, query position)
//      pairs of that KV head, so every K/V byte is read once for the whole
//      group.  It runs the online softmax of llms.blog "FlashAttention: How
//      IO-Aware Tiling and Online Softmax Solved Transformer Memory
//      Bottlenecks", "2. Online Softmax Reduction" over its key range and
//      writes a normalised partial output and its logsumexp.
//   2. decode_combine: one wave per (sequence, position, head) merges the
//      splits the way the recurrence merges two blocks: with LSE_s the
//      partial logsumexps, LSE = ln sum_s e^{LSE_s} and
//      O = sum_s e^{LSE_s - LSE} O_s (an empty split has LSE_s = -inf).
// Tiles of 32 keys go from HBM into LDS with buffer loads that write LDS
// directly, two buffers per wave; the products use the same transposed
// MFMA formulation, LDS swizzle and key permutation as the prefill kernel.

#include "fa_device.h"

namespace fa {
namespace {

constexpr int kDecBN = 32;  // keys per K/V tile
constexpr int kDecThreads = 64;
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest unrescaled score

template <int D, bool CAUSAL, bool WINDOW>
// at most 256 registers, so that two waves share a SIMD: with 32 KB of LDS
// per wave five fit a CU, and more tiles are in flight per CU
__global__ __launch_bounds__(kDecThreads) __attribute__((amdgpu_waves_per_eu(2)))
void decode_split_kernel(DecodeParams p) {
  constexpr int KS = D / 16;  // k-steps of the QK^T contraction
  constexpr int DB = D / 32;  // 32-column blocks of the output
  constexpr float kInf = __builtin_inff();
  __shared__ __attribute__((aligned(1024))) __bf16 k0[kDecBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v0[kDecBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 k1[kDecBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v1[kDecBN * D];

  const int lane = threadIdx.x, hl = lane >> 5, r32 = lane & 31;
  uint32_t id = blockIdx.x;
  const int split = id % p.num_splits;
  id /= p.num_splits;
  const int rb = id % p.row_blocks;
  id /= p.row_blocks;
  const int hkv = id % p.Hkv;
  const int b = id / p.Hkv;
  const int G = p.group, Nq = p.Nq;
  const int L = p.seqlens_k ? min(max(p.seqlens_k[b], 0), p.Nk) : p.Nk;
  const int delta = L - Nq;  // bottom-right alignment of query positions

  // this lane's row of the block: (query head g of the group, position i)
  const int R = rb * 32 + r32;
  const bool row_ok = R < G * Nq;
  const int g = row_ok ? R / Nq : 0;
  const int i = row_ok ? R % Nq : 0;
  const int h = hkv * G + g;

  // keys any row of the block can see, split into equal 32-key-aligned
  // ranges; a row at position i sees keys j < L with j <= i + delta (causal)
  // and i + delta - j < window
  int lo = 0;
  if (WINDOW) lo = max(0, delta - p.window + 1);
  lo = (lo / kDecBN) * kDecBN;
  const int hi = L;
  const int span = max(hi - lo, 0);
  const int per = ((span + p.num_splits - 1) / p.num_splits + kDecBN - 1) / kDecBN * kDecBN;
  const int s_lo = lo + split * per;
  const int s_hi = min(hi, s_lo + per);
  const int ntiles = (s_hi > s_lo) ? (s_hi - s_lo + kDecBN - 1) / kDecBN : 0;

  const int64_t kstride = (int64_t)p.Hkv * D;
  const uint32_t kstride_b = (uint32_t)(kstride * 2);
  const __bf16* Kg = (const __bf16*)p.k + (int64_t)b * p.Nk * kstride + (int64_t)hkv * D;
  const __bf16* Vg = (const __bf16*)p.v + (int64_t)b * p.Nk * kstride + (int64_t)hkv * D;
  const TileDma<D, kDecBN, 1> dma(0, lane, kstride_b);
  auto issue = [&](int t, __bf16* kb, __bf16* vb) {
    dma.issue(Kg, kstride_b, s_lo + t * kDecBN, L, kb);
    dma.issue(Vg, kstride_b, s_lo + t * kDecBN, L, vb);
  };
  if (ntiles > 0) issue(0, k0, v0);
  FA_STAGE_SYNC();

  // Q fragments (B operand of S^T = K Q^T): this lane's row, 8 columns per step
  bf16x8 qf[KS];
  if (row_ok) {
    const __bf16* qp = (const __bf16*)p.q + (((int64_t)b * Nq + i) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qf[st] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * st));
  } else {
#pragma unroll
    for (int st = 0; st < KS; ++st) qf[st] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  // lane byte offsets of the LDS reads inside a tile (rows or columns added
  // as compile-time constants): K fragments per k-step, transposed V reads
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  uint32_t koff[KS], voff[2][DB];
#pragma unroll
  for (int st = 0; st < KS; ++st) koff[st] = 2 * tile_off<D>(r32, st * 16 + hl * 8);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[h2][db] = 2 * tile_off<D>(tr_row + 8 * h2, db * 32 + tr_col);

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[db][e] = 0.f;
  float m_run = -kInf;  // reference maximum, log2 units
  float l_run = 0.f;    // this half-wave's share of the normaliser
  // The loop takes the row maximum with a positive multiplier: a negative
  // scale is applied as |scale| to -Q (sign bits flipped, exact), a zero
  // scale as a tiny positive one (every exp2(s c - m) still rounds to 1).
  float c = p.scale_log2;
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      qf[st] = as_bf16x8(__builtin_bit_cast(uint4, qf[st]) ^
                         make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u));
  }
  if (c == 0.f) c = 1e-30f;

  auto compute = [&](int j0, const __bf16* kt, const __bf16* vt) {
    // S^T: element e holds key j0 + 8(e/4) + 4hl + e%4 for this lane's row
    f32x16 s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st)
      s = mfma32(as_bf16x8(lds_read_b128_at(kt, koff[st], 0)), qf[st], s);

    // a tile straddling the sequence end, the causal diagonal of some row or
    // the window start of some row is masked element by element: invisible
    // scores become -inf after scaling to log2 units
    bool need_mask = (j0 + kDecBN > L);
    if (CAUSAL) need_mask = need_mask || (j0 + kDecBN - 1 > delta);
    if (WINDOW) need_mask = need_mask || ((Nq - 1) + delta - j0 >= p.window);
    float ce = c;
    if (need_mask) {
      const int base = j0 + 4 * hl;
      const int end = L - base, lim = i + delta - base, wlo = i + delta - p.window - base;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = (e >> 2) * 8 + (e & 3);
        bool ok = off < end;
        if (CAUSAL) ok = ok && off <= lim;
        if (WINDOW) ok = ok && off > wlo;
        s[e] = ok ? s[e] * c : -kInf;
      }
      ce = 1.f;
    }
    // row maximum in log2 units (ce is positive)
    float rm = s[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) rm = fmaxf(rm, s[e]);
    rm = max_halves(rm);
    const float tmax = __builtin_isinf(rm) ? -kInf : rm * ce;
    float m_use = m_run;
    if (tmax > m_run + kRescaleSlack) m_use = tmax;  // also when m_run = -inf
    const float m_sub = (m_use == -kInf) ? 0.f : m_use;
    const float alpha = fast_exp2(m_run - m_sub);  // exactly 1 when unchanged
    m_run = m_use;
    l_run *= alpha;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[db][e] *= alpha;
    }
    // P V over the two 16-key chunks: slots 0..3 = keys 16kc + 4hl + {0..3},
    // 4..7 = 16kc + 8 + 4hl + {0..3}, matching the transposed V reads
    const float neg = -m_sub;
    float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pv[e] = fast_exp2(fmaf(s[kc * 8 + e], ce, neg));
        if (e & 1)
          lsum1 += pv[e];
        else
          lsum0 += pv[e];
      }
      const bf16x8 pb = pack_bf16x8(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const uint32_t ro = 16 * kc * D * 2;
        acc[db] = mfma32(cat(lds_read_tr_at(vt, voff[0][db], ro),
                             lds_read_tr_at(vt, voff[1][db], ro)),
                         pb, acc[db]);
      }
    }
    l_run += lsum0 + lsum1;
  };

  // one wave owns its two buffers: waiting for its own loads is enough
  for (int t = 0; t < ntiles; t += 2) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t is in buffer 0
    if (t + 1 < ntiles) issue(t + 1, k1, v1);
    FA_STAGE_SYNC();
    compute(s_lo + t * kDecBN, k0, v0);
    FA_STAGE_SYNC();
    if (t + 1 >= ntiles) break;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // tile t + 1 is in buffer 1
    if (t + 2 < ntiles) issue(t + 2, k0, v0);
    FA_STAGE_SYNC();
    compute(s_lo + (t + 1) * kDecBN, k1, v1);
    FA_STAGE_SYNC();
  }

  // normalised partial output and its logsumexp (an empty range: 0, -inf)
  const float l_tot = sum_halves(l_run);
  if (!row_ok) return;
  const float inv = (l_tot == 0.f) ? 0.f : 1.0f / l_tot;
  float* op = p.opart + ((((int64_t)split * p.B + b) * Nq + i) * p.Hq + h) * D;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float4 w;
      w.x = acc[db][4 * r + 0] * inv;
      w.y = acc[db][4 * r + 1] * inv;
      w.z = acc[db][4 * r + 2] * inv;
      w.w = acc[db][4 * r + 3] * inv;
      *reinterpret_cast<float4*>(op + db * 32 + r * 8 + hl * 4) = w;
    }
  if (hl == 0) {
    const float m_sub = (m_run == -kInf) ? 0.f : m_run;
    p.lpart[(((int64_t)split * p.B + b) * p.Hq + h) * Nq + i] =
        (l_tot == 0.f) ? -kInf : (m_sub + __log2f(l_tot)) * kLn2;
  }
}

// One wave per (sequence b, position i, head h); lane owns D/64 consecutive
// output columns.  The split logsumexps are read in parallel (lane s holds
// split s, 64 at a time) and reduced across the wave; the partial outputs
// are then accumulated four splits at a time so that their loads overlap.
template <int D>
__global__ __launch_bounds__(kDecThreads) void decode_combine_kernel(DecodeParams p) {
  constexpr int kPer = D / 64;
  constexpr float kInf = __builtin_inff();
  const int64_t row = blockIdx.x;  // (b * Nq + i) * Hq + h
  const int h = (int)(row % p.Hq);
  const int64_t bi = row / p.Hq;
  const int i = (int)(bi % p.Nq);
  const int b = (int)(bi / p.Nq);
  const int lane = threadIdx.x;
  const int ns = p.num_splits;
  const int64_t lstride = (int64_t)p.B * p.Hq * p.Nq;         // one split of lpart
  const int64_t ostride = (int64_t)p.B * p.Nq * p.Hq * D;     // one split of opart
  const float* lp = p.lpart + ((int64_t)b * p.Hq + h) * p.Nq + i;
  const float* opp = p.opart + row * D + lane * kPer;

  // maximum of the split logsumexps
  float mx = -kInf;
  for (int s0 = 0; s0 < ns; s0 += 64)
    if (s0 + lane < ns) mx = fmaxf(mx, lp[(int64_t)(s0 + lane) * lstride]);
#pragma unroll
  for (int m = 32; m > 0; m >>= 1) mx = fmaxf(mx, __shfl_xor(mx, m, 64));

  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  float sum = 0.f;
  if (mx != -kInf) {
    for (int s0 = 0; s0 < ns; s0 += 64) {
      // weight of split s0 + lane (0 for an empty split or past the end)
      const float ls = (s0 + lane < ns) ? lp[(int64_t)(s0 + lane) * lstride] : -kInf;
      const float w = (ls == -kInf) ? 0.f : expf(ls - mx);
      float ws = w;
#pragma unroll
      for (int m = 32; m > 0; m >>= 1) ws += __shfl_xor(ws, m, 64);
      sum += ws;
      const int n = min(64, ns - s0);
      int k = 0;
      for (; k + 4 <= n; k += 4) {
        float wk[4], v[4][kPer];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          wk[u] = __shfl(w, k + u, 64);
#pragma unroll
          for (int e = 0; e < kPer; ++e) v[u][e] = opp[(int64_t)(s0 + k + u) * ostride + e];
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int e = 0; e < kPer; ++e) o[e] = fmaf(wk[u], v[u][e], o[e]);
      }
      for (; k < n; ++k) {
        const float wk = __shfl(w, k, 64);
#pragma unroll
        for (int e = 0; e < kPer; ++e) o[e] = fmaf(wk, opp[(int64_t)(s0 + k) * ostride + e], o[e]);
      }
    }
  }
  const float inv = (sum > 0.f) ? 1.0f / sum : 0.f;
  __bf16* out = (__bf16*)p.o + row * D + lane * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) out[e] = (__bf16)(o[e] * inv);
  if (lane == 0) p.lse[((int64_t)b * p.Hq + h) * p.Nq + i] = (sum > 0.f) ? mx + logf(sum) : -kInf;
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch3(const DecodeParams& p, hipStream_t stream) {
  const uint64_t nsplit_wg = (uint64_t)p.num_splits * p.row_blocks * p.Hkv * p.B;
  hipLaunchKernelGGL((decode_split_kernel<D, CAUSAL, WINDOW>), dim3((unsigned)nsplit_wg),
                     dim3(kDecThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint64_t rows = (uint64_t)p.B * p.Nq * p.Hq;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)rows), dim3(kDecThreads), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeParams& p, hipStream_t stream) {
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch3<D, true, true>(p, stream) : launch3<D, true, false>(p, stream);
  return win ? launch3<D, false, true>(p, stream) : launch3<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace fa

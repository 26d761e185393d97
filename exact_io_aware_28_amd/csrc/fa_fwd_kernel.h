// Exact attention forward, bf16 in / bf16 out, fp32 softmax state, gfx950:
// the kernel template and its launcher, shared by fa_fwd_bf16.hip (d = 64,
// bias) and fa_fwd_bf16_d128.hip (d = 128 without bias, built with the
// max-ILP scheduler).
//
// Method (llms.blog "FlashAttention: How IO-Aware Tiling and Online Softmax
// Solved Transformer Memory Bottlenecks"):
//   * "1. IO-Aware Tiling": a work-group owns a block of query rows and
//     visits the key/value blocks; only the final output block is written.
//   * "2. Online Softmax Reduction": per query row a running maximum m, a
//     running normaliser l and an unnormalised output accumulator are
//     rescaled whenever m grows, and O = acc / l once at the end.
//   * "FlashAttention-2: Parallelism Across the Sequence Dimension": the
//     grid runs over (batch, head, query block); exp is taken as exp2 with
//     the scale folded in and the division by l is done once.
//
// gfx950 mapping (one work-group = 8 waves x 32 query rows = 256 rows at
// d = 128, 4 waves = 128 rows at d = 64):
//   * The whole computation is done transposed so that every lane owns one
//     query row from start to end:  S^T = K Q^T  and  O^T += V^T P^T, both
//     on v_mfma_f32_32x32x16_bf16.  In the S^T result lane l holds query
//     l % 32 and 16 of the 32 keys of a block; the other 16 keys of the same
//     query sit in lane l ^ 32.  Row max therefore needs one cross-half
//     exchange per tile, and the row sum none until the epilogue.
//   * The exponentiated scores already sit in the B-operand layout of the
//     P*V product (after bf16 rounding), so P never leaves registers.  The
//     key order inside each 16-key chunk is permuted identically in P and in
//     the transposed V reads (ds_read_b64_tr_b16), which leaves the
//     contraction unchanged.
//   * Q fragments live in VGPRs for the whole kernel.  K and V tiles of 64
//     keys go from HBM/L2 straight into LDS (buffer loads with the LDS
//     destination), two buffers: the loads of tile j+1 are issued right
//     after the barrier that opens tile j and land while tile j is computed.
//     Rows past the sequence end read as zeros (descriptor bounds check).
//   * Causal and window masks skip whole tiles; element masks are only
//     evaluated on tiles that straddle a boundary.
//   * An optional additive bias (a custom mask, -inf hiding a key) is read
//     from global memory per tile, after the Q K^T products so that its
//     registers are not live across them, and folded into the scores in
//     log2 units before the row maximum; the rest of the update is
//     unchanged.  The other wave of the SIMD covers the load latency.
//   * Optional dropout on the probabilities (inferensys.com glossary
//     "FlashAttention", the paragraph on the one fused kernel: matrix
//     multiply, softmax, dropout and masking): a Philox4x32-10 call per
//     16-key chunk and lane gives the keep bits of the lane's eight keys
//     (16-bit slots); dropped probabilities still count
//     in l (the softmax is of the undropped scores), the kept ones go to the
//     P V product and 1 / (1 - p) is folded into the final division by l.
//   * Lazy rescaling: the running maximum used for exponentiation is only
//     raised when a row's maximum grows by more than 2^8, so most tiles skip
//     the accumulator rescale.  Scores stay <= 2^8 in fp32, and O and LSE
//     are unchanged because l and acc always use the same reference.
#pragma once

#include "fa_device.h"

namespace fa {
namespace {

// Waves per work-group (32 query rows each) is a template parameter W: eight
// (256 rows, two per SIMD) at d = 128, which halves the K/V staging per
// query row and measures 1.5-3 % faster than four; four at d = 64, where
// the grid of 256-row groups is too small.
constexpr int kBN = 64;   // keys per K/V tile
constexpr float kRescaleSlack = 8.0f;  // log2 of the largest unrescaled score

template <int D, int W, bool CAUSAL, bool WINDOW, bool VARLEN, bool F16, bool BIAS,
          bool DROP>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(2)))
void fwd_bf16_kernel(FwdParams p) {
  constexpr int kWaves = W;
  constexpr int kBM = 32 * kWaves;      // query rows per work-group
  constexpr int KS = D / 16;            // k-steps of the QK^T contraction
  constexpr int NB = kBN / 32;          // 32-key blocks per tile
  constexpr int kPrefetch = (D == 128) ? 6 : 4;  // LDS reads ahead of the S MFMAs
  constexpr int NC = kBN / 16;          // 16-key chunks per tile
  constexpr int DB = D / 32;            // 32-column blocks of the output
  constexpr float kInf = __builtin_inff();

  // two K/V buffers as distinct objects, so that reads of one buffer are not
  // ordered behind the loads still landing in the other
  __shared__ __attribute__((aligned(1024))) __bf16 k0[kBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v0[kBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 k1[kBN * D];
  __shared__ __attribute__((aligned(1024))) __bf16 v1[kBN * D];
  // d = 128 with a bias: each wave's 32 bias rows x 64 keys (fp32) of the
  // next tile are copied into LDS while the current tile is computed; the
  // 16-byte chunks of row r sit at positions chunk ^ (r & 15), so the reads
  // below are free of bank conflicts.  (With both a causal and a window mask
  // the staging spills registers; that kernel loads the bias directly.)
  constexpr bool kBiasLds = BIAS && D == 128 && !(CAUSAL && WINDOW);
  __shared__ __attribute__((aligned(1024))) float bias_s[kBiasLds ? kWaves * 32 * kBN : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  // ---- which (sequence, head, query block) this work-group computes
  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int G = p.group;
  if (CAUSAL && p.xcd_groups > 1) {
    // Each XCD's contiguous range holds whole KV-head groups; run their
    // longest query tiles first across all of them instead of group by group,
    // so that no long tile starts near the end of a short grid.
    const uint32_t per = gridDim.x / kNumXcd, x = id / per, u = id % per;
    const uint32_t g = (uint32_t)G, K = (uint32_t)p.xcd_groups, rest = u / g;
    id = x * per + u % g + g * (rest / K + (uint32_t)p.num_qtiles * (rest % K));
  }
  const int gi = id % G;
  id /= G;
  int t_ord, b, hkv;
  if (BIAS && p.bias_sh == 0) {
    // a bias shared by the heads: every head of a query tile next to each
    // other, so the work-groups that read the same bias rows run together
    // on one XCD and share them in its L2
    hkv = id % p.Hkv;
    id /= p.Hkv;
    t_ord = id % p.num_qtiles;
    b = id / p.num_qtiles;
  } else {
    t_ord = id % p.num_qtiles;
    id /= p.num_qtiles;
    // the KV head is the slowest index, so each XCD's contiguous range holds
    // whole KV heads (their query heads share the K/V in that XCD's L2) and
    // every XCD sees the same mix of sequences (balanced for packed batches)
    b = id % p.B;
    hkv = id / p.B;
  }
  const int h = hkv * G + gi;
  // causal: longest rows first so that the tail of the grid is short
  const int qt = CAUSAL ? (p.num_qtiles - 1 - t_ord) : t_ord;
  const SeqSpan sp = seq_span(VARLEN ? p.cu_seqlens : nullptr, b, p.Nq, p.Nk);
  const int q_start = qt * kBM;
  if (q_start >= sp.lq) return;
  const int delta = sp.lk - sp.lq;
  const int q_end = min(q_start + kBM, sp.lq);

  int kv_lo = 0, kv_hi = sp.lk;
  if (CAUSAL) kv_hi = min(kv_hi, q_end + delta);
  if (WINDOW) kv_lo = max(0, q_start + delta - p.window + 1);
  kv_lo = (kv_lo / kBN) * kBN;

  const int64_t qstride = (int64_t)p.Hq * D;
  const int64_t kstride = (int64_t)p.Hkv * D;
  const uint32_t kstride_b = (uint32_t)(kstride * 2);
  const __bf16* Kg = (const __bf16*)p.k + sp.k0 * kstride + (int64_t)hkv * D;
  const __bf16* Vg = (const __bf16*)p.v + sp.k0 * kstride + (int64_t)hkv * D;

  const TileDma<D, kBN, kWaves> dma(wave, lane, kstride_b);
  auto issue = [&](int j0, __bf16* kb, __bf16* vb) {
    dma.issue(Kg, kstride_b, j0, sp.lk, kb);
    dma.issue(Vg, kstride_b, j0, sp.lk, vb);
  };
  // bias rows of this wave from key j0 on into its LDS block: eight 1 KB
  // copies of four rows each.  Copy i, lane l: row 4i + l/16, stored chunk
  // l % 16, read from chunk (l % 16) ^ (row & 15) = bchunk ^ 4(i % 4); the
  // row step of 4i rows is a uniform offset.
  const float* bias_bh = BIAS ? p.bias + (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh
                              : nullptr;
  const int qlo_b = q_start + wave * 32;
  const uint32_t brow_off = (uint32_t)((lane >> 4) * p.bias_sq) * 4u;
  const uint32_t bchunk = (uint32_t)((lane & 15) ^ (lane >> 4));
  auto bias_issue = [&](int j0) __attribute__((always_inline)) {
    if constexpr (kBiasLds) {
      const __amdgpu_buffer_rsrc_t rs = bias_rsrc(bias_bh, p.bias_sq, qlo_b, sp.lq, j0, sp.lk);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        dma16(rs, reinterpret_cast<__bf16*>(bias_s + wave * 32 * kBN) + i * 512,
              brow_off + ((bchunk ^ (uint32_t)(4 * (i & 3))) << 4),
              (uint32_t)(4 * i * p.bias_sq) * 4u);
    }
  };
  if (kv_lo < kv_hi) {
    issue(kv_lo, k0, v0);
    bias_issue(kv_lo);
  }
  FA_STAGE_SYNC();

  // ---- Q fragments (B operand of S^T = K Q^T): query qi, 8 columns per step
  const int qi = q_start + wave * 32 + r32;
  bf16x8 qf[KS];
  if (qi < sp.lq) {
    const __bf16* qp = (const __bf16*)p.q + (sp.q0 + qi) * qstride +
                       (int64_t)h * D + hl * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>(qp + 16 * s));
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
  float m_run = -kInf;  // reference maximum, scaled (log2) units
  float l_run = 0.f;    // this half-wave's share of the normaliser
  // The tile loop always takes the row maximum with a positive multiplier,
  // so it has no branch between the score products and the softmax: a
  // negative scale is applied as |scale| to -Q (flipping the sign bits is
  // exact), and a zero scale becomes a tiny positive one, with which every
  // exp2(s c - m) still rounds to exactly 1 and a masked score (the -inf
  // sentinel) exponentiates to exactly 0 rather than to NaN.
  float c = p.scale_log2;
  if (c < 0.f) {
    c = -c;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = as_bf16x8(__builtin_bit_cast(uint4, qf[s]) ^
                        make_uint4(0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u));
  }
  if (c == 0.f) c = 1e-30f;
  // with a bias the scores are turned into log2 units right after the
  // product, and the softmax update below multiplies by 1
  const float cs = BIAS ? 1.0f : c;

  const int qlo_w = q_start + wave * 32;
  const int qhi_w = min(qlo_w + 31, sp.lq - 1);
  // lane-dependent parts of the transposed V read address
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  // Lane byte offsets of the LDS reads inside a tile.  The swizzle depends
  // on the low four row bits only, so 32-row blocks (K) and 16-row chunks
  // (V) differ from these by whole rows, a constant that goes into the
  // read instruction's offset field.
  uint32_t koff[KS];     // K fragment, row r32, k-step st
  uint32_t voff[2][DB];  // V transposed read, rows tr_row + 8h, column block db
#pragma unroll
  for (int st = 0; st < KS; ++st) koff[st] = 2 * tile_off<D>(r32, st * 16 + hl * 8);
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      voff[h][db] = 2 * tile_off<D>(tr_row + 8 * h, db * 32 + tr_col);

  // The bias of this lane's row at the keys its score elements hold, for a
  // whole tile (branch-free loads, bias_rsrc).
  constexpr int kBiasRegs = BIAS ? NB * 16 : 1;
  const uint32_t bias_lane = (uint32_t)(r32 * p.bias_sq) * 4u;
  auto load_bias = [&](int j0, float (&bt)[kBiasRegs]) {
    if constexpr (kBiasLds) {
      // from the LDS block filled during the previous tile
      const float* brow = bias_s + wave * 32 * kBN + r32 * kBN;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int pos = (kb * 8 + g * 2 + hl) ^ (r32 & 15);
          const f32x4 t = *reinterpret_cast<const f32x4*>(brow + 4 * pos);
#pragma unroll
          for (int e = 0; e < 4; ++e) bt[kb * 16 + 4 * g + e] = t[e];
        }
    } else if constexpr (BIAS) {
      const __amdgpu_buffer_rsrc_t rs =
          bias_rsrc(p.bias + (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh, p.bias_sq, qlo_w,
                    sp.lq, j0, sp.lk);
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 t = bias_load4(rs, bias_lane, kb * 32 + g * 8 + hl * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) bt[kb * 16 + 4 * g + e] = t[e];
        }
    }
  };

  auto compute = [&](int j0, const __bf16* kt, const __bf16* vt) __attribute__((always_inline)) {
    bool active = qlo_w <= qhi_w;
    if (CAUSAL) active = active && (j0 <= qhi_w + delta);
    if (WINDOW) active = active && (j0 + kBN - 1 > qlo_w + delta - p.window);
    if (!active) {
      // a wave that skips this tile still stages the next tile's bias
      if constexpr (kBiasLds) {
        if (j0 + kBN < kv_hi) bias_issue(j0 + kBN);
        FA_STAGE_SYNC();
      }
      return;
    }
    bool need_mask = (j0 + kBN > sp.lk);
    if (CAUSAL) need_mask = need_mask || (j0 + kBN - 1 > qlo_w + delta);
    if (WINDOW) need_mask = need_mask || (qhi_w + delta - j0 >= p.window);

    // the bias loads go out before the products, which hide part of their
    // latency
    float bt[kBiasRegs];
    if constexpr (BIAS) {
      load_bias(j0, bt);
      __builtin_amdgcn_sched_barrier(0);
    }
    // S^T block kb: rows = keys j0 + 32kb + 8(i/4) + 4hl + i%4, col = qi
    f32x16 s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
    // k-step outer, block inner: consecutive MFMAs accumulate into different
    // blocks (measured ~0.5 % faster than two back-to-back chains)
#pragma unroll
    for (int st = 0; st < KS; ++st)
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const uint4 a = lds_read_b128_at(kt, koff[st], kb * 32 * D * 2);
        s[kb] = mfma32_t<F16>(as_bf16x8(a), qf[st], s[kb]);
      }
    // Schedule: issue kPrefetch K-fragment reads before the first MFMA, then
    // alternate one MFMA with one read, so several LDS reads stay in flight
    // while the matrix core works (the default schedule keeps about two).
    __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kPrefetch, 0);
#pragma unroll
    for (int i = 0; i < NB * KS - kPrefetch; ++i) {
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(kSchedMfma, kPrefetch, 0);
    if constexpr (BIAS) {
      // scores and bias in log2 units
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = fmaf(bt[kb * 16 + i], kLog2e, s[kb][i] * c);
    }
    if constexpr (kBiasLds) {
      // this tile's bias is consumed: copy the next tile's into the block
      __builtin_amdgcn_sched_barrier(0);
      if (j0 + kBN < kv_hi) bias_issue(j0 + kBN);
      FA_STAGE_SYNC();
    }

    // A tile that straddles a mask boundary first replaces each invisible
    // score by -inf, which never wins the row maximum and whose probability
    // exp2(-inf) is exactly zero; then every tile takes the same update.  The
    // masking stays a separate, rarely taken block: with a second full copy
    // of the update for masked tiles the compiler moved the accumulators
    // between register sets or spilled, and if-converted it would run the
    // selects on every tile.
    auto key_of = [&](int kb, int i) { return j0 + kb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3); };
    if (__builtin_expect(need_mask, 0)) {
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!visible<CAUSAL, WINDOW>(qi, key_of(kb, i), delta, sp.lk, p.window))
            s[kb][i] = -kInf;
    }
    // Online-softmax update and P V product.
    {
      // row maximum of the raw scores (the multiplier cs is positive)
      float rm = s[0][0];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) rm = fmaxf(rm, s[kb][i]);
      rm = max_halves(rm);
      const float tmax = __builtin_isinf(rm) ? -kInf : rm * cs;

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
          for (int i = 0; i < 16; ++i) acc[db][i] *= alpha;
      }

      // exponentiate one 16-key chunk at a time and feed it straight to the
      // P V product, so the chunk's MFMAs overlap the next chunk's exp2s:
      // O^T[d][q] += sum_j V[j][d] P[q][j]; chunk kc holds keys
      // 16kc + 4hl + {0..3} (slots 0..3) and 16kc + 8 + 4hl + {0..3} (4..7)
      const float neg = -m_sub;
      float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        const int kb = kc >> 1, i0 = (kc & 1) * 8;
        // dropout: one generator call covers the chunk's eight keys, slot e
        // for pv[e] (the normaliser l sums the undropped probabilities)
        uint4 dw;
        if constexpr (DROP) dw = drop_call(key_of(kb, i0), qi, h, b, p.seed_lo, p.seed_hi);
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pv[e] = fast_exp2(fmaf(s[kb][i0 + e], cs, neg));  // 0 for a masked score
          if (e & 1)
            lsum1 += pv[e];
          else
            lsum0 += pv[e];
          if constexpr (DROP) pv[e] = slot_of(dw, e) >= p.drop_thresh ? pv[e] : 0.f;
        }
        const bf16x8 pb = pack8_t<F16>(pv[0], pv[1], pv[2], pv[3], pv[4], pv[5], pv[6], pv[7]);
        bf16x8 va[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          va[db] = cat(lds_read_tr_at(vt, voff[0][db], 16 * kc * D * 2),
                       lds_read_tr_at(vt, voff[1][db], 16 * kc * D * 2));
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) acc[db] = mfma32_t<F16>(va[db], pb, acc[db]);
      }
      l_run += lsum0 + lsum1;
    }
  };

  // ---- main loop over K/V tiles, two buffers (unrolled by two)
  for (int j0 = kv_lo; j0 < kv_hi; j0 += 2 * kBN) {
    dma_barrier();  // tile j0 is in buffer 0; buffer 1 is free
    if (j0 + kBN < kv_hi) issue(j0 + kBN, k1, v1);
    FA_STAGE_SYNC();
    compute(j0, k0, v0);
    FA_STAGE_SYNC();
    if (j0 + kBN >= kv_hi) break;
    dma_barrier();  // tile j0 + kBN is in buffer 1; buffer 0 is free
    if (j0 + 2 * kBN < kv_hi) issue(j0 + 2 * kBN, k0, v0);
    FA_STAGE_SYNC();
    compute(j0 + kBN, k1, v1);
    FA_STAGE_SYNC();
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (m + log2 l)
  const float l_tot = sum_halves(l_run);
  if (qi < sp.lq) {
    // dropout scales the kept probabilities by 1 / (1 - p)
    const float inv = (l_tot == 0.f) ? 0.f : (DROP ? p.drop_scale : 1.0f) / l_tot;
    __bf16* op = (__bf16*)p.o + (sp.q0 + qi) * qstride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint2 w = pack4_t<F16>(acc[db][4 * r + 0] * inv, acc[db][4 * r + 1] * inv,
                                     acc[db][4 * r + 2] * inv, acc[db][4 * r + 3] * inv);
        *reinterpret_cast<uint2*>(op + db * 32 + r * 8 + hl * 4) = w;
      }
    if (hl == 0) {
      const float m_sub = (m_run == -kInf) ? 0.f : m_run;
      const float lse = (l_tot == 0.f) ? -kInf : (m_sub + __log2f(l_tot)) * kLn2;
      p.lse[lse_index(VARLEN ? p.cu_seqlens : nullptr, p.B, p.Hq, p.Nq, b, h,
                      sp.q0, qi)] = lse;
    }
  }
}

// Launch with W waves per work-group; the query-tile count follows from W.
template <int D, int W, bool CAUSAL, bool WINDOW, bool VARLEN, bool F16, bool BIAS = false,
          bool DROP = false>
hipError_t launch_w(FwdParams p, hipStream_t stream) {
  p.num_qtiles = (p.Nq + 32 * W - 1) / (32 * W);
  // Causal dense grids of at most about two rounds of work-groups per XCD
  // finish sooner with each XCD's longest query tiles dispatched first (a
  // bigger grid balances by itself and keeps its head-major order).
  p.xcd_groups = 0;
  if (CAUSAL && !VARLEN && !(BIAS && p.bias_sh == 0)) {
    const long n = (long)p.B * p.Hq * p.num_qtiles, per = n / kNumXcd;
    const long unit = (long)p.group * p.num_qtiles;     // work-groups of one KV head
    const long slots = 32L * (D == 64 ? 3 : 1);          // resident per XCD: 32 CUs
    if (n % kNumXcd == 0 && per % unit == 0 && per / unit > 1 && per <= 2 * slots)
      p.xcd_groups = (int)(per / unit);
  }
  dim3 grid((unsigned)p.B * p.Hq * p.num_qtiles), block(64 * W);
  hipLaunchKernelGGL((fwd_bf16_kernel<D, W, CAUSAL, WINDOW, VARLEN, F16, BIAS, DROP>), grid,
                     block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace
}  // namespace fa

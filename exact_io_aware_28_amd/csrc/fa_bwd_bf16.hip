// Exact attention backward by recomputation, bf16 in / bf16 out, gfx950.
//
// llms.blog "FlashAttention: How IO-Aware Tiling and Online Softmax Solved
// Transformer Memory Bottlenecks", "3. Recomputation in the Backward Pass":
// the forward keeps only O and the row statistics; the backward reloads Q, K,
// V tiles, rebuilds the score tiles from the saved statistics and forms the
// gradients without any N x N buffer.  The row statistic saved here is
// LSE = m + ln l (the logsumexp of tokrepo.com "Flash Attention - Fast
// Memory-Efficient Exact Attention", "Architecture Overview"), so a
// probability tile is rebuilt as P = exp(S - LSE) = exp2(S c - LSE log2 e),
// c = scale log2 e.  The gradient formulas are the chain rule through the
// row softmax:
//     dV = P^T dO,  dP = dO V^T,  D_i = sum_c dO_ic O_ic,
//     dS = P (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, in stream order, no atomics (results are deterministic):
//   1. bwd_pre:  D_i from dO and the saved bf16 O, into the workspace.
//   2. bwd_dkdv: a work-group owns 128 keys of one KV head (each lane one
//      key); it walks every query head of the KV head's group and every
//      query tile that can see its keys, with Q, dO, LSE and D tiles staged
//      in LDS.  dK and dV stay in registers and are written once, so the GQA
//      sum over the group needs no atomics.  For d = 128 eight
//      waves share the work, K and V staged in LDS, each pair of waves
//      splitting every query tile's rows and adding its partial sums at the
//      end (bwd_dkdv8_kernel); otherwise four waves, one per 32 keys, with K
//      and V in registers (bwd_dkdv_kernel).
//   3. bwd_dq:   a work-group owns 128 query rows of one head (one lane per
//      query row, as in the forward) and walks the key tiles it can see,
//      rebuilding S and dP to accumulate dQ.  This recomputes two of the
//      five products a second time, in exchange for no cross-work-group
//      reduction.
// All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the
// probability and dS tiles are rounded to bf16 as MFMA operands.
// With dropout (keep-mask Z regenerated from the seed, never stored):
//     dV = (P Z / (1 - p))^T dO,  dS = P (dP Z / (1 - p) - D),
// and D = rowsum(dO * O) is unchanged, O being the dropped output.  The dQ
// kernel (one query row per lane, runs of four keys) draws one Philox call
// per eight elements (16-bit slots); so does the dK/dV kernel (one key per
// lane), whose lanes with keys in the same group of eight share each call
// through quad broadcasts and a row rotation.
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kKeyBlock = 128;  // keys per dK/dV work-group (4 waves x 32)
constexpr int kQTile = 64;      // query rows per staged tile in dK/dV
constexpr int kQBlock = 128;    // query rows per dQ work-group (4 waves x 32)
constexpr int kKTile = 64;      // keys per staged tile in dQ
constexpr int kReadsAhead = 4;  // LDS fragment reads issued ahead of the score MFMAs

// Element e of eight 16-bit values held as raw bits (bf16, or fp16 with F16).
template <bool F16>
__device__ __forceinline__ float elem_f32(const bf16x8& v, int e) {
  if constexpr (F16)
    return (float)__builtin_bit_cast(f16x8, v)[e];
  else
    return (float)v[e];
}

// ------------------------------------------------------------ 1. D = dO . O
// D/8 consecutive lanes share one (token, head) row: each reads 16 contiguous
// bytes of O and of dO, so a wave instruction covers whole rows, and the
// partial dot products are summed with lane shuffles inside the group.
template <int D, bool F16>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams p) {
  constexpr int kLanesPerRow = D / 8;
  constexpr int kRowsPerBlock = kThreads / kLanesPerRow;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kLanesPerRow;
  const int part = threadIdx.x % kLanesPerRow;
  const int64_t token = row / p.Hq;
  const int h = (int)(row % p.Hq);
  const int64_t T = p.cu_seqlens ? (int64_t)p.cu_seqlens[p.B] : (int64_t)p.B * p.Nq;
  const bool valid = token < T;
  float acc = 0.f;
  if (valid) {
    const int64_t base = (token * p.Hq + h) * D + part * 8;
    const bf16x8 a = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.o + base));
    const bf16x8 g = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.dout + base));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(elem_f32<F16>(a, e), elem_f32<F16>(g, e), acc);
  }
#pragma unroll
  for (int m = kLanesPerRow / 2; m > 0; m >>= 1) acc += __shfl_xor(acc, m, 64);
  if (!valid || part != 0) return;
  int64_t out;
  if (p.cu_seqlens) {
    out = (int64_t)h * T + token;
  } else {
    const int64_t b = token / p.Nq, i = token % p.Nq;
    out = (b * p.Hq + h) * p.Nq + i;
  }
  p.delta[out] = acc;
}

// ------------------------------------------------------------ 2. dK, dV
// Eight dropout keep bits of one row (bit s: slot s of the generator call of
// key j's group, drop_call in fa_device.h).
__device__ __forceinline__ uint32_t keep8(int j, int i, int h, int b, uint32_t seed_lo,
                                          uint32_t seed_hi, uint32_t thresh) {
  const uint4 w = drop_call(j, i, h, b, seed_lo, seed_hi);
  uint32_t bits = 0;
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) bits |= (uint32_t)(slot_of(w, s2) >= thresh) << s2;
  return bits;
}

// Value of x in lane l ^ 8 (DPP row_ror:8 inside each row of 16 lanes).
__device__ __forceinline__ uint32_t row_ror8(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x128, 0xF, 0xF, false);
}

// dK and dV accumulators plus the resident K and V fragments take about 350
// registers at d = 128 (one wave per SIMD); d = 64 fits two waves.
template <int D>
constexpr int dkdv_waves_per_simd() { return D == 64 ? 2 : 1; }

template <int D, bool CAUSAL, bool WINDOW, bool VARLEN, bool BIAS, bool DROP, bool F16>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(dkdv_waves_per_simd<D>())))
void bwd_dkdv_kernel(BwdParams p, int num_ktiles) {
  constexpr int KS = D / 16, DB = D / 32, QB = kQTile / 32;
  constexpr float kInf = __builtin_inff();
  // two Q/dO buffers as distinct objects, so that reads of one buffer are
  // not ordered behind the loads still landing in the other
  __shared__ __attribute__((aligned(1024))) __bf16 sq0[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sdo0[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sq1[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sdo1[kQTile * D];
  __shared__ __attribute__((aligned(16))) float sl0[kQTile], sd0[kQTile];
  __shared__ __attribute__((aligned(16))) float sl1[kQTile], sd1[kQTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = id % num_ktiles;  // key tile 0 first: it sees the most rows
  id /= num_ktiles;
  // the KV head is the slowest index, so each XCD's contiguous range holds
  // whole KV heads (their query heads share the K/V in that XCD's L2) and
  // every XCD sees the same mix of sequences (balanced for packed batches)
  const int b = id % p.B;
  const int hkv = id / p.B;
  const int G = p.group;
  const int32_t* cu = VARLEN ? p.cu_seqlens : nullptr;
  const SeqSpan sp = seq_span(cu, b, p.Nq, p.Nk);
  const int k_start = kt * kKeyBlock;
  if (k_start >= sp.lk) return;
  const int delta = sp.lk - sp.lq;
  const int k_end = min(k_start + kKeyBlock, sp.lk);

  int q_lo = 0, q_hi = sp.lq;
  if (CAUSAL) q_lo = max(0, k_start - delta);
  if (WINDOW) q_hi = min(q_hi, p.window + k_end - 1 - delta);
  q_lo = (q_lo / kQTile) * kQTile;
  const int n_qt = (q_hi > q_lo) ? (q_hi - q_lo + kQTile - 1) / kQTile : 0;
  const int n_it = n_qt * G;
  // iteration it -> (query head of the group, query tile).  With a bias the
  // head is the fastest index: the G heads that share a bias block (a bias
  // broadcast over heads) then read it back to back, from the caches.
  auto it_head = [&](int it) { return BIAS ? it % G : it / n_qt; };
  auto it_tile = [&](int it) { return BIAS ? it / G : it % n_qt; };

  const int64_t qstride = (int64_t)p.Hq * D, kstride = (int64_t)p.Hkv * D;
  const float c = p.scale_log2;

  // this wave's keys; lane key kj, fragments are B operands (K^T, V^T)
  const int kw_lo = k_start + wave * 32;
  const int kw_hi = min(kw_lo + 31, sp.lk - 1);
  const int kj = kw_lo + r32;
  bf16x8 kf[KS], vf[KS];
  {
    const int64_t off = (sp.k0 + kj) * kstride + (int64_t)hkv * D + hl * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if (kj < sp.lk) {
        kf[s] = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.k + off + 16 * s));
        vf[s] = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.v + off + 16 * s));
      } else {
        kf[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
        vf[s] = kf[s];
      }
    }
  }

  f32x16 dva[DB], dka[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dva[db][i] = dka[db][i] = 0.f;

  // Lane byte offsets of the LDS reads inside a Q or dO tile (swizzled like
  // the forward's K/V tiles): 128-bit fragment reads per k-step and
  // transposing reads per output column block; 32-row blocks and 16-row
  // chunks add whole rows, which go into the instruction's offset field.
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  uint32_t foff[KS], troff[2][DB];
#pragma unroll
  for (int st = 0; st < KS; ++st) foff[st] = 2 * tile_off<D>(r32, st * 16 + hl * 8);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      troff[h2][db] = 2 * tile_off<D>(tr_row + 8 * h2, db * 32 + tr_col);

  // Q and dO tiles go straight into LDS (buffer loads with the LDS
  // destination); the 64 row statistics of a tile go through registers.
  const uint32_t qstride_b = (uint32_t)(qstride * 2);
  const TileDma<D, kQTile, kThreads / 64> dma(wave, lane, qstride_b);
  float lse_r = 0.f, dl_r = 0.f;  // row statistics of the next tile (threads < kQTile)
  auto issue_it = [&](int it, __bf16* bq, __bf16* bdo) {
    const int gi = it_head(it);
    const int i0 = q_lo + it_tile(it) * kQTile;
    const int h = hkv * G + gi;
    const int64_t hoff = sp.q0 * qstride + (int64_t)h * D;
    dma.issue((const __bf16*)p.q + hoff, qstride_b, i0, sp.lq, bq);
    dma.issue((const __bf16*)p.dout + hoff, qstride_b, i0, sp.lq, bdo);
    if (tid < kQTile) {
      const int i = i0 + tid;
      float l = kInf, dd = 0.f;
      if (i < sp.lq) {
        const int64_t li = lse_index(cu, p.B, p.Hq, p.Nq, b, h, sp.q0, i);
        const float lv = p.lse[li];
        l = (lv == -kInf) ? kInf : lv * kLog2e;  // rows that see no key: P = 0
        dd = p.delta[li];
      }
      lse_r = l;
      dl_r = dd;
    }
  };

  auto compute = [&](int it, const __bf16* tq, const __bf16* tdo, const float* tl,
                     const float* td) {
    const int i0 = q_lo + it_tile(it) * kQTile;
    const int h_it = hkv * G + it_head(it);  // query head of this tile
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qr0 = i0 + qb * 32;
      const int qr1 = min(qr0 + 31, sp.lq - 1);
      bool active = (qr0 <= qr1) && (kw_lo <= kw_hi);
      if (CAUSAL) active = active && (qr1 + delta >= kw_lo);
      if (WINDOW) active = active && (qr0 + delta - kw_hi < p.window);
      if (!active) continue;
      bool need_mask = false;
      if (CAUSAL) need_mask = need_mask || (qr0 + delta < kw_hi);
      if (WINDOW) need_mask = need_mask || (qr1 + delta - kw_lo >= p.window);

      // bias at this lane's key for the block's 16 query rows (a column of
      // the bias: consecutive lanes read consecutive keys), raw values that
      // are scaled to log2 units where they are used
      float bv[BIAS ? 16 : 1];
      if constexpr (BIAS) {
        const int hb = hkv * G + it_head(it);
        const float* bcol = p.bias + (int64_t)b * p.bias_sb + (int64_t)hb * p.bias_sh +
                            min(kj, sp.lk - 1);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qr0 + 8 * (i >> 2) + 4 * hl + (i & 3);
          bv[i] = (kj < sp.lk && qr < sp.lq) ? bcol[(int64_t)qr * p.bias_sq] : 0.f;
        }
      }

      // S = Q K^T and dP = dO V^T: lane = key kj, rows = queries
      // qb*32 + 8(i/4) + 4hl + i%4 of the staged tile
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const uint32_t ro = qb * 32 * D * 2;
        s = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(tq, foff[st], ro)), kf[st], s);
        dp = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(tdo, foff[st], ro)), vf[st], dp);
      }

      // Dropout keep bits of this lane's key for the block's 16 rows.  One
      // Philox call gives a row's bits for the eight keys 16m + 4t +
      // {0..3, 8..11}, held by the eight lanes l with equal bits 2 and 4 (a
      // quad and the quad eight lanes away).  Group lane u = 4a + t (a = bit 3
      // of the lane, t = its low bits) draws block rows rho = 2u and 2u + 1
      // (rho = 4r + e is row 8r + 4hl + e), and quad broadcasts plus one row
      // rotation hand every lane all eight drawn words.  kw[u]: group lane
      // u's word, shifted so that bit 8 (rho & 1) is this lane's key.
      uint32_t kw[8];
      if constexpr (DROP) {
        const int t = r32 & 3, a = (r32 >> 3) & 1, u = 4 * a + t;
        uint32_t mine = 0;  // bit 8 (rho & 1) + s: row rho, slot s
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const int rho = 2 * u + k2;
          const int row = i0 + qb * 32 + 8 * (rho >> 2) + 4 * hl + (rho & 3);
          mine |= keep8(kj, row, h_it, b, p.seed_lo, p.seed_hi, p.drop_thresh) << (8 * k2);
        }
        const uint32_t other = row_ror8(mine);  // the quad eight lanes away
        const uint32_t own_w[4] = {quad_bcast<0>(mine), quad_bcast<1>(mine),
                                   quad_bcast<2>(mine), quad_bcast<3>(mine)};
        const uint32_t oth_w[4] = {quad_bcast<0>(other), quad_bcast<1>(other),
                                   quad_bcast<2>(other), quad_bcast<3>(other)};
#pragma unroll
        for (int v = 0; v < 8; ++v)
          kw[v] = (((v >> 2) == a) ? own_w[v & 3] : oth_w[v & 3]) >> u;
      }

      // P for every element; a block that straddles a mask boundary then
      // zeroes its invisible entries in a separate, rarely taken step, and one
      // update forms dS for every block (with a second full copy of the update
      // for masked blocks the dropout backward ran 3 % slower)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 L = *reinterpret_cast<const float4*>(&tl[qb * 32 + 8 * r + 4 * hl]);
        const float Lv[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r + e;
          float pv = fmaf(s[i], c, -Lv[e]);
          if constexpr (BIAS) pv = fmaf(bv[i], kLog2e, pv);
          s[i] = fast_exp2(pv);
        }
      }
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qb * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (!visible<CAUSAL, WINDOW>(i0 + qr, kj, delta, sp.lk, p.window)) s[i] = 0.f;
        }
      }
      {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qrow = qb * 32 + 8 * r + 4 * hl;
          const float4 Dl = *reinterpret_cast<const float4*>(&td[qrow]);
          const float Dv[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * r + e;
            const float pv = s[i];
            if constexpr (DROP) {
              // O = (P Z / (1 - p)) V: dV takes the dropped, rescaled P and
              // the gradient reaching P is dP Z / (1 - p)
              // row rho = i = 4r + e was drawn by group lane i >> 1
              const bool kp = (kw[i >> 1] >> (8 * (i & 1))) & 1u;
              s[i] = kp ? pv * p.drop_scale : 0.f;
              dp[i] = pv * ((kp ? dp[i] * p.drop_scale : 0.f) - Dv[e]);
            } else {
              s[i] = pv;
              dp[i] = pv * (dp[i] - Dv[e]);
            }
          }
        }
      }

      // dV^T += dO^T P and dK^T += Q^T dS over 16-query chunks; chunk qc
      // holds queries 16qc + 4hl + {0..3} and 16qc + 8 + 4hl + {0..3}
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const int j = qc * 8;
        const bf16x8 pb = pack8_t<F16>(s[j], s[j + 1], s[j + 2], s[j + 3], s[j + 4],
                                      s[j + 5], s[j + 6], s[j + 7]);
        const bf16x8 dsb = pack8_t<F16>(dp[j], dp[j + 1], dp[j + 2], dp[j + 3], dp[j + 4],
                                       dp[j + 5], dp[j + 6], dp[j + 7]);
        const uint32_t ro = (qb * 32 + 16 * qc) * D * 2;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          dva[db] = mfma32_t<F16>(cat(lds_read_tr_at(tdo, troff[0][db], ro),
                               lds_read_tr_at(tdo, troff[1][db], ro)),
                           pb, dva[db]);
          dka[db] = mfma32_t<F16>(cat(lds_read_tr_at(tq, troff[0][db], ro),
                               lds_read_tr_at(tq, troff[1][db], ro)),
                           dsb, dka[db]);
        }
      }
    }
  };

  // two buffers each, unrolled by two so that they are known at compile time
  if (n_it > 0) issue_it(0, sq0, sdo0);
  FA_STAGE_SYNC();
  for (int it = 0; it < n_it; it += 2) {
    if (tid < kQTile) {
      sl0[tid] = lse_r;
      sd0[tid] = dl_r;
    }
    dma_barrier();  // tile it is in buffer 0; buffer 1 is free
    if (it + 1 < n_it) issue_it(it + 1, sq1, sdo1);
    FA_STAGE_SYNC();
    compute(it, sq0, sdo0, sl0, sd0);
    FA_STAGE_SYNC();
    if (it + 1 >= n_it) break;
    if (tid < kQTile) {
      sl1[tid] = lse_r;
      sd1[tid] = dl_r;
    }
    dma_barrier();  // tile it + 1 is in buffer 1; buffer 0 is free
    if (it + 2 < n_it) issue_it(it + 2, sq0, sdo0);
    FA_STAGE_SYNC();
    compute(it + 1, sq1, sdo1, sl1, sd1);
    FA_STAGE_SYNC();
  }

  if (kj < sp.lk) {
    const int64_t off = (sp.k0 + kj) * kstride + (int64_t)hkv * D;
    __bf16* dkp = (__bf16*)p.dk + off;
    __bf16* dvp = (__bf16*)p.dv + off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int col = db * 32 + r * 8 + hl * 4;
        *reinterpret_cast<uint2*>(dkp + col) =
            pack4_t<F16>(dka[db][4 * r] * p.scale, dka[db][4 * r + 1] * p.scale,
                         dka[db][4 * r + 2] * p.scale, dka[db][4 * r + 3] * p.scale);
        *reinterpret_cast<uint2*>(dvp + col) =
            pack4_t<F16>(dva[db][4 * r], dva[db][4 * r + 1], dva[db][4 * r + 2],
                         dva[db][4 * r + 3]);
      }
  }
}

// dK/dV with eight waves (two per SIMD) for d = 128.  The one-wave-per-SIMD
// kernel above holds K and V in registers and waits on its own LDS reads and
// products about 40 % of the time with nothing else to issue.  Here K and V
// of the work-group's 128 keys sit in LDS instead (read as operand fragments
// like Q and dO), which frees the 64 registers that let two waves share each
// SIMD.  Waves w and w + 4 take the same 32 keys; wave w the first 32 rows of
// every 64-row query tile, wave w + 4 the second 32, so each holds partial dK
// and dV sums for its keys, and the pair adds them through LDS at the end
// (the sum is over disjoint row sets, fixed by the launch shape, so results
// stay deterministic).
constexpr int kDkdv8Threads = 512;

template <int D, bool CAUSAL, bool WINDOW, bool VARLEN, bool BIAS, bool DROP, bool F16>
__global__ __launch_bounds__(kDkdv8Threads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dkdv8_kernel(BwdParams p, int num_ktiles) {
  constexpr int KS = D / 16, DB = D / 32;
  constexpr float kInf = __builtin_inff();
  __shared__ __attribute__((aligned(1024))) __bf16 sk[kKeyBlock * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sv[kKeyBlock * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sq0[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sdo0[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sq1[kQTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sdo1[kQTile * D];
  __shared__ __attribute__((aligned(16))) float sl0[kQTile], sd0[kQTile];
  __shared__ __attribute__((aligned(16))) float sl1[kQTile], sd1[kQTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;
  const int kw = wave & 3, hb = wave >> 2;  // 32-key block, query-row half

  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = id % num_ktiles;
  id /= num_ktiles;
  const int b = id % p.B;
  const int hkv = id / p.B;
  const int G = p.group;
  const int32_t* cu = VARLEN ? p.cu_seqlens : nullptr;
  const SeqSpan sp = seq_span(cu, b, p.Nq, p.Nk);
  const int k_start = kt * kKeyBlock;
  if (k_start >= sp.lk) return;
  const int delta = sp.lk - sp.lq;
  const int k_end = min(k_start + kKeyBlock, sp.lk);

  int q_lo = 0, q_hi = sp.lq;
  if (CAUSAL) q_lo = max(0, k_start - delta);
  if (WINDOW) q_hi = min(q_hi, p.window + k_end - 1 - delta);
  q_lo = (q_lo / kQTile) * kQTile;
  const int n_qt = (q_hi > q_lo) ? (q_hi - q_lo + kQTile - 1) / kQTile : 0;
  const int n_it = n_qt * G;
  // iteration it -> (query head of the group, query tile).  With a bias the
  // head is the fastest index: the G heads that share a bias block (a bias
  // broadcast over heads) then read it back to back, from the caches.
  auto it_head = [&](int it) { return BIAS ? it % G : it / n_qt; };
  auto it_tile = [&](int it) { return BIAS ? it / G : it % n_qt; };

  const int64_t qstride = (int64_t)p.Hq * D, kstride = (int64_t)p.Hkv * D;
  // With dropout a hidden score is replaced by a value whose product with c
  // is -inf: -inf for a positive c, +inf for a negative one; a zero c is
  // taken as 1e-30, which leaves exp2(S c - L) as it was for a finite score.
  const float c = (DROP && p.scale_log2 == 0.f) ? 1e-30f : p.scale_log2;
  const float s_hidden = (c > 0.f) ? -kInf : kInf;

  const int kw_lo = k_start + kw * 32;
  const int kw_hi = min(kw_lo + 31, sp.lk - 1);
  const int kj = kw_lo + r32;

  // K and V of the work-group's keys, staged once (rows past the sequence
  // read as zero)
  {
    const uint32_t kstride_b = (uint32_t)(kstride * 2);
    const TileDma<D, kKeyBlock, kDkdv8Threads / 64> kv(wave, lane, kstride_b);
    const int64_t koff = sp.k0 * kstride + (int64_t)hkv * D;
    kv.issue((const __bf16*)p.k + koff, kstride_b, k_start, sp.lk, sk);
    kv.issue((const __bf16*)p.v + koff, kstride_b, k_start, sp.lk, sv);
  }

  f32x16 dva[DB], dka[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) dva[db][i] = dka[db][i] = 0.f;

  // Lane byte offsets of the LDS reads: 128-bit fragments of this wave's 32
  // query rows (Q, dO) and of its 32 keys (K, V), and transposing reads of
  // its query rows per output column block.  The swizzle depends on the row
  // modulo 16 only, so the row-half and key-block offsets are whole rows.
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  uint32_t fq[KS], fk[KS], troff[2][DB];
#pragma unroll
  for (int st = 0; st < KS; ++st) {
    const uint32_t f = 2 * tile_off<D>(r32, st * 16 + hl * 8);
    fq[st] = f + (uint32_t)(hb * 32 * D * 2);
    fk[st] = f + (uint32_t)(kw * 32 * D * 2);
  }
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      troff[h2][db] = 2 * tile_off<D>(tr_row + 8 * h2, db * 32 + tr_col) +
                      (uint32_t)(hb * 32 * D * 2);

  const uint32_t qstride_b = (uint32_t)(qstride * 2);
  const TileDma<D, kQTile, kDkdv8Threads / 64> dma(wave, lane, qstride_b);
  float lse_r = 0.f, dl_r = 0.f;  // row statistics of the next tile (threads < kQTile)
  auto issue_it = [&](int it, __bf16* bq, __bf16* bdo) {
    const int gi = it_head(it);
    const int i0 = q_lo + it_tile(it) * kQTile;
    const int h = hkv * G + gi;
    const int64_t hoff = sp.q0 * qstride + (int64_t)h * D;
    dma.issue((const __bf16*)p.q + hoff, qstride_b, i0, sp.lq, bq);
    dma.issue((const __bf16*)p.dout + hoff, qstride_b, i0, sp.lq, bdo);
    if (tid < kQTile) {
      const int i = i0 + tid;
      float l = kInf, dd = 0.f;
      if (i < sp.lq) {
        const int64_t li = lse_index(cu, p.B, p.Hq, p.Nq, b, h, sp.q0, i);
        const float lv = p.lse[li];
        l = (lv == -kInf) ? kInf : lv * kLog2e;  // rows that see no key: P = 0
        dd = p.delta[li];
      }
      lse_r = l;
      dl_r = dd;
    }
  };

  // Bias at this lane's key for its 16 query rows of the current tile (raw
  // values, scaled to log2 units where they are used).  A bias shared by the
  // heads (head stride 0) is loaded once per query tile and serves the tile's
  // G iterations (heads innermost): biased GQA backward 4.33 vs 4.83 ms.
  float bv[BIAS ? 16 : 1];
  auto compute = [&](int it, const __bf16* tq, const __bf16* tdo, const float* tl,
                     const float* td) {
    const int i0 = q_lo + it_tile(it) * kQTile;
    const int h_it = hkv * G + it_head(it);  // query head of this tile
    const int qr0 = i0 + hb * 32;
    const int qr1 = min(qr0 + 31, sp.lq - 1);
    bool active = (qr0 <= qr1) && (kw_lo <= kw_hi);
    if (CAUSAL) active = active && (qr1 + delta >= kw_lo);
    if (WINDOW) active = active && (qr0 + delta - kw_hi < p.window);
    if (!active) return;
    bool need_mask = false;
    if (CAUSAL) need_mask = need_mask || (qr0 + delta < kw_hi);
    if (WINDOW) need_mask = need_mask || (qr1 + delta - kw_lo >= p.window);

    // a new query tile, or a bias of its own per head: load it (a wave
    // that skips a tile skips all of its heads, so bv always holds this
    // tile's bias when it is used; the mask depends on the tile only)
    if (BIAS && (p.bias_sh != 0 || it_head(it) == 0)) {
      const float* bcol = p.bias + (int64_t)b * p.bias_sb + (int64_t)h_it * p.bias_sh +
                          min(kj, sp.lk - 1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qr = qr0 + 8 * (i >> 2) + 4 * hl + (i & 3);
        bv[i] = (kj < sp.lk && qr < sp.lq) ? bcol[(int64_t)qr * p.bias_sq] : 0.f;
      }
      // An element the mask hides gets the bias -inf: its probability
      // exp2(... - inf) is exactly zero, so dS is too, whatever the scale,
      // and one update serves every tile (a second, masked copy of it
      // spilled registers in the masked biased kernels).
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qr0 + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (!visible<CAUSAL, WINDOW>(qr, kj, delta, sp.lk, p.window)) bv[i] = -kInf;
        }
      }
    }

    // S = Q K^T and dP = dO V^T: lane = key kj, rows = queries
    // hb*32 + 8(i/4) + 4hl + i%4 of the staged tile
    f32x16 s, dp;
#pragma unroll
    for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
    for (int st = 0; st < KS; ++st) {
      s = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(tq, fq[st], 0)),
                 as_bf16x8(lds_read_b128_at(sk, fk[st], 0)), s);
      dp = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(tdo, fq[st], 0)),
                  as_bf16x8(lds_read_b128_at(sv, fk[st], 0)), dp);
    }

    // With dropout a tile that a mask crosses first replaces each hidden
    // score by s_hidden (a rarely taken step), so that its probability is
    // exactly zero and one update serves every tile: a second, masked copy
    // of the update next to the keep bits spilled 176 bytes per lane.  (A
    // bias carries the mask itself; without either, two copies measured
    // faster.)
    if constexpr (DROP) {
      if (__builtin_expect(need_mask, 0)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qr = qr0 + 8 * (i >> 2) + 4 * hl + (i & 3);
          if (!visible<CAUSAL, WINDOW>(qr, kj, delta, sp.lk, p.window)) s[i] = s_hidden;
        }
      }
    }

    // dropout keep bits, drawn and shared as in the four-wave kernel
    uint32_t kwd[8];
    if constexpr (DROP) {
      const int t = r32 & 3, a = (r32 >> 3) & 1, u = 4 * a + t;
      uint32_t mine = 0;
#pragma unroll
      for (int k2 = 0; k2 < 2; ++k2) {
        const int rho = 2 * u + k2;
        const int row = qr0 + 8 * (rho >> 2) + 4 * hl + (rho & 3);
        mine |= keep8(kj, row, h_it, b, p.seed_lo, p.seed_hi, p.drop_thresh) << (8 * k2);
      }
      const uint32_t other = row_ror8(mine);
      const uint32_t own_w[4] = {quad_bcast<0>(mine), quad_bcast<1>(mine),
                                 quad_bcast<2>(mine), quad_bcast<3>(mine)};
      const uint32_t oth_w[4] = {quad_bcast<0>(other), quad_bcast<1>(other),
                                 quad_bcast<2>(other), quad_bcast<3>(other)};
#pragma unroll
      for (int v = 0; v < 8; ++v)
        kwd[v] = (((v >> 2) == a) ? own_w[v & 3] : oth_w[v & 3]) >> u;
    }

    auto grads = [&](auto masked_tag) {
      constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int qrow = hb * 32 + 8 * r + 4 * hl;
        const float4 L = *reinterpret_cast<const float4*>(&tl[qrow]);
        const float4 Dl = *reinterpret_cast<const float4*>(&td[qrow]);
        const float Lv[4] = {L.x, L.y, L.z, L.w};
        const float Dv[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * r + e;
          float pv = fmaf(s[i], c, -Lv[e]);
          if constexpr (BIAS) pv = fmaf(bv[i], kLog2e, pv);
          pv = fast_exp2(pv);
          if (MASKED)
            pv = visible<CAUSAL, WINDOW>(i0 + qrow + e, kj, delta, sp.lk, p.window) ? pv : 0.f;
          if constexpr (DROP) {
            const bool kp = (kwd[i >> 1] >> (8 * (i & 1))) & 1u;
            s[i] = kp ? pv * p.drop_scale : 0.f;
            dp[i] = pv * ((kp ? dp[i] * p.drop_scale : 0.f) - Dv[e]);
          } else {
            s[i] = pv;
            dp[i] = pv * (dp[i] - Dv[e]);
          }
        }
      }
    };
    if (!BIAS && !DROP && need_mask)
      grads(std::true_type{});
    else
      grads(std::false_type{});

    // dV^T += dO^T P and dK^T += Q^T dS over 16-query chunks; chunk qc
    // holds queries 16qc + 4hl + {0..3} and 16qc + 8 + 4hl + {0..3} of the
    // wave's row half
#pragma unroll
    for (int qc = 0; qc < 2; ++qc) {
      const int j = qc * 8;
      const bf16x8 pb = pack8_t<F16>(s[j], s[j + 1], s[j + 2], s[j + 3], s[j + 4],
                                    s[j + 5], s[j + 6], s[j + 7]);
      const bf16x8 dsb = pack8_t<F16>(dp[j], dp[j + 1], dp[j + 2], dp[j + 3], dp[j + 4],
                                     dp[j + 5], dp[j + 6], dp[j + 7]);
      const uint32_t ro = 16 * qc * D * 2;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        dva[db] = mfma32_t<F16>(cat(lds_read_tr_at(tdo, troff[0][db], ro),
                             lds_read_tr_at(tdo, troff[1][db], ro)),
                         pb, dva[db]);
        dka[db] = mfma32_t<F16>(cat(lds_read_tr_at(tq, troff[0][db], ro),
                             lds_read_tr_at(tq, troff[1][db], ro)),
                         dsb, dka[db]);
      }
    }
  };

  if (n_it > 0) issue_it(0, sq0, sdo0);
  FA_STAGE_SYNC();
  for (int it = 0; it < n_it; it += 2) {
    if (tid < kQTile) {
      sl0[tid] = lse_r;
      sd0[tid] = dl_r;
    }
    dma_barrier();  // tile it (and, first, K and V) in place; buffer 1 is free
    if (it + 1 < n_it) issue_it(it + 1, sq1, sdo1);
    FA_STAGE_SYNC();
    compute(it, sq0, sdo0, sl0, sd0);
    FA_STAGE_SYNC();
    if (it + 1 >= n_it) break;
    if (tid < kQTile) {
      sl1[tid] = lse_r;
      sd1[tid] = dl_r;
    }
    dma_barrier();  // tile it + 1 is in buffer 1; buffer 0 is free
    if (it + 2 < n_it) issue_it(it + 2, sq0, sdo0);
    FA_STAGE_SYNC();
    compute(it + 1, sq1, sdo1, sl1, sd1);
    FA_STAGE_SYNC();
  }

  // Pair sum through LDS: the second row half hands over its dV partial, the
  // first its dK partial (each 16 f32x4 per lane, stored so that every
  // instruction writes 1 KB of consecutive bytes); then the first half
  // finishes dV and the second dK.  With no tile at all the K/V copies are
  // still in flight: wait for them before the buffers are reused.
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  f32x4* xv = reinterpret_cast<f32x4*>(kw < 2 ? sk : sv) + (kw & 1) * (DB * 4 * 64);
  f32x4* xk = reinterpret_cast<f32x4*>(kw == 0 ? sq0 : kw == 1 ? sdo0 : kw == 2 ? sq1 : sdo1);
  if (hb == 1) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xv[(db * 4 + r) * 64 + lane] = f32x4{dva[db][4 * r], dva[db][4 * r + 1],
                                             dva[db][4 * r + 2], dva[db][4 * r + 3]};
  } else {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        xk[(db * 4 + r) * 64 + lane] = f32x4{dka[db][4 * r], dka[db][4 * r + 1],
                                             dka[db][4 * r + 2], dka[db][4 * r + 3]};
  }
  __syncthreads();
  if (kj >= sp.lk) return;
  const int64_t off = (sp.k0 + kj) * kstride + (int64_t)hkv * D;
  if (hb == 0) {
    __bf16* dvp = (__bf16*)p.dv + off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 o = xv[(db * 4 + r) * 64 + lane];
        *reinterpret_cast<uint2*>(dvp + db * 32 + r * 8 + hl * 4) =
            pack4_t<F16>(dva[db][4 * r] + o[0], dva[db][4 * r + 1] + o[1],
                         dva[db][4 * r + 2] + o[2], dva[db][4 * r + 3] + o[3]);
      }
  } else {
    __bf16* dkp = (__bf16*)p.dk + off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const f32x4 o = xk[(db * 4 + r) * 64 + lane];
        *reinterpret_cast<uint2*>(dkp + db * 32 + r * 8 + hl * 4) =
            pack4_t<F16>((o[0] + dka[db][4 * r]) * p.scale, (o[1] + dka[db][4 * r + 1]) * p.scale,
                         (o[2] + dka[db][4 * r + 2]) * p.scale,
                         (o[3] + dka[db][4 * r + 3]) * p.scale);
      }
  }
}

// ------------------------------------------------------------ 3. dQ
// Two waves per SIMD in every instance.  With one dS update for masked and
// unmasked halves even the biased d = 128 kernels fit 256 registers; the
// unmasked one had run one wave per SIMD with each half's bias loaded a half
// ahead, and runs the biased GQA backward in 4.867 vs 5.513 ms at two.  (The
// bias entries are kept raw until use: 2.84 vs 3.32 ms for a causal GQA
// backward with a shared [8192, 8192] bias.)
template <int D, bool CAUSAL, bool WINDOW, bool VARLEN, bool BIAS, bool DROP, bool F16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2)))
void bwd_dq_kernel(BwdParams p, int num_qtiles) {
  constexpr int KS = D / 16, DB = D / 32, NB = kKTile / 32, NC = kKTile / 16;
  constexpr float kInf = __builtin_inff();
  // two K/V buffers as distinct objects, so that reads of one buffer are not
  // ordered behind the loads still landing in the other
  __shared__ __attribute__((aligned(1024))) __bf16 sk0[kKTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sv0[kKTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sk1[kKTile * D];
  __shared__ __attribute__((aligned(1024))) __bf16 sv1[kKTile * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int G = p.group;
  const int gi = id % G;
  id /= G;
  const int t_ord = id % num_qtiles;
  id /= num_qtiles;
  // the KV head is the slowest index, so each XCD's contiguous range holds
  // whole KV heads (their query heads share the K/V in that XCD's L2) and
  // every XCD sees the same mix of sequences (balanced for packed batches)
  const int b = id % p.B;
  const int hkv = id / p.B;
  const int h = hkv * G + gi;
  const int qt = CAUSAL ? (num_qtiles - 1 - t_ord) : t_ord;
  const int32_t* cu = VARLEN ? p.cu_seqlens : nullptr;
  const SeqSpan sp = seq_span(cu, b, p.Nq, p.Nk);
  const int q_start = qt * kQBlock;
  if (q_start >= sp.lq) return;
  const int delta = sp.lk - sp.lq;
  const int q_end = min(q_start + kQBlock, sp.lq);
  int kv_lo = 0, kv_hi = sp.lk;
  if (CAUSAL) kv_hi = min(kv_hi, q_end + delta);
  if (WINDOW) kv_lo = max(0, q_start + delta - p.window + 1);
  kv_lo = (kv_lo / kKTile) * kKTile;

  const int64_t qstride = (int64_t)p.Hq * D, kstride = (int64_t)p.Hkv * D;
  const __bf16* Kg = (const __bf16*)p.k + sp.k0 * kstride + (int64_t)hkv * D;
  const __bf16* Vg = (const __bf16*)p.v + sp.k0 * kstride + (int64_t)hkv * D;
  const float c = p.scale_log2;

  const int qi = q_start + wave * 32 + r32;
  bf16x8 qf[KS], dof[KS];
  float lse2 = kInf, dq_d = 0.f;
  if (qi < sp.lq) {
    const int64_t off = (sp.q0 + qi) * qstride + (int64_t)h * D + hl * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.q + off + 16 * s));
      dof[s] = as_bf16x8(*reinterpret_cast<const uint4*>((const __bf16*)p.dout + off + 16 * s));
    }
    const int64_t li = lse_index(cu, p.B, p.Hq, p.Nq, b, h, sp.q0, qi);
    const float lv = p.lse[li];
    lse2 = (lv == -kInf) ? kInf : lv * kLog2e;
    dq_d = p.delta[li];
  } else {
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = dof[s] = as_bf16x8(make_uint4(0, 0, 0, 0));
  }

  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;

  const int qlo_w = q_start + wave * 32;
  const int qhi_w = min(qlo_w + 31, sp.lq - 1);
  const float* bias_bh = BIAS ? p.bias + (int64_t)b * p.bias_sb + (int64_t)h * p.bias_sh
                              : nullptr;
  const uint32_t bias_lane = (uint32_t)(r32 * p.bias_sq) * 4u;
  // bias of this lane's row at keys j0 + 32kb + 8g + 4hl + {0..3} (branch-free
  // loads, bias_rsrc)
  auto load_bias_half = [&](int j0, int kb, float (&dst)[16]) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = bias_rsrc(bias_bh, p.bias_sq, qlo_w, sp.lq, j0, sp.lk);
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 t = bias_load4(rs, bias_lane, kb * 32 + g * 8 + hl * 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[4 * g + e] = t[e];
    }
  };

  // Lane byte offsets of the LDS reads inside a K or V tile (same swizzled
  // layout as the forward): 128-bit fragment reads per k-step, transposing
  // reads of K per output column block; 32-row blocks and 16-row chunks add
  // whole rows, which go into the instruction's offset field.
  const int tr_row = 4 * hl + ((lane & 15) >> 2);
  const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
  uint32_t foff[KS], troff[2][DB];
#pragma unroll
  for (int st = 0; st < KS; ++st) foff[st] = 2 * tile_off<D>(r32, st * 16 + hl * 8);
#pragma unroll
  for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
    for (int db = 0; db < DB; ++db)
      troff[h2][db] = 2 * tile_off<D>(tr_row + 8 * h2, db * 32 + tr_col);

  // K and V tiles go straight from global memory into LDS (buffer loads with
  // the LDS destination), two buffers each; the loads of tile j+1 are issued
  // after the barrier that opens tile j.
  const uint32_t kstride_b = (uint32_t)(kstride * 2);
  const TileDma<D, kKTile, kThreads / 64> dma(wave, lane, kstride_b);
  auto issue = [&](int j0, __bf16* kb, __bf16* vb) {
    dma.issue(Kg, kstride_b, j0, sp.lk, kb);
    dma.issue(Vg, kstride_b, j0, sp.lk, vb);
  };
  if (kv_lo < kv_hi) issue(kv_lo, sk0, sv0);
  FA_STAGE_SYNC();

  auto compute = [&](int j0, const __bf16* kt, const __bf16* vt) {
    bool active = qlo_w <= qhi_w;
    if (CAUSAL) active = active && (j0 <= qhi_w + delta);
    if (WINDOW) active = active && (j0 + kKTile - 1 > qlo_w + delta - p.window);
    if (!active) return;
    bool need_mask = (j0 + kKTile > sp.lk);
    if (CAUSAL) need_mask = need_mask || (j0 + kKTile - 1 > qlo_w + delta);
    if (WINDOW) need_mask = need_mask || (qhi_w + delta - j0 >= p.window);

    // One 32-key half kb of the tile at a time, to keep two score blocks
    // live instead of four.  S^T = K Q^T and dP^T = V dO^T: lane = query
    // qi, rows = keys j0 + 32kb + 8(i/4) + 4hl + i%4.
    // Without a bias the half computes P for every element and zeroes the
    // invisible entries of a masked half in a separate, rarely taken step
    // before one dS update (long causal backward 1.6 % faster); with a bias
    // an invisible element's bias becomes -inf in such a step instead, so
    // its probability is exactly zero (the split form spills there).  Either
    // way one dS update serves masked and unmasked halves.
    constexpr bool kSplitMask = !BIAS;
    auto half = [&](int kb) __attribute__((always_inline)) {
      float bv[BIAS ? 16 : 1];
      if constexpr (BIAS) load_bias_half(j0, kb, bv);
      // this lane's key of element i is j0 + 32kb + 4hl + 8(i/4) + i%4
      const int base = j0 + kb * 32 + 4 * hl;
      const int end = sp.lk - base, hi = qi + delta - base, lo = qi + delta - p.window - base;
      auto visible_off = [&](int i) {
        const int off = (i >> 2) * 8 + (i & 3);
        bool ok = off < end;
        if (CAUSAL) ok = ok && off <= hi;
        if (WINDOW) ok = ok && off > lo;
        return ok;
      };
      if constexpr (BIAS) {
        if (__builtin_expect(need_mask, 0)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!visible_off(i)) bv[i] = -kInf;
        }
      }
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const uint32_t ro = kb * 32 * D * 2;
        s = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(kt, foff[st], ro)), qf[st], s);
        dp = mfma32_t<F16>(as_bf16x8(lds_read_b128_at(vt, foff[st], ro)), dof[st], dp);
      }
      // a few fragment reads ahead of the MFMAs, then one read per MFMA
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, kReadsAhead, 0);
#pragma unroll
      for (int i = 0; i < 2 * KS - kReadsAhead; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, kReadsAhead, 0);

      // P = exp2(S c - LSE log2 e), dS = P (dP - D); element i holds key
      // base + off with off = 8(i/4) + i%4
      // dropout: two generator calls cover the half's 16 keys of this lane,
      // base + 16c + 8a + {0..3}: element i takes slot i & 7 of call i >> 3
      uint4 dw[2];
      if constexpr (DROP) {
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2)
          dw[c2] = drop_call(base + 16 * c2, qi, h, b, p.seed_lo, p.seed_hi);
      }
      auto ds_of = [&](int i, float pv) {
        if constexpr (DROP)
          dp[i] = pv * ((slot_of(dw[i >> 3], i & 7) >= p.drop_thresh ? dp[i] * p.drop_scale
                                                                     : 0.f) - dq_d);
        else
          dp[i] = pv * (dp[i] - dq_d);
      };
      if constexpr (kSplitMask) {
        // P for every element, then (rarely) the invisible entries zeroed
        // in a separate step, then one dS update
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = fast_exp2(fmaf(s[i], c, -lse2));
        if (__builtin_expect(need_mask, 0)) {
#pragma unroll
          for (int i = 0; i < 16; ++i)
            if (!visible_off(i)) s[i] = 0.f;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) ds_of(i, s[i]);
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fmaf(s[i], c, -lse2);
          if constexpr (BIAS) pv = fmaf(bv[i], kLog2e, pv);
          ds_of(i, fast_exp2(pv));
        }
      }

      // dQ^T += K^T dS^T over this half's two 16-key chunks (same key
      // permutation as the forward's P V product)
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const int kc = 2 * kb + h2, j = h2 * 8;
        const bf16x8 dsb = pack8_t<F16>(dp[j], dp[j + 1], dp[j + 2], dp[j + 3], dp[j + 4],
                                       dp[j + 5], dp[j + 6], dp[j + 7]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const uint32_t ro = 16 * kc * D * 2;
          acc[db] = mfma32_t<F16>(cat(lds_read_tr_at(kt, troff[0][db], ro),
                               lds_read_tr_at(kt, troff[1][db], ro)),
                           dsb, acc[db]);
        }
      }
    };
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) half(kb);
  };

#pragma nounroll
  for (int j0 = kv_lo; j0 < kv_hi; j0 += 2 * kKTile) {
    dma_barrier();  // tile j0 is in buffer 0; buffer 1 is free
    if (j0 + kKTile < kv_hi) issue(j0 + kKTile, sk1, sv1);
    FA_STAGE_SYNC();
    compute(j0, sk0, sv0);
    FA_STAGE_SYNC();
    if (j0 + kKTile >= kv_hi) break;
    dma_barrier();  // tile j0 + kKTile is in buffer 1; buffer 0 is free
    if (j0 + 2 * kKTile < kv_hi) issue(j0 + 2 * kKTile, sk0, sv0);
    FA_STAGE_SYNC();
    compute(j0 + kKTile, sk1, sv1);
    FA_STAGE_SYNC();
  }

  if (qi < sp.lq) {
    __bf16* dqp = (__bf16*)p.dq + (sp.q0 + qi) * qstride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        *reinterpret_cast<uint2*>(dqp + db * 32 + r * 8 + hl * 4) =
            pack4_t<F16>(acc[db][4 * r] * p.scale, acc[db][4 * r + 1] * p.scale,
                         acc[db][4 * r + 2] * p.scale, acc[db][4 * r + 3] * p.scale);
      }
  }
}

// dK/dV kernel choice: the eight-wave kernel for d = 128, the four-wave one
// for d = 64 (which already runs two waves per SIMD there).  With dropout too
// the eight-wave kernel (one update body) is faster than the four-wave one at
// one wave per SIMD: 2.201 vs 2.390 ms for the backward of the GQA prefill
// shape with p = 0.1.
template <int D>
constexpr bool kUseDkdv8 = D == 128;

template <int D, bool CAUSAL, bool WINDOW, bool VARLEN, bool BIAS = false, bool DROP = false,
          bool F16 = false>
hipError_t launch4(const BwdParams& p, hipStream_t stream) {
  const int nkt = (p.Nk + kKeyBlock - 1) / kKeyBlock;
  const int nqt = (p.Nq + kQBlock - 1) / kQBlock;
  if constexpr (kUseDkdv8<D>)
    hipLaunchKernelGGL((bwd_dkdv8_kernel<D, CAUSAL, WINDOW, VARLEN, BIAS, DROP, F16>),
                       dim3((unsigned)p.B * p.Hkv * nkt), dim3(kDkdv8Threads), 0, stream, p, nkt);
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, WINDOW, VARLEN, BIAS, DROP, F16>),
                       dim3((unsigned)p.B * p.Hkv * nkt), dim3(kThreads), 0, stream, p, nkt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, WINDOW, VARLEN, BIAS, DROP, F16>),
                     dim3((unsigned)p.B * p.Hq * nqt), dim3(kThreads), 0, stream, p, nqt);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool WINDOW, bool F16>
hipError_t launch3(const BwdParams& p, hipStream_t stream) {
  if constexpr (F16)  // fp16 operands: the plain backward only
    return p.cu_seqlens ? launch4<D, CAUSAL, WINDOW, true, false, false, true>(p, stream)
                        : launch4<D, CAUSAL, WINDOW, false, false, false, true>(p, stream);
  if (p.bias) return launch4<D, CAUSAL, WINDOW, false, true>(p, stream);  // dense only
  if (p.dropout)  // no bias
    return p.cu_seqlens ? launch4<D, CAUSAL, WINDOW, true, false, true>(p, stream)
                        : launch4<D, CAUSAL, WINDOW, false, false, true>(p, stream);
  return p.cu_seqlens ? launch4<D, CAUSAL, WINDOW, true>(p, stream)
                      : launch4<D, CAUSAL, WINDOW, false>(p, stream);
}

template <int D, bool F16>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Nq * p.Hq;  // >= tokens x heads, also when packed
  const int64_t rows_per_block = kThreads / (D / 8);
  hipLaunchKernelGGL((bwd_pre_kernel<D, F16>),
                     dim3((unsigned)((rows + rows_per_block - 1) / rows_per_block)),
                     dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch3<D, true, true, F16>(p, stream) : launch3<D, true, false, F16>(p, stream);
  return win ? launch3<D, false, true, F16>(p, stream) : launch3<D, false, false, F16>(p, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64, false>(p, stream) : launch_d<128, false>(p, stream);
}

hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64, true>(p, stream) : launch_d<128, true>(p, stream);
}

}  // namespace fa

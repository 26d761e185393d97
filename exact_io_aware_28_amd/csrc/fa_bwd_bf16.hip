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
//   2. bwd_dkdv: a work-group owns 128 keys of one KV head (one wave per 32
//      keys, each lane one key); it walks every query head of the KV head's
//      group and every query tile that can see its keys, with Q, dO, LSE and
//      D tiles staged in LDS.  dK and dV stay in registers and are written
//      once, so the GQA sum over the group needs no atomics.
//   3. bwd_dq:   a work-group owns 128 query rows of one head (one lane per
//      query row, as in the forward) and walks the key tiles it can see,
//      rebuilding S and dP to accumulate dQ.  This recomputes two of the
//      five products a second time, in exchange for no cross-work-group
//      reduction.
// All products run on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the
// probability and dS tiles are rounded to bf16 as MFMA operands.
#include <type_traits>

#include "fa_device.h"

namespace fa {
namespace {

constexpr int kThreads = 256;
constexpr int kKeyBlock = 128;  // keys per dK/dV work-group (4 waves x 32)
constexpr int kQTile = 64;      // query rows per staged tile in dK/dV
constexpr int kQBlock = 128;    // query rows per dQ work-group (4 waves x 32)
constexpr int kKTile = 64;      // keys per staged tile in dQ

// ------------------------------------------------------------ 1. D = dO . O
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_pre_kernel(BwdParams p) {
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t token = idx / p.Hq;
  const int h = (int)(idx % p.Hq);
  int64_t out;
  if (p.cu_seqlens) {
    const int64_t T = p.cu_seqlens[p.B];
    if (token >= T) return;
    out = (int64_t)h * T + token;
  } else {
    if (token >= (int64_t)p.B * p.Nq) return;
    const int64_t b = token / p.Nq, i = token % p.Nq;
    out = (b * p.Hq + h) * p.Nq + i;
  }
  const int64_t base = (token * p.Hq + h) * D;
  const uint4* o4 = reinterpret_cast<const uint4*>((const __bf16*)p.o + base);
  const uint4* d4 = reinterpret_cast<const uint4*>((const __bf16*)p.dout + base);
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const bf16x8 a = as_bf16x8(o4[c]), g = as_bf16x8(d4[c]);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)a[e], (float)g[e], acc);
  }
  p.delta[out] = acc;
}

// ------------------------------------------------------------ 2. dK, dV
template <int D, bool CAUSAL, bool WINDOW, bool VARLEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dkdv_kernel(BwdParams p, int num_ktiles) {
  constexpr int KS = D / 16, DB = D / 32, QB = kQTile / 32;
  constexpr float kInf = __builtin_inff();
  __shared__ __attribute__((aligned(16))) __bf16 sq[2][kQTile * D];
  __shared__ __attribute__((aligned(16))) __bf16 sdo[2][kQTile * D];
  __shared__ __attribute__((aligned(16))) float slse[2][kQTile];
  __shared__ __attribute__((aligned(16))) float sdl[2][kQTile];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int kt = id % num_ktiles;  // key tile 0 first: it sees the most rows
  id /= num_ktiles;
  const int hkv = id % p.Hkv;
  const int b = id / p.Hkv;
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

  TilePairStager<D, kQTile, kThreads> stage(tid);
  float lse_r = 0.f, dl_r = 0.f;  // staged row statistics (threads < kQTile)
  auto load_it = [&](int it) {
    const int gi = it / n_qt;
    const int i0 = q_lo + (it % n_qt) * kQTile;
    const int h = hkv * G + gi;
    const int64_t hoff = sp.q0 * qstride + (int64_t)h * D;
    stage.load((const __bf16*)p.q + hoff, (const __bf16*)p.dout + hoff, qstride, i0, sp.lq);
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

  int buf = 0;
  if (n_it > 0) load_it(0);
  for (int it = 0; it < n_it; ++it) {
    const int i0 = q_lo + (it % n_qt) * kQTile;
    stage.store(sq[buf], sdo[buf]);
    if (tid < kQTile) {
      slse[buf][tid] = lse_r;
      sdl[buf][tid] = dl_r;
    }
    __syncthreads();
    if (it + 1 < n_it) load_it(it + 1);

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

      // S = Q K^T and dP = dO V^T: lane = key kj, rows = queries
      // qb*32 + 8(i/4) + 4hl + i%4 of the staged tile
      f32x16 s, dp;
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = dp[i] = 0.f;
#pragma unroll
      for (int st = 0; st < KS; ++st) {
        const int off = tile_off<D>(qb * 32 + r32, st * 16 + hl * 8);
        s = mfma32(as_bf16x8(lds_read_b128(sq[buf], off)), kf[st], s);
        dp = mfma32(as_bf16x8(lds_read_b128(sdo[buf], off)), vf[st], dp);
      }

      auto grads = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qrow = qb * 32 + 8 * r + 4 * hl;
          const float4 L = *reinterpret_cast<const float4*>(&slse[buf][qrow]);
          const float4 Dl = *reinterpret_cast<const float4*>(&sdl[buf][qrow]);
          const float Lv[4] = {L.x, L.y, L.z, L.w};
          const float Dv[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * r + e;
            float pv = fast_exp2(fmaf(s[i], c, -Lv[e]));
            if (MASKED)
              pv = visible<CAUSAL, WINDOW>(i0 + qrow + e, kj, delta, sp.lk, p.window) ? pv : 0.f;
            s[i] = pv;
            dp[i] = pv * (dp[i] - Dv[e]);
          }
        }
      };
      if (need_mask)
        grads(std::true_type{});
      else
        grads(std::false_type{});

      // dV^T += dO^T P and dK^T += Q^T dS over 16-query chunks; chunk qc
      // holds queries 16qc + 4hl + {0..3} and 16qc + 8 + 4hl + {0..3}
      const int tr_row = qb * 32 + 4 * hl + ((lane & 15) >> 2);
      const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
      for (int qc = 0; qc < 2; ++qc) {
        const int j = qc * 8;
        const bf16x8 pb = pack_bf16x8(s[j], s[j + 1], s[j + 2], s[j + 3], s[j + 4],
                                      s[j + 5], s[j + 6], s[j + 7]);
        const bf16x8 dsb = pack_bf16x8(dp[j], dp[j + 1], dp[j + 2], dp[j + 3], dp[j + 4],
                                       dp[j + 5], dp[j + 6], dp[j + 7]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + tr_col;
          const int o0 = tile_off<D>(16 * qc + tr_row, col);
          const int o1 = tile_off<D>(16 * qc + 8 + tr_row, col);
          dva[db] = mfma32(cat(lds_read_tr(sdo[buf], o0), lds_read_tr(sdo[buf], o1)), pb, dva[db]);
          dka[db] = mfma32(cat(lds_read_tr(sq[buf], o0), lds_read_tr(sq[buf], o1)), dsb, dka[db]);
        }
      }
    }
    buf ^= 1;
  }

  if (kj < sp.lk) {
    const int64_t off = (sp.k0 + kj) * kstride + (int64_t)hkv * D;
    __bf16* dkp = (__bf16*)p.dk + off;
    __bf16* dvp = (__bf16*)p.dv + off;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = (__bf16)(dka[db][4 * r + e] * p.scale);
          wv[e] = (__bf16)(dva[db][4 * r + e]);
        }
        const int col = db * 32 + r * 8 + hl * 4;
        *reinterpret_cast<uint2*>(dkp + col) = __builtin_bit_cast(uint2, wk);
        *reinterpret_cast<uint2*>(dvp + col) = __builtin_bit_cast(uint2, wv);
      }
  }
}

// ------------------------------------------------------------ 3. dQ
template <int D, bool CAUSAL, bool WINDOW, bool VARLEN>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1)))
void bwd_dq_kernel(BwdParams p, int num_qtiles) {
  constexpr int KS = D / 16, DB = D / 32, NB = kKTile / 32, NC = kKTile / 16;
  constexpr float kInf = __builtin_inff();
  __shared__ __attribute__((aligned(16))) __bf16 sk[2][kKTile * D];
  __shared__ __attribute__((aligned(16))) __bf16 sv[2][kKTile * D];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hl = lane >> 5, r32 = lane & 31;

  uint32_t id = xcd_logical_id(blockIdx.x, gridDim.x);
  const int G = p.group;
  const int gi = id % G;
  id /= G;
  const int t_ord = id % num_qtiles;
  id /= num_qtiles;
  const int hkv = id % p.Hkv;
  const int b = id / p.Hkv;
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
  TilePairStager<D, kKTile, kThreads> stage(tid);
  int buf = 0;
  if (kv_lo < kv_hi) stage.load(Kg, Vg, kstride, kv_lo, sp.lk);
  for (int j0 = kv_lo; j0 < kv_hi; j0 += kKTile) {
    stage.store(sk[buf], sv[buf]);
    __syncthreads();
    if (j0 + kKTile < kv_hi) stage.load(Kg, Vg, kstride, j0 + kKTile, sp.lk);

    bool active = qlo_w <= qhi_w;
    if (CAUSAL) active = active && (j0 <= qhi_w + delta);
    if (WINDOW) active = active && (j0 + kKTile - 1 > qlo_w + delta - p.window);
    if (active) {
      bool need_mask = (j0 + kKTile > sp.lk);
      if (CAUSAL) need_mask = need_mask || (j0 + kKTile - 1 > qlo_w + delta);
      if (WINDOW) need_mask = need_mask || (qhi_w + delta - j0 >= p.window);

      // S^T = K Q^T and dP^T = V dO^T: lane = query qi, rows = keys
      f32x16 s[NB], dp[NB];
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[kb][i] = dp[kb][i] = 0.f;
#pragma unroll
        for (int st = 0; st < KS; ++st) {
          const int off = tile_off<D>(kb * 32 + r32, st * 16 + hl * 8);
          s[kb] = mfma32(as_bf16x8(lds_read_b128(sk[buf], off)), qf[st], s[kb]);
          dp[kb] = mfma32(as_bf16x8(lds_read_b128(sv[buf], off)), dof[st], dp[kb]);
        }
      }
      auto grads = [&](auto masked_tag) {
        constexpr bool MASKED = decltype(masked_tag)::value;
#pragma unroll
        for (int kb = 0; kb < NB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            float pv = fast_exp2(fmaf(s[kb][i], c, -lse2));
            if (MASKED) {
              const int j = j0 + kb * 32 + (i >> 2) * 8 + hl * 4 + (i & 3);
              pv = visible<CAUSAL, WINDOW>(qi, j, delta, sp.lk, p.window) ? pv : 0.f;
            }
            dp[kb][i] = pv * (dp[kb][i] - dq_d);
          }
      };
      if (need_mask)
        grads(std::true_type{});
      else
        grads(std::false_type{});

      // dQ^T += K^T dS^T over 16-key chunks (same key permutation as the
      // forward's P V product)
      const int tr_row = 4 * hl + ((lane & 15) >> 2);
      const int tr_col = ((lane >> 4) & 1) * 16 + (lane & 3) * 4;
#pragma unroll
      for (int kc = 0; kc < NC; ++kc) {
        const int kb = kc >> 1, j = (kc & 1) * 8;
        const bf16x8 dsb = pack_bf16x8(dp[kb][j], dp[kb][j + 1], dp[kb][j + 2], dp[kb][j + 3],
                                       dp[kb][j + 4], dp[kb][j + 5], dp[kb][j + 6], dp[kb][j + 7]);
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int col = db * 32 + tr_col;
          const bf16x4 lo = lds_read_tr(sk[buf], tile_off<D>(16 * kc + tr_row, col));
          const bf16x4 hi = lds_read_tr(sk[buf], tile_off<D>(16 * kc + 8 + tr_row, col));
          acc[db] = mfma32(cat(lo, hi), dsb, acc[db]);
        }
      }
    }
    buf ^= 1;
  }

  if (qi < sp.lq) {
    __bf16* dqp = (__bf16*)p.dq + (sp.q0 + qi) * qstride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * r + e] * p.scale);
        *reinterpret_cast<uint2*>(dqp + db * 32 + r * 8 + hl * 4) = __builtin_bit_cast(uint2, w);
      }
  }
}

template <int D, bool CAUSAL, bool WINDOW, bool VARLEN>
hipError_t launch4(const BwdParams& p, hipStream_t stream) {
  const int nkt = (p.Nk + kKeyBlock - 1) / kKeyBlock;
  const int nqt = (p.Nq + kQBlock - 1) / kQBlock;
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, WINDOW, VARLEN>),
                     dim3((unsigned)p.B * p.Hkv * nkt), dim3(kThreads), 0, stream, p, nkt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, WINDOW, VARLEN>),
                     dim3((unsigned)p.B * p.Hq * nqt), dim3(kThreads), 0, stream, p, nqt);
  return hipGetLastError();
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch3(const BwdParams& p, hipStream_t stream) {
  return p.cu_seqlens ? launch4<D, CAUSAL, WINDOW, true>(p, stream)
                      : launch4<D, CAUSAL, WINDOW, false>(p, stream);
}

template <int D>
hipError_t launch_d(const BwdParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.Nq * p.Hq;
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch3<D, true, true>(p, stream) : launch3<D, true, false>(p, stream);
  return win ? launch3<D, false, true>(p, stream) : launch3<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream) {
  return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace fa

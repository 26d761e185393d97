// Exact attention forward in fp32 (inputs, scores, softmax state, output).
//
// Same tiling and online-softmax recurrence as the bf16 kernel (llms.blog
// "FlashAttention: How IO-Aware Tiling and Online Softmax Solved Transformer
// Memory Bottlenecks", "1. IO-Aware Tiling" and "2. Online Softmax
// Reduction"), on the vector ALUs: fp32 inputs have no use for the bf16
// matrix cores, and this path serves small problems where launch latency, not
// arithmetic, sets the time.
//
// One wave of 64 lanes owns 64 query rows of one (sequence, head); each lane
// keeps its query row's output accumulator in VGPRs.  Q rows sit in LDS with
// a one-float row pad (lane i reads row i: distinct banks); 32-key K and V
// tiles are staged in LDS and read by all lanes at the same address
// (broadcast).
#include "fa_device.h"

namespace fa {
namespace {

constexpr int kRows = 64;  // query rows per work-group (one wave)
constexpr int kKeys = 32;  // keys per K/V tile

template <int D, bool CAUSAL, bool WINDOW, bool VARLEN>
__global__ __launch_bounds__(kRows) void fwd_f32_kernel(FwdParams p) {
  constexpr float kInf = __builtin_inff();
  __shared__ float sq[kRows * (D + 1)];
  __shared__ __attribute__((aligned(16))) float sk[kKeys * D];
  __shared__ __attribute__((aligned(16))) float sv[kKeys * D];

  const int lane = threadIdx.x;
  uint32_t id = blockIdx.x;
  const int qt = id % p.num_qtiles;
  id /= p.num_qtiles;
  const int h = id % p.Hq;
  const int b = id / p.Hq;
  const int g = h / p.group;
  const SeqSpan sp = seq_span(VARLEN ? p.cu_seqlens : nullptr, b, p.Nq, p.Nk);
  const int q_start = qt * kRows;
  if (q_start >= sp.lq) return;
  const int delta = sp.lk - sp.lq;
  const int q_end = min(q_start + kRows, sp.lq);

  const int64_t qstride = (int64_t)p.Hq * D, kstride = (int64_t)p.Hkv * D;
  const float* Qg = (const float*)p.q + sp.q0 * qstride + (int64_t)h * D;
  const float* Kg = (const float*)p.k + sp.k0 * kstride + (int64_t)g * D;
  const float* Vg = (const float*)p.v + sp.k0 * kstride + (int64_t)g * D;

  // stage the query block (rows past the sequence are zero)
  for (int e = lane; e < kRows * D; e += kRows) {
    const int r = e / D, col = e % D;
    sq[r * (D + 1) + col] = (q_start + r < sp.lq) ? Qg[(q_start + r) * qstride + col] : 0.f;
  }

  int kv_lo = 0, kv_hi = sp.lk;
  if (CAUSAL) kv_hi = min(kv_hi, q_end + delta);
  if (WINDOW) kv_lo = max(0, q_start + delta - p.window + 1);

  const int qi = q_start + lane;
  const float c = p.scale_log2;
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  float m_run = -kInf, l_run = 0.f;

  for (int j0 = kv_lo; j0 < kv_hi; j0 += kKeys) {
    __syncthreads();  // previous tile fully consumed (and Q staged)
    for (int e = lane; e < kKeys * D; e += kRows) {
      const int r = e / D, col = e % D;
      const bool in = j0 + r < sp.lk;
      sk[e] = in ? Kg[(j0 + r) * kstride + col] : 0.f;
      sv[e] = in ? Vg[(j0 + r) * kstride + col] : 0.f;
    }
    __syncthreads();

    // scaled scores x_j = (q . k_j) * scale * log2(e); invisible -> -inf
    float x[kKeys];
    float tmax = -kInf;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) dot = fmaf(sq[lane * (D + 1) + e], sk[j * D + e], dot);
      const bool ok = visible<CAUSAL, WINDOW>(qi, j0 + j, delta, sp.lk, p.window);
      x[j] = ok ? dot * c : -kInf;
      tmax = fmaxf(tmax, x[j]);
    }
    const float m_new = fmaxf(m_run, tmax);
    const float m_sub = (m_new == -kInf) ? 0.f : m_new;
    const float alpha = exp2f(m_run - m_sub);
    l_run *= alpha;
#pragma unroll
    for (int e = 0; e < D; ++e) acc[e] *= alpha;
#pragma unroll
    for (int j = 0; j < kKeys; ++j) {
      const float pj = exp2f(x[j] - m_sub);
      l_run += pj;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(pj, sv[j * D + e], acc[e]);
    }
    m_run = m_new;
  }

  if (qi < sp.lq) {
    const float inv = (l_run == 0.f) ? 0.f : 1.0f / l_run;
    float* op = (float*)p.o + (sp.q0 + qi) * qstride + (int64_t)h * D;
#pragma unroll
    for (int e = 0; e < D; e += 4)
      *reinterpret_cast<float4*>(op + e) =
          make_float4(acc[e] * inv, acc[e + 1] * inv, acc[e + 2] * inv, acc[e + 3] * inv);
    const float m_sub = (m_run == -kInf) ? 0.f : m_run;
    p.lse[lse_index(VARLEN ? p.cu_seqlens : nullptr, p.B, p.Hq, p.Nq, b, h, sp.q0, qi)] =
        (l_run == 0.f) ? -kInf : (m_sub + log2f(l_run)) * kLn2;
  }
}

template <int D, bool CAUSAL, bool WINDOW>
hipError_t launch3(const FwdParams& p, hipStream_t stream) {
  dim3 grid((unsigned)p.B * p.Hq * p.num_qtiles), block(kRows);
  if (p.cu_seqlens)
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, WINDOW, true>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, WINDOW, false>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const FwdParams& p, hipStream_t stream) {
  const bool win = p.window > 0;
  if (p.causal)
    return win ? launch3<D, true, true>(p, stream) : launch3<D, true, false>(p, stream);
  return win ? launch3<D, false, true>(p, stream) : launch3<D, false, false>(p, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdParams& p_in, hipStream_t stream) {
  FwdParams p = p_in;
  p.num_qtiles = (p.Nq + kRows - 1) / kRows;
  return p.d == 64 ? launch_d<64>(p, stream) : launch_d<128>(p, stream);
}

}  // namespace fa

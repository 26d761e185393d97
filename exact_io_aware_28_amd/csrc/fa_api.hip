// C ABI of libfa_mi355x (declared in include/fa_mi355x.h): argument
// validation, then dispatch to the kernel launchers.
//
// Validation touches no HIP API, so a rejected call enqueues nothing and the
// checks can be exercised on a machine without a GPU.  (fa_decode_noalloc
// asks the runtime for its scratch array's device address only after its
// arguments have passed.)
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <climits>
#include <mutex>

#include "fa_mi355x.h"
#include "fa_params.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Checks shared by every entry point.  `elem_align` is the required pointer
// alignment of the q/k/v/o-like tensors (16 bytes: the kernels move them in
// 128-bit pieces).
int check_common(const void* const* tensors, int ntensors, const float* const* stats,
                 int nstats, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                 float scale, int causal, int window, const int32_t* cu_seqlens,
                 int qtile_rows) {
  for (int i = 0; i < ntensors; ++i)
    if (!tensors[i] || !aligned(tensors[i], 16)) return FA_ERR_INVALID_ARG;
  for (int i = 0; i < nstats; ++i)
    if (!stats[i] || !aligned(stats[i], 4)) return FA_ERR_INVALID_ARG;
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return FA_ERR_INVALID_ARG;
  if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
  if (window < 0) return FA_ERR_INVALID_ARG;
  if (cu_seqlens && !aligned(cu_seqlens, 4)) return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (cu_seqlens && Nq != Nk) return FA_ERR_UNSUPPORTED;
  // element offsets are 64-bit; the launch grid must fit 32 bits
  const int64_t tiles = (int64_t)B * Hq * ((Nq + qtile_rows - 1) / qtile_rows);
  if (tiles > (int64_t)UINT32_MAX / 2) return FA_ERR_UNSUPPORTED;
  if ((int64_t)B * Nq * Hq > (int64_t)INT32_MAX * 64) return FA_ERR_UNSUPPORTED;
  // a staged tile (64 rows of one head) must span less than 4 GiB of its
  // tensor: the buffer descriptors that bound it count bytes in 32 bits
  if ((int64_t)Hq * d * 2 * 64 >= ((int64_t)1 << 32)) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

fa::FwdParams fwd_params(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                         int causal, int window, const int32_t* cu) {
  fa::FwdParams p;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_seqlens = cu;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.num_qtiles = 0;  // set by the launcher from its tile height
  p.xcd_groups = 0;
  p.bias = nullptr;
  p.bias_sb = p.bias_sh = p.bias_sq = 0;
  p.dropout = 0;
  p.drop_thresh = 0;
  p.seed_lo = p.seed_hi = 0;
  p.drop_scale = 1.0f;
  return p;
}

// Dropout probability in [0, 1): 16-bit threshold T = floor(p * 2^16) (a
// key is dropped iff its 16-bit Philox slot is below it) and the scale
// 2^16 / (2^16 - T), the inverse of the exact keep probability.
int check_dropout(float dropout_p, uint32_t* thresh, float* scale) {
  if (!(dropout_p >= 0.0f && dropout_p < 1.0f)) return FA_ERR_INVALID_ARG;  // also NaN
  *thresh = (uint32_t)((double)dropout_p * 65536.0);
  *scale = (float)(65536.0 / (65536.0 - (double)*thresh));
  return FA_OK;
}

// An additive bias: non-null, 4-byte aligned, non-negative element strides.
// The kernels read a wave's 32 bias rows through one buffer descriptor whose
// byte range, at most (31 sq + Nk) x 4, must stay below 2^32.
int check_bias(const float* bias, int64_t sb, int64_t sh, int64_t sq, int Nk) {
  if (!bias || !aligned(bias, 4)) return FA_ERR_INVALID_ARG;
  if (sb < 0 || sh < 0 || sq < 0) return FA_ERR_INVALID_ARG;
  if (sq > ((int64_t)1 << 40) || (31 * sq + (int64_t)Nk) * 4 >= ((int64_t)1 << 32))
    return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
           int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
           const int32_t* cu_seqlens, void* stream) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                        cu_seqlens, 64);
  if (st != FA_OK) return st;
  fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window, cu_seqlens);
  return fa::launch_fwd_bf16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_f16(const void* q, const void* k, const void* v, void* o, float* lse, int B,
               int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
               const int32_t* cu_seqlens, void* stream) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                        cu_seqlens, 64);
  if (st != FA_OK) return st;
  fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window, cu_seqlens);
  return fa::launch_fwd_f16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse, int B,
               int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
               const int32_t* cu_seqlens, void* stream) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                        cu_seqlens, 64);
  if (st != FA_OK) return st;
  fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window, cu_seqlens);
  return fa::launch_fwd_f32(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int T_q, int Hq, int d) {
  (void)d;
  if (T_q < 1 || Hq < 1) return 0;
  // D_i per (head, query row), fp32, rounded up to 256 bytes
  const size_t bytes = (size_t)T_q * (size_t)Hq * sizeof(float);
  return (bytes + 255) & ~(size_t)255;
}

int fa_fwd_bias(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                const float* bias, int64_t bias_stride_b, int64_t bias_stride_h,
                int64_t bias_stride_q, void* stream) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window, nullptr,
                        64);
  if (st != FA_OK) return st;
  st = check_bias(bias, bias_stride_b, bias_stride_h, bias_stride_q, Nk);
  if (st != FA_OK) return st;
  fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window, nullptr);
  p.bias = bias;
  p.bias_sb = bias_stride_b;
  p.bias_sh = bias_stride_h;
  p.bias_sq = bias_stride_q;
  return fa::launch_fwd_bf16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

static int bwd_impl(const void* q, const void* k, const void* v, const void* o,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                    int Nk, int d, float scale, int causal, int window,
                    const int32_t* cu_seqlens, const float* bias, int64_t sb, int64_t sh,
                    int64_t sq, int has_bias, void* stream, float dropout_p = 0.0f,
                    uint64_t seed = 0, bool f16 = false) {
  const void* t[] = {q, k, v, o, dout, dq, dk, dv, workspace};
  const float* s[] = {lse};
  int st = check_common(t, 9, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                        cu_seqlens, 64);
  if (st != FA_OK) return st;
  if (has_bias) {
    st = check_bias(bias, sb, sh, sq, Nk);
    if (st != FA_OK) return st;
  }
  uint32_t thresh = 0;
  float drop_scale = 1.0f;
  st = check_dropout(dropout_p, &thresh, &drop_scale);
  if (st != FA_OK) return st;
  // packed batches: T <= B * Nq (each sequence is at most Nq long)
  if (workspace_bytes < fa_bwd_workspace_size(B * Nq, Hq, d)) return FA_ERR_INVALID_ARG;
  fa::BwdParams p;
  p.dropout = dropout_p > 0.0f;
  p.drop_thresh = thresh;
  p.drop_scale = drop_scale;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  p.bias = has_bias ? bias : nullptr;
  p.bias_sb = sb;
  p.bias_sh = sh;
  p.bias_sq = sq;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.delta = static_cast<float*>(workspace);
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  const hipError_t e = f16 ? fa::launch_bwd_f16(p, (hipStream_t)stream)
                           : fa::launch_bwd_bf16(p, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
           const float* lse, void* dq, void* dk, void* dv, void* workspace,
           size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
           int causal, int window, const int32_t* cu_seqlens, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                  Nq, Nk, d, scale, causal, window, cu_seqlens, nullptr, 0, 0, 0, 0, stream);
}

int fa_bwd_f16(const void* q, const void* k, const void* v, const void* o, const void* dout,
               const float* lse, void* dq, void* dk, void* dv, void* workspace,
               size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
               float scale, int causal, int window, const int32_t* cu_seqlens, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                  Nq, Nk, d, scale, causal, window, cu_seqlens, nullptr, 0, 0, 0, 0, stream,
                  0.0f, 0, true);
}

int fa_bwd_bias(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, void* workspace,
                size_t workspace_bytes, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                float scale, int causal, int window, const float* bias,
                int64_t bias_stride_b, int64_t bias_stride_h, int64_t bias_stride_q,
                void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                  Nq, Nk, d, scale, causal, window, nullptr, bias, bias_stride_b,
                  bias_stride_h, bias_stride_q, 1, stream);
}

int fa_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                   int window, const int32_t* cu_seqlens, float dropout_p, uint64_t seed,
                   void* stream) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                        cu_seqlens, 64);
  if (st != FA_OK) return st;
  uint32_t thresh = 0;
  float drop_scale = 1.0f;
  st = check_dropout(dropout_p, &thresh, &drop_scale);
  if (st != FA_OK) return st;
  fa::FwdParams p = fwd_params(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                               window, cu_seqlens);
  p.dropout = dropout_p > 0.0f;  // p = 0 keeps every key: the plain kernel
  p.drop_thresh = thresh;
  p.drop_scale = drop_scale;
  p.seed_lo = (uint32_t)seed;
  p.seed_hi = (uint32_t)(seed >> 32);
  return fa::launch_fwd_bf16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_bwd_dropout(const void* q, const void* k, const void* v, const void* o,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   void* workspace, size_t workspace_bytes, int B, int Hq, int Hkv, int Nq,
                   int Nk, int d, float scale, int causal, int window,
                   const int32_t* cu_seqlens, float dropout_p, uint64_t seed, void* stream) {
  return bwd_impl(q, k, v, o, dout, lse, dq, dk, dv, workspace, workspace_bytes, B, Hq, Hkv,
                  Nq, Nk, d, scale, causal, window, cu_seqlens, nullptr, 0, 0, 0, 0, stream,
                  dropout_p, seed);
}

// Split-KV workspace: normalised partial outputs [num_splits][B][Nq][Hq][d]
// then partial LSEs [num_splits][B][Hq][Nq], both fp32, each part padded to
// 256 bytes.
static size_t decode_opart_bytes(int B, int Hq, int Nq, int d, int num_splits) {
  const size_t n = (size_t)num_splits * B * Nq * Hq * d * sizeof(float);
  return (n + 255) & ~(size_t)255;
}

size_t fa_decode_workspace_size(int B, int Hq, int Nq, int d, int num_splits) {
  if (B < 1 || Hq < 1 || Nq < 1 || d < 1 || num_splits < 1) return 0;
  const size_t l = (size_t)num_splits * B * Hq * Nq * sizeof(float);
  return decode_opart_bytes(B, Hq, Nq, d, num_splits) + ((l + 255) & ~(size_t)255);
}

int fa_decode_num_splits(int B, int Hq, int Hkv, int Nq, int Nk) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1 || Hq % Hkv != 0) return 0;
  // enough single-wave work-groups to keep every CU streaming (about six
  // per CU; measured best on 16 x 1..8K cached keys), without splitting
  // below ~256 keys per split
  const int64_t row_blocks = ((int64_t)(Hq / Hkv) * Nq + 31) / 32;
  const int64_t base = (int64_t)B * Hkv * row_blocks;
  int64_t s = (1536 + base - 1) / base;
  const int64_t cap = Nk / 256 > 1 ? Nk / 256 : 1;
  if (s > cap) s = cap;
  if (s > 128) s = 128;
  return (int)(s < 1 ? 1 : s);
}

}  // extern "C"

namespace {

// Checks and parameter block shared by fa_decode and fa_decode_noalloc;
// `workspace` may still be null here (the no-allocation entry point fills
// it in after the size check).
int decode_prepare(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
                   const int32_t* seqlens_k, int num_splits, fa::DecodeParams* p) {
  const void* t[] = {q, k, v, o};
  const float* s[] = {lse};
  int st = check_common(t, 4, s, 1, B, Hq, Hkv, Nq, Nk, d, scale, causal, window, nullptr, 64);
  if (st != FA_OK) return st;
  if (seqlens_k && !aligned(seqlens_k, 4)) return FA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > 1024) return FA_ERR_INVALID_ARG;
  const int64_t row_blocks = ((int64_t)(Hq / Hkv) * Nq + 31) / 32;
  if ((int64_t)num_splits * row_blocks * Hkv * B > (int64_t)UINT32_MAX / 2)
    return FA_ERR_UNSUPPORTED;
  p->q = q;
  p->k = k;
  p->v = v;
  p->o = o;
  p->lse = lse;
  p->seqlens_k = seqlens_k;
  p->opart = nullptr;
  p->lpart = nullptr;
  p->B = B;
  p->Hq = Hq;
  p->Hkv = Hkv;
  p->Nq = Nq;
  p->Nk = Nk;
  p->d = d;
  p->group = Hq / Hkv;
  p->causal = causal;
  p->window = window;
  p->scale = scale;
  p->scale_log2 = scale * 1.4426950408889634f;
  p->num_splits = num_splits;
  p->row_blocks = (int)row_blocks;
  return FA_OK;
}

// The split partials inside a workspace: opart first, lpart after it.
void decode_set_workspace(fa::DecodeParams* p, void* workspace) {
  p->opart = static_cast<float*>(workspace);
  p->lpart = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                      decode_opart_bytes(p->B, p->Hq, p->Nq, p->d,
                                                         p->num_splits));
}

}  // namespace

// ------------------------------------------------ allocation-free decode
// fa_decode_noalloc keeps its split partials in this fixed device array
// instead of a caller workspace.  Each GPU holds its own copy, at its own
// address, from the library's load until the process ends.  In host code
// `scratch` names a host-side stand-in, never the device memory: the device
// address of the copy on each GPU is looked up once, with that GPU current,
// and only that address is handed to kernels.
static __device__ __align__(256) unsigned char scratch[FA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on the current device (looked up on the
// first call per device).
int scratch_on_current_device(hipStream_t stream, void** addr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FA_ERR_UNSUPPORTED;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice(stream, &sdev) != hipSuccess) return FA_ERR_HIP;
    if (sdev != dev) return FA_ERR_INVALID_ARG;  // the copy looked up must be the stream's
  }
  void* a = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (!a) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    a = g_scratch_addr[dev].load(std::memory_order_relaxed);
    if (!a) {
      if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return FA_ERR_HIP;
      g_scratch_addr[dev].store(a, std::memory_order_release);
    }
  }
  *addr = a;
  return FA_OK;
}

}  // namespace

extern "C" {

int fa_decode(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
              int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
              const int32_t* seqlens_k, int num_splits, void* workspace,
              size_t workspace_bytes, void* stream) {
  fa::DecodeParams p;
  int st = decode_prepare(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                          seqlens_k, num_splits, &p);
  if (st != FA_OK) return st;
  if (!workspace || !aligned(workspace, 16)) return FA_ERR_INVALID_ARG;
  if (workspace_bytes < fa_decode_workspace_size(B, Hq, Nq, d, num_splits))
    return FA_ERR_INVALID_ARG;
  decode_set_workspace(&p, workspace);
  return fa::launch_decode_bf16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_decode_noalloc_max_splits(int B, int Hq, int Nq, int d) {
  if (B < 1 || Hq < 1 || Nq < 1 || d < 1) return 0;
  int lo = 0;
  for (int s = 1; s <= 1024; ++s) {
    if (fa_decode_workspace_size(B, Hq, Nq, d, s) > (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES)
      break;
    lo = s;
  }
  return lo;
}

int fa_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                      int window, const int32_t* seqlens_k, int num_splits, void* stream) {
  if (num_splits == 0) {  // the default count, lowered until the partials fit
    num_splits = fa_decode_num_splits(B, Hq, Hkv, Nq, Nk);
    const int cap = fa_decode_noalloc_max_splits(B, Hq, Nq, d);
    if (num_splits > cap) num_splits = cap;
    if (num_splits < 1) return FA_ERR_TOO_LARGE;
  }
  fa::DecodeParams p;
  int st = decode_prepare(q, k, v, o, lse, B, Hq, Hkv, Nq, Nk, d, scale, causal, window,
                          seqlens_k, num_splits, &p);
  if (st != FA_OK) return st;
  if (fa_decode_workspace_size(B, Hq, Nq, d, num_splits) >
      (size_t)FA_DECODE_NOALLOC_SCRATCH_BYTES)
    return FA_ERR_TOO_LARGE;
  void* addr = nullptr;
  st = scratch_on_current_device((hipStream_t)stream, &addr);
  if (st != FA_OK) return st;
  decode_set_workspace(&p, addr);
  return fa::launch_decode_bf16(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_quantize_fp8(const void* x, void* x8, float* scales, int B, int N, int H, int d,
                    int transpose, const float* signs, void* stream) {
  if (!x || !x8 || !scales || !aligned(x, 16) || !aligned(x8, 16) || !aligned(scales, 4))
    return FA_ERR_INVALID_ARG;
  if (signs && !aligned(signs, 4)) return FA_ERR_INVALID_ARG;
  if (B < 1 || N < 1 || H < 1 || d < 1 || (transpose != 0 && transpose != 1))
    return FA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  const int64_t nb = ((int64_t)N + 63) / 64;
  if ((int64_t)B * H * nb > (int64_t)INT32_MAX) return FA_ERR_UNSUPPORTED;
  fa::QuantParams p;
  p.x = x;
  p.x8 = static_cast<uint8_t*>(x8);
  p.scales = scales;
  p.signs = signs;
  p.B = B;
  p.N = N;
  p.H = H;
  p.d = d;
  p.transpose = transpose;
  p.ldn = (int)(nb * 64);
  p.nb = (int)nb;
  return fa::launch_quantize_fp8(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

int fa_fwd_fp8(const void* q8, const void* k8, const void* vt8, const float* q_scale,
               const float* k_scale, const float* v_scale, void* o, float* lse, int B, int Hq,
               int Hkv, int Nq, int Nk, int d, float scale, int causal, int window,
               void* stream) {
  const void* t[] = {q8, k8, vt8, o};
  const float* s[] = {lse, q_scale, k_scale, v_scale};
  int st = check_common(t, 4, s, 4, B, Hq, Hkv, Nq, Nk, d, scale, causal, window, nullptr, 64);
  if (st != FA_OK) return st;
  const int64_t ldv = ((int64_t)Nk + 63) / 64 * 64;
  // the V^T tile's buffer descriptor spans d - 1 rows of ldv bytes plus one tile row
  if ((int64_t)(d - 1) * ldv + 64 >= ((int64_t)1 << 32)) return FA_ERR_UNSUPPORTED;
  fa::Fp8FwdParams p;
  p.q = static_cast<const uint8_t*>(q8);
  p.k = static_cast<const uint8_t*>(k8);
  p.v = static_cast<const uint8_t*>(vt8);
  p.sq = q_scale;
  p.sk = k_scale;
  p.sv = v_scale;
  p.o = o;
  p.lse = lse;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.d = d;
  p.group = Hq / Hkv;
  p.causal = causal;
  p.window = window;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.num_qtiles = 0;
  p.ldv = (int)ldv;
  p.nbq = (Nq + 63) / 64;
  p.nbk = (Nk + 63) / 64;
  return fa::launch_fwd_fp8(p, (hipStream_t)stream) == hipSuccess ? FA_OK : FA_ERR_HIP;
}

const char* fa_status_string(int status) {
  switch (status) {
    case FA_OK:
      return "FA_OK";
    case FA_ERR_INVALID_ARG:
      return "FA_ERR_INVALID_ARG: invalid argument";
    case FA_ERR_UNSUPPORTED:
      return "FA_ERR_UNSUPPORTED: unsupported configuration";
    case FA_ERR_HIP:
      return "FA_ERR_HIP: HIP runtime error";
    case FA_ERR_TOO_LARGE:
      return "FA_ERR_TOO_LARGE: the request needs more scratch than the library's static "
             "buffer holds (FA_DECODE_NOALLOC_SCRATCH_BYTES per device)";
    default:
      return "unknown fa_status";
  }
}

}  // extern "C"

// Host/device parameter blocks and the internal launcher interface between
// the C-ABI layer (fa_api.hip) and the kernel files.  Not part of the public
// ABI: the public header is include/fa_mi355x.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

// One forward call, already validated.  Offsets are computed in the kernels
// from the token-major layouts documented in the public header.
struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;  // nullptr for dense batches
  int B, Hq, Hkv, Nq, Nk, d;
  int group;                  // Hq / Hkv
  int causal, window;
  float scale;                // multiplier of Q K^T
  float scale_log2;           // scale * log2(e): exp(x*scale) = exp2(x*scale_log2)
  int num_qtiles;             // ceil(Nq / query-tile rows) of the kernel
  int xcd_groups;             // > 1: each XCD runs the longest query tiles of its
                              // xcd_groups KV-head groups first (set by the launcher)
  // additive bias of dense batches, nullptr when there is none: element
  // (b, h, i, j) at bias[b*bias_sb + h*bias_sh + i*bias_sq + j]
  const float* bias;
  int64_t bias_sb, bias_sh, bias_sq;
  // dropout on the probabilities: element (b, h, i, j) is kept iff its 16-bit
  // slot of Philox4x32-10 (drop_call in fa_device.h), key (seed_lo,
  // seed_hi), is >= drop_thresh; kept values are multiplied by drop_scale
  int dropout;                // 0: no dropout (the other fields are unused)
  uint32_t drop_thresh;       // floor(p * 2^16)
  uint32_t seed_lo, seed_hi;
  float drop_scale;
};

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  void* dq;
  void* dk;
  void* dv;
  float* delta;               // workspace: D_i = sum_c dO_ic O_ic, LSE layout
  const int32_t* cu_seqlens;
  int B, Hq, Hkv, Nq, Nk, d;
  int group;
  int causal, window;
  float scale;
  float scale_log2;
  const float* bias;          // as in FwdParams
  int64_t bias_sb, bias_sh, bias_sq;
  int dropout;                // as in FwdParams
  uint32_t drop_thresh;
  uint32_t seed_lo, seed_hi;
  float drop_scale;
};

// One split-KV call (few query rows per sequence over a long key cache),
// already validated.  opart/lpart live in the caller's workspace.
struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seqlens_k;   // keys used per sequence, or nullptr (all Nk)
  float* opart;               // [num_splits][B][Nq][Hq][d] fp32, normalised partial O
  float* lpart;               // [num_splits][B][Hq][Nq] fp32, partial LSE (natural log)
  int B, Hq, Hkv, Nq, Nk, d;
  int group;                  // Hq / Hkv
  int causal, window;
  float scale;
  float scale_log2;
  int num_splits;             // key-range splits per (sequence, KV head, row block)
  int row_blocks;             // ceil(group * Nq / 32)
};

// One FP8 forward call (dense batches), already validated.  Codes are OCP
// E4M3 bytes; every block of 64 tokens of one head has one fp32 scale.
struct Fp8FwdParams {
  const uint8_t* q;           // [B, Nq, Hq, d]
  const uint8_t* k;           // [B, Nk, Hkv, d]
  const uint8_t* v;           // V transposed: [B, Hkv, d, ldv], keys innermost
  const float* sq;            // [B, Hq, nbq]
  const float* sk;            // [B, Hkv, nbk]
  const float* sv;            // [B, Hkv, nbk]
  void* o;                    // bf16 [B, Nq, Hq, d]
  float* lse;                 // [B, Hq, Nq]
  int B, Hq, Hkv, Nq, Nk, d;
  int group;
  int causal, window;
  float scale_log2;           // scale * log2(e)
  int num_qtiles;             // set by the launcher
  int ldv;                    // keys per V^T row: Nk rounded up to 64
  int nbq, nbk;               // scale blocks per head: ceil(Nq / 64), ceil(Nk / 64)
};

// One block quantization call (bf16 -> E4M3 codes and block scales).
struct QuantParams {
  const void* x;              // bf16 [B, N, H, d]
  uint8_t* x8;                // [B, N, H, d], or [B, H, d, ldn] when transposed
  float* scales;              // [B, H, nb]
  const float* signs;         // d values of +-1 (rotation), or nullptr
  int B, N, H, d;
  int transpose;              // write the V^T layout
  int ldn;                    // N rounded up to 64 (row length of the V^T layout)
  int nb;                     // ceil(N / 64)
};

// Launchers: enqueue on `stream`, return hipGetLastError() of the launch.
hipError_t launch_fwd_bf16(const FwdParams& p, hipStream_t stream);
hipError_t launch_fwd_f16(const FwdParams& p, hipStream_t stream);
// d = 128 forward without a bias (bf16 or fp16): fa_fwd_bf16_d128.hip
hipError_t launch_fwd_d128(const FwdParams& p, hipStream_t stream, bool f16);
hipError_t launch_fwd_f32(const FwdParams& p, hipStream_t stream);
hipError_t launch_bwd_bf16(const BwdParams& p, hipStream_t stream);
hipError_t launch_bwd_f16(const BwdParams& p, hipStream_t stream);  // plain only
hipError_t launch_decode_bf16(const DecodeParams& p, hipStream_t stream);
hipError_t launch_fwd_fp8(const Fp8FwdParams& p, hipStream_t stream);
hipError_t launch_quantize_fp8(const QuantParams& p, hipStream_t stream);

}  // namespace fa

// fa_validate.h -- host-side argument checks of the C ABI (pure C++, no HIP).
//
// Every entry point validates all of its arguments here before anything is
// launched, so an invalid call returns a status and enqueues nothing.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/fa.h"

namespace fa {

struct Problem {
  long B, Hq, Hkv, N, d;
  int causal;
  int varlen;
};

// Limits of this implementation.
constexpr long kMaxItems = 1L << 24;        // query tiles x heads x sequences per launch
constexpr long kMaxTokens = 1L << 31;       // tokens per tensor (B * N, or T)
// K/V row elements (Hkv * d): the d = 128 forward addresses 256 key tiles of a
// head from one buffer descriptor, whose offsets must stay below 2^31 bytes.
constexpr long kMaxKvRow = 1L << 15;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Sizes, head configuration and flags shared by forward and backward.
inline fa_status check_problem(const Problem& pr, float scale) {
  if (pr.B < 0 || pr.N < 0 || pr.Hq <= 0 || pr.Hkv <= 0 || pr.d <= 0) return FA_ERR_INVALID_ARGUMENT;
  if (pr.Hq % pr.Hkv != 0) return FA_ERR_INVALID_ARGUMENT;
  if (pr.causal != 0 && pr.causal != 1) return FA_ERR_INVALID_ARGUMENT;
  // finite and >= 0: the kernels take row maxima of the raw scores Q K^T and fold
  // the scale into the exponent argument, which is exact only for scale >= 0
  if (!(scale >= 0.0f) || scale > 3.0e38f) return FA_ERR_INVALID_ARGUMENT;
  if (pr.d != 64 && pr.d != 128) return FA_ERR_UNSUPPORTED;
  if (pr.B * pr.N > kMaxTokens) return FA_ERR_UNSUPPORTED;
  if (pr.Hkv * pr.d > kMaxKvRow) return FA_ERR_UNSUPPORTED;
  const long tiles = (pr.N + 127) / 128;
  if (pr.B * pr.Hq * tiles > kMaxItems) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

inline bool empty_problem(const Problem& pr) { return pr.B == 0 || pr.N == 0; }

// Forward options (NULL = defaults); `hw_exp_only` for the kernels built with
// v_exp_f32 alone (the 8-bit and split-KV variants).
inline fa_status check_options(const fa_fwd_options* opt, bool hw_exp_only = false) {
  if (!opt) return FA_OK;
  if (opt->exp_mode != FA_EXP_HW && opt->exp_mode != FA_EXP_POLY) return FA_ERR_INVALID_ARGUMENT;
  if (!(opt->rescale_tau >= 0.f && opt->rescale_tau <= 64.f)) return FA_ERR_INVALID_ARGUMENT;
  if (opt->lpt_order != 0 && opt->lpt_order != 1) return FA_ERR_INVALID_ARGUMENT;
  if (hw_exp_only && opt->exp_mode != FA_EXP_HW) return FA_ERR_UNSUPPORTED;
  return FA_OK;
}

inline fa_status check_fwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const Problem& pr, float scale, const int32_t* cu_seqlens,
                           const fa_fwd_options* opt) {
  fa_status st = check_problem(pr, scale);
  if (st != FA_OK) return st;
  st = check_options(opt);
  if (st != FA_OK) return st;
  if (empty_problem(pr)) return FA_OK;
  if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse))
    return FA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !aligned4(cu_seqlens)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

inline fa_status check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                           const void* dout, const void* dq, const void* dk, const void* dv,
                           const Problem& pr, float scale, const int32_t* cu_seqlens,
                           const void* workspace, size_t workspace_bytes, size_t needed) {
  fa_status st = check_problem(pr, scale);
  if (st != FA_OK) return st;
  if (empty_problem(pr)) return FA_OK;
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned4(lse) ||
      !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return FA_ERR_INVALID_ARGUMENT;
  if (cu_seqlens && !aligned4(cu_seqlens)) return FA_ERR_INVALID_ARGUMENT;
  if (needed > 0) {
    if (!workspace || workspace_bytes < needed) return FA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return FA_ERR_INVALID_ARGUMENT;
  }
  return FA_OK;
}

inline fa_status check_fp8(const void* q, const void* k, const void* v, const float* qd, const float* kd,
                           const void* o, const float* lse, const Problem& pr, float scale,
                           const int32_t* cu_seqlens, const fa_fwd_options* opt) {
  fa_status st = check_fwd(q, k, v, o, lse, pr, scale, cu_seqlens, nullptr);
  if (st != FA_OK) return st;
  st = check_options(opt, true);
  if (st != FA_OK) return st;
  if (pr.d != 128) return FA_ERR_UNSUPPORTED;
  if (empty_problem(pr)) return FA_OK;
  if (!qd || !kd || !aligned4(qd) || !aligned4(kd)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

constexpr long kMaxSplits = 1024;

inline fa_status check_split(const void* q, const void* k, const void* v, const float* o_part,
                             const float* lse_part, long B, long Hq, long Hkv, long Nq, long Nk, long d,
                             int causal, float scale, long n_splits, const fa_fwd_options* opt) {
  if (n_splits < 1 || n_splits > kMaxSplits) return FA_ERR_INVALID_ARGUMENT;
  if (Nk < 0 || Nq < 0) return FA_ERR_INVALID_ARGUMENT;
  if (causal == 1 && Nq > Nk) return FA_ERR_INVALID_ARGUMENT;
  const Problem pr{B, Hq, Hkv, Nq > Nk ? Nq : Nk, d, causal, 0};
  fa_status st = check_problem(pr, scale);
  if (st != FA_OK) return st;
  st = check_options(opt, true);
  if (st != FA_OK) return st;
  if (B * Hq * ((Nq + 127) / 128) * n_splits > kMaxItems) return FA_ERR_UNSUPPORTED;
  if (B * n_splits * Nq * Hq * d > (1L << 40)) return FA_ERR_UNSUPPORTED;
  if (B == 0 || Nq == 0) return FA_OK;
  if (!q || !k || !v || !o_part || !lse_part) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o_part) || !aligned4(lse_part))
    return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

inline fa_status check_merge(const float* o_part, const float* lse_part, const void* o, const float* lse,
                             long n_parts, long B, long H, long N, long d) {
  if (n_parts < 1 || n_parts > kMaxSplits || B < 0 || H <= 0 || N < 0 || d <= 0) return FA_ERR_INVALID_ARGUMENT;
  if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
  if (B * N * H > kMaxTokens) return FA_ERR_UNSUPPORTED;
  if (B == 0 || N == 0) return FA_OK;
  if (!o_part || !lse_part || !o || !lse) return FA_ERR_INVALID_ARGUMENT;
  if (!aligned16(o_part) || !aligned16(o) || !aligned4(lse_part) || !aligned4(lse)) return FA_ERR_INVALID_ARGUMENT;
  return FA_OK;
}

}  // namespace fa

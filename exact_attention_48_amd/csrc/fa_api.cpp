// fa_api.cpp -- the C ABI (include/fa.h): validate, pick the kernel variant, launch.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/fa.h"
#include "fa_exp2.h"
#include "fa_kernels.h"
#include "fa_validate.h"

namespace {

constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kDefaultTau = 32.0f;

// The exponent scale c = softmax_scale * log2(e) of the forward kernels. A zero
// scale (uniform attention over the visible keys) becomes the smallest normal
// float: masked scores are -inf, and -inf * 0 would give NaN where -inf * c
// gives the -inf that exp2 turns into 0; every finite score times c is then
// below 2^-24 in magnitude for |S| < 2^102, so exp2 of it rounds to 1.
inline float fwd_scale_log2(float softmax_scale) {
  const float c = softmax_scale * kLog2eF;
  return c > 0.f ? c : 1.17549435e-38f;
}

inline size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

namespace fa {

// Workspace layout: D_i | LSE_i * log2(e) (each laid out like the LSE) | for
// packed batches, the dK/dV schedule (8 x (B + 1) int32 at most).
size_t bwd_lse_bytes(long B, long Hq, long N) {
  const size_t rows = (size_t)B * (size_t)N;          // >= T for packed batches
  return round256(rows * (size_t)Hq * sizeof(float));
}

size_t bwd_workspace_bytes(long B, long Hq, long Hkv, long N, int d, int causal, int varlen) {
  (void)Hkv;
  (void)causal;
  (void)d;
  if (B <= 0 || N <= 0 || Hq <= 0) return 0;
  const size_t sched = varlen ? round256((size_t)8 * (size_t)(B + 1) * sizeof(int)) : 0;
  return 2 * bwd_lse_bytes(B, Hq, N) + sched;
}

// Work is dealt to the 8 XCDs by (K/V head, tile residue): with 8 / gcd(Hkv, 8)
// residues every XCD gets the same share of every sequence.
int xcd_chunks(int Hkv) {
  int g = 8;
  while (Hkv % g) g >>= 1;                             // gcd(Hkv, 8)
  return 8 / g;
}

// The backward's workspace for callers that cannot allocate (fa_bwd_noalloc):
// a fixed device array, one copy per GPU, held until the process ends. In host
// code `scratch` names a host-side stand-in, never the device memory: its
// device address comes from hipGetSymbolAddress, once per device, with that
// device current.
constexpr size_t kScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

// Device address of the current device's scratch array, or nullptr on error.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

}  // namespace fa

extern "C" {

const char* fa_status_string(fa_status s) {
  switch (s) {
    case FA_OK: return "FA_OK: success";
    case FA_ERR_INVALID_ARGUMENT: return "FA_ERR_INVALID_ARGUMENT: invalid argument";
    case FA_ERR_UNSUPPORTED: return "FA_ERR_UNSUPPORTED: valid but not supported (head size or problem size)";
    case FA_ERR_WORKSPACE: return "FA_ERR_WORKSPACE: backward workspace missing or too small";
    case FA_ERR_HIP: return "FA_ERR_HIP: HIP runtime error at launch";
  }
  return "unknown fa_status";
}

const char* fa_version(void) { return "fa-mi355x 0.1 (gfx950)"; }

fa_status fa_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                    const int32_t* cu_seqlens, const fa_fwd_options* options, void* stream) {
  const fa::Problem pr{B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr};
  fa_status st = fa::check_fwd(q, k, v, o, lse, pr, softmax_scale, cu_seqlens, options);
  if (st != FA_OK) return st;
  if (fa::empty_problem(pr)) return FA_OK;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.N = N;
  p.lpt = options ? options->lpt_order : 1;
  p.kv_chunks = fa::xcd_chunks(Hkv);
  p.scale_log2 = fwd_scale_log2(softmax_scale);
  p.tau = options ? options->rescale_tau : kDefaultTau;
  const int expmode = options ? options->exp_mode : FA_EXP_HW;
  hipError_t e = fa::fwd_launch(p, d, causal, cu_seqlens != nullptr, expmode, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                 const int32_t* cu_seqlens, void* stream) {
  return fa_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens, nullptr, stream);
}

namespace {

fa_status fwd_fp8_common(const void* q, const void* k, const void* v, const float* q_descale,
                         const float* k_descale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                         int causal, float softmax_scale, const int32_t* cu_seqlens,
                         const fa_fwd_options* options, bool blockscale, void* stream) {
  const fa::Problem pr{B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr};
  fa_status st = fa::check_fp8(q, k, v, q_descale, k_descale, o, lse, pr, softmax_scale, cu_seqlens, options);
  if (st != FA_OK) return st;
  const long nb = ((long)N + fa::kFp8Block - 1) / fa::kFp8Block;
  if (blockscale && nb > fa::kFp8MaxBlocks) return FA_ERR_UNSUPPORTED;
  if (fa::empty_problem(pr)) return FA_OK;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.N = N;
  p.lpt = options ? options->lpt_order : 1;
  p.kv_chunks = fa::xcd_chunks(Hkv);
  p.scale_log2 = fwd_scale_log2(softmax_scale);
  p.tau = options ? options->rescale_tau : kDefaultTau;
  p.q_descale = q_descale;
  p.k_descale = k_descale;
  p.fp8_nb = blockscale ? (int)nb : 1;
  hipError_t e = fa::fwd_fp8_launch(p, causal, cu_seqlens != nullptr, blockscale, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

}  // namespace

fa_status fa_fwd_fp8_ex(const void* q, const void* k, const void* v, const float* q_descale,
                        const float* k_descale, void* o, float* lse, int B, int Hq, int Hkv, int N, int d,
                        int causal, float softmax_scale, const int32_t* cu_seqlens,
                        const fa_fwd_options* options, void* stream) {
  return fwd_fp8_common(q, k, v, q_descale, k_descale, o, lse, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens,
                        options, false, stream);
}

fa_status fa_fwd_fp8_blockscale(const void* q, const void* k, const void* v, const float* q_descale,
                                const float* k_descale, void* o, float* lse, int B, int Hq, int Hkv, int N,
                                int d, int causal, float softmax_scale, const int32_t* cu_seqlens,
                                const fa_fwd_options* options, void* stream) {
  static_assert(FA_FP8_SCALE_BLOCK == fa::kFp8Block && FA_FP8_MAX_BLOCKS == fa::kFp8MaxBlocks,
                "the header's block constants must match the kernel's");
  return fwd_fp8_common(q, k, v, q_descale, k_descale, o, lse, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens,
                        options, true, stream);
}

fa_status fa_fwd_fp8(const void* q, const void* k, const void* v, const float* q_descale, const float* k_descale,
                     void* o, float* lse, int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                     const int32_t* cu_seqlens, void* stream) {
  return fa_fwd_fp8_ex(q, k, v, q_descale, k_descale, o, lse, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens,
                       nullptr, stream);
}

fa_status fa_fwd_split_ex(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                          int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale,
                          int n_splits, const fa_fwd_options* options, void* stream) {
  fa_status st = fa::check_split(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale,
                                 n_splits, options);
  if (st != FA_OK) return st;
  if (B == 0 || Nq == 0) return FA_OK;
  fa::FwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.N = Nq;
  p.lpt = options ? options->lpt_order : 1;
  p.kv_chunks = fa::xcd_chunks(Hkv);
  p.scale_log2 = fwd_scale_log2(softmax_scale);
  p.tau = options ? options->rescale_tau : kDefaultTau;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.Nk = Nk;
  p.q_off = Nk - Nq;
  p.n_splits = n_splits;
  p.chunk = (Nk + n_splits - 1) / n_splits;
  hipError_t e = fa::fwd_split_launch(p, d, causal, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_fwd_split(const void* q, const void* k, const void* v, float* o_part, float* lse_part,
                       int B, int Hq, int Hkv, int Nq, int Nk, int d, int causal, float softmax_scale,
                       int n_splits, void* stream) {
  return fa_fwd_split_ex(q, k, v, o_part, lse_part, B, Hq, Hkv, Nq, Nk, d, causal, softmax_scale, n_splits,
                         nullptr, stream);
}

fa_status fa_merge(const float* o_part, const float* lse_part, void* o, float* lse, int n_parts, int B, int H,
                   int N, int d, void* stream) {
  fa_status st = fa::check_merge(o_part, lse_part, o, lse, n_parts, B, H, N, d);
  if (st != FA_OK) return st;
  if (B == 0 || N == 0) return FA_OK;
  hipError_t e = fa::merge_launch(o_part, lse_part, o, lse, n_parts, B, H, N, d, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_exp2_eval(const float* x, float* y, int64_t n, int exp_mode, void* stream) {
  if (n < 0 || (exp_mode != FA_EXP_HW && exp_mode != FA_EXP_POLY)) return FA_ERR_INVALID_ARGUMENT;
  if (n == 0) return FA_OK;
  if (!x || !y || !fa::aligned4(x) || !fa::aligned4(y)) return FA_ERR_INVALID_ARGUMENT;
  hipError_t e = fa::exp2_eval_launch(x, y, (long)n, exp_mode, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

size_t fa_bwd_workspace_size(int B, int Hq, int Hkv, int N, int d, int causal, int varlen) {
  return fa::bwd_workspace_bytes(B, Hq, Hkv, N, d, causal, varlen);
}

fa_status fa_bwd_ex(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv,
                    int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                    const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, int stages,
                    void* stream) {
  if (stages < 1 || stages > FA_BWD_ALL) return FA_ERR_INVALID_ARGUMENT;
  const fa::Problem pr{B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr};
  const size_t needed = fa::bwd_workspace_bytes(B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr);
  fa_status st = fa::check_bwd(q, k, v, o, lse, dout, dq, dk, dv, pr, softmax_scale, cu_seqlens,
                               workspace, workspace_bytes, needed);
  if (st != FA_OK) return st;
  if (fa::empty_problem(pr)) return FA_OK;
  fa::BwdParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.dout = dout;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  p.cu_seqlens = cu_seqlens;
  const size_t half = fa::bwd_lse_bytes(B, Hq, N);
  p.dsum = (float*)workspace;
  p.lse2 = (float*)((char*)workspace + half);
  p.kt_prefix = cu_seqlens ? (int*)((char*)workspace + 2 * half) : nullptr;
  p.kv_chunks = fa::xcd_chunks(Hkv);
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.N = N;
  p.scale = softmax_scale;
  p.scale_log2 = softmax_scale * kLog2eF;
  hipError_t e = fa::bwd_launch(p, d, causal, cu_seqlens != nullptr, stages, (hipStream_t)stream);
  return e == hipSuccess ? FA_OK : FA_ERR_HIP;
}

fa_status fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 const void* dout, void* dq, void* dk, void* dv,
                 int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                 const int32_t* cu_seqlens, void* workspace, size_t workspace_bytes, void* stream) {
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens,
                   workspace, workspace_bytes, FA_BWD_ALL, stream);
}

size_t fa_bwd_noalloc_max_workspace(void) { return fa::kScratchBytes; }

fa_status fa_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                         const void* dout, void* dq, void* dk, void* dv,
                         int B, int Hq, int Hkv, int N, int d, int causal, float softmax_scale,
                         const int32_t* cu_seqlens, void* stream) {
  const fa::Problem pr{B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr};
  // every argument is checked before any HIP call (the workspace is ours: needed = 0 skips its check)
  fa_status st = fa::check_bwd(q, k, v, o, lse, dout, dq, dk, dv, pr, softmax_scale, cu_seqlens, nullptr, 0, 0);
  if (st != FA_OK) return st;
  if (fa::empty_problem(pr)) return FA_OK;
  const size_t needed = fa::bwd_workspace_bytes(B, Hq, Hkv, N, d, causal, cu_seqlens != nullptr);
  if (needed > fa::kScratchBytes) return FA_ERR_WORKSPACE;
  void* ws = fa::scratch_ptr();
  if (!ws) return FA_ERR_HIP;
  return fa_bwd_ex(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, N, d, causal, softmax_scale, cu_seqlens, ws,
                   fa::kScratchBytes, FA_BWD_ALL, stream);
}

}  // extern "C"

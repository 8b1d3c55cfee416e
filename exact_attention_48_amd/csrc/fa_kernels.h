// fa_kernels.h -- internal interface between the host dispatch and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* cu_seqlens;   // nullptr for uniform batches
  int B, Hq, Hkv, G, N;
  int n_qtiles;                // query tiles per sequence (set by fwd_launch)
  int kv_chunks;               // query-tile residues per (sequence, K/V head): 8 / gcd(Hkv, 8)
  int lpt;                     // 1: heaviest query tiles first
  float scale_log2;            // softmax_scale * log2(e)
  float tau;                   // conditional rescale threshold (log2 units)
  // split-KV partial results (fwd_split_launch); N is then the number of queries
  float* o_part;               // fp32 [n_splits, B, N, Hq, d]
  float* lse_part;             // fp32 [n_splits, B, Hq, N]
  int Nk;                      // keys per sequence
  int q_off;                   // Nk - N: key position of query 0
  int n_splits;
  int chunk;                   // keys per chunk, ceil(Nk / n_splits)
  // 8-bit Q/K (fwd_fp8_launch): q and k hold E4M3 codes, dequantised by these
  const float* q_descale;      // [B, Hq], or [B, Hq, fp8_nb] with block descales
  const float* k_descale;      // [B, Hkv], or [B, Hkv, fp8_nb]
  int fp8_nb;                  // block descales: blocks per (sequence, head), ceil(N / kFp8Block)
};

constexpr int kFp8Block = 64;        // tokens per descale block (local positions 64 j .. 64 j + 63)
constexpr int kFp8MaxBlocks = 4096;  // block descales: at most this many blocks per (sequence, head)

hipError_t fwd_launch(FwdParams p, int d, int causal, int varlen, int expmode, hipStream_t stream);
hipError_t fwd_pp_launch(FwdParams p, int causal, int varlen, int expmode, hipStream_t stream);
hipError_t fwd_pp_split_launch(FwdParams p, int causal, hipStream_t stream);
hipError_t fwd_split_launch(FwdParams p, int d, int causal, hipStream_t stream);
hipError_t fwd_fp8_launch(FwdParams p, int causal, int varlen, bool blockscale, hipStream_t stream);
hipError_t merge_launch(const float* o_part, const float* lse_part, void* o, float* lse, int n_parts, int B,
                        int H, int N, int d, hipStream_t stream);

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_seqlens;
  float* dsum;                 // workspace: -D_i = -rowsum(dO * O), laid out like LSE
  float* lse2;                 // workspace: LSE_i * log2(e), laid out like LSE
  int* kt_prefix;              // workspace (packed batches): dK/dV schedule, see bwd_sched_kernel
  int kv_chunks;               // tile residues per (sequence, K/V head): 8 / gcd(Hkv, 8)
  int B, Hq, Hkv, G, N;
  float scale;
  float scale_log2;
};

hipError_t bwd_launch(BwdParams p, int d, int causal, int varlen, int stages, hipStream_t stream);
size_t bwd_workspace_bytes(long B, long Hq, long Hkv, long N, int d, int causal, int varlen);
size_t bwd_lse_bytes(long B, long Hq, long N);
int xcd_chunks(int Hkv);

}  // namespace fa

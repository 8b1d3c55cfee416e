// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// One workgroup computes BM = 256 query rows of one (sequence, query head)
// with 4 waves, one per SIMD, each owning 64 queries as two 32-query MFMA
// blocks. The loop walks the key/value tiles of BN = 32 keys (tiling with an
// online softmax, so the N x N score matrix never leaves the chip:
// "FlashAttention-4 Conquers Asymmetric GPU Hardware Scaling", podcast.app
// episode page, second paragraph of the description).
//
// Per key/value tile j and wave (query block qb = 0, 1):
//   S^T[32 x 32] = K_j[32 x d] * Q_qb^T[d x 32]   bf16 MFMA 32x32x16, fp32 acc
//     -> every lane holds the scores of ONE query for 16 of the tile's keys,
//        so a row max is an in-lane max plus one v_permlane32_swap
//   masking only on tiles that cross the causal diagonal or the sequence end
//   conditional rescaling: each row's max m stays at its first tile's max,
//     so O and l always share one m and no pass ever rescales O; the loop
//     takes no further maxima. A row sum l above 2^tau (log2 units) at the
//     end -- the only way a later score can have outgrown m far enough to
//     threaten fp32 -- sends the workgroup through a pass that records the
//     true row maxima and a last pass with them (the threshold-gated rescale
//     of the pages, daily.dev "Summary" and the FA4 abstract on the
//     zhuanzhiai.com page, with the test moved out of the loop)
//   P = exp2(S c - m c), c = scale * log2(e), hardware v_exp_f32 or the
//     FMA-pipe polynomial (software exponential: daily.dev "Summary")
//   l += rowsum(P) (per-lane partial sums, combined once at the end)
//   O^T[d x 32] += V_j^T[d x 32] * P^T[32 x 32]  bf16 MFMA; P stays in
//     registers as the B operand; V^T comes from row-major V in LDS through
//     the transposing ds_read_b64_tr_b16
// Every K and V^T fragment read from LDS feeds both query blocks, which
// halves the LDS traffic per MFMA against one block per wave. Q fragments
// and the O accumulators sit in the accumulation registers.
//
// Software pipeline (the MMA/softmax overlap of the pages' pipeline, daily.dev
// "Summary"), iteration j of a wave, one MFMA stream:
//   phase A : S of tile j+1 (16 MFMAs), interleaved with exps of tile j
//             (the rest of query block 0 and part of block 1);
//   phase B1: O_0 += V_j P_0 (8 MFMAs), with the other exps of block 1;
//   phase B2: O_1 += V_j P_1 (8 MFMAs), with the masking of tile j+1 (its S
//             is done by then) and its first exps.
//
// K and V tiles travel HBM -> LDS with buffer_load ... lds (no register
// staging) through a 4-deep ring of distinct LDS objects, issued two
// iterations ahead; one workgroup barrier per iteration, without the memory
// fence of __syncthreads (that would drain the copies still in flight). The
// buffer form (rather than the flat global_load_lds) lets the compiler count
// outstanding LDS reads separately from the copies, so a fragment read waits
// only for itself.
//
// Work order: query tiles are ordered heaviest first (causal: the last tiles
// of a sequence see the most keys) -- longest-processing-time-first (daily.dev
// "Summary") -- and the G query heads of one K/V head are kept on one XCD
// (workgroups are dealt to the 8 XCDs round-robin) so they share its L2.
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_order.h"
#include "fa_tiles.h"

namespace fa {

using namespace tiles;

namespace {

constexpr int WQ = 64;               // queries per wave
constexpr int BM = NWAVES * WQ;      // queries per workgroup
constexpr int BN = 32;               // keys per K/V tile

// One ring stage: a K tile (bf16, or 8-bit when K8) and a bf16 V tile.
template <int D, bool K8>
struct FwdStage {
  static constexpr int ROWB = D * 2;
  static constexpr int KTILEB = BN * (K8 ? D : ROWB);
  static constexpr int VOFF = KTILEB;               // V tile offset
  static constexpr int BYTES = KTILEB + BN * ROWB;
  static constexpr int OROWB = ROWB + 16;           // output staging pitch
  static_assert(32 * OROWB <= BYTES, "32 rows of a wave's output staging must fit in one stage");
};

}  // namespace

// SPLIT: partial results over one key chunk per work item (split-KV), written
// as fp32 O_p and LSE_p; uniform batches only.
// FP8: Q and K as OCP E4M3 codes with per-(sequence, head) descales; S^T by the
// 32x32x64 8-bit MFMA (64 of the contraction per instruction), V and P bf16.
// BLK (with FP8): one descale per 64-token block of each (sequence, head)
// instead. The exp2 factor then differs per tile and per query block, so the
// row maxima are kept in scaled units (S c) rather than raw scores.
template <int D, bool CAUSAL, bool VARLEN, int EXPMODE, bool SPLIT, bool FP8, bool BLK = false>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void fa_fwd_kernel(const FwdParams p) {
  static_assert(!(SPLIT && VARLEN), "split-KV partial results are for uniform batches");
  static_assert(!(SPLIT && FP8) && (!FP8 || D == 128), "8-bit Q/K: plain forward, d = 128");
  static_assert(!BLK || FP8, "block descales are for 8-bit inputs");
  using S = FwdStage<D, FP8>;
  using RCK = RowCopy<FP8 ? D / 2 : D, BN>;         // an 8-bit row of D bytes copies like a bf16 row of D / 2
  using RCV = RowCopy<D, BN>;
  constexpr int KSTEPS = FP8 ? D / 64 : D / 16;      // S^T k-steps
  constexpr int DBLK = D / 32;
  constexpr int OPS = RCK::PER_WAVE + RCV::PER_WAVE; // copy instructions per tile and wave
  using AFrag = std::conditional_t<FP8, i32x8, bf16x8>;
  __shared__ __attribute__((aligned(1024))) char s0_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s1_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s2_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s3_raw[S::BYTES];
  // stage j (a compile-time constant wherever it is used; an array of LDS
  // pointers can end up in global memory, which the linker cannot resolve)
  auto stage = [&](int j) __attribute__((always_inline)) -> char FA_LDS* {
    switch (j) {
      case 0: return (char FA_LDS*)s0_raw;
      case 1: return (char FA_LDS*)s1_raw;
      case 2: return (char FA_LDS*)s2_raw;
      default: return (char FA_LDS*)s3_raw;
    }
  };

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  // ---- work item -> (sequence s, query head h, query tile qt), in the order
  // fa_order.h describes; a split call's items are (sequence, chunk sp) pairs
  // in place of sequences ----
  TileItem item;
  if constexpr (VARLEN) {
    if (!q_item_xcd(blockIdx.x, p.B, p.Hkv, p.G, p.kv_chunks, p.n_qtiles, p.lpt, item)) return;
  } else {
    if (!q_item_level(blockIdx.x, SPLIT ? p.B * p.n_splits : p.B, p.Hq, p.G, p.n_qtiles, p.lpt, item)) return;
  }
  const int s = SPLIT ? item.s / p.n_splits : item.s;
  const int sp = SPLIT ? item.s - s * p.n_splits : 0;
  const int h = item.h, qt = item.t;
  const int hkv = h / p.G;

  int seq0, L, kseq0, Lk;                           // queries: rows seq0.., L of them; keys: kseq0.., Lk
  if constexpr (VARLEN) {
    seq0 = p.cu_seqlens[s];
    L = p.cu_seqlens[s + 1] - seq0;
    kseq0 = seq0;
    Lk = L;
  } else {
    seq0 = s * p.N;
    L = p.N;
    kseq0 = SPLIT ? s * p.Nk : seq0;
    Lk = SPLIT ? p.Nk : L;
  }
  // keys of this work item: [kb, ke), the chunk of a split call; query i sits
  // at key position i + q_off for the causal mask
  const int q_off = SPLIT ? p.q_off : 0;
  const int kb = SPLIT ? min(sp * p.chunk, Lk) : 0;
  const int ke = SPLIT ? (int)min((long)(sp + 1) * p.chunk, (long)Lk) : Lk;
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int qw0 = q0 + wave * WQ;                   // first query of this wave
  int my_q[2];
  my_q[0] = qw0 + l32;
  my_q[1] = qw0 + 32 + l32;

  const long q_row_stride = (long)p.Hq * D;         // elements
  const long kv_stride = (long)p.Hkv * D * 2;       // bytes per token row of V (and of bf16 K)
  const long k_stride = FP8 ? (long)p.Hkv * D : kv_stride;
  const char* kbase = (const char*)p.k + ((long)kseq0 * p.Hkv + hkv) * D * (FP8 ? 1 : 2);
  const char* vbase = (const char*)p.v + ((long)kseq0 * p.Hkv + hkv) * D * 2;
  const int kv_end = CAUSAL ? min(ke, q0 + BM + q_off) : ke;   // keys this workgroup can see
  const int n_it = kv_end > kb ? (kv_end - kb + BN - 1) / BN : 0;

  // ---- Q fragments (B operands of S^T = K Q^T): lane holds queries my_q[qb];
  // bf16: elements 16 ks + 8 hl .. + 7; 8-bit: bytes 64 ks + 32 hl .. + 31 ----
  AFrag qf[2][KSTEPS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = my_q[qb] < L ? my_q[qb] : L - 1;
    if constexpr (FP8) {
      const char* qp = (const char*)p.q + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 32;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const i32x4 lo = *(const i32x4*)(qp + ks * 64);
        const i32x4 hi = *(const i32x4*)(qp + ks * 64 + 16);
        qf[qb][ks] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
    } else {
      const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) qf[qb][ks] = *(const bf16x8*)(qp + ks * 16);
    }
  }

  RCK kcopy;
  RCV vcopy;
  kcopy.init(wave, lane, (unsigned)k_stride);
  vcopy.init(wave, lane, (unsigned)kv_stride);
  // tile copies in order: the next tile starts at key kb + iss * BN, whose
  // K and V rows are at kcur and vcur
  int iss = 0;
  const char* kcur = kbase;
  const char* vcur = vbase;
  auto restart_copies = [&]() __attribute__((always_inline)) {
    iss = 0;
    kcur = kbase + (long)kb * k_stride;
    vcur = vbase + (long)kb * kv_stride;
  };
  auto issue_next = [&](char FA_LDS* stage) __attribute__((always_inline)) {
    const int r0 = kb + iss * BN;
    if (r0 + BN <= ke) {
      kcopy.issue_full(stage, kcur);
      vcopy.issue_full(stage + S::VOFF, vcur);
    } else {
      kcopy.issue_tail(stage, kcur, k_stride, ke - 1 - r0);
      vcopy.issue_tail(stage + S::VOFF, vcur, kv_stride, ke - 1 - r0);
    }
    kcur += BN * k_stride;
    vcur += BN * kv_stride;
    ++iss;
  };

  TileOffsets<D> to;
  to.init(lane);
  TileOffsetsK8 to8;
  if constexpr (FP8) to8.init(lane);
  // exp2 argument scale: softmax_scale * log2(e), times the Q and K descales of
  // this (sequence, head) for 8-bit inputs
  float c = p.scale_log2;
  if constexpr (FP8 && !BLK) c = c * p.q_descale[(long)s * p.Hq + h] * p.k_descale[(long)s * p.Hkv + hkv];
  // Block descales: the K descales of this (sequence, K/V head) go to LDS once
  // (kd_lds[j] for keys 64 j ..); each query block's Q descale folds into c_q.
  // The exp2 factor of a tile is ct = c_q * kd (at least the smallest normal
  // float, so that a masked -inf score never meets a zero factor).
  __shared__ float kd_lds[BLK ? kFp8MaxBlocks : 1];
  float c_q[2] = {c, c};
  int kd_last = 0;                           // last K block of the sequence
  if constexpr (BLK) {
    const int nbk = min((Lk + kFp8Block - 1) / kFp8Block, p.fp8_nb);   // (host: fp8_nb <= kFp8MaxBlocks)
    kd_last = nbk - 1;
    const float* kdp = p.k_descale + ((long)s * p.Hkv + hkv) * p.fp8_nb;
    for (int i = threadIdx.x; i < nbk; i += NTHREADS) kd_lds[i] = kdp[i];
    const float* qdp = p.q_descale + ((long)s * p.Hq + h) * p.fp8_nb;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int qr = my_q[qb] < L ? my_q[qb] : L - 1;
      c_q[qb] = c * qdp[min(qr / kFp8Block, p.fp8_nb - 1)];
    }
    __syncthreads();
  }
  auto kd_of = [&](int k0) __attribute__((always_inline)) -> float {   // K descale of the tile at key k0
    if constexpr (BLK) return kd_lds[min(k0 / kFp8Block, kd_last)];
    else return 1.f;
  };
  auto set_factor = [&](float kd, float (&ct)[2]) __attribute__((always_inline)) {
    if constexpr (BLK) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) ct[qb] = fmaxf(c_q[qb] * kd, 1.17549435e-38f);
    }
  };
  float ctA[2] = {c, c}, ctB[2] = {c, c};    // exp2 factor of the tile whose S^T is in sA / sB
  const float tau = p.tau;
  f32x16 oacc[2][DBLK];
  float m_run[2];                            // the max O and l are relative to (fixed in a pass)
  float mc[2];                               // m_run * c (0 for a row without a visible key yet)
  float l_run[2];                            // partial row sums over this lane's keys
  float m_seen[2];                           // true running max of the scores
  bool over[2];                              // some tile's max exceeded m_run by more than tau
  f32x16 sA[2], sB[2];                       // S^T of two consecutive tiles, per query block
  u32x4 pb[2][2];                            // P^T (bf16 pairs) of the current tile [qb][key step]

  // S^T MFMA j: k-step j / 2, query block j % 2; the K fragment of a k-step is
  // read once for both blocks.
  constexpr int NA = 2 * KSTEPS;
  auto a_frag = [&](const char FA_LDS* tile, int ks) __attribute__((always_inline)) -> AFrag {
    if constexpr (FP8) return to8.operand(tile, ks);
    else return to.row_operand(tile, ks, 0);
  };
  auto a_step = [&](f32x16 (&sx)[2], int j, const AFrag& a) __attribute__((always_inline)) {
    const int ks = j >> 1, qb = j & 1;
    if constexpr (FP8) {
      if (ks == 0) mfma8_v_first(sx[qb], a, qf[qb][ks]);
      else mfma8_v(sx[qb], a, qf[qb][ks]);
    } else {
      if (ks == 0) mfma_v_first(sx[qb], a, qf[qb][ks]);
      else mfma_v(sx[qb], a, qf[qb][ks]);
    }
  };
  // K fragments read ahead in phase A (at most one per k-step)
  constexpr int PFA = PF < KSTEPS ? PF : KSTEPS;
  // V^T fragment f: key step t = f / DBLK, d-block db = f % DBLK (both query blocks)
  constexpr int NV = 2 * DBLK;
  auto v_frag = [&](const char FA_LDS* tile, int f) __attribute__((always_inline)) {
    return to.tr_operand(tile + S::VOFF, f / DBLK, f % DBLK);
  };

  // ---- softmax pieces ----
  // exp element (qb, r) of the current tile (S^T in sc): key 8(r/4) + 4 hl + r%4
  // of the tile, query my_q[qb]
  // The 32 exp elements of a tile, u = 16 qb + r, run as a three-stage
  // software pipeline so that no instruction of a slot waits on another one
  // of the same slot: step t does x_t = S c - m c, p_{t-1} = exp2(x_{t-1}),
  // and l += p_{t-2} (packing the bf16 pair when t-2 is odd).
  float xq[3], pq[3];
  auto exp_step = [&](const f32x16 (&sc)[2], int t, const float (&ct)[2]) __attribute__((always_inline)) {
    if (t < 32) {
      const int qb = t >> 4, r = t & 15;
      xq[t % 3] = __builtin_fmaf(sc[qb][r], BLK ? ct[qb] : c, -mc[qb]);
    }
    if (t >= 1 && t <= 32) pq[(t - 1) % 3] = exp2_sel<EXPMODE>(xq[(t - 1) % 3]);
    if (t >= 2 && t <= 33) {
      const int u = t - 2, qb = u >> 4, r = u & 15;
      l_run[qb] += pq[u % 3];
      asm volatile("" : "+v"(l_run[qb]));   // keep the add in its slot (not sunk past the mask branch)
      if (r & 1) pb[qb][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(unsigned, pack_bf16(pq[(u - 1) % 3], pq[u % 3]));
    }
  };
  // Masking of a tile (keys k0..): dead scores -> -inf.
  auto mask_tile = [&](f32x16 (&sx)[2], int k0) __attribute__((always_inline)) {
    asm volatile("; masking");   // keeps the caller's branch a branch (no if-conversion)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const bool dead = (key >= ke) || (CAUSAL && key > my_q[qb] + q_off);
        if (dead) sx[qb][r] = -INFINITY;
      }
  };
  auto needs_mask = [&](int k0) __attribute__((always_inline)) {
    return (k0 + BN > ke) || (CAUSAL && k0 + BN - 1 > qw0 + q_off);
  };
  float mpart[2];
  auto max_half = [&](const f32x16 (&sx)[2], int qb, int half) __attribute__((always_inline)) {
    const int r = 8 * half;
    const float a = vmax3(sx[qb][r], sx[qb][r + 1], sx[qb][r + 2]);
    const float b = vmax3(sx[qb][r + 3], sx[qb][r + 4], sx[qb][r + 5]);
    const float m = vmax3(a, b, sx[qb][r + 6]);
    if (half == 0) mpart[qb] = vmax(m, sx[qb][r + 7]);
    else mpart[qb] = vmax3(mpart[qb], m, sx[qb][r + 7]);
  };
  auto decide = [&](int qb, const float (&ct)[2]) __attribute__((always_inline)) {
    const float mx = pair_max(mpart[qb]);
    if constexpr (BLK) {                     // scaled units: m_run and m_seen are maxima of S ct
      const float mxs = mx * ct[qb];
      m_seen[qb] = vmax(m_seen[qb], mxs);
      over[qb] = over[qb] || (mxs - m_run[qb] > tau);    // false when both are -inf
    } else {
      m_seen[qb] = vmax(m_seen[qb], mx);
      over[qb] = over[qb] || ((mx - m_run[qb]) * c > tau);   // false when both are -inf
    }
  };
  // ---- one iteration's MFMA stream ----
  // The 34 exp pipeline steps of a tile are spread over three phases:
  //   phase B2 of the previous iteration: steps 0..KB2-1, right after the
  //             tile's masking (its S^T is complete by then);
  //   phase A : steps KB2..KB2+UA-1 beside the S^T MFMAs of the next tile
  //             (P of query block 0 is complete after step 17);
  //   phase B1: the rest, beside O_0 += V^T P_0 (P of block 1 complete
  //             after step 33, before phase B2 needs it).
  // Row maxima of every tile are taken only in a tracking pass (see below).
  constexpr int KB2 = 12;
  constexpr int UA = 16;
  constexpr int UB = 34 - KB2 - UA;
  static_assert(KB2 + UA >= 18 && UB >= 0, "P of query block 0 must be complete before phase B1");
  constexpr int VPRE = (PFA < NV) ? PFA : NV;       // V^T fragments read during phase A
  auto stream = [&](const char FA_LDS* nt, const char FA_LDS* ct, f32x16 (&sx)[2], const f32x16 (&sc)[2],
                    float (&fx)[2], const float (&fc)[2], int k_next, bool issue, char FA_LDS* issue_stage,
                    bool track) __attribute__((always_inline)) {
    const float kd_next = kd_of(k_next);            // read early; used in phase B2
    AFrag qa[PFA];
#pragma unroll
    for (int i = 0; i < PFA; ++i) qa[i] = a_frag(nt, i);
    if (issue) issue_next(issue_stage);
    __builtin_amdgcn_sched_barrier(0);
    bf16x8 vf[NV];                                  // V^T fragments, kept for both query blocks
    // phase A: S^T of the next tile; fragment ks feeds MFMAs 2 ks and 2 ks + 1
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      const AFrag a = qa[ks % PFA];
      if (ks + PFA < KSTEPS) qa[ks % PFA] = a_frag(nt, ks + PFA);
      else if (ks + PFA - KSTEPS < VPRE) vf[ks + PFA - KSTEPS] = v_frag(ct, ks + PFA - KSTEPS);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = 2 * ks + x;
        a_step(sx, j, a);
#pragma unroll
        for (int t = KB2 + UA * j / NA; t < KB2 + UA * (j + 1) / NA; ++t) exp_step(sc, t, fc);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // phase B1: O_0 += V^T P_0, with the remaining exps of block 1
    asm volatile("s_nop 2");                        // VALU-written B operands -> MFMA
#pragma unroll
    for (int f = 0; f < NV; ++f) {
      if (f + VPRE < NV) vf[f + VPRE] = v_frag(ct, f + VPRE);
      mfma_a(oacc[0][f % DBLK], vf[f], __builtin_bit_cast(bf16x8, pb[0][f / DBLK]));
#pragma unroll
      for (int t = KB2 + UA + UB * f / NV; t < KB2 + UA + UB * (f + 1) / NV; ++t) exp_step(sc, t, fc);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase B2: O_1 += V^T P_1, with the next tile's masking (and, in a
    // tracking pass, its maxima) and its first exp steps. On the last
    // iteration the next tile lies past every visible key, so the masking
    // turns all of its scores into -inf and its steps add nothing.
    asm volatile("s_nop 2");
    const bool mask_next = needs_mask(k_next);
#pragma unroll
    for (int f = 0; f < NV; ++f) {
      mfma_a(oacc[1][f % DBLK], vf[f], __builtin_bit_cast(bf16x8, pb[1][f / DBLK]));
      if (f == 0 && mask_next) mask_tile(sx, k_next);
      if (f == 0) set_factor(kd_next, fx);
      if (f == 1 && track) {
        max_half(sx, 0, 0);
        max_half(sx, 0, 1);
        max_half(sx, 1, 0);
        max_half(sx, 1, 1);
        decide(0, fx);
        decide(1, fx);
      }
#pragma unroll
      for (int t = KB2 * f / NV; t < KB2 * (f + 1) / NV; ++t) exp_step(sx, t, fx);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Iteration i (BI = i % NSTAGE): tile i in stage BI (its S^T in the array of
  // parity i), tile i+1 in stage BI+1; tile i+3 is copied into stage BI+3 (last
  // read as tile i-1, before this iteration's barrier). The S^T MFMAs of tile
  // i+1 also run on the last iteration (stale LDS, results unused).
  auto iter = [&](auto bi_tag, const int i, const bool track) __attribute__((always_inline)) {
    constexpr int BI = decltype(bi_tag)::value;
    if (i + 2 < n_it) wait_vm(OPS);
    else if (i + 1 < n_it) wait_vm(0);
    barrier_no_fence();
    const bool issue = i + 3 < n_it;
    char FA_LDS* const nst = stage((BI + 3) % NSTAGE);
    const int k_next = kb + (i + 1) * BN;
    if constexpr (BI % 2 == 0) stream(stage((BI + 1) % NSTAGE), stage(BI), sB, sA, ctB, ctA, k_next, issue, nst, track);
    else stream(stage((BI + 1) % NSTAGE), stage(BI), sA, sB, ctA, ctB, k_next, issue, nst, track);
  };

  // Rescaling, taken out of the loop. In the first pass each row's max m is
  // fixed at its first tile's max, and O and l share it, so the pass is exact
  // whatever the later scores are, as long as nothing overflows. Every P is
  // at most the row sum l, so a row sum of at most 2^tau (tau in log2 units)
  // bounds every P, and with it O, far inside fp32. A row above that (or not
  // finite) sends the workgroup through a tracking pass that records each
  // row's true max, and then a last pass with that max, where every P <= 1.
  __shared__ int over_flag[NWAVES];
  bool run = true;
  if constexpr (SPLIT) {
    if (n_it == 0) {                  // the chunk holds no key any query of the workgroup sees
      run = false;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int i = 0; i < DBLK; ++i) oacc[qb][i] = f32x16{};
        l_run[qb] = 0.f;
        m_run[qb] = -INFINITY;
      }
    }
  }
  const float l_limit = exp2f(tau);
  for (int pass = 0; run; ++pass) {
    const bool track = pass == 1;
    restart_copies();
    issue_next(stage(0));
    if (n_it > 1) issue_next(stage(1));
    if (n_it > 2) issue_next(stage(2));
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int i = 0; i < DBLK; ++i) oacc[qb][i] = f32x16{};
      l_run[qb] = 0.f;
      m_run[qb] = pass == 2 ? m_seen[qb] : -INFINITY;
      m_seen[qb] = -INFINITY;
      over[qb] = false;
    }

    // ---- prologue: tile 0 in, S^T of tile 0, its maxima and first exp steps ----
    if (n_it > 2) wait_vm(2 * OPS);
    else if (n_it > 1) wait_vm(OPS);
    else wait_vm(0);
    barrier_no_fence();
    {
      AFrag qa[PFA];
#pragma unroll
      for (int i = 0; i < PFA; ++i) qa[i] = a_frag(stage(0), i);
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const AFrag a = qa[ks % PFA];
        if (ks + PFA < KSTEPS) qa[ks % PFA] = a_frag(stage(0), ks + PFA);
        a_step(sA, 2 * ks, a);
        a_step(sA, 2 * ks + 1, a);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    mfma_result_wait();
    if (needs_mask(kb)) mask_tile(sA, kb);
    set_factor(kd_of(kb), ctA);
    max_half(sA, 0, 0);
    max_half(sA, 0, 1);
    max_half(sA, 1, 0);
    max_half(sA, 1, 1);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float mx = BLK ? pair_max(mpart[qb]) * ctA[qb] : pair_max(mpart[qb]);
      m_seen[qb] = mx;
      if (pass < 2) m_run[qb] = mx;
      mc[qb] = m_run[qb] == -INFINITY ? 0.f : (BLK ? m_run[qb] : m_run[qb] * c);
    }
#pragma unroll
    for (int t = 0; t < KB2; ++t) exp_step(sA, t, ctA);

    for (int i = 0; i < n_it; i += NSTAGE) {
      iter(ic<0>{}, i, track);
      if (i + 1 < n_it) iter(ic<1>{}, i + 1, track);
      if (i + 2 < n_it) iter(ic<2>{}, i + 2, track);
      if (i + 3 < n_it) iter(ic<3>{}, i + 3, track);
    }
#pragma unroll
    for (int x = 0; x < 2; ++x) {
      keep_live(sA[x]);
      keep_live(sB[x]);
    }
    mfma_result_wait();
    if (pass == 2) break;
    if (pass == 0) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) over[qb] = !(pair_sum(l_run[qb]) <= l_limit);
    } else {
      over[0] = true;                 // after the tracking pass, the exact pass
    }
    // all copies have landed (the last iterations wait for them); LDS is free
    // once every wave is past this point
    const bool any = wave_any(over[0] || over[1]);
    if (lane == 0) over_flag[wave] = any ? 1 : 0;
    __syncthreads();
    const bool again = over_flag[0] | over_flag[1] | over_flag[2] | over_flag[3];
    __syncthreads();
    if (!again) break;
  }

  // ---- epilogue: O = O / l, LSE = m * scale + ln(l) ----
  if constexpr (SPLIT) {
    // fp32 O_p rows straight from the accumulators; rows that saw no key of
    // the chunk hold O_p = 0, LSE_p = -inf
    const long part = (long)sp * p.B + s;
    float* ob = p.o_part + (part * p.N * p.Hq + h) * D;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = pair_sum(l_run[qb]);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      store_rows_f32<D>(oacc[qb], inv, ob, q_row_stride, qw0 + 32 * qb, L, lane);
      if (hl == 0 && my_q[qb] < L) {
        const float lse = (m_run[qb] == -INFINITY || l_tot == 0.f) ? -INFINITY
                                                                  : (m_run[qb] * c + __log2f(l_tot)) * kLn2;
        p.lse_part[(part * p.Hq + h) * p.N + my_q[qb]] = lse;
      }
    }
    return;
  }
  barrier_no_fence();
  char FA_LDS* st = stage(0);
  if (wave == 1) st = stage(1);
  if (wave == 2) st = stage(2);
  if (wave == 3) st = stage(3);
  __bf16* obase = (__bf16*)p.o + ((long)seq0 * p.Hq + h) * D;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qb == 1) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    store_rows_bf16<D>(st, oacc[qb], inv, obase, q_row_stride, qw0 + 32 * qb, L, lane);
    if (hl == 0 && my_q[qb] < L) {
      const float lse = (m_run[qb] == -INFINITY) ? -INFINITY
                                                 : ((BLK ? m_run[qb] : m_run[qb] * c) + __log2f(l_tot)) * kLn2;
      long li;
      if constexpr (VARLEN) li = (long)h * p.cu_seqlens[p.B] + seq0 + my_q[qb];
      else li = ((long)s * p.Hq + h) * p.N + my_q[qb];
      p.lse[li] = lse;
    }
  }
}

// ---- instantiations and launcher ----

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_fwd(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, EXPMODE, false, false>), dim3(grid), dim3(NTHREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <int D, bool CAUSAL>
static hipError_t launch_split(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, false, 0, true, false>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
}

template <bool CAUSAL, bool VARLEN, bool BLK>
static hipError_t launch_fp8(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<128, CAUSAL, VARLEN, 0, false, true, BLK>), dim3(grid), dim3(NTHREADS), 0,
                     stream, p);
  return hipGetLastError();
}

template <bool CAUSAL, bool VARLEN>
static hipError_t launch_fp8_b(const FwdParams& p, int grid, bool blk, hipStream_t stream) {
  return blk ? launch_fp8<CAUSAL, VARLEN, true>(p, grid, stream) : launch_fp8<CAUSAL, VARLEN, false>(p, grid, stream);
}

template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_fwd_e(const FwdParams& p, int grid, int expmode, hipStream_t stream) {
  return expmode == 1 ? launch_fwd<D, CAUSAL, VARLEN, 1>(p, grid, stream)
                      : launch_fwd<D, CAUSAL, VARLEN, 0>(p, grid, stream);
}

template <int D>
static hipError_t launch_fwd_d(const FwdParams& p, int grid, int causal, int varlen, int expmode,
                               hipStream_t stream) {
  if (causal) return varlen ? launch_fwd_e<D, true, true>(p, grid, expmode, stream)
                            : launch_fwd_e<D, true, false>(p, grid, expmode, stream);
  return varlen ? launch_fwd_e<D, false, true>(p, grid, expmode, stream)
                : launch_fwd_e<D, false, false>(p, grid, expmode, stream);
}

hipError_t fwd_launch(FwdParams p, int d, int causal, int varlen, int expmode, hipStream_t stream) {
  if (d == 128) return fwd_pp_launch(p, causal, varlen, expmode, stream);   // two waves per SIMD (fa_fwd_pp.hip)
  p.n_qtiles = (p.N + BM - 1) / BM;
  const long grid_l = varlen ? q_grid_xcd(p.B, p.Hkv, p.G, p.kv_chunks, p.n_qtiles)
                             : q_grid_level(p.B, p.Hq, p.G, p.n_qtiles);
  if (grid_l == 0) return hipSuccess;
  if (grid_l > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int grid = (int)grid_l;
  if (d == 128) return launch_fwd_d<128>(p, grid, causal, varlen, expmode, stream);
  return launch_fwd_d<64>(p, grid, causal, varlen, expmode, stream);
}

hipError_t fwd_split_launch(FwdParams p, int d, int causal, hipStream_t stream) {
  if (d == 128) return fwd_pp_split_launch(p, causal, stream);   // two waves per SIMD (fa_fwd_pp.hip)
  p.n_qtiles = (p.N + BM - 1) / BM;
  const long grid_l = q_grid_level(p.B * p.n_splits, p.Hq, p.G, p.n_qtiles);
  if (grid_l == 0) return hipSuccess;
  if (grid_l > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int grid = (int)grid_l;
  if (d == 128) return causal ? launch_split<128, true>(p, grid, stream) : launch_split<128, false>(p, grid, stream);
  return causal ? launch_split<64, true>(p, grid, stream) : launch_split<64, false>(p, grid, stream);
}

hipError_t fwd_fp8_launch(FwdParams p, int causal, int varlen, bool blockscale, hipStream_t stream) {
  p.n_qtiles = (p.N + BM - 1) / BM;
  const long grid_l = varlen ? q_grid_xcd(p.B, p.Hkv, p.G, p.kv_chunks, p.n_qtiles)
                             : q_grid_level(p.B, p.Hq, p.G, p.n_qtiles);
  if (grid_l == 0) return hipSuccess;
  if (grid_l > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int grid = (int)grid_l;
  if (causal) return varlen ? launch_fp8_b<true, true>(p, grid, blockscale, stream)
                            : launch_fp8_b<true, false>(p, grid, blockscale, stream);
  return varlen ? launch_fp8_b<false, true>(p, grid, blockscale, stream)
                : launch_fp8_b<false, false>(p, grid, blockscale, stream);
}

}  // namespace fa

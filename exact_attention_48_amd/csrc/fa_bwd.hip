// fa_bwd.hip -- exact attention backward for gfx950 (MI355X).
//
// The backward pass recomputes the softmax from the forward's log-sum-exp and
// produces dQ, dK and dV (backward pass: abstract on the zhuanzhiai.com page;
// there the pages lean on tensor memory and 2-CTA MMA, which this hardware
// lacks, so that fewer bytes cross shared memory and fewer atomics run). With
// P = exp(S - LSE) and D_i = dO_i . O_i:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, all on the caller's stream:
//   1. bwd_prep_kernel: -D_i = -rowsum(dO o O) and LSE_i * log2(e), fp32, into
//      the workspace (HBM-bound, one pass; -D seeds the dP accumulators of
//      kernel 2, so dP - D costs no instruction); for packed batches also
//      bwd_sched_kernel, the order in which kernel 2 takes its work.
//   2. bwd_dkdv_kernel: one workgroup per (sequence, K/V head, 128-key tile),
//      one wave per SIMD. Each wave keeps 32 keys' K and V fragments and their
//      dK/dV accumulators in registers and streams the 64-row Q / dO tiles of
//      every query head of the group, so the group's dK/dV sum needs no
//      atomics. Per tile and wave: S = Q K^T and dP = dO V^T with the key in
//      the lane (C layout), P and dS in bf16, dV^T += dO^T P and dK^T += Q^T dS
//      with the transposed Q / dO operands read by ds_read_b64_tr_b16.
//   3. bwd_dq_kernel: one workgroup per (sequence, query head, 128-query tile),
//      one wave per SIMD: S^T = K Q^T and dP^T = V dO^T with the query in the
//      lane, then dQ^T += K^T dS^T (K^T through ds_read_b64_tr_b16).
// dQ is produced by this separate pass rather than by fp32 atomic adds from
// kernel 2: on this GPU those run at about one 4-byte add per L2 channel and
// clock, which for long sequences costs more than recomputing S and dP.
//
// Both main kernels are software-pipelined the same way. Tiles stream
// HBM -> LDS (global_load_lds_dwordx4, no register staging) through a ring of
// NSTAGE = 4 distinct LDS objects, issued two iterations ahead; one workgroup
// barrier per iteration (without the memory fence of __syncthreads, which
// would drain the copies in flight). Iteration i of a wave runs
//   phase A: the MFMAs of S, dP for tile i+1, slot by slot interleaved with the
//            softmax VALU work of tile i (its S, dP came from phase A of the
//            previous iteration), so the matrix core and the VALU overlap;
//   phase B: the MFMAs that consume tile i's P and dS (dV, dK or dQ), their
//            transposed operands read a few MFMAs ahead.
// Masking code runs only for tiles that cross the causal diagonal or the end
// of a sequence.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_order.h"
#include "fa_tiles.h"

namespace fa {

using namespace tiles;

namespace {

constexpr int TROWS = 64;     // rows per streamed tile (Q/dO or K/V)
constexpr int KV_BN = 128;    // keys per dK/dV workgroup (32 per wave)

__device__ __forceinline__ long lse_index(const BwdParams& p, int s, int h, int seq0, int row, int T, bool varlen) {
  return varlen ? (long)h * T + seq0 + row : ((long)s * p.Hq + h) * p.N + row;
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO[i,k] O[i,k]  and  LSE_i * log2(e)
// ---------------------------------------------------------------------------
// Block b takes query head b % Hq and the PREP_TOK consecutive tokens
// (b / Hq) * PREP_TOK .. of the flattened (uniform: b * N + n) or packed token
// axis. A row (token, head) of dO / O is D * 2 contiguous bytes, D / 8 lanes
// load 16 bytes each, and every thread keeps the loads of all its rows in
// flight; the block's LSE reads and D writes are then runs of consecutive
// tokens of one head, contiguous within a sequence in the [B, Hq, N] / [Hq, T]
// layout. Consecutive blocks take the heads of one token run, so the rows
// they read lie side by side.
constexpr int PREP_TOK = 64;
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_prep_kernel(const BwdParams p, long n_tok) {
  constexpr int LPR = D / 8;                 // lanes per (token, head) row, 16 B each
  constexpr int RPP = 256 / LPR;             // rows per pass of the block
  constexpr int PASSES = PREP_TOK / RPP;
  static_assert(PASSES * RPP == PREP_TOK, "token run must split into whole passes");
  const int h = (int)(blockIdx.x % (unsigned)p.Hq);
  const long t0 = (long)(blockIdx.x / (unsigned)p.Hq) * PREP_TOK;
  long T = n_tok;
  if constexpr (VARLEN) T = p.cu_seqlens[p.B];
  if (t0 >= T) return;
  const int part = threadIdx.x % LPR;
  const int sub = threadIdx.x / LPR;
  bf16x8 a[PASSES], b[PASSES];
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    const long t = t0 + u * RPP + sub;
    if (t < T) {
      const long off = (t * p.Hq + h) * D + part * 8;
      a[u] = *(const bf16x8*)((const __bf16*)p.dout + off);
      b[u] = *(const bf16x8*)((const __bf16*)p.o + off);
    } else {
      a[u] = bf16x8{};
      b[u] = bf16x8{};
    }
  }
#pragma unroll
  for (int u = 0; u < PASSES; ++u) {
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[u][e], (float)b[u][e], acc);
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
    const long t = t0 + u * RPP + sub;
    if (t < T && part == 0) {
      long idx;
      if constexpr (VARLEN) idx = (long)h * T + t;
      else {
        const long bt = t / p.N, n = t - bt * p.N;
        idx = (bt * p.Hq + h) * p.N + n;
      }
      p.dsum[idx] = -acc;
      p.lse2[idx] = p.lse[idx] * kLog2e;
    }
  }
}

// Schedule of the dK/dV kernel for packed batches: with c = 8 / gcd(Hkv, 8) and
// n_kt(s) the 128-key tiles of sequence s, kt_prefix[i * (B + 1) + s] counts the
// key tiles kt < n_kt(s') with kt = i (mod c) over the sequences s' < s (i < c).
// One workgroup; thread t scans a contiguous run of sequences.
__global__ __launch_bounds__(256) void bwd_sched_kernel(const int32_t* cu, int B, int c, int* out) {
  __shared__ int part[256];
  const int t = threadIdx.x;
  const int per = (B + 255) / 256;
  const int s0 = min(B, t * per), s1 = min(B, s0 + per);
  auto count = [&](int s, int i) {
    const int nkt = (cu[s + 1] - cu[s] + KV_BN - 1) / KV_BN;
    return nkt > i ? (nkt - i + c - 1) / c : 0;
  };
  for (int i = 0; i < c; ++i) {
    int sum = 0;
    for (int s = s0; s < s1; ++s) sum += count(s, i);
    part[t] = sum;
    __syncthreads();
    if (t == 0) {
      int run = 0;
      for (int k = 0; k < 256; ++k) {
        const int x = part[k];
        part[k] = run;
        run += x;
      }
      out[i * (B + 1) + B] = run;
    }
    __syncthreads();
    int run = part[t];
    for (int s = s0; s < s1; ++s) {
      out[i * (B + 1) + s] = run;
      run += count(s, i);
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: KV-major
// ---------------------------------------------------------------------------
template <int D>
struct KvStage {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = TROWS * ROWB;          // one Q or dO tile
  static constexpr int LSEOFF = 2 * TILEB;            // 64 x LSE*log2(e), then 64 x D
  static constexpr int BYTES = 2 * TILEB + 2 * TROWS * 4;
  static constexpr int OROWB = ROWB + 16;             // output staging pitch
  static_assert(32 * OROWB <= BYTES, "a wave's output staging must fit in one stage");
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdParams p) {
  using S = KvStage<D>;
  using RC = RowCopy<D, TROWS>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int ROWB = S::ROWB;
  constexpr int OPS = 1 + 2 * RC::PER_WAVE;          // copy instructions per tile and wave
  __shared__ __attribute__((aligned(1024))) char s0_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s1_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s2_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s3_raw[S::BYTES];
  char FA_LDS* const stg[NSTAGE] = {(char FA_LDS*)s0_raw, (char FA_LDS*)s1_raw, (char FA_LDS*)s2_raw,
                                    (char FA_LDS*)s3_raw};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  // ---- work item -> (sequence s, K/V head hkv, key tile kt), in the order
  // fa_order.h describes ----
  TileItem item;
  if constexpr (VARLEN) {
    if (!kv_item_xcd(blockIdx.x, p.B, p.Hkv, p.kv_chunks, (p.N + KV_BN - 1) / KV_BN, p.kt_prefix, item)) return;
  } else {
    if (!kv_item_level(blockIdx.x, p.B, p.Hkv, (p.N + KV_BN - 1) / KV_BN, item)) return;
  }
  const int s = item.s, hkv = item.h, kt = item.t;

  int seq0, L, T = 0;
  if constexpr (VARLEN) {
    seq0 = p.cu_seqlens[s];
    L = p.cu_seqlens[s + 1] - seq0;
    T = p.cu_seqlens[p.B];
  } else {
    seq0 = s * p.N;
    L = p.N;
  }
  const int kv0 = kt * KV_BN;
  if (kv0 >= L) return;
  const int kw0 = kv0 + wave * 32;          // first key of this wave
  const int my_key = kw0 + l32;

  const long kv_stride = (long)p.Hkv * D;    // elements per token
  const long q_stride_b = (long)p.Hq * D * 2;
  const int qt0 = CAUSAL ? kv0 / TROWS : 0;  // first query tile any key of the workgroup sees
  const int n_qt = (L + TROWS - 1) / TROWS;
  const int n_it = (n_qt - qt0) * p.G;       // (query head, query tile) pairs, head-major

  // ---- K, V fragments of this lane's key (B operands): [d = 16 ks + 8 hl + e] ----
  bf16x8 kf[KSTEPS], vf[KSTEPS];
  {
    const int kr = my_key < L ? my_key : L - 1;
    const __bf16* kp = (const __bf16*)p.k + ((long)(seq0 + kr) * p.Hkv + hkv) * D + hl * 8;
    const __bf16* vp = (const __bf16*)p.v + ((long)(seq0 + kr) * p.Hkv + hkv) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kf[ks] = *(const bf16x8*)(kp + ks * 16);
      vf[ks] = *(const bf16x8*)(vp + ks * 16);
    }
  }

  // ---- tile copies: tile `it` = (head gi, query tile qt), issued in order.
  // The sources of the next tile are kept as wave-uniform pointers: Q / dO
  // rows and the LSE*log2(e) / D rows move TROWS rows on per tile and jump to
  // the next query head's first tile after a head's last one (a few scalar
  // adds per tile instead of recomputing 64-bit addresses). ----
  RC copy;
  copy.init(wave, lane, (unsigned)q_stride_b);
  const int h_first = hkv * p.G;
  const long tile_step = (long)TROWS * q_stride_b;                 // bytes per Q / dO tile
  const long lse_head_step = VARLEN ? (long)T : (long)p.N;          // LSE elements between heads
  const char* q_head = (const char*)p.q + ((long)seq0 * p.Hq + h_first) * D * 2 + qt0 * tile_step;
  const char* o_head = (const char*)p.dout + ((long)seq0 * p.Hq + h_first) * D * 2 + qt0 * tile_step;
  // LSE*log2(e) and D of the tile's rows: wave w moves rows (w & 1) * 32 + lane
  // of array w >> 1 (lanes 0..31); rows of one (sequence, head) are contiguous
  const float* l_head = (wave < 2 ? p.lse2 : p.dsum) +
                        lse_index(p, s, h_first, seq0, qt0 * TROWS + (wave & 1) * 32, T, VARLEN);
  q_head = uniform_ptr(q_head);
  o_head = uniform_ptr(o_head);
  l_head = uniform_ptr(l_head);
  const char* q_cur = q_head;
  const char* o_cur = o_head;
  const float* l_cur = l_head;
  int iss_qt = qt0;
  auto issue_next = [&](char FA_LDS* stage) __attribute__((always_inline)) {
    const int q0 = iss_qt * TROWS;
    if (lane < 32) {
      // rows past the sequence end repeat its last row (or, for a half tile
      // wholly past it, fall outside the descriptor's range and read as 0)
      const int r0 = q0 + (wave & 1) * 32;
      const int r = min(r0 + lane, L - 1);
      buf2lds4(buffer_rsrc_uniform(l_cur), (unsigned)(r - r0) * 4u,
               stage + S::LSEOFF + (wave >> 1) * TROWS * 4 + (wave & 1) * 128);
    }
    if (q0 + TROWS <= L) {
      copy.template issue_full<true>(stage, q_cur);
      copy.template issue_full<true>(stage + S::TILEB, o_cur);
    } else {
      copy.template issue_tail<true>(stage, q_cur, q_stride_b, L - 1 - q0);
      copy.template issue_tail<true>(stage + S::TILEB, o_cur, q_stride_b, L - 1 - q0);
    }
    if (++iss_qt == n_qt) {
      iss_qt = qt0;
      q_head = uniform_ptr(q_head + D * 2);
      o_head = uniform_ptr(o_head + D * 2);
      l_head = uniform_ptr(l_head + lse_head_step);
      q_cur = q_head;
      o_cur = o_head;
      l_cur = l_head;
    } else {
      q_cur = uniform_ptr(q_cur + tile_step);
      o_cur = uniform_ptr(o_cur + tile_step);
      l_cur = uniform_ptr(l_cur + TROWS);
    }
  };
  issue_next(stg[0]);
  if (n_it > 1) issue_next(stg[1]);
  if (n_it > 2) issue_next(stg[2]);

  TileOffsets<D> to;
  to.init(lane);
  const int lse_lane = 16 * hl;                  // byte offset of rows 4 hl .. 4 hl + 3 in a group of 8
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }
  f32x16 sA[2], pA[2], sB[2], pB[2];             // S, dP of two consecutive tiles (by tile parity)
  u32x4 pb[4], dsb[4];                           // P, dS (bf16 pairs) of the current tile
  float pf[32];                                  // P of the current tile, fp32 (phase A -> phase B)
  const float c = p.scale_log2;

  // S, dP of one tile (phase-A MFMAs): slot j = (k-step j / 4, operand j % 4:
  // S block 0, S block 1, dP block 0, dP block 1).
  constexpr int NA = 4 * KSTEPS;
  // Slot j < NA/2: S block j % 2, k-step j / 2 (Q operand); slot j >= NA/2:
  // dP block j % 2, k-step (j - NA/2) / 2 (dO operand). The dP chains start
  // from the tile's -D rows (`nd`), so their results are dP - D.
  auto a_fetch = [&](const char FA_LDS* tile, int j) __attribute__((always_inline)) {
    const int dp = j >= NA / 2, ks = (j - dp * (NA / 2)) >> 1;
    return to.row_operand(tile + dp * S::TILEB, ks, j & 1);
  };
  auto a_step = [&](f32x16 (&sx)[2], f32x16 (&px)[2], int j, const bf16x8& a, const f32x16 (&nd)[2])
                    __attribute__((always_inline)) {
    const int dp = j >= NA / 2, ks = (j - dp * (NA / 2)) >> 1;
    f32x16& acc = dp ? px[j & 1] : sx[j & 1];
    const bf16x8& b = dp ? vf[ks] : kf[ks];
    if (ks == 0) {
      if (dp) mfma_v_init(acc, a, b, nd[j & 1]);
      else mfma_v_first(acc, a, b);
    } else {
      mfma_v(acc, a, b);
    }
  };
  // -D of a tile's rows in the accumulator layout: block qb, register r ->
  // row 32 qb + 8 (r/4) + 4 hl + r%4
  auto nd_fetch = [&](const char FA_LDS* tile, f32x16 (&nd)[2]) __attribute__((always_inline)) {
    const float FA_LDS* dz = (const float FA_LDS*)(tile + S::LSEOFF + TROWS * 4 + lse_lane);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 v = *(const f32x4 FA_LDS*)(dz + qb * 32 + g * 8);
#pragma unroll
        for (int u = 0; u < 4; ++u) nd[qb][4 * g + u] = v[u];
      }
  };

  // Phase A without softmax work (first tile).
  auto phase_a0 = [&](const char FA_LDS* tile, f32x16 (&sx)[2], f32x16 (&px)[2]) __attribute__((always_inline)) {
    f32x16 nd[2];
    nd_fetch(tile, nd);
    bf16x8 qa[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) qa[i] = a_fetch(tile, i);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const bf16x8 a = qa[j % PF];
      if (j + PF < NA) qa[j % PF] = a_fetch(tile, j + PF);
      a_step(sx, px, j, a, nd);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Phase A: S, dP of the next tile (`nt`, into sx/px) interleaved with the
  // softmax of the current tile (`ct`, rows q0.., S/dP in sc/pc) -> pb, dsb.
  // Element e of the current tile: block qb = e / 16, register r = e % 16,
  // query row qb*32 + 8(r/4) + 4 hl + r%4, key = this lane's key.
  // The copy of a later tile (`issue`) goes out right after the first operand
  // reads; the last PF slots also read the first PF transposed operands of
  // phase B (`pre`).
  constexpr int NB = 8 * DBLK;
  // phase B step i < NB/2: dV (dO^T operand), i >= NB/2: dK (Q^T operand);
  // key step t = (i mod NB/2) / DBLK, d-block db = i mod DBLK
  auto b_fetch = [&](const char FA_LDS* ct, int i) __attribute__((always_inline)) {
    const int dv_step = i < NB / 2, ii = i % (NB / 2);
    return to.tr_operand(ct + (dv_step ? S::TILEB : 0), ii / DBLK, ii % DBLK);
  };
  auto phase_a = [&](auto mask_tag, const char FA_LDS* nt, const char FA_LDS* ct, f32x16 (&sx)[2],
                     f32x16 (&px)[2], const f32x16 (&sc)[2], const f32x16 (&pc)[2], int q0, bool issue,
                     char FA_LDS* issue_stage, bf16x8 (&pre)[PF]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // distinct first instructions keep the compiler from hoisting the code the
    // masked and unmasked variants share above their branch (which would
    // compute all 32 elements' operands at once)
    if constexpr (MASK) asm volatile("; masked tile");
    else asm volatile("; unmasked tile");
    constexpr int EPS = 32 / NA;                 // softmax elements per MFMA slot
    const float FA_LDS* lz = (const float FA_LDS*)(ct + S::LSEOFF + lse_lane);
    f32x4 lg[8];                                 // LSE2 of the 8 row groups (qb, r/4)
    auto g_fetch = [&](int k) __attribute__((always_inline)) {
      lg[k] = *(const f32x4 FA_LDS*)(lz + (k >> 2) * 32 + (k & 3) * 8);
    };
    f32x16 nd[2];                                // -D of the next tile's rows (dP chain seeds)
    // The 32 elements of P run as a three-stage software pipeline, one step per
    // element slot, so that no instruction of a slot waits on another one of
    // the same slot: step t forms x_t = S c - LSE2 (element t), p_{t-1} =
    // exp2(x_{t-1}) (masked, kept in fp32 for phase B), and packs the pair
    // (t-3, t-2) to bf16 when t-2 is odd. Steps 32 and 33 follow the last MFMA
    // slot. dS = P (dP - D) is left to phase B, whose MFMAs have no other VALU
    // work beside them.
    float xa[4];
    auto st1 = [&](int e) __attribute__((always_inline)) {
      const int qb = e >> 4, r = e & 15, k = e >> 2, u = e & 3;
      if (u == 0 && k + 1 < 8) g_fetch(k + 1);
      xa[e & 3] = __builtin_fmaf(sc[qb][r], c, -lg[k][u]);
    };
    auto st2 = [&](int e) __attribute__((always_inline)) {
      float pe = __builtin_amdgcn_exp2f(xa[e & 3]);
      if constexpr (MASK) {
        const int qb = e >> 4, r = e & 15;
        const int q = q0 + qb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const bool dead = (q >= L) || (CAUSAL && my_key > q);
        pe = dead ? 0.f : pe;
      }
      pf[e] = pe;
    };
    auto st3 = [&](int e) __attribute__((always_inline)) {
      if (e & 1) {
        // pair (e-1, e) -> positions of the B operand of key step t = qb*2 + (r/8)
        const int qb = e >> 4, r = e & 15;
        unsigned w = __builtin_bit_cast(unsigned, pack_bf16(pf[e - 1], pf[e]));
        asm volatile("" : "+v"(w));   // keep the pack in its MFMA slot (not sunk below the last MFMA)
        pb[qb * 2 + (r >> 3)][(r & 7) >> 1] = w;
      }
    };
    auto step = [&](int t) __attribute__((always_inline)) {
      if (t >= 2 && t < 34) st3(t - 2);
      if (t >= 1 && t < 33) st2(t - 1);
      if (t < 32) st1(t);
    };
    bf16x8 qa[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) qa[i] = a_fetch(nt, i);
    if (issue) issue_next(issue_stage);
    g_fetch(0);
    nd_fetch(nt, nd);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NA; ++j) {
      const bf16x8 a = qa[j % PF];
      if (j + PF < NA) qa[j % PF] = a_fetch(nt, j + PF);
      else pre[j + PF - NA] = b_fetch(ct, j + PF - NA);
      a_step(sx, px, j, a, nd);
#pragma unroll
      for (int x = 0; x < EPS; ++x) step(j * EPS + x);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int t = 32; t < 34; ++t) step(t);
  };

  // Phase B: dV^T += dO^T P (steps 0 .. NB/2-1), then dK^T += Q^T dS (steps
  // NB/2 .. NB-1) for the current tile; `qa` holds the transposed operands of
  // steps 0 .. PF-1 (read during phase A). Beside the dV MFMAs the VALU forms
  // dS = P (dP - D) (pc holds dP - D) and packs it, a two-stage pipeline over
  // the 16 element pairs: the products of pairs 2j, 2j+1 at one step, their
  // bf16 packs at the next.
  auto phase_b = [&](const char FA_LDS* ct, bf16x8 (&qa)[PF], const f32x16 (&pc)[2]) __attribute__((always_inline)) {
    constexpr int NH = NB / 2;
    constexpr int PPS = 16 / NH;                 // element pairs per dV step
    float dsv[2][2 * PPS];
    auto ds_mul = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < PPS; ++x) {
        const int e = 2 * (st * PPS + x);
        dsv[st & 1][2 * x] = pf[e] * pc[e >> 4][e & 15];
        dsv[st & 1][2 * x + 1] = pf[e + 1] * pc[(e + 1) >> 4][(e + 1) & 15];
      }
    };
    auto ds_pack = [&](int st) __attribute__((always_inline)) {
#pragma unroll
      for (int x = 0; x < PPS; ++x) {
        const int e = 2 * (st * PPS + x), qb = e >> 4, r = e & 15;
        dsb[qb * 2 + (r >> 3)][(r & 7) >> 1] =
            __builtin_bit_cast(unsigned, pack_bf16(dsv[st & 1][2 * x], dsv[st & 1][2 * x + 1]));
      }
    };
    asm volatile("s_nop 2");   // VALU-written B operands -> first MFMA
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bf16x8 a = qa[i % PF];
      if (i + PF < NB) qa[i % PF] = b_fetch(ct, i + PF);
      if (i < NH) {
        const int t = i / DBLK, db = i % DBLK;
        mfma_a(dv[db], a, __builtin_bit_cast(bf16x8, pb[t]));
        if (i >= 1) ds_pack(i - 1);
        ds_mul(i);
      } else {
        if (i == NH) {
          ds_pack(NH - 1);
          asm volatile("s_nop 2");               // VALU-written dS -> dK MFMA
        }
        const int t = (i - NH) / DBLK, db = (i - NH) % DBLK;
        mfma_a(dk[db], a, __builtin_bit_cast(bf16x8, dsb[t]));
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- prologue: K/V fragments and tile 0 in, S/dP of tile 0 ----
  if (n_it > 2) wait_vm(2 * OPS);
  else if (n_it > 1) wait_vm(OPS);
  else wait_vm(0);
  barrier_no_fence();
  phase_a0(stg[0], sA, pA);
  mfma_result_wait();

  int cur_qt = qt0;
  // Iteration i (BI = i % NSTAGE): tile i in stg[BI], tile i+1 in stg[BI+1],
  // tile i+3 is copied into stg[BI+3] (last read as tile i-1, before this
  // iteration's barrier).
  auto iter = [&](auto bi_tag, const int i) __attribute__((always_inline)) {
    constexpr int BI = decltype(bi_tag)::value;
    if (i + 2 < n_it) wait_vm(OPS);
    else if (i + 1 < n_it) wait_vm(0);
    barrier_no_fence();
    const bool issue = i + 3 < n_it;
    char FA_LDS* const nst = stg[(BI + 3) % NSTAGE];
    const int q0 = cur_qt * TROWS;
    if (++cur_qt == n_qt) cur_qt = qt0;
    const bool need_mask = (q0 + TROWS > L) || (CAUSAL && kw0 + 31 > q0);
    // the S/dP MFMAs of tile i+1 also run on the last iteration (on stale LDS,
    // results unused) so that the code has a single shape
    bf16x8 pre[PF];
    if constexpr (BI % 2 == 0) {
      if (need_mask) phase_a(ic<1>{}, stg[(BI + 1) % NSTAGE], stg[BI], sB, pB, sA, pA, q0, issue, nst, pre);
      else phase_a(ic<0>{}, stg[(BI + 1) % NSTAGE], stg[BI], sB, pB, sA, pA, q0, issue, nst, pre);
      phase_b(stg[BI], pre, pA);
    } else {
      if (need_mask) phase_a(ic<1>{}, stg[(BI + 1) % NSTAGE], stg[BI], sA, pA, sB, pB, q0, issue, nst, pre);
      else phase_a(ic<0>{}, stg[(BI + 1) % NSTAGE], stg[BI], sA, pA, sB, pB, q0, issue, nst, pre);
      phase_b(stg[BI], pre, pB);
    }
  };
  for (int i = 0; i < n_it; i += NSTAGE) {
    iter(ic<0>{}, i);
    if (i + 1 < n_it) iter(ic<1>{}, i + 1);
    if (i + 2 < n_it) iter(ic<2>{}, i + 2);
    if (i + 3 < n_it) iter(ic<3>{}, i + 3);
  }
  // the last tile's S/dP MFMAs (results unused) and the dK/dV MFMAs must be
  // done before their registers are reused or read
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    keep_live(sA[x]);
    keep_live(pA[x]);
    keep_live(sB[x]);
    keep_live(pB[x]);
  }
  mfma_result_wait();

  // ---- epilogue: dK = scale dK^T, dV = dV^T, staged as bf16 rows ----
  barrier_no_fence();
  char FA_LDS* st = stg[0];
  if (wave == 1) st = stg[1];
  if (wave == 2) st = stg[2];
  if (wave == 3) st = stg[3];
  __bf16* dkb = (__bf16*)p.dk + ((long)seq0 * p.Hkv + hkv) * D;
  __bf16* dvb = (__bf16*)p.dv + ((long)seq0 * p.Hkv + hkv) * D;
  store_rows_bf16<D>(st, dk, p.scale, dkb, kv_stride, kw0, L, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  store_rows_bf16<D>(st, dv, 1.0f, dvb, kv_stride, kw0, L, lane);
}

// ---------------------------------------------------------------------------
// 3. dQ: Q-major
// ---------------------------------------------------------------------------
// Each wave owns 64 queries (two 32-query MFMA blocks), so every K / V / K^T
// fragment read from LDS feeds two MFMAs; the waves' Q and dO fragments and
// dQ accumulators fill the accumulation registers. K/V stream in 32-key tiles
// through the 4-stage ring (4 x 16 KiB for d = 128).
constexpr int DQ_WQ = 64;                 // queries per wave
constexpr int DQ_BM = NWAVES * DQ_WQ;     // queries per workgroup
constexpr int DQ_BN = 32;                 // keys per K/V tile

template <int D>
struct QStage {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = DQ_BN * ROWB;          // one K or V tile
  static constexpr int BYTES = 2 * TILEB;
  static constexpr int OROWB = ROWB + 16;
  static_assert(32 * OROWB <= BYTES, "32 rows of a wave's output staging must fit in one stage");
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void bwd_dq_kernel(const BwdParams p, int n_qtiles) {
  using S = QStage<D>;
  using RC = RowCopy<D, DQ_BN>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  constexpr int OPS = 2 * RC::PER_WAVE;
  __shared__ __attribute__((aligned(1024))) char s0_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s1_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s2_raw[S::BYTES];
  __shared__ __attribute__((aligned(1024))) char s3_raw[S::BYTES];
  char FA_LDS* const stg[NSTAGE] = {(char FA_LDS*)s0_raw, (char FA_LDS*)s1_raw, (char FA_LDS*)s2_raw,
                                    (char FA_LDS*)s3_raw};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hl = lane >> 5, l32 = lane & 31;

  // work item -> (sequence s, query head h, query tile qt), in the order
  // fa_order.h describes, heaviest (last) query tiles first
  TileItem item;
  if constexpr (VARLEN) {
    if (!q_item_xcd(blockIdx.x, p.B, p.Hkv, p.G, p.kv_chunks, n_qtiles, true, item)) return;
  } else {
    if (!q_item_level(blockIdx.x, p.B, p.Hq, p.G, n_qtiles, true, item)) return;
  }
  const int s = item.s, h = item.h, qt = item.t;
  const int hkv = h / p.G;

  int seq0, L, T = 0;
  if constexpr (VARLEN) {
    seq0 = p.cu_seqlens[s];
    L = p.cu_seqlens[s + 1] - seq0;
    T = p.cu_seqlens[p.B];
  } else {
    seq0 = s * p.N;
    L = p.N;
  }
  const int q0 = qt * DQ_BM;
  if (q0 >= L) return;
  const int qw0 = q0 + wave * DQ_WQ;            // first query of this wave
  int my_q[2];
  my_q[0] = qw0 + l32;
  my_q[1] = qw0 + 32 + l32;

  const long q_stride = (long)p.Hq * D;
  const long kv_stride_b = (long)p.Hkv * D * 2;
  const char* kbase = (const char*)p.k + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const char* vbase = (const char*)p.v + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const int kv_end = CAUSAL ? min(L, q0 + DQ_BM) : L;
  const int n_it = (kv_end + DQ_BN - 1) / DQ_BN;

  // ---- Q, dO fragments of this lane's two queries (B operands), LSE2 and D ----
  bf16x8 qf[2][KSTEPS], of[2][KSTEPS];
  float lse2[2], dq_d[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qr = my_q[qb] < L ? my_q[qb] : L - 1;
    const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
    const __bf16* op = (const __bf16*)p.dout + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[qb][ks] = *(const bf16x8*)(qp + ks * 16);
      of[qb][ks] = *(const bf16x8*)(op + ks * 16);
    }
    const long li = lse_index(p, s, h, seq0, qr, T, VARLEN);
    lse2[qb] = p.lse2[li];
    dq_d[qb] = p.dsum[li];
  }

  RC copy;
  copy.init(wave, lane, (unsigned)kv_stride_b);
  int iss = 0;
  auto issue_next = [&](char FA_LDS* stage) __attribute__((always_inline)) {
    copy.issue(stage, kbase, kv_stride_b, iss * DQ_BN, L);
    copy.issue(stage + S::TILEB, vbase, kv_stride_b, iss * DQ_BN, L);
    ++iss;
  };
  issue_next(stg[0]);
  if (n_it > 1) issue_next(stg[1]);
  if (n_it > 2) issue_next(stg[2]);

  TileOffsets<D> to;
  to.init(lane);
  f32x16 dq[2][DBLK];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int i = 0; i < DBLK; ++i) dq[qb][i] = f32x16{};
  f32x16 sA[2], pA[2], sB[2], pB[2];             // S^T, dP^T of a tile, per query block, two tiles
  u32x4 dsb[2][2];                               // dS^T (bf16 pairs) of the current tile [query block][key step]
  const float c = p.scale_log2;

  // Phase-A MFMA j: k-step j / 4, operand j % 4 = S block 0, S block 1, dP block
  // 0, dP block 1. The K (or V) fragment of a k-step serves both query blocks,
  // so fragment f = j / 2 is read once: k-step f / 2 of K (f even) or V.
  constexpr int NA = 4 * KSTEPS;
  constexpr int NF = NA / 2;
  auto a_frag = [&](const char FA_LDS* tile, int f) __attribute__((always_inline)) {
    return to.row_operand(tile + (f & 1) * S::TILEB, f >> 1, 0);
  };
  auto a_step = [&](f32x16 (&sx)[2], f32x16 (&px)[2], int j, const bf16x8& a) __attribute__((always_inline)) {
    const int ks = j >> 2, cc = j & 3;
    f32x16& acc = cc < 2 ? sx[cc & 1] : px[cc & 1];
    const bf16x8& b = cc < 2 ? qf[cc & 1][ks] : of[cc & 1][ks];
    if (ks == 0) mfma_v_first(acc, a, b);
    else mfma_v(acc, a, b);
  };
  auto phase_a0 = [&](const char FA_LDS* tile, f32x16 (&sx)[2], f32x16 (&px)[2]) __attribute__((always_inline)) {
    bf16x8 qa[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) qa[i] = a_frag(tile, i);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8 a = qa[f % PF];
      if (f + PF < NF) qa[f % PF] = a_frag(tile, f + PF);
      a_step(sx, px, 2 * f, a);
      a_step(sx, px, 2 * f + 1, a);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Element e of the current tile: query block qb = e / 16, register r = e % 16,
  // key k0 + 8(r/4) + 4 hl + r%4, query my_q[qb].
  // The copy of a later tile (`issue`) goes out right after the first operand
  // reads; the last PF fragment slots also read the first PF transposed
  // fragments of phase B (`pre`, from the current tile `ct`).
  constexpr int NB = 2 * DBLK;
  auto b_fetch = [&](const char FA_LDS* ct, int i) __attribute__((always_inline)) {
    return to.tr_operand(ct, i / DBLK, i % DBLK);
  };
  auto phase_a = [&](auto mask_tag, const char FA_LDS* nt, const char FA_LDS* ct, f32x16 (&sx)[2],
                     f32x16 (&px)[2], const f32x16 (&sc)[2], const f32x16 (&pc)[2], int k0, bool issue,
                     char FA_LDS* issue_stage, bf16x8 (&pre)[PF]) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_tag)::value;
    // distinct first instructions keep the compiler from hoisting the code the
    // masked and unmasked variants share above their branch
    if constexpr (MASK) asm volatile("; masked tile");
    else asm volatile("; unmasked tile");
    constexpr int EPS = 32 / NA;
    float dv2[2];
    auto elem = [&](int e) __attribute__((always_inline)) {
      const int qb = e >> 4, r = e & 15;
      // lse2 and dq_d are "redefined" (no instruction) at every element so the
      // element's arithmetic stays in its MFMA slot instead of being hoisted
      // to the top of the phase, where all 32 results would be live at once
      asm volatile("" : "+v"(lse2[qb]), "+v"(dq_d[qb]));
      float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[qb][r], c, -lse2[qb]));
      if constexpr (MASK) {
        const int key = k0 + 8 * (r >> 2) + 4 * hl + (r & 3);
        const bool dead = (key >= L) || (CAUSAL && key > my_q[qb]);
        pe = dead ? 0.f : pe;
      }
      dv2[e & 1] = pe * (pc[qb][r] + dq_d[qb]);   // dq_d holds -D
      if (e & 1) dsb[qb][r >> 3][(r & 7) >> 1] = __builtin_bit_cast(unsigned, pack_bf16(dv2[0], dv2[1]));
    };
    bf16x8 qa[PF];
#pragma unroll
    for (int i = 0; i < PF; ++i) qa[i] = a_frag(nt, i);
    if (issue) issue_next(issue_stage);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const bf16x8 a = qa[f % PF];
      if (f + PF < NF) qa[f % PF] = a_frag(nt, f + PF);
      else if (f + PF - NF < NB) pre[f + PF - NF] = b_fetch(ct, f + PF - NF);
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int j = 2 * f + x;
        a_step(sx, px, j, a);
#pragma unroll
        for (int y = 0; y < EPS; ++y) elem(j * EPS + y);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // Phase B: dQ^T += K^T dS^T. Fragment i: key step t = i / DBLK, d-block
  // db = i % DBLK, used by both query blocks; `qa` holds fragments 0 .. PF-1.
  static_assert(PF <= NB, "phase B must have at least PF fragments");
  auto phase_b = [&](const char FA_LDS* ct, bf16x8 (&qa)[PF]) __attribute__((always_inline)) {
    asm volatile("s_nop 2");   // VALU-written B operands -> first MFMA
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const bf16x8 a = qa[i % PF];
      if (i + PF < NB) qa[i % PF] = b_fetch(ct, i + PF);
      const int t = i / DBLK, db = i % DBLK;
      mfma_a(dq[0][db], a, __builtin_bit_cast(bf16x8, dsb[0][t]));
      mfma_a(dq[1][db], a, __builtin_bit_cast(bf16x8, dsb[1][t]));
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (n_it > 2) wait_vm(2 * OPS);
  else if (n_it > 1) wait_vm(OPS);
  else wait_vm(0);
  barrier_no_fence();
  phase_a0(stg[0], sA, pA);
  mfma_result_wait();

  // Iteration i (BI = i % NSTAGE): tile i in stg[BI], tile i+1 in stg[BI+1],
  // tile i+3 is copied into stg[BI+3] (last read as tile i-1, before this
  // iteration's barrier).
  auto iter = [&](auto bi_tag, const int i) __attribute__((always_inline)) {
    constexpr int BI = decltype(bi_tag)::value;
    if (i + 2 < n_it) wait_vm(OPS);
    else if (i + 1 < n_it) wait_vm(0);
    barrier_no_fence();
    const bool issue = i + 3 < n_it;
    char FA_LDS* const nst = stg[(BI + 3) % NSTAGE];
    const int k0 = i * DQ_BN;
    const bool need_mask = (k0 + DQ_BN > L) || (CAUSAL && k0 + DQ_BN - 1 > qw0);
    // the S/dP MFMAs of tile i+1 also run on the last iteration (on stale LDS,
    // results unused) so that the code has a single shape
    bf16x8 pre[PF];
    if constexpr (BI % 2 == 0) {
      if (need_mask) phase_a(ic<1>{}, stg[(BI + 1) % NSTAGE], stg[BI], sB, pB, sA, pA, k0, issue, nst, pre);
      else phase_a(ic<0>{}, stg[(BI + 1) % NSTAGE], stg[BI], sB, pB, sA, pA, k0, issue, nst, pre);
    } else {
      if (need_mask) phase_a(ic<1>{}, stg[(BI + 1) % NSTAGE], stg[BI], sA, pA, sB, pB, k0, issue, nst, pre);
      else phase_a(ic<0>{}, stg[(BI + 1) % NSTAGE], stg[BI], sA, pA, sB, pB, k0, issue, nst, pre);
    }
    phase_b(stg[BI], pre);
  };
  for (int i = 0; i < n_it; i += NSTAGE) {
    iter(ic<0>{}, i);
    if (i + 1 < n_it) iter(ic<1>{}, i + 1);
    if (i + 2 < n_it) iter(ic<2>{}, i + 2);
    if (i + 3 < n_it) iter(ic<3>{}, i + 3);
  }
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    keep_live(sA[x]);
    keep_live(pA[x]);
    keep_live(sB[x]);
    keep_live(pB[x]);
  }
  mfma_result_wait();

  barrier_no_fence();
  char FA_LDS* st = stg[0];
  if (wave == 1) st = stg[1];
  if (wave == 2) st = stg[2];
  if (wave == 3) st = stg[3];
  __bf16* dqb = (__bf16*)p.dq + ((long)seq0 * p.Hq + h) * D;
  store_rows_bf16<D>(st, dq[0], p.scale, dqb, q_stride, qw0, L, lane);
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_wave_barrier();
  store_rows_bf16<D>(st, dq[1], p.scale, dqb, q_stride, qw0 + 32, L, lane);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_bwd_t(const BwdParams& p, int stages, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (stages & 1) {
    const long n_tok = (long)p.B * p.N;          // upper bound (packed: T <= B * N)
    const long grid = (n_tok + PREP_TOK - 1) / PREP_TOK * p.Hq;
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_prep_kernel<D, VARLEN>), dim3((unsigned)grid), dim3(256), 0, stream, p, n_tok);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if constexpr (VARLEN) {
      hipLaunchKernelGGL(bwd_sched_kernel, dim3(1), dim3(256), 0, stream, p.cu_seqlens, p.B, p.kv_chunks,
                         p.kt_prefix);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
  }
  if (stages & 2) {
    const int n_kt = (p.N + KV_BN - 1) / KV_BN;
    const long grid = VARLEN ? kv_grid_xcd(p.B, p.Hkv, p.kv_chunks, n_kt) : kv_grid_level(p.B, p.Hkv, n_kt);
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4) {
    const int n_qt = (p.N + DQ_BM - 1) / DQ_BM;
    const long grid = VARLEN ? q_grid_xcd(p.B, p.Hkv, p.G, p.kv_chunks, n_qt) : q_grid_level(p.B, p.Hq, p.G, n_qt);
    if (grid > 0x7fffffffL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN>), dim3((unsigned)grid), dim3(NTHREADS), 0, stream, p, n_qt);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return e;
}

hipError_t bwd_launch(BwdParams p, int d, int causal, int varlen, int stages, hipStream_t stream) {
  if (d == 128) {
    if (causal)
      return varlen ? launch_bwd_t<128, true, true>(p, stages, stream) : launch_bwd_t<128, true, false>(p, stages, stream);
    return varlen ? launch_bwd_t<128, false, true>(p, stages, stream) : launch_bwd_t<128, false, false>(p, stages, stream);
  }
  if (causal)
    return varlen ? launch_bwd_t<64, true, true>(p, stages, stream) : launch_bwd_t<64, true, false>(p, stages, stream);
  return varlen ? launch_bwd_t<64, false, true>(p, stages, stream) : launch_bwd_t<64, false, false>(p, stages, stream);
}

}  // namespace fa

// fa_bwd.hip -- exact attention backward for gfx950 (MI355X).
//
// The backward pass recomputes the softmax from the forward's log-sum-exp and
// produces dQ, dK and dV (backward pass: abstract on the zhuanzhiai.com page;
// the pages' own design uses tensor memory and 2-CTA MMA to cut shared-memory
// traffic and atomic adds there, which this hardware does not have). With
// P = exp(S - LSE) and D_i = dO_i . O_i:
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  dQ = scale dS K,  dK = scale dS^T Q.
//
// Three kernels, all on the caller's stream:
//   1. bwd_dsum_kernel: D_i = rowsum(dO o O) in fp32 (HBM-bound, one pass).
//   2. bwd_dkdv_kernel: one workgroup per (sequence, K/V head, 128-key tile);
//      each wave keeps 32 keys' K and V fragments in registers and streams the
//      64-row Q / dO tiles of every query head of the group through LDS, so the
//      group's dK/dV sum needs no atomics. Per tile and wave: S = Q K^T and
//      dP = dO V^T with the key in the lane (C layout), dV^T += dO^T P and
//      dK^T += Q^T dS with the transposed Q / dO operands read by
//      ds_read_b64_tr_b16.
//   3. bwd_dq_kernel: one workgroup per (sequence, query head, 128-query tile),
//      mirroring the forward: S^T = K Q^T and dP^T = V dO^T with the query in
//      the lane, then dQ^T += K^T dS^T (K^T through ds_read_b64_tr_b16).
// dQ is produced by this separate pass rather than by atomic adds from kernel 2.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int KV_BN = 128;    // keys per dK/dV workgroup (32 per wave)
constexpr int KV_BM = 64;     // query rows per streamed tile in the dK/dV kernel
constexpr int Q_BM = 128;     // queries per dQ workgroup (32 per wave)
constexpr int Q_BN = 64;      // keys per streamed tile in the dQ kernel

// Copy `nrows` rows (clamped to L-1) of a [tokens][row_stride] bf16 tensor into a
// swizzled LDS tile [nrows][D]; all NTHREADS threads take part.
template <int D, int NROWS>
__device__ __forceinline__ void load_rows(char FA_LDS* dst, const char* gbase, long row_stride_b, int r0, int L,
                                          int wave, int lane) {
  constexpr int ROWB = D * 2;
  constexpr int LPR = ROWB / 16;
  constexpr int RPI = 64 / LPR;
  constexpr int NI = NROWS / RPI;
  static_assert(NI % NWAVES == 0, "tile rows must split evenly over the waves");
  constexpr int PER_WAVE = NI / NWAVES;
  const int r_in = lane / LPR;
  const int pos = lane % LPR;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int ins = wave * PER_WAVE + u;
    const int row = ins * RPI + r_in;
    int g = r0 + row;
    g = g < L ? g : L - 1;
    g2lds16(gbase + (long)g * row_stride_b + (pos ^ lds_swz<D>(row)) * 16, dst + ins * 1024);
  }
}

__device__ __forceinline__ long lse_index(const BwdParams& p, int s, int h, int seq0, int row, int T, bool varlen) {
  return varlen ? (long)h * T + seq0 + row : ((long)s * p.Hq + h) * p.N + row;
}

// Stage a wave's 32 x D fp32 accumulator (transposed C layout: lane = row
// l32, register r of block db = column db*32 + 8(r/4) + 4(l/32) + r%4) as bf16
// through LDS and write whole 16-byte row segments to global memory.
template <int D>
__device__ __forceinline__ void store_rows_bf16(char FA_LDS* st, const f32x16* acc, float mul, __bf16* gbase,
                                                long row_stride, int row0, int L, int lane) {
  constexpr int OROWB = D * 2 + 16;
  const int l32 = lane & 31, hl = lane >> 5;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + 8 * g + 4 * hl;
      const bf16x2 a = pack_bf16(acc[db][4 * g + 0] * mul, acc[db][4 * g + 1] * mul);
      const bf16x2 b = pack_bf16(acc[db][4 * g + 2] * mul, acc[db][4 * g + 3] * mul);
      *(bf16x4 FA_LDS*)(st + l32 * OROWB + dcol * 2) = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    }
  __builtin_amdgcn_wave_barrier();
  constexpr int CPR = D / 8;
  constexpr int PER_LANE = 32 * CPR / 64;
#pragma unroll
  for (int u = 0; u < PER_LANE; ++u) {
    const int idx = u * 64 + lane;
    const int row = idx / CPR, ch = idx % CPR;
    const int r = row0 + row;
    const bf16x8 v8 = *(const bf16x8 FA_LDS*)(st + row * OROWB + ch * 16);
    if (r < L) *(bf16x8*)(gbase + (long)r * row_stride + ch * 8) = v8;
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// 1. D_i = sum_k dO[i,k] O[i,k]
// ---------------------------------------------------------------------------
template <int D, bool VARLEN>
__global__ __launch_bounds__(256) void bwd_dsum_kernel(const BwdParams p, long total_rows) {
  constexpr int LPR = D / 8;                 // lanes per (token, head) row, 16 B each
  constexpr int RPB = 256 / LPR;             // rows per block
  const long r = (long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  long T = total_rows / p.Hq;
  if constexpr (VARLEN) T = p.cu_seqlens[p.B];
  const bool ok = r < T * p.Hq;
  float acc = 0.f;
  if (ok) {
    const bf16x8 a = *(const bf16x8*)((const __bf16*)p.dout + r * D + part * 8);
    const bf16x8 b = *(const bf16x8*)((const __bf16*)p.o + r * D + part * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)a[e], (float)b[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, LPR);
  if (ok && part == 0) {
    const long t = r / p.Hq;
    const int h = (int)(r - t * p.Hq);
    long idx;
    if constexpr (VARLEN) idx = (long)h * T + t;
    else {
      const long b = t / p.N, n = t - b * p.N;
      idx = (b * p.Hq + h) * p.N + n;
    }
    p.dsum[idx] = acc;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV: KV-major
// ---------------------------------------------------------------------------
template <int D>
struct KvSmem {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = KV_BM * ROWB;          // one Q or dO tile
  static constexpr int STAGEB = 2 * TILEB + 2 * KV_BM * 4;   // Q, dO, LSE, D
  static constexpr int OROWB = ROWB + 16;
  static_assert(2 * 32 * OROWB <= STAGEB, "two waves' output staging must fit in one stage");
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_kernel(const BwdParams p) {
  using S = KvSmem<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  // two distinct LDS objects so reads of one stage never wait on the copy into the other
  __shared__ __attribute__((aligned(1024))) char stage0_raw[S::STAGEB];
  __shared__ __attribute__((aligned(1024))) char stage1_raw[S::STAGEB];
  char FA_LDS* stage0 = (char FA_LDS*)stage0_raw;
  char FA_LDS* stage1 = (char FA_LDS*)stage1_raw;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  // work item: level-major (key tile 0 first: under causal masking it sees the
  // most query tiles), then (sequence, K/V head)
  const int n_kt = (p.N + KV_BN - 1) / KV_BN;
  const int per_level = p.B * p.Hkv;
  const int w = blockIdx.x;
  const int kt = w / per_level;
  const int rr = w - kt * per_level;
  const int s = rr / p.Hkv;
  const int hkv = rr - s * p.Hkv;
  (void)n_kt;

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
  const long q_stride = (long)p.Hq * D;
  // K, V fragments of this lane's key (B operands): [d = 16 ks + 8 hl + e]
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
  f32x16 dk[DBLK], dv[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) {
    dk[i] = f32x16{};
    dv[i] = f32x16{};
  }

  const int qt0 = CAUSAL ? kv0 / KV_BM : 0;
  const int n_qt = (L + KV_BM - 1) / KV_BM;
  const int per_head = n_qt - qt0;
  const int n_it = per_head * p.G;
  const float c = p.scale_log2;

  auto issue = [&](int it, char FA_LDS* stage) {
    const int gi = it / per_head;
    const int qt = qt0 + (it - gi * per_head);
    const int h = hkv * p.G + gi;
    const int q0 = qt * KV_BM;
    const char* qb = (const char*)p.q + ((long)seq0 * p.Hq + h) * D * 2;
    const char* ob = (const char*)p.dout + ((long)seq0 * p.Hq + h) * D * 2;
    load_rows<D, KV_BM>(stage, qb, q_stride * 2, q0, L, wave, lane);
    load_rows<D, KV_BM>(stage + S::TILEB, ob, q_stride * 2, q0, L, wave, lane);
    if (wave == 0) {
      int r = q0 + lane;
      r = r < L ? r : L - 1;
      const long li = lse_index(p, s, h, seq0, r, T, VARLEN);
      __builtin_amdgcn_global_load_lds(p.lse + li, stage + 2 * S::TILEB, 4, 0, 0);
      __builtin_amdgcn_global_load_lds(p.dsum + li, stage + 2 * S::TILEB + KV_BM * 4, 4, 0, 0);
    }
  };

  issue(0, stage0);
  wait_vmem();
  __syncthreads();

  const int g16 = lane & 15;
  auto step = [&](char FA_LDS* cur, char FA_LDS* nxt, const int it) __attribute__((always_inline)) {
    if (it + 1 < n_it) issue(it + 1, nxt);
    const int qt = qt0 + (it % per_head);
    const int q0 = qt * KV_BM;
    // causal: this wave's keys see queries >= kw0 only
    const bool active = !CAUSAL || (q0 + KV_BM - 1 >= kw0);
    if (active) {
      const char FA_LDS* qtile = cur;
      const char FA_LDS* otile = cur + S::TILEB;
      const float FA_LDS* lse_s = (const float FA_LDS*)(cur + 2 * S::TILEB);
      const float FA_LDS* dsum_s = lse_s + KV_BM;
      // S = Q K^T and dP = dO V^T for 2 x 32 query rows; lane = key
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const int row = qb * 32 + l32;
          const int off = row * S::ROWB + (((2 * ks + hl) ^ lds_swz<D>(row)) * 16);
          sacc[qb] = mfma32(lds_read16(qtile + off), kf[ks], sacc[qb]);
          pacc[qb] = mfma32(lds_read16(otile + off), vf[ks], pacc[qb]);
        }
      }
      // P = exp2(S c - LSE log2e); dS = P (dP - D)
      const bool need_mask = (CAUSAL && (kw0 + 31 > q0)) || (q0 + KV_BM > L) || (kw0 + 32 > L);
      bf16x8 pb[4], db8[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qr = qb * 32 + 8 * g + 4 * hl;     // first of 4 query rows
          const f32x4 lz = *(const f32x4 FA_LDS*)(lse_s + qr);
          const f32x4 dz = *(const f32x4 FA_LDS*)(dsum_s + qr);
          float pv[4], dsv[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            const int r = 4 * g + u;
            float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c, -lz[u] * kLog2e));
            if (need_mask) {
              const int q = q0 + qr + u;
              const bool dead = (q >= L) || (my_key >= L) || (CAUSAL && my_key > q);
              pe = dead ? 0.f : pe;
            }
            pv[u] = pe;
            dsv[u] = pe * (pacc[qb][r] - dz[u]);
          }
          const int t = qb * 2 + (g >> 1), e0 = (g & 1) * 4;
          const bf16x2 p01 = pack_bf16(pv[0], pv[1]), p23 = pack_bf16(pv[2], pv[3]);
          const bf16x2 d01 = pack_bf16(dsv[0], dsv[1]), d23 = pack_bf16(dsv[2], dsv[3]);
          pb[t][e0 + 0] = p01[0];
          pb[t][e0 + 1] = p01[1];
          pb[t][e0 + 2] = p23[0];
          pb[t][e0 + 3] = p23[1];
          db8[t][e0 + 0] = d01[0];
          db8[t][e0 + 1] = d01[1];
          db8[t][e0 + 2] = d23[0];
          db8[t][e0 + 3] = d23[1];
        }
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (A operands through transposing reads)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r0 = 16 * t + 4 * hl + (g16 >> 2), r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
          const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
          const int o0 = r0 * S::ROWB + ((chunk ^ lds_swz<D>(r0)) * 16) + sub;
          const int o1 = r1 * S::ROWB + ((chunk ^ lds_swz<D>(r1)) * 16) + sub;
          dv[db] = mfma32(cat(lds_read_tr(otile + o0), lds_read_tr(otile + o1)), pb[t], dv[db]);
          dk[db] = mfma32(cat(lds_read_tr(qtile + o0), lds_read_tr(qtile + o1)), db8[t], dk[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int it = 0; it < n_it; it += 2) {
    step(stage0, stage1, it);
    if (it + 1 < n_it) step(stage1, stage0, it + 1);
  }

  // epilogue: dK = scale dK^T, dV = dV^T, staged as bf16 rows
  char FA_LDS* st = (wave < 2 ? stage0 : stage1) + (wave & 1) * 32 * S::OROWB;
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
template <int D>
struct QSmem {
  static constexpr int ROWB = D * 2;
  static constexpr int TILEB = Q_BN * ROWB;
  static constexpr int STAGEB = 2 * TILEB;           // K, V
  static constexpr int OROWB = ROWB + 16;
  static_assert(2 * 32 * OROWB <= STAGEB, "two waves' output staging must fit in one stage");
};

template <int D, bool CAUSAL, bool VARLEN>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_kernel(const BwdParams p, int n_qtiles, int xcd_group) {
  using S = QSmem<D>;
  constexpr int KSTEPS = D / 16;
  constexpr int DBLK = D / 32;
  __shared__ __attribute__((aligned(1024))) char stage0_raw[S::STAGEB];
  __shared__ __attribute__((aligned(1024))) char stage1_raw[S::STAGEB];
  char FA_LDS* stage0 = (char FA_LDS*)stage0_raw;
  char FA_LDS* stage1 = (char FA_LDS*)stage1_raw;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hl = lane >> 5, l32 = lane & 31;

  int w = blockIdx.x;
  if (xcd_group > 0) {
    const int xcd = w & 7, j = w >> 3;
    w = (8 * (j / xcd_group) + xcd) * xcd_group + (j % xcd_group);
  }
  const int per_level = p.B * p.Hq;
  if (w >= per_level * n_qtiles) return;
  const int lvl = w / per_level;
  const int rr = w - lvl * per_level;
  const int s = rr / p.Hq;
  const int h = rr - s * p.Hq;
  const int qt = n_qtiles - 1 - lvl;            // heaviest (last) query tiles first
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
  const int q0 = qt * Q_BM;
  if (q0 >= L) return;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;

  const long q_stride = (long)p.Hq * D;
  const long kv_stride_b = (long)p.Hkv * D * 2;
  const char* kbase = (const char*)p.k + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const char* vbase = (const char*)p.v + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const int kv_end = CAUSAL ? min(L, q0 + Q_BM) : L;
  const int n_kv = (kv_end + Q_BN - 1) / Q_BN;

  auto issue = [&](int kt, char FA_LDS* stage) {
    load_rows<D, Q_BN>(stage, kbase, kv_stride_b, kt * Q_BN, L, wave, lane);
    load_rows<D, Q_BN>(stage + S::TILEB, vbase, kv_stride_b, kt * Q_BN, L, wave, lane);
  };
  issue(0, stage0);

  bf16x8 qf[KSTEPS], of[KSTEPS];
  float lse2, dq_d;
  {
    const int qr = my_q < L ? my_q : L - 1;
    const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
    const __bf16* op = (const __bf16*)p.dout + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qf[ks] = *(const bf16x8*)(qp + ks * 16);
      of[ks] = *(const bf16x8*)(op + ks * 16);
    }
    const long li = lse_index(p, s, h, seq0, qr, T, VARLEN);
    lse2 = p.lse[li] * kLog2e;
    dq_d = p.dsum[li];
  }
  f32x16 dq[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) dq[i] = f32x16{};
  const float c = p.scale_log2;

  wait_vmem();
  __syncthreads();
  const int g16 = lane & 15;
  auto step = [&](char FA_LDS* cur, char FA_LDS* nxt, const int kt) __attribute__((always_inline)) {
    if (kt + 1 < n_kv) issue(kt + 1, nxt);
    const int k0 = kt * Q_BN;
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      const char FA_LDS* ktile = cur;
      const char FA_LDS* vtile = cur + S::TILEB;
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      f32x16 pacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + l32;
          const int off = row * S::ROWB + (((2 * ks + hl) ^ lds_swz<D>(row)) * 16);
          sacc[kb] = mfma32(lds_read16(ktile + off), qf[ks], sacc[kb]);
          pacc[kb] = mfma32(lds_read16(vtile + off), of[ks], pacc[kb]);
        }
      }
      const bool need_mask = (k0 + Q_BN > L) || (CAUSAL && (k0 + Q_BN - 1 > qw0));
      bf16x8 db8[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8 b;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            float d2[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int r = 8 * half + e + z;
              float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][r], c, -lse2));
              if (need_mask) {
                const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
                const bool dead = (key >= L) || (CAUSAL && key > my_q);
                pe = dead ? 0.f : pe;
              }
              d2[z] = pe * (pacc[kb][r] - dq_d);
            }
            const bf16x2 t2 = pack_bf16(d2[0], d2[1]);
            b[e] = t2[0];
            b[e + 1] = t2[1];
          }
          db8[kb * 2 + half] = b;
        }
      // dQ^T += K^T dS^T
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r0 = 16 * t + 4 * hl + (g16 >> 2), r1 = r0 + 8;
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
          const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
          const int o0 = r0 * S::ROWB + ((chunk ^ lds_swz<D>(r0)) * 16) + sub;
          const int o1 = r1 * S::ROWB + ((chunk ^ lds_swz<D>(r1)) * 16) + sub;
          dq[db] = mfma32(cat(lds_read_tr(ktile + o0), lds_read_tr(ktile + o1)), db8[t], dq[db]);
        }
      }
    }
    wait_vmem();
    __syncthreads();
  };
  for (int kt = 0; kt < n_kv; kt += 2) {
    step(stage0, stage1, kt);
    if (kt + 1 < n_kv) step(stage1, stage0, kt + 1);
  }
  char FA_LDS* st = (wave < 2 ? stage0 : stage1) + (wave & 1) * 32 * S::OROWB;
  __bf16* dqb = (__bf16*)p.dq + ((long)seq0 * p.Hq + h) * D;
  store_rows_bf16<D>(st, dq, p.scale, dqb, q_stride, qw0, L, lane);
}

// ---------------------------------------------------------------------------
// launcher
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, bool VARLEN>
static hipError_t launch_bwd_t(const BwdParams& p, int stages, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (stages & 1) {
    const long rows = (long)p.B * p.N * p.Hq;    // upper bound (packed: T <= B * N)
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((bwd_dsum_kernel<D, VARLEN>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       stream, p, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 2) {
    const int n_kt = (p.N + KV_BN - 1) / KV_BN;
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, VARLEN>), dim3(n_kt * p.B * p.Hkv), dim3(NTHREADS), 0, stream,
                       p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (stages & 4) {
    const int n_qt = (p.N + Q_BM - 1) / Q_BM;
    const int items = n_qt * p.B * p.Hq;
    const int xg = p.G;
    const int grid = (items + 8 * xg - 1) / (8 * xg) * (8 * xg);
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, VARLEN>), dim3(grid), dim3(NTHREADS), 0, stream, p, n_qt, xg);
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

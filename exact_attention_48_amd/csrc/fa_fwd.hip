// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// One workgroup computes BM = 128 query rows of one (sequence, query head);
// each of its 4 waves owns 32 rows. The loop walks the key/value tiles of
// BN = 64 keys (tiling with an online softmax, so the N x N score matrix never
// leaves the chip: "FlashAttention-4 Conquers Asymmetric GPU Hardware Scaling",
// podcast.app episode page, second paragraph of the description).
//
// Per key/value tile and wave:
//   S^T[64 x 32] = K_tile[64 x d] * Q_w^T[d x 32]   bf16 MFMA 32x32x16, fp32 acc
//     -> every lane holds the scores of ONE query for 32 keys, so the row max
//        is an in-lane max plus one v_permlane32_swap with the partner lane
//   masking only on tiles that cross the causal diagonal or the sequence end
//   conditional rescaling: the running max m (and with it O and the row sum l)
//     is only moved when a row's max grows by more than tau (log2 units);
//     otherwise the stale m is kept, which is exact because O and l always
//     share the same m (conditional online softmax rescaling: daily.dev
//     "Summary"; FA4 abstract on the zhuanzhiai.com page)
//   P = exp2(S * c - m * c), c = scale * log2(e), hardware v_exp_f32 or the
//     FMA-pipe polynomial (software exponential: daily.dev "Summary")
//   l += rowsum(P) (per-lane partial sums, combined once at the end)
//   O^T[d x 32] += V^T[d x 64] * P^T[64 x 32]        bf16 MFMA; P stays in
//     registers as the B operand; V^T comes from row-major V in LDS through
//     the transposing ds_read_b64_tr_b16
// K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no register
// staging), double-buffered so the next tile loads while this one computes.
//
// Work order: query tiles are ordered heaviest first (causal: the last tiles
// of a sequence see the most keys) -- longest-processing-time-first (daily.dev
// "Summary") -- and the G query heads of one K/V head are kept on one XCD
// (workgroups are dealt to the 8 XCDs round-robin) so they share its L2.
#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int BM = 128;
constexpr int BN = 64;
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;

template <int D>
struct Smem {
  static constexpr int ROWB = D * 2;                 // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;            // bytes per K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;           // K then V
  static constexpr int OROWB = ROWB + 16;            // O staging row stride
  static_assert(2 * 32 * OROWB <= STAGEB, "two waves' O staging must fit in one stage");
};

// Issue the HBM -> LDS copy of key/value tile `kt` (rows clamped to L-1 so no
// access leaves the sequence; those columns are masked).
template <int D>
__device__ __forceinline__ void load_kv_tile(char FA_LDS* stage, const char* kbase, const char* vbase,
                                             long row_stride_b, int kt, int L, int wave, int lane) {
  constexpr int ROWB = Smem<D>::ROWB;
  constexpr int LPR = ROWB / 16;                 // lanes per row
  constexpr int RPI = 64 / LPR;                  // rows per wave instruction (1 KiB)
  constexpr int NI = BN / RPI;                   // instructions per tile
  constexpr int PER_WAVE = NI / NWAVES;
  const int r_in = lane / LPR;
  const int pos = lane % LPR;
#pragma unroll
  for (int u = 0; u < PER_WAVE; ++u) {
    const int ins = wave * PER_WAVE + u;
    const int row = ins * RPI + r_in;
    int grow = kt * BN + row;
    grow = grow < L ? grow : L - 1;
    const long goff = (long)grow * row_stride_b;
    const int kchunk = pos ^ lds_swz<D>(row);
    const int vchunk = pos ^ lds_swz<D>(row);
    g2lds16(kbase + goff + kchunk * 16, stage + ins * 1024);
    g2lds16(vbase + goff + vchunk * 16, stage + Smem<D>::TILEB + ins * 1024);
  }
}

}  // namespace

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const FwdParams p) {
  using S = Smem<D>;
  constexpr int KSTEPS = D / 16;       // MFMA k-steps of S = K Q^T
  constexpr int DBLK = D / 32;         // 32-row blocks of O^T
  // Two distinct LDS objects (not two halves of one array): the compiler then
  // knows the in-flight HBM->LDS copy into one stage cannot alias reads of the
  // other and does not stall those reads on the copy.
  __shared__ __attribute__((aligned(1024))) char stage0_raw[S::STAGEB];
  __shared__ __attribute__((aligned(1024))) char stage1_raw[S::STAGEB];
  char FA_LDS* stage0 = (char FA_LDS*)stage0_raw;
  char FA_LDS* stage1 = (char FA_LDS*)stage1_raw;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hl = lane >> 5;            // which half of the wave (0/1)
  const int l32 = lane & 31;

  // ---- work item -> (sequence, head, query tile) ----
  int w = blockIdx.x;
  if (p.xcd_group > 0) {
    // workgroup i runs on XCD i % 8; give XCD x the item groups x, x+8, ...
    const int xcd = w & 7, j = w >> 3;
    w = (8 * (j / p.xcd_group) + xcd) * p.xcd_group + (j % p.xcd_group);
  }
  if (w >= p.n_items) return;
  const int per_level = p.B * p.Hq;
  const int lvl = w / per_level;
  const int rr = w - lvl * per_level;
  const int s = rr / p.Hq;
  const int h = rr - s * p.Hq;
  const int qt = p.lpt ? (p.n_qtiles - 1 - lvl) : lvl;
  const int hkv = h / p.G;

  int seq0, L;
  if constexpr (VARLEN) {
    seq0 = p.cu_seqlens[s];
    L = p.cu_seqlens[s + 1] - seq0;
  } else {
    seq0 = s * p.N;
    L = p.N;
  }
  const int q0 = qt * BM;
  if (q0 >= L) return;
  const int qw0 = q0 + wave * 32;                     // first row of this wave

  const long q_row_stride = (long)p.Hq * D;           // elements
  const long kv_row_stride_b = (long)p.Hkv * D * 2;   // bytes
  const char* kbase = (const char*)p.k + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const char* vbase = (const char*)p.v + ((long)seq0 * p.Hkv + hkv) * D * 2;

  const int kv_end = CAUSAL ? min(L, q0 + BM) : L;    // keys this tile can see
  const int n_kv = (kv_end + BN - 1) / BN;

  // ---- prefetch tile 0 ----
  load_kv_tile<D>(stage0, kbase, vbase, kv_row_stride_b, 0, L, wave, lane);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query qw0 + l32 ----
  bf16x8 qf[KSTEPS];
  {
    const int qrow = qw0 + l32;
    const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + qrow) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (qrow < L) qf[ks] = *(const bf16x8*)(qp + ks * 16);
      else qf[ks] = bf16x8{};
    }
  }

  const float c = p.scale_log2;
  const float tau = p.tau;
  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;     // running max of raw scores (stale by < tau/c)
  float l_run = 0.f;           // partial row sum over this lane's keys
  const int my_q = qw0 + l32;  // this lane's query (local position)

  wait_vmem();
  __syncthreads();

  auto step = [&](char FA_LDS* cur, char FA_LDS* nxt, const int kt) __attribute__((always_inline)) {
    if (kt + 1 < n_kv) load_kv_tile<D>(nxt, kbase, vbase, kv_row_stride_b, kt + 1, L, wave, lane);

    const int k0 = kt * BN;
    // causal: skip tiles entirely above this wave's rows
    const bool active = !CAUSAL || (k0 <= qw0 + 31);
    if (active) {
      // ---- S^T = K Q^T ----
      f32x16 sacc[2] = {f32x16{}, f32x16{}};
      const char FA_LDS* kt_lds = cur;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int row = kb * 32 + l32;
          const int chunk = (2 * ks + hl) ^ lds_swz<D>(row);
          const bf16x8 a = lds_read16(kt_lds + row * S::ROWB + chunk * 16);
          sacc[kb] = mfma32(a, qf[ks], sacc[kb]);
        }
      }
      // ---- mask (diagonal / sequence end only) ----
      const bool need_mask = (k0 + BN > L) || (CAUSAL && (k0 + BN - 1 > qw0));
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
            const bool dead = (key >= L) || (CAUSAL && key > my_q);
            if (dead) sacc[kb][r] = -INFINITY;
          }
      }
      // ---- row max and conditional rescale ----
      float mx = sacc[0][0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[0][r]);
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[1][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const bool grow = (m_new - m_run) * c > tau;   // false when both are -inf
      if (wave_any(grow)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : exp2_sel<0>((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DBLK; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[i][r] *= alpha;
        m_run = m_new;
      }
      const float mc = (m_run == -INFINITY) ? 0.f : m_run * c;
      // ---- P = exp2(S c - m c), row sums, bf16 pack ----
      bf16x8 pb[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          float pv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pv[e] = exp2_sel<EXPMODE>(__builtin_fmaf(sacc[kb][8 * half + e], c, -mc));
            l_run += pv[e];
          }
          bf16x8 b;
#pragma unroll
          for (int e = 0; e < 8; e += 2) {
            const bf16x2 t = pack_bf16(pv[e], pv[e + 1]);
            b[e] = t[0];
            b[e + 1] = t[1];
          }
          pb[kb * 2 + half] = b;
        }
      }
      // ---- O^T += V^T P^T ----
      const char FA_LDS* vt_lds = cur + S::TILEB;
      const int g16 = lane & 15;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kbase_row = 16 * t + 4 * hl + (g16 >> 2);   // key row for the e=0..3 read
#pragma unroll
        for (int db = 0; db < DBLK; ++db) {
          const int dcol = db * 32 + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
          const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
          const int r0 = kbase_row, r1 = kbase_row + 8;
          const bf16x4 lo = lds_read_tr(vt_lds + r0 * S::ROWB + ((chunk ^ lds_swz<D>(r0)) * 16) + sub);
          const bf16x4 hi = lds_read_tr(vt_lds + r1 * S::ROWB + ((chunk ^ lds_swz<D>(r1)) * 16) + sub);
          oacc[db] = mfma32(cat(lo, hi), pb[t], oacc[db]);
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

  // ---- epilogue: O = O / l, LSE = m * scale + ln(l) ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // stage O (bf16) through LDS so global stores are whole 16-byte row segments
  char FA_LDS* ost = (wave < 2 ? stage0 : stage1) + (wave & 1) * 32 * S::OROWB;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int dcol = db * 32 + 8 * g + 4 * hl;
      const bf16x2 a = pack_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      const bf16x2 b = pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      bf16x4 v4 = __builtin_shufflevector(a, b, 0, 1, 2, 3);
      *(bf16x4 FA_LDS*)(ost + l32 * S::OROWB + dcol * 2) = v4;
    }
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int CPR = D / 8;                 // 16-byte chunks per row
    constexpr int PER_LANE = 32 * CPR / 64;
    __bf16* obase = (__bf16*)p.o + ((long)seq0 * p.Hq + h) * D;
#pragma unroll
    for (int u = 0; u < PER_LANE; ++u) {
      const int idx = u * 64 + lane;
      const int row = idx / CPR, ch = idx % CPR;
      const int q = qw0 + row;
      const bf16x8 v8 = *(const bf16x8 FA_LDS*)(ost + row * S::OROWB + ch * 16);
      if (q < L) *(bf16x8*)(obase + (long)q * q_row_stride + ch * 8) = v8;
    }
  }
  if (hl == 0 && my_q < L) {
    const float lse = (m_run == -INFINITY) ? -INFINITY : (m_run * c + __log2f(l_tot)) * kLn2;
    long li;
    if constexpr (VARLEN) li = (long)h * p.cu_seqlens[p.B] + seq0 + my_q;
    else li = ((long)s * p.Hq + h) * p.N + my_q;
    p.lse[li] = lse;
  }
}

// ---- instantiations and launcher ----

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
static hipError_t launch_fwd(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, EXPMODE>), dim3(grid), dim3(NTHREADS), 0, stream, p);
  return hipGetLastError();
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

int fwd_block_m() { return BM; }

hipError_t fwd_launch(FwdParams p, int d, int causal, int varlen, int expmode, hipStream_t stream) {
  p.n_qtiles = (p.N + BM - 1) / BM;
  p.n_items = p.n_qtiles * p.B * p.Hq;
  if (p.n_items == 0) return hipSuccess;
  int grid = p.n_items;
  if (p.xcd_group > 0) {
    const int g8 = 8 * p.xcd_group;
    grid = (p.n_items + g8 - 1) / g8 * g8;
  }
  if (d == 128) return launch_fwd_d<128>(p, grid, causal, varlen, expmode, stream);
  return launch_fwd_d<64>(p, grid, causal, varlen, expmode, stream);
}

}  // namespace fa

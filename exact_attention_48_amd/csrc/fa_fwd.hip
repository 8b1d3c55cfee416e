// fa_fwd.hip -- exact attention forward for gfx950 (MI355X).
//
// One workgroup computes BM = 256 query rows of one (sequence, query head)
// with 8 waves of 32 rows each. The loop walks the key/value tiles of BN = 64
// keys (tiling with an online softmax, so the N x N score matrix never leaves
// the chip: "FlashAttention-4 Conquers Asymmetric GPU Hardware Scaling",
// podcast.app episode page, second paragraph of the description).
//
// Per key/value tile j and wave:
//   S^T[64 x 32] = K_j[64 x d] * Q_w^T[d x 32]     bf16 MFMA 32x32x16, fp32 acc
//     -> every lane holds the scores of ONE query for 32 keys, so the row max
//        is an in-lane max plus one v_permlane32_swap with the partner lane
//   masking only on tiles that cross the causal diagonal or the sequence end
//   conditional rescaling: the running max m (and with it O and the row sum l)
//     only moves when a row's max grows by more than tau (log2 units);
//     otherwise the stale m is kept, which is exact because O and l always
//     share the same m (conditional online softmax rescaling: daily.dev
//     "Summary"; FA4 abstract on the zhuanzhiai.com page)
//   P = exp2(S c - m c), c = scale * log2(e), hardware v_exp_f32 or the
//     FMA-pipe polynomial (software exponential: daily.dev "Summary")
//   l += rowsum(P) (per-lane partial sums, combined once at the end)
//   O^T[d x 32] += V^T[d x 64] * P^T[64 x 32]      bf16 MFMA; P stays in
//     registers as the B operand; V^T comes from row-major V in LDS through
//     the transposing ds_read_b64_tr_b16
//
// Ping-pong (the MMA/softmax overlap of the pages' pipeline, daily.dev
// "Summary"): the 8 waves form two groups of 4, one wave of each group on
// every SIMD. Time is cut into phases by workgroup barriers; in a phase one
// group runs an MFMA phase (O += V_{j-1} P_{j-1}, then S_j = K_j Q^T) while
// the other runs the VALU phase of its previous tile (mask, max, rescale,
// exp2, row sums, bf16 pack). The groups are one phase apart, so every SIMD
// always has one wave feeding the matrix core and one feeding the VALU.
//
// K and V tiles travel HBM -> LDS with global_load_lds_dwordx4 (no register
// staging) into two-deep rings of distinct LDS objects; a copy issued in one
// phase is waited for at the end of the next, and the phase barriers carry
// no memory fence (that would drain the copies still in flight).
//
// Work order: query tiles are ordered heaviest first (causal: the last tiles
// of a sequence see the most keys) -- longest-processing-time-first (daily.dev
// "Summary") -- and the G query heads of one K/V head are kept on one XCD
// (workgroups are dealt to the 8 XCDs round-robin) so they share its L2.
#include <type_traits>

#include "fa_device.h"
#include "fa_kernels.h"

namespace fa {

namespace {

constexpr int BM = 256;
constexpr int BN = 64;
constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;

template <int D>
struct Geo {
  static constexpr int ROWB = D * 2;              // bytes per K/V row
  static constexpr int TILEB = BN * ROWB;         // bytes per K or V tile
  static constexpr int KSTEPS = D / 16;           // MFMA k-steps of S = K Q^T
  static constexpr int DBLK = D / 32;             // 32-row blocks of O^T
  static_assert(2 * 32 * ROWB <= TILEB, "two waves' O staging must fit in one tile buffer");
};

// HBM -> LDS copy of one K or V tile (BN rows x D, rows clamped to L-1 on the
// tail tile; those columns are masked). Each wave of group 0 moves PER_WAVE KiB.
template <int D>
struct TileCopy {
  static constexpr int LPR = Geo<D>::ROWB / 16;   // lanes per row
  static constexpr int RPI = 64 / LPR;            // rows per wave instruction (1 KiB)
  static constexpr int NI = BN / RPI;             // instructions per tile
  static constexpr int COPY_WAVES = NWAVES / 2;   // the waves of ping-pong group 0 move the tiles
  static constexpr int PER_WAVE = NI / COPY_WAVES;
  static_assert(PER_WAVE * COPY_WAVES == NI, "tile copy must split evenly over the waves");
  unsigned off[PER_WAVE];                         // row * stride + swizzled chunk * 16
  int wave, lane;

  __device__ __forceinline__ int row(int u) const { return (wave * PER_WAVE + u) * RPI + lane / LPR; }
  __device__ __forceinline__ unsigned chunk16(int u) const {
    return (unsigned)(((lane % LPR) ^ lds_swz<D>(row(u))) * 16);
  }
  __device__ __forceinline__ void init(int wave_, int lane_, unsigned stride) {
    wave = wave_;
    lane = lane_;
#pragma unroll
    for (int u = 0; u < PER_WAVE; ++u) off[u] = (unsigned)row(u) * stride + chunk16(u);
  }
  // `base` points at row 0 of this head's K (or V); kt is the tile index.
  __device__ __forceinline__ void issue(char FA_LDS* tile, const char* base, long stride, int kt, int L) const {
    const char* tb = base + (long)kt * BN * stride;
    char FA_LDS* dst = tile + wave * PER_WAVE * 1024;
    if (kt * BN + BN <= L) {
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        // keep the 64-bit address out of loop-invariant code motion: uniform
        // base + 32-bit lane offset is the SGPR-base addressing form
        unsigned o = off[u];
        asm volatile("" : "+v"(o));
        g2lds16(tb + o, dst + u * 1024);
      }
    } else {
      const int last = L - 1 - kt * BN;
#pragma unroll
      for (int u = 0; u < PER_WAVE; ++u) {
        const int r = min(row(u), last);
        g2lds16(tb + ((unsigned)r * (unsigned)stride + chunk16(u)), dst + u * 1024);
      }
    }
  }
};

}  // namespace

template <int D, bool CAUSAL, bool VARLEN, int EXPMODE>
__global__ __attribute__((amdgpu_flat_work_group_size(NTHREADS, NTHREADS), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_kernel(const FwdParams p) {
  using G = Geo<D>;
  constexpr int KSTEPS = G::KSTEPS;
  constexpr int DBLK = G::DBLK;
  constexpr int ROWB = G::ROWB;
  __shared__ __attribute__((aligned(1024))) char k0_raw[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char k1_raw[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char v0_raw[G::TILEB];
  __shared__ __attribute__((aligned(1024))) char v1_raw[G::TILEB];
  char FA_LDS* const kbuf[2] = {(char FA_LDS*)k0_raw, (char FA_LDS*)k1_raw};
  char FA_LDS* const vbuf[2] = {(char FA_LDS*)v0_raw, (char FA_LDS*)v1_raw};

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;           // ping-pong group: waves 0-3 / 4-7 (one of each per SIMD)
  const int hl = lane >> 5;            // which half of the wave (0/1)
  const int l32 = lane & 31;
  const int g16 = lane & 15;

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
  const int my_q = qw0 + l32;                         // this lane's query (local position)

  const long q_row_stride = (long)p.Hq * D;           // elements
  const long kv_stride = (long)p.Hkv * D * 2;         // bytes per token row of K/V
  const char* kbase = (const char*)p.k + ((long)seq0 * p.Hkv + hkv) * D * 2;
  const char* vbase = (const char*)p.v + ((long)seq0 * p.Hkv + hkv) * D * 2;

  const int kv_end = CAUSAL ? min(L, q0 + BM) : L;    // keys this workgroup can see
  const int n_kv = (kv_end + BN - 1) / BN;
  // tiles this wave computes (causal: stop after the tile holding its last row)
  const int n_w = CAUSAL ? min(n_kv, (qw0 + 31) / BN + 1) : n_kv;

  TileCopy<D> copy;
  copy.init(wave & 3, lane, (unsigned)kv_stride);
  if (grp == 0) copy.issue(kbuf[0], kbase, kv_stride, 0, L);

  // ---- Q fragments (B operand of S^T = K Q^T): lane holds query my_q ----
  bf16x8 qf[KSTEPS];
  {
    const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + my_q) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      if (my_q < L) qf[ks] = *(const bf16x8*)(qp + ks * 16);
      else qf[ks] = bf16x8{};
    }
  }

  // Loop-invariant per-lane LDS read offsets. The swizzle only XORs chunk
  // bits, so the offsets of other k-steps / d-blocks are these XOR a constant:
  //   K fragment of k-step ks (A operand of S^T): koff ^ (ks << 5), +32 rows for key block 1
  //   V^T fragment of d-block db (keys +0..3 / +8..11): voff[i] ^ (db << 6), +16 rows per key step t
  const int koff = l32 * ROWB + ((hl ^ lds_swz<D>(l32)) << 4);
  int voff[2];
  {
    const int dcol = 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
    const int chunk = dcol >> 3, sub = (dcol & 7) * 2;
    const int r0 = 4 * hl + (g16 >> 2), r1 = r0 + 8;
    voff[0] = r0 * ROWB + ((chunk ^ lds_swz<D>(r0)) * 16) + sub;
    voff[1] = r1 * ROWB + ((chunk ^ lds_swz<D>(r1)) * 16) + sub;
  }

  const float c = p.scale_log2;
  const float tau = p.tau;
  f32x16 oacc[DBLK];
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  float m_run = -INFINITY;     // running max of raw scores (stale by at most tau / c)
  float l_run = 0.f;           // partial row sum over this lane's keys
  f32x16 sacc[2];              // S^T of the tile between its MFMA phase and its VALU phase
  bf16x8 pb[4];                // P of the tile between its VALU phase and the next MFMA phase

  // MFMA phase m: O += V_{m-1} P_{m-1} (if the wave computed tile m-1), then
  // S_m = K_m Q^T (if the wave computes tile m).
  auto mfma_phase = [&](const char FA_LDS* kb, const char FA_LDS* vb, int m) __attribute__((always_inline)) {
    // One stream of MFMA steps: NPV steps of O += V^T P^T (t = i / DBLK,
    // db = i % DBLK), then NQK steps of S^T = K Q^T (ks = j / 2, key block
    // j % 2). A operands are read PF steps ahead through a small register
    // queue; a scheduling fence after each step keeps the compiler from
    // hoisting every read of the phase (register pressure).
    constexpr int NPV = 4 * DBLK, NQK = 2 * KSTEPS, PF = 4;
    const bool do_pv = m >= 1 && m - 1 < n_w;
    const bool do_qk = m < n_w;
    const int first = do_pv ? 0 : NPV;
    const int last = do_qk ? NPV + NQK : NPV;
    auto fetch = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < NPV) {
        const int t = i / DBLK, db = i % DBLK;
        return cat(lds_read_tr(vb + (voff[0] ^ (db << 6)) + t * 16 * ROWB),
                   lds_read_tr(vb + (voff[1] ^ (db << 6)) + t * 16 * ROWB));
      }
      const int j = i - NPV;
      return lds_read16(kb + (koff ^ ((j >> 1) << 5)) + (j & 1) * 32 * ROWB);
    };
    auto step = [&](int i, const bf16x8& a) __attribute__((always_inline)) {
      if (i < NPV) {
        oacc[i % DBLK] = mfma32(a, pb[i / DBLK], oacc[i % DBLK]);
      } else {
        const int j = i - NPV;
        sacc[j & 1] = mfma32(a, qf[j >> 1], sacc[j & 1]);
      }
    };
    (void)first;
    (void)last;
    if (do_pv) {
      bf16x8 q[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) q[i] = fetch(i);
#pragma unroll
      for (int i = 0; i < NPV; ++i) {
        const bf16x8 a = q[i % PF];
        if (i + PF < NPV) q[i % PF] = fetch(i + PF);
        step(i, a);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (do_qk) {
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
      bf16x8 q[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) q[i] = fetch(NPV + i);
#pragma unroll
      for (int i = NPV; i < NPV + NQK; ++i) {
        const bf16x8 a = q[(i - NPV) % PF];
        if (i + PF < NPV + NQK) q[(i - NPV) % PF] = fetch(i + PF);
        step(i, a);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // VALU phase of tile m: mask, row max, conditional rescale, P = exp2(S c - m c).
  auto valu_phase = [&](int m) __attribute__((always_inline)) {
    if (m >= n_w) return;
    const int k0 = m * BN;
    if ((k0 + BN > L) || (CAUSAL && (k0 + BN - 1 > qw0))) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + 8 * (r >> 2) + 4 * hl + (r & 3);
          const bool dead = (key >= L) || (CAUSAL && key > my_q);
          if (dead) sacc[kb][r] = -INFINITY;
        }
    }
    float ma = fmaxf(sacc[0][0], sacc[0][1]), mb = fmaxf(sacc[1][0], sacc[1][1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      ma = fmaxf(ma, fmaxf(sacc[0][r], sacc[0][r + 1]));
      mb = fmaxf(mb, fmaxf(sacc[1][r], sacc[1][r + 1]));
    }
    const float mx = pair_max(fmaxf(ma, mb));
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
    float lsum[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        float pv[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pv[e] = exp2_sel<EXPMODE>(__builtin_fmaf(sacc[kb][8 * half + e], c, -mc));
        lsum[kb * 2 + half] = ((pv[0] + pv[1]) + (pv[2] + pv[3])) + ((pv[4] + pv[5]) + (pv[6] + pv[7]));
        bf16x8 b;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          const bf16x2 t = pack_bf16(pv[e], pv[e + 1]);
          b[e] = t[0];
          b[e + 1] = t[1];
        }
        pb[kb * 2 + half] = b;
      }
    l_run += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  };

  wait_vmem();
  __syncthreads();

  // Both groups run the same sequence of phases; group 1 starts one barrier
  // later (and group 0 ends with one extra barrier), so when group 0 is in its
  // MFMA phase m, group 1 is in its VALU phase m-1, and the other way round.
  // Iteration m of a wave (PAR = m & 1 selects the ring slots):
  //   group 0 copies K_{m+1} -> kbuf[1-PAR] and V_m -> vbuf[PAR];
  //   MFMA phase m (K_m in kbuf[PAR], V_{m-1} in vbuf[1-PAR]); barrier;
  //   VALU phase m; group 0 waits for its copies; barrier.
  // A slot is overwritten only after its previous tile's last reader (group 1,
  // one phase behind) has passed the barrier that ends that read.
  auto iter = [&](auto par_tag, const int m) __attribute__((always_inline)) {
    constexpr int PAR = decltype(par_tag)::value;
    if (grp == 0) {
      if (m + 1 < n_kv) copy.issue(kbuf[1 - PAR], kbase, kv_stride, m + 1, L);
      if (m < n_kv) copy.issue(vbuf[PAR], vbase, kv_stride, m, L);
    }
    mfma_phase(kbuf[PAR], vbuf[1 - PAR], m);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(63));
    barrier_no_fence();
    valu_phase(m);
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    barrier_no_fence();
  };
  if (grp == 1) barrier_no_fence();
  for (int m = 0; m <= n_kv; m += 2) {
    iter(std::integral_constant<int, 0>{}, m);
    if (m + 1 <= n_kv) iter(std::integral_constant<int, 1>{}, m + 1);
  }
  if (grp == 0) barrier_no_fence();

  // ---- epilogue: O = O / l, LSE = m * scale + ln(l) ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  // Stage O (bf16) through LDS so global stores are whole 16-byte row
  // segments; row r's chunk ch sits at chunk (ch ^ r) mod (D / 8).
  constexpr int CPR = D / 8;                   // 16-byte chunks per row
  char FA_LDS* ost = (wave < 2 ? kbuf[0] : wave < 4 ? kbuf[1] : wave < 6 ? vbuf[0] : vbuf[1]) +
                     (wave & 1) * 32 * ROWB;
#pragma unroll
  for (int db = 0; db < DBLK; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int ch = db * 4 + g;               // chunk holding d = 8 ch .. 8 ch + 7
      const bf16x2 a = pack_bf16(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv);
      const bf16x2 b = pack_bf16(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv);
      *(bf16x4 FA_LDS*)(ost + l32 * ROWB + ((ch ^ l32) & (CPR - 1)) * 16 + hl * 8) =
          __builtin_shufflevector(a, b, 0, 1, 2, 3);
    }
  __builtin_amdgcn_wave_barrier();
  {
    constexpr int PER_LANE = 32 * CPR / 64;
    __bf16* obase = (__bf16*)p.o + ((long)seq0 * p.Hq + h) * D;
#pragma unroll
    for (int u = 0; u < PER_LANE; ++u) {
      const int idx = u * 64 + lane;
      const int row = idx / CPR, ch = idx % CPR;
      const int q = qw0 + row;
      const bf16x8 v8 = *(const bf16x8 FA_LDS*)(ost + row * ROWB + ((ch ^ row) & (CPR - 1)) * 16);
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

// fa_fwd_pp.hip -- exact attention forward for gfx950, d = 128, bf16: two
// waves per SIMD that take turns on the matrix core.
//
// The pages overlap the softmax of one tile with the matrix products of
// another by alternating two groups of warps between the two kinds of work
// (daily.dev "Summary" of the Together AI post; co-design list of the
// phantomic12 summary). On gfx950 a wave issues at most
// one instruction at a time, so one wave per SIMD that interleaves its own
// MFMAs with its own softmax arithmetic leaves the matrix core idle while the
// vector instructions issue. With two waves per SIMD, one wave's MFMAs run
// beside the other wave's vector work: measured on this GPU, a wave issuing
// back-to-back 32x32x16 MFMAs keeps 97-99 % of the MFMA rate while a second
// wave on the same SIMD issues 4-5 softmax-type vector instructions per MFMA.
//
// Workgroup: 8 waves, 256 query rows of one (sequence, query head), 32 per
// wave (one 32-query MFMA block). Waves 0-3 form group A, waves 4-7 group B;
// the hardware places waves w and w + 4 on the same SIMD. Keys and values
// stream in tiles of BN = 64 through a ring of 4 LDS stages. For tile i a wave
// runs two phases:
//   GEMM(i-1)  : S_i^T = K_i Q^T (16 MFMAs, key in the row, query in the lane)
//                and O^T += V_{i-1}^T P_{i-1}^T (16 MFMAs, P from registers,
//                V^T through the transposing ds_read_b64_tr_b16);
//   SOFTMAX(i) : P_i = exp2(S_i c - m c), row sums, bf16 pack (vector only).
// Group B runs one phase behind group A. The workgroup synchronises once per
// slot of two phases, and the two groups take the slot's phases in opposite
// orders, so that one wave of each SIMD is in a GEMM phase while the other is
// in a softmax phase:
//   slot i : A  GEMM(i-1), SOFTMAX(i)      B  SOFTMAX(i-1), GEMM(i-1)
// (one barrier per slot measured 2-5 % faster than one per phase: the
// order of the code keeps the groups apart, and half the barriers go). The
// GEMM wave raises its priority (s_setprio) so the arbiter issues its MFMAs
// first and the softmax wave fills the remaining issue slots.
//
// Tile copies (HBM -> LDS without register staging, buffer_load ... lds) go out
// from the softmax phases only, the four 1 KiB instructions of a wave's share
// just before the phase's exponentials (measured 0.4 % faster than one per 16
// exponentials): a copy instruction holds its wave at issue for about 65-100
// clocks (measured), which in a GEMM phase would stall the MFMA stream. In slot
// i both groups issue their shares of tile i+2 (A before SOFTMAX(i), B before
// SOFTMAX(i-1)), into the stage of tile i-2, which the slots before last read;
// at the end of slot i every wave waits for its share of tile i+1, and the
// barrier makes the whole tile visible before slot i+1 reads it. The GEMM phase
// starts with the P V MFMAs, whose first V^T fragments the wave read at the end
// of its softmax phase.
//
// LDS layout and addressing: one 128 KiB array, the 4 V stages in its lower
// 64 KiB and the 4 K stages in the upper 64 KiB, 16 KiB each. Every fragment
// read is a per-lane base register (the swizzled offset of the lane's row and
// chunk, one per K k-step and per V^T d-block and half: 16 registers, made
// opaque to the compiler once) plus an immediate offset below 64 KiB (stage,
// key block, key step), so no address is recomputed or held per stage. The
// copies are issued by inline asm: the compiler never sees them, so it adds no
// wait for them before the (opaque-address) fragment reads; the explicit waits
// and barriers above order them.
//
// Online softmax with conditional rescaling: as in the one-wave kernel, each
// row's max m stays at its first tile's max for the whole pass, and only a row
// sum l above 2^tau (or not finite) at the end sends the workgroup through a
// tracking pass (true row maxima) and an exact pass (the threshold-gated
// rescale of the pages, daily.dev "Summary" and the FA4 abstract on the
// zhuanzhiai.com page, taken out of the loop).
#include "fa_device.h"
#include "fa_kernels.h"
#include "fa_order.h"
#include "fa_tiles.h"

namespace fa {

using namespace tiles;

namespace {

constexpr int PP_WAVES = 8;
constexpr int PP_THREADS = 64 * PP_WAVES;
constexpr int PP_WQ = 32;                    // queries per wave
constexpr int PP_BM = PP_WAVES * PP_WQ;      // queries per workgroup
constexpr int PP_BN = 64;                    // keys per tile
constexpr int PP_D = 128;
constexpr int PP_TILEB = PP_BN * PP_D * 2;   // one K or V tile in LDS
constexpr int PP_PF = 4;                     // operand fragments read ahead

}  // namespace

// SPLIT: split-KV partial results (uniform batches): work item (sequence,
// key chunk, query head, query tile) over the chunk's keys [kbeg, kend) only,
// query i at key position i + q_off for the causal mask, fp32 O_p and LSE_p out.
template <bool CAUSAL, bool VARLEN, int EXPMODE, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(PP_THREADS, PP_THREADS), amdgpu_waves_per_eu(2, 2)))
void fa_fwd_pp_kernel(const FwdParams p) {
  static_assert(!(SPLIT && VARLEN), "split-KV partial results are for uniform batches");
  constexpr int D = PP_D;
  constexpr int BN = PP_BN;
  constexpr int KSTEPS = D / 16;              // S^T k-steps
  constexpr int DBLK = D / 32;                // O^T d-blocks
  constexpr int KT = BN / 16;                 // key steps of P V
  constexpr int OPS = 4;                      // copy instructions per tile and wave (2 K rows groups, 2 V)
  static_assert(32 * (D * 2 + 16) <= PP_TILEB, "a wave's output staging must fit in one tile object");
  __shared__ __attribute__((aligned(1024))) char lds[8 * PP_TILEB];
  __shared__ int over_flag[PP_WAVES];
  constexpr int VREG = 0;                     // V stages: bytes [0, 64 KiB)
  constexpr int KREG = 4 * PP_TILEB;          // K stages: bytes [64 KiB, 128 KiB)
  const unsigned lds0 = (unsigned)(size_t)lds;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const bool grp_a = wave < 4;
  const int hl = lane >> 5, l32 = lane & 31;

  // ---- work item -> (sequence s, query head h, query tile qt) (fa_order.h) ----
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
  int seq0, L, kseq0, Lk;                     // queries: rows seq0.., L of them; keys: kseq0.., Lk
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
  // keys of this work item: [kbeg, kend) (a split call's chunk); query i sits
  // at key position i + q_off for the causal mask
  const int q_off = SPLIT ? p.q_off : 0;
  const int kbeg = SPLIT ? min(sp * p.chunk, Lk) : 0;
  const int kend = SPLIT ? (int)min((long)(sp + 1) * p.chunk, (long)Lk) : Lk;
  const int q0 = qt * PP_BM;
  if (q0 >= L) return;
  const int qw0 = q0 + wave * PP_WQ;          // first query of this wave
  const int my_q = qw0 + l32;
  const int kv_end = CAUSAL ? min(kend, q0 + PP_BM + q_off) : kend;
  const int n_t = kv_end > kbeg ? (kv_end - kbeg + BN - 1) / BN : 0;   // key tiles (>= 1 unless SPLIT)

  const long q_row_stride = (long)p.Hq * D;
  const long kv_stride = (long)p.Hkv * D * 2; // bytes per token row of K and V
  const char* kbase = (const char*)p.k + ((long)(kseq0 + kbeg) * p.Hkv + hkv) * D * 2;
  const char* vbase = (const char*)p.v + ((long)(kseq0 + kbeg) * p.Hkv + hkv) * D * 2;

  // ---- Q fragments (B operands of S^T = K Q^T): query my_q, d = 16 ks + 8 hl .. + 7 ----
  bf16x8 qf[KSTEPS];
  {
    const int qr = my_q < L ? my_q : L - 1;
    const __bf16* qp = (const __bf16*)p.q + ((long)(seq0 + qr) * p.Hq + h) * D + hl * 8;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) qf[ks] = *(const bf16x8*)(qp + ks * 16);
  }

  // ---- tile copies: wave w moves rows 8 w + 4 u + lane / 16 (u = 0, 1) of the K
  // and V tiles, 16 bytes per lane, logical chunk (lane % 16) ^ swizzle(row) of
  // the row to physical chunk lane % 16 (fa_device.h lds_swz) ----
  const int crow0 = 8 * wave + lane / 16;     // + 4 u
  unsigned coff[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int r = crow0 + 4 * u;
    coff[u] = (unsigned)r * (unsigned)kv_stride + (unsigned)(((lane & 15) ^ lds_swz<D>(r)) * 16);
  }
  const unsigned m_wave = lds0 + (unsigned)wave * 2048u;   // this wave's first 1 KiB row group in a stage
  int iss = 0;                                // next tile to copy
  // one 16-byte-per-lane HBM -> LDS load: M0 = LDS address of lane 0's 16 bytes
  auto rsrc_of = [&](const char* base) __attribute__((always_inline)) {
    const unsigned long long a64 = (unsigned long long)base;
    u32x4 r;
    r[0] = __builtin_amdgcn_readfirstlane((unsigned)a64);
    r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a64 >> 32)) & 0xffffu;
    r[2] = 0x7fffffffu;
    r[3] = 0x00020000u;
    return r;
  };
  auto dma = [&](const u32x4& rsrc, unsigned voff, unsigned soff, unsigned m0v) __attribute__((always_inline)) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
  };
  // A wave's share of a tile copy is four instructions (K rows u = 0, V rows
  // u = 0, K rows u = 1, V rows u = 1); an HBM -> LDS load instruction holds its
  // wave at issue for tens of clocks while the CU's vector-memory path takes its
  // 1 KiB.
  u32x4 c_rk, c_rv;
  // After the last S^T MFMA of a GEMM phase the softmax reads sacc only 19
  // wait states later. A tile's four copy triples (s_mov m0, s_nop 0, load)
  // give 12 by themselves; s_nop 7 adds 8 more. Without copies the softmax
  // waits the full mfma_result_wait().
  auto copies_then_result_wait = [&]() __attribute__((always_inline)) {
    asm volatile("s_nop 7" ::: "memory");
  };
  auto issue_tile = [&](const int stage) __attribute__((always_inline)) {
    const int r0 = iss * BN;
    const unsigned mk = m_wave + (unsigned)(KREG + stage * PP_TILEB);
    const unsigned mv = m_wave + (unsigned)(VREG + stage * PP_TILEB);
    // Loop-invariant K and V descriptors, rebased every 256 tiles, plus a
    // scalar offset per tile: the per-tile 64-bit pointer updates would sit in
    // vector registers (the scalar file is nearly full) and cost six vector
    // instructions of the softmax phase per tile.
    if ((iss & 255) == 0) {
      c_rk = rsrc_of(kbase + (long)r0 * kv_stride);
      c_rv = rsrc_of(vbase + (long)r0 * kv_stride);
    }
    const unsigned so = (unsigned)((iss & 255) * BN) * (unsigned)kv_stride;   // < 256 * 64 rows of one window
    ++iss;
    if (kbeg + r0 + BN <= kend) {               // a full tile: the precomputed row offsets
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        dma(c_rk, coff[u], so, mk + 1024u * u);
        dma(c_rv, coff[u], so, mv + 1024u * u);
      }
    } else {                                    // the last tile: rows past the end repeat the last row
      const int last = kend - 1 - kbeg - r0;
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int r = min(crow0 + 4 * u, last);
        const unsigned toff = (unsigned)r * (unsigned)kv_stride +   // chunk order of the LDS row
                              (unsigned)(((lane & 15) ^ lds_swz<D>(crow0 + 4 * u)) * 16);
        dma(c_rk, toff, so, mk + 1024u * u);
        dma(c_rv, toff, so, mv + 1024u * u);
      }
    }
  };

  // ---- per-lane LDS read bases (byte addresses, opaque to the compiler) ----
  // K row operand of k-step ks (A operand of S^T = K Q^T): key row 32 kb + l32,
  //   logical chunk 2 ks + hl; + stage * 16 KiB + kb * 8 KiB
  // V^T operand of d-block db (A operand of O^T += V^T P^T, two transposing
  //   8-byte reads i = 0, 1): key rows 16 t + 4 hl + g16 / 4 (+ 8 for i = 1),
  //   d = 32 db + 16 ((lane / 16) & 1) + 4 (g16 % 4); + stage * 16 KiB + t * 4 KiB
  unsigned kaddr[KSTEPS], vaddr[DBLK][2];
  {
    constexpr int ROWB = D * 2;
    const int g16 = lane & 15;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      kaddr[ks] = lds0 + KREG + l32 * ROWB + (((2 * ks + hl) ^ lds_swz<D>(l32)) << 4);
      asm volatile("" : "+v"(kaddr[ks]));
    }
#pragma unroll
    for (int db = 0; db < DBLK; ++db)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (g16 & 3);
        const int row = 4 * hl + (g16 >> 2) + 8 * i;
        vaddr[db][i] = lds0 + VREG + row * ROWB + (((dcol >> 3) ^ lds_swz<D>(row)) * 16) + (dcol & 7) * 2;
        asm volatile("" : "+v"(vaddr[db][i]));
      }
  }
  auto lds_at = [&](unsigned a) __attribute__((always_inline)) { return (const char FA_LDS*)(size_t)a; };
  const float c = p.scale_log2;
  const float tau = p.tau;
  f32x16 oacc[DBLK];                           // O^T, d-block db (accumulation registers)
  f32x16 sacc[2];                              // S^T of the current tile, key block kb (keys 32 kb ..)
  u32x4 pb[KT];                                // P^T bf16 pairs, key step t (keys 16 t ..)
  float m_run = 0.f, mc = 0.f, l_run = 0.f, m_seen = -INFINITY;

  // ---- GEMM phase: O^T += V^T P^T of the V tile in stage VS (if PV), then S^T of
  // the K tile in stage KS into sacc (if S) ----
  // MFMA order: the 16 P V MFMAs (key step t, d-block db), then the 16 S^T MFMAs
  // (k-step ks, key block kb), so P is dead before S^T is written (they share
  // registers) and the first P V operands can be read before the phase starts:
  // `pre` holds V^T fragments 0 .. PP_PF-1, read at the end of the previous
  // phase (the V tile has been resident since two phases before). Every other
  // fragment is read PP_PF MFMAs ahead.
  auto vfrag = [&](int f, int vs_off) __attribute__((always_inline)) -> bf16x8 {
    const int t = f / DBLK, db = f % DBLK;
    const int off = vs_off + t * 16 * D * 2;
    return cat(lds_read_tr(lds_at(vaddr[db][0]) + off), lds_read_tr(lds_at(vaddr[db][1]) + off));
  };
  auto prefetch_v = [&](bf16x8 (&pre)[PP_PF], auto vs_tag) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < PP_PF; ++f) pre[f] = vfrag(f, decltype(vs_tag)::value * PP_TILEB);
  };
  auto gemm = [&](auto s_tag, auto pv_tag, auto ks_tag, auto vs_tag, bf16x8 (&pre)[PP_PF])
                  __attribute__((always_inline)) {
    constexpr bool S = decltype(s_tag)::value;
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr int KS = decltype(ks_tag)::value;   // stage of the K tile
    constexpr int VS = decltype(vs_tag)::value;   // stage of the V tile
    constexpr int NP = PV ? KT * DBLK : 0;
    constexpr int NS = S ? 2 * KSTEPS : 0;
    constexpr int NM = NP + NS;
    auto frag = [&](int j) __attribute__((always_inline)) -> bf16x8 {
      if (j < NP) return vfrag(j, VS * PP_TILEB);
      const int m = j - NP;
      return lds_read16(lds_at(kaddr[m >> 1]) + KS * PP_TILEB + (m & 1) * 32 * D * 2);
    };
    __builtin_amdgcn_s_setprio(1);
    bf16x8 fr[PP_PF];
#pragma unroll
    for (int j = 0; j < PP_PF && j < NM; ++j) fr[j] = (PV && j < NP) ? pre[j] : frag(j);
    if constexpr (PV) asm volatile("s_nop 2");   // VALU-written P -> MFMA B operand
#pragma unroll
    for (int j = 0; j < NM; ++j) {
      const bf16x8 a = fr[j % PP_PF];
      if (j + PP_PF < NM) fr[j % PP_PF] = frag(j + PP_PF);
      if (j < NP) {
        const int t = j / DBLK, db = j % DBLK;
        mfma_vv(oacc[db], a, __builtin_bit_cast(bf16x8, pb[t]));
      } else {
        const int m = j - NP, ks = m >> 1, kb = m & 1;
        if (ks == 0) mfma_vv_first(sacc[kb], a, qf[0]);
        else mfma_vv(sacc[kb], a, qf[ks]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // ---- softmax phase of tile i (keys k0 = kbeg + 64 i ..), S^T in sacc ----
  // element (kb, r): key k0 + 32 kb + 8 (r / 4) + 4 hl + r % 4, query my_q
  auto needs_mask = [&](int k0) __attribute__((always_inline)) {
    return (k0 + BN > kend) || (CAUSAL && k0 + BN - 1 > qw0 + q_off);
  };
  // Masked elements: key >= kend, or (causal) key > my_q + q_off. With kl = k0 +
  // 4 hl (this lane's first key of the tile) and element offset e = 32 kb +
  // 8 (r / 4) + r % 4, element e is dead iff e >= thr, thr = min(kend, my_q +
  // q_off + 1) - kl (one register per tile); each element is then one compare
  // into VCC and one select.
  auto mask_tile = [&](int k0) __attribute__((always_inline)) {
    const int kl = k0 + 4 * hl;
    const int thr = (CAUSAL ? min(kend, my_q + q_off + 1) : kend) - kl;
    const float ninf = -INFINITY;
    static_for<0, 32>([&](auto e_tag) __attribute__((always_inline)) {
      constexpr int kb = decltype(e_tag)::value >> 4, r = decltype(e_tag)::value & 15;
      sacc[kb][r] = mask_ge<32 * kb + 8 * (r >> 2) + (r & 3)>(sacc[kb][r], thr, ninf);
    });
  };
  auto tile_max = [&]() __attribute__((always_inline)) -> float {
    float a[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const float x0 = vmax3(sacc[kb][0], sacc[kb][1], sacc[kb][2]);
      const float x1 = vmax3(sacc[kb][3], sacc[kb][4], sacc[kb][5]);
      const float x2 = vmax3(sacc[kb][6], sacc[kb][7], sacc[kb][8]);
      const float x3 = vmax3(sacc[kb][9], sacc[kb][10], sacc[kb][11]);
      const float x4 = vmax3(sacc[kb][12], sacc[kb][13], sacc[kb][14]);
      a[kb] = vmax3(vmax3(x0, x1, x2), vmax3(x3, x4, sacc[kb][15]), x0);
    }
    return pair_max(vmax(a[0], a[1]));
  };
  // P of the tile: p = exp2(S c - m c), l += p (fp32), bf16 pairs into pb. (Summing
  // the rounded bf16 pairs instead, with v_dot2c_f32_bf16, saves 16 instructions
  // per tile but puts the bf16 rounding of P into l: rows with few keys then
  // miss the 1e-3 LSE tolerance.)
  auto exps = [&]() __attribute__((always_inline)) {
    float lp[4];                                 // four row-sum chains, each from its first term
#pragma unroll
    for (int t = 0; t < KT; ++t) {
      const int kb = t >> 1, r0 = 8 * (t & 1);
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        const float p0 = exp2_sel<EXPMODE>(__builtin_fmaf(sacc[kb][r0 + e], c, -mc));
        const float p1 = exp2_sel<EXPMODE>(__builtin_fmaf(sacc[kb][r0 + e + 1], c, -mc));
        if (t == 0) lp[e >> 1] = p0;           // (not 0 + p0: that add is not folded away)
        else lp[e >> 1] += p0;
        lp[e >> 1] += p1;
        pb[t][e >> 1] = __builtin_bit_cast(unsigned, pack_bf16(p0, p1));
      }
    }
    l_run += (lp[0] + lp[1]) + (lp[2] + lp[3]);
  };
  // (the callers issue the phase's copy instructions just before it)
  auto softmax = [&](int i, int pass) __attribute__((always_inline)) {
    const int k0 = kbeg + i * BN;
    if (needs_mask(k0)) mask_tile(k0);
    if (pass == 1) {                           // tracking pass: the true row maxima only
      m_seen = vmax(m_seen, tile_max());
      // P and l are not used in this pass. Defining them here too lets the
      // exponentials of the other passes land in P's own registers (otherwise
      // the merge of the two branches costs nine register moves per tile).
#pragma unroll
      for (int t = 0; t < KT; ++t) pb[t] = u32x4{0u, 0u, 0u, 0u};
      l_run = 0.f;
      return;
    }
    if (i == 0 && pass == 0) {                 // the first tile fixes m for the pass
      m_run = tile_max();
      mc = m_run == -INFINITY ? 0.f : m_run * c;
    }
    exps();
  };

  // ---- the phase loop of one pass ----
  // Every wave runs the same sequence of actions, GEMM(-1), SOFTMAX(0),
  // GEMM(0), SOFTMAX(1), ..., SOFTMAX(n_t-1), GEMM(n_t-1); group B runs it one
  // phase behind group A. GEMM(k-1) computes S_k (k < n_t) and O += V_{k-1}
  // P_{k-1} (k >= 1). The two prologue phases have a barrier each; after them
  // A synchronises after each SOFTMAX(k) and B after each GEMM(k-1), which
  // makes slot k = {A: GEMM(k-1), SOFTMAX(k); B: SOFTMAX(k-1), GEMM(k-1)}
  // (both groups pass the same number of barriers). At the end of slot j each
  // wave waits for its share of tile j+1 (tile j+2 may stay in flight).
  auto wait_tile = [&](const int j) __attribute__((always_inline)) {   // end of slot j
    if (j + 2 < n_t) wait_vm(OPS);
    else if (j + 1 < n_t) wait_vm(0);
  };
  auto sync = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    barrier_no_fence();
    __builtin_amdgcn_sched_barrier(0);
  };
  // one pair of actions: GEMM(k-1) then SOFTMAX(k), with K_k in stage k % 4 (BI),
  // V_{k-1} in the stage before it. The GEMM waves issue no copies (a copy
  // instruction would hold the MFMA stream); each wave issues its share of a
  // tile from its softmax phase, between the exponentials: group A in
  // SOFTMAX(k) (slot k) tile k+2, group B in SOFTMAX(k) (slot k+1) tile k+3,
  // each into the stage of the tile two before it, whose last readers were the
  // GEMMs of the slot before. At the end of SOFTMAX(k) the wave reads the first
  // V^T fragments of its next GEMM (V_k).
  auto pair = [&](auto bi_tag, const int k, const int pass, bf16x8 (&pre)[PP_PF]) __attribute__((always_inline)) {
    constexpr int BI = decltype(bi_tag)::value;
    gemm(ic<1>{}, ic<1>{}, ic<BI>{}, ic<(BI + 3) % 4>{}, pre);
    __builtin_amdgcn_sched_barrier(0);
    if (!grp_a) {                               // B: end of slot k
      wait_tile(k);
      sync();
    }
    const bool cp = grp_a ? k + 2 < n_t : k + 3 < n_t;
    if (cp) {                                   // one branch, the copies first
      issue_tile(grp_a ? (BI + 2) % 4 : (BI + 3) % 4);
      copies_then_result_wait();
    } else {
      mfma_result_wait();
    }
    __builtin_amdgcn_sched_barrier(0);
    softmax(k, pass);
    prefetch_v(pre, ic<BI>{});
    __builtin_amdgcn_sched_barrier(0);
    if (grp_a) {                                // A: end of slot k
      wait_tile(k);
      sync();
    }
  };
  auto run_pass = [&](const int pass) __attribute__((always_inline)) {
    bf16x8 pre[PP_PF];
    // phase 0: A GEMM(-1) = S_0; B (idle) issues its share of tile 2
    if (grp_a) gemm(ic<1>{}, ic<0>{}, ic<0>{}, ic<0>{}, pre);
    else if (2 < n_t) issue_tile(2);
    sync();
    // phase 1: A SOFTMAX(0) with its share of tile 2, then V_0's first
    // fragments; B GEMM(-1) = S_0
    if (grp_a) {
      if (2 < n_t) {
        issue_tile(2);
        copies_then_result_wait();
      } else {
        mfma_result_wait();
      }
      __builtin_amdgcn_sched_barrier(0);
      softmax(0, pass);
      prefetch_v(pre, ic<0>{});
    } else {
      gemm(ic<1>{}, ic<0>{}, ic<0>{}, ic<0>{}, pre);
    }
    __builtin_amdgcn_sched_barrier(0);
    wait_tile(0);
    sync();
    // B's SOFTMAX(0), with its share of tile 3, then V_0's first fragments,
    // opens slot 1 (no barrier before B's GEMM(0)). The pairs k = 1 .. n_t - 1
    // then run from each wave's own point of view, B one phase behind A.
    if (!grp_a) {
      if (3 < n_t) {
        issue_tile(3);
        copies_then_result_wait();
      } else {
        mfma_result_wait();
      }
      __builtin_amdgcn_sched_barrier(0);
      softmax(0, pass);
      prefetch_v(pre, ic<0>{});
    }
    int k = 1;
    for (; k + 3 < n_t; k += 4) {
      pair(ic<1>{}, k, pass, pre);
      pair(ic<2>{}, k + 1, pass, pre);
      pair(ic<3>{}, k + 2, pass, pre);
      pair(ic<0>{}, k + 3, pass, pre);
    }
    if (k < n_t) pair(ic<1>{}, k, pass, pre);
    if (k + 1 < n_t) pair(ic<2>{}, k + 1, pass, pre);
    if (k + 2 < n_t) pair(ic<3>{}, k + 2, pass, pre);
    // GEMM(n_t-1): P V of the last tile only, V in stage (n_t - 1) % 4 (its first
    // fragments are in `pre`; the V^T read bases move to that stage for this one call)
    const unsigned vshift = (unsigned)(((n_t - 1) & 3) * PP_TILEB);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      vaddr[db][0] += vshift;
      vaddr[db][1] += vshift;
    }
    gemm(ic<0>{}, ic<1>{}, ic<0>{}, ic<0>{}, pre);
#pragma unroll
    for (int db = 0; db < DBLK; ++db) {
      vaddr[db][0] -= vshift;
      vaddr[db][1] -= vshift;
    }
    __builtin_amdgcn_sched_barrier(0);
    sync();                                     // the last slot: both groups' GEMM(n_t-1)
  };

  const float l_limit = exp2f(tau);
#pragma unroll
  for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
  m_run = -INFINITY;
  // a split work item whose chunk holds no key its queries see: O_p = 0, LSE_p = -inf
  // (n_t is uniform over the workgroup, so no wave skips a barrier the others take)
  for (int pass = 0; n_t > 0; ++pass) {
    iss = 0;
    issue_tile(0);
    if (n_t > 1) issue_tile(1);
#pragma unroll
    for (int i = 0; i < DBLK; ++i) oacc[i] = f32x16{};
    l_run = 0.f;
    if (pass == 2) {
      m_run = m_seen;
      mc = m_run == -INFINITY ? 0.f : m_run * c;
    }
    m_seen = -INFINITY;
    if (n_t > 1) wait_vm(OPS);
    else wait_vm(0);
    barrier_no_fence();
    run_pass(pass);
    mfma_result_wait();
    if (pass == 2) break;
    bool over;
    if (pass == 0) over = !(pair_sum(l_run) <= l_limit);   // also true for NaN / inf
    else over = true;                                      // after the tracking pass, the exact pass
    const bool any = wave_any(over);
    if (lane == 0) over_flag[wave] = any ? 1 : 0;
    __syncthreads();
    int again = 0;
#pragma unroll
    for (int w = 0; w < PP_WAVES; ++w) again |= over_flag[w];
    // uniform by construction; readfirstlane tells the compiler so (a loop whose
    // exit it takes for divergent would make every value carried around it a
    // per-lane value)
    again = __builtin_amdgcn_readfirstlane(again);
    __syncthreads();
    if (!again) break;
  }

  // ---- epilogue: O = O / l (bf16, staged through LDS), LSE = ln 2 (m c + log2 l) ----
  if constexpr (SPLIT) {
    // fp32 O_p rows straight from the accumulators; rows that saw no key of the
    // chunk hold O_p = 0, LSE_p = -inf
    const long part = (long)sp * p.B + s;
    float* ob = p.o_part + (part * p.N * p.Hq + h) * D;
    const float l_tot = pair_sum(l_run);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    store_rows_f32<D>(oacc, inv, ob, q_row_stride, qw0, L, lane);
    if (hl == 0 && my_q < L) {
      const float lse = (m_run == -INFINITY || l_tot == 0.f) ? -INFINITY : (m_run * c + __log2f(l_tot)) * kLn2;
      p.lse_part[(part * p.Hq + h) * p.N + my_q] = lse;
    }
    return;
  }
  char FA_LDS* st = (char FA_LDS*)lds + wave * PP_TILEB;   // this wave's output staging (16 KiB)
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  __bf16* obase = (__bf16*)p.o + ((long)seq0 * p.Hq + h) * D;
  store_rows_bf16<D>(st, oacc, inv, obase, q_row_stride, qw0, L, lane);
  if (hl == 0 && my_q < L) {
    const float lse = (m_run == -INFINITY) ? -INFINITY : (m_run * c + __log2f(l_tot)) * kLn2;
    long li;
    if constexpr (VARLEN) li = (long)h * p.cu_seqlens[p.B] + seq0 + my_q;
    else li = ((long)s * p.Hq + h) * p.N + my_q;
    p.lse[li] = lse;
  }
}

template <bool CAUSAL, bool VARLEN, int EXPMODE, bool SPLIT = false>
static hipError_t launch_pp(const FwdParams& p, int grid, hipStream_t stream) {
  hipLaunchKernelGGL((fa_fwd_pp_kernel<CAUSAL, VARLEN, EXPMODE, SPLIT>), dim3(grid), dim3(PP_THREADS), 0, stream, p);
  return hipGetLastError();
}

template <bool CAUSAL, bool VARLEN>
static hipError_t launch_pp_e(const FwdParams& p, int grid, int expmode, hipStream_t stream) {
  return expmode == 1 ? launch_pp<CAUSAL, VARLEN, 1>(p, grid, stream) : launch_pp<CAUSAL, VARLEN, 0>(p, grid, stream);
}

// d = 128 bf16 forward (uniform or packed batches): the two-waves-per-SIMD kernel.
hipError_t fwd_pp_launch(FwdParams p, int causal, int varlen, int expmode, hipStream_t stream) {
  p.n_qtiles = (p.N + PP_BM - 1) / PP_BM;
  const long grid_l = varlen ? q_grid_xcd(p.B, p.Hkv, p.G, p.kv_chunks, p.n_qtiles)
                             : q_grid_level(p.B, p.Hq, p.G, p.n_qtiles);
  if (grid_l == 0) return hipSuccess;
  if (grid_l > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int grid = (int)grid_l;
  if (causal) return varlen ? launch_pp_e<true, true>(p, grid, expmode, stream)
                            : launch_pp_e<true, false>(p, grid, expmode, stream);
  return varlen ? launch_pp_e<false, true>(p, grid, expmode, stream)
                : launch_pp_e<false, false>(p, grid, expmode, stream);
}

// d = 128 split-KV partial results (uniform batches): the two-waves-per-SIMD
// kernel over (sequence, key chunk) work items.
hipError_t fwd_pp_split_launch(FwdParams p, int causal, hipStream_t stream) {
  p.n_qtiles = (p.N + PP_BM - 1) / PP_BM;
  const long grid_l = q_grid_level(p.B * p.n_splits, p.Hq, p.G, p.n_qtiles);
  if (grid_l == 0) return hipSuccess;
  if (grid_l > 0x7fffffffL) return hipErrorInvalidConfiguration;
  const int grid = (int)grid_l;
  return causal ? launch_pp<true, false, 0, true>(p, grid, stream) : launch_pp<false, false, 0, true>(p, grid, stream);
}

}  // namespace fa

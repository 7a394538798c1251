// BLASST decode over a paged latent cache, all 128 heads of a sequence in one workgroup
// (MLA-shaped: 576-dim scores, V = the first 512 latent dims).
//
// Method: each 64-token block's row maxima are compared with the running maxima of the tile, and a
// block that every row votes to skip gets no exp and no P.V product (pages: xllm-io review,
// 核心公式 and 核心思想 item 4 (MHA/GQA/MQA/MLA); fugumt.com abstract).  In latent attention V is
// the same bytes as K, so a skip saves arithmetic, not HBM traffic.
//
// MI355X design (the one-wave-per-SIMD layout; decode_latent.hip keeps the 16-heads-per-wave one
// for 64-head tiles):
//   * one workgroup = (sequence, row tile, split), 4 waves, one per SIMD, each with the full
//     512-register file; wave w owns rows 32 w .. 32 w + 31 of the 128-row tile (the 128 heads, or
//     with T query tokens per sequence T x 128 / T (token, head) pairs, token-major, each token
//     seeing keys up to seq_len - T + t), so every operand fragment read from LDS feeds a
//     32-wide MFMA (v_mfma_f32_32x32x16_bf16): 32 flops per LDS byte, twice what 16 heads per wave
//     give, which is what bounds the latent decode on this chip (LDS, not MFMA or HBM);
//   * S^T = K q^T: K rows (A operand) from LDS, the wave's 32 heads of q in 144 VGPRs (B operand);
//     each lane holds the 32 scores of one head for its half of the keys, so the block row max is
//     an in-lane max and one exchange with lane l ^ 32;
//   * O^T = V^T P^T: P^T straight from the score registers (B operand), V^T read from the same LDS
//     tile with ds_read_b64_tr_b16; O^T of 32 heads x 512 channels is 256 accumulators, held in the
//     AGPRs: the P.V MFMAs are written out with AGPR accumulators (the scores, consumed by VALU code,
//     stay in VGPRs; this file is built with the MFMA VGPR form for the score MFMAs);
//   * the accumulators are never rescaled inside the loop: probabilities are taken relative to a
//     per-head reference max fixed by the first kept block; a block max more than 2^64 (in
//     probability) above it makes the workgroup redo its blocks with the reference raised (see the
//     comment at the pass loop);
//   * wave w loads page w of each block (one uniform page base per wave, loop-invariant per-lane
//     offsets: the loads need no address arithmetic), global -> LDS directly, double-buffered: the
//     19 loads of block j + 1 are spread over block j's 36 score k-steps, one per two k-steps (a
//     wave that issued them at once sat a third of the block time in the stalled issue, unable to
//     issue MFMAs); the page ids come a 64-block window at a time into LDS, also by direct load,
//     so that no load into registers (whose wait would drain the block loads) remains in the loop;
//     rows are 1168 bytes apart (576 channels + 16 bytes), which keeps the 32-row score-operand
//     reads free of bank conflicts.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int DQK = 576, DV = 512, PAGE = 16, BK = 64, HPW = 32, NW = 4, NT = NW * 64;
constexpr int CH = DQK / 8;              // 16-byte chunks per latent row (72)
constexpr int ROW = (CH + 1) * 16;       // LDS row stride with one pad chunk (1168 bytes)
constexpr int PGB = PAGE * ROW;          // LDS bytes per page (18688)
constexpr int BUF = BK * ROW;            // LDS bytes per block (74752)
constexpr int NLD = (PGB + 1023) / 1024; // direct loads per page (19; the last one 256 bytes)
constexpr int KS = DQK / 16;             // k-steps of S^T (36)
constexpr int MT = BK / 32;              // key m-tiles of S^T (2)
constexpr int MTV = DV / 32;             // dv m-tiles of O^T (16)
constexpr int KSV = BK / 16;             // k-steps of O^T (4)
constexpr float kRefWindowLog2 = 64.f;
typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
}  // namespace

// global_load_lds_dwordx4 with a wave-uniform 64-bit base and a per-lane 32-bit offset, marked
// non-temporal (every latent block is read once: streamed this way the cache reads 7.0 TB/s on this
// chip against 6.2 TB/s with the default policy, measured with the same page pattern and no compute)
// (M0 is saved and restored around it, so the compiler's use of M0 is not disturbed)
__device__ __forceinline__ void direct_load16_saddr(const void *sbase, uint32_t voffset, uint32_t lds_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voffset), "s"(sbase), "s"(lds_base));
}

template <bool OUT_F32, bool STATS>
__global__ __launch_bounds__(NT, 1) void decode_mla_kernel(DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) unsigned char sK[2][BUF];
  __shared__ int sVote[2][NW];
  __shared__ int sIds[2][NW][64];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // workgroup -> (sequence, row tile, split); the n_rt row tiles of one (sequence, split) are 8
  // apart in launch order, so they land on the same XCD and share its L2 copy of the latent blocks
  const int rt = (blockIdx.x >> 3) % a.n_rt;
  const int ps = (blockIdx.x >> 3) / a.n_rt * 8 + (blockIdx.x & 7);
  const int split = ps % a.num_splits;
  const int b = ps / a.num_splits;
  if (b >= a.B) return;
  const int cap = a.max_pages * PAGE;
  const int L = min(a.seq_lens[b], cap);
  const int J = (L + BK - 1) / BK;
  const int chunk = (J + a.num_splits - 1) / a.num_splits;
  const int j0 = split * chunk;
  const int j1 = min(J, j0 + chunk);
  const int npg = (L + PAGE - 1) / PAGE;
  const int row = wave * HPW + l32;                            // this lane's score / output column
  const int tok = row / a.tile_rows;                           // its query token
  const int h = rt * a.tile_rows + (row - tok * a.tile_rows);  // and q head
  const int64_t qrow = ((int64_t)b * a.T + tok) * a.Hq + h;    // row of q (and of o, lse)
  const int lim = L - a.T + tok;                               // the last key this row sees

  float thr = a.thr_raw;
  if (a.thr_mode == 1) {
    const float lam = fminf(1.f, a.a / (float)L);
    thr = lam > 0.f ? __logf(lam) / a.scale : kNegInf;
  }

  // q fragments (B operand of S^T = K q^T): lane holds dims 16 kk + 8 hi .. +7 of head h
  bf16x8 qf[KS];
  const __bf16 *qp = (const __bf16 *)a.q + qrow * DQK;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = *(const bf16x8 *)(qp + kk * 16 + hi * 8);
  // consume the q loads here, so their waits are not placed inside the block loop
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) asm volatile("" ::"v"(qf[kk]));

  // per-lane source offsets of the page loads: load k of a page writes LDS bytes
  // [1024 k + 16 lane, +16) of the page region, i.e. padded row r = o / ROW, chunk c = (o % ROW) / 16
  // (the pad chunk re-reads chunk 0), from byte r * 1152 + 16 c of the page; two 16-bit offsets per
  // VGPR
  uint32_t offp[(NLD + 1) / 2];
#pragma unroll
  for (int k = 0; k < (NLD + 1) / 2; ++k) offp[k] = 0;
#pragma unroll
  for (int k = 0; k < NLD; ++k) {
    const int o = min(1024 * k + 16 * lane, PGB - 16);
    const int r = o / ROW;
    int c = (o - r * ROW) / 16;
    if (c >= CH) c = 0;
    offp[k >> 1] |= (uint32_t)(r * DQK * 2 + c * 16) << (16 * (k & 1));
  }
  const char *kc = (const char *)a.kc;
  const int32_t *table = a.table + (int64_t)b * a.max_pages;
  constexpr int64_t kPageBytes = (int64_t)PAGE * DQK * 2;  // one kv head
  // Page ids: this wave's page of blocks jw .. jw + 63 (lane i: block jw + i) go global -> LDS with
  // one direct load, a 64-block window ahead of their use.  A load into registers would not do: the
  // compiler's wait for it is a vmcnt wait, which would also drain the block loads in flight.
  auto load_ids = [&](int jw, int slot) {
    direct_load4(table + min((jw + lane) * (BK / PAGE) + wave, npg - 1), lds_addr(&sIds[slot][wave][0]));
  };
  // load k (of NLD) of this wave's page of a block: base = the page (wave-uniform), lbase = the
  // wave's page region of the LDS buffer
  auto load_part = [&](const char *base, uint32_t lbase, int k) {
    const uint32_t off = (offp[k >> 1] >> (16 * (k & 1))) & 0xffffu;
    if (k + 1 < NLD || 1024 * k + 16 * lane < PGB) direct_load16_saddr(base, off, lbase + 1024 * k);
  };
  auto page_base = [&](int pid_raw) -> const char * {
    return kc + (int64_t)__builtin_amdgcn_readfirstlane(pid_raw) * kPageBytes;
  };
  // transpose-read base for the V^T operand (the layout of prefill_bf16.hip with BC = 64)
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int tr_off = ((tr_g >> 1) * 4 + (tr_j >> 2)) * ROW + (16 * (tr_g & 1) + 4 * (tr_j & 3)) * 2;

  float m_ref = kNegInf;  // reference max of the accumulation (see the pass loop)
  float m_seen, m_dec, l_part, l_part2;
  f32x16 o_acc[MTV];
  unsigned live_cnt, skip_cnt;
  const int mask_row = (b * a.n_rt + rt) * a.nkb;  // one kv head

  // Pass loop: one pass over the split's blocks.  The accumulation takes probabilities relative to
  // the reference m_ref, set by the first kept block with a finite max; while every block max
  // stays within 2^64 (in probability) of it this is the usual online softmax (O / l does not depend
  // on the reference; bf16 P and the fp32 sums keep their relative precision, and with at most 2^64
  // per probability the sums stay far inside the fp32 range) and no accumulator is rescaled.  A
  // block max beyond that window (a logit more than 44 above the first kept block's maximum) makes
  // the whole workgroup restart the pass with the reference raised to the largest max seen.  (A
  // 2^16 window was measured to trigger restarts on ordinary score distributions: a later block
  // can easily be 11 logits above the first block of a split.)
  for (;;) {
    // orders the zeroing below after the previous pass's last P.V MFMA (XDL write -> VALU write)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    m_seen = kNegInf;
    m_dec = kNegInf;
    l_part = 0.f;
    l_part2 = 0.f;
#pragma unroll
    for (int i = 0; i < MTV; ++i) o_acc[i] = f32x16{};
    live_cnt = 0;
    skip_cnt = 0;
    bool redo = false;

    // Block j + 1 is loaded into the other buffer while block j is processed, its NLD loads spread
    // over block j's score k-steps.  A wave that issues a whole block's loads at once stalls at
    // issue until the memory pipeline takes them (measured: about a third of the block time), and a
    // wave cannot issue MFMAs meanwhile; spread out, each load finds room in the queue.
    int wbase = j0, wslot = 0;  // sIds[wslot] holds blocks wbase .. wbase + 63, the other slot the next 64
    auto page_id = [&](int jj) -> int {  // wbase <= jj < wbase + 128
      const int r = jj - wbase;
      return sIds[(wslot + (r >> 6)) & 1][wave][r & 63];
    };
    int pid_next = 0;  // page id of block j + 1 (this wave's page)
    if (j0 < j1) {
      load_ids(wbase, 0);
      load_ids(wbase + 64, 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const char *base0 = page_base(page_id(j0));
#pragma unroll
      for (int k = 0; k < NLD; ++k) load_part(base0, lds_addr(sK[0] + wave * PGB), k);
      pid_next = page_id(j0 + 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      barrier_lds_only();
    }
    for (int j = j0; j < j1; ++j) {
      const int buf = (j - j0) & 1;
      const bool has_next = j + 1 < j1;
      const char *nbase = page_base(pid_next);                  // block j + 1, this wave's page
      const uint32_t nlds = lds_addr(sK[buf ^ 1] + wave * PGB);  // into the other buffer
      const int key0 = j * BK;
      if (key0 + BK > L) {
        // slots past the sequence end hold arbitrary bytes: zero them so that P = 0 meets V = 0
        // (0 * NaN cannot appear); their scores are masked below
        for (int o16 = (L - key0) * ROW + tid * 16; o16 < BUF; o16 += NT * 16) *(u32x4 *)(sK[buf] + o16) = u32x4{};
        __syncthreads();
      }

      // ---- S^T = K_j q^T (keys 32 mt + 8 (r / 4) + 4 hi + r % 4 of register r) ----
      f32x16 s[MT];
      const unsigned char *kb = sK[buf] + l32 * ROW + hi * 16;
      // K fragments are read KPF k-steps ahead into a ring (one wave per SIMD: nothing else hides the
      // LDS latency behind the two MFMAs of a k-step)
      constexpr int KPF = 2;
      bf16x8 kf[KPF + 1][MT];
#pragma unroll
      for (int p = 0; p < KPF; ++p)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) kf[p][mt] = *(const bf16x8 *)(kb + mt * 32 * ROW + p * 32);
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        // block j + 1: load kk / 2 at the even k-steps, the last (partial) one at the last k-step
        static_assert(2 * (NLD - 1) <= KS, "one load per two k-steps");
        if (has_next && (kk & 1) == 0 && kk / 2 < NLD - 1) load_part(nbase, nlds, kk / 2);
        if (has_next && kk == KS - 1) load_part(nbase, nlds, NLD - 1);
        if (kk + KPF < KS) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            kf[(kk + KPF) % (KPF + 1)][mt] = *(const bf16x8 *)(kb + mt * 32 * ROW + (kk + KPF) * 32);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk % (KPF + 1)][mt], qf[kk], kk == 0 ? f32x16{} : s[mt], 0,
                                                          0, 0);
        if ((kk & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }
      if (key0 + BK > L - a.T + 1) {   // keys past a row's last visible key (or the sequence end)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (key0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3) > lim) s[mt][r] = kNegInf;
      }

      // ---- block row max, vote, critical value ----
      float mx = kNegInf;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      mx = max_xor32(mx);
      const bool skip_row = row_votes_skip(mx, m_dec, thr);
      const bool wave_keep = __ballot(!skip_row) != 0ull;
      const bool over = m_ref != kNegInf && (mx - m_ref) * a.scale_log2 > kRefWindowLog2;
      const bool wave_over = __ballot(over) != 0ull;
      m_seen = fmaxf(m_seen, mx);
      float wcrit = 0.f;
      if (a.crit) wcrit = max_lanes32(row_crit(mx, m_dec));
      if (lane == 0) {
        sVote[buf][wave] = (wave_keep ? 1 : 0) | (wave_over ? 2 : 0);
        sCrit[buf][wave] = wcrit;
      }
      barrier_lds_only();  // vote barrier (the next block's loads stay in flight)
      int votes = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) votes |= sVote[buf][w];
      if (votes & 2) {  // uniform over the workgroup
        redo = true;
        break;
      }
      const bool keep = (votes & 1) != 0;
      m_dec = fmaxf(m_dec, mx);
      ++live_cnt;
      if (!keep) ++skip_cnt;
      if (tid == 0) {
        if (a.mask) a.mask[mask_row + j] = keep ? kKept : kSkipped;
        if (a.crit) {
          float c = sCrit[buf][0];
#pragma unroll
          for (int w = 1; w < NW; ++w) c = fmaxf(c, sCrit[buf][w]);
          a.crit[mask_row + j] = c * a.scale;
        }
      }

      if (!STATS && keep) {
        // ---- kept block: O^T += V^T P^T with probabilities relative to the reference ----
        if (m_ref == kNegInf) m_ref = mx;  // first kept block of this head: O and l are still zero
        const float base = (m_ref == kNegInf) ? 0.f : m_ref * a.scale_log2;
        const unsigned char *vb = sK[buf] + tr_off;
        const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
        // bf16 probabilities of k-step kk (the B operand) and their sums
        auto make_pf = [&](int kk) -> bf16x8 {
          bf16x8 pf;
#pragma unroll
          for (int e = 0; e < 8; ++e)
            pf[e] = (__bf16)fast_exp2(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + e], a.scale_log2, -base));
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), one2, l_part, false);
          l_part2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), one2, l_part2, false);
          l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), one2, l_part, false);
          l_part2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), one2, l_part2, false);
          return pf;
        };
        // One pass over (k-step kk, dv tile mv) = step q: V^T fragments are read PF steps ahead into a
        // ring of PF + 1 slots, continuing across k-steps (with one wave per SIMD nothing else hides
        // the LDS latency; the written-out MFMAs keep their order, so the reads are placed ahead of
        // them in program order), and the probabilities of k-step kk + 1 are formed halfway through
        // the MFMAs of k-step kk, so their VALU work overlaps MFMAs in flight.
        constexpr int PF = 7, NQ = KSV * MTV;
        bf16x8 vring[PF + 1];
        auto read_v = [&](int q) {
          const int kk = q / MTV, mv = q % MTV;
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + kk * 16 * ROW + mv * 64));
          const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + (kk * 16 + 8) * ROW + mv * 64));
          vring[q % (PF + 1)] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        };
        bf16x8 pfs[2];
        pfs[0] = make_pf(0);
#pragma unroll
        for (int q = 0; q < PF; ++q) read_v(q);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
          const int kk = q / MTV, mv = q % MTV;
          if (q + PF < NQ) read_v(q + PF);
          // s_nop 3: wait states after the VALU writes of the operands (the compiler does not
          // track hazards of inline assembly)
          asm volatile("s_nop 3\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                       : "+a"(o_acc[mv])
                       : "v"(vring[q % (PF + 1)]), "v"(pfs[kk & 1]));
          if (mv == MTV / 2 && kk + 1 < KSV) {
            // the slot written here was last read by the MFMAs of k-step kk - 1, at least MTV / 2
            // MFMAs ago
            __builtin_amdgcn_sched_barrier(0);
            pfs[(kk + 1) & 1] = make_pf(kk + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (has_next) {
        if (j + 2 - wbase == 64) {  // block j + 2 opens the next window: refill the slot of the last one
          load_ids(wbase + 128, wslot);  // complete with the wait below, used 64 blocks later
          wslot ^= 1;
          wbase += 64;
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        barrier_lds_only();  // block j + 1 is in LDS for every wave; every wave is done with buf
        pid_next = page_id(j + 2);
      }
    }
    if (!redo) break;
    // drain the prefetch of the aborted pass, then start over with the reference raised
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    m_ref = fmaxf(m_ref, m_seen);
  }

  if (tid == 0 && a.counters) {
    atomicAdd(&a.counters[0], (unsigned long long)live_cnt);
    atomicAdd(&a.counters[1], (unsigned long long)skip_cnt);
  }
  if ((a.mask || a.crit) && split == 0)
    for (int j = J + tid; j < a.nkb; j += NT) {
      if (a.mask) a.mask[mask_row + j] = kNotLive;
      if (a.crit) a.crit[mask_row + j] = __builtin_nanf("");
    }
  if (STATS) return;

  // XDL write -> VALU read of the accumulators: wait states after the last P.V MFMA (which the
  // compiler does not know about) before the epilogue reads them
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(o_acc[0]), "+a"(o_acc[1]), "+a"(o_acc[2]), "+a"(o_acc[3]), "+a"(o_acc[4]), "+a"(o_acc[5]),
                 "+a"(o_acc[6]), "+a"(o_acc[7]), "+a"(o_acc[8]), "+a"(o_acc[9]), "+a"(o_acc[10]), "+a"(o_acc[11]),
                 "+a"(o_acc[12]), "+a"(o_acc[13]), "+a"(o_acc[14]), "+a"(o_acc[15]));

  // ---- epilogue: O^T lane layout: head h, channels 32 mv + 8 (r / 4) + 4 hi + r % 4 ----
  const float lp = l_part + l_part2;
  const float l_tot = lp + __shfl_xor(lp, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_ref * a.scale + __logf(l_tot) : kNegInf;
  if (a.num_splits == 1) {
    const int64_t ob = qrow * DV + 4 * hi;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int64_t oi = ob + 32 * mv + 8 * rg;
        if (OUT_F32) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o_acc[mv][4 * rg + e] * inv;
          *(f32x4 *)((float *)a.o + oi) = v4;
        } else {
          u32x2 w;
          w[0] = pack_bf16x2(o_acc[mv][4 * rg + 0] * inv, o_acc[mv][4 * rg + 1] * inv);
          w[1] = pack_bf16x2(o_acc[mv][4 * rg + 2] * inv, o_acc[mv][4 * rg + 3] * inv);
          *(u32x2 *)((__bf16 *)a.o + oi) = w;
        }
      }
    if (a.lse && hi == 0) a.lse[qrow] = lse;
  } else {
    const int64_t pb = qrow * a.num_splits + split;
    float *wo = a.ws_o + pb * DV + 4 * hi;
#pragma unroll
    for (int mv = 0; mv < MTV; ++mv)
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        f32x4 v4;
#pragma unroll
        for (int e = 0; e < 4; ++e) v4[e] = o_acc[mv][4 * rg + e] * inv;
        *(f32x4 *)(wo + 32 * mv + 8 * rg) = v4;
      }
    if (hi == 0) a.ws_lse[pb] = lse;
  }
}

// 128 q heads on one latent head, 576/512 dims, page 16, block 64, 128-row tiles (all heads, or T tokens x
// 128 / T heads).
hipError_t launch_decode_mla128(const DecodeArgs &a, hipStream_t st) {
  if (a.Hq != 128 || a.Hkv != 1 || a.page != PAGE || a.block_k != BK || a.T * a.tile_rows != 128)
    return hipErrorNotSupported;
  const int grid = (a.B * a.num_splits + 7) / 8 * 8 * a.n_rt;
  if (a.stats_only)
    hipLaunchKernelGGL((decode_mla_kernel<false, true>), dim3(grid), dim3(NT), 0, st, a);
  else if (a.out_f32)
    hipLaunchKernelGGL((decode_mla_kernel<true, false>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((decode_mla_kernel<false, false>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

}  // namespace blasst

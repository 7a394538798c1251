// BLASST decode over a paged KV cache, split along the keys (GQA / MHA / MQA, head dim 128).
//
// Method: for each KV block, the block-local max of the tile's query rows is compared with the
// running max, and a block that every row votes to skip is dropped: its V block is never loaded
// and it gets no exp and no P.V.  The decision is taken at the K-load stage, and K is processed in
// batches of several blocks before the V loads of the surviving blocks are issued together, so
// the skip does not stall the load pipeline (pages: xllm-io review, 解码内核优化; gist.science (de),
// 3. Kernel-Design).  Splitting the keys into num_splits chunks merged by a log-sum-exp combine is
// part of the defined semantics here (each chunk restarts the running max).
//
// MI355X design:
//   * one workgroup = (sequence, kv head, row tile, split); 4 waves; wave w owns the w-th 16-token
//     page of every 64-token block, so each wave issues page-sized, page-aligned loads;
//   * the tile's query columns are (token, head) pairs, token-major: with T query tokens per
//     sequence (the last T positions) column t * tile_rows + i is token t of the tile's head i, and
//     its keys past seq_len - T + t are masked like keys past the sequence end;
//   * K-first batch of NB blocks: each wave stages its NB K pages in LDS (whole rows per load, a
//     swizzled layout: see load_k), computes S^T = K q^T with
//     v_mfma_f32_16x16x32_bf16 (the tile's <= 16 q heads are the N columns), and publishes its
//     per-page row maxima in LDS; after one barrier every thread derives the block maxima and the
//     sequential decisions of the whole batch (the same values in every wave, so the branch is
//     uniform);
//   * then the V pages of the surviving blocks only are loaded: the V cache stores each page
//     transposed ([dv][token]), so a lane's 4 consecutive tokens of one dv row are one 8-byte load
//     and a 16-row m-tile is one 512-byte contiguous read; P^T goes from the score registers to the
//     B operand of v_mfma_f32_16x16x16_bf16 without any shuffle;
//   * the next batch's K loads are issued before the PV products of the current batch, so K
//     traffic overlaps the arithmetic;
//   * K and V loads are marked non-temporal: each cache byte is read once per launch, and streamed
//     this way the chip's reads reach 7.0 TB/s against 6.2 TB/s with the default cache policy;
//   * all waves use the same running max, so their partial outputs add up; one LDS reduction per
//     split, then either the final output (one split) or a per-split partial for the combine
//     kernel.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int D = 128, PAGE = 16, BK = 64, NWAVE = 4, NB = 4;
}

// DEC = false: no threshold at all (every live block kept, no vote, no diagnostics but the
// counters); the same kernel without the decision logic, used to measure what the decisions cost.
template <bool OUT_F32, bool DEC = true>
__global__ __launch_bounds__(256, 2) void decode_gqa_kernel(DecodeArgs a) {
  // K pages of the batch, one 4 KB page per (block, wave), in a swizzled order (see load_k); the
  // epilogue reuses the buffer for the cross-wave reduction
  __shared__ __attribute__((aligned(16))) unsigned char sKb[NB][NWAVE][PAGE * D * 2];
  __shared__ float sPmax[2][NB][NWAVE][16];  // double-buffered by batch parity
  __shared__ float sL[NWAVE][16];
  static_assert(sizeof(float) * NWAVE * 16 * (D + 4) <= sizeof(sKb), "the reduction fits the K buffer");
  float(*sRed)[16][D + 4] = reinterpret_cast<float(*)[16][D + 4]>(&sKb[0][0][0]);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // query column (q head inside the tile)
  const int grp = lane >> 4; // 16-lane group

  int bid = blockIdx.x;
  const int split = bid % a.num_splits;
  bid /= a.num_splits;
  const int rt = bid % a.n_rt;
  bid /= a.n_rt;
  const int g = bid % a.Hkv;
  const int b = bid / a.Hkv;

  const int cap = a.max_pages * PAGE;
  const int L = min(a.seq_lens[b], cap);
  const int J = (L + BK - 1) / BK;
  const int chunk = (J + a.num_splits - 1) / a.num_splits;
  const int j0 = split * chunk;
  const int j1 = min(J, j0 + chunk);
  const int ncol = a.T * a.tile_rows;       // query columns of the tile (<= 16)
  const bool col_ok = n < ncol;
  const int tok = col_ok ? n / a.tile_rows : 0;
  const int hq = g * a.G + rt * a.tile_rows + (n - tok * a.tile_rows);
  const int64_t qrow = ((int64_t)b * a.T + tok) * a.Hq + hq;  // row of q (and of o, lse)

  float thr = a.thr_raw;
  if (a.thr_mode == 1) {
    const float lam = fminf(1.f, a.a / (float)L);
    thr = lam > 0.f ? __logf(lam) / a.scale : kNegInf;
  }

  // q fragments: B operand of S^T = K q^T; lane holds dims kk*32 + grp*8 .. +7 of query column n
  bf16x8 qf[4];
  const __bf16 *qp = (const __bf16 *)a.q + qrow * D;
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qf[kk] = col_ok ? *(const bf16x8 *)(qp + kk * 32 + grp * 8) : bf16x8{};

  const __bf16 *kc = (const __bf16 *)a.kc;
  const __bf16 *vc = (const __bf16 *)a.vc;
  const int32_t *table = a.table + (int64_t)b * a.max_pages;
  const int64_t page_stride = (int64_t)a.Hkv * PAGE * D;  // elements per physical page (all heads)
  const int npg = (L + PAGE - 1) / PAGE;                   // pages of this sequence (>= 1)
  const int lim = L - a.T + tok;                           // last key this column sees

  float m_dec = kNegInf, m_acc = kNegInf, l_part = 0.f;
  f32x4 o_acc[D / 16];
#pragma unroll
  for (int i = 0; i < D / 16; ++i) o_acc[i] = f32x4{};
  unsigned live_cnt = 0, skip_cnt = 0;
  const int mask_row = ((b * a.Hkv + g) * a.n_rt + rt) * a.nkb;

  // Page ids of a batch: lane l (< 16) holds the id of page jb*4 + l, i.e. page (l % 4) of block
  // jb + l / 4; a wave picks its pages with readlane.  Pages past the sequence use its last page
  // (their keys are masked and their V is zeroed), so every load is unconditional and in bounds.
  auto load_table = [&](int jb) -> int {
    const int pg = min(jb * (BK / PAGE) + (lane & 15), npg - 1);
    return table[pg];
  };
  // K: each wave stages its page of every block of the batch in LDS (wave-private: no barrier),
  // global -> LDS directly, 1 KB of whole rows per load.  Loaded straight into MFMA operand
  // registers, a load reads 16 rows x 64 bytes, and streams 12 % slower (measured, same pages).  The
  // 16-byte chunk c of page row r sits at LDS chunk 16 r + (c ^ r): the operand reads of a k-step
  // (16 rows, one chunk each) then fall on distinct banks.
  int pid_cur[NB];
  auto load_k = [&](const int (&pid)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const __bf16 *pg = kc + (int64_t)pid[i] * page_stride + (int64_t)g * PAGE * D;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int r = kk * 4 + grp;        // page row of this lane's LDS chunk 64 kk + lane
        const int c = n ^ r;               // its source chunk
        direct_load16_nt(pg + r * D + c * 8, lds_addr(&sKb[i][wave][kk * 1024]));
      }
    }
  };
  // operand read of k-step kk: row n, chunk 4 kk + grp, i.e. LDS chunk 16 n + ((4 kk + grp) ^ n)
  const int kswz = grp ^ n;
  auto read_k = [&](int i, int kk) -> bf16x8 {
    return *(const bf16x8 *)&sKb[i][wave][n * (D * 2) + (((kk << 2) ^ kswz) << 4)];
  };
  auto pick = [&](int tabv, int (&pid)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i) pid[i] = __builtin_amdgcn_readlane(tabv, i * 4 + wave);
  };

  int tab_next = 0;
  if (j0 < j1) {
    const int tab0 = load_table(j0);
    pick(tab0, pid_cur);
    load_k(pid_cur);
    tab_next = load_table(j0 + NB);
  }
  int pbuf = 0;
  for (int jb = j0; jb < j1; jb += NB, pbuf ^= 1) {
    const int nb = min(NB, j1 - jb);
    // ---- scores of this wave's page of each block in the batch ----
    // this wave's K pages of the batch have landed (its own direct loads; every older load too)
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    f32x4 s[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      s[i] = f32x4{};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) s[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(read_k(i, kk), qf[kk], s[i], 0, 0, 0);
      // keys past the column's last visible key (and blocks past the batch) are masked out
      const int keyb = (jb + i) * BK + wave * PAGE + grp * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (i >= nb || keyb + r > lim) s[i][r] = kNegInf;
      float pm = fmaxf(fmaxf(s[i][0], s[i][1]), fmaxf(s[i][2], s[i][3]));
      pm = max_xor16_32(pm);
      if (grp == 0) sPmax[pbuf][i][wave][n] = pm;
    }
    // ---- the next batch's K loads go out now (the scores above have read this wave's K pages),
    // so they are in flight across the barrier and the decisions ----
    int pid_next[NB];
    pick(tab_next, pid_next);
    const bool more = jb + NB < j1;
    if (more) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the K operand reads are done
      load_k(pid_next);
      tab_next = load_table(jb + 2 * NB);
    }
    __syncthreads();
    // ---- in-batch sequential decisions (identical in every wave) ----
    int keep_bits = 0;
    float mblk[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float(&pm)[NWAVE][16] = sPmax[pbuf][i];
      float mb = fmaxf(fmaxf(pm[0][n], pm[1][n]), fmaxf(pm[2][n], pm[3][n]));
      if (!col_ok) mb = kNegInf;
      mblk[i] = mb;
      if (i < nb && !DEC) {
        keep_bits |= 1 << i;
        ++live_cnt;
      } else if (i < nb) {
        const int j = jb + i;
        const bool skip_row = row_votes_skip(mb, m_dec, thr);
        const bool keep = __ballot(!skip_row) != 0ull;
        if (a.crit) {
          float c = row_crit(mb, m_dec);
          c = fmaxf(c, __shfl_xor(c, 8));
          c = fmaxf(c, __shfl_xor(c, 4));
          c = fmaxf(c, __shfl_xor(c, 2));
          c = fmaxf(c, __shfl_xor(c, 1));
          if (tid == 0) a.crit[mask_row + j] = c * a.scale;
        }
        if (tid == 0 && a.mask) a.mask[mask_row + j] = keep ? kKept : kSkipped;
        m_dec = fmaxf(m_dec, mb);
        keep_bits |= (keep ? 1 : 0) << i;
        ++live_cnt;
        if (!keep) ++skip_cnt;
      }
    }
    if (a.stats_only) keep_bits = 0;
    // ---- the V loads of the surviving blocks only ----
    u32x2 vreg[NB][D / 16];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (keep_bits & (1 << i)) {
        const __bf16 *src = vc + (int64_t)pid_cur[i] * page_stride + (int64_t)g * D * PAGE + n * PAGE + grp * 4;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) vreg[i][mt] = __builtin_nontemporal_load((const u32x2 *)(src + mt * 16 * PAGE));
      }
    }
    // ---- kept blocks: online softmax and O^T += V^T P^T ----
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (!(keep_bits & (1 << i))) continue;
      const float m_new = fmaxf(m_acc, mblk[i]);
      if (__ballot(m_new > m_acc) != 0ull) {
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_acc - m_new) * a.scale_log2);
        l_part *= alpha;
#pragma unroll
        for (int mt = 0; mt < D / 16; ++mt) o_acc[mt] *= alpha;
        m_acc = m_new;
      }
      const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
      bf16x4 pf;
      const int keyb = (jb + i) * BK + wave * PAGE + grp * 4;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[i][r], a.scale_log2, -base));
        l_part += p;
        pf[r] = (__bf16)p;
      }
      // tokens past the sequence end hold arbitrary bytes: zero their V so 0 * NaN cannot appear
      const bool tail = keyb + 3 >= L;
#pragma unroll
      for (int mt = 0; mt < D / 16; ++mt) {
        u32x2 vv = vreg[i][mt];
        if (tail) {
          if (keyb + 0 >= L) vv[0] &= 0xffff0000u;
          if (keyb + 1 >= L) vv[0] &= 0x0000ffffu;
          if (keyb + 2 >= L) vv[1] &= 0xffff0000u;
          if (keyb + 3 >= L) vv[1] &= 0x0000ffffu;
        }
        o_acc[mt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4, vv), pf, o_acc[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) pid_cur[i] = pid_next[i];
    // no barrier here: the next batch writes the other sPmax buffer, and this one is rewritten only
    // after the next batch's barrier, which every wave reaches after its reads above
  }

  if (tid == 0 && a.counters) {
    atomicAdd(&a.counters[0], (unsigned long long)live_cnt);
    atomicAdd(&a.counters[1], (unsigned long long)skip_cnt);
  }
  if (a.mask || a.crit) {
    // blocks of the row that no split covers (past the sequence end) are not live; split 0 writes them
    if (split == 0)
      for (int j = J + tid; j < a.nkb; j += 256) {
        if (a.mask) a.mask[mask_row + j] = kNotLive;
        if (a.crit) a.crit[mask_row + j] = __builtin_nanf("");
      }
  }
  if (a.stats_only) return;

  // ---- reduce the 4 waves' partial sums (all used the same running max) ----
  const float lw = sum_xor16_32(l_part);
  if (grp == 0) sL[wave][n] = lw;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) sRed[wave][n][mt * 16 + grp * 4 + r] = o_acc[mt][r];
  __syncthreads();
  // 256 threads: thread -> (column, 8 dv)
  const int col = tid >> 4;          // 0..15
  const int dv0 = (tid & 15) * 8;    // 0..120
  // m_acc of column col lives in the lanes with n == col (the same value in every wave)
  const float m_col = __shfl(m_acc, col);
  if (col < ncol) {
    const float l_tot = sL[0][col] + sL[1][col] + sL[2][col] + sL[3][col];
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float ov[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
      ov[e] = (sRed[0][col][dv0 + e] + sRed[1][col][dv0 + e] + sRed[2][col][dv0 + e] + sRed[3][col][dv0 + e]) * inv;
    const float lse = l_tot > 0.f ? m_col * a.scale + __logf(l_tot) : kNegInf;
    const int ctok = col / a.tile_rows;
    const int h = g * a.G + rt * a.tile_rows + (col - ctok * a.tile_rows);
    const int64_t orow = ((int64_t)b * a.T + ctok) * a.Hq + h;
    if (a.num_splits == 1) {
      const int64_t ob = orow * D + dv0;
      if (OUT_F32) {
        f32x4 w0 = {ov[0], ov[1], ov[2], ov[3]}, w1 = {ov[4], ov[5], ov[6], ov[7]};
        *(f32x4 *)((float *)a.o + ob) = w0;
        *(f32x4 *)((float *)a.o + ob + 4) = w1;
      } else {
        u32x4 w;
        w[0] = pack_bf16x2(ov[0], ov[1]);
        w[1] = pack_bf16x2(ov[2], ov[3]);
        w[2] = pack_bf16x2(ov[4], ov[5]);
        w[3] = pack_bf16x2(ov[6], ov[7]);
        *(u32x4 *)((__bf16 *)a.o + ob) = w;
      }
      if (a.lse && dv0 == 0) a.lse[orow] = lse;
    } else {
      const int64_t pb = orow * a.num_splits + split;
      float *wo = a.ws_o + pb * D + dv0;
      f32x4 w0 = {ov[0], ov[1], ov[2], ov[3]}, w1 = {ov[4], ov[5], ov[6], ov[7]};
      *(f32x4 *)wo = w0;
      *(f32x4 *)(wo + 4) = w1;
      if (dv0 == 0) a.ws_lse[pb] = lse;
    }
  }
}

// Log-sum-exp merge of the per-split partials: one wave per (sequence, q head), four per
// workgroup.  Each lane owns CPL output channels (pairs 2 * lane + 128 k).  The splits are merged in
// chunks of SC with a running max: every load of a chunk (the SC lse values, the same in every lane,
// and the lane's channels of the SC partial rows) is issued before any is used, so a chunk costs one
// memory latency; with S <= SC (the usual case) the whole merge is one round trip.
template <bool OUT_F32, int CPL>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *ws_o, const float *ws_lse, void *o,
                                                              float *lse_out, int BH, int S) {
  constexpr int Dv = CPL * 64, NP = CPL / 2, SC = CPL == 2 ? 16 : 8;
  const int lane = threadIdx.x & 63;
  const int bh = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (bh >= BH) return;
  const float *pl = ws_lse + (int64_t)bh * S;
  const float *po = ws_o + (int64_t)bh * S * Dv + lane * 2;
  float mx = kNegInf, tot = 0.f;  // running max and sum of exp(lse_s - mx) over the merged splits
  float2 acc[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) acc[k] = make_float2(0.f, 0.f);
  for (int s0 = 0; s0 < S; s0 += SC) {
    float ls[SC];
    float2 v[SC][NP];
#pragma unroll
    for (int u = 0; u < SC; ++u) {
      const bool ok = s0 + u < S;
      ls[u] = ok ? pl[s0 + u] : kNegInf;
#pragma unroll
      for (int k = 0; k < NP; ++k)
        v[u][k] = ok ? *(const float2 *)(po + (int64_t)(s0 + u) * Dv + 128 * k) : make_float2(0.f, 0.f);
    }
    float cm = mx;
#pragma unroll
    for (int u = 0; u < SC; ++u) cm = fmaxf(cm, ls[u]);
    if (cm == kNegInf) continue;  // no split so far saw a key
    const float r = mx == kNegInf ? 0.f : __expf(mx - cm);  // rescale of what was merged before
    tot *= r;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      acc[k].x *= r;
      acc[k].y *= r;
    }
#pragma unroll
    for (int u = 0; u < SC; ++u) {
      const float w = ls[u] == kNegInf ? 0.f : __expf(ls[u] - cm);
      tot += w;
#pragma unroll
      for (int k = 0; k < NP; ++k) {
        acc[k].x += w * v[u][k].x;
        acc[k].y += w * v[u][k].y;
      }
    }
    mx = cm;
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int c = lane * 2 + 128 * k;
    if (OUT_F32) {
      *(float2 *)((float *)o + (int64_t)bh * Dv + c) = make_float2(acc[k].x * inv, acc[k].y * inv);
    } else {
      *(uint32_t *)((__bf16 *)o + (int64_t)bh * Dv + c) = pack_bf16x2(acc[k].x * inv, acc[k].y * inv);
    }
  }
  if (lse_out && lane == 0) lse_out[bh] = tot > 0.f ? mx + __logf(tot) : kNegInf;
}

// Dv is 128 (GQA / MHA / MQA) or 512 (latent attention).
hipError_t launch_decode_combine(const DecodeArgs &a, int Dv, hipStream_t st) {
  const int BH = a.B * a.T * a.Hq;  // rows of (sequence, token, q head)
  const int grid = (BH + 3) / 4;
  if (Dv == 128) {
    if (a.out_f32)
      hipLaunchKernelGGL((decode_combine_kernel<true, 2>), dim3(grid), dim3(256), 0, st, a.ws_o, a.ws_lse, a.o, a.lse,
                         BH, a.num_splits);
    else
      hipLaunchKernelGGL((decode_combine_kernel<false, 2>), dim3(grid), dim3(256), 0, st, a.ws_o, a.ws_lse, a.o, a.lse,
                         BH, a.num_splits);
  } else if (Dv == 512) {
    if (a.out_f32)
      hipLaunchKernelGGL((decode_combine_kernel<true, 8>), dim3(grid), dim3(256), 0, st, a.ws_o, a.ws_lse, a.o, a.lse,
                         BH, a.num_splits);
    else
      hipLaunchKernelGGL((decode_combine_kernel<false, 8>), dim3(grid), dim3(256), 0, st, a.ws_o, a.ws_lse, a.o, a.lse,
                         BH, a.num_splits);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

hipError_t launch_decode_gqa(const DecodeArgs &a, hipStream_t st) {
  const int grid = a.B * a.Hkv * a.n_rt * a.num_splits;
  if (!a.decide) {
    if (a.out_f32)
      hipLaunchKernelGGL((decode_gqa_kernel<true, false>), dim3(grid), dim3(256), 0, st, a);
    else
      hipLaunchKernelGGL((decode_gqa_kernel<false, false>), dim3(grid), dim3(256), 0, st, a);
  } else if (a.out_f32) {
    hipLaunchKernelGGL((decode_gqa_kernel<true, true>), dim3(grid), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((decode_gqa_kernel<false, true>), dim3(grid), dim3(256), 0, st, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1 || a.stats_only) return e;
  return launch_decode_combine(a, D, st);
}

}  // namespace blasst

// BLASST decode over a paged latent cache (MLA-shaped: 576-dim scores, V = first 512 latent dims).
//
// Method: as for the other kernels, each 64-token block's row maxima are compared with the running
// maxima of the tile, and a block every row votes to skip gets no exp and no P.V product (pages:
// xllm-io review, 核心公式 and 核心思想 item 4 (MHA/GQA/MQA/MLA); fugumt.com abstract).  In latent
// attention V is the same bytes as K, so a skip saves arithmetic, not HBM traffic.
//
// MI355X design (64-head tiles; the 128-head tile runs the one-wave-per-SIMD kernel of
// decode_mla.hip, which this file's launcher dispatches to):
//   * one workgroup = (sequence, row tile, split); the row tile is TR = 64 rows, one wave per 16
//     rows; the tile's vote is a ballot per wave and one LDS flag per wave;
//   * with T query tokens per sequence (the last T positions) the rows are (token, head) pairs,
//     token-major: row t * tile_rows + i is token t of the tile's head i (tile_rows = TR / T heads),
//     and keys past seq_len - T + t are masked for it like keys past the sequence end (the GQA
//     kernel's multi-token tiles, on the latent cache);
//   * the latent block (64 tokens x 576 channels = 72 KB) goes global -> LDS directly
//     (global_load_lds_dwordx4, issued as assembly so the compiler does not wait for it before the
//     current block's LDS reads), double-buffered and prefetched one block ahead, with the page
//     ids of the next block prefetched as one vector load;
//   * S^T = K q^T with v_mfma_f32_16x16x32_bf16: K rows from LDS (A operand, read two MFMAs ahead
//     in a ring of three), the wave's 16 q heads in registers (B operand, 72 VGPRs); each lane holds
//     16 scores of one head;
//   * O^T = V^T P^T with v_mfma_f32_16x16x32_bf16: P^T comes from the score registers; the V^T
//     operand is read from the same LDS tile with ds_read_b64_tr_b16 (transpose read), so V never
//     needs a second copy; the wave's 16 heads x 512 channels of O live in 128 registers.
//   * the latent row stride (1168 bytes = 144 mod 256) keeps the 16-row score-operand reads free of
//     bank conflicts on the 64-bank LDS (the transpose reads see at most a 2-way conflict);
//   * registers are the scarce resource (q and O of 128 heads are 400 KB of the CU's 512 KB
//     register file), so loops that would hoist every LDS read carry scheduling barriers.
#include "common.hpp"

namespace blasst {

namespace {
constexpr int DQK = 576, DV = 512, PAGE = 16, BK = 64, HPW = 16;
constexpr int CH = DQK / 8;                 // 16-byte chunks per latent row (72)
constexpr int CP = CH + 1;                  // with one pad chunk (row = 1168 bytes = 16 x odd mod 256)
constexpr int ROW = CP * 16;
constexpr int INS = (BK * CP + 63) / 64;    // wave-wide direct loads per block (74)
constexpr int BUF = INS * 1024;
constexpr int KSQ = DQK / 32;               // k-steps of S^T (18)
constexpr int MTK = BK / 16;                // key m-tiles of S^T (4)
constexpr int DVT = DV / 16;                // dv tiles of O^T (32)
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
}  // namespace

template <int TR, bool OUT_F32, bool STATS>
__global__ __launch_bounds__(TR / HPW * 64, 1) void decode_latent_kernel(DecodeArgs a) {
  constexpr int NW = TR / HPW;
  constexpr int NT = NW * 64;
  __shared__ __attribute__((aligned(16))) unsigned char sK[2][BUF];
  __shared__ int sVote[2][NW];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 15;   // row inside the wave
  const int grp = lane >> 4;

  // workgroup -> (sequence, row tile, split); the n_rt row tiles of one (sequence, split) are 8
  // apart in launch order, so they land on the same XCD (round-robin dispatch) and share its L2
  // copy of K
  const int x8 = blockIdx.x & 7;
  const int rt = (blockIdx.x >> 3) % a.n_rt;
  const int bid = (blockIdx.x >> 3) / a.n_rt * 8 + x8;
  const int split = bid % a.num_splits;
  const int b = bid / a.num_splits;
  if (b >= a.B) return;
  const int cap = a.max_pages * PAGE;
  const int L = min(a.seq_lens[b], cap);
  const int J = (L + BK - 1) / BK;
  const int chunk = (J + a.num_splits - 1) / a.num_splits;
  const int j0 = split * chunk;
  const int j1 = min(J, j0 + chunk);
  const int npg = (L + PAGE - 1) / PAGE;
  const int row = wave * HPW + n;            // row of the tile held by this lane
  const int tok = row / a.tile_rows;         // its query token
  const int h = rt * a.tile_rows + (row - tok * a.tile_rows);  // and q head
  const int64_t qrow = ((int64_t)b * a.T + tok) * a.Hq + h;    // row of q (and of o, lse)
  const int lim = L - a.T + tok;             // the last key this row sees

  float thr = a.thr_raw;
  if (a.thr_mode == 1) {
    const float lam = fminf(1.f, a.a / (float)L);
    thr = lam > 0.f ? __logf(lam) / a.scale : kNegInf;
  }

  // q fragments: lane holds dims 32 kk + 8 grp .. +7 of head h
  bf16x8 qf[KSQ];
  const __bf16 *qp = (const __bf16 *)a.q + qrow * DQK;
#pragma unroll
  for (int kk = 0; kk < KSQ; ++kk) qf[kk] = *(const bf16x8 *)(qp + kk * 32 + grp * 8);
  // consume the q loads here, so their waits are not placed inside the block loop (where they
  // would also wait for the block prefetch issued after them)
#pragma unroll
  for (int kk = 0; kk < KSQ; ++kk) asm volatile("" ::"v"(qf[kk]));

  const __bf16 *kc = (const __bf16 *)a.kc;
  const int32_t *table = a.table + (int64_t)b * a.max_pages;
  const int64_t page_stride = (int64_t)PAGE * DQK;   // one kv head

  // page ids of block j: lane l < 4 holds page 4 j + l (clamped to the sequence)
  auto load_table = [&](int j) -> int { return table[min(j * 4 + (lane & 3), npg - 1)]; };
  // direct global -> LDS load of block j (position p = (row p / CP, chunk p % CP); pads load chunk 0)
  auto load_block = [&](int tabv, int buf) {
    // the per-lane positions are recomputed at every call (an opaque copy of the lane id keeps the
    // compiler from precomputing ~20 64-bit addresses and keeping them live across the block loop)
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < (INS + NW - 1) / NW; ++i) {
      const int ins = i * NW + wave;
      const int p = ins * 64 + ln;
      int row = p / CP, c = p - (p / CP) * CP;
      if (c >= CH) c = 0;
      if (row >= BK) row = 0;
      const int pid = __shfl(tabv, row >> 4);
      if (ins < INS)
        direct_load16_nt(kc + (int64_t)pid * page_stride + (row & 15) * DQK + c * 8, lds_addr(sK[buf] + ins * 1024));
    }
  };
  // transpose-read base for the V^T operand: source lane j = 4k + q of 16-lane group G points at
  // latent row 32 t + 16 u + 4 G + k, channels 16 dvt + 4 q .. +3 (u = 0, 1 for the two halves of a
  // 32-key k-step); output lane l then holds channel 16 dvt + l % 16 and the keys of its P^T fragment
  const int tr_off = ((lane >> 4) * 4 + ((lane & 15) >> 2)) * ROW + 4 * (lane & 3) * 2;

  float m_dec = kNegInf, m_acc = kNegInf, l_part = 0.f;
  f32x4 o_acc[DVT];
#pragma unroll
  for (int i = 0; i < DVT; ++i) o_acc[i] = f32x4{};
  unsigned live_cnt = 0, skip_cnt = 0;
  const int mask_row = (b * a.n_rt + rt) * a.nkb;  // one kv head

  int tab_next = 0;
  if (j0 < j1) {
    load_block(load_table(j0), 0);
    tab_next = load_table(j0 + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  for (int j = j0; j < j1; ++j) {
    const int buf = (j - j0) & 1;
    const bool has_next = j + 1 < j1;
    if (has_next) {
      load_block(tab_next, buf ^ 1);
      tab_next = load_table(j + 2 < j1 ? j + 2 : j + 1);
    }
    const int key0 = j * BK;
    if (key0 + BK > L) {
      // slots past the sequence end hold arbitrary bytes: zero them so that P = 0 meets V = 0
      // (0 * NaN cannot appear); their scores are masked below
      const int first = (L - key0) * ROW;
      for (int off16 = first + tid * 16; off16 < BK * ROW; off16 += NT * 16)
        *(u32x4 *)(sK[buf] + off16) = u32x4{};
      __syncthreads();
    }
    // ---- S^T = K_j q^T ----
    f32x4 s[MTK];
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) s[mt] = f32x4{};
    const unsigned char *kb = sK[buf] + n * ROW + grp * 16;
    // step q = (k-step q / MTK, key m-tile q % MTK); its K fragment is read two MFMAs ahead into a
    // ring of three (left to itself, the compiler read each fragment right before its MFMA and waited
    // for it there, with one wave per SIMD and nothing else to hide the LDS latency)
    constexpr int NQK = KSQ * MTK;
    auto read_kf = [&](int q) { return *(const bf16x8 *)(kb + (q % MTK) * 16 * ROW + (q / MTK) * 64); };
    bf16x8 kr[3];
    kr[0] = read_kf(0);
    kr[1] = read_kf(1);
#pragma unroll
    for (int q = 0; q < NQK; ++q) {
      if (q + 2 < NQK) kr[(q + 2) % 3] = read_kf(q + 2);
      s[q % MTK] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[q % 3], qf[q / MTK], s[q % MTK], 0, 0, 0);
      if ((q & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
    if (key0 + BK > L - a.T + 1) {   // keys past a row's last visible key (or the sequence end)
#pragma unroll
      for (int mt = 0; mt < MTK; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key0 + mt * 16 + grp * 4 + r > lim) s[mt][r] = kNegInf;
    }
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < MTK; ++mt) mx = fmaxf(mx, fmaxf(fmaxf(s[mt][0], s[mt][1]), fmaxf(s[mt][2], s[mt][3])));
    mx = max_xor16_32(mx);
    const bool skip_row = row_votes_skip(mx, m_dec, thr);
    const bool wave_keep = __ballot(!skip_row) != 0ull;
    float wcrit = 0.f;
    if (a.crit) {
      wcrit = row_crit(mx, m_dec);
      wcrit = fmaxf(wcrit, __shfl_xor(wcrit, 8));
      wcrit = fmaxf(wcrit, __shfl_xor(wcrit, 4));
      wcrit = fmaxf(wcrit, __shfl_xor(wcrit, 2));
      wcrit = fmaxf(wcrit, __shfl_xor(wcrit, 1));
    }
    if (lane == 0) {
      sVote[buf][wave] = wave_keep ? 1 : 0;
      sCrit[buf][wave] = wcrit;
    }
    barrier_lds_only();  // vote barrier (the next block's loads stay in flight)
    int keep = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) keep |= sVote[buf][w];
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
      const float m_new = fmaxf(m_acc, mx);
      if (__ballot(m_new > m_acc) != 0ull) {
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_acc - m_new) * a.scale_log2);
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < DVT; ++i) o_acc[i] *= alpha;
        m_acc = m_new;
      }
      const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
      // P^T of 32-key k-step t: s[2t] (keys 32t + 4 grp + r) then s[2t+1] (keys 32t + 16 + 4 grp + r)
      bf16x8 pf[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float p = fast_exp2(__builtin_fmaf(s[2 * t + u][r], a.scale_log2, -base));
            l_part += p;
            pf[t][u * 4 + r] = (__bf16)p;
          }
      const unsigned char *vb = sK[buf] + tr_off;
#pragma unroll
      for (int dvt = 0; dvt < DVT; ++dvt) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + (32 * t) * ROW + dvt * 32));
          const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + (32 * t + 16) * ROW + dvt * 32));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
          o_acc[dvt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[t], o_acc[dvt], 0, 0, 0);
        }
        if ((dvt & 3) == 3) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (has_next) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();  // buffer-swap barrier
    }
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

  // ---- per-lane partial sums over its keys -> per head; O^T lane layout: head n, dv 16 dvt + 4 grp + r
  const float l_tot = sum_xor16_32(l_part);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse = l_tot > 0.f ? m_acc * a.scale + __logf(l_tot) : kNegInf;
  if (a.num_splits == 1) {
    const int64_t ob = qrow * DV + grp * 4;
#pragma unroll
    for (int dvt = 0; dvt < DVT; ++dvt) {
      if (OUT_F32) {
        *(f32x4 *)((float *)a.o + ob + dvt * 16) = o_acc[dvt] * inv;
      } else {
        u32x2 w;
        w[0] = pack_bf16x2(o_acc[dvt][0] * inv, o_acc[dvt][1] * inv);
        w[1] = pack_bf16x2(o_acc[dvt][2] * inv, o_acc[dvt][3] * inv);
        *(u32x2 *)((__bf16 *)a.o + ob + dvt * 16) = w;
      }
    }
    if (a.lse && grp == 0) a.lse[qrow] = lse;
  } else {
    const int64_t pb = qrow * a.num_splits + split;
    float *wo = a.ws_o + pb * DV + grp * 4;
#pragma unroll
    for (int dvt = 0; dvt < DVT; ++dvt) *(f32x4 *)(wo + dvt * 16) = o_acc[dvt] * inv;
    if (grp == 0) a.ws_lse[pb] = lse;
  }
}

hipError_t launch_decode_combine(const DecodeArgs &a, int Dv, hipStream_t st);

template <int TR>
static void launch_tr(const DecodeArgs &a, int grid, hipStream_t st) {
  constexpr int NT = TR / HPW * 64;
  if (a.stats_only)
    hipLaunchKernelGGL((decode_latent_kernel<TR, false, true>), dim3(grid), dim3(NT), 0, st, a);
  else if (a.out_f32)
    hipLaunchKernelGGL((decode_latent_kernel<TR, true, false>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((decode_latent_kernel<TR, false, false>), dim3(grid), dim3(NT), 0, st, a);
}

hipError_t launch_decode_mla128(const DecodeArgs &a, hipStream_t st);

hipError_t launch_decode_latent(const DecodeArgs &a, hipStream_t st) {
  if (a.Hq != 128 || a.Hkv != 1 || a.page != PAGE || a.block_k != BK) return hipErrorNotSupported;
  if (a.T * a.tile_rows == 128) {
    // 128-row tiles (all 128 heads, or T tokens x 128 / T heads): the one-wave-per-SIMD kernel
    // (decode_mla.hip)
    const hipError_t e = launch_decode_mla128(a, st);
    if (e != hipSuccess || a.num_splits == 1 || a.stats_only) return e;
    return launch_decode_combine(a, DV, st);
  } else if (a.T * a.tile_rows == 64) {
    // 64-row tiles (64 heads, or 2 tokens x 32 heads, or 4 tokens x 16 heads), n_rt per (sequence,
    // split): round the (sequence, split) count up to a multiple of 8 (see the kernel's mapping)
    const int pairs = (a.B * a.num_splits + 7) / 8 * 8;
    launch_tr<64>(a, pairs * a.n_rt, st);
  } else {
    return hipErrorNotSupported;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.num_splits == 1 || a.stats_only) return e;
  return launch_decode_combine(a, DV, st);
}

}  // namespace blasst

// BLASST prefill forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method: FlashAttention-style tiled online softmax over the KV blocks of a query tile, visited
// left to right; block j is skipped when every row of the tile has m~ - m < ln(lambda), and a
// skipped block gets no exp and no P.V product, while QK^T is still computed for every block and
// the V block is still staged (pages: xllm-io review, 核心公式 and 预填充内核优化; gist.science (de),
// 2. Methodik / Kernidee and 3. Kernel-Design).
//
// MI355X design:
//   * a workgroup owns TPW query tiles that read the same K/V stream (two q heads of one GQA group
//     at the same query position), so every staged K/V block serves 2 * BR query rows; each tile
//     has BR = 32 * WPT rows, one wave per 32 rows, and votes on its own;
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the A operand
//     (K) comes from LDS, the B operand (Q) stays in registers for the whole tile, and each lane
//     ends up holding all scores of ONE query row, so the block row max is an in-lane max plus one
//     exchange with lane l ^ 32;
//   * P^T is packed to bf16 straight from the score registers and used as the B operand of
//     O^T = V^T P^T; V is written to LDS transposed (key-contiguous rows, keys permuted to match
//     the score register layout) so that every MFMA operand read is one 16-byte LDS read;
//   * K goes global -> LDS directly (global_load_lds_dwordx4, no registers), V goes through
//     registers for the transpose; both are prefetched one block ahead into double-buffered LDS,
//     so a block costs two barriers: the vote barrier and the buffer-swap barrier;
//   * the skip vote: per-row predicate -> wave ballot -> one LDS flag per wave -> OR over the
//     tile's waves after the vote barrier; the skip is a uniform branch, so a skipped block issues
//     no v_exp and no P.V MFMA;
//   * every LDS row carries one 16-byte pad chunk, so the 32 rows an MFMA operand read touches fall
//     on distinct banks and every read address is one per-lane base plus an immediate;
//   * heavy (late, long causal) tiles launch first, and workgroups of one kv head are mapped to the
//     same XCD (workgroups are dispatched round-robin over the 8 XCDs) for L2 reuse.
#include "common.hpp"

namespace blasst {

typedef __attribute__((address_space(3))) void lds_void;

template <int D, int BC, int TPW, bool OUT_F32, bool STATS>
__global__ __launch_bounds__(64 * (BC / 32) * TPW, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int WPT = BC / 32;       // waves per tile (32 rows each)
  constexpr int BR = BC;             // rows per tile
  constexpr int NW = WPT * TPW;      // waves per workgroup
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int KCP = KCH + 1;       // ... plus the pad chunk
  constexpr int KROW = KCP * 16;     // bytes per K row in LDS
  constexpr int VROW = BC * 2 + 16;  // bytes per V^T row in LDS
  constexpr int MT = BC / 32;        // key m-tiles of S^T
  constexpr int KS = D / 16;         // k-steps over the head dim
  constexpr int MTV = D / 32;        // dv m-tiles of O^T
  constexpr int KSV = BC / 16;       // k-steps over the keys of a block
  constexpr int KPOS = BC * KCP;     // 16-byte positions of a K tile (pads included)
  constexpr int KINS = (KPOS + 63) / 64;            // wave-wide direct loads per K tile
  constexpr int KINS_W = (KINS + NW - 1) / NW;      // ... per wave
  constexpr int KBUF = KINS_W * NW * 64 * 16;       // bytes per K buffer (covers every wave's writes)
  constexpr int VBUF = D * VROW;
  constexpr int LPO = D / 2;                        // lanes per key octet (one dv pair per lane)
  constexpr int OPW = 64 / LPO;                     // key octets per wave instruction
  constexpr int V_TASKS = (BC / 8) / (NW * OPW);    // octet groups per wave
  static_assert((BC / 8) % (NW * OPW) == 0, "tile/thread mismatch");

  __shared__ __attribute__((aligned(16))) unsigned char sK[2][KBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sV[2][VBUF];
  __shared__ int sVote[2][NW];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave / WPT;       // tile of this wave inside the workgroup
  const int wit = wave % WPT;        // wave index inside its tile
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- tile coordinates: heavy causal tiles first, kv-head groups kept on one XCD ----------------
  const int groups = a.Hq / TPW;               // head groups of TPW heads sharing a kv head
  const int per_level = a.B * groups;
  const int bid = blockIdx.x;
  const int level = bid / per_level;
  int rem = bid - level * per_level;
  if ((per_level & 7) == 0) rem = (rem & 7) * (per_level >> 3) + (rem >> 3);
  const int qt = a.causal ? (a.nqt - 1 - level) : level;
  const int b = rem / groups;
  const int hq0 = (rem - b * groups) * TPW;    // first head of the group
  const int hq = hq0 + tile;
  const int g = hq0 / a.G;                     // TPW divides G, so the group shares kv head g
  const int r0 = qt * BR;
  const int off = a.Lk - a.Lq;                 // bottom-right causal alignment

  const __bf16 *qp = (const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1];
  const __bf16 *kp = (const __bf16 *)a.k + b * a.ks[0] + g * a.ks[1];
  const __bf16 *vp = (const __bf16 *)a.v + b * a.vs[0] + g * a.vs[1];

  const int last_row = min(r0 + BR, a.Lq) - 1;
  int J;  // live blocks (the same for every tile of the workgroup)
  if (a.causal) {
    const int lim = last_row + off;
    J = lim < 0 ? 0 : min(a.nkb, lim / BC + 1);
  } else {
    J = a.nkb;
  }
  const int chunk = J > 0 ? (J + a.num_splits - 1) / a.num_splits : 1;

  // ---- Q fragments (B operand of S^T = K Q^T): row l32 of this wave, 8 dims per k-step ----------
  const int my_row = r0 + wit * 32 + l32;
  const bool row_ok = my_row < a.Lq;
  bf16x8 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    qf[kk] = row_ok ? *(const bf16x8 *)(qp + (int64_t)my_row * a.qs[2] + kk * 16 + hi * 8) : bf16x8{};

  // ---- staging ---------------------------------------------------------------------------------
  // K: direct global -> LDS.  Position p of a K buffer is (row p / KCP, chunk p % KCP); pad chunks
  // and positions past the tile load row 0 / the last valid key so every lane reads valid memory.
  auto load_k = [&](int j, int buf) {
    const int key0 = j * BC;
#pragma unroll
    for (int i = 0; i < KINS_W; ++i) {
      const int ins = i * NW + wave;
      const int p = ins * 64 + lane;
      int row = p / KCP, c = p - (p / KCP) * KCP;
      if (c == KCH) c = 0;
      if (row >= BC) row = 0;
      const int key = min(key0 + row, a.Lk - 1);
      __builtin_amdgcn_global_load_lds((const void *)(kp + (int64_t)key * a.ks[2] + c * 8),
                                       (lds_void *)(sK[buf] + ins * 1024), 16, 0, 0);
    }
  };
  // V: a lane loads one dv pair (4 bytes) of each of the 8 keys of a key octet, so every load
  // instruction reads whole rows; it then writes two 16-byte V^T pieces.  Key order inside each
  // 16-key chunk is 0-3, 8-11, 4-7, 12-15: octet o (16 bytes at byte 16*o of a V^T row) holds the
  // 8 keys that lane half (o % 2) of P^T k-step (o / 2) carries.
  uint32_t vreg[V_TASKS][8];
  const int v_dp = lane % LPO;
  const int v_sub = lane / LPO;
  auto load_v = [&](int j) {
#pragma unroll
    for (int t = 0; t < V_TASKS; ++t) {
      const int o = (t * NW + wave) * OPW + v_sub;
      const int kb = j * BC + (o >> 1) * 16 + (o & 1) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb + (e >> 2) * 8 + (e & 3);
        vreg[t][e] = key < a.Lk ? *(const uint32_t *)(vp + (int64_t)key * a.vs[2] + 2 * v_dp) : 0u;
      }
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int t = 0; t < V_TASKS; ++t) {
      const int o = (t * NW + wave) * OPW + v_sub;
      u32x4 lo, hi2;  // dv 2*v_dp (low halves) and 2*v_dp+1 (high halves) of the 8 keys
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x0 = vreg[t][2 * i], x1 = vreg[t][2 * i + 1];
        lo[i] = __builtin_amdgcn_perm(x1, x0, 0x05040100u);
        hi2[i] = __builtin_amdgcn_perm(x1, x0, 0x07060302u);
      }
      *(u32x4 *)(sV[buf] + (2 * v_dp) * VROW + o * 16) = lo;
      *(u32x4 *)(sV[buf] + (2 * v_dp + 1) * VROW + o * 16) = hi2;
    }
  };

  // ---- online-softmax state (per lane: query row l32 of this wave) -----------------------------
  float m_dec = kNegInf;  // running max used by the skip rule (restarts at each split)
  float m_acc = kNegInf;  // running max of the accumulation
  float l_part = 0.f;     // partial row sum over the keys this lane holds
  f32x16 o_acc[MTV];
#pragma unroll
  for (int i = 0; i < MTV; ++i) o_acc[i] = f32x16{};
  unsigned live_cnt = 0, skip_cnt = 0;
  const int mask_row = ((b * a.Hq + hq) * a.nqt + qt) * a.nkb;
  const bool tile_leader = wit == 0 && lane == 0;

  if (J > 0) {
    load_k(0, 0);
    if (!STATS) {
      load_v(0);
      store_v(0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  for (int j = 0; j < J; ++j) {
    const int buf = j & 1;
    const bool has_next = j + 1 < J;
    if (has_next) {
      load_k(j + 1, buf ^ 1);
      if (!STATS) load_v(j + 1);
    }
    if ((j % chunk) == 0) m_dec = kNegInf;

    // ---- S^T = K_j Q^T ----
    f32x16 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = f32x16{};
    const unsigned char *kb = sK[buf] + l32 * KROW + hi * 16;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 kf = *(const bf16x8 *)(kb + mt * 32 * KROW + kk * 32);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[mt], 0, 0, 0);
      }
    }

    // ---- causal / tail mask (only blocks that need it) ----
    const int key0 = j * BC;
    const bool need_mask = (key0 + BC > a.Lk) || (a.causal && key0 + BC - 1 > r0 + off);
    if (need_mask) {
      const int lim = a.causal ? min(my_row + off, a.Lk - 1) : a.Lk - 1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = key0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (key > lim) s[mt][r] = kNegInf;
        }
    }

    // ---- block row max, vote, critical value ----
    float mx = kNegInf;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
    mx = max_xor32(mx);
    if (!row_ok) mx = kNegInf;
    const bool skip_row = row_votes_skip(mx, m_dec, a.thr_raw);
    const bool wave_keep = __ballot(!skip_row) != 0ull;
    float wcrit = 0.f;
    if (a.crit) wcrit = max_lanes32(row_crit(mx, m_dec));
    if (lane == 0) {
      sVote[buf][wave] = wave_keep ? 1 : 0;
      sCrit[buf][wave] = wcrit;
    }
    __syncthreads();  // vote barrier
    int keep = 0;
#pragma unroll
    for (int w = 0; w < WPT; ++w) keep |= sVote[buf][tile * WPT + w];
    m_dec = fmaxf(m_dec, mx);
    ++live_cnt;
    if (!keep) ++skip_cnt;
    if (tile_leader) {
      if (a.mask) a.mask[mask_row + j] = keep ? kKept : kSkipped;
      if (a.crit) {
        float c = sCrit[buf][tile * WPT];
#pragma unroll
        for (int w = 1; w < WPT; ++w) c = fmaxf(c, sCrit[buf][tile * WPT + w]);
        a.crit[mask_row + j] = c * a.scale;
      }
    }

    if (!STATS && keep) {
      // ---- kept block: online-softmax update and O^T += V^T P^T ----
      const float m_new = fmaxf(m_acc, mx);
      if (__ballot(m_new > m_acc) != 0ull) {
        const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_acc - m_new) * a.scale_log2);
        l_part *= alpha;
#pragma unroll
        for (int i = 0; i < MTV; ++i) o_acc[i] *= alpha;
        m_acc = m_new;
      }
      const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
      const unsigned char *vb = sV[buf] + l32 * VROW + hi * 16;
      // P^T for k-step kk (16 keys) is formed right before its MFMAs: keys of score registers
      // s[kk/2][8*(kk%2) .. +7], i.e. key 16*kk + 8*(e/4) + 4*hi + e%4 for element e.
#pragma unroll
      for (int kk = 0; kk < KSV; ++kk) {
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float p = fast_exp2(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + e], a.scale_log2, -base));
          l_part += p;
          pf[e] = (__bf16)p;
        }
#pragma unroll
        for (int mv = 0; mv < MTV; ++mv) {
          const bf16x8 vf = *(const bf16x8 *)(vb + mv * 32 * VROW + kk * 32);
          o_acc[mv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o_acc[mv], 0, 0, 0);
        }
      }
    }
    if (has_next) {
      if (!STATS) store_v(buf ^ 1);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the direct K loads have landed in LDS
      __syncthreads();  // buffer-swap barrier
    }
  }

  // ---- diagnostics for blocks that are not live ----
  if (a.mask || a.crit) {
    for (int j = J + wit * 64 + lane; j < a.nkb; j += WPT * 64) {
      if (a.mask) a.mask[mask_row + j] = kNotLive;
      if (a.crit) a.crit[mask_row + j] = __builtin_nanf("");
    }
  }
  if (a.counters && tile_leader) {
    atomicAdd(&a.counters[0], (unsigned long long)live_cnt);
    atomicAdd(&a.counters[1], (unsigned long long)skip_cnt);
  }
  if (STATS) return;

  // ---- epilogue: O = O^T / l, LSE = m * scale + ln l ----
  const float l_row = l_part + __shfl_xor(l_part, 32);
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  if (row_ok) {
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + my_row] =
          l_row > 0.f ? m_acc * a.scale + __logf(l_row) : kNegInf;
    if (OUT_F32) {
      float *op = (float *)a.o + b * a.os[0] + hq * a.os[1] + (int64_t)my_row * a.os[2];
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          f32x4 v4;
#pragma unroll
          for (int e = 0; e < 4; ++e) v4[e] = o_acc[mv][rg * 4 + e] * inv;
          *(f32x4 *)(op + mv * 32 + 8 * rg + 4 * hi) = v4;
        }
    } else {
      __bf16 *op = (__bf16 *)a.o + b * a.os[0] + hq * a.os[1] + (int64_t)my_row * a.os[2];
#pragma unroll
      for (int mv = 0; mv < MTV; ++mv)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          u32x2 w2;
          w2[0] = pack_bf16x2(o_acc[mv][rg * 4 + 0] * inv, o_acc[mv][rg * 4 + 1] * inv);
          w2[1] = pack_bf16x2(o_acc[mv][rg * 4 + 2] * inv, o_acc[mv][rg * 4 + 3] * inv);
          *(u32x2 *)(op + mv * 32 + 8 * rg + 4 * hi) = w2;
        }
    }
  }
}

template <int D, int BC, int TPW>
static hipError_t launch_tpw(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  constexpr int NT = 64 * (BC / 32) * TPW;
  const int grid = a.B * (a.Hq / TPW) * a.nqt;
  if (a.stats_only)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, TPW, false, true>), dim3(grid), dim3(NT), 0, st, a);
  else if (out_f32)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, TPW, true, false>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, TPW, false, false>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t launch_one(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  // two q heads of one GQA group share each staged K/V block when the group has an even size
  if (a.G % 2 == 0) return launch_tpw<D, BC, 2>(a, out_f32, st);
  return launch_tpw<D, BC, 1>(a, out_f32, st);
}

// Returns hipErrorNotSupported when no instantiation matches.
hipError_t launch_prefill_bf16(const PrefillArgs &a, int D, int BC, bool out_f32, hipStream_t st) {
  if (D == 128 && BC == 128) return launch_one<128, 128>(a, out_f32, st);
  if (D == 128 && BC == 64) return launch_one<128, 64>(a, out_f32, st);
  if (D == 64 && BC == 128) return launch_one<64, 128>(a, out_f32, st);
  if (D == 64 && BC == 64) return launch_one<64, 64>(a, out_f32, st);
  return hipErrorNotSupported;
}

}  // namespace blasst

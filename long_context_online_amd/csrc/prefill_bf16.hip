// BLASST prefill forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method: FlashAttention-style tiled online softmax over the KV blocks of a query tile, visited
// left to right; block j is skipped when every row of the tile has m~ - m < ln(lambda), and a
// skipped block gets no exp and no P.V product, while QK^T is still computed for every block and
// the V block is still staged (pages: xllm-io review, 核心公式 and 预填充内核优化; gist.science (de),
// 2. Methodik / Kernidee and 3. Kernel-Design).
//
// MI355X design:
//   * one workgroup = one query tile of BR = 32 * NW rows of one q head (NW waves, 32 rows each);
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the A operand
//     (K) comes from LDS, the B operand (Q) stays in registers for the whole tile, and each lane
//     ends up holding 64 scores of ONE query row, so the block row max is an in-lane max plus one
//     exchange with lane l ^ 32;
//   * P^T is packed to bf16 straight from the score registers and used as the B operand of
//     O^T = V^T P^T; V is written to LDS transposed (key-contiguous rows, keys permuted to match
//     the score register layout) so that every MFMA operand read is one 16-byte LDS read;
//   * the skip vote: per-row predicate -> wave ballot -> one LDS flag per wave -> workgroup OR,
//     folded into a barrier the tile loop needs anyway; the skip is a uniform branch, so a skipped
//     block issues no v_exp and no P.V MFMA;
//   * the next block's K and V are prefetched into registers while the current block computes;
//   * heavy (late, long causal) tiles launch first, and workgroups that share a kv head are
//     mapped to the same XCD (blocks are dispatched round-robin over the 8 XCDs) for L2 reuse.
#include "common.hpp"

namespace blasst {

template <int D, int BC, int NW, bool OUT_F32>
__global__ __launch_bounds__(64 * NW, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int BR = 32 * NW;
  constexpr int NT = 64 * NW;
  constexpr int KCH = D / 8;        // 16-byte chunks per K row
  constexpr int KROW = D * 2 + 16;  // bytes per K row in LDS (one 16-byte pad chunk per row)
  constexpr int VROW = BC * 2 + 16; // bytes per V^T row in LDS
  constexpr int MT = BC / 32;       // key m-tiles of S^T
  constexpr int KS = D / 16;        // k-steps over the head dim
  constexpr int MTV = D / 32;       // dv m-tiles of O^T
  constexpr int KSV = BC / 16;      // k-steps over the keys of a block
  constexpr int K_LOADS = BC * KCH / NT;          // 16-byte K chunks per thread
  constexpr int LPO = D / 2;                      // lanes per key octet (one dv pair per lane)
  constexpr int OPW = 64 / LPO;                   // key octets per wave instruction
  constexpr int V_TASKS = (BC / 8) / (NW * OPW);  // octet groups per wave
  static_assert(BC * KCH % NT == 0 && (BC / 8) % (NW * OPW) == 0, "tile/thread mismatch");
  static_assert(BR == BC, "square tiles");

  __shared__ __attribute__((aligned(16))) unsigned char sK[BC * KROW];
  __shared__ __attribute__((aligned(16))) unsigned char sV[D * VROW];
  __shared__ int sVote[2][NW];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- tile coordinates: heavy causal tiles first, kv-head groups kept on one XCD ----------------
  const int per_level = a.B * a.Hq;
  const int bid = blockIdx.x;
  const int level = bid / per_level;
  int rem = bid - level * per_level;
  if ((per_level & 7) == 0) rem = (rem & 7) * (per_level >> 3) + (rem >> 3);
  const int qt = a.causal ? (a.nqt - 1 - level) : level;
  const int b = rem / a.Hq;
  const int hq = rem - b * a.Hq;
  const int g = hq / a.G;
  const int r0 = qt * BR;
  const int off = a.Lk - a.Lq;  // bottom-right causal alignment

  const __bf16 *qp = (const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1];
  const __bf16 *kp = (const __bf16 *)a.k + b * a.ks[0] + g * a.ks[1];
  const __bf16 *vp = (const __bf16 *)a.v + b * a.vs[0] + g * a.vs[1];

  const int last_row = min(r0 + BR, a.Lq) - 1;
  int J;  // live blocks of this tile
  if (a.causal) {
    const int lim = last_row + off;
    J = lim < 0 ? 0 : min(a.nkb, lim / BC + 1);
  } else {
    J = a.nkb;
  }
  const int chunk = J > 0 ? (J + a.num_splits - 1) / a.num_splits : 1;

  // ---- Q fragments (B operand of S^T = K Q^T): row l32 of this wave, 8 dims per k-step ----------
  const int my_row = r0 + wave * 32 + l32;
  const bool row_ok = my_row < a.Lq;
  bf16x8 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    if (row_ok)
      qf[kk] = *(const bf16x8 *)(qp + (int64_t)my_row * a.qs[2] + kk * 16 + hi * 8);
    else
      qf[kk] = bf16x8{};
  }

  // ---- register staging of the K and V tiles (global -> registers -> LDS) ----------------------
  // K is stored row-major with a 16-byte pad per row: the 32 rows one MFMA operand read touches
  // fall on distinct banks, and every read address is one per-lane base plus an immediate.
  // V is stored transposed (V^T, one row per dv) with the keys of each 16-key chunk in the order
  // 0-3, 8-11, 4-7, 12-15: "octet" o (16 bytes at byte 16*o of a row) then holds exactly the 8
  // keys that lane half (o % 2) of P^T k-step (o / 2) carries.  A lane loads one dv pair (4 bytes)
  // of each of the octet's 8 keys, so every global load instruction reads whole 256-byte rows.
  u32x4 kreg[K_LOADS];
  uint32_t vreg[V_TASKS][8];
  const int v_dp = lane % LPO;              // dv pair of this lane
  const int v_sub = lane / LPO;             // octet within the wave instruction
  auto load_k = [&](int j) {
    const int key0 = j * BC;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / KCH, c = idx % KCH;
      const int key = key0 + row;
      kreg[i] = key < a.Lk ? *(const u32x4 *)(kp + (int64_t)key * a.ks[2] + c * 8) : u32x4{};
    }
  };
  auto load_v = [&](int j) {
#pragma unroll
    for (int t = 0; t < V_TASKS; ++t) {
      const int o = (t * NW + wave) * OPW + v_sub;           // octet index in the block
      const int kb = j * BC + (o >> 1) * 16 + (o & 1) * 4;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int key = kb + (e >> 2) * 8 + (e & 3);
        vreg[t][e] = key < a.Lk ? *(const uint32_t *)(vp + (int64_t)key * a.vs[2] + 2 * v_dp) : 0u;
      }
    }
  };
  auto store_k = [&]() {
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / KCH, c = idx % KCH;
      *(u32x4 *)(sK + row * KROW + c * 16) = kreg[i];
    }
  };
  auto store_v = [&]() {
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
      *(u32x4 *)(sV + (2 * v_dp) * VROW + o * 16) = lo;
      *(u32x4 *)(sV + (2 * v_dp + 1) * VROW + o * 16) = hi2;
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

  // Per block j, with single LDS buffers and three barriers:
  //   K_{j+1} -> regs | S^T from sK | vote -> barrier A | K_{j+1} -> sK, V_{j+1} -> regs |
  //   (kept) softmax, P.V from sV | barrier B | V_{j+1} -> sV | barrier C
  // so the K registers are dead before the softmax and the V registers are only live during it.
  if (J > 0) {
    load_k(0);
    load_v(0);
    store_k();
    store_v();
    __syncthreads();
  }
  for (int j = 0; j < J; ++j) {
    const bool has_next = j + 1 < J;
    if (has_next) load_k(j + 1);
    if ((j % chunk) == 0) m_dec = kNegInf;

    // ---- S^T = K_j Q^T ----
    f32x16 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const bf16x8 kf = *(const bf16x8 *)(sK + (mt * 32 + l32) * KROW + (kk * 2 + hi) * 16);
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
      sVote[j & 1][wave] = wave_keep ? 1 : 0;
      sCrit[j & 1][wave] = wcrit;
    }
    __syncthreads();  // barrier A: votes visible, every wave is done reading sK
    if (has_next) {
      store_k();
      load_v(j + 1);
    }
    int keep = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) keep |= sVote[j & 1][w];
    m_dec = fmaxf(m_dec, mx);
    ++live_cnt;
    if (!keep) ++skip_cnt;
    if (tid == 0) {
      if (a.mask) a.mask[mask_row + j] = keep ? kKept : kSkipped;
      if (a.crit) {
        float c = sCrit[j & 1][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) c = fmaxf(c, sCrit[j & 1][w]);
        a.crit[mask_row + j] = c * a.scale;
      }
    }
    if (keep && !a.stats_only) {

    // ---- kept block: online-softmax update and O^T += V^T P^T ----
    const float m_new = fmaxf(m_acc, mx);
    const bool grow = m_new > m_acc;
    if (__ballot(grow) != 0ull) {
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_acc - m_new) * a.scale_log2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < MTV; ++i) o_acc[i] *= alpha;
      m_acc = m_new;
    }
    const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
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
        const bf16x8 vf = *(const bf16x8 *)(sV + (mv * 32 + l32) * VROW + (kk * 2 + hi) * 16);
        o_acc[mv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o_acc[mv], 0, 0, 0);
      }
    }
    }  // kept block
    if (has_next) {
      __syncthreads();  // barrier B: every wave is done reading sV
      store_v();
      __syncthreads();  // barrier C: K_{j+1} and V_{j+1} visible
    }
  }

  // ---- diagnostics for blocks that are not live ----
  if (a.mask || a.crit) {
    for (int j = J + tid; j < a.nkb; j += NT) {
      if (a.mask) a.mask[mask_row + j] = kNotLive;
      if (a.crit) a.crit[mask_row + j] = __builtin_nanf("");
    }
  }
  if (a.counters && tid == 0) {
    atomicAdd(&a.counters[0], (unsigned long long)live_cnt);
    atomicAdd(&a.counters[1], (unsigned long long)skip_cnt);
  }
  if (a.stats_only) return;

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

template <int D, int BC, bool OUT_F32>
static hipError_t launch_one(const PrefillArgs &a, hipStream_t st) {
  constexpr int NW = BC / 32;
  const int grid = a.B * a.Hq * a.nqt;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, NW, OUT_F32>), dim3(grid), dim3(64 * NW), 0, st, a);
  return hipGetLastError();
}

// Returns hipErrorNotSupported when no instantiation matches.
hipError_t launch_prefill_bf16(const PrefillArgs &a, int D, int BC, bool out_f32, hipStream_t st) {
  if (D == 128 && BC == 128) return out_f32 ? launch_one<128, 128, true>(a, st) : launch_one<128, 128, false>(a, st);
  if (D == 128 && BC == 64) return out_f32 ? launch_one<128, 64, true>(a, st) : launch_one<128, 64, false>(a, st);
  if (D == 64 && BC == 128) return out_f32 ? launch_one<64, 128, true>(a, st) : launch_one<64, 128, false>(a, st);
  if (D == 64 && BC == 64) return out_f32 ? launch_one<64, 64, true>(a, st) : launch_one<64, 64, false>(a, st);
  return hipErrorNotSupported;
}

}  // namespace blasst

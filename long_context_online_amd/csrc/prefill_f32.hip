// BLASST prefill forward for fp32 inputs and outputs (fp32 MFMA, v_mfma_f32_32x32x2_f32).
//
// Same rule and tile loop as the bf16 kernel (pages: xllm-io review, 核心公式 and 预填充内核优化;
// gist.science (de), 2. Methodik / Kernidee): QK^T for every live block, block row max, tile vote,
// and for kept blocks only the exp and the P.V product.  This variant keeps full fp32 operands; it
// serves small fp32 problems (64 x 64 tiles, head dim 64 or 128).  Scores are computed transposed
// (S^T = K Q^T) so each lane holds one query row; with the k = 2 fp32 MFMA every operand is one
// float per lane, so K and V are staged in LDS row-major (one padding float per row keeps the
// 32 rows read by one MFMA operand on distinct banks) and P^T is the score register itself.
#include "common.hpp"

namespace blasst {

template <int D>
__global__ __launch_bounds__(128, 2) void prefill_f32_kernel(PrefillArgs a) {
  constexpr int NW = 2, BR = 64, BC = 64, NT = 128;
  constexpr int LD = D + 1;          // padded LDS row (floats)
  constexpr int MT = BC / 32;        // key m-tiles
  constexpr int KS = D / 2;          // k-steps of S^T
  constexpr int MTV = D / 32;        // dv m-tiles
  constexpr int CH = D / 4;          // float4 chunks per row
  constexpr int LOADS = BC * CH / NT;

  __shared__ float sK[BC * LD];
  __shared__ float sV[BC * LD];
  __shared__ int sVote[2][NW];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  const int per_level = a.B * a.Hq;
  const int bid = blockIdx.x;
  const int level = bid / per_level;
  const int rem = bid - level * per_level;
  const int qt = a.causal ? (a.nqt - 1 - level) : level;
  const int b = rem / a.Hq;
  const int hq = rem - b * a.Hq;
  const int g = hq / a.G;
  const int r0 = qt * BR;
  const int off = a.Lk - a.Lq;

  const float *qp = (const float *)a.q + b * a.qs[0] + hq * a.qs[1];
  const float *kp = (const float *)a.k + b * a.ks[0] + g * a.ks[1];
  const float *vp = (const float *)a.v + b * a.vs[0] + g * a.vs[1];

  const int last_row = min(r0 + BR, a.Lq) - 1;
  int J;
  if (a.causal) {
    const int lim = last_row + off;
    J = lim < 0 ? 0 : min(a.nkb, lim / BC + 1);
  } else {
    J = a.nkb;
  }
  const int chunk = J > 0 ? (J + a.num_splits - 1) / a.num_splits : 1;

  const int my_row = r0 + wave * 32 + l32;
  const bool row_ok = my_row < a.Lq;
  float qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) qf[kk] = row_ok ? qp[(int64_t)my_row * a.qs[2] + kk * 2 + hi] : 0.f;

  f32x4 kreg[LOADS], vreg[LOADS];
  auto load_tiles = [&](int j) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CH, c = idx % CH;
      const int key = j * BC + row;
      kreg[i] = key < a.Lk ? *(const f32x4 *)(kp + (int64_t)key * a.ks[2] + c * 4) : f32x4{};
      vreg[i] = key < a.Lk ? *(const f32x4 *)(vp + (int64_t)key * a.vs[2] + c * 4) : f32x4{};
    }
  };
  auto store_tiles = [&]() {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int idx = tid + i * NT;
      const int row = idx / CH, c = idx % CH;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sK[row * LD + c * 4 + e] = kreg[i][e];
        sV[row * LD + c * 4 + e] = vreg[i][e];
      }
    }
  };

  float m_dec = kNegInf, m_acc = kNegInf, l_part = 0.f;
  f32x16 o_acc[MTV];
#pragma unroll
  for (int i = 0; i < MTV; ++i) o_acc[i] = f32x16{};
  unsigned live_cnt = 0, skip_cnt = 0;
  const int mask_row = ((b * a.Hq + hq) * a.nqt + qt) * a.nkb;

  if (J > 0) load_tiles(0);
  for (int j = 0; j < J; ++j) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (j + 1 < J) load_tiles(j + 1);
    if ((j % chunk) == 0) m_dec = kNegInf;

    f32x16 s[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) s[mt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x2f32(sK[(mt * 32 + l32) * LD + kk * 2 + hi], qf[kk], s[mt], 0, 0, 0);

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
    __syncthreads();
    const int keep = sVote[j & 1][0] | sVote[j & 1][1];
    m_dec = fmaxf(m_dec, mx);
    ++live_cnt;
    if (!keep) ++skip_cnt;
    if (tid == 0) {
      if (a.mask) a.mask[mask_row + j] = keep ? kKept : kSkipped;
      if (a.crit) a.crit[mask_row + j] = fmaxf(sCrit[j & 1][0], sCrit[j & 1][1]) * a.scale;
    }
    if (!keep || a.stats_only) continue;

    const float m_new = fmaxf(m_acc, mx);
    if (__ballot(m_new > m_acc) != 0ull) {
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2((m_acc - m_new) * a.scale_log2);
      l_part *= alpha;
#pragma unroll
      for (int i = 0; i < MTV; ++i) o_acc[i] *= alpha;
      m_acc = m_new;
    }
    const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[mt][r], a.scale_log2, -base));
        l_part += p;
        s[mt][r] = p;
      }
    // O^T += V^T P^T: k-step (mt, r) pairs key mt*32 + 8*(r/4) + 4*hi + r%4 of lane half hi
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
#pragma unroll
        for (int mv = 0; mv < MTV; ++mv)
          o_acc[mv] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[key * LD + mv * 32 + l32], s[mt][r], o_acc[mv], 0, 0, 0);
      }
  }

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
  if (a.head_counters && tid == 0) {
    unsigned long long *hc = a.head_counters + 2 * (b * a.Hq + hq);
    atomicAdd(&hc[0], (unsigned long long)live_cnt);
    atomicAdd(&hc[1], (unsigned long long)skip_cnt);
  }
  if (a.stats_only) return;

  const float l_row = l_part + __shfl_xor(l_part, 32);
  const float inv = l_row > 0.f ? 1.f / l_row : 0.f;
  if (row_ok) {
    if (a.lse && hi == 0)
      a.lse[((int64_t)b * a.Hq + hq) * a.Lq + my_row] = l_row > 0.f ? m_acc * a.scale + __logf(l_row) : kNegInf;
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
  }
}

hipError_t launch_prefill_f32(const PrefillArgs &a, int D, hipStream_t st) {
  const int grid = a.B * a.Hq * a.nqt;
  if (D == 64) {
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(grid), dim3(128), 0, st, a);
  } else if (D == 128) {
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(grid), dim3(128), 0, st, a);
  } else {
    return hipErrorNotSupported;
  }
  return hipGetLastError();
}

}  // namespace blasst

// BLASST prefill backward: gradients of the sparse prefill with the forward's decisions held fixed.
//
// Method: sparsity-aware training runs the BLASST forward and lets the skipped blocks receive no
// gradient (pages: xllm-io review, 训练流程 / 稀疏感知训练).  The backward differentiates what the
// forward evaluated: for each query row, softmax attention over the visible keys of the blocks its
// tile kept.  With P = exp(scale * Q K^T - LSE) on those (row, key) pairs and D_i = sum_d dO_id O_id:
//     dV = P^T dO,   dP = dO V^T,   dS = scale * P * (dP - D),   dQ = dS K,   dK = dS^T Q,
// with the products taken over P * (dP - D) and the scale applied once to each finished dQ and dK
// value (one multiply per output instead of one per probability),
// and a tile-block that the forward skipped (or that is not live) adds nothing to any of them.
//
// MI355X design (head dim 128, 128 x 128 tile-blocks, bf16 inputs; v_mfma_f32_32x32x16_bf16 in the dQ
// kernel and v_mfma_f32_16x16x32_bf16 in the dK/dV kernel, with the operand arrangement of the
// forward kernel: products are taken in the orientation that lets probabilities go from accumulator
// registers straight into the B operand of the next product, and the one transposed operand of each
// product is read with the gfx950 transpose read ds_read_b64_tr_b16 from a row-major LDS tile):
//   * dQ kernel: one workgroup per (two q heads of a GQA group, query tile), or for a group of odd
//     size per (one q head, two consecutive query tiles), 4 waves of 32 rows per tile; the rows' Q
//     and dO stay in registers; K and V blocks go global -> LDS with direct loads
//     into double-buffered tiles, one barrier per block, and only blocks that a tile of the workgroup
//     kept are staged at all.  Per kept block: S^T = K Q^T, dP^T = V dO^T, dS^T, dQ^T += K^T dS^T.  It
//     also forms D from dO and O and stores it for the second kernel;
//   * dK/dV kernel: one workgroup per (kv head, key block), 8 waves of 16 keys whose K and V rows stay
//     in registers; it walks the (q head of the group, query tile) pairs whose forward decision for
//     this block was "keep", staging their Q and dO tiles double-buffered; per pair and 32-row k-step
//     (two 16-row slices): S = Q K^T, dP = dO V^T, P, dS, then dV^T += dO^T P and dK^T += Q^T dS,
//     software-pipelined by one k-step.  The q heads of the group
//     accumulate in the same registers, so no atomics and no reduction pass are needed;
//   * a skipped tile-block costs nothing at all (no staging, no product; the forward's QK^T is not
//     repeated), so the backward's work follows the kept fraction;
//   * which blocks (pairs) are kept is read 64 at a time: every lane reads one mask byte and a wave
//     ballot gives a 64-bit word that the loop walks with count-trailing-zeros.
#include "common.hpp"

namespace blasst {

namespace {
typedef __attribute__((ext_vector_type(4))) short bv4i16;
typedef __attribute__((address_space(3))) bv4i16 lds_bv4i16;

constexpr int BD = 128;               // head dim of q, k and v
constexpr int BB = 128;               // rows of a query tile = keys of a key block
// LDS row strides of the staged 128 x 128 bf16 tiles (256 data bytes + pad), chosen per tile from
// the LDS bank conflicts measured for each read pattern (a probe of the exact patterns, stride by
// stride): rows read as the A operand of 32x32x16 products are conflict-free at 16 mod 64 bytes;
// transpose reads for 32x32x16 operands only at 64 mod 256; rows and transpose reads for
// 16x16x32 operands only at 32 mod 256.
constexpr int ROW_DQ_K = 304;   // dQ kernel K tile: rows for S^T, transpose reads for dQ^T (2-way there)
constexpr int ROW_DQ_V = 272;   // dQ kernel V tile: rows only
constexpr int ROW_DKV = 288;    // dK/dV kernel Q and dO tiles: 16x16x32 rows and transpose reads
template <int ROWB>
constexpr int tile_ins() { return BB * (ROWB / 16) / 64; }   // wave-wide direct loads per tile
template <int ROWB>
constexpr int tile_bytes() { return tile_ins<ROWB>() * 1024; }

// Direct global -> LDS loads of one 128-row x 128-element bf16 tile (rows row0 ... row0 + 127 of a
// row-major matrix with `stride` elements per row) into an LDS tile of ROWB-byte rows (pad positions
// re-read chunk 0 of their row).  Wave `wave` of `nw` issues instructions wave, wave + nw, ...; rows
// at or past `nrows` re-read row nrows - 1, so every lane reads valid memory.
template <int ROWB>
__device__ __forceinline__ void stage_tile(const __bf16 *base, int64_t stride, int row0, int nrows,
                                           unsigned char *dst, int wave, int nw, int lane) {
  constexpr int CPR = ROWB / 16;
  for (int ins = wave; ins < tile_ins<ROWB>(); ins += nw) {
    const int p = ins * 64 + lane;
    const int row = p / CPR;
    int c = p - row * CPR;
    if (c >= 16) c = 0;
    const int src = min(row0 + row, nrows - 1);
    direct_load16(base + (int64_t)src * stride + c * 8, lds_addr(dst + ins * 1024));
  }
}

// Instruction i of stage_tile's loop only (ins = wave + i * nw), if it exists.
template <int ROWB>
__device__ __forceinline__ void stage_tile_part(const __bf16 *base, int64_t stride, int row0, int nrows,
                                                unsigned char *dst, int wave, int nw, int lane, int i) {
  constexpr int CPR = ROWB / 16;
  const int ins = wave + i * nw;
  if (ins < tile_ins<ROWB>()) {
    const int p = ins * 64 + lane;
    const int row = p / CPR;
    int c = p - row * CPR;
    if (c >= 16) c = 0;
    const int src = min(row0 + row, nrows - 1);
    direct_load16(base + (int64_t)src * stride + c * 8, lds_addr(dst + ins * 1024));
  }
}

// Transpose read of one k-step (16 rows of the tile) for an A operand X^T, X row-major in LDS:
// output lane l holds column 32 mv + l % 32 of X and the 8 rows of its lane half in the order of the
// B operand taken from accumulator registers 8 (ks % 2) ... + 7 of m-tile ks / 2.
template <int ROWB>
__device__ __forceinline__ bf16x8 tr_operand(const unsigned char *t, int ks, int mv) {
  const bv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16 *)(t + ks * 16 * ROWB + mv * 64));
  const bv4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16 *)(t + (ks * 16 + 8) * ROWB + mv * 64));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Byte offset of a lane's transpose reads inside a tile (16-lane group G, lane j of it: row
// 4 (G / 2) + j / 4, columns 16 (G % 2) + 4 (j % 4) ... + 3).
template <int ROWB>
__device__ __forceinline__ int tr_lane_offset(int lane) {
  const int g = lane >> 4, j = lane & 15;
  return ((g >> 1) * 4 + (j >> 2)) * ROWB + (16 * (g & 1) + 4 * (j & 3)) * 2;
}

template <bool OUT_F32>
__device__ __forceinline__ void store4(void *base, int64_t idx, float x0, float x1, float x2, float x3) {
  if (OUT_F32) {
    f32x4 w = {x0, x1, x2, x3};
    *(f32x4 *)((float *)base + idx) = w;
  } else {
    u32x2 w;
    w[0] = pack_bf16x2(x0, x1);
    w[1] = pack_bf16x2(x2, x3);
    *(u32x2 *)((__bf16 *)base + idx) = w;
  }
}
}  // namespace

// ---------------------------------------------------------------------------------------------
// dQ (and D)
// ---------------------------------------------------------------------------------------------
// QP = true (GQA groups of odd size, MHA among them): the two tiles are two consecutive query tiles
// of one head instead of one query tile of two heads; tile 0 is the heavier, and the workgroup walks
// the blocks either tile kept.
template <int TPW, bool OUT_F32, bool QP = false>
__global__ __launch_bounds__(256 * TPW, 1) void prefill_bwd_dq_kernel(BwdArgs a) {
  static_assert(!QP || TPW == 2, "query pairs are two tiles");
  constexpr int NW = 4 * TPW;    // waves per workgroup
  constexpr int KS = BD / 16;    // k-steps over the head dim
  constexpr int MT = BB / 32;    // key m-tiles of a block
  constexpr int MV = BD / 32;    // dim m-tiles of dQ^T
  __shared__ __attribute__((aligned(16))) unsigned char sK[2][tile_bytes<ROW_DQ_K>()];
  __shared__ __attribute__((aligned(16))) unsigned char sV[2][tile_bytes<ROW_DQ_V>()];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave >> 2;
  const int wit = wave & 3;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // heavy causal tiles first; TPW heads of one kv head share the staged K/V blocks (QP: two query
  // tiles of one head; an odd tile count leaves the last pair's tile 1 empty)
  const int groups = QP ? a.Hq : a.Hq / TPW;
  const int per_level = a.B * groups;
  const int level = blockIdx.x / per_level;
  const int rem = blockIdx.x - level * per_level;
  auto qt_of = [&](int tl) {
    return QP ? (a.causal ? a.nqt - 1 - (2 * level + tl) : 2 * level + tl) : (a.causal ? a.nqt - 1 - level : level);
  };
  const int qt0 = qt_of(0), qt1 = qt_of(1);
  const int qt = tile ? qt1 : qt0;
  const bool tile_on = qt >= 0 && qt < a.nqt;
  const int b = rem / groups;
  const int hq0 = QP ? rem - b * groups : (rem - b * groups) * TPW;
  const int hq = QP ? hq0 : hq0 + tile;
  const int g = hq0 / a.G;
  const int r0 = qt * BB;
  const int off = a.Lk - a.Lq;
  auto live_blocks = [&](int qtx) {   // live key blocks of query tile qtx
    if (!a.causal) return a.nkb;
    const int lim = min(qtx * BB + BB, a.Lq) - 1 + off;
    return lim < 0 ? 0 : min(a.nkb, lim / BB + 1);
  };
  const int J = live_blocks(qt0);                                          // tile 0 (the heavier)
  const int J1 = TPW == 2 && qt1 >= 0 && qt1 < a.nqt ? live_blocks(qt1) : 0;   // tile 1

  const __bf16 *qp = (const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1];
  const __bf16 *dop = (const __bf16 *)a.dout + b * a.dos[0] + hq * a.dos[1];
  const int64_t obase = b * a.os[0] + hq * a.os[1];
  const __bf16 *kp = (const __bf16 *)a.k + b * a.ks[0] + g * a.ks[1];
  const __bf16 *vp = (const __bf16 *)a.v + b * a.vs[0] + g * a.vs[1];

  // ---- this lane's query row: Q and dO fragments (B operands), D = dO . O, LSE ----
  const int my_row = r0 + wit * 32 + l32;
  const bool row_ok = tile_on && my_row < a.Lq;
  bf16x8 qf[KS], df[KS];
  float dsum = 0.f;
#pragma unroll
  for (int kk = 0; kk < KS; ++kk) {
    const int c = kk * 16 + hi * 8;
    qf[kk] = row_ok ? *(const bf16x8 *)(qp + (int64_t)my_row * a.qs[2] + c) : bf16x8{};
    df[kk] = row_ok ? *(const bf16x8 *)(dop + (int64_t)my_row * a.dos[2] + c) : bf16x8{};
    float of[8] = {};
    if (row_ok) {
      const int64_t oi = obase + (int64_t)my_row * a.os[2] + c;
      if (a.o_f32) {
        const f32x4 lo = *(const f32x4 *)((const float *)a.o + oi);
        const f32x4 up = *(const f32x4 *)((const float *)a.o + oi + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          of[e] = lo[e];
          of[e + 4] = up[e];
        }
      } else {
        const bf16x8 ob = *(const bf16x8 *)((const __bf16 *)a.o + oi);
#pragma unroll
        for (int e = 0; e < 8; ++e) of[e] = (float)ob[e];
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dsum = __builtin_fmaf((float)df[kk][e], of[e], dsum);
  }
  dsum += __shfl_xor(dsum, 32);
  const int64_t row_idx = ((int64_t)b * a.Hq + hq) * a.Lq + my_row;
  const float lse = row_ok ? a.lse[row_idx] : kNegInf;
  // a row without any kept key (LSE = -inf) and a row past the end get P = 0
  const float lse_l2 = lse == kNegInf ? __builtin_huge_valf() : lse * kLog2e;
  if (row_ok && hi == 0) a.dvec[row_idx] = dsum;

  // ---- kept blocks, 64 per word: bit of block base + x = tile keeps block base + x ----
  const uint8_t *mrow = a.mask ? a.mask + (((int64_t)b * a.Hq + hq0) * a.nqt + qt0) * a.nkb : nullptr;
  // distance from tile 0's mask row to tile 1's: the next head's row, or (QP) the other query tile's
  const int64_t mtile = QP ? (int64_t)(qt1 - qt0) * a.nkb : (int64_t)a.nqt * a.nkb;
  uint64_t w0 = 0, w1 = 0;
  int wbase = -64;
  auto fetch = [&](int base) {
    wbase = base;
    const int j = base + lane;
    bool k0 = j < J, k1 = j < J1;
    if (mrow) {
      k0 = k0 && mrow[j] == kKept;
      if (TPW == 2) k1 = k1 && mrow[mtile + j] == kKept;
    }
    w0 = __ballot(k0);
    w1 = TPW == 2 ? __ballot(k1) : 0ull;
  };
  auto next = [&](int from) -> int {   // first block >= from that some tile keeps, or J
    while (from < J) {
      if (from < wbase || from >= wbase + 64) fetch(from & ~63);
      const uint64_t w = (w0 | w1) >> (from - wbase);
      if (w) return from + (int)__builtin_ctzll(w);
      from = wbase + 64;
    }
    return J;
  };
  auto mine = [&](int j) -> bool { return (((tile ? w1 : w0) >> (j - wbase)) & 1ull) != 0ull; };
  auto stage = [&](int j, int buf) {
    stage_tile<ROW_DQ_K>(kp, a.ks[2], j * BB, a.Lk, sK[buf], wave, NW, lane);
    stage_tile<ROW_DQ_V>(vp, a.vs[2], j * BB, a.Lk, sV[buf], wave, NW, lane);
  };
  constexpr int NSPQ = (tile_ins<ROW_DQ_K>() + NW - 1) / NW;   // >= the V tile's count
  auto stage_part = [&](int j, int buf, int i) {
    stage_tile_part<ROW_DQ_K>(kp, a.ks[2], j * BB, a.Lk, sK[buf], wave, NW, lane, i);
    stage_tile_part<ROW_DQ_V>(vp, a.vs[2], j * BB, a.Lk, sV[buf], wave, NW, lane, i);
  };

  const int tr_off = tr_lane_offset<ROW_DQ_K>(lane);
  f32x16 dq_acc[MV];
#pragma unroll
  for (int i = 0; i < MV; ++i) dq_acc[i] = f32x16{};

  int jc = next(0);
  bool keep_c = jc < J && mine(jc);
  if (jc < J) stage(jc, 0);
  int buf = 0;
  while (jc < J) {
    const int jn = next(jc + 1);
    const bool keep_n = jn < J && mine(jn);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // block jc has landed in LDS
    __syncthreads();                                   // ... for every wave; buffer buf ^ 1 is free
    if (jn < J && !keep_c) stage(jn, buf ^ 1);   // no products to spread the loads over
    if (keep_c) {
      const unsigned char *kb = sK[buf] + l32 * ROW_DQ_K + hi * 16;
      const unsigned char *vb = sV[buf] + l32 * ROW_DQ_V + hi * 16;
      const unsigned char *kt = sK[buf] + tr_off;
      const int key0 = jc * BB;
      const bool need_mask = (key0 + BB > a.Lk) || (a.causal && key0 + BB - 1 > r0 + off);
      const int lim = a.causal ? min(my_row + off, a.Lk - 1) : a.Lk - 1;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        // the next block's staging, spread over the first m-tiles (issued at once, the loads held each
        // wave in the stalled issue)
#pragma unroll
        for (int i = 0; i < NSPQ; ++i)
          if (jn < J && i * (MT - 1) / NSPQ == mt) stage_part(jn, buf ^ 1, i);
        f32x16 s = f32x16{}, dp = f32x16{};
        // K and V fragments two k-steps ahead of their MFMAs, in rings of three (left to itself, the
        // compiler read each fragment right before its MFMA and waited for it there)
        bf16x8 kr[3], vr[3];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          kr[kk] = *(const bf16x8 *)(kb + mt * 32 * ROW_DQ_K + kk * 32);
          vr[kk] = *(const bf16x8 *)(vb + mt * 32 * ROW_DQ_V + kk * 32);
        }
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          if (kk + 2 < KS) {
            kr[(kk + 2) % 3] = *(const bf16x8 *)(kb + mt * 32 * ROW_DQ_K + (kk + 2) * 32);
            vr[(kk + 2) % 3] = *(const bf16x8 *)(vb + mt * 32 * ROW_DQ_V + (kk + 2) * 32);
          }
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk % 3], qf[kk], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[kk % 3], df[kk], dp, 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
        }
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = key0 + mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > lim) s[r] = kNegInf;
          }
        }
        // dS^T / scale = P^T (dP^T - D), packed as the B operand of the two k-steps over these keys
        bf16x8 dsf[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = fast_exp2(__builtin_fmaf(s[r], a.scale_log2, -lse_l2));
          dsf[r >> 3][r & 7] = (__bf16)(p * (dp[r] - dsum));
        }
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
          for (int mv = 0; mv < MV; ++mv)
            dq_acc[mv] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_operand<ROW_DQ_K>(kt, 2 * mt + k2, mv), dsf[k2],
                                                                 dq_acc[mv], 0, 0, 0);
      }
    }
    buf ^= 1;
    jc = jn;
    keep_c = keep_n;
  }

  // ---- dQ: lane holds row my_row, dims 32 mv + 8 q + 4 hi ... + 3 in dq_acc[mv][4 q ... 4 q + 3] ----
  if (row_ok) {
    const int64_t base = b * a.dqs[0] + hq * a.dqs[1] + (int64_t)my_row * a.dqs[2];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        store4<OUT_F32>(a.dq, base + 32 * mv + 8 * q4 + 4 * hi, dq_acc[mv][4 * q4] * a.scale,
                        dq_acc[mv][4 * q4 + 1] * a.scale, dq_acc[mv][4 * q4 + 2] * a.scale,
                        dq_acc[mv][4 * q4 + 3] * a.scale);
  }
}

// ---------------------------------------------------------------------------------------------
// dK and dV
// ---------------------------------------------------------------------------------------------
// Transpose read for the A operand of v_mfma_f32_16x16x32_bf16 over 32 tile rows (k-step ks) and 16
// columns (tile mv) of a row-major LDS tile X: lane l (16-lane group q = l / 16) gets column
// 16 mv + l % 16 and rows 32 ks + 4 q ... + 3 and 32 ks + 16 + 4 q ... + 3, the order in which the
// C layout of two consecutive 16-row S slices holds them (so P and dS feed the B operand as they are).
__device__ __forceinline__ bf16x8 tr_operand16(const unsigned char *t, int ks, int mv) {
  constexpr int ROWB = ROW_DKV;
  const bv4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16 *)(t + ks * 32 * ROWB + mv * 32));
  const bv4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_bv4i16 *)(t + (ks * 32 + 16) * ROWB + mv * 32));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <bool OUT_F32>
__global__ __launch_bounds__(512) void prefill_bwd_dkdv_kernel(BwdArgs a) {
  constexpr int NW = 8;          // 8 waves of 16 keys: two waves per SIMD
  constexpr int KS = BD / 32;    // k-steps of 32 over the head dim
  constexpr int NSL = BB / 16;   // 16-row slices of a query tile
  constexpr int MV = BD / 16;    // 16-wide dim tiles of dK^T, dV^T
  constexpr int ROWB = ROW_DKV;
  __shared__ __attribute__((aligned(16))) unsigned char sQ[2][tile_bytes<ROWB>()];
  __shared__ __attribute__((aligned(16))) unsigned char sO[2][tile_bytes<ROWB>()];   // dO tiles
  __shared__ __attribute__((aligned(16))) float sL[2][BB];              // LSE * log2(e) of the tile's rows
  __shared__ __attribute__((aligned(16))) float sD[2][BB];              // -D of the tile's rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;
  const int q4 = lane >> 4;      // 16-lane group

  // key blocks with the most causal query tiles first
  const int per_level = a.B * a.Hkv;
  const int j = blockIdx.x / per_level;
  const int rem = blockIdx.x - j * per_level;
  const int b = rem / a.Hkv;
  const int g = rem - b * a.Hkv;
  const int key0 = j * BB;
  const int off = a.Lk - a.Lq;
  const int my_key = key0 + wave * 16 + l16;
  const bool key_ok = my_key < a.Lk;

  const __bf16 *kp = (const __bf16 *)a.k + b * a.ks[0] + g * a.ks[1];
  const __bf16 *vp = (const __bf16 *)a.v + b * a.vs[0] + g * a.vs[1];

  // ---- this lane's key: K and V fragments (B operands of S = Q K^T and dP = dO V^T) ----
  bf16x8 kf[KS], vf[KS];
  {
    const int key = min(my_key, a.Lk - 1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      kf[kk] = *(const bf16x8 *)(kp + (int64_t)key * a.ks[2] + kk * 32 + q4 * 8);
      vf[kk] = *(const bf16x8 *)(vp + (int64_t)key * a.vs[2] + kk * 32 + q4 * 8);
    }
    // a wait the compiler sees: otherwise it takes these fragments as possibly in flight inside the
    // pair loop and waits there for vector loads, i.e. for the next pair's staging as well
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  // ---- (q head of the group, query tile) pairs p = h * nqt + t that kept this block ----
  const int npairs = a.G * a.nqt;
  auto live = [&](int t) -> bool {
    if (!a.causal) return true;
    const int lim = min(t * BB + BB, a.Lq) - 1 + off;
    return lim >= key0;
  };
  uint64_t word = 0;
  int wbase = -64;
  auto fetch = [&](int base) {
    wbase = base;
    const int p = base + lane;
    bool k = false;
    if (p < npairs) {
      const int h = p / a.nqt, t = p - (p / a.nqt) * a.nqt;
      k = live(t);
      if (a.mask && k) k = a.mask[(((int64_t)b * a.Hq + g * a.G + h) * a.nqt + t) * a.nkb + j] == kKept;
    }
    word = __ballot(k);
  };
  auto next = [&](int from) -> int {
    while (from < npairs) {
      if (from < wbase || from >= wbase + 64) fetch(from & ~63);
      const uint64_t w = word >> (from - wbase);
      if (w) return from + (int)__builtin_ctzll(w);
      from = wbase + 64;
    }
    return npairs;
  };
  // A pair's Q and dO tiles and the LSE and D of its rows are staged by direct loads (waves 0-1: LSE,
  // 2-3: D, 64 rows each; rows past the end read the last row), all in flight while the previous
  // pair is processed.
  static_assert(BB == 128, "four 64-row instructions cover LSE and D of a tile");
  constexpr int NSP = (tile_ins<ROWB>() + NW - 1) / NW;   // instructions per wave per tile
  // part i < NSP: instruction i of the Q and the dO tile; part NSP: the LSE and D values
  auto stage_part = [&](int p, int buf, int i) {
    const int h = p / a.nqt, t = p - (p / a.nqt) * a.nqt;
    const int hq = g * a.G + h;
    if (i < NSP) {
      stage_tile_part<ROWB>((const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1], a.qs[2], t * BB, a.Lq, sQ[buf], wave,
                            NW, lane, i);
      stage_tile_part<ROWB>((const __bf16 *)a.dout + b * a.dos[0] + hq * a.dos[1], a.dos[2], t * BB, a.Lq, sO[buf],
                            wave, NW, lane, i);
    } else if (wave < 4) {
      const int row = min(t * BB + (wave & 1) * 64 + lane, a.Lq - 1);
      const int64_t idx = ((int64_t)b * a.Hq + hq) * a.Lq + row;
      const float *src = (wave < 2 ? (const float *)a.lse : (const float *)a.dvec) + idx;
      direct_load4(src, lds_addr((wave < 2 ? sL[buf] : sD[buf]) + (wave & 1) * 64));
    }
  };
  auto stage = [&](int p, int buf) {
    const int h = p / a.nqt, t = p - (p / a.nqt) * a.nqt;
    const int hq = g * a.G + h;
    stage_tile<ROWB>((const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1], a.qs[2], t * BB, a.Lq, sQ[buf], wave, NW,
                     lane);
    stage_tile<ROWB>((const __bf16 *)a.dout + b * a.dos[0] + hq * a.dos[1], a.dos[2], t * BB, a.Lq, sO[buf], wave,
                     NW, lane);
    if (wave < 4) {
      const int row = min(t * BB + (wave & 1) * 64 + lane, a.Lq - 1);
      const int64_t idx = ((int64_t)b * a.Hq + hq) * a.Lq + row;
      const float *src = (wave < 2 ? (const float *)a.lse : (const float *)a.dvec) + idx;
      direct_load4(src, lds_addr((wave < 2 ? sL[buf] : sD[buf]) + (wave & 1) * 64));
    }
  };
  // After a wave's staging loads have landed (its own vmcnt(0)), each lane of waves 0-3 rewrites the
  // value its own load wrote: LSE becomes the exponent offset LSE log2(e), +inf (P = 0 exactly) for
  // rows without any kept key (LSE = -inf) and rows past the end; D becomes -D, 0 for rows past the
  // end.  The next barrier publishes them.
  auto fix_ld = [&](int p, int buf) {
    if (wave < 4) {
      const int t = p - (p / a.nqt) * a.nqt;
      const int i = (wave & 1) * 64 + lane;
      const bool ok = t * BB + i < a.Lq;
      if (wave < 2) {
        const float l = sL[buf][i];
        sL[buf][i] = (!ok || l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
      } else {
        const float d = sD[buf][i];
        sD[buf][i] = ok ? -d : 0.f;
      }
    }
  };

  // transpose reads: 16-lane group q reads rows 4 q + (l16 / 4), columns 4 (l16 % 4) ... + 3
  const int tr_off = (4 * q4 + (l16 >> 2)) * ROWB + 4 * (l16 & 3) * 2;
  f32x4 dv_acc[MV], dk_acc[MV];
#pragma unroll
  for (int i = 0; i < MV; ++i) {
    dv_acc[i] = f32x4{};
    dk_acc[i] = f32x4{};
  }

  int pc = next(0);
  if (pc < npairs) {
    stage(pc, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    fix_ld(pc, 0);
  }
  int buf = 0;
  while (pc < npairs) {
    const int pn = next(pc + 1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // pair pc's tiles have landed in LDS
    __syncthreads();                                   // ... for every wave; buffer buf ^ 1 is free
    {
      const int t = pc - (pc / a.nqt) * a.nqt;
      const int row0 = t * BB;
      const bool need_mask = a.causal && (key0 + BB - 1 > row0 + off);
      const unsigned char *qb = sQ[buf] + l16 * ROWB + q4 * 16;
      const unsigned char *ob = sO[buf] + l16 * ROWB + q4 * 16;
      const unsigned char *qtr = sQ[buf] + tr_off;
      const unsigned char *otr = sO[buf] + tr_off;
      // one k-step of 32 rows = two 16-row slices: S and dP (C layout: lane holds key my_key and
      // rows 16 sl + 4 q4 ... + 3), then P and dS as B operands, then dV^T and dK^T.  Software-
      // pipelined by one k-step: the S and dP products of k-step ks + 1 are issued before the
      // exponentials and the dV^T / dK^T products of k-step ks, so the MFMA and LDS pipes are fed
      // while a k-step's products are still in flight.
      f32x4 s[2][2], dp[2][2];   // [k-step parity][slice]
      auto sdp = [&](int ks) {
        const int u = ks & 1;
        // the dP accumulators start from -D of their rows, so the products leave dP - D
        s[u][0] = s[u][1] = f32x4{};
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) dp[u][h2] = *(const f32x4 *)&sD[buf][(2 * ks + h2) * 16 + 4 * q4];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk)
#pragma unroll
          for (int h2 = 0; h2 < 2; ++h2) {
            const int sl = 2 * ks + h2;
            const bf16x8 qa = *(const bf16x8 *)(qb + sl * 16 * ROWB + kk * 64);
            const bf16x8 oa = *(const bf16x8 *)(ob + sl * 16 * ROWB + kk * 64);
            s[u][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qa, kf[kk], s[u][h2], 0, 0, 0);
            dp[u][h2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oa, vf[kk], dp[u][h2], 0, 0, 0);
          }
      };
      sdp(0);
#pragma unroll
      for (int ks = 0; ks < NSL / 2; ++ks) {
        // the next pair's staging, parts spread over the first k-steps (issued at once, the loads held
        // each wave in the stalled issue)
#pragma unroll
        for (int i = 0; i <= NSP; ++i)
          if (pn < npairs && i * (NSL / 2 - 1) / (NSP + 1) == ks) stage_part(pn, buf ^ 1, i);
        if (ks + 1 < NSL / 2) sdp(ks + 1);
        const int u = ks & 1;
        bf16x8 pf, dsf;
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int rr = (2 * ks + h2) * 16 + 4 * q4;
          const f32x4 l4 = *(const f32x4 *)&sL[buf][rr];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float p = fast_exp2(__builtin_fmaf(s[u][h2][e], a.scale_log2, -l4[e]));
            if (need_mask && my_key > row0 + rr + e + off) p = 0.f;
            pf[4 * h2 + e] = (__bf16)p;
            dsf[4 * h2 + e] = (__bf16)(p * dp[u][h2][e]);
          }
        }
#pragma unroll
        for (int mv = 0; mv < MV; ++mv) {
          dv_acc[mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand16(otr, ks, mv), pf, dv_acc[mv], 0, 0, 0);
          dk_acc[mv] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_operand16(qtr, ks, mv), dsf, dk_acc[mv], 0, 0, 0);
        }
      }
    }
    if (pn < npairs) {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // pair pn's staging has landed
      fix_ld(pn, buf ^ 1);
    }
    buf ^= 1;
    pc = pn;
  }

  // ---- dK, dV: lane holds key my_key, dims 16 mv + 4 q4 ... + 3 in acc[mv] ----
  if (key_ok) {
    const int64_t kb = b * a.dks[0] + g * a.dks[1] + (int64_t)my_key * a.dks[2];
    const int64_t vb = b * a.dvs[0] + g * a.dvs[1] + (int64_t)my_key * a.dvs[2];
#pragma unroll
    for (int mv = 0; mv < MV; ++mv) {
      const int d0 = 16 * mv + 4 * q4;
      store4<OUT_F32>(a.dk, kb + d0, dk_acc[mv][0] * a.scale, dk_acc[mv][1] * a.scale, dk_acc[mv][2] * a.scale,
                      dk_acc[mv][3] * a.scale);
      store4<OUT_F32>(a.dv, vb + d0, dv_acc[mv][0], dv_acc[mv][1], dv_acc[mv][2], dv_acc[mv][3]);
    }
  }
}

template <bool QP>
static void launch_dq(const BwdArgs &a, hipStream_t st) {
  const int grid = QP ? a.B * a.Hq * ((a.nqt + 1) / 2) : a.B * (a.Hq / 2) * a.nqt;
  if (a.out_f32)
    hipLaunchKernelGGL((prefill_bwd_dq_kernel<2, true, QP>), dim3(grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_bwd_dq_kernel<2, false, QP>), dim3(grid), dim3(512), 0, st, a);
}

// The dQ kernel runs first: it writes D, which the dK/dV kernel reads (same stream).
hipError_t launch_prefill_bwd(const BwdArgs &a, hipStream_t st) {
  // two heads of a GQA group per workgroup, or (odd groups) two query tiles of one head
  if (a.G % 2 == 0)
    launch_dq<false>(a, st);
  else
    launch_dq<true>(a, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid = a.B * a.Hkv * a.nkb;
  if (a.out_f32)
    hipLaunchKernelGGL((prefill_bwd_dkdv_kernel<true>), dim3(grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_bwd_dkdv_kernel<false>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

}  // namespace blasst

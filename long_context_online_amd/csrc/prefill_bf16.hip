// BLASST prefill forward, bf16 inputs, fp32 accumulation, gfx950 MFMA.
//
// Method: FlashAttention-style tiled online softmax over the KV blocks of a query tile, visited
// left to right; block j is skipped when every row of the tile has m~ - m < ln(lambda), and a
// skipped block gets no exp and no P.V product, while QK^T is still computed for every block
// (pages: xllm-io review, 核心公式 and 预填充内核优化; gist.science (de), 2. Methodik / Kernidee and
// 3. Kernel-Design).  The pages keep staging the V block of a skipped block; here a skipped block's
// V is not loaded either.
//
// MI355X design:
//   * a workgroup owns TPW = 2 query tiles that read the same K/V stream (two q heads of one GQA
//     group at the same query position; for a group of odd size, MHA among them, two consecutive
//     query tiles of one head), so every staged K/V block serves 2 * BR query rows; each tile has
//     BR = 32 * WPT rows, one wave per 32 rows, and votes on its own; each SIMD runs one wave of
//     each tile, and tile 1's waves issue at a raised priority after the vote barrier (without it
//     tile 0's wave ran ahead into the next block while tile 1's wave, the laggard, was still in its
//     exponentials);
//   * scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16: the A operand
//     (K) comes from LDS, the B operand (Q) stays in registers for the whole tile, and each lane
//     ends up holding all scores of ONE query row, so the block row max is an in-lane max plus one
//     exchange with lane l ^ 32;
//   * P^T is packed to bf16 straight from the score registers and used as the B operand of
//     O^T = V^T P^T; the V^T operand is read from a row-major V tile with the gfx950 transpose
//     read ds_read_b64_tr_b16 (within a 16-lane group, output lane i, element k is element i%4 of
//     source lane 4k + i/4's 8-byte read), so no transpose pass is needed anywhere;
//   * K and V go global -> LDS directly (buffer_load ... lds, no registers) into double-buffered
//     LDS; the block loop is software-pipelined by one block: iteration t computes QK^T and the
//     vote of block t, then ONE barrier publishes the votes and makes K_{t+1} (its loads spread
//     over block t's score MFMAs) and V_{t-1} visible; then the P.V product of block t - 1 runs from its
//     probabilities packed in registers, and only if block t was kept by a tile of the workgroup
//     are its probabilities formed and V_t loaded, so a skipped block costs QK^T, the row max and
//     the vote and nothing else;
//   * the skip vote: per-row predicate -> wave ballot -> one LDS byte per wave -> one read of all
//     the workgroup's bytes after the vote barrier, OR over the tile's; the skip is a uniform branch,
//     so a skipped block issues no v_exp and no P.V MFMA;
//   * LDS operands (K fragments of the scores, V^T fragments of P.V) are read two MFMAs ahead of use
//     in rings of three, written out: left to itself the compiler read some right before their MFMA;
//   * LDS rows are padded so that reads are free of bank conflicts on the 64-bank (256-byte) LDS:
//     K rows are 16 mod 256 bytes apart (16 rows x 16 bytes of one read pass fall on distinct
//     banks), V rows 64 mod 256 bytes apart (the two 16-lane groups of a transpose-read pass read
//     4 rows x 32 bytes each at column offsets 0 and 32); every read address is one per-lane base
//     plus an immediate;
//   * heavy (late, long causal) tiles launch first, and the q heads of one kv head share an XCD's L2
//     for a stripe of levels (the mapping is described at the tile coordinates below).
#include <type_traits>

#include "common.hpp"

namespace blasst {

typedef __attribute__((ext_vector_type(4))) short v4i16;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;

// Paged key order inside each 32-key group of a K tile: LDS row m = 8 a + 4 h + b holds key
// 16 (a / 2) + 8 h + 4 (a % 2) + b.  The 32x32 score layout gives register r of lane half h the row
// 8 (r / 4) + 4 h + r % 4, so with this order the 8 probabilities a lane packs for one k-step of the
// P.V product (registers 8 s ... 8 s + 7) are the consecutive keys 16 s + 8 h ... + 7, and their V^T
// operand is one 16-byte read of a V^T row (the natural order needs two 8-byte reads, which conflict
// on LDS banks at every row stride).
// floor(p / d) == (p * ceil(2^16 / d)) >> 16 for every p < n (checked at compile time where used)
constexpr bool div_by_magic_exact(int d, int n) {
  for (int p = 0; p < n; ++p)
    if ((p * ((65536 + d - 1) / d)) >> 16 != p / d) return false;
  return true;
}

__device__ __forceinline__ int paged_key_of_row(int m) {
  const int a = m >> 3, h = (m >> 2) & 1, b = m & 3;
  return (m & ~31) + 16 * ((a & 3) >> 1) + 8 * h + 4 * (a & 1) + b;
}

// DEC = false: no threshold at all (every live block kept, no vote); used to measure what the
// decisions cost.  PAGED = true: K and V come from a paged cache (chunked prefill; head dim 128,
// 128-key blocks of eight 16-token pages): K rows are gathered page by page, and V, which the cache
// stores transposed inside each page, is staged page-major as a V^T tile ([page][dv][16 keys], each
// page a plain 4 KB copy), so the A operand of O^T += V^T P^T is one 16-byte LDS read per lane (1 KB
// of consecutive bytes per wave) instead of transpose reads.
//
// QP = true (query pairs, for GQA groups of odd size, MHA among them): the two tiles of a workgroup are
// two consecutive query tiles of ONE q head instead of one query tile of two heads of a group; they
// read the same K/V stream, so every staged block still serves two tiles.  The workgroup runs the
// block loop of its heavier tile; for the other tile the blocks past its causal range are not live
// (its waves still issue their share of the K/V loads, vote skip and form no probabilities).
template <int D, int BC, int TPW, bool OUT_F32, bool STATS, bool DEC = true, bool PAGED = false, bool QP = false>
__global__ __launch_bounds__(64 * (BC / 32) * TPW, 2) void prefill_bf16_kernel(PrefillArgs a) {
  constexpr int WPT = BC / 32;       // waves per tile (32 rows each)
  constexpr int BR = BC;             // rows per tile
  constexpr int NW = WPT * TPW;      // waves per workgroup
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int KCP = KCH + 1;       // ... plus the pad chunk
  constexpr int KROW = KCP * 16;     // bytes per K row in LDS
  constexpr int VCH = D / 8;         // 16-byte chunks per V row
  constexpr int VCP = VCH + 4;       // ... plus four pad chunks (row stride = 64 mod 256 bytes)
  constexpr int VROW = VCP * 16;     // bytes per V row in LDS
  constexpr int MT = BC / 32;        // key m-tiles of S^T
  constexpr int KS = D / 16;         // k-steps over the head dim
  constexpr int MTV = D / 32;        // dv m-tiles of O^T
  constexpr int KSV = BC / 16;       // k-steps over the keys of a block
  constexpr int KINS = (BC * KCP + 63) / 64;        // wave-wide direct loads per K tile
  constexpr int VINS = (BC * VCP + 63) / 64;        // ... per V tile
  constexpr int KBUF = KINS * 1024;
  constexpr int VBUF = VINS * 1024;

  __shared__ __attribute__((aligned(16))) unsigned char sK[2][KBUF];
  __shared__ __attribute__((aligned(16))) unsigned char sV[2][VBUF];
  // one byte per wave (wave w's vote in byte w), so that one 4- or 8-byte LDS read after the vote
  // barrier gets every vote (with an int per wave the compiler issued two reads one after the other,
  // each waited for, before the exponentials could start)
  static_assert(NW == 4 || NW == 8, "one byte per wave in a 32- or 64-bit word");
  __shared__ __attribute__((aligned(8))) unsigned char sVote[2][NW];
  // paged: ids of the 8 pages of blocks t .. t + 3 (a ring indexed by block & 3), staged two blocks
  // ahead by wave 0
  __shared__ int sIds[PAGED ? 4 : 1][BC / 16];
  __shared__ float sCrit[2][NW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = wave / WPT;       // tile of this wave inside the workgroup
  const int wit = wave % WPT;        // wave index inside its tile
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  // ---- tile coordinates: heavy causal tiles first, kv-head groups kept on one XCD per level -------
  static_assert(!QP || TPW == 2, "query pairs are two tiles");
  const int groups = QP ? a.Hq : a.Hq / TPW;   // head groups of TPW heads sharing a kv head (QP: heads)
  const int per_level = a.B * groups;
  const int bid = blockIdx.x;
  int level = bid / per_level;
  int rem = bid - level * per_level;
  // Workgroups go to the 8 XCDs round robin.  A level's head groups are cut into 8 contiguous
  // chunks; the q heads of one kv head stay together and share its K/V in that XCD's L2, and an
  // XCD keeps a chunk for a stripe of consecutive levels (about half the levels it holds at once,
  // 512 / per_level), so tiles in flight on it still share one kv head.  The chunk rotates from
  // stripe to stripe, forward over 8 stripes and back over the next 8, so every XCD takes every
  // chunk on stripes of equal total causal work: heads whose sparsity differs then load all XCDs
  // alike instead of one XCD getting every tile of the densest heads and finishing last.
  if (PAGED && (gridDim.x & 7) == 0) {
    // Chunked prefill: every query tile of a chunk reads nearly all of its sequence's context, and
    // one kv head's K/V stream (16 MB at 32K keys) is several times an XCD's L2, so tiles share it
    // only while they run together.  XCD x takes the contiguous run x * n / 8 ... of workgroups
    // ordered stream-major ((sequence, kv head), then level, then head group), so the workgroups
    // resident on an XCD read the same stream side by side and each stream is fetched by one XCD.
    const int gpk = groups / (a.Hq / a.G);           // head groups per kv head
    const int per_stream = gpk * (int)(gridDim.x / per_level);
    const int lid = (bid & 7) * (int)(gridDim.x >> 3) + (bid >> 3);
    const int stream = lid / per_stream;
    const int w = lid - stream * per_stream;
    const int lvl = w / gpk;
    const int sb = stream / (a.Hq / a.G), skv = stream - sb * (a.Hq / a.G);
    level = lvl;
    rem = sb * groups + skv * gpk + (w - lvl * gpk);
  } else if ((per_level & 7) == 0) {
    const int stripe = level / max(1, 256 / per_level);
    const int p = stripe & 15;
    const int rot = p < 8 ? p : 15 - p;
    rem = (((rem & 7) + rot) & 7) * (per_level >> 3) + (rem >> 3);
  }
  // QP: level p holds query tiles 2p and 2p + 1 counted from the heavy end (tile 0 the heavier); an
  // odd tile count leaves the last pair's tile 1 empty
  const int qt = QP ? (a.causal ? a.nqt - 1 - (2 * level + tile) : 2 * level + tile)
                    : (a.causal ? (a.nqt - 1 - level) : level);
  const bool tile_on = !QP || (qt >= 0 && qt < a.nqt);
  const int b = rem / groups;
  const int hq0 = QP ? rem - b * groups : (rem - b * groups) * TPW;   // first head of the group
  const int hq = QP ? hq0 : hq0 + tile;
  const int g = hq0 / a.G;                     // TPW divides G, so the group shares kv head g
  const int r0 = qt * BR;
  int Lk = a.Lk;                               // keys of this sequence
  float thr_raw = a.thr_raw;
  if constexpr (PAGED) {
    Lk = min(a.seq_lens[b], a.max_pages * 16);
    if (a.thr_mode == 1) {
      const float lam = fminf(1.f, a.a_thr / (float)Lk);
      thr_raw = lam > 0.f ? __logf(lam) / a.scale : kNegInf;
    }
  }
  const int off = Lk - a.Lq;                   // bottom-right causal alignment

  const __bf16 *qp = (const __bf16 *)a.q + b * a.qs[0] + hq * a.qs[1];
  const __bf16 *kp = (const __bf16 *)a.k + (PAGED ? 0 : b * a.ks[0] + g * a.ks[1]);
  const __bf16 *vp = (const __bf16 *)a.v + (PAGED ? 0 : b * a.vs[0] + g * a.vs[1]);
  const int32_t *tab = PAGED ? a.table + (int64_t)b * a.max_pages : nullptr;  // the sequence's page ids
  const int last_page = PAGED ? (Lk - 1) >> 4 : 0;

  auto live_blocks = [&](int qtx) {  // live key blocks of query tile qtx
    if (!a.causal) return a.nkb;
    const int lim = min(qtx * BR + BR, a.Lq) - 1 + off;
    return lim < 0 ? 0 : min(a.nkb, lim / BC + 1);
  };
  // J: blocks the workgroup's loop runs (its heavier tile's live blocks); J_me: this tile's live blocks
  const int J_me = tile_on ? live_blocks(qt) : 0;
  const int J = QP ? live_blocks(a.causal ? a.nqt - 1 - 2 * level : 2 * level) : J_me;
  const int chunk = J_me > 0 ? (J_me + a.num_splits - 1) / a.num_splits : 1;

  // ---- Q fragments (B operand of S^T = K Q^T): row l32 of this wave, 8 dims per k-step ----------
  const int my_row = r0 + wit * 32 + l32;
  const bool row_ok = tile_on && my_row < a.Lq;
  bf16x8 qf[KS];
#pragma unroll
  for (int kk = 0; kk < KS; ++kk)
    qf[kk] = row_ok ? *(const bf16x8 *)(qp + (int64_t)my_row * a.qs[2] + kk * 16 + hi * 8) : bf16x8{};

  // ---- staging: direct global -> LDS ---------------------------------------------------------
  // paged tiles: a page id times the kv head count counts the pool's 4 KB (one head, 16 tokens)
  // units before that page; it stays below 2^32 (validated), so it is one 32-bit multiply
  const uint32_t hkv_u = (uint32_t)a.Hkv;
  // One wave instruction fills 1 KB = 64 consecutive 16-byte positions of a buffer; position p is
  // (row p / CP, chunk p % CP); pad chunks load chunk 0 of their row.  Contiguous K/V go through a
  // buffer resource per block whose extent ends at the last key, so keys past the end read as zero
  // (and are masked) without any clamping, and a load costs a few 24-bit integer ops for its offset.
  auto load_tile_part = [&](const __bf16 *base, int64_t stride, int j, unsigned char *dst, auto CPc, auto CHc,
                            auto INSc, int i, uint32_t ids) {
    constexpr int CP = decltype(CPc)::value, CH = decltype(CHc)::value, INS = decltype(INSc)::value;
    const int key0 = j * BC;
    const int ins = i * NW + wave;
    if (ins >= INS) return;
    if constexpr (!PAGED) {
      static_assert(INS * 64 == BC * CP, "every position of a tile is one row chunk");
      const uint32_t row_b = (uint32_t)stride * 2u;
      const uint64_t addr = (uint64_t)(uintptr_t)(base + (int64_t)key0 * stride);
      u32x4 rsrc;
      rsrc[0] = (uint32_t)addr;
      rsrc[1] = (uint32_t)(addr >> 32) & 0xffffu;  // stride 0
      rsrc[2] = (uint32_t)min(Lk - key0, BC) * row_b;
      rsrc[3] = 0x00020000u;
      const int p = ins * 64 + lane;
      const int row = p / CP;
      int c = p - row * CP;
      if (c >= CH) c = 0;
      buffer_load16_lds(rsrc, __mul24(row, row_b) + c * 16, lds_addr(dst) + ins * 1024);
      return;
    }
    // the lane index through an empty asm: the per-lane offsets below are then recomputed at every
    // load instead of being kept in registers across the block loop (where they spilled)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    static_assert(!PAGED || (INS * 64 == BC * CP && div_by_magic_exact(CP, INS * 64)),
                  "every position is a chunk of a tile row, and the 24-bit division below is exact");
    const int p = ins * 64 + ln;
    const int row = (int)(__umul24((unsigned)p, (65536u + CP - 1) / CP) >> 16);   // p / CP
    int c = p - row * CP;
    if (c >= CH) c = 0;
    // K row of the key's page (16 tokens per page); keys past the sequence's end read rows of its
    // last page (the ids are clamped to it) and are masked.  The page id comes from `ids` (lane l
    // holds the id of the block's page l % 8): the rows of one instruction span at most two pages,
    // the first lane's and the next, so two lane reads and a select give it without an LDS read (and
    // its wait, which would also drain the K fragment reads in flight).
    const int kr = paged_key_of_row(row);
    const int slot = row >> 4;   // = kr >> 4: the key order only permutes rows inside 16-row groups
    const int slot0 = __builtin_amdgcn_readfirstlane(slot);
    const uint32_t pid_a = (uint32_t)__builtin_amdgcn_readlane((int)ids, slot0);
    const uint32_t pid_b = (uint32_t)__builtin_amdgcn_readlane((int)ids, min(slot0 + 1, BC / 16 - 1));
    const uint32_t pid = slot == slot0 ? pid_a : pid_b;
    const uint64_t src = (uint64_t)(uintptr_t)(base + g * (16 * D)) + (uint32_t)((kr & 15) * (D * 2) + c * 16) +
                         (uint64_t)(pid * hkv_u) * (16 * D * 2);
    direct_load16((const void *)src, lds_addr(dst + ins * 1024));
  };
  constexpr int NPK = (KINS + NW - 1) / NW;  // direct loads per wave per K tile
  auto load_k_part = [&](int j, int buf, int i, uint32_t ids) {
    load_tile_part(kp, a.ks[2], j, sK[buf], std::integral_constant<int, KCP>{}, std::integral_constant<int, KCH>{},
                   std::integral_constant<int, KINS>{}, i, ids);
  };
  // Paged V^T tile, page-major: page s of the block holds its 16 keys for every dv as the cache
  // stores them ([dv][16 keys], 4 KB), so each 4 KB page is one plain copy: a direct load covers a
  // quarter of one page, whose id comes from a lane read of `ids`, and a lane's offset is its own
  // index.  Keys past the sequence's last page read that page (their values are zeroed before use).
  constexpr int VTPAGE = D * 16 * 2, VTINS = BC / 16 * VTPAGE / 1024;
  static_assert(!PAGED || (D == 128 && BC == 128 && VTINS * 1024 <= VBUF), "paged tiles are 128 x 128");
  constexpr int NPV = ((PAGED ? VTINS : VINS) + NW - 1) / NW;  // direct loads per wave per V tile
  auto load_v_part = [&](int j, int buf, int i, uint32_t ids) {
    if constexpr (PAGED) {
      const int ins = i * NW + wave;
      if (ins < VTINS) {
        constexpr int QPP = VTPAGE / 1024;   // direct loads per page
        const uint32_t pid = (uint32_t)__builtin_amdgcn_readlane((int)ids, ins / QPP);
        const uint64_t src = (uint64_t)(uintptr_t)(vp + g * (D * 16)) + (ins % QPP) * 1024 + lane * 16 +
                             (uint64_t)(pid * hkv_u) * (16 * D * 2);
        direct_load16((const void *)src, lds_addr(sV[buf] + ins * 1024));
      }
    } else {
      load_tile_part(vp, a.vs[2], j, sV[buf], std::integral_constant<int, VCP>{}, std::integral_constant<int, VCH>{},
                     std::integral_constant<int, VINS>{}, i, 0u);
    }
  };
  // The K tile of block t + 1 is loaded during block t's score MFMAs, spread evenly over them: a
  // wave that issues a tile's loads at once sits in the stalled issue until the memory pipeline
  // takes them, and issues no MFMA meanwhile.
  // Paged: wave 0 stages the ids of block j's 8 pages (clamped to the sequence's last page) into ring
  // slot j & 3, 4 bytes per lane.  Slot j & 3 is refilled (for block j + 4, at the top of iteration
  // j + 2) only after the barrier of iteration j + 1, which every wave reaches after its last read of
  // the slot (the V_j loads at the end of iteration j); the ids are read after the barrier that
  // follows the loads' wait.
  auto stage_ids = [&](int j) {
    if constexpr (PAGED) {
      if (wave == 0 && lane < BC / 16) direct_load4(tab + min(j * (BC / 16) + lane, last_page), lds_addr(sIds[j & 3]));
    }
  };

  // Transpose-read addressing for the V^T operand of k-step kk, dv m-tile mv: source lane
  // j = 4k + q of 16-lane group G points at V[16 kk + 4 (G / 2) + k][32 mv + 16 (G % 2) + 4 q ...+3];
  // the second read covers keys + 8.  Output lane l then holds dv 32 mv + l % 32 and the keys of
  // its lane half, in the order of its P^T fragment.
  const int tr_g = lane >> 4, tr_j = lane & 15;
  const int tr_off = ((tr_g >> 1) * 4 + (tr_j >> 2)) * VROW + (16 * (tr_g & 1) + 4 * (tr_j & 3)) * 2;

  // ---- online-softmax state (per lane: query row l32 of this wave) -----------------------------
  float m_dec = kNegInf;  // running max used by the skip rule (restarts at each split)
  float m_acc = kNegInf;  // running max of the accumulation
  // partial row sums over the keys this lane holds, of the bf16-rounded probabilities that also
  // enter P.V (two accumulators, summed in the epilogue, to shorten the dependency chain)
  float l_part = 0.f, l_part2 = 0.f;
  f32x16 o_acc[MTV];
#pragma unroll
  for (int i = 0; i < MTV; ++i) o_acc[i] = f32x16{};
  unsigned live_cnt = 0, skip_cnt = 0;
  const int mask_row = ((b * a.Hq + hq) * a.nqt + qt) * a.nkb;
  const bool tile_leader = wit == 0 && lane == 0;

  // ---- block loop, software-pipelined by one block.  Iteration t computes QK^T, row max and vote
  // of block t, then one barrier publishes the votes and makes K_{t+1} (loaded during block t's
  // score MFMAs) and V_{t-1} visible; then the P.V product of block t - 1 (its probabilities
  // packed in registers), and for a kept block t its probabilities and the direct loads of V_t.
  // So V is staged only for blocks that a tile of the workgroup kept. ----
  f32x16 s[MT];            // scores of block t
  bf16x8 pf_pend[KSV];     // bf16 probabilities of the kept block whose P.V is pending
  bool keep_pend = false;  // block t - 1 was kept by this tile
  if (PAGED && J > 0) {
    stage_ids(0);
    if (J > 1) stage_ids(1);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
  uint32_t ids_blk = 0u;   // paged: lane l holds the id of block t's page l % 8 (for the V_t loads)
  if (J > 0) {
    if (PAGED) ids_blk = (uint32_t)sIds[0][lane & 7];
#pragma unroll
    for (int i = 0; i < NPK; ++i) load_k_part(0, 0, i, ids_blk);
  }
  // a wait the compiler sees (not inline asm), on every path into the loop: without it the compiler
  // takes the Q fragments as possibly in flight at the loop head and waits for vmcnt(0), i.e. for the
  // K prefetch just issued, before the first QK^T product of every block
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  int to_split = 0;  // blocks left in the current split
  for (int t = 0; t <= J; ++t) {
    const int buf = t & 1;
    if (t + 2 < J) stage_ids(t + 2);
    const bool k_next = t + 1 < J;
    // paged: lane l holds the id of block t + 1's page l % 8 (published by the previous barrier)
    const uint32_t ids_next = PAGED && k_next ? (uint32_t)sIds[(t + 1) & 3][lane & 7] : 0u;
    float mx = kNegInf;
    if (t < J) {
      if (to_split == 0) {  // a split starts at this block
        m_dec = kNegInf;
        to_split = chunk;
      }
      --to_split;

      // ---- S^T = K_t Q^T one 32-key m-tile at a time; a finished tile is masked (blocks that need
      // it) while the next tile's MFMAs run, and folded into the row max (the compiler places the
      // maxima after the last tile's MFMAs; pinned between the tiles they measured no faster) ----
      const unsigned char *kb = sK[buf] + l32 * KROW + hi * 16;
      const int key0 = t * BC;
      const bool need_mask = (key0 + BC > Lk) || (a.causal && key0 + BC - 1 > r0 + off);
      const int lim = a.causal ? min(my_row + off, Lk - 1) : Lk - 1;
      auto fold = [&](int mt) {
        if (need_mask) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int kr = mt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);   // K tile row
            const int key = key0 + (PAGED ? paged_key_of_row(kr) : kr);
            if (key > lim) s[mt][r] = kNegInf;
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[mt][r]);
      };
      constexpr int NQ = MT * KS;
      constexpr int KSTEP = NQ / NPK;  // score MFMAs between two direct loads of the next K tile
      static_assert(KSTEP >= 1, "at most one K load per score MFMA");
      // K fragments two MFMAs ahead of their use, in a ring of three
      bf16x8 kf[3];
      kf[0] = *(const bf16x8 *)(kb);
      kf[1] = *(const bf16x8 *)(kb + (1 / KS) * 32 * KROW + (1 % KS) * 32);
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const int mt = q / KS, kk = q % KS;
        if (q + 2 < NQ) kf[(q + 2) % 3] = *(const bf16x8 *)(kb + ((q + 2) / KS) * 32 * KROW + ((q + 2) % KS) * 32);
        // one call site with the part index computed from q: with a call per part in the body, the
        // paged kernel's loop body outgrew the unroller's budget, the loop stayed rolled and the K
        // fragment ring was indexed at run time (select chains over every slot)
        if (k_next && q % KSTEP == 0 && q / KSTEP < NPK) load_k_part(t + 1, buf ^ 1, q / KSTEP, ids_next);
        s[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[q % 3], qf[kk], kk == 0 ? f32x16{} : s[mt], 0, 0, 0);
        if (mt > 0 && kk == 1) fold(mt - 1);
        if (q & 1) __builtin_amdgcn_sched_barrier(0);
      }
      fold(MT - 1);
      mx = max_xor32(mx);
      if (!row_ok || (QP && t >= J_me)) mx = kNegInf;   // every row of a block that is not live votes skip
      if (DEC) {
        const bool skip_row = row_votes_skip(mx, m_dec, thr_raw);
        const bool wave_keep = __ballot(!skip_row) != 0ull;
        float wcrit = 0.f;
        if (a.crit) wcrit = max_lanes32(row_crit(mx, m_dec));
        if (lane == 0) {
          sVote[buf][wave] = wave_keep ? 1 : 0;
          sCrit[buf][wave] = wcrit;
        }
      }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // K_{t+1} and V_{t-1} have landed in LDS
    __syncthreads();
    // Each SIMD runs one wave of each tile (waves w and w + 4).  From here to the end of the
    // iteration, tile 1's waves issue first: measured by phase timestamps, tile 0's wave otherwise ran
    // ahead into the next block's score MFMAs while tile 1's wave, slowed by them, was still in its
    // exponentials, and then waited for it at the next barrier.
    if (tile == 1) __builtin_amdgcn_s_setprio(2);

    if (!STATS && keep_pend) {
      // ---- kept block t - 1: O^T += V^T P^T ----
      const unsigned char *vb = sV[buf ^ 1] + tr_off;
      // paged: V^T row reads from the page-major tile; keys past the sequence end hold arbitrary
      // bytes and get V = 0
      const unsigned char *vtb = sV[buf ^ 1] + l32 * 32 + hi * 16;
      const int vkey0 = (t - 1) * BC;
      const bool vtail = PAGED && vkey0 + BC > Lk;
      // V^T operand of step q = (k-step q / MTV, dv m-tile q % MTV)
      auto read_vf = [&](int q) -> bf16x8 {
        const int kk = q / MTV, mv = q % MTV;
        bf16x8 vf;
        if constexpr (PAGED) {
          // keys 16 kk + 8 hi ... + 7 (page kk) of dv row 32 mv + l32 (the paged key order of the
          // scores): the wave reads 1 KB of consecutive bytes
          vf = *(const bf16x8 *)(vtb + kk * VTPAGE + mv * 32 * 32);
          if (vtail) {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (vkey0 + 16 * kk + 8 * hi + e >= Lk) vf[e] = (__bf16)0.f;
          }
        } else {
          const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + kk * 16 * VROW + mv * 64));
          const v4i16 up = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(vb + (kk * 16 + 8) * VROW + mv * 64));
          vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, up, 0, 1, 2, 3, 4, 5, 6, 7));
        }
        return vf;
      };
      // V^T fragments two MFMAs ahead of their use, in a ring of three (left to itself, the compiler
      // placed each fragment's reads right before its MFMA here, so every MFMA waited for its own LDS
      // reads)
      constexpr int NQV = KSV * MTV;
      bf16x8 vr[3];
      vr[0] = read_vf(0);
      vr[1] = read_vf(1);
#pragma unroll
      for (int q = 0; q < NQV; ++q) {
        if (q + 2 < NQV) vr[(q + 2) % 3] = read_vf(q + 2);
        o_acc[q % MTV] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[q % 3], pf_pend[q / MTV], o_acc[q % MTV], 0, 0, 0);
        if (q & 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t == J) break;

    const bool live = !QP || t < J_me;   // block t is live for this tile
    int keep = live ? 1 : 0, keep_any = 1;
    if (DEC) {
      keep = 0;
      keep_any = 0;
      const unsigned long long votes = NW == 8 ? *(const unsigned long long *)sVote[buf]
                                               : (unsigned long long)*(const unsigned *)sVote[buf];
      keep_any = votes != 0ull;
      // (a block that is not live for this tile is never kept: at lambda = 0 the threshold is -inf and
      // its rows, max -inf, would vote keep)
      keep = live && ((votes >> (tile * WPT * 8)) & ((1ull << (WPT * 8)) - 1ull)) != 0ull;
    }
    m_dec = fmaxf(m_dec, mx);
    if (live) {
      ++live_cnt;
      if (!keep) ++skip_cnt;
    }
    if (DEC && tile_leader && live) {
      if (a.mask) a.mask[mask_row + t] = keep ? kKept : kSkipped;
      if (a.crit) {
        float c = sCrit[buf][tile * WPT];
#pragma unroll
        for (int w = 1; w < WPT; ++w) c = fmaxf(c, sCrit[buf][tile * WPT + w]);
        a.crit[mask_row + t] = c * a.scale;
      }
    }
    if (!STATS && keep) {
      // ---- kept block t: online-softmax update and its probabilities ----
      // Lazy rescaling: the accumulation reference m_acc is raised only when a row's block max
      // exceeds it by more than 2^8 in probability (a row's first finite max just sets it: O and l
      // are still zero); below that, probabilities relative to the stale reference are at most 256,
      // which bf16 P and the fp32 sums hold with the same relative precision, and O / l and the
      // LSE are unchanged.  So the accumulators are rescaled only when the max jumps.  (O already
      // holds block t - 1: its P.V ran above.)
      if (m_acc == kNegInf) m_acc = mx;
      if (__ballot((mx - m_acc) * a.scale_log2 > 8.f) != 0ull) {
        const float m_new = fmaxf(m_acc, mx);
        const float alpha = fast_exp2((m_acc - m_new) * a.scale_log2);
        l_part *= alpha;
        l_part2 *= alpha;
#pragma unroll
        for (int i = 0; i < MTV; ++i) o_acc[i] *= alpha;
        m_acc = m_new;
      }
      const float base = (m_acc == kNegInf) ? 0.f : m_acc * a.scale_log2;
      // P^T for k-step kk (16 keys): keys of score registers s[kk/2][8*(kk%2) .. +7], i.e. key
      // 16*kk + 8*(e/4) + 4*hi + e%4 for element e.
      const bf16x2 one2 = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int kk = 0; kk < KSV; ++kk) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pf_pend[kk][e] = (__bf16)fast_exp2(__builtin_fmaf(s[kk >> 1][8 * (kk & 1) + e], a.scale_log2, -base));
        // row sum: one bf16 dot2 with (1, 1) per pair of probabilities
        const bf16x8 pf = pf_pend[kk];
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 0, 1), one2, l_part, false);
        l_part2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 2, 3), one2, l_part2, false);
        l_part = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 4, 5), one2, l_part, false);
        l_part2 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf, pf, 6, 7), one2, l_part2, false);
      }
    }
    // V_t only for a block that a tile of the workgroup kept, unless every live block's V is staged
    // (the buffer held V_{t-2}, whose P.V every wave finished before this iteration's barrier)
    if (!STATS && (keep_any || a.v_all)) {
#pragma unroll
      for (int i = 0; i < NPV; ++i) load_v_part(t, buf, i, ids_blk);
    }
    if (PAGED) ids_blk = ids_next;
    keep_pend = keep != 0;
    __builtin_amdgcn_s_setprio(0);
  }

  // ---- diagnostics for blocks that are not live ----
  if ((a.mask || a.crit) && tile_on) {
    for (int j = J_me + wit * 64 + lane; j < a.nkb; j += WPT * 64) {
      if (a.mask) a.mask[mask_row + j] = kNotLive;
      if (a.crit) a.crit[mask_row + j] = __builtin_nanf("");
    }
  }
  if (a.counters && tile_leader) {
    atomicAdd(&a.counters[0], (unsigned long long)live_cnt);
    atomicAdd(&a.counters[1], (unsigned long long)skip_cnt);
  }
  if (a.head_counters && tile_leader) {
    unsigned long long *hc = a.head_counters + 2 * (b * a.Hq + hq);
    atomicAdd(&hc[0], (unsigned long long)live_cnt);
    atomicAdd(&hc[1], (unsigned long long)skip_cnt);
  }
  if (STATS) return;

  // ---- epilogue: O = O^T / l, LSE = m * scale + ln l ----
  l_part += l_part2;
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

// QP: the two tiles of a workgroup are two query tiles of one head (odd GQA groups); otherwise two
// heads of one group at one query tile
template <int D, int BC, bool QP>
static hipError_t launch_pair(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  constexpr int NT = 64 * (BC / 32) * 2;
  const int grid = QP ? a.B * a.Hq * ((a.nqt + 1) / 2) : a.B * (a.Hq / 2) * a.nqt;
  if (a.stats_only)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, 2, false, true, true, false, QP>), dim3(grid), dim3(NT), 0, st, a);
  else if (out_f32)
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, 2, true, false, true, false, QP>), dim3(grid), dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, 2, false, false, true, false, QP>), dim3(grid), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int D, int BC>
static hipError_t launch_one(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  if constexpr (D == 128 && BC == 128) {
    // no threshold: the variant without decision logic (other shapes run with lambda = 0)
    if (!a.decide && a.G % 2 == 0 && !a.stats_only) {
      constexpr int NT = 64 * (BC / 32) * 2;
      const int grid = a.B * (a.Hq / 2) * a.nqt;
      if (out_f32)
        hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, 2, true, false, false>), dim3(grid), dim3(NT), 0, st, a);
      else
        hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, 2, false, false, false>), dim3(grid), dim3(NT), 0, st, a);
      return hipGetLastError();
    }
  }
  // two q heads of one GQA group share each staged K/V block when the group has an even size; for an
  // odd group, two query tiles of one head do
  if (a.G % 2 == 0) return launch_pair<D, BC, false>(a, out_f32, st);
  return launch_pair<D, BC, true>(a, out_f32, st);
}

// Chunked prefill against a paged cache (head dim 128, 128 x 128 blocks, 16-token pages).
template <bool QP>
static hipError_t launch_paged_pair(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  const int grid = QP ? a.B * a.Hq * ((a.nqt + 1) / 2) : a.B * (a.Hq / 2) * a.nqt;
  if (a.stats_only)
    hipLaunchKernelGGL((prefill_bf16_kernel<128, 128, 2, false, true, true, true, QP>), dim3(grid), dim3(512), 0, st, a);
  else if (out_f32)
    hipLaunchKernelGGL((prefill_bf16_kernel<128, 128, 2, true, false, true, true, QP>), dim3(grid), dim3(512), 0, st, a);
  else
    hipLaunchKernelGGL((prefill_bf16_kernel<128, 128, 2, false, false, true, true, QP>), dim3(grid), dim3(512), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_prefill_paged(const PrefillArgs &a, bool out_f32, hipStream_t st) {
  return a.G % 2 == 0 ? launch_paged_pair<false>(a, out_f32, st) : launch_paged_pair<true>(a, out_f32, st);
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

// Shared device helpers of the BLASST HIP kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blasst {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Mask byte values.
constexpr uint8_t kKept = 0, kSkipped = 1, kNotLive = 2;

// Arguments of the prefill kernels (one launch = the whole problem).
struct PrefillArgs {
  const void *q, *k, *v;
  void *o;
  float *lse;
  uint8_t *mask;
  float *crit;
  unsigned long long *counters;
  unsigned long long *head_counters;  // [B][Hq][2] or null
  int64_t qs[3], ks[3], vs[3], os[3];  // element strides: batch, head, token
  int B, Lq, Lk, Hq, Hkv, G;           // G = Hq / Hkv
  int nqt, nkb;                        // query tiles per head, key blocks per row of the mask
  int causal, num_splits, stats_only;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e): exp(scale*(s - m)) = exp2(scale_log2*(s - m))
  float thr_raw;     // ln(lambda) / scale: skip iff (m~ - m) < thr_raw on raw logits
  int decide;        // 0: no threshold at all (every live block kept, no vote)
  int v_all;         // 1: stage V for every live block, skipped or not (else only for kept blocks)
  // Paged K/V (chunked prefill against a paged cache; the kernel's PAGED variant): k is the key
  // cache [pages][Hkv][16][D], v the value cache [pages][Hkv][D][16] (V transposed inside each
  // page), table [B][max_pages] page ids, seq_lens [B] the context length of each sequence, whose
  // last Lq positions are the queries (Lk above is unused then).
  const int32_t *table, *seq_lens;
  int max_pages;
  int thr_mode;      // 0: thr_raw; 1: lambda_b = min(1, a_thr / seq_lens[b]) per sequence
  float a_thr;
};

// Arguments of the prefill backward kernels (bf16 inputs, head dim 128, 128 x 128 tile-blocks).
struct BwdArgs {
  const void *q, *k, *v, *o, *dout;   // bf16 (o: bf16 or fp32, o_f32)
  const float *lse;                   // forward LSE [B][Hq][Lq] (natural log, softmax scale included)
  const uint8_t *mask;                // forward skip mask [B][Hq][nqt][nkb]; null: every live block kept
  void *dq, *dk, *dv;                 // gradients, bf16 or fp32 (out_f32)
  float *dvec;                        // [B][Hq][Lq] rowsum(dO * O), written by the dQ kernel
  int64_t qs[3], ks[3], vs[3], os[3], dos[3], dqs[3], dks[3], dvs[3];  // element strides
  int B, Lq, Lk, Hq, Hkv, G, nqt, nkb, causal, out_f32, o_f32;
  float scale, scale_log2;
};

// Arguments of the paged decode kernels.
struct DecodeArgs {
  const void *q, *kc, *vc;
  const int32_t *table, *seq_lens;
  void *o;
  float *lse;
  uint8_t *mask;
  float *crit;
  unsigned long long *counters;
  float *ws_o;    // [B][Hq][S][Dv] per-split normalised outputs (num_splits > 1)
  float *ws_lse;  // [B][Hq][S]
  int B, Hq, Hkv, G, tile_rows, n_rt;
  int T;           // query tokens per sequence (the last T positions; token t sees keys <= L - T + t)
  int page, max_pages, block_k, nkb;
  int num_splits, stats_only, out_f32;
  int thr_mode;    // 0: fixed lambda (thr_raw valid); 1: lambda_b = min(1, a / seq_lens[b])
  float thr_raw;   // ln(lambda) / scale
  float a;         // for thr_mode 1
  float scale, scale_log2;
  int decide;      // 0: no threshold at all (every live block kept; the GQA kernel runs without votes)
};

// Row vote of the skip rule on raw (unscaled) logits: the row votes "skip" when
// m~ - m < thr, written as !(m~ - m >= thr) so that a row without visible keys (m~ = -inf, giving
// -inf or NaN) votes skip, and a row whose running max is still -inf (giving +inf) votes keep.
__device__ __forceinline__ bool row_votes_skip(float m_blk, float m_run, float thr) {
  return !((m_blk - m_run) >= thr);
}

// Critical value of one row in raw units: m~ - m with (-inf) - x = -inf, x - (-inf) = +inf.
__device__ __forceinline__ float row_crit(float m_blk, float m_run) {
  return m_blk == kNegInf ? kNegInf : m_blk - m_run;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8) that
// waits for vmcnt(0) only.  Passed to __builtin_amdgcn_s_waitcnt, the wait is visible to the
// compiler's own wait insertion, which then takes every earlier vector load as complete (a wait
// written as inline assembly is not).
constexpr int kWaitVmcnt0 = 0x0F70;

// Workgroup barrier that waits only for this wave's LDS operations.  __syncthreads() also waits for
// every outstanding global load (vmcnt(0)), which would stall on the next block's direct-to-LDS
// prefetch; here those loads stay in flight and are waited for explicitly before the buffer swap.
// Must be reached by every wave of the workgroup (uniform control flow).
__device__ __forceinline__ void barrier_lds_only() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4: lane i writes LDS bytes
// [lds_base + 16 i, lds_base + 16 i + 16) with lds_base taken from M0; lds_base must be the same
// in every lane).  Written out as assembly so that the compiler does not treat it as an LDS store
// it must wait for (s_waitcnt vmcnt(0)) before every later LDS read: kernels that use it order
// these loads themselves, with s_waitcnt vmcnt and a barrier before a buffer is read or refilled.
// The instruction has no register results.
// M0 is saved and restored around it, so the compiler's own use of M0 is not disturbed.
__device__ __forceinline__ void direct_load16(const void *addr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(addr), "s"(lds_base));
}

// direct_load16 marked non-temporal, for data that is read once (a decode's KV cache): streaming
// reads reach 7.0 TB/s on this chip this way against 6.2 TB/s with the default cache policy.
__device__ __forceinline__ void direct_load16_nt(const void *addr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(addr), "s"(lds_base));
}

// 4-byte form of direct_load16 (global_load_lds_dword: lane i writes LDS bytes [lds_base + 4 i,
// lds_base + 4 i + 4)); the same rules apply.
__device__ __forceinline__ void direct_load4(const void *addr, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(addr), "s"(lds_base));
}

// Buffer-resource form of the same direct load: 16 bytes per lane from the resource's base plus
// voff (a 32-bit byte offset per lane; reads past the resource's num_records return zero) into LDS
// bytes [lds_base + 16 i, lds_base + 16 i + 16).  rsrc = {base low 32 bits, base high 16 bits
// (stride 0), num_records in bytes, 0x00020000}; every operand but voff must be wave-uniform.
// Assembly for the same reason as direct_load16: written with the compiler builtin, a later LDS
// read of the other half of a double buffer waits for this load (vmcnt(0)).
__device__ __forceinline__ void buffer_load16_lds(u32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  uint32_t saved;
  asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds\n\ts_mov_b32 m0, %0"
               : "=&s"(saved)
               : "v"(voff), "s"(rsrc), "s"(lds_base));
}

// LDS byte address of a pointer into __shared__ memory
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void *)p;
}

// max over lanes l and l ^ 32
__device__ __forceinline__ float max_xor32(float x) { return fmaxf(x, __shfl_xor(x, 32)); }

// max over the 32 lanes that share l / 32 ... used for per-wave reductions of per-row values that
// are replicated in both halves: a full butterfly over offsets 16, 8, 4, 2, 1.
__device__ __forceinline__ float max_lanes32(float x) {
#pragma unroll
  for (int off = 16; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

// max over the 16-lane groups: lanes l, l ^ 16, l ^ 32, l ^ 48
__device__ __forceinline__ float max_xor16_32(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float sum_xor16_32(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 r;
  r[0] = (__bf16)lo;
  r[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

}  // namespace blasst

// Read-only streaming ceilings for the benchmark (measurement only, not part of the attention
// library): every byte of a buffer is read once with 16-byte non-temporal loads and folded into one
// word per thread, so the memory system serves nothing but reads.  Two access patterns:
//   * contiguous: a plain linear sweep, the practical HBM read rate of this GPU;
//   * pages: 4 KB pages in the order a table gives (a random permutation for a paged KV cache of
//     16-token pages of a 128-dim bf16 head), each page read whole by one wave, two pages in flight.
// Both are persistent grids: a workgroup of 256 threads strides over the buffer until it is done.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int TPB = 256;
constexpr int UNROLL = 8;        // 16-byte loads in flight per thread (contiguous)
constexpr int PAGE = 4096;       // bytes per page (pages pattern)
constexpr int NLD = PAGE / 1024; // wave-wide 1 KB loads per page

__global__ __launch_bounds__(TPB) void stream_contiguous(const u32x4 *__restrict__ src, uint64_t n16,
                                                         uint32_t *__restrict__ out) {
  const uint64_t step = (uint64_t)gridDim.x * TPB * UNROLL;
  uint64_t i = (uint64_t)blockIdx.x * TPB * UNROLL + threadIdx.x;
  u32x4 acc = {};
  // whole chunks of TPB * UNROLL vectors
  for (; i + (uint64_t)(UNROLL - 1) * TPB < n16; i += step) {
    u32x4 v[UNROLL];
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) v[k] = __builtin_nontemporal_load(src + i + (uint64_t)k * TPB);
#pragma unroll
    for (int k = 0; k < UNROLL; ++k) acc ^= v[k];
  }
  // the last, partial chunk (only the thread block whose chunk reaches past the end gets here with
  // i < n16, and it stays inside that chunk)
  for (; i < n16; i += TPB) acc ^= __builtin_nontemporal_load(src + i);
  out[(uint64_t)blockIdx.x * TPB + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

__global__ __launch_bounds__(TPB) void stream_pages(const unsigned char *__restrict__ pool, const int32_t *__restrict__ table,
                                                    int64_t n_pages, uint32_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (TPB / 64);
  const int64_t w0 = (int64_t)blockIdx.x * (TPB / 64) + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  u32x4 acc = {};
  // the page ids of 64 iterations come in with one load (lane l holds iteration l's id), so a page's
  // loads never wait on a table load
  for (int64_t base = w0; base < n_pages; base += 64 * waves) {
    const int64_t mine = base + lane * waves;
    const int32_t id = mine < n_pages ? table[mine] : 0;
    for (int k = 0; k < 64; k += 2) {
      const int64_t p = base + k * waves;
      if (p >= n_pages) break;
      const bool two = p + waves < n_pages;
      const int32_t ida = __builtin_amdgcn_readlane(id, k);
      const int32_t idb = __builtin_amdgcn_readlane(id, k + 1);
      const u32x4 *a = (const u32x4 *)(pool + (int64_t)ida * PAGE) + lane;
      const u32x4 *b = (const u32x4 *)(pool + (int64_t)(two ? idb : ida) * PAGE) + lane;
      u32x4 v[2 * NLD];
#pragma unroll
      for (int i = 0; i < NLD; ++i) v[i] = __builtin_nontemporal_load(a + 64 * i);
#pragma unroll
      for (int i = 0; i < NLD; ++i) v[NLD + i] = two ? __builtin_nontemporal_load(b + 64 * i) : u32x4{};
#pragma unroll
      for (int i = 0; i < 2 * NLD; ++i) acc ^= v[i];
    }
  }
  out[(uint64_t)blockIdx.x * TPB + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

// src: device buffer of `bytes` bytes (a multiple of 16, 16-byte aligned); out: device buffer of
// grid * 256 words (written, contents meaningless); stream: a hipStream_t (null = default stream).
// Returns 0, or the HIP error code of the launch; -1 for invalid arguments.
extern "C" int blasst_ceiling_stream_read(const void *src, uint64_t bytes, uint32_t *out, int grid, void *stream) {
  if (!src || !out || grid <= 0 || bytes % 16 != 0 || ((uintptr_t)src & 15) != 0) return -1;
  hipLaunchKernelGGL(stream_contiguous, dim3(grid), dim3(TPB), 0, (hipStream_t)stream, (const u32x4 *)src,
                     (uint64_t)(bytes / 16), out);
  return (int)hipGetLastError();
}

// pool: device buffer of n_pages pages of 4096 bytes (16-byte aligned); table: device array of
// n_pages page ids, each in [0, n_pages) (not checked: a permutation from the caller); out: device
// buffer of grid * 256 words; stream as above.  Returns 0, the HIP error code, or -1.
extern "C" int blasst_ceiling_stream_pages(const void *pool, const int32_t *table, int64_t n_pages, uint32_t *out,
                                           int grid, void *stream) {
  if (!pool || !table || !out || grid <= 0 || n_pages <= 0 || ((uintptr_t)pool & 15) != 0) return -1;
  hipLaunchKernelGGL(stream_pages, dim3(grid), dim3(TPB), 0, (hipStream_t)stream, (const unsigned char *)pool,
                     table, n_pages, out);
  return (int)hipGetLastError();
}

// page size of the pages pattern, for the caller's byte count
extern "C" int blasst_ceiling_page_bytes(void) { return PAGE; }

// Load-time demux and repack (moe_repack): kept-tier tensors are copied to their
// tier-local slots; the two NF3 code planes a checkpoint stores (a 2-bit low plane and a
// 1-bit high plane per row) become the 3-bit stream the forward kernels read (element j
// at bits [3 j, 3 j + 3) of its row, 12 bytes per 32 elements). The loader of the pages
// demuxes experts into tier-local storage and repacks them into its kernels' formats at
// load time (local-inference-lab/vllm PR #92, review walkthrough of the hybrid quant
// method; PR #104, "Summary").
//
// Jobs travel in the kernel arguments, kRepackJobs per launch; the blocks of a launch are
// dealt to its jobs by a prefix of block counts.
#include "device_common.h"
#include "hmoe_internal.h"

namespace hmoe {

// Eight elements: x holds their low code bits (element i at bits 2i..2i+1), h their
// high bits (element i at bit i); returns the 24-bit stream (element i at bits 3i..3i+2).
// Each 2-bit field moves up by i and each high bit by 2i + 2, done as three masked
// moves by 4, 2 and 1 (2i: 8, 4, 2), the largest first so no field lands on another.
__device__ __forceinline__ uint32_t nf3_spread8(uint32_t x, uint32_t h) {
  uint32_t t = (x & 0x00FFu) | ((x & 0xFF00u) << 4);       // fields 4..7 up by 4
  t = (t & ~0x000F00F0u) | ((t & 0x000F00F0u) << 2);       // fields 2, 3, 6, 7 up by 2
  t = (t & ~0x0030C30Cu) | ((t & 0x0030C30Cu) << 1);       // fields 1, 3, 5, 7 up by 1
  uint32_t u = (h & 0x0Fu) | ((h & 0xF0u) << 8);            // bits 4..7 up by 8
  u = (u & ~0x0000C00Cu) | ((u & 0x0000C00Cu) << 4);        // bits 2, 3, 6, 7 up by 4
  u = (u & ~0x00082082u) | ((u & 0x00082082u) << 2);        // bits 1, 3, 5, 7 up by 2
  return t | (u << 2);
}

// 32-element NF3 units: 8 low-plane bytes and 4 high-plane bytes in, 12 stream bytes out
__device__ __forceinline__ void nf3_unit(const uint32_t* lo, const uint32_t* hi, uint32_t* out, long u) {
  const uint32_t l0 = lo[2 * u], l1 = lo[2 * u + 1], h = hi[u];
  const uint32_t g0 = nf3_spread8(l0 & 0xFFFFu, h & 0xFFu);
  const uint32_t g1 = nf3_spread8(l0 >> 16, (h >> 8) & 0xFFu);
  const uint32_t g2 = nf3_spread8(l1 & 0xFFFFu, (h >> 16) & 0xFFu);
  const uint32_t g3 = nf3_spread8(l1 >> 16, h >> 24);
  out[3 * u] = g0 | (g1 << 24);
  out[3 * u + 1] = (g1 >> 8) | (g2 << 16);
  out[3 * u + 2] = (g2 >> 16) | (g3 << 8);
}

__global__ __launch_bounds__(kRepackThreads) void repack_kernel(RepackBatch b) {
  int j = 0;
  while (j + 1 < b.njobs && (int)blockIdx.x >= b.first_block[j + 1]) ++j;
  const RepackJob& job = b.job[j];
  const long i = (long)(blockIdx.x - b.first_block[j]) * kRepackThreads + threadIdx.x;
  if (job.kind == kRepackNf3) {
    if (i < job.n) nf3_unit(static_cast<const uint32_t*>(job.src), static_cast<const uint32_t*>(job.src_hi),
                            static_cast<uint32_t*>(job.dst), i);
  } else {
    // n bytes: 16-byte pieces where both ends allow it, bytes otherwise
    const uint8_t* s = static_cast<const uint8_t*>(job.src);
    uint8_t* d = static_cast<uint8_t*>(job.dst);
    const bool vec = ((reinterpret_cast<uintptr_t>(s) | reinterpret_cast<uintptr_t>(d)) & 15) == 0;
    if (vec) {
      const long nv = job.n / 16;
      if (i < nv) reinterpret_cast<uint4*>(d)[i] = reinterpret_cast<const uint4*>(s)[i];
      const long t = nv * 16 + i;  // tail bytes
      if (i < 16 && t < job.n) d[t] = s[t];
    } else {
      for (long k = i; k < job.n; k += (long)job.blocks * kRepackThreads) d[k] = s[k];
    }
  }
}

// blocks a job needs: one thread per NF3 unit or per 16 copied bytes
static int job_blocks(const RepackJob& j) {
  const long items = j.kind == kRepackNf3 ? j.n : (j.n + 15) / 16;
  const long b = (items + kRepackThreads - 1) / kRepackThreads;
  return (int)(b > 0 ? b : 1);
}

hipError_t launch_repack(RepackBatch& b, hipStream_t s) {
  int total = 0;
  for (int j = 0; j < b.njobs; ++j) {
    b.job[j].blocks = job_blocks(b.job[j]);
    b.first_block[j] = total;
    total += b.job[j].blocks;
  }
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(repack_kernel, dim3(total), dim3(kRepackThreads), 0, s, b);
  return hipGetLastError();
}

}  // namespace hmoe

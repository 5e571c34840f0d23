// Whole-block copies between block pools.
//
// [P2] "Unlocking long context ..." section 3.1: blocks of a shared prefix are
// reused with copy-on-write, so a sequence about to write into a shared, partly
// filled block first gets a private copy of it (the allocator names the pair).
// [P1] "Long-context inference engineering truths 2026 ..." section 4: KV
// blocks not needed for a while move from HBM to host memory and back.  Both
// are the same operation: copy every kv head's K and V page (and, for E4M3
// pools, the two scales) of block src_ids[i] of one pool to block dst_ids[i]
// of another.  A pool in pinned host memory is addressed by the kernel
// directly (its loads or stores cross PCIe), so an offload or a page-in is one
// launch on the caller's stream, which can overlap attention on another.
#include <algorithm>

#include "pkv_common.h"

namespace pkv {
namespace {

constexpr int CT = 256;
constexpr int kHostCopyGroups = 16;        // workgroups of a copy that crosses PCIe

// Workgroup x takes block pairs x, x + gridDim.x, ... and copies a
// 1/gridDim.y share of each with 16-byte non-temporal loads and stores (each
// byte is moved once); K and V regions of a block are contiguous runs of
// `region` bytes in their pools.
__global__ __launch_bounds__(CT) void copy_blocks_kernel(CopyArgs a, int n) {
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int sb = a.src_ids[i], db = a.dst_ids[i];
    if ((unsigned)sb >= (unsigned)a.src_blocks || (unsigned)db >= (unsigned)a.dst_blocks) continue;
    const u32x4* sk = reinterpret_cast<const u32x4*>(a.src_k + sb * a.src_stride);
    const u32x4* sv = reinterpret_cast<const u32x4*>(a.src_v + sb * a.src_stride);
    u32x4* dk = reinterpret_cast<u32x4*>(a.dst_k + db * a.dst_stride);
    u32x4* dv = reinterpret_cast<u32x4*>(a.dst_v + db * a.dst_stride);
    const int64_t n16 = a.region >> 4;
    for (int64_t o = (int64_t)blockIdx.y * CT + threadIdx.x; o < n16;
         o += (int64_t)CT * gridDim.y) {
      const u32x4 k = __builtin_nontemporal_load(sk + o);
      const u32x4 v = __builtin_nontemporal_load(sv + o);
      __builtin_nontemporal_store(k, dk + o);
      __builtin_nontemporal_store(v, dv + o);
    }
    if (a.src_ks && blockIdx.y == 0) {
      for (int h = threadIdx.x; h < a.hkv; h += CT) {
        a.dst_ks[(int64_t)db * a.hkv + h] = a.src_ks[(int64_t)sb * a.hkv + h];
        a.dst_vs[(int64_t)db * a.hkv + h] = a.src_vs[(int64_t)sb * a.hkv + h];
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_blocks(const CopyArgs& a, int n, hipStream_t s, bool host_pool) {
  if (n <= 0) return hipSuccess;
  if (host_pool) {
    // PCIe, not the CUs, bounds a copy to or from host memory: 16 workgroups
    // keep the link busy (56 GB/s measured, as with one workgroup per block)
    // and disturb an attention running beside the copy far less than many
    // (8192-token decode of 32 sequences, four-wave workgroups, beside a
    // 128 MiB page-in: 73 % of the page-in hidden with 16, 62 % with 32, 23 %
    // with 64; 8 no longer fill the link; beside the two-wave decode, which
    // leaves no CU idle, 16 hide 54 %).
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(std::min(n, kHostCopyGroups), 1), dim3(CT), 0, s,
                       a, n);
    return hipGetLastError();
  }
  const int64_t per_block = (a.region >> 4) / CT;            // full passes of one workgroup
  // few pairs (a copy-on-write): split each block over several workgroups
  int split = (int)std::max<int64_t>(1, std::min<int64_t>(per_block, (512 + n - 1) / n));
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n, split), dim3(CT), 0, s, a, n);
  return hipGetLastError();
}

}  // namespace pkv

// lq_ceiling.hip — memory-system ceilings for liblq's lane-contiguous
// fake-quant kernels (declared in include/lq_ceiling.h): a copy, and the exact
// load/store pattern of a bf16 call with the quantization arithmetic left out.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lq_ceiling.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <typename V>
__device__ __forceinline__ void nt_store(V* p, V v) {
  __builtin_nontemporal_store(v, p);
}

struct Pair {
  u32x4 a, b;   // half A (elements 8L..8L+7) and half B (512+8L..512+8L+7) of one chunk
};

__device__ __forceinline__ Pair load_pair(const void* x, int64_t chunk, int lane) {
  const u32x4* p = (const u32x4*)((const char*)x + (chunk * 1024 + 8 * lane) * 2);
  return Pair{p[0], p[64]};   // 1024 bytes on
}

// s_waitcnt vmcnt(0): the first chunk lands before the loop, so the loop's
// own waits only cover the prefetch (as in liblq's kernels)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int NT>
__global__ void __launch_bounds__(NT) k_copy(const void* src, void* dst, int64_t nchunks) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  Pair r;
  if (w0 < nchunks) r = load_pair(src, w0, lane);
  wait_vmem_all();
  for (int64_t c = w0; c < nchunks; c += stride) {
    const Pair cur = r;
    if (c + stride < nchunks) r = load_pair(src, c + stride, lane);
    u32x4* q = (u32x4*)((char*)dst + (c * 1024 + 8 * lane) * 2);
    nt_store(q, cur.a);
    nt_store(q + 64, cur.b);
  }
}

// Read-only stream in the same layout: a wave's 2 KB chunk per pass (two
// 16-byte loads per lane), the next chunk's loads issued before this one's are
// folded in (xor). A lane writes its fold, to its wave's word of sink, only
// when the fold equals one fixed value: the store keeps the loads, and almost
// never happens.
template <int NT>
__global__ void __launch_bounds__(NT) k_read(const void* src, int64_t nchunks, uint32_t* sink) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  uint32_t acc = 0;
  Pair r;
  if (w0 < nchunks) r = load_pair(src, w0, lane);
  wait_vmem_all();
  for (int64_t c = w0; c < nchunks; c += stride) {
    const Pair cur = r;
    if (c + stride < nchunks) r = load_pair(src, c + stride, lane);
    acc ^= cur.a[0] ^ cur.a[1] ^ cur.a[2] ^ cur.a[3] ^ cur.b[0] ^ cur.b[1] ^ cur.b[2] ^ cur.b[3];
  }
  if (acc == 0x9E3779B9u) sink[w0] = acc;   // w0 < gridDim.x * kWaves
}

// Write-only stream: a wave's 1 KB (16 bytes per lane, whole lines) per pass,
// non-temporal, of values made from the unit index.
template <int NT>
__global__ void __launch_bounds__(NT) k_write(void* dst, int64_t nunits) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  for (int64_t u = w0; u < nunits; u += stride) {
    const uint32_t v = (uint32_t)u;
    nt_store((u32x4*)((char*)dst + u * 1024 + 16 * lane), (u32x4){v, v ^ (uint32_t)lane, v + 1u, ~v});
  }
}

// codes: the high byte of each bf16 (8-bit codes) or its top nibble packed
// two per byte (4-bit codes), so every store depends on the loaded data
__device__ __forceinline__ u32x2 hi_bytes(const u32x4& v) {
  return (u32x2){__builtin_amdgcn_perm(v[1], v[0], 0x07050301u), __builtin_amdgcn_perm(v[3], v[2], 0x07050301u)};
}
__device__ __forceinline__ uint32_t hi_nibbles(const u32x4& v) {
  const u32x2 b = hi_bytes(v);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 8; i++) w |= ((((i < 4 ? b[0] : b[1]) >> (8 * (i & 3) + 4)) & 0xFu) << (4 * i));
  return w;
}

template <int NT, int CODE_BITS>
__global__ void __launch_bounds__(NT) k_pattern(const void* x, int64_t nchunks, uint8_t* codes, uint8_t* scales,
                                               int block_shift, int block_lanes, void* y) {
  constexpr int kWaves = NT / 64;
  const int lane = threadIdx.x & 63;
  const int64_t w0 = (int64_t)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t stride = (int64_t)gridDim.x * kWaves;
  Pair r;
  if (w0 < nchunks) r = load_pair(x, w0, lane);
  wait_vmem_all();
  for (int64_t c = w0; c < nchunks; c += stride) {
    const Pair cur = r;
    if (c + stride < nchunks) r = load_pair(x, c + stride, lane);
    const int64_t e0 = c * 1024 + 8 * lane;
    if ((lane & (block_lanes - 1)) == 0) {
      scales[e0 >> block_shift] = (uint8_t)(cur.a[0] >> 24);
      scales[(e0 + 512) >> block_shift] = (uint8_t)(cur.b[0] >> 24);
    }
    if constexpr (CODE_BITS == 8) {
      u32x2* p = (u32x2*)(codes + e0);
      nt_store(p, hi_bytes(cur.a));
      nt_store(p + 64, hi_bytes(cur.b));   // 512 bytes on
    } else if constexpr (CODE_BITS == 6) {
      // a half's eight 6-bit codes are 6 bytes at 6L of the half's 384: a
      // dword and a short, each naturally aligned (even lanes dword first)
      uint8_t* p = codes + c * 768 + 6 * lane;
      const bool odd = (lane & 1) != 0;
#pragma unroll
      for (int h = 0; h < 2; h++) {
        const u32x2 b = hi_bytes(h == 0 ? cur.a : cur.b);
        uint8_t* q = p + 384 * h;
        nt_store((uint32_t*)(q + (odd ? 2 : 0)), b[0]);
        nt_store((uint16_t*)(q + (odd ? 0 : 4)), (uint16_t)b[1]);
      }
    } else {
      uint32_t* p = (uint32_t*)(codes + e0 / 2);
      nt_store(p, hi_nibbles(cur.a));
      nt_store(p + 64, hi_nibbles(cur.b)); // 256 bytes on
    }
    u32x4* q = (u32x4*)((char*)y + e0 * 2);
    nt_store(q, cur.a);
    nt_store(q + 64, cur.b);
  }
}

bool aligned(const void* p) { return ((uintptr_t)p & 15u) == 0u; }

int log2i(int v) {
  int s = 0;
  while ((1 << s) < v) s++;
  return s;
}

}  // namespace

extern "C" {

int lqc_copy(const void* src, size_t src_bytes, void* dst, size_t dst_bytes, int64_t n, int threads, int workgroups,
             void* stream) {
  if (!src || !dst) return -1;
  if (n <= 0 || n % 1024 != 0 || workgroups < 1 || (threads != 256 && threads != 1024)) return -3;
  if (src_bytes < (size_t)n * 2 || dst_bytes < (size_t)n * 2) return -3;
  if (!aligned(src) || !aligned(dst)) return -4;
  hipStream_t s = (hipStream_t)stream;
  if (threads == 256) hipLaunchKernelGGL(k_copy<256>, dim3(workgroups), dim3(256), 0, s, src, dst, n / 1024);
  else hipLaunchKernelGGL(k_copy<1024>, dim3(workgroups), dim3(1024), 0, s, src, dst, n / 1024);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int lqc_read(const void* src, size_t src_bytes, int64_t bytes, void* sink, size_t sink_bytes, int threads,
             int workgroups, void* stream) {
  if (!src || !sink) return -1;
  if (bytes <= 0 || bytes % 2048 != 0 || workgroups < 1 || (threads != 256 && threads != 1024)) return -3;
  if (src_bytes < (size_t)bytes || sink_bytes < (size_t)workgroups * (size_t)(threads / 64) * 4u) return -3;
  if (!aligned(src) || !aligned(sink)) return -4;
  hipStream_t s = (hipStream_t)stream;
  uint32_t* k = (uint32_t*)sink;
  if (threads == 256) hipLaunchKernelGGL(k_read<256>, dim3(workgroups), dim3(256), 0, s, src, bytes / 2048, k);
  else hipLaunchKernelGGL(k_read<1024>, dim3(workgroups), dim3(1024), 0, s, src, bytes / 2048, k);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int lqc_write(void* dst, size_t dst_bytes, int64_t bytes, int threads, int workgroups, void* stream) {
  if (!dst) return -1;
  if (bytes <= 0 || bytes % 1024 != 0 || workgroups < 1 || (threads != 256 && threads != 1024)) return -3;
  if (dst_bytes < (size_t)bytes) return -3;
  if (!aligned(dst)) return -4;
  hipStream_t s = (hipStream_t)stream;
  if (threads == 256) hipLaunchKernelGGL(k_write<256>, dim3(workgroups), dim3(256), 0, s, dst, bytes / 1024);
  else hipLaunchKernelGGL(k_write<1024>, dim3(workgroups), dim3(1024), 0, s, dst, bytes / 1024);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

int lqc_pattern(const void* x, size_t x_bytes, int64_t n, void* codes, size_t codes_bytes, int code_bits, void* scales,
                size_t scales_bytes, int block, void* y, size_t y_bytes, int threads, int workgroups, void* stream) {
  if (!x || !codes || !scales || !y) return -1;
  if (n <= 0 || n % 1024 != 0 || workgroups < 1 || (threads != 256 && threads != 1024)) return -3;
  if ((code_bits != 4 && code_bits != 6 && code_bits != 8) ||
      (block != 16 && block != 32 && block != 64 && block != 128 && block != 256))
    return -3;
  if (x_bytes < (size_t)n * 2 || y_bytes < (size_t)n * 2 || codes_bytes < (size_t)n / 8 * code_bits ||
      scales_bytes < (size_t)(n / block))
    return -3;
  if (!aligned(x) || !aligned(codes) || !aligned(scales) || !aligned(y)) return -4;
  hipStream_t s = (hipStream_t)stream;
  const int64_t nch = n / 1024;
  uint8_t* c = (uint8_t*)codes;
  uint8_t* sc = (uint8_t*)scales;
  const int bs = log2i(block), bl = block / 8;
  if (threads == 256) {
    if (code_bits == 8) hipLaunchKernelGGL((k_pattern<256, 8>), dim3(workgroups), dim3(256), 0, s, x, nch, c, sc, bs, bl, y);
    else if (code_bits == 6) hipLaunchKernelGGL((k_pattern<256, 6>), dim3(workgroups), dim3(256), 0, s, x, nch, c, sc, bs, bl, y);
    else hipLaunchKernelGGL((k_pattern<256, 4>), dim3(workgroups), dim3(256), 0, s, x, nch, c, sc, bs, bl, y);
  } else {
    if (code_bits == 8) hipLaunchKernelGGL((k_pattern<1024, 8>), dim3(workgroups), dim3(1024), 0, s, x, nch, c, sc, bs, bl, y);
    else if (code_bits == 6) hipLaunchKernelGGL((k_pattern<1024, 6>), dim3(workgroups), dim3(1024), 0, s, x, nch, c, sc, bs, bl, y);
    else hipLaunchKernelGGL((k_pattern<1024, 4>), dim3(workgroups), dim3(1024), 0, s, x, nch, c, sc, bs, bl, y);
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"

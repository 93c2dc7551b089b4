// Router logits on the matrix cores for bf16 activations: L = x @ Wr^T with
// fp32 accumulation (the gating product of the Edge0 "MoE Spec and Routing"
// page, router_logits; the gate of the "Mixture of Experts" blog page's
// route function).
//
// * bf16 router weights: one bf16 x bf16 product per element, exact in
//   fp32, accumulated in fp32 by v_mfma_f32_32x32x16_bf16.
// * fp32 router weights: each weight is split once per call into three
//   bf16 parts w = hi + mid + lo (hi = bf16(w), mid = bf16(w - hi), lo =
//   w - hi - mid, which has at most 8 significant bits and so is exact in
//   bf16); the product x*w is then the sum of three exact bf16 products, so
//   the logit is an fp32-accumulated sum of 3d exact terms -- fp32 accuracy
//   from the bf16 matrix cores.  The three parts are laid out as one row of
//   length 3d per expert ([hi | mid | lo]); each K step loads one x tile
//   and the three matching weight tiles.
// * the reduction is split over S workgroups per tile (S chosen so the
//   launch fills the chip); split s writes its partial logits to plane s
//   of a [S][T][E] fp32 buffer, and the selection kernel adds the planes in
//   order s = 0..S-1, so the result does not depend on timing.
//
// Tile: 128 tokens x BN experts (BN = 32, 64, 128 or 256) per 256-thread
// workgroup; wave w owns tokens 32w..32w+31 and every expert of the tile.
// Both operands are K-contiguous and go straight to LDS with direct loads
// (double-buffered K steps of 64); rows past T or E get an out-of-range
// offset and load as zeros.
#include <algorithm>

#include "moe_internal.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int RBM = 128;        // tokens per tile
constexpr int RBK = 64;         // K step (elements)
constexpr int kRowB = RBK * 2;  // 128 bytes per tile row and K step
constexpr int kRThreads = 256;

// same XOR swizzle of 16-byte chunks as the expert GEMM's 128-byte rows
__device__ __forceinline__ int rswz(int r, int c) {
  return r * kRowB + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// fp32 [E][d] -> bf16 [E][3d] = [hi | mid | lo]
__global__ void __launch_bounds__(256)
router_split_kernel(const float* __restrict__ w, uint16_t* __restrict__ w3,
                    int E, int d) {
  const int64_t n = static_cast<int64_t>(E) * d;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
       i < n; i += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t e = i / d, k = i - e * d;
    const float v = w[i];
    const uint16_t hi = f32_to_bf16(v);
    const float r1 = v - bf16_to_f32(hi);
    const uint16_t mid = f32_to_bf16(r1);
    const float r2 = r1 - bf16_to_f32(mid);
    const uint16_t lo = f32_to_bf16(r2);
    uint16_t* row = w3 + e * 3 * d;
    row[k] = hi;
    row[d + k] = mid;
    row[2 * d + k] = lo;
  }
}

// The tile body is a device function template instantiated by one plain
// kernel per tile width (the host compiler does not emit launch stubs for
// a kernel template whose body holds these direct-to-LDS loads).
template <int NBLK, int NPASS>
__device__ __forceinline__ void router_tile(const uint16_t* __restrict__ x,
                                            uint32_t x_bytes, int64_t T, int d,
                                            const uint16_t* __restrict__ w,
                                            uint32_t w_bytes, int wld, int E,
                                            int kt_total, int kt_split,
                                            float* __restrict__ part,
                                            int64_t pstride) {
  constexpr int BN = 32 * NBLK;
  constexpr int kXBytes = RBM * kRowB;          // 16 KiB
  constexpr int kWBytes = NPASS * BN * kRowB;   // the weight parts of one K step
  __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (kXBytes + kWBytes)];
  uint8_t* sX = smem;
  uint8_t* sW = smem + 2 * kXBytes;

  const int mt = blockIdx.x, nt = blockIdx.y, sp = blockIdx.z;
  const int k0 = sp * kt_split;
  const int k1 = min(kt_total, k0 + kt_split);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  const __amdgpu_buffer_rsrc_t rsX = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(x), (short)0, static_cast<int>(x_bytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(w), (short)0, static_cast<int>(w_bytes), 0x00020000);
  // 1 KiB direct loads: x tile = 16 blocks (4 per wave), W tile = 4*NBLK
  // blocks (NBLK per wave); lane l fills position l%8 of row l/8
  uint32_t voffX[4], voffW[NBLK];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = (j * 4 + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    const int64_t t = static_cast<int64_t>(mt) * RBM + r;
    voffX[j] = t < T ? static_cast<uint32_t>(t * d * 2 + c * 16) : x_bytes;
  }
#pragma unroll
  for (int j = 0; j < NBLK; ++j) {
    const int r = (j * 4 + wave) * 8 + (lane >> 3);
    const int c = (lane & 7) ^ ((r ^ (r >> 3)) & 7);
    const int e = nt * BN + r;
    voffW[j] = e < E ? static_cast<uint32_t>(static_cast<int64_t>(e) * wld * 2 + c * 16)
                     : w_bytes;
  }
  auto issue = [&](int ks, int buf) {
    const int xo = ks * kRowB;
    uint8_t* xs = sX + buf * kXBytes;
    uint8_t* ws = sW + buf * kWBytes;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsX, (__attribute__((address_space(3))) void*)(xs + (j * 4 + wave) * 1024), 16,
          voffX[j], xo, 0, 0);
#pragma unroll
    for (int q = 0; q < NPASS; ++q)
#pragma unroll
      for (int j = 0; j < NBLK; ++j)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsW,
            (__attribute__((address_space(3))) void*)(ws + q * BN * kRowB +
                                                      (j * 4 + wave) * 1024),
            16, voffW[j], (q * d + ks * RBK) * 2, 0, 0);
  };

  f32x16 acc[NBLK];
#pragma unroll
  for (int i = 0; i < NBLK; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  const int fr = lane & 31, fh = lane >> 5;
  if (k0 < k1) {
    issue(k0, 0);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    for (int ks = k0; ks < k1; ++ks) {
      const int cur = (ks - k0) & 1;
      if (ks + 1 < k1) issue(ks + 1, cur ^ 1);
      const uint8_t* xs = sX + cur * kXBytes;
      const uint8_t* ws = sW + cur * kWBytes;
#pragma unroll
      for (int kk = 0; kk < RBK / 16; ++kk) {
        const int ch = kk * 2 + fh;
        const bf16x8 xf = *reinterpret_cast<const bf16x8*>(xs + rswz(wave * 32 + fr, ch));
#pragma unroll
        for (int q = 0; q < NPASS; ++q)
#pragma unroll
          for (int nb = 0; nb < NBLK; ++nb) {
            const bf16x8 wf = *reinterpret_cast<const bf16x8*>(
                ws + q * BN * kRowB + rswz(nb * 32 + fr, ch));
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf, xf, acc[nb], 0, 0, 0);
          }
      }
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
      __syncthreads();
    }
  }

  // lane holds, for block nb and item v: expert nt*BN + 32nb + 8(v/4) +
  // 4(lane/32) + v%4 of token 32*wave + lane%32
  const int64_t t = static_cast<int64_t>(mt) * RBM + wave * 32 + fr;
  if (t >= T) return;
  float* prow = part + sp * pstride + t * E;
#pragma unroll
  for (int nb = 0; nb < NBLK; ++nb)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int e0 = nt * BN + nb * 32 + 8 * q + 4 * fh;
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (e0 + v < E) prow[e0 + v] = acc[nb][4 * q + v];
    }
}

#define MOE_ROUTER_KERNEL(N, P)                                                 \
  __global__ void __launch_bounds__(kRThreads, 1) router_mfma_kernel_##N##_##P( \
      const uint16_t* x, uint32_t x_bytes, int64_t T, int d, const uint16_t* w, \
      uint32_t w_bytes, int wld, int E, int kt_total, int kt_split, float* part, \
      int64_t pstride) {                                                        \
    router_tile<N, P>(x, x_bytes, T, d, w, w_bytes, wld, E, kt_total, kt_split, \
                      part, pstride);                                           \
  }
MOE_ROUTER_KERNEL(1, 1)
MOE_ROUTER_KERNEL(2, 1)
MOE_ROUTER_KERNEL(4, 1)
MOE_ROUTER_KERNEL(8, 1)
MOE_ROUTER_KERNEL(1, 3)
MOE_ROUTER_KERNEL(2, 3)
MOE_ROUTER_KERNEL(4, 3)
#undef MOE_ROUTER_KERNEL

}  // namespace

RouterPlan router_plan(const Dims& D, int router_dtype) {
  RouterPlan p{};
  // a few tokens (decode) stay on the vector-ALU kernels: one tile would
  // hold mostly padding and the split of fp32 weights would dominate
  p.mfma = D.bf16 && D.d % RBK == 0 && D.T >= 256;
  if (!p.mfma) {
    p.S = 1;
    return p;
  }
  p.npass = router_dtype == MOE_DTYPE_F32 ? 3 : 1;
  // a K step's weight parts share LDS with the x tile: three parts fit up
  // to 128 experts per tile
  p.BN = D.E <= 32 ? 32 : D.E <= 64 ? 64 : (D.E <= 128 || p.npass == 3) ? 128 : 256;
  p.mtiles = static_cast<int>((D.T + RBM - 1) / RBM);
  p.ntiles = (D.E + p.BN - 1) / p.BN;
  p.kt_total = D.d / RBK;
  const int64_t tiles = static_cast<int64_t>(p.mtiles) * p.ntiles;
  // about two workgroups per CU of a 256-CU part, at least 4 K steps each
  int S = static_cast<int>(std::min<int64_t>(kMaxLogitPlanes, (512 + tiles - 1) / tiles));
  S = std::max(1, std::min(S, p.kt_total / 4));
  p.kt_split = (p.kt_total + S - 1) / S;
  p.S = (p.kt_total + p.kt_split - 1) / p.kt_split;
  return p;
}

hipError_t launch_router_mfma(const Dims& D, const RouterPlan& p, const void* x,
                              const void* wr, uint16_t* w3, float* part,
                              hipStream_t s) {
  const uint16_t* w = static_cast<const uint16_t*>(wr);
  int wld = D.d;
  if (p.npass == 3) {
    const int64_t n = static_cast<int64_t>(D.E) * D.d;
    const int blocks = static_cast<int>(std::min<int64_t>((n + 255) / 256, 4096));
    hipLaunchKernelGGL(router_split_kernel, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(wr), w3, D.E, D.d);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    w = w3;
    wld = 3 * D.d;
  }
  const uint32_t x_bytes = static_cast<uint32_t>(D.T * D.d * 2);
  const uint32_t w_bytes = static_cast<uint32_t>(static_cast<int64_t>(D.E) * wld * 2);
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  const dim3 grid(p.mtiles, p.ntiles, p.S), block(kRThreads);
  const int64_t ps = D.T * D.E;
#define MOE_RMFMA(N, P)                                                              \
  hipLaunchKernelGGL(router_mfma_kernel_##N##_##P, grid, block, 0, s, xp, x_bytes, D.T, \
                     D.d, w, w_bytes, wld, D.E, p.kt_total, p.kt_split, part, ps)
  if (p.npass == 3) {
    switch (p.BN) {
      case 32: MOE_RMFMA(1, 3); break;
      case 64: MOE_RMFMA(2, 3); break;
      default: MOE_RMFMA(4, 3); break;
    }
  } else {
    switch (p.BN) {
      case 32: MOE_RMFMA(1, 1); break;
      case 64: MOE_RMFMA(2, 1); break;
      case 128: MOE_RMFMA(4, 1); break;
      default: MOE_RMFMA(8, 1); break;
    }
  }
#undef MOE_RMFMA
  return hipGetLastError();
}

}  // namespace moe

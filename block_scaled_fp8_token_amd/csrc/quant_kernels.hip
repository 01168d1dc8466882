// Quantization kernels for gfx950 (kernel family (a) of the library):
//   * per-token 1x128 group quant with the UE8M0 scale pack done in the same
//     pass (vLLM PR #29546 "Deepgemm fused layout kernel for activations",
//     Purpose: pack the scales into a uint32 early instead of in a second kernel);
//   * fused SiLU-and-mul + the same quant over a masked expert batch, skipping
//     padded rows (vLLM PR #19885 "Optimize the little operations in the
//     DeepGEMM + DeepEP low latency case", Summary item 2);
//   * 128x128 weight block quant (the offline weight step of the vLLM DeepGEMM
//     FP8 block GEMM benchmark post, section 4.1).
//
// All three are HBM-bound streams.  The activation kernels give one wavefront
// one (row, packed word) unit: 64 lanes x 8 bf16 = 512 columns = the four
// 128-column groups whose exponent bytes share a word.  Each 16-lane row of the
// wavefront owns one group, so the group amax is a 16-lane reduction and the
// word is assembled from lanes 0, 16, 32 and 48 without touching LDS.
#include "fp8bs_device.hpp"
#include "fp8bs_launch.hpp"

namespace fp8bs {

namespace {

__device__ __forceinline__ void unpack8(const uint4 v, float* f) {
  f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x);
  f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
  f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z);
  f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
}

// Quantize the eight values a lane holds for one group and return (e4m3 bytes,
// exponent byte).  The eight values are already in registers as fp32.
__device__ __forceinline__ uint2 quant8(float* f, bool valid, uint32_t* ebyte) {
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
  amax = max16(amax);
  const int e = ue8m0_exponent(amax);
  const float s = exp2i(-e);  // exact: -e in [-120, 42]
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] *= s;
  *ebyte = valid ? (uint32_t)(e + 127) : 0u;
  return e4m3x8(f);
}

__device__ __forceinline__ uint32_t gather_word(uint32_t ebyte) {
  const uint32_t b0 = __shfl(ebyte, 0), b1 = __shfl(ebyte, 16);
  const uint32_t b2 = __shfl(ebyte, 32), b3 = __shfl(ebyte, 48);
  return b0 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

__global__ __launch_bounds__(256) void quant_group_pack_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t M, int64_t K,
    uint8_t* __restrict__ q, int64_t ldq, uint32_t* __restrict__ sf, int64_t ld_sf, int64_t W) {
  const int lane = threadIdx.x & 63;
  const int64_t units = M * W;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
    const int64_t r = u / W, w = u - r * W;
    const int64_t col = w * 512 + lane * 8;
    const bool valid = col < K;  // K % 128 == 0, so validity is uniform per group
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (valid) v = *reinterpret_cast<const uint4*>(x + r * ldx + col);
    float f[8];
    unpack8(v, f);
    uint32_t eb;
    const uint2 o = quant8(f, valid, &eb);
    if (valid) *reinterpret_cast<uint2*>(q + r * ldq + col) = o;
    const uint32_t word = gather_word(eb);
    if (lane == 0) sf[w * ld_sf + r] = word;
  }
}

// y = silu(g) * u = g / (1 + exp(-g)) * u in fp32 for the rows r < masked_m[e] of
// expert e; gate is columns [0, H) and up is [H, 2H) of each input row.
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ masked_m, int64_t M_max, int64_t H,
    uint8_t* __restrict__ q, uint32_t* __restrict__ sf, int64_t W, int rows_per_block) {
  const int64_t e = blockIdx.y;
  int64_t c = masked_m[e];
  c = c < 0 ? 0 : (c > M_max ? M_max : c);
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  if (r0 >= c) return;  // padded rows: nothing is read or written
  const int64_t r1 = (r0 + rows_per_block < c) ? r0 + rows_per_block : c;
  const int lane = threadIdx.x & 63;
  const int64_t units = (r1 - r0) * W;
  for (int64_t u = threadIdx.x >> 6; u < units; u += 4) {
    const int64_t r = r0 + u / W, w = u % W;
    const int64_t col = w * 512 + lane * 8;
    const bool valid = col < H;
    const uint16_t* row = x + (e * M_max + r) * 2 * H;
    uint4 gv = make_uint4(0u, 0u, 0u, 0u), uv = make_uint4(0u, 0u, 0u, 0u);
    if (valid) {
      gv = *reinterpret_cast<const uint4*>(row + col);
      uv = *reinterpret_cast<const uint4*>(row + H + col);
    }
    float g[8], up[8];
    unpack8(gv, g);
    unpack8(uv, up);
#pragma unroll
    for (int i = 0; i < 8; ++i) g[i] = g[i] / (1.0f + expf(-g[i])) * up[i];
    uint32_t eb;
    const uint2 o = quant8(g, valid, &eb);
    if (valid) *reinterpret_cast<uint2*>(q + (e * M_max + r) * H + col) = o;
    const uint32_t word = gather_word(eb);
    if (lane == 0) sf[(e * W + w) * M_max + r] = word;
  }
}

// One workgroup per 128x128 block: 2048 16-byte chunks, eight per thread, held in
// registers between the block-amax reduction and the quantization.
__global__ __launch_bounds__(256) void block_quant_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, uint8_t* __restrict__ q,
    float* __restrict__ sfb, int64_t KB) {
  __shared__ float wmax[4];
  const int64_t kb = blockIdx.x, nb = blockIdx.y;
  const int t = threadIdx.x;
  uint4 v[8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cidx = t + 256 * i, row = cidx >> 4, ch = cidx & 15;
    const int64_t n = nb * 128 + row;
    v[i] = make_uint4(0u, 0u, 0u, 0u);
    if (n < N) v[i] = *reinterpret_cast<const uint4*>(w + n * K + kb * 128 + ch * 8);
    float f[8];
    unpack8(v[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[j]));
  }
  amax = max16(amax);
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 16));
  amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32));
  if ((t & 63) == 0) wmax[t >> 6] = amax;
  __syncthreads();
  amax = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
  const int e = ue8m0_exponent(amax);
  const float s = exp2i(-e);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cidx = t + 256 * i, row = cidx >> 4, ch = cidx & 15;
    const int64_t n = nb * 128 + row;
    float f[8];
    unpack8(v[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] *= s;
    if (n < N) *reinterpret_cast<uint2*>(q + n * K + kb * 128 + ch * 8) = e4m3x8(f);
  }
  if (t == 0) sfb[nb * KB + kb] = exp2i(e);
}

}  // namespace

hipError_t launch_quant_group_pack(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                   int64_t ldq, uint32_t* sf, int64_t ld_sf, hipStream_t stream) {
  const int64_t W = (K / 128 + 3) / 4;
  const int64_t units = M * W;
  int64_t blocks = (units + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(quant_group_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, M, K,
                     q, ldq, sf, ld_sf, W);
  return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t* x, const int32_t* masked_m, int64_t E, int64_t M_max,
                                 int64_t H, uint8_t* q, uint32_t* sf, hipStream_t stream) {
  const int64_t W = (H / 128 + 3) / 4;
  // about four units (one per wavefront) per workgroup
  int rows_per_block = (int)((4 + W - 1) / W);
  if (rows_per_block < 1) rows_per_block = 1;
  const int64_t bx = (M_max + rows_per_block - 1) / rows_per_block;
  if (bx < 1 || E < 1) return hipSuccess;
  hipLaunchKernelGGL(silu_mul_quant_kernel, dim3((unsigned)bx, (unsigned)E), dim3(256), 0, stream, x,
                     masked_m, M_max, H, q, sf, W, rows_per_block);
  return hipGetLastError();
}

hipError_t launch_block_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb,
                              hipStream_t stream) {
  const int64_t KB = K / 128, NB = (N + 127) / 128;
  if (KB < 1 || NB < 1) return hipSuccess;
  hipLaunchKernelGGL(block_quant_kernel, dim3((unsigned)KB, (unsigned)NB), dim3(256), 0, stream, w, N, K,
                     q, sfb, KB);
  return hipGetLastError();
}

}  // namespace fp8bs

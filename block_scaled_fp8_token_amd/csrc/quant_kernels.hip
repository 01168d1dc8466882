// Quantization kernels for gfx950 (kernel family (a) of the library):
//   * per-token 1x128 group quant with the UE8M0 scale pack done in the same
//     pass (vLLM PR #29546 "Deepgemm fused layout kernel for activations",
//     Purpose: pack the scales into a uint32 early instead of in a second kernel);
//   * fused SiLU-and-mul + the same quant over a masked expert batch, skipping
//     padded rows (vLLM PR #19885 "Optimize the little operations in the
//     DeepGEMM + DeepEP low latency case", Summary item 2);
//   * 128x128 weight block quant (the offline weight step of the vLLM DeepGEMM
//     FP8 block GEMM benchmark post, section 4.1);
//   * float-scale variants of the activation and weight quant (scale = amax / 448
//     unrounded: the non-UE8M0 format of the benchmark post, section 4.1);
//   * the same per-token quant written straight into the masked expert layout of
//     the routed tokens (the quantization half of FP8 dispatch: PR #19885,
//     Summary item 1, DeepEP puts the scales in DeepGEMM's layout; PR #19111 review,
//     the TODO asking for a batched quant).
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
    // streaming store: the codes are read by the next kernel, not through this CU's caches
    // (2048x7168: 9.28 -> 8.32 us)
    if (valid) __builtin_nontemporal_store(((uint64_t)o.y << 32) | o.x, reinterpret_cast<uint64_t*>(q + r * ldq + col));
    const uint32_t word = gather_word(eb);
    if (lane == 0) sf[w * ld_sf + r] = word;
  }
}

// y = silu(g) * u = g / (1 + exp(-g)) * u in fp32 for the rows r < masked_m[e] of
// expert e; gate is columns [0, H) and up is [H, 2H) of each input row.  The division
// is a hardware reciprocal (1 ulp) and a multiply: y stays within a few fp32 ulps of
// the exact value, far inside the 2^-19 relative window around e4m3 rounding points
// where the quantized byte may differ from a double evaluation; g = 0, large g and
// exp overflow give the same +-0, g*u and -0 as the division (measured 10% faster:
// the IEEE division sequence was a fifth of the kernel's VALU instructions).  Units are
// (row, packed word) pairs in row-major order; each wavefront takes UPW consecutive
// units of expert blockIdx.y, issues the gate and up loads of all of them before
// the first is converted (2 UPW loads in flight), and skips units of rows at or past
// the count (no loads, no stores).
template <int UPW>
__global__ __launch_bounds__(256) void silu_mul_quant_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ masked_m, int64_t M_max, int64_t H,
    uint8_t* __restrict__ q, uint32_t* __restrict__ sf, int64_t W) {
  const int64_t e = blockIdx.y;
  int64_t c = masked_m[e];
  c = c < 0 ? 0 : (c > M_max ? M_max : c);
  // wavefront-uniform unit index, computed on the scalar unit
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t u0 = ((int64_t)blockIdx.x * 4 + wave) * UPW;
  if (u0 / W >= c) return;  // padded rows: nothing is read or written
  const int lane = threadIdx.x & 63;
  uint4 gv[UPW], uv[UPW];
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int64_t u = u0 + i, r = u / W, w = u - r * W;
    const int64_t col = w * 512 + lane * 8;
    gv[i] = make_uint4(0u, 0u, 0u, 0u);
    uv[i] = make_uint4(0u, 0u, 0u, 0u);
    if (r < c && col < H) {
      const uint16_t* row = x + (e * M_max + r) * 2 * H;
      gv[i] = *reinterpret_cast<const uint4*>(row + col);
      uv[i] = *reinterpret_cast<const uint4*>(row + H + col);
    }
  }
#pragma unroll
  for (int i = 0; i < UPW; ++i) {
    const int64_t u = u0 + i, r = u / W, w = u - r * W;
    if (r >= c) break;  // uniform per wavefront
    const int64_t col = w * 512 + lane * 8;
    const bool valid = col < H;
    float g[8], up[8];
    unpack8(gv[i], g);
    unpack8(uv[i], up);
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = g[k] * __builtin_amdgcn_rcpf(1.0f + expf(-g[k])) * up[k];
    uint32_t eb;
    const uint2 o = quant8(g, valid, &eb);
    if (valid) *reinterpret_cast<uint2*>(q + (e * M_max + r) * H + col) = o;
    const uint32_t word = gather_word(eb);
    if (lane == 0) sf[(e * W + w) * M_max + r] = word;
  }
}

constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past every row: the load returns zeros

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* ptr = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(ptr, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}

// The same operation over the valid rows only.  Every wavefront forms the prefix
// sums of the clamped counts (E <= 64, one expert per lane), so the dense index of a
// valid row maps to its expert (the first lane whose running sum passes it) and its
// row in that expert; a grid sized to the GPU strides over the (row, word) units of
// the valid rows, and each wavefront issues the gate and up loads of its next unit
// before it converts the current one.  Padded rows cost neither a load nor a
// workgroup.  The arithmetic per unit is the kernel's above, value for value.
__global__ __launch_bounds__(256) void silu_mul_quant_compact_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ masked_m, int E, int64_t M_max, int64_t H,
    uint8_t* __restrict__ q, uint32_t* __restrict__ sf, int W) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int cnt = 0;
  if (lane < E) {
    const int64_t c = masked_m[lane];
    cnt = (int)(c < 0 ? 0 : (c > M_max ? M_max : c));
  }
  int incl = cnt;  // running sum of the counts of experts 0 .. lane
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  // from here on every index is wavefront-uniform (scalar registers): the unit's
  // dense row rr, word w, expert e and the expert's dense row range [beg, end)
  const int total = __builtin_amdgcn_readlane(incl, 63);
  const int units = total * W;  // < 2^31 (host)
  const int stride = (int)gridDim.x * 4;
  int u = (int)blockIdx.x * 4 + wave;
  if (u >= units) return;
  const int sr = stride / W, sw = stride - sr * W;
  int rr = u / W, w = u - rr * W;
  int e = 0, beg = 0, end = __builtin_amdgcn_readlane(incl, 0);
  auto seek = [&]() {  // the expert of rr: rr < total, so e stays below E
    while (end <= rr) {
      ++e;
      beg = end;
      end = __builtin_amdgcn_readlane(incl, e);
    }
  };
  seek();
  const int64_t lcol = lane * 8;
  // buffer loads over one input row (2H bf16): lanes past H and the look-ahead past
  // the last unit read out of range and get zeros, so the loop body has no branch
  // around its loads and the compiler's wait before a unit's conversion leaves the
  // next unit's loads in flight
  const uint32_t row_bytes = (uint32_t)(4 * H);
  auto load = [&](int64_t row, int ww, bool ok, uint4& gv, uint4& uv) {
    const __amdgpu_buffer_rsrc_t rs = row_rsrc(x + row * 2 * H, row_bytes);
    const int64_t col = (int64_t)ww * 512 + lcol;
    const uint32_t off = (ok && col < H) ? (uint32_t)(col * 2) : kOutOfRange;
    gv = bload16(rs, off);
    uv = bload16(rs, off + (uint32_t)(2 * H));
  };
  int64_t row = (int64_t)e * M_max + (rr - beg);  // row of x, q: expert e, row rr - beg
  // one unit: look ahead to the next unit and issue its loads into (gn, un), then
  // convert and store the current one from (gv, uv); false after the last unit.
  // The loop below alternates two register sets, so no loaded register is copied
  // (a copy would wait for the look-ahead loads).
  auto unit = [&](const uint4& gv, const uint4& uv, uint4& gn, uint4& un) -> bool {
    const bool more = u < units - stride;  // uniform per wavefront
    const int64_t cur_row = row;
    const int cur_w = w;
    const int64_t cur_r = rr - beg;
    const int cur_e = e;
    if (more) {
      u += stride;
      w += sw;
      rr += sr;
      if (w >= W) {
        w -= W;
        ++rr;
      }
      seek();
      row = (int64_t)e * M_max + (rr - beg);
    }
    load(row, w, more, gn, un);
    __builtin_amdgcn_sched_barrier(0);  // the look-ahead loads go out before any use of (gv, uv)
    const int64_t col = (int64_t)cur_w * 512 + lcol;
    const bool valid = col < H;
    float g[8], up[8];
    unpack8(gv, g);
    unpack8(uv, up);
#pragma unroll
    for (int k = 0; k < 8; ++k) g[k] = g[k] * __builtin_amdgcn_rcpf(1.0f + expf(-g[k])) * up[k];
    uint32_t eb;
    const uint2 o = quant8(g, valid, &eb);
    // streaming store ([32, 256, 4096] with Zipf counts: 8.96 -> 8.64 us)
    if (valid) __builtin_nontemporal_store(((uint64_t)o.y << 32) | o.x, reinterpret_cast<uint64_t*>(q + cur_row * H + col));
    const uint32_t word = gather_word(eb);
    if (lane == 0) sf[((int64_t)cur_e * W + cur_w) * M_max + cur_r] = word;
    return more;
  };
  uint4 g0, u0, g1, u1;
  load(row, w, true, g0, u0);
  while (unit(g0, u0, g1, u1) && unit(g1, u1, g0, u0)) {
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

// Float-scale variants (the non-UE8M0 format of the benchmark post, section 4.1:
// the scale of a group or block is amax / 448 itself, not rounded to a power of
// two).  All in IEEE fp32 with correctly rounded division:
//   s = max(amax, 1e-10f) / 448,  q = e4m3_rne(clamp(x / s, -448, 448)).
__device__ __forceinline__ float float_scale(float amax) {
  const float a = amax > 1e-10f ? amax : 1e-10f;
  return a / 448.0f;
}

// One wavefront per (row, 512 columns): four groups, lanes 16g..16g+15 hold group g.
// Scales fp32 [K/128][ld_sf] (one float per group, M-major).
__global__ __launch_bounds__(256) void quant_group_float_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t M, int64_t K, uint8_t* __restrict__ q,
    int64_t ldq, float* __restrict__ sf, int64_t ld_sf, int64_t W) {
  const int lane = threadIdx.x & 63;
  const int64_t units = M * W;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
    const int64_t r = u / W, w = u - r * W;
    const int64_t col = w * 512 + lane * 8;
    const bool valid = col < K;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (valid) v = *reinterpret_cast<const uint4*>(x + r * ldx + col);
    float f[8];
    unpack8(v, f);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(f[i]));
    amax = max16(amax);
    const float sc = float_scale(amax);
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = f[i] / sc;
    if (valid) {
      *reinterpret_cast<uint2*>(q + r * ldq + col) = e4m3x8(f);
      if ((lane & 15) == 0) sf[(w * 4 + (lane >> 4)) * ld_sf + r] = sc;
    }
  }
}

// One workgroup per 128x128 block (as block_quant_kernel) with the float scale.
__global__ __launch_bounds__(256) void block_quant_float_kernel(
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
  const float sc = float_scale(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int cidx = t + 256 * i, row = cidx >> 4, ch = cidx & 15;
    const int64_t n = nb * 128 + row;
    float f[8];
    unpack8(v[i], f);
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = f[j] / sc;
    if (n < N) *reinterpret_cast<uint2*>(q + n * K + kb * 128 + ch * 8) = e4m3x8(f);
  }
  if (t == 0) sfb[nb * KB + kb] = sc;
}

// Expert slots of routed tokens (the dispatch half of FP8 dispatch on one GPU): pair
// p = t * topk + j of token t's choice j goes to expert ids[p]; its slot is the
// number of earlier pairs (in p order) routed to the same expert, and pairs whose
// slot reaches M_max, or whose id names no expert, get slot -1.  Two parallel
// passes, fully deterministic:
//   * route_rank_kernel: one workgroup per chunk of 1024 pairs ranks every pair
//     among the chunk's earlier pairs of its expert (inside a wavefront with
//     ballots, across wavefronts with per-wavefront counts in LDS) and writes the
//     chunk's per-expert counts;
//   * quant_to_experts_kernel adds the counts of the earlier chunks to a pair's
//     rank when it needs the slot.
constexpr int kRouteThreads = 1024;
constexpr int kRouteMaxExperts = 1024;

__global__ __launch_bounds__(kRouteThreads) void route_rank_kernel(
    const int32_t* __restrict__ ids, int64_t P, int64_t E, int32_t* __restrict__ rank_of,
    int32_t* __restrict__ chunk_counts) {
  constexpr int NW = kRouteThreads / 64;
  __shared__ int wcnt[NW][kRouteMaxExperts];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int e = tid; e < E; e += kRouteThreads)
#pragma unroll
    for (int w = 0; w < NW; ++w) wcnt[w][e] = 0;
  const int64_t p = (int64_t)blockIdx.x * kRouteThreads + tid;
  const int e = p < P ? ids[p] : -1;
  const bool valid = e >= 0 && e < E;
  __syncthreads();
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int rank = 0;
  uint64_t pending = __ballot(valid);
  while (pending) {  // one pass per distinct expert of this wavefront (uniform)
    const int leader = __builtin_ctzll(pending);
    const int el = __builtin_amdgcn_readlane(e, leader);
    const uint64_t m = __ballot(valid && e == el);
    if (valid && e == el) rank = __builtin_popcountll(m & below);
    if (lane == leader) wcnt[wave][el] = __builtin_popcountll(m);
    pending &= ~m;
  }
  __syncthreads();
  if (p < P) {
    int r = -1;
    if (valid) {
      r = rank;
      for (int w = 0; w < wave; ++w) r += wcnt[w][e];
    }
    rank_of[p] = r;
  }
  for (int e2 = tid; e2 < E; e2 += kRouteThreads) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += wcnt[w][e2];
    chunk_counts[blockIdx.x * E + e2] = tot;
  }
}

// Quantize every token once (the per-token group quant above, one wavefront per
// (token, packed word)) and write its e4m3 row and scale word to the slot of each
// of its routed choices in the masked expert layout q [E][M_max][K],
// sf [E][W][M_max].  Pairs with slot -1 write nothing.  The wavefronts of word 0
// also store the slots; workgroup 0 stores the per-expert row counts.
__global__ __launch_bounds__(256) void quant_to_experts_kernel(
    const uint16_t* __restrict__ x, int64_t ldx, int64_t T, int64_t K, const int32_t* __restrict__ ids,
    const int32_t* __restrict__ rank_of, const int32_t* __restrict__ chunk_counts, int64_t nchunks, int topk,
    int64_t E, int64_t M_max, uint8_t* __restrict__ q, uint32_t* __restrict__ sf, int64_t W,
    int32_t* __restrict__ masked_m, int32_t* __restrict__ slot_of) {
  const int lane = threadIdx.x & 63;
  if (blockIdx.x == 0)
    for (int64_t e = threadIdx.x; e < E; e += 256) {
      int64_t tot = 0;
      for (int64_t c = 0; c < nchunks; ++c) tot += chunk_counts[c * E + e];
      masked_m[e] = (int32_t)(tot < M_max ? tot : M_max);
    }
  const int64_t units = T * W;
  const int64_t nwaves = (int64_t)gridDim.x * 4;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < units; u += nwaves) {
    const int64_t t = u / W, w = u - t * W;
    const int64_t col = w * 512 + lane * 8;
    const bool valid = col < K;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (valid) v = *reinterpret_cast<const uint4*>(x + t * ldx + col);
    // lane j < topk resolves choice j's slot: its rank in its chunk plus the counts
    // of its expert in the earlier chunks
    const int64_t pj = t * topk + lane;
    int32_t my_slot = -1, my_e = 0;
    if (lane < topk) {
      const int32_t r = rank_of[pj];
      my_e = ids[pj];
      if (r >= 0) {
        int64_t sl = r;
        const int64_t cj = pj / kRouteThreads;
        for (int64_t c = 0; c < cj; ++c) sl += chunk_counts[c * E + my_e];
        my_slot = sl < M_max ? (int32_t)sl : -1;
      }
      if (w == 0) slot_of[pj] = my_slot;
    }
    float f[8];
    unpack8(v, f);
    uint32_t eb;
    const uint2 o = quant8(f, valid, &eb);
    const uint32_t word = gather_word(eb);
    for (int j = 0; j < topk; ++j) {
      const int32_t s = __builtin_amdgcn_readlane(my_slot, j);
      if (s < 0) continue;  // uniform per wavefront
      const int64_t e = __builtin_amdgcn_readlane(my_e, j);
      // streaming store (512 tokens x top-8 into the expert layout: 13.8 -> 12.3 us)
      if (valid)
        __builtin_nontemporal_store(((uint64_t)o.y << 32) | o.x, reinterpret_cast<uint64_t*>(q + (e * M_max + s) * K + col));
      if (lane == 0) sf[(e * W + w) * M_max + s] = word;
    }
  }
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
  // more than 64 experts: one unit per wavefront over the whole padded grid (two
  // units, or a whole row of four, per wavefront measured 13% / 33% slower)
  constexpr int UPW = 1;
  const int64_t W = (H / 128 + 3) / 4;
  const int64_t bx = (M_max * W + 4 * UPW - 1) / (4 * UPW);  // four wavefronts of UPW units per workgroup
  if (bx < 1 || E < 1) return hipSuccess;
  if (E <= 64 && E * M_max * W < (int64_t)1 << 30) {
    // valid rows only, four workgroups per compute unit (of 256): 32 experts x 256
    // rows x H = 2048 with Zipf counts (2780 valid rows) 11.0 -> 8.8 us, with every
    // row valid 20.4 -> 20.9 us; more workgroups were slower in both cases
    int64_t blocks = (E * M_max * W + 3) / 4;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(silu_mul_quant_compact_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, masked_m,
                       (int)E, M_max, H, q, sf, (int)W);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(silu_mul_quant_kernel<UPW>, dim3((unsigned)bx, (unsigned)E), dim3(256), 0, stream, x,
                     masked_m, M_max, H, q, sf, W);
  return hipGetLastError();
}

hipError_t launch_quant_to_experts(const uint16_t* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids,
                                  int topk, int64_t E, int64_t M_max, uint8_t* q, uint32_t* sf,
                                  int32_t* masked_m, int32_t* slot_of, int32_t* scratch, hipStream_t stream) {
  if (E < 1 || E > kRouteMaxExperts) return hipErrorInvalidValue;
  const int64_t P = T * topk;
  const int64_t nchunks = (P + kRouteThreads - 1) / kRouteThreads;
  int32_t* rank_of = scratch;
  int32_t* chunk_counts = scratch + P;
  if (nchunks > 0) {
    hipLaunchKernelGGL(route_rank_kernel, dim3((unsigned)nchunks), dim3(kRouteThreads), 0, stream, ids, P, E,
                       rank_of, chunk_counts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t W = (K / 128 + 3) / 4;
  int64_t blocks = (T * W + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;  // workgroup 0 still stores the counts
  hipLaunchKernelGGL(quant_to_experts_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, T, K, ids,
                     rank_of, chunk_counts, nchunks, topk, E, M_max, q, sf, W, masked_m, slot_of);
  return hipGetLastError();
}

size_t quant_to_experts_scratch_bytes(int64_t T, int topk, int64_t E) {
  const int64_t P = T * topk;
  const int64_t nchunks = (P + kRouteThreads - 1) / kRouteThreads;
  return (size_t)(P + nchunks * E) * sizeof(int32_t);
}

hipError_t launch_quant_group_float(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                   int64_t ldq, float* sf, int64_t ld_sf, hipStream_t stream) {
  const int64_t W = (K / 128 + 3) / 4;
  int64_t blocks = (M * W + 3) / 4;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) return hipSuccess;
  hipLaunchKernelGGL(quant_group_float_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ldx, M, K, q,
                     ldq, sf, ld_sf, W);
  return hipGetLastError();
}

hipError_t launch_block_quant_float(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb,
                                   hipStream_t stream) {
  const int64_t KB = K / 128, NB = (N + 127) / 128;
  if (KB < 1 || NB < 1) return hipSuccess;
  hipLaunchKernelGGL(block_quant_float_kernel, dim3((unsigned)KB, (unsigned)NB), dim3(256), 0, stream, w, N, K,
                     q, sfb, KB);
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

// Pre-shuffled weight layout: thread t moves the 16 bytes of output chunk t.  With
// t = ((g * KB + kb) * 4 + q) * 64 + l, the chunk holds row 32 g + (l & 31), bytes
// 128 kb + 64 (q >> 1) + 32 (l >> 5) + 16 (q & 1) .. + 15: the bytes lane l of a
// wavefront loads with its q-th 16-byte load of K-block kb for the 32 x 64 operands
// of two scaled MFMAs, so that every such load reads 1 KB of contiguous memory.
__global__ __launch_bounds__(256) void weight_preshuffle_kernel(const uint8_t* __restrict__ w,
                                                                uint8_t* __restrict__ out, int64_t rows,
                                                                int64_t K) {
  const int64_t KB = K / 128;
  const int64_t chunks = rows * (K / 16);
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < chunks; t += (int64_t)gridDim.x * 256) {
    const int l = (int)(t & 63), q = (int)((t >> 6) & 3);
    const int64_t gk = t >> 8, g = gk / KB, kb = gk - g * KB;
    const int64_t row = 32 * g + (l & 31);
    const int64_t col = 128 * kb + 64 * (q >> 1) + 32 * (l >> 5) + 16 * (q & 1);
    *reinterpret_cast<uint4*>(out + 16 * t) = *reinterpret_cast<const uint4*>(w + row * K + col);
  }
}

hipError_t launch_weight_preshuffle(const uint8_t* w, int64_t rows, int64_t K, uint8_t* out, hipStream_t stream) {
  const int64_t chunks = rows * (K / 16);
  if (chunks < 1) return hipSuccess;
  int64_t blocks = (chunks + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(weight_preshuffle_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, out, rows, K);
  return hipGetLastError();
}

}  // namespace fp8bs

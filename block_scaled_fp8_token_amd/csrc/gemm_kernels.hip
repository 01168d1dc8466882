// Block-scaled FP8 GEMM kernels for gfx950 (kernel families (b) dense NT and
// (c) masked grouped).
//
//   C[m][n] = bf16( sum over K-blocks kb of 2^ea[m][kb] * sfb[n/128][kb]
//                   * sum_{k in kb} a[m][k] * b[n][k] )
//
// which is the per-K-block scale-then-accumulate loop of the vLLM DeepGEMM FP8
// block GEMM benchmark post, section 4.2 (the Triton kernel multiplies each
// K-block dot product by the A and B scales before adding it to the fp32
// accumulator), with the activation scales of section 4.1 (1x128 groups, UE8M0,
// packed four to a word, M-major) and 128x128 weight blocks.  The masked form
// follows vLLM PR #19111 "Integrate batched/masked deepgemm kernel": a batch of
// [E][M_max][K] activations where only the first masked_m[e] rows of group e
// are valid; the counts stay on the device.
//
// Kernel families in this file (the automatic choice is in choose_gemm_config):
//   * wsd_kernel: dense M <= 64 on pre-shuffled weights.  Weight streaming: each
//     lane loads its MFMA operand bytes (one contiguous kilobyte per wavefront load)
//     straight into registers several K-blocks ahead, the activation K-blocks go to
//     LDS by LDS-DMA, K is split over workgroups and the splits of a tile sum their
//     fp32 partials inside the kernel (last arriver, in part order: deterministic).
//   * decode_kernel: dense M <= 64 on the plain [N][K] layout (weights through an LDS
//     ring) and the float-scale decode; partials summed by splitk_reduce_kernel.
//   * ring2_kernel: prefill, masked and contiguous grouped, on either weight layout.
//     LDS-DMA rings of whole 128-byte K-block rows (or, on pre-shuffled weights, one
//     contiguous kilobyte per weight DMA instruction), one barrier per K-block,
//     v_mfma_scale_f32_32x32x64_f8f6f4 with the packed UE8M0 bytes as scale operands
//     (the scale-then-accumulate of each K-block happens in the matrix core), bf16
//     epilogue staged through LDS, XCD-aware tile order; the grouped forms stream their
//     weights with non-temporal DMA.  Its float-scale form runs the MFMAs unscaled and
//     adds P * (sa * sb) on the VALU.
//   * scaled_ring_kernel (K-half stages; where K is past ring2_kernel's scale tables),
//     scaled_tile_kernel (two-stage tiles), stream_kernel and gemm_kernel (the
//     first design: LDS via registers, 16x16x128 MFMA on zero then a VALU scale FMA):
//     fallbacks for shapes and K ranges the others do not take.
// The MFMA is issued with the weight tile as its first operand, so all of a lane's
// results share one output row m: one activation scale per lane.  Workgroups whose
// rows all lie past the mask return before any load; 32-row groups past the mask
// issue no operand reads or MFMAs.
#include <atomic>

#include "fp8bs_device.hpp"
#include "fp8bs_launch.hpp"

namespace fp8bs {

namespace {

constexpr int LDS_ROW = 144;  // 128 data bytes + 16 pad bytes per row of a K-block tile
constexpr uint32_t kOOB = 0x80000000u;  // buffer offset past every descriptor range: loads return 0

// Raw buffer resource over [base, base + bytes); gfx9 descriptor word 3 (raw, 32-bit format).
// The fields are passed through readfirstlane: they are wave-uniform, and saying so
// keeps the compiler from wrapping every load in a per-lane descriptor loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* u = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(u, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4((uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]);
}
__device__ __forceinline__ uint32_t bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0);
}

struct KArgs {
  const uint8_t* a;
  const uint32_t* sfa;
  const uint8_t* b;
  const float* sfb;
  uint16_t* c;
  const int32_t* masked_m;
  int64_t M, N, K, ld_sfa, ldc;
  int64_t sa_e, ssfa_e, sb_e, ssfb_e, sc_e;  // per-group strides (elements)
  int tiles_m, tiles_n, splits, kb_per_split;
  int sa_words;  // activation-scale words per row a split can touch (LDS table height)
  float* ws;  // split-K partials [splits][M][N]
  uint32_t* counters;  // per-tile arrival counters of the fused split-K (zero between calls)
  const int32_t* m_indices;  // contiguous grouped layout: weight group of every row, or nullptr
  int64_t groups;            // weight groups m_indices may name
  const float* sfa_f;        // float activation scales [K/128][ld_sfa] (float-scale kernels), or nullptr
};

// Weight group of the tile whose first row is m0: the grid's group e (dense and
// masked calls), or in the contiguous grouped layout the group of row m0, where
// every aligned tile holds rows of one group followed by padding; -1 (tile
// skipped) when that row is padding or names no group.
__device__ __forceinline__ int64_t weight_group(const KArgs& p, int64_t e, int64_t m0) {
  if (!p.m_indices) return e;
  const int64_t g = p.m_indices[m0];
  return (g < 0 || g >= p.groups) ? -1 : g;
}

__device__ __forceinline__ v8i frag(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

// Epilogue shared by the kernels.  Lane l holds, for sub-tile (i, j), output row
// row0 + 16i + (l & 15) and the four columns col0 + 16j + 4(l >> 4) + 0..3.
// Without a K split the values go straight to bf16.  With a split every workgroup
// stores its fp32 partial to the workspace and splitk_reduce_kernel finishes.
template <int SM, int SN>
__device__ __forceinline__ void store_tile(const float (&acc)[SM][SN][4], const KArgs& p, uint16_t* __restrict__ C,
                                           int64_t row0, int64_t col0, int64_t m_limit, int split, int tile,
                                           int lane, int tid) {
  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = row0 + 16 * i + (lane & 15);
      if (m >= m_limit) continue;
#pragma unroll
      for (int j = 0; j < SN; ++j) {
        const int64_t n = col0 + 16 * j + 4 * (lane >> 4);
        if (n < p.N) {
          uint2 o;
          o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
          o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
          *reinterpret_cast<uint2*>(C + m * p.ldc + n) = o;
        }
      }
    }
    return;
  }
  // Split K: publish this split's scaled fp32 partial; a second kernel on the same
  // stream adds the partials in split order and writes bf16 (the kernel boundary
  // makes the partials visible, so no fence, atomic or counter is needed here).
  const size_t slice = (size_t)p.M * (size_t)p.N;
  float* __restrict__ ws = p.ws;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int64_t m = row0 + 16 * i + (lane & 15);
    if (m >= m_limit) continue;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = col0 + 16 * j + 4 * (lane >> 4);
      if (n < p.N)
        *reinterpret_cast<float4*>(ws + (size_t)split * slice + (size_t)m * p.N + n) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
  (void)tile;
  (void)tid;
}

// Split-K reduction: thread t owns 8 consecutive columns of one row, adds the
// partials of every split in split order (deterministic), and stores 8 bf16.
// The loads of eight splits are issued before any is added.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ ws, int splits, int64_t M,
                                                            int64_t N, uint16_t* __restrict__ C, int64_t ldc) {
  const int64_t per_row = N / 8;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * per_row) return;
  const int64_t m = idx / per_row, n = (idx - m * per_row) * 8;
  const size_t slice = (size_t)M * (size_t)N;
  const float* src = ws + (size_t)m * N + n;
  float t[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int sp0 = 0; sp0 < splits; sp0 += 8) {
    float4 v[8][2];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int sp = (sp0 + u < splits) ? sp0 + u : sp0;
      v[u][0] = *reinterpret_cast<const float4*>(src + (size_t)sp * slice);
      v[u][1] = *reinterpret_cast<const float4*>(src + (size_t)sp * slice + 4);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      if (sp0 + u < splits) {
        t[0] += v[u][0].x; t[1] += v[u][0].y; t[2] += v[u][0].z; t[3] += v[u][0].w;
        t[4] += v[u][1].x; t[5] += v[u][1].y; t[6] += v[u][1].z; t[7] += v[u][1].w;
      }
    }
  }
  uint4 o;
  o.x = bf16_rne(t[0]) | (bf16_rne(t[1]) << 16);
  o.y = bf16_rne(t[2]) | (bf16_rne(t[3]) << 16);
  o.z = bf16_rne(t[4]) | (bf16_rne(t[5]) << 16);
  o.w = bf16_rne(t[6]) | (bf16_rne(t[7]) << 16);
  *reinterpret_cast<uint4*>(C + m * ldc + n) = o;
}

// FS: the float-scale format (activation scales fp32 [K/128][ld_sfa], weight scales
// any fp32): the MFMA runs unscaled and the two scales multiply its result.
template <int BM, int BN, int WM, int WN, bool FS = false>
__global__ __launch_bounds__(256) void gemm_kernel(const KArgs p) {
  constexpr int NWN = BN / WN;
  constexpr int SM = WM / 16, SN = WN / 16;
  constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;  // 16-byte chunks per thread
  static_assert((BM / WM) * (BN / WN) == 4, "four wavefronts per workgroup");
  static_assert((BM * 8) % 256 == 0 && (BN * 8) % 256 == 0, "tile rows must fill the loaders");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int wm = wave / NWN, wn = wave % NWN;
  const int64_t e = blockIdx.z;
  const int split = blockIdx.y;
  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;

  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  if (m0 >= m_limit) return;  // whole tile past the mask: no loads, no MFMA
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;

  const uint8_t* __restrict__ A = p.a + e * p.sa_e;
  const uint32_t* __restrict__ SA = p.sfa + e * p.ssfa_e;
  const uint8_t* __restrict__ B = p.b + eb * p.sb_e;
  const float* __restrict__ SB = p.sfb + eb * p.ssfb_e;
  uint16_t* __restrict__ C = p.c + e * p.sc_e;
  const int KB = (int)(p.K / 128);
  const int kb0 = split * p.kb_per_split;
  const int kb1 = (kb0 + p.kb_per_split < KB) ? kb0 + p.kb_per_split : KB;

  // sub-tiles of this wavefront that hold at least one valid row
  const int64_t wrow0 = m0 + wm * WM;
  int sm_live = 0;
#pragma unroll
  for (int i = 0; i < SM; ++i) sm_live += (wrow0 + 16 * i < m_limit) ? 1 : 0;

  uint4 ra[CA], rb[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) ra[i] = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int i = 0; i < CB; ++i) rb[i] = make_uint4(0u, 0u, 0u, 0u);

  auto gload = [&](int kb) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      const int64_t m = m0 + row;
      if (m < m_limit) ra[i] = *reinterpret_cast<const uint4*>(A + m * p.K + (int64_t)kb * 128 + ch * 16);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      const int64_t n = n0 + row;
      if (n < p.N) rb[i] = *reinterpret_cast<const uint4*>(B + n * p.K + (int64_t)kb * 128 + ch * 16);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      *reinterpret_cast<uint4*>(&lds[buf][row * LDS_ROW + ch * 16]) = ra[i];
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int cidx = tid + 256 * i, row = cidx >> 3, ch = cidx & 7;
      *reinterpret_cast<uint4*>(&lds[buf][(BM + row) * LDS_ROW + ch * 16]) = rb[i];
    }
  };

  float acc[SM][SN][4];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  if (kb0 < kb1) {  // an empty split range loads nothing and publishes zeros
    gload(kb0);
    lstore(0);
  }
  __syncthreads();
  int buf = 0;
  for (int kb = kb0; kb < kb1; ++kb) {
    const bool more = kb + 1 < kb1;
    if (more) gload(kb + 1);

    float sa[SM], sb[SN];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = wrow0 + 16 * i + (lane & 15);
      if constexpr (FS) {
        sa[i] = (m < m_limit) ? p.sfa_f[(int64_t)kb * p.ld_sfa + m] : 0.0f;
      } else {
        const uint32_t wd = (m < m_limit) ? SA[(int64_t)(kb >> 2) * p.ld_sfa + m] : 0u;
        sa[i] = __uint_as_float(((wd >> (8 * (kb & 3))) & 0xFFu) << 23);
      }
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = n0 + wn * WN + 16 * j;
      // UE8M0 entries read a weight block scale's exponent field only (its power of
      // two), as the scaled-MFMA kernels do; float-scale entries take the whole value
      const float s = (n < p.N) ? SB[(n >> 7) * KB + kb] : 0.0f;
      sb[j] = FS ? s : __uint_as_float(__float_as_uint(s) & 0x7F800000u);
    }

    const uint8_t* As = lds[buf];
    const uint8_t* Bs = lds[buf] + BM * LDS_ROW;
    v8i bfr[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j) bfr[j] = frag(Bs + (wn * WN + 16 * j + (lane & 15)) * LDS_ROW + (lane >> 4) * 32);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      if (i < sm_live) {
        const v8i af = frag(As + (wm * WM + 16 * i + (lane & 15)) * LDS_ROW + (lane >> 4) * 32);
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bfr[j], af, zero, 0, 0, 0, 0, 0, 0);
          const float s = sa[i] * sb[j];
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(d[r], s, acc[i][j][r]);
        }
      }
    }
    if (more) lstore(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  store_tile<SM, SN>(acc, p, C, wrow0, n0 + wn * WN, m_limit, split, tile, lane, tid);
}

// ---------------------------------------------------------------------------
// Weight-streaming kernel for few rows per group (decode-sized M, masked MoE
// experts).  Every weight byte is used by exactly one wavefront, so B skips LDS:
// each lane loads its MFMA operand bytes straight from global memory into
// registers, DEPTH K-blocks ahead of use (a register ring), which keeps enough
// bytes in flight to stream HBM.  The few activation rows are shared by the four
// wavefronts through an LDS double buffer, fed from the same ring.  Wavefront w
// owns WSN 16-column sub-tiles; all MS 16-row sub-tiles of the tile are computed
// by every wavefront (sub-tiles past the mask are skipped).
//
// All global loads are buffer loads whose descriptor covers exactly the valid
// rows of the tile (and of the wavefront's columns): rows past the mask, columns
// past N and K-blocks past the split are given an offset outside the range, so
// the hardware returns zeros without touching memory and without a branch.  With
// no divergent branches around loads, the compiler's wait counts track the ring
// exactly instead of draining it.  The activation-scale words and weight block
// scales a workgroup needs for its K range are copied into LDS once, up front.
//
// Operand byte order: lane l carries bytes [16(l>>4), +16) and [64 + 16(l>>4), +16)
// of its row's K-block, for A and B alike (the MFMA pairs A and B bytes by
// position, so any order shared by both operands gives the same dot product);
// each 16-lane row of a load then touches 64 contiguous bytes of one matrix row.
template <int MS, int WSN, int DEPTH>
__global__ __launch_bounds__(256) void stream_kernel(const KArgs p) {
  constexpr int BM = MS * 16, BN = 4 * WSN * 16;
  constexpr int ACH = BM * 8;                 // 16-byte chunks in one A K-block tile
  constexpr int CA = (ACH + 255) / 256;       // chunks per thread
  constexpr int NBW = (BN + 127) / 128;       // weight-scale blocks a tile can span
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  const int64_t e = blockIdx.z;
  const int split = blockIdx.y;
  const int tile = blockIdx.x;
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;

  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= m_limit) return;  // whole tile past the mask: no loads, no MFMA
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;
  const int64_t n0 = (int64_t)tn * BN;
  const int64_t nw0 = n0 + wave * (WSN * 16);  // this wavefront's first column

  const int KB = (int)(p.K / 128);
  const int per = p.kb_per_split;
  const int kb0 = split * per;
  const int kb1 = (kb0 + per < KB) ? kb0 + per : KB;
  const int w0 = kb0 >> 2;
  const int nwords = (kb1 > kb0) ? ((kb1 - 1) >> 2) - w0 + 1 : 0;
  const int nb0 = (int)(n0 >> 7);
  const int NB = (int)((p.N + 127) / 128);
  const int Wd = (KB + 3) / 4;

  uint8_t* lds_a = smem;                                              // [2][BM * LDS_ROW]
  uint32_t* lds_sa = reinterpret_cast<uint32_t*>(smem + 2 * BM * LDS_ROW);  // [sa_words][BM]
  float* lds_sb = reinterpret_cast<float*>(lds_sa + p.sa_words * BM);       // [NBW][per]

  const int64_t rows_valid = (m_limit - m0 < BM) ? m_limit - m0 : BM;
  int64_t cols_valid = p.N - nw0;
  cols_valid = cols_valid < 0 ? 0 : (cols_valid > WSN * 16 ? WSN * 16 : cols_valid);
  const auto rA = make_rsrc(p.a + e * p.sa_e + m0 * p.K, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + eb * p.sb_e + (cols_valid > 0 ? nw0 : 0) * p.K, (uint32_t)(cols_valid * p.K));
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + eb * p.ssfb_e, (uint32_t)(NB * KB * 4));
  uint16_t* __restrict__ C = p.c + e * p.sc_e;

  uint4 ar[DEPTH][CA];
  v8i br[DEPTH][WSN];
  auto issue = [&](int d, int kb) {
    const bool in = kb < kb1;
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int cidx = tid + 256 * c;
      const uint32_t off = (in && cidx < ACH) ? (uint32_t)((cidx >> 3) * p.K + kb * 128 + (cidx & 7) * 16) : kOOB;
      ar[d][c] = bload16(rA, off);
    }
#pragma unroll
    for (int j = 0; j < WSN; ++j) {
      const uint32_t off = in ? (uint32_t)((16 * j + (lane & 15)) * p.K + kb * 128 + (lane >> 4) * 16) : kOOB;
      const uint4 lo = bload16(rB, off);
      const uint4 hi = bload16(rB, off + 64);
      br[d][j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
  };
  auto astore = [&](int d, int stage) {
#pragma unroll
    for (int c = 0; c < CA; ++c) {
      const int cidx = tid + 256 * c;
      if (cidx < ACH)
        *reinterpret_cast<uint4*>(&lds_a[stage * BM * LDS_ROW + (cidx >> 3) * LDS_ROW + (cidx & 7) * 16]) = ar[d][c];
    }
  };

  // prologue: fill the ring, then the scale tables (one latency for both)
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(d, kb0 + d);
  for (int idx = tid; idx < nwords * BM; idx += 256) {
    const int wl = idx / BM, row = idx - wl * BM;
    const int64_t m = m0 + row;
    const uint32_t off = (m < m_limit) ? (uint32_t)(((int64_t)(w0 + wl) * p.ld_sfa + m) * 4) : kOOB;
    lds_sa[wl * BM + row] = bload4(rSA, off);
  }
  for (int idx = tid; idx < NBW * per; idx += 256) {
    const int b = idx / per, kk = idx - b * per;
    const int k = kb0 + kk, nb = nb0 + b;
    const uint32_t off = (k < kb1 && nb < NB) ? (uint32_t)((nb * KB + k) * 4) : kOOB;
    lds_sb[b * per + kk] = __uint_as_float(bload4(rSB, off) & 0x7F800000u);  // exponent field only (UE8M0)
  }
  astore(0, 0);
  __syncthreads();

  float acc[MS][WSN][4];
#pragma unroll
  for (int i = 0; i < MS; ++i)
#pragma unroll
    for (int j = 0; j < WSN; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

  // Straight-line body: whole groups of DEPTH K-blocks.  Steps past kb1 multiply
  // zeros (their loads were out of range) and get a zero scale, so they add nothing.
  const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int kb = kb0; kb < kb1; kb += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      const int k = kb + d;
      const bool live = k < kb1;
      const int kk = live ? k - kb0 : 0;
      const int stage = (k - kb0) & 1;
      const uint8_t* As = lds_a + stage * BM * LDS_ROW;
      float sb[WSN];
#pragma unroll
      for (int j = 0; j < WSN; ++j) {
        const float v = lds_sb[(int)(((nw0 + 16 * j) >> 7) - nb0) * per + kk];
        sb[j] = live ? v : 0.0f;
      }
      const uint32_t* saw = lds_sa + (((kb0 + kk) >> 2) - w0) * BM + (lane & 15);
      const int sh = 8 * ((kb0 + kk) & 3);
#pragma unroll
      for (int i = 0; i < MS; ++i) {
        const uint8_t* pa = As + (16 * i + (lane & 15)) * LDS_ROW + (lane >> 4) * 16;
        const uint4 lo = *reinterpret_cast<const uint4*>(pa);
        const uint4 hi = *reinterpret_cast<const uint4*>(pa + 64);
        const v8i af = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        const float sa = __uint_as_float(((saw[16 * i] >> sh) & 0xFFu) << 23);
#pragma unroll
        for (int j = 0; j < WSN; ++j) {
          const v4f r = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(br[d][j], af, zero, 0, 0, 0, 0, 0, 0);
          const float sc = sa * sb[j];
#pragma unroll
          for (int q = 0; q < 4; ++q) acc[i][j][q] = __builtin_fmaf(r[q], sc, acc[i][j][q]);
        }
      }
      // stage the next K-block's activations, then refill this ring slot
      astore((d + 1) % DEPTH, stage ^ 1);
      issue(d, k + DEPTH);
      __syncthreads();
    }
  }

  store_tile<MS, WSN>(acc, p, C, m0, nw0, m_limit, split, tile, lane, tid);
}

// ---------------------------------------------------------------------------
// Scaled-MFMA tile kernel (prefill-sized M).
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 computes C + 2^(ea + eb) * sum(a*b)
// with E8M0 exponents ea, eb taken from a byte of a scale register (selected by an
// immediate), which is exactly the per-K-block scale-then-accumulate of the
// method: one instruction covers one 128-wide K-block, the packed activation word
// (four groups per uint32) is the scale register of the activation operand with
// the byte picked by kb % 4, and the weight block's exponent (the UE8M0 value of
// its power-of-two scale) is the other.  The fp32 accumulator therefore stays in
// the MFMA C operand and no VALU work is spent on scales.
//
// Tiles move global -> LDS by LDS-DMA (buffer loads with the lds flag): each
// wavefront instruction writes 1 KiB = 8 rows of a K-block tile, lane l to byte
// 16 l, so the tile is stored row-major without padding and the 16-byte chunks of
// row r are XOR-swizzled (chunk c in slot c ^ (r & 7)) for conflict-free operand
// reads.  Two LDS stages: after the barrier that opens step kb, the DMA of kb + 1
// goes into the stage kb - 1 used.  Rows past M (or past an
// expert's count) and K-blocks past the range fall outside the buffer
// descriptors and arrive as zeros.  Workgroups are mapped to tiles XCD by XCD
// (a workgroup's XCD is its linear id mod 8), each XCD taking a compact block of
// tiles so that its L2 serves the shared A and B panels.
// Chunk swizzle of a 128-byte tile row: slot = chunk ^ (row & 7).  Measured on
// gfx950 with SQ_LDS_BANK_CONFLICT for the MFMA operand read pattern (lane l: row
// l & 15, chunks l >> 4 and 4 + (l >> 4)): no conflicts, where unswizzled rows or
// 144-byte padded rows cost 4-12 conflict cycles per ds_read_b128.
__device__ __forceinline__ int swz(int r) { return r & 7; }

template <int V>
struct IntC {
  static constexpr int value = V;
};

// FS: the float-scale format.  The tables then hold one fp32 per K-block (activations
// [K-block][row], weights [column block][K-block]), each MFMA runs with unit scales on
// zero, and acc += product * (s_a * s_b).
template <int BM, int BN, int WGM, int WGN, int STAGES, bool FS = false>
__global__ __launch_bounds__(WGM * WGN * 64) void scaled_tile_kernel(const KArgs p) {
  constexpr int NW = WGM * WGN;  // wavefronts per workgroup (4 or 8)
  constexpr int NT = NW * 64;
  constexpr int WM = BM / WGM, WN = BN / WGN;
  constexpr int SM = WM / 16, SN = WN / 16;
  constexpr int A_INST = BM / 8, B_INST = BN / 8;          // 1 KiB DMA instructions per stage
  constexpr int IPW = (A_INST + B_INST) / NW;              // per wavefront
  constexpr int STAGE = (BM + BN) * 128;
  static_assert((NW == 4 || NW == 8) && (A_INST + B_INST) % NW == 0, "tile shape");
  static_assert(STAGES == 2, "two LDS stages; see the step schedule below");
  // One LDS array per ring stage, indexed with compile-time stage numbers, so the
  // compiler can tell operand reads of one stage from DMA writes into another and
  // does not make every read wait for all loads in flight.
  __shared__ __attribute__((aligned(1024))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[STAGE];
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];  // scale tables

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t e = blockIdx.z;

  // XCD-aware tile order: workgroup id -> (XCD, slot) -> a compact run of tiles per
  // XCD, walked in groups of GM tile rows.
  const int T = p.tiles_m * p.tiles_n;
  const int bid = blockIdx.x;
  const int per_xcd = (T + 7) / 8;
  int lin = (bid & 7) * per_xcd + (bid >> 3);
  if ((T & 7) != 0) lin = bid;  // uneven split: plain order
  constexpr int GM = 4;
  const int group = lin / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gsz = (p.tiles_m - first_m) < GM ? (p.tiles_m - first_m) : GM;
  const int in_g = lin - group * GM * p.tiles_n;
  const int tm = first_m + in_g % gsz, tn = in_g / gsz;

  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  if (m0 >= m_limit) return;
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;

  const int KB = (int)(p.K / 128);
  const int Wd = (KB + 3) / 4;
  const int NB = (int)((p.N + 127) / 128);
  constexpr int NBT = (BN + 127) / 128;
  const int TW = FS ? KB : Wd;                          // table columns: K-blocks or words
  uint32_t* lds_sa = reinterpret_cast<uint32_t*>(smem);  // [TW][BM] activation words / fp32 scales
  uint32_t* lds_sb = lds_sa + TW * BM;                  // [NBT][TW] packed weight exponents / fp32 scales

  const int64_t rows_valid = (m_limit - m0 < BM) ? m_limit - m0 : BM;
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > BN ? BN : cols_valid;
  const auto rA = make_rsrc(p.a + e * p.sa_e + m0 * p.K, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + eb * p.sb_e + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + eb * p.ssfb_e, (uint32_t)(NB * KB * 4));

  auto stage_ptr = [&](auto st_tag) -> uint8_t* {
    constexpr int S = decltype(st_tag)::value;
    if constexpr (S == 0) return st0;
    else return st1;
  };
  // DMA of K-block kb into a stage: instruction t of wavefront w covers rows
  // 8*i..8*i+7 of A (i < A_INST) or of B (i - A_INST), lane l -> row 8i + l/8,
  // LDS slot l % 8 holding chunk (l % 8) ^ swz(row).
  auto issue = [&](int kb, auto st_tag) {
    uint8_t* base = stage_ptr(st_tag);
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const int inst = wave * IPW + t;
      const bool isA = inst < A_INST;
      const int ri = isA ? inst : inst - A_INST;
      const int r = ri * 8 + (lane >> 3);
      const int chunk = (lane & 7) ^ swz(r);
      const uint32_t off = (kb < KB) ? (uint32_t)(r * p.K + kb * 128 + chunk * 16) : kOOB;
      uint8_t* dst = base + (isA ? 0 : BM * 128) + ri * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rA : rB, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  // scale tables: activation words for this tile's rows, weight exponents packed
  // four K-blocks to a word (byte kb % 4), matching the MFMA's byte select (float
  // scales: the fp32 values per K-block)
  if constexpr (FS) {
    const auto rSAF = make_rsrc(p.sfa_f + e * p.ssfa_e, (uint32_t)(KB * p.ld_sfa * 4));
    for (int idx = tid; idx < KB * BM; idx += NT) {
      const int k = idx / BM, row = idx - k * BM;
      const int64_t m = m0 + row;
      lds_sa[idx] = bload4(rSAF, (m < m_limit) ? (uint32_t)(((int64_t)k * p.ld_sfa + m) * 4) : kOOB);
    }
    for (int idx = tid; idx < NBT * KB; idx += NT) {
      const int b = idx / KB, k = idx - b * KB;
      const int nb = (int)(n0 >> 7) + b;
      lds_sb[idx] = bload4(rSB, nb < NB ? (uint32_t)((nb * KB + k) * 4) : kOOB);
    }
  } else {
  for (int idx = tid; idx < Wd * BM; idx += NT) {
    const int w = idx / BM, row = idx - w * BM;
    const int64_t m = m0 + row;
    const uint32_t off = (m < m_limit) ? (uint32_t)(((int64_t)w * p.ld_sfa + m) * 4) : kOOB;
    lds_sa[idx] = bload4(rSA, off);
  }
  for (int idx = tid; idx < NBT * Wd; idx += NT) {
    const int b = idx / Wd, w = idx - b * Wd;
    const int nb = (int)(n0 >> 7) + b;
    uint32_t word = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int k = 4 * w + q;
      const uint32_t off = (nb < NB && k < KB) ? (uint32_t)((nb * KB + k) * 4) : kOOB;
      word |= ((bload4(rSB, off) >> 23) & 0xFFu) << (8 * q);
    }
    lds_sb[idx] = word;
  }
  }
  issue(0, IntC<0>{});

  // accumulators: [SM][SN] 16x16 sub-tiles, lane holds row 16i + (l & 15) and
  // columns 16j + 4(l >> 4) + 0..3 (the weight tile is the MFMA's first operand)
  v4f acc[SM][SN];
#pragma unroll
  for (int i = 0; i < SM; ++i)
#pragma unroll
    for (int j = 0; j < SN; ++j) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

  // One K-block: OPS = kb % 4 (scale byte), ST = kb % 2 (its stage).
  auto step = [&](int kb, auto ops_tag, auto st_tag) {
    constexpr int OPS = decltype(ops_tag)::value;
    constexpr int ST = decltype(st_tag)::value;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wavefront's DMA of kb has landed
    __syncthreads();                     // ... and everyone's; kb - 1's stage is free
    const uint8_t* As = stage_ptr(st_tag);
    const uint8_t* Bs = As + BM * 128;
    const int w = FS ? kb : kb >> 2;
    uint32_t sa[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) sa[i] = lds_sa[w * BM + wm * WM + 16 * i + (lane & 15)];
    uint32_t sbw[SN];
#pragma unroll
    for (int j = 0; j < SN; ++j) sbw[j] = lds_sb[((wn * WN + 16 * j) >> 7) * TW + w];
    v8i af[SM], bf[SN];
    const int c0 = (lane >> 4), c1 = 4 + (lane >> 4);
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int r = wm * WM + 16 * i + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(As + r * 128 + ((c0 ^ swz(r)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(As + r * 128 + ((c1 ^ swz(r)) << 4));
      af[i] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int r = wn * WN + 16 * j + (lane & 15);
      const uint4 lo = *reinterpret_cast<const uint4*>(Bs + r * 128 + ((c0 ^ swz(r)) << 4));
      const uint4 hi = *reinterpret_cast<const uint4*>(Bs + r * 128 + ((c1 ^ swz(r)) << 4));
      bf[j] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
    }
    // Keep the DMA below the operand reads: the compiler would hoist it above them
    // (the buffers differ) and then make the reads wait for it.
    __builtin_amdgcn_sched_barrier(0);
    issue(kb + 1, IntC<1 - ST>{});
    if constexpr (FS) {
      const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int i = 0; i < SM; ++i) {
          const v4f d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], zero, 0, 0, 0, 127, 0, 127);
          const float sc = __uint_as_float(sa[i]) * __uint_as_float(sbw[j]);
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[i][j][r] = __builtin_fmaf(d[r], sc, acc[i][j][r]);
        }
    } else {
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int i = 0; i < SM; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(bf[j], af[i], acc[i][j], 0, 0, OPS,
                                                                       (int)sbw[j], OPS, (int)sa[i]);
    }
  };

  // K loop unrolled by four: the scale byte (kb % 4) and the ring stage are static
  for (int kb = 0; kb < KB; kb += 4) {
    step(kb, IntC<0>{}, IntC<0>{});
    if (kb + 1 < KB) step(kb + 1, IntC<1>{}, IntC<1 % STAGES>{});
    if (kb + 2 < KB) step(kb + 2, IntC<2>{}, IntC<2 % STAGES>{});
    if (kb + 3 < KB) step(kb + 3, IntC<3>{}, IntC<3 % STAGES>{});
  }

  // epilogue straight from the accumulators (this kernel never splits K)
  uint16_t* __restrict__ C = p.c + e * p.sc_e;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int64_t m = m0 + wm * WM + 16 * i + (lane & 15);
    if (m >= m_limit) continue;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = n0 + wn * WN + 16 * j + 4 * (lane >> 4);
      if (n < p.N) {
        uint2 o;
        o.x = bf16_rne(acc[i][j][0]) | (bf16_rne(acc[i][j][1]) << 16);
        o.y = bf16_rne(acc[i][j][2]) | (bf16_rne(acc[i][j][3]) << 16);
        *reinterpret_cast<uint2*>(C + m * p.ldc + n) = o;
      }
    }
  }
}

inline size_t scaled_tile_lds_bytes(int bm, int bn, int stages, int K, bool float_scales = false) {
  // dynamic part only (the stage buffers are static): the two scale tables, one word
  // per four K-blocks (packed UE8M0) or one fp32 per K-block (float scales)
  (void)stages;
  const int KB = K / 128, Wd = float_scales ? KB : (KB + 3) / 4;
  return (size_t)Wd * bm * 4 + (size_t)((bn + 127) / 128) * Wd * 4;
}

inline size_t scaled_tile_static_bytes(int bm, int bn, int stages) {
  return (size_t)(stages > 2 ? 4 : 2) * (bm + bn) * 128 + (stages > 2 ? 0 : 32);
}

// ---------------------------------------------------------------------------
// Ring kernel.  Four wavefronts in a WGM x WGN grid, each owning a (BM/WGM) x
// (BN/WGN) sub-tile accumulated with v_mfma_scale_f32_32x32x64_f8f6f4.  One such
// MFMA covers half of a 128-wide K-block, so the LDS ring is kept in K-halves:
// four slots of (BM + BN) rows x 64 bytes, filled by LDS-DMA three half-steps
// before they are read.  Half-step h of every wavefront:
//   s_waitcnt: its own DMA of h + 1 has landed and its reads of h have returned;
//   barrier:   so has everyone's, and nobody reads slot h any more;
//   the MFMAs of h from registers, interleaved with the LDS reads of the
//   operands of h + 1 and with the DMA of h + 4 into slot h.
// LDS reads and DMA thus run under the MFMAs.  The UE8M0 exponents are the
// MFMA's scale operands (byte kb % 4 of the packed words), so the block scaling
// costs no VALU work; the activation words of the tile's rows and the packed
// weight exponents are staged in LDS tables once per tile.  The K loop runs in
// groups of four K-blocks; a ragged last group reads zeros (out-of-range DMA)
// with zero scale bytes.
//
// Valid rows: each wavefront runs a copy of the loop specialised to the number
// IV of its 32-row groups that hold valid rows (all of them except in the last
// M tile or a masked group's partial tile) and issues neither operand reads nor
// MFMAs for the others; it still takes its share of the DMA and every barrier.
// In the 1 x 4 grid all four wavefronts share the same rows, so a masked group
// with few rows still spreads its MFMAs over the four SIMDs.
//
// LDS slot layout: A rows [0, BM) then B rows [BM, BM + BN), 64 bytes each
// (one K-half); 16-byte chunk c of row r sits at position c ^ ((r >> 2) & 3).
// Measured on gfx950 with SQ_LDS_BANK_CONFLICT for the operand reads (lane l:
// row l & 31, chunks 2(l >> 5) and 2(l >> 5) + 1): no conflicts with this
// swizzle or with (r >> 3) & 3, about 4 conflict cycles per ds_read_b128 with
// (r >> 1) & 3 and 12 without a swizzle.
__device__ __forceinline__ int swz64(int r) { return (r >> 2) & 3; }

typedef float v16f __attribute__((ext_vector_type(16)));
// one 16-byte LDS load per operand half: a vector type keeps it a single load
// of the slot array (a struct would be split into four), which is what lets the
// compiler see which slot it reads
typedef int v4i __attribute__((ext_vector_type(4)));

// s_waitcnt immediate (gfx9 encoding): vmcnt split over bits 3:0 and 15:14,
// expcnt (bits 6:4) left at its maximum.
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | ((lgkm & 15) << 8); }

constexpr int kRingSlots = 4;

template <int BM, int BN, int WGM, int WGN>
struct RingShape {
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int SM = WM / 32, SN = WN / 32;
  static constexpr int SLOT = (BM + BN) * 64;
  static constexpr int A_INST = BM / 16, B_INST = BN / 16;  // 1 KiB DMA instructions per slot
  static constexpr int IPA = A_INST / 4, IPB = B_INST / 4;  // ... per wavefront, of A and of B
  static constexpr int IPW = IPA + IPB;
  static constexpr int NBT = BN / 128;                      // weight blocks across the tile
  static constexpr int FIT = (160 * 1024 - kRingSlots * SLOT - 256) / (BM * 4 + NBT * 4);
  static constexpr int WD_MAX = FIT < 32 ? FIT : 32;        // scale words per row the tables hold
};

// XCD-aware tile order: workgroup id -> (XCD, slot) -> a compact run of tiles per
// XCD (a workgroup's XCD is its linear id mod 8), walked in groups of four tile rows.
__device__ __forceinline__ void xcd_tile(const KArgs& p, int bid, int& tm, int& tn) {
  const int T = p.tiles_m * p.tiles_n;
  const int per_xcd = (T + 7) / 8;
  int lin = (bid & 7) * per_xcd + (bid >> 3);
  if ((T & 7) != 0) lin = bid;  // uneven split: plain order
  constexpr int GM = 4;
  const int group = lin / (GM * p.tiles_n);
  const int first_m = group * GM;
  const int gsz = (p.tiles_m - first_m) < GM ? (p.tiles_m - first_m) : GM;
  const int in_g = lin - group * GM * p.tiles_n;
  tm = first_m + in_g % gsz;
  tn = in_g / gsz;
}

// Scheduling pattern for one half-step: NM MFMAs, each followed by its share of the
// NR operand reads and of the NV DMA instructions (spread evenly).
template <int NM, int NR, int NV, int Q = 0>
__device__ __forceinline__ void mfma_read_dma_pattern() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int r = (Q + 1) * NR / NM - Q * NR / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    constexpr int v = (Q + 1) * NV / NM - Q * NV / NM;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);
    mfma_read_dma_pattern<NM, NR, NV, Q + 1>();
  }
}

// The same with the operand reads front-loaded: two reads after each of the first
// MFMAs, so that the last read of the half-step is issued long before its end.
template <int NM, int NR, int NV, int Q = 0>
__device__ __forceinline__ void mfma_front_read_dma_pattern() {
  if constexpr (Q < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    constexpr int r0 = 2 * Q < NR ? 2 * Q : NR, r1 = 2 * (Q + 1) < NR ? 2 * (Q + 1) : NR;
    if constexpr (r1 > r0) __builtin_amdgcn_sched_group_barrier(0x100, r1 - r0, 0);
    constexpr int v = (Q + 1) * NV / NM - Q * NV / NM;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x010, v, 0);
    mfma_front_read_dma_pattern<NM, NR, NV, Q + 1>();
  }
}

template <int BM, int BN, int WGM, int WGN, bool SHUF = false, int RP = 0>
__global__ __launch_bounds__(256) void scaled_ring_kernel(const KArgs p) {
  using R = RingShape<BM, BN, WGM, WGN>;
  constexpr int S = kRingSlots;
  constexpr int WM = R::WM, WN = R::WN, SM = R::SM, SN = R::SN, IPW = R::IPW;
  constexpr int IPA = R::IPA, WD_MAX = R::WD_MAX, NBT = R::NBT;
  static_assert(WGM * WGN == 4 && WM % 32 == 0 && WN % 32 == 0 && BN % 128 == 0 && BM % 64 == 0, "ring tile shape");
  static_assert(WD_MAX >= 1, "scale tables do not fit");
  // one array per slot: the compiler's LDS-DMA tracking tells them apart, so an
  // operand read waits only for the DMA into its own slot
  __shared__ __attribute__((aligned(1024))) uint8_t sl0[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t sl1[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t sl2[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t sl3[R::SLOT];
  __shared__ __attribute__((aligned(16))) uint32_t sa_tab[WD_MAX * BM];   // [w][row]
  __shared__ __attribute__((aligned(16))) uint32_t sb_tab[NBT * WD_MAX];  // [block][w], byte kb % 4

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t e = blockIdx.z;
  int tm, tn;
  xcd_tile(p, blockIdx.x, tm, tn);

  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  if (m0 >= m_limit) return;
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;

  const int KB = (int)(p.K / 128);
  const int Wd = (KB + 3) / 4;  // <= WD_MAX (checked by the host)
  const int NB = (int)((p.N + 127) / 128);
  const int H = 8 * Wd;         // half-steps, K padded to whole groups of four blocks
  const int64_t rows_valid = (m_limit - m0 < BM) ? m_limit - m0 : BM;
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > BN ? BN : cols_valid;
  const auto rA = make_rsrc(p.a + e * p.sa_e + m0 * p.K, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + eb * p.sb_e + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + eb * p.ssfb_e, (uint32_t)(NB * KB * 4));

  auto slot = [&](auto sl_tag) -> uint8_t* {
    constexpr int I = decltype(sl_tag)::value;
    if constexpr (I == 0) return sl0;
    else if constexpr (I == 1) return sl1;
    else if constexpr (I == 2) return sl2;
    else return sl3;
  };

  // DMA: instruction t < IPA of this wavefront covers A rows 16 ri .. 16 ri + 15 with
  // ri = wave * IPA + t, the others B rows likewise; lane l -> row 16 ri + (l >> 2),
  // slot position l & 3 holding chunk (l & 3) ^ swz64(row) of the K-half.  The
  // swizzle of row 16 ri + (l >> 2) is ((l >> 4) & 3) for every ri, so one per-lane
  // offset serves all instructions (the row base is added per instruction, which
  // keeps eight registers free for the loop).
  const uint32_t lane_off = (uint32_t)((lane >> 2) * p.K) + (uint32_t)((((lane & 3) ^ ((lane >> 4) & 3)) << 4));
  // SHUF: weights in the pre-shuffled layout, where chunk c of a K-half of row r (of
  // 32-row group g) is 16-byte chunk 32 (c >> 1) + (r & 31) of load 2 hh + (c & 1) of
  // its K-block: the 16 rows x 4 chunks of one instruction are four contiguous 256-byte
  // runs.  Per lane: chunk c = (l & 3) ^ swizzle, row 16 ri + (l >> 2); per instruction:
  // group ri >> 1, half-group (ri & 1) * 256; per K-half h: K-block h >> 1, hh = h & 1.
  const int cB = (lane & 3) ^ ((lane >> 4) & 3);
  const uint32_t lane_off_b = SHUF ? (uint32_t)((cB & 1) * 1024 + (32 * (cB >> 1) + (lane >> 2)) * 16) : lane_off;
  auto issue = [&](int h, auto sl_tag) {
    uint8_t* base = slot(sl_tag);
    // past the last K-half the offset gets the top bit: out of range, zero-filled
    // (an OR rather than a select keeps the loop body free of branches)
    const uint32_t hoff = (uint32_t)h * 64u, oob = h < 2 * KB ? 0u : kOOB;
    const uint32_t hoff_b = SHUF ? (uint32_t)(h >> 1) * 4096u + (uint32_t)(h & 1) * 2048u : hoff;
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const bool isA = t < IPA;  // static after unrolling
      const int ri = isA ? wave * IPA + t : wave * R::IPB + (t - IPA);
      uint8_t* dst = base + (isA ? 0 : BM * 64) + ri * 1024;
      const uint32_t off =
          (isA || !SHUF) ? (lane_off + (uint32_t)(ri * 16 * p.K) + hoff) | oob
                         : (lane_off_b + (uint32_t)((ri >> 1) * KB * 4096 + (ri & 1) * 256) + hoff_b) | oob;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rA : rB, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)off, 0, 0, 0);
    }
  };

  // Scale tables.  Activation words: zero for rows past the mask and for the bytes
  // of K-blocks past K in the last word.  Weight exponents: byte kb % 4 of word
  // kb / 4, zero past N or K.  The global loads are issued before the first DMAs
  // and written to LDS after them, so the DMAs are in flight meanwhile.
  constexpr int SA_IT = (WD_MAX * BM + 255) / 256;
  constexpr int SB_IT = (NBT * WD_MAX * 4 + 255) / 256;
  uint32_t sav[SA_IT], sbv[SB_IT];
#pragma unroll
  for (int t = 0; t < SA_IT; ++t) {
    const int idx = t * 256 + tid;
    const int w = idx / BM, row = idx - w * BM;
    const bool ok = idx < WD_MAX * BM && w < Wd && m0 + row < m_limit;
    sav[t] = bload4(rSA, ok ? (uint32_t)(((int64_t)w * p.ld_sfa + m0 + row) * 4) : kOOB);
  }
#pragma unroll
  for (int t = 0; t < SB_IT; ++t) {
    const int idx = t * 256 + tid;
    const int b = idx / (WD_MAX * 4), k = idx - b * (WD_MAX * 4);
    const int nb = (int)(n0 >> 7) + b;
    const bool ok = idx < NBT * WD_MAX * 4 && nb < NB && k < KB;
    sbv[t] = bload4(rSB, ok ? (uint32_t)((nb * KB + k) * 4) : kOOB);
  }
  issue(0, IntC<0>{});
  issue(1, IntC<1>{});
  issue(2, IntC<2>{});
  issue(3, IntC<3>{});
#pragma unroll
  for (int t = 0; t < SA_IT; ++t) {
    const int idx = t * 256 + tid;
    const int w = idx / BM;
    uint32_t v = sav[t];
    const int left = KB - 4 * w;  // K-blocks of this word that exist
    if (left < 4) v &= left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
    if (idx < WD_MAX * BM) sa_tab[idx] = v;
  }
  uint8_t* sb_bytes = reinterpret_cast<uint8_t*>(sb_tab);
#pragma unroll
  for (int t = 0; t < SB_IT; ++t) {
    const int idx = t * 256 + tid;
    if (idx < NBT * WD_MAX * 4) sb_bytes[idx] = (uint8_t)((sbv[t] >> 23) & 0xFFu);
  }

  // first DMA and the tables in place everywhere
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((S - 1) * IPW, 0));
  __builtin_amdgcn_s_barrier();

  // operand reads: lane l takes row l & 31 of a 32-row group and the 32 bytes of
  // K-half chunks 2(l >> 5), 2(l >> 5) + 1 (the same k order for both operands)
  const int lr = lane & 31, c0 = 2 * (lane >> 5);
  const uint32_t rd0 = (uint32_t)(lr * 64 + ((c0 ^ swz64(lr)) << 4));
  const uint32_t rd1 = (uint32_t)(lr * 64 + (((c0 + 1) ^ swz64(lr)) << 4));
  const int sb_blk = (wn * WN) >> 7;  // this wavefront's weight block within the tile
  uint16_t* __restrict__ C = p.c + e * p.sc_e;

  // The loop and epilogue for IV valid 32-row groups of this wavefront.
  auto body = [&](auto iv_tag) {
    constexpr int IV = decltype(iv_tag)::value;
    auto read_frags = [&](auto sl_tag, v8i (&xf)[SM], v8i (&wf)[SN]) {
      const uint8_t* base = slot(sl_tag);
#pragma unroll
      for (int i = 0; i < IV; ++i) {
        const uint8_t* q = base + (wm * WM + 32 * i) * 64;
        const v4i lo = *reinterpret_cast<const v4i*>(q + rd0);
        const v4i hi = *reinterpret_cast<const v4i*>(q + rd1);
        xf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      if constexpr (IV > 0) {
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          const uint8_t* q = base + (BM + wn * WN + 32 * j) * 64;
          const v4i lo = *reinterpret_cast<const v4i*>(q + rd0);
          const v4i hi = *reinterpret_cast<const v4i*>(q + rd1);
          wf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
    };

    uint32_t sa[SM], sa_n[SM];
    uint32_t sb = sb_tab[sb_blk * WD_MAX], sb_n;
#pragma unroll
    for (int i = 0; i < SM; ++i) sa[i] = i < IV ? sa_tab[wm * WM + 32 * i + lr] : 0u;
    v8i xf[SM], wf[SN];
    read_frags(IntC<0>{}, xf, wf);

    v16f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;

    // half-step hb + HS of a group of four K-blocks (hb a multiple of 8): K-block
    // kb = hb / 2 + HS / 2, so the scale byte kb % 4 is HS / 2
    auto half = [&](int hb, auto hs_tag) {
      constexpr int HS = decltype(hs_tag)::value;
      constexpr int OPS = HS / 2;
      const int h = hb + HS;
      // nothing moves across the half-step boundary: the MFMAs below use registers
      // only, and would otherwise drift past later barriers
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((S - 2) * IPW, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(h + S, IntC<HS % S>{});
      if constexpr (HS == 0) {
#pragma unroll
        for (int i = 0; i < SM; ++i) sa[i] = sa_n[i];
        sb = sb_n;
      }
      if constexpr (HS == 4) {
        // scale words of the next group (clamped to the table; unused past the end)
        const int wnx = (hb >> 3) + 1 < WD_MAX ? (hb >> 3) + 1 : WD_MAX - 1;
#pragma unroll
        for (int i = 0; i < SM; ++i) sa_n[i] = i < IV ? sa_tab[wnx * BM + wm * WM + 32 * i + lr] : 0u;
        sb_n = sb_tab[sb_blk * WD_MAX + wnx];
      }
      v8i xn[SM], wnf[SN];
      read_frags(IntC<(HS + 1) % S>{}, xn, wnf);
#pragma unroll
      for (int i = 0; i < IV; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 0, 0, OPS, (int)sb,
                                                                      OPS, (int)sa[i]);
      // one operand read after every MFMA (two at the start while there are more
      // reads than MFMAs) and the DMA spread over the half-step: a DMA that waits
      // for room in the memory queue then stalls this wavefront's issue while an
      // MFMA runs, rather than holding back the first MFMA
      if constexpr (RP == 1) mfma_front_read_dma_pattern<IV * SN, 2 * (IV > 0 ? IV + SN : 0), IPW>();
      else mfma_read_dma_pattern<IV * SN, 2 * (IV > 0 ? IV + SN : 0), IPW>();
#pragma unroll
      for (int i = 0; i < IV; ++i) xf[i] = xn[i];
#pragma unroll
      for (int j = 0; j < SN; ++j) wf[j] = wnf[j];
    };

    // the first group's scale words were read above; sa_n / sb_n feed HS == 0
#pragma unroll
    for (int i = 0; i < SM; ++i) sa_n[i] = sa[i];
    sb_n = sb;
    for (int hb = 0; hb < H; hb += 8) {
      half(hb, IntC<0>{});
      half(hb, IntC<1>{});
      half(hb, IntC<2>{});
      half(hb, IntC<3>{});
      half(hb, IntC<4>{});
      half(hb, IntC<5>{});
      half(hb, IntC<6>{});
      half(hb, IntC<7>{});
    }
    // the DMAs issued past the end (out of range, zero-filled) must land, and every
    // wavefront must be done with the slots, before they are reused below
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    if constexpr (IV == 0) return;

    // Epilogue through LDS.  Lane l holds, for sub-tile (i, j), row 32 i + (l & 31)
    // and the columns 32 j + 8 q + 4 (l >> 5) + 0..3, q = 0..3 (registers 4q..4q+3):
    // 16-byte pieces scattered over 32 rows per store.  Each wavefront instead
    // writes its bf16 sub-tile to its own LDS slot (rows of WN * 2 bytes, 16-byte
    // chunk c of row r at position c ^ (r % CPR)) and stores it back row by row,
    // 16 bytes per lane, so every store instruction writes whole contiguous rows.
    constexpr int RB = WN * 2, CPR = RB / 16, RPI = 64 / CPR;  // row bytes, chunks per row, rows per store
    static_assert(WM * RB <= R::SLOT, "staging needs one slot per wavefront");
    uint8_t* stg = wave == 0 ? sl0 : wave == 1 ? sl1 : wave == 2 ? sl2 : sl3;
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int row = 32 * i + lr;
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int chunk = 4 * j + q;
          uint2 o;
          o.x = bf16_rne(acc[i][j][4 * q]) | (bf16_rne(acc[i][j][4 * q + 1]) << 16);
          o.y = bf16_rne(acc[i][j][4 * q + 2]) | (bf16_rne(acc[i][j][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(stg + row * RB + ((chunk ^ (row % CPR)) << 4) + 8 * (lane >> 5)) = o;
        }
    }
    // (a wavefront reads back only what it wrote itself: LDS operations of one
    // wavefront complete in order, so no barrier is needed; rows of the groups
    // past IV are past the valid rows and are not stored)
    const int c = lane % CPR;
    const int64_t n = n0 + wn * WN + 8 * c;
#pragma unroll
    for (int t = 0; t < (IV * 32) / RPI; ++t) {
      const int row = t * RPI + lane / CPR;
      const v4i v = *reinterpret_cast<const v4i*>(stg + row * RB + ((c ^ (row % CPR)) << 4));
      const int64_t m = m0 + wm * WM + row;
      if (m < m_limit && n < p.N) *reinterpret_cast<v4i*>(C + m * p.ldc + n) = v;
    }
  };

  // valid 32-row groups of this wavefront (uniform across the wavefront)
  int64_t mine = m_limit - (m0 + wm * WM);
  mine = mine < 0 ? 0 : (mine > WM ? WM : mine);
  const int iv = __builtin_amdgcn_readfirstlane((int)((mine + 31) / 32));
  switch (iv) {
    case 0: body(IntC<0>{}); break;
    case 1: body(IntC<1>{}); break;
    case 2: if constexpr (SM >= 2) body(IntC<2 <= SM ? 2 : SM>{}); break;
    case 3: if constexpr (SM >= 3) body(IntC<3 <= SM ? 3 : SM>{}); break;
    case 4: if constexpr (SM >= 4) body(IntC<4 <= SM ? 4 : SM>{}); break;
    case 5: if constexpr (SM >= 5) body(IntC<5 <= SM ? 5 : SM>{}); break;
    case 6: if constexpr (SM >= 6) body(IntC<6 <= SM ? 6 : SM>{}); break;
    case 7: if constexpr (SM >= 7) body(IntC<7 <= SM ? 7 : SM>{}); break;
    default: if constexpr (SM >= 8) body(IntC<8 <= SM ? 8 : SM>{}); break;
  }
}

template <int BM, int BN, int WGM, int WGN>
constexpr int ring_wd_max() { return RingShape<BM, BN, WGM, WGN>::WD_MAX; }

// ---------------------------------------------------------------------------
// Full-row ring kernel.  The same tile, wavefront grid, scaled MFMA and scale
// tables as the ring kernel above, but the LDS stages hold whole 128-wide
// K-blocks, so each LDS-DMA instruction of a wavefront moves 8 rows x 128 bytes:
// every 128-byte line of A and B is fetched from L2 by one request.  (A stage of
// K-halves, 16 rows x 64 bytes per instruction, requests each line twice; at
// 4096 x 4096 x 7168 that put 1.75x the lines through the L1-to-L2 path and kept the
// texture units busy ~68% of the time.)  16-byte chunk c of a row r sits at
// position c ^ ((r >> 1) & 7): sixteen consecutive rows (two per 256-byte cycle of
// the banks) then cover all 64 banks four bytes at a time, so the operand reads,
// which take one row per lane, are conflict-free (c ^ (r & 7) left rows r and
// r + 8 on the same banks: 7.7e6 conflict cycles at 4096 x 4096 x 7168).  With S stages, K-block j:
//   half 0: the MFMAs of j's first K-half (operands read during the previous
//           half), interleaved with the operand reads of j's second K-half;
//   half 1: wait for this wavefront's DMA of j + 1 and its reads, barrier (every
//           wavefront's DMA of j + 1 has landed and nobody reads j's stage any
//           more), DMA of j + S into j's stage, then the MFMAs of j's second half
//           interleaved with the operand reads of j + 1's first half and the DMA.
// One barrier per K-block; a DMA has S - 1 K-blocks to land.  At one tile per compute
// unit the two-stage ring waits on that DMA: its K-block time follows the latency of
// the L2 misses among a stage's lines, not the MFMA time, and a third stage (2048 x 4096
// x 7168 on 256 x 128 tiles: 64.8 -> 54.4 us) gives each DMA two K-blocks.  S = 3 turns
// the ring in trips of twelve K-blocks (three turns, three scale words) so that the stage
// and the scale byte of every K-block stay static.
// FS: the float-scale format (fp32 activation scales per row and K-block, fp32 weight
// block scales).  The MFMA then runs unscaled: the two MFMAs of a K-block (its two
// K-halves) add into a block partial P, and P * (sa * sb) is added to the
// accumulator on the VALU, which needs the accumulators in the architectural
// registers: only the 1 x 4 wavefront grid of 128 x 128 tiles (64 accumulators and
// 64 partials per lane) leaves room for the operands.  The tables then hold one fp32
// per K-block instead of one packed word per four K-blocks.
template <int BM, int BN, int WGM, int WGN, int S, bool FS = false>
struct Ring2Shape {
  static constexpr int WM = BM / WGM, WN = BN / WGN;
  static constexpr int SM = WM / 32, SN = WN / 32;
  static constexpr int SLOT = (BM + BN) * 128;
  static constexpr int IPA = BM / 32, IPB = BN / 32;  // 1 KiB DMA instructions per wavefront per K-block
  static constexpr int IPW = IPA + IPB;
  static constexpr int NBT = BN / 128;
  static constexpr int FIT = (160 * 1024 - S * SLOT - 256) / (BM * 4 + NBT * 4);
  static constexpr int WD_MAX = FIT < (FS ? 128 : 32) ? FIT : (FS ? 128 : 32);  // table entries per row
};

// NTB: the weight DMA carries the non-temporal cache policy (the weights of a masked
// call are streamed once per column tile: 939 MB at the MoE gate_up shape).
// SHUF: the weights are in the pre-shuffled layout, where K-block kb of 32-row group g
// is 4 contiguous KiB at ((g KB + kb) 4 + q) 1 KiB, q = 0..3, each KiB holding 16 bytes
// per lane in MFMA operand order.  Each DMA instruction then moves one such KiB into LDS
// lane by lane, and a lane's operand for K-half h is the two 16-byte pieces q = 2h, 2h+1
// at its own lane position (consecutive lanes, consecutive 16 bytes: conflict-free): the
// same bytes as the plain layout's operand reads, so the results are identical.
template <int BM, int BN, int WGM, int WGN, int S, bool FS = false, bool NTB = false, bool SHUF = false,
          bool NTC = false>
__global__ __launch_bounds__(256) void ring2_kernel(const KArgs p) {
  using R = Ring2Shape<BM, BN, WGM, WGN, S, FS>;
  constexpr int WM = R::WM, WN = R::WN, SM = R::SM, SN = R::SN, IPW = R::IPW, IPA = R::IPA;
  constexpr int WD_MAX = R::WD_MAX, NBT = R::NBT;
  static_assert(WGM * WGN == 4 && WM % 32 == 0 && WN % 32 == 0 && BN % 128 == 0 && BM % 32 == 0, "tile shape");
  static_assert(S >= 2 && S <= 4, "stages");
  static_assert(WD_MAX >= 1, "scale tables do not fit");
  static_assert(!FS || (WGM == 1 && BM == 128 && BN == 128 && S != 3), "float scales: 128 x 128 tiles, 1 x 4 wavefronts");
  // K-blocks per unrolled trip: whole scale words (four K-blocks) and whole turns of the ring
  constexpr int UNR = S == 3 ? 12 : 4;
  __shared__ __attribute__((aligned(1024))) uint8_t sl0[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t sl1[R::SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t sl2[S > 2 ? R::SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t sl3[S > 3 ? R::SLOT : 16];
  __shared__ __attribute__((aligned(16))) uint32_t sa_tab[WD_MAX * BM];   // [w][row]
  __shared__ __attribute__((aligned(16))) uint32_t sb_tab[NBT * WD_MAX];  // [block][w], byte kb % 4

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int64_t e = blockIdx.z;
  int tm, tn;
  xcd_tile(p, blockIdx.x, tm, tn);

  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  if (m0 >= m_limit) return;
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;

  const int KB = (int)(p.K / 128);
  const int Wd = (KB + 3) / 4;  // <= WD_MAX (checked by the host)
  const int NB = (int)((p.N + 127) / 128);
  const int KB4 = 4 * Wd;       // K-blocks, padded to whole groups of four
  const int64_t rows_valid = (m_limit - m0 < BM) ? m_limit - m0 : BM;
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > BN ? BN : cols_valid;
  const auto rA = make_rsrc(p.a + e * p.sa_e + m0 * p.K, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + eb * p.sb_e + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + eb * p.ssfb_e, (uint32_t)(NB * KB * 4));

  auto slot = [&](auto sl_tag) -> uint8_t* {
    constexpr int I = decltype(sl_tag)::value;
    if constexpr (I == 0) return sl0;
    else if constexpr (I == 1) return sl1;
    else if constexpr (I == 2) return sl2;
    else return sl3;
  };

  // DMA: instruction t < IPA of this wavefront covers A rows 8 ri .. 8 ri + 7 with
  // ri = wave * IPA + t, the others B rows likewise; lane l -> row 8 ri + (l >> 3),
  // LDS position l & 7 holding chunk (l & 7) ^ swizzle: for row 8 ri + (l >> 3) the
  // swizzle is (l >> 4) ^ 4 (ri & 1), so one offset serves even ri and one odd ri
  const uint32_t lane_row = (uint32_t)((lane >> 3) * p.K);
  const uint32_t lane_off0 = lane_row + (uint32_t)(((lane & 7) ^ (lane >> 4)) << 4);
  const uint32_t lane_off1 = lane_row + (uint32_t)(((lane & 7) ^ (lane >> 4) ^ 4) << 4);
  auto issue = [&](int kb, auto sl_tag) {
    uint8_t* base = slot(sl_tag);
    const uint32_t koff = (uint32_t)kb * 128u, oob = kb < KB ? 0u : kOOB;
#pragma unroll
    for (int t = 0; t < IPW; ++t) {
      const bool isA = t < IPA;  // static after unrolling
      const int ri = isA ? wave * IPA + t : wave * R::IPB + (t - IPA);
      uint8_t* dst = base + (isA ? 0 : BM * 128) + ri * 1024;
      // pre-shuffled weights: KiB ri of the B stage is piece q = ri & 3 of 32-row group ri >> 2
      const uint32_t off =
          (isA || !SHUF) ? ((ri & 1 ? lane_off1 : lane_off0) + (uint32_t)(ri * 8 * p.K) + koff) | oob
                         : ((uint32_t)((((ri >> 2) * KB + kb) * 4 + (ri & 3)) * 1024) + (uint32_t)(lane * 16)) | oob;
      if (isA || !NTB)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(isA ? rA : rB, (__attribute__((address_space(3))) void*)dst, 16,
                                                 (int)off, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (__attribute__((address_space(3))) void*)dst, 16, (int)off, 0, 0,
                                                 2 /* nt */);
    }
  };

  // scale tables (as in the ring kernel; FS: one fp32 per row and K-block, one fp32
  // per weight block and K-block)
  constexpr int SA_IT = (WD_MAX * BM + 255) / 256;
  constexpr int SB_IT = (NBT * WD_MAX * (FS ? 1 : 4) + 255) / 256;
  uint32_t sav[SA_IT], sbv[SB_IT];
  const auto rSAF = make_rsrc(p.sfa_f, (uint32_t)(FS ? KB * p.ld_sfa * 4 : 0));
#pragma unroll
  for (int t = 0; t < SA_IT; ++t) {
    const int idx = t * 256 + tid;
    const int w = idx / BM, row = idx - w * BM;
    if constexpr (FS) {
      const bool ok = idx < WD_MAX * BM && w < KB && m0 + row < m_limit;
      sav[t] = bload4(rSAF, ok ? (uint32_t)(((int64_t)w * p.ld_sfa + m0 + row) * 4) : kOOB);
    } else {
      const bool ok = idx < WD_MAX * BM && w < Wd && m0 + row < m_limit;
      sav[t] = bload4(rSA, ok ? (uint32_t)(((int64_t)w * p.ld_sfa + m0 + row) * 4) : kOOB);
    }
  }
#pragma unroll
  for (int t = 0; t < SB_IT; ++t) {
    const int idx = t * 256 + tid;
    const int b = idx / (WD_MAX * (FS ? 1 : 4)), k = idx - b * (WD_MAX * (FS ? 1 : 4));
    const int nb = (int)(n0 >> 7) + b;
    const bool ok = idx < NBT * WD_MAX * (FS ? 1 : 4) && nb < NB && k < KB;
    sbv[t] = bload4(rSB, ok ? (uint32_t)((nb * KB + k) * 4) : kOOB);
  }
  issue(0, IntC<0>{});
  issue(1, IntC<1>{});
  if constexpr (S > 2) issue(2, IntC<2>{});
  if constexpr (S > 3) issue(3, IntC<3>{});
#pragma unroll
  for (int t = 0; t < SA_IT; ++t) {
    const int idx = t * 256 + tid;
    const int w = idx / BM;
    uint32_t v = sav[t];
    if constexpr (!FS) {
      const int left = KB - 4 * w;
      if (left < 4) v &= left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
    }
    if (idx < WD_MAX * BM) sa_tab[idx] = v;
  }
  if constexpr (FS) {
#pragma unroll
    for (int t = 0; t < SB_IT; ++t) {
      const int idx = t * 256 + tid;
      if (idx < NBT * WD_MAX) sb_tab[idx] = sbv[t];
    }
  } else {
    uint8_t* sb_bytes = reinterpret_cast<uint8_t*>(sb_tab);
#pragma unroll
    for (int t = 0; t < SB_IT; ++t) {
      const int idx = t * 256 + tid;
      if (idx < NBT * WD_MAX * 4) sb_bytes[idx] = (uint8_t)((sbv[t] >> 23) & 0xFFu);
    }
  }
  // the first stage and the tables in place everywhere
  __builtin_amdgcn_s_waitcnt(waitcnt_imm((S - 1) * IPW, 0));
  __builtin_amdgcn_s_barrier();

  // operand reads: lane l takes row l & 31 of a 32-row group and 32 bytes of K-half
  // h: chunks 4 h + 2 (l >> 5) and the next, at positions chunk ^ ((row >> 1) & 7)
  const int lr = lane & 31, cc = 2 * (lane >> 5);
  auto rdo = [&](int h, int j) -> uint32_t {
    return (uint32_t)(lr * 128 + (((4 * h + cc + j) ^ ((lr >> 1) & 7)) << 4));
  };
  const uint32_t rd00 = rdo(0, 0), rd01 = rdo(0, 1), rd10 = rdo(1, 0), rd11 = rdo(1, 1);
  const uint32_t rds = (uint32_t)lane * 16u;  // SHUF: this lane's 16 bytes in each kilobyte
  const int sb_blk = (wn * WN) >> 7;
  uint16_t* __restrict__ C = p.c + e * p.sc_e;

  auto body = [&](auto iv_tag) {
    constexpr int IV = decltype(iv_tag)::value;
    // operands of K-half h of the K-block in stage sl_tag
    auto read_frags = [&](auto sl_tag, auto h_tag, v8i (&xf)[SM], v8i (&wf)[SN]) {
      constexpr int H = decltype(h_tag)::value;
      const uint8_t* base = slot(sl_tag);
      const uint32_t r0 = H == 0 ? rd00 : rd10, r1 = H == 0 ? rd01 : rd11;
#pragma unroll
      for (int i = 0; i < IV; ++i) {
        const uint8_t* q = base + (wm * WM + 32 * i) * 128;
        const v4i lo = *reinterpret_cast<const v4i*>(q + r0);
        const v4i hi = *reinterpret_cast<const v4i*>(q + r1);
        xf[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      if constexpr (IV > 0) {
#pragma unroll
        for (int j = 0; j < SN; ++j) {
          if constexpr (SHUF) {
            // one offset per read, added to the stage's base once: the compiler marks
            // an LDS access as disjoint from other stages only when its address is a
            // short chain of offsets from the stage (else every operand read would
            // wait for all DMA in flight)
            const uint32_t o = (uint32_t)(BM * 128 + (((wn * WN) / 32 + j) * 4 + 2 * H) * 1024) + rds;
            const v4i lo = *reinterpret_cast<const v4i*>(base + o);
            const v4i hi = *reinterpret_cast<const v4i*>(base + (o + 1024u));
            wf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          } else {
            const uint8_t* q = base + (BM + wn * WN + 32 * j) * 128;
            const v4i lo = *reinterpret_cast<const v4i*>(q + r0);
            const v4i hi = *reinterpret_cast<const v4i*>(q + r1);
            wf[j] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      }
    };

    uint32_t sa[SM], sa_n[SM];
    uint32_t sb = 0, sb_n = sb_tab[sb_blk * WD_MAX];
#pragma unroll
    for (int i = 0; i < SM; ++i) sa_n[i] = i < IV ? sa_tab[wm * WM + 32 * i + lr] : 0u;
    v8i xc[SM], wc[SN], xn[SM], wn_[SN];
    read_frags(IntC<0>{}, IntC<0>{}, xc, wc);

    v16f acc[SM][SN];
#pragma unroll
    for (int i = 0; i < SM; ++i)
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.0f;
    // FS: block partials of the current K-block (unscaled MFMAs)
    v16f part[FS ? SM : 1][FS ? SN : 1];

    auto mfmas = [&](const v8i (&xf)[SM], const v8i (&wf)[SN], auto ops_tag) {
      constexpr int OPS = decltype(ops_tag)::value;
#pragma unroll
      for (int i = 0; i < IV; ++i)
#pragma unroll
        for (int j = 0; j < SN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], acc[i][j], 0, 0, OPS, (int)sb,
                                                                      OPS, (int)sa[i]);
    };
    // FS: K-half h of a K-block into the block partials (h = 0 starts them at zero)
    auto mfmas_fs = [&](const v8i (&xf)[SM], const v8i (&wf)[SN], auto h_tag) {
      constexpr int H = decltype(h_tag)::value;
      if constexpr (FS) {
#pragma unroll
        for (int i = 0; i < IV; ++i)
#pragma unroll
          for (int j = 0; j < SN; ++j) {
            v16f c = {};
            if constexpr (H == 1) c = part[i][j];
            part[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wf[j], xf[i], c, 0, 0, 0, 0, 0, 0);
          }
      }
    };
    // FS: acc += P * (sa * sb) for K-block kb: one activation scale per lane (its
    // output row) and one weight scale per wavefront (its 128-column block)
    auto scale_add = [&](int kb) {
      if constexpr (FS) {
        const float sbf = __uint_as_float(sb_tab[sb_blk * WD_MAX + kb]);
#pragma unroll
        for (int i = 0; i < IV; ++i) {
          const float s = __uint_as_float(sa_tab[kb * BM + wm * WM + 32 * i + lr]) * sbf;
#pragma unroll
          for (int j = 0; j < SN; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = __builtin_fmaf(part[i][j][q], s, acc[i][j][q]);
        }
      }
    };

    // K-block kb = kbu + U (kbu a multiple of UNR): scale byte U % 4, stage U % S
    auto kblock = [&](int kbu, auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int ST = U % S, STN = (U + 1) % S, OPS = U % 4;
      const int kb = kbu + U;
      // half 0: MFMAs of the first K-half, reads of the second
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (OPS == 0 && !FS) {
#pragma unroll
        for (int i = 0; i < SM; ++i) sa[i] = sa_n[i];
        sb = sb_n;
      }
      read_frags(IntC<ST>{}, IntC<1>{}, xn, wn_);
      if constexpr (FS) mfmas_fs(xc, wc, IntC<0>{});
      else mfmas(xc, wc, IntC<OPS>{});
      mfma_read_dma_pattern<IV * SN, 2 * (IV > 0 ? IV + SN : 0), 0>();
      if constexpr (OPS == 2 && !FS) {
        // scale words of the next group (clamped to the table; unused past the end)
        const int wnx = (kb >> 2) + 1 < WD_MAX ? (kb >> 2) + 1 : WD_MAX - 1;
#pragma unroll
        for (int i = 0; i < SM; ++i) sa_n[i] = i < IV ? sa_tab[wnx * BM + wm * WM + 32 * i + lr] : 0u;
        sb_n = sb_tab[sb_blk * WD_MAX + wnx];
      }
      // half 1: this wavefront's DMA of kb + 1 and its reads are in; then everyone's
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm((S - 2) * IPW, 0));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue(kb + S, IntC<ST>{});
      read_frags(IntC<STN>{}, IntC<0>{}, xc, wc);
      if constexpr (FS) mfmas_fs(xn, wn_, IntC<1>{});
      else mfmas(xn, wn_, IntC<OPS>{});
      mfma_read_dma_pattern<IV * SN, 2 * (IV > 0 ? IV + SN : 0), IPW>();
      if constexpr (FS) scale_add(kb < WD_MAX ? kb : WD_MAX - 1);  // (K-blocks past the end: zero partials)
    };

    int kbu = 0;
    for (; kbu + UNR <= KB4; kbu += UNR) {
      kblock(kbu, IntC<0>{});
      kblock(kbu, IntC<1>{});
      kblock(kbu, IntC<2>{});
      kblock(kbu, IntC<3>{});
      if constexpr (UNR == 12) {
        kblock(kbu, IntC<4>{}); kblock(kbu, IntC<5>{}); kblock(kbu, IntC<6>{}); kblock(kbu, IntC<7>{});
        kblock(kbu, IntC<8>{}); kblock(kbu, IntC<9>{}); kblock(kbu, IntC<10>{}); kblock(kbu, IntC<11>{});
      }
    }
    if constexpr (UNR == 12) {
      // the last 4 or 8 K-blocks continue the ring where the trips left it
      if (kbu < KB4) {
        kblock(kbu, IntC<0>{}); kblock(kbu, IntC<1>{}); kblock(kbu, IntC<2>{}); kblock(kbu, IntC<3>{});
      }
      if (kbu + 4 < KB4) {
        kblock(kbu, IntC<4>{}); kblock(kbu, IntC<5>{}); kblock(kbu, IntC<6>{}); kblock(kbu, IntC<7>{});
      }
    }
    // the DMAs issued past the end must land, and every wavefront must be done with
    // the stages, before they are reused below
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    if constexpr (IV == 0) return;

    // epilogue through LDS (as in the ring kernel): each wavefront stages its bf16
    // sub-tile in its own LDS region and stores whole rows
    constexpr int RB = WN * 2, CPR = RB / 16, RPI = 64 / CPR;
    static_assert(4 * WM * RB <= S * R::SLOT, "staging needs the stages");
    uint8_t* stg = (wave < 2 ? sl0 : sl1) + (wave & 1) * (WM * RB);
    static_assert(2 * WM * RB <= R::SLOT, "two wavefronts per stage");
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int row = 32 * i + lr;
#pragma unroll
      for (int j = 0; j < SN; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int chunk = 4 * j + q;
          uint2 o;
          o.x = bf16_rne(acc[i][j][4 * q]) | (bf16_rne(acc[i][j][4 * q + 1]) << 16);
          o.y = bf16_rne(acc[i][j][4 * q + 2]) | (bf16_rne(acc[i][j][4 * q + 3]) << 16);
          *reinterpret_cast<uint2*>(stg + row * RB + ((chunk ^ (row % CPR)) << 4) + 8 * (lane >> 5)) = o;
        }
    }
    const int c = lane % CPR;
    const int64_t n = n0 + wn * WN + 8 * c;
#pragma unroll
    for (int t = 0; t < (IV * 32) / RPI; ++t) {
      const int row = t * RPI + lane / CPR;
      const v4i v = *reinterpret_cast<const v4i*>(stg + row * RB + ((c ^ (row % CPR)) << 4));
      const int64_t m = m0 + wm * WM + row;
      if (m < m_limit && n < p.N) {
        // NTC: streaming stores (C is not read back here; with one tile per compute unit the
        // whole of C is stored at the end of the call: 2048x4096x7168 52.6 -> 51.3 us,
        // 2048x2048x7168 on 128x128 tiles 34.1 -> 33.1 us)
        if constexpr (NTC) __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(C + m * p.ldc + n));
        else *reinterpret_cast<v4i*>(C + m * p.ldc + n) = v;
      }
    }
  };

  int64_t mine = m_limit - (m0 + wm * WM);
  mine = mine < 0 ? 0 : (mine > WM ? WM : mine);
  const int iv = __builtin_amdgcn_readfirstlane((int)((mine + 31) / 32));
  switch (iv) {
    case 0: body(IntC<0>{}); break;
    case 1: body(IntC<1>{}); break;
    case 2: if constexpr (SM >= 2) body(IntC<2 <= SM ? 2 : SM>{}); break;
    case 3: if constexpr (SM >= 3) body(IntC<3 <= SM ? 3 : SM>{}); break;
    case 4: if constexpr (SM >= 4) body(IntC<4 <= SM ? 4 : SM>{}); break;
    case 5: if constexpr (SM >= 5) body(IntC<5 <= SM ? 5 : SM>{}); break;
    case 6: if constexpr (SM >= 6) body(IntC<6 <= SM ? 6 : SM>{}); break;
    case 7: if constexpr (SM >= 7) body(IntC<7 <= SM ? 7 : SM>{}); break;
    default: if constexpr (SM >= 8) body(IntC<8 <= SM ? 8 : SM>{}); break;
  }
}

template <int BM, int BN, int WGM, int WGN, int S, bool FS = false>
constexpr int ring2_wd_max() { return Ring2Shape<BM, BN, WGM, WGN, S, FS>::WD_MAX; }


// ---------------------------------------------------------------------------
// Decode kernel: weight streaming for small M.  NW wavefronts, each owning 32
// output columns of a 64 x (32 NW) tile; K is split across workgroups (grid y).
// Per K-block kb of the workgroup's range:
//   * weights: each lane loads its two 32-byte pieces of the block straight from
//     HBM into registers in the 32x32x64 MFMA layout (lane l: row l & 31, bytes
//     32 (l >> 5) + 64 h .. + 31 for K-half h), DB K-blocks ahead of use (three
//     measured best on MI355X);
//   * activations: the 64 x 128-byte block goes to LDS by DMA (DB - 1 blocks
//     ahead, one stage per block in flight, K-half rows of 64 bytes with chunk c
//     of row r at c ^ ((r >> 2) & 3)) and every wavefront reads it from there;
//   * scales: UE8M0 exponent bytes from LDS tables filled once per workgroup
//     go to the MFMA's scale operands.
// Iteration kb waits for its own DMA of kb (and, in order, its loads of kb), meets
// the other wavefronts at a barrier, DMAs kb + DB - 1 into the stage kb - 1 used,
// reads the activation operands of kb, issues the weight loads of kb + DB and the
// four MFMAs of kb.  The epilogue stages the tile through LDS: without a K split
// the bf16 result goes to C; with one, every split's fp32 partial goes to the
// workspace and the last split of the tile to arrive adds them in split order and
// writes C (see the reduction below).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
// An empty use of a register pair: the loads that wrote it must be issued.
__device__ __forceinline__ void keep_issued(const v8i (&r)[2]) { asm volatile("" ::"v"(r[0]), "v"(r[1])); }
__device__ __forceinline__ void keep_issued4(const v4i (&r)[4]) {
  asm volatile("" ::"v"(r[0]), "v"(r[1]), "v"(r[2]), "v"(r[3]));
}
constexpr int kSC1 = 16;              // cache-policy bit sc1 of buffer loads/stores (gfx940 family)
constexpr int kNT = 2;                // cache-policy bit nt: streamed data, not kept in the caches
constexpr int kDecodeMaxSplits = 8;   // K splits the decode kernel reduces itself
constexpr int kDecodeSepMaxSplits = 16;  // K splits of the decode kernel left to splitk_reduce_kernel
constexpr int kCounterBytes = 65536;  // split-K arrival counters at the front of the workspace

template <int NW, int DB_>
struct DecodeShape {
  static constexpr int DB = DB_;               // K-blocks of weights in flight per wavefront
  static constexpr int UN = DB == 3 ? 12 : 4;  // unrolled iterations: stage/register ring and scale byte static
  static constexpr int IA = 8 / NW;            // activation DMA instructions per wavefront per K-block
  static constexpr int WMAX = 40;              // scale words per row the table holds (K <= 20480 per split)
  static constexpr int NBT = (32 * NW + 127) / 128;
};

// FS: the float-scale format.  The tables then hold fp32 scales per K-block of the
// split (activations [K-block][row], weights [column block][K-block]; at most WMAX
// K-blocks per split), the MFMAs run with unit scales into a per-K-block product,
// and acc += product * (s_a * s_b) on the VALU.
//
// WL: the weights go through LDS too.  Each wavefront DMAs its own 32 rows of the
// K-block, 8 whole 128-byte rows per instruction (chunk c of row r stored at
// c ^ (r & 7): the operand reads below are conflict-free), into a ring of DB stages
// filled DB - 1 K-blocks ahead with the activations; the MFMA operands are then read
// from LDS in the lane layout the register path loads directly.
template <int NW, int DB_, bool FS = false, bool SHUF = false, bool WL = false, bool NTL = false>
__global__ __launch_bounds__(NW * 64) void decode_kernel(const KArgs p) {
  using D = DecodeShape<NW, DB_>;
  constexpr int DB = D::DB, UN = D::UN, IA = D::IA, WMAX = D::WMAX, NBT = D::NBT;
  constexpr int NT = NW * 64, BN = 32 * NW;
  static_assert((NW == 4 || NW == 8) && IA >= 1, "decode shape");
  static_assert(!(WL && SHUF), "one weight path");
  constexpr int WST = WL ? BN * 128 : 16;  // bytes of one weight stage
  // one array per stage (see the ring kernel: the compiler's LDS-DMA tracking then
  // tells a stage's reads from the other stages' DMA)
  __shared__ __attribute__((aligned(1024))) uint8_t st0[8192];
  __shared__ __attribute__((aligned(1024))) uint8_t st1[8192];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[8192];
  __shared__ __attribute__((aligned(1024))) uint8_t st3[8192];
  __shared__ __attribute__((aligned(16))) uint32_t sa_tab[WMAX * 64];       // [w][row]
  __shared__ __attribute__((aligned(16))) uint32_t sb_tab[NBT * WMAX];      // [block][w], byte kb % 4
  __shared__ __attribute__((aligned(16))) uint8_t stage_out[NW * 64 * 32 * 4];  // epilogue: [wave][64][32] fp32
  __shared__ __attribute__((aligned(1024))) uint8_t wt0[WST];
  __shared__ __attribute__((aligned(1024))) uint8_t wt1[WST];
  __shared__ __attribute__((aligned(1024))) uint8_t wt2[WST];
  __shared__ __attribute__((aligned(1024))) uint8_t wt3[WST];
  static_assert(DB >= 2 && DB <= 4, "two to four stages");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t e = blockIdx.z;
  const int split = blockIdx.y;
  const int tm = blockIdx.x / p.tiles_n, tn = blockIdx.x - tm * p.tiles_n;
  int64_t m_limit = p.M;
  if (p.masked_m) {
    const int64_t cnt = p.masked_m[e];
    m_limit = cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt);
  }
  const int64_t m0 = (int64_t)tm * 64, n0 = (int64_t)tn * BN;
  if (m0 >= m_limit) return;
  const int64_t eb = weight_group(p, e, m0);
  if (eb < 0) return;

  const int KB = (int)(p.K / 128);
  const int kb0 = split * p.kb_per_split;
  const int nk = (KB - kb0 < p.kb_per_split) ? KB - kb0 : p.kb_per_split;  // >= 1 (host)
  const int nk4 = (nk + 3) & ~3;            // iterations: K-blocks padded to a whole scale word
  const int nfull = nk4 / UN * UN;          // iterations in whole unrolled groups; a tail of 4 or 8 follows
  const int NB = (int)((p.N + 127) / 128);
  const int64_t rows_valid = (m_limit - m0 < 64) ? m_limit - m0 : 64;
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > BN ? BN : cols_valid;
  const auto rA = make_rsrc(p.a + e * p.sa_e + m0 * p.K, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + eb * p.sb_e + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const int Wd = (KB + 3) / 4;
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + eb * p.ssfb_e, (uint32_t)(NB * KB * 4));

  auto stage = [&](auto tag) -> uint8_t* {
    constexpr int I = decltype(tag)::value;
    if constexpr (I == 0) return st0;
    else if constexpr (I == 1) return st1;
    else if constexpr (I == 2) return st2;
    else return st3;
  };
  auto wstage = [&](auto tag) -> uint8_t* {
    constexpr int I = decltype(tag)::value;
    if constexpr (I == 0) return wt0;
    else if constexpr (I == 1) return wt1;
    else if constexpr (I == 2) return wt2;
    else return wt3;
  };
  // WL weight DMA: instruction t of this wavefront covers rows 32 wave + 8 t + (l >> 3),
  // LDS chunk l & 7 holding row chunk (l & 7) ^ (row & 7)
  const uint32_t wdma_lane = (uint32_t)((lane >> 3) * p.K) + (uint32_t)((((lane & 7) ^ ((lane >> 3) & 7)) << 4));

  // activation DMA: instruction t of this wavefront covers K-half hh of rows
  // 16 rq .. 16 rq + 15 (rq, hh from the instruction index i = wave * IA + t:
  // hh = i >> 2, rq = i & 3); lane l -> row 16 rq + (l >> 2), position l & 3
  uint32_t aoff[IA];
#pragma unroll
  for (int t = 0; t < IA; ++t) {
    const int i = wave * IA + t;
    const int r = (i & 3) * 16 + (lane >> 2);
    aoff[t] = (uint32_t)(r * p.K) + (uint32_t)((i >> 2) * 64) + (uint32_t)((((lane & 3) ^ swz64(r)) << 4));
  }
  auto issue_a = [&](int j, auto tag) {  // j: iteration index of the K-block
    uint8_t* base = stage(tag);
    const uint32_t koff = (uint32_t)(kb0 + j) * 128u, oob = j < nk ? 0u : kOOB;
#pragma unroll
    for (int t = 0; t < IA; ++t) {
      const int i = wave * IA + t;
      uint8_t* dst = base + (i >> 2) * 4096 + (i & 3) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)dst, 16,
                                               (int)((aoff[t] + koff) | oob), 0, 0, 0);
    }
    if constexpr (WL) {
      uint8_t* wbase = wstage(tag) + wave * 32 * 128;
#pragma unroll
      for (int t = 0; t < 4; ++t)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (__attribute__((address_space(3))) void*)(wbase + t * 1024), 16,
                                                 (int)((wdma_lane + (uint32_t)((wave * 32 + 8 * t) * p.K) + koff) | oob),
                                                 0, 0, NTL ? kNT : 0);
    }
  };
  // weight loads: lane l, row n0 + 32 wave + (l & 31), bytes 32 (l >> 5) + 64 h .. + 31.
  // SHUF: the same bytes from the pre-shuffled layout, where every 32-row group's
  // K-block is 4 KB in load order (one contiguous 1 KB per load instruction)
  const uint32_t boff = SHUF ? (uint32_t)(wave * 32 * p.K) + (uint32_t)(16 * lane)
                             : (uint32_t)((wave * 32 + (lane & 31)) * p.K) + (uint32_t)(32 * (lane >> 5));
  constexpr uint32_t KB_STEP = SHUF ? 4096u : 128u, H_STEP = SHUF ? 2048u : 64u, P_STEP = SHUF ? 1024u : 16u;
  auto load_b = [&](int j, v8i (&bh)[2]) {
    if constexpr (WL) return;  // the weights come with the activation DMA
    const uint32_t off = (boff + (uint32_t)(kb0 + j) * KB_STEP) | (j < nk ? 0u : kOOB);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const v4i lo = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(off + H_STEP * h), 0, NTL ? kNT : 0));
      const v4i hi = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(off + H_STEP * h + P_STEP), 0, NTL ? kNT : 0));
      bh[h] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
  };

  // scale tables for this split's K-blocks: activation words of the 64 rows (zero
  // past the rows and for K-blocks past the split), weight exponent bytes.  The
  // global loads go out first, then the prologue prefetch, then the LDS writes, so
  // the table loads' latency overlaps the prefetch.
  const int w0 = kb0 / 4;                   // kb0 is a multiple of 4 (host)
  const int nw = nk4 / 4;                   // words of this split, <= WMAX (host)
  constexpr int SA_PT = (WMAX * 64 + NT - 1) / NT, SB_PT = (NBT * WMAX * 4 + NT - 1) / NT;
  uint32_t sav[SA_PT], sbv[SB_PT];
  if constexpr (FS) {
    // fp32 scales: activations [j][row], weights [block][j] for K-blocks j < nk
    const auto rSAF = make_rsrc(p.sfa_f + e * p.ssfa_e, (uint32_t)(KB * p.ld_sfa * 4));
#pragma unroll
    for (int t = 0; t < SA_PT; ++t) {
      const int idx = t * NT + tid, j = idx >> 6, row = idx & 63;
      const bool ok = idx < WMAX * 64 && j < nk && m0 + row < m_limit;
      sav[t] = bload4(rSAF, ok ? (uint32_t)(((int64_t)(kb0 + j) * p.ld_sfa + m0 + row) * 4) : kOOB);
    }
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * NT + tid, b = idx / WMAX, j = idx - b * WMAX;
      const int nb = (int)(n0 >> 7) + b;
      const bool ok = idx < NBT * WMAX && nb < NB && j < nk;
      sbv[t] = bload4(rSB, ok ? (uint32_t)((nb * KB + kb0 + j) * 4) : kOOB);
    }
  } else {
#pragma unroll
    for (int t = 0; t < SA_PT; ++t) {
      const int idx = t * NT + tid, w = idx >> 6, row = idx & 63;
      const bool ok = idx < nw * 64 && m0 + row < m_limit && w0 + w < Wd;
      sav[t] = bload4(rSA, ok ? (uint32_t)(((int64_t)(w0 + w) * p.ld_sfa + m0 + row) * 4) : kOOB);
    }
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * NT + tid, b = idx / (WMAX * 4), j = idx - b * (WMAX * 4);
      const int nb = (int)(n0 >> 7) + b;
      const bool ok = idx < NBT * WMAX * 4 && nb < NB && j < nk;
      sbv[t] = bload4(rSB, ok ? (uint32_t)((nb * KB + kb0 + j) * 4) : kOOB);
    }
  }

  // prologue: weights of iterations 0 .. DB-1 and activations of 0 .. DB-2, in the
  // order the loop keeps (activations of j + DB - 1, then weights of j + DB)
  v8i b0[2], b1[2], b2[2], b3[2];
  auto breg = [&](auto tag) -> v8i (&)[2] {
    constexpr int I = decltype(tag)::value;
    if constexpr (I == 0) return b0;
    else if constexpr (I == 1) return b1;
    else if constexpr (I == 2) return b2;
    else return b3;
  };
  load_b(0, b0);
  issue_a(0, IntC<0>{});
  load_b(1, b1);
  if constexpr (DB > 2) {
    issue_a(1, IntC<1>{});
    load_b(2, b2);
  }
  if constexpr (DB > 3) {
    issue_a(2, IntC<2>{});
    load_b(3, b3);
  }

  if constexpr (FS) {
#pragma unroll
    for (int t = 0; t < SA_PT; ++t) {
      const int idx = t * NT + tid;
      if (idx < WMAX * 64) sa_tab[idx] = sav[t];
    }
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * NT + tid;
      if (idx < NBT * WMAX) sb_tab[idx] = sbv[t];
    }
  } else {
#pragma unroll
    for (int t = 0; t < SA_PT; ++t) {
      const int idx = t * NT + tid, w = idx >> 6;
      uint32_t v = sav[t];
      const int left = kb0 + nk - 4 * (w0 + w);  // K-blocks of this word inside the split
      if (left < 4) v &= left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
      if (idx < WMAX * 64) sa_tab[idx] = v;
    }
    uint8_t* sbb = reinterpret_cast<uint8_t*>(sb_tab);
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * NT + tid;
      if (idx < NBT * WMAX * 4) sbb[idx] = (uint8_t)((sbv[t] >> 23) & 0xFFu);
    }
  }
  // VMEM instructions younger than the activation DMA of the current iteration (WL:
  // the DMA groups of the next DB - 2 K-blocks; else also the weight loads of the next)
  constexpr int YOUNGER = WL ? (DB - 2) * (IA + 4) : 4 + (DB - 2) * (IA + 4);

  const int lr = lane & 31, c0 = 2 * (lane >> 5);
  const uint32_t rd0 = (uint32_t)(lr * 64 + ((c0 ^ swz64(lr)) << 4));
  const uint32_t rd1 = (uint32_t)(lr * 64 + (((c0 + 1) ^ swz64(lr)) << 4));
  const int sb_blk = (wave * 32) >> 7;

  auto body = [&](auto iv_tag) {
    constexpr int IV = decltype(iv_tag)::value;  // 32-row groups with valid rows (1 or 2)
    v16f acc[IV];
#pragma unroll
    for (int i = 0; i < IV; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
    uint32_t sa[IV], sb = 0;

    // iteration j = jb + U (jb a multiple of UN): K-block kb0 + j, scale byte U % 4,
    // LDS stage and weight registers U % DB
    auto iter = [&](int jb, auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int OPS = U % 4;
      v8i(&bcur)[2] = breg(IntC<U % DB>{});
      const int j = jb + U;
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_waitcnt(waitcnt_imm(YOUNGER, 15));
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_a(j + DB - 1, IntC<(U + DB - 1) % DB>{});
      if constexpr (FS) {
#pragma unroll
        for (int i = 0; i < IV; ++i) sa[i] = sa_tab[j * 64 + 32 * i + lr];
        sb = sb_tab[sb_blk * WMAX + j];
      } else if constexpr (OPS == 0) {
#pragma unroll
        for (int i = 0; i < IV; ++i) sa[i] = sa_tab[(j >> 2) * 64 + 32 * i + lr];
        sb = sb_tab[sb_blk * WMAX + (j >> 2)];
      }
      const uint8_t* base = stage(IntC<U % DB>{});
      if constexpr (WL) {
        // this wavefront's 32 rows from the weight stage: lane l, row l & 31, logical
        // chunks 4 h + 2 (l >> 5) and the next (the register path's byte order)
        const uint8_t* wb = wstage(IntC<U % DB>{}) + (wave * 32 + lr) * 128;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int wc = 4 * h + 2 * (lane >> 5);
          const v4i lo = *reinterpret_cast<const v4i*>(wb + ((wc ^ (lr & 7)) << 4));
          const v4i hi = *reinterpret_cast<const v4i*>(wb + (((wc + 1) ^ (lr & 7)) << 4));
          bcur[h] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      }
      v8i af[2][IV];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < IV; ++i) {
          const uint8_t* q = base + h * 4096 + (32 * i) * 64;
          const v4i lo = *reinterpret_cast<const v4i*>(q + rd0);
          const v4i hi = *reinterpret_cast<const v4i*>(q + rd1);
          af[h][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
      if constexpr (FS) {
        // unit scales (byte 127) into the K-block's product, then the two fp32 scales
#pragma unroll
        for (int i = 0; i < IV; ++i) {
          v16f d = {};
#pragma unroll
          for (int h = 0; h < 2; ++h)
            d = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bcur[h], af[h][i], d, 0, 0, 0, 127, 0, 127);
          const float sc = __uint_as_float(sa[i]) * __uint_as_float(sb);
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[i][r] = __builtin_fmaf(d[r], sc, acc[i][r]);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < IV; ++i)
            acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bcur[h], af[h][i], acc[i], 0, 0, OPS, (int)sb,
                                                                     OPS, (int)sa[i]);
      }
      load_b(j + DB, bcur);  // the registers of kb are free again: fetch kb + DB
    };

    for (int jb = 0; jb < nfull; jb += UN) {
      iter(jb, IntC<0>{});
      iter(jb, IntC<1>{});
      iter(jb, IntC<2>{});
      iter(jb, IntC<3>{});
      if constexpr (UN == 12) {
        iter(jb, IntC<4>{});
        iter(jb, IntC<5>{});
        iter(jb, IntC<6>{});
        iter(jb, IntC<7>{});
        iter(jb, IntC<8>{});
        iter(jb, IntC<9>{});
        iter(jb, IntC<10>{});
        iter(jb, IntC<11>{});
      }
    }
    if constexpr (UN == 12) {
      // tail of 4 or 8 iterations: a multiple of three unrolled groups precede it, so
      // the stage / register ring and the scale byte continue from U = 0
      if (nk4 - nfull >= 4) {
        iter(nfull, IntC<0>{});
        iter(nfull, IntC<1>{});
        iter(nfull, IntC<2>{});
        iter(nfull, IntC<3>{});
      }
      if (nk4 - nfull >= 8) {
        iter(nfull, IntC<4>{});
        iter(nfull, IntC<5>{});
        iter(nfull, IntC<6>{});
        iter(nfull, IntC<7>{});
      }
    }
    // The weight prefetches past the last K-block are never read, so in straight-line
    // code after the loop the compiler would drop them; every iteration's vmcnt wait
    // counts them as issued after its activation DMA, so without them the wait would
    // no longer cover the DMA.  An empty use keeps them.
    keep_issued(b0);
    keep_issued(b1);
    if constexpr (DB > 2) keep_issued(b2);
    if constexpr (DB > 3) keep_issued(b3);
    // the prefetches past the range (out of range, zero-filled) must land before
    // the LDS is reused or released
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));

    // epilogue: lane l holds, for row group i, row 32 i + (l & 31) and the columns
    // 8 q + 4 (l >> 5) + 0..3 of the wavefront's 32 (registers 4q..4q+3).  Stage the
    // wavefront's 64 x 32 fp32 block in LDS (16-byte chunk c of row r at c ^ (r & 7))
    // and move it 8 rows of 128 bytes per instruction.
    float* so = reinterpret_cast<float*>(stage_out + wave * 64 * 128);
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int row = 32 * i + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = 2 * q + (lane >> 5);
        *reinterpret_cast<v4f*>(reinterpret_cast<uint8_t*>(so) + row * 128 + ((chunk ^ (row & 7)) << 4)) =
            v4f{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]};
      }
    }
    const int ch = lane & 7;
    const int64_t n = n0 + wave * 32 + 4 * ch;
    auto staged = [&](int t) -> v4f {
      const int row = t * 8 + (lane >> 3);
      return *reinterpret_cast<const v4f*>(reinterpret_cast<const uint8_t*>(so) + row * 128 + ((ch ^ (row & 7)) << 4));
    };
    uint16_t* __restrict__ C = p.c + e * p.sc_e;
    auto store_c = [&](int t, v4f v) {
      const int64_t m = m0 + t * 8 + (lane >> 3);
      if (m >= m_limit || n >= p.N) return;
      uint2 o;
      o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
      o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(C + m * p.ldc + n) = o;
    };
    if (p.splits == 1) {
#pragma unroll
      for (int t = 0; t < IV * 4; ++t) store_c(t, staged(t));
      return;
    }
    const size_t slice = (size_t)p.M * (size_t)p.N;
    if (!p.counters) {
      // K split finished by splitk_reduce_kernel on the same stream: publish this
      // split's partial (the kernel boundary makes it visible to the reduction)
#pragma unroll
      for (int t = 0; t < IV * 4; ++t) {
        const int64_t m = m0 + t * 8 + (lane >> 3);
        if (m < m_limit && n < p.N)
          *reinterpret_cast<v4f*>(p.ws + (size_t)split * slice + (size_t)m * p.N + n) = staged(t);
      }
      return;
    }
    // K split, reduced in this kernel by the last split of the tile to arrive.  The
    // partials are written with sc1 (coherent across the XCDs' L2 caches: written
    // through) and complete (s_waitcnt) before this split bumps the tile's arrival
    // counter; the last arrival reads the other partials with sc1 loads, adds all of
    // them in split order (deterministic) and writes bf16, and sets the counter back
    // to zero for the next call.  No cache-wide fence is needed: only the partials
    // cross workgroups, and they never sit dirty in an L2.
    const auto rW = make_rsrc(p.ws, (uint32_t)(((size_t)p.splits * slice) * 4 > 0x7FFFFFFFull
                                                   ? 0x7FFFFFFFu : (size_t)p.splits * slice * 4));
    auto woff = [&](int sp, int t) -> uint32_t {
      const int64_t m = m0 + t * 8 + (lane >> 3);
      return (m < m_limit && n < p.N) ? (uint32_t)(((size_t)sp * slice + (size_t)m * p.N + n) * 4) : kOOB;
    };
#pragma unroll
    for (int t = 0; t < IV * 4; ++t)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, staged(t)), rW, (int)woff(split, t), 0, kSC1);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __shared__ int last_flag;
    const int tile = blockIdx.x;
    if (tid == 0) {
      const uint32_t old = __hip_atomic_fetch_add(p.counters + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_flag = (old == (uint32_t)(p.splits - 1)) ? 1 : 0;
    }
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    if (!last_flag) return;
    if (tid == 0) __hip_atomic_store(p.counters + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    // the other splits' partials, four splits at a time: every load of a batch is
    // issued before the first add (one memory round trip per batch, not one per
    // row group), and the adds keep split order
    v4f sum[IV * 4];
#pragma unroll
    for (int t = 0; t < IV * 4; ++t) sum[t] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int sb = 0; sb < p.splits; sb += 4) {
      v4f part[4][IV * 4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < IV * 4; ++t) {
          const int sp = sb + u;
          part[u][t] = __builtin_bit_cast(
              v4f, __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(sp < p.splits && sp != split ? woff(sp, t) : kOOB), 0, kSC1));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < IV * 4; ++t)
          if (sb + u < p.splits) sum[t] += sb + u == split ? staged(t) : part[u][t];
    }
#pragma unroll
    for (int t = 0; t < IV * 4; ++t) store_c(t, sum[t]);
  };

  // tables and the first DMA in place everywhere
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
  __builtin_amdgcn_s_barrier();
  if (rows_valid > 32) body(IntC<2>{});
  else body(IntC<1>{});
}

// ---------------------------------------------------------------------------
// Weight-streaming decode kernel (dense M <= 64, weights in the pre-shuffled
// layout).  Four wavefronts; wavefront w owns the 32 output columns n0 + 32 w ..
// + 31 of a 64 x 128 tile, and K is split over workgroups.  The time of a
// decode-sized GEMM is the time to stream its weights, and a workgroup streams at
// the rate (bytes in flight) / (memory latency), so the kernel is built to keep
// many weight bytes in flight with little else on the issue path:
//   * weights: each lane loads its operand bytes straight into registers (one
//     contiguous kilobyte per load instruction in the pre-shuffled layout), D
//     K-blocks ahead of use, as non-temporal loads (streamed data that no other
//     workgroup reads: on MI355X a streaming read reaches ~6.4 TB/s this way
//     against ~5.7 TB/s with ordinary loads);
//   * activations: the 64 x 128-byte K-blocks go to LDS by DMA in groups of four,
//     one group ahead, so the workgroup meets at a barrier once per four K-blocks;
//   * UE8M0 exponents from LDS tables are the MFMA scale operands.
// With RED the K split is summed in the kernel: after its loop a workgroup takes a
// ticket on its tile (device-scope atomic); all but the last store their fp32
// partials with device-coherent stores and then count themselves ready; the last
// waits until the others are ready (they hold tickets, so they are running and
// will be), loads their partials and adds all of them in split order (so the sum
// does not depend on who arrived last) and writes bf16.  It leaves both counters
// at zero for the next call.  Without RED the partials go to splitk_reduce_kernel.
template <int D, int RED>
struct WsdShape {
  static constexpr int AG = 4;                       // K-blocks per activation group
  static constexpr int UN = D == 4 ? 8 : 24;         // unroll: weight ring, group buffer and scale byte static
  static constexpr int WMAX = 40;                    // scale words per row per split
  static constexpr int ASZ = AG * 8192;              // one activation group in LDS
};

template <int D, int RED>
__global__ __launch_bounds__(256) void wsd_kernel(const KArgs p) {
  using S_ = WsdShape<D, RED>;
  constexpr int AG = S_::AG, UN = S_::UN, WMAX = S_::WMAX, ASZ = S_::ASZ;
  static_assert(D == 3 || D == 4 || D == 6, "weight ring depth");
  __shared__ __attribute__((aligned(1024))) uint8_t ab0[ASZ];
  __shared__ __attribute__((aligned(1024))) uint8_t ab1[ASZ];
  __shared__ __attribute__((aligned(16))) uint32_t sa_tab[WMAX * 64];  // [w][row]
  __shared__ __attribute__((aligned(16))) uint32_t sb_tab[WMAX];       // [w], byte kb % 4
  __shared__ int s_ticket;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (column tile, split): workgroups are dispatched to the eight XCDs
  // in turn (a workgroup's XCD is its linear id mod 8), so tile tn's splits get ids
  // congruent to tn mod 8 and share one XCD and its L2.  The grid is padded to
  // 8 ceil(T / 8) S workgroups; those past the last tile have nothing to do.
  const int id = blockIdx.x, S = p.splits, T = p.tiles_n;
  const int jj = id >> 3;
  const int tn = (id & 7) + 8 * (jj / S), split = jj - (jj / S) * S;
  if (tn >= T) return;
  const int64_t m_limit = p.M;
  const int64_t n0 = (int64_t)tn * 128;
  const int KB = (int)(p.K / 128);
  const int kb0 = split * p.kb_per_split;
  const int nk = (KB - kb0 < p.kb_per_split) ? KB - kb0 : p.kb_per_split;  // >= 1 (host)
  const int nk4 = (nk + 3) & ~3;
  const int nfull = nk4 / UN * UN;
  const int NB = (int)((p.N + 127) / 128);
  const int64_t rows_valid = m_limit < 64 ? m_limit : 64;
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > 128 ? 128 : cols_valid;
  const auto rA = make_rsrc(p.a, (uint32_t)(rows_valid * p.K));
  const auto rB = make_rsrc(p.b + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const int Wd = (KB + 3) / 4;
  const auto rSA = make_rsrc(p.sfa, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb, (uint32_t)(NB * KB * 4));

  // activation DMA of K-block j into group buffer `buf` at position u: instruction t
  // (0, 1) of this wavefront covers K-half hh = i >> 2 of rows 16 (i & 3) .. + 15,
  // i = 2 wave + t; lane l -> row 16 (i & 3) + (l >> 2), LDS chunk l & 3 holding
  // chunk (l & 3) ^ swz64(row) of the K-half
  uint32_t aoff[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int i = wave * 2 + t;
    const int r = (i & 3) * 16 + (lane >> 2);
    aoff[t] = (uint32_t)(r * p.K) + (uint32_t)((i >> 2) * 64) + (uint32_t)((((lane & 3) ^ swz64(r)) << 4));
  }
  auto dma_group = [&](int g, uint8_t* buf) {
#pragma unroll
    for (int u = 0; u < AG; ++u) {
      const int j = g * AG + u;
      const uint32_t koff = (uint32_t)(kb0 + j) * 128u, oob = j < nk ? 0u : kOOB;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int i = wave * 2 + t;
        uint8_t* dst = buf + u * 8192 + (i >> 2) * 4096 + (i & 3) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)dst, 16,
                                                 (int)((aoff[t] + koff) | oob), 0, 0, 0);
      }
    }
  };
  // weight loads of K-block j: lane l, 16 bytes at 1 KB steps (pre-shuffled layout,
  // 32-row group of this wavefront)
  const uint32_t boff = (uint32_t)(wave * 32 * p.K) + (uint32_t)(16 * lane);
  auto load_w = [&](int j, v4i (&w)[4]) {
    const uint32_t off = (boff + (uint32_t)(kb0 + j) * 4096u) | (j < nk ? 0u : kOOB);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(off + 1024u * q), 0, kNT));
  };

  // scale tables of this split: activation words of the 64 rows (zero past the
  // rows and for K-blocks past the split), weight exponent bytes of this tile's
  // column block
  const int w0 = kb0 / 4;  // kb0 is a multiple of 4 (host)
  const int nw = nk4 / 4;  // <= WMAX (host)
  constexpr int SA_PT = (WMAX * 64 + 255) / 256, SB_PT = (WMAX * 4 + 255) / 256;
  uint32_t sav[SA_PT], sbv[SB_PT];
  dma_group(0, ab0);
#pragma unroll
  for (int t = 0; t < SA_PT; ++t) {
    const int idx = t * 256 + tid, w = idx >> 6, row = idx & 63;
    const bool ok = idx < nw * 64 && row < m_limit && w0 + w < Wd;
    sav[t] = bload4(rSA, ok ? (uint32_t)(((int64_t)(w0 + w) * p.ld_sfa + row) * 4) : kOOB);
  }
#pragma unroll
  for (int t = 0; t < SB_PT; ++t) {
    const int idx = t * 256 + tid;
    const bool ok = idx < WMAX * 4 && idx < nk;
    sbv[t] = bload4(rSB, ok ? (uint32_t)(((n0 >> 7) * KB + kb0 + idx) * 4) : kOOB);
  }
  v4i wr[D][4];
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d, wr[d]);
#pragma unroll
  for (int t = 0; t < SA_PT; ++t) {
    const int idx = t * 256 + tid, w = idx >> 6;
    uint32_t v = sav[t];
    const int left = kb0 + nk - 4 * (w0 + w);  // K-blocks of this word inside the split
    if (left < 4) v &= left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
    if (idx < WMAX * 64) sa_tab[idx] = v;
  }
  {
    uint8_t* sbb = reinterpret_cast<uint8_t*>(sb_tab);
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * 256 + tid;
      if (idx < WMAX * 4) sbb[idx] = (uint8_t)((sbv[t] >> 23) & 0xFFu);
    }
  }
  // the first activation group and the tables in place everywhere (the weight loads
  // issued after them may still be in flight)
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * D, 0));
  __builtin_amdgcn_s_barrier();

  const int lr = lane & 31, c0 = 2 * (lane >> 5);
  const uint32_t rd0 = (uint32_t)(lr * 64 + ((c0 ^ swz64(lr)) << 4));
  const uint32_t rd1 = (uint32_t)(lr * 64 + (((c0 + 1) ^ swz64(lr)) << 4));

  auto body = [&](auto iv_tag) {
    constexpr int IV = decltype(iv_tag)::value;  // 32-row groups with valid rows (1 or 2)
    v16f acc[IV];
#pragma unroll
    for (int i = 0; i < IV; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
    uint32_t sa[IV], sb = 0;

    // iteration j = jb + U (jb a multiple of UN)
    auto iter = [&](int jb, auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int OPS = U % 4, SLOT = U % D, GB = (U / AG) % 2, POS = U % AG;
      const int j = jb + U;
      if constexpr (POS == 0) {
        // a new activation group: its DMA (issued one group ago, followed by that
        // group's AG x 4 weight loads) has landed here and everywhere, and nobody
        // reads the other buffer any more: refill it with the next group
        __builtin_amdgcn_sched_barrier(0);
        if (j > 0) {  // the prologue's barrier opens group 0
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * AG, 15));
          __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        dma_group(j / AG + 1, GB == 0 ? ab1 : ab0);
        // the group barrier's wait counts exactly the AG x 4 weight loads issued
        // after this DMA: nothing may move above it
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (OPS == 0) {
#pragma unroll
        for (int i = 0; i < IV; ++i) sa[i] = sa_tab[(j >> 2) * 64 + 32 * i + lr];
        sb = sb_tab[j >> 2];
      }
      const uint8_t* base = (GB == 0 ? ab0 : ab1) + POS * 8192;
      v8i af[2][IV];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < IV; ++i) {
          const uint8_t* q = base + h * 4096 + (32 * i) * 64;
          const v4i lo = *reinterpret_cast<const v4i*>(q + rd0);
          const v4i hi = *reinterpret_cast<const v4i*>(q + rd1);
          af[h][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v8i bw = __builtin_shufflevector(wr[SLOT][2 * h], wr[SLOT][2 * h + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int i = 0; i < IV; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bw, af[h][i], acc[i], 0, 0, OPS, (int)sb, OPS,
                                                                   (int)sa[i]);
      }
      load_w(j + D, wr[SLOT]);  // the registers of j are free again: fetch j + D
      // issue the loads here: left to itself the scheduler sinks them towards the
      // end of the activation group, which shortens the prefetch distance
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int jb = 0; jb < nfull; jb += UN) {
      iter(jb, IntC<0>{}); iter(jb, IntC<1>{}); iter(jb, IntC<2>{}); iter(jb, IntC<3>{});
      iter(jb, IntC<4>{}); iter(jb, IntC<5>{}); iter(jb, IntC<6>{}); iter(jb, IntC<7>{});
      if constexpr (UN == 24) {
        iter(jb, IntC<8>{}); iter(jb, IntC<9>{}); iter(jb, IntC<10>{}); iter(jb, IntC<11>{});
        iter(jb, IntC<12>{}); iter(jb, IntC<13>{}); iter(jb, IntC<14>{}); iter(jb, IntC<15>{});
        iter(jb, IntC<16>{}); iter(jb, IntC<17>{}); iter(jb, IntC<18>{}); iter(jb, IntC<19>{});
        iter(jb, IntC<20>{}); iter(jb, IntC<21>{}); iter(jb, IntC<22>{}); iter(jb, IntC<23>{});
      }
    }
    // tail: the remaining K-blocks (a multiple of four, fewer than UN) continue the
    // ring from U = 0, one activation group at a time
    const int rest = nk4 - nfull;
    if (rest >= 4) { iter(nfull, IntC<0>{}); iter(nfull, IntC<1>{}); iter(nfull, IntC<2>{}); iter(nfull, IntC<3>{}); }
    if (rest >= 8) { iter(nfull, IntC<4>{}); iter(nfull, IntC<5>{}); iter(nfull, IntC<6>{}); iter(nfull, IntC<7>{}); }
    if constexpr (UN == 24) {
      if (rest >= 12) { iter(nfull, IntC<8>{}); iter(nfull, IntC<9>{}); iter(nfull, IntC<10>{}); iter(nfull, IntC<11>{}); }
      if (rest >= 16) { iter(nfull, IntC<12>{}); iter(nfull, IntC<13>{}); iter(nfull, IntC<14>{}); iter(nfull, IntC<15>{}); }
      if (rest >= 20) { iter(nfull, IntC<16>{}); iter(nfull, IntC<17>{}); iter(nfull, IntC<18>{}); iter(nfull, IntC<19>{}); }
    }
    // the loads issued past the range (out of range: zeros, into registers and the
    // spare group buffer) must land before the LDS is reused or released
#pragma unroll
    for (int d = 0; d < D; ++d) keep_issued4(wr[d]);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();

    // epilogue: stage the wavefront's 64 x 32 fp32 block in LDS (16-byte chunk c of
    // row r at c ^ (r & 7)); lane l then holds 4 consecutive columns of row
    // 8 t + (l >> 3) for t < 4 IV
    float* so = reinterpret_cast<float*>(ab0 + wave * 64 * 128);
#pragma unroll
    for (int i = 0; i < IV; ++i) {
      const int row = 32 * i + lr;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int chunk = 2 * q + (lane >> 5);
        *reinterpret_cast<v4f*>(reinterpret_cast<uint8_t*>(so) + row * 128 + ((chunk ^ (row & 7)) << 4)) =
            v4f{acc[i][4 * q], acc[i][4 * q + 1], acc[i][4 * q + 2], acc[i][4 * q + 3]};
      }
    }
    const int ch = lane & 7;
    const int64_t n = n0 + wave * 32 + 4 * ch;
    v4f part[IV * 4];
#pragma unroll
    for (int t = 0; t < IV * 4; ++t) {
      const int row = t * 8 + (lane >> 3);
      part[t] = *reinterpret_cast<const v4f*>(reinterpret_cast<const uint8_t*>(so) + row * 128 + ((ch ^ (row & 7)) << 4));
    }
    auto store_c = [&](int t, v4f v) {
      const int64_t m = t * 8 + (lane >> 3);
      if (m >= m_limit || n >= p.N) return;
      uint2 o;
      o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
      o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(p.c + m * p.ldc + n) = o;
    };
    if (S == 1) {
#pragma unroll
      for (int t = 0; t < IV * 4; ++t) store_c(t, part[t]);
      return;
    }
    if constexpr (RED == 0) {
      const size_t slice = (size_t)p.M * (size_t)p.N;
#pragma unroll
      for (int t = 0; t < IV * 4; ++t) {
        const int64_t m = t * 8 + (lane >> 3);
        if (m < m_limit && n < p.N) *reinterpret_cast<v4f*>(p.ws + (size_t)split * slice + (size_t)m * p.N + n) = part[t];
      }
      return;
    } else {
      // partials [split][M][N] fp32, as for splitk_reduce_kernel
      const size_t slice = (size_t)p.M * (size_t)p.N;
      uint32_t* cnt = p.counters + 2 * tn;
      const auto rW = make_rsrc(p.ws, (uint32_t)((size_t)S * slice * 4));
      auto poff = [&](int sp, int t) -> uint32_t {
        const int64_t m = t * 8 + (lane >> 3);
        return (m < m_limit && n < p.N) ? (uint32_t)(((size_t)sp * slice + (size_t)m * p.N + n) * 4) : kOOB;
      };
      auto sum_and_store = [&](auto pol_tag) {
        constexpr int load_pol = decltype(pol_tag)::value;
        v4f sum[IV * 4];
#pragma unroll
        for (int t = 0; t < IV * 4; ++t) sum[t] = v4f{0.f, 0.f, 0.f, 0.f};
        for (int sb0 = 0; sb0 < S; sb0 += 4) {
          v4f pt[4][IV * 4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int t = 0; t < IV * 4; ++t) {
              const int sp = sb0 + u;
              pt[u][t] = __builtin_bit_cast(
                  v4f, __builtin_amdgcn_raw_buffer_load_b128(rW, (int)(sp < S && sp != split ? poff(sp, t) : kOOB), 0, load_pol));
            }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int t = 0; t < IV * 4; ++t)
              if (sb0 + u < S) sum[t] += sb0 + u == split ? part[t] : pt[u][t];
        }
#pragma unroll
        for (int t = 0; t < IV * 4; ++t) store_c(t, sum[t]);
      };
      if constexpr (RED == 1) {
        // ticket first: all but the last store their partials and count themselves
        // ready; the last waits for that, then sums (device-coherent accesses)
        if (tid == 0) s_ticket = (int)__hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const int ticket = s_ticket;
        if (ticket < S - 1) {
#pragma unroll
          for (int t = 0; t < IV * 4; ++t)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, part[t]), rW, (int)poff(split, t), 0, kSC1);
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
          __syncthreads();
          if (tid == 0) __hip_atomic_fetch_add(cnt + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          return;
        }
        if (tid == 0) {
          for (int it = 0; it < (1 << 24); ++it) {
            if (__hip_atomic_load(cnt + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)(S - 1)) break;
            __builtin_amdgcn_s_sleep(1);
          }
          __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(cnt + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __syncthreads();
        sum_and_store(IntC<kSC1>{});
      } else {
        // store first, then the ticket: the last to arrive finds every other partial
        // stored.  Mode 2 keeps the partials in the L2 of the XCD the tile's splits
        // share (plain stores, loads that skip only the CU cache) and checks from the
        // ticket that they did share one; mode 3 writes them through to memory.
        const uint32_t xcc = (uint32_t)__builtin_amdgcn_s_getreg((20) | (0 << 6) | ((4 - 1) << 11)) & 15u;
#pragma unroll
        for (int t = 0; t < IV * 4; ++t)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, part[t]), rW, (int)poff(split, t), 0,
                                                 RED == 2 ? 0 : kSC1);
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __syncthreads();
        // ticket word: arrivals in bits 0-3, arrivals per XCD in 3-bit fields from bit 4
        const uint32_t add = 1u | (xcc < 8 ? (1u << (4 + 3 * xcc)) : 0u);
        if (tid == 0) s_ticket = (int)__hip_atomic_fetch_add(cnt, add, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        const uint32_t all = (uint32_t)s_ticket + add;
        if ((int)(all & 15u) != S) return;
        if (tid == 0) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (RED == 2 && (xcc >= 8 || (int)((all >> (4 + 3 * xcc)) & 7u) != S)) {
          // the splits did not share an XCD: their partials are not all visible here
#pragma unroll
          for (int t = 0; t < IV * 4; ++t) {
            const float nanv = __uint_as_float(0x7FC00000u);
            store_c(t, v4f{nanv, nanv, nanv, nanv});
          }
          return;
        }
        sum_and_store(IntC<1>{});  // sc0: past the CU cache, from L2
      }
    }
  };
  if (rows_valid > 32) body(IntC<2>{});
  else body(IntC<1>{});
}

// Masked grouped GEMM on pre-shuffled weights by weight streaming (the decode
// kernel's scheme applied to each expert): one workgroup per (expert, 128-column
// tile) holds every valid row of its expert (up to RG 32-row groups) and runs the whole
// K, so each expert's weights are read exactly once, straight into MFMA operand
// registers D K-blocks ahead with non-temporal loads.  The expert's activation
// K-blocks (its valid rows only) go to LDS by DMA in groups of AG, one group ahead; the
// column tiles of an expert get workgroup ids congruent mod 8, so they run on one XCD
// and read those rows from its L2.  Results are the ring kernels' bits (same
// per-K-block scaled MFMAs in the same order).
template <int RG>
struct MwsdShape {
  static constexpr int AG = 2;               // K-blocks per activation group
  static constexpr int D = 4;                // weight K-blocks in flight per wavefront
  static constexpr int UN = 8;               // unroll: weight ring, group buffer and scale byte static
  static constexpr int WMAX = 16;            // scale words per row (K <= 8192)
  static constexpr int KBB = RG * 32 * 128;  // one activation K-block in LDS
  static constexpr int ASZ = AG * KBB;
};

template <int RG, bool NTC = false>
__global__ __launch_bounds__(256) void mwsd_kernel(const KArgs p) {
  using S_ = MwsdShape<RG>;
  constexpr int AG = S_::AG, D = S_::D, UN = S_::UN, WMAX = S_::WMAX, KBB = S_::KBB, ASZ = S_::ASZ;
  constexpr int HB = KBB / 2;   // one K-half of a K-block: RG * 32 rows x 64 bytes
  constexpr int ROWS = RG * 32;
  __shared__ __attribute__((aligned(1024))) uint8_t ab0[ASZ];
  __shared__ __attribute__((aligned(1024))) uint8_t ab1[ASZ];
  __shared__ __attribute__((aligned(16))) uint32_t sa_tab[WMAX * ROWS];  // [w][row]
  __shared__ __attribute__((aligned(16))) uint32_t sb_tab[WMAX];         // [w], byte kb % 4

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // workgroup -> (expert, column tile): ids of one expert are congruent mod 8 (one XCD);
  // the grid is padded to 8 ceil(E / 8) T workgroups (p.groups = E)
  const int id = blockIdx.x, T = p.tiles_n;
  const int jj = id >> 3;
  const int64_t e = (id & 7) + 8 * (jj / T);
  const int tn = jj - (jj / T) * T;
  if (e >= p.groups) return;
  const int64_t cnt = p.masked_m[e];
  const int count = (int)(cnt < 0 ? 0 : (cnt > p.M ? p.M : cnt));
  if (count == 0) return;  // nothing is read or written
  const int64_t n0 = (int64_t)tn * 128;
  const int KB = (int)(p.K / 128);
  const int nk4 = (KB + 3) & ~3;
  const int nfull = nk4 / UN * UN;
  const int NB = (int)((p.N + 127) / 128);
  int64_t cols_valid = p.N - n0;
  cols_valid = cols_valid > 128 ? 128 : cols_valid;
  const auto rA = make_rsrc(p.a + e * p.sa_e, (uint32_t)(count * p.K));
  const auto rB = make_rsrc(p.b + e * p.sb_e + n0 * p.K, (uint32_t)(cols_valid * p.K));
  const int Wd = (KB + 3) / 4;  // <= WMAX (host)
  const auto rSA = make_rsrc(p.sfa + e * p.ssfa_e, (uint32_t)(Wd * p.ld_sfa * 4));
  const auto rSB = make_rsrc(p.sfb + e * p.ssfb_e, (uint32_t)(NB * KB * 4));

  // activation DMA: wavefront w moves K-half w >> 1 of the 16-row blocks rb = 2 t + (w & 1)
  // of a K-block, one 1 KB instruction each; lane l -> row 16 rb + (l >> 2), LDS chunk
  // l & 3 holding chunk (l & 3) ^ swz64(row) of the K-half.  NT (a compile-time count)
  // bounds t by the valid 32-row groups; blocks at or past the count read nothing (their
  // offsets are out of range: no branch in the unrolled loop).
  const int hh = wave >> 1, rb0 = wave & 1;
  uint32_t aoff[RG];
#pragma unroll
  for (int t = 0; t < RG; ++t) {
    const int rb = 2 * t + rb0, r = rb * 16 + (lane >> 2);
    aoff[t] = (rb * 16 < count ? (uint32_t)(r * p.K) + (uint32_t)(hh * 64) + (uint32_t)((((lane & 3) ^ swz64(r)) << 4))
                               : kOOB);
  }
  auto dma_group = [&](int g, uint8_t* buf, auto nt_tag) {
    constexpr int NT = decltype(nt_tag)::value;
#pragma unroll
    for (int u = 0; u < AG; ++u) {
      const int j = g * AG + u;
      const uint32_t koff = (uint32_t)j * 128u, oob = j < KB ? 0u : kOOB;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint8_t* dst = buf + u * KBB + hh * HB + (2 * t + rb0) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rA, (__attribute__((address_space(3))) void*)dst, 16,
                                                 (int)((aoff[t] + koff) | oob), 0, 0, 0);
      }
    }
  };
  // weight loads of K-block j: lane l, 16 bytes at 1 KB steps (the 32-row group of this
  // wavefront in the pre-shuffled layout)
  const uint32_t boff = (uint32_t)(wave * 32 * p.K) + (uint32_t)(16 * lane);
  auto load_w = [&](int j, v4i (&w)[4]) {
    const uint32_t off = (boff + (uint32_t)j * 4096u) | (j < KB ? 0u : kOOB);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      w[q] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rB, (int)(off + 1024u * q), 0, kNT));
  };

  // scale tables: activation words of the valid rows (zero past the count and for the
  // bytes of K-blocks past K), weight exponent bytes of this tile's column block
  constexpr int SA_PT = (WMAX * ROWS + 255) / 256, SB_PT = (WMAX * 4 + 255) / 256;
  uint32_t sav[SA_PT], sbv[SB_PT];
  dma_group(0, ab0, IntC<RG>{});
#pragma unroll
  for (int t = 0; t < SA_PT; ++t) {
    const int idx = t * 256 + tid, w = idx / ROWS, row = idx % ROWS;
    const bool ok = idx < WMAX * ROWS && row < count && w < Wd;
    sav[t] = bload4(rSA, ok ? (uint32_t)(((int64_t)w * p.ld_sfa + row) * 4) : kOOB);
  }
#pragma unroll
  for (int t = 0; t < SB_PT; ++t) {
    const int idx = t * 256 + tid;
    const bool ok = idx < WMAX * 4 && idx < KB;
    sbv[t] = bload4(rSB, ok ? (uint32_t)(((n0 >> 7) * KB + idx) * 4) : kOOB);
  }
  v4i wr[D][4];
#pragma unroll
  for (int d = 0; d < D; ++d) load_w(d, wr[d]);
#pragma unroll
  for (int t = 0; t < SA_PT; ++t) {
    const int idx = t * 256 + tid, w = idx / ROWS;
    uint32_t v = sav[t];
    const int left = KB - 4 * w;
    if (left < 4) v &= left <= 0 ? 0u : ((1u << (8 * left)) - 1u);
    if (idx < WMAX * ROWS) sa_tab[idx] = v;
  }
  {
    uint8_t* sbb = reinterpret_cast<uint8_t*>(sb_tab);
#pragma unroll
    for (int t = 0; t < SB_PT; ++t) {
      const int idx = t * 256 + tid;
      if (idx < WMAX * 4) sbb[idx] = (uint8_t)((sbv[t] >> 23) & 0xFFu);
    }
  }
  // the first activation group and the tables in place everywhere (the weight loads
  // issued after them may still be in flight)
  __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * D, 0));
  __builtin_amdgcn_s_barrier();

  const int lr = lane & 31, c0 = 2 * (lane >> 5);
  const uint32_t rd0 = (uint32_t)(lr * 64 + ((c0 ^ swz64(lr)) << 4));
  const uint32_t rd1 = (uint32_t)(lr * 64 + (((c0 + 1) ^ swz64(lr)) << 4));
  uint16_t* __restrict__ C = p.c + e * p.sc_e;

  auto body = [&](auto iv_tag) {
    constexpr int IV = decltype(iv_tag)::value;  // 32-row groups with valid rows
    v16f acc[IV];
#pragma unroll
    for (int i = 0; i < IV; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][q] = 0.0f;
    uint32_t sa[IV], sb = 0;

    // iteration j = jb + U (jb a multiple of UN)
    auto iter = [&](int jb, auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      constexpr int OPS = U % 4, SLOT = U % D, GB = (U / AG) % 2, POS = U % AG;
      const int j = jb + U;
      if constexpr (POS == 0) {
        // a new activation group: its DMA (issued one group ago, followed by that
        // group's AG x 4 weight loads) has landed here and everywhere, and nobody
        // reads the other buffer any more: refill it with the next group
        __builtin_amdgcn_sched_barrier(0);
        if (j > 0) {
          __builtin_amdgcn_s_waitcnt(waitcnt_imm(4 * AG, 15));
          __builtin_amdgcn_s_barrier();
        }
        __builtin_amdgcn_sched_barrier(0);
        dma_group(j / AG + 1, GB == 0 ? ab1 : ab0, IntC<IV>{});
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (OPS == 0) {
#pragma unroll
        for (int i = 0; i < IV; ++i) sa[i] = sa_tab[(j >> 2) * ROWS + 32 * i + lr];
        sb = sb_tab[j >> 2];
      }
      const uint8_t* base = (GB == 0 ? ab0 : ab1) + POS * KBB;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        v8i af[IV];
#pragma unroll
        for (int i = 0; i < IV; ++i) {
          const uint32_t o = (uint32_t)(h * HB + i * 2048);
          const v4i lo = *reinterpret_cast<const v4i*>(base + (o + rd0));
          const v4i hi = *reinterpret_cast<const v4i*>(base + (o + rd1));
          af[i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
        const v8i bw = __builtin_shufflevector(wr[SLOT][2 * h], wr[SLOT][2 * h + 1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
        for (int i = 0; i < IV; ++i)
          acc[i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bw, af[i], acc[i], 0, 0, OPS, (int)sb, OPS,
                                                                   (int)sa[i]);
      }
      load_w(j + D, wr[SLOT]);  // the registers of j are free again: fetch j + D
      __builtin_amdgcn_sched_barrier(0);
    };
    for (int jb = 0; jb < nfull; jb += UN) {
      iter(jb, IntC<0>{}); iter(jb, IntC<1>{}); iter(jb, IntC<2>{}); iter(jb, IntC<3>{});
      iter(jb, IntC<4>{}); iter(jb, IntC<5>{}); iter(jb, IntC<6>{}); iter(jb, IntC<7>{});
    }
    // tail: the remaining K-blocks (four: nk4 - nfull is 0 or 4) continue the ring
    if (nk4 - nfull >= 4) { iter(nfull, IntC<0>{}); iter(nfull, IntC<1>{}); iter(nfull, IntC<2>{}); iter(nfull, IntC<3>{}); }
    // the loads issued past the range must land before the LDS is reused or released
#pragma unroll
    for (int d = 0; d < D; ++d) keep_issued4(wr[d]);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();

    // epilogue, 64 rows at a time: stage the wavefront's 64 x 32 fp32 block in LDS
    // (16-byte chunk c of row r at c ^ (r & 7)); lane l then holds 4 consecutive
    // columns of row 8 t + (l >> 3), stored as bf16 for the rows below the count
    float* so = reinterpret_cast<float*>(ab0 + wave * 64 * 128);
    const int ch = lane & 7;
    const int64_t n = n0 + wave * 32 + 4 * ch;
#pragma unroll
    for (int i0 = 0; i0 < IV; i0 += 2) {
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        if (i0 + ii < IV) {
          const int row = 32 * ii + lr;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int chunk = 2 * q + (lane >> 5);
            *reinterpret_cast<v4f*>(reinterpret_cast<uint8_t*>(so) + row * 128 + ((chunk ^ (row & 7)) << 4)) =
                v4f{acc[i0 + ii][4 * q], acc[i0 + ii][4 * q + 1], acc[i0 + ii][4 * q + 2], acc[i0 + ii][4 * q + 3]};
          }
        }
      }
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        const int row = t * 8 + (lane >> 3);
        const int64_t m = 64 * (i0 / 2) + row;
        if (row < 32 * (IV - i0) && m < count && n < p.N) {
          const v4f v = *reinterpret_cast<const v4f*>(reinterpret_cast<const uint8_t*>(so) + row * 128 +
                                                      ((ch ^ (row & 7)) << 4));
          uint2 o;
          o.x = bf16_rne(v[0]) | (bf16_rne(v[1]) << 16);
          o.y = bf16_rne(v[2]) | (bf16_rne(v[3]) << 16);
          // NTC: streaming stores, so that C does not stand in the weight stream's way through
          // the caches (masked gate_up 195-198 -> 186.5-187 us)
          if constexpr (NTC)
            __builtin_nontemporal_store(((uint64_t)o.y << 32) | o.x, reinterpret_cast<uint64_t*>(C + m * p.ldc + n));
          else *reinterpret_cast<uint2*>(C + m * p.ldc + n) = o;
        }
      }
    }
  };
  const int iv = __builtin_amdgcn_readfirstlane((count + 31) / 32);
  switch (iv) {
    case 1: body(IntC<1>{}); break;
    case 2: if constexpr (RG >= 2) body(IntC<2 <= RG ? 2 : RG>{}); break;
    case 3: if constexpr (RG >= 3) body(IntC<3 <= RG ? 3 : RG>{}); break;
    case 4: if constexpr (RG >= 4) body(IntC<4 <= RG ? 4 : RG>{}); break;
    case 5: if constexpr (RG >= 5) body(IntC<5 <= RG ? 5 : RG>{}); break;
    case 6: if constexpr (RG >= 6) body(IntC<6 <= RG ? 6 : RG>{}); break;
    case 7: if constexpr (RG >= 7) body(IntC<7 <= RG ? 7 : RG>{}); break;
    default: if constexpr (RG >= 8) body(IntC<8 <= RG ? 8 : RG>{}); break;
  }
}

// ---------------------------------------------------------------------------
// compiled tile table

typedef void (*KernelFn)(const KArgs);

enum Kind { kTile = 0, kStream = 1, kScaled = 2, kRing = 3, kDecode = 4, kTileFloat = 5, kDecodeFloat = 6,
            kScaledFloat = 7, kDecodeSep = 8, kDecodeShuf = 9, kDecodeShufSep = 10, kRingShuf = 11,
            kDecodeFloatShuf = 12, kDecodeFloatSep = 13, kDecodeFloatShufSep = 14, kWsd = 15, kWsdSep = 16,
            kRingFloat = 17, kMwsd = 18 };

// Weight-streaming decode entries (pre-shuffled weights, dense M <= 64, 1-D grid).
inline bool is_wsd(int kind) { return kind == kWsd || kind == kWsdSep; }

// Entries that read the float-scale format.
inline bool reads_float_scales(int kind) {
  return kind == kTileFloat || kind == kDecodeFloat || kind == kScaledFloat || kind == kDecodeFloatShuf ||
         kind == kDecodeFloatSep || kind == kDecodeFloatShufSep || kind == kRingFloat;
}
// LDS-DMA tile entries (dynamic LDS for the scale tables).
inline bool is_scaled_tile(int kind) { return kind == kScaled || kind == kScaledFloat; }
// Entries that reduce their own K split (arrival counters in the workspace).
inline bool reduces_in_kernel(int kind) {
  return kind == kDecode || kind == kDecodeFloat || kind == kDecodeShuf || kind == kDecodeFloatShuf || kind == kWsd;
}
// Entries that read the weights in the pre-shuffled layout.
inline bool reads_shuffled(int kind) {
  return kind == kDecodeShuf || kind == kDecodeShufSep || kind == kRingShuf || kind == kDecodeFloatShuf ||
         kind == kDecodeFloatShufSep || is_wsd(kind) || kind == kMwsd;
}
// Ring entries (K never split; the scale tables bound K).
inline bool is_ring(int kind) { return kind == kRing || kind == kRingShuf || kind == kRingFloat; }
// Decode-kernel entries (K split in whole scale words; the *Sep kinds leave the sum of
// the partials to splitk_reduce_kernel).
inline bool is_decode(int kind) {
  return reduces_in_kernel(kind) || kind == kDecodeSep || kind == kDecodeShufSep || kind == kDecodeFloatSep ||
         kind == kDecodeFloatShufSep || is_wsd(kind);
}

struct TileEntry {
  KernelFn fn;
  int bm, bn;
  int kind;    // kTile: both operands via LDS (VALU scale FMA); kStream: weight streaming;
               // kScaled: LDS-DMA tiles + scaled MFMA (no K split)
  int stages;  // LDS ring depth of kScaled / kRing
  int threads;  // workgroup size
  int max_wd;   // kRing: most activation-scale words per row (K-blocks / 4) its tables hold
                // (kRingFloat: most K-blocks, one fp32 each);
                // kDecode: the same per K split
};

const TileEntry kTiles[] = {
    {gemm_kernel<64, 128, 64, 32>, 64, 128, kTile, 2, 256},
    {gemm_kernel<128, 128, 64, 64>, 128, 128, kTile, 2, 256},
    {gemm_kernel<64, 256, 64, 64>, 64, 256, kTile, 2, 256},
    {gemm_kernel<128, 256, 64, 128>, 128, 256, kTile, 2, 256},
    {stream_kernel<4, 2, 4>, 64, 128, kStream, 0, 256},
    {stream_kernel<4, 1, 4>, 64, 64, kStream, 0, 256},
    {stream_kernel<1, 2, 4>, 16, 128, kStream, 0, 256},
    {stream_kernel<2, 2, 4>, 32, 128, kStream, 0, 256},
    {stream_kernel<4, 1, 8>, 64, 64, kStream, 0, 256},
    {stream_kernel<4, 2, 6>, 64, 128, kStream, 0, 256},
    {scaled_tile_kernel<256, 256, 2, 2, 2>, 256, 256, kScaled, 2, 256},
    {scaled_tile_kernel<128, 256, 2, 2, 2>, 128, 256, kScaled, 2, 256},
    {scaled_tile_kernel<256, 128, 2, 2, 2>, 256, 128, kScaled, 2, 256},
    {scaled_tile_kernel<128, 128, 2, 2, 2>, 128, 128, kScaled, 2, 256},
    {scaled_tile_kernel<256, 256, 2, 4, 2>, 256, 256, kScaled, 2, 512},
    {scaled_tile_kernel<256, 256, 4, 2, 2>, 256, 256, kScaled, 2, 512},
    {scaled_tile_kernel<256, 128, 4, 2, 2>, 256, 128, kScaled, 2, 512},
    {scaled_ring_kernel<256, 256, 2, 2>, 256, 256, kRing, 4, 256, ring_wd_max<256, 256, 2, 2>()},
    {scaled_ring_kernel<256, 128, 2, 2>, 256, 128, kRing, 4, 256, ring_wd_max<256, 128, 2, 2>()},
    {scaled_ring_kernel<128, 256, 2, 2>, 128, 256, kRing, 4, 256, ring_wd_max<128, 256, 2, 2>()},
    {scaled_ring_kernel<256, 256, 1, 4>, 256, 256, kRing, 4, 256, ring_wd_max<256, 256, 1, 4>()},
    {scaled_ring_kernel<128, 256, 1, 4>, 128, 256, kRing, 4, 256, ring_wd_max<128, 256, 1, 4>()},
    {decode_kernel<4, 3>, 64, 128, kDecode, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<8, 2>, 64, 256, kDecode, 2, 512, DecodeShape<8, 2>::WMAX},
    {decode_kernel<4, 2>, 64, 128, kDecode, 2, 256, DecodeShape<4, 2>::WMAX},
    {decode_kernel<8, 3>, 64, 256, kDecode, 3, 512, DecodeShape<8, 3>::WMAX},
    {gemm_kernel<64, 128, 64, 32, true>, 64, 128, kTileFloat, 2, 256},
    {gemm_kernel<128, 128, 64, 64, true>, 128, 128, kTileFloat, 2, 256},
    {gemm_kernel<64, 256, 64, 64, true>, 64, 256, kTileFloat, 2, 256},
    {gemm_kernel<128, 256, 64, 128, true>, 128, 256, kTileFloat, 2, 256},
    // float scales: one fp32 per K-block in the tables, so WMAX K-blocks per split
    {decode_kernel<4, 3, true>, 64, 128, kDecodeFloat, 3, 256, DecodeShape<4, 3>::WMAX / 4},
    {scaled_tile_kernel<128, 128, 2, 2, 2, true>, 128, 128, kScaledFloat, 2, 256},
    {scaled_tile_kernel<128, 256, 2, 2, 2, true>, 128, 256, kScaledFloat, 2, 256},
    {decode_kernel<8, 3>, 64, 256, kDecodeSep, 3, 512, DecodeShape<8, 3>::WMAX},
    {decode_kernel<4, 3>, 64, 128, kDecodeSep, 3, 256, DecodeShape<4, 3>::WMAX},
    // pre-shuffled weights
    {decode_kernel<4, 3, false, true>, 64, 128, kDecodeShuf, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<4, 3, false, true>, 64, 128, kDecodeShufSep, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<8, 3, false, true>, 64, 256, kDecodeShufSep, 3, 512, DecodeShape<8, 3>::WMAX},
    {scaled_ring_kernel<256, 256, 1, 4, true>, 256, 256, kRingShuf, 4, 256, ring_wd_max<256, 256, 1, 4>()},
    {scaled_ring_kernel<256, 256, 2, 2, true>, 256, 256, kRingShuf, 4, 256, ring_wd_max<256, 256, 2, 2>()},
    {scaled_ring_kernel<128, 256, 2, 2, true>, 128, 256, kRingShuf, 4, 256, ring_wd_max<128, 256, 2, 2>()},
    {decode_kernel<4, 3, true, true>, 64, 128, kDecodeFloatShuf, 3, 256, DecodeShape<4, 3>::WMAX / 4},
    // weights through LDS (whole 128-byte rows per DMA instruction) on the plain layout
    {decode_kernel<4, 4, false, false, true>, 64, 128, kDecode, 4, 256, DecodeShape<4, 4>::WMAX},
    {decode_kernel<4, 3, false, false, true>, 64, 128, kDecode, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<4, 3, true, false, true>, 64, 128, kDecodeFloat, 3, 256, DecodeShape<4, 3>::WMAX / 4},
    {decode_kernel<4, 3, false, false, true>, 64, 128, kDecodeSep, 3, 256, DecodeShape<4, 3>::WMAX},
    // float scales, partials summed by splitk_reduce_kernel: weights through LDS / pre-shuffled
    {decode_kernel<4, 3, true, false, true>, 64, 128, kDecodeFloatSep, 3, 256, DecodeShape<4, 3>::WMAX / 4},
    {decode_kernel<4, 3, true, true>, 64, 128, kDecodeFloatShufSep, 3, 256, DecodeShape<4, 3>::WMAX / 4},
    {scaled_ring_kernel<128, 128, 2, 2>, 128, 128, kRing, 4, 256, ring_wd_max<128, 128, 2, 2>()},
    {scaled_ring_kernel<128, 128, 1, 4>, 128, 128, kRing, 4, 256, ring_wd_max<128, 128, 1, 4>()},
    {scaled_ring_kernel<128, 128, 2, 2, true>, 128, 128, kRingShuf, 4, 256, ring_wd_max<128, 128, 2, 2>()},
    // weights loaded non-temporally (streamed past the caches)
    {decode_kernel<4, 3, false, true, false, true>, 64, 128, kDecodeShufSep, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<4, 3, false, false, true, true>, 64, 128, kDecodeSep, 3, 256, DecodeShape<4, 3>::WMAX},
    {decode_kernel<8, 3, false, true, false, true>, 64, 256, kDecodeShufSep, 3, 512, DecodeShape<8, 3>::WMAX},
    {decode_kernel<4, 2, false, true, false, true>, 64, 128, kDecodeShufSep, 2, 256, DecodeShape<4, 2>::WMAX},
    // weight streaming: registers D K-blocks ahead, activation groups, split summed in the kernel or not
    {wsd_kernel<4, 1>, 64, 128, kWsd, 4, 256, WsdShape<4, 1>::WMAX},
    {wsd_kernel<4, 2>, 64, 128, kWsd, 4, 256, WsdShape<4, 2>::WMAX},
    {wsd_kernel<4, 3>, 64, 128, kWsd, 4, 256, WsdShape<4, 3>::WMAX},
    {wsd_kernel<4, 0>, 64, 128, kWsdSep, 4, 256, WsdShape<4, 0>::WMAX},
    {wsd_kernel<3, 2>, 64, 128, kWsd, 3, 256, WsdShape<3, 2>::WMAX},
    // ring tiles with the operand reads front-loaded in each half-step
    {scaled_ring_kernel<256, 256, 2, 2, false, 1>, 256, 256, kRing, 4, 256, ring_wd_max<256, 256, 2, 2>()},
    {scaled_ring_kernel<256, 128, 2, 2, false, 1>, 256, 128, kRing, 4, 256, ring_wd_max<256, 128, 2, 2>()},
    {scaled_ring_kernel<128, 128, 1, 4, false, 1>, 128, 128, kRing, 4, 256, ring_wd_max<128, 128, 1, 4>()},
    // full-row stages: one L2 request per 128-byte line
    {ring2_kernel<256, 256, 2, 2, 2>, 256, 256, kRing, 2, 256, ring2_wd_max<256, 256, 2, 2, 2>()},
    {ring2_kernel<256, 128, 2, 2, 2>, 256, 128, kRing, 2, 256, ring2_wd_max<256, 128, 2, 2, 2>()},
    // (128x128: chosen for one round of tiles only, so C goes out with streaming stores; 2 x 2
    // wavefronts read 64 KB of operands from LDS per K-block against 80 KB for 1 x 4:
    // 2048x2048x7168 33.2 -> 32.5 us, 1024x4096x7168 36.7 -> 36.3 us)
    {ring2_kernel<128, 128, 2, 2, 4, false, false, false, true>, 128, 128, kRing, 4, 256, ring2_wd_max<128, 128, 2, 2, 4>()},
    {ring2_kernel<128, 256, 2, 2, 2>, 128, 256, kRing, 2, 256, ring2_wd_max<128, 256, 2, 2, 2>()},
    {ring2_kernel<256, 256, 1, 4, 2>, 256, 256, kRing, 2, 256, ring2_wd_max<256, 256, 1, 4, 2>()},
    // float scales: the full-row 128x128 ring, unscaled MFMAs, block partials scaled on the VALU
    // (C with streaming stores: 2048x4096 to 2048x18432 (K 7168) 0.3-0.8% shorter)
    {ring2_kernel<128, 128, 1, 4, 4, true, false, false, true>, 128, 128, kRingFloat, 4, 256, ring2_wd_max<128, 128, 1, 4, 4, true>()},
    // masked: the full-row ring with the wavefronts side by side in N, weights streamed non-temporally
    // (the grouped GEMMs, bound by their weight streams, also store C with streaming stores)
    {ring2_kernel<256, 256, 1, 4, 2, false, true, false, true>, 256, 256, kRing, 2, 256, ring2_wd_max<256, 256, 1, 4, 2>()},
    // contiguous grouped: the same at 128-row tiles (one aligned run each)
    {ring2_kernel<128, 256, 1, 4, 2, false, true, false, true>, 128, 256, kRing, 2, 256, ring2_wd_max<128, 256, 1, 4, 2>()},
    // the full-row ring on pre-shuffled weights (dense 256x256 / 256x128 / 128x128, masked)
    {ring2_kernel<256, 256, 2, 2, 2, false, false, true>, 256, 256, kRingShuf, 2, 256, ring2_wd_max<256, 256, 2, 2, 2>()},
    {ring2_kernel<256, 128, 2, 2, 2, false, false, true>, 256, 128, kRingShuf, 2, 256, ring2_wd_max<256, 128, 2, 2, 2>()},
    {ring2_kernel<128, 128, 2, 2, 4, false, false, true, true>, 128, 128, kRingShuf, 4, 256, ring2_wd_max<128, 128, 2, 2, 4>()},
    {ring2_kernel<256, 256, 1, 4, 2, false, true, true, true>, 256, 256, kRingShuf, 2, 256, ring2_wd_max<256, 256, 1, 4, 2>()},
    // masked, pre-shuffled weights: weight streaming, every valid row of an expert per
    // workgroup (M_max <= 256), the whole K (K <= 8192)
    {mwsd_kernel<8, true>, 256, 128, kMwsd, 0, 256, MwsdShape<8>::WMAX},
    // three-stage 256x128 rings (DMA two K-blocks ahead; streaming stores of C), plain and
    // pre-shuffled weights
    {ring2_kernel<256, 128, 2, 2, 3, false, false, false, true>, 256, 128, kRing, 3, 256, ring2_wd_max<256, 128, 2, 2, 3>()},
    {ring2_kernel<256, 128, 2, 2, 3, false, false, true, true>, 256, 128, kRingShuf, 3, 256, ring2_wd_max<256, 128, 2, 2, 3>()},
    // contiguous grouped: the 128x256 ring with three stages
    {ring2_kernel<128, 256, 1, 4, 3, false, true, false, true>, 128, 256, kRing, 3, 256, ring2_wd_max<128, 256, 1, 4, 3>()},
    // one round of 256x256 tiles: the same with streaming stores of C, plain and pre-shuffled weights
    {ring2_kernel<256, 256, 2, 2, 2, false, false, false, true>, 256, 256, kRing, 2, 256, ring2_wd_max<256, 256, 2, 2, 2>()},
    {ring2_kernel<256, 256, 2, 2, 2, false, false, true, true>, 256, 256, kRingShuf, 2, 256, ring2_wd_max<256, 256, 2, 2, 2>()},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);
// table entries the automatic choice uses
constexpr int kCfgStream64x128 = 4;
constexpr int kCfgScaled128x128 = 13;
constexpr int kCfgScaled256x256 = 15;
// (the ring entries the automatic choice uses are the full-row ones: one L2 request
// per 128-byte line; 4096x4096x7168 99 -> 90 us, 2048x4096x7168 69 -> 64 us,
// 1024x4096x7168 45.5 -> 37.2 us against the K-half ring entries 17, 18, 49)
// The masked and contiguous grouped GEMMs, bound by their weight streams, keep the
// K-half ring (masked gate_up 214 against 217 us, contiguous 272.5 against 276 us).
constexpr int kCfgRing256x256 = 63;        // 2 x 2 wavefronts, two full K-block stages
constexpr int kCfgRing256x256Rows = 20;    // K-half ring, 1 x 4 wavefronts (all share the rows)
constexpr int kCfgRing2Masked = 69;        // full-row ring, 1 x 4 wavefronts, non-temporal weight DMA
constexpr int kCfgRing2Contiguous = 70;    // the same, 128 x 256 tiles
constexpr int kCfgRing128x256 = 19;        // K-half ring, 2 x 2 wavefronts, 128-row tiles
constexpr int kCfgRing256x128 = 64;        // 2 x 2 wavefronts, 128-column tiles, two full K-block stages
constexpr int kCfgFloat64x128 = 26;        // float-scale VALU-scaled tiles
constexpr int kCfgFloat128x128 = 27;
constexpr int kCfgFloat128x256 = 29;
constexpr int kCfgFloatDecode64x128 = 46;  // decode kernel, float scales, weights through LDS, reduction kernel
constexpr int kCfgFloatScaled128x128 = 31; // LDS-DMA tiles, float scales
constexpr int kCfgFloatScaled128x256 = 32;
constexpr int kCfgRingFloat128x128 = 68;   // full-row ring 128x128, float scales on the VALU
constexpr int kCfgDecode64x128 = 45;       // decode kernel, 4 wavefronts, weights through a 3-stage LDS ring,
                                           // partials summed by splitk_reduce_kernel
constexpr int kCfgShufDecode64x128 = 36;   // the same on pre-shuffled weights (register loads)
constexpr int kCfgWsd64x128 = 56;          // weight streaming, pre-shuffled, split summed within one XCD
constexpr int kCfgShufRing256x256Rows = 38;  // pre-shuffled weights: ring 256x256, 1 x 4 wavefronts
constexpr int kCfgShufRing256x256 = 39;      // 2 x 2 wavefronts
constexpr int kCfgShufRing128x256 = 40;
constexpr int kCfgFloatShufDecode64x128 = 47;  // float scales, pre-shuffled weights, reduction kernel
constexpr int kCfgRing128x128 = 65;          // ring 128x128, 2 x 2 wavefronts, four full K-block stages
constexpr int kCfgShufRing128x128 = 50;      // the same (2 x 2) on pre-shuffled weights
constexpr int kCfgShufRing2_256x256 = 71;    // full-row ring on pre-shuffled weights, 2 x 2 wavefronts
constexpr int kCfgShufRing2_256x128 = 72;
constexpr int kCfgShufRing2_128x128 = 73;    // 2 x 2 wavefronts, four stages
constexpr int kCfgShufRing2Masked = 74;      // 1 x 4 wavefronts, non-temporal weight DMA
constexpr int kCfgMwsd = 75;                 // masked weight streaming, all rows of an expert per workgroup
// three-stage rings (DMA two K-blocks ahead; their scale tables hold K <= 7680 / 15872)
constexpr int kCfgRing256x128S3 = 76;        // 2 x 2 wavefronts, plain weights
constexpr int kCfgShufRing2_256x128S3 = 77;  // the same on pre-shuffled weights
constexpr int kCfgRing2ContiguousS3 = 78;    // 128 x 256, 1 x 4 wavefronts, non-temporal weight DMA
constexpr int kCfgRing256x256NTC = 79;       // 256 x 256 with streaming stores of C (one round of tiles)
constexpr int kCfgShufRing2_256x256NTC = 80;  // the same on pre-shuffled weights
static_assert(kCfgDecode64x128 < kNumTiles && kCfgFloatScaled128x256 < kNumTiles, "tile table");
static_assert(kCfgRingFloat128x128 < kNumTiles && kCfgRing2Masked < kNumTiles && kCfgRing2Contiguous < kNumTiles,
              "tile table");
static_assert(kCfgFloatShufDecode64x128 < kNumTiles && kCfgFloatDecode64x128 < kNumTiles, "tile table");
static_assert(kCfgRing128x128 < kNumTiles && kCfgShufRing128x128 < kNumTiles, "tile table");
static_assert(kCfgRing256x256 < kNumTiles && kCfgRing256x256Rows < kNumTiles && kCfgRing128x256 < kNumTiles &&
                  kCfgRing256x128 < kNumTiles, "tile table");
static_assert(kCfgWsd64x128 < kNumTiles, "tile table");
static_assert(kCfgShufRing2_256x256 < kNumTiles && kCfgShufRing2_256x128 < kNumTiles &&
                  kCfgShufRing2_128x128 < kNumTiles && kCfgShufRing2Masked < kNumTiles && kCfgMwsd < kNumTiles,
              "tile table");
static_assert(kCfgRing256x128S3 < kNumTiles && kCfgShufRing2_256x128S3 < kNumTiles && kCfgRing2ContiguousS3 < kNumTiles &&
                  kCfgRing256x256NTC < kNumTiles && kCfgShufRing2_256x256NTC < kNumTiles,
              "tile table");

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

constexpr size_t kMaxLds = 160 * 1024 - 1024;  // gfx950 LDS per workgroup, less room for static LDS

// Dynamic LDS of a weight-streaming launch: two A stages, the activation-scale
// word table [sa_words][bm] and the weight-scale table [ceil(bn/128)][per].
inline size_t stream_lds_bytes(int bm, int bn, int per) {
  const int sa_words = (per + 3) / 4 + 1;
  return (size_t)2 * bm * LDS_ROW + (size_t)sa_words * bm * 4 + (size_t)((bn + 127) / 128) * per * 4;
}


}  // namespace

int gemm_config_count() { return kNumTiles; }

bool gemm_config_by_index(int idx, const GemmProblem& p, int splits, GemmConfig* out) {
  if (idx < 0 || idx >= kNumTiles || splits < 1) return false;
  const int KB = (int)(p.K / 128);
  if (splits > KB) splits = KB > 0 ? KB : 1;
  if ((p.masked_m || p.m_indices) && splits != 1) return false;
  // the float-scale format runs on the float-scale entries only (dense calls)
  if (reads_float_scales(kTiles[idx].kind) != p.float_scales) return false;
  if (p.float_scales && (p.masked_m || p.m_indices || p.E != 1)) return false;
  // pre-shuffled weights run on the entries that read that layout (dense calls)
  if (reads_shuffled(kTiles[idx].kind) != p.b_shuffled) return false;
  if (p.b_shuffled && p.m_indices) return false;
  // contiguous grouped layout: a tile must not straddle two aligned runs
  if (p.m_indices && kContiguousAlign % kTiles[idx].bm != 0) return false;
  if (is_ring(kTiles[idx].kind)) {
    splits = 1;  // never splits K; the scale tables bound K (words of four K-blocks, or
                 // one fp32 per K-block in the float-scale format)
    if ((kTiles[idx].kind == kRingFloat ? KB : (KB + 3) / 4) > kTiles[idx].max_wd) return false;
  }
  if (is_scaled_tile(kTiles[idx].kind)) {
    splits = 1;  // this family never splits K
    const bool fs = kTiles[idx].kind == kScaledFloat;
    if (scaled_tile_lds_bytes(kTiles[idx].bm, kTiles[idx].bn, kTiles[idx].stages, (int)p.K, fs) +
            scaled_tile_static_bytes(kTiles[idx].bm, kTiles[idx].bn, kTiles[idx].stages) >
        kMaxLds)
      return false;
  }
  if ((kTiles[idx].kind == kStream)) {
    // split K further if the scale tables would not fit next to the A stages
    while (splits < KB && stream_lds_bytes(kTiles[idx].bm, kTiles[idx].bn, (int)cdiv(KB, splits)) > kMaxLds) {
      if (p.masked_m || p.m_indices) return false;  // grouped layouts never split K
      ++splits;
    }
  }
  if (is_wsd(kTiles[idx].kind) && (p.M > 64 || p.E != 1 || p.masked_m || p.m_indices)) return false;
  if (kTiles[idx].kind == kMwsd) {
    // masked calls only; every row of an expert in one workgroup, the whole K in its tables
    if (!p.masked_m || p.M > kTiles[idx].bm || (KB + 3) / 4 > kTiles[idx].max_wd) return false;
    splits = 1;
  }
  if (is_decode(kTiles[idx].kind)) {
    // K-blocks per split: a multiple of four (whole words of packed scales, so the
    // scale byte of every unrolled iteration is static), at most four per word of
    // the scale table
    const bool in_kernel = reduces_in_kernel(kTiles[idx].kind);
    // (the weight-streaming kernel's arrival word counts at most seven splits per XCD)
    const int max_splits = kTiles[idx].kind == kWsd ? 7 : in_kernel ? kDecodeMaxSplits : kDecodeSepMaxSplits;
    if (splits > max_splits) splits = max_splits;
    int per = (int)cdiv(cdiv(KB, splits), 4) * 4;
    if (per > 4 * kTiles[idx].max_wd) {
      if (p.masked_m || p.m_indices) return false;  // grouped layouts never split K
      per = 4 * kTiles[idx].max_wd;
    }
    const int64_t tiles = cdiv(p.M, kTiles[idx].bm) * cdiv(p.N, kTiles[idx].bn);
    if (cdiv(KB, per) > 1 &&
        (cdiv(KB, per) > max_splits || (in_kernel && tiles > kCounterBytes / 8) ||
         cdiv(KB, per) * p.M * p.N * 4 > 0x7FFFFFFF))
      return false;
    out->kernel = idx;
    out->bm = kTiles[idx].bm;
    out->bn = kTiles[idx].bn;
    out->kb_per_split = per;
    out->splits = (int)cdiv(KB, per);
    return true;
  }
  out->kernel = idx;
  out->bm = kTiles[idx].bm;
  out->bn = kTiles[idx].bn;
  // normalise so that every split owns at least one K-block
  const int per = (int)cdiv(KB, splits);
  out->kb_per_split = per > 0 ? per : 1;
  out->splits = per > 0 ? (int)cdiv(KB, per) : 1;
  return true;
}

GemmConfig choose_gemm_config(const GemmProblem& p) {
  GemmConfig cfg;
  const int KB = (int)(p.K / 128);
  if (p.b_shuffled && p.float_scales) {
    // float scales on pre-shuffled weights: the float-scale decode kernel, K split
    // until about 224 workgroups (the only entry reading both)
    const int64_t tiles = cdiv(p.M, 64) * cdiv(p.N, kTiles[kCfgFloatShufDecode64x128].bn);
    int splits = (int)(224 / (tiles > 0 ? tiles : 1));
    if (splits < 1) splits = 1;
    if (!gemm_config_by_index(kCfgFloatShufDecode64x128, p, splits, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  if (p.b_shuffled) {
    // pre-shuffled weights (256 x 128 ring tiles with three stages where their tables
    // hold K, as for the plain layout: 2048x4096x7168 63.2 -> 54.9 us).  Masked: weight
    // streaming with every valid row of an expert
    // in one workgroup when M_max <= 256 and K <= 8192 (MoE down 124.5 -> 113.8 us, gate_up
    // 192.7 -> 193.4 us against the full-row ring), else the 256 x 256 full-row ring with
    // the wavefronts side by side in N and non-temporal weight DMA.  Dense
    // M <= 64: the weight-streaming kernel (below).  Larger M: the full-row ring
    // tiles chosen as for the plain layout (the layout only changes where a B stage's
    // kilobytes come from); the K-half ring tiles when K is past the full-row ring's
    // tables, the decode kernel past those.
    if (p.masked_m) {
      if (gemm_config_by_index(kCfgMwsd, p, 1, &cfg)) return cfg;
      if (gemm_config_by_index(kCfgShufRing2Masked, p, 1, &cfg)) return cfg;
      if (gemm_config_by_index(kCfgShufRing256x256Rows, p, 1, &cfg)) return cfg;
    } else if (p.M > 64) {
      const int64_t tm256 = cdiv(p.M, 256), big_tiles = tm256 * cdiv(p.N, 256);
      const int64_t mid_tiles = tm256 * cdiv(p.N, 128);
      const bool one_round_128 = cdiv(p.M, 128) * cdiv(p.N, 128) <= 256;
      // one round of 256 x 256 tiles: the entry with streaming stores of C
      if (big_tiles == 256 && gemm_config_by_index(kCfgShufRing2_256x256NTC, p, 1, &cfg)) return cfg;
      if (big_tiles >= 256 && gemm_config_by_index(kCfgShufRing2_256x256, p, 1, &cfg)) {
        // a last round of at most half the compute units: its columns in a second
        // launch, as for the plain layout (a 32-row group of the layout is 32 K
        // contiguous bytes, so the column offset of the tail is the plain one)
        const int64_t rem = big_tiles % 256;
        if (rem != 0 && rem <= 128 && p.E == 1) {
          const int64_t n_split = (big_tiles / 256) * 256 / tm256 * 256;
          GemmProblem tp = p;
          tp.N = p.N - n_split;
          GemmConfig tc;
          const bool one_round = cdiv(tp.M, 128) * cdiv(tp.N, 128) <= 256;
          const bool one_round_mid = cdiv(tp.M, 256) * cdiv(tp.N, 128) <= 256;
          if (n_split > 0 && n_split < p.N &&
              ((one_round && gemm_config_by_index(kCfgShufRing2_128x128, tp, 1, &tc)) ||
               (one_round_mid && (gemm_config_by_index(kCfgShufRing2_256x128S3, tp, 1, &tc) ||
                                  gemm_config_by_index(kCfgShufRing2_256x128, tp, 1, &tc))))) {
            cfg.n_split = n_split;
            cfg.tail_kernel = tc.kernel;
            cfg.tail_bm = tc.bm;
            cfg.tail_bn = tc.bn;
            cfg.tail_kb_per_split = tc.kb_per_split;
          }
        }
        return cfg;
      }
      if (mid_tiles >= 256 && (mid_tiles % 256 == 0 || mid_tiles % 256 > 128) &&
          (gemm_config_by_index(kCfgShufRing2_256x128S3, p, 1, &cfg) ||
           gemm_config_by_index(kCfgShufRing2_256x128, p, 1, &cfg)))
        return cfg;
      if (one_round_128 && gemm_config_by_index(kCfgShufRing2_128x128, p, 1, &cfg)) return cfg;
      if (mid_tiles <= 256 && (gemm_config_by_index(kCfgShufRing2_256x128S3, p, 1, &cfg) ||
                               gemm_config_by_index(kCfgShufRing2_256x128, p, 1, &cfg)))
        return cfg;
      // K past the full-row ring's tables: the K-half ring tiles
      if (one_round_128 && gemm_config_by_index(kCfgShufRing128x128, p, 1, &cfg)) return cfg;
      if (gemm_config_by_index(big_tiles >= 256 ? kCfgShufRing256x256 : kCfgShufRing128x256, p, 1, &cfg))
        return cfg;
    }
    const int64_t tiles = cdiv(p.M, kTiles[kCfgShufDecode64x128].bm) * cdiv(p.N, kTiles[kCfgShufDecode64x128].bn);
    int splits = p.masked_m ? 1 : (int)(224 / (tiles > 0 ? tiles : 1));
    if (splits < 1) splits = 1;
    // dense M <= 64: the weight-streaming kernel, its K split summed in the kernel
    // within one XCD's L2 (64x7168x18432: 29.7 us per call against 30.5 us for the
    // decode kernel and the reduction kernel)
    if (!p.masked_m && p.M <= 64 && gemm_config_by_index(kCfgWsd64x128, p, splits, &cfg)) return cfg;
    if (!gemm_config_by_index(kCfgShufDecode64x128, p, splits, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  if (p.float_scales) {
    // float-scale format: VALU-scaled tiles; small M splits K until about 224
    // workgroups, large M takes 128 x 256 tiles once they fill the compute units
    if (p.M <= 64) {
      {
        const int64_t tiles = cdiv(p.N, kTiles[kCfgFloatDecode64x128].bn);
        int splits = (int)(224 / (tiles > 0 ? tiles : 1));
        if (splits < 1) splits = 1;
        if (gemm_config_by_index(kCfgFloatDecode64x128, p, splits, &cfg)) return cfg;
      }
      const int64_t tiles = cdiv(p.N, kTiles[kCfgFloat64x128].bn);
      int splits = (int)(224 / (tiles > 0 ? tiles : 1));
      const int max_splits = KB / 4 > 1 ? KB / 4 : 1;
      if (splits > max_splits) splits = max_splits;
      if (splits < 1) splits = 1;
      if (!gemm_config_by_index(kCfgFloat64x128, p, splits, &cfg)) cfg.kernel = -1;
      return cfg;
    }
    // larger M: the full-row 128 x 128 ring with the scales on the VALU when its
    // tables hold K (1024x4096x7168: 71.2 -> 41.8 us, 4096x4096x7168: 231 -> 165 us,
    // 2048x18432x7168: 586 -> 369 us against the LDS-DMA 128 x 128 / 128 x 256 tiles);
    // else LDS-DMA tiles (128 x 256 once they fill the compute units), the VALU-scaled
    // register-staged tiles when no scale table fits
    if (gemm_config_by_index(kCfgRingFloat128x128, p, 1, &cfg)) return cfg;
    const int64_t t256 = cdiv(p.M, 128) * cdiv(p.N, 256);
    if (t256 >= 256 && gemm_config_by_index(kCfgFloatScaled128x256, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgFloatScaled128x128, p, 1, &cfg)) return cfg;
    if (!gemm_config_by_index(t256 >= 256 ? kCfgFloat128x256 : kCfgFloat128x128, p, 1, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  if (p.m_indices) {
    // contiguous grouped layout: 128-row tiles (one aligned run each); the full-row
    // 128 x 256 ring with non-temporal weight DMA, three stages when its tables hold K
    // (gate_up workload: 273 -> 247 us against the K-half 128 x 256 ring, 247 -> 215.5 us
    // with the third stage), the K-half ring when K is past its tables, then the
    // 128 x 128 scaled tiles
    if (gemm_config_by_index(kCfgRing2ContiguousS3, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgRing2Contiguous, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgRing128x256, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgScaled128x128, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgStream64x128, p, 1, &cfg)) return cfg;
    if (!gemm_config_by_index(1, p, 1, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  if (p.masked_m) {
    // 256 x 256 ring tiles with the four wavefronts side by side in N: a group's
    // weights are read once per column tile, and a group's valid rows are spread
    // over all four SIMDs (no operand reads or MFMAs for 32-row groups past the
    // count).  The full-row ring with non-temporal weight DMA first (the weights are
    // streamed once: MoE gate_up 213.4 -> 198.3 us, down 123.4 -> 117.3 us against
    // the K-half ring; with ordinary DMA the two rings are within 1.5%; streaming stores of
    // C: 199 -> 193 us, 120 -> 115 us), the K-half
    // ring when K is past its tables, weight streaming over 64-row tiles past both
    if (gemm_config_by_index(kCfgRing2Masked, p, 1, &cfg)) return cfg;
    if (gemm_config_by_index(kCfgRing256x256Rows, p, 1, &cfg)) return cfg;
    if (!gemm_config_by_index(kCfgStream64x128, p, 1, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  if (p.M <= 64) {
    // decode: weight streaming over 128-column tiles, weights and activations through
    // an LDS ring (whole 128-byte weight rows per DMA instruction: 36.9 -> 33.1 us at
    // 64x7168x18432 against operand-layout register loads), K split until about 224
    // workgroups and the partials summed by splitk_reduce_kernel (0.9 us shorter per
    // call and per graph-replayed step than the reduction by the last split)
    {
      const int64_t tiles = cdiv(p.N, kTiles[kCfgDecode64x128].bn);
      int splits = (int)(224 / (tiles > 0 ? tiles : 1));
      if (splits < 1) splits = 1;
      if (gemm_config_by_index(kCfgDecode64x128, p, splits, &cfg)) return cfg;
    }
    const int idx = kCfgStream64x128;
    const int64_t tiles = cdiv(p.N, kTiles[idx].bn);
    int splits = (int)(224 / (tiles > 0 ? tiles : 1));
    const int max_splits = KB / 8 > 1 ? KB / 8 : 1;
    if (splits > max_splits) splits = max_splits;
    if (splits < 1) splits = 1;
    if (!gemm_config_by_index(idx, p, splits, &cfg)) cfg.kernel = -1;
    return cfg;
  }
  // prefill: LDS-DMA tiles + scaled MFMA.  256x256 ring tiles once they fill the
  // compute units (the 8-wavefront two-stage kernel when K is past the ring's
  // scale tables), 128x128 tiles (two workgroups per compute unit) below that;
  // the VALU-scaled tile kernel when no scale table fits
  const int64_t tm256 = cdiv(p.M, 256), tn256 = cdiv(p.N, 256), big_tiles = tm256 * tn256;
  // one round of 256x256 tiles: the entry with streaming stores of C (4096x4096x7168 89.0 ->
  // 88.1 us); several rounds keep ordinary stores (4096x16384x7168: 345 against 346 us)
  if (big_tiles == 256 && gemm_config_by_index(kCfgRing256x256NTC, p, 1, &cfg)) return cfg;
  if (big_tiles >= 256 && gemm_config_by_index(kCfgRing256x256, p, 1, &cfg)) {
    // With 256x256 tiles, one per compute unit at a time, a last round of at most
    // half the compute units would leave the rest idle for a whole tile time: run
    // the leading columns in whole rounds and the remaining columns with smaller
    // tiles in a second launch: the 128x128 ring when its tiles make at most one
    // round, else the 256x128 ring when its tiles do (4096x18432x7168: the 4096x2048
    // tail 80 -> ~64 us against 512 two-stage 128x128 tiles at 35% MFMA use), else
    // the two-stage 128x128 tiles (two per compute unit).
    const int64_t rem = big_tiles % 256;
    if (rem != 0 && rem <= 128 && p.E == 1 && !p.masked_m && !p.m_indices) {
      const int64_t lead_tn = (big_tiles / 256) * 256 / tm256;
      const int64_t n_split = lead_tn * 256;
      GemmProblem tp = p;
      tp.N = p.N - n_split;
      GemmConfig tc;
      const bool one_round = cdiv(tp.M, 128) * cdiv(tp.N, 128) <= 256;
      const bool one_round_mid = cdiv(tp.M, 256) * cdiv(tp.N, 128) <= 256;
      if (n_split > 0 && n_split < p.N &&
          ((one_round && gemm_config_by_index(kCfgRing128x128, tp, 1, &tc)) ||
           (one_round_mid && (gemm_config_by_index(kCfgRing256x128S3, tp, 1, &tc) ||
                              gemm_config_by_index(kCfgRing256x128, tp, 1, &tc))) ||
           gemm_config_by_index(kCfgScaled128x128, tp, 1, &tc))) {
        cfg.n_split = n_split;
        cfg.tail_kernel = tc.kernel;
        cfg.tail_bm = tc.bm;
        cfg.tail_bn = tc.bn;
        cfg.tail_kb_per_split = tc.kb_per_split;
      }
    }
    return cfg;
  }
  if (big_tiles >= 256 && gemm_config_by_index(kCfgScaled256x256, p, 1, &cfg)) return cfg;
  // 256x128 ring tiles when they fill whole rounds of the compute units, or leave a
  // last round more than half full (2048x4096x7168: 67.5 us against 70.5 us for the
  // 128x128 tiles below), with three stages when the tables hold K: at one tile per
  // compute unit the ring waits on its DMA, and the third stage issues it two K-blocks
  // ahead instead of one (2048x4096x7168: 64.8 -> 54.4 us)
  const int64_t mid_tiles = tm256 * cdiv(p.N, 128);
  if (mid_tiles >= 256 && (mid_tiles % 256 == 0 || mid_tiles % 256 > 128) &&
      (gemm_config_by_index(kCfgRing256x128S3, p, 1, &cfg) || gemm_config_by_index(kCfgRing256x128, p, 1, &cfg)))
    return cfg;
  // at most one round of 128x128 tiles: the 128x128 ring, four K-blocks in flight
  // (1024x4096x7168: 63.2 -> 45.0 us against the two-stage tiles); more: the
  // two-stage tiles, two per compute unit (the ring is slower there: 2048x4096x7168
  // 87.7 us against 66.2 us for 256x128 ring tiles)
  if (cdiv(p.M, 128) * cdiv(p.N, 128) <= 256 && gemm_config_by_index(kCfgRing128x128, p, 1, &cfg)) return cfg;
  // more than one round of 128x128 tiles but at most one of 256x128: the 256x128 ring,
  // one tile per compute unit (against the two-stage 128x128 tiles: 1024x7168x7168
  // 73.8 -> 66.4 us, 1536x4096x7168 64.9 -> 61.2 us, 768x8192x7168 68.2 -> 64.3 us)
  if (mid_tiles <= 256 &&
      (gemm_config_by_index(kCfgRing256x128S3, p, 1, &cfg) || gemm_config_by_index(kCfgRing256x128, p, 1, &cfg)))
    return cfg;
  if (gemm_config_by_index(kCfgScaled128x128, p, 1, &cfg)) return cfg;
  const int idx = 1;
  const int64_t tiles = cdiv(p.M, kTiles[idx].bm) * cdiv(p.N, kTiles[idx].bn);
  int splits = 1;
  if (tiles < 256) {
    splits = (int)cdiv(512, tiles);
    const int max_splits = KB / 8 > 1 ? KB / 8 : 1;
    if (splits > max_splits) splits = max_splits;
  }
  if (!gemm_config_by_index(idx, p, splits, &cfg)) cfg.kernel = -1;
  return cfg;
}

size_t gemm_workspace_bytes(const GemmProblem& p, const GemmConfig& cfg) {
  if (cfg.splits <= 1) return 0;
  return (size_t)kCounterBytes + (size_t)cfg.splits * (size_t)p.M * (size_t)p.N * sizeof(float);
}

size_t gemm_workspace_zeroed_prefix() { return (size_t)kCounterBytes; }

hipError_t launch_gemm(const GemmProblem& p, const GemmConfig& cfg, void* ws, hipStream_t stream) {
  if (cfg.kernel < 0 || cfg.kernel >= kNumTiles) return hipErrorInvalidValue;
  if (cfg.n_split > 0) {
    // column split: [0, n_split) with cfg's kernel, [n_split, N) with the tail entry
    if (p.E != 1 || p.masked_m || p.m_indices || cfg.n_split % 128 != 0 || cfg.n_split >= p.N)
      return hipErrorInvalidValue;
    GemmProblem lead = p;
    lead.N = cfg.n_split;
    GemmConfig lc = cfg;
    lc.n_split = 0;
    hipError_t e = launch_gemm(lead, lc, ws, stream);
    if (e != hipSuccess) return e;
    GemmProblem tail = p;
    tail.N = p.N - cfg.n_split;
    tail.b = p.b + cfg.n_split * p.K;
    tail.sfb = p.sfb + (cfg.n_split / 128) * (p.K / 128);
    tail.c = p.c + cfg.n_split;
    GemmConfig tc;
    tc.kernel = cfg.tail_kernel;
    tc.bm = cfg.tail_bm;
    tc.bn = cfg.tail_bn;
    tc.splits = 1;
    tc.kb_per_split = cfg.tail_kb_per_split;
    return launch_gemm(tail, tc, ws, stream);
  }
  const TileEntry& t = kTiles[cfg.kernel];
  KArgs k;
  k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.masked_m = p.masked_m;
  k.m_indices = p.m_indices;
  k.groups = p.groups;
  k.sfa_f = p.float_scales ? reinterpret_cast<const float*>(p.sfa) : nullptr;
  if (p.float_scales != reads_float_scales(t.kind)) return hipErrorInvalidValue;
  if (p.b_shuffled != reads_shuffled(t.kind)) return hipErrorInvalidValue;
  if (p.m_indices && (p.E != 1 || p.masked_m || cfg.splits != 1 || kContiguousAlign % t.bm != 0))
    return hipErrorInvalidValue;
  k.M = p.M; k.N = p.N; k.K = p.K; k.ld_sfa = p.ld_sfa; k.ldc = p.ldc;
  const int64_t W = (p.K / 128 + 3) / 4, NB = cdiv(p.N, 128), KB = p.K / 128;
  k.sa_e = p.M * p.K; k.ssfa_e = W * p.ld_sfa; k.sb_e = p.N * p.K; k.ssfb_e = NB * KB; k.sc_e = p.M * p.ldc;
  k.tiles_m = (int)cdiv(p.M, t.bm);
  k.tiles_n = (int)cdiv(p.N, t.bn);
  k.splits = cfg.splits;
  k.kb_per_split = cfg.kb_per_split;
  if ((int64_t)cfg.kb_per_split * (cfg.splits - 1) >= KB) return hipErrorInvalidValue;
  k.ws = nullptr;
  k.counters = nullptr;
  if (cfg.splits > 1) {
    // workspace: the arrival counters (zero between calls), then the fp32 partials;
    // only the kernels that reduce their own split use the counters
    if (ws == nullptr) return hipErrorInvalidValue;
    k.counters = reduces_in_kernel(t.kind) ? static_cast<uint32_t*>(ws) : nullptr;
    k.ws = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  k.sa_words = (cfg.kb_per_split + 3) / 4 + 1;
  const int64_t tiles = (int64_t)k.tiles_m * k.tiles_n;
  if (tiles < 1 || p.E < 1 || KB < 1) return hipSuccess;
  size_t dyn = 0;
  if (t.kind == kStream || is_scaled_tile(t.kind)) {
    dyn = (t.kind == kStream) ? stream_lds_bytes(t.bm, t.bn, cfg.kb_per_split)
                              : scaled_tile_lds_bytes(t.bm, t.bn, t.stages, (int)p.K, t.kind == kScaledFloat);
    if (dyn > kMaxLds) return hipErrorInvalidValue;
    // raise the kernel's dynamic-LDS limit to what this launch needs (never lowered)
    static std::atomic<int> attr_bytes[kNumTiles];
    if ((int)dyn > attr_bytes[cfg.kernel].load()) {
      hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(t.fn),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)dyn);
      if (e != hipSuccess) return e;
      int cur = attr_bytes[cfg.kernel].load();
      while ((int)dyn > cur && !attr_bytes[cfg.kernel].compare_exchange_weak(cur, (int)dyn)) {
      }
    }
  }
  if (is_wsd(t.kind)) {
    if (p.E != 1 || k.tiles_m != 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL(t.fn, dim3((unsigned)(cdiv(tiles, 8) * 8 * cfg.splits)), dim3(t.threads), 0, stream, k);
  } else if (t.kind == kMwsd) {
    // one workgroup per (expert, column tile), the experts' tiles grouped by XCD
    if (!p.masked_m || k.tiles_m != 1 || cfg.splits != 1) return hipErrorInvalidValue;
    k.groups = p.E;
    hipLaunchKernelGGL(t.fn, dim3((unsigned)(cdiv(p.E, 8) * 8 * k.tiles_n)), dim3(t.threads), 0, stream, k);
  } else {
    hipLaunchKernelGGL(t.fn, dim3((unsigned)tiles, (unsigned)cfg.splits, (unsigned)p.E), dim3(t.threads), dyn, stream,
                       k);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || cfg.splits == 1 || reduces_in_kernel(t.kind)) return e;  // the decode kernels reduce themselves
  const int64_t threads = p.M * (p.N / 8);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)cdiv(threads, 256)), dim3(256), 0, stream,
                     static_cast<const float*>(k.ws), cfg.splits, p.M, p.N, p.c, p.ldc);
  return hipGetLastError();
}

}  // namespace fp8bs

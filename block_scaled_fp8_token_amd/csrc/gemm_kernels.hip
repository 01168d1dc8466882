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
// Design (CDNA4): a K-block of 128 is exactly one v_mfma_f32_16x16x128_f8f6f4,
// so each MFMA produces one block partial P for a 16x16 sub-tile and the scale
// is applied as acc += P * (2^ea * sfb) with four FMAs per lane.  The MFMA is
// issued with the weight tile as its first operand so that each lane's four
// results share one output row m: one activation scale per lane per sub-tile,
// and four consecutive bf16 columns per lane in the epilogue.  A and B tiles go
// global -> registers -> LDS, double-buffered, with a 16-byte pad per 128-byte
// row so that the 16 rows read by one MFMA operand fall in distinct banks.
// Workgroups whose rows all lie past the mask return before any load; sub-tiles
// past the mask issue no MFMA.  Decode-sized M splits K across workgroups; the
// last workgroup of a tile to finish sums the fp32 partials in split order
// (deterministic) and writes bf16.
#include "fp8bs_device.hpp"
#include "fp8bs_launch.hpp"

namespace fp8bs {

namespace {

constexpr int LDS_ROW = 144;  // 128 data bytes + 16 pad bytes per row of a K-block tile

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
  float* ws;
  uint32_t* counters;
};

__device__ __forceinline__ v8i frag(const uint8_t* p) {
  const uint4 lo = *reinterpret_cast<const uint4*>(p);
  const uint4 hi = *reinterpret_cast<const uint4*>(p + 16);
  v8i r;
  r[0] = (int)lo.x; r[1] = (int)lo.y; r[2] = (int)lo.z; r[3] = (int)lo.w;
  r[4] = (int)hi.x; r[5] = (int)hi.y; r[6] = (int)hi.z; r[7] = (int)hi.w;
  return r;
}

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(256) void gemm_kernel(const KArgs p) {
  constexpr int NWN = BN / WN;
  constexpr int SM = WM / 16, SN = WN / 16;
  constexpr int CA = BM * 8 / 256, CB = BN * 8 / 256;  // 16-byte chunks per thread
  static_assert((BM / WM) * (BN / WN) == 4, "four wavefronts per workgroup");
  static_assert((BM * 8) % 256 == 0 && (BN * 8) % 256 == 0, "tile rows must fill the loaders");
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BM + BN) * LDS_ROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  const uint8_t* __restrict__ A = p.a + e * p.sa_e;
  const uint32_t* __restrict__ SA = p.sfa + e * p.ssfa_e;
  const uint8_t* __restrict__ B = p.b + e * p.sb_e;
  const float* __restrict__ SB = p.sfb + e * p.ssfb_e;
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
      const uint32_t wd = (m < m_limit) ? SA[(int64_t)(kb >> 2) * p.ld_sfa + m] : 0u;
      sa[i] = __uint_as_float(((wd >> (8 * (kb & 3))) & 0xFFu) << 23);
    }
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = n0 + wn * WN + 16 * j;
      sb[j] = (n < p.N) ? SB[(n >> 7) * KB + kb] : 0.0f;
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

  if (p.splits == 1) {
#pragma unroll
    for (int i = 0; i < SM; ++i) {
      const int64_t m = wrow0 + 16 * i + (lane & 15);
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
    return;
  }

  // split-K: publish this split's scaled partial, then the last arriver reduces
  const size_t slice = (size_t)p.M * (size_t)p.N;
  float* __restrict__ ws = p.ws;
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int64_t m = wrow0 + 16 * i + (lane & 15);
    if (m >= m_limit) continue;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = n0 + wn * WN + 16 * j + 4 * (lane >> 4);
      if (n < p.N)
        *reinterpret_cast<float4*>(ws + (size_t)split * slice + (size_t)m * p.N + n) =
            make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
    }
  }
  __threadfence();
  __syncthreads();
  __shared__ int is_last;
  if (tid == 0) {
    const unsigned old = atomicAdd(&p.counters[tile], 1u);
    is_last = (old == (unsigned)(p.splits - 1)) ? 1 : 0;
  }
  __syncthreads();
  if (!is_last) return;
  __threadfence();
#pragma unroll
  for (int i = 0; i < SM; ++i) {
    const int64_t m = wrow0 + 16 * i + (lane & 15);
    if (m >= m_limit) continue;
#pragma unroll
    for (int j = 0; j < SN; ++j) {
      const int64_t n = n0 + wn * WN + 16 * j + 4 * (lane >> 4);
      if (n >= p.N) continue;
      float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
      for (int sp = 0; sp < p.splits; ++sp) {
        float4 v;
        if (sp == split) {
          v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
        } else {
          v = *reinterpret_cast<const float4*>(ws + (size_t)sp * slice + (size_t)m * p.N + n);
        }
        s0 += v.x; s1 += v.y; s2 += v.z; s3 += v.w;
      }
      uint2 o;
      o.x = bf16_rne(s0) | (bf16_rne(s1) << 16);
      o.y = bf16_rne(s2) | (bf16_rne(s3) << 16);
      *reinterpret_cast<uint2*>(C + m * p.ldc + n) = o;
    }
  }
  if (tid == 0) p.counters[tile] = 0u;  // ready for the next call on this workspace
}

// ---------------------------------------------------------------------------
// compiled tile table

typedef void (*KernelFn)(const KArgs);

struct TileEntry {
  KernelFn fn;
  int bm, bn;
};

const TileEntry kTiles[] = {
    {gemm_kernel<64, 128, 64, 32>, 64, 128},
    {gemm_kernel<128, 128, 64, 64>, 128, 128},
    {gemm_kernel<64, 256, 64, 64>, 64, 256},
    {gemm_kernel<128, 256, 64, 128>, 128, 256},
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Workspace layout: a fixed region of tile counters at offset 0 (only ever written
// by the split-K protocol, which leaves every counter at zero), then the fp32
// partials.  Keeping the counters at a fixed place means a later call with other
// shapes never finds partial data where it expects a zero counter.
constexpr size_t kCounterBytes = 64 * 1024;
constexpr int64_t kMaxSplitTiles = (int64_t)(kCounterBytes / sizeof(uint32_t));

}  // namespace

int gemm_config_count() { return kNumTiles; }

bool gemm_config_by_index(int idx, const GemmProblem& p, int splits, GemmConfig* out) {
  if (idx < 0 || idx >= kNumTiles || splits < 1) return false;
  const int KB = (int)(p.K / 128);
  if (splits > KB) splits = KB > 0 ? KB : 1;
  if (p.masked_m && splits != 1) return false;
  if (splits > 1 && cdiv(p.M, kTiles[idx].bm) * cdiv(p.N, kTiles[idx].bn) > kMaxSplitTiles) splits = 1;
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
  if (p.masked_m) {
    gemm_config_by_index(0, p, 1, &cfg);
    return cfg;
  }
  const int idx = (p.M <= 64) ? 0 : 1;
  const int64_t tiles = cdiv(p.M, kTiles[idx].bm) * cdiv(p.N, kTiles[idx].bn);
  int splits = 1;
  if (tiles < 256) {
    // fill about two workgroups per compute unit, keeping at least 8 K-blocks per split
    splits = (int)cdiv(512, tiles);
    const int max_splits = KB / 8 > 1 ? KB / 8 : 1;
    if (splits > max_splits) splits = max_splits;
  }
  gemm_config_by_index(idx, p, splits, &cfg);
  return cfg;
}

size_t gemm_workspace_bytes(const GemmProblem& p, const GemmConfig& cfg) {
  if (cfg.splits <= 1) return 0;
  const size_t part = (size_t)cfg.splits * (size_t)p.M * (size_t)p.N * sizeof(float);
  return kCounterBytes + part;
}

hipError_t launch_gemm(const GemmProblem& p, const GemmConfig& cfg, void* ws, hipStream_t stream) {
  if (cfg.kernel < 0 || cfg.kernel >= kNumTiles) return hipErrorInvalidValue;
  const TileEntry& t = kTiles[cfg.kernel];
  KArgs k;
  k.a = p.a; k.sfa = p.sfa; k.b = p.b; k.sfb = p.sfb; k.c = p.c; k.masked_m = p.masked_m;
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
    if ((int64_t)k.tiles_m * k.tiles_n > kMaxSplitTiles || ws == nullptr) return hipErrorInvalidValue;
    k.counters = static_cast<uint32_t*>(ws);
    k.ws = reinterpret_cast<float*>(static_cast<char*>(ws) + kCounterBytes);
  }
  const int64_t tiles = (int64_t)k.tiles_m * k.tiles_n;
  if (tiles < 1 || p.E < 1 || KB < 1) return hipSuccess;
  hipLaunchKernelGGL(t.fn, dim3((unsigned)tiles, (unsigned)cfg.splits, (unsigned)p.E), dim3(256), 0, stream, k);
  return hipGetLastError();
}

}  // namespace fp8bs

// Internal launchers of the gfx950 kernels.  The C-ABI layer validates every
// argument before calling these; the launchers only pick grid shapes and launch
// on the caller's stream.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8bs {

hipError_t launch_quant_group_pack(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                   int64_t ldq, uint32_t* sf, int64_t ld_sf, hipStream_t stream);

hipError_t launch_silu_mul_quant(const uint16_t* x, const int32_t* masked_m, int64_t E, int64_t M_max,
                                 int64_t H, uint8_t* q, uint32_t* sf, hipStream_t stream);

hipError_t launch_block_quant(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb,
                              hipStream_t stream);

// e4m3 weights [rows][K] -> the pre-shuffled layout read by the decode kernel
// (rows % 32 == 0, K % 128 == 0).
hipError_t launch_weight_preshuffle(const uint8_t* w, int64_t rows, int64_t K, uint8_t* out, hipStream_t stream);

// Float-scale (non-UE8M0) variants: scale = max(amax, 1e-10) / 448 in fp32.
hipError_t launch_quant_group_float(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, uint8_t* q,
                                   int64_t ldq, float* sf, int64_t ld_sf, hipStream_t stream);
hipError_t launch_block_quant_float(const uint16_t* w, int64_t N, int64_t K, uint8_t* q, float* sfb,
                                   hipStream_t stream);

// Routing ranks (one workgroup per 1024 pairs) then the quantization into the masked
// expert layout; scratch: quant_to_experts_scratch_bytes() of device memory (pair
// ranks and per-chunk expert counts), free for other use once the launches are done.
hipError_t launch_quant_to_experts(const uint16_t* x, int64_t ldx, int64_t T, int64_t K, const int32_t* ids,
                                  int topk, int64_t E, int64_t M_max, uint8_t* q, uint32_t* sf,
                                  int32_t* masked_m, int32_t* slot_of, int32_t* scratch, hipStream_t stream);
size_t quant_to_experts_scratch_bytes(int64_t T, int topk, int64_t E);
constexpr int64_t kQuantToExpertsMaxExperts = 1024;

// One GEMM problem: dense (masked_m == nullptr, m_indices == nullptr, E == 1), masked
// grouped (masked_m set), or contiguous grouped (m_indices set, E == 1: the rows of A
// and C are grouped by weight group in aligned runs, B holds `groups` weight sets).
struct GemmProblem {
  const uint8_t* a;          // e4m3 [E][M][K]
  const uint32_t* sfa;       // packed UE8M0 [E][W][ld_sfa]
  const uint8_t* b;          // e4m3 [E][N][K] ([groups][N][K] for the contiguous layout)
  const float* sfb;          // fp32 [E][ceil(N/128)][K/128] (likewise)
  uint16_t* c;               // bf16 [E][M][ldc]
  const int32_t* masked_m;   // [E] valid rows per group, or nullptr (all M rows valid)
  int64_t E, M, N, K;
  int64_t ld_sfa, ldc;
  const int32_t* m_indices = nullptr;  // [M] weight group of every row (-1: padding), or nullptr
  int64_t groups = 1;                  // weight groups of the contiguous layout
  // float-scale format (dense only): sfa points at fp32 [K/128][ld_sfa] scales and the
  // weight scales are any fp32 values
  bool float_scales = false;
  // weights in the pre-shuffled layout of fp8_weight_preshuffle (dense only)
  bool b_shuffled = false;
};

// Rows per aligned run of one weight group in the contiguous grouped layout.
constexpr int64_t kContiguousAlign = 128;

// Tile configuration chosen for a problem (exposed for reporting and tuning).
struct GemmConfig {
  int kernel = 0;   // index into the compiled tile table
  int bm = 0, bn = 0;   // workgroup tile
  int splits = 1;   // K splits (1 = no split)
  int kb_per_split = 1;  // K-blocks per split; every split owns at least one
  // Column split (dense only): columns [0, n_split) with this configuration and
  // columns [n_split, N) with table entry tail_kernel (splits 1), so that the first
  // launch runs whole rounds of its large tiles.  n_split == 0: no column split.
  int64_t n_split = 0;
  int tail_kernel = 0, tail_bm = 0, tail_bn = 0, tail_kb_per_split = 1;
};

GemmConfig choose_gemm_config(const GemmProblem& p);
size_t gemm_workspace_bytes(const GemmProblem& p, const GemmConfig& cfg);
// Bytes at the front of every workspace that must be zero when it is first used
// (split-K arrival counters; every call leaves them at zero again).
size_t gemm_workspace_zeroed_prefix();
// ws: the fp32 split partials [splits][M][N] (gemm_workspace_bytes); a split-K
// launch runs the GEMM kernel and then the reduction kernel on `stream`.
hipError_t launch_gemm(const GemmProblem& p, const GemmConfig& cfg, void* ws, hipStream_t stream);
int gemm_config_count();
bool gemm_config_by_index(int idx, const GemmProblem& p, int splits, GemmConfig* out);

}  // namespace fp8bs

// C-ABI layer of the block-scaled FP8 library: argument validation, status codes,
// the per-(device, stream) split-K workspace, and dispatch to the gfx950 kernels.
// The operations and their preconditions are stated in include/fp8bs.h.
#include <hip/hip_runtime.h>

#include <climits>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/fp8bs.h"
#include "fp8bs_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

int fail_hip(hipError_t e) {
  g_last_hip_error = (int)e;
  return FP8BS_ERR_LAUNCH;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// gfx950 check, cached per device.
int check_device() {
  static std::mutex mu;
  static std::map<int, bool> ok;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  std::lock_guard<std::mutex> lk(mu);
  auto it = ok.find(dev);
  if (it == ok.end()) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return fail_hip(e);
    const bool is950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    it = ok.emplace(dev, is950).first;
  }
  return it->second ? FP8BS_OK : FP8BS_ERR_DEVICE;
}

// Fill kernel: clears the arrival counters at the front of a fresh workspace on the
// caller's stream (stream-ordered, and a kernel rather than a memset node when the
// call is being captured into a HIP graph).
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = 0u;
}

hipError_t zero_words(void* p, size_t bytes, hipStream_t stream) {
  const int64_t n = (int64_t)(bytes / 4);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
  return hipGetLastError();
}

// Split-K workspace: one buffer per (device, stream), grown on demand.  It holds
// the per-tile arrival counters of the fused split-K reduction (zeroed once, on the
// caller's stream, when the buffer is allocated; every call leaves them at zero)
// and the fp32 partials
// of the call in flight on that stream, which every split overwrites before they
// are read.  A buffer that is outgrown is kept, never freed: a HIP graph captured
// earlier on the stream still launches kernels that use it.
struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;
};

int get_workspace(size_t need, hipStream_t stream, void** out) {
  static std::mutex mu;
  static std::map<std::pair<int, uintptr_t>, Workspace> pool;
  *out = nullptr;
  if (need == 0) return FP8BS_OK;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  std::lock_guard<std::mutex> lk(mu);
  Workspace& w = pool[std::make_pair(dev, reinterpret_cast<uintptr_t>(stream))];
  if (w.bytes >= need) {
    *out = w.ptr;
    return FP8BS_OK;
  }
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  e = hipStreamIsCapturing(stream, &cap);
  if (e != hipSuccess) return fail_hip(e);
  if (cap != hipStreamCaptureStatusNone) return FP8BS_ERR_ALLOC;
  // at least double on growth, so that the retired buffers add up to less than the
  // live one
  size_t sz = need < (size_t(1) << 20) ? (size_t(1) << 20) : need;
  if (sz < 2 * w.bytes) sz = 2 * w.bytes;
  sz = (sz + (size_t(1) << 20) - 1) & ~((size_t(1) << 20) - 1);
  void* p = nullptr;
  e = hipMalloc(&p, sz);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return FP8BS_ERR_ALLOC;
  }
  e = zero_words(p, fp8bs::gemm_workspace_zeroed_prefix(), stream);
  if (e != hipSuccess) {
    (void)hipFree(p);
    return fail_hip(e);
  }
  if (w.ptr) w.retired.push_back(w.ptr);  // earlier work or captured graphs may still use it
  w.ptr = p;
  w.bytes = sz;
  *out = p;
  return FP8BS_OK;
}

// Scratch of the entry point that allocates nothing: one file-scope device array
// (each GPU the library runs on holds its own copy until the process ends).  Host
// code never uses the array's name as an address: its device address comes from
// hipGetSymbolAddress, once per device, with that device current.  The arrival
// counters at its front are cleared by a fill kernel on the first call's stream;
// every call leaves them at zero.  All calls on one GPU share it.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

int static_scratch(hipStream_t stream, void** out) {
  static std::mutex mu;
  static std::map<int, void*> ptrs;
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail_hip(e);
  std::lock_guard<std::mutex> lk(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) return fail_hip(e != hipSuccess ? e : hipErrorInvalidSymbol);
    e = zero_words(ptr, fp8bs::gemm_workspace_zeroed_prefix(), stream);
    if (e != hipSuccess) return fail_hip(e);
    it = ptrs.emplace(dev, ptr).first;
  }
  *out = it->second;
  return FP8BS_OK;
}

int run_gemm(const fp8bs::GemmProblem& prob, const fp8bs::GemmConfig& cfg, hipStream_t stream) {
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;  // no table entry takes this problem
  void* ws = nullptr;
  const size_t need = fp8bs::gemm_workspace_bytes(prob, cfg);
  int st = get_workspace(need, stream, &ws);
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_gemm(prob, cfg, ws, stream);
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int check_dense(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b, const float* sfb,
                const void* c, int64_t ldc, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || N % 64 != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || N == 0) return 1;  // no-op
  if (!a || !sfa || !b || !sfb || !c) return FP8BS_ERR_NULL;
  if (ld_sfa < M || ldc < N) return FP8BS_ERR_SHAPE;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16) || ldc % 8 != 0) return FP8BS_ERR_ALIGN;
  if (!aligned(sfa, 4) || !aligned(sfb, 4)) return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

int check_masked(const void* a, const uint32_t* sfa, const void* b, const float* sfb, const void* c,
                 const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N, int64_t K) {
  if (E < 0 || M_max < 0 || N < 0 || K < 0) return FP8BS_ERR_SHAPE;
  if (K < 128 || K % 128 != 0 || N % 64 != 0) return FP8BS_ERR_SHAPE;
  if (E == 0 || M_max == 0 || N == 0) return 1;  // no-op
  if (!a || !sfa || !b || !sfb || !c || !masked_m) return FP8BS_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(c, 16)) return FP8BS_ERR_ALIGN;
  if (!aligned(sfa, 4) || !aligned(sfb, 4) || !aligned(masked_m, 4)) return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

fp8bs::GemmProblem dense_problem(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                 const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K) {
  fp8bs::GemmProblem p;
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<uint16_t*>(c);
  p.masked_m = nullptr;
  p.E = 1;
  p.M = M;
  p.N = N;
  p.K = K;
  p.ld_sfa = ld_sfa;
  p.ldc = ldc;
  return p;
}

fp8bs::GemmProblem masked_problem(const void* a, const uint32_t* sfa, const void* b, const float* sfb,
                                  void* c, const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N,
                                  int64_t K) {
  fp8bs::GemmProblem p;
  p.a = static_cast<const uint8_t*>(a);
  p.sfa = sfa;
  p.b = static_cast<const uint8_t*>(b);
  p.sfb = sfb;
  p.c = static_cast<uint16_t*>(c);
  p.masked_m = masked_m;
  p.E = E;
  p.M = M_max;
  p.N = N;
  p.K = K;
  p.ld_sfa = M_max;
  p.ldc = N;
  return p;
}

int check_contiguous(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b, const float* sfb,
                     const void* c, int64_t ldc, const int32_t* m_indices, int64_t E, int64_t M, int64_t N,
                     int64_t K) {
  if (E < 0) return FP8BS_ERR_SHAPE;
  const int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st;
  if (E == 0) return 1;  // no expert: every row is padding
  if (!m_indices) return FP8BS_ERR_NULL;
  if (!aligned(m_indices, 4)) return FP8BS_ERR_ALIGN;
  return FP8BS_OK;
}

fp8bs::GemmProblem contiguous_problem(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                      const float* sfb, void* c, int64_t ldc, const int32_t* m_indices,
                                      int64_t E, int64_t M, int64_t N, int64_t K) {
  fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  p.m_indices = m_indices;
  p.groups = E;
  return p;
}

// A problem of the given layout (0 dense, 1 masked, 2 contiguous) for host-side
// configuration queries only: its pointers are placeholders that are never read.
// (3: dense with float scales, 4: dense with pre-shuffled weights, 5: masked with
// pre-shuffled weights, 6: dense with float scales and pre-shuffled weights)
fp8bs::GemmProblem host_problem(int layout, int64_t M, int64_t N, int64_t K) {
  static const int32_t placeholder = 0;
  if (layout == 1 || layout == 5) {
    fp8bs::GemmProblem p = masked_problem(nullptr, nullptr, nullptr, nullptr, nullptr, &placeholder, 1, M, N, K);
    p.b_shuffled = layout == 5;
    return p;
  }
  if (layout == 2)
    return contiguous_problem(nullptr, nullptr, M, nullptr, nullptr, nullptr, N, &placeholder, 1, M, N, K);
  fp8bs::GemmProblem p = dense_problem(nullptr, nullptr, M, nullptr, nullptr, nullptr, N, M, N, K);
  p.float_scales = layout == 3 || layout == 6;
  p.b_shuffled = layout == 4 || layout == 6;
  return p;
}

}  // namespace

extern "C" {

int fp8_quant_group_pack(const void* x, int64_t ldx, int64_t M, int64_t K, void* q, int64_t ldq,
                         uint32_t* sf, int64_t ld_sf, void* stream) {
  if (M < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8BS_OK;
  if (!x || !q || !sf) return FP8BS_ERR_NULL;
  if (ldx < K || ldq < K || ld_sf < M) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || ldx % 8 != 0 || ldq % 16 != 0 || !aligned(sf, 4))
    return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_quant_group_pack(static_cast<const uint16_t*>(x), ldx, M, K,
                                                static_cast<uint8_t*>(q), ldq, sf, ld_sf,
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int silu_mul_quant_group_pack(const void* x, const int32_t* masked_m, int64_t E, int64_t M_max, int64_t H,
                              void* q, uint32_t* sf, void* stream) {
  if (E < 0 || M_max < 0 || H < 0 || H % 128 != 0) return FP8BS_ERR_SHAPE;
  if (E == 0 || M_max == 0 || H == 0) return FP8BS_OK;
  if (!x || !masked_m || !q || !sf) return FP8BS_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(sf, 4) || !aligned(masked_m, 4)) return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_silu_mul_quant(static_cast<const uint16_t*>(x), masked_m, E, M_max, H,
                                              static_cast<uint8_t*>(q), sf, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_quant_group_float(const void* x, int64_t ldx, int64_t M, int64_t K, void* q, int64_t ldq, float* sf,
                          int64_t ld_sf, void* stream) {
  if (M < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (M == 0 || K == 0) return FP8BS_OK;
  if (!x || !q || !sf) return FP8BS_ERR_NULL;
  if (ldx < K || ldq < K || ld_sf < M) return FP8BS_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(q, 16) || ldx % 8 != 0 || ldq % 16 != 0 || !aligned(sf, 4))
    return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_quant_group_float(static_cast<const uint16_t*>(x), ldx, M, K,
                                                 static_cast<uint8_t*>(q), ldq, sf, ld_sf,
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_block_quant_128x128_float(const void* w, int64_t N, int64_t K, void* q, float* sfb, void* stream) {
  if (N < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8BS_OK;
  if (!w || !q || !sfb) return FP8BS_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(sfb, 4)) return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_block_quant_float(static_cast<const uint16_t*>(w), N, K,
                                                 static_cast<uint8_t*>(q), sfb, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_quant_group_pack_to_experts(const void* x, int64_t ldx, int64_t T, int64_t K, const int32_t* topk_ids,
                                    int32_t topk, int64_t E, int64_t M_max, void* q, uint32_t* sf,
                                    int32_t* masked_m, int32_t* slot_of, void* stream) {
  if (T < 0 || K < 0 || K % 128 != 0 || E < 0 || M_max < 0) return FP8BS_ERR_SHAPE;
  if (topk < 1 || topk > 64 || E > fp8bs::kQuantToExpertsMaxExperts || T * (int64_t)topk > INT32_MAX)
    return FP8BS_ERR_SHAPE;
  if (E == 0) return FP8BS_OK;
  if (!masked_m || (T > 0 && (!x || !topk_ids || !slot_of)) || (M_max > 0 && K > 0 && (!q || !sf)))
    return FP8BS_ERR_NULL;
  if (T > 0 && ldx < K) return FP8BS_ERR_SHAPE;
  if ((x && !aligned(x, 16)) || (q && !aligned(q, 16)) || ldx % 8 != 0 || (sf && !aligned(sf, 4)) ||
      !aligned(masked_m, 4) || (topk_ids && !aligned(topk_ids, 4)) || (slot_of && !aligned(slot_of, 4)))
    return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  // pair ranks and per-chunk counts live in the stream's workspace past the counters
  const size_t off = fp8bs::gemm_workspace_zeroed_prefix();
  void* ws = nullptr;
  st = get_workspace(off + fp8bs::quant_to_experts_scratch_bytes(T, topk, E), static_cast<hipStream_t>(stream),
                     &ws);
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_quant_to_experts(static_cast<const uint16_t*>(x), ldx, T, K, topk_ids, topk, E,
                                                M_max, static_cast<uint8_t*>(q), sf, masked_m, slot_of,
                                                reinterpret_cast<int32_t*>(static_cast<char*>(ws) + off),
                                                static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_block_quant_128x128(const void* w, int64_t N, int64_t K, void* q, float* sfb, void* stream) {
  if (N < 0 || K < 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (N == 0 || K == 0) return FP8BS_OK;
  if (!w || !q || !sfb) return FP8BS_ERR_NULL;
  if (!aligned(w, 16) || !aligned(q, 16) || !aligned(sfb, 4)) return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_block_quant(static_cast<const uint16_t*>(w), N, K, static_cast<uint8_t*>(q),
                                           sfb, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_block_gemm_nt(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b, const float* sfb,
                      void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  return run_gemm(p, fp8bs::choose_gemm_config(p), static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b, const float* sfb,
                          void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t kernel, int32_t splits,
                          void* stream) {
  int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, splits < 1 ? 1 : splits, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_weight_preshuffle(const void* w, int64_t rows, int64_t K, void* out, void* stream) {
  if (rows < 0 || K < 0 || rows % 32 != 0 || K % 128 != 0) return FP8BS_ERR_SHAPE;
  if (rows == 0 || K == 0) return FP8BS_OK;
  if (!w || !out) return FP8BS_ERR_NULL;
  if (!aligned(w, 16) || !aligned(out, 16)) return FP8BS_ERR_ALIGN;
  int st = check_device();
  if (st != FP8BS_OK) return st;
  hipError_t e = fp8bs::launch_weight_preshuffle(static_cast<const uint8_t*>(w), rows, K, static_cast<uint8_t*>(out),
                                                 static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_block_gemm_nt_preshuffled(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                  const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                  void* stream) {
  int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  p.b_shuffled = true;
  const fp8bs::GemmConfig cfg = fp8bs::choose_gemm_config(p);
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_preshuffled_noalloc(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                          const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                          void* stream) {
  int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  p.b_shuffled = true;
  const fp8bs::GemmConfig cfg = fp8bs::choose_gemm_config(p);
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;
  const size_t need = fp8bs::gemm_workspace_bytes(p, cfg);
  if (need > kStaticScratchBytes) return FP8BS_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = static_scratch(static_cast<hipStream_t>(stream), &ws);
    if (st != FP8BS_OK) return st;
  }
  hipError_t e = fp8bs::launch_gemm(p, cfg, ws, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? FP8BS_OK : fail_hip(e);
}

int fp8_block_gemm_nt_preshuffled_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                      const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                      int32_t kernel, int32_t splits, void* stream) {
  int st = check_dense(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, sfa, ld_sfa, b, sfb, c, ldc, M, N, K);
  p.b_shuffled = true;
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, splits < 1 ? 1 : splits, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_masked_preshuffled(const void* a, const uint32_t* sfa, const void* b, const float* sfb,
                                              void* c, const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N,
                                              int64_t K, void* stream) {
  int st = check_masked(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = masked_problem(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  p.b_shuffled = true;
  const fp8bs::GemmConfig cfg = fp8bs::choose_gemm_config(p);
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_masked_preshuffled_cfg(const void* a, const uint32_t* sfa, const void* b,
                                                  const float* sfb, void* c, const int32_t* masked_m, int64_t E,
                                                  int64_t M_max, int64_t N, int64_t K, int32_t kernel,
                                                  void* stream) {
  int st = check_masked(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = masked_problem(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  p.b_shuffled = true;
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, 1, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_masked(const void* a, const uint32_t* sfa, const void* b, const float* sfb, void* c,
                                  const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N, int64_t K,
                                  void* stream) {
  int st = check_masked(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = masked_problem(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  return run_gemm(p, fp8bs::choose_gemm_config(p), static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_masked_cfg(const void* a, const uint32_t* sfa, const void* b, const float* sfb,
                                      void* c, const int32_t* masked_m, int64_t E, int64_t M_max, int64_t N,
                                      int64_t K, int32_t kernel, void* stream) {
  int st = check_masked(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = masked_problem(a, sfa, b, sfb, c, masked_m, E, M_max, N, K);
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, 1, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_contiguous(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                      const float* sfb, void* c, int64_t ldc, const int32_t* m_indices, int64_t E,
                                      int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_contiguous(a, sfa, ld_sfa, b, sfb, c, ldc, m_indices, E, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = contiguous_problem(a, sfa, ld_sfa, b, sfb, c, ldc, m_indices, E, M, N, K);
  return run_gemm(p, fp8bs::choose_gemm_config(p), static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_grouped_contiguous_cfg(const void* a, const uint32_t* sfa, int64_t ld_sfa, const void* b,
                                          const float* sfb, void* c, int64_t ldc, const int32_t* m_indices,
                                          int64_t E, int64_t M, int64_t N, int64_t K, int32_t kernel,
                                          void* stream) {
  int st = check_contiguous(a, sfa, ld_sfa, b, sfb, c, ldc, m_indices, E, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  const fp8bs::GemmProblem p = contiguous_problem(a, sfa, ld_sfa, b, sfb, c, ldc, m_indices, E, M, N, K);
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, 1, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_float_scales(const void* a, const float* sfa, int64_t ld_sfa, const void* b, const float* sfb,
                                   void* c, int64_t ldc, int64_t M, int64_t N, int64_t K, void* stream) {
  int st = check_dense(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  p.float_scales = true;
  return run_gemm(p, fp8bs::choose_gemm_config(p), static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_float_scales_cfg(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                       const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N, int64_t K,
                                       int32_t kernel, int32_t splits, void* stream) {
  int st = check_dense(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  p.float_scales = true;
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, splits < 1 ? 1 : splits, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_float_scales_preshuffled(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                                const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                                int64_t K, void* stream) {
  int st = check_dense(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  p.float_scales = true;
  p.b_shuffled = true;
  const fp8bs::GemmConfig cfg = fp8bs::choose_gemm_config(p);
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8_block_gemm_nt_float_scales_preshuffled_cfg(const void* a, const float* sfa, int64_t ld_sfa, const void* b,
                                                    const float* sfb, void* c, int64_t ldc, int64_t M, int64_t N,
                                                    int64_t K, int32_t kernel, int32_t splits, void* stream) {
  int st = check_dense(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  if (st != FP8BS_OK) return st > 0 ? FP8BS_OK : st;
  st = check_device();
  if (st != FP8BS_OK) return st;
  fp8bs::GemmProblem p = dense_problem(a, reinterpret_cast<const uint32_t*>(sfa), ld_sfa, b, sfb, c, ldc, M, N, K);
  p.float_scales = true;
  p.b_shuffled = true;
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, splits < 1 ? 1 : splits, &cfg)) return FP8BS_ERR_SHAPE;
  return run_gemm(p, cfg, static_cast<hipStream_t>(stream));
}

int fp8bs_gemm_config_count(void) { return fp8bs::gemm_config_count(); }

int fp8bs_gemm_config(int masked, int64_t M, int64_t N, int64_t K, int32_t* kernel, int32_t* bm, int32_t* bn,
                      int32_t* splits) {
  if (M < 0 || N < 0 || K < 128 || K % 128 != 0 || N % 64 != 0) return FP8BS_ERR_SHAPE;
  if (!kernel || !bm || !bn || !splits) return FP8BS_ERR_NULL;
  if (masked < 0 || masked > 6) return FP8BS_ERR_SHAPE;
  const fp8bs::GemmProblem p = host_problem(masked, M, N, K);
  const fp8bs::GemmConfig cfg = fp8bs::choose_gemm_config(p);
  if (cfg.kernel < 0) return FP8BS_ERR_SHAPE;  // no entry takes this problem (K past every scale table)
  *kernel = cfg.kernel;
  *bm = cfg.bm;
  *bn = cfg.bn;
  *splits = cfg.splits;
  return FP8BS_OK;
}

int fp8bs_gemm_config_of(int32_t kernel, int masked, int64_t M, int64_t N, int64_t K, int32_t splits, int32_t* bm,
                         int32_t* bn, int32_t* splits_out) {
  if (M < 0 || N < 0 || K < 128 || K % 128 != 0 || N % 64 != 0) return FP8BS_ERR_SHAPE;
  if (!bm || !bn || !splits_out) return FP8BS_ERR_NULL;
  if (masked < 0 || masked > 6) return FP8BS_ERR_SHAPE;
  const fp8bs::GemmProblem p = host_problem(masked, M, N, K);
  fp8bs::GemmConfig cfg;
  if (!fp8bs::gemm_config_by_index(kernel, p, splits < 1 ? 1 : splits, &cfg)) return FP8BS_ERR_SHAPE;
  *bm = cfg.bm;
  *bn = cfg.bn;
  *splits_out = cfg.splits;
  return FP8BS_OK;
}

const char* fp8bs_status_string(int status) {
  switch (status) {
    case FP8BS_OK: return "ok";
    case FP8BS_ERR_NULL: return "null pointer";
    case FP8BS_ERR_SHAPE: return "invalid shape or leading dimension";
    case FP8BS_ERR_ALIGN: return "misaligned pointer or row stride";
    case FP8BS_ERR_DEVICE: return "device is not gfx950";
    case FP8BS_ERR_LAUNCH: return "HIP call failed";
    case FP8BS_ERR_ALLOC: return "workspace allocation failed or refused during graph capture";
    case FP8BS_ERR_SCRATCH: return "the problem needs more scratch than the static buffer of the no-allocation entry holds";
    default: return "unknown status";
  }
}

int fp8bs_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
